// Seeded random exerciser of the library's host code (mask builders, block
// schedules, split unit lists, transposes and the launch entry points'
// argument checks), for sanitizer builds: every result is compared with a
// brute-force dense matrix built here, and malformed CSR inputs must be
// refused.  Prints "ok" and exits 0 on success.
//
// Usage: mask_fuzz [iterations] [seed]
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "attn_jvp.h"

namespace {

#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

// xorshift64*: a small seeded generator (test input only)
struct Rng {
  uint64_t s;
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 0x2545F4914F6CDD1DULL;
  }
  int below(int n) { return n <= 0 ? 0 : int(next() % uint64_t(n)); }
};

struct Csr {
  int n_q = 0, n_k = 0;
  std::vector<int32_t> gq, rp, kb, ke;
};

// Random groups with sorted, disjoint (possibly touching or empty) ranges.
Csr random_csr(Rng &r) {
  Csr c;
  c.n_q = 1 + r.below(300);
  c.n_k = 1 + r.below(300);
  const int groups = 1 + r.below(std::min(8, c.n_q));
  c.gq.push_back(0);
  for (int g = 1; g < groups; ++g) {
    const int lo = c.gq.back() + 1, hi = c.n_q - (groups - g);
    c.gq.push_back(lo + r.below(hi - lo + 1));
  }
  c.gq.push_back(c.n_q);
  c.rp.push_back(0);
  for (int g = 0; g < groups; ++g) {
    int at = 0;
    const int ranges = r.below(4);
    for (int i = 0; i < ranges && at <= c.n_k; ++i) {
      const int b = at + r.below(c.n_k - at + 1);
      const int e = b + r.below(c.n_k - b + 1);
      c.kb.push_back(b);
      c.ke.push_back(e);
      at = e + r.below(3);  // touching ranges are allowed
    }
    c.rp.push_back(int32_t(c.kb.size()));
  }
  return c;
}

std::vector<uint8_t> dense(const Csr &c) {
  std::vector<uint8_t> M(size_t(c.n_q) * c.n_k, 0);
  for (size_t g = 0; g + 1 < c.gq.size(); ++g)
    for (int r = c.rp[g]; r < c.rp[g + 1]; ++r)
      for (int i = c.gq[g]; i < c.gq[g + 1]; ++i)
        for (int j = c.kb[r]; j < c.ke[r]; ++j) M[size_t(i) * c.n_k + j] = 1;
  return M;
}

Csr export_mask(const attn_jvp_mask *m) {
  Csr c;
  int32_t ng = 0, nr = 0, nq = 0, nk = 0;
  int64_t pairs = 0;
  CHECK(attn_jvp_mask_info(m, &nq, &nk, &ng, &nr, &pairs) == ATTN_JVP_OK);
  c.n_q = nq;
  c.n_k = nk;
  c.gq.resize(ng + 1);
  c.rp.resize(ng + 1);
  c.kb.resize(nr);
  c.ke.resize(nr);
  CHECK(attn_jvp_mask_export(m, c.gq.data(), c.rp.data(), c.kb.data(), c.ke.data()) ==
        ATTN_JVP_OK);
  return c;
}

// The schedule of a tile shape against the dense matrix: every listed block
// is touched, every touched block listed once, full flags and bits exact.
void check_schedule(const attn_jvp_mask *m, const std::vector<uint8_t> &M, int n_q, int n_k,
                    int BM, int BN) {
  int32_t nt = 0;
  int64_t ne = 0, np = 0;
  CHECK(attn_jvp_mask_schedule(m, BM, BN, &nt, &ne, &np, nullptr, nullptr, nullptr, nullptr,
                               nullptr) == ATTN_JVP_OK);
  const int words = BN / 32;
  std::vector<int32_t> off(nt + 1), order(nt), eb(ne), ep(ne);
  std::vector<uint32_t> bits(size_t(np) * BM * words);
  CHECK(attn_jvp_mask_schedule(m, BM, BN, &nt, &ne, &np, off.data(), order.data(), eb.data(),
                               ep.data(), bits.data()) == ATTN_JVP_OK);
  CHECK(nt == (n_q + BM - 1) / BM && off[0] == 0 && off[nt] == ne);
  const int n_kb = (n_k + BN - 1) / BN;
  for (int t = 0; t < nt; ++t) {
    std::vector<int> seen(n_kb, 0);
    for (int e = off[t]; e < off[t + 1]; ++e) {
      const int kb = eb[e];
      CHECK(kb >= 0 && kb < n_kb && !seen[kb]);
      seen[kb] = 1;
      bool any = false, all = true;
      for (int i = 0; i < BM; ++i)
        for (int j = 0; j < BN; ++j) {
          const int row = t * BM + i, key = kb * BN + j;
          const bool in = row < n_q && key < n_k && M[size_t(row) * n_k + key];
          any |= in;
          if (row < n_q) all &= in;
          if (ep[e] >= 0) {
            CHECK(ep[e] < np);
            const uint32_t w = bits[(size_t(ep[e]) * BM + i) * words + j / 32];
            CHECK(bool((w >> (j % 32)) & 1u) == in);
          }
        }
      CHECK(any);
      CHECK((ep[e] < 0) == all);
    }
    for (int kb = 0; kb < n_kb; ++kb) {
      if (seen[kb]) continue;
      for (int i = t * BM; i < std::min(n_q, t * BM + BM); ++i)
        for (int j = kb * BN; j < std::min(n_k, kb * BN + BN); ++j) CHECK(!M[size_t(i) * n_k + j]);
    }
  }
  // split unit lists cover each tile's entries in order
  for (int S : {1, 2, 3, 7}) {
    int32_t nu = 0, nparts = 0;
    CHECK(attn_jvp_mask_split_schedule(m, BM, BN, S, &nu, &nparts, nullptr, nullptr, nullptr,
                                       nullptr) == ATTN_JVP_OK);
    std::vector<int32_t> uo(nu + 1), uord(nu), ut(nu), up(nu);
    CHECK(attn_jvp_mask_split_schedule(m, BM, BN, S, &nu, &nparts, uo.data(), uord.data(),
                                       ut.data(), up.data()) == ATTN_JVP_OK);
    std::vector<int32_t> covered(nt, 0);
    for (int u = 0; u < nu; ++u) {
      CHECK(ut[u] >= 0 && ut[u] < nt && uo[u] <= uo[u + 1]);
      CHECK(uo[u] >= off[ut[u]] && uo[u + 1] <= off[ut[u] + 1]);
      covered[ut[u]] += uo[u + 1] - uo[u];
      CHECK(up[u] >= -1 && up[u] < nparts);
    }
    for (int t = 0; t < nt; ++t) CHECK(covered[t] == off[t + 1] - off[t]);
  }
}

void check_mask(const attn_jvp_mask *m, const std::vector<uint8_t> &M, int n_q, int n_k) {
  const Csr e = export_mask(m);
  CHECK(e.n_q == n_q && e.n_k == n_k);
  CHECK(dense(e) == M);
  int64_t pairs = 0;
  CHECK(attn_jvp_mask_info(m, nullptr, nullptr, nullptr, nullptr, &pairs) == ATTN_JVP_OK);
  int64_t cnt = 0;
  for (uint8_t x : M) cnt += x;
  CHECK(pairs == cnt);
  for (int BM : {1, 16, 64, 256})
    for (int BN : {32, 64}) check_schedule(m, M, n_q, n_k, BM, BN);
  attn_jvp_mask *t = nullptr;
  CHECK(attn_jvp_mask_transpose(m, &t) == ATTN_JVP_OK);
  const Csr te = export_mask(t);
  const std::vector<uint8_t> TM = dense(te);
  for (int i = 0; i < n_q; ++i)
    for (int j = 0; j < n_k; ++j) CHECK(TM[size_t(j) * n_q + i] == M[size_t(i) * n_k + j]);
  attn_jvp_mask_free(t);
}

// Placeholder device addresses: the argument checks never dereference them.
void check_args(const attn_jvp_mask *m, Rng &r) {
  int32_t nq = 0, nk = 0;
  CHECK(attn_jvp_mask_info(m, &nq, &nk, nullptr, nullptr, nullptr) == ATTN_JVP_OK);
  attn_jvp_args a = {};
  a.dtype = r.below(2) ? ATTN_JVP_BF16 : ATTN_JVP_F32;
  a.B = 1 + r.below(2);
  a.H = 1 + r.below(3);
  a.n_q = nq;
  a.n_k = nk;
  a.D = r.below(2) ? 64 : 128;
  a.q_stride_h = a.D + 4 * r.below(3);
  a.q_stride_n = a.H * a.q_stride_h;
  a.q_stride_b = int64_t(nq) * a.q_stride_n;
  a.k_stride_h = a.q_stride_h;
  a.k_stride_n = a.q_stride_n;
  a.k_stride_b = int64_t(nk) * a.k_stride_n;
  const uintptr_t sp = uintptr_t(1) << 32;
  a.q = reinterpret_cast<void *>(sp);
  a.k = reinterpret_cast<void *>(2 * sp);
  a.v = reinterpret_cast<void *>(3 * sp);
  a.dq = reinterpret_cast<void *>(4 * sp);
  a.dk = reinterpret_cast<void *>(5 * sp);
  a.dv = reinterpret_cast<void *>(6 * sp);
  a.o = reinterpret_cast<void *>(7 * sp);
  a.d_o = reinterpret_cast<void *>(8 * sp);
  a.lse = reinterpret_cast<float *>(9 * sp);
  // an output moved onto a random input position must be refused
  uint64_t need = 0;
  const int st = attn_jvp_fwd_split_workspace(&a, m, 1 + r.below(4), &need);
  const bool aligned = (a.q_stride_h * (a.dtype == ATTN_JVP_BF16 ? 2 : 4)) % 16 == 0;
  CHECK(st == (aligned ? ATTN_JVP_OK : ATTN_JVP_ERR_ALIGN));
  if (aligned) {
    a.o = reinterpret_cast<void *>(sp + 16 * r.below(8));  // inside q's first row
    CHECK(attn_jvp_fwd_split_workspace(&a, m, 1, &need) == ATTN_JVP_ERR_UNSUPPORTED);
  }
  int32_t chosen = 0;
  (void)attn_jvp_split_choose(&a, m, 1 + r.below(300), &chosen);
}

}  // namespace

int main(int argc, char **argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200;
  Rng r{argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 0x9e3779b97f4a7c15ULL};
  for (int it = 0; it < iters; ++it) {
    Csr c = random_csr(r);
    const int ng = int(c.gq.size()) - 1;
    // occasionally corrupt the input: the builder must refuse, never read past it
    const int corrupt = r.below(5) == 0 ? 1 + r.below(5) : 0;
    if (corrupt == 1 && !c.kb.empty()) c.kb[r.below(int(c.kb.size()))] = -1 - r.below(5);
    if (corrupt == 2 && !c.ke.empty()) c.ke[r.below(int(c.ke.size()))] = c.n_k + 1 + r.below(5);
    if (corrupt == 3 && ng > 1) std::swap(c.rp[1], c.rp[ng]);
    if (corrupt == 4 && ng > 1) c.gq[1] = c.gq[0];
    if (corrupt == 5 && c.kb.size() > 1) std::swap(c.kb[0], c.kb[1]);
    attn_jvp_mask *m = nullptr;
    const int st = attn_jvp_mask_rects(c.n_q, c.n_k, ng, c.gq.data(), c.rp.data(),
                                       c.kb.empty() ? nullptr : c.kb.data(),
                                       c.ke.empty() ? nullptr : c.ke.data(), &m);
    if (st != ATTN_JVP_OK) {
      CHECK(corrupt != 0 && m == nullptr);
      continue;
    }
    check_mask(m, dense(c), c.n_q, c.n_k);
    check_args(m, r);
    attn_jvp_mask_free(m);
  }
  // the structured builders on small shapes
  for (int nf = 1; nf <= 6; ++nf)
    for (int tpf = 1; tpf <= 40; tpf += 13)
      for (int fpc = 1; fpc <= nf; ++fpc) {
        if (nf % fpc) continue;
        attn_jvp_mask *m = nullptr;
        CHECK(attn_jvp_mask_tf(nf, tpf, fpc, &m) == ATTN_JVP_OK);
        const Csr e = export_mask(m);
        check_mask(m, dense(e), e.n_q, e.n_k);
        attn_jvp_mask_free(m);
        CHECK(attn_jvp_mask_block_causal(nf, tpf, &m) == ATTN_JVP_OK);
        const Csr b = export_mask(m);
        check_mask(m, dense(b), b.n_q, b.n_k);
        attn_jvp_mask_free(m);
      }
  std::printf("ok\n");
  return 0;
}
