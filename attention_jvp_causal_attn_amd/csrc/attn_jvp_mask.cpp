// Mask descriptors (query groups with admissible key ranges) and the block
// schedule derived from them.
//
// "Causal-rCM ..." summary, Appendix B: custom masks are query groups with
// admissible key ranges (query-key rectangles, covering dense and structured
// causal masks), and one sparse schedule drives both the primal and the
// tangent scores, so no dense mask is ever materialised.  The teacher-forcing
// layout (packed [clean | noisy] tokens) follows Section 3 of that page and
// "Causal Forcing ..." Section 2.
#include <algorithm>
#include <cstring>
#include <new>

#include "internal.h"

using attnjvp::HostSchedule;

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 30;

// Canonicalise groups: drop empty ranges, merge touching ones (input already
// validated: sorted and non-overlapping), then merge adjacent groups whose
// key sets are identical.
int finish_mask(attn_jvp_mask *m, const std::vector<int32_t> &gq,
                const std::vector<std::vector<std::pair<int32_t, int32_t>>> &granges) {
  std::vector<std::vector<std::pair<int32_t, int32_t>>> clean(granges.size());
  for (size_t g = 0; g < granges.size(); ++g) {
    for (auto r : granges[g]) {
      if (r.first == r.second) continue;
      if (!clean[g].empty() && clean[g].back().second == r.first)
        clean[g].back().second = r.second;
      else
        clean[g].push_back(r);
    }
  }
  m->group_q_begin.clear();
  m->range_ptr.clear();
  m->k_begin.clear();
  m->k_end.clear();
  m->range_ptr.push_back(0);
  m->n_visible = 0;
  for (size_t g = 0; g < clean.size(); ++g) {
    bool same_as_prev = g > 0 && !m->group_q_begin.empty() && clean[g] == clean[g - 1];
    if (!same_as_prev) {
      m->group_q_begin.push_back(gq[g]);
      for (auto r : clean[g]) {
        m->k_begin.push_back(r.first);
        m->k_end.push_back(r.second);
      }
      m->range_ptr.push_back(int32_t(m->k_begin.size()));
    }
    int64_t keys = 0;
    for (auto r : clean[g]) keys += r.second - r.first;
    m->n_visible += keys * int64_t(gq[g + 1] - gq[g]);
  }
  m->group_q_begin.push_back(gq.back());
  return ATTN_JVP_OK;
}

}  // namespace

extern "C" int attn_jvp_mask_rects(int32_t n_q, int32_t n_k, int32_t n_groups,
                                   const int32_t *group_q_begin, const int32_t *range_ptr,
                                   const int32_t *k_begin, const int32_t *k_end,
                                   attn_jvp_mask **out) {
  if (!out || !group_q_begin || !range_ptr) return ATTN_JVP_ERR_NULL;
  if (n_q <= 0 || n_k <= 0 || n_q > kMaxTokens || n_k > kMaxTokens || n_groups <= 0)
    return ATTN_JVP_ERR_SHAPE;
  if (group_q_begin[0] != 0 || group_q_begin[n_groups] != n_q) return ATTN_JVP_ERR_MASK;
  for (int g = 0; g < n_groups; ++g)
    if (group_q_begin[g + 1] <= group_q_begin[g]) return ATTN_JVP_ERR_MASK;
  if (range_ptr[0] != 0) return ATTN_JVP_ERR_MASK;
  for (int g = 0; g < n_groups; ++g)
    if (range_ptr[g + 1] < range_ptr[g]) return ATTN_JVP_ERR_MASK;
  if (range_ptr[n_groups] > 0 && (!k_begin || !k_end)) return ATTN_JVP_ERR_NULL;
  std::vector<int32_t> gq(group_q_begin, group_q_begin + n_groups + 1);
  std::vector<std::vector<std::pair<int32_t, int32_t>>> granges(n_groups);
  try {
    for (int g = 0; g < n_groups; ++g) {
      int32_t prev_end = 0;
      for (int r = range_ptr[g]; r < range_ptr[g + 1]; ++r) {
        int32_t b = k_begin[r], e = k_end[r];
        if (b < 0 || e < b || e > n_k) return ATTN_JVP_ERR_MASK;
        if (b == e) continue;
        if (b < prev_end) return ATTN_JVP_ERR_MASK;  // unsorted or overlapping
        prev_end = e;
        granges[g].push_back({b, e});
      }
    }
    auto *m = new attn_jvp_mask();
    m->n_q = n_q;
    m->n_k = n_k;
    finish_mask(m, gq, granges);
    *out = m;
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_tf(int32_t n_frames, int32_t tokens_per_frame,
                                int32_t frames_per_chunk, attn_jvp_mask **out) {
  if (!out) return ATTN_JVP_ERR_NULL;
  if (n_frames <= 0 || tokens_per_frame <= 0 || frames_per_chunk <= 0)
    return ATTN_JVP_ERR_SHAPE;
  if (n_frames % frames_per_chunk) return ATTN_JVP_ERR_SHAPE;
  const int64_t n_clean = int64_t(n_frames) * tokens_per_frame;
  if (2 * n_clean > kMaxTokens) return ATTN_JVP_ERR_SHAPE;
  const int32_t C = tokens_per_frame * frames_per_chunk;  // tokens per unit
  const int32_t F = n_frames / frames_per_chunk;          // units per stream
  const int32_t Nc = int32_t(n_clean), N = 2 * Nc;
  // Groups: clean units 0..F-1, then noisy units 0..F-1.
  std::vector<int32_t> gq;
  std::vector<std::vector<std::pair<int32_t, int32_t>>> granges;
  try {
    for (int u = 0; u < F; ++u) {  // clean unit u: clean keys of units <= u
      gq.push_back(u * C);
      granges.push_back({{0, (u + 1) * C}});
    }
    for (int u = 0; u < F; ++u) {  // noisy unit u: clean units < u, own noisy unit
      gq.push_back(Nc + u * C);
      std::vector<std::pair<int32_t, int32_t>> r;
      if (u > 0) r.push_back({0, u * C});
      r.push_back({Nc + u * C, Nc + (u + 1) * C});
      granges.push_back(r);
    }
    gq.push_back(N);
    auto *m = new attn_jvp_mask();
    m->n_q = m->n_k = N;
    finish_mask(m, gq, granges);
    *out = m;
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_block_causal(int32_t n_units, int32_t unit_tokens,
                                          attn_jvp_mask **out) {
  if (!out) return ATTN_JVP_ERR_NULL;
  if (n_units <= 0 || unit_tokens <= 0) return ATTN_JVP_ERR_SHAPE;
  if (int64_t(n_units) * unit_tokens > kMaxTokens) return ATTN_JVP_ERR_SHAPE;
  const int32_t N = n_units * unit_tokens;
  std::vector<int32_t> gq;
  std::vector<std::vector<std::pair<int32_t, int32_t>>> granges;
  try {
    for (int u = 0; u < n_units; ++u) {  // unit u: keys of units <= u
      gq.push_back(u * unit_tokens);
      granges.push_back({{0, (u + 1) * unit_tokens}});
    }
    gq.push_back(N);
    auto *m = new attn_jvp_mask();
    m->n_q = m->n_k = N;
    finish_mask(m, gq, granges);
    *out = m;
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_dense(int32_t n_q, int32_t n_k, attn_jvp_mask **out) {
  const int32_t gq[2] = {0, n_q}, rp[2] = {0, 1}, kb[1] = {0}, ke[1] = {n_k};
  if (!out) return ATTN_JVP_ERR_NULL;
  return attn_jvp_mask_rects(n_q, n_k, 1, gq, rp, kb, ke, out);
}

extern "C" int attn_jvp_mask_info(const attn_jvp_mask *m, int32_t *n_q, int32_t *n_k,
                                  int32_t *n_groups, int32_t *n_ranges,
                                  int64_t *n_visible_pairs) {
  if (!m) return ATTN_JVP_ERR_NULL;
  if (n_q) *n_q = m->n_q;
  if (n_k) *n_k = m->n_k;
  if (n_groups) *n_groups = int32_t(m->group_q_begin.size()) - 1;
  if (n_ranges) *n_ranges = int32_t(m->k_begin.size());
  if (n_visible_pairs) *n_visible_pairs = m->n_visible;
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_export(const attn_jvp_mask *m, int32_t *group_q_begin,
                                    int32_t *range_ptr, int32_t *k_begin, int32_t *k_end) {
  if (!m || !group_q_begin || !range_ptr) return ATTN_JVP_ERR_NULL;
  if (!m->k_begin.empty() && (!k_begin || !k_end)) return ATTN_JVP_ERR_NULL;
  std::copy(m->group_q_begin.begin(), m->group_q_begin.end(), group_q_begin);
  std::copy(m->range_ptr.begin(), m->range_ptr.end(), range_ptr);
  std::copy(m->k_begin.begin(), m->k_begin.end(), k_begin);
  std::copy(m->k_end.begin(), m->k_end.end(), k_end);
  return ATTN_JVP_OK;
}

namespace attnjvp {

int transpose_mask(const attn_jvp_mask *m, attn_jvp_mask **out) {
  try {
    // elementary key intervals: cut [0, n_k) at every range boundary
    std::vector<int32_t> cuts = {0, m->n_k};
    cuts.insert(cuts.end(), m->k_begin.begin(), m->k_begin.end());
    cuts.insert(cuts.end(), m->k_end.begin(), m->k_end.end());
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    const size_t n_int = cuts.size() - 1;
    // each interval collects the query ranges of the groups that admit it, in
    // increasing query order (groups are visited in order)
    std::vector<std::vector<std::pair<int32_t, int32_t>>> qr(n_int);
    const size_t n_groups = m->group_q_begin.size() - 1;
    for (size_t g = 0; g < n_groups; ++g) {
      const std::pair<int32_t, int32_t> rows{m->group_q_begin[g], m->group_q_begin[g + 1]};
      for (int32_t r = m->range_ptr[g]; r < m->range_ptr[g + 1]; ++r) {
        const size_t a = std::lower_bound(cuts.begin(), cuts.end(), m->k_begin[r]) - cuts.begin();
        const size_t b = std::lower_bound(cuts.begin(), cuts.end(), m->k_end[r]) - cuts.begin();
        for (size_t i = a; i < b; ++i) {
          if (!qr[i].empty() && qr[i].back().second == rows.first)
            qr[i].back().second = rows.second;  // touching groups
          else
            qr[i].push_back(rows);
        }
      }
    }
    auto *t = new attn_jvp_mask();
    t->n_q = m->n_k;
    t->n_k = m->n_q;
    finish_mask(t, cuts, qr);
    *out = t;
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  return ATTN_JVP_OK;
}

// Number of (query tile, key block) entries of the schedule, counted without
// building it: per tile, the union of the key-block intervals that the ranges
// of its groups touch.  Exact, in 64 bits.
static int64_t count_entries(const attn_jvp_mask *m, int BM, int BN) {
  const int n_tiles = (m->n_q + BM - 1) / BM;
  const int n_groups = int(m->group_q_begin.size()) - 1;
  std::vector<std::pair<int64_t, int64_t>> iv;
  int64_t total = 0;
  int g0 = 0;
  for (int t = 0; t < n_tiles; ++t) {
    const int r0 = t * BM, r1 = std::min(m->n_q, r0 + BM);
    while (g0 + 1 < n_groups && m->group_q_begin[g0 + 1] <= r0) ++g0;
    iv.clear();
    for (int g = g0; g < n_groups && m->group_q_begin[g] < r1; ++g)
      for (int r = m->range_ptr[g]; r < m->range_ptr[g + 1]; ++r)
        iv.push_back({m->k_begin[r] / BN, (int64_t(m->k_end[r]) + BN - 1) / BN});
    std::sort(iv.begin(), iv.end());
    int64_t hi = -1;
    for (auto &x : iv) {
      const int64_t lo = std::max(x.first, hi);
      if (x.second > lo) total += x.second - lo;
      hi = std::max(hi, x.second);
    }
  }
  return total;
}

// Classify every key block for every query tile.  A block is listed when some
// row of the tile admits some key of it; it is full when every existing row
// of the tile admits all block_n keys (so a block reaching past n_k is never
// full).  Partial blocks get one bit per (row, key).
static void build_schedule(const attn_jvp_mask *m, int BM, int BN, HostSchedule &s) {
  const int n_tiles = (m->n_q + BM - 1) / BM;
  const int n_kb = (m->n_k + BN - 1) / BN;
  const int words = BN / 32;
  const int n_groups = int(m->group_q_begin.size()) - 1;
  s.block_m = BM;
  s.block_n = BN;
  s.n_tiles = n_tiles;
  s.tile_offsets.assign(1, 0);
  s.tile_nfull.clear();
  s.entry_block.clear();
  s.entry_partial.clear();
  s.partial_bits.clear();
  s.n_partial = 0;
  std::vector<int32_t> touched_cnt(n_kb, 0), full_groups(n_kb, 0), any_group(n_kb, 0);
  std::vector<int32_t> touched;
  std::vector<int32_t> group_cnt(n_kb, 0);
  std::vector<int32_t> gtouch;
  for (int t = 0; t < n_tiles; ++t) {
    const int r0 = t * BM, r1 = std::min(m->n_q, r0 + BM);
    // groups intersecting [r0, r1)
    int g0 = int(std::upper_bound(m->group_q_begin.begin(), m->group_q_begin.end(), r0) -
                 m->group_q_begin.begin()) - 1;
    int g1 = g0;
    while (g1 < n_groups && m->group_q_begin[g1] < r1) ++g1;  // [g0, g1)
    const int n_tile_groups = g1 - g0;
    touched.clear();
    for (int g = g0; g < g1; ++g) {
      gtouch.clear();
      for (int r = m->range_ptr[g]; r < m->range_ptr[g + 1]; ++r) {
        int b = m->k_begin[r], e = m->k_end[r];
        for (int kb = b / BN; kb * BN < e; ++kb) {
          int lo = std::max(b, kb * BN), hi = std::min(e, kb * BN + BN);
          if (group_cnt[kb] == 0) gtouch.push_back(kb);
          group_cnt[kb] += hi - lo;
        }
      }
      for (int kb : gtouch) {
        if (!any_group[kb]) {
          any_group[kb] = 1;
          touched.push_back(kb);
        }
        if (group_cnt[kb] == BN) full_groups[kb]++;
        group_cnt[kb] = 0;
      }
    }
    // Full blocks first (increasing), then partial blocks (increasing): the
    // kernels run the full blocks in a software-pipelined loop without any
    // mask arithmetic and the few partial ones after them.
    std::sort(touched.begin(), touched.end(), [&](int a, int b) {
      const bool fa = full_groups[a] == n_tile_groups, fb = full_groups[b] == n_tile_groups;
      return fa != fb ? fa : a < b;
    });
    int32_t n_full = 0;
    for (int kb : touched) n_full += full_groups[kb] == n_tile_groups;
    s.tile_nfull.push_back(n_full);
    for (int kb : touched) {
      const bool full = full_groups[kb] == n_tile_groups;
      s.entry_block.push_back(kb);
      if (full) {
        s.entry_partial.push_back(-1);
      } else {
        s.entry_partial.push_back(int32_t(s.n_partial));
        s.n_partial++;
        size_t base = s.partial_bits.size();
        s.partial_bits.resize(base + size_t(BM) * words, 0u);
        const int k0 = kb * BN, k1 = k0 + BN;
        for (int g = g0; g < g1; ++g) {
          const int gr0 = std::max(r0, m->group_q_begin[g]);
          const int gr1 = std::min(r1, m->group_q_begin[g + 1]);
          for (int r = m->range_ptr[g]; r < m->range_ptr[g + 1]; ++r) {
            int lo = std::max(k0, m->k_begin[r]), hi = std::min(k1, m->k_end[r]);
            for (int key = lo; key < hi; ++key) {
              const int w = (key - k0) >> 5, bit = (key - k0) & 31;
              for (int row = gr0; row < gr1; ++row)
                s.partial_bits[base + size_t(row - r0) * words + w] |= 1u << bit;
            }
          }
        }
      }
      any_group[kb] = 0;
      full_groups[kb] = 0;
    }
    s.tile_offsets.push_back(int32_t(s.entry_block.size()));
  }
  s.tile_order.resize(n_tiles);
  for (int t = 0; t < n_tiles; ++t) s.tile_order[t] = t;
  std::stable_sort(s.tile_order.begin(), s.tile_order.end(), [&](int a, int b) {
    return s.tile_offsets[a + 1] - s.tile_offsets[a] > s.tile_offsets[b + 1] - s.tile_offsets[b];
  });
}

const HostSchedule *host_schedule_locked(const attn_jvp_mask *m, int block_m, int block_n,
                                         int *status) {
  auto key = std::make_pair(block_m, block_n);
  auto it = m->host_sched.find(key);
  if (it != m->host_sched.end()) {
    *status = ATTN_JVP_OK;
    return &it->second;
  }
  // entry and partial-block indices are 32-bit on the device
  if (count_entries(m, block_m, block_n) > int64_t(kMaxScheduleEntries)) {
    *status = ATTN_JVP_ERR_SHAPE;
    return nullptr;
  }
  try {
    HostSchedule s;
    build_schedule(m, block_m, block_n, s);
    auto res = m->host_sched.emplace(key, std::move(s));
    *status = ATTN_JVP_OK;
    return &res.first->second;
  } catch (const std::bad_alloc &) {
    *status = ATTN_JVP_ERR_OOM;
    return nullptr;
  }
}

int split_schedule(const HostSchedule &s, int max_splits, HostSplit *out) {
  if (max_splits < 1) return ATTN_JVP_ERR_SHAPE;
  try {
    HostSplit h;
    int32_t longest = 0;
    for (int t = 0; t < s.n_tiles; ++t)
      longest = std::max(longest, s.tile_offsets[t + 1] - s.tile_offsets[t]);
    h.unit_len = std::max<int32_t>(1, (longest + max_splits - 1) / max_splits);
    h.unit_offsets.assign(1, 0);
    for (int t = 0; t < s.n_tiles; ++t) {
      const int32_t e0 = s.tile_offsets[t], n = s.tile_offsets[t + 1] - e0;
      const int32_t k = std::max<int32_t>(1, (n + h.unit_len - 1) / h.unit_len);
      // k near-equal consecutive runs (the first n % k one entry longer)
      for (int32_t u = 0; u < k; ++u) {
        h.unit_tile.push_back(t);
        h.unit_part.push_back(k > 1 ? h.n_parts + u : -1);
        h.unit_offsets.push_back(e0 + int32_t((int64_t(n) * (u + 1)) / k));
      }
      if (k > 1) {
        h.split_tiles.insert(h.split_tiles.end(), {t, h.n_parts, k, 0});
        h.n_parts += k;
      }
    }
    h.n_units = int32_t(h.unit_tile.size());
    h.unit_order.resize(h.n_units);
    for (int u = 0; u < h.n_units; ++u) h.unit_order[u] = u;
    std::stable_sort(h.unit_order.begin(), h.unit_order.end(), [&](int a, int b) {
      return h.unit_offsets[a + 1] - h.unit_offsets[a] > h.unit_offsets[b + 1] - h.unit_offsets[b];
    });
    *out = std::move(h);
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  return ATTN_JVP_OK;
}

const HostSplit *host_split_locked(const attn_jvp_mask *m, int block_m, int block_n,
                                   int max_splits, int *status) {
  auto key = std::make_tuple(block_m, block_n, max_splits);
  auto it = m->host_split.find(key);
  if (it != m->host_split.end()) {
    *status = ATTN_JVP_OK;
    return &it->second;
  }
  const HostSchedule *s = host_schedule_locked(m, block_m, block_n, status);
  if (!s) return nullptr;
  HostSplit h;
  *status = split_schedule(*s, max_splits, &h);
  if (*status != ATTN_JVP_OK) return nullptr;
  try {
    auto res = m->host_split.emplace(key, std::move(h));
    return &res.first->second;
  } catch (const std::bad_alloc &) {
    *status = ATTN_JVP_ERR_OOM;
    return nullptr;
  }
}

}  // namespace attnjvp

extern "C" int attn_jvp_mask_split_schedule(const attn_jvp_mask *m, int32_t block_m,
                                            int32_t block_n, int32_t max_splits,
                                            int32_t *n_units, int32_t *n_parts,
                                            int32_t *unit_offsets, int32_t *unit_order,
                                            int32_t *unit_tile, int32_t *unit_part) {
  if (!m || !n_units || !n_parts) return ATTN_JVP_ERR_NULL;
  if (block_m <= 0 || block_n <= 0 || block_n % 32 || block_m > 4096 || block_n > 4096 ||
      max_splits < 1)
    return ATTN_JVP_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(m->mu);
  int st = ATTN_JVP_OK;
  const attnjvp::HostSplit *hp = attnjvp::host_split_locked(m, block_m, block_n, max_splits, &st);
  if (!hp) return st;
  const attnjvp::HostSplit &h = *hp;
  *n_units = h.n_units;
  *n_parts = h.n_parts;
  if (unit_offsets) std::copy(h.unit_offsets.begin(), h.unit_offsets.end(), unit_offsets);
  if (unit_order) std::copy(h.unit_order.begin(), h.unit_order.end(), unit_order);
  if (unit_tile) std::copy(h.unit_tile.begin(), h.unit_tile.end(), unit_tile);
  if (unit_part) std::copy(h.unit_part.begin(), h.unit_part.end(), unit_part);
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_schedule(const attn_jvp_mask *m, int32_t block_m, int32_t block_n,
                                      int32_t *n_tiles, int64_t *n_entries, int64_t *n_partial,
                                      int32_t *tile_offsets, int32_t *tile_order,
                                      int32_t *entry_block, int32_t *entry_partial,
                                      uint32_t *partial_bits) {
  if (!m || !n_tiles || !n_entries || !n_partial) return ATTN_JVP_ERR_NULL;
  if (block_m <= 0 || block_n <= 0 || block_n % 32 || block_m > 4096 || block_n > 4096)
    return ATTN_JVP_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(m->mu);
  int st = ATTN_JVP_OK;
  const HostSchedule *s = attnjvp::host_schedule_locked(m, block_m, block_n, &st);
  if (!s) return st;
  *n_tiles = s->n_tiles;
  *n_entries = int64_t(s->entry_block.size());
  *n_partial = s->n_partial;
  if (tile_offsets) std::copy(s->tile_offsets.begin(), s->tile_offsets.end(), tile_offsets);
  if (tile_order) std::copy(s->tile_order.begin(), s->tile_order.end(), tile_order);
  if (entry_block) std::copy(s->entry_block.begin(), s->entry_block.end(), entry_block);
  if (entry_partial) std::copy(s->entry_partial.begin(), s->entry_partial.end(), entry_partial);
  if (partial_bits) std::copy(s->partial_bits.begin(), s->partial_bits.end(), partial_bits);
  return ATTN_JVP_OK;
}

extern "C" int attn_jvp_mask_transpose(const attn_jvp_mask *m, attn_jvp_mask **out) {
  if (!m || !out) return ATTN_JVP_ERR_NULL;
  return attnjvp::transpose_mask(m, out);
}
