// Fused primal + tangent masked attention for gfx950 (bf16 in, fp32 accumulate).
//
// One online-softmax pass computes O, LSE and dO ("Causal-rCM ..." summary,
// Appendix B: the tangent rides the primal FlashAttention pass with shared
// rescaling, masked pairs carry no tangent, one sparse schedule of admissible
// key blocks serves the primal and the tangent scores).  Per query row the
// pass keeps the running max m, the sum l of exp(s - m), the sum mu of
// exp(s - m) * ds, and two D-wide accumulators
//     A = sum exp(s - m) v,   T = sum exp(s - m) (ds v + dv),
// all rescaled by the same factor exp(m_old - m_new) when m grows, and ends
// with O = A / l, dO = T / l - O * (mu / l), LSE = m + ln l.
//
// Work decomposition (MI355X-first):
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows, one lane per row in each half-wave, so per-row softmax
//    state lives in a lane and only the two half-waves need a swap;
//  * scores are computed transposed, S^T = K Q^T and dS^T = K dQ^T + dK Q^T,
//    with v_mfma_f32_32x32x16_bf16: K / dK come from LDS as the A operand, Q
//    and dQ stay in registers as the B operand for the whole key loop;
//  * the accumulators are transposed too, A^T += V^T P^T and
//    T^T += V^T (P*dS)^T + dV^T P^T, so the MFMA output of the score step is
//    already the B operand of the value step (no shuffle of P);
//  * V and dV are transposed once while being staged into LDS (4 keys x 8
//    dims per thread, repacked in registers), so every MFMA operand read is a
//    single 16-byte LDS load; K rows are read in a permuted order (bits 2 and
//    3 of the row swapped) so that each lane's 8 probabilities of a 16-key
//    step are 8 consecutive keys of V^T;
//  * key blocks of 32 are double-buffered in LDS; the next block's global
//    loads are in flight while the current block is computed;
//  * full blocks run without any mask arithmetic; partial blocks read one
//    32-bit word of admissible-key bits per row;
//  * workgroups are renumbered so that the ones the dispatcher places on one
//    XCD are consecutive tiles of the same (batch, head), heaviest first:
//    they stream the same key blocks through that XCD's L2.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attnjvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BM = kBf16BlockM;  // 128 query rows per workgroup
constexpr int BN = kBf16BlockN;  // 32 keys per block
static_assert(BM == 128 && BN == 32, "kernel layout assumes 4 waves x 32 rows, 32-key blocks");

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// Position of K row m of the 32x32 score tile: bits 2 and 3 swapped.  The
// MFMA output element (row 8j + 4h + i) then holds key 16(j/2) + 8h + 4(j%2) + i,
// so lane-half h owns keys 16s + 8h + 0..7 of value step s, in register order.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte-chunk XOR swizzles of the LDS tiles (bank spread for the MFMA
// operand reads, where 16 or 32 lanes read one chunk column of many rows).
template <int D>
__device__ __forceinline__ int k_chunk(int row, int c) {
  constexpr int KCH = D / 8;
  return row * KCH + (c ^ ((row ^ (row >> 3)) & (KCH - 1)));
}
__device__ __forceinline__ int vt_chunk(int d, int c) {
  constexpr int VCH = BN / 8;  // 4 chunks per V^T row
  return d * VCH + (c ^ (((d >> 1) ^ (d >> 3)) & (VCH - 1)));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float *x) {
  uint4 u;
  u.x = pack_bf16(x[0], x[1]);
  u.y = pack_bf16(x[2], x[3]);
  u.z = pack_bf16(x[4], x[5]);
  u.w = pack_bf16(x[6], x[7]);
  return as_bf16x8(u);
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// Workgroup w is dispatched to XCD w % 8.  Renumber so that each XCD receives
// a contiguous range of logical work items.
__device__ __forceinline__ int xcd_logical(int w, int G) {
  const int xcd = w & 7, local = w >> 3;
  const int q = G >> 3, r = G & 7;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int D>
struct Stage {
  // Per-thread registers holding one key block on its way to LDS.
  static constexpr int KCH = D / 8;                     // chunks per K row
  static constexpr int K_CHUNKS = BN * KCH;             // per tensor
  static constexpr int K_PER_THREAD = (K_CHUNKS + kThreads - 1) / kThreads;
  static constexpr int V_UNITS = (BN / 4) * KCH;        // 4 keys x 8 dims
  static constexpr int V_PER_THREAD = (2 * V_UNITS + kThreads - 1) / kThreads;
  static_assert(K_CHUNKS % kThreads == 0, "K staging must tile the workgroup");
  static_assert(V_PER_THREAD == 1, "one V or dV unit per thread");
  uint4 k[K_PER_THREAD], dk[K_PER_THREAD];
  uint4 v[4];
};

template <int D, bool TAN>
__device__ __forceinline__ void load_block(Stage<D> &st, const KernelParams &p,
                                           const __bf16 *kb_, const __bf16 *dkb_,
                                           const __bf16 *vb_, const __bf16 *dvb_, int key0) {
  constexpr int KCH = D / 8;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D>::K_PER_THREAD; ++i) {
    const int id = tid + i * kThreads;
    const int row = id / KCH, c = id % KCH;
    const int key = key0 + row;
    uint4 z = {0u, 0u, 0u, 0u};
    if (key < p.n_k) {
      st.k[i] = *reinterpret_cast<const uint4 *>(kb_ + int64_t(key) * p.k_sn + c * 8);
      if (TAN) st.dk[i] = *reinterpret_cast<const uint4 *>(dkb_ + int64_t(key) * p.k_sn + c * 8);
    } else {
      st.k[i] = z;
      if (TAN) st.dk[i] = z;
    }
  }
  // V / dV: thread u < V_UNITS handles V, the next V_UNITS handle dV.
  const int u = tid;
  if (u < 2 * Stage<D>::V_UNITS && (TAN || u < Stage<D>::V_UNITS)) {
    const bool is_dv = u >= Stage<D>::V_UNITS;
    const int uu = is_dv ? u - Stage<D>::V_UNITS : u;
    const int kg = uu / KCH, c = uu % KCH;
    const __bf16 *base = is_dv ? dvb_ : vb_;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * kg + r;
      uint4 z = {0u, 0u, 0u, 0u};
      st.v[r] = key < p.n_k ? *reinterpret_cast<const uint4 *>(base + int64_t(key) * p.k_sn + c * 8) : z;
    }
  }
}

template <int D, bool TAN>
__device__ __forceinline__ void store_block(const Stage<D> &st, uint4 *lds) {
  constexpr int KCH = D / 8;
  constexpr int TILE = BN * D / 8;  // chunks per tensor tile
  uint4 *Ks = lds, *dKs = lds + TILE, *Vt = lds + 2 * TILE, *dVt = lds + 3 * TILE;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D>::K_PER_THREAD; ++i) {
    const int id = tid + i * kThreads;
    const int row = id / KCH, c = id % KCH;
    Ks[k_chunk<D>(row, c)] = st.k[i];
    if (TAN) dKs[k_chunk<D>(row, c)] = st.dk[i];
  }
  const int u = tid;
  if (u < 2 * Stage<D>::V_UNITS && (TAN || u < Stage<D>::V_UNITS)) {
    const bool is_dv = u >= Stage<D>::V_UNITS;
    const int uu = is_dv ? u - Stage<D>::V_UNITS : u;
    const int kg = uu / KCH, c = uu % KCH;
    uint4 *dst = is_dv ? dVt : Vt;
    // 4 keys x 8 dims -> 8 rows (dims) of 4 keys: rows 8c + e, keys 4kg..4kg+3
    const uint32_t w[4][4] = {{st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w},
                              {st.v[1].x, st.v[1].y, st.v[1].z, st.v[1].w},
                              {st.v[2].x, st.v[2].y, st.v[2].z, st.v[2].w},
                              {st.v[3].x, st.v[3].y, st.v[3].z, st.v[3].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int wi = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (w[0][wi] >> 16) | (w[1][wi] & 0xffff0000u);
        hi = (w[2][wi] >> 16) | (w[3][wi] & 0xffff0000u);
      } else {
        lo = (w[0][wi] & 0xffffu) | (w[1][wi] << 16);
        hi = (w[2][wi] & 0xffffu) | (w[3][wi] << 16);
      }
      const int d = 8 * c + e;
      uint2 *row = reinterpret_cast<uint2 *>(dst + vt_chunk(d, kg >> 1));
      row[kg & 1] = make_uint2(lo, hi);
    }
  }
}

template <int D, bool TAN, bool PARTIAL>
__device__ __forceinline__ void compute_block(const uint4 *lds, const bf16x8 *qf, const bf16x8 *dqf,
                                              f32x16 *accO, f32x16 *accT, float &m_run, float &l_run,
                                              float &mu_run, uint32_t bits, float scale_log2,
                                              float scale) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = BN * D / 8;
  const uint4 *Ks = lds, *dKs = lds + TILE, *Vt = lds + 2 * TILE, *dVt = lds + 3 * TILE;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int krow = swap_bits23(col);

  f32x16 S = {}, dS = {};
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    const int c = 2 * t + hh;
    const bf16x8 kf = as_bf16x8(Ks[k_chunk<D>(krow, c)]);
    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], S, 0, 0, 0);
    if (TAN) {
      const bf16x8 dkf = as_bf16x8(dKs[k_chunk<D>(krow, c)]);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, dqf[t], dS, 0, 0, 0);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dkf, qf[t], dS, 0, 0, 0);
    }
  }

  float s[16];
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = r >> 2, i = r & 3;
    const int key = 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
    bool ok = true;
    if (PARTIAL) ok = (bits >> key) & 1u;
    s[r] = ok ? S[r] * scale_log2 : kNegInf;
    mx = fmaxf(mx, s[r]);
  }
  mx = fmaxf(mx, xor32(mx));
  const float m_new = fmaxf(m_run, mx);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  float pr[16], pds[16];
  float lsum = 0.f, musum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
    lsum += pr[r];
    if (TAN) {
      const int j = r >> 2, i = r & 3;
      const int key = 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
      bool ok = true;
      if (PARTIAL) ok = (bits >> key) & 1u;
      const float ds = ok ? dS[r] * scale : 0.f;
      pds[r] = pr[r] * ds;
      musum += pds[r];
    }
  }
  l_run = l_run * alpha + lsum;
  if (TAN) mu_run = mu_run * alpha + musum;
  m_run = m_new;

  bf16x8 pb[2], pdsb[2];
  pb[0] = to_bf16x8(pr);
  pb[1] = to_bf16x8(pr + 8);
  if (TAN) {
    pdsb[0] = to_bf16x8(pds);
    pdsb[1] = to_bf16x8(pds + 8);
  }
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    accO[nt] *= alpha;
    if (TAN) accT[nt] *= alpha;
  }
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int c = 2 * st + hh;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const int d = 32 * nt + col;
      const bf16x8 vf = as_bf16x8(Vt[vt_chunk(d, c)]);
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[st], accO[nt], 0, 0, 0);
      if (TAN) {
        const bf16x8 dvf = as_bf16x8(dVt[vt_chunk(d, c)]);
        accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pdsb[st], accT[nt], 0, 0, 0);
        accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dvf, pb[st], accT[nt], 0, 0, 0);
      }
    }
  }
}

template <int D, bool TAN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_jvp_bf16_kernel(KernelParams p) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = BN * D / 8;
  __shared__ uint4 smem[2 * 4 * TILE];

  const int G = p.n_tiles * p.B * p.H;
  const int L = xcd_logical(int(blockIdx.x), G);
  const int slot = L % p.n_tiles;
  const int bh = L / p.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int tile = p.tile_order[slot];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int row_in_tile = wave * 32 + col;
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;

  const __bf16 *qb = static_cast<const __bf16 *>(p.q) + int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;
  const __bf16 *dqb = static_cast<const __bf16 *>(p.dq) + int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;
  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + koff;
  const __bf16 *vb_ = static_cast<const __bf16 *>(p.v) + koff;
  const __bf16 *dkb_ = TAN ? static_cast<const __bf16 *>(p.dk) + koff : nullptr;
  const __bf16 *dvb_ = TAN ? static_cast<const __bf16 *>(p.dv) + koff : nullptr;

  bf16x8 qf[KSTEPS], dqf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    uint4 z = {0u, 0u, 0u, 0u};
    const int64_t off = int64_t(qrow) * p.q_sn + 16 * t + 8 * hh;
    qf[t] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4 *>(qb + off) : z);
    if (TAN) dqf[t] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4 *>(dqb + off) : z);
  }

  f32x16 accO[DT], accT[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    accO[nt] = f32x16{};
    accT[nt] = f32x16{};
  }
  float m_run = kNegInf, l_run = 0.f, mu_run = 0.f;

  const int e0 = p.tile_offsets[tile], e1 = p.tile_offsets[tile + 1];
  if (e0 < e1) {
    Stage<D> st;
    load_block<D, TAN>(st, p, kb_, dkb_, vb_, dvb_, p.entries[e0].x * BN);
    store_block<D, TAN>(st, smem);
    __syncthreads();
    for (int e = e0; e < e1; ++e) {
      const int stage = (e - e0) & 1;
      const int2 ent = p.entries[e];
      const bool has_next = e + 1 < e1;
      if (has_next) load_block<D, TAN>(st, p, kb_, dkb_, vb_, dvb_, p.entries[e + 1].x * BN);
      const uint4 *lds = smem + stage * 4 * TILE;
      if (ent.y >= 0) {
        const uint32_t bits = p.partial_bits[int64_t(ent.y) * BM + row_in_tile];
        compute_block<D, TAN, true>(lds, qf, dqf, accO, accT, m_run, l_run, mu_run, bits,
                                    p.scale_log2, p.scale);
      } else {
        compute_block<D, TAN, false>(lds, qf, dqf, accO, accT, m_run, l_run, mu_run, ~0u,
                                     p.scale_log2, p.scale);
      }
      if (has_next) store_block<D, TAN>(st, smem + (stage ^ 1) * 4 * TILE);
      __syncthreads();
    }
  }

  const float l_tot = l_run + xor32(l_run);
  const float mu_tot = TAN ? mu_run + xor32(mu_run) : 0.f;
  if (!qvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float mu_n = mu_tot * inv;
  if (hh == 0) {
    p.lse[(int64_t(batch) * p.H + head) * p.n_q + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
  __bf16 *ob = static_cast<__bf16 *>(p.o) + int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh +
               int64_t(qrow) * p.q_sn;
  __bf16 *dob = TAN ? static_cast<__bf16 *>(p.d_o) + int64_t(batch) * p.q_sb +
                          int64_t(head) * p.q_sh + int64_t(qrow) * p.q_sn
                    : nullptr;
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * nt + 8 * j + 4 * hh;
      float o[4], dout[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = accO[nt][4 * j + i] * inv;
        if (TAN) dout[i] = accT[nt][4 * j + i] * inv - o[i] * mu_n;
      }
      *reinterpret_cast<uint2 *>(ob + d0) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
      if (TAN)
        *reinterpret_cast<uint2 *>(dob + d0) =
            make_uint2(pack_bf16(dout[0], dout[1]), pack_bf16(dout[2], dout[3]));
    }
  }
}

template <int D, bool TAN>
hipError_t launch(const KernelParams &p, hipStream_t stream) {
  const int64_t G = int64_t(p.n_tiles) * p.B * p.H;
  hipLaunchKernelGGL((attn_jvp_bf16_kernel<D, TAN>), dim3(unsigned(G)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int launch_bf16(const KernelParams &p, int D, bool tangent, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return tangent ? launch<128, true>(p, s) : launch<128, false>(p, s);
  if (D == 64) return tangent ? launch<64, true>(p, s) : launch<64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
