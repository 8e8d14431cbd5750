// Fused primal + tangent masked attention for gfx950, head dims 64 and 128
// (bf16 in, fp32 accumulate).
//
// One online-softmax pass computes O, LSE and dO ("Causal-rCM ..." summary,
// Appendix B: the tangent rides the primal FlashAttention pass with shared
// rescaling, masked pairs carry no tangent, one sparse schedule of admissible
// key blocks serves the primal and the tangent scores).  Per query row the
// pass keeps a reference max m, the sum l of exp(s - m), the sum mu of
// exp(s - m) * ds, and two D-wide accumulators
//     A = sum exp(s - m) v,   T = sum exp(s - m) (ds v + dv),
// all rescaled by the same factor exp(m_old - m_new) when m moves, and ends
// with O = A / l, dO = T / l - O * (mu / l), LSE = m + ln l.
//
// Work decomposition (MI355X-first):
//  * one workgroup = 8 waves = 256 query rows of one (batch, head), two waves
//    per SIMD: while one wave of a SIMD runs its vector-ALU softmax, scalar
//    and LDS work, the other keeps the matrix core busy (one wave alone
//    cannot: an MFMA holds its own wave's issue for about half its run time);
//  * each wave owns 32 rows, one lane per row in each half-wave, so the
//    per-row softmax state lives in a lane and only the two half-waves
//    exchange the row max (and only when it moves);
//  * scores are computed transposed, S^T = K Q^T and dS^T = K dQ^T + dK Q^T,
//    with v_mfma_f32_32x32x16_bf16: K / dK from LDS as the A operand, Q in
//    registers and dQ in LDS (staged once per tile) as the B operand;
//  * the accumulators are transposed too, A^T += V^T P^T and
//    T^T += V^T (P*dS)^T + dV^T P^T, so the MFMA output of the score step is
//    already the B operand of the value step (no shuffle of P); K rows are
//    read in a permuted order (bits 2 and 3 of the row swapped) so that each
//    lane's 8 probabilities of a 16-key step are 8 consecutive keys;
//  * V and dV stay row-major in LDS; the transposed V^T operand comes from
//    ds_read_b64_tr_b16 (each group of 16 lanes turns 4 keys x 16 dims into
//    16 lanes x 4 keys);
//  * key blocks of 32 rows of K, dK, V, dV (and the admissible-key bits of
//    the block) go HBM -> LDS with direct-to-LDS loads, 16 bytes per lane per
//    copy, into a 2-stage ring: block j + 1 is copied while block j is
//    computed; tiles are XOR-swizzled in 16-byte chunks so the operand reads
//    hit distinct banks.  The head-dim-128 primal-only kernel, which has the
//    registers for two score tiles, takes blocks of 64 keys, halving the
//    per-block barrier, copy and schedule work per key;
//  * head dim 64 runs the same code with half the k-steps and output tiles
//    (and 128-byte rows: other swizzles, two tensors per copy round);
//  * every value lives in the 256 VGPRs a wave has at two waves per SIMD
//    (accumulators included, so the rare rescale is plain vector code); the
//    reference max moves only when a row max exceeds it by more than 2^16, so
//    p = exp2(s - m) stays below 2^16, far inside fp32 and bf16 range (bf16
//    keeps 8 significant bits at any magnitude);
//  * workgroups are mapped to work so that each XCD receives an equal share
//    of every group of (batch, head) slices, as interleaved heavy-first tile
//    slots, while the workgroups resident on one XCD at a time belong to the
//    same slice and stream the same key blocks through that XCD's L2
//    (work_item).
#include <hip/hip_runtime.h>

#include <cstddef>

#include "internal.h"

namespace attnjvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int BM = kBf16BlockMWide;  // 256 query rows per workgroup
constexpr int BN = kBf16BlockN;      // 32 keys per block
constexpr int kStages = 2;           // block j + 1 is copied while block j is computed
static_assert(BM == 32 * kWaves && BN == 32, "one wave per 32 rows, 32-key blocks");

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 16.0f;  // log2 units: p <= 2^16 between rescales
constexpr int kEntChunk = 512;        // schedule entries staged in LDS at a time

// Per head dim: 16-byte chunks per row, 16-wide k-steps, 32-wide output tiles.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int KCH = D / 8;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE = BN * KCH;  // chunks of one 32-row tile
};

// Keys per block: 32, or 64 for the head-dim-128 primal kernel (two score
// tiles per block: half the barriers and per-block scalar work per key, and
// two independent score chains).  The host builds the schedule for the same
// width (attn_jvp_tile_shape).
template <int D, bool TAN>
constexpr int kBlockN = (!TAN && D == 128) ? 64 : 32;
static_assert(kBlockN<128, false> == kBf16BlockNPrimal128, "host and kernel block widths");

template <int D, bool TAN>
struct alignas(16) StageTile {
  uint4 k[Geo<D>::TILE];
  uint4 dk[Geo<D>::TILE];
  uint4 v[Geo<D>::TILE];
  uint4 dv[Geo<D>::TILE];
  uint32_t bits[BM];
};
template <int D>
struct alignas(16) StageTile<D, false> {  // primal: no tangent tiles
  static constexpr int W = kBlockN<D, false> / 32;  // mask words per row
  uint4 k[W * Geo<D>::TILE];
  uint4 v[W * Geo<D>::TILE];
  uint32_t bits[BM * W];
};
// LDS byte offset of tensor t (0 K, 1 V, 2 dK, 3 dV) inside a stage.
template <int D, bool TAN>
constexpr uint32_t tile_offset(int t) {
  using ST = StageTile<D, TAN>;
  if constexpr (TAN)
    return uint32_t(t == 0 ? offsetof(ST, k) : t == 1 ? offsetof(ST, v)
                    : t == 2 ? offsetof(ST, dk) : offsetof(ST, dv));
  else
    return uint32_t(t == 0 ? offsetof(ST, k) : offsetof(ST, v));
}

// Position of K row m of the 32x32 score tile: bits 2 and 3 swapped.  The
// MFMA output element (row 8j + 4h + i) then holds key 16(j/2) + 8h + 4(j%2) + i,
// so lane-half h owns keys 16s + 8h + 0..7 of value step s, in register order.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// 16-byte-chunk XOR swizzles, with 64 banks of 4 bytes: row-operand reads
// (K, dK, dQ; ds_read_b128, 16 lanes per cycle) touch 16 aligned rows at one
// chunk; transposed reads (V, dV; ds_read_b64_tr_b16, 32 lanes per cycle)
// touch 4 aligned consecutive rows x 4 consecutive chunks.  Head dim 128
// (256-byte rows): one swizzle for each access; head dim 64 (128-byte rows,
// two per bank cycle): one swizzle conflict-free for both (a bijection of 0..7
// within each row parity over 16 rows whose top bit differs between rows 4a
// and 4a+2).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : (4 * ((row >> 1) & 1) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : (4 * ((row >> 1) & 1) | ((row >> 2) & 3));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Round to nearest even, two values per v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x8 to_bf16x8(const float *x) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// 16 bytes per lane from global memory (wave-uniform base + per-lane byte
// offset) straight into LDS at lds_wave + 16 * lane (lds_wave wave-uniform).
// Tracked by vmcnt; the kernel waits for it explicitly before the barrier that
// publishes a stage.  One wait state separates the M0 write from the copy.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_wave) {
  lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);  // wave-uniform: keep it scalar
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_wave)
               : "memory", "m0");
}
// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0): this wave's LDS writes are done, so a following
// s_barrier publishes them to the workgroup (the compiler adds no such wait
// before a bare s_barrier).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// A zero row: the copy source of an absent (zero) tangent tensor, read with
// row-independent offsets.
__device__ __align__(16) uint4 kZeroRow[16];

// Per-lane byte offsets of chunk c of a 32-row tile (K-swizzled, V-swizzled).
struct DmaOffsets {
  uint32_t k, v;
};
template <int D>
__device__ __forceinline__ DmaOffsets dma_offsets(int c, int64_t k_sn, int rows_valid) {
  constexpr int KCH = Geo<D>::KCH;
  const int row = c / KCH, pch = c % KCH;
  const uint32_t roff = uint32_t(min(row, rows_valid - 1)) * uint32_t(k_sn) * 2u;
  return {roff + uint32_t(pch ^ k_swz<D>(row)) * 16u, roff + uint32_t(pch ^ v_swz<D>(row)) * 16u};
}

// Issue the direct-to-LDS copies of the key block starting at key key0 into
// the stage tile at LDS byte address st.  The block's tensors (K, V, then dK,
// dV) are consecutive runs of Geo<D>::TILE chunks; copy i of wave w fills the
// 64 chunks from i * 512 + 64 w, which lie inside one tensor (head dim 128:
// one copy per tensor per wave; head dim 64: waves 0-3 and 4-7 take the two
// tensors of a pair).
template <int D, bool TAN>
__device__ __forceinline__ void issue_block(uint32_t st, int wave, const KernelParams &p,
                                            const __bf16 *kb_, const __bf16 *dkb_,
                                            const __bf16 *vb_, const __bf16 *dvb_, int key0,
                                            const uint32_t *bits_src) {
  using ST = StageTile<D, TAN>;
  constexpr int TILE = Geo<D>::TILE;
  constexpr int COPIES = (TAN ? 4 : 2) * TILE / kThreads;
  const int lane = threadIdx.x & 63;
  const int64_t boff = int64_t(key0) * p.k_sn;
  // rebuilt per block (cheaper than holding them in registers); rows past n_k
  // re-read the last key, masked out by the schedule
  const int rows_valid = min(kBlockN<D, TAN>, p.n_k - key0);
  if constexpr (kBlockN<D, TAN> == 64) {
    // 64 rows of K and V: two copies per tensor per wave; mask bits: BM x 2
    // words = 128 chunks, wave w copies chunks 16w .. 16w+15 (lanes 0..15)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const DmaOffsets o = dma_offsets<D>(i * kThreads + int(threadIdx.x), p.k_sn, rows_valid);
      const uint32_t chunk = uint32_t(i * kThreads + wave * 64) * 16u;
      dma16(kb_ + boff, o.k, st + uint32_t(offsetof(ST, k)) + chunk);
      dma16(vb_ + boff, o.v, st + uint32_t(offsetof(ST, v)) + chunk);
    }
    if (lane < 16)
      dma16(bits_src, uint32_t(wave * 16 + lane) * 16u,
            st + uint32_t(offsetof(ST, bits)) + uint32_t(wave) * 256u);
    return;
  } else if constexpr (D == 128) {
    // one copy per tensor per wave, all at this lane's chunk: one offset pair
    // serves the four tensors (the general loop below compiles slower here)
    const DmaOffsets o = dma_offsets<D>(int(threadIdx.x), p.k_sn, rows_valid);
    const uint32_t chunk = uint32_t(wave * 64) * 16u;
    dma16(kb_ + boff, o.k, st + tile_offset<D, TAN>(0) + chunk);
    dma16(vb_ + boff, o.v, st + tile_offset<D, TAN>(1) + chunk);
    if constexpr (TAN) {
      // an absent tangent tensor is zero: copy the zero row into every row
      const DmaOffsets oz = dma_offsets<D>(int(threadIdx.x), 0, 1);
      const bool zk = dkb_ == nullptr, zv = dvb_ == nullptr;
      dma16(zk ? static_cast<const void *>(kZeroRow) : dkb_ + boff, zk ? oz.k : o.k,
            st + tile_offset<D, TAN>(2) + chunk);
      dma16(zv ? static_cast<const void *>(kZeroRow) : dvb_ + boff, zv ? oz.v : o.v,
            st + tile_offset<D, TAN>(3) + chunk);
    }
  } else {
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
      const int c0 = i * kThreads + wave * 64;  // wave-uniform
      const int t = c0 / TILE;                  // 0 K, 1 V, 2 dK, 3 dV
      const int c = c0 % TILE + lane;
      const uint32_t dst = st + uint32_t(c0 % TILE) * 16u + tile_offset<D, TAN>(t);
      // an absent tangent tensor is zero: copy the zero row into every row
      const __bf16 *src = t == 0 ? kb_ : t == 1 ? vb_ : t == 2 ? dkb_ : dvb_;
      if (src == nullptr) {
        const DmaOffsets oz = dma_offsets<D>(c, 0, 1);
        dma16(kZeroRow, (t & 1) ? oz.v : oz.k, dst);
      } else {
        const DmaOffsets o = dma_offsets<D>(c, p.k_sn, rows_valid);
        dma16(src + boff, (t & 1) ? o.v : o.k, dst);
      }
    }
  }
  // mask bits: BM words = 64 chunks; wave w copies chunks 8w .. 8w+7 (lanes 0..7)
  if (lane < 8)
    dma16(bits_src, uint32_t(wave * 8 + lane) * 16u,
          st + uint32_t(offsetof(ST, bits)) + uint32_t(wave) * 128u);
}

// Key-loop code shape: every kernel holds its per-lane LDS read offsets
// across the key loop and runs the loop unrolled by two, so that each block's
// ring stage is an immediate offset of those reads (primal kernels -7 %,
// head-dim-64 JVP kernel -17 %, head-dim-128 JVP kernel -3 %).  The
// head-dim-128 JVP kernel writes its score-phase row reads as one xor-add
// each (below), which is what leaves it the registers to do so.
template <int D, bool TAN>
constexpr bool kXadReads = D == 128 && TAN;

// Row-operand read of chunk (2t + hh) ^ x of a row, as an index or as the
// byte offset 32 t ^ y, y = 16 (hh ^ x): one xor-add per read with the step's
// constant (fewer vector instructions and registers in the head-dim-128 JVP
// kernel; 1 % slower in the head-dim-64 one).
template <bool XAD>
__device__ __forceinline__ bf16x8 row_read(const uint4 *row, int t, int hh, int x, uint32_t y) {
  if constexpr (XAD)
    return as_bf16x8(*reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(row) +
                                                      ((32u * uint32_t(t)) ^ y)));
  else
    return as_bf16x8(row[(2 * t + hh) ^ x]);
}

// The dK tile of a stage (JVP kernels only).
template <int D, bool TAN>
__device__ __forceinline__ const uint4 *dk_tile(const StageTile<D, TAN> *st) {
  if constexpr (TAN) return st->dk; else return nullptr;
}

// S^T = K Q^T and dS^T = K dQ^T + dK Q^T; Q from registers, dQ from LDS.
template <int D, bool TAN>
__device__ __forceinline__ void score_block(const StageTile<D, TAN> *st, const uint4 *dq_lds,
                                            const bf16x8 *qf, int row_in_tile, f32x16 &S,
                                            f32x16 &dS) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int krow = swap_bits23(col);
  constexpr int KCH = Geo<D>::KCH, KSTEPS = Geo<D>::KSTEPS;
  const uint4 *Ks = st->k + krow * KCH;
  const uint4 *dKs = dk_tile(st) + krow * KCH;
  const uint4 *dQs = dq_lds + row_in_tile * KCH;
  constexpr bool kXad = kXadReads<D, TAN>;
  const int kx = k_swz<D>(krow), qx = k_swz<D>(row_in_tile);
  const uint32_t ky = 16u * uint32_t(hh ^ kx), qy = 16u * uint32_t(hh ^ qx);
  S = f32x16{};
  dS = f32x16{};
  if constexpr (!TAN) {
    // primal: every K operand of the block read up front (registers allow)
    bf16x8 kfs[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) kfs[t] = row_read<kXad>(Ks, t, hh, kx, ky);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfs[t], qf[t], S, 0, 0, 0);
    return;
  }
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    const bf16x8 kf = row_read<kXad>(Ks, t, hh, kx, ky);
    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], S, 0, 0, 0);
    if (TAN) {
      const bf16x8 dkf = row_read<kXad>(dKs, t, hh, kx, ky);
      const bf16x8 dqf = row_read<kXad>(dQs, t, hh, qx, qy);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, dqf, dS, 0, 0, 0);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dkf, qf[t], dS, 0, 0, 0);
    }
    // bound the operand prefetch: four k-steps (no bound spills), or two in
    // the head-dim-128 JVP kernel (0.5 % faster there)
    constexpr int kFence = (D == 128 && TAN) ? 2 : 4;
    if (t % kFence == kFence - 1) __builtin_amdgcn_sched_barrier(0);
  }
}

// max(a, b, c) as one v_max3_f32.  Through fmaxf the compiler first
// quiets each MFMA result (one v_max_f32 x, x per score: it cannot know they
// are not signalling NaNs) and then forms the tree from two-input maxima; the
// scores here are finite or -inf, for which v_max3_f32 is the exact maximum.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Maximum of n scores (n even) as a v_max3_f32 tree (used by the 64-key
// primal kernel: 3.8 % faster there; the 32-key kernels, whose compiled max
// has few such quieting moves, gain nothing).
template <int n>
__device__ __forceinline__ float max_of(const float *x) {
  float m = max3(x[0], x[1], x[2]);
#pragma unroll
  for (int i = 3; i + 1 < n; i += 2) m = max3(m, x[i], x[i + 1]);
  if constexpr (n % 2 == 0) m = max3(m, x[n - 1], x[n - 1]);
  return m;
}

// Masking of a partial block (inadmissible scores to -inf and, with a
// tangent, their score tangents to 0), the block's row max, and the shared
// rescale of the running sums and accumulators when the reference max moves
// by more than the slack.  Returns the reference max the weights use.
template <int D, bool TAN>
__device__ __forceinline__ float mask_and_rescale(const uint32_t *bits_row, f32x16 &S, f32x16 &dS,
                                                  f32x16 *accO, f32x16 *accT, float &m_ref,
                                                  float &l_run, float &mu_run, bool partial,
                                                  float scale_log2) {
  constexpr int DT = Geo<D>::DT;
  const int hh = (threadIdx.x & 63) >> 5;
  if (partial) {
    // this lane-half's keys 8hh + {0..7, 16..23}, so the bit positions below
    // are constants
    const uint32_t bits = *bits_row >> (8 * hh);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = r >> 2, i = r & 3;
      const int key = 16 * (j >> 1) + 4 * (j & 1) + i;
      const bool ok = (bits >> key) & 1u;
      S[r] = ok ? S[r] : kNegInf;
      if (TAN) dS[r] = ok ? dS[r] : 0.f;
    }
  }
  float mh = S[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mh = fmaxf(mh, S[r]);
  mh *= scale_log2;
  if (__builtin_amdgcn_ballot_w64(mh > m_ref + kRescaleSlack) != 0) {
    const float mx = fmaxf(mh, xor32(mh));
    const bool grow = mx > m_ref + kRescaleSlack;
    const float m_new = grow ? mx : m_ref;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    l_run *= alpha;
    mu_run *= alpha;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      accO[nt] *= alpha;
      if (TAN) accT[nt] *= alpha;
    }
    m_ref = m_new;
  }
  return m_ref == kNegInf ? 0.f : m_ref;
}

// The V^T operands of a block's value step: within each group of 16 lanes,
// lane jl reads keys 16s + 4half + krel at dims d0 + 4(jl % 4) .. +3,
// transposed by ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const uint4 *v_tile, int s, int nt) {
  constexpr int KCH = Geo<D>::KCH;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, jl = lane & 15;
  const int dcol = 16 * (g & 1) + 4 * (jl & 3);
  const int krel = 8 * (lane >> 5) + (jl >> 2);
  const int d = 32 * nt + dcol;
  bf16x4 vh[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int key = 16 * s + 4 * half + krel;
    const int chunk = key * KCH + ((d >> 3) ^ v_swz<D>(key));
    const char *vp = reinterpret_cast<const char *>(v_tile + chunk) + (d & 7) * 2;
    vh[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4 *)(vp));
  }
  return __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// l (and mu) summed from the bf16 weights the value MFMAs consume, two per
// v_dot2 (half the vector instructions of fp32 sums, and O, dO are then
// normalised by exactly the weights they were accumulated with).
__device__ __forceinline__ float sum_bf16x8(const bf16x8 &w, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pp = {w[2 * i], w[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc, false);
  }
  return acc;
}

// Primal: every V operand of the block is read before the softmax (its LDS
// latency hides behind it; the registers allow it), then the weights, then
// A^T += V^T P^T.
template <int D>
__device__ __forceinline__ void softmax_value_primal(const StageTile<D, false> *st, f32x16 S,
                                                     f32x16 *accO, float &m_ref, float &l_run,
                                                     bool partial, int row_in_tile,
                                                     float scale_log2) {
  constexpr int DT = Geo<D>::DT;
  bf16x8 vf[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) vf[s][nt] = v_operand<D>(st->v, s, nt);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 no_dS;
  float no_mu = 0.f;
  const float m_use = mask_and_rescale<D, false>(&st->bits[row_in_tile], S, no_dS, accO, nullptr,
                                                 m_ref, l_run, no_mu, partial, scale_log2);
  float pr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], scale_log2, -m_use));
  bf16x8 pb[2];
  pb[0] = to_bf16x8(pr);
  pb[1] = to_bf16x8(pr + 8);
  l_run += sum_bf16x8(pb[1], sum_bf16x8(pb[0], 0.f));
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s][nt], pb[s], accO[nt], 0, 0, 0);
}

// JVP (head dim 128): mask and rescale over the block, the weights P and
// P*dS of keys 0-15, then their value MFMAs (A^T += V^T P^T, T^T += V^T (P*dS)^T + dV^T P^T)
// interleaved two vector instructions per MFMA with the weights of keys
// 16-31, then those of keys 16-31 with the l and mu sums: the matrix core
// works while the second half of the softmax runs.  The sums see the same
// operations in the same order as a plain softmax-then-MFMA block.
template <int D>
__device__ __forceinline__ void softmax_value_jvp(const StageTile<D, true> *st, f32x16 S,
                                                  f32x16 dS, f32x16 *accO, f32x16 *accT,
                                                  float &m_ref, float &l_run, float &mu_run,
                                                  bool partial, int row_in_tile, float scale_log2,
                                                  float scale) {
  constexpr int DT = Geo<D>::DT;
  const float m_use = mask_and_rescale<D, true>(&st->bits[row_in_tile], S, dS, accO, accT, m_ref,
                                                l_run, mu_run, partial, scale_log2);
  auto weights = [&](int h, bf16x8 &pb, bf16x8 &pdsb) __attribute__((always_inline)) {
    float pr[8], pds[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * h + r], scale_log2, -m_use));
      pds[r] = pr[r] * (dS[8 * h + r] * scale);
    }
    pb = to_bf16x8(pr);
    pdsb = to_bf16x8(pds);
  };
  auto value_step = [&](int s, const bf16x8 &pb, const bf16x8 &pdsb) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const bf16x8 vf = v_operand<D>(st->v, s, nt);
      const bf16x8 dvf = v_operand<D>(st->dv, s, nt);
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, accO[nt], 0, 0, 0);
      accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pdsb, accT[nt], 0, 0, 0);
      accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dvf, pb, accT[nt], 0, 0, 0);
    }
  };
  bf16x8 pb0, pdsb0, pb1, pdsb1;
  if constexpr (D == 64) {
    // head dim 64 (half the MFMAs per block): the plain order is faster
    // (the interleaved one measured 1 % slower)
    weights(0, pb0, pdsb0);
    weights(1, pb1, pdsb1);
    l_run += sum_bf16x8(pb1, sum_bf16x8(pb0, 0.f));
    mu_run += sum_bf16x8(pdsb1, sum_bf16x8(pdsb0, 0.f));
    value_step(0, pb0, pdsb0);
    __builtin_amdgcn_sched_barrier(0);
    value_step(1, pb1, pdsb1);
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
  weights(0, pb0, pdsb0);
  __builtin_amdgcn_sched_barrier(0);
  value_step(0, pb0, pdsb0);
  weights(1, pb1, pdsb1);
#pragma unroll
  for (int i = 0; i < 3 * DT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two vector instructions
  }
  __builtin_amdgcn_sched_barrier(0);
  value_step(1, pb1, pdsb1);
  const float lsum = sum_bf16x8(pb1, sum_bf16x8(pb0, 0.f));
  const float musum = sum_bf16x8(pdsb1, sum_bf16x8(pdsb0, 0.f));
#pragma unroll
  for (int i = 0; i < 3 * DT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  l_run += lsum;
  mu_run += musum;
}

// Primal kernel with 64-key blocks: S0^T = K[0:32] Q^T and S1^T = K[32:64] Q^T
// as two interleaved MFMA chains (every K operand read first), then the mask,
// max and rescale over both tiles, the weights, and A^T += V^T P^T over four
// 16-key steps (the V operands of the first two read before the softmax).
template <int D>
__device__ __forceinline__ void score_primal64(const StageTile<D, false> *st, const bf16x8 *qf,
                                               f32x16 &S0, f32x16 &S1) {
  constexpr int KCH = Geo<D>::KCH, KSTEPS = Geo<D>::KSTEPS;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int krow = swap_bits23(col);
  const int kx = k_swz<D>(krow);
  const uint4 *K0 = st->k + krow * KCH, *K1 = st->k + (32 + krow) * KCH;
  bf16x8 k0[KSTEPS], k1[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    k0[t] = as_bf16x8(K0[(2 * t + hh) ^ kx]);
    k1[t] = as_bf16x8(K1[(2 * t + hh) ^ kx]);
  }
  __builtin_amdgcn_sched_barrier(0);
  S0 = f32x16{};
  S1 = f32x16{};
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0[t], qf[t], S0, 0, 0, 0);
    S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[t], qf[t], S1, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void softmax_value_primal64(const StageTile<D, false> *st, f32x16 S0,
                                                       f32x16 S1, f32x16 *accO, float &m_ref,
                                                       float &l_run, bool partial,
                                                       int row_in_tile, float scale_log2) {
  constexpr int DT = Geo<D>::DT;
  const int hh = (threadIdx.x & 63) >> 5;
  bf16x8 vf[2][DT];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) vf[s][nt] = v_operand<D>(st->v, s, nt);
  __builtin_amdgcn_sched_barrier(0);
  if (partial) {
    // this lane-half's keys 8hh + {0..7, 16..23} of each 32-key tile
    const uint32_t b0 = st->bits[2 * row_in_tile] >> (8 * hh);
    const uint32_t b1 = st->bits[2 * row_in_tile + 1] >> (8 * hh);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = r >> 2, i = r & 3;
      const int key = 16 * (j >> 1) + 4 * (j & 1) + i;
      S0[r] = (b0 >> key) & 1u ? S0[r] : kNegInf;
      S1[r] = (b1 >> key) & 1u ? S1[r] : kNegInf;
    }
  }
  float sv[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sv[r] = S0[r];
    sv[16 + r] = S1[r];
  }
  float mh = max_of<32>(sv) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mh > m_ref + kRescaleSlack) != 0) {
    const float mx = fmaxf(mh, xor32(mh));
    const bool grow = mx > m_ref + kRescaleSlack;
    const float m_new = grow ? mx : m_ref;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) accO[nt] *= alpha;
    m_ref = m_new;
  }
  const float m_use = m_ref == kNegInf ? 0.f : m_ref;
  float pr[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S0[r], scale_log2, -m_use));
    pr[16 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S1[r], scale_log2, -m_use));
  }
  bf16x8 pb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) pb[s] = to_bf16x8(pr + 8 * s);
  l_run += sum_bf16x8(pb[3], sum_bf16x8(pb[2], sum_bf16x8(pb[1], sum_bf16x8(pb[0], 0.f))));
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s][nt], pb[s], accO[nt], 0, 0, 0);
#pragma unroll
  for (int s = 2; s < 4; ++s)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(st->v, s, nt), pb[s],
                                                         accO[nt], 0, 0, 0);
}

// Masking, online-softmax update and value step of one key block.
template <int D, bool TAN>
__device__ __forceinline__ void softmax_value_block(const StageTile<D, TAN> *st, f32x16 S, f32x16 dS,
                                                    f32x16 *accO, f32x16 *accT, float &m_ref,
                                                    float &l_run, float &mu_run, bool partial,
                                                    int row_in_tile, float scale_log2,
                                                    float scale) {
  if constexpr (TAN)
    softmax_value_jvp<D>(st, S, dS, accO, accT, m_ref, l_run, mu_run, partial, row_in_tile,
                         scale_log2, scale);
  else
    softmax_value_primal<D>(st, S, accO, m_ref, l_run, partial, row_in_tile, scale_log2);
}

// Waves per SIMD: two (one workgroup per CU), or four (two workgroups per
// CU) for the head-dim-64 primal kernel, which fits in 128 VGPRs without a
// spill (24 % faster; the kernels that would spill at 128 run 20-26 % slower).
template <int D, bool TAN>
constexpr int kWavesPerSimd = (!TAN && D == 64) ? 4 : 2;

template <int D, bool TAN>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, TAN>, kWavesPerSimd<D, TAN>)))
void attn_jvp_bf16_wide_kernel(KernelParams p) {
  constexpr int KCH = Geo<D>::KCH, KSTEPS = Geo<D>::KSTEPS, DT = Geo<D>::DT;
  using Stage = StageTile<D, TAN>;
  __shared__ Stage ring[kStages];
  __shared__ uint4 dq_lds[TAN ? BM * KCH : 1];
  __shared__ int2 ents[2][kEntChunk];

  const int L = work_item(int(blockIdx.x), p);
  const int slot = L % p.n_tiles;
  const int bh = L / p.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int unit = p.tile_order[slot];  // a query tile, or a piece of one (split launch)
  const int tile = p.unit_tile ? p.unit_tile[unit] : unit;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int row_in_tile = wave * 32 + col;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0]));
  auto stage_lds = [&](int s) { return ring_lds + uint32_t(s) * uint32_t(sizeof(Stage)); };
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;

  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + koff;
  const __bf16 *vb_ = static_cast<const __bf16 *>(p.v) + koff;
  // absent tangent tensors (NULL) are zero
  const __bf16 *dkb_ = TAN && p.dk ? static_cast<const __bf16 *>(p.dk) + koff : nullptr;
  const __bf16 *dvb_ = TAN && p.dv ? static_cast<const __bf16 *>(p.dv) + koff : nullptr;
  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;

  const int e0 = p.tile_offsets[unit], e1 = p.tile_offsets[unit + 1];
  const int n = e1 - e0;
  auto load_entries = [&](int c) {
    int2 *dst = ents[c & 1];
    const int base = e0 + c * kEntChunk;
#pragma unroll
    for (int i = threadIdx.x; i < kEntChunk; i += kThreads)
      dst[i] = base + i < e1 ? p.entries[base + i] : make_int2(0, -1);
  };
  auto entry = [&](int j) {
    const int2 e = ents[(j / kEntChunk) & 1][j % kEntChunk];
    return make_int2(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y));
  };
  constexpr int BNK = kBlockN<D, TAN>;  // keys per block
  auto bits_of = [&](int2 ent) {
    return p.partial_bits + int64_t(ent.y >= 0 ? ent.y : p.n_partial) * (BM * BNK / 32);
  };

  load_entries(0);
  __syncthreads();
  const int2 no_ent = make_int2(0, -1);
  int2 ent_c = n > 0 ? entry(0) : no_ent;
  int2 ent_1 = n > 1 ? entry(1) : no_ent;
  if (n > 0)
    issue_block<D, TAN>(stage_lds(0), wave, p, kb_, dkb_, vb_, dvb_, ent_c.x * BNK, bits_of(ent_c));

  // dQ tile -> LDS (rows past n_q re-read the last row), Q -> registers.
  if (TAN) {
    const uint32_t dq_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&dq_lds[0]));
    const bool zq = p.dq == nullptr;
    const void *dqb = zq ? static_cast<const void *>(kZeroRow)
                         : static_cast<const void *>(static_cast<const __bf16 *>(p.dq) + qoff);
#pragma unroll
    for (int i = 0; i < BM * KCH / kThreads; ++i) {
      // 32 rows per step: a 64-bit base at the step's first (clamped) row,
      // 32-bit lane offsets inside it
      const int q = i * kThreads + threadIdx.x;
      const int row = q / KCH, pch = q % KCH;
      const int rb = min(tile * BM + i * (kThreads / KCH), p.n_q - 1);
      const int grow = min(tile * BM + row, p.n_q - 1);
      const void *src = zq ? dqb
                           : static_cast<const void *>(static_cast<const __bf16 *>(dqb) +
                                                       int64_t(rb) * p.q_sn);
      const uint32_t roff = zq ? 0u : uint32_t(grow - rb) * uint32_t(p.q_sn) * 2u;
      dma16(src, roff + uint32_t(pch ^ k_swz<D>(row)) * 16u,
            dq_base + uint32_t(i * kThreads + wave * 64) * 16u);
    }
  }
  bf16x8 qf[KSTEPS];
  {
    const int qr = qvalid ? qrow : 0;
    const __bf16 *qb = static_cast<const __bf16 *>(p.q) + qoff + int64_t(qr) * p.q_sn + 8 * hh;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) qf[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + 16 * t));
  }

  f32x16 accO[DT], accT[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    accO[nt] = f32x16{};
    accT[nt] = f32x16{};
  }
  float m_ref = kNegInf, l_run = 0.f, mu_run = 0.f;

  {
    // the block loop, unrolled by two: each block's ring stage is an
    // immediate offset of the (held) per-lane read addresses
    auto step = [&](int j, const Stage *st, int next_stage) __attribute__((always_inline)) {
      if ((j + 2) % kEntChunk == 0 && j + 2 < n) {
        // the next chunk of entries, read after this barrier (entry(j + 2))
        load_entries((j + 2) / kEntChunk);
        wait_lgkmcnt0();
      }
      wait_vmcnt<0>();  // block j (and, first time, dQ and Q) has landed
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // the entry of block j + 2, read now (ahead of the operand reads) and
      // made uniform at the end of the block, so that its LDS latency is not
      // waited for just before the next barrier
      // (past the last block it reads a placeholder or a stale slot, never used)
      const int2 raw2 = ents[((j + 2) / kEntChunk) & 1][(j + 2) % kEntChunk];
      f32x16 S, dS;
      if constexpr (BNK == 64)
        score_primal64<D>(st, qf, S, dS);  // (the two score tiles)
      else
        score_block<D, TAN>(st, dq_lds, qf, row_in_tile, S, dS);
      // block j + 1 into the other stage (released by the barrier)
      if (j + 1 < n)
        issue_block<D, TAN>(stage_lds(next_stage), wave, p, kb_, dkb_, vb_, dvb_, ent_1.x * BNK,
                         bits_of(ent_1));
      if constexpr (BNK == 64)
        softmax_value_primal64<D>(st, S, dS, accO, m_ref, l_run, ent_c.y >= 0, row_in_tile,
                                  p.scale_log2);
      else
        softmax_value_block<D, TAN>(st, S, dS, accO, accT, m_ref, l_run, mu_run, ent_c.y >= 0,
                                    row_in_tile, p.scale_log2, p.scale);
      ent_c = ent_1;
      ent_1 = make_int2(__builtin_amdgcn_readfirstlane(raw2.x), __builtin_amdgcn_readfirstlane(raw2.y));
    };
    for (int j = 0; j < n; j += 2) {
      step(j, &ring[0], 1);
      if (j + 1 < n) step(j + 1, &ring[1], 0);
    }
  }

  const float l_tot = l_run + xor32(l_run);
  const float mu_tot = TAN ? mu_run + xor32(mu_run) : 0.f;
  if (!qvalid) return;
  const int part = p.unit_part ? p.unit_part[unit] : -1;
  if (part >= 0) {
    // one piece of a split tile: running statistics and unnormalised sums,
    // combined by the merge kernel
    const int64_t prow = (int64_t(bh) * p.n_parts + part) * BM + row_in_tile;
    if (hh == 0)
      *reinterpret_cast<float4 *>(p.part_stats + prow * 4) = make_float4(m_ref, l_tot, mu_tot, 0.f);
    float *pa = p.part_acc + prow * (2 * D);
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * nt + 8 * j + 4 * hh;
        *reinterpret_cast<float4 *>(pa + d0) =
            make_float4(accO[nt][4 * j], accO[nt][4 * j + 1], accO[nt][4 * j + 2], accO[nt][4 * j + 3]);
        if (TAN)
          *reinterpret_cast<float4 *>(pa + D + d0) =
              make_float4(accT[nt][4 * j], accT[nt][4 * j + 1], accT[nt][4 * j + 2], accT[nt][4 * j + 3]);
      }
    }
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float mu_n = mu_tot * inv;
  if (hh == 0) {
    const int64_t li = (int64_t(batch) * p.H + head) * p.n_q + qrow;
    p.lse[li] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : kNegInf;
    if (TAN && p.d_lse) p.d_lse[li] = mu_n;
  }
  const int64_t ooff = qoff + int64_t(qrow) * p.q_sn;
  __bf16 *ob = static_cast<__bf16 *>(p.o) + ooff;
  __bf16 *dob = TAN ? static_cast<__bf16 *>(p.d_o) + ooff : nullptr;
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * nt + 8 * j + 4 * hh;
      float o[4], dout[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = accO[nt][4 * j + i] * inv;
        if (TAN) dout[i] = __builtin_fmaf(-o[i], mu_n, accT[nt][4 * j + i] * inv);
      }
      *reinterpret_cast<uint2 *>(ob + d0) = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
      if (TAN)
        *reinterpret_cast<uint2 *>(dob + d0) =
            make_uint2(pack_bf16(dout[0], dout[1]), pack_bf16(dout[2], dout[3]));
    }
  }
}

}  // namespace

int launch_bf16(const KernelParams &p, int D, bool tangent, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(int64_t(p.n_tiles) * p.B * p.H));
  if (D == 128 && tangent)
    hipLaunchKernelGGL((attn_jvp_bf16_wide_kernel<128, true>), grid, dim3(kThreads), 0, s, p);
  else if (D == 128)
    hipLaunchKernelGGL((attn_jvp_bf16_wide_kernel<128, false>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64 && tangent)
    hipLaunchKernelGGL((attn_jvp_bf16_wide_kernel<64, true>), grid, dim3(kThreads), 0, s, p);
  else if (D == 64)
    hipLaunchKernelGGL((attn_jvp_bf16_wide_kernel<64, false>), grid, dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace attnjvp
