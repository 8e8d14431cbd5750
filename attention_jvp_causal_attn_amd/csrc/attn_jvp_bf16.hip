// Fused primal + tangent masked attention for gfx950, head dim 64 (bf16 in,
// fp32 accumulate); head dim 128 runs the eight-wave kernel of
// attn_jvp_bf16_wide.hip.
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
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows, one lane per row in each half-wave, so the per-row softmax
//    state lives in a lane and only the two half-waves exchange the row max;
//  * scores are computed transposed, S^T = K Q^T and dS^T = K dQ^T + dK Q^T,
//    with v_mfma_f32_32x32x16_bf16: K / dK come from LDS as the A operand, Q
//    and dQ stay in registers as the B operand for the whole key loop;
//  * the accumulators are transposed too, A^T += V^T P^T and
//    T^T += V^T (P*dS)^T + dV^T P^T, so the MFMA output of the score step is
//    already the B operand of the value step (no shuffle of P); K rows are
//    read in a permuted order (bits 2 and 3 of the row swapped) so that each
//    lane's 8 probabilities of a 16-key step are 8 consecutive keys;
//  * V and dV stay row-major in LDS; the transposed V^T operand comes from
//    ds_read_b64_tr_b16 (each group of 16 lanes turns 4 keys x 16 dims into
//    16 lanes x 4 keys);
//  * key blocks of 32 rows of K, dK, V, dV (and the admissible-key bits of
//    partial blocks) go HBM -> LDS with direct-to-LDS loads through a
//    3-stage ring, two blocks ahead of the MFMAs, without staging registers;
//    each tile is XOR-swizzled in 16-byte chunks so the MFMA operand reads hit
//    distinct banks;
//  * the MFMA accumulators live in AGPRs for the whole pass; the reference
//    max moves only when a row max exceeds it by more than 2^8 (a rare,
//    wave-uniform branch that multiplies the accumulators in place), so no
//    vector ALU work touches them in the steady state; p = exp2(s - m) then
//    stays below 2^8, far inside fp32 and bf16 range;
//  * workgroups are mapped to work so that each XCD (the dispatcher sends
//    workgroup w to XCD w % 8) receives an equal share of every group of
//    (batch, head) slices, as interleaved heavy-first tile slots, while the
//    workgroups resident on one XCD at a time belong to the same slice and
//    stream the same key blocks through that XCD's L2 (work_item);
//  * the copies of key block j + 2 go out once the score operands of block j
//    have been read, so the score MFMAs start right after the barrier; the
//    schedule entries of the next blocks ride in scalar registers.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "internal.h"

namespace attnjvp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int BM = kBf16BlockM;  // 128 query rows per workgroup
constexpr int BN = kBf16BlockN;  // 32 keys per block
constexpr int kStages = 3;
static_assert(BM == 128 && BN == 32, "kernel layout assumes 4 waves x 32 rows, 32-key blocks");

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales
constexpr int kEntChunk = 512;        // schedule entries staged in LDS at a time

template <int D>
struct alignas(16) StageTile {
  uint4 k[BN * D / 8];
  uint4 dk[BN * D / 8];
  uint4 v[BN * D / 8];
  uint4 dv[BN * D / 8];
  uint32_t bits[BM];
};

// Position of K row m of the 32x32 score tile: bits 2 and 3 swapped.  The
// MFMA output element (row 8j + 4h + i) then holds key 16(j/2) + 8h + 4(j%2) + i,
// so lane-half h owns keys 16s + 8h + 0..7 of value step s, in register order.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// XOR swizzles of 16-byte chunks within a key row.
// K / dK: the 16 lanes of one read touch 16 different rows at one chunk.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
// V / dV: a transposed read touches 4 consecutive rows x 4 consecutive chunks.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
// publishes a stage.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_wave) {
  lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);  // wave-uniform: keep it scalar
  // one wait state between the M0 write and the LDS-DMA that reads it
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

// A zero row: the copy source of an absent (zero) tangent tensor, read with
// row-independent offsets.
__device__ __align__(16) uint4 kZeroRow[16];

template <int D, bool TAN>
struct Dma {
  static constexpr int KCH = D / 8;                 // 16-byte chunks per key row
  static constexpr int CHUNKS = BN * KCH;           // per tensor tile
  static constexpr int PER_TENSOR = CHUNKS / kThreads;
  static constexpr int PER_STAGE = (TAN ? 4 : 2) * PER_TENSOR + 1;  // + mask bits
  static_assert(CHUNKS % kThreads == 0, "tiles must be whole workgroup loads");
  static_assert(BM * 4 == kWaves * 8 * 16, "mask bits: 8 lanes x 16 bytes per wave");
};

// Per-lane byte offsets of the direct-to-LDS copies inside a key block: one
// K-swizzled and one V-swizzled offset per wave-instruction.  Constant across
// blocks (the block base moves in scalar registers).
template <int D, bool TAN>
struct DmaOffsets {
  uint32_t k[Dma<D, TAN>::PER_TENSOR], v[Dma<D, TAN>::PER_TENSOR];
};

template <int D, bool TAN>
__device__ __forceinline__ void dma_offsets(DmaOffsets<D, TAN> &o, int64_t k_sn, int rows_valid) {
  using M = Dma<D, TAN>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < M::PER_TENSOR; ++i) {
    const int q = i * kThreads + wave * 64 + lane;
    const int row = q / M::KCH, pch = q % M::KCH;
    // rows past the last key re-read the last key (masked out by the schedule)
    const uint32_t roff = uint32_t(min(row, rows_valid - 1)) * uint32_t(k_sn) * 2u;
    o.k[i] = roff + uint32_t(pch ^ k_swz<D>(row)) * 16u;
    o.v[i] = roff + uint32_t(pch ^ v_swz<D>(row)) * 16u;
  }
}

// Issue the direct-to-LDS loads of one key block starting at key key0 into
// the stage tile at LDS byte address st (wave-uniform); wave is the
// wave-uniform wave index.
template <int D, bool TAN>
__device__ __forceinline__ void issue_block(uint32_t st, int wave, const KernelParams &p,
                                            const DmaOffsets<D, TAN> &full_off, const __bf16 *kb_,
                                            const __bf16 *dkb_, const __bf16 *vb_,
                                            const __bf16 *dvb_, int key0, const uint32_t *bits_src) {
  using M = Dma<D, TAN>;
  using T = StageTile<D>;
  const int lane = threadIdx.x & 63;
  const int64_t boff = int64_t(key0) * p.k_sn;
  DmaOffsets<D, TAN> o = full_off;
  if (key0 + BN > p.n_k) dma_offsets<D, TAN>(o, p.k_sn, p.n_k - key0);  // last block only
  // an absent tangent tensor is zero: copy the zero row into every row
  DmaOffsets<D, TAN> oz;
  if (TAN) dma_offsets<D, TAN>(oz, 0, 1);
  const bool zk = dkb_ == nullptr, zv = dvb_ == nullptr;
#pragma unroll
  for (int i = 0; i < M::PER_TENSOR; ++i) {
    const uint32_t chunk = uint32_t(i * kThreads + wave * 64) * 16u;  // this wave-instruction
    dma16(kb_ + boff, o.k[i], st + uint32_t(offsetof(T, k)) + chunk);
    dma16(vb_ + boff, o.v[i], st + uint32_t(offsetof(T, v)) + chunk);
    if (TAN) {
      dma16(zk ? static_cast<const void *>(kZeroRow) : dkb_ + boff, zk ? oz.k[i] : o.k[i],
            st + uint32_t(offsetof(T, dk)) + chunk);
      dma16(zv ? static_cast<const void *>(kZeroRow) : dvb_ + boff, zv ? oz.v[i] : o.v[i],
            st + uint32_t(offsetof(T, dv)) + chunk);
    }
  }
  // mask bits: BM words = 32 chunks; wave w copies chunks 8w .. 8w+7 (lanes 0..7)
  if (lane < 8)
    dma16(bits_src, uint32_t(wave * 8 + lane) * 16u,
          st + uint32_t(offsetof(T, bits)) + uint32_t(wave) * 128u);
}

// Score step of one key block: S^T = K Q^T and dS^T = K dQ^T + dK Q^T.
template <int D, bool TAN>
__device__ __forceinline__ void score_block(const StageTile<D> *st, const bf16x8 *qf,
                                            const bf16x8 *dqf, f32x16 &S, f32x16 &dS) {
  constexpr int KSTEPS = D / 16;
  constexpr int KCH = D / 8;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, hh = lane >> 5;
  const int krow = swap_bits23(col);
  const uint4 *Ks = st->k + krow * KCH;
  const uint4 *dKs = st->dk + krow * KCH;
  const int kx = k_swz<D>(krow);

  S = f32x16{};
  dS = f32x16{};
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    const int c = (2 * t + hh) ^ kx;
    const bf16x8 kf = as_bf16x8(Ks[c]);
    S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], S, 0, 0, 0);
    if (TAN) {
      const bf16x8 dkf = as_bf16x8(dKs[c]);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, dqf[t], dS, 0, 0, 0);
      dS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dkf, qf[t], dS, 0, 0, 0);
    }
  }
}

// Masking, online-softmax update and value step of one key block.
template <int D, bool TAN>
__device__ __forceinline__ void softmax_value_block(const StageTile<D> *st, f32x16 S, f32x16 dS,
                                                    f32x16 *accO, f32x16 *accT, float &m_ref,
                                                    float &l_run, float &mu_run, bool partial,
                                                    int row_in_tile, float scale_log2,
                                                    float scale) {
  constexpr int DT = D / 32;
  constexpr int KCH = D / 8;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;

  if (partial) {  // workgroup-uniform: only blocks that straddle a mask edge
    const uint32_t bits = st->bits[row_in_tile];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = r >> 2, i = r & 3;
      const int key = 16 * (j >> 1) + 8 * hh + 4 * (j & 1) + i;
      const bool ok = (bits >> key) & 1u;
      S[r] = ok ? S[r] : kNegInf;
      if (TAN) dS[r] = ok ? dS[r] : 0.f;
    }
  }

  // Max over this lane's 16 keys; the two half-waves exchange it only when
  // one of them crosses the slack, since a row can grow only then.
  float mh = S[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mh = fmaxf(mh, S[r]);
  mh *= scale_log2;
  if (__builtin_amdgcn_ballot_w64(mh > m_ref + kRescaleSlack) != 0) {
    // Move the reference max (rare after the first block of a row).  Only the
    // rows that crossed the slack move, so every row's arithmetic depends on
    // its own admissible scores alone (alpha = 1 is exact for the others).
    const float mx = fmaxf(mh, xor32(mh));
    const bool grow = mx > m_ref + kRescaleSlack;
    const float m_new = grow ? mx : m_ref;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
    l_run *= alpha;
    mu_run *= alpha;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = accO[nt][i], tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(tmp) : "v"(alpha));
        accO[nt][i] = x;
        if (TAN) {
          float y = accT[nt][i], tmp2;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(y), "=&v"(tmp2) : "v"(alpha));
          accT[nt][i] = y;
        }
      }
    }
    asm volatile("s_nop 4" ::: "memory");
    m_ref = m_new;
  }
  const float m_use = m_ref == kNegInf ? 0.f : m_ref;

  float pr[16], pds[16];
  float lsum = 0.f, musum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], scale_log2, -m_use));
    lsum += pr[r];
    if (TAN) {
      const float dss = dS[r] * scale;
      pds[r] = pr[r] * dss;
      musum = __builtin_fmaf(pr[r], dss, musum);
    }
  }
  l_run += lsum;
  if (TAN) mu_run += musum;

  bf16x8 pb[2], pdsb[2];
  pb[0] = to_bf16x8(pr);
  pb[1] = to_bf16x8(pr + 8);
  if (TAN) {
    pdsb[0] = to_bf16x8(pds);
    pdsb[1] = to_bf16x8(pds + 8);
  }

  // Value step s covers keys 16s .. 16s+15; lane-half hh supplies keys
  // 16s + 8hh + 0..7.  Transposed reads: within each 16-lane group, lane j
  // points at key (16s + 8hh + 4*half + j/4), dims (d0 + 4*(j%4)) .. +3.
  const int g = lane >> 4, jl = lane & 15;
  const int dcol = 16 * (g & 1) + 4 * (jl & 3);  // + 32 * nt
  const int krel = 8 * hh + (jl >> 2);            // + 16 * s + 4 * half
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const int d = 32 * nt + dcol;
      bf16x4 vh[2], dvh[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key = 16 * s + 4 * half + krel;
        const int chunk = key * KCH + ((d >> 3) ^ v_swz<D>(key));
        const char *vp = reinterpret_cast<const char *>(st->v + chunk) + (d & 7) * 2;
        vh[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(vp));
        if (TAN) {
          const char *dvp = reinterpret_cast<const char *>(st->dv + chunk) + (d & 7) * 2;
          dvh[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4 *)(dvp));
        }
      }
      const bf16x8 vf = __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7);
      accO[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[s], accO[nt], 0, 0, 0);
      if (TAN) {
        const bf16x8 dvf = __builtin_shufflevector(dvh[0], dvh[1], 0, 1, 2, 3, 4, 5, 6, 7);
        accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pdsb[s], accT[nt], 0, 0, 0);
        accT[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dvf, pb[s], accT[nt], 0, 0, 0);
      }
    }
  }
}

template <int D, bool TAN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_jvp_bf16_kernel(KernelParams p) {
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;
  using M = Dma<D, TAN>;
  __shared__ StageTile<D> ring[kStages];

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
  auto stage_lds = [&](int slot) { return ring_lds + uint32_t(slot) * uint32_t(sizeof(StageTile<D>)); };
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;

  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const __bf16 *kb_ = static_cast<const __bf16 *>(p.k) + koff;
  const __bf16 *vb_ = static_cast<const __bf16 *>(p.v) + koff;
  // absent tangent tensors (NULL) are zero
  const __bf16 *dkb_ = TAN && p.dk ? static_cast<const __bf16 *>(p.dk) + koff : nullptr;
  const __bf16 *dvb_ = TAN && p.dv ? static_cast<const __bf16 *>(p.dv) + koff : nullptr;

  const int e0 = p.tile_offsets[unit], e1 = p.tile_offsets[unit + 1];
  const int n = e1 - e0;
  // Schedule entries of this tile, staged in LDS in chunks (read with LDS
  // loads inside the key loop, so no global load sits between the
  // direct-to-LDS copies and the MFMAs).
  __shared__ int2 ents[2][kEntChunk];
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
  // Full blocks take their (all-ones) mask words from one extra block that
  // the schedule keeps after the partial ones.
  auto bits_of = [&](int2 ent) {
    return p.partial_bits + int64_t(ent.y >= 0 ? ent.y : p.n_partial) * BM;
  };

  DmaOffsets<D, TAN> doff;
  dma_offsets<D, TAN>(doff, p.k_sn, BN);
  load_entries(0);
  __syncthreads();
  // Entries of blocks j, j + 1 and j + 2 ride in scalar registers; the one of
  // block j + 3 is read from LDS during block j.
  const int2 no_ent = make_int2(0, -1);
  int2 ent_c = n > 0 ? entry(0) : no_ent;
  int2 ent_1 = n > 1 ? entry(1) : no_ent;
  int2 ent_2 = n > 2 ? entry(2) : no_ent;
  if (n > 0)
    issue_block<D, TAN>(stage_lds(0), wave, p, doff, kb_, dkb_, vb_, dvb_, ent_c.x * BN, bits_of(ent_c));

  bf16x8 qf[KSTEPS], dqf[KSTEPS];
  {
    const int qr = qvalid ? qrow : 0;
    const int64_t off = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh + int64_t(qr) * p.q_sn + 8 * hh;
    const __bf16 *qb = static_cast<const __bf16 *>(p.q) + off;
    const __bf16 *dqb = TAN && p.dq ? static_cast<const __bf16 *>(p.dq) + off : nullptr;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      qf[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + 16 * t));
      if (TAN) dqf[t] = dqb ? as_bf16x8(*reinterpret_cast<const uint4 *>(dqb + 16 * t)) : bf16x8{};
    }
  }
  // Q, dQ and the first block are in before the loop: the loop itself then
  // waits only on the direct-to-LDS copies.
  wait_vmcnt<0>();
  if (n > 1)
    issue_block<D, TAN>(stage_lds(1), wave, p, doff, kb_, dkb_, vb_, dvb_, ent_1.x * BN, bits_of(ent_1));

  f32x16 accO[DT], accT[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    accO[nt] = f32x16{};
    accT[nt] = f32x16{};
  }
  float m_ref = kNegInf, l_run = 0.f, mu_run = 0.f;

  int cur = 0;  // ring slot of block j
  for (int j = 0; j < n; ++j) {
    if ((j + 3) % kEntChunk == 0 && j + 3 < n) load_entries((j + 3) / kEntChunk);
    if (j + 1 < n)
      wait_vmcnt<M::PER_STAGE>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int2 raw3 = ents[((j + 3) / kEntChunk) & 1][(j + 3) % kEntChunk];
    f32x16 S, dS;
    score_block<D, TAN>(&ring[cur], qf, dqf, S, dS);
    // The copies of block j + 2 go out after the score operands of block j
    // have been read, so the score MFMAs start right after the barrier.
    if (j + 2 < n) {
      const int nxt = cur >= 1 ? cur - 1 : cur + 2;  // (cur + 2) % 3
      issue_block<D, TAN>(stage_lds(nxt), wave, p, doff, kb_, dkb_, vb_, dvb_, ent_2.x * BN, bits_of(ent_2));
    }
    softmax_value_block<D, TAN>(&ring[cur], S, dS, accO, accT, m_ref, l_run, mu_run, ent_c.y >= 0,
                                row_in_tile, p.scale_log2, p.scale);
    ent_c = ent_1;
    ent_1 = ent_2;
    ent_2 = make_int2(__builtin_amdgcn_readfirstlane(raw3.x), __builtin_amdgcn_readfirstlane(raw3.y));
    cur = cur == kStages - 1 ? 0 : cur + 1;
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
  const int64_t ooff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh + int64_t(qrow) * p.q_sn;
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

template <int D, bool TAN>
hipError_t launch(const KernelParams &p, hipStream_t stream) {
  const int64_t G = int64_t(p.n_tiles) * p.B * p.H;
  hipLaunchKernelGGL((attn_jvp_bf16_kernel<D, TAN>), dim3(unsigned(G)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int launch_bf16(const KernelParams &p, int D, bool tangent, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return launch_bf16_wide(p, tangent, stream);
  if (D == 64) return tangent ? launch<64, true>(p, s) : launch<64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
