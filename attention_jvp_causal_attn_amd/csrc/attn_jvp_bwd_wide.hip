// Gradients of masked attention (the backward of the primal) for gfx950,
// bf16 in and out, fp32 accumulate, head dim 64 or 128.
//
// The forward returns the row log-sum-exp so that a backward of the same
// masked operator can reuse it ("Causal-rCM ..." summary, Appendix B: the
// kernel's outputs are O, LSE and dO; the student is trained through the
// TF-masked packed forward, Section 3).  With P_ij = exp(s_ij - LSE_i) over
// the admissible pairs and g = dL/dO:
//     D_i   = <g_i, O_i>
//     dP_ij = <g_i, v_j>,   dS_ij = P_ij (dP_ij - D_i)
//     dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i,
//     dV_j  = sum_i P_ij g_i.
// Two passes, no atomics (deterministic):
//  * dQ pass: a workgroup owns 256 query rows and walks the mask's schedule
//    of admissible 32-key blocks: S^T = K Q^T and dP^T = V g^T (Q and g in
//    registers as MFMA B operands, K and V from LDS), dS^T, then
//    dQ^T += K^T dS^T with K^T read transposed from the same LDS tile.  It
//    also computes D_i (from O and g) and stores it for the second pass;
//  * dK/dV pass: a workgroup owns 256 keys and walks the schedule of the
//    transposed mask (admissible 32-query blocks): S = Q K^T, dP = g V^T (K
//    in registers, V and the Q and g blocks from LDS), then dV^T += g^T P
//    and dK^T += Q^T dS.
// Eight waves per workgroup, two per SIMD, 32 rows (or keys) each: one
// wave's softmax-side vector work runs while the other keeps the matrix core
// busy; at head dim 128 the two waves of a SIMD are held half a block apart
// (one forms a block's scores while the other finishes the previous block's
// gradient update), over a 3-stage ring.  Every value lives in the 256 VGPRs a wave has at two waves per
// SIMD; the dK/dV pass therefore stages its V rows in LDS (read as the MFMA
// B operand) while K stays in registers.  Both passes use one lane per row
// in each half-wave, the row permutation that puts a lane's 8 weights of a
// 16-wide step in register order, direct-to-LDS copies into a ring (block
// j + 1 is copied while block j is computed), and tiles swizzled so
// that both row reads (ds_read_b128) and transposed reads
// (ds_read_b64_tr_b16) hit distinct banks.
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
constexpr int BM = kBwdBlockMWide;  // 256 rows (or keys) per workgroup
constexpr int BN = kBwdBlockN;      // 32 keys (or queries) per block
constexpr int kEntChunk = 512;
static_assert(BM == 256 && BN == 32, "8 waves x 32 rows, 32-row blocks");

// Per head dim: 16-byte chunks per row, 16-wide k-steps, 32-wide dim tiles.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static constexpr int KCH = D / 8;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE = BN * KCH;  // chunks of one 32-row tile
};
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x8 to_bf16x8(const float *x) {
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }
// Bits 2 and 3 of a 32-row tile index swapped: the MFMA output element
// (row 8j + 4h + i) of a tile whose A-operand rows are read in this order
// holds row 16(j/2) + 8h + 4(j%2) + i, so lane-half h owns rows 16s + 8h + 0..7
// of step s in register order.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// 16-byte-chunk XOR swizzle of a row, conflict-free both for row reads
// (ds_read_b128: 16 lanes per cycle read 16 aligned rows at one chunk) and for
// transposed reads (ds_read_b64_tr_b16: 32 lanes per cycle read 4 aligned
// consecutive rows x 4 consecutive chunks), with 64 banks of 4 bytes.  Head
// dim 128 (256-byte rows, 16 chunk slots per bank cycle): a bijection of the
// row's low 4 bits whose top two bits (the 64-byte window) differ across 4
// consecutive rows.  Head dim 64 (128-byte rows, two rows per bank cycle): a
// bijection of 0..7 within each row parity over 16 rows whose top bit differs
// between rows 4a and 4a+2 (and 4a+1, 4a+3).
template <int D>
__device__ __forceinline__ int sw(int row) {
  return D == 128 ? (4 * (row & 3) | ((row >> 2) & 3)) : (4 * ((row >> 1) & 1) | ((row >> 2) & 3));
}

// 16 bytes per lane straight into LDS at lds_wave + 16 * lane (lds_wave
// wave-uniform); tracked by vmcnt and waited for explicitly.  One wait state
// separates the M0 write from the copy.
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds_wave) {
  lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds_wave)
               : "memory", "m0");
}
// 4 bytes per lane from a per-lane address into LDS at lds_wave + 4 * lane.
__device__ __forceinline__ void dma4(const void *addr, uint32_t lds_wave) {
  lds_wave = __builtin_amdgcn_readfirstlane(lds_wave);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(addr), "s"(lds_wave)
               : "memory", "m0");
}
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

// Byte offset of chunk q of a 32-row block (swizzled); rows past the last
// valid one re-read it (masked out by the schedule).
template <int D>
__device__ __forceinline__ uint32_t copy_offset(int q, int64_t row_stride, int rows_valid) {
  constexpr int KCH = Geo<D>::KCH;
  const int row = q / KCH, pch = q % KCH;
  return uint32_t(min(row, rows_valid - 1)) * uint32_t(row_stride) * 2u +
         uint32_t(pch ^ sw<D>(row)) * 16u;
}

// Two 32 x D tiles (rows r0 .. r0+31 of a and b) and the block's 256 mask
// words into a stage.  Head dim 128: one chunk per lane per tile; head dim
// 64: waves 0-3 copy a, waves 4-7 copy b.
template <int D>
__device__ __forceinline__ void copy_pair(uint32_t st, uint32_t a_at, uint32_t b_at,
                                          uint32_t bits_at, int wave, const __bf16 *a,
                                          const __bf16 *b, int64_t row_stride, int r0, int n_rows,
                                          const uint32_t *bits_src) {
  const int lane = threadIdx.x & 63;
  const int64_t boff = int64_t(r0) * row_stride;
  if constexpr (D == 128) {
    const uint32_t off = copy_offset<D>(int(threadIdx.x), row_stride, min(BN, n_rows - r0));
    const uint32_t chunk = uint32_t(wave * 64) * 16u;
    dma16(a + boff, off, st + a_at + chunk);
    dma16(b + boff, off, st + b_at + chunk);
  } else {
    const int c0 = (wave & 3) * 64;  // this wave's chunks of its tile
    const uint32_t off = copy_offset<D>(c0 + lane, row_stride, min(BN, n_rows - r0));
    dma16((wave < 4 ? a : b) + boff, off, st + (wave < 4 ? a_at : b_at) + uint32_t(c0) * 16u);
  }
  // mask bits: BM words = 64 chunks; wave w copies chunks 8w .. 8w+7 (lanes 0..7)
  if (lane < 8)
    dma16(bits_src, uint32_t(wave * 8 + lane) * 16u, st + bits_at + uint32_t(wave) * 128u);
}

// A-operand row read of a swizzled 32 x D tile: this lane's row (permuted)
// at k-step t.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint4 *tile, int prow, int t, int hh) {
  return as_bf16x8(tile[prow * Geo<D>::KCH + ((2 * t + hh) ^ sw<D>(prow))]);
}
// The same read as the byte offset 32 t ^ y from the row's start, y = 16 (hh ^
// sw(row)): one xor-add per read with the step's constant, for a pass that
// rebuilds its offsets per block.
__device__ __forceinline__ bf16x8 row_read_xad(const char *row, int t, uint32_t y) {
  return as_bf16x8(*reinterpret_cast<const uint4 *>(row + ((32u * uint32_t(t)) ^ y)));
}
// A-operand transposed read of a swizzled 32 x D tile for step s of 16
// rows and dim tile nt: within each 16-lane group, lane jl reads row
// (16s + 4*half + krel) at dims (d0 + 4*(jl%4)) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint4 *tile, int s, int nt, int dcol, int krel) {
  bf16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 16 * s + 4 * half + krel;
    const int d = 32 * nt + dcol;
    const int chunk = row * Geo<D>::KCH + ((d >> 3) ^ sw<D>(row));
    const char *ptr = reinterpret_cast<const char *>(tile + chunk) + (d & 7) * 2;
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4 *)(ptr));
  }
  return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
}
// Register-order position of element r of a 16-wide half-tile: row (or
// column) 16(j/2) + 8h + 4(j%2) + i for r = 4j + i; shifted by 8h, the bit of a
// 32-bit mask word.
__device__ __forceinline__ int reg_pos(int r) {
  const int j = r >> 2, i = r & 3;
  return 16 * (j >> 1) + 4 * (j & 1) + i;
}

// Per-lane constants of the transposed reads (held across the key loop).
struct TrLane {
  int dcol, krel;
};
__device__ __forceinline__ TrLane tr_lane() {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, jl = lane & 15;
  return {16 * (g & 1) + 4 * (jl & 3), 8 * (lane >> 5) + (jl >> 2)};
}

// Head dim 128 (both passes): the two waves of a SIMD run half a block apart
// over a 3-stage ring.  Head dim 64 keeps one phase and 2 stages (its dQ pass
// runs four waves per SIMD within 128 registers, which the carried scores
// would exceed).
template <int D>
constexpr bool kPingPong = D == 128;

// ---------------------------------------------------------------- dQ pass

template <int D>
struct alignas(16) KVTile {
  uint4 k[Geo<D>::TILE];
  uint4 v[Geo<D>::TILE];
  uint32_t bits[BM];
};

// Waves per SIMD of the dQ pass: two, or four (two workgroups per CU) at head
// dim 64, where it fits in 128 VGPRs without a spill (the backward 6 % faster).
template <int D>
constexpr int kDqWavesPerSimd = D == 64 ? 4 : 2;

template <int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kDqWavesPerSimd<D>, kDqWavesPerSimd<D>)))
void bwd_dq_wide_kernel(BwdParams p) {
  constexpr int KSTEPS = Geo<D>::KSTEPS, DT = Geo<D>::DT;
  using KVTile = attnjvp::KVTile<D>;
  __shared__ KVTile ring[kPingPong<D> ? 3 : 2];
  __shared__ int2 ents[2][kEntChunk];
  const int L = work_item(int(blockIdx.x), p.r_map);
  const int slot = L % p.r_map.n_tiles;
  const int bh = L / p.r_map.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int tile = p.r_order[slot];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int row_in_tile = wave * 32 + col;
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0]));
  auto stage_lds = [&](int s) { return ring_lds + uint32_t(s) * uint32_t(sizeof(KVTile)); };

  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const __bf16 *kb = static_cast<const __bf16 *>(p.k) + koff;
  const __bf16 *vb = static_cast<const __bf16 *>(p.v) + koff;
  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;
  const int64_t lrow = (int64_t(batch) * p.H + head) * p.n_q;

  const int e0 = p.r_offsets[tile], e1 = p.r_offsets[tile + 1];
  const int n = e1 - e0;
  auto load_entries = [&](int c) {
    int2 *dst = ents[c & 1];
    const int base = e0 + c * kEntChunk;
    for (int i = threadIdx.x; i < kEntChunk; i += kThreads)
      dst[i] = base + i < e1 ? p.r_entries[base + i] : make_int2(0, -1);
  };
  auto entry = [&](int j) {
    const int2 e = ents[(j / kEntChunk) & 1][j % kEntChunk];
    return make_int2(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y));
  };
  auto bits_of = [&](int2 e) { return p.r_bits + int64_t(e.y >= 0 ? e.y : p.r_partial) * BM; };
  auto issue = [&](int s, int2 e) {
    copy_pair<D>(stage_lds(s), offsetof(KVTile, k), offsetof(KVTile, v), offsetof(KVTile, bits), wave,
              kb, vb, p.k_sn, e.x * BN, p.n_k, bits_of(e));
  };

  load_entries(0);
  __syncthreads();
  if (n > 0) issue(0, entry(0));

  bf16x8 qf[KSTEPS], gf[KSTEPS];
  float dsum = 0.f;
  {
    const int qr = qvalid ? qrow : 0;
    const int64_t off = qoff + int64_t(qr) * p.q_sn + 8 * hh;
    const __bf16 *qb = static_cast<const __bf16 *>(p.q) + off;
    const __bf16 *gb = static_cast<const __bf16 *>(p.g_o) + off;
    const __bf16 *ob = static_cast<const __bf16 *>(p.o) + off;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      qf[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + 16 * t));
      gf[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(gb + 16 * t));
      const bf16x8 of = as_bf16x8(*reinterpret_cast<const uint4 *>(ob + 16 * t));
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf(float(gf[t][e]), float(of[e]), dsum);
    }
  }
  dsum += xor32(dsum);
  const float lse2 = qvalid ? p.lse[lrow + qrow] * kLog2e : 0.f;
  if (qvalid && hh == 0) p.delta[lrow + qrow] = dsum;

  f32x16 acc[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) acc[nt] = f32x16{};
  const float sl2 = p.scale_log2;
  // dP^T - D accumulates from -D: the MFMA chain starts from these registers
  // (kept for the tile), so the subtraction costs no instruction per block
  // (head dim 128 only: the head-dim-64 pass must fit 128 registers)
  constexpr bool kInitD = D == 128;
  f32x16 g_init = {};
  if constexpr (kInitD) {
#pragma unroll
    for (int r = 0; r < 16; ++r) g_init[r] = -dsum;
  }

  // Per-lane LDS read offsets, held across the key loop (registers allow it
  // in this pass); the loop below is unrolled by the ring's stage count (two,
  // three at head dim 128) so that the ring stage of every read is an
  // immediate offset.
  const int krow = swap_bits23(col);
  const TrLane tl = tr_lane();
  // A block in two halves.  h1: S^T and dP^T - D (MFMAs from the block's K, V
  // rows).  h2: exponents, mask, dS^T and the dQ update (K^T read transposed).
  auto h1 = [&](const KVTile *st, f32x16 &S, f32x16 &G) __attribute__((always_inline)) {
    S = f32x16{};
    G = g_init;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(st->k, krow, t, hh), qf[t], S, 0, 0, 0);
      G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(st->v, krow, t, hh), gf[t], G, 0, 0, 0);
      if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound the operand prefetch
    }
  };
  auto h2 = [&](int2 ent, const KVTile *st, const f32x16 &S, const f32x16 &G) __attribute__((always_inline)) {
    // exponents; in a partial block those of inadmissible pairs become -inf
    // (exp2 then gives exactly 0, also for a row without keys, whose LSE is
    // -inf); full blocks skip the mask
    float x[16], gs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = __builtin_fmaf(S[r], sl2, -lse2);
    if (ent.y >= 0) {
      const uint32_t bits = st->bits[row_in_tile] >> (8 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = (bits >> reg_pos(r)) & 1u ? x[r] : -__builtin_inff();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
      gs[r] = __builtin_amdgcn_exp2f(x[r]) * (kInitD ? G[r] : G[r] - dsum);
    bf16x8 gsb[2];
    gsb[0] = to_bf16x8(gs);
    gsb[1] = to_bf16x8(gs + 8);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(st->k, s, nt, tl.dcol, tl.krel),
                                                          gsb[s], acc[nt], 0, 0, 0);
        if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto sync = [&](int j) __attribute__((always_inline)) {
    if ((j + 1) % kEntChunk == 0 && j + 1 < n) {
      // the next chunk of entries, read after this barrier (entry(j + 1))
      load_entries((j + 1) / kEntChunk);
      wait_lgkmcnt0();
    }
    wait_vmcnt<0>();  // block j (and, first time, Q, g, O) has landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (!kPingPong<D>) {
    auto step = [&](int j, const KVTile *st, int next_stage) __attribute__((always_inline)) {
      sync(j);
      const int2 ent = entry(j);
      f32x16 S, G;
      h1(st, S, G);
      if (j + 1 < n) issue(next_stage, entry(j + 1));  // its stage was released by the barrier
      h2(ent, st, S, G);
    };
    for (int j = 0; j < n; j += 2) {
      step(j, &ring[0], 1);
      if (j + 1 < n) step(j + 1, &ring[1], 0);
    }
  } else if (wave < 4) {
    // The two waves that share a SIMD (w and w + 4) run half a block apart:
    // between two barriers, waves 0-3 do h1 and h2 of block j while waves 4-7
    // do h2 of block j - 1 and h1 of block j, so one wave's vector work runs
    // under the other's MFMAs.  Block j is read from its stage between
    // barriers j and j + 2, hence a 3-stage ring; the copy for block j + 1,
    // issued after barrier j, goes to the stage of block j - 2.
    auto step = [&](int j, const KVTile *st, int next_stage) __attribute__((always_inline)) {
      sync(j);
      const int2 ent = entry(j);
      f32x16 S, G;
      h1(st, S, G);
      if (j + 1 < n) issue(next_stage, entry(j + 1));  // its stage was released by the barrier
      h2(ent, st, S, G);
    };
    for (int j = 0; j < n; j += 3) {
      step(j, &ring[0], 1);
      if (j + 1 < n) step(j + 1, &ring[1], 2);
      if (j + 2 < n) step(j + 2, &ring[2], 0);
    }
  } else {
    f32x16 S = {}, G = {};
    int2 ent = make_int2(0, -1);
    auto step = [&](int j, const KVTile *st, const KVTile *prev, int next_stage) __attribute__((always_inline)) {
      sync(j);
      if (j + 1 < n) issue(next_stage, entry(j + 1));
      if (j > 0) h2(ent, prev, S, G);
      ent = entry(j);
      h1(st, S, G);
    };
    for (int j = 0; j < n; j += 3) {
      step(j, &ring[0], &ring[2], 1);
      if (j + 1 < n) step(j + 1, &ring[1], &ring[0], 2);
      if (j + 2 < n) step(j + 2, &ring[2], &ring[1], 0);
    }
    if (n > 0) h2(ent, &ring[(n - 1) % 3], S, G);
  }
  wait_vmcnt<0>();

  if (!qvalid) return;
  __bf16 *out = static_cast<__bf16 *>(p.g_q) + qoff + int64_t(qrow) * p.q_sn;
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * nt + 8 * jj + 4 * hh;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = acc[nt][4 * jj + i] * p.scale;
      *reinterpret_cast<uint2 *>(out + d0) = make_uint2(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]));
    }
  }
}

// ------------------------------------------------------------ dK/dV pass

template <int D>
struct alignas(16) QGTile {
  uint4 q[Geo<D>::TILE];
  uint4 g[Geo<D>::TILE];
  float ld[8 * 8];  // wave w's region: LSE of queries 4w .. 4w+3, then their D
  uint32_t bits[BM];
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkv_wide_kernel(BwdParams p) {
  constexpr int KCH = Geo<D>::KCH, KSTEPS = Geo<D>::KSTEPS, DT = Geo<D>::DT;
  using QGTile = attnjvp::QGTile<D>;
  __shared__ QGTile ring[kPingPong<D> ? 3 : 2];
  __shared__ uint4 v_lds[BM * KCH];  // this tile's V rows (B operands), 64 KB at D = 128
  __shared__ int2 ents[2][kEntChunk];
  const int L = work_item(int(blockIdx.x), p.c_map);
  const int slot = L % p.c_map.n_tiles;
  const int bh = L / p.c_map.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int tile = p.c_order[slot];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int key_in_tile = wave * 32 + col;
  const int krow_g = tile * BM + key_in_tile;
  const bool kvalid = krow_g < p.n_k;
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[0]));
  auto stage_lds = [&](int s) { return ring_lds + uint32_t(s) * uint32_t(sizeof(QGTile)); };

  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;
  const __bf16 *qb = static_cast<const __bf16 *>(p.q) + qoff;
  const __bf16 *gb = static_cast<const __bf16 *>(p.g_o) + qoff;
  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const int64_t lrow = (int64_t(batch) * p.H + head) * p.n_q;

  const int e0 = p.c_offsets[tile], e1 = p.c_offsets[tile + 1];
  const int n = e1 - e0;
  auto load_entries = [&](int c) {
    int2 *dst = ents[c & 1];
    const int base = e0 + c * kEntChunk;
    for (int i = threadIdx.x; i < kEntChunk; i += kThreads)
      dst[i] = base + i < e1 ? p.c_entries[base + i] : make_int2(0, -1);
  };
  auto entry = [&](int j) {
    const int2 e = ents[(j / kEntChunk) & 1][j % kEntChunk];
    return make_int2(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y));
  };
  auto bits_of = [&](int2 e) { return p.c_bits + int64_t(e.y >= 0 ? e.y : p.c_partial) * BM; };
  auto issue = [&](int s, int2 e) {
    const int q0 = e.x * BN;
    copy_pair<D>(stage_lds(s), offsetof(QGTile, q), offsetof(QGTile, g), offsetof(QGTile, bits), wave,
              qb, gb, p.q_sn, q0, p.n_q, bits_of(e));
    // LSE and D of queries q0 + 4w .. q0 + 4w + 3 (lanes 0..3, 4..7), clamped
    if (lane < 8) {
      const int qi = min(q0 + 4 * wave + (lane & 3), p.n_q - 1);
      const float *src = lane < 4 ? p.lse + lrow + qi : p.delta + lrow + qi;
      dma4(src, stage_lds(s) + uint32_t(offsetof(QGTile, ld)) + uint32_t(wave) * 32u);
    }
  };

  load_entries(0);
  __syncthreads();
  if (n > 0) issue(0, entry(0));
  // V rows of the tile -> LDS (rows past n_k re-read the last key), K -> registers
  {
    const uint32_t v_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&v_lds[0]));
    const __bf16 *vb = static_cast<const __bf16 *>(p.v) + koff;
#pragma unroll
    for (int i = 0; i < BM * KCH / kThreads; ++i) {
      // kThreads / KCH rows per step: a 64-bit base at the step's first
      // (clamped) row, 32-bit lane offsets inside it
      const int q = i * kThreads + threadIdx.x;
      const int row = q / KCH, pch = q % KCH;
      const int rb = min(tile * BM + i * (kThreads / KCH), p.n_k - 1);
      const int grow = min(tile * BM + row, p.n_k - 1);
      dma16(vb + int64_t(rb) * p.k_sn,
            uint32_t(grow - rb) * uint32_t(p.k_sn) * 2u + uint32_t(pch ^ sw<D>(row)) * 16u,
            v_base + uint32_t(i * kThreads + wave * 64) * 16u);
    }
  }
  bf16x8 kf[KSTEPS];
  {
    const int kr = kvalid ? krow_g : 0;
    const __bf16 *kp = static_cast<const __bf16 *>(p.k) + koff + int64_t(kr) * p.k_sn + 8 * hh;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) kf[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(kp + 16 * t));
  }
  // The staged V rows are negated in place (each lane flips the sign bits of
  // the chunks its own copies wrote, once they have landed), so that the
  // per-block MFMA chain H = D + g (-V)^T, started from the queries' D,
  // gives D - dP without a subtraction per element.
  wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < BM * KCH / kThreads; ++i) {
    uint4 *c = v_lds + i * kThreads + threadIdx.x;
    uint4 x = *c;
    x.x ^= 0x80008000u; x.y ^= 0x80008000u; x.z ^= 0x80008000u; x.w ^= 0x80008000u;
    *c = x;
  }
  wait_lgkmcnt0();  // published by the first block's barrier

  f32x16 accK[DT], accV[DT];
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
    accK[nt] = f32x16{};
    accV[nt] = f32x16{};
  }
  const float sl2 = p.scale_log2;

  // Per-lane LDS read offsets: held across the key loop at head dim 64; at
  // head dim 128, where registers are short, the row-read offsets are rebuilt
  // per block (one xor-add per read) and only the transposed-read offsets are
  // held.  The loop is unrolled by the stage count as in the dQ pass.
  constexpr bool kHoist = D == 64;
  const int qperm_h = swap_bits23(col);
  const TrLane tl_h = tr_lane();
  // A block of 32 queries in two halves.  h1: S = Q K^T and H = D - dP
  // (MFMAs from the block's Q, g rows).  h2: mask, P and -dS, then the dV, dK
  // updates (transposed Q, g reads).
  auto h1 = [&](const QGTile *st, f32x16 &S, f32x16 &G) __attribute__((always_inline)) {
    int qperm = qperm_h;
    if (!kHoist) {
      qperm = swap_bits23(col);
      asm volatile("" : "+v"(qperm));
    }
    const uint4 *vrow = v_lds + key_in_tile * KCH;
    // D of this lane's 16 queries 8hh + {0..7} and 16 + 8hh + {0..7} (query q
    // sits in region q / 4 at slot 4 + q % 4); element r of the score tile
    // holds query r of that list, so D goes straight into the accumulator
    // that H = D - dP starts from
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const float4 b = reinterpret_cast<const float4 *>(st->ld + 8 * (4 * half + 2 * hh + rg))[1];
        G[8 * half + 4 * rg + 0] = b.x; G[8 * half + 4 * rg + 1] = b.y;
        G[8 * half + 4 * rg + 2] = b.z; G[8 * half + 4 * rg + 3] = b.w;
      }
    }
    S = f32x16{};
    if constexpr (kHoist) {
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const bf16x8 vf = as_bf16x8(vrow[(2 * t + hh) ^ sw<D>(key_in_tile)]);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(st->q, qperm, t, hh), kf[t], S, 0, 0, 0);
        G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand<D>(st->g, qperm, t, hh), vf, G, 0, 0, 0);
        if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound the operand prefetch
      }
    } else {
      uint32_t qy = 16u * uint32_t(hh ^ sw<D>(qperm)), vy = 16u * uint32_t(hh ^ sw<D>(key_in_tile));
      asm volatile("" : "+v"(qy), "+v"(vy));
      const char *qrow = reinterpret_cast<const char *>(st->q + qperm * KCH);
      const char *grow = reinterpret_cast<const char *>(st->g + qperm * KCH);
      const char *vr = reinterpret_cast<const char *>(vrow);
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const bf16x8 vf = row_read_xad(vr, t, vy);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_xad(qrow, t, qy), kf[t], S, 0, 0, 0);
        G = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_xad(grow, t, qy), vf, G, 0, 0, 0);
        if (t % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound the operand prefetch
      }
    }
  };
  auto h2 = [&](int2 ent, const QGTile *st, f32x16 S, const f32x16 &G) __attribute__((always_inline)) {
    // LSE of the same 16 queries (slot q % 4 of region q / 4)
    float lq[16];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        const float4 a = reinterpret_cast<const float4 *>(st->ld + 8 * (4 * half + 2 * hh + rg))[0];
        lq[8 * half + 4 * rg + 0] = a.x; lq[8 * half + 4 * rg + 1] = a.y;
        lq[8 * half + 4 * rg + 2] = a.z; lq[8 * half + 4 * rg + 3] = a.w;
      }
    }
    // partial block: scores of inadmissible pairs to -inf (scale > 0), whose
    // probability exp2 then makes exactly 0, and the LSE of a query without
    // keys (-inf) to 0 so that its pairs, all inadmissible, stay at exp2(-inf);
    // full blocks skip the mask
    if (ent.y >= 0) {
      const uint32_t bits = st->bits[key_in_tile] >> (8 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = (bits >> reg_pos(r)) & 1u ? S[r] : -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) lq[e] = lq[e] == -__builtin_inff() ? 0.f : lq[e];
    }
    // element r holds query r of the lane's list (8 (pos / 16) + pos % 8 = r
    // for pos = reg_pos(r)); gs = P (D - dP) = -dS, so dK is negated at the end
    float pr[16], gs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], sl2, -lq[r] * kLog2e));
      gs[r] = pr[r] * G[r];
    }
    bf16x8 pb[2], gsb[2];
    pb[0] = to_bf16x8(pr);
    pb[1] = to_bf16x8(pr + 8);
    gsb[0] = to_bf16x8(gs);
    gsb[1] = to_bf16x8(gs + 8);
    const TrLane tl = tl_h;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        accV[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(st->g, s, nt, tl.dcol, tl.krel),
                                                           pb[s], accV[nt], 0, 0, 0);
        accK[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(st->q, s, nt, tl.dcol, tl.krel),
                                                           gsb[s], accK[nt], 0, 0, 0);
        if (nt % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto sync = [&](int j) __attribute__((always_inline)) {
    if ((j + 1) % kEntChunk == 0 && j + 1 < n) {
      // the next chunk of entries, read after this barrier (entry(j + 1))
      load_entries((j + 1) / kEntChunk);
      wait_lgkmcnt0();
    }
    wait_vmcnt<0>();  // block j (and, first time, V and K) has landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Head dim 128 runs the two waves of a SIMD half a block apart, as the dQ
  // pass does.
  if constexpr (!kPingPong<D>) {
    auto step = [&](int j, const QGTile *st, int next_stage) __attribute__((always_inline)) {
      sync(j);
      const int2 ent = entry(j);
      f32x16 S, G;
      h1(st, S, G);
      if (j + 1 < n) issue(next_stage, entry(j + 1));  // its stage was released by the barrier
      h2(ent, st, S, G);
    };
    for (int j = 0; j < n; j += 2) {
      step(j, &ring[0], 1);
      if (j + 1 < n) step(j + 1, &ring[1], 0);
    }
  } else if (wave < 4) {
    auto step = [&](int j, const QGTile *st, int next_stage) __attribute__((always_inline)) {
      sync(j);
      const int2 ent = entry(j);
      f32x16 S, G;
      h1(st, S, G);
      if (j + 1 < n) issue(next_stage, entry(j + 1));  // its stage was released by the barrier
      h2(ent, st, S, G);
    };
    for (int j = 0; j < n; j += 3) {
      step(j, &ring[0], 1);
      if (j + 1 < n) step(j + 1, &ring[1], 2);
      if (j + 2 < n) step(j + 2, &ring[2], 0);
    }
  } else {
    f32x16 S = {}, G = {};
    int2 ent = make_int2(0, -1);
    auto step = [&](int j, const QGTile *st, const QGTile *prev, int next_stage) __attribute__((always_inline)) {
      sync(j);
      if (j + 1 < n) issue(next_stage, entry(j + 1));
      if (j > 0) h2(ent, prev, S, G);
      ent = entry(j);
      h1(st, S, G);
    };
    for (int j = 0; j < n; j += 3) {
      step(j, &ring[0], &ring[2], 1);
      if (j + 1 < n) step(j + 1, &ring[1], &ring[0], 2);
      if (j + 2 < n) step(j + 2, &ring[2], &ring[1], 0);
    }
    if (n > 0) h2(ent, &ring[(n - 1) % 3], S, G);
  }
  wait_vmcnt<0>();

  if (!kvalid) return;
  const int64_t ooff = koff + int64_t(krow_g) * p.k_sn;
  __bf16 *gk = static_cast<__bf16 *>(p.g_k) + ooff;
  __bf16 *gv = static_cast<__bf16 *>(p.g_v) + ooff;
#pragma unroll
  for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * nt + 8 * jj + 4 * hh;
      float xk[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xk[i] = accK[nt][4 * jj + i] * -p.scale;  // the accumulated -dS
        xv[i] = accV[nt][4 * jj + i];
      }
      *reinterpret_cast<uint2 *>(gk + d0) = make_uint2(pack_bf16(xk[0], xk[1]), pack_bf16(xk[2], xk[3]));
      *reinterpret_cast<uint2 *>(gv + d0) = make_uint2(pack_bf16(xv[0], xv[1]), pack_bf16(xv[2], xv[3]));
    }
  }
}

template <int D>
hipError_t launch(const BwdParams &p, hipStream_t s) {
  const int64_t Gq = int64_t(p.r_map.n_tiles) * p.B * p.H;
  const int64_t Gk = int64_t(p.c_map.n_tiles) * p.B * p.H;
  // the dQ pass stores D, which the dK/dV pass reads: same stream, in order
  hipLaunchKernelGGL((bwd_dq_wide_kernel<D>), dim3(unsigned(Gq)), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkv_wide_kernel<D>), dim3(unsigned(Gk)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int launch_bwd_bf16_wide(const BwdParams &p, int D, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return launch<128>(p, s);
  if (D == 64) return launch<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
