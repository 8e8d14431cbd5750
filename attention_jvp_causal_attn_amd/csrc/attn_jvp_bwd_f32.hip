// Masked attention backward in fp32 (fp32 in, fp32 arithmetic): the gradients
// of L = sum(g_o * O) with respect to Q, K and V, reusing the forward's LSE
// ("Causal-rCM ..." summary, Appendix B: LSE is returned so that later passes
// need not recompute the softmax normaliser).  With s = scale q.k over the
// admissible pairs, P = exp(s - LSE), dP = g_o V^T and D_i = <g_o_i, O_i>:
//     dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T g_o.
// Two launches, like the bf16 path: a dQ pass over the mask's query tiles
// (which also writes D) and a dK/dV pass over the key tiles of the
// transposed mask.  Every output element is written once; no atomics.
//
// Layout: a workgroup of 256 threads owns 64 rows (query rows, or key rows
// in the second pass) of one (batch, head); 4 consecutive lanes share a row,
// each holding D/4 of its dimensions.  Blocks of 32 rows of the other side
// are staged in LDS; per pair the 4 lanes reduce their partial dot products
// with two xor-shuffles.  This path serves small fp32 problems, bound by the
// fp32 vector ALUs.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attnjvp {
namespace {

constexpr int kThreads = 256;
constexpr int BM = kF32BlockM;  // 64 rows
constexpr int BN = kF32BlockN;  // 32 rows of the other side per block
constexpr int TPR = 4;          // lanes per row
static_assert(BM * TPR == kThreads, "one row per 4 lanes");

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

// Stage rows r0 .. r0 + BN - 1 of two [n, D] fp32 tensors (row stride sn) into
// LDS with padded rows; rows at or past n are zero.
template <int D>
__device__ __forceinline__ void stage_two(float *A, float *B, const float *a, const float *b,
                                          int64_t sn, int r0, int n) {
  constexpr int LD = D + 4;
  for (int i = threadIdx.x; i < BN * D / 4; i += kThreads) {
    const int r = i / (D / 4), c = (i % (D / 4)) * 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
    if (r0 + r < n) {
      const int64_t off = int64_t(r0 + r) * sn + c;
      x = *reinterpret_cast<const float4 *>(a + off);
      y = *reinterpret_cast<const float4 *>(b + off);
    }
    *reinterpret_cast<float4 *>(&A[r * LD + c]) = x;
    *reinterpret_cast<float4 *>(&B[r * LD + c]) = y;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(BwdParams p) {
  constexpr int DS = D / TPR, LD = D + 4;
  __shared__ float Ks[BN * LD], Vs[BN * LD];

  const int L = work_item(int(blockIdx.x), p.r_map);
  const int slot = L % p.r_map.n_tiles;
  const int bh = L / p.r_map.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int tile = p.r_order[slot];
  const int tid = threadIdx.x;
  const int row_in_tile = tid / TPR, d0 = (tid % TPR) * DS;
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;

  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh + int64_t(qrow) * p.q_sn;
  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const float *kg = static_cast<const float *>(p.k) + koff;
  const float *vg = static_cast<const float *>(p.v) + koff;

  float q[DS], g[DS], acc[DS];
  float dsum = 0.f;
#pragma unroll
  for (int x = 0; x < DS; ++x) {
    q[x] = qvalid ? static_cast<const float *>(p.q)[qoff + d0 + x] : 0.f;
    g[x] = qvalid ? static_cast<const float *>(p.g_o)[qoff + d0 + x] : 0.f;
    const float o = qvalid ? static_cast<const float *>(p.o)[qoff + d0 + x] : 0.f;
    dsum = __builtin_fmaf(g[x], o, dsum);
    acc[x] = 0.f;
  }
  const float delta = quad_sum(dsum);
  const int64_t li = (int64_t(batch) * p.H + head) * p.n_q + qrow;
  const float lse = qvalid ? p.lse[li] : 0.f;
  if (qvalid && tid % TPR == 0) p.delta[li] = delta;

  const int e0 = p.r_offsets[tile], e1 = p.r_offsets[tile + 1];
  for (int e = e0; e < e1; ++e) {
    const int2 ent = p.r_entries[e];
    __syncthreads();
    stage_two<D>(Ks, Vs, kg, vg, p.k_sn, ent.x * BN, p.n_k);
    __syncthreads();
    const uint32_t bits = ent.y >= 0 ? p.r_bits[int64_t(ent.y) * BM + row_in_tile] : ~0u;
#pragma unroll 4
    for (int j = 0; j < BN; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < DS; ++x) {
        s = __builtin_fmaf(q[x], Ks[j * LD + d0 + x], s);
        dp = __builtin_fmaf(g[x], Vs[j * LD + d0 + x], dp);
      }
      s = quad_sum(s);
      dp = quad_sum(dp);
      const bool ok = qvalid && ((bits >> j) & 1u);
      const float pr = ok ? expf(__builtin_fmaf(s, p.scale, -lse)) : 0.f;
      const float ds = pr * (dp - delta);
#pragma unroll
      for (int x = 0; x < DS; ++x) acc[x] = __builtin_fmaf(ds, Ks[j * LD + d0 + x], acc[x]);
    }
  }
  if (!qvalid) return;
  float *out = static_cast<float *>(p.g_q) + qoff + d0;
#pragma unroll
  for (int x = 0; x < DS; ++x) out[x] = acc[x] * p.scale;
}

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkv_f32_kernel(BwdParams p) {
  constexpr int DS = D / TPR, LD = D + 4;
  __shared__ float Qs[BN * LD], Gs[BN * LD], Ls[BN], Dl[BN];

  const int L = work_item(int(blockIdx.x), p.c_map);
  const int slot = L % p.c_map.n_tiles;
  const int bh = L / p.c_map.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int tile = p.c_order[slot];
  const int tid = threadIdx.x;
  const int row_in_tile = tid / TPR, d0 = (tid % TPR) * DS;
  const int krow = tile * BM + row_in_tile;
  const bool kvalid = krow < p.n_k;

  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh + int64_t(krow) * p.k_sn;
  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh;
  const float *qg = static_cast<const float *>(p.q) + qoff;
  const float *gg = static_cast<const float *>(p.g_o) + qoff;
  const float *lse = p.lse + (int64_t(batch) * p.H + head) * p.n_q;
  const float *dl = p.delta + (int64_t(batch) * p.H + head) * p.n_q;

  float k[DS], v[DS], dk[DS], dv[DS];
#pragma unroll
  for (int x = 0; x < DS; ++x) {
    k[x] = kvalid ? static_cast<const float *>(p.k)[koff + d0 + x] : 0.f;
    v[x] = kvalid ? static_cast<const float *>(p.v)[koff + d0 + x] : 0.f;
    dk[x] = 0.f;
    dv[x] = 0.f;
  }

  const int e0 = p.c_offsets[tile], e1 = p.c_offsets[tile + 1];
  for (int e = e0; e < e1; ++e) {
    const int2 ent = p.c_entries[e];
    const int q0 = ent.x * BN;
    __syncthreads();
    stage_two<D>(Qs, Gs, qg, gg, p.q_sn, q0, p.n_q);
    if (tid < BN) {
      const bool in = q0 + tid < p.n_q;
      Ls[tid] = in ? lse[q0 + tid] : 0.f;
      Dl[tid] = in ? dl[q0 + tid] : 0.f;
    }
    __syncthreads();
    const uint32_t bits = ent.y >= 0 ? p.c_bits[int64_t(ent.y) * BM + row_in_tile] : ~0u;
#pragma unroll 4
    for (int i = 0; i < BN; ++i) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < DS; ++x) {
        s = __builtin_fmaf(k[x], Qs[i * LD + d0 + x], s);
        dp = __builtin_fmaf(v[x], Gs[i * LD + d0 + x], dp);
      }
      s = quad_sum(s);
      dp = quad_sum(dp);
      const bool ok = kvalid && ((bits >> i) & 1u);
      const float pr = ok ? expf(__builtin_fmaf(s, p.scale, -Ls[i])) : 0.f;
      const float ds = pr * (dp - Dl[i]);
#pragma unroll
      for (int x = 0; x < DS; ++x) {
        dv[x] = __builtin_fmaf(pr, Gs[i * LD + d0 + x], dv[x]);
        dk[x] = __builtin_fmaf(ds, Qs[i * LD + d0 + x], dk[x]);
      }
    }
  }
  if (!kvalid) return;
  float *ok_ = static_cast<float *>(p.g_k) + koff + d0;
  float *ov = static_cast<float *>(p.g_v) + koff + d0;
#pragma unroll
  for (int x = 0; x < DS; ++x) {
    ok_[x] = dk[x] * p.scale;
    ov[x] = dv[x];
  }
}

template <int D>
hipError_t launch(const BwdParams &p, hipStream_t stream) {
  const int64_t slices = int64_t(p.B) * p.H;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3(unsigned(p.r_map.n_tiles * slices)),
                     dim3(kThreads), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_dkv_f32_kernel<D>), dim3(unsigned(p.c_map.n_tiles * slices)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int launch_bwd_f32(const BwdParams &p, int D, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return launch<128>(p, s);
  if (D == 64) return launch<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
