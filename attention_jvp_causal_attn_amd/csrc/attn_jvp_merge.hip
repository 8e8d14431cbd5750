// Merge of the pieces of split query tiles (split-key launches).
//
// "Causal-rCM ..." summary, Appendix B: the kernel works through the
// admissible key ranges of a tile in parallel.  A piece s of a query row
// leaves its running max m_s, its sums l_s = sum exp(s - m_s) and
// mu_s = sum exp(s - m_s) ds, and its unnormalised accumulators
// A_s = sum exp(s - m_s) v and T_s = sum exp(s - m_s) (ds v + dv).  With
// M = max_s m_s and w_s = exp(m_s - M) the row's full sums are the w-weighted
// sums of the pieces' (pieces without an admissible key, l_s = 0, drop out),
// and the row finishes as in the unsplit kernels: O = A / l,
// dO = T / l - O mu / l, LSE = M + ln l, dLSE = mu / l.
//
// Layout: TPR = D / 4 lanes per row, each owning 4 consecutive dimensions
// (one 16-byte load per piece and accumulator); a workgroup covers
// 256 / TPR rows of one cut tile of one (batch, head) slice.  The kernel is
// bound by reading the partials (2 * D * 4 bytes per piece and row).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attnjvp {
namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round to nearest even, two values at a time.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// BF16: partials come from the bf16 kernels (m in log2 units, outputs bf16);
// else from the fp32 kernel (m in natural units, outputs fp32).
template <int D, bool BF16, bool TAN>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;
  constexpr int RPW = kThreads / TPR;
  const int groups = p.block_m / RPW;
  const int64_t w = blockIdx.x;
  const int g = int(w % groups);
  const int64_t rest = w / groups;
  const int cut = int(rest % p.n_split);
  const int bh = int(rest / p.n_split);
  const int tile = p.split_tiles[4 * cut];
  const int first = p.split_tiles[4 * cut + 1];
  const int count = p.split_tiles[4 * cut + 2];
  const int r = g * RPW + int(threadIdx.x) / TPR;
  const int c = (int(threadIdx.x) % TPR) * 4;
  const int qrow = tile * p.block_m + r;
  if (qrow >= p.n_q) return;
  const int head = bh % p.H, batch = bh / p.H;
  const int64_t row0 = (int64_t(bh) * p.n_parts + first) * p.block_m + r;

  float M = kNegInf;
  for (int s = 0; s < count; ++s) {
    const float4 st = *reinterpret_cast<const float4 *>(p.part_stats + (row0 + int64_t(s) * p.block_m) * 4);
    if (st.y > 0.f) M = fmaxf(M, st.x);
  }
  float l = 0.f, mu = 0.f;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, t[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < count; ++s) {
    const int64_t row = row0 + int64_t(s) * p.block_m;
    const float4 st = *reinterpret_cast<const float4 *>(p.part_stats + row * 4);
    if (!(st.y > 0.f)) continue;
    const float wgt = BF16 ? exp2f(st.x - M) : expf(st.x - M);
    l = __builtin_fmaf(wgt, st.y, l);
    if (TAN) mu = __builtin_fmaf(wgt, st.z, mu);
    const float *pa = p.part_acc + row * (2 * D) + c;
    const float4 av = *reinterpret_cast<const float4 *>(pa);
    a[0] = __builtin_fmaf(wgt, av.x, a[0]);
    a[1] = __builtin_fmaf(wgt, av.y, a[1]);
    a[2] = __builtin_fmaf(wgt, av.z, a[2]);
    a[3] = __builtin_fmaf(wgt, av.w, a[3]);
    if (TAN) {
      const float4 tv = *reinterpret_cast<const float4 *>(pa + D);
      t[0] = __builtin_fmaf(wgt, tv.x, t[0]);
      t[1] = __builtin_fmaf(wgt, tv.y, t[1]);
      t[2] = __builtin_fmaf(wgt, tv.z, t[2]);
      t[3] = __builtin_fmaf(wgt, tv.w, t[3]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float mu_n = mu * inv;
  float o[4], dout[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = a[i] * inv;
    if (TAN) dout[i] = __builtin_fmaf(-o[i], mu_n, t[i] * inv);
  }
  const int64_t ooff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh + int64_t(qrow) * p.q_sn + c;
  if (BF16) {
    *reinterpret_cast<uint2 *>(static_cast<__bf16 *>(p.o) + ooff) =
        make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
    if (TAN)
      *reinterpret_cast<uint2 *>(static_cast<__bf16 *>(p.d_o) + ooff) =
          make_uint2(pack_bf16(dout[0], dout[1]), pack_bf16(dout[2], dout[3]));
  } else {
    *reinterpret_cast<float4 *>(static_cast<float *>(p.o) + ooff) = make_float4(o[0], o[1], o[2], o[3]);
    if (TAN)
      *reinterpret_cast<float4 *>(static_cast<float *>(p.d_o) + ooff) =
          make_float4(dout[0], dout[1], dout[2], dout[3]);
  }
  if (c == 0) {
    const int64_t li = (int64_t(batch) * p.H + head) * p.n_q + qrow;
    p.lse[li] = l > 0.f ? (BF16 ? (M + log2f(l)) * kLn2 : M + logf(l)) : kNegInf;
    if (TAN && p.d_lse) p.d_lse[li] = mu_n;
  }
}

template <int D, bool BF16, bool TAN>
hipError_t launch(const MergeParams &p, hipStream_t stream) {
  constexpr int RPW = kThreads / (D / 4);
  const int64_t G = int64_t(p.block_m / RPW) * p.n_split * p.B * p.H;
  hipLaunchKernelGGL((merge_kernel<D, BF16, TAN>), dim3(unsigned(G)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const MergeParams &p, bool bf16, bool tangent, hipStream_t s) {
  if (bf16) return tangent ? launch<D, true, true>(p, s) : launch<D, true, false>(p, s);
  return tangent ? launch<D, false, true>(p, s) : launch<D, false, false>(p, s);
}

}  // namespace

int launch_merge(const MergeParams &p, int D, bool bf16, bool tangent, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.block_m % (kThreads / (D / 4)) != 0) return hipErrorInvalidValue;
  if (D == 128) return launch_d<128>(p, bf16, tangent, s);
  if (D == 64) return launch_d<64>(p, bf16, tangent, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
