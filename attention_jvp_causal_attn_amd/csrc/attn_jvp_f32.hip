// Fused primal + tangent masked attention in fp32 (fp32 in, fp32 arithmetic).
//
// The same online-softmax recurrence as the bf16 kernel ("Causal-rCM ..."
// summary, Appendix B: tangent and primal share one pass and one rescaling;
// masked pairs carry no tangent) done on the vector ALUs in full fp32, so the
// result stays within fp32 rounding of the exact operator (no reduced-
// precision products anywhere).  This path serves small fp32 problems; it is
// not the throughput path.
//
// Layout: a workgroup of 512 threads owns 64 query rows of one (batch, head);
// 8 aligned lanes share a row, each holding D/8 of its dimensions of q, dq
// and the two accumulators.  Key blocks of 32 rows of K, dK, V, dV are staged
// in LDS and taken 16 keys at a time by the online softmax; per key the 8
// lanes reduce their partial dot products in three DPP steps (every lane
// ends with the same bits).  On small problems this path is bound by each
// wave's chain of dependent vector instructions, which more lanes per row
// (fewer dimensions each) shorten.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace attnjvp {
namespace {

constexpr int kThreads = 512;
constexpr int BM = kF32BlockM;  // 64 rows
constexpr int BN = kF32BlockN;  // 32 keys per staged block
constexpr int HB = 16;          // keys per online-softmax step
constexpr int TPR = 8;          // lanes per row
static_assert(BM * TPR == kThreads, "one row per 8 lanes");
constexpr float kNegInf = -__builtin_inff();

// DPP move within rows of 16 lanes (bound_ctrl off, all rows and banks).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Sum over the 8 aligned lanes of a row: add the value of lane l ^ 1 and
// l ^ 2 (quad permutations), then of the lane mirrored within 8.  Each step
// adds two sums of the same shape and a + b == b + a, so every lane ends
// with the same bits.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_mov<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  return x;
}

template <int D, bool TAN>
__global__ __launch_bounds__(kThreads) void attn_jvp_f32_kernel(KernelParams p) {
  constexpr int DS = D / TPR;   // dims per lane
  constexpr int LD = D + 4;     // padded LDS row (floats)
  __shared__ float Ks[BN * LD], dKs[BN * LD], Vs[BN * LD], dVs[BN * LD];

  const int L = work_item(int(blockIdx.x), p);
  const int slot = L % p.n_tiles;
  const int bh = L / p.n_tiles;
  const int head = bh % p.H, batch = bh / p.H;
  const int unit = p.tile_order[slot];  // a query tile, or a piece of one (split launch)
  const int tile = p.unit_tile ? p.unit_tile[unit] : unit;

  const int tid = threadIdx.x;
  const int row_in_tile = tid / TPR, part = tid % TPR;
  const int qrow = tile * BM + row_in_tile;
  const bool qvalid = qrow < p.n_q;
  const int d0 = part * DS;

  const int64_t qoff = int64_t(batch) * p.q_sb + int64_t(head) * p.q_sh + int64_t(qrow) * p.q_sn;
  const int64_t koff = int64_t(batch) * p.k_sb + int64_t(head) * p.k_sh;
  const float *kg = static_cast<const float *>(p.k) + koff;
  const float *vg = static_cast<const float *>(p.v) + koff;
  // absent tangent tensors (NULL) are zero
  const float *dkg = TAN && p.dk ? static_cast<const float *>(p.dk) + koff : nullptr;
  const float *dvg = TAN && p.dv ? static_cast<const float *>(p.dv) + koff : nullptr;

  float q[DS], dq[DS], acc[DS], tac[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    q[e] = qvalid ? static_cast<const float *>(p.q)[qoff + d0 + e] : 0.f;
    dq[e] = (TAN && qvalid && p.dq) ? static_cast<const float *>(p.dq)[qoff + d0 + e] : 0.f;
    acc[e] = 0.f;
    tac[e] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f, mu_run = 0.f;

  const int e0 = p.tile_offsets[unit], e1 = p.tile_offsets[unit + 1];
  for (int e = e0; e < e1; ++e) {
    const int2 ent = p.entries[e];
    const int key0 = ent.x * BN;
    __syncthreads();
    for (int i = tid; i < BN * D / 4; i += kThreads) {
      const int r = i / (D / 4), c = (i % (D / 4)) * 4;
      const int key = key0 + r;
      float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      float4 kk = z, vv = z, dkk = z, dvv = z;
      if (key < p.n_k) {
        const int64_t off = int64_t(key) * p.k_sn + c;
        kk = *reinterpret_cast<const float4 *>(kg + off);
        vv = *reinterpret_cast<const float4 *>(vg + off);
        if (TAN && dkg) dkk = *reinterpret_cast<const float4 *>(dkg + off);
        if (TAN && dvg) dvv = *reinterpret_cast<const float4 *>(dvg + off);
      }
      *reinterpret_cast<float4 *>(&Ks[r * LD + c]) = kk;
      *reinterpret_cast<float4 *>(&Vs[r * LD + c]) = vv;
      if (TAN) {
        *reinterpret_cast<float4 *>(&dKs[r * LD + c]) = dkk;
        *reinterpret_cast<float4 *>(&dVs[r * LD + c]) = dvv;
      }
    }
    __syncthreads();
    const uint32_t bits = ent.y >= 0 ? p.partial_bits[int64_t(ent.y) * BM + row_in_tile] : ~0u;

#pragma unroll
    for (int h = 0; h < BN / HB; ++h) {
      float s[HB], ds[HB];
      float mx = kNegInf;
#pragma unroll
      for (int jj = 0; jj < HB; ++jj) {
        const int j = h * HB + jj;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int x = 0; x < DS; ++x) {
          a = fmaf(q[x], Ks[j * LD + d0 + x], a);
          if (TAN) {
            b = fmaf(dq[x], Ks[j * LD + d0 + x], b);
            b = fmaf(q[x], dKs[j * LD + d0 + x], b);
          }
        }
        a = sum8(a);
        if (TAN) b = sum8(b);
        const bool ok = (bits >> j) & 1u;
        s[jj] = ok ? a * p.scale : kNegInf;
        ds[jj] = ok ? b * p.scale : 0.f;
        mx = fmaxf(mx, s[jj]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = expf(m_run - m_use);
      float lsum = 0.f, musum = 0.f;
#pragma unroll
      for (int jj = 0; jj < HB; ++jj) {
        s[jj] = expf(s[jj] - m_use);  // now the weight p_j
        lsum += s[jj];
        if (TAN) musum = __builtin_fmaf(s[jj], ds[jj], musum);
      }
      l_run = l_run * alpha + lsum;
      if (TAN) mu_run = mu_run * alpha + musum;
      m_run = m_new;
#pragma unroll
      for (int x = 0; x < DS; ++x) {
        float a = acc[x] * alpha, t = tac[x] * alpha;
#pragma unroll
        for (int jj = 0; jj < HB; ++jj) {
          const int j = h * HB + jj;
          const float vj = Vs[j * LD + d0 + x];
          a = fmaf(s[jj], vj, a);
          if (TAN) t = fmaf(s[jj], fmaf(ds[jj], vj, dVs[j * LD + d0 + x]), t);
        }
        acc[x] = a;
        tac[x] = t;
      }
    }
  }

  if (!qvalid) return;
  const int slot_part = p.unit_part ? p.unit_part[unit] : -1;
  if (slot_part >= 0) {
    // one piece of a split tile: running statistics (natural units) and
    // unnormalised sums, combined by the merge kernel
    const int64_t prow = (int64_t(bh) * p.n_parts + slot_part) * BM + row_in_tile;
    if (part == 0)
      *reinterpret_cast<float4 *>(p.part_stats + prow * 4) =
          make_float4(m_run, l_run, TAN ? mu_run : 0.f, 0.f);
    float *pa = p.part_acc + prow * (2 * D) + d0;
#pragma unroll
    for (int x = 0; x < DS; ++x) {
      pa[x] = acc[x];
      if (TAN) pa[D + x] = tac[x];
    }
    return;
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float mu_n = mu_run * inv;
  if (part == 0) {
    const int64_t li = (int64_t(batch) * p.H + head) * p.n_q + qrow;
    p.lse[li] = l_run > 0.f ? m_run + logf(l_run) : kNegInf;
    if (TAN && p.d_lse) p.d_lse[li] = mu_n;
  }
  float *o = static_cast<float *>(p.o) + qoff + d0;
  float *dout = TAN ? static_cast<float *>(p.d_o) + qoff + d0 : nullptr;
#pragma unroll
  for (int x = 0; x < DS; ++x) {
    const float ov = acc[x] * inv;
    o[x] = ov;
    if (TAN) dout[x] = __builtin_fmaf(-ov, mu_n, tac[x] * inv);
  }
}

template <int D, bool TAN>
hipError_t launch(const KernelParams &p, hipStream_t stream) {
  const int64_t G = int64_t(p.n_tiles) * p.B * p.H;
  hipLaunchKernelGGL((attn_jvp_f32_kernel<D, TAN>), dim3(unsigned(G)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int launch_f32(const KernelParams &p, int D, bool tangent, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128) return tangent ? launch<128, true>(p, s) : launch<128, false>(p, s);
  if (D == 64) return tangent ? launch<64, true>(p, s) : launch<64, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attnjvp
