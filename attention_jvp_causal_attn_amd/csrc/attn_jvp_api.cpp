// C ABI entry points: argument validation, per-device schedule upload and
// kernel dispatch.  Every tensor stays caller-owned device memory; the only
// device memory the library owns is the per-mask tile schedule.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"

using attnjvp::DeviceSchedule;
using attnjvp::HostSchedule;
using attnjvp::KernelParams;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The bytes a strided tensor view covers: base + sum_k i_k * stride_k + e with
// 0 <= i_k < count_k and 0 <= e < width (the contiguous last dimension), all
// in bytes.  A contiguous buffer is a view without strided dimensions.
struct Extent {
  const void *base = nullptr;
  int n = 0;
  int64_t stride[3] = {0, 0, 0};
  int64_t count[3] = {1, 1, 1};
  int64_t width = 0;
};

Extent view_extent(const void *p, int64_t B, int64_t N, int64_t H, int64_t sb, int64_t sn,
                   int64_t sh, int64_t D, int64_t es) {
  Extent e;
  e.base = p;
  e.n = 3;
  e.stride[0] = sb * es; e.count[0] = B;
  e.stride[1] = sn * es; e.count[1] = N;
  e.stride[2] = sh * es; e.count[2] = H;
  e.width = D * es;
  return e;
}

Extent range_extent(const void *p, int64_t bytes) {
  Extent e;
  e.base = p;
  e.width = bytes;
  return e;
}

// Is some sum of c_k x_k, with lo_k <= x_k <= hi_k, inside [L, U] (and, with
// nonzero, some x_k != 0)?  Depth-first over the terms in decreasing |c|, each
// term's digits limited to those the remaining terms can still complete; a
// search that exceeds its node budget answers yes (the caller then refuses).
struct Term {
  __int128 c;
  int64_t lo, hi;
};

bool reachable(const Term *t, int n, __int128 L, __int128 U, bool nonzero, int64_t *budget) {
  if (--*budget < 0) return true;
  if (n == 0) return !nonzero && L <= 0 && 0 <= U;
  __int128 rmin = 0, rmax = 0;  // what terms 1 .. n-1 can add
  for (int k = 1; k < n; ++k) {
    const __int128 a = t[k].c * t[k].lo, b = t[k].c * t[k].hi;
    rmin += a < b ? a : b;
    rmax += a < b ? b : a;
  }
  // c x in [L - rmax, U - rmin]
  const __int128 c = t[0].c, lo_v = L - rmax, hi_v = U - rmin;
  auto fdiv = [](__int128 a, __int128 b) {  // floor(a / b), b > 0
    __int128 q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
  };
  __int128 x0, x1;
  if (c > 0) {
    x0 = -fdiv(-lo_v, c);  // ceil(lo_v / c)
    x1 = fdiv(hi_v, c);
  } else {
    x0 = -fdiv(hi_v, -c);  // ceil(hi_v / c) for c < 0
    x1 = fdiv(-lo_v, -c);
  }
  if (x0 < t[0].lo) x0 = t[0].lo;
  if (x1 > t[0].hi) x1 = t[0].hi;
  for (__int128 x = x0; x <= x1; ++x)
    if (reachable(t + 1, n - 1, L - c * x, U - c * x, nonzero && x == 0, budget)) return true;
  return false;
}

// At most two extents of three strided dimensions meet in a search.
constexpr int kMaxTerms = 6;

// Normalises the terms (positive coefficients, fixed terms folded into the
// target, terms of equal coefficient merged: x + y over two ranges takes
// every value of the summed range) and runs the search.  Only for the
// existence of a solution, so not with the nonzero condition.  No heap use.
bool search(const Term *terms, int n_terms, __int128 L, __int128 U) {
  Term live[kMaxTerms];
  int n = 0;
  for (int i = 0; i < n_terms; ++i) {
    Term t = terms[i];
    if (t.c < 0) t = {-t.c, -t.hi, -t.lo};
    if (t.c == 0 || t.hi == t.lo) {
      L -= t.c * t.lo;
      U -= t.c * t.lo;
      continue;
    }
    bool merged = false;
    for (int k = 0; k < n; ++k)
      if (live[k].c == t.c) {
        live[k].lo += t.lo;
        live[k].hi += t.hi;
        merged = true;
      }
    if (!merged) live[n++] = t;
  }
  std::sort(live, live + n, [](const Term &a, const Term &b) { return a.c > b.c; });
  int64_t budget = 1 << 20;
  return reachable(live, n, L, U, false, &budget);
}

// Do two extents share a byte?  (Exact unless the search budget runs out,
// which answers yes.)
bool extents_overlap(const Extent &a, const Extent &b) {
  if (!a.base || !b.base || a.width <= 0 || b.width <= 0) return false;
  Term t[kMaxTerms];
  int n = 0;
  for (int k = 0; k < a.n; ++k) t[n++] = {a.stride[k], 0, a.count[k] - 1};
  for (int k = 0; k < b.n; ++k) t[n++] = {-__int128(b.stride[k]), 0, b.count[k] - 1};
  const __int128 d = __int128(reinterpret_cast<uintptr_t>(b.base)) -
                     __int128(reinterpret_cast<uintptr_t>(a.base));
  // a + sa + e == b + sb + f  <=>  sa - sb == d + f - e, f - e in (-wa, wb)
  return search(t, n, d - (a.width - 1), d + (b.width - 1));
}

// Do two different index tuples of one extent share a byte (a view that
// writes some element twice)?
bool extent_self_overlaps(const Extent &a) {
  if (!a.base || a.width <= 0) return false;
  Term t[kMaxTerms];
  int n = 0;
  for (int k = 0; k < a.n; ++k) {
    if (a.count[k] < 2) continue;
    const int64_t c = a.stride[k] < 0 ? -a.stride[k] : a.stride[k];
    // a zero stride, or two strides of one size, give one address twice
    if (c == 0) return true;
    for (int i = 0; i < n; ++i)
      if (t[i].c == c) return true;
    t[n++] = {c, -(a.count[k] - 1), a.count[k] - 1};
  }
  std::sort(t, t + n, [](const Term &x, const Term &y) { return x.c > y.c; });
  int64_t budget = 1 << 20;
  return reachable(t, n, -(a.width - 1), a.width - 1, true, &budget);
}

// Outputs must not share a byte with any input, with another output or with
// themselves (a write race or a read of a value being overwritten).
int check_disjoint(const Extent *ins, int n_in, const Extent *outs, int n_out) {
  for (int i = 0; i < n_out; ++i) {
    if (extent_self_overlaps(outs[i])) return ATTN_JVP_ERR_UNSUPPORTED;
    for (int j = 0; j < n_in; ++j)
      if (extents_overlap(outs[i], ins[j])) return ATTN_JVP_ERR_UNSUPPORTED;
    for (int j = i + 1; j < n_out; ++j)
      if (extents_overlap(outs[i], outs[j])) return ATTN_JVP_ERR_UNSUPPORTED;
  }
  return ATTN_JVP_OK;
}

// Upload (once per device and tile shape) the schedule of m; caller holds m->mu.
int device_schedule_locked(const attn_jvp_mask *m, int device, int BM, int BN,
                           const DeviceSchedule **out) {
  auto key = std::make_tuple(device, BM, BN);
  auto it = m->dev_sched.find(key);
  if (it != m->dev_sched.end()) {
    *out = &it->second;
    return ATTN_JVP_OK;
  }
  int st = ATTN_JVP_OK;
  const HostSchedule *hs = attnjvp::host_schedule_locked(m, BM, BN, &st);
  if (!hs) return st;
  const size_t n_entries = hs->entry_block.size();
  const size_t off_bytes = (hs->tile_offsets.size() * 4 + 15) & ~size_t(15);
  const size_t ord_bytes = (hs->tile_order.size() * 4 + 15) & ~size_t(15);
  const size_t nf_bytes = (hs->tile_nfull.size() * 4 + 15) & ~size_t(15);
  const size_t ent_bytes = (n_entries * 8 + 15) & ~size_t(15);
  // partial blocks, then one all-ones block that full blocks point at
  const size_t ones_words = size_t(BM) * (BN / 32);
  const size_t bit_bytes = (hs->partial_bits.size() + ones_words) * 4;
  const size_t total = off_bytes + ord_bytes + nf_bytes + ent_bytes + bit_bytes + 16;
  std::vector<uint8_t> blob;
  try {
    blob.assign(total, 0);
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  std::memcpy(blob.data(), hs->tile_offsets.data(), hs->tile_offsets.size() * 4);
  std::memcpy(blob.data() + off_bytes, hs->tile_order.data(), hs->tile_order.size() * 4);
  std::memcpy(blob.data() + off_bytes + ord_bytes, hs->tile_nfull.data(), hs->tile_nfull.size() * 4);
  const size_t ent_at = off_bytes + ord_bytes + nf_bytes;
  int32_t *ent = reinterpret_cast<int32_t *>(blob.data() + ent_at);
  for (size_t e = 0; e < n_entries; ++e) {
    ent[2 * e] = hs->entry_block[e];
    ent[2 * e + 1] = hs->entry_partial[e];
  }
  uint8_t *bits_dst = blob.data() + ent_at + ent_bytes;
  if (!hs->partial_bits.empty())
    std::memcpy(bits_dst, hs->partial_bits.data(), hs->partial_bits.size() * 4);
  std::memset(bits_dst + hs->partial_bits.size() * 4, 0xff, ones_words * 4);
  void *dptr = nullptr;
  hipError_t err = hipMalloc(&dptr, total);
  if (err == hipErrorOutOfMemory) return ATTN_JVP_ERR_OOM;
  if (err != hipSuccess) return ATTN_JVP_ERR_HIP;
  err = hipMemcpy(dptr, blob.data(), total, hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    (void)hipFree(dptr);
    return ATTN_JVP_ERR_HIP;
  }
  DeviceSchedule ds;
  uint8_t *b = static_cast<uint8_t *>(dptr);
  ds.base = dptr;
  ds.tile_offsets = reinterpret_cast<const int32_t *>(b);
  ds.tile_order = reinterpret_cast<const int32_t *>(b + off_bytes);
  ds.tile_nfull = reinterpret_cast<const int32_t *>(b + off_bytes + ord_bytes);
  ds.entries = reinterpret_cast<const int2 *>(b + ent_at);
  ds.partial_bits = reinterpret_cast<const uint32_t *>(b + ent_at + ent_bytes);
  ds.n_tiles = hs->n_tiles;
  ds.n_partial = int32_t(hs->n_partial);
  auto res = m->dev_sched.emplace(key, ds);
  *out = &res.first->second;
  return ATTN_JVP_OK;
}

// Upload (once per device, tile shape and split count) the unit list of a
// split-key launch; caller holds m->mu.
int device_split_locked(const attn_jvp_mask *m, int device, int BM, int BN, int max_splits,
                        const attnjvp::DeviceSplit **out) {
  auto key = std::make_tuple(device, BM, BN, max_splits);
  auto it = m->dev_split.find(key);
  if (it != m->dev_split.end()) {
    *out = &it->second;
    return ATTN_JVP_OK;
  }
  int st = ATTN_JVP_OK;
  const attnjvp::HostSplit *hp = attnjvp::host_split_locked(m, BM, BN, max_splits, &st);
  if (!hp) return st;
  const attnjvp::HostSplit &h = *hp;
  const std::vector<int32_t> *parts[5] = {&h.unit_offsets, &h.unit_order, &h.unit_tile,
                                          &h.unit_part, &h.split_tiles};
  size_t at[5], total = 0;
  for (int i = 0; i < 5; ++i) {
    at[i] = total;
    total += (parts[i]->size() * 4 + 15) & ~size_t(15);
  }
  total += 16;
  std::vector<uint8_t> blob;
  try {
    blob.assign(total, 0);
  } catch (const std::bad_alloc &) {
    return ATTN_JVP_ERR_OOM;
  }
  for (int i = 0; i < 5; ++i)
    if (!parts[i]->empty()) std::memcpy(blob.data() + at[i], parts[i]->data(), parts[i]->size() * 4);
  void *dptr = nullptr;
  hipError_t err = hipMalloc(&dptr, total);
  if (err == hipErrorOutOfMemory) return ATTN_JVP_ERR_OOM;
  if (err != hipSuccess) return ATTN_JVP_ERR_HIP;
  err = hipMemcpy(dptr, blob.data(), total, hipMemcpyHostToDevice);
  if (err != hipSuccess) {
    (void)hipFree(dptr);
    return ATTN_JVP_ERR_HIP;
  }
  attnjvp::DeviceSplit ds;
  const uint8_t *b = static_cast<const uint8_t *>(dptr);
  ds.base = dptr;
  ds.unit_offsets = reinterpret_cast<const int32_t *>(b + at[0]);
  ds.unit_order = reinterpret_cast<const int32_t *>(b + at[1]);
  ds.unit_tile = reinterpret_cast<const int32_t *>(b + at[2]);
  ds.unit_part = reinterpret_cast<const int32_t *>(b + at[3]);
  ds.split_tiles = reinterpret_cast<const int32_t *>(b + at[4]);
  ds.n_units = h.n_units;
  ds.n_parts = h.n_parts;
  ds.n_split = int32_t(h.split_tiles.size() / 4);
  auto res = m->dev_split.emplace(key, ds);
  *out = &res.first->second;
  return ATTN_JVP_OK;
}

}  // namespace

// Free the device schedules of a mask (and of its cached transpose).
static void free_device_schedules(attn_jvp_mask *m) {
  int cur = -1;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto &kv : m->dev_sched) {
    const int dev = std::get<0>(kv.first);
    if (hipSetDevice(dev) == hipSuccess) (void)hipFree(kv.second.base);
  }
  for (auto &kv : m->dev_split) {
    const int dev = std::get<0>(kv.first);
    if (hipSetDevice(dev) == hipSuccess) (void)hipFree(kv.second.base);
  }
  if (have_cur && !(m->dev_sched.empty() && m->dev_split.empty())) (void)hipSetDevice(cur);
  m->dev_sched.clear();
  m->dev_split.clear();
  if (m->transposed) free_device_schedules(m->transposed.get());
}

extern "C" void attn_jvp_mask_free(attn_jvp_mask *m) {
  if (!m) return;
  free_device_schedules(m);
  delete m;
}

extern "C" int attn_jvp_tile_shape(int32_t dtype, int32_t D, int32_t tangent, int32_t *block_m,
                                   int32_t *block_n) {
  if (!block_m || !block_n) return ATTN_JVP_ERR_NULL;
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_F32) return ATTN_JVP_ERR_DTYPE;
  if (D != 64 && D != 128) return ATTN_JVP_ERR_UNSUPPORTED;
  if (dtype == ATTN_JVP_BF16) {
    *block_m = attnjvp::kBf16BlockMWide;
    // the head-dim-128 primal-only kernel works through 64-key blocks
    *block_n = (!tangent && D == 128) ? attnjvp::kBf16BlockNPrimal128 : attnjvp::kBf16BlockN;
  } else {
    *block_m = attnjvp::kF32BlockM;
    *block_n = attnjvp::kF32BlockN;
  }
  return ATTN_JVP_OK;
}

// Workgroup -> work item map (see work_item in internal.h).  The 8 XCDs are
// split into gcd(S, 8) groups sharing the S = B * H slices equally; the XCDs
// of a group interleave the tile slots of each of its slices.  Needs the
// slot count to split evenly over a group, else the identity map (which
// interleaves slots over all 8 XCDs) is used.
static attnjvp::WorkMap make_work_map(int64_t slices, int32_t n_tiles) {
  int64_t g = 8;
  while (slices % g != 0) g /= 2;
  const int m = int(8 / g);
  if (n_tiles % m == 0) return {n_tiles, m, int32_t(slices / g), n_tiles / m};
  return {n_tiles, 0, 0, 0};
}

static void set_work_map(attnjvp::KernelParams &p) {
  const attnjvp::WorkMap w = make_work_map(int64_t(p.B) * p.H, p.n_tiles);
  p.map_group = w.group;
  p.map_slices = w.slices;
  p.map_slots = w.slots;
}

// Argument checks shared by the forward entry points (no device access).
static int validate_fwd(const attn_jvp_args *a, const attn_jvp_mask *m, bool *tangent_out) {
  if (!a || !m) return ATTN_JVP_ERR_NULL;
  if (a->dtype != ATTN_JVP_BF16 && a->dtype != ATTN_JVP_F32) return ATTN_JVP_ERR_DTYPE;
  if (!a->q || !a->k || !a->v || !a->o || !a->lse) return ATTN_JVP_ERR_NULL;
  // any tangent given: JVP, the absent ones zero; none: primal only
  const bool tangent = a->dq != nullptr || a->dk != nullptr || a->dv != nullptr;
  if (tangent && !a->d_o) return ATTN_JVP_ERR_NULL;
  if (a->B <= 0 || a->H <= 0 || a->n_q <= 0 || a->n_k <= 0) return ATTN_JVP_ERR_SHAPE;
  if (a->D != 64 && a->D != 128) return ATTN_JVP_ERR_UNSUPPORTED;
  if (a->n_q != m->n_q || a->n_k != m->n_k) return ATTN_JVP_ERR_MASK;
  if (!(std::isfinite(a->scale))) return ATTN_JVP_ERR_SHAPE;
  if (int64_t(a->B) * a->H * a->n_q > (int64_t(1) << 40)) return ATTN_JVP_ERR_SHAPE;
  const int64_t es = a->dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int64_t qs[3] = {a->q_stride_b, a->q_stride_n, a->q_stride_h};
  const int64_t ks[3] = {a->k_stride_b, a->k_stride_n, a->k_stride_h};
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || ks[i] < 0) return ATTN_JVP_ERR_SHAPE;
    if ((qs[i] * es) % 16 || (ks[i] * es) % 16) return ATTN_JVP_ERR_ALIGN;
  }
  // the kernels address a 32-row block with 32-bit byte offsets
  if (ks[1] * es * 32 > int64_t(0x7fffffff) || qs[1] * es * 32 > int64_t(0x7fffffff))
    return ATTN_JVP_ERR_SHAPE;
  // rows of one head must not overlap the D contiguous elements of another
  if (a->H > 1 && (qs[2] < a->D || ks[2] < a->D)) return ATTN_JVP_ERR_SHAPE;
  const void *ins[6] = {a->q, a->k, a->v, a->dq, a->dk, a->dv};
  const void *outs[4] = {a->o, a->d_o, a->lse, a->d_lse};
  for (const void *p : ins)
    if (p && !aligned16(p)) return ATTN_JVP_ERR_ALIGN;
  for (const void *p : outs)
    if (p && !aligned16(p)) return ATTN_JVP_ERR_ALIGN;
  if (a->d_lse && !tangent) return ATTN_JVP_ERR_UNSUPPORTED;
  // no output may share a byte with an input or another output
  const Extent in_ext[6] = {
      view_extent(a->q, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
      view_extent(a->dq, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
      view_extent(a->k, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
      view_extent(a->v, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
      view_extent(a->dk, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
      view_extent(a->dv, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es)};
  const int64_t lse_bytes = int64_t(a->B) * a->H * a->n_q * 4;
  const Extent out_ext[4] = {
      view_extent(a->o, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
      range_extent(a->lse, lse_bytes),
      view_extent(tangent ? a->d_o : nullptr, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
      range_extent(tangent ? a->d_lse : nullptr, lse_bytes)};
  const int st = check_disjoint(in_ext, 6, out_ext, 4);
  if (st != ATTN_JVP_OK) return st;
  *tangent_out = tangent;
  return ATTN_JVP_OK;
}

static KernelParams fwd_params(const attn_jvp_args *a, bool tangent, const DeviceSchedule *ds) {
  KernelParams p;
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.o = a->o; p.d_o = tangent ? a->d_o : nullptr;
  p.lse = a->lse;
  p.d_lse = tangent ? a->d_lse : nullptr;
  p.q_sb = a->q_stride_b; p.q_sn = a->q_stride_n; p.q_sh = a->q_stride_h;
  p.k_sb = a->k_stride_b; p.k_sn = a->k_stride_n; p.k_sh = a->k_stride_h;
  p.B = a->B; p.H = a->H; p.n_q = a->n_q; p.n_k = a->n_k;
  p.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt(float(a->D));
  p.scale_log2 = float(double(p.scale) * 1.4426950408889634);
  p.tile_offsets = ds->tile_offsets;
  p.tile_order = ds->tile_order;
  p.tile_nfull = ds->tile_nfull;
  p.entries = ds->entries;
  p.partial_bits = ds->partial_bits;
  p.n_tiles = ds->n_tiles;
  p.n_partial = ds->n_partial;
  p.unit_tile = nullptr;
  p.unit_part = nullptr;
  p.part_stats = nullptr;
  p.part_acc = nullptr;
  p.n_parts = 0;
  set_work_map(p);
  return p;
}

static int launch_fwd(const KernelParams &p, const attn_jvp_args *a, bool tangent, void *stream) {
  const int err = a->dtype == ATTN_JVP_BF16 ? attnjvp::launch_bf16(p, a->D, tangent, stream)
                                            : attnjvp::launch_f32(p, a->D, tangent, stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ERR_HIP;
}

extern "C" int attn_jvp_fwd(const attn_jvp_args *a, const attn_jvp_mask *m, void *stream) {
  bool tangent = false;
  int st = validate_fwd(a, m, &tangent);
  if (st != ATTN_JVP_OK) return st;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return ATTN_JVP_ERR_HIP;
  int BM = 0, BN = 0;
  attn_jvp_tile_shape(a->dtype, a->D, tangent, &BM, &BN);
  const DeviceSchedule *ds = nullptr;
  {
    std::lock_guard<std::mutex> lock(m->mu);
    st = device_schedule_locked(m, device, BM, BN, &ds);
    if (st != ATTN_JVP_OK) return st;
  }
  if (int64_t(ds->n_tiles) * a->B * a->H > int64_t(0x7fffffff)) return ATTN_JVP_ERR_SHAPE;
  return launch_fwd(fwd_params(a, tangent, ds), a, tangent, stream);
}

// Workspace bytes of a split launch with n_parts partial slots per slice:
// float4 statistics, then 2 * D fp32 accumulators, per (slice, slot, row).
static int64_t split_workspace_bytes(const attn_jvp_args *a, int BM, int64_t n_parts) {
  const int64_t rows = int64_t(a->B) * a->H * n_parts * BM;
  return rows * 16 + rows * 2 * a->D * 4;
}

extern "C" int attn_jvp_fwd_split_workspace(const attn_jvp_args *a, const attn_jvp_mask *m,
                                            int32_t max_splits, uint64_t *bytes) {
  if (!bytes) return ATTN_JVP_ERR_NULL;
  bool tangent = false;
  int st = validate_fwd(a, m, &tangent);
  if (st != ATTN_JVP_OK) return st;
  if (max_splits < 1) return ATTN_JVP_ERR_SHAPE;
  int BM = 0, BN = 0;
  attn_jvp_tile_shape(a->dtype, a->D, tangent, &BM, &BN);
  std::lock_guard<std::mutex> lock(m->mu);
  const attnjvp::HostSplit *h = attnjvp::host_split_locked(m, BM, BN, max_splits, &st);
  if (!h) return st;
  *bytes = uint64_t(split_workspace_bytes(a, BM, h->n_parts));
  return ATTN_JVP_OK;
}

// Predicted time, in units of one key block, of running the unit list of a
// split on `slots` concurrent workgroups: units start heaviest first, each on
// the slot that frees up first (the dispatcher's behaviour for a grid larger
// than the chip); a unit costs its entries plus a fixed start-up cost, and a
// unit of a cut tile a further cost for its partial sums and their merge.
static double predicted_blocks(const attnjvp::HostSplit &h, int64_t slices, int64_t slots) {
  constexpr double kStart = 2.0, kPartial = 2.0;
  std::vector<double> cost;
  cost.reserve(h.unit_order.size());
  for (int u : h.unit_order)
    cost.push_back(double(h.unit_offsets[u + 1] - h.unit_offsets[u]) + kStart +
                   (h.unit_part[u] >= 0 ? kPartial : 0.0));
  // min-heap of slot finish times; every slice walks the same unit list
  std::vector<double> heap(size_t(std::max<int64_t>(1, slots)), 0.0);
  auto cmp = [](double x, double y) { return x > y; };
  double makespan = 0.0;
  for (int64_t s = 0; s < slices; ++s)
    for (double c : cost) {
      std::pop_heap(heap.begin(), heap.end(), cmp);
      heap.back() += c;
      makespan = std::max(makespan, heap.back());
      std::push_heap(heap.begin(), heap.end(), cmp);
    }
  return makespan;
}

extern "C" int attn_jvp_split_choose(const attn_jvp_args *a, const attn_jvp_mask *m,
                                     int32_t n_cu, int32_t *max_splits) {
  if (!max_splits) return ATTN_JVP_ERR_NULL;
  bool tangent = false;
  int st = validate_fwd(a, m, &tangent);
  if (st != ATTN_JVP_OK) return st;
  if (n_cu < 1) return ATTN_JVP_ERR_SHAPE;
  int BM = 0, BN = 0;
  attn_jvp_tile_shape(a->dtype, a->D, tangent, &BM, &BN);
  // workgroups resident per compute unit: one for the bf16 kernels (their
  // registers fill the SIMDs) but the head-dim-64 primal one (four waves per
  // SIMD: two), two for the fp32 kernel
  const bool two = a->dtype != ATTN_JVP_BF16 || (!tangent && a->D == 64);
  const int64_t slots = int64_t(n_cu) * (two ? 2 : 1);
  const int64_t slices = int64_t(a->B) * a->H;
  std::lock_guard<std::mutex> lock(m->mu);
  const attnjvp::HostSplit *h1 = attnjvp::host_split_locked(m, BM, BN, 1, &st);
  if (!h1) return st;
  // no split unless the grid leaves compute units idle: then splitting
  // only adds partial sums
  if (int64_t(h1->n_units) * slices >= 2 * slots) {
    *max_splits = 1;
    return ATTN_JVP_OK;
  }
  const double base = predicted_blocks(*h1, slices, slots);
  int best = 1;
  double best_t = base;
  for (int S = 2; S <= 16; ++S) {
    const attnjvp::HostSplit *h = attnjvp::host_split_locked(m, BM, BN, S, &st);
    if (!h) return st;
    const double t = predicted_blocks(*h, slices, slots);
    if (t < best_t) {
      best_t = t;
      best = S;
    }
  }
  // keep the plain launch unless the split is clearly faster
  *max_splits = best_t < 0.85 * base ? best : 1;
  return ATTN_JVP_OK;
}

// The split-key launch on a given workspace (see attn_jvp_fwd_split).  With
// resident_only, nothing is built, uploaded or allocated: the mask's unit
// list and its device copies for this device must already be cached
// (ERR_NOT_READY otherwise), and a workspace smaller than the launch needs is
// ERR_SCRATCH rather than ERR_SHAPE.
int attnjvp::fwd_split(const attn_jvp_args *a, const attn_jvp_mask *m, int32_t max_splits,
                       void *workspace, uint64_t workspace_bytes, void *stream,
                       bool resident_only) {
  bool tangent = false;
  int st = validate_fwd(a, m, &tangent);
  if (st != ATTN_JVP_OK) return st;
  if (max_splits < 1) return ATTN_JVP_ERR_SHAPE;
  if (workspace && !aligned16(workspace)) return ATTN_JVP_ERR_ALIGN;
  int BM = 0, BN = 0;
  attn_jvp_tile_shape(a->dtype, a->D, tangent, &BM, &BN);
  int64_t need = 0, n_units = 0, n_split = 0;
  {
    std::lock_guard<std::mutex> lock(m->mu);
    const attnjvp::HostSplit *h = nullptr;
    if (resident_only) {
      auto it = m->host_split.find(std::make_tuple(BM, BN, int(max_splits)));
      if (it == m->host_split.end()) return ATTN_JVP_ERR_NOT_READY;
      h = &it->second;
    } else {
      h = attnjvp::host_split_locked(m, BM, BN, max_splits, &st);
      if (!h) return st;
    }
    need = split_workspace_bytes(a, BM, h->n_parts);
    n_units = h->n_units;
    n_split = int64_t(h->split_tiles.size() / 4);
  }
  if (need > 0 && !workspace) return ATTN_JVP_ERR_NULL;
  if (uint64_t(need) > workspace_bytes)
    return resident_only ? ATTN_JVP_ERR_SCRATCH : ATTN_JVP_ERR_SHAPE;
  const int64_t slices = int64_t(a->B) * a->H;
  if (n_units * slices > int64_t(0x7fffffff) || n_split * slices * BM > int64_t(0x7fffffff))
    return ATTN_JVP_ERR_SHAPE;
  if (workspace && need > 0) {
    // the workspace must not share a byte with a tensor the launch reads or
    // writes
    const int64_t es = a->dtype == ATTN_JVP_BF16 ? 2 : 4;
    const int64_t lse_bytes = int64_t(a->B) * a->H * a->n_q * 4;
    const void *qside[4] = {a->q, a->dq, a->o, tangent ? a->d_o : nullptr};
    const void *kside[4] = {a->k, a->v, a->dk, a->dv};
    Extent t[10];
    for (int i = 0; i < 4; ++i) {
      t[i] = view_extent(qside[i], a->B, a->n_q, a->H, a->q_stride_b, a->q_stride_n,
                         a->q_stride_h, a->D, es);
      t[4 + i] = view_extent(kside[i], a->B, a->n_k, a->H, a->k_stride_b, a->k_stride_n,
                             a->k_stride_h, a->D, es);
    }
    t[8] = range_extent(a->lse, lse_bytes);
    t[9] = range_extent(tangent ? a->d_lse : nullptr, lse_bytes);
    const Extent w = range_extent(workspace, need);
    for (const Extent &x : t)
      if (extents_overlap(w, x)) return ATTN_JVP_ERR_UNSUPPORTED;
  }
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return ATTN_JVP_ERR_HIP;
  const DeviceSchedule *ds = nullptr;
  const attnjvp::DeviceSplit *sp = nullptr;
  {
    std::lock_guard<std::mutex> lock(m->mu);
    if (resident_only) {
      auto is = m->dev_sched.find(std::make_tuple(device, BM, BN));
      auto ip = m->dev_split.find(std::make_tuple(device, BM, BN, int(max_splits)));
      if (is == m->dev_sched.end() || ip == m->dev_split.end()) return ATTN_JVP_ERR_NOT_READY;
      ds = &is->second;
      sp = &ip->second;
    } else {
      st = device_schedule_locked(m, device, BM, BN, &ds);
      if (st != ATTN_JVP_OK) return st;
      st = device_split_locked(m, device, BM, BN, max_splits, &sp);
      if (st != ATTN_JVP_OK) return st;
    }
  }

  KernelParams p = fwd_params(a, tangent, ds);
  p.tile_offsets = sp->unit_offsets;
  p.tile_order = sp->unit_order;
  p.n_tiles = sp->n_units;
  p.unit_tile = sp->unit_tile;
  p.unit_part = sp->unit_part;
  p.n_parts = sp->n_parts;
  const int64_t rows = slices * sp->n_parts * BM;
  p.part_stats = static_cast<float *>(workspace);
  p.part_acc = sp->n_parts ? static_cast<float *>(workspace) + rows * 4 : nullptr;
  set_work_map(p);
  st = launch_fwd(p, a, tangent, stream);
  if (st != ATTN_JVP_OK || sp->n_split == 0) return st;

  attnjvp::MergeParams mp;
  mp.o = a->o; mp.d_o = tangent ? a->d_o : nullptr;
  mp.lse = a->lse; mp.d_lse = p.d_lse;
  mp.q_sb = a->q_stride_b; mp.q_sn = a->q_stride_n; mp.q_sh = a->q_stride_h;
  mp.B = a->B; mp.H = a->H; mp.n_q = a->n_q;
  mp.block_m = BM;
  mp.split_tiles = sp->split_tiles;
  mp.n_split = sp->n_split;
  mp.part_stats = p.part_stats;
  mp.part_acc = p.part_acc;
  mp.n_parts = sp->n_parts;
  const int err = attnjvp::launch_merge(mp, a->D, a->dtype == ATTN_JVP_BF16, tangent, stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ERR_HIP;
}

extern "C" int attn_jvp_fwd_split(const attn_jvp_args *a, const attn_jvp_mask *m,
                                  int32_t max_splits, void *workspace, uint64_t workspace_bytes,
                                  void *stream) {
  return attnjvp::fwd_split(a, m, max_splits, workspace, workspace_bytes, stream, false);
}

extern "C" int attn_jvp_bwd(const attn_jvp_bwd_args *a, const attn_jvp_mask *m, void *stream) {
  if (!a || !m) return ATTN_JVP_ERR_NULL;
  if (a->dtype != ATTN_JVP_BF16 && a->dtype != ATTN_JVP_F32) return ATTN_JVP_ERR_DTYPE;
  if (!a->q || !a->k || !a->v || !a->o || !a->g_o || !a->lse || !a->g_q || !a->g_k || !a->g_v ||
      !a->delta)
    return ATTN_JVP_ERR_NULL;
  if (a->B <= 0 || a->H <= 0 || a->n_q <= 0 || a->n_k <= 0) return ATTN_JVP_ERR_SHAPE;
  if (a->D != 64 && a->D != 128) return ATTN_JVP_ERR_UNSUPPORTED;
  if (a->n_q != m->n_q || a->n_k != m->n_k) return ATTN_JVP_ERR_MASK;
  if (!(std::isfinite(a->scale))) return ATTN_JVP_ERR_SHAPE;
  if (int64_t(a->B) * a->H * std::max(a->n_q, a->n_k) > (int64_t(1) << 40)) return ATTN_JVP_ERR_SHAPE;
  const int64_t es = a->dtype == ATTN_JVP_BF16 ? 2 : 4;
  const int64_t qs[3] = {a->q_stride_b, a->q_stride_n, a->q_stride_h};
  const int64_t ks[3] = {a->k_stride_b, a->k_stride_n, a->k_stride_h};
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || ks[i] < 0) return ATTN_JVP_ERR_SHAPE;
    if ((qs[i] * es) % 16 || (ks[i] * es) % 16) return ATTN_JVP_ERR_ALIGN;
  }
  // 32-row blocks are addressed with 32-bit byte offsets
  if (ks[1] * es * 32 > int64_t(0x7fffffff) || qs[1] * es * 32 > int64_t(0x7fffffff))
    return ATTN_JVP_ERR_SHAPE;
  if (a->H > 1 && (qs[2] < a->D || ks[2] < a->D)) return ATTN_JVP_ERR_SHAPE;
  const void *ins[6] = {a->q, a->k, a->v, a->o, a->g_o, a->lse};
  const void *outs[4] = {a->g_q, a->g_k, a->g_v, a->delta};
  for (const void *p : ins)
    if (!aligned16(p)) return ATTN_JVP_ERR_ALIGN;
  for (const void *p : outs)
    if (!aligned16(p)) return ATTN_JVP_ERR_ALIGN;
  {
    // no output may share a byte with an input or another output
    const int64_t rows_bytes = int64_t(a->B) * a->H * a->n_q * 4;
    const Extent in_ext[6] = {
        view_extent(a->q, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
        view_extent(a->o, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
        view_extent(a->g_o, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
        view_extent(a->k, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
        view_extent(a->v, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
        range_extent(a->lse, rows_bytes)};
    const Extent out_ext[4] = {
        view_extent(a->g_q, a->B, a->n_q, a->H, qs[0], qs[1], qs[2], a->D, es),
        view_extent(a->g_k, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
        view_extent(a->g_v, a->B, a->n_k, a->H, ks[0], ks[1], ks[2], a->D, es),
        range_extent(a->delta, rows_bytes)};
    const int st = check_disjoint(in_ext, 6, out_ext, 4);
    if (st != ATTN_JVP_OK) return st;
  }

  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return ATTN_JVP_ERR_HIP;
  const bool bf16 = a->dtype == ATTN_JVP_BF16;
  const int BM = !bf16 ? attnjvp::kF32BlockM
                       : attnjvp::kBwdBlockMWide;
  const int BN = bf16 ? attnjvp::kBwdBlockN : attnjvp::kF32BlockN;
  const DeviceSchedule *rs = nullptr, *cs = nullptr;
  const attn_jvp_mask *t = nullptr;
  {
    std::lock_guard<std::mutex> lock(m->mu);
    int st = device_schedule_locked(m, device, BM, BN, &rs);
    if (st != ATTN_JVP_OK) return st;
    if (!m->transposed) {
      attn_jvp_mask *tm = nullptr;
      st = attnjvp::transpose_mask(m, &tm);
      if (st != ATTN_JVP_OK) return st;
      m->transposed.reset(tm);
    }
    t = m->transposed.get();
  }
  {
    std::lock_guard<std::mutex> lock(t->mu);
    int st = device_schedule_locked(t, device, BM, BN, &cs);
    if (st != ATTN_JVP_OK) return st;
  }
  const int64_t slices = int64_t(a->B) * a->H;
  if (int64_t(rs->n_tiles) * slices > int64_t(0x7fffffff) ||
      int64_t(cs->n_tiles) * slices > int64_t(0x7fffffff))
    return ATTN_JVP_ERR_SHAPE;

  attnjvp::BwdParams p;
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.g_o = a->g_o; p.lse = a->lse;
  p.g_q = a->g_q; p.g_k = a->g_k; p.g_v = a->g_v; p.delta = a->delta;
  p.q_sb = a->q_stride_b; p.q_sn = a->q_stride_n; p.q_sh = a->q_stride_h;
  p.k_sb = a->k_stride_b; p.k_sn = a->k_stride_n; p.k_sh = a->k_stride_h;
  p.B = a->B; p.H = a->H; p.n_q = a->n_q; p.n_k = a->n_k;
  p.scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt(float(a->D));
  p.scale_log2 = float(double(p.scale) * 1.4426950408889634);
  p.r_offsets = rs->tile_offsets; p.r_order = rs->tile_order; p.r_entries = rs->entries;
  p.r_bits = rs->partial_bits; p.r_partial = rs->n_partial;
  p.r_map = make_work_map(slices, rs->n_tiles);
  p.c_offsets = cs->tile_offsets; p.c_order = cs->tile_order; p.c_entries = cs->entries;
  p.c_bits = cs->partial_bits; p.c_partial = cs->n_partial;
  p.c_map = make_work_map(slices, cs->n_tiles);
  const int err = !bf16 ? attnjvp::launch_bwd_f32(p, a->D, stream)
                       : attnjvp::launch_bwd_bf16_wide(p, a->D, stream);
  return err == hipSuccess ? ATTN_JVP_OK : ATTN_JVP_ERR_HIP;
}

extern "C" const char *attn_jvp_status_str(int status) {
  switch (status) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_ERR_NULL: return "required pointer is NULL";
    case ATTN_JVP_ERR_SHAPE: return "invalid or inconsistent sizes";
    case ATTN_JVP_ERR_DTYPE: return "unknown dtype";
    case ATTN_JVP_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case ATTN_JVP_ERR_MASK: return "malformed mask or mask size mismatch";
    case ATTN_JVP_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_JVP_ERR_HIP: return "HIP device unavailable or HIP call failed";
    case ATTN_JVP_ERR_OOM: return "out of memory";
    case ATTN_JVP_ERR_NOT_READY:
      return "mask schedule not resident on this device for this split count (run "
             "attn_jvp_fwd_split once first)";
    case ATTN_JVP_ERR_SCRATCH:
      return "launch needs more workspace than the fixed scratch buffer holds";
    default: return "unknown status";
  }
}

extern "C" int attn_jvp_version(void) { return ATTN_JVP_API_VERSION; }
