// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <tuple>
#include <vector>

#include <hip/hip_runtime.h>

#include "attn_jvp.h"

namespace attnjvp {

// Host-side block schedule of one mask for one tile shape (see
// attn_jvp_mask_schedule in attn_jvp.h for the meaning of every array).
struct HostSchedule {
  int32_t block_m = 0, block_n = 0;
  int32_t n_tiles = 0;
  std::vector<int32_t> tile_offsets;   // n_tiles + 1
  std::vector<int32_t> tile_order;     // n_tiles, heaviest first
  std::vector<int32_t> tile_nfull;     // n_tiles: full blocks lead each tile's entries
  std::vector<int32_t> entry_block;    // n_entries
  std::vector<int32_t> entry_partial;  // n_entries, -1 = full block
  std::vector<uint32_t> partial_bits;  // n_partial * block_m * (block_n / 32)
  int64_t n_partial = 0;
};

// The pieces (units) of a split-key launch, derived from a HostSchedule:
// every query tile's entries are cut into consecutive runs of at most
// unit_len entries (a tile without entries is one empty unit).
struct HostSplit {
  int32_t unit_len = 0;
  int32_t n_units = 0;
  int32_t n_parts = 0;                 // units of tiles that were cut
  std::vector<int32_t> unit_offsets;   // n_units + 1, into the schedule's entries
  std::vector<int32_t> unit_order;     // n_units, most entries first
  std::vector<int32_t> unit_tile;      // n_units
  std::vector<int32_t> unit_part;      // n_units, -1 for a tile's only unit
  std::vector<int32_t> split_tiles;    // 4 per cut tile: tile, first slot, count, 0
};

// Device copy of a HostSplit (one allocation); entries and mask bits stay
// those of the unsplit DeviceSchedule.
struct DeviceSplit {
  void *base = nullptr;
  const int32_t *unit_offsets = nullptr;
  const int32_t *unit_order = nullptr;
  const int32_t *unit_tile = nullptr;
  const int32_t *unit_part = nullptr;
  const int32_t *split_tiles = nullptr;
  int32_t n_units = 0;
  int32_t n_parts = 0;
  int32_t n_split = 0;
};

// One device copy of a schedule: a single allocation holding, in order,
// tile_offsets, tile_order, entries (block, partial) interleaved, bits.
struct DeviceSchedule {
  void *base = nullptr;
  const int32_t *tile_offsets = nullptr;
  const int32_t *tile_order = nullptr;
  const int32_t *tile_nfull = nullptr;
  const int2 *entries = nullptr;
  const uint32_t *partial_bits = nullptr;  // n_partial + 1 blocks; the last is all ones
  int32_t n_tiles = 0;
  int32_t n_partial = 0;
};

// Everything a kernel launch needs, passed by value.
struct KernelParams {
  const void *q, *k, *v, *dq, *dk, *dv;
  void *o, *d_o;
  float *lse;
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int32_t B, H, n_q, n_k;
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e): scores go to exp2 directly
  const int32_t *tile_offsets;
  const int32_t *tile_order;
  const int32_t *tile_nfull;
  const int2 *entries;
  const uint32_t *partial_bits;  // n_partial blocks, then one all-ones block
  int32_t n_tiles;
  int32_t n_partial;
  // Workgroup -> (slice, tile slot) map, see work_item().  map_group = 0:
  // identity; else XCDs form groups of map_group, each group owning
  // map_slices consecutive (batch, head) slices, member XCD u of a group
  // taking tile slots u, u + map_group, ... (map_slots of them) of each.
  int32_t map_group;
  int32_t map_slices;
  int32_t map_slots;
  float *d_lse;  // optional tangent of LSE (JVP kernels only)
  // Split-key launches: the schedule's "tiles" are pieces (units) of query
  // tiles; unit_tile maps a unit to its query tile and unit_part to its
  // partial slot (-1: the unit is its tile's only one and finishes itself).
  // Units with a slot write float4 (m, l, mu, 0) per row to part_stats and
  // the unnormalised accumulators (A, then T: 2 * D floats) per row to
  // part_acc, at row (slice * n_parts + slot) * block_m + row in tile.  m is
  // in the kernel's exponent base (bf16 kernels: log2 units of scale * q.k;
  // fp32 kernel: natural units).  NULL unit_tile: units are the tiles.
  const int32_t *unit_tile;
  const int32_t *unit_part;
  float *part_stats;
  float *part_acc;
  int32_t n_parts;
};

// The merge of split units: for every query tile that was cut, combine its
// units' partials (rescaled to the largest m) and write O, dO, LSE, d_lse.
struct MergeParams {
  void *o, *d_o;
  float *lse, *d_lse;
  int64_t q_sb, q_sn, q_sh;
  int32_t B, H, n_q;
  int32_t block_m;
  const int32_t *split_tiles;  // n_split x (tile, first slot, slot count, 0)
  int32_t n_split;
  const float *part_stats;
  const float *part_acc;
  int32_t n_parts;
};

// One grid's workgroup -> work item map (see work_item).
struct WorkMap {
  int32_t n_tiles;  // tiles per (batch, head) slice
  int32_t group;    // 0: identity map
  int32_t slices;
  int32_t slots;
};

// Everything the two backward launches need, passed by value.  The dQ pass
// walks query tiles over key blocks (the mask's schedule); the dK/dV pass
// walks key tiles over query blocks (the schedule of the transposed mask).
struct BwdParams {
  const void *q, *k, *v, *o, *g_o;
  const float *lse;
  void *g_q, *g_k, *g_v;
  float *delta;
  int64_t q_sb, q_sn, q_sh;
  int64_t k_sb, k_sn, k_sh;
  int32_t B, H, n_q, n_k;
  float scale, scale_log2;
  // query tiles x key blocks
  const int32_t *r_offsets, *r_order;
  const int2 *r_entries;
  const uint32_t *r_bits;  // r_partial blocks, then one all-ones block
  int32_t r_partial;
  WorkMap r_map;
  // key tiles x query blocks
  const int32_t *c_offsets, *c_order;
  const int2 *c_entries;
  const uint32_t *c_bits;  // c_partial blocks, then one all-ones block
  int32_t c_partial;
  WorkMap c_map;
};

#if defined(__HIP__)
// Workgroup w is dispatched to XCD w % 8 (its position in that XCD's stream
// is w / 8).  Returns the work item (slice * n_tiles + slot) of w: each XCD
// receives an equal share of work (interleaved heavy-first slots) and the
// workgroups resident on one XCD at a time belong to the same slice, so they
// stream the same key blocks through that XCD's L2.
__device__ __forceinline__ int work_item(int w, const WorkMap &m) {
  if (m.group == 0) return w;
  const int x = w & 7, local = w >> 3;
  const int grp = x / m.group, mem = x % m.group;
  const int sl = local / m.slots, k = local % m.slots;
  return (grp * m.slices + sl) * m.n_tiles + mem + k * m.group;
}
__device__ __forceinline__ int work_item(int w, const KernelParams &p) {
  return work_item(w, WorkMap{p.n_tiles, p.map_group, p.map_slices, p.map_slots});
}
#endif

}  // namespace attnjvp

struct attn_jvp_mask {
  int32_t n_q = 0, n_k = 0;
  std::vector<int32_t> group_q_begin;  // n_groups + 1
  std::vector<int32_t> range_ptr;      // n_groups + 1
  std::vector<int32_t> k_begin, k_end; // n_ranges
  int64_t n_visible = 0;

  mutable std::mutex mu;
  // (block_m, block_n) -> host schedule
  mutable std::map<std::pair<int, int>, attnjvp::HostSchedule> host_sched;
  // (device, block_m, block_n) -> device copy
  mutable std::map<std::tuple<int, int, int>, attnjvp::DeviceSchedule> dev_sched;
  // (block_m, block_n, max_splits) -> host split schedule
  mutable std::map<std::tuple<int, int, int>, attnjvp::HostSplit> host_split;
  // (device, block_m, block_n, max_splits) -> device split schedule
  mutable std::map<std::tuple<int, int, int, int>, attnjvp::DeviceSplit> dev_split;
  // the transposed mask (keys as rows), built on first use by the backward
  mutable std::unique_ptr<attn_jvp_mask> transposed;
};

namespace attnjvp {

// The mask with query and key roles swapped: key j admits query i exactly
// when query i admits key j.  Canonical like every other mask.
int transpose_mask(const attn_jvp_mask *m, attn_jvp_mask **out);

// Build (or fetch the cached) host schedule; caller holds m->mu.
const HostSchedule *host_schedule_locked(const attn_jvp_mask *m, int block_m,
                                         int block_n, int *status);

// Cut the tiles of a schedule into units of at most
// ceil(max entries of a tile / max_splits) entries (max_splits >= 1).
int split_schedule(const HostSchedule &s, int max_splits, HostSplit *out);

// Build (or fetch the cached) split of the (block_m, block_n) schedule;
// caller holds m->mu.
const HostSplit *host_split_locked(const attn_jvp_mask *m, int block_m, int block_n,
                                   int max_splits, int *status);

// The split-key launch of attn_jvp_fwd_split on a given workspace; with
// resident_only it builds, uploads and allocates nothing (ERR_NOT_READY when
// the mask's split schedule is not cached for this device, ERR_SCRATCH when
// the workspace is too small).
int fwd_split(const attn_jvp_args *a, const attn_jvp_mask *m, int32_t max_splits,
              void *workspace, uint64_t workspace_bytes, void *stream, bool resident_only);

// Kernel launchers (defined in the .hip files).  Return a hipError_t value.
int launch_bf16(const KernelParams &p, int D, bool tangent, void *stream);
int launch_bwd_bf16_wide(const BwdParams &p, int D, void *stream);
int launch_bwd_f32(const BwdParams &p, int D, void *stream);
int launch_f32(const KernelParams &p, int D, bool tangent, void *stream);
int launch_merge(const MergeParams &p, int D, bool bf16, bool tangent, void *stream);

// Tile shapes of the kernels.
constexpr int kBf16BlockMWide = 256;  // 8 waves x 32 rows (head dims 64 and 128)
constexpr int kBf16BlockN = 32;
constexpr int kBf16BlockNPrimal128 = 64;  // head-dim-128 primal-only kernel
constexpr int kBwdBlockMWide = 256;   // backward: 8 waves x 32 rows (or keys)
constexpr int kBwdBlockN = 32;        // backward: blocks of 32 keys (or queries)
constexpr int kF32BlockM = 64;
constexpr int kF32BlockN = 32;
// Largest schedule (query tile, key block entries) of one tile shape: entry
// offsets and partial-block indices are int32 on the device.
constexpr int32_t kMaxScheduleEntries = 0x7fffffff;

}  // namespace attnjvp
