// lora_host.h -- host-side launchers shared by the library's translation
// units.  Internal to the library (not part of the ABI).
#pragma once

#include <algorithm>
#include <atomic>

#include "../../include/lora_mi355x.h"
#include "lora_common.h"

namespace lora {

constexpr int kMaxDevices = 64;

// Workgroups of one kernel that fit on the current device at once: its
// occupancy per CU (registers, LDS) times the CU count.  `cache` is the
// caller's table for that kernel, filled on first use per device.
inline int resident_groups(std::atomic<int> (&cache)[kMaxDevices], const void *kernel, int threads,
                           size_t lds_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_bytes) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 8;
  (void)hipGetLastError();  // a failed query must not be reported by the next launch
  const int v = per_cu * cus;
  if (cached) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Grid of a work-list kernel: a multiple of 8 (one share per XCD), no more
// than `resident` workgroups and no more than `bound` items need.
inline int xcd_grid(int64_t bound, int resident) {
  const int64_t per_xcd = std::max<int64_t>(1, std::min<int64_t>((bound + 7) / 8, resident / 8));
  return (int)(8 * per_xcd);
}

struct ShrinkConfig {
  int use_mma_mode;  // 1: matrix-core kernel, 0: vector kernel
  int kc, kch;       // k-chunk length and count
  int64_t bound;     // items at most
  int grid;          // vector kernel's grid
};

ShrinkConfig plan_shrink(int64_t T, int32_t S, int64_t d_in, int32_t R, bool bf16, int mode);
size_t shrink_ws_bytes(const ShrinkConfig &c, int64_t T, int32_t n_slices, int32_t R);

// Rendezvous words of the split decode kernel, at the start of every apply
// workspace: per work tile one range of kSplitMembers words for each of up to
// kSplitRanges slices that run side by side, for tile indices below
// kSyncTiles, then one row of counters (word 0: waits that gave up; word 1:
// flags found raised from another XCD).  A word holds the number of split
// calls that raised it (bits 31:17, modulo 2^15), its tile (bits 16:6), its
// range (bits 5:4) and the XCD of the member that raised it last (bits 3:0).
// The region must be zero before the first call on a workspace; every call raises each word of each range it uses exactly once,
// so the words of a range stay equal between calls.  The split kernel runs
// only for T * n_slices * max(r, 16) <= 2^17 tokens x ranks, so T <= 8192 and
// a batch has at most 8192 / 64 + 1023 + 1 = 1152 tiles.
constexpr int kSplitMembers = 16;
constexpr int kSplitRanges = 4;
constexpr int kSplitFlagWords = kSplitMembers * kSplitRanges;  // per tile
constexpr int kSyncTiles = 1152;
constexpr size_t kSyncBytes = sizeof(uint32_t) * kSplitFlagWords * (kSyncTiles + 1);
static_assert(kSyncBytes % 256 == 0, "the rank buffer after the count words stays 256-byte aligned");
static_assert(kSyncBytes == LORA_APPLY_SYNC_BYTES, "the C header states the region's size");

// The metadata workspace past the tile list holds the counts of the
// several-workgroup metadata path: per part of the rows, its count of each key
// and its bad ids.
constexpr int kMetaPartRows = 1024;  // rows per part, up to kMetaMaxParts parts
constexpr int kMetaMaxParts = 64;
inline int meta_parts(int64_t T) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(kMetaMaxParts, (T + kMetaPartRows - 1) / kMetaPartRows));
}
inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }
inline size_t meta_tiles_bytes(int64_t T, int32_t S) {
  return round256(sizeof(int32_t) * kTileInts * (size_t)max_tiles(T, S));
}
inline size_t meta_counts_bytes(int64_t T, int32_t S) {
  const size_t K = (size_t)S + 1;
  return round256(sizeof(int32_t) * (size_t)meta_parts(T) * (K + 1));
}
int meta_multi_knob();

hipError_t launch_meta(const int32_t *token_slot, int64_t T, int32_t S, int32_t *sorted,
                       int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count, int32_t *seg_start,
                       int32_t *info, int32_t *tiles, hipStream_t stream);
// the same over the T * topk (token, choice) pairs of a top-k routing step,
// keyed by (slot, local expert): S * E_local keys
hipError_t launch_meta_moe(const int32_t *topk_ids, int64_t T, int32_t topk, const int32_t *token_slot,
                           int32_t S, int32_t E_global, int32_t E_local, const int32_t *expert_map,
                           int32_t *sorted, int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count,
                           int32_t *seg_start, int32_t *info, int32_t *tiles, hipStream_t stream);

// R: the rank the kernels are built for (8, 16, 32, 64 or 128); ra: the
// caller's r_max (a multiple of 8, at most R), the row stride of A and of the
// caller's u.  for_apply: u is written in sorted-position order with row
// stride R, and with a split d_in the
// partial sums are left in ws for the expand to add (kch_out reports the
// split); to_partials: the sums go to ws even without a split (kch = 1);
// a_rank_rows: A_s[slot] is [ra][d_in] (the matrix-core path only: bf16,
// R >= 16, mode AUTO or SGMV)
// The rank the kernels are built for: the smallest of 8, 16, 32, 64, 128 that
// holds r_max (0 when r_max is not a multiple of 8 in [8, 128]).
inline int32_t tile_rank(int32_t r_max) {
  if (r_max < 8 || r_max > 128 || r_max % 8) return 0;
  int32_t R = 8;
  while (R < r_max) R *= 2;
  return R;
}

hipError_t launch_shrink(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                         int32_t n_slices, const void *const *A, const int64_t *a_stride,
                         int32_t R, int32_t ra, float scale, const float *slot_scale, const int32_t *slot_rank,
                         float *u, int mode, void *ws, bool for_apply, int *kch_out, hipStream_t stream,
                         bool to_partials = false, bool a_rank_rows = false);
// R, ra: as for the shrink (B holds ra rank rows per slot).  u_mode 0: u
// [n_slices][T][ra] in token order (the caller's); 1: [n_slices][T][R] in
// sorted-position order; 2: kch partial sums [kch][n_slices][T][R] in
// sorted-position order.  b_out_rows: B_s[slot] is [w][ra] (the matrix-core
// kernel only: bf16, R <= 64)
hipError_t launch_expand(const MetaView &meta, const float *u, int u_mode, int kch, int32_t n_slices,
                         const void *const *B, const int64_t *b_stride, const int64_t *width,
                         const int64_t *offset, int32_t R, int32_t ra, const int32_t *slot_rank, void *y,
                         int64_t ldy, bool bf16, int add, int mode, hipStream_t stream, bool b_out_rows = false);

// The long-segment expand (whole 64-token tiles, 512-column chunks) serves
// this call?  Decided from host-known sizes only.
bool expand_rows_fits(int64_t T, int32_t S, bool bf16, int mode, int32_t R);
bool expand_rows_addressable(int64_t T, int32_t n_slices, const int64_t *width, const int64_t *offset, int64_t ldy,
                             int32_t R);
int expand_rows_knob();
// It runs on the shrink's partial sums [kch][n_slices][T][R] (sorted order),
// folded into one bf16 plane at `planes` (n_slices * T * R * 2 bytes).
hipError_t launch_expand_rows(const MetaView &meta, const float *part, int kch, uint16_t *planes, int32_t n_slices,
                              const void *const *B, const int64_t *b_stride, const int64_t *width,
                              const int64_t *offset, int32_t R, int32_t ra, const int32_t *slot_rank, void *y,
                              int64_t ldy, int add, hipStream_t stream);

// The fused BGMV kernel (one workgroup per token) serves this call?  Decided
// from host-known sizes only.
bool bgmv_fits(int64_t T, int32_t S, int64_t d_in, int32_t n_slices, const int64_t *width, int32_t R,
               int64_t ldy, bool bf16, int mode);
hipError_t launch_bgmv(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                       int32_t n_slices, const void *const *A, const int64_t *a_stride,
                       const void *const *B, const int64_t *b_stride, const int64_t *width,
                       const int64_t *offset, int32_t R, float scale, const float *slot_scale,
                       const int32_t *slot_rank, void *y, int64_t ldy, int add, hipStream_t stream);
bool fused_disabled();

// The fused kernel with each work tile split over several workgroups (bf16,
// decode-shaped calls).  sync: the count words (kSyncBytes, above);
// part: workspace of split_ws_bytes bytes for the partial rank rows.  *used is
// false when the call is not one it takes.
size_t split_ws_bytes(int64_t T, int32_t S, int32_t n_slices, int32_t R);
hipError_t launch_bgmv_split(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, int32_t n_slices,
                             const void *const *A, const int64_t *a_stride, const void *const *B,
                             const int64_t *b_stride, const int64_t *width, const int64_t *offset, int32_t R,
                             float scale, const float *slot_scale, const int32_t *slot_rank, void *y, int64_t ldy,
                             int add, uint32_t *sync, float *part, size_t part_bytes, hipStream_t stream,
                             bool *used);
bool split_disabled();
int split_spin_limit();
int split_members();

// A measurement build (-DLORA_PHASE_CLOCK): the buffer lora_debug_phase_clock
// set and its size in 64-bit words, and the tile kernel asked to record into
// it (environment LORA_PHASE_KERNEL: "shrink" 1, "expand" 2, else 0; the split
// decode kernel always records).  Other builds: null, 0.
unsigned long long *phase_clock_buffer(size_t *words);
int phase_clock_kernel();

}  // namespace lora
