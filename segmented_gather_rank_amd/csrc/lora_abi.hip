// lora_abi.hip -- the extern "C" entry points declared in include/lora_mi355x.h:
// argument checks, workspace layout, dispatch to the kernels.  Every check that
// can fail runs before the first HIP call, so a rejected call enqueues nothing.
#include <algorithm>
#include <cstdlib>
#include <mutex>

#include "../../include/lora_mi355x.h"
#include "lora_host.h"

// Workspace of lora_apply_noalloc: a static device array of the library, one
// copy per device, zero at load (so its count words start initialised).
// In host code its name stands for a host-side shadow, not a device address:
// a device's copy is reached only through the address hipGetSymbolAddress
// gives on that device (scratch_of_current_device, below).
static constexpr size_t kScratchBytes = (size_t)LORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= lora::kSyncBytes, "scratch holds the count words");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace lora {

static int env_int(const char *name, int dflt) {
  const char *v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int x = std::atoi(v);
  return x > 0 ? x : dflt;
}
// Tuning override: LORA_DISABLE_FUSED_BGMV=1 keeps lora_apply on the
// shrink + expand kernels even where the fused kernel fits.
bool fused_disabled() {
  static const bool v = env_int("LORA_DISABLE_FUSED_BGMV", 0) > 0;
  return v;
}
// LORA_DISABLE_SPLIT_BGMV=1 keeps decode-shaped bf16 calls on the one-workgroup-
// per-token fused kernel.
bool split_disabled() {
  static const bool v = env_int("LORA_DISABLE_SPLIT_BGMV", 0) > 0;
  return v;
}
// Looks a workgroup of the split kernel takes at its peers' partials before it
// computes the missing members' partials itself (LORA_SPLIT_SPIN_LIMIT, 0
// allowed): each look is one L2 round trip and a short sleep, under a
// microsecond.
int split_spin_limit() {
  static const int v = [] {
    const char *e = std::getenv("LORA_SPLIT_SPIN_LIMIT");
    return e && *e ? std::max(0, std::atoi(e)) : 4096;
  }();
  return v;
}
// LORA_EXPAND_ROWS=0 or 1: keep long batches off, or put every bf16 AUTO/SGMV
// batch on, the long-segment expand (tuning); unset: chosen by size.
int expand_rows_knob() {
  static const int v = [] {
    const char *e = std::getenv("LORA_EXPAND_ROWS");
    return e && *e ? (std::atoi(e) > 0 ? 1 : 0) : -1;
  }();
  return v;
}
// LORA_META_MULTI=0 or 1: build the metadata on one workgroup, or on several,
// whatever the batch size (tuning); unset: chosen by size.
int meta_multi_knob() {
  static const int v = [] {
    const char *e = std::getenv("LORA_META_MULTI");
    return e && *e ? (std::atoi(e) > 0 ? 1 : 0) : -1;
  }();
  return v;
}
// LORA_SPLIT_MEMBERS=n (1, 2, 4, 8 or 16): workgroups per tile of the split
// kernel, instead of the count chosen from the batch (tuning).
int split_members() {
  static const int v = [] {
    const int m = env_int("LORA_SPLIT_MEMBERS", 0);
    return (m == 1 || m == 2 || m == 4 || m == 8 || m == 16) ? m : 0;
  }();
  return v;
}

}  // namespace lora

using namespace lora;

namespace {

// Clears n words with vector stores (a fill kernel rather than hipMemsetAsync,
// so that a captured graph holds a kernel node).
__global__ void zero_words_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t stream) {
  const int grid = (int)std::min<int64_t>(256, (n + 255) / 256);
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// Kernels address one slot's factor matrix with 32-bit byte offsets.
constexpr int64_t kMaxFactorElems = (int64_t)1 << 28;

constexpr int32_t kAbiVersion = 10;

size_t align256(size_t b) { return (b + 255) / 256 * 256; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool rank_ok(int32_t r) { return tile_rank(r) != 0; }
bool dtype_ok(lora_dtype d) { return d == LORA_F32 || d == LORA_BF16; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool mode_ok(lora_mode m) { return m == LORA_MODE_AUTO || m == LORA_MODE_BGMV || m == LORA_MODE_SGMV; }
size_t esize(lora_dtype d) { return d == LORA_F32 ? 4 : 2; }

struct MetaLayout {
  size_t sorted, sorted_slot, seg_slot, seg_count, seg_start, info, tiles, total;
};
MetaLayout meta_layout(int64_t T, int32_t S) {
  MetaLayout L{};
  size_t off = 0;
  L.sorted = off;
  off += align256(sizeof(int32_t) * (size_t)std::max<int64_t>(T, 1));
  L.sorted_slot = off;
  off += align256(sizeof(int32_t) * (size_t)std::max<int64_t>(T, 1));
  L.seg_slot = off;
  off += align256(sizeof(int32_t) * (size_t)(S + 1));
  L.seg_count = off;
  off += align256(sizeof(int32_t) * (size_t)(S + 1));
  L.seg_start = off;
  off += align256(sizeof(int32_t) * (size_t)(S + 2));
  L.info = off;
  off += align256(sizeof(int32_t) * 8);
  L.tiles = off;
  off += meta_tiles_bytes(T, S);
  off += meta_counts_bytes(T, S);  // the several-workgroup path's counts
  L.total = off;
  return L;
}

lora_status check_meta(const lora_meta *m) {
  if (!m || m->num_tokens < 0 || m->num_slots < 1 || m->num_slots > kMaxSlots || m->x_row_div < 1)
    return LORA_ERR_INVALID_ARG;
  if (!m->sorted || !m->sorted_slot || !m->seg_slot || !m->seg_count || !m->seg_start || !m->info ||
      !m->tiles)
    return LORA_ERR_INVALID_ARG;
  return LORA_OK;
}

MetaView view_of(const lora_meta *m) {
  MetaView v;
  v.sorted = m->sorted;
  v.sorted_slot = m->sorted_slot;
  v.seg_slot = m->seg_slot;
  v.seg_count = m->seg_count;
  v.seg_start = m->seg_start;
  v.info = m->info;
  v.tiles = m->tiles;
  v.T = m->num_tokens;
  v.S = m->num_slots;
  v.x_row_div = m->x_row_div;
  return v;
}

lora_status check_shrink_args(const lora_meta *meta, const void *x, int64_t ldx, int64_t d_in,
                              lora_dtype dtype, int32_t n_slices, const lora_weight *A,
                              int32_t r_max, const float *slot_scale, const float *u,
                              lora_mode mode) {
  lora_status st = check_meta(meta);
  if (st != LORA_OK) return st;
  if (!dtype_ok(dtype) || !mode_ok(mode)) return LORA_ERR_UNSUPPORTED;
  if (n_slices < 1 || n_slices > kMaxSlices) return LORA_ERR_UNSUPPORTED;
  if (!rank_ok(r_max)) return LORA_ERR_UNSUPPORTED;
  if (d_in < 8 || d_in % 8 || ldx < d_in || ldx % 8) return LORA_ERR_INVALID_ARG;
  if ((int64_t)(r_max + 1) * d_in >= kMaxFactorElems) return LORA_ERR_UNSUPPORTED;  // 32-bit offsets
  // with no tokens nothing is read or written, so empty buffers may be null
  const bool empty = meta->num_tokens == 0;
  if (!A || (!empty && (!x || !u)) || !aligned16(x) || !aligned16(u)) return LORA_ERR_INVALID_ARG;
  if (slot_scale && (reinterpret_cast<uintptr_t>(slot_scale) & 3u)) return LORA_ERR_INVALID_ARG;
  for (int s = 0; s < n_slices; ++s) {
    if (!A[s].ptr || !aligned16(A[s].ptr) || A[s].slot_stride % 8 ||
        A[s].slot_stride < d_in * r_max || A[s].reserved != 0 || A[s].layout != A[0].layout)
      return LORA_ERR_INVALID_ARG;
  }
  if (A[0].layout != LORA_LAYOUT_DEFAULT && A[0].layout != LORA_LAYOUT_RANK_ROWS) return LORA_ERR_UNSUPPORTED;
  // rank-major A is read by the matrix-core shrink only
  if (A[0].layout == LORA_LAYOUT_RANK_ROWS && (dtype != LORA_BF16 || tile_rank(r_max) < 16 || mode == LORA_MODE_BGMV))
    return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

lora_status check_expand_args(const lora_meta *meta, const float *u, int32_t n_slices,
                              const lora_weight *B, const int64_t *width, const int64_t *offset,
                              int32_t r_max, const void *y, int64_t ldy, lora_dtype dtype,
                              lora_mode mode) {
  lora_status st = check_meta(meta);
  if (st != LORA_OK) return st;
  if (!dtype_ok(dtype) || !mode_ok(mode)) return LORA_ERR_UNSUPPORTED;
  if (n_slices < 1 || n_slices > kMaxSlices) return LORA_ERR_UNSUPPORTED;
  if (!rank_ok(r_max)) return LORA_ERR_UNSUPPORTED;
  const bool empty = meta->num_tokens == 0;
  if (!B || !width || !offset || (!empty && (!u || !y)) || !aligned16(u) || !aligned16(y))
    return LORA_ERR_INVALID_ARG;
  if (ldy < 8 || ldy % 8) return LORA_ERR_INVALID_ARG;
  for (int s = 0; s < n_slices; ++s) {
    const int64_t w = width[s], o = offset[s];
    if (w < 8 || w % 8 || o < 0 || o % 8 || o + w > ldy) return LORA_ERR_INVALID_ARG;
    if ((int64_t)(r_max + 1) * w >= kMaxFactorElems) return LORA_ERR_UNSUPPORTED;  // 32-bit offsets
    if (!B[s].ptr || !aligned16(B[s].ptr) || B[s].slot_stride % 8 || B[s].slot_stride < r_max * w ||
        B[s].reserved != 0 || B[s].layout != B[0].layout)
      return LORA_ERR_INVALID_ARG;
    for (int q = 0; q < s; ++q) {
      if (o < offset[q] + width[q] && offset[q] < o + w) return LORA_ERR_INVALID_ARG;
    }
  }
  if (B[0].layout != LORA_LAYOUT_DEFAULT && B[0].layout != LORA_LAYOUT_OUT_ROWS) return LORA_ERR_UNSUPPORTED;
  // B in the output-rows layout is read by the matrix-core expand only
  if (B[0].layout == LORA_LAYOUT_OUT_ROWS && (dtype != LORA_BF16 || tile_rank(r_max) > 64 || mode == LORA_MODE_BGMV))
    return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

void unpack(const lora_weight *W, int32_t n, const void **ptrs, int64_t *strides) {
  for (int s = 0; s < n; ++s) {
    ptrs[s] = W[s].ptr;
    strides[s] = W[s].slot_stride;
  }
}


// lora_apply on a workspace that holds the count words, then the rank-r
// buffer, then the partial sums (ws_bytes in all, already checked to be
// enough).
lora_status apply_in(const lora_meta *meta, const void *d_x, int64_t ldx, int64_t d_in, lora_dtype dtype,
                     int32_t n_slices, const lora_weight *A, const lora_weight *B, const int64_t *width,
                     const int64_t *offset, int32_t r_max, float scale, const float *d_slot_scale,
                     const int32_t *d_slot_rank, void *d_y, int64_t ldy, int add_into_y, lora_mode mode,
                     char *ws, size_t ws_bytes, hipStream_t s) {
  uint32_t *sync = reinterpret_cast<uint32_t *>(ws);
  float *u = reinterpret_cast<float *>(ws + kSyncBytes);
  lora_status st = check_shrink_args(meta, d_x, ldx, d_in, dtype, n_slices, A, r_max, d_slot_scale, u, mode);
  if (st != LORA_OK) return st;
  st = check_expand_args(meta, u, n_slices, B, width, offset, r_max, d_y, ldy, dtype, mode);
  if (st != LORA_OK) return st;
  if (!aligned4(d_slot_rank)) return LORA_ERR_INVALID_ARG;
  const int32_t R = tile_rank(r_max);  // the kernels' rank; A, B and the caller's u keep r_max
  const size_t ubytes = align256(sizeof(float) * (size_t)n_slices * (size_t)meta->num_tokens * (size_t)R);
  void *sh_ws = ws + kSyncBytes + ubytes;
  const size_t sh_bytes = ws_bytes - kSyncBytes - ubytes;
  const void *aptr[kMaxSlices], *bptr[kMaxSlices];
  int64_t astr[kMaxSlices], bstr[kMaxSlices];
  unpack(A, n_slices, aptr, astr);
  unpack(B, n_slices, bptr, bstr);
  const MetaView mv = view_of(meta);
  // decode-shaped (BGMV requested, or few tokens per slot): the split kernel
  // first (bf16; it checks its own limits), then the per-token kernel when
  // its limits hold; both take r_max of 8, 16, 32 or 64 only
  const bool decode = (int)mode != 2 && ((int)mode == 1 || meta->num_tokens <= 16 * (int64_t)meta->num_slots);
  const bool a_rows = A[0].layout == LORA_LAYOUT_RANK_ROWS;  // rank-major A: the tile shrink reads it
  const bool b_out = B[0].layout == LORA_LAYOUT_OUT_ROWS;    // output-rows B: the tile expand reads it
  const bool fused_rank = r_max == R && R <= 64 && !a_rows && !b_out;
  if (fused_rank && !fused_disabled() && decode && dtype == LORA_BF16 && !split_disabled()) {
    bool used = false;
    const hipError_t e = launch_bgmv_split(mv, d_x, ldx, d_in, n_slices, aptr, astr, bptr, bstr, width, offset,
                                           r_max, scale, d_slot_scale, d_slot_rank, d_y, ldy, add_into_y, sync,
                                           static_cast<float *>(sh_ws), sh_bytes, s, &used);
    if (e != hipSuccess) return LORA_ERR_HIP;
    if (used) return LORA_OK;
  }
  if (fused_rank && !fused_disabled() &&
      bgmv_fits(meta->num_tokens, meta->num_slots, d_in, n_slices, width, r_max, ldy, dtype == LORA_BF16,
                (int)mode)) {
    const hipError_t e = launch_bgmv(mv, d_x, ldx, d_in, dtype == LORA_BF16, n_slices, aptr, astr,
                                     bptr, bstr, width, offset, r_max, scale, d_slot_scale,
                                     d_slot_rank, d_y, ldy, add_into_y, s);
    return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  int kch = 1;
  const bool rows = !b_out && expand_rows_fits(meta->num_tokens, meta->num_slots, dtype == LORA_BF16, (int)mode, R) &&
                    expand_rows_addressable(meta->num_tokens, n_slices, width, offset, ldy, R);
  hipError_t e = launch_shrink(mv, d_x, ldx, d_in, dtype == LORA_BF16, n_slices, aptr, astr, R, r_max,
                               scale, d_slot_scale, d_slot_rank, u, (int)mode, sh_ws, true, &kch, s, rows, a_rows);
  if (e != hipSuccess) return LORA_ERR_HIP;
  if (rows) {  // long segments: the sums become bf16 planes in the rank buffer, then the row-stream expand
    e = launch_expand_rows(mv, static_cast<const float *>(sh_ws), kch, reinterpret_cast<uint16_t *>(u), n_slices,
                           bptr, bstr, width, offset, R, r_max, d_slot_rank, d_y, ldy, add_into_y, s);
    return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  // the rank-r rows are in sorted order; with a split d_in they are still the
  // partial sums, which the expand adds
  const float *ue = kch > 1 ? static_cast<const float *>(sh_ws) : u;
  e = launch_expand(mv, ue, kch > 1 ? 2 : 1, kch, n_slices, bptr, bstr, width, offset, R, r_max,
                    d_slot_rank, d_y, ldy, dtype == LORA_BF16, add_into_y, (int)mode, s, b_out);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

std::mutex g_scratch_mu;
char *g_scratch_dev[kMaxDevices];

// This device's copy of the scratch array, looked up once per device.
hipError_t scratch_of_current_device(char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = static_cast<char *>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t lora_abi_version(void) { return kAbiVersion; }

const char *lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "LORA_OK";
    case LORA_ERR_INVALID_ARG: return "LORA_ERR_INVALID_ARG";
    case LORA_ERR_UNSUPPORTED: return "LORA_ERR_UNSUPPORTED";
    case LORA_ERR_WORKSPACE: return "LORA_ERR_WORKSPACE";
    case LORA_ERR_HIP: return "LORA_ERR_HIP";
    default: break;
  }
  return "LORA_ERR_UNKNOWN";
}

lora_status lora_meta_workspace_bytes(int64_t T, int32_t S, size_t *bytes) {
  if (!bytes || T < 0 || T > INT32_MAX || S < 1) return LORA_ERR_INVALID_ARG;
  if (S > kMaxSlots) return LORA_ERR_UNSUPPORTED;
  *bytes = meta_layout(T, S).total;
  return LORA_OK;
}

// Points the metadata struct at its arrays inside the workspace.
static void place_meta(lora_meta *out, void *d_ws, const MetaLayout &L, int64_t T, int32_t S) {
  char *base = static_cast<char *>(d_ws);
  out->num_tokens = T;
  out->num_slots = S;
  out->x_row_div = 1;
  out->sorted = reinterpret_cast<int32_t *>(base + L.sorted);
  out->sorted_slot = reinterpret_cast<int32_t *>(base + L.sorted_slot);
  out->seg_slot = reinterpret_cast<int32_t *>(base + L.seg_slot);
  out->seg_count = reinterpret_cast<int32_t *>(base + L.seg_count);
  out->seg_start = reinterpret_cast<int32_t *>(base + L.seg_start);
  out->info = reinterpret_cast<int32_t *>(base + L.info);
  out->tiles = reinterpret_cast<int32_t *>(base + L.tiles);
}

lora_status lora_prepare_meta(const int32_t *d_token_slot, int64_t T, int32_t S, void *d_ws,
                              size_t ws_bytes, lora_meta *out, void *stream) {
  if (!out || T < 0 || T > INT32_MAX || S < 1 || !d_ws || !aligned16(d_ws))
    return LORA_ERR_INVALID_ARG;
  if (S > kMaxSlots) return LORA_ERR_UNSUPPORTED;
  if (T > 0 && !d_token_slot) return LORA_ERR_INVALID_ARG;
  const MetaLayout L = meta_layout(T, S);
  if (ws_bytes < L.total) return LORA_ERR_WORKSPACE;
  place_meta(out, d_ws, L, T, S);
  const hipError_t e = launch_meta(d_token_slot, T, S, out->sorted, out->sorted_slot, out->seg_slot,
                                   out->seg_count, out->seg_start, out->info, out->tiles,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_moe_meta_workspace_bytes(int64_t T, int32_t topk, int32_t S, int32_t E_local,
                                          size_t *bytes) {
  if (!bytes || T < 0 || topk < 1 || S < 1 || E_local < 1) return LORA_ERR_INVALID_ARG;
  if (T * topk > INT32_MAX) return LORA_ERR_INVALID_ARG;
  if ((int64_t)S * E_local > kMaxSlots) return LORA_ERR_UNSUPPORTED;
  *bytes = meta_layout(T * topk, S * E_local).total;
  return LORA_OK;
}

lora_status lora_prepare_moe_meta(const int32_t *d_topk_ids, int64_t T, int32_t topk,
                                  const int32_t *d_token_slot, int32_t S, int32_t E_global,
                                  int32_t E_local, const int32_t *d_expert_map, void *d_ws,
                                  size_t ws_bytes, lora_meta *out, void *stream) {
  if (!out || T < 0 || topk < 1 || S < 1 || E_global < 1 || E_local < 1 || !d_ws || !aligned16(d_ws))
    return LORA_ERR_INVALID_ARG;
  if (T * topk > INT32_MAX) return LORA_ERR_INVALID_ARG;
  if ((int64_t)S * E_local > kMaxSlots) return LORA_ERR_UNSUPPORTED;
  if (T > 0 && (!d_topk_ids || !d_token_slot)) return LORA_ERR_INVALID_ARG;
  if (!aligned4(d_topk_ids) || !aligned4(d_token_slot) || !aligned4(d_expert_map)) return LORA_ERR_INVALID_ARG;
  size_t need = 0;
  const lora_status st = lora_moe_meta_workspace_bytes(T, topk, S, E_local, &need);
  if (st != LORA_OK) return st;
  if (ws_bytes < need) return LORA_ERR_WORKSPACE;
  const int64_t n = T * topk;
  place_meta(out, d_ws, meta_layout(n, S * E_local), n, S * E_local);
  const hipError_t e = launch_meta_moe(d_topk_ids, T, topk, d_token_slot, S, E_global, E_local, d_expert_map,
                                       out->sorted, out->sorted_slot, out->seg_slot, out->seg_count,
                                       out->seg_start, out->info, out->tiles, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return LORA_ERR_HIP;
  out->x_row_div = topk;
  return LORA_OK;
}

lora_status lora_shrink_workspace_bytes(int64_t T, int32_t S, int64_t d_in, int32_t n_slices,
                                        int32_t r_max, lora_dtype dtype, lora_mode mode,
                                        size_t *bytes) {
  if (!bytes || T < 0 || T > INT32_MAX || S < 1 || d_in < 8 || d_in % 8)
    return LORA_ERR_INVALID_ARG;
  if (S > kMaxSlots || n_slices < 1 || n_slices > kMaxSlices || !rank_ok(r_max) ||
      !dtype_ok(dtype) || !mode_ok(mode))
    return LORA_ERR_UNSUPPORTED;
  const int32_t R = tile_rank(r_max);
  const ShrinkConfig c = plan_shrink(T, S, d_in, R, dtype == LORA_BF16, (int)mode);
  *bytes = shrink_ws_bytes(c, T, n_slices, R);
  return LORA_OK;
}

lora_status lora_shrink(const lora_meta *meta, const void *d_x, int64_t ldx, int64_t d_in,
                        lora_dtype dtype, int32_t n_slices, const lora_weight *A, int32_t r_max,
                        float scale, const float *d_slot_scale, const int32_t *d_slot_rank,
                        float *d_u, lora_mode mode, void *d_ws, size_t ws_bytes, void *stream) {
  lora_status st = check_shrink_args(meta, d_x, ldx, d_in, dtype, n_slices, A, r_max,
                                     d_slot_scale, d_u, mode);
  if (st != LORA_OK) return st;
  if (!aligned4(d_slot_rank)) return LORA_ERR_INVALID_ARG;
  size_t need = 0;
  st = lora_shrink_workspace_bytes(meta->num_tokens, meta->num_slots, d_in, n_slices, r_max,
                                   dtype, mode, &need);
  if (st != LORA_OK) return st;
  if (ws_bytes < need || (need && (!d_ws || !aligned16(d_ws)))) return LORA_ERR_WORKSPACE;
  const void *ptrs[kMaxSlices];
  int64_t strides[kMaxSlices];
  unpack(A, n_slices, ptrs, strides);
  const hipError_t e =
      launch_shrink(view_of(meta), d_x, ldx, d_in, dtype == LORA_BF16, n_slices, ptrs, strides,
                    tile_rank(r_max), r_max, scale, d_slot_scale, d_slot_rank, d_u, (int)mode, d_ws, false, nullptr,
                    static_cast<hipStream_t>(stream), false, A[0].layout == LORA_LAYOUT_RANK_ROWS);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_expand(const lora_meta *meta, const float *d_u, int32_t n_slices,
                        const lora_weight *B, const int64_t *width, const int64_t *offset,
                        int32_t r_max, const int32_t *d_slot_rank, void *d_y, int64_t ldy,
                        lora_dtype dtype, int add_into_y, lora_mode mode, void *stream) {
  const lora_status st =
      check_expand_args(meta, d_u, n_slices, B, width, offset, r_max, d_y, ldy, dtype, mode);
  if (st != LORA_OK) return st;
  if (!aligned4(d_slot_rank)) return LORA_ERR_INVALID_ARG;
  const void *ptrs[kMaxSlices];
  int64_t strides[kMaxSlices];
  unpack(B, n_slices, ptrs, strides);
  const hipError_t e = launch_expand(view_of(meta), d_u, 0, 1, n_slices, ptrs, strides, width,
                                     offset, tile_rank(r_max), r_max, d_slot_rank, d_y, ldy, dtype == LORA_BF16,
                                     add_into_y, (int)mode, static_cast<hipStream_t>(stream),
                                     B[0].layout == LORA_LAYOUT_OUT_ROWS);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_apply_workspace_bytes(int64_t T, int32_t S, int64_t d_in, int32_t n_slices,
                                       int32_t r_max, lora_dtype dtype, lora_mode mode,
                                       size_t *bytes) {
  size_t sh = 0;
  const lora_status st = lora_shrink_workspace_bytes(T, S, d_in, n_slices, r_max, dtype, mode, &sh);
  if (st != LORA_OK) return st;
  const int32_t R = tile_rank(r_max);  // the kernels' rank
  // the split decode kernel's partial rank rows share the shrink's region
  if (dtype == LORA_BF16 && mode != LORA_MODE_SGMV && r_max == R && R <= 64)
    sh = std::max(sh, split_ws_bytes(T, S, n_slices, R));
  // the long-segment expand takes the shrink's sums from that region even
  // without a split of d_in
  if (expand_rows_fits(T, S, dtype == LORA_BF16, (int)mode, R))
    sh = std::max(sh, align256(sizeof(float) * (size_t)n_slices * (size_t)T * (size_t)R));
  // count words, then the rank-R buffer, then the shrink's or the split
  // kernel's partial sums
  *bytes = kSyncBytes + align256(sizeof(float) * (size_t)n_slices * (size_t)T * (size_t)R) + sh;
  return LORA_OK;
}

lora_status lora_apply_workspace_init(void *d_ws, size_t ws_bytes, void *stream) {
  if (!d_ws || !aligned16(d_ws)) return LORA_ERR_INVALID_ARG;
  if (ws_bytes < kSyncBytes) return LORA_ERR_WORKSPACE;
  const hipError_t e = launch_zero_words(static_cast<uint32_t *>(d_ws), kSyncBytes / sizeof(uint32_t),
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_apply(const lora_meta *meta, const void *d_x, int64_t ldx, int64_t d_in,
                       lora_dtype dtype, int32_t n_slices, const lora_weight *A,
                       const lora_weight *B, const int64_t *width, const int64_t *offset,
                       int32_t r_max, float scale, const float *d_slot_scale,
                       const int32_t *d_slot_rank, void *d_y, int64_t ldy, int add_into_y,
                       lora_mode mode, void *d_ws, size_t ws_bytes, void *stream) {
  if (!meta) return LORA_ERR_INVALID_ARG;
  size_t need = 0;
  lora_status st = lora_apply_workspace_bytes(meta->num_tokens, meta->num_slots, d_in, n_slices,
                                              r_max, dtype, mode, &need);
  if (st != LORA_OK) return st;
  if (ws_bytes < need || !d_ws || !aligned16(d_ws)) return LORA_ERR_WORKSPACE;
  return apply_in(meta, d_x, ldx, d_in, dtype, n_slices, A, B, width, offset, r_max, scale, d_slot_scale,
                  d_slot_rank, d_y, ldy, add_into_y, mode, static_cast<char *>(d_ws), ws_bytes,
                  static_cast<hipStream_t>(stream));
}

lora_status lora_apply_noalloc(const lora_meta *meta, const void *d_x, int64_t ldx, int64_t d_in,
                               lora_dtype dtype, int32_t n_slices, const lora_weight *A,
                               const lora_weight *B, const int64_t *width, const int64_t *offset,
                               int32_t r_max, float scale, const float *d_slot_scale,
                               const int32_t *d_slot_rank, void *d_y, int64_t ldy, int add_into_y,
                               lora_mode mode, void *stream) {
  if (!meta) return LORA_ERR_INVALID_ARG;
  size_t need = 0;
  const lora_status st = lora_apply_workspace_bytes(meta->num_tokens, meta->num_slots, d_in, n_slices, r_max,
                                                    dtype, mode, &need);
  if (st != LORA_OK) return st;
  if (need > kScratchBytes) return LORA_ERR_WORKSPACE;
  char *ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) {
    (void)hipGetLastError();  // the failed lookup must not be reported by the next launch
    return LORA_ERR_HIP;
  }
  return apply_in(meta, d_x, ldx, d_in, dtype, n_slices, A, B, width, offset, r_max, scale, d_slot_scale,
                  d_slot_rank, d_y, ldy, add_into_y, mode, ws, kScratchBytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
