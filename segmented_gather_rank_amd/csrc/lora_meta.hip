// lora_meta.hip -- slot metadata of a batch on one workgroup of 16 waves.
//
// Page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "LoRAKernelMeta:先按槽位
// 排序": tokens are stably sorted by slot id (no-adapter id -1 first), the
// distinct ids are listed in ascending order with their token counts, and the
// start offsets are the running sum of the counts with a leading 0.
//
// Design (gfx950, wave64): keys are slot+1 in [0, S].
//   1. histogram of keys with LDS integer atomics (order-free, exact);
//   2. one wave scans the key counts (ballot + popcount for the segment index,
//      a wave prefix sum for the offsets) and writes the segment arrays;
//   3. a stable scatter over chunks of 1024 tokens in batch order: inside a
//      wave, lanes holding the same key find each other with one ballot per
//      key bit (a wave-wide match), and a lane's rank among equal keys is the
//      popcount of the matching lanes below it; the per-(wave, key) counts are
//      prefix-summed across the 16 waves in wave order (one 16-lane DPP row
//      scan per key), so equal keys keep batch order across waves and across
//      chunks;
//   4. while scattering, every token also lands in its work tile (its
//      segment's sorted range cut into runs of 64), and the token that opens a
//      tile writes the tile's header.
#include <algorithm>

#include "lora_host.h"

namespace lora {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / kWave;

// Inclusive prefix sum inside each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row contribute 0).
__device__ __forceinline__ int row16_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

__global__ __launch_bounds__(kMetaThreads) void meta_kernel(
    const int32_t *__restrict__ token_slot, int64_t T, int32_t S,
    int32_t *__restrict__ sorted, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ seg_slot,
    int32_t *__restrict__ seg_count, int32_t *__restrict__ seg_start,
    int32_t *__restrict__ info, int32_t *__restrict__ tiles) {
  extern __shared__ int32_t lds[];
  const int K = S + 1;                      // number of keys
  int32_t *cnt = lds;                       // [K] tokens per key
  int32_t *next = lds + K;                  // [K] next free position per key
  int32_t *kstart = lds + 2 * K;            // [K] first sorted position per key
  int32_t *tbase = lds + 3 * K;             // [K] first work tile per key
  int32_t *wcnt = lds + 4 * K;              // [16][K] per-wave counts, then offsets
  __shared__ int32_t nbad;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;

  for (int i = tid; i < K; i += kMetaThreads) cnt[i] = 0;
  for (int i = tid; i < kMetaWaves * K; i += kMetaThreads) wcnt[i] = 0;
  if (tid == 0) nbad = 0;
  __syncthreads();

  // 1. histogram (the first 1024 slot ids stay in registers for the scatter)
  int mybad = 0;
  int first_v = -1;
  for (int64_t t = tid; t < T; t += kMetaThreads) {
    const int v = token_slot[t];
    if (t < kMetaThreads) first_v = v;
    const bool ok = v >= -1 && v < S;
    mybad += ok ? 0 : 1;
    atomicAdd(&cnt[ok ? v + 1 : 0], 1);
  }
  if (mybad) atomicAdd(&nbad, mybad);
  __syncthreads();

  // 2. segments: one wave walks the keys in ascending order
  if (wave == 0) {
    int seg_base = 0, pos_base = 0, tile_base = 0;
    for (int k0 = 0; k0 < K; k0 += kWave) {
      const int k = k0 + lane;
      const int c = k < K ? cnt[k] : 0;
      const uint64_t present = __ballot(c > 0);
      const int seg = seg_base + __popcll(present & lanemask_lt());
      const int incl = wave_inclusive_scan(c);
      const int start = pos_base + incl - c;
      const int nt = (c + kTileRows - 1) / kTileRows;
      const int tincl = wave_inclusive_scan(nt);
      if (k < K) {
        next[k] = start;
        kstart[k] = start;
        tbase[k] = tile_base + tincl - nt;
      }
      if (c > 0) {
        seg_slot[seg] = k - 1;
        seg_count[seg] = c;
        seg_start[seg] = start;
      }
      seg_base += __popcll(present);
      pos_base += __shfl(incl, kWave - 1, kWave);
      tile_base += __shfl(tincl, kWave - 1, kWave);
    }
    // padding past the last segment, and the closing offset
    for (int i = seg_base + lane; i < K; i += kWave) {
      seg_slot[i] = -1;
      seg_count[i] = 0;
    }
    for (int i = seg_base + lane; i < K + 1; i += kWave) seg_start[i] = (int32_t)T;
    if (lane == 0) {
      info[0] = seg_base;
      info[1] = (T - cnt[0] == 0) ? 1 : 0;
      info[2] = nbad;
      info[3] = cnt[0];
      info[4] = tile_base;
      info[5] = info[6] = info[7] = 0;
    }
  }
  __syncthreads();

  // 3. stable scatter, 1024 tokens per pass in batch order
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  for (int64_t base = 0; base < T; base += kMetaThreads) {
    const int64_t t = base + tid;
    const bool valid = t < T;
    int key = 0;
    if (valid) {
      const int v = base == 0 ? first_v : token_slot[t];
      key = (v >= -1 && v < S) ? v + 1 : 0;
    }
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((key >> b) & 1));
      same &= ((key >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(same & lanemask_lt());
    const bool leader = valid && rank == 0;
    if (leader) wcnt[wave * K + key] = __popcll(same);
    __syncthreads();
    // per key, prefix of the 16 waves' counts in wave order: the 16 counts of
    // one key sit in one 16-lane row (thread = 16 key + wave) and are scanned
    // with DPP row shifts; the row's last lane advances the key's next position
    for (int k0 = 0; k0 < K; k0 += kMetaThreads / kMetaWaves) {
      const int k = k0 + tid / kMetaWaves, w = tid % kMetaWaves;
      const int c = k < K ? wcnt[w * K + k] : 0;
      const int incl = row16_inclusive_scan(c);
      const int at = k < K ? next[k] : 0;
      if (k < K) wcnt[w * K + k] = at + incl - c;
      if (k < K && w == kMetaWaves - 1) next[k] = at + incl;
    }
    __syncthreads();
    if (valid) {
      const int dst = wcnt[wave * K + key] + rank;
      sorted[dst] = (int32_t)t;
      sorted_slot[dst] = key - 1;
      const int off = dst - kstart[key];
      int32_t *tl = tiles + (int64_t)(tbase[key] + off / kTileRows) * kTileInts;
      tl[4 + off % kTileRows] = (int32_t)t;
      if (off % kTileRows == 0) {
        tl[0] = key - 1;
        tl[1] = min(kTileRows, cnt[key] - off);
        tl[2] = dst;
        tl[3] = 0;
      }
    }
    if (base + kMetaThreads < T) {  // the count table starts the next pass at zero
      __syncthreads();
      for (int k = tid; k < kMetaWaves * K; k += kMetaThreads) wcnt[k] = 0;
      __syncthreads();
    }
  }
}

// Key of pair p = t * topk + j: slot * E_local + local expert, -1 for no
// adapter or a remote expert, -2 (counted as bad by the metadata kernel) for
// ids out of range.
__global__ __launch_bounds__(256) void moe_keys_kernel(const int32_t *__restrict__ topk_ids, int64_t n,
                                                       int32_t topk, const int32_t *__restrict__ token_slot,
                                                       int32_t S, int32_t E_global, int32_t E_local,
                                                       const int32_t *__restrict__ expert_map,
                                                       int32_t *__restrict__ keys) {
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < n; p += (int64_t)gridDim.x * 256) {
    const int slot = token_slot[p / topk];
    const int e = topk_ids[p];
    int key;
    if (slot < -1 || slot >= S || e < 0 || e >= E_global) {
      key = -2;
    } else {
      const int le = expert_map ? expert_map[e] : (e < E_local ? e : -2);
      if (le < -1 || le >= E_local) key = -2;
      else key = (slot < 0 || le < 0) ? -1 : slot * E_local + le;
    }
    keys[p] = key;
  }
}

hipError_t launch_moe_keys(const int32_t *topk_ids, int64_t T, int32_t topk, const int32_t *token_slot,
                           int32_t S, int32_t E_global, int32_t E_local, const int32_t *expert_map,
                           int32_t *keys, hipStream_t stream) {
  const int64_t n = T * topk;
  if (n == 0) return hipSuccess;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(moe_keys_kernel, dim3(grid), dim3(256), 0, stream, topk_ids, n, topk, token_slot, S,
                     E_global, E_local, expert_map, keys);
  return hipGetLastError();
}

size_t meta_lds_bytes(int32_t S) { return sizeof(int32_t) * (size_t)(S + 1) * (4 + kMetaWaves); }

hipError_t launch_meta(const int32_t *token_slot, int64_t T, int32_t S, int32_t *sorted,
                       int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count, int32_t *seg_start,
                       int32_t *info, int32_t *tiles, hipStream_t stream) {
  const size_t lds = meta_lds_bytes(S);
  if (lds > 65536) {
    // large slot counts need more than the default 64 KB of dynamic LDS
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&meta_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(kMetaThreads), lds, stream,
                     token_slot, T, S, sorted, sorted_slot, seg_slot, seg_count, seg_start, info, tiles);
  return hipGetLastError();
}

}  // namespace lora
