// lora_meta.hip -- slot metadata of a batch on one workgroup of 16 waves.
//
// Page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "LoRAKernelMeta:先按槽位
// 排序": tokens are stably sorted by slot id (no-adapter id -1 first), the
// distinct ids are listed in ascending order with their token counts, and the
// start offsets are the running sum of the counts with a leading 0.
//
// Design (gfx950, wave64): keys are slot+1 in [0, S], K = S + 1 <= 1024.
//   1. the keys of up to 1024 rows stay in registers (thread t holds row t);
//      more rows are loaded in batches of 8 per thread, every load of a batch
//      issued before any is used, and kept in LDS when they fit;
//   2. every wave counts the keys of its own contiguous run of rows, 64 at a
//      time: lanes holding the same key find each other through a per-wave
//      table of lane masks in LDS (each lane ORs its bit into its key's entry
//      and reads it back), or with one ballot per key bit when the tables do
//      not fit; a step of one key (a long segment) needs neither, and skips
//      the table, whose word 64 lanes would update one after another (a
//      batch of four 1024-token segments: 4.8 us of counting, 2.1 without);
//      a lane's rank among equal keys is the popcount of the matching lanes
//      below it, and one lane per key adds their number;
//   3. per key, the 16 waves' counts are prefix-summed in wave order (one
//      16-lane DPP row scan per key): each wave's first position per key;
//   4. one thread per key prefix-sums counts, tile counts and presence over
//      the keys (wave scans with DPP row shifts and row broadcasts): start
//      offsets, first work tiles, segment indices;
//   5. the segment arrays are written (no barrier follows global stores);
//   6. a stable scatter: every wave walks its run again, a row going to its
//      key's start + earlier waves' and earlier steps' counts + its rank, and
//      into its work tile (the key's sorted range cut into runs of 64); the
//      row that opens a tile writes the tile's header.  Equal keys keep batch
//      order: within a step by lane, across steps and waves by run order.
//      When they fit, there are at least kMetaStageMin rows and at least half
//      of them sit in steps of several keys, the sorted arrays and the tile
//      list are scattered into LDS and then stored as whole 16-byte pieces:
//      one CU writes scattered 4-byte values at about one cache line per
//      cycle (4096 rows over 128 keys: a 4.0 us scatter, 2.8 us through LDS),
//      while rows in long runs already land in whole lines (there the copy
//      out of LDS only adds time).
// MoE pairs (page "vLLM 源码完全拆解(十八)", section "融合计算:add_lora_w13 与
// add_lora_w2": tokens regrouped by adapter and expert; section "EP
// 下只装载本地专家的权重": a rank holds its local experts): row p = t * topk + j
// is keyed here by slot(t) * E_local + local(topk_ids[p]), with the expert map
// staged in LDS, so the pairs need no pass of their own.
#include <algorithm>

#include "lora_host.h"

namespace lora {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / kWave;
constexpr int kMetaBatch = 8;                           // keys per thread per batch of loads
constexpr int kMetaBatchRows = kMetaBatch * kMetaThreads;
constexpr int kMetaMapLds = 4096;                       // expert maps up to this size go to LDS
constexpr size_t kMetaLdsMax = 159 * 1024;              // dynamic LDS of the workgroup, at most
constexpr int64_t kMetaMultiMin = 8192;                 // rows from which several workgroups build the metadata
constexpr int64_t kMetaStageMin = 3072;                 // rows from which the scatter may go through LDS

// Where the keys come from: a slot id per row, or (MoE) the pair's slot and
// expert, with key = slot * E_local + local expert (-1: no adapter or a remote
// expert, -2: an id out of range, counted as bad).
struct MetaSrc {
  const int32_t *token_slot;  // per row (plain), or per token (MoE)
  const int32_t *topk_ids;    // MoE: [T / topk][topk]
  const int32_t *expert_map;  // MoE: [E_global] or null
  int32_t topk, S_adapters, E_global, E_local;
};

// Inclusive prefix sum inside each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row contribute 0).
__device__ __forceinline__ int row16_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

template <bool MOE>
__device__ __forceinline__ int moe_key(const MetaSrc &src, const int32_t *emap, int e, int slot) {
  if (slot < -1 || slot >= src.S_adapters || e < 0 || e >= src.E_global) return -2;
  const int le = !src.expert_map ? (e < src.E_local ? e : -2) : (emap ? emap[e] : src.expert_map[e]);
  if (le < -1 || le >= src.E_local) return -2;
  return (slot < 0 || le < 0) ? -1 : slot * src.E_local + le;
}

// Lanes of a wave holding the same key (valid lanes only): one ballot per key
// bit.
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 10; ++b) {  // keys < 1024
    if (b < nbits) {
      const uint64_t ones = __ballot(valid && ((key >> b) & 1));
      same &= ((key >> b) & 1) ? ones : ~ones;
    }
  }
  return valid ? same : 0;
}

// Steps 4 and 5 of the metadata, for all 1024 threads of a workgroup (it holds
// barriers): over the keys in ascending order (thread k, K <= 1024), start
// offsets, first tiles and segment indices are prefix sums of the counts
// cnt[k] (LDS), tile counts and presence; kstart and tbase (LDS) get the first
// two.  Then, with `store`, the segment arrays, their padding past the last
// segment, the closing offset and the counters are stored (no barrier follows
// these stores: a barrier after global stores would wait for them).
__device__ __forceinline__ void key_tables(int K, int64_t T, const int32_t *cnt, int32_t *kstart, int32_t *tbase,
                                           int32_t (*wsum)[3], int nbad, int32_t *seg_slot, int32_t *seg_count,
                                           int32_t *seg_start, int32_t *info, bool store = true) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int k = tid;
  int c = 0, start = 0, nseg = 0, ntiles = 0, seg = 0;
  if (K <= kWave) {  // every key in wave 0: no exchange between waves
    if (wave == 0) {
      c = k < K ? cnt[k] : 0;
      const int nt = (c + kTileRows - 1) / kTileRows, pr = c > 0 ? 1 : 0;
      const int ic = wave_inclusive_scan(c), it = wave_inclusive_scan(nt), ip = wave_inclusive_scan(pr);
      nseg = __builtin_amdgcn_readlane(ip, kWave - 1);
      ntiles = __builtin_amdgcn_readlane(it, kWave - 1);
      start = ic - c;
      seg = ip - pr;
      if (k < K) {
        kstart[k] = start;
        tbase[k] = it - nt;
      }
    }
  } else {
    c = k < K ? cnt[k] : 0;
    const int nt = (c + kTileRows - 1) / kTileRows, pr = c > 0 ? 1 : 0;
    const int ic = wave_inclusive_scan(c), it = wave_inclusive_scan(nt), ip = wave_inclusive_scan(pr);
    if (lane == kWave - 1) {
      wsum[wave][0] = ic;
      wsum[wave][1] = it;
      wsum[wave][2] = ip;
    }
    __syncthreads();
    // only the waves that hold keys need the others' sums, and only theirs
    const int nkw = (K + kWave - 1) / kWave;
    if (wave < nkw) {
      int bc = 0, bt = 0, bp = 0;
      for (int w = 0; w < nkw; ++w) {
        const int a = wsum[w][0], b2 = wsum[w][1], d = wsum[w][2];
        if (w < wave) {
          bc += a;
          bt += b2;
          bp += d;
        }
        nseg += d;
        ntiles += b2;
      }
      start = bc + ic - c;
      seg = bp + ip - pr;
      if (k < K) {
        kstart[k] = start;
        tbase[k] = bt + it - nt;
      }
    }
  }
  __syncthreads();
  if (!store) return;

  if (c > 0) {
    seg_slot[seg] = k - 1;
    seg_count[seg] = c;
    seg_start[seg] = start;
  }
  if (k >= nseg && k < K) {
    seg_slot[k] = -1;
    seg_count[k] = 0;
    seg_start[k] = (int32_t)T;
  }
  if (tid == 0) {
    seg_start[K] = (int32_t)T;
    info[0] = nseg;
    info[1] = (T - c == 0) ? 1 : 0;  // thread 0 holds key 0: the rows without an adapter
    info[2] = nbad;
    info[3] = c;
    info[4] = ntiles;
    info[5] = info[6] = info[7] = 0;
  }
}

// KIND 0 (kSmall): at most 1024 rows; thread tid holds row tid in registers
// throughout (each wave's run below is then its own 64 rows).  KIND 1
// (kCached): the keys of all rows are kept in LDS.  KIND 2 (kStreamed): rows
// are read from memory again in each pass.  MLDS: the per-wave lane-mask
// tables fit in LDS (else keys are matched with ballots).  STAGE: LDS holds
// room for the sorted arrays and the tile list, which scattered batches are
// built in and stored whole from (kCached only).  Each instantiation carries only its own code: code that
// runs once is fetched cold, so its size is time.
constexpr int kSmall = 0, kCached = 1, kStreamed = 2;

template <bool MOE, int KIND, bool MLDS, bool STAGE>
__global__ __launch_bounds__(kMetaThreads) void meta_kernel(
    const int32_t *__restrict__ token_slot, const int32_t *__restrict__ topk_ids, int64_t T, MetaSrc src,
    int32_t S,
    int32_t *__restrict__ sorted, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ seg_slot,
    int32_t *__restrict__ seg_count, int32_t *__restrict__ seg_start,
    int32_t *__restrict__ info, int32_t *__restrict__ tiles) {
  extern __shared__ __align__(16) int32_t lds[];  // 16-byte aligned: the lane-mask tables take 8-byte LDS atomics
  const int K = S + 1;                      // number of keys (slot + 1; 0: none or bad)
  int32_t *cnt = lds;                       // [K] rows per key
  int32_t *kstart = lds + K;                // [K] first sorted position per key
  int32_t *tbase = lds + 2 * K;             // [K] first work tile per key
  int32_t *woff = lds + 3 * K;              // [16][K] per-wave counts, then offsets
  // [T] the keys, when they fit in LDS (an LDS-typed pointer, so that its
  // reads are LDS reads even next to the global path)
  typedef __attribute__((address_space(3))) int32_t lds_i32;
  lds_i32 *vcache = (lds_i32 *)(woff + kMetaWaves * K);
  const bool map_lds = MOE && src.expert_map && src.E_global <= kMetaMapLds;
  int32_t *emap = map_lds ? woff + kMetaWaves * K + (KIND == kCached ? T : 0) : nullptr;  // [E_global]
  // [16][K] per-wave lane masks of one group of rows, per key (8-byte aligned)
  const int64_t masks_at = ((3 + kMetaWaves) * K + (KIND == kCached ? T : 0) + (map_lds ? src.E_global : 0) + 1) / 2 * 2;
  uint64_t *masks = reinterpret_cast<uint64_t *>(lds + masks_at);
  // STAGE: [T] sorted rows, [T] their slots, then the tile list (16-byte
  // aligned pieces, after the match tables)
  const int64_t t4 = (T + 3) / 4 * 4;
  lds_i32 *st_sorted = (lds_i32 *)(lds + (masks_at + (MLDS ? 2 * kMetaWaves * K : 0) + 3) / 4 * 4);
  lds_i32 *st_slot = st_sorted + t4;
  lds_i32 *st_tiles = st_slot + t4;
  __shared__ int32_t nbad, nmixed;  // rows with an id out of range; steps holding several keys
  __shared__ int32_t wsum[kMetaWaves][3];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;

  // raw inputs of one batch of rows, all loads issued before any is used
  int raw[kMetaBatch], rsl[kMetaBatch];
  auto load_raw = [&](int64_t b0) {
    // MoE: the token of row t is t / topk, stepped along the batch's rows
    // (rows < 2^31) instead of divided for each
    uint32_t q = 0, r = 0, dq = 0, dr = 0;
    if constexpr (MOE) {
      const uint32_t t0 = (uint32_t)(b0 + tid), k = (uint32_t)src.topk;
      q = t0 / k;
      r = t0 - q * k;
      dq = (uint32_t)kMetaThreads / k;
      dr = (uint32_t)kMetaThreads - dq * k;
    }
#pragma unroll
    for (int i = 0; i < (KIND == kSmall ? 1 : kMetaBatch); ++i) {
      const int64_t t = b0 + tid + (int64_t)kMetaThreads * i;
      if (t < T) {
        if constexpr (MOE) {
          raw[i] = topk_ids[t];
          rsl[i] = token_slot[q];
        } else {
          raw[i] = token_slot[t];
        }
      }
      if constexpr (MOE) {
        q += dq;
        r += dr;
        if (r >= (uint32_t)src.topk) {
          r -= (uint32_t)src.topk;
          ++q;
        }
      }
    }
  };
  // the key of row t in [-2, S): from LDS when cached, else from memory
  auto value_at = [&](int64_t t) -> int {
    if constexpr (KIND == kCached) return vcache[(int)t];
    if constexpr (MOE) return moe_key<MOE>(src, emap, topk_ids[t], token_slot[(uint32_t)t / (uint32_t)src.topk]);
    return token_slot[t];
  };

  // 1. keys into LDS, in batches of up to 8 rows per thread (a batch's loads
  //    are all issued before any is used)
  if (KIND == kSmall) load_raw(0);
  for (int i = tid; i < kMetaWaves * K; i += kMetaThreads) woff[i] = 0;
  if (MLDS)
    for (int i = tid; i < kMetaWaves * K; i += kMetaThreads) masks[i] = 0;
  if (map_lds)
    for (int i = tid; i < src.E_global; i += kMetaThreads) emap[i] = src.expert_map[i];
  if (tid == 0) nbad = nmixed = 0;
  __syncthreads();
  if constexpr (KIND == kCached) {
    for (int64_t b0 = 0; b0 < T; b0 += kMetaBatchRows) {
      load_raw(b0);
#pragma unroll
      for (int i = 0; i < kMetaBatch; ++i) {
        const int64_t t = b0 + tid + (int64_t)kMetaThreads * i;
        if (t < T) vcache[(int)t] = MOE ? moe_key<MOE>(src, emap, raw[i], rsl[i]) : raw[i];
      }
    }
    __syncthreads();
  }

  // 2. every wave counts the keys of its own contiguous run of rows, 64 rows
  //    at a time: lanes with the same key find each other (through a per-wave
  //    table of lane masks in LDS when it fits: every lane ORs its bit into
  //    its key's entry and reads the entry back; else one ballot per key bit),
  //    and one of them adds their number (no atomics on the counts: a wave
  //    owns its row).  With the keys in LDS, each row's key, rank among equal
  //    keys of its group and the group's count of that key replace it there
  //    (10 + 6 + 7 bits), so the scatter needs no second match.
  const int64_t per_w = (T + kMetaWaves * kWave - 1) / (kMetaWaves * kWave) * kWave;
  const int64_t w_lo = wave * per_w, w_hi = min(T, w_lo + per_w);
  uint64_t *wmask = masks + wave * K;
  int mybad = 0, mixed = 0;
  int pk_small = 0;  // kSmall: this thread's row, packed as in LDS
  for (int64_t b = w_lo; b < w_hi; b += kWave) {
    const int64_t t = b + lane;
    const bool valid = t < w_hi;
    int key = 0;
    if (valid) {
      int v;
      if constexpr (KIND == kSmall) v = MOE ? moe_key<MOE>(src, emap, raw[0], rsl[0]) : raw[0];
      else v = value_at(t);
      const bool ok = v >= -1 && v < S;
      mybad += ok ? 0 : 1;
      key = ok ? v + 1 : 0;
    }
    // one key over the whole step (a long segment): no table, whose word 64
    // lanes would update one after another.  Lane 0 is valid whenever any
    // lane is.
    const uint64_t vm = __ballot(valid);
    const bool uniform = __ballot(valid && key == __builtin_amdgcn_readfirstlane(key)) == vm;
    mixed += uniform ? 0 : 1;
    uint64_t same;
    if (MLDS && !uniform) {
      if (valid) atomicOr(reinterpret_cast<unsigned long long *>(&wmask[key]), 1ull << lane);
      same = valid ? wmask[key] : 0;
    } else if (MLDS) {
      same = valid ? vm : 0;
    } else {
      same = match_key(key, valid, nbits);
    }
    const int rank = __popcll(same & lanemask_lt()), n = __popcll(same);
    if (valid && rank == 0) {
      woff[wave * K + key] += n;
      if (MLDS) wmask[key] = 0;
    }
    const int pk = key | (rank << 10) | (n << 16);
    if (KIND == kSmall) pk_small = pk;
    else if (KIND == kCached && valid) vcache[(int)t] = pk;
  }
  if (mybad) atomicAdd(&nbad, mybad);
  if (STAGE && lane == 0 && mixed) atomicAdd(&nmixed, mixed);
  __syncthreads();
  // scattered rows: at least half of them in steps of several keys
  const bool staged = STAGE && (int64_t)nmixed * kWave * 2 >= T;

  // 3. per key, exclusive prefix of the 16 waves' counts in wave order: the
  //    16 counts of one key sit in one 16-lane row (thread = 16 key + wave)
  //    and are scanned with DPP row shifts; the row total is the key's count
  for (int k0 = 0; k0 < K; k0 += kMetaThreads / kMetaWaves) {
    const int k = k0 + tid / kMetaWaves, w = tid % kMetaWaves;
    const int c = k < K ? woff[w * K + k] : 0;
    const int incl = row16_inclusive_scan(c);
    if (k < K) woff[w * K + k] = incl - c;
    if (k < K && w == kMetaWaves - 1) cnt[k] = incl;
  }
  __syncthreads();

  // 4-5. the key tables, segment arrays and counters
  key_tables(K, T, cnt, kstart, tbase, wsum, nbad, seg_slot, seg_count, seg_start, info);

  // 6. stable scatter: every wave walks its run again, 64 rows at a time; a
  //    row goes to its key's start + the counts of earlier waves and earlier
  //    steps of this wave + its rank among equal keys of the step.  Rows also
  //    land in their work tiles (the key's sorted range cut into runs of 64),
  //    and the row that opens a tile writes the tile's header.
  for (int64_t b = w_lo; b < w_hi; b += kWave) {
    const int64_t t = b + lane;
    const bool valid = t < w_hi;
    int key = 0, rank = 0, n = 0;
    if constexpr (KIND != kStreamed) {
      if (valid) {
        const int pk = KIND == kSmall ? pk_small : vcache[(int)t];
        key = pk & 1023;
        rank = (pk >> 10) & 63;
        n = pk >> 16;
      }
    } else {
      if (valid) {
        const int v = value_at(t);
        key = (v >= -1 && v < S) ? v + 1 : 0;
      }
      const uint64_t same = match_key(key, valid, nbits);
      rank = __popcll(same & lanemask_lt());
      n = __popcll(same);
    }
    if (valid) {
      const int off = woff[wave * K + key] + rank;  // position inside the key's range
      const int dst = kstart[key] + off;
      const int tile = tbase[key] + off / kTileRows;
      auto put = [&](auto o_sorted, auto o_slot, auto tl) __attribute__((always_inline)) {
        o_sorted[dst] = (int32_t)t;
        o_slot[dst] = key - 1;
        tl[4 + off % kTileRows] = (int32_t)t;
        if (off % kTileRows == 0) {
          tl[0] = key - 1;
          tl[1] = min(kTileRows, cnt[key] - off);
          tl[2] = dst;
          tl[3] = 0;
        }
      };
      if (staged) put(st_sorted, st_slot, st_tiles + tile * kTileInts);
      else put(sorted, sorted_slot, tiles + (int64_t)tile * kTileInts);
      if (rank == 0) woff[wave * K + key] += n;
    }
  }
  if (staged) {
    // the staged arrays go out as whole 16-byte pieces (the buffers are
    // 16-byte aligned; the tile list is 17 pieces per tile)
    __syncthreads();
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    const int nt = tbase[K - 1] + (cnt[K - 1] + kTileRows - 1) / kTileRows;
    const int q = (int)(T / 4);
    for (int i = tid; i < q; i += kMetaThreads) {
      *reinterpret_cast<u32x4 *>(sorted + 4 * i) = *(const lds_u32x4 *)(st_sorted + 4 * i);
      *reinterpret_cast<u32x4 *>(sorted_slot + 4 * i) = *(const lds_u32x4 *)(st_slot + 4 * i);
    }
    for (int i = 4 * q + tid; i < T; i += kMetaThreads) {
      sorted[i] = st_sorted[i];
      sorted_slot[i] = st_slot[i];
    }
    for (int i = tid; i < nt * (kTileInts / 4); i += kMetaThreads)
      *reinterpret_cast<u32x4 *>(tiles + 4 * i) = *(const lds_u32x4 *)(st_tiles + 4 * i);
  }
}

// ---------------------------------------------------------------- several workgroups
//
// Past several thousand rows one workgroup is bound by its own CU.  Then the
// rows are cut into P contiguous parts and two short kernels share the work:
// every part's workgroup counts its keys; then every part's workgroup reads
// all parts' counts, takes its own first position inside every key and the
// key tables from them (part 0 stores the segment arrays and counters), and
// scatters its rows.
// A part's rows of a key follow those of the parts before it, and inside a
// part the rows keep batch order (by wave and lane, as in the one-workgroup
// kernel): the sort stays stable, and its result is the same.

template <bool MOE>
__device__ __forceinline__ int meta_row_key(const MetaSrc &src, int64_t t, int32_t S, int &bad) {
  const int v = MOE ? moe_key<MOE>(src, nullptr, src.topk_ids[t], src.token_slot[(uint32_t)t / (uint32_t)src.topk])
                    : src.token_slot[t];
  const bool ok = v >= -1 && v < S;
  bad += ok ? 0 : 1;
  return ok ? v + 1 : 0;
}

// Part p's rows [p q, min(T, (p + 1) q)), q = ceil(T / P).
__device__ __forceinline__ void meta_part(int64_t T, int64_t &lo, int64_t &hi) {
  const int64_t q = (T + gridDim.x - 1) / gridDim.x;
  lo = (int64_t)blockIdx.x * q;
  hi = min(T, lo + q);
}

// 1. counts of part p: counts[p][k] (k < K), counts[p][K] = its bad ids
template <bool MOE>
__global__ __launch_bounds__(kMetaThreads) void meta_count_kernel(MetaSrc src, int64_t T, int32_t S,
                                                                  int32_t *__restrict__ counts) {
  extern __shared__ __align__(16) int32_t lds[];  // [K] this part's count per key
  __shared__ int32_t nbad;
  const int K = S + 1, tid = threadIdx.x;
  for (int i = tid; i < K; i += kMetaThreads) lds[i] = 0;
  if (tid == 0) nbad = 0;
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  __syncthreads();
  int64_t lo, hi;
  meta_part(T, lo, hi);
  int mybad = 0;
  for (int64_t b = lo; b < hi; b += kMetaThreads) {
    const int64_t t = b + tid;
    const bool valid = t < hi;
    const int key = valid ? meta_row_key<MOE>(src, t, S, mybad) : 0;
    const uint64_t same = match_key(key, valid, nbits);
    if (valid && __popcll(same & lanemask_lt()) == 0) atomicAdd(&lds[key], __popcll(same));
  }
  if (mybad) atomicAdd(&nbad, mybad);
  __syncthreads();
  int32_t *out = counts + (int64_t)blockIdx.x * (K + 1);
  for (int i = tid; i < K; i += kMetaThreads) out[i] = lds[i];
  if (tid == 0) out[K] = nbad;
}

// 2. part p: per key (and for the bad ids), the count of the parts before p
// (its first position inside the key) and of all parts; the key tables from
// those (part 0 also stores the segment arrays and counters).  Then the
// scatter, 1024 rows at a time: per step, every wave counts its rows of each
// key (lanes with the same key find each other by ballots), the 16 waves'
// counts per key are prefix-summed in wave order on top of the part's running
// position in the key, and every row goes to its key's start + that position
// + its rank among the wave's equal keys; rows also land in their work tiles,
// the row that opens a tile writing the tile's header
template <bool MOE>
__global__ __launch_bounds__(kMetaThreads) void meta_scatter_kernel(MetaSrc src, int64_t T, int32_t S,
                                                                    const int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ sorted,
                                                                    int32_t *__restrict__ sorted_slot,
                                                                    int32_t *__restrict__ seg_slot,
                                                                    int32_t *__restrict__ seg_count,
                                                                    int32_t *__restrict__ seg_start,
                                                                    int32_t *__restrict__ info,
                                                                    int32_t *__restrict__ tiles) {
  // [K] counts, [K] first positions, [K] first tiles, [K] this part's next
  // position inside each key, [16][K] per-wave counts of a step, then offsets
  extern __shared__ __align__(16) int32_t lds[];
  __shared__ int32_t nbad;
  __shared__ int32_t wsum[kMetaWaves][3];
  const int K = S + 1, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int part = (int)blockIdx.x, nparts = (int)gridDim.x;
  int32_t *cnt = lds, *kstart = lds + K, *tbase = lds + 2 * K, *run = lds + 3 * K, *woff = lds + 4 * K;
  for (int k = tid; k <= K; k += kMetaThreads) {
    int before = 0, all = 0;
    for (int p0 = 0; p0 < nparts; p0 += 8) {  // 8 loads in flight
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = p0 + j < nparts ? counts[(int64_t)(p0 + j) * (K + 1) + k] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        before += p0 + j < part ? c[j] : 0;
        all += c[j];
      }
    }
    if (k < K) {
      cnt[k] = all;
      run[k] = before;
    } else {
      nbad = all;
    }
  }
  for (int i = tid; i < kMetaWaves * K; i += kMetaThreads) woff[i] = 0;
  int nbits = 0;
  while ((1 << nbits) < K) ++nbits;
  __syncthreads();
  key_tables(K, T, cnt, kstart, tbase, wsum, nbad, seg_slot, seg_count, seg_start, info, part == 0);
  int64_t lo, hi;
  meta_part(T, lo, hi);
  for (int64_t b = lo; b < hi; b += kMetaThreads) {
    const int64_t t = b + tid;
    const bool valid = t < hi;
    int unused = 0;
    const int key = valid ? meta_row_key<MOE>(src, t, S, unused) : 0;
    const uint64_t same = match_key(key, valid, nbits);
    const int rank = __popcll(same & lanemask_lt());
    if (valid && rank == 0) woff[wave * K + key] = __popcll(same);
    __syncthreads();
    // per key, the 16 waves' counts sit in one 16-lane row (thread = 16 key +
    // wave): exclusive offsets on top of the running position, which the
    // row's last lane then advances (a wave reads before it writes)
    for (int k0 = 0; k0 < K; k0 += kMetaThreads / kMetaWaves) {
      const int k = k0 + tid / kMetaWaves, w = tid % kMetaWaves;
      const int c = k < K ? woff[w * K + k] : 0;
      const int base = k < K ? run[k] : 0;
      const int incl = row16_inclusive_scan(c);
      if (k < K) woff[w * K + k] = base + incl - c;
      if (k < K && w == kMetaWaves - 1) run[k] = base + incl;
    }
    __syncthreads();
    if (valid) {
      const int off = woff[wave * K + key] + rank;  // position inside the key's range
      const int dst = kstart[key] + off;
      sorted[dst] = (int32_t)t;
      sorted_slot[dst] = key - 1;
      int32_t *tl = tiles + (int64_t)(tbase[key] + off / kTileRows) * kTileInts;
      tl[4 + off % kTileRows] = (int32_t)t;
      if (off % kTileRows == 0) {
        tl[0] = key - 1;
        tl[1] = min(kTileRows, cnt[key] - off);
        tl[2] = dst;
        tl[3] = 0;
      }
    }
    __syncthreads();  // every row has its offset before the next step's counts
    for (int i = tid; i < kMetaWaves * K; i += kMetaThreads) woff[i] = 0;
    __syncthreads();
  }
}

template <bool MOE>
static hipError_t launch_meta_multi(const MetaSrc &src, int64_t T, int32_t S, int32_t *sorted, int32_t *sorted_slot,
                                    int32_t *seg_slot, int32_t *seg_count, int32_t *seg_start, int32_t *info,
                                    int32_t *tiles, hipStream_t stream) {
  const int K = S + 1;
  const int parts = meta_parts(T);
  // the counts sit past the tile list (the workspace layout reserves them)
  int32_t *counts = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(tiles) + meta_tiles_bytes(T, S));
  const size_t scatter_lds = sizeof(int32_t) * (size_t)K * (4 + kMetaWaves);
  if (scatter_lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&meta_scatter_kernel<MOE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)scatter_lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((meta_count_kernel<MOE>), dim3(parts), dim3(kMetaThreads), sizeof(int32_t) * K, stream, src, T,
                     S, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((meta_scatter_kernel<MOE>), dim3(parts), dim3(kMetaThreads), scatter_lds, stream, src, T, S,
                     counts, sorted, sorted_slot, seg_slot, seg_count, seg_start, info, tiles);
  return hipGetLastError();
}

// Dynamic LDS of the metadata kernel: the key tables, the expert map when it
// fits, the keys themselves when they fit too, then the per-wave match tables
// when those fit as well.
static size_t meta_lds_bytes(int32_t S, int64_t T, int32_t E_map, bool &cached, bool &match_lds, bool &stage) {
  size_t b = sizeof(int32_t) * (size_t)(S + 1) * (3 + kMetaWaves);
  if (E_map > 0 && E_map <= kMetaMapLds) b += sizeof(int32_t) * (size_t)E_map;
  // up to 1024 rows the keys stay in registers
  cached = T > kMetaThreads && b + sizeof(int32_t) * (size_t)T <= kMetaLdsMax;
  if (cached) b += sizeof(int32_t) * (size_t)T;
  b = (b + 7) / 8 * 8;
  const size_t tables = sizeof(uint64_t) * (size_t)(S + 1) * kMetaWaves;
  match_lds = b + tables <= kMetaLdsMax;
  if (match_lds) b += tables;
  // the staged sorted arrays and tile list, 16-byte aligned
  b = (b + 15) / 16 * 16;
  const size_t staged = sizeof(int32_t) * (2 * (size_t)((T + 3) / 4 * 4) + (size_t)kTileInts * max_tiles(T, S));
  stage = T >= kMetaStageMin && cached && b + staged <= kMetaLdsMax;
  if (stage) b += staged;
  return b;
}

template <bool MOE, int KIND, bool MLDS, bool STAGE>
static hipError_t launch_meta_k(const MetaSrc &src, int64_t T, int32_t S, size_t lds, int32_t *sorted,
                                int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count, int32_t *seg_start,
                                int32_t *info, int32_t *tiles, hipStream_t stream) {
  if (lds > 65536) {
    // more than the default 64 KB of dynamic LDS
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&meta_kernel<MOE, KIND, MLDS, STAGE>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((meta_kernel<MOE, KIND, MLDS, STAGE>), dim3(1), dim3(kMetaThreads), lds, stream, src.token_slot,
                     src.topk_ids, T, src, S, sorted, sorted_slot, seg_slot, seg_count, seg_start,
                     info, tiles);
  return hipGetLastError();
}

template <bool MOE>
static hipError_t launch_meta_t(const MetaSrc &src, int64_t T, int32_t S, int32_t *sorted,
                                int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count,
                                int32_t *seg_start, int32_t *info, int32_t *tiles, hipStream_t stream) {
  // several workgroups from a few thousand rows on (LORA_META_MULTI forces
  // either way)
  const int knob = meta_multi_knob();
  if (T > 0 && (knob == 1 || (knob < 0 && T >= kMetaMultiMin)))
    return launch_meta_multi<MOE>(src, T, S, sorted, sorted_slot, seg_slot, seg_count, seg_start, info, tiles,
                                  stream);
  bool cached = false, match_lds = false, stage = false;
  const size_t lds = meta_lds_bytes(S, T, MOE && src.expert_map ? src.E_global : 0, cached, match_lds, stage);
  const int kind = T <= kMetaThreads ? kSmall : (cached ? kCached : kStreamed);
  // few keys (at most 4 key bits): one ballot per bit is cheaper than lanes
  // contending for a handful of lane-mask words (measured: 9 keys over 17705
  // rows, 10 us against 18 us of counting)
  if (S + 1 <= 16) match_lds = false;
#define LORA_META_LAUNCH(K, M, G)                                                                                  \
  return launch_meta_k<MOE, K, M, G>(src, T, S, lds, sorted, sorted_slot, seg_slot, seg_count, seg_start, info,     \
                                     tiles, stream)
  if (kind == kSmall) {
    if (match_lds) LORA_META_LAUNCH(kSmall, true, false);
    LORA_META_LAUNCH(kSmall, false, false);
  }
  if (kind == kCached) {
    if (match_lds) {
      if (stage) LORA_META_LAUNCH(kCached, true, true);
      LORA_META_LAUNCH(kCached, true, false);
    }
    if (stage) LORA_META_LAUNCH(kCached, false, true);
    LORA_META_LAUNCH(kCached, false, false);
  }
  if (match_lds) LORA_META_LAUNCH(kStreamed, true, false);
  LORA_META_LAUNCH(kStreamed, false, false);
#undef LORA_META_LAUNCH
}

hipError_t launch_meta(const int32_t *token_slot, int64_t T, int32_t S, int32_t *sorted,
                       int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count, int32_t *seg_start,
                       int32_t *info, int32_t *tiles, hipStream_t stream) {
  MetaSrc src{};
  src.token_slot = token_slot;
  return launch_meta_t<false>(src, T, S, sorted, sorted_slot, seg_slot, seg_count, seg_start, info, tiles, stream);
}

hipError_t launch_meta_moe(const int32_t *topk_ids, int64_t T, int32_t topk, const int32_t *token_slot,
                           int32_t S, int32_t E_global, int32_t E_local, const int32_t *expert_map,
                           int32_t *sorted, int32_t *sorted_slot, int32_t *seg_slot, int32_t *seg_count,
                           int32_t *seg_start, int32_t *info, int32_t *tiles, hipStream_t stream) {
  MetaSrc src{};
  src.token_slot = token_slot;
  src.topk_ids = topk_ids;
  src.expert_map = expert_map;
  src.topk = topk;
  src.S_adapters = S;
  src.E_global = E_global;
  src.E_local = E_local;
  return launch_meta_t<true>(src, T * topk, S * E_local, sorted, sorted_slot, seg_slot, seg_count, seg_start, info,
                             tiles, stream);
}

}  // namespace lora
