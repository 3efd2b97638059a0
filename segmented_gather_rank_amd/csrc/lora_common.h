// lora_common.h -- shared device helpers and kernel argument blocks of the
// gfx950 multi-LoRA kernels.  Internal to the library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lora {

constexpr int kMaxSlices = 8;

// Kernels are instantiated for at most NS slices, NS = 1, 2, 4 or 8: f is
// called with std::integral_constant<int, NS> for the smallest NS >= n.
template <typename F>
inline auto with_slice_bound(int n, F &&f) {
  if (n <= 1) return f(std::integral_constant<int, 1>{});
  if (n <= 2) return f(std::integral_constant<int, 2>{});
  if (n <= 4) return f(std::integral_constant<int, 4>{});
  return f(std::integral_constant<int, 8>{});
}
constexpr int kMaxSlots = 1023;
constexpr int kWave = 64;

// ---------------------------------------------------------------- element types

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

struct F32Tag {};
struct BF16Tag {};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32 converts two values in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Plain loads and stores through the global address space.  A pointer that
// the compiler cannot trace to a global allocation (one rebuilt from integers,
// say) would otherwise be accessed with flat instructions, which count against
// both memory wait counters and so force coarser waits.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
__device__ __forceinline__ u32x4 gload16(const void *p) { return *(const g_u32x4 *)p; }
__device__ __forceinline__ f32x4 gload16f(const void *p) { return *(const g_f32x4 *)p; }
__device__ __forceinline__ void gstore16(void *p, u32x4 v) { *(g_u32x4 *)p = v; }
__device__ __forceinline__ void gstore16f(void *p, f32x4 v) { *(g_f32x4 *)p = v; }

// Sum of kch split-K partial rows of 4 floats at p, p + plane, ..., added in
// k-chunk order.  The loads go out 8 at a time before any of them is waited
// for (a loop that waits for each partial would pay one memory round trip per
// chunk); past the end the last partial is read again and not added.
__device__ __forceinline__ f32x4 sum_partials4(const float *p, int64_t plane, int kch) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < kch; k0 += 8) {
    f32x4 w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = gload16f(p + (int64_t)min(k0 + q, kch - 1) * plane);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (k0 + q < kch) {
        v[0] += w[q][0];
        v[1] += w[q][1];
        v[2] += w[q][2];
        v[3] += w[q][3];
      }
    }
  }
  return v;
}

// Load 8 consecutive elements (16 B of bf16 or 32 B of fp32) as fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
  u32x4 w = gload16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
  f32x4 a = gload16f(p);
  f32x4 b = gload16f(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8(uint16_t *p, const float v[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  gstore16(p, w);
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = v[i];
    b[i] = v[4 + i];
  }
  gstore16f(p, a);
  gstore16f(p + 4, b);
}

// ---------------------------------------------------------------- buffer loads

// Raw buffer resource over [base, base + bytes): a load past the end returns
// zeros instead of touching memory, and offsets are 32-bit, so a kernel walks
// one slot's matrix from a scalar base with unsigned byte offsets and needs no
// branch for a ragged tail.  The base must be uniform across the wave.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------- bf16 pairs

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// (low half of a, low half of b) and (high half of a, high half of b)
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
// c + a.lo * b.lo + a.hi * b.hi, bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
}
// fp32 v split into bf16 hi + lo (v - hi, rounded): about 16 significant bits
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - __uint_as_float(hi << 16));
}

// ---------------------------------------------------------------- wave primitives

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP: a scan inside
// every row of 16 lanes (row shifts; lanes shifted in from outside the row add
// 0), then the last lane of row 0 / row 2 is added into rows 1 / 3
// (row_bcast:15) and the last lane of row 1 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// ---------------------------------------------------------------- parameter arrays

// A value read from the kernel's parameter block, passed through
// v_readfirstlane so that it lives in scalar registers and is opaque to the
// optimiser.  Without it, a chain of selects between such values (below) can be
// folded back into one indexed per-lane load from the parameter block: a vector
// memory load, whose wait would also wait for every vector load issued before it.
template <typename T>
__device__ __forceinline__ T uniform_value(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values only");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
  } else {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    i32x2 w = __builtin_bit_cast(i32x2, v);
    w.x = __builtin_amdgcn_readfirstlane(w.x);
    w.y = __builtin_amdgcn_readfirstlane(w.y);
    return __builtin_bit_cast(T, w);
  }
}

// a[i] for a small array held in a kernel's by-value parameter block, where i
// may differ between lanes and only the first n entries are in use (n is
// uniform).  Indexing the array with a runtime value would make the compiler
// copy the whole block to scratch memory; an unrolled select over scalar
// copies keeps it in registers.  M bounds the entries looked at at compile
// time: kernels instantiated for at most M slices carry no code for more
// (code that runs once per workgroup is fetched cold, so its size is time).
template <int M = 1 << 20, typename T, int N>
__device__ __forceinline__ T pick(const T (&a)[N], int i, int n = N) {
  constexpr int L = M < N ? M : N;
  T v = uniform_value(a[0]);
#pragma unroll
  for (int k = 1; k < L; ++k) {
    if (k >= n) break;
    v = (i == k) ? uniform_value(a[k]) : v;
  }
  return v;
}

// Index of the last entry of prefix[0..n) (non-decreasing, prefix[0] = 0)
// that is <= v.
template <int M = 1 << 20, int N>
__device__ __forceinline__ int last_le(const int32_t (&prefix)[N], int n, int v) {
  constexpr int L = M < N ? M : N;
  int s = 0;
#pragma unroll
  for (int k = 1; k < L; ++k) {
    if (k >= n) break;
    s = (uniform_value(prefix[k]) <= v) ? k : s;
  }
  return s;
}

// ---------------------------------------------------------------- slot ranks

// Ranks a kernel reads for a slot: its own rank rounded up to whole octets of
// 8, clamped to [0, R]; R when no per-slot ranks are given.  (The rank is
// uniform across a workgroup.)
__device__ __forceinline__ int slot_rank_of(const int32_t *slot_rank, int slot, int R) {
  if (!slot_rank) return R;
  const int r = __builtin_amdgcn_readfirstlane(slot_rank[slot]);
  return r <= 0 ? 0 : (r >= R ? R : (r + 7) & ~7);
}

// ---------------------------------------------------------------- factor rows

// The kernels are built for a rank R in {8, 16, 32, 64, 128} and walk a
// slot's A as a packed [k][R] block; the caller's matrix is [d_in][ra] with
// ra = r_max, a multiple of 8 and at most R.  Element e of the packed block
// (row e / R, rank e % R) lives at e / R * ra + e % R, and ranks past ra read
// as zeros (rank_limit caps the ranks a kernel reads at ra).
template <int R>
__device__ __forceinline__ int64_t packed_to_factor(int64_t e, int ra) {
  return R == 0 ? e : (e / R) * ra + (e % R);
}

// ---------------------------------------------------------------- measurement build
// With -DLORA_PHASE_CLOCK (a measurement build) the tile shrink and the tile
// expand can record, per workgroup, the 100 MHz real-time counter at their
// phase boundaries into kTilePhaseWords 64-bit words; `rec` is null unless the
// host asked the kernel to record.  Other builds compile the stamps out.
constexpr int kTilePhaseWords = 16;
#ifdef LORA_PHASE_CLOCK
constexpr bool kPhaseClock = true;
#else
constexpr bool kPhaseClock = false;
#endif
__device__ __forceinline__ void phase_stamp(unsigned long long *rec, int k) {
  if constexpr (kPhaseClock) {
    if (rec && threadIdx.x == 0) rec[k] = (unsigned long long)__builtin_amdgcn_s_memrealtime();
  }
}
__device__ __forceinline__ void phase_put(unsigned long long *rec, int k, unsigned long long v) {
  if constexpr (kPhaseClock) {
    if (rec && threadIdx.x == 0) rec[k] = v;
  }
}
__device__ __forceinline__ unsigned long long *phase_record(unsigned long long *clk) {
  return kPhaseClock && clk ? clk + (int64_t)blockIdx.x * kTilePhaseWords : nullptr;
}

// ---------------------------------------------------------------- metadata view

struct MetaView {
  const int32_t *sorted;
  const int32_t *sorted_slot;
  const int32_t *seg_slot;
  const int32_t *seg_count;
  const int32_t *seg_start;
  const int32_t *info;   // num_segments, no_lora, num_bad, lora_begin, num_tiles
  const int32_t *tiles;  // kTileInts int32 per tile: slot, rows, pos0, 0, tokens[kTileRows]
  int64_t T;
  int32_t S;
  int32_t x_row_div;     // batch row i reads x row i / x_row_div
};

// x row read by batch row i.
__device__ __forceinline__ int64_t x_row_of(const MetaView &m, int64_t i) {
  return m.x_row_div == 1 ? i : i / m.x_row_div;
}

// Work tiles of the metadata: every segment cut into runs of at most
// kTileRows sorted positions.
constexpr int kTileRows = 64;
constexpr int kTileInts = 4 + kTileRows;
__host__ __device__ constexpr int64_t max_tiles(int64_t T, int32_t S) {
  return (T + kTileRows - 1) / kTileRows + S + 1;
}

// ---------------------------------------------------------------- work lists
//
// Both compute kernels walk a list of items derived in-kernel from the segment
// table: every segment is cut into m-chunks (the chunk size depends on the path
// the segment takes) and every m-chunk into items (k-chunks for the shrink,
// slice x n-tile pairs for the expand).  The segment table is copied to LDS
// with one memory round trip (every entry's load is issued before any wait),
// one wave prefix-sums the item counts, and each item is located by binary
// search over that prefix.

struct SegTable {
  int32_t *count, *slot, *start;  // LDS copies of seg_count, seg_slot, seg_start
  int32_t *item_end;              // inclusive prefix of items per used segment
  int32_t *scal;                  // [0] used segments, [1] first used, [2] items, [3] nseg
};

// LDS bytes of a segment table for S slots
__host__ __device__ constexpr size_t seg_table_bytes(int S) {
  return sizeof(int32_t) * (4 * (size_t)(S + 2) + 4);
}

__device__ __forceinline__ SegTable seg_table_at(void *lds, int S) {
  int32_t *b = reinterpret_cast<int32_t *>(lds);
  const int n = S + 2;
  return SegTable{b, b + n, b + 2 * n, b + 3 * n, b + 4 * n};
}

// Fill the table.  Segments from index `first` on are used, where first = 1
// when skip_none is set and the leading segment is the no-adapter one; used
// segment i gets items_of(count, slot) items.  Ends with a barrier.
template <typename F>
__device__ __forceinline__ void build_items(const MetaView &m, SegTable tb, bool skip_none, F items_of) {
  const int K = m.S + 1;
  for (int i = threadIdx.x; i < K; i += blockDim.x) {
    tb.count[i] = m.seg_count[i];
    tb.slot[i] = m.seg_slot[i];
    tb.start[i] = m.seg_start[i];
  }
  if (threadIdx.x == 0) tb.scal[3] = m.info[0];
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int nseg = tb.scal[3];
    const int first = (skip_none && nseg > 0 && tb.slot[0] == -1) ? 1 : 0;
    const int nl = nseg - first;
    int base = 0;
    for (int i0 = 0; i0 < nl; i0 += kWave) {
      const int i = i0 + lane;
      const int items = i < nl ? items_of(tb.count[first + i], tb.slot[first + i]) : 0;
      const int incl = wave_inclusive_scan(items);
      if (i < nl) tb.item_end[i] = base + incl;
      base += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) {
      tb.scal[0] = nl;
      tb.scal[1] = first;
      tb.scal[2] = base;
    }
  }
  __syncthreads();
}

// Used-segment index of an item (binary search over the item prefix).
__device__ __forceinline__ int find_item_segment(SegTable tb, int item) {
  int lo = 0, hi = tb.scal[0] - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (tb.item_end[mid] > item) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// ---------------------------------------------------------------- LDS transposing read

typedef short i16x4 __attribute__((ext_vector_type(4)));

// MFMA 16x16x32 operand from a row-major bf16 tile in LDS: this lane (column
// n = lane % 16 of a 16-column block starting at `col0`) receives
// tile[row0 + e][col0 + n] for e = 0..7, where `ld` is the row stride in
// elements.  Two gfx950 transposing reads: inside each group of 16 lanes,
// lane 4e + c names 4 consecutive elements (row row0 + e, columns col0 + 4c ..
// + 3) and lane i receives element i % 4 of the chunks named by lanes 4e + i/4,
// e = 0..3, i.e. column col0 + i of rows row0 .. row0 + 3.
__device__ __forceinline__ bf16x8 lds_col8(const uint16_t *tile, int ld, int row0, int col0) {
  const int l = threadIdx.x % 16;
  const uint16_t *a = tile + (row0 + l / 4) * ld + col0 + 4 * (l % 4);
  typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(a)));
  const u32x2 hi =
      __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(a + 4 * ld)));
  const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, w);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A operand of v_mfma_f32_16x16x16_bf16 from a row-major bf16 tile in LDS:
// lane i of each 16-lane group receives tile[row0 + e][col0 + i], e = 0..3,
// where row0 is this lane's group's first row.
__device__ __forceinline__ s16x4 lds_col4(const uint16_t *tile, int ld, int row0, int col0) {
  const int l = threadIdx.x % 16;
  const uint16_t *a = tile + (row0 + l / 4) * ld + col0 + 4 * (l % 4);
  typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
  return __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(a)));
}

// ---------------------------------------------------------------- DPP helpers

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the lanes of a wave that share (lane mod JO), JO in {1,2,4,8,16}: DPP
// row rotations inside each 16-lane row, then the gfx950 permlane16 and
// permlane32 swaps across rows.
template <int JO>
__device__ __forceinline__ float wave_sum_mod(float v) {
  static_assert(JO == 1 || JO == 2 || JO == 4 || JO == 8 || JO == 16, "lanes share a residue mod 1..16");
  if constexpr (JO < 2) v += dpp_f32<0x121>(v);   // row_ror:1
  if constexpr (JO < 4) v += dpp_f32<0x122>(v);   // row_ror:2
  if constexpr (JO < 8) v += dpp_f32<0x124>(v);   // row_ror:4
  if constexpr (JO < 16) v += dpp_f32<0x128>(v);  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 8 consecutive elements held as raw words (bf16: 4 words, fp32: 8 words),
// widened to fp32 on use.
template <typename E> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t *p) { w = gload16(p); }
  __device__ __forceinline__ void zero() { w = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float operator[](int i) const {
    return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = gload16f(p);
    b = gload16f(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ float operator[](int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

}  // namespace lora
