// lora_common.h -- shared device helpers and kernel argument blocks of the
// gfx950 multi-LoRA kernels.  Internal to the library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kMaxSlices = 8;
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

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Load 8 consecutive elements (16 B of bf16 or 32 B of fp32) as fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
  u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(w[i]);
    v[2 * i + 1] = bf16_hi(w[i]);
  }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
  f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
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
  *reinterpret_cast<u32x4 *>(p) = w;
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = v[i];
    b[i] = v[4 + i];
  }
  *reinterpret_cast<f32x4 *>(p) = a;
  *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// ---------------------------------------------------------------- wave primitives

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// ---------------------------------------------------------------- metadata view

struct MetaView {
  const int32_t *sorted;
  const int32_t *sorted_slot;
  const int32_t *seg_slot;
  const int32_t *seg_count;
  const int32_t *seg_start;
  const int32_t *info;  // num_segments, no_lora, num_bad, lora_begin
  int64_t T;
  int32_t S;
};

// ---------------------------------------------------------------- work lists
//
// Both compute kernels walk a list of items derived in-kernel from the segment
// counts: every segment with an adapter is cut into m-chunks of `mc` tokens
// (mc depends on the path the segment takes), and every m-chunk into `per_chunk`
// items (k-chunks for the shrink, slice x n-tile pairs for the expand).  The
// per-segment item counts are prefix-summed in LDS by one wave, and each item
// is located by binary search over that prefix.

struct SegPlan {
  int32_t item_end[kMaxSlots + 2];   // inclusive prefix of items per segment
  int32_t nseg;
  int32_t total_items;
};

}  // namespace lora
