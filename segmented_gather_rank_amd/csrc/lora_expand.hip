// lora_expand.hip -- y[t][off_s + n] (+)= u[s][t][:] . B_s[a][:][n], a = slot(t).
//
// Page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩 GEMM:shrink、
// expand 与 fp32 中转缓冲": the expand multiplies each segment's fp32 rank-r rows
// by the segment's B and adds them into the column window
// [offset_start, offset_start + width) of the base output, one window per packed
// slice, each slice with its own width; ADD_INPUTS chooses add or store.  Section
// "双流:让 LoRA 与基座前向并行": rows without an adapter must end up holding the
// base output (add) or zero (store).
//
// Work items: (segment, m-chunk, slice, n-tile) in a grid-stride loop.
//  * vector path (the BGMV form; fp32, and short bf16 segments): a wave owns 512
//    output columns, 8 per lane; B rows are read with 16-byte loads straight
//    into registers and reused for every token of the m-chunk, whose u rows sit
//    in LDS; the y row segment is read, updated and written with 16-byte
//    accesses.  Rows without an adapter are zero-filled here when storing.
//  * matrix-core path (the SGMV form; bf16 segments of at least `mfma_min`
//    tokens): 64 tokens x 128 columns per item, v_mfma_f32_16x16x32_bf16 with
//    K = rank; u is split into bf16 hi + lo parts (two products), so the result
//    carries about 16 mantissa bits of u rather than 8; B tile transposed into
//    LDS with an XOR swizzle; the fp32 tile goes through LDS so that y is read
//    and written 16 bytes per lane.
#include "lora_host.h"

namespace lora {

constexpr int kExpThreads = 256;
constexpr int kEVecRows = 8;    // tokens per vector m-chunk (2 per wave)
constexpr int kEVecCols = 512;  // columns per vector n-tile (64 lanes x 8)
constexpr int kEMmaRows = 64;   // tokens per matrix-core m-chunk
constexpr int kEMmaCols = 128;  // columns per matrix-core n-tile

struct ExpandParams {
  MetaView meta;
  const float *u;  // [n_slices][T][R]
  const void *B[kMaxSlices];
  int64_t b_stride[kMaxSlices];
  int64_t width[kMaxSlices];
  int64_t offset[kMaxSlices];
  int32_t tiles_vec[kMaxSlices + 1];  // exclusive prefix of n-tiles per slice
  int32_t tiles_mma[kMaxSlices + 1];
  int32_t n_slices;
  void *y;
  int64_t ldy;
  int32_t add;
  int32_t use_mma_mode, mfma_min;
};

template <int R>
struct ExpandLds {
  SegPlan plan;
  union {
    struct {
      float us[kEVecRows][R];
    } vec;
    struct {
      uint16_t bt[kEMmaCols][(R < 32 ? 32 : R) + 8];
    } mma;
    struct {
      float out[kEMmaRows][kEMmaCols + 4];
    } epi;
  };
};

__device__ __forceinline__ bool exp_takes_mma(const ExpandParams &p, int count, int slot) {
  return slot >= 0 && (p.use_mma_mode == 2 || (p.use_mma_mode == 1 && count >= p.mfma_min));
}

template <int R>
__device__ void exp_build_plan(const ExpandParams &p, SegPlan &plan, int first) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int nl = p.meta.info[0] - first;
    int item_base = 0;
    for (int i0 = 0; i0 < nl; i0 += kWave) {
      const int i = i0 + lane;
      int items = 0;
      if (i < nl) {
        const int c = p.meta.seg_count[first + i];
        const int slot = p.meta.seg_slot[first + i];
        const bool mma = exp_takes_mma(p, c, slot);
        const int mc = mma ? kEMmaRows : kEVecRows;
        items = ((c + mc - 1) / mc) * (mma ? p.tiles_mma[p.n_slices] : p.tiles_vec[p.n_slices]);
      }
      const int ii = wave_inclusive_scan(items);
      if (i < nl) plan.item_end[i] = item_base + ii;
      item_base += __shfl(ii, kWave - 1, kWave);
    }
    if (lane == 0) {
      plan.nseg = nl;
      plan.total_items = item_base;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int exp_find_segment(const SegPlan &plan, int item) {
  int lo = 0, hi = plan.nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (plan.item_end[mid] > item) hi = mid; else lo = mid + 1;
  }
  return lo;
}

__device__ __forceinline__ int slice_of_tile(const int32_t *prefix, int n_slices, int tile) {
  int s = 0;
  while (s + 1 < n_slices && prefix[s + 1] <= tile) ++s;
  return s;
}

// ------------------------------------------------------------------ vector path

template <typename E, int R>
__device__ void exp_vec_item(const ExpandParams &p, ExpandLds<R> &lds, int slot, int64_t pos0,
                             int rows, int s, int nt) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t T = p.meta.T;
  if (slot >= 0) {
    for (int idx = tid; idx < rows * R; idx += kExpThreads) {
      const int mm = idx / R, j = idx % R;
      const int64_t t = p.meta.sorted[pos0 + mm];
      lds.vec.us[mm][j] = p.u[((int64_t)s * T + t) * R + j];
    }
  }
  __syncthreads();
  const int64_t w = p.width[s];
  const int64_t n0 = (int64_t)nt * kEVecCols + 8 * lane;
  if (n0 < w) {
    E *y = reinterpret_cast<E *>(p.y);
    // the y segments do not depend on u or B: read them first
    E *yp[2] = {nullptr, nullptr};
    float v[2][8], acc[2][8];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mm = wave + 4 * m;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[m][c] = acc[m][c] = 0.f;
      if (mm < rows) {
        yp[m] = y + (int64_t)p.meta.sorted[pos0 + mm] * p.ldy + p.offset[s] + n0;
        if (p.add) load8(yp[m], v[m]);
      }
    }
    if (slot >= 0) {
      const E *Bb = reinterpret_cast<const E *>(p.B[s]) + (int64_t)slot * p.b_stride[s] + n0;
#pragma unroll
      for (int j0 = 0; j0 < R; j0 += 8) {
        float b[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) load8(Bb + (int64_t)(j0 + i) * w, b[i]);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int mm = wave + 4 * m;
          if (mm < rows) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float uv = lds.vec.us[mm][j0 + i];
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[m][c] = fmaf(uv, b[i][c], acc[m][c]);
            }
          }
        }
      }
    }
    // the delta is summed on its own, then added to y once
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (yp[m]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[m][c] += acc[m][c];
        store8(yp[m], v[m]);
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------- matrix-core path

template <int R>
__device__ void exp_mma_item(const ExpandParams &p, ExpandLds<R> &lds, int slot, int64_t pos0,
                             int rows, int s, int nt) {
  constexpr int RP = R < 32 ? 32 : R;  // K padded to whole 32-wide steps
  constexpr int SWZ = RP / 8 - 1;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t T = p.meta.T;
  const int64_t w = p.width[s];
  const int64_t nbase = (int64_t)nt * kEMmaCols;
  const uint16_t *Bb = reinterpret_cast<const uint16_t *>(p.B[s]) + (int64_t)slot * p.b_stride[s];

  // B tile [R][128] -> LDS transposed: bt[n][j ^ swz(n)]
  for (int idx = tid; idx < RP * (kEMmaCols / 8); idx += kExpThreads) {
    const int j = idx / (kEMmaCols / 8);
    const int n0 = 8 * (idx % (kEMmaCols / 8));
    uint16_t v[8];
    if (j < R && nbase + n0 < w) {
      u32x4 q = *reinterpret_cast<const u32x4 *>(Bb + (int64_t)j * w + nbase + n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = (uint16_t)(q[i] & 0xffffu);
        v[2 * i + 1] = (uint16_t)(q[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + i;
      lds.mma.bt[n][j ^ (((n >> 3) & SWZ) << 3)] = v[i];
    }
  }
  // u fragments, split into bf16 hi + lo: lane (mrow, g), step c holds k = 32c + 8g + e
  const int mrow = lane % 16, g = lane / 16;
  const int row = 16 * wave + mrow;
  const int64_t trow = row < rows ? (int64_t)p.meta.sorted[pos0 + row] : -1;
  bf16x8 uh[RP / 32], ul[RP / 32];
#pragma unroll
  for (int c = 0; c < RP / 32; ++c) {
    const int k = 32 * c + 8 * g;
    float v[8];
    if (trow >= 0 && k < R) {
      const float *src = p.u + ((int64_t)s * T + trow) * R + k;
      f32x4 a = *reinterpret_cast<const f32x4 *>(src);
      f32x4 b = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t hb = f32_to_bf16(v[i]);
      const float hf = __uint_as_float(hb << 16);
      const uint32_t lb = f32_to_bf16(v[i] - hf);
      uh[c][i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
      ul[c][i] = __builtin_bit_cast(__bf16, (uint16_t)lb);
    }
  }
  __syncthreads();
  f32x4 acc[kEMmaCols / 16];
#pragma unroll
  for (int b = 0; b < kEMmaCols / 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < RP / 32; ++c) {
    const int k = 32 * c + 8 * g;
#pragma unroll
    for (int b = 0; b < kEMmaCols / 16; ++b) {
      const int n = 16 * b + mrow;
      const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&lds.mma.bt[n][k ^ (((n >> 3) & SWZ) << 3)]);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[c], bv, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul[c], bv, acc[b], 0, 0, 0);
    }
  }
  __syncthreads();  // bt fully read before the epilogue reuses the LDS
#pragma unroll
  for (int b = 0; b < kEMmaCols / 16; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) lds.epi.out[16 * wave + 4 * g + v][16 * b + mrow] = acc[b][v];
  __syncthreads();
  uint16_t *y = reinterpret_cast<uint16_t *>(p.y);
  for (int idx = tid; idx < kEMmaRows * (kEMmaCols / 8); idx += kExpThreads) {
    const int r_ = idx / (kEMmaCols / 8);
    const int o = idx % (kEMmaCols / 8);
    const int64_t n = nbase + 8 * o;
    if (r_ < rows && n < w) {
      const int64_t t = p.meta.sorted[pos0 + r_];
      uint16_t *yp = y + t * p.ldy + p.offset[s] + n;
      float v[8];
      if (p.add) load8(yp, v);
      else {
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] += lds.epi.out[r_][8 * o + c];
      store8(yp, v);
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ the kernel

template <typename E, int R>
__global__ __launch_bounds__(kExpThreads) void expand_kernel(ExpandParams p) {
  __shared__ ExpandLds<R> lds;
  const int nseg = p.meta.info[0];
  // the no-adapter segment (always first) is visited only to store zeros
  const int first = (nseg > 0 && p.meta.seg_slot[0] == -1 && p.add) ? 1 : 0;
  exp_build_plan<R>(p, lds.plan, first);
  for (int item = blockIdx.x; item < lds.plan.total_items; item += gridDim.x) {
    const int si = exp_find_segment(lds.plan, item);
    const int seg = first + si;
    const int count = p.meta.seg_count[seg];
    const int slot = p.meta.seg_slot[seg];
    const int local = item - (si > 0 ? lds.plan.item_end[si - 1] : 0);
    if constexpr (sizeof(E) == 2) {
      if (exp_takes_mma(p, count, slot)) {
        const int ntiles = p.tiles_mma[p.n_slices];
        const int chunk = local / ntiles, tile = local % ntiles;
        const int s = slice_of_tile(p.tiles_mma, p.n_slices, tile);
        const int64_t pos0 = (int64_t)p.meta.seg_start[seg] + (int64_t)chunk * kEMmaRows;
        exp_mma_item<R>(p, lds, slot, pos0, min(kEMmaRows, count - chunk * kEMmaRows), s,
                        tile - p.tiles_mma[s]);
        continue;
      }
    }
    const int ntiles = p.tiles_vec[p.n_slices];
    const int chunk = local / ntiles, tile = local % ntiles;
    const int s = slice_of_tile(p.tiles_vec, p.n_slices, tile);
    const int64_t pos0 = (int64_t)p.meta.seg_start[seg] + (int64_t)chunk * kEVecRows;
    exp_vec_item<E, R>(p, lds, slot, pos0, min(kEVecRows, count - chunk * kEVecRows), s,
                       tile - p.tiles_vec[s]);
  }
}

// ------------------------------------------------------------------ host side

template <typename E, int R>
static hipError_t launch_t(const ExpandParams &p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((expand_kernel<E, R>), dim3(grid), dim3(kExpThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_expand(const MetaView &meta, const float *u, int32_t n_slices,
                         const void *const *B, const int64_t *b_stride, const int64_t *width,
                         const int64_t *offset, int32_t R, void *y, int64_t ldy, bool bf16,
                         int add, int mode, hipStream_t stream) {
  ExpandParams p{};
  p.meta = meta;
  p.u = u;
  p.n_slices = n_slices;
  p.tiles_vec[0] = p.tiles_mma[0] = 0;
  int64_t cols = 0;
  for (int s = 0; s < n_slices; ++s) {
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
    p.tiles_vec[s + 1] = p.tiles_vec[s] + (int32_t)((width[s] + kEVecCols - 1) / kEVecCols);
    p.tiles_mma[s + 1] = p.tiles_mma[s] + (int32_t)((width[s] + kEMmaCols - 1) / kEMmaCols);
    cols += width[s];
  }
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  p.use_mma_mode = !bf16 ? 0 : (mode == 1 ? 0 : (mode == 2 ? 2 : 1));
  p.mfma_min = expand_mma_min_default();
  if (meta.T == 0) return hipSuccess;
  const int64_t T = meta.T, S = meta.S;
  const int64_t bound_vec = ((T + kEVecRows - 1) / kEVecRows + S + 1) * p.tiles_vec[n_slices];
  const int64_t bound_mma =
      p.use_mma_mode ? ((T + kEMmaRows - 1) / kEMmaRows + S + 1) * p.tiles_mma[n_slices] : 0;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(bound_vec + bound_mma, 4096));
  (void)cols;
  switch (R) {
    case 8: return bf16 ? launch_t<uint16_t, 8>(p, grid, stream) : launch_t<float, 8>(p, grid, stream);
    case 16: return bf16 ? launch_t<uint16_t, 16>(p, grid, stream) : launch_t<float, 16>(p, grid, stream);
    case 32: return bf16 ? launch_t<uint16_t, 32>(p, grid, stream) : launch_t<float, 32>(p, grid, stream);
    case 64: return bf16 ? launch_t<uint16_t, 64>(p, grid, stream) : launch_t<float, 64>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
