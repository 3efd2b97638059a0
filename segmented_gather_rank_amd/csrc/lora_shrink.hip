// lora_shrink.hip -- u[s][t][:] = scale * slot_scale[a] * x[t] . A_s[a], a = slot(t).
//
// Page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩 GEMM:shrink、
// expand 与 fp32 中转缓冲": the shrink gathers each segment's token rows through
// the sorted token order, multiplies them by the segment's A and writes an fp32
// buffer laid out [slice][token][rank]; row offsets are 64-bit.  Page "多 LoRA
// 服务：分段矩阵乘与适配器调度", section "不合并权重，批量计算": BGMV (one small
// matrix-vector product per token) suits decode, SGMV (one small matrix product
// per segment) suits prefill.
//
// One kernel, a grid-stride loop over work items.  Every segment with an adapter
// is cut into m-chunks (8 tokens on the vector path, 64 on the matrix-core
// path) and every m-chunk into k-chunks of d_in.  Each item reads its slot's A
// chunk once and applies it to all tokens of the m-chunk, so a slot's A is read
// from HBM once per m-chunk rather than once per token.
//
//  * vector path (the BGMV form; fp32, and short bf16 segments): x rows staged
//    in LDS as fp32; each thread reads 8 contiguous A values (one rank octet of
//    one k row) per pass with a coalesced 16-byte load and accumulates 8 ranks
//    x 8 tokens in registers; the contraction over k is finished in registers
//    by DPP row rotations and the gfx950 permlane16/32 swaps, then by a
//    fixed-order sum over the 4 waves in LDS.
//  * matrix-core path (the SGMV form; bf16 segments of at least `mfma_min`
//    tokens): v_mfma_f32_16x16x32_bf16, 16 token rows per wave; the A tile
//    (128 k x n_slices*r) is transposed into LDS with an XOR swizzle so both the
//    transposing writes and the 16-byte operand reads are bank-conflict free;
//    x fragments go straight from global memory to registers.
//
// With more than one k-chunk, items write scaled fp32 partial sums indexed by
// sorted position, and a second small kernel adds them in k-chunk order into u:
// the result does not depend on scheduling, and no workgroup ever waits for or
// synchronises with another (a cross-XCD release fence costs an L2 write-back).
#include "lora_host.h"

namespace lora {

constexpr int kShrinkThreads = 256;
constexpr int kVecRows = 8;        // tokens per vector m-chunk
constexpr int kVecSub = 1024;      // k per staged x sub-chunk on the vector path
constexpr int kMmaRows = 64;       // tokens per matrix-core m-chunk (4 waves x 16)
constexpr int kMmaKT = 128;        // k per staged A tile on the matrix-core path
constexpr int kMmaCols = 128;      // n_slices*r columns per pass (8 MFMA blocks)
constexpr int kAtStride = kMmaKT + 8;  // bf16 elements per transposed A row

struct ShrinkParams {
  MetaView meta;
  const void *x;
  int64_t ldx, d_in;
  const void *A[kMaxSlices];
  int64_t a_stride[kMaxSlices];
  int32_t n_slices;
  float scale;
  const float *slot_scale;
  // kch == 1: out is u [n_slices][T][R] in token order; otherwise the partial
  // sums [kch][n_slices][T][R] in sorted-position order
  float *out;
  int32_t use_mma_mode;  // 0 = never, 1 = by segment length, 2 = always
  int32_t mfma_min;
  int32_t kc, kch;       // k-chunk length (a multiple of 128) and count
};

struct ShrinkLds {
  SegPlan plan;
  union {
    struct {
      float xs[kVecRows][kVecSub];
      float red[4][kVecRows][64];
    } vec;
    struct {
      uint16_t at[kMmaCols][kAtStride];
    } mma;
  };
};

__device__ __forceinline__ bool seg_takes_mma(const ShrinkParams &p, int count) {
  return p.use_mma_mode == 2 || (p.use_mma_mode == 1 && count >= p.mfma_min);
}

// One wave fills the per-segment item prefix of the adapter segments.
__device__ void build_plan(const ShrinkParams &p, SegPlan &plan) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int nseg = p.meta.info[0];
    const int first = (nseg > 0 && p.meta.seg_slot[0] == -1) ? 1 : 0;
    const int nl = nseg - first;
    int item_base = 0;
    for (int i0 = 0; i0 < nl; i0 += kWave) {
      const int i = i0 + lane;
      int items = 0;
      if (i < nl) {
        const int c = p.meta.seg_count[first + i];
        const int mc = seg_takes_mma(p, c) ? kMmaRows : kVecRows;
        items = ((c + mc - 1) / mc) * p.kch;
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

__device__ __forceinline__ int find_segment(const SegPlan &plan, int item) {
  int lo = 0, hi = plan.nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (plan.item_end[mid] > item) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Store one result of row `mm` of an m-chunk: straight into u (token order)
// when d_in is not split, else into the partial sums (sorted-position order).
__device__ __forceinline__ void put(const ShrinkParams &p, int R, int s, int64_t pos, int j,
                                   int kc, float v) {
  const int64_t T = p.meta.T;
  if (p.kch == 1) {
    const int64_t t = p.meta.sorted[pos];
    p.out[((int64_t)s * T + t) * R + j] = v;
  } else {
    p.out[(((int64_t)kc * p.n_slices + s) * T + pos) * R + j] = v;
  }
}

// ------------------------------------------------------------------ vector path

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the lanes of a wave that share (lane mod JO): DPP row rotations
// inside each 16-lane row, then the permlane16 / permlane32 swaps across rows.
template <int JO>
__device__ __forceinline__ float reduce_lanes(float v) {
  if constexpr (JO < 2) v += dpp<0x121>(v);   // row_ror:1
  if constexpr (JO < 4) v += dpp<0x122>(v);   // row_ror:2
  if constexpr (JO < 8) v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x128>(v);                         // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename E, int R>
__device__ void vec_item(const ShrinkParams &p, ShrinkLds &lds, int slot, int64_t pos0,
                         int rows, int kc, float sc) {
  constexpr int JO = R / 8;  // rank octets per k row
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t k0 = (int64_t)kc * p.kc;
  const int klen = (int)min((int64_t)p.kc, p.d_in - k0);
  const E *x = reinterpret_cast<const E *>(p.x);
  const int jo = tid % JO;
  int staged = -1;  // which x sub-chunk sits in LDS

  for (int s = 0; s < p.n_slices; ++s) {
    float acc[kVecRows][8];
#pragma unroll
    for (int m = 0; m < kVecRows; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[m][i] = 0.f;

    for (int sub = 0; sub < klen; sub += kVecSub) {
      const int slen = min(kVecSub, klen - sub);
      if (staged != sub) {
        __syncthreads();  // earlier readers of xs are done
        const int oct = slen / 8;
        for (int idx = tid; idx < rows * oct; idx += kShrinkThreads) {
          const int row = idx / oct, c = idx - row * oct;
          const int64_t t = p.meta.sorted[pos0 + row];
          float v[8];
          load8(x + t * p.ldx + k0 + sub + 8 * c, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) lds.vec.xs[row][8 * c + i] = v[i];
        }
        __syncthreads();
        staged = sub;
      }
      const E *Ab = reinterpret_cast<const E *>(p.A[s]) + (int64_t)slot * p.a_stride[s] +
                    (k0 + sub) * R;
      const int nel = slen * R;
      for (int e = 8 * tid; e < nel; e += 8 * kShrinkThreads) {
        float a[8];
        load8(Ab + e, a);
        const int k = e / R;
#pragma unroll
        for (int m = 0; m < kVecRows; ++m) {
          const float xv = lds.vec.xs[m][k];   // rows >= `rows` hold stale data, never stored
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[m][i] = fmaf(xv, a[i], acc[m][i]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kVecRows; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[m][i] = reduce_lanes<JO>(acc[m][i]);
    if (lane < JO) {
#pragma unroll
      for (int m = 0; m < kVecRows; ++m)
#pragma unroll
        for (int i = 0; i < 8; ++i) lds.vec.red[wave][m][8 * jo + i] = acc[m][i];
    }
    __syncthreads();
    for (int idx = tid; idx < rows * R; idx += kShrinkThreads) {
      const int mm = idx / R, j = idx % R;
      const float v = ((lds.vec.red[0][mm][j] + lds.vec.red[1][mm][j]) + lds.vec.red[2][mm][j]) +
                      lds.vec.red[3][mm][j];
      put(p, R, s, pos0 + mm, j, kc, v * sc);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- matrix-core path

template <int R>
__device__ void mma_item(const ShrinkParams &p, ShrinkLds &lds, int slot, int64_t pos0,
                         int rows, int kc, float sc) {
  constexpr int SG = kMmaCols / R;  // slices per pass
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t kbeg = (int64_t)kc * p.kc;
  const int64_t kend = min(p.d_in, kbeg + p.kc);
  const uint16_t *x = reinterpret_cast<const uint16_t *>(p.x);

  const int mrow = lane % 16, g = lane / 16;
  const int row = 16 * wave + mrow;               // this lane's operand row
  const int64_t trow = row < rows ? (int64_t)p.meta.sorted[pos0 + row] : -1;

  for (int s0 = 0; s0 < p.n_slices; s0 += SG) {
    const int ns = min(SG, p.n_slices - s0);
    const int nblk = ns * R / 16;
    f32x4 acc[kMmaCols / 16];
#pragma unroll
    for (int b = 0; b < kMmaCols / 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t kt = kbeg; kt < kend; kt += kMmaKT) {
      const int klen = (int)min((int64_t)kMmaKT, kend - kt);
      __syncthreads();  // previous tile fully consumed
      // A tile -> LDS, transposed: at[n][k ^ swz(n)], n = slice*R + j
      const int per_slice = kMmaKT * R / 8;
      for (int idx = tid; idx < ns * per_slice; idx += kShrinkThreads) {
        const int sl = idx / per_slice;
        const int e = 8 * (idx - sl * per_slice);
        const int k = e / R, j0 = e % R;
        const int n0 = sl * R + j0;
        uint16_t v[8];
        if (k < klen) {
          const uint16_t *src = reinterpret_cast<const uint16_t *>(p.A[s0 + sl]) +
                                (int64_t)slot * p.a_stride[s0 + sl] + (kt + k) * R + j0;
          u32x4 w = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] = (uint16_t)(w[i] & 0xffffu);
            v[2 * i + 1] = (uint16_t)(w[i] >> 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = 0;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int n = n0 + i;
          lds.mma.at[n][k ^ (((n >> 3) & 7) << 3)] = v[i];
        }
      }
      // x fragments: lane (mrow, g) holds x[trow][kt + 32g + 8c + e], c = 0..3
      bf16x8 xf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kk = 32 * g + 8 * c;
        if (trow >= 0 && kk < klen) {
          xf[c] = *reinterpret_cast<const bf16x8 *>(x + trow * p.ldx + kt + kk);
        } else {
          xf[c] = bf16x8{};
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kk = 32 * g + 8 * c;
#pragma unroll
        for (int b = 0; b < kMmaCols / 16; ++b) {
          if (b < nblk) {
            const int n = 16 * b + mrow;
            const bf16x8 bv =
                *reinterpret_cast<const bf16x8 *>(&lds.mma.at[n][kk ^ (((n >> 3) & 7) << 3)]);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[c], bv, acc[b], 0, 0, 0);
          }
        }
      }
    }
    // epilogue: acc[b][v] = C[16*wave + 4*g + v][16*b + mrow]
#pragma unroll
    for (int b = 0; b < kMmaCols / 16; ++b) {
      if (b < nblk) {
        const int n = 16 * b + mrow;
        const int s = s0 + n / R, j = n % R;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r_ = 16 * wave + 4 * g + v;
          if (r_ < rows) put(p, R, s, pos0 + r_, j, kc, acc[b][v] * sc);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ the kernels

template <typename E, int R>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
  __shared__ ShrinkLds lds;
  build_plan(p, lds.plan);
  const int nseg_first = (p.meta.info[0] > 0 && p.meta.seg_slot[0] == -1) ? 1 : 0;
  for (int item = blockIdx.x; item < lds.plan.total_items; item += gridDim.x) {
    __syncthreads();  // the previous item's LDS reads are done before this item writes
    const int si = find_segment(lds.plan, item);
    const int seg = nseg_first + si;
    const int count = p.meta.seg_count[seg];
    const int slot = p.meta.seg_slot[seg];
    const int local = item - (si > 0 ? lds.plan.item_end[si - 1] : 0);
    const int chunk = local / p.kch, kc = local % p.kch;
    const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
    if constexpr (sizeof(E) == 2 && R >= 16) {
      if (seg_takes_mma(p, count)) {
        const int64_t pos0 = (int64_t)p.meta.seg_start[seg] + (int64_t)chunk * kMmaRows;
        mma_item<R>(p, lds, slot, pos0, min(kMmaRows, count - chunk * kMmaRows), kc, sc);
        continue;
      }
    }
    const int64_t pos0 = (int64_t)p.meta.seg_start[seg] + (int64_t)chunk * kVecRows;
    vec_item<E, R>(p, lds, slot, pos0, min(kVecRows, count - chunk * kVecRows), kc, sc);
  }
}

// u[s][sorted[pos]][:] = sum over k-chunks, in order, of the partial sums at pos,
// for every sorted position of a token with an adapter.
__global__ __launch_bounds__(256) void shrink_reduce_kernel(MetaView meta, const float *partial,
                                                            float *u, int32_t n_slices, int32_t R,
                                                            int32_t kch) {
  const int64_t T = meta.T;
  const int64_t begin = meta.info[3];
  const int64_t q_per_row = R / 4;
  const int64_t total = (T - begin) * n_slices * q_per_row;
  const int64_t plane = (int64_t)n_slices * T * R;
  for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t q = idx % q_per_row;
    const int64_t rest = idx / q_per_row;
    const int64_t pos = begin + rest % (T - begin);
    const int64_t s = rest / (T - begin);
    const float *src = partial + (s * T + pos) * R + 4 * q;
    f32x4 v = *reinterpret_cast<const f32x4 *>(src);
    for (int kc = 1; kc < kch; ++kc) {
      const f32x4 w = *reinterpret_cast<const f32x4 *>(src + kc * plane);
      v[0] += w[0];
      v[1] += w[1];
      v[2] += w[2];
      v[3] += w[3];
    }
    const int64_t t = meta.sorted[pos];
    *reinterpret_cast<f32x4 *>(u + (s * T + t) * R + 4 * q) = v;
  }
}

// ------------------------------------------------------------------ host side

// Chunking chosen from host-known sizes only (no device read), so a call
// never synchronises: split d_in so that there are about 512 items.
ShrinkConfig plan_shrink(int64_t T, int32_t S, int64_t d_in, int32_t R, bool bf16, int mode) {
  ShrinkConfig c{};
  c.use_mma_mode = (!bf16 || R < 16) ? 0 : (mode == 1 ? 0 : (mode == 2 ? 2 : 1));
  c.mfma_min = shrink_mma_min_default();
  const int64_t rows = c.use_mma_mode ? kMmaRows : kVecRows;
  const int64_t chunks = (T + rows - 1) / rows + S;
  const int64_t tiles = (d_in + kMmaKT - 1) / kMmaKT;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(tiles, (512 + chunks - 1) / chunks));
  c.kc = (int)(((tiles + want - 1) / want) * kMmaKT);
  c.kch = (int)((d_in + c.kc - 1) / c.kc);
  const int64_t bound = ((T + kVecRows - 1) / kVecRows + S) * c.kch;
  c.grid = (int)std::max<int64_t>(1, std::min<int64_t>(bound, 2048));
  return c;
}

size_t shrink_ws_bytes(const ShrinkConfig &c, int64_t T, int32_t n_slices, int32_t R) {
  const size_t part = c.kch > 1 ? (size_t)c.kch * n_slices * T * R * sizeof(float) : 0;
  return (part + 255) / 256 * 256;
}

template <typename E, int R>
static hipError_t launch_t(const ShrinkParams &p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((shrink_kernel<E, R>), dim3(grid), dim3(kShrinkThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_shrink(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                         int32_t n_slices, const void *const *A, const int64_t *a_stride,
                         int32_t R, float scale, const float *slot_scale, float *u, int mode,
                         void *ws, hipStream_t stream) {
  const ShrinkConfig c = plan_shrink(meta.T, meta.S, d_in, R, bf16, mode);
  ShrinkParams p{};
  p.meta = meta;
  p.x = x;
  p.ldx = ldx;
  p.d_in = d_in;
  for (int s = 0; s < n_slices; ++s) {
    p.A[s] = A[s];
    p.a_stride[s] = a_stride[s];
  }
  p.n_slices = n_slices;
  p.scale = scale;
  p.slot_scale = slot_scale;
  p.out = c.kch == 1 ? u : reinterpret_cast<float *>(ws);
  p.use_mma_mode = c.use_mma_mode;
  p.mfma_min = c.mfma_min;
  p.kc = c.kc;
  p.kch = c.kch;
  if (meta.T == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  switch (R) {
    case 8: e = bf16 ? launch_t<uint16_t, 8>(p, c.grid, stream) : launch_t<float, 8>(p, c.grid, stream); break;
    case 16: e = bf16 ? launch_t<uint16_t, 16>(p, c.grid, stream) : launch_t<float, 16>(p, c.grid, stream); break;
    case 32: e = bf16 ? launch_t<uint16_t, 32>(p, c.grid, stream) : launch_t<float, 32>(p, c.grid, stream); break;
    case 64: e = bf16 ? launch_t<uint16_t, 64>(p, c.grid, stream) : launch_t<float, 64>(p, c.grid, stream); break;
  }
  if (e != hipSuccess || c.kch == 1) return e;
  const int64_t work = meta.T * n_slices * (R / 4);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 1024));
  hipLaunchKernelGGL(shrink_reduce_kernel, dim3(grid), dim3(256), 0, stream, meta,
                     reinterpret_cast<const float *>(ws), u, n_slices, R, c.kch);
  return hipGetLastError();
}

}  // namespace lora
