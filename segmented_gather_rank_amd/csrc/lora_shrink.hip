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
// One kernel, a grid-stride loop over work items; every item issues the loads
// that do not depend on each other before it waits for any of them.  Every segment with an adapter
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
//    (128 k x n_slices*r) is stored row-major in LDS with 16-byte writes and
//    read back as MFMA operands with the gfx950 transposing LDS read; rows are
//    padded so the 4 rows of a read group fall in distinct banks; the next
//    tile's loads are in flight while one tile is multiplied; x fragments go
//    straight from global memory to registers.
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
constexpr int kMmaKT = 128;        // k per A tile on the matrix-core path
constexpr int kMmaCols = 128;      // n_slices*r columns per pass (8 MFMA blocks)
constexpr int kAlStride = kMmaCols + 16;  // bf16 elements per LDS row of the A tile
constexpr int kMmaOct = kMmaKT * kMmaCols / 8 / kShrinkThreads;  // A octets per thread per tile

struct ShrinkParams {
  MetaView meta;
  const void *x;
  int64_t ldx, d_in;
  const void *A[kMaxSlices];
  int64_t a_stride[kMaxSlices];
  int32_t n_slices;
  float scale;
  const float *slot_scale;
  // kch == 1: out is u [n_slices][T][R], rows in token order, or in sorted-
  // position order when u_sorted is set; kch > 1: out holds the partial sums
  // [kch][n_slices][T][R] in sorted-position order
  float *out;
  int32_t u_sorted;
  int32_t use_mma_mode;  // 0 = never, 1 = by segment length, 2 = always
  int32_t mfma_min;
  int32_t kc, kch;       // k-chunk length (a multiple of 128) and count
};

struct ShrinkLds {
  union {
    struct {
      float xs[kVecRows][kVecSub];
      float red[4][kVecRows][64];
    } vec;
    struct {
      uint16_t al[kMmaKT * kAlStride];  // A tile, row k, column slice*R + j
    } mma;
  };
};

__device__ __forceinline__ bool seg_takes_mma(const ShrinkParams &p, int count) {
  return p.use_mma_mode == 2 || (p.use_mma_mode == 1 && count >= p.mfma_min);
}

// Store one result: into u (token or sorted order) when d_in is not split,
// else into the partial sums of k-chunk kc.
__device__ __forceinline__ void put(const ShrinkParams &p, int R, int s, int64_t pos, int j,
                                   int kc, float v) {
  const int64_t T = p.meta.T;
  if (p.kch == 1) {
    const int64_t row = p.u_sorted ? pos : (int64_t)p.meta.sorted[pos];
    p.out[((int64_t)s * T + row) * R + j] = v;
  } else {
    p.out[(((int64_t)kc * p.n_slices + s) * T + pos) * R + j] = v;
  }
}

// ------------------------------------------------------------------ vector path

template <typename E, int R>
__device__ __forceinline__ void vec_item(const ShrinkParams &p, ShrinkLds &lds, int slot, int64_t pos0,
                         int rows, int kc, float sc) {
  constexpr int JO = R / 8;                       // rank octets per k row
  constexpr int VA = sizeof(E) == 2 ? 8 : 4;      // A loads in flight per thread
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
      const int nel = slen * R;
      const E *Ab = reinterpret_cast<const E *>(pick(p.A, s)) + (int64_t)slot * pick(p.a_stride, s) +
                    (k0 + sub) * R;
      // the first A batch goes out before the x rows are staged
      Raw8<E> a[VA];
#pragma unroll
      for (int q = 0; q < VA; ++q) {
        const int e = 8 * (tid + kShrinkThreads * q);
        if (e < nel) a[q].load(Ab + e);
      }
      if (staged != sub) {
        __syncthreads();  // earlier readers of xs are done
        const int oct = slen / 8;
        for (int idx = tid; idx < rows * oct; idx += kShrinkThreads) {
          const int row = idx / oct, c = idx - row * oct;
          const int64_t t = p.meta.sorted[pos0 + row];
          float v[8];
          load8(x + t * p.ldx + k0 + sub + 8 * c, v);
          *reinterpret_cast<f32x4 *>(&lds.vec.xs[row][8 * c]) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4 *>(&lds.vec.xs[row][8 * c + 4]) = f32x4{v[4], v[5], v[6], v[7]};
        }
        __syncthreads();
        staged = sub;
      }
      for (int base = 0; base < nel; base += 8 * kShrinkThreads * VA) {
        if (base > 0) {
#pragma unroll
          for (int q = 0; q < VA; ++q) {
            const int e = base + 8 * (tid + kShrinkThreads * q);
            if (e < nel) a[q].load(Ab + e);
          }
        }
#pragma unroll
        for (int q = 0; q < VA; ++q) {
          const int e = base + 8 * (tid + kShrinkThreads * q);
          if (e < nel) {
            const int k = e / R;
#pragma unroll
            for (int m = 0; m < kVecRows; ++m) {
              const float xv = lds.vec.xs[m][k];  // rows >= `rows` are stale, never stored
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[m][i] = fmaf(xv, a[q][i], acc[m][i]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < kVecRows; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[m][i] = wave_sum_mod<JO>(acc[m][i]);
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

// One A tile (kMmaKT k rows x ns*R columns) and this lane's x fragments, held
// in registers between their load and their use.
struct MmaTile {
  u32x4 a[kMmaOct];
  bf16x8 xf[4];
};

template <int R>
__device__ __forceinline__ void mma_load_tile(const ShrinkParams &p, MmaTile &tl, int slot, int s0,
                                              int ns, int64_t kt, int klen, int64_t trow, int g) {
  const int tid = threadIdx.x;
  const int per_slice = kMmaKT * R / 8;
#pragma unroll
  for (int q = 0; q < kMmaOct; ++q) {
    const int idx = tid + kShrinkThreads * q;
    const int sl = idx / per_slice;
    const int e = 8 * (idx - sl * per_slice);
    const int k = e / R, j0 = e % R;
    if (sl < ns && k < klen) {
      tl.a[q] = *reinterpret_cast<const u32x4 *>(
          reinterpret_cast<const uint16_t *>(pick(p.A, s0 + sl)) + (int64_t)slot * pick(p.a_stride, s0 + sl) +
          (kt + k) * R + j0);
    } else {
      tl.a[q] = u32x4{0, 0, 0, 0};
    }
  }
  const uint16_t *x = reinterpret_cast<const uint16_t *>(p.x);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kk = 32 * g + 8 * c;
    if (trow >= 0 && kk < klen) {
      tl.xf[c] = *reinterpret_cast<const bf16x8 *>(x + trow * p.ldx + kt + kk);
    } else {
      tl.xf[c] = bf16x8{};
    }
  }
}

// Row-major store of a tile's A octets (16-byte LDS writes).
template <int R>
__device__ __forceinline__ void mma_store_al(ShrinkLds &lds, const MmaTile &tl, int ns) {
  const int tid = threadIdx.x;
  const int per_slice = kMmaKT * R / 8;
#pragma unroll
  for (int q = 0; q < kMmaOct; ++q) {
    const int idx = tid + kShrinkThreads * q;
    const int sl = idx / per_slice;
    if (sl < ns) {
      const int e = 8 * (idx - sl * per_slice);
      *reinterpret_cast<u32x4 *>(&lds.mma.al[(e / R) * kAlStride + sl * R + e % R]) = tl.a[q];
    }
  }
}

template <int R>
__device__ __forceinline__ void mma_item(const ShrinkParams &p, ShrinkLds &lds, int slot, int64_t pos0,
                         int rows, int kc, float sc) {
  constexpr int SG = kMmaCols / R;  // slices per pass
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int64_t kbeg = (int64_t)kc * p.kc;
  const int64_t kend = min(p.d_in, kbeg + p.kc);
  const int mrow = lane % 16, g = lane / 16;
  const int row = 16 * wave + mrow;               // this lane's operand row
  const int64_t trow = row < rows ? (int64_t)p.meta.sorted[pos0 + row] : -1;

  for (int s0 = 0; s0 < p.n_slices; s0 += SG) {
    const int ns = min(SG, p.n_slices - s0);
    const int nblk = ns * R / 16;
    f32x4 acc[kMmaCols / 16];
#pragma unroll
    for (int b = 0; b < kMmaCols / 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // software pipeline: the next tile's loads are in flight while this one
    // is multiplied
    MmaTile tl;
    mma_load_tile<R>(p, tl, slot, s0, ns, kbeg, (int)min((int64_t)kMmaKT, kend - kbeg), trow, g);
    for (int64_t kt = kbeg; kt < kend; kt += kMmaKT) {
      __syncthreads();  // the previous tile's LDS reads are done
      mma_store_al<R>(lds, tl, ns);
      bf16x8 xf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) xf[c] = tl.xf[c];
      const int64_t kn = kt + kMmaKT;
      if (kn < kend) mma_load_tile<R>(p, tl, slot, s0, ns, kn, (int)min((int64_t)kMmaKT, kend - kn), trow, g);
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kk = 32 * g + 8 * c;
#pragma unroll
        for (int b = 0; b < kMmaCols / 16; ++b) {
          if (b < nblk) {
            const bf16x8 bv = lds_col8(lds.mma.al, kAlStride, kk, 16 * b);
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
  extern __shared__ __align__(16) unsigned char shrink_dyn[];
  const SegTable tb = seg_table_at(shrink_dyn, p.meta.S);
  build_items(p.meta, tb, true, [&](int c, int) {
    const int mc = seg_takes_mma(p, c) ? kMmaRows : kVecRows;
    return ((c + mc - 1) / mc) * p.kch;
  });
  const int first = tb.scal[1];
  for (int item = blockIdx.x; item < tb.scal[2]; item += gridDim.x) {
    __syncthreads();  // the previous item's LDS reads are done before this item writes
    const int si = find_item_segment(tb, item);
    const int seg = first + si;
    const int count = tb.count[seg];
    const int slot = tb.slot[seg];
    const int local = item - (si > 0 ? tb.item_end[si - 1] : 0);
    const int chunk = local / p.kch, kc = local % p.kch;
    const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
    if constexpr (sizeof(E) == 2 && R >= 16) {
      if (seg_takes_mma(p, count)) {
        const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kMmaRows;
        mma_item<R>(p, lds, slot, pos0, min(kMmaRows, count - chunk * kMmaRows), kc, sc);
        continue;
      }
    }
    const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kVecRows;
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
  hipLaunchKernelGGL((shrink_kernel<E, R>), dim3(grid), dim3(kShrinkThreads),
                     seg_table_bytes(p.meta.S), stream, p);
  return hipGetLastError();
}

hipError_t launch_shrink(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                         int32_t n_slices, const void *const *A, const int64_t *a_stride,
                         int32_t R, float scale, const float *slot_scale, float *u, int mode,
                         void *ws, bool for_apply, int *kch_out, hipStream_t stream) {
  const ShrinkConfig c = plan_shrink(meta.T, meta.S, d_in, R, bf16, mode);
  if (kch_out) *kch_out = c.kch;
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
  p.u_sorted = for_apply ? 1 : 0;
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
  // lora_apply's expand reads the partial sums itself; lora_shrink must hand
  // back a finished u
  if (e != hipSuccess || c.kch == 1 || for_apply) return e;
  const int64_t work = meta.T * n_slices * (R / 4);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 1024));
  hipLaunchKernelGGL(shrink_reduce_kernel, dim3(grid), dim3(256), 0, stream, meta,
                     reinterpret_cast<const float *>(ws), u, n_slices, R, c.kch);
  return hipGetLastError();
}

}  // namespace lora
