// lora_bgmv.hip -- the BGMV form fused into one kernel, for decode-shaped
// batches: y[t][window_s] (+)= (scale_a * x[t] . A_s[a]) . B_s[a], a = slot(t).
//
// Page "多 LoRA 服务：分段矩阵乘与适配器调度", section "不合并权重，批量计算":
// BGMV lets every token fetch its own adapter's A and B and do a small
// matrix-vector product, which suits decode; the real kernels fuse the fetch
// with the product, shrink first and expand straight into the base output.
// Page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩 GEMM:shrink、expand
// 与 fp32 中转缓冲": the rank-r intermediate is kept in fp32 and the result is
// rounded once when it is added into the output window of each packed slice.
//
// One workgroup per token.  The rank-r vector never leaves LDS, so the whole
// delta of a token is one workgroup's work: no partial sums, no second kernel,
// no workgroup waits for another.  Tokens are taken in slot-sorted order, and
// the sorted list is cut into 8 contiguous runs, run k going to the workgroups
// that the dispatcher places on XCD k (blockIdx mod 8): the tokens of a slot
// are handled inside one XCD, whose L2 then serves that slot's A and B to all
// of them after the first read from HBM.
//
//  * shrink: x row staged in LDS; each thread loads 16 contiguous bytes of A
//    (one rank octet of one k row) per pass, many passes in flight, and
//    accumulates 8 ranks; the contraction over k finishes in registers (DPP
//    row rotations, permlane16/32 swaps) and in a fixed-order sum over the 4
//    waves;
//  * expand: each thread owns 8-column octets of the output windows; the y
//    octets are read at the start (they do not depend on the shrink); B rows
//    are read with 16-byte loads; the delta is summed on its own in fp32 and
//    added to y once.
#include "lora_host.h"

namespace lora {

constexpr int kBThreads = 1024;  // 16 waves: enough loads in flight for one token's factors
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBMaxLds = 32768;  // bytes of the staged x row
constexpr int kBMaxOct = 1024;   // output octets (sum of slice widths / 8)
// loads per thread per batch: 16 bytes each for bf16, 32 for fp32
template <typename E> constexpr int kBNA = sizeof(E) == 2 ? 8 : 4;
template <typename E> constexpr int kBNB = sizeof(E) == 2 ? 8 : 4;

struct BgmvParams {
  MetaView meta;
  const void *x;
  int64_t ldx, d_in;
  const void *A[kMaxSlices];
  int64_t a_stride[kMaxSlices];
  const void *B[kMaxSlices];
  int64_t b_stride[kMaxSlices];
  int64_t width[kMaxSlices];
  int64_t offset[kMaxSlices];
  int32_t oct_base[kMaxSlices + 1];  // prefix of output octets per slice
  int32_t n_slices;
  int32_t jg;                        // threads sharing one output octet (rank split)
  float scale;
  const float *slot_scale;
  void *y;
  int64_t ldy;
  int32_t add;
};

// Sum over aligned groups of `jg` adjacent lanes (jg in 1..16, a power of 2).
__device__ __forceinline__ float group_sum(float v, int jg) {
  if (jg >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  if (jg >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  if (jg >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if (jg >= 16) v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ int slice_of_oct(const BgmvParams &p, int o) {
  return last_le(p.oct_base, p.n_slices, o);
}

template <typename E, int R>
__global__ __launch_bounds__(kBThreads) void bgmv_fused_kernel(BgmvParams p) {
  constexpr int JO = R / 8;
  extern __shared__ __align__(16) unsigned char bgmv_lds[];
  E *xs = reinterpret_cast<E *>(bgmv_lds);
  constexpr int NA = kBNA<E>, NB = kBNB<E>;
  __shared__ float red[kBWaves][R];
  __shared__ float us[kMaxSlices][R];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t T = p.meta.T;
  // positions handled: [first, T); the no-adapter tokens lead the sorted
  // order and only need work when the windows are stored, not added
  const int64_t first = p.add ? p.meta.info[3] : 0;
  const int64_t run = (T - first + 7) / 8;
  const int64_t local = blockIdx.x / 8;
  if (local >= run) return;
  const int64_t pos = first + (int64_t)(blockIdx.x % 8) * run + local;
  if (pos >= T) return;
  const int64_t t = p.meta.sorted[pos];
  const int slot = p.meta.sorted_slot[pos];
  const int n_oct = pick(p.oct_base, p.n_slices);
  E *y = reinterpret_cast<E *>(p.y) + t * p.ldy;

  if (slot < 0) {  // store mode, no adapter: the windows become 0
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int o = tid; o < n_oct; o += kBThreads) {
      const int s = slice_of_oct(p, o);
      store8(y + pick(p.offset, s) + 8 * (o - pick(p.oct_base, s)), z);
    }
    return;
  }

  // ---- issue every independent load first: A (first batch of slice 0), B
  // (first batch), y, then x; one memory round trip covers them all
  const int64_t nel = p.d_in * R;  // A elements per slice
  const E *A0 = reinterpret_cast<const E *>(p.A[0]) + (int64_t)slot * p.a_stride[0];
  Raw8<E> a[NA];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int64_t e = 8 * ((int64_t)tid + (int64_t)kBThreads * q);
    if (e < nel) a[q].load(A0 + e);
  }
  // expand mapping: thread -> (octet o = tid / jg + (kBThreads / jg) * i, rank group g)
  const int jg = p.jg, g = tid % jg, rj = R / jg;
  const int o0 = tid / jg, ostep = kBThreads / jg;
  int s0 = 0;
  int64_t n00 = 0;
  const E *Bb0 = nullptr;
  Raw8<E> b[NB];
  if (o0 < n_oct) {
    s0 = slice_of_oct(p, o0);
    n00 = 8 * (int64_t)(o0 - pick(p.oct_base, s0));
    Bb0 = reinterpret_cast<const E *>(pick(p.B, s0)) + (int64_t)slot * pick(p.b_stride, s0) + n00;
#pragma unroll
    for (int jj = 0; jj < NB; ++jj)
      if (jj < rj) b[jj].load(Bb0 + (int64_t)(g * rj + jj) * pick(p.width, s0));
  }
  float yv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (o0 < n_oct && g == 0 && p.add) load8(y + pick(p.offset, s0) + n00, yv);
  const E *xr = reinterpret_cast<const E *>(p.x) + t * p.ldx;
  for (int o = tid; o < p.d_in / 8; o += kBThreads) {
    Raw8<E> v;
    v.load(xr + 8 * o);
    if constexpr (sizeof(E) == 2) {
      *reinterpret_cast<u32x4 *>(xs + 8 * o) = v.w;
    } else {
      *reinterpret_cast<f32x4 *>(xs + 8 * o) = v.a;
      *reinterpret_cast<f32x4 *>(xs + 8 * o + 4) = v.b;
    }
  }
  __syncthreads();

  // ---- shrink: thread owns rank octet jo of k rows (8 tid + 8192 q) / R
  const int jo = tid % JO;
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  for (int s = 0; s < p.n_slices; ++s) {
    const E *As = reinterpret_cast<const E *>(pick(p.A, s)) + (int64_t)slot * pick(p.a_stride, s);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t base = 0; base < nel; base += (int64_t)8 * kBThreads * NA) {
      if (s > 0 || base > 0) {
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          const int64_t e = base + 8 * ((int64_t)tid + (int64_t)kBThreads * q);
          if (e < nel) a[q].load(As + e);
        }
      }
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        const int64_t e = base + 8 * ((int64_t)tid + (int64_t)kBThreads * q);
        if (e < nel) {
          const int k = (int)(e / R);
          float xv;
          if constexpr (sizeof(E) == 2) {
            xv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(xs)[k] << 16);
          } else {
            xv = reinterpret_cast<const float *>(xs)[k];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(xv, a[q][i], acc[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = wave_sum_mod<JO>(acc[i]);
    if (lane < JO) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][8 * jo + i] = acc[i];
    }
    __syncthreads();
    if (tid < R) {  // fixed-order sum over the waves
      float v = 0.f;
      for (int w = 0; w < kBWaves; ++w) v += red[w][tid];
      us[s][tid] = sc * v;
    }
    __syncthreads();
  }

  // ---- expand: thread group (jg lanes) owns an 8-column octet; lane g takes
  // rank rows [g * rj, (g + 1) * rj); the group sum lands in lane g == 0
  for (int o = o0, it = 0; o < n_oct; o += ostep, ++it) {
    int s = s0;
    int64_t n0 = n00;
    const E *Bb = Bb0;
    if (it > 0) {
      s = slice_of_oct(p, o);
      n0 = 8 * (int64_t)(o - pick(p.oct_base, s));
      Bb = reinterpret_cast<const E *>(pick(p.B, s)) + (int64_t)slot * pick(p.b_stride, s) + n0;
      if (g == 0 && p.add) load8(y + pick(p.offset, s) + n0, yv);
    }
    const int64_t w = pick(p.width, s);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int jb = 0; jb < rj; jb += NB) {
      if (it > 0 || jb > 0) {
#pragma unroll
        for (int jj = 0; jj < NB; ++jj)
          if (jb + jj < rj) b[jj].load(Bb + (int64_t)(g * rj + jb + jj) * w);
      }
#pragma unroll
      for (int jj = 0; jj < NB; ++jj) {
        if (jb + jj < rj) {
          const float uv = us[s][g * rj + jb + jj];
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[c] = fmaf(uv, b[jj][c], acc[c]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = group_sum(acc[c], jg);
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) yv[c] += acc[c];
      store8(y + pick(p.offset, s) + n0, yv);
    }
  }
}

// ------------------------------------------------------------------ host side

bool bgmv_fits(int64_t T, int32_t S, int64_t d_in, int32_t n_slices, const int64_t *width, int32_t R,
               bool bf16, int mode) {
  if (mode == 2) return false;  // SGMV requested
  const int64_t e = bf16 ? 2 : 4;
  int64_t sw = 0;
  for (int s = 0; s < n_slices; ++s) sw += width[s];
  const int64_t w_tok = ((int64_t)n_slices * d_in + sw) * R * e;  // weight bytes per token
  if (sw / 8 > kBMaxOct || d_in * e > kBMaxLds || w_tok > (1 << 20)) return false;
  return mode == 1 || T <= 16 * (int64_t)S;  // BGMV requested, or few tokens per slot
}

template <typename E, int R>
static hipError_t launch_t(const BgmvParams &p, int grid, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((bgmv_fused_kernel<E, R>), dim3(grid), dim3(kBThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_bgmv(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                       int32_t n_slices, const void *const *A, const int64_t *a_stride,
                       const void *const *B, const int64_t *b_stride, const int64_t *width,
                       const int64_t *offset, int32_t R, float scale, const float *slot_scale,
                       void *y, int64_t ldy, int add, hipStream_t stream) {
  BgmvParams p{};
  p.meta = meta;
  p.x = x;
  p.ldx = ldx;
  p.d_in = d_in;
  p.oct_base[0] = 0;
  for (int s = 0; s < n_slices; ++s) {
    p.A[s] = A[s];
    p.a_stride[s] = a_stride[s];
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
    p.oct_base[s + 1] = p.oct_base[s] + (int32_t)(width[s] / 8);
  }
  p.n_slices = n_slices;
  // split the rank over jg adjacent lanes when there are fewer octets than threads
  const int n_oct = p.oct_base[n_slices];
  int jg = 1;
  while (jg < 16 && jg < R && (int64_t)n_oct * jg * 2 <= kBThreads) jg *= 2;
  p.jg = jg;
  p.scale = scale;
  p.slot_scale = slot_scale;
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  if (meta.T == 0) return hipSuccess;
  const int grid = (int)(8 * ((meta.T + 7) / 8));
  const size_t lds = (size_t)d_in * (bf16 ? 2 : 4);
  switch (R) {
    case 8: return bf16 ? launch_t<uint16_t, 8>(p, grid, lds, stream) : launch_t<float, 8>(p, grid, lds, stream);
    case 16: return bf16 ? launch_t<uint16_t, 16>(p, grid, lds, stream) : launch_t<float, 16>(p, grid, lds, stream);
    case 32: return bf16 ? launch_t<uint16_t, 32>(p, grid, lds, stream) : launch_t<float, 32>(p, grid, lds, stream);
    case 64: return bf16 ? launch_t<uint16_t, 64>(p, grid, lds, stream) : launch_t<float, 64>(p, grid, lds, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
