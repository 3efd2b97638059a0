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
// Loads are issued in the order they are consumed (x row, A, B, y) before the
// first wait, so the shrink starts while A and B are still arriving.
//
//  * shrink: thread (row rr, rank octet jo) loads 16-byte rank octets of A
//    rows rr, rr + RB, rr + 2 RB, ... (RB = rows covered by one load across the
//    workgroup), so every load instruction reads contiguous memory.  bf16:
//    rows k and k + RB are paired, the x row is staged in LDS as matching
//    (x[k], x[k + RB]) pairs, and one v_dot2_f32_bf16 does two multiply-adds
//    per rank (a byte permute builds the A pair); fp32 uses plain FMAs.  The
//    contraction over k finishes with DPP row rotations, permlane16/32 swaps
//    and a fixed-order sum over the 16 waves.
//  * expand: jg adjacent lanes own an 8-column octet of an output window and
//    split its rank rows; bf16 pairs rank rows j, j + 1 the same way, with u
//    split into bf16 high and low parts (u ~ hi + lo to about 16 bits) so the
//    rank-r vector keeps fp32-level precision; the delta is summed on its own
//    in fp32 and added to y once.
#include "lora_host.h"

namespace lora {

constexpr int kBThreads = 1024;  // 16 waves: enough loads in flight for one token's factors
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBMaxX = 32768;    // bytes of one x row
constexpr int kBMaxOct = 1024;   // output octets (sum of slice widths / 8)
// A / B rank octets per thread per batch (16 bytes each for bf16, 32 for fp32)
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
  int32_t n_inst;                    // A load instructions per slice, rounded up to the batch
  int32_t x_tasks;                   // x staging tasks (<= 2 per thread)
  float scale;
  const float *slot_scale;
  const int32_t *slot_rank;  // per-slot ranks, or null (every slot uses R)
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

template <int NS>
__device__ __forceinline__ int slice_of_oct(const BgmvParams &p, int o) {
  return last_le<NS>(p.oct_base, p.n_slices, o);
}

// One rank octet of A (8 consecutive ranks of one k row) as raw words.
template <typename E> struct AOct;
template <> struct AOct<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) { w = buf_load16(r, off); }
};
template <> struct AOct<float> {
  u32x4 a, b;
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off) {
    a = buf_load16(r, off);
    b = buf_load16(r, off + 16);
  }
  __device__ __forceinline__ float operator[](int i) const {
    return __uint_as_float(i < 4 ? a[i] : b[i - 4]);
  }
};

// RK: per-slot ranks are given (a separate instantiation, so that the common
// case carries none of the extra registers).
// The sorted order and T come first among the arguments, so that they are
// preloaded into scalar registers and the first loads need no argument fetch.
// ONE: one slice, one batch of A loads per thread, at most one output octet
// per lane group and one batch of B rows (the common decode shape): the code
// for the next batches is left out.
template <typename E, int R, bool RK, int NS, bool ONE>
__global__ __launch_bounds__(kBThreads) void bgmv_fused_kernel(const int32_t *__restrict__ sorted,
                                                               const int32_t *__restrict__ sorted_slot,
                                                               int64_t T, BgmvParams p) {
  constexpr bool kBf16 = sizeof(E) == 2;
  constexpr int JO = R / 8;             // rank octets per A row
  constexpr int RB = kBThreads / JO;    // A rows covered by one load across the workgroup
  constexpr int NA = kBNA<E>, NB = kBNB<E>;
  // x row: bf16 -> (x[k], x[k + RB]) pair words, fp32 -> values; zero-padded
  extern __shared__ __align__(16) unsigned char bgmv_lds[];
  __shared__ float red[kBWaves][R];
  __shared__ float us[NS][R];
  __shared__ uint32_t uh[NS][R / 2], ul[NS][R / 2];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t run = (T + 7) / 8;
  const int64_t local = blockIdx.x / 8;
  if (local >= run) return;
  const int64_t pos = (int64_t)(blockIdx.x % 8) * run + local;
  if (pos >= T) return;
  // both metadata loads go out before either is waited for
  const int slot = __builtin_amdgcn_readfirstlane(sorted_slot[pos]);
  const int64_t t = __builtin_amdgcn_readfirstlane(sorted[pos]);
  // ranks this slot's adapter really has (rank 0: nothing to add)
  const int rk = slot < 0 ? 0 : (RK ? slot_rank_of(p.slot_rank, slot, R) : R);
  if ((rk == 0 && p.add) || t < 0) return;  // no adapter, add mode: nothing to do
  const int n_oct = pick<NS + 1>(p.oct_base, p.n_slices);
  E *y = reinterpret_cast<E *>(p.y) + t * p.ldy;

  if (rk == 0) {  // store mode, no adapter: the windows become 0
    const float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int o = tid; o < n_oct; o += kBThreads) {
      const int s = slice_of_oct<NS>(p, o);
      store8(y + pick<NS>(p.offset, s) + 8 * (o - pick<NS + 1>(p.oct_base, s)), z);
    }
    return;
  }

  // ---- addresses first, then every load of the first batch, in the order the
  // loads are consumed: x, A, B, y.  None of them sits behind a branch, so the
  // compiler's waits count exactly the loads issued after the one a use needs.
  const int rr = tid / JO, jo = tid % JO;
  const uint32_t a_bytes = (uint32_t)(p.d_in * R * sizeof(E));
  // expand mapping: thread -> (octet o = tid / jg + (kBThreads / jg) * i, rank group g)
  const int jg = p.jg, g = tid % jg, rj = R / jg;
  const int span = rj < NB ? rj : NB;  // rank rows per batch (even)
  const int o0 = tid / jg, ostep = kBThreads / jg;
  // threads without an octet read octet 0's rows and drop them
  const int oc = o0 < n_oct ? o0 : 0;
  const int s0 = slice_of_oct<NS>(p, oc);
  const int64_t n00 = 8 * (int64_t)(oc - pick<NS + 1>(p.oct_base, s0, p.n_slices));
  const E *Bb0 = reinterpret_cast<const E *>(pick<NS>(p.B, s0, p.n_slices)) +
                 (int64_t)slot * pick<NS>(p.b_stride, s0, p.n_slices) + n00;  // rank row 0 of the octet
  const int64_t w0 = pick<NS>(p.width, s0, p.n_slices);
  const int64_t yoff0 = pick<NS>(p.offset, s0, p.n_slices) + n00;
  const rsrc_t xr = make_rsrc(reinterpret_cast<const E *>(p.x) + x_row_of(p.meta, t) * p.ldx,
                              (uint32_t)(p.d_in * sizeof(E)));
  const rsrc_t ar0 = make_rsrc(reinterpret_cast<const E *>(p.A[0]) + (int64_t)slot * p.a_stride[0], a_bytes);
  const rsrc_t yr = make_rsrc(y, (uint32_t)(p.ldy * sizeof(E)));
  const bool a_live = !RK || 8 * jo < rk;  // this lane's A rank octet is within the slot's rank
  const bool ymine = o0 < n_oct && g == 0 && p.add;
  const uint32_t yoff_b = ymine ? (uint32_t)(yoff0 * sizeof(E)) : 0x7FFFFFF0u;  // past the row: zeros

  u32x4 xv[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // tasks past x_tasks read past the row (zeros) and are not stored
    const int task = tid + kBThreads * u;
    if constexpr (kBf16) {  // words [pp * RB + i0, + 8): rows 2 pp RB + i0 and that + RB
      const int pp = task / (RB / 8), i0 = 8 * (task % (RB / 8));
      const uint32_t k = (uint32_t)(2 * pp * RB + i0);
      xv[u][0] = buf_load16(xr, 2 * k);
      xv[u][1] = buf_load16(xr, 2 * (k + RB));
    } else {                // values [8 task, + 8)
      xv[u][0] = buf_load16(xr, 32 * task);
      xv[u][1] = buf_load16(xr, 32 * task + 16);
    }
  }
  // a[q] holds load instruction q of its batch: k row q * RB + rr, rank octet
  // jo; q pairs (2m, 2m + 1) are the k rows paired by one dot2
  AOct<E> a[NA];
#pragma unroll
  for (int q = 0; q < NA; ++q)
    a[q].load(ar0, a_live ? (uint32_t)(((q * RB + rr) * R + 8 * jo) * sizeof(E)) : 0x7FFFFFF0u);
  // b[jj] holds rank row jj of the batch (jj < span; later ones repeat the last)
  Raw8<E> b[NB];
  // rank row g * rj + jj; rows at or past the slot's rank are not read: row 0
  // (live, and read by other lanes anyway) stands in, and meets u = 0 there
  // (the shrink read no A column past the rank)
  {
    const E *Bg = Bb0 + (int64_t)g * rj * w0;
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int jc = jj < span ? jj : span - 1;
      const E *ptr = Bg + (int64_t)jc * w0;
      if constexpr (RK) ptr = g * rj + jc < rk ? ptr : Bb0;
      b[jj].load(ptr);
    }
  }
  float yv[8];
  if constexpr (kBf16) {
    const u32x4 w = buf_load16(yr, yoff_b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      yv[2 * i] = bf16_lo(w[i]);
      yv[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    const u32x4 w = buf_load16(yr, yoff_b), v = buf_load16(yr, yoff_b + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      yv[i] = __uint_as_float(w[i]);
      yv[4 + i] = __uint_as_float(v[i]);
    }
  }

  // ---- x row into LDS
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int task = tid + kBThreads * u;
    if (task < p.x_tasks) {
      if constexpr (kBf16) {
        const int pp = task / (RB / 8), i0 = 8 * (task % (RB / 8));
        u32x4 w0, w1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          w0[2 * m] = pair_lo(xv[u][0][m], xv[u][1][m]);
          w0[2 * m + 1] = pair_hi(xv[u][0][m], xv[u][1][m]);
          w1[2 * m] = pair_lo(xv[u][0][m + 2], xv[u][1][m + 2]);
          w1[2 * m + 1] = pair_hi(xv[u][0][m + 2], xv[u][1][m + 2]);
        }
        uint32_t *xw = reinterpret_cast<uint32_t *>(bgmv_lds) + pp * RB + i0;
        *reinterpret_cast<u32x4 *>(xw) = w0;
        *reinterpret_cast<u32x4 *>(xw + 4) = w1;
      } else {
        u32x4 *xf = reinterpret_cast<u32x4 *>(bgmv_lds) + 2 * task;
        xf[0] = xv[u][0];
        xf[1] = xv[u][1];
      }
    }
  }
  __syncthreads();

  // ---- shrink
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  for (int s = 0; s < p.n_slices; ++s) {
    const rsrc_t ar = make_rsrc(reinterpret_cast<const E *>(pick<NS>(p.A, s, p.n_slices)) +
                                    (int64_t)slot * pick<NS>(p.a_stride, s, p.n_slices),
                                a_bytes);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int bb = 0; bb < p.n_inst; bb += NA) {
      if (!ONE && (s > 0 || bb > 0)) {
#pragma unroll
        for (int q = 0; q < NA; ++q)
          a[q].load(ar, a_live ? (uint32_t)((((bb + q) * RB + rr) * R + 8 * jo) * sizeof(E)) : 0x7FFFFFF0u);
      }
      if constexpr (kBf16) {
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(bgmv_lds) + rr;
#pragma unroll
        for (int m = 0; m < NA / 2; ++m) {
          const uint32_t xp = xw[(bb / 2 + m) * RB];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = dot2_bf16(pair_lo(a[2 * m].w[i], a[2 * m + 1].w[i]), xp, acc[2 * i]);
            acc[2 * i + 1] = dot2_bf16(pair_hi(a[2 * m].w[i], a[2 * m + 1].w[i]), xp, acc[2 * i + 1]);
          }
        }
      } else {
        const float *xf = reinterpret_cast<const float *>(bgmv_lds) + rr;
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          const float xq = xf[(bb + q) * RB];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(xq, a[q][i], acc[i]);
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
    if constexpr (kBf16) {
      if (tid < R / 2) {  // fixed-order sum over the waves, then the bf16 hi/lo split of u
        float v0 = 0.f, v1 = 0.f;
        for (int w = 0; w < kBWaves; ++w) {
          v0 += red[w][2 * tid];
          v1 += red[w][2 * tid + 1];
        }
        uint32_t h0, l0, h1, l1;
        split_bf16(sc * v0, h0, l0);
        split_bf16(sc * v1, h1, l1);
        uh[s][tid] = h0 | (h1 << 16);
        ul[s][tid] = l0 | (l1 << 16);
      }
    } else {
      if (tid < R) {  // fixed-order sum over the waves
        float v = 0.f;
        for (int w = 0; w < kBWaves; ++w) v += red[w][tid];
        us[s][tid] = sc * v;
      }
    }
    __syncthreads();
  }

  // ---- expand: thread group (jg lanes) owns an 8-column octet; lane g takes
  // rank rows [g * rj, (g + 1) * rj); the group sum lands in lane g == 0
  for (int o = o0, it = 0; o < n_oct; o += ostep, ++it) {
    int s = s0;
    int64_t n0 = n00, w = w0, yoff = yoff0;
    const E *Bb = Bb0;  // rank row 0 of this octet's columns
    if (!ONE && it > 0) {
      s = slice_of_oct<NS>(p, o);
      n0 = 8 * (int64_t)(o - pick<NS + 1>(p.oct_base, s, p.n_slices));
      w = pick<NS>(p.width, s, p.n_slices);
      Bb = reinterpret_cast<const E *>(pick<NS>(p.B, s, p.n_slices)) + (int64_t)slot * pick<NS>(p.b_stride, s, p.n_slices) +
           n0;
      yoff = pick<NS>(p.offset, s, p.n_slices) + n0;
      if (g == 0 && p.add) load8(y + yoff, yv);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int jb = 0; jb < rj; jb += NB) {
      if (!ONE && (it > 0 || jb > 0)) {
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          const int jc = jb + (jj < span ? jj : span - 1);
          const E *ptr = Bb + ((int64_t)g * rj + jc) * w;
          if constexpr (RK) ptr = g * rj + jc < rk ? ptr : Bb;
          b[jj].load(ptr);
        }
      }
      if constexpr (kBf16) {  // rank rows come in pairs (j even, j + 1)
#pragma unroll
        for (int m = 0; m < NB / 2; ++m) {
          if (2 * m < span) {
            const int pj = (g * rj + jb) / 2 + m;
            const uint32_t hp = uh[s][pj], lp = ul[s][pj];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t e0 = pair_lo(b[2 * m].w[i], b[2 * m + 1].w[i]);
              const uint32_t e1 = pair_hi(b[2 * m].w[i], b[2 * m + 1].w[i]);
              acc[2 * i] = dot2_bf16(e0, hp, dot2_bf16(e0, lp, acc[2 * i]));
              acc[2 * i + 1] = dot2_bf16(e1, hp, dot2_bf16(e1, lp, acc[2 * i + 1]));
            }
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
          if (jj < span) {
            const float uv = us[s][g * rj + jb + jj];
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = fmaf(uv, b[jj][c], acc[c]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = group_sum(acc[c], jg);
    if (g == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) yv[c] += acc[c];
      store8(y + yoff, yv);
    }
  }
}

// ------------------------------------------------------------------ host side

// A load instructions per slice (rounded up to whole batches), x staging
// tasks and LDS bytes of the staged x row.
static void bgmv_x_plan(int64_t d_in, int32_t R, bool bf16, int32_t &n_inst, int32_t &x_tasks, size_t &lds) {
  const int64_t rb = (int64_t)kBThreads / (R / 8);
  const int64_t na = bf16 ? kBNA<uint16_t> : kBNA<float>;
  n_inst = (int32_t)(((d_in + rb - 1) / rb + na - 1) / na * na);
  x_tasks = (int32_t)(bf16 ? n_inst * rb / 16 : n_inst * rb / 8);
  lds = (size_t)n_inst * rb * (bf16 ? 2 : 4);
}

bool bgmv_fits(int64_t T, int32_t S, int64_t d_in, int32_t n_slices, const int64_t *width, int32_t R,
               int64_t ldy, bool bf16, int mode) {
  if (mode == 2) return false;  // SGMV requested
  const int64_t e = bf16 ? 2 : 4;
  int64_t sw = 0;
  for (int s = 0; s < n_slices; ++s) sw += width[s];
  const int64_t w_tok = ((int64_t)n_slices * d_in + sw) * R * e;  // weight bytes per token
  if (sw / 8 > kBMaxOct || d_in * e > kBMaxX || w_tok > (1 << 20)) return false;
  if (ldy * e >= (int64_t)1 << 30) return false;  // y rows are addressed with 32-bit buffer offsets
  int32_t n_inst, x_tasks;
  size_t lds;
  bgmv_x_plan(d_in, R, bf16, n_inst, x_tasks, lds);
  if (x_tasks > 2 * kBThreads || lds > 49152) return false;
  return mode == 1 || T <= 16 * (int64_t)S;  // BGMV requested, or few tokens per slot
}

template <typename E, int R, int NS, bool ONE>
static hipError_t launch_k(const BgmvParams &p, int grid, size_t lds, hipStream_t stream) {
  if (p.slot_rank)
    hipLaunchKernelGGL((bgmv_fused_kernel<E, R, true, NS, ONE>), dim3(grid), dim3(kBThreads), lds, stream,
                       p.meta.sorted, p.meta.sorted_slot, p.meta.T, p);
  else
    hipLaunchKernelGGL((bgmv_fused_kernel<E, R, false, NS, ONE>), dim3(grid), dim3(kBThreads), lds, stream,
                       p.meta.sorted, p.meta.sorted_slot, p.meta.T, p);
  return hipGetLastError();
}

template <typename E, int R>
static hipError_t launch_t(const BgmvParams &p, int grid, size_t lds, hipStream_t stream) {
  // one batch of everything: A rows (n_inst <= NA), the lane groups' octets
  // (n_oct <= threads / jg) and their rank rows (R / jg <= NB)
  const bool one = p.n_slices == 1 && p.n_inst <= kBNA<E> && p.oct_base[1] * p.jg <= kBThreads &&
                   R / p.jg <= kBNB<E>;
  if (one) return launch_k<E, R, 1, true>(p, grid, lds, stream);
  return with_slice_bound(p.n_slices, [&](auto ns) { return launch_k<E, R, decltype(ns)::value, false>(p, grid, lds, stream); });
}

hipError_t launch_bgmv(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                       int32_t n_slices, const void *const *A, const int64_t *a_stride,
                       const void *const *B, const int64_t *b_stride, const int64_t *width,
                       const int64_t *offset, int32_t R, float scale, const float *slot_scale,
                       const int32_t *slot_rank, void *y, int64_t ldy, int add, hipStream_t stream) {
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
  int jg = 1;  // at most R / 2, so every lane keeps whole pairs of rank rows
  while (jg < 16 && jg < R / 2 && (int64_t)n_oct * jg * 2 <= kBThreads) jg *= 2;
  p.jg = jg;
  size_t lds = 0;
  bgmv_x_plan(d_in, R, bf16, p.n_inst, p.x_tasks, lds);
  p.scale = scale;
  p.slot_scale = slot_scale;
  p.slot_rank = slot_rank;
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  if (meta.T == 0) return hipSuccess;
  const int grid = (int)(8 * ((meta.T + 7) / 8));
  switch (R) {
    case 8: return bf16 ? launch_t<uint16_t, 8>(p, grid, lds, stream) : launch_t<float, 8>(p, grid, lds, stream);
    case 16: return bf16 ? launch_t<uint16_t, 16>(p, grid, lds, stream) : launch_t<float, 16>(p, grid, lds, stream);
    case 32: return bf16 ? launch_t<uint16_t, 32>(p, grid, lds, stream) : launch_t<float, 32>(p, grid, lds, stream);
    case 64: return bf16 ? launch_t<uint16_t, 64>(p, grid, lds, stream) : launch_t<float, 64>(p, grid, lds, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
