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
//  * vector path (the BGMV form; fp32, and short bf16 segments): the B tile of
//    an item (r rows x up to 512 columns) is read once with 16-byte loads into
//    LDS and shared by every token of the m-chunk; each thread owns 8-column
//    octets of one token row.  Rows without an adapter are zero-filled here
//    when storing.
//  * matrix-core path (the SGMV form; bf16 segments of at least `mfma_min`
//    tokens): 64 tokens x 128 columns per item, v_mfma_f32_16x16x32_bf16 with
//    K = rank; u is split into bf16 hi + lo parts (two products), so the result
//    carries about 16 mantissa bits of u rather than 8; the B tile is stored
//    row-major in LDS with 16-byte writes and read back as MFMA operands with
//    the gfx950 transposing LDS read; the fp32 tile goes through LDS so that y
//    is read and written 16 bytes per lane.
//
// Every item reads the token indices, the B tile, the rank-r rows and the y
// segments it updates before it waits for any of them.  Inside lora_apply the
// rank-r rows arrive in sorted-position order, possibly as split-K partial
// sums that are added here in k-chunk order.
#include "lora_host.h"

namespace lora {

constexpr int kExpThreads = 256;
constexpr int kEVecRows = 8;       // tokens per vector m-chunk
constexpr int kEVecLds = 32768;    // bytes of the shared B tile on the vector path
constexpr int kEMmaRows = 64;      // tokens per matrix-core m-chunk
constexpr int kEMmaCols = 128;     // columns per matrix-core n-tile

struct ExpandParams {
  MetaView meta;
  const float *u;
  int32_t u_mode;  // 0: token order, 1: sorted order, 2: kch partial sums (sorted order)
  int32_t kch;
  const void *B[kMaxSlices];
  int64_t b_stride[kMaxSlices];
  int64_t width[kMaxSlices];
  int64_t offset[kMaxSlices];
  int32_t ntiles_vec, ntiles_mma;     // n-tiles over all slices, per path
  int32_t vec_cols;                   // columns per vector n-tile
  int32_t n_slices;
  void *y;
  int64_t ldy;
  int32_t add;
  int32_t use_mma_mode, mfma_min;
};

template <typename E, int R>
struct ExpandLds {
  union {
    struct {
      E bt[kEVecLds / sizeof(E)];  // B tile [R][vec_cols]
      float us[kEVecRows][R];
    } vec;
    struct {
      uint16_t bl[(R < 32 ? 32 : R) * (kEMmaCols + 16)];  // B tile, row j, column n
    } mma;
    struct {
      float out[kEMmaRows][kEMmaCols + 4];
    } epi;
  };
};

// Slice and slice-local index of n-tile `tile` when every slice is cut into
// tiles of nc columns (unrolled over the slice table: no runtime indexing).
__device__ __forceinline__ void tile_slice(const ExpandParams &p, int nc, int tile, int &s,
                                           int &local) {
  int base = 0;
  s = 0;
  local = tile;
#pragma unroll
  for (int k = 0; k < kMaxSlices; ++k) {
    if (k < p.n_slices) {
      const int nt = (int)((p.width[k] + nc - 1) / nc);
      if (tile >= base && tile < base + nt) {
        s = k;
        local = tile - base;
      }
      base += nt;
    }
  }
}

__device__ __forceinline__ bool exp_takes_mma(const ExpandParams &p, int count, int slot) {
  return slot >= 0 && (p.use_mma_mode == 2 || (p.use_mma_mode == 1 && count >= p.mfma_min));
}


// 8 rank values j..j+7 of slice s for sorted position pos (token t).
__device__ __forceinline__ void load_u8(const ExpandParams &p, int R, int s, int64_t pos,
                                        int64_t t, int j, float v[8]) {
  const int64_t T = p.meta.T;
  const int64_t row = p.u_mode == 0 ? t : pos;
  load8(p.u + ((int64_t)s * T + row) * R + j, v);
  if (p.u_mode == 2) {
    const int64_t plane = (int64_t)p.n_slices * T * R;
    for (int kc = 1; kc < p.kch; ++kc) {
      float w[8];
      load8(p.u + kc * plane + ((int64_t)s * T + pos) * R + j, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += w[i];
    }
  }
}

// ------------------------------------------------------------------ vector path

template <typename E, int R>
__device__ __forceinline__ void exp_vec_item(const ExpandParams &p, ExpandLds<E, R> &lds, int slot, int64_t pos0,
                             int rows, int s, int nt) {
  const int tid = threadIdx.x;
  const int NC = p.vec_cols;           // columns of this tile (a multiple of 8)
  const int OCT = NC / 8;
  const int64_t w = pick(p.width, s);
  const int64_t nbase = (int64_t)nt * NC;
  E *y = reinterpret_cast<E *>(p.y);

  // pairs (row m, octet o) owned by this thread: idx = tid + 256 i
  constexpr int MAXP = kEVecRows * 512 / 8 / kExpThreads;  // 2
  int64_t tok[MAXP];
  float yv[MAXP][8];
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int idx = tid + kExpThreads * i;
    const int m = idx / OCT, o = idx % OCT;
    tok[i] = -1;
    if (idx < kEVecRows * OCT && m < rows && nbase + 8 * o < w)
      tok[i] = p.meta.sorted[pos0 + m];
  }
  if (slot >= 0) {
    // B tile rows j, columns [nbase, nbase + NC) -> LDS, 16-byte loads
    const E *Bb = reinterpret_cast<const E *>(pick(p.B, s)) + (int64_t)slot * pick(p.b_stride, s) + nbase;
    for (int idx = tid; idx < R * OCT; idx += kExpThreads) {
      const int j = idx / OCT, o = idx % OCT;
      Raw8<E> v;
      if (nbase + 8 * o < w) v.load(Bb + (int64_t)j * w + 8 * o); else v.zero();
      if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<u32x4 *>(&lds.vec.bt[j * NC + 8 * o]) = v.w;
      } else {
        *reinterpret_cast<f32x4 *>(&lds.vec.bt[j * NC + 8 * o]) = v.a;
        *reinterpret_cast<f32x4 *>(&lds.vec.bt[j * NC + 8 * o + 4]) = v.b;
      }
    }
    // rank-r rows
    for (int idx = tid; idx < rows * (R / 8); idx += kExpThreads) {
      const int m = idx / (R / 8), j = 8 * (idx % (R / 8));
      const int64_t t = p.u_mode == 0 ? (int64_t)p.meta.sorted[pos0 + m] : 0;
      float v[8];
      load_u8(p, R, s, pos0 + m, t, j, v);
      *reinterpret_cast<f32x4 *>(&lds.vec.us[m][j]) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4 *>(&lds.vec.us[m][j + 4]) = f32x4{v[4], v[5], v[6], v[7]};
    }
  }
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) yv[i][c] = 0.f;
    if (tok[i] >= 0 && p.add) {
      const int o = (tid + kExpThreads * i) % OCT;
      load8(y + tok[i] * p.ldy + pick(p.offset, s) + nbase + 8 * o, yv[i]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    if (tok[i] < 0) continue;
    const int idx = tid + kExpThreads * i;
    const int m = idx / OCT, o = idx % OCT;
    if (slot >= 0) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < R; ++j) {
        Raw8<E> b;
        if constexpr (sizeof(E) == 2) {
          b.w = *reinterpret_cast<const u32x4 *>(&lds.vec.bt[j * NC + 8 * o]);
        } else {
          b.a = *reinterpret_cast<const f32x4 *>(&lds.vec.bt[j * NC + 8 * o]);
          b.b = *reinterpret_cast<const f32x4 *>(&lds.vec.bt[j * NC + 8 * o + 4]);
        }
        const float uv = lds.vec.us[m][j];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(uv, b[c], acc[c]);
      }
      // the delta is summed on its own, then added to y once
#pragma unroll
      for (int c = 0; c < 8; ++c) yv[i][c] += acc[c];
    }
    store8(y + tok[i] * p.ldy + pick(p.offset, s) + nbase + 8 * o, yv[i]);
  }
  __syncthreads();
}

// ------------------------------------------------------------- matrix-core path

template <typename E, int R>
__device__ __forceinline__ void exp_mma_item(const ExpandParams &p, ExpandLds<E, R> &lds, int slot, int64_t pos0,
                             int rows, int s, int nt) {
  constexpr int RP = R < 32 ? 32 : R;  // K padded to whole 32-wide steps
  constexpr int LDB = kEMmaCols + 16;   // LDS row stride of the B tile
  constexpr int BOCT = RP * kEMmaCols / 8 / kExpThreads;  // B octets per thread
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t w = pick(p.width, s);
  const int64_t nbase = (int64_t)nt * kEMmaCols;
  const uint16_t *Bb = reinterpret_cast<const uint16_t *>(pick(p.B, s)) + (int64_t)slot * pick(p.b_stride, s);
  uint16_t *y = reinterpret_cast<uint16_t *>(p.y);

  // epilogue ownership: rows tid/16 + 16 i, octet tid % 16; token indices first
  const int eo = tid % 16;
  const int64_t en = nbase + 8 * eo;
  int64_t tok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r_ = tid / 16 + 16 * i;
    tok[i] = (r_ < rows && en < w) ? (int64_t)p.meta.sorted[pos0 + r_] : -1;
  }
  // B tile [R][128] into registers
  u32x4 bq[BOCT];
#pragma unroll
  for (int q = 0; q < BOCT; ++q) {
    const int idx = tid + kExpThreads * q;
    const int j = idx / (kEMmaCols / 8), n0 = 8 * (idx % (kEMmaCols / 8));
    if (j < R && nbase + n0 < w)
      bq[q] = *reinterpret_cast<const u32x4 *>(Bb + (int64_t)j * w + nbase + n0);
    else
      bq[q] = u32x4{0, 0, 0, 0};
  }
  // u fragments: lane (mrow, g), step c holds k = 32c + 8g + e, split into bf16 hi + lo
  const int mrow = lane % 16, g = lane / 16;
  const int row = 16 * wave + mrow;
  float uf[RP / 32][8];
#pragma unroll
  for (int c = 0; c < RP / 32; ++c) {
    const int k = 32 * c + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) uf[c][i] = 0.f;
    if (row < rows && k < R) {
      const int64_t t = p.u_mode == 0 ? (int64_t)p.meta.sorted[pos0 + row] : 0;
      load_u8(p, R, s, pos0 + row, t, k, uf[c]);
    }
  }
  // y segments
  float yv[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) yv[i][c] = 0.f;
    if (tok[i] >= 0 && p.add) load8(y + tok[i] * p.ldy + pick(p.offset, s) + en, yv[i]);
  }
  // B tile -> LDS, row-major (16-byte writes)
#pragma unroll
  for (int q = 0; q < BOCT; ++q) {
    const int idx = tid + kExpThreads * q;
    const int j = idx / (kEMmaCols / 8), n0 = 8 * (idx % (kEMmaCols / 8));
    *reinterpret_cast<u32x4 *>(&lds.mma.bl[j * LDB + n0]) = bq[q];
  }
  bf16x8 uh[RP / 32], ul[RP / 32];
#pragma unroll
  for (int c = 0; c < RP / 32; ++c) {
    u32x4 hw, lw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float v = uf[c][2 * i + h];
        hb[h] = f32_to_bf16(v);
        lb[h] = f32_to_bf16(v - __uint_as_float(hb[h] << 16));
      }
      hw[i] = hb[0] | (hb[1] << 16);
      lw[i] = lb[0] | (lb[1] << 16);
    }
    uh[c] = __builtin_bit_cast(bf16x8, hw);
    ul[c] = __builtin_bit_cast(bf16x8, lw);
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
      const bf16x8 bv = lds_col8(lds.mma.bl, LDB, k, 16 * b);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uh[c], bv, acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ul[c], bv, acc[b], 0, 0, 0);
    }
  }
  __syncthreads();  // the B tile is fully read before the epilogue reuses the LDS
#pragma unroll
  for (int b = 0; b < kEMmaCols / 16; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) lds.epi.out[16 * wave + 4 * g + v][16 * b + mrow] = acc[b][v];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (tok[i] < 0) continue;
    const int r_ = tid / 16 + 16 * i;
#pragma unroll
    for (int c = 0; c < 8; ++c) yv[i][c] += lds.epi.out[r_][8 * eo + c];
    store8(y + tok[i] * p.ldy + pick(p.offset, s) + en, yv[i]);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ the kernel

template <typename E, int R>
__global__ __launch_bounds__(kExpThreads) void expand_kernel(ExpandParams p) {
  __shared__ ExpandLds<E, R> lds;
  extern __shared__ __align__(16) unsigned char expand_dyn[];
  const SegTable tb = seg_table_at(expand_dyn, p.meta.S);
  // the no-adapter segment (always first) is visited only to store zeros
  build_items(p.meta, tb, p.add != 0, [&](int c, int slot) {
    const bool mma = exp_takes_mma(p, c, slot);
    const int mc = mma ? kEMmaRows : kEVecRows;
    return ((c + mc - 1) / mc) * (mma ? p.ntiles_mma : p.ntiles_vec);
  });
  const int first = tb.scal[1];
  for (int item = blockIdx.x; item < tb.scal[2]; item += gridDim.x) {
    const int si = find_item_segment(tb, item);
    const int seg = first + si;
    const int count = tb.count[seg];
    const int slot = tb.slot[seg];
    const int local = item - (si > 0 ? tb.item_end[si - 1] : 0);
    if constexpr (sizeof(E) == 2) {
      if (exp_takes_mma(p, count, slot)) {
        const int chunk = local / p.ntiles_mma;
        int s, nt;
        tile_slice(p, kEMmaCols, local % p.ntiles_mma, s, nt);
        const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kEMmaRows;
        exp_mma_item<E, R>(p, lds, slot, pos0, min(kEMmaRows, count - chunk * kEMmaRows), s, nt);
        continue;
      }
    }
    const int chunk = local / p.ntiles_vec;
    int s, nt;
    tile_slice(p, p.vec_cols, local % p.ntiles_vec, s, nt);
    const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kEVecRows;
    exp_vec_item<E, R>(p, lds, slot, pos0, min(kEVecRows, count - chunk * kEVecRows), s, nt);
  }
}

// ------------------------------------------------------------------ host side

template <typename E, int R>
static hipError_t launch_t(const ExpandParams &p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((expand_kernel<E, R>), dim3(grid), dim3(kExpThreads), seg_table_bytes(p.meta.S),
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_expand(const MetaView &meta, const float *u, int u_mode, int kch, int32_t n_slices,
                         const void *const *B, const int64_t *b_stride, const int64_t *width,
                         const int64_t *offset, int32_t R, void *y, int64_t ldy, bool bf16,
                         int add, int mode, hipStream_t stream) {
  ExpandParams p{};
  p.meta = meta;
  p.u = u;
  p.u_mode = u_mode;
  p.kch = kch;
  p.n_slices = n_slices;
  // vector n-tile: up to 512 columns, as many as fit the shared B tile
  const int64_t e = bf16 ? 2 : 4;
  p.vec_cols = (int)std::min<int64_t>(512, kEVecLds / (R * e));
  p.ntiles_vec = p.ntiles_mma = 0;
  for (int s = 0; s < n_slices; ++s) {
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
    p.ntiles_vec += (int32_t)((width[s] + p.vec_cols - 1) / p.vec_cols);
    p.ntiles_mma += (int32_t)((width[s] + kEMmaCols - 1) / kEMmaCols);
  }
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  p.use_mma_mode = !bf16 ? 0 : (mode == 1 ? 0 : (mode == 2 ? 2 : 1));
  p.mfma_min = expand_mma_min_default();
  if (meta.T == 0) return hipSuccess;
  const int64_t T = meta.T, S = meta.S;
  const int64_t bound_vec = ((T + kEVecRows - 1) / kEVecRows + S + 1) * p.ntiles_vec;
  const int64_t bound_mma =
      p.use_mma_mode ? ((T + kEMmaRows - 1) / kEMmaRows + S + 1) * p.ntiles_mma : 0;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(bound_vec + bound_mma, 4096));
  switch (R) {
    case 8: return bf16 ? launch_t<uint16_t, 8>(p, grid, stream) : launch_t<float, 8>(p, grid, stream);
    case 16: return bf16 ? launch_t<uint16_t, 16>(p, grid, stream) : launch_t<float, 16>(p, grid, stream);
    case 32: return bf16 ? launch_t<uint16_t, 32>(p, grid, stream) : launch_t<float, 32>(p, grid, stream);
    case 64: return bf16 ? launch_t<uint16_t, 64>(p, grid, stream) : launch_t<float, 64>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
