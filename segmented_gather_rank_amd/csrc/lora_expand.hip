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

struct ExpandParams {
  MetaView meta;
  const float *u;
  int32_t u_mode;  // 0: token order, 1: sorted order, 2: kch partial sums (sorted order)
  int32_t kch;
  const void *B[kMaxSlices];
  int64_t b_stride[kMaxSlices];
  int64_t width[kMaxSlices];
  int64_t offset[kMaxSlices];
  int32_t ntiles_vec;                 // vector n-tiles over all slices
  int32_t vec_cols;                   // columns per vector n-tile
  int32_t steps[kMaxSlices];          // matrix-core path: 128-column steps per slice
  int32_t steps_total;                // and over all slices
  int32_t nck_tab[17];                // [c]: column chunks over all slices at c steps per item
  int32_t n_slices;
  void *y;
  int64_t ldy;
  int32_t add;
  const int32_t *slot_rank;  // per-slot ranks, or null (every slot uses R)
  // long-segment path: the rank-r rows rounded to bf16 [n_slices][T][R], in
  // sorted-position order, and 512-column chunks
  const uint16_t *uh;
  int32_t rows_nck[kMaxSlices];       // 512-column chunks per slice
  int32_t rows_nck_total;
  uint32_t y_bytes;                   // bytes of y the windows reach (< 2^31)
  uint32_t plane_bytes;               // bytes of one u plane (< 2^30)
  int32_t ra;                         // the caller's r_max: B rows and ranks read (ra <= R)
  int32_t u_ld;                       // row stride of u in token order (the caller's u: ra)
  unsigned long long *clk;            // a measurement build's phase records, or null
};

template <typename E, int R>
struct ExpandLds {
  E bt[kEVecLds / sizeof(E)];  // B tile [R][vec_cols]
  float us[kEVecRows][R];
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



// 8 rank values j..j+7 of slice s for sorted position pos (token t).
__device__ __forceinline__ void load_u8(const ExpandParams &p, int R, int s, int64_t pos,
                                        int64_t t, int j, float v[8]) {
  const int64_t T = p.meta.T;
  const int64_t row = p.u_mode == 0 ? t : pos;
  const int ld = p.u_mode == 0 ? p.u_ld : R;  // the caller's u is [n_slices][T][ra]
  const float *src = p.u + ((int64_t)s * T + row) * ld + j;
  const int64_t plane = (int64_t)p.n_slices * T * R;
  const int kch = p.u_mode == 2 ? p.kch : 1;
  const f32x4 a = sum_partials4(src, plane, kch), b = sum_partials4(src + 4, plane, kch);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// ------------------------------------------------------------------ vector path

template <typename E, int R>
__device__ __forceinline__ void exp_vec_item(const ExpandParams &p, ExpandLds<E, R> &lds, int slot, int64_t pos0,
                             int rows, int s, int nt) {
  const int rk = slot >= 0 ? slot_rank_of(p.slot_rank, slot, p.ra) : 0;  // ranks past rk are not read
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
      if (nbase + 8 * o < w && j < rk) v.load(Bb + (int64_t)j * w + 8 * o); else v.zero();
      if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<u32x4 *>(&lds.bt[j * NC + 8 * o]) = v.w;
      } else {
        *reinterpret_cast<f32x4 *>(&lds.bt[j * NC + 8 * o]) = v.a;
        *reinterpret_cast<f32x4 *>(&lds.bt[j * NC + 8 * o + 4]) = v.b;
      }
    }
    // rank-r rows
    for (int idx = tid; idx < rows * (R / 8); idx += kExpThreads) {
      const int m = idx / (R / 8), j = 8 * (idx % (R / 8));
      const int64_t t = p.u_mode == 0 ? (int64_t)p.meta.sorted[pos0 + m] : 0;
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < rk) load_u8(p, R, s, pos0 + m, t, j, v);
      *reinterpret_cast<f32x4 *>(&lds.us[m][j]) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4 *>(&lds.us[m][j + 4]) = f32x4{v[4], v[5], v[6], v[7]};
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
          b.w = *reinterpret_cast<const u32x4 *>(&lds.bt[j * NC + 8 * o]);
        } else {
          b.a = *reinterpret_cast<const f32x4 *>(&lds.bt[j * NC + 8 * o]);
          b.b = *reinterpret_cast<const f32x4 *>(&lds.bt[j * NC + 8 * o + 4]);
        }
        const float uv = lds.us[m][j];
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
//
// One item = (segment, tile of up to 64 sorted tokens, chunk of `cpi` columns of
// one slice), walked in steps of W columns.  The product is taken transposed,
// D'[col][token] = B^T u^T with v_mfma_f32_16x16x16_bf16: the A operand (16
// columns x 4 ranks per lane) comes from the step's B tile in LDS through the
// gfx950 transposing read, the B operand (4 ranks of one token per lane) is u
// split into bf16 hi + lo and held in registers for the whole item.  The tile's
// rank rows are read once per workgroup (split-K partial sums added in k-chunk
// order) and handed to the lanes through LDS.  The B tile is written to LDS
// with its columns permuted inside every 32-column group so that, for each
// pair of 16-column blocks, a lane's 8 results are 8 consecutive columns of one
// token: y is read and written 16 bytes per lane, with no LDS round trip.  The
// next step's B tile and y octets are loaded while the current step is
// multiplied (two LDS buffers, one barrier per step).
//
// Waves and tokens: a tile has nb = ceil(rows / 16) blocks of 16 tokens; the 4
// waves are spread over them (4, 2 or 1 waves per block) and the waves that
// share a block split the step's columns.  A step is 128 columns, or up to
// 512 for tiles of at most 32 tokens and ranks below 64, so that every step
// moves the same RP x W block of B and a short tile needs few steps.

constexpr int kXThreads = 256;
constexpr int kXStep = 128;          // columns per step (the narrowest step)

// BO: B in the output-rows layout; a step's B tile then sits in LDS as one
// row of RP ranks per column (row stride LDO: the 16 columns that one MFMA
// operand read touches fall in distinct banks), else as RP rank rows of W
// columns
template <int R, bool BO>
struct XLds {
  static constexpr int RP = R < 16 ? 16 : R;  // ranks padded to whole 16-wide steps
  static constexpr int WMAX = kXStep * (64 / RP);  // widest step (short tiles)
  static constexpr int LDO = RP + 8;
  uint16_t bl[2][BO ? WMAX * LDO : RP * (WMAX + 16)];
  uint16_t uh[kTileRows][RP], ul[kTileRows][RP];  // the tile's rank rows, bf16 hi and lo parts
  int32_t tok[kTileRows];                         // the tile's tokens
};

template <int R, int NS, bool BO>
__global__ __launch_bounds__(kXThreads, 3) void expand_mma_kernel(const int32_t *__restrict__ info,
                                                                  const int32_t *__restrict__ tiles,
                                                                  ExpandParams p) {
  constexpr int RP = XLds<R, BO>::RP;
  constexpr int LDO = XLds<R, BO>::LDO;
  constexpr int KS = RP / 16;                     // MFMA k-steps
  constexpr int BQ = 4;                           // B octets per thread per step, at most
  __shared__ XLds<R, BO> lds;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // measurement build, the first item with an adapter: 0 start, 1 header
  // in, 2 prologue done (B's first step staged, the rank rows in LDS), 3 + i
  // after step i < 10, 13 steps | rows << 8, 14 XCC_ID, 15 end (stores
  // acknowledged)
  unsigned long long *rec = phase_record(p.clk);
  unsigned long long *const rec0 = rec;
  phase_stamp(rec, 0);
  const int n = lane % 16, kg = lane / 16;
  const int64_t T = p.meta.T;
  // live tiles: the tile list is in key order, so the tiles of tokens without
  // an adapter come first, and adding into y they need no work
  const int ntl = uniform_value(info[4]);
  const int nneg = p.add ? uniform_value(info[3]) : 0;
  const int t0 = (nneg + kTileRows - 1) / kTileRows;
  const int live = ntl - t0;
  if (live <= 0) return;
  // steps (128 columns) per item, spi: from spi0, the live tiles' steps spread
  // evenly over the grid (when the live tiles average at most 32 tokens, at
  // least the width of one wide step), up to 16, the choice with the fewest
  // steps on the busiest workgroup (the smallest on ties).  An item is (column
  // chunk of one slice, tile), chunk-major, so tiles that share a chunk of B
  // are neighbours, and XCD x (blockIdx mod 8) takes a contiguous run of items
  const uint32_t live_u = (uint32_t)live;
  const int avg_rows = (int)((uint32_t)(T - nneg) / live_u);  // rows < 2^31
  const int wide = avg_rows <= 16 ? 4 : (avg_rows <= 32 ? 2 : 1);
  const int spi_min = min(wide, 64 / RP);
  const uint32_t per = gridDim.x / 8;
  const int spi0 = min(16, max(spi_min, (int)((live_u * (uint32_t)p.steps_total + gridDim.x - 1) / gridDim.x)));
  // lane l < 16 scores c = l + 1 steps per item (if c >= spi0): the steps on
  // the busiest workgroup, ceil(ceil(live * chunks(c) / 8) / per) * c; the
  // first row of lanes takes the lowest (cost, c) with DPP row rotations
  uint32_t score = 0xffffffffu;
  if (lane < 16 && lane + 1 >= spi0) {
    const uint32_t c = (uint32_t)lane + 1;
    const uint32_t run_c = (live_u * (uint32_t)pick<17>(p.nck_tab, (int)c) + 7) / 8;
    const uint32_t cost = (run_c + per - 1) / per * c;
    score = (cost < 0x7ffffffu ? cost : 0x7ffffffu) << 5 | c;
  }
  auto row_min = [](uint32_t v, auto ctrl) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)0xffffffff, (int)v, decltype(ctrl)::value, 0xf, 0xf,
                                                             false);
    return o < v ? o : v;
  };
  score = row_min(score, std::integral_constant<int, 0x128>{});  // row_ror:8
  score = row_min(score, std::integral_constant<int, 0x124>{});  // row_ror:4
  score = row_min(score, std::integral_constant<int, 0x122>{});  // row_ror:2
  score = row_min(score, std::integral_constant<int, 0x121>{});  // row_ror:1
  const int spi = (int)(__builtin_amdgcn_readfirstlane(score) & 31);
  const int nck = pick<17>(p.nck_tab, spi);
  // column chunks per slice at spi steps per item, once per workgroup
  int nk_s[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) nk_s[k] = k < p.n_slices ? (uniform_value(p.steps[k]) + spi - 1) / spi : 0;
  const int cpi = spi * kXStep;
  const int total = live * nck;
  const int run = (total + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int hi = min(total, xcd * run + run);
  int item = xcd * run + (int)blockIdx.x / 8;
  if (item >= hi) return;
  uint16_t *y = reinterpret_cast<uint16_t *>(p.y);

  // tile header, and this lane's token for each possible spread of waves over
  // token blocks (which one applies depends on rows); the next item's header
  // is loaded while the current item runs
  struct Header {
    int slot, rows, pos0, tk1, tk2, tk4, tfirst;
  };
  auto read_header = [&](int it) {
    const int32_t *tl = tiles + (int64_t)(t0 + it % live) * kTileInts;
    return Header{tl[0], tl[1], tl[2], tl[4 + 16 * wave + n], tl[4 + 16 * (wave / 2) + n], tl[4 + n], tl[4]};
  };
  Header hnext = read_header(item);

  for (; item < hi; item += per) {
    const int ck = item / live;
    const Header hd = hnext;
    if (item + per < hi) hnext = read_header(item + per);
    const int slot = uniform_value(hd.slot), rows = uniform_value(hd.rows);
    const int64_t pos0 = uniform_value(hd.pos0);
    phase_stamp(rec, 1);
    // chunk ck -> slice s and the chunk's first column in it
    int s = 0, cbase = 0, acc = 0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k >= p.n_slices) break;
      if (ck >= acc) {
        s = k;
        cbase = acc;
      }
      acc += nk_s[k];
    }
    const int64_t w = pick<NS>(p.width, s, p.n_slices);
    const int64_t col0 = (int64_t)(ck - cbase) * cpi;
    const int ncols = (int)min((int64_t)cpi, w - col0);
    const int nb = (rows + 15) / 16;
    const int wpt = nb == 1 ? 4 : (nb == 2 ? 2 : 1);  // waves per token block
    const int tbw = wave / wpt, wq = wave % wpt;
    // step width: 128 columns, or up to 64 / RP times that for short tiles,
    // so that a step always moves RP x W = up to 8192 B elements
    const int wx = min(wpt, 64 / RP);                 // 1, 2 or 4
    const int W = kXStep * wx, ldb = W + 16;
    const int osh = wx == 1 ? 4 : (wx == 2 ? 5 : 6);  // log2(W / 8): octets per B row
    const int nq = RP * W / 8 / kXThreads;            // B octets per thread per step
    const int nsteps = (ncols + W - 1) / W;
    const int cw = W / wpt;                           // columns of this wave per step
    const int nbp = cw / 32;                          // 16-column block pairs per step
    const int r = 16 * tbw + n;
    const bool rv = tbw < nb && r < rows;
    const int64_t t = rv ? (int64_t)(wpt == 4 ? hd.tk4 : (wpt == 2 ? hd.tk2 : hd.tk1)) : (int64_t)hd.tfirst;
    const int64_t yo = pick<NS>(p.offset, s, p.n_slices) + col0;
    uint16_t *yrow = y + t * p.ldy + yo;
    // this lane's y octet of block pair pp in step i: columns
    // i * W + wq * cw + 32 pp + 8 kg (clamped to the first one when not ours)
    auto ycol = [&](int i, int pp) -> int {
      const int c = i * W + wq * cw + 32 * pp + 8 * kg;
      return (pp < nbp && c < ncols) ? c : 0;
    };

    if (slot < 0) {  // store mode, no adapter: the windows become 0
      for (int i = 0; i < nsteps; ++i)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int c = i * W + wq * cw + 32 * pp + 8 * kg;
          if (rv && pp < nbp && c < ncols) gstore16(yrow + c, u32x4{0, 0, 0, 0});
        }
      continue;
    }

    // ---- B step tiles: rows j < RP, W columns; thread octet q covers row
    // idx / (W / 8), columns 8 (idx % (W / 8)) .. + 7 of the step
    // (idx = tid + 256 q); with BO (B_s[slot] is [w][ra]) it covers ranks
    // 8 (idx % (RP / 8)) .. + 7 of column idx / (RP / 8).  Loads past the slot
    // block (ranks >= R), past the slot's rank or past the chunk read zeros
    // without touching memory.
    const int rk = slot_rank_of(p.slot_rank, slot, p.ra);  // ranks past rk are not read
    const rsrc_t br = make_rsrc(reinterpret_cast<const uint16_t *>(pick<NS>(p.B, s, p.n_slices)) +
                                    (int64_t)slot * pick<NS>(p.b_stride, s, p.n_slices),
                                (uint32_t)(p.ra * w * 2));
    u32x4 bq[BQ];
    auto load_b = [&](int i) {
#pragma unroll
      for (int q = 0; q < BQ; ++q) {
        if (q < nq) {
          const int idx = tid + kXThreads * q;
          if constexpr (BO) {
            const int c = i * W + idx / (RP / 8), j = 8 * (idx % (RP / 8));
            bq[q] = buf_load16(br, (j < rk && c < ncols) ? (uint32_t)(((col0 + c) * p.ra + j) * 2) : 0x7FFFFFF0u);
          } else {
            const int j = idx >> osh, h = idx & ((1 << osh) - 1);
            const int c = i * W + 8 * h;
            bq[q] = buf_load16(br, (j < rk && c < ncols) ? (uint32_t)(((int64_t)j * w + col0 + c) * 2) : 0x7FFFFFF0u);
          }
        }
      }
    };
    // permuted store: the 8 columns 32 g32 + 8 g4 .. + 7 go to block 2 g32
    // (rows 4 g4 .. + 3) and block 2 g32 + 1 (same rows); with BO each
    // column's rank octet goes to the row of its permuted column
    auto store_b = [&](int buf) {
#pragma unroll
      for (int q = 0; q < BQ; ++q) {
        if (q < nq && BO) {
          const int idx = tid + kXThreads * q;
          const int c = idx / (RP / 8), j = 8 * (idx % (RP / 8)), h = c / 8, e = c % 8;
          const int col = 32 * (h / 4) + 4 * (h % 4) + (e < 4 ? e : 12 + e);
          *reinterpret_cast<u32x4 *>(&lds.bl[buf][col * LDO + j]) = bq[q];
        } else if (q < nq) {
          const int idx = tid + kXThreads * q;
          const int j = idx >> osh, h = idx & ((1 << osh) - 1);
          const int col = 32 * (h / 4) + 4 * (h % 4);
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<u32x2 *>(&lds.bl[buf][j * ldb + col]) = u32x2{bq[q][0], bq[q][1]};
          *reinterpret_cast<u32x2 *>(&lds.bl[buf][j * ldb + col + 16]) = u32x2{bq[q][2], bq[q][3]};
        }
      }
    };
    u32x4 ycur[4], ynext[4];
    auto load_y = [&](int i, u32x4 (&yy)[4]) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) yy[pp] = gload16(yrow + ycol(i, pp));
    };

    load_b(0);
    load_y(0, ycur);
    // ---- rank-r rows of the tile, read once per workgroup (rows x quads of
    // 4 ranks, two per thread and batch), split-K sums added in k-chunk order,
    // split into bf16 hi + lo parts in LDS; lane (token n, kg) then takes
    // ranks 16 c + 4 kg .. + 3 of its token for k-step c.  Rows in token
    // order need the tile's tokens, which the header already brought.
    if (p.u_mode == 0 && kg == 0) lds.tok[16 * wave + n] = hd.tk1;
    __syncthreads();  // the previous item's last step has read every buffer
    {
      constexpr int QR = RP / 4;
      const int uld = p.u_mode == 0 ? p.u_ld : R;  // the caller's u is [n_slices][T][ra]
      const float *ubase = p.u + (int64_t)s * T * uld;
      const int64_t plane = (int64_t)p.n_slices * T * R;
      for (int pi = tid; pi < rows * QR; pi += 2 * kXThreads) {
        f32x4 v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int pe = pi + kXThreads * e;
          const int row = pe / QR, j = 4 * (pe % QR);
          const int64_t urow = p.u_mode == 0 ? (int64_t)lds.tok[row < kTileRows ? row : 0] : pos0 + row;
          v[e] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (pe < rows * QR && j < rk) v[e] = sum_partials4(ubase + urow * uld + j, plane, p.kch);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int pe = pi + kXThreads * e;
          if (pe < rows * QR) {
            const int row = pe / QR, j = 4 * (pe % QR);
            uint32_t h[4], l[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) split_bf16(v[e][m], h[m], l[m]);
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2 *>(&lds.uh[row][j]) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            *reinterpret_cast<u32x2 *>(&lds.ul[row][j]) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
          }
        }
      }
    }
    store_b(0);
    __syncthreads();
    phase_stamp(rec, 2);
    // rows past the tile hold stale values: their results are never stored
    s16x4 uh[KS], ul[KS];
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      uh[c] = *reinterpret_cast<const s16x4 *>(&lds.uh[r][16 * c + 4 * kg]);
      ul[c] = *reinterpret_cast<const s16x4 *>(&lds.ul[r][16 * c + 4 * kg]);
    }
    for (int i = 0; i < nsteps; ++i) {
      // next step's loads
      const bool more = i + 1 < nsteps;
      if (more) {
        load_b(i + 1);
        load_y(i + 1, ynext);
      }
      const uint16_t *bt = lds.bl[i & 1];
      // per 16-column block pair: products, then the lane's 8 columns of y
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        if (pp < nbp) {
          f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          if (tbw < nb) {
            const int blk0 = (wq * cw) / 16 + 2 * pp;
#pragma unroll
            for (int c = 0; c < KS; ++c) {
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const s16x4 a =
                    BO ? *reinterpret_cast<const s16x4 *>(bt + (16 * (blk0 + hh) + n) * LDO + 16 * c + 4 * kg)
                       : lds_col4(bt, ldb, 16 * c + 4 * kg, 16 * (blk0 + hh));
                acc[hh] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ul[c], acc[hh], 0, 0, 0);
                acc[hh] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, uh[c], acc[hh], 0, 0, 0);
              }
            }
          }
          // lane (token n, kg) holds columns 32 pp + 8 kg + 0..7 of its share
          const int c = i * W + wq * cw + 32 * pp + 8 * kg;
          if (rv && c < ncols) {
            float v[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              v[2 * m] = p.add ? bf16_lo(ycur[pp][m]) : 0.f;
              v[2 * m + 1] = p.add ? bf16_hi(ycur[pp][m]) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] += acc[0][e];
              v[4 + e] += acc[1][e];
            }
            store8(yrow + c, v);
          }
        }
      }
      if (more) {
        store_b((i + 1) & 1);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) ycur[pp] = ynext[pp];
      }
      __syncthreads();
      if (i < 10) phase_stamp(rec, 3 + i);
    }
    phase_put(rec, 13, (unsigned long long)(nsteps | rows << 8));
    if constexpr (kPhaseClock) phase_put(rec, 14, __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u);
    rec = nullptr;
  }
  if constexpr (kPhaseClock) {
    if (rec0) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      phase_stamp(rec0, 15);
    }
  }
}

// ------------------------------------------------------------------ the vector kernel

template <typename E, int R>
__global__ __launch_bounds__(kExpThreads) void expand_kernel(ExpandParams p) {
  __shared__ ExpandLds<E, R> lds;
  extern __shared__ __align__(16) unsigned char expand_dyn[];
  const SegTable tb = seg_table_at(expand_dyn, p.meta.S);
  // the no-adapter segment (always first) is visited only to store zeros
  build_items(p.meta, tb, p.add != 0, [&](int c, int) {
    return ((c + kEVecRows - 1) / kEVecRows) * p.ntiles_vec;
  });
  const int first = tb.scal[1];
  for (int item = blockIdx.x; item < tb.scal[2]; item += gridDim.x) {
    const int si = find_item_segment(tb, item);
    const int seg = first + si;
    const int count = tb.count[seg];
    const int slot = tb.slot[seg];
    const int local = item - (si > 0 ? tb.item_end[si - 1] : 0);
    const int chunk = local / p.ntiles_vec;
    int s, nt;
    tile_slice(p, p.vec_cols, local % p.ntiles_vec, s, nt);
    const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kEVecRows;
    exp_vec_item<E, R>(p, lds, slot, pos0, min(kEVecRows, count - chunk * kEVecRows), s, nt);
  }
}

// ------------------------------------------------------------- long-segment path
//
// Prefill batches: segments of hundreds of tokens, so every work tile is full
// (64 tokens) and the expand is a stream over y.  How that stream is cut
// decides its speed: measured on a 1 GB bf16 y, an in-place add in steps of
// 64 rows x 128 columns (the tile kernel's step) runs at about 4.2 TB/s, and
// in steps of 16 rows x 512 columns, neighbouring workgroups on neighbouring
// columns of the same rows, at about 4.8 TB/s (a plain contiguous stream:
// 5.3 TB/s).  So here a workgroup owns one 512-column chunk of one slice and
// walks a range of consecutive tiles 16 tokens at a time: wave w owns columns
// 128 w .. + 127 of the chunk, the four waves on the same 16 rows, and the
// workgroups of one range (one per chunk) sweep the same rows together.  The
// B^T operands of a wave's columns stay in registers while the slot does not
// change (the chunk goes to LDS straight from memory, then into registers
// through the transposing read).  The rank-r rows come as one bf16 plane that
// a small kernel folds from the shrink's partial sums once per call: u is
// rounded to bf16 once, as the matrix cores take it, so a 32-rank step is one
// product (a high and a low part, two products, cost 9 % of the call here).
// The loop prefetches the next token block's plane rows and y, across tile
// boundaries too.  A block's results leave through LDS: the accumulators give
// a lane 8 columns of one token (a store of 16 rows x 64 bytes per wave
// instruction), so the 16 x 512 results meet in LDS and each wave stores 4
// whole 1 KB rows, one per instruction; the same y-only stream runs 10-15 %
// faster stored that way.

constexpr int kRowsCols = 512;             // columns per item, 128 per wave
constexpr int kRowsLdb = kRowsCols + 16;   // LDS row stride of the B chunk
constexpr int kXchLdb = kRowsCols + 8;     // ... of a token block's results: 16 B lanes of 16 rows hit
                                           // distinct banks
static_assert(2 * 16 * kXchLdb <= 32 * kRowsLdb, "two result blocks fit the B chunk's buffer");

// u plane: ub[i] = the sum over k-chunks, in order, of the partial sums at i,
// rounded once to bf16 (nearest even), as the MFMA operand takes it.  Rows of
// tokens without an adapter are skipped.
__global__ __launch_bounds__(256) void u_planes_kernel(const int32_t *__restrict__ info, const float *part,
                                                       int64_t T, int32_t n_slices, int32_t R, int32_t kch,
                                                       uint16_t *ub) {
  const int64_t plane = (int64_t)n_slices * T * R;
  const int64_t lo_pos = info[3];  // first sorted position with an adapter
  const int64_t quads = plane / 4;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = 4 * q;
    const int64_t pos = (i / R) % T;
    if (pos < lo_pos) continue;
    const f32x4 v = sum_partials4(part + i, plane, kch);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2 *>(ub + i) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

template <int R, int NS>
__global__ __launch_bounds__(kXThreads, R >= 64 ? 2 : 3) void expand_rows_kernel(const int32_t *__restrict__ info,
                                                                   const int32_t *__restrict__ tiles,
                                                                   ExpandParams p) {
  constexpr int RK = R < 32 ? 32 : R;          // ranks padded to whole 32-rank MFMA steps
  constexpr int KS = RK / 32;                  // MFMA k-steps
  constexpr uint32_t kOut = 0x7FFFFFF0u;       // past every resource: reads as zeros
  extern __shared__ __align__(16) uint16_t rows_lds[];  // one 32-rank step of the B chunk [32][kRowsLdb]
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i16x4 *lds_i16x4;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = lane % 16, kg = lane / 16;
  const int64_t T = p.meta.T;
  const int ntl = uniform_value(info[4]);
  const int nneg = p.add ? uniform_value(info[3]) : 0;
  const int t0 = (nneg + kTileRows - 1) / kTileRows;  // the no-adapter tiles lead; adding, they need no work
  const int live = ntl - t0;
  if (live <= 0) return;
  // work: nr ranges of consecutive live tiles x nck column chunks; a
  // workgroup takes one (range, chunk) and walks the range's tiles, so its B
  // chunk changes only where the slot does, and the workgroups of one range
  // (one per chunk) sweep the same rows together
  const int nck = p.rows_nck_total;
  const int G = (int)gridDim.x;
  const int nr = max(1, G / nck);
  const int tpr = (live + nr - 1) / nr;
  uint16_t *y = reinterpret_cast<uint16_t *>(p.y);

  // tile header; tk[q] is this lane's token of block q (unspecified past the
  // tile's rows, so never used there), tfirst the tile's first token, which
  // lanes past the rows read instead
  struct Header {
    int slot, rows, pos0, tfirst, tk[4];
  };
  auto read_header = [&](int i) {
    const int32_t *tl = tiles + (int64_t)(t0 + i) * kTileInts;
    return Header{tl[0], tl[1], tl[2], tl[4], {tl[4 + n], tl[4 + 16 + n], tl[4 + 32 + n], tl[4 + 48 + n]}};
  };
  auto tok_of = [](const Header h, int tb) __attribute__((always_inline)) {
    return tb == 0 ? h.tk[0] : (tb == 1 ? h.tk[1] : (tb == 2 ? h.tk[2] : h.tk[3]));
  };

  for (int unit = (int)blockIdx.x; unit < nr * nck; unit += G) {
    const int ck = unit % nck, rng = unit / nck;
    const int ta = rng * tpr, tz = min(live, ta + tpr);
    if (ta >= tz) continue;
    // chunk -> slice s and its first column in the slice
    int s = 0, cbase = 0, acc = 0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      if (k >= p.n_slices) break;
      if (ck >= acc) {
        s = k;
        cbase = acc;
      }
      acc += uniform_value(p.rows_nck[k]);
    }
    const int w = (int)pick<NS>(p.width, s, p.n_slices);
    const int col0 = (ck - cbase) * kRowsCols;
    const int64_t yo = pick<NS>(p.offset, s, p.n_slices) + col0 + 128 * wave;  // this wave's first column
    const int wcol = col0 + 128 * wave;                                      // ... in the slice
    const int64_t yrow = pick<NS>(p.offset, s, p.n_slices) + col0;          // the workgroup's first column
    const uint16_t *bslice = reinterpret_cast<const uint16_t *>(pick<NS>(p.B, s, p.n_slices));
    const int64_t bstride = pick<NS>(p.b_stride, s, p.n_slices);

    // the rank rows and y of token block tb of a tile into register set b.
    // Both go through buffer resources with 32-bit offsets: the four y
    // pieces of a lane share one row offset (the 64-byte steps are immediate
    // offsets), the low plane follows the high one; pieces past the slice
    // are read anyway (they are never stored) and reads past y return zeros
    const rsrc_t yr = make_rsrc(p.y, p.y_bytes);
    const rsrc_t ur = make_rsrc(p.uh, p.plane_bytes);
    u32x4 uhv[2][KS];
    u32x4 yv[2][4];
    auto row_off = [&](int64_t row) { return (uint32_t)((row * p.ldy + yo + 8 * kg) * 2); };
    // issued for every block slot, even past the tile's last block (then
    // every piece reads zeros): no load sits behind a branch, so the wait
    // before a block's products counts only the loads issued after it
    // (the register set is a compile-time constant: a runtime index would put
    // the sets in scratch memory)
    auto load_block = [&](const Header h, int tb, auto bc) __attribute__((always_inline)) {
      constexpr int b = decltype(bc)::value;
      const int rows = uniform_value(h.rows);
      const bool bv = 16 * tb < rows;                // the block exists
      const bool rv = 16 * tb + n < rows;
      const int64_t pos = uniform_value(h.pos0) + 16 * tb + (rv ? n : 0);
      // ranks 32 c + 8 kg .. + 7 of k-step c; ranks past R read zeros
      const uint32_t uo = bv ? (uint32_t)((((int64_t)s * T + pos) * R + 8 * kg) * 2) : kOut;
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        const uint32_t o = 32 * c + 8 * kg < R ? uo + 64 * c : kOut;
        uhv[b][c] = buf_load16(ur, o);
      }
      const uint32_t yo32 =
          p.add && bv ? row_off(rv ? (int64_t)tok_of(h, tb < 4 ? tb : 0) : (int64_t)h.tfirst) : kOut;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) yv[b][pp] = buf_load16(yr, yo32 + 64 * pp);
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    bf16x8 bt[KS][8];
    int cur = -2;      // slot whose chunk is in bt
    Header hd = read_header(ta);
    Header hn = hd;
    if (ta + 1 < tz) hn = read_header(ta + 1);
    // block 0 of every tile with an adapter is in flight in set 0 when the
    // tile starts: the previous tile (or this line, for the range's first)
    // issued it, so a workgroup's stream of blocks has no gap at tile
    // boundaries.  A header with rows = 0 issues only reads past the
    // resources.
    {
      Header h0 = hd;
      if (uniform_value(hd.slot) < 0) h0.rows = 0;
      load_block(h0, 0, S0{});
    }
    for (int ti = ta; ti < tz; ++ti) {
      const int slot = uniform_value(hd.slot), rows = uniform_value(hd.rows);
      const int nb = (rows + 15) / 16;
      Header hx = hn;  // the next tile's header, for its block 0
      if (ti + 1 >= tz || uniform_value(hn.slot) < 0) hx.rows = 0;
      if (slot < 0) {  // store mode, no adapter: the windows become 0
        for (int tb = 0; tb < nb; ++tb) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const int c = 32 * pp + 8 * kg;
            if (16 * tb + n < rows && wcol + c < w)
              gstore16(y + (int64_t)tok_of(hd, tb) * p.ldy + yo + c, u32x4{0, 0, 0, 0});
          }
        }
        load_block(hx, 0, S0{});
      } else {
        if (slot != cur) {
          // ---- the slot's chunk of B (rows j < RP, 512 columns) into LDS
          // straight from memory, one row per wave instruction (lane l's 16
          // bytes at 16 l; ranks past the slot's rank and columns past the
          // slice read as zeros), then this wave's B^T operands into
          // registers.  Block pair pp of the wave: columns 128 w + 32 pp +
          // 8 h + i (h, i < 4) go to block 2 pp (i < 4) and 2 pp + 1 (i + 4):
          // lane 4 e + h of a 16-lane group names 4 columns of rank row e, and
          // the transposing read hands lane m the column 8 (m / 4) + m % 4
          // (+ 4), so a lane's 8 outputs of the pair are 8 consecutive
          // columns of one token.
          const int rk = slot_rank_of(p.slot_rank, slot, p.ra);
          const rsrc_t br = make_rsrc(bslice + (int64_t)slot * bstride, (uint32_t)(p.ra * w * 2));
          const int c8 = col0 + 8 * lane;
          const int l = lane % 16;
          // one 32-rank step at a time through a 32-row LDS buffer
#pragma unroll
          for (int c = 0; c < KS; ++c) {
            __syncthreads();  // every wave has read the buffer's previous contents
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int jl = wave + 4 * jj, j = 32 * c + jl;
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  br, (__attribute__((address_space(3))) void *)(rows_lds + jl * kRowsLdb), 16,
                  (j < rk && c8 < w) ? (uint32_t)((j * w + c8) * 2) : kOut, 0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);  // loads return in order: these rows (and the block loads) are in
            __syncthreads();
            // 8 ranks a lane: two transposing reads, rank rows 8 kg .. + 3 and + 4 .. + 7
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              const uint16_t *a = rows_lds + (8 * kg + l / 4) * kRowsLdb + 128 * wave + 32 * (b / 2) + 8 * (l % 4) +
                                  4 * (b % 2);
              const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(a)));
              const u32x2 hi =
                  __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(a + 4 * kRowsLdb)));
              bt[c][b] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
            }
          }
          cur = slot;
          __syncthreads();  // every wave holds its operands before results reuse the buffer
        }
        // ---- token blocks, two per trip (register sets 0 and 1 named at
        // compile time; a runtime trip count keeps the compiler from hoisting
        // later blocks' loads): products, then y, 16 bytes per lane; the next
        // block's rank rows and y are in flight meanwhile
        auto compute = [&](int tb, auto bc) __attribute__((always_inline)) {
          constexpr int b = decltype(bc)::value;
          uint16_t *xb = rows_lds + (tb & 1) * 16 * kXchLdb;  // results of blocks of this parity
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KS; ++c) {
              const bf16x8 u8 = __builtin_bit_cast(bf16x8, uhv[b][c]);
              a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[c][2 * pp], u8, a0, 0, 0, 0);
              a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt[c][2 * pp + 1], u8, a1, 0, 0, 0);
            }
            const u32x4 old = yv[b][pp];
            u32x4 o;
            o[0] = pack_bf16x2(bf16_lo(old[0]) + a0[0], bf16_hi(old[0]) + a0[1]);
            o[1] = pack_bf16x2(bf16_lo(old[1]) + a0[2], bf16_hi(old[1]) + a0[3]);
            o[2] = pack_bf16x2(bf16_lo(old[2]) + a1[0], bf16_hi(old[2]) + a1[1]);
            o[3] = pack_bf16x2(bf16_lo(old[3]) + a1[2], bf16_hi(old[3]) + a1[3]);
            *reinterpret_cast<u32x4 *>(xb + n * kXchLdb + 128 * wave + 32 * pp + 8 * kg) = o;
          }
          // the block's 16 x 512 results meet in LDS, and each wave stores 4
          // whole rows of 1 KB, one row per instruction: y goes out in long
          // contiguous runs.  Rows past the tile and columns past the slice go
          // past the resource and are dropped (no store behind a branch).
          __syncthreads();
          const int tkb = tok_of(hd, tb);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = 4 * wave + rr;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(xb + r * kXchLdb + 8 * lane);
            const int64_t tok = __builtin_amdgcn_readlane(tkb, r);
            __builtin_amdgcn_raw_buffer_store_b128(
                v, yr, 16 * tb + r < rows && col0 + 8 * lane < w ? (uint32_t)((tok * p.ldy + yrow + 8 * lane) * 2) : kOut,
                0, 0);
          }
        };
        // an odd block count runs one more block of zeros (reads and stores
        // past the resources), so every tile ends in set 1 and the next
        // tile's block 0 goes to set 0
        for (int tb = 0; tb < nb; tb += 2) {
          load_block(hd, tb + 1, S1{});
          compute(tb, S0{});
          const bool last = tb + 2 >= nb;
          load_block(last ? hx : hd, last ? 0 : tb + 2, S0{});
          compute(tb + 1, S1{});
        }
      }
      hd = hn;
      if (ti + 2 < tz) hn = read_header(ti + 2);
    }
  }
}

// ------------------------------------------------------------------ host side

template <typename E, int R>
static hipError_t launch_t(const ExpandParams &p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((expand_kernel<E, R>), dim3(grid), dim3(kExpThreads), seg_table_bytes(p.meta.S),
                     stream, p);
  return hipGetLastError();
}

template <int R, int NS, bool BO>
static hipError_t launch_mma_ns(const ExpandParams &p0, int64_t bound, hipStream_t stream) {
  static std::atomic<int> resident[kMaxDevices];
  const int grid = xcd_grid(
      bound, resident_groups(resident, reinterpret_cast<const void *>(&expand_mma_kernel<R, NS, BO>), kXThreads, 0));
  ExpandParams p = p0;
  size_t words = 0;
  unsigned long long *clk = phase_clock_buffer(&words);
  p.clk = phase_clock_kernel() == 2 && (size_t)grid * kTilePhaseWords <= words ? clk : nullptr;
  hipLaunchKernelGGL((expand_mma_kernel<R, NS, BO>), dim3(grid), dim3(kXThreads), 0, stream, p.meta.info,
                     p.meta.tiles, p);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_mma_t(const ExpandParams &p, int64_t bound, bool b_out_rows, hipStream_t stream) {
  return with_slice_bound(p.n_slices, [&](auto ns) {
    constexpr int NS = decltype(ns)::value;
    return b_out_rows ? launch_mma_ns<R, NS, true>(p, bound, stream) : launch_mma_ns<R, NS, false>(p, bound, stream);
  });
}

// Long-segment expand, one instantiation (dynamic LDS: the B chunk).
template <int R, int NS>
static hipError_t launch_rows_ns(const ExpandParams &p, int64_t bound, hipStream_t stream) {
  static std::atomic<int> resident[kMaxDevices];
  constexpr size_t lds = (size_t)32 * kRowsLdb * 2;
  const void *fn = reinterpret_cast<const void *>(&expand_rows_kernel<R, NS>);
  if (lds > 65536) {  // more than the default dynamic LDS
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int grid = xcd_grid(bound, resident_groups(resident, fn, kXThreads, lds));
  hipLaunchKernelGGL((expand_rows_kernel<R, NS>), dim3(grid), dim3(kXThreads), lds, stream, p.meta.info,
                     p.meta.tiles, p);
  return hipGetLastError();
}

// The long-segment expand serves this call?  Whole tiles are likely when the
// batch has at least 64 tokens per possible segment.  LORA_EXPAND_ROWS=0 or 1
// forces the choice (tuning).
bool expand_rows_fits(int64_t T, int32_t S, bool bf16, int mode, int32_t R) {
  if (!bf16 || mode == 1 || R > 64) return false;  // rank 128 would not keep its B chunk in registers
  const int v = expand_rows_knob();
  if (v >= 0) return v == 1;
  return T >= 64 * ((int64_t)S + 1);
}

// y bytes a call's windows reach, and whether y and the u planes fit the
// long-segment expand's 32-bit buffer offsets (with room past their ends for
// the pieces it reads and never stores).
static int64_t rows_y_bytes(int64_t T, int32_t n_slices, const int64_t *width, const int64_t *offset, int64_t ldy) {
  int64_t y_end = 0;
  for (int s = 0; s < n_slices; ++s) y_end = std::max(y_end, offset[s] + width[s]);
  return ((T - 1) * ldy + y_end) * 2;
}
bool expand_rows_addressable(int64_t T, int32_t n_slices, const int64_t *width, const int64_t *offset, int64_t ldy,
                             int32_t R) {
  if (T == 0) return true;
  return rows_y_bytes(T, n_slices, width, offset, ldy) + 4096 < 0x7FFFFFF0LL &&
         (int64_t)n_slices * T * R * 2 < ((int64_t)1 << 30);
}

hipError_t launch_expand_rows(const MetaView &meta, const float *part, int kch, uint16_t *planes, int32_t n_slices,
                              const void *const *B, const int64_t *b_stride, const int64_t *width,
                              const int64_t *offset, int32_t R, int32_t ra, const int32_t *slot_rank, void *y,
                              int64_t ldy,
                              int add, hipStream_t stream) {
  const int64_t T = meta.T;
  if (T == 0) return hipSuccess;
  const int64_t plane = (int64_t)n_slices * T * R;
  {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((plane / 4 + 255) / 256, 2048));
    hipLaunchKernelGGL(u_planes_kernel, dim3(grid), dim3(256), 0, stream, meta.info, part, T, n_slices, R, kch,
                       planes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ExpandParams p{};
  p.meta = meta;
  p.n_slices = n_slices;
  p.uh = planes;
  p.ra = ra;
  p.u_ld = R;
  p.rows_nck_total = 0;
  for (int s = 0; s < n_slices; ++s) {
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
    p.rows_nck[s] = (int32_t)((width[s] + kRowsCols - 1) / kRowsCols);
    p.rows_nck_total += p.rows_nck[s];
  }
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  p.slot_rank = slot_rank;
  p.y_bytes = (uint32_t)rows_y_bytes(T, n_slices, width, offset, ldy);
  p.plane_bytes = (uint32_t)(plane * 2);
  // one workgroup per (tile range, chunk): as many as stay resident
  const int64_t bound = max_tiles(T, meta.S) * p.rows_nck_total;
  return with_slice_bound(n_slices, [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    switch (R) {
      case 8: return launch_rows_ns<8, NS>(p, bound, stream);
      case 16: return launch_rows_ns<16, NS>(p, bound, stream);
      case 32: return launch_rows_ns<32, NS>(p, bound, stream);
      case 64: return launch_rows_ns<64, NS>(p, bound, stream);
    }
    return hipErrorInvalidValue;
  });
}

// Matrix-core expand: the bf16 path of SGMV and AUTO (tile heights follow the
// segment lengths); the vector kernel serves fp32 and BGMV.
bool expand_uses_mma(bool bf16, int mode) { return bf16 && mode != 1; }

hipError_t launch_expand(const MetaView &meta, const float *u, int u_mode, int kch, int32_t n_slices,
                         const void *const *B, const int64_t *b_stride, const int64_t *width,
                         const int64_t *offset, int32_t R, int32_t ra, const int32_t *slot_rank, void *y,
                         int64_t ldy, bool bf16, int add, int mode, hipStream_t stream, bool b_out_rows) {
  ExpandParams p{};
  p.meta = meta;
  p.u = u;
  p.u_mode = u_mode;
  p.kch = kch;
  p.n_slices = n_slices;
  p.ra = ra;
  p.u_ld = ra;
  const int64_t e = bf16 ? 2 : 4;
  // rank 128: the vector kernel; B in the output-rows layout: the matrix-core
  // kernel only (the argument checks keep such calls to bf16, R <= 64 and
  // mode AUTO or SGMV)
  const bool mma = (expand_uses_mma(bf16, mode) && R <= 64) || b_out_rows;
  if (b_out_rows && !(bf16 && R <= 64)) return hipErrorInvalidValue;
  const int64_t T = meta.T, S = meta.S;
  for (int s = 0; s < n_slices; ++s) {
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
  }
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  p.slot_rank = slot_rank;
  if (T == 0) return hipSuccess;
  if (mma) {
    // the kernel sizes its items from the live tile count; the grid is at most
    // the workgroups that stay resident together, and no more than the items
    // could ever number
    p.steps_total = 0;
    for (int s = 0; s < kMaxSlices; ++s) {
      p.steps[s] = s < n_slices ? (int32_t)((width[s] + kXStep - 1) / kXStep) : 0;
      p.steps_total += p.steps[s];
    }
    p.nck_tab[0] = 0;
    for (int c = 1; c <= 16; ++c) {
      p.nck_tab[c] = 0;
      for (int s = 0; s < n_slices; ++s) p.nck_tab[c] += (p.steps[s] + c - 1) / c;
    }
    const int64_t bound = max_tiles(T, (int32_t)S) * p.steps_total;
    switch (R) {
      case 8: return launch_mma_t<8>(p, bound, b_out_rows, stream);
      case 16: return launch_mma_t<16>(p, bound, b_out_rows, stream);
      case 32: return launch_mma_t<32>(p, bound, b_out_rows, stream);
      case 64: return launch_mma_t<64>(p, bound, b_out_rows, stream);
    }
    return hipErrorInvalidValue;
  }
  // vector n-tile: up to 512 columns, as many as fit the shared B tile
  p.vec_cols = (int)std::min<int64_t>(512, kEVecLds / (R * e));
  p.ntiles_vec = 0;
  for (int s = 0; s < n_slices; ++s) p.ntiles_vec += (int32_t)((width[s] + p.vec_cols - 1) / p.vec_cols);
  const int64_t bound_vec = ((T + kEVecRows - 1) / kEVecRows + S + 1) * p.ntiles_vec;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(bound_vec, 4096));
  switch (R) {
    case 8: return bf16 ? launch_t<uint16_t, 8>(p, grid, stream) : launch_t<float, 8>(p, grid, stream);
    case 16: return bf16 ? launch_t<uint16_t, 16>(p, grid, stream) : launch_t<float, 16>(p, grid, stream);
    case 32: return bf16 ? launch_t<uint16_t, 32>(p, grid, stream) : launch_t<float, 32>(p, grid, stream);
    case 64: return bf16 ? launch_t<uint16_t, 64>(p, grid, stream) : launch_t<float, 64>(p, grid, stream);
    case 128: return bf16 ? launch_t<uint16_t, 128>(p, grid, stream) : launch_t<float, 128>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lora
