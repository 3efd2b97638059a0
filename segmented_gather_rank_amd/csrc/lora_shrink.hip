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

struct ShrinkParams {
  MetaView meta;
  const void *x;
  int64_t ldx, d_in;
  const void *A[kMaxSlices];
  int64_t a_stride[kMaxSlices];
  int32_t n_slices;
  float scale;
  const float *slot_scale;
  const int32_t *slot_rank;  // per-slot ranks, or null (every slot uses R)
  // kch == 1: out is u [n_slices][T][R], rows in token order, or in sorted-
  // position order when u_sorted is set; kch > 1: out holds the partial sums
  // [kch][n_slices][T][R] in sorted-position order
  float *out;
  int32_t u_sorted;
  int32_t kc, kch;       // k-chunk length (a multiple of 128) and count
  int32_t ra;            // the caller's r_max: A row stride, ranks read (ra <= R)
  int32_t u_ld;          // row stride of u written in token order (the caller's u: ra)
  int32_t a_rank_rows;   // A_s[slot] is [ra][d_in] (rank-major), not [d_in][ra]
  unsigned long long *clk;  // a measurement build's phase records, or null
};

struct ShrinkLds {
  float xs[kVecRows][kVecSub];
  float red[4][kVecRows][128];
};

// Store one result: into u (token or sorted order) when d_in is not split,
// else into the partial sums of k-chunk kc.
__device__ __forceinline__ void put(const ShrinkParams &p, int R, int s, int64_t pos, int j,
                                   int kc, float v) {
  const int64_t T = p.meta.T;
  if (p.kch == 1) {
    if (p.u_sorted) {
      p.out[((int64_t)s * T + pos) * R + j] = v;
    } else if (j < p.ra) {  // the caller's u: [n_slices][T][ra]
      p.out[((int64_t)s * T + p.meta.sorted[pos]) * p.u_ld + j] = v;
    }
  } else {
    p.out[(((int64_t)kc * p.n_slices + s) * T + pos) * R + j] = v;
  }
}

// Four consecutive ranks j..j+3 of one result row, as one 16-byte store.
__device__ __forceinline__ void put4(const ShrinkParams &p, int R, int s, int64_t pos, int j, int kc,
                                    f32x4 v) {
  const int64_t T = p.meta.T;
  float *dst;
  if (p.kch == 1) {
    if (p.u_sorted) {
      dst = p.out + ((int64_t)s * T + pos) * R + j;
    } else {
      if (j >= p.ra) return;  // the caller's u: [n_slices][T][ra] (ra and j multiples of 4)
      dst = p.out + ((int64_t)s * T + p.meta.sorted[pos]) * p.u_ld + j;
    }
  } else {
    dst = p.out + (((int64_t)kc * p.n_slices + s) * T + pos) * R + j;
  }
  gstore16f(dst, v);
}

// ------------------------------------------------------------------ vector path

template <typename E, int R>
__device__ __forceinline__ void vec_item(const ShrinkParams &p, ShrinkLds &lds, int slot, int64_t pos0,
                         int rows, int kc, float sc, int rk) {
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
                    (k0 + sub) * p.ra;
      // the first A batch goes out before the x rows are staged
      Raw8<E> a[VA];
#pragma unroll
      for (int q = 0; q < VA; ++q) {
        const int e = 8 * (tid + kShrinkThreads * q);
        if (e < nel && e % R < rk) a[q].load(Ab + packed_to_factor<R>(e, p.ra)); else a[q].zero();
      }
      if (staged != sub) {
        __syncthreads();  // earlier readers of xs are done
        const int oct = slen / 8;
        for (int idx = tid; idx < rows * oct; idx += kShrinkThreads) {
          const int row = idx / oct, c = idx - row * oct;
          const int64_t t = p.meta.sorted[pos0 + row];
          float v[8];
          load8(x + x_row_of(p.meta, t) * p.ldx + k0 + sub + 8 * c, v);
          *reinterpret_cast<f32x4 *>(&lds.xs[row][8 * c]) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4 *>(&lds.xs[row][8 * c + 4]) = f32x4{v[4], v[5], v[6], v[7]};
        }
        __syncthreads();
        staged = sub;
      }
      for (int base = 0; base < nel; base += 8 * kShrinkThreads * VA) {
        if (base > 0) {
#pragma unroll
          for (int q = 0; q < VA; ++q) {
            const int e = base + 8 * (tid + kShrinkThreads * q);
            if (e < nel && e % R < rk) a[q].load(Ab + packed_to_factor<R>(e, p.ra)); else a[q].zero();
          }
        }
#pragma unroll
        for (int q = 0; q < VA; ++q) {
          const int e = base + 8 * (tid + kShrinkThreads * q);
          if (e < nel) {
            const int k = e / R;
#pragma unroll
            for (int m = 0; m < kVecRows; ++m) {
              const float xv = lds.xs[m][k];  // rows >= `rows` are stale, never stored
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
        for (int i = 0; i < 8; ++i) lds.red[wave][m][8 * jo + i] = acc[m][i];
    }
    __syncthreads();
    for (int idx = tid; idx < rows * R; idx += kShrinkThreads) {
      const int mm = idx / R, j = idx % R;
      const float v = ((lds.red[0][mm][j] + lds.red[1][mm][j]) + lds.red[2][mm][j]) +
                      lds.red[3][mm][j];
      put(p, R, s, pos0 + mm, j, kc, v * sc);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- matrix-core path
//
// One item = (segment, tile of up to 64 sorted tokens, k-chunk of d_in), all
// slices' ranks as output columns, in passes of CB 16-column blocks.
// v_mfma_f32_16x16x32_bf16: the A operand is 8 consecutive x values of one
// token (straight from global memory), the B operand 8 k rows of one output
// column, read from the A tile in LDS with the gfx950 transposing read.
//
// Waves and tokens: a tile has nb = ceil(rows / 16) blocks of 16 tokens.  The
// 4 waves are spread over them, 4, 2 or 1 waves per block (wpt); the waves that
// share a block split the k-steps of every A tile between them, and their
// partial products are added in a fixed order in the epilogue.  So a tile of
// few tokens still has each wave load only its share of x, and an A batch can
// hold more tiles: A tiles (128 k rows) move in batches of up to NTB tiles
// (at most wpt), double-buffered in LDS: the next batch and its x fragments
// are loaded while the current one is multiplied, with one barrier per batch.
// The result goes out through LDS as 16-byte row pieces.

constexpr int kMThreads = 256;
constexpr int kMKT = 128;    // k rows per A tile

// LDS row stride (elements) of an A tile with CB column blocks: the 4 rows that
// one 16-lane transposing read touches fall in distinct banks
template <int CB> constexpr int kMLda = CB == 1 ? 16 : CB * 16 + 16;
// A tiles per batch at most (register and LDS budget)
template <int CB> constexpr int kMNtb = CB == 1 ? 4 : (CB == 2 ? 2 : 1);
// A rank-major A tile sits in LDS as CB * 16 rank rows of 128 k values, row
// stride kMLdk: 16 lanes reading 16 bytes of 16 consecutive rank rows fall in
// distinct banks (272 bytes apart)
constexpr int kMLdk = kMKT + 8;
template <int CB, bool RM> constexpr int kMTile = RM ? CB * 16 * kMLdk : kMKT * kMLda<CB>;

// RM: A is rank-major, [ra][d_in] per slot (the pages' A layout): a slot's
// ranks past its own are whole rows, never fetched.  The tile then goes to LDS
// as rank rows, and the MFMA reads 8 consecutive k of one rank with a plain
// 16-byte read instead of the transposing one.
template <int R, int CB, int NS, bool RM>
__global__ __launch_bounds__(kMThreads, 2) void shrink_mma_kernel(const int32_t *__restrict__ info,
                                                                  const int32_t *__restrict__ tiles,
                                                                  ShrinkParams p) {
  constexpr int SG = CB * 16 / R;   // slices per pass
  constexpr int QS = R / 16;        // octets of one slice per thread per tile
  constexpr int LDA = kMLda<CB>;
  constexpr int NTB = kMNtb<CB>;
  constexpr int TILE = kMTile<CB, RM>;
  static_assert(SG >= 1 && SG * QS == CB, "column blocks hold whole slices");
  __shared__ uint16_t at[2][NTB * TILE];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int mrow = lane % 16, kg = lane / 16;
  // live tiles: the tile list is in key order, so the tiles of tokens without
  // an adapter come first and are skipped.  Items (k-chunk, live tile),
  // chunk-major, so the tiles of one segment that share an A chunk are
  // neighbours; XCD x (blockIdx mod 8) takes a contiguous run of items, and
  // those tiles meet in one L2
  const int ntl = uniform_value(info[4]);
  const int t0 = (uniform_value(info[3]) + kTileRows - 1) / kTileRows;
  const int live = ntl - t0;
  if (live <= 0) return;
  const int total = live * p.kch;
  const int run = (total + 7) / 8;
  const int xcd = blockIdx.x % 8, per = gridDim.x / 8;
  const int hi = min(total, xcd * run + run);
  int item = xcd * run + (int)blockIdx.x / 8;
  // measurement build: 0 start, 1 + 2n / 2 + 2n start and end of item n < 6,
  // 13 items, 14 the last item's rows, 15 end (stores acknowledged)
  unsigned long long *const rec = phase_record(p.clk);
  phase_stamp(rec, 0);
  int nit = 0;
  if (item >= hi) return;
  const uint16_t *x = reinterpret_cast<const uint16_t *>(p.x);
  float *red = reinterpret_cast<float *>(&at[0][0]);  // [64 rows][CB * 16] after the k loop

  // tile header, and this lane's token for each possible spread of waves over
  // token blocks (which one applies depends on rows); the next item's header
  // is loaded while the current item runs
  struct Header {
    int slot, rows, pos0, tk1, tk2, tk4, tfirst;
  };
  auto read_header = [&](int it) {
    const int32_t *tl = tiles + (int64_t)(t0 + it % live) * kTileInts;
    return Header{tl[0], tl[1], tl[2], tl[4 + 16 * wave + mrow], tl[4 + 16 * (wave / 2) + mrow], tl[4 + mrow],
                  tl[4]};
  };
  Header hnext = read_header(item);

  for (; item < hi; item += per) {
    if (nit < 6) phase_stamp(rec, 1 + 2 * nit);
    const int kc = item / live;
    const Header hd = hnext;
    if (item + per < hi) hnext = read_header(item + per);
    const int slot = uniform_value(hd.slot), rows = uniform_value(hd.rows);
    const int64_t pos0 = uniform_value(hd.pos0);
    if (slot < 0) continue;  // (never: live tiles hold adapter tokens)
    const int64_t kbeg = (int64_t)kc * p.kc;
    const int64_t kend = min(p.d_in, kbeg + p.kc);
    const int ntiles = (int)((kend - kbeg + kMKT - 1) / kMKT);
    const int nb = (rows + 15) / 16;
    const int wpt = nb == 1 ? 4 : (nb == 2 ? 2 : 1);  // waves per token block
    const int tb = wave / wpt, kq = wave % wpt;       // token block, k-step share
    const int fpt = 4 / wpt;                          // k-steps (x fragments) per tile and wave
    const int ntb = min(NTB, wpt);                    // A tiles per batch
    const int nbatch = (ntiles + ntb - 1) / ntb;
    const int r = 16 * tb + mrow;                     // this lane's row of the tile
    const bool rv = tb < nb && r < rows;
    const int64_t trow = rv ? (int64_t)(wpt == 4 ? hd.tk4 : (wpt == 2 ? hd.tk2 : hd.tk1)) : (int64_t)hd.tfirst;
    const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
    const int rk = slot_rank_of(p.slot_rank, slot, p.ra);  // ranks past rk are not read
    const uint16_t *xrow = x + x_row_of(p.meta, trow) * p.ldx;

    for (int s0 = 0; s0 < p.n_slices; s0 += SG) {
      const int ns = min(SG, p.n_slices - s0);
      rsrc_t ar[SG];
#pragma unroll
      for (int g = 0; g < SG; ++g) {
        const int sidx = s0 + (g < ns ? g : 0);
        ar[g] = make_rsrc(reinterpret_cast<const uint16_t *>(pick<NS>(p.A, sidx, p.n_slices)) +
                              (int64_t)slot * pick<NS>(p.a_stride, sidx, p.n_slices),
                          (uint32_t)(p.d_in * p.ra * 2));
      }
      // A octet q = t * CB + sl * QS + qq of this thread: tile t of the
      // batch, slice sl, flat element 8 (tid + 256 qq) of that slice's
      // [128][R] block (rank-major: of its [R][128] block); rows past the
      // k-chunk, ranks past the slot's rank and slices past n_slices read
      // zeros, tiles past the chunk are not loaded
      u32x4 aq[NTB * CB];
      auto load_a = [&](int bi) {
#pragma unroll
        for (int t = 0; t < NTB; ++t) {
          const int it = bi * ntb + t;
          if (t < ntb && it < ntiles) {
            const int64_t k0 = kbeg + (int64_t)it * kMKT;
#pragma unroll
            for (int q = 0; q < CB; ++q) {
              const int sl = q / QS, e = 8 * (tid + kMThreads * (q % QS));
              if constexpr (RM) {
                const int j = e / kMKT, k = e % kMKT;
                const bool ok = sl < ns && k0 + k < kend && j < rk;
                aq[t * CB + q] = buf_load16(ar[sl], ok ? (uint32_t)(((int64_t)j * p.d_in + k0 + k) * 2) : 0x7FFFFFF0u);
              } else {
                const int k = e / R, j0 = e % R;
                const bool ok = sl < ns && k0 + k < kend && j0 < rk;
                aq[t * CB + q] = buf_load16(ar[sl], ok ? (uint32_t)(((k0 + k) * p.ra + j0) * 2) : 0x7FFFFFF0u);
              }
            }
          }
        }
      };
      auto store_a = [&](int buf, int bi) {
#pragma unroll
        for (int t = 0; t < NTB; ++t) {
          if (t < ntb && bi * ntb + t < ntiles) {
#pragma unroll
            for (int q = 0; q < CB; ++q) {
              const int sl = q / QS, e = 8 * (tid + kMThreads * (q % QS));
              if constexpr (RM)
                *reinterpret_cast<u32x4 *>(&at[buf][t * TILE + (sl * R + e / kMKT) * kMLdk + e % kMKT]) =
                    aq[t * CB + q];
              else
                *reinterpret_cast<u32x4 *>(&at[buf][(t * kMKT + e / R) * LDA + sl * R + e % R]) = aq[t * CB + q];
            }
          }
        }
      };
      // x fragment m of a batch: tile m / fpt, k-step wpt (m % fpt) + kq of
      // that tile, lane k offset 32 (k-step) + 8 kg.  Past the chunk a lane
      // reads a valid element of its row instead: those products meet zero A
      // rows.  Rows that are not ours are never stored.
      u32x4 xf[4];
      auto frag_ok = [&](int bi, int m) { return m < ntb * fpt && bi * ntb + m / fpt < ntiles; };
      auto load_x = [&](int bi) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (frag_ok(bi, m)) {
            const int it = bi * ntb + m / fpt, i = wpt * (m % fpt) + kq;
            const int64_t k = kbeg + (int64_t)it * kMKT + 32 * i + 8 * kg;
            xf[m] = gload16(xrow + (k < kend ? k : kbeg));
          }
        }
      };

      f32x4 acc[CB];
#pragma unroll
      for (int b = 0; b < CB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      load_a(0);
      load_x(0);
      __syncthreads();  // earlier readers of both buffers are done
      store_a(0, 0);
      __syncthreads();
      for (int bi = 0; bi < nbatch; ++bi) {
        u32x4 xc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) xc[m] = xf[m];
        const bool more = bi + 1 < nbatch;
        if (more) {
          load_a(bi + 1);
          load_x(bi + 1);
        }
        const uint16_t *a_b = at[bi & 1];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (frag_ok(bi, m)) {
            const int t = m / fpt, i = wpt * (m % fpt) + kq;
            const bf16x8 xa = __builtin_bit_cast(bf16x8, xc[m]);
#pragma unroll
            for (int b = 0; b < CB; ++b) {
              bf16x8 bv;
              if constexpr (RM)
                bv = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(a_b + t * TILE + (16 * b + mrow) * kMLdk + 32 * i + 8 * kg));
              else
                bv = lds_col8(a_b + t * TILE, LDA, 32 * i + 8 * kg, 16 * b);
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bv, acc[b], 0, 0, 0);
            }
          }
        }
        if (more) store_a((bi + 1) & 1, bi + 1);
        __syncthreads();
      }
      // epilogue through LDS: acc[b][v] = this wave's share of
      // C[16 tb + 4 kg + v][16 b + mrow], at red row 16 wave + 4 kg + v; the
      // shares of a token block are added in wave order, then whole row pieces
      // of 4 ranks are written with 16-byte stores
#pragma unroll
      for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(16 * wave + 4 * kg + v) * (CB * 16) + 16 * b + mrow] = acc[b][v];
      __syncthreads();
      const int C4 = ns * R / 4;
      for (int idx = tid; idx < rows * C4; idx += kMThreads) {
        const int r_ = idx / C4, n4 = 4 * (idx - r_ * C4);
        const int row0 = 16 * ((r_ / 16) * wpt) + r_ % 16;  // red row of share 0
        f32x4 v = *reinterpret_cast<const f32x4 *>(&red[row0 * (CB * 16) + n4]);
        for (int q = 1; q < wpt; ++q) {
          const f32x4 w = *reinterpret_cast<const f32x4 *>(&red[(row0 + 16 * q) * (CB * 16) + n4]);
          v = f32x4{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
        }
        put4(p, R, s0 + n4 / R, pos0 + r_, n4 % R, kc, f32x4{v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc});
      }
    }
    if (nit < 6) phase_stamp(rec, 2 + 2 * nit);
    phase_put(rec, 14, (unsigned long long)rows);
    ++nit;
  }
  if constexpr (kPhaseClock) {
    phase_put(rec, 13, (unsigned long long)nit);
    if (rec) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      phase_stamp(rec, 15);
    }
  }
}

// ------------------------------------------------------------------ the kernels

template <typename E, int R>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
  __shared__ ShrinkLds lds;
  extern __shared__ __align__(16) unsigned char shrink_dyn[];
  const SegTable tb = seg_table_at(shrink_dyn, p.meta.S);
  build_items(p.meta, tb, true, [&](int c, int) { return ((c + kVecRows - 1) / kVecRows) * p.kch; });
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
    const int64_t pos0 = (int64_t)tb.start[seg] + (int64_t)chunk * kVecRows;
    vec_item<E, R>(p, lds, slot, pos0, min(kVecRows, count - chunk * kVecRows), kc, sc,
                   slot_rank_of(p.slot_rank, slot, p.ra));
  }
}

// u[s][sorted[pos]][:] = sum over k-chunks, in order, of the partial sums at pos,
// for every sorted position of a token with an adapter.
__global__ __launch_bounds__(256) void shrink_reduce_kernel(MetaView meta, const float *partial,
                                                            float *u, int32_t n_slices, int32_t R,
                                                            int32_t kch, int32_t ra) {
  const int64_t T = meta.T;
  const int64_t begin = meta.info[3];
  const int64_t q_per_row = ra / 4;  // the caller's u holds ranks < ra, row stride ra
  const int64_t total = (T - begin) * n_slices * q_per_row;
  const int64_t plane = (int64_t)n_slices * T * R;
  for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int64_t q = idx % q_per_row;
    const int64_t rest = idx / q_per_row;
    const int64_t pos = begin + rest % (T - begin);
    const int64_t s = rest / (T - begin);
    const float *src = partial + (s * T + pos) * R + 4 * q;
    const f32x4 v = sum_partials4(src, plane, kch);
    const int64_t t = meta.sorted[pos];
    *reinterpret_cast<f32x4 *>(u + (s * T + t) * ra + 4 * q) = v;
  }
}

// ------------------------------------------------------------------ host side

// Matrix-core shrink: the bf16 path of SGMV and AUTO for r >= 16 (tile heights
// follow the segment lengths); the vector kernel serves fp32, r = 8 and BGMV.
static bool shrink_uses_mma(bool bf16, int32_t R, int mode) { return bf16 && R >= 16 && mode != 1; }

// Chunking chosen from host-known sizes only (no device read), so a call
// never synchronises: split d_in so that there are about 1024 items.
ShrinkConfig plan_shrink(int64_t T, int32_t S, int64_t d_in, int32_t R, bool bf16, int mode) {
  ShrinkConfig c{};
  c.use_mma_mode = shrink_uses_mma(bf16, R, mode) ? 1 : 0;
  const int64_t chunks = c.use_mma_mode ? max_tiles(T, S) : (T + kVecRows - 1) / kVecRows + S;
  const int64_t tiles = (d_in + kMKT - 1) / kMKT;
  // matrix-core path: about 1024 items, or 2048 when the tiles are short
  // (fewer than 32 tokens on average: an item's time is then mostly its A
  // chunk, and smaller items even out the workgroups' finishing times); at
  // most 8 k-chunks, so that the expand adds the partial sums with one batch
  // of loads
  const bool short_tiles = T < 32 * chunks;
  const int64_t target = c.use_mma_mode ? (short_tiles ? 2048 : 1024) : 512;
  const int64_t cap = c.use_mma_mode ? 8 : tiles;
  const int64_t want = std::max<int64_t>(1, std::min<int64_t>(std::min(tiles, cap), (target + chunks - 1) / chunks));
  c.kc = (int)(((tiles + want - 1) / want) * kMKT);
  c.kch = (int)((d_in + c.kc - 1) / c.kc);
  c.bound = chunks * c.kch;
  c.grid = (int)std::max<int64_t>(1, std::min<int64_t>(c.bound, 2048));  // vector kernel
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

template <int R, int CB, int NS, bool RM>
static hipError_t launch_mma_ns(const ShrinkParams &p0, int64_t bound, hipStream_t stream) {
  static std::atomic<int> resident[kMaxDevices];
  const int grid = xcd_grid(bound, resident_groups(resident,
                                                   reinterpret_cast<const void *>(&shrink_mma_kernel<R, CB, NS, RM>),
                                                   kMThreads, 0));
  ShrinkParams p = p0;
  size_t words = 0;
  unsigned long long *clk = phase_clock_buffer(&words);
  p.clk = phase_clock_kernel() == 1 && (size_t)grid * kTilePhaseWords <= words ? clk : nullptr;
  hipLaunchKernelGGL((shrink_mma_kernel<R, CB, NS, RM>), dim3(grid), dim3(kMThreads), 0, stream, p.meta.info,
                     p.meta.tiles, p);
  return hipGetLastError();
}

template <int R, int CB>
static hipError_t launch_mma_t(const ShrinkParams &p, int64_t bound, hipStream_t stream) {
  return with_slice_bound(p.n_slices, [&](auto ns) {
    constexpr int NS = decltype(ns)::value;
    return p.a_rank_rows ? launch_mma_ns<R, CB, NS, true>(p, bound, stream)
                         : launch_mma_ns<R, CB, NS, false>(p, bound, stream);
  });
}

// column blocks per pass: the smallest power of two covering every slice's
// ranks, at most 8 (whole slices per pass)
static int mma_col_blocks(int32_t n_slices, int32_t R) {
  int cb = R / 16;
  while (cb < 8 && cb * 16 < n_slices * R) cb *= 2;
  return cb;
}

hipError_t launch_shrink(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, bool bf16,
                         int32_t n_slices, const void *const *A, const int64_t *a_stride,
                         int32_t R, int32_t ra, float scale, const float *slot_scale, const int32_t *slot_rank,
                         float *u, int mode, void *ws, bool for_apply, int *kch_out, hipStream_t stream,
                         bool to_partials, bool a_rank_rows) {
  const ShrinkConfig c = plan_shrink(meta.T, meta.S, d_in, R, bf16, mode);
  if (a_rank_rows && !c.use_mma_mode) return hipErrorInvalidValue;  // the caller checks the layout's limits
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
  p.slot_rank = slot_rank;
  p.out = c.kch == 1 && !to_partials ? u : reinterpret_cast<float *>(ws);
  p.u_sorted = for_apply ? 1 : 0;
  p.kc = c.kc;
  p.kch = c.kch;
  p.ra = ra;
  p.u_ld = ra;
  p.a_rank_rows = a_rank_rows ? 1 : 0;
  if (meta.T == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
  if (c.use_mma_mode) {
    const int cb = mma_col_blocks(n_slices, R);
    switch (R * 16 + cb) {
      case 16 * 16 + 1: e = launch_mma_t<16, 1>(p, c.bound, stream); break;
      case 16 * 16 + 2: e = launch_mma_t<16, 2>(p, c.bound, stream); break;
      case 16 * 16 + 4: e = launch_mma_t<16, 4>(p, c.bound, stream); break;
      case 16 * 16 + 8: e = launch_mma_t<16, 8>(p, c.bound, stream); break;
      case 32 * 16 + 2: e = launch_mma_t<32, 2>(p, c.bound, stream); break;
      case 32 * 16 + 4: e = launch_mma_t<32, 4>(p, c.bound, stream); break;
      case 32 * 16 + 8: e = launch_mma_t<32, 8>(p, c.bound, stream); break;
      case 64 * 16 + 4: e = launch_mma_t<64, 4>(p, c.bound, stream); break;
      case 64 * 16 + 8: e = launch_mma_t<64, 8>(p, c.bound, stream); break;
      case 128 * 16 + 8: e = launch_mma_t<128, 8>(p, c.bound, stream); break;
    }
  } else {
    switch (R) {
      case 8: e = bf16 ? launch_t<uint16_t, 8>(p, c.grid, stream) : launch_t<float, 8>(p, c.grid, stream); break;
      case 16: e = bf16 ? launch_t<uint16_t, 16>(p, c.grid, stream) : launch_t<float, 16>(p, c.grid, stream); break;
      case 32: e = bf16 ? launch_t<uint16_t, 32>(p, c.grid, stream) : launch_t<float, 32>(p, c.grid, stream); break;
      case 64: e = bf16 ? launch_t<uint16_t, 64>(p, c.grid, stream) : launch_t<float, 64>(p, c.grid, stream); break;
      case 128: e = bf16 ? launch_t<uint16_t, 128>(p, c.grid, stream) : launch_t<float, 128>(p, c.grid, stream); break;
    }
  }
  // lora_apply's expand reads the partial sums itself; lora_shrink must hand
  // back a finished u
  if (e != hipSuccess || c.kch == 1 || for_apply) return e;
  const int64_t work = meta.T * n_slices * (ra / 4);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 1024));
  hipLaunchKernelGGL(shrink_reduce_kernel, dim3(grid), dim3(256), 0, stream, meta,
                     reinterpret_cast<const float *>(ws), u, n_slices, R, c.kch, ra);
  return hipGetLastError();
}

}  // namespace lora
