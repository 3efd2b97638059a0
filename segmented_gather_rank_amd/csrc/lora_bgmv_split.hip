// lora_bgmv_split.hip -- the fused decode kernel with each work tile spread
// over G workgroups: y[t][window_s] (+)= (scale_a * x[t] . A_s[a]) . B_s[a]
// for the tokens t of one tile (one slot a, up to 64 tokens).
//
// Page "多 LoRA 服务：分段矩阵乘与适配器调度", section "不合并权重，批量计算":
// the batched form gathers each token's adapter and fuses the gather with the
// two products; page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩
// GEMM:shrink、expand 与 fp32 中转缓冲": the rank-r intermediate stays fp32 and
// each output window is rounded once.  Page "多 LoRA 服务：分段矩阵乘与适配器调度",
// section "分段矩阵乘 SGMV": the tokens of one adapter form a segment and share
// one read of that adapter's factors.
//
// Why split a tile: one workgroup per token (or per tile) pulls the slot's
// whole A and B through one CU, and a CU's load rate, not HBM, then bounds the
// call.  Here member g of G (G workgroups per tile, all on the XCD the
// dispatcher picks for blockIdx mod 8) owns
//   * k rows [g kc, (g + 1) kc) of every slice's A: the partial rank-r rows of
//     the tile's tokens over that chunk (v_mfma_f32_16x16x32_bf16, x straight
//     from global memory, the A chunk read transposed from LDS), and
//   * 16-column blocks [g bpm, (g + 1) bpm) of the concatenated slices: the
//     expand D'[col][token] = B^T u^T (v_mfma_f32_16x16x16_bf16, u split into
//     bf16 hi + lo parts) and the read-modify-write of those y columns.
// The members exchange the partial rank rows through the L2 of their XCD.
// Workgroups go to the XCDs in turn (blockIdx mod 8 names the XCD) and a
// tile's members share that residue.  Each member stores its fragments with
// plain 16-byte stores (the write-through L1 passes them to L2), waits until
// L2 has acknowledged them, and raises its own flag word of the tile the same
// way; the others read both with agent-coherent loads, which skip L1.
// (Agent-coherent stores also go on to memory: twice the acknowledgement time,
// and a flag took about 0.9 us instead of 0.2 us to reach a peer.)  Once every
// member's flag is up, the G partial fragments are added in one fixed order
// (each wave a quarter of the members, then the four sums in wave order
// through LDS), so every member gets the same u, bit for bit.
//
// The flag words live at the start of the caller's apply workspace, so calls
// with workspaces of their own share nothing.  A word counts the calls that
// raised it and names the XCD (hardware register XCC_ID) of the member that
// raised it last.  Each call raises each of a tile's 16 words exactly once
// (member 0 also raises the words of members >= G), so the words of a range
// stay equal between calls, and a member waits for "my count + 1".  A member
// trusts a peer's word only when it names its own XCD: plain stores stay in
// the L2 of the XCD that made them until that L2 writes them back, in any
// order, so a flag seen from another XCD (evicted early, say) does not prove
// that the fragments it guards are visible here.  The B chunk is loaded with
// the A chunk and x, and so is the y of the first 16 rows except with the
// longest chunks, so that none of them is outstanding at the acknowledgement
// wait or the polls (loads complete in order).  The wait is bounded.  A
// member computes itself, with the same code (so the same bits), the partials
// of every peer it does not trust: still low at the spin limit, or raised from
// another XCD.  It stores them into those peers' slots, where the peer writes
// equal values, and reads them back through its own L2.  The result therefore
// depends neither on the members being resident together nor on their sharing
// an XCD: a member placed elsewhere costs the spin limit and is counted (a
// status word beside the flags), never a wrong value.  Workgroups are
// dispatched in order on each XCD and a tile's members are neighbours there,
// so the tiles within the resident part of a larger grid finish and make room
// for the rest.
//
// Only bf16.
#include "lora_host.h"

namespace lora {

constexpr int kSThreads = 256;
constexpr int kSBatch = 8;               // 16-byte loads per thread and operand, first batch
constexpr int kSPieces = kSThreads * kSBatch;  // A (and B) pieces of 16 bytes per member, at most
constexpr int kSMaxBpm = 32;             // 16-column blocks per member (8 per wave)

struct SplitParams {
  const void *x;
  int64_t ldx, d_in;
  int32_t x_row_div;
  int32_t n_slices;
  const void *A[kMaxSlices];
  int64_t a_stride[kMaxSlices];
  const void *B[kMaxSlices];
  int64_t b_stride[kMaxSlices];
  int64_t width[kMaxSlices];
  int64_t offset[kMaxSlices];
  int32_t blk_base[kMaxSlices + 1];  // prefix of 16-column blocks per slice
  int32_t gsh;                       // log2 G
  int32_t ksh;                       // log2 kc (kc >= 128)
  int32_t bpm;                       // 16-column blocks per member
  int32_t ldb;                       // row stride of the B chunk in LDS (elements)
  int32_t bs_off;                    // LDS byte offset of the B chunk (after the A chunk)
  int32_t max_tiles;
  int32_t n_frag;                    // 16-row fragments per member plane
  int32_t spin_limit;
  uint32_t part_bytes;
  float scale;
  const float *slot_scale;
  const int32_t *slot_rank;
  void *y;
  int64_t ldy;
  int32_t add;
  float *part;  // partial fragments [G][n_frag][n_slices][R16 blocks][64 lanes][4]
  uint32_t *sync;  // rendezvous words (host side only: the kernels take them as an argument)
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Zero the member's columns of the tile's rows (store mode, no adapter).
__device__ __forceinline__ void split_zero(const SplitParams &p, const int32_t *tl, int rows, int gb0, int nbm) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int row = wave; row < rows; row += kSThreads / kWave) {
    uint16_t *yr = reinterpret_cast<uint16_t *>(p.y) + (int64_t)tl[4 + row] * p.ldy;
    for (int h = lane; h < 2 * nbm; h += kWave) {
      const int gb = gb0 + h / 2;
      const int s = last_le(p.blk_base, p.n_slices, gb);
      const int64_t col = 16 * (int64_t)(gb - p.blk_base[s]) + 8 * (h & 1);
      if (col < p.width[s]) gstore16(yr + p.offset[s] + col, u32x4{0, 0, 0, 0});
    }
  }
}

// XCD this workgroup runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u; }

// Raise this member's flag word of the tile (member 0 also those of members
// >= G) to the next call count, tagged with this workgroup's XCD, then wait
// until the G members' words carry that count: one wave, at most spin_limit
// polls.  A peer's word is trusted only when its tag names this XCD: flags and
// the partial fragments they guard are stored with plain stores, which stay in
// the L2 of the XCD that made them until that L2 writes them back, so only a
// peer on this XCD is known to have its fragments where this workgroup reads
// them.  Returns the members (bit g') whose partials this workgroup computes
// itself: those still low when it gave up, and those raised from another XCD.
// status[0] counts waits that gave up, status[1] waits that met a word raised
// on another XCD.
__device__ __forceinline__ uint32_t split_wait(uint32_t *fl, uint32_t f, int g, int G, int spin_limit,
                                               uint32_t xcc, uint32_t *status) {
  const int lane = threadIdx.x % kWave;
  const uint32_t want = (f & ~15u) + 16u;  // this call's count, in bits 31:4
  if (lane < kSplitMembers && (lane == g || (g == 0 && lane >= G)))
    __builtin_amdgcn_raw_buffer_store_b32(want | xcc, make_rsrc(fl, kSplitMembers * 4), lane * 4, 0, 0);
  for (int polls = 0;; ++polls) {
    const uint32_t v =
        lane < G ? __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : (want | xcc);
    const bool up = (int32_t)((v & ~15u) - want) >= 0;
    const uint64_t low = __ballot(!up);
    if (low == 0 || polls >= spin_limit) {
      const uint64_t foreign = __ballot(up && (v & 15u) != xcc);
      if (lane == 0) {
        if (low) atomicAdd(status, 1u);
        if (foreign) atomicAdd(status + 1, 1u);
      }
      return (uint32_t)(low | foreign);
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The NF fragments u[i] = sum over the G members gm of the partial fragment
// at off[i] + gm * plane, shared by the 4 waves: wave w loads members
// w MG .. w MG + MG - 1 (agent-coherent loads, all issued before the first is
// used; members past G read as zeros), adds them in member order and leaves
// its sums in LDS; then every wave adds the 4 waves' sums in wave order.  The
// additions run in one fixed order for every member of a tile, so all of them
// get the same bits, and each fragment crosses from L2 once per workgroup, not
// once per wave.  Only the first nf fragments are gathered (the others come
// out as zeros).  At most 16 loads a lane are in flight (64 registers): more
// fragments go in chunks.  stage: nf * 4 * 64 f32x4 of LDS that no wave uses
// on entry; it is read until every wave has its u, so the caller passes a
// barrier before writing it again.
template <int MG, int NF>
__device__ __forceinline__ void gather_waves(rsrc_t pr, const uint32_t (&off)[NF], uint32_t plane, int G, int nf,
                                             f32x4 *stage, f32x4 (&u)[NF]) {
  constexpr int FC = 16 / MG < NF ? 16 / MG : NF;  // fragments per chunk
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int f0 = 0; f0 < NF; f0 += FC) {
    f32x4 v[FC][MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      const int gm = wave * MG + i;
#pragma unroll
      for (int f = 0; f < FC; ++f)
        v[f][i] = f0 + f < NF ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              pr, gm < G ? off[f0 + f] + gm * plane : 0x7FFFFFF0u, 0, 16))
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      f32x4 w = v[f][0];
#pragma unroll
      for (int i = 1; i < MG; ++i) w += v[f][i];
      if (f0 + f < nf) stage[((f0 + f) * 4 + wave) * kWave + lane] = w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const f32x4 *st = stage + f * 4 * kWave + lane;
    u[f] = f < nf ? ((st[0] + st[kWave]) + st[2 * kWave]) + st[3 * kWave] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// gather_waves with the members per wave the member count G = 2^gsh needs
template <int NF>
__device__ __forceinline__ void gather_members(rsrc_t pr, const uint32_t (&off)[NF], uint32_t plane, int gsh, int nf,
                                               f32x4 *stage, f32x4 (&u)[NF]) {
  switch (gsh) {
    case 0:
    case 1:
    case 2: gather_waves<1, NF>(pr, off, plane, 1 << gsh, nf, stage, u); break;
    case 3: gather_waves<2, NF>(pr, off, plane, 8, nf, stage, u); break;
    default: gather_waves<4, NF>(pr, off, plane, 16, nf, stage, u); break;
  }
}

template <int R, int NS>
__global__ __launch_bounds__(kSThreads, 2) void bgmv_split_kernel(const int32_t *__restrict__ info,
                                                               const int32_t *__restrict__ tiles,
                                                               uint32_t *__restrict__ flags, SplitParams p) {
  constexpr int RP = R < 16 ? 16 : R;       // ranks padded to 16-wide MFMA blocks
  constexpr int RB = RP / 16;
  constexpr int PR = RP / 8;                // 16-byte pieces per A row
  constexpr int LPR = PR == 2 ? 1 : (PR == 4 ? 2 : 3);
  constexpr int LDA = RP == 64 ? 80 : RP;   // A chunk row stride: conflict-free transposing reads
  constexpr int XB = 16;                    // k-steps of 32 per member, at most (kc <= 512)
  constexpr int QB = kSMaxBpm / 4;          // column blocks per wave, at most
  extern __shared__ __align__(16) unsigned char split_lds[];
  uint16_t *const As = reinterpret_cast<uint16_t *>(split_lds);
  uint16_t *const Bs = reinterpret_cast<uint16_t *>(split_lds + p.bs_off);

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l16 = lane % 16, kg = lane / 16;
  const int G = 1 << p.gsh;
  const int lb8 = blockIdx.x >> 3;
  const int g = lb8 & (G - 1);
  const int ti = ((lb8 >> p.gsh) << 3) | (blockIdx.x & 7);
  if (ti >= p.max_tiles) return;

  // ---- first round trip: tile count, tile header, the tokens of the four
  // 16-row blocks this lane may serve, and this member's flag
  const int32_t *tl = tiles + (int64_t)ti * kTileInts;
  const int ntiles = info[4];
  const int slot = tl[0], rows = tl[1], pos0 = tl[2];
  int tok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) tok[q] = tl[4 + 16 * q + l16];
  uint32_t *fl = flags + (int64_t)ti * kSplitFlagWords;  // the first range
  const uint32_t f = __builtin_amdgcn_readfirstlane(__hip_atomic_load(fl + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (ti >= ntiles) return;
  const int gb0 = g * p.bpm;
  const int nbm = min(p.bpm, p.blk_base[p.n_slices] - gb0);  // this member's blocks (may be <= 0)
  if (slot < 0) {  // no adapter: nothing to add, or windows to clear
    if (!p.add) split_zero(p, tl, rows, gb0, nbm);
    return;
  }

  // ---- second round trip: every load of the first batch (A chunk, x
  // fragments of this wave's token block, B chunk, y of the first 16 rows),
  // then the slot's rank and scale
  const int kc = 1 << p.ksh, nsteps = kc >> 5;
  const int nb = (rows + 15) >> 4;  // 16-row token blocks: wave t takes block t in the shrink
  const int pa = p.n_slices << (p.ksh + LPR);  // A pieces: n_slices * kc * PR
  // pieces outside the chunk read the slot's first row and are stored as
  // zeros (aok); loaded values are never selected, so no load sits in a branch
  u32x4 av[kSBatch];
  uint32_t aok = 0;
  auto load_a = [&](int gm) {  // member gm's A chunk of every slice
    const int64_t k0 = (int64_t)gm << p.ksh;
    aok = 0;
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      const int q = tid + kSThreads * i;
      const int s = q >> (p.ksh + LPR);
      const int rem = q & ((kc * PR) - 1);
      const int row = rem / PR, c8 = rem % PR;
      const bool ok = q < pa && k0 + row < p.d_in && 8 * c8 < R;
      aok |= (uint32_t)ok << i;
      const int ss = ok ? s : 0;
      const uint16_t *ptr = reinterpret_cast<const uint16_t *>(pick<NS>(p.A, ss, p.n_slices)) +
                            (int64_t)slot * pick<NS>(p.a_stride, ss, p.n_slices) +
                            (ok ? (k0 + row) * R + 8 * c8 : 0);
      av[i] = gload16(ptr);
    }
  };
  load_a(g);
  const bool xw = wave < nb;  // this wave shrinks token block `wave`
  const bool xok = xw && 16 * wave + l16 < rows;
  const int xt = wave == 0 ? tok[0] : (wave == 1 ? tok[1] : (wave == 2 ? tok[2] : tok[3]));
  const uint16_t *xbase = reinterpret_cast<const uint16_t *>(p.x) +
                          (xok ? (p.x_row_div == 1 ? (int64_t)xt : (int64_t)xt / p.x_row_div) * p.ldx : 0);
  // x fragments past d_in meet zero A rows, and rows past the tile feed
  // outputs that are never used: both read the row's first values instead
  u32x4 xa[XB];
  auto load_x = [&](int gm) {  // member gm's x fragments of this wave's token block
    const int64_t kx = ((int64_t)gm << p.ksh) + 8 * kg;  // this lane's k at step 0
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int64_t k = kx + 32 * (int64_t)i;
      xa[i] = gload16(xbase + (i < nsteps && k < p.d_in ? k : 0));
    }
  };
  if (xw) load_x(g);
  u32x4 bv[kSBatch];
  uint32_t bok = 0;
#pragma unroll
  for (int i = 0; i < kSBatch; ++i) {
    const int q = tid + kSThreads * i;
    const int lb = q / (2 * RP), j = (q >> 1) % RP, half = q & 1;
    const int gb = gb0 + lb;
    const int s = last_le<NS>(p.blk_base, p.n_slices, lb < nbm ? gb : gb0);
    const int64_t w = pick<NS>(p.width, s, p.n_slices);
    const int64_t col = 16 * (int64_t)(gb - pick<NS + 1>(p.blk_base, s, p.n_slices + 1)) + 8 * half;
    const bool ok = lb < nbm && j < R && col < w;
    bok |= (uint32_t)ok << i;
    const uint16_t *ptr = reinterpret_cast<const uint16_t *>(pick<NS>(p.B, s, p.n_slices)) +
                          (int64_t)slot * pick<NS>(p.b_stride, s, p.n_slices) + (ok ? j * w + col : 0);
    bv[i] = gload16(ptr);
  }
  // this wave's column blocks wave + 4 q: slice, column of this lane's 4
  // outputs, y offset; y of rows 0..15 loaded now
  uint16_t *const y = reinterpret_cast<uint16_t *>(p.y);
  int qs[QB];
  int64_t qcol[QB];
  bool qok[QB];
  u32x2 yv[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int lb = wave + 4 * q, gb = gb0 + lb;
    qs[q] = last_le<NS>(p.blk_base, p.n_slices, lb < nbm ? gb : gb0);
    const int64_t col = 16 * (int64_t)(gb - pick<NS + 1>(p.blk_base, qs[q], p.n_slices + 1)) + 4 * kg;
    qok[q] = lb < nbm && col < pick<NS>(p.width, qs[q], p.n_slices);
    qcol[q] = pick<NS>(p.offset, qs[q], p.n_slices) + col;
    const bool ok = p.add && qok[q] && l16 < rows;  // else unused
    yv[q] = *reinterpret_cast<const u32x2 *>(y + (ok ? (int64_t)tok[0] * p.ldy + qcol[q] : 0));
  }
  const int rk = p.slot_rank ? min(max(p.slot_rank[slot], 0), R) : R;
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  if (rk == 0) {  // the adapter adds nothing
    if (!p.add) split_zero(p, tl, rows, gb0, nbm);
    return;
  }
  const int rk8 = (rk + 7) & ~7;  // ranks read, as the other kernels read them

  // ---- A chunk into LDS (ranks past the slot's rank as zeros)
  auto stage_a = [&]() {
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      const int q = tid + kSThreads * i;
      if (q < pa) {
        const int s = q >> (p.ksh + LPR);
        const int rem = q & ((kc * PR) - 1);
        const int row = rem / PR, c8 = rem % PR;
        *reinterpret_cast<u32x4 *>(As + ((s << p.ksh) + row) * LDA + 8 * c8) =
            ((aok >> i) & 1) && 8 * c8 < rk8 ? av[i] : u32x4{0, 0, 0, 0};
      }
    }
  };
  stage_a();
  __syncthreads();

  // ---- shrink: wave t, all k-steps of token block t.  D' = A^T x^T, so that
  // lane (token l16, kg) ends with ranks 4 kg .. + 3 of its token: the
  // operand layout the expand takes
  const rsrc_t pr = make_rsrc(p.part, p.part_bytes);
  const int fr0 = ((pos0 + 15) >> 4) + ti;  // the tile's first fragment
  auto frag_off = [&](int gg, int t, int s, int c) {
    return (uint32_t)(((((gg * p.n_frag + fr0 + t) * p.n_slices + s) * RB + c) * kWave + lane) * 16);
  };
  // member gm's partial rows of token block `wave`, from the staged A chunk
  // and xa, into member gm's slot
  auto shrink_store = [&](int gm) {
    f32x4 acc[NS][RB];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[s][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      if (i < nsteps) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s < p.n_slices) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              const bf16x8 aw = lds_col8(As + (s << p.ksh) * LDA, LDA, 32 * i + 8 * kg, 16 * rb);
              acc[s][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, __builtin_bit_cast(bf16x8, xa[i]),
                                                                   acc[s][rb], 0, 0, 0);
            }
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (s < p.n_slices) __builtin_amdgcn_raw_buffer_store_b128(acc[s][rb], pr, frag_off(gm, wave, s, rb), 0, 0);
  };
  if (xw) shrink_store(g);
  // ---- B chunk into LDS (rank rows past the slot's rank as zeros)
#pragma unroll
  for (int i = 0; i < kSBatch; ++i) {
    const int q = tid + kSThreads * i;
    if (q < 2 * RP * p.bpm) {
      const int lb = q / (2 * RP), j = (q >> 1) % RP, half = q & 1;
      *reinterpret_cast<u32x4 *>(Bs + j * p.ldb + 16 * lb + 8 * half) =
          ((bok >> i) & 1) && j < rk8 ? bv[i] : u32x4{0, 0, 0, 0};
    }
  }
  // ---- rendezvous: the fragments are acknowledged before the flag goes up
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (G > 1) {
    __shared__ uint32_t missing;
    if (wave == 0) {
      const uint32_t m = split_wait(fl, f, g, G, p.spin_limit, xcc_id(), flags + (int64_t)kSyncTiles * kSplitFlagWords);
      if (lane == 0) missing = m;
    }
    __syncthreads();
    // members that did not arrive in time: their partials are computed here,
    // by the same code, so they are the bits those members store themselves
    for (uint32_t m = missing; m; m &= m - 1) {
      const int gm = __builtin_ctz(m);
      load_a(gm);
      if (xw) load_x(gm);
      __syncthreads();  // the A chunk's LDS is free
      stage_a();
      __syncthreads();
      if (xw) shrink_store(gm);
    }
    if (missing) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- expand, token block by token block: u = scale * (the members'
  // partials added in the gather's fixed order), split into bf16 hi + lo operands; then
  // every column block of this wave: B^T from LDS, two MFMAs, y.  The y of
  // the next token block is loaded at the end of each block.
  for (int t = 0; t < nb; ++t) {
    s16x4 uh[NS][RB], ul[NS][RB];
    {
      uint32_t off[NS * RB];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int c = 0; c < RB; ++c) off[s * RB + c] = s < p.n_slices ? frag_off(0, t, s, c) : 0x7FFFFFF0u;
      f32x4 u[NS * RB];
      // the stage (n_slices RB 4 KB) fits the A chunk's region: kc >= 128
      gather_members<NS * RB>(pr, off, p.n_frag * p.n_slices * RB * 1024, p.gsh, p.n_slices * RB,
                              reinterpret_cast<f32x4 *>(split_lds), u);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int c = 0; c < RB; ++c) {
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_bf16(sc * u[s * RB + c][e], h[e], l[e]);
          uh[s][c] = __builtin_bit_cast(s16x4, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
          ul[s][c] = __builtin_bit_cast(s16x4, u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)});
        }
      }
    }
    const int row = 16 * t + l16;
    const int tk = t == 0 ? tok[0] : (t == 1 ? tok[1] : (t == 2 ? tok[2] : tok[3]));
    uint16_t *const yrow = y + (int64_t)tk * p.ldy;
    s16x4 bw[QB][RB];
#pragma unroll
    for (int q = 0; q < QB; ++q)
      if (wave + 4 * q < nbm)
#pragma unroll
        for (int c = 0; c < RB; ++c) bw[q][c] = lds_col4(Bs, p.ldb, 16 * c + 4 * kg, 16 * (wave + 4 * q));
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (wave + 4 * q < nbm) {
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
        const int s = qs[q];
#pragma unroll
        for (int c = 0; c < RB; ++c) {
          s16x4 lo = ul[0][c], hi = uh[0][c];
#pragma unroll
          for (int k = 1; k < NS; ++k) {
            if (k == s) {
              lo = ul[k][c];
              hi = uh[k][c];
            }
          }
          d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bw[q][c], lo, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bw[q][c], hi, d, 0, 0, 0);
        }
        if (qok[q] && row < rows) {
          const u32x2 old = p.add ? yv[q] : u32x2{0, 0};
          *reinterpret_cast<u32x2 *>(yrow + qcol[q]) =
              u32x2{pack_bf16x2(bf16_lo(old[0]) + d[0], bf16_hi(old[0]) + d[1]),
                    pack_bf16x2(bf16_lo(old[1]) + d[2], bf16_hi(old[1]) + d[3])};
        }
      }
    }
    if (t + 1 < nb) {
      if (p.add) {  // y of the next token block
        const int tn = t + 1 == 1 ? tok[1] : (t + 1 == 2 ? tok[2] : tok[3]);
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const bool ok = qok[q] && row + 16 < rows;  // else unused
          yv[q] = *reinterpret_cast<const u32x2 *>(y + (ok ? (int64_t)tn * p.ldy + qcol[q] : 0));
        }
      }
      __syncthreads();  // every wave has read the gather's LDS
    }
  }
}

// ------------------------------------------------------------------ one slice
//
// The same algorithm for one output slice per workgroup (separate
// projections, the common decode case; packed slices, up to four, run side by
// side as rows of the grid), written for the fewest executed instructions: every
// operand is read through a buffer resource with a uniform base (the slot's A
// and B matrices, x, y), 32-bit offsets and immediate steps; pieces outside a
// matrix read as zeros by the resource bound instead of by selects.  A
// workgroup runs this code once, so its length is its latency.

struct Split1Params {
  const void *x;
  void *y;
  float *part;
  const float *slot_scale;
  const int32_t *slot_rank;
  uint32_t x_bytes, y_bytes, part_bytes, part_slice;  // part_slice: bytes between slices' partials
  int32_t ldx, d_in, x_row_div, ldy;
  int32_t gsh, ksh, ldb, bs_off, max_tiles, n_frag, spin_limit, add, x_full;
  float scale;
#ifdef LORA_PHASE_CLOCK
  unsigned long long *clk;  // kPhaseWords per workgroup (a measurement build only)
#endif
};

#ifdef LORA_PHASE_CLOCK
// A measurement build: each workgroup of the one-slice kernel records the
// 100 MHz real-time counter when it starts (0), has its tile header (1), its
// A chunk in LDS (2), every load of the batch landed and its partial rows
// acknowledged (3), the rendezvous done (4), the first token block's u
// gathered (5) and its y stores acknowledged (6); then (7) ti | g << 16 |
// slice << 24, (8) the HW_ID register, (9) XCC_ID.  Workgroups that leave
// early record nothing.
constexpr int kPhaseWords = 10;
static unsigned long long *g_phase_clock = nullptr;
static size_t g_phase_words = 0;
#define LORA_PHASE(i)                                                                      \
  do {                                                                                     \
    if (threadIdx.x == 0) clk_rec[i] = (unsigned long long)__builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define LORA_PHASE(i) \
  do {                \
  } while (0)
#endif

// The slices' own values, a kernel argument of their own: it is indexed by
// the slice at run time, which would otherwise make the compiler load every
// field of Split1Params at its use instead of once at the start.
struct Split1Slices {
  const void *A[kSplitRanges], *B[kSplitRanges];
  int64_t a_stride[kSplitRanges], b_stride[kSplitRanges];
  int32_t width[kSplitRanges], offset[kSplitRanges], nbt[kSplitRanges], bpm[kSplitRanges];
};

// p[s] for a workgroup-uniform s < kSplitRanges: one scalar load from the
// argument block at an offset known at launch (selecting among all four
// entries kept every slice's values in scalar registers, which spilled)
template <typename V>
__device__ __forceinline__ V sel_slice(const V (&p)[kSplitRanges], int s) {
  return p[s];
}

// Zero the member's columns of the tile's rows in the window [offset,
// offset + width) (store mode, no adapter).
__device__ __forceinline__ void split1_zero(const Split1Params &p, const int32_t *tl, int rows, int gb0, int nbm,
                                            int offset, int width) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int row = wave; row < rows; row += kSThreads / kWave) {
    uint16_t *yr = reinterpret_cast<uint16_t *>(p.y) + (int64_t)tl[4 + row] * p.ldy + offset;
    for (int h = lane; h < 2 * nbm; h += kWave) {
      const int col = 16 * (gb0 + h / 2) + 8 * (h & 1);
      if (col < width) gstore16(yr + col, u32x4{0, 0, 0, 0});
    }
  }
}

template <int R, int KS>
__global__ __launch_bounds__(kSThreads, 2) void bgmv_split1_kernel(const int32_t *__restrict__ info,
                                                                const int32_t *__restrict__ tiles,
                                                                uint32_t *__restrict__ flags, Split1Params p,
                                                                Split1Slices q) {
  constexpr int RP = R < 16 ? 16 : R;
  constexpr int RB = RP / 16;
  constexpr int LDA = RP == 64 ? 80 : RP;
  constexpr int KC = 32 * KS;                               // k rows per member
  constexpr int KQ = KS / 4;                                // k-steps per wave in a one-block tile
  constexpr int NPA = KC * R / 8;                           // A pieces of the chunk
  constexpr int NA = (NPA + kSThreads - 1) / kSThreads;     // ... per thread
  constexpr int NBQ = (RP == 64 ? 16 : kSMaxBpm) * 2 * RP / kSThreads;  // B pieces per thread, at most
  constexpr int QB = kSMaxBpm / 4;
  constexpr uint32_t kOut = 0x7FFFFFF0u;                    // past every resource: reads as zeros
  static_assert(KC * LDA * 2 >= RB * 4 * kWave * 16, "the gather's stage fits the A chunk's region");
  extern __shared__ __align__(16) unsigned char split_lds[];
  uint16_t *const As = reinterpret_cast<uint16_t *>(split_lds);
  uint16_t *const Bs = reinterpret_cast<uint16_t *>(split_lds + p.bs_off);

#ifdef LORA_PHASE_CLOCK
  const unsigned long long t_start = (unsigned long long)__builtin_amdgcn_s_memrealtime();
  unsigned long long *const clk_rec = p.clk + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kPhaseWords;
#endif
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int l16 = lane % 16, kg = lane / 16;
  const int G = 1 << p.gsh;
  // slices run side by side: slice blockIdx.y is a row of the grid whose
  // width is a multiple of 8, so blockIdx.x mod 8 still names the XCD (the
  // grid is dispatched row after row)
  const int sl = blockIdx.y, lbx = blockIdx.x;
  const int lb8 = lbx >> 3;
  const int g = lb8 & (G - 1);
  const int ti = ((lb8 >> p.gsh) << 3) | (lbx & 7);
  if (ti >= p.max_tiles) return;
  // this slice's values
  const int width = sel_slice(q.width, sl), offset = sel_slice(q.offset, sl);
  const int nbt = sel_slice(q.nbt, sl), bpm = sel_slice(q.bpm, sl);
  const void *a_base = sel_slice(q.A, sl), *b_base = sel_slice(q.B, sl);
  const int64_t a_stride = sel_slice(q.a_stride, sl), b_stride = sel_slice(q.b_stride, sl);

  // ---- first round trip: tile count and header, the tokens of the four
  // 16-row blocks this lane may serve, this member's flag
  const int32_t *tl = tiles + (int64_t)ti * kTileInts;
  const int ntiles = info[4];
  const int slot = tl[0], rows = tl[1], pos0 = tl[2];
  int tok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) tok[q] = tl[4 + 16 * q + l16];
  uint32_t *fl = flags + (int64_t)ti * kSplitFlagWords + kSplitMembers * sl;  // this slice's range
  const uint32_t f = __builtin_amdgcn_readfirstlane(__hip_atomic_load(fl + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (ti >= ntiles) return;
  const int gb0 = g * bpm;
  const int nbm = min(bpm, nbt - gb0);
  if (slot < 0) {
    if (!p.add) split1_zero(p, tl, rows, gb0, nbm, offset, width);
    return;
  }
#ifdef LORA_PHASE_CLOCK
  if (tid == 0) {
    clk_rec[0] = t_start;
    clk_rec[7] = (unsigned long long)(ti | g << 16 | sl << 24);
    clk_rec[8] = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    clk_rec[9] = xcc_id();
  }
#endif
  LORA_PHASE(1);

  // ---- second round trip: every load is issued, none behind a branch;
  // pieces that are not needed take an offset past their resource
  const int nb = (rows + 15) >> 4;
  const rsrc_t ar = make_rsrc(reinterpret_cast<const uint16_t *>(a_base) + (int64_t)slot * a_stride,
                              (uint32_t)(p.d_in * R * 2));
  u32x4 av[NA];
  auto load_a = [&](int gm) {  // member gm's A chunk
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + kSThreads * i;
      av[i] = buf_load16(ar, q < NPA ? (uint32_t)(gm * KC * R * 2 + q * 16) : kOut);
    }
  };
  load_a(g);
  // the shrink: up to rank 32, a tile of one 16-row block (decode) spreads
  // its k-steps over the four waves, wave w taking steps w KQ .. + KQ - 1; a
  // taller tile, or rank 64, gives wave t every step of token block t
  const bool one = RB <= 2 && nb == 1;
  const int blk = one ? 0 : wave;
  const bool xw = blk < nb;
  const int xt = blk == 0 ? tok[0] : (blk == 1 ? tok[1] : (blk == 2 ? tok[2] : tok[3]));
  const int xrow = 16 * blk + l16 < rows ? (p.x_row_div == 1 ? xt : xt / p.x_row_div) : 0;
  const rsrc_t xr = make_rsrc(p.x, p.x_bytes);
  u32x4 xa[KS];
  // member gm's x fragments of this wave's steps; rows past the tile read
  // zeros (their partial rows are never stored)
  auto load_x = [&](int gm) {
    const uint32_t xo = xw && 16 * blk + l16 < rows
                            ? (uint32_t)((xrow * p.ldx + gm * KC + (one ? 32 * KQ * wave : 0) + 8 * kg) * 2)
                            : kOut;
    if (one) {
#pragma unroll
      for (int i = 0; i < KQ; ++i) xa[i] = buf_load16(xr, xo + 64 * i);
    } else {
#pragma unroll
      for (int i = 0; i < KS; ++i) xa[i] = buf_load16(xr, xo + 64 * i);
    }
  };
  load_x(g);
  const rsrc_t br = make_rsrc(reinterpret_cast<const uint16_t *>(b_base) + (int64_t)slot * b_stride,
                              (uint32_t)(R * width * 2));
  u32x4 bv[NBQ];
#pragma unroll
  for (int i = 0; i < NBQ; ++i) {
    const int q = tid + kSThreads * i;
    const int lb = q / (2 * RP), j = (q >> 1) % RP, half = q & 1;
    const int col = 16 * (gb0 + lb) + 8 * half;
    const bool ok = lb < nbm && j < R && col < width;
    bv[i] = buf_load16(br, ok ? (uint32_t)((j * width + col) * 2) : kOut);
  }
  // y of the first token block.  Up to 512-row chunks it is loaded here and
  // arrives with the rest of the batch, so it holds neither the
  // acknowledgement wait nor the polls (loads complete in order).  With
  // 1024-row chunks (32 x loads a lane) it is loaded once the fragments are
  // acknowledged: each order measured faster for its own chunk length.
  constexpr bool kYEarly = KS <= 16;
  const rsrc_t yr = make_rsrc(p.y, p.y_bytes);
  const uint32_t yo0 = (uint32_t)((offset + 16 * (gb0 + wave) + 4 * kg) * 2);  // + 128 q: block wave + 4 q
  uint32_t yrow = (uint32_t)(tok[0] * p.ldy * 2);
  u32x2 yv[QB];
  auto load_y0 = [&]() {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const bool ok = p.add && wave + 4 * q < nbm;
      yv[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(yr, ok ? yrow + yo0 + 128 * q : kOut, 0, 0));
    }
  };
  if constexpr (kYEarly) load_y0();
  const int rk = p.slot_rank ? min(max(p.slot_rank[slot], 0), R) : R;
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  if (rk == 0) {
    if (!p.add) split1_zero(p, tl, rows, gb0, nbm, offset, width);
    return;
  }
  const int rk8 = (rk + 7) & ~7;

  // ---- A chunk into LDS: piece q = row q / (R / 8), ranks 8 (q % (R / 8)) ..
  auto stage_a = [&]() {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + kSThreads * i;
      if (q < NPA) {
        const int row = q / (R / 8), c8 = q % (R / 8);
        *reinterpret_cast<u32x4 *>(As + row * LDA + 8 * c8) = 8 * c8 < rk8 ? av[i] : u32x4{0, 0, 0, 0};
        if constexpr (R == 8) *reinterpret_cast<u32x4 *>(As + row * LDA + 8) = u32x4{0, 0, 0, 0};
      }
    }
  };
  stage_a();
  __syncthreads();
  LORA_PHASE(2);

  // ---- shrink (D' = A^T x^T, so that lane (token l16, kg) ends with ranks
  // 4 kg .. + 3 of its token)
  const rsrc_t pr = make_rsrc(p.part, p.part_bytes);
  const uint32_t fbase = (uint32_t)((((pos0 + 15) >> 4) + ti) * RB * 1024 + lane * 16) + sl * p.part_slice;
  const uint32_t plane = (uint32_t)(p.n_frag * RB * 1024);  // between members
  // member gm's partial rows, from the staged A chunk and xa, into member
  // gm's slot.  Two accumulator chains (even and odd k-steps) added at the
  // end: the MFMAs of one chain wait for each other, the two chains do not.
  // A one-block tile's four waves add their sums in wave order through LDS
  // (RB x 4 waves x 64 lanes, a region of its own after the B chunk), and
  // wave 0 stores them.  Called by every wave.
  f32x4 *const red = reinterpret_cast<f32x4 *>(split_lds + p.bs_off + RP * p.ldb * 2);
  auto shrink_store = [&](int gm) {
    f32x4 acc[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[0][rb] = acc[1][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // x values of this lane past d_in are dropped
    const int kleft = p.d_in - gm * KC - (one ? 32 * KQ * wave : 0) - 8 * kg;
    if (one) {
#pragma unroll
      for (int i = 0; i < KQ; ++i) {
        const u32x4 xv = p.x_full || 32 * i < kleft ? xa[i] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[i & 1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              lds_col8(As, LDA, 32 * (KQ * wave + i) + 8 * kg, 16 * rb), __builtin_bit_cast(bf16x8, xv), acc[i & 1][rb],
              0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) red[(rb * 4 + wave) * kWave + lane] = acc[0][rb] + acc[1][rb];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 *r4 = red + rb * 4 * kWave + lane;
          __builtin_amdgcn_raw_buffer_store_b128(((r4[0] + r4[kWave]) + r4[2 * kWave]) + r4[3 * kWave], pr,
                                                 fbase + gm * plane + rb * 1024, 0, 0);
        }
      }
    } else if (xw) {
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const u32x4 xv = p.x_full || 32 * i < kleft ? xa[i] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[i & 1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_col8(As, LDA, 32 * i + 8 * kg, 16 * rb),
                                                                   __builtin_bit_cast(bf16x8, xv), acc[i & 1][rb], 0, 0,
                                                                   0);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        __builtin_amdgcn_raw_buffer_store_b128(acc[0][rb] + acc[1][rb], pr,
                                               fbase + gm * plane + (wave * RB + rb) * 1024, 0, 0);
    }
  };
  shrink_store(g);
  // ---- B chunk into LDS (rank rows past the slot's rank as zeros)
#pragma unroll
  for (int i = 0; i < NBQ; ++i) {
    const int q = tid + kSThreads * i;
    if (q < 2 * RP * bpm) {
      const int lb = q / (2 * RP), j = (q >> 1) % RP, half = q & 1;
      *reinterpret_cast<u32x4 *>(Bs + j * p.ldb + 16 * lb + 8 * half) = j < rk8 ? bv[i] : u32x4{0, 0, 0, 0};
    }
  }
  // ---- rendezvous: the fragments are acknowledged before the flag goes up
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  LORA_PHASE(3);
  if constexpr (!kYEarly) load_y0();
  if (G > 1) {
    __shared__ uint32_t missing;
    if (wave == 0) {
      const uint32_t m = split_wait(fl, f, g, G, p.spin_limit, xcc_id(), flags + (int64_t)kSyncTiles * kSplitFlagWords);
      if (lane == 0) missing = m;
    }
    __syncthreads();
    // members that did not arrive in time: their partials are computed here,
    // by the same code, so they are the bits those members store themselves
    // (a late member and this workgroup then write equal values)
    for (uint32_t m = missing; m; m &= m - 1) {
      const int gm = __builtin_ctz(m);
      load_a(gm);
      load_x(gm);
      __syncthreads();  // the A chunk's LDS is free
      stage_a();
      __syncthreads();
      shrink_store(gm);
    }
    if (missing) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
  LORA_PHASE(4);

  // ---- expand, token block by token block: u = scale * (members' partials
  // in the gather's fixed order) as bf16 hi + lo operands; every column block
  // of this wave (a block past the member's share reads block 0 and stores
  // nothing).  Each block's y is stored as soon as its two products are done:
  // that measured faster than issuing every product first, and than one
  // 16x16x32 product with hi and lo as the two halves of K.
  // B^T operands first: their LDS reads overlap the gather's loads
  s16x4 bw[QB][RB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int lb = wave + 4 * q < nbm ? wave + 4 * q : 0;
#pragma unroll
    for (int c = 0; c < RB; ++c) bw[q][c] = lds_col4(Bs, p.ldb, 16 * c + 4 * kg, 16 * lb);
  }
  for (int t = 0; t < nb; ++t) {
    s16x4 uh[RB], ul[RB];
    {
      uint32_t off[RB];
#pragma unroll
      for (int c = 0; c < RB; ++c) off[c] = fbase + (t * RB + c) * 1024;
      f32x4 u[RB];
      gather_members<RB>(pr, off, plane, p.gsh, RB, reinterpret_cast<f32x4 *>(split_lds), u);
#pragma unroll
      for (int c = 0; c < RB; ++c) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(sc * u[c][e], h[e], l[e]);
        uh[c] = __builtin_bit_cast(s16x4, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
        ul[c] = __builtin_bit_cast(s16x4, u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)});
      }
    }
    if (t == 0) LORA_PHASE(5);
    const bool rok = 16 * t + l16 < rows;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < RB; ++c) {
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bw[q][c], ul[c], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bw[q][c], uh[c], d, 0, 0, 0);
      }
      const u32x2 old = p.add ? yv[q] : u32x2{0, 0};
      const u32x2 v = {pack_bf16x2(bf16_lo(old[0]) + d[0], bf16_hi(old[0]) + d[1]),
                       pack_bf16x2(bf16_lo(old[1]) + d[2], bf16_hi(old[1]) + d[3])};
      if (rok && wave + 4 * q < nbm && 16 * (gb0 + wave + 4 * q) + 4 * kg < width)
        __builtin_amdgcn_raw_buffer_store_b64(v, yr, yrow + yo0 + 128 * q, 0, 0);
    }
    if (t + 1 < nb) {  // y of the next token block
      const int tn = t + 1 == 1 ? tok[1] : (t + 1 == 2 ? tok[2] : tok[3]);
      yrow = (uint32_t)(tn * p.ldy * 2);
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const bool ok = p.add && wave + 4 * q < nbm;
        yv[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(yr, ok ? yrow + yo0 + 128 * q : kOut, 0, 0));
      }
      __syncthreads();  // every wave has read the gather's LDS
    }
  }
#ifdef LORA_PHASE_CLOCK
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  LORA_PHASE(6);
#endif
}

// ------------------------------------------------------------------ host side

struct SplitPlan {
  bool ok;
  int G, ksh, bpm, ldb, bs_off, grid;
  size_t lds;
};

static int ilog2(int64_t v) {
  int r = 0;
  while (((int64_t)1 << r) < v) ++r;
  return r;
}

// Workspace bytes of the partial fragments for up to kSplitMembers members
// (0 when the batch is too large for the split kernel).
size_t split_ws_bytes(int64_t T, int32_t S, int32_t n_slices, int32_t R) {
  const int64_t RP = R < 16 ? 16 : R;
  if (T * n_slices * RP > ((int64_t)1 << 17)) return 0;
  const int64_t n_frag = (T + 15) / 16 + max_tiles(T, S);
  return (size_t)kSplitMembers * n_frag * n_slices * (RP / 16) * 1024;
}

static std::atomic<int> g_split_resident[4][4][kMaxDevices];

// LDS bytes of the A chunk (the B chunk follows it).
static size_t split_region1(int n_slices, int64_t kc, int R) {
  const int RP = R < 16 ? 16 : R, LDA = RP == 64 ? 80 : RP;
  return ((size_t)n_slices * kc * LDA * 2 + 15) / 16 * 16;
}
static int split_ldb(int bpm) { return 16 * bpm + ((16 - 16 * bpm) & 127); }  // = 16 (mod 128): conflict-free

// Largest LDS a plan can ask for at rank R and at most NS slices (every
// budget at its bound).
static size_t split_lds_max(int R, int NS) {
  const int RP = R < 16 ? 16 : R;
  const int bpm = std::min(kSMaxBpm, kSPieces / (2 * RP));
  size_t r1 = 0;
  for (int ns = 1; ns <= NS; ++ns)
    r1 = std::max(r1, split_region1(ns, std::max(128, kSPieces * 8 / (ns * RP)), R));
  return r1 + (size_t)RP * split_ldb(bpm) * 2;
}

// G, k-chunk and column share of a call: G from the tiles the batch can have
// (about one workgroup per CU), raised until each member's A chunk and B
// chunk are at most kSPieces 16-byte pieces.  Not ok when no G <= 16 fits or
// the partial fragments exceed the workspace.
// side: the slices run side by side (one slice per workgroup, the one-slice
// kernel): the A budget is one slice's chunk and the column share is the
// widest slice's; otherwise one workgroup holds every slice's A chunk and a
// share of all their column blocks.
static SplitPlan plan_split(int64_t T, int32_t S, int64_t d_in, int32_t n_slices, const int64_t *width,
                            int32_t R, size_t ws_bytes, int g_cap, int kc_max = 512, bool side = false) {
  SplitPlan pl{};
  const int RP = R < 16 ? 16 : R, RB = RP / 16;
  const int NSb = n_slices <= 1 ? 1 : (n_slices <= 2 ? 2 : (n_slices <= 4 ? 4 : 8));
  if ((side ? n_slices > kSplitRanges : NSb * RB > 8) || split_ws_bytes(T, S, n_slices, R) == 0) return pl;
  int64_t nbt = 0;
  for (int s = 0; s < n_slices; ++s)
    nbt = side ? std::max<int64_t>(nbt, (width[s] + 15) / 16) : nbt + (width[s] + 15) / 16;
  const int a_slices = side ? 1 : n_slices;
  const int64_t mt = max_tiles(T, S);
  const int64_t est = std::min<int64_t>(mt, T);  // live tiles, at most
  int G = 1;
  while (G < kSplitMembers && G < g_cap && 2 * G * est <= 384) G *= 2;
  if (split_members() > 0) G = std::min(split_members(), g_cap);  // tuning override
  for (;; G *= 2) {
    if (G > kSplitMembers || G > g_cap) return pl;
    const int64_t kc = std::max<int64_t>(128, (int64_t)1 << ilog2((d_in + G - 1) / G));
    const int64_t bpm = (nbt + G - 1) / G;
    if (kc <= kc_max && (int64_t)a_slices * kc * (RP / 8) <= kSPieces && bpm <= kSMaxBpm && bpm * 2 * RP <= kSPieces) {
      pl.ksh = ilog2(kc);
      pl.bpm = (int)bpm;
      break;
    }
  }
  pl.G = G;
  pl.ldb = split_ldb(pl.bpm);
  pl.bs_off = (int)split_region1(a_slices, (int64_t)1 << pl.ksh, R);
  pl.lds = pl.bs_off + (size_t)RP * pl.ldb * 2;
  pl.grid = (int)(8 * G * ((mt + 7) / 8)) * (side ? n_slices : 1);
  const size_t need = (size_t)G * ((T + 15) / 16 + mt) * n_slices * RB * 1024;
  if (need > ws_bytes) return pl;
  pl.ok = true;
  return pl;
}

// Plans the call for this instantiation and launches it, unless its grid
// exceeds the workgroups the device holds at once (then *used stays false).
template <int R, int NS>
static hipError_t launch_split_k(const MetaView &meta, SplitParams &p, const int64_t *width, size_t part_bytes,
                                 hipStream_t stream, bool *used) {
  const void *fn = reinterpret_cast<const void *>(&bgmv_split_kernel<R, NS>);
  constexpr int ri = R == 8 ? 0 : (R == 16 ? 1 : (R == 32 ? 2 : 3));
  constexpr int ni = NS == 1 ? 0 : (NS == 2 ? 1 : (NS == 4 ? 2 : 3));
  int g_cap = kSplitMembers;
  for (;;) {
    const SplitPlan pl = plan_split(meta.T, meta.S, p.d_in, p.n_slices, width, R, part_bytes, g_cap);
    if (!pl.ok) return hipSuccess;
    // the residency count is cached per device and taken at this
    // instantiation's largest LDS, which the function is allowed first
    const size_t lds_max = split_lds_max(R, NS);
    if (lds_max > 65536) {  // more than the default dynamic LDS
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
      if (e != hipSuccess) return e;
    }
    const int resident = resident_groups(g_split_resident[ri][ni], fn, kSThreads, lds_max);
    // this kernel runs only when its whole grid is resident: with more
    // workgroups than that it measured slower than the one-workgroup-per-token
    // kernel (packed q/k/v at G = 16, 21 us against 15 us)
    if (pl.G > 1 && pl.grid > resident) {
      g_cap = pl.G / 2;
      continue;
    }
    *used = true;
    p.gsh = ilog2(pl.G);
    p.ksh = pl.ksh;
    p.bpm = pl.bpm;
    p.ldb = pl.ldb;
    p.bs_off = pl.bs_off;
    hipLaunchKernelGGL((bgmv_split_kernel<R, NS>), dim3(pl.grid), dim3(kSThreads), pl.lds, stream, meta.info,
                       meta.tiles, p.sync, p);
    return hipGetLastError();
  }
}

// One-slice kernel: plan (as above, with the first LDS region holding only
// the A chunk), residency, launch.
static std::atomic<int> g_split1_resident[16][kMaxDevices];

// Launches the one-slice kernel for a plan whose chunk is 32 KS rows, unless
// one XCD cannot hold a whole tile's members (*too_many).
template <int R, int KS>
static hipError_t launch_split1_k(const MetaView &meta, const SplitParams &sp, const int64_t *width, SplitPlan pl,
                                  uint32_t x_bytes, uint32_t y_bytes, hipStream_t stream, bool *used, bool *too_many) {
  constexpr int RP = R < 16 ? 16 : R, LDA = RP == 64 ? 80 : RP;
  const void *fn = reinterpret_cast<const void *>(&bgmv_split1_kernel<R, KS>);
  constexpr int ri = (R == 8 ? 0 : (R == 16 ? 1 : (R == 32 ? 2 : 3))) * 4 + (KS == 4 ? 0 : (KS == 8 ? 1 : (KS == 16 ? 2 : 3)));
  // the one-block shrink's sums (up to rank 32), after the B chunk
  constexpr size_t kRed = RP <= 32 ? (size_t)(RP / 16) * 4 * kWave * 16 : 0;
  pl.bs_off = (32 * KS * LDA * 2 + 15) / 16 * 16;
  pl.lds = pl.bs_off + (size_t)RP * pl.ldb * 2 + kRed;
  // the residency count is cached per device and taken at this
  // instantiation's largest LDS, which the function is allowed first
  const size_t lds_max = (size_t)32 * KS * LDA * 2 +
                         (size_t)RP * split_ldb(std::min(kSMaxBpm, kSPieces / (2 * RP))) * 2 + kRed;
  if (lds_max > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
    if (e != hipSuccess) return e;
  }
  const int resident = resident_groups(g_split1_resident[ri], fn, kSThreads, lds_max);
  // workgroups are dispatched in order on each XCD and a tile's members are
  // neighbours there, so the tiles within the resident part of the grid
  // finish and make room for the rest; only an XCD that cannot hold one whole
  // tile would leave members waiting for the spin limit
  if (pl.G > 1 && resident / 8 < pl.G) {
    *too_many = true;
    return hipSuccess;
  }
  *used = true;
  Split1Params p{};
  Split1Slices q{};
  p.x = sp.x;
  const int RB = RP / 16;
  for (int s = 0; s < sp.n_slices; ++s) {
    q.A[s] = sp.A[s];
    q.B[s] = sp.B[s];
    q.a_stride[s] = sp.a_stride[s];
    q.b_stride[s] = sp.b_stride[s];
    q.width[s] = (int32_t)width[s];
    q.offset[s] = (int32_t)sp.offset[s];
    q.nbt[s] = sp.blk_base[s + 1] - sp.blk_base[s];
    q.bpm[s] = (q.nbt[s] + pl.G - 1) / pl.G;
  }
  p.part_slice = (uint32_t)((size_t)pl.G * sp.n_frag * RB * 1024);
  p.y = sp.y;
  p.part = sp.part;
  p.slot_scale = sp.slot_scale;
  p.slot_rank = sp.slot_rank;
  p.x_bytes = x_bytes;
  p.y_bytes = y_bytes;
  p.part_bytes = sp.part_bytes;
  p.ldx = (int32_t)sp.ldx;
  p.d_in = (int32_t)sp.d_in;
  p.x_row_div = sp.x_row_div;
  p.ldy = (int32_t)sp.ldy;
  p.gsh = ilog2(pl.G);
  p.ksh = pl.ksh;
  p.ldb = pl.ldb;
  p.bs_off = pl.bs_off;
  p.max_tiles = sp.max_tiles;
  p.n_frag = sp.n_frag;
  p.spin_limit = sp.spin_limit;
  p.add = sp.add;
  p.x_full = ((int64_t)pl.G << pl.ksh) == sp.d_in ? 1 : 0;
  p.scale = sp.scale;
#ifdef LORA_PHASE_CLOCK
  p.clk = g_phase_clock;
  // lora_debug_phase_clock not called, or its buffer too small for the grid
  if (!p.clk || (size_t)pl.grid * kPhaseWords > g_phase_words) return hipErrorInvalidValue;
#endif
  hipLaunchKernelGGL((bgmv_split1_kernel<R, KS>), dim3(pl.grid / sp.n_slices, sp.n_slices), dim3(kSThreads), pl.lds,
                     stream, meta.info, meta.tiles, sp.sync, p, q);
  return hipGetLastError();
}

// One slice, or up to four side by side: plan, then the instantiation for
// the plan's chunk (128, 256, 512 or 1024 rows); when an XCD cannot hold a
// tile's members, plan again with G halved.
template <int R>
static hipError_t launch_split1(const MetaView &meta, const SplitParams &sp, const int64_t *width,
                                size_t part_bytes, hipStream_t stream, bool *used) {
  // 32-bit offsets into x and y
  const int64_t x_rows = (meta.T + meta.x_row_div - 1) / meta.x_row_div;
  const int64_t x_bytes = ((x_rows - 1) * sp.ldx + sp.d_in) * 2;
  int64_t y_end = 0;
  for (int s = 0; s < sp.n_slices; ++s) y_end = std::max(y_end, sp.offset[s] + width[s]);
  const int64_t y_bytes = ((meta.T - 1) * sp.ldy + y_end) * 2;
  // offsets from 0x7FFFFFF0 up must lie past both resources (pieces and
  // stores that are not wanted are sent there)
  if (x_bytes > 0x7FFFFFF0LL || y_bytes > 0x7FFFFFF0LL) return hipSuccess;
  // ranks up to 16 also take 1024-row chunks (32 steps), so that d_in up to
  // 16384 splits 16 ways
  const int kc_max = R <= 16 ? 1024 : 512;
  for (int g_cap = kSplitMembers; g_cap >= 1; g_cap /= 2) {
    const SplitPlan pl = plan_split(meta.T, meta.S, sp.d_in, sp.n_slices, width, R, part_bytes, g_cap, kc_max, true);
    if (!pl.ok) return hipSuccess;
    bool too_many = false;
    hipError_t e = hipSuccess;
    if (pl.ksh == 10) {
      if constexpr (R <= 16)
        e = launch_split1_k<R, 32>(meta, sp, width, pl, (uint32_t)x_bytes, (uint32_t)y_bytes, stream, used, &too_many);
    } else if (pl.ksh == 7)
      e = launch_split1_k<R, 4>(meta, sp, width, pl, (uint32_t)x_bytes, (uint32_t)y_bytes, stream, used, &too_many);
    else if (pl.ksh == 8)
      e = launch_split1_k<R, 8>(meta, sp, width, pl, (uint32_t)x_bytes, (uint32_t)y_bytes, stream, used, &too_many);
    else
      e = launch_split1_k<R, 16>(meta, sp, width, pl, (uint32_t)x_bytes, (uint32_t)y_bytes, stream, used, &too_many);
    if (e != hipSuccess || !too_many) return e;
    g_cap = std::min(g_cap, pl.G);
  }
  return hipSuccess;
}

template <int R>
static hipError_t launch_split_t(const MetaView &meta, SplitParams &p, const int64_t *width, size_t part_bytes,
                                 hipStream_t stream, bool *used) {
  return with_slice_bound(p.n_slices, [&](auto ns) -> hipError_t {
    constexpr int NS = decltype(ns)::value;
    constexpr int RB = (R < 16 ? 16 : R) / 16;
    if constexpr (NS * RB > 8) {
      return hipSuccess;  // not a shape this kernel takes
    } else {
      return launch_split_k<R, NS>(meta, p, width, part_bytes, stream, used);
    }
  });
}

// Tries the split kernel; *used = false when the call's shape is not one it
// takes (the caller then runs another path).
hipError_t launch_bgmv_split(const MetaView &meta, const void *x, int64_t ldx, int64_t d_in, int32_t n_slices,
                             const void *const *A, const int64_t *a_stride, const void *const *B,
                             const int64_t *b_stride, const int64_t *width, const int64_t *offset, int32_t R,
                             float scale, const float *slot_scale, const int32_t *slot_rank, void *y, int64_t ldy,
                             int add, uint32_t *sync, float *part, size_t part_bytes, hipStream_t stream,
                             bool *used) {
  *used = false;
  if (meta.T == 0 || part_bytes >= ((size_t)1 << 32) || ldy >= ((int64_t)1 << 30)) return hipSuccess;
  if (max_tiles(meta.T, meta.S) > kSyncTiles) return hipSuccess;  // tiles past the rendezvous region
  SplitParams p{};
  p.x = x;
  p.ldx = ldx;
  p.d_in = d_in;
  p.x_row_div = meta.x_row_div;
  p.n_slices = n_slices;
  p.blk_base[0] = 0;
  for (int s = 0; s < n_slices; ++s) {
    p.A[s] = A[s];
    p.a_stride[s] = a_stride[s];
    p.B[s] = B[s];
    p.b_stride[s] = b_stride[s];
    p.width[s] = width[s];
    p.offset[s] = offset[s];
    p.blk_base[s + 1] = p.blk_base[s] + (int32_t)((width[s] + 15) / 16);
  }
  for (int s = n_slices + 1; s <= kMaxSlices; ++s) p.blk_base[s] = p.blk_base[n_slices];
  p.max_tiles = (int32_t)max_tiles(meta.T, meta.S);
  p.n_frag = (int32_t)((meta.T + 15) / 16 + p.max_tiles);
  p.spin_limit = split_spin_limit();
  p.part_bytes = (uint32_t)part_bytes;
  p.scale = scale;
  p.slot_scale = slot_scale;
  p.slot_rank = slot_rank;
  p.y = y;
  p.ldy = ldy;
  p.add = add ? 1 : 0;
  p.part = part;
  p.sync = sync;
  // one slice, or up to four side by side, on the one-slice kernel (ldx and
  // ldy also enter its 32-bit offsets); else every slice in one workgroup
  if (n_slices <= kSplitRanges && ldx < ((int64_t)1 << 31) && ldy < ((int64_t)1 << 31)) {
    hipError_t e = hipSuccess;
    switch (R) {
      case 8: e = launch_split1<8>(meta, p, width, part_bytes, stream, used); break;
      case 16: e = launch_split1<16>(meta, p, width, part_bytes, stream, used); break;
      case 32: e = launch_split1<32>(meta, p, width, part_bytes, stream, used); break;
      case 64: e = launch_split1<64>(meta, p, width, part_bytes, stream, used); break;
    }
    if (e != hipSuccess || *used || n_slices == 1) return e;
  }
  switch (R) {
    case 8: return launch_split_t<8>(meta, p, width, part_bytes, stream, used);
    case 16: return launch_split_t<16>(meta, p, width, part_bytes, stream, used);
    case 32: return launch_split_t<32>(meta, p, width, part_bytes, stream, used);
    case 64: return launch_split_t<64>(meta, p, width, part_bytes, stream, used);
  }
  return hipSuccess;
}

}  // namespace lora

#ifdef LORA_PHASE_CLOCK
// The buffer the one-slice split kernel writes its phase timestamps to
// (kPhaseWords 64-bit words per workgroup of its grid), a measurement build
// only.
extern "C" void lora_debug_phase_clock(void *d_buf, size_t words) {
  lora::g_phase_clock = static_cast<unsigned long long *>(d_buf);
  lora::g_phase_words = words;
}
#endif
