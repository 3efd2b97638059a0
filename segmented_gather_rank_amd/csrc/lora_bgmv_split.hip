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
// plain 16-byte stores (the write-through L1 passes them to L2), every fp32
// value beside a tag word that names the call, in one 8-byte word with it;
// the others poll the fragments themselves with agent-coherent loads, which
// skip L1, until every tag they read names this call.  A value read beside
// this call's tag is the value stored with that tag (one store wrote both,
// one load read both), so no flag has to order anything and no member waits
// for its own stores to be acknowledged: the exchange costs the polls alone.
// The G partial fragments are then added in one fixed order (each wave a
// quarter of the members, then the four sums in wave order through LDS), so
// every member gets the same u, bit for bit.
//
// The tag is the call count of the tile's range (bits 31:17, modulo 2^15),
// the tile (bits 16:6), the range (bits 5:4) and the XCD (hardware register
// XCC_ID) of the storing member (bits 3:0).  The counts live in count words at
// the start of the caller's apply workspace, so calls with workspaces of
// their own share nothing: a member reads its word at the start and tags with
// "count + 1", and raises the word to that tag for the next call (member 0
// also raises the words of members >= G), so the words of a range stay equal
// between calls.  A fragment slot written by an earlier call of another shape
// belongs to another tile or range there, or carries an earlier count of this
// one: either way its tags differ from this call's (until the range's count
// comes round again after 32768 calls and the slot was never rewritten since).
//
// The B chunk is loaded with the A chunk and x, and so is the y of the first
// 16 rows except with the longest chunks, so that none of them is outstanding
// at the polls (loads complete in order).
// The polls are bounded: a member computes itself, with the same code (so the
// same bits), the partials of every peer whose tags have not all arrived at
// the spin limit, stores them into those peers' slots (where the peer writes
// equal values) and reads them back through its own L2.  A member on another
// XCD is no hazard either: whatever its tagged words are seen to hold, a word
// with this call's tag carries its value.  The result therefore depends
// neither on the members being resident together nor on their sharing an
// XCD: a late member costs the spin limit and is counted (a status word
// beside the count words), never a wrong value.  Workgroups are dispatched in
// order on each XCD and a tile's members are neighbours there, so the tiles
// within the resident part of a larger grid finish and make room for the
// rest.
//
// Only bf16.
#include <cstdlib>
#include <cstring>

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
  uint32_t *sync;  // count words (host side only: the kernels take them as an argument)
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

// This call's tag of (tile ti, range sl) without the XCD bits, from the
// member's count word f: the count, one more than the word's (bits 31:17,
// modulo 2^15), the tile (bits 16:6) and the range (bits 5:4).  Calls of
// other shapes on the same workspace lay their fragments out differently, so
// a fragment slot may hold another tile's or range's partials from an earlier
// call, whose own count can equal this one; naming the tile and the range in
// the tag keeps those from passing for this call's.
static_assert(kSyncTiles <= 2048 && kSplitRanges <= 4, "tile and range fit their tag fields");
__device__ __forceinline__ uint32_t split_want(uint32_t f, int ti, int sl) {
  return ((((f >> 17) + 1u) & 0x7FFFu) << 17) | ((uint32_t)ti << 6) | ((uint32_t)sl << 4);
}

// XCD this workgroup runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & 15u; }

// Raise this member's count word of the tile (member 0 also those of members
// >= G) to this call's tag: the next call's members read their count there.
// No peer waits for these words; a plain store that reaches L2 whenever it does.
__device__ __forceinline__ void raise_count(uint32_t *fl, int g, int G, uint32_t tag) {
  const int lane = threadIdx.x % kWave;
  if (lane < kSplitMembers && (lane == g || (g == 0 && lane >= G)))
    __builtin_amdgcn_raw_buffer_store_b32(tag, make_rsrc(fl, kSplitMembers * 4), lane * 4, 0, 0);
}

// A lane's four fp32 partials of a fragment, each beside the call's tag:
// (v0, tag, v1, tag) at off and (v2, tag, v3, tag) at off + 1024, so that a
// fragment of 64 lanes takes 2048 bytes.  A value and its tag share one
// naturally aligned 8-byte word, written by one store and read by one load:
// a reader that finds this call's tag has the value stored with it, whichever
// XCD stored it and however the line travelled.
// The bits of a value as another type of the same size.  The value comes in
// by value: applied to an element of a vector directly (v[1]), the bit cast
// has been seen to read the vector's first element instead.
template <typename T, typename S>
__device__ __forceinline__ T bits_as(S s) {
  return __builtin_bit_cast(T, s);
}

__device__ __forceinline__ void store_tagged(rsrc_t pr, uint32_t off, f32x4 v, uint32_t tag) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{bits_as<uint32_t>(v[0]), tag, bits_as<uint32_t>(v[1]), tag}, pr, off,
                                         0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{bits_as<uint32_t>(v[2]), tag, bits_as<uint32_t>(v[3]), tag}, pr,
                                         off + 1024, 0, 0);
}

// Wave w's part of gathering the nf fragments (of NF) at off[f] + gm plane
// over the G members gm: it polls members w MG .. w MG + MG - 1 (those below
// G) with agent-coherent loads, every load of a look issued before the first
// is used, until each tag of a member, XCD bits aside, equals `want`, at
// most spin_limit + 1 looks.  Then it adds each fragment's values in member
// order into stage[f][wave] (fragments past nf: nothing), so that the caller
// adds the four waves' sums in wave order after a barrier, and every member
// of a tile gets the same bits.  Returns the members (bit gm) whose tags were
// still not all there at the last look, and with `guard` also those whose
// tags name another XCD (*foreign gets those): their values in the sums are
// not used, the caller computes their partials itself and gathers again.
// At most 16 loads a lane are in flight: more fragments go in chunks.
template <int MG, int NF>
__device__ __forceinline__ uint32_t poll_wave(rsrc_t pr, const uint32_t (&off)[NF], uint32_t plane, int G, int nf,
                                              uint32_t want, uint32_t xcc, int spin_limit, bool guard, f32x4 *stage,
                                              uint32_t *foreign) {
  constexpr int FC = 8 / MG < NF ? 8 / MG : NF;  // fragments per chunk
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t missing = 0, other = 0;
#pragma unroll
  for (int f0 = 0; f0 < NF; f0 += FC) {
    u32x4 lo[FC][MG], hi[FC][MG];
    uint32_t late = 0;  // bit i: member w MG + i
    for (int polls = 0;; ++polls) {
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        const int gm = wave * MG + i;
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          const uint32_t o = f0 + f < nf && gm < G ? off[f0 + f] + gm * plane : 0x7FFFFFF0u;
          lo[f][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, 16));
          hi[f][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, o + 1024, 0, 16));
        }
      }
      late = 0;
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        bool ok = true;
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          if (f0 + f < nf) {
            const uint32_t t0 = lo[f][i][1], t1 = lo[f][i][3], t2 = hi[f][i][1], t3 = hi[f][i][3];
            ok = ok && (t0 & ~15u) == want && (t1 & ~15u) == want && (t2 & ~15u) == want && (t3 & ~15u) == want;
          }
        }
        if (wave * MG + i < G && __ballot(!ok) != 0) late |= 1u << i;
      }
      if (late == 0 || polls >= spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      const uint32_t bit = 1u << (wave * MG + i);
      if ((late >> i) & 1)
        missing |= bit;
      else if (guard && wave * MG + i < G && f0 < nf && __ballot((lo[0][i][1] & 15u) != xcc) != 0)
        other |= bit;
    }
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        const f32x4 v = {bits_as<float>(lo[f][i][0]), bits_as<float>(lo[f][i][2]), bits_as<float>(hi[f][i][0]),
                         bits_as<float>(hi[f][i][2])};
        w = i == 0 ? v : w + v;
      }
      if (f0 + f < nf) stage[((f0 + f) * 4 + wave) * kWave + lane] = w;
    }
  }
  *foreign = other;
  return missing | other;
}

// poll_wave with the members per wave the member count G = 2^gsh needs
template <int NF>
__device__ __forceinline__ uint32_t poll_members(rsrc_t pr, const uint32_t (&off)[NF], uint32_t plane, int gsh,
                                                 int nf, uint32_t want, uint32_t xcc, int spin_limit, bool guard,
                                                 f32x4 *stage, uint32_t *foreign) {
  switch (gsh) {
    case 0:
    case 1:
    case 2: return poll_wave<1, NF>(pr, off, plane, 1 << gsh, nf, want, xcc, spin_limit, guard, stage, foreign);
    case 3: return poll_wave<2, NF>(pr, off, plane, 8, nf, want, xcc, spin_limit, guard, stage, foreign);
    default: return poll_wave<4, NF>(pr, off, plane, 16, nf, want, xcc, spin_limit, guard, stage, foreign);
  }
}

// Polls that the later token blocks of a tile may take: by then every member
// is known to run on this XCD or was computed here, so its fragments are on
// their way to this L2 and the bound is never reached (if it were, status[0]
// counts it).
constexpr int kLaterPolls = 1 << 20;

// The four waves' sums of each fragment, added in wave order (after the
// barrier that follows poll_members).
template <int NF>
__device__ __forceinline__ void stage_sums(const f32x4 *stage, int nf, f32x4 (&u)[NF]) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const f32x4 *st = stage + f * 4 * kWave + lane;
    u[f] = f < nf ? ((st[0] + st[kWave]) + st[2 * kWave]) + st[3 * kWave] : f32x4{0.f, 0.f, 0.f, 0.f};
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
  const uint32_t want = split_want(f, ti, 0);  // this call's tag, XCD bits aside
  const uint32_t xcc = xcc_id(), tag = want | xcc;
  uint32_t *const status = flags + (int64_t)kSyncTiles * kSplitFlagWords;
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
  // (the operand arrays are parameters, so that the fallback below holds
  // arrays of its own and these die after the first shrink)
  u32x4 av[kSBatch];
  uint32_t aok = 0;
  auto load_a = [&](int gm, u32x4 (&av)[kSBatch], uint32_t &aok) {  // member gm's A chunk of every slice
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
  load_a(g, av, aok);
  const bool xw = wave < nb;  // this wave shrinks token block `wave`
  const bool xok = xw && 16 * wave + l16 < rows;
  const int xt = wave == 0 ? tok[0] : (wave == 1 ? tok[1] : (wave == 2 ? tok[2] : tok[3]));
  const uint16_t *xbase = reinterpret_cast<const uint16_t *>(p.x) +
                          (xok ? (p.x_row_div == 1 ? (int64_t)xt : (int64_t)xt / p.x_row_div) * p.ldx : 0);
  // x fragments past d_in meet zero A rows, and rows past the tile feed
  // outputs that are never used: both read the row's first values instead
  u32x4 xa[XB];
  auto load_x = [&](int gm, u32x4 (&xa)[XB]) {  // member gm's x fragments of this wave's token block
    const int64_t kx = ((int64_t)gm << p.ksh) + 8 * kg;  // this lane's k at step 0
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int64_t k = kx + 32 * (int64_t)i;
      xa[i] = gload16(xbase + (i < nsteps && k < p.d_in ? k : 0));
    }
  };
  if (xw) load_x(g, xa);
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
  }
  auto load_yv = [&](int t) {  // y of token block t (rows past the tile: unused)
    const int tk = t == 0 ? tok[0] : (t == 1 ? tok[1] : (t == 2 ? tok[2] : tok[3]));
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const bool ok = p.add && qok[q] && 16 * t + l16 < rows;
      yv[q] = *reinterpret_cast<const u32x2 *>(y + (ok ? (int64_t)tk * p.ldy + qcol[q] : 0));
    }
  };
  load_yv(0);
  const int rk = p.slot_rank ? min(max(p.slot_rank[slot], 0), R) : R;
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  if (rk == 0) {  // the adapter adds nothing
    if (!p.add) split_zero(p, tl, rows, gb0, nbm);
    return;
  }
  const int rk8 = (rk + 7) & ~7;  // ranks read, as the other kernels read them

  // ---- A chunk into LDS (ranks past the slot's rank as zeros)
  auto stage_a = [&](const u32x4 (&av)[kSBatch], uint32_t aok) {
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
  __shared__ uint32_t missing_s;  // members whose partials this workgroup computes itself
  if (tid == 0) missing_s = 0;
  stage_a(av, aok);
  __syncthreads();

  // ---- shrink: wave t, all k-steps of token block t.  D' = A^T x^T, so that
  // lane (token l16, kg) ends with ranks 4 kg .. + 3 of its token: the
  // operand layout the expand takes
  const rsrc_t pr = make_rsrc(p.part, p.part_bytes);
  const int fr0 = ((pos0 + 15) >> 4) + ti;  // the tile's first fragment
  auto frag_off = [&](int gg, int t, int s, int c) {
    return (uint32_t)((((gg * p.n_frag + fr0 + t) * p.n_slices + s) * RB + c) * 2048 + lane * 16);
  };
  // member gm's partial rows of token block `wave`, from the staged A chunk
  // and xa, into member gm's slot
  auto shrink_store = [&](int gm, const u32x4 (&xa)[XB]) {
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
        if (s < p.n_slices) store_tagged(pr, frag_off(gm, wave, s, rb), acc[s][rb], tag);
  };
  if (xw) shrink_store(g, xa);
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
  // ---- the count word for the next call (the peers read the partials' own tags)
  if (wave == 0) raise_count(fl, g, G, tag);

  // ---- rendezvous: the members' fragments of token block 0 are polled.
  // Members whose partials do not arrive in time, or arrive tagged by
  // another XCD (whose later blocks could stay in that XCD's L2 until the
  // kernel ends), are computed here, by the same code, so they are the bits
  // those members store themselves; block 0 is then gathered again, from
  // this workgroup's own stores for those members.  The stage (n_slices RB
  // 4 KB) fits the A chunk's region: kc >= 128.
  f32x4 *const stage = reinterpret_cast<f32x4 *>(split_lds);
  const uint32_t plane = (uint32_t)(p.n_frag * p.n_slices * RB * 2048);
  bool regather = false;
  {
    uint32_t off[NS * RB];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int c = 0; c < RB; ++c) off[s * RB + c] = s < p.n_slices ? frag_off(0, 0, s, c) : 0x7FFFFFF0u;
    uint32_t foreign = 0;
    const uint32_t miss = poll_members<NS * RB>(pr, off, plane, p.gsh, p.n_slices * RB, want, xcc, p.spin_limit,
                                                true, stage, &foreign);
    if (miss && lane == 0) atomicOr(&missing_s, miss);
    if (lane == 0) {
      if (miss & ~foreign) atomicAdd(status, 1u);
      if (foreign) atomicAdd(status + 1, 1u);
    }
    __syncthreads();
    const uint32_t m_all = missing_s;
    if (m_all) {
      for (uint32_t m = m_all; m; m &= m - 1) {
        const int gm = __builtin_ctz(m);
        u32x4 av2[kSBatch], xa2[XB];
        uint32_t aok2 = 0;
        load_a(gm, av2, aok2);
        if (xw) load_x(gm, xa2);
        __syncthreads();  // the A chunk's LDS (the stage too) is free
        stage_a(av2, aok2);
        __syncthreads();
        if (xw) shrink_store(gm, xa2);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      load_yv(0);  // again: the block's y is not kept over this path
      regather = true;
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
      if (t > 0 || regather) {  // the fragments of block t (of every member: see above)
        uint32_t foreign = 0;
        const uint32_t miss = poll_members<NS * RB>(pr, off, plane, p.gsh, p.n_slices * RB, want, xcc, kLaterPolls,
                                                    false, stage, &foreign);
        if (miss && lane == 0) atomicAdd(status, 1u);
        __syncthreads();
      }
      stage_sums<NS * RB>(stage, p.n_slices * RB, u);
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
// A chunk in LDS (2), its partial rows stored and the B chunk staged (3), the
// members' first-block partials polled in (4, the rendezvous), the first
// token block's u summed (5) and its y stores acknowledged (6); then (7) ti |
// g << 16 | slice << 24, (8) the HW_ID register, (9) XCC_ID.  Workgroups that
// leave early record nothing.
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
  const uint32_t want = split_want(f, ti, sl);  // this call's tag, XCD bits aside
  const uint32_t xcc = xcc_id(), tag = want | xcc;
  uint32_t *const status = flags + (int64_t)kSyncTiles * kSplitFlagWords;
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
  // (the operand arrays are parameters, so that the fallback below holds
  // arrays of its own and these die after the first shrink)
  u32x4 av[NA];
  auto load_a = [&](int gm, u32x4 (&av)[NA]) {  // member gm's A chunk
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + kSThreads * i;
      av[i] = buf_load16(ar, q < NPA ? (uint32_t)(gm * KC * R * 2 + q * 16) : kOut);
    }
  };
  load_a(g, av);
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
  auto load_x = [&](int gm, u32x4 (&xa)[KS]) {
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
  load_x(g, xa);
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
  // arrives with the rest of the batch, so it does not hold the polls (loads
  // complete in order).  With 1024-row chunks (32 x loads a lane) it is
  // loaded once the partials are stored.
  constexpr bool kYEarly = KS <= 16;
  const rsrc_t yr = make_rsrc(p.y, p.y_bytes);
  const uint32_t yo0 = (uint32_t)((offset + 16 * (gb0 + wave) + 4 * kg) * 2);  // + 128 q: block wave + 4 q
  uint32_t yrow = 0;
  u32x2 yv[QB];
  auto load_y = [&](int t) {  // y of token block t
    const int tk = t == 0 ? tok[0] : (t == 1 ? tok[1] : (t == 2 ? tok[2] : tok[3]));
    yrow = (uint32_t)(tk * p.ldy * 2);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const bool ok = p.add && wave + 4 * q < nbm;
      yv[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(yr, ok ? yrow + yo0 + 128 * q : kOut, 0, 0));
    }
  };
  if constexpr (kYEarly) load_y(0);
  const int rk = p.slot_rank ? min(max(p.slot_rank[slot], 0), R) : R;
  const float sc = p.scale * (p.slot_scale ? p.slot_scale[slot] : 1.f);
  if (rk == 0) {
    if (!p.add) split1_zero(p, tl, rows, gb0, nbm, offset, width);
    return;
  }
  const int rk8 = (rk + 7) & ~7;

  // ---- A chunk into LDS: piece q = row q / (R / 8), ranks 8 (q % (R / 8)) ..
  auto stage_a = [&](const u32x4 (&av)[NA]) {
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
  __shared__ uint32_t missing_s;  // members whose partials this workgroup computes itself
  if (tid == 0) missing_s = 0;
  stage_a(av);
  __syncthreads();
  LORA_PHASE(2);

  // ---- shrink (D' = A^T x^T, so that lane (token l16, kg) ends with ranks
  // 4 kg .. + 3 of its token)
  const rsrc_t pr = make_rsrc(p.part, p.part_bytes);
  const uint32_t fbase = (uint32_t)((((pos0 + 15) >> 4) + ti) * RB * 2048 + lane * 16) + sl * p.part_slice;
  const uint32_t plane = (uint32_t)(p.n_frag * RB * 2048);  // between members
  // member gm's partial rows, from the staged A chunk and xa, into member
  // gm's slot.  Two accumulator chains (even and odd k-steps) added at the
  // end: the MFMAs of one chain wait for each other, the two chains do not.
  // A one-block tile's four waves add their sums in wave order through LDS
  // (RB x 4 waves x 64 lanes, a region of its own after the B chunk), and
  // wave 0 stores them.  Called by every wave.
  f32x4 *const red = reinterpret_cast<f32x4 *>(split_lds + p.bs_off + RP * p.ldb * 2);
  auto shrink_store = [&](int gm, const u32x4 (&xa)[KS]) {
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
          store_tagged(pr, fbase + gm * plane + rb * 2048, ((r4[0] + r4[kWave]) + r4[2 * kWave]) + r4[3 * kWave],
                       tag);
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
        store_tagged(pr, fbase + gm * plane + (wave * RB + rb) * 2048, acc[0][rb] + acc[1][rb], tag);
    }
  };
  shrink_store(g, xa);
  // ---- B chunk into LDS (rank rows past the slot's rank as zeros)
#pragma unroll
  for (int i = 0; i < NBQ; ++i) {
    const int q = tid + kSThreads * i;
    if (q < 2 * RP * bpm) {
      const int lb = q / (2 * RP), j = (q >> 1) % RP, half = q & 1;
      *reinterpret_cast<u32x4 *>(Bs + j * p.ldb + 16 * lb + 8 * half) = j < rk8 ? bv[i] : u32x4{0, 0, 0, 0};
    }
  }
  // ---- the count word for the next call (the peers read the partials' own
  // tags); the B chunk is staged before any wave reads it
  if (wave == 0) raise_count(fl, g, G, tag);
  __syncthreads();
  LORA_PHASE(3);
  if constexpr (!kYEarly) load_y(0);

  // ---- rendezvous: the members' fragments of token block 0 are polled.
  // Members whose partials do not arrive in time, or arrive tagged by
  // another XCD (whose later blocks could stay in that XCD's L2 until the
  // kernel ends), are computed here, by the same code, so they are the bits
  // those members store themselves (a late member and this workgroup then
  // write equal values); block 0 is then gathered again, from this
  // workgroup's own stores for those members.
  f32x4 *const stage = reinterpret_cast<f32x4 *>(split_lds);
  bool regather = false;
  {
    uint32_t off[RB];
#pragma unroll
    for (int c = 0; c < RB; ++c) off[c] = fbase + c * 2048;
    uint32_t foreign = 0;
    const uint32_t miss = poll_members<RB>(pr, off, plane, p.gsh, RB, want, xcc, p.spin_limit, true, stage, &foreign);
    if (miss && lane == 0) atomicOr(&missing_s, miss);
    if (lane == 0) {
      if (miss & ~foreign) atomicAdd(status, 1u);
      if (foreign) atomicAdd(status + 1, 1u);
    }
    __syncthreads();
    const uint32_t m_all = missing_s;
    if (m_all) {
      for (uint32_t m = m_all; m; m &= m - 1) {
        const int gm = __builtin_ctz(m);
        u32x4 av2[NA], xa2[KS];
        load_a(gm, av2);
        load_x(gm, xa2);
        __syncthreads();  // the A chunk's LDS (the stage too) is free
        stage_a(av2);
        __syncthreads();
        shrink_store(gm, xa2);
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (kYEarly) load_y(0);  // again: the block's y is not kept over this path
      regather = true;
    }
  }
  LORA_PHASE(4);

  // ---- expand, token block by token block: u = scale * (members' partials
  // in the gather's fixed order) as bf16 hi + lo operands; every column block
  // of this wave (a block past the member's share reads block 0 and stores
  // nothing).  Each block's y is stored as soon as its two products are done:
  // that measured faster than issuing every product first, and than one
  // 16x16x32 product with hi and lo as the two halves of K.
  for (int t = 0; t < nb; ++t) {
    s16x4 uh[RB], ul[RB];
    {
      f32x4 u[RB];
      if (t > 0 || regather) {  // the fragments of block t (of every member: see above)
        uint32_t off[RB];
#pragma unroll
        for (int c = 0; c < RB; ++c) off[c] = fbase + (t * RB + c) * 2048;
        uint32_t foreign = 0;
        const uint32_t miss = poll_members<RB>(pr, off, plane, p.gsh, RB, want, xcc, kLaterPolls, false, stage, &foreign);
        if (miss && lane == 0) atomicAdd(status, 1u);
        __syncthreads();
      }
      stage_sums<RB>(stage, RB, u);
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
    // B^T operands of this wave's column blocks (the B chunk stays in LDS)
    s16x4 bw[QB][RB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int lb = wave + 4 * q < nbm ? wave + 4 * q : 0;
#pragma unroll
      for (int c = 0; c < RB; ++c) bw[q][c] = lds_col4(Bs, p.ldb, 16 * c + 4 * kg, 16 * lb);
    }
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
    if (t + 1 < nb) {
      load_y(t + 1);
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
  return (size_t)kSplitMembers * n_frag * n_slices * (RP / 16) * 2048;  // tagged fragments of 2048 bytes
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
  const size_t need = (size_t)G * ((T + 15) / 16 + mt) * n_slices * RB * 2048;
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
  p.part_slice = (uint32_t)((size_t)pl.G * sp.n_frag * RB * 2048);
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
  if (max_tiles(meta.T, meta.S) > kSyncTiles) return hipSuccess;  // tiles past the count words
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

#ifdef LORA_PHASE_CLOCK
unsigned long long *phase_clock_buffer(size_t *words) {
  *words = g_phase_words;
  return g_phase_clock;
}
int phase_clock_kernel() {
  const char *k = getenv("LORA_PHASE_KERNEL");
  if (!k) return 0;
  return strcmp(k, "shrink") == 0 ? 1 : (strcmp(k, "expand") == 0 ? 2 : 0);
}
#else
unsigned long long *phase_clock_buffer(size_t *words) {
  *words = 0;
  return nullptr;
}
int phase_clock_kernel() { return 0; }
#endif

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
