// gemm_tile.hip -- the DualScale x SegLinear W8A8 linear layer as one gfx950
// kernel launch (large M).
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes): "DualScale" section
//      (split, scales, reconstruction; both polarity products run as one
//      batched launch with the scaled results combined in a fused epilogue)
//      and "SegLinear" section (input-segmented sum over K-segments).
// [P2] "SegQuant" (hliangzhao.me): section 3, the same reconstruction and
//      one batched integer GEMM with a fused epilogue.
//
// Design (CDNA4, written for gfx950 rather than after the pages' CUTLASS
// kernel):
//   * A workgroup of 4 waves (one per SIMD) owns a BM x BN output tile.  K is
//     walked in LDS stages of 128 (two 64-wide k-steps; K-segment boundaries
//     are multiples of 64, so a k-step never straddles two segments), one
//     barrier per stage.  The products run on the int8 32x32x32 matrix-core
//     instruction.
//   * Wave w owns output columns [w*BN/4, (w+1)*BN/4) for all BM rows.  The
//     packed weight (lane-ordered 1 KiB tiles of 64 k x 16 n) gives every
//     lane its 16-byte piece of a 32x32x32 B operand as one buffer load
//     (wave-uniform base and k offset, a fixed per-lane offset), so the
//     weight goes from memory straight into registers, never through LDS;
//     each operand register is refilled with the stage two ahead right after
//     its last use.  Both polarity halves multiply the same B registers.
//   * The activation tile (BM x 128) is shared through LDS: every thread
//     loads 16-byte pieces of bf16 X into register slots (three stages
//     ahead with one K-segment, two when segments are folded and the
//     registers are needed for the fp32 sums), quantises them one stage
//     ahead (the sign picks the half's inverse scale, one fp32 multiply,
//     clamp, round half to even) and writes the codes as two int8 planes
//     (X+, X-), rows padded to 144 bytes so that the 16-byte operand reads
//     are free of bank conflicts.  Pre-quantised int8 input skips the
//     arithmetic.  In the single-segment loop the quantisation of a stage
//     is spread over all four sub-blocks, one piece beside each twelve
//     matrix-core instructions.
//   * Single-scale modes (the W8A8 baseline): one plane of signed codes, one
//     product per block, the + half's scales only.
//   * The stage loop is straight-line: prefetch indices are clamped instead
//     of branched on, K is padded to whole stage pairs with zero codes, and
//     per-segment values (ends, scales, inverse scales) are read from tables
//     spread across the lanes with wave-uniform indices, so no vector load
//     or LDS access ever waits behind the prefetches it should overlap.
//   * Folding K-segments (the pages' reconstruction):
//       SINGLE  one K-segment: int32 sums over all of K, scaled once at the
//               end: y = s_w*s+*A+ + s_w*s-*A-.
//       STEP    every K-segment is one 64-wide k-step (one attention head per
//               segment): each k-step's products start from zero and are
//               folded into an fp32 sum held in registers.
//       MULTI   general segments on bf16 input with K up to 132104
//               (MULTI64 when a segment ends inside a 128-wide stage; other
//               multi-segment calls go to the LDS-staged kernel of
//               gemm_lds.hip).  The int32 sums S run over all of K and are
//               never reset; at the end of segment i the fold adds
//               (c_i - c_{i+1}) * S_i (c_i = s_i * s_w,i per column and half,
//               c past the last segment = 0), which telescopes to
//               sum_i c_i * A_i.  The fp32 sum lives in registers.  (The variant
//               that dumps accumulators dumps the S_i; a second launch turns
//               them into the per-segment sums.)
//   * Tile shapes: 64 x 384 for one K-segment (one workgroup per CU), or
//     32 x 128 when that would leave most CUs idle (two workgroups per CU);
//     32 x 256 for STEP, 64 x 256 for MULTI.
//   * Workgroup -> tile order is XCD-aware: workgroups are dealt to the 8
//     XCDs round-robin, so XCD x is given one contiguous range of logical
//     tiles, ordered in groups of 8 row tiles so that the tiles an XCD runs
//     at once share weight and activation slices in its L2.
#include <stddef.h>

#include <type_traits>

#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kAPitch = 144;  // bytes per LDS row of one A plane (128 + 16 pad)
constexpr int kBK = 128;      // K per LDS stage
constexpr int kSmallTileGrid = 128;  // single segment: below this many 64 x 384 tiles, use 32 x 128
// MULTI keeps int32 sums over all of K: |sum| <= K * 128 * 127 < 2^31
constexpr int64_t kRunningSumMaxK = 132104;

// Activation input: bf16 (quantised here), signed codes, two planes; and the
// single-scale forms of the first two (one product on the signed code, the
// + half's scales for both signs).
enum AMode { A_BF16 = 0, A_SIGNED = 1, A_PLANES = 2, A_BF16_1 = 3, A_SIGNED_1 = 4 };
// MULTI folds at stage ends (every segment end but the last on a multiple of
// 128); MULTI64 checks after every 64-wide k-step.
enum Mode { SINGLE = 0, STEP = 1, MULTI = 2, MULTI64 = 3 };

template <int V>
using ic = std::integral_constant<int, V>;

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct TileArgs {
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  const uint16_t *x;
  int64_t ld_x;
  const int8_t *xq;
  int64_t ld_q;
  int64_t plane_stride;
  const int8_t *w;
  const float *w_scale;
  const float *act;  // [4][n_kseg]
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc;  // [2][n_kseg][M][N] or null
  int32_t n_kseg;
  int32_t seg_end_tile[kMaxKSeg];  // exclusive end of each segment, in k-tiles of 64
};

// Activation pieces quantised in 32-k sub-block ks of a stage: piece i goes
// to sub-block (3 i) / xp (none to the last one, which follows the barrier).
constexpr int pieces_in_sub(int xp, int ks) {
  int n = 0;
  for (int i = 0; i < xp; ++i) n += (i * 3) / xp == ks ? 1 : 0;
  return n;
}

// With bf16 input in the single-segment loop (three activation slots, four
// pieces a stage) the quantisation is spread over all four sub-blocks: pieces
// 0-2 of stage u + 1 in sub-blocks 0-2 of stage u, and piece 3 of stage u + 2
// in sub-block 3 (after the barrier; its buffer was last read in stage u - 1).
// Each sub-block then carries one piece's vector ALU work beside its twelve
// matrix-core instructions instead of two, one, one and none.
constexpr bool spread_quant(int mode, int amode, int xp) {
  return mode == 0 && (amode == 0 || amode == 3) && xp == 4;
}

// Segment end i, read straight from the kernel-argument segment (the
// argument is the only one, at offset 0).  Indexing the by-value argument
// itself with a run-time index would make the compiler copy all of it into
// scratch memory first.
__device__ __forceinline__ int seg_end_at(int i) {
  const char *base = (const char *)__builtin_amdgcn_kernarg_segment_ptr();
  return reinterpret_cast<const int32_t *>(base + offsetof(TileArgs, seg_end_tile))[i];
}

__device__ __forceinline__ v16i mfma32(const v4u &a, const v4u &b, const v16i &c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(reinterpret_cast<const v4i &>(a),
                                               reinterpret_cast<const v4i &>(b), c, 0, 0, 0);
}

template <int BM, int BN, int AMODE, int MODE, bool DEBUG>
__global__ __launch_bounds__(256, (BM == 32 && (MODE == SINGLE || (AMODE != A_BF16 && AMODE != A_BF16_1))) ? 2 : 1) void gemm_tile_kernel(TileArgs a) {
  constexpr int WN = BN / 4;   // columns per wave
  constexpr int MB = BM / 32;  // 32-row blocks
  constexpr int NB = WN / 32;  // 32-column blocks per wave
  constexpr int A_PLANE = BM * kAPitch, A_STAGE = 2 * A_PLANE;
  // 16-byte activation pieces per thread per stage
  constexpr bool IN_BF16 = AMODE == A_BF16 || AMODE == A_BF16_1;
  constexpr bool ONE = AMODE == A_BF16_1 || AMODE == A_SIGNED_1;  // single scale
  constexpr int XP = (AMODE == A_SIGNED || AMODE == A_SIGNED_1) ? BM / 32 : BM / 16;
  static_assert(BM % 32 == 0 && WN % 32 == 0, "tile sizes");

  // three stage buffers of quantised planes: stage u is read from buffer
  // u % 3 while stage u + 1 is written to (u + 1) % 3, so one barrier per
  // stage suffices and it can sit before the stage's last sub-block
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * A_STAGE];


  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // ---- tile of this workgroup (XCD-aware order) ----
  const int T = a.tiles_m * a.tiles_n;
  int logical;
  {
    const int bid = blockIdx.x, per = T / 8, rem = T % 8, x = bid % 8, i = bid / 8;
    logical = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  }
  // Logical order: groups of up to 8 row tiles, within a group the row
  // tile fastest.  The 32 workgroups an XCD runs at once then cover about 8
  // row tiles x 4 column tiles, so each weight slice is read by 8 of them
  // and each activation slice by 4 while it is in that XCD's L2.
  int tm, tn;
  {
    const int GM = min(8, a.tiles_m);
    const int group = logical / (GM * a.tiles_n);
    const int first_m = group * GM;
    const int gm = min(a.tiles_m - first_m, GM);
    const int in = logical - group * GM * a.tiles_n;
    tm = first_m + in % gm;
    tn = in / gm;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = a.K / 64, NT = a.N / 16;
  const int KS = (KT + 1) / 2;    // stages
  const int KSV = (KS + 1) & ~1;  // stages rounded up to pairs (padding: zero codes)

  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;
  const float *i_pos = a.act + 2 * nS, *i_neg = a.act + 3 * nS;

  // ---- weight stream: 32x32x32 B operands straight into registers ----
  // Lane l of block nb, 32-k sub-block ks of a stage reads 16 bytes of the
  // 1 KiB tile (n-tile nt, k-tile 2u + ks/2) at g*256 + j*16: column
  // j = l % 16 of n-tile 2*nb + (l % 32) / 16, k group g = 2*(ks % 2) + l / 32.
  // Buffer loads from the wave's first n-tile: the base and the k-tile
  // offset are wave-uniform (scalar registers), each lane adds a fixed
  // 32-bit offset, so a load costs no vector address arithmetic.
  const int lane_j = lane & 15, lane_g = lane >> 5;
  const int nt_wave = n0 / 16 + wave * (WN / 16);
  const int nt_base = min(nt_wave, NT - 1);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t *>(a.w + (int64_t)nt_base * KT * 1024), 0, 0x7fffffff, 0x00020000);
  int woff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // n-tiles past N read the last valid tile: those columns are never stored
    const int nt = min(nt_wave + 2 * nb + ((lane & 31) >> 4), NT - 1);
    woff[nb] = (nt - nt_base) * KT * 1024 + lane_j * 16 + lane_g * 256;
  }
  v4u wr[2][NB][4];
  auto load_w1 = [&](auto SLOT, int nb, int ks, int u) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    const int kt = min(2 * u + (ks >> 1), KT - 1);
    wr[s][nb][ks] = __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, woff[nb] + (ks & 1) * 512, kt * 1024, 0));
  };

  // ---- activation stream: 16-byte pieces, three stages ahead ----
  // bf16:   piece i of thread t is row i*16 + t/16, elements (t%16)*8 .. +8 of
  //         the stage (256 bytes a row, 16 lanes a row: coalesced).
  // signed: piece i is row i*32 + t/8, codes (t%8)*16 .. +16.
  // planes: as signed, the first BM/32 pieces from the + plane, then the -.
  // A thread's pieces lie in one 64-wide half of the stage (k-tile 2u or
  // 2u+1); a half past K loads the last k-tile instead (in bounds) and
  // stores zero codes.
  const int my_half = IN_BF16 ? (tid & 15) >> 3 : (tid & 7) >> 2;
  const int half_off = IN_BF16 ? (tid & 7) * 8 : (tid & 3) * 16;  // elements
  // XS register slots: stage v's pieces go to slot v % XS, loaded at the
  // start of stage v - XS and quantised during stage v - 1 (XS - 1 stages of
  // memory latency hidden).  Three for the single-segment loop; the fold
  // modes need the registers and keep two.
  constexpr int XS = (MODE == SINGLE && BM == 64) ? 3 : 2;
  constexpr bool SPREAD = spread_quant(MODE, AMODE, XP);
  v4u xr[XS][XP];
  auto load_x = [&](auto SLOT, int u) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    const int kt = min(2 * min(u, KS - 1) + my_half, KT - 1);
    const int64_t col = (int64_t)kt * 64 + half_off;  // element column of the piece
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint8_t *p;
      if (IN_BF16) {
        const int m = min(m0 + i * 16 + (tid >> 4), a.M - 1);  // rows past M: any valid row
        p = reinterpret_cast<const uint8_t *>(a.x) + ((int64_t)m * a.ld_x + col) * 2;
      } else {
        const int half = AMODE == A_PLANES ? i / (BM / 32) : 0;
        const int ii = AMODE == A_PLANES ? i % (BM / 32) : i;
        const int m = min(m0 + ii * 32 + (tid >> 3), a.M - 1);
        p = reinterpret_cast<const uint8_t *>(a.xq) + half * a.plane_stride + (int64_t)m * a.ld_q + col;
      }
      xr[s][i] = *reinterpret_cast<const v4u *>(p);
    }
  };

  // quantise (or split) piece i of X slot SLOT into the stage buffer at `buf`
  auto quant_piece = [&](auto SLOT, int i, uint8_t *buf, float inv_pos, float inv_neg,
                         bool valid) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    uint8_t *ap = buf;
    uint8_t *an = buf + A_PLANE;
    v4u xv = xr[s][i];
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[e] = valid ? xv[e] : 0u;
    if (AMODE == A_BF16_1) {  // one plane of signed codes, the + half's inverse for both signs
      const int off = (i * 16 + (tid >> 4)) * kAPitch + (tid & 15) * 8;
      *reinterpret_cast<v2u *>(ap + off) = quant8_signed(xv, inv_pos, inv_pos);
    } else if (AMODE == A_SIGNED_1) {
      const int off = (i * 32 + (tid >> 3)) * kAPitch + (tid & 7) * 16;
      *reinterpret_cast<v4u *>(ap + off) = xv;
    } else if (AMODE == A_BF16) {
      const int off = (i * 16 + (tid >> 4)) * kAPitch + (tid & 15) * 8;
      v2u p, n;
      quant8_planes(xv, inv_pos, inv_neg, p, n);
      *reinterpret_cast<v2u *>(ap + off) = p;
      *reinterpret_cast<v2u *>(an + off) = n;
    } else if (AMODE == A_SIGNED) {
      const int off = (i * 32 + (tid >> 3)) * kAPitch + (tid & 7) * 16;
      v4u p, n;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t pp, nn;
        split_signed(xv[j], pp, nn);
        p[j] = pp;
        n[j] = nn;
      }
      *reinterpret_cast<v4u *>(ap + off) = p;
      *reinterpret_cast<v4u *>(an + off) = n;
    } else {
      const int half = i / (BM / 32), ii = i % (BM / 32);
      const int off = (ii * 32 + (tid >> 3)) * kAPitch + (tid & 7) * 16;
      *reinterpret_cast<v4u *>((half ? an : ap) + off) = xv;
    }
  };

  // A-operand fragments of one 32-k sub-block, double-buffered
  v4u fa[2][MB], fb[2][MB];
  const int arow = (lane & 31) * kAPitch + lane_g * 16;
  auto read_frags = [&](auto SLOT, const uint8_t *buf, int ks) __attribute__((always_inline)) {
    constexpr int f = decltype(SLOT)::value;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      fa[f][mb] = *reinterpret_cast<const v4u *>(buf + arow + mb * 32 * kAPitch + ks * 32);
      if (!ONE) fb[f][mb] = *reinterpret_cast<const v4u *>(buf + A_PLANE + arow + mb * 32 * kAPitch + ks * 32);
    }
  };

  // ---- accumulators ----
  v16i accp[MB][NB], accn[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      accp[i][j] = v16i{};
      accn[i][j] = v16i{};
    }
  constexpr bool YREG = MODE != SINGLE;  // fp32 sums of the segment folds
  constexpr int YM = YREG ? MB : 1, YN = YREG ? NB : 1;
  v16f yacc[YM][YN];
#pragma unroll
  for (int i = 0; i < YM; ++i)
#pragma unroll
    for (int j = 0; j < YN; ++j) yacc[i][j] = v16f{};

  // 32x32 output block: lane l holds column l % 32 and, in register r, row
  // (r / 4) * 8 + (l / 32) * 4 + r % 4.
  const int col_lane = n0 + wave * WN + (lane & 31);
  const int row_lane = m0 + (lane >> 5) * 4;
  auto out_row = [&](int mb, int r) __attribute__((always_inline)) { return row_lane + mb * 32 + (r >> 2) * 8 + (r & 3); };

  auto dump = [&](int seg, int mb, int nb, const v16i &p, const v16i &n) __attribute__((always_inline)) {
    const int col = col_lane + 32 * nb;
    if (col >= a.N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = out_row(mb, r);
      if (m >= a.M) continue;
      const int64_t o = ((int64_t)seg * a.M + m) * a.N + col;
      a.acc[o] = p[r];
      if (!ONE) a.acc[(int64_t)nS * a.M * a.N + o] = n[r];
    }
  };

  // weight scale of segment `seg` (clamped) for this lane's column of block nb
  auto col_ws = [&](int seg, int nb) __attribute__((always_inline)) {
    const int col = min(col_lane + 32 * nb, a.N - 1);  // past N: never stored
    return a.w_scale[(int64_t)min(seg, nS - 1) * a.N + col];
  };

  // ---- per-segment tables, held across lanes ----
  // Lane l of entry j holds segment 64 j + l (clamped).  Looked up with
  // readlane, so the index must be wave-uniform; no scalar-memory loads in
  // the stage loop, whose results would need a wait for every outstanding
  // LDS access.
  int t_end[2];
  float t_sp[2], t_sn[2], t_ip[2], t_in[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sg = min(64 * j + lane, nS - 1);
    t_end[j] = seg_end_at(sg);
    t_sp[j] = s_pos[sg];
    t_sn[j] = s_neg[sg];
    t_ip[j] = i_pos[sg];
    t_in[j] = i_neg[sg];
  }
  auto seg_i = [&](const int (&t)[2], int idx) __attribute__((always_inline)) {
    const int lo = __builtin_amdgcn_readlane(t[0], idx & 63);
    const int hi = __builtin_amdgcn_readlane(t[1], idx & 63);
    return idx < 64 ? lo : hi;
  };
  auto seg_f = [&](const float (&t)[2], int idx) __attribute__((always_inline)) {
    const int lo = __builtin_amdgcn_readlane(__float_as_int(t[0]), idx & 63);
    const int hi = __builtin_amdgcn_readlane(__float_as_int(t[1]), idx & 63);
    return __int_as_float(idx < 64 ? lo : hi);
  };

  // ---- fold state ----
  // STEP: the scales of the k-step being folded, fetched a stage ahead.
  // MULTI: the column scales of the current and the next segment.
  float wsa[NB], wsb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    wsa[nb] = col_ws(0, nb);
    wsb[nb] = MODE == SINGLE ? 0.0f : col_ws(1, nb);
  }
  // STEP: s+/s- of the k-steps being folded (even in *a, odd in *b)
  float spa = seg_f(t_sp, 0), sna = seg_f(t_sn, 0);
  float spb = seg_f(t_sp, min(1, nS - 1)), snb = seg_f(t_sn, min(1, nS - 1));

  // STEP: fold k-step t into the fp32 registers (products started from 0)
  auto fold_step = [&](int t) __attribute__((always_inline)) {
    const float sp = (t & 1) ? spb : spa, sn = (t & 1) ? snb : sna;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float ws = (t & 1) ? wsb[nb] : wsa[nb];
      const float cp = sp * ws, cn = sn * ws;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (DEBUG && t < KT) dump(t, mb, nb, accp[mb][nb], accn[mb][nb]);
        v16f &yv = yacc[YREG ? mb : 0][YREG ? nb : 0];
#pragma unroll
        for (int r = 0; r < 16; ++r) {  // element by element: few temporaries
          const float t = __builtin_fmaf(cp, (float)accp[mb][nb][r], yv[r]);
          yv[r] = ONE ? t : __builtin_fmaf(cn, (float)accn[mb][nb][r], t);
        }
      }
    }
  };

  // MULTI: fold at the end of segment seg into the fp32 registers
  auto fold_multi = [&](int seg) __attribute__((always_inline)) {
    const float sp = seg_f(t_sp, seg), sn = seg_f(t_sn, seg);
    const bool last = seg + 1 >= nS;
    const float sp1 = last ? 0.0f : seg_f(t_sp, min(seg + 1, nS - 1));
    const float sn1 = last ? 0.0f : seg_f(t_sn, min(seg + 1, nS - 1));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // telescoped: S_i * (c_i - c_{i+1})
      const float cp = sp * wsa[nb] - sp1 * wsb[nb], cn = sn * wsa[nb] - sn1 * wsb[nb];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // (the dump holds the running sums S_i; the launcher differences them)
        if (DEBUG) dump(seg, mb, nb, accp[mb][nb], accn[mb][nb]);
        v16f &yv = yacc[YREG ? mb : 0][YREG ? nb : 0];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = __builtin_fmaf(cp, (float)accp[mb][nb][r], yv[r]);
          yv[r] = ONE ? t : __builtin_fmaf(cn, (float)accn[mb][nb][r], t);
        }
      }
      wsa[nb] = wsb[nb];
      wsb[nb] = col_ws(seg + 2, nb);
    }
  };

  // ---- segment of each half of the stage being quantised (wave-uniform) ----
  // k-tiles only move forward, so each index only grows; a stage advances a
  // half by 2 k-tiles, so at most two steps per stage.
  // Branch-free on purpose: as branches, the compiler carried the condition
  // through a vector register that an in-flight load targets, and waited for
  // every outstanding prefetch (vmcnt(0)) twice a stage.
  auto advance = [&](int &sg, int kt) __attribute__((always_inline)) {
    const int in_k = kt < KT ? 1 : 0;
    const int e1 = seg_i(t_end, sg);  // sg < nS throughout
    sg = min(sg + (in_k & (kt >= e1 ? 1 : 0)), nS - 1);
    const int e2 = seg_i(t_end, sg);
    sg = min(sg + (in_k & (kt >= e2 ? 1 : 0)), nS - 1);
  };
  int q_lo = 0, q_hi = 0;  // segments of k-tiles 2v, 2v+1 of the stage v being quantised
  const float ip0 = i_pos[0], in0 = i_neg[0];

  // ---- prologue ----
  // (activation first, then weights: the loop's waits are computed from the
  // order of loads on entry as well as in steady state, and this order keeps
  // the two alike, so no wait in the loop is stricter than it needs to be)
  load_x(ic<0>{}, 0);
  load_x(ic<1>{}, 1);
  if (XS == 3) load_x(ic<XS == 3 ? 2 : 0>{}, 2);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) load_w1(ic<0>{}, nb, ks, 0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) load_w1(ic<1>{}, nb, ks, 1);
  {
    float ip = ip0, in = in0;
    if (MODE != SINGLE) {
      advance(q_hi, 1);
      // (the table look-up needs a wave-uniform index: read both halves'
      // scales, then pick per lane)
      const float ip_lo = seg_f(t_ip, q_lo), ip_hi = seg_f(t_ip, q_hi);
      const float in_lo = seg_f(t_in, q_lo), in_hi = seg_f(t_in, q_hi);
      ip = my_half ? ip_hi : ip_lo;
      in = my_half ? in_hi : in_lo;
    }
#pragma unroll
    for (int i = 0; i < XP; ++i) quant_piece(ic<0>{}, i, smem, ip, in, my_half < KT);
    // (spread: piece 3 of stage 1 belongs to the sub-block 3 of a stage -1)
    if (SPREAD) quant_piece(ic<1>{}, XP - 1, smem + A_STAGE, ip, in, 2 + my_half < KT);
  }
  __syncthreads();
  read_frags(ic<0>{}, smem, 0);

  int seg = 0;                        // MULTI: segment of the k-step being multiplied
  int next_end = seg_i(t_end, 0);     // MULTI: its end, in k-tiles

  // one stage u; S = u % 2 (weight slots), S3 = u % 3 (activation slots)
  auto stage = [&](auto S, auto S3, int u) __attribute__((always_inline)) {
    constexpr int s = decltype(S)::value;
    constexpr int s3 = decltype(S3)::value;
    // segments and inverse scales of the stage being quantised (u + 1)
    float q_ip = ip0, q_in = in0;
    if (MODE != SINGLE) {
      advance(q_lo, 2 * (u + 1));
      q_hi = max(q_hi, q_lo);
      advance(q_hi, 2 * (u + 1) + 1);
      const float ip_lo = seg_f(t_ip, q_lo), ip_hi = seg_f(t_ip, q_hi);
      const float in_lo = seg_f(t_in, q_lo), in_hi = seg_f(t_in, q_hi);
      q_ip = my_half ? ip_hi : ip_lo;
      q_in = my_half ? in_hi : in_lo;
    }
    // activation of stage u + XS (into slot u % XS, whose stage u was
    // quantised during stage u - 1)
    constexpr int x_load = XS == 3 ? s3 : s, x_quant = XS == 3 ? (s3 + 1) % 3 : 1 - s;
    load_x(ic<x_load>{}, u + XS);
    const int b_rd = u % 3;
    const int b_wr = b_rd == 2 ? 0 : b_rd + 1;
    const uint8_t *rd = smem + b_rd * A_STAGE;
    uint8_t *wrb = smem + b_wr * A_STAGE;
    const bool q_valid = 2 * (u + 1) + my_half < KT;  // halves past K store zeros
    // Four 32-k sub-blocks.  Each issues the operand reads of the next one
    // first, then its matrix-core work, with a share of the quantisation of
    // stage u + 1 (into buffer b_wr) and the weight refills for stage u + 2
    // between the matrix-core instructions.  The barrier comes before the
    // last sub-block: by then every wave has written its share of stage
    // u + 1, so the last sub-block can already read the first operands of
    // stage u + 1 (and buffer b_wr was last read in stage u - 2).
    auto sub = [&](auto KS) __attribute__((always_inline)) {
      constexpr int ks = decltype(KS)::value;
      if (ks == 3) {
        __syncthreads();
        read_frags(ic<0>{}, wrb, 0);
      } else if (ks == 0 || ks == 2) {
        read_frags(ic<1>{}, rd, ks + 1);
      } else {
        read_frags(ic<0>{}, rd, ks + 1);
      }
      // the reads stay ahead of this sub-block's matrix-core work, which
      // hides their latency (left to itself the scheduler sinks them below)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const v4u &xa = (ks & 1) ? fa[1][mb] : fa[0][mb];
          const v4u &xb = (ks & 1) ? fb[1][mb] : fb[0][mb];
          if (MODE == STEP && (ks & 1) == 0) {  // a k-step's products start from 0
            accp[mb][nb] = mfma32(xa, wr[s][nb][ks], v16i{});
            if (!ONE) accn[mb][nb] = mfma32(xb, wr[s][nb][ks], v16i{});
          } else {
            accp[mb][nb] = mfma32(xa, wr[s][nb][ks], accp[mb][nb]);
            if (!ONE) accn[mb][nb] = mfma32(xb, wr[s][nb][ks], accn[mb][nb]);
          }
        }
        load_w1(ic<s>{}, nb, ks, u + 2);  // refill with the stage two ahead
      }
      // this sub-block's share of the quantisation of stage u + 1
      if (SPREAD) {
        if (ks < 3) {
          quant_piece(ic<x_quant>{}, ks, wrb, q_ip, q_in, q_valid);
        } else {  // piece 3 of stage u + 2: slot and buffer (u + 2) % 3
          uint8_t *wrb2 = smem + (b_rd == 0 ? 2 : b_rd - 1) * A_STAGE;
          quant_piece(ic<SPREAD ? (s3 + 2) % 3 : 0>{}, XP - 1, wrb2, q_ip, q_in,
                      2 * (u + 2) + my_half < KT);
        }
      } else {
#pragma unroll
        for (int i = 0; i < XP; ++i)
          if ((i * 3) / XP == ks) quant_piece(ic<x_quant>{}, i, wrb, q_ip, q_in, q_valid);
      }
      {
        // Interleave: one matrix-core instruction, then an even share of the
        // vector ALU work (quantisation), the weight refills spread among
        // them, the LDS writes last.  Without it the ALU work comes in
        // clumps of ~100 instructions during which the matrix cores idle.
        constexpr int NMF = (ONE ? 1 : 2) * MB * NB;
        constexpr int nq = SPREAD ? 1 : pieces_in_sub(XP, ks);
        constexpr int vpq = AMODE == A_BF16 ? 56 : AMODE == A_BF16_1 ? 38 : AMODE == A_SIGNED ? 16 : 0;
        constexpr int vfold = (MODE == STEP && (ks & 1)) ? MB * NB * 16 * (ONE ? 2 : 4) : 0;
        constexpr int per = (nq * vpq + vfold + NMF - 1) / NMF + 1;
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, per, 0);  // VALU
          if (j % (NMF / NB) == NMF / NB - 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 16, 0);  // LDS writes
      }
      if (ks & 1) {
        const int t = 2 * u + (ks >> 1);  // the k-step that just ended
        if (MODE == STEP) {
          fold_step(t);
          // the scales of k-step t + 2, which reuses this slot
          const int sg = min(t + 2, nS - 1);
          if (t & 1) {
            spb = seg_f(t_sp, sg);
            snb = seg_f(t_sn, sg);
          } else {
            spa = seg_f(t_sp, sg);
            sna = seg_f(t_sn, sg);
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            if (t & 1) wsb[nb] = col_ws(t + 2, nb);
            else wsa[nb] = col_ws(t + 2, nb);
          }
        } else if ((MODE == MULTI64 || (MODE == MULTI && ks == 3)) && t + 1 >= next_end) {
          // (>=: at a stage end, a segment that ends with K on an odd k-tile
          // has ended one padding k-step before)
          fold_multi(seg);
          ++seg;
          next_end = seg < nS ? seg_i(t_end, seg) : 1 << 30;
        }
      }
      // keep the next sub-block's operand reads and refills below this one:
      // hoisted, they would hold two copies of the operands live at once
      __builtin_amdgcn_sched_barrier(0);
    };
    sub(ic<0>{});
    sub(ic<1>{});
    sub(ic<2>{});
    sub(ic<3>{});
  };

  // six stages per iteration when the activation slots repeat every 3 (the
  // weight slots every 2), then the remaining 0, 2 or 4 stages
  int u0 = 0;
  if (XS == 2) {
    for (; u0 < KSV; u0 += 2) {
      stage(ic<0>{}, ic<0>{}, u0);
      stage(ic<1>{}, ic<0>{}, u0 + 1);
    }
  }
  for (; u0 + 6 <= KSV; u0 += 6) {
    stage(ic<0>{}, ic<0>{}, u0);
    stage(ic<1>{}, ic<1>{}, u0 + 1);
    stage(ic<0>{}, ic<2>{}, u0 + 2);
    stage(ic<1>{}, ic<0>{}, u0 + 3);
    stage(ic<0>{}, ic<1>{}, u0 + 4);
    stage(ic<1>{}, ic<2>{}, u0 + 5);
  }
  if (u0 + 2 <= KSV) {
    stage(ic<0>{}, ic<0>{}, u0);
    stage(ic<1>{}, ic<1>{}, u0 + 1);
  }
  if (u0 + 4 <= KSV) {
    stage(ic<0>{}, ic<2>{}, u0 + 2);
    stage(ic<1>{}, ic<0>{}, u0 + 3);
  }

  // ---- epilogue: bf16 store ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = col_lane + 32 * nb;
    float cp = 0.0f, cn = 0.0f;
    if (MODE == SINGLE) {
      cp = s_pos[0] * wsa[nb];
      cn = s_neg[0] * wsa[nb];
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (MODE == SINGLE && DEBUG) dump(0, mb, nb, accp[mb][nb], accn[mb][nb]);
      v16f v;
      if (MODE == SINGLE) {
        const v16f P = __builtin_convertvector(accp[mb][nb], v16f);
        if (ONE) {
          v = v16f(cp) * P;
        } else {
          const v16f Q = __builtin_convertvector(accn[mb][nb], v16f);
          v = __builtin_elementwise_fma(v16f(cn), Q, v16f(cp) * P);
        }
      } else {
        v = yacc[YREG ? mb : 0][YREG ? nb : 0];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = out_row(mb, r);
        if (m < a.M && col < a.N) a.y[(int64_t)m * a.ld_y + col] = (uint16_t)f32_to_bf16_rne(v[r]);
      }
    }
  }
}

// The accumulator dump of a multi-segment launch holds running sums S_i;
// turn them into per-segment sums A_i = S_i - S_{i-1} (exact in int32).
// (planes: 2, or 1 when only the single-scale product was dumped)
__global__ __launch_bounds__(256) void acc_difference_kernel(int32_t *acc, int n_kseg, int64_t mn,
                                                             int planes) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= planes * mn) return;
  const int64_t h = e / mn, o = e - h * mn;
  int32_t *base = acc + h * n_kseg * mn + o;
  for (int seg = n_kseg - 1; seg >= 1; --seg) base[seg * mn] -= base[(seg - 1) * mn];
}

template <int BM, int BN, int MODE>
hipError_t launch_variant(TileArgs t, int amode, bool debug, hipStream_t s) {
  t.tiles_m = (t.M + BM - 1) / BM;
  t.tiles_n = (t.N + BN - 1) / BN;
  dim3 grid((unsigned)(t.tiles_m * t.tiles_n)), block(256);
#define SQ_LAUNCH(AM, DBG) \
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, AM, MODE, DBG>), grid, block, 0, s, t)
  if (debug) {
    if (amode == A_BF16) SQ_LAUNCH(A_BF16, true);
    else if (amode == A_SIGNED) SQ_LAUNCH(A_SIGNED, true);
    else if (amode == A_PLANES) SQ_LAUNCH(A_PLANES, true);
    else if (amode == A_BF16_1) SQ_LAUNCH(A_BF16_1, true);
    else SQ_LAUNCH(A_SIGNED_1, true);
  } else {
    if (amode == A_BF16) SQ_LAUNCH(A_BF16, false);
    else if (amode == A_SIGNED) SQ_LAUNCH(A_SIGNED, false);
    else if (amode == A_PLANES) SQ_LAUNCH(A_PLANES, false);
    else if (amode == A_BF16_1) SQ_LAUNCH(A_BF16_1, false);
    else SQ_LAUNCH(A_SIGNED_1, false);
  }
#undef SQ_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tile(const GemmProblem &p, hipStream_t s) {
  TileArgs t{};
  t.M = (int32_t)p.M;
  t.N = (int32_t)p.N;
  t.K = (int32_t)p.K;
  t.x = p.x;
  t.ld_x = p.ld_x;
  t.xq = p.xq;
  t.ld_q = p.ld_q;
  t.plane_stride = p.q_layout == 1 ? p.M * p.ld_q : 0;
  t.w = p.w_packed;
  t.w_scale = p.w_scale;
  t.act = p.act;
  t.y = p.y;
  t.ld_y = p.ld_y;
  t.acc = p.acc_debug;
  t.n_kseg = p.ks.n;
  bool every_step = true;
  for (int i = 0; i < p.ks.n; ++i) {
    t.seg_end_tile[i] = p.ks.end[i] / 64;
    every_step = every_step && (p.ks.end[i] - p.ks.off[i] == 64);
  }
  const int amode = p.single_scale ? (p.x ? A_BF16_1 : A_SIGNED_1)
                                   : p.x ? A_BF16 : (p.q_layout == 1 ? A_PLANES : A_SIGNED);
  const bool debug = p.acc_debug != nullptr;
  // (the tile widths here and in tile_columns() go together)
  if (p.ks.n == 1) {
    // Fewer 64 x 384 tiles than half the CUs leave the chip mostly idle and
    // the call latency-bound: 32 x 128 tiles give six times as many
    // workgroups, two per CU.  (M=64, K=256, N=768 on MI355X: 11.6 us with
    // two 64 x 384 tiles, 4.7 us with twelve 32 x 128 tiles.)
    const int64_t big = ((p.M + 63) / 64) * ((p.N + 383) / 384);
    if (big < kSmallTileGrid) return launch_variant<32, 128, SINGLE>(t, amode, debug, s);
    return launch_variant<64, 384, SINGLE>(t, amode, debug, s);
  }
  if (every_step) return launch_variant<32, 256, STEP>(t, amode, debug, s);
  // Several K-segments on int8 codes, or a K beyond what MULTI's running
  // int32 sums hold (K * 128 * 127 < 2^31): the kernel that stages both
  // operands through LDS and folds each segment's own sums.
  if (!p.x || p.K > kRunningSumMaxK) return launch_gemm_lds(p, s);
  bool even_ends = true;  // every segment end but the last on a whole stage
  for (int i = 0; i + 1 < p.ks.n; ++i) even_ends = even_ends && (p.ks.end[i] % 128 == 0);
  hipError_t e = even_ends ? launch_variant<64, 256, MULTI>(t, amode, debug, s)
                           : launch_variant<64, 256, MULTI64>(t, amode, debug, s);
  if (e != hipSuccess || !debug) return e;
  const int64_t mn = p.M * p.N;
  const int planes = p.single_scale ? 1 : 2;
  hipLaunchKernelGGL(acc_difference_kernel, dim3((unsigned)((planes * mn + 255) / 256)), dim3(256),
                     0, s, p.acc_debug, p.ks.n, mn, planes);
  return hipGetLastError();
}

int tile_columns(const SegTable &ks) { return ks.n == 1 ? 384 : 256; }

// With bf16 input the tile kernel quantises each activation tile once per
// column tile, N / BN times over.  Quantising once into int8 codes instead
// (one HBM pass: 2 bytes read and 1 written per element) and running the
// GEMM from the codes costs less from about six column tiles on.  Measured
// on MI355X: M=4429, K=1536, N=1536 in 24 K-segments (six tiles of 256)
// 57 us against 67 us fused; M=9216, K=12288, N=3072 in 4 K-segments
// (twelve tiles) 733 us against 991 us; M=4096, K=6144, N=1536 in one
// segment (four tiles of 384) 84 us either way.
bool tile_quantize_first(int64_t M, int64_t N, const SegTable &ks) {
  const int bn = tile_columns(ks);
  return M > kSmallMMax && (N + bn - 1) / bn >= 6;
}

}  // namespace sq
