// gemm_lds.hip -- the DualScale x SegLinear W8A8 linear layer for large M on
// gfx950, with the weight and the activation codes of each K-stage shared by
// the workgroup's waves through LDS.
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes): "DualScale" (split,
//      scales, reconstruction; both polarity products in one batched launch
//      whose epilogue combines the scaled results) and "SegLinear" (the
//      input-segmented sum over K-segments).
// [P2] "SegQuant" (hliangzhao.me): section 3, the same reconstruction as one
//      batched integer GEMM with a fused epilogue; section 2, the segment sums.
//
// Used for calls with several K-segments whose activation arrives as int8
// codes (the quantise-first path of wide layers, or codes from the caller),
// and for every multi-segment call whose K exceeds the int32 bound of the
// other large-M kernel's running sums: here each segment's products start
// from zero and are folded at the segment's end, so only one segment's
// products ever sit in an int32 accumulator.
//
// Design (CDNA4):
//   * A workgroup of NWV waves (4, or 8 for int8 input) owns a BM x BN
//     output tile; the waves form a WGM x (NWV / WGM) grid, each owning a
//     WM x WN sub-tile of 32 x 32 blocks computed by the int8 32x32x32
//     matrix-core instruction.
//   * K advances in stages of 64 (one packed weight k-tile; K-segment
//     boundaries are multiples of 64, so every stage lies in one segment).
//     NST stage buffers rotate in LDS.  Each holds the stage's weight tiles,
//     copied verbatim from the packed layout by 16-byte global->LDS loads (a
//     packed 1 KiB tile is already in the lane order of the B operand), the
//     weight-scale row of its segment (4-byte copies), and its activation:
//       - int8 codes: copied the same way, 16 rows x 64 codes per load
//         instruction, each row's four 16-byte chunks rotated by (row / 4) % 4
//         so that the operand reads of 16 consecutive rows hit 16 different
//         bank groups;
//       - bf16: loaded into registers three stages ahead, quantised one stage
//         ahead (sign picks the half's inverse scale, one fp32 multiply,
//         clamp, round half to even) and written as the + and - planes in the
//         same rotated layout.
//   * Each 32-k sub-step's operands are read from LDS one sub-step ahead of
//     its products.  One barrier per stage, between its two sub-steps: after
//     it the next stage's first operands are read while this stage's second
//     sub-step hides their latency, and this stage's buffer takes the copies
//     of stage u + NST.  Before it, this wave waits for its own copies into
//     stage u + 1 only; later stages' copies stay in flight.  The waits are
//     explicit: the compiler does not count the global->LDS copies.
//   * Signed-code input: the codes feed one product directly (A_t = Q W) and
//     their + plane, split off in registers, the other (A+ = P W).  The fold
//     uses y += (c+ - c-) A+ + c- A_t, which equals c+ A+ + c- A- because
//     A- = A_t - A+.  Two-plane and bf16 input multiply the planes as they
//     are: y += c+ A+ + c- A-.  Single-scale: one product on the signed code.
//     (c+-_i = s+-_i * w_scale[i][n].)
//   * int8 input: 64 x 64 per wave, two waves per SIMD (256 registers per
//     lane each): 128 x 128 tiles of four waves, two workgroups per CU.
//     Measured on MI355X, the copies' issue costs about a sixth of the time
//     (the kernel runs that much faster with them removed), and the shader
//     clock under it (about 1.8 GHz) is set by the power the matrix cores
//     draw on changing operands, as for a matrix-core-only loop on random
//     data.
//   * Tile order is XCD-aware: workgroups are dealt to the 8 XCDs in turn, so
//     XCD x receives one contiguous range of logical tiles, ordered in
//     groups of 8 row tiles so that the tiles one XCD runs at once share
//     weight and activation slices in its L2.
#include <stddef.h>

#include <type_traits>

#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

// activation input of the kernel
enum LAMode {
  LA_BF16 = 0,      // bf16, quantised here into two planes
  LA_SIGNED = 1,    // signed codes [M][ld_q]
  LA_PLANES = 2,    // planes [2][M][ld_q]
  LA_BF16_1 = 3,    // single scale: bf16, one plane of signed codes
  LA_SIGNED_1 = 4,  // single scale: signed codes
};

template <int V>
using lc = std::integral_constant<int, V>;

typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

struct LdsArgs {
  int32_t M, N, K;
  int32_t tiles_m, tiles_n;
  const uint16_t *x;
  int64_t ld_x;
  const int8_t *xq;
  int64_t ld_q;
  int64_t plane_stride;
  const int8_t *w;
  const float *w_scale;
  const float *act;  // [4][n_kseg]: s+, s-, inv+, inv-
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc;  // [2][n_kseg][M][N] or null
  int32_t n_kseg;
  int32_t seg_end_tile[kMaxKSeg];  // exclusive end of each segment, in k-tiles of 64
};

// Segment end i straight from the kernel-argument segment (indexing the
// by-value argument with a run-time index would copy it to scratch memory).
__device__ __forceinline__ int lds_seg_end(int i) {
  const char *base = (const char *)__builtin_amdgcn_kernarg_segment_ptr();
  return reinterpret_cast<const int32_t *>(base + offsetof(LdsArgs, seg_end_tile))[i];
}

// s_waitcnt: vector-memory count n, LDS count 0 when LGK (else untouched),
// export count untouched (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N, bool LGK>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGK ? 0 : 15) << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

__device__ __forceinline__ v16i mfma(const v4u &a, const v4u &b, const v16i &c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(reinterpret_cast<const v4i &>(a),
                                               reinterpret_cast<const v4i &>(b), c, 0, 0, 0);
}

// + plane of four signed codes: the bytes whose sign bit is set become 0.
// The byte permute's selectors 8-11 replicate the top bit of bytes 1 and 3
// of each source; shifting one source left by 8 brings bytes 0 and 2 there.
__device__ __forceinline__ uint32_t pos_plane(uint32_t q) {
  const uint32_t m = __builtin_amdgcn_perm(q << 8, q, 0x090B080Au);
  return q & ~m;
}

__device__ __forceinline__ void lds_dma16(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)l, 16, 0, 0);
}

template <int BM, int BN, int WGM, int AM, int NST, bool DEBUG, int OCC, int NWV>
__global__ __launch_bounds__(64 * NWV, OCC) void gemm_lds_kernel(LdsArgs a) {
  constexpr int WGN = NWV / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, MB = WM / 32, NB = WN / 32;
  constexpr bool BF16 = AM == LA_BF16 || AM == LA_BF16_1;
  constexpr bool ONE = AM == LA_BF16_1 || AM == LA_SIGNED_1;
  constexpr bool DERIVE = AM == LA_SIGNED;  // + plane split off the codes in registers
  constexpr int NPL = (AM == LA_PLANES || AM == LA_BF16) ? 2 : 1;  // activation planes in LDS
  constexpr int A_PL = BM * 64;   // bytes of one activation plane per stage
  constexpr int W_ST = BN * 64;   // bytes of weight per stage
  constexpr int NWS = (BN + 64 * NWV - 1) / (64 * NWV);  // 4-byte copies per wave per stage of the weight scales
  constexpr int WS_OFF = W_ST + NPL * A_PL;  // the stage's weight-scale row (fp32 per column)
  constexpr int ST = WS_OFF + NWS * NWV * 256;
  constexpr int NW = BN / (16 * NWV);                // weight copies per wave per stage
  constexpr int RB = BM / (16 * NWV);                // 16-row activation blocks per wave and plane
  constexpr int NA = BF16 ? 0 : NPL * RB;            // activation copies per wave per stage
  constexpr int XP = BF16 ? BM / 32 : 0;             // bf16 16-byte loads per thread per stage
  constexpr int ND = NW + NWS + NA;                  // copies per wave per stage
  constexpr int NV = ND + XP;                        // vector-memory instructions per stage
  static_assert(BM % 64 == 0 && BN % 64 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(BN % (16 * NWV) == 0 && BM % (16 * NWV) == 0 && (!BF16 || NWV == 4),
                "each wave copies whole 1 KiB tiles; bf16 input uses four waves");
  static_assert(NST >= 3 && OCC * NST * ST <= 160 * 1024, "stages");
  static_assert((NST - 2) * NV < 64 && (NST - 1) * NV < 64, "wait count");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * ST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // ---- tile of this workgroup (XCD-aware order) ----
  const int T = a.tiles_m * a.tiles_n;
  int logical;
  {
    const int bid = blockIdx.x, per = T / 8, rem = T % 8, xcd = bid % 8, i = bid / 8;
    logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + i;
  }
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
  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;
  const float *i_pos = a.act + 2 * nS, *i_neg = a.act + 3 * nS;

  // ---- per-segment tables, held across lanes ----
  // Lane l of entry j holds segment 64 j + l (clamped), read back with
  // readlane at wave-uniform indices: no scalar-memory load in the stage
  // loop (waiting for one would also wait for every LDS access in flight)
  // and no vector load (waiting for one would wait for every copy in flight).
  int t_end[2];
  float t_sp[2], t_sn[2], t_ip[2], t_in[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sg = min(64 * j + lane, nS - 1);
    t_end[j] = lds_seg_end(sg);
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
  // the tables land before the first copy is issued, so no later wait for
  // them can also wait for copies in flight
  wait_vm<0, false>();
  __builtin_amdgcn_sched_barrier(0);

  // ---- global -> LDS copies of one stage ----
  // (wave-uniform bases with 32-bit lane offsets)
  // weight: n-tile j of the workgroup (j = wave * NW + i), clamped to the
  // last n-tile past N (those columns are never stored)
  const int nt0 = min(n0 / 16, NT - 1);
  const int8_t *wb = a.w + (int64_t)nt0 * KT * 1024;
  uint32_t woff[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int nt = min(n0 / 16 + wave * NW + i, NT - 1);
    woff[i] = (uint32_t)((nt - nt0) * KT * 1024 + lane * 16);
  }
  // weight-scale row: wave w copies floats (i * 4 + w) * 64 + l
  uint32_t wsoff[NWS];
#pragma unroll
  for (int i = 0; i < NWS; ++i) wsoff[i] = (uint32_t)min(n0 + (i * NWV + wave) * 64 + lane, a.N - 1);
  // activation codes: 16-row block b = wave * (BM / 64) + i of each plane;
  // lane l copies row l / 4 of the block, chunk (l % 4) ^ ((l / 16) % 4)
  const int8_t *ab = a.xq + (int64_t)m0 * a.ld_q;
  uint32_t aoff[BF16 ? 1 : RB];
  if (!BF16) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int r = min(m0 + (wave * RB + i) * 16 + (lane >> 2), a.M - 1);
      const int c = (lane & 3) ^ ((lane >> 4) & 3);
      aoff[i] = (uint32_t)((r - m0) * a.ld_q + c * 16);
    }
  }
  int pseg = 0;  // segment of the stage whose copies are issued next (only grows)
  auto copy_stage = [&](int kt, int buf) __attribute__((always_inline)) {
    kt = min(kt, KT - 1);  // past K: a valid stage into a free buffer, never read
    uint8_t *sb = smem + buf * ST;
    const int8_t *wk = wb + kt * 1024;
#pragma unroll
    for (int i = 0; i < NW; ++i) lds_dma16(wk + woff[i], sb + (wave * NW + i) * 1024);
    pseg += (kt >= seg_i(t_end, pseg) && pseg + 1 < nS) ? 1 : 0;
    const float *wsr = a.w_scale + (int64_t)pseg * a.N;
#pragma unroll
    for (int i = 0; i < NWS; ++i)
      __builtin_amdgcn_global_load_lds(wsr + wsoff[i],
                                       (lds_void *)(sb + WS_OFF + (i * NWV + wave) * 256), 4, 0, 0);
    if (!BF16) {
#pragma unroll
      for (int p = 0; p < NPL; ++p) {
        const int8_t *ak = ab + p * a.plane_stride + kt * 64;
#pragma unroll
        for (int i = 0; i < RB; ++i)
          lds_dma16(ak + aoff[i], sb + W_ST + p * A_PL + (wave * RB + i) * 1024);
      }
    }
  };

  // ---- bf16 activation: two register slots, quantisation into LDS ----
  // load i of thread t: row i * 32 + t / 8, elements (t % 8) * 8 .. +8 of
  // the stage (128 bytes a row, 8 threads a row: coalesced)
  v4u xr[2][XP > 0 ? XP : 1];
  const uint16_t *xb = a.x + (int64_t)m0 * a.ld_x;
  uint32_t xoff[XP > 0 ? XP : 1];
  if (BF16) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int r = min(m0 + i * 32 + (tid >> 3), a.M - 1);  // rows past M: any valid row
      xoff[i] = (uint32_t)((r - m0) * a.ld_x + (tid & 7) * 8);
    }
  }
  auto load_x = [&](auto SLOT, int kt) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    kt = min(max(kt, 0), KT - 1);
    const uint16_t *xk = xb + kt * 64;
#pragma unroll
    for (int i = 0; i < XP; ++i) xr[s][i] = *reinterpret_cast<const v4u *>(xk + xoff[i]);
  };
  // load i is half (t % 2) of chunk (t % 8) / 2 of its row
  const int q_chunk = (tid & 7) >> 1, q_half = tid & 1;
  int qseg = 0;  // segment of the stage being quantised (only grows)
  auto quant_stage = [&](auto SLOT, int kt, int buf) __attribute__((always_inline)) {
    constexpr int s = decltype(SLOT)::value;
    qseg += (kt >= seg_i(t_end, qseg) && qseg + 1 < nS) ? 1 : 0;
    const float ip = seg_f(t_ip, qseg), in = ONE ? ip : seg_f(t_in, qseg);
    uint8_t *ap = smem + buf * ST + W_ST;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int r = i * 32 + (tid >> 3);
      const int off = r * 64 + 16 * (q_chunk ^ ((r >> 2) & 3)) + 8 * q_half;
      if (ONE) {
        *reinterpret_cast<v2u *>(ap + off) = quant8_signed(xr[s][i], ip, ip);
      } else {
        v2u p, n;
        quant8_planes(xr[s][i], ip, in, p, n);
        *reinterpret_cast<v2u *>(ap + off) = p;
        *reinterpret_cast<v2u *>(ap + A_PL + off) = n;
      }
    }
  };

  // ---- operand reads of one 32-k sub-step ----
  // A: row rb + (l % 32) of block mb; chunk 2 ks + l / 32, rotated
  const int a_lane = ((lane & 31) >> 4) * 1024 + (lane & 15) * 64;
  const int a_rot = (lane >> 2) & 3;
  const int a_sub0 = 16 * ((0 + (lane >> 5)) ^ a_rot), a_sub1 = 16 * ((2 + (lane >> 5)) ^ a_rot);
  // B: n-tile (wn * WN + 32 nb) / 16 + (l % 32) / 16, column l % 16, k group 2 ks + l / 32
  const int b_lane = ((lane & 31) >> 4) * 1024 + (lane & 15) * 16 + (lane >> 5) * 256;
  // operands of one sub-step; p: the + plane split off signed codes
  struct Frags {
    v4u a[MB][NPL], b[NB], p[DERIVE ? MB : 1];
  };
  auto derive = [&](Frags &f) __attribute__((always_inline)) {
    if (DERIVE) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) f.p[mb][e] = pos_plane(f.a[mb][0][e]);
    }
  };
  auto read_frags = [&](Frags &f, const uint8_t *sb, int ks) __attribute__((always_inline)) {
    const int asub = ks ? a_sub1 : a_sub0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int rb = wm * WM + 32 * mb;
#pragma unroll
      for (int p = 0; p < NPL; ++p)
        f.a[mb][p] = *reinterpret_cast<const v4u *>(sb + W_ST + p * A_PL + (rb / 16) * 1024 +
                                                     a_lane + asub);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      f.b[nb] = *reinterpret_cast<const v4u *>(sb + ((wn * WN + 32 * nb) / 16) * 1024 + b_lane +
                                                ks * 512);
  };

  // ---- accumulators ----
  constexpr int NACC = ONE ? 1 : 2;
  v16i acc[NACC][MB][NB];
#pragma unroll
  for (int h = 0; h < NACC; ++h)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[h][i][j] = v16i{};
  v16f yacc[MB][NB];  // fp32 sums of the folded segments
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) yacc[i][j] = v16f{};

  // products of one 32-k sub-step; ZERO: they start from zero (a segment's
  // first).  The products on the codes as read (signed code, or the - plane)
  // come first, so that they can run while the + plane is split off.
  auto mma = [&](const Frags &f, bool zero) __attribute__((always_inline)) {
    if (!ONE) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const v4u &qb = DERIVE ? f.a[mb][0] : f.a[mb][1];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[1][mb][nb] = mfma(qb, f.b[nb], zero ? v16i{} : acc[1][mb][nb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const v4u &pa = DERIVE ? f.p[mb] : f.a[mb][0];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[0][mb][nb] = mfma(pa, f.b[nb], zero ? v16i{} : acc[0][mb][nb]);
    }
  };

  // 32 x 32 output block: lane l holds column l % 32 and, in register r,
  // row (r / 4) * 8 + (l / 32) * 4 + r % 4
  const int col_lane = n0 + wn * WN + (lane & 31);
  const int row_lane = m0 + wm * WM + (lane >> 5) * 4;
  auto out_row = [&](int mb, int r) __attribute__((always_inline)) {
    return row_lane + mb * 32 + (r >> 2) * 8 + (r & 3);
  };
  // per-segment sums of this lane's outputs into acc_debug: A+ and A- (or
  // the one single-scale product in plane 0)
  auto dump = [&](int seg) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = col_lane + 32 * nb;
      if (col >= a.N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = out_row(mb, r);
          if (m >= a.M) continue;
          const int64_t o = ((int64_t)seg * a.M + m) * a.N + col;
          a.acc[o] = acc[0][mb][nb][r];
          if (!ONE)
            a.acc[(int64_t)nS * a.M * a.N + o] =
                DERIVE ? acc[1][mb][nb][r] - acc[0][mb][nb][r] : acc[1][mb][nb][r];
        }
    }
  };
  // fold the int32 sums of segment seg into the fp32 sums, with the
  // segment's weight scales ws[nb] for this lane's columns
  auto fold = [&](int seg, const float (&ws)[NB]) __attribute__((always_inline)) {
    if (DEBUG) dump(seg);
    // (scalar loads: the lane tables' registers would make the compiler wait
    // for every copy in flight at the segment loop's head)
    const float sp = s_pos[seg], sn = s_neg[seg];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float cp = sp * ws[nb], cn = sn * ws[nb];
      const float k0 = DERIVE ? cp - cn : cp;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        v16f &yv = yacc[mb][nb];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float t = __builtin_fmaf(k0, (float)acc[0][mb][nb][r], yv[r]);
          yv[r] = ONE ? t : __builtin_fmaf(cn, (float)acc[1][mb][nb][r], t);
        }
        // one block at a time: its accumulators leave the matrix registers
        // only for their own conversions
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- the pipeline ----
  // Stage u (64 k) is read from buffer u % NST.  Its copies were issued
  // NST stages earlier, right after the barrier that freed that buffer.
  // Each 32-k sub-step's operands are read from LDS one sub-step ahead of
  // their products.  Within stage u: the sub-step-1 operands are read;
  // sub-step 0's products run (operands read during stage u - 1), with
  // (bf16) the quantisation of stage u + 1 between them; this wave waits
  // for its copies into stage u + 1 and for its reads of buffer u, and the
  // barrier makes every wave's copies and quantised codes of stage u + 1
  // visible and proves buffer u no longer read; the copies of stage u + NST
  // go into buffer u, stage u + 1's sub-step-0 operands are read, and
  // sub-step 1's products hide those reads.  Per stage and wave, in order:
  // (bf16) the loads of stage u + 3 into the slot stage u + 1 used, then the
  // stage's copies.
  constexpr int NBLK = MB * NB;
  auto issue = [&](auto XSLOT, int s, int buf) __attribute__((always_inline)) {
    if (BF16) load_x(XSLOT, s - NST + 3);
    copy_stage(s, buf);
  };
  // Prologue: the steady state's pattern for virtual stages -NST .. -1.
  // Virtual stage v issues the loads of stage v + 3 (a stage below 0 loads
  // stage 0 into a slot that is loaded again before use) and the copies of
  // stage v + NST; stage -1 quantises stage 0 before its barrier.
  static_assert(!BF16 || NST == 4, "bf16 input: loads lead by NST - 1 = 3 stages (two slots)");
#pragma unroll
  for (int v = -NST; v <= -2; ++v) {
    if (((v + 3) & 1) == 0) issue(lc<0>{}, v + NST, v + NST);
    else issue(lc<1>{}, v + NST, v + NST);
  }
  if (BF16) quant_stage(lc<0>{}, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (DEBUG) wait_vm<0, true>();
  else wait_vm<(NST - 2) * NV, true>();  // stage 0's copies (issued at v = -NST)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  issue(lc<0>{}, NST - 1, NST - 1);  // v = -1: loads of stage 2 into slot 0
  __builtin_amdgcn_sched_barrier(0);
  Frags f0, f1;
  read_frags(f0, smem, 0);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);

  float wsf[NB];  // the weight scales of the segment being folded
  int buf = 0;
  // Interleave the region's matrix-core instructions with its vector ALU
  // work: NM of them, VPM vector instructions after each (the rest after).
  auto interleave = [&](auto NMC, auto VPMC) __attribute__((always_inline)) {
    constexpr int NMI = decltype(NMC)::value, VPM = decltype(VPMC)::value;
#pragma unroll
    for (int j = 0; j < NMI; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
    }
  };
  constexpr int NM_SUB = NACC * NBLK;                        // products of one sub-step
  constexpr int V_DER = DERIVE ? MB * 4 * 3 : 0;              // + plane split of one sub-step
  constexpr int V_Q = BF16 ? XP * (ONE ? 44 : 52) : 0;        // quantisation of one stage
  auto stage = [&](auto XSLOT, int u, bool first, bool last_of_seg) __attribute__((always_inline)) {
    constexpr int xs = decltype(XSLOT)::value;  // bf16: the slot of stage u + 1 ((u + 1) % 2)
    const uint8_t *sb = smem + buf * ST;
    const int nbuf = buf == NST - 1 ? 0 : buf + 1;
    // (1) sub-step 1's operands: their latency hides behind sub-step 0
    read_frags(f1, sb, 1);
    __builtin_amdgcn_sched_barrier(0);
    // (2) sub-step 0: the + plane split off (before the products in program
    //     order, which read it; the products on the codes as read can run
    //     meanwhile) and (bf16) the quantisation of stage u + 1, spread
    //     between the products
    derive(f0);
    if (first) {
      mma(f0, true);
    } else {
      mma(f0, false);
    }
    if (BF16) quant_stage(lc<xs>{}, u + 1, nbuf);
    interleave(lc<NM_SUB>{}, lc<(V_Q + V_DER + NM_SUB - 1) / NM_SUB>{});
    __builtin_amdgcn_sched_barrier(0);
    if (last_of_seg) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        wsf[nb] = *reinterpret_cast<const float *>(sb + WS_OFF + 4 * (wn * WN + 32 * nb + (lane & 31)));
    }
    __builtin_amdgcn_sched_barrier(0);
    // (3) this wave's copies into stage u + 1 have landed and its reads of
    //     buffer u are done; after the barrier every wave's are, and every
    //     wave's quantised codes of stage u + 1 are written
    if (DEBUG) {
      wait_vm<0, true>();  // (the accumulator dump's stores also count)
    } else {
      // stage u + 1's copies came NST - 2 stages' issues before the latest
      wait_vm<(NST - 2) * NV, true>();
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // (4) the copies of stage u + NST into buffer u (bf16: the loads of
    //     stage u + 3 into the slot just quantised), and stage u + 1's
    //     sub-step-0 operands
    issue(lc<xs>{}, u + NST, buf);
    read_frags(f0, smem + nbuf * ST, 0);
    __builtin_amdgcn_sched_barrier(0);
    // (5) sub-step 1, as sub-step 0, hiding those reads; the stage ends with
    //     every LDS read complete, so the next stage's products wait for
    //     nothing
    derive(f1);
    mma(f1, false);
    interleave(lc<NM_SUB>{}, lc<(V_DER + NM_SUB - 1) / NM_SUB>{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    buf = nbuf;
  };
  auto run_stage = [&](int u, bool first, bool last_of_seg) __attribute__((always_inline)) {
    if (BF16 && (u & 1) == 0) stage(lc<1>{}, u, first, last_of_seg);
    else stage(lc<0>{}, u, first, last_of_seg);
  };
  // Segment by segment: its stages (the first starts its products from
  // zero), then the fold of its sums.
  int u = 0;
  for (int sg = 0; sg < nS; ++sg) {
    const int end = lds_seg_end(sg);
    for (bool first = true; u < end; ++u, first = false) run_stage(u, first, u + 1 >= end);
    fold(sg, wsf);
  }
  // the copies past K must land before the workgroup's LDS is released
  wait_vm<0, true>();

  // ---- epilogue: bf16 store ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = col_lane + 32 * nb;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const v16f v = yacc[mb][nb];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = out_row(mb, r);
        if (m < a.M && col < a.N) a.y[(int64_t)m * a.ld_y + col] = (uint16_t)f32_to_bf16_rne(v[r]);
      }
    }
  }
}

// Bytes of one stage buffer, and the stage count for a tile and input mode:
// four when they fit in 160 KiB of LDS (bf16 input needs four), else three;
// 0 when the configuration does not fit.
constexpr int lds_stage_bytes(int BM, int BN, int AM, int NWV) {
  return BN * 64 + ((AM == LA_PLANES || AM == LA_BF16) ? 2 : 1) * BM * 64 +
         ((BN + 64 * NWV - 1) / (64 * NWV)) * NWV * 256;
}
// (occ workgroups per CU share its 160 KiB)
constexpr int lds_stages(int BM, int BN, int AM, int occ, int NWV) {
  // bf16 input: exactly four (the register slots' parity); int8 input: as
  // many as fit, up to seven (copies in flight NST - 1 stages ahead)
  return (AM == LA_BF16 || AM == LA_BF16_1)
             ? (4 * lds_stage_bytes(BM, BN, AM, NWV) <= 160 * 1024 / occ ? 4 : 0)
             : ((160 * 1024 / occ) / lds_stage_bytes(BM, BN, AM, NWV) >= 7
                    ? 7
                    : ((160 * 1024 / occ) / lds_stage_bytes(BM, BN, AM, NWV) >= 3
                           ? (160 * 1024 / occ) / lds_stage_bytes(BM, BN, AM, NWV)
                           : 0));
}

// One configuration per activation input:
//   int8 codes  128 x 128 tiles of four waves (64 x 64 each), two
//               workgroups per CU.  (128 x 256 tiles of eight waves, one
//               workgroup per CU, copy a quarter fewer bytes per product;
//               measured on four MI355X boxes they were 2.5-4 % faster on
//               two and 7-13 % slower on the other two.)
//   bf16        128 x 192 tiles, one workgroup per CU (the quantisation
//               needs the registers)
template <int BM, int BN, int WGM, int AM, int OCC, int NWV>
hipError_t launch_lds_mode(LdsArgs t, bool debug, hipStream_t s) {
  constexpr int NST = lds_stages(BM, BN, AM, OCC, NWV);
  static_assert(NST > 0, "configuration does not fit in LDS");
  t.tiles_m = (t.M + BM - 1) / BM;
  t.tiles_n = (t.N + BN - 1) / BN;
  dim3 grid((unsigned)(t.tiles_m * t.tiles_n)), block(64 * NWV);
  if (debug)
    hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, WGM, AM, NST, true, OCC, NWV>), grid, block, 0,
                       s, t);
  else
    hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, WGM, AM, NST, false, OCC, NWV>), grid, block,
                       0, s, t);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_lds(const GemmProblem &p, hipStream_t s) {
  LdsArgs t{};
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
  for (int i = 0; i < p.ks.n; ++i) t.seg_end_tile[i] = (p.ks.end[i] + 63) / 64;
  const bool debug = p.acc_debug != nullptr;
  if (p.x)
    return p.single_scale ? launch_lds_mode<128, 192, 2, LA_BF16_1, 1, 4>(t, debug, s)
                          : launch_lds_mode<128, 192, 2, LA_BF16, 1, 4>(t, debug, s);
  if (p.single_scale) return launch_lds_mode<128, 128, 2, LA_SIGNED_1, 2, 4>(t, debug, s);
  return p.q_layout == 1 ? launch_lds_mode<128, 128, 2, LA_PLANES, 2, 4>(t, debug, s)
                         : launch_lds_mode<128, 128, 2, LA_SIGNED, 2, 4>(t, debug, s);
}

}  // namespace sq
