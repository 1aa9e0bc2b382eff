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
//   * A workgroup of 4 waves (one per SIMD) owns a BM x BN output tile and
//     walks K in 64-wide steps, one int8 16x16x64 matrix-core step; K-segment
//     boundaries are multiples of 64, so a step never straddles two.
//   * Wave w owns output columns [w*BN/4, (w+1)*BN/4) for all BM rows.  The
//     packed weight is laid out as lane-ordered 1 KiB tiles, so each wave
//     loads its B operands straight from memory into registers (one 16-byte
//     load per lane per 16 columns) through a 4-step register ring: the
//     weight never touches LDS.  Both polarity halves multiply the same B
//     registers.
//   * The activation tile (BM x 64) is shared by the 4 waves through LDS:
//     every thread loads 16-byte pieces of bf16 X two steps ahead, quantises
//     them one step ahead (the sign selects the half's inverse scale, one fp32
//     multiply, clamp, round half to even) and writes the codes as two int8
//     planes (X+, X-) into the other LDS stage, rows padded to 80 bytes so
//     the operand reads are free of bank conflicts.  Pre-quantised int8
//     input skips the arithmetic.  One barrier per step.
//   * The quantisation VALU work of step t+1 is interleaved with the matrix
//     core instructions of step t (sched_group_barrier), so both units run
//     at once.
//   * Folding K-segments (the epilogue of the pages' reconstruction):
//       SINGLE  one K-segment: int32 accumulators over all of K, scaled once
//               at the end: y = s_w*s+*A+ + s_w*s-*A-.
//       STEP    every K-segment is one step (e.g. one attention head per
//               segment): each step's products start from zero and are
//               folded into an fp32 sum right away.
//       MULTI   general segments: int32 accumulators per segment, folded
//               into the fp32 sum at each segment end.
//     The per-column weight scales are fetched ahead of their use.
//   * Workgroup -> tile order is XCD-aware: workgroups are dealt to the 8
//     XCDs round-robin, so XCD x is given one contiguous range of row-major
//     tiles; a block of X rows is then quantised and cached inside one L2.
#include <type_traits>

#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kAPitch = 80;  // bytes per LDS row of one A plane (64 + 16 pad)

enum AMode { A_BF16 = 0, A_SIGNED = 1, A_PLANES = 2 };
enum Mode { SINGLE = 0, STEP = 1, MULTI = 2 };

template <int V>
using ic = std::integral_constant<int, V>;

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
  int32_t seg_end_tile[kMaxKSeg];  // exclusive end of each segment, in 64-steps
};

__device__ __forceinline__ v4u lds_read16(const uint8_t *p) {
  return *reinterpret_cast<const v4u *>(p);
}

__device__ __forceinline__ v4i mfma(const v4u &a, const v4u &b, const v4i &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(a),
                                               reinterpret_cast<const v4i &>(b), c, 0, 0, 0);
}

template <int BM, int BN, int AMODE, int MODE, bool DEBUG>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(TileArgs a) {
  constexpr int WN = BN / 4, FM = BM / 16, FN = WN / 16;
  constexpr int A_PLANE = BM * kAPitch, A_STAGE = 2 * A_PLANE;
  // 16-byte activation pieces per thread per step
  constexpr int XP = AMODE == A_SIGNED ? BM / 64 : BM / 32;
  constexpr int WR = 4;  // weight register ring depth (steps)
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");

  // MULTI keeps its fp32 running sum in LDS: four floats per lane and
  // fragment, [wave][i][j][lane][r] (16-byte accesses, conflict free)
  constexpr int Y_LDS = MODE == MULTI ? 4 * FM * FN * 4 * 64 * 4 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * A_STAGE + Y_LDS];
  v4f *ylds4 = reinterpret_cast<v4f *>(smem + 2 * A_STAGE);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // ---- tile of this workgroup (XCD-aware order) ----
  const int T = a.tiles_m * a.tiles_n;
  int logical;
  {
    const int bid = blockIdx.x, per = T / 8, rem = T % 8, x = bid % 8, i = bid / 8;
    logical = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  }
  const int tm = logical / a.tiles_n, tn = logical - tm * a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = a.K / 64, NT = a.N / 16;
  const int nt0 = n0 / 16 + wave * FN;  // first 16-column tile of this wave

  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;
  const float *i_pos = a.act + 2 * nS, *i_neg = a.act + 3 * nS;

  // ---- weight stream: B operands straight into registers ----
  const int8_t *wbase = a.w + (int64_t)nt0 * KT * 1024 + lane * 16;
  v4u wr[WR][FN];
  // Loads are branch-free (indices clamped into range; the extra values are
  // never used), so the count of loads in flight is the same on every pass
  // and the compiler's waits stay exact: prefetching keeps working.
  auto load_w = [&](auto SLOT, int kt) {
    constexpr int s = decltype(SLOT)::value;
    kt = min(kt, KT - 1);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      // n-tiles past N load the last valid tile: their columns are never stored
      const int jj = min(j, NT - 1 - nt0);
      wr[s][j] = *reinterpret_cast<const v4u *>(wbase + ((int64_t)jj * KT + kt) * 1024);
    }
  };

  // ---- activation stream: 16-byte pieces, two steps ahead ----
  v4u xr[2][XP];
  auto load_x = [&](auto SLOT, int kt) {
    constexpr int s = decltype(SLOT)::value;
    kt = min(kt, KT - 1);
    {
#pragma unroll
      for (int i = 0; i < XP; ++i) {
        const uint8_t *p;
        if (AMODE == A_BF16) {
          const int m = min(m0 + i * 32 + (tid >> 3), a.M - 1);  // rows past M: any valid row
          p = reinterpret_cast<const uint8_t *>(a.x) + (int64_t)m * a.ld_x * 2 +
              (int64_t)kt * 128 + (tid & 7) * 16;
        } else if (AMODE == A_SIGNED) {
          const int m = min(m0 + i * 64 + (tid >> 2), a.M - 1);
          p = reinterpret_cast<const uint8_t *>(a.xq) + (int64_t)m * a.ld_q + (int64_t)kt * 64 +
              (tid & 3) * 16;
        } else {
          const int half = i / (BM / 64), ii = i % (BM / 64);
          const int m = min(m0 + ii * 64 + (tid >> 2), a.M - 1);
          p = reinterpret_cast<const uint8_t *>(a.xq) + half * a.plane_stride +
              (int64_t)m * a.ld_q + (int64_t)kt * 64 + (tid & 3) * 16;
        }
        xr[s][i] = *reinterpret_cast<const v4u *>(p);
      }
    }
  };

  // quantise the staged pieces of slot SLOT into LDS stage `stage`
  auto quant_store = [&](auto SLOT, int stage, float inv_pos, float inv_neg, bool valid) {
    constexpr int s = decltype(SLOT)::value;
    uint8_t *ap = smem + stage * A_STAGE;
    uint8_t *an = ap + A_PLANE;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      // a padding step past K stores zero codes (x = 0 quantises to 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) xr[s][i][e] = valid ? xr[s][i][e] : 0u;
      if (AMODE == A_BF16) {
        const int off = (i * 32 + (tid >> 3)) * kAPitch + (tid & 7) * 8;
        v2u p, n;
        quant8_planes(xr[s][i], inv_pos, inv_neg, p, n);
        *reinterpret_cast<v2u *>(ap + off) = p;
        *reinterpret_cast<v2u *>(an + off) = n;
      } else if (AMODE == A_SIGNED) {
        const int off = (i * 64 + (tid >> 2)) * kAPitch + (tid & 3) * 16;
        v4u p, n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t pp, nn;
          split_signed(xr[s][i][j], pp, nn);
          p[j] = pp;
          n[j] = nn;
        }
        *reinterpret_cast<v4u *>(ap + off) = p;
        *reinterpret_cast<v4u *>(an + off) = n;
      } else {
        const int half = i / (BM / 64), ii = i % (BM / 64);
        const int off = (ii * 64 + (tid >> 2)) * kAPitch + (tid & 3) * 16;
        *reinterpret_cast<v4u *>((half ? an : ap) + off) = xr[s][i];
      }
    }
  };

  // ---- accumulators ----
  constexpr bool KEEP_F32 = MODE == STEP;  // fp32 sum in registers
  constexpr int IM = MODE == STEP ? 1 : FM, IN = MODE == STEP ? 1 : FN;
  constexpr int YM = KEEP_F32 ? FM : 1, YN = KEEP_F32 ? FN : 1;
  v4i accp[IM][IN], accn[IM][IN];
  float yacc[YM][YN][4];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j) {
      accp[i][j] = v4i{0, 0, 0, 0};
      accn[i][j] = v4i{0, 0, 0, 0};
    }
#pragma unroll
  for (int i = 0; i < YM; ++i)
#pragma unroll
    for (int j = 0; j < YN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[i][j][r] = 0.0f;

  if (MODE == MULTI) {
    for (int e = tid; e < Y_LDS / 16; e += 256) ylds4[e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  auto yidx4 = [&](int i, int j) { return ((wave * FM + i) * FN + j) * 64 + lane; };

  const int col_lane = n0 + wave * WN + (lane & 15);  // column of fragment j: + 16*j
  const int row_lane = m0 + (lane >> 4) * 4;          // row of fragment i, reg r: + 16*i + r

  // per-column weight scales of a segment (fetched ahead of use)
  constexpr int WSR = MODE == STEP ? WR : 1;
  float wsr[WSR][FN];
  auto load_ws = [&](auto SLOT, int seg) {
    constexpr int s = decltype(SLOT)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = min(col_lane + 16 * j, a.N - 1);  // past N: never stored
      wsr[s][j] = a.w_scale[(int64_t)min(seg, nS - 1) * a.N + col];
    }
  };

  auto dump = [&](int seg, int i, int j, const v4i &p, const v4i &n) {
    const int col = col_lane + 16 * j;
    if (col >= a.N) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = row_lane + 16 * i + r;
      if (m >= a.M) continue;
      const int64_t o = ((int64_t)seg * a.M + m) * a.N + col;
      a.acc[o] = p[r];
      a.acc[(int64_t)nS * a.M * a.N + o] = n[r];
    }
  };

  // fold the int32 accumulators of segment `seg` into the fp32 sum
  auto fold_multi = [&](int seg) {
    const float sp = s_pos[seg], sn = s_neg[seg];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (DEBUG) dump(seg, i, j, accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j],
                        accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j]);
        const float cp = sp * wsr[0][j], cn = sn * wsr[0][j];
        const v4f P = __builtin_convertvector(accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j], v4f);
        const v4f Q = __builtin_convertvector(accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j], v4f);
        v4f &yv = ylds4[yidx4(i, j)];
        yv = __builtin_elementwise_fma(v4f{cn, cn, cn, cn}, Q,
                                       __builtin_elementwise_fma(v4f{cp, cp, cp, cp}, P, yv));
        accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j] = v4i{0, 0, 0, 0};
        accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j] = v4i{0, 0, 0, 0};
      }
  };

  // ---- prologue ----
  load_w(ic<0>{}, 0);
  load_w(ic<1>{}, 1);
  load_w(ic<2>{}, 2);
  load_x(ic<0>{}, 0);
  load_x(ic<1>{}, 1);
  load_ws(ic<0>{}, 0);
  if (MODE == STEP) {
    load_ws(ic<1 % WSR>{}, 1);
    load_ws(ic<2 % WSR>{}, 2);
  }
  const float ip0 = i_pos[0], in0 = i_neg[0];
  quant_store(ic<0>{}, 0, ip0, in0, true);
  __syncthreads();

  int qseg = 0;  // segment of the step being quantised (t + 1)
  int seg = 0;   // segment of the step being multiplied (t)

  // one K-step; s = t mod 4 (t0 is a multiple of 4)
  // one K-step t = t0 + s of the loop over K rounded up to a multiple of 4;
  // steps t >= KT multiply zero codes (padding)
  auto step = [&](auto S, int t0) {
    constexpr int s = decltype(S)::value;
    const int t = t0 + s;
    // segment of step t+1 and its inverse scales, first (branch-free, so the
    // whole step stays one basic block the scheduler can interleave)
    if (MODE != SINGLE) qseg += (t + 1 < KT && t + 1 >= a.seg_end_tile[qseg]) ? 1 : 0;
    const float q_ip = MODE == SINGLE ? ip0 : i_pos[qseg];
    const float q_in = MODE == SINGLE ? in0 : i_neg[qseg];
    // issue the loads of later steps first
    load_w(ic<(s + 3) % 4>{}, t + 3);
    load_x(ic<s % 2>{}, t + 2);
    if (MODE == STEP) load_ws(ic<(s + 3) % WSR>{}, t + 3);
    const uint8_t *ap = smem + (s % 2) * A_STAGE;
    const uint8_t *an = ap + A_PLANE;
    const int aoff = (lane & 15) * kAPitch + (lane >> 4) * 16;
    v4u fa_p[FM], fa_n[FM];
    if (MODE != STEP) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        fa_p[i] = lds_read16(ap + aoff + i * 16 * kAPitch);
        fa_n[i] = lds_read16(an + aoff + i * 16 * kAPitch);
      }
    }
    if (MODE == STEP) {
      const float sp = s_pos[min(t, nS - 1)], sn = s_neg[min(t, nS - 1)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v4i zero = {0, 0, 0, 0};
          if (j == 0) {
            fa_p[i] = lds_read16(ap + aoff + i * 16 * kAPitch);
            fa_n[i] = lds_read16(an + aoff + i * 16 * kAPitch);
          }
          const v4i P = mfma(fa_p[i], wr[s][j], zero);
          const v4i Q = mfma(fa_n[i], wr[s][j], zero);
          if (DEBUG && t < KT) dump(t, i, j, P, Q);
          const float cp = sp * wsr[s % WSR][j], cn = sn * wsr[s % WSR][j];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float &yv = yacc[KEEP_F32 ? i : 0][KEEP_F32 ? j : 0][r];
            yv = __builtin_fmaf(cn, (float)Q[r], __builtin_fmaf(cp, (float)P[r], yv));
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          v4i &P = accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j];
          v4i &Q = accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j];
          P = mfma(fa_p[i], wr[s][j], P);
          Q = mfma(fa_n[i], wr[s][j], Q);
        }
    }
    // quantise step t+1 (past the end: harmless, the stage is never read)
    quant_store(ic<(s + 1) % 2>{}, (s + 1) % 2, q_ip, q_in, t + 1 < KT);
    // Interleave: loads, operand reads, then matrix-core instructions
    // alternating with the VALU work (quantisation of the next step, STEP
    // folds), LDS writes last.
    constexpr int NMFMA = 2 * FM * FN;
    constexpr int NQ = AMODE == A_BF16 ? 64 * XP : 12 * XP;  // quantisation VALU
    __builtin_amdgcn_sched_group_barrier(0x020, FN + XP + (MODE == STEP ? FN : 0), 0);
    if (MODE == STEP) {
      // per row block: its two operand reads, then pairs of matrix-core ops
      // each followed by the fold of the pair before and a share of the
      // quantisation work
      constexpr int PER = 16 + (NQ + FM * FN - 1) / (FM * FN);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
        }
      }
    } else {
      constexpr int PER = (NQ + NMFMA - 1) / NMFMA;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM, 0);
#pragma unroll
      for (int g = 0; g < NMFMA; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2 * XP, 0);
    if (MODE == MULTI && seg < nS && t + 1 == a.seg_end_tile[seg]) {
      fold_multi(seg);
      ++seg;
      load_ws(ic<0>{}, seg);  // the next segment's scales, needed at its end
    }
    __syncthreads();
  };

  // main loop: groups of 4 steps, straight-line (K rounded up to a multiple
  // of 4 steps; padding steps multiply zero codes)
  const int KTV = (KT + 3) & ~3;
  for (int t0 = 0; t0 < KTV; t0 += 4) {
    step(ic<0>{}, t0);
    step(ic<1>{}, t0);
    step(ic<2>{}, t0);
    step(ic<3>{}, t0);
  }

  // ---- epilogue: bf16 store ----
  float cp[FN], cn[FN];
  if (MODE == SINGLE) {
    const float sp = s_pos[0], sn = s_neg[0];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      cp[j] = sp * wsr[0][j];
      cn[j] = sn * wsr[0][j];
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (MODE == SINGLE && DEBUG)
        dump(0, i, j, accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j],
             accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j]);
      const int col = col_lane + 16 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row_lane + 16 * i + r;
        float v;
        if (MODE == SINGLE)
          v = __builtin_fmaf(cn[j], (float)accn[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j][r],
                             cp[j] * (float)accp[MODE == STEP ? 0 : i][MODE == STEP ? 0 : j][r]);
        else if (MODE == STEP)
          v = yacc[KEEP_F32 ? i : 0][KEEP_F32 ? j : 0][r];
        else
          v = ylds4[yidx4(i, j)][r];
        if (m < a.M && col < a.N) a.y[(int64_t)m * a.ld_y + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
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
    else SQ_LAUNCH(A_PLANES, true);
  } else {
    if (amode == A_BF16) SQ_LAUNCH(A_BF16, false);
    else if (amode == A_SIGNED) SQ_LAUNCH(A_SIGNED, false);
    else SQ_LAUNCH(A_PLANES, false);
  }
#undef SQ_LAUNCH
  return hipGetLastError();
}

// Estimated time of a tile shape: waves of 256 workgroups (one per CU) times
// the time of one K-step of one tile, taken as the larger of the matrix-core
// time (BM*BN/32 cycles) and, with bf16 input, the quantisation VALU time
// (BM*64/256 elements per thread, about 7.5 instructions of 4 cycles each).
double tile_cost(int64_t M, int64_t N, int BM, int BN, bool bf16) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t waves = (tiles + 255) / 256;
  const double mfma = (double)BM * BN / 32.0;
  const double valu = bf16 ? (double)BM * 64 / 256.0 * 7.5 * 4.0 : 0.0;
  return (double)waves * (mfma > valu ? mfma : valu);
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
  const int amode = p.x ? A_BF16 : (p.q_layout == 1 ? A_PLANES : A_SIGNED);
  const bool debug = p.acc_debug != nullptr;
  const bool bf16 = amode == A_BF16;
  if (p.ks.n == 1) {
    if (tile_cost(p.M, p.N, 64, 384, bf16) <= tile_cost(p.M, p.N, 128, 256, bf16))
      return launch_variant<64, 384, SINGLE>(t, amode, debug, s);
    return launch_variant<128, 256, SINGLE>(t, amode, debug, s);
  }
  if (every_step) return launch_variant<64, 256, STEP>(t, amode, debug, s);
  return launch_variant<64, 384, MULTI>(t, amode, debug, s);
}

}  // namespace sq
