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
// Design (CDNA4, not a port of the pages' CUTLASS kernel):
//   * One workgroup = 4 waves (256 threads) owns a BM x BN output tile and
//     walks K in steps of 64, one int8 16x16x64 matrix-core step.  K-segment
//     boundaries are multiples of 64, so every step lies in one segment.
//   * Prologue per step: the bf16 X tile (BM x 64) is loaded coalesced (8
//     lanes per 128-byte row piece), quantised in registers with the step's
//     segment scales and written to LDS as two int8 planes (X+ codes, X-
//     codes), each row padded to 80 bytes so the matrix-core operand reads
//     are free of bank conflicts.  A pre-quantised int8 input skips the
//     arithmetic and only splits or copies.
//   * The W tile (64 x BN) is read once from the packed weight (1 KiB
//     lane-ordered tiles, one 16-byte load per lane) into LDS and feeds both
//     halves: each wave runs mfma(X+, W) and mfma(X-, W) on the same B
//     operand registers.
//   * Two LDS stages: step t+1 is loaded and quantised while step t's
//     matrix-core work runs; one barrier per step.
//   * At the end of each K-segment the int32 accumulators are folded into
//     fp32: y += (s+_i w_scale[i][n]) A+ + (s-_i w_scale[i][n]) A-, then
//     cleared (only when K has more than one segment; a single segment folds
//     straight into the bf16 store).  Optionally the int32 accumulators are
//     also stored (acc_debug) for exact checking.
//   * Workgroup -> tile order is XCD-aware: the 8 XCDs each take one
//     contiguous range of tiles (row-block major), so a row block of X is
//     quantised and cached inside one XCD's L2.
#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kAPitch = 80;  // bytes per LDS row of one A plane (64 + 16 pad)

enum AMode { A_BF16 = 0, A_SIGNED = 1, A_PLANES = 2 };

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

// Accumulation modes (how K-segments are folded):
//   SINGLE  one K-segment: int32 accumulators over all of K, scaled once in
//           the epilogue.
//   STEP    every K-segment is one 64-wide step (e.g. one attention head
//           per segment): each step's matrix-core result starts from zero and
//           is folded into the fp32 sum right away.
//   MULTI   general segments: int32 accumulators per segment, folded into an
//           fp32 sum at each segment end (three accumulator sets, so this
//           mode uses a smaller wave tile).
enum Mode { SINGLE = 0, STEP = 1, MULTI = 2 };

template <int BM, int BN, int WM, int WN, int AMODE, int MODE, bool DEBUG, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_tile_kernel(TileArgs a) {
  static_assert((BM / WM) * (BN / WN) == 4, "4 waves per workgroup");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int NWN = BN / WN;
  constexpr int A_BYTES = BM * kAPitch;  // one plane
  constexpr int B_BYTES = BN * 64;       // BN/16 tiles of 1 KiB
  constexpr int STAGE = 2 * A_BYTES + B_BYTES;
  // global -> register staging per thread (16-byte pieces)
  constexpr int XCH = (AMODE == A_BF16) ? BM / 32 : (AMODE == A_SIGNED ? BM / 64 : BM / 32);
  constexpr int WCH = BN / 64;
  constexpr bool KEEP_F32 = MODE != SINGLE;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile sizes");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;

  // XCD-aware tile order: workgroups are dealt to the 8 XCDs round-robin;
  // give XCD x the logical tiles [x*T/8, (x+1)*T/8), row-block major.
  const int T = a.tiles_m * a.tiles_n;
  const int bid = blockIdx.x;
  int logical;
  {
    const int per = T / 8, rem = T % 8, x = bid % 8, i = bid / 8;
    logical = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  }
  const int tm = logical / a.tiles_n, tn = logical % a.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int KT = a.K / 64, NT = a.N / 16;

  v4u xr[XCH];
  v4u wr[WCH];

  auto load_x = [&](int kt) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      int row, coff;
      const uint8_t *base;
      int64_t ld_bytes;
      if (AMODE == A_BF16) {
        row = i * 32 + (tid >> 3);
        coff = (tid & 7) * 16;
        base = reinterpret_cast<const uint8_t *>(a.x) + (int64_t)kt * 128;
        ld_bytes = a.ld_x * 2;
      } else if (AMODE == A_SIGNED) {
        row = i * 64 + (tid >> 2);
        coff = (tid & 3) * 16;
        base = reinterpret_cast<const uint8_t *>(a.xq) + (int64_t)kt * 64;
        ld_bytes = a.ld_q;
      } else {
        const int half = i / (BM / 64), ii = i % (BM / 64);
        row = ii * 64 + (tid >> 2);
        coff = (tid & 3) * 16;
        base = reinterpret_cast<const uint8_t *>(a.xq) + (int64_t)kt * 64 + half * a.plane_stride;
        ld_bytes = a.ld_q;
      }
      const int m = m0 + row;
      if (m < a.M)
        xr[i] = *reinterpret_cast<const v4u *>(base + (int64_t)m * ld_bytes + coff);
      else
        xr[i] = v4u{0u, 0u, 0u, 0u};
    }
  };

  auto load_w = [&](int kt) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int nt = n0 / 16 + i * 4 + wave;  // tile slot i*4+wave of the BN window
      if (nt < NT)
        wr[i] = *reinterpret_cast<const v4u *>(a.w + ((int64_t)nt * KT + kt) * 1024 + lane * 16);
      else
        wr[i] = v4u{0u, 0u, 0u, 0u};
    }
  };

  auto store_stage = [&](int stage, float inv_pos, float inv_neg) {
    uint8_t *ap = smem + stage * STAGE;
    uint8_t *an = ap + A_BYTES;
    uint8_t *bw = an + A_BYTES;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      if (AMODE == A_BF16) {
        const int row = i * 32 + (tid >> 3);
        const int off = row * kAPitch + (tid & 7) * 8;
        v2u p, n;
        quant8_planes(xr[i], inv_pos, inv_neg, p, n);
        *reinterpret_cast<v2u *>(ap + off) = p;
        *reinterpret_cast<v2u *>(an + off) = n;
      } else if (AMODE == A_SIGNED) {
        const int row = i * 64 + (tid >> 2);
        const int off = row * kAPitch + (tid & 3) * 16;
        v4u p, n;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t pp, nn;
          split_signed(xr[i][j], pp, nn);
          p[j] = pp;
          n[j] = nn;
        }
        *reinterpret_cast<v4u *>(ap + off) = p;
        *reinterpret_cast<v4u *>(an + off) = n;
      } else {
        const int half = i / (BM / 64), ii = i % (BM / 64);
        const int row = ii * 64 + (tid >> 2);
        const int off = row * kAPitch + (tid & 3) * 16;
        *reinterpret_cast<v4u *>((half ? an : ap) + off) = xr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i)
      *reinterpret_cast<v4u *>(bw + (i * 4 + wave) * 1024 + lane * 16) = wr[i];
  };

  constexpr int YM = KEEP_F32 ? FM : 1, YN = KEEP_F32 ? FN : 1;
  v4i accp[FM][FN], accn[FM][FN];
  float yacc[YM][YN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      accp[i][j] = v4i{0, 0, 0, 0};
      accn[i][j] = v4i{0, 0, 0, 0};
    }
#pragma unroll
  for (int i = 0; i < YM; ++i)
#pragma unroll
    for (int j = 0; j < YN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[i][j][r] = 0.0f;

  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;
  const float *i_pos = a.act + 2 * nS, *i_neg = a.act + 3 * nS;

  // this lane's output columns (one per B fragment) and first output row
  const int col_base = n0 + wn * WN + (lane & 15);
  const int row_base = m0 + wm * WM + (lane >> 4) * 4;

  auto dump_frag = [&](int seg, int i, int j, const v4i &p, const v4i &n) {
    const int col = col_base + j * 16;
    if (col >= a.N) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = row_base + i * 16 + r;
      if (m >= a.M) continue;
      const int64_t o = ((int64_t)seg * a.M + m) * a.N + col;
      a.acc[o] = p[r];
      a.acc[(int64_t)nS * a.M * a.N + o] = n[r];
    }
  };

  // per-column scale of segment seg for fragment column j: s_w * s+, s_w * s-
  auto col_scales = [&](int seg, float *cp, float *cn) {
    const float sp = s_pos[seg], sn = s_neg[seg];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col_base + j * 16;
      const float ws = col < a.N ? a.w_scale[(int64_t)seg * a.N + col] : 0.0f;
      cp[j] = sp * ws;
      cn[j] = sn * ws;
    }
  };


  // ---- prologue ----
  int qseg = 0;  // segment of the step being staged
  load_x(0);
  load_w(0);
  store_stage(0, i_pos[0], i_neg[0]);
  __syncthreads();

  int seg = 0;  // segment of the step being multiplied
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) {
      load_x(kt + 1);
      load_w(kt + 1);
    }
    // ---- matrix-core work on stage `cur` ----
    {
      const uint8_t *ap = smem + cur * STAGE;
      const uint8_t *an = ap + A_BYTES;
      const uint8_t *bw = an + A_BYTES;
      v4u fa_p[FM], fa_n[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int off = (wm * WM + i * 16 + (lane & 15)) * kAPitch + (lane >> 4) * 16;
        fa_p[i] = lds_read16(ap + off);
        fa_n[i] = lds_read16(an + off);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4u fb = lds_read16(bw + (wn * FN + j) * 1024 + lane * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const v4i &A_p = reinterpret_cast<const v4i &>(fa_p[i]);
          const v4i &A_n = reinterpret_cast<const v4i &>(fa_n[i]);
          const v4i &B = reinterpret_cast<const v4i &>(fb);
          v4i &P = accp[i][j];
          v4i &Nn = accn[i][j];
          if (MODE == STEP) {  // each step is a segment: start from zero
            const v4i zero = {0, 0, 0, 0};
            P = __builtin_amdgcn_mfma_i32_16x16x64_i8(A_p, B, zero, 0, 0, 0);
            Nn = __builtin_amdgcn_mfma_i32_16x16x64_i8(A_n, B, zero, 0, 0, 0);
          } else {
            P = __builtin_amdgcn_mfma_i32_16x16x64_i8(A_p, B, P, 0, 0, 0);
            Nn = __builtin_amdgcn_mfma_i32_16x16x64_i8(A_n, B, Nn, 0, 0, 0);
          }
        }
      }
    }
    if (more) {
      if (kt + 1 >= a.seg_end_tile[qseg]) ++qseg;
      store_stage(cur ^ 1, i_pos[qseg], i_neg[qseg]);
    }
    const bool seg_end = MODE == STEP || (MODE == MULTI && kt + 1 == a.seg_end_tile[seg]);
    if (MODE != SINGLE && seg_end) {
      float cp[FN], cn[FN];
      col_scales(seg, cp, cn);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          v4i &P = accp[i][j];
          v4i &Nn = accn[i][j];
          if (DEBUG) dump_frag(seg, i, j, P, Nn);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float &y = yacc[KEEP_F32 ? i : 0][KEEP_F32 ? j : 0][r];
            y = __builtin_fmaf(cn[j], (float)Nn[r], __builtin_fmaf(cp[j], (float)P[r], y));
          }
          if (MODE == MULTI) {
            P = v4i{0, 0, 0, 0};
            Nn = v4i{0, 0, 0, 0};
          }
        }
      ++seg;
    }
    __syncthreads();
  }

  // ---- epilogue: bf16 store ----
  float cp[FN], cn[FN];
  if (MODE == SINGLE) col_scales(0, cp, cn);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (MODE == SINGLE && DEBUG) dump_frag(0, i, j, accp[i][j],
                                             accn[i][j]);
      const int col = col_base + j * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row_base + i * 16 + r;
        float v;
        if (MODE == SINGLE)
          v = __builtin_fmaf(cn[j], (float)accn[i][j][r],
                             cp[j] * (float)accp[i][j][r]);
        else
          v = yacc[KEEP_F32 ? i : 0][KEEP_F32 ? j : 0][r];
        if (m < a.M && col < a.N) a.y[(int64_t)m * a.ld_y + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

template <int BM, int BN, int WM, int WN, int MODE, int OCC>
hipError_t launch_variant(TileArgs t, int amode, bool debug, hipStream_t s) {
  t.tiles_m = (t.M + BM - 1) / BM;
  t.tiles_n = (t.N + BN - 1) / BN;
  dim3 grid((unsigned)(t.tiles_m * t.tiles_n)), block(256);
#define SQ_LAUNCH(AM, DBG) \
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WM, WN, AM, MODE, DBG, OCC>), grid, block, 0, s, t)
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
  if (p.ks.n == 1) return launch_variant<128, 256, 64, 128, SINGLE, 1>(t, amode, debug, s);
  if (every_step) return launch_variant<64, 256, 32, 128, STEP, 2>(t, amode, debug, s);
  return launch_variant<64, 256, 32, 128, MULTI, 2>(t, amode, debug, s);
}

}  // namespace sq
