// gemm_smallm.hip -- the DualScale x SegLinear W8A8 layer for small M
// (M <= 16, e.g. the AdaNorm projection of a DiT block: one row per image),
// one launch, bound by streaming the int8 weight from HBM once.
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes): "DualScale" (split,
//      scales, reconstruction, one batched launch with a fused epilogue);
//      "SegLinear" (AdaNorm outputs chunked into shift/scale: the
//      output-segmented pattern).
// [P2] "SegQuant" (hliangzhao.me): section 1 (AdaNorm emits shift, scale
//      and gate for two branches), section 3 (reconstruction).
//
// Design: each wave owns one 16-column n-tile and walks all of K.  The
// packed weight keeps an n-tile's K as consecutive 1 KiB tiles, so a wave's
// weight stream is one contiguous range read with one 16-byte load per lane
// per tile -- the matrix-core B operand as loaded.  A wave requests up to
// kRing tiles before doing anything else, so for K <= 2048 the whole weight
// is in flight from the first instructions; the workgroup meanwhile
// quantises X (M rows, a chunk of K at a time) into two LDS planes.  Rows of
// the 16-row A operand at or beyond M are zero.  Both halves run on the int8
// 16x16x64 matrix cores against the same B registers (the padding rows cost
// nothing: the kernel is bound by HBM).  Index math uses shifts only; the
// scale table is staged once in LDS.
#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kXBytes = 32768;  // both planes of one K-chunk
constexpr int kRing = 32;       // weight tiles in flight per wave
constexpr int kXRegs = 8;       // 16-byte X pieces staged per thread

struct SmallArgs {
  int32_t M, N, K;
  int32_t rows_log2;   // log2 of M rounded up to a power of two
  int32_t kc_tiles;    // K-chunk in 64-steps
  const uint16_t *x;
  int64_t ld_x;
  const int8_t *xq;
  int64_t ld_q;
  int64_t plane_stride;
  int32_t q_layout;  // -1: bf16 input, 0: signed codes, 1: planes
  const int8_t *w;
  const float *w_scale;
  const float *act;
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc;
  int32_t n_kseg;
  int32_t seg_end_tile[kMaxKSeg];
};

// QL: activation input, -1 bf16 (quantised here), 0 signed codes, 1 planes.
// ONE: all of K is one chunk that fits the weight ring (no refills, no
// chunk loop: straight-line code with an exact count of loads in flight).
template <int WPG, int QL, bool ONE, bool DEBUG>
__global__ __launch_bounds__(64 * WPG) void gemm_smallm_kernel(SmallArgs a) {
  constexpr int NTHR = 64 * WPG;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kXBytes];
  __shared__ float inv_tab[2 * kMaxKSeg];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int NT = a.N / 16, KT = a.K / 64;
  const int nt = blockIdx.x * WPG + wave;
  const bool active = nt < NT;
  const int pitch = a.kc_tiles * 64 + 16;  // LDS row pitch (bytes)
  uint8_t *plane_p = xs;
  uint8_t *plane_n = xs + a.M * pitch;
  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;

  // thread -> (row, first 16-byte piece) for staging X: threads per row is a
  // power of two
  const int tpr_log2 = __builtin_ctz(NTHR) - a.rows_log2;
  const int xrow = tid >> tpr_log2;
  const int xp0 = tid & ((1 << tpr_log2) - 1);
  const int tpr = 1 << tpr_log2;

  const int row = lane & 15;        // A-operand row of this lane
  const int kq = (lane >> 4) * 16;  // its 16-byte k offset inside a step
  const int n = nt * 16 + (lane & 15);
  const int8_t *wcol = a.w + (int64_t)(active ? nt : 0) * KT * 1024 + lane * 16;

  v4i accp = {0, 0, 0, 0}, accn = {0, 0, 0, 0};
  float yacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int seg = 0;

  for (int kc0 = 0; kc0 < (ONE ? 1 : KT); kc0 += (ONE ? 1 : a.kc_tiles)) {
    const int ktn = ONE ? KT : min(a.kc_tiles, KT - kc0);
    const int ppr = ktn * (QL < 0 ? 8 : 4);  // 16-byte pieces per row
    // (1) this thread's X pieces (issued before the weight stream, so that
    //     waiting for them does not wait for the weights)
    // one address form for both inputs: 16-byte pieces of a row
    constexpr bool bf16_in = QL < 0;
    const uint8_t *xsrc = bf16_in ? reinterpret_cast<const uint8_t *>(a.x)
                                  : reinterpret_cast<const uint8_t *>(a.xq);
    const int64_t xstride = bf16_in ? a.ld_x * 2 : a.ld_q;
    const int64_t xcol0 = (int64_t)kc0 * (bf16_in ? 128 : 64);
    v4u xr[kXRegs];
#pragma unroll
    for (int i = 0; i < kXRegs; ++i) {
      const int p = xp0 + i * tpr;
      xr[i] = v4u{0u, 0u, 0u, 0u};
      if (xrow < a.M && p < ppr)
        xr[i] = *reinterpret_cast<const v4u *>(xsrc + (int64_t)xrow * xstride + xcol0 + p * 16);
    }
    v4u xn[QL == 1 ? kXRegs : 1];  // the - plane of pre-split input
    if (QL == 1) {
#pragma unroll
      for (int i = 0; i < kXRegs; ++i) {
        const int p = xp0 + i * tpr;
        xn[QL == 1 ? i : 0] = v4u{0u, 0u, 0u, 0u};
        if (xrow < a.M && p < ppr)
          xn[QL == 1 ? i : 0] = *reinterpret_cast<const v4u *>(a.xq + a.plane_stride + (int64_t)xrow * a.ld_q +
                                                 (int64_t)kc0 * 64 + p * 16);
      }
    }
    // (2) the weight stream of this chunk, up to kRing tiles ahead
    // (slots past the chunk re-read its last tile: branch-free, so the
    //  count of loads in flight is known and the wait for X below is exact)
    v4u ring[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d)
      ring[d] = *reinterpret_cast<const v4u *>(wcol + (int64_t)(kc0 + min(d, ktn - 1)) * 1024);
    // the inverse scales, staged in LDS (uniform index: scalar loads, which
    // do not wait behind the vector loads above)
    if (ONE || kc0 == 0) {
      for (int i = 0; i < nS; ++i) {
        const float ip = a.act[2 * nS + i], in = a.act[3 * nS + i];
        if (tid == (i & (NTHR - 1))) {
          inv_tab[2 * i] = ip;
          inv_tab[2 * i + 1] = in;
        }
      }
    }
    // (3) quantise (or split) into the two LDS planes
    __syncthreads();  // previous chunk's operand reads are done; inv_tab is ready
#pragma unroll
    for (int i = 0; i < kXRegs; ++i) {
      const int p = xp0 + i * tpr;
      if (xrow < a.M && p < ppr) {
        if (QL < 0) {
          const int kt = kc0 + (p >> 3);
          int s = 0;
          while (kt >= a.seg_end_tile[s]) ++s;
          v2u pp, nn;
          quant8_planes(xr[i], inv_tab[2 * s], inv_tab[2 * s + 1], pp, nn);
          *reinterpret_cast<v2u *>(plane_p + xrow * pitch + p * 8) = pp;
          *reinterpret_cast<v2u *>(plane_n + xrow * pitch + p * 8) = nn;
        } else if (QL == 0) {
          v4u pp, nn;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t u, v;
            split_signed(xr[i][j], u, v);
            pp[j] = u;
            nn[j] = v;
          }
          *reinterpret_cast<v4u *>(plane_p + xrow * pitch + p * 16) = pp;
          *reinterpret_cast<v4u *>(plane_n + xrow * pitch + p * 16) = nn;
        } else {
          *reinterpret_cast<v4u *>(plane_p + xrow * pitch + p * 16) = xr[i];
          *reinterpret_cast<v4u *>(plane_n + xrow * pitch + p * 16) = xn[QL == 1 ? i : 0];
        }
      }
    }
    __syncthreads();
    // (4) matrix-core steps over the chunk, the ring kept kRing tiles ahead
    for (int t0 = 0; t0 < (ONE ? 1 : ktn); t0 += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        const int t = t0 + d;
        if (t < ktn) {
          v4u fp = {0u, 0u, 0u, 0u}, fn = {0u, 0u, 0u, 0u};
          if (row < a.M) {
            fp = *reinterpret_cast<const v4u *>(plane_p + row * pitch + t * 64 + kq);
            fn = *reinterpret_cast<const v4u *>(plane_n + row * pitch + t * 64 + kq);
          }
          const v4u b = ring[d];
          if (!ONE && t + kRing < ktn)
            ring[d] = *reinterpret_cast<const v4u *>(wcol + (int64_t)(kc0 + t + kRing) * 1024);
          accp = __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(fp),
                                                       reinterpret_cast<const v4i &>(b), accp, 0, 0, 0);
          accn = __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(fn),
                                                       reinterpret_cast<const v4i &>(b), accn, 0, 0, 0);
          if (kc0 + t + 1 == a.seg_end_tile[seg]) {
            if (DEBUG) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int m = (lane >> 4) * 4 + r;
                if (active && m < a.M) {
                  const int64_t o = ((int64_t)seg * a.M + m) * a.N + n;
                  a.acc[o] = accp[r];
                  a.acc[(int64_t)nS * a.M * a.N + o] = accn[r];
                }
              }
            }
            const float ws = active ? a.w_scale[(int64_t)seg * a.N + n] : 0.0f;
            const float cp = s_pos[seg] * ws, cn = s_neg[seg] * ws;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              yacc[r] = __builtin_fmaf(cn, (float)accn[r], __builtin_fmaf(cp, (float)accp[r], yacc[r]));
            accp = v4i{0, 0, 0, 0};
            accn = v4i{0, 0, 0, 0};
            ++seg;
          }
        }
      }
    }
  }
  // epilogue: rows (lane/16)*4 + r of column n
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = (lane >> 4) * 4 + r;
    if (active && m < a.M) a.y[(int64_t)m * a.ld_y + n] = (uint16_t)f32_to_bf16_rne(yacc[r]);
  }
}

}  // namespace

hipError_t launch_gemm_smallm(const GemmProblem &p, hipStream_t s) {
  constexpr int WPG = 2;
  constexpr int NTHR = 64 * WPG;
  SmallArgs a{};
  a.M = (int32_t)p.M;
  a.N = (int32_t)p.N;
  a.K = (int32_t)p.K;
  int rl = 0;
  while ((1 << rl) < p.M) ++rl;
  a.rows_log2 = rl;
  // K-chunk: both planes (row pitch chunk*64 + 16) fit the LDS buffer, and a
  // row's pieces fit the staging registers of its threads
  const int pieces_per_tile = p.x ? 8 : 4;
  int kc = (int)((kXBytes / (2 * p.M) - 16) / 64);
  const int tpr = NTHR >> rl;
  const int max_tiles_regs = (tpr * kXRegs) / pieces_per_tile;
  if (kc > max_tiles_regs) kc = max_tiles_regs;
  if (kc < 1) kc = 1;
  a.kc_tiles = kc;
  a.x = p.x;
  a.ld_x = p.ld_x;
  a.xq = p.xq;
  a.ld_q = p.ld_q;
  a.plane_stride = p.q_layout == 1 ? p.M * p.ld_q : 0;
  a.q_layout = p.x ? -1 : p.q_layout;
  a.w = p.w_packed;
  a.w_scale = p.w_scale;
  a.act = p.act;
  a.y = p.y;
  a.ld_y = p.ld_y;
  a.acc = p.acc_debug;
  a.n_kseg = p.ks.n;
  for (int i = 0; i < p.ks.n; ++i) a.seg_end_tile[i] = p.ks.end[i] / 64;
  dim3 grid((unsigned)((p.N / 16 + WPG - 1) / WPG)), block(NTHR);
#define SQ_SMALL(QLV, ONEV, DBG) \
  hipLaunchKernelGGL((gemm_smallm_kernel<WPG, QLV, ONEV, DBG>), grid, block, 0, s, a)
#define SQ_SMALL_Q(ONEV, DBG)              \
  do {                                     \
    if (ql < 0) SQ_SMALL(-1, ONEV, DBG);    \
    else if (ql == 0) SQ_SMALL(0, ONEV, DBG); \
    else SQ_SMALL(1, ONEV, DBG);            \
  } while (0)
  const int ql = a.q_layout;
  const int KT = (int)(p.K / 64);
  const bool one = KT <= kRing && KT <= a.kc_tiles;
  if (p.acc_debug) {
    if (one) SQ_SMALL_Q(true, true); else SQ_SMALL_Q(false, true);
  } else {
    if (one) SQ_SMALL_Q(true, false); else SQ_SMALL_Q(false, false);
  }
#undef SQ_SMALL_Q
#undef SQ_SMALL
  return hipGetLastError();
}

}  // namespace sq
