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
// per tile (the matrix-core B operand as loaded).  The workgroup first
// quantises the whole of X (M rows, a chunk of K at a time) into two LDS
// planes; every row of the 16-row A operand at or beyond M is zero.  Both
// halves run on the int8 16x16x64 matrix cores against the same B registers
// (the padding rows cost nothing: the kernel is bound by HBM).  The weight
// loads for a chunk are issued before X is quantised, so their latency
// overlaps the quantisation.
#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kLdsBytes = 32768;  // both planes of one K-chunk
constexpr int kRing = 16;         // weight tiles in flight per wave
constexpr int kXRegs = 8;         // 16-byte X pieces staged per thread

struct SmallArgs {
  int32_t M, N, K;
  int32_t kc_tiles;  // K-chunk in 64-steps (2 * M * kc_tiles * (64+16) <= kLdsBytes)
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

template <int WPG, bool DEBUG>
__global__ __launch_bounds__(64 * WPG) void gemm_smallm_kernel(SmallArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NT = a.N / 16, KT = a.K / 64;
  const int nt = blockIdx.x * WPG + wave;
  const bool active = nt < NT;
  const int pitch = a.kc_tiles * 64 + 16;  // LDS row pitch (bytes)
  uint8_t *plane_p = xs;
  uint8_t *plane_n = xs + a.M * pitch;
  const int nS = a.n_kseg;
  const float *s_pos = a.act, *s_neg = a.act + nS;
  const float *i_pos = a.act + 2 * nS, *i_neg = a.act + 3 * nS;

  const int row = lane & 15;      // A-operand row of this lane
  const int kq = (lane >> 4) * 16;  // its 16-byte k offset inside a step
  const int n = nt * 16 + (lane & 15);
  const int8_t *wcol = a.w + (int64_t)(active ? nt : 0) * KT * 1024 + lane * 16;

  v4i accp = {0, 0, 0, 0}, accn = {0, 0, 0, 0};
  float yacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int seg = 0;

  auto fold = [&](int s) {
    const float ws = active ? a.w_scale[(int64_t)s * a.N + n] : 0.0f;
    const float cp = s_pos[s] * ws, cn = s_neg[s] * ws;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      yacc[r] = __builtin_fmaf(cn, (float)accn[r], __builtin_fmaf(cp, (float)accp[r], yacc[r]));
    }
  };
  auto dump = [&](int s) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = (lane >> 4) * 4 + r;
      if (active && m < a.M) {
        const int64_t o = ((int64_t)s * a.M + m) * a.N + n;
        a.acc[o] = accp[r];
        a.acc[(int64_t)nS * a.M * a.N + o] = accn[r];
      }
    }
  };

  for (int kc0 = 0; kc0 < KT; kc0 += a.kc_tiles) {
    const int ktn = min(a.kc_tiles, KT - kc0);
    const int pieces_per_row = ktn * (a.q_layout < 0 ? 8 : 4);  // 16-byte pieces
    const int pieces = a.M * pieces_per_row;
    // (1) stage this thread's X pieces (issued before the weight loads so
    //     that waiting for them does not wait for the weight stream)
    v4u xr[kXRegs];
#pragma unroll
    for (int i = 0; i < kXRegs; ++i) {
      const int c = tid + i * 64 * WPG;
      xr[i] = v4u{0u, 0u, 0u, 0u};
      if (c < pieces) {
        const int r = c / pieces_per_row, p = c - r * pieces_per_row;
        if (a.q_layout < 0)
          xr[i] = *reinterpret_cast<const v4u *>(a.x + (int64_t)r * a.ld_x + (int64_t)kc0 * 64 + p * 8);
        else
          xr[i] = *reinterpret_cast<const v4u *>(a.xq + (int64_t)r * a.ld_q + (int64_t)kc0 * 64 + p * 16);
      }
    }
    // (2) weight ring prologue
    v4u ring[kRing];
#pragma unroll
    for (int d = 0; d < kRing; ++d)
      if (d < ktn) ring[d] = *reinterpret_cast<const v4u *>(wcol + (int64_t)(kc0 + d) * 1024);
    // (3) quantise into the two LDS planes
    if (kc0 > 0) __syncthreads();  // previous chunk's readers are done
#pragma unroll
    for (int i = 0; i < kXRegs; ++i) {
      const int c = tid + i * 64 * WPG;
      if (c < pieces) {
        const int r = c / pieces_per_row, p = c - r * pieces_per_row;
        if (a.q_layout < 0) {
          const int kt = kc0 + (p >> 3);
          int s = 0;
          while (kt >= a.seg_end_tile[s]) ++s;
          v2u pp, nn;
          quant8_planes(xr[i], i_pos[s], i_neg[s], pp, nn);
          *reinterpret_cast<v2u *>(plane_p + r * pitch + p * 8) = pp;
          *reinterpret_cast<v2u *>(plane_n + r * pitch + p * 8) = nn;
        } else {
          v4u pp, nn;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t u, v;
            split_signed(xr[i][j], u, v);
            pp[j] = u;
            nn[j] = v;
          }
          *reinterpret_cast<v4u *>(plane_p + r * pitch + p * 16) = pp;
          *reinterpret_cast<v4u *>(plane_n + r * pitch + p * 16) = nn;
        }
      }
    }
    // pre-split planes: the + plane was staged above (its split leaves the
    // - plane zero); copy the - plane from its own buffer
    if (a.q_layout == 1) {
      for (int c = tid; c < pieces; c += 64 * WPG) {
        const int r = c / pieces_per_row, p = c - r * pieces_per_row;
        const v4u q = *reinterpret_cast<const v4u *>(a.xq + a.plane_stride + (int64_t)r * a.ld_q +
                                                     (int64_t)kc0 * 64 + p * 16);
        *reinterpret_cast<v4u *>(plane_n + r * pitch + p * 16) = q;
      }
    }
    __syncthreads();
    // (4) matrix-core steps over the chunk, the ring kept kRing tiles ahead
    for (int t0 = 0; t0 < ktn; t0 += kRing) {
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
          if (t + kRing < ktn) ring[d] = *reinterpret_cast<const v4u *>(wcol + (int64_t)(kc0 + t + kRing) * 1024);
          accp = __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(fp),
                                                       reinterpret_cast<const v4i &>(b), accp, 0, 0, 0);
          accn = __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(fn),
                                                       reinterpret_cast<const v4i &>(b), accn, 0, 0, 0);
          if (kc0 + t + 1 == a.seg_end_tile[seg]) {
            if (DEBUG) dump(seg);
            fold(seg);
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
  constexpr int WPG = 4;
  SmallArgs a{};
  a.M = (int32_t)p.M;
  a.N = (int32_t)p.N;
  a.K = (int32_t)p.K;
  // chunk of K whose two planes (row pitch chunk+16) fit the LDS buffer
  int kc = (int)((kLdsBytes / (2 * p.M) - 16) / 64);
  const int max_pieces_tiles = (kXRegs * 64 * WPG) / ((int)p.M * (p.x ? 8 : 4));
  if (kc > max_pieces_tiles) kc = max_pieces_tiles;
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
  dim3 grid((unsigned)((p.N / 16 + WPG - 1) / WPG)), block(64 * WPG);
  if (p.acc_debug)
    hipLaunchKernelGGL((gemm_smallm_kernel<WPG, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemm_smallm_kernel<WPG, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace sq
