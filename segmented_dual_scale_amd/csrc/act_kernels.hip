// act_kernels.hip -- activation-side kernels for gfx950:
//   * AMax calibration of the static DualScale scales
//     [P1 framework table, AMax calibrator; P1 "DualScale" scale equation;
//      P2 section 3, s+ = max/127 and s- = |min|/128], and
//   * the single-scale variant of the calibration (one symmetric scale per
//     K-segment, amax/127, written into both halves of the table): the
//     plain W8A8 baseline that DualScale is compared with [P2 deployment-cost
//     table, INT8 baseline row; P1 limitations section, enabling DualScale
//     only where the polarity asymmetry calls for it], and
//   * the producer-fused variant: SiLU or exact-erf GELU of a bf16
//     pre-activation, rounded to bf16, then quantised, in one HBM pass, so
//     the activated bf16 X never round-trips through memory (SiLU and GELU
//     are where the polarity asymmetry comes from [P1 DualScale motivation;
//     P2 section 3]), and
//   * the standalone polarity split + dual-scale quantisation
//     [P1 "DualScale" split and quantisation; P2 section 3, Q_dual], an
//     HBM-streaming kernel: 2 bytes read and 1 (signed code) or 2 (two
//     planes) bytes written per element.
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes).
// [P2] "SegQuant" (hliangzhao.me).
//
// Work split: a 2-D grid, blockIdx.y = K-segment (so its scales are uniform
// across the workgroup and live in scalar registers), blockIdx.x = a block
// of rows.  Inside a workgroup each wave walks rows; L lanes (a power of two
// up to 64) share one row and step through it 8 elements (16 bytes) at a
// time, so narrow segments (64 columns = 8 chunks) still fill the wave.
#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

struct ActArgs {
  const uint16_t *x;
  int64_t M, K, ld_x;
  int32_t rows_per_block;
  int32_t lanes_log2;  // lanes sharing one row
  const float *act;    // [4][n_kseg]
  float *act_out;      // the same table, written by calibration
  int8_t *q;
  int64_t ld_q;
  int64_t plane_stride;  // elements between the + and - planes (0: signed)
  int32_t n_kseg;
  int32_t single;        // quantise both signs with the + half's inverse
  SegTable ks;
  uint16_t *x_out;       // producer-fused kernel: optional bf16 copy of the activation
  int64_t ld_xo;
};

__device__ __forceinline__ v4u load_x8(const uint16_t *p) {
  return *reinterpret_cast<const v4u *>(p);
}

// Tail of a row whose length is not a multiple of 8: element by element.
__device__ __forceinline__ uint32_t load_bf16(const uint16_t *p) { return *p; }

__global__ void calib_init_kernel(float *act, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2 * n) act[i] = 0.0f;
}

__global__ __launch_bounds__(256) void calib_reduce_kernel(ActArgs a) {
  const int seg = blockIdx.y;
  const int64_t k0 = a.ks.off[seg], k1 = a.ks.end[seg];
  const int L = 1 << a.lanes_log2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> a.lanes_log2, col = lane & (L - 1);
  const int rows_per_step = (64 >> a.lanes_log2) * (blockDim.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
  const int64_t r1 = min(r0 + a.rows_per_block, a.M);
  float mp = 0.0f, mn = 0.0f;
  for (int64_t r = r0 + wave * (64 >> a.lanes_log2) + sub; r < r1; r += rows_per_step) {
    const uint16_t *row = a.x + r * a.ld_x;
    int64_t k = k0 + 8 * col;
    for (; k + 8 <= k1; k += 8 * L) {
      v4u v = load_x8(row + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo = bf16_lo(v[j]), hi = bf16_hi(v[j]);
        mp = fmaxf(mp, fmaxf(pos_part(lo), pos_part(hi)));
        mn = fmaxf(mn, fmaxf(neg_mag(lo), neg_mag(hi)));
      }
    }
    for (int64_t kk = k; kk < k1 && kk < k + 8; ++kk) {
      float f = __uint_as_float(load_bf16(row + kk) << 16);
      mp = fmaxf(mp, pos_part(f));
      mn = fmaxf(mn, neg_mag(f));
    }
  }
  mp = wave_max(mp);
  mn = wave_max(mn);
  if (lane == 0) {
    atomicMax(reinterpret_cast<unsigned *>(a.act_out) + seg, __float_as_uint(mp));
    atomicMax(reinterpret_cast<unsigned *>(a.act_out) + a.n_kseg + seg, __float_as_uint(mn));
  }
}

// DualScale: s+ = max/127, s- = |min|/128.  Single scale (one symmetric
// range per segment): s = max(max, |min|)/127 in both halves, so that the
// dual-scale quantiser then produces the plain symmetric codes in
// [-127, 127].
__global__ void calib_finalize_kernel(float *act, int n, int single) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float mx = act[i], mn = act[n + i];
  float sp, ip, sn, in;
  if (single) {
    scale_pair(fmaxf(mx, mn), 127.0, sp, ip);
    sn = sp;
    in = ip;
  } else {
    scale_pair(mx, 127.0, sp, ip);
    scale_pair(mn, 128.0, sn, in);
  }
  act[i] = sp;
  act[n + i] = sn;
  act[2 * n + i] = ip;
  act[3 * n + i] = in;
}

// Each thread owns rows r0 + wave * (64 / L) + sub + j * rows_per_step of the
// block and, in each, the 8-element chunks col, col + L, ... of the segment.
// Its (row, chunk) items are taken kBatch at a time, all loads first: the
// int8 stores may alias the bf16 input as far as the compiler can tell, so
// one item's store would otherwise hold back the next item's load.
constexpr int kBatch = 4;

struct ThreadItems {
  int64_t rfirst, k0;
  int rows_per_step, L, col, nrows, nch, items;
  int full;   // whole 8-element chunks in the segment
  bool tail;  // this lane also takes the elements past the last whole chunk
};

__device__ __forceinline__ ThreadItems thread_items(const ActArgs &a, int64_t k0, int64_t k1) {
  ThreadItems it;
  it.L = 1 << a.lanes_log2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane >> a.lanes_log2;
  it.col = lane & (it.L - 1);
  it.rows_per_step = (64 >> a.lanes_log2) * (blockDim.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_block;
  const int64_t r1 = min(r0 + a.rows_per_block, a.M);
  it.rfirst = r0 + wave * (64 >> a.lanes_log2) + sub;
  it.nrows = it.rfirst < r1 ? (int)((r1 - it.rfirst + it.rows_per_step - 1) / it.rows_per_step) : 0;
  it.k0 = k0;
  it.full = (int)((k1 - k0) / 8);
  it.nch = it.col < it.full ? (it.full - it.col + it.L - 1) / it.L : 0;
  it.items = it.nrows * it.nch;
  it.tail = k0 + 8 * (int64_t)it.full < k1 && it.col == it.full % it.L;
  return it;
}

// Row and first column of item t (0 <= t < items).
__device__ __forceinline__ void item_at(const ThreadItems &it, int t, int64_t &r, int64_t &k) {
  const int j = t / it.nch, i = t - j * it.nch;
  r = it.rfirst + (int64_t)j * it.rows_per_step;
  k = it.k0 + 8 * (it.col + (int64_t)i * it.L);
}

template <bool PLANES>
__global__ __launch_bounds__(256) void quantize_kernel(ActArgs a) {
  const int seg = blockIdx.y;
  const int64_t k0 = a.ks.off[seg], k1 = a.ks.end[seg];
  const float inv_pos = a.act[2 * a.n_kseg + seg];
  const float inv_neg = a.single ? inv_pos : a.act[3 * a.n_kseg + seg];
  const ThreadItems it = thread_items(a, k0, k1);
  for (int t0 = 0; t0 < it.items; t0 += kBatch) {
    v4u v[kBatch];
    int64_t off[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      int64_t r, k;
      item_at(it, min(t0 + u, it.items - 1), r, k);  // past the end: repeat the last item
      v[u] = load_x8(a.x + r * a.ld_x + k);
      off[u] = r * a.ld_q + k;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (t0 + u < it.items) {
        if (PLANES) {
          v2u p, n;
          quant8_planes(v[u], inv_pos, inv_neg, p, n);
          *reinterpret_cast<v2u *>(a.q + off[u]) = p;
          *reinterpret_cast<v2u *>(a.q + a.plane_stride + off[u]) = n;
        } else {
          *reinterpret_cast<v2u *>(a.q + off[u]) = quant8_signed(v[u], inv_pos, inv_neg);
        }
      }
    }
  }
  // a segment width that is not a multiple of 8: the lane next in turn takes
  // the last few elements of each of its rows one by one
  if (it.tail) {
    for (int j = 0; j < it.nrows; ++j) {
      const int64_t r = it.rfirst + (int64_t)j * it.rows_per_step;
      const uint16_t *row = a.x + r * a.ld_x;
      int8_t *qrow = a.q + r * a.ld_q;
      for (int64_t kk = k0 + 8 * (int64_t)it.full; kk < k1; ++kk) {
        float f = __uint_as_float(load_bf16(row + kk) << 16);
        int8_t code = (int8_t)(quant_magic(f, inv_pos, inv_neg) & 0xffu);
        if (PLANES) {
          qrow[kk] = code > 0 ? code : 0;
          qrow[a.plane_stride + kk] = code < 0 ? code : 0;
        } else {
          qrow[kk] = code;
        }
      }
    }
  }
}

// GELU in its exact form z/2 (1 + erf(z / sqrt 2)), evaluated as
// z/2 erfc(-z / sqrt 2): the same function, but 1 + erf cancels to nothing in
// fp32 for z below about -4 while erfc keeps its relative precision.
// erfc(x), x = |z| / sqrt 2 >= 0, in the form of Numerical Recipes (Press et
// al., "Numerical Recipes in C", 2nd ed., section 6.2): t exp(-x^2 + P(t)),
// t = 1 / (1 + x/2), P a degree-9 Chebyshev fit, relative error below 1.2e-7
// for every x >= 0.  Branch free: erfc(-x) = 2 - erfc(x) gives z >= 0.
// Rounding x itself would cost about 2 x^2 ulps in the tail, so x enters
// only t; -x^2 = -z^2/2 is carried as an exact pair (one product and its FMA
// error), and its product with log2 e is split so that exp2 of the large
// part sees none of the small part's rounding.  With one-ulp reciprocal and
// exp2 the result is within 2^-20 of the true value, relative, over the
// whole bf16 input range (swept on the CPU with those errors injected).
// Large parts below -120 are evaluated 64 binades up and scaled back
// exactly, so results in the subnormal range are not flushed.
__device__ __forceinline__ float gelu_f32(float z) {
  const float kLog2e = 1.44269504f;             // log2 e, rounded to fp32
  const float kLog2eLo = 1.92596303e-08f;       // log2 e - kLog2e
  const float a = fminf(fabsf(z), 20.0f);  // erfc(20 / sqrt 2) underflows: the same result
  const float x = a * 0.70710678f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, x, 1.0f));
  float P = __builtin_fmaf(t, 0.17087277f, -0.82215223f);
  P = __builtin_fmaf(t, P, 1.48851587f);
  P = __builtin_fmaf(t, P, -1.13520398f);
  P = __builtin_fmaf(t, P, 0.27886807f);
  P = __builtin_fmaf(t, P, -0.18628806f);
  P = __builtin_fmaf(t, P, 0.09678418f);
  P = __builtin_fmaf(t, P, 0.37409196f);
  P = __builtin_fmaf(t, P, 1.00002368f);
  P = __builtin_fmaf(t, P, -1.26551223f);
  const float p = a * a, e = __builtin_fmaf(a, a, -p);  // z^2 = p + e exactly
  const float q = -0.5f * p, qe = -0.5f * e;           // -x^2 = q + qe exactly
  const float hi = q * kLog2e;
  float lo = __builtin_fmaf(q, kLog2e, -hi);
  lo = __builtin_fmaf(q, kLog2eLo, lo);
  lo = __builtin_fmaf(qe + P, kLog2e, lo);
  const bool deep = hi < -120.0f;
  const float eh = __builtin_amdgcn_exp2f(deep ? hi + 64.0f : hi) * (deep ? 0x1p-64f : 1.0f);
  const float E = t * eh * __builtin_amdgcn_exp2f(lo);
  return 0.5f * z * (z < 0.0f ? E : 2.0f - E);
}

// SiLU z / (1 + e^-z) as z sigmoid(z), the sigmoid from e^-|z| (library
// expf): e^-z itself overflows for z below about -88.7, where z / (1 + e^-z)
// would give 0 while the true value is still a normal float.
__device__ __forceinline__ float silu_f32(float z) {
  const float ez = expf(-fabsf(z));
  const float r = 1.0f / (1.0f + ez);
  return z * (z >= 0.0f ? r : ez * r);
}

// Activation of one element in fp32 [P1/P2: the SiLU and GELU outputs whose
// polarity asymmetry DualScale serves].
template <int ACT>
__device__ __forceinline__ float activate(float z) {
  if (ACT == 1) return silu_f32(z);
  return gelu_f32(z);
}

// Two bf16 pre-activations (one dword) -> two bf16 activations (one dword).
template <int ACT>
__device__ __forceinline__ uint32_t activate2(uint32_t u) {
  const uint32_t lo = f32_to_bf16_rne(activate<ACT>(bf16_lo(u)));
  const uint32_t hi = f32_to_bf16_rne(activate<ACT>(bf16_hi(u)));
  return lo | (hi << 16);
}

// ACT: 1 SiLU, 2 GELU.  WQ: write codes (PLANES: two planes, else signed);
// WX: write the bf16 activation.
template <int ACT, bool WQ, bool PLANES, bool WX>
__global__ __launch_bounds__(256) void act_quantize_kernel(ActArgs a) {
  const int seg = blockIdx.y;
  const int64_t k0 = a.ks.off[seg], k1 = a.ks.end[seg];
  const float inv_pos = WQ ? a.act[2 * a.n_kseg + seg] : 0.0f;
  const float inv_neg = WQ ? (a.single ? inv_pos : a.act[3 * a.n_kseg + seg]) : 0.0f;
  const ThreadItems it = thread_items(a, k0, k1);
  for (int t0 = 0; t0 < it.items; t0 += kBatch) {
    v4u z[kBatch];
    int64_t rr[kBatch], kk[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      item_at(it, min(t0 + u, it.items - 1), rr[u], kk[u]);  // past the end: repeat the last item
      z[u] = load_x8(a.x + rr[u] * a.ld_x + kk[u]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (t0 + u < it.items) {
        v4u v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = activate2<ACT>(z[u][j]);
        if (WX) *reinterpret_cast<v4u *>(a.x_out + rr[u] * a.ld_xo + kk[u]) = v;
        if (WQ) {
          int8_t *q = a.q + rr[u] * a.ld_q + kk[u];
          if (PLANES) {
            v2u p, n;
            quant8_planes(v, inv_pos, inv_neg, p, n);
            *reinterpret_cast<v2u *>(q) = p;
            *reinterpret_cast<v2u *>(q + a.plane_stride) = n;
          } else {
            *reinterpret_cast<v2u *>(q) = quant8_signed(v, inv_pos, inv_neg);
          }
        }
      }
    }
  }
  if (it.tail) {  // the elements past the last whole chunk, one by one
    for (int j = 0; j < it.nrows; ++j) {
      const int64_t r = it.rfirst + (int64_t)j * it.rows_per_step;
      const uint16_t *row = a.x + r * a.ld_x;
      for (int64_t k = k0 + 8 * (int64_t)it.full; k < k1; ++k) {
        const uint32_t xb = f32_to_bf16_rne(activate<ACT>(__uint_as_float(load_bf16(row + k) << 16)));
        if (WX) a.x_out[r * a.ld_xo + k] = (uint16_t)xb;
        if (WQ) {
          const int8_t code = (int8_t)(quant_magic(__uint_as_float(xb << 16), inv_pos, inv_neg) & 0xffu);
          int8_t *qrow = a.q + r * a.ld_q;
          if (PLANES) {
            qrow[k] = code > 0 ? code : 0;
            qrow[a.plane_stride + k] = code < 0 ? code : 0;
          } else {
            qrow[k] = code;
          }
        }
      }
    }
  }
}

// Rows per workgroup and lanes per row for a segment layout: aim for about
// `elems` elements per workgroup on the widest segment.
void plan_rows(int64_t M, const SegTable &ks, ActArgs &a, int64_t elems = 16384) {
  int64_t wmax = 0;
  for (int i = 0; i < ks.n; ++i) wmax = wmax > ks.end[i] - ks.off[i] ? wmax : ks.end[i] - ks.off[i];
  int64_t chunks = (wmax + 7) / 8;
  int lg = 0;
  while ((1 << lg) < chunks && lg < 6) ++lg;
  a.lanes_log2 = lg;
  int64_t rows_per_step = (64 >> lg) * 4;
  int64_t rows = (elems + wmax - 1) / wmax;
  rows = ((rows + rows_per_step - 1) / rows_per_step) * rows_per_step;
  // at most about four 16-byte pieces per thread: one batch of loads in
  // flight each, and more workgroups for narrow segments (24 segments of
  // 64: 7.5 instead of 8.3 us on MI355X)
  const int64_t per_row = (chunks + (1 << lg) - 1) >> lg;  // pieces per thread per row
  int64_t r4 = (4 * rows_per_step + per_row - 1) / per_row;
  r4 = ((r4 + rows_per_step - 1) / rows_per_step) * rows_per_step;
  if (r4 < rows) rows = r4;
  if (rows > M) rows = M < 1 ? 1 : M;
  a.rows_per_block = (int32_t)rows;
}

}  // namespace

hipError_t launch_calibrate(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                            const SegTable &ks, float *act, bool single, hipStream_t s) {
  const int n = ks.n;
  hipLaunchKernelGGL(calib_init_kernel, dim3((2 * n + 255) / 256), dim3(256), 0, s, act, n);
  if (M > 0) {
    ActArgs a{};
    a.x = x; a.M = M; a.K = K; a.ld_x = ld_x; a.act = act; a.act_out = act; a.n_kseg = n; a.ks = ks;
    plan_rows(M, ks, a);
    dim3 grid((unsigned)((M + a.rows_per_block - 1) / a.rows_per_block), (unsigned)n);
    hipLaunchKernelGGL(calib_reduce_kernel, grid, dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(calib_finalize_kernel, dim3((n + 255) / 256), dim3(256), 0, s, act, n,
                     single ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                           const SegTable &ks, const float *act, int8_t *q, int64_t ld_q,
                           int32_t layout, bool single, hipStream_t s) {
  if (M == 0) return hipSuccess;
  ActArgs a{};
  a.single = single ? 1 : 0;
  a.x = x; a.M = M; a.K = K; a.ld_x = ld_x; a.act = act; a.q = q; a.ld_q = ld_q;
  a.n_kseg = ks.n; a.ks = ks;
  a.plane_stride = layout ? M * ld_q : 0;
  plan_rows(M, ks, a);
  dim3 grid((unsigned)((M + a.rows_per_block - 1) / a.rows_per_block), (unsigned)ks.n);
  if (layout)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_act_quantize(const uint16_t *z, int64_t M, int64_t K, int64_t ld_z, int32_t act,
                               const SegTable &ks, const float *scales, int8_t *q, int64_t ld_q,
                               int32_t layout, uint16_t *x_out, int64_t ld_xo, hipStream_t s) {
  if (M == 0) return hipSuccess;
  ActArgs a{};
  a.x = z; a.M = M; a.K = K; a.ld_x = ld_z; a.act = scales; a.q = q; a.ld_q = ld_q;
  a.n_kseg = ks.n; a.ks = ks;
  a.plane_stride = layout ? M * ld_q : 0;
  a.x_out = x_out; a.ld_xo = ld_xo;
  plan_rows(M, ks, a);
  dim3 grid((unsigned)((M + a.rows_per_block - 1) / a.rows_per_block), (unsigned)ks.n);
  const bool wq = q != nullptr, wx = x_out != nullptr;
#define SQ_ACTQ(ACT, WQ, PL, WX) \
  hipLaunchKernelGGL((act_quantize_kernel<ACT, WQ, PL, WX>), grid, dim3(256), 0, s, a)
#define SQ_ACTQ_ALL(ACT)                                  \
  if (!wq) SQ_ACTQ(ACT, false, false, true);              \
  else if (layout && wx) SQ_ACTQ(ACT, true, true, true);  \
  else if (layout) SQ_ACTQ(ACT, true, true, false);       \
  else if (wx) SQ_ACTQ(ACT, true, false, true);           \
  else SQ_ACTQ(ACT, true, false, false);
  if (act == 1) {
    SQ_ACTQ_ALL(1)
  } else {
    SQ_ACTQ_ALL(2)
  }
#undef SQ_ACTQ_ALL
#undef SQ_ACTQ
  return hipGetLastError();
}

}  // namespace sq
