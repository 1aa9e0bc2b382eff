// weight_kernels.hip -- offline symmetric int8 weight quantisation per group
// and packing for the gfx950 matrix cores.
//
// [P1] "SegQuant: A Semantics-Aware and Generalizable Quantization Framework
//      for Diffusion Models" (papernotes.org notes), "SegLinear" section:
//      output-segmented (column segments) and input-segmented (row segments)
//      patterns, each segment quantised independently.
// [P2] "SegQuant" (hliangzhao.me), section 2, the same two equations.
//
// Group of (k, n): (K-segment of k) x (N-segment of n), or (K-segment of k) x
// {n} when per_column.  Per group a = max |w|, s_w = a/127, inv_w = 127/a,
// w_q = clamp(rne(fp32(w * inv_w)), -127, 127).
//
// Steps (four launches, offline):
//   1. colmax:   w_scale[i][n] <- max |w| over the rows of K-segment i
//                (atomic max over row chunks; w_scale doubles as the buffer)
//   2. groupmax: unless per_column, every column of an N-segment takes the
//                max over the segment's columns
//   3. pack:     w_q from the group's amax, written in the packed tile layout
//   4. finalize: w_scale[i][n] <- s_w = amax/127
// Packed layout (n-tile major; 1 KiB tiles of 64 k x 16 n): tile (nt, kt) at
// byte (nt*KT + kt)*1024, and inside it byte (g*16 + j)*16 + b holds
// w_q[kt*64 + g*16 + b][nt*16 + j] -- lane l = g*16 + j of a wave reads the
// 16 bytes of its matrix-core operand as one contiguous 16-byte load.
//
// 4-bit weights (W4A8, the pages' second precision [P2 deployment-cost
// table, SegQuant-4 row; P1 experiments, W4A8]): s_w = a/7, codes in
// [-7, 7], the same groups; stored biased (code + 8, 1..15) as nibbles in
// 512-byte tiles, lane l's 8 bytes at l*8: in its first dword byte i holds
// b = i (low nibble) and b = i + 4 (high nibble), in its second b = 8 + i
// and b = 12 + i.  Masking the low and the high nibbles of a dword then
// gives the operand bytes in order, four at a time.
#include "sq_device.hpp"
#include "sq_launch.hpp"

namespace sq {

namespace {

constexpr int kRowChunk = 256;

__global__ void zero_kernel(float *p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

struct ColMaxArgs {
  const float *w;
  int64_t K, N, ld_w;
  float *w_scale;
  SegTable ks;
};

// grid: x = column blocks of 256, y = row chunks of kRowChunk (global rows),
// each thread one column; the chunk is cut at segment boundaries.
__global__ __launch_bounds__(256) void colmax_kernel(ColMaxArgs a) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kRowChunk;
  const int64_t r1 = min(r0 + kRowChunk, a.K);
  if (n >= a.N) return;
  int seg = 0;
  while (a.ks.end[seg] <= r0) ++seg;
  int64_t r = r0;
  while (r < r1) {
    const int64_t e = min(r1, (int64_t)a.ks.end[seg]);
    float m = 0.0f;
    for (; r < e; ++r) m = fmaxf(m, fabsf(a.w[r * a.ld_w + n]));
    atomicMax(reinterpret_cast<unsigned *>(a.w_scale) + (int64_t)seg * a.N + n, __float_as_uint(m));
    ++seg;
  }
}

struct GroupMaxArgs {
  float *w_scale;
  int64_t N;
  NSegTable ns;
};

// grid: x = N-segment, y = K-segment.
__global__ __launch_bounds__(256) void groupmax_kernel(GroupMaxArgs a) {
  const int j = blockIdx.x, i = blockIdx.y;
  float *row = a.w_scale + (int64_t)i * a.N;
  const int64_t c0 = a.ns.off[j], c1 = a.ns.end[j];
  float m = 0.0f;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += 256) m = fmaxf(m, row[c]);
  m = wave_max(m);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  for (int64_t c = c0 + threadIdx.x; c < c1; c += 256) row[c] = m;
}

struct PackArgs {
  const float *w;
  int64_t K, N, ld_w;
  const float *w_amax;  // [n_kseg][N], the group amax
  int8_t *w_packed;
  SegTable ks;
};

// One thread per 16-byte lane-row of a packed tile: grid-stride over
// (tile, lane) = (nt*KT + kt)*64 + l.  W4: 4-bit codes, 8 bytes per lane-row.
template <bool W4>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr double kLevels = W4 ? 7.0 : 127.0;
  const int64_t KT = a.K / 64, NT = a.N / 16;
  const int64_t total = NT * KT * 64;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const int l = (int)(t & 63);
    const int64_t tile = t >> 6;
    const int64_t nt = tile / KT, kt = tile - nt * KT;
    const int g = l >> 4, j = l & 15;
    const int64_t n = nt * 16 + j;
    const int64_t kbase = kt * 64 + g * 16;
    int seg = 0;
    while (a.ks.end[seg] <= kbase) ++seg;
    float s, inv;
    scale_pair(a.w_amax[(int64_t)seg * a.N + n], kLevels, s, inv);
    const float lim = (float)kLevels;
    uint32_t code[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      float v = a.w[(kbase + b) * a.ld_w + n] * inv;
      v = __builtin_amdgcn_fmed3f(v, -lim, lim);
      code[b] = (__float_as_uint(v + kMagic) + (W4 ? 8u : 0u)) & 0xffu;  // W4: biased, 1..15
    }
    if (W4) {
      v2u out;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t wd = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) wd |= (code[8 * h + i] | (code[8 * h + i + 4] << 4)) << (8 * i);
        out[h] = wd;
      }
      *reinterpret_cast<v2u *>(a.w_packed + t * 8) = out;
    } else {
      v4u out;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        out[q] = code[4 * q] | (code[4 * q + 1] << 8) | (code[4 * q + 2] << 16) | (code[4 * q + 3] << 24);
      *reinterpret_cast<v4u *>(a.w_packed + t * 16) = out;
    }
  }
}

__global__ void finalize_kernel(float *w_scale, int64_t n, double levels) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s, inv;
  scale_pair(w_scale[i], levels, s, inv);
  w_scale[i] = s;
}

// W4 packed tiles -> the int8 packed layout (the GEMM's tile path).
__global__ __launch_bounds__(256) void widen_w4_kernel(const int8_t *w4, int64_t lanes, int8_t *w8) {
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < lanes; t += (int64_t)gridDim.x * 256)
    *reinterpret_cast<v4u *>(w8 + t * 16) = unpack_w4(*reinterpret_cast<const v2u *>(w4 + t * 8));
}

template <bool W4>
__global__ __launch_bounds__(256) void unpack_kernel(const int8_t *w_packed, int64_t K, int64_t N,
                                                     int8_t *w_kn, int64_t ld_w) {
  const int64_t KT = K / 64, NT = N / 16;
  const int64_t total = NT * KT * 64;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * 256) {
    const int l = (int)(t & 63);
    const int64_t tile = t >> 6;
    const int64_t nt = tile / KT, kt = tile - nt * KT;
    const int64_t n = nt * 16 + (l & 15);
    const int64_t kbase = kt * 64 + (l >> 4) * 16;
    const v4u in = W4 ? unpack_w4(*reinterpret_cast<const v2u *>(w_packed + t * 8))
                      : *reinterpret_cast<const v4u *>(w_packed + t * 16);
#pragma unroll
    for (int b = 0; b < 16; ++b)
      w_kn[(kbase + b) * ld_w + n] = (int8_t)((in[b >> 2] >> (8 * (b & 3))) & 0xffu);
  }
}

unsigned grid_for(int64_t threads) {
  int64_t b = (threads + 255) / 256;
  if (b > 65536) b = 65536;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_quantize_weight(const float *w, int64_t K, int64_t N, int64_t ld_w,
                                  const SegTable &ks, const NSegTable &ns, bool per_column,
                                  int8_t *w_packed, float *w_scale, bool w4, hipStream_t s) {
  const int64_t nscale = (int64_t)ks.n * N;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(nscale)), dim3(256), 0, s, w_scale, nscale);
  ColMaxArgs c{w, K, N, ld_w, w_scale, ks};
  hipLaunchKernelGGL(colmax_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)((K + kRowChunk - 1) / kRowChunk)),
                     dim3(256), 0, s, c);
  if (!per_column) {
    GroupMaxArgs g{w_scale, N, ns};
    hipLaunchKernelGGL(groupmax_kernel, dim3((unsigned)ns.n, (unsigned)ks.n), dim3(256), 0, s, g);
  }
  PackArgs p{w, K, N, ld_w, w_scale, w_packed, ks};
  if (w4)
    hipLaunchKernelGGL(pack_kernel<true>, dim3(grid_for((K / 64) * (N / 16) * 64)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3(grid_for((K / 64) * (N / 16) * 64)), dim3(256), 0, s, p);
  hipLaunchKernelGGL(finalize_kernel, dim3(grid_for(nscale)), dim3(256), 0, s, w_scale, nscale,
                     w4 ? 7.0 : 127.0);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                                int64_t ld_w, bool w4, hipStream_t s) {
  if (w4)
    hipLaunchKernelGGL(unpack_kernel<true>, dim3(grid_for((K / 64) * (N / 16) * 64)), dim3(256), 0,
                       s, w_packed, K, N, w_kn, ld_w);
  else
    hipLaunchKernelGGL(unpack_kernel<false>, dim3(grid_for((K / 64) * (N / 16) * 64)), dim3(256), 0,
                       s, w_packed, K, N, w_kn, ld_w);
  return hipGetLastError();
}

hipError_t launch_widen_w4(const int8_t *w4, int64_t K, int64_t N, int8_t *w8, hipStream_t s) {
  const int64_t lanes = (K / 64) * (N / 16) * 64;
  hipLaunchKernelGGL(widen_w4_kernel, dim3(grid_for(lanes)), dim3(256), 0, s, w4, lanes, w8);
  return hipGetLastError();
}

}  // namespace sq
