// probes.hip -- ceilings of this GPU, measured next to the layer's kernels:
// the int8 matrix-core rate with nothing else in the loop, the shader clock
// while it runs, and the HBM read rate of a plain streaming kernel.  The
// benchmark reports the layer's rates against these as well as against the
// published peaks.  Built as its own library (libsegquant_probe.so); the
// layer's library does not contain or need it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kChains = 12;  // independent accumulators per wave, as in the GEMM tile loop

// Every wave issues iters * kChains int8 32x32x32 matrix-core instructions
// on independent accumulators, then stores one checksum per lane (so the
// work cannot be dropped) and, from lane 0, its shader-clock and
// constant-clock spans.
__global__ __launch_bounds__(256) void mfma_i8_kernel(int64_t iters, int32_t *sink,
                                                      uint64_t *spans) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane + 1, lane + 2, lane + 3};
  const v4i b = {3 * lane, lane ^ 5, 7, lane >> 1};
  v16i acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16i{};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[c][r];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  sink[gw * 64 + lane] = s;
  if (lane == 0) {
    spans[2 * gw] = c1 - c0;
    spans[2 * gw + 1] = w1 - w0;
  }
}

// The same loop on operands that change from one instruction to the next:
// each lane loads eight A and eight B fragments of random bytes (256 bytes,
// at src + (wave * 64 + lane) * 256) and every instruction of an iteration
// pairs a different A with a different B, the pairing shifting between
// even and odd iterations.  Constant operands leave the matrix core's data
// path idle; the layer's operands do not, and the power they draw sets the
// clock the layer gets.
constexpr int kDataFrags = 8;
__global__ __launch_bounds__(256) void mfma_i8_data_kernel(int64_t iters, const v4i *src,
                                                           int32_t *sink, uint64_t *spans) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const v4i *mine = src + (gw * 64 + lane) * (2 * kDataFrags);
  v4i a[kDataFrags], b[kDataFrags];
#pragma unroll
  for (int f = 0; f < kDataFrags; ++f) {
    a[f] = mine[f];
    b[f] = mine[kDataFrags + f];
  }
  v16i acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = v16i{};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t w0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t i = 0; i < iters; i += 2) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c % kDataFrags], b[(c + 3) % kDataFrags],
                                                     acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(c + 5) % kDataFrags],
                                                     b[(c + 1) % kDataFrags], acc[c], 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[c][r];
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t w1 = __builtin_amdgcn_s_memrealtime();
  sink[gw * 64 + lane] = s;
  if (lane == 0) {
    spans[2 * gw] = c1 - c0;
    spans[2 * gw + 1] = w1 - w0;
  }
}

// Grid-stride read of n16 16-byte vectors; one XOR checksum per thread.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4u *src, int64_t n16,
                                                          uint32_t *sink) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  v4u acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride], x3 = src[i + 3 * stride];
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// Matrix-core probe: `waves_per_block` * 64 threads per block (1..4 waves),
// `blocks` blocks.  sink: device int32 [blocks * waves_per_block * 64];
// spans: device uint64 [blocks * waves_per_block][2] (shader clocks, then
// constant-clock ticks -- see sqprobe_wall_clock_khz -- over each wave's
// loop).  Returns 0, or -1 on a
// bad argument, -6 on a launch failure.
int sqprobe_mfma_i8(int64_t iters, int32_t blocks, int32_t waves_per_block, int32_t *sink,
                    uint64_t *spans, void *stream) {
  if (iters < 1 || blocks < 1 || waves_per_block < 1 || waves_per_block > 4 || !sink || !spans)
    return -1;
  hipLaunchKernelGGL(mfma_i8_kernel, dim3((unsigned)blocks), dim3(64u * waves_per_block), 0,
                     (hipStream_t)stream, iters, sink, spans);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The matrix-core probe on changing operands (see mfma_i8_data_kernel):
// `iters` even; src: device bytes [blocks * waves_per_block * 64 * 256],
// 16-byte aligned, random; sink and spans as for sqprobe_mfma_i8.
int sqprobe_mfma_i8_data(int64_t iters, int32_t blocks, int32_t waves_per_block, const void *src,
                         int32_t *sink, uint64_t *spans, void *stream) {
  if (iters < 2 || iters % 2 || blocks < 1 || waves_per_block < 1 || waves_per_block > 4 ||
      !src || (reinterpret_cast<uintptr_t>(src) & 15u) || !sink || !spans)
    return -1;
  hipLaunchKernelGGL(mfma_i8_data_kernel, dim3((unsigned)blocks), dim3(64u * waves_per_block), 0,
                     (hipStream_t)stream, iters, static_cast<const v4i *>(src), sink, spans);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Bytes of random operand data sqprobe_mfma_i8_data reads per wave.
int64_t sqprobe_mfma_data_bytes_per_wave(void) { return 64LL * 2 * kDataFrags * 16; }

// Streaming-read probe over `bytes` (a multiple of 16, 16-byte aligned src).
// sink: device uint32 [blocks * 256].
int sqprobe_stream_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *sink,
                        void *stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || blocks < 1 ||
      (reinterpret_cast<uintptr_t>(src) & 15u))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, static_cast<const v4u *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Rate of the constant clock that s_memrealtime counts, in kHz (current
// device), or -6 when the runtime cannot say.
int sqprobe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -6;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -6;
  return khz;
}

// Number of matrix-core instructions one wave of the probe issues per
// iteration, and the int8 ops of one instruction (32*32*32 multiply-adds).
int sqprobe_mfma_chains(void) { return kChains; }
int64_t sqprobe_ops_per_mfma(void) { return 2LL * 32 * 32 * 32; }

}  // extern "C"
