// noalloc.hip -- segquant_gemm_w8a8_seg_noalloc: the layer call of
// segquant_gemm_w8a8_seg without a caller workspace and without any device
// allocation, for callers that cannot allocate (code under stream capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The memory the ordinary call takes a workspace for -- the int8 codes of a
// quantise-first call, the int8 widening of 4-bit weight tiles -- comes from
// `scratch`, a file-scope device array of SEGQ_NOALLOC_SCRATCH_BYTES that
// every GPU the library runs on holds until the process ends.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current); host code passes that address, never the array's name, to the
// kernels.  Every call on one GPU shares that GPU's array, so calls that
// overlap on one GPU race (order them on one stream).  Nothing in it has to
// start at zero: each use writes every byte it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/segquant.h"
#include "sq_api.hpp"

namespace {

__device__ __align__(256) uint8_t scratch[SEGQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The device address of `scratch` on the device that runs `stream`.
int scratch_for(hipStream_t stream, void **out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return sq::api_hip_status(e, "hipGetDevice");
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return sq::api_hip_status(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return sq::api_fail(SEGQ_ERR_UNSUPPORTED, "device %d: the no-allocation call serves devices "
                        "0..%d", dev, kMaxDevices - 1);
  std::call_once(g_once[dev], [dev, cur] {
    hipError_t s = hipSuccess;
    if (dev != cur) s = hipSetDevice(dev);
    void *p = nullptr;
    if (s == hipSuccess) s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (s == hipSuccess) s = r;
    }
    g_status[dev] = s;
    g_ptr[dev] = s == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess)
    return sq::api_hip_status(g_status[dev], "hipGetSymbolAddress(scratch)");
  *out = g_ptr[dev];
  return SEGQ_OK;
}

}  // namespace

extern "C" int segquant_gemm_w8a8_seg_noalloc(int64_t M, int64_t N, int64_t K,
                                              const uint16_t *x_bf16, int64_t ld_x,
                                              const int8_t *xq, int64_t ld_q, int32_t q_layout,
                                              const int8_t *w_packed, const float *w_scale,
                                              int32_t n_kseg, const int32_t *kseg_offset,
                                              const int32_t *kseg_width, const float *act_scales,
                                              uint16_t *y_bf16, int64_t ld_y, int32_t *acc_debug,
                                              uint32_t flags, void *stream) {
  sq::GemmCall c{M,          N,          K,      x_bf16, ld_x,      xq,       ld_q,
                 q_layout,   w_packed,   w_scale, n_kseg, kseg_offset, kseg_width, act_scales,
                 y_bf16,     ld_y,       acc_debug, flags, stream};
  sq::SegTable ks{};
  int st = sq::gemm_validate(c, ks);  // every check before any HIP call
  if (st) return st;
  size_t need = sq::gemm_workspace_need(c, ks, c.flags);
  if (need > (size_t)SEGQ_NOALLOC_SCRATCH_BYTES) {
    // The quantise-first codes are optional (the fused launch computes the
    // same codes and products); the widened 4-bit weight is not.
    const size_t required = sq::gemm_workspace_need(c, ks, c.flags | SEGQ_GEMM_FUSED_QUANT);
    if (required > (size_t)SEGQ_NOALLOC_SCRATCH_BYTES)
      return sq::api_fail(SEGQ_ERR_UNSUPPORTED,
                          "this call needs %zu bytes of scratch (4-bit weights are widened to "
                          "K*N int8 bytes); the no-allocation call holds %zu",
                          required, (size_t)SEGQ_NOALLOC_SCRATCH_BYTES);
    c.flags |= SEGQ_GEMM_FUSED_QUANT;
    need = required;
  }
  void *ws = nullptr;
  if (need > 0 && M > 0) {
    if ((st = scratch_for((hipStream_t)stream, &ws))) return st;
  }
  return sq::gemm_enqueue(c, ks, ws, ws ? (size_t)SEGQ_NOALLOC_SCRATCH_BYTES : 0);
}
