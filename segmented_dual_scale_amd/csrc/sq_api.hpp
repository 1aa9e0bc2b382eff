// sq_api.hpp -- internal interface between the C ABI front end (api.cpp) and
// the other entry points built on its GEMM call (noalloc.hip): argument
// validation and the enqueue step of segquant_gemm_w8a8_seg, kept apart so a
// caller can validate before it makes any HIP call of its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sq_launch.hpp"

namespace sq {

// The arguments of segquant_gemm_w8a8_seg, less the workspace.
struct GemmCall {
  int64_t M, N, K;
  const uint16_t *x;
  int64_t ld_x;
  const int8_t *xq;
  int64_t ld_q;
  int32_t q_layout;
  const int8_t *w_packed;
  const float *w_scale;
  int32_t n_kseg;
  const int32_t *kseg_offset;
  const int32_t *kseg_width;
  const float *act;
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc;
  uint32_t flags;
  void *stream;
};

// Every check of the call; no HIP call.  Fills the K-segment table.
int gemm_validate(const GemmCall &c, SegTable &ks);
// Workspace bytes the call would use with these flags (validated call).
size_t gemm_workspace_need(const GemmCall &c, const SegTable &ks, uint32_t flags);
// Enqueue a validated call; workspace may be null.
int gemm_enqueue(const GemmCall &c, const SegTable &ks, void *workspace, size_t workspace_bytes);
// Set the thread's error text and return status.
int api_fail(int status, const char *fmt, ...);
// SEGQ_OK, or SEGQ_ERR_HIP with the runtime's text.
int api_hip_status(hipError_t e, const char *what);

}  // namespace sq
