// sq_launch.hpp -- host-side launch interface between the C-ABI front end
// (api.cpp) and the kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

constexpr int kMaxKSeg = 128;
constexpr int kMaxNSeg = 128;

// A segmented dimension in the form the kernels read from their arguments.
struct SegTable {
  int32_t n;
  int32_t off[kMaxKSeg];
  int32_t end[kMaxKSeg];  // exclusive
};

struct NSegTable {
  int32_t n;
  int32_t off[kMaxNSeg];
  int32_t end[kMaxNSeg];
};

// single: one symmetric scale per segment, written into both halves
hipError_t launch_calibrate(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                            const SegTable &ks, float *act, bool single, hipStream_t s);

// single: both signs quantised with the + half's inverse
hipError_t launch_quantize(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                           const SegTable &ks, const float *act, int8_t *q, int64_t ld_q,
                           int32_t layout, bool single, hipStream_t s);

// act: 1 SiLU, 2 GELU.  q (codes, with scales) and x_out (bf16 activation)
// are each optional; at least one is given.
hipError_t launch_act_quantize(const uint16_t *z, int64_t M, int64_t K, int64_t ld_z, int32_t act,
                               const SegTable &ks, const float *scales, int8_t *q, int64_t ld_q,
                               int32_t layout, uint16_t *x_out, int64_t ld_xo, hipStream_t s);

// w4: 4-bit codes in the nibble layout (K*N/2 bytes) instead of int8
hipError_t launch_quantize_weight(const float *w, int64_t K, int64_t N, int64_t ld_w,
                                  const SegTable &ks, const NSegTable &ns, bool per_column,
                                  int8_t *w_packed, float *w_scale, bool w4, hipStream_t s);

hipError_t launch_unpack_weight(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                                int64_t ld_w, bool w4, hipStream_t s);

// 4-bit packed tiles -> int8 packed tiles (K*N bytes)
hipError_t launch_widen_w4(const int8_t *w4, int64_t K, int64_t N, int8_t *w8, hipStream_t s);

struct GemmProblem {
  int64_t M, N, K;
  const uint16_t *x;
  int64_t ld_x;
  const int8_t *xq;
  int64_t ld_q;
  int32_t q_layout;
  const int8_t *w_packed;
  const float *w_scale;
  const float *act;
  SegTable ks;
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc_debug;
  bool single_scale;  // one product on the signed code, + half's scales only
  bool w4;            // w_packed holds 4-bit codes (small-M streaming kernel only)
};

hipError_t launch_gemm_tile(const GemmProblem &p, hipStream_t s);
hipError_t launch_gemm_smallm(const GemmProblem &p, hipStream_t s);
// the large-M kernel with both operands staged through LDS
hipError_t launch_gemm_lds(const GemmProblem &p, hipStream_t s);

constexpr int kSmallMMax = 16;

// Whether the streaming small-M kernel takes this shape (and so reads
// 4-bit weight tiles directly).
bool smallm_reads_w4(int64_t M, int64_t K, int n_kseg, bool bf16_input);

// Output columns per workgroup of the tile kernel for these K-segments.
int tile_columns(const SegTable &ks);
// Whether the tile kernel should run from int8 codes quantised beforehand
// (one extra launch) rather than quantise bf16 input itself.
bool tile_quantize_first(int64_t M, int64_t N, const SegTable &ks);

}  // namespace sq
