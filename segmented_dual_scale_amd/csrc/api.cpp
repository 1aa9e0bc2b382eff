// api.cpp -- the C ABI of libsegquant (declared in include/segquant.h):
// argument validation, segment tables, kernel choice and launch.
//
// Every check runs before the first HIP call, so an invalid call enqueues
// nothing, touches no buffer and behaves the same on a machine without a
// GPU.  Errors are returned as status codes with a thread-local detail text;
// nothing is thrown across the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/segquant.h"
#include "sq_api.hpp"
#include "sq_launch.hpp"

namespace {

thread_local std::string g_err;

int vfail(int status, const char *fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_err = buf;
  return status;
}

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(status, fmt, ap);
  va_end(ap);
  return r;
}

int ok() {
  g_err.clear();
  return SEGQ_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kI32Max = 0x7fffffff;

// K-segment list -> kernel table.  require64: every boundary but the end of
// K is a multiple of 64; max_width: 0 for no limit.
int read_kseg(int32_t n, const int32_t *off, const int32_t *wid, int64_t K, int64_t max_width,
              sq::SegTable &t) {
  if (n < 1) return fail(SEGQ_ERR_SEGMENTS, "K-segment count %d < 1", n);
  if (n > SEGQ_MAX_KSEG)
    return fail(SEGQ_ERR_UNSUPPORTED, "K-segment count %d > %d", n, SEGQ_MAX_KSEG);
  if (!off || !wid) return fail(SEGQ_ERR_NULL, "K-segment offset/width array is NULL");
  int64_t at = 0;
  t.n = n;
  for (int32_t i = 0; i < n; ++i) {
    if (off[i] != at)
      return fail(SEGQ_ERR_SEGMENTS, "K-segment %d starts at %d, expected %lld", i, off[i],
                  (long long)at);
    if (wid[i] <= 0) return fail(SEGQ_ERR_SEGMENTS, "K-segment %d has width %d", i, wid[i]);
    if (max_width > 0 && wid[i] > max_width)
      return fail(SEGQ_ERR_UNSUPPORTED, "K-segment %d width %d exceeds %lld (int32 bound)", i,
                  wid[i], (long long)max_width);
    at += wid[i];
    if (at < K && at % 64 != 0)
      return fail(SEGQ_ERR_ALIGN, "K-segment boundary %lld is not a multiple of 64",
                  (long long)at);
    t.off[i] = off[i];
    t.end[i] = (int32_t)at;
  }
  if (at != K)
    return fail(SEGQ_ERR_SEGMENTS, "K-segments cover %lld columns, K is %lld", (long long)at,
                (long long)K);
  return SEGQ_OK;
}

int read_nseg(int32_t n, const int32_t *off, const int32_t *wid, int64_t N, sq::NSegTable &t) {
  if (n < 1) return fail(SEGQ_ERR_SEGMENTS, "N-segment count %d < 1", n);
  if (n > sq::kMaxNSeg) return fail(SEGQ_ERR_UNSUPPORTED, "N-segment count %d > %d", n, sq::kMaxNSeg);
  if (!off || !wid) return fail(SEGQ_ERR_NULL, "N-segment offset/width array is NULL");
  int64_t at = 0;
  t.n = n;
  for (int32_t i = 0; i < n; ++i) {
    if (off[i] != at)
      return fail(SEGQ_ERR_SEGMENTS, "N-segment %d starts at %d, expected %lld", i, off[i],
                  (long long)at);
    if (wid[i] <= 0) return fail(SEGQ_ERR_SEGMENTS, "N-segment %d has width %d", i, wid[i]);
    at += wid[i];
    t.off[i] = off[i];
    t.end[i] = (int32_t)at;
  }
  if (at != N)
    return fail(SEGQ_ERR_SEGMENTS, "N-segments cover %lld columns, N is %lld", (long long)at,
                (long long)N);
  return SEGQ_OK;
}

int check_x(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x) {
  if (M < 0 || K < 1 || M > kI32Max || K > kI32Max)
    return fail(SEGQ_ERR_SHAPE, "bad shape M=%lld K=%lld", (long long)M, (long long)K);
  if (ld_x < K) return fail(SEGQ_ERR_SHAPE, "ld_x %lld < K %lld", (long long)ld_x, (long long)K);
  if (M > 0 && !x) return fail(SEGQ_ERR_NULL, "x_bf16 is NULL");
  if (ld_x % 8 != 0) return fail(SEGQ_ERR_ALIGN, "ld_x %lld is not a multiple of 8", (long long)ld_x);
  if (x && !aligned16(x)) return fail(SEGQ_ERR_ALIGN, "x_bf16 is not 16-byte aligned");
  return SEGQ_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(SEGQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace sq {

int api_fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(status, fmt, ap);
  va_end(ap);
  return r;
}

int api_hip_status(hipError_t e, const char *what) { return hip_status(e, what); }

static int gemm_check_shape(int64_t M, int64_t N, int64_t K, uint32_t flags);

int gemm_validate(const GemmCall &c, SegTable &ks) {
  int st = gemm_check_shape(c.M, c.N, c.K, c.flags);
  if (st) return st;
  if (c.M > 0) {
    if ((c.x != nullptr) == (c.xq != nullptr))
      return fail(SEGQ_ERR_NULL, "exactly one of x_bf16 and xq must be given");
    if (c.x) {
      if ((st = check_x(c.x, c.M, c.K, c.ld_x))) return st;
    } else {
      if (c.q_layout != SEGQ_Q_SIGNED && c.q_layout != SEGQ_Q_PLANES)
        return fail(SEGQ_ERR_SHAPE, "unknown q_layout %d", c.q_layout);
      if (c.q_layout == SEGQ_Q_PLANES && (c.flags & SEGQ_GEMM_SINGLE_SCALE))
        return fail(SEGQ_ERR_UNSUPPORTED, "the single-scale product takes bf16 or signed-code input");
      if (c.ld_q < c.K)
        return fail(SEGQ_ERR_SHAPE, "ld_q %lld < K %lld", (long long)c.ld_q, (long long)c.K);
      if (c.ld_q % 16 != 0)
        return fail(SEGQ_ERR_ALIGN, "ld_q %lld is not a multiple of 16", (long long)c.ld_q);
      if (!aligned16(c.xq)) return fail(SEGQ_ERR_ALIGN, "xq is not 16-byte aligned");
    }
    if (!c.w_packed || !c.w_scale || !c.act || !c.y)
      return fail(SEGQ_ERR_NULL, "w_packed, w_scale, act_scales or y_bf16 is NULL");
    if (!aligned16(c.w_packed)) return fail(SEGQ_ERR_ALIGN, "w_packed is not 16-byte aligned");
    if (c.ld_y < c.N)
      return fail(SEGQ_ERR_SHAPE, "ld_y %lld < N %lld", (long long)c.ld_y, (long long)c.N);
    if ((reinterpret_cast<uintptr_t>(c.y) & 1u) ||
        (c.acc && (reinterpret_cast<uintptr_t>(c.acc) & 3u)))
      return fail(SEGQ_ERR_ALIGN, "y_bf16 or acc_debug is misaligned");
  }
  if ((st = read_kseg(c.n_kseg, c.kseg_offset, c.kseg_width, c.K, SEGQ_MAX_KSEG_WIDTH, ks)))
    return st;
  return ok();
}

static bool quantize_first(int kernel, int64_t M, int64_t N, const sq::SegTable &ks,
                           uint32_t flags);
static size_t w4_widen_bytes(int kernel, int64_t M, int64_t N, int64_t K, const sq::SegTable &ks,
                             uint32_t flags, bool bf16_input);

size_t gemm_workspace_need(const GemmCall &c, const SegTable &ks, uint32_t flags) {
  const int kernel = segquant_gemm_kernel_for(c.M, c.N, c.K, flags);
  return w4_widen_bytes(kernel, c.M, c.N, c.K, ks, flags, c.x != nullptr) +
         (c.x && quantize_first(kernel, c.M, c.N, ks, flags) ? (size_t)(c.M * c.K) : 0);
}

int gemm_enqueue(const GemmCall &c, const SegTable &ks, void *workspace, size_t workspace_bytes) {
  if (c.M == 0) return ok();
  const int64_t M = c.M, N = c.N, K = c.K;
  const uint32_t flags = c.flags;
  sq::GemmProblem p{};
  p.M = M; p.N = N; p.K = K;
  p.x = c.x; p.ld_x = c.ld_x;
  p.xq = c.xq; p.ld_q = c.ld_q; p.q_layout = c.q_layout;
  p.w_packed = c.w_packed; p.w_scale = c.w_scale; p.act = c.act;
  p.ks = ks;
  p.y = c.y; p.ld_y = c.ld_y; p.acc_debug = c.acc;
  p.single_scale = (flags & SEGQ_GEMM_SINGLE_SCALE) != 0;
  hipStream_t stream = (hipStream_t)c.stream;
  const int kernel = segquant_gemm_kernel_for(M, N, K, flags);
  // 4-bit weights: the streaming small-M kernel reads them as they are;
  // every other path first widens them to int8 tiles in the workspace
  const size_t widen = w4_widen_bytes(kernel, M, N, K, ks, flags, c.x != nullptr);
  if (widen && (!workspace || workspace_bytes < widen))
    return fail(SEGQ_ERR_UNSUPPORTED,
                "4-bit weights on this shape need a workspace of at least %zu bytes "
                "(segquant_gemm_workspace_bytes)", widen);
  p.w4 = (flags & SEGQ_GEMM_W4) && !widen;
  if (widen) {
    int8_t *w8 = static_cast<int8_t *>(workspace);
    hipError_t e = sq::launch_widen_w4(c.w_packed, K, N, w8, stream);
    if (e != hipSuccess) return hip_status(e, "widen launch");
    p.w_packed = w8;
  }
  uint8_t *ws_rest = workspace ? static_cast<uint8_t *>(workspace) + widen : nullptr;
  const size_t ws_rest_bytes = workspace ? workspace_bytes - widen : 0;
  if (c.x && ws_rest && quantize_first(kernel, M, N, ks, flags) &&
      ws_rest_bytes >= (size_t)(M * K)) {
    // quantise once into the workspace, then the GEMM from the signed codes
    int8_t *codes = reinterpret_cast<int8_t *>(ws_rest);
    hipError_t e = sq::launch_quantize(c.x, M, K, c.ld_x, ks, c.act, codes, K, SEGQ_Q_SIGNED,
                                       p.single_scale, stream);
    if (e != hipSuccess) return hip_status(e, "quantize launch");
    p.x = nullptr;
    p.ld_x = 0;
    p.xq = codes;
    p.ld_q = K;
    p.q_layout = SEGQ_Q_SIGNED;
  }
  hipError_t e = kernel == SEGQ_KERNEL_SMALLM ? sq::launch_gemm_smallm(p, stream)
                                              : sq::launch_gemm_tile(p, stream);
  return hip_status(e, "gemm launch");
}

}  // namespace sq

extern "C" {

const char *segquant_status_string(int status) {
  switch (status) {
    case SEGQ_OK: return "ok";
    case SEGQ_ERR_NULL: return "null pointer";
    case SEGQ_ERR_SHAPE: return "invalid shape";
    case SEGQ_ERR_SEGMENTS: return "invalid segment list";
    case SEGQ_ERR_ALIGN: return "misaligned size, boundary or pointer";
    case SEGQ_ERR_UNSUPPORTED: return "unsupported (beyond library limits)";
    case SEGQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *segquant_last_error(void) { return g_err.c_str(); }

int segquant_version(void) { return 100; }

size_t segquant_weight_packed_bytes_w4(int64_t K, int64_t N) {
  return segquant_weight_packed_bytes(K, N) / 2;
}

size_t segquant_weight_packed_bytes(int64_t K, int64_t N) {
  if (K < 64 || N < 16 || K % 64 || N % 16 || K > kI32Max || N > kI32Max) return 0;
  return (size_t)K * (size_t)N;
}

static int calibrate(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x, int32_t n_kseg,
                     const int32_t *kseg_offset, const int32_t *kseg_width, float *act_scales,
                     bool single, void *stream) {
  int st = check_x(x_bf16, M, K, ld_x);
  if (st) return st;
  if (!act_scales) return fail(SEGQ_ERR_NULL, "act_scales is NULL");
  sq::SegTable ks{};
  if ((st = read_kseg(n_kseg, kseg_offset, kseg_width, K, 0, ks))) return st;
  return hip_status(
      sq::launch_calibrate(x_bf16, M, K, ld_x, ks, act_scales, single, (hipStream_t)stream),
      "calibrate launch");
}

int segquant_calibrate_amax(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                            int32_t n_kseg, const int32_t *kseg_offset,
                            const int32_t *kseg_width, float *act_scales, void *stream) {
  return calibrate(x_bf16, M, K, ld_x, n_kseg, kseg_offset, kseg_width, act_scales, false, stream);
}

int segquant_calibrate_amax_single(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                   int32_t n_kseg, const int32_t *kseg_offset,
                                   const int32_t *kseg_width, float *act_scales, void *stream) {
  return calibrate(x_bf16, M, K, ld_x, n_kseg, kseg_offset, kseg_width, act_scales, true, stream);
}

int segquant_quantize_dualscale(const uint16_t *x_bf16, int64_t M, int64_t K, int64_t ld_x,
                                int32_t n_kseg, const int32_t *kseg_offset,
                                const int32_t *kseg_width, const float *act_scales,
                                int8_t *q_out, int64_t ld_q, int32_t q_layout, void *stream) {
  int st = check_x(x_bf16, M, K, ld_x);
  if (st) return st;
  if (!act_scales) return fail(SEGQ_ERR_NULL, "act_scales is NULL");
  if (M > 0 && !q_out) return fail(SEGQ_ERR_NULL, "q_out is NULL");
  if (q_layout != SEGQ_Q_SIGNED && q_layout != SEGQ_Q_PLANES)
    return fail(SEGQ_ERR_SHAPE, "unknown q_layout %d", q_layout);
  if (ld_q < K) return fail(SEGQ_ERR_SHAPE, "ld_q %lld < K %lld", (long long)ld_q, (long long)K);
  if (ld_q % 16 != 0) return fail(SEGQ_ERR_ALIGN, "ld_q %lld is not a multiple of 16", (long long)ld_q);
  if (q_out && !aligned16(q_out)) return fail(SEGQ_ERR_ALIGN, "q_out is not 16-byte aligned");
  sq::SegTable ks{};
  if ((st = read_kseg(n_kseg, kseg_offset, kseg_width, K, 0, ks))) return st;
  return hip_status(sq::launch_quantize(x_bf16, M, K, ld_x, ks, act_scales, q_out, ld_q, q_layout,
                                        false, (hipStream_t)stream),
                    "quantize launch");
}

int segquant_activate_quantize(const uint16_t *z_bf16, int64_t M, int64_t K, int64_t ld_z,
                               int32_t act_kind, int32_t n_kseg, const int32_t *kseg_offset,
                               const int32_t *kseg_width, const float *act_scales,
                               int8_t *q_out, int64_t ld_q, int32_t q_layout, uint16_t *x_out,
                               int64_t ld_xo, void *stream) {
  int st = check_x(z_bf16, M, K, ld_z);
  if (st) return st;
  if (act_kind != SEGQ_ACT_SILU && act_kind != SEGQ_ACT_GELU)
    return fail(SEGQ_ERR_SHAPE, "unknown act_kind %d", act_kind);
  if (!q_out && !x_out) return fail(SEGQ_ERR_NULL, "neither q_out nor x_out is given");
  if (q_out) {
    if (!act_scales) return fail(SEGQ_ERR_NULL, "act_scales is NULL");
    if (q_layout != SEGQ_Q_SIGNED && q_layout != SEGQ_Q_PLANES)
      return fail(SEGQ_ERR_SHAPE, "unknown q_layout %d", q_layout);
    if (ld_q < K) return fail(SEGQ_ERR_SHAPE, "ld_q %lld < K %lld", (long long)ld_q, (long long)K);
    if (ld_q % 16 != 0)
      return fail(SEGQ_ERR_ALIGN, "ld_q %lld is not a multiple of 16", (long long)ld_q);
    if (!aligned16(q_out)) return fail(SEGQ_ERR_ALIGN, "q_out is not 16-byte aligned");
  }
  if (x_out) {
    if (ld_xo < K) return fail(SEGQ_ERR_SHAPE, "ld_xo %lld < K %lld", (long long)ld_xo, (long long)K);
    if (ld_xo % 8 != 0 || !aligned16(x_out))
      return fail(SEGQ_ERR_ALIGN, "x_out must be 16-byte aligned with ld_xo a multiple of 8");
  }
  sq::SegTable ks{};
  if ((st = read_kseg(n_kseg, kseg_offset, kseg_width, K, 0, ks))) return st;
  return hip_status(sq::launch_act_quantize(z_bf16, M, K, ld_z, act_kind, ks, act_scales, q_out,
                                            ld_q, q_layout, x_out, ld_xo, (hipStream_t)stream),
                    "activate-quantize launch");
}

static int quantize_weight(const float *w, int64_t K, int64_t N, int64_t ld_w, int32_t n_kseg,
                           const int32_t *kseg_offset, const int32_t *kseg_width, int32_t n_nseg,
                           const int32_t *nseg_offset, const int32_t *nseg_width,
                           int32_t per_column, int8_t *w_packed, float *w_scale, bool w4,
                           void *stream) {
  if (K < 1 || N < 1 || K > kI32Max || N > kI32Max)
    return fail(SEGQ_ERR_SHAPE, "bad shape K=%lld N=%lld", (long long)K, (long long)N);
  if (ld_w < N) return fail(SEGQ_ERR_SHAPE, "ld_w %lld < N %lld", (long long)ld_w, (long long)N);
  if (!w || !w_packed || !w_scale) return fail(SEGQ_ERR_NULL, "w, w_packed or w_scale is NULL");
  if (K % 64 || N % 16)
    return fail(SEGQ_ERR_ALIGN, "weight needs K %% 64 == 0 and N %% 16 == 0 (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (!aligned16(w_packed) || (reinterpret_cast<uintptr_t>(w) & 3u))
    return fail(SEGQ_ERR_ALIGN, "w_packed must be 16-byte and w 4-byte aligned");
  sq::SegTable ks{};
  int st = read_kseg(n_kseg, kseg_offset, kseg_width, K, 0, ks);
  if (st) return st;
  sq::NSegTable ns{};
  ns.n = 1;
  ns.off[0] = 0;
  ns.end[0] = (int32_t)N;
  if (!per_column && (st = read_nseg(n_nseg, nseg_offset, nseg_width, N, ns))) return st;
  return hip_status(sq::launch_quantize_weight(w, K, N, ld_w, ks, ns, per_column != 0, w_packed,
                                               w_scale, w4, (hipStream_t)stream),
                    "quantize_weight launch");
}

int segquant_quantize_weight(const float *w, int64_t K, int64_t N, int64_t ld_w,
                             int32_t n_kseg, const int32_t *kseg_offset,
                             const int32_t *kseg_width, int32_t n_nseg,
                             const int32_t *nseg_offset, const int32_t *nseg_width,
                             int32_t per_column, int8_t *w_packed, float *w_scale,
                             void *stream) {
  return quantize_weight(w, K, N, ld_w, n_kseg, kseg_offset, kseg_width, n_nseg, nseg_offset,
                         nseg_width, per_column, w_packed, w_scale, false, stream);
}

int segquant_quantize_weight_w4(const float *w, int64_t K, int64_t N, int64_t ld_w,
                                int32_t n_kseg, const int32_t *kseg_offset,
                                const int32_t *kseg_width, int32_t n_nseg,
                                const int32_t *nseg_offset, const int32_t *nseg_width,
                                int32_t per_column, int8_t *w_packed, float *w_scale,
                                void *stream) {
  return quantize_weight(w, K, N, ld_w, n_kseg, kseg_offset, kseg_width, n_nseg, nseg_offset,
                         nseg_width, per_column, w_packed, w_scale, true, stream);
}

static int unpack_weight(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                         int64_t ld_w, bool w4, void *stream) {
  if (segquant_weight_packed_bytes(K, N) == 0)
    return fail(SEGQ_ERR_ALIGN, "weight needs K %% 64 == 0 and N %% 16 == 0 (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (ld_w < N) return fail(SEGQ_ERR_SHAPE, "ld_w %lld < N %lld", (long long)ld_w, (long long)N);
  if (!w_packed || !w_kn) return fail(SEGQ_ERR_NULL, "w_packed or w_kn is NULL");
  if (!aligned16(w_packed)) return fail(SEGQ_ERR_ALIGN, "w_packed is not 16-byte aligned");
  return hip_status(sq::launch_unpack_weight(w_packed, K, N, w_kn, ld_w, w4, (hipStream_t)stream),
                    "unpack launch");
}

int segquant_unpack_weight(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                           int64_t ld_w, void *stream) {
  return unpack_weight(w_packed, K, N, w_kn, ld_w, false, stream);
}

int segquant_unpack_weight_w4(const int8_t *w_packed, int64_t K, int64_t N, int8_t *w_kn,
                              int64_t ld_w, void *stream) {
  return unpack_weight(w_packed, K, N, w_kn, ld_w, true, stream);
}

}  // extern "C"

namespace sq {
static int gemm_check_shape(int64_t M, int64_t N, int64_t K, uint32_t flags) {
  if (M < 0 || N < 1 || K < 1 || M > kI32Max || N > kI32Max || K > kI32Max)
    return fail(SEGQ_ERR_SHAPE, "bad shape M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                (long long)K);
  if (K % 64 || N % 16)
    return fail(SEGQ_ERR_ALIGN, "GEMM needs K %% 64 == 0 and N %% 16 == 0 (K=%lld N=%lld)",
                (long long)K, (long long)N);
  if (flags & ~(SEGQ_GEMM_FORCE_TILE | SEGQ_GEMM_FORCE_SMALLM | SEGQ_GEMM_FUSED_QUANT |
                SEGQ_GEMM_SINGLE_SCALE | SEGQ_GEMM_W4))
    return fail(SEGQ_ERR_SHAPE, "unknown flags 0x%x", flags);
  if ((flags & SEGQ_GEMM_FORCE_TILE) && (flags & SEGQ_GEMM_FORCE_SMALLM))
    return fail(SEGQ_ERR_SHAPE, "both kernels forced");
  if ((flags & SEGQ_GEMM_FORCE_SMALLM) && M > sq::kSmallMMax)
    return fail(SEGQ_ERR_UNSUPPORTED, "the small-M kernel takes M <= %d (M=%lld)", sq::kSmallMMax,
                (long long)M);
  return SEGQ_OK;
}
}  // namespace sq

extern "C" {

int segquant_gemm_kernel_for(int64_t M, int64_t N, int64_t K, uint32_t flags) {
  int st = sq::gemm_check_shape(M, N, K, flags);
  if (st) return st;
  if (flags & SEGQ_GEMM_FORCE_TILE) return SEGQ_KERNEL_TILE;
  if (flags & SEGQ_GEMM_FORCE_SMALLM) return SEGQ_KERNEL_SMALLM;
  return M <= sq::kSmallMMax ? SEGQ_KERNEL_SMALLM : SEGQ_KERNEL_TILE;
}

int segquant_gemm_halves(const float *act_scales_host, int32_t n_kseg) {
  if (!act_scales_host) return fail(SEGQ_ERR_NULL, "act_scales_host is NULL");
  if (n_kseg < 1 || n_kseg > SEGQ_MAX_KSEG)
    return fail(SEGQ_ERR_SEGMENTS, "K-segment count %d outside [1, %d]", n_kseg, SEGQ_MAX_KSEG);
  for (int32_t i = 0; i < n_kseg; ++i) {
    const float s_neg = act_scales_host[n_kseg + i], inv_neg = act_scales_host[3 * n_kseg + i];
    if (s_neg != 0.0f || inv_neg != 0.0f) return 0;  // the - half carries values: both halves
  }
  return (int)SEGQ_GEMM_SINGLE_SCALE;
}

}  // extern "C"

namespace sq {
static bool quantize_first(int kernel, int64_t M, int64_t N, const sq::SegTable &ks,
                           uint32_t flags) {
  return kernel == SEGQ_KERNEL_TILE && !(flags & SEGQ_GEMM_FUSED_QUANT) &&
         sq::tile_quantize_first(M, N, ks);
}

// Bytes of the widened int8 weight a W4 call needs in its workspace (0 when
// the small-M streaming kernel reads the 4-bit tiles itself).
static size_t w4_widen_bytes(int kernel, int64_t M, int64_t N, int64_t K, const sq::SegTable &ks,
                             uint32_t flags, bool bf16_input) {
  if (!(flags & SEGQ_GEMM_W4)) return 0;
  if (kernel == SEGQ_KERNEL_SMALLM && sq::smallm_reads_w4(M, K, ks.n, bf16_input)) return 0;
  return (size_t)K * (size_t)N;
}
}  // namespace sq

extern "C" {

size_t segquant_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t n_kseg,
                                     const int32_t *kseg_offset, const int32_t *kseg_width,
                                     uint32_t flags) {
  if (sq::gemm_check_shape(M, N, K, flags)) return 0;
  sq::SegTable ks{};
  if (read_kseg(n_kseg, kseg_offset, kseg_width, K, SEGQ_MAX_KSEG_WIDTH, ks)) return 0;
  ok();
  const int kernel = segquant_gemm_kernel_for(M, N, K, flags);
  return sq::w4_widen_bytes(kernel, M, N, K, ks, flags, true) +
         (sq::quantize_first(kernel, M, N, ks, flags) ? (size_t)(M * K) : 0);
}

int segquant_gemm_w8a8_seg(int64_t M, int64_t N, int64_t K,
                           const uint16_t *x_bf16, int64_t ld_x,
                           const int8_t *xq, int64_t ld_q, int32_t q_layout,
                           const int8_t *w_packed, const float *w_scale,
                           int32_t n_kseg, const int32_t *kseg_offset,
                           const int32_t *kseg_width, const float *act_scales,
                           uint16_t *y_bf16, int64_t ld_y, int32_t *acc_debug,
                           void *workspace, size_t workspace_bytes,
                           uint32_t flags, void *stream) {
  const sq::GemmCall c{M,       N,          K,        x_bf16,      ld_x,        xq,
                       ld_q,    q_layout,   w_packed, w_scale,     n_kseg,      kseg_offset,
                       kseg_width, act_scales, y_bf16, ld_y,     acc_debug,   flags,
                       stream};
  if (workspace && !aligned16(workspace))
    return fail(SEGQ_ERR_ALIGN, "workspace is not 16-byte aligned");
  sq::SegTable ks{};
  int st = sq::gemm_validate(c, ks);
  if (st) return st;
  return sq::gemm_enqueue(c, ks, workspace, workspace ? workspace_bytes : 0);
}

}  // extern "C"
