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
// Each wave owns one 16-column n-tile and walks all of K.  The packed weight
// keeps an n-tile's K as consecutive 1 KiB tiles, so a wave's weight stream
// is one contiguous range, one 16-byte load per lane per tile -- the
// matrix-core B operand as loaded.  Rows of the 16-row A operand at or beyond
// M are zero; both halves run on the int8 16x16x64 matrix cores against the
// same B registers (the padding rows cost nothing: the kernel is bound by
// HBM).
//
// Two kernels:
//   gemm_smallm_kernel          K <= 2048 and X small enough to stage in
//                               registers (the AdaNorm shapes): every load
//                               of the call is issued up front: the first
//                               two weight tiles, then the small ones, so
//                               the tables and X never queue behind the
//                               rest of the weight stream; then quantise
//                               into LDS, fetch every A fragment, and run
//                               the matrix-core chain as the weight tiles
//                               arrive.
//   gemm_smallm_chunked_kernel  any other small-M shape: K in chunks that fit
//                               LDS, a ring of weight tiles kept ahead.
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
  int32_t single;  // single scale: the + half's scales for both signs, one dumped product
  int32_t seg_end_tile[kMaxKSeg];
};

// QL: activation input, -1 bf16 (quantised here), 0 signed codes, 1 planes.
// ONE: all of K is one chunk that fits the weight ring (no refills, no
// chunk loop: straight-line code with an exact count of loads in flight).
template <int WPG, int QL, bool ONE, bool DEBUG>
__global__ __launch_bounds__(64 * WPG) void gemm_smallm_chunked_kernel(SmallArgs a) {
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
  const float *s_pos = a.act, *s_neg = a.act + (a.single ? 0 : nS);

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
        const float ip = a.act[2 * nS + i], in = a.act[(a.single ? 2 : 3) * nS + i];
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
                  if (a.single) {
                    a.acc[o] = accp[r] + accn[r];
                  } else {
                    a.acc[o] = accp[r];
                    a.acc[(int64_t)nS * a.M * a.N + o] = accn[r];
                  }
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


// ---------------------------------------------------------------------------
// Streaming kernel (K <= 2048).

// An empty use of a loaded value.  Placed after the weight stream has been
// issued, it keeps an earlier load where it was written: a load whose only
// use sits in a branch may otherwise be sunk into that branch, behind the
// weight stream, and then wait for all of it.  (The wait it implies is for
// loads issued before the weights, which are needed next anyway.)
template <typename T>
__device__ __forceinline__ void pin_load(const T &v) {
  asm volatile("" ::"v"(v));
}

constexpr int kStreamThreads = 256;  // 4 waves, one n-tile each
constexpr int kStreamXR = 8;         // 16-byte X pieces staged per thread
constexpr int kStreamMaxKT = 32;     // k-tiles (K <= 2048)
constexpr int kStreamPitch = kStreamMaxKT * 64 + 16;
constexpr int kStreamPre = 4;        // segments whose weight scales are fetched up front

struct StreamArgs {
  int32_t M, N, K;
  int32_t pieces_per_row;  // 16-byte pieces per input row (bf16: K/8, int8: K/16)
  int32_t pieces;          // M * pieces_per_row
  uint32_t ppr_magic;      // ceil(2^32 / pieces_per_row): row = umulhi(piece, magic), exact
                           // for pieces < 4096 and pieces_per_row <= 4096
  const uint8_t *x;        // bf16 X, signed codes, or the + plane
  int64_t ld_bytes;        // row stride of x in bytes
  int64_t plane_stride;    // bytes from the + plane to the - plane (planes input)
  const int8_t *w;
  const float *w_scale;
  const float *act;  // [4][n_kseg]
  uint16_t *y;
  int64_t ld_y;
  int32_t *acc;
  int32_t n_kseg;      // <= kStreamMaxKT (every segment is whole k-tiles)
  uint32_t fold_mask;  // bit t: a K-segment ends with k-tile t
  int32_t single;      // single scale: the + half's scales for both signs, one dumped product
};

// QL: activation input, -1 bf16 (quantised here), 0 signed codes, 1 planes.
// RING: weight tiles requested per wave, a multiple of 8 with K/64 <= RING.
// SEG1: the call has one K-segment.
// PACK: M <= 8.  Both halves share one A operand, in groups of four rows:
// rows 4j, 4j+1 hold the + plane of X rows 2j, 2j+1 and rows 4j+2, 4j+3 their
// - plane.  One matrix-core instruction per weight tile then computes both
// products (half the chain), and since a lane's four result registers are
// four consecutive rows, each lane holds both halves of its two X rows: the
// fold needs no data from other lanes.  Otherwise each half has its own A
// operand (rows at or past M zero).
// W4: 4-bit weight tiles (512 bytes, 8 per lane), widened in registers.
// XR: 16-byte activation pieces staged per thread (up to XR * 256 pieces):
// every slot is loaded, before the weight stream, whether a thread has a
// piece there or not (a branch around the loads would break the
// straight-line load order the chain's waits rely on), so calls with few
// pieces take XR = 2 and issue six loads per thread fewer.
template <int QL, int RING, bool SEG1, bool PACK, bool W4, bool DEBUG, int XR>
__global__ __launch_bounds__(kStreamThreads) void gemm_smallm_kernel(StreamArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t planes[2 * kSmallMMax * kStreamPitch];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int NT = a.N / 16, KT = a.K / 64, nS = a.n_kseg;
  const int nt = blockIdx.x * 4 + wave;
  const bool active = nt < NT;
  const int ntc = min(nt, NT - 1);  // idle waves work on a valid tile and store nothing
  const int n = ntc * 16 + (lane & 15);
  const int pitch = a.K + 16;
  uint8_t *pp = planes;
  uint8_t *pn = planes + a.M * pitch;

  // (0) the first two weight tiles, so the stream starts at once; waiting
  //     for X below also waits for them, and the chain needs them first.
  //     (c2 on MI355X: 4.55 against 4.62 us per call with X issued first;
  //     four or eight tiles ahead gained less.)
  constexpr int kLead = RING < 2 ? RING : 2;
  constexpr int kTileBytes = W4 ? 512 : 1024;
  const int8_t *wcol = a.w + (int64_t)ntc * KT * kTileBytes + lane * (W4 ? 8 : 16);
  v4u ring[W4 ? 1 : RING];
  v2u ring4[W4 ? RING : 1];
#pragma unroll
  for (int d = 0; d < kLead; ++d) {
    const int8_t *src = wcol + (int64_t)min(d, KT - 1) * kTileBytes;
    if (W4) ring4[W4 ? d : 0] = *reinterpret_cast<const v2u *>(src);
    else ring[W4 ? 0 : d] = *reinterpret_cast<const v4u *>(src);
    __builtin_amdgcn_sched_barrier(0);  // in tile order
  }

  // (1) this thread's pieces of X and, for bf16 input, the inverse scales of
  //     their segments (the segment of k-tile kt is the number of segment
  //     ends before it).  Pieces past the end load a valid piece and are
  //     never stored.  These go before the rest of the weight stream: what
  //     is issued after it waits behind it.
  v4u xr[XR], xn[QL == 1 ? XR : 1];
  float ipv[QL < 0 ? XR : 1], inv_[QL < 0 ? XR : 1];
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int pc = min(tid + i * kStreamThreads, a.pieces - 1);
    const int row = (int)__umulhi((uint32_t)pc, a.ppr_magic), c = pc - row * a.pieces_per_row;
    const uint8_t *src = a.x + row * a.ld_bytes + c * 16;
    xr[i] = *reinterpret_cast<const v4u *>(src);
    if (QL == 1) xn[QL == 1 ? i : 0] = *reinterpret_cast<const v4u *>(src + a.plane_stride);
    if (QL < 0) {
      if (SEG1 && i > 0) {  // one K-segment: every piece has the same pair, loaded once
        ipv[QL < 0 ? i : 0] = ipv[0];
        inv_[QL < 0 ? i : 0] = inv_[0];
      } else {
        const int sg = SEG1 ? 0 : __builtin_popcount(a.fold_mask & ((1u << (c >> 3)) - 1u));
        ipv[QL < 0 ? i : 0] = a.act[2 * nS + sg];
        inv_[QL < 0 ? i : 0] = a.act[(a.single ? 2 : 3) * nS + sg];
      }
    }
  }

  // (2) what the folds need: this lane's segment pair s+/s- (lane i holds
  //     segment i) and the weight scales of the first kStreamPre segments for
  //     column n (a queue: each fold takes the head and fetches one more)
  const int ti = min(lane & 31, nS - 1);
  const float sp_l = a.act[ti];
  const float sn_l = a.act[(a.single ? 0 : nS) + ti];
  float wsp[kStreamPre];
#pragma unroll
  for (int j = 0; j < kStreamPre; ++j)  // (one K-segment: one scale, loaded once)
    wsp[j] = SEG1 && j > 0 ? wsp[0] : a.w_scale[(int64_t)min(j, nS - 1) * a.N + n];

  // (3) the rest of this wave's weight stream (the scheduling barriers keep
  //     the loads above ahead of it in issue order)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = kLead; d < RING; ++d) {
    const int8_t *src = wcol + (int64_t)min(d, KT - 1) * kTileBytes;
    if (W4) ring4[W4 ? d : 0] = *reinterpret_cast<const v2u *>(src);
    else ring[W4 ? 0 : d] = *reinterpret_cast<const v4u *>(src);
    __builtin_amdgcn_sched_barrier(0);  // in tile order, as the chain below waits for them
  }

#pragma unroll
  for (int i = 0; i < XR; ++i) {
    pin_load(xr[i]);
    if (QL == 1) pin_load(xn[QL == 1 ? i : 0]);
    if (QL < 0 && !(SEG1 && i > 0)) {
      pin_load(ipv[QL < 0 ? i : 0]);
      pin_load(inv_[QL < 0 ? i : 0]);
    }
  }
  pin_load(sp_l);
  pin_load(sn_l);
#pragma unroll
  for (int j = 0; j < (SEG1 ? 1 : kStreamPre); ++j) pin_load(wsp[j]);

  // (4) quantise (or split) X into the two planes
#pragma unroll
  for (int i = 0; i < XR; ++i) {
    const int p = tid + i * kStreamThreads;
    if (p < a.pieces) {
      const int row = (int)__umulhi((uint32_t)p, a.ppr_magic), c = p - row * a.pieces_per_row;
      if (QL < 0) {
        v2u qp, qn;
        quant8_planes(xr[i], ipv[QL < 0 ? i : 0], inv_[QL < 0 ? i : 0], qp, qn);
        *reinterpret_cast<v2u *>(pp + row * pitch + c * 8) = qp;
        *reinterpret_cast<v2u *>(pn + row * pitch + c * 8) = qn;
      } else if (QL == 0) {
        v4u qp, qn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t u, v;
          split_signed(xr[i][j], u, v);
          qp[j] = u;
          qn[j] = v;
        }
        *reinterpret_cast<v4u *>(pp + row * pitch + c * 16) = qp;
        *reinterpret_cast<v4u *>(pn + row * pitch + c * 16) = qn;
      } else {
        *reinterpret_cast<v4u *>(pp + row * pitch + c * 16) = xr[i];
        *reinterpret_cast<v4u *>(pn + row * pitch + c * 16) = xn[QL == 1 ? i : 0];
      }
    }
  }
  __syncthreads();

  // (5) every A fragment of the call (rows at or past M are zero).  Lane l
  //     supplies row l % 16, k-bytes 16 (l / 16) .. +16 of each k-tile.
  const int row = lane & 15, kq = (lane >> 4) * 16;
  // PACK: operand row 4j + p is X row 2j + (p & 1), - plane when p >= 2
  const int xrow = PACK ? ((row >> 2) << 1) + (row & 1) : row;
  const bool row_ok = xrow < a.M;
  const uint8_t *fsrc = (PACK && (row & 2) ? pn : pp) + xrow * pitch + kq;
  v4u fa[RING], fb[PACK ? 1 : RING];
#pragma unroll
  for (int t = 0; t < RING; ++t) {
    fa[t] = v4u{0u, 0u, 0u, 0u};
    if (!PACK) fb[PACK ? 0 : t] = v4u{0u, 0u, 0u, 0u};
  }
  if (row_ok) {  // the other lanes' rows are zero padding: no LDS traffic for them
    const int tmax = KT - 1;
#pragma unroll
    for (int t = 0; t < RING; ++t) {
      const int tt = min(t, tmax);
      fa[t] = *reinterpret_cast<const v4u *>(fsrc + tt * 64);
      if (!PACK) fb[PACK ? 0 : t] = *reinterpret_cast<const v4u *>(pn + row * pitch + tt * 64 + kq);
    }
  }
  // Ring slots past K hold a repeat of the last weight tile; their A
  // fragments are zero, so they add nothing.  (Masking the A side, not the
  // loaded weights: a select on a weight register would make the chain wait
  // for that load early, and the compiler hoists such selects.)
#pragma unroll
  for (int t = RING - 7; t < RING; ++t) {
    if (t < 0) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      fa[t][e] = t < KT ? fa[t][e] : 0u;
      if (!PACK) fb[PACK ? 0 : t][e] = t < KT ? fb[PACK ? 0 : t][e] : 0u;
    }
  }

  // (6) matrix-core chain as the weight tiles arrive; fold at segment ends.
  //     The 16x16 result: lane l holds column l % 16, rows 4 (l / 16) + r.
  float yacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // segments fold in order: wsp[0] is this segment's scale; shift the queue
  // and fetch the one kStreamPre segments ahead
  auto next_wscale = [&](int seg) {
    const float ws = wsp[0];
#pragma unroll
    for (int j = 0; j + 1 < kStreamPre; ++j) wsp[j] = wsp[j + 1];
    if (!SEG1) wsp[kStreamPre - 1] = a.w_scale[(int64_t)min(seg + kStreamPre, nS - 1) * a.N + n];
    return ws;
  };
  // PACK: lane l holds, for column n and X rows 2j, 2j+1 (j = l / 16), the
  // + products in registers 0, 1 and the - products in registers 2, 3
  auto fold_packed = [&](int seg, const v4i &C) {
    if (DEBUG) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (lane >> 4) * 2 + (r & 1);
        if (active && m < a.M && !(a.single && r >= 2))
          a.acc[((int64_t)((r >> 1) * nS + seg) * a.M + m) * a.N + n] =
              a.single ? C[r] + C[(r + 2) & 3] : C[r];
      }
    }
    const float ws = next_wscale(seg);
    const float sp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sp_l), seg));
    const float sn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sn_l), seg));
    const float cp = sp * ws, cn = sn * ws;
#pragma unroll
    for (int r = 0; r < 2; ++r)
      yacc[r] = __builtin_fmaf(cn, (float)C[r + 2], __builtin_fmaf(cp, (float)C[r], yacc[r]));
  };
  auto fold = [&](int seg, const v4i &P, const v4i &Q) {
    if (DEBUG) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (lane >> 4) * 4 + r;
        if (active && m < a.M) {
          const int64_t o = ((int64_t)seg * a.M + m) * a.N + n;
          if (a.single) {
            a.acc[o] = P[r] + Q[r];
          } else {
            a.acc[o] = P[r];
            a.acc[(int64_t)nS * a.M * a.N + o] = Q[r];
          }
        }
      }
    }
    const float ws = next_wscale(seg);
    const float sp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sp_l), seg));
    const float sn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sn_l), seg));
    const float cp = sp * ws, cn = sn * ws;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      yacc[r] = __builtin_fmaf(cn, (float)Q[r], __builtin_fmaf(cp, (float)P[r], yacc[r]));
  };
  auto wtile = [&](int t) { return W4 ? unpack_w4(ring4[W4 ? t : 0]) : ring[W4 ? 0 : t]; };
  auto mfma = [](const v4u &x, const v4u &w, const v4i &c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(reinterpret_cast<const v4i &>(x),
                                                 reinterpret_cast<const v4i &>(w), c, 0, 0, 0);
  };
  if (PACK && SEG1) {
    // one instruction per tile, two independent chains (even, odd tiles)
    v4i acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int t = 0; t < RING; ++t) acc[t & 1] = mfma(fa[t], wtile(t), acc[t & 1]);
    fold_packed(0, acc[0] + acc[1]);
  } else if (PACK) {
    v4i acc = {0, 0, 0, 0};
    int seg = 0;
#pragma unroll
    for (int t = 0; t < RING; ++t) {
      acc = mfma(fa[t], wtile(t), acc);
      if ((a.fold_mask >> t) & 1u) {
        fold_packed(seg, acc);
        acc = v4i{0, 0, 0, 0};
        ++seg;
      }
    }
  } else if (SEG1) {
    // one K-segment: no fold until the end, so the chain is branch-free; even
    // and odd k-tiles accumulate separately (two independent chains per
    // half) and are added at the end (exact in int32)
    v4i acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int t = 0; t < RING; ++t) {
      const v4u b = wtile(t);
      acc[(t & 1) * 2] = mfma(fa[t], b, acc[(t & 1) * 2]);
      acc[(t & 1) * 2 + 1] = mfma(fb[PACK ? 0 : t], b, acc[(t & 1) * 2 + 1]);
    }
    fold(0, acc[0] + acc[2], acc[1] + acc[3]);
  } else {
    v4i accp = {0, 0, 0, 0}, accn = {0, 0, 0, 0};
    int seg = 0;
#pragma unroll
    for (int t = 0; t < RING; ++t) {
      const v4u b = wtile(t);
      accp = mfma(fa[t], b, accp);
      accn = mfma(fb[PACK ? 0 : t], b, accn);
      if ((a.fold_mask >> t) & 1u) {
        fold(seg, accp, accn);
        accp = v4i{0, 0, 0, 0};
        accn = v4i{0, 0, 0, 0};
        ++seg;
      }
    }
  }

  // epilogue: rows (lane/16)*4 + r of column n (PACK: rows (lane/16)*2 + r)
#pragma unroll
  for (int r = 0; r < (PACK ? 2 : 4); ++r) {
    const int m = (lane >> 4) * (PACK ? 2 : 4) + r;
    if (active && m < a.M) a.y[(int64_t)m * a.ld_y + n] = (uint16_t)f32_to_bf16_rne(yacc[r]);
  }
}

template <int RING, bool SEG1, bool PACK, bool W4, int XR>
void launch_stream_ring(const StreamArgs &a, int ql, bool debug, dim3 grid, hipStream_t s) {
#define SQ_STREAM(QLV, DBG)                                                           \
  hipLaunchKernelGGL((gemm_smallm_kernel<QLV, RING, SEG1, PACK, W4, DBG, XR>), grid,  \
                     dim3(kStreamThreads), 0, s, a)
  if (debug) {
    if (ql < 0) SQ_STREAM(-1, true);
    else if (ql == 0) SQ_STREAM(0, true);
    else SQ_STREAM(1, true);
  } else {
    if (ql < 0) SQ_STREAM(-1, false);
    else if (ql == 0) SQ_STREAM(0, false);
    else SQ_STREAM(1, false);
  }
#undef SQ_STREAM
}

template <int RING, bool W4>
void launch_stream_w(const StreamArgs &a, int ql, bool debug, dim3 grid, hipStream_t s) {
  const bool pack = a.M <= 8;
  const bool few = a.pieces <= 2 * kStreamThreads;  // (M <= 8 only: XR = 2)
  if (a.n_kseg == 1) {
    if (pack && few) launch_stream_ring<RING, true, true, W4, 2>(a, ql, debug, grid, s);
    else if (pack) launch_stream_ring<RING, true, true, W4, kStreamXR>(a, ql, debug, grid, s);
    else launch_stream_ring<RING, true, false, W4, kStreamXR>(a, ql, debug, grid, s);
  } else {
    if (pack && few) launch_stream_ring<RING, false, true, W4, 2>(a, ql, debug, grid, s);
    else if (pack) launch_stream_ring<RING, false, true, W4, kStreamXR>(a, ql, debug, grid, s);
    else launch_stream_ring<RING, false, false, W4, kStreamXR>(a, ql, debug, grid, s);
  }
}

template <int RING>
void launch_stream_segs(const StreamArgs &a, int ql, bool debug, bool w4, dim3 grid,
                        hipStream_t s) {
  if (w4) launch_stream_w<RING, true>(a, ql, debug, grid, s);
  else launch_stream_w<RING, false>(a, ql, debug, grid, s);
}

// Shapes the streaming kernel takes; the rest go to the chunked kernel.
bool stream_fits(const GemmProblem &p) { return smallm_reads_w4(p.M, p.K, p.ks.n, p.x != nullptr); }

hipError_t launch_stream(const GemmProblem &p, hipStream_t s) {
  StreamArgs a{};
  a.M = (int32_t)p.M;
  a.N = (int32_t)p.N;
  a.K = (int32_t)p.K;
  const int ql = p.x ? -1 : p.q_layout;
  a.pieces_per_row = (int32_t)(p.x ? p.K / 8 : p.K / 16);
  a.pieces = (int32_t)(p.M * a.pieces_per_row);
  a.ppr_magic = (uint32_t)(((1ull << 32) + a.pieces_per_row - 1) / a.pieces_per_row);
  if (p.x) {
    a.x = reinterpret_cast<const uint8_t *>(p.x);
    a.ld_bytes = p.ld_x * 2;
  } else {
    a.x = reinterpret_cast<const uint8_t *>(p.xq);
    a.ld_bytes = p.ld_q;
  }
  a.plane_stride = ql == 1 ? p.M * p.ld_q : 0;
  a.w = p.w_packed;
  a.w_scale = p.w_scale;
  a.act = p.act;
  a.y = p.y;
  a.ld_y = p.ld_y;
  a.acc = p.acc_debug;
  a.single = p.single_scale ? 1 : 0;
  a.n_kseg = p.ks.n;
  a.fold_mask = 0;
  for (int i = 0; i < p.ks.n; ++i) a.fold_mask |= 1u << (p.ks.end[i] / 64 - 1);
  const int KT = (int)(p.K / 64);
  const dim3 grid((unsigned)((p.N / 16 + 3) / 4));
  const bool debug = p.acc_debug != nullptr;
  if (KT <= 8) launch_stream_segs<8>(a, ql, debug, p.w4, grid, s);
  else if (KT <= 16) launch_stream_segs<16>(a, ql, debug, p.w4, grid, s);
  else if (KT <= 24) launch_stream_segs<24>(a, ql, debug, p.w4, grid, s);
  else launch_stream_segs<32>(a, ql, debug, p.w4, grid, s);
  return hipGetLastError();
}

}  // namespace

bool smallm_reads_w4(int64_t M, int64_t K, int n_kseg, bool bf16_input) {
  const int64_t KT = K / 64;
  const int64_t ppr = bf16_input ? K / 8 : K / 16;
  return KT <= kStreamMaxKT && n_kseg <= kStreamMaxKT && M * ppr <= kStreamXR * kStreamThreads;
}

hipError_t launch_gemm_smallm(const GemmProblem &p, hipStream_t s) {
  if (stream_fits(p)) return launch_stream(p, s);
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
  a.single = p.single_scale ? 1 : 0;
  a.n_kseg = p.ks.n;
  for (int i = 0; i < p.ks.n; ++i) a.seg_end_tile[i] = p.ks.end[i] / 64;
  dim3 grid((unsigned)((p.N / 16 + WPG - 1) / WPG)), block(NTHR);
#define SQ_SMALL(QLV, ONEV, DBG) \
  hipLaunchKernelGGL((gemm_smallm_chunked_kernel<WPG, QLV, ONEV, DBG>), grid, block, 0, s, a)
#define SQ_SMALL_Q(ONEV, DBG)              \
  do {                                     \
    if (ql < 0) SQ_SMALL(-1, ONEV, DBG);    \
    else if (ql == 0) SQ_SMALL(0, ONEV, DBG); \
    else SQ_SMALL(1, ONEV, DBG);            \
  } while (0)
  const int ql = a.q_layout;
  if (p.acc_debug) SQ_SMALL_Q(false, true);
  else SQ_SMALL_Q(false, false);
#undef SQ_SMALL_Q
#undef SQ_SMALL
  return hipGetLastError();
}

}  // namespace sq
