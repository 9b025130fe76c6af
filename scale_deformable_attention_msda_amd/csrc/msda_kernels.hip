// MSDA forward and backward kernels for gfx950 (CDNA4, wave64).
//
// What is computed: "1. Deformable attention, from scratch" (msda-triton
// course, chapter 1), sections "The equation, term by term", "Bilinear
// interpolation: reading between the pixels" and "The simplest possible
// implementation".  The gradients are those of <out, grad_out>, derived by
// differentiating that loop (grad_value by scattered accumulation, as the
// course index and "Efficient Multi-Scale Deformable Attention on GPUs",
// section "The backward pass is an atomics problem", describe it).
//
// Work decomposition (both kernels).  A "head-query" is one (b, q, m); its
// L*K samples all read rows of head m of batch b.  A block owns `hqb`
// consecutive head-queries, so its samples are one contiguous range of
// sampling_locations / attention_weights:
//   phase 1  one lane per sample: read (x, y, A), compute the four corner
//            byte offsets and weights once, store them in LDS (sample-major
//            so the groups of a wave read neighbouring LDS words);
//   phase 2  one group of G lanes per head-query: each lane owns VEC
//            consecutive channels, so the four corner rows are read with one
//            coalesced 4..16-byte-per-lane buffer load each.  Corners outside
//            the level carry an offset past the buffer end, which the
//            hardware turns into zeros (loads) or no-ops (atomics).
// The operator is a data-dependent gather / scatter with one FMA per loaded
// element: it is memory-bound, so there is no MFMA here.
//
// "softmax" method (DeformOps documentation, section "Multi-scale deformable
// attention"): the weights of one head-query are the softmax of its L*K raw
// logits taken jointly over levels and points.  The forward kernel forms them
// on chip (phase 0 below) from the logits it reads in place of the weights;
// the backward uses the two row passes at the end of this file around the
// regular backward.
#include "msda_device.h"
#include "msda_launch.h"

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include <type_traits>

namespace msda {
namespace {

// lanes per forward / atomic-backward block at most (the sweep builds variants)
#ifndef MSDA_FWD_BLOCK
#define MSDA_FWD_BLOCK 256
#endif
constexpr int kMaxBlock = MSDA_FWD_BLOCK;
static_assert(kMaxBlock == 128 || kMaxBlock == 256 || kMaxBlock == 512 || kMaxBlock == 1024,
              "block of 128..1024 lanes");
constexpr int kGeoLdsBudget = 64 * 1024;

// Per-sample data the backward needs beyond the corners.
struct SampleAux {
  float a;   // attention weight (0 for a sample with no corner inside)
  float u;   // normalised location (the fractions are recomputed in fp64)
  float v;
  int l;     // level
};

template <typename T>
__device__ inline float ld(const void *base, int64_t i) {
  return to_float<T>(reinterpret_cast<const T *>(base)[i]);
}

// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin by
// block index.  Remap so that XCD x runs one contiguous range of logical
// blocks: neighbouring head-queries, which sample neighbouring pixels, then
// share that XCD's L2.  The grid is a multiple of 8; logical blocks past the
// end return at once.
constexpr int kXcds = 8;

__device__ inline int64_t logical_block() {
  const uint32_t per = gridDim.x / kXcds;
  return (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
}

inline int64_t padded_grid(int64_t blocks) { return (blocks + kXcds - 1) / kXcds * kXcds; }

__device__ inline void stage_levels(Level *lv, const LaunchArgs &a) {
  if (threadIdx.x < a.L) {
    lv[threadIdx.x].H = (int)a.shapes[2 * threadIdx.x];
    lv[threadIdx.x].W = (int)a.shapes[2 * threadIdx.x + 1];
    lv[threadIdx.x].start = (int)a.starts[threadIdx.x];
    lv[threadIdx.x].pad = 0;
  }
}

// ------------------------------------------------------------------ forward

// SOFTMAX: a.attn holds raw logits; the weight of sample j of head-query h is
// exp(z_j - max_h) / sum_i exp(z_i - max_h) over the L*K samples of h.  Phase 1
// gives lane s of each pass sample s of the block (passes start at multiples
// of the block size), so for L*K a power of two (at most 64) a head-query's
// logits sit in an aligned lane group and each lane forms its weight there;
// otherwise phase 0 stages the logits in LDS first.
// PIPE: samples whose corner loads a lane keeps in flight (4 * PIPE buffer
// loads); the loop runs over L*K rounded up to a multiple of PIPE, the padding
// samples reading nothing (offset past the buffer end, weight 0).
template <typename T, int D, bool SOFTMAX, int PIPE>
__global__ __launch_bounds__(kMaxBlock) void fwd_kernel(LaunchArgs a, int hqb) {
  using RL = RowLayout<T, D>;
  constexpr int G = RL::G;
  __shared__ Level lv[kMaxLevels];
  // [L*K][hqb + 1]: the odd row stride (in 32-byte entries) spreads the
  // phase-1 stores of consecutive samples (consecutive j) over all LDS banks
  extern __shared__ Corners geo[];
  const int gs_stride = hqb + 1;

  const int K = (int)a.K, LK = (int)(a.L * a.K), M = (int)a.M;
  const int64_t total_hq = a.nb * a.Q * a.M;
  const int64_t hq0 = logical_block() * hqb;
  if (hq0 >= total_hq) return;
  const int nhq = (int)min((int64_t)hqb, total_hq - hq0);
  stage_levels(lv, a);

  // phase 0 (softmax, L*K not a power of two): the block's logits,
  // [hqb][L*K + 1] in LDS, become exp(z - max) in place, with 1 / sum per
  // head-query beside them
  float *zb = reinterpret_cast<float *>(geo + LK * gs_stride);
  float *inv = zb + hqb * (LK + 1);
  const bool in_lanes = LK <= 64 && (LK & (LK - 1)) == 0;
  if (SOFTMAX && !in_lanes) {
    const int zs = LK + 1;
    for (int s = threadIdx.x; s < nhq * LK; s += blockDim.x) {
      const int hl = s / LK;
      zb[hl * zs + s - hl * LK] = ld<T>(a.attn, hq0 * LK + s);
    }
    __syncthreads();
    for (int hl = threadIdx.x; hl < nhq; hl += blockDim.x) {
      float *z = zb + hl * zs;
      float mx = z[0];
      for (int j = 1; j < LK; ++j) mx = z[j] > mx ? z[j] : mx;
      float sum = 0.0f;
      for (int j = 0; j < LK; ++j) {
        const float e = expf(z[j] - mx);
        z[j] = e;
        sum += e;
      }
      inv[hl] = 1.0f / sum;
    }
  }
  __syncthreads();

  // phase 1: geometry, one lane per sample
  const uint32_t row_stride = (uint32_t)(M * D * (int)sizeof(T));
  for (int s = threadIdx.x; s < nhq * LK; s += blockDim.x) {
    const int hl = s / LK;
    const int j = s - hl * LK;
    const int64_t hq = hq0 + hl;
    const int64_t gs = hq * LK + j;
    const int m = (int)(hq % M);
    const int64_t b = hq / M / a.Q;
    const float u = ld<T>(a.loc, 2 * gs), v = ld<T>(a.loc, 2 * gs + 1);
    float w;
    if constexpr (SOFTMAX)
      w = in_lanes ? group_softmax(ld<T>(a.attn, gs), LK) : zb[hl * (LK + 1) + j] * inv[hl];
    else
      w = ld<T>(a.attn, gs);
    Corners cs;
    float lx, ly;
    sample_corners(u, v, lv[j / K], (uint32_t)(b * a.S), row_stride,
                   (uint32_t)(m * D * (int)sizeof(T)), cs, lx, ly);
#pragma unroll
    for (int c = 0; c < 4; ++c) cs.w[c] *= w;
    geo[j * gs_stride + hl] = cs;
  }
  __syncthreads();

  // phase 2: gather-accumulate, one group of G lanes per head-query
  const int grp = threadIdx.x / G, lane = threadIdx.x % G;
  if (grp >= nhq) return;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.value, a.value_bytes);
  const uint32_t lane_off = (uint32_t)(lane * RL::kLaneBytes);
  float acc[RL::VEC];
#pragma unroll
  for (int i = 0; i < RL::VEC; ++i) acc[i] = 0.0f;
  // software pipeline: buffer u holds the four corner rows of one sample; it
  // is consumed, then refilled with the sample PIPE further on, so a lane
  // always has 4 * (PIPE - 1) to 4 * PIPE loads outstanding
  const int lk_pad = (LK + PIPE - 1) / PIPE * PIPE;
  uint32_t raw[PIPE][4][RL::WORDS];
  float wt[PIPE][4];
  auto issue = [&](int u, int j) {
    Corners cs = geo[min(j, LK - 1) * gs_stride + grp];
    if (j >= LK) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cs.off[c] = kOutside;
        cs.w[c] = 0.0f;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      buffer_load<RL::WORDS>(rsrc, cs.off[c] + lane_off, raw[u][c]);
      wt[u][c] = cs.w[c];
    }
  };
  auto consume = [&](int u) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x[RL::VEC];
      unpack<T, RL::WORDS>(raw[u][c], x);
#pragma unroll
      for (int i = 0; i < RL::VEC; ++i) acc[i] = fmaf(wt[u][c], x[i], acc[i]);
    }
  };
#pragma unroll
  for (int u = 0; u < PIPE; ++u) issue(u, u);
  for (int j0 = 0; j0 + PIPE < lk_pad; j0 += PIPE) {
#pragma unroll
    for (int u = 0; u < PIPE; ++u) {
      consume(u);
      issue(u, j0 + PIPE + u);
    }
  }
#pragma unroll
  for (int u = 0; u < PIPE; ++u) consume(u);
  uint32_t ow[RL::WORDS];
  pack<T, RL::WORDS>(acc, ow);
  char *out = reinterpret_cast<char *>(a.out) + (hq0 + grp) * (int64_t)RL::kRowBytes + lane_off;
  global_store<RL::WORDS>(out, ow);
}

// ---------------------------------------------- forward, LDS-resident levels
//
// The corner rows of the coarse levels are read over and over: every query
// samples every level, and the coarsest levels hold few pixels, so on the
// encoder workloads half the samples fall on levels 2 and 3 (1.3 K of the
// pyramid's 22 K pixels).  Every row the direct gather reads passes the
// vector L1 / texture path, which returns at most ~60 B per clock per CU on
// this GPU, while LDS returns ~110 B per clock per CU: both paths work at once
// when the coarse levels are read from LDS and the fine ones from the L1.
//
// A block owns one (batch b, head m) and a run of queries [q0, q0 + nq).  It
// keeps in LDS, for head m of image b:
//   - every level whose rows fit whole (smallest levels first), and
//   - for the first level that does not fit, a window of the rows left room
//     for: the consecutive rows that hold the most of the block's samples on
//     that level (a histogram of their cell rows, taken before staging);
// all other levels, and samples whose cell leaves the window, are gathered
// from global memory as in fwd_kernel.  The choice only decides where a row
// is read from, never the result: each corner still gets its value and weight.
// After staging, every wavefront walks its own chunks of 64 / G head-queries
// with fwd_kernel's two phases (geometry one lane per sample into the wave's
// LDS table; gather one lane group per head-query), with no block barrier, so
// the geometry of one wave overlaps the gathers of the others.  LDS-mode
// corners carry kLdsFlag in their offset; an invalid corner of an LDS-mode
// sample reads the zero row at the window area's head.
constexpr uint32_t kLdsFlag = 0x40000000u;   // bit 30 set, bit 31 clear: an LDS offset
constexpr int kWinThreads = 1024;
constexpr int kWinMinRows = 4;               // a window level holds at least this many rows
constexpr int kWinHistMax = 4096;            // rows a window level may have

struct WinLevel {
  int mode;  // 0 global, 1 whole level in LDS, 2 window of rows
  int rows;  // rows held
  int y0;    // first row held
  int lds;   // byte offset of the level's first held row in the window area
};

// Window-area placement of the levels for this launch's shapes (one thread):
// whole levels smallest first while they fit, then one window level.
template <int RB>
__device__ inline void plan_windows(const Level *lv, int L, uint32_t budget, WinLevel *wl) {
  uint32_t used = RB;  // the zero row
  bool done = false;
  uint32_t taken = 0;  // bit l: level l placed
  for (int n = 0; n < L; ++n) {
    int best = -1;
    for (int l = 0; l < L; ++l)
      if (!(taken >> l & 1u) &&
          (best < 0 || (int64_t)lv[l].H * lv[l].W < (int64_t)lv[best].H * lv[best].W))
        best = l;
    taken |= 1u << best;
    const int H = lv[best].H, W = lv[best].W;
    const uint64_t row = (uint64_t)W * RB;
    WinLevel w{0, 0, 0, 0};
    if (!done && H >= 1 && W >= 1) {
      if ((uint64_t)H * row <= budget - used) {
        w = WinLevel{1, H, 0, (int)used};
        used += (uint32_t)(H * row);
      } else {
        // the window level's area first holds the histogram of its H + 1 cell rows
        const uint64_t fit = (budget - used) / row;
        if (fit >= (uint64_t)kWinMinRows && H <= kWinHistMax &&
            (uint64_t)(H + 1) * 4u <= budget - used)
          w = WinLevel{2, (int)fit, 0, (int)used};
        done = true;  // larger levels get nothing
      }
    }
    wl[best] = w;
  }
}

// 32-bit LDS addresses: the byte offset of a __shared__ location in the
// workgroup's LDS, and a load of WORDS dwords from such an offset.
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ inline uint32_t lds_offset_of(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_char_t *)p;
}
template <int WORDS>
__device__ inline void lds_load_at(uint32_t addr, uint32_t (&w)[WORDS]) {
  typedef uint32_t vec_t __attribute__((ext_vector_type(WORDS)));
  const vec_t x = *(const __attribute__((address_space(3))) vec_t *)(uintptr_t)addr;
#pragma unroll
  for (int i = 0; i < WORDS; ++i) w[i] = x[i];
}

template <int WORDS>
__device__ inline void lds_load(const char *base, uint32_t off, uint32_t (&w)[WORDS]) {
  if constexpr (WORDS == 4) {
    const uint4 x = *reinterpret_cast<const uint4 *>(base + off);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (WORDS == 2) {
    const uint2 x = *reinterpret_cast<const uint2 *>(base + off);
    w[0] = x.x; w[1] = x.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(base + off);
  }
}

// Geometry of one sample for the window schedule, one path for every level
// (the lanes of a wave hold samples of several levels): LDS offsets with
// kLdsFlag when the level is held and both of the cell's rows inside the
// level are among the held rows (an invalid corner reads the zero row), else
// the global offsets of sample_corners.  The coordinate and its floor are
// taken in fp64, exactly as sample_corners does.
__device__ inline void sample_corners_any(float u, float v, const Level &lv, const WinLevel &wl,
                                          uint32_t RB, uint32_t row_base, uint32_t row_stride,
                                          uint32_t head_off, Corners &cs) {
  const double x = (double)u * (double)lv.W - 0.5;
  const double y = (double)v * (double)lv.H - 0.5;
  const double xf = floor(x), yf = floor(y);
  const bool any = xf >= -1.0 && xf < (double)lv.W && yf >= -1.0 && yf < (double)lv.H;
  const int x0 = any ? (int)xf : 0, y0 = any ? (int)yf : 0;
  const float fx = any ? (float)(x - xf) : 0.0f, fy = any ? (float)(y - yf) : 0.0f;
  const bool xin0 = any && x0 >= 0, xin1 = any && x0 + 1 < lv.W;
  const bool yin0 = any && y0 >= 0, yin1 = any && y0 + 1 < lv.H;
  const bool held0 = !yin0 || (y0 >= wl.y0 && y0 < wl.y0 + wl.rows);
  const bool held1 = !yin1 || (y0 + 1 >= wl.y0 && y0 + 1 < wl.y0 + wl.rows);
  const bool lds = wl.mode != 0 && held0 && held1;
  // corner 00 and the steps to corners 01 and 10, in LDS or global bytes
  const uint32_t b00 = lds ? (uint32_t)wl.lds + (uint32_t)((y0 - wl.y0) * lv.W + x0) * RB
                           : (row_base + (uint32_t)lv.start + (uint32_t)(y0 * lv.W + x0)) *
                                 row_stride + head_off;
  const uint32_t sx = lds ? RB : row_stride;
  const uint32_t sy = (uint32_t)lv.W * sx;
  const uint32_t flag = lds ? kLdsFlag : 0u;
  const uint32_t none = lds ? kLdsFlag : kOutside;  // the zero row, or past the buffer end
  cs.off[0] = (xin0 && yin0) ? (b00 | flag) : none;
  cs.off[1] = (xin1 && yin0) ? ((b00 + sx) | flag) : none;
  cs.off[2] = (xin0 && yin1) ? ((b00 + sy) | flag) : none;
  cs.off[3] = (xin1 && yin1) ? ((b00 + sy + sx) | flag) : none;
  cs.w[0] = (xin0 && yin0) ? (1.0f - fx) * (1.0f - fy) : 0.0f;
  cs.w[1] = (xin1 && yin0) ? fx * (1.0f - fy) : 0.0f;
  cs.w[2] = (xin0 && yin1) ? (1.0f - fx) * fy : 0.0f;
  cs.w[3] = (xin1 && yin1) ? fx * fy : 0.0f;
}

struct WinArgs {
  int nwaves;         // waves per block; each walks its own chunks of 64 / G head-queries
  int qb;             // queries per block
  int nsplit;         // blocks per (batch, head)
  uint32_t geo_bytes; // LDS bytes before the window area (the waves' geometry tables)
  uint32_t win_bytes; // LDS bytes of the window area
  FastDiv div_lk, div_k;  // by L*K and by K
};

// Ordering of LDS traffic between the lanes of one wavefront: LDS operations
// of a wave complete in order, so a compiler barrier is all that is needed.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bytes of one wave's LDS tables: geometry [L*K][64/G + 1] and, for the softmax
// method with L*K not a power of two, the chunk's logits and 1 / sum.
__host__ __device__ inline uint32_t win_wave_bytes(int lk, int g, bool staged) {
  const int hpw = 64 / g;
  uint32_t b = (uint32_t)lk * (hpw + 1) * (uint32_t)sizeof(Corners);
  if (staged) b += (uint32_t)(hpw * (lk + 1) + hpw) * 4u;
  return (b + 15u) / 16u * 16u;
}

template <typename T, int D, bool SOFTMAX, int PIPE>
__global__ __launch_bounds__(kWinThreads) void fwd_win_kernel(LaunchArgs a, WinArgs wa) {
  using RL = RowLayout<T, D>;
  constexpr int G = RL::G;
  constexpr int RB = RL::kRowBytes;
  constexpr int HPW = 64 / G;  // head-queries per wave chunk
  __shared__ Level lv[kMaxLevels];
  __shared__ WinLevel wl[kMaxLevels];
  __shared__ uint8_t jlist[2][64];       // sample indices j on global / LDS-held levels
  __shared__ int jcount[2];
  __shared__ int best_shared;
  extern __shared__ __align__(16) char smem[];
  char *win = smem + wa.geo_bytes;

  const int K = (int)a.K, LK = (int)(a.L * a.K), M = (int)a.M, L = (int)a.L;
  const int64_t lb = logical_block();
  if (lb >= a.nb * a.M * wa.nsplit) return;
  const int bm = (int)(lb / wa.nsplit), split = (int)(lb - (int64_t)bm * wa.nsplit);
  const int b = bm / M, m = bm - b * M;
  const int64_t q0 = (int64_t)split * wa.qb;
  if (q0 >= a.Q) return;
  const int nq = (int)min((int64_t)wa.qb, a.Q - q0);
  stage_levels(lv, a);
  __syncthreads();
  if (threadIdx.x == 0) {
    plan_windows<RB>(lv, L, wa.win_bytes, wl);
    int n[2] = {0, 0};
    for (int j = 0; j < LK; ++j) {
      const int c = wl[j / K].mode != 0 ? 1 : 0;
      jlist[c][n[c]++] = (uint8_t)j;
    }
    jcount[0] = n[0];
    jcount[1] = n[1];
  }
  __syncthreads();

  const uint32_t row_stride = (uint32_t)(M * RB);
  const uint32_t head_off = (uint32_t)(m * RB);
  const uint32_t row_base = (uint32_t)(b * a.S);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.value, a.value_bytes);
  constexpr int P = RB / 16;  // 16-byte pieces per head row (RB >= 16)

  // Stage the held rows of the levels in mode `only`, eight 16-byte loads in
  // flight per thread (the level loop is uniform, so nothing waits per load).
  auto stage = [&](int only) {
    constexpr int kBatch = 8;
    for (int l = 0; l < L; ++l) {
      if (wl[l].mode != only) continue;
      const int W = lv[l].W, n = wl[l].rows * W * P;
      const uint32_t first = row_base + (uint32_t)lv[l].start + (uint32_t)(wl[l].y0 * W);
      for (int c0 = 0; c0 < n; c0 += kBatch * (int)blockDim.x) {
        uint32_t w[kBatch][4];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int c = min(c0 + k * (int)blockDim.x + (int)threadIdx.x, n - 1);
          const int p = c / P, piece = c - p * P;
          buffer_load<4>(rsrc, (first + (uint32_t)p) * row_stride + head_off + (uint32_t)(piece * 16),
                         w[k]);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int c = c0 + k * (int)blockDim.x + (int)threadIdx.x;
          if (c < n)
            *reinterpret_cast<uint4 *>(win + wl[l].lds + c * 16) =
                make_uint4(w[k][0], w[k][1], w[k][2], w[k][3]);
        }
      }
    }
  };

  // the zero row, and the levels held whole
  for (int i = threadIdx.x; i < RB / 4; i += blockDim.x) reinterpret_cast<uint32_t *>(win)[i] = 0u;
  stage(1);

  // the window level's rows: histogram of the block's cell rows on it (staged
  // past the whole levels), then the R consecutive rows that hold the most
  // samples whole
  int wlev = -1;
  for (int l = 0; l < L; ++l)
    if (wl[l].mode == 2) wlev = l;
  if (wlev >= 0) {
    const int H = lv[wlev].H, W = lv[wlev].W, R = wl[wlev].rows;
    uint32_t *hist = reinterpret_cast<uint32_t *>(win + wl[wlev].lds);  // H + 1 bins: row y0 + 1
    for (int i = threadIdx.x; i <= H; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    constexpr int kBatch = 4;
    for (int t0 = 0; t0 < nq * K; t0 += kBatch * (int)blockDim.x) {
      float u[kBatch], v[kBatch];
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        int t = t0 + r * (int)blockDim.x + (int)threadIdx.x;
        t = t < nq * K ? t : 0;
        const int i = t / K, k = t - i * K;
        const int64_t gs = (((int64_t)b * a.Q + q0 + i) * M + m) * LK + wlev * K + k;
        u[r] = ld<T>(a.loc, 2 * gs);
        v[r] = ld<T>(a.loc, 2 * gs + 1);
      }
#pragma unroll
      for (int r = 0; r < kBatch; ++r) {
        if (t0 + r * (int)blockDim.x + (int)threadIdx.x >= nq * K) break;
        const double xf = floor((double)u[r] * (double)W - 0.5);
        const double yf = floor((double)v[r] * (double)H - 0.5);
        if (xf >= -1.0 && xf < (double)W && yf >= -1.0 && yf < (double)H)
          __hip_atomic_fetch_add(&hist[(int)yf + 1], 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // inclusive prefix sums of hist, in place (one wave, 64 bins a round)
      uint32_t carry = 0;
      for (int base = 0; base <= H; base += 64) {
        const int i = base + (int)threadIdx.x;
        uint32_t x = i <= H ? hist[i] : 0u;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(x, o);
          if ((int)threadIdx.x >= o) x += y;
        }
        if (i <= H) hist[i] = x + carry;
        carry += __shfl(x, 63);
      }
      // coverage of the rows [w0, w0 + R): cells y0 in [w0, w0 + R - 2], plus
      // y0 = -1 when w0 = 0 and y0 = H - 1 when w0 = H - R
      uint32_t best = 0;
      int best_w0 = 0;
      for (int w0 = threadIdx.x; w0 <= H - R; w0 += 64) {
        uint32_t cov = hist[w0 + R - 1] - hist[w0];
        if (w0 == 0) cov += hist[0];
        if (w0 == H - R) cov += hist[H] - hist[H - 1];
        if (cov > best) {
          best = cov;
          best_w0 = w0;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t ob = __shfl_xor(best, o);
        const int ow = __shfl_xor(best_w0, o);
        if (ob > best || (ob == best && ow < best_w0)) {
          best = ob;
          best_w0 = ow;
        }
      }
      if (threadIdx.x == 0) best_shared = best_w0;
    }
    __syncthreads();
    if (threadIdx.x == 0) wl[wlev].y0 = best_shared;
    __syncthreads();
    stage(2);
  }
  __syncthreads();

  // Every wave walks chunks of HPW head-queries on its own (chunks wave,
  // wave + nwaves, ...): geometry into its own LDS table, then the gather; no
  // block barrier, so one wave's geometry overlaps the others' gathers.
  const int wave = (int)threadIdx.x / 64, wlane = (int)threadIdx.x % 64;
  const bool in_lanes = LK <= 64 && (LK & (LK - 1)) == 0;
  const bool staged = SOFTMAX && !in_lanes;
  const int gs_stride = HPW + 1;
  char *wbase = smem + (uint32_t)wave * win_wave_bytes(LK, G, staged);
  Corners *geo = reinterpret_cast<Corners *>(wbase);
  float *zb = reinterpret_cast<float *>(geo + LK * gs_stride);  // [HPW][L*K + 1]
  float *inv = zb + HPW * (LK + 1);
  const int grp = wlane / G, lane = wlane % G;
  const uint32_t lane_off = (uint32_t)(lane * RL::kLaneBytes);

  // sample s of a chunk (s = entry * L*K + j): location and raw weight
  auto load_sample = [&](const T *locp, const T *attp, int s, float &u, float &v, float &wraw) {
    const int hl = (int)fdiv((uint32_t)s, wa.div_lk);
    const int j = s - hl * LK;
    const uint32_t gs = (uint32_t)hl * (uint32_t)(M * LK) + (uint32_t)j;
    if constexpr (sizeof(T) == 4) {
      const float2 uv = reinterpret_cast<const float2 *>(locp)[gs];
      u = uv.x;
      v = uv.y;
    } else {
      const uint32_t uv = reinterpret_cast<const uint32_t *>(locp)[gs];
      u = Half<T>::lo(uv);
      v = Half<T>::hi(uv);
    }
    wraw = to_float<T>(attp[gs]);
  };
  // the first kPf samples of each lane in the chunk at h0n, loaded ahead
  // (where a chunk holds at most 8 head-queries: with more, two samples a
  // lane cover too little of it to pay for the registers; the softmax forms
  // hold more registers already)
  constexpr int kPf = !SOFTMAX && HPW <= 8 ? 2 : 0;
  float pf_u[kPf > 0 ? kPf : 1], pf_v[kPf > 0 ? kPf : 1], pf_w[kPf > 0 ? kPf : 1];
  auto prefetch = [&](int h0n) {
    const int nhn = min(HPW, nq - h0n);
    const int64_t hqf = ((int64_t)b * a.Q + q0 + min(h0n, nq - 1)) * M + m;
    const T *locp = reinterpret_cast<const T *>(a.loc) + 2 * hqf * LK;
    const T *attp = reinterpret_cast<const T *>(a.attn) + hqf * LK;
#pragma unroll
    for (int k = 0; k < kPf; ++k) {
      pf_u[k] = pf_v[k] = pf_w[k] = 0.0f;
      if (wlane + 64 * k < nhn * LK) load_sample(locp, attp, wlane + 64 * k, pf_u[k], pf_v[k], pf_w[k]);
    }
  };
  prefetch(wave * HPW);

  for (int h0 = wave * HPW; h0 < nq; h0 += wa.nwaves * HPW) {
    const int nh = min(HPW, nq - h0);
    const int64_t hq_first = ((int64_t)b * a.Q + q0 + h0) * M + m;  // hq of chunk entry 0
    if (staged) {
      // the chunk's logits; lane hl < nh turns its row into exp(z - max) and 1 / sum
      const int zs = LK + 1;
      for (int s = wlane; s < nh * LK; s += 64) {
        const int hl = s / LK;
        zb[hl * zs + s - hl * LK] = ld<T>(a.attn, (hq_first + (int64_t)hl * M) * LK + s - hl * LK);
      }
      wave_lds_sync();
      if (wlane < nh) {
        float *z = zb + wlane * zs;
        float mx = z[0];
        for (int j = 1; j < LK; ++j) mx = z[j] > mx ? z[j] : mx;
        float sum = 0.0f;
        for (int j = 0; j < LK; ++j) {
          const float e = expf(z[j] - mx);
          z[j] = e;
          sum += e;
        }
        inv[wlane] = 1.0f / sum;
      }
      wave_lds_sync();
    }
    // geometry, one lane per sample (32-bit sample offsets from the chunk's
    // first); the first kPf samples of each lane come from the prefetch
    const T *locp = reinterpret_cast<const T *>(a.loc) + 2 * hq_first * LK;
    const T *attp = reinterpret_cast<const T *>(a.attn) + hq_first * LK;
    auto geometry = [&](int s, float u, float v, float wraw) {
      const int hl = (int)fdiv((uint32_t)s, wa.div_lk);
      const int j = s - hl * LK;
      float w;
      if constexpr (SOFTMAX)
        w = in_lanes ? group_softmax(wraw, LK) : zb[hl * (LK + 1) + j] * inv[hl];
      else
        w = wraw;
      const int l = (int)fdiv((uint32_t)j, wa.div_k);
      Corners cs;
      sample_corners_any(u, v, lv[l], wl[l], (uint32_t)RB, row_base, row_stride, head_off, cs);
#pragma unroll
      for (int c = 0; c < 4; ++c) cs.w[c] *= w;
      geo[j * gs_stride + hl] = cs;
    };
#pragma unroll
    for (int k = 0; k < kPf; ++k)
      if (wlane + 64 * k < nh * LK) geometry(wlane + 64 * k, pf_u[k], pf_v[k], pf_w[k]);
    for (int s = wlane + 64 * kPf; s < nh * LK; s += 64) {
      float u, v, wraw;
      load_sample(locp, attp, s, u, v, wraw);
      geometry(s, u, v, wraw);
    }
    // the next chunk's locations and weights: in flight during this gather
    prefetch(h0 + wa.nwaves * HPW);
    wave_lds_sync();

    // gather, in two passes, so that the registers LDS reads fill are never
    // targets of global loads still in flight (no LDS read then waits for them):
    //   1. samples on global levels, buffer loads, PIPE samples in flight (a
    //      sample's buffer u is consumed and refilled with the sample PIPE on);
    //   2. samples on LDS-held levels.
    // Each head-query adds its samples in the same order in every block.
    if (grp < nh) {
      float acc[RL::VEC];
#pragma unroll
      for (int i = 0; i < RL::VEC; ++i) acc[i] = 0.0f;
      auto fma_rows = [&](const uint32_t (&raw)[4][RL::WORDS], const float (&w)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float x[RL::VEC];
          unpack<T, RL::WORDS>(raw[c], x);
#pragma unroll
          for (int i = 0; i < RL::VEC; ++i) acc[i] = fmaf(w[c], x[i], acc[i]);
        }
      };
      // pass 1: whole rounds of PIPE samples pipelined, then the tail one by one
      {
        const int n = jcount[0];
        const int n_main = n / PIPE * PIPE;
        uint32_t raw[PIPE][4][RL::WORDS];
        float wt[PIPE][4];
        auto issue = [&](int u, int t) {
          const Corners cs = geo[(int)jlist[0][t] * gs_stride + grp];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            buffer_load<RL::WORDS>(rsrc, cs.off[c] + lane_off, raw[u][c]);
            wt[u][c] = cs.w[c];
          }
        };
        if (n_main > 0) {
#pragma unroll
          for (int u = 0; u < PIPE; ++u) issue(u, u);
          for (int t0 = PIPE; t0 < n_main; t0 += PIPE) {
#pragma unroll
            for (int u = 0; u < PIPE; ++u) {
              fma_rows(raw[u], wt[u]);
              issue(u, t0 + u);
            }
          }
#pragma unroll
          for (int u = 0; u < PIPE; ++u) fma_rows(raw[u], wt[u]);
        }
        for (int t = n_main; t < n; ++t) {
          issue(0, t);
          fma_rows(raw[0], wt[0]);
        }
      }
      // pass 2, in the samples' order: LDS reads, or for a sample whose cell
      // leaves the held rows (rare), global loads in its place, so that the
      // order of the additions does not depend on which samples fall back
      const int n = jcount[1];
      // an LDS-mode offset carries kLdsFlag: adding (window + lane - kLdsFlag)
      // yields the LDS address
      const uint32_t lane_win_flag = lds_offset_of(win) + lane_off - kLdsFlag;
      auto rows = [&](int t, uint32_t (&raw)[4][RL::WORDS], float (&wt)[4]) {
        const Corners cs = geo[(int)jlist[1][t] * gs_stride + grp];
        if ((cs.off[0] >> 30) == 1u) {
#pragma unroll
          for (int c = 0; c < 4; ++c) lds_load_at<RL::WORDS>(cs.off[c] + lane_win_flag, raw[c]);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) buffer_load<RL::WORDS>(rsrc, cs.off[c] + lane_off, raw[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) wt[c] = cs.w[c];
      };
      int t = 0;
      for (; t + 2 <= n; t += 2) {
        uint32_t raw[2][4][RL::WORDS];
        float wt[2][4];
        rows(t, raw[0], wt[0]);
        rows(t + 1, raw[1], wt[1]);
        fma_rows(raw[0], wt[0]);
        fma_rows(raw[1], wt[1]);
      }
      if (t < n) {
        uint32_t raw[4][RL::WORDS];
        float wt[4];
        rows(t, raw, wt);
        fma_rows(raw, wt);
      }
      uint32_t ow[RL::WORDS];
      pack<T, RL::WORDS>(acc, ow);
      char *out = reinterpret_cast<char *>(a.out) +
                  (hq_first + (int64_t)grp * M) * (int64_t)RL::kRowBytes + lane_off;
      global_store<RL::WORDS>(out, ow);
    }
    wave_lds_sync();  // the next chunk rewrites this wave's tables
  }
}

// ----------------------------------------------------------------- backward

// Scatter of a * w_c * g into the grad_value accumulator for one corner.
template <typename T, typename AccT, int WORDS, int VEC>
__device__ inline void scatter_corner(const __amdgpu_buffer_rsrc_t acc_rsrc, char *acc_base,
                                      uint32_t acc_bytes, uint32_t off, uint32_t lane_off_acc,
                                      float wc, const float (&g)[VEC]) {
  if constexpr (sizeof(AccT) == 4) {
    // fp32 accumulator: off is the byte offset of the corner row in T units;
    // the accumulator row is sizeof(float)/sizeof(T) times wider.
    const uint32_t aoff = (sizeof(T) == 4 ? off : off * 2u) + lane_off_acc;
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(wc * g[i], acc_rsrc, (int)(aoff + 4u * i), 0, 0);
  } else {
    // 16-bit accumulator (the data type): packed pairs, straight into
    // grad_value through plain global atomics, so the range test is explicit here.
    if (off >= acc_bytes) return;
    unsigned int *p = reinterpret_cast<unsigned int *>(acc_base + off + lane_off_acc);
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      const unsigned short x = (unsigned short)Half<AccT>::bits(wc * g[2 * i]);
      const unsigned short y = (unsigned short)Half<AccT>::bits(wc * g[2 * i + 1]);
      if constexpr (std::is_same_v<AccT, bf16_t>) {
        __hip_bfloat162_raw r;
        r.x = x;
        r.y = y;
        unsafeAtomicAdd(reinterpret_cast<__hip_bfloat162 *>(p + i), __hip_bfloat162(r));
      } else {
        unsafeAtomicAdd(reinterpret_cast<__half2 *>(p + i),
                        __halves2half2(__ushort_as_half(x), __ushort_as_half(y)));
      }
    }
  }
}

template <typename T, int D, typename AccT>
__global__ __launch_bounds__(kMaxBlock) void bwd_kernel(LaunchArgs a, int hqb) {
  using RL = RowLayout<T, D>;
  constexpr int G = RL::G;
  __shared__ Level lv[kMaxLevels];
  extern __shared__ char smem[];

  const int K = (int)a.K, LK = (int)(a.L * a.K), M = (int)a.M;
  // [LK][hqb + 1]: odd row strides spread the phase-1 stores over all banks
  const int gs_stride = hqb + 1;
  Corners *geo = reinterpret_cast<Corners *>(smem);                      // [LK][hqb + 1]
  SampleAux *aux = reinterpret_cast<SampleAux *>(geo + LK * gs_stride);  // [LK][hqb + 1]
  float *res = reinterpret_cast<float *>(aux + LK * gs_stride);          // [hqb*LK][3] in sample order

  const int64_t total_hq = a.nb * a.Q * a.M;
  const int64_t hq0 = logical_block() * hqb;
  if (hq0 >= total_hq) return;
  const int nhq = (int)min((int64_t)hqb, total_hq - hq0);
  stage_levels(lv, a);
  __syncthreads();

  // phase 1: geometry, one lane per sample
  const uint32_t row_stride = (uint32_t)(M * D * (int)sizeof(T));
  for (int s = threadIdx.x; s < nhq * LK; s += blockDim.x) {
    const int hl = s / LK;
    const int j = s - hl * LK;
    const int64_t hq = hq0 + hl;
    const int64_t gs = hq * LK + j;
    const int m = (int)(hq % M);
    const int64_t b = hq / M / a.Q;
    const float u = ld<T>(a.loc, 2 * gs), v = ld<T>(a.loc, 2 * gs + 1);
    const float w = ld<T>(a.attn, gs);
    Corners cs;
    SampleAux ax;
    float lx, ly;
    const bool any = sample_corners(u, v, lv[j / K], (uint32_t)(b * a.S), row_stride,
                                    (uint32_t)(m * D * (int)sizeof(T)), cs, lx, ly);
    ax.a = any ? w : 0.0f;
    ax.u = u;
    ax.v = v;
    ax.l = j / K;
    geo[j * gs_stride + hl] = cs;
    aux[j * gs_stride + hl] = ax;
  }
  __syncthreads();

  // phase 2: gather, reduce, scatter; one group of G lanes per head-query
  const int grp = threadIdx.x / G, lane = threadIdx.x % G;
  if (grp < nhq) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.value, a.value_bytes);
    const __amdgpu_buffer_rsrc_t acc_rsrc = make_rsrc(a.grad_acc, a.acc_bytes);
    char *acc_base = reinterpret_cast<char *>(a.grad_acc);
    const uint32_t lane_off = (uint32_t)(lane * RL::kLaneBytes);
    const uint32_t lane_off_acc = (uint32_t)(lane * RL::VEC * (int)sizeof(AccT));
    float g[RL::VEC];
    {
      uint32_t gw[RL::WORDS];
      global_load<RL::WORDS>(reinterpret_cast<const char *>(a.grad_out) +
                                 (hq0 + grp) * (int64_t)RL::kRowBytes + lane_off, gw);
      unpack<T, RL::WORDS>(gw, g);
    }
    for (int j = 0; j < LK; ++j) {
      const Corners cs = geo[j * gs_stride + grp];
      const SampleAux ax = aux[j * gs_stride + grp];
      uint32_t raw[4][RL::WORDS];
#pragma unroll
      for (int c = 0; c < 4; ++c) buffer_load<RL::WORDS>(rsrc, cs.off[c] + lane_off, raw[c]);
      // fp64 partial dot products <g, V_c> (exact products), reduced across the group
      double p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x[RL::VEC];
        unpack<T, RL::WORDS>(raw[c], x);
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < RL::VEC; ++i) s = fma((double)g[i], (double)x[i], s);
        p[c] = s;
      }
      const int W = lv[ax.l].W, H = lv[ax.l].H;
      const double x = (double)ax.u * (double)W - 0.5, y = (double)ax.v * (double)H - 0.5;
      const double lx = x - floor(x), ly = y - floor(y);
      // bilinear weights in fp64; 0 for corners outside the level (their p_c is 0 too)
      const double w0 = (1.0 - lx) * (1.0 - ly), w1 = lx * (1.0 - ly);
      const double w2 = (1.0 - lx) * ly, w3 = lx * ly;
      const double ga = group_sum_f64<G>(w0 * p[0] + w1 * p[1] + w2 * p[2] + w3 * p[3]);
      const double gx = group_sum_f64<G>((1.0 - ly) * (p[1] - p[0]) + ly * (p[3] - p[2]));
      const double gy = group_sum_f64<G>((1.0 - lx) * (p[2] - p[0]) + lx * (p[3] - p[1]));
      if (lane == 0) {
        const int s = grp * LK + j;
        const bool live = ax.a != 0.0f || cs.off[0] != kOutside || cs.off[1] != kOutside ||
                          cs.off[2] != kOutside || cs.off[3] != kOutside;
        res[3 * s] = live ? (float)ga : 0.0f;
        res[3 * s + 1] = live ? (float)((double)ax.a * W * gx) : 0.0f;
        res[3 * s + 2] = live ? (float)((double)ax.a * H * gy) : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        scatter_corner<T, AccT, RL::WORDS, RL::VEC>(acc_rsrc, acc_base, a.acc_bytes, cs.off[c],
                                                    lane_off_acc, ax.a * cs.w[c], g);
    }
  }
  __syncthreads();

  // coalesced write-back of grad_attn and grad_loc for the block's samples
  const int64_t s0 = hq0 * LK;
  for (int i = threadIdx.x; i < nhq * LK; i += blockDim.x) {
    store_scalar<T>(reinterpret_cast<T *>(a.grad_attn) + s0 + i, res[3 * i]);
    store_scalar<T>(reinterpret_cast<T *>(a.grad_loc) + 2 * (s0 + i), res[3 * i + 1]);
    store_scalar<T>(reinterpret_cast<T *>(a.grad_loc) + 2 * (s0 + i) + 1, res[3 * i + 2]);
  }
}

// ------------------------------------------------------------- utilities

__global__ __launch_bounds__(256) void zero_kernel(uint4 *p, size_t n16) {
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// fp32 -> a 16-bit type H, eight elements per thread and step.
template <typename H>
__global__ __launch_bounds__(256) void cast_kernel(const float4 *src, uint4 *dst, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 x = src[2 * i], y = src[2 * i + 1];
    dst[i] = make_uint4(Half<H>::bits(x.x) | (Half<H>::bits(x.y) << 16),
                        Half<H>::bits(x.z) | (Half<H>::bits(x.w) << 16),
                        Half<H>::bits(y.x) | (Half<H>::bits(y.y) << 16),
                        Half<H>::bits(y.z) | (Half<H>::bits(y.w) << 16));
  }
}

// Softmax row passes of the backward.  A row is the L*K logits of one
// head-query.  A block of 256 lanes owns `rows` consecutive rows at a time
// (one contiguous range of the tensor): it stages them in LDS with 16-byte
// loads, one lane then works through one row, and the results leave with
// 16-byte stores.  LDS rows are `zs` = L*K | 1 floats apart: an odd stride
// puts the per-row reads of the 64 lanes of a wave on distinct banks.
constexpr int kRowThreads = 256;

struct RowPass {
  int64_t n_rows;
  int lk, zs, rows;  // rows per pass: a multiple of 64, at most 256
  FastDiv div_lk;
};

template <typename T>
struct Vec16 {
  static constexpr int N = 16 / (int)sizeof(T);
};

template <typename T>
__device__ inline void unpack16(const uint4 &w, float (&f)[Vec16<T>::N]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = Half<T>::lo(u[i]);
      f[2 * i + 1] = Half<T>::hi(u[i]);
    }
  }
}

template <typename T>
__device__ inline uint4 pack16(const float (&f)[Vec16<T>::N]) {
  uint32_t u[4];
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = __float_as_uint(f[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = Half<T>::bits(f[2 * i]) | (Half<T>::bits(f[2 * i + 1]) << 16);
  }
  return make_uint4(u[0], u[1], u[2], u[3]);
}

// n elements of src (16-byte aligned) -> LDS rows of stride zs
template <typename T>
__device__ inline void stage_rows(const T *src, float *lds, int n, const RowPass &p) {
  constexpr int V = Vec16<T>::N;
  const int nv = n / V;
  for (int v = threadIdx.x; v < nv; v += kRowThreads) {
    float f[V];
    unpack16<T>(*reinterpret_cast<const uint4 *>(src + (int64_t)v * V), f);
    uint32_t r = fdiv((uint32_t)(v * V), p.div_lk);
    int c = v * V - (int)r * p.lk;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      lds[r * p.zs + c] = f[e];
      if (++c == p.lk) {
        c = 0;
        ++r;
      }
    }
  }
  for (int k = nv * V + threadIdx.x; k < n; k += kRowThreads) {
    const uint32_t r = fdiv((uint32_t)k, p.div_lk);
    lds[r * p.zs + k - (int)r * p.lk] = to_float<T>(src[k]);
  }
}

// LDS rows -> n elements of dst (16-byte aligned)
template <typename T>
__device__ inline void unstage_rows(T *dst, const float *lds, int n, const RowPass &p) {
  constexpr int V = Vec16<T>::N;
  const int nv = n / V;
  for (int v = threadIdx.x; v < nv; v += kRowThreads) {
    float f[V];
    uint32_t r = fdiv((uint32_t)(v * V), p.div_lk);
    int c = v * V - (int)r * p.lk;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      f[e] = lds[r * p.zs + c];
      if (++c == p.lk) {
        c = 0;
        ++r;
      }
    }
    *reinterpret_cast<uint4 *>(dst + (int64_t)v * V) = pack16<T>(f);
  }
  for (int k = nv * V + threadIdx.x; k < n; k += kRowThreads) {
    const uint32_t r = fdiv((uint32_t)k, p.div_lk);
    store_scalar<T>(dst + k, lds[r * p.zs + k - (int)r * p.lk]);
  }
}

// One row in registers: a[j] = exp(z[j] - max) / sum for j < lk (LKMAX >= lk,
// fully unrolled so that the row's LDS reads are issued together).
template <int LKMAX>
__device__ inline void softmax_row(const float *z, int lk, float (&a)[LKMAX]) {
  float mx = z[0];
#pragma unroll
  for (int j = 0; j < LKMAX; ++j) {
    a[j] = j < lk ? z[j] : -INFINITY;
    mx = a[j] > mx ? a[j] : mx;
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < LKMAX; ++j) {
    a[j] = j < lk ? expf(a[j] - mx) : 0.0f;
    sum += a[j];
  }
  const float r = 1.0f / sum;
#pragma unroll
  for (int j = 0; j < LKMAX; ++j) a[j] *= r;
}

// weights[r][j] = exp(z[r][j] - max_r) / sum_i exp(z[r][i] - max_r)
template <typename T, int LKMAX>
__global__ __launch_bounds__(kRowThreads) void softmax_rows_kernel(const T *__restrict__ logits,
                                                                   T *__restrict__ weights,
                                                                   RowPass p) {
  extern __shared__ float zrow[];
  for (int64_t r0 = (int64_t)blockIdx.x * p.rows; r0 < p.n_rows;
       r0 += (int64_t)gridDim.x * p.rows) {
    const int nr = (int)min((int64_t)p.rows, p.n_rows - r0);
    stage_rows<T>(logits + r0 * p.lk, zrow, nr * p.lk, p);
    __syncthreads();
    if ((int)threadIdx.x < nr) {
      float *z = zrow + threadIdx.x * p.zs;
      float a[LKMAX];
      softmax_row<LKMAX>(z, p.lk, a);
#pragma unroll
      for (int j = 0; j < LKMAX; ++j)
        if (j < p.lk) z[j] = a[j];
    }
    __syncthreads();
    unstage_rows<T>(weights + r0 * p.lk, zrow, nr * p.lk, p);
    __syncthreads();
  }
}

// Derivative through the softmax, in place: on entry g holds dLoss/dA (the
// regular backward's grad_attn for weights A = softmax(z)); on exit
// dLoss/dz_j = A_j (g_j - sum_i A_i g_i), with A recomputed from z in fp32.
template <typename T, int LKMAX>
__global__ __launch_bounds__(kRowThreads) void softmax_grad_rows_kernel(
    const T *__restrict__ logits, T *g, RowPass p) {
  extern __shared__ float zrow[];
  float *grow = zrow + p.rows * p.zs;
  for (int64_t r0 = (int64_t)blockIdx.x * p.rows; r0 < p.n_rows;
       r0 += (int64_t)gridDim.x * p.rows) {
    const int nr = (int)min((int64_t)p.rows, p.n_rows - r0);
    stage_rows<T>(logits + r0 * p.lk, zrow, nr * p.lk, p);
    stage_rows<T>(g + r0 * p.lk, grow, nr * p.lk, p);
    __syncthreads();
    if ((int)threadIdx.x < nr) {
      float *gr = grow + threadIdx.x * p.zs;
      float a[LKMAX], ga[LKMAX];
      softmax_row<LKMAX>(zrow + threadIdx.x * p.zs, p.lk, a);
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < LKMAX; ++j) {
        ga[j] = j < p.lk ? gr[j] : 0.0f;
        dot = fmaf(a[j], ga[j], dot);
      }
#pragma unroll
      for (int j = 0; j < LKMAX; ++j)
        if (j < p.lk) gr[j] = a[j] * (ga[j] - dot);
    }
    __syncthreads();
    unstage_rows<T>(g + r0 * p.lk, grow, nr * p.lk, p);
    __syncthreads();
  }
}

RowPass make_row_pass(int64_t n_rows, int lk) {
  RowPass p{};
  p.n_rows = n_rows;
  p.lk = lk;
  p.zs = lk | 1;
  // about 33 KB of LDS per staged tensor
  p.rows = std::max(64, std::min(kRowThreads, (33 * kRowThreads) / p.zs / 64 * 64));
  p.div_lk = make_fastdiv((uint32_t)lk);
  return p;
}

// Head-queries per block: one block of up to 256 lanes, shrunk so the
// per-sample LDS stays within budget; always a whole number of wavefronts.
int pick_hqb(int G, int LK, int bytes_per_sample) {
  int hqb = kMaxBlock / G;
  while (hqb > 64 / G && hqb * LK * bytes_per_sample > kGeoLdsBudget) hqb /= 2;
  return hqb;
}

// Samples in flight per lane in the forward gather: the deepest compiled depth
// (at most MSDA_FWD_PIPE) whose padding adds at most a quarter to the L*K
// rounds, else 2 (L*K = 16 takes MSDA_FWD_PIPE, 12 takes 4, 9 takes 2).
#ifndef MSDA_FWD_PIPE
#define MSDA_FWD_PIPE 2
#endif
constexpr int kFwdPipe = MSDA_FWD_PIPE;
static_assert(kFwdPipe == 2 || kFwdPipe == 4 || kFwdPipe == 8, "forward pipeline depth 2, 4 or 8");

int fwd_pipe_depth(int lk) {
  for (int p = kFwdPipe; p > 2; p /= 2)
    if ((lk + p - 1) / p * p * 4 <= lk * 5) return p;
  return 2;
}

template <typename T, int D, bool SOFTMAX>
void launch_fwd_pipe(int pipe, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                     const LaunchArgs &a, int hqb) {
  if (kFwdPipe >= 8 && pipe == 8)
    hipLaunchKernelGGL((fwd_kernel<T, D, SOFTMAX, (kFwdPipe >= 8 ? 8 : 2)>), grid, block, lds,
                       stream, a, hqb);
  else if (kFwdPipe >= 4 && pipe == 4)
    hipLaunchKernelGGL((fwd_kernel<T, D, SOFTMAX, (kFwdPipe >= 4 ? 4 : 2)>), grid, block, lds,
                       stream, a, hqb);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, SOFTMAX, 2>), grid, block, lds, stream, a, hqb);
}

template <typename T, int D>
hipError_t fwd_launch(const LaunchArgs &a, bool softmax, hipStream_t stream) {
  using RL = RowLayout<T, D>;
  const int LK = (int)(a.L * a.K);
  // softmax staged in LDS (L*K not a power of two): one more fp32 per sample
  // (the logit) and one per head-query (1 / sum)
  const bool staged = softmax && !(LK <= 64 && (LK & (LK - 1)) == 0);
  const int hqb = pick_hqb(RL::G, LK, (int)sizeof(Corners) + (staged ? 8 : 0));
  const int64_t total_hq = a.nb * a.Q * a.M;
  const int64_t blocks = padded_grid((total_hq + hqb - 1) / hqb);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  size_t lds = (size_t)LK * (hqb + 1) * sizeof(Corners);
  if (staged) lds += ((size_t)hqb * (LK + 1) + hqb) * sizeof(float);
  prof_begin(stream, softmax ? "fwd_softmax" : "fwd");
  const int pipe = fwd_pipe_depth(LK);
  if (softmax)
    launch_fwd_pipe<T, D, true>(pipe, dim3((unsigned)blocks), dim3(hqb * RL::G), lds, stream, a, hqb);
  else
    launch_fwd_pipe<T, D, false>(pipe, dim3((unsigned)blocks), dim3(hqb * RL::G), lds, stream, a, hqb);
  prof_end(stream, softmax ? "fwd_softmax" : "fwd");
  return hipGetLastError();
}

template <typename T, int D, typename AccT>
hipError_t bwd_launch(const LaunchArgs &a, hipStream_t stream) {
  using RL = RowLayout<T, D>;
  const int LK = (int)(a.L * a.K);
  constexpr int per_sample = (int)(sizeof(Corners) + sizeof(SampleAux) + 3 * sizeof(float));
  const int hqb = pick_hqb(RL::G, LK, per_sample);
  const int64_t total_hq = a.nb * a.Q * a.M;
  const int64_t blocks = padded_grid((total_hq + hqb - 1) / hqb);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)LK * (hqb + 1) * (sizeof(Corners) + sizeof(SampleAux)) +
                    (size_t)LK * hqb * 3 * sizeof(float);
  prof_begin(stream, "bwd_atomic");
  hipLaunchKernelGGL((bwd_kernel<T, D, AccT>), dim3((unsigned)blocks), dim3(hqb * RL::G), lds,
                     stream, a, hqb);
  prof_end(stream, "bwd_atomic");
  return hipGetLastError();
}

// The LDS-window forward's launch shape: head-queries per sub-batch (the
// geometry table, at most kWinGeoMax bytes), the LDS split, queries per block
// (about two blocks per CU over the launch).  False when it does not suit the
// launch: too few queries per (batch, head) for the staging to pay off, or
// too little LDS; the direct gather runs then.
constexpr size_t kWinGeoMax = 75 * 1024;  // the waves' geometry tables together
#ifndef MSDA_WIN_PIPE
#define MSDA_WIN_PIPE 4
#endif
#ifndef MSDA_WIN_BLOCKS_PER_CU
#define MSDA_WIN_BLOCKS_PER_CU 2
#endif
#ifndef MSDA_WIN_LDS_BLOCKS
#define MSDA_WIN_LDS_BLOCKS 1
#endif
constexpr int kWinPipe = MSDA_WIN_PIPE;              // samples in flight per lane
constexpr int kWinLdsBlocks = MSDA_WIN_LDS_BLOCKS;   // blocks sharing one CU's LDS
constexpr int kWinBlocksPerCu = MSDA_WIN_BLOCKS_PER_CU;  // blocks per CU over the launch
constexpr size_t kWinStaticReserve = 1024;  // the kernel's static LDS (levels, plan)

struct WinLaunch {
  WinArgs wa;
  int threads;
  size_t lds;
  int64_t blocks;
};

// 0: the window schedule when it suits the launch; 1: always the direct gather;
// 2: the window schedule whenever the LDS holds it (a test hook, per thread)
thread_local int g_fwd_schedule = 0;

template <typename T, int D>
bool plan_win_launch(const LaunchArgs &a, bool softmax, WinLaunch &w) {
  if (g_fwd_schedule == 1) return false;
  using RL = RowLayout<T, D>;
  const int LK = (int)(a.L * a.K);
  const bool staged = softmax && !(LK <= 64 && (LK & (LK - 1)) == 0);
  const size_t per_wave = win_wave_bytes(LK, RL::G, staged);
  const int nwaves = (int)std::min<size_t>(kWinThreads / 64 / kWinLdsBlocks,
                                           kWinGeoMax / kWinLdsBlocks / per_wave);
  // the blocks of a CU share its LDS: with fewer than 16 waves on the CU they
  // hide too little latency (measured slower than the direct gather: bf16 rows
  // with L*K = 12 or 32 get 11 and 4 waves), unless a test forces the schedule
  if (nwaves * kWinLdsBlocks < (g_fwd_schedule == 2 ? 4 : kWinThreads / 64)) return false;
  int dev = 0, max_lds = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  const size_t block_lds = (size_t)max_lds / kWinLdsBlocks;
  const size_t total = block_lds > kWinStaticReserve ? block_lds - kWinStaticReserve : 0;
  const size_t geo = per_wave * nwaves;
  // the window area must hold the zero row and the cell-row histogram of a window level
  if (total < geo + 32 * 1024) return false;
  const int64_t bm = a.nb * a.M;
  int64_t nsplit = std::max<int64_t>(1, (kWinBlocksPerCu * (int64_t)cus + bm - 1) / bm);
  int64_t qb = (a.Q + nsplit - 1) / nsplit;
  const int64_t hq_block = (int64_t)nwaves * (64 / RL::G);
  if (qb < 4 * hq_block && g_fwd_schedule != 2) return false;
  nsplit = (a.Q + qb - 1) / qb;
  w.wa.div_lk = make_fastdiv((uint32_t)LK);
  w.wa.div_k = make_fastdiv((uint32_t)a.K);
  w.wa.nwaves = nwaves;
  w.wa.qb = (int)qb;
  w.wa.nsplit = (int)nsplit;
  w.wa.geo_bytes = (uint32_t)geo;
  w.wa.win_bytes = (uint32_t)((total - geo) / 16 * 16);
  w.threads = nwaves * 64;
  w.lds = geo + w.wa.win_bytes;
  w.blocks = padded_grid(bm * nsplit);
  return w.blocks <= 0x7fffffff;
}

template <typename T, int D>
hipError_t fwd_launch_any(const LaunchArgs &a, bool softmax, hipStream_t stream) {
  WinLaunch w;
  if (!plan_win_launch<T, D>(a, softmax, w)) return fwd_launch<T, D>(a, softmax, stream);
  const char *name = softmax ? "fwd_softmax" : "fwd";
  prof_begin(stream, name);
  if (softmax)
    hipLaunchKernelGGL((fwd_win_kernel<T, D, true, kWinPipe>), dim3((unsigned)w.blocks),
                       dim3(w.threads), w.lds, stream, a, w.wa);
  else
    hipLaunchKernelGGL((fwd_win_kernel<T, D, false, kWinPipe>), dim3((unsigned)w.blocks),
                       dim3(w.threads), w.lds, stream, a, w.wa);
  prof_end(stream, name);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_dispatch_d(const LaunchArgs &a, bool softmax, hipStream_t s) {
  switch (a.D) {
    case 8: return fwd_launch_any<T, 8>(a, softmax, s);
    case 16: return fwd_launch_any<T, 16>(a, softmax, s);
    case 32: return fwd_launch_any<T, 32>(a, softmax, s);
    case 64: return fwd_launch_any<T, 64>(a, softmax, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename AccT>
hipError_t bwd_dispatch_d(const LaunchArgs &a, hipStream_t s) {
  switch (a.D) {
    case 8: return bwd_launch<T, 8, AccT>(a, s);
    case 16: return bwd_launch<T, 16, AccT>(a, s);
    case 32: return bwd_launch<T, 32, AccT>(a, s);
    case 64: return bwd_launch<T, 64, AccT>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

void set_forward_schedule(int schedule) { g_fwd_schedule = schedule; }

hipError_t launch_forward(const LaunchArgs &a, Dtype dt, hipStream_t stream, bool softmax) {
  if (a.nb * a.Q * a.M == 0) return hipSuccess;
  switch (dt) {
    case Dtype::F32: return fwd_dispatch_d<float>(a, softmax, stream);
    case Dtype::BF16: return fwd_dispatch_d<bf16_t>(a, softmax, stream);
    case Dtype::F16: return fwd_dispatch_d<f16_t>(a, softmax, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_backward(const LaunchArgs &a, Dtype dt, Accum acc, hipStream_t stream) {
  if (a.nb * a.Q * a.M == 0) return hipSuccess;
  switch (dt) {
    case Dtype::F32: return bwd_dispatch_d<float, float>(a, stream);
    case Dtype::BF16:
      return acc == Accum::F32 ? bwd_dispatch_d<bf16_t, float>(a, stream)
                               : bwd_dispatch_d<bf16_t, bf16_t>(a, stream);
    case Dtype::F16:
      return acc == Accum::F32 ? bwd_dispatch_d<f16_t, float>(a, stream)
                               : bwd_dispatch_d<f16_t, f16_t>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int LKMAX>
void enqueue_softmax_rows_t(const void *logits, void *weights, const RowPass &p, int64_t blocks,
                            size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((softmax_rows_kernel<T, LKMAX>), dim3((unsigned)blocks), dim3(kRowThreads),
                     lds, stream, static_cast<const T *>(logits), static_cast<T *>(weights), p);
}

template <int LKMAX>
void enqueue_softmax_rows(const void *logits, void *weights, const RowPass &p, int64_t blocks,
                          size_t lds, Dtype dt, hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: enqueue_softmax_rows_t<float, LKMAX>(logits, weights, p, blocks, lds, stream); break;
    case Dtype::BF16: enqueue_softmax_rows_t<bf16_t, LKMAX>(logits, weights, p, blocks, lds, stream); break;
    case Dtype::F16: enqueue_softmax_rows_t<f16_t, LKMAX>(logits, weights, p, blocks, lds, stream); break;
  }
}

template <typename T, int LKMAX>
void enqueue_softmax_grad_rows_t(const void *logits, void *grad, const RowPass &p, int64_t blocks,
                                 size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL((softmax_grad_rows_kernel<T, LKMAX>), dim3((unsigned)blocks),
                     dim3(kRowThreads), lds, stream, static_cast<const T *>(logits),
                     static_cast<T *>(grad), p);
}

template <int LKMAX>
void enqueue_softmax_grad_rows(const void *logits, void *grad, const RowPass &p, int64_t blocks,
                               size_t lds, Dtype dt, hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: enqueue_softmax_grad_rows_t<float, LKMAX>(logits, grad, p, blocks, lds, stream); break;
    case Dtype::BF16: enqueue_softmax_grad_rows_t<bf16_t, LKMAX>(logits, grad, p, blocks, lds, stream); break;
    case Dtype::F16: enqueue_softmax_grad_rows_t<f16_t, LKMAX>(logits, grad, p, blocks, lds, stream); break;
  }
}

hipError_t launch_softmax_rows(const void *logits, void *weights, int64_t n_rows, int lk,
                               Dtype dt, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (lk < 1 || lk > 64) return hipErrorInvalidValue;
  const RowPass p = make_row_pass(n_rows, lk);
  const int64_t blocks = std::min<int64_t>((n_rows + p.rows - 1) / p.rows, int64_t(1) << 20);
  const size_t lds = (size_t)p.rows * p.zs * sizeof(float);
  prof_begin(stream, "softmax_rows");
  if (lk <= 16)
    enqueue_softmax_rows<16>(logits, weights, p, blocks, lds, dt, stream);
  else if (lk <= 32)
    enqueue_softmax_rows<32>(logits, weights, p, blocks, lds, dt, stream);
  else
    enqueue_softmax_rows<64>(logits, weights, p, blocks, lds, dt, stream);
  prof_end(stream, "softmax_rows");
  return hipGetLastError();
}

hipError_t launch_softmax_grad_rows(const void *logits, void *grad, int64_t n_rows, int lk,
                                    Dtype dt, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (lk < 1 || lk > 64) return hipErrorInvalidValue;
  const RowPass p = make_row_pass(n_rows, lk);
  const int64_t blocks = std::min<int64_t>((n_rows + p.rows - 1) / p.rows, int64_t(1) << 20);
  const size_t lds = 2 * (size_t)p.rows * p.zs * sizeof(float);
  prof_begin(stream, "softmax_grad_rows");
  if (lk <= 16)
    enqueue_softmax_grad_rows<16>(logits, grad, p, blocks, lds, dt, stream);
  else if (lk <= 32)
    enqueue_softmax_grad_rows<32>(logits, grad, p, blocks, lds, dt, stream);
  else
    enqueue_softmax_grad_rows<64>(logits, grad, p, blocks, lds, dt, stream);
  prof_end(stream, "softmax_grad_rows");
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 4096);
  prof_begin(stream, "zero");
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4 *>(p), n16);
  prof_end(stream, "zero");
  return hipGetLastError();
}

hipError_t launch_cast_f32_to_half(const float *src, void *dst, size_t n, Dtype dt,
                                   hipStream_t stream) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  if (dt == Dtype::F32) return hipErrorInvalidValue;
  const size_t blocks = std::min<size_t>((n8 + 255) / 256, 4096);
  prof_begin(stream, "cast");
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(cast_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(src), reinterpret_cast<uint4 *>(dst), n8);
  else
    hipLaunchKernelGGL(cast_kernel<f16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(src), reinterpret_cast<uint4 *>(dst), n8);
  prof_end(stream, "cast");
  return hipGetLastError();
}

}  // namespace msda
