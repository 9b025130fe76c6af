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
#include "msda_device.h"
#include "msda_launch.h"

#include <hip/hip_bf16.h>

namespace msda {
namespace {

constexpr int kMaxBlock = 256;
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
#ifdef MSDA_NO_XCD_REMAP
  return blockIdx.x;
#else
  const uint32_t per = gridDim.x / kXcds;
  return (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
#endif
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

template <typename T, int D>
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
#pragma unroll 2
  for (int j = 0; j < LK; ++j) {
    const Corners cs = geo[j * gs_stride + grp];
    uint32_t raw[4][RL::WORDS];
#pragma unroll
    for (int c = 0; c < 4; ++c) buffer_load<RL::WORDS>(rsrc, cs.off[c] + lane_off, raw[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x[RL::VEC];
      unpack<T, RL::WORDS>(raw[c], x);
#pragma unroll
      for (int i = 0; i < RL::VEC; ++i) acc[i] = fmaf(cs.w[c], x[i], acc[i]);
    }
  }
  uint32_t ow[RL::WORDS];
  pack<T, RL::WORDS>(acc, ow);
  char *out = reinterpret_cast<char *>(a.out) + (hq0 + grp) * (int64_t)RL::kRowBytes + lane_off;
  global_store<RL::WORDS>(out, ow);
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
    // bf16 accumulator: packed pairs, straight into grad_value through plain
    // global atomics, so the range test is explicit here.
    if (off >= acc_bytes) return;
    unsigned int *p = reinterpret_cast<unsigned int *>(acc_base + off + lane_off_acc);
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      __hip_bfloat162_raw r;
      r.x = (unsigned short)bf16_bits_rne(wc * g[2 * i]);
      r.y = (unsigned short)bf16_bits_rne(wc * g[2 * i + 1]);
      unsafeAtomicAdd(reinterpret_cast<__hip_bfloat162 *>(p + i), __hip_bfloat162(r));
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

__global__ __launch_bounds__(256) void cast_kernel(const float4 *src, uint4 *dst, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 x = src[2 * i], y = src[2 * i + 1];
    dst[i] = make_uint4(bf16_bits_rne(x.x) | (bf16_bits_rne(x.y) << 16),
                        bf16_bits_rne(x.z) | (bf16_bits_rne(x.w) << 16),
                        bf16_bits_rne(y.x) | (bf16_bits_rne(y.y) << 16),
                        bf16_bits_rne(y.z) | (bf16_bits_rne(y.w) << 16));
  }
}

// Head-queries per block: one block of up to 256 lanes, shrunk so the
// per-sample LDS stays within budget; always a whole number of wavefronts.
int pick_hqb(int G, int LK, int bytes_per_sample) {
  int hqb = kMaxBlock / G;
  while (hqb > 64 / G && hqb * LK * bytes_per_sample > kGeoLdsBudget) hqb /= 2;
  return hqb;
}

template <typename T, int D>
hipError_t fwd_launch(const LaunchArgs &a, hipStream_t stream) {
  using RL = RowLayout<T, D>;
  const int LK = (int)(a.L * a.K);
  const int hqb = pick_hqb(RL::G, LK, (int)sizeof(Corners));
  const int64_t total_hq = a.nb * a.Q * a.M;
  const int64_t blocks = padded_grid((total_hq + hqb - 1) / hqb);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)LK * (hqb + 1) * sizeof(Corners);
  prof_begin(stream);
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(hqb * RL::G), lds, stream,
                     a, hqb);
  prof_end(stream, "fwd");
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
  prof_begin(stream);
  hipLaunchKernelGGL((bwd_kernel<T, D, AccT>), dim3((unsigned)blocks), dim3(hqb * RL::G), lds,
                     stream, a, hqb);
  prof_end(stream, "bwd_atomic");
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_dispatch_d(const LaunchArgs &a, hipStream_t s) {
  switch (a.D) {
    case 8: return fwd_launch<T, 8>(a, s);
    case 16: return fwd_launch<T, 16>(a, s);
    case 32: return fwd_launch<T, 32>(a, s);
    case 64: return fwd_launch<T, 64>(a, s);
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

hipError_t launch_forward(const LaunchArgs &a, Dtype dt, hipStream_t stream) {
  if (a.nb * a.Q * a.M == 0) return hipSuccess;
  return dt == Dtype::F32 ? fwd_dispatch_d<float>(a, stream) : fwd_dispatch_d<bf16_t>(a, stream);
}

hipError_t launch_backward(const LaunchArgs &a, Dtype dt, Accum acc, hipStream_t stream) {
  if (a.nb * a.Q * a.M == 0) return hipSuccess;
  if (dt == Dtype::F32) return bwd_dispatch_d<float, float>(a, stream);
  if (acc == Accum::F32) return bwd_dispatch_d<bf16_t, float>(a, stream);
  return bwd_dispatch_d<bf16_t, bf16_t>(a, stream);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 4096);
  prof_begin(stream);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint4 *>(p), n16);
  prof_end(stream, "zero");
  return hipGetLastError();
}

hipError_t launch_cast_f32_to_bf16(const float *src, void *dst, size_t n, hipStream_t stream) {
  const size_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n8 + 255) / 256, 4096);
  prof_begin(stream);
  hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const float4 *>(src), reinterpret_cast<uint4 *>(dst), n8);
  prof_end(stream, "cast");
  return hipGetLastError();
}

}  // namespace msda
