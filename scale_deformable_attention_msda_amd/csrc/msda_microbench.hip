// Microbenchmarks of the gfx950 memory paths the MSDA kernels depend on.
//
// They measure the ceilings the operator's kernels are measured against: what a
// streaming read and a copy reach in HBM, how many fp32 and packed-bf16
// global atomic adds per second the memory side retires (spread over a large
// span, or piled on a small hot set, as the coarse pyramid levels pile the
// scatter of the backward), and how fast a wavefront can gather random
// 128-byte rows (one head row of 32 fp32 channels) from the vector L1, from
// LDS, and from a span the size of a value tensor.  The pages frame the
// backward as an atomics problem and the forward as a question of how bytes
// move ("Efficient Multi-Scale Deformable Attention on GPUs", sections "Key
// findings" and "The backward pass is an atomics problem").
//
// Each kernel is launched `reps` times back to back on the caller's stream and
// timed with HIP events; the caller passes every buffer.
#include "msda_bench.h"

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;       // one head row of 32 fp32 channels
constexpr int kLanesPerRow = 8;      // 16 bytes per lane, as the forward gathers
constexpr int kGatherIters = 64;     // gather rounds per lane
constexpr int kGatherInflight = 8;   // independent rows a lane has in flight
constexpr int kLdsSpan = 64 * 1024;  // bytes of LDS the LDS gather reads from

__device__ inline uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(kThreads) void fill_kernel(uint4 *p, size_t n16, uint32_t seed) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kThreads) {
    const uint32_t h = mix((uint32_t)i ^ seed);
    // small finite floats: (h & 0x007fffff) | 0x3f000000 lies in [0.5, 1)
    const uint32_t f = (h & 0x007fffffu) | 0x3f000000u;
    p[i] = make_uint4(f, f ^ 1u, f ^ 2u, f ^ 3u);
  }
}

// Streaming read: four 16-byte loads per thread in flight per round.
__global__ __launch_bounds__(kThreads) void read_kernel(const uint4 *__restrict__ p, size_t n16,
                                                        float *sink) {
  float acc = 0.0f;
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc += __uint_as_float(a.x ^ b.y ^ c.z ^ d.w);
  }
  for (; i < n16; i += stride) acc += __uint_as_float(p[i].x);
  if (acc == -1.0f) sink[0] = acc;  // never true for the filled data; keeps the loads
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Whole-row atomics: a wavefront covers two 128-byte rows (32 lanes x 4 bytes
// each, fp32) or four rows of packed pairs (16 lanes x 4 bytes, bf16x2) per
// instruction; rows are picked at random among `nrows` (a power of two).
// ops counts element adds (fp32) or packed-pair adds (bf16x2).
template <bool PACKED>
__global__ __launch_bounds__(kThreads) void atomic_kernel(float *p, uint32_t row_mask,
                                                          uint32_t rounds, uint32_t seed) {
  constexpr int kLanes = PACKED ? 16 : 32;  // lanes per 128-byte row
  const uint32_t lane = threadIdx.x % kLanes;
  const uint32_t grp = (blockIdx.x * kThreads + threadIdx.x) / kLanes;
  for (uint32_t r = 0; r < rounds; ++r) {
    const uint32_t row = mix(grp * 0x9E3779B9u + r * 0x85ebca6bu + seed) & row_mask;
    float *dst = p + (size_t)row * (kRowBytes / 4) + lane;
    if constexpr (PACKED) {
      __hip_bfloat162_raw v;
      v.x = 0x3c00;  // 2^-7
      v.y = 0x3c00;
      unsafeAtomicAdd(reinterpret_cast<__hip_bfloat162 *>(dst), __hip_bfloat162(v));
    } else {
      unsafeAtomicAdd(dst, 0.0078125f);
    }
  }
}

// Random 128-byte rows gathered by 8-lane groups, 16 bytes per lane, with four
// FMAs per loaded 16 bytes (what the forward does with a corner row).
// SRC 0: buffer loads from a span of `span` bytes of global memory (L1 / L2 /
// MALL / HBM, depending on the span); SRC 1: LDS reads from a kLdsSpan-byte
// copy of the buffer's head.  Every lane keeps kGatherInflight rows in flight.
template <int SRC>
__global__ __launch_bounds__(kThreads) void gather_kernel(const float *src, uint32_t span,
                                                          float *sink, uint32_t seed) {
  __shared__ uint4 lds[SRC == 1 ? kLdsSpan / 16 : 1];
  const uint32_t lane = threadIdx.x % kLanesPerRow;
  const uint32_t grp = (blockIdx.x * kThreads + threadIdx.x) / kLanesPerRow;
  const uint32_t nrows = (SRC == 1 ? (uint32_t)kLdsSpan : span) / kRowBytes;  // a power of two
  uint32_t off[kGatherInflight];
#pragma unroll
  for (int k = 0; k < kGatherInflight; ++k)
    off[k] = (mix(grp * 0x9E3779B9u + (uint32_t)k * 0x632be5abu + seed) & (nrows - 1)) * kRowBytes +
             lane * 16;
  if constexpr (SRC == 1) {
    const uint4 *g = reinterpret_cast<const uint4 *>(src);
    for (int i = threadIdx.x; i < kLdsSpan / 16; i += kThreads) lds[i] = g[i];
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), (short)0, (int)span, 0x00020000);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const float w = 0.5f + (float)(threadIdx.x & 3);
  for (int it = 0; it < kGatherIters; ++it) {
    // a wave-uniform row flip per round: offsets stay inside the span
    const uint32_t flip = (mix((uint32_t)it + seed) & (nrows - 1)) * kRowBytes;
    uint4 v[kGatherInflight];
#pragma unroll
    for (int k = 0; k < kGatherInflight; ++k) {
      const uint32_t o = off[k] ^ flip;
      if constexpr (SRC == 1) {
        v[k] = lds[o / 16];
      } else {
        typedef uint32_t v4 __attribute__((ext_vector_type(4)));
        const v4 x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)o, 0, 0);
        v[k] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
#pragma unroll
    for (int k = 0; k < kGatherInflight; ++k) {
      acc[0] = fmaf(w, __uint_as_float(v[k].x), acc[0]);
      acc[1] = fmaf(w, __uint_as_float(v[k].y), acc[1]);
      acc[2] = fmaf(w, __uint_as_float(v[k].z), acc[2]);
      acc[3] = fmaf(w, __uint_as_float(v[k].w), acc[3]);
    }
  }
  if (acc[0] + acc[1] + acc[2] + acc[3] == -1.0f) sink[0] = acc[0];
}

// LDS fp32 atomic adds (ds_add_f32, no return) to random words of a 64 KB array.
__global__ __launch_bounds__(kThreads) void lds_atomic_kernel(float *sink, uint32_t rounds,
                                                              uint32_t seed) {
  __shared__ float acc[kLdsSpan / 4];
  for (int i = threadIdx.x; i < kLdsSpan / 4; i += kThreads) acc[i] = 0.0f;
  __syncthreads();
  uint32_t x = mix(blockIdx.x * kThreads + threadIdx.x + seed);
  for (uint32_t r = 0; r < rounds; ++r) {
    x = x * 1664525u + 1013904223u;
    atomicAdd(&acc[(x >> 8) & (kLdsSpan / 4 - 1)], 1.0f);
  }
  __syncthreads();
  if (acc[threadIdx.x] == -1.0f) sink[0] = 1.0f;
}

bool pow2(uint64_t x) { return x && !(x & (x - 1)); }

}  // namespace

extern "C" {

int msda_microbench_run(msda_microbench kind, void *buf, size_t bytes, size_t span, int reps,
                        void *stream, double *ms_per_launch, double *units_per_launch) {
  if (!buf || !ms_per_launch || !units_per_launch || reps < 1) return 1;
  if (((uintptr_t)buf & 255) != 0 || bytes < (1u << 20)) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 2;
  // the last 4 KiB of the buffer take the never-written sink
  const size_t usable = (bytes - 4096) & ~size_t(255);
  float *sink = reinterpret_cast<float *>(static_cast<char *>(buf) + usable);
  uint4 *p16 = static_cast<uint4 *>(buf);
  const unsigned stream_blocks = (unsigned)cus * 8;
  hipLaunchKernelGGL(fill_kernel, dim3(stream_blocks), dim3(kThreads), 0, s, p16, usable / 16,
                     0x1234u);
  double units = 0.0;
  auto launch = [&](int rep) {
    const uint32_t seed = 0x51ed270bu * (uint32_t)(rep + 1);
    switch (kind) {
      case MSDA_MB_READ:
        hipLaunchKernelGGL(read_kernel, dim3(stream_blocks), dim3(kThreads), 0, s, p16,
                           usable / 16, sink);
        units = (double)(usable / 16 * 16);
        break;
      case MSDA_MB_COPY: {
        const size_t half16 = usable / 32;
        hipLaunchKernelGGL(copy_kernel, dim3(stream_blocks), dim3(kThreads), 0, s, p16,
                           p16 + half16, half16);
        units = 2.0 * (double)(half16 * 16);
        break;
      }
      case MSDA_MB_ATOMIC_F32:
      case MSDA_MB_ATOMIC_PK_BF16: {
        // span: bytes of the row set the adds land on (a power of two, >= 128)
        const uint32_t rows = (uint32_t)(span / kRowBytes);
        const uint32_t rounds = 64;
        const unsigned blocks = (unsigned)cus * 16;
        if (kind == MSDA_MB_ATOMIC_F32)
          hipLaunchKernelGGL(atomic_kernel<false>, dim3(blocks), dim3(kThreads), 0, s,
                             static_cast<float *>(buf), rows - 1, rounds, seed);
        else
          hipLaunchKernelGGL(atomic_kernel<true>, dim3(blocks), dim3(kThreads), 0, s,
                             static_cast<float *>(buf), rows - 1, rounds, seed);
        units = (double)blocks * kThreads * rounds;
        break;
      }
      case MSDA_MB_GATHER_GLOBAL:
      case MSDA_MB_GATHER_LDS: {
        const unsigned blocks = (unsigned)cus * 16;
        if (kind == MSDA_MB_GATHER_GLOBAL)
          hipLaunchKernelGGL(gather_kernel<0>, dim3(blocks), dim3(kThreads), 0, s,
                             static_cast<const float *>(buf), (uint32_t)span, sink, seed);
        else
          hipLaunchKernelGGL(gather_kernel<1>, dim3(blocks), dim3(kThreads), 0, s,
                             static_cast<const float *>(buf), (uint32_t)kLdsSpan, sink, seed);
        units = (double)blocks * kThreads * kGatherIters * kGatherInflight * 16;
        break;
      }
      case MSDA_MB_LDS_ATOMIC_F32: {
        const unsigned blocks = (unsigned)cus * 8;
        const uint32_t rounds = 256;
        hipLaunchKernelGGL(lds_atomic_kernel, dim3(blocks), dim3(kThreads), 0, s, sink, rounds,
                           seed);
        units = (double)blocks * kThreads * rounds;
        break;
      }
    }
  };
  switch (kind) {
    case MSDA_MB_READ:
    case MSDA_MB_COPY:
    case MSDA_MB_LDS_ATOMIC_F32:
      break;
    case MSDA_MB_ATOMIC_F32:
    case MSDA_MB_ATOMIC_PK_BF16:
      if (!pow2(span) || span < (size_t)kRowBytes || span > usable) return 1;
      break;
    case MSDA_MB_GATHER_GLOBAL:
      if (!pow2(span) || span < 4096 || span > usable || span > (size_t(1) << 30))
        return 1;
      break;
    case MSDA_MB_GATHER_LDS:
      if (usable < (size_t)kLdsSpan) return 1;
      break;
    default:
      return 1;
  }
  launch(0);  // warm-up (also sizes `units`)
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return 2;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return 2;
  }
  (void)hipEventRecord(e0, s);
  for (int r = 1; r <= reps; ++r) launch(r);
  (void)hipEventRecord(e1, s);
  float ms = 0.0f;
  const bool ok = hipEventSynchronize(e1) == hipSuccess &&
                  hipEventElapsedTime(&ms, e0, e1) == hipSuccess && hipGetLastError() == hipSuccess;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (!ok) return 2;
  *ms_per_launch = (double)ms / reps;
  *units_per_launch = units;
  return 0;
}

}  // extern "C"
