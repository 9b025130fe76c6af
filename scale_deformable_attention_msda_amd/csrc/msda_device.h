// Device-side building blocks of the MSDA kernels for gfx950 (CDNA4, wave64).
//
// Operator definition: "1. Deformable attention, from scratch" (msda-triton
// course, chapter 1), sections "Bilinear interpolation: reading between the
// pixels" (corners, weights, pixel-centre mapping, zero padding) and "The
// simplest possible implementation" (floor, per-corner bounds test, row index
// start_l + yy*W_l + xx of the flattened pyramid).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

// Byte offset used for a corner outside its level.  Every launch keeps the
// value image it addresses below 2^30 bytes, so this offset (and twice it, the
// fp32-workspace offset of a bf16 corner) lies past the end of every buffer
// descriptor: buffer loads there return 0 and buffer atomics there are dropped
// by the hardware, with no memory access.
constexpr uint32_t kOutside = 0xC0000000u;

// Word 3 of a gfx9 raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kRawBufferWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}

// One pyramid level, staged in LDS by every block.
struct Level {
  int H, W, start, pad;
};

// Per-sample geometry handed from the sample lanes to the channel lanes.
struct Corners {
  uint32_t off[4];  // byte offset of corner 00, 01, 10, 11 (head row), or kOutside
  float w[4];       // bilinear weight of each corner (0 when outside)
};

// Geometry of one sample at normalised (u, v) on level `lv`.
//   x = u*W - 0.5, y = v*H - 0.5 (pixel-centre mapping), x0 = floor(x),
//   lx = x - x0; corners (y0,x0) (y0,x0+1) (y0+1,x0) (y0+1,x0+1) with weights
//   (1-lx)(1-ly), lx(1-ly), (1-lx)ly, lx*ly.
// The coordinate and its floor are taken in fp64: u*W is exact there (a 24-bit
// significand times an integer below 2^29), so the cell a point falls in is
// the exact one.  The fraction is then rounded once to fp32 for the weights.
// The range test runs on the floating-point cell before any integer
// conversion, so NaN / Inf / huge coordinates yield "no corner inside".
// `row_base` is the first pyramid row of this sample's batch image within the
// launch, `row_stride` the bytes of one pyramid row (M*D*sizeof(T)) and
// `head_off` the byte offset of head m inside a row.
// Returns false when no corner lies inside the level.
__device__ inline bool sample_corners(float u, float v, const Level &lv, uint32_t row_base,
                                      uint32_t row_stride, uint32_t head_off, Corners &cs,
                                      float &lx, float &ly) {
  const double x = (double)u * (double)lv.W - 0.5;
  const double y = (double)v * (double)lv.H - 0.5;
  const double xf = floor(x);
  const double yf = floor(y);
  const bool any = xf >= -1.0 && xf < (double)lv.W && yf >= -1.0 && yf < (double)lv.H;
  if (!any) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      cs.off[c] = kOutside;
      cs.w[c] = 0.0f;
    }
    lx = 0.0f;
    ly = 0.0f;
    return false;
  }
  const int x0 = (int)xf;
  const int y0 = (int)yf;
  const float fx = (float)(x - xf);
  const float fy = (float)(y - yf);
  const bool xin0 = x0 >= 0, xin1 = x0 + 1 < lv.W;
  const bool yin0 = y0 >= 0, yin1 = y0 + 1 < lv.H;
  const uint32_t r00 = row_base + (uint32_t)lv.start + (uint32_t)(y0 * lv.W + x0);
  const uint32_t b00 = r00 * row_stride + head_off;
  const uint32_t bW = (uint32_t)lv.W * row_stride;
  cs.off[0] = (xin0 && yin0) ? b00 : kOutside;
  cs.off[1] = (xin1 && yin0) ? b00 + row_stride : kOutside;
  cs.off[2] = (xin0 && yin1) ? b00 + bW : kOutside;
  cs.off[3] = (xin1 && yin1) ? b00 + bW + row_stride : kOutside;
  cs.w[0] = (xin0 && yin0) ? (1.0f - fx) * (1.0f - fy) : 0.0f;
  cs.w[1] = (xin1 && yin0) ? fx * (1.0f - fy) : 0.0f;
  cs.w[2] = (xin0 && yin1) ? (1.0f - fx) * fy : 0.0f;
  cs.w[3] = (xin1 && yin1) ? fx * fy : 0.0f;
  lx = fx;
  ly = fy;
  return true;
}

// ------------------------------------------------------- integer division

// Division of a 32-bit unsigned numerator by a divisor fixed at launch time,
// as a multiply-high, an add and a shift (exact for every 32-bit numerator):
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// n / d = (mulhi(n, m) + n) >> s.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while (s < 32 && (uint64_t(1) << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ inline uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

// ---------------------------------------------------------------- dtypes

struct bf16_t {
  uint16_t bits;
};
struct f16_t {  // IEEE binary16
  uint16_t bits;
};

template <typename T>
__device__ inline float to_float(T x);
template <>
__device__ inline float to_float<float>(float x) { return x; }
template <>
__device__ inline float to_float<bf16_t>(bf16_t x) {
  return __uint_as_float((uint32_t)x.bits << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ inline uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// The 16-bit storage types: the fp32 value of the low and the high half of a
// 32-bit word, and the bits of an fp32 rounded to the type (nearest even).
template <typename T>
struct Half;
template <>
struct Half<bf16_t> {
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static uint32_t bits(float x) { return bf16_bits_rne(x); }
};
template <>
struct Half<f16_t> {
  __device__ static float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  // the hardware conversion rounds to nearest even (overflow to infinity)
  __device__ static uint32_t bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};

template <>
__device__ inline float to_float<f16_t>(f16_t x) { return Half<f16_t>::lo(x.bits); }

template <typename T>
__device__ inline void store_scalar(T *p, float x);
template <>
__device__ inline void store_scalar<float>(float *p, float x) { *p = x; }
template <>
__device__ inline void store_scalar<bf16_t>(bf16_t *p, float x) {
  p->bits = (uint16_t)bf16_bits_rne(x);
}
template <>
__device__ inline void store_scalar<f16_t>(f16_t *p, float x) {
  p->bits = (uint16_t)Half<f16_t>::bits(x);
}

// Two consecutive elements (p 8-byte aligned for fp32, 4-byte aligned for 16-bit types).
template <typename T>
__device__ inline void store_pair(T *p, float x, float y);
template <>
__device__ inline void store_pair<float>(float *p, float x, float y) {
  *reinterpret_cast<float2 *>(p) = make_float2(x, y);
}
template <>
__device__ inline void store_pair<bf16_t>(bf16_t *p, float x, float y) {
  *reinterpret_cast<uint32_t *>(p) = bf16_bits_rne(x) | (bf16_bits_rne(y) << 16);
}
template <>
__device__ inline void store_pair<f16_t>(f16_t *p, float x, float y) {
  *reinterpret_cast<uint32_t *>(p) = Half<f16_t>::bits(x) | (Half<f16_t>::bits(y) << 16);
}

// Unpack the 32-bit words of a row slice into fp32 channels.
template <typename T, int WORDS>
__device__ inline void unpack(const uint32_t (&w)[WORDS], float *out);

template <>
__device__ inline void unpack<float, 1>(const uint32_t (&w)[1], float *o) { o[0] = __uint_as_float(w[0]); }
template <>
__device__ inline void unpack<float, 2>(const uint32_t (&w)[2], float *o) {
  o[0] = __uint_as_float(w[0]);
  o[1] = __uint_as_float(w[1]);
}
template <>
__device__ inline void unpack<float, 4>(const uint32_t (&w)[4], float *o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(w[i]);
}
template <typename H, int WORDS>
__device__ inline void unpack_half(const uint32_t (&w)[WORDS], float *o) {
#pragma unroll
  for (int i = 0; i < WORDS; ++i) {
    o[2 * i] = Half<H>::lo(w[i]);
    o[2 * i + 1] = Half<H>::hi(w[i]);
  }
}
template <>
__device__ inline void unpack<bf16_t, 1>(const uint32_t (&w)[1], float *o) { unpack_half<bf16_t, 1>(w, o); }
template <>
__device__ inline void unpack<bf16_t, 2>(const uint32_t (&w)[2], float *o) { unpack_half<bf16_t, 2>(w, o); }
template <>
__device__ inline void unpack<bf16_t, 4>(const uint32_t (&w)[4], float *o) { unpack_half<bf16_t, 4>(w, o); }
template <>
__device__ inline void unpack<f16_t, 1>(const uint32_t (&w)[1], float *o) { unpack_half<f16_t, 1>(w, o); }
template <>
__device__ inline void unpack<f16_t, 2>(const uint32_t (&w)[2], float *o) { unpack_half<f16_t, 2>(w, o); }
template <>
__device__ inline void unpack<f16_t, 4>(const uint32_t (&w)[4], float *o) { unpack_half<f16_t, 4>(w, o); }

// Range-checked load of WORDS dwords at byte offset `off` of a buffer.
template <int WORDS>
__device__ inline void buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[WORDS]);
template <>
__device__ inline void buffer_load<1>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[1]) {
  w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
template <>
__device__ inline void buffer_load<2>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[2]) {
  typedef uint32_t v2 __attribute__((ext_vector_type(2)));
  v2 x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  w[0] = x.x;
  w[1] = x.y;
}
template <>
__device__ inline void buffer_load<4>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[4]) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  w[0] = x.x;
  w[1] = x.y;
  w[2] = x.z;
  w[3] = x.w;
}

// Plain vector load / store of WORDS dwords (16-byte aligned rows).
template <int WORDS>
__device__ inline void global_load(const void *p, uint32_t (&w)[WORDS]) {
  if constexpr (WORDS == 4) {
    uint4 x = *reinterpret_cast<const uint4 *>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (WORDS == 2) {
    uint2 x = *reinterpret_cast<const uint2 *>(p);
    w[0] = x.x; w[1] = x.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  }
}
template <int WORDS>
__device__ inline void global_store(void *p, const uint32_t (&w)[WORDS]) {
  if constexpr (WORDS == 4) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (WORDS == 2) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
  } else {
    *reinterpret_cast<uint32_t *>(p) = w[0];
  }
}

// Pack fp32 channels into the storage words of T.
template <typename T, int WORDS>
__device__ inline void pack(const float *x, uint32_t (&w)[WORDS]) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < WORDS; ++i) w[i] = __float_as_uint(x[i]);
  } else {
#pragma unroll
    for (int i = 0; i < WORDS; ++i) w[i] = Half<T>::bits(x[2 * i]) | (Half<T>::bits(x[2 * i + 1]) << 16);
  }
}

// ------------------------------------------------------------ reductions

// Workgroup barrier for data handed between waves through LDS only: unlike
// __syncthreads() it does not wait for the wave's outstanding global stores.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// DPP lane moves inside a 16-lane row (gfx9 encodings of dpp_ctrl).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppQuadXor3 = 0x1B;       // quad_perm [3,2,1,0]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within 16

template <int CTRL>
__device__ inline float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over an aligned group of G (4, 8 or 16) lanes; every lane of the group
// receives the same, bit-identical total (each step adds a commuted pair).
template <int G>
__device__ inline float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
  x += dpp_move<kDppQuadXor1>(x);
  x += dpp_move<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp_move<kDppRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_move<kDppRowMirror>(x);
  return x;
}

template <int CTRL>
__device__ inline double dpp_move_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}

// fp64 sum over an aligned group of G lanes (same pattern as group_sum).
template <int G>
__device__ inline double group_sum_f64(double x) {
  static_assert(G == 4 || G == 8 || G == 16, "group of 4, 8 or 16 lanes");
  x += dpp_move_f64<kDppQuadXor1>(x);
  x += dpp_move_f64<kDppQuadXor2>(x);
  if constexpr (G >= 8) x += dpp_move_f64<kDppRowHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_move_f64<kDppRowMirror>(x);
  return x;
}

// "softmax" method (DeformOps documentation, section "Multi-scale deformable
// attention"): the lanes of an aligned group of lk lanes (lk a power of two, at
// most 64) hold the lk logits of one head-query; each lane returns its weight
// exp(z - max) / sum over the group.  A NaN or +Inf logit, or all -Inf, makes
// the group's weights NaN, as the definition does.
// Groups of up to 16 lanes combine by DPP moves inside a row (pairs, quads,
// mirrored halves, mirrored rows: every lane ends with the whole group);
// groups of 32 and 64 by lane shuffles.
template <bool MAX>
__device__ inline float group_reduce(float x, int lk) {
  auto op = [](float a, float b) { return MAX ? (b > a ? b : a) : a + b; };
  if (lk <= 16) {
    if (lk >= 2) x = op(x, dpp_move<kDppQuadXor1>(x));
    if (lk >= 4) x = op(x, dpp_move<kDppQuadXor2>(x));
    if (lk >= 8) x = op(x, dpp_move<kDppRowHalfMirror>(x));
    if (lk >= 16) x = op(x, dpp_move<kDppRowMirror>(x));
  } else {
    for (int off = 1; off < lk; off <<= 1) x = op(x, __shfl_xor(x, off));
  }
  return x;
}

__device__ inline float group_softmax(float z, int lk) {
  const float mx = group_reduce<true>(z, lk);
  const float e = expf(z - mx);
  return e * (1.0f / group_reduce<false>(e, lk));
}

// ----------------------------------------------------------- lane layout

// How a head row (D channels of T) is spread over a group of lanes: each lane
// owns VEC consecutive channels (WORDS dwords, at most 16 bytes), and a group
// of G = 4, 8 or 16 lanes covers one row with one coalesced load.
template <typename T, int D>
struct RowLayout {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kLaneBytes = kRowBytes >= 64 ? 16 : kRowBytes / 4;
  static constexpr int G = kRowBytes / kLaneBytes;
  static constexpr int WORDS = kLaneBytes / 4;
  static constexpr int VEC = kLaneBytes / (int)sizeof(T);
  static_assert(G == 4 || G == 8 || G == 16, "unsupported row layout");
};

}  // namespace msda
