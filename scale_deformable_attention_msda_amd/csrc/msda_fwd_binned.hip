// Query-binned MSDA forward for gfx950 (CDNA4, wave64).
//
// Computes the same operator as the direct gather (fwd_kernel): out[b, q,
// m*D + d] = sum over levels l and points k of A * bilinear(value_l, loc),
// "1. Deformable attention, from scratch" (msda-triton course, chapter 1),
// sections "The equation, term by term", "Bilinear interpolation: reading
// between the pixels" and "The simplest possible implementation".  Only the
// schedule differs.
//
// Why a second schedule.  The direct gather reads every corner row (one
// 128-byte line for fp32, D = 32) through the vector L1, whose hit path
// returns about 58 bytes per clock per CU; LDS returns about 114.  When the
// queries of a region sample the region itself (an encoder: one query per
// pyramid pixel), every value row is read ~20 times per pass, so reading it
// once into LDS and gathering from there could move the bound from the L1 to
// LDS.  On MI355X the staging, the per-sample geometry broadcasts and the sort
// passes cost more VALU time than the L1 time they save, so this schedule is
// a measured comparison (msda_forward_binned), not the default forward.
//
// Passes (one launch of nb batches):
//   count    one thread per head-query (b, q, m): its key is the bin (a square
//            of T x T pixels of the finest level) of the mean location of its K
//            points on the finest level.  A block takes 1024/M queries of one
//            batch, all heads; its LDS histograms (one per head) are stored per
//            block (no global atomics).
//   scatter  every block of a (b, m) adds up that (b, m)'s histograms, scans
//            them into bin starts and writes its query indices in bin order.
//            Block 0 of each (b, m) appends that (b, m)'s chunks (bins cut into
//            near-equal pieces of at most `quads` head-queries) to one list.
//   tile     persistent blocks of 4 * quads lanes walk the chunk list; each
//            4-lane group (quad) owns one head-query and each lane a quarter of
//            its D channels.  For every level, smallest window first, the block
//            gathers from one LDS buffer holding the window (the bin's extent on
//            that level plus R pixels, zeros outside the level) while the next
//            phase's window streams into the other.  Lane j of a quad computes
//            the geometry of points k = j, j + 4, ... once; quad broadcasts hand
//            it to the other lanes.  A sample whose cell leaves the window is
//            flagged and gathered from global memory after the chunk's last
//            level.
#include "msda_device.h"
#include "msda_launch.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace msda {
namespace {

template <typename T>
__device__ inline void ld_loc(const void *loc, uint32_t s, float &u, float &v) {
  if constexpr (sizeof(T) == 4) {
    const float2 x = reinterpret_cast<const float2 *>(loc)[s];
    u = x.x;
    v = x.y;
  } else {
    const uint32_t x = reinterpret_cast<const uint32_t *>(loc)[s];
    u = Half<T>::lo(x);
    v = Half<T>::hi(x);
  }
}

template <typename T>
__device__ inline float ld_w(const void *attn, uint32_t s) {
  return to_float<T>(reinterpret_cast<const T *>(attn)[s]);
}

// Bin (within its (b, m)) of head-query hq = (b Q + q) M + m: the finest-level
// pixel under the mean of its K finest-level points.  NaN or negative means go
// to pixel 0, means past the map to its last pixel.
template <typename T>
struct KeyPts {
  float u[8], v[8];
};

// Issue the loads of the K (<= KMAX) finest-level points of head-query hq;
// slots past K reload the last point and are masked in key_bin.
template <typename T, int KMAX>
__device__ inline void key_load(const FwdPlan &p, const void *loc, uint32_t hq, KeyPts<T> &pt) {
  const uint32_t s0 = hq * (uint32_t)(p.L * p.K) + (uint32_t)(p.f * p.K);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) ld_loc<T>(loc, s0 + (uint32_t)min(k, p.K - 1), pt.u[k], pt.v[k]);
}

template <typename T, int KMAX>
__device__ inline int key_bin(const FwdPlan &p, const KeyPts<T> &pt) {
  float su = 0.0f, sv = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    su += k < p.K ? pt.u[k] : 0.0f;
    sv += k < p.K ? pt.v[k] : 0.0f;
  }
  const float kinv = 1.0f / (float)p.K;
  const int Wf = p.W[p.f], Hf = p.H[p.f];
  float x = su * kinv * (float)Wf, y = sv * kinv * (float)Hf;
  x = x >= 0.0f ? fminf(x, (float)(Wf - 1)) : 0.0f;
  y = y >= 0.0f ? fminf(y, (float)(Hf - 1)) : 0.0f;
  const int bx = min((int)x / p.T, p.GX - 1), by = min((int)y / p.T, p.GY - 1);
  return by * p.GX + bx;
}

// Exclusive prefix sum of one value per thread over a block of NT threads
// (Hillis-Steele in LDS); *total receives the block sum.  Ends with a barrier.
template <int NT>
__device__ inline uint32_t block_excl_sum(uint32_t v, uint32_t *part, uint32_t *total) {
  part[threadIdx.x] = v;
  __syncthreads();
  for (int d = 1; d < NT; d <<= 1) {
    const uint32_t x = threadIdx.x >= (unsigned)d ? part[threadIdx.x - d] : 0u;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  const uint32_t incl = part[threadIdx.x];
  *total = part[NT - 1];
  __syncthreads();
  return incl - v;
}

// -------------------------------------------------------------- count pass

// Block (x, b) keys the head-queries of queries [x cq, x cq + cq) of batch b,
// all M heads (cq M <= 1024, one per thread): head-query i of the block is
// (q0 + i / M, i % M), so consecutive lanes read consecutive location rows.
// Keys are stored in head-query order; the histogram of every (b, m) is
// stored per block.

template <typename T, int KMAX>
__global__ __launch_bounds__(kFwdCountQ) void fwd_count_kernel(FwdArgs fa) {
  extern __shared__ uint32_t hist[];  // [M][nbm]
  const FwdPlan &p = fa.p;
  const int b = blockIdx.y;
  const int M = p.M;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *fa.w.nchunks = 0;
  for (int e = threadIdx.x; e < M * p.nbm; e += kFwdCountQ) hist[e] = 0;
  __syncthreads();
  const uint32_t q0 = blockIdx.x * (uint32_t)p.cq;
  const uint32_t n = min((uint32_t)p.cq, (uint32_t)p.Q - q0) * (uint32_t)M;
  const uint32_t hq0 = ((uint32_t)b * (uint32_t)p.Q + q0) * (uint32_t)M;
  const uint32_t i = threadIdx.x;
  KeyPts<T> pts;
  key_load<T, KMAX>(p, fa.a.loc, hq0 + min(i, n - 1), pts);
  if (i < n) {
    const int key = key_bin<T, KMAX>(p, pts);
    fa.w.keys[hq0 + i] = (uint32_t)key;
    const int m = (int)(i % (uint32_t)M);
    __hip_atomic_fetch_add(&hist[m * p.nbm + key], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < M * p.nbm; idx += kFwdCountQ) {
    const int m = idx / p.nbm, e = idx - m * p.nbm;
    fa.w.hist[(((size_t)b * M + m) * p.nqc + blockIdx.x) * p.nbm + e] = hist[idx];
  }
}

// ------------------------------------------------------------ scatter pass

__global__ __launch_bounds__(kFwdCountQ) void fwd_scatter_kernel(FwdArgs fa) {
  extern __shared__ uint32_t sm[];  // cursor, count, start: [nbm] each
  __shared__ uint32_t part[kFwdCountQ];
  __shared__ uint32_t list_off;
  const FwdPlan &p = fa.p;
  uint32_t *cur = sm, *cnt = sm + p.nbm, *bstart = sm + 2 * p.nbm;
  const int bm = blockIdx.y;
  const uint32_t *h = fa.w.hist + (size_t)bm * p.nqc * p.nbm;
  // per bin: the count of this (b, m) (cnt) and the part keyed by the count
  // blocks of earlier queries (cur); every lane adds kCols histogram entries
  // per round, their loads in flight together
  for (int e = threadIdx.x; e < p.nbm; e += kFwdCountQ) {
    cur[e] = 0;
    cnt[e] = 0;
  }
  __syncthreads();
  constexpr int kCols = 8;
  const uint32_t entries = (uint32_t)p.nqc * (uint32_t)p.nbm;
  const uint32_t first_mine = blockIdx.x * (uint32_t)(kFwdCountQ / p.cq) * (uint32_t)p.nbm;
  for (uint32_t i0 = threadIdx.x; i0 < entries; i0 += kFwdCountQ * kCols) {
    uint32_t v[kCols];
#pragma unroll
    for (int u = 0; u < kCols; ++u) v[u] = h[min(i0 + u * kFwdCountQ, entries - 1)];
#pragma unroll
    for (int u = 0; u < kCols; ++u) {
      const uint32_t idx = i0 + u * kFwdCountQ;
      if (idx >= entries || v[u] == 0) continue;
      const uint32_t e = idx % (uint32_t)p.nbm;
      __hip_atomic_fetch_add(&cnt[e], v[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (idx < first_mine)
        __hip_atomic_fetch_add(&cur[e], v[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  // bin starts: thread t owns bins [t per, t per + per)
  const int per = (p.nbm + kFwdCountQ - 1) / kFwdCountQ;
  const int e0 = min((int)threadIdx.x * per, p.nbm), e1 = min(e0 + per, p.nbm);
  uint32_t local = 0;
  for (int e = e0; e < e1; ++e) local += cnt[e];
  uint32_t total;
  uint32_t run = block_excl_sum<kFwdCountQ>(local, part, &total);
  for (int e = e0; e < e1; ++e) {
    bstart[e] = run;
    cur[e] += run;
    run += cnt[e];
  }
  __syncthreads();
  const uint32_t q = blockIdx.x * kFwdCountQ + threadIdx.x;
  uint32_t *sorted = fa.w.sorted + (size_t)bm * p.Q;
  if (q < (uint32_t)p.Q) {
    const int b = bm / p.M, m = bm - b * p.M;
    const uint32_t key = fa.w.keys[((uint32_t)b * (uint32_t)p.Q + q) * (uint32_t)p.M + m];
    const uint32_t pos =
        __hip_atomic_fetch_add(&cur[key], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    sorted[pos] = q;
  }
  if (blockIdx.x != 0) return;
  // chunk list of this (b, m): bin e in ceil(n / quads) near-equal pieces
  const uint32_t qb = (uint32_t)p.quads;
  uint32_t nch = 0;
  for (int e = e0; e < e1; ++e) nch += (cnt[e] + qb - 1) / qb;
  uint32_t all;
  uint32_t c = block_excl_sum<kFwdCountQ>(nch, part, &all);
  if (threadIdx.x == 0)
    list_off = __hip_atomic_fetch_add(fa.w.nchunks, all, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  c += list_off;
  for (int e = e0; e < e1; ++e) {
    const uint32_t n = cnt[e];
    if (n == 0) continue;
    const uint32_t pieces = (n + qb - 1) / qb;
    for (uint32_t i = 0; i < pieces; ++i) {
      const uint32_t lo = i * n / pieces, hi = (i + 1) * n / pieces;
      fa.w.chunks[c++] = make_uint4((uint32_t)bm, bstart[e] + lo, (uint32_t)e, hi - lo);
    }
  }
}

// --------------------------------------------------------------- tile pass

template <int SRC>
__device__ inline uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, SRC * 0x55, 0xF, 0xF, true);
}
template <int SRC>
__device__ inline float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), SRC * 0x55, 0xF, 0xF, true));
}

// Window of level l for bin column bx / row by: first pixel (x0w, y0w).  The
// window may reach one pixel past each side of the level (zeros there).
struct Window {
  int x0, y0, ww, wh;
};

__device__ inline Window window_of(const FwdPlan &p, int l, int bx, int by) {
  Window w;
  w.ww = p.ww[l];
  w.wh = p.wh[l];
  w.x0 = (int)floorf((float)bx * p.sx[l] - 0.5f) - p.R[l];
  w.y0 = (int)floorf((float)by * p.sy[l] - 0.5f) - p.R[l];
  w.x0 = min(max(w.x0, -1), p.W[l] + 1 - w.ww);
  w.y0 = min(max(w.y0, -1), p.H[l] + 1 - w.wh);
  return w;
}

typedef int sgpr4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (base, 32-bit record count, no swizzle) for
// the inline-asm loads below.
__device__ inline sgpr4 raw_rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  sgpr4 r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)(a >> 32) & 0xffff;
  r.z = (int)bytes;
  r.w = kRawBufferWord3;
  return r;
}

// One 16-byte direct-to-LDS buffer load per lane: lane i's bytes land at LDS
// byte lds_dst + 16 i (lds_dst is wave-uniform).  Issued as inline asm so the
// compiler does not make the gathers that follow wait for it (it cannot tell
// the two LDS buffers apart); stage_window's caller waits with vmcnt(0)
// before the barrier that publishes the window.  m0 is restored afterwards.
__device__ inline void lds_dma16(const sgpr4 &rsrc, uint32_t voff, uint32_t lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(m0)
      : "memory");
}

// Stage a window into LDS at byte `lds_buf` of the LDS space (kRow bytes per
// pixel row of head m, pixel rows in window order) with direct-to-LDS buffer
// loads: 16-byte piece idx of the window lands at lds_buf + 16 idx, so a
// wave's loads of one round fill 1 KiB of consecutive LDS.  A thread's piece
// within its row is fixed (the block size is a multiple of the pieces per
// row) and its row advances by a fixed stride each round, so the pixel index
// is kept incrementally.  Pixels outside the level read as zeros through the
// descriptor.  The caller waits (vmcnt) and synchronises.
template <int kRow, int NT>
__device__ inline void stage_window(const FwdPlan &p, const sgpr4 &rsrc, int l, const Window &w,
                                    uint32_t pix0, int m, uint32_t lds_buf, uint32_t wave_off) {
  constexpr int kPPR = kRow / 16;
  constexpr int kRowsPerRound = NT / kPPR;
  static_assert(NT % kPPR == 0, "whole rows per round");
  const int nrows = w.ww * w.wh;
  const int H = p.H[l], W = p.W[l];
  const uint32_t piece = threadIdx.x % kPPR;
  int row = (int)(threadIdx.x / kPPR);
  int wy = (int)fdiv((uint32_t)row, p.div_ww[l]);
  int wx = row - wy * w.ww;
  const int dy = kRowsPerRound / w.ww, dx = kRowsPerRound - dy * w.ww;  // stride per round
  const uint32_t mrow = (uint32_t)p.M * kRow;
  const uint32_t lane_off = (uint32_t)m * kRow + piece * 16;
#pragma unroll
  for (int t = 0; t < kFwdMaxPieces; ++t) {
    if (t * kRowsPerRound >= nrows) break;
    const int x = w.x0 + wx, y = w.y0 + wy;
    const bool in = row < nrows && (unsigned)x < (unsigned)W && (unsigned)y < (unsigned)H;
    const uint32_t off = in ? (pix0 + (uint32_t)(y * W + x)) * mrow + lane_off : kOutside;
    if (row < nrows) lds_dma16(rsrc, off, lds_buf + (uint32_t)(t * NT) * 16 + wave_off);
    row += kRowsPerRound;
    wx += dx;
    wy += dy;
    if (wx >= w.ww) {
      wx -= w.ww;
      ++wy;
    }
  }
}

// Wait for this wave's direct-to-LDS loads (vmcnt 0; expcnt and lgkmcnt
// left at their maxima), then for the whole block.
__device__ inline void staged_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

template <typename T, int N>
__device__ inline void fma_piece(const uint4 &x, float w, float *acc) {
  const uint32_t raw[4] = {x.x, x.y, x.z, x.w};
  float v[N];
  unpack<T, 4>(raw, v);
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = fmaf(w, v[i], acc[i]);
}

// One chunk of the list: batch, head, bin (column bx, row by) and the number
// of head-queries, plus where its query indices start in the sorted list.
struct Chunk {
  int b, m, bx, by, n;
  uint32_t pos;  // first sorted position within (b, m)
};

// Every field is clamped to the plan's ranges: a list written by this plan's
// scatter pass is unchanged by that, and a list left by another plan (a
// violated precondition of msda_forward_binned_reuse) cannot send an access
// out of range.
__device__ inline Chunk decode_chunk(const FwdPlan &p, const uint4 &ch) {
  Chunk c;
  const int bm = (int)min(ch.x, (uint32_t)(p.nb * p.M - 1));
  const int e = (int)min(ch.z, (uint32_t)(p.GX * p.GY - 1));
  c.b = bm / p.M;
  c.m = bm - c.b * p.M;
  c.by = e / p.GX;
  c.bx = e - c.by * p.GX;
  c.n = (int)min(ch.w, (uint32_t)p.quads);
  c.pos = min(ch.y, (uint32_t)p.Q - (uint32_t)c.n);
  return c;
}

// (u, v, A) of this lane's samples of head-query hq: level order[i], point
// j + 4 r in slot i KR + r.  All loads are issued together; dead slots (no
// head-query, a point past K, a level past L) reload sample 0 and get a NaN
// location, which places them outside every level.
template <typename T, int KR, int NS>
__device__ inline void load_slots(const FwdPlan &p, const LaunchArgs &a, uint32_t hq, bool has_q,
                                  int j, float (&su)[NS], float (&sv)[NS], float (&sa)[NS]) {
  const uint32_t LK = (uint32_t)(p.L * p.K);
#pragma unroll
  for (int i = 0; i < NS / KR; ++i) {
    const int l = p.order[i];
#pragma unroll
    for (int r = 0; r < KR; ++r) {
      const int k = j + 4 * r;
      const bool live = has_q && i < p.L && k < p.K;
      const uint32_t s = live ? hq * LK + (uint32_t)(l * p.K + k) : 0u;
      float u, v;
      ld_loc<T>(a.loc, s, u, v);
      const float A = ld_w<T>(a.attn, s);
      su[i * KR + r] = live ? u : __int_as_float(0x7fc00000);
      sv[i * KR + r] = v;
      sa[i * KR + r] = live ? A : 0.0f;
    }
  }
}

// Persistent tile pass.  The blocks of XCD x (= blockIdx % 8) share the list
// entries [x per, (x + 1) per) and take every (gridDim / 8)-th of them, so
// neighbouring bins run together on one L2.  A block streams the phases
// (chunk, level) of its chunks through two LDS window buffers: while phase p
// gathers from one buffer, the window of phase p + 1 (the next level, or the
// first level of the next chunk) streams into the other.  The next chunk's
// descriptor, query indices and locations are fetched one link per level of
// the current chunk, so no phase waits on more than one round trip.
// NS: (level, point-round) slots per lane, L * KR <= NS; NT: lanes per block.
template <typename T, int LB, int KR, int NS, int NT>
__global__ __launch_bounds__(NT) void fwd_tile_kernel(FwdArgs fa) {
  extern __shared__ __attribute__((aligned(16))) char win[];
  __shared__ int lstart[kMaxLevels];             // level_start_index
  constexpr int kRow = 4 * LB;                   // bytes of one head row
  constexpr int kPieces = LB / 16;               // 16-byte reads per lane and corner
  constexpr int kPerPiece = 16 / (int)sizeof(T); // channels per piece
  constexpr int CH = LB / (int)sizeof(T);        // channels per lane
  constexpr int kLevels = NS / KR;               // levels a lane can hold
  static_assert(NS <= kFwdMaxSlots, "slot budget");
  const FwdPlan &p = fa.p;
  const LaunchArgs &a = fa.a;

  const uint32_t nlist = min(*fa.w.nchunks, (uint32_t)p.max_chunks);
  const uint32_t per = (nlist + 7) / 8;
  const uint32_t xcd = blockIdx.x % 8, stride = gridDim.x / 8;
  const uint32_t cend = min((xcd + 1) * per, nlist);
  uint32_t ci = xcd * per + blockIdx.x / 8;
  if (ci >= cend) return;

  const int quad = threadIdx.x >> 2, j = threadIdx.x & 3;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(a.value, a.value_bytes);
  const sgpr4 rsrc_words = raw_rsrc_words(a.value, a.value_bytes);
  if (threadIdx.x < (unsigned)p.L) lstart[threadIdx.x] = (int)a.starts[threadIdx.x];
  const uint32_t win_lds =
      (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char *)win);
  const uint32_t wave_off = __builtin_amdgcn_readfirstlane(threadIdx.x & ~63u) * 16;
  // Lane j of quad q owns the 16-byte pieces j, j + 4, j + 8, ... of a head row
  // and reads them in an order rotated by q, so that the quads served together
  // by one LDS read cover all 32 banks evenly.  Read r always feeds the same
  // accumulators; only the final store address follows the rotation.
  uint32_t loff[kPieces];
  const int rot = (quad ^ (quad >> 1)) & (kPieces - 1);  // measured best of the quad-bit choices
#pragma unroll
  for (int r = 0; r < kPieces; ++r) loff[r] = (uint32_t)(16 * j + 64 * ((rot + r) % kPieces));
  const uint32_t row_stride = (uint32_t)(p.M * kRow);

  // the first chunk: descriptor, query index, locations (one exposed chain)
  Chunk C = decode_chunk(p, fa.w.chunks[ci]);
  bool has_q = quad < C.n;
  uint32_t hq;
  {
    const uint32_t q =
        has_q ? min(fa.w.sorted[((size_t)C.b * p.M + C.m) * p.Q + C.pos + quad], (uint32_t)p.Q - 1)
              : 0u;
    hq = ((uint32_t)C.b * (uint32_t)p.Q + q) * (uint32_t)p.M + (uint32_t)C.m;
  }
  float su[NS], sv[NS], sa[NS];
  load_slots<T, KR, NS>(p, a, hq, has_q, j, su, sv, sa);
  __syncthreads();  // level starts
  uint32_t par = 0;  // buffer parity of the current chunk's first level
  {
    const int l0 = p.order[0];
    stage_window<kRow, NT>(p, rsrc_words, l0, window_of(p, l0, C.bx, C.by),
                           (uint32_t)C.b * (uint32_t)p.S + lstart[l0], C.m, win_lds, wave_off);
  }
  staged_barrier();

  for (;;) {
    const uint32_t cn = ci + stride;
    const bool has_next = cn < cend;
    // next chunk, fetched one link per level
    uint4 nd = make_uint4(0, 0, 0, 0);
    Chunk N{};
    bool nhas_q = false;
    uint32_t nhq = 0;
    float nu[NS], nv[NS], na[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      nu[s] = 0.0f;
      nv[s] = 0.0f;
      na[s] = 0.0f;
    }
    const bool wave_busy = (int)(threadIdx.x >> 6) * 16 < C.n;
    const uint32_t row_base = (uint32_t)C.b * (uint32_t)p.S;
    float acc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) acc[i] = 0.0f;
    uint32_t fb = 0;  // slots i KR + r of this lane whose cell leaves the window

#pragma unroll
    for (int i = 0; i < kLevels; ++i) {
      if (i >= p.L) break;
      const int l = p.order[i];
      const bool last = i + 1 == p.L;
      // links of the next chunk: descriptor, then query index, then locations
      if (has_next && i == 0) nd = fa.w.chunks[cn];
      if (has_next && i == min(1, p.L - 1)) {
        N = decode_chunk(p, nd);
        nhas_q = quad < N.n;
        const uint32_t q =
            nhas_q ? min(fa.w.sorted[((size_t)N.b * p.M + N.m) * p.Q + N.pos + quad],
                         (uint32_t)p.Q - 1)
                   : 0u;
        nhq = ((uint32_t)N.b * (uint32_t)p.Q + q) * (uint32_t)p.M + (uint32_t)N.m;
      }
      if (has_next && i == min(2, p.L - 1)) load_slots<T, KR, NS>(p, a, nhq, nhas_q, j, nu, nv, na);
      // the window of the next phase streams in while this one is gathered
      const uint32_t buf_this = ((i + par) & 1u) ? (uint32_t)p.half : 0u;
      const uint32_t buf_next = ((i + par) & 1u) ? 0u : (uint32_t)p.half;
      if (!last) {
        const int ln = p.order[i + 1];
        stage_window<kRow, NT>(p, rsrc_words, ln, window_of(p, ln, C.bx, C.by),
                               row_base + lstart[ln], C.m, win_lds + buf_next, wave_off);
      } else if (has_next) {
        const int ln = p.order[0];
        stage_window<kRow, NT>(p, rsrc_words, ln, window_of(p, ln, N.bx, N.by),
                               (uint32_t)N.b * (uint32_t)p.S + lstart[ln], N.m,
                               win_lds + buf_next, wave_off);
      }
      if (wave_busy) {  // waves whose quads all lack a head-query skip the gather
        const Window w = window_of(p, l, C.bx, C.by);
        const char *wb = win + buf_this;
        const int H = p.H[l], W = p.W[l];
        // geometry of this lane's points on level l
        uint32_t off[KR];
        float wc[KR][4];
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          const float u = su[i * KR + r], v = sv[i * KR + r], A = sa[i * KR + r];
          const double x = (double)u * (double)W - 0.5;
          const double y = (double)v * (double)H - 0.5;
          const double xf = floor(x), yf = floor(y);
          const bool any = xf >= -1.0 && xf < (double)W && yf >= -1.0 && yf < (double)H;
          const int cx = any ? (int)xf - w.x0 : -1, cy = any ? (int)yf - w.y0 : -1;
          const bool in =
              (unsigned)cx <= (unsigned)(w.ww - 2) && (unsigned)cy <= (unsigned)(w.wh - 2);
          if (any && !in) fb |= 1u << (i * KR + r);
          const float fx = (float)(x - xf), fy = (float)(y - yf);
          off[r] = in ? (uint32_t)((cy * w.ww + cx) * kRow) : 0u;
          wc[r][0] = in ? (1.0f - fx) * (1.0f - fy) * A : 0.0f;
          wc[r][1] = in ? fx * (1.0f - fy) * A : 0.0f;
          wc[r][2] = in ? (1.0f - fx) * fy * A : 0.0f;
          wc[r][3] = in ? fx * fy * A : 0.0f;
        }
        const uint32_t dy = (uint32_t)(w.ww * kRow);
#pragma unroll
        for (int k = 0; k < 4 * KR; ++k) {
          if (k >= p.K) break;
          const int r = k >> 2;
          uint32_t o;
          float w0, w1, w2, w3;
          switch (k & 3) {
            case 0: o = quad_bcast<0>(off[r]); w0 = quad_bcast<0>(wc[r][0]); w1 = quad_bcast<0>(wc[r][1]);
                    w2 = quad_bcast<0>(wc[r][2]); w3 = quad_bcast<0>(wc[r][3]); break;
            case 1: o = quad_bcast<1>(off[r]); w0 = quad_bcast<1>(wc[r][0]); w1 = quad_bcast<1>(wc[r][1]);
                    w2 = quad_bcast<1>(wc[r][2]); w3 = quad_bcast<1>(wc[r][3]); break;
            case 2: o = quad_bcast<2>(off[r]); w0 = quad_bcast<2>(wc[r][0]); w1 = quad_bcast<2>(wc[r][1]);
                    w2 = quad_bcast<2>(wc[r][2]); w3 = quad_bcast<2>(wc[r][3]); break;
            default: o = quad_bcast<3>(off[r]); w0 = quad_bcast<3>(wc[r][0]); w1 = quad_bcast<3>(wc[r][1]);
                     w2 = quad_bcast<3>(wc[r][2]); w3 = quad_bcast<3>(wc[r][3]); break;
          }
          const char *c0 = wb + o;
#pragma unroll
          for (int pc = 0; pc < kPieces; ++pc) {
            const char *c = c0 + loff[pc];
            const uint4 v00 = *reinterpret_cast<const uint4 *>(c);
            const uint4 v01 = *reinterpret_cast<const uint4 *>(c + kRow);
            const uint4 v10 = *reinterpret_cast<const uint4 *>(c + dy);
            const uint4 v11 = *reinterpret_cast<const uint4 *>(c + dy + kRow);
            float *ap = acc + pc * kPerPiece;
            fma_piece<T, kPerPiece>(v00, w0, ap);
            fma_piece<T, kPerPiece>(v01, w1, ap);
            fma_piece<T, kPerPiece>(v10, w2, ap);
            fma_piece<T, kPerPiece>(v11, w3, ap);
          }
        }
      }
      if (!last) staged_barrier();
    }
    // samples whose cell left their window, recomputed from this lane's
    // registers and gathered from global memory, one (slot, source lane)
    // of the quad at a time
#pragma unroll
    for (int i2 = 0; i2 < kLevels; ++i2) {
      if (i2 >= p.L) break;
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const int slot = i2 * KR + r;
        uint32_t q4 = ((fb >> slot) & 1u) << j;
        q4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q4, kDppQuadXor1, 0xF, 0xF, true);
        q4 |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q4, kDppQuadXor2, 0xF, 0xF, true);
        if (q4 == 0) continue;
        const int ll = p.order[i2];
        const Level lv{p.H[ll], p.W[ll], lstart[ll], 0};
        Corners cs;
        float fx, fy;
        sample_corners(su[slot], sv[slot], lv, row_base, row_stride, (uint32_t)(C.m * kRow), cs,
                       fx, fy);
#pragma unroll
        for (int c = 0; c < 4; ++c) cs.w[c] *= sa[slot];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          if (!((q4 >> k4) & 1u)) continue;
          uint32_t o4[4];
          float w4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            switch (k4) {
              case 0: o4[c] = quad_bcast<0>(cs.off[c]); w4[c] = quad_bcast<0>(cs.w[c]); break;
              case 1: o4[c] = quad_bcast<1>(cs.off[c]); w4[c] = quad_bcast<1>(cs.w[c]); break;
              case 2: o4[c] = quad_bcast<2>(cs.off[c]); w4[c] = quad_bcast<2>(cs.w[c]); break;
              default: o4[c] = quad_bcast<3>(cs.off[c]); w4[c] = quad_bcast<3>(cs.w[c]); break;
            }
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int pc = 0; pc < kPieces; ++pc) {
              uint32_t raw[4];
              buffer_load<4>(rsrc, o4[c] + loff[pc], raw);
              fma_piece<T, kPerPiece>(make_uint4(raw[0], raw[1], raw[2], raw[3]), w4[c],
                                      acc + pc * kPerPiece);
            }
          }
        }
      }
    }
    if (has_q) {
      char *dst = reinterpret_cast<char *>(a.out) + (size_t)hq * kRow;
#pragma unroll
      for (int pc = 0; pc < kPieces; ++pc) {
        uint32_t ow[4];
        pack<T, 4>(acc + pc * kPerPiece, ow);
        global_store<4>(dst + loff[pc], ow);
      }
    }
    staged_barrier();
    if (!has_next) break;
    // the next chunk becomes the current one
    par ^= (uint32_t)(p.L & 1);
    ci = cn;
    C = N;
    has_q = nhas_q;
    hq = nhq;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      su[s] = nu[s];
      sv[s] = nv[s];
      sa[s] = na[s];
    }
  }
}

// Launch the persistent tile pass with as many blocks as fit on the device at
// once (a multiple of 8, at most one per list entry).
template <typename T, int LB, int KR, int NS, int NT>
hipError_t launch_tile_one(const FwdArgs &fa, hipStream_t s) {
  auto kernel = fwd_tile_kernel<T, LB, KR, NS, NT>;
  const size_t lds = (size_t)fa.p.lds_bytes;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NT, lds);
  if (e != hipSuccess) return e;
  const int64_t resident = (int64_t)std::max(1, cus * std::max(1, per_cu));
  const int64_t grid = std::min((resident + 7) / 8 * 8, ((int64_t)fa.p.max_chunks + 7) / 8 * 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NT), lds, s, fa);
  return hipGetLastError();
}

template <typename T, int LB, int NT>
hipError_t launch_tile_kr(const FwdArgs &fa, hipStream_t s) {
  if (fa.p.KR == 1 && fa.p.L <= 4) return launch_tile_one<T, LB, 1, 4, NT>(fa, s);
  if (fa.p.KR == 1) return launch_tile_one<T, LB, 1, 8, NT>(fa, s);
  return launch_tile_one<T, LB, 2, 8, NT>(fa, s);
}

template <typename T, int LB>
hipError_t launch_tile_nt(const FwdArgs &fa, hipStream_t s) {
  return fa.p.quads == 128 ? launch_tile_kr<T, LB, 512>(fa, s) : launch_tile_kr<T, LB, 1024>(fa, s);
}

template <typename T>
hipError_t launch_tile_pass(const FwdArgs &fa, hipStream_t s) {
  const int row = fa.p.D * (int)sizeof(T);
  hipError_t e;
  prof_begin(s, "fwd_tile");
  switch (row) {
    case 64: e = launch_tile_nt<T, 16>(fa, s); break;
    case 128: e = launch_tile_nt<T, 32>(fa, s); break;
    case 256:
      if constexpr (sizeof(T) == 4) {
        e = launch_tile_nt<T, 64>(fa, s);
        break;
      }
      [[fallthrough]];
    default: e = hipErrorInvalidValue; break;
  }
  prof_end(s, "fwd_tile");
  return e;
}

// reuse_order: skip the sort and walk the chunk list already in the workspace
template <typename T>
hipError_t launch_binned_t(const FwdArgs &fa, bool reuse_order, hipStream_t s) {
  const FwdPlan &p = fa.p;
  if (reuse_order) return launch_tile_pass<T>(fa, s);
  const dim3 grid((unsigned)p.nqb, (unsigned)(p.nb * p.M));
  hipError_t e;
  prof_begin(s, "fwd_count");
  const dim3 cgrid((unsigned)p.nqc, (unsigned)p.nb);
  const size_t clds = (size_t)p.M * p.nbm * 4;
  if (p.K <= 4)
    hipLaunchKernelGGL((fwd_count_kernel<T, 4>), cgrid, dim3(kFwdCountQ), clds, s, fa);
  else
    hipLaunchKernelGGL((fwd_count_kernel<T, 8>), cgrid, dim3(kFwdCountQ), clds, s, fa);
  prof_end(s, "fwd_count");
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(s, "fwd_scatter");
  hipLaunchKernelGGL(fwd_scatter_kernel, grid, dim3(kFwdCountQ), (size_t)p.nbm * 12, s, fa);
  prof_end(s, "fwd_scatter");
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_tile_pass<T>(fa, s);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t fwd_layout(const FwdPlan &p, FwdScratch *w, char *base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return base ? base + o : nullptr;
  };
  const size_t hqs = (size_t)p.nb * p.M * p.Q;
  char *keys = take(hqs * 4);
  char *hist = take((size_t)p.nb * p.M * p.nqc * p.nbm * 4);
  char *sorted = take(hqs * 4);
  char *nch = take(4);
  char *chunks = take((size_t)p.max_chunks * 16);
  if (w) {
    w->keys = reinterpret_cast<uint32_t *>(keys);
    w->hist = reinterpret_cast<uint32_t *>(hist);
    w->sorted = reinterpret_cast<uint32_t *>(sorted);
    w->nchunks = reinterpret_cast<uint32_t *>(nch);
    w->chunks = reinterpret_cast<uint4 *>(chunks);
  }
  return off;
}

// LDS a gfx950 workgroup may allocate (160 KiB), less the kernel's static LDS.
constexpr int kLdsLimit = 160 * 1024 - 1024;

}  // namespace

bool make_fwd_plan(FwdPlan &p, int64_t nb, int64_t Q, int64_t S, int M, int D, int L, int K,
                   int elt, const int64_t *shapes_host) {
  std::memset(&p, 0, sizeof(p));
  const int row = D * elt;
  if (!shapes_host || (row != 64 && row != 128 && row != 256)) return false;
  if (K > 8 || L > kMaxLevels) return false;
  const int KR = (K + 3) / 4;
  if (L * KR > kFwdMaxSlots || L * K > 64) return false;
  if (nb * M > 65535 || nb * Q * M * L * K >= (int64_t(1) << 31) || Q < 1) return false;
  p.Q = Q;
  p.S = S;
  p.nb = (int)nb;
  p.M = M;
  p.D = D;
  p.L = L;
  p.K = K;
  p.KR = KR;
  int64_t best = -1;
  for (int l = 0; l < L; ++l) {
    const int64_t h = shapes_host[2 * l], w = shapes_host[2 * l + 1];
    if (h < 1 || w < 1 || h > (1 << 20) || w > (1 << 20)) return false;
    p.H[l] = (int)h;
    p.W[l] = (int)w;
    if (h * w > best) {
      best = h * w;
      p.f = l;
    }
  }
  const int Hf = p.H[p.f], Wf = p.W[p.f];
  const double density = (double)Q / ((double)Hf * (double)Wf);
  // Two tile-block shapes: 512 lanes (128 head-queries) whose windows fit in
  // half of a CU's LDS, so that two blocks share a CU and cover each other's
  // barriers and load latency; else 1024 lanes (256) with up to all of it.
  // The bin edge T aims at ~85% of the quads busy when the queries cover the
  // finest level evenly.
  constexpr int kShapes = 2;
  const int shape_quads[kShapes] = {128, 256};
  const int shape_lds[kShapes] = {kLdsLimit / 2 - 512, kLdsLimit};
  bool planned = false;
  for (int sh = 0; sh < kShapes && !planned; ++sh) {
    const int quads = shape_quads[sh];
    int T = (int)std::floor(std::sqrt(0.85 * quads / density));
    T = std::max(4, std::min(T, 64));
    for (; T >= 4; --T) {
      p.T = T;
      p.GX = (Wf + T - 1) / T;
      p.GY = (Hf + T - 1) / T;
      p.nbm = p.GX * p.GY;
      if (p.nbm > kFwdMaxBinsBM || M * p.nbm > kFwdMaxBinsBM * 3) break;
      bool fits = true;
      int bytes[kMaxLevels];
      for (int l = 0; l < L; ++l) {
        p.sx[l] = (float)((double)T * p.W[l] / Wf);
        p.sy[l] = (float)((double)T * p.H[l] / Hf);
        // margin: 4 pixels on every level (measured: wider margins on the
        // coarse levels miss fewer points but force a smaller bin and cost more)
        p.R[l] = 4;
        p.ww[l] = std::min((int)std::ceil(p.sx[l]) + 2 * p.R[l] + 2, p.W[l] + 2);
        p.wh[l] = std::min((int)std::ceil(p.sy[l]) + 2 * p.R[l] + 2, p.H[l] + 2);
        p.div_ww[l] = make_fastdiv((uint32_t)p.ww[l]);
        bytes[l] = p.ww[l] * p.wh[l] * row;
        if (bytes[l] > kFwdMaxPieces * 4 * quads * 16) fits = false;
        p.order[l] = l;
      }
      if (!fits) continue;
      std::stable_sort(p.order, p.order + L, [&](int x, int y) { return bytes[x] < bytes[y]; });
      // windows alternate between two buffers phase by phase; with an even L a
      // level keeps its buffer from chunk to chunk, with an odd L it swaps
      int even = 0, odd = 0, widest = 0;
      for (int i = 0; i < L; ++i) {
        (i % 2 ? odd : even) = std::max(i % 2 ? odd : even, bytes[p.order[i]]);
        widest = std::max(widest, bytes[p.order[i]]);
      }
      if (L % 2) even = odd = widest;
      p.half = even;
      p.lds_bytes = even + odd;
      if (p.lds_bytes > shape_lds[sh]) continue;
      // staging must stay well below the gathers it replaces
      const double per_bin = std::min((double)quads, (double)Q / p.nbm);
      double staged = 0;
      for (int l = 0; l < L; ++l) staged += (double)p.ww[l] * p.wh[l];
      if (staged > 0.5 * per_bin * L * K * 4) break;
      p.quads = quads;
      planned = true;
      break;
    }
  }
  if (!planned) return false;
  p.nqb = (int)((Q + kFwdCountQ - 1) / kFwdCountQ);
  p.cq = kFwdCountQ;
  while (p.cq > 1 && p.cq * M > kFwdCountQ) p.cq /= 2;
  p.nqc = (int)((Q + p.cq - 1) / p.cq);
  const int64_t chunks = nb * M * (p.nbm + (Q + p.quads - 1) / p.quads);
  if (chunks > (int64_t(1) << 28)) return false;
  p.max_chunks = (int)chunks;
  return true;
}

size_t fwd_workspace_bytes(const FwdPlan &p) { return fwd_layout(p, nullptr, nullptr); }

FwdScratch carve_fwd_scratch(const FwdPlan &p, void *workspace) {
  FwdScratch w{};
  fwd_layout(p, &w, static_cast<char *>(workspace));
  return w;
}

hipError_t launch_forward_binned(const FwdArgs &fa, Dtype dt, bool reuse_order,
                                 hipStream_t stream) {
  switch (dt) {
    case Dtype::F32: return launch_binned_t<float>(fa, reuse_order, stream);
    case Dtype::BF16: return launch_binned_t<bf16_t>(fa, reuse_order, stream);
    case Dtype::F16: return launch_binned_t<f16_t>(fa, reuse_order, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace msda
