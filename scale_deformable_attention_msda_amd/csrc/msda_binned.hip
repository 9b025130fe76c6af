// Destination-binned MSDA backward for gfx950: grad_value without global
// floating-point atomics.
//
// The gradients are those of <out, grad_out> for the operator of "1.
// Deformable attention, from scratch" (msda-triton course, chapter 1):
//   p_c         = <grad_out[b,q,m,:], V_c>           (V_c = corner row, 0 outside)
//   grad_attn   = sum_c w_c p_c
//   grad_loc_x  = A * W * ((1-ly)(p01-p00) + ly(p11-p10))
//   grad_loc_y  = A * H * ((1-lx)(p10-p00) + lx(p11-p01))
//   grad_value[row_c] += A * w_c * grad_out[b,q,m,:]
// The pages' kernels scatter grad_value with global atomics ("Efficient
// Multi-Scale Deformable Attention on GPUs", section "The backward pass is an
// atomics problem").  On this GPU a device-scope fp32 atomic add sustains far
// fewer updates per second than the gather side needs, so this path first
// sorts the samples by destination and then accumulates each tile of
// grad_value in LDS, writing every row once with plain stores:
//   count    per-block LDS histogram of samples per bin, one global integer
//            atomic per touched bin (dead samples get zero gradients here);
//   plan     blocks of kPlanBlock bins, chained by a decoupled look-back:
//            exclusive scans -> bin starts, chunks of <= `chunk` samples per
//            bin with each chunk's bin position, partial-tile slots for bins
//            split in chunks;
//   scatter  recount in LDS, reserve each block's range per bin with one
//            atomic, write a 16-byte record (id, location, weight) of every
//            sample in bin order, so the tile pass reads its samples
//            contiguously instead of gathering 8- and 4-byte pieces;
//   tile     persistent blocks, one chunk at a time (the next chunk's records
//            and value rows are loaded while the current one writes its
//            results): stage the (T+1)^2 value rows of the tile
//            (plus rim) in LDS, counting-sort the chunk's samples by their
//            bilinear cell (integer LDS atomics), cut each cell's samples
//            into pieces, then one lane group per piece keeps the cell's four
//            corner rows and four accumulators in registers while it walks
//            the piece's samples: p_c, grad_loc, grad_attn, and A * w_c *
//            grad_out summed in registers.  Each piece stores its four sums
//            once to LDS; every pixel then adds the pieces of the (up to
//            four) cells around it.  Interior rows go straight to
//            grad_value, edge / rim rows (or the whole partial tile of a
//            split bin) to scratch.  No floating-point atomics: on this GPU
//            they are an order of magnitude slower than plain LDS traffic;
//   merge    one block per bin: add the neighbours' rims and the partial
//            tiles into the rows still missing, store them once.
#include "msda_device.h"
#include "msda_launch.h"

#include <algorithm>
#include <cstring>

namespace msda {
namespace {

// Tuning constants (the sweep builds variants with -D overrides).
#ifndef MSDA_BIN_TILE
#define MSDA_BIN_TILE 8
#endif
#ifndef MSDA_BIN_CHUNK
#define MSDA_BIN_CHUNK 1024
#endif
#ifndef MSDA_COUNT_SAMPLES
#define MSDA_COUNT_SAMPLES 4096
#endif
constexpr int kTile = MSDA_BIN_TILE;          // tile edge in pixels
constexpr int kEdge = kTile + 1;              // tile plus its one-pixel rim, per side
constexpr int kCells = kEdge * kEdge;         // bilinear cells whose top-left corner is in [-1, T)
constexpr int kChunk = MSDA_BIN_CHUNK;        // samples per tile-kernel block at most
constexpr int kCountSamples = MSDA_COUNT_SAMPLES;  // samples per count / scatter block
// wave 0 of the tile kernel plans with two cells per lane, cells j and j + 64
// of lane j, and indexes the first 64 cells and items without a bound check, so
// the tile holds 64..128 cells; the item fields hold 10-bit positions; count and
// scatter threads own whole rounds of 256 samples
static_assert(kCells >= 64 && kCells <= 128, "tile edge 7..10");
static_assert(kChunk % 256 == 0 && kChunk <= 1024, "chunk a multiple of 256, at most 1024");
static_assert(kCountSamples % 256 == 0 && kCountSamples <= 16384, "count block of 256..16384");
constexpr int kHistLdsBytes = 48 * 1024;
// Per-bin counters are striped over kStripes addresses (block index modulo
// kStripes): a coarse-level bin collects counts from ~100 blocks, and integer
// atomics on one address from many blocks serialize.
constexpr int kStripes = 8;
// Every (bin, stripe) counter sits on a 64-byte line of its own: device-scope
// atomics execute at the memory side one line at a time, so counters sharing
// a line would serialize the blocks that update different ones.
constexpr int kCounterWords = 16;
__host__ __device__ inline size_t counter_index(int bin, int stripe) {
  return ((size_t)bin * kStripes + stripe) * kCounterWords;
}
constexpr uint32_t kNoSlot = 0xffffffffu;

// -------------------------------------------------------------- geometry

struct Cell {
  int x0, y0;     // top-left corner of the bilinear cell
  float lx, ly;   // fractional parts
};

// Cell of normalised (u, v) on an H x W level: x = u*W - 0.5, y = v*H - 0.5,
// x0 = floor(x).  Coordinates are formed and floored in fp64, where u*W is
// exact, so the cell is the exact one.  Returns false when no corner of the
// cell lies inside the map (also for NaN / Inf / huge coordinates).
__device__ inline bool cell_of(float u, float v, int H, int W, Cell &c) {
  const double x = (double)u * (double)W - 0.5;
  const double y = (double)v * (double)H - 0.5;
  const double xf = floor(x), yf = floor(y);
  if (!(xf >= -1.0 && xf < (double)W && yf >= -1.0 && yf < (double)H)) return false;
  c.x0 = (int)xf;
  c.y0 = (int)yf;
  c.lx = (float)(x - xf);
  c.ly = (float)(y - yf);
  return true;
}

template <typename T>
__device__ inline float ldf(const void *base, int64_t i) {
  return to_float<T>(reinterpret_cast<const T *>(base)[i]);
}

// Per-level plan entries, staged in LDS at block start: indexing the kernel
// argument's arrays with a per-sample level would turn every access into a
// dependent load from the argument segment.
struct LevelTab {
  int H, W, ntx, ntiles, tile_off, bin_base;
};

__device__ inline void stage_level_tab(const BinPlan &p, LevelTab *t) {
  if (threadIdx.x < (unsigned)p.L) {
    const int l = threadIdx.x;
    t[l] = LevelTab{p.H[l], p.W[l], p.ntx[l], p.ntiles[l], p.tile_off[l], p.bin_base[l]};
  }
}

// Global bin of histogram slot e (a tile of one head, levels coarsest first)
// of batch b, head m.
__device__ inline int bin_of_slot(const BinPlan &p, const LevelTab *lt, int bm, int e) {
  int l = 0;
  while (l + 1 < p.L && !(e >= lt[l].tile_off && e < lt[l].tile_off + lt[l].ntiles)) ++l;
  return lt[l].bin_base + bm * lt[l].ntiles + (e - lt[l].tile_off);
}

// The count and scatter passes walk the samples of one (batch b, head m):
// t = q * (L K) + j over the queries q and points j, sample id
// ((b Q + q) M + m) (L K) + j.  A thread's samples t0 + 256 r (r = 0, 1, ...)
// advance j and the id by fixed steps instead of dividing t for every sample.
struct SampleWalk {
  uint32_t j, id;
};

__device__ inline SampleWalk walk_start(const BinPlan &p, int b, int m, uint32_t t) {
  const uint32_t LK = (uint32_t)(p.L * p.K);
  const uint32_t q = fdiv(t, p.div_lk);
  SampleWalk w;
  w.j = t - q * LK;
  w.id = (((uint32_t)b * (uint32_t)p.Q + q) * (uint32_t)p.M + (uint32_t)m) * LK + w.j;
  return w;
}

__device__ inline void walk_step(const BinPlan &p, SampleWalk &w) {
  w.j += p.step_j;
  w.id += p.step_id;
  if (w.j >= (uint32_t)(p.L * p.K)) {  // one more query: j wraps, the id skips the other heads
    w.j -= (uint32_t)(p.L * p.K);
    w.id += p.wrap_id;
  }
}

// Histogram slot (tile of the head, levels coarsest first) of the walk's
// current sample at normalised (u, v), or -1 for a dead sample (no corner
// inside its level).  The level is j / K through a 16-bit fixed-point
// reciprocal (exact for j < L K <= 64).
__device__ inline int slot_of_sample(const BinPlan &p, const LevelTab *lt, const SampleWalk &w,
                                     float u, float v) {
  const LevelTab t = lt[__umul24(w.j, p.magic_k) >> 16];
  Cell c;
  if (!cell_of(u, v, t.H, t.W, c)) return -1;
  const uint32_t x = (uint32_t)max(c.x0, 0), y = (uint32_t)max(c.y0, 0);
  return t.tile_off + (int)(__umul24(y / kTile, (uint32_t)t.ntx) + x / kTile);
}

// Sampling location of sample `id` (both coordinates in one load).
template <typename T>
__device__ inline void load_loc(const void *loc, int64_t id, float &u, float &v) {
  if constexpr (sizeof(T) == 4) {
    const float2 x = reinterpret_cast<const float2 *>(loc)[id];
    u = x.x;
    v = x.y;
  } else {
    const uint32_t x = reinterpret_cast<const uint32_t *>(loc)[id];
    u = Half<T>::lo(x);
    v = Half<T>::hi(x);
  }
}

// --------------------------------------------------------------- count pass

// Every thread owns kPer samples t0 + r*256 of its block's (batch, head); all their locations
// are loaded before any is used, so the loads overlap.
constexpr int kPer = kCountSamples / 256;

template <typename T>
__global__ __launch_bounds__(256) void count_kernel(BinArgs a) {
  extern __shared__ uint32_t hist[];
  const BinPlan &p = a.p;
  const int bm = blockIdx.y;  // batch * M + head
  const int b = bm / p.M, m = bm - b * p.M;
  const int stripe = (int)((blockIdx.x + blockIdx.y * gridDim.x) % kStripes);
  __shared__ LevelTab lt[kMaxLevels];
  stage_level_tab(p, lt);
  const uint32_t per_head = (uint32_t)p.Q * (uint32_t)(p.L * p.K);  // samples of one (batch, head)
  const uint32_t t0 = blockIdx.x * kCountSamples + threadIdx.x;
  for (int e = threadIdx.x; e < p.tiles_bm; e += blockDim.x) hist[e] = 0;
  // the plan was made from the host's copy of the level shapes: block (0, 0)
  // compares it with the device's spatial_shapes and level_start_index
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < (unsigned)p.L) {
    const int l = threadIdx.x;
    if (a.shapes[2 * l] != p.H[l] || a.shapes[2 * l + 1] != p.W[l] || a.starts[l] != p.start[l])
      __hip_atomic_fetch_or(a.w.error, kBinErrShapes, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // all kPer loads in flight together (samples past the head's end reload its
  // first one); each sample is binned as soon as its own load has arrived
  const uint32_t first_id = ((uint32_t)b * (uint32_t)p.Q * (uint32_t)p.M + (uint32_t)m) *
                            (uint32_t)(p.L * p.K);
  float u[kPer], v[kPer];
  {
    SampleWalk w = walk_start(p, b, m, t0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      load_loc<T>(a.loc, t0 + r * 256 < per_head ? w.id : first_id, u[r], v[r]);
      walk_step(p, w);
    }
  }
  SampleWalk w = walk_start(p, b, m, t0);
  uint32_t dead = 0;  // bit r: sample r has no corner inside its level
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if (t0 + r * 256 >= per_head) break;
    const int e = slot_of_sample(p, lt, w, u[r], v[r]);
    if (e < 0) dead |= 1u << r;
    else __hip_atomic_fetch_add(&hist[e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    walk_step(p, w);
  }
  // dead samples get zero gradients here and are never binned
  while (dead) {
    const int r = __builtin_ctz(dead);
    dead &= dead - 1;
    const int64_t id = walk_start(p, b, m, t0 + r * 256).id;
    store_scalar<T>(reinterpret_cast<T *>(a.grad_attn) + id, 0.0f);
    store_pair<T>(reinterpret_cast<T *>(a.grad_loc) + 2 * id, 0.0f, 0.0f);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.tiles_bm; e += blockDim.x) {
    const uint32_t n = hist[e];
    if (n) __hip_atomic_fetch_add(&a.w.counts[counter_index(bin_of_slot(p, lt, bm, e), stripe)], n,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- wave-wide integer scans and reductions (DPP inside 16-lane rows, then
// the row totals through readlane)
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes.
__device__ inline uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<0x111>(x);  // row_shr:1
  x += dpp_u32<0x112>(x);  // row_shr:2
  x += dpp_u32<0x114>(x);  // row_shr:4
  x += dpp_u32<0x118>(x);  // row_shr:8
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t t1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(x, 47);
  const uint32_t row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

__device__ inline uint32_t wave_sum(uint32_t x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

__device__ inline uint32_t wave_max(uint32_t x) {
  x = max(x, dpp_u32<kDppQuadXor1>(x));
  x = max(x, dpp_u32<kDppQuadXor2>(x));
  x = max(x, dpp_u32<kDppRowHalfMirror>(x));
  x = max(x, dpp_u32<kDppRowMirror>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

__device__ inline uint32_t ceil_div(uint32_t n, uint32_t d) { return (n + d - 1) / d; }

// Level, batch, head and tile of a bin.  The search runs over compile-time
// level indices only, so the plan arrays stay in scalar registers instead of
// being fetched from the argument segment with a computed index.
struct BinPos {
  int l, b, m, ty, tx, H, W, ntx;
  int64_t start;  // first pyramid row of the level
};

__device__ inline BinPos decode_bin(const BinPlan &p, int bin) {
  const int BM = (int)p.B * p.M;
  int l = 0, base = 0, nt = 1, ntx = 1, H = 1, W = 1;
  int64_t start = 0;
#pragma unroll
  for (int k = 0; k < kMaxLevels; ++k) {
    if (k < p.L && bin >= p.bin_base[k] && bin < p.bin_base[k] + BM * p.ntiles[k]) {
      l = k;
      base = p.bin_base[k];
      nt = p.ntiles[k];
      ntx = p.ntx[k];
      H = p.H[k];
      W = p.W[k];
      start = p.start[k];
    }
  }
  BinPos r;
  const int rem = bin - base;
  const int bm = rem / nt, t = rem - bm * nt;
  r.l = l;
  r.b = bm / p.M;
  r.m = bm - r.b * p.M;
  r.ty = t / ntx;
  r.tx = t - r.ty * ntx;
  r.H = H;
  r.W = W;
  r.ntx = ntx;
  r.start = start;
  return r;
}

// ---------------------------------------------------------------- plan pass
//
// Many blocks of kPlanBlock bins each, in chunk order, one bin per thread.
// Positions are exclusive scans over the chunk order of three counts per bin
// (samples, chunks, split-bin slots): a block scans its own bins, publishes
// its totals, and adds the totals every earlier block has published
// (decoupled look-back).  A block only ever waits for lower-numbered blocks,
// which are dispatched before it and wait for nobody later, so the waits end.

#ifndef MSDA_PLAN_BLOCK
#define MSDA_PLAN_BLOCK 64
#endif
// bins (and lanes) per plan block: one wave measured faster than 128, 256,
// 512 or 1024 bins a block (the per-block scan and chunk writes outweigh the
// longer look-back)
constexpr int kPlanBlock = MSDA_PLAN_BLOCK;
static_assert(kPlanBlock % 64 == 0 && kPlanBlock <= 1024, "plan block of whole waves");

// Position j of the chunk order is a bin: (batch, head) major, then the
// levels coarsest first, then the tiles of a level row-major, so that the
// chunks running at one time share the grad_out rows of one head of one image.
struct OrderTab {
  int tile_off, ntiles, bin_base, ntx;
};

// Bin at position j of the chunk order, and its position (level | head << 4,
// batch, tile row, tile column) for the tile pass.
__device__ inline int bin_of_order(const BinPlan &p, const OrderTab *ot, int j, uint4 &where) {
  const int bm = j / p.tiles_bm;
  const int off = j - bm * p.tiles_bm;
  int k = 0;
  while (k + 1 < p.L && !(off >= ot[k].tile_off && off < ot[k].tile_off + ot[k].ntiles)) ++k;
  const int t = off - ot[k].tile_off;
  const int b = bm / p.M, ty = t / ot[k].ntx;
  where = make_uint4((uint32_t)k | ((uint32_t)(bm - b * p.M) << 4), (uint32_t)b, (uint32_t)ty,
                     (uint32_t)(t - ty * ot[k].ntx));
  return ot[k].bin_base + bm * ot[k].ntiles + t;
}

__device__ inline uint32_t chunks_of(const BinPlan &p, uint32_t c) {
  return c == 0 ? 1u : (c + p.chunk - 1) / p.chunk;
}

// Exclusive scans over the block of three per-thread values: wave scans
// (DPP), then the kPlanBlock / 64 wave totals through LDS.  tot receives the
// block totals.  wsum holds 3 * (kPlanBlock / 64) words.
__device__ inline void block_scan3(uint32_t (&v)[3], uint32_t (&tot)[3], uint32_t *wsum) {
  constexpr int kWaves = kPlanBlock / 64;
  const int w = threadIdx.x >> 6;
  uint32_t inc[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) inc[k] = wave_incl_scan(v[k]);
  if ((threadIdx.x & 63) == 63)
#pragma unroll
    for (int k = 0; k < 3; ++k) wsum[k * kWaves + w] = inc[k];
  lds_barrier();
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const uint32_t t = wsum[k * kWaves + i];
      before += i < w ? t : 0u;
      all += t;
    }
    v[k] = before + inc[k] - v[k];
    tot[k] = all;
  }
  lds_barrier();  // wsum may be reused right away
}

// Default bound on the polls of one predecessor's published totals.
// Predecessors always publish (see above); the bound only guarantees that
// every wave ends.  A block that stops waiting raises kBinErrPlanWait, and the
// later passes then write NaN gradients instead of using overlapping ranges.
constexpr uint32_t kPlanSpinLimit = 1u << 24;
thread_local uint32_t g_spin_limit = kPlanSpinLimit;
// test hook: the tile pass takes its 64-bit addressing path at every size
thread_local bool g_tile_wide = false;

__global__ __launch_bounds__(kPlanBlock) void plan_kernel(BinArgs a) {
  __shared__ uint32_t wsum[3 * (kPlanBlock / 64)];
  __shared__ OrderTab ot[kMaxLevels];
  const BinPlan &p = a.p;
  if (threadIdx.x < (unsigned)p.L) {
    const int l = threadIdx.x;
    ot[l] = OrderTab{p.tile_off[l], p.ntiles[l], p.bin_base[l], p.ntx[l]};
  }
  lds_barrier();
  const int n = p.nbins;
  const int j = (int)blockIdx.x * kPlanBlock + (int)threadIdx.x;
  const bool live = j < n;
  uint4 where;
  const int i = bin_of_order(p, ot, min(j, n - 1), where);
  uint32_t cs[kStripes];
#pragma unroll
  for (int k = 0; k < kStripes; ++k) cs[k] = a.w.counts[counter_index(i, k)];
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < kStripes; ++k) c += cs[k];
  const uint32_t nch = live ? chunks_of(p, c) : 0u;
  uint32_t v[3] = {live ? c : 0u, nch, nch > 1 ? nch : 0u}, tot[3];
  block_scan3(v, tot, wsum);
  // publish this block's totals: value << 1 | 1, so a zero word means "not yet"
  unsigned long long *status = a.w.plan_status;
  if (threadIdx.x == 0)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      __hip_atomic_store(&status[3 * blockIdx.x + k], ((unsigned long long)tot[k] << 1) | 1ull,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // add the totals of all earlier blocks
  uint32_t pre[3] = {0, 0, 0};
  bool expired = false;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += kPlanBlock)
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      unsigned long long x = 0;
      for (uint32_t spin = 0; spin < p.spin_limit; ++spin) {
        x = __hip_atomic_load(&status[3 * b + k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (x & 1ull) break;
        __builtin_amdgcn_s_sleep(1);
      }
      expired |= !(x & 1ull);
      pre[k] += (uint32_t)(x >> 1);
    }
  if (expired)
    __hip_atomic_fetch_or(a.w.error, kBinErrPlanWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t pre_tot[3];
  block_scan3(pre, pre_tot, wsum);
  if (live) {
    const uint32_t pos = pre_tot[0] + v[0], ch = pre_tot[1] + v[1], slot = pre_tot[2] + v[2];
    uint32_t run = pos;
#pragma unroll
    for (int k = 0; k < kStripes; ++k) {
      a.w.cursor[counter_index(i, k)] = run;
      run += cs[k];
    }
    a.w.bin_start[i] = pos;
    a.w.bin_nch[i] = nch;
    a.w.bin_slot0[i] = nch > 1 ? slot : kNoSlot;
    // the bin's position is stored with each chunk, so that the tile pass
    // decodes no bin index
    for (uint32_t k = 0; k < nch; ++k) {
      const uint32_t first = k * (uint32_t)p.chunk;
      const uint32_t cnt = c > first ? min((uint32_t)p.chunk, c - first) : 0u;
      a.w.chunks[ch + k] = make_uint4((uint32_t)i, pos + first, cnt, nch > 1 ? slot + k : kNoSlot);
      a.w.chunk_pos[ch + k] = where;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    a.w.nchunks[0] = pre_tot[1] + tot[1];
    a.w.nchunks[1] = 0;  // the tile pass's chunk counter
  }
}

// ------------------------------------------------------------- scatter pass

// SOFTMAX: a.attn holds logits.  The walk gives lane t0 + 256 r sample
// q L K + j of its (batch, head) with t0 and 256 multiples of L K, so the
// samples of one head-query sit in L K consecutive lanes of one wave (whole
// head-queries also past the end of the walk).
template <typename T, bool SOFTMAX>
__global__ __launch_bounds__(256) void scatter_kernel(BinArgs a) {
  extern __shared__ uint32_t hist[];
  const BinPlan &p = a.p;
  if (*a.w.error) return;  // a failed check: the merge pass writes NaN gradients
  const int bm = blockIdx.y;  // batch * M + head
  const int b = bm / p.M, m = bm - b * p.M;
  const int stripe = (int)((blockIdx.x + blockIdx.y * gridDim.x) % kStripes);
  __shared__ LevelTab lt[kMaxLevels];
  stage_level_tab(p, lt);
  const uint32_t per_head = (uint32_t)p.Q * (uint32_t)(p.L * p.K);
  const uint32_t t0 = blockIdx.x * kCountSamples + threadIdx.x;
  const uint32_t first_id = ((uint32_t)b * (uint32_t)p.Q * (uint32_t)p.M + (uint32_t)m) *
                            (uint32_t)(p.L * p.K);
  for (int e = threadIdx.x; e < p.tiles_bm; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  // all loads in flight together (samples past the head's end reload its
  // first one); each sample is ranked as soon as its own location has arrived
  float u[kPer], v[kPer], aw[kPer];
  uint32_t sid[kPer];
  {
    SampleWalk w = walk_start(p, b, m, t0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      sid[r] = t0 + r * 256 < per_head ? w.id : first_id;
      walk_step(p, w);
    }
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) load_loc<T>(a.loc, sid[r], u[r], v[r]);
#pragma unroll
  for (int r = 0; r < kPer; ++r) aw[r] = ldf<T>(a.attn, sid[r]);
  if constexpr (SOFTMAX) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) aw[r] = group_softmax(aw[r], p.L * p.K);
  }
  int slot[kPer];
  uint32_t rank[kPer];
  SampleWalk w = walk_start(p, b, m, t0);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    slot[r] = -1;
    rank[r] = 0;
    if (t0 + r * 256 < per_head) {
      slot[r] = slot_of_sample(p, lt, w, u[r], v[r]);
      if (slot[r] >= 0)
        rank[r] = __hip_atomic_fetch_add(&hist[slot[r]], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    walk_step(p, w);
  }
  __syncthreads();
  // reserve every touched bin's range: the cursor of (bin, stripe) starts at
  // that stripe's first sorted position; kReserve returning atomics per
  // thread are in flight together
  constexpr int kReserve = 8;
  for (int e0 = 0; e0 < p.tiles_bm; e0 += 256 * kReserve) {
    uint32_t n[kReserve], got[kReserve];
#pragma unroll
    for (int k = 0; k < kReserve; ++k) {
      const int e = e0 + k * 256 + (int)threadIdx.x;
      n[k] = e < p.tiles_bm ? hist[e] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kReserve; ++k) {
      const int e = e0 + k * 256 + (int)threadIdx.x;
      got[k] = n[k] ? __hip_atomic_fetch_add(&a.w.cursor[counter_index(bin_of_slot(p, lt, bm, e), stripe)],
                                             n[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0u;
    }
#pragma unroll
    for (int k = 0; k < kReserve; ++k) {
      const int e = e0 + k * 256 + (int)threadIdx.x;
      if (n[k]) hist[e] = got[k];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if (slot[r] >= 0)
      a.w.recs[hist[slot[r]] + rank[r]] = make_uint4(sid[r], __float_as_uint(u[r]),
                                                     __float_as_uint(v[r]), __float_as_uint(aw[r]));
  }
}

// ---------------------------------------------------------------- tile pass

// One sample of a chunk, as the cell loop needs it.
struct SampleRec {
  uint32_t id;  // sample id
  float a;      // attention weight
  float u, v;   // normalised sampling location
};

// Lanes per sample and channels per lane for fp32 rows of D channels in LDS:
// 4 lanes x 8 channels for D = 32 keeps the cross-lane reductions to two
// steps; RS pads LDS rows by 16 bytes against bank conflicts.
template <int D>
struct TileLayout {
  static constexpr int VEC = D >= 32 ? 8 : D / 4;
  static constexpr int G = D / VEC;
  static constexpr int RS = D + 4;
};

// Work items of a chunk.  The samples of every cell (in cell order) are cut
// into pieces of at most P samples, P the smallest multiple of kU that leaves
// at most kMaxItems pieces, so that one lane group can own a piece's four
// corner rows and four accumulators in registers while the lane groups get
// similar amounts of work even when a few cells hold most of the chunk.
constexpr int kU = 4;               // samples a lane group loads and processes together
constexpr int kMaxItems = kCells;   // stage slots, one per item

// LDS carve-up of the tile kernel (bytes):
//   vt     [kEdge^2 + 1][RS] f32   value rows of the tile and its rim, then one zero row
//   stage  [kMaxItems][4][RS] f32  per-item corner sums; holds the unsorted records in phase A
//   sorted [kChunk] SampleRec      samples sorted by cell
//   tag    [kChunk] u32            cell | rank << 8 of each unsorted record, after the
//                                  sort its sorted position (~0: dropped)
//   cnt    [kCells + 1] u32        samples per cell
//   cstart [kCells + 1] u32        first sorted position of each cell
//   istart [kCells + 1] u32        first item of each cell; istart[kCells] = items in all
//   items  [kMaxItems] u32         first | (len - 1) << 10 | cell << 20 of each item
//   sched  [kMaxItems] u32         items by decreasing number of batches
//   next   u32                     the block's next chunk, claimed by thread 0
//   lvl    [kMaxLevels] LevelTab   level extents for the positions of later chunks
//   lstart [kMaxLevels] i64        first pyramid row of each level
template <int D>
struct TileSmem {
  static constexpr int RS = TileLayout<D>::RS;
  static constexpr size_t vt = 0;
  static constexpr size_t stage = vt + (size_t)(kEdge * kEdge + 1) * RS * 4;
  static constexpr size_t item_bytes = (size_t)kMaxItems * 4 * RS * 4;
  static constexpr size_t rec_bytes = (size_t)kChunk * sizeof(SampleRec);
  static constexpr size_t stage_bytes = item_bytes > rec_bytes ? item_bytes : rec_bytes;
  static constexpr size_t sorted = stage + stage_bytes;
  static constexpr size_t tag = sorted + (size_t)kChunk * sizeof(SampleRec);
  static constexpr size_t cnt = tag + (size_t)kChunk * 4;
  static constexpr size_t cstart = cnt + (size_t)(kCells + 1) * 4;
  static constexpr size_t istart = cstart + (size_t)(kCells + 1) * 4;
  static constexpr size_t items = istart + (size_t)(kCells + 1) * 4;
  static constexpr size_t sched = items + (size_t)kMaxItems * 4;
  static constexpr size_t next = sched + (size_t)kMaxItems * 4;
  static constexpr size_t lvl = next + 16;
  // the planner's batch-count histogram: in the stage area past the unsorted
  // records when it fits there (that part is free until the item loop), else
  // after the level table
  static constexpr size_t hist_bytes = 4 * ((size_t)kChunk / kU + 1);
  static constexpr bool hist_in_stage = item_bytes >= rec_bytes + hist_bytes;
  static constexpr size_t lstart = (lvl + (size_t)kMaxLevels * sizeof(LevelTab) + 7) / 8 * 8;
  static constexpr size_t tail = (lstart + (size_t)kMaxLevels * 8 + 15) / 16 * 16;
  static constexpr size_t hist = hist_in_stage ? stage + rec_bytes : tail;
  static constexpr size_t bytes = hist_in_stage ? tail : tail + hist_bytes;
};
static_assert(kChunk <= 1024, "item packing keeps 10-bit first / length fields");
// with the default 8x8 tiles the histogram costs the D = 32 rows no LDS
static_assert(kTile != 8 || TileSmem<32>::hist_in_stage, "no LDS growth for the D = 32 rows");

// A chunk's bin position as the plan pass stored it (chunk_pos), with the
// level's extent from the level table in LDS: no search and no division in the
// tile pass's chunk loop.  The entry is wave-uniform, and so are the results.
__device__ inline BinPos chunk_bin_pos(const uint4 &c, const LevelTab *lt, const int64_t *lstart) {
  BinPos r;
  r.l = __builtin_amdgcn_readfirstlane((int)(c.x & 15u));
  r.m = __builtin_amdgcn_readfirstlane((int)(c.x >> 4));
  r.b = __builtin_amdgcn_readfirstlane((int)c.y);
  r.ty = __builtin_amdgcn_readfirstlane((int)c.z);
  r.tx = __builtin_amdgcn_readfirstlane((int)c.w);
  r.H = __builtin_amdgcn_readfirstlane(lt[r.l].H);
  r.W = __builtin_amdgcn_readfirstlane(lt[r.l].W);
  r.ntx = __builtin_amdgcn_readfirstlane(lt[r.l].ntx);
  const int64_t st = lstart[r.l];
  r.start = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)((uint64_t)st >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)st));
  return r;
}

// Rim row (0 .. 4T-1) of tile-local pixel (iy, ix) that is an edge or halo pixel:
//   [0, T]        bottom halo row iy = T, ix = 0..T
//   [T+1, 2T]     right halo column ix = T, iy = 0..T-1
//   [2T+1, 3T]    top edge row iy = 0, ix = 0..T-1
//   [3T+1, 4T-1]  left edge column ix = 0, iy = 1..T-1
__device__ inline int rim_row(int iy, int ix) {
  if (iy == kTile) return ix;
  if (ix == kTile) return kTile + 1 + iy;
  if (iy == 0) return 2 * kTile + 1 + ix;
  return 3 * kTile + iy;  // ix == 0, iy >= 1
}

// VEC consecutive elements of T at element offset e (a multiple of VEC), as fp32.
template <typename T, int VEC>
__device__ inline void load_vec(const void *base, int64_t e, float (&o)[VEC]) {
  const T *src = reinterpret_cast<const T *>(base) + e;
  if constexpr (sizeof(T) == 4 && VEC % 4 == 0) {
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      const float4 v = reinterpret_cast<const float4 *>(src)[k];
      o[4 * k] = v.x; o[4 * k + 1] = v.y; o[4 * k + 2] = v.z; o[4 * k + 3] = v.w;
    }
  } else if constexpr (sizeof(T) == 2 && VEC == 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = Half<T>::lo(w[k]);
      o[2 * k + 1] = Half<T>::hi(w[k]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = to_float<T>(src[i]);
  }
}

// VEC elements of T at byte offset `off` of a buffer, as fp32.
template <typename T, int VEC>
__device__ inline void load_vec_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&o)[VEC]) {
  if constexpr (sizeof(T) == 4 && VEC % 4 == 0) {
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      uint32_t w[4];
      buffer_load<4>(r, off + 16 * k, w);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[4 * k + i] = __uint_as_float(w[i]);
    }
  } else if constexpr (sizeof(T) == 2 && VEC == 8) {
    uint32_t w[4];
    buffer_load<4>(r, off, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = Half<T>::lo(w[k]);
      o[2 * k + 1] = Half<T>::hi(w[k]);
    }
  } else if constexpr (sizeof(T) * VEC == 8) {
    uint32_t w[2];
    buffer_load<2>(r, off, w);
    unpack<T, 2>(w, o);
  } else {
    uint32_t w[1];
    buffer_load<1>(r, off, w);
    unpack<T, 1>(w, o);
  }
}

// ceil(n / d) for n <= 2^12 and 1 <= d <= 2^12, rd ~ 1/d within a few ulp: the
// float quotient is off by less than 2^-10 from n / d, so at most the floor of
// an exact integer quotient comes out one low, and one integer check fixes it.
__device__ inline uint32_t ceil_div_small(uint32_t n, uint32_t d, float rd) {
  uint32_t q = (uint32_t)((float)n * rd);
  q += (q + 1) * d <= n ? 1u : 0u;  // exact floor(n / d)
  return q + (q * d < n ? 1u : 0u);
}

// Cell starts in registers, computed by every wave of the tile kernel: lane j
// holds the exclusive starts s0, s1 of cells j and j + 64 (the count of cell
// kCells reads as 0, so the start of cell kCells is the number of live samples).
struct CellScan {
  uint32_t n0, n1, s0, s1, total;
};
__device__ inline CellScan cell_scan(const uint32_t *cnt) {
  const uint32_t lane = threadIdx.x & 63, c1 = lane + 64;
  CellScan r;
  r.n0 = cnt[lane];
  r.n1 = c1 < (uint32_t)kCells ? cnt[c1] : 0u;
  const uint32_t inc0 = wave_incl_scan(r.n0);
  const uint32_t inc1 = __builtin_amdgcn_readlane(inc0, 63) + wave_incl_scan(r.n1);
  r.s0 = inc0 - r.n0;
  r.s1 = inc1 - r.n1;
  r.total = __builtin_amdgcn_readlane(inc1, 63);
  return r;
}

// Value v of lane src (0..63) of the wave; every lane must be active.
__device__ inline uint32_t lane_value(uint32_t src, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)v);
}

// Set bits of a 64-lane mask below the calling lane.
__device__ inline uint32_t lanes_below(uint64_t k) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(k >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)k, 0u));
}

// Inclusive prefix maximum over the 64 lanes (values >= 0).
__device__ inline uint32_t wave_incl_max(uint32_t x) {
  x = max(x, dpp_u32<0x111>(x));  // row_shr:1 (lanes past a row's start read 0)
  x = max(x, dpp_u32<0x112>(x));  // row_shr:2
  x = max(x, dpp_u32<0x114>(x));  // row_shr:4
  x = max(x, dpp_u32<0x118>(x));  // row_shr:8
  const uint32_t t0 = __builtin_amdgcn_readlane(x, 15);
  const uint32_t t1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t t2 = __builtin_amdgcn_readlane(x, 47);
  const uint32_t row = (threadIdx.x & 63) >> 4;
  return max(x, max(row >= 1 ? t0 : 0u, max(row >= 2 ? t1 : 0u, row >= 3 ? t2 : 0u)));
}

// Wave 0 of the tile kernel, after the cell scan: the item table and the schedule.  Past
// the choice of P every step is a fixed sequence of wave-wide operations (no
// loop over the pieces of a cell or over the batch counts present), since this
// runs on one wave while the block waits for it.
//   - items: lane j holds items j and j + 64.  The first item of every
//     non-empty cell is marked with the cell (+1) in `sched`, and a prefix
//     maximum over the items gives each item its cell; the piece index follows
//     from the cell's first item.
//   - schedule: items by decreasing number of batches (ceil(length / kU)), a
//     counting sort with the histogram in `scratch` (at least kChunk / kU + 1
//     words); the order inside one batch count is free, since the schedule
//     only decides which lane group runs an item, never a result.
__device__ inline void plan_items(const CellScan &cs, const uint32_t *cnt, const uint32_t *cstart,
                                  uint32_t *istart, uint32_t *items, uint32_t *sched,
                                  uint32_t *scratch) {
  const uint32_t lane = threadIdx.x;
  const uint32_t c0 = lane, c1 = lane + 64;
  const uint32_t n0 = cs.n0, n1 = cs.n1;
  const uint32_t total = cs.total;
  // smallest P = kU * m with at most kMaxItems pieces: linear steps up from
  // the lower bound total / kMaxItems, then a binary search if that is slow
  // (m = kChunk / kU leaves one piece per non-empty cell, at most kCells)
  auto pieces = [&](uint32_t P) {
    const float rp = __builtin_amdgcn_rcpf((float)P);
    return wave_sum(ceil_div_small(n0, P, rp) + ceil_div_small(n1, P, rp));
  };
  uint32_t m = max(1u, ceil_div(total, kU * kMaxItems));
  for (int step = 0; pieces(kU * m) > (uint32_t)kMaxItems; ++step) {
    if (step < 3) {
      ++m;
      continue;
    }
    uint32_t lo = m + 1, hi = kChunk / kU;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (pieces(kU * mid) <= (uint32_t)kMaxItems) hi = mid;
      else lo = mid + 1;
    }
    m = lo;
    break;
  }
  const uint32_t P = kU * m;
  const float rp = __builtin_amdgcn_rcpf((float)P);
  const uint32_t k0 = ceil_div_small(n0, P, rp), k1 = ceil_div_small(n1, P, rp);
  const uint32_t iinc0 = wave_incl_scan(k0);
  const uint32_t itotal0 = __builtin_amdgcn_readlane(iinc0, 63);
  const uint32_t iinc1 = itotal0 + wave_incl_scan(k1);
  const uint32_t is0 = iinc0 - k0, is1 = iinc1 - k1;
  const uint32_t nitems = __builtin_amdgcn_readlane(iinc1, 63);
  istart[c0] = is0;
  if (c1 <= (uint32_t)kCells) istart[c1] = is1;  // istart[kCells] = number of items
  // cell of every item: markers, then a prefix maximum (one wave: its LDS
  // operations complete in program order)
  const uint32_t i0 = lane, i1 = lane + 64;
  sched[i0] = 0u;
  if (i1 < (uint32_t)kMaxItems) sched[i1] = 0u;
  if (k0) sched[is0] = c0 + 1;
  if (k1) sched[is1] = c1 + 1;
  const uint32_t mk0 = i0 < nitems ? sched[i0] : 0u;
  const uint32_t mk1 = i1 < nitems ? sched[i1] : 0u;
  const uint32_t own0 = wave_incl_max(mk0);
  const uint32_t own1 = max(wave_incl_max(mk1), __builtin_amdgcn_readlane(own0, 63));
  // (cell, piece) of items i0 and i1; batch counts b0, b1 (0: no such item)
  uint32_t b[2] = {0u, 0u};
  const uint32_t ii[2] = {i0, i1}, own[2] = {own0, own1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (ii[h] >= nitems) continue;
    const uint32_t c = own[h] - 1;
    const uint32_t j = ii[h] - istart[c];
    const uint32_t first = cstart[c] + j * P, len = min(P, cnt[c] - j * P);
    items[ii[h]] = first | ((len - 1) << 10) | (c << 20);
    b[h] = (len + kU - 1) / kU;
  }
  // schedule: items by decreasing batch count (1 .. m); the order inside one
  // count is free.  With few counts (the common case) one pair of wave
  // ballots per count places the items; else a counting sort with the
  // histogram in scratch
  if (m <= 16) {
    uint32_t base = 0;
    for (uint32_t bb = m; bb >= 1; --bb) {
      const uint64_t k0 = __ballot(b[0] == bb), k1 = __ballot(b[1] == bb);
      const uint32_t n0 = (uint32_t)__popcll(k0);
      if (b[0] == bb) sched[base + lanes_below(k0)] = ii[0];
      if (b[1] == bb) sched[base + n0 + lanes_below(k1)] = ii[1];
      base += n0 + (uint32_t)__popcll(k1);
    }
    return;
  }
  for (uint32_t e = lane; e <= m; e += 64) scratch[e] = 0u;
  uint32_t rank[2] = {0u, 0u};
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (b[h]) rank[h] = __hip_atomic_fetch_add(&scratch[b[h]], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
  // first position of batch count b = items with more batches: lane L sums the
  // counts m - 4L .. m - 4L - 3, a wave scan puts the lanes in order
  uint32_t h4[4], run = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int bb = (int)m - (int)(4 * lane) - t;
    h4[t] = bb >= 1 ? scratch[bb] : 0u;
    run += h4[t];
  }
  uint32_t pos = wave_incl_scan(run) - run;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int bb = (int)m - (int)(4 * lane) - t;
    if (bb >= 1) scratch[bb] = pos;
    pos += h4[t];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (b[h]) sched[scratch[b[h]] + rank[h]] = ii[h];
}

// n / d for n < 2^31: the magic product is below n, so its sum with n stays
// below 2^32 and the division needs no 64-bit step.
__device__ inline uint32_t fdiv31(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

template <int CTRL>
__device__ inline uint32_t dpp_move_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

// Diagnostic build (-DMSDA_TILE_PHASE_CLOCKS): every wave of a tile block
// reads the shader clock (s_memtime) after each phase of a chunk and sums the
// intervals; thread 0 leaves its block's sums, wave 0's view of the block's
// phases, in g_tile_phase when the block ends.  The default build compiles
// none of it.  Slots: 0 staging and the chunk claim, 1 cell pass, 2 cell scan,
// plan and record sort, 3 item loop, 4 the next chunk's position, 5 its loads
// issued, 6 result pass, 7 pixel pass, 8 last barrier; slot 11 counts chunks.
constexpr int kPhaseSlots = 12;
constexpr int kPhaseBlocks = 2048;
#ifdef MSDA_TILE_PHASE_CLOCKS
__device__ unsigned long long g_tile_phase[kPhaseBlocks][kPhaseSlots];
#define TILE_PHASE(k)                                  \
  do {                                                 \
    const unsigned long long now = __builtin_amdgcn_s_memtime(); \
    phase_sum[k] += now - phase_t;                     \
    phase_t = now;                                     \
  } while (0)
#else
#define TILE_PHASE(k) do { } while (0)
#endif

// FAST: every sample id is below 2^31 and the launch's grad_out image below
// 2^31 bytes (the launch checks both), so ids divide in 32 bits and grad_out
// rows load through a buffer descriptor with 32-bit offsets: fewer
// instructions per sample in the item loop than 64-bit addresses.
template <typename T, int D, bool FAST>
__global__ __launch_bounds__(256) void tile_kernel(BinArgs a) {
  using TL = TileLayout<D>;
  using SM = TileSmem<D>;
  constexpr int VEC = TL::VEC, G = TL::G, RS = TL::RS;
  constexpr int NROWS = kEdge * kEdge;
  constexpr int kZeroRow = NROWS;
  constexpr int NG = 256 / G;
  constexpr int kPer = kChunk / 256;                 // phase-A samples per thread
  constexpr int kRowIters = (NROWS + 1 + NG - 1) / NG;
  constexpr uint32_t kDropped = 0xffffffffu;
  constexpr int kRowShift = __builtin_ctz(D * (int)sizeof(T));  // bytes of a grad_out row, log2
  extern __shared__ __align__(16) char smem[];
  float *vt = reinterpret_cast<float *>(smem + SM::vt);
  float *stage = reinterpret_cast<float *>(smem + SM::stage);
  SampleRec *raw = reinterpret_cast<SampleRec *>(smem + SM::stage);  // phase A only
  SampleRec *sorted = reinterpret_cast<SampleRec *>(smem + SM::sorted);
  uint32_t *tag = reinterpret_cast<uint32_t *>(smem + SM::tag);
  uint32_t *cnt = reinterpret_cast<uint32_t *>(smem + SM::cnt);
  uint32_t *cstart = reinterpret_cast<uint32_t *>(smem + SM::cstart);
  uint32_t *istart = reinterpret_cast<uint32_t *>(smem + SM::istart);
  uint32_t *items = reinterpret_cast<uint32_t *>(smem + SM::items);
  uint32_t *sched = reinterpret_cast<uint32_t *>(smem + SM::sched);
  uint32_t *next_slot = reinterpret_cast<uint32_t *>(smem + SM::next);
  LevelTab *lt = reinterpret_cast<LevelTab *>(smem + SM::lvl);
  int64_t *lstart = reinterpret_cast<int64_t *>(smem + SM::lstart);

  const BinPlan &p = a.p;
  const __amdgpu_buffer_rsrc_t gsrc =
      make_rsrc(a.grad_out, FAST ? (uint32_t)((uint64_t)p.B * (uint64_t)p.Q * (uint64_t)p.M *
                                               (uint64_t)(D * (int)sizeof(T)))
                                  : 0u);
  // the chunk count and this block's first chunk entry do not depend on each
  // other: issue the loads together
  const uint32_t nchunks = *a.w.nchunks;
  const uint32_t failed = *a.w.error;
  uint4 ck = a.w.chunks[blockIdx.x];
  if (blockIdx.x >= nchunks || failed) return;

  // The block is persistent: after its first chunk (= blockIdx.x) it claims
  // chunks gridDim.x, gridDim.x + 1, ... from a counter, one at a time, until
  // they run out.  A chunk's records and value rows are loaded into registers
  // while the previous chunk writes its results and rows, so their latency
  // hides behind that work.
  uint4 rc[kPer];
  float vrow[kRowIters][VEC];
  bool vin[kRowIters];
  int64_t loaded_start;  // first pyramid row of the loaded chunk's level
  // all branch-free (clamped indices), so the loads are in flight together
  auto load_chunk = [&](const uint4 &c, const BinPos &q, uint32_t tid) {
    const int grp = (int)tid / G, lane = (int)tid % G;
    const uint32_t f = c.y, n = min(c.z, (uint32_t)kChunk);
    const int64_t st = q.start;
    loaded_start = st;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const uint32_t i = tid + r * 256;
      rc[r] = a.w.recs[n > 0 ? f + min(i, n - 1) : 0u];
    }
#pragma unroll
    for (int k = 0; k < kRowIters; ++k) {
      const int r = grp + k * NG;
      const int iy = r / kEdge, ix = r - (r / kEdge) * kEdge;
      const int py = q.ty * kTile + iy, px = q.tx * kTile + ix;
      const int64_t prow = st + (int64_t)py * q.W + px;  // pyramid row inside the batch image
      vin[k] = n > 0 && r < NROWS && py < q.H && px < q.W && prow >= 0 && prow < p.S;
      // rows outside the map load the level's first row and are zeroed when staged
      const int64_t row = vin[k] ? prow : (st >= 0 && st < p.S ? st : 0);
      load_vec<T, VEC>(a.value, (((int64_t)q.b * p.S + row) * p.M + q.m) * D + lane * VEC, vrow[k]);
    }
  };
  BinPos loaded_pos = decode_bin(p, (int)ck.x);
  load_chunk(ck, loaded_pos, threadIdx.x);
  stage_level_tab(p, lt);  // read after the first barrier below
  if (threadIdx.x < (unsigned)p.L) lstart[threadIdx.x] = p.start[threadIdx.x];

#ifdef MSDA_TILE_PHASE_CLOCKS
  unsigned long long phase_sum[kPhaseSlots] = {};
  unsigned long long phase_t = __builtin_amdgcn_s_memtime();
#endif
  for (;;) {
    // the thread index, made opaque to the compiler once per chunk: otherwise it
    // hoists the index arithmetic of every phase out of the loop, and those
    // values would hold registers through the item loop
    uint32_t tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int grp = (int)tid / G, lane = (int)tid % G;
    const int bin = (int)ck.x;
    const uint32_t count = min(ck.z, (uint32_t)kChunk), slot = ck.w;
    const BinPos bp = loaded_pos;
    const int l = bp.l, b = bp.b, m = bp.m, ty = bp.ty, tx = bp.tx, H = bp.H, W = bp.W;
    const int64_t start = loaded_start;
    const int px0 = tx * kTile, py0 = ty * kTile;
    const int64_t row0 = (int64_t)b * p.S + start;  // first pyramid row of this level and batch

    for (int c = tid; c < kCells + 1; c += blockDim.x) cnt[c] = 0;
#pragma unroll
    for (int k = 0; k < kRowIters; ++k) {
      const int r = grp + k * NG;
      if (r < NROWS + 1)
#pragma unroll
        for (int i = 0; i < VEC; ++i) vt[r * RS + lane * VEC + i] = vin[k] ? vrow[k][i] : 0.0f;
    }
    if (tid == 0)
      *next_slot = gridDim.x + __hip_atomic_fetch_add(a.w.nchunks + 1, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    TILE_PHASE(0);
    // the next chunk's entry: needed only for the prefetch after the item loop
    const uint32_t cn = __builtin_amdgcn_readfirstlane(*next_slot);
    const uint4 ck_next = a.w.chunks[min(cn, nchunks - 1)];
    const uint4 cp_next = a.w.chunk_pos[min(cn, nchunks - 1)];

    // ---- phase A: cell of each sample and its rank inside the cell
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const uint32_t i = tid + r * 256;
      if (i >= count) break;
      uint32_t t = kDropped;
      const uint32_t id = rc[r].x;
      const float su = __uint_as_float(rc[r].y), sv = __uint_as_float(rc[r].z);
      if (id < p.total) {
        const uint32_t hq = FAST ? fdiv31(id, p.div_lk) : fdiv(id, p.div_lk);
        const uint32_t j = id - hq * (uint32_t)(p.L * p.K);
        Cell c;
        if ((int)fdiv31(j, p.div_k) == l && cell_of(su, sv, H, W, c)) {
          const int cy = c.y0 - py0 + 1, cx = c.x0 - px0 + 1;
          if (cy >= 0 && cy < kEdge && cx >= 0 && cx < kEdge) {
            const uint32_t cell = (uint32_t)(cy * kEdge + cx);
            const uint32_t rank = __hip_atomic_fetch_add(&cnt[cell], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP);
            raw[i] = SampleRec{id, __uint_as_float(rc[r].w), su, sv};
            t = cell | (rank << 8);
          }
        }
      }
      tag[i] = t;
    }
    __syncthreads();
    TILE_PHASE(1);
    // every wave scans the cell counts itself; wave 0 stores the starts and
    // plans the items while the other waves put the records in cell order,
    // looking the starts up in their own registers
    const CellScan cs = cell_scan(cnt);
    if (tid < 64) {
      cstart[tid] = cs.s0;
      if (tid + 64 <= (uint32_t)kCells) cstart[tid + 64] = cs.s1;
      plan_items(cs, cnt, cstart, istart, items, sched, reinterpret_cast<uint32_t *>(smem + SM::hist));
    } else {
      // whole waves per step, so that every lane takes part in the lane lookups
      for (uint32_t base = 0; base < count; base += blockDim.x - 64) {
        const uint32_t i = base + tid - 64;
        const uint32_t t = i < count ? tag[i] : kDropped;
        const uint32_t c = t & 63u;
        const uint32_t lo = lane_value(c, cs.s0), hi = lane_value(c, cs.s1);
        if (t != kDropped) {
          const uint32_t d = ((t & 0xffu) < 64u ? lo : hi) + (t >> 8);
          sorted[d] = raw[i];
          tag[i] = d;  // the result pass finds the record here
        }
      }
    }
    __syncthreads();
    TILE_PHASE(2);

    // ---- item loop: lane group g takes the schedule's entries g, 2NG-1-g,
    // 2NG+g, ... (largest items first, snaking so the groups of a wave get items
    // of similar size); an item's four corner rows (fp64) and its four corner
    // sums (fp32) stay in registers
    const uint32_t nitems = istart[kCells];
    for (int round = 0; round * NG < (int)nitems; ++round) {
      const int r = round * NG + ((round & 1) ? NG - 1 - grp : grp);
      if (r >= (int)nitems) continue;
      const int item = (int)sched[r];
      const uint32_t desc = items[item];
      const uint32_t s0 = desc & 0x3ffu, n = ((desc >> 10) & 0x3ffu) + 1, cell = desc >> 20;
      const int cy = (int)cell / kEdge, cx = (int)cell - ((int)cell / kEdge) * kEdge;
      const double x0 = (double)(px0 + cx - 1), y0 = (double)(py0 + cy - 1);
      double V[4][VEC];
      float acc[4][VEC];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // corner q of cell (cy, cx) is tile-local pixel (cy - 1 + q/2, cx - 1 + q%2)
        const int iy = cy - 1 + (q >> 1), ix = cx - 1 + (q & 1);
        const bool in = iy >= 0 && ix >= 0 && py0 + iy < H && px0 + ix < W;
        const float *src = vt + (in ? iy * kEdge + ix : kZeroRow) * RS + lane * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          V[q][i] = (double)src[i];
          if constexpr (G != 4) acc[q][i] = 0.0f;
        }
      }
      if constexpr (G == 4) {
        // transposed batches of kU = 4 samples: slot t of lane j holds sample
        // k0 + (j ^ t), so after the lane-wise partial dots one quad permutation
        // per slot hands lane j the full p_c of sample k0 + j, and every lane
        // does the per-sample work (weights, grad_attn, grad_loc) for its own
        // sample instead of all four lanes repeating it
        static_assert(kU == 4, "one sample per lane of a group");
        uint4 own[1];          // record of the lane's own sample
        uint32_t ids[1][4];    // sample ids of the four slots
        float g[1][4][VEC];    // grad_out rows (this lane's channels) of the four slots
        auto fetch = [&](uint32_t k0, int buf) {
          // slot t of lane j is lane (j ^ t)'s own sample: its id comes by a lane move
          own[buf] = reinterpret_cast<const uint4 *>(sorted)[s0 + min(k0 + (uint32_t)lane, n - 1)];
          ids[buf][0] = own[buf].x;
          ids[buf][1] = dpp_move_u32<kDppQuadXor1>(own[buf].x);
          ids[buf][2] = dpp_move_u32<kDppQuadXor2>(own[buf].x);
          ids[buf][3] = dpp_move_u32<kDppQuadXor3>(own[buf].x);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if constexpr (FAST) {
              const uint32_t off = (fdiv31(ids[buf][t], p.div_lk) << kRowShift) +
                                   (uint32_t)(lane * VEC * (int)sizeof(T));
              load_vec_buf<T, VEC>(gsrc, off, g[buf][t]);
            } else {
              load_vec<T, VEC>(a.grad_out, (int64_t)fdiv(ids[buf][t], p.div_lk) * D + lane * VEC,
                               g[buf][t]);
            }
          }
        };
        auto consume = [&](uint32_t k0, int buf, auto first) {
          double P[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            double pd[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              double sum = 0.0;
#pragma unroll
              for (int i = 0; i < VEC; ++i) sum = fma((double)g[buf][t][i], V[q][i], sum);
              pd[t] = sum;
            }
            P[q] = (pd[0] + dpp_move_f64<kDppQuadXor1>(pd[1])) +
                   (dpp_move_f64<kDppQuadXor2>(pd[2]) + dpp_move_f64<kDppQuadXor3>(pd[3]));
          }
          const bool valid = k0 + (uint32_t)lane < n;
          const uint32_t id = own[buf].x;
          const float av = __uint_as_float(own[buf].y);
          const double lx = ((double)__uint_as_float(own[buf].z) * (double)W - 0.5) - x0;
          const double ly = ((double)__uint_as_float(own[buf].w) * (double)H - 0.5) - y0;
          const double w0 = (1.0 - lx) * (1.0 - ly), w1 = lx * (1.0 - ly);
          const double w2 = (1.0 - lx) * ly, w3 = lx * ly;
          if (valid) {
            const double ga = w0 * P[0] + w1 * P[1] + w2 * P[2] + w3 * P[3];
            const double gx = (1.0 - ly) * (P[1] - P[0]) + ly * (P[3] - P[2]);
            const double gy = (1.0 - lx) * (P[2] - P[0]) + lx * (P[3] - P[1]);
            // the record has been read for good: it now holds the sample's results
            reinterpret_cast<uint4 *>(sorted)[s0 + k0 + lane] =
                make_uint4(id, __float_as_uint((float)ga),
                           __float_as_uint((float)((double)av * (double)W * gx)),
                           __float_as_uint((float)((double)av * (double)H * gy)));
          }
          const float as = valid ? av : 0.0f;
          const float aw[4] = {as * (float)w0, as * (float)w1, as * (float)w2, as * (float)w3};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float at[4] = {aw[q], dpp_move<kDppQuadXor1>(aw[q]),
                                 dpp_move<kDppQuadXor2>(aw[q]), dpp_move<kDppQuadXor3>(aw[q])};
            if constexpr (decltype(first)::value) {
              // the item's first batch starts its sums
#pragma unroll
              for (int i = 0; i < VEC; ++i) acc[q][i] = at[0] * g[buf][0][i];
            } else {
#pragma unroll
              for (int i = 0; i < VEC; ++i) acc[q][i] = fmaf(at[0], g[buf][0][i], acc[q][i]);
            }
#pragma unroll
            for (int t = 1; t < 4; ++t)
#pragma unroll
              for (int i = 0; i < VEC; ++i) acc[q][i] = fmaf(at[t], g[buf][t][i], acc[q][i]);
          }
        };
        fetch(0, 0);
        consume(0, 0, std::true_type{});
        for (uint32_t k0 = kU; k0 < n; k0 += kU) {
          fetch(k0, 0);
          consume(k0, 0, std::false_type{});
        }
      } else {
        // batches of kU samples; the records and grad_out rows of the next batch
        // are loaded before the current one is processed
        SampleRec rec[2][kU];
        float g[2][kU][VEC];
        auto fetch = [&](uint32_t k0, int buf) {
    #pragma unroll
          for (int u = 0; u < kU; ++u) {
            rec[buf][u] = sorted[s0 + min(k0 + u, n - 1)];
            load_vec<T, VEC>(a.grad_out, (int64_t)fdiv(rec[buf][u].id, p.div_lk) * D + lane * VEC,
                             g[buf][u]);
          }
        };
        auto consume = [&](uint32_t k0, int buf) {
    #pragma unroll
          for (int u = 0; u < kU; ++u) {
            if (k0 + u >= n) break;
            const SampleRec &sr = rec[buf][u];
            const float(&gu)[VEC] = g[buf][u];
            // fp64 partial dot products <g, V_c> over this lane's channels (exact products)
            double pc[4];
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
              double sum = 0.0;
    #pragma unroll
              for (int i = 0; i < VEC; ++i) sum = fma((double)gu[i], V[q][i], sum);
              pc[q] = sum;
            }
            const double lx = ((double)sr.u * (double)W - 0.5) - x0;
            const double ly = ((double)sr.v * (double)H - 0.5) - y0;
            const double w0 = (1.0 - lx) * (1.0 - ly), w1 = lx * (1.0 - ly);
            const double w2 = (1.0 - lx) * ly, w3 = lx * ly;
            // grad_attn = sum_c w_c p_c ; grad_loc = (A W d/dlx, A H d/dly), all linear in the p_c
            const double ga = group_sum_f64<G>(w0 * pc[0] + w1 * pc[1] + w2 * pc[2] + w3 * pc[3]);
            const double gx = group_sum_f64<G>((1.0 - ly) * (pc[1] - pc[0]) + ly * (pc[3] - pc[2]));
            const double gy = group_sum_f64<G>((1.0 - lx) * (pc[2] - pc[0]) + lx * (pc[3] - pc[1]));
            const float av = sr.a;
            if (lane == 0)
              reinterpret_cast<uint4 *>(sorted)[s0 + k0 + u] =
                  make_uint4(sr.id, __float_as_uint((float)ga),
                             __float_as_uint((float)((double)av * (double)W * gx)),
                             __float_as_uint((float)((double)av * (double)H * gy)));
            const float aw[4] = {av * (float)w0, av * (float)w1, av * (float)w2, av * (float)w3};
    #pragma unroll
            for (int q = 0; q < 4; ++q)
    #pragma unroll
              for (int i = 0; i < VEC; ++i) acc[q][i] = fmaf(aw[q], gu[i], acc[q][i]);
          }
        };
        fetch(0, 0);
        for (uint32_t k0 = 0; k0 < n; k0 += 2 * kU) {
          if (k0 + kU < n) fetch(k0 + kU, 1);
          consume(k0, 0);
          if (k0 + kU >= n) break;
          if (k0 + 2 * kU < n) fetch(k0 + 2 * kU, 0);
          consume(k0 + kU, 1);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < VEC; ++i) stage[(item * 4 + q) * RS + lane * VEC + i] = acc[q][i];
    }
    __syncthreads();
    TILE_PHASE(3);

    // the next chunk's records and value rows: in flight during the two passes
    // below (after the last chunk this loads a chunk again and leaves it unused,
    // which keeps the registers of the loads out of the item loop)
    loaded_pos = chunk_bin_pos(cp_next, lt, lstart);
    TILE_PHASE(4);
    load_chunk(ck_next, loaded_pos, tid);
    TILE_PHASE(5);

    // ---- per-sample results back in record order: the scatter pass wrote a
    // bin's records in sample order, so neighbouring lanes store neighbouring
    // ids and the stores of a sample's points merge
    // (the thread's kPer records go through each step together, so their LDS
    // reads are in flight at once)
    {
      uint32_t tg[kPer], pos[kPer];
      uint4 rr[kPer];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        const uint32_t i = tid + r * 256;
        tg[r] = i < count ? tag[i] : kDropped;
      }
#pragma unroll
      for (int r = 0; r < kPer; ++r)
        pos[r] = tg[r] != kDropped ? tg[r] : 0u;
#pragma unroll
      for (int r = 0; r < kPer; ++r) rr[r] = reinterpret_cast<const uint4 *>(sorted)[pos[r]];
#pragma unroll
      for (int r = 0; r < kPer; ++r) {
        if (tg[r] == kDropped) continue;
        store_scalar<T>(reinterpret_cast<T *>(a.grad_attn) + rr[r].x, __uint_as_float(rr[r].y));
        store_pair<T>(reinterpret_cast<T *>(a.grad_loc) + 2 * (int64_t)rr[r].x,
                      __uint_as_float(rr[r].z), __uint_as_float(rr[r].w));
      }
    }

    TILE_PHASE(6);
    // ---- every pixel of the tile and its rim sums the items of the cells it is
    // a corner of, then goes to grad_value (interior), the rim (edge / halo) or
    // the chunk's slot
    for (int r = grp; r < NROWS; r += NG) {
      const int iy = r / kEdge, ix = r - (r / kEdge) * kEdge;
      const int py = py0 + iy, px = px0 + ix;
      if (py >= H || px >= W) continue;
      // pixel (iy, ix) is corner 00 of cell (iy+1, ix+1), 01 of (iy+1, ix),
      // 10 of (iy, ix+1) and 11 of (iy, ix).  The first piece of each of the
      // four cells (the zero row for a cell with none) is read with all loads
      // in flight together; the further pieces of split cells follow.
      uint32_t ib[4], ie[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cy = iy + 1 - (q >> 1), cx = ix + 1 - (q & 1);
        const bool in = cy < kEdge && cx < kEdge;
        const int c = in ? cy * kEdge + cx : 0;
        ib[q] = in ? istart[c] : 0u;
        ie[q] = in ? istart[c + 1] : 0u;
      }
      float f[4][VEC];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float *src = ib[q] < ie[q] ? stage + (ib[q] * 4 + q) * RS + lane * VEC
                                         : vt + kZeroRow * RS + lane * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) f[q][i] = src[i];
      }
      float v[VEC];
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] = (f[0][i] + f[1][i]) + (f[2][i] + f[3][i]);
      // further pieces: step s reads piece s of all four cells together (the
      // zero row where a cell has fewer), so four loads are in flight per step
      uint32_t steps = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) steps = max(steps, ie[q] - ib[q]);
      for (uint32_t st = 1; st < steps; ++st) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t it = ib[q] + st;
          const float *src = it < ie[q] ? stage + (it * 4 + q) * RS + lane * VEC
                                        : vt + kZeroRow * RS + lane * VEC;
#pragma unroll
          for (int i = 0; i < VEC; ++i) f[q][i] = src[i];
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] += (f[0][i] + f[1][i]) + (f[2][i] + f[3][i]);
      }
      if (slot != kNoSlot) {
        float *dst = a.w.slots + ((int64_t)slot * NROWS + r) * D + lane * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) dst[i] = v[i];
      } else if (iy > 0 && ix > 0 && iy < kTile && ix < kTile) {
        const int64_t prow = start + (int64_t)py * W + px;
        if (prow < 0 || prow >= p.S) continue;  // inconsistent level_start_index: skip
        T *dst = reinterpret_cast<T *>(a.grad_value) +
                 ((row0 + (int64_t)py * W + px) * p.M + m) * D + lane * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) store_scalar<T>(dst + i, v[i]);
      } else {
        float *dst = a.w.rim + ((int64_t)bin * 4 * kTile + rim_row(iy, ix)) * D + lane * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) dst[i] = v[i];
      }
    }
    TILE_PHASE(7);
#ifdef MSDA_TILE_PHASE_CLOCKS
    phase_sum[kPhaseSlots - 1] += 1;
#endif
    if (cn >= nchunks) break;
    __syncthreads();  // the next chunk reuses every LDS array
    TILE_PHASE(8);
    ck = ck_next;
  }
#ifdef MSDA_TILE_PHASE_CLOCKS
  if (threadIdx.x == 0 && blockIdx.x < (unsigned)kPhaseBlocks)
    for (int k = 0; k < kPhaseSlots; ++k) g_tile_phase[blockIdx.x][k] = phase_sum[k];
#endif
}

// --------------------------------------------------------------- merge pass

// Contribution of bin `nb` (a neighbour, or the tile itself) at its tile-local
// pixel (iy, ix), from its rim (single-chunk) or its partial-tile slots.
template <int VEC, int D>
__device__ inline void add_part(const BinArgs &a, int nb, int iy, int ix, int lane, float *v) {
  constexpr int E = kTile + 1;
  const uint32_t nch = a.w.bin_nch[nb];
  if (nch <= 1) {
    const float *src = a.w.rim + ((int64_t)nb * 4 * kTile + rim_row(iy, ix)) * D + lane * VEC;
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] += src[i];
  } else {
    // four independent partial sums so the slot loads overlap
    const uint32_t s0 = a.w.bin_slot0[nb];
    const int64_t stride = (int64_t)E * E * D;
    const float *base = a.w.slots + ((int64_t)s0 * E * E + iy * E + ix) * D + lane * VEC;
    float part[4][VEC] = {};
    uint32_t k = 0;
    for (; k + 4 <= nch; k += 4)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < VEC; ++i) part[j][i] += base[(k + j) * stride + i];
    for (; k < nch; ++k)
#pragma unroll
      for (int i = 0; i < VEC; ++i) part[0][i] += base[k * stride + i];
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] += (part[0][i] + part[1][i]) + (part[2][i] + part[3][i]);
  }
}

// After a failed check (BinScratch::error) every gradient of the call is NaN.
template <typename T>
__device__ void poison_gradients(const BinArgs &a) {
  const BinPlan &p = a.p;
  const float nan = __int_as_float(0x7fc00000);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nv = p.B * p.S * p.M * p.D, ns = (int64_t)p.total;
  for (int64_t i = t0; i < nv; i += stride) store_scalar<T>(reinterpret_cast<T *>(a.grad_value) + i, nan);
  for (int64_t i = t0; i < 2 * ns; i += stride) store_scalar<T>(reinterpret_cast<T *>(a.grad_loc) + i, nan);
  for (int64_t i = t0; i < ns; i += stride) store_scalar<T>(reinterpret_cast<T *>(a.grad_attn) + i, nan);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(BinArgs a) {
  using TL = TileLayout<D>;
  constexpr int VEC = TL::VEC, G = TL::G;
  constexpr int NG = 256 / G;
  const BinPlan &p = a.p;
  if (*a.w.error) {
    poison_gradients<T>(a);
    return;
  }
  const int bin = blockIdx.x;
  const BinPos bp = decode_bin(p, bin);
  const int l = bp.l, b = bp.b, m = bp.m, ty = bp.ty, tx = bp.tx, H = bp.H, W = bp.W;
  const int ntx = bp.ntx;
  const int px0 = tx * kTile, py0 = ty * kTile;
  const int64_t row0 = (int64_t)b * p.S + a.starts[l];
  const bool split = a.w.bin_nch[bin] > 1;
  const int grp = threadIdx.x / G, lane = threadIdx.x % G;
  // rows to finish: the whole interior of a split bin, else its top row and left column
  const int nrows = split ? kTile * kTile : 2 * kTile - 1;
  for (int r = grp; r < nrows; r += NG) {
    int iy, ix;
    if (split) {
      iy = r / kTile;
      ix = r - iy * kTile;
    } else if (r < kTile) {
      iy = 0;
      ix = r;
    } else {
      iy = r - kTile + 1;
      ix = 0;
    }
    const int py = py0 + iy, px = px0 + ix;
    if (py >= H || px >= W) continue;
    const int64_t prow = a.starts[l] + (int64_t)py * W + px;
    if (prow < 0 || prow >= p.S) continue;  // inconsistent level_start_index: skip
    float v[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = 0.0f;
    add_part<VEC, D>(a, bin, iy, ix, lane, v);                       // own rows
    if (ix == 0 && tx > 0) add_part<VEC, D>(a, bin - 1, iy, kTile, lane, v);        // left's right halo
    if (iy == 0 && ty > 0) add_part<VEC, D>(a, bin - ntx, kTile, ix, lane, v);      // top's bottom halo
    if (ix == 0 && iy == 0 && tx > 0 && ty > 0)
      add_part<VEC, D>(a, bin - ntx - 1, kTile, kTile, lane, v);                    // top-left corner
    T *dst = reinterpret_cast<T *>(a.grad_value) + ((row0 + (int64_t)py * W + px) * p.M + m) * D +
             lane * VEC;
#pragma unroll
    for (int i = 0; i < VEC; ++i) store_scalar<T>(dst + i, v[i]);
  }
}

// Rows [pyramid_rows, S) of every batch image belong to no level: zero them.
template <typename T>
__global__ __launch_bounds__(256) void zero_tail_kernel(BinArgs a) {
  const BinPlan &p = a.p;
  const int64_t per_row = (int64_t)p.M * p.D;
  const int64_t tail = (p.S - p.pyramid_rows) * per_row;
  const int64_t n = p.B * tail;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / tail, r = i - b * tail;
    store_scalar<T>(reinterpret_cast<T *>(a.grad_value) + b * p.S * per_row +
                        p.pyramid_rows * per_row + r, 0.0f);
  }
}

template <typename T, int D>
size_t tile_lds_bytes() {
  return TileSmem<D>::bytes;
}

template <typename T, int D>
hipError_t launch_tile_and_merge(const BinArgs &a, hipStream_t s) {
  const size_t lds = tile_lds_bytes<T, D>();
  // persistent tile blocks: as many as fit on the device at once, at most one per chunk
  const uint64_t gout_bytes =
      (uint64_t)a.p.B * (uint64_t)a.p.Q * (uint64_t)a.p.M * (uint64_t)D * sizeof(T);
  const bool fast = !g_tile_wide && a.p.total < (1u << 31) && gout_bytes < (uint64_t(1) << 31);
  auto kernel = fast ? tile_kernel<T, D, true> : tile_kernel<T, D, false>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds);
  if (e != hipSuccess) return e;
  const int64_t resident = (int64_t)std::max(1, cus * std::max(1, per_cu));
  const int64_t grid = std::min(resident, (int64_t)a.p.max_chunks);
  prof_begin(s, "bin_tile");
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), lds, s, a);
  prof_end(s, "bin_tile");
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(s, "bin_merge");
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(a.p.nbins), dim3(256), 0, s, a);
  prof_end(s, "bin_merge");
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The striped bin counts and, after them, the plan blocks' published totals
// (3 words each): one region, cleared by one fill before the count pass.
size_t status_offset(const BinPlan &p) {
  return align256(counter_index(p.nbins, 0) * sizeof(uint32_t));
}
size_t error_offset_in_counts(const BinPlan &p) {
  const size_t blocks = ((size_t)p.nbins + kPlanBlock - 1) / kPlanBlock;
  return status_offset(p) + blocks * 3 * sizeof(unsigned long long);
}
size_t counts_and_status_bytes(const BinPlan &p) {
  return align256(error_offset_in_counts(p) + 16);
}

template <typename T>
hipError_t launch_binned_t(const BinArgs &a, hipStream_t s) {
  const BinPlan &p = a.p;
  hipError_t e;
  // the striped counts start at zero; the plan writes the cursors
  e = launch_zero(a.w.counts, counts_and_status_bytes(p), s);
  if (e != hipSuccess) return e;
  if (p.S > p.pyramid_rows) {
    prof_begin(s, "bin_zero_tail");
  hipLaunchKernelGGL((zero_tail_kernel<T>), dim3(1024), dim3(256), 0, s, a);
  prof_end(s, "bin_zero_tail");
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t per_head = p.Q * p.L * p.K;
  const dim3 grid((unsigned)((per_head + kCountSamples - 1) / kCountSamples),
                  (unsigned)(p.B * p.M));
  const size_t hist = (size_t)p.tiles_bm * sizeof(uint32_t);
  prof_begin(s, "bin_count");
  hipLaunchKernelGGL((count_kernel<T>), grid, dim3(256), hist, s, a);
  prof_end(s, "bin_count");
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(s, "bin_plan");
  hipLaunchKernelGGL(plan_kernel, dim3((unsigned)((p.nbins + kPlanBlock - 1) / kPlanBlock)),
                     dim3(kPlanBlock), 0, s, a);
  prof_end(s, "bin_plan");
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(s, "bin_scatter");
  if (a.softmax)
    hipLaunchKernelGGL((scatter_kernel<T, true>), grid, dim3(256), hist, s, a);
  else
    hipLaunchKernelGGL((scatter_kernel<T, false>), grid, dim3(256), hist, s, a);
  prof_end(s, "bin_scatter");
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (p.D) {
    case 8: return launch_tile_and_merge<T, 8>(a, s);
    case 16: return launch_tile_and_merge<T, 16>(a, s);
    case 32: return launch_tile_and_merge<T, 32>(a, s);
    case 64: return launch_tile_and_merge<T, 64>(a, s);
  }
  return hipErrorInvalidValue;
}


}  // namespace

bool make_bin_plan(BinPlan &p, int64_t B, int64_t Q, int64_t S, int M, int D, int L, int K,
                   const int64_t *shapes_host, const char **why) {
  std::memset(&p, 0, sizeof(p));
  p.B = B;
  p.Q = Q;
  p.S = S;
  p.M = M;
  p.D = D;
  p.L = L;
  p.K = K;
  p.tile = kTile;
  p.chunk = kChunk;
  if (L > kMaxLevels) {
    *why = "too many levels for the binned backward";
    return false;
  }
  int64_t rows = 0, tiles = 0;
  for (int l = 0; l < L; ++l) {
    const int64_t h = shapes_host[2 * l], w = shapes_host[2 * l + 1];
    if (h < 1 || w < 1 || h > (1 << 20) || w > (1 << 20)) {
      *why = "level shapes must be between 1 and 2^20 pixels per side";
      return false;
    }
    p.H[l] = (int)h;
    p.W[l] = (int)w;
    p.ntx[l] = (int)((w + kTile - 1) / kTile);
    p.ntiles[l] = (int)(((h + kTile - 1) / kTile) * p.ntx[l]);
    p.start[l] = rows;
    rows += h * w;
    tiles += p.ntiles[l];
  }
  p.spin_limit = g_spin_limit;
  if (rows > S) {
    *why = "the levels hold more pixels than num_keys";
    return false;
  }
  p.pyramid_rows = rows;
  const int64_t total = B * Q * M * L * K;
  const int64_t nbins = B * M * tiles;
  if (total >= (int64_t(1) << 32) - 1 || nbins >= (int64_t(1) << 30)) {
    *why = "too many samples or bins for the binned backward";
    return false;
  }
  if (B * M > 65535) {  // one grid row of the count and scatter passes per (batch, head)
    *why = "batch x num_heads exceeds 65535 for the binned backward";
    return false;
  }
  if ((int64_t)tiles * 4 > kHistLdsBytes) {
    *why = "the tiles of the pyramid exceed the per-block histogram";
    return false;
  }
  p.total = (uint32_t)total;
  p.div_lk = make_fastdiv((uint32_t)(L * K));
  p.div_k = make_fastdiv((uint32_t)K);
  p.step_j = 256u % (uint32_t)(L * K);
  p.step_id = 256u / (uint32_t)(L * K) * (uint32_t)(M * L * K) + p.step_j;
  p.wrap_id = (uint32_t)((M - 1) * L * K);
  p.magic_k = ((1u << 16) + (uint32_t)K - 1) / (uint32_t)K;
  p.nbins = (int)nbins;
  // coarsest level (highest index) first
  int run_bins = 0, run_tiles = 0;
  for (int l = L - 1; l >= 0; --l) {
    p.bin_base[l] = run_bins;
    p.tile_off[l] = run_tiles;
    run_bins += (int)(B * M) * p.ntiles[l];
    run_tiles += p.ntiles[l];
  }
  p.tiles_bm = run_tiles;
  const int64_t extra = (total + kChunk - 1) / kChunk;
  p.max_chunks = (int)(nbins + extra);
  p.max_slots = (int)(2 * extra);
  return true;
}

static size_t layout(const BinPlan &p, BinScratch *w, char *base) {
  const int E = kTile + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return base ? base + o : nullptr;
  };
  const size_t nb4 = (size_t)(p.nbins + 3) / 4 * 4;
  char *cc = take(counts_and_status_bytes(p));
  char *cu = take(counter_index(p.nbins, 0) * sizeof(uint32_t));
  char *bs = take(nb4 * sizeof(uint32_t));
  char *bn = take(nb4 * sizeof(uint32_t));
  char *b0 = take(nb4 * sizeof(uint32_t));
  char *nc = take(16);
  char *ch = take((size_t)p.max_chunks * sizeof(uint4));
  char *cp = take((size_t)p.max_chunks * sizeof(uint4));
  char *recs = take((size_t)p.total * sizeof(uint4));
  char *rim = take((size_t)p.nbins * 4 * kTile * p.D * sizeof(float));
  char *sl = take((size_t)p.max_slots * E * E * p.D * sizeof(float));
  if (w) {
    w->counts = reinterpret_cast<uint32_t *>(cc);
    w->plan_status = reinterpret_cast<unsigned long long *>(cc + status_offset(p));
    w->error = reinterpret_cast<uint32_t *>(cc + error_offset_in_counts(p));
    w->cursor = reinterpret_cast<uint32_t *>(cu);
    w->bin_start = reinterpret_cast<uint32_t *>(bs);
    w->bin_nch = reinterpret_cast<uint32_t *>(bn);
    w->bin_slot0 = reinterpret_cast<uint32_t *>(b0);
    w->nchunks = reinterpret_cast<uint32_t *>(nc);
    w->chunks = reinterpret_cast<uint4 *>(ch);
    w->chunk_pos = reinterpret_cast<uint4 *>(cp);
    w->recs = reinterpret_cast<uint4 *>(recs);
    w->rim = reinterpret_cast<float *>(rim);
    w->slots = reinterpret_cast<float *>(sl);
  }
  return off;
}

size_t binned_workspace_bytes(const BinPlan &p) { return layout(p, nullptr, nullptr); }

// the counts region is the first one the layout carves
size_t binned_error_offset(const BinPlan &p) { return error_offset_in_counts(p); }

void set_plan_spin_limit(uint32_t polls) { g_spin_limit = polls; }
void set_tile_wide_addressing(bool wide) { g_tile_wide = wide; }

hipError_t tile_phase_clocks(unsigned long long *host, int nblocks) {
#ifdef MSDA_TILE_PHASE_CLOCKS
  if (host == nullptr || nblocks < 0 || nblocks > kPhaseBlocks) return hipErrorInvalidValue;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_tile_phase),
                             (size_t)nblocks * kPhaseSlots * sizeof(unsigned long long));
#else
  (void)host;
  (void)nblocks;
  return hipErrorNotSupported;
#endif
}
uint32_t plan_spin_limit() { return g_spin_limit; }

BinScratch carve_bin_scratch(const BinPlan &p, void *workspace) {
  BinScratch w{};
  layout(p, &w, static_cast<char *>(workspace));
  return w;
}

hipError_t launch_backward_binned(const BinArgs &a, Dtype dt, hipStream_t stream) {
  if (a.p.total == 0) return hipSuccess;
  switch (dt) {
    case Dtype::F32: return launch_binned_t<float>(a, stream);
    case Dtype::BF16: return launch_binned_t<bf16_t>(a, stream);
    case Dtype::F16: return launch_binned_t<f16_t>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace msda
