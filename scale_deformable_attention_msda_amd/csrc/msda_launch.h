// Internal launch interface between the C ABI (msda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda_device.h"

namespace msda {

// One launch covers batches [b0, b0 + nb) of a call.  Pointers are already
// offset to batch b0; all byte offsets inside a launch fit in 32 bits.
struct LaunchArgs {
  const void *value;            // [nb, S, M, D] of T
  const int64_t *shapes;        // [L, 2]
  const int64_t *starts;        // [L]
  const void *loc;              // [nb, Q, M, L, K, 2] of T
  const void *attn;             // [nb, Q, M, L, K] of T
  const void *grad_out;         // [nb, Q, M*D] of T            (backward)
  void *out;                    // [nb, Q, M*D] of T            (forward)
  void *grad_acc;               // [nb, S, M, D] of the accumulator type (backward)
  void *grad_loc;               // [nb, Q, M, L, K, 2] of T      (backward)
  void *grad_attn;              // [nb, Q, M, L, K] of T         (backward)
  int64_t nb, S, M, D, L, Q, K;
  uint32_t value_bytes;         // nb*S*M*D*sizeof(T)
  uint32_t acc_bytes;           // nb*S*M*D*sizeof(accumulator)
};

// ------------------------------------------------ destination-binned backward
//
// The pyramid of every (batch b, head m, level l) is cut into square tiles of
// `tile` x `tile` pixels.  A sample belongs to the tile that holds its
// top-left corner (x0, y0) (clamped to the map), so its four corners lie in
// that tile or in the one-pixel rim to its right / below.  Bins (one per tile
// of every (b, m)) are numbered coarsest level first, so the largest bins are
// scheduled first:
//   bin = bin_base[l] + (b*M + m) * ntiles[l] + ty * ntx[l] + tx.
constexpr int kMaxLevels = 16;

struct BinPlan {
  int64_t B, Q, S;
  int M, D, L, K;
  int tile;                    // tile edge T in pixels
  int chunk;                   // most samples one tile-kernel block processes
  int H[kMaxLevels], W[kMaxLevels];
  int ntx[kMaxLevels];         // tiles per row of level l
  int ntiles[kMaxLevels];      // tiles of level l (per batch and head)
  int bin_base[kMaxLevels];    // first bin of level l
  int tile_off[kMaxLevels];    // first tile of level l among the tiles of one (batch, head),
                               // coarsest level first
  int tiles_bm;                // tiles of all levels of one (batch, head)
  int nbins;                   // B * M * (tiles of all levels)
  int max_chunks;              // nbins + ceil(total / chunk)
  int max_slots;               // 2 * ceil(total / chunk)
  int64_t pyramid_rows;        // sum_l H_l * W_l
  uint32_t total;              // B*Q*M*L*K samples
  int64_t start[kMaxLevels];   // first pyramid row of level l (prefix sum of H*W)
  uint32_t spin_limit;         // polls of one predecessor's totals before the plan gives up
  FastDiv div_lk, div_k;       // by L*K and K
  // a stride of 256 samples of one (batch, head), t = q (L K) + j: the points
  // it advances (256 % (L K)), the sample ids it advances without and the
  // extra ids with a wrap of j (one query more: the other M - 1 heads)
  uint32_t step_j, step_id, wrap_id;
  uint32_t magic_k;              // ceil(2^16 / K): j / K = (j * magic_k) >> 16 for j < L K
};

// Device scratch carved out of the caller's workspace (byte offsets into it
// are fixed by binned_layout()).
struct BinScratch {
  uint32_t *counts;     // [nbins][stripes] samples per bin, per block stripe, one 64-byte line each
  unsigned long long *plan_status;  // [plan blocks][3] published totals (value << 1 | 1)
  uint32_t *error;      // [1] kBinErr* flags of this call (cleared with the counts)
  uint32_t *cursor;     // [nbins][stripes] fill cursor of the record scatter, one 64-byte line each
  uint32_t *bin_start;  // [nbins] first sorted position of a bin
  uint32_t *bin_nch;    // [nbins] chunks of a bin
  uint32_t *bin_slot0;  // [nbins] first partial-tile slot of a split bin
  uint32_t *nchunks;    // [2] chunks in use; the tile pass's counter of claimed chunks
  uint4 *chunks;        // [max_chunks] (bin, first position, count, slot or ~0) in chunk order
  uint4 *chunk_pos;     // [max_chunks] (level | head << 4, batch, tile row, tile column) of each
                        // chunk's bin
  uint4 *recs;          // [total] (id, u, v, A) of every live sample, sorted by bin
  float *rim;           // [nbins][4*tile][D] edge rows and halo of single-chunk tiles
  float *slots;         // [max_slots][(tile+1)^2][D] whole partial tiles of split bins
};

// Error flags the binned backward leaves in its workspace (BinScratch::error).
// A call that sets one writes NaN into all three gradients.
constexpr uint32_t kBinErrShapes = 1u;    // device spatial_shapes / level_start_index differ
                                          // from the host plan
constexpr uint32_t kBinErrPlanWait = 2u;  // a plan block stopped waiting for a predecessor

struct BinArgs {
  const void *value;
  const int64_t *shapes;  // device spatial_shapes
  const int64_t *starts;  // device level_start_index
  const void *loc;
  const void *attn;
  const void *grad_out;
  void *grad_value;
  void *grad_loc;
  void *grad_attn;
  BinPlan p;
  BinScratch w;
  // attn holds raw logits: the scatter pass forms each head-query's softmax
  // weights (L*K a power of two, at most 64)
  bool softmax = false;
};

// ------------------------------------------------ query-binned forward
//
// The head-queries (b, q, m) of one launch are sorted by a spatial key: the
// mean location of their points on the finest level (most pixels), cut into
// square bins of `T` x `T` finest-level pixels.  One tile block per bin (or
// per piece of at most `quads` head-queries of a bin) stages, level after
// level, the window of value rows its samples can reach (the bin's extent on
// that level plus a margin of R pixels) in LDS and gathers from there; the
// rare sample whose cell leaves the window is read from global memory.
constexpr int kFwdCountQ = 1024;             // queries (threads) per count / scatter block
constexpr int kFwdMaxBinsBM = 4096;          // bins per (batch, head)
constexpr int kFwdMaxPieces = 8;             // 16-byte staging pieces per thread and level
constexpr int kFwdMaxSlots = 8;              // (level, point-round) slots a lane holds

struct FwdPlan {
  int64_t Q, S;
  int nb, M, D, L, K;
  int KR;                      // point rounds: ceil(K / 4)
  int quads;                   // 4-lane groups per tile block (one head-query each): 128 or 256
  int f;                       // finest level
  int T, GX, GY, nbm;          // bin edge (finest-level pixels), bins per row and column, per (b, m)
  int nqb;                     // scatter blocks per (b, m) (kFwdCountQ queries each)
  int cq, nqc;                 // queries per count block (all heads; a power of two that
                               // divides kFwdCountQ) and count blocks per batch
  int max_chunks;              // chunk-list capacity
  int H[kMaxLevels], W[kMaxLevels], start[kMaxLevels];
  float sx[kMaxLevels], sy[kMaxLevels];  // bin edge in pixels of level l
  int R[kMaxLevels];                     // window margin on level l (its pixels)
  int ww[kMaxLevels], wh[kMaxLevels];    // window width and height (pixels of level l)
  FastDiv div_ww[kMaxLevels];
  int order[kMaxLevels];       // levels in processing order (smallest window first)
  int half;                    // LDS byte offset of the second window buffer; phase
                               // (chunk, level position i) uses buffer (i + parity) % 2,
                               // the parity flipping after each chunk when L is odd
  int lds_bytes;               // both window buffers
};

struct FwdScratch {
  uint32_t *keys;     // [nb*M][Q] bin of each head-query
  uint32_t *hist;     // [nb*M][nqc][nbm] per-count-block bin counts
  uint32_t *sorted;   // [nb*M][Q] query index, sorted by bin within each (b, m)
  uint32_t *nchunks;  // [1] chunks in the list
  uint4 *chunks;      // [max_chunks] (b*M + m, first sorted position, bin, count)
};

struct FwdArgs {
  LaunchArgs a;
  FwdPlan p;
  FwdScratch w;
};

// Kernel timing hooks (no-ops unless a profiling session is open on this
// thread): every launch site calls prof_begin() before and prof_end() after
// enqueueing its kernel, with the same name.
void prof_begin(hipStream_t stream, const char *name);
void prof_end(hipStream_t stream, const char *name);

// Set the thread's msda_last_error() text (entry points outside msda_api.hip).
void set_last_error(const char *msg);

enum class Dtype { F32, BF16, F16 };
// grad_value accumulator of the atomic scatter: fp32, or packed 16-bit atomics
// in the data type (BF16 or F16 data only)
enum class Accum { F32, PACKED };

// Tile pass of the binned backward on this thread (test hook): its 64-bit
// addressing path at every size instead of only where ids or the grad_out
// image reach 2^31.
void set_tile_wide_addressing(bool wide);
// Per-block phase clock sums of the last tile pass (diagnostic build only, see
// msda_binned.hip): nblocks x 12 values into host; hipErrorNotSupported in the
// default build.
hipError_t tile_phase_clocks(unsigned long long *host, int nblocks);
// Forward schedule for later launches on this thread (test hook): 0 automatic,
// 1 always the direct gather, 2 the LDS-window gather whenever it fits.
void set_forward_schedule(int schedule);
// softmax: a.attn holds raw logits, normalised per head-query inside the kernel
hipError_t launch_forward(const LaunchArgs &a, Dtype dt, hipStream_t stream, bool softmax = false);
// Row passes of the softmax method over n_rows rows of lk logits each:
// weights = softmax(logits); grad (dLoss/dA on entry) becomes dLoss/dlogits.
hipError_t launch_softmax_rows(const void *logits, void *weights, int64_t n_rows, int lk,
                               Dtype dt, hipStream_t stream);
hipError_t launch_softmax_grad_rows(const void *logits, void *grad, int64_t n_rows, int lk,
                                    Dtype dt, hipStream_t stream);
hipError_t launch_backward(const LaunchArgs &a, Dtype dt, Accum acc, hipStream_t stream);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);

// Binned backward: plan from host-side level shapes (returns false and a
// reason when the pyramid cannot be tiled within the kernel limits), size and
// carve the workspace, and enqueue the passes.
bool make_bin_plan(BinPlan &p, int64_t B, int64_t Q, int64_t S, int M, int D, int L, int K,
                   const int64_t *shapes_host, const char **why);
size_t binned_workspace_bytes(const BinPlan &p);
BinScratch carve_bin_scratch(const BinPlan &p, void *workspace);
// Byte offset of the error word inside the workspace.
size_t binned_error_offset(const BinPlan &p);
// Polls of one predecessor before a plan block gives up (this thread's later
// plans; a test hook, the default never expires on a working device).
void set_plan_spin_limit(uint32_t polls);
uint32_t plan_spin_limit();
hipError_t launch_backward_binned(const BinArgs &a, Dtype dt, hipStream_t stream);
// Query-binned forward: plan from host-side level shapes for a launch of
// `nb` batches (false when the sizes do not suit it: the caller then runs
// the direct gather), size and carve the workspace, enqueue the passes.
bool make_fwd_plan(FwdPlan &p, int64_t nb, int64_t Q, int64_t S, int M, int D, int L, int K,
                   int elt, const int64_t *shapes_host);
size_t fwd_workspace_bytes(const FwdPlan &p);
FwdScratch carve_fwd_scratch(const FwdPlan &p, void *workspace);
// reuse_order: only the tile pass, on the chunk list an earlier launch of the
// same plan left in the workspace
hipError_t launch_forward_binned(const FwdArgs &a, Dtype dt, bool reuse_order, hipStream_t stream);
hipError_t launch_cast_f32_to_half(const float *src, void *dst, size_t n, Dtype dt,
                                   hipStream_t stream);

}  // namespace msda
