// Internal launch interface between the C ABI (msda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

enum class Dtype { F32, BF16 };
enum class Accum { F32, BF16 };

hipError_t launch_forward(const LaunchArgs &a, Dtype dt, hipStream_t stream);
hipError_t launch_backward(const LaunchArgs &a, Dtype dt, Accum acc, hipStream_t stream);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_cast_f32_to_bf16(const float *src, void *dst, size_t n, hipStream_t stream);

}  // namespace msda
