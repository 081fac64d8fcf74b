// Workgroup synchronisation and instruction-scheduling helpers shared by the
// streaming kernels (backward, attention-KL).
#pragma once

#include <hip/hip_runtime.h>

namespace mha {
namespace sync {

// Workgroup barrier without a memory fence (a fenced barrier would also wait
// for this wave's copy of the next tile). The waits that matter are explicit
// before it; the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling pins for a run of TOTAL MFMAs that each consume R LDS reads:
// the reads of the first AHEAD MFMAs, then for every MFMA n the MFMA and the
// reads of MFMA n + AHEAD. Keeps few operands in flight (registers) while
// the reads of later MFMAs overlap earlier ones.
template <int N, int TOTAL, int R, int AHEAD>
struct PinReads {
  static __device__ __forceinline__ void apply() {
    if constexpr (N == 0) __builtin_amdgcn_sched_group_barrier(0x100, R * AHEAD, 0);
    if constexpr (N < TOTAL) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (N + AHEAD < TOTAL) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
      PinReads<N + 1, TOTAL, R, AHEAD>::apply();
    }
  }
};

}  // namespace sync
}  // namespace mha
