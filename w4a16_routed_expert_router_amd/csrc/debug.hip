// Test support for the slot pool's ordering: a kernel that occupies the side
// stream for a fixed time before a host-to-device copy, so that a reader that
// does not wait for the copy's completion reads the old row ("F51 Nitro /
// Nitro-MoE", "When forced on, the cache was slower - and once corrupt": an
// event-ordering mistake corrupted outputs there).  The wait is bounded by
// the clock and by an iteration count, whichever ends first.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

__global__ __launch_bounds__(64) void copy_delay_kernel(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();  // 100 MHz
  // each pass sleeps at least 64 x 32 cycles; the pass count alone ends the
  // wait even if the clock did not advance
  const uint64_t max_pass = ticks + 64;
  for (uint64_t i = 0; i < max_pass; ++i) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(32);
  }
}

void launch_copy_delay(hipStream_t stream, int microseconds) {
  hipLaunchKernelGGL(copy_delay_kernel, dim3(1), dim3(64), 0, stream, (uint64_t)microseconds * 100u);
}

}  // namespace moe
