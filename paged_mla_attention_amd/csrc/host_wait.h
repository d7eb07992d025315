// Bounded host wait on flags the device stores into pinned host memory.
// Header-only and free of HIP, so a plain C++ test program can exercise the
// deadline on a machine without a GPU.
#pragma once

#include <chrono>
#include <cstdint>
#include <thread>

namespace mla {

// Seconds mla_plan / mla_plan_reserve / mla_plan_destroy wait for the
// kernels of an earlier run to release a staging slot before giving up.
constexpr double kSlotWaitTimeoutS = 30.0;

// Waits until every flags[i] (i < n) has reached `seq` (sequence numbers
// compare modulo 2^32, so a later run's number also counts).  Returns true
// when they have, false when `timeout_s` passed first; *first_late then
// holds the first flag still short of `seq`.
inline bool wait_for_flags(const volatile int32_t* flags, int n, int32_t seq, double timeout_s,
                           int* first_late) {
  using clock = std::chrono::steady_clock;
  const auto deadline =
      clock::now() + std::chrono::duration_cast<clock::duration>(std::chrono::duration<double>(timeout_s));
  for (int i = 0; i < n; ++i) {
    unsigned spins = 0;
    while (static_cast<int32_t>(static_cast<uint32_t>(flags[i]) - static_cast<uint32_t>(seq)) < 0) {
      // (the clock is read every 64 spins: the common wait is a few us)
      if ((++spins & 63u) == 0 && clock::now() >= deadline) {
        if (first_late) *first_late = i;
        return false;
      }
      std::this_thread::yield();
    }
  }
  return true;
}

}  // namespace mla
