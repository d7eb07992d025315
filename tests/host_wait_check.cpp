// Drives the bounded flag wait (csrc/host_wait.h) without a GPU: flags that
// are already set return at once, flags another thread sets later end the
// wait, flags that never reach the sequence number end it at the deadline.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <thread>

#include "host_wait.h"

int main() {
  using clock = std::chrono::steady_clock;
  volatile int32_t flags[8] = {5, 5, 6, 5, 7, 5, 5, 5};
  int late = -1;
  if (!mla::wait_for_flags(flags, 8, 5, 1.0, &late)) return std::puts("set flags timed out"), 1;
  // a later sequence number also counts, across the 2^31 wrap too
  volatile int32_t wrap[2] = {static_cast<int32_t>(0x80000001u), 3};
  if (!mla::wait_for_flags(wrap, 1, 0x7fffffff, 1.0, &late)) return std::puts("wrap failed"), 1;
  // the last short flag is set by another thread after 50 ms
  for (int i = 0; i < 8; ++i) flags[i] = 8;
  flags[3] = 5;
  std::thread t([&] {
    std::this_thread::sleep_for(std::chrono::milliseconds(50));
    flags[3] = 8;
  });
  auto t0 = clock::now();
  const bool ok = mla::wait_for_flags(flags, 8, 8, 5.0, &late);
  t.join();
  const double dt = std::chrono::duration<double>(clock::now() - t0).count();
  if (!ok || dt < 0.04 || dt > 1.0) return std::printf("set later: ok=%d dt=%.3f\n", ok, dt), 1;
  // every flag at 9 except one that never gets there: the deadline ends it
  for (int i = 0; i < 8; ++i) flags[i] = 9;
  flags[6] = 8;
  t0 = clock::now();
  const bool ok2 = mla::wait_for_flags(flags, 8, 9, 0.2, &late);
  const double dt2 = std::chrono::duration<double>(clock::now() - t0).count();
  if (ok2 || late != 6 || dt2 < 0.19 || dt2 > 2.0)
    return std::printf("deadline: ok=%d late=%d dt=%.3f\n", ok2, late, dt2), 1;
  // flags reaching the number while waited for end the wait before the deadline
  flags[6] = 8;
  std::thread t2([&] {
    std::this_thread::sleep_for(std::chrono::milliseconds(30));
    flags[6] = 10;
  });
  t0 = clock::now();
  const bool ok3 = mla::wait_for_flags(flags, 8, 9, 5.0, &late);
  t2.join();
  const double dt3 = std::chrono::duration<double>(clock::now() - t0).count();
  if (!ok3 || dt3 > 1.0) return std::printf("late set: ok=%d dt=%.3f\n", ok3, dt3), 1;
  std::puts("ok");
  return 0;
}
