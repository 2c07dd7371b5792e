// Host helper for kernels whose dynamic LDS exceeds the default 64 KB limit.
#pragma once

#include <mutex>
#include <set>
#include <utility>

#include <hip/hip_runtime.h>

namespace h3attn {

// Raises the dynamic-LDS limit of `kernel` to `bytes` once per (kernel, device): the attribute is
// set while a device is current, so a process that launches on several GPUs sets it on each.
// A failure is left to the launch, whose error the entry point reports.
inline void allow_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev}) != 0) return;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess)
    done.insert({kernel, dev});
}

}  // namespace h3attn
