// workspace.cpp — library-owned device memory for the kernels that need more
// than their inputs and outputs (split-K partials and arrival counters, the
// expert map of the grouped product, the arrival counters of the fused
// quantizing mat-vec).
//
// One buffer per (kind, device, stream), so calls on different streams never
// share one; allocated and zeroed on a stream's first call of that kind
// (hipMalloc, hipMemset, then a device synchronize, so the buffer is ready
// before any kernel of any stream uses it) and kept until the process ends.
// Each kind always asks for the same size.
#include <mutex>
#include <unordered_map>

#include "xq_launch.h"

namespace xq {

hipError_t stream_workspace(int kind, size_t bytes, hipStream_t stream, void** out) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, void*> spaces;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t key = (static_cast<uint64_t>(dev) << 52) ^ (static_cast<uint64_t>(kind) << 48) ^
                       reinterpret_cast<uintptr_t>(stream);
  std::lock_guard<std::mutex> lock(mu);
  auto it = spaces.find(key);
  if (it != spaces.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  if ((e = hipMalloc(&p, bytes)) != hipSuccess) return e;
  if ((e = hipMemset(p, 0, bytes)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
    (void)hipFree(p);
    return e;
  }
  *out = spaces[key] = p;
  return hipSuccess;
}

}  // namespace xq
