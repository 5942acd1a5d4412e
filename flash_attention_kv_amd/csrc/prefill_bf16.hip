// prefill_bf16.hip -- launch side of the bf16 prefill kernel (the kernel
// itself is in prefill_bf16_kernel.h): query tile heights, the persistent
// grid of jagged batches and the dispatch by head dim.  The jagged d = 64
// and 128 instances live in prefill_bf16_jagged.hip and the d = 256 ones in
// prefill_bf16_d256.hip, each built with its own instruction scheduling
// strategy; this unit holds the dense d = 64 and 128 instances.
#include <atomic>

#include "prefill_bf16_kernel.h"

namespace fakv {

int prefill_bf16_query_rows(int d, int qh, bool jagged, bool window) {
  return 32 * ((jagged ? kWavesJagged : dense_waves(d, window)) / qh);
}

// Workgroups of the persistent (jagged) launch: all that fit at once.
int prefill_bf16_persistent_grid(int d, int qh) {
  static std::atomic<int> cache[32][9];   // per device, per (d, qh)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int key = (d == 64 ? 0 : d == 128 ? 3 : 6) + (qh == 1 ? 0 : qh == 2 ? 1 : 2);
  int g = cache[dev & 31][key].load(std::memory_order_relaxed);
  if (g > 0) return g;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  const int per = d == 256 ? prefill_bf16_resident_d256(qh) : prefill_bf16_resident_jagged(d, qh);
  // a multiple of 8 (one share per XCD queue), at least 8
  g = ((per * cus) / 8) * 8;
  if (g < 8) g = 8;
  cache[dev & 31][key].store(g, std::memory_order_relaxed);
  return g;
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int d, int qh, int grid, hipStream_t stream) {
  const bool jagged = p.sched != nullptr;
  switch (d) {
    case 64: return jagged ? launch_prefill_bf16_jagged(p, 64, qh, grid, stream) : launch_qh<64, false>(p, qh, grid, stream);
    case 128: return jagged ? launch_prefill_bf16_jagged(p, 128, qh, grid, stream) : launch_qh<128, false>(p, qh, grid, stream);
    case 256: return launch_prefill_bf16_d256(p, qh, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fakv
