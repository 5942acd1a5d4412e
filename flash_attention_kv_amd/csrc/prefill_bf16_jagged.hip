// prefill_bf16_jagged.hip -- the persistent (jagged-batch) instances of the
// bf16 prefill kernel for d = 64 and 128, in a translation unit of their own
// so that they build with their own instruction scheduling strategy (the
// flags are in build.py; measured 1.8 % faster on the U[64, 2048] jagged mix
// than with the strategy of the dense instances, which it did not help).
// These instances are instantiated here only.
#include "prefill_bf16_kernel.h"

namespace fakv {

hipError_t launch_prefill_bf16_jagged(const PrefillParams& p, int d, int qh, int grid, hipStream_t stream) {
  switch (d) {
    case 64: return launch_qh<64, true>(p, qh, grid, stream);
    case 128: return launch_qh<128, true>(p, qh, grid, stream);
  }
  return hipErrorInvalidValue;
}

int prefill_bf16_resident_jagged(int d, int qh) { return d == 64 ? resident_qh<64>(qh) : resident_qh<128>(qh); }

}  // namespace fakv
