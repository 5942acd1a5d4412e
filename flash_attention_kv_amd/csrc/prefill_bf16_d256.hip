// prefill_bf16_d256.hip -- the d = 256 instances of the bf16 prefill kernel.
//
// A translation unit of their own so that they can be built with the
// max-ILP instruction scheduler (-mllvm -amdgpu-sched-strategy=max-ilp, set
// for this file by the build): at d = 256 the operand-read and MFMA chains of
// a tile are long enough for it to pay (+2.5 % on the dense causal d = 256
// batch), while the d = 64 and 128 instances lose 0.5-1.5 % with it.
#include "prefill_bf16_kernel.h"

namespace fakv {

hipError_t launch_prefill_bf16_d256(const PrefillParams& p, int qh, int grid, hipStream_t stream) {
  return p.sched != nullptr ? launch_qh<256, true>(p, qh, grid, stream)
                            : launch_qh<256, false>(p, qh, grid, stream);
}

int prefill_bf16_resident_d256(int qh) { return resident_qh<256>(qh); }

}  // namespace fakv
