// Narrow kernel, bf16 compute mode instance (the device code is in narrow_kernel.h).
#include "narrow_kernel.h"

namespace smla {

hipError_t launch_narrow(const KParams &p, int heads_per_group, bool fp8_q, hipStream_t s) {
  // One instance per compute mode: with 32 heads per item every head count splits its keys
  // over the logit waves the same way, so a head's result does not depend on the head count.
  if (heads_per_group != 32) return hipErrorInvalidValue;
  if (fp8_q) return launch_narrow_fp8(p, s);
  hipLaunchKernelGGL((smla_narrow_kernel<2, false>), dim3((unsigned)p.grid), dim3(kNThreads), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace smla
