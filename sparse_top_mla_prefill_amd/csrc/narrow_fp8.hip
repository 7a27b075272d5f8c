// Narrow kernel, fp8 compute mode instance (the device code is in narrow_kernel.h).
#include "narrow_kernel.h"

namespace smla {

hipError_t launch_narrow_fp8(const KParams &p, hipStream_t s) {
  hipLaunchKernelGGL((smla_narrow_kernel<2, true>), dim3((unsigned)p.grid), dim3(kNThreads), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace smla
