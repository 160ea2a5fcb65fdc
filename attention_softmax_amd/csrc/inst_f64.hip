// Kernel instantiations for fp64 I/O (computed in fp64); see kernels.hpp.
#include "kernels.hpp"

hipError_t sms_launch_f64(const sms::FwdParams* fp, const sms::BwdParams* bp, int tpr,
                          uint32_t blocks, hipStream_t st) {
  return sms::launch_f64(fp, bp, tpr, blocks, st);
}
