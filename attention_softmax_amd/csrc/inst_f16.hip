// Kernel instantiations for one I/O format (f16); see kernels.hpp.
#include "kernels.hpp"

hipError_t sms_launch_f16(const sms::FwdParams* fp, const sms::BwdParams* bp, int family, int tpr,
                             int nv, uint32_t blocks, hipStream_t st) {
  return sms::launch<sms::Fp16>(fp, bp, family, tpr, nv, blocks, st);
}
