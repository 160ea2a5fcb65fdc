// Kernel instantiations for one I/O format (f32); see kernels.hpp.
#include "kernels.hpp"

hipError_t sms_launch_f32(const sms::FwdParams* fp, const sms::BwdParams* bp, int family, int tpr,
                             int nv, uint32_t blocks, hipStream_t st) {
  return sms::launch<sms::Fp32>(fp, bp, family, tpr, nv, blocks, st);
}
