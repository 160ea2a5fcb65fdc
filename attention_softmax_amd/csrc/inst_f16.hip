// Kernel instantiations for one I/O format (f16); see kernels.hpp.
#include "kernels.hpp"

hipError_t sms_launch_fwd_f16(const sms::FwdParams& p, int tpr, int nv, uint32_t blocks,
                             hipStream_t st) {
  return sms::launch_fwd<sms::Fp16>(p, tpr, nv, blocks, st);
}

hipError_t sms_launch_bwd_f16(const sms::BwdParams& p, int tpr, int nv, uint32_t blocks,
                             hipStream_t st) {
  return sms::launch_bwd<sms::Fp16>(p, tpr, nv, blocks, st);
}

hipError_t sms_launch_fast_f16(const sms::FastFwdArgs* fa, const sms::FastBwdArgs* ba, int tpr,
                              int nv, uint32_t blocks, hipStream_t st) {
  return sms::launch_fast<sms::Fp16>(fa, ba, tpr, nv, blocks, st);
}

hipError_t sms_launch_stream_f16(const sms::FwdParams* fp, const sms::BwdParams* bp, uint32_t rows,
                                   hipStream_t st) {
  return sms::launch_stream<sms::Fp16>(fp, bp, rows, st);
}
