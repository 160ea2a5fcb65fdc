// copy_ref.hip -- a plain device copy, the bandwidth reference the softmax
// kernels are measured against (not a step of the method).
//
// The fused operator's point is to read its inputs from HBM once and write
// its output once, where the unfused chain reads and writes the score tensor
// again at every step (lmnt.cn "Custom fused Softmax operator in CUDA, wrapped
// into PyTorch", sec. 1.1 and 1.2): a kernel that moves the same bytes with
// no arithmetic at all bounds what any such kernel can reach on the same
// chip. This one moves 16 bytes per lane with a nontemporal load and a
// nontemporal, device-scope store, 64 lanes (1 KB) per workgroup: the fastest
// of the copies measured on MI355X (3.25 GB each way: 64 lanes 6747 GB/s,
// 128 lanes 6703, 256 lanes 6671, 512 lanes 6448, two vectors per lane
// 6413-6016; plain nontemporal stores 6386-6708; the runtime's own copy
// kernel 4700-5400).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "sms.h"

namespace {

constexpr int kCopyLanes = 64;
constexpr int64_t kCopyChunk = kCopyLanes * 16;  // bytes per workgroup

// Workgroup w copies bytes [w * 1 KB, w * 1 KB + 1 KB) clipped to n16 vectors;
// its stores go through a buffer range over exactly its own bytes.
__global__ void __launch_bounds__(kCopyLanes) sms_copy_kernel(const char* src, char* dst,
                                                              uint64_t n16) {
  const uint64_t v = (uint64_t)blockIdx.x * kCopyLanes + threadIdx.x;
  const uint64_t first = (uint64_t)blockIdx.x * kCopyLanes;
  const uint32_t span = (uint32_t)(min<uint64_t>(n16 - first, kCopyLanes) * 16);
  const sms::RowStream ds = sms::row_stream(dst + first * 16, span);
  if (v < n16) {
    const sms::u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const sms::u32x4*>(src + v * 16));
    sms::buf_store<sms::kAuxNtDevice>(ds, threadIdx.x * 16u, x);
  }
}

}  // namespace

extern "C" sms_status sms_copy_reference(const void* src, void* dst, int64_t bytes,
                                         void* stream) {
  if (bytes < 0) return SMS_ERR_SHAPE;
  if (bytes == 0) return SMS_OK;
  if (!src || !dst) return SMS_ERR_NULL;
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15) || (bytes & 15)) return SMS_ERR_ALIGN;
  // One dispatch holds at most 2^32 - 1 work-items: 64 lanes per KiB.
  const int64_t blocks = (bytes + kCopyChunk - 1) / kCopyChunk;
  if (blocks * kCopyLanes > (int64_t)UINT32_MAX) return SMS_ERR_SHAPE;
  hipLaunchKernelGGL(sms_copy_kernel, dim3((uint32_t)blocks), dim3(kCopyLanes), 0,
                     (hipStream_t)stream, static_cast<const char*>(src), static_cast<char*>(dst),
                     (uint64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}
