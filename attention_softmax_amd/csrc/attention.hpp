// attention.hpp -- parameters of the fused attention forward kernel
// (attention.hip) shared with the C ABI entry point (api.hip).
//
// O = softmax(Q K^T * scale + mask) V over keys, per query row, the fusion of
// the QK^T product into the scaled-masked softmax that the pnsm.cn
// ScaledMaskSoftmax article proposes in sec. 4.4 (FlashAttention-style
// tiling: the score tensor never reaches memory), with the online softmax of
// the 0539edu.com notes' fused-attention section.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sms {

struct AttnParams {
  const char* q;
  const char* k;
  const char* v;
  const char* mask;  // additive (dtype), bool (bytes) or int32 key lengths [B]; or null
  char* o;
  float* lse;        // [B, H, Sq] natural-log log-sum-exp, or null
  int64_t sq_b, sq_h, sq_s;  // element strides of Q (head dim contiguous)
  int64_t sk_b, sk_h, sk_s;  // K
  int64_t sv_b, sv_h, sv_s;  // V
  int64_t so_b, so_h, so_s;  // O
  int64_t sm_b, sm_h, sm_q;  // mask, 0 on broadcast axes (keys contiguous)
  uint32_t B, H, Hk, Sq, Sk;
  uint32_t group;    // H / Hk: query heads per key/value head
  float scale_log2;  // scale * log2(e): scores are kept in the log2 domain
  int causal;        // 0 none, 1 key k > q excluded, 2 key k > q + Sk - Sq excluded
  int mask_kind;     // 0 none, 1 additive, 2 bool, 3 key lengths
};

enum : int { ATTN_MASK_NONE = 0, ATTN_MASK_ADD = 1, ATTN_MASK_BOOL = 2, ATTN_MASK_LEN = 3 };

// Queries per workgroup (four wavefronts of 32 queries) and keys per tile.
constexpr int kAttnBq = 128;
constexpr int kAttnBk = 64;

}  // namespace sms

// Launch of the forward for dtype 1 (fp16) or 2 (bf16) and head dim 64 or 128;
// hipErrorInvalidValue for anything else. Grid: H * B * ceil(Sq / 128).
hipError_t sms_attn_launch(const sms::AttnParams* p, int dtype, int head_dim, hipStream_t st);
