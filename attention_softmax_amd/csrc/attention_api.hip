// attention_api.hip -- the fused-attention part of the C ABI declared in
// include/sms.h: argument checks, parameter blocks and the launches of the
// forward (attention.hip) and backward (attention_bwd.hip) kernels.
//
// The operation: scores Q K^T * scale + mask with the causal exclusion, the
// softmax of the softmax kernels over them and the product with V, without
// storing the scores (0539edu.com notes "From GEMM to Transformer:
// hand-written CUDA operator optimisation", the fused attention section, and
// the pnsm.cn ScaledMaskSoftmax article, sec. 4.4, which names fusing the
// softmax with the products around it as the next step).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "attention.hpp"
#include "sms.h"

namespace {

sms_status check_strides(const int64_t st[4]) {
  if (!st) return SMS_ERR_NULL;
  if (st[3] != 1) return SMS_ERR_STRIDE;
  for (int d = 0; d < 3; ++d)
    if (st[d] < 0) return SMS_ERR_STRIDE;
  return SMS_OK;
}

bool aligned_to(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

// Per-score masks whose rows start on 16-byte lines (8 additive values or 16
// boolean bytes; mask strides are multiples of Sk) go through LDS in tiles of
// 128 rows, whose byte range must fit 31 bits.
bool tile_mask(int kind, const void* mask, int64_t Sk) {
  if (kind == sms::ATTN_MASK_ADD) return Sk % 8 == 0 && aligned_to(mask, 16) && 128 * Sk * 2 < INT32_MAX;
  if (kind == sms::ATTN_MASK_BOOL) return Sk % 16 == 0 && aligned_to(mask, 16) && 128 * Sk < INT32_MAX;
  return false;
}

// Largest key / value row stride (elements): a tile of 64 rows is read
// through one buffer range, whose byte count must fit 31 bits.
constexpr int64_t kMaxRowStride = int64_t(1) << 24;

// A fused attention launch over `rows` rows per (head, batch) in tiles of 128
// is one workgroup of 256 threads per (tile, head, batch): the dispatch's
// work-item count must fit 32 bits.
bool attn_grid_too_large(int64_t rows, int64_t heads, int64_t B) {
  const int64_t tiles = (rows + 127) / 128;
  const int64_t limit = (int64_t)UINT32_MAX / 256;
  return tiles > limit || heads > limit || B > limit || tiles * heads > limit ||
         tiles * heads * B > limit;
}

// Element strides of a fused-attention mask over [B, H, Sq, Sk] scores (keys
// contiguous; 0 on broadcast axes; nothing to index for key lengths).
void attn_mask_strides(int shape_mode, int64_t H, int64_t Sq, int64_t Sk, int64_t& sb,
                       int64_t& sh, int64_t& sq) {
  sb = sh = sq = 0;
  switch (shape_mode) {
    case SMS_MASK_SQ_SK: sq = Sk; break;
    case SMS_MASK_B_SQ_SK: sb = Sq * Sk; sq = Sk; break;
    case SMS_MASK_B_1_SK: sb = Sk; break;
    case SMS_MASK_FULL: sb = H * Sq * Sk; sh = Sq * Sk; sq = Sk; break;
    default: break;
  }
}

}  // namespace

extern "C" {

sms_status sms_attention_forward(const void* q, const int64_t q_strides[4], const void* k,
                                 const int64_t k_strides[4], const void* v,
                                 const int64_t v_strides[4], const void* mask, int mask_mode,
                                 void* o, const int64_t o_strides[4], float* lse,
                                 sms_dtype dtype, int64_t B, int64_t H, int64_t Hk, int64_t Sq,
                                 int64_t Sk, int64_t D, float scale, int is_causal,
                                 void* stream) {
  if (dtype != SMS_F16 && dtype != SMS_BF16) return SMS_ERR_DTYPE;
  if (B < 0 || H < 0 || Hk < 0 || Sq < 0 || Sk < 0 || D < 0) return SMS_ERR_SHAPE;
  if (is_causal < SMS_CAUSAL_NONE || is_causal > SMS_CAUSAL_BOTTOM_RIGHT) return SMS_ERR_CAUSAL;
  const bool is_bool = (mask_mode & SMS_MASK_BOOL) != 0;
  const int shape_mode = mask_mode & ~SMS_MASK_BOOL;
  if (shape_mode < SMS_MASK_NONE || shape_mode > SMS_MASK_KEY_LENGTHS) return SMS_ERR_MASK_MODE;
  if (is_bool && (shape_mode == SMS_MASK_NONE || shape_mode == SMS_MASK_KEY_LENGTHS))
    return SMS_ERR_MASK_MODE;
  if (D != 64 && D != 128) return SMS_ERR_SHAPE;
  if (B == 0 || H == 0 || Sq == 0) return SMS_OK;  // no output row
  if (Hk < 1 || H % Hk != 0) return SMS_ERR_SHAPE;
  const bool has_mask = shape_mode != SMS_MASK_NONE;
  // With no key, K and V are never read (O = 0, LSE = -inf) and may be NULL.
  if (!q || !o || (Sk > 0 && (!k || !v)) ||
      (has_mask && !mask && (Sk > 0 || shape_mode == SMS_MASK_KEY_LENGTHS)))
    return SMS_ERR_NULL;
  sms_status st;
  for (const int64_t* s : {q_strides, k_strides, v_strides, o_strides})
    if ((st = check_strides(s)) != SMS_OK) return st;
  if (Sq > INT32_MAX || Sk > INT32_MAX || attn_grid_too_large(Sq, H, B)) return SMS_ERR_SHAPE;
  if (k_strides[2] > kMaxRowStride || v_strides[2] > kMaxRowStride) return SMS_ERR_STRIDE;
  // Every row of Q, K, V and O starts on a 16-byte line (head dims of 8 elements).
  for (const auto& t : {std::make_pair(q, q_strides), std::make_pair(k, k_strides),
                        std::make_pair(v, v_strides),
                        std::make_pair(static_cast<const void*>(o), o_strides)})
    if (((uintptr_t)t.first & 15) || (t.second[0] & 7) || (t.second[1] & 7) || (t.second[2] & 7))
      return SMS_ERR_ALIGN;
  const int mask_bytes = shape_mode == SMS_MASK_KEY_LENGTHS ? 4 : (is_bool ? 1 : 2);
  if (has_mask && !aligned_to(mask, mask_bytes)) return SMS_ERR_ALIGN;
  if (((uintptr_t)lse & 3) != 0) return SMS_ERR_ALIGN;

  sms::AttnParams p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.mask = static_cast<const char*>(mask);
  p.o = static_cast<char*>(o);
  p.lse = lse;
  p.sq_b = q_strides[0]; p.sq_h = q_strides[1]; p.sq_s = q_strides[2];
  p.sk_b = k_strides[0]; p.sk_h = k_strides[1]; p.sk_s = k_strides[2];
  p.sv_b = v_strides[0]; p.sv_h = v_strides[1]; p.sv_s = v_strides[2];
  p.so_b = o_strides[0]; p.so_h = o_strides[1]; p.so_s = o_strides[2];
  attn_mask_strides(shape_mode, H, Sq, Sk, p.sm_b, p.sm_h, p.sm_q);
  p.B = (uint32_t)B; p.H = (uint32_t)H; p.Hk = (uint32_t)Hk;
  p.Sq = (uint32_t)Sq; p.Sk = (uint32_t)Sk;
  p.group = (uint32_t)(H / Hk);
  p.scale_log2 = scale * sms::attn::kLog2eA;
  p.causal = is_causal;
  p.mask_kind = !has_mask ? sms::ATTN_MASK_NONE
                : shape_mode == SMS_MASK_KEY_LENGTHS ? sms::ATTN_MASK_LEN
                : is_bool ? sms::ATTN_MASK_BOOL : sms::ATTN_MASK_ADD;
  // Mask rows start on 4 elements (strides are multiples of Sk) and runs of 4
  // keys stay inside a row: vector mask loads.
  p.mask_vec = (p.mask_kind == sms::ATTN_MASK_ADD || p.mask_kind == sms::ATTN_MASK_BOOL) &&
               Sk % 4 == 0 && aligned_to(mask, p.mask_kind == sms::ATTN_MASK_ADD ? 8 : 4);
  // Mask rows on 16-byte lines (8 additive values or 16 boolean bytes), and a
  // tile of 128 rows within a 31-bit byte range.
  p.mask_tile = tile_mask(p.mask_kind, mask, Sk);
  const hipError_t e = sms_attn_launch(&p, (int)dtype, (int)D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

int64_t sms_attention_workspace_bytes(int64_t B, int64_t H, int64_t Sq) {
  if (B < 0 || H < 0 || Sq < 0) return -1;
  if (B > UINT32_MAX || H > UINT32_MAX || Sq > UINT32_MAX) return -1;
  const int64_t rows = B * H;
  if (H != 0 && rows / H != B) return -1;
  const int64_t n = rows * Sq;
  if (Sq != 0 && n / Sq != rows) return -1;
  if (n > (int64_t(1) << 40)) return -1;
  return n * 4;
}

sms_status sms_attention_backward(const void* q, const int64_t q_strides[4], const void* k,
                                  const int64_t k_strides[4], const void* v,
                                  const int64_t v_strides[4], const void* o,
                                  const int64_t o_strides[4], const void* dout,
                                  const int64_t dout_strides[4], const float* lse,
                                  const void* mask, int mask_mode, void* dq,
                                  const int64_t dq_strides[4], void* dk,
                                  const int64_t dk_strides[4], void* dv,
                                  const int64_t dv_strides[4], sms_dtype dtype, int64_t B,
                                  int64_t H, int64_t Hk, int64_t Sq, int64_t Sk, int64_t D,
                                  float scale, int is_causal, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  if (dtype != SMS_F16 && dtype != SMS_BF16) return SMS_ERR_DTYPE;
  if (B < 0 || H < 0 || Hk < 0 || Sq < 0 || Sk < 0 || D < 0) return SMS_ERR_SHAPE;
  if (is_causal < SMS_CAUSAL_NONE || is_causal > SMS_CAUSAL_BOTTOM_RIGHT) return SMS_ERR_CAUSAL;
  const bool is_bool = (mask_mode & SMS_MASK_BOOL) != 0;
  const int shape_mode = mask_mode & ~SMS_MASK_BOOL;
  if (shape_mode < SMS_MASK_NONE || shape_mode > SMS_MASK_KEY_LENGTHS) return SMS_ERR_MASK_MODE;
  if (is_bool && (shape_mode == SMS_MASK_NONE || shape_mode == SMS_MASK_KEY_LENGTHS))
    return SMS_ERR_MASK_MODE;
  if (D != 64 && D != 128) return SMS_ERR_SHAPE;
  if (B == 0 || H == 0 || (Sq == 0 && Sk == 0)) return SMS_OK;  // no gradient element
  if (Hk < 1 || H % Hk != 0) return SMS_ERR_SHAPE;
  const bool has_mask = shape_mode != SMS_MASK_NONE;
  // Tensors over queries may be NULL when Sq == 0, tensors over keys when Sk == 0.
  if ((Sq > 0 && (!q || !o || !dout || !dq || !lse)) || (Sk > 0 && (!k || !v || !dk || !dv)) ||
      (has_mask && !mask && ((Sq > 0 && Sk > 0) || shape_mode == SMS_MASK_KEY_LENGTHS)))
    return SMS_ERR_NULL;
  sms_status st;
  for (const int64_t* s : {q_strides, k_strides, v_strides, o_strides, dout_strides, dq_strides,
                           dk_strides, dv_strides})
    if ((st = check_strides(s)) != SMS_OK) return st;
  if (Sq > INT32_MAX || Sk > INT32_MAX) return SMS_ERR_SHAPE;
  if (attn_grid_too_large(Sq, H, B) || attn_grid_too_large(Sk, Hk, B)) return SMS_ERR_SHAPE;
  for (const int64_t* s : {q_strides, k_strides, v_strides, dout_strides})
    if (s[2] > kMaxRowStride) return SMS_ERR_STRIDE;
  const int64_t need = sms_attention_workspace_bytes(B, H, Sq);
  if (need < 0) return SMS_ERR_SHAPE;
  for (const auto& t :
       {std::make_pair(q, q_strides), std::make_pair(k, k_strides), std::make_pair(v, v_strides),
        std::make_pair(o, o_strides), std::make_pair(dout, dout_strides),
        std::make_pair(static_cast<const void*>(dq), dq_strides),
        std::make_pair(static_cast<const void*>(dk), dk_strides),
        std::make_pair(static_cast<const void*>(dv), dv_strides)})
    if (((uintptr_t)t.first & 15) || (t.second[0] & 7) || (t.second[1] & 7) || (t.second[2] & 7))
      return SMS_ERR_ALIGN;
  const int mask_bytes = shape_mode == SMS_MASK_KEY_LENGTHS ? 4 : (is_bool ? 1 : 2);
  if (has_mask && !aligned_to(mask, mask_bytes)) return SMS_ERR_ALIGN;
  if (((uintptr_t)lse & 3) != 0) return SMS_ERR_ALIGN;
  if (need > 0 && (!workspace || workspace_bytes < need)) return SMS_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 3) != 0) return SMS_ERR_ALIGN;

  sms::AttnBwdParams p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.o = static_cast<const char*>(o);
  p.dout = static_cast<const char*>(dout);
  p.mask = static_cast<const char*>(mask);
  p.lse = lse;
  p.delta = static_cast<float*>(workspace);
  p.dq = static_cast<char*>(dq);
  p.dk = static_cast<char*>(dk);
  p.dv = static_cast<char*>(dv);
  p.sq_b = q_strides[0]; p.sq_h = q_strides[1]; p.sq_s = q_strides[2];
  p.sk_b = k_strides[0]; p.sk_h = k_strides[1]; p.sk_s = k_strides[2];
  p.sv_b = v_strides[0]; p.sv_h = v_strides[1]; p.sv_s = v_strides[2];
  p.so_b = o_strides[0]; p.so_h = o_strides[1]; p.so_s = o_strides[2];
  p.sdo_b = dout_strides[0]; p.sdo_h = dout_strides[1]; p.sdo_s = dout_strides[2];
  p.sdq_b = dq_strides[0]; p.sdq_h = dq_strides[1]; p.sdq_s = dq_strides[2];
  p.sdk_b = dk_strides[0]; p.sdk_h = dk_strides[1]; p.sdk_s = dk_strides[2];
  p.sdv_b = dv_strides[0]; p.sdv_h = dv_strides[1]; p.sdv_s = dv_strides[2];
  attn_mask_strides(shape_mode, H, Sq, Sk, p.sm_b, p.sm_h, p.sm_q);
  p.B = (uint32_t)B; p.H = (uint32_t)H; p.Hk = (uint32_t)Hk;
  p.Sq = (uint32_t)Sq; p.Sk = (uint32_t)Sk;
  p.group = (uint32_t)(H / Hk);
  p.scale = scale;
  p.scale_log2 = scale * sms::attn::kLog2eA;
  p.causal = is_causal;
  p.mask_kind = !has_mask ? sms::ATTN_MASK_NONE
                : shape_mode == SMS_MASK_KEY_LENGTHS ? sms::ATTN_MASK_LEN
                : is_bool ? sms::ATTN_MASK_BOOL : sms::ATTN_MASK_ADD;
  // Mask rows start on 4 elements (strides are multiples of Sk) and runs of 4
  // keys stay inside a row: vector mask loads.
  p.mask_vec = (p.mask_kind == sms::ATTN_MASK_ADD || p.mask_kind == sms::ATTN_MASK_BOOL) &&
               Sk % 4 == 0 && aligned_to(mask, p.mask_kind == sms::ATTN_MASK_ADD ? 8 : 4);
  // Mask tiles in LDS, as in the forward.
  p.mask_tile = tile_mask(p.mask_kind, mask, Sk);
  const hipError_t e =
      sms_attn_bwd_launch(&p, (int)dtype, (int)D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

}  // extern "C"
