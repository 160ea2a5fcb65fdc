/*
 * sms.h -- C ABI of the fused scaled-masked softmax library (libsms.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation, for every row (b, h, q) of a score tensor x[B, H, Sq, Sk]:
 *
 *     s_k = x[b,h,q,k] * scale + mask[.., k]        (mask optional, additive)
 *     s_k = -inf                 if key k is excluded (boolean mask, key
 *                                length, or the causal rule)
 *     y[b,h,q,k] = exp(s_k - max_j s_j) / sum_j exp(s_j - max_j s_j)
 *
 * as defined in lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into
 * PyTorch", sec. 1.2 (scaled scores plus an additive mask, softmax over the key
 * axis; causal hides key j > query i) and sec. 2.1 (subtract the row maximum);
 * the causal rule is applied after the additive mask (sec. 3.1). A boolean mask
 * excludes keys inside the kernel instead of adding a large negative value
 * (pnsm.cn article on a custom ScaledMaskSoftmax operator, sec. 2.3). A row whose
 * every key is excluded is written as all zeros instead of 0/0 (same article,
 * sec. 4.2 and 4.3).
 *
 * The backward (same lmnt.cn page, sec. 3.3) is
 *
 *     dx[b,h,q,k] = scale * y_k * (dy_k - sum_j dy_j * y_j)
 *
 * which needs only the forward's output y, the upstream gradient dy and scale.
 *
 * Arithmetic: fp32, fp16 and bf16 inputs are widened to fp32; the row maximum,
 * the exponentials, the normaliser and the normalisation are fp32; the
 * backward's row dot product is accumulated in fp64. Outputs are rounded to the
 * I/O dtype with round-to-nearest-even, keeping subnormals. fp64 inputs (the
 * lmnt.cn page's wrapper dispatches float, double and half, sec. 4.2) are
 * computed in fp64 throughout; `scale` is still a 32-bit float.
 *
 * Common rules for both entry points
 * ----------------------------------
 * - All tensor pointers are DEVICE pointers (memory of the current HIP device),
 *   owned by the caller. The library allocates nothing (the split-row entry
 *   points take their workspace from the caller), keeps no state between
 *   calls and never synchronises: work is enqueued on `stream` (a hipStream_t;
 *   NULL = the null stream) and the call returns before it runs.
 * - Strides are in ELEMENTS, for the axes (B, H, Sq, Sk) in that order. The key
 *   axis must be contiguous (stride[3] == 1); other strides are any value >= 0.
 * - Every pointer must be aligned to its element size. Rows whose start is
 *   16-byte aligned in every operand take 128-bit loads and stores; other rows
 *   are still correct (element accesses for the unaligned head and tail).
 * - Outputs must not overlap inputs, except exactly in place: y == x with
 *   identical strides (forward), or dx == dy (or dx == y) with identical
 *   strides (backward). Every element is read before it is written, by the same
 *   thread, and rows do not share elements, so exact in-place use is safe.
 * - A size of zero in any dimension is a successful no-op.
 * - On any error nothing is launched and a status other than SMS_OK is
 *   returned; no function throws or aborts. SMS_ERR_HIP reports a failure the
 *   HIP runtime gave for the launch (hipGetLastError after enqueueing).
 */
#ifndef SMS_H
#define SMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMS_ABI_VERSION 7

typedef enum {
  SMS_OK = 0,
  SMS_ERR_NULL = 1,      /* a required pointer is NULL                            */
  SMS_ERR_SHAPE = 2,     /* negative dim, or a size beyond what the library runs  */
  SMS_ERR_STRIDE = 3,    /* stride[3] != 1 or a negative stride                   */
  SMS_ERR_DTYPE = 4,     /* unknown dtype                                         */
  SMS_ERR_MASK_MODE = 5, /* unknown mask mode                                     */
  SMS_ERR_ALIGN = 6,     /* a pointer not aligned to its element size             */
  SMS_ERR_HIP = 7,       /* the HIP runtime reported an error for the launch      */
  SMS_ERR_CAUSAL = 8,    /* unknown causal mode                                   */
  SMS_ERR_WORKSPACE = 9  /* workspace smaller than sms_workspace_bytes(), or not
                            8-byte aligned                                       */
} sms_status;

typedef enum {
  SMS_F32 = 0,  /* IEEE binary32                                */
  SMS_F16 = 1,  /* IEEE binary16                                */
  SMS_BF16 = 2, /* bfloat16 (upper 16 bits of a binary32 value) */
  SMS_F64 = 3   /* IEEE binary64, computed in binary64          */
} sms_dtype;

/* The mask's own shape; the mask is contiguous (row-major) in that shape and
 * axes it lacks are broadcast. The shapes follow the pnsm.cn ScaledMaskSoftmax
 * article, sec. 2.1 ([Sq,Sk] shared by all samples, or [B,Sq,Sk] per sample),
 * the lmnt.cn page's full mask (sec. 5.1 test), a per-batch key-padding mask
 * [B,1,Sk], and key padding given as lengths.
 *
 * Modes 1-4 alone: an ADDITIVE mask with x's dtype (0 keeps a key; a large
 * negative value or -inf masks it). Modes 1-4 OR'ed with SMS_MASK_BOOL: a
 * BOOLEAN mask of one byte per key, nonzero = the key is excluded (score
 * -inf), zero = kept. SMS_MASK_KEY_LENGTHS: `mask` points to int32 lengths[B];
 * keys k >= lengths[b] are excluded (lengths <= 0 exclude every key, lengths
 * >= Sk none), and no per-key mask is read. */
typedef enum {
  SMS_MASK_NONE = 0,        /* no mask; the mask pointer is ignored                */
  SMS_MASK_SQ_SK = 1,       /* [Sq, Sk],     broadcast over B and H                */
  SMS_MASK_B_SQ_SK = 2,     /* [B, Sq, Sk],  broadcast over H                      */
  SMS_MASK_B_1_SK = 3,      /* [B, 1, Sk],   broadcast over H and Sq (key padding) */
  SMS_MASK_FULL = 4,        /* [B, H, Sq, Sk]                                      */
  SMS_MASK_KEY_LENGTHS = 5  /* int32 lengths [B]: keys k >= lengths[b] excluded    */
} sms_mask_mode;

#define SMS_MASK_BOOL 0x10  /* OR with modes 1-4: uint8 mask, nonzero = excluded */

/* Causal rule: key k of row (b, h, q) is excluded when k > q (TOP_LEFT: query q
 * sees keys 0..q, as on the lmnt.cn page, sec. 1.2) or when k > q + Sk - Sq
 * (BOTTOM_RIGHT: the last query sees every key; for Sq != Sk, e.g. queries that
 * continue a longer key sequence). Both are the same rule when Sq == Sk. */
typedef enum {
  SMS_CAUSAL_NONE = 0,
  SMS_CAUSAL_TOP_LEFT = 1,
  SMS_CAUSAL_BOTTOM_RIGHT = 2
} sms_causal;

/*
 * sms_forward -- y = softmax(x * scale + mask) over the key axis, with the
 * optional causal rule (q = the row's index on the Sq axis).
 *
 *   x, x_strides   input scores [B,H,Sq,Sk] (dtype), device memory
 *   mask           device memory as `mask_mode` describes (additive: dtype,
 *                  values finite or -inf; boolean: uint8; lengths: int32);
 *                  may be NULL only with SMS_MASK_NONE
 *   mask_mode      an sms_mask_mode, modes 1-4 optionally OR'ed with SMS_MASK_BOOL
 *   y, y_strides   output [B,H,Sq,Sk] (dtype), device memory; every element of
 *                  every row is written (0 where excluded, all zeros for a row
 *                  with every key excluded)
 *   scale          multiplier applied to x before the mask (e.g. 1/sqrt(d_k))
 *   is_causal      an sms_causal value; the causal rule is applied after the mask
 *   stream         hipStream_t to enqueue on
 *
 * Limits: B*H*Sq < 2^32 rows, Sk <= sms_max_sk(dtype) = 2^30, and at most
 * 2^32 - 1 work-items per launch (rows of more than 4096 16-byte vectors take
 * one 1024-lane workgroup each, so at most 4194303 such rows per call).
 * Longer rows cost a second read of the row (two passes), except in the
 * backward of rows of up to 8192 vectors whose every operand row starts on a
 * 16-byte line and holds whole vectors, when the causal rule (if any) keeps at
 * least half of the keys (one pass). sms_forward never
 * splits a row across workgroups (see sms_forward_ws).
 */
sms_status sms_forward(const void* x, const int64_t x_strides[4],
                       const void* mask, int mask_mode,
                       void* y, const int64_t y_strides[4],
                       sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                       float scale, int is_causal, void* stream);

/*
 * sms_backward -- dx = scale * y * (dy - sum_k dy_k * y_k), row by row.
 *
 *   y, y_strides     the forward's output (dtype), device memory
 *   dy, dy_strides   upstream gradient (dtype), device memory
 *   dx, dx_strides   output gradient (dtype), device memory; every element written
 *   scale            the forward's scale
 *   is_causal        an sms_causal value other than NONE is a promise that y is
 *                    0 at the keys that rule excludes (true of any y sms_forward
 *                    wrote with the same rule); those y and dy are then not read
 *                    and dx there is written as 0. SMS_CAUSAL_NONE is always
 *                    correct.
 *   stream           hipStream_t to enqueue on
 *
 * Limits as for sms_forward.
 */
sms_status sms_backward(const void* y, const int64_t y_strides[4],
                        const void* dy, const int64_t dy_strides[4],
                        void* dx, const int64_t dx_strides[4],
                        sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                        float scale, int is_causal, void* stream);

/*
 * Split rows. When a call has too few rows to fill the GPU at one workgroup
 * per row (fewer than 256) and its rows are long (at least 16384 16-byte
 * vectors, 256 KB), each row is
 * cut into chunks with a workgroup each, in two launches: per-chunk partial
 * results -- (running max, sum of exponentials) forward, the partial dot
 * product backward -- go to a caller-provided workspace, and the second launch
 * merges a row's partials (the online-softmax merge of two (max, sum) pairs,
 * 0539edu.com notes, fused-attention section, where a row shared by several
 * blocks needs their statistics combined) and writes its chunk, re-reading
 * the chunk's inputs. The pnsm.cn ScaledMaskSoftmax article, sec. 2.2, cuts
 * rows beyond 4096 keys into blocks for the same reason of size.
 *
 * sms_workspace_bytes -- bytes of device workspace a call of sms_forward_ws
 * (backward = 0) or sms_backward_ws (backward = 1) with these sizes may use:
 * 0 when it would not split rows (any workspace, NULL included, is then
 * ignored; always 0 for SMS_F64, whose kernels never split rows), -1 for
 * invalid sizes or dtype. It depends only on the arguments
 * and on the SMS_SPLIT / SMS_FORCE_SPLIT environment overrides; 8 bytes per
 * (row, chunk), a few KB to tens of KB in practice.
 */
int64_t sms_workspace_bytes(sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                            int backward);

/*
 * sms_forward_ws / sms_backward_ws -- sms_forward / sms_backward with a
 * workspace (device memory owned by the caller, 8-byte aligned, of
 * `workspace_bytes` bytes, not shared with any call that may run at the same
 * time). With workspace == NULL they are exactly sms_forward / sms_backward.
 * Otherwise, if sms_workspace_bytes() > 0, rows are split as described above
 * and workspace_bytes must be at least that (else SMS_ERR_WORKSPACE, nothing
 * launched). The workspace holds no state between calls: its contents on entry
 * do not matter and are garbage on exit.
 */
sms_status sms_forward_ws(const void* x, const int64_t x_strides[4],
                          const void* mask, int mask_mode,
                          void* y, const int64_t y_strides[4],
                          sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                          float scale, int is_causal, void* workspace, int64_t workspace_bytes,
                          void* stream);
sms_status sms_backward_ws(const void* y, const int64_t y_strides[4],
                           const void* dy, const int64_t dy_strides[4],
                           void* dx, const int64_t dx_strides[4],
                           sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                           float scale, int is_causal, void* workspace, int64_t workspace_bytes,
                           void* stream);

/*
 * sms_forward_noalloc -- sms_forward_ws for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. It takes no workspace: a split forward keeps its
 * per-(row, chunk) partials in a scratch array the library holds in device
 * memory, one copy per GPU, until the process ends; the call itself allocates
 * nothing (no hipMalloc, no hipFree). Arguments, results and errors are those
 * of sms_forward_ws given that scratch as its workspace: a call whose split
 * needs more than sms_noalloc_scratch_bytes() bytes (possible only when
 * SMS_FORCE_SPLIT forces a large split) returns SMS_ERR_WORKSPACE and launches
 * nothing. The scratch of the device current at the call is used, so
 * `stream` must belong to that device. Every call on one GPU shares its
 * scratch: calls that may overlap on one GPU (different streams, different
 * host threads) race on it and must be ordered by the caller. Its contents on
 * entry do not matter.
 */
sms_status sms_forward_noalloc(const void* x, const int64_t x_strides[4],
                               const void* mask, int mask_mode,
                               void* y, const int64_t y_strides[4],
                               sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                               float scale, int is_causal, void* stream);

/* Bytes of the per-GPU scratch sms_forward_noalloc uses (65536). */
int64_t sms_noalloc_scratch_bytes(void);

/*
 * sms_attention_forward -- fused attention forward on the matrix cores,
 *
 *     O = softmax(Q K^T * scale + mask) V      (over keys, per query row)
 *
 * without writing the scores to memory: the fusion of the QK^T product into the
 * operator that the pnsm.cn ScaledMaskSoftmax article proposes in sec. 4.4
 * (FlashAttention-style tiling), with the online softmax of the 0539edu.com
 * notes' fused-attention section. The softmax step is exactly sms_forward's:
 * same scale, mask modes and kinds, causal rules, and fully-masked rows give
 * zeros.
 *
 *   q, q_strides   queries [B, H, Sq, D] (dtype), device memory
 *   k, k_strides   keys    [B, Hk, Sk, D]: query head h reads key/value head
 *                  h / (H / Hk) (grouped-query attention; Hk = H is plain
 *                  multi-head attention)
 *   v, v_strides   values  [B, Hk, Sk, D]
 *   mask, mask_mode  as for sms_forward, over [B, H, Sq, Sk] scores
 *   o, o_strides   output  [B, H, Sq, D] (dtype); every element written
 *   lse            NULL, or fp32 [B, H, Sq] contiguous: the natural log of
 *                  sum_k exp(score_k) over the visible keys (-inf if none), as
 *                  a backward pass would need it
 *   dtype          SMS_F16 or SMS_BF16 (products exact, fp32 accumulation; the
 *                  probabilities enter the P V product rounded to dtype)
 *   D              head dimension, 64 or 128
 *   scale, is_causal, stream   as for sms_forward
 *
 * Every row of q, k, v and o must start on a 16-byte boundary (base 16-byte
 * aligned, strides multiples of 8 elements; else SMS_ERR_ALIGN); the head dim
 * is contiguous (stride[3] == 1). With Sk == 0, k, v and a mask other than
 * key lengths are never read and may be NULL. Limits: Sq, Sk < 2^31 and
 * ceil(Sq / 128) * H * B < 2^24 (one 256-thread workgroup per 128 queries of a
 * head; else SMS_ERR_SHAPE); the key and value row strides k_strides[2] and
 * v_strides[2] at most 2^24 elements (tiles are read through 32-bit buffer
 * ranges; else SMS_ERR_STRIDE). The backward is sms_attention_backward.
 */
sms_status sms_attention_forward(const void* q, const int64_t q_strides[4],
                                 const void* k, const int64_t k_strides[4],
                                 const void* v, const int64_t v_strides[4],
                                 const void* mask, int mask_mode,
                                 void* o, const int64_t o_strides[4], float* lse,
                                 sms_dtype dtype, int64_t B, int64_t H, int64_t Hk,
                                 int64_t Sq, int64_t Sk, int64_t D,
                                 float scale, int is_causal, void* stream);

/*
 * sms_attention_workspace_bytes -- bytes of device workspace
 * sms_attention_backward needs: 4 * B * H * Sq (one fp32 per query row); -1
 * for negative or oversized arguments.
 */
int64_t sms_attention_workspace_bytes(int64_t B, int64_t H, int64_t Sq);

/*
 * sms_attention_backward -- gradients of the fused attention forward,
 *
 *     dV = P^T dO,  dP = dO V^T,  dS = scale * P * (dP - rowsum(dO * O)),
 *     dQ = dS K,    dK = dS^T Q
 *
 * for P = softmax(Q K^T * scale + mask): the probabilities are recomputed from
 * Q, K and the forward's log-sum-exp (never stored), FlashAttention-style, the
 * scheme the pnsm.cn ScaledMaskSoftmax article, sec. 4.4, points to; the dS
 * step is the softmax gradient of the lmnt.cn custom-softmax page, sec. 3.3,
 * with sum_j dP_j P_j computed as rowsum(dO * O). A key/value head shared by
 * several query heads receives the sum of their contributions. Deterministic:
 * no atomics, every gradient element written once (zeros where no visible
 * score reaches it).
 *
 *   q, k, v, mask, mask_mode, dtype, B, H, Hk, Sq, Sk, D, scale, is_causal
 *                  exactly as passed to sms_attention_forward
 *   o, o_strides   the forward's output O [B, H, Sq, D]
 *   dout, dout_strides   upstream gradient dO [B, H, Sq, D] (dtype)
 *   lse            the forward's fp32 log-sum-exp [B, H, Sq], contiguous
 *                  (may be NULL only when Sq == 0)
 *   dq, dk, dv (+ strides)   outputs [B, H, Sq, D], [B, Hk, Sk, D],
 *                  [B, Hk, Sk, D] (dtype), fp32-accumulated and rounded once;
 *                  they must not overlap the inputs
 *   workspace, workspace_bytes   device memory of at least
 *                  sms_attention_workspace_bytes(B, H, Sq) bytes, 4-byte
 *                  aligned, owned by the caller and not used by any call that
 *                  may run at the same time (else SMS_ERR_WORKSPACE); its
 *                  contents on entry do not matter
 *   stream         hipStream_t to enqueue on (two kernel launches; three
 *                  with D = 128, a per-score mask and 512 or more key
 *                  blocks of 128 (B * Hk * ceil(Sk / 128)), where dK and
 *                  dV take a launch each)
 *
 * Row alignment and limits as for sms_attention_forward, and also
 * ceil(Sk / 128) * Hk * B < 2^24 and the q and dout row strides at most 2^24
 * elements (else SMS_ERR_STRIDE). Pointers to tensors over queries (q, o,
 * dout, lse, dq) may be NULL when Sq == 0, those over keys (k, v, dk, dv)
 * when Sk == 0, and a mask other than key lengths when either is 0.
 */
sms_status sms_attention_backward(const void* q, const int64_t q_strides[4],
                                  const void* k, const int64_t k_strides[4],
                                  const void* v, const int64_t v_strides[4],
                                  const void* o, const int64_t o_strides[4],
                                  const void* dout, const int64_t dout_strides[4],
                                  const float* lse, const void* mask, int mask_mode,
                                  void* dq, const int64_t dq_strides[4],
                                  void* dk, const int64_t dk_strides[4],
                                  void* dv, const int64_t dv_strides[4],
                                  sms_dtype dtype, int64_t B, int64_t H, int64_t Hk,
                                  int64_t Sq, int64_t Sk, int64_t D, float scale,
                                  int is_causal, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* Largest key length Sk the library runs for `dtype` (2^30; 0 for an unknown
 * dtype). */
int64_t sms_max_sk(sms_dtype dtype);

/* Which kernel family a call with these sizes takes (rows 16-byte aligned, no
 * causal rule; a causal forward may take narrower workgroups):
 * 0 = several rows per wavefront, 1 = one wavefront per row, 2 = several
 * wavefronts per row (LDS cross-wave reduction), 3 = streaming (one 1024-lane
 * workgroup per row, two passes: online max/sum, then normalise; for rows of
 * more than 4096 16-byte vectors, but the backward of rows of up to 8192
 * vectors that hold whole vectors stays in 2), 4 = the fp64 kernels (two passes, one
 * wavefront or 256 lanes per row). -1 for an unsupported size or dtype.
 * `backward` selects the backward's choice. Host-only; launches nothing. */
int sms_path(sms_dtype dtype, int64_t Sk, int backward);

/*
 * sms_copy_reference -- dst[0, bytes) = src[0, bytes): a plain device copy,
 * 16 bytes per lane, nontemporal. Not a step of the method: the bandwidth
 * reference for the kernels above, which read their inputs once and write their
 * outputs once where the unfused chain re-reads and re-writes the score tensor
 * at every step (lmnt.cn page, sec. 1.1 and 1.2); a copy of the same bytes
 * with no arithmetic bounds what such a kernel can reach on the same chip.
 *
 *   src, dst   device memory, 16-byte aligned, not overlapping, caller-owned
 *   bytes      a multiple of 16 (else SMS_ERR_ALIGN); 0 is a no-op; at most
 *              (2^32 - 1) / 64 KiB, about 64 GiB (else SMS_ERR_SHAPE)
 *   stream     hipStream_t to enqueue on
 */
sms_status sms_copy_reference(const void* src, void* dst, int64_t bytes, void* stream);

/* Static text naming a status code. */
const char* sms_status_str(sms_status s);

/* SMS_ABI_VERSION of the library that was loaded. */
int sms_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMS_H */
