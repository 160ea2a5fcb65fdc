// api.hip -- the C ABI declared in include/sms.h: argument checks, the choice
// of kernel shape (lanes per row, vectors per lane, row order) and the launch.
//
// Interface after lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into
// PyTorch", sec. 4.2 (forward takes x, an optional mask, scale and is_causal;
// an empty mask means none; runs on the caller's stream) and sec. 4.3 (backward
// takes the saved output y, the upstream gradient and scale), with explicit
// strides and mask-broadcast modes in place of tensor objects.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>

#include "kernels.hpp"
#include "sms.h"

namespace {

using sms::BwdParams;
using sms::FwdParams;
using sms::RowGeom;

// Workgroups are dealt round-robin over the XCDs of an MI355X.
constexpr uint32_t kXcds = 8;
// Query rows per group in a grouped row order (SMS_QBLOCK overrides).
constexpr int kDefaultQBlock = 16;
// The grouped row order (rows sharing a mask row on one XCD, back to back) is
// available on request (SMS_ORDER=grouped); by default rows run in memory
// order, which measured faster on MI355X even for a 128 MB [B,Sq,Sk] mask:
// the x / y streams keep their DRAM-page locality and the re-read mask rows
// are served by the 256 MB Infinity Cache.

int dtype_bytes(sms_dtype d) {
  switch (d) {
    case SMS_F32: return 4;
    case SMS_F16: return 2;
    case SMS_BF16: return 2;
    default: return 0;
  }
}

// Largest vectors-per-row a (TPR, NV) pair in the build covers; longer rows
// take the streaming kernels (one workgroup per row, two passes).
constexpr int64_t kMaxVecPerRow = 1024 * 4;
// Longest row: keeps every in-kernel element index far inside int32.
constexpr int64_t kMaxSk = int64_t(1) << 30;

// Optional override of the lanes per row, for tests and tuning:
// SMS_FORCE_TPR=<4..1024>. Unset or 0 = automatic.
int forced_tpr() {
  const char* s = getenv("SMS_FORCE_TPR");
  return s ? atoi(s) : 0;
}

// Optional override of the row order: SMS_ORDER=rows | grouped. Unset = automatic.
int forced_order() {
  const char* s = getenv("SMS_ORDER");
  if (!s) return -1;
  if (!strcmp(s, "rows")) return 0;
  if (!strcmp(s, "grouped")) return 1;
  return -1;
}

struct Plan {
  int tpr = 0;
  int nv = 0;
};

// Vectors a row may span: ceil(Sk/E) when every row starts on a 16-byte line,
// otherwise up to ceil((Sk + E - 1)/E).
int64_t vectors_per_row(int64_t Sk, int E, bool aligned) {
  return aligned ? (Sk + E - 1) / E : (Sk + 2 * E - 2) / E;
}

// Fewest lanes per row that hold the row in at most `want` vectors per lane,
// then the fewest vectors that cover it; rows too long for 1024 lanes at that
// count take up to 4. Measured on MI355X: the forward runs best at 2 vectors
// per lane up to 256 vectors per row and at 4 beyond; the backward (two input
// streams) at 2 below 256 vectors per row and at 1 from there.
int vectors_per_lane(int64_t nvec, bool backward) {
  if (backward) return nvec >= 256 ? 1 : 2;
  return nvec > 256 ? 4 : 2;
}

bool choose_plan(int64_t nvec, bool backward, Plan& out) {
  const int force = forced_tpr();
  const int want = vectors_per_lane(nvec, backward);
  for (int per_lane : {want, 2, 4}) {
    for (int tpr : sms::kTprList) {
      if (force && tpr != force) continue;
      if (!force && (int64_t)tpr * per_lane < nvec) continue;
      for (int nv : sms::kNvList) {
        if ((int64_t)tpr * nv >= nvec) {
          out.tpr = tpr;
          out.nv = nv;
          return true;
        }
      }
    }
  }
  return false;
}

bool rows_aligned16(const void* base, const int64_t st[4], int64_t B, int64_t H, int64_t Sq,
                    int bytes) {
  if ((uintptr_t)base & 15) return false;
  const int64_t ext[3] = {B, H, Sq};
  for (int d = 0; d < 3; ++d)
    if (ext[d] > 1 && ((st[d] * bytes) & 15)) return false;
  return true;
}

sms_status check_strides(const int64_t st[4]) {
  if (!st) return SMS_ERR_NULL;
  if (st[3] != 1) return SMS_ERR_STRIDE;
  for (int d = 0; d < 3; ++d)
    if (st[d] < 0) return SMS_ERR_STRIDE;
  return SMS_OK;
}

sms_status check_common(sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                        bool& empty) {
  if (dtype_bytes(dtype) == 0) return SMS_ERR_DTYPE;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return SMS_ERR_SHAPE;
  empty = (B == 0 || H == 0 || Sq == 0 || Sk == 0);
  return SMS_OK;
}

sms_status check_sizes(int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  if (Sk > INT32_MAX) return SMS_ERR_SHAPE;
  if (H > UINT32_MAX || Sq > UINT32_MAX || B > UINT32_MAX) return SMS_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > UINT32_MAX) return SMS_ERR_SHAPE;
  const int64_t rows = bh * Sq;
  if (Sq != 0 && rows / Sq != bh) return SMS_ERR_SHAPE;
  if (rows > UINT32_MAX) return SMS_ERR_SHAPE;
  return SMS_OK;
}

bool aligned_to(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}

// The fast path needs whole 16-byte vectors everywhere: every row of every
// operand starts on a 16-byte line and the row length is a multiple of 16
// bytes. SMS_FAST=0 turns it off (tests of the general kernels).
bool fast_ok(int64_t Sk, int bytes) {
  return ((Sk * bytes) & 15) == 0 && env_int("SMS_FAST", 1) != 0;
}

// Rows beyond the register-resident kernels' reach stream; SMS_FORCE_STREAM=1
// sends every row there (tests of the streaming kernels on short rows).
bool use_stream(int64_t nvec) {
  return nvec > kMaxVecPerRow || env_int("SMS_FORCE_STREAM", 0) != 0;
}

// Cache hints of the fast path: nontemporal loads of the streamed inputs and
// nontemporal stores of the outputs (SMS_CACHE_POLICY overrides: bit 1 loads,
// bit 2 stores).
constexpr int kDefaultPolicy = sms::POL_NT_LOAD | sms::POL_NT_STORE;

// Grid for `rows` rows at `tpr` lanes per row; false if it exceeds what one
// dispatch can hold (2^31-1 workgroups, 2^32-1 work-items).
bool grid_for(int64_t rows, int tpr, uint32_t& blocks) {
  const int block = sms::block_of(tpr);
  const int rpb = block / tpr;
  const int64_t nb = (rows + rpb - 1) / rpb;
  if (nb > INT32_MAX || nb * block > (int64_t)UINT32_MAX) return false;
  blocks = (uint32_t)nb;
  return true;
}

}  // namespace

extern "C" {

int sms_abi_version(void) { return SMS_ABI_VERSION; }

const char* sms_status_str(sms_status s) {
  switch (s) {
    case SMS_OK: return "ok";
    case SMS_ERR_NULL: return "a required pointer is NULL";
    case SMS_ERR_SHAPE: return "negative dimension or size beyond the library's limits";
    case SMS_ERR_STRIDE: return "key-axis stride is not 1 or a stride is negative";
    case SMS_ERR_DTYPE: return "unknown dtype";
    case SMS_ERR_MASK_MODE: return "unknown mask mode";
    case SMS_ERR_ALIGN: return "pointer not aligned to its element size";
    case SMS_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int64_t sms_max_sk(sms_dtype dtype) { return dtype_bytes(dtype) ? kMaxSk : 0; }

int sms_path(sms_dtype dtype, int64_t Sk, int backward) {
  const int bytes = dtype_bytes(dtype);
  if (!bytes || Sk < 0 || Sk > kMaxSk) return -1;
  const int64_t nvec = vectors_per_row(Sk, 16 / bytes, true);
  if (use_stream(nvec)) return 3;
  Plan pl;
  if (!choose_plan(nvec, backward != 0, pl)) return -1;
  return pl.tpr < 64 ? 0 : (pl.tpr == 64 ? 1 : 2);
}

sms_status sms_forward(const void* x, const int64_t x_strides[4], const void* mask,
                       sms_mask_mode mask_mode, void* y, const int64_t y_strides[4],
                       sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, float scale,
                       int is_causal, void* stream) {
  bool empty = false;
  sms_status st = check_common(dtype, B, H, Sq, Sk, empty);
  if (st != SMS_OK) return st;
  if ((unsigned)mask_mode > (unsigned)SMS_MASK_FULL) return SMS_ERR_MASK_MODE;
  if (empty) return SMS_OK;
  const bool has_mask = mask_mode != SMS_MASK_NONE;
  if (!x || !y || (has_mask && !mask)) return SMS_ERR_NULL;
  if ((st = check_strides(x_strides)) != SMS_OK) return st;
  if ((st = check_strides(y_strides)) != SMS_OK) return st;
  if ((st = check_sizes(B, H, Sq, Sk)) != SMS_OK) return st;
  const int bytes = dtype_bytes(dtype);
  if (!aligned_to(x, bytes) || !aligned_to(y, bytes) || (has_mask && !aligned_to(mask, bytes)))
    return SMS_ERR_ALIGN;
  if (Sk > kMaxSk) return SMS_ERR_SHAPE;

  const int E = 16 / bytes;
  const bool aligned = rows_aligned16(x, x_strides, B, H, Sq, bytes);
  const int64_t nvec = vectors_per_row(Sk, E, aligned);
  const bool streaming = use_stream(nvec);
  Plan pl;
  if (streaming) {
    pl.tpr = sms::kStreamTpr;
    pl.nv = 0;
  } else if (!choose_plan(nvec, false, pl)) {
    return SMS_ERR_SHAPE;
  }

  FwdParams p;
  p.x = static_cast<const char*>(x);
  p.mask = static_cast<const char*>(mask);
  p.y = static_cast<char*>(y);
  p.sx_b = x_strides[0]; p.sx_h = x_strides[1]; p.sx_q = x_strides[2];
  p.sy_b = y_strides[0]; p.sy_h = y_strides[1]; p.sy_q = y_strides[2];
  p.sm_b = p.sm_h = p.sm_q = 0;
  switch (mask_mode) {
    case SMS_MASK_SQ_SK: p.sm_q = Sk; break;
    case SMS_MASK_B_SQ_SK: p.sm_b = Sq * Sk; p.sm_q = Sk; break;
    case SMS_MASK_B_1_SK: p.sm_b = Sk; break;
    case SMS_MASK_FULL: p.sm_b = H * Sq * Sk; p.sm_h = Sq * Sk; p.sm_q = Sk; break;
    default: break;
  }
  p.scale = scale;
  p.causal = is_causal ? 1 : 0;
  p.has_mask = has_mask ? 1 : 0;

  RowGeom& g = p.g;
  g.B = (uint32_t)B; g.H = (uint32_t)H; g.Sq = (uint32_t)Sq; g.Sk = (uint32_t)Sk;
  g.rows = (uint32_t)(B * H * Sq);
  g.order = sms::ORDER_ROWS;
  g.xcds = kXcds;
  g.members = 1;
  g.qblock = 1;

  // Grouped order: rows that read the same block of mask rows run back to back
  // on one XCD.
  const int rpb = sms::block_of(pl.tpr) / pl.tpr;
  const int64_t Q = std::max(1, env_int("SMS_QBLOCK", kDefaultQBlock));
  int64_t members = 0, groups = 0;
  uint32_t order = sms::ORDER_ROWS;
  if (mask_mode == SMS_MASK_B_SQ_SK) { members = H * Q; groups = B * (Sq / Q); order = sms::ORDER_HEADS; }
  if (mask_mode == SMS_MASK_SQ_SK) { members = B * H * Q; groups = Sq / Q; order = sms::ORDER_SAMPLES; }
  const int fo = forced_order();
  const bool want = fo == 1;
  if (want && members > 1 && Sq % Q == 0 && members % rpb == 0 && groups > 0 &&
      groups % kXcds == 0 && members <= UINT32_MAX) {
    g.order = order;
    g.members = (uint32_t)members;
    g.qblock = (uint32_t)Q;
  }

  uint32_t blocks = 0;
  if (!grid_for(g.rows, pl.tpr, blocks)) return SMS_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (streaming) {
    g.order = sms::ORDER_ROWS;
    switch (dtype) {
      case SMS_F32: e = sms_launch_stream_f32(&p, nullptr, blocks, s); break;
      case SMS_F16: e = sms_launch_stream_f16(&p, nullptr, blocks, s); break;
      default: e = sms_launch_stream_bf16(&p, nullptr, blocks, s); break;
    }
    return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
  }
  if (fast_ok(Sk, bytes) && aligned && rows_aligned16(y, y_strides, B, H, Sq, bytes) &&
      (!has_mask || ((uintptr_t)mask & 15) == 0)) {
    sms::FastFwdArgs fa;
    fa.p = p;
    fa.policy = env_int("SMS_CACHE_POLICY", kDefaultPolicy);
    switch (dtype) {
      case SMS_F32: e = sms_launch_fast_f32(&fa, nullptr, pl.tpr, pl.nv, blocks, s); break;
      case SMS_F16: e = sms_launch_fast_f16(&fa, nullptr, pl.tpr, pl.nv, blocks, s); break;
      default: e = sms_launch_fast_bf16(&fa, nullptr, pl.tpr, pl.nv, blocks, s); break;
    }
    return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
  }
  switch (dtype) {
    case SMS_F32: e = sms_launch_fwd_f32(p, pl.tpr, pl.nv, blocks, s); break;
    case SMS_F16: e = sms_launch_fwd_f16(p, pl.tpr, pl.nv, blocks, s); break;
    default: e = sms_launch_fwd_bf16(p, pl.tpr, pl.nv, blocks, s); break;
  }
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

sms_status sms_backward(const void* y, const int64_t y_strides[4], const void* dy,
                        const int64_t dy_strides[4], void* dx, const int64_t dx_strides[4],
                        sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, float scale,
                        int is_causal, void* stream) {
  bool empty = false;
  sms_status st = check_common(dtype, B, H, Sq, Sk, empty);
  if (st != SMS_OK) return st;
  if (empty) return SMS_OK;
  if (!y || !dy || !dx) return SMS_ERR_NULL;
  if ((st = check_strides(y_strides)) != SMS_OK) return st;
  if ((st = check_strides(dy_strides)) != SMS_OK) return st;
  if ((st = check_strides(dx_strides)) != SMS_OK) return st;
  if ((st = check_sizes(B, H, Sq, Sk)) != SMS_OK) return st;
  const int bytes = dtype_bytes(dtype);
  if (!aligned_to(y, bytes) || !aligned_to(dy, bytes) || !aligned_to(dx, bytes))
    return SMS_ERR_ALIGN;
  if (Sk > kMaxSk) return SMS_ERR_SHAPE;

  const bool aligned = rows_aligned16(y, y_strides, B, H, Sq, bytes);
  const int64_t nvec = vectors_per_row(Sk, 16 / bytes, aligned);
  const bool streaming = use_stream(nvec);
  Plan pl;
  if (streaming) {
    pl.tpr = sms::kStreamTpr;
    pl.nv = 0;
  } else if (!choose_plan(nvec, true, pl)) {
    return SMS_ERR_SHAPE;
  }

  BwdParams p;
  p.y = static_cast<const char*>(y);
  p.dy = static_cast<const char*>(dy);
  p.dx = static_cast<char*>(dx);
  p.sy_b = y_strides[0]; p.sy_h = y_strides[1]; p.sy_q = y_strides[2];
  p.sd_b = dy_strides[0]; p.sd_h = dy_strides[1]; p.sd_q = dy_strides[2];
  p.sx_b = dx_strides[0]; p.sx_h = dx_strides[1]; p.sx_q = dx_strides[2];
  p.scale = scale;
  p.causal = is_causal ? 1 : 0;
  RowGeom& g = p.g;
  g.B = (uint32_t)B; g.H = (uint32_t)H; g.Sq = (uint32_t)Sq; g.Sk = (uint32_t)Sk;
  g.rows = (uint32_t)(B * H * Sq);
  g.order = sms::ORDER_ROWS;
  g.xcds = kXcds;
  g.members = 1;
  g.qblock = 1;

  uint32_t blocks = 0;
  if (!grid_for(g.rows, pl.tpr, blocks)) return SMS_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (streaming) {
    switch (dtype) {
      case SMS_F32: e = sms_launch_stream_f32(nullptr, &p, blocks, s); break;
      case SMS_F16: e = sms_launch_stream_f16(nullptr, &p, blocks, s); break;
      default: e = sms_launch_stream_bf16(nullptr, &p, blocks, s); break;
    }
    return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
  }
  if (fast_ok(Sk, bytes) && aligned && rows_aligned16(dy, dy_strides, B, H, Sq, bytes) &&
      rows_aligned16(dx, dx_strides, B, H, Sq, bytes)) {
    sms::FastBwdArgs ba;
    ba.p = p;
    ba.policy = env_int("SMS_CACHE_POLICY", kDefaultPolicy);
    switch (dtype) {
      case SMS_F32: e = sms_launch_fast_f32(nullptr, &ba, pl.tpr, pl.nv, blocks, s); break;
      case SMS_F16: e = sms_launch_fast_f16(nullptr, &ba, pl.tpr, pl.nv, blocks, s); break;
      default: e = sms_launch_fast_bf16(nullptr, &ba, pl.tpr, pl.nv, blocks, s); break;
    }
    return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
  }
  switch (dtype) {
    case SMS_F32: e = sms_launch_bwd_f32(p, pl.tpr, pl.nv, blocks, s); break;
    case SMS_F16: e = sms_launch_bwd_f16(p, pl.tpr, pl.nv, blocks, s); break;
    default: e = sms_launch_bwd_bf16(p, pl.tpr, pl.nv, blocks, s); break;
  }
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

}  // extern "C"
