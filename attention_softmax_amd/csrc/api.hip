// api.hip -- the C ABI declared in include/sms.h: argument checks, the choice
// of kernel family and shape (lanes per row, vectors per lane) and the launch.
//
// Interface after lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into
// PyTorch", sec. 4.2 (forward takes x, an optional mask, scale and is_causal;
// an empty mask means none; runs on the caller's stream) and sec. 4.3 (backward
// takes the saved output y, the upstream gradient and scale), with explicit
// strides and mask modes in place of tensor objects.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <utility>

#include "kernels.hpp"
#include "sms.h"

namespace {

using sms::BwdParams;
using sms::FwdParams;
using sms::RowGeom;

// Largest vectors-per-row a (TPR, NV) pair in the build covers; longer rows
// take the streaming kernels (one workgroup per row, two passes).
constexpr int64_t kMaxVecPerRow = 1024 * 4;
// Longest row: keeps every in-kernel element index far inside int32.
constexpr int64_t kMaxSk = int64_t(1) << 30;
// Split rows (calls with a workspace): rows are split when there are fewer
// than kSplitRowsBelow of them (one workgroup per row would leave CUs idle)
// and each holds at least kSplitMinVec vectors (256 KB; shorter rows finish
// sooner at one workgroup each than the split's two launches take); chunks of
// at least kSplitMinChunk vectors (16 KB), aiming at kSplitTargetWgs
// workgroups in all. The grid's second dimension holds at most kSplitGridRows
// rows. Measured on MI355X (fp16/bf16/fp32, 1 to 1024 rows of 16K-4M keys):
// 8 fp16 rows of 2^20 keys 158 -> 25 us, one bf16 row of 2^22 keys 675 ->
// 25 us; 64 fp32 rows of 16384 keys 13 -> 24 us (hence the length floor).
constexpr int64_t kSplitRowsBelow = 256;
constexpr int64_t kSplitMinVec = 16384;
constexpr int64_t kSplitMinChunk = 1024;
constexpr int64_t kSplitTargetWgs = 2048;
constexpr int64_t kSplitGridRows = 65535;

int dtype_bytes(sms_dtype d) {
  switch (d) {
    case SMS_F32: return 4;
    case SMS_F16: return 2;
    case SMS_BF16: return 2;
    case SMS_F64: return 8;
    default: return 0;
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}

// Tuning and test overrides, read per call:
//   SMS_FORCE_TPR=<4..1024>  lanes per row (0 = automatic)
//   SMS_FAST=0               never take the aligned-row kernels
//   SMS_FORCE_STREAM=1       take the streaming kernels for every row
//   SMS_FORCE_SPLIT=<C>      split every row into C chunks (calls with a workspace)
//   SMS_SPLIT=0              never split rows
struct Plan {
  int family = sms::FAMILY_GENERAL;
  int tpr = 0;
  int nv = 0;
  int64_t chunks = 1, chunk_vec = 0;  // FAMILY_SPLIT
};

// Vectors a row may span: ceil(Sk/E) when every row starts on a 16-byte line,
// otherwise up to ceil((Sk + E - 1)/E).
int64_t vectors_per_row(int64_t Sk, int E, bool aligned) {
  return aligned ? (Sk + E - 1) / E : (Sk + 2 * E - 2) / E;
}

bool use_stream(int64_t nvec) {
  return nvec > kMaxVecPerRow || env_int("SMS_FORCE_STREAM", 0) != 0;
}

// Longest row (16-byte vectors) the aligned backward holds in VGPRs at 1024
// lanes x 8 vectors: one pass where the streaming kernels take two. Measured
// on MI355X (us, streaming -> one pass): fp16 rows of 65536 keys (8192 rows)
// 730 -> 575, causal 719 -> 585; of 40000 keys (13416 rows) 662 -> 550,
// causal 625 -> 582. The forward at 1024 x 8 measured equal to the streaming
// kernels (425 against 430 us, 451 against 445) and keeps them.
// Rows that keep few of their keys (a top-left causal rule over Sq << Sk)
// are mostly zero stores, which the streaming kernels' two workgroups per CU
// issue faster: fp16 [1,8,1677,40000] top-left causal 197 us streaming against
// 265 in one pass. The one pass is taken when the causal rule keeps at least
// half of the keys overall.
constexpr int64_t kMaxVecPerRowBwd = 1024 * 8;
// Sum over t = 1 .. n of min(t, Sk) (0 for n <= 0).
__int128 kept_prefix(int64_t n, int64_t Sk) {
  if (n <= 0) return 0;
  if (n <= Sk) return (__int128)n * (n + 1) / 2;
  return (__int128)Sk * (Sk + 1) / 2 + (__int128)(n - Sk) * Sk;
}
// Keys the causal rule keeps over all Sq rows of a (b, h) plane, at least half of Sq * Sk.
bool keeps_half(int64_t Sq, int64_t Sk, int causal) {
  if (causal == SMS_CAUSAL_NONE) return true;
  const int64_t d = causal == SMS_CAUSAL_BOTTOM_RIGHT ? Sk - Sq : 0;
  const __int128 kept = kept_prefix(Sq + d, Sk) - kept_prefix(d, Sk);
  return 2 * kept >= (__int128)Sq * Sk;
}
bool bwd_one_pass_long(int64_t nvec) {
  return nvec > kMaxVecPerRow && nvec <= kMaxVecPerRowBwd && env_int("SMS_FORCE_STREAM", 0) == 0 &&
         env_int("SMS_FORCE_TPR", 0) == 0;
}

// Chunks per row for `rows` rows of up to `nvec` vectors: 1 = no split.
int64_t split_chunks(int64_t rows, int64_t nvec) {
  if (rows > kSplitGridRows || nvec < 1) return 1;
  const int force = env_int("SMS_FORCE_SPLIT", 0);
  if (force > 0) return std::min<int64_t>(force, nvec);
  if (env_int("SMS_SPLIT", 1) == 0 || rows >= kSplitRowsBelow || nvec < kSplitMinVec) return 1;
  const int64_t want = (kSplitTargetWgs + rows - 1) / rows;
  return std::max<int64_t>(1, std::min(want, nvec / kSplitMinChunk));
}

// Vectors per chunk for `chunks` chunks of a row of nvec vectors: a multiple
// of the workgroup width (unless forced), then the chunk count that covers
// the row at that size (never more than asked for).
void split_shape(int64_t nvec, int64_t chunks, Plan& pl) {
  int64_t cv = (nvec + chunks - 1) / chunks;
  if (env_int("SMS_FORCE_SPLIT", 0) <= 0)
    cv = (cv + sms::kSplitTpr - 1) / sms::kSplitTpr * sms::kSplitTpr;
  pl.family = sms::FAMILY_SPLIT;
  pl.chunk_vec = cv;
  pl.chunks = (nvec + cv - 1) / cv;
}

// Workspace bytes of a split launch: 8 per (row, chunk); 0 without a split.
// Sized for unaligned rows, which span the most vectors.
int64_t workspace_bytes(int64_t rows, int64_t Sk, int E) {
  const int64_t c = split_chunks(rows, vectors_per_row(Sk, E, false));
  return c > 1 ? rows * c * 8 : 0;
}

// 16-byte vectors per lane for a row of nvec vectors, from sweeps of every
// width on MI355X (fp32/fp16/bf16 rows of 125 to 1024 vectors, causal and
// not): one vector per lane (the widest workgroup) wins for the backward up to
// 512 vectors and for the forward up to 128, and up to 512 when no causal
// bound cuts the loads short; causal forward rows keep two vectors per lane,
// which halves the lanes that only store zeros. Longer rows: two, then four.
int vectors_per_lane(int64_t nvec, bool backward, bool causal) {
  if (nvec <= 128 || (nvec <= 512 && (backward || !causal))) return 1;
  return nvec <= 2048 ? 2 : 4;
}

// Fewest lanes per row that hold the row at vectors_per_lane() vectors per
// lane, then the fewest vectors that cover it; rows too long for 1024 lanes at
// that count take up to 4.
bool choose_plan(int64_t nvec, bool backward, bool causal, Plan& out) {
  if (use_stream(nvec)) {
    out.family = sms::FAMILY_STREAM;
    out.tpr = sms::kStreamTpr;
    out.nv = 0;
    return true;
  }
  const int force = env_int("SMS_FORCE_TPR", 0);
  const int want = vectors_per_lane(nvec, backward, causal);
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

// Heads per workgroup for an aligned forward plan (1: one row per
// workgroup). A group takes query q of G heads that read the same mask row,
// so the mask (a stride of 0 over heads) is read once for them and their
// reductions share two barriers. Needs G | H and a plan the head-group kernels
// are built for (heads_built). Automatic choice: two heads for rows of 65 to
// 128 vectors (128 lanes, one vector each) that have a causal rule or a mask,
// where the per-row fixed cost is largest: measured on MI355X (us, one row
// per workgroup -> two heads) fp16 [8,32,1024,1024] causal 158 -> 128; bf16
// [16,16,1000,1000] with a [1000,1000] mask 185 -> 175, causal 177 -> 138;
// fp16 [8,16,800,800] with key padding 68 -> 57. Without either the two are
// within run-to-run noise (fp16 [8,32,1024,1024] 168 / 165, fp32
// [16,32,512,512] 161 / 166). Longer rows gain at most 2 % and some lose
// (fp32 [8,32,1024,1024] with key padding 319 -> 340; fp16 [4,32,2048,2048]
// causal 255 -> 280; fp16 [4,32,4096,4096] with a [4,4096,4096] mask, causal,
// 1095 -> 1153), so they keep one row per workgroup. Groups of consecutive
// rows instead of heads, forward or backward, measured no better.
// SMS_HEADS=<1|2|4> overrides the choice.
int heads_per_group(const Plan& pl, int64_t H, int64_t mask_head_stride, bool causal,
                    bool has_mask) {
  if (mask_head_stride != 0) return 1;
  int want = env_int("SMS_HEADS", 0);
  if (want == 0) want = (pl.tpr == 128 && pl.nv == 1 && (causal || has_mask)) ? 2 : 1;
  for (int g : sms::kHeadsList)
    if (g == want && H % g == 0 && sms::heads_built(pl.tpr, pl.nv, g)) return g;
  return 1;
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
                        int is_causal, bool& empty) {
  if (dtype_bytes(dtype) == 0) return SMS_ERR_DTYPE;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return SMS_ERR_SHAPE;
  if (is_causal < SMS_CAUSAL_NONE || is_causal > SMS_CAUSAL_BOTTOM_RIGHT) return SMS_ERR_CAUSAL;
  empty = (B == 0 || H == 0 || Sq == 0 || Sk == 0);
  return SMS_OK;
}

sms_status check_sizes(int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  if (Sk > kMaxSk) return SMS_ERR_SHAPE;
  if (H > UINT32_MAX || Sq > UINT32_MAX || B > UINT32_MAX) return SMS_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > UINT32_MAX) return SMS_ERR_SHAPE;
  const int64_t rows = bh * Sq;
  if (rows / Sq != bh || rows > UINT32_MAX) return SMS_ERR_SHAPE;
  return SMS_OK;
}

bool aligned_to(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

// Element strides of a mask over [B, H, Sq, Sk] scores (keys contiguous; 0 on
// broadcast axes; nothing to index for key lengths).
void mask_strides(int shape_mode, int64_t H, int64_t Sq, int64_t Sk, int64_t& sb, int64_t& sh,
                  int64_t& sq) {
  sb = sh = sq = 0;
  switch (shape_mode) {
    case SMS_MASK_SQ_SK: sq = Sk; break;
    case SMS_MASK_B_SQ_SK: sb = Sq * Sk; sq = Sk; break;
    case SMS_MASK_B_1_SK: sb = Sk; break;
    case SMS_MASK_FULL: sb = H * Sq * Sk; sh = Sq * Sk; sq = Sk; break;
    default: break;
  }
}

// Every row (b, h, q) of the tensor starts on a 128-byte line and fills whole
// lines: the base, every stride of a non-trivial axis and the row length are
// multiples of 128 bytes.
bool rows_line_exact(const void* p, const int64_t st[4], int64_t B, int64_t H, int64_t Sq,
                     int64_t Sk, int bytes) {
  if (((uintptr_t)p & 127) != 0 || ((Sk * bytes) & 127) != 0) return false;
  if (B > 1 && ((st[0] * bytes) & 127) != 0) return false;
  if (H > 1 && ((st[1] * bytes) & 127) != 0) return false;
  if (Sq > 1 && ((st[2] * bytes) & 127) != 0) return false;
  return true;
}

// Grid for `rows` rows; false if it exceeds what one dispatch holds (2^31-1
// workgroups, 2^32-1 work-items).
bool grid_for(int64_t rows, const Plan& pl, uint32_t& blocks) {
  if (pl.family == sms::FAMILY_SPLIT) {  // grid chunks x rows, 256 lanes
    if (rows > kSplitGridRows || pl.chunks * rows * sms::kSplitTpr > (int64_t)UINT32_MAX)
      return false;
    blocks = (uint32_t)rows;
    return true;
  }
  const bool st = pl.family == sms::FAMILY_STREAM;
  const int block = st ? sms::kStreamTpr : sms::block_of(pl.tpr);
  const int rpb = st ? 1 : block / pl.tpr;
  const int64_t nb = (rows + rpb - 1) / rpb;
  if (nb > INT32_MAX || nb * block > (int64_t)UINT32_MAX) return false;
  blocks = (uint32_t)nb;
  return true;
}

void fill_geom(RowGeom& g, int64_t B, int64_t H, int64_t Sq, int64_t Sk) {
  g.B = (uint32_t)B;
  g.H = (uint32_t)H;
  g.Sq = (uint32_t)Sq;
  g.Sk = (uint32_t)Sk;
  g.rows = (uint32_t)(B * H * Sq);
  g.div_sq = sms::make_fastdiv(g.Sq);
  g.div_h = sms::make_fastdiv(g.H);
}

hipError_t launch(sms_dtype dtype, const FwdParams* fp, const BwdParams* bp, const Plan& pl,
                  uint32_t blocks, hipStream_t s) {
  if (pl.family == sms::FAMILY_F64) return sms_launch_f64(fp, bp, pl.tpr, blocks, s);
  switch (dtype) {
    case SMS_F32: return sms_launch_f32(fp, bp, pl.family, pl.tpr, pl.nv, blocks, s);
    case SMS_F16: return sms_launch_f16(fp, bp, pl.family, pl.tpr, pl.nv, blocks, s);
    default: return sms_launch_bf16(fp, bp, pl.family, pl.tpr, pl.nv, blocks, s);
  }
}

// Scratch for sms_forward_noalloc: the split forward's per-(row, chunk)
// partials live in this file-scope device array instead of a caller
// workspace. One copy per GPU, held until the process ends. The largest split
// the plan chooses by itself takes rows * chunks <= 2048 + 255 pairs of 8 bytes
// (18,424 bytes); 64 KiB leaves room for small forced splits.
constexpr int64_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`. Host code never
// passes the array's own name (a host-side stand-in) to a kernel or a copy.
sms_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMS_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SMS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SMS_OK;
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
    case SMS_ERR_CAUSAL: return "unknown causal mode";
    case SMS_ERR_WORKSPACE: return "workspace smaller than sms_workspace_bytes() asks for";
    default: return "unknown status";
  }
}

int64_t sms_max_sk(sms_dtype dtype) { return dtype_bytes(dtype) ? kMaxSk : 0; }

int sms_path(sms_dtype dtype, int64_t Sk, int backward) {
  const int bytes = dtype_bytes(dtype);
  if (!bytes || Sk < 0 || Sk > kMaxSk) return -1;
  if (dtype == SMS_F64) return 4;
  Plan pl;
  const int64_t nvec = vectors_per_row(Sk, 16 / bytes, true);
  if (backward && ((Sk * bytes) & 15) == 0 && bwd_one_pass_long(nvec)) return 2;
  if (!choose_plan(nvec, backward != 0, false, pl)) return -1;
  if (pl.family == sms::FAMILY_STREAM) return 3;
  return pl.tpr < 64 ? 0 : (pl.tpr == 64 ? 1 : 2);
}

int64_t sms_workspace_bytes(sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                            int backward) {
  (void)backward;  // 8 bytes per (row, chunk) either way
  const int bytes = dtype_bytes(dtype);
  if (!bytes || B < 0 || H < 0 || Sq < 0 || Sk < 0) return -1;
  if (B == 0 || H == 0 || Sq == 0 || Sk == 0) return 0;
  if (check_sizes(B, H, Sq, Sk) != SMS_OK) return -1;
  if (dtype == SMS_F64) return 0;  // the fp64 kernels never split rows
  return workspace_bytes(B * H * Sq, Sk, 16 / bytes);
}

sms_status sms_forward(const void* x, const int64_t x_strides[4], const void* mask,
                       int mask_mode, void* y, const int64_t y_strides[4], sms_dtype dtype,
                       int64_t B, int64_t H, int64_t Sq, int64_t Sk, float scale, int is_causal,
                       void* stream) {
  return sms_forward_ws(x, x_strides, mask, mask_mode, y, y_strides, dtype, B, H, Sq, Sk, scale,
                        is_causal, nullptr, 0, stream);
}

int64_t sms_noalloc_scratch_bytes(void) { return kScratchBytes; }

sms_status sms_forward_noalloc(const void* x, const int64_t x_strides[4], const void* mask,
                               int mask_mode, void* y, const int64_t y_strides[4],
                               sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                               float scale, int is_causal, void* stream) {
  // The same validation and kernels as sms_forward_ws, with this device's
  // scratch as the workspace: a split that needs more than kScratchBytes is
  // SMS_ERR_WORKSPACE there, before anything is launched. The split kernels
  // write every partial they later read, so nothing needs clearing.
  void* ws = nullptr;
  const sms_status st = scratch_of_current_device(&ws);
  if (st != SMS_OK) return st;
  return sms_forward_ws(x, x_strides, mask, mask_mode, y, y_strides, dtype, B, H, Sq, Sk, scale,
                        is_causal, ws, kScratchBytes, stream);
}

sms_status sms_forward_ws(const void* x, const int64_t x_strides[4], const void* mask,
                          int mask_mode, void* y, const int64_t y_strides[4], sms_dtype dtype,
                          int64_t B, int64_t H, int64_t Sq, int64_t Sk, float scale,
                          int is_causal, void* workspace, int64_t workspace_bytes_given,
                          void* stream) {
  bool empty = false;
  sms_status st = check_common(dtype, B, H, Sq, Sk, is_causal, empty);
  if (st != SMS_OK) return st;
  const bool is_bool = (mask_mode & SMS_MASK_BOOL) != 0;
  const int shape_mode = mask_mode & ~SMS_MASK_BOOL;
  if (shape_mode < SMS_MASK_NONE || shape_mode > SMS_MASK_KEY_LENGTHS) return SMS_ERR_MASK_MODE;
  if (is_bool && (shape_mode == SMS_MASK_NONE || shape_mode == SMS_MASK_KEY_LENGTHS))
    return SMS_ERR_MASK_MODE;
  if (empty) return SMS_OK;
  const bool has_mask = shape_mode != SMS_MASK_NONE;
  if (!x || !y || (has_mask && !mask)) return SMS_ERR_NULL;
  if ((st = check_strides(x_strides)) != SMS_OK) return st;
  if ((st = check_strides(y_strides)) != SMS_OK) return st;
  if ((st = check_sizes(B, H, Sq, Sk)) != SMS_OK) return st;
  const int bytes = dtype_bytes(dtype);
  const int mask_bytes = shape_mode == SMS_MASK_KEY_LENGTHS ? 4 : (is_bool ? 1 : bytes);
  if (!aligned_to(x, bytes) || !aligned_to(y, bytes) ||
      (has_mask && !aligned_to(mask, mask_bytes)))
    return SMS_ERR_ALIGN;
  const int E = 16 / bytes;
  const bool f64 = dtype == SMS_F64;
  const int64_t need = workspace && !f64 ? workspace_bytes(B * H * Sq, Sk, E) : 0;
  if (need > 0 && (workspace_bytes_given < need || !aligned_to(workspace, 8)))
    return SMS_ERR_WORKSPACE;

  const bool aligned = rows_aligned16(x, x_strides, B, H, Sq, bytes);
  const int64_t nvec = vectors_per_row(Sk, E, aligned);
  Plan pl;
  if (f64) {
    pl.family = sms::FAMILY_F64;
    pl.tpr = sms::f64_tpr(Sk);
  } else if (!choose_plan(nvec, false, is_causal != 0, pl)) {
    return SMS_ERR_SHAPE;
  }
  const int64_t chunks = need > 0 ? split_chunks(B * H * Sq, nvec) : 1;
  if (chunks > 1) split_shape(nvec, chunks, pl);

  FwdParams p;
  p.x = static_cast<const char*>(x);
  p.mask = static_cast<const char*>(mask);
  p.y = static_cast<char*>(y);
  p.sx_b = x_strides[0]; p.sx_h = x_strides[1]; p.sx_q = x_strides[2];
  p.sy_b = y_strides[0]; p.sy_h = y_strides[1]; p.sy_q = y_strides[2];
  mask_strides(shape_mode, H, Sq, Sk, p.sm_b, p.sm_h, p.sm_q);
  p.scale = scale;
  p.causal = is_causal;
  p.lines = rows_line_exact(x, x_strides, B, H, Sq, Sk, bytes) &&
            rows_line_exact(y, y_strides, B, H, Sq, Sk, bytes);
  p.mask_kind = !has_mask ? sms::MASK_NONE
                : shape_mode == SMS_MASK_KEY_LENGTHS ? sms::MASK_LEN
                : is_bool ? sms::MASK_BOOL : sms::MASK_ADD;
  fill_geom(p.g, B, H, Sq, Sk);
  p.chunks = (uint32_t)pl.chunks;
  p.chunk_vec = (uint32_t)pl.chunk_vec;
  p.ws = static_cast<float2*>(workspace);
  p.heads = 1;
  p.div_hg = sms::make_fastdiv(1);
  // Only a causal rule or key lengths can leave a wavefront with no key.
  p.early = (is_causal != 0 || p.mask_kind == sms::MASK_LEN) && env_int("SMS_EARLY", 1) != 0;

  if (pl.family != sms::FAMILY_STREAM && pl.family != sms::FAMILY_SPLIT && !f64) {
    // Aligned-row kernels: every operand's rows on 16-byte lines, whole vectors.
    const bool mask_whole = !has_mask || p.mask_kind == sms::MASK_LEN ||
                            (p.mask_kind == sms::MASK_ADD && ((uintptr_t)mask & 15) == 0) ||
                            (p.mask_kind == sms::MASK_BOOL && ((uintptr_t)mask % E) == 0);
    if (((Sk * bytes) & 15) == 0 && env_int("SMS_FAST", 1) != 0 && aligned && mask_whole &&
        rows_aligned16(y, y_strides, B, H, Sq, bytes))
      pl.family = sms::FAMILY_ALIGNED;
  }

  uint32_t blocks = 0;
  if (!grid_for(p.g.rows, pl, blocks)) return SMS_ERR_SHAPE;
  const int heads = pl.family == sms::FAMILY_ALIGNED
                        ? heads_per_group(pl, H, p.sm_h, is_causal != 0, has_mask)
                        : 1;
  if (heads > 1) {
    pl.family = sms::FAMILY_HEADS;
    p.heads = (uint32_t)heads;
    p.div_hg = sms::make_fastdiv((uint32_t)(H / heads));
    blocks = p.g.rows / (uint32_t)heads;
  }
  const hipError_t e = launch(dtype, &p, nullptr, pl, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

sms_status sms_backward(const void* y, const int64_t y_strides[4], const void* dy,
                        const int64_t dy_strides[4], void* dx, const int64_t dx_strides[4],
                        sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk, float scale,
                        int is_causal, void* stream) {
  return sms_backward_ws(y, y_strides, dy, dy_strides, dx, dx_strides, dtype, B, H, Sq, Sk, scale,
                         is_causal, nullptr, 0, stream);
}

sms_status sms_backward_ws(const void* y, const int64_t y_strides[4], const void* dy,
                           const int64_t dy_strides[4], void* dx, const int64_t dx_strides[4],
                           sms_dtype dtype, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
                           float scale, int is_causal, void* workspace,
                           int64_t workspace_bytes_given, void* stream) {
  bool empty = false;
  sms_status st = check_common(dtype, B, H, Sq, Sk, is_causal, empty);
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
  const int E = 16 / bytes;
  const bool f64 = dtype == SMS_F64;
  const int64_t need = workspace && !f64 ? workspace_bytes(B * H * Sq, Sk, E) : 0;
  if (need > 0 && (workspace_bytes_given < need || !aligned_to(workspace, 8)))
    return SMS_ERR_WORKSPACE;

  const bool aligned = rows_aligned16(y, y_strides, B, H, Sq, bytes);
  const int64_t nvec = vectors_per_row(Sk, E, aligned);
  // Every operand's rows on 16-byte lines holding whole vectors: the aligned kernels.
  const bool fast_rows = !f64 && ((Sk * bytes) & 15) == 0 && env_int("SMS_FAST", 1) != 0 &&
                         aligned && rows_aligned16(dy, dy_strides, B, H, Sq, bytes) &&
                         rows_aligned16(dx, dx_strides, B, H, Sq, bytes);
  Plan pl;
  if (f64) {
    pl.family = sms::FAMILY_F64;
    pl.tpr = sms::f64_tpr(Sk);
  } else if (fast_rows && bwd_one_pass_long(nvec) && keeps_half(Sq, Sk, is_causal)) {
    pl.family = sms::FAMILY_ALIGNED;
    pl.tpr = 1024;
    pl.nv = 8;
  } else if (!choose_plan(nvec, true, is_causal != 0, pl)) {
    return SMS_ERR_SHAPE;
  }
  const int64_t chunks = need > 0 ? split_chunks(B * H * Sq, nvec) : 1;
  if (chunks > 1) split_shape(nvec, chunks, pl);

  BwdParams p;
  p.y = static_cast<const char*>(y);
  p.dy = static_cast<const char*>(dy);
  p.dx = static_cast<char*>(dx);
  p.sy_b = y_strides[0]; p.sy_h = y_strides[1]; p.sy_q = y_strides[2];
  p.sd_b = dy_strides[0]; p.sd_h = dy_strides[1]; p.sd_q = dy_strides[2];
  p.sx_b = dx_strides[0]; p.sx_h = dx_strides[1]; p.sx_q = dx_strides[2];
  p.scale = scale;
  p.causal = is_causal;
  p.lines = rows_line_exact(y, y_strides, B, H, Sq, Sk, bytes) &&
            rows_line_exact(dy, dy_strides, B, H, Sq, Sk, bytes) &&
            rows_line_exact(dx, dx_strides, B, H, Sq, Sk, bytes);
  fill_geom(p.g, B, H, Sq, Sk);
  p.chunks = (uint32_t)pl.chunks;
  p.chunk_vec = (uint32_t)pl.chunk_vec;
  p.ws = static_cast<double*>(workspace);
  // Only the causal promise can leave a wavefront with no key.
  p.early = is_causal != 0 && env_int("SMS_EARLY", 1) != 0;

  if (pl.family != sms::FAMILY_STREAM && pl.family != sms::FAMILY_SPLIT && fast_rows)
    pl.family = sms::FAMILY_ALIGNED;

  uint32_t blocks = 0;
  if (!grid_for(p.g.rows, pl, blocks)) return SMS_ERR_SHAPE;
  const hipError_t e = launch(dtype, nullptr, &p, pl, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SMS_OK : SMS_ERR_HIP;
}

}  // extern "C"
