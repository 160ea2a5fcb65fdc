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
  int mask_vec;      // every mask row starts on 4 elements and Sk % 4 == 0 (runs of 4 keys)
  int mask_tile;     // additive, every mask row starts on a 16-byte line (mask tiles in LDS)
};

enum : int { ATTN_MASK_NONE = 0, ATTN_MASK_ADD = 1, ATTN_MASK_BOOL = 2, ATTN_MASK_LEN = 3 };

// Backward: dQ, dK, dV of L = sum(dO * O) given the forward's O and LSE.
struct AttnBwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* o;
  const char* dout;  // dO
  const char* mask;  // as in AttnParams
  const float* lse;  // [B, H, Sq] from the forward
  float* delta;      // workspace [B, H, Sq]: rowsum(dO * O)
  char* dq;
  char* dk;
  char* dv;
  int64_t sq_b, sq_h, sq_s;
  int64_t sk_b, sk_h, sk_s;
  int64_t sv_b, sv_h, sv_s;
  int64_t so_b, so_h, so_s;    // O
  int64_t sdo_b, sdo_h, sdo_s; // dO
  int64_t sdq_b, sdq_h, sdq_s;
  int64_t sdk_b, sdk_h, sdk_s;
  int64_t sdv_b, sdv_h, sdv_s;
  int64_t sm_b, sm_h, sm_q;
  uint32_t B, H, Hk, Sq, Sk;
  uint32_t group;
  float scale;       // the forward's scale
  float scale_log2;  // scale * log2(e)
  int causal;
  int mask_kind;
  int mask_vec;      // as in AttnParams
  int mask_tile;     // as in AttnParams
};

// Keys per workgroup of the dK / dV kernel (four wavefronts x 32); the
// queries per tile it streams are a template parameter of that kernel.
constexpr int kAttnBwdBk = 128;

// Queries per workgroup (four wavefronts of 32 queries) and keys per tile.
// A compile-time bool carried by a value (for generic lambdas).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

constexpr int kAttnBq = 128;
constexpr int kAttnBk = 64;

// Device helpers shared by the forward and backward kernels.
namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2eA = 1.4426950408889634f;
constexpr float kLn2A = 0.6931471805599453f;
constexpr float kNegInfA = -__builtin_inff();
// Growth of the row maximum (log2 units) that the running output absorbs
// before it is rescaled; probabilities stay below 2^kLazy.
constexpr float kLazy = 8.0f;

template <bool BF16>
__device__ inline __attribute__((always_inline)) f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values to a packed pair of 16-bit values, round to nearest even.
template <bool BF16>
__device__ inline __attribute__((always_inline)) uint32_t pack2(float a, float b) {
  if constexpr (BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <bool BF16>
__device__ inline __attribute__((always_inline)) float to_float(uint32_t bits16) {
  if constexpr (BF16) return __uint_as_float(bits16 << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// The value of lane l ^ 32 (same query, the other 16 keys of a 32-key block).
__device__ inline __attribute__((always_inline)) float other_half_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline __attribute__((always_inline)) float other_half_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A raw buffer (stride 0) over `rows` rows of `row_bytes` bytes, `pitch`
// bytes apart, from `base` (wave-uniform): loads at offsets past the last
// row's bytes return zero without touching memory. Row pitches are at most
// 2^25 bytes (checked on the host), so a tile of up to 64 rows fits the
// 31-bit record count.
constexpr int kRsrcWord3A = 0x00020000;  // fourth descriptor word of a raw buffer (gfx9)
__device__ inline __attribute__((always_inline)) __amdgpu_buffer_rsrc_t
rows_rsrc(const char* base, int rows, int64_t pitch, int row_bytes) {
  const int bytes = rows > 0 ? (int)((int64_t)(rows - 1) * pitch + row_bytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, bytes, kRsrcWord3A);
}
// Scheduling of a run of N matrix products fed from LDS, RPP reads per
// product: the reads of the first LA products go out together, then each
// product is followed by the reads of the one LA places later, so that every
// read has LA products' time to arrive. (Left to itself the scheduler issues
// each read just before its product and waits on it, holding few registers.)
// Applies to the scheduling region it is placed in, after the products.
template <int N, int LA, int RPP>
__device__ inline __attribute__((always_inline)) void pin_reads_ahead() {
  constexpr int L = LA < N ? LA : N;
  __builtin_amdgcn_sched_group_barrier(0x100, RPP * L, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - L; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one product
    __builtin_amdgcn_sched_group_barrier(0x100, RPP, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, L, 0);
}

// Tiles loaded straight from global memory into LDS (buffer loads with the
// LDS flag): rows of D 16-bit values in 16-byte chunks, no padding. A load
// instruction fills 1 KB of LDS in lane order, so the conflict-free layout
// comes from which chunk each lane fetches: chunk position h of row r holds
// logical chunk h ^ dswz<D>(r). The swizzle suits both operand read
// patterns: 16-byte row reads (a 16-lane phase reads one logical chunk of 16
// consecutive rows, so dswz must be one-to-one on every aligned 16 rows, and
// for D = 64, where two rows share a 256-byte bank line, on each parity class
// of them) and transposing 8-byte reads (a 32-lane phase reads 4 consecutive
// rows x 4 consecutive chunks, so bits 2-3 of dswz -- bit 2 for D = 64 --
// must differ over every aligned 4 rows).
// (D = 32 is the layout of 64-byte rows of bytes, four chunks: a boolean mask
// tile; its reads are row reads.)
template <int D>
__host__ __device__ constexpr int dswz(int r) {
  return D == 128  ? (((r & 3) << 2) | ((r >> 2) & 3))
         : D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                   : ((r >> 2) & 3);
}
// Byte offset of logical chunk ch of row r in such a tile.
template <int D>
__host__ __device__ constexpr int dtile_off(int r, int ch) {
  return r * D * 2 + ((ch ^ dswz<D>(r)) * 16);
}
template <int D>
constexpr bool dswz_conflict_free() {
  constexpr int CH = D / 8;
  for (int r0 = 0; r0 < 64; r0 += 16)  // row reads: 16 rows, one chunk
    for (int ch = 0; ch < CH; ++ch) {
      bool used[16] = {};
      for (int r = r0; r < r0 + 16; ++r) {
        const int grp = (dtile_off<D>(r, ch) / 16) % 16;  // 4-bank group of the 64 banks
        if (used[grp]) return false;
        used[grp] = true;
      }
    }
  for (int r0 = 0; r0 < 64; r0 += 4)  // transposing reads: 4 rows x 4 chunks
    for (int c0 = 0; c0 < CH; c0 += 4) {
      bool used[16] = {};
      for (int r = r0; r < r0 + 4; ++r)
        for (int ch = c0; ch < c0 + 4; ++ch) {
          const int grp = (dtile_off<D>(r, ch) / 16) % 16;
          if (used[grp]) return false;
          used[grp] = true;
        }
    }
  return true;
}
static_assert(dswz_conflict_free<32>() && dswz_conflict_free<64>() && dswz_conflict_free<128>(),
              "dswz must spread both read patterns");

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define SMS_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// One transposing LDS read (ds_read_b64_tr_b16, probed on MI355X): within each
// 16-lane group, lane 4a + e receives element e of the 8-byte rows addressed by
// lanes a, a + 4, a + 8 and a + 12. A group addressing 4 rows x 16 columns
// (lane j: row j / 4, columns 4 (j % 4) .. + 3) so hands each lane the 4 rows
// of its own column.
__device__ inline __attribute__((always_inline)) u32x2 lds_read_tr(const uint8_t* a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(SMS_LDS(s16x4, a)));
}

// Loads of a tile of TR rows into LDS in the dswz layout: instruction i of
// wavefront w fills the RPI rows (1 KB) from R = RPI (w + 4 i), lane n row
// R + n / (D / 8), chunk position n % (D / 8). In that order the swizzle of a
// lane's row depends on the lane and w only (dswz reads the row's low 4 bits,
// which 4 RPI i never reaches), so one offset register per source serves every
// instruction, the rows' offsets going in the scalar offset. Rows past the
// buffer range read as zero.
template <int D>
__device__ inline __attribute__((always_inline)) uint32_t dma_lane_off(int lane, int w, int64_t pitch) {
  constexpr int CH = D / 8, RPI = 64 / CH;
  const int r = lane / CH;
  return (uint32_t)(r * pitch + 16 * ((lane % CH) ^ dswz<D>(RPI * w + r)));
}
// The same loads issued from inline assembly, which the compiler does not
// see as LDS writes: it then inserts no wait for them before LDS reads of the
// other buffer (it cannot tell the buffers apart when one code path serves
// both), and the caller waits for them itself (vmcnt) before its barrier. The
// compiler keeps no value in m0 here (its only other users are the builtin
// LDS loads, not used alongside). src: the four descriptor words.
// dma_one issues load i of the wavefront's dma_loads<D, TR>() loads of a tile
// (rows RPI (w + 4 i) ..); dma_tile_asm issues all of them.
template <int D, int TR>
constexpr int dma_loads() {
  constexpr int CH = D / 8, RPI = 64 / CH, NI = TR / RPI / 4;
  static_assert(NI * RPI * 4 == TR, "whole 1 KB loads, four wavefronts");
  return NI;
}
template <int D>
__device__ inline __attribute__((always_inline)) void dma_one(u32x4 src, uint32_t voff, int64_t pitch, int w,
                                                              uint32_t dst, int i) {
  constexpr int CH = D / 8, RPI = 64 / CH;
  const int r0 = RPI * (w + 4 * i);
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(src), "s"((uint32_t)(r0 * pitch)), "s"(dst + (uint32_t)(r0 * D * 2))
               : "memory");
}
template <int D, int TR>
__device__ inline __attribute__((always_inline)) void dma_tile_asm(u32x4 src, uint32_t voff, int64_t pitch,
                                                                   int w, uint32_t dst) {
#pragma unroll
  for (int i = 0; i < dma_loads<D, TR>(); ++i) dma_one<D>(src, voff, pitch, w, dst, i);
}
// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima: no wait).
constexpr int kWaitLgkm0 = 0xF | (7 << 4) | (0 << 8) | (3 << 14);
// Descriptor words of rows_rsrc.
__device__ inline __attribute__((always_inline)) u32x4 rows_desc(const char* base, int rows, int64_t pitch,
                                                                 int row_bytes) {
  const uint32_t bytes = rows > 0 ? (uint32_t)((int64_t)(rows - 1) * pitch + row_bytes) : 0u;
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3A};
}
// LDS byte address of a __shared__ object.
__device__ inline __attribute__((always_inline)) uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
template <int D, int TR>
__device__ inline __attribute__((always_inline)) void dma_tile(__amdgpu_buffer_rsrc_t src, uint32_t voff,
                                                               int64_t pitch, int w, uint8_t* dst) {
  constexpr int CH = D / 8, RPI = 64 / CH, NI = TR / RPI / 4;
  static_assert(NI * RPI * 4 == TR, "whole 1 KB loads, four wavefronts");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r0 = RPI * (w + 4 * i);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, SMS_LDS(void, dst + r0 * D * 2), 16, (int)voff,
                                             (int)(r0 * pitch), 0, 0);
  }
}

// 16-bit element j (0..7) of an 8-element vector.
__device__ inline __attribute__((always_inline)) uint32_t elem(const u32x4& v, int j) {
  return (v[j >> 1] >> ((j & 1) * 16)) & 0xffffu;
}

// Mask values of one lane's 32 keys of a 64-key tile in the query-stationary
// layout (block kb, register r: key kt + 32 kb + 8 (r / 4) + 4 g + r % 4):
// run i = 4 kb + r / 4 holds keys kt + 32 kb + 8 (i % 4) + 4 g .. + 3, read
// as one 8-byte load (additive: four 16-bit values, .x keys 0-1, .y 2-3) or
// one 4-byte load (boolean: four bytes in .x). Needs every mask row to start
// on 4 elements and Sk % 4 == 0 (host-checked). The loads are unconditional:
// `mrow` is the row of a query clamped into the mask and a run past the row
// is read at the row's last run, so every address is inside the mask; the
// values of keys the caller excludes (past its bounds) are never used. Being
// straight-line, the loads are counted exactly by the wait that precedes
// their first use, and since they are issued at the start of a tile, before
// the next tile's prefetch, that wait leaves the prefetch in flight.
template <int KIND>
__device__ inline __attribute__((always_inline)) void load_mask_runs(
    const char* mask, int64_t mrow, int kt, int g, int Sk, u32x2 (&mv)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k0 = min(kt + (i >> 2) * 32 + 8 * (i & 3) + 4 * g, Sk - 4);
    if constexpr (KIND == 1) {
      mv[i] = *reinterpret_cast<const u32x2*>(mask + (mrow + k0) * 2);
    } else {
      mv[i].x = *reinterpret_cast<const uint32_t*>(mask + mrow + k0);
      mv[i].y = 0;
    }
  }
}

// Value of register r (0..15) of block kb from load_mask_runs: the 16-bit
// additive value, or the boolean byte.
__device__ inline __attribute__((always_inline)) uint32_t mask_run_value(const u32x2 (&mv)[8],
                                                                         int kb, int r, bool is_bool) {
  const u32x2 run = mv[4 * kb + (r >> 2)];
  const int e = r & 3;
  if (is_bool) return (run.x >> (8 * e)) & 0xffu;
  return (run[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

}  // namespace attn

}  // namespace sms

// Launch of the forward for dtype 1 (fp16) or 2 (bf16) and head dim 64 or 128;
// hipErrorInvalidValue for anything else. Grid: H * B * ceil(Sq / 128).
hipError_t sms_attn_launch(const sms::AttnParams* p, int dtype, int head_dim, hipStream_t st);

// The backward's launches (dQ, which also forms rowsum(dO * O) in the
// workspace; dK and dV in one launch, or two for D = 128 with a per-score mask
// on larger grids), same dtype / head-dim rules.
hipError_t sms_attn_bwd_launch(const sms::AttnBwdParams* p, int dtype, int head_dim,
                               hipStream_t st);
