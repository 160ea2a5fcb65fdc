// kernels.hpp -- HIP kernels of the fused scaled-masked softmax for gfx950.
//
// Forward, per row (b, h, q) of x[B,H,Sq,Sk]: s_k = x_k*scale + mask_k, keys
// after the causal bound masked, y_k = exp(s_k - max s) / sum exp(s - max s)
// (lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into PyTorch",
// sec. 1.2 and 2.1; causal after the additive mask as in sec. 3.1). A fully
// masked row is written as zeros (pnsm.cn ScaledMaskSoftmax article, sec. 4.3).
// Backward: dx_k = scale * y_k * (dy_k - sum_j dy_j y_j) (lmnt.cn page, sec. 3.3).
//
// Masks: additive (x's dtype), boolean (one byte per key, nonzero = excluded,
// turned into -inf inside the kernel as the pnsm.cn article, sec. 2.3,
// suggests), or per-batch key lengths (keys k >= len[b] excluded; nothing per
// key is read). Causal: key k is excluded when k > q (top-left alignment) or
// k > q + Sk - Sq (bottom-right alignment, for Sq != Sk). Key lengths and both
// causal rules are one bound per row, kload: keys [0, kload) are read, the
// rest are neither loaded nor exponentiated and are written as zeros.
//
// Mapping. A row is owned by TPR consecutive lanes. TPR <= 64 packs 64/TPR rows
// into each wavefront (four wavefronts per 256-thread workgroup); TPR >= 128
// gives one row to a workgroup of TPR/64 wavefronts. Each lane holds NV 16-byte
// vectors of the row in VGPRs: vector v = j*TPR + lane (j < NV), so one wave
// instruction moves TPR*16 contiguous bytes. The row is read from HBM once,
// reduced in registers and written once; exponentials are computed once per
// element and kept in the same registers. Rows too long for that stream (two
// passes, one workgroup per row; see the streaming kernels).
//
// Reductions. Within a wavefront: DPP quad_perm / row_half_mirror / row_mirror
// steps reduce 4, 8 and 16 lanes, then the gfx950 lane-swap instructions
// v_permlane16_swap and v_permlane32_swap combine rows of 16 and halves of 32.
// No LDS traffic and no barrier. Across the wavefronts of a workgroup: one LDS
// slot per wavefront and one barrier per reduction (max and sum use distinct
// slots, so the forward takes exactly two barriers).
//
// Alignment. Vector v covers the row's elements [v*E - a, v*E - a + E), where a
// is the input row start's element offset inside its 16-byte line, so full
// vectors are 16-byte aligned in the input. The general kernels read and write
// the partial first and last vectors of a row one element at a time, and use
// element accesses for any operand whose rows sit at another offset. The
// aligned-row kernels serve the common case where every operand's rows start
// on 16-byte lines and hold whole vectors.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

#define SMS_DEV __device__ __forceinline__

namespace sms {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Exponentials are taken as 2^64 * exp(s - m) = v_exp_f32((s - m)*log2(e) + 64):
// the bias rides in the same FMA, and it keeps every exponential that can
// matter in the normal fp32 range (the hardware exp2 does not return
// subnormals, while bf16 and fp32 outputs reach down to 2^-133 and 2^-149).
// The row sum carries the same 2^64 (at most 2^64 * Sk, far from overflow),
// so y = e' / sum' equals e / sum with the power of two cancelled exactly.
constexpr float kExpBias = 64.0f;
SMS_DEV float exp_biased(float s, float m) {
  return __builtin_amdgcn_exp2f(fmaf(s - m, kLog2e, kExpBias));
}

// ----------------------------------------------------------------- formats

struct Fp32 {
  static constexpr int kBytes = 4;
  static constexpr int kE = 4;  // elements per 16-byte vector
  SMS_DEV static void unpack(const u32x4& u, float (&f)[kE]) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  SMS_DEV static u32x4 pack(const float (&f)[kE]) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
  SMS_DEV static float ld(const char* p) { return *reinterpret_cast<const float*>(p); }
  SMS_DEV static void st(char* p, float v) { *reinterpret_cast<float*>(p) = v; }
  // fp32 products are not exact in fp32: widen before multiplying.
  SMS_DEV static double prod(float a, float b) { return (double)a * (double)b; }
};

struct Fp16 {
  static constexpr int kBytes = 2;
  static constexpr int kE = 8;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  SMS_DEV static void unpack(const u32x4& u, float (&f)[kE]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h2 h = __builtin_bit_cast(h2, w[i]);
      f[2 * i] = (float)h.x;
      f[2 * i + 1] = (float)h.y;
    }
  }
  SMS_DEV static u32x4 pack(const float (&f)[kE]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h2 h;
      h.x = (_Float16)f[2 * i];  // round to nearest even, subnormals kept
      h.y = (_Float16)f[2 * i + 1];
      w[i] = __builtin_bit_cast(uint32_t, h);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }
  SMS_DEV static float ld(const char* p) { return (float)*reinterpret_cast<const _Float16*>(p); }
  SMS_DEV static void st(char* p, float v) { *reinterpret_cast<_Float16*>(p) = (_Float16)v; }
  // Product of two fp16 values (11-bit significands) is exact in fp32.
  SMS_DEV static double prod(float a, float b) { return (double)(a * b); }
};

struct Bf16 {
  static constexpr int kBytes = 2;
  static constexpr int kE = 8;
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  SMS_DEV static void unpack(const u32x4& u, float (&f)[kE]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  SMS_DEV static u32x4 pack(const float (&f)[kE]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b2 b;
      b.x = (__bf16)f[2 * i];  // v_cvt_pk_bf16_f32: round to nearest even
      b.y = (__bf16)f[2 * i + 1];
      w[i] = __builtin_bit_cast(uint32_t, b);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
  }
  SMS_DEV static float ld(const char* p) {
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
  SMS_DEV static void st(char* p, float v) { *reinterpret_cast<__bf16*>(p) = (__bf16)v; }
  SMS_DEV static double prod(float a, float b) { return (double)(a * b); }  // exact
};

// ------------------------------------------------------ wavefront reductions

template <int CTRL>
SMS_DEV float dpp(float v) {
  const int i = __float_as_int(v);
  return __int_as_float(__builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false));
}

template <int CTRL>
SMS_DEV double dpp(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  const uint32_t lo2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint32_t hi2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi2 << 32) | lo2);
}

// The pair of values a lane sees after exchanging rows of 16 lanes (SWAP32 =
// false) or halves of 32 lanes (true) with itself: its own and its partner's.
template <bool SWAP32>
SMS_DEV void swap_pair(float v, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (SWAP32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

template <bool SWAP32>
SMS_DEV void swap_pair(double v, double& a, double& b) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t lo_a, lo_b, hi_a, hi_b;
  if constexpr (SWAP32) {
    const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    lo_a = rl[0]; lo_b = rl[1]; hi_a = rh[0]; hi_b = rh[1];
  } else {
    const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    lo_a = rl[0]; lo_b = rl[1]; hi_a = rh[0]; hi_b = rh[1];
  }
  a = __builtin_bit_cast(double, ((uint64_t)hi_a << 32) | lo_a);
  b = __builtin_bit_cast(double, ((uint64_t)hi_b << 32) | lo_b);
}

struct OpMax {
  SMS_DEV float operator()(float a, float b) const { return fmaxf(a, b); }
  SMS_DEV double operator()(double a, double b) const { return fmax(a, b); }
};
struct OpAdd {
  template <class T>
  SMS_DEV T operator()(T a, T b) const { return a + b; }
};

// All-reduce over aligned groups of G lanes (G a power of two, <= 64); every
// lane of a group ends with the group's result. Fixed order: deterministic.
template <int G, class T, class Op>
SMS_DEV T group_reduce(T v, Op op) {
  if constexpr (G > 1) v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (G > 2) v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (G > 4) v = op(v, dpp<0x141>(v));  // row_half_mirror: other quad of 8
  if constexpr (G > 8) v = op(v, dpp<0x140>(v));  // row_mirror: other half of 16
  if constexpr (G > 16) {
    T a, b;
    swap_pair<false>(v, a, b);  // rows 0<->1 and 2<->3
    v = op(a, b);
  }
  if constexpr (G > 32) {
    T a, b;
    swap_pair<true>(v, a, b);   // lanes 0-31 <-> 32-63
    v = op(a, b);
  }
  return v;
}

// Reduction over the TPR lanes that own a row. For TPR > 64 the wavefronts of
// the workgroup meet in LDS (`slots` holds TPR/64 values) behind one barrier.
// With nw < TPR/64 only the first nw wavefronts take part (the others have
// ended: a barrier waits only for wavefronts that have not terminated).
template <int TPR, class T, class Op>
SMS_DEV T row_reduce(T v, Op op, T* slots, int nw = TPR / 64) {
  if constexpr (TPR <= 64) {
    return group_reduce<TPR>(v, op);
  } else {
    constexpr int W = TPR / 64;
    v = group_reduce<64>(v, op);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) slots[wave] = v;
    __syncthreads();
    T r = slots[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
      if (i < nw) r = op(r, slots[i]);
    return r;
  }
}

// -------------------------------------------------------------- row mapping

// Rows are numbered r = (b*H + h)*Sq + q (q fastest) and run in that order:
// consecutive workgroups take consecutive rows, which keeps the x / y streams
// contiguous in memory. (b, h, q) come from two divisions by launch-time
// constants (fastdiv.hpp); a row starts at b*s_b + h*s_h + q*s_q. With 64 or
// more lanes per row all of it is scalar work, once per wave, free of branches
// so that the kernel-argument loads it needs are issued together.
struct RowGeom {
  uint32_t B, H, Sq, Sk;
  uint32_t rows;     // B*H*Sq
  FastDiv div_sq;    // by Sq
  FastDiv div_h;     // by H
};

SMS_DEV void row_bhq(const RowGeom& g, uint32_t r, uint32_t& b, uint32_t& h, uint32_t& q) {
  const uint32_t t = fast_div(r, g.div_sq);
  q = r - t * g.Sq;
  b = fast_div(t, g.div_h);
  h = t - b * g.H;
}

// Element offset of row (b, h, q) of an operand with strides (sb, sh, sq).
SMS_DEV int64_t row_offset(uint32_t b, uint32_t h, uint32_t q, int64_t sb, int64_t sh,
                           int64_t sq) {
  return (int64_t)b * sb + (int64_t)h * sh + (int64_t)q * sq;
}

constexpr int block_of(int tpr) { return tpr <= 64 ? 256 : tpr; }

// Index of this thread's row inside its workgroup. With 64 or more lanes per
// row it is the same for the whole wavefront, and readfirstlane says so: the
// row's coordinates, offsets and key bound are then computed once per wave in
// scalar registers instead of per lane (integer division and 64-bit products
// on the vector unit measured ~9 % of a bandwidth-bound backward).
template <int TPR>
SMS_DEV uint32_t local_row() {
  if constexpr (TPR >= 64) return __builtin_amdgcn_readfirstlane(threadIdx.x / TPR);
  else return threadIdx.x / TPR;
}

// Work item of this workgroup in the aligned-row kernels. Workgroups are dealt
// to the 8 XCDs round-robin (workgroup i runs on XCD i % 8, each XCD with its
// own L2), so consecutive rows land on different XCDs. Where rows share
// 128-byte lines with their neighbours (a launch that is not line-exact), a
// line two rows share then reaches HBM as two partial writes from two L2s.
// For those launches workgroup i takes work item (i % 8) * (N / 8) + i / 8
// (the tail past 8 * (N / 8) as is): each XCD walks a contiguous range of
// rows and both halves of a shared line meet in its L2. Measured on MI355X,
// bf16 [16,16,1000,1000] with a [1000,1000] mask: forward 175.2 -> 172.2 us,
// backward 234.3 -> 226.0 us. Line-exact launches measured 1-7 % slower with
// it (eight streams through memory instead of one) and keep the dealt order.
SMS_DEV uint32_t work_item(int lines) {
  const uint32_t i = blockIdx.x;
  if (lines) return i;
  const uint32_t per = gridDim.x >> 3;
  return i < (per << 3) ? (i & 7u) * per + (i >> 3) : i;
}

// ------------------------------------------------------------- parameters

enum : int { MASK_NONE = 0, MASK_ADD = 1, MASK_BOOL = 2, MASK_LEN = 3 };
enum : int { CAUSAL_NONE = 0, CAUSAL_TOP_LEFT = 1, CAUSAL_BOTTOM_RIGHT = 2 };
// Cache hints, fixed at build time. The score and output streams (x, y, dy,
// dx) are touched once: their 16-byte vectors are loaded and stored with the
// nontemporal hint. The mask, which other rows read again, goes through the
// caches. Building with SMS_NT_LOADS=0 / SMS_NT_STORES=0 drops the hints.
#ifndef SMS_NT_LOADS
#define SMS_NT_LOADS 1
#endif
#ifndef SMS_NT_STORES
#define SMS_NT_STORES 1
#endif
constexpr bool kNtLoads = SMS_NT_LOADS != 0;
constexpr bool kNtStores = SMS_NT_STORES != 0;

struct FwdParams {
  const char* x;
  const char* mask;          // additive (x's dtype), bool (bytes) or int32 lengths [B]
  char* y;
  int64_t sx_b, sx_h, sx_q;  // element strides of x
  int64_t sy_b, sy_h, sy_q;  // element strides of y
  int64_t sm_b, sm_h, sm_q;  // element strides of the mask, 0 on broadcast axes
  RowGeom g;
  float scale;
  int causal;     // CAUSAL_*
  int mask_kind;  // MASK_*
  int lines;      // every row of x and y starts on a 128-byte line and fills whole lines
  // Split rows (FAMILY_SPLIT): chunks per row, vectors per chunk, and the
  // workspace of rows * chunks (max, sum) pairs.
  uint32_t chunks, chunk_vec;
  float2* ws;
  // Head groups (FAMILY_HEADS): heads per workgroup, and division by H / heads.
  uint32_t heads;
  FastDiv div_hg;
  int early;  // aligned kernels: wavefronts holding only keys past the bound exit early
};

struct BwdParams {
  const char* y;
  const char* dy;
  char* dx;
  int64_t sy_b, sy_h, sy_q;
  int64_t sd_b, sd_h, sd_q;  // dy
  int64_t sx_b, sx_h, sx_q;  // dx
  RowGeom g;
  float scale;
  int causal;  // CAUSAL_*: a promise that y is 0 past the bound
  int lines;   // every row of y, dy and dx starts on a 128-byte line and fills whole lines
  int early;   // aligned kernels: wavefronts holding only keys past the bound exit early
  // Split rows (FAMILY_SPLIT): chunks per row, vectors per chunk, and the
  // workspace of rows * chunks partial dot products.
  uint32_t chunks, chunk_vec;
  double* ws;
};

// Keys [0, bound) of row q survive the causal rule.
SMS_DEV int causal_bound(int causal, uint32_t q, uint32_t Sq, int Sk) {
  int64_t c = Sk;
  if (causal == CAUSAL_TOP_LEFT) c = (int64_t)q + 1;
  if (causal == CAUSAL_BOTTOM_RIGHT) c = (int64_t)q + 1 + (int64_t)Sk - (int64_t)Sq;
  return (int)(c < 0 ? 0 : (c > Sk ? Sk : c));
}

// 16-byte vector of a streamed operand (x, y, dy) / of the mask, and a
// 16-byte store to an output row (y, dx).
template <bool NT = kNtLoads>
SMS_DEV u32x4 ld_stream(const char* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}
SMS_DEV u32x4 ld_cached(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Rows whose base is the same for the whole wavefront (64 or more lanes per
// row) are read and written through buffer resources, which carry a cache
// policy word per access (sc0 = 1, nt = 2, sc1 = 16). Two layouts:
//  * line-exact rows (each starts on a 128-byte line and fills whole lines;
//    decided on the host for the whole launch): plain nontemporal global
//    loads; stores nontemporal with the device-scope bit, which measured
//    ~1 % faster than the hint alone on MI355X (5 % for a pure write stream);
//  * other rows: a 16-byte vector in a line that the row shares with a
//    neighbouring row takes the default policy, so the line waits in L2 for
//    the neighbour's part (a partial line stored to HBM on its own costs a
//    read-modify-write there, and a partial line evicted after one read is
//    fetched again); the other vectors load and store nontemporal. Measured
//    on bf16 rows of 1000 keys: backward 12 % and forward 4.5 % faster than
//    nontemporal everywhere. The device-scope bit made these rows slower.
// SMS_BUF_ROWS=0 keeps plain global accesses (for measurement).
#ifndef SMS_BUF_ROWS
#define SMS_BUF_ROWS 1
#endif
constexpr bool kBufRows = SMS_BUF_ROWS != 0;
constexpr int kAuxDefault = 0;
constexpr int kAuxNt = 2;
constexpr int kAuxNtDevice = 18;  // nt | sc1
// Fourth descriptor word of a raw (stride 0) buffer of 32-bit data on gfx9.
constexpr int kRsrcWord3 = 0x00020000;

struct RowStream {
  __amdgpu_buffer_rsrc_t r;
  uint32_t lo, hi;  // byte offsets [lo, hi) lie in 128-byte lines the row owns whole
};

// The row of `bytes` bytes at `base` (wave-uniform).
SMS_DEV RowStream row_stream(const char* base, uint32_t bytes) {
  RowStream s;
  s.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, (int)bytes, kRsrcWord3);
  const uint32_t a = (uint32_t)(uintptr_t)base & 127u;
  const uint32_t e = (uint32_t)((uintptr_t)base + bytes) & 127u;
  s.lo = a ? 128u - a : 0u;
  s.hi = e ? bytes - e : bytes;  // wraps when the row sits inside one line: then lo > bytes
  return s;
}
template <int AUX>
SMS_DEV u32x4 buf_load(const RowStream& s, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(s.r, (int)off, 0, AUX);
}
template <int AUX>
SMS_DEV void buf_store(const RowStream& s, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, s.r, (int)off, 0, AUX);
}
// Loads / stores of rows that are not line-exact (see above).
SMS_DEV u32x4 rs_load(const RowStream& s, uint32_t off) {
  if (off >= s.lo && off < s.hi) return buf_load<kAuxNt>(s, off);
  return buf_load<kAuxDefault>(s, off);
}
SMS_DEV void rs_store(const RowStream& s, uint32_t off, u32x4 v) {
  if (off >= s.lo && off < s.hi) buf_store<kAuxNt>(s, off, v);
  else buf_store<kAuxDefault>(s, off, v);
}


SMS_DEV void st_stream(char* p, u32x4 v) {
  u32x4* q = reinterpret_cast<u32x4*>(p);
  if constexpr (kNtStores) __builtin_nontemporal_store(v, q);
  else *q = v;
}

// 16-byte store of vector v of an aligned output row: through the row's
// buffer resource (BUF; line-exact launch or not) or a nontemporal global store.
template <bool BUF>
SMS_DEV void out_store(const RowStream& rs, char* row, bool exact, int v, u32x4 val) {
  if constexpr (BUF) {
    if (exact) buf_store<kAuxNtDevice>(rs, (uint32_t)v * 16, val);
    else rs_store(rs, (uint32_t)v * 16, val);
  } else {
    st_stream(row + (int64_t)v * 16, val);
  }
}

// E mask bytes starting at p (aligned to E), zero-extended.
template <int E>
SMS_DEV uint64_t ld_bits(const char* p) {
  if constexpr (E == 8) return *reinterpret_cast<const uint64_t*>(p);
  else return *reinterpret_cast<const uint32_t*>(p);
}
SMS_DEV bool bit_set(uint64_t bits, int e) { return ((bits >> (8 * e)) & 0xffu) != 0; }

// ----------------------------------------------------------- row descriptors

struct FwdRow {
  const char* x;
  const char* m;  // the row's mask row (additive / bool), unused otherwise
  char* y;
  int ax;         // elements from x's row start back to its 16-byte line
  int kload;      // keys [0, kload) are read
  bool yvec;      // y's row sits at x's offset: whole-vector stores
  bool mvec;      // the mask row sits at x's offset: whole-vector mask loads
  bool valid;
};

template <class F, int RPB>
SMS_DEV FwdRow fwd_row(const FwdParams& p, uint32_t w, uint32_t local) {
  constexpr int BY = F::kBytes;
  constexpr int E = F::kE;
  FwdRow r;
  const uint32_t row = w * RPB + local;
  r.valid = RPB == 1 || row < p.g.rows;  // RPB == 1: the grid is exactly the rows
  uint32_t b, h, q;
  row_bhq(p.g, row, b, h, q);
  const int Sk = (int)p.g.Sk;
  r.x = p.x + row_offset(b, h, q, p.sx_b, p.sx_h, p.sx_q) * BY;
  r.y = p.y + row_offset(b, h, q, p.sy_b, p.sy_h, p.sy_q) * BY;
  r.ax = (int)(((uintptr_t)r.x & 15) / BY);
  r.yvec = ((((uintptr_t)r.y & 15) / BY) == (uintptr_t)r.ax);
  int kload = causal_bound(p.causal, q, p.g.Sq, Sk);
  const int64_t moff = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)q * p.sm_q;
  r.m = nullptr;
  r.mvec = false;
  if (p.mask_kind == MASK_ADD) {
    r.m = p.mask + moff * BY;
    r.mvec = ((((uintptr_t)r.m & 15) / BY) == (uintptr_t)r.ax);
  } else if (p.mask_kind == MASK_BOOL) {
    r.m = p.mask + moff;
    r.mvec = ((((uintptr_t)r.m - (uintptr_t)r.ax) & (E - 1)) == 0);
  } else if (p.mask_kind == MASK_LEN && r.valid) {
    const int len = reinterpret_cast<const int32_t*>(p.mask)[b];
    kload = min(kload, max(len, 0));
  }
  r.kload = r.valid ? kload : 0;
  return r;
}

struct BwdRow {
  const char* y;
  const char* d;
  char* x;
  int ay;      // elements from y's row start back to its 16-byte line
  int kload;   // keys [0, kload) are read
  bool dvec;   // dy's row at y's offset
  bool xvec;   // dx's row at y's offset
  bool valid;
};

template <class F, int RPB>
SMS_DEV BwdRow bwd_row(const BwdParams& p, uint32_t w, uint32_t local) {
  constexpr int BY = F::kBytes;
  BwdRow r;
  const uint32_t row = w * RPB + local;
  r.valid = RPB == 1 || row < p.g.rows;
  uint32_t b, h, q;
  row_bhq(p.g, row, b, h, q);
  r.y = p.y + row_offset(b, h, q, p.sy_b, p.sy_h, p.sy_q) * BY;
  r.d = p.dy + row_offset(b, h, q, p.sd_b, p.sd_h, p.sd_q) * BY;
  r.x = p.dx + row_offset(b, h, q, p.sx_b, p.sx_h, p.sx_q) * BY;
  r.ay = (int)(((uintptr_t)r.y & 15) / BY);
  r.dvec = ((((uintptr_t)r.d & 15) / BY) == (uintptr_t)r.ay);
  r.xvec = ((((uintptr_t)r.x & 15) / BY) == (uintptr_t)r.ay);
  r.kload = r.valid ? causal_bound(p.causal, q, p.g.Sq, (int)p.g.Sk) : 0;
  return r;
}

// ------------------------------------------------ element and vector access

// Scores of vector v of a row: x*scale + mask for keys [0, kload), -inf for
// every other key. Any alignment. NT: nontemporal vector loads of x (off for a
// first pass over a row that is read again).
template <class F, bool NT = kNtLoads>
SMS_DEV void row_scores(const FwdRow& r, int kind, int v, float scale, float (&s)[F::kE]) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  const int k0 = v * E - r.ax;
  if (k0 < r.kload && k0 + E > 0) {
    // Every vector holding a key of [0, kload) loads its 16-byte line (x + k0*BY
    // sits on one: k0 + ax is a multiple of E) before the whole / partial
    // branch, so that the wavefront issues one load for both kinds of lane
    // instead of one per branch, each waited for in turn. A partial vector's
    // line (the row's head or tail, or the key bound inside it) holds at least
    // one key of the row, so it lies in a page the row occupies; its keys
    // outside [0, kload), which belong to other rows or to no row, are set to
    // -inf whatever was read there. A mask row at another offset inside its
    // line is read element by element. Measured on MI355X, bf16
    // [16,16,1000,1001] with a [1000,1001] additive mask (128 lanes per row):
    // forward 294 -> 229 us and backward 304 -> 252 us against a load in
    // each branch (element loads of x had been 2-3 x slower still).
    float xv[E], m[E];
    uint64_t bits = 0;
    F::unpack(ld_stream<NT>(r.x + (int64_t)k0 * BY), xv);
    if (kind == MASK_ADD && r.mvec) F::unpack(ld_cached(r.m + (int64_t)k0 * BY), m);
    if (kind == MASK_BOOL && r.mvec) bits = ld_bits<E>(r.m + k0);
    if (k0 >= 0 && k0 + E <= r.kload) {
      if (kind == MASK_ADD) {
        if (!r.mvec) {
#pragma unroll
          for (int e = 0; e < E; ++e) m[e] = F::ld(r.m + (int64_t)(k0 + e) * BY);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = fmaf(xv[e], scale, m[e]);
      } else if (kind == MASK_BOOL) {
        if (!r.mvec) {
#pragma unroll
          for (int e = 0; e < E; ++e) bits |= (uint64_t)(uint8_t)r.m[k0 + e] << (8 * e);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = bit_set(bits, e) ? kNegInf : xv[e] * scale;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = xv[e] * scale;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = k0 + e;
        float v2 = kNegInf;
        if (k >= 0 && k < r.kload) {
          if (kind == MASK_ADD) v2 = fmaf(xv[e], scale, r.mvec ? m[e] : F::ld(r.m + (int64_t)k * BY));
          else if (kind == MASK_BOOL) v2 = (r.mvec ? bit_set(bits, e) : r.m[k] != 0) ? kNegInf : xv[e] * scale;
          else v2 = xv[e] * scale;
        }
        s[e] = v2;
      }
    }
  } else {
    // None of the vector's keys is read.
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = kNegInf;
  }
}

// y and dy of vector v for keys [0, kload), zeros elsewhere. Any alignment.
template <class F, bool NT = kNtLoads>
SMS_DEV void row_pair(const BwdRow& r, int v, float (&yv)[F::kE], float (&gv)[F::kE]) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  const int k0 = v * E - r.ay;
  if (k0 < r.kload && k0 + E > 0) {
    // One load of each 16-byte line for whole and partial vectors alike, as in
    // row_scores; a partial vector's keys outside [0, kload) read as zeros
    // whatever the line held there, and a dy row at another offset inside its
    // line is read element by element.
    float ya[E], ga[E];
    F::unpack(ld_stream<NT>(r.y + (int64_t)k0 * BY), ya);
    if (r.dvec) F::unpack(ld_stream<NT>(r.d + (int64_t)k0 * BY), ga);
    if (k0 >= 0 && k0 + E <= r.kload) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        yv[e] = ya[e];
        gv[e] = r.dvec ? ga[e] : F::ld(r.d + (int64_t)(k0 + e) * BY);
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = k0 + e;
        const bool in = (k >= 0 && k < r.kload);
        yv[e] = in ? ya[e] : 0.0f;
        gv[e] = in ? (r.dvec ? ga[e] : F::ld(r.d + (int64_t)k * BY)) : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      yv[e] = 0.0f;
      gv[e] = 0.0f;
    }
  }
}

// The same two reads with each vector's loads inside its whole / partial
// branch, for the streaming and split kernels: there the loads of a lane's
// several vectors per chunk are already in flight together, and the shared
// load measured no better on MI355X (us, branch loads -> shared load; one
// 1024-lane workgroup per row): fp16 rows of 65536 keys forward 426 -> 440,
// backward 725 -> 741; fp32 rows of 20000 keys 395 -> 392 and 652 -> 656;
// fp16 rows of 40001 keys at every offset 489 -> 483 and 698 -> 664.
template <class F, bool NT = kNtLoads>
SMS_DEV void row_scores_branch_loads(const FwdRow& r, int kind, int v, float scale, float (&s)[F::kE]) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  const int k0 = v * E - r.ax;
  if (k0 >= 0 && k0 + E <= r.kload) {
    // x + k0*BY sits on a 16-byte line: k0 + ax is a multiple of E.
    F::unpack(ld_stream<NT>(r.x + (int64_t)k0 * BY), s);
    if (kind == MASK_ADD) {
      float m[E];
      if (r.mvec) {
        F::unpack(ld_cached(r.m + (int64_t)k0 * BY), m);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) m[e] = F::ld(r.m + (int64_t)(k0 + e) * BY);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = fmaf(s[e], scale, m[e]);
    } else if (kind == MASK_BOOL) {
      uint64_t bits = 0;
      if (r.mvec) {
        bits = ld_bits<E>(r.m + k0);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
          bits |= (uint64_t)(uint8_t)r.m[k0 + e] << (8 * e);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = bit_set(bits, e) ? kNegInf : s[e] * scale;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] *= scale;
    }
  } else if (k0 < r.kload && k0 + E > 0) {
    // A partial vector (the row's head or tail, or the key bound inside it):
    // its 16-byte line is loaded whole -- the line holds at least one key of
    // the row, so it lies in a page the row occupies -- and the keys outside
    // [0, kload), which belong to other rows or to no row, are set to -inf
    // whatever was read there. A mask row at another offset inside its line
    // is read element by element. (Element loads of x measured 2-3 x slower
    // per row on bf16 rows of 1001 keys.)
    float xv[E], m[E];
    F::unpack(ld_stream<NT>(r.x + (int64_t)k0 * BY), xv);
    if (kind == MASK_ADD && r.mvec) F::unpack(ld_cached(r.m + (int64_t)k0 * BY), m);
    uint64_t bits = 0;
    if (kind == MASK_BOOL && r.mvec) bits = ld_bits<E>(r.m + k0);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int k = k0 + e;
      float v2 = kNegInf;
      if (k >= 0 && k < r.kload) {
        if (kind == MASK_ADD) v2 = fmaf(xv[e], scale, r.mvec ? m[e] : F::ld(r.m + (int64_t)k * BY));
        else if (kind == MASK_BOOL) v2 = (r.mvec ? bit_set(bits, e) : r.m[k] != 0) ? kNegInf : xv[e] * scale;
        else v2 = xv[e] * scale;
      }
      s[e] = v2;
    }
  } else {
    // None of the vector's keys is read.
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = kNegInf;
  }
}

template <class F, bool NT = kNtLoads>
SMS_DEV void row_pair_branch_loads(const BwdRow& r, int v, float (&yv)[F::kE], float (&gv)[F::kE]) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  const int k0 = v * E - r.ay;
  if (k0 >= 0 && k0 + E <= r.kload) {
    F::unpack(ld_stream<NT>(r.y + (int64_t)k0 * BY), yv);
    if (r.dvec) {
      F::unpack(ld_stream<NT>(r.d + (int64_t)k0 * BY), gv);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) gv[e] = F::ld(r.d + (int64_t)(k0 + e) * BY);
    }
  } else if (k0 < r.kload && k0 + E > 0) {
    // A partial vector: whole 16-byte lines, as in row_scores, and zeros
    // outside [0, kload) whatever was read there; a dy row at another offset
    // inside its line element by element.
    float ya[E], ga[E];
    F::unpack(ld_stream<NT>(r.y + (int64_t)k0 * BY), ya);
    if (r.dvec) F::unpack(ld_stream<NT>(r.d + (int64_t)k0 * BY), ga);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int k = k0 + e;
      const bool in = (k >= 0 && k < r.kload);
      yv[e] = in ? ya[e] : 0.0f;
      gv[e] = in ? (r.dvec ? ga[e] : F::ld(r.d + (int64_t)k * BY)) : 0.0f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      yv[e] = 0.0f;
      gv[e] = 0.0f;
    }
  }
}

// Stores vector v of an output row (keys [0, Sk)); a whole vector goes out as
// one 16-byte store when the output row sits at the input row's offset.
template <class F>
SMS_DEV void row_store(char* orow, bool ovec, int a, int v, int Sk, const float (&o)[F::kE]) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  const int k0 = v * E - a;
  if (k0 >= Sk || k0 + E <= 0) return;
  if (ovec && k0 >= 0 && k0 + E <= Sk) {
    st_stream(orow + (int64_t)k0 * BY, F::pack(o));
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int k = k0 + e;
    if (k >= 0 && k < Sk) F::st(orow + (int64_t)k * BY, o[e]);
  }
}

// Max, exponentials (in place) and normalisation of a row held as s[NV][E];
// k0 of vector j is (j*TPR + lane)*E - a. Returns the reciprocal sum through
// the values: s becomes y.
template <int TPR, int NV, int E>
SMS_DEV void softmax_in_registers(float (&s)[NV][E], int lane, int a, int kload, float* smax,
                                  float* ssum, int nw = TPR / 64) {
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) mx = fmaxf(mx, s[j][e]);
  mx = row_reduce<TPR>(mx, OpMax(), smax, nw);
  // Every key masked: exponentiate against 0 so every term is exp(-inf) = 0.
  const float mref = (mx == kNegInf) ? 0.0f : mx;
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k0 = (j * TPR + lane) * E - a;
    if (k0 < kload) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s[j][e] = exp_biased(s[j][e], mref);
        sum += s[j][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) s[j][e] = 0.0f;
    }
  }
  sum = row_reduce<TPR>(sum, OpAdd(), ssum, nw);
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;  // fully masked row -> zeros
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) s[j][e] *= inv;
}

// -------------------------------------------------- general kernels (any alignment)

template <class F, int TPR, int NV>
__global__ void __launch_bounds__(block_of(TPR)) sms_fwd_kernel(FwdParams p) {
  constexpr int E = F::kE;
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ float red[2][TPR > 64 ? TPR / 64 : 1];
  const int lane = (int)(threadIdx.x % TPR);
  const FwdRow r = fwd_row<F, RPB>(p, blockIdx.x, local_row<TPR>());
  if (!r.valid) return;  // only a tail group of a TPR <= 64 launch, which has no barrier
  float s[NV][E];
#pragma unroll
  for (int j = 0; j < NV; ++j) row_scores<F>(r, p.mask_kind, j * TPR + lane, p.scale, s[j]);
  softmax_in_registers<TPR, NV, E>(s, lane, r.ax, r.kload, red[0], red[1]);
#pragma unroll
  for (int j = 0; j < NV; ++j) row_store<F>(r.y, r.yvec, r.ax, j * TPR + lane, (int)p.g.Sk, s[j]);
}

template <class F, int TPR, int NV>
__global__ void __launch_bounds__(block_of(TPR)) sms_bwd_kernel(BwdParams p) {
  constexpr int E = F::kE;
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ double red[TPR > 64 ? TPR / 64 : 1];
  const int lane = (int)(threadIdx.x % TPR);
  const BwdRow r = bwd_row<F, RPB>(p, blockIdx.x, local_row<TPR>());
  if (!r.valid) return;
  float yv[NV][E], gv[NV][E];
#pragma unroll
  for (int j = 0; j < NV; ++j) row_pair<F>(r, j * TPR + lane, yv[j], gv[j]);
  // dot = sum_k dy_k * y_k, accumulated in fp64 (no cancellation loss when
  // dy_k - dot is small).
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) acc += F::prod(yv[j][e], gv[j][e]);
  acc = row_reduce<TPR>(acc, OpAdd(), red);
  const float dot_hi = (float)acc;
  const float dot_lo = (float)(acc - (double)dot_hi);
  const float scale = p.scale;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    float o[E];
    if (v * E - r.ay >= r.kload) {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = 0.0f;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = (yv[j][e] * scale) * ((gv[j][e] - dot_hi) - dot_lo);
    }
    row_store<F>(r.x, r.xvec, r.ay, v, (int)p.g.Sk, o);
  }
}

// ---------------------------------------------------- aligned-row kernels
//
// When every row of every operand starts on a 16-byte line and Sk is a
// multiple of E, every vector of a row is whole: no element accesses remain,
// and a bound inside a vector is a register select. One workgroup per slot
// (RPB rows), launched once: short-lived workgroups dealt in order keep the
// set of DRAM pages in use compact, which measured faster on MI355X than a
// persistent grid with next-row prefetch.

// Mask kinds the aligned forward is compiled for (a compile-time choice keeps
// the per-row setup and the per-vector work of unused kinds out of the code:
// short rows, such as 1000 bf16 keys, measured up to 9 % faster for it).
enum : int { FAST_PLAIN = 0 /* none, or key lengths */, FAST_ADD = 1, FAST_BOOL = 2 };

template <class F, int TPR, int NV, int KIND, bool EARLY>
__global__ void __launch_bounds__(block_of(TPR)) sms_fwd_fast_kernel(FwdParams p) {
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ float red[2][TPR > 64 ? TPR / 64 : 1];
  // Rows with a key bound (causal, key lengths): a new wavefront issues its
  // loads at the highest issue priority and drops to the lowest once they are
  // out, so that the loads of waves just started pass ahead of the arithmetic
  // and stores of older ones on the same SIMD. Measured on MI355X: fp16
  // [4,32,2048,2048] causal 252 -> 249 us, fp16 [4,32,4096,4096] with a
  // [4,4096,4096] mask, causal, 1098 -> 1093 us; the fp32 [8,32,1024,1024]
  // forward with a padding mask (no bound) and every backward measured slower
  // with it, so they keep the default.
  if constexpr (EARLY) __builtin_amdgcn_s_setprio(3);
  const int lane = (int)(threadIdx.x % TPR);
  const uint32_t row = work_item(p.lines) * RPB + local_row<TPR>();
  if (RPB > 1 && row >= p.g.rows) return;  // a tail group of a TPR <= 64 launch (no barrier)
  uint32_t b, h, q;
  row_bhq(p.g, row, b, h, q);
  // Host-checked: every row of x, y and the mask starts on a 16-byte line (an
  // E-byte line for a boolean mask) and holds whole vectors.
  const int Sk = (int)p.g.Sk;
  const char* xrow = p.x + row_offset(b, h, q, p.sx_b, p.sx_h, p.sx_q) * BY;
  char* yrow = p.y + row_offset(b, h, q, p.sy_b, p.sy_h, p.sy_q) * BY;
  int kload = p.causal ? causal_bound(p.causal, q, p.g.Sq, Sk) : Sk;
  const char* mrow = nullptr;
  if constexpr (KIND != FAST_PLAIN) {
    const int64_t moff = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)q * p.sm_q;
    mrow = p.mask + moff * (KIND == FAST_ADD ? BY : 1);
  } else {
    if (p.mask_kind == MASK_LEN)
      kload = min(kload, max(reinterpret_cast<const int32_t*>(p.mask)[b], 0));
  }
  constexpr bool kBuf = TPR >= 64 && kBufRows;
  RowStream xs, ys;
  const bool exact = p.lines != 0;
  if constexpr (kBuf) {
    xs = row_stream(xrow, (uint32_t)Sk * BY);
    ys = row_stream(yrow, (uint32_t)Sk * BY);
  }
  u32x4 xr[NV], mr[NV];
  uint64_t mb[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    if (v * E < kload) {
      if (kBuf && !exact) xr[j] = rs_load(xs, (uint32_t)v * 16);
      else xr[j] = ld_stream(xrow + (int64_t)v * 16);
      if constexpr (KIND == FAST_ADD) mr[j] = ld_cached(mrow + (int64_t)v * 16);
      if constexpr (KIND == FAST_BOOL) mb[j] = ld_bits<E>(mrow + (int64_t)v * E);
    }
  }
  if constexpr (EARLY) __builtin_amdgcn_s_setprio(0);
  // Wavefronts whose every vector lies past the key bound (the causal future,
  // padding) loaded nothing: they store zeros and end, and the others reduce
  // among themselves. (Tested after the loads are issued, so that the test
  // does not delay them.)
  // (A compile-time choice: the kernels without it are left exactly as they
  // were, since any change to their code measurably moved the compiler's
  // schedule of the non-causal fp32 forward.)
  int nw = TPR > 64 ? TPR / 64 : 1;
  if constexpr (EARLY && TPR > 64) {
    nw = min(TPR / 64, (kload + 64 * E - 1) / (64 * E));
    if ((int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= nw) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int v = j * TPR + lane;
        if (v * E < Sk) out_store<kBuf>(ys, yrow, exact, v, u32x4{0, 0, 0, 0});
      }
      return;
    }
  }
  const float scale = p.scale;
  float s[NV][E];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k0 = (j * TPR + lane) * E;
    if (k0 < kload) {
      F::unpack(xr[j], s[j]);
      if constexpr (KIND == FAST_ADD) {
        float m[E];
        F::unpack(mr[j], m);
#pragma unroll
        for (int e = 0; e < E; ++e) s[j][e] = fmaf(s[j][e], scale, m[e]);
      } else if constexpr (KIND == FAST_BOOL) {
#pragma unroll
        for (int e = 0; e < E; ++e) s[j][e] = bit_set(mb[j], e) ? kNegInf : s[j][e] * scale;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[j][e] *= scale;
      }
      if (k0 + E > kload) {  // the vector that holds the row's key bound
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (k0 + e >= kload) s[j][e] = kNegInf;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) s[j][e] = kNegInf;
    }
  }
  softmax_in_registers<TPR, NV, E>(s, lane, 0, kload, red[0], red[1], nw);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    if (v * E < Sk) out_store<kBuf>(ys, yrow, exact, v, F::pack(s[j]));
  }
}

// Reduction of G values per lane over the TPR (>= 128) lanes of a
// workgroup that owns G rows: one LDS slot per row and wavefront, one barrier
// for all G rows.
template <int TPR, int G, class Op>
SMS_DEV void rows_reduce(float (&v)[G], Op op, float (*slots)[TPR / 64]) {
  constexpr int W = TPR / 64;
#pragma unroll
  for (int i = 0; i < G; ++i) v[i] = group_reduce<64>(v[i], op);
  if constexpr (W > 1) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) slots[i][wave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float r = slots[i][0];
#pragma unroll
      for (int k = 1; k < W; ++k) r = op(r, slots[i][k]);
      v[i] = r;
    }
  }
}

// Aligned forward over head groups: one workgroup takes query q of heads
// h0 .. h0 + G - 1 of batch b, for masks that do not depend on the head
// (mask shapes [Sq,Sk], [B,Sq,Sk], [B,1,Sk], key lengths, or none). The mask
// row is read once for the G rows, and the G rows' maxima and sums meet in
// LDS behind the same two barriers. Workgroups run q fastest, then head
// group, then batch, so each of the G x and y streams stays contiguous.
template <class F, int TPR, int NV, int KIND, int G>
__global__ void __launch_bounds__(TPR) sms_fwd_heads_kernel(FwdParams p) {
  static_assert(TPR >= 64, "one row per workgroup");
  constexpr int E = F::kE;
  constexpr int BY = F::kBytes;
  __shared__ float red[2][G][TPR / 64];
  const int lane = (int)threadIdx.x;
  // Host-checked: H % G == 0 and grid = B * (H / G) * Sq.
  const uint32_t w = work_item(p.lines);
  const uint32_t t = fast_div(w, p.g.div_sq);
  const uint32_t q = w - t * p.g.Sq;
  const uint32_t b = fast_div(t, p.div_hg);
  const uint32_t h0 = (t - b * (p.g.H / G)) * G;
  const int Sk = (int)p.g.Sk;
  int kload = p.causal ? causal_bound(p.causal, q, p.g.Sq, Sk) : Sk;
  const char* mrow = nullptr;
  if constexpr (KIND != FAST_PLAIN) {
    const int64_t moff = (int64_t)b * p.sm_b + (int64_t)q * p.sm_q;  // sm_h == 0
    mrow = p.mask + moff * (KIND == FAST_ADD ? BY : 1);
  } else {
    if (p.mask_kind == MASK_LEN)
      kload = min(kload, max(reinterpret_cast<const int32_t*>(p.mask)[b], 0));
  }
  const char* xrow[G];
  char* yrow[G];
  RowStream xs[G], ys[G];
  const bool exact = p.lines != 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    xrow[i] = p.x + row_offset(b, h0 + i, q, p.sx_b, p.sx_h, p.sx_q) * BY;
    yrow[i] = p.y + row_offset(b, h0 + i, q, p.sy_b, p.sy_h, p.sy_q) * BY;
    if constexpr (kBufRows) {
      xs[i] = row_stream(xrow[i], (uint32_t)Sk * BY);
      ys[i] = row_stream(yrow[i], (uint32_t)Sk * BY);
    }
  }
  u32x4 xr[G][NV], mr[NV];
  uint64_t mb[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    if (v * E < kload) {
      if constexpr (KIND == FAST_ADD) mr[j] = ld_cached(mrow + (int64_t)v * 16);
      if constexpr (KIND == FAST_BOOL) mb[j] = ld_bits<E>(mrow + (int64_t)v * E);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (kBufRows && !exact) xr[i][j] = rs_load(xs[i], (uint32_t)v * 16);
        else xr[i][j] = ld_stream(xrow[i] + (int64_t)v * 16);
      }
    }
  }
  const float scale = p.scale;
  float s[G][NV][E];
  float mx[G];
#pragma unroll
  for (int i = 0; i < G; ++i) mx[i] = kNegInf;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k0 = (j * TPR + lane) * E;
    float m[E];
    if constexpr (KIND == FAST_ADD) {
      if (k0 < kload) F::unpack(mr[j], m);
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (k0 < kload) {
        F::unpack(xr[i][j], s[i][j]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if constexpr (KIND == FAST_ADD) s[i][j][e] = fmaf(s[i][j][e], scale, m[e]);
          else if constexpr (KIND == FAST_BOOL)
            s[i][j][e] = bit_set(mb[j], e) ? kNegInf : s[i][j][e] * scale;
          else s[i][j][e] *= scale;
        }
        if (k0 + E > kload) {  // the vector that holds the row's key bound
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (k0 + e >= kload) s[i][j][e] = kNegInf;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[i][j][e] = kNegInf;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) mx[i] = fmaxf(mx[i], s[i][j][e]);
    }
  }
  rows_reduce<TPR, G>(mx, OpMax(), red[0]);
  float sum[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    // Every key masked: exponentiate against 0 so every term is exp(-inf) = 0.
    const float mref = (mx[i] == kNegInf) ? 0.0f : mx[i];
    sum[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if ((j * TPR + lane) * E < kload) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s[i][j][e] = exp_biased(s[i][j][e], mref);
          sum[i] += s[i][j][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[i][j][e] = 0.0f;
      }
    }
  }
  rows_reduce<TPR, G>(sum, OpAdd(), red[1]);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float inv = sum[i] > 0.0f ? 1.0f / sum[i] : 0.0f;  // fully masked row -> zeros
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = j * TPR + lane;
      if (v * E < Sk) {
#pragma unroll
        for (int e = 0; e < E; ++e) s[i][j][e] *= inv;
        out_store<kBufRows>(ys[i], yrow[i], exact, v, F::pack(s[i][j]));
      }
    }
  }
}

template <class F, int TPR, int NV, bool EARLY>
__global__ void __launch_bounds__(block_of(TPR)) sms_bwd_fast_kernel(BwdParams p) {
  constexpr int E = F::kE;
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ double red[TPR > 64 ? TPR / 64 : 1];
  const int lane = (int)(threadIdx.x % TPR);
  const BwdRow r = bwd_row<F, RPB>(p, work_item(p.lines), local_row<TPR>());
  if (!r.valid) return;
  const int kload = r.kload;
  const uint32_t row_bytes = p.g.Sk * F::kBytes;
  constexpr bool kBuf = TPR >= 64 && kBufRows;
  RowStream ys, ds, xs;
  const bool exact = p.lines != 0;
  if constexpr (kBuf) {
    ys = row_stream(r.y, row_bytes);
    ds = row_stream(r.d, row_bytes);
    xs = row_stream(r.x, row_bytes);
  }
  u32x4 yr[NV], dr[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    if (v * E < kload) {
      if (kBuf && !exact) {
        yr[j] = rs_load(ys, (uint32_t)v * 16);
        dr[j] = rs_load(ds, (uint32_t)v * 16);
      } else {
        yr[j] = ld_stream(r.y + (int64_t)v * 16);
        dr[j] = ld_stream(r.d + (int64_t)v * 16);
      }
    }
  }
  // Wavefronts whose every vector lies past the causal bound (y = 0 there)
  // loaded nothing: they store zeros and end, and the others reduce among
  // themselves (tested after the loads are issued, so as not to delay them).
  int nw = TPR > 64 ? TPR / 64 : 1;
  if constexpr (EARLY && TPR > 64) {
    nw = min(TPR / 64, (kload + 64 * E - 1) / (64 * E));
    if ((int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >= nw) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int v = j * TPR + lane;
        if (v * E < (int)p.g.Sk) out_store<kBuf>(xs, r.x, exact, v, u32x4{0, 0, 0, 0});
      }
      return;
    }
  }
  double acc = 0.0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k0 = (j * TPR + lane) * E;
    if (k0 < kload) {
      float yv[E], gv[E];
      F::unpack(yr[j], yv);
      F::unpack(dr[j], gv);
      if (k0 + E > kload) {  // keys past the bound are not used
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (k0 + e >= kload) yv[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc += F::prod(yv[e], gv[e]);
    }
  }
  acc = row_reduce<TPR>(acc, OpAdd(), red, nw);
  const float dot_hi = (float)acc;
  const float dot_lo = (float)(acc - (double)dot_hi);
  const float scale = p.scale;
  const int Sk = (int)p.g.Sk;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * TPR + lane;
    const int k0 = v * E;
    if (k0 < Sk) {
      float o[E];
      if (k0 < kload) {
        float yv[E], gv[E];
        F::unpack(yr[j], yv);
        F::unpack(dr[j], gv);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = (yv[e] * scale) * ((gv[e] - dot_hi) - dot_lo);
        if (k0 + E > kload) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (k0 + e >= kload) o[e] = 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = 0.0f;
      }
      out_store<kBuf>(xs, r.x, exact, v, F::pack(o));
    }
  }
}

// ------------------------------------------------------ long rows: streaming
//
// Rows longer than a workgroup's registers hold (more than 4096 vectors) run
// one 1024-lane workgroup per row in two passes. Pass 1 reads the row in
// chunks of kStreamCv vectors per lane and keeps, per lane, a running maximum
// and a running sum of exponentials, rescaled by exp(m_old - m_new) whenever
// the maximum grows -- the online softmax of the 0539edu.com notes (fused
// attention section) applied to one row; the lanes' (max, sum) pairs are then
// merged across the workgroup. Pass 2 reads the row again and writes y. The
// backward likewise accumulates the row's dot product in pass 1 and writes dx
// in pass 2. The second read of a row usually hits the L2 or the Infinity
// Cache; the HBM traffic grows by at most the re-read. Any alignment.

constexpr int kStreamTpr = 1024;
constexpr int kStreamCv = 4;

// Folds the (max, biased sum) pair (pm, pl) into (m, l).
SMS_DEV void merge_ml(float& m, float& l, float pm, float pl) {
  if (pm == kNegInf) return;
  if (pm > m) {
    l = (m == kNegInf) ? pl : l * __builtin_amdgcn_exp2f((m - pm) * kLog2e) + pl;
    m = pm;
  } else {
    l += pl * __builtin_amdgcn_exp2f((pm - m) * kLog2e);
  }
}

// The workgroup's (max, biased sum) from every lane's pair, in a fixed order.
template <int TPR>
SMS_DEV void block_ml(float m, float l, float (&red)[2][TPR / 64], float& M, float& L) {
  M = row_reduce<TPR>(m, OpMax(), red[0]);
  const float mine = (m == kNegInf) ? 0.0f : l * __builtin_amdgcn_exp2f((m - M) * kLog2e);
  L = row_reduce<TPR>(mine, OpAdd(), red[1]);
}

// Pass 1 over vectors [v0, v1) of a row: this lane's running (max, biased sum).
template <class F, int TPR>
SMS_DEV void online_ml(const FwdRow& r, int kind, float scale, int v0, int v1, float& m_run,
                       float& l_run) {
  constexpr int E = F::kE;
  constexpr int CV = kStreamCv;
  const int lane = (int)(threadIdx.x % TPR);
  for (int base = v0; base < v1; base += TPR * CV) {
    float s[CV][E];
#pragma unroll
    for (int j = 0; j < CV; ++j) {
      const int v = base + j * TPR + lane;
      if (v < v1) {
        row_scores_branch_loads<F, false>(r, kind, v, scale, s[j]);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[j][e] = kNegInf;
      }
    }
    float cm = kNegInf;
#pragma unroll
    for (int j = 0; j < CV; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) cm = fmaxf(cm, s[j][e]);
    if (cm > m_run) {
      l_run = (m_run == kNegInf) ? 0.0f : l_run * __builtin_amdgcn_exp2f((m_run - cm) * kLog2e);
      m_run = cm;
    }
    if (m_run != kNegInf) {
#pragma unroll
      for (int j = 0; j < CV; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) l_run += exp_biased(s[j][e], m_run);
    }
  }
}

// Pass 2 over vectors [v0, v1) of a row: y = exp(s - M) / L, zeros past the bound.
template <class F, int TPR>
SMS_DEV void write_probs(const FwdRow& r, int kind, float scale, float mref, float inv, int v0,
                         int v1, int Sk) {
  constexpr int E = F::kE;
  constexpr int CV = kStreamCv;
  const int lane = (int)(threadIdx.x % TPR);
  for (int base = v0; base < v1; base += TPR * CV) {
#pragma unroll
    for (int j = 0; j < CV; ++j) {
      const int v = base + j * TPR + lane;
      if (v < v1) {
        float o[E];
        if (v * E - r.ax >= r.kload) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = 0.0f;
        } else {
          row_scores_branch_loads<F>(r, kind, v, scale, o);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = exp_biased(o[e], mref) * inv;
        }
        row_store<F>(r.y, r.yvec, r.ax, v, Sk, o);
      }
    }
  }
}

// Pass 1 of the backward over vectors [v0, v1): this lane's part of sum dy*y.
template <class F, int TPR>
SMS_DEV double dot_part(const BwdRow& r, int v0, int v1) {
  constexpr int E = F::kE;
  constexpr int CV = kStreamCv;
  const int lane = (int)(threadIdx.x % TPR);
  double acc = 0.0;
  for (int base = v0; base < v1; base += TPR * CV) {
#pragma unroll
    for (int j = 0; j < CV; ++j) {
      const int v = base + j * TPR + lane;
      if (v < v1) {
        float yv[E], gv[E];
        row_pair_branch_loads<F, false>(r, v, yv, gv);
#pragma unroll
        for (int e = 0; e < E; ++e) acc += F::prod(yv[e], gv[e]);
      }
    }
  }
  return acc;
}

// Pass 2 of the backward over vectors [v0, v1): dx = scale*y*(dy - dot).
template <class F, int TPR>
SMS_DEV void write_grads(const BwdRow& r, float scale, double dot, int v0, int v1, int Sk) {
  constexpr int E = F::kE;
  constexpr int CV = kStreamCv;
  const int lane = (int)(threadIdx.x % TPR);
  const float dot_hi = (float)dot;
  const float dot_lo = (float)(dot - (double)dot_hi);
  for (int base = v0; base < v1; base += TPR * CV) {
#pragma unroll
    for (int j = 0; j < CV; ++j) {
      const int v = base + j * TPR + lane;
      if (v < v1) {
        float o[E];
        if (v * E - r.ay >= r.kload) {
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = 0.0f;
        } else {
          float yv[E], gv[E];
          row_pair_branch_loads<F>(r, v, yv, gv);
#pragma unroll
          for (int e = 0; e < E; ++e) o[e] = (yv[e] * scale) * ((gv[e] - dot_hi) - dot_lo);
        }
        row_store<F>(r.x, r.xvec, r.ay, v, Sk, o);
      }
    }
  }
}

template <class F>
__global__ void __launch_bounds__(kStreamTpr) sms_fwd_stream_kernel(FwdParams p) {
  constexpr int E = F::kE;
  constexpr int TPR = kStreamTpr;
  __shared__ float red[2][TPR / 64];
  const FwdRow r = fwd_row<F, 1>(p, blockIdx.x, 0);  // one row per workgroup, grid = rows
  const int Sk = (int)p.g.Sk;
  const int nvec = (int)(((int64_t)r.ax + r.kload + E - 1) / E);  // vectors holding read keys
  const int nvec_out = (int)(((int64_t)r.ax + Sk + E - 1) / E);
  float m = kNegInf, l = 0.0f, M, L;
  online_ml<F, TPR>(r, p.mask_kind, p.scale, 0, nvec, m, l);
  block_ml<TPR>(m, l, red, M, L);
  const float mref = (M == kNegInf) ? 0.0f : M;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // fully masked row -> zeros
  write_probs<F, TPR>(r, p.mask_kind, p.scale, mref, inv, 0, nvec_out, Sk);
}

template <class F>
__global__ void __launch_bounds__(kStreamTpr) sms_bwd_stream_kernel(BwdParams p) {
  constexpr int E = F::kE;
  constexpr int TPR = kStreamTpr;
  __shared__ double red[TPR / 64];
  const BwdRow r = bwd_row<F, 1>(p, blockIdx.x, 0);
  const int Sk = (int)p.g.Sk;
  const int nvec = (int)(((int64_t)r.ay + r.kload + E - 1) / E);
  const int nvec_out = (int)(((int64_t)r.ay + Sk + E - 1) / E);
  const double dot = row_reduce<TPR>(dot_part<F, TPR>(r, 0, nvec), OpAdd(), red);
  write_grads<F, TPR>(r, p.scale, dot, 0, nvec_out, Sk);
}

// ------------------------------------------------- long rows, few of them: split
//
// With too few rows to fill the GPU at one workgroup per row, each row is cut
// into `chunks` chunks of `chunk_vec` vectors and every (chunk, row) pair gets
// a 256-lane workgroup (grid chunks x rows), in two launches. The first writes
// each chunk's (max, biased sum) -- the backward: its partial dot product -- to
// the workspace; the second merges the row's partials lane-strided and then
// across the workgroup, in a fixed order (deterministic), and writes its
// chunk's outputs, reading the chunk's inputs again (from the caches when the
// rows fit in them). The per-chunk pairs merge as in the streaming pass 1.

constexpr int kSplitTpr = 256;

template <class F>
__global__ void __launch_bounds__(kSplitTpr) sms_fwd_split_partial_kernel(FwdParams p) {
  constexpr int E = F::kE;
  __shared__ float red[2][kSplitTpr / 64];
  const FwdRow r = fwd_row<F, 1>(p, blockIdx.y, 0);  // grid.y = rows
  const int nvec = (int)(((int64_t)r.ax + r.kload + E - 1) / E);
  const int v0 = (int)(blockIdx.x * p.chunk_vec);
  const int v1 = min(v0 + (int)p.chunk_vec, nvec);
  float m = kNegInf, l = 0.0f, M, L;
  online_ml<F, kSplitTpr>(r, p.mask_kind, p.scale, v0, v1, m, l);
  block_ml<kSplitTpr>(m, l, red, M, L);
  if (threadIdx.x == 0) p.ws[(size_t)blockIdx.y * p.chunks + blockIdx.x] = make_float2(M, L);
}

template <class F>
__global__ void __launch_bounds__(kSplitTpr) sms_fwd_split_final_kernel(FwdParams p) {
  constexpr int E = F::kE;
  __shared__ float red[2][kSplitTpr / 64];
  const FwdRow r = fwd_row<F, 1>(p, blockIdx.y, 0);
  const int Sk = (int)p.g.Sk;
  const float2* part = p.ws + (size_t)blockIdx.y * p.chunks;
  float m = kNegInf, l = 0.0f, M, L;
  for (uint32_t c = threadIdx.x; c < p.chunks; c += kSplitTpr) {
    const float2 pc = part[c];
    merge_ml(m, l, pc.x, pc.y);
  }
  block_ml<kSplitTpr>(m, l, red, M, L);
  const float mref = (M == kNegInf) ? 0.0f : M;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int nvec_out = (int)(((int64_t)r.ax + Sk + E - 1) / E);
  const int v0 = (int)(blockIdx.x * p.chunk_vec);
  const int v1 = min(v0 + (int)p.chunk_vec, nvec_out);
  write_probs<F, kSplitTpr>(r, p.mask_kind, p.scale, mref, inv, v0, v1, Sk);
}

template <class F>
__global__ void __launch_bounds__(kSplitTpr) sms_bwd_split_partial_kernel(BwdParams p) {
  constexpr int E = F::kE;
  __shared__ double red[kSplitTpr / 64];
  const BwdRow r = bwd_row<F, 1>(p, blockIdx.y, 0);
  const int nvec = (int)(((int64_t)r.ay + r.kload + E - 1) / E);
  const int v0 = (int)(blockIdx.x * p.chunk_vec);
  const int v1 = min(v0 + (int)p.chunk_vec, nvec);
  const double d = row_reduce<kSplitTpr>(dot_part<F, kSplitTpr>(r, v0, v1), OpAdd(), red);
  if (threadIdx.x == 0) p.ws[(size_t)blockIdx.y * p.chunks + blockIdx.x] = d;
}

template <class F>
__global__ void __launch_bounds__(kSplitTpr) sms_bwd_split_final_kernel(BwdParams p) {
  constexpr int E = F::kE;
  __shared__ double red[kSplitTpr / 64];
  const BwdRow r = bwd_row<F, 1>(p, blockIdx.y, 0);
  const int Sk = (int)p.g.Sk;
  const double* part = p.ws + (size_t)blockIdx.y * p.chunks;
  double d = 0.0;
  for (uint32_t c = threadIdx.x; c < p.chunks; c += kSplitTpr) d += part[c];
  const double dot = row_reduce<kSplitTpr>(d, OpAdd(), red);
  const int nvec_out = (int)(((int64_t)r.ay + Sk + E - 1) / E);
  const int v0 = (int)(blockIdx.x * p.chunk_vec);
  const int v1 = min(v0 + (int)p.chunk_vec, nvec_out);
  write_grads<F, kSplitTpr>(r, p.scale, dot, v0, v1, Sk);
}

// ------------------------------------------------------- double precision
//
// fp64 inputs are computed in fp64 throughout (the lmnt.cn page's wrapper
// dispatches float, double and half; widening double to fp32 would lose the
// precision the caller asked for). One kernel pair for every row length and
// alignment: TPR lanes per row, lane k takes keys k, k + TPR, ...: 8-byte
// loads and stores, coalesced across the wavefront. Forward: pass 1 keeps a
// per-lane running (max, sum of exp(s - max)), merged across the row; pass 2
// reads the row again and writes exp(s - M) / L (fp64 exp from the device math
// library). Backward: pass 1 the fp64 dot product, pass 2 dx.

struct Fp64 {  // row geometry only (fwd_row / bwd_row)
  static constexpr int kBytes = 8;
  static constexpr int kE = 2;
};

constexpr double kNegInfD = -__builtin_inf();

// Score of key k < kload of a row: x*scale (+ additive mask), -inf if excluded.
SMS_DEV double score_f64(const FwdRow& r, int kind, double scale, int k, bool nt) {
  const double* xp = reinterpret_cast<const double*>(r.x) + k;
  const double xv = nt ? __builtin_nontemporal_load(xp) : *xp;
  if (kind == MASK_ADD) return fma(xv, scale, reinterpret_cast<const double*>(r.m)[k]);
  if (kind == MASK_BOOL && r.m[k] != 0) return kNegInfD;
  return xv * scale;
}

template <int TPR>
__global__ void __launch_bounds__(block_of(TPR)) sms_fwd_f64_kernel(FwdParams p) {
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ double red[2][TPR > 64 ? TPR / 64 : 1];
  const int lane = (int)(threadIdx.x % TPR);
  const FwdRow r = fwd_row<Fp64, RPB>(p, blockIdx.x, local_row<TPR>());
  if (!r.valid) return;  // only a tail group of a TPR <= 64 launch, which has no barrier
  const int Sk = (int)p.g.Sk;
  const int kind = p.mask_kind;
  const double scale = p.scale;
  double m = kNegInfD, l = 0.0;
  for (int k = lane; k < r.kload; k += TPR) {
    const double s = score_f64(r, kind, scale, k, false);
    if (s > m) {
      l = (m == kNegInfD) ? 0.0 : l * exp(m - s);
      m = s;
    }
    if (s != kNegInfD) l += exp(s - m);
  }
  const double M = row_reduce<TPR>(m, OpMax(), red[0]);
  const double mine = (m == kNegInfD) ? 0.0 : l * exp(m - M);
  const double L = row_reduce<TPR>(mine, OpAdd(), red[1]);
  const double inv = L > 0.0 ? 1.0 / L : 0.0;  // fully masked row -> zeros
  double* yp = reinterpret_cast<double*>(r.y);
  for (int k = lane; k < Sk; k += TPR) {
    double o = 0.0;
    if (k < r.kload && inv != 0.0) o = exp(score_f64(r, kind, scale, k, true) - M) * inv;
    __builtin_nontemporal_store(o, yp + k);
  }
}

template <int TPR>
__global__ void __launch_bounds__(block_of(TPR)) sms_bwd_f64_kernel(BwdParams p) {
  constexpr int RPB = block_of(TPR) / TPR;
  __shared__ double red[TPR > 64 ? TPR / 64 : 1];
  const int lane = (int)(threadIdx.x % TPR);
  const BwdRow r = bwd_row<Fp64, RPB>(p, blockIdx.x, local_row<TPR>());
  if (!r.valid) return;
  const int Sk = (int)p.g.Sk;
  const double* yp = reinterpret_cast<const double*>(r.y);
  const double* dp = reinterpret_cast<const double*>(r.d);
  double acc = 0.0;
  for (int k = lane; k < r.kload; k += TPR) acc = fma(yp[k], dp[k], acc);
  const double dot = row_reduce<TPR>(acc, OpAdd(), red);
  const double scale = p.scale;
  double* xp = reinterpret_cast<double*>(r.x);
  for (int k = lane; k < Sk; k += TPR) {
    double o = 0.0;
    if (k < r.kload) {
      const double yv = __builtin_nontemporal_load(yp + k);
      const double dv = __builtin_nontemporal_load(dp + k);
      o = (yv * scale) * (dv - dot);
    }
    __builtin_nontemporal_store(o, xp + k);
  }
}

// Lanes per fp64 row: one wavefront for rows up to 256 keys (four rows per
// workgroup), else 256.
constexpr int f64_tpr(int64_t Sk) { return Sk <= 256 ? 64 : 256; }

inline hipError_t launch_f64(const FwdParams* fp, const BwdParams* bp, int tpr, uint32_t blocks,
                             hipStream_t st) {
  const dim3 grid(blocks), block(256);
  if (tpr == 64) {
    if (fp) hipLaunchKernelGGL((sms_fwd_f64_kernel<64>), grid, block, 0, st, *fp);
    else hipLaunchKernelGGL((sms_bwd_f64_kernel<64>), grid, block, 0, st, *bp);
  } else if (tpr == 256) {
    if (fp) hipLaunchKernelGGL((sms_fwd_f64_kernel<256>), grid, block, 0, st, *fp);
    else hipLaunchKernelGGL((sms_bwd_f64_kernel<256>), grid, block, 0, st, *bp);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- launchers

// Kernel families.
enum : int {
  FAMILY_GENERAL = 0,
  FAMILY_ALIGNED = 1,
  FAMILY_STREAM = 2,
  FAMILY_SPLIT = 3,
  FAMILY_F64 = 4,
  FAMILY_HEADS = 5  // aligned forward over head groups (forward only, TPR >= 128)
};

// Heads per workgroup the head-group forward is built with.
constexpr int kHeadsList[] = {2, 4};

// Head groups are built for 128 to 512 lanes and heads * NV <= 4 (the G rows
// then fit in VGPRs without spilling).
constexpr bool heads_built(int tpr, int nv, int g) { return tpr >= 128 && tpr <= 512 && g * nv <= 4; }

template <class F, int TPR, int NV, int KIND>
hipError_t launch_heads(const FwdParams* fp, uint32_t blocks, hipStream_t st) {
  const dim3 grid(blocks), block(TPR);
  if constexpr (heads_built(TPR, NV, 2)) {
    if (fp->heads == 2) {
      hipLaunchKernelGGL((sms_fwd_heads_kernel<F, TPR, NV, KIND, 2>), grid, block, 0, st, *fp);
      return hipGetLastError();
    }
  }
  if constexpr (heads_built(TPR, NV, 4)) {
    if (fp->heads == 4) {
      hipLaunchKernelGGL((sms_fwd_heads_kernel<F, TPR, NV, KIND, 4>), grid, block, 0, st, *fp);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

// TPR and NV values the library is built with.
constexpr int kTprList[] = {4, 8, 16, 32, 64, 128, 256, 512, 1024};
constexpr int kNvList[] = {1, 2, 4};

template <class F, int TPR, int NV, bool EARLY>
hipError_t launch_fwd_fast(const FwdParams* fp, uint32_t blocks, hipStream_t st) {
  if constexpr (EARLY && TPR <= 64) {
    return hipErrorInvalidValue;  // rows of one wavefront or less: nothing ends early
  } else {
    const dim3 grid(blocks), block(block_of(TPR));
    if (fp->mask_kind == MASK_ADD)
      hipLaunchKernelGGL((sms_fwd_fast_kernel<F, TPR, NV, FAST_ADD, EARLY>), grid, block, 0, st, *fp);
    else if (fp->mask_kind == MASK_BOOL)
      hipLaunchKernelGGL((sms_fwd_fast_kernel<F, TPR, NV, FAST_BOOL, EARLY>), grid, block, 0, st, *fp);
    else
      hipLaunchKernelGGL((sms_fwd_fast_kernel<F, TPR, NV, FAST_PLAIN, EARLY>), grid, block, 0, st, *fp);
    return hipGetLastError();
  }
}

template <class F, int TPR, int NV>
hipError_t launch_nv(const FwdParams* fp, const BwdParams* bp, int family, uint32_t blocks,
                     hipStream_t st) {
  const dim3 grid(blocks), block(block_of(TPR));
  if (fp) {
    if (family == FAMILY_HEADS) {
      if (fp->mask_kind == MASK_ADD) return launch_heads<F, TPR, NV, FAST_ADD>(fp, blocks, st);
      if (fp->mask_kind == MASK_BOOL) return launch_heads<F, TPR, NV, FAST_BOOL>(fp, blocks, st);
      return launch_heads<F, TPR, NV, FAST_PLAIN>(fp, blocks, st);
    }
    if (family == FAMILY_ALIGNED) {
      if (fp->early && TPR > 64) return launch_fwd_fast<F, TPR, NV, true>(fp, blocks, st);
      return launch_fwd_fast<F, TPR, NV, false>(fp, blocks, st);
    } else {
      hipLaunchKernelGGL((sms_fwd_kernel<F, TPR, NV>), grid, block, 0, st, *fp);
    }
  } else {
    if (family == FAMILY_ALIGNED) {
      if constexpr (TPR > 64) {
        if (bp->early) {
          hipLaunchKernelGGL((sms_bwd_fast_kernel<F, TPR, NV, true>), grid, block, 0, st, *bp);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((sms_bwd_fast_kernel<F, TPR, NV, false>), grid, block, 0, st, *bp);
    } else
      hipLaunchKernelGGL((sms_bwd_kernel<F, TPR, NV>), grid, block, 0, st, *bp);
  }
  return hipGetLastError();
}

template <class F, int TPR>
hipError_t launch_tpr(const FwdParams* fp, const BwdParams* bp, int family, int nv,
                      uint32_t blocks, hipStream_t st) {
  switch (nv) {
    case 1: return launch_nv<F, TPR, 1>(fp, bp, family, blocks, st);
    case 2: return launch_nv<F, TPR, 2>(fp, bp, family, blocks, st);
    case 4: return launch_nv<F, TPR, 4>(fp, bp, family, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

// One launch: exactly one of fp / bp is non-null. The streaming family
// ignores tpr / nv and takes one workgroup per row (blocks = rows); the split
// family launches twice over a grid of chunks x rows (blocks = rows).
template <class F>
hipError_t launch(const FwdParams* fp, const BwdParams* bp, int family, int tpr, int nv,
                  uint32_t blocks, hipStream_t st) {
  if (family == FAMILY_SPLIT) {
    const dim3 grid(fp ? fp->chunks : bp->chunks, blocks), block(kSplitTpr);
    if (fp) hipLaunchKernelGGL((sms_fwd_split_partial_kernel<F>), grid, block, 0, st, *fp);
    else hipLaunchKernelGGL((sms_bwd_split_partial_kernel<F>), grid, block, 0, st, *bp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fp) hipLaunchKernelGGL((sms_fwd_split_final_kernel<F>), grid, block, 0, st, *fp);
    else hipLaunchKernelGGL((sms_bwd_split_final_kernel<F>), grid, block, 0, st, *bp);
    return hipGetLastError();
  }
  if (bp && family == FAMILY_ALIGNED && tpr == 1024 && nv == 8) {
    // Long rows of the aligned backward, held in VGPRs in one pass (built for
    // this width only).
    if (bp->early)
      hipLaunchKernelGGL((sms_bwd_fast_kernel<F, 1024, 8, true>), dim3(blocks), dim3(1024), 0, st, *bp);
    else
      hipLaunchKernelGGL((sms_bwd_fast_kernel<F, 1024, 8, false>), dim3(blocks), dim3(1024), 0, st, *bp);
    return hipGetLastError();
  }
  if (family == FAMILY_STREAM) {
    if (fp)
      hipLaunchKernelGGL((sms_fwd_stream_kernel<F>), dim3(blocks), dim3(kStreamTpr), 0, st, *fp);
    else
      hipLaunchKernelGGL((sms_bwd_stream_kernel<F>), dim3(blocks), dim3(kStreamTpr), 0, st, *bp);
    return hipGetLastError();
  }
  switch (tpr) {
    case 4: return launch_tpr<F, 4>(fp, bp, family, nv, blocks, st);
    case 8: return launch_tpr<F, 8>(fp, bp, family, nv, blocks, st);
    case 16: return launch_tpr<F, 16>(fp, bp, family, nv, blocks, st);
    case 32: return launch_tpr<F, 32>(fp, bp, family, nv, blocks, st);
    case 64: return launch_tpr<F, 64>(fp, bp, family, nv, blocks, st);
    case 128: return launch_tpr<F, 128>(fp, bp, family, nv, blocks, st);
    case 256: return launch_tpr<F, 256>(fp, bp, family, nv, blocks, st);
    case 512: return launch_tpr<F, 512>(fp, bp, family, nv, blocks, st);
    case 1024: return launch_tpr<F, 1024>(fp, bp, family, nv, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sms

// Per-format launch entry points, one translation unit each (inst_*.hip).
hipError_t sms_launch_f32(const sms::FwdParams*, const sms::BwdParams*, int family, int tpr,
                          int nv, uint32_t blocks, hipStream_t);
hipError_t sms_launch_f16(const sms::FwdParams*, const sms::BwdParams*, int family, int tpr,
                          int nv, uint32_t blocks, hipStream_t);
hipError_t sms_launch_bf16(const sms::FwdParams*, const sms::BwdParams*, int family, int tpr,
                           int nv, uint32_t blocks, hipStream_t);
hipError_t sms_launch_f64(const sms::FwdParams*, const sms::BwdParams*, int tpr, uint32_t blocks,
                          hipStream_t);
