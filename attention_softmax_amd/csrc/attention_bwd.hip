// attention_bwd.hip -- fused attention backward on the gfx950 matrix cores:
// dQ, dK, dV of L = sum(dO * O) for O = softmax(Q K^T * scale + mask) V,
// recomputing the probabilities from the forward's log-sum-exp instead of
// storing them (the FlashAttention-style scheme the pnsm.cn article's sec. 4.4
// points to; the softmax gradient itself is the lmnt.cn page's sec. 3.3 rule,
// dS = P * (dP - rowsum(dP * P)), with rowsum(dP * P) = rowsum(dO * O)).
//
// Two launches (three for D = 128 with a per-score mask on grids of 512 or
// more dK/dV workgroups, where dK and dV take a pass each), all deterministic
// (no atomics):
//  1. dQ, one workgroup per 128 queries (query-stationary, as the forward);
//     it first forms delta = rowsum(dO * O) of its queries in fp32 and stores
//     it in the workspace for step 2. S^T = K Q^T and dP^T = V dO^T leave
//     each lane 16 keys of one query;
//     P = exp(S*scale + mask - LSE); dS^T = P (dP^T - delta); dQ^T += K^T dS^T
//     with the dS registers as the B operand (keys contracted in the order the
//     S^T layout holds them, K^T read from the row-major K tile by
//     transposing LDS reads);
//  2. dK and dV, one workgroup per 128 keys of one key/value head
//     (key-stationary): for every query head of its group and every tile of
//     32 or 64 queries, S = Q K^T and dP = dO V^T leave each lane 16 queries
//     of one key per 32-query block; dV^T += dO^T P and dK^T += Q^T dS with P
//     and dS as B operands.
// The tiles (K and V in 1, Q and dO in 2) come from global memory straight
// into double-buffered LDS (dswz layout, loads issued from inline assembly,
// dma_tile_asm), one barrier per tile or query step.
// Lane layouts of v_mfma_f32_32x32x16: see attention.hip.

#include "attention.hpp"

namespace sms {
namespace {

using namespace attn;

// ---------------------------------------------------------------- 1. dQ

// K and V tiles of 64 keys come straight from global memory into
// double-buffered LDS (dswz layout): one barrier per tile, after which the
// next tile's loads go out into the other buffer. K serves both the row reads
// of S^T = K Q^T and the transposing reads that form the K^T operand of
// dQ^T += K^T dS^T; V the row reads of dP^T = V dO^T.
// Three wavefronts per SIMD for D = 64 (140-146 VGPRs: the backward 1.5-3 %
// faster than at two on fp16 [8,32,2048,64] and [4,32,4096,64]), two for D = 128.
// Per-score masks, MV: 2 / 3 (additive / boolean masks whose rows start on
// 16-byte lines): the tile's mask values for the workgroup's 128 queries come
// into one LDS buffer (a 128 x 64 tile, the dswz layout of D = 64 / 32), each
// lane reads its runs at the start of the tile, and after a second barrier
// (all runs read) the next tile's values go out into it, as in the forward;
// 1: the runs are loaded from global memory at the start of the tile; 0: each
// value where it is used.
template <bool BF16, int D, int KIND, int MV>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
attn_bwd_dq_kernel(AttnBwdParams p) {
  static_assert(MV == 0 || KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL, "mask runs need a per-score mask");
  static_assert(MV != 2 || KIND == ATTN_MASK_ADD, "mask tiles of 16-bit values");
  static_assert(MV != 3 || KIND == ATTN_MASK_BOOL, "mask tiles of bytes");
  constexpr int BK = kAttnBk;
  constexpr int TB = BK * D * 2;  // bytes per tile
  constexpr int MB = MV == 3 ? 1 : 2;  // bytes per mask value
  constexpr int MD = 32 * MB;          // the mask tile's dswz layout
  constexpr int TM = kAttnBq * BK * MB;  // bytes per mask tile (MV >= 2)
  // K tiles at 0 and TB, V tiles at 2 TB and 3 TB; bit TB of the offsets
  // picks a tile's buffer and flips every tile.
  __shared__ __align__(1024) uint8_t kv[4 * TB];
  __shared__ __align__(1024) uint8_t ms[MV >= 2 ? TM : 16];

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Same workgroup order as the forward.
  const uint32_t N = gridDim.x, per = N / 8, HB = p.H * p.B;
  const uint32_t ntq = N / HB;
  uint32_t t = blockIdx.x, hb, qt;
  if (p.causal) {
    hb = t % HB;
    qt = ntq - 1 - t / HB;
  } else {
    if (t < per * 8) t = (t % 8) * per + t / 8;
    hb = t / ntq;
    qt = t % ntq;
  }
  const uint32_t h = hb % p.H, b = hb / p.H;
  const int q0 = (int)(qt * kAttnBq);
  const int qi = q0 + wave * 32 + c;
  const int Sq = (int)p.Sq, Sk = (int)p.Sk;
  const uint32_t hk = h / p.group;
  const char* kbase = p.k + ((int64_t)b * p.sk_b + (int64_t)hk * p.sk_h) * 2;
  const char* vbase = p.v + ((int64_t)b * p.sv_b + (int64_t)hk * p.sv_h) * 2;

  const int off = p.causal == 2 ? Sk - Sq : 0;
  int klen = Sk;
  if constexpr (KIND == ATTN_MASK_LEN)
    klen = max(min(reinterpret_cast<const int32_t*>(p.mask)[b], Sk), 0);
  int kend = klen;
  if (p.causal) kend = min(kend, max(q0 + kAttnBq + off, 0));
  int kq = klen;
  if (p.causal) kq = min(kq, max(qi + off + 1, 0));
  const bool qvalid = qi < Sq;
  const int64_t mrow = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)qi * p.sm_q;
  // The same for a query clamped into the mask (unconditional vector loads).
  const int64_t mrow_c =
      (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)min(qi, Sq - 1) * p.sm_q;
  const int64_t lrow = ((int64_t)b * p.H + h) * Sq + qi;
  const float lse = qvalid ? p.lse[lrow] : kNegInfA;
  const bool live = lse != kNegInfA;  // a query that sees no key has no gradient
  const float lse2 = live ? lse * kLog2eA : 0.0f;

  // Q and dO fragments: the B operands of S^T = K Q^T and dP^T = V dO^T.
  // Lanes c and c + 32 hold the two halves of query qi's rows, so the same
  // loads of O give delta = rowsum(dO * O) of the query with one exchange;
  // lanes of the first half store it for the dK pass.
  u32x4 qf[D / 16], df[D / 16];
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    df[s] = u32x4{0, 0, 0, 0};
    if (qvalid) {
      qf[s] = *reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)b * p.sq_b + (int64_t)h * p.sq_h + (int64_t)qi * p.sq_s + s * 16 + 8 * g) * 2);
      df[s] = *reinterpret_cast<const u32x4*>(
          p.dout + ((int64_t)b * p.sdo_b + (int64_t)h * p.sdo_h + (int64_t)qi * p.sdo_s + s * 16 + 8 * g) * 2);
      const u32x4 of = *reinterpret_cast<const u32x4*>(
          p.o + ((int64_t)b * p.so_b + (int64_t)h * p.so_h + (int64_t)qi * p.so_s + s * 16 + 8 * g) * 2);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        dpart = fmaf(to_float<BF16>(elem(df[s], j)), to_float<BF16>(elem(of, j)), dpart);
    }
  }
  const float delta = dpart + __shfl_xor(dpart, 32);
  if (qvalid && g == 0) p.delta[lrow] = delta;
  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.0f;

  // Tile loads (rows past the last key read as zero; a tile past it loads
  // nothing but zeros).
  const uint32_t kdo = dma_lane_off<D>(lane, wave_u, p.sk_s * 2);
  const uint32_t vdo = dma_lane_off<D>(lane, wave_u, p.sv_s * 2);
  const uint32_t kv_lds = lds_addr(kv);
  auto dma = [&](int kt, int buf) {
    const int rows = min(Sk - kt, BK);
    const u32x4 kr = rows_desc(kbase + (int64_t)kt * p.sk_s * 2, rows, p.sk_s * 2, D * 2);
    const u32x4 vr = rows_desc(vbase + (int64_t)kt * p.sv_s * 2, rows, p.sv_s * 2, D * 2);
    dma_tile_asm<D, BK>(kr, kdo, p.sk_s * 2, wave_u, kv_lds + buf * TB);
    dma_tile_asm<D, BK>(vr, vdo, p.sv_s * 2, wave_u, kv_lds + (2 + buf) * TB);
  };
  // Mask tiles (MV >= 2): the workgroup's query rows through one buffer range
  // ending at the last row's last key; keys past Sk of the other rows read
  // the next row's first values, whose scores are excluded.
  const uint32_t mdo = dma_lane_off<MD>(lane, wave_u, p.sm_q * MB);
  const int mrows = min(Sq - q0, kAttnBq);
  auto dma_mask = [&](int kt) {
    const int rows = min(Sk - kt, BK);
    u32x4 mr = rows_desc(p.mask + ((int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)q0 * p.sm_q + kt) * MB,
                         rows > 0 ? mrows : 0, p.sm_q * MB, max(rows, 0) * MB);
#pragma unroll
    for (int j = 0; j < 4; ++j) mr[j] = __builtin_amdgcn_readfirstlane(mr[j]);
    dma_tile_asm<MD, kAttnBq>(mr, mdo, p.sm_q * MB, wave_u, lds_addr(ms));
  };
  if (kend > 0) {
    dma(0, 0);
    if constexpr (MV >= 2) dma_mask(0);
  }

  // LDS byte offsets of this lane's reads. Row reads: row c (+ 32 kb),
  // logical chunk 2 s + g, at rao ^ 32 s (dswz reads the row's low 4 bits
  // only; XOR-ing 2 s into the chunk index is XOR-ing 32 s into the offset).
  // K^T operand (transposing reads): keys 8 hf + 4 g + (c % 16) / 4 (+ 16 s),
  // dims 32 db + 16 ((c / 16) % 2) + 4 (c % 4) .. + 3, at
  // (tao ^ 64 db ^ 32 hf) + 8 hf rows (dswz's bits 0-1 hold bits 2-3 of the
  // key, which hf sets and s leaves).
  uint32_t rao = (uint32_t)dtile_off<D>(c, g);
  uint32_t tao =
      (uint32_t)(dtile_off<D>(4 * g + ((c & 15) >> 2), 2 * ((c >> 4) & 1) + ((c >> 1) & 1)) + 8 * (c & 1));

  for (int kt = 0; kt < kend; kt += BK) {
    const uint8_t* kl = kv;
    const uint8_t* vl = kv + 2 * TB;
    const uint32_t ra = rao, ta = tao;
    // This wavefront's loads of the tile have landed; after the barrier every
    // wavefront's have, and every wavefront is done with the previous tile,
    // whose buffers the next loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    u32x2 mv[8];  // this tile's mask values, loaded before the next tile's loads
    if constexpr (MV == 2) {
      // The lane's runs (keys 32 (i / 4) + 8 (i % 4) + 4 g .. + 3 of its
      // query's row: chunk 4 (i / 4) + i % 4, half g).
#pragma unroll
      for (int i = 0; i < 8; ++i)
        mv[i] = *reinterpret_cast<const u32x2*>(ms + dtile_off<64>(wave * 32 + c, 4 * (i >> 2) + (i & 3)) + 8 * g);
    } else if constexpr (MV == 3) {
      // Boolean runs: run i is the 4 bytes at 8 i + 4 g, in chunk i / 2.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t* ch = ms + dtile_off<32>(wave * 32 + c, j);
        mv[2 * j] = u32x2{*reinterpret_cast<const uint32_t*>(ch + 4 * g), 0u};
        mv[2 * j + 1] = u32x2{*reinterpret_cast<const uint32_t*>(ch + 8 + 4 * g), 0u};
      }
    } else if constexpr (MV == 1) {
      load_mask_runs<KIND>(p.mask, mrow_c, kt, g, Sk, mv);
      __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the loads
    }
    if (MV == 1 || kt + BK < kend) dma(kt + BK, ((kt / BK) & 1) ^ 1);
    if constexpr (MV == 1) __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products

    // dS^T = P (dP^T - delta), P recomputed from the forward's LSE, one
    // 32-key block at a time (the block's products, probabilities and dQ
    // contribution before the next block's, which keeps half the score
    // registers live). A tile whose every score is visible to every query of
    // the workgroup (keys in range and before the first query's causal bound,
    // all queries in range, no per-score mask) skips the exclusion tests.
    const bool inb = kt + BK <= klen && (!p.causal || kt + BK <= q0 + off + 1);
    const bool full = KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL && q0 + kAttnBq <= Sq && inb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.0f;
        dpacc[r] = 0.0f;
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + (ra ^ (32 * s)) + kb * 32 * D * 2);
        sacc = mfma_32x32x16<BF16>(a, qf[s], sacc);
        const u32x4 av = *reinterpret_cast<const u32x4*>(vl + (ra ^ (32 * s)) + kb * 32 * D * 2);
        dpacc = mfma_32x32x16<BF16>(av, df[s], dpacc);
      }
      pin_reads_ahead<2 * (D / 16), 4, 1>();  // K / V reads four products ahead
      if constexpr (MV >= 2) {
        if (kb == 0) {
          // Every wavefront has its runs; the next tile's mask values may
          // overwrite them (a plain barrier: it does not wait for the loads).
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          asm volatile("s_barrier" ::: "memory");
          if (kt + BK < kend) dma_mask(kt + BK);
        }
      }
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], p.scale_log2, -lse2));
          sacc[r] = pv * (dpacc[r] - delta);
        }
      } else if ((KIND == ATTN_MASK_BOOL || (KIND == ATTN_MASK_ADD && MV == 0)) && inb) {
        // Every key in bounds for every query: the mask (and a query without
        // any visible key) alone. (Not for additive runs: the extra code path
        // made that variant spill.)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float tv = sacc[r] * p.scale_log2;
          bool excluded = !live;
          if constexpr (KIND == ATTN_MASK_ADD) {
            uint32_t bits;
            if constexpr (MV != 0) {
              bits = mask_run_value(mv, kb, r, false);
            } else {
              const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              bits = live ? *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2) : 0u;
            }
            tv = fmaf(to_float<BF16>(bits), kLog2eA, tv);
          } else {
            uint32_t byte;
            if constexpr (MV != 0) {
              byte = mask_run_value(mv, kb, r, true);
            } else {
              const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              byte = live ? (uint32_t)(uint8_t)p.mask[mrow + key] : 0u;
            }
            if (byte != 0) excluded = true;
          }
          const float pv = excluded ? 0.0f : __builtin_amdgcn_exp2f(tv - lse2);
          sacc[r] = pv * (dpacc[r] - delta);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          float tv = sacc[r] * p.scale_log2;
          bool excluded = key >= kq || key >= Sk || !live;
          if constexpr (KIND == ATTN_MASK_ADD) {
            if (!excluded) {
              uint32_t bits;
              if constexpr (MV != 0) bits = mask_run_value(mv, kb, r, false);
              else bits = *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2);
              tv = fmaf(to_float<BF16>(bits), kLog2eA, tv);
            }
          } else if constexpr (KIND == ATTN_MASK_BOOL) {
            if (!excluded) {
              uint32_t byte;
              if constexpr (MV != 0) byte = mask_run_value(mv, kb, r, true);
              else byte = (uint32_t)(uint8_t)p.mask[mrow + key];
              if (byte != 0) excluded = true;
            }
          }
          const float pv = excluded ? 0.0f : __builtin_amdgcn_exp2f(tv - lse2);
          sacc[r] = pv * (dpacc[r] - delta);
        }
      }
      // B operands of the block's two k-steps (keys 16 s2 + 8 (j / 4) + 4 g
      // + j % 4 of the block for element j).
      u32x4 pb[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int base = 8 * s2;
        pb[s2] = u32x4{pack2<BF16>(sacc[base + 0], sacc[base + 1]),
                       pack2<BF16>(sacc[base + 2], sacc[base + 3]),
                       pack2<BF16>(sacc[base + 4], sacc[base + 5]),
                       pack2<BF16>(sacc[base + 6], sacc[base + 7])};
      }
      // A operand of k-step s: keys 16 s + 4 g + 0..3 (elements 0-3) and
      // 16 s + 8 + 4 g + 0..3 (elements 4-7) of the lane's dim of K.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int s = 2 * kb + s2;
          const u32x2 a0 = lds_read_tr(kl + (ta ^ (64 * db)) + 16 * s * D * 2);
          const u32x2 a1 = lds_read_tr(kl + (ta ^ (64 * db) ^ 32) + (16 * s + 8) * D * 2);
          dq[db] = mfma_32x32x16<BF16>(u32x4{a0.x, a0.y, a1.x, a1.y}, pb[s2], dq[db]);
        }
      }
      // K^T reads two products ahead for D = 128.
      if constexpr (D == 128) pin_reads_ahead<2 * (D / 32), 2, 2>();
    }
    rao ^= TB;
    tao ^= TB;
  }
  // The last tile's loads into LDS (issued unconditionally with per-score
  // masks) complete before the workgroup, and its LDS, can end.
  __builtin_amdgcn_s_waitcnt(0);

  if (!qvalid) return;
  char* orow = p.dq + ((int64_t)b * p.sdq_b + (int64_t)h * p.sdq_h + (int64_t)qi * p.sdq_s) * 2;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const u32x2 w{pack2<BF16>(dq[db][4 * rg] * sc, dq[db][4 * rg + 1] * sc),
                    pack2<BF16>(dq[db][4 * rg + 2] * sc, dq[db][4 * rg + 3] * sc)};
      *reinterpret_cast<u32x2*>(orow + (db * 32 + 8 * rg + 4 * g) * 2) = w;
    }
}

// ------------------------------------------------------------ 2. dK, dV

// PASS 2 accumulates dK and dV together; for D = 128 that needs more than 256
// registers (one wavefront per SIMD). PASS 0 (dV alone: S, P) and PASS 1 (dK
// alone: S, dP, dS) are the same work as two launches at two or three
// wavefronts per SIMD, recomputing S in both (see launch_dkdv for which).
// MT: mask tiles in LDS (mask rows on 16-byte lines): the step's BQ x 128
// values (additive: the dswz layout of D = 128; boolean: that of D = 64;
// double-buffered) come with its Q and dO tiles. For additive masks each lane
// takes its key's values for 4 consecutive queries per transposing read, as
// the forward reads V; for boolean ones it reads its 16 bytes one by one.
// VL (one pass, D = 128, no per-score mask): V read by rows from an LDS copy
// of the workgroup's 128 keys (32 KB, loaded once) instead of being held in
// registers, which brings the pass within 256 registers: two wavefronts per
// SIMD with 32-query steps (two workgroups' LDS fit a CU).
template <bool BF16, int D, int KIND, int PASS, int BQ, bool MT, bool VL>
__device__ inline __attribute__((always_inline)) void dkdv_body(const AttnBwdParams& p) {
  constexpr bool kDV = PASS != 1, kDK = PASS != 0;
  static_assert(BQ == 32 || BQ == 64, "query tiles of one or two 32-query blocks");
  static_assert(BQ == 32 || (KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL),
                "per-score masks are loaded for one 32-query block per step");
  static_assert(!MT || KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL, "mask tiles of a per-score mask");
  static_assert(!VL || (PASS == 2 && D == 128 && !MT), "the V copy serves the one-pass D = 128 kernel");
  constexpr int NSUB = BQ / 32;
  constexpr int TQ = BQ * D * 2;  // bytes per Q or dO tile
  constexpr int MB = KIND == ATTN_MASK_BOOL ? 1 : 2;  // bytes per mask value
  constexpr int MD = 64 * MB;                            // the mask tile's dswz layout
  constexpr int TMQ = BQ * kAttnBwdBk * MB;  // bytes per mask tile (MT)
  // Q and dO tiles of a step (dswz layout) at 0 and TQ, the next step's at
  // 2 TQ and 3 TQ; bit 2 TQ of the offsets picks a step's buffer. Q serves the
  // row reads of S = Q K^T and the transposing reads of the Q^T operand of
  // dK^T += Q^T dS; dO those of dP = dO V^T and dV^T += dO^T P.
  __shared__ __align__(1024) uint8_t qd[4 * TQ];
  __shared__ __align__(16) float lses[2][BQ];  // LSE * log2(e) of the step's queries
  __shared__ __align__(16) float dels[2][BQ];
  __shared__ __align__(1024) uint8_t mt[MT ? 2 * TMQ : 16];
  __shared__ __align__(1024) uint8_t vl[VL ? kAttnBwdBk * D * 2 : 16];

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int Sq = (int)p.Sq, Sk = (int)p.Sk;
  const uint32_t nkt = (p.Sk + kAttnBwdBk - 1) / kAttnBwdBk;
  // Workgroup order: with a causal rule a key block's work shrinks with its
  // position (its first visible query moves up), so every head's first
  // (longest) block goes first, then every head's second, ...; the short
  // blocks fill the end. Without one: a head's key blocks together, which
  // then read the head's Q / dO tiles at about the same time.
  uint32_t kti, hkb;
  if (p.causal) {
    const uint32_t HKB = p.Hk * p.B;
    kti = blockIdx.x / HKB;
    hkb = blockIdx.x % HKB;
  } else {
    kti = blockIdx.x % nkt;
    hkb = blockIdx.x / nkt;
  }
  const uint32_t hk = hkb % p.Hk, b = hkb / p.Hk;
  const int k0 = (int)(kti * kAttnBwdBk);
  const int kj = k0 + wave * 32 + c;  // this lane's key
  const bool kvalid = kj < Sk;
  const char* kbase = p.k + ((int64_t)b * p.sk_b + (int64_t)hk * p.sk_h) * 2;
  const char* vbase = p.v + ((int64_t)b * p.sv_b + (int64_t)hk * p.sv_h) * 2;

  // K and V fragments: the B operands of S = Q K^T and dP = dO V^T.
  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = u32x4{0, 0, 0, 0};
    vf[s] = u32x4{0, 0, 0, 0};
    if (kvalid) {
      kf[s] = *reinterpret_cast<const u32x4*>(kbase + ((int64_t)kj * p.sk_s + s * 16 + 8 * g) * 2);
      if constexpr (kDK && !VL)
        vf[s] = *reinterpret_cast<const u32x4*>(vbase + ((int64_t)kj * p.sv_s + s * 16 + 8 * g) * 2);
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.0f;
      dv[db][r] = 0.0f;
    }

  const int off = p.causal == 2 ? Sk - Sq : 0;
  int klen = Sk;
  if constexpr (KIND == ATTN_MASK_LEN)
    klen = max(min(reinterpret_cast<const int32_t*>(p.mask)[b], Sk), 0);
  // Queries that may see one of the workgroup's keys: i >= k0 - off (causal).
  int qstart = p.causal ? max(k0 - off, 0) : 0;
  qstart = qstart / BQ * BQ;
  const bool any = k0 < klen;

  // A step's Q and dO tiles are loaded straight into LDS during the step
  // before (rows past Sq read as zero); LSE and delta through a register of
  // the first BQ lanes of wavefronts 0 and 1, written to LDS at the start of
  // the step (scaled, and filled past Sq). Every choice of source is uniform
  // over a wavefront and made once here.
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  const bool is_stat = wave < 2 && lane < BQ;  // LSE (wavefront 0) or delta (wavefront 1)
  const float sfill = swave == 0 ? kNegInfA : 0.0f;
  const float smul = swave == 0 ? kLog2eA : 1.0f;  // LSE is kept in log2 units
  float sreg = 0.0f;
  const float* fssrc = swave == 1 ? p.delta : p.lse;
  const uint32_t soff = (uint32_t)(lane & (BQ - 1)) * 4;
  const char* const qsrc = p.q + (int64_t)b * p.sq_b * 2;
  const char* const dsrc = p.dout + (int64_t)b * p.sdo_b * 2;
  const uint32_t qdo = dma_lane_off<D>(lane, swave, p.sq_s * 2);
  const uint32_t ddo = dma_lane_off<D>(lane, swave, p.sdo_s * 2);
  const uint32_t qd_lds = lds_addr(qd);
  const uint32_t mt_lds = lds_addr(mt);
  const uint32_t mdo = dma_lane_off<MD>(lane, swave, p.sm_q * MB);
  auto fetch = [&](uint32_t h, int qt, int buf) {
    const int rows = min(Sq - qt, BQ);
    const u32x4 qr = rows_desc(qsrc + ((int64_t)h * p.sq_h + (int64_t)qt * p.sq_s) * 2, rows, p.sq_s * 2, D * 2);
    const u32x4 dr = rows_desc(dsrc + ((int64_t)h * p.sdo_h + (int64_t)qt * p.sdo_s) * 2, rows, p.sdo_s * 2, D * 2);
    dma_tile_asm<D, BQ>(qr, qdo, p.sq_s * 2, swave, qd_lds + buf * 2 * TQ);
    dma_tile_asm<D, BQ>(dr, ddo, p.sdo_s * 2, swave, qd_lds + buf * 2 * TQ + TQ);
    if constexpr (MT) {
      // The step's query rows, keys k0 .. k0 + 127 (past Sk: the next row's
      // first values, or zeros past the last row; those scores are excluded).
      u32x4 mr = rows_desc(p.mask + ((int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)qt * p.sm_q + k0) * MB,
                           rows, p.sm_q * MB, min(Sk - k0, kAttnBwdBk) * MB);
#pragma unroll
      for (int j = 0; j < 4; ++j) mr[j] = __builtin_amdgcn_readfirstlane(mr[j]);
      dma_tile_asm<MD, BQ>(mr, mdo, p.sm_q * MB, swave, mt_lds + buf * TMQ);
    }
    const auto sr = rows_rsrc(reinterpret_cast<const char*>(fssrc + ((int64_t)b * p.H + h) * Sq + qt),
                              rows, 4, 4);
    sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (int)soff, 0, 0));
  };
  // With per-score mask loads the loop's fetch is unconditional.
  constexpr bool kFlat = KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL;
  // LDS byte offsets of this lane's reads (as in the dQ kernel): row reads
  // (query 32 qb + c, logical chunk 2 s + g) at (ra ^ 32 s) + 32 qb rows;
  // transposing reads (queries 8 hf + 4 g + (c % 16) / 4 + 16 ks, dims
  // 32 db + 16 ((c / 16) % 2) + 4 (c % 4) .. + 3) at (ta ^ 64 db ^ 32 hf)
  // + (16 ks + 8 hf) rows. Both carry the step's buffer bit.
  uint32_t rao = (uint32_t)dtile_off<D>(c, g);
  uint32_t tao =
      (uint32_t)(dtile_off<D>(4 * g + ((c & 15) >> 2), 2 * ((c >> 4) & 1) + ((c >> 1) & 1)) + 8 * (c & 1));
  // V copy (VL): the lane's key row, logical chunk 2 s + g at vra ^ 32 s; the
  // first step's barrier covers its loads.
  const uint32_t vra = rao + 32 * wave * D * 2;
  if constexpr (VL) {
    if (any) {
      const u32x4 vr = rows_desc(vbase + (int64_t)k0 * p.sv_s * 2, min(Sk - k0, kAttnBwdBk), p.sv_s * 2, D * 2);
      dma_tile_asm<D, kAttnBwdBk>(vr, dma_lane_off<D>(lane, swave, p.sv_s * 2), p.sv_s * 2, swave, lds_addr(vl));
    }
  }
  // Mask tile (MT): transposing read m hands the lane its key's values for
  // queries 8 m + 4 g + 0..3 of the step (registers 4 m .. 4 m + 3): the lane
  // addresses query 8 m + 4 g + (c % 16) / 4, keys 32 w + 16 ((c / 16) % 2)
  // + 4 (c % 4) .. + 3, at mao[m % 2] + 16 (m / 2) rows (dswz depends on
  // bits 0-3 of the row, which 16 rows leave).
  uint32_t mao[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    mao[hf] = (uint32_t)(dtile_off<kAttnBwdBk>(8 * hf + 4 * g + ((c & 15) >> 2),
                                               4 * wave + 2 * ((c >> 4) & 1) + ((c >> 1) & 1)) +
                         8 * (c & 1));

  if (any && qstart < Sq) {
    // One sequence of (query head, query tile) steps over the heads of the
    // group, so that the next step's fetch is a single code path.
    const int ntile = (Sq - qstart + BQ - 1) / BQ;
    const int nstep = ntile * (int)p.group;
    uint32_t h = hk * p.group, nh = h;
    int qt = qstart, nqt = qstart;
    fetch(h, qt, 0);
    for (int step = 0; step < nstep; ++step) {
      const int buf = step & 1;
      h = nh;
      qt = nqt;
      nqt = qt + BQ;
      if (nqt >= Sq) {
        nqt = qstart;
        ++nh;
      }
      const int64_t mbase = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h;
      {
        // This wavefront's loads of the step have landed; after the barrier
        // every wavefront's have, and every wavefront is done with the
        // previous step, whose buffers the next loads overwrite.
        __builtin_amdgcn_s_waitcnt(0);
        if (is_stat) (swave == 0 ? lses : dels)[buf][lane] = qt + lane < Sq ? sreg * smul : sfill;
        __syncthreads();
        const uint8_t* const ql = qd;
        const uint8_t* const dl_ = qd + TQ;
        const float* const lsb = lses[buf];
        const float* const deb = dels[buf];
        const uint32_t ra = rao, ta = tao;
        // This step's mask values of the lane's key, one per query (register
        // r: query qt + 8 (r / 4) + 4 g + r % 4), loaded before the prefetch
        // so that waiting for them leaves it in flight: 16-bit additive values
        // two to a register, boolean bytes four to a register.
        // (Each value in a register of its own until it is used: packing them
        // as they arrive made the compiler wait for each load in turn.)
        // The loads are unconditional, at a query and key clamped into the
        // mask (values of excluded scores are never used), so that the wait
        // for them is counted exactly instead of for every load in flight.
        uint32_t mvk[16];
        if constexpr (MT && KIND == ATTN_MASK_BOOL) {
          // One byte per query: query 8 (r / 4) + 4 g + r % 4, the lane's key
          // 32 w + c (chunk 2 w + c / 16, byte c % 16).
          const uint8_t* const mtb = mt + buf * TMQ;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            mvk[r] = mtb[dtile_off<64>(8 * (r >> 2) + 4 * g + (r & 3), 2 * wave + (c >> 4)) + (c & 15)];
        } else if constexpr (MT) {
          const uint8_t* const mtb = mt + buf * TMQ;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x2 t = lds_read_tr(mtb + mao[m & 1] + 16 * (m >> 1) * kAttnBwdBk * 2);
            mvk[4 * m + 0] = t.x & 0xffffu;
            mvk[4 * m + 1] = t.x >> 16;
            mvk[4 * m + 2] = t.y & 0xffffu;
            mvk[4 * m + 3] = t.y >> 16;
          }
        } else if constexpr (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) {
          const int kjc = min(kj, Sk - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qq = min(qt + 8 * (r >> 2) + 4 * g + (r & 3), Sq - 1);
            const int64_t at = mbase + (int64_t)qq * p.sm_q + kjc;
            if constexpr (KIND == ATTN_MASK_ADD)
              mvk[r] = *reinterpret_cast<const uint16_t*>(p.mask + at * 2);
            else
              mvk[r] = (uint8_t)p.mask[at];
          }
          __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the prefetch
        }
        if (kFlat) {
          // Branch-free: the last step fetches its own tile again.
          const bool more = step + 1 < nstep;
          fetch(more ? nh : h, more ? nqt : qt, buf ^ 1);
          __builtin_amdgcn_sched_barrier(0);  // keep the fetch ahead of the products
        } else if (step + 1 < nstep) {
          fetch(nh, nqt, buf ^ 1);
        }

        // The tile's 32-query blocks in turn (the block's products,
        // probabilities and gradient contributions before the next block's).
        // A block that no key of the workgroup can see (causal) is skipped.
#pragma unroll
        for (int qb = 0; qb < NSUB; ++qb) {
          const int qb0 = qt + 32 * qb;  // the block's first query
          if (NSUB > 1 && (qb0 >= Sq || (p.causal && k0 > qb0 + 31 + off))) continue;
          f32x16 sacc, dpacc;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[r] = 0.0f;
            dpacc[r] = 0.0f;
          }
          if constexpr (VL) {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
              const u32x4 a = *reinterpret_cast<const u32x4*>(ql + (ra ^ (32 * s)) + 32 * qb * D * 2);
              const u32x4 ad = *reinterpret_cast<const u32x4*>(dl_ + (ra ^ (32 * s)) + 32 * qb * D * 2);
              const u32x4 vv = *reinterpret_cast<const u32x4*>(vl + (vra ^ (32 * s)));
              sacc = mfma_32x32x16<BF16>(a, kf[s], sacc);
              dpacc = mfma_32x32x16<BF16>(ad, vv, dpacc);
            }
            // The Q, dO and V reads of a k-step two k-steps ahead of its products.
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
            for (int i = 0; i < D / 16 - 2; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          } else {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
              const u32x4 a = *reinterpret_cast<const u32x4*>(ql + (ra ^ (32 * s)) + 32 * qb * D * 2);
              sacc = mfma_32x32x16<BF16>(a, kf[s], sacc);
              if constexpr (kDK) {
                const u32x4 ad = *reinterpret_cast<const u32x4*>(dl_ + (ra ^ (32 * s)) + 32 * qb * D * 2);
                dpacc = mfma_32x32x16<BF16>(ad, vf[s], dpacc);
              }
            }
            // Q / dO reads four products ahead (1-2 % faster); not with
            // per-score masks, whose registers are short already.
            if constexpr (KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL)
              pin_reads_ahead<(kDK ? 2 : 1) * (D / 16), 4, 1>();
          }
          // Register r holds query qb0 + 8*(r/4) + 4g + r%4 of this lane's key.
          float pr[16], dsr[16];
          // A block whose every (query, key) score is visible (all queries and
          // keys in range, past the causal boundary, no per-score mask) takes
          // the probabilities without any exclusion test.
          const bool inb = k0 + kAttnBwdBk <= klen && (!p.causal || k0 + kAttnBwdBk - 1 <= qb0 + off);
          const bool full = KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL && qb0 + 32 <= Sq && inb;
          if (full) {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int qo = 32 * qb + 8 * rg + 4 * g;  // first of 4 consecutive queries
              const float4 l2 = *reinterpret_cast<const float4*>(&lsb[qo]);
              const float4 dl = *reinterpret_cast<const float4*>(&deb[qo]);
              const float lv[4] = {l2.x, l2.y, l2.z, l2.w}, dv4[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e;
                const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], p.scale_log2, -lv[e]));
                pr[r] = pv;
                dsr[r] = pv * (dpacc[r] - dv4[e]);
              }
            }
          } else if ((KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) && inb) {
            // Every key in bounds for every query: the mask alone (a query
            // past Sq or without any visible key has LSE -inf here).
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int qo = 32 * qb + 8 * rg + 4 * g;
              const float4 l2 = *reinterpret_cast<const float4*>(&lsb[qo]);
              const float4 dl = *reinterpret_cast<const float4*>(&deb[qo]);
              const float lv[4] = {l2.x, l2.y, l2.z, l2.w}, dv4[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e;
                float tv = sacc[r] * p.scale_log2;
                bool excluded = lv[e] == kNegInfA;
                if constexpr (KIND == ATTN_MASK_ADD) tv = fmaf(to_float<BF16>(mvk[r]), kLog2eA, tv);
                else if (mvk[r] != 0) excluded = true;
                const float pv = excluded ? 0.0f : __builtin_amdgcn_exp2f(tv - lv[e]);
                pr[r] = pv;
                dsr[r] = pv * (dpacc[r] - dv4[e]);
              }
            }
          } else {
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const int qo = 32 * qb + 8 * rg + 4 * g;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e, qq = qt + qo + e;
                const float lse2 = lsb[qo + e];
                float tv = sacc[r] * p.scale_log2;
                bool excluded = qq >= Sq || kj >= klen || !kvalid || lse2 == kNegInfA ||
                                (p.causal && kj > qq + off);
                if constexpr (KIND == ATTN_MASK_ADD) {
                  if (!excluded) tv = fmaf(to_float<BF16>(mvk[r]), kLog2eA, tv);
                } else if constexpr (KIND == ATTN_MASK_BOOL) {
                  if (!excluded && mvk[r] != 0) excluded = true;
                }
                const float pv = excluded ? 0.0f : __builtin_amdgcn_exp2f(tv - lse2);
                pr[r] = pv;
                dsr[r] = pv * (dpacc[r] - deb[qo + e]);
              }
            }
          }
          // B operands: k-step s takes registers 8s .. 8s+7 (queries
          // qb0 + 16s + 8*(j/4) + 4g + j%4 for element j).
          u32x4 pb[2], sb[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            pb[s] = u32x4{pack2<BF16>(pr[8 * s + 0], pr[8 * s + 1]), pack2<BF16>(pr[8 * s + 2], pr[8 * s + 3]),
                          pack2<BF16>(pr[8 * s + 4], pr[8 * s + 5]), pack2<BF16>(pr[8 * s + 6], pr[8 * s + 7])};
            sb[s] = u32x4{pack2<BF16>(dsr[8 * s + 0], dsr[8 * s + 1]), pack2<BF16>(dsr[8 * s + 2], dsr[8 * s + 3]),
                          pack2<BF16>(dsr[8 * s + 4], dsr[8 * s + 5]), pack2<BF16>(dsr[8 * s + 6], dsr[8 * s + 7])};
          }
          // A operands of k-step ks: queries 16 ks + 4 g + 0..3 (elements
          // 0-3) and 16 ks + 8 + 4 g + 0..3 (elements 4-7) of the lane's dim.
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int ks = 2 * qb + s;  // the k-step's 16 queries within the tile
              const uint32_t t0 = (ta ^ (64 * db)) + 16 * ks * D * 2;
              const uint32_t t1 = (ta ^ (64 * db) ^ 32) + (16 * ks + 8) * D * 2;
              if constexpr (kDV) {
                const u32x2 a0 = lds_read_tr(dl_ + t0), a1 = lds_read_tr(dl_ + t1);
                dv[db] = mfma_32x32x16<BF16>(u32x4{a0.x, a0.y, a1.x, a1.y}, pb[s], dv[db]);
              }
              if constexpr (kDK) {
                const u32x2 b0 = lds_read_tr(ql + t0), b1 = lds_read_tr(ql + t1);
                dk[db] = mfma_32x32x16<BF16>(u32x4{b0.x, b0.y, b1.x, b1.y}, sb[s], dk[db]);
              }
            }
          }
          // dO^T / Q^T reads two products ahead for D = 128, as in dQ.
          if constexpr (D == 128 && KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL)
            pin_reads_ahead<((kDV ? 1 : 0) + (kDK ? 1 : 0)) * 2 * (D / 32), 2, 2>();
        }
        rao ^= 2 * TQ;
        tao ^= 2 * TQ;
      }
    }
  }
  // The last step's loads into LDS (issued unconditionally with per-score
  // masks) complete before the workgroup, and its LDS, can end.
  __builtin_amdgcn_s_waitcnt(0);

  if (!kvalid) return;
  char* dkrow = p.dk + ((int64_t)b * p.sdk_b + (int64_t)hk * p.sdk_h + (int64_t)kj * p.sdk_s) * 2;
  char* dvrow = p.dv + ((int64_t)b * p.sdv_b + (int64_t)hk * p.sdv_h + (int64_t)kj * p.sdv_s) * 2;
  const float sc = p.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = db * 32 + 8 * rg + 4 * g;
      if constexpr (kDK) {
        const u32x2 wk{pack2<BF16>(dk[db][4 * rg] * sc, dk[db][4 * rg + 1] * sc),
                       pack2<BF16>(dk[db][4 * rg + 2] * sc, dk[db][4 * rg + 3] * sc)};
        *reinterpret_cast<u32x2*>(dkrow + d * 2) = wk;
      }
      if constexpr (kDV) {
        const u32x2 wv{pack2<BF16>(dv[db][4 * rg], dv[db][4 * rg + 1]),
                       pack2<BF16>(dv[db][4 * rg + 2], dv[db][4 * rg + 3])};
        *reinterpret_cast<u32x2*>(dvrow + d * 2) = wv;
      }
    }
}

// Entry points: the single passes (per-score masks, D = 128) at two
// wavefronts per SIMD, except the dV pass with additive mask tiles, which
// fits three (168 VGPRs, no spills; 3 % faster than two; with mask values
// from global memory, or the boolean tile's byte reads, they would spill
// there; without a mask, 149 VGPRs, 1-3 % faster); both gradients together
// with the registers the compiler needs (one wavefront per SIMD for D = 128;
// D = 64 fits two as it is).
template <int KIND, int PASS, bool MT>
constexpr int dkdv_waves() {
  return PASS == 0 && ((KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL) || (MT && KIND == ATTN_MASK_ADD)) ? 3 : 2;
}
template <bool BF16, int D, int KIND, int PASS, int BQ, bool MT>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(dkdv_waves<KIND, PASS, MT>(), dkdv_waves<KIND, PASS, MT>())))
attn_bwd_dkdv_kernel(AttnBwdParams p) {
  dkdv_body<BF16, D, KIND, PASS, BQ, MT, false>(p);
}
template <bool BF16, int D, int KIND, int BQ, bool MT>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_both_kernel(AttnBwdParams p) {
  dkdv_body<BF16, D, KIND, 2, BQ, MT, false>(p);
}
template <bool BF16, int KIND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_vl_kernel(AttnBwdParams p) {
  dkdv_body<BF16, 128, KIND, 2, 32, false, true>(p);
}

// Queries per dK/dV step. Two 32-query blocks per loaded tile halve the
// per-step work (barrier, LSE / delta) per product: measured 4 % faster for
// D = 64 (fp16 [8,32,2048,64] backward, register-staged tiles) and 2-4 % for
// the one-pass D = 128 kernel (fp16 [4,32,4096,128] backward, causal 2195
// against 2250 us). Per-score masks keep one block (their values take
// registers per block).
template <int KIND, int D>
constexpr int dkdv_bq() {
  return (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) ? 32 : 64;
}

// Workgroups from which D = 128 dK / dV run at two wavefronts per SIMD (two
// passes with a per-score mask, else one pass with the V copy): two per CU
// of the MI355X's 256.
constexpr uint32_t kTwoPassGrid = 512;

template <bool BF16, int D, int KIND, bool MT>
hipError_t launch_dkdv(const AttnBwdParams& p, hipStream_t st) {
  const dim3 block(256);
  const dim3 gk(p.Hk * p.B * ((p.Sk + kAttnBwdBk - 1) / kAttnBwdBk));
  // D = 128 on grids of two workgroups per CU or more: without a per-score
  // mask one pass with the V copy at two wavefronts per SIMD (fp16
  // [4,32,4096,128] backward: causal 2028 against 2225 us for one pass at
  // one wavefront and 2325 for two passes; not causal 3610 against 3795 and
  // 4070), with one the two passes (additive mask, causal: 2784 against
  // 2830-3000 for one pass at one wavefront). Smaller grids: one pass at one
  // wavefront per SIMD (bf16 [2,8,1000,128], 128 workgroups: 78 against 85
  // with the V copy and 103 for two passes; 107 against 131 with an
  // additive mask).
  constexpr int BQ = dkdv_bq<KIND, D>();
  constexpr bool kPerScore = KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL;
  if constexpr (D == 128 && !kPerScore) {
    if (gk.x >= kTwoPassGrid) {
      hipLaunchKernelGGL((attn_bwd_dkdv_vl_kernel<BF16, KIND>), gk, block, 0, st, p);
      return hipGetLastError();
    }
  }
  if constexpr (D == 128 && kPerScore) {
    if (gk.x >= kTwoPassGrid) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<BF16, D, KIND, 0, BQ, MT>), gk, block, 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<BF16, D, KIND, 1, BQ, MT>), gk, block, 0, st, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_bwd_dkdv_both_kernel<BF16, D, KIND, BQ, MT>), gk, block, 0, st, p);
  return hipGetLastError();
}

template <bool BF16, int D, int KIND>
hipError_t launch_bwd_kind(const AttnBwdParams& p, hipStream_t st) {
  const dim3 block(256);
  if (p.Sq > 0) {
    const dim3 gq(p.H * p.B * ((p.Sq + kAttnBq - 1) / kAttnBq));
    if constexpr (KIND == ATTN_MASK_ADD) {
      if (p.mask_tile) hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 2>), gq, block, 0, st, p);
      else if (p.mask_vec) hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 1>), gq, block, 0, st, p);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 0>), gq, block, 0, st, p);
    } else if constexpr (KIND == ATTN_MASK_BOOL) {
      if (p.mask_tile) hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 3>), gq, block, 0, st, p);
      else if (p.mask_vec) hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 1>), gq, block, 0, st, p);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 0>), gq, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, 0>), gq, block, 0, st, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Sk > 0) {
    if constexpr (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) {
      if (p.mask_tile) return launch_dkdv<BF16, D, KIND, true>(p, st);
    }
    return launch_dkdv<BF16, D, KIND, false>(p, st);
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_bwd(const AttnBwdParams& p, hipStream_t st) {
  switch (p.mask_kind) {
    case ATTN_MASK_NONE: return launch_bwd_kind<BF16, D, ATTN_MASK_NONE>(p, st);
    case ATTN_MASK_ADD: return launch_bwd_kind<BF16, D, ATTN_MASK_ADD>(p, st);
    case ATTN_MASK_BOOL: return launch_bwd_kind<BF16, D, ATTN_MASK_BOOL>(p, st);
    case ATTN_MASK_LEN: return launch_bwd_kind<BF16, D, ATTN_MASK_LEN>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace sms

hipError_t sms_attn_bwd_launch(const sms::AttnBwdParams* p, int dtype, int head_dim,
                               hipStream_t st) {
  if (dtype == 1 && head_dim == 64) return sms::launch_bwd<false, 64>(*p, st);
  if (dtype == 1 && head_dim == 128) return sms::launch_bwd<false, 128>(*p, st);
  if (dtype == 2 && head_dim == 64) return sms::launch_bwd<true, 64>(*p, st);
  if (dtype == 2 && head_dim == 128) return sms::launch_bwd<true, 128>(*p, st);
  return hipErrorInvalidValue;
}
