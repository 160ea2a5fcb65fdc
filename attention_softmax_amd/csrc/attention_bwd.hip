// attention_bwd.hip -- fused attention backward on the gfx950 matrix cores:
// dQ, dK, dV of L = sum(dO * O) for O = softmax(Q K^T * scale + mask) V,
// recomputing the probabilities from the forward's log-sum-exp instead of
// storing them (the FlashAttention-style scheme the pnsm.cn article's sec. 4.4
// points to; the softmax gradient itself is the lmnt.cn page's sec. 3.3 rule,
// dS = P * (dP - rowsum(dP * P)), with rowsum(dP * P) = rowsum(dO * O)).
//
// Two launches (three for D = 128, where dK and dV take a pass each), all
// deterministic (no atomics):
//  1. dQ, one workgroup per 128 queries (query-stationary, as the forward);
//     it first forms delta = rowsum(dO * O) of its queries in fp32 and stores
//     it in the workspace for step 2. S^T = K Q^T and dP^T = V dO^T leave
//     each lane 16 keys of one query;
//     P = exp(S*scale + mask - LSE); dS^T = P (dP^T - delta); dQ^T += K^T dS^T
//     with the dS registers as the B operand (keys contracted in the order the
//     S^T layout holds them, K^T read from a transposed LDS tile);
//  2. dK and dV, one workgroup per 128 keys of one key/value head
//     (key-stationary): for every query head of its group and every tile of
//     32 or 64 queries, S = Q K^T and dP = dO V^T leave each lane 16 queries
//     of one key per 32-query block; dV^T += dO^T P and dK^T += Q^T dS with P
//     and dS as B operands.
// Lane layouts of v_mfma_f32_32x32x16: see attention.hip.

#include "attention.hpp"

namespace sms {
namespace {

using namespace attn;

// ---------------------------------------------------------------- 1. dQ

template <bool BF16, int D, int KIND, bool MV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(AttnBwdParams p) {
  constexpr int BK = kAttnBk;
  constexpr int KP = D + 8;   // row-major tile pitch, elements
  constexpr int TP = BK + 4;  // transposed tile pitch, elements
  __shared__ __align__(16) uint16_t ks[BK * KP];   // K, row-major: A of S^T = K Q^T
  __shared__ __align__(16) uint16_t kts[D * TP];   // K^T: A of dQ^T += K^T dS^T
  __shared__ __align__(16) uint16_t vs[BK * KP];   // V, row-major: A of dP^T = V dO^T

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
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

  // Tiles fetched one ahead: K as (4 keys x 8 dims) per thread, staged
  // row-major and transposed; V as 16-byte chunks, staged row-major.
  constexpr int KITEMS = (BK / 4) * (D / 8);
  constexpr int KCH = D / 8;
  constexpr int VC = BK * KCH / 256;
  const int kdg = tid % (D / 8), kkg = tid / (D / 8);
  const bool kthread = tid < KITEMS;
  u32x4 kreg[4], vreg[VC];
  // The fetch reads through buffer ranges re-based on each tile that end at
  // the last key (rows past it read as zero), with fixed per-thread offsets
  // and no per-load test or branch; threads past the K items (D = 64) load a
  // copy of another thread's item, so that the wait for a tile's mask values
  // does not cover the fetch.
  uint32_t koff[4], voff[VC];
  const int ktid = tid % KITEMS, kdgl = ktid % (D / 8), kkgl = ktid / (D / 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) koff[i] = (uint32_t)((4 * kkgl + i) * p.sk_s * 2 + kdgl * 16);
#pragma unroll
  for (int i = 0; i < VC; ++i) {
    const int idx = tid + 256 * i, row = idx / KCH, ch = idx - row * KCH;
    voff[i] = (uint32_t)(row * p.sv_s * 2 + ch * 16);
  }
  auto fetch = [&](int kt) {
    const int rows = min(Sk - kt, BK);
    const auto kr = rows_rsrc(kbase + (int64_t)kt * p.sk_s * 2, rows, p.sk_s * 2, D * 2);
    const auto vr = rows_rsrc(vbase + (int64_t)kt * p.sv_s * 2, rows, p.sv_s * 2, D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) kreg[i] = rsrc_load(kr, koff[i]);
#pragma unroll
    for (int i = 0; i < VC; ++i) vreg[i] = rsrc_load(vr, voff[i]);
  };
  auto stage = [&]() {
    if (kthread) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&ks[(4 * kkg + i) * KP + 8 * kdg]) = kreg[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x2 w{pair(kreg[0], kreg[1], j), pair(kreg[2], kreg[3], j)};
        *reinterpret_cast<u32x2*>(&kts[(8 * kdg + j) * TP + tcol(8 * kdg + j, kkg)]) = w;
      }
    }
#pragma unroll
    for (int i = 0; i < VC; ++i) {
      const int idx = tid + 256 * i, row = idx / KCH, ch = idx - row * KCH;
      *reinterpret_cast<u32x4*>(&vs[row * KP + ch * 8]) = vreg[i];
    }
  };
  if (kend > 0) fetch(0);

  // This lane's K^T operand rows c, c + 32, ... (tcol's lane part included).
  const uint16_t* const klane = &kts[c * TP + tcol_lane(c, g)];
  for (int kt = 0; kt < kend; kt += BK) {
    __syncthreads();
    stage();
    __syncthreads();
    u32x2 mv[8];  // this tile's mask values, loaded before the prefetch
    if constexpr (MV) {
      load_mask_runs<KIND>(p.mask, mrow_c, kt, g, Sk, mv);
      __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the prefetch
    }
    if (MV || kt + BK < kend) fetch(kt + BK);
    if constexpr (MV) __builtin_amdgcn_sched_barrier(0);  // keep the fetch ahead of the products

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
        const u32x4 a = *reinterpret_cast<const u32x4*>(&ks[(kb * 32 + c) * KP + s * 16 + 8 * g]);
        sacc = mfma_32x32x16<BF16>(a, qf[s], sacc);
        const u32x4 av = *reinterpret_cast<const u32x4*>(&vs[(kb * 32 + c) * KP + s * 16 + 8 * g]);
        dpacc = mfma_32x32x16<BF16>(av, df[s], dpacc);
      }
      pin_reads_ahead<2 * (D / 16), 4, 1>();  // K / V reads four products ahead (1-2 % faster)
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[r], p.scale_log2, -lse2));
          sacc[r] = pv * (dpacc[r] - delta);
        }
      } else if ((KIND == ATTN_MASK_BOOL || (KIND == ATTN_MASK_ADD && !MV)) && inb) {
        // Every key in bounds for every query: the mask (and a query without
        // any visible key) alone. (Not for additive runs: the extra code path
        // made that variant spill.)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float tv = sacc[r] * p.scale_log2;
          bool excluded = !live;
          if constexpr (KIND == ATTN_MASK_ADD) {
            uint32_t bits;
            if constexpr (MV) {
              bits = mask_run_value(mv, kb, r, false);
            } else {
              const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              bits = live ? *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2) : 0u;
            }
            tv = fmaf(to_float<BF16>(bits), kLog2eA, tv);
          } else {
            uint32_t byte;
            if constexpr (MV) {
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
              if constexpr (MV) bits = mask_run_value(mv, kb, r, false);
              else bits = *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2);
              tv = fmaf(to_float<BF16>(bits), kLog2eA, tv);
            }
          } else if constexpr (KIND == ATTN_MASK_BOOL) {
            if (!excluded) {
              uint32_t byte;
              if constexpr (MV) byte = mask_run_value(mv, kb, r, true);
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
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* krow = klane + db * 32 * TP;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int s = 2 * kb + s2;
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(krow + tcol_const(db, 2 * s));
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(krow + tcol_const(db, 2 * s + 1));
          dq[db] = mfma_32x32x16<BF16>(u32x4{a0.x, a0.y, a1.x, a1.y}, pb[s2], dq[db]);
        }
      }
      // K^T reads two products ahead for D = 128 (backward 2 % faster; equal
      // or slower for D = 64).
      if constexpr (D == 128) pin_reads_ahead<2 * (D / 32), 2, 2>();
    }
  }

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
// registers (one wavefront per SIMD), so there PASS 0 (dV alone: S, P) and
// PASS 1 (dK alone: S, dP, dS) run as two launches, each at two wavefronts
// per SIMD, recomputing S in both.
template <bool BF16, int D, int KIND, int PASS, int BQ>
__device__ inline __attribute__((always_inline)) void dkdv_body(const AttnBwdParams& p) {
  constexpr bool kDV = PASS != 1, kDK = PASS != 0;
  static_assert(BQ == 32 || BQ == 64, "query tiles of one or two 32-query blocks");
  static_assert(BQ == 32 || (KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL),
                "per-score masks are loaded for one 32-query block per step");
  constexpr int NSUB = BQ / 32;
  constexpr int RP = D + 8;   // row-major tile pitch, elements
  constexpr int TP = BQ + 4;  // transposed tile pitch, elements (BQ / 2 + 2 dwords)
  __shared__ __align__(16) uint16_t qs[BQ * RP];    // Q: A of S = Q K^T
  __shared__ __align__(16) uint16_t qts[D * TP];    // Q^T: A of dK^T += Q^T dS
  __shared__ __align__(16) uint16_t dos[BQ * RP];   // dO: A of dP = dO V^T
  __shared__ __align__(16) uint16_t dots[D * TP];   // dO^T: A of dV^T += dO^T P
  __shared__ __align__(16) float lses[BQ];  // LSE * log2(e) of the tile's queries
  __shared__ __align__(16) float dels[BQ];

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
      if constexpr (kDK)
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

  // Tiles of BQ queries fetched one ahead as items of (4 queries x 8 dims):
  // the QITEMS items of Q, then those of dO, dealt to the threads in order
  // (item tid + 256 i is thread tid's i-th), staged row-major and
  // transposed; LSE by the first BQ lanes of wavefront 0 and delta by those
  // of wavefront 1. Every choice of source is uniform over a wavefront and
  // made once here: a per-lane choice between kernel-argument fields inside
  // the loop made the compiler fetch the fields with vector loads and wait
  // for every outstanding load, prefetch included.
  constexpr int QITEMS = (BQ / 4) * (D / 8);  // 64, 128 or 256: whole wavefronts
  constexpr int NITEMS = 2 * QITEMS;
  constexpr int NIT = (NITEMS + 255) / 256;    // items per thread
  static_assert(QITEMS % 64 == 0, "Q / dO loads by whole wavefronts");
  // This lane's Q^T and dO^T operand rows c, c + 32, ... (tcol's lane part included).
  const uint16_t* const qlane = &qts[c * TP + tcol_lane(c, g)];
  const uint16_t* const dolane = &dots[c * TP + tcol_lane(c, g)];
  const bool is_stat = wave < 2 && lane < BQ;  // LSE (wavefront 0) or delta (wavefront 1)
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  float* const sdst = swave == 0 ? lses : dels;
  const float sfill = swave == 0 ? kNegInfA : 0.0f;
  const float smul = swave == 0 ? kLog2eA : 1.0f;  // LSE is staged in log2 units
  u32x4 treg[NIT][4];
  float sreg = 0.0f;
  // The fetch reads through buffer ranges re-based on each step (scalar
  // registers) that end at the last query (rows past it read as zero; the
  // stage fills LSE / delta there), with fixed per-thread offsets. Every
  // thread loads: threads past the last item load a copy of another's, and
  // wavefronts past the LSE / delta lanes a copy of the LSE, so that no branch
  // makes the wait for a step's mask values cover the fetch.
  const char* fsrc[NIT];
  int64_t fs_h[NIT], fs_s[NIT];
  bool fstage[NIT], fdo[NIT];
  int fqdg[NIT], fqqg[NIT];
  uint32_t toff[NIT][4];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int it = (tid + 256 * i) % NITEMS;
    fstage[i] = tid + 256 * i < NITEMS;
    fdo[i] = __builtin_amdgcn_readfirstlane(it / QITEMS) == 1;
    const int local = it % QITEMS;
    fqdg[i] = local % (D / 8);
    fqqg[i] = local / (D / 8);
    fsrc[i] = fdo[i] ? p.dout + (int64_t)b * p.sdo_b * 2 : p.q + (int64_t)b * p.sq_b * 2;
    fs_h[i] = fdo[i] ? p.sdo_h : p.sq_h;
    fs_s[i] = fdo[i] ? p.sdo_s : p.sq_s;
#pragma unroll
    for (int k = 0; k < 4; ++k) toff[i][k] = (uint32_t)((4 * fqqg[i] + k) * fs_s[i] * 2 + fqdg[i] * 16);
  }
  const float* fssrc = swave == 1 ? p.delta : p.lse;
  const uint32_t soff = (uint32_t)(lane & (BQ - 1)) * 4;
  // With per-score mask loads the loop's fetch is unconditional too.
  constexpr bool kFlat = KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL;
  int sq_staged = 0;  // first query of the staged tile (the fill of LSE / delta past Sq)
  auto fetch = [&](uint32_t h, int qt) {
    const int rows = min(Sq - qt, BQ);
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const auto tr = rows_rsrc(fsrc[i] + ((int64_t)h * fs_h[i] + (int64_t)qt * fs_s[i]) * 2, rows,
                                fs_s[i] * 2, D * 2);
#pragma unroll
      for (int k = 0; k < 4; ++k) treg[i][k] = rsrc_load(tr, toff[i][k]);
    }
    const auto sr = rows_rsrc(reinterpret_cast<const char*>(fssrc + ((int64_t)b * p.H + h) * Sq + qt),
                              rows, 4, 4);
    sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (int)soff, 0, 0));
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      if (!fstage[i]) continue;
      uint16_t* const srm = fdo[i] ? dos : qs;
      uint16_t* const stp = fdo[i] ? dots : qts;
      const int qdg = fqdg[i], qqg = fqqg[i];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<u32x4*>(&srm[(4 * qqg + k) * RP + 8 * qdg]) = treg[i][k];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x2 w{pair(treg[i][0], treg[i][1], j), pair(treg[i][2], treg[i][3], j)};
        *reinterpret_cast<u32x2*>(&stp[(8 * qdg + j) * TP + tcol(8 * qdg + j, qqg)]) = w;
      }
    }
    // (LSE scaled to log2 units here, not as it arrives: an operation on the
    // loaded value in the fetch would wait for it, and with it for the tile.)
    if (is_stat) sdst[lane] = sq_staged + lane < Sq ? sreg * smul : sfill;
  };

  if (any && qstart < Sq) {
    // One sequence of (query head, query tile) steps over the heads of the
    // group, so that the next step's fetch is a single code path.
    const int ntile = (Sq - qstart + BQ - 1) / BQ;
    const int nstep = ntile * (int)p.group;
    uint32_t h = hk * p.group, nh = h;
    int qt = qstart, nqt = qstart;
    fetch(h, qt);
    for (int step = 0; step < nstep; ++step) {
      h = nh;
      qt = nqt;
      nqt = qt + BQ;
      if (nqt >= Sq) {
        nqt = qstart;
        ++nh;
      }
      const int64_t mbase = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h;
      {
        __syncthreads();
        sq_staged = qt;
        stage();
        __syncthreads();
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
        if constexpr (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) {
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
          fetch(more ? nh : h, more ? nqt : qt);
          __builtin_amdgcn_sched_barrier(0);  // keep the fetch ahead of the products
        } else if (step + 1 < nstep) {
          fetch(nh, nqt);
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
#pragma unroll
          for (int s = 0; s < D / 16; ++s) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(&qs[(32 * qb + c) * RP + s * 16 + 8 * g]);
            sacc = mfma_32x32x16<BF16>(a, kf[s], sacc);
            if constexpr (kDK) {
              const u32x4 ad = *reinterpret_cast<const u32x4*>(&dos[(32 * qb + c) * RP + s * 16 + 8 * g]);
              dpacc = mfma_32x32x16<BF16>(ad, vf[s], dpacc);
            }
          }
          // Q / dO reads four products ahead (1-2 % faster); not with per-score
          // masks, whose registers are short already.
          if constexpr (KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL)
            pin_reads_ahead<(kDK ? 2 : 1) * (D / 16), 4, 1>();
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
              const int ql = 32 * qb + 8 * rg + 4 * g;  // first of 4 consecutive queries
              const float4 l2 = *reinterpret_cast<const float4*>(&lses[ql]);
              const float4 dl = *reinterpret_cast<const float4*>(&dels[ql]);
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
              const int ql = 32 * qb + 8 * rg + 4 * g;
              const float4 l2 = *reinterpret_cast<const float4*>(&lses[ql]);
              const float4 dl = *reinterpret_cast<const float4*>(&dels[ql]);
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
              const int ql = 32 * qb + 8 * rg + 4 * g;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e, qq = qt + ql + e;
                const float lse2 = lses[ql + e];
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
                dsr[r] = pv * (dpacc[r] - dels[ql + e]);
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
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const uint16_t* dorow = dolane + db * 32 * TP;
            const uint16_t* qrow = qlane + db * 32 * TP;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const int ks = 2 * qb + s;  // the k-step's 16 queries within the tile
              if constexpr (kDV) {
                const u32x2 a0 = *reinterpret_cast<const u32x2*>(dorow + tcol_const(db, 2 * ks));
                const u32x2 a1 = *reinterpret_cast<const u32x2*>(dorow + tcol_const(db, 2 * ks + 1));
                dv[db] = mfma_32x32x16<BF16>(u32x4{a0.x, a0.y, a1.x, a1.y}, pb[s], dv[db]);
              }
              if constexpr (kDK) {
                const u32x2 b0 = *reinterpret_cast<const u32x2*>(qrow + tcol_const(db, 2 * ks));
                const u32x2 b1 = *reinterpret_cast<const u32x2*>(qrow + tcol_const(db, 2 * ks + 1));
                dk[db] = mfma_32x32x16<BF16>(u32x4{b0.x, b0.y, b1.x, b1.y}, sb[s], dk[db]);
              }
            }
          }
          // dO^T / Q^T reads two products ahead for D = 128, as in dQ.
          if constexpr (D == 128 && KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL)
            pin_reads_ahead<((kDV ? 1 : 0) + (kDK ? 1 : 0)) * 2 * (D / 32), 2, 2>();
        }
      }
    }
  }

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

// Entry points: the single passes at two wavefronts per SIMD, except the dV
// pass without a per-score mask, which fits three (167 VGPRs, no spills; 1-3 %
// faster than two; with a mask its values would spill there); both gradients
// together with the registers the compiler needs (D = 64 fits two wavefronts
// per SIMD as it is).
template <int KIND, int PASS>
constexpr int dkdv_waves() {
  return PASS == 0 && KIND != ATTN_MASK_ADD && KIND != ATTN_MASK_BOOL ? 3 : 2;
}
template <bool BF16, int D, int KIND, int PASS, int BQ>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(dkdv_waves<KIND, PASS>(), dkdv_waves<KIND, PASS>())))
attn_bwd_dkdv_kernel(AttnBwdParams p) {
  dkdv_body<BF16, D, KIND, PASS, BQ>(p);
}
template <bool BF16, int D, int KIND, int BQ>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_both_kernel(AttnBwdParams p) {
  dkdv_body<BF16, D, KIND, 2, BQ>(p);
}

// Queries per dK/dV step. Two 32-query blocks per staged tile halve the
// per-step work (barriers, staging, LSE / delta) per product: measured 4 %
// faster for D = 64 (fp16 [8,32,2048,64] backward), equal within noise for
// D = 128, where one block keeps the LDS and registers smaller. Per-score
// masks keep one block (their values take registers per block).
template <int KIND, int D>
constexpr int dkdv_bq() {
  return (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL || D == 128) ? 32 : 64;
}

template <bool BF16, int D, int KIND>
hipError_t launch_bwd_kind(const AttnBwdParams& p, hipStream_t st) {
  const dim3 block(256);
  if (p.Sq > 0) {
    const dim3 gq(p.H * p.B * ((p.Sq + kAttnBq - 1) / kAttnBq));
    if constexpr (KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL) {
      if (p.mask_vec) hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, true>), gq, block, 0, st, p);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, false>), gq, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_kernel<BF16, D, KIND, false>), gq, block, 0, st, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.Sk > 0) {
    const dim3 gk(p.Hk * p.B * ((p.Sk + kAttnBwdBk - 1) / kAttnBwdBk));
    // D = 128: two passes at two wavefronts per SIMD, measured faster than
    // both gradients in one pass at one (fp16 [4,32,4096,128] causal
    // backward 4.72 against 5.28 ms; not causal 6.02 against 6.66 ms).
    constexpr int BQ = dkdv_bq<KIND, D>();
    if constexpr (D == 128) {
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<BF16, D, KIND, 0, BQ>), gk, block, 0, st, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<BF16, D, KIND, 1, BQ>), gk, block, 0, st, p);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkdv_both_kernel<BF16, D, KIND, BQ>), gk, block, 0, st, p);
    }
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
