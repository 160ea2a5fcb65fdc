// attention.hip -- fused attention forward on the gfx950 matrix cores:
//
//     O = softmax(Q K^T * scale + mask) V,   LSE = log sum_k exp(score_k)
//
// per query row, without the score tensor ever reaching memory (the QK^T
// fusion of the pnsm.cn ScaledMaskSoftmax article, sec. 4.4), with the online
// softmax of the 0539edu.com notes' fused-attention section: a running row
// maximum and sum, and the output rescaled by exp(m_old - m_new) whenever the
// maximum grows.
//
// Workgroup: 4 wavefronts x 32 queries = 128 queries of one (batch, head).
// Keys arrive in tiles of 64, loaded from global memory straight into
// double-buffered LDS. Per tile a wavefront computes S^T = K Q^T (keys x
// queries) with
// v_mfma_f32_32x32x16_{f16,bf16}, so each lane holds 16 keys of one query:
// the row maximum and sum are mostly in-lane plus one swap with the lane 32
// away (which holds the other 16 keys of the same query). The probabilities
// are then, register for register, the B operand of O^T += V^T P^T (the
// contraction over keys in an order that matches the S^T output layout; the
// A operand reads the matching keys of V), so P never leaves registers.
//
// MFMA 32x32x16 lane layout (probed on MI355X): A (32x16): lane l holds row
// l%32, k = 8*(l/32)..+7; B (16x32): lane l holds column l%32, same k; D
// (32x32): lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4 in its
// registers r = 0..15.

#include "attention.hpp"

namespace sms {
namespace {

using namespace attn;

// K and V come from global memory straight into LDS: tiles of 64 keys x D
// values in the dswz layout, double-buffered, so that each tile starts with
// one barrier, after which the loads of the next tile go out into the other
// buffer and stay in flight during this tile's products; the data never
// passes through registers. K is read by rows (16 bytes per lane) for
// S^T = K Q^T; V stays row-major (keys x dims) and the A operand of
// O^T += V^T P^T is assembled by transposing LDS reads (lds_read_tr: a lane
// group addressing 4 keys x 16 dims hands every lane its own dim's 4
// consecutive keys). The buffers are separate LDS objects and the tiles go
// in pairs, so that every read has a fixed buffer and the read offsets are
// loop-invariant registers plus immediates. Without a per-score mask, and
// with mask tiles (MV 2 and 3, below), the loads are issued from inline assembly
// (dma_one), which the compiler does not see (the kernel waits for them
// itself before each barrier), one after each k-step of the tile's S
// products instead of all together after the barrier: 2 % faster without a
// mask (fp16 [4,32,4096,128] causal: 618 against 631 us), 4-6 % with an
// additive [B,Sq,Sk] mask (723 against 752, 1267 against 1343 not causal).
// Otherwise they are the compiler-visible builtin loads, issued together;
// since they fill the other buffer object, the compiler knows that the reads
// do not touch it and inserts no wait for them.
//
// Per-score masks (additive / boolean), MV: 2 / 3 (additive / boolean masks
// whose rows start on 16-byte lines): the tile's mask values for the
// workgroup's 128 queries (a 128 x 64 tile of 128-byte rows, the dswz layout
// of D = 64, or of 64-byte rows, that of D = 32) come into one LDS buffer by
// loads of the same kind; each lane reads its runs of 4 keys from it at the
// start of the tile, and after a second barrier in the middle of the tile
// (all runs read) the next tile's mask values go out into it (boolean tiles
// against runs from global memory: 13-25 % faster); 1 (mask rows on 4
// elements and Sk % 4 == 0): the runs are loaded from
// global memory one tile ahead (load_mask_runs), before the next tile's K and
// V, so that they have landed by the barrier that starts their tile; 0: each
// mask value is read where it is used, and the next tile's loads go out after
// those reads, so that waiting for them does not wait for the loads.

// Wavefronts per SIMD: three for D = 64 (at most 168 VGPRs: 4-7 % faster
// than two on fp16 [8,32,2048,64] and [4,32,4096,64]), except with additive
// mask runs, which spill there; two for D = 128.
template <int D, int KIND, int MV>
constexpr int fwd_waves() {
  return D == 64 && !(KIND == ATTN_MASK_ADD && MV == 1) ? 3 : 2;
}

template <bool BF16, int D, int KIND, int MV>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(fwd_waves<D, KIND, MV>(), fwd_waves<D, KIND, MV>())))
attn_fwd_kernel(AttnParams p) {
  constexpr bool MASKED = KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL;
  // Without a per-score mask, and with mask tiles, the K / V loads are
  // issued from inline assembly, spread over the tile's S products (below).
  constexpr bool kSpread = !MASKED || MV >= 2;
  static_assert(MV == 0 || MASKED, "mask runs need a per-score mask");
  static_assert(MV != 2 || KIND == ATTN_MASK_ADD, "mask tiles of 16-bit values");
  static_assert(MV != 3 || KIND == ATTN_MASK_BOOL, "mask tiles of bytes");
  constexpr int BK = kAttnBk;
  constexpr int TB = BK * D * 2;  // bytes per tile
  constexpr int TM = kAttnBq * BK * (MV == 3 ? 1 : 2);  // bytes per mask tile (MV >= 2)
  __shared__ __align__(1024) uint8_t ks0[TB];
  __shared__ __align__(1024) uint8_t ks1[TB];
  __shared__ __align__(1024) uint8_t vs0[TB];
  __shared__ __align__(1024) uint8_t vs1[TB];
  __shared__ __align__(1024) uint8_t ms[MV >= 2 ? TM : 16];

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // One-dimensional grid of (query tile, head, batch) triples, in dispatch
  // order. With a causal rule: every head's last (longest) query tile first,
  // then the next-to-last, ..., which balances the uneven tiles. Without one:
  // the query tiles of one head before the next head, and since workgroups are
  // dealt round-robin over the 8 XCDs (each with its own L2; workgroup x runs
  // on XCD x % 8), x is remapped to t = (x % 8) * (N / 8) + x / 8 so that each
  // XCD takes a contiguous range of t and a head's K and V stay in one L2.
  // (The remap measured slower under a causal rule, where the longest-first
  // order matters more.)
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
  const char* qbase = p.q + ((int64_t)b * p.sq_b + (int64_t)h * p.sq_h) * 2;
  const char* kbase = p.k + ((int64_t)b * p.sk_b + (int64_t)hk * p.sk_h) * 2;
  const char* vbase = p.v + ((int64_t)b * p.sv_b + (int64_t)hk * p.sv_h) * 2;

  // Keys the workgroup visits ([0, kend)) and this lane's query sees ([0, kq)).
  const int off = p.causal == 2 ? Sk - Sq : 0;
  int klen = Sk;
  if constexpr (KIND == ATTN_MASK_LEN)
    klen = max(min(reinterpret_cast<const int32_t*>(p.mask)[b], Sk), 0);
  int kend = klen;
  if (p.causal) kend = min(kend, max(q0 + kAttnBq + off, 0));
  int kq = klen;
  if (p.causal) kq = min(kq, max(qi + off + 1, 0));
  const bool qvalid = qi < Sq;
  // Tiles may skip the per-score tests (see the loops) without a per-score
  // mask and with a positive scale. Queries past Sq need no test: their rows
  // are finite (Q = 0) and never stored.
  const bool fast_ok = !MASKED && p.scale_log2 > 0.0f;
  const int64_t mrow = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)qi * p.sm_q;
  // The same for a query clamped into the mask (unconditional vector loads).
  const int64_t mrow_c =
      (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)min(qi, Sq - 1) * p.sm_q;

  // Q fragment: the B operand of S^T = K Q^T (query qi, dims ks*16 + 8g .. +7).
  u32x4 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = u32x4{0, 0, 0, 0};
    if (qvalid)
      qf[s] = *reinterpret_cast<const u32x4*>(qbase + ((int64_t)qi * p.sq_s + s * 16 + 8 * g) * 2);
  }

  float m_i = kNegInfA, l_i = 0.0f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

  // Tile loads (rows past the last key read as zero).
  const uint32_t kdo = dma_lane_off<D>(lane, wave_u, p.sk_s * 2);
  const uint32_t vdo = dma_lane_off<D>(lane, wave_u, p.sv_s * 2);
  auto dma = [&](int kt, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const int rows = min(Sk - kt, BK);
    const auto kr = rows_rsrc(kbase + (int64_t)kt * p.sk_s * 2, rows, p.sk_s * 2, D * 2);
    const auto vr = rows_rsrc(vbase + (int64_t)kt * p.sv_s * 2, rows, p.sv_s * 2, D * 2);
    dma_tile<D, BK>(kr, kdo, p.sk_s * 2, wave_u, BUF ? ks1 : ks0);
    dma_tile<D, BK>(vr, vdo, p.sv_s * 2, wave_u, BUF ? vs1 : vs0);
  };
  // Descriptors of tile kt's K and V rows for the inline-assembly loads
  // (kSpread); past kend none (the loads then write zeros into a buffer that
  // no tile reads again).
  auto tile_desc = [&](int kt, u32x4& kr, u32x4& vr) {
    const int rows = kt < kend ? min(Sk - kt, BK) : 0;
    kr = rows_desc(kbase + (int64_t)kt * p.sk_s * 2, rows, p.sk_s * 2, D * 2);
    vr = rows_desc(vbase + (int64_t)kt * p.sv_s * 2, rows, p.sv_s * 2, D * 2);
  };
  // Mask tiles (MV >= 2): the workgroup's query rows (past Sq: none, or the
  // one broadcast row) through one buffer range ending at the last row's last
  // key; keys past Sk of the other rows read the next row's first values,
  // whose scores are excluded. Rows of 64 values: 128 bytes (additive, the
  // dswz layout of D = 64) or 64 (boolean, that of D = 32).
  constexpr int MB = MV == 3 ? 1 : 2;  // bytes per mask value
  constexpr int MD = 32 * MB;          // the tile's dswz layout
  const int64_t mtile = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)q0 * p.sm_q;
  const int mrows = min(Sq - q0, kAttnBq);
  const uint32_t mdo = dma_lane_off<MD>(lane, wave_u, p.sm_q * MB);
  auto dma_mask = [&](int kt) {
    const int rows = min(Sk - kt, BK);
    u32x4 mr = rows_desc(p.mask + (mtile + kt) * MB, rows > 0 ? mrows : 0, p.sm_q * MB, max(rows, 0) * MB);
    // (Uniform words, which the compiler kept in vector registers here; the
    // inline assembly takes them in scalar registers.)
#pragma unroll
    for (int j = 0; j < 4; ++j) mr[j] = __builtin_amdgcn_readfirstlane(mr[j]);
    dma_tile_asm<MD, kAttnBq>(mr, mdo, p.sm_q * MB, wave_u, lds_addr(ms));
  };
  if (kend > 0) {
    if constexpr (kSpread) {
      u32x4 kr, vr;
      tile_desc(0, kr, vr);
      dma_tile_asm<D, BK>(kr, kdo, p.sk_s * 2, wave_u, lds_addr(ks0));
      dma_tile_asm<D, BK>(vr, vdo, p.sv_s * 2, wave_u, lds_addr(vs0));
    } else {
      dma(0, BoolC<false>{});
    }
    if constexpr (MV >= 2) dma_mask(0);
  }
  u32x2 mv[8], mv_next[8];  // mask runs of this tile and (MV == 1) of the next
  if constexpr (MV == 1) load_mask_runs<KIND>(p.mask, mrow_c, 0, g, Sk, mv);

  // LDS byte offsets of this lane's operand reads. K: row c (+ 32 kb), logical
  // chunk 2 s + g. V (transposing reads): keys 8 hf + 4 g + (c % 16) / 4
  // (+ 16 s), dims 32 db + 16 ((c / 16) % 2) + 4 (c % 4) .. + 3.
  uint32_t kao[D / 16], vao[D / 32][2];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kao[s] = (uint32_t)dtile_off<D>(c, 2 * s + g);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 8 * hf + 4 * g + ((c & 15) >> 2);
      const int col = 32 * db + 16 * ((c >> 4) & 1) + 4 * (c & 3);
      vao[db][hf] = (uint32_t)(dtile_off<D>(row, col >> 3) + (col & 7) * 2);
    }

  // One key tile. FULL tiles have every score visible to every query of the
  // workgroup (see below); the loop over them is compiled apart from the loop
  // over the other tiles, so that neither carries the other's branches (with
  // both in one body the compiler copied the 32 score registers between the
  // products and the softmax of every tile).
  auto tile = [&](const int kt, auto full_c, auto buf_c) {
    constexpr bool FULL = decltype(full_c)::value;
    constexpr int BUF = decltype(buf_c)::value;
    const uint8_t* kt_lds = BUF ? ks1 : ks0;
    const uint8_t* vt_lds = BUF ? vs1 : vs0;
    // This wavefront's loads of the tile have landed; after the barrier every
    // wavefront's have, and every wavefront is done with the previous tile,
    // whose buffers the next tile's loads overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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
      // (Runs past the last key read at the row's last run: never used.)
      load_mask_runs<KIND>(p.mask, mrow_c, kt + BK, g, Sk, mv_next);
      if (kt + BK < kend) dma(kt + BK, BoolC<BUF == 0>{});
    }
    // A wavefront whose queries all precede the tile's first key (causal)
    // sees none of its scores: it only issues its share of the next tile's
    // loads (without a per-score mask, which has no barrier inside the tile).
    // 1-3 % faster causal forwards.
    if constexpr (!FULL && !MASKED) {
      if (p.causal && kt > q0 + 32 * wave_u + 31 + off) {
        if (kt + BK < kend) {
          u32x4 kr, vr;
          tile_desc(kt + BK, kr, vr);
          dma_tile_asm<D, BK>(kr, kdo, p.sk_s * 2, wave_u, lds_addr(BUF ? ks0 : ks1));
          dma_tile_asm<D, BK>(vr, vdo, p.sv_s * 2, wave_u, lds_addr(BUF ? vs0 : vs1));
        }
        return;
      }
    }

    // S^T for the tile's two 32-key blocks, alternating between the blocks so
    // that consecutive products are independent (each K fragment's LDS read
    // then has a product's time to arrive).
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
    if constexpr (kSpread) {
      // The next tile's loads, one after each k-step (K and V in turn), in
      // source order with the K fragments read five k-steps ahead: the loads
      // are inline assembly with a memory clobber, which no LDS read crosses,
      // and a scheduling barrier after each keeps the products between them.
      constexpr int NS = D / 16, AH = NS < 5 ? NS : 5;
      static_assert(NS == 2 * dma_loads<D, BK>(), "one K or V load per k-step");
      u32x4 kr, vr;
      tile_desc(kt + BK, kr, vr);
      const uint32_t kn = lds_addr(BUF ? ks0 : ks1), vn = lds_addr(BUF ? vs0 : vs1);
      u32x4 ka[NS][2];
#pragma unroll
      for (int s = 0; s < AH; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[s][kb] = *reinterpret_cast<const u32x4*>(kt_lds + kao[s] + kb * 32 * D * 2);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma_32x32x16<BF16>(ka[s][kb], qf[s], sacc[kb]);
        if (s + AH < NS) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ka[s + AH][kb] = *reinterpret_cast<const u32x4*>(kt_lds + kao[s + AH] + kb * 32 * D * 2);
        }
        if ((s & 1) == 0) dma_one<D>(kr, kdo, p.sk_s * 2, wave_u, kn, s >> 1);
        else dma_one<D>(vr, vdo, p.sv_s * 2, wave_u, vn, s >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + kao[s] + kb * 32 * D * 2);
          sacc[kb] = mfma_32x32x16<BF16>(a, qf[s], sacc[kb]);
        }
    }
    // With mask values read one by one: K reads ten products ahead (2-5 %
    // faster than the scheduler's own order, measured before the spread loads
    // above; not with mask runs, whose loads share the region).
    if constexpr (MV == 0 && MASKED) pin_reads_ahead<2 * (D / 16), 10, 1>();
    if constexpr (MV >= 2) {
      // Every wavefront has its runs (LDS reads complete, then the barrier:
      // a plain one, which unlike __syncthreads does not wait for the K / V
      // loads in flight); the next tile's mask values may overwrite them.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("s_barrier" ::: "memory");
      if (kt + BK < kend) dma_mask(kt + BK);
    }

    // Scores in the log2 domain, the mask and the key bounds. A tile whose
    // every score is visible to every query of the workgroup (keys in range
    // and, with a causal rule, before the first query's bound; no per-score
    // mask) skips the exclusion tests, and with a positive scale it takes the
    // maximum of the raw scores (scaling is monotonic, so the scaled maximum
    // is the same rounded value) and folds the scale into the exponential's
    // argument below. With a per-score mask, a tile with every key in bounds
    // for every query applies the mask alone.
    const bool inb = FULL || (kt + BK <= klen && (!p.causal || kt + BK <= q0 + off + 1));
    float mloc = kNegInfA;
    if constexpr (FULL) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
      mloc *= p.scale_log2;
    } else if (MASKED && inb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = sacc[kb][r] * p.scale_log2;
          if constexpr (KIND == ATTN_MASK_ADD) {
            uint32_t bits;
            if constexpr (MV != 0) {
              bits = mask_run_value(mv, kb, r, false);
            } else {
              const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              bits = qvalid ? *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2) : 0u;
            }
            t = fmaf(to_float<BF16>(bits), kLog2eA, t);
          } else {
            uint32_t byte;
            if constexpr (MV != 0) {
              byte = mask_run_value(mv, kb, r, true);
            } else {
              const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
              byte = qvalid ? (uint32_t)(uint8_t)p.mask[mrow + key] : 0u;
            }
            if (byte != 0) t = kNegInfA;
          }
          sacc[kb][r] = t;
          mloc = fmaxf(mloc, t);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          float t = sacc[kb][r] * p.scale_log2;
          if (key >= kq || key >= Sk) {
            t = kNegInfA;
          } else if constexpr (KIND == ATTN_MASK_ADD) {
            uint32_t bits;
            if constexpr (MV != 0) bits = mask_run_value(mv, kb, r, false);
            else bits = qvalid ? *reinterpret_cast<const uint16_t*>(p.mask + (mrow + key) * 2) : 0u;
            t = fmaf(to_float<BF16>(bits), kLog2eA, t);
          } else if constexpr (KIND == ATTN_MASK_BOOL) {
            uint32_t byte;
            if constexpr (MV != 0) byte = mask_run_value(mv, kb, r, true);
            else byte = qvalid ? (uint32_t)(uint8_t)p.mask[mrow + key] : 0u;
            if (byte != 0) t = kNegInfA;
          }
          sacc[kb][r] = t;
          mloc = fmaxf(mloc, t);
        }
      }
    }
    // Mask values read one by one: the next tile's loads go out after them,
    // so that waiting for them does not wait for the loads.
    if constexpr (MV == 0 && MASKED) {
      if (kt + BK < kend) dma(kt + BK, BoolC<BUF == 0>{});
    }
    mloc = other_half_max(mloc);
    // The reference maximum m_i moves only when a score exceeds it by more
    // than kLazy (log2 units): probabilities then stay below 2^kLazy, far
    // inside fp16 / bf16 range, and the running output and sum are rescaled
    // only on those tiles -- and skipped by the whole wavefront when none of
    // its queries needs it.
    const bool grow = mloc > m_i + kLazy || (m_i == kNegInfA && mloc != kNegInfA);
    float corr = 1.0f;
    if (grow) {
      corr = __builtin_amdgcn_exp2f(m_i - mloc);  // 0 from the first visible key on
      m_i = mloc;
      l_i *= corr;
    }
    const float m_use = (m_i == kNegInfA) ? 0.0f : m_i;  // nothing visible yet
    float psum = 0.0f;
    if constexpr (FULL) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.scale_log2, -m_use));
          sacc[kb][r] = pv;
          psum += pv;
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
          sacc[kb][r] = pv;
          psum += pv;
        }
    }
    l_i += psum;
    const bool rescale = __builtin_amdgcn_ballot_w64(grow) != 0;
    // P as the B operand of O^T += V^T P^T: k-step s takes registers
    // 8*(s%2) .. +7 of block s/2 (keys 16s + 8*(j/4) + 4g + j%4 for element j).
    u32x4 pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kb = s >> 1, base = 8 * (s & 1);
      pb[s] = u32x4{pack2<BF16>(sacc[kb][base + 0], sacc[kb][base + 1]),
                    pack2<BF16>(sacc[kb][base + 2], sacc[kb][base + 3]),
                    pack2<BF16>(sacc[kb][base + 4], sacc[kb][base + 5]),
                    pack2<BF16>(sacc[kb][base + 6], sacc[kb][base + 7])};
    }
    if (rescale) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= corr;
    }
    // A operand of k-step s: keys 16 s + 4 g + 0..3 (elements 0-3) and
    // 16 s + 8 + 4 g + 0..3 (elements 4-7) of the lane's dim. (k-steps outer,
    // dimension blocks inner: consecutive products independent.)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 w0 = lds_read_tr(vt_lds + vao[db][0] + 16 * s * D * 2);
        const u32x2 w1 = lds_read_tr(vt_lds + vao[db][1] + 16 * s * D * 2);
        oacc[db] = mfma_32x32x16<BF16>(u32x4{w0.x, w0.y, w1.x, w1.y}, pb[s], oacc[db]);
      }
    if constexpr (MV == 0) pin_reads_ahead<4 * (D / 32), 4, 2>();  // V reads, as above
    if constexpr (MV == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) mv[i] = mv_next[i];
    }
  };
  // Tile kt is fully visible when kt + BK <= lim: the tiles before the last
  // multiple of BK at or below lim, none without the fast path's conditions.
  // Tiles go in pairs (buffer 0, then 1), so that each buffer is a separate
  // LDS object throughout and no branch picks between two copies of the tile;
  // a fully visible tile left over from an odd count takes the general path.
  int kfull = 0;
  if (fast_ok) {
    int lim = klen;
    if (p.causal) lim = min(lim, q0 + off + 1);
    kfull = min(max(lim, 0) / BK * BK, kend);
  }
  kfull = kfull / (2 * BK) * (2 * BK);
  int kt = 0;
  for (; kt < kfull; kt += 2 * BK) {
    tile(kt, BoolC<true>{}, BoolC<false>{});
    tile(kt + BK, BoolC<true>{}, BoolC<true>{});
  }
  while (kt < kend) {
    tile(kt, BoolC<false>{}, BoolC<false>{});
    kt += BK;
    if (kt >= kend) break;
    tile(kt, BoolC<false>{}, BoolC<true>{});
    kt += BK;
  }
  __builtin_amdgcn_s_waitcnt(0);  // (no load outlives the workgroup)

  const float L = other_half_sum(l_i);  // both halves of the query's keys
  if (!qvalid) return;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;  // no visible key: zeros
  char* orow = p.o + ((int64_t)b * p.so_b + (int64_t)h * p.so_h + (int64_t)qi * p.so_s) * 2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const u32x2 w{pack2<BF16>(oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv),
                    pack2<BF16>(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + (db * 32 + 8 * rg + 4 * g) * 2) = w;
    }
  if (p.lse && g == 0)
    p.lse[((int64_t)b * p.H + h) * Sq + qi] = L > 0.0f ? (m_i + log2f(L)) * kLn2A : kNegInfA;
}

template <bool BF16, int D>
hipError_t launch_kind(const AttnParams& p, hipStream_t st) {
  const dim3 grid(p.H * p.B * ((p.Sq + kAttnBq - 1) / kAttnBq)), block(256);
  switch (p.mask_kind) {
    case ATTN_MASK_NONE: hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_NONE, 0>), grid, block, 0, st, p); break;
    case ATTN_MASK_ADD:
      if (p.mask_tile) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 2>), grid, block, 0, st, p);
      else if (p.mask_vec) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 1>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 0>), grid, block, 0, st, p);
      break;
    case ATTN_MASK_BOOL:
      if (p.mask_tile) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 3>), grid, block, 0, st, p);
      else if (p.mask_vec) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 1>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 0>), grid, block, 0, st, p);
      break;
    case ATTN_MASK_LEN: hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_LEN, 0>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace sms

hipError_t sms_attn_launch(const sms::AttnParams* p, int dtype, int head_dim, hipStream_t st) {
  if (dtype == 1 && head_dim == 64) return sms::launch_kind<false, 64>(*p, st);
  if (dtype == 1 && head_dim == 128) return sms::launch_kind<false, 128>(*p, st);
  if (dtype == 2 && head_dim == 64) return sms::launch_kind<true, 64>(*p, st);
  if (dtype == 2 && head_dim == 128) return sms::launch_kind<true, 128>(*p, st);
  return hipErrorInvalidValue;
}
