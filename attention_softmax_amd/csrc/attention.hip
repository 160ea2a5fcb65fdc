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
// Keys arrive in tiles of 64 through LDS: without a per-score mask straight
// from global memory into double-buffered tiles (attn_fwd_dma_kernel), with
// one through registers (attn_fwd_kernel, V stored transposed). Per tile
// a wavefront computes S^T = K Q^T (keys x queries) with
// v_mfma_f32_32x32x16_{f16,bf16}, so each lane holds 16 keys of one query:
// the row maximum and sum are mostly in-lane plus one swap with the lane 32
// away (which holds the other 16 keys of the same query). The probabilities
// are then, register for register, the B operand of O^T += V^T P^T (the
// contraction over keys in an order that matches the S^T output layout; the
// A operand reads the matching keys of V^T), so P never leaves registers.
//
// MFMA 32x32x16 lane layout (probed on MI355X): A (32x16): lane l holds row
// l%32, k = 8*(l/32)..+7; B (16x32): lane l holds column l%32, same k; D
// (32x32): lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4 in its
// registers r = 0..15.

#include "attention.hpp"

namespace sms {
namespace {

using namespace attn;

// Forward with a per-score mask (additive or boolean). K and V tiles pass
// through registers into LDS (K row-major, V transposed), single-buffered.
// MV: 2 when every mask row of the workgroup's
// queries starts on a 16-byte line, so that a tile's mask values (128 queries
// x 64 keys) come with its K / V fetch as whole-line 16-byte loads and are
// staged in LDS; 1 when mask rows start on 4 elements (runs of 4 keys per
// lane, loaded at the start of each tile by load_mask_runs); 0: each mask
// value is read where it is used.
template <bool BF16, int D, int KIND, int MV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(AttnParams p) {
  static_assert(KIND == ATTN_MASK_ADD || KIND == ATTN_MASK_BOOL, "a per-score mask");
  constexpr int BK = kAttnBk;
  constexpr int KP = D + 8;   // K tile row pitch, elements (conflict-free 16-byte reads)
  constexpr int VP = BK + 4;  // V^T tile row pitch, elements (34 dwords: 8-byte reads spread)
  __shared__ __align__(16) uint16_t ks[BK * KP];
  __shared__ __align__(16) uint16_t vt[D * VP];
  // Mask tile (MV == 2): kAttnBq rows of BK values; row pitch 144 bytes for
  // 16-bit values, 80 for bytes (16-byte rows for the staging stores; the
  // lanes' 8- or 4-byte run reads spread over the banks).
  constexpr int MB = KIND == ATTN_MASK_ADD ? 2 : 1;  // bytes per mask value
  constexpr int MP = MB == 2 ? 144 : 80;             // mask tile row pitch, bytes
  constexpr int MCH = BK * MB / 16;                  // 16-byte chunks per row
  constexpr int MC = MV == 2 ? kAttnBq * MCH / 256 : 1;  // chunks per thread
  __shared__ __align__(16) uint8_t ms[MV == 2 ? kAttnBq * MP : 16];

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
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
  int kend = Sk;
  if (p.causal) kend = min(kend, max(q0 + kAttnBq + off, 0));
  int kq = Sk;
  if (p.causal) kq = min(kq, max(qi + off + 1, 0));
  const bool qvalid = qi < Sq;
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

  // Key/value tiles are fetched one tile ahead into registers (KC 16-byte
  // chunks of K and VR rows of V per thread), so their global-memory latency
  // overlaps the current tile's products; a thread then stores its K chunks
  // row-major and its 4 keys x 8 dims of V transposed into LDS.
  constexpr int KCH = D / 8;                     // 16-byte chunks per K row
  constexpr int KC = BK * KCH / 256;              // K chunks per thread
  constexpr int VITEMS = (BK / 4) * (D / 8);      // (4 keys x 8 dims) items per tile
  const int vdg = tid % (D / 8), vkg = tid / (D / 8);
  const bool vthread = tid < VITEMS;
  u32x4 kreg[KC], vreg[4], mreg[MC];
  // The fetch reads through buffer resources re-based on each tile (scalar
  // registers) that end at the last key: rows past it read as zero, with no
  // per-load test or branch, and each thread's byte offsets within a tile
  // stay fixed. Being unconditional, the loads also keep the wait for a
  // tile's mask values (issued before the fetch) from covering the fetch.
  uint32_t koff[KC], voff[4];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int idx = tid + 256 * i, row = idx / KCH, ch = idx - row * KCH;
    koff[i] = (uint32_t)(row * p.sk_s * 2 + ch * 16);
  }
  // (Threads past the V items, with D = 64, load a copy of another
  // thread's item: a branch around their loads would make the wait for the
  // mask values cover the fetch too.)
  const int vtid = tid % VITEMS, vdgl = vtid % (D / 8), vkgl = vtid / (D / 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((4 * vkgl + i) * p.sv_s * 2 + vdgl * 16);
  // Mask tile (MV == 2): the workgroup's query rows (past Sq: none) through
  // one buffer range ending at the last row's last key; keys past Sk of the
  // other rows read the next row's first values, whose scores are excluded.
  uint32_t moff[MC];
  const int64_t mtile = (int64_t)b * p.sm_b + (int64_t)h * p.sm_h + (int64_t)q0 * p.sm_q;
  const int mrows = min(Sq - q0, kAttnBq);
#pragma unroll
  for (int i = 0; i < MC; ++i) {
    const int idx = tid + 256 * i, row = idx / MCH, ch = idx - row * MCH;
    moff[i] = (uint32_t)(row * p.sm_q * MB + ch * 16);
  }
  auto fetch = [&](int kt) {
    const int rows = min(Sk - kt, BK);
    const auto kr = rows_rsrc(kbase + (int64_t)kt * p.sk_s * 2, rows, p.sk_s * 2, D * 2);
    const auto vr = rows_rsrc(vbase + (int64_t)kt * p.sv_s * 2, rows, p.sv_s * 2, D * 2);
#pragma unroll
    for (int i = 0; i < KC; ++i) kreg[i] = rsrc_load(kr, koff[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vreg[i] = rsrc_load(vr, voff[i]);
    if constexpr (MV == 2) {
      const auto mr = rows_rsrc(p.mask + (mtile + kt) * MB, rows > 0 ? mrows : 0, p.sm_q * MB,
                                max(rows, 0) * MB);
#pragma unroll
      for (int i = 0; i < MC; ++i) mreg[i] = rsrc_load(mr, moff[i]);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int idx = tid + 256 * i, row = idx / KCH, ch = idx - row * KCH;
      *reinterpret_cast<u32x4*>(&ks[row * KP + ch * 8]) = kreg[i];
    }
    if (vthread) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x2 w{pair(vreg[0], vreg[1], j), pair(vreg[2], vreg[3], j)};
        *reinterpret_cast<u32x2*>(&vt[(8 * vdg + j) * VP + tcol(8 * vdg + j, vkg)]) = w;
      }
    }
    if constexpr (MV == 2) {
#pragma unroll
      for (int i = 0; i < MC; ++i) {
        const int idx = tid + 256 * i, row = idx / MCH, ch = idx - row * MCH;
        *reinterpret_cast<u32x4*>(&ms[row * MP + ch * 16]) = mreg[i];
      }
    }
  };
  if (kend > 0) fetch(0);
  // This lane's V^T operand rows c, c + 32, ... (tcol's lane part included).
  const uint16_t* vlane = &vt[c * VP + tcol_lane(c, g)];

  // One key tile.
  auto tile = [&](const int kt) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    u32x2 mv[8];  // this tile's mask values (additive / boolean masks)
    if constexpr (MV == 1) {
      load_mask_runs<KIND>(p.mask, mrow_c, kt, g, Sk, mv);
      __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the prefetch
    }
    if (MV == 1 || kt + BK < kend) fetch(kt + BK);  // in flight during this tile's products
    // Keep the fetch ahead of the products (under register pressure the
    // scheduler otherwise sinks the loads to the end of the loop, where the
    // next tile's stage waits for them at once).
    if constexpr (MV == 1) __builtin_amdgcn_sched_barrier(0);
    if constexpr (MV == 2) {
      // The lane's runs of 4 keys (the layout of load_mask_runs) from the tile.
      const uint8_t* mrow_l = &ms[(wave * 32 + c) * MP];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kk = (i >> 2) * 32 + 8 * (i & 3) + 4 * g;
        if constexpr (MB == 2) {
          mv[i] = *reinterpret_cast<const u32x2*>(mrow_l + kk * 2);
        } else {
          mv[i].x = *reinterpret_cast<const uint32_t*>(mrow_l + kk);
          mv[i].y = 0;
        }
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
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&ks[(kb * 32 + c) * KP + s * 16 + 8 * g]);
        sacc[kb] = mfma_32x32x16<BF16>(a, qf[s], sacc[kb]);
      }
    // K reads ten products ahead: 2-5 % faster than the scheduler's own order
    // (measured without per-score mask runs, whose loads share the region).
    if constexpr (MV == 0) pin_reads_ahead<2 * (D / 16), 10, 1>();

    // Scores in the log2 domain, the mask and the key bounds (tested only on
    // tiles with a key past Sk or, with a causal rule, past the first query's
    // bound).
    const bool inb = kt + BK <= Sk && (!p.causal || kt + BK <= q0 + off + 1);
    float mloc = kNegInfA;
    if (inb) {
      // Every key in bounds for every query: the mask alone.
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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(sacc[kb][r] - m_use);
        sacc[kb][r] = pv;
        psum += pv;
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
    // (k-steps outer, dimension blocks inner: consecutive products independent.)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vrow = vlane + db * 32 * VP;
        const u32x2 a0 = *reinterpret_cast<const u32x2*>(vrow + tcol_const(db, 2 * s));
        const u32x2 a1 = *reinterpret_cast<const u32x2*>(vrow + tcol_const(db, 2 * s + 1));
        oacc[db] = mfma_32x32x16<BF16>(u32x4{a0.x, a0.y, a1.x, a1.y}, pb[s], oacc[db]);
      }
    if constexpr (MV == 0) pin_reads_ahead<4 * (D / 32), 4, 2>();  // V^T reads, as above
  };
  for (int kt = 0; kt < kend; kt += BK) tile(kt);

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

// Forward without a per-score mask (none, or key lengths), fed by loads
// from global memory straight into LDS. The K and V tiles (64 keys x D
// values, dswz layout) are double-buffered: each tile starts with one
// barrier, after which the loads of the next tile go out into the other
// buffer and stay in flight during this tile's products; the data never
// passes through registers. K is read by rows (16 bytes per lane) for
// S^T = K Q^T; V stays row-major (keys x dims) and the A operand of
// O^T += V^T P^T is assembled by transposing LDS reads (lds_read_tr: a lane
// group addressing 4 keys x 16 dims hands every lane its own dim's 4
// consecutive keys). The buffers are separate LDS objects and the tiles go
// in pairs, so that every read has a fixed buffer: the compiler then knows
// that the reads do not touch the buffer the loads (compiler-visible here)
// are filling and inserts no wait for them, and the read offsets are
// loop-invariant registers plus immediates. (The backward kernels issue the
// loads from inline assembly instead, with one tile body for both buffers;
// here that measured 1-2 % slower.)

template <bool BF16, int D, int KIND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_dma_kernel(AttnParams p) {
  static_assert(KIND == ATTN_MASK_NONE || KIND == ATTN_MASK_LEN, "no per-score mask");
  constexpr int BK = kAttnBk;
  constexpr int TB = BK * D * 2;  // bytes per tile
  __shared__ __align__(1024) uint8_t ks0[TB];
  __shared__ __align__(1024) uint8_t ks1[TB];
  __shared__ __align__(1024) uint8_t vs0[TB];
  __shared__ __align__(1024) uint8_t vs1[TB];

  const int tid = (int)threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, c = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Grid order as in attn_fwd_kernel.
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

  const int off = p.causal == 2 ? Sk - Sq : 0;
  int klen = Sk;
  if constexpr (KIND == ATTN_MASK_LEN)
    klen = max(min(reinterpret_cast<const int32_t*>(p.mask)[b], Sk), 0);
  int kend = klen;
  if (p.causal) kend = min(kend, max(q0 + kAttnBq + off, 0));
  int kq = klen;
  if (p.causal) kq = min(kq, max(qi + off + 1, 0));
  const bool qvalid = qi < Sq;
  const bool fast_ok = p.scale_log2 > 0.0f;

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
  if (kend > 0) dma(0, BoolC<false>{});

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
    if (kt + BK < kend) dma(kt + BK, BoolC<BUF == 0>{});

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt_lds + kao[s] + kb * 32 * D * 2);
        sacc[kb] = mfma_32x32x16<BF16>(a, qf[s], sacc[kb]);
      }
    pin_reads_ahead<2 * (D / 16), 10, 1>();

    float mloc = kNegInfA;
    if constexpr (FULL) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kb][r]);
      mloc *= p.scale_log2;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          float t = sacc[kb][r] * p.scale_log2;
          if (key >= kq || key >= Sk) t = kNegInfA;
          sacc[kb][r] = t;
          mloc = fmaxf(mloc, t);
        }
    }
    mloc = other_half_max(mloc);
    const bool grow = mloc > m_i + kLazy || (m_i == kNegInfA && mloc != kNegInfA);
    float corr = 1.0f;
    if (grow) {
      corr = __builtin_amdgcn_exp2f(m_i - mloc);
      m_i = mloc;
      l_i *= corr;
    }
    const float m_use = (m_i == kNegInfA) ? 0.0f : m_i;
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
    // 16 s + 8 + 4 g + 0..3 (elements 4-7) of the lane's dim.
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2 w0 = lds_read_tr(vt_lds + vao[db][0] + 16 * s * D * 2);
        const u32x2 w1 = lds_read_tr(vt_lds + vao[db][1] + 16 * s * D * 2);
        oacc[db] = mfma_32x32x16<BF16>(u32x4{w0.x, w0.y, w1.x, w1.y}, pb[s], oacc[db]);
      }
    pin_reads_ahead<4 * (D / 32), 4, 2>();
  };
  int kfull = 0;
  if (fast_ok) {
    int lim = klen;
    if (p.causal) lim = min(lim, q0 + off + 1);
    kfull = min(max(lim, 0) / BK * BK, kend);
  }
  // Tiles go in pairs (buffer 0, then 1), so that each buffer is a separate
  // LDS object throughout (which keeps the compiler from waiting for the next
  // tile's loads before this tile's reads) and no branch picks between two
  // copies of the tile; a fully visible tile left over from an odd count takes
  // the general path.
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

  const float L = other_half_sum(l_i);
  if (!qvalid) return;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
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
  const int mv = p.mask_tile ? 2 : p.mask_vec ? 1 : 0;
  switch (p.mask_kind) {
    case ATTN_MASK_NONE: hipLaunchKernelGGL((attn_fwd_dma_kernel<BF16, D, ATTN_MASK_NONE>), grid, block, 0, st, p); break;
    case ATTN_MASK_ADD:
      if (mv == 2) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 2>), grid, block, 0, st, p);
      else if (mv == 1) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 1>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_ADD, 0>), grid, block, 0, st, p);
      break;
    case ATTN_MASK_BOOL:
      if (mv == 2) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 2>), grid, block, 0, st, p);
      else if (mv == 1) hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 1>), grid, block, 0, st, p);
      else hipLaunchKernelGGL((attn_fwd_kernel<BF16, D, ATTN_MASK_BOOL, 0>), grid, block, 0, st, p);
      break;
    case ATTN_MASK_LEN: hipLaunchKernelGGL((attn_fwd_dma_kernel<BF16, D, ATTN_MASK_LEN>), grid, block, 0, st, p); break;
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
