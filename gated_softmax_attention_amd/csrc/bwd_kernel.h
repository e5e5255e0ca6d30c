// FiX attention backward kernels for gfx950 (m held constant).
//
// With P_ij = exp(s_ij - m_i), D_ij = exp(G_i - G_j) and delta_i the gradient
// reaching x_i (see bwd_prep.hip), the gradients are
//   dP_ij = sum_d delta_i,d D_ij,d v_j,d ,   dS_ij = P_ij dP_ij
//   dq_i = scale sum_j dS_ij k_j ,  dk_j = scale sum_i dS_ij q_i (over the head group)
//   dv_j = sum_i P_ij D_ij (.) delta_i (over the head group)
// (no softmax row-sum term: the denominator is not part of FiX, FiX ICML
// 2026 poster page, abstract).
//
// Split of the work.  Sequences are cut into 128-token chunks.
//  * Pairs in different chunks: k_bwd_dq (one workgroup per 128 query rows,
//    key chunks visited last to first) and k_bwd_dkv (one workgroup per 128
//    keys, query chunks from two after the key chunk on, first to last).  The decay between the query
//    chunk I and the key chunk J factors as
//        exp(Gl_i) * gamma_IJ * exp(Gl_end(J) - Gl_j),
//    gamma_IJ the product of the chunk decays strictly between, all <= 1.
//    gamma is folded into the operand tiles while they are staged into LDS
//    (V of chunk J in k_bwd_dq, scaled dhat of chunk I in k_bwd_dkv), so the
//    waves' inner loop is a plain four-product attention backward:
//    S = QK^T (bf16 MFMA), dP (fp16 MFMA), dV += P^T dhat, dK += dS^T Q,
//    dQ += dS K (fp16 MFMA).
//  * Pairs inside one chunk: k_bwd_intra_dq (a wave per 32 query rows) and
//    k_bwd_intra_dkv (a wave per 32 keys, which also takes the queries of
//    the next chunk).  Between different 32-token blocks
//    the decay is split at a token between them (both factors <= 1, fp16
//    operands); inside a 32x32 diagonal block it is split at the token before
//    the block, where the key side is >= 1 and needs fp32 range: those
//    products run as three bf16 MFMAs (hi*hi + hi*lo + lo*hi).  A block whose
//    gate range exceeds 2^BGUARD is evaluated with direct per-pair decays.
//    These kernels write fp32 partials that the chunk kernels add in their
//    epilogues.
#pragma once
#include "common.h"
#include "launch.h"

namespace fix {

constexpr float BGUARD = 100.f;  // largest factored gate range of a 32-token block (log2 units)

template <int D> struct Pad32 { static constexpr int value = D < 32 ? 32 : D; };

// Exact per-pair decays for a diagonal 32x32 block whose gate range exceeds
// 2^BGUARD (rare): dP for the pairs held by this lane, evaluated directly.
// Register j of lane (hh, n) holds the pair (row q0 + rowof(j, n), key k0 + keyof(j, n)).
// (Arguments by value: passing the kernel's argument struct by reference
// would force a stack copy of it in every kernel that can call this.)
template <int DV, bool F32IN, bool ROW_IS_LANE>
__device__ __noinline__ void direct_dp(const float *delta, const float *sig, const float *Gl2, const void *v, int Hq,
                                       int Hkv, int64_t st, int c, int h, int L, int q0, int k0, int hh, int n,
                                       float *dp) {
  for (int j = 0; j < 16; ++j) {
    const int r = ROW_IS_LANE ? n : acc_row(hh, j);
    const int kk = ROW_IS_LANE ? acc_row(hh, j) : n;
    const int qi = q0 + r, kj = k0 + kk;
    float t = 0.f;
    if (qi < L && kj <= qi) {
      const float *dr = delta + ((st + qi) * Hq + h) * DV;
      const float sg = sig[(st + qi) * Hq + h];
      for (int d = 0; d < DV; ++d) {
        const float gq = Gl2[((st + qi) * Hkv + c) * DV + d], gk = Gl2[((st + kj) * Hkv + c) * DV + d];
        t += dr[d] * sg * fast_exp2(gq - gk) * load_in(v, ((st + kj) * Hkv + c) * DV + d, F32IN);
      }
    }
    dp[j] = t;
  }
}

// ---------------------------------------------------------------------------
// Within-chunk contributions to dq.  Workgroup = one 128-chunk of one q head;
// wave w owns query rows c0 + 32w .. +31 (query block w).  Key blocks b are
// copied into LDS one per step (double buffered): K rows, transposed K, V
// scaled to the end of its block (VE), and for the diagonal block of wave b
// its V relative to the token before it and query block b's dhat (bf16 hi /
// lo each), so every wave's diagonal block is computed in the step of its
// own key block.  With E(b) the chunk-local log2
// gate prefix at the end of block b (E(-1) = 0), the decay of a pair in
// query block a > b splits as
//     exp2(Gl_i - E(a-1)) * exp2(E(a-1) - E(b)) * exp2(E(b) - Gl_j),
// all three <= 1: the first is the prepared block-relative dhat (X16), the
// middle one gamma_ab multiplies the wave's dhat operand per channel, the
// last is VE.  On the diagonal block the split is at the token before it:
// the key side exp2(E(a-1) - Gl_j) >= 1 needs fp32 range and is multiplied
// as bf16x3 (hi*hi + hi*lo + lo*hi); a block whose gate range exceeds
// 2^BGUARD is evaluated with direct per-pair decays.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 1) k_bwd_intra_dq(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, NBK = DKP / 32;
  using KT = LdsTile<32, DK * 2>;   // K rows of the key block
  using TT = LdsTile<DKP, 64>;     // transposed K, rows padded to DKP
  using TTD = LdsTile<DK, 64>;
  using VT = LdsTile<32, DV * 2>;  // VE rows of the key block
  // One LDS object for every tile (see the forward kernel).
  constexpr int O_K = 0, O_T = O_K + 2 * KT::BYTES, O_V = O_T + 2 * TT::BYTES, O_E = O_V + 2 * VT::BYTES;
  // Per stage also, for the diagonal block of the wave whose block it is, the
  // key block's V relative to the token before it and the same block's
  // block-relative dhat rows (bf16 hi, lo each).
  constexpr int O_BH = O_E + 5 * DV * 4, O_BL = O_BH + 2 * VT::BYTES, O_XH = O_BL + 2 * VT::BYTES;
  constexpr int O_XL = O_XH + 2 * VT::BYTES;
  __shared__ __align__(1024) char smem[O_XL + 2 * VT::BYTES];
  auto BHs = [&](int b) { return smem + O_BH + b * VT::BYTES; };
  auto BLs = [&](int b) { return smem + O_BL + b * VT::BYTES; };
  auto XHs = [&](int b) { return smem + O_XH + b * VT::BYTES; };
  auto XLs = [&](int b) { return smem + O_XL + b * VT::BYTES; };
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Kts = [&](int b) { return smem + O_T + b * TT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  float(*BE)[DV] = (float(*)[DV])(smem + O_E);  // BE[b + 1] = E(b), BE[0] = 0

  const Plan &pl = a.plan;
  const int gc = blockIdx.x, hq = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = uniform((gc - pl.cb128[s]) * CB);
  const int L = uniform(pl.seq_len[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int Hq = a.Hq, Hkv = a.Hkv, c = hq / (Hq / Hkv);
  const int nblk = min(4, (L - c0 + 31) / 32);  // query (and key) blocks present in the chunk
  const int r0 = c0 + 32 * wave;
  const int row = r0 + n;
  const bool active = wave < nblk;
  const bool rv = active && row < L;
  const float sl2 = a.sl2;
  auto gl_at = [&](int tok, int d) { return a.Gl2[((st + tok) * Hkv + c) * DV + d]; };

  for (int e = tid; e < 5 * DV; e += 256) {
    const int b = e / DV - 1, d = e % DV;
    BE[b + 1][d] = b < 0 ? 0.f : gl_at(min(c0 + 32 * b + 31, L - 1), d);
  }
  if (DK < DKP)
    for (int e = tid; e < (DKP - DK) * 64 / 4; e += 256) {
      ((uint32_t *)(Kts(0) + DK * 64))[e] = 0u;
      ((uint32_t *)(Kts(1) + DK * 64))[e] = 0u;
    }
  kfrag qf[NS];
  f16x8 xr[NSV];  // the row's block-relative dhat, B operand of dP^T (k = channel)
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = rv ? IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();
#pragma unroll
  for (int i = 0; i < NSV; ++i)
    xr[i] = rv ? *(const f16x8 *)(a.X16 + ((st + row) * Hq + hq) * DV + 16 * i + 8 * hh)
               : __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  const float mbn = rv ? a.mb[(st + row) * Hq + hq] : INFINITY;
  f32x16 acc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) acc[b] = zero16();

  // Key block b is staged with the rows before the sequence end only (the
  // rest read as zeros): off the diagonal every key is valid, on the diagonal
  // the keys past the end meet only masked pairs.
  uint32_t ok[KT::NW], ot[TTD::NW], ov[VT::NW], oxq[VT::NW];
  VT::lane_offsets(Hq * DV * 2, wave, lane, oxq);
  KT::lane_offsets(Hkv * DK * 2, wave, lane, ok);
  TTD::lane_offsets(CB * 2, wave, lane, ot);
  VT::lane_offsets(Hkv * DV * 2, wave, lane, ov);
  auto stage_tile = [&](int b, int buf) {
    const int kb = c0 + 32 * b;
    const int64_t kr = (st + kb) * Hkv + c;
    const int nrow = min(32, L - kb);
    if constexpr (!F32IN) {
      const u32x4 rk = rsrc_words((const uint16_t *)a.k + kr * DK, (int64_t)nrow * Hkv * DK * 2);
#pragma unroll
      for (int t = 0; t < KT::NW; ++t) KT::dma_piece_untracked(Ks(buf), rk, ok, t, wave);
    } else {
      for (int p = tid; p < KT::NCH; p += 256) {
        const int r = p / KT::CPR, cc = p % KT::CPR;
        *(f16x8 *)(Ks(buf) + KT::off(r, cc)) = IF::load(a.k, ((st + min(kb + r, L - 1)) * Hkv + c) * DK + 8 * cc);
      }
    }
    const u32x4 rt = rsrc_words(a.Kt + ((int64_t)gc * Hkv + c) * DK * CB + 32 * b, (int64_t)DK * CB * 2);
#pragma unroll
    for (int t = 0; t < TTD::NW; ++t) TTD::dma_piece_untracked(Kts(buf), rt, ot, t, wave);
    const u32x4 rv = rsrc_words(a.VE + kr * DV, (int64_t)nrow * Hkv * DV * 2);
    const u32x4 rbh = rsrc_words(a.VBH + kr * DV, (int64_t)nrow * Hkv * DV * 2);
    const u32x4 rbl = rsrc_words(a.VBL + kr * DV, (int64_t)nrow * Hkv * DV * 2);
    const int64_t xq = ((st + kb) * Hq + hq) * DV;  // query block b = key block b
    const u32x4 rxh = rsrc_words(a.XH + xq, (int64_t)nrow * Hq * DV * 2);
    const u32x4 rxl = rsrc_words(a.XL + xq, (int64_t)nrow * Hq * DV * 2);
#pragma unroll
    for (int t = 0; t < VT::NW; ++t) {
      VT::dma_piece_untracked(Vs(buf), rv, ov, t, wave);
      VT::dma_piece_untracked(BHs(buf), rbh, ov, t, wave);
      VT::dma_piece_untracked(BLs(buf), rbl, ov, t, wave);
      VT::dma_piece_untracked(XHs(buf), rxh, oxq, t, wave);
      VT::dma_piece_untracked(XLs(buf), rxl, oxq, t, wave);
    }
  };

  // Key blocks b <= wave through LDS: the blocks before the wave's own, then
  // (at b = wave) its diagonal block, unless that block's gate range needs
  // exact per-pair decays (then it is done afterwards from global memory).
  const int nsteps = nblk;
  wait_all();  // every load above is complete before the first untracked copy
  if (nsteps > 0) stage_tile(0, 0);
  wait_all();
  __syncthreads();
  bool direct;
  {
    float rng = 0.f;
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[wave][d] - BE[wave + 1][d]);
      }
    direct = __any(rng > BGUARD);
  }
  for (int b = 0; b < nsteps; ++b) {
    const int buf = b & 1;
    const bool diag = wave == b;
    const bool act = active && (wave > b || (diag && !direct));
    // gamma_ab (an LDS table) is applied before the next copies are issued:
    // LDS reads that follow a copy issue in the same step can make the
    // compiler wait for it.
    f16x8 xg[NSV];
    if (act && !diag) {
#pragma unroll
      for (int i = 0; i < NSV; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 16 * i + 8 * hh + e;
          xg[i][e] = (_Float16)((float)xr[i][e] * fast_exp2(BE[wave][d] - BE[b + 1][d]));
        }
    }
    stage_tile(min(b + 1, nsteps - 1), buf ^ 1);
    if (act) {
      // S^T[key][row]: lane = row, register j = key acc_row(hh, j)
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const kfrag *)(Ks(buf) + KT::off(n, 2 * i + hh)), qf[i], sc);
      f16x8 dsf[2];
      if (diag) {
        // split at the token before the block: V and dhat as bf16 hi / lo (bf16x3)
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          const bf16x8 vh = *(const bf16x8 *)(BHs(buf) + VT::off(n, 2 * i + hh));
          const bf16x8 vl = *(const bf16x8 *)(BLs(buf) + VT::off(n, 2 * i + hh));
          const bf16x8 xh = *(const bf16x8 *)(XHs(buf) + VT::off(n, 2 * i + hh));
          const bf16x8 xl = *(const bf16x8 *)(XLs(buf) + VT::off(n, 2 * i + hh));
          dp = mma32(vh, xh, dp);
          dp = mma32(vh, xl, dp);
          dp = mma32(vl, xh, dp);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int j = 8 * u + i;
            dsf[u][i] = (_Float16)(acc_row(hh, j) > n ? 0.f : fast_exp2(sc[j] * sl2 - mbn) * dp[j]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)(Vs(buf) + VT::off(n, 2 * i + hh)), xg[i], dp);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) dsf[u][i] = (_Float16)(fast_exp2(sc[8 * u + i] * sl2 - mbn) * dp[8 * u + i]);
      }
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[bk] = mma32(dsf[u], *(const f16x8 *)(Kts(buf) + TT::off(32 * bk + n, 2 * u + hh)), acc[bk]);
    }
    wait_all();
    __syncthreads();
  }
  if (!active) return;
  // Diagonal block with exact per-pair decays (gate range beyond 2^BGUARD),
  // per wave from global memory; the staged loop did the others.
  if (direct) {
    const int kb = r0;
    const int key = min(kb + n, L - 1);
    float rng = 0.f;
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[wave][d] - BE[wave + 1][d]);
      }
    const bool direct = __any(rng > BGUARD);
    f32x16 sc = zero16(), dp = zero16();
#pragma unroll
    for (int i = 0; i < NS; ++i)
      sc = mma32(IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh), qf[i], sc);
    if (!direct) {
      const int64_t kr = ((st + key) * Hkv + c) * DV, xrw = ((st + min(row, L - 1)) * Hq + hq) * DV;
#pragma unroll
      for (int i = 0; i < NSV; ++i) {
        // the key's V relative to the token before the block, bf16 hi / lo
        const bf16x8 zero = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        const bf16x8 vh = kb + n < L ? *(const bf16x8 *)(a.VBH + kr + 16 * i + 8 * hh) : zero;
        const bf16x8 vl = kb + n < L ? *(const bf16x8 *)(a.VBL + kr + 16 * i + 8 * hh) : zero;
        const bf16x8 xh = *(const bf16x8 *)(a.XH + xrw + 16 * i + 8 * hh);
        const bf16x8 xl = *(const bf16x8 *)(a.XL + xrw + 16 * i + 8 * hh);
        dp = mma32(vh, xh, dp);
        dp = mma32(vh, xl, dp);
        dp = mma32(vl, xh, dp);
      }
    } else {
      float t[16];
      direct_dp<DV, F32IN, true>(a.delta, a.sig, a.Gl2, a.v, Hq, Hkv, st, c, hq, L, r0, kb, hh, n, t);
#pragma unroll
      for (int j = 0; j < 16; ++j) dp[j] = t[j];
    }
    f16x8 dsf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = 8 * u + i;
        dsf[u][i] = (_Float16)(acc_row(hh, j) > n ? 0.f : fast_exp2(sc[j] * sl2 - mbn) * dp[j]);
      }
    const _Float16 *ktile = a.Kt + ((int64_t)gc * Hkv + c) * DK * CB + 32 * wave;
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      const int col = min(32 * bk + n, DK - 1);  // padded columns are never stored
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[bk] = mma32(dsf[u], *(const f16x8 *)(ktile + (int64_t)col * CB + 16 * u + 8 * hh), acc[bk]);
    }
  }
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + acc_row(hh, j);
      if (r < L) a.dq_i[((st + r) * Hq + hq) * DK + col] = a.scale * acc[bk][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Near contributions to dk, dv: workgroup = one 128-chunk J of one kv head;
// wave w owns keys c0 + 32w .. +31 (key block w), against the query blocks
// qa = 0..7 of chunk J and of the next chunk (the pairs with the largest
// decay weights), summed over the head group.  Each step copies one query
// block into LDS (double buffered): Q rows, transposed Q, the block-relative
// dhat as fp16 rows (dP off the diagonal), bf16 hi/lo rows (dP on the
// diagonal) and bf16 hi/lo transposed (dV, always bf16x3: dv feeds the gate
// gradient, whose suffix sums accumulate the rounding of every token).  With
// E(b) the log2 gate prefix at the end of block b, continued into the next
// chunk, the decay of a pair in query block qa > w splits as
//     exp2(Gl_i - E(qa-1)) * exp2(E(qa-1) - E(w)) * exp2(E(w) - Gl_j):
// the first factor is in the staged dhat, the middle one gamma multiplies
// the wave's V-to-block-end operand (dP) and each dV step's result per
// channel, and the last one scales dV in the epilogue.  The diagonal block
// (the step whose query block is the wave's own) uses gamma =
// exp2(E(w-1) - E(w)) >= 1 and V from the token before the block, as in the
// dq kernel, from tiles staged with that step; past 2^BGUARD its pairs are
// evaluated directly after the loop.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 1) k_bwd_intra_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, DVP = Pad32<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  using QT = LdsTile<32, DK * 2>;   // Q rows of the step
  using QTT = LdsTile<DKP, 64>;     // transposed Q (dk rows x 32 queries)
  using QTTD = LdsTile<DK, 64>;
  using XR = LdsTile<32, DV * 2>;   // block-relative dhat rows (fp16)
  using XTT = LdsTile<DVP, 64>;     // the same transposed (bf16 hi, lo), rows padded to DVP
  using XTTD = LdsTile<DV, 64>;
  // One LDS object for every tile (see the forward kernel).
  constexpr int O_Q = 0, O_QT = O_Q + 2 * QT::BYTES, O_X = O_QT + 2 * QTT::BYTES;
  constexpr int O_TH = O_X + 2 * XR::BYTES, O_TL = O_TH + 2 * XTT::BYTES;
  constexpr int O_M = O_TL + 2 * XTT::BYTES, O_E = O_M + 2 * 256, O_GW = O_E + 9 * DV * 4;
  // Diagonal steps also stage the query block's dhat as bf16 hi / lo rows and
  // the key block's V relative to the token before it (bf16 hi / lo rows).
  constexpr int O_XH = O_GW + 4 * DV * 4, O_XL = O_XH + 2 * XR::BYTES, O_BH = O_XL + 2 * XR::BYTES;
  constexpr int O_BL = O_BH + 2 * XR::BYTES;
  __shared__ __align__(1024) char smem[O_BL + 2 * XR::BYTES];
  auto XHs = [&](int b) { return smem + O_XH + b * XR::BYTES; };
  auto XLs = [&](int b) { return smem + O_XL + b * XR::BYTES; };
  auto BHs = [&](int b) { return smem + O_BH + b * XR::BYTES; };
  auto BLs = [&](int b) { return smem + O_BL + b * XR::BYTES; };
  auto Qs = [&](int b) { return smem + O_Q + b * QT::BYTES; };
  auto Qts = [&](int b) { return smem + O_QT + b * QTT::BYTES; };
  auto Xs = [&](int b) { return smem + O_X + b * XR::BYTES; };
  auto Ths = [&](int b) { return smem + O_TH + b * XTT::BYTES; };
  auto Tls = [&](int b) { return smem + O_TL + b * XTT::BYTES; };
  auto Ms = [&](int b) { return (float *)(smem + O_M + b * 256); };  // 64 floats, 32 used
  float(*BE)[DV] = (float(*)[DV])(smem + O_E);  // BE[b + 1] = E(b), b = -1..7
  float *gw = (float *)(smem + O_GW) + (threadIdx.x >> 6) * DV;  // this wave's gamma of the step, per channel

  const Plan &pl = a.plan;
  const int gc = blockIdx.x, c = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = uniform((gc - pl.cb128[s]) * CB);
  const int L = uniform(pl.seq_len[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int kb = c0 + 32 * wave;
  const bool active = kb < L;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;
  const int nqb = min(8, (L - c0 + 31) / 32);  // query blocks in this chunk and the next
  auto gl_at = [&](int tok, int d) { return a.Gl2[((st + tok) * Hkv + c) * DV + d]; };

  for (int e = tid; e < 9 * DV; e += 256) {
    const int b = e / DV - 1, d = e % DV;
    float v = 0.f;
    if (b >= 0 && b < 4) v = gl_at(min(c0 + 32 * b + 31, L - 1), d);
    if (b >= 4) {
      v = gl_at(min(c0 + CB - 1, L - 1), d);
      if (c0 + CB < L) v += gl_at(min(c0 + CB + 32 * (b - 4) + 31, L - 1), d);
    }
    BE[b + 1][d] = v;
  }
  if (DK < DKP)
    for (int e = tid; e < (DKP - DK) * 64 / 4; e += 256) {
      ((uint32_t *)(Qts(0) + DK * 64))[e] = 0u;
      ((uint32_t *)(Qts(1) + DK * 64))[e] = 0u;
    }
  if (DV < DVP)
    for (int e = tid; e < (DVP - DV) * 64 / 4; e += 256) {
      ((uint32_t *)(Ths(0) + DV * 64))[e] = 0u;
      ((uint32_t *)(Ths(1) + DV * 64))[e] = 0u;
      ((uint32_t *)(Tls(0) + DV * 64))[e] = 0u;
      ((uint32_t *)(Tls(1) + DV * 64))[e] = 0u;
    }
  kfrag kf[NS];
  f16x8 ve[NSV];  // the key's V to the end of its block, B operand of dP (k = channel)
#pragma unroll
  for (int i = 0; i < NS; ++i)
    kf[i] = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
#pragma unroll
  for (int i = 0; i < NSV; ++i)
    ve[i] = kv ? *(const f16x8 *)(a.VE + ((st + key) * Hkv + c) * DV + 16 * i + 8 * hh)
               : __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  f32x16 accK[NBK], accV[NBV];
#pragma unroll
  for (int b = 0; b < NBK; ++b) accK[b] = zero16();
#pragma unroll
  for (int b = 0; b < NBV; ++b) accV[b] = zero16();

  // Query blocks qa = 0 .. nqb - 1 of every head through LDS.  Wave w takes
  // the blocks after its own (qa > w) and, at qa = w, its diagonal block,
  // unless the block's gate range needs exact per-pair decays (then that
  // block is done afterwards, from global memory).
  const int nqo = nqb;
  const int nsteps = G * nqo;
  // Rows past the end of the sequence read as zeros; their probabilities are
  // masked to zero when the step is computed.
  uint32_t oq[QT::NW], oqt[QTTD::NW], ox[XR::NW], oxt[XTTD::NW], ob[XR::NW];
  XR::lane_offsets(Hkv * DV * 2, wave, lane, ob);
  QT::lane_offsets(Hq * DK * 2, wave, lane, oq);
  QTTD::lane_offsets(CB * 2, wave, lane, oqt);
  XR::lane_offsets(Hq * DV * 2, wave, lane, ox);
  XTTD::lane_offsets(CB * 2, wave, lane, oxt);
  auto stage_tile = [&](int k, int buf) {
    const int gq = k / nqo, qa = k % nqo;
    const int h = c * G + gq;
    const int q0 = c0 + 32 * qa;
    const int64_t qr = (st + q0) * Hq + h;
    const int nrow = L - q0;
    if constexpr (!F32IN) {
      const u32x4 rq = rsrc_words((const uint16_t *)a.q + qr * DK, (int64_t)nrow * Hq * DK * 2);
#pragma unroll
      for (int t = 0; t < QT::NW; ++t) QT::dma_piece_untracked(Qs(buf), rq, oq, t, wave);
    } else {
      for (int p = tid; p < QT::NCH; p += 256) {
        const int r = p / QT::CPR, cc = p % QT::CPR;
        *(f16x8 *)(Qs(buf) + QT::off(r, cc)) = IF::load(a.q, ((st + min(q0 + r, L - 1)) * Hq + h) * DK + 8 * cc);
      }
    }
    const int64_t ch = (int64_t)(gc + (qa >> 2)) * Hq + h;
    const u32x4 rqt = rsrc_words(a.Qt + ch * DK * CB + 32 * (qa & 3), (int64_t)DK * CB * 2);
#pragma unroll
    for (int t = 0; t < QTTD::NW; ++t) QTTD::dma_piece_untracked(Qts(buf), rqt, oqt, t, wave);
    const u32x4 rx = rsrc_words(a.X16 + qr * DV, (int64_t)nrow * Hq * DV * 2);
#pragma unroll
    for (int t = 0; t < XR::NW; ++t) XR::dma_piece_untracked(Xs(buf), rx, ox, t, wave);
    const u32x4 rth = rsrc_words(a.XTH + ch * DV * CB + 32 * (qa & 3), (int64_t)DV * CB * 2);
    const u32x4 rtl = rsrc_words(a.XTL + ch * DV * CB + 32 * (qa & 3), (int64_t)DV * CB * 2);
#pragma unroll
    for (int t = 0; t < XTTD::NW; ++t) {
      XTTD::dma_piece_untracked(Ths(buf), rth, oxt, t, wave);
      XTTD::dma_piece_untracked(Tls(buf), rtl, oxt, t, wave);
    }
    // lane r fills Ms[r] (every wave, the same bytes)
    dma4_untracked(Ms(buf), rsrc_words(a.mb + qr, (int64_t)nrow * Hq * 4), (uint32_t)lane * Hq * 4);
    if (qa < 4) {  // the diagonal block of wave qa
      const u32x4 rxh = rsrc_words(a.XH + qr * DV, (int64_t)nrow * Hq * DV * 2);
      const u32x4 rxl = rsrc_words(a.XL + qr * DV, (int64_t)nrow * Hq * DV * 2);
      const int64_t kr = (st + q0) * Hkv + c;  // the key block is the query block
      const u32x4 rbh = rsrc_words(a.VBH + kr * DV, (int64_t)nrow * Hkv * DV * 2);
      const u32x4 rbl = rsrc_words(a.VBL + kr * DV, (int64_t)nrow * Hkv * DV * 2);
#pragma unroll
      for (int t = 0; t < XR::NW; ++t) {
        XR::dma_piece_untracked(XHs(buf), rxh, ox, t, wave);
        XR::dma_piece_untracked(XLs(buf), rxl, ox, t, wave);
        XR::dma_piece_untracked(BHs(buf), rbh, ob, t, wave);
        XR::dma_piece_untracked(BLs(buf), rbl, ob, t, wave);
      }
    }
  };
  // Whether this wave's diagonal block needs exact per-pair decays (gate
  // range of the block beyond 2^BGUARD; BE is complete after the barrier below).
  auto exact_diag = [&]() {
    float rng = 0.f;
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[wave][d] - BE[wave + 1][d]);
      }
    return __any(rng > BGUARD);
  };

  if (nsteps > 0) stage_tile(0, 0);
  wait_all();
  __syncthreads();
  const bool direct = exact_diag();
  for (int k = 0; k < nsteps; ++k) {
    const int buf = k & 1;
    const int qa = k % nqo;
    const int q0 = c0 + 32 * qa;
    const bool diag = qa == wave;
    const bool act = active && (qa > wave || (diag && !direct));
    // The next step's copies first: they are issued from inline assembly that
    // the compiler's wait counts do not see, so the LDS reads below do not
    // wait for them, and they have the whole step to land.
    stage_tile(min(k + 1, nsteps - 1), buf ^ 1);
    float4 mq[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) mq[q4] = *(const float4 *)&Ms(buf)[8 * q4 + 4 * hh];
    float gcol[NBV];  // gamma of the lane's dV output columns
    f16x8 kop[NSV];   // V to block end (.) gamma, B operand of dP
    if (act) {
      // gamma[d] = exp2(E(qa - 1) - E(wave)) depends on the channel only: each
      // lane evaluates two channels into the wave's table, then every lane
      // reads the channels it needs (a wave's LDS accesses complete in order).
#pragma unroll
      for (int t = 0; t < (DV + 63) / 64; ++t) {
        const int d = lane + 64 * t;
        if (d < DV) gw[d] = fast_exp2(BE[qa][d] - BE[wave + 1][d]);
      }
#pragma unroll
      for (int bv = 0; bv < NBV; ++bv) gcol[bv] = gw[min(32 * bv + n, DV - 1)];
      if (!diag)
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          const float4 g0 = *(const float4 *)(gw + 16 * i + 8 * hh), g1 = *(const float4 *)(gw + 16 * i + 8 * hh + 4);
          const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) kop[i][e] = (_Float16)((float)ve[i][e] * gv[e]);
        }
    }
    if (act) {
      // S[q][key] and dP[q][key]: lane = key, register j = query acc_row(hh, j)
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const kfrag *)(Qs(buf) + QT::off(n, 2 * i + hh)), kf[i], sc);
      if (diag) {
        // split at the token before the block: dhat and V as bf16 hi / lo (bf16x3)
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          const bf16x8 xh = *(const bf16x8 *)(XHs(buf) + XR::off(n, 2 * i + hh));
          const bf16x8 xl = *(const bf16x8 *)(XLs(buf) + XR::off(n, 2 * i + hh));
          const bf16x8 vh = *(const bf16x8 *)(BHs(buf) + XR::off(n, 2 * i + hh));
          const bf16x8 vl = *(const bf16x8 *)(BLs(buf) + XR::off(n, 2 * i + hh));
          dp = mma32(xh, vh, dp);
          dp = mma32(xl, vh, dp);
          dp = mma32(xh, vl, dp);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)(Xs(buf) + XR::off(n, 2 * i + hh)), kop[i], dp);
      }
      f16x8 dsf[2];
      bf16x8 ph[2], plo[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float mv[4] = {mq[q4].x, mq[q4].y, mq[q4].z, mq[q4].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * q4 + e;
          const int r = acc_row(hh, j);
          const float pv = q0 + r < L && (!diag || r >= n) ? fast_exp2(sc[j] * sl2 - mv[e]) : 0.f;
          dsf[j >> 3][j & 7] = (_Float16)(pv * dp[j]);
          split_bf16(pv, ph[j >> 3], plo[j >> 3], j & 7);
        }
      }
      // dV[key][d] += gamma[d] * sum_q P[q][key] dhat[q][d]  (bf16x3)
#pragma unroll
      for (int bv = 0; bv < NBV; ++bv) {
        f32x16 tmp = zero16();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 th = *(const bf16x8 *)(Ths(buf) + XTT::off(32 * bv + n, 2 * u + hh));
          const bf16x8 tl = *(const bf16x8 *)(Tls(buf) + XTT::off(32 * bv + n, 2 * u + hh));
          tmp = mma32(ph[u], th, tmp);
          tmp = mma32(ph[u], tl, tmp);
          tmp = mma32(plo[u], th, tmp);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) accV[bv][j] += gcol[bv] * tmp[j];
      }
      // dK[key][dk] += dS[q][key] Q[q][dk]
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          accK[bk] = mma32(dsf[u], *(const f16x8 *)(Qts(buf) + QTT::off(32 * bk + n, 2 * u + hh)), accK[bk]);
    }
    wait_all();
    __syncthreads();
  }
  if (!active) return;

  // Diagonal block with exact per-pair decays (gate range beyond 2^BGUARD),
  // per head from global memory.  (Otherwise the staged loop did it: split at
  // the token before the block, gamma = exp2(E(w-1) - E(w)) >= 1, V from the
  // token before the block as bf16x3.)
  bool dflag = false;  // exact diagonal contributions written to dv_i
  {
    float rng = 0.f, gd[NBV];
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[wave][d] - BE[wave + 1][d]);
      }
#pragma unroll
    for (int bv = 0; bv < NBV; ++bv) {
      const int d = min(32 * bv + n, DV - 1);
      gd[bv] = fast_exp2(BE[wave][d] - BE[wave + 1][d]);
    }
    const bool direct = __any(rng > BGUARD);
    // (the staged loop computed this block unless it needs the exact decays)
    bf16x8 vh[NSV], vl[NSV];
#pragma unroll
    for (int i = 0; i < NSV; ++i) vh[i] = vl[i] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    const int q0 = kb;
    const int qrow = min(q0 + n, L - 1);  // A-operand row of this lane
    for (int gq = 0; direct && gq < G; ++gq) {
      const int h = c * G + gq;
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i)
        sc = mma32(IF::load(a.q, ((st + qrow) * Hq + h) * DK + 16 * i + 8 * hh), kf[i], sc);
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = acc_row(hh, j);
        p[j] = (q0 + r < L && r >= n) ? fast_exp2(sc[j] * sl2 - a.mb[(st + q0 + r) * Hq + h]) : 0.f;
      }
      if (!direct) {
        const int64_t xrw = ((st + qrow) * Hq + h) * DV;
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          const bf16x8 xh = *(const bf16x8 *)(a.XH + xrw + 16 * i + 8 * hh);
          const bf16x8 xl = *(const bf16x8 *)(a.XL + xrw + 16 * i + 8 * hh);
          dp = mma32(xh, vh[i], dp);
          dp = mma32(xl, vh[i], dp);
          dp = mma32(xh, vl[i], dp);
        }
      } else {
        float t[16];
        direct_dp<DV, F32IN, false>(a.delta, a.sig, a.Gl2, a.v, Hq, Hkv, st, c, h, L, q0, kb, hh, n, t);
#pragma unroll
        for (int j = 0; j < 16; ++j) dp[j] = t[j];
      }
      f16x8 dsf[2];
      bf16x8 ph[2], plo[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dsf[u][i] = (_Float16)(p[8 * u + i] * dp[8 * u + i]);
          split_bf16(p[8 * u + i], ph[u], plo[u], i);
        }
      const int64_t qtb = ((int64_t)gc * Hq + h) * DK * CB + 32 * wave;
      const int64_t xtb = ((int64_t)gc * Hq + h) * DV * CB + 32 * wave;
      if (!direct) {
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv) {
          const int col = min(32 * bv + n, DV - 1);  // padded columns are never stored
          f32x16 tmp = zero16();
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 th = *(const bf16x8 *)(a.XTH + xtb + (int64_t)col * CB + 16 * u + 8 * hh);
            const bf16x8 tl = *(const bf16x8 *)(a.XTL + xtb + (int64_t)col * CB + 16 * u + 8 * hh);
            tmp = mma32(ph[u], th, tmp);
            tmp = mma32(ph[u], tl, tmp);
            tmp = mma32(plo[u], th, tmp);
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) accV[bv][j] += gd[bv] * tmp[j];
        }
      } else {
        // exact per-pair decays, written straight to the within-chunk partial
        // (this wave owns these keys): P[q][kj] lives in lane kj, register of q
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv) {
          const int col = 32 * bv + n;
          float t[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) t[j] = 0.f;
#pragma unroll 1
          for (int qq = 0; qq < 32; ++qq) {
            const int qk = q0 + qq;
            const int jsrc = (qq >> 3) * 4 + (qq & 3), hsrc = (qq >> 2) & 1;
            float pj = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) pj = (j == jsrc) ? p[j] : pj;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int kl = acc_row(hh, j);
              const float pv = __shfl(pj, kl + 32 * hsrc);
              const int kj = kb + kl;
              if (col < DV && qk < L && kj <= qk)
                t[j] += pv * fast_exp2(gl_at(qk, col) - gl_at(kj, col)) * a.delta[((st + qk) * Hq + h) * DV + col] *
                        a.sig[(st + qk) * Hq + h];
            }
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kj = kb + acc_row(hh, j);
            if (col < DV && kj < L) {
              const int64_t idx = ((st + kj) * Hkv + c) * DV + col;
              a.dv_i[idx] = (dflag ? a.dv_i[idx] : 0.f) + t[j];
            }
          }
        }
        dflag = true;
      }
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) {
        const int col = min(32 * bk + n, DK - 1);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          accK[bk] = mma32(dsf[u], *(const f16x8 *)(a.Qt + qtb + (int64_t)col * CB + 16 * u + 8 * hh), accK[bk]);
      }
    }
  }
  // dv relative to the end of the key's block: exp2(E(w) - Gl_j).  Each
  // block's inputs are loaded before any of its stores (the compiler cannot
  // tell the buffers apart, so a load after a store would wait for it).
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int col = 32 * bv + n;
    if (col >= DV) continue;
    const float ew = BE[wave + 1][col];
    float gl[16], part[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t idx = ((st + min(kb + acc_row(hh, j), L - 1)) * Hkv + c) * DV + col;
      gl[j] = a.Gl2[idx];
      part[j] = dflag ? a.dv_i[idx] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) a.dv_i[((st + kj) * Hkv + c) * DV + col] = fast_exp2(ew - gl[j]) * accV[bv][j] + part[j];
    }
  }
  // dk after dv: the dv block loads then wait for no earlier stores
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) a.dk_i[((st + kj) * Hkv + c) * DK + col] = a.scale * accK[bk][j];
    }
  }
}

// ---------------------------------------------------------------------------
// dq from key chunks before the query chunk.  Workgroup = 128 query rows of
// one q head (4 waves x 32 rows); key chunks are visited from the first on
// (so the workgroups of a head, started together, read the same key chunk at
// the same time and share it in L2), 32 keys per step copied straight into
// LDS, two steps ahead through three stages: K rows (bf16) for S^T,
// transposed K (fp16) for dS.K, and V scaled to its chunk end (fp16) for
// dP^T.  Many copies come from HBM (the L2 holds only part of a head's key
// chunks), so a step's copies get two steps to land.  The decay product
// between the chunks, gamma_IJ = exp2(Lam[I-1] - Lam[J]), multiplies the
// query-side operand (the scaled dhat rows, kept in registers), rebuilt once
// per key chunk; gamma_IJ itself is computed into LDS at the end of the step
// before the chunk starts, from the Lam row copied with that step's tiles.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 2) k_bwd_dq(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, NBK = DKP / 32;
  using KT = LdsTile<32, DK * 2>;   // K rows of the step
  using TT = LdsTile<DKP, 64>;     // transposed K (dk rows x 32 keys), rows padded to DKP
  using TTD = LdsTile<DK, 64>;
  using VT = LdsTile<32, DV * 2>;  // V rows of the step (scaled to their chunk end)
  // One LDS object for every tile (see the forward kernel).  Three stages:
  // a step's copies are issued two steps ahead.  Each stage also holds the
  // Lam row of the key chunk after the step's (DV doubles, 1 KB reserved).
  constexpr int NBQ = 3;
  constexpr int O_K = 0, O_T = O_K + NBQ * KT::BYTES, O_V = O_T + NBQ * TT::BYTES, O_L = O_V + NBQ * VT::BYTES;
  constexpr int O_G = O_L + NBQ * 1024;
  __shared__ __align__(1024) char smem[O_G + 2 * DV * 4];
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Kts = [&](int b) { return smem + O_T + b * TT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  auto Ls = [&](int b) { return smem + O_L + b * 1024; };
  auto gam = [&](int b) { return (float *)(smem + O_G) + b * DV; };

  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // Items ordered (kv head, sequence, query chunk from the last, q head of
  // the group): the workgroups of one (sequence, kv head) run together on an
  // XCD and walk the same key chunks upward in step, sharing them in L2.
  const int nchunk = pl.counts[0];
  const int idx = xcd_item(nchunk * Hq);
  if (idx < 0) return;
  const int c = uniform(idx / (nchunk * G)), rem = uniform(idx % (nchunk * G));
  const int gci = rem / G, gq = rem % G;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gci);
  const int cbs = uniform(pl.cb128[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int L = uniform(pl.seq_len[s]);
  const int nchs = (L + CB - 1) / CB;
  const int I = nchs - 1 - (gci - cbs);  // longest first within the sequence
  const int hq = c * G + gq;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = I * CB + 32 * wave;
  const int row = r0 + n;
  const bool rv = row < L;
  const float sl2 = a.sl2;

  kfrag qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = rv ? IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();
  const float mbn = rv ? a.mb[(st + row) * Hq + hq] : INFINITY;
  // Rows past the end of the sequence read the last row; their mbn = +inf
  // zeroes their probabilities.
  const _Float16 *dhrow = a.dh + ((st + min(row, L - 1)) * Hq + hq) * DV;
  f16x8 dhf[NSV];
  if (DK < DKP)
    for (int e = tid; e < (DKP - DK) * 64 / 4; e += 256)
      for (int b = 0; b < NBQ; ++b) ((uint32_t *)(Kts(b) + DK * 64))[e] = 0u;
  f32x16 acc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) acc[b] = zero16();

  // gamma_IJ[d] for d = tid (threads tid < DV): Lam[I-1] is fixed, Lam[J] is
  // loaded one step ahead of the chunk that uses it.
  const int dt = min(tid, DV - 1);
  const double lamI = I > 0 ? a.Lam[((int64_t)(cbs + I - 1) * Hkv + c) * DV + dt] : 0.0;
  auto lam_of = [&](int J) { return a.Lam[((int64_t)(cbs + J) * Hkv + c) * DV + dt]; };

  const int nsteps = 4 * I;
  uint32_t ok[KT::NW], ot[TTD::NW], ov[VT::NW];
  KT::lane_offsets(Hkv * DK * 2, wave, lane, ok);
  TTD::lane_offsets(CB * 2, wave, lane, ot);
  VT::lane_offsets(DV * 2, wave, lane, ov);
  auto stage_tile = [&](int k, int b) {
    const int J = k >> 2, u = k & 3;
    const int kt0 = J * CB + 32 * u;
    b = uniform(b);
    if constexpr (!F32IN) {
      const u32x4 rk = rsrc_words((const uint16_t *)a.k + ((st + kt0) * Hkv + c) * DK, (int64_t)32 * Hkv * DK * 2);
#pragma unroll
      for (int t = 0; t < KT::NW; ++t) KT::dma_piece_untracked(Ks(b), rk, ok, t, wave);
    } else {
      for (int p = tid; p < KT::NCH; p += 256) {
        const int r = p / KT::CPR, cc = p % KT::CPR;
        *(f16x8 *)(Ks(b) + KT::off(r, cc)) = IF::load(a.k, ((st + kt0 + r) * Hkv + c) * DK + 8 * cc);
      }
    }
    const int64_t ch = (int64_t)(cbs + J) * Hkv + c;
    const u32x4 rt = rsrc_words(a.Kt + ch * DK * CB + 32 * u, (int64_t)DK * CB * 2);
#pragma unroll
    for (int t = 0; t < TTD::NW; ++t) TTD::dma_piece_untracked(Kts(b), rt, ot, t, wave);
    const u32x4 rv = rsrc_words(a.Vr + (ch * CB + 32 * u) * DV, 32 * DV * 2);
#pragma unroll
    for (int t = 0; t < VT::NW; ++t) VT::dma_piece_untracked(Vs(b), rv, ov, t, wave);
    // Lam row of key chunk J + 1 (clamped): wave w copies bytes 256 w .. +255
    // (zeros past DV doubles)
    const double *lrow = a.Lam + ((int64_t)(cbs + min(J + 1, I - 1)) * Hkv + c) * DV;
    dma4_untracked(Ls(b) + 256 * wave, rsrc_words(lrow, (int64_t)DV * 8), (uint32_t)(256 * wave + 4 * lane));
  };
  // Copies a step issues from inline assembly (the compiler's wait counts do
  // not see them); with fp32 inputs the K rows are stored by the threads
  // instead, and the compiler's own wait for those loads covers every earlier
  // copy.
  constexpr int NCOPYQ = (F32IN ? 0 : KT::NW) + TTD::NW + VT::NW + 1;

  // The unscaled dhat rows stay in registers; they are scaled by gamma_IJ at
  // the top of each key chunk's first step.  Every load of the kernel's own
  // is complete before the first copy is issued, and the loop makes none.
  f16x8 raw[NSV];
#pragma unroll
  for (int i = 0; i < NSV; ++i) raw[i] = *(const f16x8 *)(dhrow + 16 * i + 8 * hh);
  if (nsteps > 0 && tid < DV) gam(0)[tid] = fast_exp2((float)(lamI - lam_of(0)));
  wait_all();
  if (nsteps > 0) {
    stage_tile(0, 0);
    stage_tile(min(1, nsteps - 1), 1);
  }
  wait_vm<NCOPYQ>();  // step 0 has landed
  lds_barrier();
  for (int k = 0; k < nsteps; ++k) {
    const int b = uniform(k % NBQ);
    const bool next_chunk = (k & 3) == 3 && k + 1 < nsteps;
    if ((k & 3) == 0) {  // entered key chunk J: dhat operand times gamma_IJ
      const float *gm = gam((k >> 2) & 1);
#pragma unroll
      for (int i = 0; i < NSV; ++i) {
        const float4 g0 = *(const float4 *)(gm + 16 * i + 8 * hh), g1 = *(const float4 *)(gm + 16 * i + 8 * hh + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dhf[i][e] = (_Float16)((float)raw[i][e] * gv[e]);
      }
    }
    // Same copies on every step (past the last step, the last step's tile
    // again, into a stage nobody reads); step k + 2's stage was last read in
    // step k - 1.
    stage_tile(min(k + 2, nsteps - 1), uniform((k + 2) % NBQ));
    {
      // (Operands are read from LDS per product: batching them needs more
      // registers than this kernel has at two workgroups per CU.)
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const kfrag *)(Ks(b) + KT::off(n, 2 * i + hh)), qf[i], sc);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)(Vs(b) + VT::off(n, 2 * i + hh)), dhf[i], dp);
      f16x8 dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 8 * u + i;
          dsf[u][i] = (_Float16)(fast_exp2(sc[j] * sl2 - mbn) * dp[j]);
        }
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[bk] = mma32(dsf[u], *(const f16x8 *)(Kts(b) + TT::off(32 * bk + n, 2 * u + hh)), acc[bk]);
    }
    // gamma of the next chunk, into the other buffer (its last readers passed
    // the barrier that began this chunk).
    if (next_chunk && tid < DV)
      gam(((k >> 2) + 1) & 1)[tid] = fast_exp2((float)(lamI - ((const double *)Ls(b))[tid]));
    wait_vm<NCOPYQ>();  // step k + 1 has landed (step k + 2's copies stay in flight)
    lds_barrier();
  }
  wait_all();  // copies issued past the last step
  // The block's inputs are loaded before any of its stores (the compiler
  // cannot tell dq and dq_i apart, so interleaving would serialize them).
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int h8 = 0; h8 < 16; h8 += 8) {
      float part[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        part[j] = a.dq_i[((st + min(r0 + acc_row(hh, h8 + j), L - 1)) * Hq + hq) * DK + col];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = r0 + acc_row(hh, h8 + j);
        if (r < L) store_out(a.dq, ((st + r) * Hq + hq) * DK + col, a.scale * acc[bk][h8 + j] + part[j], a.out_f32);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk, dv from query chunks two or more after the key chunk.  Workgroup = the
// 128 keys of one key chunk J and kv head (4 waves x 32 keys), visiting the
// query chunks from the last to J + 2 and, within each, the G query heads of
// the group, 64 query rows per step copied straight into LDS (fp16 Q rows and
// scaled dhat rows only) and computed as two 32-row halves.  With one wave
// per SIMD every instruction of the step's bookkeeping (positions, copy
// addresses, the barrier and the wait for the copies) is issue time the
// products do not hide, so a step spans as many rows as the LDS stages allow.
// The dV and dK products take those rows as their k-major operands through
// the transposing LDS read (tr_frag), so no transposed copy of either is
// stored or moved.
// The decay product between the chunks, gamma_IJ = exp2(Lam[I-1] - Lam[J]),
// enters both products through per-chunk operands: V (.) gamma_IJ (rebuilt
// per query chunk from an LDS copy of the chunk's V rows) for dP, and the
// transposed dhat times gamma_IJ[d] (a per-lane factor, d being the lane's
// output column) for dV, so the accumulators are only ever touched by MFMAs.
// gamma_IJ is computed into LDS during the step before its chunk.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 1) k_bwd_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, DVP = Pad32<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  constexpr int NB = 2;             // LDS stages
  constexpr int DIST = NB - 1;      // steps copied ahead of the one computed
  constexpr int RS = 64;            // query rows per step (two halves of 32)
  using QT = LdsTile<RS, DK * 2>;   // Q rows of the step (fp16)
  using DR = LdsTile<RS, DV * 2>;   // scaled dhat rows (fp16)
  using VRT = LdsTile<CB, DV * 2>;  // the key chunk's V rows, scaled to the chunk end
  // Loads a step issues after its copies' predecessors: the copies themselves
  // (fixed per wave) and nothing else, so waiting for the next step's copies
  // is waiting until this many are left in flight.
  constexpr int NCOPY = QT::NW + DR::NW + 1;
  // One LDS object for every tile (see the forward kernel).  The transposed
  // operands of the dV and dK products are read from the row tiles with the
  // transposing LDS load (tr_frag).
  constexpr int O_Q = 0, O_D = O_Q + NB * QT::BYTES;
  constexpr int O_V = O_D + NB * DR::BYTES, O_M = O_V + VRT::BYTES, O_G = O_M + NB * 256, O_GH = O_G + 2 * DVP * 4;
  __shared__ __align__(1024) char smem[O_GH + 2 * DVP * 2];
  auto Qs = [&](int b) { return smem + O_Q + b * QT::BYTES; };
  auto Ds = [&](int b) { return smem + O_D + b * DR::BYTES; };
  auto Ms = [&](int b) { return (float *)(smem + O_M + b * 256); };  // 64 floats, 32 used
  auto gam = [&](int b) { return (float *)(smem + O_G) + b * DVP; };
  auto gamh = [&](int b) { return (_Float16 *)(smem + O_GH) + b * DVP; };  // the same, fp16

  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // Items ordered (kv head, sequence, key chunk): the workgroups of one
  // (sequence, kv head) run together on an XCD and walk the same query
  // chunks downward in step, sharing them in L2.
  const int nchunk = pl.counts[0];
  const int idx = xcd_item(nchunk * Hkv);
  if (idx < 0) return;
  const int c = uniform(idx / nchunk), gci = uniform(idx % nchunk);
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gci);
  const int cbs = uniform(pl.cb128[s]);
  const int J = gci - cbs;
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int L = uniform(pl.seq_len[s]);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = J * CB + 32 * wave;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;

  const int nch = (L + CB - 1) / CB;
  const int I0 = J + 2, I1 = nch - 1;                  // query chunks visited: I1 down to I0
  const int ns1 = (L - I1 * CB + RS - 1) / RS;          // slices of the last (possibly partial) chunk
  const int nsteps = I0 <= I1 ? G * ns1 + (CB / RS) * G * (I1 - I0) : 0;
  // The key as an fp16 operand: Q is staged as fp16 (q converted once, exact
  // for |q| in [2^-14, 65504]), so the score product runs in fp16 and equals
  // the bf16 one for such inputs.
  f16x8 kf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const kfrag kr = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[i][e] = (_Float16)(float)kr[e];
  }
  f32x16 accK[NBK], accV[NBV];
#pragma unroll
  for (int b = 0; b < NBK; ++b) accK[b] = zero16();
#pragma unroll
  for (int b = 0; b < NBV; ++b) accV[b] = zero16();

  // Step position: query chunk I, query head of the group gq, 32-row slice
  // u, and the ordinal of the chunk among the visited ones (0 for I1).
  struct Pos {
    int I, gq, u, ord;
  };
  auto advance = [&](Pos &p) {
    if (++p.u == (p.I == I1 ? ns1 : CB / RS)) {
      p.u = 0;
      if (++p.gq == G) {
        p.gq = 0;
        --p.I;
        ++p.ord;
      }
    }
  };
  // Rows past the end of the sequence read as zeros (see the probabilities).
  uint32_t oq[QT::NW], od[DR::NW];
  QT::lane_offsets(Hq * DK * 2, wave, lane, oq);
  DR::lane_offsets(Hq * DV * 2, wave, lane, od);
  auto stage_tile = [&](const Pos &p, int b) {
    const int h = c * G + p.gq;
    const int qt0 = p.I * CB + RS * p.u;
    const int64_t qr = (st + qt0) * Hq + h;
    const int nrow = L - qt0;
    QT::dma(Qs(b), make_rsrc(a.Q16 + qr * DK, (int64_t)nrow * Hq * DK * 2), oq, wave);
    DR::dma(Ds(b), make_rsrc(a.dh + qr * DV, (int64_t)nrow * Hq * DV * 2), od, wave);
    // lane r fills Ms[r] (every wave, the same bytes)
    dma4(Ms(b), make_rsrc(a.mb + qr, (int64_t)nrow * Hq * 4), (uint32_t)lane * Hq * 4);
  };

  // gamma_IJ[d] for d = tid (threads tid < DV).
  const int dt = min(tid, DV - 1);
  const double lamJ = a.Lam[((int64_t)(cbs + J) * Hkv + c) * DV + dt];
  auto lam_of = [&](int I) { return a.Lam[((int64_t)(cbs + I - 1) * Hkv + c) * DV + dt]; };

  Pos cur{I1, 0, 0, 0}, ahead{I1, 0, 0, 0};  // the step computed, the step being copied
  if (nsteps > 0) {
    uint32_t ovr[VRT::NW];
    VRT::lane_offsets(DV * 2, wave, lane, ovr);
    VRT::dma(smem + O_V, make_rsrc(a.Vr + ((int64_t)(cbs + J) * Hkv + c) * CB * DV, (int64_t)CB * DV * 2), ovr, wave);
    if (tid < DV) {
      const float g0 = fast_exp2((float)(lam_of(I1) - lamJ));
      gam(0)[tid] = g0;
      gamh(0)[tid] = (_Float16)g0;
    }
    for (int k = 0; k < DIST; ++k) {  // steps 0 .. DIST - 1 (the last step again past the end)
      stage_tile(ahead, k);
      if (k + 1 < nsteps) advance(ahead);
    }
    // `ahead` is now step DIST (or the last step)
  }
  wait_all();
  __syncthreads();

  f16x8 vf[NSV];        // key-side dP operand V (.) gamma_IJ, rebuilt per query chunk
  _Float16 gh[NBV];     // gamma_IJ of the lane's dV output columns
  int prev_ord = -1;
  for (int k = 0; k < nsteps; ++k) {
    const int b = k % NB;
    const int I = cur.I, qt0 = I * CB + RS * cur.u;
    if (cur.ord != prev_ord) {  // first step of a query chunk
      prev_ord = cur.ord;
      const float *gm = gam(cur.ord & 1);
      const _Float16 *gmh = gamh(cur.ord & 1);
      // every read of the rebuild first (no copies are in flight here: the
      // previous step waited for all of them)
      f16x8 r[NSV], gv[NSV];
      float gcol[NBV];
#pragma unroll
      for (int i = 0; i < NSV; ++i) {
        r[i] = *(const f16x8 *)(smem + O_V + VRT::off(32 * wave + n, 2 * i + hh));
        gv[i] = *(const f16x8 *)(gmh + 16 * i + 8 * hh);
      }
#pragma unroll
      for (int i = 0; i < NBV; ++i) gcol[i] = gm[min(32 * i + n, DV - 1)];
#pragma unroll
      for (int i = 0; i < NSV; ++i) vf[i] = r[i] * gv[i];
      // gamma of the lane's dV column 32 bv + n
#pragma unroll
      for (int i = 0; i < NBV; ++i) gh[i] = 32 * i + n < DV ? (_Float16)gcol[i] : (_Float16)0.f;
    }
    // The position after this step: its chunk's gamma is due at the end of
    // this step if the chunk changes.
    Pos nxt = cur;
    if (k + 1 < nsteps) advance(nxt);
    const bool next_chunk = nxt.ord != cur.ord;
    double lamI = 0.0;
    // Two 32-row halves in turn, kept as a loop (unrolled, the compiler
    // interleaves the halves' live ranges and spends vector instructions moving
    // values between register files); the second half is skipped when it lies
    // past the sequence end.
#pragma unroll 1
    for (int h2 = 0; h2 < 2; ++h2) {
      if (h2 == 1 && qt0 + 32 >= L) break;
      // Exponent offsets of the step's rows: read before the step's copies are
      // issued (an LDS read after them can make the compiler wait for them) and
      // used only after the products.
      float4 mq[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) mq[q4] = *(const float4 *)&Ms(b)[32 * h2 + 8 * q4 + 4 * hh];
      {
        // S[q][key] and dP[q][key]: lane = key, register j = query acc_row(hh, j).
        // Operands of a group of products are read from LDS in one batch (one
        // wait for all of them rather than one per product).
        f16x8 qa[NS];
        f16x8 da[NSV];
#pragma unroll
        for (int i = 0; i < NS; ++i) qa[i] = *(const f16x8 *)(Qs(b) + QT::off(32 * h2 + n, 2 * i + hh));
#pragma unroll
        for (int i = 0; i < NSV; ++i) da[i] = *(const f16x8 *)(Ds(b) + DR::off(32 * h2 + n, 2 * i + hh));
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sc = zero16(), dp = zero16();
#pragma unroll
        for (int i = 0; i < NS; ++i) sc = mma32(qa[i], kf[i], sc);
#pragma unroll
        for (int i = 0; i < NSV; ++i) dp = mma32(da[i], vf[i], dp);
        // While the products run, between them: the copies of step k + DIST
        // (the last step again near the end, so that every step issues the
        // same copies; `ahead` is that step's position), the next chunk's Lam
        // row, the step's row offsets and the dV / dK operands.
        f16x8 ta[NBV][2], tq[NBK][2];  // dhat^T and Q^T operands (k = query, in the result tiles' order)
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) ta[bv][uu] = tr_frag<DR>(Ds(b), 32 * h2 + 16 * uu, 32 * bv, lane);
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) tq[bk][uu] = tr_frag<QT>(Qs(b), 32 * h2 + 16 * uu, 32 * bk, lane);
        if (h2 == 0) {
          stage_tile(ahead, (k + DIST) % NB);
          if (k + DIST + 1 < nsteps) advance(ahead);
          lamI = lam_of(nxt.I);
        }
        constexpr int NTR = 4 * (NBV + NBK);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x100, (NTR + NS - 1) / NS, 0);  // transposing LDS reads
        }
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy / global load
        }
        __builtin_amdgcn_sched_barrier(0);
        // Rows past the end of the sequence need no mask: their Q, dhat and
        // row-offset copies read as zeros, so their probability is exp2(0) = 1
        // (finite), their dP and hence dS are 0, and the dV product meets it
        // only against their zero dhat rows.
        f16x8 pf[2], dsf[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float mv[4] = {mq[q4].x, mq[q4].y, mq[q4].z, mq[q4].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * q4 + e;
            const float pv = fast_exp2(sc[j] * sl2 - mv[e]);
            pf[j >> 3][j & 7] = (_Float16)pv;
            dsf[j >> 3][j & 7] = (_Float16)(pv * dp[j]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) accV[bv] = mma32(pf[uu], ta[bv][uu] * gh[bv], accV[bv]);
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) accK[bk] = mma32(dsf[uu], tq[bk][uu], accK[bk]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // gamma of the next chunk, into the other buffer (its last readers passed
    // the barrier that ended the first step of the previous chunk).
    if (next_chunk && tid < DV) {
      const float gn = fast_exp2((float)(lamI - lamJ));
      gam(nxt.ord & 1)[tid] = gn;
      gamh(nxt.ord & 1)[tid] = (_Float16)gn;
    }
    cur = nxt;
    wait_vm<(DIST - 1) * NCOPY>();  // the copies of step k + 1 have landed
    lds_barrier();
  }
  if (kb >= L) return;
  // epilogue: dk, dv (inter part scaled to the key: exp(Gl_end(J) - Gl_key)), dG = qside - v (.) dv.
  // The compiler cannot tell the output and input buffers apart, so a load
  // placed after a store waits for it: each block's inputs are loaded one
  // block ahead, before the previous block's stores.
  const int tend = min((J + 1) * CB, L) - 1;
  auto kidx = [&](int j) { return min(kb + acc_row(hh, j), L - 1); };
  float pk[2][16];
  auto load_dk = [&](int bk, float (&part)[16]) {
    const int col = min(32 * bk + n, DK - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) part[j] = a.dk_i[((st + kidx(j)) * Hkv + c) * DK + col];
  };
  load_dk(0, pk[0]);
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    if (bk + 1 < NBK) load_dk(bk + 1, pk[(bk + 1) & 1]);
    const int col = 32 * bk + n;
    if (col < DK)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (kj < L) store_out(a.dk, ((st + kj) * Hkv + c) * DK + col, a.scale * accK[bk][j] + pk[bk & 1][j], a.out_f32);
      }
  }
  float in[2][4][16];  // [slot][prefix sum, partial, qside, v][row]
  float gend[NBV];
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) gend[bv] = a.Gl2[((st + tend) * Hkv + c) * DV + min(32 * bv + n, DV - 1)];
  auto load_dv = [&](int bv, float (&x)[4][16]) {
    const int col = min(32 * bv + n, DV - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t idx = ((st + kidx(j)) * Hkv + c) * DV + col;
      x[0][j] = a.Gl2[idx];
      x[1][j] = a.dv_i[idx];
      x[2][j] = a.qside[idx];
      x[3][j] = load_in(a.v, idx, F32IN);
    }
  };
  load_dv(0, in[0]);
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    if (bv + 1 < NBV) load_dv(bv + 1, in[(bv + 1) & 1]);
    const int col = 32 * bv + n;
    if (col < DV)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (kj < L) {
          const int64_t idx = ((st + kj) * Hkv + c) * DV + col;
          const float(&x)[4][16] = in[bv & 1];
          const float dvv = fast_exp2(gend[bv] - x[0][j]) * accV[bv][j] + x[1][j];
          store_out(a.dv, idx, dvv, a.out_f32);
          a.dG[idx] = x[2][j] - x[3][j] * dvv;
        }
      }
  }
}

template <int DK, int DV>
hipError_t launch_bwd_dk_dv(BwdKernel kind, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st) {
#define FIX_BWD_LAUNCH(KERN)                                                                  \
  if (f32in) hipLaunchKernelGGL((KERN<DK, DV, true>), grid, dim3(256), 0, st, a);             \
  else hipLaunchKernelGGL((KERN<DK, DV, false>), grid, dim3(256), 0, st, a);
  switch (kind) {
    case BK_INTRA_DQ: FIX_BWD_LAUNCH(k_bwd_intra_dq); break;
    case BK_INTRA_DKV: FIX_BWD_LAUNCH(k_bwd_intra_dkv); break;
    case BK_DQ: FIX_BWD_LAUNCH(k_bwd_dq); break;
    case BK_DKV: FIX_BWD_LAUNCH(k_bwd_dkv); break;
  }
#undef FIX_BWD_LAUNCH
  return hipGetLastError();
}

template <int DK>
hipError_t launch_bwd_dk(BwdKernel kind, int dv, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st) {
  switch (dv) {
    case 16: return launch_bwd_dk_dv<DK, 16>(kind, f32in, a, grid, st);
    case 32: return launch_bwd_dk_dv<DK, 32>(kind, f32in, a, grid, st);
    case 64: return launch_bwd_dk_dv<DK, 64>(kind, f32in, a, grid, st);
    case 128: return launch_bwd_dk_dv<DK, 128>(kind, f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fix
