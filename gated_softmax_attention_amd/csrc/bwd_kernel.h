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
template <int V> struct IC { static constexpr int value = V; };  // a compile-time int argument

// The gradient reaching x (delta) of element (row, d), row = token * Hq +
// head, recomputed as the preprocess forms it (see bwd_prep.hip): dn = dO (.)
// z, and with the norm delta = rstd (dn w - x rstd prj), prj the row's
// stored projection.  Only the exact-decay paths below need it.
struct DeltaSrc {
  const float *x, *rstd, *prj;
  const void *dO, *z, *w;
  int o_norm;
};
template <int DV, bool F32IN> __device__ inline float delta_at(const DeltaSrc &s, int64_t row, int d) {
  const int64_t i = row * DV + d;
  const float dn = load_in(s.dO, i, F32IN) * (s.z ? load_in(s.z, i, F32IN) : 1.f);
  if (!s.o_norm) return dn;
  const float rs = s.rstd[row], wv = s.w ? load_in(s.w, d, F32IN) : 1.f;
  return rs * (dn * wv - s.x[i] * rs * s.prj[row]);
}

// Exact per-pair decays for a diagonal 32x32 block whose gate range exceeds
// 2^BGUARD (rare): dP for the pairs held by this lane, evaluated directly.
// Register j of lane (hh, n) holds the pair (row q0 + rowof(j, n), key k0 + keyof(j, n)).
// (Arguments by value: passing the kernel's argument struct by reference
// would force a stack copy of it in every kernel that can call this.)
template <int DV, bool F32IN, bool ROW_IS_LANE>
__device__ __noinline__ void direct_dp(const float *x, const float *rstd, const float *prj, const void *dO,
                                       const void *z, const void *w, int o_norm, const float *sig, const float *Gl2,
                                       const void *v, int Hq, int Hkv, int64_t st, int c, int h, int L, int q0, int k0,
                                       int hh, int n, float *dp) {
  const DeltaSrc ds{x, rstd, prj, dO, z, w, o_norm};
  for (int j = 0; j < 16; ++j) {
    const int r = ROW_IS_LANE ? n : acc_row(hh, j);
    const int kk = ROW_IS_LANE ? acc_row(hh, j) : n;
    const int qi = q0 + r, kj = k0 + kk;
    float t = 0.f;
    if (qi < L && kj <= qi) {
      const int64_t row = (st + qi) * Hq + h;
      const float sg = sig[row];
      for (int d = 0; d < DV; ++d) {
        const float gq = Gl2[((st + qi) * Hkv + c) * DV + d], gk = Gl2[((st + kj) * Hkv + c) * DV + d];
        t += delta_at<DV, F32IN>(ds, row, d) * sg * fast_exp2(gq - gk) * load_in(v, ((st + kj) * Hkv + c) * DV + d, F32IN);
      }
    }
    dp[j] = t;
  }
}

// ---------------------------------------------------------------------------
// Within-chunk contributions to dq.  Workgroup = one 128-chunk of one q
// head; query block p (rows c0 + 32p .. +31) is shared by wave p (A) and wave
// p + 4 (B), which the hardware places on the same SIMD.  Key blocks b are
// copied into LDS one per step: K, V scaled to the end of its block
// (VE), and for the diagonal block of pair b its V relative to the token
// before it and query block b's dhat (bf16 hi / lo each).  K is staged twice:
// as rows (bf16, fp16 for fp32 inputs) for S^T and as its transposed fp16
// tile (three stages: B reads it one step late) for dQ.  With E(b) the
// chunk-local log2 gate prefix at the end of block b (E(-1) = 0), the decay
// of a pair in query block a > b splits as
//     exp2(Gl_i - E(a-1)) * exp2(E(a-1) - E(b)) * exp2(E(b) - Gl_j),
// all three <= 1: the first is the prepared block-relative dhat (X16), the
// middle one gamma_ab multiplies B's dhat operand per channel, the last is
// VE.  On the diagonal block the split is at the token before it: the key
// side exp2(E(a-1) - Gl_j) >= 1 needs fp32 range and is multiplied as bf16x3
// (hi*hi + hi*lo + lo*hi); a block whose gate range exceeds 2^BGUARD is
// evaluated with direct per-pair decays.
//   A, step b: S^T = K Q^T (lane = query row), P = exp2(S sl2 - m) (fp32
//              into LDS); the copies of step b+1's K rows and tile.
//   B, step b: dS_{b-1} = P_{b-1} (LDS) (.) the dP_{b-1} it kept, dQ +=
//              dS_{b-1} K_{b-1}; dP_b^T = V (dhat (.) gamma)^T; the copies of
//              step b+1's V rows and diagonal tiles.
// ---------------------------------------------------------------------------
// The diagonal block of query block r0 with exact per-pair decays (its gate
// range beyond 2^BGUARD; rare), for one wave, from global memory, after the
// wave has stored its dq rows: the block's dQ is added to them (the same
// lanes wrote them).  A function of its own so that the kernel's loops keep
// their registers.
template <int DK, int DV, bool F32IN>
__device__ __noinline__ void near_exact_diag_dq(const float *x, const float *rstd, const float *prj, const void *dO,
                                                const void *z, const void *w, int o_norm, const float *sig,
                                                const float *Gl2, const void *v, const void *kp, const void *qp,
                                                const _Float16 *Kt, const float *mb, float *dq_i, float scale, float sl2,
                                                int Hq, int Hkv, int64_t st, int c, int hq, int L, int gc, int r0) {
  using IF = InFrag<F32IN>;
  constexpr int NS = DK / 16, NBK = Pad32<DK>::value / 32;
  const int lane = threadIdx.x & 63, hh = lane >> 5, n = lane & 31;
  const int row = r0 + n, kb = r0;
  const int key = min(kb + n, L - 1), qrow = min(row, L - 1);
  float t[16];
  direct_dp<DV, F32IN, true>(x, rstd, prj, dO, z, w, o_norm, sig, Gl2, v, Hq, Hkv, st, c, hq, L, r0, kb, hh, n, t);
  // S^T[key][row]: lane = row, register j = key acc_row(hh, j)
  f32x16 sc = zero16();
#pragma unroll
  for (int i = 0; i < NS; ++i)
    sc = mma32(IF::load(kp, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh),
               IF::load(qp, ((st + qrow) * Hq + hq) * DK + 16 * i + 8 * hh), sc);
  const float mbn = row < L ? mb[(st + row) * Hq + hq] : INFINITY;
  f16x8 dsf[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * u + i;
      dsf[u][i] = (_Float16)(acc_row(hh, j) > n ? 0.f : fast_exp2(sc[j] * sl2 - mbn) * t[j]);
    }
  // dQ[row][dk] += dS[row][key] K[key][dk], K from its transposed tile
  const _Float16 *ktile = Kt + ((int64_t)gc * Hkv + c) * DK * CB + (r0 % CB);
#pragma unroll 1
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = min(32 * bk + n, DK - 1);  // padded columns are never stored
    f32x16 dacc = zero16();
#pragma unroll
    for (int u = 0; u < 2; ++u) dacc = mma32(dsf[u], *(const f16x8 *)(ktile + (int64_t)col * CB + 16 * u + 8 * hh), dacc);
    if (32 * bk + n < DK)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = r0 + acc_row(hh, j);
        if (r < L) dq_i[((st + r) * Hq + hq) * DK + col] += scale * dacc[j];
      }
  }
}

// Minimum waves per SIMD (HIP's second launch bound) of the 512-thread
// kernels: at head dims up to 32 their LDS holds two workgroups per CU, i.e.
// four waves per SIMD, which caps a wave at 128 VGPRs (a few registers more
// leave one workgroup per CU); otherwise one.
constexpr int small_head_waves(int dk, int dv) { return (dk <= 32 && dv <= 32) ? 4 : 1; }

template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(512, small_head_waves(DK, DV)) k_bwd_intra_dq(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, NBK = DKP / 32;
  using KT = LdsTile<32, DK * 2>;  // K rows of the key block
  using TT = LdsTile<DKP, 64>;     // transposed K (dk rows x 32 keys, key_pos order), rows padded to DKP
  using TTD = LdsTile<DK, 64>;
  using VT = LdsTile<32, DV * 2>;  // VE rows of the key block; the diagonal's bf16 hi / lo rows
  constexpr int PX = 4 * 64 * 16;  // one pair's P of a step: [j / 4][lane] float4
  // One LDS object for every tile (see the forward kernel).  Per stage, for
  // the diagonal block of the pair whose block it is: the key block's V
  // relative to the token before it and the same block's block-relative
  // dhat rows (bf16 hi, lo each), at fixed distances from the VE tile.
  constexpr int O_K = 0, O_T = O_K + 2 * KT::BYTES, O_V = O_T + 3 * TT::BYTES, O_P = O_V + 10 * VT::BYTES;
  constexpr int O_E = O_P + 2 * 4 * PX, O_GW = O_E + 5 * DV * 4;
  __shared__ __align__(1024) char smem[O_GW + 4 * DV * 2];
  float(*BE)[DV] = (float(*)[DV])(smem + O_E);  // BE[b + 1] = E(b), BE[0] = 0

  const Plan &pl = a.plan;
  const int gc = blockIdx.x, hq = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isA = wave < 4;
  const int p = wave & 3;
  _Float16 *gw = (_Float16 *)(smem + O_GW) + p * DV;  // B's gamma of the step, per channel (fp16)
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = uniform((gc - pl.cb128[s]) * CB);
  const int L = uniform(pl.seq_len[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int Hq = a.Hq, Hkv = a.Hkv, c = hq / (Hq / Hkv);
  const int nsteps = min(4, (L - c0 + 31) / 32);  // query (and key) blocks present in the chunk
  const int r0 = c0 + 32 * p;
  const int row = r0 + n;
  const bool active = p < nsteps;
  const bool rv = active && row < L;
  const float sl2 = a.sl2;
  auto gl_at = [&](int tok, int d) { return a.Gl2[((st + tok) * Hkv + c) * DV + d]; };
  const uint32_t sbase = lds_addr(smem);

  // Copies of key block b.  Rows past the sequence end read as zeros: off
  // the diagonal every key is valid, on the diagonal the keys past the end
  // meet only masked pairs.
  uint32_t ok[KT::NW], ot[TTD::NW], ov[VT::NW], oxq[VT::NW];
  KT::lane_offsets(Hkv * DK * 2, p, lane, ok);
  TTD::lane_offsets(CB * 2, p, lane, ot);
  VT::lane_offsets(Hkv * DV * 2, p, lane, ov);
  VT::lane_offsets(Hq * DV * 2, p, lane, oxq);
  auto stage_tile = [&](int b) {
    const int kb = c0 + 32 * b;
    const int64_t kr = (st + kb) * Hkv + c;
    const int nrow = L - kb;
    if (isA) {
      char *ks = smem + O_K + (b & 1) * KT::BYTES;
      if constexpr (!F32IN) {
        const u32x4 rk = rsrc_words((const uint16_t *)a.k + kr * DK, (int64_t)nrow * Hkv * DK * 2);
#pragma unroll
        for (int t = 0; t < KT::NW; ++t) KT::dma_piece_untracked(ks, rk, ok, t, p);
      } else {
        for (int q = tid; q < KT::NCH; q += 256) {
          const int r = q / KT::CPR, cc = q % KT::CPR;
          *(f16x8 *)(ks + KT::off(r, cc)) = IF::load(a.k, ((st + min(kb + r, L - 1)) * Hkv + c) * DK + 8 * cc);
        }
      }
      const u32x4 rt = rsrc_words(a.Kt + ((int64_t)gc * Hkv + c) * DK * CB + 32 * b, (int64_t)DK * CB * 2);
#pragma unroll
      for (int t = 0; t < TTD::NW; ++t) TTD::dma_piece_untracked(smem + O_T + (b % 3) * TT::BYTES, rt, ot, t, p);
    } else {
      char *v0 = smem + O_V + (b & 1) * VT::BYTES;  // VE, BH, BL, XH, XL at 2 tiles' distance each
      const int64_t xq = ((st + kb) * Hq + hq) * DV;  // query block b = key block b
      const u32x4 rv = rsrc_words(a.VE + kr * DV, (int64_t)nrow * Hkv * DV * 2);
      const u32x4 rbh = rsrc_words(a.VBH + kr * DV, (int64_t)nrow * Hkv * DV * 2);
      const u32x4 rbl = rsrc_words(a.VBL + kr * DV, (int64_t)nrow * Hkv * DV * 2);
      const u32x4 rxh = rsrc_words(a.XH + xq, (int64_t)nrow * Hq * DV * 2);
      const u32x4 rxl = rsrc_words(a.XL + xq, (int64_t)nrow * Hq * DV * 2);
#pragma unroll
      for (int t = 0; t < VT::NW; ++t) {
        VT::dma_piece_untracked(v0, rv, ov, t, p);
        VT::dma_piece_untracked(v0 + 2 * VT::BYTES, rbh, ov, t, p);
        VT::dma_piece_untracked(v0 + 4 * VT::BYTES, rbl, ov, t, p);
        VT::dma_piece_untracked(v0 + 6 * VT::BYTES, rxh, oxq, t, p);
        VT::dma_piece_untracked(v0 + 8 * VT::BYTES, rxl, oxq, t, p);
      }
    }
  };

  // Prologue: the block-end gate values (E), the row operand of the wave's
  // role (A: q as fp16 and the row offset; B: the block-relative dhat) and
  // the first step's copies, all issued before one wait.
  constexpr int NBE = (5 * DV + 511) / 512;
  float be[NBE];
#pragma unroll
  for (int t = 0; t < NBE; ++t) {
    const int e = tid + 512 * t, b = e / DV - 1, d = e % DV;
    be[t] = e < 5 * DV && b >= 0 ? gl_at(min(c0 + 32 * b + 31, L - 1), d) : 0.f;
  }
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  if (DK < DKP)  // the transposed tiles' padding rows
    for (int e = tid; e < (DKP - DK) * 64 / 4; e += 512)
      for (int b = 0; b < 3; ++b) ((uint32_t *)(smem + O_T + b * TT::BYTES + DK * 64))[e] = 0u;
  kfrag qf[NS];  // A: the row's q
#pragma unroll
  for (int i = 0; i < NS; ++i) qf[i] = IF::zero();
  f16x8 rop[NSV];  // B: the row's block-relative dhat (k = channel)
#pragma unroll
  for (int i = 0; i < NSV; ++i) rop[i] = zf;
  float mbn = INFINITY;
  if (isA) {
    if (rv) {
#pragma unroll
      for (int i = 0; i < NS; ++i) qf[i] = IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh);
      mbn = a.mb[(st + row) * Hq + hq];
    }
  } else if (rv) {
#pragma unroll
    for (int i = 0; i < NSV; ++i) rop[i] = *(const f16x8 *)(a.X16 + ((st + row) * Hq + hq) * DV + 16 * i + 8 * hh);
  }
  if (nsteps > 0) stage_tile(0);
  wait_all();
#pragma unroll
  for (int t = 0; t < NBE; ++t) {
    const int e = tid + 512 * t, b = e / DV - 1, d = e % DV;
    if (e < 5 * DV) BE[b + 1][d] = be[t];
  }
  __syncthreads();
  // Whether a block's diagonal needs exact per-pair decays (its gate range
  // beyond 2^BGUARD): this pair's.
  bool direct;
  {
    float rng = 0.f;
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[p][d] - BE[p + 1][d]);
      }
    direct = __any(rng > BGUARD);
  }
  auto act_of = [&](int b) { return active && (b < p || (b == p && !direct)); };
  const uint32_t apx = sbase + O_P + p * PX + 16 * lane;  // this lane's P exchange slot

  if (isA) {
    uint32_t ak[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) ak[i] = sbase + O_K + KT::off(n, min(2 * i + hh, KT::CPR - 1));
    const uint32_t apx_ = opaque(apx);
    for (int b = 0; b < nsteps; ++b) {
      wait_all();
      __syncthreads();  // step b's tiles landed; step b - 1's readers are done
      if (b + 1 < nsteps) stage_tile(b + 1);
      if (!act_of(b)) continue;
      // S^T[key][row]: lane = row, register j = key acc_row(hh, j)
      f32x16 sc = zero16();
      {
        const uint32_t so = (b & 1) * KT::BYTES;
        kfrag fk[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) fk[i] = __builtin_bit_cast(kfrag, lds_row16p(lds_at(ak[i]) + so));
#pragma unroll
        for (int i = 0; i < NS; ++i) sc = mma32(fk[i], qf[i], sc);
      }
      const bool diag = b == p;
      float pv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pv[j] = diag && acc_row(hh, j) > n ? 0.f : fast_exp2(sc[j] * sl2 - mbn);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *(__attribute__((address_space(3))) f32x4 *)(lds_at(apx_ + (b & 1) * 4 * PX) + 1024 * j4) =
            f32x4{pv[4 * j4], pv[4 * j4 + 1], pv[4 * j4 + 2], pv[4 * j4 + 3]};
    }
    wait_all();
    __syncthreads();  // the barrier B's last dQ step waits at
    return;
  }

  // B: per-lane LDS addresses in stage 0: V row fragments (dP^T; the
  // diagonal's tiles lie at fixed distances) and the transposed K fragments
  // per output block and k slice (dQ)
  uint32_t av[NSV], akt[NBK][2];
#pragma unroll
  for (int i = 0; i < NSV; ++i) av[i] = sbase + O_V + VT::off(n, min(2 * i + hh, VT::CPR - 1));
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
    for (int u = 0; u < 2; ++u) akt[bk][u] = sbase + O_T + TT::off(32 * bk + n, 2 * u + hh);
  const uint32_t apx_ = opaque(apx);
  f32x16 acc[NBK];
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) acc[bk] = zero16();
  f32x16 dpk = zero16();  // dP^T of the previous step
  // dS of step bb from A's P (LDS) and the kept dP, then dQ += dS K_bb with
  // K from its transposed tile
  auto dq_step = [&](int bb) {
    f16x8 dsf[2];
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const f32x4 pq = *(const __attribute__((address_space(3))) f32x4 *)(lds_at(apx_ + (bb & 1) * 4 * PX) + 1024 * j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 4 * j4 + e;
        dsf[j >> 3][j & 7] = (_Float16)(pq[e] * dpk[j]);
      }
    }
    const uint32_t so = (bb % 3) * TT::BYTES;
    f16x8 tk[2][NBK];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) tk[u][bk] = lds_row16p(lds_at(akt[bk][u]) + so);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) acc[bk] = mma32(dsf[u], tk[u][bk], acc[bk]);
  };
  for (int b = 0; b < nsteps; ++b) {
    wait_all();
    __syncthreads();  // step b's tiles landed; step b - 1's readers are done
    if (b + 1 < nsteps) stage_tile(b + 1);
    if (b > 0 && act_of(b - 1)) dq_step(b - 1);
    if (!act_of(b)) continue;
    const uint32_t so = (b & 1) * VT::BYTES;
    // dP^T[key][row] (lane = row, register j = key acc_row(hh, j))
    f32x16 dp = zero16();
    if (b == p) {
      // split at the token before the block: V and dhat as bf16 hi / lo (bf16x3)
#pragma unroll
      for (int i = 0; i < NSV; ++i) {
        const uint32_t ai = av[i] + so;
        const bf16x8 vh = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 2 * VT::BYTES));
        const bf16x8 vl = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 4 * VT::BYTES));
        const bf16x8 xh = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 6 * VT::BYTES));
        const bf16x8 xl = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 8 * VT::BYTES));
        dp = mma32(vh, xh, dp);
        dp = mma32(vh, xl, dp);
        dp = mma32(vl, xh, dp);
      }
    } else {
      // gamma_pb[d] = exp2(E(p - 1) - E(b)) <= 1 depends on the channel only:
      // each lane evaluates two channels into the wave's table (fp16), then
      // every lane reads the channels it needs (a wave's LDS accesses
      // complete in order) and scales its dhat operand with packed products
#pragma unroll
      for (int t = 0; t < (DV + 63) / 64; ++t) {
        const int d = lane + 64 * t;
        if (d < DV) gw[d] = (_Float16)fast_exp2(BE[p][d] - BE[b + 1][d]);
      }
      f16x8 fv[NSV];
#pragma unroll
      for (int i = 0; i < NSV; ++i) fv[i] = lds_row16p(lds_at(av[i]) + so);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(fv[i], rop[i] * *(const f16x8 *)(gw + 16 * i + 8 * hh), dp);
    }
    dpk = dp;
  }
  wait_all();
  __syncthreads();  // A's last P is in LDS
  if (nsteps > 0 && act_of(nsteps - 1)) dq_step(nsteps - 1);
  if (!active) return;
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
  // Diagonal block with exact per-pair decays (gate range beyond 2^BGUARD),
  // added to the stored rows.  (Otherwise the staged loop did it.)
  if (direct)
    near_exact_diag_dq<DK, DV, F32IN>(a.x, a.rstd, a.prj, a.dO, a.z, a.w, a.o_norm, a.sig, a.Gl2, a.v, a.k, a.q, a.Kt,
                                      a.mb, a.dq_i, a.scale, sl2, Hq, Hkv, st, c, hq, L, gc, r0);
}

// The diagonal block of key block kb with exact per-pair decays (its gate
// range beyond 2^BGUARD; rare), for one wave, from global memory, after the
// wave has stored its dk rows: dK is added to the stored rows (the same
// lanes wrote them), dV goes straight into the within-chunk partial.  A
// function of its own so that the kernel's loops keep their registers.
template <int DK, int DV, bool F32IN>
__device__ __noinline__ void near_exact_diag(const float *x, const float *rstd, const float *prj, const void *dO,
                                             const void *z, const void *w, int o_norm, const float *sig,
                                             const float *Gl2, const void *v, const void *kp, const _Float16 *Q16,
                                             const float *mb, float *dv_i, float *dk_i, float scale, float sl2, int Hq,
                                             int Hkv, int G, int64_t st, int c, int L, int kb) {
  const DeltaSrc ds{x, rstd, prj, dO, z, w, o_norm};
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NBK = Pad32<DK>::value / 32, NBV = Pad32<DV>::value / 32;
  const int lane = threadIdx.x & 63, hh = lane >> 5, n = lane & 31;
  const int key = kb + n;
  const bool kv = key < L;
  auto gl_at = [&](int tok, int d) { return Gl2[((st + tok) * Hkv + c) * DV + d]; };
  const int q0 = kb;
  const int qrow = min(q0 + n, L - 1);  // A-operand row of this lane
  for (int gq = 0; gq < G; ++gq) {
    const int h = c * G + gq;
    float dpe[16];
    direct_dp<DV, F32IN, false>(x, rstd, prj, dO, z, w, o_norm, sig, Gl2, v, Hq, Hkv, st, c, h, L, q0, kb, hh, n, dpe);
    f32x16 sc = zero16();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const kfrag k8 = kv ? IF::load(kp, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
      f16x8 kf;
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = (_Float16)(float)k8[e];
      sc = mma32(*(const f16x8 *)(Q16 + ((st + qrow) * Hq + h) * DK + 16 * i + 8 * hh), kf, sc);
    }
    float pe[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = acc_row(hh, j);
      pe[j] = (q0 + r < L && r >= n) ? fast_exp2(sc[j] * sl2 - mb[(st + q0 + r) * Hq + h]) : 0.f;
    }
    f16x8 dsf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) dsf[u][i] = (_Float16)(pe[8 * u + i] * dpe[8 * u + i]);
    // exact per-pair decays: P[q][kj] lives in lane kj, register of q
#pragma unroll 1
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
        for (int j = 0; j < 16; ++j) pj = (j == jsrc) ? pe[j] : pj;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kl = acc_row(hh, j);
          const float pvv = __shfl(pj, kl + 32 * hsrc);
          const int kj = kb + kl;
          if (col < DV && qk < L && kj <= qk)
            t[j] += pvv * fast_exp2(gl_at(qk, col) - gl_at(kj, col)) * delta_at<DV, F32IN>(ds, (st + qk) * Hq + h, col) *
                    sig[(st + qk) * Hq + h];
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (col < DV && kj < L) {
          const int64_t idx = ((st + kj) * Hkv + c) * DV + col;
          dv_i[idx] = (gq > 0 ? dv_i[idx] : 0.f) + t[j];
        }
      }
    }
    // dK[key][dk] += dS[q][key] Q[q][dk]: element i of lane (hh, n) of the
    // B operand is Q[q0 + 16u + acc_row(hh, i)][32bk + n], the k order of dsf
#pragma unroll 1
    for (int bk = 0; bk < NBK; ++bk) {
      const int col = min(32 * bk + n, DK - 1);
      f32x16 dacc = zero16();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f16x8 qb;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          qb[i] = Q16[((st + min(q0 + 16 * u + acc_row(hh, i), L - 1)) * Hq + h) * DK + col];
        dacc = mma32(dsf[u], qb, dacc);
      }
      if (32 * bk + n < DK)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kj = kb + acc_row(hh, j);
          if (kj < L) dk_i[((st + kj) * Hkv + c) * DK + col] += scale * dacc[j];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Near contributions to dk, dv: workgroup = one 128-chunk J of one kv head;
// key block p (keys c0 + 32p .. +31) is shared by wave p (A) and wave p + 4
// (B), which the hardware places on the same SIMD.  Steps run over the query
// blocks qa = 0..7 of chunk J and of the next chunk (the pairs with the
// largest decay weights), each head of the group in turn.  Each step copies
// one query block into LDS as row tiles: Q (fp16, three stages: B reads it
// one step late, transposed, for dK), the block-relative dhat as fp16 (dP off
// the diagonal) and as bf16 hi / lo (dP on the diagonal; read transposed for
// dV, which is always bf16x3: dv feeds the gate gradient, whose suffix sums
// accumulate the rounding of every token).  With E(b) the log2 gate prefix
// at the end of block b, continued into the next chunk, the decay of a pair
// in query block qa > p splits as
//     exp2(Gl_i - E(qa-1)) * exp2(E(qa-1) - E(p)) * exp2(E(p) - Gl_j):
// the first factor is in the staged dhat, the middle one gamma multiplies
// B's V-to-block-end operand (dP) and each of A's dV step results per
// channel, and the last one scales dV in the epilogue.  The diagonal block
// (the step whose query block is the pair's own) uses gamma =
// exp2(E(p-1) - E(p)) >= 1 and V from the token before the block (bf16x3,
// tiles staged with that step); past 2^BGUARD its pairs are evaluated
// directly after the loop.
//   A, step k: S_k = Q K^T, P_k = exp2(S sl2 - m) (fp32 into LDS), dV +=
//              gamma (.) (P_k^T dhat_k); the copies of step k+1's Q and fp16
//              dhat rows and row offsets.
//   B, step k: dS_{k-1} = P_{k-1} (LDS) (.) the dP_{k-1} it kept, dK +=
//              dS_{k-1}^T Q_{k-1}; dP_k = dhat_k (V (.) gamma)^T; the copies
//              of step k+1's bf16 hi / lo rows.
// One barrier per step; every wave waits for its own copies before it.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(512, 1) k_bwd_intra_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, DVP = Pad32<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  using QT = LdsTile<32, DK * 2>;  // Q rows (fp16)
  using XR = LdsTile<32, DV * 2>;  // block-relative dhat rows (fp16, bf16 hi, bf16 lo); V rows of the diagonal
  constexpr int PX = 4 * 64 * 16;  // one pair's P of a step: [j / 4][lane] float4
  // One LDS object for every tile (see the forward kernel).
  constexpr int O_Q = 0, O_X = O_Q + 3 * QT::BYTES, O_XH = O_X + 2 * XR::BYTES, O_XL = O_XH + 2 * XR::BYTES;
  constexpr int O_BH = O_XL + 2 * XR::BYTES, O_BL = O_BH + 2 * XR::BYTES, O_P = O_BL + 2 * XR::BYTES;
  constexpr int O_M = O_P + 2 * 4 * PX, O_E = O_M + 2 * 256, O_GW = O_E + 9 * DV * 4;
  __shared__ __align__(1024) char smem[O_GW + 4 * DV * 4];
  auto Qs = [&](int b) { return smem + O_Q + b * QT::BYTES; };
  auto Xs = [&](int b) { return smem + O_X + b * XR::BYTES; };
  auto XHs = [&](int b) { return smem + O_XH + b * XR::BYTES; };
  auto XLs = [&](int b) { return smem + O_XL + b * XR::BYTES; };
  auto BHs = [&](int b) { return smem + O_BH + b * XR::BYTES; };
  auto BLs = [&](int b) { return smem + O_BL + b * XR::BYTES; };
  auto Ms = [&](int b) { return (float *)(smem + O_M + b * 256); };  // 64 floats, 32 used
  float(*BE)[DV] = (float(*)[DV])(smem + O_E);  // BE[b + 1] = E(b), b = -1..7

  const Plan &pl = a.plan;
  const int gc = blockIdx.x, c = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isA = wave < 4;
  const int p = wave & 3;
  float *gw = (float *)(smem + O_GW) + p * DV;  // B's gamma of the step, per channel
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = uniform((gc - pl.cb128[s]) * CB);
  const int L = uniform(pl.seq_len[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int kb = c0 + 32 * p;
  const bool active = kb < L;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;
  const int nqo = min(8, (L - c0 + 31) / 32);  // query blocks in this chunk and the next
  const int nsteps = G * nqo;
  // Step k: query block nqo - 1 - k / G (the farthest first), head k % G.
  auto qa_of = [&](int k) { return nqo - 1 - k / G; };
  auto gl_at = [&](int tok, int d) { return a.Gl2[((st + tok) * Hkv + c) * DV + d]; };

  // Copies.  Rows past the end of the sequence read as zeros; their
  // probabilities are masked to zero when the step is computed.
  uint32_t oq[QT::NW], ox[XR::NW], ob[XR::NW];
  QT::lane_offsets(Hq * DK * 2, p, lane, oq);
  XR::lane_offsets(Hq * DV * 2, p, lane, ox);
  XR::lane_offsets(Hkv * DV * 2, p, lane, ob);
  auto stage_tile = [&](int k) {
    const int gq = k % G, qa = qa_of(k);
    const int h = c * G + gq, q0 = c0 + 32 * qa;
    const int64_t qr = (st + q0) * Hq + h;
    const int nrow = L - q0;
    if (isA) {
      const u32x4 rq = rsrc_words(a.Q16 + qr * DK, (int64_t)nrow * Hq * DK * 2);
      const u32x4 rx = rsrc_words(a.X16 + qr * DV, (int64_t)nrow * Hq * DV * 2);
#pragma unroll
      for (int t = 0; t < QT::NW; ++t) QT::dma_piece_untracked(Qs(k % 3), rq, oq, t, p);
#pragma unroll
      for (int t = 0; t < XR::NW; ++t) XR::dma_piece_untracked(Xs(k & 1), rx, ox, t, p);
      // lane r fills Ms[r] (every A wave, the same bytes)
      dma4_untracked(Ms(k & 1), rsrc_words(a.mb + qr, (int64_t)nrow * Hq * 4), (uint32_t)lane * Hq * 4);
    } else {
      const u32x4 rxh = rsrc_words(a.XH + qr * DV, (int64_t)nrow * Hq * DV * 2);
      const u32x4 rxl = rsrc_words(a.XL + qr * DV, (int64_t)nrow * Hq * DV * 2);
#pragma unroll
      for (int t = 0; t < XR::NW; ++t) {
        XR::dma_piece_untracked(XHs(k & 1), rxh, ox, t, p);
        XR::dma_piece_untracked(XLs(k & 1), rxl, ox, t, p);
      }
      if (qa < 4) {  // the diagonal block of pair qa: its key block is the query block
        const int64_t kr = (st + q0) * Hkv + c;
        const u32x4 rbh = rsrc_words(a.VBH + kr * DV, (int64_t)nrow * Hkv * DV * 2);
        const u32x4 rbl = rsrc_words(a.VBL + kr * DV, (int64_t)nrow * Hkv * DV * 2);
#pragma unroll
        for (int t = 0; t < XR::NW; ++t) {
          XR::dma_piece_untracked(BHs(k & 1), rbh, ob, t, p);
          XR::dma_piece_untracked(BLs(k & 1), rbl, ob, t, p);
        }
      }
    }
  };

  // Prologue: the block-end gate values (E), the key-side operand of the
  // wave's role (A: K as fp16, exact for |k| in [2^-14, 65504], since Q is
  // staged as fp16; B: V to the end of its block) and the first step's
  // copies, all issued before one wait.
  constexpr int NBE = (9 * DV + 511) / 512;
  float be0[NBE], be1[NBE];
#pragma unroll
  for (int t = 0; t < NBE; ++t) {
    const int e = tid + 512 * t, b = e / DV - 1, d = e % DV;
    be0[t] = be1[t] = 0.f;
    if (e < 9 * DV && b >= 0) {
      if (b < 4) {
        be0[t] = gl_at(min(c0 + 32 * b + 31, L - 1), d);
      } else {
        be0[t] = gl_at(min(c0 + CB - 1, L - 1), d);
        if (c0 + CB < L) be1[t] = gl_at(min(c0 + CB + 32 * (b - 4) + 31, L - 1), d);
      }
    }
  }
  constexpr int NKS = NS > NSV ? NS : NSV;
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  kfrag kr[NS];
  f16x8 kop[NKS];  // A: K (fp16); B: V to the end of its block
#pragma unroll
  for (int i = 0; i < NKS; ++i) kop[i] = zf;
  if (isA) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      kr[i] = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
  } else if (kv) {
#pragma unroll
    for (int i = 0; i < NSV; ++i) kop[i] = *(const f16x8 *)(a.VE + ((st + key) * Hkv + c) * DV + 16 * i + 8 * hh);
  }
  if (nsteps > 0) stage_tile(0);
  wait_all();
  if (isA)
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) kop[i][e] = (_Float16)(float)kr[i][e];
#pragma unroll
  for (int t = 0; t < NBE; ++t) {
    const int e = tid + 512 * t, b = e / DV - 1, d = e % DV;
    if (e < 9 * DV) BE[b + 1][d] = be0[t] + be1[t];
  }
  __syncthreads();
  // Whether a key block's diagonal needs exact per-pair decays (its gate
  // range beyond 2^BGUARD): this pair's, and whether any pair's does.
  bool direct = false, direct_any = false;
#pragma unroll 1
  for (int pb = 0; pb < 4; ++pb) {
    float rng = 0.f;
#pragma unroll
    for (int i = 0; i < NSV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 16 * i + 8 * hh + e;
        rng = fmaxf(rng, BE[pb][d] - BE[pb + 1][d]);
      }
    const bool x = __any(rng > BGUARD);
    direct_any |= x;
    if (pb == p) direct = x;
  }
  auto act_of = [&](int qa) { return active && (qa > p || (qa == p && !direct)); };
  const uint32_t sbase = lds_addr(smem);
  const uint32_t apx = sbase + O_P + p * PX + 16 * lane;  // this lane's P exchange slot
  constexpr uint32_t RQ = 2 * DK, RX = 2 * DV;  // row bytes of the Q and dhat tiles

  f32x16 acc[NBK > NBV ? NBK : NBV];  // A: dV (relative to gamma of the current query block); B: dK
#pragma unroll
  for (int b = 0; b < (NBK > NBV ? NBK : NBV); ++b) acc[b] = zero16();
  // A: the query block whose gamma acc is relative to (its last one, after
  // the loop); dv then carries exp2(E(qlast - 1) - Gl_j) per key and channel
  int qlast = p + 1;
  if (isA) {
    // per-lane LDS addresses in stage 0: Q row fragments (S) and the two
    // transposing-read pieces of the dhat hi rows per output block (dV)
    uint32_t aq[NS], adv[NBV][2];
#pragma unroll
    for (int i = 0; i < NS; ++i) aq[i] = sbase + O_Q + QT::off(n, min(2 * i + hh, QT::CPR - 1));
#pragma unroll
    for (int bv = 0; bv < NBV; ++bv) {
      uint32_t o[2];
      tr_offsets<XR>(32 * bv, lane, o);
      adv[bv][0] = sbase + O_XH + o[0];
      adv[bv][1] = sbase + O_XH + o[1];
    }
    const uint32_t apx_ = opaque(apx);
    int qcur = -1;
    for (int k = 0; k < nsteps; ++k) {
      const int qa = qa_of(k);
      const bool diag = qa == p;
      wait_all();
      __syncthreads();  // step k's tiles landed; step k - 1's readers are done
      if (k + 1 < nsteps) stage_tile(k + 1);
      if (!act_of(qa)) continue;
      const int q0 = c0 + 32 * qa;
      f32x4 mq[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        mq[q4] = *(const __attribute__((address_space(3))) f32x4 *)(lds_at(sbase + O_M + 16 * hh + (k & 1) * 256) + 32 * q4);
      // S[q][key]: lane = key, register j = query acc_row(hh, j)
      f32x16 sc = zero16();
      {
        const uint32_t so = (k % 3) * QT::BYTES;
        f16x8 fq[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) fq[i] = lds_row16p(lds_at(aq[i]) + so);
#pragma unroll
        for (int i = 0; i < NS; ++i) sc = mma32(fq[i], kop[i], sc);
      }
      // entering a nearer query block: dV so far times gamma_old / gamma_new
      // = exp2(E(qcur - 1) - E(qa - 1)) <= 1 (query blocks are visited last first)
      if (qa != qcur) {
        if (qcur >= 0)
#pragma unroll
          for (int bv = 0; bv < NBV; ++bv) {
            const int d = min(32 * bv + n, DV - 1);
            const float r = fast_exp2(BE[qcur][d] - BE[qa][d]);
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[bv][j] *= r;
          }
        qcur = qa;
      }
      float pv[16];
      bf16x8 ph[2], plo[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = acc_row(hh, j);
        pv[j] = q0 + r < L && (!diag || r >= n) ? fast_exp2(sc[j] * sl2 - mq[j >> 2][j & 3]) : 0.f;
        split_bf16(pv[j], ph[j >> 3], plo[j >> 3], j & 7);
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        *(__attribute__((address_space(3))) f32x4 *)(lds_at(apx_ + (k & 1) * 4 * PX) + 1024 * j4) =
            f32x4{pv[4 * j4], pv[4 * j4 + 1], pv[4 * j4 + 2], pv[4 * j4 + 3]};
      // dV[key][d] += sum_q P[q][key] dhat[q][d] (bf16x3), output blocks
      // interleaved; the transposing reads of a k slice run one slice ahead
      {
        const uint32_t so = (k & 1) * XR::BYTES;
        f16x4 th[2][NBV][2], tl[2][NBV][2];
        auto rd = [&](int u, int s2) {
#pragma unroll
          for (int bv = 0; bv < NBV; ++bv)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              th[s2][bv][t] = lds_tr8p(lds_at(adv[bv][t]) + so + 16 * u * RX);
              tl[s2][bv][t] = lds_tr8p(lds_at(adv[bv][t]) + so + 16 * u * RX + 2 * XR::BYTES);
            }
        };
        rd(0, 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (u == 0) rd(1, 1);
#pragma unroll
          for (int bv = 0; bv < NBV; ++bv) {
            const bf16x8 h8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(th[u][bv][0], th[u][bv][1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[bv] = mma32(ph[u], h8, acc[bv]);
          }
#pragma unroll
          for (int bv = 0; bv < NBV; ++bv) {
            const bf16x8 l8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tl[u][bv][0], tl[u][bv][1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[bv] = mma32(ph[u], l8, acc[bv]);
          }
#pragma unroll
          for (int bv = 0; bv < NBV; ++bv) {
            const bf16x8 h8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(th[u][bv][0], th[u][bv][1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[bv] = mma32(plo[u], h8, acc[bv]);
          }
        }
      }
    }
    wait_all();
    __syncthreads();  // the barrier B's last dK step waits at
    if (qcur >= 0) qlast = qcur;
  } else {
    // per-lane LDS addresses in stage 0: dhat row fragments (dP; the other
    // row tiles lie at fixed distances) and the two transposing-read pieces
    // of the Q rows per output block (dK)
    uint32_t ax[NSV], aqt[NBK][2];
#pragma unroll
    for (int i = 0; i < NSV; ++i) ax[i] = sbase + O_X + XR::off(n, min(2 * i + hh, XR::CPR - 1));
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      uint32_t o[2];
      tr_offsets<QT>(32 * bk, lane, o);
      aqt[bk][0] = sbase + O_Q + o[0];
      aqt[bk][1] = sbase + O_Q + o[1];
    }
    const uint32_t apx_ = opaque(apx);
    f32x16 dpk = zero16();  // dP of the previous step
    f16x8 kg[NSV];          // V to the end of its block times gamma of the current query block
#pragma unroll
    for (int i = 0; i < NSV; ++i) kg[i] = zf;
    int qcur = -1;
    // dS of step kk from A's P (LDS) and the kept dP, then dK += dS^T Q_kk
    // with Q read transposed from its row stage
    auto dk_step = [&](int kk) {
      f16x8 dsf[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 pq = *(const __attribute__((address_space(3))) f32x4 *)lds_at(apx_ + (kk & 1) * 4 * PX + 1024 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * j4 + e;
          dsf[j >> 3][j & 7] = (_Float16)(pq[e] * dpk[j]);
        }
      }
      const uint32_t so = (kk % 3) * QT::BYTES;
      f16x4 tq[2][NBK][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
          for (int t = 0; t < 2; ++t) tq[u][bk][t] = lds_tr8p(lds_at(aqt[bk][t]) + so + 16 * u * RQ);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
          acc[bk] = mma32(dsf[u], __builtin_shufflevector(tq[u][bk][0], tq[u][bk][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[bk]);
    };
    for (int k = 0; k < nsteps; ++k) {
      const int qa = qa_of(k);
      const bool diag = qa == p;
      wait_all();
      __syncthreads();  // step k's tiles landed; step k - 1's readers are done
      if (k + 1 < nsteps) stage_tile(k + 1);
      if (k > 0 && act_of(qa_of(k - 1))) dk_step(k - 1);
      if (!act_of(qa)) continue;
      const uint32_t so = (k & 1) * XR::BYTES;
      // dP[q][key] (lane = key, register j = query acc_row(hh, j))
      f32x16 dp = zero16();
      if (diag) {
        // split at the token before the block: dhat and V as bf16 hi / lo (bf16x3)
#pragma unroll
        for (int i = 0; i < NSV; ++i) {
          const uint32_t ai = ax[i] + so;
          const bf16x8 xh = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 2 * XR::BYTES));
          const bf16x8 xl = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 4 * XR::BYTES));
          const bf16x8 vh = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 6 * XR::BYTES));
          const bf16x8 vl = __builtin_bit_cast(bf16x8, lds_row16p(lds_at(ai) + 8 * XR::BYTES));
          dp = mma32(xh, vh, dp);
          dp = mma32(xl, vh, dp);
          dp = mma32(xh, vl, dp);
        }
      } else {
        if (qa != qcur) {
          // gamma[d] = exp2(E(qa - 1) - E(p)) depends on the channel only: each
          // lane evaluates two channels into the wave's table, then every lane
          // reads the channels it needs (a wave's LDS accesses complete in order)
#pragma unroll
          for (int t = 0; t < (DV + 63) / 64; ++t) {
            const int d = lane + 64 * t;
            if (d < DV) gw[d] = fast_exp2(BE[qa][d] - BE[p + 1][d]);
          }
#pragma unroll
          for (int i = 0; i < NSV; ++i) {
            const float4 g0 = *(const float4 *)(gw + 16 * i + 8 * hh), g1 = *(const float4 *)(gw + 16 * i + 8 * hh + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) kg[i][e] = (_Float16)((float)kop[i][e] * gv[e]);
          }
          qcur = qa;
        }
        f16x8 fx[NSV];
#pragma unroll
        for (int i = 0; i < NSV; ++i) fx[i] = lds_row16p(lds_at(ax[i]) + so);
#pragma unroll
        for (int i = 0; i < NSV; ++i) dp = mma32(fx[i], kg[i], dp);
      }
      dpk = dp;
    }
    wait_all();
    __syncthreads();  // A's last P is in LDS
    if (nsteps > 0 && act_of(qa_of(nsteps - 1))) dk_step(nsteps - 1);
  }

  if (!isA && active) {
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      const int col = 32 * bk + n;
      if (col >= DK) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (kj < L) a.dk_i[((st + kj) * Hkv + c) * DK + col] = a.scale * acc[bk][j];
      }
    }
  }
  // Diagonal block with exact per-pair decays (gate range beyond 2^BGUARD),
  // by B after its dk store; A's epilogue reads its dV partials after the
  // barrier below.  (Otherwise the staged loop did it: split at the token
  // before the block, gamma = exp2(E(p-1) - E(p)) >= 1, V from the token
  // before the block as bf16x3.)
  if (!isA && direct && active)
    near_exact_diag<DK, DV, F32IN>(a.x, a.rstd, a.prj, a.dO, a.z, a.w, a.o_norm, a.sig, a.Gl2, a.v, a.k, a.Q16, a.mb,
                                   a.dv_i, a.dk_i, a.scale, sl2, Hq, Hkv, G, st, c, L, kb);
  if (direct_any) __syncthreads();  // B's exact diagonal dV partials are written
  if (!active || !isA) return;
  // dv relative to the last query block's gamma: exp2(E(qlast - 1) - Gl_j).  Each
  // column block's inputs are loaded one block ahead, before the previous
  // block's stores (the compiler cannot tell the buffers apart, so a load
  // after a store would wait for it).
  float in[2][2][16];  // [slot][gate value, exact partial][row]
  auto load_dv = [&](int bv, float (&x)[2][16]) {
    const int col = min(32 * bv + n, DV - 1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t idx = ((st + min(kb + acc_row(hh, j), L - 1)) * Hkv + c) * DV + col;
      x[0][j] = a.Gl2[idx];
      x[1][j] = direct ? a.dv_i[idx] : 0.f;
    }
  };
  load_dv(0, in[0]);
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    if (bv + 1 < NBV) load_dv(bv + 1, in[(bv + 1) & 1]);
    const int col = 32 * bv + n;
    if (col >= DV) continue;
    const float ew = BE[qlast][col];
    const float(&x)[2][16] = in[bv & 1];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) a.dv_i[((st + kj) * Hkv + c) * DV + col] = fast_exp2(ew - x[0][j]) * acc[bv][j] + x[1][j];
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
  __shared__ __align__(1024) char smem[O_G + 2 * DV * 2];
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Kts = [&](int b) { return smem + O_T + b * TT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  auto Ls = [&](int b) { return smem + O_L + b * 1024; };
  auto gam = [&](int b) { return (_Float16 *)(smem + O_G) + b * DV; };  // gamma_IJ (fp16)

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

  // The dhat rows stay in registers; gamma_IJ multiplies the V operand as it
  // is read (a per-lane fp16 vector per k slab, read from LDS each step).
  // Every load of the kernel's own is complete before the first copy is
  // issued, and the loop makes none.
#pragma unroll
  for (int i = 0; i < NSV; ++i) dhf[i] = *(const f16x8 *)(dhrow + 16 * i + 8 * hh);
  if (nsteps > 0 && tid < DV) gam(0)[tid] = (_Float16)fast_exp2((float)(lamI - lam_of(0)));
  // Per-lane LDS addresses in stage 0: K and V row fragments, transposed K
  // rows, and the gamma vectors.
  uint32_t ak[NS], av[NSV], at[NBK][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) ak[i] = lds_addr(Ks(0)) + KT::off(n, 2 * i + hh);
#pragma unroll
  for (int i = 0; i < NSV; ++i) av[i] = lds_addr(Vs(0)) + VT::off(n, 2 * i + hh);
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
    for (int u = 0; u < 2; ++u) at[bk][u] = lds_addr(Kts(0)) + TT::off(32 * bk + n, 2 * u + hh);
  const uint32_t ag = lds_addr(gam(0)) + 2 * (8 * hh);
  wait_all();
  if (nsteps > 0) {
    stage_tile(0, 0);
    stage_tile(min(1, nsteps - 1), 1);
  }
  wait_vm<NCOPYQ>();  // step 0 has landed
  lds_barrier();
  // One step; its stage b = k % 3 is a compile-time constant (the loop
  // below runs three steps per trip), so each LDS read's stage offset folds
  // into the instruction's offset field.
  auto step = [&](int k, auto bc) {
    constexpr int b = decltype(bc)::value;
    const bool next_chunk = (k & 3) == 3 && k + 1 < nsteps;
    // Same copies on every step (past the last step, the last step's tile
    // again, into a stage nobody reads); step k + 2's stage was last read in
    // step k - 1.
    stage_tile(min(k + 2, nsteps - 1), (b + 2) % NBQ);
    {
      const uint32_t go = opaque(((k >> 2) & 1) * DV * 2);
      // S^T and dP^T, their chains alternating, operand reads two products
      // ahead (the chunk's gamma vectors first; four ahead made the
      // three-step loop spill)
      f16x8 gv[NSV];
#pragma unroll
      for (int i = 0; i < NSV; ++i) gv[i] = lds_row16p(lds_at(ag + go) + 2 * 16 * i);
      f32x16 sc = zero16(), dp = zero16();
      constexpr int NM = NS > NSV ? NS : NSV;
      kfrag fk[NM];
      f16x8 fv[NM];
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i < NS) fk[i] = *(const __attribute__((address_space(3))) kfrag *)(lds_at(ak[i]) + b * KT::BYTES);
        if (i < NSV) fv[i] = lds_row16p(lds_at(av[i]) + b * VT::BYTES);
      }
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if (i < NS) sc = mma32(fk[i], qf[i], sc);
        if (i < NSV) dp = mma32(fv[i] * gv[i], dhf[i], dp);
      }
      {
        constexpr int NP = NS + NSV, LA = NP < 2 ? NP : 2;
        __builtin_amdgcn_sched_group_barrier(0x100, LA + NSV, 0);
#pragma unroll
        for (int m = 0; m < NP - LA; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      f16x8 dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 8 * u + i;
          dsf[u][i] = (_Float16)(fast_exp2(sc[j] * sl2 - mbn) * dp[j]);
        }
      // dQ += dS K with the transposed K rows, reads two products ahead
      f16x8 tk[NBK][2];
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u) tk[bk][u] = lds_row16p(lds_at(at[bk][u]) + b * TT::BYTES);
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[bk] = mma32(dsf[u], tk[bk][u], acc[bk]);
      {
        constexpr int NP = 2 * NBK, LA = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
        for (int m = 0; m < NP - LA; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // gamma of the next chunk, into the other buffer (its last readers passed
    // the barrier that began this chunk).
    if (next_chunk && tid < DV)
      gam(((k >> 2) + 1) & 1)[tid] = (_Float16)fast_exp2((float)(lamI - ((const double *)Ls(b))[tid]));
    wait_vm<NCOPYQ>();  // step k + 1 has landed (step k + 2's copies stay in flight)
    lds_barrier();
  };
  for (int k = 0; k < nsteps; k += NBQ) {
    step(k, IC<0>{});
    if (k + 1 < nsteps) step(k + 1, IC<1>{});
    if (k + 2 < nsteps) step(k + 2, IC<2>{});
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
// 128 keys of one key chunk J and kv head, 8 waves: the 32 keys of pair p are
// shared by wave p (A) and wave p + 4 (B), which the hardware places on the
// same SIMD.  Query chunks go from the last to J + 2 and, within each, the G
// query heads of the group, 64 query rows per step, one barrier per step:
//   A: S_k = Q K^T, P_k (fp16, into LDS and kept), dV += P_k^T dhat_k, and
//      the copies of step k + 1's Q and dhat rows and row maxima
//   B: dS_{k-1} = P_{k-1} (from LDS) times the dP_{k-1} it kept, dK +=
//      dS_{k-1}^T Q_{k-1}, dP_k = dhat_k (V (.) gamma)^T, and the copy of
//      step k + 1's transposed dhat tile
// so that the waves of a pair never wait for each other within a step and
// A's exponentials run beside B's products.  S and dP read row tiles, dV the
// transposed dhat tile (key_pos column order: the eight rows a lane needs
// are side by side) and dK the Q rows through the transposing LDS read; all
// reads run a few products ahead of their MFMAs.  Q rows are kept three
// steps (dK uses the previous step's), the other tiles two.  All query rows
// lie at least a chunk after the keys, so no pair is masked; rows past the
// sequence end read as zeros (their dP, dS and dhat are zero).
// The decay product between the chunks, gamma_IJ = exp2(Lam[I-1] - Lam[J]),
// enters dP through V (.) gamma_IJ (B rebuilds it per query chunk from the V
// rows it keeps in registers) and dV through the accumulator: A accumulates
// dV relative to the current chunk's gamma and, entering the next (nearer)
// chunk, multiplies it by gamma_I / gamma_{I-1} = exp2(Lam[I-1] - Lam[I-2]) <= 1
// per column; the epilogue applies gamma_{J+2,J}.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(512, small_head_waves(DK, DV)) k_bwd_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, DVP = Pad32<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  constexpr int RS = 64;             // query rows per step (two halves of 32)
  using QT = LdsTile<RS, DK * 2>;    // Q rows of a step (fp16)
  using DR = LdsTile<RS, DV * 2>;    // scaled dhat rows of a step (fp16)
  using DX = LdsTile<DVP, RS * 2>;   // transposed dhat of a step [channel][row, key_pos order], rows padded to DVP
  using DXD = LdsTile<DV, RS * 2>;   // the rows a copy fills
  using QW = typename QT::template Waves<4>;  // copies issued by the four A waves
  using DW = typename DR::template Waves<4>;
  using DXW = typename DXD::template Waves<4>;  // copies issued by the four B waves
  constexpr int PEX = 2 * 2 * 64 * 16;  // one pair's P of a step (fp16): [half][u][lane] 16 bytes
  constexpr int O_Q = 0, O_D = O_Q + 3 * QT::BYTES, O_DX = O_D + 2 * DR::BYTES, O_P = O_DX + 2 * DX::BYTES;
  constexpr int O_M = O_P + 2 * 4 * PEX, O_G = O_M + 2 * 256, O_GH = O_G + 2 * DVP * 4;
  __shared__ __align__(1024) char smem[O_GH + 2 * DVP * 2];
  auto rat = [&](int b) { return (float *)(smem + O_G) + b * DVP; };        // gamma_I / gamma_{I-1} per column
  auto gamh = [&](int b) { return (_Float16 *)(smem + O_GH) + b * DVP; };  // gamma_IJ (fp16)

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
  const bool isA = wave < 4;
  const int pr = wave & 3;
  const int kb = J * CB + 32 * pr;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;

  const int nch = (L + CB - 1) / CB;
  const int I0 = J + 2, I1 = nch - 1;                  // query chunks visited: I1 down to I0
  const int ns1 = (L - I1 * CB + RS - 1) / RS;          // slices of the last (possibly partial) chunk
  const int nsteps = I0 <= I1 ? G * ns1 + (CB / RS) * G * (I1 - I0) : 0;
  // Step position: query chunk I, query head of the group gq, 64-row slice
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

  // Key-side operand: K for S (A), V (.) gamma for dP (B, rebuilt per chunk
  // from its V rows, vr).
  constexpr int NKS = NS > NSV ? NS : NSV;
  f16x8 kf[NKS], vr[NSV];
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int i = 0; i < NKS; ++i) kf[i] = zf;
#pragma unroll
  for (int i = 0; i < NSV; ++i) vr[i] = zf;
  if (isA) {
    // The key as an fp16 operand: Q is staged as fp16 (q converted once,
    // exact for |q| in [2^-14, 65504]), so the score product runs in fp16 and
    // equals the bf16 one for such inputs.
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const kfrag kr = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[i][e] = (_Float16)(float)kr[e];
    }
  } else if (kv) {
#pragma unroll
    for (int i = 0; i < NSV; ++i)
      vr[i] = *(const f16x8 *)(a.Vr + (((int64_t)(cbs + J) * Hkv + c) * CB + 32 * pr + n) * DV + 16 * i + 8 * hh);
  }

  // Per-lane LDS addresses in stage 0: the first product's row fragments (Q
  // for A, dhat for B) and the second's fragments (transposed dhat for A per
  // output block and 16-row group; the two transposing-read pieces of the Q
  // rows for B per output block); a step adds its stage's offset.
  const uint32_t sbase = lds_addr(smem);
  constexpr int NBA = NBK > NBV ? NBK : NBV;
  uint32_t a1[NKS], a2[NBA][4];
  auto addresses = [&]() {  // computed in each wave's own loop branch
#pragma unroll
    for (int i = 0; i < NKS; ++i)
      a1[i] = sbase + (isA ? O_Q + QT::off(n, min(2 * i + hh, QT::CPR - 1)) : O_D + DR::off(n, min(2 * i + hh, DR::CPR - 1)));
#pragma unroll
    for (int b = 0; b < NBA; ++b) {
      uint32_t oq[2];
      tr_offsets<QT>(32 * b, lane, oq);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        a2[b][g] = isA ? sbase + O_DX + DX::off(min(32 * b + n, DVP - 1), 2 * g + hh) : sbase + O_Q + (g < 2 ? oq[g] : 0);
    }
  };
  const uint32_t apx = sbase + O_P + PEX * pr + 16 * lane, ams = sbase + O_M + 4 * (4 * hh);
  const uint32_t rb1 = isA ? 2 * DK : 2 * DV;  // row bytes of the first product's tile

  // Copies: A the row tiles and row maxima of a step, B its transposed dhat tile.
  const int wb = wave & 3;
  uint32_t oq[QW::NWW], od[DW::NWW], odx[DXW::NWW];
  QW::lane_offsets(Hq * DK * 2, wb, lane, oq);
  DW::lane_offsets(Hq * DV * 2, wb, lane, od);
  DXW::lane_offsets(CB * 2, wb, lane, odx);
  auto stage_rows = [&](const Pos &p, int qs, int b) {
    const int h = c * G + p.gq, qt0 = p.I * CB + RS * p.u;
    const int64_t qr = (st + qt0) * Hq + h;
    const int64_t nrow = L - qt0;  // rows past the sequence read as zeros
    QW::dma_untracked(smem + O_Q + qs * QT::BYTES, rsrc_words(a.Q16 + qr * DK, nrow * Hq * DK * 2), oq, wb);
    DW::dma_untracked(smem + O_D + b * DR::BYTES, rsrc_words(a.dh + qr * DV, nrow * Hq * DV * 2), od, wb);
    if (wb == 0) dma4_untracked(smem + O_M + b * 256, rsrc_words(a.mb + qr, nrow * Hq * 4), (uint32_t)lane * Hq * 4);
  };
  auto stage_cols = [&](const Pos &p, int b) {
    const int64_t ch = (int64_t)(cbs + p.I) * Hq + c * G + p.gq;
    DXW::dma_untracked(smem + O_DX + b * DX::BYTES, rsrc_words(a.dhT + ch * DV * CB + RS * p.u, (int64_t)DV * CB * 2),
                       odx, wb);
  };
  // zero rows of the narrow transposed tiles (never copied)
  if (DV < DVP)
    for (int e = tid; e < (DVP - DV) * RS * 2 / 4; e += 512)
      for (int b = 0; b < 2; ++b) ((uint32_t *)(smem + O_DX + b * DX::BYTES + DV * RS * 2))[e] = 0u;

  // gamma per column d = tid (A threads below DV): gamma_IJ (fp16, for
  // V (.) gamma) and the ratio to the next chunk's, into buffer ord & 1.
  const int dt = min(tid, DV - 1);
  const bool gthread = isA && tid < DV;
  const double lamJ = gthread ? a.Lam[((int64_t)(cbs + J) * Hkv + c) * DV + dt] : 0.0;
  auto lam_of = [&](int I) { return a.Lam[((int64_t)(cbs + I - 1) * Hkv + c) * DV + dt]; };  // Lam[I-1]

  f32x16 acc[NBA];  // A: dV (relative to the current chunk's gamma), B: dK
#pragma unroll
  for (int b = 0; b < NBA; ++b) acc[b] = zero16();
  constexpr bool SAME = NS == NSV;
  const int n1 = isA ? NS : NSV;     // k slabs of the first product
  const int n2 = isA ? NBV : NBK;    // output blocks of the second

  // First product (A: S = Q K^T, B: dP = dhat (V (.) gamma)^T); lane = key,
  // register j = row r0 + 32 h2 + acc_row(hh, j).  The halves' chains
  // alternate, reads run four products ahead.
  auto first = [&](uint32_t so1, f32x16 (&xr)[2]) {
    f16x8 fr[NKS][2];
#pragma unroll
    for (int i = 0; i < NKS; ++i)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        if (SAME || i < n1) fr[i][h2] = lds_row16p(lds_at(a1[i] + so1) + 32 * h2 * rb1);
    xr[0] = xr[1] = zero16();
#pragma unroll
    for (int i = 0; i < NKS; ++i)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        if (SAME || i < n1) xr[h2] = mma32(fr[i][h2], kf[i], xr[h2]);
    if (SAME && NKS >= 2) {
      constexpr int LA = 2 * NKS < 4 ? 2 * NKS : 4;
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int m = 0; m < 2 * NKS - LA; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  Pos cur{I1, 0, 0, 0}, nxt = cur;
  if (nsteps > 0) {
    if (isA) stage_rows(cur, 0, 0);
    else stage_cols(cur, 0);
    if (gthread) gamh(0)[tid] = (_Float16)fast_exp2((float)(lam_of(I1) - lamJ));
  }

  // The two waves of a pair run separate loops with the same barriers, so
  // each keeps only its own values live.
  if (isA) {
    addresses();
    const uint32_t apx_ = opaque(apx), ams_ = opaque(ams);
    int prev_ord = 0;
    double lamI = gthread ? lam_of(I1) : 0.0, lamN = 0.0;
    for (int k = 0; k < nsteps; ++k) {
      const int b = k & 1;
      if (k + 1 < nsteps) advance(nxt);
      const bool first_of_chunk = k == 0 || cur.ord != prev_ord;
      const bool last_of_chunk = k + 1 < nsteps && nxt.ord != cur.ord;
      wait_all();
      __syncthreads();  // step k's tiles landed; step k - 1's readers are done
      // the next chunk's Lam row (used at this chunk's last step; the wait at
      // the top of the next step covers it)
      if (first_of_chunk && gthread && cur.I - 1 >= I0) lamN = lam_of(cur.I - 1);
      f32x16 xr[2];
      first((k % 3) * QT::BYTES, xr);
      // P of both halves: fp16, into the exchange buffer of the step's parity
      // and kept as the A operand of dV
      f16x8 pf[2][2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        f32x4 mq[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          mq[q4] = *(const __attribute__((address_space(3))) f32x4 *)(lds_at(ams_ + b * 256) + 4 * (32 * h2 + 8 * q4));
#pragma unroll
        for (int j = 0; j < 16; ++j) pf[h2][j >> 3][j & 7] = (_Float16)fast_exp2(xr[h2][j] * sl2 - mq[j >> 2][j & 3]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          *(__attribute__((address_space(3))) f16x8 *)(lds_at(apx_ + b * 4 * PEX) + 16 * 64 * (2 * h2 + u)) = pf[h2][u];
      }
      // the row copies of the next step (their stages were last read in step k - 1)
      if (k + 1 < nsteps) stage_rows(nxt, (k + 1) % 3, b ^ 1);
      if (cur.ord != prev_ord) {  // entered a nearer chunk: dV so far times gamma_I / gamma_{I-1}
        prev_ord = cur.ord;
        const float *rt = rat(cur.ord & 1);
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv) {
          const float r = rt[min(32 * bv + n, DVP - 1)];
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[bv][j] *= r;
        }
      }
      // dV += P^T dhat: output block fastest, reads four products ahead
      {
        constexpr int NM = 4 * NBV, LA = NM < 4 ? NM : 4;
        const uint32_t off = b * DX::BYTES;
        f16x8 tf[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) tf[m] = lds_row16(a2[m % NBV][m / NBV] + off);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int g = m / NBV;
          acc[m % NBV] = mma32(pf[g >> 1][g & 1], tf[m], acc[m % NBV]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
        for (int m = 0; m < NM - LA; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (last_of_chunk && gthread) {
        // the next chunk's gamma and the ratio applied on entering it (the
        // buffer's last readers passed the barrier that began this chunk)
        gamh(nxt.ord & 1)[tid] = (_Float16)fast_exp2((float)(lamN - lamJ));
        rat(nxt.ord & 1)[tid] = fast_exp2((float)(lamI - lamN));
        lamI = lamN;
      }
      cur = nxt;
    }
    wait_all();
    __syncthreads();  // the barrier B's last dK step waits at
  } else {
    addresses();
    const uint32_t apx_ = opaque(apx);
    int prev_ord = -1;
    f32x16 dpk[2];  // dP of the previous step
    // dS of step k - 1 from A's P (LDS, exchange buffer pb) and the kept dP,
    // then dK += dS^T Q_{k-1} with Q read transposed from its row stage qs
    auto dk_step = [&](int pb, int qs) {
      f16x8 dsp[2][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f16x8 p = *(const __attribute__((address_space(3))) f16x8 *)(lds_at(apx_ + pb * 4 * PEX) + 16 * 64 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) dsp[g >> 1][g & 1][i] = (_Float16)((float)p[i] * dpk[g >> 1][8 * (g & 1) + i]);
      }
      constexpr int NM = 4 * NBK, LA = NM < 4 ? NM : 4;
      const uint32_t off = qs * QT::BYTES;
      f16x4 tp[NM][2];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t) tp[m][t] = lds_tr8p(lds_at(a2[m % NBK][t] + off) + 16 * (m / NBK) * (2 * DK));
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int g = m / NBK;
        acc[m % NBK] = mma32(dsp[g >> 1][g & 1], __builtin_shufflevector(tp[m][0], tp[m][1], 0, 1, 2, 3, 4, 5, 6, 7),
                             acc[m % NBK]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
      for (int m = 0; m < NM - LA; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int k = 0; k < nsteps; ++k) {
      const int b = k & 1;
      if (k + 1 < nsteps) advance(nxt);
      wait_all();
      __syncthreads();  // step k's tiles landed; step k - 1's readers are done
      // the transposed dhat copy of the next step (its stage was last read in step k - 1)
      if (k + 1 < nsteps) stage_cols(nxt, b ^ 1);
      if (k > 0) dk_step(b ^ 1, (k + 2) % 3);
      if (cur.ord != prev_ord) {  // first step of a query chunk: V (.) gamma_IJ
        prev_ord = cur.ord;
        const _Float16 *gmh = gamh(cur.ord & 1);
#pragma unroll
        for (int i = 0; i < NSV; ++i) kf[i] = vr[i] * *(const f16x8 *)(gmh + 16 * i + 8 * hh);
      }
      first(b * DR::BYTES, dpk);
      cur = nxt;
    }
    wait_all();
    __syncthreads();  // A's last P is in LDS
    if (nsteps > 0) dk_step((nsteps - 1) & 1, (nsteps - 1) % 3);
  }
  // A waves of key blocks past the end: zero partial sums of dG (below)
  if (isA && kb >= L) {
    for (int d = lane; d < DV; d += 64) a.dg_tot[(((int64_t)gci * Hkv + c) * 4 + pr) * DV + d] = 0.f;
    return;
  }
  if (kb >= L) return;
  // epilogue: dk (B), dv (A; inter part scaled to the key: exp(Gl_end(J) -
  // Gl_key) and by gamma_{J+2,J}), dG = qside - v (.) dv.  Addresses are the
  // workgroup's first key row (uniform) plus 32-bit offsets.  The compiler
  // cannot tell the output and input buffers apart, so a load placed after a
  // store waits for it: inputs are loaded one half block ahead, before the
  // previous half block's stores.
  // (lane indices taken afresh: values kept from before the loops would stay
  // live across them)
  const int le = (int)(opaque((uint32_t)threadIdx.x) & 63), hhe = le >> 5, ne = le & 31;
  const int tend = min((J + 1) * CB, L) - 1;
  // element offset of register j's key row from the workgroup's first key row
  auto krow = [&](int j) { return (uint32_t)min(acc_row(hhe, j), L - 1 - kb) * (uint32_t)Hkv; };
  const int64_t row0 = (st + kb) * Hkv + c;
  const int64_t nk = (int64_t)min(32, L - kb) * Hkv;  // rows covered by the resources below
  if (!isA) {
    const rsrc_t rki = make_rsrc(a.dk_i + row0 * DK, nk * DK * 4);
    const rsrc_t rk = make_rsrc((const char *)a.dk + row0 * DK * (a.out_f32 ? 4 : 2), nk * DK * (a.out_f32 ? 4 : 2));
    float pk[2][16];
    auto load_dk = [&](int bk, float (&part)[16]) {
      const uint32_t col = min(32 * bk + ne, DK - 1);
#pragma unroll
      for (int j = 0; j < 16; ++j) part[j] = buf_ld_f32(rki, 4 * (krow(j) * DK + col));
    };
    load_dk(0, pk[0]);
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      if (bk + 1 < NBK) load_dk(bk + 1, pk[(bk + 1) & 1]);
      const int col = 32 * bk + ne;
      if (col < DK)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (kb + acc_row(hhe, j) < L) buf_st_out(rk, krow(j) * DK + col, a.scale * acc[bk][j] + pk[bk & 1][j], a.out_f32);
    }
    return;
  }
  const int64_t nb = nk * DV * 4;
  const rsrc_t rgl = make_rsrc(a.Gl2 + row0 * DV, nb), rdi = make_rsrc(a.dv_i + row0 * DV, nb);
  const rsrc_t rqs = make_rsrc(a.qside + row0 * DV, nb), rdg = make_rsrc(a.dG + row0 * DV, nb);
  const rsrc_t rv = make_rsrc((const char *)a.v + row0 * DV * (F32IN ? 4 : 2), nk * DV * (F32IN ? 4 : 2));
  const rsrc_t rdv = make_rsrc((const char *)a.dv + row0 * DV * (a.out_f32 ? 4 : 2), nk * DV * (a.out_f32 ? 4 : 2));
  float gend[NBV];
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int col = min(32 * bv + ne, DV - 1);
    gend[bv] = a.Gl2[((st + tend) * Hkv + c) * DV + col];
    if (nsteps > 0) {  // gamma_{J+2,J} = exp2(Lam[J+1] - Lam[J]) joins the key-side factor
      const double l1 = a.Lam[((int64_t)(cbs + J + 1) * Hkv + c) * DV + col];
      const double l0 = a.Lam[((int64_t)(cbs + J) * Hkv + c) * DV + col];
      gend[bv] += (float)(l1 - l0);
    }
  }
  // half blocks (8 rows of one column block)
  float in[2][4][8];  // [slot][prefix sum, partial, qside, v][row]
  auto load_dv = [&](int u, float (&x)[4][8]) {
    const uint32_t col = min(32 * (u >> 1) + ne, DV - 1), h8 = 8 * (u & 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t o = krow(h8 + j) * DV + col;
      x[0][j] = buf_ld_f32(rgl, 4 * o);
      x[1][j] = buf_ld_f32(rdi, 4 * o);
      x[2][j] = buf_ld_f32(rqs, 4 * o);
      x[3][j] = buf_ld_in(rv, o, F32IN);
    }
  };
  // the key block's column sums of dG (its 32 keys, in a fixed order) go to
  // the reverse scan that forms dg
  float dgs[NBV];
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) dgs[bv] = 0.f;
  load_dv(0, in[0]);
#pragma unroll
  for (int u = 0; u < 2 * NBV; ++u) {
    if (u + 1 < 2 * NBV) load_dv(u + 1, in[(u + 1) & 1]);
    const int bv = u >> 1, h8 = 8 * (u & 1), col = 32 * bv + ne;
    if (col < DV)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (kb + acc_row(hhe, h8 + j) < L) {
          const uint32_t o = krow(h8 + j) * DV + col;
          const float(&x)[4][8] = in[u & 1];
          const float dvv = fast_exp2(gend[bv] - x[0][j]) * acc[bv][h8 + j] + x[1][j];
          const float dgv = x[2][j] - x[3][j] * dvv;
          buf_st_out(rdv, o, dvv, a.out_f32);
          buf_st_f32(rdg, 4 * o, dgv);
          dgs[bv] += dgv;
        }
  }
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const float t = dgs[bv] + __shfl_xor(dgs[bv], 32);
    const int col = 32 * bv + ne;
    if (hhe == 0 && col < DV) a.dg_tot[(((int64_t)gci * Hkv + c) * 4 + pr) * DV + col] = t;
  }
}

template <int DK, int DV>
hipError_t launch_bwd_dk_dv(BwdKernel kind, bool f32in, const BwdArgs &a, dim3 grid, hipStream_t st) {
#define FIX_BWD_LAUNCH(KERN)                                                                  \
  if (f32in) hipLaunchKernelGGL((KERN<DK, DV, true>), grid, dim3(kind == BK_DQ ? 256 : 512), 0, st, a); \
  else hipLaunchKernelGGL((KERN<DK, DV, false>), grid, dim3(kind == BK_DQ ? 256 : 512), 0, st, a);
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
