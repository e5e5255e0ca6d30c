// Scalar-gate backward (the forgetting-attention case, "Forgetting
// Transformer" page, abstract: the forget gate down-weights the unnormalised
// attention scores).  With one gate value per token and kv head the decay is
// a bias on the logits, s'_ij = s_ij + G_i - G_j, and m is held constant, so
//   P_ij = exp(s'_ij - m_i),  dP_ij = <delta_i, v_j>,  dS_ij = P_ij dP_ij
//   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i P_ij delta_i       (dk, dv summed over the head group)
//   dL/dG_t = sum_j dS_tj - sum_i dS_it
// and the gate gradient is the suffix sum of dL/dG over the sequence.  No
// value vector is decayed.
//
// Two kernels compute the same fp32 dS values (the same products of the same
// fp16 operands, the same exponent arithmetic in the same order): the dq
// kernel takes the row sums of dS, the dk/dv kernel the column sums.  A pair
// (i, j) with both ends at or after t enters dg_t once as a row term and once
// as a column term, which then cancel exactly, so dg_t carries only the
// pairs that cross t: no sum of nearly cancelling terms from different
// computations is ever formed.
//
// Operands are fp16 (exact copies of bf16 inputs with |x| in [2^-14, 65504]);
// probabilities come out as P / sigma with sigma = 2^-e the row scale of
// delta, so every product with the scaled delta rows is unchanged.
#pragma once
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fix {

template <int D> struct FoxPad { static constexpr int value = D < 32 ? 32 : D; };

// The probability of a pair, shared by both kernels: exp2 of s sl2 + tq - loc_j,
// where tq = (G_i - ref_J) - mb_i is the query-side term (rounded from fp64
// once per row and 64-key block) minus the row's maximum, formed in fp32.
__device__ inline float fox_pair_exp(float s, float sl2, float tq, float gk) {
  return fast_exp2(__builtin_fmaf(s, sl2, tq) - gk);
}

// ---------------------------------------------------------------------------
// dq and the row sums of dS.  Workgroup = 128 query rows (4 waves x 32) of one
// q head; keys in 64-token blocks from the first, K and V rows (fp16) double
// buffered in LDS.  A wave forms S^T = K Q^T and dP^T = V delta^T (lane =
// query row, registers = keys), so the row sum is a sum within a lane, and
// dS (as fp16) is the A operand of dQ = dS K with K read from the same rows
// through the transposing LDS load.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(256, 2) k_fox_bwd_dq(FoxBwdArgs a) {
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = FoxPad<DK>::value, NBK = DKP / 32;
  using KT = LdsTile<CH, DKP * 2>;  // K rows of a key block (padded to DKP columns)
  using VT = LdsTile<CH, DV * 2>;   // V rows of a key block
  constexpr int O_K = 0, O_V = O_K + 2 * KT::BYTES, O_G = O_V + 2 * VT::BYTES, O_R = O_G + 2 * 256;
  __shared__ __align__(1024) char smem[O_R + 2 * 256];
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  auto Gk = [&](int b) { return (const float *)(smem + O_G + b * 256); };  // the block's local prefixes
  auto Rf = [&](int b) { return (const double *)(smem + O_R + b * 256); };  // [0]: the block's reference

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // Items ordered (kv head, sequence, query block from the last, q head):
  // the workgroups of one (sequence, kv head) walk the same key blocks.
  const int nblk = pl.counts[0];
  const int idx = xcd_item(nblk * Hq);
  if (idx < 0) return;
  const int c = uniform(idx / (nblk * G)), rem = uniform(idx % (nblk * G));
  const int bi = rem / G, gq = rem % G;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, bi);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int L = uniform(pl.seq_len[s]);
  const int cb = uniform(pl.chunk_base[s]);
  const int qb = (L + QB - 1) / QB - 1 - (bi - uniform(pl.cb128[s]));
  const int hq = c * G + gq;
  const int q0 = qb * QB;
  const int nrows = min(QB, L - q0);
  const int rbase = q0 + 32 * wave;
  const int row = rbase + n;
  const bool active = 32 * wave < nrows;
  const bool rv = active && row < L;
  const int nJ = (q0 + nrows + CH - 1) / CH;
  const float sl2 = a.sl2;

  f16x8 qf[NS], df[NSV];
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int i = 0; i < NS; ++i) qf[i] = rv ? *(const f16x8 *)(a.Q16 + ((st + row) * Hq + hq) * DKP + 16 * i + 8 * hh) : zf;
#pragma unroll
  for (int i = 0; i < NSV; ++i)
    df[i] = rv ? *(const f16x8 *)(a.D16 + ((st + row) * Hq + hq) * FoxPad<DV>::value + 16 * i + 8 * hh) : zf;
  // rows past the end: an infinite offset zeroes their probabilities
  const float mbr = rv ? a.mb[(st + row) * Hq + hq] : INFINITY;
  const int rr = min(row, L - 1);
  const double grow = a.ref[(int64_t)(cb + rr / CH) * Hkv + c] + (double)a.loc[(st + rr) * Hkv + c];

  uint32_t ok[KT::NW], ov[VT::NW];
  KT::lane_offsets(Hkv * DKP * 2, wave, lane, ok);
  VT::lane_offsets(Hkv * DV * 2, wave, lane, ov);
  // Copies of key block J, untracked (the loop reads the other buffer while
  // they are in flight; the wait at the top of each step orders them).
  auto stage = [&](int J, int b) {
    const int64_t kr = (st + J * CH) * Hkv + c;
    const int64_t nrow = (int64_t)(L - J * CH) * Hkv;  // rows past the sequence read as zeros
    const u32x4 sk = rsrc_words(a.K16 + kr * DKP, nrow * DKP * 2);
#pragma unroll
    for (int t = 0; t < KT::NW; ++t) KT::dma_piece_untracked(Ks(b), sk, ok, t, wave);
    const u32x4 sv = rsrc_words(a.V16 + kr * DV, nrow * DV * 2);
#pragma unroll
    for (int t = 0; t < VT::NW; ++t) VT::dma_piece_untracked(Vs(b), sv, ov, t, wave);
    dma4_untracked(smem + O_G + b * 256, rsrc_words(a.loc + kr, nrow * 4), (uint32_t)lane * Hkv * 4);
    dma4_untracked(smem + O_R + b * 256, rsrc_words(a.ref + (int64_t)(cb + J) * Hkv + c, 8), (uint32_t)lane * 4);
  };

  f32x16 acc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) acc[b] = zero16();
  float rsum = 0.f;
  // Per-lane LDS addresses in buffer 0: the K and V row fragments, the
  // transposed K pieces and the key-side exponent terms.
  uint32_t ak[NS], av[NSV], at[NBK][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) ak[i] = lds_addr(Ks(0)) + KT::off(n, 2 * i + hh);
#pragma unroll
  for (int i = 0; i < NSV; ++i) av[i] = lds_addr(Vs(0)) + VT::off(n, 2 * i + hh);
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    uint32_t o[2];
    tr_offsets<KT>(32 * bk, lane, o);
    at[bk][0] = lds_addr(Ks(0)) + o[0];
    at[bk][1] = lds_addr(Ks(0)) + o[1];
  }
  const uint32_t ag = lds_addr(smem + O_G) + 4 * (4 * hh);

  if (nJ > 0) stage(0, 0);
  for (int J = 0; J < nJ; ++J) {
    const int b = J & 1;
    wait_all();
    __syncthreads();  // block J landed in every wave's copy; block J - 1's readers are done
    if (J + 1 < nJ) stage(J + 1, b ^ 1);
    const int k0 = J * CH;
    if (!active || k0 > rbase + 31) continue;
    const float tqr = (float)(grow - Rf(b)[0]) - mbr;
    const bool mask = !(k0 + CH - 1 <= rbase && k0 + CH <= L);
    const uint32_t bo = opaque(b * KT::BYTES), bv = opaque(b * VT::BYTES), bg = opaque(b * 256);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (k0 + 32 * h > rbase + 31) break;  // the half lies after every row of the wave
      // S^T and dP^T, their chains alternating, operand reads four products
      // ahead; the half's key-side exponent terms read first
      f32x4 g4[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        g4[q4] = *(const __attribute__((address_space(3))) f32x4 *)lds_at(ag + bg + 4 * (32 * h + 8 * q4));
      f32x16 sc = zero16(), dp = zero16();
      {
        constexpr int NM = NS > NSV ? NS : NSV;
        f16x8 fk[NM], fv[NM];
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i < NS) fk[i] = lds_row16(ak[i] + bo + 32 * h * (DKP * 2));
          if (i < NSV) fv[i] = lds_row16(av[i] + bv + 32 * h * (DV * 2));
        }
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          if (i < NS) sc = mma32(fk[i], qf[i], sc);
          if (i < NSV) dp = mma32(fv[i], df[i], dp);
        }
        constexpr int NP = NS + NSV, LA = NP < 4 ? NP : 4;
        __builtin_amdgcn_sched_group_barrier(0x100, LA + 4, 0);
#pragma unroll
        for (int m = 0; m < NP - LA; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      f16x8 dsf[2];
      auto probs = [&](auto mc) {
        constexpr bool MASK = decltype(mc)::value;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * q4 + e;
            float p = fox_pair_exp(sc[j], sl2, tqr, g4[q4][e]);
            if (MASK) {
              const int key = k0 + 32 * h + acc_row(hh, j);
              p = (key <= row && key < L) ? p : 0.f;
            }
            const float ds = p * dp[j];
            rsum += ds;
            dsf[j >> 3][j & 7] = (_Float16)ds;
          }
        }
      };
      if (mask) probs(std::true_type());
      else probs(std::false_type());
      // dQ += dS K, K read transposed, reads two products ahead
      {
        f16x4 tp[NBK][2][2];
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 2; ++t) tp[bk][u][t] = lds_tr8(at[bk][t] + bo + (32 * h + 16 * u) * (DKP * 2));
#pragma unroll
        for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[bk] = mma32(dsf[u], __builtin_shufflevector(tp[bk][u][0], tp[bk][u][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[bk]);
        constexpr int NP = 2 * NBK, LA = 2;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
        for (int m = 0; m < NP - LA; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  rsum += __shfl_xor(rsum, 32);
  if (!active) return;
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = rbase + acc_row(hh, j);
      if (r < L) store_out(a.dq, ((st + r) * Hq + hq) * DK + col, a.scale * acc[bk][j], a.out_f32);
    }
  }
  if (hh == 0 && row < L) a.rsum[(st + row) * Hq + hq] = rsum;
}

// ---------------------------------------------------------------------------
// dk, dv and the column sums of dS (over the head group).  Workgroup = 128
// keys of one kv head and 8 waves: the 32 keys of pair p are shared by wave
// p (A) and wave p + 4 (B), which the hardware places on the same SIMD.  The
// query rows from the key chunk's first on go in 64-row steps (from the
// sequence end down, every q head of the group per slice), Q rows (three
// stages) and scaled delta rows (two stages, fp16) in LDS.  Step k runs as
// two phases, split by a barrier:
//   phase 1  A: S_k = Q K^T, P_k (fp32) into LDS
//            B: the copies of step k + 1, dK += dS_{k-1}^T Q_{k-1} with the
//               dS it formed in step k - 1, then dP_k = delta V^T
//   phase 2  A: dV += P_k^T delta_k
//            B: dS_k = P_k dP_k (kept in registers for the next step) and
//               its column sums
// so that each wave's vector work (A's exponentials, B's products of P and
// dP) runs while the other wave's matrix products fill the SIMD.  Each wave
// holds one accumulator set and one key-side operand (about half the
// registers of a wave doing all four products), so two waves share each
// SIMD.  The transposed operands are the LDS rows read with the transposing
// load.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(512, 1) k_fox_bwd_dkv(FoxBwdArgs a) {
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = FoxPad<DK>::value, DVP = FoxPad<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  constexpr int RS = 64;            // query rows per step (two halves of 32)
  using QT = LdsTile<RS, DKP * 2>;  // Q rows of a step (padded)
  using DT = LdsTile<RS, DVP * 2>;  // scaled delta rows of a step (padded)
  using QW = typename QT::template Waves<4>;  // copies issued by the four B waves
  using DW = typename DT::template Waves<4>;
  constexpr int O_Q = 0, O_D = O_Q + 3 * QT::BYTES, O_M = O_D + 2 * DT::BYTES, O_L = O_M + 2 * 256;
  constexpr int O_R = O_L + 2 * 256, O_T = O_R + 2 * 256, O_P = O_T + 4 * 256;
  constexpr int PEX = 2 * 64 * 16 * 4;  // one pair's P of a step: two halves, 64 lanes x 16 floats
  __shared__ __align__(1024) char smem[O_P + 4 * PEX];
  auto Rf = [&](int b) { return (const double *)(smem + O_R + b * 256); };  // [0]: the rows' block reference

  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int nchunk = pl.counts[0];
  const int idx = xcd_item(nchunk * Hkv);
  if (idx < 0) return;
  const int c = uniform(idx / nchunk), gci = uniform(idx % nchunk);
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gci);
  const int J = gci - uniform(pl.cb128[s]);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int L = uniform(pl.seq_len[s]);
  const int cb = uniform(pl.chunk_base[s]);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool isA = wave < 4;
  const int pr = wave & 3;
  float *gqt = (float *)(smem + O_T + 256 * pr);  // the step's query-side exponent terms (A)
  float *pex = (float *)(smem + O_P + PEX * pr);  // the pair's P of the step, [half][quad][lane][4]
  const int kb = J * CB + 32 * pr;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;
  const int r00 = J * CB;
  const int nsl = (L - r00 + RS - 1) / RS;
  const int nsteps = nsl * G;

  // Key-side operand: K for S (A), V for dP (B).
  constexpr int NKS = NS > NSV ? NS : NSV;
  f16x8 kf[NKS];
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int i = 0; i < NKS; ++i) {
    if (isA) kf[i] = (kv && i < NS) ? *(const f16x8 *)(a.K16 + ((st + key) * Hkv + c) * DKP + 16 * i + 8 * hh) : zf;
    else kf[i] = (kv && i < NSV) ? *(const f16x8 *)(a.V16 + ((st + key) * Hkv + c) * DV + 16 * i + 8 * hh) : zf;
  }
  const float gk = (isA && kv) ? a.loc[(st + key) * Hkv + c] : 0.f;
  const double refk = (isA && kb < L) ? a.ref[(int64_t)(cb + kb / CH) * Hkv + c] : 0.0;

  // Per-lane LDS addresses in stage 0: the first product's row fragments (Q
  // for A, delta for B) and the second's transposed pieces (delta for A, Q
  // for B); a step adds its stage's offset.
  const uint32_t sbase = lds_addr(smem);
  constexpr int NBA = NBK > NBV ? NBK : NBV;
  uint32_t a1[NKS], a2[NBA][2];
#pragma unroll
  for (int i = 0; i < NKS; ++i)
    a1[i] = sbase + (isA ? O_Q + QT::off(n, 2 * i + hh) : O_D + DT::off(n, 2 * i + hh));
#pragma unroll
  for (int bo = 0; bo < NBA; ++bo) {
    uint32_t oq[2], od[2];
    tr_offsets<QT>(32 * bo, lane, oq);
    tr_offsets<DT>(32 * bo, lane, od);
#pragma unroll
    for (int t = 0; t < 2; ++t) a2[bo][t] = sbase + (isA ? O_D + od[t] : O_Q + oq[t]);
  }
  const uint32_t apx = lds_addr(pex) + 16 * lane, agq = lds_addr(gqt) + 4 * (4 * hh);
  const uint32_t rb1 = isA ? 2 * DKP : 2 * DVP, rb2 = isA ? 2 * DVP : 2 * DKP;  // row bytes of the two tiles

  uint32_t oq[QW::NWW], od[DW::NWW];
  const int wb = wave & 3;
  QW::lane_offsets(Hq * DKP * 2, wb, lane, oq);
  DW::lane_offsets(Hq * DVP * 2, wb, lane, od);
  // Copies of the step at (slice sl, q head gq) into Q stage qs and stage ds
  // (B waves only).
  auto stage = [&](int sl, int gq, int qs, int ds) {
    const int h = c * G + gq, r0 = r00 + RS * sl;
    const int64_t qr = (st + r0) * Hq + h;
    const int64_t nrow = L - r0;  // rows past the sequence read as zeros
    QW::dma_untracked(smem + O_Q + qs * QT::BYTES, rsrc_words(a.Q16 + qr * DKP, nrow * Hq * DKP * 2), oq, wb);
    DW::dma_untracked(smem + O_D + ds * DT::BYTES, rsrc_words(a.D16 + qr * DVP, nrow * Hq * DVP * 2), od, wb);
    if (wb == 0) {
      dma4_untracked(smem + O_M + ds * 256, rsrc_words(a.mb + qr, nrow * Hq * 4), (uint32_t)lane * Hq * 4);
      dma4_untracked(smem + O_L + ds * 256, rsrc_words(a.loc + (st + r0) * Hkv + c, nrow * Hkv * 4),
                     (uint32_t)lane * Hkv * 4);
      dma4_untracked(smem + O_R + ds * 256, rsrc_words(a.ref + (int64_t)(cb + r0 / CH) * Hkv + c, 8),
                     (uint32_t)lane * 4);
    }
  };

  f32x16 acc[NBA];  // A: dV, B: dK
#pragma unroll
  for (int b = 0; b < NBA; ++b) acc[b] = zero16();
  float csum = 0.f;
  constexpr bool SAME = NS == NSV;
  const int n1 = isA ? NS : NSV;     // k slabs of the first product
  const int n2 = isA ? NBV : NBK;    // output blocks of the second

  // Second product, both halves: acc[b] += of[h2][u]^T (tile rows 32 h2 + 16 u,
  // read transposed at base + off).  The MFMAs go output block fastest (four
  // independent chains); the reads run LA products ahead of them.
  auto second = [&](const f16x8 (&of)[2][2], uint32_t off) {
    constexpr int NM = 4 * NBA, LA = 4;
    f16x4 tp[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int hu = m / NBA, b = m % NBA;
      if (SAME || b < n2)
#pragma unroll
        for (int t = 0; t < 2; ++t) tp[m][t] = lds_tr8p(lds_at(a2[b][t] + off) + 16 * hu * rb2);
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int hu = m / NBA, b = m % NBA;
      if (SAME || b < n2)
        acc[b] = mma32(of[hu >> 1][hu & 1], __builtin_shufflevector(tp[m][0], tp[m][1], 0, 1, 2, 3, 4, 5, 6, 7), acc[b]);
    }
    if (SAME) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
      for (int m = 0; m < NM - LA; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Phase 1's first product, the same shape for both waves (A: S = Q K^T, B:
  // dP = delta V^T); lane = key, register j = row r0 + 32 h2 + acc_row(hh, j).
  // The two halves' chains alternate and the reads run four products ahead.
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
    if (SAME) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int m = 0; m < 2 * NKS - 4; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // The two waves of a pair run separate loops with the same barriers, so
  // each keeps only its own values live.
  if (isA) {
    const uint32_t agq_ = opaque(agq), apx_ = opaque(apx);
    int sl = nsl - 1, gq = 0;
    for (int k = 0; k < nsteps; ++k) {
      const int qs = k % 3, ds = k & 1;
      wait_all();
      __syncthreads();  // step k landed; every read of step k - 1 is done
      const int r0 = r00 + RS * sl;
      const bool mask = r0 < kb + 31 || r0 + RS > L;
      // the step's query-side exponent terms minus the row maxima
      const float gv = (float)((Rf(ds)[0] + (double)((const float *)(smem + O_L + ds * 256))[lane]) - refk);
      gqt[lane] = gv - ((const float *)(smem + O_M + ds * 256))[lane];
      f32x16 xr[2];
      first(qs * QT::BYTES, xr);
      // P (fp32) of both halves into the pair's exchange buffer; P (fp16)
      // kept as the A operand of dV
      f16x8 pf[2][2];
      auto probs = [&](auto mc) {
        constexpr bool MASK = decltype(mc)::value;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x4 tv[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            tv[q4] = *(const __attribute__((address_space(3))) f32x4 *)(lds_at(agq_) + 4 * (32 * h2 + 8 * q4));
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 p4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = 4 * q4 + e;
              float p = fox_pair_exp(xr[h2][j], sl2, tv[q4][e], gk);
              if (MASK) {
                const int r = r0 + 32 * h2 + acc_row(hh, j);
                p = (key <= r && r < L) ? p : 0.f;
              }
              p4[e] = p;
              pf[h2][j >> 3][j & 7] = (_Float16)p;
            }
            *(__attribute__((address_space(3))) f32x4 *)(lds_at(apx_) + 16 * 64 * (h2 * 4 + q4)) = p4;
          }
        }
      };
      if (mask) probs(std::true_type());
      else probs(std::false_type());
      lds_barrier();  // P is in LDS
      second(pf, ds * DT::BYTES);  // dV += P^T delta
      if (++gq == G) { gq = 0; --sl; }
    }
  } else {
    const uint32_t apx_ = opaque(apx);
    f16x8 dsp[2][2];  // dS of the previous step (both halves), the A operand of its dK product
    int sl = nsl - 1, gq = 0;
    if (nsteps > 0) stage(sl, gq, 0, 0);
    for (int k = 0; k < nsteps; ++k) {
      const int ds = k & 1;
      int nsl_ = sl, ngq = gq + 1;
      if (ngq == G) { ngq = 0; --nsl_; }
      wait_all();
      __syncthreads();  // step k landed; every read of step k - 1 is done
      if (k + 1 < nsteps) stage(nsl_, ngq, (k + 1) % 3, ds ^ 1);
      if (k > 0) second(dsp, ((k + 2) % 3) * QT::BYTES);  // dK of the previous step
      f32x16 xr[2];
      first(ds * DT::BYTES, xr);
      lds_barrier();  // A's P is in LDS
      f32x4 p4[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          p4[h2][q4] = *(const __attribute__((address_space(3))) f32x4 *)(lds_at(apx_) + 16 * 64 * (h2 * 4 + q4));
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float d = p4[h2][j >> 2][j & 3] * xr[h2][j];  // dS, exactly as the dq kernel forms it
          csum += d;
          dsp[h2][j >> 3][j & 7] = (_Float16)d;
        }
      sl = nsl_;
      gq = ngq;
    }
    if (nsteps > 0) second(dsp, ((nsteps - 1) % 3) * QT::BYTES);  // dK of the last step
  }
  csum += __shfl_xor(csum, 32);
  if (kb >= L) return;
  if (isA) {
#pragma unroll
    for (int bv = 0; bv < NBV; ++bv) {
      const int col = 32 * bv + n;
      if (col >= DV) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (kj < L) store_out(a.dv, ((st + kj) * Hkv + c) * DV + col, acc[bv][j], a.out_f32);
      }
    }
  } else {
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      const int col = 32 * bk + n;
      if (col >= DK) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kj = kb + acc_row(hh, j);
        if (kj < L) store_out(a.dk, ((st + kj) * Hkv + c) * DK + col, a.scale * acc[bk][j], a.out_f32);
      }
    }
    if (hh == 0 && kv) a.csum[(st + key) * Hkv + c] = csum;
  }
}

template <int DK>
hipError_t launch_fox_bwd_dk(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st) {
#define FIX_FOX_BWD(DVC)                                                                              \
  case DVC:                                                                                           \
    if (kind == FK_DQ) hipLaunchKernelGGL((k_fox_bwd_dq<DK, DVC>), dim3(grid), dim3(256), 0, st, a);  \
    else hipLaunchKernelGGL((k_fox_bwd_dkv<DK, DVC>), dim3(grid), dim3(512), 0, st, a);               \
    break;
  switch (dv) {
    FIX_FOX_BWD(16)
    FIX_FOX_BWD(32)
    FIX_FOX_BWD(64)
    FIX_FOX_BWD(128)
    default: return hipErrorInvalidValue;
  }
#undef FIX_FOX_BWD
  return hipGetLastError();
}

}  // namespace fix
