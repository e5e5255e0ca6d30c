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
#include "common.h"
#include "launch.h"

namespace fix {

template <int D> struct FoxPad { static constexpr int value = D < 32 ? 32 : D; };

// The exponent of a pair, shared by both kernels: s sl2 - mb + (G_i - ref_J) - loc_j
// with the query-side term rounded from fp64 once per (row, 64-key block).
__device__ inline float fox_pair_exp(float s, float sl2, float mb, float gq, float gk) {
  return fast_exp2((__builtin_fmaf(s, sl2, -mb) + gq) - gk);
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

  if (nJ > 0) stage(0, 0);
  for (int J = 0; J < nJ; ++J) {
    const int b = J & 1;
    wait_all();
    __syncthreads();  // block J landed in every wave's copy; block J - 1's readers are done
    if (J + 1 < nJ) stage(J + 1, b ^ 1);
    const int k0 = J * CH;
    if (!active || k0 > rbase + 31) continue;
    const float gqr = (float)(grow - Rf(b)[0]);
    const bool mask = !(k0 + CH - 1 <= rbase && k0 + CH <= L);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (k0 + 32 * h > rbase + 31) break;  // the half lies after every row of the wave
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const f16x8 *)(Ks(b) + KT::off(32 * h + n, 2 * i + hh)), qf[i], sc);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)(Vs(b) + VT::off(32 * h + n, 2 * i + hh)), df[i], dp);
      f16x8 dsf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 g4 = *(const float4 *)(Gk(b) + 32 * h + 8 * q4 + 4 * hh);
        const float gk[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * q4 + e;
          float p = fox_pair_exp(sc[j], sl2, mbr, gqr, gk[e]);
          if (mask) {
            const int key = k0 + 32 * h + acc_row(hh, j);
            p = (key <= row && key < L) ? p : 0.f;
          }
          const float ds = p * dp[j];
          rsum += ds;
          dsf[j >> 3][j & 7] = (_Float16)ds;
        }
      }
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[bk] = mma32(dsf[u], tr_frag<KT>(Ks(b), 32 * h + 16 * u, 32 * bk, lane), acc[bk]);
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
// keys (4 waves x 32) of one kv head; for each q head of the group, the query
// rows from the key chunk's first on in 64-row steps, Q rows and scaled delta
// rows (fp16) double buffered in LDS.  A wave forms S = Q K^T and dP = delta
// V^T (lane = key, registers = query rows), so P and dS are the A operands of
// dV = P^T delta and dK = dS^T Q, whose B operands are the same LDS rows read
// with the transposing load; the column sum is a sum within a lane.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void __launch_bounds__(256, 1) k_fox_bwd_dkv(FoxBwdArgs a) {
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = FoxPad<DK>::value, DVP = FoxPad<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  constexpr int RS = 64;            // query rows per step (two halves of 32)
  using QT = LdsTile<RS, DKP * 2>;  // Q rows of the step (padded)
  using DT = LdsTile<RS, DVP * 2>;  // scaled delta rows of the step (padded)
  constexpr int O_Q = 0, O_D = O_Q + 2 * QT::BYTES, O_M = O_D + 2 * DT::BYTES, O_L = O_M + 2 * 256;
  constexpr int O_R = O_L + 2 * 256, O_T = O_R + 2 * 256;
  __shared__ __align__(1024) char smem[O_T + 4 * 256];
  auto Qs = [&](int b) { return smem + O_Q + b * QT::BYTES; };
  auto Ds = [&](int b) { return smem + O_D + b * DT::BYTES; };
  auto Ms = [&](int b) { return (const float *)(smem + O_M + b * 256); };  // row offsets mb
  auto Lc = [&](int b) { return (const float *)(smem + O_L + b * 256); };  // rows' local gate prefixes
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
  float *gqt = (float *)(smem + O_T + 256 * wave);  // the step's query-side exponent terms, per wave
  const int kb = J * CB + 32 * wave;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;
  const int r00 = J * CB;
  const int nsl = (L - r00 + RS - 1) / RS;
  const int nsteps = G * nsl;

  f16x8 kf[NS], vf[NSV];
  const f16x8 zf = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int i = 0; i < NS; ++i) kf[i] = kv ? *(const f16x8 *)(a.K16 + ((st + key) * Hkv + c) * DKP + 16 * i + 8 * hh) : zf;
#pragma unroll
  for (int i = 0; i < NSV; ++i) vf[i] = kv ? *(const f16x8 *)(a.V16 + ((st + key) * Hkv + c) * DV + 16 * i + 8 * hh) : zf;
  const float gk = kv ? a.loc[(st + key) * Hkv + c] : 0.f;
  const double refk = kb < L ? a.ref[(int64_t)(cb + kb / CH) * Hkv + c] : 0.0;

  uint32_t oq[QT::NW], od[DT::NW];
  QT::lane_offsets(Hq * DKP * 2, wave, lane, oq);
  DT::lane_offsets(Hq * DVP * 2, wave, lane, od);
  auto stage = [&](int k, int b) {
    const int gq = k / nsl, sl = k % nsl;
    const int h = c * G + gq, r0 = r00 + RS * sl;
    const int64_t qr = (st + r0) * Hq + h;
    const int64_t nrow = L - r0;  // rows past the sequence read as zeros
    const u32x4 sq = rsrc_words(a.Q16 + qr * DKP, nrow * Hq * DKP * 2);
#pragma unroll
    for (int t = 0; t < QT::NW; ++t) QT::dma_piece_untracked(Qs(b), sq, oq, t, wave);
    const u32x4 sd = rsrc_words(a.D16 + qr * DVP, nrow * Hq * DVP * 2);
#pragma unroll
    for (int t = 0; t < DT::NW; ++t) DT::dma_piece_untracked(Ds(b), sd, od, t, wave);
    dma4_untracked(smem + O_M + b * 256, rsrc_words(a.mb + qr, nrow * Hq * 4), (uint32_t)lane * Hq * 4);
    dma4_untracked(smem + O_L + b * 256, rsrc_words(a.loc + (st + r0) * Hkv + c, nrow * Hkv * 4),
                   (uint32_t)lane * Hkv * 4);
    dma4_untracked(smem + O_R + b * 256, rsrc_words(a.ref + (int64_t)(cb + r0 / CH) * Hkv + c, 8), (uint32_t)lane * 4);
  };

  f32x16 accK[NBK], accV[NBV];
#pragma unroll
  for (int b = 0; b < NBK; ++b) accK[b] = zero16();
#pragma unroll
  for (int b = 0; b < NBV; ++b) accV[b] = zero16();
  float csum = 0.f;

  if (nsteps > 0) stage(0, 0);
  for (int k = 0; k < nsteps; ++k) {
    const int b = k & 1;
    wait_all();
    __syncthreads();
    if (k + 1 < nsteps) stage(k + 1, b ^ 1);
    const int r0 = r00 + RS * (k % nsl);
    if (kb >= L || r0 + RS - 1 < kb) continue;  // no key of the wave, or every row before them
    // query-side term of each row (lane r: row r0 + r), as the dq kernel forms it
    gqt[lane] = (float)((Rf(b)[0] + (double)Lc(b)[lane]) - refk);
    const bool mask = r0 < kb + 31 || r0 + RS > L;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int rb2 = r0 + 32 * h2;
      if (rb2 + 31 < kb) continue;  // the half lies before every key of the wave
      if (rb2 >= L) break;
      float4 mq[4], gv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        mq[q4] = *(const float4 *)(Ms(b) + 32 * h2 + 8 * q4 + 4 * hh);
        gv[q4] = *(const float4 *)(gqt + 32 * h2 + 8 * q4 + 4 * hh);
      }
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const f16x8 *)(Qs(b) + QT::off(32 * h2 + n, 2 * i + hh)), kf[i], sc);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)(Ds(b) + DT::off(32 * h2 + n, 2 * i + hh)), vf[i], dp);
      f16x8 pf[2], dsf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float mv[4] = {mq[q4].x, mq[q4].y, mq[q4].z, mq[q4].w};
        const float gr[4] = {gv[q4].x, gv[q4].y, gv[q4].z, gv[q4].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * q4 + e;
          float p = fox_pair_exp(sc[j], sl2, mv[e], gr[e], gk);
          if (mask) {
            const int r = rb2 + acc_row(hh, j);
            p = (key <= r && r < L) ? p : 0.f;
          }
          const float ds = p * dp[j];
          csum += ds;
          pf[j >> 3][j & 7] = (_Float16)p;
          dsf[j >> 3][j & 7] = (_Float16)ds;
        }
      }
#pragma unroll
      for (int bv = 0; bv < NBV; ++bv)
#pragma unroll
        for (int u = 0; u < 2; ++u) accV[bv] = mma32(pf[u], tr_frag<DT>(Ds(b), 32 * h2 + 16 * u, 32 * bv, lane), accV[bv]);
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u) accK[bk] = mma32(dsf[u], tr_frag<QT>(Qs(b), 32 * h2 + 16 * u, 32 * bk, lane), accK[bk]);
    }
  }
  csum += __shfl_xor(csum, 32);
  if (kb >= L) return;
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) store_out(a.dk, ((st + kj) * Hkv + c) * DK + col, a.scale * accK[bk][j], a.out_f32);
    }
  }
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int col = 32 * bv + n;
    if (col >= DV) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) store_out(a.dv, ((st + kj) * Hkv + c) * DV + col, accV[bv][j], a.out_f32);
    }
  }
  if (hh == 0 && kv) a.csum[(st + key) * Hkv + c] = csum;
}

template <int DK>
hipError_t launch_fox_bwd_dk(FoxBwdKernel kind, int dv, const FoxBwdArgs &a, int grid, hipStream_t st) {
#define FIX_FOX_BWD(DVC)                                                                              \
  case DVC:                                                                                           \
    if (kind == FK_DQ) hipLaunchKernelGGL((k_fox_bwd_dq<DK, DVC>), dim3(grid), dim3(256), 0, st, a);  \
    else hipLaunchKernelGGL((k_fox_bwd_dkv<DK, DVC>), dim3(grid), dim3(256), 0, st, a);               \
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
