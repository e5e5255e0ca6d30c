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

// ---------------------------------------------------------------------------
// Within-chunk contributions to dq: wave w of the workgroup owns query rows
// c0 + 32w .. +31 of one 128-chunk and one q head.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256) k_bwd_intra_dq(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, NBK = Pad32<DK>::value / 32;
  const Plan &pl = a.plan;
  const int gc = blockIdx.x, hq = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = (gc - pl.cb128[s]) * CB;
  const int L = pl.seq_len[s];
  const int64_t st = pl.seq_start[s];
  const int Hq = a.Hq, Hkv = a.Hkv, c = hq / (Hq / Hkv);
  const int r0 = c0 + 32 * wave;
  if (r0 >= L) return;
  const int row = r0 + n;
  const bool rv = row < L;
  const float sl2 = a.sl2;
  auto gl = [&](int tok, int d) { return a.Gl2[((st + tok) * Hkv + c) * DV + d]; };
  auto vv = [&](int tok, int d) { return load_in(a.v, ((st + tok) * Hkv + c) * DV + d, F32IN); };

  kfrag qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = rv ? IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();
  const float mbn = rv ? a.mb[(st + row) * Hq + hq] : INFINITY;
  const float sgn = rv ? a.sig[(st + row) * Hq + hq] : 0.f;
  const float *drow = a.delta + ((st + row) * Hq + hq) * DV;

  f32x16 acc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) acc[b] = zero16();

  for (int b = 0; b <= wave; ++b) {
    const int kb = c0 + 32 * b;
    const int key = kb + n;
    const bool diag = b == wave;
    const int ref = diag ? kb - 1 : kb + 31;  // token the decay is split at (c0 - 1: chunk start)
    // S^T[key][row]
    f32x16 sc = zero16();
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      kfrag kf = key < L ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
      sc = mma32(kf, qf[i], sc);
    }
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = fast_exp2(sc[j] * sl2 - mbn);
      if (diag && acc_row(hh, j) > n) p[j] = 0.f;
    }
    // dP^T[key][row] = sum_d Vx[key][d] dx[row][d]
    f32x16 dp = zero16();
    bool direct = false;
    if (!diag) {
#pragma unroll
      for (int sv = 0; sv < NSV; ++sv) {
        f16x8 va, db;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 16 * sv + 8 * hh + e;
          const float gr = gl(ref, d);
          va[e] = (_Float16)(fast_exp2(gr - gl(key, d)) * vv(key, d));
          db[e] = (_Float16)(rv ? fast_exp2(gl(row, d) - gr) * drow[d] * sgn : 0.f);
        }
        dp = mma32(va, db, dp);
      }
    } else {
      const int klast = min(kb + 31, L - 1);
      float rng = 0.f;
#pragma unroll
      for (int sv = 0; sv < NSV; ++sv)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 16 * sv + 8 * hh + e;
          rng = fmaxf(rng, (ref >= c0 ? gl(ref, d) : 0.f) - gl(klast, d));
        }
      direct = __any(rng > BGUARD);
      if (!direct) {
#pragma unroll
        for (int sv = 0; sv < NSV; ++sv) {
          bf16x8 vh, vl, dh_, dl_;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 16 * sv + 8 * hh + e;
            const float gr = ref >= c0 ? gl(ref, d) : 0.f;
            const float vx = key < L ? fast_exp2(gr - gl(key, d)) * vv(key, d) : 0.f;
            const float dx = rv ? fast_exp2(gl(row, d) - gr) * drow[d] * sgn : 0.f;
            split_bf16(vx, vh, vl, e);
            split_bf16(dx, dh_, dl_, e);
          }
          dp = mma32(vh, dh_, dp);
          dp = mma32(vh, dl_, dp);
          dp = mma32(vl, dh_, dp);
        }
      } else {
        // exact per-pair decays (rare: block gate range beyond 2^BGUARD)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kj = kb + acc_row(hh, j);
          float t = 0.f;
          if (rv && kj <= row) {
#pragma unroll 1
            for (int d = 0; d < DV; ++d) t += drow[d] * sgn * fast_exp2(gl(row, d) - gl(kj, d)) * vv(kj, d);
          }
          dp[j] = t;
        }
      }
    }
    f16x8 dsf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) dsf[u][i] = (_Float16)(p[8 * u + i] * dp[8 * u + i]);
    // dQ[row][dk] += dS[row][key] K[key][dk]
#pragma unroll
    for (int bk = 0; bk < NBK; ++bk) {
      const int col = 32 * bk + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f16x8 kt;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kk = kb + slab_key(u, hh, i);
          kt[i] = (_Float16)((col < DK && kk < L) ? load_in(a.k, ((st + kk) * Hkv + c) * DK + col, F32IN) : 0.f);
        }
        acc[bk] = mma32(dsf[u], kt, acc[bk]);
      }
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
// Near contributions to dk, dv: wave w owns keys c0 + 32w .. +31 of one
// 128-chunk and one kv head, summed over the head group, against the queries
// of the same chunk and of the next one (the pairs with the largest decay
// weights).  dP is fp16 except on the diagonal block; P^T dhat for dv is
// always bf16x3, because dv feeds the gate gradient, whose suffix sums
// accumulate the rounding of every token.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256) k_bwd_intra_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, NBK = Pad32<DK>::value / 32, NBV = Pad32<DV>::value / 32;
  const Plan &pl = a.plan;
  const int gc = blockIdx.x, c = blockIdx.y;
  if (gc >= pl.counts[0]) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int c0 = (gc - pl.cb128[s]) * CB;
  const int L = pl.seq_len[s];
  const int64_t st = pl.seq_start[s];
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int kb = c0 + 32 * wave;
  if (kb >= L) return;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;
  // log2 prefix sums relative to the start of this chunk, continued into the next chunk
  auto glx = [&](int tok, int d) {
    if (tok < c0) return 0.f;
    float gv = a.Gl2[((st + tok) * Hkv + c) * DV + d];
    if (tok >= c0 + CB) gv += a.Gl2[((st + c0 + CB - 1) * Hkv + c) * DV + d];
    return gv;
  };
  auto vv = [&](int tok, int d) { return load_in(a.v, ((st + tok) * Hkv + c) * DV + d, F32IN); };

  kfrag kf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    kf[i] = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
  f32x16 accK[NBK], accV[NBV];
#pragma unroll
  for (int b = 0; b < NBK; ++b) accK[b] = zero16();
#pragma unroll
  for (int b = 0; b < NBV; ++b) accV[b] = zero16();

  for (int gq = 0; gq < G; ++gq) {
    const int h = c * G + gq;
    for (int qa = wave; qa < 2 * CB / 32; ++qa) {
      const int q0 = c0 + 32 * qa;
      if (q0 >= L) break;
      const bool diag = qa == wave;
      const int ref = q0 - 1;  // token the decay is split at
      const int qrow = q0 + n;
      const bool qv = qrow < L;
      // S[q][key]
      f32x16 sc = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        kfrag qf = qv ? IF::load(a.q, ((st + qrow) * Hq + h) * DK + 16 * i + 8 * hh) : IF::zero();
        sc = mma32(qf, kf[i], sc);
      }
      float p[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int qj = q0 + acc_row(hh, j);
        const float mbq = qj < L ? a.mb[(st + qj) * Hq + h] : INFINITY;
        p[j] = fast_exp2(sc[j] * sl2 - mbq);
        if (diag && acc_row(hh, j) < n) p[j] = 0.f;
      }
      const float *dq_row = a.delta + ((st + qrow) * Hq + h) * DV;
      const float sgq = qv ? a.sig[(st + qrow) * Hq + h] : 0.f;
      // dP[q][key] = sum_d dx[q][d] Vx[key][d]
      f32x16 dp = zero16();
      bool direct = false;
      if (!diag) {
#pragma unroll
        for (int sv = 0; sv < NSV; ++sv) {
          f16x8 da, vb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 16 * sv + 8 * hh + e;
            const float gr = glx(ref, d);
            da[e] = (_Float16)(qv ? fast_exp2(glx(qrow, d) - gr) * dq_row[d] * sgq : 0.f);
            vb[e] = (_Float16)(fast_exp2(gr - glx(key, d)) * vv(key, d));
          }
          dp = mma32(da, vb, dp);
        }
      } else {
        const int klast = min(kb + 31, L - 1);
        float rng = 0.f;
#pragma unroll
        for (int sv = 0; sv < NSV; ++sv)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = 16 * sv + 8 * hh + e;
            rng = fmaxf(rng, glx(ref, d) - glx(klast, d));
          }
        direct = __any(rng > BGUARD);
        if (!direct) {
#pragma unroll
          for (int sv = 0; sv < NSV; ++sv) {
            bf16x8 dh_, dl_, vh, vl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int d = 16 * sv + 8 * hh + e;
              const float gr = glx(ref, d);
              const float dx = qv ? fast_exp2(glx(qrow, d) - gr) * dq_row[d] * sgq : 0.f;
              const float vx = kv ? fast_exp2(gr - glx(key, d)) * vv(key, d) : 0.f;
              split_bf16(dx, dh_, dl_, e);
              split_bf16(vx, vh, vl, e);
            }
            dp = mma32(dh_, vh, dp);
            dp = mma32(dl_, vh, dp);
            dp = mma32(dh_, vl, dp);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int qj = q0 + acc_row(hh, j);
            float t = 0.f;
            if (kv && qj < L && qj >= key) {
              const float *dr = a.delta + ((st + qj) * Hq + h) * DV;
              const float sgj = a.sig[(st + qj) * Hq + h];
#pragma unroll 1
              for (int d = 0; d < DV; ++d) t += dr[d] * sgj * fast_exp2(glx(qj, d) - glx(key, d)) * vv(key, d);
            }
            dp[j] = t;
          }
        }
      }
      f16x8 dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) dsf[u][i] = (_Float16)(p[8 * u + i] * dp[8 * u + i]);
      // dV[key][dv] += F[key][dv] * sum_q P[q][key] dx[q][dv], with F = exp(Gl_ref - Gl_key)
      // the key side of the split decay (<= 1 off the diagonal block, >= 1 on it)
#pragma unroll
      for (int bv = 0; bv < NBV; ++bv) {
        const int col = 32 * bv + n;
        const bool cv = col < DV;
        const float grc = cv ? glx(ref, col) : 0.f;
        if (!direct) {
          f32x16 tmp = zero16();
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            bf16x8 ph, plo, th, tl;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              split_bf16(p[8 * u + i], ph, plo, i);
              const int qk = q0 + slab_key(u, hh, i);
              float val = 0.f;
              if (cv && qk < L)
                val = fast_exp2(glx(qk, col) - grc) * a.delta[((st + qk) * Hq + h) * DV + col] *
                      a.sig[(st + qk) * Hq + h];
              split_bf16(val, th, tl, i);
            }
            tmp = mma32(ph, th, tmp);
            tmp = mma32(ph, tl, tmp);
            tmp = mma32(plo, th, tmp);
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kj = kb + acc_row(hh, j);
            const float f = (cv && kj < L) ? fast_exp2(grc - glx(kj, col)) : 0.f;
            accV[bv][j] += f * tmp[j];
          }
        } else {
          // exact per-pair decays: P[q][kj] lives in lane kj, register of q
#pragma unroll
          for (int qq = 0; qq < 32; ++qq) {
            const int jsrc = (qq >> 3) * 4 + (qq & 3), hsrc = (qq >> 2) & 1;
            const int qk = q0 + qq;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int kl = acc_row(hh, j);
              const float pv = __shfl(p[jsrc], kl + 32 * hsrc);
              const int kj = kb + kl;
              if (cv && qk < L && kj <= qk)
                accV[bv][j] += pv * fast_exp2(glx(qk, col) - glx(kj, col)) *
                               a.delta[((st + qk) * Hq + h) * DV + col] * a.sig[(st + qk) * Hq + h];
            }
          }
        }
      }
      // dK[key][dk] += dS[q][key] Q[q][dk]
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk) {
        const int col = 32 * bk + n;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f16x8 qt;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int qk = q0 + slab_key(u, hh, i);
            qt[i] = (_Float16)((col < DK && qk < L) ? load_in(a.q, ((st + qk) * Hq + h) * DK + col, F32IN) : 0.f);
          }
          accK[bk] = mma32(dsf[u], qt, accK[bk]);
        }
      }
    }
  }
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
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int col = 32 * bv + n;
    if (col >= DV) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) a.dv_i[((st + kj) * Hkv + c) * DV + col] = accV[bv][j];
    }
  }
}

// ---------------------------------------------------------------------------
// dq from key chunks before the query chunk.  Workgroup = 128 query rows of
// one q head (4 waves x 32 rows); steps of 32 keys staged through LDS
// (double buffered): K rows (bf16) for S^T, transposed K (fp16) for dS.K,
// and V scaled to the query chunk start (fp16) for dP^T.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 2) k_bwd_dq(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, NBK = DKP / 32;
  constexpr int KSTR = DK + 8, TSTR = 32 + 8, VSTR = DV + 8;
  constexpr int KP = 32 * DK / 8, TP = DK * 32 / 8, VP = 32 * DV / 8;  // 16-byte pieces per step
  constexpr int KPT = (KP + 255) / 256, TPT = (TP + 255) / 256, VPT = (VP + 255) / 256;
  __shared__ __align__(16) uint16_t Ks[2][32 * KSTR];
  __shared__ __align__(16) _Float16 Kts[2][DKP * TSTR];
  __shared__ __align__(16) _Float16 Vs[2][32 * VSTR];

  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  int bid = blockIdx.x;
  const int c = bid % Hkv;
  bid /= Hkv;
  const int gq = bid % G;
  const int item = bid / G;
  if (item >= pl.counts[0]) return;
  const int hq = c * G + gq;
  const int2 it = pl.qitems[item];
  const int s = it.x, I = it.y;
  const int64_t st = pl.seq_start[s];
  const int L = pl.seq_len[s];
  const int cbs = pl.cb128[s];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int r0 = I * CB + 32 * wave;
  const int row = r0 + n;
  const bool rv = row < L;
  const float sl2 = a.sl2;

  kfrag qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = rv ? IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();
  const float mbn = rv ? a.mb[(st + row) * Hq + hq] : INFINITY;
  f16x8 dhf[NSV];
#pragma unroll
  for (int i = 0; i < NSV; ++i)
    dhf[i] = rv ? *(const f16x8 *)(a.dh + ((st + row) * Hq + hq) * DV + 16 * i + 8 * hh)
                : __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  if (DK < DKP) {
    for (int e = tid; e < (DKP - DK) * TSTR; e += 256) {
      Kts[0][DK * TSTR + e] = (_Float16)0.f;
      Kts[1][DK * TSTR + e] = (_Float16)0.f;
    }
  }
  f32x16 acc[NBK];
#pragma unroll
  for (int b = 0; b < NBK; ++b) acc[b] = zero16();

  // staging state: this thread's V pieces always cover channels 8*d8 .. +7
  const int d8 = tid % (DV / 8);
  float gam[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gam[e] = 1.f;
  uint4 kreg[KPT], treg[TPT], vreg[VPT];
  const int nsteps = 4 * I;
  auto load_tile = [&](int k) {
    const int J = I - 1 - (k >> 2), u = k & 3;
    if (k > 0 && (k & 3) == 0) {  // entered chunk J: gamma_IJ = gamma_I,J+1 * Gam_J+1
      const float *gp = a.Gam + ((int64_t)(cbs + J + 1) * Hkv + c) * DV + 8 * d8;
#pragma unroll
      for (int e = 0; e < 8; ++e) gam[e] *= gp[e];
    }
    const int kt0 = J * CB + 32 * u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = tid + 256 * i;
      if (p < KP) {
        const int kr = p / (DK / 8), e8 = p % (DK / 8);
        kreg[i] = __builtin_bit_cast(uint4, IF::load(a.k, ((st + kt0 + kr) * Hkv + c) * DK + 8 * e8));
      }
    }
    const _Float16 *ktile = a.Kt + ((int64_t)(cbs + J) * Hkv + c) * DK * CB + 32 * u;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int p = tid + 256 * i;
      if (p < TP) {
        const int dr = p >> 2, q8 = p & 3;
        treg[i] = *(const uint4 *)(ktile + dr * CB + 8 * q8);
      }
    }
    const _Float16 *vtile = a.Vr + ((int64_t)(cbs + J) * Hkv + c) * CB * DV + (32 * u) * DV;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int p = tid + 256 * i;
      if (p < VP) {
        const int vr = p / (DV / 8);
        f16x8 x = *(const f16x8 *)(vtile + vr * DV + 8 * d8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (_Float16)((float)x[e] * gam[e]);
        vreg[i] = __builtin_bit_cast(uint4, x);
      }
    }
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int p = tid + 256 * i;
      if (p < KP) {
        const int kr = p / (DK / 8), e8 = p % (DK / 8);
        *(uint4 *)&Ks[b][kr * KSTR + 8 * e8] = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int p = tid + 256 * i;
      if (p < TP) *(uint4 *)&Kts[b][(p >> 2) * TSTR + 8 * (p & 3)] = treg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int p = tid + 256 * i;
      if (p < VP) *(uint4 *)&Vs[b][(p / (DV / 8)) * VSTR + 8 * d8] = vreg[i];
    }
  };

  if (nsteps > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int k = 0; k < nsteps; ++k) {
    const int b = k & 1;
    if (k + 1 < nsteps) load_tile(k + 1);
    {
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const kfrag *)&Ks[b][n * KSTR + 16 * i + 8 * hh], qf[i], sc);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)&Vs[b][n * VSTR + 16 * i + 8 * hh], dhf[i], dp);
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
          acc[bk] = mma32(dsf[u], *(const f16x8 *)&Kts[b][(32 * bk + n) * TSTR + 16 * u + 8 * hh], acc[bk]);
    }
    if (k + 1 < nsteps) store_tile(b ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = r0 + acc_row(hh, j);
      if (r < L) {
        const int64_t idx = ((st + r) * Hq + hq) * DK + col;
        store_out(a.dq, idx, a.scale * acc[bk][j] + a.dq_i[idx], a.out_f32);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk, dv from query chunks after the key chunk.  Workgroup = 128 keys of one
// kv head (4 waves x 32 keys); steps of 32 queries of one head of the group
// staged through LDS (double buffered): Q rows (bf16) for S, transposed Q
// (fp16) for dK, the scaled dhat (fp16, times gamma) as rows for dP and
// transposed for dV, and the per-row exponent offsets.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 2) k_bwd_dkv(BwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int NS = DK / 16, NSV = DV / 16, DKP = Pad32<DK>::value, DVP = Pad32<DV>::value;
  constexpr int NBK = DKP / 32, NBV = DVP / 32;
  constexpr int QSTR = DK + 8, TSTR = 32 + 8, DSTR = DV + 8;
  constexpr int QP = 32 * DK / 8, QTP = DK * 4, DP_ = 32 * DV / 8, DTP = DV * 4;
  constexpr int QPT = (QP + 255) / 256, QTPT = (QTP + 255) / 256, DPT = (DP_ + 255) / 256, DTPT = (DTP + 255) / 256;
  __shared__ __align__(16) uint16_t Qs[2][32 * QSTR];
  __shared__ __align__(16) _Float16 Qts[2][DKP * TSTR];
  __shared__ __align__(16) _Float16 Ds[2][32 * DSTR];
  __shared__ __align__(16) _Float16 Dts[2][DVP * TSTR];
  __shared__ __align__(16) float Ms[2][32];

  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int c = blockIdx.x % Hkv;
  const int rank = blockIdx.x / Hkv;
  if (rank >= pl.counts[0]) return;
  const int2 it = pl.qitems[pl.counts[0] - 1 - rank];  // earliest chunks (most queries after them) first
  const int s = it.x, J = it.y;
  const int64_t st = pl.seq_start[s];
  const int L = pl.seq_len[s];
  const int cbs = pl.cb128[s];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int kb = J * CB + 32 * wave;
  const int key = kb + n;
  const bool kv = key < L;
  const float sl2 = a.sl2;

  kfrag kf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    kf[i] = kv ? IF::load(a.k, ((st + key) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
  f16x8 vf[NSV];
  const _Float16 *vrow = a.Vr + (((int64_t)(cbs + J) * Hkv + c) * CB + 32 * wave + n) * DV;
#pragma unroll
  for (int i = 0; i < NSV; ++i) vf[i] = *(const f16x8 *)(vrow + 16 * i + 8 * hh);
  if (DK < DKP || DV < DVP) {
    for (int e = tid; e < (DKP - DK) * TSTR; e += 256) {
      Qts[0][DK * TSTR + e] = (_Float16)0.f;
      Qts[1][DK * TSTR + e] = (_Float16)0.f;
    }
    for (int e = tid; e < (DVP - DV) * TSTR; e += 256) {
      Dts[0][DV * TSTR + e] = (_Float16)0.f;
      Dts[1][DV * TSTR + e] = (_Float16)0.f;
    }
  }
  f32x16 accK[NBK], accV[NBV];
#pragma unroll
  for (int b = 0; b < NBK; ++b) accK[b] = zero16();
#pragma unroll
  for (int b = 0; b < NBV; ++b) accV[b] = zero16();

  const int after = L - (J + 2) * CB;                // queries two chunks or more after the key chunk
  const int nsph = after > 0 ? (after + 31) / 32 : 0;  // 32-query steps per head
  const int nsteps = G * nsph;
  // staging state: row pieces cover channels 8*d8 .. +7; transposed pieces
  // cover channel rows (tid >> 2) + 64 i
  const int d8 = tid % (DV / 8);
  float gr[8], gt[DTPT];
  uint4 qreg[QPT], qtreg[QTPT], dreg[DPT], dtreg[DTPT];
  float mreg = INFINITY;
  auto load_tile = [&](int k) {
    const int gq = k / nsph, kk = k % nsph;
    const int h = c * G + gq;
    const int I = J + 2 + (kk >> 2), u = kk & 3;
    if (kk == 0 || (kk & 3) == 0) {  // entered chunk I: gamma_IJ = gamma_I-1,J * Gam_I-1 (gamma_J+1,J = 1)
      if (kk == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gr[e] = 1.f;
#pragma unroll
        for (int i = 0; i < DTPT; ++i) gt[i] = 1.f;
      }
      const float *gp = a.Gam + ((int64_t)(cbs + I - 1) * Hkv + c) * DV;
#pragma unroll
      for (int e = 0; e < 8; ++e) gr[e] *= gp[8 * d8 + e];
#pragma unroll
      for (int i = 0; i < DTPT; ++i) {
        const int dr = (tid >> 2) + 64 * i;
        if (dr < DV) gt[i] *= gp[dr];
      }
    }
    const int qt0 = I * CB + 32 * u;
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int p = tid + 256 * i;
      if (p < QP) {
        const int qr = p / (DK / 8), e8 = p % (DK / 8);
        qreg[i] = (qt0 + qr < L)
                      ? __builtin_bit_cast(uint4, IF::load(a.q, ((st + qt0 + qr) * Hq + h) * DK + 8 * e8))
                      : make_uint4(0, 0, 0, 0);
      }
    }
    const _Float16 *qtile = a.Qt + ((int64_t)(cbs + I) * Hq + h) * DK * CB + 32 * u;
#pragma unroll
    for (int i = 0; i < QTPT; ++i) {
      const int p = tid + 256 * i;
      if (p < QTP) qtreg[i] = *(const uint4 *)(qtile + (p >> 2) * CB + 8 * (p & 3));
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int p = tid + 256 * i;
      if (p < DP_) {
        const int qr = p / (DV / 8);
        f16x8 x = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
        if (qt0 + qr < L) {
          x = *(const f16x8 *)(a.dh + ((st + qt0 + qr) * Hq + h) * DV + 8 * d8);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (_Float16)((float)x[e] * gr[e]);
        }
        dreg[i] = __builtin_bit_cast(uint4, x);
      }
    }
    const _Float16 *dtile = a.dht + ((int64_t)(cbs + I) * Hq + h) * DV * CB + 32 * u;
#pragma unroll
    for (int i = 0; i < DTPT; ++i) {
      const int p = tid + 256 * i;
      if (p < DTP) {
        f16x8 x = *(const f16x8 *)(dtile + (p >> 2) * CB + 8 * (p & 3));
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (_Float16)((float)x[e] * gt[i]);
        dtreg[i] = __builtin_bit_cast(uint4, x);
      }
    }
    if (tid < 32) mreg = (qt0 + tid < L) ? a.mb[(st + qt0 + tid) * Hq + h] : INFINITY;
  };
  auto store_tile = [&](int b) {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int p = tid + 256 * i;
      if (p < QP) *(uint4 *)&Qs[b][(p / (DK / 8)) * QSTR + 8 * (p % (DK / 8))] = qreg[i];
    }
#pragma unroll
    for (int i = 0; i < QTPT; ++i) {
      const int p = tid + 256 * i;
      if (p < QTP) *(uint4 *)&Qts[b][(p >> 2) * TSTR + 8 * (p & 3)] = qtreg[i];
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int p = tid + 256 * i;
      if (p < DP_) *(uint4 *)&Ds[b][(p / (DV / 8)) * DSTR + 8 * d8] = dreg[i];
    }
#pragma unroll
    for (int i = 0; i < DTPT; ++i) {
      const int p = tid + 256 * i;
      if (p < DTP) *(uint4 *)&Dts[b][(p >> 2) * TSTR + 8 * (p & 3)] = dtreg[i];
    }
    if (tid < 32) Ms[b][tid] = mreg;
  };

  if (nsteps > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int k = 0; k < nsteps; ++k) {
    const int b = k & 1;
    if (k + 1 < nsteps) load_tile(k + 1);
    {
      // S[q][key] and dP[q][key]: lane = key, register j = query acc_row(hh, j)
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc = mma32(*(const kfrag *)&Qs[b][n * QSTR + 16 * i + 8 * hh], kf[i], sc);
#pragma unroll
      for (int i = 0; i < NSV; ++i) dp = mma32(*(const f16x8 *)&Ds[b][n * DSTR + 16 * i + 8 * hh], vf[i], dp);
      f16x8 pf[2], dsf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 mq = *(const float4 *)&Ms[b][8 * q4 + 4 * hh];
        const float mv[4] = {mq.x, mq.y, mq.z, mq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * q4 + e;
          const float pv = fast_exp2(sc[j] * sl2 - mv[e]);
          pf[j >> 3][j & 7] = (_Float16)pv;
          dsf[j >> 3][j & 7] = (_Float16)(pv * dp[j]);
        }
      }
#pragma unroll
      for (int bv = 0; bv < NBV; ++bv)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          accV[bv] = mma32(pf[u], *(const f16x8 *)&Dts[b][(32 * bv + n) * TSTR + 16 * u + 8 * hh], accV[bv]);
#pragma unroll
      for (int bk = 0; bk < NBK; ++bk)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          accK[bk] = mma32(dsf[u], *(const f16x8 *)&Qts[b][(32 * bk + n) * TSTR + 16 * u + 8 * hh], accK[bk]);
    }
    if (k + 1 < nsteps) store_tile(b ^ 1);
    __syncthreads();
  }
  if (kb >= L) return;
  // epilogue: dk, dv (inter part scaled to the key: exp(Gl_end(J) - Gl_key)), dG = qside - v (.) dv
  const int tend = min((J + 1) * CB, L) - 1;
#pragma unroll
  for (int bk = 0; bk < NBK; ++bk) {
    const int col = 32 * bk + n;
    if (col >= DK) continue;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) {
        const int64_t idx = ((st + kj) * Hkv + c) * DK + col;
        store_out(a.dk, idx, a.scale * accK[bk][j] + a.dk_i[idx], a.out_f32);
      }
    }
  }
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int col = 32 * bv + n;
    if (col >= DV) continue;
    const float gend = a.Gl2[((st + tend) * Hkv + c) * DV + col];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kj = kb + acc_row(hh, j);
      if (kj < L) {
        const int64_t idx = ((st + kj) * Hkv + c) * DV + col;
        const float dvv = fast_exp2(gend - a.Gl2[idx]) * accV[bv][j] + a.dv_i[idx];
        store_out(a.dv, idx, dvv, a.out_f32);
        a.dG[idx] = a.qside[idx] - load_in(a.v, idx, F32IN) * dvv;
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
