// Backward preprocessing: gate chunks of CB = 128 tokens, operand tiles in
// the layouts the backward MFMA kernels read, and the output-side backward.
//
// The backward of o = RMSNorm(x) (.) w (.) z with respect to x (FiX README,
// "Quick Start": optional o_norm weight and o_gate), with r = rstd and
// xh = x r:
//   dz = dO (.) n  (n = xh (.) w under the norm, x without it),  dn = dO (.) z
//   dw = sum over rows of dn (.) xh
//   delta = r (dn (.) w - xh * mean_d(dn (.) w (.) xh))   (or dn without the norm)
// delta is the gradient reaching x_i = sum_j P_ij D_ij (.) v_j.  For the
// chunk-factored products the query side needs dhat_i = exp(Gl_i) delta_i
// (Gl the 128-chunk-local prefix sum of g, so the factor is <= 1); it is
// stored fp16 after a per-row power-of-two scale sigma_i = 2^-e_i with
// max_d |sigma_i delta_i| about 1, which keeps it, and the within-chunk
// operands exp(Gl_i - Gl_ref) sigma_i delta_i, inside fp16 range.  The kernels compute probabilities as
// exp2(s log2e - (m log2e - e_i)) = P_ij / sigma_i, so every product of a
// probability with a scaled dhat is unchanged.  The gate's own gradient
// needs, per kv head, sum over the group's q heads of delta (.) x (the query
// side of dG).  delta itself is not stored: the rare exact-decay paths of the
// backward recompute it from dO, z, w, x, r and the row's projection
// mean_d(dn (.) w (.) xh), which is stored.
#include "common.h"
#include "launch.h"

namespace fix {

// Two 16-bit values packed into one 32-bit word (element 0 in the low half).
template <class T> __device__ inline uint32_t pack2(const T (&x)[2]) {
  return (uint32_t)__builtin_bit_cast(uint16_t, x[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, x[1]) << 16);
}

// Gl2 (log2 units, 128-chunk local), Gam per 128-chunk, row-major fp16 V
// scaled to its chunk end, Vr[chunk][kvh][t][d] = exp(Gl_end - Gl_t) v_t, V
// scaled to the end of its 32-token block, VE[t][kvh][d] (the block end
// clamped to the sequence end), and V relative to the token before its
// 32-token block, VB = exp(Gl_blockstart-1 - Gl_t) v_t (>= |v_t|, fp32 range)
// as bf16 hi / lo parts, the key operand of the diagonal blocks.
template <int DV, bool LOGITS>
__global__ void __launch_bounds__(4 * DV) k_gate_prep_rows(const float *__restrict__ g, const void *__restrict__ v,
                                                           bool in_f32, Plan plan, int Hkv, float *__restrict__ Gl2,
                                                           float *__restrict__ Gam, _Float16 *__restrict__ Vr,
                                                           _Float16 *__restrict__ VE, __bf16 *__restrict__ VBH,
                                                           __bf16 *__restrict__ VBL) {
  // Thread (blk, d): channels d, d + 1 of the chunk's 16-token piece blk (two
  // channels per thread: every load and store moves 8 or 4 bytes per lane).
  // Each piece's local prefix sums, then the totals of the pieces before it
  // (through LDS).
  constexpr int NP = CB / 16, TPP = DV / 2;
  __shared__ float tot[NP][DV];
  const int gc = blockIdx.x, c = blockIdx.y, d = 2 * (threadIdx.x % TPP), blk = threadIdx.x / TPP;
  if (gc >= plan.counts[0]) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  const int j0 = 16 * blk;
  // every load of the piece first (rows past the end repeat the last row, unused)
  float gl[16][2], vv[16][2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t idx = ((tok0 + min(j0 + j, n - 1)) * Hkv + c) * DV + d;
    const float2 g2 = *(const float2 *)(g + idx);
    gl[j][0] = g2.x;
    gl[j][1] = g2.y;
    if (in_f32) {
      const float2 v2 = *(const float2 *)((const float *)v + idx);
      vv[j][0] = v2.x;
      vv[j][1] = v2.y;
    } else {
      const uint32_t w = *(const uint32_t *)((const uint16_t *)v + idx);
      vv[j][0] = __uint_as_float(w << 16);
      vv[j][1] = __uint_as_float(w & 0xffff0000u);
    }
  }
  if constexpr (LOGITS)
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e) gl[j][e] = log_sigmoid(gl[j][e]);
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (j0 + j < n) acc[e] += gl[j][e] * LOG2E;
      gl[j][e] = acc[e];  // past the end the prefix stops growing
    }
  tot[blk][d] = acc[0];
  tot[blk][d + 1] = acc[1];
  __syncthreads();
  // totals of the pieces before this one, and of the pieces of this one's
  // 32-token block (for the block end) and of the whole chunk
  float before[2], all[2], gbe[2], gbs[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float bf = 0.f, al = 0.f, be = 0.f, bs = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const float tq = tot[q][d + e];
      bf += q < blk ? tq : 0.f;
      be += q <= (blk | 1) ? tq : 0.f;
      bs += q < (blk & ~1) ? tq : 0.f;
      al += tq;
    }
    before[e] = bf;
    all[e] = al;
    gbe[e] = be - bf;  // 32-token block end (clamped to the sequence end), piece-local
    gbs[e] = bs - bf;  // the token before the 32-token block, piece-local
  }
  const int64_t cidx = ((int64_t)gc * Hkv + c);
  if (blk == 0) *(float2 *)(Gam + cidx * DV + d) = make_float2(fast_exp2(all[0]), fast_exp2(all[1]));
  _Float16 *dst = Vr + cidx * CB * DV + d;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int t = j0 + j;
    _Float16 vr[2] = {(_Float16)0.f, (_Float16)0.f};
    if (t < n) {
      const int64_t idx = ((tok0 + t) * Hkv + c) * DV + d;
      float gv[2];
      _Float16 ve[2];
      __bf16 bh[2], bl[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        gv[e] = before[e] + gl[j][e];
        vr[e] = (_Float16)(fast_exp2(all[e] - before[e] - gl[j][e]) * vv[j][e]);
        ve[e] = (_Float16)(fast_exp2(gbe[e] - gl[j][e]) * vv[j][e]);
        const float vb = fast_exp2(gbs[e] - gl[j][e]) * vv[j][e];
        bh[e] = (__bf16)vb;
        bl[e] = (__bf16)(vb - (float)bh[e]);
      }
      *(float2 *)(Gl2 + idx) = make_float2(gv[0], gv[1]);
      *(uint32_t *)(VE + idx) = pack2(ve);
      *(uint32_t *)(VBH + idx) = pack2(bh);
      *(uint32_t *)(VBL + idx) = pack2(bl);
    }
    *(uint32_t *)(dst + (int64_t)t * DV) = pack2(vr);
  }
}

// Lam[chunk][kvh][d] = sum over the sequence's chunks n <= chunk of the chunk
// total of the log2 gate (fp64, so that differences of far-apart prefixes keep
// their precision): the decay product of the chunks strictly between J and I
// is exp2(Lam[I-1] - Lam[J]).
template <int DV>
__global__ void __launch_bounds__(128) k_chunk_logprefix(const float *__restrict__ Gl2, Plan plan, int Hkv,
                                                         double *__restrict__ Lam) {
  const int s = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (d >= DV) return;
  const int L = plan.seq_len[s];
  const int64_t st = plan.seq_start[s];
  double run = 0.0;
  for (int gc = plan.cb128[s]; gc < plan.cb128[s + 1]; ++gc) {
    const int tend = min((gc - plan.cb128[s] + 1) * CB, L) - 1;
    run += (double)Gl2[((st + tend) * Hkv + c) * DV + d];
    Lam[((int64_t)gc * Hkv + c) * DV + d] = run;
  }
}

// Transposed fp16 tiles of a [Ttot, H, D] input: out[chunk][h][d][key_pos(t)]
// for the CB tokens of each 128-chunk (zero past the end of the sequence).
// in_kind: 0 bf16, 1 fp32, 2 fp16.
template <int D>
__global__ void __launch_bounds__(256) k_tiles_t(const void *__restrict__ in, int in_kind, Plan plan, int H,
                                                 _Float16 *__restrict__ out) {
  // LDS tile [d][CB] with the 16-byte chunk index of row d XORed with
  // (d / 8) % 16: the eight channels one thread stores (rows d8 .. d8 + 7,
  // one column) and the rows of the threads beside it (d8 + 8, ...) land in
  // different banks, and the copy-out still reads whole 16-byte chunks.
  __shared__ __align__(16) _Float16 tile[D * CB];
  auto at = [](int d, int col) { return d * CB + ((((col >> 3) ^ (d >> 3)) & 15) << 3) + (col & 7); };
  const int gc = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (gc >= plan.counts[0]) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  // 8 consecutive channels of one token per thread and pass (16-byte loads for bf16)
  for (int e = tid; e < CB * D / 8; e += 256) {
    const int t = e / (D / 8), d8 = 8 * (e % (D / 8));
    const int64_t base = ((tok0 + min(t, n - 1)) * H + h) * D + d8;
    float val[8];
    if (in_kind == 2) {
      const f16x8 r = *(const f16x8 *)((const _Float16 *)in + base);
#pragma unroll
      for (int i = 0; i < 8; ++i) val[i] = (float)r[i];
    } else if (in_kind == 1) {
      const float4 lo = *(const float4 *)((const float *)in + base), hi = *(const float4 *)((const float *)in + base + 4);
      val[0] = lo.x; val[1] = lo.y; val[2] = lo.z; val[3] = lo.w; val[4] = hi.x; val[5] = hi.y; val[6] = hi.z; val[7] = hi.w;
    } else {
      const uint4 r = *(const uint4 *)((const uint16_t *)in + base);
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        val[2 * i] = __uint_as_float(w[i] << 16);
        val[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[at(d8 + i, key_pos(t))] = (_Float16)(t < n ? val[i] : 0.f);
  }
  __syncthreads();
  uint4 *dst = (uint4 *)(out + ((int64_t)gc * H + h) * D * CB);
  for (int e = tid; e < D * CB / 8; e += 256) {
    int d = e / (CB / 8), p8 = e % (CB / 8);
    dst[e] = *(const uint4 *)&tile[at(d, 8 * p8)];
  }
}

// Eight consecutive elements of a row, as fp32.
__device__ inline void load8(const void *p, int64_t idx, bool is_f32, float (&v)[8]) {
  if (is_f32) {
    const float4 lo = *(const float4 *)((const float *)p + idx), hi = *(const float4 *)((const float *)p + idx + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
    const uint4 r = *(const uint4 *)((const uint16_t *)p + idx);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}
__device__ inline void load8f(const float *p, int64_t idx, float (&v)[8]) { load8(p, idx, true, v); }
__device__ inline void store8f(float *p, int64_t idx, const float (&v)[8]) {
  *(float4 *)(p + idx) = make_float4(v[0], v[1], v[2], v[3]);
  *(float4 *)(p + idx + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ inline void store8(void *p, int64_t idx, const float (&v)[8], bool is_f32) {
  if (is_f32) {
    store8f((float *)p, idx, v);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
    *(uint4 *)((uint16_t *)p + idx) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
template <class T> __device__ inline void store8h(T *p, int64_t idx, const T (&v)[8]) {
  uint16_t u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = __builtin_bit_cast(uint16_t, v[i]);
  *(uint4 *)((uint16_t *)p + idx) = make_uint4(u[0] | (u[1] << 16), u[2] | (u[3] << 16), u[4] | (u[5] << 16), u[6] | (u[7] << 16));
}

// One workgroup per 128-token chunk and kv head, each query head of the group
// in turn.  A thread owns eight consecutive channels of a token row (16-byte
// loads and stores; DV / 8 threads per row, row reductions by lane shuffles
// inside that group).  Rows are taken 32 tokens at a time; all of a thread's
// rows of such a segment are loaded before the first of them is computed.
template <int DV>
__global__ void __launch_bounds__(256) k_bwd_prep(PrepArgs a) {
  constexpr int TPR = DV / 8;        // threads per token row
  constexpr int RPP = 256 / TPR;     // rows per pass of the workgroup
  constexpr int SEG = 32;            // tokens per segment
  constexpr int NR = SEG / RPP > 0 ? SEG / RPP : 1;  // rows of a segment per thread
  __shared__ __align__(16) char smem[RPP * DV * 4];
  const int gc = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  if (gc >= a.plan.counts[0]) return;
  const Plan &pl = a.plan;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int t0 = (gc - pl.cb128[s]) * CB;
  const int n = min(CB, pl.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)pl.seq_start[s] + t0;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const bool in_f32 = a.in_f32, o_norm = a.o_norm;
  const int sub = tid % TPR, d0 = 8 * sub, rr = tid / TPR;  // channels d0 .. d0 + 7 of row rr (+ RPP k)

  float wv[8], dwacc[8];
  if (o_norm && a.w) load8(a.w, d0, in_f32, wv);
  else
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) dwacc[i] = 0.f;

  for (int gq = 0; gq < G; ++gq) {
    const int h = c * G + gq;
    for (int hf = 0; hf < CB / SEG; ++hf) {
      if (rr < SEG) {
        // every input of the thread's rows first, then each row's arithmetic and
        // outputs (the compiler cannot tell the buffers apart, so a load placed
        // after a store would wait for it)
        float xv[NR][8], go[NR][8], zz[NR][8], gl[NR][8], gbs[NR][8], qo[NR][8], rs[NR], mrow[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int tc = min(SEG * hf + rr + k * RPP, n - 1);  // rows past the end repeat the last (nothing stored)
          const int64_t tok = tok0 + tc;
          const int64_t rb = (tok * Hq + h) * DV + d0, gi = (tok * Hkv + c) * DV + d0;
          load8f(a.x, rb, xv[k]);
          load8(a.dO, rb, in_f32, go[k]);
          if (a.z) load8(a.z, rb, in_f32, zz[k]);
          else
#pragma unroll
            for (int i = 0; i < 8; ++i) zz[k][i] = 1.f;
          load8f(a.Gl2, gi, gl[k]);
          if (tc & ~31) load8f(a.Gl2, ((tok0 + (tc & ~31) - 1) * Hkv + c) * DV + d0, gbs[k]);
          else
#pragma unroll
            for (int i = 0; i < 8; ++i) gbs[k][i] = 0.f;
          if (gq > 0) load8f(a.qside, gi, qo[k]);
          else
#pragma unroll
            for (int i = 0; i < 8; ++i) qo[k][i] = 0.f;
          rs[k] = a.rstd[tok * Hq + h];
          mrow[k] = a.m[tok * Hq + h];
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int r = rr + k * RPP, t = SEG * hf + r;  // token within the chunk
          const int64_t tok = tok0 + min(t, n - 1);
          const int64_t rb = (tok * Hq + h) * DV + d0, gi = (tok * Hkv + c) * DV + d0;
          float dn[8], nval[8], proj = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            dn[i] = go[k][i] * zz[k][i];
            nval[i] = o_norm ? xv[k][i] * rs[k] * wv[i] : xv[k][i];
            proj += dn[i] * wv[i] * xv[k][i] * rs[k];
          }
          if (o_norm) {
#pragma unroll
            for (int off = TPR / 2; off > 0; off >>= 1) proj += __shfl_xor(proj, off);
            proj *= 1.f / DV;
          }
          // sigma = 2^-e scales the row so that max |sigma delta| is about 1; every
          // fp16 operand built from the row (exp(Gl) sigma delta, within a block
          // exp(Gl_i - Gl_ref) sigma delta, all factors <= 1) stays in range
          float del[8], amax = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            del[i] = o_norm ? rs[k] * (dn[i] * wv[i] - xv[k][i] * rs[k] * proj) : dn[i];
            amax = fmaxf(amax, fabsf(del[i]));
          }
#pragma unroll
          for (int off = TPR / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
          int e = 0;
          if (amax > 0.f) e = min(15, max(-15, (int)ceilf(__log2f(amax))));
          const float sg = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
          _Float16 hv[8], x16[8];
          __bf16 xh[8], xl[8];
          float qs[8], dzv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            // query side of dG, summed over the group ((token, channel) is owned by
            // this thread for every head of the group)
            qs[i] = qo[k][i] + del[i] * xv[k][i];
            dzv[i] = go[k][i] * nval[i];
            hv[i] = (_Float16)(fast_exp2(gl[k][i]) * del[i] * sg);
            // relative to the token before the row's 32-token block (<= 1)
            const float xb = fast_exp2(gl[k][i] - gbs[k][i]) * del[i] * sg;
            x16[i] = (_Float16)xb;
            xh[i] = (__bf16)xb;
            xl[i] = (__bf16)(xb - (float)xh[i]);
          }
          if (t < n) {
            if (o_norm)
#pragma unroll
              for (int i = 0; i < 8; ++i) dwacc[i] += dn[i] * xv[k][i] * rs[k];
            if (a.dz) store8(a.dz, rb, dzv, a.out_f32);
            store8f(a.qside, gi, qs);
            store8h(a.dh, rb, hv);
            store8h(a.X16, rb, x16);
            store8h(a.XH, rb, xh);
            store8h(a.XL, rb, xl);
            if (sub == 0) {
              a.mb[tok * Hq + h] = mrow[k] * LOG2E - (float)e;
              a.sig[tok * Hq + h] = sg;
              if (o_norm) a.prj[tok * Hq + h] = proj;
            }
          }
        }
      }
    }
  }
  if (a.dw_part) {
    // per-block partials: the rows of the block's threads summed in LDS,
    // then one row per block
    float *red = (float *)smem;  // [RPP][DV]
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rr * DV + d0 + i] = dwacc[i];
    __syncthreads();
    for (int d = tid; d < DV; d += 256) {
      float acc = 0.f;
      for (int q = 0; q < RPP; ++q) acc += red[q * DV + d];
      a.dw_part[((int64_t)gc * Hkv + c) * DV + d] = acc;
    }
  }
}

// dw[d] = sum over blocks of the partials, in a fixed order.  One workgroup of
// 1024 threads: thread t owns channel t % dv of partial rows t / dv, t / dv +
// 1024 / dv, ... (each wave reads whole rows of consecutive channels, eight
// independent sums per thread), then the 1024 / dv groups meet in LDS in
// group order.
__global__ void __launch_bounds__(1024) k_dw_reduce(const float *__restrict__ part, const int *__restrict__ counts,
                                                    int Hkv, int dv, float *__restrict__ dw) {
  __shared__ float red[1024];
  const int t = threadIdx.x, d = t % dv, grp = t / dv, ng = 1024 / dv;
  const int nb = counts[0] * Hkv;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int b = grp;
  for (; b + 7 * ng < nb; b += 8 * ng)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += part[(int64_t)(b + u * ng) * dv + d];
  for (int u = 0; b < nb; b += ng, ++u) acc[u & 7] += part[(int64_t)b * dv + d];
  red[t] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (grp == 0) {
    float s = 0.f;
    for (int q = 0; q < ng; ++q) s += red[q * dv + d];
    dw[d] = s;
  }
}

// dg_t = sum over t' >= t of the same sequence of dG_t' (the gate enters
// through G_t = sum_{u<=t} g_u).  Two passes over 128-chunks: exclusive
// suffix carries per sequence (from the chunk totals, which the dk/dv
// kernel leaves as four 32-key partial sums per chunk, added here in a fixed
// order), then in-chunk suffix sums.
template <int DV>
__global__ void __launch_bounds__(128) k_dg_carry(const float *__restrict__ tot, Plan plan, int Hkv,
                                                  float *__restrict__ carry) {
  const int s = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (d >= DV) return;
  float run = 0.f;
  for (int gc = plan.cb128[s + 1] - 1; gc >= plan.cb128[s]; --gc) {
    const int64_t idx = ((int64_t)gc * Hkv + c) * DV + d;
    const float *t4 = tot + ((int64_t)gc * Hkv + c) * 4 * DV + d;
    carry[idx] = run;
    run += ((t4[0] + t4[DV]) + t4[2 * DV]) + t4[3 * DV];
  }
}

template <int DV, bool LOGITS>
__global__ void __launch_bounds__(128) k_dg_final(const float *__restrict__ dG, const float *__restrict__ carry,
                                                  const float *__restrict__ logits, Plan plan, int Hkv,
                                                  float *__restrict__ dg) {
  const int gc = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (gc >= plan.counts[0] || d >= DV) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  // 32-token blocks from the chunk end down, each block's loads issued together
  // (with logits, times dg/dx = sigmoid(-x) of the token)
  float run = carry[((int64_t)gc * Hkv + c) * DV + d];
#pragma unroll 1
  for (int b = CB / 32 - 1; b >= 0; --b) {
    float x[32], f[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int64_t idx = ((tok0 + min(32 * b + j, n - 1)) * Hkv + c) * DV + d;
      x[j] = dG[idx];
      f[j] = LOGITS ? logits[idx] : 0.f;
    }
#pragma unroll
    for (int j = 31; j >= 0; --j) {
      const int t = 32 * b + j;
      if (t < n) {
        run += x[j];
        dg[((tok0 + t) * Hkv + c) * DV + d] = LOGITS ? run * sigmoid_neg(f[j]) : run;
      }
    }
  }
}

// fp16 copy of a bf16 or fp32 tensor, 8 elements per thread (n a multiple of 8).
__global__ void __launch_bounds__(256) k_to_f16(const void *__restrict__ in, bool in_f32, int64_t n8,
                                                _Float16 *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n8) return;
  float v[8];
  if (in_f32) {
    const float4 lo = ((const float4 *)in)[2 * e], hi = ((const float4 *)in)[2 * e + 1];
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w; v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  } else {
    const uint4 r = ((const uint4 *)in)[e];
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  f16x8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (_Float16)v[i];
  ((f16x8 *)out)[e] = h;
}

// Largest |x| over n elements (bf16 or fp32), as the bit pattern of a
// non-negative float (whose integer order is the float order; a NaN sorts
// above +inf), folded into *out with an atomic max.
__global__ void __launch_bounds__(256) k_absmax(const void *__restrict__ in, bool in_f32, int64_t n,
                                                unsigned *__restrict__ out) {
  unsigned mx = 0;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const float v = in_f32 ? ((const float *)in)[e] : __uint_as_float((uint32_t)((const uint16_t *)in)[e] << 16);
    mx = max(mx, __float_as_uint(fabsf(v)));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (unsigned)__shfl_xor((int)mx, o));
  if ((threadIdx.x & 63) == 0 && mx) atomicMax(out, mx);
}

hipError_t launch_absmax(const void *in, bool in_f32, int64_t n, unsigned *out, hipStream_t st) {
  const int64_t blocks = min((int64_t)2048, (n + 255) / 256);
  if (blocks > 0) hipLaunchKernelGGL(k_absmax, dim3((unsigned)blocks), dim3(256), 0, st, in, in_f32, n, out);
  return hipGetLastError();
}

hipError_t launch_to_f16(const void *in, bool in_f32, int64_t n, _Float16 *out, hipStream_t st) {
  const int64_t n8 = n / 8;
  if (n8 > 0) hipLaunchKernelGGL(k_to_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, in, in_f32, n8, out);
  return hipGetLastError();
}

#define FIX_DV_SWITCH(dv, ...)                         \
  switch (dv) {                                        \
    case 16: { constexpr int DVC = 16; __VA_ARGS__; } break;   \
    case 32: { constexpr int DVC = 32; __VA_ARGS__; } break;   \
    case 64: { constexpr int DVC = 64; __VA_ARGS__; } break;   \
    case 128: { constexpr int DVC = 128; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;              \
  }

hipError_t launch_gate_prep_rows(int dv, const float *g, bool logits, const void *v, bool in_f32, const Plan &plan,
                                 int Hkv, int ncb_ub, float *Gl2, float *Gam, _Float16 *Vr, _Float16 *VE, __bf16 *VBH,
                                 __bf16 *VBL, hipStream_t st) {
  dim3 grid(ncb_ub, Hkv);
  if (logits)
    FIX_DV_SWITCH(dv, hipLaunchKernelGGL((k_gate_prep_rows<DVC, true>), grid, dim3(4 * DVC), 0, st, g, v, in_f32,
                                         plan, Hkv, Gl2, Gam, Vr, VE, VBH, VBL))
  else
    FIX_DV_SWITCH(dv, hipLaunchKernelGGL((k_gate_prep_rows<DVC, false>), grid, dim3(4 * DVC), 0, st, g, v, in_f32,
                                         plan, Hkv, Gl2, Gam, Vr, VE, VBH, VBL));
  return hipGetLastError();
}

hipError_t launch_chunk_logprefix(int dv, const float *Gl2, const Plan &plan, int Hkv, double *Lam, hipStream_t st) {
  dim3 grid(plan.nseq, Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_chunk_logprefix<DVC>, grid, dim3(128), 0, st, Gl2, plan, Hkv, Lam));
  return hipGetLastError();
}

hipError_t launch_tiles_t(int D, const void *in, int in_kind, const Plan &plan, int H, int ncb_ub, _Float16 *out,
                          hipStream_t st) {
  dim3 grid(ncb_ub, H);
  FIX_DV_SWITCH(D, hipLaunchKernelGGL(k_tiles_t<DVC>, grid, dim3(256), 0, st, in, in_kind, plan, H, out));
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int dv, const PrepArgs &a, int ncb_ub, hipStream_t st) {
  dim3 grid(ncb_ub, a.Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_bwd_prep<DVC>, grid, dim3(256), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_dg_scan(int dv, const float *dG, const float *logits, const Plan &plan, int Hkv, int ncb_ub,
                          float *tot, float *carry, float *dg, hipStream_t st) {
  dim3 grid(ncb_ub, Hkv), gs(plan.nseq, Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_dg_carry<DVC>, gs, dim3(128), 0, st, tot, plan, Hkv, carry));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (logits)
    FIX_DV_SWITCH(dv, hipLaunchKernelGGL((k_dg_final<DVC, true>), grid, dim3(128), 0, st, dG, carry, logits, plan,
                                         Hkv, dg))
  else
    FIX_DV_SWITCH(dv, hipLaunchKernelGGL((k_dg_final<DVC, false>), grid, dim3(128), 0, st, dG, carry, logits, plan,
                                         Hkv, dg));
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *part, const int *counts, int Hkv, int dv, float *dw, hipStream_t st) {
  if (dv < 1 || dv > 1024 || 1024 % dv) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_dw_reduce, dim3(1), dim3(1024), 0, st, part, counts, Hkv, dv, dw);
  return hipGetLastError();
}

}  // namespace fix
