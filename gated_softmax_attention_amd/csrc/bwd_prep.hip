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
// side of dG).
#include "common.h"
#include "launch.h"

namespace fix {

// Gl2 (log2 units, 128-chunk local), Gam per 128-chunk, row-major fp16 V
// scaled to its chunk end, Vr[chunk][kvh][t][d] = exp(Gl_end - Gl_t) v_t, and
// V scaled to the end of its 32-token block, VE[t][kvh][d] (the block end
// clamped to the sequence end).
template <int DV>
__global__ void __launch_bounds__(128) k_gate_prep_rows(const float *__restrict__ g, const void *__restrict__ v,
                                                        bool in_f32, Plan plan, int Hkv, float *__restrict__ Gl2,
                                                        float *__restrict__ Gam, _Float16 *__restrict__ Vr,
                                                        _Float16 *__restrict__ VE) {
  const int gc = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (gc >= plan.counts[0] || d >= DV) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  float acc = 0.f;
  for (int j = 0; j < n; ++j) {
    int64_t idx = ((tok0 + j) * Hkv + c) * DV + d;
    acc += g[idx] * LOG2E;
    Gl2[idx] = acc;
  }
  const int64_t cidx = ((int64_t)gc * Hkv + c);
  Gam[cidx * DV + d] = fast_exp2(acc);
  _Float16 *dst = Vr + cidx * CB * DV + d;
  for (int j = 0; j < CB; ++j) {
    float val = 0.f;
    if (j < n) {
      int64_t idx = ((tok0 + j) * Hkv + c) * DV + d;
      const float gj = Gl2[idx], vj = load_in(v, idx, in_f32);
      val = fast_exp2(acc - gj) * vj;
      const float gbe = Gl2[((tok0 + min((j | 31), n - 1)) * Hkv + c) * DV + d];
      VE[idx] = (_Float16)(fast_exp2(gbe - gj) * vj);
    }
    dst[(int64_t)j * DV] = (_Float16)val;
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
template <int D>
__global__ void __launch_bounds__(256) k_tiles_t(const void *__restrict__ in, bool in_f32, Plan plan, int H,
                                                 _Float16 *__restrict__ out) {
  constexpr int STR = CB + 8;
  __shared__ _Float16 tile[D * STR];
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
    if (in_f32) {
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
    for (int i = 0; i < 8; ++i) tile[(d8 + i) * STR + key_pos(t)] = (_Float16)(t < n ? val[i] : 0.f);
  }
  __syncthreads();
  uint4 *dst = (uint4 *)(out + ((int64_t)gc * H + h) * D * CB);
  for (int e = tid; e < D * CB / 8; e += 256) {
    int d = e / (CB / 8), p8 = e % (CB / 8);
    dst[e] = *(const uint4 *)&tile[d * STR + 8 * p8];
  }
}

template <int DV>
__global__ void __launch_bounds__(256) k_bwd_prep(PrepArgs a) {
  constexpr int STR = CB + 8;
  constexpr int PER = (DV + 63) / 64;  // channels per lane
  __shared__ _Float16 tile[DV * STR];
  __shared__ __bf16 tileh[DV * STR], tilel[DV * STR];
  const int gc = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (gc >= a.plan.counts[0]) return;
  const Plan &pl = a.plan;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int t0 = (gc - pl.cb128[s]) * CB;
  const int n = min(CB, pl.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)pl.seq_start[s] + t0;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const bool in_f32 = a.in_f32;

  float wv[PER], dwacc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    int d = lane + 64 * k;
    wv[k] = (a.o_norm && a.w && d < DV) ? load_in(a.w, d, in_f32) : 1.f;
    dwacc[k] = 0.f;
  }
  for (int gq = 0; gq < G; ++gq) {
    const int h = c * G + gq;
    // U tokens per wave at a time: every input of the U rows is loaded
    // before any output is stored (the compiler cannot tell the buffers
    // apart, so interleaving would make each row wait for the previous
    // row's stores).
    constexpr int U = 4;
#pragma unroll 1
    for (int i0 = 0; i0 < CB / 4; i0 += U) {
      float r[U], mrow[U], xv[U][PER], go[U][PER], zz[U][PER], gl[U][PER], gbs[U][PER], qo[U][PER];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = min(wave + 4 * (i0 + u), n - 1);  // rows past the end repeat the last (not stored)
        const int64_t tok = tok0 + t;
        const int64_t rb = (tok * Hq + h) * DV;
        r[u] = a.rstd[tok * Hq + h];
        mrow[u] = a.m[tok * Hq + h];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int d = min(lane + 64 * k, DV - 1);
          const int64_t gi = (tok * Hkv + c) * DV + d;
          xv[u][k] = a.x[rb + d];
          go[u][k] = load_in(a.dO, rb + d, in_f32);
          zz[u][k] = a.z ? load_in(a.z, rb + d, in_f32) : 1.f;
          gl[u][k] = a.Gl2[gi];
          gbs[u][k] = (t & ~31) ? a.Gl2[((tok0 + (t & ~31) - 1) * Hkv + c) * DV + d] : 0.f;
          qo[u][k] = gq == 0 ? 0.f : a.qside[gi];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = wave + 4 * (i0 + u);  // token within the chunk
        if (t < n) {
          const int64_t tok = tok0 + t;
          const int64_t rb = (tok * Hq + h) * DV;
          float dn[PER], del[PER];
          float proj = 0.f;
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int d = lane + 64 * k;
            dn[k] = 0.f;
            if (d < DV) {
              dn[k] = go[u][k] * zz[u][k];
              const float nval = a.o_norm ? xv[u][k] * r[u] * wv[k] : xv[u][k];
              if (a.dz) store_out(a.dz, rb + d, go[u][k] * nval, a.out_f32);
              if (a.o_norm) {
                dwacc[k] += dn[k] * xv[u][k] * r[u];
                proj += dn[k] * wv[k] * xv[u][k] * r[u];
              }
            }
          }
          if (a.o_norm) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) proj += __shfl_xor(proj, off);
            proj *= 1.f / DV;
          }
          // sigma = 2^-e scales the row so that max |sigma delta| is about 1; every
          // fp16 operand built from the row (here exp(Gl) sigma delta, within a
          // block exp(Gl_i - Gl_ref) sigma delta, all factors <= 1) stays in range
          float amax = 0.f;
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            del[k] = a.o_norm ? r[u] * (dn[k] * wv[k] - xv[u][k] * r[u] * proj) : dn[k];
            if (lane + 64 * k < DV) amax = fmaxf(amax, fabsf(del[k]));
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
          int e = 0;
          if (amax > 0.f) e = min(15, max(-15, (int)ceilf(__log2f(amax))));
          const float sg = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int d = lane + 64 * k;
            if (d < DV) {
              a.delta[rb + d] = del[k];
              // query side of dG, summed over the group; (token, channel) is
              // owned by this thread for every head of the group
              a.qside[(tok * Hkv + c) * DV + d] = qo[u][k] + del[k] * xv[u][k];
              const _Float16 hv = (_Float16)(fast_exp2(gl[u][k]) * del[k] * sg);
              a.dh[rb + d] = hv;
              tile[d * STR + key_pos(t)] = hv;
              // relative to the token before the row's 32-token block (<= 1)
              const float xb = fast_exp2(gl[u][k] - gbs[u][k]) * del[k] * sg;
              const __bf16 xh = (__bf16)xb, xl = (__bf16)(xb - (float)xh);
              a.X16[rb + d] = (_Float16)xb;
              a.XH[rb + d] = xh;
              a.XL[rb + d] = xl;
              tileh[d * STR + key_pos(t)] = xh;
              tilel[d * STR + key_pos(t)] = xl;
            }
          }
          if (lane == 0) {
            a.mb[tok * Hq + h] = mrow[u] * LOG2E - (float)e;
            a.sig[tok * Hq + h] = sg;
          }
        } else {
#pragma unroll
          for (int k = 0; k < PER; ++k) {
            const int d = lane + 64 * k;
            if (d < DV) {
              tile[d * STR + key_pos(t)] = (_Float16)0.f;
              tileh[d * STR + key_pos(t)] = (__bf16)0.f;
              tilel[d * STR + key_pos(t)] = (__bf16)0.f;
            }
          }
        }
      }
    }
    __syncthreads();
    const int64_t tb = ((int64_t)gc * Hq + h) * DV * CB;
    uint4 *dst = (uint4 *)(a.dht + tb), *dsth = (uint4 *)(a.XTH + tb), *dstl = (uint4 *)(a.XTL + tb);
    for (int e = tid; e < DV * CB / 8; e += 256) {
      int d = e / (CB / 8), p8 = e % (CB / 8);
      dst[e] = *(const uint4 *)&tile[d * STR + 8 * p8];
      dsth[e] = *(const uint4 *)&tileh[d * STR + 8 * p8];
      dstl[e] = *(const uint4 *)&tilel[d * STR + 8 * p8];
    }
    __syncthreads();
  }
  if (a.dw_part) {
    // per-block partials: reduce the four waves in LDS, then one row per block
    __shared__ float red[4][DV];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int d = lane + 64 * k;
      if (d < DV) red[wave][d] = dwacc[k];
    }
    __syncthreads();
    for (int d = tid; d < DV; d += 256)
      a.dw_part[((int64_t)gc * Hkv + c) * DV + d] = red[0][d] + red[1][d] + red[2][d] + red[3][d];
  }
}

// dw[d] = sum over blocks of the partials, in a fixed order.
__global__ void __launch_bounds__(256) k_dw_reduce(const float *__restrict__ part, const int *__restrict__ counts,
                                                   int Hkv, int dv, float *__restrict__ dw) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= dv) return;
  const int nb = counts[0] * Hkv;
  float acc = 0.f;
  for (int b = 0; b < nb; ++b) acc += part[(int64_t)b * dv + d];
  dw[d] = acc;
}

// dg_t = sum over t' >= t of the same sequence of dG_t' (the gate enters
// through G_t = sum_{u<=t} g_u).  Three passes over 128-chunks: chunk
// totals, exclusive suffix carries per sequence, then in-chunk suffix sums.
template <int DV>
__global__ void __launch_bounds__(128) k_dg_totals(const float *__restrict__ dG, Plan plan, int Hkv,
                                                   float *__restrict__ tot) {
  const int gc = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (gc >= plan.counts[0] || d >= DV) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  // fixed trip count, masked, so that the loads are issued together
  float acc = 0.f;
#pragma unroll 32
  for (int j = 0; j < CB; ++j) {
    const float x = dG[((tok0 + min(j, n - 1)) * Hkv + c) * DV + d];
    acc += j < n ? x : 0.f;
  }
  tot[((int64_t)gc * Hkv + c) * DV + d] = acc;
}

template <int DV>
__global__ void __launch_bounds__(128) k_dg_carry(const float *__restrict__ tot, Plan plan, int Hkv,
                                                  float *__restrict__ carry) {
  const int s = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (d >= DV) return;
  float run = 0.f;
  for (int gc = plan.cb128[s + 1] - 1; gc >= plan.cb128[s]; --gc) {
    const int64_t idx = ((int64_t)gc * Hkv + c) * DV + d;
    carry[idx] = run;
    run += tot[idx];
  }
}

template <int DV>
__global__ void __launch_bounds__(128) k_dg_final(const float *__restrict__ dG, const float *__restrict__ carry,
                                                  Plan plan, int Hkv, float *__restrict__ dg) {
  const int gc = blockIdx.x, c = blockIdx.y, d = threadIdx.x;
  if (gc >= plan.counts[0] || d >= DV) return;
  const int s = seq_of_chunk(plan.cb128, plan.nseq, gc);
  const int t0 = (gc - plan.cb128[s]) * CB;
  const int n = min(CB, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  // 32-token blocks from the chunk end down, each block's loads issued together
  float run = carry[((int64_t)gc * Hkv + c) * DV + d];
#pragma unroll 1
  for (int b = CB / 32 - 1; b >= 0; --b) {
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = dG[((tok0 + min(32 * b + j, n - 1)) * Hkv + c) * DV + d];
#pragma unroll
    for (int j = 31; j >= 0; --j) {
      const int t = 32 * b + j;
      if (t < n) {
        run += x[j];
        dg[((tok0 + t) * Hkv + c) * DV + d] = run;
      }
    }
  }
}

#define FIX_DV_SWITCH(dv, ...)                         \
  switch (dv) {                                        \
    case 16: { constexpr int DVC = 16; __VA_ARGS__; } break;   \
    case 32: { constexpr int DVC = 32; __VA_ARGS__; } break;   \
    case 64: { constexpr int DVC = 64; __VA_ARGS__; } break;   \
    case 128: { constexpr int DVC = 128; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;              \
  }

hipError_t launch_gate_prep_rows(int dv, const float *g, const void *v, bool in_f32, const Plan &plan, int Hkv,
                                 int ncb_ub, float *Gl2, float *Gam, _Float16 *Vr, _Float16 *VE, hipStream_t st) {
  dim3 grid(ncb_ub, Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_gate_prep_rows<DVC>, grid, dim3(128), 0, st, g, v, in_f32, plan, Hkv,
                                       Gl2, Gam, Vr, VE));
  return hipGetLastError();
}

hipError_t launch_chunk_logprefix(int dv, const float *Gl2, const Plan &plan, int Hkv, double *Lam, hipStream_t st) {
  dim3 grid(plan.nseq, Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_chunk_logprefix<DVC>, grid, dim3(128), 0, st, Gl2, plan, Hkv, Lam));
  return hipGetLastError();
}

hipError_t launch_tiles_t(int D, const void *in, bool in_f32, const Plan &plan, int H, int ncb_ub, _Float16 *out,
                          hipStream_t st) {
  dim3 grid(ncb_ub, H);
  FIX_DV_SWITCH(D, hipLaunchKernelGGL(k_tiles_t<DVC>, grid, dim3(256), 0, st, in, in_f32, plan, H, out));
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int dv, const PrepArgs &a, int ncb_ub, hipStream_t st) {
  dim3 grid(ncb_ub, a.Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_bwd_prep<DVC>, grid, dim3(256), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_dg_scan(int dv, const float *dG, const Plan &plan, int Hkv, int ncb_ub, float *tot, float *carry,
                          float *dg, hipStream_t st) {
  dim3 grid(ncb_ub, Hkv), gs(plan.nseq, Hkv);
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_dg_totals<DVC>, grid, dim3(128), 0, st, dG, plan, Hkv, tot));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_dg_carry<DVC>, gs, dim3(128), 0, st, tot, plan, Hkv, carry));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  FIX_DV_SWITCH(dv, hipLaunchKernelGGL(k_dg_final<DVC>, grid, dim3(128), 0, st, dG, carry, plan, Hkv, dg));
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const float *part, const int *counts, int Hkv, int dv, float *dw, hipStream_t st) {
  hipLaunchKernelGGL(k_dw_reduce, dim3((dv + 255) / 256), dim3(256), 0, st, part, counts, Hkv, dv, dw);
  return hipGetLastError();
}

}  // namespace fix
