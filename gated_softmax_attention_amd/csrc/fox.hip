// Scalar-gate fast path: the FiX operation when the forget gate is one value
// per token and kv head (the forgetting-attention case, "Forgetting
// Transformer" page, abstract: a forget gate that down-weights the
// unnormalised attention scores).  With g_t a scalar, the decay
// exp(G_i - G_j) is the same for every channel and enters as a bias on the
// logits:
//   x_i = sum_{j<=i} exp(s_ij - m_i + G_i - G_j) v_j,   m_i = max_{j<=i} s_ij
// so no value vector is scaled: the kernel is a causal attention pass with
// an additive bias, an exact online row max and no softmax denominator,
// followed by the same output transform as the per-channel path.
//
// The gate prefix is kept as an fp64 value at the start of every 64-token
// block of a sequence plus an fp32 prefix local to the block, so that
// G_i - G_j is exact to fp32 rounding of block-sized terms however long the
// sequence is.
#include "common.h"
#include "launch.h"

namespace fix {

// Gate prefix per (sequence, kv head): for 64-token block n of the sequence
// (global index chunk_base[s] + n), ref[n] = log2-prefix of g before the
// block (fp64) and loc[t] = log2-prefix of g from the block start to t,
// inclusive (fp32).  Block = 256 threads, a thread per 64-token block; the
// block totals are scanned through LDS, 256 blocks at a time.
template <bool LOGITS>
__global__ void __launch_bounds__(256) k_fox_prefix(const float *__restrict__ g, Plan plan, int Hkv,
                                                    float *__restrict__ loc, double *__restrict__ ref) {
  const int s = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  if (s >= plan.nseq) return;
  const int64_t st = plan.seq_start[s];
  const int L = plan.seq_len[s], cb = plan.chunk_base[s];
  __shared__ double tot[256];
  double carry = 0.0;
  for (int b0 = 0; b0 * CH < L; b0 += 256) {
    const int blk = b0 + tid, t0 = blk * CH;
    double sum = 0.0;
    float acc = 0.f;
    if (t0 < L) {
      const int n = min(CH, L - t0);
      for (int j = 0; j < n; ++j) {
        float gv = g[(st + t0 + j) * Hkv + c];
        if (LOGITS) gv = log_sigmoid(gv);
        acc += gv * LOG2E;
        loc[(st + t0 + j) * Hkv + c] = acc;
      }
      sum = (double)acc;
    }
    tot[tid] = sum;
    __syncthreads();
    // exclusive prefix of the block totals (simple: thread tid sums those before it)
    double before = carry;
    for (int u = 0; u < tid; ++u) before += tot[u];
    if (t0 < L) ref[(int64_t)(cb + blk) * Hkv + c] = before;
    double all = 0.0;
    for (int u = 0; u < 256; ++u) all += tot[u];
    carry += all;
    __syncthreads();
  }
}

// Forward.  Workgroup = 128 query rows (4 waves x 32) of one q head, keys
// visited in 64-token blocks from the first, K and V tiles staged in LDS
// (double buffered, shared by the waves; V as fp16 rows).  A wave computes
// S^T = K Q^T (lane = query row, registers = keys), so the exact online row
// max is a reduction within a lane; P = exp2(s sl2 - m + bias) (<= 1 for a
// forget gate) is the A operand of P V, whose B operand is read from the V
// rows with the transposing LDS load.
template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 2) k_fox_fwd(FoxArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int DVP = DV < 32 ? 32 : DV;
  constexpr int NB = DVP / 32, NS = DK / 16;
  using KT = LdsTile<CH, DK * 2>;  // K rows of a key block (bf16, or fp16 for fp32 inputs)
  using VT = LdsTile<CH, DV * 2>;  // V rows of a key block (fp16)
  constexpr int O_K = 0, O_V = O_K + 2 * KT::BYTES, O_G = O_V + 2 * VT::BYTES, O_R = O_G + 2 * 256;
  constexpr int O_S = O_R + 2 * 256;  // per wave, the 32 row factors of a rescale
  __shared__ __align__(1024) char smem[O_S + 4 * 32 * 4];
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  auto Gk = [&](int b) { return (float *)(smem + O_G + b * 256); };  // the block's local prefixes
  auto Rf = [&](int b) { return (double *)(smem + O_R + b * 256); };  // [0]: the block's reference

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int nblk = pl.counts[0];
  const int idx = xcd_item(nblk * Hq);
  if (idx < 0) return;
  const int c = uniform(idx / (nblk * G)), rem = uniform(idx % (nblk * G));
  const int bi = rem / G, gq = rem % G;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, bi);
  const int64_t st = uniform((int64_t)pl.seq_start[s]);
  const int L = uniform(pl.seq_len[s]);
  const int cb = uniform(pl.chunk_base[s]);
  const int qb = (L + QB - 1) / QB - 1 - (bi - uniform(pl.cb128[s]));  // longest first within the sequence
  const int hq = c * G + gq;
  const int q0 = qb * QB;
  const int nrows = min(QB, L - q0);
  const int rbase = q0 + 32 * wave;       // the wave's first row
  const int row = rbase + n;              // the lane's query row
  const bool active = 32 * wave < nrows;
  const int nJ = (q0 + nrows + CH - 1) / CH;  // key blocks the workgroup needs
  const float sl2 = a.sl2;

  kfrag qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = (active && row < L) ? IF::load(a.q, ((st + row) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();
  // the row's gate prefix (fp64): block reference + block-local part
  const int rr = min(row, L - 1);
  const double grow = a.ref[(int64_t)(cb + rr / CH) * Hkv + c] + (double)a.loc[(st + rr) * Hkv + c];

  uint32_t ok[KT::NW], ov[VT::NW];
  KT::lane_offsets(Hkv * DK * 2, wave, lane, ok);
  VT::lane_offsets(Hkv * DV * 2, wave, lane, ov);
  // Copies of key block J (untracked: the loop reads the other buffer while
  // they are in flight, ordered by the explicit waits below).
  auto stage = [&](int J, int b) {
    const int64_t kr = (st + J * CH) * Hkv + c;
    const int64_t nrow = (int64_t)(L - J * CH) * Hkv;  // rows past the sequence read as zeros
    if constexpr (!F32IN) {
      const u32x4 sk = rsrc_words((const uint16_t *)a.k + kr * DK, nrow * DK * 2);
#pragma unroll
      for (int t = 0; t < KT::NW; ++t) KT::dma_piece_untracked(Ks(b), sk, ok, t, wave);
    } else {
      for (int p = tid; p < KT::NCH; p += 256) {
        const int r = p / KT::CPR, cc = p % KT::CPR;
        *(f16x8 *)(Ks(b) + KT::off(r, cc)) = IF::load(a.k, ((st + min(J * CH + r, L - 1)) * Hkv + c) * DK + 8 * cc);
      }
    }
    const u32x4 sv = rsrc_words(a.V16 + kr * DV, nrow * DV * 2);
#pragma unroll
    for (int t = 0; t < VT::NW; ++t) VT::dma_piece_untracked(Vs(b), sv, ov, t, wave);
    // the block's local gate prefixes (lane l: token l) and its fp64 reference
    // (lanes 0 and 1), in every wave (the same bytes)
    dma4_untracked(Gk(b), rsrc_words(a.loc + kr, nrow * 4), (uint32_t)lane * Hkv * 4);
    dma4_untracked(Rf(b), rsrc_words(a.ref + (int64_t)(cb + J) * Hkv + c, 8), (uint32_t)lane * 4);
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = zero16();
  float m = -INFINITY;  // exact running row max of the lane's row (log2 units)

  if (nJ > 0) stage(0, 0);
  for (int J = 0; J < nJ; ++J) {
    const int b = J & 1;
    wait_all();
    __syncthreads();  // block J landed in every wave's copy; block J - 1's readers are done
    if (J + 1 < nJ) stage(J + 1, b ^ 1);
    const int k0 = J * CH;
    if (!active || k0 > rbase + 31) continue;  // keys all after the wave's rows
    // S^T per 32-key half: lane = row n, register j = key k0 + 32 h + acc_row(hh, j)
    f32x16 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i)
        sc[h] = mma32(*(const kfrag *)(Ks(b) + KT::off(32 * h + n, 2 * i + hh)), qf[i], sc[h]);
    }
    // bias G_row - G_key = (G_row - ref_J) - loc_key
    const float gq = (float)(grow - Rf(b)[0]);
    float mb = -INFINITY;
    // Only a block that reaches past the wave's first row or the sequence end
    // needs the causal mask.
    if (k0 + CH - 1 <= rbase && k0 + CH <= L) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sc[h][j] *= sl2;
          mb = fmaxf(mb, sc[h][j]);
        }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 32 * h + acc_row(hh, j);
          sc[h][j] = (key <= row && key < L) ? sc[h][j] * sl2 : -INFINITY;
          mb = fmaxf(mb, sc[h][j]);
        }
    }
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mn = fmaxf(m, mb);
    if (__any(mn > m)) {
      // row factors through LDS: lane n (hh = 0) writes its row's, every lane
      // reads the four rows of each of its register groups as one float4 (one
      // write and four reads where a shuffle per register took sixteen)
      float *rs = (float *)(smem + O_S) + 32 * wave;
      if (hh == 0) rs[n] = m == -INFINITY ? 0.f : fast_exp2(m - mn);
      // a wave's LDS accesses complete in order: its own write is visible to
      // its reads once it has completed
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 r4 = *(const float4 *)(rs + 8 * q4 + 4 * hh);
#pragma unroll
        for (int bv = 0; bv < NB; ++bv) {
          acc[bv][4 * q4 + 0] *= r4.x;
          acc[bv][4 * q4 + 1] *= r4.y;
          acc[bv][4 * q4 + 2] *= r4.z;
          acc[bv][4 * q4 + 3] *= r4.w;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    m = mn;
    f16x8 pf[2][2];
    const float *gk = Gk(b);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        pf[h][j >> 3][j & 7] = (_Float16)fast_exp2(sc[h][j] - m + gq - gk[32 * h + acc_row(hh, j)]);
#pragma unroll
    for (int bv = 0; bv < NB; ++bv)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          acc[bv] = mma32(pf[h][u], tr_frag<VT>(Vs(b), 32 * h + 16 * u, 32 * bv, lane), acc[bv]);
  }

  // epilogue: RMSNorm over the row, weight, output gate; x, m, rstd (for dv
  // < 32 the columns past dv hold values read past the narrow V rows: left out)
  float ss[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float t = 0.f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
      if (32 * bb + n < DV) t += acc[bb][j] * acc[bb][j];
    ss[j] = t;
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j) ss[j] += __shfl_xor(ss[j], off);
  if (!active) return;
  float wv[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int d = 32 * bb + n;
    wv[bb] = (a.o_norm && a.w && d < DV) ? load_in(a.w, d, F32IN) : 1.f;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = rbase + acc_row(hh, j);
    if (r >= L) continue;
    const float rs = 1.f / sqrtf(ss[j] * (1.f / DV) + a.eps);
    const int64_t rb = ((st + r) * Hq + hq) * DV;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int d = 32 * bb + n;
      if (d >= DV) continue;
      const float xv = acc[bb][j];
      if (a.x) a.x[rb + d] = xv;
      float ov = a.o_norm ? xv * rs * wv[bb] : xv;
      if (a.z) ov *= load_in(a.z, rb + d, F32IN);
      store_out(a.o, rb + d, ov, a.out_f32);
    }
    if (n == j) a.rstd[(st + r) * Hq + hq] = rs;
  }
  if (hh == 0 && row < L) a.m[(st + row) * Hq + hq] = m * LN2;
}

hipError_t launch_fox_prefix(const float *g, bool logits, const Plan &plan, int nseq, int Hkv, float *loc,
                             double *ref, hipStream_t st) {
  if (logits) hipLaunchKernelGGL(k_fox_prefix<true>, dim3(nseq, Hkv), dim3(256), 0, st, g, plan, Hkv, loc, ref);
  else hipLaunchKernelGGL(k_fox_prefix<false>, dim3(nseq, Hkv), dim3(256), 0, st, g, plan, Hkv, loc, ref);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t fox_dv(bool f32in, const FoxArgs &a, int grid, hipStream_t st) {
  if (f32in) hipLaunchKernelGGL((k_fox_fwd<DK, DV, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_fox_fwd<DK, DV, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <int DK>
static hipError_t fox_dk(int dv, bool f32in, const FoxArgs &a, int grid, hipStream_t st) {
  switch (dv) {
    case 16: return fox_dv<DK, 16>(f32in, a, grid, st);
    case 32: return fox_dv<DK, 32>(f32in, a, grid, st);
    case 64: return fox_dv<DK, 64>(f32in, a, grid, st);
    case 128: return fox_dv<DK, 128>(f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}
hipError_t launch_fox_fwd(int dk, int dv, bool f32in, const FoxArgs &a, int grid, hipStream_t st) {
  switch (dk) {
    case 16: return fox_dk<16>(dv, f32in, a, grid, st);
    case 32: return fox_dk<32>(dv, f32in, a, grid, st);
    case 64: return fox_dk<64>(dv, f32in, a, grid, st);
    case 128: return fox_dk<128>(dv, f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}

// Backward preprocessing of the scalar-gate path: the output-side backward
// (as for the per-channel gate: with r = rstd and xh = x r,
//   dz = dO (.) n (n = xh (.) w under the norm, x without it), dn = dO (.) z,
//   dw = sum over rows of dn (.) xh,
//   delta = r (dn (.) w - xh mean_d(dn (.) w (.) xh))   (dn without the norm))
// and the fp16 operand sigma delta with sigma = 2^-e, max_d |sigma delta|
// about 1, plus the row offset mb = m log2e - e.  One workgroup per 128-chunk
// and kv head, every q head of the group in turn; a thread owns eight
// consecutive channels of a row (DV / 8 threads per row, row reductions by
// shuffles inside that group).
template <int DV>
__global__ void __launch_bounds__(256) k_fox_bwd_prep(FoxPrepArgs a) {
  constexpr int TPR = DV / 8, RPP = 256 / TPR, DVP = DV < 32 ? 32 : DV;
  __shared__ float red[RPP * DV];
  const int gc = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  if (gc >= a.plan.counts[0]) return;
  const Plan &pl = a.plan;
  const int s = seq_of_chunk(pl.cb128, pl.nseq, gc);
  const int t0 = (gc - pl.cb128[s]) * CB;
  const int n = min(CB, pl.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)pl.seq_start[s] + t0;
  const int Hq = a.Hq, G = Hq / a.Hkv;
  const bool in_f32 = a.in_f32, o_norm = a.o_norm;
  const int sub = tid % TPR, d0 = 8 * sub, rr = tid / TPR;
  float wv[8], dwacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    wv[i] = (o_norm && a.w) ? load_in(a.w, d0 + i, in_f32) : 1.f;
    dwacc[i] = 0.f;
  }
  for (int gq = 0; gq < G; ++gq) {
    const int h = c * G + gq;
    for (int r = rr; r < n; r += RPP) {
      const int64_t tok = tok0 + r;
      const int64_t rb = (tok * Hq + h) * DV + d0;
      float xv[8], go[8], zz[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xv[i] = a.x[rb + i];
        go[i] = load_in(a.dO, rb + i, in_f32);
        zz[i] = a.z ? load_in(a.z, rb + i, in_f32) : 1.f;
      }
      const float rs = a.rstd[tok * Hq + h], mrow = a.m[tok * Hq + h];
      float dn[8], proj = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dn[i] = go[i] * zz[i];
        proj += dn[i] * wv[i] * xv[i] * rs;
      }
      if (o_norm) {
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) proj += __shfl_xor(proj, off);
        proj *= 1.f / DV;
      }
      float del[8], amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        del[i] = o_norm ? rs * (dn[i] * wv[i] - xv[i] * rs * proj) : dn[i];
        amax = fmaxf(amax, fabsf(del[i]));
      }
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      int e = 0;
      if (amax > 0.f) e = min(15, max(-15, (int)ceilf(__log2f(amax))));
      const float sg = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
      f16x8 hv;
#pragma unroll
      for (int i = 0; i < 8; ++i) hv[i] = (_Float16)(del[i] * sg);
      _Float16 *drow = a.D16 + (tok * Hq + h) * DVP;
      *(f16x8 *)(drow + d0) = hv;
      if (DV < DVP) *(f16x8 *)(drow + DV + d0) = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
      if (a.dz)
#pragma unroll
        for (int i = 0; i < 8; ++i) store_out(a.dz, rb + i, go[i] * (o_norm ? xv[i] * rs * wv[i] : xv[i]), a.out_f32);
      if (o_norm)
#pragma unroll
        for (int i = 0; i < 8; ++i) dwacc[i] += dn[i] * xv[i] * rs;
      if (sub == 0) a.mb[tok * Hq + h] = mrow * LOG2E - (float)e;
    }
  }
  if (a.dw_part) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rr * DV + d0 + i] = dwacc[i];
    __syncthreads();
    for (int d = tid; d < DV; d += 256) {
      float acc = 0.f;
      for (int q = 0; q < RPP; ++q) acc += red[q * DV + d];
      a.dw_part[((int64_t)gc * a.Hkv + c) * DV + d] = acc;
    }
  }
}

hipError_t launch_fox_bwd_prep(int dv, const FoxPrepArgs &a, int ncb_ub, hipStream_t st) {
  dim3 grid(ncb_ub, a.Hkv);
  switch (dv) {
    case 16: hipLaunchKernelGGL(k_fox_bwd_prep<16>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(k_fox_bwd_prep<32>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(k_fox_bwd_prep<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_fox_bwd_prep<128>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The gate gradient: dL/dG_t = sum over the group of rsum_t,h - csum_t; dg_t is
// its suffix sum over the sequence (fp64 accumulation), times sigmoid(-x_t)
// when the gate was given as logits x.  One workgroup per (sequence, kv head);
// thread u owns a contiguous run of tokens, the runs' totals are combined
// through LDS.
template <bool LOGITS>
__global__ void __launch_bounds__(256) k_fox_dg_scan(const float *__restrict__ rsum, const float *__restrict__ csum,
                                                     const float *__restrict__ logits, Plan plan, int Hq, int Hkv,
                                                     float *__restrict__ dg) {
  const int s = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
  if (s >= plan.nseq) return;
  const int L = plan.seq_len[s];
  const int64_t st = plan.seq_start[s];
  const int G = Hq / Hkv;
  const int per = (L + 255) / 256, t0 = min(L, tid * per), t1 = min(L, t0 + per);
  auto dF = [&](int t) {
    const int64_t tok = st + t;
    float r = 0.f;
    for (int gq = 0; gq < G; ++gq) r += rsum[tok * Hq + c * G + gq];
    return (double)r - (double)csum[tok * Hkv + c];
  };
  __shared__ double tot[256];
  double sum = 0.0;
  for (int t = t0; t < t1; ++t) sum += dF(t);
  tot[tid] = sum;
  __syncthreads();
  double run = 0.0;
  for (int u = tid + 1; u < 256; ++u) run += tot[u];
  for (int t = t1 - 1; t >= t0; --t) {
    run += dF(t);
    const int64_t i = (st + t) * Hkv + c;
    dg[i] = LOGITS ? (float)run * sigmoid_neg(logits[i]) : (float)run;
  }
}

hipError_t launch_fox_dg_scan(const float *rsum, const float *csum, const float *logits, const Plan &plan, int nseq,
                              int Hq, int Hkv, float *dg, hipStream_t st) {
  dim3 grid(nseq, Hkv);
  if (logits) hipLaunchKernelGGL(k_fox_dg_scan<true>, grid, dim3(256), 0, st, rsum, csum, logits, plan, Hq, Hkv, dg);
  else hipLaunchKernelGGL(k_fox_dg_scan<false>, grid, dim3(256), 0, st, rsum, csum, logits, plan, Hq, Hkv, dg);
  return hipGetLastError();
}

// fp16 copy of a [rows, D] tensor into rows of DP >= D elements (zeros past D),
// eight elements per thread.
__global__ void __launch_bounds__(256) k_to_f16_pad(const void *__restrict__ in, bool in_f32, int64_t rows, int D,
                                                    int DP, _Float16 *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per = DP / 8;
  if (e >= rows * per) return;
  const int64_t r = e / per;
  const int c8 = 8 * (int)(e % per);
  f16x8 h;
  if (c8 < D) {
    const int64_t src = r * D + c8;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)load_in(in, src + i, in_f32);
  } else {
    h = __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0));
  }
  *(f16x8 *)(out + r * DP + c8) = h;
}

hipError_t launch_to_f16_pad(const void *in, bool in_f32, int64_t rows, int D, int DP, _Float16 *out, hipStream_t st) {
  if (D % 8 || DP % 8 || DP < D) return hipErrorInvalidValue;
  const int64_t tot = rows * (DP / 8);
  if (tot > 0)
    hipLaunchKernelGGL(k_to_f16_pad, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, in, in_f32, rows, D, DP,
                       out);
  return hipGetLastError();
}

}  // namespace fix
