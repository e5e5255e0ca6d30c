// Decode: the FiX output of the newest token of each sequence against a cache
// of the sequence's earlier keys, values and gates (FiX ICML 2026 poster page,
// abstract: inference memory is one of the challenges the method addresses;
// the operation is the one of the FiX README, "Quick Start").
//
// For the newest token t of a sequence and query head h (kv head c):
//   x_t = sum_{j<=t} exp(s_tj - m_t) * exp(G_t - G_j) (.) v_j
// with the per-channel decay exp(G_t - G_j) factored around chunks of
// CH = 64 tokens, as in the forward: a closed chunk n holds its values scaled
// to the chunk end, Vt_j = exp(G_end(n) - G_j) v_j (every factor <= 1 for a
// forget gate), so that its contribution is exp(G_t - G_end(n)) (.) sum_j
// p_tj Vt_j, the chunk factor taken from fp64 prefixes of the chunk totals.
// The open (partial) chunk keeps raw values and its chunk-local prefix, and
// its tokens are decayed one by one.
//
// Cache layout (one caller buffer, carved in this order, 256-byte aligned):
//   len  [B]                      int32   tokens held per sequence
//   K    [B, Hkv, cap, dk]        fp16    keys (a chunk's keys of one head contiguous)
//   VT   [B, cap/64, Hkv, dv, 64] fp16    closed chunks: V scaled to the chunk
//                                         end, transposed, keys in key_pos order
//   Vo   [B, 64, Hkv, dv]         fp16    the open chunk's values (slot t % 64)
//   Go   [B, 64, Hkv, dv]         fp32    its chunk-local inclusive prefix of
//                                         g * log2(e)
//   Lam  [B, cap/64 + 1, Hkv, dv] fp64    log2 decay prefix at each chunk start
// fp16 operands assume |k|, |v| and |q| in [2^-14, 65504] like the backward.
#include "common.h"
#include "launch.h"

namespace fix {

// Appends up to n tokens to every sequence (row b appends the first n_seq[b]
// rows of its [n, Hkv, d] block, or all n when n_seq is null); tokens past
// the capacity are dropped.  The chunk-local prefix restarts at every chunk,
// so the chunks an append touches are independent: workgroup (sequence * Hkv
// + kv head, w) takes the w-th of them, thread i channel i of k and of v / g,
// its tokens in order.  The chunk's prefixes and values stay in LDS (the ring
// only holds the chunk left open); a chunk that fills is sealed (its
// transposed tile, and its total in the Lam slot after it, which
// k_decode_finish turns into the running prefix).  The ring is written here
// only when the chunk left open is the first one touched (the same workgroup
// read its earlier tokens); otherwise k_decode_finish writes it, after every
// reader of the old ring is done.
__global__ void __launch_bounds__(128) k_decode_append(DecodeCache dc, const void *__restrict__ k,
                                                       const void *__restrict__ v, const float *__restrict__ g,
                                                       int n, const int *__restrict__ n_seq, bool in_f32,
                                                       bool logits, int nw) {
  __shared__ float sg[CH][128];      // chunk-local prefixes, [slot][channel]
  __shared__ _Float16 sv[CH][128];   // values
  const int Hkv = dc.Hkv, dk = dc.dk, dv = dc.dv;
  const int b = blockIdx.x / Hkv, c = blockIdx.x % Hkv, i = threadIdx.x;
  const int len0 = dc.len[b];
  const int cnt = min(n_seq ? min(max(n_seq[b], 0), n) : n, dc.cap - len0);
  const int nch = dc.cap / CH;
  for (int w = blockIdx.y; w < nw; w += gridDim.y) {  // each thread only touches its own channel's LDS column
    const int ch = len0 / CH + w, c0 = ch * CH;
    const int ta = max(len0, c0), tb = min(len0 + cnt, c0 + CH);  // tokens of this chunk appended now
    if (ta >= tb) continue;
    // the chunk's earlier tokens (an open chunk from an earlier append) from the ring
    float glp = 0.f;
    if (i < dv)
      for (int t = c0; t < ta; ++t) {
        const int64_t o = (((int64_t)b * CH + t % CH) * Hkv + c) * dv + i;
        glp = dc.Go[o];
        sg[t % CH][i] = glp;
        sv[t % CH][i] = dc.Vo[o];
      }
    for (int t = ta; t < tb; ++t) {
      const int slot = t % CH;
      const int64_t src = (((int64_t)b * n + (t - len0)) * Hkv + c);
      if (i < dk) dc.K[(((int64_t)b * Hkv + c) * dc.cap + t) * dk + i] = (_Float16)load_in(k, src * dk + i, in_f32);
      if (i < dv) {
        float gv = g[src * dv + i];
        if (logits) gv = log_sigmoid(gv);
        glp += gv * LOG2E;
        sg[slot][i] = glp;
        sv[slot][i] = (_Float16)load_in(v, src * dv + i, in_f32);
      }
    }
    if (i >= dv) continue;
    if (tb == c0 + CH) {  // the chunk is full: seal it
      _Float16 row[CH];
      for (int j = 0; j < CH; ++j) row[key_pos(j)] = (_Float16)(fast_exp2(glp - sg[j][i]) * (float)sv[j][i]);
      uint4 *dst = (uint4 *)(dc.VT + ((((int64_t)b * nch + ch) * Hkv + c) * dv + i) * CH);
      for (int p = 0; p < CH / 8; ++p) dst[p] = *(const uint4 *)(row + 8 * p);
      dc.Lam[(((int64_t)b * (nch + 1) + ch + 1) * Hkv + c) * dv + i] = (double)glp;  // the chunk total, for now
    } else if (w == 0) {  // it stays open: its new tokens go to the ring
      for (int t = ta; t < tb; ++t) {
        const int64_t o = (((int64_t)b * CH + t % CH) * Hkv + c) * dv + i;
        dc.Go[o] = sg[t % CH][i];
        dc.Vo[o] = sv[t % CH][i];
      }
    }
  }
}

// After k_decode_append: Lam after every chunk it sealed (the slot holds the
// chunk total, added to the prefix before it, chunk after chunk, fp64), and
// the ring of a chunk left open that started in this append (its prefixes
// recomputed from the inputs, as the append computes them).  Before the new
// lengths are written (it reads the old ones).
__global__ void __launch_bounds__(128) k_decode_finish(DecodeCache dc, const void *__restrict__ v,
                                                       const float *__restrict__ g, int n,
                                                       const int *__restrict__ n_seq, bool in_f32, bool logits) {
  const int Hkv = dc.Hkv, dv = dc.dv, nch = dc.cap / CH;
  const int b = blockIdx.x / Hkv, c = blockIdx.x % Hkv, i = threadIdx.x;
  if (i >= dv) return;
  const int len0 = dc.len[b];
  const int cnt = min(n_seq ? min(max(n_seq[b], 0), n) : n, dc.cap - len0);
  double run = 0.0;
  for (int ch = len0 / CH; ch < (len0 + cnt) / CH; ++ch) {
    const int64_t l = (((int64_t)b * (nch + 1) + ch) * Hkv + c) * dv + i;
    if (ch == len0 / CH) run = dc.Lam[l];
    run += dc.Lam[l + (int64_t)Hkv * dv];
    dc.Lam[l + (int64_t)Hkv * dv] = run;
  }
  const int end = len0 + cnt, c0 = end / CH * CH;
  if (end % CH != 0 && c0 > len0) {
    float glp = 0.f;
    for (int t = c0; t < end; ++t) {
      const int64_t src = (((int64_t)b * n + (t - len0)) * Hkv + c);
      float gv = g[src * dv + i];
      if (logits) gv = log_sigmoid(gv);
      glp += gv * LOG2E;
      const int64_t o = (((int64_t)b * CH + t % CH) * Hkv + c) * dv + i;
      dc.Go[o] = glp;
      dc.Vo[o] = (_Float16)load_in(v, src * dv + i, in_f32);
    }
  }
}

// New lengths, after every workgroup of the append has read the old ones.
__global__ void k_decode_len(DecodeCache dc, int n, const int *__restrict__ n_seq) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < dc.B) dc.len[b] = min(dc.cap, dc.len[b] + (n_seq ? min(max(n_seq[b], 0), n) : n));
}

// Empties every sequence: lengths 0 and a zero decay prefix at chunk 0.
__global__ void k_decode_reset(DecodeCache dc) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)dc.Hkv * dc.dv, nch1 = dc.cap / CH + 1;
  if (e < (int64_t)dc.B * per) dc.Lam[(e / per) * nch1 * per + e % per] = 0.0;
  if (e < dc.B) dc.len[e] = 0;
}

// The open chunk of every (sequence, kv head) as a tile of the closed-chunk
// layout, its values decayed to the newest token: exp2(Gl_t - Gl_j) v_j (zero
// past t), so that the step treats it like a closed chunk with factor 1.
// Block = dv threads (channel d).
__global__ void __launch_bounds__(128) k_decode_open(DecodeCache dc, _Float16 *__restrict__ vto) {
  const int b = blockIdx.x, c = blockIdx.y, d = threadIdx.x, Hkv = dc.Hkv, dv = dc.dv;
  if (d >= dv) return;
  const int len = dc.len[b], open = len % CH, last = (len - 1) % CH;
  _Float16 row[CH];
  const float glt = open ? dc.Go[(((int64_t)b * CH + last) * Hkv + c) * dv + d] : 0.f;
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int64_t o = (((int64_t)b * CH + j) * Hkv + c) * dv + d;
    row[key_pos(j)] = j < open ? (_Float16)(fast_exp2(glt - dc.Go[o]) * (float)dc.Vo[o]) : (_Float16)0.f;
  }
  uint4 *dst = (uint4 *)(vto + (((int64_t)b * Hkv + c) * dv + d) * CH);
  for (int p = 0; p < CH / 8; ++p) dst[p] = *(const uint4 *)(row + 8 * p);
}

// One decode step, split over the cached chunks.  Grid (split, sequence *
// kv head), 4 waves; unit = 4 * split + wave takes chunks unit, unit + U, ...
// (U = 4 * splits), the open chunk being the one numbered nclosed.  A wave
// holds the G query rows of the group padded to 32 (rows >= G are zero) and
// computes S^T = K Q^T per 32-key half (lane = query, registers = keys), so
// the row max is a reduction within a lane; P then is the A operand of the
// P V product with the transposed chunk tile as B (the forward's layout).
// The wave keeps an online row max: on a new maximum its accumulator rows are
// rescaled.  It writes its partial (row max and x over dv) to the workspace.
// The open chunk comes from k_decode_open's tile.
template <int DK, int DV>
__global__ void __launch_bounds__(256, 2) k_decode_step(DecodeCache dc, const void *__restrict__ q, bool in_f32, float sl2,
                                                     int units, const _Float16 *__restrict__ vto,
                                                     float *__restrict__ part, float *__restrict__ mpart) {
  constexpr int NS = DK / 16, NBV = (DV < 32 ? 32 : DV) / 32;
  const int Hkv = dc.Hkv, G = dc.G, nch = dc.cap / CH;
  const int bc = blockIdx.y, b = bc / Hkv, c = bc % Hkv;
  const int lane = threadIdx.x & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = 4 * blockIdx.x + wave;
  const int len = uniform(dc.len[b]);
  const int t = len - 1, nclosed = len / CH, open = len % CH;
  const int nwork = nclosed + (open ? 1 : 0);

  // query of the lane's row n (zero past the group)
  f16x8 qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int64_t o = ((int64_t)b * dc.Hq + c * G + min(n, G - 1)) * DK + 16 * i + 8 * hh;
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[i][e] = n < G ? (_Float16)load_in(q, o + e, in_f32) : (_Float16)0.f;
  }
  // log2 decay prefix of the newest token, per output column of the lane
  double lam_t[NBV];
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int d = min(32 * bv + n, DV - 1);
    const int64_t l = (((int64_t)b * (nch + 1) + nclosed) * Hkv + c) * DV + d;
    lam_t[bv] = len > 0 ? dc.Lam[l] : 0.0;
    if (open) lam_t[bv] += (double)dc.Go[(((int64_t)b * CH + t % CH) * Hkv + c) * DV + d];
  }

  f32x16 acc[NBV];
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) acc[bv] = zero16();
  float mrun = -INFINITY;  // row max (log2 units) of the lane's query row n
  for (int w = unit; w < nwork; w += units) {
    const bool is_open = w == nclosed;
    const int t0 = w * CH;
    // S^T[key][row]: lane = row n, register j = key acc_row(hh, j) of the half.
    f32x16 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = t0 + 32 * h + n;
      const _Float16 *kr = dc.K + (((int64_t)b * Hkv + c) * dc.cap + min(key, t)) * DK;
      sc[h] = zero16();
#pragma unroll
      for (int i = 0; i < NS; ++i) sc[h] = mma32(*(const f16x8 *)(kr + 16 * i + 8 * hh), qf[i], sc[h]);
    }
    float mc = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = t0 + 32 * h + acc_row(hh, j);
        sc[h][j] = key <= t ? sc[h][j] * sl2 : -INFINITY;
        mc = fmaxf(mc, sc[h][j]);
      }
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mnew = fmaxf(mrun, mc);
    if (__any(mnew > mrun)) {
      // rescale accumulator rows: register j holds row acc_row(hh, j)
      const float r = mrun == -INFINITY ? 0.f : fast_exp2(mrun - mnew);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float rj = __shfl(r, acc_row(hh, j));
#pragma unroll
        for (int bv = 0; bv < NBV; ++bv) acc[bv][j] *= rj;
      }
    }
    mrun = mnew;
    // P^T as the A operand: fragment (h, u) = registers 8u .. 8u + 7 of half h
    f16x8 pf[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j) pf[h][j >> 3][j & 7] = (_Float16)fast_exp2(sc[h][j] - mnew);
    // B operand: column d = 32 bv + n, keys of positions 32 h + 16 u + 8 hh ..
    // of the chunk's transposed tile (the open chunk: its decayed copy, factor 1)
#pragma unroll
    for (int bv = 0; bv < NBV; ++bv) {
      const int d = min(32 * bv + n, DV - 1);
      const _Float16 *vt = is_open ? vto + (((int64_t)b * Hkv + c) * DV + d) * CH
                                   : dc.VT + ((((int64_t)b * nch + w) * Hkv + c) * DV + d) * CH;
      f32x16 part_c = zero16();
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 2; ++u) part_c = mma32(pf[h][u], *(const f16x8 *)(vt + 32 * h + 16 * u + 8 * hh), part_c);
      // chunk factor exp2(G_t - G_end(w)) of column d (<= 1; 1 for the open chunk)
      float f = 1.f;
      if (!is_open) f = fast_exp2((float)(lam_t[bv] - dc.Lam[(((int64_t)b * (nch + 1) + w + 1) * Hkv + c) * DV + d]));
      if (32 * bv + n >= DV) f = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[bv][j] += f * part_c[j];
    }
  }
  // partial of this unit: rows r < G, columns d
  const int64_t pbase = ((int64_t)bc * units + unit) * G;
  if (hh == 0 && n < G) mpart[pbase + n] = mrun;
#pragma unroll
  for (int bv = 0; bv < NBV; ++bv) {
    const int d = 32 * bv + n;
    if (d < DV)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = acc_row(hh, j);
        if (r < G) part[(pbase + r) * DV + d] = acc[bv][j];
      }
  }
}

// Combines the units of one (sequence, query head) and applies the output
// transform.  Block = 4 groups of max(DV, 64) threads (thread d of a group:
// channel d); group j sums units j, j + 4, ..., and the four sums are added
// in LDS in a fixed order.
template <int DV>
__global__ void __launch_bounds__(512) k_decode_combine(DecodeCache dc, int units, const float *__restrict__ part,
                                                        const float *__restrict__ mpart, const void *__restrict__ w,
                                                        const void *__restrict__ z, bool in_f32, bool out_f32,
                                                        bool o_norm, float eps, void *__restrict__ o,
                                                        float *__restrict__ m_out) {
  constexpr int DW = DV < 64 ? 64 : DV, NG = 4, NT = NG * DW, NW = NT / 64;
  const int bh = blockIdx.x, b = bh / dc.Hq, h = bh % dc.Hq, G = dc.G, c = h / G, r = h % G;
  const int tid = threadIdx.x, gq = tid / DW, dd = tid % DW, d = min(dd, DV - 1);  // lanes dd >= DV add nothing
  const int64_t bc = (int64_t)b * dc.Hkv + c;
  // the units' row maxima into LDS (units <= 256), their maximum over the block
  __shared__ float mu_s[256];
  __shared__ float red[NW];
  __shared__ float xs[NG][DW];
  float m = -INFINITY;
  for (int u = tid; u < units; u += NT) {
    const float mu = mpart[(bc * units + u) * G + r];
    mu_s[u] = mu;
    m = fmaxf(m, mu);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
  __syncthreads();  // red is reused below
  float x = 0.f;
#pragma unroll 8
  for (int u = gq; u < units; u += NG) {
    const float mu = mu_s[u];
    const float pv = part[((bc * units + u) * G + r) * DV + d];
    if (mu != -INFINITY) x += fast_exp2(mu - m) * pv;
  }
  xs[gq][dd] = x;
  __syncthreads();
  x = ((xs[0][dd] + xs[1][dd]) + xs[2][dd]) + xs[3][dd];
  // RMSNorm over the DV channels of group 0 (every thread takes part in the
  // reductions and barriers; only group 0 writes)
  float ss = gq == 0 && dd < DV ? x * x : 0.f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  ss = red[0];
#pragma unroll
  for (int i = 1; i < DW / 64; ++i) ss += red[i];
  if (gq != 0 || dd >= DV) return;
  const float rs = rsqrtf(ss / DV + eps);
  float y = x;
  if (o_norm) y = x * rs * (w ? load_in(w, d, in_f32) : 1.f);
  if (z) y *= load_in(z, (int64_t)bh * DV + d, in_f32);
  store_out(o, (int64_t)bh * DV + d, y, out_f32);
  if (m_out && d == 0) m_out[bh] = dc.len[b] > 0 ? m / LOG2E : 0.f;
}

hipError_t launch_decode_reset(const DecodeCache &dc, hipStream_t st) {
  const int64_t nthr = (int64_t)dc.B * dc.Hkv * dc.dv;
  hipLaunchKernelGGL(k_decode_reset, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, dc);
  return hipGetLastError();
}

hipError_t launch_decode_append(const DecodeCache &dc, const void *k, const void *v, const float *g, int n,
                                const int *n_seq, bool in_f32, bool logits, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // chunks an append of up to n tokens can touch: an open chunk, then n more tokens
  const int nw = (CH - 1 + n + CH - 1) / CH;
  hipLaunchKernelGGL(k_decode_append, dim3(dc.B * dc.Hkv, min(nw, 65535)), dim3(128), 0, st, dc, k, v, g, n, n_seq,
                     in_f32, logits, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_finish, dim3(dc.B * dc.Hkv), dim3(128), 0, st, dc, v, g, n, n_seq, in_f32, logits);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_len, dim3((dc.B + 63) / 64), dim3(64), 0, st, dc, n, n_seq);
  return hipGetLastError();
}

template <int DK, int DV>
static void step_dv(const DecodeCache &dc, const void *q, bool in_f32, float sl2, int splits, const _Float16 *vto,
                    float *part, float *mpart, hipStream_t st) {
  hipLaunchKernelGGL((k_decode_step<DK, DV>), dim3(splits, dc.B * dc.Hkv), dim3(256), 0, st, dc, q, in_f32, sl2,
                     4 * splits, vto, part, mpart);
}
template <int DK>
static hipError_t step_dk(const DecodeCache &dc, const void *q, bool in_f32, float sl2, int splits,
                          const _Float16 *vto, float *part, float *mpart, hipStream_t st) {
  switch (dc.dv) {
    case 16: step_dv<DK, 16>(dc, q, in_f32, sl2, splits, vto, part, mpart, st); break;
    case 32: step_dv<DK, 32>(dc, q, in_f32, sl2, splits, vto, part, mpart, st); break;
    case 64: step_dv<DK, 64>(dc, q, in_f32, sl2, splits, vto, part, mpart, st); break;
    case 128: step_dv<DK, 128>(dc, q, in_f32, sl2, splits, vto, part, mpart, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_open(const DecodeCache &dc, _Float16 *vto, hipStream_t st) {
  hipLaunchKernelGGL(k_decode_open, dim3(dc.B, dc.Hkv), dim3(dc.dv), 0, st, dc, vto);
  return hipGetLastError();
}

hipError_t launch_decode_step(const DecodeCache &dc, const void *q, bool in_f32, float sl2, int splits,
                              const _Float16 *vto, float *part, float *mpart, hipStream_t st) {
  switch (dc.dk) {
    case 16: return step_dk<16>(dc, q, in_f32, sl2, splits, vto, part, mpart, st);
    case 32: return step_dk<32>(dc, q, in_f32, sl2, splits, vto, part, mpart, st);
    case 64: return step_dk<64>(dc, q, in_f32, sl2, splits, vto, part, mpart, st);
    case 128: return step_dk<128>(dc, q, in_f32, sl2, splits, vto, part, mpart, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeCache &dc, int units, const float *part, const float *mpart,
                                 const void *w, const void *z, bool in_f32, bool out_f32, bool o_norm, float eps,
                                 void *o, float *m, hipStream_t st) {
  const dim3 grid(dc.B * dc.Hq);
  switch (dc.dv) {
    case 16: hipLaunchKernelGGL((k_decode_combine<16>), grid, dim3(256), 0, st, dc, units, part, mpart, w, z, in_f32, out_f32, o_norm, eps, o, m); break;
    case 32: hipLaunchKernelGGL((k_decode_combine<32>), grid, dim3(256), 0, st, dc, units, part, mpart, w, z, in_f32, out_f32, o_norm, eps, o, m); break;
    case 64: hipLaunchKernelGGL((k_decode_combine<64>), grid, dim3(256), 0, st, dc, units, part, mpart, w, z, in_f32, out_f32, o_norm, eps, o, m); break;
    case 128: hipLaunchKernelGGL((k_decode_combine<128>), grid, dim3(512), 0, st, dc, units, part, mpart, w, z, in_f32, out_f32, o_norm, eps, o, m); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fix
