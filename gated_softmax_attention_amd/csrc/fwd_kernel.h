// Fused FiX attention forward for gfx950.
//
// Computes, per query row i of a sequence (FiX README, "Quick Start"; FiX
// ICML 2026 poster page, abstract):
//   x_i = sum_{j<=i} exp(s_ij - m_i) exp(G_i - G_j) (.) v_j,  m_i = max_j s_ij
//   o_i = RMSNorm(x_i) (.) w (.) z_i      (norm and gate optional)
// with no softmax denominator.
//
// Work decomposition.  A workgroup owns QB = 128 query rows of one q head
// (4 waves x 32 rows); keys are visited in gate chunks of CH = 64.
//  * Key chunks at least two before the wave's own chunk use the chunk
//    factoring of the decay (see gate_prep.hip): with A the accumulator
//    relative to the end of the last visited chunk,
//        A <- A (.) Gam_J + P_J . Vt_J
//    where Vt_J (fp16, decay to its chunk end applied) and Gam_J come from
//    the gate preprocess.  Tiles of K and Vt are staged through LDS (double
//    buffered) and shared by the four waves; S = Q K^T is a bf16 MFMA and
//    P.Vt an fp16 MFMA, both with fp32 accumulation.
//  * The chunk before the wave's own chunk and the wave's own chunk are
//    handled in registers, with P and V as bf16x3 (hi*hi + hi*lo + lo*hi):
//    these nearest keys carry the largest decay weights, and their fp16
//    rounding would dominate the error of x (and of the gate gradient built
//    from it).  The previous chunk is one more factored step; if the wave
//    holds the second half of its chunk, the first 32 keys are another one
//    (decay taken to key 31 of the chunk); then the 32x32 diagonal block is
//    factored around the token before the block, V'' = exp(Gl_ref - Gl_j) v_j
//    (>= 1, up to 2^GUARD), which needs fp32 range: it is multiplied as
//    three bf16 MFMAs (hi*hi + hi*lo + lo*hi).  Finally every row is scaled
//    by exp(Gl_i - Gl_ref) <= 1.  If a block's gate range exceeds 2^GUARD,
//    that wave evaluates the block's decays directly instead.
//  * Online max: m is raised only when a row max exceeds it by more than
//    TAU (log2 units), so most steps need no accumulator rescale; P stays
//    <= 2^TAU, well inside fp16.  The exact max is tracked alongside and the
//    rows are corrected by exp(m_used - m_exact) at the end, so x_i is exact
//    for the true row max.
//  * Epilogue: RMSNorm over the row, weight, output gate, stores of o, x,
//    m and rstd.
#pragma once
#include "common.h"
#include "launch.h"

namespace fix {

constexpr float TAU = 8.f;      // lazy max threshold (log2 units)
constexpr float GUARD = 100.f;  // largest factored gate range of a diagonal block (log2 units)

template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, 2) k_fix_fwd(FwdArgs a) {
  using IF = InFrag<F32IN>;
  using kfrag = typename IF::type;
  constexpr int DVP = DV < 32 ? 32 : DV;  // output columns padded to whole 32-wide MFMA blocks
  constexpr int NB = DVP / 32;
  constexpr int NS = DK / 16;
  using KT = LdsTile<CH, DK * 2>;   // K rows of a key chunk (bf16, or fp16 for fp32 inputs)
  using VT = LdsTile<DVP, CH * 2>;  // transposed V tile, rows padded to DVP (zero rows)
  using VTD = LdsTile<DV, CH * 2>;  // the rows a copy fills

  // One LDS object for every tile: with a single object the compiler does not
  // make LDS reads wait for copies in flight into the other buffer.
  constexpr int O_K = 0, O_V = O_K + 2 * KT::BYTES, O_G = O_V + 2 * VT::BYTES, O_A = O_G + 2 * 1024;
  __shared__ __align__(1024) char smem[O_A + 4 * 32 * 4];
  auto Ks = [&](int b) { return smem + O_K + b * KT::BYTES; };
  auto Vs = [&](int b) { return smem + O_V + b * VT::BYTES; };
  auto Gs = [&](int b) { return (float *)(smem + O_G + b * 1024); };  // 256 floats, DV used
  float(*Asc)[32] = (float(*)[32])(smem + O_A);

  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Plan &pl = a.plan;
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  // Items ordered (kv head, sequence, query block from the last, q head of
  // the group): the workgroups of one (sequence, kv head) run together on an
  // XCD and walk the same key chunks upward in step, sharing them in L2.
  const int nblk = pl.counts[0];  // 128-row query blocks
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
  const bool active = wave * 32 < nrows;
  const int Iw = (q0 / CH) + (wave >> 1);          // chunk holding this wave's rows
  // Key chunks before Iw - 1 go through LDS; chunk Iw - 1 and the wave's own
  // chunk are handled per wave from registers at higher precision.
  const int nJ = (nrows > CH) ? (q0 / CH) : max(0, q0 / CH - 1);
  const float sl2 = a.sl2;

  // Q^T operand: lane (hh, n) holds row n of the wave, dims 16s + 8hh .. +7.
  const int qrow = q0 + wave * 32 + n;
  kfrag qf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
    qf[i] = (active && qrow < L) ? IF::load(a.q, ((st + qrow) * Hq + hq) * DK + 16 * i + 8 * hh) : IF::zero();

  // Padding rows of narrow Vt tiles stay zero (their Gam entries, zero too,
  // only scale accumulator columns that stay zero).
  if (DV < DVP) {
    for (int e = tid; e < (DVP - DV) * CH * 2 / 4; e += 256) {
      ((uint32_t *)(Vs(0) + DV * CH * 2))[e] = 0u;
      ((uint32_t *)(Vs(1) + DV * CH * 2))[e] = 0u;
    }
  }

  // Stage key chunk J into LDS buffer b: direct copies for bf16 inputs; fp32
  // inputs are converted to fp16 through registers into the same layout.
  uint32_t ok[KT::NW], ov[VTD::NW];
  KT::lane_offsets(Hkv * DK * 2, wave, lane, ok);
  VTD::lane_offsets(CH * 2, wave, lane, ov);
  auto stage_tile = [&](int J, int b) {
    const int64_t gcJ = cb + J;
    if constexpr (!F32IN) {
      const int64_t kr = (st + J * CH) * Hkv + c;
      KT::dma(Ks(b), make_rsrc((const uint16_t *)a.k + kr * DK, (int64_t)(L - J * CH) * Hkv * DK * 2), ok, wave);
    } else {
      for (int p = tid; p < KT::NCH; p += 256) {
        const int r = p / KT::CPR, cc = p % KT::CPR;
        *(f16x8 *)(Ks(b) + KT::off(r, cc)) = IF::load(a.k, ((st + J * CH + r) * Hkv + c) * DK + 8 * cc);
      }
    }
    VTD::dma(Vs(b), make_rsrc(a.VtT + (gcJ * Hkv + c) * DV * CH, DV * CH * 2), ov, wave);
    // every wave (the same bytes); lanes past DV / 4 read zeros
    dma16(Gs(b), make_rsrc(a.Gam + (gcJ * Hkv + c) * DV, DV * 4), 16 * lane);
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[b][j] = 0.f;
  float m_used = -INFINITY, m_true = -INFINITY;  // per row n, log2 units

  // Multiply accumulator row r by the row factor held in lane r of this half-wave pair.
  auto row_scale = [&](float f) {
    if (hh == 0) Asc[wave][n] = f;
    // A wave's LDS accesses complete in order: waiting for its own write is
    // enough (a memory fence would also wait for the tile copies in flight).
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float4 al = *(const float4 *)&Asc[wave][8 * q4 + 4 * hh];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b][4 * q4 + 0] *= al.x;
        acc[b][4 * q4 + 1] *= al.y;
        acc[b][4 * q4 + 2] *= al.z;
        acc[b][4 * q4 + 3] *= al.w;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // Fold a new row max (log2 units, identical in lanes n and n+32) into the running state.
  auto update_max = [&](float mx) {
    m_true = fmaxf(m_true, mx);
    if (__any(mx > m_used + TAU)) {
      float m_new = fmaxf(m_used, mx);
      float alpha = fast_exp2(m_used - m_new);
      m_used = m_new;
      row_scale(alpha);
    }
  };
  auto row_max = [&](const f32x16 &v) {
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = fmaxf(mx, v[j]);
    return mx;
  };

  // ---------------- inter-chunk loop ----------------
  if (nJ > 0) stage_tile(0, 0);
  wait_all();
  __syncthreads();
  for (int J = 0; J < nJ; ++J) {
    const int b = J & 1;
    const bool comp = active && J < Iw - 1;
    // Operands of a group of products are read from LDS in one batch (one
    // wait for all of them rather than one per product).  The next tile's
    // copies are issued between the first score products (the last step
    // copies its own tile again into the idle buffer, so that every step
    // issues the same copies).
    f32x16 sc[2];
    if (comp) {
#pragma unroll
      for (int be = 0; be < 2; ++be) {
        kfrag ka[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) ka[i] = *(const kfrag *)(Ks(b) + KT::off(32 * be + n, 2 * i + hh));
        __builtin_amdgcn_sched_barrier(0);
        sc[be] = zero16();
#pragma unroll
        for (int i = 0; i < NS; ++i) sc[be] = mma32(ka[i], qf[i], sc[be]);
        if (be == 0) {
          stage_tile(min(J + 1, nJ - 1), b ^ 1);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // two copies
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      stage_tile(min(J + 1, nJ - 1), b ^ 1);
    }
    if (comp) {
      float mx = fmaxf(row_max(sc[0]), row_max(sc[1]));
      mx = max_across_halves(mx) * sl2;
      update_max(mx);
      f16x8 pf[4];
#pragma unroll
      for (int be = 0; be < 2; ++be)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[2 * be + u][i] = (_Float16)fast_exp2(sc[be][8 * u + i] * sl2 - m_used);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        f16x8 vb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) vb[t] = *(const f16x8 *)(Vs(b) + VT::off(32 * bb + n, 2 * t + hh));
        float gam = Gs(b)[32 * bb + n];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[bb][j] *= gam;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[bb] = mma32(pf[t], vb[t], acc[bb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_all();
    __syncthreads();
  }
  if (!active) return;

  // ---------------- own chunk ----------------
  const int wp = wave & 1;
  const int c0 = Iw * CH;      // first token of the chunk (sequence relative)
  const int kb = c0 + 32 * wp;  // first key of the diagonal block
  const float *Gl2 = a.Gl2;
  auto gl_at = [&](int tok, int d) { return Gl2[((st + tok) * Hkv + c) * DV + d]; };
  auto v_at = [&](int tok, int d) { return load_in(a.v, ((st + tok) * Hkv + c) * DV + d, F32IN); };
  float glref[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    int d = 32 * bb + n;
    glref[bb] = (wp == 1 && d < DV) ? gl_at(c0 + 31, d) : 0.f;
  }
  // 32 keys kb0 .. kb0+31 that precede every row of the wave, with the decay
  // taken to the token whose chunk-local log2 prefix sum is gref (>= every
  // key's, so each factor is <= 1).  P and V are multiplied as bf16x3: these
  // nearest keys carry the largest decay weights.
  auto near_block = [&](int kb0, const float *gref) {
    f32x16 s1 = zero16();
#pragma unroll
    for (int i = 0; i < NS; ++i)
      s1 = mma32(IF::load(a.k, ((st + kb0 + n) * Hkv + c) * DK + 16 * i + 8 * hh), qf[i], s1);
    update_max(max_across_halves(row_max(s1)) * sl2);
    bf16x8 ph[2], plo[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) split_bf16(fast_exp2(s1[8 * u + i] * sl2 - m_used), ph[u], plo[u], i);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int d = 32 * bb + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 vh, vl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = kb0 + slab_key(u, hh, i);
          const float val = (d < DV) ? fast_exp2(gref[bb] - gl_at(tok, d)) * v_at(tok, d) : 0.f;
          split_bf16(val, vh, vl, i);
        }
        acc[bb] = mma32(ph[u], vh, acc[bb]);
        acc[bb] = mma32(ph[u], vl, acc[bb]);
        acc[bb] = mma32(plo[u], vh, acc[bb]);
      }
    }
  };
  if (Iw >= 1) {
    // previous chunk: A <- A (.) Gam + P V~ with V~ to the chunk end
    const int jc = (Iw - 1) * CH;
    float gend[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int d = 32 * bb + n;
      gend[bb] = d < DV ? gl_at(jc + CH - 1, d) : 0.f;
      const float gam = fast_exp2(gend[bb]);
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[bb][j] *= gam;
    }
    near_block(jc, gend);
    near_block(jc + 32, gend);
  }
  if (wp == 1) {
    // keys c0 .. c0+31 precede every row of this wave: decay to key 31 of the chunk
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const float gam = fast_exp2(glref[bb]);
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[bb][j] *= gam;
    }
    near_block(c0, glref);
  }

  // Diagonal 32x32 block: keys kb .. kb+31 against rows kb .. kb+31.
  f32x16 s2;
#pragma unroll
  for (int j = 0; j < 16; ++j) s2[j] = 0.f;
  {
    const bool kval = kb + n < L;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      kfrag kf = kval ? IF::load(a.k, ((st + kb + n) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
      s2 = mma32(kf, qf[i], s2);
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (acc_row(hh, j) > n) s2[j] = -INFINITY;
  {
    float mx = row_max(s2);
    mx = max_across_halves(mx) * sl2;
    update_max(mx);
  }
  float p2[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) p2[j] = fast_exp2(s2[j] * sl2 - m_used);

  const int klast = min(kb + 31, L - 1);
  float range = 0.f;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    int d = 32 * bb + n;
    if (d < DV) range = fmaxf(range, glref[bb] - gl_at(klast, d));
  }
  const bool direct = __any(range > GUARD);
  if (!direct) {
    bf16x8 ph[2], plo[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float pv = p2[8 * u + i];
        __bf16 hi = (__bf16)pv;
        ph[u][i] = hi;
        plo[u][i] = (__bf16)(pv - (float)hi);
      }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int d = 32 * bb + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 vh, vl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int tok = kb + slab_key(u, hh, i);
          float val = (tok < L && d < DV) ? fast_exp2(glref[bb] - gl_at(tok, d)) * v_at(tok, d) : 0.f;
          __bf16 hi = (__bf16)val;
          vh[i] = hi;
          vl[i] = (__bf16)(val - (float)hi);
        }
        acc[bb] = mma32(ph[u], vh, acc[bb]);
        acc[bb] = mma32(ph[u], vl, acc[bb]);
        acc[bb] = mma32(plo[u], vh, acc[bb]);
      }
    }
  }
  // Query-side factor exp(Gl_i - Gl_ref) <= 1 for every row of the wave.
  const int rbase = q0 + wave * 32;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int d = 32 * bb + n;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int row = rbase + acc_row(hh, j);
      float gi = (row < L && d < DV) ? gl_at(row, d) : glref[bb];
      acc[bb][j] *= fast_exp2(gi - glref[bb]);
    }
  }
  if (direct) {
    // Rare path (gate range of the block beyond 2^GUARD): exact per-pair decays.
#pragma unroll
    for (int key = 0; key < 32; ++key) {
      const int jsrc = (key >> 3) * 4 + (key & 3), hsrc = (key >> 2) & 1;
      const int tok = kb + key;
      float pk = p2[jsrc];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int d = 32 * bb + n;
        const bool ok = tok < L && d < DV;
        const float gk = ok ? gl_at(tok, d) : 0.f;
        const float vk = ok ? v_at(tok, d) : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          int r = acc_row(hh, j);
          float pij = __shfl(pk, r + 32 * hsrc);
          int row = rbase + r;
          if (ok && row < L && key <= r) acc[bb][j] += pij * fast_exp2(gl_at(row, d) - gk) * vk;
        }
      }
    }
  }
  if (__any(m_used != m_true)) {
    float alpha = fast_exp2(m_used - m_true);
    m_used = m_true;
    row_scale(alpha);
  }

  // ---------------- epilogue ----------------
  float ss[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float t = 0.f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) t += acc[bb][j] * acc[bb][j];
    ss[j] = t;
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j) ss[j] += __shfl_xor(ss[j], off);
  float rs[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) rs[j] = 1.f / sqrtf(ss[j] * (1.f / DV) + a.eps);
  float wv[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    int d = 32 * bb + n;
    wv[bb] = (a.o_norm && a.w && d < DV) ? load_in(a.w, d, F32IN) : 1.f;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = rbase + acc_row(hh, j);
    if (row >= L) continue;
    const int64_t rb = ((st + row) * Hq + hq) * DV;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int d = 32 * bb + n;
      if (d >= DV) continue;
      float xv = acc[bb][j];
      if (a.x) a.x[rb + d] = xv;
      float ov = a.o_norm ? xv * rs[j] * wv[bb] : xv;
      if (a.z) ov *= load_in(a.z, rb + d, F32IN);
      store_out(a.o, rb + d, ov, a.out_f32);
    }
    if (n == j) a.rstd[(st + row) * Hq + hq] = rs[j];
  }
  if (hh == 0 && qrow < L) a.m[(st + qrow) * Hq + hq] = m_true * LN2;
}

template <int DK, int DV>
static hipError_t launch_fwd_dk_dv(bool f32in, const FwdArgs &a, int grid, hipStream_t st) {
  if (f32in) hipLaunchKernelGGL((k_fix_fwd<DK, DV, true>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((k_fix_fwd<DK, DV, false>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_fwd_dk(int dv, bool f32in, const FwdArgs &a, int grid, hipStream_t st) {
  switch (dv) {
    case 16: return launch_fwd_dk_dv<DK, 16>(f32in, a, grid, st);
    case 32: return launch_fwd_dk_dv<DK, 32>(f32in, a, grid, st);
    case 64: return launch_fwd_dk_dv<DK, 64>(f32in, a, grid, st);
    case 128: return launch_fwd_dk_dv<DK, 128>(f32in, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace fix
