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

// Minimum waves per SIMD (HIP's second launch bound; one wave per SIMD per
// workgroup here): three at head dim 64, whose LDS holds four workgroups per
// CU (unbounded it took 179 VGPRs, two workgroups), two otherwise.
constexpr int fwd_waves(int dk, int dv) { return (dk == 64 && dv == 64) ? 3 : 2; }

template <int DK, int DV, bool F32IN>
__global__ void __launch_bounds__(256, fwd_waves(DK, DV)) k_fix_fwd(FwdArgs a) {
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
  // The nearest-key phase after the far loop reuses the same memory (below).
  using KB = LdsTile<32, DK * 2>;    // K rows of a 32-key block (bf16, or fp16 for fp32 inputs)
  using OT = LdsTile<32, DVP * 2>;   // built operand tiles [key][channel], padded columns zero
  constexpr int VRB = DV * (F32IN ? 4 : 2), GRB = DV * 4;  // raw v and gate row bytes (plain layout)
  constexpr int N_NK = 0, N_NV = N_NK + KB::BYTES, N_NG = N_NV + 32 * VRB, N_O = N_NG + 32 * GRB;
  constexpr int N_E = N_O + 4 * OT::BYTES, N_END = N_E + 4 * DVP * 4;
  constexpr int O_K = 0, O_V = O_K + 2 * KT::BYTES, O_G = O_V + 2 * VT::BYTES, O_FAR = O_G + 2 * 1024;
  constexpr int O_A = O_FAR > N_END ? O_FAR : N_END;
  __shared__ __align__(1024) char smem[O_A + 2 * 4 * 32 * 4];
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
  float m_used = -INFINITY;  // per row n, log2 units
  // The exact row max: a register through the far loop (m_far, one max per
  // step), then an LDS slot through the nearest-key phase (this wave's slot of
  // row n; lanes n and n + 32 hold the same value), where a register was
  // spilled and the reload's wait for vector memory also waited for the copies
  // in flight.  The slot address is formed where it is used, from the lane id,
  // so that it is not a register kept (and spilled) across the loops either.
  const uint32_t mt_base = uniform((int)lds_addr(smem + O_A + 4 * 32 * 4)) + 128 * wave;
  auto mt_addr = [&]() {
    uint32_t z = 0;
    asm volatile("" : "+s"(z));
    return mt_base + 4 * (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, z)) & 31);
  };
  auto mt_write = [&](float v) { asm volatile("ds_write_b32 %0, %1" ::"v"(mt_addr()), "v"(v) : "memory"); };
  auto mt_read = [&]() {
    float v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(mt_addr()) : "memory");
    return v;
  };

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
  // Lazy running max (the exact one is kept apart, see above).
  auto raise_max = [&](float mx) {
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
  float m_far = -INFINITY;
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
        // the key fragments in groups of (at most) four
        constexpr int NG = NS < 4 ? NS : 4;
        sc[be] = zero16();
#pragma unroll
        for (int i0 = 0; i0 < NS; i0 += NG) {
          kfrag ka[NG];
#pragma unroll
          for (int i = 0; i < NG; ++i) ka[i] = *(const kfrag *)(Ks(b) + KT::off(32 * be + n, 2 * (i0 + i) + hh));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NG; ++i) sc[be] = mma32(ka[i], qf[i0 + i], sc[be]);
        }
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
      m_far = fmaxf(m_far, mx);
      raise_max(mx);
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
  mt_write(m_far);
  // ---------------- nearest keys: the previous chunk and the own chunk ----------------
  // Key blocks of 32 from the first block of the chunk before the workgroup's
  // first chunk up to the block of its last rows, one per step.  Per block the
  // workgroup stages K, v and the chunk-local log2 gate prefix rows in LDS and
  // builds two operand tiles from them, each as bf16 hi and lo parts (fp32
  // range, about 16 significant bits):
  //   VE_j = exp2(E_b - Gl_j) v_j      (<= |v_j|)   V to the block end E_b
  //   VB_j = exp2(E_p - Gl_j) v_j      (>= |v_j|)   V to the token before the
  //                                                  block (E_p = E_{b-1}, 0 at
  //                                                  a chunk start)
  // A wave whose rows lie after block b takes it as one more factored step,
  // A <- A (.) exp2(E_b - E_p) + P VE; the block of its own rows takes P VB
  // (causal mask) and then scales row i by exp2(Gl_i - E_p) <= 1.  P and the
  // operands are multiplied as bf16x3 (hi*hi + hi*lo + lo*hi): these nearest
  // keys carry the largest decay weights.  A diagonal block whose gate range
  // exceeds 2^GUARD is finished after the loop with exact per-pair decays.
  // (LDS: K rows, raw v and gate rows, the four operand tiles, then E_p, E_b,
  // exp2(E_b - E_p) and the previous block's E_b, DVP floats each.)
  char *nk = smem + N_NK, *nv = smem + N_NV, *ng = smem + N_NG;
  char *tEH = smem + N_O, *tEL = tEH + OT::BYTES, *tBH = tEL + OT::BYTES, *tBL = tBH + OT::BYTES;
  float *Ep = (float *)(smem + N_E), *Eb = Ep + DVP, *Gb = Eb + DVP, *Eprev = Gb + DVP;

  const int a0 = q0 / 32;                      // the workgroup's first row block
  const int aw = a0 + wave;                    // this wave's row block
  const int bmin_w = max(0, 2 * (aw / 2) - 2);  // its nearest key blocks: bmin_w .. aw
  const int nb_lo = max(0, a0 - 2);
  const int nb_hi = (q0 + nrows - 1) / 32;
  uint32_t okn[KB::NW];
  KB::lane_offsets(Hkv * DK * 2, wave, lane, okn);
  // plain row-major copy of a [32][RB] tile whose global rows are `stride` bytes apart
  auto copy_plain = [&](char *dst, const void *src, int64_t bytes, int RB, int stride) {
    const rsrc_t r = make_rsrc(src, bytes);
    const int npieces = 32 * RB / 16, cpr = RB / 16;
    for (int p0 = wave * 64; p0 < npieces; p0 += 256) {
      const int p = p0 + lane, rr = p / cpr, pc = p % cpr;
      dma16(dst + p0 * 16, r, (uint32_t)(rr * stride + pc * 16));
    }
  };
  bool direct = false;

  for (int bk = nb_lo; bk <= nb_hi; ++bk) {
    const int kb0 = bk * 32;
    const int64_t kr = (st + kb0) * Hkv + c;
    const int64_t nrow = (int64_t)(L - kb0) * Hkv;  // rows past the sequence read as zeros
    // stage K, v and Gl rows of the block
    if constexpr (!F32IN) {
      KB::dma(nk, make_rsrc((const uint16_t *)a.k + kr * DK, nrow * DK * 2), okn, wave);
    } else {
      for (int p = tid; p < KB::NCH; p += 256) {
        const int r = p / KB::CPR, cc = p % KB::CPR;
        *(f16x8 *)(nk + KB::off(r, cc)) = kb0 + r < L ? IF::load(a.k, ((st + kb0 + r) * Hkv + c) * DK + 8 * cc) : IF::zero();
      }
    }
    copy_plain(nv, (const char *)a.v + kr * DV * (F32IN ? 4 : 2), nrow * VRB, VRB, Hkv * VRB);
    copy_plain(ng, a.Gl2 + kr * DV, nrow * GRB, GRB, Hkv * GRB);
    wait_all();
    __syncthreads();
    // block end and the factor between the block ends (E_p = 0 at a chunk start)
    for (int d = tid; d < DVP; d += 256) {
      const float ep = (bk & 1) ? Eprev[d] : 0.f;
      const float eb = d < DV ? ((const float *)ng)[31 * DV + d] : 0.f;
      Ep[d] = ep;
      Eb[d] = eb;
      Gb[d] = fast_exp2(eb - ep);
    }
    __syncthreads();
    // operand tiles: thread item (key r, 8 channels).  VE is read only by
    // waves whose rows lie after the block (none after the last one), VB only
    // on a wave's own block (the workgroup's blocks from a0 on); a tile no
    // wave reads is not built.
    const bool needE = bk < nb_hi, needB = bk >= a0;
    auto build = [&](auto wantE, auto wantB) {
      for (int it = tid; it < 32 * (DVP / 8); it += 256) {
        const int r = it / (DVP / 8), c8 = 8 * (it % (DVP / 8));
        bf16x8 eh, el, bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = c8 + e;
          float ve = 0.f, vb = 0.f;
          if (d < DV) {
            const float gl = ((const float *)ng)[r * DV + d];
            const float vv = F32IN ? ((const float *)nv)[r * DV + d] : bf16_to_f32(((const uint16_t *)nv)[r * DV + d]);
            if constexpr (decltype(wantE)::value) ve = fast_exp2(Eb[d] - gl) * vv;
            if constexpr (decltype(wantB)::value) vb = fast_exp2(Ep[d] - gl) * vv;
          }
          if constexpr (decltype(wantE)::value) split_bf16(ve, eh, el, e);
          if constexpr (decltype(wantB)::value) split_bf16(vb, bh, bl, e);
        }
        if constexpr (decltype(wantE)::value) {
          *(bf16x8 *)(tEH + OT::off(r, c8 / 8)) = eh;
          *(bf16x8 *)(tEL + OT::off(r, c8 / 8)) = el;
        }
        if constexpr (decltype(wantB)::value) {
          *(bf16x8 *)(tBH + OT::off(r, c8 / 8)) = bh;
          *(bf16x8 *)(tBL + OT::off(r, c8 / 8)) = bl;
        }
      }
    };
    if (needE && needB) build(std::true_type{}, std::true_type{});
    else if (needE) build(std::true_type{}, std::false_type{});
    else build(std::false_type{}, std::true_type{});
    __syncthreads();
    if (active && bk >= bmin_w && bk <= aw) {
      const bool diag = bk == aw;
      // S^T of the block: lane = the wave's row n, register j = key kb0 + acc_row(hh, j)
      f32x16 s1 = zero16();
      {
        kfrag ka[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) ka[i] = *(const kfrag *)(nk + KB::off(n, 2 * i + hh));
#pragma unroll
        for (int i = 0; i < NS; ++i) s1 = mma32(ka[i], qf[i], s1);
      }
      if (diag)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (acc_row(hh, j) > n) s1[j] = -INFINITY;
      const float mx = max_across_halves(row_max(s1)) * sl2;
      mt_write(fmaxf(mt_read(), mx));
      raise_max(mx);
      float pv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) pv[j] = fast_exp2(s1[j] * sl2 - m_used);
      if (!diag) {
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const float gb = Gb[32 * bb + n];
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[bb][j] *= gb;
        }
      } else {
        // gate range of the block: E_p - Gl at its last key
        const int kl = min(31, L - 1 - kb0);
        float range = 0.f;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const int d = 32 * bb + n;
          if (d < DV) range = fmaxf(range, Ep[d] - ((const float *)ng)[kl * DV + d]);
        }
        direct = __any(range > GUARD);
      }
      if (!direct) {
        bf16x8 ph[2], plo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) split_bf16(pv[8 * u + i], ph[u], plo[u], i);
        const char *th = diag ? tBH : tEH, *tl = diag ? tBL : tEL;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          bf16x8 vh[2], vl[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            vh[u] = __builtin_bit_cast(bf16x8, tr_frag<OT>(th, 16 * u, 32 * bb, lane));
            vl[u] = __builtin_bit_cast(bf16x8, tr_frag<OT>(tl, 16 * u, 32 * bb, lane));
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            acc[bb] = mma32(ph[u], vh[u], acc[bb]);
            acc[bb] = mma32(ph[u], vl[u], acc[bb]);
            acc[bb] = mma32(plo[u], vh[u], acc[bb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (diag) {
        // row i: exp2(Gl_i - E_p) <= 1 (rows of the block are the wave's rows)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const int d = 32 * bb + n;
          const float ep = Ep[d];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = acc_row(hh, j);
            const float gi = (kb0 + r < L && d < DV) ? ((const float *)ng)[r * DV + d] : ep;
            acc[bb][j] *= fast_exp2(gi - ep);
          }
        }
      }
    }
    // keep this block's end for the next (odd) block, once every wave is done with the tiles
    __syncthreads();
    for (int d = tid; d < DVP; d += 256) Eprev[d] = Eb[d];
  }
  if (!active) return;
  const int kb = aw * 32;  // the diagonal block of the wave
  const float *Gl2 = a.Gl2;
  auto gl_at = [&](int tok, int d) { return Gl2[((st + tok) * Hkv + c) * DV + d]; };
  auto v_at = [&](int tok, int d) { return load_in(a.v, ((st + tok) * Hkv + c) * DV + d, F32IN); };
  const int rbase = q0 + wave * 32;
  if (direct) {
    // Rare path (gate range of the block beyond 2^GUARD): exact per-pair decays,
    // with the block's probabilities formed again (m_used is final: the
    // diagonal block is the wave's last).
    float p2[16];
    {
      f32x16 s2 = zero16();
      const bool kval = kb + n < L;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        kfrag kf = kval ? IF::load(a.k, ((st + kb + n) * Hkv + c) * DK + 16 * i + 8 * hh) : IF::zero();
        s2 = mma32(kf, qf[i], s2);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) p2[j] = acc_row(hh, j) > n ? 0.f : fast_exp2(s2[j] * sl2 - m_used);
    }
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
  const float m_true = mt_read();
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
