// Gate preprocess: chunk-local prefix sums of the log-space forget gate and
// the decay-scaled value tiles the forward consumes.
//
// FiX multiplies a cumulative, per-channel decay onto the value vectors (FiX
// ICML 2026 poster page, abstract; the gate is fp32 and shaped like v, FiX
// README, "Quick Start").  Writing G for the per-sequence inclusive prefix
// sum of g, the decay between key j and query i is exp(G_i - G_j).  Every
// sequence is cut into chunks of CH tokens starting at its first token; for
// a chunk n with local prefix sums Gl (restarting at the chunk), the factor
// splits around chunk ends into pieces that are all <= 1 when g <= 0:
//   exp(G_i - G_j) = exp(Gl_i) * prod_{chunks strictly between} Gam_n
//                    * exp(Gl_end(j's chunk) - Gl_j)
// This kernel writes, per (chunk, kv head, channel):
//   Gl2 = log2(e) * Gl        fp32, [Ttot, Hkv, dv] (token-major like g)
//   Gam = exp(Gl at the chunk's last token)   fp32, [chunk, Hkv, dv]
//   VtT = exp(Gl_end - Gl_j) * v_j            fp16, [chunk, Hkv, dv, CH]
// VtT is stored transposed (keys contiguous per channel) in the key_pos
// order, zero past the end of the sequence, which is the operand layout of
// the forward kernel's P.V product.
#include "common.h"

namespace fix {

template <int DV, bool LOGITS>
__global__ void __launch_bounds__(2 * DV) k_gate_prep(const float *__restrict__ g, const void *__restrict__ v,
                                                      bool in_f32, Plan plan, int Hkv, float *__restrict__ Gl2,
                                                      float *__restrict__ Gam, _Float16 *__restrict__ VtT) {
  // Thread (blk, d): channels d, d + 1 of the chunk's 16-token piece blk (two
  // channels per thread: every load and store moves 8 bytes per lane):
  // piece-local prefix sums, then the totals of the pieces before it (through
  // LDS).
  constexpr int STR = CH + 8, NP = CH / 16, TPP = DV / 2;
  __shared__ float tot[NP][DV];
  __shared__ __align__(16) _Float16 tile[DV * STR];
  const int gc = blockIdx.x, c = blockIdx.y, d = 2 * (threadIdx.x % TPP), blk = threadIdx.x / TPP;
  if (gc >= plan.counts[1]) return;
  int lo = 0, hi = plan.nseq - 1;
  while (lo < hi) {  // last sequence whose first chunk is <= gc (skips empty sequences)
    int mid = (lo + hi + 1) >> 1;
    if (plan.chunk_base[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int t0 = (gc - plan.chunk_base[s]) * CH;
  const int n = min(CH, plan.seq_len[s] - t0);
  const int64_t tok0 = (int64_t)plan.seq_start[s] + t0;
  const int j0 = 16 * blk;

  // All loads first (rows past the end repeat the last row and are not
  // used), so that they are in flight together.
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
  float before[2] = {0.f, 0.f}, all[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      before[e] += q < blk ? tot[q][d + e] : 0.f;
      all[e] += tot[q][d + e];
    }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j0 + j < n)
      *(float2 *)(Gl2 + ((tok0 + j0 + j) * Hkv + c) * DV + d) = make_float2(before[0] + gl[j][0], before[1] + gl[j][1]);
  const int64_t cidx = ((int64_t)gc * Hkv + c) * DV + d;
  if (blk == 0) *(float2 *)(Gam + cidx) = make_float2(fast_exp2(all[0]), fast_exp2(all[1]));

  // The transposed tile goes through LDS (this thread's 16 keys of its two
  // channels, then the workgroup's DV x CH tile back out as consecutive
  // 16-byte pieces, so that each store instruction writes whole cache lines).
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    _Float16 row[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      row[key_pos(j)] = (_Float16)(j0 + j < n ? fast_exp2(all[e] - before[e] - gl[j][e]) * vv[j][e] : 0.f);
#pragma unroll
    for (int p = 0; p < 2; ++p) *(uint4 *)&tile[(d + e) * STR + j0 + 8 * p] = *(const uint4 *)(row + 8 * p);
  }
  __syncthreads();
  uint4 *dst = (uint4 *)(VtT + ((int64_t)gc * Hkv + c) * DV * CH);
#pragma unroll
  for (int e = threadIdx.x; e < DV * CH / 8; e += 2 * DV)
    dst[e] = *(const uint4 *)&tile[(e / (CH / 8)) * STR + 8 * (e % (CH / 8))];
}

hipError_t launch_gate_prep(int dv, const float *g, bool logits, const void *v, bool in_f32, const Plan &plan,
                            int Hkv, int nch_ub, float *Gl2, float *Gam, _Float16 *VtT, hipStream_t st) {
  dim3 grid(nch_ub, Hkv);
  switch (dv) {
    case 16:
      if (logits) hipLaunchKernelGGL((k_gate_prep<16, true>), grid, dim3(2 * 16), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      else hipLaunchKernelGGL((k_gate_prep<16, false>), grid, dim3(2 * 16), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      break;
    case 32:
      if (logits) hipLaunchKernelGGL((k_gate_prep<32, true>), grid, dim3(2 * 32), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      else hipLaunchKernelGGL((k_gate_prep<32, false>), grid, dim3(2 * 32), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      break;
    case 64:
      if (logits) hipLaunchKernelGGL((k_gate_prep<64, true>), grid, dim3(2 * 64), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      else hipLaunchKernelGGL((k_gate_prep<64, false>), grid, dim3(2 * 64), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      break;
    case 128:
      if (logits) hipLaunchKernelGGL((k_gate_prep<128, true>), grid, dim3(2 * 128), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      else hipLaunchKernelGGL((k_gate_prep<128, false>), grid, dim3(2 * 128), 0, st, g, v, in_f32, plan, Hkv, Gl2, Gam, VtT);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fix
