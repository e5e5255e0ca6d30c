// Device-side work plan: sequence table, chunk offsets and the forward query
// block list, built from cu_seqlens without copying it to the host.
//
// Packed sequences follow the FlashAttention offsets convention the FiX
// README names (section "Quick Start"); a dense [B, T] batch is planned as
// B sequences of length T.  Query blocks are listed longest rows first (the
// causal work of a block grows with its position), so the largest blocks are
// dispatched first and short ones fill the tail of the grid.
#include "common.h"

namespace fix {

constexpr int PLAN_THREADS = 256;

// Block-wide exclusive scan of one int per thread; returns the total.
__device__ static int block_scan(int v, int *tmp, int &excl) {
  int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    int add = (t >= off) ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  int incl = tmp[t];
  int total = tmp[PLAN_THREADS - 1];
  __syncthreads();
  excl = incl - v;
  return total;
}

__global__ void __launch_bounds__(PLAN_THREADS) k_plan(const int64_t *cu, int nseq, int T, int64_t Ttot,
                                                        Plan plan) {
  __shared__ int tmp[PLAN_THREADS];
  __shared__ int red[PLAN_THREADS];
  int t = threadIdx.x;
  // Sequence table and chunk prefix sums.  Sequence s spans [P_s, P_{s+1})
  // with P the running maximum of the offsets clamped into [0, Ttot], so a
  // malformed cu_seqlens (decreasing or out of range) can neither overlap
  // sequences nor exceed the token range or the planned grid sizes.
  __shared__ int64_t mx64[PLAN_THREADS];
  int64_t carry = cu ? min(max(cu[0], (int64_t)0), Ttot) : 0;
  int run = 0, run128 = 0, maxlen = 0;
  for (int base = 0; base < nseq; base += PLAN_THREADS) {
    int s = base + t;
    int64_t b = 0;
    if (s < nseq) {
      b = cu ? cu[s + 1] : (int64_t)(s + 1) * T;
      b = min(max(b, (int64_t)0), Ttot);
    }
    mx64[t] = b;
    __syncthreads();
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {
      int64_t o = (t >= off) ? mx64[t - off] : 0;
      __syncthreads();
      mx64[t] = max(mx64[t], o);
      __syncthreads();
    }
    const int64_t en = max(carry, mx64[t]);
    const int64_t st = (t == 0) ? carry : max(carry, mx64[t - 1]);
    const int64_t tile_max = mx64[PLAN_THREADS - 1];
    __syncthreads();
    carry = max(carry, tile_max);
    int len = 0;
    if (s < nseq) {
      len = (int)(en - st);
      plan.seq_start[s] = (int)st;
      plan.seq_len[s] = len;
    }
    int nch = (len + CH - 1) / CH;
    int excl;
    int tot = block_scan(nch, tmp, excl);
    if (s < nseq) plan.chunk_base[s] = run + excl;
    run += tot;
    int nb = (len + CB - 1) / CB;
    tot = block_scan(nb, tmp, excl);
    if (s < nseq) plan.cb128[s] = run128 + excl;
    run128 += tot;
    maxlen = max(maxlen, len);
  }
  red[t] = maxlen;
  __syncthreads();
  for (int off = PLAN_THREADS / 2; off > 0; off >>= 1) {
    if (t < off) red[t] = max(red[t], red[t + off]);
    __syncthreads();
  }
  int longest = red[0];
  if (t == 0) {
    plan.chunk_base[nseq] = run;
    plan.cb128[nseq] = run128;
    plan.counts[1] = run;
    plan.counts[2] = longest;
  }
  if (t == 0) plan.counts[0] = run128;
}

hipError_t launch_plan(const int64_t *cu, int nseq, int T, int64_t Ttot, const Plan &plan, hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(PLAN_THREADS), 0, st, cu, nseq, T, Ttot, plan);
  return hipGetLastError();
}

}  // namespace fix
