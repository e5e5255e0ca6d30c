// Measured peaks of MI355X (gfx950) for the roofline denominators the
// benchmark reports beside the published ones: a loop of independent
// 32x32x16 bf16 matrix products, a loop of independent v_exp_f32 chains, a
// plain 16-byte-per-lane device copy, and LDS read bandwidth (16-byte row
// reads and the 8-byte transposing reads the matrix-product kernels use).
// Not part of the attention library: only `bench.py --peak-probe` loads this.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Four independent accumulator chains per wave, iters products each.
__global__ void __launch_bounds__(256) k_probe_mfma(int iters, float *out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 1e-3f * (float)((t + i) & 7));
    b[i] = (__bf16)(1e-3f * (float)((t * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  out[(int64_t)blockIdx.x * 256 + t] = s;
}

// Eight independent chains x <- exp2(-x) per lane (values stay in (0.5, 1]).
__global__ void __launch_bounds__(256) k_probe_exp(int iters, float *out) {
  const int t = threadIdx.x;
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = 1e-3f * (float)((t + j) & 63);
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(int64_t)blockIdx.x * 256 + t] = s;
}

__global__ void __launch_bounds__(256) k_probe_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                    int64_t n16) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n16; e += (int64_t)gridDim.x * 256) dst[e] = src[e];
}

// The dq traffic of a key-stationary fused backward at the training shape
// (B sequences of T tokens, H heads, dk = 128, 128-key workgroups): workgroup
// (head, sequence, key chunk J) adds a 64-row x 128-column fp32 tile into
// dq[b, rows, h, :] for every 64-row slice of the sequence from its end down
// to row 128 J, with hardware fp32 atomics (no return); workgroups of one
// (sequence, head) are contiguous in launch order.  Values are 1.0.
// stagger != 0: workgroup J walks its slices starting at a rotated position,
// so that concurrent workgroups of one (sequence, head) add to different rows.
__global__ void __launch_bounds__(256) k_probe_atomic_dq(float *__restrict__ dq, int B, int T, int H, int nchunk,
                                                         int stagger) {
  const int item = blockIdx.x, J = item % nchunk, bh = item / nchunk, h = bh % H, b = bh / H;
  const int t = threadIdx.x, col = t & 127, r0 = t >> 7;  // a wave adds 64 consecutive floats of a row
  const int first = 2 * J, n = T / 64 - first;            // slices first .. T/64 - 1
  for (int i = 0; i < n; ++i) {
    const int s0 = 64 * (first + (stagger ? (i + 7 * J) % n : n - 1 - i));
#pragma unroll 8
    for (int r = r0; r < 64; r += 2) unsafeAtomicAdd(dq + (((int64_t)b * T + s0 + r) * H + h) * 128 + col, 1.0f);
  }
}

// LDS reads: 8 waves per workgroup, 64 KiB of LDS, every lane 8 independent
// reads per iteration at conflict-free addresses (consecutive lanes on
// consecutive 16- or 8-byte words).  MODE 0: 16-byte reads; MODE 1: 8-byte
// transposing reads (ds_read_b64_tr_b16).  The empty asm makes the address
// look changed on every iteration so the loads stay in the loop.
template <int MODE>
__global__ void __launch_bounds__(512) k_probe_lds(int iters, unsigned *out) {
  __shared__ __align__(16) unsigned lds[16384];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < 16384; i += 512) lds[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  constexpr uint32_t W = MODE == 0 ? 16 : 8;
  uint32_t a = (uint32_t)(uintptr_t)lds + W * lane + 1024 * wave;
  unsigned x = 0;
  for (int i = 0; i < iters; ++i) {
    asm volatile("" : "+v"(a));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t aj = a + 8192 * j;  // eight 8 KiB windows: every address stays inside the 64 KiB array
      if (MODE == 0) {
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)aj;
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else {
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(uintptr_t)aj);
        x ^= (unsigned)(v[0] ^ v[1] ^ v[2] ^ v[3]);
      }
    }
  }
  out[(int64_t)blockIdx.x * 512 + t] = x;
}

extern "C" {
int fix_probe_lds(int mode, int blocks, int iters, unsigned *out, void *stream) {
  if (mode == 0) hipLaunchKernelGGL(k_probe_lds<0>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, out);
  else hipLaunchKernelGGL(k_probe_lds<1>, dim3(blocks), dim3(512), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}
int fix_probe_atomic_dq(float *dq, int B, int T, int H, int stagger, void *stream) {
  const int nchunk = T / 128;
  hipLaunchKernelGGL(k_probe_atomic_dq, dim3(B * H * nchunk), dim3(256), 0, (hipStream_t)stream, dq, B, T, H, nchunk,
                     stagger);
  return (int)hipGetLastError();
}
// Grid sizes: enough workgroups for several waves per SIMD on every CU.
int fix_probe_mfma(int blocks, int iters, float *out, void *stream) {
  hipLaunchKernelGGL(k_probe_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}
int fix_probe_exp(int blocks, int iters, float *out, void *stream) {
  hipLaunchKernelGGL(k_probe_exp, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, out);
  return (int)hipGetLastError();
}
int fix_probe_copy(int blocks, const void *src, void *dst, int64_t bytes, void *stream) {
  hipLaunchKernelGGL(k_probe_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4 *)src, (uint4 *)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}
}
