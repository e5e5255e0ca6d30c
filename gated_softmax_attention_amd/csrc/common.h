// Shared device-side definitions for the FiX attention kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fix {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tiling constants shared by every kernel.
constexpr int CH = 64;        // forward gate chunk: chunk-local cumsums restart every CH tokens of a sequence
constexpr int QB = 128;       // forward query block (4 waves x 32 rows)
constexpr int CB = 128;       // backward gate chunk (= one backward workgroup's rows or keys)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Device plan written by k_plan: every sequence's place in the packed token
// order, its first chunk, and the number of chunks.
struct Plan {
  int *seq_start;   // [nseq] first token of each sequence
  int *seq_len;     // [nseq]
  int *chunk_base;  // [nseq + 1] prefix sum of ceil(len / CH)
  int *cb128;       // [nseq + 1] prefix sum of ceil(len / CB)
  int *counts;      // [0] 128-token blocks, [1] 64-token chunks, [2] longest sequence
  int nseq;
};

// Last sequence whose first chunk (of the given table) is <= gc.
__device__ inline int seq_of_chunk(const int *base, int nseq, int gc) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= gc) lo = mid; else hi = mid - 1;
  }
  return __builtin_amdgcn_readfirstlane(lo);  // the same in every lane (gc is per workgroup)
}

// XCD-aware work order.  Workgroups are dispatched round-robin over the 8
// XCDs (blockIdx.x % 8 picks the XCD), each with its own L2.  Item idx =
// xcd * per + slot gives every XCD a contiguous range of an ordered item
// list, so the workgroups running together on one XCD are neighbours in the
// list (the same sequence and head, reading the same tiles at about the same
// time).  Returns -1 for workgroups past the end; the grid must hold at least
// 8 * ceil(nitems / 8) workgroups.
__device__ inline int xcd_item(int nitems) {
  const int x = blockIdx.x & 7, slot = blockIdx.x >> 3, per = (nitems + 7) >> 3;
  const int idx = x * per + slot;
  return (slot < per && idx < nitems) ? idx : -1;
}

// Values that are the same in every lane, marked so for the compiler (they
// then live in SGPRs, as buffer resources built from them must).
__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x), hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Position of key j (0..63) inside a transposed V tile: the two middle
// quads of every 16-key group trade places, so that the eight keys one MFMA
// half-wave contributes (see the 32x32x16 operand layout) are contiguous.
__device__ __host__ inline int key_pos(int j) {
  int q = (j >> 2) & 3;
  int nq = (q == 1) ? 2 : (q == 2) ? 1 : q;
  return (j & ~15) | (nq << 2) | (j & 3);
}

// Operand and result layout of the 32x32x16 MFMA (lane l = 32 * hh + n):
//  * an operand element i of lane (hh, n) carries row/column n and k-index
//    8 * hh + i of its 16-wide k-slab;
//  * result register j of lane (hh, n) holds row acc_row(hh, j), column n.
// A result can feed the next product directly when its rows become the
// k-index: register j = 8 * u + i of a 32-row result then carries k-slab u,
// element i, i.e. row slab_key(u, hh, i) of the 32-row block.
__device__ inline int acc_row(int hh, int j) { return 8 * (j >> 2) + 4 * hh + (j & 3); }
__device__ inline int slab_key(int u, int hh, int i) { return 16 * u + 8 * (i >> 2) + 4 * hh + (i & 3); }

// x = hi + lo to about 16 significant bits, both parts bf16 (fp32 exponent range).
__device__ inline void split_bf16(float x, bf16x8 &hi, bf16x8 &lo, int e) {
  __bf16 h = (__bf16)x;
  hi[e] = h;
  lo[e] = (__bf16)(x - (float)h);
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = 0.f;
  return z;
}

__device__ inline f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Gate given as logits x: the forget gate logsigmoid(x) = min(x, 0) - log1p(exp(-|x|)) (no
// overflow for either sign), and its derivative sigmoid(-x) = 1 / (1 + exp(x)).  log1p(t) for
// t in (0, 1] is log(u) * t / (u - 1) with u = fl(1 + t), which cancels the rounding of u
// (or t itself where u rounds to 1): a few ulp with the hardware log and exp.
__device__ inline float log_sigmoid(float x) {
  const float t = fast_exp2(-fabsf(x) * LOG2E), u = 1.f + t;
  const float l1p = u == 1.f ? t : __logf(u) * __fdividef(t, u - 1.f);
  return fminf(x, 0.f) - l1p;
}
__device__ inline float sigmoid_neg(float x) { return __frcp_rn(1.f + fast_exp2(x * LOG2E)); }

// Maximum of x over lanes l and l ^ 32.  v_permlane32_swap with both
// operands equal to x leaves the low half of x in both halves of one result
// and the high half in both halves of the other, so their maximum is the
// maximum across the two halves in every lane.
__device__ inline float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- LDS tiles filled by direct global->LDS copies ----
// gfx950's buffer_load_dwordx4 ... lds moves 16 bytes per lane from global
// memory straight into LDS, the wave's 64 pieces landing contiguously (1 KB)
// at the wave-uniform base, piece of lane l at base + 16 l.  The source is a
// buffer resource (base and byte count in SGPRs) plus a 32-bit per-lane
// offset: a tile's per-lane offsets are fixed for a kernel (computed once),
// the per-step base goes into the resource, and offsets at or past the
// resource's byte count read as zeros (rows past the end of a sequence).
//
// Tiles are unpadded, [ROWS][RB bytes], and the 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r), with no padding.  swz is a bijection of
// the row bits that select a chunk position within a 256-byte bank period, so
// that the MFMA operand reads (32 lanes reading the same chunk of 32
// consecutive rows) have every 16 lanes on 16 distinct 16-byte bank groups;
// its bits are rotated so that the two lowest row bits (those that differ
// among 4 consecutive rows) land on the top chunk bits, which keeps the
// transposing reads (tr_frag: 4 consecutive rows times 4 consecutive chunks
// per 32 lanes) free of conflicts as well.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes) (raw, stride 0).  Both are the
// same in every lane wherever it is used; that is asserted to the compiler
// so that the resource lives in SGPRs.
__device__ inline rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int nrec = (int)(bytes < 0 ? 0 : bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
}

template <int ROWS, int RB> struct LdsTile {
  static constexpr int CPR = RB / 16;     // 16-byte chunks per row (2..16)
  static constexpr int NCH = ROWS * CPR;  // chunks per tile
  static constexpr int BYTES = ROWS * RB;
  static_assert(CPR >= 2 && CPR <= 16 && NCH % 64 == 0, "tile shape");
  // Every wave issues the same number of copies, NW (a wave with nothing left
  // repeats a piece another wave copies, same bytes to the same place), so
  // that the number of loads in flight never depends on the path taken: the
  // compiler's wait counts stay exact instead of falling back to waiting for
  // everything.
  static constexpr int NI = NCH / 64;             // 1 KB wave copies per tile
  static constexpr int NW = NI < 4 ? 1 : (NI + 3) / 4;
  __device__ static int swz(int r) {
    constexpr int LG = CPR == 16 ? 4 : CPR == 8 ? 3 : CPR == 4 ? 2 : 1;  // log2(CPR)
    constexpr int K = CPR == 16 ? 2 : CPR == 8 ? 1 : 0;                 // row bits below 4 in u
    const int u = (r / (16 / CPR)) % CPR;
    return ((u >> K) | (u << (LG - K))) & (CPR - 1);
  }
  __device__ static int off(int r, int c) { return r * RB + ((c ^ swz(r)) << 4); }
  __device__ static int piece(int t, int wave) { return NI < 4 ? wave % NI : min(wave + 4 * t, NI - 1); }
  // This lane's source offsets in a global tile whose rows are `stride` bytes apart.
  __device__ static void lane_offsets(uint32_t stride, int wave, int lane, uint32_t (&o)[NW]) {
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int p = piece(t, wave) * 64 + lane, r = p / CPR, pc = p % CPR;
      o[t] = (uint32_t)r * stride + (uint32_t)((pc ^ swz(r)) << 4);
    }
  }
  // Copy t of the tile (t < NW), untracked (dma16_untracked, defined below).
  __device__ static void dma_piece_untracked(char *lds, const u32x4 &src, const uint32_t (&o)[NW], int t, int wave);
  // The same split over the W waves of a larger workgroup (NWW copies per wave).
  template <int W> struct Waves {
    static constexpr int NWW = NI < W ? 1 : (NI + W - 1) / W;
    __device__ static int piece(int t, int wave) { return NI < W ? wave % NI : min(wave + W * t, NI - 1); }
    __device__ static void lane_offsets(uint32_t stride, int wave, int lane, uint32_t (&o)[NWW]) {
#pragma unroll
      for (int t = 0; t < NWW; ++t) {
        const int p = piece(t, wave) * 64 + lane, r = p / CPR, pc = p % CPR;
        o[t] = (uint32_t)r * stride + (uint32_t)((pc ^ swz(r)) << 4);
      }
    }
    __device__ static void dma_untracked(char *lds, const u32x4 &src, const uint32_t (&o)[NWW], int wave);
  };
  // Copy the tile.  `wave` must be wave-uniform (an SGPR value).
  __device__ static void dma(char *lds, rsrc_t src, const uint32_t (&o)[NW], int wave) {
#pragma unroll
    for (int t = 0; t < NW; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (void __attribute__((address_space(3))) *)(lds + piece(t, wave) * 1024),
                                               16, o[t], 0, 0, 0);
  }
};

// B operand of a 32x32x16 MFMA whose k index runs over the rows of a row-major
// fp16 LdsTile, read with gfx950's transposing LDS load (ds_read_b64_tr_b16).
// Within each 16-lane group, lane i receives element i % 4 of the 8-byte words
// that lanes 4e + i / 4 (e = 0..3) address, so lane j of a group addresses row
// j / 4 of four rows and columns 4 (j % 4) .. + 3 of the group's sixteen.
// Lane (n, hh) then holds column col0 + n of rows row0 + 8t + 4hh + e as
// element 4t + e (t = 0, 1): the k order of a product's result tile when it is
// the next product's A operand (see slab_key).  row0 is a multiple of 16.
// (The result is reinterpreted as a whole vector: a bit cast of one element
// of an ext_vector_type value reads element 0 with this compiler.)
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <class T> __device__ inline f16x8 tr_frag(const char *tile, int row0, int col0, int lane) {
  const int j = lane & 15, hh = lane >> 5, col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  auto *base = (__attribute__((address_space(3))) char *)tile;
  f16x4 h[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = row0 + 8 * t + 4 * hh + (j >> 2);
    auto *p = (__attribute__((address_space(3))) s16x4 *)(base + T::off(row, col >> 3) + 2 * (col & 7));
    h[t] = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
  }
  return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS reads from a precomputed per-lane byte address (plus a constant), so a
// loop body with a fixed buffer needs no address arithmetic: a 16-byte row
// fragment, and one 8-byte transposing read (ds_read_b64_tr_b16; tr_frag's
// layout, one of its two halves).
typedef __attribute__((address_space(3))) char lds_char;
__device__ inline const lds_char *lds_at(uint32_t a) { return (const lds_char *)(uintptr_t)a; }
__device__ inline f16x8 lds_row16(uint32_t a) { return *(const __attribute__((address_space(3))) f16x8 *)lds_at(a); }
__device__ inline f16x4 lds_tr8(uint32_t a) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4 *)(uintptr_t)a));
}
// The same from an LDS pointer: a constant added to the pointer (rather than
// to the integer address) folds into the instruction's offset field, where
// an integer sum costs a vector add per read.
__device__ inline f16x8 lds_row16p(const lds_char *p) { return *(const __attribute__((address_space(3))) f16x8 *)p; }
__device__ inline f16x4 lds_tr8p(const lds_char *p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p));
}
// A value the compiler must treat as changed here: keeps it from hoisting
// base + constant address sums out of a loop as registers of their own (the
// constant then folds into each instruction's offset field).
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Byte offsets within a tile T of the two 8-byte pieces tr_frag reads for
// (row0 = 0, col0): the pieces for another row0 (a multiple of 16) are
// row0 * RB further on.
template <class T> __device__ inline void tr_offsets(int col0, int lane, uint32_t (&o)[2]) {
  const int j = lane & 15, hh = lane >> 5, col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 8 * t + 4 * hh + (j >> 2);
    o[t] = (uint32_t)(T::off(row, col >> 3) + 2 * (col & 7));
  }
}

// The same copies issued from inline assembly, which the compiler's wait-count
// pass does not see.  That pass makes any LDS read wait for every direct copy
// in flight that it cannot prove to write elsewhere (with a buffer index that
// is not a constant it never can), which stalls loops that keep copies in
// flight across reads of other buffers.  The caller orders these copies with
// explicit waits (wait_vm): loads complete in issue order, so the compiler's
// own counts stay conservative when these are issued between its loads.  The
// resource is given as its four descriptor words; m0 (the LDS base of the
// copy, which must be the same in every lane: it is taken from the first
// active lane, since the compiler cannot always prove it uniform) is declared
// clobbered, so the compiler keeps nothing there across the copy.
// LDS byte address of a pointer into LDS.
__device__ inline uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
// The same for a pointer known to be into LDS (never null): the low 32 bits of
// its flat address, which is the LDS byte address (the generic-to-LDS cast
// above adds only a null check, four scalar instructions per copy).
__device__ inline uint32_t lds_low32(const void *p) { return (uint32_t)(uintptr_t)p; }
__device__ inline u32x4 rsrc_words(const void *base, int64_t bytes) {
  const int nrec = (int)(bytes < 0 ? 0 : bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu,
               (uint32_t)__builtin_amdgcn_readfirstlane(nrec), 0x00020000u};
}
__device__ inline void dma16_untracked(void *lds, const u32x4 &src, uint32_t o) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_low32(lds))), "v"(o), "s"(src) : "memory", "m0");
}
__device__ inline void dma4_untracked(void *lds, const u32x4 &src, uint32_t o) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_low32(lds))), "v"(o), "s"(src) : "memory", "m0");
}

template <int ROWS, int RB>
__device__ inline void LdsTile<ROWS, RB>::dma_piece_untracked(char *lds, const u32x4 &src, const uint32_t (&o)[NW], int t,
                                                              int wave) {
  dma16_untracked(lds + piece(t, wave) * 1024, src, o[t]);
}
template <int ROWS, int RB>
template <int W>
__device__ inline void LdsTile<ROWS, RB>::Waves<W>::dma_untracked(char *lds, const u32x4 &src,
                                                                  const uint32_t (&o)[NWW], int wave) {
#pragma unroll
  for (int t = 0; t < NWW; ++t) dma16_untracked(lds + piece(t, wave) * 1024, src, o[t]);
}

// One copy of 16 (or 4) bytes per lane from a buffer resource at byte offset
// `o`; lane l's piece lands at lds + 16 l (lds + 4 l).  Wave-uniform control
// flow only.
__device__ inline void dma16(void *lds, rsrc_t src, uint32_t o) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (void __attribute__((address_space(3))) *)lds, 16, o, 0, 0, 0);
}
__device__ inline void dma4(void *lds, rsrc_t src, uint32_t o) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (void __attribute__((address_space(3))) *)lds, 4, o, 0, 0, 0);
}

// Wait until at most N of the wave's vector-memory loads are in flight
// (loads, direct LDS copies included, complete in issue order); LDS and
// export counters are left alone.
template <int N> __device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Four 16-byte LDS reads the compiler does not track: it would otherwise
// make them wait for every direct copy in flight into LDS (it cannot tell
// that they touch other regions).  The block waits for its own reads before
// it ends, so its outputs are complete when it returns.
__device__ inline void lds_read4(uint4 &r0, uint4 &r1, uint4 &r2, uint4 &r3, const void *p0, const void *p1,
                                 const void *p2, const void *p3) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3))
      : "memory");
}

__device__ inline void lds_read3(uint4 &r0, uint4 &r1, uint4 &r2, const void *p0, const void *p1, const void *p2) {
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b128 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2))
      : "memory");
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() is a
// release/acquire for every address space, which makes each wave wait for
// all its vector-memory loads before the barrier, direct LDS copies issued for
// later steps included; the copies a step needs are waited for explicitly
// (each wave its own, with wait_vm) before this barrier.
__device__ inline void lds_barrier() {
  // this wave's LDS stores are done (lgkmcnt 0; vmcnt and expcnt at their
  // maxima, i.e. not waited for), then the barrier; the empty asm statements
  // keep the compiler from moving memory accesses across it
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for every outstanding memory operation of the wave (direct LDS copies included).
__device__ inline void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Scalar loads and stores through a buffer resource at a 32-bit byte offset
// (a read past the resource's end returns 0, a write there is dropped).
__device__ inline float buf_ld_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline float buf_ld_in(rsrc_t r, uint32_t idx, bool is_f32) {
  return is_f32 ? buf_ld_f32(r, 4 * idx) : bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, 2 * idx, 0, 0));
}
__device__ inline void buf_st_f32(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}
__device__ inline void buf_st_out(rsrc_t r, uint32_t idx, float v, bool is_f32) {
  if (is_f32) buf_st_f32(r, 4 * idx, v);
  else __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), r, 2 * idx, 0, 0);
}

// Load one scalar of an input tensor stored as bf16 (is_f32 = false) or fp32.
__device__ inline float load_in(const void *p, int64_t idx, bool is_f32) {
  return is_f32 ? ((const float *)p)[idx] : bf16_to_f32(((const uint16_t *)p)[idx]);
}
__device__ inline void store_out(void *p, int64_t idx, float v, bool is_f32) {
  if (is_f32) ((float *)p)[idx] = v;
  else ((uint16_t *)p)[idx] = f32_to_bf16_rne(v);
}

// Eight consecutive input elements as an MFMA operand.  bf16 inputs stay
// bf16; fp32 inputs are rounded to fp16 (their exact products keep the
// logits accurate where bf16 rounding would not).
template <bool F32IN> struct InFrag;
template <> struct InFrag<false> {
  typedef bf16x8 type;
  __device__ static type load(const void *base, int64_t idx) {
    uint4 u = *(const uint4 *)((const uint16_t *)base + idx);
    return __builtin_bit_cast(bf16x8, u);
  }
  __device__ static type zero() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }
};
template <> struct InFrag<true> {
  typedef f16x8 type;
  __device__ static type load(const void *base, int64_t idx) {
    const float4 *p = (const float4 *)((const float *)base + idx);
    float4 a = p[0], b = p[1];
    f16x8 r;
    r[0] = (_Float16)a.x; r[1] = (_Float16)a.y; r[2] = (_Float16)a.z; r[3] = (_Float16)a.w;
    r[4] = (_Float16)b.x; r[5] = (_Float16)b.y; r[6] = (_Float16)b.z; r[7] = (_Float16)b.w;
    return r;
  }
  __device__ static type zero() { return __builtin_bit_cast(f16x8, make_uint4(0, 0, 0, 0)); }
};

}  // namespace fix
