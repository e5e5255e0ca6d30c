/*
 * fixattn.h -- C ABI of the FiX parallel attention library for AMD MI355X
 * (gfx950 / CDNA4).  Library: gated_softmax_attention_amd/libfixattn.so.
 *
 * The operation (FiX repository README, section "Quick Start"; FiX ICML 2026
 * poster page, abstract).  Per sequence, for query head h with kv head
 * c = h / (Hq / Hkv) (contiguous head groups, the FlashAttention convention):
 *
 *   s_ij = scale * <q_i, k_j>            for j <= i in the same sequence
 *   m_i  = max_{j<=i} s_ij
 *   x_i  = sum_{j<=i} exp(s_ij - m_i) * exp(G_i - G_j) (.) v_j,
 *          with G_t = sum_{u<=t} g_u the inclusive per-channel prefix sum of
 *          the log-space forget gate g over the sequence
 *   o_i  = x_i * (mean_d x_i^2 + eps)^-1/2 (.) o_norm_weight   if o_norm
 *        = x_i                                                   otherwise
 *   o_i  = o_i (.) o_gate_i                                     if o_gate given
 *
 * The softmax denominator is not formed: the RMSNorm that follows removes
 * any positive per-row scale (FiX ICML 2026 poster page, abstract), so the
 * gate can act directly on v as an element-wise multiplication.  g is fp32
 * and shaped like v; head dimensions are 16, 32, 64 or 128 (FiX README,
 * "Quick Start", closing note).  Sequences may be packed with cu_seqlens
 * offsets as in FlashAttention (same section).
 *
 * Conventions shared by every entry point
 *  - Layout: every tensor is a contiguous row-major [B, T, H, D] device
 *    buffer (packed: B = 1, T = total tokens), 16-byte aligned.
 *  - Ownership: all buffers belong to the caller.  The library never
 *    allocates or frees device memory and keeps no state between calls
 *    (apart from the opt-in, per-thread event trace setting below);
 *    scratch memory is the caller's `ws` of at least the size the matching
 *    *_workspace_size function returns.  Calls are reentrant.
 *  - Asynchrony: work is enqueued on `hip_stream` (a hipStream_t, NULL for
 *    the null stream); calls return after enqueueing, without a host sync.
 *  - Outputs are fully overwritten, never accumulated into.
 *  - Errors: validation runs on the host before anything is enqueued, so a
 *    call that returns FIX_E_INVALID / FIX_E_UNSUPPORTED / FIX_E_WORKSPACE
 *    wrote nothing.  FIX_E_HIP reports a failed launch; the HIP error code is
 *    then available from fix_attn_last_hip_error() on the calling thread.
 *  - Gate as logits: with gate_logits set, the g argument holds raw
 *    unconstrained logits x and the forget gate is g = logsigmoid(x) =
 *    log(sigmoid(x)) <= 0, applied inside the kernels; dg is then the
 *    gradient with respect to x (dg/dx = sigmoid(-x)).  The pages fix g as a
 *    log-space gate shaped like v (FiX README, "Quick Start"); logsigmoid of
 *    unconstrained logits is the usual way to produce one.
 *  - Scalar gate: with gate_scalar = 1, g (and dg) hold one value per token
 *    and kv head, [B,T,Hkv] fp32, the decay being the same for every channel
 *    (the forgetting-attention case, "Forgetting Transformer" page,
 *    abstract).  Forward and backward then apply it as a bias on the
 *    logits, exp(s_ij - m_i + G_i - G_j), with no value scaling (kernels of
 *    their own); dg is the suffix sum over tokens of the row sums minus the
 *    column sums of dS.  Results equal those of the per-channel call with g
 *    broadcast over dv (dg summed over the channels).
 *  - Range: the backward (and the forward with fp32 inputs) runs some
 *    products on q and k rounded to fp16, so |q| and |k| must not exceed
 *    65504 (fix_attn_check_inputs reports whether they do).  Elements below
 *    2^-14 become fp16 subnormals: each keeps an absolute error below 2^-25.
 *  - Preconditions not checked (they would need a device scan): g <= 0
 *    (a forget gate; results for positive g are only as accurate as fp32
 *    range allows), cu_seqlens non-decreasing with cu[0] = 0 and
 *    cu[num_seqs] = T.
 */
#ifndef FIXATTN_H
#define FIXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FIX_OK = 0,
  FIX_E_INVALID = 1,     /* malformed descriptor or a required NULL pointer */
  FIX_E_UNSUPPORTED = 2, /* well formed but outside what the kernels handle */
  FIX_E_WORKSPACE = 3,   /* workspace smaller than required */
  FIX_E_HIP = 4,         /* a HIP launch failed */
  FIX_E_RANGE = 5        /* fix_attn_check_inputs: q or k outside the fp16 range */
} fix_status;

typedef enum {
  FIX_BF16 = 0, /* bfloat16 */
  FIX_F32 = 1   /* float32 */
} fix_dtype;

typedef struct {
  int64_t B, T;        /* batch and sequence length; packed input: B = 1, T = total tokens */
  int64_t Hq, Hkv;     /* query heads and key/value heads, Hq % Hkv == 0 */
  int64_t dk, dv;      /* head dims of q/k and of v/g/o, each in {16, 32, 64, 128} */
  const int64_t *cu_seqlens; /* device int64 [num_seqs + 1] offsets, or NULL (B dense rows) */
  int64_t num_seqs;    /* number of packed sequences (host-known); ignored without cu_seqlens */
  fix_dtype in_dtype;  /* q, k, v, o_norm_weight, o_gate and d_o */
  fix_dtype out_dtype; /* o, dq, dk, dv and d_o_gate */
  float scale;         /* logit scale; <= 0 selects dk^-1/2 */
  float eps;           /* RMSNorm epsilon (used when o_norm != 0) */
  int32_t o_norm;      /* nonzero: apply RMSNorm and o_norm_weight to the output */
  int32_t gate_logits; /* nonzero: g holds logits x, the gate is logsigmoid(x), dg is d/dx */
  int32_t gate_scalar; /* 1: one gate value per token and kv head, g and dg [B,T,Hkv] (see below); 0: [B,T,Hkv,dv] */
} fix_attn_desc;

/* Checks a descriptor on the host; makes no HIP call (usable without a GPU).
 * FIX_E_INVALID: B, T, Hq, Hkv, dk or dv < 1; Hq % Hkv != 0; cu_seqlens with
 *   B != 1 or num_seqs < 1; unknown dtype; negative eps; NaN scale or eps;
 *   gate_scalar not 0 or 1.
 * FIX_E_UNSUPPORTED: dk or dv not in {16, 32, 64, 128}; B*T*max(Hq, Hkv) *
 *   max(dk, dv) >= 2^40 or B*T >= 2^31 (index ranges of the kernels). */
fix_status fix_attn_validate(const fix_attn_desc *d);

/* Bytes of device scratch fix_attn_fwd / fix_attn_bwd need for this
 * descriptor (0 when the descriptor does not validate).  The size depends
 * only on the descriptor, not on the contents of cu_seqlens. */
size_t fix_attn_fwd_workspace_size(const fix_attn_desc *d);
size_t fix_attn_bwd_workspace_size(const fix_attn_desc *d);

/* Forward pass.
 *   q [B,T,Hq,dk], k [B,T,Hkv,dk], v [B,T,Hkv,dv]       in_dtype
 *   g [B,T,Hkv,dv] ([B,T,Hkv] with gate_scalar)          fp32, log-space forget gate (or its logits)
 *   o_norm_weight [dv] in_dtype or NULL (ones); read only when o_norm
 *   o_gate [B,T,Hq,dv] in_dtype or NULL (no output gate)
 * Outputs (all required except x):
 *   o [B,T,Hq,dv] out_dtype
 *   m [B,T,Hq] fp32: m_i = max_{j<=i} s_ij (natural-log units)
 *   rstd [B,T,Hq] fp32: (mean_d x_i^2 + eps)^-1/2 (written also when o_norm == 0)
 *   x [B,T,Hq,dv] fp32: the un-normalised x_i, or NULL when no backward follows
 * m, rstd and x are the saved state fix_attn_bwd consumes.  Rows of a packed
 * buffer past cu_seqlens[num_seqs] are left untouched. */
fix_status fix_attn_fwd(const fix_attn_desc *d, const void *q, const void *k, const void *v,
                        const float *g, const void *o_norm_weight, const void *o_gate, void *o,
                        float *m, float *rstd, float *x, void *ws, size_t ws_bytes,
                        void *hip_stream);

/* Backward pass, with m held constant (as in FlashAttention-style backward
 * passes; exact when eps = 0, where o does not depend on m).
 *   q, k, v, g, o_norm_weight, o_gate: as given to fix_attn_fwd
 *   m, rstd, x: as written by fix_attn_fwd for the same inputs
 *   d_o [B,T,Hq,dv] in_dtype: gradient of the loss with respect to o
 * Outputs:
 *   dq [B,T,Hq,dk], dk [B,T,Hkv,dk], dv [B,T,Hkv,dv]   out_dtype (required)
 *   dg [B,T,Hkv,dv] fp32 (required; [B,T,Hkv] with gate_scalar): gradient with respect to g
 *      (to the logits with gate_logits)
 *   d_o_norm_weight [dv] fp32, or NULL to skip (written only when o_norm)
 *   d_o_gate [B,T,Hq,dv] out_dtype, or NULL to skip (needs o_gate) */
fix_status fix_attn_bwd(const fix_attn_desc *d, const void *q, const void *k, const void *v,
                        const float *g, const void *o_norm_weight, const void *o_gate,
                        const float *m, const float *rstd, const float *x, const void *d_o,
                        void *dq, void *dk, void *dv, float *dg, float *d_o_norm_weight,
                        void *d_o_gate, void *ws, size_t ws_bytes, void *hip_stream);

/* Input range check for callers that cannot bound q and k: max |q| and
 * max |k| over the whole descriptor (every row of B x T) on the device.
 * Unlike the other entry points it synchronizes hip_stream (the result is
 * read back).  ws: at least 8 bytes of device scratch (the start of the
 * forward or backward workspace will do; contents overwritten).
 * Returns FIX_OK when every |q|, |k| <= 65504 (finite fp16), FIX_E_RANGE
 * when one is larger, infinite or NaN; FIX_E_INVALID / FIX_E_UNSUPPORTED as
 * fix_attn_validate, or for a NULL pointer; FIX_E_WORKSPACE when ws_bytes < 8;
 * FIX_E_HIP when a launch, copy or the synchronization fails. */
fix_status fix_attn_check_inputs(const fix_attn_desc *d, const void *q, const void *k, void *ws, size_t ws_bytes,
                                 void *hip_stream);

/* ---- Decode: the newest token of each sequence against a cache ----
 * Inference runs the operation above one token at a time (FiX ICML 2026
 * poster page, abstract: the method's inference memory).  For the newest
 * token t of sequence b and query head h, fix_decode_step computes o_t (and
 * m_t) exactly as fix_attn_fwd would for row t of the whole sequence held in
 * the cache.  The cache is one caller-owned device buffer of
 * fix_decode_cache_size bytes (256-byte aligned), laid out by the library:
 * keys (fp16), closed 64-token chunks of values scaled to their chunk end
 * (fp16, transposed), the open chunk's values (fp16) and chunk-local gate
 * prefix (fp32), fp64 decay prefixes at chunk starts, and per-sequence
 * lengths.  It holds up to cap tokens per sequence; its contents are only
 * meaningful to these entry points.  fp16 storage assumes |k|, |v|, |q| in
 * [2^-14, 65504] (smaller magnitudes keep an absolute error below 2^-25).
 * Calls on one cache are ordered by their stream; calls that overlap on one
 * cache race. */
typedef struct {
  int64_t B;           /* sequences held by the cache */
  int64_t cap;         /* tokens per sequence, a positive multiple of 64 */
  int64_t Hq, Hkv;     /* query heads and key/value heads, Hq % Hkv == 0, Hq / Hkv <= 32 */
  int64_t dk, dv;      /* head dims, each in {16, 32, 64, 128} */
  fix_dtype in_dtype;  /* q, k, v, o_norm_weight and o_gate */
  fix_dtype out_dtype; /* o */
  float scale;         /* logit scale; <= 0 selects dk^-1/2 */
  float eps;           /* RMSNorm epsilon (used when o_norm != 0) */
  int32_t o_norm;      /* nonzero: apply RMSNorm and o_norm_weight */
  int32_t gate_logits; /* nonzero: g holds logits x and the gate is logsigmoid(x) */
} fix_decode_desc;

/* Host-only check of a decode descriptor (no HIP call).
 * FIX_E_INVALID: B, cap, Hq, Hkv, dk or dv < 1; cap % 64 != 0; Hq % Hkv != 0;
 *   unknown dtype; negative eps; NaN or infinite scale or eps.
 * FIX_E_UNSUPPORTED: dk or dv not in {16, 32, 64, 128}; Hq / Hkv > 32;
 *   cap >= 2^30; B >= 2^20; B * Hq >= 2^31; B * cap * Hkv * max(dk, dv) >= 2^40. */
fix_status fix_decode_validate(const fix_decode_desc *d);

/* Bytes of the cache buffer, and of the scratch fix_decode_step needs (0
 * when the descriptor does not validate). */
size_t fix_decode_cache_size(const fix_decode_desc *d);
size_t fix_decode_workspace_size(const fix_decode_desc *d);

/* Empties every sequence of the cache (lengths 0). */
fix_status fix_decode_reset(const fix_decode_desc *d, void *cache, void *hip_stream);

/* Appends tokens to every sequence: row b of
 *   k [B,n,Hkv,dk], v [B,n,Hkv,dv]   in_dtype
 *   g [B,n,Hkv,dv]                   fp32 log-space gate (or logits)
 * contributes its first n_seq[b] tokens (n_seq: device int32 [B] with
 * 0 <= n_seq[b] <= n, or NULL for all n).  1 <= n <= cap is checked on the
 * host; tokens that would take a sequence past cap are dropped (a device
 * condition the host cannot see). */
fix_status fix_decode_append(const fix_decode_desc *d, void *cache, const void *k, const void *v, const float *g,
                             int64_t n, const int32_t *n_seq, void *hip_stream);

/* One decode step: the output for the newest cached token of every sequence.
 *   q [B,Hq,dk] in_dtype: the query of that token
 *   o_norm_weight [dv] in_dtype or NULL (ones); read only when o_norm
 *   o_gate [B,Hq,dv] in_dtype or NULL
 * Outputs: o [B,Hq,dv] out_dtype (required); m [B,Hq] fp32 or NULL.  A
 * sequence with no tokens gets o = 0 and m = 0.  ws: at least
 * fix_decode_workspace_size bytes. */
fix_status fix_decode_step(const fix_decode_desc *d, const void *cache, const void *q, const void *o_norm_weight,
                           const void *o_gate, void *o, float *m, void *ws, size_t ws_bytes, void *hip_stream);

/* fix_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same kernels and results as fix_decode_step, with the step's scratch
 * taken from a device array inside the library (FIX_DECODE_SCRATCH_BYTES per
 * GPU, held by each GPU the library runs on until the process ends) instead
 * of a caller buffer.  No allocation is made.  The first call on a device
 * resolves that device's copy of the array (a runtime query, best made
 * before any graph capture); every later call on the device reuses it.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams without ordering) race and give undefined results.
 * FIX_E_WORKSPACE: fix_decode_workspace_size(d) > FIX_DECODE_SCRATCH_BYTES.
 * FIX_E_HIP: the current device or the array's address could not be
 * queried. */
#define FIX_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
fix_status fix_decode_step_noalloc(const fix_decode_desc *d, const void *cache, const void *q,
                                   const void *o_norm_weight, const void *o_gate, void *o, float *m,
                                   void *hip_stream);

/* Opt-in launch timing for benchmarks (host side, per calling thread).
 * With events non-NULL and capacity > 0, every later fix_attn_fwd /
 * fix_attn_bwd / fix_decode_step call on this thread records events[0] on its stream before
 * its first kernel and events[i] after its i-th launch, at most capacity
 * events; the events are hipEvent_t created by the caller and stay the
 * caller's.  fix_attn_event_trace_count() gives the number recorded by the
 * last call, fix_attn_event_trace_label(i) (i >= 1) the name of the launch
 * that events[i] closes (NULL out of range).  events == NULL turns it off.
 * A failed hipEventRecord ends the call with FIX_E_HIP.
 *
 * Launch log: with the environment variable FIX_ATTN_LOG set (to anything but
 * "0") when the library first needs it, fix_attn_fwd, fix_attn_bwd and
 * fix_decode_step (and its allocation-free form) write one line to stderr
 * per kernel they enqueue: "[fixattn] <entry point>: <kernel> enqueued on
 * stream <hip_stream>", the kernel names being those of the event trace. */
void fix_attn_set_event_trace(void **events, int capacity);
int fix_attn_event_trace_count(void);
const char *fix_attn_event_trace_label(int i);

/* Static, NUL-terminated description of a status code. */
const char *fix_attn_status_string(fix_status s);

/* hipError_t value of the last FIX_E_HIP returned on the calling thread (0 if none). */
int fix_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FIXATTN_H */
