// Host-side paths of the C ABI, for a build with AddressSanitizer on the host
// code: descriptor validation, workspace and cache sizing, and the rejections
// every entry point makes before it enqueues anything.  No call here reaches a
// kernel, so the program runs without a GPU.  Exit status 0 when every
// expectation holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "fixattn.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static fix_attn_desc base_desc() {
  fix_attn_desc d;
  memset(&d, 0, sizeof d);
  d.B = 2; d.T = 300; d.Hq = 4; d.Hkv = 2; d.dk = 64; d.dv = 64;
  d.cu_seqlens = NULL; d.num_seqs = 0;
  d.in_dtype = FIX_BF16; d.out_dtype = FIX_BF16;
  d.scale = 0.f; d.eps = 1e-5f; d.o_norm = 1; d.gate_logits = 0; d.gate_scalar = 0;
  return d;
}

static fix_decode_desc base_decode() {
  fix_decode_desc d;
  memset(&d, 0, sizeof d);
  d.B = 2; d.cap = 256; d.Hq = 4; d.Hkv = 2; d.dk = 64; d.dv = 64;
  d.in_dtype = FIX_BF16; d.out_dtype = FIX_BF16; d.scale = 0.f; d.eps = 1e-5f; d.o_norm = 1;
  return d;
}

int main() {
  // descriptors
  fix_attn_desc d = base_desc();
  EXPECT(fix_attn_validate(&d) == FIX_OK);
  EXPECT(fix_attn_validate(NULL) == FIX_E_INVALID);
  const int dims[] = {16, 32, 64, 128};
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      fix_attn_desc e = base_desc();
      e.dk = dims[a]; e.dv = dims[b];
      EXPECT(fix_attn_validate(&e) == FIX_OK);
      EXPECT(fix_attn_fwd_workspace_size(&e) > 0);
      EXPECT(fix_attn_bwd_workspace_size(&e) > 0);
      e.gate_scalar = 1;
      EXPECT(fix_attn_validate(&e) == FIX_OK);
      EXPECT(fix_attn_bwd_workspace_size(&e) > 0);
    }
  struct { void (*set)(fix_attn_desc &); fix_status want; } cases[] = {
      {[](fix_attn_desc &e) { e.B = 0; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.T = -1; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.Hq = 3; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.Hkv = 0; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.in_dtype = (fix_dtype)7; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.out_dtype = (fix_dtype)-1; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.eps = -1.f; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.scale = NAN; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.eps = NAN; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.gate_scalar = 2; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.cu_seqlens = (const int64_t *)0x1000; e.num_seqs = 2; }, FIX_E_INVALID},  // B != 1
      {[](fix_attn_desc &e) { e.B = 1; e.cu_seqlens = (const int64_t *)0x1000; e.num_seqs = 0; }, FIX_E_INVALID},
      {[](fix_attn_desc &e) { e.dk = 48; }, FIX_E_UNSUPPORTED},
      {[](fix_attn_desc &e) { e.dv = 256; }, FIX_E_UNSUPPORTED},
      {[](fix_attn_desc &e) { e.B = 1; e.T = (int64_t)1 << 31; }, FIX_E_UNSUPPORTED},
      {[](fix_attn_desc &e) { e.B = 1 << 10; e.T = 1 << 20; e.Hq = 64; e.Hkv = 64; e.dk = 128; e.dv = 128; }, FIX_E_UNSUPPORTED},
  };
  for (auto &c : cases) {
    fix_attn_desc e = base_desc();
    c.set(e);
    EXPECT(fix_attn_validate(&e) == c.want);
    EXPECT(fix_attn_fwd_workspace_size(&e) == 0);
    EXPECT(fix_attn_bwd_workspace_size(&e) == 0);
  }
  // entry points: rejected on the host, pointers never dereferenced
  void *fake = (void *)0x10000;
  EXPECT(fix_attn_fwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == FIX_E_INVALID);
  EXPECT(fix_attn_bwd(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                      NULL, NULL, 0, NULL) == FIX_E_INVALID);
  EXPECT(fix_attn_fwd(&d, fake, fake, fake, (const float *)fake, NULL, NULL, fake, (float *)fake, (float *)fake, NULL,
                      fake, 16, NULL) == FIX_E_WORKSPACE);
  EXPECT(fix_attn_fwd(&d, (char *)fake + 2, fake, fake, (const float *)fake, NULL, NULL, fake, (float *)fake,
                      (float *)fake, NULL, fake, (size_t)1 << 40, NULL) == FIX_E_INVALID);
  fix_attn_desc bad = base_desc();
  bad.dk = 48;
  EXPECT(fix_attn_fwd(&bad, fake, fake, fake, (const float *)fake, NULL, NULL, fake, (float *)fake, (float *)fake,
                      NULL, fake, (size_t)1 << 40, NULL) == FIX_E_UNSUPPORTED);
  EXPECT(fix_attn_check_inputs(&bad, fake, fake, fake, 64, NULL) == FIX_E_UNSUPPORTED);
  EXPECT(fix_attn_check_inputs(&d, NULL, fake, fake, 64, NULL) == FIX_E_INVALID);
  EXPECT(fix_attn_check_inputs(&d, fake, fake, NULL, 64, NULL) == FIX_E_INVALID);
  EXPECT(fix_attn_check_inputs(&d, fake, fake, fake, 4, NULL) == FIX_E_WORKSPACE);
  // decode
  fix_decode_desc dd = base_decode();
  EXPECT(fix_decode_validate(&dd) == FIX_OK);
  EXPECT(fix_decode_validate(NULL) == FIX_E_INVALID);
  EXPECT(fix_decode_cache_size(&dd) > 0);
  EXPECT(fix_decode_workspace_size(&dd) > 0);
  struct { void (*set)(fix_decode_desc &); fix_status want; } dcases[] = {
      {[](fix_decode_desc &e) { e.cap = 100; }, FIX_E_INVALID},
      {[](fix_decode_desc &e) { e.B = 0; }, FIX_E_INVALID},
      {[](fix_decode_desc &e) { e.Hq = 5; }, FIX_E_INVALID},
      {[](fix_decode_desc &e) { e.scale = INFINITY; }, FIX_E_INVALID},
      {[](fix_decode_desc &e) { e.dv = 96; }, FIX_E_UNSUPPORTED},
      {[](fix_decode_desc &e) { e.Hq = 64; e.Hkv = 1; }, FIX_E_UNSUPPORTED},
      {[](fix_decode_desc &e) { e.cap = (int64_t)1 << 30; }, FIX_E_UNSUPPORTED},
  };
  for (auto &c : dcases) {
    fix_decode_desc e = base_decode();
    c.set(e);
    EXPECT(fix_decode_validate(&e) == c.want);
    EXPECT(fix_decode_cache_size(&e) == 0);
    EXPECT(fix_decode_workspace_size(&e) == 0);
  }
  EXPECT(fix_decode_reset(&dd, NULL, NULL) == FIX_E_INVALID);
  EXPECT(fix_decode_reset(&dd, (char *)fake + 8, NULL) == FIX_E_INVALID);  // not 256-byte aligned
  EXPECT(fix_decode_append(&dd, fake, fake, fake, (const float *)fake, 0, NULL, NULL) == FIX_E_INVALID);
  EXPECT(fix_decode_append(&dd, fake, fake, fake, (const float *)fake, dd.cap + 1, NULL, NULL) == FIX_E_INVALID);
  // status strings and the host-only trace setting
  for (int s = 0; s <= 6; ++s) {
    const char *msg = fix_attn_status_string((fix_status)s);
    EXPECT(msg != NULL && strlen(msg) > 0);
  }
  EXPECT(strstr(fix_attn_status_string(FIX_E_RANGE), "65504") != NULL);
  fix_attn_set_event_trace(NULL, 0);
  EXPECT(fix_attn_event_trace_count() == 0);
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("host paths: all expectations hold\n");
  return failures ? 1 : 0;
}
