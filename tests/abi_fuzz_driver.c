/* Argument-validation fuzzer for the C ABI in include/gha.h, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer around the host code of the
 * library (tests/test_abi_sanitized_host.py builds and runs it).
 *
 * It only runs where no HIP device is visible: every call it makes either
 * fails an argument check or, with all arguments acceptable, fails the
 * device check that comes after them, so no kernel is ever launched and the
 * fake pointers below are never dereferenced.  What the sanitizers watch is
 * the validation arithmetic itself (sizes, strides, workspace formulas) over
 * extreme values.  Exit status 0 and a final "ok" line mean every call
 * returned a documented error status with a detail string; 77 means a device
 * was visible and nothing was run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gha.h"

int hipGetDeviceCount(int* count); /* from the HIP runtime (C linkage) */

static uint64_t g_state = 0x243F6A8885A308D3ull;

/* SplitMix64 (Steele, Lea and Flood, 2014) */
static uint64_t next_u64(void) {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static unsigned below(unsigned n) { return (unsigned)(next_u64() % n); }

static const int kInts[] = {-2147483647 - 1, -65536, -1, 0, 1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 33,
                            63, 64, 65, 96, 127, 128, 129, 192, 255, 256, 511, 512, 576, 1024,
                            4096, 8191, 65536, 1 << 20, 1 << 24, 1 << 30, 2147483647};
static const int kSmall[] = {1, 2, 3, 4, 8, 16, 32, 64, 128};
static const int64_t kStrides[] = {-1, 0, 1, 8, 16, 64, 128, 192, 576, 1152, 4096, 1 << 20,
                                   (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX / 4, INT64_MAX};
static const uintptr_t kPtrs[] = {0, 0x10000, 0x10008, 0x7f0000000000ull};
static const float kFloats[] = {0.f, -1.f, 0.0883883f, 1.f, 1e30f, 1.0f / 0.0f};

/* mostly plausible values, sometimes anything */
static int any_int(void) { return below(4) ? kSmall[below(sizeof kSmall / sizeof *kSmall)] : kInts[below(sizeof kInts / sizeof *kInts)]; }
static int dim(void) { static const int d[] = {64, 128, 192, 256, 512, 32, 96, 0, -64}; return below(3) ? d[below(2)] : d[below(sizeof d / sizeof *d)]; }
static gha_dtype dtype(void) { return below(4) ? GHA_BF16 : (gha_dtype)below(4); }
static float flt(void) { return kFloats[below(sizeof kFloats / sizeof *kFloats)]; }
static void* ptr(void) { return (void*)(below(8) ? kPtrs[1] : kPtrs[below(sizeof kPtrs / sizeof *kPtrs)]); }

static gha_tensor tensor(void) {
  gha_tensor t;
  t.ptr = ptr();
  if (below(3)) { /* a plausible (B, H, S, D) layout */
    t.ss = kStrides[5 + below(5)];
    t.sh = t.ss * (1 + below(4096));
    t.sb = t.sh * (1 + below(128));
  } else {
    t.sb = kStrides[below(sizeof kStrides / sizeof *kStrides)];
    t.sh = kStrides[below(sizeof kStrides / sizeof *kStrides)];
    t.ss = kStrides[below(sizeof kStrides / sizeof *kStrides)];
  }
  return t;
}
static const gha_tensor* maybe(const gha_tensor* t) { return below(40) ? t : NULL; }
static size_t ws_bytes(void) {
  static const size_t w[] = {0, 8, 4096, (size_t)1 << 20, (size_t)1 << 30, (size_t)1 << 40, SIZE_MAX};
  return w[below(sizeof w / sizeof *w)];
}

static long g_calls = 0;
static long g_by_status[11];

static int fail_check(const char* what, gha_status s) {
  const char* e = gha_last_error();
  const char* name = gha_status_string(s);
  if (s == GHA_OK || (int)s < 1 || (int)s > 10 || e == NULL || strlen(e) == 0 || strlen(e) >= 512 ||
      strcmp(name, "GHA_ERR_UNKNOWN") == 0) {
    fprintf(stderr, "%s returned %d (%s) with detail \"%s\"\n", what, (int)s, name, e ? e : "(null)");
    return 1;
  }
  ++g_calls;
  ++g_by_status[(int)s];
  return 0;
}

static int expect(const char* what, gha_status s, gha_status want) {
  if (s != want) {
    fprintf(stderr, "%s: got %s, want %s (%s)\n", what, gha_status_string(s), gha_status_string(want),
            gha_last_error());
    return 1;
  }
  return fail_check(what, s);
}

static int fuzz_one(void) {
  gha_tensor a = tensor(), b = tensor(), c = tensor(), d = tensor(), e = tensor(), o = tensor();
  void* ws = ptr();
  const int32_t* sl = (const int32_t*)ptr();
  const int32_t* bt = below(2) ? NULL : (const int32_t*)ptr();
  float* lse = below(2) ? NULL : (float*)ptr();
  int B = any_int(), h = any_int(), g = any_int(), sq = any_int(), L = any_int(), Lh = any_int();
  if (below(2)) { Lh = L; } /* often consistent hints */
  switch (below(11)) {
    case 0:
      return fail_check("gqa_prefill", gqa_prefill(maybe(&a), maybe(&b), maybe(&c), maybe(&o), lse, B, h, g, sq, L,
                                                    dim(), dtype(), dtype(), flt(), (int)below(2), NULL));
    case 1:
      return fail_check("gqa_decode", gqa_decode(maybe(&a), maybe(&b), maybe(&c), sl, maybe(&o), lse, B, h, g, sq, L,
                                                  Lh, dim(), dtype(), dtype(), flt(), ws, ws_bytes(), NULL));
    case 2:
      return fail_check("gqa_decode_paged",
                        gqa_decode_paged(maybe(&a), maybe(&b), maybe(&c), bt, any_int(), any_int(), sl, maybe(&o), lse,
                                         B, h, g, sq, L, Lh, any_int(), dim(), dtype(), dtype(), flt(), ws,
                                         ws_bytes(), NULL));
    case 3:
      return fail_check("gqa_decode_fp8",
                        gqa_decode_fp8(maybe(&a), maybe(&b), maybe(&c), flt(), flt(), bt, any_int(), any_int(), sl,
                                       maybe(&o), lse, B, h, g, sq, L, Lh, any_int(), dim(), dtype(), flt(), ws,
                                       ws_bytes(), NULL));
    case 4:
      return fail_check("gta_shared_score_prefill",
                        gta_shared_score_prefill(maybe(&a), maybe(&b), maybe(&c), maybe(&o), lse, B, h, g, L, dim(),
                                                 dim(), dtype(), dtype(), flt(), (int)below(2), NULL));
    case 5:
      return fail_check("gta_shared_score_decode",
                        gta_shared_score_decode(maybe(&a), maybe(&b), maybe(&c), sl, maybe(&o), lse, B, h, g, sq, L,
                                                Lh, dim(), dim(), dtype(), dtype(), flt(), ws, ws_bytes(), NULL));
    case 6:
      return fail_check("gqla_gqa_decode",
                        gqla_gqa_decode(maybe(&a), maybe(&b), maybe(&c), maybe(&d), maybe(&e), sl, maybe(&o), lse, B,
                                        h, g, sq, L, Lh, dim(), dim(), dtype(), dtype(), flt(), ws, ws_bytes(), NULL));
    case 7:
      return fail_check("gqla_gqa_prefill",
                        gqla_gqa_prefill(maybe(&a), maybe(&b), maybe(&c), maybe(&d), maybe(&e), maybe(&o), lse, B, h,
                                         g, sq, L, dim(), dim(), dtype(), dtype(), flt(), (int)below(2), NULL));
    case 8:
      return fail_check("latent_absorb_decode",
                        latent_absorb_decode(maybe(&a), maybe(&b), maybe(&c), maybe(&d), sl, maybe(&o), lse, B, h, sq,
                                             L, Lh, dim(), dim(), dtype(), dtype(), flt(), ws, ws_bytes(), NULL));
    case 9:
      return fail_check("gqla_absorb_decode",
                        gqla_absorb_decode(maybe(&a), maybe(&b), ptr(), ptr(), maybe(&c), maybe(&d), sl, maybe(&o),
                                           lse, B, h, g, sq, L, Lh, dim(), dim(), dim(), dtype(), dtype(), flt(), ws,
                                           ws_bytes(), NULL));
    default:
      return fail_check("gqa_decode_noalloc",
                        gqa_decode_noalloc(maybe(&a), maybe(&b), maybe(&c), sl, maybe(&o), lse, B, h, g, sq, L, Lh,
                                           dim(), dtype(), dtype(), flt(), NULL));
  }
}

/* the workspace queries are pure host arithmetic: any arguments are allowed */
static void fuzz_queries(void) {
  volatile size_t sink = 0;
  sink += gqa_decode_workspace_bytes(any_int(), any_int(), any_int(), any_int(), any_int(), dim());
  sink += gqa_decode_paged_workspace_bytes(any_int(), any_int(), any_int(), any_int(), any_int(), any_int(), dim());
  sink += gta_shared_score_decode_workspace_bytes(any_int(), any_int(), any_int(), any_int(), any_int(), dim());
  sink += gqla_gqa_decode_workspace_bytes(any_int(), any_int(), any_int(), any_int(), any_int(), dim());
  sink += latent_absorb_decode_workspace_bytes(any_int(), any_int(), any_int(), any_int(), dim());
  sink += gqla_absorb_decode_workspace_bytes(any_int(), any_int(), any_int(), any_int(), dim());
  sink += gqa_decode_noalloc_scratch_bytes();
  (void)sink;
}

/* a few calls whose status is fixed by the contract */
static int pinned(void) {
  gha_tensor q = {(void*)0x10000, 1 << 20, 1 << 14, 128}, misaligned = {(void*)0x10008, 1 << 20, 1 << 14, 128};
  gha_tensor neg = {(void*)0x10000, -1, 1 << 14, 128};
  void* ws = (void*)0x10000;
  const int32_t* sl = (const int32_t*)0x10000;
  int bad = 0;
  bad |= expect("prefill null q", gqa_prefill(NULL, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_NULL);
  bad |= expect("prefill grouping", gqa_prefill(&q, &q, &q, &q, NULL, 1, 8, 3, 16, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_GROUPING);
  bad |= expect("prefill head dim", gqa_prefill(&q, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 96, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_HEAD_DIM);
  bad |= expect("prefill align", gqa_prefill(&misaligned, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_ALIGN);
  bad |= expect("prefill stride", gqa_prefill(&neg, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_STRIDE);
  bad |= expect("prefill dtype", gqa_prefill(&q, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 128, GHA_F32, GHA_BF16, 0.f, 1, NULL), GHA_ERR_DTYPE);
  bad |= expect("prefill causal S_q > S_k", gqa_prefill(&q, &q, &q, &q, NULL, 1, 8, 2, 17, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_SHAPE);
  bad |= expect("prefill valid, no device", gqa_prefill(&q, &q, &q, &q, NULL, 1, 8, 2, 16, 16, 128, GHA_BF16, GHA_BF16, 0.f, 1, NULL), GHA_ERR_HIP);
  bad |= expect("decode null seqlens", gqa_decode(&q, &q, &q, NULL, &q, NULL, 1, 8, 2, 1, 128, 128, 128, GHA_BF16, GHA_BF16, 0.f, ws, 1 << 30, NULL), GHA_ERR_NULL);
  bad |= expect("decode small workspace", gqa_decode(&q, &q, &q, sl, &q, NULL, 1, 8, 2, 1, 128, 128, 128, GHA_BF16, GHA_BF16, 0.f, ws, 8, NULL), GHA_ERR_WORKSPACE);
  bad |= expect("decode s_q > L_max_hint", gqa_decode(&q, &q, &q, sl, &q, NULL, 1, 8, 2, 4, 128, 2, 128, GHA_BF16, GHA_BF16, 0.f, ws, 1 << 30, NULL), GHA_ERR_SHAPE);
  bad |= expect("decode valid, no device", gqa_decode(&q, &q, &q, sl, &q, NULL, 1, 8, 2, 1, 128, 128, 128, GHA_BF16, GHA_BF16, 0.f, ws, 1 << 30, NULL), GHA_ERR_HIP);
  bad |= expect("noalloc beyond its scratch", gqa_decode_noalloc(&q, &q, &q, sl, &q, NULL, 1 << 16, 64, 64, 1, 1 << 20, 1 << 20, 128, GHA_BF16, GHA_BF16, 0.f, NULL), GHA_ERR_WORKSPACE);
  bad |= expect("fp8 zero scale", gqa_decode_fp8(&q, &q, &q, 0.f, 1.f, NULL, 0, 0, sl, &q, NULL, 1, 8, 2, 1, 128, 128, 0, 128, GHA_BF16, 0.f, ws, 1 << 30, NULL), GHA_ERR_SHAPE);
  if (gqa_decode_workspace_bytes(0, 8, 2, 1, 128, 128) != 0 || gqa_decode_workspace_bytes(1, 8, 2, 1, 128, 128) == 0) {
    fprintf(stderr, "gqa_decode_workspace_bytes: 0 for bad sizes, > 0 for good ones\n");
    bad = 1;
  }
  return bad;
}

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 20000;
  if (argc > 2) g_state ^= (uint64_t)strtoull(argv[2], NULL, 0);
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == 0 && n_dev > 0) {
    printf("a HIP device is visible: not fuzzing with fake pointers\n");
    return 77;
  }
  if (pinned()) return 1;
  for (long i = 0; i < iters; ++i) {
    if (fuzz_one()) return 1;
    fuzz_queries();
  }
  printf("statuses:");
  for (int i = 1; i <= 10; ++i) printf(" %s=%ld", gha_status_string((gha_status)i), g_by_status[i]);
  printf("\nok %ld calls\n", g_calls);
  return 0;
}
