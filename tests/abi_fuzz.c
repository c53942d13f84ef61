/* Host-side fuzz of the C ABI's argument validation, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
 *
 * Every launching entry point is called with at least one required pointer or the
 * workspace missing, so validation must refuse the call before any HIP call: the driver
 * checks that no such call returns MOE_OK or MOE_ERR_HIP.  The pure host queries (workspace
 * sizes, amax slots, can-implement) run on the same random shapes, including values at and
 * beyond every documented limit, so that an overflow in the size arithmetic is reported by
 * the sanitizer.  Deterministic: a fixed xorshift seed.  Prints "ok <calls>" on success. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_nvfp4.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {
  uint64_t x = rng_state;
  x ^= x << 13;
  x ^= x >> 7;
  x ^= x << 17;
  rng_state = x;
  return x;
}

static int64_t pick64(const int64_t *v, int n) { return v[next_u64() % (uint64_t)n]; }

/* sizes near every limit the ABI documents, negative and huge values included */
static const int64_t kSizes[] = {-1, 0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 33, 64, 65, 255, 256, 257,
                                 512, 768, 1024, 2048, 4096, 6144, 7168, 65536, 65537, 1 << 20,
                                 INT_MAX, (int64_t)INT_MAX + 1, (int64_t)1 << 40, INT64_MAX};
#define NSIZES ((int)(sizeof(kSizes) / sizeof(kSizes[0])))

static int64_t rand_size(void) {
  if (next_u64() % 4 == 0) return (int64_t)(next_u64() % 100000) - 10;
  return pick64(kSizes, NSIZES);
}

static int rand_int(void) {
  const int64_t v = rand_size();
  return v > INT_MAX ? INT_MAX : (v < INT_MIN ? INT_MIN : (int)v);
}

static long calls = 0;
static int failures = 0;

static void refused(moe_status st, const char *what) {
  calls++;
  if (st == MOE_OK || st == MOE_ERR_HIP) {
    if (failures++ < 10) fprintf(stderr, "%s: returned %d (%s) with a missing pointer\n", what, (int)st,
                                 moe_status_string(st));
  }
}

/* any non-null device-looking address: never dereferenced on the host */
#define FAKE ((void *)(uintptr_t)0x1000)

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 20000;
  for (int s = -2; s < 8; s++) {
    if (moe_status_string((moe_status)s) == NULL) {
      fprintf(stderr, "moe_status_string(%d) is NULL\n", s);
      return 1;
    }
  }
  for (long it = 0; it < iters; it++) {
    /* grouped GEMM: queries on random shapes, launches with a required pointer missing */
    moe_gemm_args a;
    a.A = FAKE;
    a.A_sf = FAKE;
    a.A_gs = FAKE;
    a.A_rows = (next_u64() & 1) ? FAKE : NULL;
    a.rows_A = rand_size();
    a.B = FAKE;
    a.B_sf = FAKE;
    a.B_gs = FAKE;
    a.expert_offsets = FAKE;
    a.E = rand_int();
    a.N = rand_int();
    a.K = rand_int();
    a.R = rand_size();
    a.epilogue = (int)(next_u64() % 5) - 1;
    a.D = FAKE;
    a.amax_out = FAKE;
    a.B_layout = (int)(next_u64() % 4) - 1;
    a.D_sf = FAKE;
    a.D_gs = FAKE;
    const size_t ws = moe_grouped_gemm_nvfp4_workspace(&a);
    const int64_t slots = moe_grouped_gemm_nvfp4_amax_slots(&a);
    const moe_status can = moe_grouped_gemm_nvfp4_can_implement(&a);
    calls += 3;
    if ((ws == 0) != (can != MOE_OK) || (slots == 0) != (can != MOE_OK)) {
      if (failures++ < 10)
        fprintf(stderr, "queries disagree: E=%d N=%d K=%d R=%lld ws=%zu slots=%lld can=%d\n", a.E, a.N, a.K,
                (long long)a.R, ws, (long long)slots, (int)can);
    }
    /* the workspace missing, or too small by one byte */
    refused(moe_grouped_gemm_nvfp4(&a, NULL, ws, NULL), "moe_grouped_gemm_nvfp4(ws NULL)");
    if (ws > 0) refused(moe_grouped_gemm_nvfp4(&a, FAKE, ws - 1, NULL), "moe_grouped_gemm_nvfp4(ws short)");
    /* the weights missing (always required) */
    moe_gemm_args b = a;
    b.B = NULL;
    refused(moe_grouped_gemm_nvfp4(&b, FAKE, (size_t)1 << 40, NULL), "moe_grouped_gemm_nvfp4(B NULL)");
    refused(moe_grouped_gemm_nvfp4_noalloc(&b, NULL), "moe_grouped_gemm_nvfp4_noalloc(B NULL)");
    calls++;
    if (moe_grouped_gemm_nvfp4_can_implement(&b) == MOE_OK && failures++ < 10)
      fprintf(stderr, "can_implement accepted B = NULL\n");
    refused(moe_grouped_gemm_nvfp4_can_implement(NULL), "moe_grouped_gemm_nvfp4_can_implement(NULL)");

    /* routing: the offsets array missing */
    const int T = rand_int(), E = rand_int(), k = rand_int();
    (void)moe_route_permute_workspace(T, E, k);
    calls++;
    refused(moe_route_permute(FAKE, T, E, k, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, (size_t)1 << 40, NULL),
            "moe_route_permute(offsets NULL)");

    /* quantisation: the global-scale pointer missing */
    const int64_t rows = rand_size(), C = rand_size();
    (void)moe_quantize_nvfp4_workspace(rows, C);
    calls++;
    refused(moe_quantize_nvfp4(FAKE, (int)(next_u64() % 3), rows, C, FAKE, FAKE, NULL, (int)(next_u64() % 3),
                               NULL, rand_size(), FAKE, (size_t)1 << 40, NULL),
            "moe_quantize_nvfp4(gs NULL)");

    /* packing: the codes missing, at least one row */
    const int64_t prow = rand_size();
    const int pk = rand_int();
    (void)moe_pack_weights_nvfp4_bytes(prow, pk);
    calls++;
    refused(moe_pack_weights_nvfp4(NULL, FAKE, prow > 0 ? prow : 16, pk, FAKE, NULL), "moe_pack_weights_nvfp4(B NULL)");

    /* FINALIZE: the rows missing, at least one token */
    const int ft = rand_int();
    refused(moe_finalize(NULL, rand_size(), FAKE, FAKE, ft > 0 ? ft : 1, rand_int(), rand_int(), FAKE, NULL),
            "moe_finalize(Y NULL)");
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok %ld\n", calls);
  return 0;
}
