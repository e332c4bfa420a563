/* Host-side checks of the C ABI's argument validation, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by test_abi_sanitize.py.
 *
 * Every call here either is a host-only query or fails validation before the
 * library makes any HIP call, so no GPU is needed.  Problems span the valid
 * range, its edges and far outside it (int32 extremes, NaN and infinite
 * scales, sizes whose products overflow 32 bits); tensor pointers are fake,
 * never dereferenced on the host.  The program exits non-zero when a status
 * differs from the expected one; the sanitizers abort on any finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fm.h"

static int failures = 0;

static void expect(const char* what, int line, fm_status got, fm_status want) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d (%s), expected %d\n", line, what, (int)got, fm_status_str(got),
            (int)want);
    ++failures;
  }
}
#define EXPECT(call, want) expect(#call, __LINE__, (call), (want))

static fm_problem prob(int32_t b, int32_t h, int32_t hm, int32_t sq, int32_t sk, int32_t d, float scale) {
  fm_problem p;
  p.batch = b; p.heads = h; p.mask_heads = hm; p.seqlen_q = sq; p.seqlen_k = sk; p.head_dim = d;
  p.softmax_scale = scale;
  p.fwd_rows = 0;
  return p;
}

/* fake device pointers: 256-byte aligned, and one 2 bytes off */
#define FAKE ((void*)(uintptr_t)0x100000)
#define FAKE2 ((void*)(uintptr_t)0x200000)
#define MISAL ((void*)(uintptr_t)0x300002)

int main(void) {
  /* status names, including codes outside the enum */
  for (int s = -3; s < 12; ++s) {
    const char* name = fm_status_str((fm_status)s);
    if (!name || !name[0]) { fprintf(stderr, "fm_status_str(%d) empty\n", s); ++failures; }
  }

  /* host queries over valid, edge and invalid problems */
  const int32_t ext[] = {INT32_MIN, -1, 0, 1, 127, 128, 129, 4096, 32768 * 128, 32768 * 128 + 1, INT32_MAX};
  const float scales[] = {0.125f, 1e-30f, 0.f, -1.f, INFINITY, NAN};
  const int n_ext = (int)(sizeof ext / sizeof ext[0]);
  long checked = 0;
  for (int i = 0; i < n_ext; ++i)
    for (int j = 0; j < n_ext; ++j)
      for (int s = 0; s < 6; ++s) {
        const int32_t shapes[4][2] = {{1, 2}, {ext[i], 8}, {2, ext[i]}, {ext[i], ext[j]}};
        for (int k = 0; k < 4; ++k) {
          fm_problem p = prob(shapes[k][0], shapes[k][1], 1, ext[i], ext[j], (s & 1) ? 64 : 128, scales[s]);
          int32_t bq = 0, bk = 0;
          fm_tileinfo_layout lay;
          size_t bytes = 0;
          const fm_status st = fm_tile_shape(&p, &bq, &bk);
          EXPECT(fm_tileinfo_layout_query(&p, &lay), st);
          EXPECT(fm_bwd_workspace_bytes(&p, &bytes), st);
          const uint64_t tiles[] = {0, 1, 1000, 0xFFFFFFFEull, 0xFFFFFFFFull, UINT64_MAX};
          for (int t = 0; t < 6; ++t) {
            const fm_status cs = fm_bwd_cache_bytes(&p, tiles[t], &bytes);
            if (st != FM_OK) EXPECT(cs, st);
            else if (tiles[t] >= 0xFFFFFFFFull) EXPECT(cs, FM_ERR_SHAPE);
            else EXPECT(cs, FM_OK);
          }
          if (st == FM_OK && lay.total < lay.colbase) { fprintf(stderr, "layout total below colbase\n"); ++failures; }
          ++checked;
        }
      }
  /* NULL outputs and problems */
  fm_problem ok = prob(2, 4, 1, 1000, 900, 128, 0.1f);
  fm_tileinfo_layout lay;
  size_t bytes;
  int32_t bq, bk;
  EXPECT(fm_tile_shape(NULL, &bq, &bk), FM_ERR_NULL);
  EXPECT(fm_tile_shape(&ok, NULL, &bk), FM_ERR_NULL);
  EXPECT(fm_tileinfo_layout_query(&ok, NULL), FM_ERR_NULL);
  EXPECT(fm_tileinfo_layout_query(NULL, &lay), FM_ERR_NULL);
  EXPECT(fm_bwd_workspace_bytes(&ok, NULL), FM_ERR_NULL);
  EXPECT(fm_bwd_cache_bytes(&ok, 5, NULL), FM_ERR_NULL);
  EXPECT(fm_tileinfo_layout_query(&ok, &lay), FM_OK);
  EXPECT(fm_set_kernel_events(NULL, NULL, NULL, NULL), FM_OK);

  /* the entry points that enqueue work: each call fails validation */
  fm_problem bad = prob(2, 4, 3, 1000, 900, 128, 0.1f);      /* mask_heads neither 1 nor heads */
  fm_problem neg = prob(-1, 4, 1, 1000, 900, 128, 0.1f);
  float* lse = (float*)FAKE2;
  EXPECT(fm_tile_bounds(&bad, (const int32_t*)FAKE, FAKE, NULL), FM_ERR_UNSUPPORTED);
  EXPECT(fm_tile_bounds(&neg, (const int32_t*)FAKE, FAKE, NULL), FM_ERR_SHAPE);
  EXPECT(fm_tile_bounds(&ok, NULL, FAKE, NULL), FM_ERR_NULL);
  EXPECT(fm_tile_bounds(&ok, (const int32_t*)FAKE, NULL, NULL), FM_ERR_NULL);
  EXPECT(fm_tile_bounds(&ok, (const int32_t*)MISAL, FAKE, NULL), FM_ERR_ALIGN);
  EXPECT(fm_tile_bounds(&ok, (const int32_t*)FAKE, MISAL, NULL), FM_ERR_ALIGN);
  EXPECT(fm_attn_fwd(&bad, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL), FM_ERR_UNSUPPORTED);
  EXPECT(fm_attn_fwd(&ok, NULL, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL), FM_ERR_NULL);
  EXPECT(fm_attn_fwd(&ok, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE, NULL, NULL), FM_ERR_NULL);
  EXPECT(fm_attn_fwd(&ok, FAKE, MISAL, FAKE, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL), FM_ERR_ALIGN);
  EXPECT(fm_attn_fwd(&ok, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, FAKE, (float*)MISAL, NULL), FM_ERR_ALIGN);
  /* an empty problem enqueues nothing and succeeds without tensors */
  fm_problem empty = prob(0, 4, 1, 1000, 900, 128, 0.1f);
  EXPECT(fm_attn_fwd(&empty, NULL, NULL, NULL, NULL, FAKE, NULL, NULL, NULL), FM_OK);
  const float descale[3] = {1.f, 1.f, 1.f};
  const float bad_descale[3] = {1.f, NAN, 1.f};
  EXPECT(fm_attn_fwd_fp8(&ok, FAKE, FAKE, FAKE, NULL, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL), FM_ERR_NULL);
  EXPECT(fm_attn_fwd_fp8(&ok, FAKE, FAKE, FAKE, bad_descale, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL),
         FM_ERR_UNSUPPORTED);
  fm_problem d64 = prob(2, 4, 1, 1000, 900, 64, 0.1f);
  EXPECT(fm_attn_fwd_fp8(&d64, FAKE, FAKE, FAKE, descale, (const int32_t*)FAKE, FAKE, FAKE, lse, NULL),
         FM_ERR_UNSUPPORTED);
  EXPECT(fm_attn_bwd(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                     1 << 20, NULL), FM_ERR_UNSUPPORTED);
  EXPECT(fm_attn_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE, NULL,
                     1 << 20, NULL), FM_ERR_NULL);
  /* a workspace smaller than Delta (2 x 4 x 1000 fp32) */
  EXPECT(fm_attn_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                     NULL), FM_ERR_SHAPE);
  EXPECT(fm_attn_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                     31996, NULL), FM_ERR_SHAPE);
  EXPECT(fm_attn_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, MISAL, FAKE, FAKE,
                     1 << 20, NULL), FM_ERR_ALIGN);
  EXPECT(fm_attn_bwd_noalloc(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE,
                             NULL), FM_ERR_UNSUPPORTED);
  EXPECT(fm_attn_bwd_noalloc(&ok, FAKE, FAKE, NULL, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE, FAKE,
                             NULL), FM_ERR_NULL);
  fm_problem huge = prob(64, 64, 1, 131072, 131072, 128, 0.1f);   /* Delta beyond the static scratch */
  EXPECT(fm_attn_bwd_noalloc(&huge, FAKE, FAKE, FAKE, FAKE, FAKE, lse, (const int32_t*)FAKE, FAKE, FAKE, FAKE,
                             FAKE, NULL), FM_ERR_SCRATCH);

  /* localisation: chunk lists that are empty, too long, unordered,
   * overlapping, negative or beyond the supported length */
  int32_t start[70], len[70];
  for (int c = 0; c < 70; ++c) { start[c] = 1000 * c; len[c] = 100; }
  const int32_t* gb = (const int32_t*)FAKE;
  int32_t* lb = (int32_t*)FAKE2;
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 0, start, len, lb, NULL), FM_ERR_SHAPE);
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 65, start, len, lb, NULL), FM_ERR_SHAPE);
  EXPECT(fm_localize_bounds(-1, 1, 512, gb, 2, start, len, lb, NULL), FM_ERR_SHAPE);
  EXPECT(fm_localize_bounds(1, 0, 512, gb, 2, start, len, lb, NULL), FM_ERR_SHAPE);
  EXPECT(fm_localize_bounds(1, 1, -4, gb, 2, start, len, lb, NULL), FM_ERR_SHAPE);
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, NULL, len, lb, NULL), FM_ERR_NULL);
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, start, NULL, lb, NULL), FM_ERR_NULL);
  EXPECT(fm_localize_bounds(1, 1, 512, NULL, 2, start, len, lb, NULL), FM_ERR_NULL);
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, start, len, NULL, NULL), FM_ERR_NULL);
  EXPECT(fm_localize_bounds(1, 1, 512, (const int32_t*)MISAL, 2, start, len, lb, NULL), FM_ERR_ALIGN);
  int32_t s2[2] = {500, 100}, l2[2] = {10, 10};        /* decreasing */
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, s2, l2, lb, NULL), FM_ERR_SHAPE);
  int32_t s3[2] = {100, 105}, l3[2] = {10, 10};        /* overlapping */
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, s3, l3, lb, NULL), FM_ERR_SHAPE);
  int32_t s4[2] = {0, 100}, l4[2] = {-1, 10};          /* negative length */
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, s4, l4, lb, NULL), FM_ERR_SHAPE);
  int32_t s5[2] = {0, INT32_MAX - 5}, l5[2] = {10, 10}; /* end past int32 */
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, s5, l5, lb, NULL), FM_ERR_SHAPE);
  int32_t s6[2] = {0, 10}, l6[2] = {3000000, 3000000};  /* more local rows than one problem holds */
  EXPECT(fm_localize_bounds(1, 1, 512, gb, 2, s6, l6, lb, NULL), FM_ERR_SHAPE);

  printf("%ld problem shapes, %d failures\n", checked, failures);
  return failures ? 1 : 0;
}
