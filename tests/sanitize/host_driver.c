/* Host-code exercise for the sanitizer test: every configuration check, level progression,
 * parameter layout, workspace plan and argument check of the C ABI, run under
 * AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.  No call reaches a kernel
 * launch: sizes are queried, and every compute entry point is handed arguments it must
 * reject before launching.  Exit status 0 when every return code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hashenc.h"
#include "hashenc_diag.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static hashenc_config base(int d, int L, int F, int kind, uint32_t T) {
  hashenc_config c;
  memset(&c, 0, sizeof c);
  c.d = d;
  c.n_levels = L;
  c.n_features = F;
  c.kind = kind;
  c.d2_mode = kind == HASHENC_DLINEAR ? 0 : HASHENC_D2_DIAG;
  c.n_min = 16;
  c.n_max = 1024;
  for (int k = 0; k < 5; ++k) c.table_size[k] = T;
  c.rbf_eps = 1.0;
  c.rbf_rings = 3;
  return c;
}

static void exercise(const hashenc_config* c) {
  hashenc* h = NULL;
  EXPECT(hashenc_create(c, &h) == HASHENC_OK);
  if (!h) return;
  int64_t np = 0;
  int32_t width = 0, res[HASHENC_MAX_LEVELS];
  EXPECT(hashenc_info(h, &np, &width, res) == HASHENC_OK);
  const int ntab = c->kind == HASHENC_HERMITE ? c->d + 1 : 1;
  int64_t next = 0;
  for (int k = 0; k < ntab; ++k)
    for (int l = 0; l < c->n_levels; ++l) {
      int64_t off = -1, rows = -1;
      int32_t w = -1, dense = -1;
      EXPECT(hashenc_param_layout(h, k, l, &off, &rows, &w, &dense) == HASHENC_OK);
      EXPECT(off == next);
      next = off + rows * w;
    }
  EXPECT(next == np);
  EXPECT(hashenc_param_layout(h, ntab, 0, NULL, NULL, NULL, NULL) == HASHENC_EINVAL);
  const int64_t sizes[] = {0, 1, 63, 1024, 1 << 20, (1 << 21) + 777, (int64_t)1 << 26};
  for (unsigned i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) {
    size_t b = 0;
    EXPECT(hashenc_forward_workspace_size(h, sizes[i], &b) == HASHENC_OK);
    EXPECT(hashenc_backward_workspace_size(h, sizes[i], &b) == HASHENC_OK);
  }
  size_t b = 0;
  EXPECT(hashenc_backward_workspace_size(h, -1, &b) == HASHENC_EINVAL);
  hashenc_mlp m = {c->n_levels * c->n_features, 64, 2, 1, 30.0f, 0};
  const int rc_res = hashenc_residual_workspace_size(h, &m, 1 << 20, &b);
  const int rc_fd = hashenc_fd_residual_workspace_size(h, &m, 1 << 20, &b);
  if (c->kind == HASHENC_HERMITE && c->d < 4 && m.in <= 64) EXPECT(rc_res == HASHENC_OK);
  else EXPECT(rc_res != HASHENC_OK);
  if (c->kind == HASHENC_DLINEAR && m.in <= 64) EXPECT(rc_fd == HASHENC_OK);
  else EXPECT(rc_fd != HASHENC_OK);
  /* derived handles */
  for (int a = 1; a <= c->n_levels; a += c->n_levels > 2 ? c->n_levels / 2 : 1) {
    hashenc* dh = NULL;
    EXPECT(hashenc_derive_active(h, a, &dh) == HASHENC_OK);
    int32_t got = 0;
    EXPECT(hashenc_active_levels(dh, &got) == HASHENC_OK && got == a);
    EXPECT(hashenc_backward_workspace_size(dh, 1 << 20, &b) == HASHENC_OK);
    EXPECT(hashenc_forward_workspace_size(dh, 1 << 20, &b) == HASHENC_OK);
    hashenc_destroy(dh);
  }
  hashenc* dh = NULL;
  EXPECT(hashenc_derive_active(h, 0, &dh) == HASHENC_EINVAL);
  EXPECT(hashenc_derive_active(h, c->n_levels + 1, &dh) == HASHENC_EINVAL);
  /* compute entry points with arguments rejected before any launch */
  float* a16 = (float*)(uintptr_t)0x10000;
  float* mis = (float*)(uintptr_t)0x10004;
  EXPECT(hashenc_forward(h, -1, a16, a16, a16, NULL, NULL, NULL) == HASHENC_EINVAL);
  EXPECT(hashenc_forward(h, 5, NULL, a16, a16, NULL, NULL, NULL) == HASHENC_EINVAL);
  EXPECT(hashenc_forward(h, 5, a16, mis, a16, NULL, NULL, NULL) == HASHENC_EALIGN);
  EXPECT(hashenc_backward(h, 5, a16, a16, NULL, NULL, NULL, NULL) == HASHENC_EINVAL);
  EXPECT(hashenc_backward(h, 5, a16, a16, NULL, NULL, mis, NULL) == HASHENC_EALIGN);
  EXPECT(hashenc_forward_ws(h, 5, a16, a16, a16, NULL, NULL, NULL, 0, NULL) != HASHENC_OK);
  EXPECT(hashenc_backward_ws(h, 5, NULL, a16, NULL, NULL, a16, a16, 1 << 30, NULL) != HASHENC_OK);
  int32_t* rows = (int32_t*)(uintptr_t)0x20000;
  EXPECT(hashenc_debug_indices(h, 5, a16, ntab, rows, NULL) == HASHENC_EINVAL);
  EXPECT(hashenc_residual(h, &m, 0, a16, a16, a16, NULL, a16, NULL, NULL, a16, 0, NULL) != HASHENC_OK);
  hashenc_destroy(h);
}

int main(void) {
  const int kinds[] = {HASHENC_DLINEAR, HASHENC_HERMITE, HASHENC_RBF};
  for (int ki = 0; ki < 3; ++ki)
    for (int d = 2; d <= 4; ++d) {
      if (d == 4 && kinds[ki] != HASHENC_HERMITE) continue;
      const int Ls[] = {1, 4, 16, 32};
      const int Fs[] = {1, 2, 4, 8};
      const uint32_t Ts[] = {1u, 4096u, 1000003u, 1u << 19, 1u << 24};
      for (int li = 0; li < 4; ++li)
        for (int fi = 0; fi < 4; ++fi)
          for (int ti = 0; ti < 5; ++ti) {
            hashenc_config c = base(d, Ls[li], Fs[fi], kinds[ki], Ts[ti]);
            if (d == 4) c.n_max = 64;
            if (kinds[ki] == HASHENC_RBF) c.n_max = 512;
            exercise(&c);
          }
    }
  /* unequal order-table sizes and explicit resolutions */
  hashenc_config c = base(3, 16, 2, HASHENC_HERMITE, 1u << 14);
  c.table_size[3] = 1u << 10;
  exercise(&c);
  const int32_t res[4] = {3, 7, 1 << 20, 5};
  c = base(2, 4, 2, HASHENC_DLINEAR, 1u << 12);
  c.resolutions = res;
  exercise(&c);
  /* configurations that must be rejected */
  hashenc* h = NULL;
  c = base(5, 4, 2, HASHENC_DLINEAR, 64);
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  c = base(3, 33, 2, HASHENC_DLINEAR, 64);
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  c = base(3, 4, 3, HASHENC_DLINEAR, 64);
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  c = base(3, 4, 2, HASHENC_DLINEAR, 0);
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  c = base(3, 4, 2, HASHENC_DLINEAR, 64);
  c.growth = 1e9;
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  c = base(3, 4, 2, HASHENC_RBF, 64);
  c.rbf_rings = 9;
  EXPECT(hashenc_create(&c, &h) == HASHENC_EINVAL);
  EXPECT(hashenc_create(NULL, &h) == HASHENC_EINVAL);
  EXPECT(strlen(hashenc_last_error()) > 0);
  int32_t a = 0;
  EXPECT(hashenc_c2f_active_levels(16, 2, 1000, 100, &a) == HASHENC_OK && a == 12);
  EXPECT(hashenc_c2f_active_levels(16, 0, 1000, 100, &a) == HASHENC_EINVAL);
  EXPECT(hashenc_diag_copy(NULL, NULL, 8, NULL) == HASHENC_EINVAL);
  hashenc_destroy(NULL);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host driver: all expectations met\n");
  return 0;
}
