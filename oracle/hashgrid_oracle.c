/*
 * Plain CPU oracle for the multiresolution hash-grid encoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the package smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * HIP library and is written to be checked against the pages by eye: no
 * blocking, no fusion, fp64 arithmetic after the fp32 position stage.
 *
 * Sources (each function cites the passage it follows):
 *   [INGP-explainer]  "SIGGRAPH 2022 | InstantNGP and multiresolution hash encoding"
 *                     (nxrte.com), section "InstantNGP 与多分辨率哈希编码流程与原理".
 *   [INGP-news]       "NVIDIA cuts NeRF training from 5 hours to 5 seconds"
 *                     (antipu.com.cn), the adaptivity / efficiency paragraphs and
 *                     the paragraph under Figure 3 (geometric progression of levels).
 *   [DInf-Grid]       "DInf-Grid: a neural differential equation solver with
 *                     differentiable feature grids" summary (shdxiang-github-io), sections
 *                     可微的径向基函数插值 (normalised Gaussian RBF weights, precomputed
 *                     k-ring neighbourhoods) and 多分辨率特征网格 (concatenated levels).
 *   [HNGP]            "Hermite-NGP: Gradient-Augmented Hash Encoding for Learning
 *                     PDEs" reading notes (m0rtzz.github.io), section 方法详解,
 *                     key design 1 (reconstruction equation, 1D basis), key
 *                     design 2 (basis derivatives, SIREN chain rule) and key
 *                     design 3 (coarse-to-fine level activation); the 现有痛点
 *                     paragraph (INGP-FD: Laplacian by central differences over
 *                     2d+1 forward passes); section 损失函数 / 训练策略 (omega_0 = 30).
 *
 * Readings taken where the pages are silent or garbled (the formula bodies for
 * the level progression and the spatial hash did not survive extraction):
 *   - level resolution N_l = floor(N_min * b^l + 1e-6), b = (N_max/N_min)^(1/(L-1))
 *     unless b is given;
 *   - hash = XOR over axes of (uint32(v_i) * pi_i mod 2^32), then mod T, with
 *     pi = (1, 2654435761, 805459861) and, for the 4D space-time Hermite grid, the
 *     fourth prime 3674653429 of the same customary list;
 *   - dense level (1:1 map) iff (N_l+1)^d <= T, index sum_i v_i (N_l+1)^i;
 *   - vertices at v / N_l, p = fl32(x * N_l) (one rounded multiply),
 *     base = min(floor(p), N_l - 1), t = p - base;
 *   - rows stored per level = min(T, (N_l+1)^d);
 *   - Hermite: d+1 tables bucketed by derivative order |alpha|, row = the
 *     C(d,k) slots of order k in lexicographic axis order, times F features;
 *   - near-corner basis is the reflection of the far-corner basis printed on
 *     the Hermite-NGP page;
 *   - colliding rows receive the sum of their contributions;
 *   - Gaussian RBF (kind 2): distances in units of the level's grid spacing
 *     (r = |p - v| with p = fl32(x N_l)); the k-ring neighbourhood of a point is the box
 *     of (2k)^d vertices base_i - k + 1 .. base_i + k around its cell, clipped to the
 *     grid; weights phi(r) / sum phi over that box, phi(r) = exp(-(eps r)^2); storage as
 *     for d-linear (one table per level, dense 1:1 where the vertices fit);
 *   - coarse-to-fine activation: L_active counts the active levels (levels
 *     l < L_active); an inactive level contributes zeros to the encoding and
 *     receives no gradient, and the encoding keeps its full L*F width.
 *
 * Parity of the hash against any third-party implementation is unpinned (the
 * pages print no example value); it is pinned against its own definition's
 * special cases and invariants in the test-suite.
 *
 * Working precision.  Everything after the fp32 position stage is computed in
 * `real`: fp64 in the oracle proper.  A second build with -DORC_FP32 reruns the
 * same per-point arithmetic in fp32 (float operations, float sin / cos / exp /
 * pow), which measures the fp32 rounding floor of each output; the buffers at the
 * interface stay fp64 and sums over points (gradients, loss) stay fp64 in both
 * builds, so the floor is that of the per-point arithmetic alone.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORC_FP32
typedef float real;
#define R_SIN sinf
#define R_COS cosf
#define R_EXP expf
#define R_POW powf
#else
typedef double real;
#define R_SIN sin
#define R_COS cos
#define R_EXP exp
#define R_POW pow
#endif

#define ORC_MAX_LEVELS 32
#define ORC_MAX_D 4
#define ORC_MAX_F 8

typedef struct {
  int32_t d;          /* spatial dimension, 1..3 */
  int32_t L;          /* number of levels */
  int32_t F;          /* features per slot */
  int32_t kind;       /* 0 = d-linear, 1 = cubic Hermite, 2 = Gaussian RBF */
  int32_t d2_mode;    /* Hermite second-order output: 1 = Laplacian [n,L*F], 2 = diagonal [n,d,L*F] */
  uint32_t T[ORC_MAX_D + 1]; /* rows of table k (derivative order k); d-linear uses T[0] */
  int32_t N[ORC_MAX_LEVELS]; /* level resolutions */
  int32_t active;     /* levels l < active are active [HNGP key design 3]; 0 = all L */
  int32_t rings;      /* Gaussian RBF: neighbourhood rings k (1..4) */
  double eps;         /* Gaussian RBF: shape parameter epsilon (> 0) */
} orc_cfg;

#define ORC_MAX_RBF_VERTS 512 /* (2k)^d for k <= 4, d <= 3 */

/* Number of active levels of a configuration (0 in the field means all of them). */
static int active_levels(const orc_cfg* c) {
  return (c->active > 0 && c->active < c->L) ? c->active : c->L;
}

/* Coarse-to-fine schedule [HNGP key design 3]: at step t the first L0 + floor(t / tau)
 * levels are active, at most L.  Returns -1 on L < 1, L0 < 1, t < 0 or tau < 1. */
int32_t orc_c2f_active(int32_t L, int32_t L0, int64_t t, int64_t tau) {
  if (L < 1 || L0 < 1 || t < 0 || tau < 1) return -1;
  const int64_t a = (int64_t)L0 + t / tau;
  return a < (int64_t)L ? (int32_t)a : L;
}

/* one prime per axis; the first is 1 so that the x axis maps to itself */
static const uint32_t ORC_PRIMES[4] = {1u, 2654435761u, 805459861u, 3674653429u};

/* ---- levels: geometric progression between N_min and N_max [INGP-news, Fig. 3 paragraph] ---- */
int orc_levels(int32_t L, int32_t n_min, int32_t n_max, double growth, int32_t* out) {
  if (L < 1 || L > ORC_MAX_LEVELS || n_min < 1) return -1;
  double b = growth;
  if (!(b > 0.0)) {
    if (L == 1) b = 1.0;
    else b = exp((log((double)n_max) - log((double)n_min)) / (double)(L - 1));
  }
  for (int l = 0; l < L; ++l) {
    double v = floor((double)n_min * pow(b, (double)l) + 1e-6);
    out[l] = (int32_t)v;
  }
  return 0;
}

static int64_t ipow64(int64_t base, int e) {
  int64_t r = 1;
  for (int i = 0; i < e; ++i) r *= base;
  return r;
}

static int64_t binom(int n, int k) {
  int64_t r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

static int popcount_bits(int a) {
  int c = 0;
  while (a) { c += a & 1; a >>= 1; }
  return c;
}

/* Rank of the derivative multi-index alpha (bitmask over axes) among the alphas of the
 * same order, in lexicographic order of their sorted axis tuples:
 * order 1: x, y, z;  order 2: xy, xz, yz;  order 3: xyz.   [HNGP key design 1: the
 * 2^d mixed partials bucketed by derivative order] */
static int slot_of_alpha(int d, int alpha) {
  int k = popcount_bits(alpha);
  /* enumerate all masks with k bits in lexicographic order of their axis tuples */
  int rank = 0;
  int axes_target[ORC_MAX_D];
  int na = 0;
  for (int i = 0; i < d; ++i) if (alpha & (1 << i)) axes_target[na++] = i;
  /* count combinations of k axes that sort before axes_target */
  int idx[ORC_MAX_D];
  for (int i = 0; i < k; ++i) idx[i] = i;
  for (;;) {
    int same = 1;
    for (int i = 0; i < k; ++i) if (idx[i] != axes_target[i]) { same = 0; break; }
    if (same) return rank;
    ++rank;
    /* next combination */
    int i = k - 1;
    while (i >= 0 && idx[i] == d - k + i) --i;
    if (i < 0) return -1;
    ++idx[i];
    for (int j = i + 1; j < k; ++j) idx[j] = idx[j - 1] + 1;
  }
}

static int n_tables(const orc_cfg* c) { return c->kind == 1 ? c->d + 1 : 1; }

static int64_t row_width(const orc_cfg* c, int k) {
  return c->kind == 1 ? binom(c->d, k) * c->F : (int64_t)c->F;
}

/* Vertices per level (N_l+1)^d, as a double to survive any size. */
static double level_vertices(const orc_cfg* c, int l) {
  return pow((double)c->N[l] + 1.0, (double)c->d);
}

static int is_dense(const orc_cfg* c, int k, int l) {
  /* coarse level with no more vertices than the table has rows: 1:1 map
   * [INGP-explainer, collision paragraph; INGP-news, adaptivity paragraph] */
  return level_vertices(c, l) <= (double)c->T[k];
}

static int64_t level_rows(const orc_cfg* c, int k, int l) {
  return is_dense(c, k, l) ? ipow64((int64_t)c->N[l] + 1, c->d) : (int64_t)c->T[k];
}

/* Parameter layout: table k, then level l, then row, then [slot][feature].
 * Returns the total number of floats; fills per-(k,l) arrays indexed k*L+l. */
int64_t orc_layout(const orc_cfg* c, int64_t* offsets, int64_t* rows, int32_t* width,
                   int32_t* dense) {
  int64_t off = 0;
  for (int k = 0; k < n_tables(c); ++k) {
    for (int l = 0; l < c->L; ++l) {
      int64_t r = level_rows(c, k, l);
      int64_t w = row_width(c, k);
      if (offsets) offsets[k * c->L + l] = off;
      if (rows) rows[k * c->L + l] = r;
      if (width) width[k * c->L + l] = (int32_t)w;
      if (dense) dense[k * c->L + l] = is_dense(c, k, l);
      off += r * w;
    }
  }
  return off;
}

/* Spatial hash of an integer vertex [INGP-explainer, 空间哈希函数 (formula lost; reading
 * stated in the file header)].  Products wrap mod 2^32, XOR combines the axes. */
uint32_t orc_hash(int d, const uint32_t* v) {
  uint32_t h = 0;
  for (int i = 0; i < d; ++i) h ^= (uint32_t)(v[i] * ORC_PRIMES[i]);
  return h;
}

/* Row index of vertex v in table k at level l. */
static int64_t vertex_row(const orc_cfg* c, int k, int l, const uint32_t* v) {
  if (is_dense(c, k, l)) {
    int64_t idx = 0, stride = 1;
    for (int i = 0; i < c->d; ++i) {
      idx += (int64_t)v[i] * stride;
      stride *= (int64_t)c->N[l] + 1;
    }
    return idx;
  }
  return (int64_t)(orc_hash(c->d, v) % c->T[k]);
}

/* Cell of point x at level l [INGP-explainer, step 1: the 2^d grid vertices around x].
 * Position stage in IEEE fp32: p = x*N_l rounded once, base = floor, t = p - base. */
static void locate(const orc_cfg* c, int l, const float* x, uint32_t* base, real* t) {
  volatile float nl = (float)c->N[l];
  for (int i = 0; i < c->d; ++i) {
    float xi = x[i];
    if (!(xi >= 0.0f)) xi = 0.0f; /* also maps NaN to 0 */
    if (xi > 1.0f) xi = 1.0f;
    volatile float p = xi * nl; /* volatile: one rounded fp32 product, never fused */
    float fl = floorf(p);
    int32_t b = (int32_t)fl;
    if (b > c->N[l] - 1) b = c->N[l] - 1;
    float tf = p - (float)b; /* exact (Sterbenz) */
    base[i] = (uint32_t)b;
    t[i] = (real)tf;
  }
}

/* Corner indices of every point, every level, table k: out[n][L][2^d], corner bit i = axis i.
 * Debug/parity export for the bit-exact comparison of the lookup stage. */
void orc_indices(const orc_cfg* c, int64_t n, const float* x, int k, int32_t* out) {
  const int nc = 1 << c->d;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < n; ++p) {
    for (int l = 0; l < c->L; ++l) {
      uint32_t base[ORC_MAX_D];
      real t[ORC_MAX_D];
      locate(c, l, x + p * c->d, base, t);
      for (int cc = 0; cc < nc; ++cc) {
        uint32_t v[ORC_MAX_D];
        for (int i = 0; i < c->d; ++i) v[i] = base[i] + (uint32_t)((cc >> i) & 1);
        out[(p * c->L + l) * nc + cc] = (int32_t)vertex_row(c, k, l, v);
      }
    }
  }
}

/* ---- cubic Hermite 1D factors [HNGP key design 1 (basis), key design 2 (derivatives)] ----
 * corner bit cb (0 = near vertex at t=0, 1 = far vertex at t=1), derivative bit a.
 * Far corner: value basis 3t^2-2t^3, derivative basis t^3-t^2 (printed on the page);
 * near corner: their reflections t -> 1-t (derivative basis changes sign). */
static void hermite_1d(int cb, int a, real t, real* B, real* dB, real* d2B) {
  if (!a && !cb) { *B = 1 - 3 * t * t + 2 * t * t * t; *dB = -6 * t + 6 * t * t; *d2B = -6 + 12 * t; }
  else if (!a && cb) { *B = 3 * t * t - 2 * t * t * t; *dB = 6 * t - 6 * t * t; *d2B = 6 - 12 * t; }
  else if (a && !cb) { *B = t - 2 * t * t + t * t * t; *dB = 1 - 4 * t + 3 * t * t; *d2B = -4 + 6 * t; }
  else { *B = -t * t + t * t * t; *dB = -2 * t + 3 * t * t; *d2B = -2 + 6 * t; }
}

/* Per-(corner, alpha) weights of one point at one level: the coefficient that multiplies
 * theta^(alpha) at that corner in gamma (w0), in d gamma/dx_i (w1[i]) and in
 * d^2 gamma/dx_i^2 (w2[i]).  Hermite: Delta x^{|alpha|} H^(alpha)(t) with the chain rule
 * d/dx = N_l d/dt; d-linear: prod_i (c_i ? t_i : 1-t_i), alpha = 0 only. */
static void corner_weights(const orc_cfg* c, int l, int cc, int alpha, const real* t,
                           real* w0, real* w1, real* w2) {
  const real Nl = (real)c->N[l];
  if (c->kind == 0) {
    real w = 1.0;
    for (int i = 0; i < c->d; ++i) w *= ((cc >> i) & 1) ? t[i] : 1.0 - t[i];
    *w0 = w;
    return;
  }
  real B[ORC_MAX_D], dB[ORC_MAX_D], d2B[ORC_MAX_D];
  for (int i = 0; i < c->d; ++i)
    hermite_1d((cc >> i) & 1, (alpha >> i) & 1, t[i], &B[i], &dB[i], &d2B[i]);
  real s = R_POW(Nl, -(real)popcount_bits(alpha)); /* Delta x_l^{|alpha|} */
  real prod = 1.0;
  for (int i = 0; i < c->d; ++i) prod *= B[i];
  *w0 = s * prod;
  for (int i = 0; i < c->d; ++i) {
    real others = 1.0;
    for (int k = 0; k < c->d; ++k) if (k != i) others *= B[k];
    w1[i] = s * Nl * dB[i] * others;
    w2[i] = s * Nl * Nl * d2B[i] * others;
  }
}

/* Gaussian-RBF weights of one point at one level [DInf-Grid, 可微的径向基函数插值]: for
 * every vertex v of the point's k-ring box (clipped to the grid) its row, and the weight
 * that multiplies its coefficient in gamma (w), in d gamma / dx_i (w1[.][i]) and in
 * d^2 gamma / dx_i^2 (w2[.][i]):
 *     phi_v = exp(-eps^2 |p - v|^2),  S = sum_v phi_v,  w_v = phi_v / S,
 * differentiated by the quotient rule, with d/dx_i = N_l d/dp_i:
 *     dphi/dp_i = -2 eps^2 (p_i - v_i) phi,  d^2phi/dp_i^2 = (4 eps^4 (p_i - v_i)^2 - 2 eps^2) phi,
 *     dw = (dphi - w dS) / S,  d^2w = (d^2phi - 2 dw dS - w d^2S) / S.
 * Returns the number of vertices. */
static int rbf_weights(const orc_cfg* c, int l, const float* x, int64_t* rows, real* w,
                       real (*w1)[ORC_MAX_D], real (*w2)[ORC_MAX_D]) {
  const int d = c->d, k = c->rings;
  const real e2 = (real)(c->eps * c->eps), N = (real)c->N[l];
  uint32_t base[ORC_MAX_D];
  real t[ORC_MAX_D];
  locate(c, l, x, base, t);
  real p[ORC_MAX_D];
  for (int i = 0; i < d; ++i) p[i] = (real)base[i] + t[i]; /* = fl32(x N), exactly */
  real phi[ORC_MAX_RBF_VERTS], d1[ORC_MAX_RBF_VERTS][ORC_MAX_D], d2[ORC_MAX_RBF_VERTS][ORC_MAX_D];
  int nv = 0;
  const int side = 2 * k;
  int total = 1;
  for (int i = 0; i < d; ++i) total *= side;
  if (total > ORC_MAX_RBF_VERTS) return 0; /* (2k)^d beyond the supported box (d <= 3) */
  for (int m = 0; m < total; ++m) {
    int64_t v[ORC_MAX_D];
    int inside = 1, mm = m;
    for (int i = 0; i < d; ++i) {
      v[i] = (int64_t)base[i] - k + 1 + mm % side;
      mm /= side;
      if (v[i] < 0 || v[i] > (int64_t)c->N[l]) inside = 0;
    }
    if (!inside) continue;
    real r2 = 0.0;
    for (int i = 0; i < d; ++i) r2 += (p[i] - (real)v[i]) * (p[i] - (real)v[i]);
    phi[nv] = R_EXP(-e2 * r2);
    for (int i = 0; i < d; ++i) {
      const real del = p[i] - (real)v[i];
      d1[nv][i] = -2.0 * e2 * del * phi[nv] * N;
      d2[nv][i] = (4.0 * e2 * e2 * del * del - 2.0 * e2) * phi[nv] * N * N;
    }
    uint32_t vu[ORC_MAX_D];
    for (int i = 0; i < d; ++i) vu[i] = (uint32_t)v[i];
    rows[nv] = vertex_row(c, 0, l, vu);
    ++nv;
  }
  real S = 0.0, S1[ORC_MAX_D] = {0}, S2[ORC_MAX_D] = {0};
  for (int q = 0; q < nv; ++q) {
    S += phi[q];
    for (int i = 0; i < d; ++i) { S1[i] += d1[q][i]; S2[i] += d2[q][i]; }
  }
  for (int q = 0; q < nv; ++q) {
    w[q] = phi[q] / S;
    for (int i = 0; i < d; ++i) {
      w1[q][i] = (d1[q][i] - w[q] * S1[i]) / S;
      w2[q][i] = (d2[q][i] - 2.0 * w1[q][i] * S1[i] - w[q] * S2[i]) / S;
    }
  }
  return nv;
}

/* Forward encoding [INGP-explainer steps 1-4; HNGP key design 1].
 * gamma[n][L*F]; Hermite only: dgamma[n][d][L*F], d2gamma per d2_mode
 * (Laplacian [n][L*F] or diagonal [n][d][L*F]).  Any output may be NULL.
 * Columns of inactive levels (l >= active) are zero. */
void orc_forward(const orc_cfg* c, int64_t n, const float* x, const double* params,
                 double* gamma, double* dgamma, double* d2gamma) {
  int64_t offs[(ORC_MAX_D + 1) * ORC_MAX_LEVELS];
  int32_t wid[(ORC_MAX_D + 1) * ORC_MAX_LEVELS];
  orc_layout(c, offs, NULL, wid, NULL);
  const int nc = 1 << c->d;
  const int na = c->kind == 1 ? nc : 1;
  const int LF = c->L * c->F;
  const int d = c->d;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < n; ++p) {
    for (int l = 0; l < c->L; ++l) {
      uint32_t base[ORC_MAX_D];
      real t[ORC_MAX_D];
      locate(c, l, x + p * d, base, t);
      real g0[ORC_MAX_F] = {0}, g1[ORC_MAX_F][ORC_MAX_D] = {{0}}, g2[ORC_MAX_F][ORC_MAX_D] = {{0}};
      if (c->kind == 2 && l < active_levels(c)) {
        /* Gaussian RBF: sum over the k-ring box [DInf-Grid] */
        int64_t rows[ORC_MAX_RBF_VERTS];
        real w[ORC_MAX_RBF_VERTS], w1[ORC_MAX_RBF_VERTS][ORC_MAX_D], w2[ORC_MAX_RBF_VERTS][ORC_MAX_D];
        const int nv = rbf_weights(c, l, x + p * d, rows, w, w1, w2);
        for (int q = 0; q < nv; ++q) {
          const double* th = params + offs[l] + rows[q] * wid[l];
          for (int f = 0; f < c->F; ++f) {
            const real v = (real)th[f];
            g0[f] += w[q] * v;
            for (int i = 0; i < d; ++i) {
              g1[f][i] += w1[q][i] * v;
              g2[f][i] += w2[q][i] * v;
            }
          }
        }
      }
      /* an inactive level keeps its columns at zero [HNGP key design 3] */
      const int ncorner = (c->kind != 2 && l < active_levels(c)) ? nc : 0;
      for (int cc = 0; cc < ncorner; ++cc) {
        uint32_t v[ORC_MAX_D];
        for (int i = 0; i < d; ++i) v[i] = base[i] + (uint32_t)((cc >> i) & 1);
        for (int alpha = 0; alpha < na; ++alpha) {
          const int k = popcount_bits(alpha);
          const int64_t row = vertex_row(c, k, l, v);
          const int slot = c->kind == 1 ? slot_of_alpha(d, alpha) : 0;
          const double* th = params + offs[k * c->L + l] + row * wid[k * c->L + l] + (int64_t)slot * c->F;
          real w0, w1[ORC_MAX_D], w2[ORC_MAX_D];
          corner_weights(c, l, cc, alpha, t, &w0, w1, w2);
          for (int f = 0; f < c->F; ++f) {
            const real v = (real)th[f];
            g0[f] += w0 * v;
            if (c->kind == 1)
              for (int i = 0; i < d; ++i) {
                g1[f][i] += w1[i] * v;
                g2[f][i] += w2[i] * v;
              }
          }
        }
      }
      for (int f = 0; f < c->F; ++f) {
        const int col = l * c->F + f;
        if (gamma) gamma[p * LF + col] = g0[f];
        if (c->kind != 0) {
          if (dgamma) for (int i = 0; i < d; ++i) dgamma[(p * d + i) * LF + col] = g1[f][i];
          if (d2gamma) {
            if (c->d2_mode == 2) {
              for (int i = 0; i < d; ++i) d2gamma[(p * d + i) * LF + col] = g2[f][i];
            } else {
              real lap = 0.0;
              for (int i = 0; i < d; ++i) lap += g2[f][i];
              d2gamma[p * LF + col] = lap;
            }
          }
        }
      }
    }
  }
}

/* Backward into the tables [INGP-news, adaptivity paragraph: gradients of colliding
 * vertices combine; here they sum, the exact gradient of the linear map theta -> gamma].
 * Upstream in fp64 (any may be NULL = zero); g_d2 is [n][L*F] in Laplacian mode, else
 * [n][d][L*F].  grad (fp64, same layout as params) is ACCUMULATED; inactive levels
 * (l >= active) are left untouched.  Deterministic: each
 * (table, level) slice is owned by one thread, points in ascending order. */
void orc_backward_f64(const orc_cfg* c, int64_t n, const float* x, const double* g_gamma,
                      const double* g_dgamma, const double* g_d2, double* grad) {
  int64_t offs[(ORC_MAX_D + 1) * ORC_MAX_LEVELS];
  int32_t wid[(ORC_MAX_D + 1) * ORC_MAX_LEVELS];
  orc_layout(c, offs, NULL, wid, NULL);
  const int nc = 1 << c->d;
  const int na = c->kind == 1 ? nc : 1;
  const int LF = c->L * c->F;
  const int d = c->d;
  const int ntab = n_tables(c);
#pragma omp parallel for schedule(dynamic, 1)
  for (int task = 0; task < ntab * c->L; ++task) {
    const int k = task / c->L, l = task % c->L;
    if (l >= active_levels(c)) continue; /* inactive level: no gradient [HNGP key design 3] */
    if (c->kind == 2) {
      /* Gaussian RBF: each box vertex receives its weights times the upstream */
      for (int64_t p = 0; p < n; ++p) {
        int64_t rows[ORC_MAX_RBF_VERTS];
        real w[ORC_MAX_RBF_VERTS], w1[ORC_MAX_RBF_VERTS][ORC_MAX_D], w2[ORC_MAX_RBF_VERTS][ORC_MAX_D];
        const int nv = rbf_weights(c, l, x + p * d, rows, w, w1, w2);
        for (int q = 0; q < nv; ++q)
          for (int f = 0; f < c->F; ++f) {
            const int col = l * c->F + f;
            real acc = 0.0;
            if (g_gamma) acc += w[q] * (real)g_gamma[p * LF + col];
            for (int i = 0; i < d; ++i) {
              if (g_dgamma) acc += w1[q][i] * (real)g_dgamma[(p * d + i) * LF + col];
              if (g_d2) {
                real up = (real)(c->d2_mode == 2 ? g_d2[(p * d + i) * LF + col] : g_d2[p * LF + col]);
                acc += w2[q][i] * up;
              }
            }
            grad[offs[l] + rows[q] * wid[l] + f] += acc;
          }
      }
      continue;
    }
    for (int64_t p = 0; p < n; ++p) {
      uint32_t base[ORC_MAX_D];
      real t[ORC_MAX_D];
      locate(c, l, x + p * d, base, t);
      for (int cc = 0; cc < nc; ++cc) {
        uint32_t v[ORC_MAX_D];
        for (int i = 0; i < d; ++i) v[i] = base[i] + (uint32_t)((cc >> i) & 1);
        for (int alpha = 0; alpha < na; ++alpha) {
          if (popcount_bits(alpha) != k) continue;
          int64_t row = vertex_row(c, k, l, v);
          int slot = c->kind == 1 ? slot_of_alpha(d, alpha) : 0;
          real w0, w1[ORC_MAX_D], w2[ORC_MAX_D];
          corner_weights(c, l, cc, alpha, t, &w0, w1, w2);
          for (int f = 0; f < c->F; ++f) {
            const int col = l * c->F + f;
            real acc = 0.0;
            if (g_gamma) acc += w0 * (real)g_gamma[p * LF + col];
            if (c->kind == 1) {
              for (int i = 0; i < d; ++i) {
                if (g_dgamma) acc += w1[i] * (real)g_dgamma[(p * d + i) * LF + col];
                if (g_d2) {
                  real up = (real)(c->d2_mode == 2 ? g_d2[(p * d + i) * LF + col] : g_d2[p * LF + col]);
                  acc += w2[i] * up;
                }
              }
            }
            grad[offs[k * c->L + l] + row * wid[k * c->L + l] + (int64_t)slot * c->F + f] += acc;
          }
        }
      }
    }
  }
}

/* ---- fused PINN residual [HNGP key design 2: SIREN activations sin(omega .) and the
 * second-order chain rule; loss section: the residual term of the PINN loss] ----
 * MLP: `depth` hidden layers of width H, a = sin(omega (W v + b)), then a linear output.
 * Parameters, row-major (out x in): W1[H][in], b1[H], (Wk[H][H], bk[H])..., Wo[1][H], bo[1].
 * Forward mode carries, per layer, the value row v, the d gradient rows V_i and the
 * Laplacian row V_lap:
 *     z = W v + b,  Z_i = W V_i,  Z_lap = W V_lap,
 *     a = sin(omega z),  A_i = omega cos(omega z) Z_i,
 *     A_lap = -omega^2 sin(omega z) sum_i Z_i^2 + omega cos(omega z) Z_lap.
 * Residual r = Lap u - g(x) with the manufactured Poisson source
 * g = -d pi^2 prod_i sin(pi x_i) (the Laplacian of prod_i sin(pi x_i)); loss = mean r^2.
 * The reverse sweep differentiates those same expressions (one product rule per term).
 * Outputs (fp64, each may be NULL): u[n], grad_u[n][d], lap_u[n], residual[n], loss[1],
 * grad_params (+=, table layout), grad_mlp (+=, parameter layout above).
 * Returns 0, or -1 on a bad shape. */
int orc_residual(const orc_cfg* c, int32_t hidden, int32_t depth, double omega, int64_t n,
                 const float* x, const double* params, const double* mlp, double* u_out,
                 double* gu_out, double* lu_out, double* residual, double* loss,
                 double* grad_params, double* grad_mlp) {
  if (c->kind != 1 || depth < 1 || depth > 14 || hidden < 1) return -1;
  const int d = c->d, LF = c->L * c->F, H = hidden;
  const int R = d + 2; /* rows carried per layer: value, d gradients, Laplacian */
  const int W = H > LF ? H : LF;
  orc_cfg lc = *c;
  lc.d2_mode = 1;
  int64_t woff[16], boff[16], in_w[16];
  int64_t off = 0;
  for (int k = 0; k <= depth; ++k) {
    int64_t fan_in = k == 0 ? LF : H;
    int64_t fan_out = k == depth ? 1 : H;
    in_w[k] = fan_in;
    woff[k] = off; off += fan_in * fan_out;
    boff[k] = off; off += fan_out;
  }
  const int64_t n_mlp = off;
  /* encoder outputs: gamma, grad gamma, Laplacian gamma */
  double* g = (double*)malloc(sizeof(double) * (size_t)(n * LF + 1));
  double* dg = (double*)malloc(sizeof(double) * (size_t)(n * d * LF + 1));
  double* lp = (double*)malloc(sizeof(double) * (size_t)(n * LF + 1));
  orc_forward(&lc, n, x, params, g, dg, lp);
  /* encoder upstream produced by the reverse sweep */
  double* ug = (double*)calloc((size_t)(n * LF + 1), sizeof(double));
  double* ud = (double*)calloc((size_t)(n * d * LF + 1), sizeof(double));
  double* ul = (double*)calloc((size_t)(n * LF + 1), sizeof(double));
  double* rr = (double*)malloc(sizeof(double) * (size_t)(n + 1));
  int nthreads = 1;
#ifdef _OPENMP
  nthreads = omp_get_max_threads();
#endif
  double* gm_all = (double*)calloc((size_t)(nthreads * n_mlp), sizeof(double));
  const double inv_n = n > 0 ? 1.0 / (double)n : 0.0;
  const real PI = (real)3.14159265358979323846;
  const real om = (real)omega;
#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* gm = gm_all + (int64_t)tid * n_mlp;
    /* tape: act[k] = inputs of layer k (R rows of width W), zs[k] = z, Z_i, Z_lap */
    real* act = (real*)malloc(sizeof(real) * (size_t)((depth + 1) * R * W));
    real* zs = (real*)malloc(sizeof(real) * (size_t)(depth * R * H));
    real* bar = (real*)malloc(sizeof(real) * (size_t)(R * W));
    real* nbar = (real*)malloc(sizeof(real) * (size_t)(R * W));
#pragma omp for schedule(static)
    for (int64_t p = 0; p < n; ++p) {
      for (int j = 0; j < LF; ++j) {
        act[0 * W + j] = (real)g[p * LF + j];
        for (int i = 0; i < d; ++i) act[(1 + i) * W + j] = (real)dg[(p * d + i) * LF + j];
        act[(1 + d) * W + j] = (real)lp[p * LF + j];
      }
      for (int k = 0; k < depth; ++k) {
        const double* Wk = mlp + woff[k];
        const double* bk = mlp + boff[k];
        const int64_t fi = in_w[k];
        for (int o = 0; o < H; ++o) {
          for (int r = 0; r < R; ++r) {
            real z = (r == 0) ? (real)bk[o] : 0.0; /* the bias enters the value row only */
            for (int j = 0; j < fi; ++j) z += (real)Wk[o * fi + j] * act[(k * R + r) * W + j];
            zs[(k * R + r) * H + o] = z;
          }
          const real z0 = zs[(k * R + 0) * H + o];
          const real s = R_SIN(om * z0), co = R_COS(om * z0);
          real sumsq = 0.0;
          for (int i = 0; i < d; ++i) { real zi = zs[(k * R + 1 + i) * H + o]; sumsq += zi * zi; }
          act[((k + 1) * R + 0) * W + o] = s;
          for (int i = 0; i < d; ++i)
            act[((k + 1) * R + 1 + i) * W + o] = om * co * zs[(k * R + 1 + i) * H + o];
          act[((k + 1) * R + 1 + d) * W + o] =
              -om * om * s * sumsq + om * co * zs[(k * R + 1 + d) * H + o];
        }
      }
      /* linear output layer */
      const double* Wo = mlp + woff[depth];
      real uval = (real)mlp[boff[depth]], lap_u = 0.0, gu[ORC_MAX_D] = {0};
      for (int j = 0; j < H; ++j) {
        uval += (real)Wo[j] * act[(depth * R + 0) * W + j];
        for (int i = 0; i < d; ++i) gu[i] += (real)Wo[j] * act[(depth * R + 1 + i) * W + j];
        lap_u += (real)Wo[j] * act[(depth * R + 1 + d) * W + j];
      }
      if (u_out) u_out[p] = uval;
      if (gu_out) for (int i = 0; i < d; ++i) gu_out[p * d + i] = gu[i];
      if (lu_out) lu_out[p] = lap_u;
      real src = -(real)d * PI * PI;
      for (int i = 0; i < d; ++i) src *= R_SIN(PI * (real)x[p * d + i]);
      const real r = lap_u - src;
      rr[p] = r;
      /* reverse sweep: d loss / d Lap u = 2 r / n seeds the Laplacian row only */
      const real seed = (real)(2.0 * (double)r * inv_n);
      for (int j = 0; j < H; ++j) {
        gm[woff[depth] + j] += seed * act[(depth * R + 1 + d) * W + j];
        for (int q = 0; q < R; ++q) bar[q * W + j] = 0.0;
        bar[(1 + d) * W + j] = seed * (real)Wo[j];
      }
      for (int k = depth - 1; k >= 0; --k) {
        const double* Wk = mlp + woff[k];
        const int64_t fi = in_w[k];
        for (int q = 0; q < R; ++q) for (int j = 0; j < fi; ++j) nbar[q * W + j] = 0.0;
        for (int o = 0; o < H; ++o) {
          const real z0 = zs[(k * R + 0) * H + o];
          const real s = R_SIN(om * z0), co = R_COS(om * z0);
          const real zl = zs[(k * R + 1 + d) * H + o];
          real sumsq = 0.0;
          for (int i = 0; i < d; ++i) { real zi = zs[(k * R + 1 + i) * H + o]; sumsq += zi * zi; }
          const real abar = bar[0 * W + o];
          const real lbar = bar[(1 + d) * W + o];
          real zbar[ORC_MAX_D + 2];
          /* d a/dz = w cos;  d A_i/dz = -w^2 sin Z_i;  d A_lap/dz = -w^3 cos sum Z_i^2 - w^2 sin Z_lap */
          real z0bar = abar * om * co +
                       lbar * (-om * om * om * co * sumsq - om * om * s * zl);
          for (int i = 0; i < d; ++i) {
            const real aib = bar[(1 + i) * W + o];
            const real zi = zs[(k * R + 1 + i) * H + o];
            z0bar += aib * (-om * om * s * zi);
            /* d A_i/dZ_i = w cos;  d A_lap/dZ_i = -2 w^2 sin Z_i */
            zbar[1 + i] = aib * om * co + lbar * (-(real)2.0 * om * om * s * zi);
          }
          zbar[0] = z0bar;
          zbar[1 + d] = lbar * om * co; /* d A_lap/dZ_lap = w cos */
          gm[boff[k] + o] += z0bar;
          for (int q = 0; q < R; ++q) {
            const real zb = zbar[q];
            for (int j = 0; j < fi; ++j) {
              gm[woff[k] + o * fi + j] += zb * act[(k * R + q) * W + j];
              nbar[q * W + j] += (real)Wk[o * fi + j] * zb;
            }
          }
        }
        real* tmp = bar; bar = nbar; nbar = tmp;
      }
      for (int j = 0; j < LF; ++j) {
        ug[p * LF + j] = bar[0 * W + j];
        for (int i = 0; i < d; ++i) ud[(p * d + i) * LF + j] = bar[(1 + i) * W + j];
        ul[p * LF + j] = bar[(1 + d) * W + j];
      }
    }
    free(act); free(zs); free(bar); free(nbar);
  }
  /* per-thread MLP gradients reduced in thread order (static schedule: deterministic) */
  if (grad_mlp)
    for (int tdx = 0; tdx < nthreads; ++tdx)
      for (int64_t j = 0; j < n_mlp; ++j) grad_mlp[j] += gm_all[(int64_t)tdx * n_mlp + j];
  double sum_sq = 0.0;
  for (int64_t p = 0; p < n; ++p) sum_sq += rr[p] * rr[p];
  if (loss) *loss = sum_sq * inv_n;
  if (residual) for (int64_t p = 0; p < n; ++p) residual[p] = rr[p];
  if (grad_params) orc_backward_f64(&lc, n, x, ug, ud, ul, grad_params);
  free(g); free(dg); free(lp); free(ug); free(ud); free(ul); free(rr); free(gm_all);
  return 0;
}

/* ---- INGP-FD comparator [HNGP 现有痛点 paragraph and key design 2's comparison: the
 * Laplacian of an Instant-NGP encoding + network by central finite differences, 2d+1
 * forward passes per point] ----
 * Stencil point s of point p: s = 0 is x itself, s = 2i+1 is x + eps e_i and s = 2i+2 is
 * x - eps e_i, the shifted coordinate being one fp32 addition (it is an fp32 encoder input;
 * the encoder clamps to [0, 1] as always).  Every stencil point goes through the d-linear
 * encoding and the same SIREN as the fused residual (value only): a = sin(omega (W v + b)),
 * u = Wo a + bo.  Then
 *     Lap_FD u = sum_i (u(x + eps e_i) - 2 u(x) + u(x - eps e_i)) / eps^2,
 *     r = Lap_FD u - g(x),  loss = mean r^2,  g as for the fused residual.
 * The reverse sweep seeds d loss / d u_s = (2 r / n) c_s, c_0 = -2d / eps^2, c_s = 1 / eps^2
 * otherwise, through each stencil point's network and encoding.  The stencil weights sum to
 * zero, so the output bias does not enter r: its gradient is zero.
 * Outputs (fp64, each may be NULL): u_stencil [n][2d+1], residual [n], loss [1],
 * grad_params (+=, table layout), grad_mlp (+=).  Returns 0, or -1 on a bad shape. */
int orc_fd_residual(const orc_cfg* c, int32_t hidden, int32_t depth, double omega, double eps, int64_t n,
                    const float* x, const double* params, const double* mlp, double* u_stencil,
                    double* residual, double* loss, double* grad_params, double* grad_mlp) {
  if (c->kind != 0 || depth < 1 || depth > 14 || hidden < 1 || !(eps > 0.0)) return -1;
  const int d = c->d, LF = c->L * c->F, H = hidden, S = 2 * d + 1;
  const int W = H > LF ? H : LF;
  int64_t woff[16], boff[16], in_w[16];
  int64_t off = 0;
  for (int k = 0; k <= depth; ++k) {
    int64_t fan_in = k == 0 ? LF : H;
    int64_t fan_out = k == depth ? 1 : H;
    in_w[k] = fan_in;
    woff[k] = off; off += fan_in * fan_out;
    boff[k] = off; off += fan_out;
  }
  const int64_t n_mlp = off;
  const int64_t ns = n * S;
  /* the shifted point sets */
  float* xs = (float*)malloc(sizeof(float) * (size_t)(ns * d + 1));
  const float e32 = (float)eps;
  for (int64_t p = 0; p < n; ++p)
    for (int s = 0; s < S; ++s) {
      float* q = xs + (p * S + s) * d;
      for (int i = 0; i < d; ++i) q[i] = x[p * d + i];
      if (s > 0) {
        const int i = (s - 1) / 2;
        volatile float shifted = (s % 2 == 1) ? x[p * d + i] + e32 : x[p * d + i] - e32;
        q[i] = shifted;
      }
    }
  double* g = (double*)malloc(sizeof(double) * (size_t)(ns * LF + 1));
  orc_forward(c, ns, xs, params, g, NULL, NULL);
  double* ug = (double*)calloc((size_t)(ns * LF + 1), sizeof(double));
  double* rr = (double*)malloc(sizeof(double) * (size_t)(n + 1));
  int nthreads = 1;
#ifdef _OPENMP
  nthreads = omp_get_max_threads();
#endif
  double* gm_all = (double*)calloc((size_t)(nthreads * n_mlp), sizeof(double));
  const double inv_n = n > 0 ? 1.0 / (double)n : 0.0;
  const real PI = (real)3.14159265358979323846;
  const real om = (real)omega, ep = (real)eps;
#pragma omp parallel
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* gm = gm_all + (int64_t)tid * n_mlp;
    /* tape per stencil point: act[s][k] = inputs of layer k (width W), zs[s][k] = z */
    real* act = (real*)malloc(sizeof(real) * (size_t)(S * (depth + 1) * W));
    real* zs = (real*)malloc(sizeof(real) * (size_t)(S * depth * H));
    real* bar = (real*)malloc(sizeof(real) * (size_t)W);
    real* nbar = (real*)malloc(sizeof(real) * (size_t)W);
    real u[2 * ORC_MAX_D + 1];
#pragma omp for schedule(static)
    for (int64_t p = 0; p < n; ++p) {
      for (int s = 0; s < S; ++s) {
        real* a_s = act + (int64_t)s * (depth + 1) * W;
        real* z_s = zs + (int64_t)s * depth * H;
        for (int j = 0; j < LF; ++j) a_s[j] = (real)g[(p * S + s) * LF + j];
        for (int k = 0; k < depth; ++k) {
          const double* Wk = mlp + woff[k];
          for (int o = 0; o < H; ++o) {
            real z = (real)mlp[boff[k] + o];
            for (int j = 0; j < in_w[k]; ++j) z += (real)Wk[o * in_w[k] + j] * a_s[k * W + j];
            z_s[k * H + o] = z;
            a_s[(k + 1) * W + o] = R_SIN(om * z);
          }
        }
        real us = (real)mlp[boff[depth]];
        for (int j = 0; j < H; ++j) us += (real)mlp[woff[depth] + j] * a_s[depth * W + j];
        u[s] = us;
        if (u_stencil) u_stencil[p * S + s] = us;
      }
      real lap = 0.0;
      for (int i = 0; i < d; ++i) lap += (u[2 * i + 1] - (real)2.0 * u[0] + u[2 * i + 2]) / (ep * ep);
      real src = -(real)d * PI * PI;
      for (int i = 0; i < d; ++i) src *= R_SIN(PI * (real)x[p * d + i]);
      const real r = lap - src;
      rr[p] = r;
      const real seed = (real)(2.0 * (double)r * inv_n);
      for (int s = 0; s < S; ++s) {
        const real cs = s == 0 ? -(real)2.0 * (real)d / (ep * ep) : (real)1.0 / (ep * ep);
        const real ubar = seed * cs;
        real* a_s = act + (int64_t)s * (depth + 1) * W;
        real* z_s = zs + (int64_t)s * depth * H;
        for (int j = 0; j < H; ++j) {
          gm[woff[depth] + j] += ubar * a_s[depth * W + j];
          bar[j] = ubar * (real)mlp[woff[depth] + j];
        }
        for (int k = depth - 1; k >= 0; --k) {
          const double* Wk = mlp + woff[k];
          const int64_t fi = in_w[k];
          for (int j = 0; j < fi; ++j) nbar[j] = 0.0;
          for (int o = 0; o < H; ++o) {
            const real zbar = bar[o] * om * R_COS(om * z_s[k * H + o]); /* d sin(w z)/dz */
            gm[boff[k] + o] += zbar;
            for (int j = 0; j < fi; ++j) {
              gm[woff[k] + o * fi + j] += zbar * a_s[k * W + j];
              nbar[j] += (real)Wk[o * fi + j] * zbar;
            }
          }
          real* tmp = bar; bar = nbar; nbar = tmp;
        }
        for (int j = 0; j < LF; ++j) ug[(p * S + s) * LF + j] = bar[j];
      }
    }
    free(act); free(zs); free(bar); free(nbar);
  }
  if (grad_mlp) {
    for (int tdx = 0; tdx < nthreads; ++tdx)
      for (int64_t j = 0; j < n_mlp; ++j) grad_mlp[j] += gm_all[(int64_t)tdx * n_mlp + j];
    /* the output bias is not in r (the stencil weights sum to zero) */
  }
  double sum_sq = 0.0;
  for (int64_t p = 0; p < n; ++p) sum_sq += rr[p] * rr[p];
  if (loss) *loss = sum_sq * inv_n;
  if (residual) for (int64_t p = 0; p < n; ++p) residual[p] = rr[p];
  if (grad_params) orc_backward_f64(c, ns, xs, ug, NULL, NULL, grad_params);
  free(xs); free(g); free(ug); free(rr); free(gm_all);
  return 0;
}

int64_t orc_mlp_param_count(int32_t in, int32_t hidden, int32_t depth) {
  int64_t off = 0;
  for (int k = 0; k <= depth; ++k) {
    int64_t fan_in = k == 0 ? in : hidden;
    int64_t fan_out = k == depth ? 1 : hidden;
    off += fan_in * fan_out + fan_out;
  }
  return off;
}

/* Threads the OpenMP loops above use. */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
