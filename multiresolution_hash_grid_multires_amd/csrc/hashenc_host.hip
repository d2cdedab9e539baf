// Host side of the C ABI: configuration checks, level progression, parameter layout,
// argument validation and kernel dispatch.  No device memory is owned by a handle.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "hashenc.h"
#include "hashenc_diag.h"
#include "binned_backward.h"
#include "hashenc_internal.h"

using hg::Grid;
using hg::kMaxLevels;
using hg::kMaxTables;

struct hashenc {
  int32_t d, L, F, kind, d2_mode, n_tables;
  int32_t N[kMaxLevels];
  int64_t rows[kMaxTables][kMaxLevels];
  int32_t width[kMaxTables][kMaxLevels];
  bool dense[kMaxTables][kMaxLevels];
  int64_t off[kMaxTables][kMaxLevels];
  int64_t n_params;
  Grid grid;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  return HASHENC_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HASHENC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t binom(int n, int k) {
  int64_t r = 1;
  for (int i = 1; i <= k; ++i) r = r * (n - k + i) / i;
  return r;
}

// Largest point count: every 1-D launch (level-major forward with up to 32 levels, backward
// with up to 16 lanes per point) then stays below 2^31 workgroups.
constexpr int64_t kMaxPoints = int64_t(1) << 33;

}  // namespace

// Scratch of the allocation-free backward (hashenc_backward_noalloc): a file-scope device
// array that each GPU holds from module load to process end.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get its per-device address from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {
static __device__ __align__(256) unsigned char scratch[HASHENC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch (the current device), or NULL with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}
}  // namespace

// Hermite forward_ws workspace: the packed order tables (when their sizes are equal), then
// the level-major output staging.
static size_t hermite_forward_ws_bytes(const hashenc* h, int64_t n) {
  const size_t pk = hg::hermite_packed_bytes(h->grid, h->d, h->F);
  return ((pk + 255) & ~size_t(255)) + hg::hermite_stage_bytes(h->grid, h->d, h->F, h->d2_mode, n);
}

extern "C" {

const char* hashenc_last_error(void) { return g_last_error.c_str(); }

int hashenc_create(const hashenc_config* cfg, hashenc** out) {
  if (!cfg || !out) return fail(HASHENC_EINVAL, "hashenc_create: cfg and out must not be NULL");
  if (cfg->d != 2 && cfg->d != 3 && !(cfg->d == 4 && cfg->kind == HASHENC_HERMITE))
    return fail(HASHENC_EINVAL, "d must be 2 or 3, or 4 for the Hermite kind (got %d)", cfg->d);
  if (cfg->n_levels < 1 || cfg->n_levels > kMaxLevels)
    return fail(HASHENC_EINVAL, "n_levels must be in 1..%d (got %d)", kMaxLevels, cfg->n_levels);
  if (cfg->n_features != 1 && cfg->n_features != 2 && cfg->n_features != 4 && cfg->n_features != 8)
    return fail(HASHENC_EINVAL, "n_features must be 1, 2, 4 or 8 (got %d)", cfg->n_features);
  if (cfg->kind != HASHENC_DLINEAR && cfg->kind != HASHENC_HERMITE && cfg->kind != HASHENC_RBF)
    return fail(HASHENC_EINVAL, "kind must be HASHENC_DLINEAR, HASHENC_HERMITE or HASHENC_RBF (got %d)", cfg->kind);
  if (cfg->kind != HASHENC_DLINEAR && cfg->d2_mode != HASHENC_D2_LAPLACIAN && cfg->d2_mode != HASHENC_D2_DIAG)
    return fail(HASHENC_EINVAL, "d2_mode must be HASHENC_D2_LAPLACIAN or HASHENC_D2_DIAG (got %d)",
                cfg->d2_mode);
  if (cfg->reserved != 0 || cfg->reserved2 != 0) return fail(HASHENC_EINVAL, "reserved fields must be 0");
  if (cfg->kind == HASHENC_RBF) {
    if (!(cfg->rbf_eps > 0.0) || !std::isfinite(cfg->rbf_eps))
      return fail(HASHENC_EINVAL, "rbf_eps must be > 0 and finite");
    if (cfg->rbf_rings < 1 || cfg->rbf_rings > 4)
      return fail(HASHENC_EINVAL, "rbf_rings must be in 1..4 (got %d)", cfg->rbf_rings);
  }

  hashenc* h = new (std::nothrow) hashenc();
  if (!h) return fail(HASHENC_ENOMEM, "hashenc_create: out of host memory");
  h->d = cfg->d;
  h->L = cfg->n_levels;
  h->F = cfg->n_features;
  h->kind = cfg->kind;
  h->d2_mode = cfg->kind != HASHENC_DLINEAR ? cfg->d2_mode : 0;
  h->n_tables = cfg->kind == HASHENC_HERMITE ? cfg->d + 1 : 1;

  // Level resolutions: explicit list, or the geometric progression N_min * b^l (floored,
  // with a 1e-6 guard so exact powers are not lost to fp64 rounding).
  if (cfg->resolutions) {
    for (int l = 0; l < h->L; ++l) h->N[l] = cfg->resolutions[l];
  } else {
    if (cfg->n_min < 1) { delete h; return fail(HASHENC_EINVAL, "n_min must be >= 1 (got %d)", cfg->n_min); }
    double b = cfg->growth;
    if (!(b > 0.0)) {
      if (h->L > 1 && cfg->n_max < cfg->n_min) {
        delete h;
        return fail(HASHENC_EINVAL, "n_max (%d) must be >= n_min (%d)", cfg->n_max, cfg->n_min);
      }
      b = h->L == 1 ? 1.0
                    : std::exp((std::log((double)cfg->n_max) - std::log((double)cfg->n_min)) /
                               (double)(h->L - 1));
    }
    for (int l = 0; l < h->L; ++l) {
      const double v = std::floor((double)cfg->n_min * std::pow(b, (double)l) + 1e-6);
      if (!(v >= 1.0 && v <= (double)(1 << 20))) {
        delete h;
        return fail(HASHENC_EINVAL, "level %d resolution %.0f outside 1..2^20", l, v);
      }
      h->N[l] = (int32_t)v;
    }
  }
  for (int l = 0; l < h->L; ++l)
    if (h->N[l] < 1 || h->N[l] > (1 << 20)) {
      const int bad = h->N[l];
      delete h;
      return fail(HASHENC_EINVAL, "level %d resolution %d outside 1..2^20", l, bad);
    }

  // Layout: table k (derivative order), then level, then rows of C(d,k) * F floats.
  int64_t off = 0;
  for (int k = 0; k < h->n_tables; ++k) {
    const uint32_t T = cfg->table_size[k];
    if (T < 1) {
      delete h;
      return fail(HASHENC_EINVAL, "table_size[%d] must be >= 1", k);
    }
    const int32_t w = (int32_t)((h->kind == HASHENC_HERMITE ? binom(h->d, k) : 1) * h->F);
    for (int l = 0; l < h->L; ++l) {
      const double verts = std::pow((double)h->N[l] + 1.0, (double)h->d);
      const bool dense = verts <= (double)T;
      int64_t r = dense ? (int64_t)verts : (int64_t)T;
      h->rows[k][l] = r;
      h->width[k][l] = w;
      h->dense[k][l] = dense;
      h->off[k][l] = off;
      off += r * w;
    }
  }
  h->n_params = off;
  if (off > ((int64_t)1 << 40)) {
    delete h;
    return fail(HASHENC_EINVAL, "parameter count %lld too large", (long long)off);
  }

  Grid& g = h->grid;
  std::memset(&g, 0, sizeof g);
  g.L = h->L;
  g.Lrow = h->L;
  if (h->kind == HASHENC_RBF) {
    g.rbf_e2 = (float)(cfg->rbf_eps * cfg->rbf_eps);
    g.rings = cfg->rbf_rings;
  }
  g.n_tables = h->n_tables;
  for (int l = 0; l < h->L; ++l) {
    g.N[l] = h->N[l];
    g.Nf[l] = (float)h->N[l];
    g.invN[l] = 1.0f / (float)h->N[l];
  }
  for (int k = 0; k < h->n_tables; ++k) {
    const uint32_t T = cfg->table_size[k];
    g.T[k] = T;
    g.Tmask[k] = (T > 1 && (T & (T - 1)) == 0) ? T - 1 : 0u;
    for (int l = 0; l < h->L; ++l) {
      if (h->dense[k][l]) g.dense[k] |= 1u << l;
      g.off[k][l] = h->off[k][l];
    }
  }
  *out = h;
  return ok();
}

void hashenc_destroy(hashenc* h) { delete h; }

int hashenc_info(const hashenc* h, int64_t* n_params, int32_t* out_width, int32_t* resolutions) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_info: NULL handle");
  if (n_params) *n_params = h->n_params;
  if (out_width) *out_width = h->L * h->F;
  if (resolutions)
    for (int l = 0; l < h->L; ++l) resolutions[l] = h->N[l];
  return ok();
}

int hashenc_derive_active(const hashenc* h, int32_t n_active, hashenc** out) {
  if (!h || !out) return fail(HASHENC_EINVAL, "hashenc_derive_active: h and out must not be NULL");
  if (n_active < 1 || n_active > h->L)
    return fail(HASHENC_EINVAL, "hashenc_derive_active: n_active must be in 1..%d (got %d)", h->L, n_active);
  hashenc* c = new (std::nothrow) hashenc(*h);
  if (!c) return fail(HASHENC_ENOMEM, "hashenc_derive_active: out of host memory");
  c->grid.L = n_active;  // kernels compute levels < n_active; rows keep h->L levels
  *out = c;
  return ok();
}

int hashenc_active_levels(const hashenc* h, int32_t* n_active) {
  if (!h || !n_active) return fail(HASHENC_EINVAL, "hashenc_active_levels: NULL pointer");
  *n_active = h->grid.L;
  return ok();
}

int hashenc_c2f_active_levels(int32_t n_levels, int32_t l0, int64_t step, int64_t tau, int32_t* n_active) {
  if (!n_active) return fail(HASHENC_EINVAL, "hashenc_c2f_active_levels: NULL n_active");
  if (n_levels < 1 || l0 < 1 || step < 0 || tau < 1)
    return fail(HASHENC_EINVAL, "hashenc_c2f_active_levels: need n_levels >= 1, l0 >= 1, step >= 0, tau >= 1");
  const int64_t a = (int64_t)l0 + step / tau;
  *n_active = a < (int64_t)n_levels ? (int32_t)a : n_levels;
  return ok();
}

int hashenc_param_layout(const hashenc* h, int32_t order, int32_t level, int64_t* offset,
                         int64_t* rows, int32_t* row_width, int32_t* is_dense) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_param_layout: NULL handle");
  if (order < 0 || order >= h->n_tables)
    return fail(HASHENC_EINVAL, "order %d outside 0..%d", order, h->n_tables - 1);
  if (level < 0 || level >= h->L) return fail(HASHENC_EINVAL, "level %d outside 0..%d", level, h->L - 1);
  if (offset) *offset = h->off[order][level];
  if (rows) *rows = h->rows[order][level];
  if (row_width) *row_width = h->width[order][level];
  if (is_dense) *is_dense = h->dense[order][level] ? 1 : 0;
  return ok();
}

int hashenc_forward(const hashenc* h, int64_t n, const float* x, const float* params,
                    float* gamma, float* dgamma, float* d2gamma, hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_forward: NULL handle");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_forward: n = %lld out of range", (long long)n);
  if (h->kind == HASHENC_DLINEAR && (dgamma || d2gamma))
    return fail(HASHENC_EUNSUPPORTED, "hashenc_forward: derivative outputs need the Hermite or RBF kind");
  if (n == 0 || (!gamma && !dgamma && !d2gamma)) return ok();
  if (!x || !params) return fail(HASHENC_EINVAL, "hashenc_forward: x and params must not be NULL");
  if (!aligned16(x) || !aligned16(params) || !aligned16(gamma) || !aligned16(dgamma) || !aligned16(d2gamma))
    return fail(HASHENC_EALIGN, "hashenc_forward: device pointers must be 16-byte aligned");
  hipError_t e;
  if (h->kind == HASHENC_DLINEAR)
    e = hg::launch_dlinear_forward(h->grid, h->d, h->F, n, x, params, gamma, nullptr, stream);
  else if (h->kind == HASHENC_RBF)
    e = hg::launch_rbf_forward(h->grid, h->d, h->F, h->d2_mode, n, x, params, gamma, dgamma, d2gamma, stream);
  else if (h->d == 4)
    e = hg::launch_hermite4_forward(h->grid, h->F, h->d2_mode, n, x, params, nullptr, gamma, dgamma, d2gamma,
                                    stream);
  else
    e = hg::launch_hermite_forward(h->grid, h->d, h->F, h->d2_mode, n, x, params, nullptr, nullptr, false, gamma,
                                   dgamma, d2gamma, stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_forward launch");
  return ok();
}

int hashenc_forward_workspace_size(const hashenc* h, int64_t n, size_t* bytes) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_forward_workspace_size: NULL handle");
  if (!bytes) return fail(HASHENC_EINVAL, "hashenc_forward_workspace_size: NULL bytes");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_forward_workspace_size: n out of range");
  *bytes = h->kind == HASHENC_DLINEAR                 ? hg::dlinear_forward_workspace_bytes(h->grid, h->d, h->F, n)
           : (h->kind == HASHENC_HERMITE && h->d < 4) ? hermite_forward_ws_bytes(h, n)
           : h->kind == HASHENC_HERMITE               ? hg::hermite4_packed_bytes(h->grid, h->F)  // 4D: packed copy
                                                      : 0;  // RBF: no workspace
  return ok();
}

// The workspace forward (who: the entry point named in messages).  With direct_small, 2D and
// 3D Hermite batches below kPackMinPoints take the direct forward: there the fixed cost of
// packing every order table (about 0.14 ms for four 2^19-row tables) exceeds what the packed
// gather saves (measured on MI355X: at 4096 points of the 16-level 3D grid 0.028 ms direct
// against 0.147 ms packed; equal near 32 K points; the 2D 2^14-row grid about 50 K points).
// The 4D packed copy costs little (five 2^16-row tables) and is taken at every n.
static int forward_ws_impl(const char* who, const hashenc* h, int64_t n, const float* x, const float* params,
                           float* gamma, float* dgamma, float* d2gamma, void* workspace, size_t workspace_bytes,
                           hashenc_stream_t stream, bool direct_small) {
  if (!h) return fail(HASHENC_EINVAL, "%s: NULL handle", who);
  if (h->kind == HASHENC_RBF || (h->d == 4 && hg::hermite4_packed_bytes(h->grid, h->F) == 0))
    return hashenc_forward(h, n, x, params, gamma, dgamma, d2gamma, stream);
  if (h->d == 4) {
    // workspace: the packed copy of the five order tables, written and then read by the forward
    const size_t need = hg::hermite4_packed_bytes(h->grid, h->F);
    if (n == 0 || (!gamma && !dgamma && !d2gamma))
      return hashenc_forward(h, n, x, params, gamma, dgamma, d2gamma, stream);
    if (n < 0 || n > kMaxPoints)
      return fail(HASHENC_EINVAL, "%s: n = %lld out of range", who, (long long)n);
    if (!x || !params || !workspace)
      return fail(HASHENC_EINVAL, "%s: x, params and workspace must not be NULL", who);
    if (!aligned16(x) || !aligned16(params) || !aligned16(gamma) || !aligned16(dgamma) || !aligned16(d2gamma) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspace 256-byte)", who);
    if (workspace_bytes < need)
      return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, need);
    hipError_t e = hg::launch_hermite4_forward(h->grid, h->F, h->d2_mode, n, x, params, static_cast<float*>(workspace),
                                               gamma, dgamma, d2gamma, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
  }
  if (h->kind == HASHENC_HERMITE) {
    // workspace: [packed copy of the order tables (equal table sizes) | level-major staging]
    const size_t need = hermite_forward_ws_bytes(h, n);
    if (n == 0 || (!gamma && !dgamma && !d2gamma) || (direct_small && n < hg::kPackMinPoints))
      return hashenc_forward(h, n, x, params, gamma, dgamma, d2gamma, stream);
    if (n < 0 || n > kMaxPoints)
      return fail(HASHENC_EINVAL, "%s: n = %lld out of range", who, (long long)n);
    if (!x || !params || !workspace)
      return fail(HASHENC_EINVAL, "%s: x, params and workspace must not be NULL", who);
    if (!aligned16(x) || !aligned16(params) || !aligned16(gamma) || !aligned16(dgamma) || !aligned16(d2gamma) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspace 256-byte)", who);
    if (workspace_bytes < need)
      return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, need);
    const size_t pk = hg::hermite_packed_bytes(h->grid, h->d, h->F);
    float* packed = pk ? static_cast<float*>(workspace) : nullptr;
    float* stage = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((pk + 255) & ~size_t(255)));
    hipError_t e = packed ? hg::launch_hermite_pack(h->grid, h->d, h->F, params, packed, stream) : hipSuccess;
    if (e == hipSuccess)
      e = hg::launch_hermite_forward(h->grid, h->d, h->F, h->d2_mode, n, x, params, packed, stage, true, gamma,
                                     dgamma, d2gamma, stream);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
  }
  if (!gamma || n == 0) return hashenc_forward(h, n, x, params, gamma, dgamma, d2gamma, stream);
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "%s: n = %lld out of range", who, (long long)n);
  if (dgamma || d2gamma)
    return fail(HASHENC_EUNSUPPORTED, "%s: derivative outputs need the Hermite kind", who);
  if (!x || !params || !workspace)
    return fail(HASHENC_EINVAL, "%s: x, params and workspace must not be NULL", who);
  if (!aligned16(x) || !aligned16(params) || !aligned16(gamma) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspace 256-byte)", who);
  const size_t need = hg::dlinear_forward_workspace_bytes(h->grid, h->d, h->F, n);
  if (workspace_bytes < need)
    return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, need);
  hipError_t e = hg::launch_dlinear_forward(h->grid, h->d, h->F, n, x, params, gamma,
                                            static_cast<float*>(workspace), stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int hashenc_forward_ws(const hashenc* h, int64_t n, const float* x, const float* params, float* gamma,
                       float* dgamma, float* d2gamma, void* workspace, size_t workspace_bytes,
                       hashenc_stream_t stream) {
  return forward_ws_impl("hashenc_forward_ws", h, n, x, params, gamma, dgamma, d2gamma, workspace, workspace_bytes,
                         stream, true);
}

int hashenc_diag_forward_packed(const hashenc* h, int64_t n, const float* x, const float* params, float* gamma,
                                float* dgamma, float* d2gamma, void* workspace, size_t workspace_bytes,
                                hashenc_stream_t stream) {
  return forward_ws_impl("hashenc_diag_forward_packed", h, n, x, params, gamma, dgamma, d2gamma, workspace,
                         workspace_bytes, stream, false);
}

int hashenc_backward(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                     const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                     hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_backward: NULL handle");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_backward: n = %lld out of range", (long long)n);
  if (h->kind == HASHENC_DLINEAR && (g_dgamma || g_d2gamma))
    return fail(HASHENC_EUNSUPPORTED, "hashenc_backward: derivative upstream needs the Hermite or RBF kind");
  if (n == 0 || (!g_gamma && !g_dgamma && !g_d2gamma)) return ok();
  if (!x || !grad_params) return fail(HASHENC_EINVAL, "hashenc_backward: x and grad_params must not be NULL");
  if (!aligned16(x) || !aligned16(grad_params) || !aligned16(g_gamma) || !aligned16(g_dgamma) ||
      !aligned16(g_d2gamma))
    return fail(HASHENC_EALIGN, "hashenc_backward: device pointers must be 16-byte aligned");
  hipError_t e;
  if (h->kind == HASHENC_DLINEAR)
    e = hg::launch_dlinear_backward(h->grid, h->d, h->F, n, x, g_gamma, nullptr, grad_params, stream);
  else if (h->kind == HASHENC_RBF)
    e = hg::launch_rbf_backward(h->grid, h->d, h->F, h->d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params,
                                stream);
  else if (h->d == 4)
    e = hg::launch_hermite4_backward(h->grid, h->F, h->d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params,
                                     stream);
  else
    e = hg::launch_hermite_backward(h->grid, h->d, h->F, h->d2_mode, n, x, g_gamma, g_dgamma,
                                         g_d2gamma, nullptr, grad_params, stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_backward launch");
  return ok();
}

// The binned path keeps per-bin counters and staging in LDS; larger configurations take the
// atomic path.
static bool binned_supported(const hashenc* h) {
  if (h->kind == HASHENC_RBF) return false;  // the RBF backward accumulates per level in LDS
  return hg::binned_fits(h->grid, h->d, h->F, h->kind == HASHENC_HERMITE);
}

// The binned path for a backward of n points: small d-linear batches scatter faster with
// atomics (measured on MI355X: at 4096 points of the 16-level 3D grid 26 us against 76 us,
// at 65536 points 277 us against 114 us; the binned path's fixed cost is a few scans and
// passes over its bins), so below n * L = 2^18 they take the atomic path.  The Hermite
// kind's atomic scatter-add issues one request per coefficient row and stays slower down to
// 4096 points.
static bool binned_for(const hashenc* h, int64_t n) {
  if (!binned_supported(h)) return false;
  return !(h->kind == HASHENC_DLINEAR && n * (int64_t)h->grid.L < (int64_t(1) << 18));
}

static int check_mlp(const hashenc* h, const hashenc_mlp* mlp, const char* who) {
  if (!h) return fail(HASHENC_EINVAL, "%s: NULL handle", who);
  if (!mlp) return fail(HASHENC_EINVAL, "%s: NULL mlp", who);
  if (h->kind != HASHENC_HERMITE)
    return fail(HASHENC_EUNSUPPORTED, "%s: the residual needs a Hermite handle (second derivatives)", who);
  if (h->d == 4) return fail(HASHENC_EUNSUPPORTED, "%s: the residual covers d = 2 and 3", who);
  if (mlp->in != h->L * h->F)
    return fail(HASHENC_EINVAL, "%s: mlp.in (%d) must equal L*F (%d)", who, mlp->in, h->L * h->F);
  if (mlp->in > 64) return fail(HASHENC_EUNSUPPORTED, "%s: mlp.in must be <= 64", who);
  if (mlp->hidden < 1 || mlp->hidden > 64)
    return fail(HASHENC_EUNSUPPORTED, "%s: hidden width must be in 1..64 (got %d)", who, mlp->hidden);
  if (mlp->depth < 1 || mlp->depth > 4)
    return fail(HASHENC_EUNSUPPORTED, "%s: depth must be in 1..4 (got %d)", who, mlp->depth);
  if (mlp->out != 1) return fail(HASHENC_EUNSUPPORTED, "%s: output width must be 1", who);
  if (mlp->reserved != 0) return fail(HASHENC_EINVAL, "%s: mlp.reserved must be 0", who);
  if (!std::isfinite(mlp->omega)) return fail(HASHENC_EINVAL, "%s: omega must be finite", who);
  return HASHENC_OK;
}

int hashenc_residual_workspace_size(const hashenc* h, const hashenc_mlp* mlp, int64_t n,
                                    size_t* bytes) {
  int rc = check_mlp(h, mlp, "hashenc_residual_workspace_size");
  if (rc) return rc;
  if (n < 1 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_residual_workspace_size: n out of range");
  if (!bytes) return fail(HASHENC_EINVAL, "hashenc_residual_workspace_size: NULL bytes");
  *bytes = hg::residual_workspace_bytes(h->grid, h->d, h->F, n, mlp->in, mlp->hidden, mlp->depth,
                                        binned_supported(h));
  return ok();
}

int hashenc_residual(const hashenc* h, const hashenc_mlp* mlp, int64_t n, const float* x,
                     const float* params, const float* mlp_params, float* residual, float* loss,
                     float* grad_params, float* grad_mlp, void* workspace, size_t workspace_bytes,
                     hashenc_stream_t stream) {
  int rc = check_mlp(h, mlp, "hashenc_residual");
  if (rc) return rc;
  if (n < 1 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_residual: n = %lld out of range", (long long)n);
  if (!x || !params || !mlp_params || !loss || !workspace)
    return fail(HASHENC_EINVAL, "hashenc_residual: x, params, mlp_params, loss and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(params) || !aligned16(mlp_params) || !aligned16(residual) ||
      !aligned16(loss) || !aligned16(grad_params) || !aligned16(grad_mlp) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(HASHENC_EALIGN, "hashenc_residual: pointers must be 16-byte aligned (workspace 256-byte)");
  const size_t need = hg::residual_workspace_bytes(h->grid, h->d, h->F, n, mlp->in, mlp->hidden, mlp->depth,
                                                   binned_supported(h));
  if (workspace_bytes < need)
    return fail(HASHENC_EINVAL, "hashenc_residual: workspace of %zu bytes < %zu needed", workspace_bytes, need);
  hipError_t e = hg::run_residual(h->grid, h->d, h->F, n, x, params, mlp->in, mlp->hidden, mlp->depth,
                                  mlp->omega, mlp_params, residual, loss, grad_params, grad_mlp,
                                  workspace, binned_supported(h), stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_residual launch");
  return ok();
}

static int check_fd(const hashenc* h, const hashenc_mlp* mlp, const char* who) {
  if (!h) return fail(HASHENC_EINVAL, "%s: NULL handle", who);
  if (!mlp) return fail(HASHENC_EINVAL, "%s: NULL mlp", who);
  if (h->kind != HASHENC_DLINEAR)
    return fail(HASHENC_EUNSUPPORTED, "%s: the finite-difference comparator takes a d-linear handle", who);
  if (mlp->in != h->L * h->F)
    return fail(HASHENC_EINVAL, "%s: mlp.in (%d) must equal L*F (%d)", who, mlp->in, h->L * h->F);
  if (mlp->in > 64) return fail(HASHENC_EUNSUPPORTED, "%s: mlp.in must be <= 64", who);
  if (mlp->hidden < 1 || mlp->hidden > 64)
    return fail(HASHENC_EUNSUPPORTED, "%s: hidden width must be in 1..64 (got %d)", who, mlp->hidden);
  if (mlp->depth < 1 || mlp->depth > 4)
    return fail(HASHENC_EUNSUPPORTED, "%s: depth must be in 1..4 (got %d)", who, mlp->depth);
  if (mlp->out != 1) return fail(HASHENC_EUNSUPPORTED, "%s: output width must be 1", who);
  if (mlp->reserved != 0) return fail(HASHENC_EINVAL, "%s: mlp.reserved must be 0", who);
  if (!std::isfinite(mlp->omega)) return fail(HASHENC_EINVAL, "%s: omega must be finite", who);
  return HASHENC_OK;
}

int hashenc_fd_residual_workspace_size(const hashenc* h, const hashenc_mlp* mlp, int64_t n, size_t* bytes) {
  int rc = check_fd(h, mlp, "hashenc_fd_residual_workspace_size");
  if (rc) return rc;
  if (n < 1 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_fd_residual_workspace_size: n out of range");
  if (!bytes) return fail(HASHENC_EINVAL, "hashenc_fd_residual_workspace_size: NULL bytes");
  *bytes = hg::fd_residual_workspace_bytes(h->grid, h->d, h->F, n, mlp->in, mlp->hidden, mlp->depth,
                                           binned_supported(h));
  return ok();
}

int hashenc_fd_residual(const hashenc* h, const hashenc_mlp* mlp, float eps, int64_t n, const float* x,
                        const float* params, const float* mlp_params, float* u_stencil, float* residual,
                        float* loss, float* grad_params, float* grad_mlp, void* workspace, size_t workspace_bytes,
                        hashenc_stream_t stream) {
  int rc = check_fd(h, mlp, "hashenc_fd_residual");
  if (rc) return rc;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(HASHENC_EINVAL, "hashenc_fd_residual: eps must be > 0 and finite");
  if (n < 1 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_fd_residual: n = %lld out of range", (long long)n);
  if (!x || !params || !mlp_params || !loss || !workspace)
    return fail(HASHENC_EINVAL, "hashenc_fd_residual: x, params, mlp_params, loss and workspace must not be NULL");
  if (!aligned16(x) || !aligned16(params) || !aligned16(mlp_params) || !aligned16(u_stencil) ||
      !aligned16(residual) || !aligned16(loss) || !aligned16(grad_params) || !aligned16(grad_mlp) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(HASHENC_EALIGN, "hashenc_fd_residual: pointers must be 16-byte aligned (workspace 256-byte)");
  const size_t need = hg::fd_residual_workspace_bytes(h->grid, h->d, h->F, n, mlp->in, mlp->hidden, mlp->depth,
                                                      binned_supported(h));
  if (workspace_bytes < need)
    return fail(HASHENC_EINVAL, "hashenc_fd_residual: workspace of %zu bytes < %zu needed", workspace_bytes, need);
  hipError_t e = hg::run_fd_residual(h->grid, h->d, h->F, n, x, params, mlp->in, mlp->hidden, mlp->depth,
                                     mlp->omega, eps, mlp_params, u_stencil, residual, loss, grad_params, grad_mlp,
                                     workspace, binned_supported(h), stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_fd_residual launch");
  return ok();
}

int hashenc_backward_workspace_size(const hashenc* h, int64_t n, size_t* bytes) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_backward_workspace_size: NULL handle");
  if (!bytes) return fail(HASHENC_EINVAL, "hashenc_backward_workspace_size: NULL bytes");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_backward_workspace_size: n out of range");
  *bytes = (n == 0 || !binned_for(h, n))
               ? 0
               : hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, h->kind == HASHENC_HERMITE, n);
  return ok();
}

// The binned backward with caller workspace, after the common argument checks (who: the
// entry point's name for messages).
static int backward_binned(const char* who, const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                           const float* g_dgamma, const float* g_d2gamma, float* grad_params, void* workspace,
                           size_t workspace_bytes, hashenc_stream_t stream) {
  if (!x || !grad_params || !workspace)
    return fail(HASHENC_EINVAL, "%s: x, grad_params and workspace must not be NULL", who);
  if (!aligned16(x) || !aligned16(grad_params) || !aligned16(g_gamma) || !aligned16(g_dgamma) ||
      !aligned16(g_d2gamma) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspace 256-byte)", who);
  const size_t need = hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, h->kind == HASHENC_HERMITE, n);
  if (workspace_bytes < need)
    return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, need);
  hipError_t e = hg::run_binned_backward(h->grid, h->d, h->F, h->kind == HASHENC_HERMITE, h->d2_mode, n, x,
                                         g_gamma, g_dgamma, g_d2gamma, nullptr, grad_params, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int hashenc_backward_ws(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                        const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                        void* workspace, size_t workspace_bytes, hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_backward_ws: NULL handle");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_backward_ws: n = %lld out of range", (long long)n);
  if (h->kind == HASHENC_DLINEAR && (g_dgamma || g_d2gamma))
    return fail(HASHENC_EUNSUPPORTED, "hashenc_backward_ws: derivative upstream needs the Hermite kind");
  if (n == 0 || (!g_gamma && !g_dgamma && !g_d2gamma)) return ok();
  if (!binned_for(h, n))
    return hashenc_backward(h, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params, stream);
  return backward_binned("hashenc_backward_ws", h, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params, workspace,
                         workspace_bytes, stream);
}

// Whether hashenc_forward_counting leaves counts for a backward of these n points: the
// d-linear binned path, one chunk, and forward passes whose bins fit its LDS counters.  The
// counting forward and the counted backward decide alike from (h, n) alone.
static bool counting_for(const hashenc* h, int64_t n) {
  return h->kind == HASHENC_DLINEAR && n > 0 && binned_for(h, n) &&
         n <= hg::bin_chunk_points(h->grid, h->d, false) && hg::dlinear_forward_counts(h->grid, h->d, h->F);
}

int hashenc_forward_counting(const hashenc* h, int64_t n, const float* x, const float* params, float* gamma,
                             float* dgamma, float* d2gamma, void* workspace, size_t workspace_bytes,
                             void* bwd_workspace, size_t bwd_workspace_bytes, hashenc_stream_t stream) {
  const char* who = "hashenc_forward_counting";
  if (!h) return fail(HASHENC_EINVAL, "%s: NULL handle", who);
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "%s: n = %lld out of range", who, (long long)n);
  if (!counting_for(h, n))
    return forward_ws_impl(who, h, n, x, params, gamma, dgamma, d2gamma, workspace, workspace_bytes, stream, true);
  if (dgamma || d2gamma)
    return fail(HASHENC_EUNSUPPORTED, "%s: derivative outputs need the Hermite kind", who);
  if (!x || !params || !gamma || !workspace || !bwd_workspace)
    return fail(HASHENC_EINVAL, "%s: x, params, gamma and both workspaces must not be NULL", who);
  if (!aligned16(x) || !aligned16(params) || !aligned16(gamma) || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      (reinterpret_cast<uintptr_t>(bwd_workspace) & 255u))
    return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspaces 256-byte)", who);
  const size_t need = hg::dlinear_forward_workspace_bytes(h->grid, h->d, h->F, n);
  if (workspace_bytes < need)
    return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, workspace_bytes, need);
  const size_t bneed = hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, false, n);
  if (bwd_workspace_bytes < bneed)
    return fail(HASHENC_EINVAL, "%s: backward workspace of %zu bytes < %zu needed", who, bwd_workspace_bytes, bneed);
  const uintptr_t f0 = reinterpret_cast<uintptr_t>(workspace), b0 = reinterpret_cast<uintptr_t>(bwd_workspace);
  if (f0 < b0 + bneed && b0 < f0 + need)
    return fail(HASHENC_EINVAL, "%s: the two workspaces overlap", who);
  hipError_t e = hg::launch_dlinear_forward_counting(h->grid, h->d, h->F, n, x, params, gamma,
                                                     static_cast<float*>(workspace), bwd_workspace, stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int hashenc_backward_counted(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                             const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                             void* bwd_workspace, size_t bwd_workspace_bytes, hashenc_stream_t stream) {
  const char* who = "hashenc_backward_counted";
  if (!h) return fail(HASHENC_EINVAL, "%s: NULL handle", who);
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "%s: n = %lld out of range", who, (long long)n);
  if (!counting_for(h, n))
    return hashenc_backward_ws(h, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params, bwd_workspace,
                               bwd_workspace_bytes, stream);
  if (g_dgamma || g_d2gamma)
    return fail(HASHENC_EUNSUPPORTED, "%s: derivative upstream needs the Hermite kind", who);
  if (!g_gamma) return ok();
  if (!x || !grad_params || !bwd_workspace)
    return fail(HASHENC_EINVAL, "%s: x, grad_params and the workspace must not be NULL", who);
  if (!aligned16(x) || !aligned16(grad_params) || !aligned16(g_gamma) ||
      (reinterpret_cast<uintptr_t>(bwd_workspace) & 255u))
    return fail(HASHENC_EALIGN, "%s: pointers must be 16-byte aligned (workspace 256-byte)", who);
  const size_t need = hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, false, n);
  if (bwd_workspace_bytes < need)
    return fail(HASHENC_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, bwd_workspace_bytes, need);
  hipError_t e = hg::run_binned_backward(h->grid, h->d, h->F, false, h->d2_mode, n, x, g_gamma, nullptr, nullptr,
                                         nullptr, grad_params, bwd_workspace, stream, 0, true);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

int hashenc_diag_binned_workspace_size(const hashenc* h, int64_t n, size_t* bytes) {
  if (!h || !bytes) return fail(HASHENC_EINVAL, "hashenc_diag_binned_workspace_size: NULL pointer");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_diag_binned_workspace_size: n out of range");
  if (!binned_supported(h)) return fail(HASHENC_EUNSUPPORTED, "hashenc_diag_binned_workspace_size: no binned plan");
  *bytes = n == 0 ? 0 : hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, h->kind == HASHENC_HERMITE, n);
  return ok();
}

int hashenc_diag_backward_binned(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                                 const float* g_dgamma, const float* g_d2gamma, float* grad_params, void* workspace,
                                 size_t workspace_bytes, hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_diag_backward_binned: NULL handle");
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_diag_backward_binned: n out of range");
  if (h->kind == HASHENC_DLINEAR && (g_dgamma || g_d2gamma))
    return fail(HASHENC_EUNSUPPORTED, "hashenc_diag_backward_binned: derivative upstream needs the Hermite kind");
  if (!binned_supported(h)) return fail(HASHENC_EUNSUPPORTED, "hashenc_diag_backward_binned: no binned plan");
  if (n == 0 || (!g_gamma && !g_dgamma && !g_d2gamma)) return ok();
  return backward_binned("hashenc_diag_backward_binned", h, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params,
                         workspace, workspace_bytes, stream);
}

int hashenc_backward_noalloc(const hashenc* h, int64_t n, const float* x, const float* g_gamma,
                             const float* g_dgamma, const float* g_d2gamma, float* grad_params,
                             hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_backward_noalloc: NULL handle");
  if (n < 0 || n > kMaxPoints)
    return fail(HASHENC_EINVAL, "hashenc_backward_noalloc: n = %lld out of range", (long long)n);
  if (h->kind == HASHENC_DLINEAR && (g_dgamma || g_d2gamma))
    return fail(HASHENC_EUNSUPPORTED, "hashenc_backward_noalloc: derivative upstream needs the Hermite kind");
  if (n == 0 || (!g_gamma && !g_dgamma && !g_d2gamma)) return ok();
  if (!binned_for(h, n))  // the atomic scatter-add uses no scratch
    return hashenc_backward(h, n, x, g_gamma, g_dgamma, g_d2gamma, grad_params, stream);
  if (!x || !grad_params) return fail(HASHENC_EINVAL, "hashenc_backward_noalloc: x and grad_params must not be NULL");
  if (!aligned16(x) || !aligned16(grad_params) || !aligned16(g_gamma) || !aligned16(g_dgamma) ||
      !aligned16(g_d2gamma))
    return fail(HASHENC_EALIGN, "hashenc_backward_noalloc: device pointers must be 16-byte aligned");
  const bool hermite = h->kind == HASHENC_HERMITE;
  // the largest chunk (a multiple of 1024 points) whose binned workspace fits the scratch
  const size_t cap = HASHENC_NOALLOC_SCRATCH_BYTES;
  if (hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, hermite, 1024) > cap)
    return fail(HASHENC_EINVAL,
                "hashenc_backward_noalloc: a 1024-point chunk of this configuration needs %zu bytes of scratch; "
                "the static scratch holds %zu (use hashenc_backward_ws with a workspace)",
                hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, hermite, 1024), cap);
  int64_t lo = 1, hi = (n + 1023) / 1024;  // in units of 1024 points; lo always fits
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (hg::binned_backward_workspace_bytes(h->grid, h->d, h->F, hermite, mid * 1024) <= cap) lo = mid;
    else hi = mid - 1;
  }
  const int64_t chunk = lo * 1024;
  hipError_t e = hipSuccess;
  void* ptr = scratch_ptr(&e);
  if (!ptr) return hip_fail(e, "hashenc_backward_noalloc: address of the static scratch");
  e = hg::run_binned_backward(h->grid, h->d, h->F, hermite, h->d2_mode, n, x, g_gamma, g_dgamma, g_d2gamma,
                              nullptr, grad_params, ptr, stream, chunk);
  if (e != hipSuccess) return hip_fail(e, "hashenc_backward_noalloc launch");
  return ok();
}

int hashenc_debug_indices(const hashenc* h, int64_t n, const float* x, int32_t order,
                          int32_t* out_rows, hashenc_stream_t stream) {
  if (!h) return fail(HASHENC_EINVAL, "hashenc_debug_indices: NULL handle");
  if (order < 0 || order >= h->n_tables) return fail(HASHENC_EINVAL, "order %d outside 0..%d", order, h->n_tables - 1);
  if (n < 0 || n > kMaxPoints) return fail(HASHENC_EINVAL, "hashenc_debug_indices: n out of range");
  if (n == 0) return ok();
  if (!x || !out_rows) return fail(HASHENC_EINVAL, "hashenc_debug_indices: NULL pointer");
  if (!aligned16(x) || !aligned16(out_rows)) return fail(HASHENC_EALIGN, "hashenc_debug_indices: pointers must be 16-byte aligned");
  Grid g = h->grid;
  g.L = g.Lrow;  // the lookup stage of every level, active or not
  hipError_t e = h->d == 4 ? hg::launch_debug_indices4(g, order, n, x, out_rows, stream)
                           : hg::launch_debug_indices(g, h->d, order, n, x, out_rows, stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_debug_indices launch");
  return ok();
}

int hashenc_diag_copy(const float* src, float* dst, int64_t n_floats, hashenc_stream_t stream) {
  if (n_floats < 0) return fail(HASHENC_EINVAL, "hashenc_diag_copy: negative size");
  if (n_floats == 0) return ok();
  if (!src || !dst) return fail(HASHENC_EINVAL, "hashenc_diag_copy: NULL pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(HASHENC_EALIGN, "hashenc_diag_copy: pointers must be 16-byte aligned");
  hipError_t e = hg::launch_copy(src, dst, n_floats, stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_diag_copy launch");
  return ok();
}

int hashenc_diag_cache_read(const float* buf, int64_t n_floats, int32_t reps, float* out,
                            hashenc_stream_t stream) {
  if (n_floats <= 0 || n_floats % hg::cache_read_granule() != 0)
    return fail(HASHENC_EINVAL, "hashenc_diag_cache_read: n_floats must be a positive multiple of 32");
  if (reps < 1) return fail(HASHENC_EINVAL, "hashenc_diag_cache_read: reps must be at least 1");
  if (!buf || !out) return fail(HASHENC_EINVAL, "hashenc_diag_cache_read: NULL pointer");
  if (!aligned16(buf)) return fail(HASHENC_EALIGN, "hashenc_diag_cache_read: buf must be 16-byte aligned");
  hipError_t e = hg::launch_cache_read(buf, n_floats, reps, out, stream);
  if (e != hipSuccess) return hip_fail(e, "hashenc_diag_cache_read launch");
  return ok();
}

}  // extern "C"
