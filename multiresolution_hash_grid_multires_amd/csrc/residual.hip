// Fused PINN residual step on the Hermite encoding, gfx950.
//
// Method: "Hermite-NGP: Gradient-Augmented Hash Encoding for Learning PDEs" notes
// (m0rtzz.github.io), key design 2: the encoding (gamma, grad gamma, Laplacian gamma from
// one Hermite pass) feeds a SIREN MLP with activation sin(omega .); because
// sin'' = -omega^2 sin, forward-mode propagation of the value, the d gradient rows and the
// Laplacian row through each layer needs only the forward intermediates:
//   z = W v + b,  Z_i = W V_i,  Z_lap = W V_lap,
//   a = sin(omega z),  A_i = omega cos(omega z) Z_i,
//   A_lap = -omega^2 sin(omega z) sum_i Z_i^2 + omega cos(omega z) Z_lap;
// loss section: the PDE residual term, here mean (Lap u - g)^2 for the Poisson problem with
// source g = -d pi^2 prod_i sin(pi x_i).
//
// Pipeline per chunk of points (workspace-backed):
//   1. Hermite forward, Laplacian mode -> gamma, grad gamma, Lap gamma   (hermite kernels)
//   2. siren_residual_kernel: one wavefront per point at a time, lane = neuron (width <= 64,
//      zero-padded), weights resident in LDS in both orientations; forward mode, residual,
//      reverse sweep; per-lane register accumulation of the lane's weight-gradient rows;
//      writes the encoder upstream and per-wave partial MLP gradients
//   3. Hermite backward with that upstream                                (hermite kernels)
//   4. reduce_partials_*: MLP gradients and the loss, summed over waves in fp64
#include <cmath>

#include "binned_backward.h"
#include "hashenc.h"
#include "hashenc_internal.h"

namespace hg {
namespace {

constexpr int kW = 64;           // padded layer width (one wavefront)
constexpr int kMaxWavesPerBlock = 8;
constexpr int kMaxDepth = 4;

struct MlpArgs {
  int32_t in, H, depth;
  int32_t ain;     // encoder inputs of the active levels (the rest are zero, coarse-to-fine)
  int32_t fshift;  // log2 F: encoder feature j is feature j % F of level j / F
  float omega;
  int64_t n_mlp;
  int64_t woff[kMaxDepth + 1], boff[kMaxDepth + 1];
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Make this wavefront's LDS writes visible to its other lanes before they read them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// sin and cos of x in fp32, within about 2 ulp for |x| <= 2^22: Cody and Waite's reduction
// x = k pi/2 + r with pi/2 split into three fp32 parts, each product k * part folded in with
// one fma; the Taylor series of sin r (through r^11) and cos r (through r^12) on |r| <= pi/4,
// whose truncation (below 1e-11) is far under fp32 rounding; then k mod 4 picks the roles
// and signs.  Beyond 2^22, where neighbouring fp32 arguments lie over 0.25 apart, r leaves
// the polynomials' range and the results are unspecified; NaN and infinity give NaN.  No
// large-argument branch and no clamp: their registers made the seven-row finite-difference
// kernel spill.  A caller that uses only one of the two results pays only for its polynomial.
__device__ __forceinline__ void sincos_red(float x, float& s, float& c) {
  constexpr float kTwoOverPi = 0x1.45f306p-1f;
  constexpr float kPio2A = 0x1.921fb6p+0f;    // pi/2 = A + B + C to about 2^-73
  constexpr float kPio2B = -0x1.777a5cp-25f;
  constexpr float kPio2C = -0x1.ee59dap-50f;
  const float k = rintf(x * kTwoOverPi);
  float r = fmaf(-k, kPio2A, x);
  r = fmaf(-k, kPio2B, r);
  r = fmaf(-k, kPio2C, r);
  const float r2 = r * r;
  float ps = fmaf(r2, -1.0f / 39916800.0f, 1.0f / 362880.0f);
  ps = fmaf(r2, ps, -1.0f / 5040.0f);
  ps = fmaf(r2, ps, 1.0f / 120.0f);
  ps = fmaf(r2, ps, -1.0f / 6.0f);
  const float sr = fmaf(r * r2, ps, r);
  float pc = fmaf(r2, 1.0f / 479001600.0f, -1.0f / 3628800.0f);
  pc = fmaf(r2, pc, 1.0f / 40320.0f);
  pc = fmaf(r2, pc, -1.0f / 720.0f);
  pc = fmaf(r2, pc, 1.0f / 24.0f);
  pc = fmaf(r2, pc, -0.5f);
  const float cr = fmaf(r2, pc, 1.0f);
  const int q = __float2int_rz(k) & 3;  // x = q pi/2 + r (mod 2 pi)
  const float sv = (q & 1) ? cr : sr;
  const float cv = (q & 1) ? sr : cr;
  s = (q & 2) ? -sv : sv;
  c = ((q + 1) & 2) ? -cv : cv;
}

// Encoder outputs and their upstream are level-major, [L][n][R][F] (R = value, d gradient
// rows, Laplacian): the index of feature j = l F + f, row r of point p.
__device__ __forceinline__ int64_t lm_index(const MlpArgs& a, int64_t n, int64_t p, int j, int r, int R) {
  const int l = j >> a.fshift, f = j & ((1 << a.fshift) - 1);
  return ((((int64_t)l * n + p) * R + r) << a.fshift) + f;
}

// Points per wavefront iteration: every LDS weight read feeds PB * R FMAs and the
// activation rows of the PB points are read as 16-byte broadcasts.
constexpr int kPB = 4;

// Wavefronts per workgroup: as many as the workgroup's LDS (mostly per-wave activation
// rows) allows within the CU's 160 KB.
__host__ __device__ constexpr int siren_waves(int depth, int inp) {
  return depth <= 2 ? 8 : (depth == 3 || inp <= 32) ? 4 : 2;
}
// Layer-0 fan-in as compiled: the encoder width rounded up to 16, 32 or 64.
constexpr int siren_inp(int in) { return in <= 16 ? 16 : in <= 32 ? 32 : 64; }

// LDS of one workgroup (a single orientation of the weights, padded to kW + 1 columns so
// that both the forward read W[lane][j] and the reverse read W[o][lane] are conflict-free).
template <int D, int DEPTH, int INP>
struct SirenLds {
  static constexpr int R = D + 2;
  static constexpr int RB = kPB * R;  // floats per activation row (PB points x R rows)
  static constexpr int WV = siren_waves(DEPTH, INP);
  float W[DEPTH][kW][kW + 1];         // W[k][o][j] = W_k[o][j]
  float bias[DEPTH][kW];
  float wout[kW];
  __attribute__((aligned(16))) float act0[WV][INP][RB];                       // layer-0 inputs
  __attribute__((aligned(16))) float act[WV][DEPTH > 1 ? DEPTH - 1 : 1][kW][RB];  // inputs of layers 1..
  __attribute__((aligned(16))) float zb[WV][kW][RB];                         // z-adjoints, reverse
};

// INP: the encoder width rounded up to 16, 32 or 64 (the first layer's fan-in).  One
// wavefront handles kPB points at a time, lane = neuron o.
template <int D, int DEPTH, int INP>
__global__ __launch_bounds__(kW * siren_waves(DEPTH, INP)) void siren_residual_kernel(
    const MlpArgs a, int64_t n, double inv_n_total, const float* __restrict__ x,
    const float* __restrict__ enc, const float* __restrict__ mlp, float* __restrict__ up,
    float* __restrict__ residual, float* __restrict__ partial) {
  using Sh = SirenLds<D, DEPTH, INP>;
  constexpr int R = Sh::R;
  constexpr int RB = Sh::RB;
  constexpr int WV = Sh::WV;
  static_assert(sizeof(Sh) <= 160 * 1024, "SIREN workgroup LDS exceeds the CU's 160 KB");
  __shared__ Sh sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kW - 1);
  const int wv = tid / kW;
  const float w = a.omega;

  for (int k = 0; k < DEPTH; ++k) {
    const int fi = k == 0 ? a.in : a.H;
    const float* Wk = mlp + a.woff[k];
    for (int e = tid; e < kW * kW; e += kW * WV) {
      const int o = e / kW, j = e % kW;
      sh.W[k][o][j] = (o < a.H && j < fi) ? Wk[o * fi + j] : 0.0f;
    }
    for (int o = tid; o < kW; o += kW * WV) sh.bias[k][o] = o < a.H ? mlp[a.boff[k] + o] : 0.0f;
  }
  for (int o = tid; o < kW; o += kW * WV) sh.wout[o] = o < a.H ? mlp[a.woff[DEPTH] + o] : 0.0f;
  __syncthreads();

  // lane o: row o of dL/dW_k (layer 0 has INP columns, the others kW)
  float gW0[INP];
  float gW[DEPTH > 1 ? DEPTH - 1 : 1][kW];
  float gb[DEPTH];
  float gWo = 0.0f, sq = 0.0f;
#pragma unroll
  for (int j = 0; j < INP; ++j) gW0[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) gb[k] = 0.0f;
#pragma unroll
  for (int k = 0; k + 1 < DEPTH; ++k)
#pragma unroll
    for (int j = 0; j < kW; ++j) gW[k][j] = 0.0f;

  auto in_row = [&](int k, int j) -> float* { return k == 0 ? sh.act0[wv][j] : sh.act[wv][k - 1][j]; };

  const int64_t wave_id = (int64_t)blockIdx.x * WV + wv;
  const int64_t n_waves = (int64_t)gridDim.x * WV;
  for (int64_t p0 = wave_id * kPB; p0 < n; p0 += n_waves * kPB) {
    // encoder outputs of points p0 .. p0 + kPB - 1 -> layer-0 input rows (lane j = column)
    if (lane < INP) {
      float row[RB];
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const int64_t p = p0 + b;
        const bool on = lane < a.ain && p < n;
#pragma unroll
        for (int r = 0; r < R; ++r) row[b * R + r] = on ? enc[lm_index(a, n, p, lane, r, R)] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < RB; q += 4)
        *reinterpret_cast<float4*>(&sh.act0[wv][lane][q]) = make_float4(row[q], row[q + 1], row[q + 2], row[q + 3]);
    }
    wave_lds_sync();

    // forward mode through the hidden layers
    float ts[DEPTH][kPB], tc[DEPTH][kPB], tz[DEPTH][kPB][R];  // tape: sin, cos, Z rows
    float a_lap_top[kPB];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      const int fi = k == 0 ? INP : kW;
      float z[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) z[q] = (q % R == 0) ? sh.bias[k][lane] : 0.0f;
#pragma unroll 4
      for (int j = 0; j < fi; ++j) {
        const float wj = sh.W[k][lane][j];
        const float* v = in_row(k, j);
#pragma unroll
        for (int q = 0; q < RB; q += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(v + q);
          z[q] = fmaf(wj, a4.x, z[q]);
          z[q + 1] = fmaf(wj, a4.y, z[q + 1]);
          z[q + 2] = fmaf(wj, a4.z, z[q + 2]);
          z[q + 3] = fmaf(wj, a4.w, z[q + 3]);
        }
      }
      float out[RB];
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const float* zz = z + b * R;
        float s, c;
        sincos_red(w * zz[0], s, c);
        ts[k][b] = s;
        tc[k][b] = c;
        float sumsq = 0.0f;
#pragma unroll
        for (int i = 1; i <= D; ++i) sumsq = fmaf(zz[i], zz[i], sumsq);
#pragma unroll
        for (int r = 0; r < R; ++r) tz[k][b][r] = zz[r];
        const float wc = w * c;
        const float a_lap = fmaf(-w * w * s, sumsq, wc * zz[R - 1]);
        out[b * R] = s;
#pragma unroll
        for (int i = 1; i <= D; ++i) out[b * R + i] = wc * zz[i];
        out[b * R + R - 1] = a_lap;
        a_lap_top[b] = a_lap;
      }
      if (k + 1 < DEPTH) {
#pragma unroll
        for (int q = 0; q < RB; q += 4)
          *reinterpret_cast<float4*>(&sh.act[wv][k][lane][q]) = make_float4(out[q], out[q + 1], out[q + 2], out[q + 3]);
        wave_lds_sync();
      }
    }
    // linear output: Lap u = wout . A_lap; residual and seed per point
    float seed[kPB];
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
      const int64_t p = p0 + b;
      const float lap_u = wave_sum(sh.wout[lane] * a_lap_top[b]);
      float res = 0.0f;
      if (p < n) {
        float src = -(float)D * 9.8696044010893586f;  // -d pi^2
#pragma unroll
        for (int i = 0; i < D; ++i) src *= sinpif(x[p * D + i]);
        res = lap_u - src;
        if (lane == 0) {
          sq = fmaf(res, res, sq);
          if (residual) residual[p] = res;
        }
      }
      seed[b] = (float)(2.0 * (double)res * inv_n_total);
      gWo = fmaf(seed[b], a_lap_top[b], gWo);
    }

    // reverse sweep; the output layer seeds only the Laplacian rows
    float ab[RB];
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
#pragma unroll
      for (int r = 0; r < R; ++r) ab[b * R + r] = 0.0f;
      ab[b * R + R - 1] = seed[b] * sh.wout[lane];
    }
#pragma unroll
    for (int k = DEPTH - 1; k >= 0; --k) {
      float zbar[RB];
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const float s = ts[k][b], c = tc[k][b];
        const float wc = w * c, w2s = w * w * s;
        const float* zz = tz[k][b];
        const float* aa = ab + b * R;
        float sumsq = 0.0f;
#pragma unroll
        for (int i = 1; i <= D; ++i) sumsq = fmaf(zz[i], zz[i], sumsq);
        // d a/dz = w cos; d A_i/dz = -w^2 sin Z_i; d A_lap/dz = -w^3 cos sum Z_i^2 - w^2 sin Z_lap
        float z0 = aa[0] * wc + aa[R - 1] * (-w * w * wc * sumsq - w2s * zz[R - 1]);
#pragma unroll
        for (int i = 1; i <= D; ++i) {
          z0 = fmaf(aa[i], -w2s * zz[i], z0);
          // d A_i/dZ_i = w cos; d A_lap/dZ_i = -2 w^2 sin Z_i
          zbar[b * R + i] = aa[i] * wc + aa[R - 1] * (-2.0f * w2s * zz[i]);
        }
        zbar[b * R] = z0;
        zbar[b * R + R - 1] = aa[R - 1] * wc;  // d A_lap/dZ_lap = w cos
        gb[k] += z0;
      }
      // dL/dW_k row `lane` += sum over points and rows of zbar * input row
      if (k == 0) {
#pragma unroll
        for (int j = 0; j < INP; ++j) {
          const float* v = sh.act0[wv][j];
          float acc = gW0[j];
#pragma unroll
          for (int q = 0; q < RB; q += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(v + q);
            acc = fmaf(zbar[q], a4.x, acc);
            acc = fmaf(zbar[q + 1], a4.y, acc);
            acc = fmaf(zbar[q + 2], a4.z, acc);
            acc = fmaf(zbar[q + 3], a4.w, acc);
          }
          gW0[j] = acc;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kW; ++j) {
          const float* v = sh.act[wv][k - 1][j];
          float acc = gW[k - 1][j];
#pragma unroll
          for (int q = 0; q < RB; q += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(v + q);
            acc = fmaf(zbar[q], a4.x, acc);
            acc = fmaf(zbar[q + 1], a4.y, acc);
            acc = fmaf(zbar[q + 2], a4.z, acc);
            acc = fmaf(zbar[q + 3], a4.w, acc);
          }
          gW[k - 1][j] = acc;
        }
      }
      // input adjoint: lane j <- sum_o W_k[o][j] zbar_o
#pragma unroll
      for (int q = 0; q < RB; q += 4)
        *reinterpret_cast<float4*>(&sh.zb[wv][lane][q]) = make_float4(zbar[q], zbar[q + 1], zbar[q + 2], zbar[q + 3]);
      wave_lds_sync();
#pragma unroll
      for (int q = 0; q < RB; ++q) ab[q] = 0.0f;
#pragma unroll 4
      for (int o = 0; o < kW; ++o) {
        const float wo = sh.W[k][o][lane];
        const float* zr = sh.zb[wv][o];
#pragma unroll
        for (int q = 0; q < RB; q += 4) {
          const float4 z4 = *reinterpret_cast<const float4*>(zr + q);
          ab[q] = fmaf(wo, z4.x, ab[q]);
          ab[q + 1] = fmaf(wo, z4.y, ab[q + 1]);
          ab[q + 2] = fmaf(wo, z4.z, ab[q + 2]);
          ab[q + 3] = fmaf(wo, z4.w, ab[q + 3]);
        }
      }
      wave_lds_sync();  // zb is rewritten by the next layer
    }
    if (lane < a.ain) {
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const int64_t p = p0 + b;
        if (p >= n) break;
#pragma unroll
        for (int r = 0; r < R; ++r) up[lm_index(a, n, p, lane, r, R)] = ab[b * R + r];
      }
    }
  }

  // this wave's partial MLP gradient and sum of r^2
  float* part = partial + wave_id * (a.n_mlp + 1);
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) {
    const int fi = k == 0 ? a.in : a.H;
    if (lane < a.H) {
      if (k == 0) {
#pragma unroll
        for (int j = 0; j < INP; ++j)
          if (j < fi) part[a.woff[0] + (int64_t)lane * fi + j] = gW0[j];
      } else {
#pragma unroll
        for (int j = 0; j < kW; ++j)
          if (j < fi) part[a.woff[k] + (int64_t)lane * fi + j] = gW[k - 1][j];
      }
      part[a.boff[k] + lane] = gb[k];
    }
  }
  if (lane < a.H) part[a.woff[DEPTH] + lane] = gWo;
  if (lane == 0) {
    part[a.boff[DEPTH]] = 0.0f;  // the output bias does not enter Lap u
    part[a.n_mlp] = sq;
  }
}

// ---------------------------------------------------------------------------------------
// Matrix-core formulation for SIREN depth <= 2.  A workgroup of 4 wavefronts takes 16 points
// per iteration; the columns of every layer's matrices are (row kind r, point p), c = 16 r + p,
// r over value, d gradients, Laplacian.  Wavefront w owns neurons 16w..16w+15 on the output
// side of each product.  The three products per layer run on v_mfma_f32_16x16x4_f32
// (lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]; D[4 (l / 16) + i][l % 16] in
// register i):
//   forward          Z_k = W_k V_k (+ b_k on the value rows)   A = W_k rows (registers),
//                                                             B = V_k from LDS
//   input adjoint    Vbar_k = W_k^T Zbar_k                   A = W_k columns (registers),
//                                                             B = Zbar_k from LDS
//   weight gradient  dL/dW_k += Zbar_k V_k^T (over columns)  A = Zbar_k, B = V_k, both read
//                                                             from LDS transposed; the
//                                                             accumulator lives across
//                                                             iterations
// The elementwise forward-mode activation and its reverse are lane-local: a lane's D registers
// hold the same (neuron, point) for every row kind.  Layer inputs V_k and the z-adjoints are
// exchanged through LDS as [row][column] matrices (pitch kMPitch, bank-conflict-free for both
// access patterns); the Z tape of a wavefront's own neurons stays in registers.
typedef float mf4 __attribute__((ext_vector_type(4)));
constexpr int kMP = 16;      // points per workgroup iteration
constexpr int kMWaves = 4;   // wavefronts per workgroup (kW / 16 neuron tiles)
constexpr int kMPitch = 84;  // LDS row pitch in floats (columns: 16 * (d + 2) <= 80)
constexpr int kMfmaBlocks = 512;  // two resident workgroups per CU, all in one round

template <int D, int DEPTH, int NI>
struct MfmaLds {
  float w0[kW][NI + 4];                               // W_0 (padded rows)
  float w1[DEPTH > 1 ? DEPTH - 1 : 1][kW][kW + 4];    // W_1 .. W_{DEPTH-1}
  float act0[NI][kMPitch];                            // V_0: encoder rows
  float act1[DEPTH > 1 ? DEPTH - 1 : 1][kW][kMPitch]; // V_1 ..: the hidden layers' inputs
  float zb[kW][kMPitch];                              // Zbar of the layer in reverse
  float lapw[kMWaves][kMP];                           // per-wave partial Laplacians
};

__device__ __forceinline__ mf4 mfma16(float a, float b, mf4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The matrix-core runs of the SIREN kernels are issued at raised wavefront priority (the
// instruction arbiter's, per wave): of the two wavefronts on a SIMD, the one in a run of
// MFMAs keeps the matrix core fed while the other does its LDS and VALU work.
__device__ __forceinline__ void mfma_prio_hi() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_prio_lo() { __builtin_amdgcn_s_setprio(0); }

template <int D, int DEPTH, int NI>
__global__ __launch_bounds__(kW * kMWaves, (DEPTH <= 2 ? 2 : 1)) void siren_mfma_kernel(
    const MlpArgs a, int64_t n, double inv_n_total, const float* __restrict__ x,
    const float* __restrict__ enc, const float* __restrict__ mlp, float* __restrict__ up,
    float* __restrict__ residual, float* __restrict__ partial) {
  static_assert(DEPTH >= 1 && DEPTH <= 4, "matrix-core SIREN covers one to four hidden layers");
  constexpr int R = D + 2;
  constexpr int NC = kMP * R;  // columns
  __shared__ MfmaLds<D, DEPTH, NI> sh;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lm = lane & 15, lq = lane >> 4;
  const int H = a.H;
  const float om = a.omega;

  // weights into LDS, zero-padded to the compiled widths; the forward reads W_k[16w + lm][4kk + lq]
  // (conflict-free with rows padded by 4 floats), the input adjoint W_k[4kk + lq][16w + lm]
  for (int e = threadIdx.x; e < kW * NI; e += kW * kMWaves) {
    const int o = e / NI, j = e % NI;
    sh.w0[o][j] = (o < H && j < a.in) ? mlp[a.woff[0] + o * a.in + j] : 0.0f;
  }
#pragma unroll
  for (int k = 1; k < DEPTH; ++k)
    for (int e = threadIdx.x; e < kW * kW; e += kW * kMWaves) {
      const int o = e / kW, j = e % kW;
      sh.w1[k - 1][o][j] = (o < H && j < H) ? mlp[a.woff[k] + o * H + j] : 0.0f;
    }
  // per-lane neurons in D layout: o = 16w + 4lq + i
  float bias[DEPTH][4], wout[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 16 * w + 4 * lq + i;
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) bias[k][i] = o < H ? mlp[a.boff[k] + o] : 0.0f;
    wout[i] = o < H ? mlp[a.woff[DEPTH] + o] : 0.0f;
  }
  mf4 gW0[NI / 16];
  mf4 gW1[DEPTH > 1 ? DEPTH - 1 : 1][4];
#pragma unroll
  for (int t = 0; t < NI / 16; ++t) gW0[t] = mf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < (DEPTH > 1 ? DEPTH - 1 : 1); ++k)
#pragma unroll
    for (int t = 0; t < 4; ++t) gW1[k][t] = mf4{0.f, 0.f, 0.f, 0.f};
  float gb[DEPTH][4], gWo[4], sq = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gWo[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) gb[k][i] = 0.0f;
  }

  // Encoder rows -> V_0[j][16 r + p]: element e of an iteration's rows, walked level by level
  // (the 16 points' R rows of F features of one level are contiguous in the level-major
  // encoder output), goes to thread e % T.  The next iteration's rows are loaded into
  // registers right after this iteration's are parked in LDS, so their memory latency hides
  // behind the iteration's products instead of stalling its start.
  constexpr int T = kW * kMWaves;
  constexpr int EPT = kMP * R * NI / T;
  static_assert(kMP * R * NI % T == 0, "encoder rows split evenly over the workgroup");
  // Byte offsets from the iteration's first row are 32-bit (one chunk's encoder output is
  // below 4 GiB, checked at launch): one offset register per load from a uniform base.
  const uint32_t level_bytes = (uint32_t)(((uint64_t)n * R << a.fshift) * sizeof(float));
  auto rows_load = [&](int64_t q0, float (&ev)[EPT]) {
    const char* base = reinterpret_cast<const char*>(enc + ((q0 * R) << a.fshift));
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = threadIdx.x + u * T;
      const int f = e & ((1 << a.fshift) - 1), t = e >> a.fshift;
      const int t2 = t / R;
      const int p = t2 % kMP, l = t2 / kMP;
      const int j = (l << a.fshift) + f;
      const uint32_t off = (uint32_t)l * level_bytes + (uint32_t)(e - ((l * kMP * R) << a.fshift)) * 4u;
      ev[u] = (j < a.ain && q0 + p < n) ? *reinterpret_cast<const float*>(base + off) : 0.0f;
    }
  };
  auto rows_park = [&](const float (&ev)[EPT]) {
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = threadIdx.x + u * T;
      const int f = e & ((1 << a.fshift) - 1), t = e >> a.fshift;
      const int r = t % R, t2 = t / R;
      const int p = t2 % kMP, l = t2 / kMP;
      sh.act0[(l << a.fshift) + f][r * kMP + p] = ev[u];
    }
  };
  const int64_t n_iter = (n + kMP - 1) / kMP;
  float ev[EPT];
  if (blockIdx.x < n_iter) rows_load((int64_t)blockIdx.x * kMP, ev);
  for (int64_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
    const int64_t p0 = it * kMP;
    rows_park(ev);
    __syncthreads();
    // this iteration's coordinates (the source term), used after the forward
    const int64_t pp = p0 + lm;
    float xs[D];
#pragma unroll
    for (int i = 0; i < D; ++i) xs[i] = pp < n ? x[pp * D + i] : 0.0f;

    // forward mode
    mf4 z[DEPTH][R];  // tape: the wavefront's neurons
    float sn[DEPTH][4], cs[DEPTH][4];  // sin and cos of omega z, reused by the reverse sweep
    float alap[4];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      mf4 acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = mf4{0.f, 0.f, 0.f, 0.f};
      mfma_prio_hi();
      if (k == 0) {
#pragma unroll
        for (int kk = 0; kk < NI / 4; ++kk) {
          const float aw = sh.w0[16 * w + lm][4 * kk + lq];
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] = mfma16(aw, sh.act0[4 * kk + lq][r * kMP + lm], acc[r]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float aw = sh.w1[k - 1][16 * w + lm][4 * kk + lq];
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r] = mfma16(aw, sh.act1[k - 1][4 * kk + lq][r * kMP + lm], acc[r]);
        }
      }
      mfma_prio_lo();
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[0][i] += bias[k][i];
#pragma unroll
      for (int r = 0; r < R; ++r) z[k][r] = acc[r];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s, c;
        sincos_red(om * acc[0][i], s, c);
        sn[k][i] = s;
        cs[k][i] = c;
        float sumsq = 0.0f;
#pragma unroll
        for (int r = 1; r <= D; ++r) sumsq = fmaf(acc[r][i], acc[r][i], sumsq);
        const float wc = om * c;
        const float a_lap = fmaf(-om * om * s, sumsq, wc * acc[R - 1][i]);
        if (k + 1 < DEPTH) {
          const int o = 16 * w + 4 * lq + i;
          sh.act1[k][o][lm] = s;
#pragma unroll
          for (int r = 1; r <= D; ++r) sh.act1[k][o][r * kMP + lm] = wc * acc[r][i];
          sh.act1[k][o][(R - 1) * kMP + lm] = a_lap;
        } else {
          alap[i] = a_lap;
        }
      }
      if (k + 1 < DEPTH) __syncthreads();
    }
    // linear output: Lap u = wout . A_lap (sum over the 64 neurons of 4 wavefronts)
    {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(wout[i], alap[i], part);
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (lq == 0) sh.lapw[w][lm] = part;
    }
    __syncthreads();
    float seed = 0.0f;
    if (pp < n) {
      float lap_u = 0.0f;
#pragma unroll
      for (int v = 0; v < kMWaves; ++v) lap_u += sh.lapw[v][lm];
      float src = -(float)D * 9.8696044010893586f;  // -d pi^2
#pragma unroll
      for (int i = 0; i < D; ++i) src *= sinpif(xs[i]);
      const float res = lap_u - src;
      if (w == 0 && lq == 0) {
        sq = fmaf(res, res, sq);
        if (residual) residual[pp] = res;
      }
      seed = (float)(2.0 * (double)res * inv_n_total);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) gWo[i] = fmaf(seed, alap[i], gWo[i]);

    // reverse sweep, top layer down; abar: adjoint of the layer's output rows (D layout)
    mf4 abar[R];
#pragma unroll
    for (int r = 0; r < R; ++r) abar[r] = mf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) abar[R - 1][i] = seed * wout[i];
#pragma unroll
    for (int k = DEPTH - 1; k >= 0; --k) {
      // the next iteration's encoder rows, issued where the tape of the upper layer is dead
      if (k == 0 && it + gridDim.x < n_iter) rows_load((it + gridDim.x) * kMP, ev);
      mf4 zbar[R];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sn[k][i], c = cs[k][i];
        const float wc = om * c, w2s = om * om * s;
        float sumsq = 0.0f;
#pragma unroll
        for (int r = 1; r <= D; ++r) sumsq = fmaf(z[k][r][i], z[k][r][i], sumsq);
        const float al = abar[R - 1][i];
        // d a/dz = w cos; d A_i/dz = -w^2 sin Z_i; d A_lap/dz = -w^3 cos sum Z_i^2 - w^2 sin Z_lap
        float z0 = abar[0][i] * wc + al * (-om * om * wc * sumsq - w2s * z[k][R - 1][i]);
#pragma unroll
        for (int r = 1; r <= D; ++r) {
          z0 = fmaf(abar[r][i], -w2s * z[k][r][i], z0);
          // d A_i/dZ_i = w cos; d A_lap/dZ_i = -2 w^2 sin Z_i
          zbar[r][i] = abar[r][i] * wc + al * (-2.0f * w2s * z[k][r][i]);
        }
        zbar[0][i] = z0;
        zbar[R - 1][i] = al * wc;  // d A_lap/dZ_lap = w cos
        gb[k][i] += z0;
        const int o = 16 * w + 4 * lq + i;
#pragma unroll
        for (int r = 0; r < R; ++r) sh.zb[o][r * kMP + lm] = zbar[r][i];
      }
      __syncthreads();
      // weight gradient: dL/dW_k[16w + .][j] += sum_c Zbar[o][c] V_k[j][c]
      mfma_prio_hi();
#pragma unroll
      for (int kk = 0; kk < NC / 4; ++kk) {
        const float az = sh.zb[16 * w + lm][4 * kk + lq];
        if (k == 0) {
#pragma unroll
          for (int t = 0; t < NI / 16; ++t) gW0[t] = mfma16(az, sh.act0[16 * t + lm][4 * kk + lq], gW0[t]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) gW1[k - 1][t] = mfma16(az, sh.act1[k - 1][16 * t + lm][4 * kk + lq], gW1[k - 1][t]);
        }
      }
      mfma_prio_lo();
      if (k > 0) {
        // input adjoint for the wavefront's tile of input neurons j = 16w + .
        mf4 vbar[R];
#pragma unroll
        for (int r = 0; r < R; ++r) vbar[r] = mf4{0.f, 0.f, 0.f, 0.f};
        mfma_prio_hi();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float aw = sh.w1[k - 1][4 * kk + lq][16 * w + lm];
#pragma unroll
          for (int r = 0; r < R; ++r) vbar[r] = mfma16(aw, sh.zb[4 * kk + lq][r * kMP + lm], vbar[r]);
        }
        mfma_prio_lo();
        __syncthreads();  // zb and the layer's inputs are rewritten next
#pragma unroll
        for (int r = 0; r < R; ++r) abar[r] = vbar[r];
      } else {
        // encoder upstream: the NI / 16 tiles of input neurons times the R row kinds, dealt
        // round-robin over the wavefronts (with NI = 32 two wavefronts would otherwise carry
        // all of it while the other two wait at the barrier), each stored as soon as it is
        // done: inputs j = 16 jt + 4 lq + i of point pp (the encoder output's layout, 32-bit
        // byte offsets from the iteration's first row)
        constexpr int NT = NI / 16;
        char* ubase = reinterpret_cast<char*>(up + ((p0 * R) << a.fshift));
        for (int T = w; T < NT * R; T += kMWaves) {
          const int jt = T % NT, r = T / NT;
          mf4 acc = mf4{0.f, 0.f, 0.f, 0.f};
          mfma_prio_hi();
#pragma unroll
          for (int kk = 0; kk < 16; ++kk)
            acc = mfma16(sh.w0[4 * kk + lq][16 * jt + lm], sh.zb[4 * kk + lq][r * kMP + lm], acc);
          mfma_prio_lo();
          if (pp < n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 16 * jt + 4 * lq + i;
              if (j < a.ain) {
                const int l = j >> a.fshift, f = j & ((1 << a.fshift) - 1);
                const uint32_t off = (uint32_t)l * level_bytes + (uint32_t)(((lm * R) << a.fshift) + f) * 4u;
                *reinterpret_cast<float*>(ubase + off + ((uint32_t)r << a.fshift) * 4u) = acc[i];
              }
            }
          }
        }
        __syncthreads();  // zb and the layer's inputs are rewritten next
      }
    }
  }

  // this workgroup's partial MLP gradient and sum of r^2
  float* part = partial + (int64_t)blockIdx.x * (a.n_mlp + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 16 * w + 4 * lq + i;
    if (o < H) {
#pragma unroll
      for (int t = 0; t < NI / 16; ++t) {
        const int j = 16 * t + lm;
        if (j < a.in) part[a.woff[0] + (int64_t)o * a.in + j] = gW0[t][i];
      }
#pragma unroll
      for (int k = 1; k < DEPTH; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = 16 * t + lm;
          if (j < H) part[a.woff[k] + (int64_t)o * H + j] = gW1[k - 1][t][i];
        }
    }
  }
  // bias and output-weight gradients: sum over the 16 points (lanes lm) of each lane group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[DEPTH + 1];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) v[k] = gb[k][i];
    v[DEPTH] = gWo[i];
#pragma unroll
    for (int k = 0; k <= DEPTH; ++k)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v[k] += __shfl_xor(v[k], off, 64);
    const int o = 16 * w + 4 * lq + i;
    if (lm == 0 && o < H) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) part[a.boff[k] + o] = v[k];
      part[a.woff[DEPTH] + o] = v[DEPTH];
    }
  }
  if (w == 0) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sq += __shfl_xor(sq, off, 64);
    if (lane == 0) {
      part[a.boff[DEPTH]] = 0.0f;  // the output bias does not enter Lap u
      part[a.n_mlp] = sq;
    }
  }
}

// ---------------------------------------------------------------------------------------
// INGP-FD comparator (Hermite-NGP notes, the 现有痛点 paragraph: the Laplacian of an
// Instant-NGP encoding + network by central differences, 2d+1 forward passes).  The same
// matrix-core layout as above, but the R = 2d+1 column groups are the stencil points
// x, x + eps e_i, x - eps e_i of each of the 16 points (s = 0, 2i+1, 2i+2), each a plain value
// row with its own nonlinearity:
//   forward   z_s = W v_s + b,  a_s = sin(omega z_s),  u_s = Wo a_s + bo
//   FD        Lap u = sum_i (u_{2i+1} - 2 u_0 + u_{2i+2}) / eps^2,  r = Lap u - g(x)
//   reverse   ubar_s = (2 r / n) c_s (c_0 = -2d / eps^2, else 1 / eps^2),
//             zbar_s = abar_s omega cos(omega z_s),  vbar_s = W^T zbar_s
// A point's 2d+1 stencil copies share their cells on all but the finest levels.  The forward
// runs them point-major (copies on neighbouring lanes share the gathers' cache lines), so the
// encoder rows arrive in lm_index's layout with R = 2d+1; the upstream goes out
// stencil-major, [L][2d+1][n][F], and the backward runs on the stencil-major copy of the
// point sets, which keeps a point's copies out of one wavefront (no same-row conflicts in the
// reduction's LDS accumulation).
constexpr int fd_pitch(int D) { return kMP * (2 * D + 1) + 4; }

__device__ __forceinline__ int64_t fd_index(const MlpArgs& a, int64_t n, int64_t p, int j, int r, int R) {
  const int l = j >> a.fshift, f = j & ((1 << a.fshift) - 1);
  return ((((int64_t)l * R + r) * n + p) << a.fshift) + f;
}

template <int D, int DEPTH, int NI>
struct FdLds {
  float w0[kW][NI + 4];
  float w1[DEPTH > 1 ? kW : 1][kW + 4];
  float act0[NI][fd_pitch(D)];                        // V_0: encoder rows of the stencil points
  float act1[DEPTH > 1 ? kW : 1][fd_pitch(D)];        // V_1
  float zb[kW][fd_pitch(D)];                          // Zbar of the layer in reverse
  float uw[kMWaves][2 * D + 1][kMP];                  // per-wave partial u of each stencil point
};

// Two row groups of four wavefronts: wavefront w owns neurons 16 (w % 4) .. + 15 for the
// stencil rows of group w / 4 (rows 0..3 and 4..2d), so each wavefront carries about half the
// rows' tape and accumulators and two wavefronts share every SIMD.  Every row group writes its
// own partial-gradient row.
constexpr int kFdGroups = 2;
constexpr int kFdWaves = kMWaves * kFdGroups;

template <int D, int DEPTH, int NI>
__global__ __launch_bounds__(kW * kFdWaves) void siren_fd_mfma_kernel(
    const MlpArgs a, int64_t n, double inv_n_total, float inv_eps2, const float* __restrict__ x,
    const float* __restrict__ enc, const float* __restrict__ mlp, float* __restrict__ up,
    float* __restrict__ u_stencil, float* __restrict__ residual, float* __restrict__ partial) {
  static_assert(DEPTH == 1 || DEPTH == 2, "matrix-core SIREN covers one or two hidden layers");
  constexpr int R = 2 * D + 1;
  constexpr int RG = (R + kFdGroups - 1) / kFdGroups;  // rows per group (the last may have fewer)
  static_assert(sizeof(FdLds<D, DEPTH, NI>) <= 160 * 1024, "FD SIREN workgroup LDS exceeds the CU's 160 KB");
  __shared__ FdLds<D, DEPTH, NI> sh;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wn = w & (kMWaves - 1), rg = w / kMWaves;  // neuron tile, row group
  const int r0 = rg * RG;                              // first row of the group
  const int lm = lane & 15, lq = lane >> 4;
  const int H = a.H;
  const float om = a.omega;

  for (int e = threadIdx.x; e < kW * NI; e += kW * kFdWaves) {
    const int o = e / NI, j = e % NI;
    sh.w0[o][j] = (o < H && j < a.in) ? mlp[a.woff[0] + o * a.in + j] : 0.0f;
  }
  if constexpr (DEPTH > 1) {
    for (int e = threadIdx.x; e < kW * kW; e += kW * kFdWaves) {
      const int o = e / kW, j = e % kW;
      sh.w1[o][j] = (o < H && j < H) ? mlp[a.woff[1] + o * H + j] : 0.0f;
    }
  }
  float bias[DEPTH][4], wout[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 16 * wn + 4 * lq + i;
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) bias[k][i] = o < H ? mlp[a.boff[k] + o] : 0.0f;
    wout[i] = o < H ? mlp[a.woff[DEPTH] + o] : 0.0f;
  }
  const float bo = mlp[a.boff[DEPTH]];
  mf4 gW0[NI / 16];
  mf4 gW1[DEPTH > 1 ? 4 : 1];
#pragma unroll
  for (int t = 0; t < NI / 16; ++t) gW0[t] = mf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < (DEPTH > 1 ? 4 : 1); ++t) gW1[t] = mf4{0.f, 0.f, 0.f, 0.f};
  float gb[DEPTH][4], gWo[4], sq = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gWo[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) gb[k][i] = 0.0f;
  }

  // Encoder rows of the stencil points, walked level by level (the 16 points' R stencil rows
  // of F features are contiguous): element e to thread e % T.  The next iteration's rows are
  // loaded into registers during this iteration's reverse sweep, so their latency hides
  // behind its products.  Byte offsets from the iteration's first row are 32-bit
  // (one chunk's encoder output is below 4 GiB, checked at launch).
  constexpr int T = kW * kFdWaves;
  constexpr int TOT = kMP * R * NI;
  constexpr int EPT = (TOT + T - 1) / T;
  const uint32_t level_bytes = (uint32_t)(((uint64_t)n * R << a.fshift) * sizeof(float));
  auto rows_load = [&](int64_t q0, float (&ev)[EPT]) {
    const char* base = reinterpret_cast<const char*>(enc + ((q0 * R) << a.fshift));
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = threadIdx.x + u * T;
      const int f = e & ((1 << a.fshift) - 1), t = e >> a.fshift;
      const int t2 = t / R;
      const int p = t2 % kMP, l = t2 / kMP;
      const int j = (l << a.fshift) + f;
      const uint32_t off = (uint32_t)l * level_bytes + (uint32_t)(e - ((l * kMP * R) << a.fshift)) * 4u;
      ev[u] = (e < TOT && j < a.ain && q0 + p < n) ? *reinterpret_cast<const float*>(base + off) : 0.0f;
    }
  };
  auto rows_park = [&](const float (&ev)[EPT]) {
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = threadIdx.x + u * T;
      const int f = e & ((1 << a.fshift) - 1), t = e >> a.fshift;
      const int r = t % R, t2 = t / R;
      const int p = t2 % kMP, l = t2 / kMP;
      if (e < TOT) sh.act0[(l << a.fshift) + f][r * kMP + p] = ev[u];
    }
  };
  const int64_t n_iter = (n + kMP - 1) / kMP;
  float ev[EPT];
  if (blockIdx.x < n_iter) rows_load((int64_t)blockIdx.x * kMP, ev);
  for (int64_t it = blockIdx.x; it < n_iter; it += gridDim.x) {
    const int64_t p0 = it * kMP;
    rows_park(ev);
    __syncthreads();
    // this iteration's coordinates (the source term), used after the forward
    const int64_t pp = p0 + lm;
    float xs[D];
#pragma unroll
    for (int i = 0; i < D; ++i) xs[i] = pp < n ? x[pp * D + i] : 0.0f;

    // forward: every column group is a value row; layers as compile-time steps so the tape
    // stays in registers
    mf4 z[DEPTH][RG];
    mf4 atop[RG];
    auto fwd_layer = [&]<int K>() {
      mf4 acc[RG];
#pragma unroll
      for (int rr = 0; rr < RG; ++rr) acc[rr] = mf4{0.f, 0.f, 0.f, 0.f};
      mfma_prio_hi();
      if constexpr (K == 0) {
#pragma unroll
        for (int kk = 0; kk < NI / 4; ++kk) {
          const float aw = sh.w0[16 * wn + lm][4 * kk + lq];
#pragma unroll
          for (int rr = 0; rr < RG; ++rr)
            if (r0 + rr < R) acc[rr] = mfma16(aw, sh.act0[4 * kk + lq][(r0 + rr) * kMP + lm], acc[rr]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float aw = sh.w1[16 * wn + lm][4 * kk + lq];
#pragma unroll
          for (int rr = 0; rr < RG; ++rr)
            if (r0 + rr < R) acc[rr] = mfma16(aw, sh.act1[4 * kk + lq][(r0 + rr) * kMP + lm], acc[rr]);
        }
      }
      mfma_prio_lo();
#pragma unroll
      for (int rr = 0; rr < RG; ++rr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rr][i] += bias[K][i];
        z[K][rr] = acc[rr];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 16 * wn + 4 * lq + i;
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
          float sv, cv_unused;
          sincos_red(om * acc[rr][i], sv, cv_unused);
          if constexpr (K + 1 < DEPTH) {
            if (r0 + rr < R) sh.act1[o][(r0 + rr) * kMP + lm] = sv;
          } else {
            atop[rr][i] = sv;
          }
        }
      }
      if constexpr (K + 1 < DEPTH) __syncthreads();
    };
    fwd_layer.template operator()<0>();
    if constexpr (DEPTH > 1) fwd_layer.template operator()<1>();

    // u_s = wout . a_s (+ bo): partial sums over the wavefront's 16 neurons, then over waves
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(wout[i], atop[rr][i], part);
      part += __shfl_xor(part, 16, 64);
      part += __shfl_xor(part, 32, 64);
      if (lq == 0 && r0 + rr < R) sh.uw[wn][r0 + rr][lm] = part;
    }
    __syncthreads();
    float seed = 0.0f;
    if (pp < n) {
      float u0 = 0.0f, lap = 0.0f;  // the output bias cancels in every second difference
#pragma unroll
      for (int q = 0; q < kMWaves; ++q) u0 += sh.uw[q][0][lm];
#pragma unroll
      for (int i = 0; i < D; ++i) {
        float up1 = 0.0f, um1 = 0.0f;
#pragma unroll
        for (int q = 0; q < kMWaves; ++q) {
          up1 += sh.uw[q][2 * i + 1][lm];
          um1 += sh.uw[q][2 * i + 2][lm];
        }
        // (u+ - u0) + (u- - u0): for a step small enough that the stencil values lie within
        // a factor 2 of u0 both differences are exact in fp32 (Sterbenz), so only the last
        // addition rounds, relative to the second difference itself
        lap += ((up1 - u0) + (um1 - u0)) * inv_eps2;
        if (u_stencil && w == 0 && lq == 0) {
          u_stencil[pp * R + 2 * i + 1] = up1 + bo;
          u_stencil[pp * R + 2 * i + 2] = um1 + bo;
        }
      }
      float src = -(float)D * 9.8696044010893586f;  // -d pi^2
#pragma unroll
      for (int i = 0; i < D; ++i) src *= sinpif(xs[i]);
      const float res = lap - src;
      if (w == 0 && lq == 0) {
        sq = fmaf(res, res, sq);
        if (residual) residual[pp] = res;
        if (u_stencil) u_stencil[pp * R] = u0 + bo;
      }
      seed = (float)(2.0 * (double)res * inv_n_total) * inv_eps2;  // times c_s / (-2d) or 1
    }
    // seeds of the group's stencil rows: c_0 = -2d / eps^2, the others 1 / eps^2
    mf4 abar[RG];
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) {
      const int r = r0 + rr;
      const float sr = r >= R ? 0.0f : r == 0 ? -2.0f * (float)D * seed : seed;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gWo[i] = fmaf(sr, atop[rr][i], gWo[i]);
        abar[rr][i] = sr * wout[i];
      }
    }
    auto rev_layer = [&]<int K>() {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = 16 * wn + 4 * lq + i;
        float zsum = 0.0f;
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) {
          if (r0 + rr < R) {
            float sv_unused, cv;
            sincos_red(om * z[K][rr][i], sv_unused, cv);
            const float zbar = abar[rr][i] * om * cv;
            zsum += zbar;
            sh.zb[o][(r0 + rr) * kMP + lm] = zbar;
          }
        }
        gb[K][i] += zsum;
      }
      __syncthreads();
      // weight gradient over the group's columns: dL/dW_K[16wn + .][j] += sum_c Zbar[o][c] V_K[j][c]
      const int nc4 = (R - r0 < RG ? R - r0 : RG) * (kMP / 4);
      mfma_prio_hi();
      for (int kk = 0; kk < nc4; ++kk) {
        const int c = r0 * kMP + 4 * kk + lq;
        const float az = sh.zb[16 * wn + lm][c];
        if constexpr (K == 0) {
#pragma unroll
          for (int t = 0; t < NI / 16; ++t) gW0[t] = mfma16(az, sh.act0[16 * t + lm][c], gW0[t]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) gW1[t] = mfma16(az, sh.act1[16 * t + lm][c], gW1[t]);
        }
      }
      mfma_prio_lo();
      if constexpr (K > 0) {
        // input adjoint for the wavefront's tile of input neurons j = 16 wn + .
        mf4 vbar[RG];
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) vbar[rr] = mf4{0.f, 0.f, 0.f, 0.f};
        mfma_prio_hi();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float aw = sh.w1[4 * kk + lq][16 * wn + lm];
#pragma unroll
          for (int rr = 0; rr < RG; ++rr)
            if (r0 + rr < R) vbar[rr] = mfma16(aw, sh.zb[4 * kk + lq][(r0 + rr) * kMP + lm], vbar[rr]);
        }
        mfma_prio_lo();
        __syncthreads();  // zb and the layer's inputs are rewritten next
#pragma unroll
        for (int rr = 0; rr < RG; ++rr) abar[rr] = vbar[rr];
      } else {
        // encoder upstream: the group's (input tile, row) pairs dealt round-robin over its four
        // wavefronts (with NI = 32 two of them would otherwise carry all of it), each stored
        // as soon as it is done
        constexpr int NT = NI / 16;
        const int nrows = R - r0 < RG ? R - r0 : RG;
        for (int T = wn; T < NT * nrows; T += kMWaves) {
          const int jt = T % NT, rr = T / NT;
          mf4 acc = mf4{0.f, 0.f, 0.f, 0.f};
          mfma_prio_hi();
#pragma unroll
          for (int kk = 0; kk < 16; ++kk)
            acc = mfma16(sh.w0[4 * kk + lq][16 * jt + lm], sh.zb[4 * kk + lq][(r0 + rr) * kMP + lm], acc);
          mfma_prio_lo();
          if (pp < n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 16 * jt + 4 * lq + i;
              if (j < a.ain) up[fd_index(a, n, pp, j, r0 + rr, R)] = acc[i];
            }
          }
        }
        __syncthreads();  // zb and the layer's inputs are rewritten next
      }
    };
    if constexpr (DEPTH > 1) rev_layer.template operator()<1>();
    // the next iteration's encoder rows, issued where the upper layer's tape is dead
    if (it + gridDim.x < n_iter) rows_load((it + gridDim.x) * kMP, ev);
    rev_layer.template operator()<0>();
  }

  // this row group's partial MLP gradient (and, for group 0, the sum of r^2)
  float* part = partial + ((int64_t)blockIdx.x * kFdGroups + rg) * (a.n_mlp + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = 16 * wn + 4 * lq + i;
    if (o < H) {
#pragma unroll
      for (int t = 0; t < NI / 16; ++t) {
        const int j = 16 * t + lm;
        if (j < a.in) part[a.woff[0] + (int64_t)o * a.in + j] = gW0[t][i];
      }
      if constexpr (DEPTH > 1) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = 16 * t + lm;
          if (j < H) part[a.woff[1] + (int64_t)o * H + j] = gW1[t][i];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[DEPTH + 1];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) v[k] = gb[k][i];
    v[DEPTH] = gWo[i];
#pragma unroll
    for (int k = 0; k <= DEPTH; ++k)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v[k] += __shfl_xor(v[k], off, 64);
    const int o = 16 * wn + 4 * lq + i;
    if (lm == 0 && o < H) {
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) part[a.boff[k] + o] = v[k];
      part[a.woff[DEPTH] + o] = v[DEPTH];
    }
  }
  if (wn == 0) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) sq += __shfl_xor(sq, off, 64);
    if (lane == 0) {
      part[a.boff[DEPTH]] = 0.0f;  // the output bias cancels in the stencil
      part[a.n_mlp] = rg == 0 ? sq : 0.0f;
    }
  }
}

// Stencil point sets, s = 0: x; s = 2i+1: x + eps e_i; s = 2i+2: x - eps e_i (one fp32
// addition, as any fp32 input of the encoder), written point-major (xp[p][s][d], for the
// forward) and stencil-major (xs[s][p][d], for the backward).
template <int D>
__global__ __launch_bounds__(kBlock) void fd_stencil_kernel(int64_t n, float eps, const float* __restrict__ x,
                                                            float* __restrict__ xp, float* __restrict__ xs) {
  constexpr int S = 2 * D + 1;
  const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;  // one point, all its stencil points
  if (p >= n) return;
  float x0[D];
#pragma unroll
  for (int i = 0; i < D; ++i) x0[i] = x[p * D + i];
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float v = (s > 0 && i == (s - 1) / 2) ? ((s & 1) ? x0[i] + eps : x0[i] - eps) : x0[i];
      xp[(p * S + s) * D + i] = v;
      xs[((int64_t)s * n + p) * D + i] = v;
    }
  }
}

// Sum of the partial rows, in two passes: each workgroup of the first pass adds a slice of
// about sqrt(rows) rows for 256 columns in fp64; the second pass adds the slices and applies
// the result (grad_mlp += ..., loss (+)= ... / n).  Both passes thus run about sqrt(rows)
// loads per thread, four independent sums in flight: a few hundred rows of a small batch
// take a few microseconds instead of one long serial chain per column.
int slice_rows_for(int64_t rows) {
  int r = 4;
  while ((int64_t)r * r < rows) ++r;
  return r;
}
// slices of a pass over at most max_rows rows: ceil(rows / slice_rows_for(rows)) <=
// ceil(sqrt(rows)) <= slice_rows_for(max_rows)
int max_slices_for(int64_t max_rows) { return slice_rows_for(max_rows); }

__global__ __launch_bounds__(256) void reduce_partials_slices_kernel(const float* __restrict__ partial,
                                                                     int64_t n_waves, int64_t n_cols,
                                                                     int slice_rows,
                                                                     double* __restrict__ slices) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n_cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * slice_rows;
  const int64_t r1 = r0 + slice_rows < n_waves ? r0 + slice_rows : n_waves;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    s0 += (double)partial[r * n_cols + c];
    s1 += (double)partial[(r + 1) * n_cols + c];
    s2 += (double)partial[(r + 2) * n_cols + c];
    s3 += (double)partial[(r + 3) * n_cols + c];
  }
  for (; r < r1; ++r) s0 += (double)partial[r * n_cols + c];
  slices[(int64_t)blockIdx.y * n_cols + c] = (s0 + s1) + (s2 + s3);
}

__global__ __launch_bounds__(256) void reduce_partials_apply_kernel(const double* __restrict__ slices,
                                                                    int n_slices, int64_t n_mlp,
                                                                    double inv_n_total, int first,
                                                                    float* __restrict__ grad_mlp,
                                                                    float* __restrict__ loss) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c > n_mlp) return;
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int i = 0;
  for (; i + 4 <= n_slices; i += 4) {
    s0 += slices[(int64_t)i * (n_mlp + 1) + c];
    s1 += slices[(int64_t)(i + 1) * (n_mlp + 1) + c];
    s2 += slices[(int64_t)(i + 2) * (n_mlp + 1) + c];
    s3 += slices[(int64_t)(i + 3) * (n_mlp + 1) + c];
  }
  for (; i < n_slices; ++i) s0 += slices[(int64_t)i * (n_mlp + 1) + c];
  const double s = (s0 + s1) + (s2 + s3);
  if (c < n_mlp) {
    if (grad_mlp) grad_mlp[c] += (float)s;
  } else {
    const float v = (float)(s * inv_n_total);
    *loss = first ? v : *loss + v;
  }
}

constexpr int64_t kChunk = int64_t(1) << 21;  // points per pass over the workspace (at most)

// Points per pass: one binned-backward chunk, so the SIREN kernel's level-major upstream
// feeds the binned backward directly.
int64_t residual_chunk_points(const Grid& g, int d) {
  const int64_t b = bin_chunk_points(g, d, true);
  return b < kChunk ? b : kChunk;
}
constexpr int kSirenBlocks = 256;  // one workgroup per CU (LDS-limited)

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct WorkspaceLayout {
  size_t enc, up, partial, slices, packed, bins, total;
};

WorkspaceLayout workspace_layout(const Grid& g, int d, int F, int64_t n, int64_t n_mlp, bool binned) {
  const int LF = g.L * F;
  const int64_t cmax = residual_chunk_points(g, d);
  const int64_t c = n < cmax ? n : cmax;
  WorkspaceLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  // encoder outputs and their upstream, level-major [L][c][d + 2][F] (value, gradient, Laplacian)
  w.enc = take(sizeof(float) * c * LF * (d + 2));
  w.up = take(sizeof(float) * c * LF * (d + 2));
  w.partial = take(sizeof(float) * (size_t)kSirenBlocks * kMaxWavesPerBlock * (n_mlp + 1));
  w.slices = take(sizeof(double) * (size_t)max_slices_for(kSirenBlocks * kMaxWavesPerBlock) *
                  (n_mlp + 1));
  w.packed = take(hermite_packed_bytes(g, d, F));  // packed order tables for the forward
  w.bins = take(binned ? binned_backward_workspace_bytes(g, d, F, true, c) : 0);
  w.total = off;
  return w;
}

template <int D, int DEPTH, int INP>
hipError_t launch_siren(const MlpArgs& a, int64_t n, double inv_n, const float* x, const float* enc,
                        const float* mlp, float* up, float* residual, float* partial, int& rows, hipStream_t s) {
  // matrix cores whenever the layers' weights and inputs fit one workgroup's LDS (all but
  // depth 4 with a 64-wide encoder); deeper networks hold one workgroup per CU
  if constexpr (DEPTH <= 2 || sizeof(MfmaLds<D, DEPTH, INP>) <= 160 * 1024) {
    // one partial row per workgroup; the kernel addresses the encoder output with 32-bit
    // byte offsets
    if ((uint64_t)n * (D + 2) * a.in * sizeof(float) >= (uint64_t(1) << 32)) return hipErrorInvalidValue;
    int blocks = (int)((n + kMP - 1) / kMP);
    const int max_blocks = DEPTH <= 2 ? kMfmaBlocks : kSirenBlocks;
    if (blocks > max_blocks) blocks = max_blocks;
    rows = blocks;
    hipLaunchKernelGGL((siren_mfma_kernel<D, DEPTH, INP>), dim3(blocks), dim3(kW * kMWaves), 0, s, a, n, inv_n, x,
                       enc, mlp, up, residual, partial);
  } else {
    // vector ALUs: one partial row per wavefront
    const int wpb = siren_waves(DEPTH, INP);
    int blocks = (int)((n + wpb * kPB - 1) / (wpb * kPB));
    if (blocks > kSirenBlocks) blocks = kSirenBlocks;
    rows = blocks * wpb;
    hipLaunchKernelGGL((siren_residual_kernel<D, DEPTH, INP>), dim3(blocks), dim3(kW * wpb), 0, s, a, n, inv_n, x,
                       enc, mlp, up, residual, partial);
  }
  return hipGetLastError();
}

template <int D, int DEPTH>
hipError_t dispatch_in(int in, const MlpArgs& a, int64_t n, double inv_n, const float* x, const float* enc, const float* mlp, float* up,
                       float* residual, float* partial, int& rows, hipStream_t s) {
  if (in <= 16) return launch_siren<D, DEPTH, 16>(a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
  if (in <= 32) return launch_siren<D, DEPTH, 32>(a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
  return launch_siren<D, DEPTH, 64>(a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
}

template <int D>
hipError_t dispatch_depth(int depth, int in, const MlpArgs& a, int64_t n, double inv_n, const float* x,
                          const float* enc, const float* mlp, float* up, float* residual, float* partial, int& rows, hipStream_t s) {
  switch (depth) {
    case 1: return dispatch_in<D, 1>(in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
    case 2: return dispatch_in<D, 2>(in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
    case 3: return dispatch_in<D, 3>(in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
    default: return dispatch_in<D, 4>(in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
  }
}

hipError_t dispatch_siren(int d, int depth, int in, const MlpArgs& a, int64_t n, double inv_n,
                          const float* x, const float* enc,
                          const float* mlp, float* up, float* residual,
                          float* partial, int& rows, hipStream_t s) {
  if (d == 2) return dispatch_depth<2>(depth, in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
  return dispatch_depth<3>(depth, in, a, n, inv_n, x, enc, mlp, up, residual, partial, rows, s);
}

// INGP-FD comparator for SIREN depth 3 and 4 on the vector ALUs (the matrix-core kernel
// above holds the tape of at most two layers).  The layout of the fused residual's vector
// kernel: a wavefront takes kPB points at a time, lane = neuron, and the columns are the
// (point, stencil copy) pairs, each a plain value row: z = W v + b, a = sin(omega z) on
// every column, u_s = wout . a_s, Lap u by the second differences of the copies, and the
// reverse seeds ubar_s = (2 r / n) c_s / eps^2 (c_0 = -2d, else 1), zbar = abar omega
// cos(omega z).
// Wavefronts per workgroup: the most (4, 2 or 1) whose activation rows fit the CU's 160 KB
// beside the weights.
__host__ __device__ constexpr int fd_vec_waves(int d, int depth, int inp) {
  const int rb = kPB * (2 * d + 1);
  const int fixed_bytes = 4 * (depth * kW * (kW + 1) + depth * kW + kW);
  const int wave_bytes = 4 * rb * (inp + (depth - 1) * kW + kW);
  return fixed_bytes + 4 * wave_bytes <= 160 * 1024 ? 4 : fixed_bytes + 2 * wave_bytes <= 160 * 1024 ? 2 : 1;
}

template <int D, int DEPTH, int INP>
struct FdVecLds {
  static constexpr int R = 2 * D + 1;
  static constexpr int RB = kPB * R;  // columns: kPB points x R stencil copies
  static constexpr int WV = fd_vec_waves(D, DEPTH, INP);
  float W[DEPTH][kW][kW + 1];  // W[k][o][j] = W_k[o][j]
  float bias[DEPTH][kW];
  float wout[kW];
  __attribute__((aligned(16))) float act0[WV][INP][RB];
  __attribute__((aligned(16))) float act[WV][DEPTH - 1][kW][RB];
  __attribute__((aligned(16))) float zb[WV][kW][RB];
};

template <int D, int DEPTH, int INP>
__global__ __launch_bounds__(kW * fd_vec_waves(D, DEPTH, INP)) void siren_fd_vec_kernel(
    const MlpArgs a, int64_t n, double inv_n_total, float inv_eps2, const float* __restrict__ x,
    const float* __restrict__ enc, const float* __restrict__ mlp, float* __restrict__ up,
    float* __restrict__ u_stencil, float* __restrict__ residual, float* __restrict__ partial) {
  using Sh = FdVecLds<D, DEPTH, INP>;
  constexpr int R = Sh::R;
  constexpr int RB = Sh::RB;
  constexpr int WV = Sh::WV;
  static_assert(DEPTH >= 2, "depth 1 and 2 run on the matrix cores");
  static_assert(RB % 4 == 0, "activation rows move as 16-byte pieces");
  static_assert(sizeof(Sh) <= 160 * 1024, "FD workgroup LDS exceeds the CU's 160 KB");
  __shared__ Sh sh;

  const int tid = threadIdx.x;
  const int lane = tid & (kW - 1);
  const int wv = tid / kW;
  const float w = a.omega;
  for (int k = 0; k < DEPTH; ++k) {
    const int fi = k == 0 ? a.in : a.H;
    const float* Wk = mlp + a.woff[k];
    for (int e = tid; e < kW * kW; e += kW * WV) {
      const int o = e / kW, j = e % kW;
      sh.W[k][o][j] = (o < a.H && j < fi) ? Wk[o * fi + j] : 0.0f;
    }
    for (int o = tid; o < kW; o += kW * WV) sh.bias[k][o] = o < a.H ? mlp[a.boff[k] + o] : 0.0f;
  }
  for (int o = tid; o < kW; o += kW * WV) sh.wout[o] = o < a.H ? mlp[a.woff[DEPTH] + o] : 0.0f;
  const float bo = mlp[a.boff[DEPTH]];
  __syncthreads();

  float gW0[INP];
  float gW[DEPTH - 1][kW];
  float gb[DEPTH];
  float gWo = 0.0f, sq = 0.0f;
#pragma unroll
  for (int j = 0; j < INP; ++j) gW0[j] = 0.0f;
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) gb[k] = 0.0f;
#pragma unroll
  for (int k = 0; k + 1 < DEPTH; ++k)
#pragma unroll
    for (int j = 0; j < kW; ++j) gW[k][j] = 0.0f;

  auto in_row = [&](int k, int j) -> float* { return k == 0 ? sh.act0[wv][j] : sh.act[wv][k - 1][j]; };

  const int64_t wave_id = (int64_t)blockIdx.x * WV + wv;
  const int64_t n_waves = (int64_t)gridDim.x * WV;
  for (int64_t p0 = wave_id * kPB; p0 < n; p0 += n_waves * kPB) {
    // encoder rows of the points' stencil copies (lm_index layout, R = 2d + 1)
    if (lane < INP) {
      float row[RB];
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const int64_t p = p0 + b;
        const bool on = lane < a.ain && p < n;
#pragma unroll
        for (int r = 0; r < R; ++r) row[b * R + r] = on ? enc[lm_index(a, n, p, lane, r, R)] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < RB; q += 4)
        *reinterpret_cast<float4*>(&sh.act0[wv][lane][q]) = make_float4(row[q], row[q + 1], row[q + 2], row[q + 3]);
    }
    wave_lds_sync();

    // forward: every column a value row; the tape keeps omega cos(omega z)
    float tc[DEPTH][RB];
    float atop[RB];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) {
      const int fi = k == 0 ? INP : kW;
      float z[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) z[q] = sh.bias[k][lane];
#pragma unroll 4
      for (int j = 0; j < fi; ++j) {
        const float wj = sh.W[k][lane][j];
        const float* v = in_row(k, j);
#pragma unroll
        for (int q = 0; q < RB; q += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(v + q);
          z[q] = fmaf(wj, a4.x, z[q]);
          z[q + 1] = fmaf(wj, a4.y, z[q + 1]);
          z[q + 2] = fmaf(wj, a4.z, z[q + 2]);
          z[q + 3] = fmaf(wj, a4.w, z[q + 3]);
        }
      }
      float out[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        float sv, cv;
        sincos_red(w * z[q], sv, cv);
        out[q] = sv;
        tc[k][q] = w * cv;
      }
      if (k + 1 < DEPTH) {
#pragma unroll
        for (int q = 0; q < RB; q += 4)
          *reinterpret_cast<float4*>(&sh.act[wv][k][lane][q]) = make_float4(out[q], out[q + 1], out[q + 2], out[q + 3]);
        wave_lds_sync();
      } else {
#pragma unroll
        for (int q = 0; q < RB; ++q) atop[q] = out[q];
      }
    }
    // u_s = wout . a_s per column (the output bias cancels in every second difference),
    // the residual and the seeds
    float ab[RB];
#pragma unroll
    for (int b = 0; b < kPB; ++b) {
      const int64_t p = p0 + b;
      float u[R];
#pragma unroll
      for (int r = 0; r < R; ++r) u[r] = wave_sum(sh.wout[lane] * atop[b * R + r]);
      float seed = 0.0f;
      if (p < n) {
        float lap = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) lap += ((u[2 * i + 1] - u[0]) + (u[2 * i + 2] - u[0])) * inv_eps2;
        float src = -(float)D * 9.8696044010893586f;  // -d pi^2
#pragma unroll
        for (int i = 0; i < D; ++i) src *= sinpif(x[p * D + i]);
        const float res = lap - src;
        if (lane == 0) {
          sq = fmaf(res, res, sq);
          if (residual) residual[p] = res;
          if (u_stencil)
#pragma unroll
            for (int r = 0; r < R; ++r) u_stencil[p * R + r] = u[r] + bo;
        }
        seed = (float)(2.0 * (double)res * inv_n_total) * inv_eps2;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float ubar = r == 0 ? -2.0f * (float)D * seed : seed;
        gWo = fmaf(ubar, atop[b * R + r], gWo);
        ab[b * R + r] = ubar * sh.wout[lane];
      }
    }
    // reverse sweep
#pragma unroll
    for (int k = DEPTH - 1; k >= 0; --k) {
      float zbar[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        zbar[q] = ab[q] * tc[k][q];
        gb[k] += zbar[q];
      }
      if (k == 0) {
#pragma unroll
        for (int j = 0; j < INP; ++j) {
          const float* v = sh.act0[wv][j];
          float acc = gW0[j];
#pragma unroll
          for (int q = 0; q < RB; q += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(v + q);
            acc = fmaf(zbar[q], a4.x, acc);
            acc = fmaf(zbar[q + 1], a4.y, acc);
            acc = fmaf(zbar[q + 2], a4.z, acc);
            acc = fmaf(zbar[q + 3], a4.w, acc);
          }
          gW0[j] = acc;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kW; ++j) {
          const float* v = sh.act[wv][k - 1][j];
          float acc = gW[k - 1][j];
#pragma unroll
          for (int q = 0; q < RB; q += 4) {
            const float4 a4 = *reinterpret_cast<const float4*>(v + q);
            acc = fmaf(zbar[q], a4.x, acc);
            acc = fmaf(zbar[q + 1], a4.y, acc);
            acc = fmaf(zbar[q + 2], a4.z, acc);
            acc = fmaf(zbar[q + 3], a4.w, acc);
          }
          gW[k - 1][j] = acc;
        }
      }
      // input adjoint: lane j <- sum_o W_k[o][j] zbar_o
#pragma unroll
      for (int q = 0; q < RB; q += 4)
        *reinterpret_cast<float4*>(&sh.zb[wv][lane][q]) = make_float4(zbar[q], zbar[q + 1], zbar[q + 2], zbar[q + 3]);
      wave_lds_sync();
#pragma unroll
      for (int q = 0; q < RB; ++q) ab[q] = 0.0f;
#pragma unroll 4
      for (int o = 0; o < kW; ++o) {
        const float wo = sh.W[k][o][lane];
        const float* zr = sh.zb[wv][o];
#pragma unroll
        for (int q = 0; q < RB; q += 4) {
          const float4 z4 = *reinterpret_cast<const float4*>(zr + q);
          ab[q] = fmaf(wo, z4.x, ab[q]);
          ab[q + 1] = fmaf(wo, z4.y, ab[q + 1]);
          ab[q + 2] = fmaf(wo, z4.z, ab[q + 2]);
          ab[q + 3] = fmaf(wo, z4.w, ab[q + 3]);
        }
      }
      wave_lds_sync();  // zb is rewritten by the next layer
    }
    // encoder upstream, stencil-major ([L][R][n][F]), for the inputs this lane owns
    if (lane < a.ain) {
#pragma unroll
      for (int b = 0; b < kPB; ++b) {
        const int64_t p = p0 + b;
        if (p >= n) break;
#pragma unroll
        for (int r = 0; r < R; ++r) up[fd_index(a, n, p, lane, r, R)] = ab[b * R + r];
      }
    }
  }

  // this wave's partial MLP gradient and sum of r^2
  float* part = partial + wave_id * (a.n_mlp + 1);
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) {
    const int fi = k == 0 ? a.in : a.H;
    if (lane < a.H) {
      if (k == 0) {
#pragma unroll
        for (int j = 0; j < INP; ++j)
          if (j < fi) part[a.woff[0] + (int64_t)lane * fi + j] = gW0[j];
      } else {
#pragma unroll
        for (int j = 0; j < kW; ++j)
          if (j < fi) part[a.woff[k] + (int64_t)lane * fi + j] = gW[k - 1][j];
      }
      part[a.boff[k] + lane] = gb[k];
    }
  }
  if (lane < a.H) part[a.woff[DEPTH] + lane] = gWo;
  if (lane == 0) {
    part[a.boff[DEPTH]] = 0.0f;  // the output bias cancels in the stencil
    part[a.n_mlp] = sq;
  }
}

constexpr int kFdBlocks = 256;  // one workgroup per CU (LDS-limited)

// Partial rows of the FD network kernels: one per row group (matrix cores) or per wavefront
// (vector ALUs, depth 3 and 4).
constexpr int kFdPartialRows = kSirenBlocks * kMaxWavesPerBlock;

template <int D, int DEPTH, int NI>
hipError_t launch_fd_siren(const MlpArgs& a, int64_t n, double inv_n, float inv_eps2, const float* x,
                           const float* enc, const float* mlp, float* up, float* u_stencil, float* residual,
                           float* partial, int& rows, hipStream_t s) {
  if constexpr (DEPTH > 2) {
    constexpr int wpb = FdVecLds<D, DEPTH, NI>::WV;
    int blocks = (int)((n + wpb * kPB - 1) / (wpb * kPB));
    if (blocks > kSirenBlocks) blocks = kSirenBlocks;
    rows = blocks * wpb;
    hipLaunchKernelGGL((siren_fd_vec_kernel<D, DEPTH, NI>), dim3(blocks), dim3(kW * wpb), 0, s, a, n, inv_n, inv_eps2,
                       x, enc, mlp, up, u_stencil, residual, partial);
    return hipGetLastError();
  } else {
    // the kernel addresses the encoder output with 32-bit byte offsets
    if ((uint64_t)n * (2 * D + 1) * a.in * sizeof(float) >= (uint64_t(1) << 32)) return hipErrorInvalidValue;
    int blocks = (int)((n + kMP - 1) / kMP);
    if (blocks > kFdBlocks) blocks = kFdBlocks;
    rows = blocks * kFdGroups;  // one partial row per row group
    hipLaunchKernelGGL((siren_fd_mfma_kernel<D, DEPTH, NI>), dim3(blocks), dim3(kW * kFdWaves), 0, s, a, n, inv_n,
                       inv_eps2, x, enc, mlp, up, u_stencil, residual, partial);
    return hipGetLastError();
  }
}

template <int D, int DEPTH>
hipError_t fd_dispatch_in(int in, const MlpArgs& a, int64_t n, double inv_n, float inv_eps2, const float* x,
                          const float* enc, const float* mlp, float* up, float* u_stencil, float* residual,
                          float* partial, int& rows, hipStream_t s) {
  if (in <= 16)
    return launch_fd_siren<D, DEPTH, 16>(a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s);
  if (in <= 32)
    return launch_fd_siren<D, DEPTH, 32>(a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s);
  return launch_fd_siren<D, DEPTH, 64>(a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s);
}

hipError_t fd_dispatch(int d, int depth, int in, const MlpArgs& a, int64_t n, double inv_n, float inv_eps2,
                       const float* x, const float* enc, const float* mlp, float* up, float* u_stencil,
                       float* residual, float* partial, int& rows, hipStream_t s) {
#define HASHENC_FD_DEPTHS(DD)                                                                                  \
  switch (depth) {                                                                                             \
    case 1: return fd_dispatch_in<DD, 1>(in, a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s); \
    case 2: return fd_dispatch_in<DD, 2>(in, a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s); \
    case 3: return fd_dispatch_in<DD, 3>(in, a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s); \
    case 4: return fd_dispatch_in<DD, 4>(in, a, n, inv_n, inv_eps2, x, enc, mlp, up, u_stencil, residual, partial, rows, s); \
  }                                                                                                            \
  return hipErrorInvalidValue
  if (d == 2) { HASHENC_FD_DEPTHS(2); }
  HASHENC_FD_DEPTHS(3);
#undef HASHENC_FD_DEPTHS
}

// Centre points per FD chunk: the chunk's 2d+1 stencil sets fit one binned-backward chunk,
// whose level-major upstream then comes straight from the SIREN kernel.
int64_t fd_chunk_points(const Grid& g, int d) {
  return (bin_chunk_points(g, d, false) / (2 * d + 1)) & ~int64_t(kMP - 1);
}

struct FdWorkspaceLayout {
  size_t xp, xs, enc, up, partial, slices, bins, total;
};

FdWorkspaceLayout fd_workspace_layout(const Grid& g, int d, int F, int64_t n, int64_t n_mlp, bool binned) {
  const int64_t cmax = fd_chunk_points(g, d);
  const int64_t c = n < cmax ? n : cmax;
  const int64_t cs = c * (2 * d + 1);
  FdWorkspaceLayout w;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  w.xp = take(sizeof(float) * (size_t)cs * d);
  w.xs = take(sizeof(float) * (size_t)cs * d);
  w.enc = take(dlinear_forward_workspace_bytes(g, d, F, cs));  // level-major [L][c (2d+1)][F]
  w.up = take(dlinear_forward_workspace_bytes(g, d, F, cs));
  w.partial = take(sizeof(float) * (size_t)kFdPartialRows * (n_mlp + 1));
  w.slices = take(sizeof(double) * (size_t)max_slices_for(kFdPartialRows) * (n_mlp + 1));
  w.bins = take(binned ? binned_backward_workspace_bytes(g, d, F, false, cs) : 0);
  w.total = off;
  return w;
}

MlpArgs make_mlp_args(const Grid& g, int F, int in, int H, int depth, float omega) {
  MlpArgs a;
  a.in = in;
  a.ain = g.L * F;  // levels l >= g.L are inactive: zero inputs, no upstream
  a.H = H;
  a.depth = depth;
  a.omega = omega;
  a.fshift = F == 1 ? 0 : F == 2 ? 1 : F == 4 ? 2 : 3;
  a.n_mlp = 0;
  for (int k = 0; k <= kMaxDepth; ++k) { a.woff[k] = 0; a.boff[k] = 0; }
  int64_t off = 0;
  for (int k = 0; k <= depth; ++k) {
    const int64_t fi = k == 0 ? in : H;
    const int64_t fo = k == depth ? 1 : H;
    a.woff[k] = off; off += fi * fo;
    a.boff[k] = off; off += fo;
  }
  a.n_mlp = off;
  return a;
}

// Sum the partial rows of one chunk into grad_mlp and the loss (first chunk: loss = ...).
hipError_t reduce_partials(const MlpArgs& a, const float* partial, int64_t rows, double* slices, double inv_n,
                           bool first, float* grad_mlp, float* loss, hipStream_t s) {
  const int sr = slice_rows_for(rows);
  const int n_slices = (int)((rows + sr - 1) / sr);
  const unsigned col_blocks = (unsigned)((a.n_mlp + 1 + 255) / 256);
  hipLaunchKernelGGL(reduce_partials_slices_kernel, dim3(col_blocks, (unsigned)n_slices), dim3(256), 0, s,
                     partial, rows, a.n_mlp + 1, sr, slices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_partials_apply_kernel, dim3(col_blocks), dim3(256), 0, s, slices, n_slices, a.n_mlp,
                     inv_n, first ? 1 : 0, grad_mlp, loss);
  return hipGetLastError();
}

}  // namespace

size_t fd_residual_workspace_bytes(const Grid& g, int d, int F, int64_t n, int in, int H, int depth, bool binned) {
  return fd_workspace_layout(g, d, F, n, mlp_param_count(in, H, depth), binned).total;
}

hipError_t run_fd_residual(const Grid& g, int d, int F, int64_t n, const float* x, const float* params, int in,
                           int H, int depth, float omega, float eps, const float* mlp, float* u_stencil,
                           float* residual, float* loss, float* grad_params, float* grad_mlp, void* workspace,
                           bool binned, hipStream_t s) {
  const MlpArgs a = make_mlp_args(g, F, in, H, depth, omega);
  const FdWorkspaceLayout wl = fd_workspace_layout(g, d, F, n, a.n_mlp, binned);
  char* ws = static_cast<char*>(workspace);
  float* xp = reinterpret_cast<float*>(ws + wl.xp);
  float* xs = reinterpret_cast<float*>(ws + wl.xs);
  float* enc = reinterpret_cast<float*>(ws + wl.enc);
  float* up = reinterpret_cast<float*>(ws + wl.up);
  float* partial = reinterpret_cast<float*>(ws + wl.partial);
  double* slices = reinterpret_cast<double*>(ws + wl.slices);
  const double inv_n = 1.0 / (double)n;
  const float inv_eps2 = (float)(1.0 / ((double)eps * (double)eps));
  const int S = 2 * d + 1;
  const int64_t cmax = fd_chunk_points(g, d);
  for (int64_t p0 = 0; p0 < n; p0 += cmax) {
    const int64_t c = (n - p0) < cmax ? (n - p0) : cmax;
    const float* xc = x + p0 * d;
    const int64_t cs = c * S;
    const dim3 sgrid((unsigned)((c + kBlock - 1) / kBlock));
    if (d == 2) hipLaunchKernelGGL(fd_stencil_kernel<2>, sgrid, dim3(kBlock), 0, s, c, eps, xc, xp, xs);
    else hipLaunchKernelGGL(fd_stencil_kernel<3>, sgrid, dim3(kBlock), 0, s, c, eps, xc, xp, xs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the 2d+1 encodings of every point, point-major then level-major: the SIREN kernel's input
    e = launch_dlinear_forward(g, d, F, cs, xp, params, nullptr, enc, s);
    if (e != hipSuccess) return e;
    int rows = 0;
    e = fd_dispatch(d, depth, in, a, c, inv_n, inv_eps2, xc, enc, mlp, up, u_stencil ? u_stencil + p0 * S : nullptr,
                    residual ? residual + p0 : nullptr, partial, rows, s);
    if (e != hipSuccess) return e;
    e = reduce_partials(a, partial, rows, slices, inv_n, p0 == 0, grad_mlp, loss, s);
    if (e != hipSuccess) return e;
    if (grad_params) {
      e = binned ? run_binned_backward(g, d, F, false, 0, cs, xs, nullptr, nullptr, nullptr, up, grad_params,
                                       ws + wl.bins, s)
                 : launch_dlinear_backward(g, d, F, cs, xs, nullptr, up, grad_params, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

int64_t mlp_param_count(int in, int H, int depth) {
  int64_t n = 0;
  for (int k = 0; k <= depth; ++k) {
    const int64_t fi = k == 0 ? in : H;
    const int64_t fo = k == depth ? 1 : H;
    n += fi * fo + fo;
  }
  return n;
}

size_t residual_workspace_bytes(const Grid& g, int d, int F, int64_t n, int in, int H, int depth,
                                bool binned) {
  return workspace_layout(g, d, F, n, mlp_param_count(in, H, depth), binned).total;
}

hipError_t run_residual(const Grid& g, int d, int F, int64_t n, const float* x, const float* params,
                        int in, int H, int depth, float omega, const float* mlp, float* residual,
                        float* loss, float* grad_params, float* grad_mlp, void* workspace,
                        bool binned, hipStream_t s) {
  MlpArgs a;
  a.in = in;
  a.ain = g.L * F;  // levels l >= g.L are inactive: zero inputs, no upstream
  a.H = H;
  a.depth = depth;
  a.omega = omega;
  a.fshift = F == 1 ? 0 : F == 2 ? 1 : F == 4 ? 2 : 3;
  a.n_mlp = mlp_param_count(in, H, depth);
  int64_t off = 0;
  for (int k = 0; k <= kMaxDepth; ++k) { a.woff[k] = 0; a.boff[k] = 0; }
  for (int k = 0; k <= depth; ++k) {
    const int64_t fi = k == 0 ? in : H;
    const int64_t fo = k == depth ? 1 : H;
    a.woff[k] = off; off += fi * fo;
    a.boff[k] = off; off += fo;
  }
  const WorkspaceLayout wl = workspace_layout(g, d, F, n, a.n_mlp, binned);
  char* ws = static_cast<char*>(workspace);
  float* enc = reinterpret_cast<float*>(ws + wl.enc);
  float* up = reinterpret_cast<float*>(ws + wl.up);
  float* partial = reinterpret_cast<float*>(ws + wl.partial);
  const double inv_n = 1.0 / (double)n;
  // the parameters do not change between chunks: pack the order tables once (batches of at
  // least kPackMinPoints; smaller ones gather from the tables)
  float* packed =
      hermite_packed_bytes(g, d, F) && n >= kPackMinPoints ? reinterpret_cast<float*>(ws + wl.packed) : nullptr;
  if (packed) {
    hipError_t e = launch_hermite_pack(g, d, F, params, packed, s);
    if (e != hipSuccess) return e;
  }
  const int64_t cmax = residual_chunk_points(g, d);
  for (int64_t p0 = 0; p0 < n; p0 += cmax) {
    const int64_t c = (n - p0) < cmax ? (n - p0) : cmax;
    const float* xc = x + p0 * d;
    // Hermite forward straight into the level-major layout the SIREN kernels read
    hipError_t e = launch_hermite_forward(g, d, F, HASHENC_D2_LAPLACIAN, c, xc, params, packed, enc, false, nullptr,
                                          nullptr, nullptr, s);
    if (e != hipSuccess) return e;
    float* rc = residual ? residual + p0 : nullptr;
    int rows = 0;  // partial rows written (per wavefront or per workgroup)
    e = dispatch_siren(d, depth, in, a, c, inv_n, xc, enc, mlp, up, rc, partial, rows, s);
    if (e != hipSuccess) return e;
    e = reduce_partials(a, partial, rows, reinterpret_cast<double*>(ws + wl.slices), inv_n, p0 == 0, grad_mlp, loss,
                        s);
    if (e != hipSuccess) return e;
    if (grad_params) {
      // the SIREN kernels wrote the upstream level-major, as the backward reads it
      e = binned ? run_binned_backward(g, d, F, true, HASHENC_D2_LAPLACIAN, c, xc, nullptr, nullptr, nullptr, up,
                                       grad_params, ws + wl.bins, s)
                 : launch_hermite_backward(g, d, F, HASHENC_D2_LAPLACIAN, c, xc, nullptr, nullptr, nullptr, up,
                                           grad_params, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace hg
