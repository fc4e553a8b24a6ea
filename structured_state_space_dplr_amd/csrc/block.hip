// The block around the layer ("The S4 kernel, from scratch", section 6: a
// pre-norm, a GLU-gated projection and a residual connection):
//   z   = LayerNorm over the H channels at every (b, t), with gain and shift,
//   s   = the layer applied to z (kernel generation + causal convolution),
//   out = x + a * sigmoid(g),  [a; g] = W s + bias,  W: (2H x H).
//
// The projection is the block's only dense contraction: per batch row it is a
// GEMM with M = H output channels (for each of the two halves), N = L time
// steps and K = H input channels, done on the matrix cores with fp32 MFMA
// (v_mfma_f32_32x32x2f32), so that the block keeps fp32 accuracy.  The bias,
// the gate and the residual are applied to the accumulators in registers.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace s4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kLnThreads = 256;
// Projection tile: a block computes 64 channels x 128 time steps of both
// halves; wave w owns channels [32 (w / 2), +32) and time steps [64 (w % 2), +64)
// as two 32 x 32 MFMA tiles per half.
constexpr int kPM = 64, kPN = 128, kPK = 32;
constexpr int kPThreads = 256;

}  // namespace

// mean and 1/sqrt(var + eps) over h of x[b][h][t] (fp64 sums), then
// z[b][h][t] = (x - mean) rstd gamma_h + beta_h.  Block (64 time steps, b):
// wave g sums the channels h = g, g + 4, ... of its lane's time step; the four
// partial sums meet in LDS, and the normalization is split the same way.
__global__ __launch_bounds__(kLnThreads) void layer_norm_kernel(
    const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
    float* __restrict__ z, int H, int L, float eps) {
  constexpr int G = kLnThreads / 64;
  __shared__ double red[2][G][64];
  __shared__ float stat[2][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const bool on = t < L;
  const float* xb = x + (size_t)b * H * L + t;
  double s1 = 0.0, s2 = 0.0;
  if (on) {
#pragma unroll 8
    for (int h = g; h < H; h += G) {
      const double v = (double)xb[(size_t)h * L];
      s1 += v;
      s2 += v * v;
    }
  }
  red[0][g][lane] = s1;
  red[1][g][lane] = s2;
  __syncthreads();
  if (g == 0) {
    double a = 0.0, q = 0.0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      a += red[0][i][lane];
      q += red[1][i][lane];
    }
    const double mean = a / H;
    const double var = fmax(q / H - mean * mean, 0.0);
    stat[0][lane] = (float)mean;
    stat[1][lane] = (float)(1.0 / sqrt(var + (double)eps));
  }
  __syncthreads();
  if (!on) return;
  const float m = stat[0][lane], r = stat[1][lane];
  float* zb = z + (size_t)b * H * L + t;
#pragma unroll 8
  for (int h = g; h < H; h += G) {
    const size_t o = (size_t)h * L;
    zb[o] = fmaf((xb[o] - m) * r, gamma[h], beta[h]);
  }
}

// out[b][c][t] = x[b][c][t] + (Wa s + ba)[c][t] * sigmoid((Wg s + bg)[c][t]).
// out may be x itself: every element is read and then written by one lane.
// Each K stage stages 64 rows x 32 of each W half and 32 x 128 of s through
// LDS with float4 loads; the next stage's loads are issued before the current
// stage's MFMAs.  Fully in-range tiles (H % 32 == 0 and L % 128 == 0 here)
// take the vector path; edge tiles load element by element with zero fill.
__global__ __launch_bounds__(kPThreads) void glu_proj_kernel(
    const float* x, const float* __restrict__ s, const float* __restrict__ W,
    const float* __restrict__ bias, float* out, int H, int L) {
  __shared__ float sWa[kPM][kPK + 1];
  __shared__ float sWg[kPM][kPK + 1];
  __shared__ float sS[kPK][kPN + 4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.z, c0 = blockIdx.y * kPM, t0 = blockIdx.x * kPN;
  const int cw = 32 * (w >> 1), tw = 64 * (w & 1);
  const float* sb = s + (size_t)b * H * L;
  const bool vec = (H % kPK == 0) && (c0 + kPM <= H) && (t0 + kPN <= L) && (L % 4 == 0);
  // float4 slots of a stage: W halves 2 x 64 rows x 8, s 32 rows x 32; slot Q
  // of thread tid is i = tid + 256 Q (half = Q / 2 for the W slots), held in
  // named registers (an indexed array here ends up in scratch memory)
  float4 rw0, rw1, rw2, rw3, rs0, rs1, rs2, rs3;
#define PROJ_FETCH(Q, H0)                                                                        \
  do {                                                                                           \
    const int i_ = tid + (Q) * kPThreads;                                                        \
    rw##Q = *reinterpret_cast<const float4*>(                                                    \
        W + (size_t)(((Q) >> 1) * H + c0 + ((i_ >> 3) & 63)) * H + (H0) + (i_ & 7) * 4);          \
    rs##Q = *reinterpret_cast<const float4*>(sb + (size_t)((H0) + (i_ >> 5)) * L + t0 +          \
                                             (i_ & 31) * 4);                                     \
  } while (0)
#define PROJ_STAGE(Q, DST)                                                                       \
  do {                                                                                           \
    const int i_ = tid + (Q) * kPThreads;                                                        \
    float* d_ = &DST[(i_ >> 3) & 63][(i_ & 7) * 4];                                              \
    d_[0] = rw##Q.x;                                                                             \
    d_[1] = rw##Q.y;                                                                             \
    d_[2] = rw##Q.z;                                                                             \
    d_[3] = rw##Q.w;                                                                             \
    *reinterpret_cast<float4*>(&sS[i_ >> 5][(i_ & 31) * 4]) = rs##Q;                             \
  } while (0)
  v16f acc_a0 = {}, acc_a1 = {}, acc_g0 = {}, acc_g1 = {};
  if (vec) {
    PROJ_FETCH(0, 0);
    PROJ_FETCH(1, 0);
    PROJ_FETCH(2, 0);
    PROJ_FETCH(3, 0);
  }
  for (int h0 = 0; h0 < H; h0 += kPK) {
    if (vec) {
      PROJ_STAGE(0, sWa);
      PROJ_STAGE(1, sWa);
      PROJ_STAGE(2, sWg);
      PROJ_STAGE(3, sWg);
    } else {
      for (int i = tid; i < kPM * kPK; i += kPThreads) {
        const int r = i / kPK, k = i % kPK;
        const int c = c0 + r, h = h0 + k;
        const bool ok = c < H && h < H;
        sWa[r][k] = ok ? W[(size_t)c * H + h] : 0.f;
        sWg[r][k] = ok ? W[(size_t)(H + c) * H + h] : 0.f;
      }
      for (int i = tid; i < kPK * kPN; i += kPThreads) {
        const int k = i / kPN, n = i % kPN;
        const int h = h0 + k, t = t0 + n;
        sS[k][n] = (h < H && t < L) ? sb[(size_t)h * L + t] : 0.f;
      }
    }
    __syncthreads();
    if (vec && h0 + kPK < H) {   // the next stage's loads, in flight during the MFMAs
      PROJ_FETCH(0, h0 + kPK);
      PROJ_FETCH(1, h0 + kPK);
      PROJ_FETCH(2, h0 + kPK);
      PROJ_FETCH(3, h0 + kPK);
    }
#pragma unroll
    for (int kk = 0; kk < kPK; kk += 2) {
      const int k = kk + (lane >> 5), i = lane & 31;
      const float av = sWa[cw + i][k], gv = sWg[cw + i][k];
      const float b0 = sS[k][tw + i], b1 = sS[k][tw + 32 + i];
      acc_a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc_a0, 0, 0, 0);
      acc_a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc_a1, 0, 0, 0);
      acc_g0 = __builtin_amdgcn_mfma_f32_32x32x2f32(gv, b0, acc_g0, 0, 0, 0);
      acc_g1 = __builtin_amdgcn_mfma_f32_32x32x2f32(gv, b1, acc_g1, 0, 0, 0);
    }
    __syncthreads();
  }
  // accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4,
  // column l % 32 of the 32 x 32 tile
  const size_t base = (size_t)b * H * L;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int c = c0 + cw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (c >= H) continue;
    const float ba = bias[c], bg = bias[H + c];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = t0 + tw + 32 * j + (lane & 31);
      if (t >= L) continue;
      const float a = (j ? acc_a1[r] : acc_a0[r]) + ba;
      const float g = (j ? acc_g1[r] : acc_g0[r]) + bg;
      const size_t o = base + (size_t)c * L + t;
      out[o] = x[o] + a * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
    }
  }
#undef PROJ_FETCH
#undef PROJ_STAGE
}

hipError_t launch_block_epilogue(const s4dplr_plan* p, const float* x, const float* s,
                                 const float* W, const float* bias, float* out, hipStream_t st) {
  const dim3 grid((p->L + kPN - 1) / kPN, (p->H + kPM - 1) / kPM, p->batch);
  glu_proj_kernel<<<grid, kPThreads, 0, st>>>(x, s, W, bias, out, p->H, p->L);
  return hipGetLastError();
}

hipError_t launch_layer_norm(const s4dplr_plan* p, const float* x, const float* gamma,
                             const float* beta, float* z, hipStream_t st) {
  const dim3 grid((p->L + 63) / 64, p->batch);
  layer_norm_kernel<<<grid, kLnThreads, 0, st>>>(x, gamma, beta, z, p->H, p->L, 1e-5f);
  return hipGetLastError();
}

}  // namespace s4
