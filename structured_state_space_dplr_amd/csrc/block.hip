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
// z[b][h][t] = (x - mean) rstd gamma_h + beta_h.
__global__ __launch_bounds__(kLnThreads) void layer_norm_kernel(
    const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
    float* __restrict__ z, int H, int L, float eps) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * kLnThreads + threadIdx.x;
  if (t >= L) return;
  const float* xb = x + (size_t)b * H * L + t;
  double s1 = 0.0, s2 = 0.0;
  for (int h = 0; h < H; ++h) {
    const double v = (double)xb[(size_t)h * L];
    s1 += v;
    s2 += v * v;
  }
  const double mean = s1 / H;
  const double var = fmax(s2 / H - mean * mean, 0.0);
  const float m = (float)mean, r = (float)(1.0 / sqrt(var + (double)eps));
  float* zb = z + (size_t)b * H * L + t;
  for (int h = 0; h < H; ++h) {
    const size_t o = (size_t)h * L;
    zb[o] = fmaf((xb[o] - m) * r, gamma[h], beta[h]);
  }
}

// out[b][c][t] = x[b][c][t] + (Wa s + ba)[c][t] * sigmoid((Wg s + bg)[c][t]).
// out may be x itself: every element is read and then written by one lane.
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
  v16f acc_a0 = {}, acc_a1 = {}, acc_g0 = {}, acc_g1 = {};
  for (int h0 = 0; h0 < H; h0 += kPK) {
    // stage W rows [c0, c0 + 64) of both halves and s rows [h0, h0 + 32)
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
    __syncthreads();
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
      out[o] = x[o] + a / (1.0f + expf(-g));
    }
  }
}

hipError_t launch_block_epilogue(const s4dplr_plan* p, const float* x, const float* s,
                                 const float* W, const float* bias, float* out, hipStream_t st) {
  const dim3 grid((p->L + kPN - 1) / kPN, (p->H + kPM - 1) / kPM, p->batch);
  glu_proj_kernel<<<grid, kPThreads, 0, st>>>(x, s, W, bias, out, p->H, p->L);
  return hipGetLastError();
}

hipError_t launch_layer_norm(const s4dplr_plan* p, const float* x, const float* gamma,
                             const float* beta, float* z, hipStream_t st) {
  const dim3 grid((p->L + kLnThreads - 1) / kLnThreads, p->batch);
  layer_norm_kernel<<<grid, kLnThreads, 0, st>>>(x, gamma, beta, z, p->H, p->L, 1e-5f);
  return hipGetLastError();
}

}  // namespace s4
