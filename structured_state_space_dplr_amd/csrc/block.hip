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
//
// The products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) with
// fp32 accuracy kept by splitting every operand into two bf16 parts,
// w = w_hi + w_lo with w_hi = bf16(w) and w_lo = bf16(w - w_hi) (16
// significant bits together), and summing the three products
// w_hi s_hi + w_hi s_lo + w_lo s_hi in the fp32 accumulators; the dropped
// w_lo s_lo and the split's own rounding are below 2^-16 relative per term.
// Each K stage of 32 channels stages 64 rows x 32 of each W half as [row][k]
// and 32 x 128 of s transposed as [t][k] through LDS, both split, so that a
// lane's eight consecutive k of an operand are one 16-byte read; the next
// stage's global loads are issued before the current stage's MFMAs.  Fully
// in-range tiles (H % 32 == 0 and L % 128 == 0 here) take the vector path;
// edge tiles load element by element with zero fill.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  // round to nearest even; finite inputs
  const unsigned int u = __float_as_uint(x);
  return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_value(unsigned short b) {
  return __uint_as_float((unsigned int)b << 16);
}
// hi and lo parts of x
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_value(hi));
}

constexpr int kPKP = kPK + 8;   // padded k extent of a staged row (bf16 elements)

__global__ __launch_bounds__(kPThreads) void glu_proj_kernel(
    const float* x, const float* __restrict__ s, const float* __restrict__ W,
    const float* __restrict__ bias, float* out, int H, int L) {
  // [part][row][k]: part 0 = hi, 1 = lo
  __shared__ __attribute__((aligned(16))) unsigned short sWa[2][kPM][kPKP];
  __shared__ __attribute__((aligned(16))) unsigned short sWg[2][kPM][kPKP];
  __shared__ __attribute__((aligned(16))) unsigned short sS[2][kPN][kPKP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.z, c0 = blockIdx.y * kPM, t0 = blockIdx.x * kPN;
  const int cw = 32 * (w >> 1), tw = 64 * (w & 1);
  const float* sb = s + (size_t)b * H * L;
  const bool vec = (H % kPK == 0) && (c0 + kPM <= H) && (t0 + kPN <= L) && (L % 4 == 0);
  // float4 slots of a stage, in named registers (an indexed array here ends
  // up in scratch memory): W slot Q of thread tid is i = tid + 256 Q (half
  // Q / 2, row (i >> 3) & 63, k 4 (i & 7)); s slots Q = 0, 1 hold channels
  // 2p and 2p + 1, p = (tid >> 5) + 8 Q, of time steps 4 (tid & 31) .. + 3
  float4 rw0, rw1, rw2, rw3, rs0, rs1, rs2, rs3;
#define PROJ_FETCH_W(Q, H0)                                                                      \
  do {                                                                                           \
    const int i_ = tid + (Q) * kPThreads;                                                        \
    rw##Q = *reinterpret_cast<const float4*>(                                                    \
        W + (size_t)(((Q) >> 1) * H + c0 + ((i_ >> 3) & 63)) * H + (H0) + (i_ & 7) * 4);          \
  } while (0)
#define PROJ_FETCH_S(Q, H0)                                                                      \
  do {                                                                                           \
    const int p_ = (tid >> 5) + 8 * (Q);                                                         \
    const float* r_ = sb + (size_t)((H0) + 2 * p_) * L + t0 + (tid & 31) * 4;                    \
    rs##Q = *reinterpret_cast<const float4*>(r_);                                                \
    rs##Q##b = *reinterpret_cast<const float4*>(r_ + L);                                         \
  } while (0)
#define PROJ_STAGE_W(Q, DST)                                                                     \
  do {                                                                                           \
    const int i_ = tid + (Q) * kPThreads;                                                        \
    const int r_ = (i_ >> 3) & 63, k_ = (i_ & 7) * 4;                                            \
    unsigned short h_[4], l_[4];                                                                 \
    split_bf16(rw##Q.x, h_[0], l_[0]);                                                           \
    split_bf16(rw##Q.y, h_[1], l_[1]);                                                           \
    split_bf16(rw##Q.z, h_[2], l_[2]);                                                           \
    split_bf16(rw##Q.w, h_[3], l_[3]);                                                           \
    *reinterpret_cast<uint2*>(&DST[0][r_][k_]) =                                                 \
        make_uint2(h_[0] | ((unsigned)h_[1] << 16), h_[2] | ((unsigned)h_[3] << 16));            \
    *reinterpret_cast<uint2*>(&DST[1][r_][k_]) =                                                 \
        make_uint2(l_[0] | ((unsigned)l_[1] << 16), l_[2] | ((unsigned)l_[3] << 16));            \
  } while (0)
#define PROJ_STAGE_S1(T_, A_, B_)                                                                \
  do {                                                                                           \
    unsigned short ha_, la_, hb_, lb_;                                                           \
    split_bf16(A_, ha_, la_);                                                                    \
    split_bf16(B_, hb_, lb_);                                                                    \
    *reinterpret_cast<unsigned int*>(&sS[0][T_][2 * p_]) = ha_ | ((unsigned)hb_ << 16);          \
    *reinterpret_cast<unsigned int*>(&sS[1][T_][2 * p_]) = la_ | ((unsigned)lb_ << 16);          \
  } while (0)
#define PROJ_STAGE_S(Q)                                                                          \
  do {                                                                                           \
    const int p_ = (tid >> 5) + 8 * (Q), tt_ = (tid & 31) * 4;                                   \
    PROJ_STAGE_S1(tt_ + 0, rs##Q.x, rs##Q##b.x);                                                 \
    PROJ_STAGE_S1(tt_ + 1, rs##Q.y, rs##Q##b.y);                                                 \
    PROJ_STAGE_S1(tt_ + 2, rs##Q.z, rs##Q##b.z);                                                 \
    PROJ_STAGE_S1(tt_ + 3, rs##Q.w, rs##Q##b.w);                                                 \
  } while (0)
  float4 rs0b, rs1b;
  (void)rs2;
  (void)rs3;
  v16f acc_a0 = {}, acc_a1 = {}, acc_g0 = {}, acc_g1 = {};
  if (vec) {
    PROJ_FETCH_W(0, 0);
    PROJ_FETCH_W(1, 0);
    PROJ_FETCH_W(2, 0);
    PROJ_FETCH_W(3, 0);
    PROJ_FETCH_S(0, 0);
    PROJ_FETCH_S(1, 0);
  }
  for (int h0 = 0; h0 < H; h0 += kPK) {
    if (vec) {
      PROJ_STAGE_W(0, sWa);
      PROJ_STAGE_W(1, sWa);
      PROJ_STAGE_W(2, sWg);
      PROJ_STAGE_W(3, sWg);
      PROJ_STAGE_S(0);
      PROJ_STAGE_S(1);
    } else {
      for (int i = tid; i < kPM * kPK; i += kPThreads) {
        const int r = i / kPK, k = i % kPK;
        const int c = c0 + r, h = h0 + k;
        const bool ok = c < H && h < H;
        unsigned short hi, lo;
        split_bf16(ok ? W[(size_t)c * H + h] : 0.f, hi, lo);
        sWa[0][r][k] = hi;
        sWa[1][r][k] = lo;
        split_bf16(ok ? W[(size_t)(H + c) * H + h] : 0.f, hi, lo);
        sWg[0][r][k] = hi;
        sWg[1][r][k] = lo;
      }
      for (int i = tid; i < kPK * kPN; i += kPThreads) {
        const int k = i / kPN, n = i % kPN;
        const int h = h0 + k, t = t0 + n;
        unsigned short hi, lo;
        split_bf16((h < H && t < L) ? sb[(size_t)h * L + t] : 0.f, hi, lo);
        sS[0][n][k] = hi;
        sS[1][n][k] = lo;
      }
    }
    __syncthreads();
    if (vec && h0 + kPK < H) {   // the next stage's loads, in flight during the MFMAs
      PROJ_FETCH_W(0, h0 + kPK);
      PROJ_FETCH_W(1, h0 + kPK);
      PROJ_FETCH_W(2, h0 + kPK);
      PROJ_FETCH_W(3, h0 + kPK);
      PROJ_FETCH_S(0, h0 + kPK);
      PROJ_FETCH_S(1, h0 + kPK);
    }
    // lane l: operand rows/columns l % 32, k = kk + 8 (l / 32) .. + 7
    const int i = lane & 31, kq = 8 * (lane >> 5);
#pragma unroll
    for (int kk = 0; kk < kPK; kk += 16) {
      const v8bf ah = *reinterpret_cast<const v8bf*>(&sWa[0][cw + i][kk + kq]);
      const v8bf al = *reinterpret_cast<const v8bf*>(&sWa[1][cw + i][kk + kq]);
      const v8bf gh = *reinterpret_cast<const v8bf*>(&sWg[0][cw + i][kk + kq]);
      const v8bf gl = *reinterpret_cast<const v8bf*>(&sWg[1][cw + i][kk + kq]);
      const v8bf b0h = *reinterpret_cast<const v8bf*>(&sS[0][tw + i][kk + kq]);
      const v8bf b0l = *reinterpret_cast<const v8bf*>(&sS[1][tw + i][kk + kq]);
      const v8bf b1h = *reinterpret_cast<const v8bf*>(&sS[0][tw + 32 + i][kk + kq]);
      const v8bf b1l = *reinterpret_cast<const v8bf*>(&sS[1][tw + 32 + i][kk + kq]);
      acc_a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b0h, acc_a0, 0, 0, 0);
      acc_a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b1h, acc_a1, 0, 0, 0);
      acc_g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, b0h, acc_g0, 0, 0, 0);
      acc_g1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, b1h, acc_g1, 0, 0, 0);
      acc_a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b0l, acc_a0, 0, 0, 0);
      acc_a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b1l, acc_a1, 0, 0, 0);
      acc_g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, b0l, acc_g0, 0, 0, 0);
      acc_g1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, b1l, acc_g1, 0, 0, 0);
      acc_a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b0h, acc_a0, 0, 0, 0);
      acc_a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b1h, acc_a1, 0, 0, 0);
      acc_g0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gl, b0h, acc_g0, 0, 0, 0);
      acc_g1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gl, b1h, acc_g1, 0, 0, 0);
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
#undef PROJ_FETCH_W
#undef PROJ_FETCH_S
#undef PROJ_STAGE_W
#undef PROJ_STAGE_S
#undef PROJ_STAGE_S1
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
