// The block around the layer ("The S4 kernel, from scratch", section 6: a
// pre-norm, a GLU-gated projection and a residual connection):
//   z   = LayerNorm over the H channels at every (b, t), with gain and shift,
//   s   = the layer applied to z (kernel generation + causal convolution),
//   out = x + a * sigmoid(g),  [a; g] = W s + bias,  W: (2H x H).
//
// The projection is the block's only dense contraction: per batch row it is a
// GEMM with M = H output channels (for each of the two halves), N = L time
// steps and K = H input channels, done on the bf16 matrix cores with split
// operands (three products per k) so that the block keeps fp32 accuracy.  The
// bias, the gate and the residual are applied to the accumulators in
// registers.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace s4 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kLnThreads = 256;
// Projection tile: 128 time steps by K stages of 32 channels (the channel
// extent of a tile is the kernel's template argument).
constexpr int kPN = 128, kPK = 32;

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
// W is split once per call by split_w_kernel (every tile reads it); s is
// split while staged.  A block owns CM channels x 128 time steps of both
// halves, CM = 128 when H allows it (s is then split by half as many blocks),
// else 64; wave w owns channels [32 (w / 2), +32) and time steps
// [64 (w % 2), +64) as two 32 x 32 tiles per half.  Each K stage of 32
// channels stages CM rows x 32 of each W part as [row][k] and 32 x 128 of s
// transposed as [t][k] through LDS, so that a lane's eight consecutive k of
// an operand are one 16-byte read; the next stage's global loads are issued
// before the current stage's MFMAs.  Fully in-range tiles take the vector
// path; edge tiles load element by element with zero fill.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  // round to nearest even; finite inputs
  const unsigned int u = __float_as_uint(x);
  return (unsigned short)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_value(unsigned short b) {
  return __uint_as_float((unsigned int)b << 16);
}
__device__ __forceinline__ void split_bf16(float x, unsigned short& hi, unsigned short& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - bf16_value(hi));
}

// Wp[part][r][h] (part 0 = hi, 1 = lo) for the 2H x H matrix W
__global__ __launch_bounds__(256) void split_w_kernel(const float* __restrict__ W,
                                                      unsigned short* __restrict__ Wp,
                                                      size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  unsigned short hi, lo;
  split_bf16(W[i], hi, lo);
  Wp[i] = hi;
  Wp[n + i] = lo;
}

constexpr int kPKP = kPK + 8;   // padded k extent of a staged row (bf16 elements)

template <int CM>
__global__ __launch_bounds__(CM * 4) void glu_proj_kernel(
    const float* x, const float* __restrict__ s, const unsigned short* __restrict__ Wp,
    const float* __restrict__ bias, float* out, int H, int L) {
  constexpr int NT = CM * 4;                       // threads: 2 (CM / 32) waves
  // W slots: 2 parts x 2 halves x CM rows x 32 k = 16 CM uint4 (8 bf16 each);
  // s slots: 32 x 128 floats = 1024 float4, taken as channel pairs
  constexpr int NWQ = 16 * CM / NT;                // uint4 of W per thread (4)
  constexpr int NSG = 512 / NT;                    // groups of 8 channels of s per thread
  static_assert(NWQ == 4 && (NSG == 1 || NSG == 2), "tile shape");
  __shared__ __attribute__((aligned(16))) unsigned short sWa[2][CM][kPKP];
  __shared__ __attribute__((aligned(16))) unsigned short sWg[2][CM][kPKP];
  __shared__ __attribute__((aligned(16))) unsigned short sS[2][kPN][kPKP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.z, c0 = blockIdx.y * CM, t0 = blockIdx.x * kPN;
  const int cw = 32 * (w >> 1), tw = 64 * (w & 1);
  const float* sb = s + (size_t)b * H * L;
  const size_t nW = (size_t)2 * H * H;
  const bool vec = (H % kPK == 0) && (c0 + CM <= H) && (t0 + kPN <= L) && (L % 4 == 0);
  // W slots in named registers (indexed through a macro argument); s slots in
  // an array indexed by unrolled loops only
  uint4 rw0, rw1, rw2, rw3;
  float rs[NSG * 8];
  // W slot i in [0, 16 CM): part = i / (8 CM), half = (i / (4 CM)) & 1,
  // row = (i >> 2) % CM, k = 8 (i & 3)
#define PROJ_FETCH_W(Q, H0)                                                                      \
  do {                                                                                           \
    const int i_ = tid + (Q) * NT;                                                               \
    const int part_ = i_ / (8 * CM), half_ = (i_ / (4 * CM)) & 1, r_ = (i_ >> 2) % CM;           \
    rw##Q = *reinterpret_cast<const uint4*>(Wp + part_ * nW +                                    \
                                            (size_t)(half_ * H + c0 + r_) * H + (H0) +           \
                                            8 * (i_ & 3));                                       \
  } while (0)
#define PROJ_STAGE_W(Q)                                                                          \
  do {                                                                                           \
    const int i_ = tid + (Q) * NT;                                                               \
    const int part_ = i_ / (8 * CM), half_ = (i_ / (4 * CM)) & 1, r_ = (i_ >> 2) % CM;           \
    unsigned short* d_ = half_ ? &sWg[part_][r_][8 * (i_ & 3)] : &sWa[part_][r_][8 * (i_ & 3)];  \
    *reinterpret_cast<uint4*>(d_) = rw##Q;                                                       \
  } while (0)
  // s slots: thread tid takes time step t0 + (tid & 127) and channels
  // h0 + 8 g + j, j < 8, of its groups g = (tid >> 7) + (NT / 128) G; the
  // loads are coalesced over the lanes' consecutive time steps, and each group
  // is one 16-byte LDS store per part (rows 80 bytes apart: no bank conflicts)
#define PROJ_FETCH_S(H0)                                                                         \
  do {                                                                                           \
    _Pragma("unroll") for (int G_ = 0; G_ < NSG; ++G_) {                                         \
      const int g_ = (tid >> 7) + (NT / 128) * G_;                                               \
      const float* r_ = sb + (size_t)((H0) + 8 * g_) * L + t0 + (tid & 127);                     \
      _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) rs[G_ * 8 + j_] = r_[(size_t)j_ * L];     \
    }                                                                                            \
  } while (0)
#define PROJ_STAGE_S()                                                                           \
  do {                                                                                           \
    _Pragma("unroll") for (int G_ = 0; G_ < NSG; ++G_) {                                         \
      const int g_ = (tid >> 7) + (NT / 128) * G_;                                               \
      unsigned short h_[8], l_[8];                                                               \
      _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) split_bf16(rs[G_ * 8 + j_], h_[j_], l_[j_]); \
      *reinterpret_cast<uint4*>(&sS[0][tid & 127][8 * g_]) =                                     \
          make_uint4(h_[0] | ((unsigned)h_[1] << 16), h_[2] | ((unsigned)h_[3] << 16),           \
                     h_[4] | ((unsigned)h_[5] << 16), h_[6] | ((unsigned)h_[7] << 16));          \
      *reinterpret_cast<uint4*>(&sS[1][tid & 127][8 * g_]) =                                     \
          make_uint4(l_[0] | ((unsigned)l_[1] << 16), l_[2] | ((unsigned)l_[3] << 16),           \
                     l_[4] | ((unsigned)l_[5] << 16), l_[6] | ((unsigned)l_[7] << 16));          \
    }                                                                                            \
  } while (0)
  v16f acc_a0 = {}, acc_a1 = {}, acc_g0 = {}, acc_g1 = {};
  if (vec) {
    PROJ_FETCH_W(0, 0);
    PROJ_FETCH_W(1, 0);
    PROJ_FETCH_W(2, 0);
    PROJ_FETCH_W(3, 0);
    PROJ_FETCH_S(0);
  }
  for (int h0 = 0; h0 < H; h0 += kPK) {
    if (vec) {
      PROJ_STAGE_W(0);
      PROJ_STAGE_W(1);
      PROJ_STAGE_W(2);
      PROJ_STAGE_W(3);
      PROJ_STAGE_S();
    } else {
      for (int i = tid; i < CM * kPK; i += NT) {
        const int r = i / kPK, k = i % kPK;
        const int c = c0 + r, h = h0 + k;
        const bool ok = c < H && h < H;
        const size_t ia = (size_t)c * H + h, ig = (size_t)(H + c) * H + h;
        sWa[0][r][k] = ok ? Wp[ia] : 0;
        sWa[1][r][k] = ok ? Wp[nW + ia] : 0;
        sWg[0][r][k] = ok ? Wp[ig] : 0;
        sWg[1][r][k] = ok ? Wp[nW + ig] : 0;
      }
      for (int i = tid; i < kPK * kPN; i += NT) {
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
      PROJ_FETCH_S(h0 + kPK);
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
}

hipError_t launch_block_epilogue(const s4dplr_plan* p, const float* x, const float* s,
                                 const float* W, const float* bias, float* out,
                                 unsigned char* ws, hipStream_t st) {
  unsigned short* Wp = reinterpret_cast<unsigned short*>(ws + p->off_bw);
  const size_t nW = (size_t)2 * p->H * p->H;
  split_w_kernel<<<(unsigned)((nW + 255) / 256), 256, 0, st>>>(W, Wp, nW);
  if (p->H % 128 == 0) {
    const dim3 grid((p->L + kPN - 1) / kPN, p->H / 128, p->batch);
    glu_proj_kernel<128><<<grid, 512, 0, st>>>(x, s, Wp, bias, out, p->H, p->L);
  } else {
    const dim3 grid((p->L + kPN - 1) / kPN, (p->H + 63) / 64, p->batch);
    glu_proj_kernel<64><<<grid, 256, 0, st>>>(x, s, Wp, bias, out, p->H, p->L);
  }
  return hipGetLastError();
}

hipError_t launch_layer_norm(const s4dplr_plan* p, const float* x, const float* gamma,
                             const float* beta, float* z, hipStream_t st) {
  const dim3 grid((p->L + 63) / 64, p->batch);
  layer_norm_kernel<<<grid, kLnThreads, 0, st>>>(x, gamma, beta, z, p->H, p->L, 1e-5f);
  return hipGetLastError();
}

}  // namespace s4
