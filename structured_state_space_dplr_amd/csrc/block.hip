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
// Projection tiles: K stages of 32 channels; 128 time steps per tile for
// 64-channel tiles, 2 * 128 = 256 for 128-channel tiles (the channel and time
// extents of a tile are the kernel's template arguments).
constexpr int kPN = 128, kPK = 32;

}  // namespace

// mean and 1/sqrt(var + eps) over h of x[b][h][t] (fp64 sums), then
// z[b][h][t] = (x - mean) rstd gamma_h + beta_h.  Block (64 time steps, b):
// wave g sums the channels h = g, g + 4, ... of its lane's time step; the four
// partial sums meet in LDS, and the normalization is split the same way.
// HPT > 0 (H = 4 HPT): the thread keeps its HPT values of x in registers
// between the two steps, so x is read from memory once; HPT = 0: any H, x is
// read again for the normalization.
template <int HPT>
__global__ __launch_bounds__(kLnThreads) void layer_norm_kernel(
    const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ beta,
    float* __restrict__ z, int H, int L, float eps) {
  constexpr int G = kLnThreads / 64;
  __shared__ double red[2][G][64];
  __shared__ float stat[2][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x * 64 + lane;
  const bool on = t < L;
  const float* xb = x + (size_t)b * H * L + t;
  float xv[HPT > 0 ? HPT : 1];
  double s1 = 0.0, s2 = 0.0;
  if (on) {
    if constexpr (HPT > 0) {
#pragma unroll
      for (int i = 0; i < HPT; ++i) xv[i] = xb[(size_t)(g + G * i) * L];
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const double v = (double)xv[i];
        s1 += v;
        s2 += v * v;
      }
    } else {
#pragma unroll 8
      for (int h = g; h < H; h += G) {
        const double v = (double)xb[(size_t)h * L];
        s1 += v;
        s2 += v * v;
      }
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
  if constexpr (HPT > 0) {
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int h = g + G * i;
      zb[(size_t)h * L] = fmaf((xv[i] - m) * r, gamma[h], beta[h]);
    }
  } else {
#pragma unroll 8
    for (int h = g; h < H; h += G) {
      const size_t o = (size_t)h * L;
      zb[o] = fmaf((xb[o] - m) * r, gamma[h], beta[h]);
    }
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
// split while staged.  A block owns CM channels x TN time steps of both
// halves: CM = 128 and TN = 256 (512 threads) when H is a multiple of 128,
// else CM = 64 and TN = 128 (256 threads); wave w owns channels
// [32 (w / 2), +32) and time steps [(TN / 2) (w % 2), +TN / 2) as TN / 64
// 32 x 32 tiles per half.  Each K stage of 32 channels stages CM rows x 32 of
// each W part as [row][k] and 32 x TN of s as [t][k] through double-buffered
// LDS, so that a lane's eight consecutive k of an operand are one 16-byte
// read; the next stage's global loads are issued before the current stage's
// MFMAs.  Fully in-range tiles take the vector
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


// Offset (bf16 elements) of the 16-byte chunk c (k = 8 c .. 8 c + 7) of row r
// in a staged [row][32] operand: 64-byte rows with the chunk index XORed by
// (r / 4) mod 4, so that 16-byte reads of 32 consecutive rows at one chunk and
// 16-byte writes of consecutive rows or chunks meet no bank conflicts.
__device__ __forceinline__ int swz(int r, int c) { return 32 * r + 8 * (c ^ ((r >> 2) & 3)); }

template <int CM, int TN>
__global__ __launch_bounds__(CM * 4) void glu_proj_kernel(
    const float* x, const float* __restrict__ s, const unsigned short* __restrict__ Wp,
    const float* __restrict__ bias, float* out, int H, int L) {
  constexpr int NT = CM * 4;                       // threads: 2 (CM / 32) waves
  constexpr int JT = TN / 64;                      // 32 x 32 tiles per half and wave
  // W slots: 2 parts x 2 halves x CM rows x 32 k = 16 CM uint4 (8 bf16 each);
  // s slots: TN time steps x 4 groups of 8 channels
  constexpr int NWQ = 16 * CM / NT;                // uint4 of W per thread (4)
  constexpr int NSG = 4 * TN / NT;                 // groups of 8 channels of s per thread
  static_assert(NWQ == 4 && NSG >= 1 && NSG <= 4 && (NT % TN == 0 || TN % NT == 0), "tile shape");
  static_assert(kPK == 32, "swizzle assumes 32-channel stages");
  // two buffers of each staged operand: stage k is read from buffer k % 2
  // while stage k + 1 is written to the other
  constexpr int WB = 2 * 2 * CM * kPK;             // [half][part][row][32] per buffer
  constexpr int SB = 2 * TN * kPK;                 // [part][t][32] per buffer
  __shared__ __attribute__((aligned(16))) unsigned short sW[2 * WB];
  __shared__ __attribute__((aligned(16))) unsigned short sS[2 * SB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.z, c0 = blockIdx.y * CM, t0 = blockIdx.x * TN;
  const int cw = 32 * (w >> 1), tw = (TN / 2) * (w & 1);
  const float* sb = s + (size_t)b * H * L;
  const size_t nW = (size_t)2 * H * H;
  const bool vec = (H % kPK == 0) && (c0 + CM <= H) && (t0 + TN <= L);
  auto wofs = [](int half, int part, int r, int c) { return ((half * 2 + part) * CM) * kPK + swz(r, c); };
  auto sofs = [](int part, int t, int c) { return part * TN * kPK + swz(t, c); };
  // W slots in named registers (indexed through a macro argument); s slots in
  // an array indexed by unrolled loops only
  uint4 rw0, rw1, rw2, rw3;
  float rs[NSG * 8];
  // W slot i in [0, 16 CM): part = i / (8 CM), half = (i / (4 CM)) & 1,
  // row = (i >> 2) % CM, chunk = i & 3
#define PROJ_FETCH_W(Q, H0)                                                                      \
  do {                                                                                           \
    const int i_ = tid + (Q) * NT;                                                               \
    const int part_ = i_ / (8 * CM), half_ = (i_ / (4 * CM)) & 1, r_ = (i_ >> 2) % CM;           \
    rw##Q = *reinterpret_cast<const uint4*>(Wp + part_ * nW +                                    \
                                            (size_t)(half_ * H + c0 + r_) * H + (H0) +           \
                                            8 * (i_ & 3));                                       \
  } while (0)
#define PROJ_STAGE_W(Q, BUF)                                                                     \
  do {                                                                                           \
    const int i_ = tid + (Q) * NT;                                                               \
    const int part_ = i_ / (8 * CM), half_ = (i_ / (4 * CM)) & 1, r_ = (i_ >> 2) % CM;           \
    *reinterpret_cast<uint4*>(&sW[(BUF) * WB + wofs(half_, part_, r_, i_ & 3)]) = rw##Q;         \
  } while (0)
  // s slots: thread tid takes time step t0 + tid % TN and channels h0 + 8 g + j,
  // j < 8, of its groups g = tid / TN + (NT / TN) G; the loads are coalesced
  // over the lanes' consecutive time steps, and each group is one 16-byte LDS
  // store per part
#define PROJ_FETCH_S(H0)                                                                         \
  do {                                                                                           \
    _Pragma("unroll") for (int G_ = 0; G_ < NSG; ++G_) {                                         \
      const int g_ = tid / TN + (NT / TN) * G_;                                                  \
      const float* r_ = sb + (size_t)((H0) + 8 * g_) * L + t0 + tid % TN;                        \
      _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) rs[G_ * 8 + j_] = r_[(size_t)j_ * L];     \
    }                                                                                            \
  } while (0)
#define PROJ_STAGE_S(BUF)                                                                        \
  do {                                                                                           \
    _Pragma("unroll") for (int G_ = 0; G_ < NSG; ++G_) {                                         \
      const int g_ = tid / TN + (NT / TN) * G_;                                                  \
      unsigned short h_[8], l_[8];                                                               \
      _Pragma("unroll") for (int j_ = 0; j_ < 8; ++j_) split_bf16(rs[G_ * 8 + j_], h_[j_], l_[j_]); \
      *reinterpret_cast<uint4*>(&sS[(BUF) * SB + sofs(0, tid % TN, g_)]) =                       \
          make_uint4(h_[0] | ((unsigned)h_[1] << 16), h_[2] | ((unsigned)h_[3] << 16),           \
                     h_[4] | ((unsigned)h_[5] << 16), h_[6] | ((unsigned)h_[7] << 16));          \
      *reinterpret_cast<uint4*>(&sS[(BUF) * SB + sofs(1, tid % TN, g_)]) =                       \
          make_uint4(l_[0] | ((unsigned)l_[1] << 16), l_[2] | ((unsigned)l_[3] << 16),           \
                     l_[4] | ((unsigned)l_[5] << 16), l_[6] | ((unsigned)l_[7] << 16));          \
    }                                                                                            \
  } while (0)
  // edge tiles: element by element with zero fill
  auto stage_elements = [&](int h0, int buf) {
    for (int i = tid; i < CM * kPK; i += NT) {
      const int r = i / kPK, k = i % kPK;
      const int c = c0 + r, h = h0 + k;
      const bool ok = c < H && h < H;
      const size_t ia = (size_t)c * H + h, ig = (size_t)(H + c) * H + h;
      const int o = buf * WB + (k & 7);
      sW[o + wofs(0, 0, r, k >> 3)] = ok ? Wp[ia] : 0;
      sW[o + wofs(0, 1, r, k >> 3)] = ok ? Wp[nW + ia] : 0;
      sW[o + wofs(1, 0, r, k >> 3)] = ok ? Wp[ig] : 0;
      sW[o + wofs(1, 1, r, k >> 3)] = ok ? Wp[nW + ig] : 0;
    }
    for (int i = tid; i < kPK * TN; i += NT) {
      const int k = i / TN, n = i % TN;
      const int h = h0 + k, t = t0 + n;
      unsigned short hi, lo;
      split_bf16((h < H && t < L) ? sb[(size_t)h * L + t] : 0.f, hi, lo);
      sS[buf * SB + sofs(0, n, k >> 3) + (k & 7)] = hi;
      sS[buf * SB + sofs(1, n, k >> 3) + (k & 7)] = lo;
    }
  };
  v16f acc_a[JT], acc_g[JT];
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    acc_a[j] = v16f{};
    acc_g[j] = v16f{};
  }
  const int nst = (H + kPK - 1) / kPK;
  if (vec) {
    PROJ_FETCH_W(0, 0);
    PROJ_FETCH_W(1, 0);
    PROJ_FETCH_W(2, 0);
    PROJ_FETCH_W(3, 0);
    PROJ_FETCH_S(0);
    PROJ_STAGE_W(0, 0);
    PROJ_STAGE_W(1, 0);
    PROJ_STAGE_W(2, 0);
    PROJ_STAGE_W(3, 0);
    PROJ_STAGE_S(0);
    if (nst > 1) {
      PROJ_FETCH_W(0, kPK);
      PROJ_FETCH_W(1, kPK);
      PROJ_FETCH_W(2, kPK);
      PROJ_FETCH_W(3, kPK);
      PROJ_FETCH_S(kPK);
    }
  } else {
    stage_elements(0, 0);
  }
  __syncthreads();
  // lane l: operand rows/columns l % 32, k = kk + 8 (l / 32) .. + 7
  const int i = lane & 31, kq = lane >> 5;
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const unsigned short* bW = sW + cur * WB;
    const unsigned short* bS = sS + cur * SB;
#pragma unroll
    for (int kc = 0; kc < 4; kc += 2) {           // 16-channel halves of the stage
      const v8bf ah = *reinterpret_cast<const v8bf*>(&bW[wofs(0, 0, cw + i, kc + kq)]);
      const v8bf al = *reinterpret_cast<const v8bf*>(&bW[wofs(0, 1, cw + i, kc + kq)]);
      const v8bf gh = *reinterpret_cast<const v8bf*>(&bW[wofs(1, 0, cw + i, kc + kq)]);
      const v8bf gl = *reinterpret_cast<const v8bf*>(&bW[wofs(1, 1, cw + i, kc + kq)]);
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const v8bf bh = *reinterpret_cast<const v8bf*>(&bS[sofs(0, tw + 32 * j + i, kc + kq)]);
        const v8bf bl = *reinterpret_cast<const v8bf*>(&bS[sofs(1, tw + 32 * j + i, kc + kq)]);
        acc_a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc_a[j], 0, 0, 0);
        acc_g[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, bh, acc_g[j], 0, 0, 0);
        acc_a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc_a[j], 0, 0, 0);
        acc_g[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, bl, acc_g[j], 0, 0, 0);
        acc_a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc_a[j], 0, 0, 0);
        acc_g[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gl, bh, acc_g[j], 0, 0, 0);
      }
    }
    // the next stage into the other buffer (last read before the previous
    // barrier), then the loads of the stage after it
    if (st + 1 < nst) {
      if (vec) {
        PROJ_STAGE_W(0, cur ^ 1);
        PROJ_STAGE_W(1, cur ^ 1);
        PROJ_STAGE_W(2, cur ^ 1);
        PROJ_STAGE_W(3, cur ^ 1);
        PROJ_STAGE_S(cur ^ 1);
        if (st + 2 < nst) {
          const int h2 = (st + 2) * kPK;
          PROJ_FETCH_W(0, h2);
          PROJ_FETCH_W(1, h2);
          PROJ_FETCH_W(2, h2);
          PROJ_FETCH_W(3, h2);
          PROJ_FETCH_S(h2);
        }
      } else {
        stage_elements((st + 1) * kPK, cur ^ 1);
      }
    }
    __syncthreads();
  }
  // accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4,
  // column l % 32 of the 32 x 32 tile
  const size_t base = (size_t)b * H * L;
  if (vec) {
    // every residual and bias value first, then the outputs: the loads are in
    // flight together (out may alias x, so a load placed after a store would
    // wait for it; each element is still read and then written by one lane)
    const float* xr = x + base + (size_t)(c0 + cw + 4 * (lane >> 5)) * L + t0 + tw + (lane & 31);
    float* orow = out + base + (size_t)(c0 + cw + 4 * (lane >> 5)) * L + t0 + tw + (lane & 31);
    float xv[16][JT], ba[16], bg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dc = 8 * (r >> 2) + (r & 3);
      ba[r] = bias[c0 + cw + 4 * (lane >> 5) + dc];
      bg[r] = bias[H + c0 + cw + 4 * (lane >> 5) + dc];
#pragma unroll
      for (int j = 0; j < JT; ++j) xv[r][j] = xr[(size_t)dc * L + 32 * j];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dc = 8 * (r >> 2) + (r & 3);
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const float a = acc_a[j][r] + ba[r];
        const float g = acc_g[j][r] + bg[r];
        orow[(size_t)dc * L + 32 * j] = xv[r][j] + a * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = c0 + cw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (c >= H) continue;
      const float ba = bias[c], bg = bias[H + c];
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int t = t0 + tw + 32 * j + (lane & 31);
        if (t >= L) continue;
        const float a = acc_a[j][r] + ba;
        const float g = acc_g[j][r] + bg;
        const size_t o = base + (size_t)c * L + t;
        out[o] = x[o] + a * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      }
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
    constexpr int TN = 2 * kPN;
    const dim3 grid((p->L + TN - 1) / TN, p->H / 128, p->batch);
    glu_proj_kernel<128, TN><<<grid, 512, 0, st>>>(x, s, Wp, bias, out, p->H, p->L);
  } else {
    const dim3 grid((p->L + kPN - 1) / kPN, (p->H + 63) / 64, p->batch);
    glu_proj_kernel<64, kPN><<<grid, 256, 0, st>>>(x, s, Wp, bias, out, p->H, p->L);
  }
  return hipGetLastError();
}

hipError_t launch_layer_norm(const s4dplr_plan* p, const float* x, const float* gamma,
                             const float* beta, float* z, hipStream_t st) {
  const dim3 grid((p->L + 63) / 64, p->batch);
  auto run = [&](auto kernel) {
    kernel<<<grid, kLnThreads, 0, st>>>(x, gamma, beta, z, p->H, p->L, 1e-5f);
  };
  switch (p->H) {   // x held in registers between the two steps where H allows
    case 64: run(layer_norm_kernel<16>); break;
    case 128: run(layer_norm_kernel<32>); break;
    case 256: run(layer_norm_kernel<64>); break;
    case 512: run(layer_norm_kernel<128>); break;
    default: run(layer_norm_kernel<0>); break;
  }
  return hipGetLastError();
}

}  // namespace s4
