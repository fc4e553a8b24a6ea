// Device building blocks: complex arithmetic on float2, in-register DFTs of
// radix 2..16 with constant twiddles, and in-place Stockham FFT passes over
// LDS with each thread holding its points in registers between passes.
#pragma once

#include <hip/hip_runtime.h>

#include "fft_sched.h"

namespace s4 {

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(fmaf(a.x, b.x, a.y * b.y), fmaf(a.y, b.x, -a.x * b.y));
}
// Multiply by a stored forward twiddle w (forward) or by conj(w) (inverse).
template <bool INV>
__device__ __forceinline__ float2 cmulw(float2 a, float2 w) {
  if constexpr (INV) return cmulc(a, w);
  else return cmul(a, w);
}

// cos and sin of 2*pi*k/16, k = 0..7 (exact values of the 16th roots of unity).
__device__ constexpr float kCos16[8] = {1.0f, 0.923879532511286756f, 0.707106781186547524f,
                                        0.382683432365089772f, 0.0f, -0.382683432365089772f,
                                        -0.707106781186547524f, -0.923879532511286756f};
__device__ constexpr float kSin16[8] = {0.0f, 0.382683432365089772f, 0.707106781186547524f,
                                        0.923879532511286756f, 1.0f, 0.923879532511286756f,
                                        0.707106781186547524f, 0.382683432365089772f};

// x * exp(-+ 2 pi i IDX / 16), sign - for the forward transform.
template <int IDX, bool INV>
__device__ __forceinline__ float2 rot16(float2 x) {
  if constexpr (IDX == 0) {
    return x;
  } else if constexpr (IDX == 4) {
    if constexpr (INV) return make_float2(-x.y, x.x);
    else return make_float2(x.y, -x.x);
  } else {
    constexpr float c = kCos16[IDX], s = kSin16[IDX];
    if constexpr (INV) return make_float2(fmaf(x.x, c, -x.y * s), fmaf(x.y, c, x.x * s));
    else return make_float2(fmaf(x.x, c, x.y * s), fmaf(x.y, c, -x.x * s));
  }
}

template <int RL>
__host__ __device__ constexpr int bitrev(int s) {
  int r = 0;
  for (int b = 0; b < RL; ++b) r |= ((s >> b) & 1) << (RL - 1 - b);
  return r;
}

// One radix-2 decimation-in-frequency stage with span S on R points.
template <int R, int S, bool INV, int I = 0>
__device__ __forceinline__ void dif_stage_block(float2* v, int b) {
  if constexpr (I < S) {
    float2 a = v[b + I], c = v[b + I + S];
    v[b + I] = cadd(a, c);
    v[b + I + S] = rot16<I * (8 / S), INV>(csub(a, c));
    dif_stage_block<R, S, INV, I + 1>(v, b);
  }
}
template <int R, int S, bool INV>
__device__ __forceinline__ void dif_stage(float2* v) {
#pragma unroll
  for (int b = 0; b < R; b += 2 * S) dif_stage_block<R, S, INV>(v, b);
}
template <int R, int S, bool INV>
__device__ __forceinline__ void dif_all(float2* v) {
  if constexpr (S >= 1) {
    dif_stage<R, S, INV>(v);
    dif_all<R, S / 2, INV>(v);
  }
}
// In-register DFT of R = 2..16 points; output X[s] is left in v[bitrev(s)].
template <int R, bool INV>
__device__ __forceinline__ void dft_dif(float2* v) {
  static_assert(R >= 2 && R <= 16 && (R & (R - 1)) == 0, "radix");
  dif_all<R, R / 2, INV>(v);
}

// Stockham pass P of an in-place LDS transform of 2^LOG2N points.  `lt` is
// the thread's index within the transform (0 .. n/E-1); `on` = false lets a
// thread take part in the barriers without touching data.
template <int LOG2N, int P, bool INV>
struct FftPass {
  static __device__ __forceinline__ void run(float2* __restrict__ buf, int lt, bool on,
                                             const float2* __restrict__ tw) {
    constexpr int N = 1 << LOG2N;
    constexpr int E = 1 << fft_elems_log(LOG2N);
    constexpr int NT = N / E;
    constexpr int RL = fft_radix_log(LOG2N, P);
    constexpr int R = 1 << RL;
    constexpr int NB = E / R;
    constexpr int NSL = fft_ns_log(LOG2N, P);
    constexpr int NS = 1 << NSL;
    constexpr int STRIDE = N / R;
    constexpr int TWOFF = fft_tw_offset(LOG2N, P);
    float2 v[NB][R];
    if (on) {
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) v[q][r] = buf[lds_pad(lt + q * NT + r * STRIDE)];
    }
    __syncthreads();
    if (on) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int j = lt + q * NT;
        const int k = j & (NS - 1);
        if constexpr (NS > 1) {
          const float4* t4 = reinterpret_cast<const float4*>(tw + TWOFF + k * R);
#pragma unroll
          for (int r2 = 0; r2 < R / 2; ++r2) {
            const float4 w = t4[r2];
            if (r2 > 0) v[q][2 * r2] = cmulw<INV>(v[q][2 * r2], make_float2(w.x, w.y));
            v[q][2 * r2 + 1] = cmulw<INV>(v[q][2 * r2 + 1], make_float2(w.z, w.w));
          }
        }
        dft_dif<R, INV>(v[q]);
        const int base = ((j >> NSL) << (NSL + RL)) + k;
#pragma unroll
        for (int s = 0; s < R; ++s) buf[lds_pad(base + s * NS)] = v[q][bitrev<RL>(s)];
      }
    }
    __syncthreads();
    if constexpr (P + 1 < fft_num_passes(LOG2N)) FftPass<LOG2N, P + 1, INV>::run(buf, lt, on, tw);
  }
};

// In-place, unnormalized transform of 2^LOG2N points held in LDS (padded
// indexing).  Forward: sum_r x_r e^{-2 pi i r s / n}; inverse: e^{+...}.
// Ends with a barrier; all threads of the workgroup must call it.
template <int LOG2N, bool INV>
__device__ __forceinline__ void lds_fft(float2* __restrict__ buf, int lt, bool on,
                                        const float2* __restrict__ tw) {
  if constexpr (LOG2N > 0) FftPass<LOG2N, 0, INV>::run(buf, lt, on, tw);
}

// Blocks are placed on the 8 XCDs round-robin by block id.  Map block ids to
// logical tiles so that each XCD gets one contiguous range of tiles, which
// keeps the rows of one channel (sharing its spectrum) in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  constexpr int X = 8;
  const int q = nblk / X, r = nblk % X;
  const int x = bid % X, i = bid / X;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace s4
