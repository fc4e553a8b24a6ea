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
// The bin X_j of the 2M-point DFT of a real sequence x from the M-point DFT Z
// of its packing z_k = x_2k + i x_2k+1, given Z_j and Z_{M-j};
// csj = (cos, sin)(pi j / M).
__device__ __forceinline__ float2 rfft_x(float2 zj, float2 zmj, float2 csj) {
  const float2 p = make_float2(0.5f * (1.0f - csj.y), -0.5f * csj.x);
  const float2 q = make_float2(0.5f * (1.0f + csj.y), 0.5f * csj.x);
  return cadd(cmul(p, zj), cmul(q, cconj(zmj)));
}

// Multiply by a stored forward twiddle w (forward) or by conj(w) (inverse).
template <bool INV>
__device__ __forceinline__ float2 cmulw(float2 a, float2 w) {
  if constexpr (INV) return cmulc(a, w);
  else return cmul(a, w);
}

// cos and sin of 2*pi*k/16, k = 0..7 (exact values of the 16th roots of unity).
// (cos, sin)(pi s / 16), s < 16
__device__ constexpr float kCos32[16] = {1.000000000e+00f, 9.807852804e-01f, 9.238795325e-01f, 8.314696123e-01f, 7.071067812e-01f, 5.555702330e-01f, 3.826834324e-01f, 1.950903220e-01f, 0.0f, -1.950903220e-01f, -3.826834324e-01f, -5.555702330e-01f, -7.071067812e-01f, -8.314696123e-01f, -9.238795325e-01f, -9.807852804e-01f};
__device__ constexpr float kSin32[16] = {0.000000000e+00f, 1.950903220e-01f, 3.826834324e-01f, 5.555702330e-01f, 7.071067812e-01f, 8.314696123e-01f, 9.238795325e-01f, 9.807852804e-01f, 1.000000000e+00f, 9.807852804e-01f, 9.238795325e-01f, 8.314696123e-01f, 7.071067812e-01f, 5.555702330e-01f, 3.826834324e-01f, 1.950903220e-01f};

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

// ---------------------------------------------------------------------------
// Wave-resident transforms: a transform of M = 2^LOG2M points (32 <= M <=
// 1024) is held by T = M/16 lanes of one wavefront, 16 points per lane, and
// the passes exchange data through a wave-private LDS region, so only
// wave-level ordering is needed between passes (no workgroup barrier).
// ---------------------------------------------------------------------------

// pad(x + c) - pad(x) for a compile-time c: exactly c + c/16 when c is a
// multiple of 16; otherwise computed from x.
__device__ __forceinline__ int pad_shift(int x, int c) {
  if ((c & 15) == 0) return c + (c >> 4);
  return lds_pad(x + c) - lds_pad(x);
}

// Streaming accesses for data a launch touches once: the convolution's input
// u and output y.  The non-temporal hint keeps them from displacing what is
// reused from the caches (the spectral weights, shared by a channel's batch
// rows, and the four-step intermediate at L >= 32768).
typedef float f2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 load_stream(const float2* p) {
  const f2v v = __builtin_nontemporal_load(reinterpret_cast<const f2v*>(p));
  return make_float2(v.x, v.y);
}
__device__ __forceinline__ void store_stream(float2* p, float2 x) {
  f2v v;
  v.x = x.x;
  v.y = x.y;
  __builtin_nontemporal_store(v, reinterpret_cast<f2v*>(p));
}

// Orders this wave's LDS accesses before and after the call.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int LOG2M, int P>
struct WPass {
  static constexpr int M = 1 << LOG2M;
  static constexpr int T = M / 16;
  static constexpr int RL = fft_radix_log(LOG2M, P);
  static constexpr int R = 1 << RL;
  static constexpr int NB = 16 / R;
  static constexpr int NSL = fft_ns_log(LOG2M, P);
  static constexpr int NS = 1 << NSL;
  static constexpr int STRIDE = M / R;
  static constexpr int TWOFF = fft_tw_offset(LOG2M, P);

  // v[q*R + r] = x[j + r*STRIDE], j = lt + q*T
  static __device__ __forceinline__ void load(float2 (&v)[16], const float2* __restrict__ buf, int lt) {
    const float2* __restrict__ b0 = buf + lds_pad(lt);
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int r = 0; r < R; ++r) v[q * R + r] = b0[pad_shift(lt, q * T + r * STRIDE)];
  }
  // this pass's twiddles for the lane (entries r = 0 are 1 and unused)
  static __device__ __forceinline__ void load_tw(float2 (&w)[16], const float2* __restrict__ tw, int lt) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int k = (lt + q * T) & (NS - 1);
      const float4* t4 = reinterpret_cast<const float4*>(tw + TWOFF + k * R);
#pragma unroll
      for (int r2 = 0; r2 < R / 2; ++r2) {
        const float4 x = t4[r2];
        w[q * R + 2 * r2] = make_float2(x.x, x.y);
        w[q * R + 2 * r2 + 1] = make_float2(x.z, x.w);
      }
    }
  }
  template <bool INV>
  static __device__ __forceinline__ void compute(float2 (&v)[16], const float2 (&w)[16]) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      if constexpr (NS > 1) {
#pragma unroll
        for (int r = 1; r < R; ++r) v[q * R + r] = cmulw<INV>(v[q * R + r], w[q * R + r]);
      }
      dft_dif<R, INV>(&v[q * R]);
    }
  }
  // y[base(j) + s*NS] = X_s of butterfly j (X_s sits in v[q*R + bitrev(s)]).
  // base is a multiple of 16 when NS = 1 and s*NS is one when NS >= 16, so
  // pad(base + s*NS) = pad(base) + s*NS + (s*NS >> 4) in both cases.
  static __device__ __forceinline__ void store(const float2 (&v)[16], float2* __restrict__ buf, int lt) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int j = lt + q * T;
      const int k = j & (NS - 1);
      const int base = ((j >> NSL) << (NSL + RL)) + k;
      float2* __restrict__ b0 = buf + lds_pad(base);
#pragma unroll
      for (int s = 0; s < R; ++s) b0[s * NS + ((s * NS) >> 4)] = v[q * R + bitrev<RL>(s)];
    }
  }
};

// Twiddles of pass PASS for the butterflies of thread lt, rebuilt at each use
// from the table entries W^k (and W^{4k} for radix 16), W = W_{Ns R}: the
// other powers W^{rk} follow by at most three complex products, so only two
// (radix 16) or NB (shorter radix) values per pass stay in registers across
// the rows of a block instead of fifteen.
template <int LOG2M, int PASS>
struct PassTwiddles {
  using W = WPass<LOG2M, PASS>;
  static constexpr int NBASE = W::R == 16 ? 2 : W::NB;
  float2 b[NBASE];
  __device__ __forceinline__ void load(const float2* __restrict__ tw, int lt) {
    if constexpr (W::R == 16) {
      const int k = lt & (W::NS - 1);
      b[0] = tw[W::TWOFF + k * 16 + 1];
      b[1] = tw[W::TWOFF + k * 16 + 4];
    } else {
#pragma unroll
      for (int q = 0; q < W::NB; ++q) {
        const int k = (lt + q * W::T) & (W::NS - 1);
        b[q] = tw[W::TWOFF + k * W::R + 1];
      }
    }
  }
  // w[q R + r] = W^{r k_q}, r = 1 .. R-1
  __device__ __forceinline__ void expand(float2 (&w)[16]) const {
    float2 e[NBASE];
#pragma unroll
    for (int i = 0; i < NBASE; ++i) {
      e[i] = b[i];
      // an opaque copy: keeps the products inside the row loop rather than
      // hoisted out of it, where all of them would hold registers
      asm volatile("" : "+v"(e[i].x), "+v"(e[i].y));
    }
    if constexpr (W::R == 16) {
      const float2 w1 = e[0], w4 = e[1];
      const float2 w2 = cmul(w1, w1), w3 = cmul(w2, w1), w8 = cmul(w4, w4);
      const float2 w12 = cmul(w8, w4);
      w[1] = w1;
      w[2] = w2;
      w[3] = w3;
      w[4] = w4;
      w[5] = cmul(w4, w1);
      w[6] = cmul(w4, w2);
      w[7] = cmul(w4, w3);
      w[8] = w8;
      w[9] = cmul(w8, w1);
      w[10] = cmul(w8, w2);
      w[11] = cmul(w8, w3);
      w[12] = w12;
      w[13] = cmul(w12, w1);
      w[14] = cmul(w12, w2);
      w[15] = cmul(w12, w3);
    } else {
#pragma unroll
      for (int q = 0; q < W::NB; ++q) {
        const float2 w1 = e[q];
        w[q * W::R + 1] = w1;
        if constexpr (W::R >= 4) {
          const float2 w2 = cmul(w1, w1), w3 = cmul(w2, w1);
          w[q * W::R + 2] = w2;
          w[q * W::R + 3] = w3;
          if constexpr (W::R == 8) {
            const float2 w4 = cmul(w2, w2);
            w[q * W::R + 4] = w4;
            w[q * W::R + 5] = cmul(w4, w1);
            w[q * W::R + 6] = cmul(w4, w2);
            w[q * W::R + 7] = cmul(w4, w3);
          }
        }
      }
    }
  }
};

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
    // with 16 points per thread the twiddles come from two (radix 16) or NB
    // table entries fetched before the barrier, so their latency overlaps it
    constexpr bool BASES = E == 16 && NS > 1;
    PassTwiddles<(BASES ? LOG2N : 4), (BASES ? P : 1)> pt;
    if constexpr (BASES) {
      if (on) pt.load(tw, lt);
    }
    float2 v[NB][R];
    if (on) {
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) v[q][r] = buf[lds_pad(lt + q * NT + r * STRIDE)];
    }
    __syncthreads();
    if (on) {
      float2 wb[16];
      if constexpr (BASES) pt.expand(wb);
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int j = lt + q * NT;
        const int k = j & (NS - 1);
        if constexpr (BASES) {
#pragma unroll
          for (int r = 1; r < R; ++r) v[q][r] = cmulw<INV>(v[q][r], wb[q * R + r]);
        } else if constexpr (NS > 1) {
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

// First forward pass (radix 16, span 1) when the upper half of the input is
// zero: the first DIF stage reduces to v[i+8] = v[i] W_16^i.
__device__ __forceinline__ void dft16_fwd_half_input(float2 (&v)[16]) {
  v[8] = v[0];
  v[9] = rot16<1, false>(v[1]);
  v[10] = rot16<2, false>(v[2]);
  v[11] = rot16<3, false>(v[3]);
  v[12] = rot16<4, false>(v[4]);
  v[13] = rot16<5, false>(v[5]);
  v[14] = rot16<6, false>(v[6]);
  v[15] = rot16<7, false>(v[7]);
  dif_all<16, 4, false>(v);   // the remaining stages over all 16 points
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
