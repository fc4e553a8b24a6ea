// HIP kernels (gfx950) of the S4 DPLR convolution-mode forward pass.
//
// Pages cited: "The S4 kernel, from scratch" (sections 3-5), "S4" wiki
// ("Structured Transition Matrix", "S4D").
//
// Stage 1 (kernel generation):
//   pack    -- per (channel, pole): weights C B, C P, conj(Q) B, conj(Q) P and
//              the pole's Re^2, Im; per channel 2/dt and the z = -1 limit.
//   cauchy  -- per (channel, frequency): the four Cauchy sums over the poles,
//              the rank-1 Woodbury correction and the 2/(1+z) factor.
//   kspec   -- per channel: inverse FFT of length L, real part -> K; then the
//              spectrum of (K + D delta) zero-padded to 2L, stored as the two
//              complex weights per bin that the convolution applies.
// Stage 2 (convolution):
//   conv    -- per (batch, channel) row: real FFT of length 2L of the
//              zero-padded input, spectral product, inverse, first L outputs.
//
// Frequency-node algebra (exact rewrites of section 4's formulas): with
// theta = 2 pi l / L and z = e^{-i theta},
//   g(z) = (2/dt) (1-z)/(1+z) = i (2/dt) tan(theta/2),
//   2/(1+z) = 1 + i tan(theta/2),
// so every Cauchy term is 1/(i G - Lambda_n) with a real G per frequency.
//
// Real FFT of length 2L in halves: the zero-padded input x (2L reals) is
// packed as z_k = x_2k + i x_2k+1 (M = L complex points, the upper half zero).
// The even bins of its M-point DFT are the (M/2)-point DFT of a_k = z_k, the
// odd bins that of b_k = z_k W_M^k.  The real-FFT pairing of bins j and M-j
// never mixes the two halves, and the inverse of the spectral product is
// z'_k = IDFT(a')_k + W_M^-k IDFT(b')_k for the first M/2 points, which are
// exactly the L outputs kept.  So each row is two independent transforms of
// L/2 points forward and two back, joined only at the ends.
#include <hip/hip_runtime.h>

#include "cauchy.h"
#include "device_fft.h"
#include "internal.h"

namespace s4 {

// Convolution weights of bin j of the padded spectrum from S_j, its partner
// S_{L-j} and (c, s) = (cos, sin)(pi j / L), with sc = 1 / (2L):
//   alpha_j = sc ((1 - s) S_j + (1 + s) conj(S_{L-j})),
//   beta_j  = sc i c (S_j - conj(S_{L-j})),
// returned as (alpha, beta).  The convolution's spectral step is then
// Z'_j = alpha_j Z_j + beta_j conj(Z_{L-j}) on the packed row's transform.
__device__ __forceinline__ float4 bin_weights(float2 sj, float2 sm, float2 csj, float sc) {
  const float a = sc * (1.0f - csj.y), b = sc * (1.0f + csj.y), c = sc * csj.x;
  const float2 al = make_float2(fmaf(a, sj.x, b * sm.x), fmaf(a, sj.y, -b * sm.y));
  const float2 df = make_float2(sj.x - sm.x, sj.y + sm.y);   // S_j - conj(S_{L-j})
  return make_float4(al.x, al.y, -c * df.y, c * df.x);
}

// General kernel generation step: the generating function at the L roots of
// unity in natural order, F frequencies per thread, 256 threads, one channel
// per blockIdx.y.

template <int F, bool DIAG, bool TIED>
__global__ __launch_bounds__(kCauchyThreads) void cauchy_kernel(
    ParamPtrs pp, const float* __restrict__ tanT, float2* __restrict__ khat, int N, int NP,
    int L) {
  __shared__ float4 rec[kRec * kMaxPoles];
  __shared__ float2 red[kCauchyThreads / 64];
  const int h = blockIdx.y, tid = threadIdx.x;
  const float2 part = build_pole_records(pp, h, N, NP, DIAG, rec, tid, kCauchyThreads);
  const float2 sum = block_sum2<kCauchyThreads>(part, red, tid);
  const float dt = pp.dt[h];
  const float2 nyq = make_float2(0.5f * dt * sum.x, 0.5f * dt * sum.y);
  const float two_dt = 2.0f / dt;
  int l[F];
  float T[F], G[F];
  float acc[F][8];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    l[f] = (blockIdx.x * F + f) * kCauchyThreads + tid;
    T[f] = l[f] < L ? tanT[l[f]] : 0.f;
    G[f] = two_dt * T[f];
#pragma unroll
    for (int a = 0; a < 8; ++a) acc[f][a] = 0.f;
  }
  cauchy_sums<F, DIAG, TIED>(rec, NP, G, acc);
#pragma unroll
  for (int f = 0; f < F; ++f)
    if (l[f] < L) khat[(size_t)h * L + l[f]] = cauchy_epilogue<DIAG>(acc[f], T[f], 2 * l[f] == L, nyq);
}

// The generating function reduced to what the time-domain kernel needs, for
// the four-step path.  K = Re IDFT_L(K-hat) / L depends on K-hat only through
// its Hermitian part Xh_m = (X_m + conj(X_{L-m})) / 2, and the packed kernel
// z_n = K_2n + i K_2n+1 (n < L/2) is IDFT_{L/2}(Y) / L with
//   Y_m = (Xh_m + Xh_{m+L/2}) + i e^{2 pi i m / L} (Xh_m - Xh_{m+L/2}),
// an L/2-point transform instead of an L-point one.  Y_l and Y_{L/2-l}
// (0 < l < L/4) both depend on X at l, L - l, L/2 + l and L/2 - l: a lane pair
// takes them, the even lane l and L - l, the odd lane L/2 - l and L/2 + l,
// swaps its two values with its partner and stores Y_l (even) or Y_{L/2-l}
// (odd).  The pair with l = 0 needs no swap: the even lane takes 0 and L/2
// for Y_0, the odd lane L/4 and 3L/4 for Y_{L/4}.
// Y is stored in the four-step order of an L/2-point transform: Y_m at
// (m mod M1) 256 + m / M1, M1 = L / 512.  Pair q = 128 a + b (a < M1,
// b < 128) takes l = a + M1 b, so Y_l goes to 256 a + b and Y_{L/2-l} to
// 256 (M1 - a) + 255 - b (256 - b for a = 0): each half of a wave stores
// one contiguous run.
// The lane also writes the even bin of the padded spectrum that its Hermitian
// part gives, S_2m = Xh_m + D, into `spec` (bin k at (k mod L/256) 256 +
// k div (L/256); bin 0's slot holds the real pair (S_0, S_L)).
// (Seven waves per SIMD, what the pole records' LDS allows: without the
// bound the scheduler issues all four poles' record reads ahead, 107 VGPRs.)
template <bool DIAG, bool TIED>
__global__ __launch_bounds__(kCauchyThreads) __attribute__((amdgpu_waves_per_eu(7)))
void cauchy_half_kernel(
    ParamPtrs pp, const float* __restrict__ tanT, const float2* __restrict__ cs,
    float2* __restrict__ yhat, float2* __restrict__ spec, const float* __restrict__ D, int N,
    int NP, int L) {
  __shared__ float4 rec[kRec * kMaxPoles];
  __shared__ float2 red[kCauchyThreads / 64];
  const int h = blockIdx.y, tid = threadIdx.x;
  const float2 part = build_pole_records(pp, h, N, NP, DIAG, rec, tid, kCauchyThreads);
  const float2 sum = block_sum2<kCauchyThreads>(part, red, tid);
  const float dt = pp.dt[h];
  const float2 nyq = make_float2(0.5f * dt * sum.x, 0.5f * dt * sum.y);
  const float two_dt = 2.0f / dt;
  const int M1 = L / 512, H2 = L / 2, Q = L / 4;
  const int g = blockIdx.x * kCauchyThreads + tid;          // < L/2 (the grid is exact)
  const bool odd = g & 1;
  const int q = g >> 1;
  const int l = (q >> 7) + M1 * (q & 127);
  int f[2];
  if (l == 0) {
    f[0] = odd ? Q : 0;
    f[1] = odd ? H2 + Q : H2;
  } else {
    f[0] = odd ? H2 - l : l;
    f[1] = odd ? H2 + l : L - l;
  }
  float T[2], G[2], acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    T[i] = tanT[f[i]];
    G[i] = two_dt * T[i];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[i][k] = 0.f;
  }
  cauchy_sums<2, DIAG, TIED>(rec, NP, G, acc);
  const float2 A = cauchy_epilogue<DIAG>(acc[0], T[0], 2 * f[0] == L, nyq);
  const float2 B = cauchy_epilogue<DIAG>(acc[1], T[1], 2 * f[1] == L, nyq);
  const float2 pA = make_float2(__shfl_xor(A.x, 1), __shfl_xor(A.y, 1));
  const float2 pB = make_float2(__shfl_xor(B.x, 1), __shfl_xor(B.y, 1));
  // Y_m from X at m, L - m, m + L/2 and L/2 - m
  float2 xm = A, xlm = B, xmh = pB, xlmh = pA;
  if (l == 0) {
    if (odd) {
      xmh = B;
      xlmh = A;
    } else {
      xlm = A;
      xmh = B;
      xlmh = B;
    }
  }
  const int m = odd ? (l == 0 ? Q : H2 - l) : l;
  const float2 h1 = make_float2(0.5f * (xm.x + xlm.x), 0.5f * (xm.y - xlm.y));
  const float2 h2 = make_float2(0.5f * (xmh.x + xlmh.x), 0.5f * (xmh.y - xlmh.y));
  const float2 t = cmul(cs[2 * m], csub(h1, h2));           // e^{2 pi i m / L} (Xh_m - Xh_{m+L/2})
  yhat[(size_t)h * H2 + (m % M1) * 256 + m / M1] =
      make_float2(h1.x + h2.x - t.y, h1.y + h2.y + t.x);
  const float Dh = D ? D[h] : 0.f;
  const int M1L = 2 * M1, k = 2 * m;
  spec[(size_t)h * L + (k % M1L) * 256 + k / M1L] =
      (l == 0 && !odd) ? make_float2(h1.x + Dh, h2.x + Dh) : make_float2(h1.x + Dh, h1.y);
}

// ---------------------------------------------------------------------------
// Stage 1 fused for 32 <= L <= 1024: one block per channel.  All threads form
// the generating function (one frequency each) in LDS; one wave takes the
// inverse transform to K and the transform of the zero-padded K; all threads
// then form the convolution weights.  Also the kernel-spectrum step alone
// (FROM_TIME: K given).
// ---------------------------------------------------------------------------
template <int LOG2L>
struct KgenShape {
  static constexpr int L = 1 << LOG2L;
  static constexpr int F = L >= 512 ? 2 : 1;               // frequencies per thread
  static constexpr int NF = L / F < 256 ? 256 : L / F;     // threads over the frequencies
  // L >= 512: the poles are split in two halves over two sets of NF threads
  // (four waves per SIMD for the Cauchy sums, each wave reading half the
  // pole records), the halves' sums meeting in LDS
  static constexpr int PS = LOG2L >= 9 ? 2 : 1;
  static constexpr int NTHR = NF * PS;
  static constexpr int T = L / 16;
  static constexpr int P = fft_num_passes(LOG2L);
  static constexpr int MP = lds_padded_size(L);
  static_assert(LOG2L >= 5 && LOG2L <= 10, "fused range");
};


// Convolution weights of the bin pair (j, L-j), j in [0, L/2], from the
// spectrum Z (natural order, padded, in LDS) of the packed zero-padded kernel:
//   S_j = X_j + D,  alpha_j = ((1 - s_j) S_j + (1 + s_j) conj(S_{L-j})) / (2L),
//   beta_j = i c_j (S_j - conj(S_{L-j})) / (2L),   (c_j, s_j) = (cos, sin)(pi j / L).
// With conj set, S_j is replaced by conj(S_j): the weights of the correlation
// with (K + D delta), sum_j K_j x_{t+j} + D x_t, instead of the convolution.
__device__ __forceinline__ void weights_pair(const float2* __restrict__ Zb, float4* __restrict__ cf,
                                             float2 csj, float2 csm, int L, int j, float Dh,
                                             int conj) {
  const float sc = 0.5f / (float)L;
  const int jm = L - j;
  const float2 zj = Zb[lds_pad(j)], zm = Zb[lds_pad(jm & (L - 1))];
  float2 sj = rfft_x(zj, zm, csj), sm = rfft_x(zm, zj, csm);
  sj.x += Dh;
  sm.x += Dh;
  if (conj) {
    sj.y = -sj.y;
    sm.y = -sm.y;
  }
  cf[j] = bin_weights(sj, sm, csj, sc);
  if (j != 0 && jm != j) cf[jm] = bin_weights(sm, sj, csm, sc);
}

// exp(-i pi idx / L) from the (cos, sin)(pi j / L) table, 0 <= idx < 2L
__device__ __forceinline__ float2 wneg(const float2* __restrict__ cs, int L, int idx) {
  if (idx <= L) {
    const float2 c = cs[idx];
    return make_float2(c.x, -c.y);
  }
  return cs[2 * L - idx];
}

// x * i^n (n taken mod 4; n uniform over the wave)
__device__ __forceinline__ float2 mul_ipow(float2 x, int n) {
  switch (n & 3) {
    case 1: return make_float2(-x.y, x.x);
    case 2: return make_float2(-x.x, -x.y);
    case 3: return make_float2(x.y, -x.x);
    default: return x;
  }
}

// Pass P of a 256-point Stockham transform held by the 64 lanes of one wave,
// four points per lane: on entry a[r] = x[lane + 64 r]; the twiddles of pass
// P >= 1 are tw[r - 1] = W_{4 NS}^{k r}, NS = 4^P, k = lane mod NS (conjugated
// for the inverse); xb is the wave's own LDS buffer.  After pass 3 the lane
// holds X[lane + 64 s] in a[bitrev(s)] (no store).
template <int P, bool INV>
__device__ __forceinline__ void r4_pass(float2 (&a)[4], float2* __restrict__ xb, int lane,
                                        const float2 (&tw)[3]) {
  constexpr int NS = 1 << (2 * P);
  if constexpr (P > 0) {
#pragma unroll
    for (int r = 1; r < 4; ++r) a[r] = INV ? cmulc(a[r], tw[r - 1]) : cmul(a[r], tw[r - 1]);
  }
  dft_dif<4, INV>(a);
  if constexpr (P < 3) {
    const int k = lane & (NS - 1);
    const int base = (lane / NS) * 4 * NS + k;
#pragma unroll
    for (int t = 0; t < 4; ++t) xb[lds_pad(base + NS * t)] = a[bitrev<2>(t)];
    wave_sync();
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = xb[lds_pad(lane + 64 * r)];
    wave_sync();
  }
}

template <int LOG2L, bool DIAG, bool FROM_TIME, bool TIED = false>
__global__ __launch_bounds__(KgenShape<LOG2L>::NTHR) void kgen_wave_kernel(
    ParamPtrs pp, const float* __restrict__ D, const float* __restrict__ Kin,
    float* __restrict__ Kout, float4* __restrict__ coef, const float* __restrict__ tanT,
    const float2* __restrict__ tw, const float2* __restrict__ cs, int N, int NP, int conj) {
  using S = KgenShape<LOG2L>;
  constexpr int L = S::L, T = S::T, NTHR = S::NTHR, P = S::P;
  __shared__ float4 rec[FROM_TIME ? 1 : kRec * kMaxPoles];
  __shared__ float2 red[NTHR / 64];
  __shared__ float2 buf[S::MP];
  __shared__ float xs[(FROM_TIME || S::PS == 1) ? 1 : S::NF * S::F * 8];
  // L = 1024: the tail runs on four waves, each a quarter of each transform
  // (a radix-4 step over the whole transform, then a 256-point transform per
  // wave), with K in kb and each wave's exchanges in its own slice of xb
  constexpr bool PAR = LOG2L == 10 && !FROM_TIME;
  __shared__ float kb[PAR ? L : 1];
  __shared__ float2 xb[PAR ? 4 * lds_padded_size(256) : 1];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63;
  const bool fft_lane = tid < T;          // lanes of wave 0 that hold the transform
  float2 v[16], wA[16], wB[16];
  // the serial tail's twiddles: fetched up front when the Cauchy sums do not
  // need the registers (one set of poles per thread), else after the sums
  auto load_tail_tw = [&]() {
    if (fft_lane) {
      if constexpr (P > 2) WPass<LOG2L, 1>::load_tw(wA, tw, lane);
      WPass<LOG2L, P - 1>::load_tw(wB, tw, lane);
    }
  };
  // parallel tail (waves 0..3): pre[i] = W_L^{k q} for k = lane + 64 i, the
  // wave's quarter q; t1..t3 the 256-point passes' W_{4 NS}^{k r}
  const int tq = tid >> 6;
  float2 pre[4], t1[3], t2[3], t3[3];
  auto load_par_tw = [&]() {
    if (tid < 256) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pre[i] = wneg(cs, L, (2 * (lane + 64 * i) * tq) % (2 * L));
#pragma unroll
      for (int r = 1; r < 4; ++r) {
        t1[r - 1] = wneg(cs, L, (lane & 3) * r * (2 * L / 16));
        t2[r - 1] = wneg(cs, L, (lane & 15) * r * (2 * L / 64));
        t3[r - 1] = wneg(cs, L, (lane & 63) * r * (2 * L / 256));
      }
    }
  };
  if constexpr (!PAR && (S::PS == 1 || FROM_TIME)) load_tail_tw();
  constexpr int NW = (L / 2 + NTHR) / NTHR;     // bin pairs per thread in the weight step
  float2 csj[NW], csm[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int j = tid + i * NTHR;
    if (j <= L / 2) {
      csj[i] = cs[j];
      csm[i] = cs[L - j];
    }
  }
  const float Dh = D ? D[h] : 0.f;
  if constexpr (!FROM_TIME) {
    const float2 part = build_pole_records(pp, h, N, NP, DIAG, rec, tid, NTHR);
    const float2 sum = block_sum2<NTHR>(part, red, tid);
    const float dt = pp.dt[h];
    const float2 nyq = make_float2(0.5f * dt * sum.x, 0.5f * dt * sum.y);
    {
      constexpr int F = S::F, NF = S::NF;
      const int ft = tid % NF, ph = tid / NF;     // frequency thread, pole half
      float T0[F], G[F], acc[F][8];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int l = ft + f * NF;
        T0[f] = l < L ? tanT[l] : 0.f;
        G[f] = (2.0f / dt) * T0[f];
#pragma unroll
        for (int a = 0; a < 8; ++a) acc[f][a] = 0.f;
      }
      if constexpr (S::PS == 2) {
        const int nmid = (NP / 2) / kPoleUnroll * kPoleUnroll;
        if (ph == 0) cauchy_sums<F, DIAG, TIED>(rec, nmid, G, acc);
        else cauchy_sums<F, DIAG, TIED>(rec + kRec * nmid, NP - nmid, G, acc);
        if constexpr (PAR) load_par_tw();
        else load_tail_tw();
        if (ph == 1) {
#pragma unroll
          for (int f = 0; f < F; ++f)
#pragma unroll
            for (int a = 0; a < 8; ++a) xs[(f * 8 + a) * NF + ft] = acc[f][a];
        }
        __syncthreads();
        if (ph == 0) {
#pragma unroll
          for (int f = 0; f < F; ++f)
#pragma unroll
            for (int a = 0; a < 8; ++a) acc[f][a] += xs[(f * 8 + a) * NF + ft];
        }
      } else {
        cauchy_sums<F, DIAG, TIED>(rec, NP, G, acc);
      }
      if (ph == 0) {
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const int l = ft + f * NF;
          if (l < L) buf[lds_pad(l)] = cauchy_epilogue<DIAG>(acc[f], T0[f], 2 * l == L, nyq);
        }
      }
    }
    __syncthreads();
    if constexpr (PAR) {
      // inverse, decimated in frequency by 4: for the wave's quarter q,
      // y_q[k] = W_L^{-k q} sum_p X[k + 256 p] i^{p q} (k < 256), and
      // K[4 m + q] = Re IDFT_256(y_q)[m] / L
      if (tid < 256) {
        float2* __restrict__ xw = xb + tq * lds_padded_size(256);
        float2 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = lane + 64 * i;
          float2 y = buf[lds_pad(k)];
#pragma unroll
          for (int p = 1; p < 4; ++p) y = cadd(y, mul_ipow(buf[lds_pad(k + 256 * p)], p * tq));
          a[i] = cmulc(y, pre[i]);
        }
        r4_pass<0, true>(a, xw, lane, t1);
        r4_pass<1, true>(a, xw, lane, t1);
        r4_pass<2, true>(a, xw, lane, t2);
        r4_pass<3, true>(a, xw, lane, t3);
        const float invL = 1.0f / (float)L;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int n = 4 * (lane + 64 * t) + tq;
          const float kv = a[bitrev<2>(t)].x * invL;
          kb[n] = kv;
          if (Kout) Kout[(size_t)h * L + n] = kv;
        }
      }
      __syncthreads();
      // forward transform of the packed zero-padded K (z_k = K_2k + i K_2k+1,
      // k < L/2), decimated by 4: y_q[j] = W_L^{j q} (z_j + (-i)^q z_{j+256}),
      // Z[4 k + q] = DFT_256(y_q)[k]
      if (tid < 256) {
        float2* __restrict__ xw = xb + tq * lds_padded_size(256);
        float2 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = lane + 64 * i;
          const float2 z0 = make_float2(kb[2 * j], kb[2 * j + 1]);
          const float2 z1 = make_float2(kb[2 * j + 512], kb[2 * j + 513]);
          a[i] = cmul(cadd(z0, mul_ipow(z1, -tq)), pre[i]);
        }
        r4_pass<0, false>(a, xw, lane, t1);
        r4_pass<1, false>(a, xw, lane, t1);
        r4_pass<2, false>(a, xw, lane, t2);
        r4_pass<3, false>(a, xw, lane, t3);
#pragma unroll
        for (int t = 0; t < 4; ++t) buf[lds_pad(4 * (lane + 64 * t) + tq)] = a[bitrev<2>(t)];
      }
    } else if (fft_lane) {
    // inverse transform of length L; K_k = Re / L
      WPass<LOG2L, 0>::load(v, buf, lane);
      WPass<LOG2L, 0>::template compute<true>(v, wA);
      WPass<LOG2L, 0>::store(v, buf, lane);
      wave_sync();
      if constexpr (P > 2) {
        WPass<LOG2L, 1>::load(v, buf, lane);
        WPass<LOG2L, 1>::template compute<true>(v, wA);
        WPass<LOG2L, 1>::store(v, buf, lane);
        wave_sync();
      }
      using LP = WPass<LOG2L, P - 1>;
      LP::load(v, buf, lane);
      LP::template compute<true>(v, wB);
      const float invL = 1.0f / (float)L;
      wave_sync();
#pragma unroll
      for (int q = 0; q < LP::NB; ++q) {
        const int j = lane + q * T;               // j < NS in the last pass
#pragma unroll
        for (int s = 0; s < LP::R; ++s) {
          const int k = j + s * LP::NS;
          const float kv = v[q * LP::R + bitrev<LP::RL>(s)].x * invL;
          if (Kout) Kout[(size_t)h * L + k] = kv;
          buf[lds_pad(k)] = make_float2(kv, 0.f);
        }
      }
      wave_sync();
    }
  } else {
    for (int k = tid; k < L; k += NTHR) buf[lds_pad(k)] = make_float2(Kin[(size_t)h * L + k], 0.f);
    __syncthreads();
  }
  // transform of the packed zero-padded kernel z_k = K_2k + i K_2k+1 (k < L/2)
  if (!PAR && fft_lane) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int k = lane + T * r;
      v[r] = make_float2(buf[lds_pad(2 * k)].x, buf[lds_pad(2 * k + 1)].x);
    }
    wave_sync();
    dft16_fwd_half_input(v);
    WPass<LOG2L, 0>::store(v, buf, lane);
    wave_sync();
    if constexpr (P > 2) {
      WPass<LOG2L, 1>::load(v, buf, lane);
      WPass<LOG2L, 1>::template compute<false>(v, wA);
      WPass<LOG2L, 1>::store(v, buf, lane);
      wave_sync();
    }
    using LP = WPass<LOG2L, P - 1>;
    LP::load(v, buf, lane);
    LP::template compute<false>(v, wB);
    LP::store(v, buf, lane);
    wave_sync();
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int j = tid + i * NTHR;
    if (j <= L / 2) weights_pair(buf, coef + (size_t)h * L, csj[i], csm[i], L, j, Dh, conj);
  }
}

// ---------------------------------------------------------------------------
// Stage 1c: time-domain kernel and its zero-padded spectrum (LDS-resident)
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int LOG2L>
struct KspecShape {
  static constexpr int L = 1 << LOG2L, H2 = L / 2, LOG2H2 = LOG2L - 1;
  static constexpr int EL = 1 << fft_elems_log(LOG2L);
  static constexpr int EH = 1 << fft_elems_log(LOG2H2);
  static constexpr int NTL = L / EL;       // threads of the length-L transform
  static constexpr int TPH = H2 / EH;      // threads per half transform
  static constexpr int NT = cmax(NTL, 2 * TPH);
  static constexpr int HP = lds_padded_size(H2);
  static constexpr int BUF = cmax(lds_padded_size(L), 2 * HP);
  static constexpr int ZPT = (H2 + NT - 1) / NT;
};

template <int LOG2L, bool FROM_TIME>
__global__ __launch_bounds__(KspecShape<LOG2L>::NT) void kspec_kernel(
    const float2* __restrict__ khat, const float* __restrict__ Kin, const float* __restrict__ D,
    float* __restrict__ Kout, float4* __restrict__ coef, const float2* __restrict__ twL,
    const float2* __restrict__ twH, const float2* __restrict__ cs, int conj) {
  using S = KspecShape<LOG2L>;
  constexpr int L = S::L, H2 = S::H2, NT = S::NT;
  __shared__ float2 buf[S::BUF];
  const int h = blockIdx.x, tid = threadIdx.x;
  float2 z[S::ZPT];
  if constexpr (!FROM_TIME) {
    for (int k = tid; k < L; k += NT) buf[lds_pad(k)] = khat[(size_t)h * L + k];
    __syncthreads();
    lds_fft<LOG2L, true>(buf, tid, tid < S::NTL, twL);
    const float invL = 1.0f / (float)L;
#pragma unroll
    for (int i = 0; i < S::ZPT; ++i) {
      const int k = tid + i * NT;
      if (k < H2) {
        z[i] = make_float2(buf[lds_pad(2 * k)].x * invL, buf[lds_pad(2 * k + 1)].x * invL);
        if (Kout) reinterpret_cast<float2*>(Kout + (size_t)h * L)[k] = z[i];
      }
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < S::ZPT; ++i) {
      const int k = tid + i * NT;
      if (k < H2) z[i] = reinterpret_cast<const float2*>(Kin + (size_t)h * L)[k];
    }
  }
  float2* A = buf;
  float2* Bq = buf + S::HP;
#pragma unroll
  for (int i = 0; i < S::ZPT; ++i) {
    const int k = tid + i * NT;
    if (k < H2) {
      const float2 c = cs[2 * k];                        // W_L^k = cos - i sin of 2 pi k / L
      A[lds_pad(k)] = z[i];
      Bq[lds_pad(k)] = cmul(z[i], make_float2(c.x, -c.y));
    }
  }
  __syncthreads();
  {
    const int half = tid / S::TPH, lt = tid % S::TPH;
    lds_fft<S::LOG2H2, false>(half ? Bq : A, lt, tid < 2 * S::TPH, twH);
  }
  // Spectrum S_j = X_j + D of (K + D delta) padded to 2L, for bins j in
  // [0, L]; weights for the convolution's pairing step (scaled by 1/(2L)):
  //   alpha_j = ((1 - s_j) S_j + (1 + s_j) conj(S_{L-j})) / (2L)
  //   beta_j  = i c_j (S_j - conj(S_{L-j})) / (2L)
  const float Dh = D ? D[h] : 0.f;
  const float sc = 0.5f / (float)L;
  float4* cf = coef + (size_t)h * L;
  auto zget = [&](int j) -> float2 { return (j & 1) ? Bq[lds_pad(j >> 1)] : A[lds_pad(j >> 1)]; };
  for (int j = tid; j <= L / 2; j += NT) {
    const int jm = L - j;
    const float2 zj = zget(j), zm = zget(jm & (L - 1));
    const float2 csj = cs[j], csm = cs[jm];
    float2 sj = rfft_x(zj, zm, csj), sm = rfft_x(zm, zj, csm);
    sj.x += Dh;
    sm.x += Dh;
    if (conj) {   // correlation instead of convolution (see weights_pair)
      sj.y = -sj.y;
      sm.y = -sm.y;
    }
    cf[j] = bin_weights(sj, sm, csj, sc);
    if (j != 0 && jm != j) cf[jm] = bin_weights(sm, sj, csm, sc);
  }
}

// ---------------------------------------------------------------------------
// Stage 2: fused causal convolution, one row per thread group (LDS-resident)
// ---------------------------------------------------------------------------
template <int LOG2L>
struct ConvShape {
  static constexpr int L = 1 << LOG2L, H2 = L / 2, LOG2H2 = LOG2L - 1;
  static constexpr int E = 1 << fft_elems_log(LOG2H2);
  static constexpr int TPH = H2 / E;
  static constexpr int TPR = 2 * TPH;                      // threads per row
  static constexpr int NTHR = TPR > 64 ? TPR : 64;
  static constexpr int RPW = NTHR / TPR;                   // rows per workgroup
  static constexpr int HP = lds_padded_size(H2);
};

template <int LOG2L>
__global__ __launch_bounds__(ConvShape<LOG2L>::NTHR) void conv_kernel(
    const float* __restrict__ u, float* __restrict__ y, const float4* __restrict__ coef,
    const float2* __restrict__ twH, const float2* __restrict__ cs, int H, int batch) {
  using S = ConvShape<LOG2L>;
  constexpr int L = S::L, H2 = S::H2, TPR = S::TPR, TPH = S::TPH;
  __shared__ float2 lds[S::RPW * 2 * S::HP];
  const int tid = threadIdx.x;
  const int rloc = tid / TPR, t = tid % TPR;
  const int half = t / TPH, lt = t % TPH;
  const int lblk = xcd_remap(blockIdx.x, gridDim.x);
  const int lrow = lblk * S::RPW + rloc;          // logical row: channel-major
  const int rows = batch * H;
  const bool active = lrow < rows;
  const int h = active ? lrow / batch : 0;
  const int b = active ? lrow - h * batch : 0;
  const size_t roff = ((size_t)b * H + h) * L;
  float2* A = lds + rloc * 2 * S::HP;
  float2* Bq = A + S::HP;
  // 1. load the row as z_k = (u_2k, u_2k+1); a = z, b = z W_L^k
  for (int k = t; k < H2; k += TPR) {
    const float2 zk = active ? reinterpret_cast<const float2*>(u + roff)[k] : make_float2(0.f, 0.f);
    const float2 c = cs[2 * k];
    A[lds_pad(k)] = zk;
    Bq[lds_pad(k)] = cmul(zk, make_float2(c.x, -c.y));
  }
  __syncthreads();
  float2* mine = half ? Bq : A;
  // 2. forward transforms of L/2 points
  lds_fft<S::LOG2H2, false>(mine, lt, true, twH);
  // 3. spectral step on bin pairs (j, L-j): Z'_j = alpha_j Z_j + beta_j conj(Z_{L-j})
  // weights of bin j = 2m + half are at coef[h][j]
  const float4* __restrict__ cf = coef + (size_t)h * L + half;
  if (half == 0) {
    for (int m = lt; m <= H2 / 2; m += TPH) {
      const int mp = (H2 - m) & (H2 - 1);
      const float2 z1 = A[lds_pad(m)], z2 = A[lds_pad(mp)];
      const float4 c1 = cf[2 * m], c2 = cf[2 * mp];
      const float2 o1 = cadd(cmul(make_float2(c1.x, c1.y), z1), cmul(make_float2(c1.z, c1.w), cconj(z2)));
      const float2 o2 = cadd(cmul(make_float2(c2.x, c2.y), z2), cmul(make_float2(c2.z, c2.w), cconj(z1)));
      A[lds_pad(m)] = o1;
      if (mp != m) A[lds_pad(mp)] = o2;
    }
  } else {
    for (int m = lt; m < (H2 + 1) / 2; m += TPH) {
      const int mp = H2 - 1 - m;
      const float2 z1 = Bq[lds_pad(m)], z2 = Bq[lds_pad(mp)];
      const float4 c1 = cf[2 * m], c2 = cf[2 * mp];
      const float2 o1 = cadd(cmul(make_float2(c1.x, c1.y), z1), cmul(make_float2(c1.z, c1.w), cconj(z2)));
      const float2 o2 = cadd(cmul(make_float2(c2.x, c2.y), z2), cmul(make_float2(c2.z, c2.w), cconj(z1)));
      Bq[lds_pad(m)] = o1;
      if (mp != m) Bq[lds_pad(mp)] = o2;
    }
  }
  __syncthreads();
  // 4. inverse transforms
  lds_fft<S::LOG2H2, true>(mine, lt, true, twH);
  // 5. join the halves: z'_k = a'_k + W_L^-k b'_k -> (y_2k, y_2k+1)
  for (int k = t; k < H2; k += TPR) {
    const float2 c = cs[2 * k];
    const float2 zz = cadd(A[lds_pad(k)], cmul(Bq[lds_pad(k)], c));
    if (active) reinterpret_cast<float2*>(y + roff)[k] = zz;
  }
}

// ---------------------------------------------------------------------------
// Stage 2 for 32 <= L <= 1024: wave-resident rows
// ---------------------------------------------------------------------------
// The packed zero-padded row z (M = L complex points, upper half zero) is
// transformed with M/16 lanes of one wavefront; the spectrum Z becomes that of
// the output by Z'_j = alpha_j Z_j + beta_j conj(Z_{M-j}); the inverse
// transform's first M/2 points are the L outputs (y_2k, y_2k+1) = z'_k.
// Each wave loops over rows; the twiddles stay in registers across rows.
constexpr int kWaveConvThreads = 256;

template <int LOG2M>
struct WaveConvShape {
  static constexpr int M = 1 << LOG2M;
  static constexpr int T = M / 16;                 // lanes per row
  static constexpr int RPW = 64 / T;               // rows per wave
  static constexpr int P = fft_num_passes(LOG2M);
  static constexpr int MP = lds_padded_size(M);
  static_assert(LOG2M >= 5 && LOG2M <= 10, "wave-resident range");
};

template <int LOG2M>
__global__ __launch_bounds__(kWaveConvThreads) void conv_wave_kernel(
    const float* __restrict__ u, float* __restrict__ y, const float4* __restrict__ coef,
    const float2* __restrict__ tw, int H, int batch, int groups_per_wave) {
  using S = WaveConvShape<LOG2M>;
  constexpr int M = S::M, T = S::T, P = S::P;
  __shared__ float2 lds[(kWaveConvThreads / 64) * S::RPW * S::MP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rw = lane / T, lt = lane % T;
  float2* buf = lds + (wave * S::RPW + rw) * S::MP;
  float2 w1[16], w2[16];
  if constexpr (P > 1) WPass<LOG2M, 1>::load_tw(w1, tw, lt);
  if constexpr (P > 2) WPass<LOG2M, 2>::load_tw(w2, tw, lt);
  const int rows = H * batch;
  const int ngroups = (rows + S::RPW - 1) / S::RPW;
  const int gw = xcd_remap(blockIdx.x, gridDim.x) * (kWaveConvThreads / 64) + wave;
  // The next row's input and the current channel's weights are fetched ahead
  // of their use so that their memory latency overlaps the transforms.
  auto row_of = [&](int g, int& h, size_t& roff) -> bool {
    const int lrow = g * S::RPW + rw;            // logical row: channel-major
    const bool act = lrow < rows;
    h = act ? lrow / batch : 0;
    const int b = act ? lrow - h * batch : 0;
    roff = ((size_t)b * H + h) * M;
    return act;
  };
  float2 upre[8];
  {
    int h0;
    size_t r0;
    const bool a0 = row_of(gw * groups_per_wave, h0, r0);
    const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (a0 ? r0 : 0));
#pragma unroll
    for (int r = 0; r < 8; ++r) upre[r] = load_stream(&ur[lt + T * r]);
    if (!a0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) upre[r] = make_float2(0.f, 0.f);
    }
  }
  float4 cw[16];
  int hc = -1;
  for (int gi = 0; gi < groups_per_wave; ++gi) {
    const int g = gw * groups_per_wave + gi;
    if (g >= ngroups) break;
    int h;
    size_t roff;
    const bool active = row_of(g, h, roff);
    float2 v[16];
    // forward pass 0 straight from memory: z_{lt + T r}, r < 8; the rest is padding
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = upre[r];
    if (h != hc) {
      const float4* __restrict__ cf = coef + (size_t)h * M;
#pragma unroll
      for (int r = 0; r < 16; ++r) cw[r] = cf[lt + T * r];
      hc = h;
    }
    dft16_fwd_half_input(v);
    WPass<LOG2M, 0>::store(v, buf, lt);
    wave_sync();
    if constexpr (P > 2) {
      WPass<LOG2M, 1>::load(v, buf, lt);
      WPass<LOG2M, 1>::template compute<false>(v, w1);
      WPass<LOG2M, 1>::store(v, buf, lt);
      wave_sync();
    }
    // last forward pass; its outputs X_s of butterfly q are the bins
    // lt + T (q + s NB), which is exactly the inverse pass-0 input set of this
    // lane, so Z_j stays in registers and only Z_{M-j} comes from LDS
    using FL = WPass<LOG2M, P - 1>;
    FL::load(v, buf, lt);
    if constexpr (P == 2) FL::template compute<false>(v, w1);
    else FL::template compute<false>(v, w2);
    FL::store(v, buf, lt);
    float2 z[16];
#pragma unroll
    for (int q = 0; q < FL::NB; ++q)
#pragma unroll
      for (int s2 = 0; s2 < FL::R; ++s2) z[q + s2 * FL::NB] = v[q * FL::R + bitrev<FL::RL>(s2)];
    wave_sync();
    // spectral weights: Z'_j = alpha_j Z_j + beta_j conj(Z_{M-j}), j = lt + T r
    {
      // Z_{M-j} at pad(M - T r - lt) = (M - T r) + (M - T r)/16 + pad(-lt) for
      // M - T r a multiple of 16 (j = 0 maps to 0)
      const int nlt = -lt;
      const float2* __restrict__ bm = buf + (nlt + (nlt >> 4));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = lt + T * r;
        float2 zm;
        if (r == 0) zm = buf[lds_pad((M - lt) & (M - 1))];
        else if (((M - T * r) & 15) == 0) zm = bm[(M - T * r) + ((M - T * r) >> 4)];
        else zm = buf[lds_pad(M - j)];
        const float4 c = cw[r];
        v[r] = cadd(cmul(make_float2(c.x, c.y), z[r]), cmul(make_float2(c.z, c.w), cconj(zm)));
      }
    }
    // next row's input, in flight during the inverse transform
    if (gi + 1 < groups_per_wave && g + 1 < ngroups) {
      int hn;
      size_t rn;
      const bool an = row_of(g + 1, hn, rn);
      const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (an ? rn : 0));
#pragma unroll
      for (int r = 0; r < 8; ++r) upre[r] = load_stream(&ur[lt + T * r]);
      if (!an) {
#pragma unroll
        for (int r = 0; r < 8; ++r) upre[r] = make_float2(0.f, 0.f);
      }
    }
    wave_sync();
    WPass<LOG2M, 0>::template compute<true>(v, w1);
    WPass<LOG2M, 0>::store(v, buf, lt);
    wave_sync();
    if constexpr (P > 2) {
      WPass<LOG2M, 1>::load(v, buf, lt);
      WPass<LOG2M, 1>::template compute<true>(v, w1);
      WPass<LOG2M, 1>::store(v, buf, lt);
      wave_sync();
    }
    // last inverse pass: only the outputs k < M/2 are kept
    using LP = WPass<LOG2M, P - 1>;
    LP::load(v, buf, lt);
    if constexpr (P == 2) LP::template compute<true>(v, w1);
    else LP::template compute<true>(v, w2);
    float2* __restrict__ yr = reinterpret_cast<float2*>(y + roff);
#pragma unroll
    for (int q = 0; q < LP::NB; ++q) {
      const int j = lt + q * T;                   // j < NS in the last pass
#pragma unroll
      for (int s2 = 0; s2 < LP::R / 2; ++s2)
        if (active) store_stream(&yr[j + s2 * LP::NS], v[q * LP::R + bitrev<LP::RL>(s2)]);
    }
    wave_sync();
  }
}

// ---------------------------------------------------------------------------
// Stage 2 at L = 1024 (M = 1024): the wave-resident row with paired lanes
// ---------------------------------------------------------------------------
// As conv_wave_kernel, one wave per row and 16 points per lane, with two
// changes that remove one of the row's five LDS exchanges.  The last forward
// pass (radix 4, span 256) gives lane lt the butterflies a in
// {lt, 64 + lt, 192 - lt, 256 - lt} (lane 0: {0, 64, 192, 128}), so the bins
// a + 256 s and their real-FFT partners M - a - 256 s = (256 - a) + 256 (3 - s)
// sit in the same lane and the spectral weights are applied in registers.
// The inverse is then taken over that layout:
//   Y[a][n1] = W_M^{-n1 a} sum_s Z'[a + 256 s] W_4^{-n1 s}          (registers)
//   S[n1][a1][m] = W_256^{-m a1} sum_{a2} Y[a1 + 16 a2][n1] W_16^{-m a2}
//   x[n1 + 4 m + 64 m'] = sum_{a1} S[n1][a1][m] W_16^{-m' a1},  m' < 8,
// the last line giving exactly the kept outputs n < M/2 (y_2n, y_2n+1).
// The twiddles of the forward passes serve the inverse too (conjugated).
__device__ __forceinline__ int pair_butterfly(int lt, int q) {
  if (lt == 0) return q == 0 ? 0 : q == 1 ? 64 : q == 2 ? 192 : 128;
  return q == 0 ? lt : q == 1 ? 64 + lt : q == 2 ? 192 - lt : 256 - lt;
}

__global__ __launch_bounds__(kWaveConvThreads) void conv_pair1024_kernel(
    const float* __restrict__ u, float* __restrict__ y, const float4* __restrict__ coef,
    const float2* __restrict__ tw, int H, int batch, int groups_per_wave) {
  constexpr int LOG2M = 10, M = 1024, T = 64;
  using S = WaveConvShape<LOG2M>;
  using P1 = WPass<LOG2M, 1>;
  static_assert(S::RPW == 1 && S::P == 3, "one row per wave, passes 16 x 16 x 4");
  __shared__ float2 lds[(kWaveConvThreads / 64) * S::MP];
  const int wave = threadIdx.x >> 6, lt = threadIdx.x & 63;
  float2* buf = lds + wave * S::MP;
  // w1: pass-1 twiddles W_256^{k r}, k = lt & 15 (inverse pass 1: conj, index m)
  // w2: the last pass's W_M^{a r} for this lane's butterflies a (inverse step 1: conj)
  float2 w1[16], w2[16];
  P1::load_tw(w1, tw, lt);
  int bq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bq[q] = pair_butterfly(lt, q);
    const float4 t0 = reinterpret_cast<const float4*>(tw + WPass<LOG2M, 2>::TWOFF + bq[q] * 4)[0];
    const float4 t1 = reinterpret_cast<const float4*>(tw + WPass<LOG2M, 2>::TWOFF + bq[q] * 4)[1];
    w2[q * 4 + 1] = make_float2(t0.z, t0.w);
    w2[q * 4 + 2] = make_float2(t1.x, t1.y);
    w2[q * 4 + 3] = make_float2(t1.z, t1.w);
  }
  const int rows = H * batch;
  const int gw = xcd_remap(blockIdx.x, gridDim.x) * (kWaveConvThreads / 64) + wave;
  auto row_of = [&](int g, int& h, size_t& roff) -> bool {
    const bool act = g < rows;                   // logical row g: channel-major
    h = act ? g / batch : 0;
    const int b = act ? g - h * batch : 0;
    roff = ((size_t)b * H + h) * M;
    return act;
  };
  float2 upre[8];
  {
    int h0;
    size_t r0;
    const bool a0 = row_of(gw * groups_per_wave, h0, r0);
    const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (a0 ? r0 : 0));
#pragma unroll
    for (int r = 0; r < 8; ++r) upre[r] = a0 ? load_stream(&ur[lt + T * r]) : make_float2(0.f, 0.f);
  }
  float4 cw[16];
  int hc = -1;
  for (int gi = 0; gi < groups_per_wave; ++gi) {
    const int g = gw * groups_per_wave + gi;
    if (g >= rows) break;
    int h;
    size_t roff;
    const bool active = row_of(g, h, roff);
    float2 v[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = upre[r];
    if (h != hc) {
      // weights of the lane's bins a_q + 256 s, held across the channel's rows
      const float4* __restrict__ cf = coef + (size_t)h * M;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int s = 0; s < 4; ++s) cw[q * 4 + s] = cf[bq[q] + 256 * s];
      hc = h;
    }
    // forward passes 0 and 1 (Stockham, as the generic kernel)
    dft16_fwd_half_input(v);
    WPass<LOG2M, 0>::store(v, buf, lt);
    wave_sync();
    P1::load(v, buf, lt);
    P1::template compute<false>(v, w1);
    P1::store(v, buf, lt);
    wave_sync();
    // last forward pass on the paired butterflies: X[a + 256 s] -> v[q*4 + bitrev(s)]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // pad(a + 256 r) = pad(a) + 272 r
      const float2* __restrict__ bb = buf + lds_pad(bq[q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[q * 4 + r] = bb[272 * r];
#pragma unroll
      for (int r = 1; r < 4; ++r) v[q * 4 + r] = cmul(v[q * 4 + r], w2[q * 4 + r]);
      dft_dif<4, false>(&v[q * 4]);
    }
    // next row's input, in flight during the spectral step and the inverse
    if (gi + 1 < groups_per_wave && g + 1 < rows) {
      int hn;
      size_t rn;
      const bool an = row_of(g + 1, hn, rn);
      const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (an ? rn : 0));
#pragma unroll
      for (int r = 0; r < 8; ++r) upre[r] = an ? load_stream(&ur[lt + T * r]) : make_float2(0.f, 0.f);
    }
    // spectral weights in registers: Z'_j = alpha_j Z_j + beta_j conj(Z_{M-j})
    float2 zs[16];
    const bool l0 = lt == 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // partner slot: butterfly 256 - a, output 3 - s; lane 0's butterflies
        // 0 and 128 pair with themselves (outputs -s mod 4 and 3 - s)
        const float2 zp_gen = v[(3 - q) * 4 + bitrev<2>(3 - s)];
        float2 zp = zp_gen;
        if (q == 0) zp = l0 ? v[bitrev<2>((4 - s) & 3)] : zp_gen;
        if (q == 3) zp = l0 ? v[12 + bitrev<2>(3 - s)] : zp_gen;
        const float4 c = cw[q * 4 + s];
        zs[q * 4 + s] = cadd(cmul(make_float2(c.x, c.y), v[q * 4 + bitrev<2>(s)]),
                             cmul(make_float2(c.z, c.w), cconj(zp)));
      }
    // inverse step 1 (registers): Y[a][n1], stored at [n1][a]
    wave_sync();                                 // pass-2 reads of this row are done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dft_dif<4, true>(&zs[q * 4]);              // n1 at position bitrev(n1)
      float2* __restrict__ bb = buf + lds_pad(bq[q]);
#pragma unroll
      for (int n1 = 0; n1 < 4; ++n1) {
        float2 yv = zs[q * 4 + bitrev<2>(n1)];
        if (n1 > 0) yv = cmulc(yv, w2[q * 4 + n1]);
        bb[272 * n1] = yv;                       // [n1][a] at pad(256 n1 + a)
      }
    }
    wave_sync();
    // inverse pass 1: lane (n1, a1) = (lt >> 4, lt & 15), radix 16 over a2
    {
      const int n1 = lt >> 4, a1 = lt & 15;
      // pad(256 n1 + a1 + 16 c) = 272 n1 + a1 + 17 c for a1 < 16
      float2* __restrict__ bb = buf + 272 * n1 + a1;
#pragma unroll
      for (int a2 = 0; a2 < 16; ++a2) v[a2] = bb[17 * a2];
      dft_dif<16, true>(v);                      // m at position bitrev(m)
      wave_sync();
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        float2 sv = v[bitrev<4>(m)];
        if (m > 0) sv = cmulc(sv, w1[m]);
        bb[17 * m] = sv;                         // [n1][m][a1] at pad(256 n1 + 16 m + a1)
      }
    }
    wave_sync();
    // inverse pass 2: lane (n1, m) = (lt >> 4, lt & 15), radix 16 over a1,
    // outputs m' < 8 only: x[n1 + 4 m + 64 m']
    {
      const int n1 = lt >> 4, m = lt & 15;
      const float2* __restrict__ bb = buf + 272 * n1 + 17 * m;
#pragma unroll
      for (int a1 = 0; a1 < 16; ++a1) v[a1] = bb[a1];
      dft_dif<16, true>(v);
      float2* __restrict__ yr = reinterpret_cast<float2*>(y + roff);
#pragma unroll
      for (int mp = 0; mp < 8; ++mp)
        if (active) store_stream(&yr[n1 + 4 * m + 64 * mp], v[bitrev<4>(mp)]);
    }
    wave_sync();
  }
}

// ---------------------------------------------------------------------------
// Stage 2 for 2048 <= L <= 16384: block-resident rows
// ---------------------------------------------------------------------------
// The same transform layout as the wave-resident kernel (M/16 threads per
// row, 16 points each), with the row spread over several wavefronts, so the
// passes are separated by workgroup barriers.  The padded row occupies M*17/16
// complex of LDS (139 KB at L = 16384).
template <int LOG2M>
struct RowConvShape {
  static constexpr int M = 1 << LOG2M;
  static constexpr int T = M / 16;                 // threads per row
  static constexpr int NTHR = T < 256 ? 256 : T;
  static constexpr int RPB = NTHR / T;             // rows per block
  static constexpr int P = fft_num_passes(LOG2M);
  static constexpr int MP = lds_padded_size(M);
  static_assert(LOG2M >= 11 && LOG2M <= 14, "block-resident range");
};

template <int LOG2M, int PASS, bool INV>
__device__ __forceinline__ void row_pass(float2 (&v)[16], float2* __restrict__ buf, int lt,
                                         const PassTwiddles<LOG2M, PASS>& pt) {
  using W = WPass<LOG2M, PASS>;
  float2 w[16];
  pt.expand(w);
  W::load(v, buf, lt);
  __syncthreads();
  W::template compute<INV>(v, w);
  W::store(v, buf, lt);
  __syncthreads();
}

template <int LOG2M>
__global__ __launch_bounds__(RowConvShape<LOG2M>::NTHR) void conv_rows_kernel(
    const float* __restrict__ u, float* __restrict__ y, const float4* __restrict__ coef,
    const float2* __restrict__ tw, int H, int batch, int groups_per_block) {
  using S = RowConvShape<LOG2M>;
  constexpr int M = S::M, T = S::T, P = S::P;
  using FL = WPass<LOG2M, P - 1>;
  __shared__ float2 lds[S::RPB * S::MP];
  const int tid = threadIdx.x;
  const int rw = tid / T, lt = tid % T;
  float2* buf = lds + rw * S::MP;
  const int rows = H * batch;
  const int ngroups = (rows + S::RPB - 1) / S::RPB;
  const int gb = xcd_remap(blockIdx.x, gridDim.x);
  // the twiddle bases of every pass, fetched once for all rows of the block
  PassTwiddles<LOG2M, 1> pt1;
  PassTwiddles<LOG2M, (P > 3 ? 2 : 1)> pt2;
  PassTwiddles<LOG2M, P - 1> ptl;
  if constexpr (P > 2) pt1.load(tw, lt);
  if constexpr (P > 3) pt2.load(tw, lt);
  ptl.load(tw, lt);
  auto row_of = [&](int g, int& h, size_t& roff) -> bool {
    const int lrow = g * S::RPB + rw;            // logical row: channel-major
    const bool act = lrow < rows;
    h = act ? lrow / batch : 0;
    const int b = act ? lrow - h * batch : 0;
    roff = ((size_t)b * H + h) * M;
    return act;
  };
  // the next row's input in flight during the inverse transform, except at
  // M = 4096, where its 16 registers buy a third wave per SIMD instead (161
  // instead of 178 VGPRs with the weights cached)
  constexpr bool kPrefetch = LOG2M != 12;
  float2 upre[8];
  if constexpr (kPrefetch) {
    int h0;
    size_t r0;
    const bool a0 = row_of(gb * groups_per_block, h0, r0);
    const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (a0 ? r0 : 0));
#pragma unroll
    for (int r = 0; r < 8; ++r) upre[r] = a0 ? load_stream(&ur[lt + T * r]) : make_float2(0.f, 0.f);
  }
  // weights of the thread's bins, held across the rows of a channel where the
  // registers allow it (M <= 4096)
  constexpr bool kCache = LOG2M <= 12;
  float4 cw[kCache ? 16 : 1];
  int hc = -1;
  for (int gi = 0; gi < groups_per_block; ++gi) {
    const int g = gb * groups_per_block + gi;
    if (g >= ngroups) break;                     // uniform over the block
    int h;
    size_t roff;
    const bool active = row_of(g, h, roff);
    float2 v[16];
    if constexpr (kPrefetch) {
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = upre[r];
    } else {
      const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (active ? roff : 0));
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = active ? load_stream(&ur[lt + T * r]) : make_float2(0.f, 0.f);
    }
    if constexpr (kCache) {
      if (h != hc) {
        const float4* __restrict__ cf = coef + (size_t)h * M;
#pragma unroll
        for (int r = 0; r < 16; ++r) cw[r] = cf[lt + T * r];
        hc = h;
      }
    }
    dft16_fwd_half_input(v);
    __syncthreads();                             // the previous row's last reads are done
    WPass<LOG2M, 0>::store(v, buf, lt);
    __syncthreads();
    if constexpr (P > 2) row_pass<LOG2M, 1, false>(v, buf, lt, pt1);
    if constexpr (P > 3) row_pass<LOG2M, 2, false>(v, buf, lt, pt2);
    // last forward pass: the bins lt + T (q + s NB) stay in registers
    float2 z[16];
    {
      float2 w[16];
      ptl.expand(w);
      FL::load(v, buf, lt);
      __syncthreads();
      FL::template compute<false>(v, w);
      FL::store(v, buf, lt);
#pragma unroll
      for (int q = 0; q < FL::NB; ++q)
#pragma unroll
        for (int s2 = 0; s2 < FL::R; ++s2) z[q + s2 * FL::NB] = v[q * FL::R + bitrev<FL::RL>(s2)];
      __syncthreads();
    }
    {
      const float4* __restrict__ cf = coef + (size_t)h * M;
      const int nlt = -lt;
      const float2* __restrict__ bm = buf + (nlt + (nlt >> 4));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float2 zm;
        if (r == 0) zm = buf[lds_pad((M - lt) & (M - 1))];
        else zm = bm[(M - T * r) + ((M - T * r) >> 4)];
        float4 c;
        if constexpr (kCache) c = cw[r];
        else c = cf[lt + T * r];
        v[r] = cadd(cmul(make_float2(c.x, c.y), z[r]), cmul(make_float2(c.z, c.w), cconj(zm)));
      }
    }
    // next row's input, in flight during the inverse transform
    if (kPrefetch && gi + 1 < groups_per_block && g + 1 < ngroups) {
      int hn;
      size_t rn;
      const bool an = row_of(g + 1, hn, rn);
      const float2* __restrict__ ur = reinterpret_cast<const float2*>(u + (an ? rn : 0));
#pragma unroll
      for (int r = 0; r < 8; ++r) upre[r] = an ? load_stream(&ur[lt + T * r]) : make_float2(0.f, 0.f);
    }
    __syncthreads();                             // all partner reads done
    WPass<LOG2M, 0>::template compute<true>(v, z);
    WPass<LOG2M, 0>::store(v, buf, lt);
    __syncthreads();
    if constexpr (P > 2) row_pass<LOG2M, 1, true>(v, buf, lt, pt1);
    if constexpr (P > 3) row_pass<LOG2M, 2, true>(v, buf, lt, pt2);
    {
      float2 w[16];
      ptl.expand(w);
      FL::load(v, buf, lt);
      FL::template compute<true>(v, w);
    }
    float2* __restrict__ yr = reinterpret_cast<float2*>(y + roff);
#pragma unroll
    for (int q = 0; q < FL::NB; ++q) {
      const int j = lt + q * T;                   // j < NS in the last pass
#pragma unroll
      for (int s2 = 0; s2 < FL::R / 2; ++s2)
        if (active) store_stream(&yr[j + s2 * FL::NS], v[q * FL::R + bitrev<FL::RL>(s2)]);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
bool lds_path(const s4dplr_plan* p) { return p->log2L <= S4DPLR_LDS_MAX_LOG2L; }

template <typename T>
static T* at(unsigned char* ws, size_t off) { return reinterpret_cast<T*>(ws + off); }

static ParamPtrs param_ptrs(const float* lam, const float* P, const float* Q, const float* B,
                            const float* C, const float* dt) {
  return ParamPtrs{reinterpret_cast<const float2*>(lam), reinterpret_cast<const float2*>(P),
                   reinterpret_cast<const float2*>(Q), reinterpret_cast<const float2*>(B),
                   reinterpret_cast<const float2*>(C), dt};
}

static bool fused_path(const s4dplr_plan* p) { return p->log2L >= 5 && p->log2L <= 10; }

template <int LOG2L>
static void kgen_launch(const s4dplr_plan* p, const ParamPtrs& pp, const float* D,
                        const float* Ktime, float* Kout, unsigned char* ws, hipStream_t s,
                        int conj) {
  if constexpr (LOG2L >= 5 && LOG2L <= 10) {
    using S = KgenShape<LOG2L>;
    float4* coef = at<float4>(ws, p->off_coef);
    const float* tanT = at<const float>(ws, p->off_tan);
    const float2* tw = at<const float2>(ws, p->off_twL);
    const float2* cs = at<const float2>(ws, p->off_cs);
    if (Ktime)
      kgen_wave_kernel<LOG2L, false, true><<<p->H, S::NTHR, 0, s>>>(pp, D, Ktime, nullptr, coef,
                                                                  tanT, tw, cs, p->N, p->NP, conj);
    else if (p->flags & S4DPLR_DIAGONAL)
      kgen_wave_kernel<LOG2L, true, false><<<p->H, S::NTHR, 0, s>>>(pp, D, nullptr, Kout, coef,
                                                                  tanT, tw, cs, p->N, p->NP, 0);
    else if (!pp.Q)   // Q tied to P
      kgen_wave_kernel<LOG2L, false, false, true><<<p->H, S::NTHR, 0, s>>>(
          pp, D, nullptr, Kout, coef, tanT, tw, cs, p->N, p->NP, 0);
    else
      kgen_wave_kernel<LOG2L, false, false><<<p->H, S::NTHR, 0, s>>>(pp, D, nullptr, Kout, coef,
                                                                   tanT, tw, cs, p->N, p->NP, 0);
  }
}

static hipError_t launch_cauchy_to(const s4dplr_plan* p, const ParamPtrs& pp, float2* khat,
                                   unsigned char* ws, hipStream_t s) {
  constexpr int F = 2;
  const int per_block = F * kCauchyThreads;
  dim3 grid((p->L + per_block - 1) / per_block, p->H);
  const float* tanT = at<const float>(ws, p->off_tan);
  if (p->flags & S4DPLR_DIAGONAL)
    cauchy_kernel<F, true, false><<<grid, kCauchyThreads, 0, s>>>(pp, tanT, khat, p->N, p->NP,
                                                                  p->L);
  else if (!pp.Q)   // Q tied to P: w11 = |P|^2 is real
    cauchy_kernel<F, false, true><<<grid, kCauchyThreads, 0, s>>>(pp, tanT, khat, p->N, p->NP,
                                                                  p->L);
  else
    cauchy_kernel<F, false, false><<<grid, kCauchyThreads, 0, s>>>(pp, tanT, khat, p->N, p->NP,
                                                                   p->L);
  return hipGetLastError();
}

template <bool DIAG, bool TIED>
static void cauchy_half_launch(const s4dplr_plan* p, const ParamPtrs& pp, const float* D,
                               unsigned char* ws, hipStream_t s) {
  const dim3 grid(p->L / 2 / kCauchyThreads, p->H);
  cauchy_half_kernel<DIAG, TIED><<<grid, kCauchyThreads, 0, s>>>(
      pp, at<const float>(ws, p->off_tan), at<const float2>(ws, p->off_cs),
      at<float2>(ws, p->off_khat), at<float2>(ws, p->off_coef), D, p->N, p->NP, p->L);
}

// The generating function for stage 1 (rank 1).  L >= 32768: the packed
// kernel's L/2-point spectrum and the even bins of the padded spectrum (D
// folded in) instead of K-hat.
static hipError_t launch_cauchy(const s4dplr_plan* p, const ParamPtrs& pp, const float* D,
                                unsigned char* ws, hipStream_t s) {
  if (!lds_path(p)) {
    if (p->flags & S4DPLR_DIAGONAL) cauchy_half_launch<true, false>(p, pp, D, ws, s);
    else if (!pp.Q) cauchy_half_launch<false, true>(p, pp, D, ws, s);
    else cauchy_half_launch<false, false>(p, pp, D, ws, s);
    return hipGetLastError();
  }
  return launch_cauchy_to(p, pp, at<float2>(ws, p->off_khat), ws, s);
}

hipError_t launch_generating_function(const s4dplr_plan* p, const float* lam, const float* P,
                                      const float* Q, const float* B, const float* C,
                                      const float* dt, float* khat, unsigned char* ws,
                                      hipStream_t s) {
  const ParamPtrs pp = param_ptrs(lam, P, Q, B, C, dt);
  float2* out = reinterpret_cast<float2*>(khat);
  if (p->rank > 1) return launch_cauchy_rank(p, pp, out, 0, ws, s);
  return launch_cauchy_to(p, pp, out, ws, s);
}

template <int LOG2L>
static void kspec_launch(const s4dplr_plan* p, const float* Ktime, const float* D, float* Kout,
                         unsigned char* ws, hipStream_t s, int conj) {
  using S = KspecShape<LOG2L>;
  const float2* khat = at<const float2>(ws, p->off_khat);
  float4* coef = at<float4>(ws, p->off_coef);
  const float2* twL = at<const float2>(ws, p->off_twL);
  const float2* twH = at<const float2>(ws, p->off_twH);
  const float2* cs = at<const float2>(ws, p->off_cs);
  if (Ktime)
    kspec_kernel<LOG2L, true><<<p->H, S::NT, 0, s>>>(khat, Ktime, D, Kout, coef, twL, twH, cs,
                                                     conj);
  else
    kspec_kernel<LOG2L, false><<<p->H, S::NT, 0, s>>>(khat, Ktime, D, Kout, coef, twL, twH, cs,
                                                      conj);
}

template <int LOG2L>
static void conv_launch(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                        hipStream_t s) {
  if constexpr (LOG2L >= 5 && LOG2L <= 10) {
    using W = WaveConvShape<LOG2L>;
    const int rows = p->batch * p->H;
    const int ngroups = (rows + W::RPW - 1) / W::RPW;
    constexpr int kTargetWaves = 256 * 8;        // two waves per SIMD
    const int gpw = (ngroups + kTargetWaves - 1) / kTargetWaves;
    const int waves = (ngroups + gpw - 1) / gpw;
    const int blocks = (waves + 3) / 4;
    if constexpr (LOG2L == 10) {
      conv_pair1024_kernel<<<blocks, kWaveConvThreads, 0, s>>>(
          u, y, at<const float4>(ws, p->off_coef), at<const float2>(ws, p->off_twL), p->H,
          p->batch, gpw);
      return;
    }
    conv_wave_kernel<LOG2L><<<blocks, kWaveConvThreads, 0, s>>>(
        u, y, at<const float4>(ws, p->off_coef), at<const float2>(ws, p->off_twL), p->H,
        p->batch, gpw);
    return;
  }
  if constexpr (LOG2L >= 11 && LOG2L <= 14) {
    using R = RowConvShape<LOG2L>;
    const int rows = p->batch * p->H;
    const int ngroups = (rows + R::RPB - 1) / R::RPB;
    // blocks resident per CU, limited by LDS (160 KB) and 32 waves; at
    // L = 4096 by registers (three waves per SIMD, three blocks per CU):
    // persistent blocks sized to that ran 2-3% faster than two rounds of
    // four-per-CU blocks
    constexpr int by_lds = (160 * 1024) / (R::RPB * R::MP * 8);
    constexpr int by_waves = 32 / (R::NTHR / 64);
    constexpr int per_cu = LOG2L == 12 ? 3 : (by_lds < by_waves ? by_lds : by_waves);
    // Persistent blocks, one round of the resident capacity; at one block per
    // CU (L = 16384) two rounds: 2 rows per block at 1024 rows ran 3.5% faster
    // than 4 (one round) and than 1 or 3.
    const int target = 256 * (per_cu > 1 ? per_cu : 2);
    const int gpb = (ngroups + target - 1) / target;
    const int blocks = (ngroups + gpb - 1) / gpb;
    conv_rows_kernel<LOG2L><<<blocks, R::NTHR, 0, s>>>(
        u, y, at<const float4>(ws, p->off_coef), at<const float2>(ws, p->off_twL), p->H,
        p->batch, gpb);
    return;
  }
  using S = ConvShape<LOG2L>;
  const int rows = p->batch * p->H;
  const int blocks = (rows + S::RPW - 1) / S::RPW;
  conv_kernel<LOG2L><<<blocks, S::NTHR, 0, s>>>(u, y, at<const float4>(ws, p->off_coef),
                                                at<const float2>(ws, p->off_twH),
                                                at<const float2>(ws, p->off_cs), p->H, p->batch);
}

#define S4_DISPATCH_LOG2L(fn, ...)          \
  switch (p->log2L) {                       \
    case 1: fn<1>(__VA_ARGS__); break;      \
    case 2: fn<2>(__VA_ARGS__); break;      \
    case 3: fn<3>(__VA_ARGS__); break;      \
    case 4: fn<4>(__VA_ARGS__); break;      \
    case 5: fn<5>(__VA_ARGS__); break;      \
    case 6: fn<6>(__VA_ARGS__); break;      \
    case 7: fn<7>(__VA_ARGS__); break;      \
    case 8: fn<8>(__VA_ARGS__); break;      \
    case 9: fn<9>(__VA_ARGS__); break;      \
    case 10: fn<10>(__VA_ARGS__); break;    \
    case 11: fn<11>(__VA_ARGS__); break;    \
    case 12: fn<12>(__VA_ARGS__); break;    \
    case 13: fn<13>(__VA_ARGS__); break;    \
    case 14: fn<14>(__VA_ARGS__); break;    \
    default: return hipErrorInvalidValue;   \
  }

static hipError_t launch_kspec(const s4dplr_plan* p, const float* Ktime, const float* D,
                               float* Kout, unsigned char* ws, hipStream_t s, int conj,
                               bool half = false) {
  if (!lds_path(p)) return launch_big_kspec(p, Ktime, D, Kout, ws, s, conj, half);
  S4_DISPATCH_LOG2L(kspec_launch, p, Ktime, D, Kout, ws, s, conj);
  return hipGetLastError();
}

hipError_t launch_kernel_gen(const s4dplr_plan* p, const float* lam, const float* P,
                             const float* Q, const float* B, const float* C, const float* dt,
                             const float* D, float* Kout, unsigned char* ws, hipStream_t s) {
  if (p->flags & S4DPLR_ZOH) {
    // zero-order hold: the Vandermonde kernel, then the spectrum of (K + D delta)
    float* K = Kout ? Kout : at<float>(ws, p->off_kbuf);
    hipError_t e = launch_vandermonde(p, lam, B, C, dt, K, s);
    if (e != hipSuccess) return e;
    return launch_spectrum_from_time(p, K, D, ws, s, 0);
  }
  const ParamPtrs pp = param_ptrs(lam, P, Q, B, C, dt);
  if (p->rank > 1) {
    // rank r: the (r+1)^2 Cauchy sums and the r x r Woodbury solve, then the
    // kernel spectrum from K-hat (every length, the block-level transform up
    // to 2^14)
    hipError_t e = launch_cauchy_rank(p, pp, at<float2>(ws, p->off_khat),
                                      lds_path(p) ? 0 : p->L / 256, ws, s);
    if (e != hipSuccess) return e;
    return launch_kspec(p, nullptr, D, Kout, ws, s, 0);
  }
  if (fused_path(p)) {
    S4_DISPATCH_LOG2L(kgen_launch, p, pp, D, nullptr, Kout, ws, s, 0);
    return hipGetLastError();
  }
  hipError_t e = launch_cauchy(p, pp, D, ws, s);
  if (e != hipSuccess) return e;
  // L >= 32768: launch_cauchy wrote the half-length spectrum Y and the even bins
  return launch_kspec(p, nullptr, D, Kout, ws, s, 0, !lds_path(p));
}

hipError_t launch_spectrum_from_time(const s4dplr_plan* p, const float* Ktime, const float* D,
                                     unsigned char* ws, hipStream_t s, int conj) {
  if (fused_path(p)) {
    const ParamPtrs pp{};
    S4_DISPATCH_LOG2L(kgen_launch, p, pp, D, Ktime, nullptr, ws, s, conj);
    return hipGetLastError();
  }
  return launch_kspec(p, Ktime, D, nullptr, ws, s, conj);
}

hipError_t launch_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                       hipStream_t s) {
  if (!lds_path(p)) return launch_big_conv(p, u, y, ws, s);
  S4_DISPATCH_LOG2L(conv_launch, p, u, y, ws, s);
  return hipGetLastError();
}

}  // namespace s4
