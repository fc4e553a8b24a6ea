// Pole records and the Cauchy sums of the generating function at the L roots
// of unity ("The S4 kernel, from scratch", section 4), shared by the forward
// kernel generation and its backward pass.
#pragma once

#include <hip/hip_runtime.h>

#include "device_fft.h"
#include "internal.h"

namespace s4 {

// A block first writes its channel's pole records into LDS (5 float4 each):
//   rec[5n]   = (Im Lambda_n, (Re Lambda_n)^2, K00),  rec[5n+1] = (w00, K01),
//   rec[5n+2] = (w01, K10),  rec[5n+3] = (w10, K11),  rec[5n+4] = (w11, 0)
// with w00 = C B, w01 = C P, w10 = conj(Q) B, w11 = conj(Q) P and
// K_ab = -Re(Lambda_n) w_ab (both parts).  Poles n in [N, NP) (NP = N rounded
// up to kPoleUnroll) are inert: zero weights, Lambda = -1.  Per term, with
// y = G - Im Lambda and r = 1 / ((Re Lambda)^2 + y^2),
//   w_ab / (i G - Lambda) = r (K_ab.re + w_ab.im y) + i r (K_ab.im - w_ab.re y),
// i.e. two FMAs for the numerator and two for the accumulation per sum.
constexpr int kPoleUnroll = 4;
constexpr int kMaxPoles = 256;
constexpr int kCauchyThreads = 256;   // threads of the frequency-parallel Cauchy kernels

struct ParamPtrs {
  const float2* lam;
  const float2* P;
  const float2* Q;   // nullptr: Q = P
  const float2* B;
  const float2* C;
  const float* dt;
};

constexpr int kRec = 5;   // float4 per pole record

// Generating function for plans of rank 2 .. 4 (rank.hip): khat [H][L] in
// natural order (perm_m1 = 0) or the four-step permuted order (perm_m1 = M1).
hipError_t launch_cauchy_rank(const s4dplr_plan* p, const ParamPtrs& pp, float2* khat,
                              int perm_m1, unsigned char* ws, hipStream_t s);

// Builds the records of channel h with threads [0, nthr); returns this
// thread's partial sum of w00 = C B over its poles.
__device__ __forceinline__ float2 build_pole_records(const ParamPtrs& pp, int h, int N, int NP,
                                                     bool diag, float4* __restrict__ rec, int tid,
                                                     int nthr) {
  float2 s = make_float2(0.f, 0.f);
  for (int n = tid; n < NP; n += nthr) {
    float4* rn = rec + kRec * n;
    if (n < N) {
      const size_t idx = (size_t)h * N + n;
      const float2 l = pp.lam[idx], b = pp.B[idx], c = pp.C[idx];
      const float2 pv = diag ? make_float2(0.f, 0.f) : pp.P[idx];
      const float2 qv = diag ? make_float2(0.f, 0.f) : (pp.Q ? pp.Q[idx] : pv);
      const float2 w00 = cmul(c, b), w01 = cmul(c, pv);
      const float2 w10 = cmul(cconj(qv), b), w11 = cmul(cconj(qv), pv);
      const float na = -l.x;
      rn[0] = make_float4(l.y, l.x * l.x, na * w00.x, na * w00.y);
      rn[1] = make_float4(w00.x, w00.y, na * w01.x, na * w01.y);
      rn[2] = make_float4(w01.x, w01.y, na * w10.x, na * w10.y);
      rn[3] = make_float4(w10.x, w10.y, na * w11.x, na * w11.y);
      rn[4] = make_float4(w11.x, w11.y, 0.f, 0.f);
      s = cadd(s, w00);
    } else {
      rn[0] = make_float4(0.f, 1.f, 0.f, 0.f);
      rn[1] = make_float4(0.f, 0.f, 0.f, 0.f);
      rn[2] = make_float4(0.f, 0.f, 0.f, 0.f);
      rn[3] = make_float4(0.f, 0.f, 0.f, 0.f);
      rn[4] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  return s;
}

// Sum of a float2 over the block (blockDim a multiple of 64); ends with a
// barrier, so LDS written before the call is visible to all threads after it.
template <int NTHR>
__device__ __forceinline__ float2 block_sum2(float2 v, float2* __restrict__ red, int tid) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    v.x += __shfl_xor(v.x, off);
    v.y += __shfl_xor(v.y, off);
  }
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float2 s = make_float2(0.f, 0.f);
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) s = cadd(s, red[w]);
  return s;
}

// acc[f][0..7] += the four Cauchy sums (re, im) at G[f], over poles [0, NP).
// TIED (Q = P): w11 = conj(P) P = |P|^2 is real, so the last sum takes
// r K11 (one FMA) and -|P|^2 (r y) (one product shared with nothing else and
// one FMA) instead of two nested FMAs per part: 17 VALU + 1 reciprocal per
// term instead of 18 + 1.
template <int F, bool DIAG, bool TIED = false>
__device__ __forceinline__ void cauchy_sums(const float4* __restrict__ rec, int NP,
                                            const float (&G)[F], float (&acc)[F][8]) {
  for (int n0 = 0; n0 < NP; n0 += kPoleUnroll) {
#pragma unroll
    for (int n = n0; n < n0 + kPoleUnroll; ++n) {
      const float4* rn = rec + kRec * n;
      const float4 p0 = rn[0], p1 = rn[1];
      float4 p2 = make_float4(0.f, 0.f, 0.f, 0.f), p3 = p2, p4 = p2;
      if constexpr (!DIAG) {
        p2 = rn[2];
        p3 = rn[3];
        p4 = rn[4];
      }
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const float yv = G[f] - p0.x;
        const float r = __builtin_amdgcn_rcpf(fmaf(yv, yv, p0.y));
        // sum 00: w = p1.xy, K = p0.zw
        acc[f][0] = fmaf(r, fmaf(p1.y, yv, p0.z), acc[f][0]);
        acc[f][1] = fmaf(r, fmaf(-p1.x, yv, p0.w), acc[f][1]);
        if constexpr (!DIAG) {
          // sum 01: w = p2.xy, K = p1.zw; sum 10: w = p3.xy, K = p2.zw; sum 11: w = p4.xy, K = p3.zw
          acc[f][2] = fmaf(r, fmaf(p2.y, yv, p1.z), acc[f][2]);
          acc[f][3] = fmaf(r, fmaf(-p2.x, yv, p1.w), acc[f][3]);
          acc[f][4] = fmaf(r, fmaf(p3.y, yv, p2.z), acc[f][4]);
          acc[f][5] = fmaf(r, fmaf(-p3.x, yv, p2.w), acc[f][5]);
          if constexpr (TIED) {
            acc[f][6] = fmaf(r, p3.z, acc[f][6]);
            acc[f][7] = fmaf(-p4.x, r * yv, acc[f][7]);
          } else {
            acc[f][6] = fmaf(r, fmaf(p4.y, yv, p3.z), acc[f][6]);
            acc[f][7] = fmaf(r, fmaf(-p4.x, yv, p3.w), acc[f][7]);
          }
        }
      }
    }
  }
}

// Woodbury correction and the 2/(1+z) = 1 + i tan(theta/2) factor; at z = -1
// (the frequency l = L/2) the limit `nyq` = (dt/2) sum_n C_n B_n.
template <bool DIAG>
__device__ __forceinline__ float2 cauchy_epilogue(const float (&a)[8], float T, bool at_nyquist,
                                                  float2 nyq) {
  float2 kv = make_float2(a[0], a[1]);
  if constexpr (!DIAG) {
    // k00 - k01 k10 / (1 + k11)
    const float2 k01 = make_float2(a[2], a[3]);
    const float2 k10 = make_float2(a[4], a[5]);
    const float2 den = make_float2(1.0f + a[6], a[7]);
    const float2 num = cmul(k01, k10);
    const float inv = 1.0f / fmaf(den.x, den.x, den.y * den.y);
    const float2 t = cmulc(num, den);
    kv = make_float2(fmaf(-t.x, inv, kv.x), fmaf(-t.y, inv, kv.y));
  }
  const float2 kh = cmul(make_float2(1.0f, T), kv);
  return at_nyquist ? nyq : kh;
}

}  // namespace s4
