// Diagonal systems discretized by zero-order hold ("The S4 kernel, from
// scratch", section 3: A-bar = exp(dt a); "S4" wiki, "S4D": A diagonal).  The
// kernel is evaluated from its definition as a Vandermonde product,
//   K[h][k] = Re(sum_n W_n A-bar_n^k),  W_n = C_n B-bar_n,
//   A-bar_n = exp(z_n),  B-bar_n = B_n expm1(z_n) / Lambda_n,  z_n = dt Lambda_n
// (B-bar_n = dt B_n at Lambda_n = 0), for k = 0 .. L-1: the kernel itself, not
// an aliased one.
//
// Each thread owns TAPS consecutive taps (16, or 32 for L >= 4096, where
// the per-pole start below is then spread over twice the taps): it forms
// W A-bar^k0 once per pole (exp of k0 z with the phase reduced modulo 2 pi in
// fp64, so the rounding does not grow with k0) and steps the rest by complex
// products.
//
// Backward: with S0_n = sum_k dK_k conj(A-bar_n)^k and
// S1_n = sum_k k dK_k conj(A-bar_n)^k, and grad(v) = dloss/dRe v + i dloss/dIm v,
//   grad(C_n) = conj(B-bar_n) S0_n,       grad(B_n) = conj(C_n e_n) S0_n,
//   grad(Lambda_n) = conj(C_n B_n de_n) S0_n + conj(W_n dt) S1_n,
//   dloss/ddt = Re sum_n (conj(C_n B_n A-bar_n) S0_n + conj(W_n Lambda_n) S1_n),
// where e_n = expm1(z_n) / Lambda_n and de_n = d e_n / d Lambda_n
// = (dt A-bar_n - e_n) / Lambda_n (a series in z_n near 0).
#include <hip/hip_runtime.h>

#include <math.h>

#include "device_fft.h"
#include "internal.h"

namespace s4 {

namespace {

constexpr int kVanderKT = 64;                      // tap threads per block (one wave)
constexpr int kVanderPG = 4;                       // pole groups per block (waves)
constexpr int kMaxPolesZoh = 256;
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

struct cd {
  double re, im;
};
__device__ __forceinline__ cd cd_mul(cd a, cd b) {
  return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
}
__device__ __forceinline__ cd cd_div(cd a, cd b) {
  const double inv = 1.0 / (b.re * b.re + b.im * b.im);
  return {(a.re * b.re + a.im * b.im) * inv, (a.im * b.re - a.re * b.im) * inv};
}
__device__ __forceinline__ cd cd_load(const float2* p, size_t i) {
  const float2 v = p[i];
  return {(double)v.x, (double)v.y};
}
__device__ __forceinline__ float2 to_f(cd a) { return make_float2((float)a.re, (float)a.im); }

// exp(z) and expm1(z) / lambda for z = dt lambda, in fp64; e -> dt at lambda = 0.
struct ZohPole {
  cd abar, e;
};
__device__ __forceinline__ ZohPole zoh_pole(cd lam, double dt) {
  const cd z = {dt * lam.re, dt * lam.im};
  const double ex = exp(z.re);
  double s, c;
  sincos(z.im, &s, &c);
  ZohPole r;
  r.abar = {ex * c, ex * s};
  if (lam.re == 0.0 && lam.im == 0.0) {
    r.e = {dt, 0.0};
  } else {
    // expm1(x + iy) = expm1(x) cos y - 2 sin^2(y/2) + i e^x sin y
    const double sh = sin(0.5 * z.im);
    const cd em1 = {expm1(z.re) * c - 2.0 * sh * sh, ex * s};
    r.e = cd_div(em1, lam);
  }
  return r;
}

// exp(k z) for an integer k >= 0 with the phase reduced in fp64.
__device__ __forceinline__ float2 power_of(double zre, double zim, double k) {
  double ph = k * zim;
  ph = fma(-kTwoPi, rint(ph * kInvTwoPi), ph);
  const float mag = expf((float)(k * zre));
  float s, c;
  sincosf((float)ph, &s, &c);
  return make_float2(mag * c, mag * s);
}

}  // namespace

// Pole records in LDS: (W re, W im, A-bar re, A-bar im) and (z re, z im) in fp64.
// Block (tap range, h): wave g of the PG waves sums the poles n = g, g + PG,
// ... for TAPS taps per lane; the waves' partial sums meet in LDS.  Short
// kernels (few tap ranges per channel) take PG = 16 so that the grid still
// gives every SIMD several waves.
template <int TAPS, int PG>
__global__ __launch_bounds__(kVanderKT * PG) void vander_kernel(
    const float2* __restrict__ lam, const float2* __restrict__ B, const float2* __restrict__ C,
    const float* __restrict__ dt, float* __restrict__ K, int N, int L) {
  static_assert(TAPS % PG == 0, "each thread finishes TAPS / PG taps");
  __shared__ float4 wa[kMaxPolesZoh];
  __shared__ double2 zz[kMaxPolesZoh];
  __shared__ float red[PG][kVanderKT][TAPS + 1];
  const int h = blockIdx.y, tid = threadIdx.x;
  const double d = (double)dt[h];
  for (int n = tid; n < N; n += kVanderKT * PG) {
    const size_t i = (size_t)h * N + n;
    const cd l = cd_load(lam, i);
    const ZohPole zp = zoh_pole(l, d);
    const cd w = cd_mul(cd_load(C, i), cd_mul(cd_load(B, i), zp.e));
    const float2 wf = to_f(w), af = to_f(zp.abar);
    wa[n] = make_float4(wf.x, wf.y, af.x, af.y);
    zz[n] = make_double2(d * l.re, d * l.im);
  }
  __syncthreads();
  const int kt = tid % kVanderKT, pg = tid / kVanderKT;
  const int k0 = (blockIdx.x * kVanderKT + kt) * TAPS;
  float acc[TAPS];
#pragma unroll
  for (int j = 0; j < TAPS; ++j) acc[j] = 0.f;
  if (k0 < L) {
    for (int n = pg; n < N; n += PG) {
      const float4 r = wa[n];
      const double2 z = zz[n];
      const float2 a = make_float2(r.z, r.w);
      float2 q = cmul(make_float2(r.x, r.y), power_of(z.x, z.y, (double)k0));
#pragma unroll
      for (int j = 0; j < TAPS; ++j) {
        acc[j] += q.x;
        q = cmul(q, a);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TAPS; ++j) red[pg][kt][j] = acc[j];
  __syncthreads();
  // thread (kt, pg) finishes taps [pg T/G, (pg + 1) T/G) of its tap range
  constexpr int TPG = TAPS / PG;
  if (k0 < L) {
    float* out = K + (size_t)h * L + k0;
#pragma unroll
    for (int m = 0; m < TPG; ++m) {
      const int j = pg * TPG + m;
      float v = 0.f;
#pragma unroll
      for (int g = 0; g < PG; ++g) v += red[g][kt][j];
      if (k0 + j < L) out[j] = v;
    }
  }
}

// Backward partial sums S0, S1 over a chunk of kBwdChunk taps: block
// (chunk, h); thread = (pole n, a run of consecutive taps of the chunk).
__global__ __launch_bounds__(256) void vander_bwd_kernel(
    const float2* __restrict__ lam, const float* __restrict__ dt, const float* __restrict__ dK,
    float2* __restrict__ part, int N, int L, int log2npp) {
  __shared__ float sk[kBwdChunk];
  __shared__ float red[256 * 4];
  const int h = blockIdx.y, lc = blockIdx.x, tid = threadIdx.x;
  const int l0 = lc * kBwdChunk;
  const int nl = min(kBwdChunk, L - l0);
  for (int i = tid; i < nl; i += 256) sk[i] = dK[(size_t)h * L + l0 + i];
  const int npp = 1 << log2npp, sub_n = 256 >> log2npp;
  const int n = tid & (npp - 1), sub = tid >> log2npp;
  const int run = (kBwdChunk + sub_n - 1) / sub_n;
  const int i0 = sub * run, i1 = min(nl, i0 + run);
  __syncthreads();
  float2 s0 = make_float2(0.f, 0.f), s1 = s0;
  if (n < N && i0 < i1) {
    const double d = (double)dt[h];
    const float2 l = lam[(size_t)h * N + n];
    const double zre = d * (double)l.x, zim = -d * (double)l.y;   // conj(z)
    float2 p = power_of(zre, zim, (double)(l0 + i0));
    const float2 ac = power_of(zre, zim, 1.0);
    for (int i = i0; i < i1; ++i) {
      const float g = sk[i];
      const float gk = g * (float)(l0 + i);
      s0 = make_float2(fmaf(g, p.x, s0.x), fmaf(g, p.y, s0.y));
      s1 = make_float2(fmaf(gk, p.x, s1.x), fmaf(gk, p.y, s1.y));
      p = cmul(p, ac);
    }
  }
  float* rv = red + 4 * tid;
  rv[0] = s0.x;
  rv[1] = s0.y;
  rv[2] = s1.x;
  rv[3] = s1.y;
  __syncthreads();
  if (sub == 0 && n < N) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < sub_n; ++q) {
      const float* o = red + 4 * (q * npp + n);
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] += o[c];
    }
    float2* out = part + 2 * (((size_t)h * gridDim.x + lc) * N + n);
    out[0] = make_float2(a[0], a[1]);
    out[1] = make_float2(a[2], a[3]);
  }
}

__global__ __launch_bounds__(256) void vander_bwd_final_kernel(
    const float2* __restrict__ lam, const float2* __restrict__ B, const float2* __restrict__ C,
    const float* __restrict__ dt, const float2* __restrict__ part, float2* __restrict__ dlam,
    float2* __restrict__ dB, float2* __restrict__ dC, float* __restrict__ ddt, int N,
    int nchunks) {
  __shared__ double red[4];
  const int h = blockIdx.x, tid = threadIdx.x;
  const double d = (double)dt[h];
  double dsum = 0.0;
  for (int n = tid; n < N; n += 256) {
    const size_t i = (size_t)h * N + n;
    cd S0 = {0.0, 0.0}, S1 = {0.0, 0.0};
    for (int lc = 0; lc < nchunks; ++lc) {
      const float2* o = part + 2 * (((size_t)h * nchunks + lc) * N + n);
      S0.re += o[0].x;
      S0.im += o[0].y;
      S1.re += o[1].x;
      S1.im += o[1].y;
    }
    const cd l = cd_load(lam, i), b = cd_load(B, i), c = cd_load(C, i);
    const ZohPole zp = zoh_pole(l, d);
    const cd cb = cd_mul(c, b);
    const cd w = cd_mul(cb, zp.e);
    // de = d e / d lambda = (dt A-bar - e) / lambda, or its series near z = 0:
    // dt^2 (1/2 + z/3 + z^2/8 + z^3/30 + z^4/144)
    const cd z = {d * l.re, d * l.im};
    cd de;
    if (z.re * z.re + z.im * z.im < 1e-6) {
      cd s = {1.0 / 144.0, 0.0};
      const double cf[4] = {1.0 / 30.0, 1.0 / 8.0, 1.0 / 3.0, 0.5};
      for (int m = 0; m < 4; ++m) {
        s = cd_mul(s, z);
        s.re += cf[m];
      }
      de = {d * d * s.re, d * d * s.im};
    } else {
      de = cd_div({d * zp.abar.re - zp.e.re, d * zp.abar.im - zp.e.im}, l);
    }
    auto cmulconj = [](cd a, cd s) {   // conj(a) s
      return cd{a.re * s.re + a.im * s.im, a.re * s.im - a.im * s.re};
    };
    const cd bbar = cd_mul(b, zp.e);
    const cd gC = cmulconj(bbar, S0);
    const cd gB = cmulconj(cd_mul(c, zp.e), S0);
    const cd g1 = cmulconj(cd_mul(cb, de), S0), g2 = cmulconj({w.re * d, w.im * d}, S1);
    if (dC) dC[i] = to_f(gC);
    if (dB) dB[i] = to_f(gB);
    if (dlam) dlam[i] = make_float2((float)(g1.re + g2.re), (float)(g1.im + g2.im));
    dsum += cmulconj(cd_mul(cb, zp.abar), S0).re + cmulconj(cd_mul(w, l), S1).re;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off);
  if ((tid & 63) == 0) red[tid >> 6] = dsum;
  __syncthreads();
  if (tid == 0 && ddt) ddt[h] = (float)(red[0] + red[1] + red[2] + red[3]);
}

hipError_t launch_vandermonde(const s4dplr_plan* p, const float* lam, const float* B,
                              const float* C, const float* dt, float* K, hipStream_t s) {
  auto run = [&](auto kern, int taps, int pg) {
    const int per_block = kVanderKT * taps;
    const dim3 grid((p->L + per_block - 1) / per_block, p->H);
    kern<<<grid, kVanderKT * pg, 0, s>>>(
        reinterpret_cast<const float2*>(lam), reinterpret_cast<const float2*>(B),
        reinterpret_cast<const float2*>(C), dt, K, p->N, p->L);
  };
  const int blocks16 = (p->L + kVanderKT * 16 - 1) / (kVanderKT * 16) * p->H;
  if (p->L >= 4096) run(vander_kernel<32, kVanderPG>, 32, kVanderPG);
  else if (blocks16 < 1024) run(vander_kernel<16, 16>, 16, 16);
  else run(vander_kernel<16, kVanderPG>, 16, kVanderPG);
  return hipGetLastError();
}

hipError_t launch_vandermonde_bwd(const s4dplr_plan* p, const float* lam, const float* B,
                                  const float* C, const float* dt, const float* dK, float* dlam,
                                  float* dB, float* dC, float* ddt, unsigned char* ws,
                                  hipStream_t s) {
  int log2npp = 0;
  while ((1 << log2npp) < p->N) ++log2npp;
  const int nchunks = (p->L + kBwdChunk - 1) / kBwdChunk;
  float2* part = reinterpret_cast<float2*>(ws + p->off_bpart);
  const float2* l2 = reinterpret_cast<const float2*>(lam);
  vander_bwd_kernel<<<dim3(nchunks, p->H), 256, 0, s>>>(l2, dt, dK, part, p->N, p->L, log2npp);
  vander_bwd_final_kernel<<<p->H, 256, 0, s>>>(
      l2, reinterpret_cast<const float2*>(B), reinterpret_cast<const float2*>(C), dt, part,
      reinterpret_cast<float2*>(dlam), reinterpret_cast<float2*>(dB),
      reinterpret_cast<float2*>(dC), ddt, p->N, nchunks);
  return hipGetLastError();
}

}  // namespace s4
