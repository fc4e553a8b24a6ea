// Generating function for a rank-r low-rank term ("S4" wiki, "Structured
// Transition Matrix": A = Lambda - P Q^* with low-rank P, Q, the correction
// handled by the Woodbury identity; "The S4 kernel, from scratch", section 4
// for g(z), the roots of unity and the 2/(1+z) factor), 2 <= r <= 4.
//
// With R = (g - Lambda)^{-1} (diagonal), the Woodbury identity gives
//   C (g - A)^{-1} B = k00 - k01 (I_r + k11)^{-1} k10,
// k00 = C R B, k01[j] = C R P_j, k10[i] = Q_i^* R B, k11[i][j] = Q_i^* R P_j:
// (r + 1)^2 Cauchy sums over the poles that share each pole's reciprocal.
// Per frequency the r x r complex system (I + k11) x = k10 is solved by
// Gaussian elimination with partial pivoting, unrolled in registers.
#include <hip/hip_runtime.h>

#include "cauchy.h"
#include "internal.h"

namespace s4 {

namespace {

constexpr int kRankThreads = 256;
constexpr int kRankChunk = 64;          // poles staged in LDS at a time

template <int R>
struct RankShape {
  static constexpr int E = (R + 1) * (R + 1);   // Cauchy sums
  static constexpr int REC = 1 + E;             // float4 per pole record
  static constexpr int F = R <= 2 ? 2 : 1;      // frequencies per thread
};

__device__ __forceinline__ float2 cdiv(float2 a, float2 b) {
  const float inv = 1.0f / fmaf(b.x, b.x, b.y * b.y);
  const float2 t = cmulc(a, b);   // a conj(b)
  return make_float2(t.x * inv, t.y * inv);
}

// Solves (I + k11) x = k10 in place: on return rhs holds x.
template <int R>
__device__ __forceinline__ void woodbury_solve(float2 (&M)[R][R], float2 (&rhs)[R]) {
#pragma unroll
  for (int k = 0; k < R; ++k) {
    // partial pivoting over rows k .. R-1
    int piv = k;
    float best = fmaf(M[k][k].x, M[k][k].x, M[k][k].y * M[k][k].y);
#pragma unroll
    for (int i = k + 1; i < R; ++i) {
      const float m = fmaf(M[i][k].x, M[i][k].x, M[i][k].y * M[i][k].y);
      if (m > best) {
        best = m;
        piv = i;
      }
    }
#pragma unroll
    for (int i = k + 1; i < R; ++i) {
      if (piv == i) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const float2 t = M[k][j];
          M[k][j] = M[i][j];
          M[i][j] = t;
        }
        const float2 t = rhs[k];
        rhs[k] = rhs[i];
        rhs[i] = t;
      }
    }
#pragma unroll
    for (int i = k + 1; i < R; ++i) {
      const float2 f = cdiv(M[i][k], M[k][k]);
#pragma unroll
      for (int j = k + 1; j < R; ++j) M[i][j] = csub(M[i][j], cmul(f, M[k][j]));
      rhs[i] = csub(rhs[i], cmul(f, rhs[k]));
    }
  }
#pragma unroll
  for (int k = R - 1; k >= 0; --k) {
    float2 s = rhs[k];
#pragma unroll
    for (int j = k + 1; j < R; ++j) s = csub(s, cmul(M[k][j], rhs[j]));
    rhs[k] = cdiv(s, M[k][k]);
  }
}

// Block (frequency tile, channel h).  P and Q are [H][R][N] complex (Q NULL:
// Q = P).  The records of each chunk of poles are staged in LDS:
//   rec[0] = (Im Lambda_n, (Re Lambda_n)^2, 0, 0),
//   rec[1 + a (R+1) + b] = (w_ab, -Re(Lambda_n) w_ab),
//   w_ab = left_a right_b, left = (C, conj(Q_1), ..), right = (B, P_1, ..),
// and, per term, w_ab / (i G - Lambda_n) = r (K.re + w.im y) + i r (K.im - w.re y)
// with y = G - Im Lambda_n and r = 1 / ((Re Lambda_n)^2 + y^2).
//
// The node G = (2/dt) tan(pi l / L) is carried as two floats, G = Gh + Gl
// (from the plan's two-float tan table, combined in fp64), and each term takes
// y = (Gh - Im Lambda_n) + Gl: next to a sharp pole (small |Re Lambda|) a
// single-float node misplaces r by |r| ulp(G) relatively, which the r x r
// solve then amplifies (2.5e-4 of max |K-hat| on a rank-2 case at L = 65536;
// 8e-7 with the two-float node).
template <int R>
__global__ __launch_bounds__(kRankThreads) void cauchy_rank_kernel(
    ParamPtrs pp, const float2* __restrict__ tan2, float2* __restrict__ khat, int N, int L,
    int perm_m1) {
  using S = RankShape<R>;
  constexpr int E = S::E, REC = S::REC, F = S::F;
  __shared__ float4 rec[kRankChunk * REC];
  __shared__ float2 red[kRankThreads / 64];
  const int h = blockIdx.y, tid = threadIdx.x;
  const float dt = pp.dt[h];
  const double two_dt = 2.0 / (double)dt;
  int l[F], pos[F];
  float T[F], G[F], Gl[F];
  float acc[F][E][2];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    pos[f] = (blockIdx.x * F + f) * kRankThreads + tid;
    l[f] = perm_m1 ? ((pos[f] >> 8) + perm_m1 * (pos[f] & 255)) : pos[f];
    const float2 t2 = pos[f] < L ? tan2[l[f]] : make_float2(0.f, 0.f);
    const double g = two_dt * ((double)t2.x + (double)t2.y);
    T[f] = t2.x;
    G[f] = (float)g;
    Gl[f] = (float)(g - (double)G[f]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[f][e][0] = acc[f][e][1] = 0.f;
  }
  const size_t hN = (size_t)h * N;
  const float2* Qs = pp.Q ? pp.Q : pp.P;
  float2 cb = make_float2(0.f, 0.f);    // this thread's part of sum_n C_n B_n
  for (int c0 = 0; c0 < N; c0 += kRankChunk) {
    const int nc = N - c0 < kRankChunk ? N - c0 : kRankChunk;
    __syncthreads();   // the previous chunk's records are no longer read
    if (tid < kRankChunk) {
      float4* rn = rec + REC * tid;
      if (tid < nc) {
        const int n = c0 + tid;
        const float2 lam = pp.lam[hN + n];
        float2 left[R + 1], right[R + 1];
        left[0] = pp.C[hN + n];
        right[0] = pp.B[hN + n];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const size_t idx = ((size_t)h * R + j) * N + n;
          left[1 + j] = cconj(Qs[idx]);
          right[1 + j] = pp.P[idx];
        }
        const float na = -lam.x;
        rn[0] = make_float4(lam.y, lam.x * lam.x, 0.f, 0.f);
#pragma unroll
        for (int a = 0; a <= R; ++a)
#pragma unroll
          for (int b = 0; b <= R; ++b) {
            const float2 w = cmul(left[a], right[b]);
            rn[1 + a * (R + 1) + b] = make_float4(w.x, w.y, na * w.x, na * w.y);
          }
        cb = cadd(cb, cmul(left[0], right[0]));
      } else {
        rn[0] = make_float4(0.f, 1.f, 0.f, 0.f);     // inert pole: Lambda = -1, zero weights
#pragma unroll
        for (int e = 0; e < E; ++e) rn[1 + e] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __syncthreads();
    const int nr = (nc + 3) & ~3;     // unrolled by 4 over inert padding
    for (int n0 = 0; n0 < nr; n0 += 4) {
#pragma unroll
      for (int n = n0; n < n0 + 4; ++n) {
        const float4* rn = rec + REC * n;
        const float4 p0 = rn[0];
#pragma unroll
        for (int f = 0; f < F; ++f) {
          const float yv = (G[f] - p0.x) + Gl[f];
          const float r = __builtin_amdgcn_rcpf(fmaf(yv, yv, p0.y));
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float4 q = rn[1 + e];
            acc[f][e][0] = fmaf(r, fmaf(q.y, yv, q.z), acc[f][e][0]);
            acc[f][e][1] = fmaf(r, fmaf(-q.x, yv, q.w), acc[f][e][1]);
          }
        }
      }
    }
  }
  const float2 sum = block_sum2<kRankThreads>(cb, red, tid);
  const float2 nyq = make_float2(0.5f * dt * sum.x, 0.5f * dt * sum.y);
#pragma unroll
  for (int f = 0; f < F; ++f) {
    if (pos[f] >= L) continue;
    float2 M[R][R], x[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int e = (1 + i) * (R + 1);
      x[i] = make_float2(acc[f][e][0], acc[f][e][1]);                  // k10[i]
#pragma unroll
      for (int j = 0; j < R; ++j)
        M[i][j] = make_float2((i == j ? 1.0f : 0.0f) + acc[f][e + 1 + j][0],
                              acc[f][e + 1 + j][1]);                      // I + k11
    }
    woodbury_solve<R>(M, x);
    float2 kv = make_float2(acc[f][0][0], acc[f][0][1]);                 // k00
#pragma unroll
    for (int j = 0; j < R; ++j)
      kv = csub(kv, cmul(make_float2(acc[f][1 + j][0], acc[f][1 + j][1]), x[j]));   // k01 x
    const float2 kh = cmul(make_float2(1.0f, T[f]), kv);                 // 2/(1+z) = 1 + i tan
    khat[(size_t)h * L + pos[f]] = (2 * l[f] == L) ? nyq : kh;
  }
}

template <int R>
static void rank_launch(const s4dplr_plan* p, const ParamPtrs& pp, const float2* tan2,
                        float2* khat, int perm_m1, hipStream_t s) {
  constexpr int per_block = RankShape<R>::F * kRankThreads;
  const dim3 grid((p->L + per_block - 1) / per_block, p->H);
  cauchy_rank_kernel<R><<<grid, kRankThreads, 0, s>>>(pp, tan2, khat, p->N, p->L, perm_m1);
}

}  // namespace

hipError_t launch_cauchy_rank(const s4dplr_plan* p, const ParamPtrs& pp, float2* khat,
                              int perm_m1, unsigned char* ws, hipStream_t s) {
  const float2* tan2 = reinterpret_cast<const float2*>(ws + p->off_tan2);
  switch (p->rank) {
    case 2: rank_launch<2>(p, pp, tan2, khat, perm_m1, s); break;
    case 3: rank_launch<3>(p, pp, tan2, khat, perm_m1, s); break;
    case 4: rank_launch<4>(p, pp, tan2, khat, perm_m1, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace s4
