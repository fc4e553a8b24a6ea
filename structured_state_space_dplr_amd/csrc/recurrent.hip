// The recurrent view of the same layer ("The S4 kernel, from scratch",
// section 5; "Structured state-space sequence model and S4", "One linear
// layer, two computational views"):
//   x_t = A-bar x_{t-1} + B-bar u_t,   y_t = Re(C x_t) + D u_t,
// with the bilinear A-bar = (I - s A)^{-1} (I + s A), B-bar = (I - s A)^{-1} dt B,
// s = dt/2 (section 3), and A = Lambda - P Q^* ("S4" wiki, "Structured
// Transition Matrix").
//
// O(N) per step through the rank-1 structure.  With D0 = I - s Lambda
// (diagonal), I - s A = D0 + s P Q^*, and the Sherman-Morrison identity gives
//   (I - s A)^{-1} = D0^{-1} - s D0^{-1} P Q^* D0^{-1} / (1 + s Q^* D0^{-1} P).
// Per pole n, once per parameter set:
//   Abar0_n = (1 + s Lambda_n) / (1 - s Lambda_n),  e_n = s P_n / (1 - s Lambda_n),
//   Bbar0_n = dt B_n / (1 - s Lambda_n),            g_n = e_n / den,
//   den = 1 + s sum_n conj(Q_n) P_n / (1 - s Lambda_n),
//   qa_n = conj(Q_n) Abar0_n,  S1 = sum_n conj(Q_n) e_n,  S2 = sum_n conj(Q_n) Bbar0_n.
// One step, with qx = Q^* x and r2 = sum_n qa_n x_n carried over from the
// previous step's sums:
//   qw = r2 - S1 qx + S2 u   (= Q^* w),
//   w_n = Abar0_n x_n - e_n qx + Bbar0_n u,   x'_n = w_n - g_n qw,
// and one set of sums gives y = Re(sum_n C_n x'_n) + D u and the next qx, r2.
// With the diagonal flag (P = Q = 0; "S4" wiki, "S4D") the step is
// x'_n = Abar0_n x_n + Bbar0_n u.
//
// Work split: each (batch, channel) sequence is scanned by a group of G
// lanes (G a power of two, 1..32), each lane holding PPL poles
// (n = j + G k for lane j of the group) with their parameters in registers.
// The per-step sums over the group are DPP butterflies (xor 1, 2, then the
// half-row and row mirrors, then a cross-row swap for G = 32), so every lane
// of a group ends with the same, bit-identical sum.
#include <hip/hip_runtime.h>

#include "device_fft.h"
#include "internal.h"

namespace s4 {

// Per-pole record (4 float4): (Abar0, e), (Bbar0, g), (qa, conj Q), (C, 0).
constexpr int kRecurRec = 4;

namespace {

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

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the aligned group of 2^LOG2G lanes; every lane of the group gets
// the same value.
template <int LOG2G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LOG2G >= 1) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LOG2G >= 2) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LOG2G >= 3) v += dpp<0x141>(v);   // row_half_mirror: other quad of 8
  if constexpr (LOG2G >= 4) v += dpp<0x140>(v);   // row_mirror: other half of 16
  if constexpr (LOG2G >= 5) v += __shfl_xor(v, 16);
  return v;
}

// The lane's share of the sums conj(Q)^T x (a0 + i a1) and qa^T x (a2 + i a3)
// over its poles, as fused multiply-adds.
template <int PPL>
__device__ __forceinline__ void partial_sums(const float2 (&qc)[PPL], const float2 (&qa)[PPL],
                                             const float2 (&x)[PPL], float& a0, float& a1,
                                             float& a2, float& a3) {
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    a0 = fmaf(-qc[k].y, x[k].y, fmaf(qc[k].x, x[k].x, a0));
    a1 = fmaf(qc[k].y, x[k].x, fmaf(qc[k].x, x[k].y, a1));
    a2 = fmaf(-qa[k].y, x[k].y, fmaf(qa[k].x, x[k].x, a2));
    a3 = fmaf(qa[k].y, x[k].x, fmaf(qa[k].x, x[k].y, a3));
  }
}

}  // namespace

// One wave per channel; the records are formed in fp64 and rounded once.
__global__ __launch_bounds__(64) void recurrent_prepare_kernel(
    const float2* __restrict__ lam, const float2* __restrict__ P, const float2* __restrict__ Q,
    const float2* __restrict__ B, const float2* __restrict__ C, const float* __restrict__ dt,
    float4* __restrict__ rec, float4* __restrict__ chan, int N, int diag, int zoh) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const double d = (double)dt[h], s = 0.5 * d;
  double den_re = 0.0, den_im = 0.0;
  if (!diag) {
    for (int n = lane; n < N; n += 64) {
      const size_t i = (size_t)h * N + n;
      const cd l = cd_load(lam, i), p = cd_load(P, i), q = cd_load(Q ? Q : P, i);
      const cd t = cd_div(cd_mul({q.re, -q.im}, p), {1.0 - s * l.re, -s * l.im});
      den_re += t.re;
      den_im += t.im;
    }
    den_re = wave_sum_d(den_re);
    den_im = wave_sum_d(den_im);
  }
  const cd den = {1.0 + s * den_re, s * den_im};
  double s1r = 0.0, s1i = 0.0, s2r = 0.0, s2i = 0.0;
  for (int n = lane; n < N; n += 64) {
    const size_t i = (size_t)h * N + n;
    const cd l = cd_load(lam, i), b = cd_load(B, i), c = cd_load(C, i);
    const cd p = diag ? cd{0.0, 0.0} : cd_load(P, i);
    const cd q = diag ? cd{0.0, 0.0} : cd_load(Q ? Q : P, i);
    const cd d0 = {1.0 - s * l.re, -s * l.im};
    cd ab = cd_div({1.0 + s * l.re, s * l.im}, d0);
    const cd e = cd_div({s * p.re, s * p.im}, d0);
    cd bb = cd_div({d * b.re, d * b.im}, d0);
    if (zoh) {
      // zero-order hold (diagonal): A-bar = exp(dt lambda), B-bar = b expm1(dt lambda) / lambda
      const double ex = exp(d * l.re);
      double sn, cs;
      sincos(d * l.im, &sn, &cs);
      ab = {ex * cs, ex * sn};
      if (l.re == 0.0 && l.im == 0.0) {
        bb = {d * b.re, d * b.im};
      } else {
        const double sh = sin(0.5 * d * l.im);
        bb = cd_mul(b, cd_div({expm1(d * l.re) * cs - 2.0 * sh * sh, ex * sn}, l));
      }
    }
    const cd g = cd_div(e, den);
    const cd qc = {q.re, -q.im};
    const cd qa = cd_mul(qc, ab);
    const cd t1 = cd_mul(qc, e), t2 = cd_mul(qc, bb);
    s1r += t1.re;
    s1i += t1.im;
    s2r += t2.re;
    s2i += t2.im;
    float4* r = rec + kRecurRec * i;
    r[0] = make_float4((float)ab.re, (float)ab.im, (float)e.re, (float)e.im);
    r[1] = make_float4((float)bb.re, (float)bb.im, (float)g.re, (float)g.im);
    r[2] = make_float4((float)qa.re, (float)qa.im, (float)qc.re, (float)qc.im);
    r[3] = make_float4((float)c.re, (float)c.im, 0.f, 0.f);
  }
  s1r = wave_sum_d(s1r);
  s1i = wave_sum_d(s1i);
  s2r = wave_sum_d(s2r);
  s2i = wave_sum_d(s2i);
  if (lane == 0) chan[h] = make_float4((float)s1r, (float)s1i, (float)s2r, (float)s2i);
}

// Memory row = b * H + h; the group of 2^LOG2G lanes handles one row.
// u and y are moved 16 steps at a time: lane j of a group holds the steps
// t0 + j + G m, and each step's input is broadcast to the group.
//
// Chunked form (mode != kScanWhole): the sequence of memory row r is cut into
// nc chunks of C steps (the last may be shorter); a launch takes the chunks
// [c0, c0 + ncl) of every row, group v = r ncl + (c - c0).  kScanLocal starts
// each chunk from a zero state, writes its zero-state output and leaves the
// chunk's final state in cst[r nc + c]; kScanCarried starts from that entry
// (the true state before the chunk), writes y, and the last chunk leaves the
// final state in `state`.
constexpr int kScanWhole = 0, kScanLocal = 1, kScanCarried = 2;

template <int PPL, int LOG2G, bool DIAG>
__global__ __launch_bounds__(256) void recurrent_scan_kernel(
    const float4* __restrict__ rec, const float4* __restrict__ chan, const float* __restrict__ D,
    const float* __restrict__ u, float2* __restrict__ state, float* __restrict__ y, int H,
    int vrows, int N, int T, int C, int nc, int c0, int ncl, int mode,
    float2* __restrict__ cst) {
  constexpr int G = 1 << LOG2G;
  constexpr int CH = 16;
  constexpr int NU = G >= CH ? 1 : CH / G;
  const int lane = threadIdx.x & 63;
  const int j = lane & (G - 1);
  const int gbase = lane - j;
  const long grow = ((long)blockIdx.x * 256 + threadIdx.x) >> LOG2G;
  const bool valid = grow < vrows;  // the whole group agrees
  const int v = valid ? (int)grow : 0;
  const int row = v / ncl, ck = c0 + (v - row * ncl);   // memory row, chunk
  const size_t cv = (size_t)row * nc + ck;               // its chunk-state entry (64 wide)
  const int h = row % H;
  const int tb = ck * C;                       // first step of the chunk
  const int len = min(C, T - tb);              // steps of the chunk

  float2 ab[PPL], e[PPL], bb[PPL], g[PPL], qa[PPL], qc[PPL], c[PPL], x[PPL];
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int n = j + G * k;
    ab[k] = e[k] = bb[k] = g[k] = qa[k] = qc[k] = c[k] = x[k] = make_float2(0.f, 0.f);
    if (valid && n < N) {
      const float4* r = rec + kRecurRec * ((size_t)h * N + n);
      const float4 r0 = r[0], r1 = r[1], r2v = r[2], r3 = r[3];
      ab[k] = make_float2(r0.x, r0.y);
      e[k] = make_float2(r0.z, r0.w);
      bb[k] = make_float2(r1.x, r1.y);
      g[k] = make_float2(r1.z, r1.w);
      qa[k] = make_float2(r2v.x, r2v.y);
      qc[k] = make_float2(r2v.z, r2v.w);
      c[k] = make_float2(r3.x, r3.y);
      if (mode == kScanWhole) x[k] = state[(size_t)row * N + n];
      else if (mode == kScanCarried) x[k] = cst[cv * 64 + n];
    }
  }
  float2 S1 = make_float2(0.f, 0.f), S2 = make_float2(0.f, 0.f);
  float Dh = 0.f;
  if (valid) {
    const float4 ch = chan[h];
    S1 = make_float2(ch.x, ch.y);
    S2 = make_float2(ch.z, ch.w);
    Dh = D ? D[h] : 0.f;
  }

  float2 qx = make_float2(0.f, 0.f), r2 = make_float2(0.f, 0.f);
  if constexpr (!DIAG) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    partial_sums<PPL>(qc, qa, x, a0, a1, a2, a3);
    qx = make_float2(group_sum<LOG2G>(a0), group_sum<LOG2G>(a1));
    r2 = make_float2(group_sum<LOG2G>(a2), group_sum<LOG2G>(a3));
  }

  const float* __restrict__ ur = u + (size_t)row * T + tb;
  float* __restrict__ yr = y + (size_t)row * T + tb;
  for (int t0 = 0; t0 < len; t0 += CH) {
    float uv[NU], yv[NU];
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int o = j + G * m, t = t0 + o;
      uv[m] = (valid && o < CH && t < len) ? ur[t] : 0.f;
      yv[m] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      if (t0 + i >= len) continue;   // the same for every lane
      float ut;
      if constexpr (G == 1) ut = uv[i];
      else ut = __shfl(uv[i / G], gbase + (i % G));
      float yre = 0.f;
      if constexpr (DIAG) {
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const float2 ax = cmul(ab[k], x[k]);
          x[k] = make_float2(fmaf(bb[k].x, ut, ax.x), fmaf(bb[k].y, ut, ax.y));
          yre = fmaf(c[k].x, x[k].x, fmaf(-c[k].y, x[k].y, yre));
        }
      } else {
        const float2 qw = make_float2(fmaf(S2.x, ut, r2.x - fmaf(S1.x, qx.x, -S1.y * qx.y)),
                                      fmaf(S2.y, ut, r2.y - fmaf(S1.x, qx.y, S1.y * qx.x)));
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          // x' = Abar0 x - e qx + Bbar0 u - g qw, one chain of fmas per part
          const float2 xo = x[k];
          float re = bb[k].x * ut, im = bb[k].y * ut;
          re = fmaf(-ab[k].y, xo.y, fmaf(ab[k].x, xo.x, re));
          im = fmaf(ab[k].y, xo.x, fmaf(ab[k].x, xo.y, im));
          re = fmaf(e[k].y, qx.y, fmaf(-e[k].x, qx.x, re));
          im = fmaf(-e[k].y, qx.x, fmaf(-e[k].x, qx.y, im));
          re = fmaf(g[k].y, qw.y, fmaf(-g[k].x, qw.x, re));
          im = fmaf(-g[k].y, qw.x, fmaf(-g[k].x, qw.y, im));
          x[k] = make_float2(re, im);
          yre = fmaf(-c[k].y, im, fmaf(c[k].x, re, yre));
        }
        partial_sums<PPL>(qc, qa, x, a0, a1, a2, a3);
        qx = make_float2(group_sum<LOG2G>(a0), group_sum<LOG2G>(a1));
        r2 = make_float2(group_sum<LOG2G>(a2), group_sum<LOG2G>(a3));
      }
      const float yt = fmaf(Dh, ut, group_sum<LOG2G>(yre));
      if (j == (i % G)) yv[i / G] = yt;
    }
#pragma unroll
    for (int m = 0; m < NU; ++m) {
      const int o = j + G * m, t = t0 + o;
      if (valid && o < CH && t < len) yr[t] = yv[m];
    }
  }
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int n = j + G * k;
    if (!valid || n >= N) continue;
    if (mode == kScanLocal) cst[cv * 64 + n] = x[k];
    else if (mode == kScanWhole || ck == nc - 1) state[(size_t)row * N + n] = x[k];
  }
}

// A-bar^C of channel h (C = 2^log2C), zero-padded to 64 x 64: A-bar from the
// per-pole quantities of the step above, column j being the step applied to
// the unit vector e_j,
//   A-bar[i][j] = Abar0_j delta_ij - e_i conj(Q_j) - g_i conj(Q_j) (Abar0_j - S1),
// then log2C squarings, all in fp64 in LDS, rounded once.  N <= 64.
constexpr int kPowDim = 64;

__global__ __launch_bounds__(256) void recurrent_power_kernel(
    const float2* __restrict__ lam, const float2* __restrict__ P, const float2* __restrict__ Q,
    const float* __restrict__ dt, float2* __restrict__ pw, int N, int diag, int zoh,
    int log2C) {
  constexpr int D = kPowDim;
  __shared__ cd m0[D * D], m1[D * D];
  __shared__ cd pab[D], pe[D], pg[D], pqc[D];
  __shared__ cd s1s;
  const int h = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    const int n = tid;
    const double d = (double)dt[h], s = 0.5 * d;
    cd l = {0.0, 0.0}, p = {0.0, 0.0}, q = {0.0, 0.0};
    if (n < N) {
      const size_t i = (size_t)h * N + n;
      l = cd_load(lam, i);
      if (!diag) {
        p = cd_load(P, i);
        q = cd_load(Q ? Q : P, i);
      }
    }
    const cd d0 = {1.0 - s * l.re, -s * l.im};
    cd t = {0.0, 0.0};
    if (n < N && !diag) t = cd_div(cd_mul({q.re, -q.im}, p), d0);
    const cd den = {1.0 + s * wave_sum_d(t.re), s * wave_sum_d(t.im)};
    cd ab = {0.0, 0.0}, e = {0.0, 0.0}, g = {0.0, 0.0};
    const cd qc = {q.re, -q.im};
    if (n < N) {
      ab = cd_div({1.0 + s * l.re, s * l.im}, d0);
      if (zoh) {
        const double ex = exp(d * l.re);
        double sn, cs;
        sincos(d * l.im, &sn, &cs);
        ab = {ex * cs, ex * sn};
      }
      e = cd_div({s * p.re, s * p.im}, d0);
      g = cd_div(e, den);
    }
    const cd qe = cd_mul(qc, e);
    const cd s1 = {wave_sum_d(qe.re), wave_sum_d(qe.im)};
    pab[n] = ab;
    pe[n] = e;
    pg[n] = g;
    pqc[n] = qc;
    if (n == 0) s1s = s1;
  }
  __syncthreads();
  for (int idx = tid; idx < D * D; idx += 256) {
    const int i = idx / D, jj = idx % D;
    cd v = {0.0, 0.0};
    if (i < N && jj < N) {
      const cd a = pab[jj], qj = pqc[jj];
      const cd w = cd_mul(qj, {a.re - s1s.re, a.im - s1s.im});
      const cd t1 = cd_mul(pe[i], qj), t2 = cd_mul(pg[i], w);
      v = {(i == jj ? a.re : 0.0) - t1.re - t2.re, (i == jj ? a.im : 0.0) - t1.im - t2.im};
    }
    m0[idx] = v;
  }
  __syncthreads();
  // squarings: thread tid forms the 4 x 4 block at rows 4 (tid / 16), columns 4 (tid % 16)
  cd* src = m0;
  cd* dst = m1;
  const int i0 = 4 * (tid >> 4), j0 = 4 * (tid & 15);
  for (int sq = 0; sq < log2C; ++sq) {
    cd acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = {0.0, 0.0};
    for (int k = 0; k < D; ++k) {
      cd ra[4], rb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) ra[a] = src[(i0 + a) * D + k];
#pragma unroll
      for (int b = 0; b < 4; ++b) rb[b] = src[k * D + j0 + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[a][b].re = fma(ra[a].re, rb[b].re, fma(-ra[a].im, rb[b].im, acc[a][b].re));
          acc[a][b].im = fma(ra[a].re, rb[b].im, fma(ra[a].im, rb[b].re, acc[a][b].im));
        }
    }
    __syncthreads();                             // every read of src is done
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) dst[(i0 + a) * D + j0 + b] = acc[a][b];
    __syncthreads();
    cd* t = src;
    src = dst;
    dst = t;
  }
  float2* out = pw + (size_t)h * D * D;
  for (int idx = tid; idx < D * D; idx += 256)
    out[idx] = make_float2((float)src[idx].re, (float)src[idx].im);
}

// The chunk carries of memory row `row` (one wave): starting from the state
// passed in, s_0 = state, s_{c+1} = A-bar^C s_c + f_c, where f_c (in cst,
// from the zero-state scan of chunk c) is replaced by s_c.  With `full` (the
// last chunk has C steps too) the final state s_nc is written to `state`.
// Lane i holds row i of A-bar^C; s_j reaches every lane as a scalar.  Chunk
// states are 64 entries wide, zero beyond N after this kernel.
__global__ __launch_bounds__(64) void recurrent_carry_kernel(const float2* __restrict__ pw,
                                                             float2* __restrict__ state,
                                                             float2* __restrict__ cst, int H,
                                                             int N, int nc, int full) {
  constexpr int D = kPowDim;
  const int row = blockIdx.x, lane = threadIdx.x, h = row % H;
  const bool on = lane < N;
  float2 m[D];
  const float2* mr = pw + ((size_t)h * D + lane) * D;
#pragma unroll
  for (int jj = 0; jj < D; ++jj) m[jj] = mr[jj];
  float2 sv = on ? state[(size_t)row * N + lane] : make_float2(0.f, 0.f);
  float2* cr = cst + (size_t)row * nc * D;
  for (int c = 0; c < nc; ++c) {
    const float2 f = on ? cr[(size_t)c * D + lane] : make_float2(0.f, 0.f);
    cr[(size_t)c * D + lane] = sv;
    if (c == nc - 1 && !full) break;
    float re = f.x, im = f.y;
#pragma unroll
    for (int jj = 0; jj < D; ++jj) {
      const float sr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv.x), jj));
      const float si = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv.y), jj));
      re = fmaf(m[jj].x, sr, fmaf(-m[jj].y, si, re));
      im = fmaf(m[jj].x, si, fmaf(m[jj].y, sr, im));
    }
    sv = make_float2(re, im);
  }
  if (full && on) state[(size_t)row * N + lane] = sv;
}

// c_tau = C A-bar^(tau + 1), tau < C, of channel h (one wave, lane n holds
// entry n), for the outputs' dependence on the state s before a chunk (the
// chunk's first step already multiplies s by A-bar):
// y_{t0 + tau} = (zero-state output) + Re(c_tau . s).  The transposed step,
// with A-bar = (I - g conj(Q)^T)(diag(Abar0) - e conj(Q)^T), is
//   c1 = c - (c . g) conj(Q)^T,   c' = c1 o Abar0 - (c1 . e) conj(Q)^T,
// in fp64, each row rounded once.  ct: [H][C][N] float2.
__global__ __launch_bounds__(64) void recurrent_ctab_kernel(
    const float2* __restrict__ lam, const float2* __restrict__ P, const float2* __restrict__ Q,
    const float2* __restrict__ Cp, const float* __restrict__ dt, float2* __restrict__ ct, int N,
    int diag, int zoh, int C) {
  const int h = blockIdx.x, n = threadIdx.x;
  const bool on = n < N;
  const double d = (double)dt[h], s = 0.5 * d;
  cd l = {0.0, 0.0}, p = {0.0, 0.0}, q = {0.0, 0.0}, c = {0.0, 0.0};
  if (on) {
    const size_t i = (size_t)h * N + n;
    l = cd_load(lam, i);
    c = cd_load(Cp, i);
    if (!diag) {
      p = cd_load(P, i);
      q = cd_load(Q ? Q : P, i);
    }
  }
  const cd d0 = {1.0 - s * l.re, -s * l.im};
  cd t = {0.0, 0.0};
  if (on && !diag) t = cd_div(cd_mul({q.re, -q.im}, p), d0);
  const cd den = {1.0 + s * wave_sum_d(t.re), s * wave_sum_d(t.im)};
  cd ab = {0.0, 0.0}, e = {0.0, 0.0}, g = {0.0, 0.0};
  const cd qc = {q.re, -q.im};
  if (on) {
    ab = cd_div({1.0 + s * l.re, s * l.im}, d0);
    if (zoh) {
      const double ex = exp(d * l.re);
      double sn, cs;
      sincos(d * l.im, &sn, &cs);
      ab = {ex * cs, ex * sn};
    }
    e = cd_div({s * p.re, s * p.im}, d0);
    g = cd_div(e, den);
  }
  float2* out = ct + (size_t)h * C * N;
  for (int tau = 0; tau < C; ++tau) {
    const cd cg = cd_mul(c, g);
    const cd sg = {wave_sum_d(cg.re), wave_sum_d(cg.im)};
    const cd t1 = cd_mul(sg, qc);
    const cd c1 = {c.re - t1.re, c.im - t1.im};
    const cd ce = cd_mul(c1, e);
    const cd se = {wave_sum_d(ce.re), wave_sum_d(ce.im)};
    const cd a1 = cd_mul(c1, ab), t2 = cd_mul(se, qc);
    c = {a1.re - t2.re, a1.im - t2.im};
    if (on) out[(size_t)tau * N + n] = make_float2((float)c.re, (float)c.im);
  }
}

// y[b][h][c C + tau] += Re(c_tau . s_{b,c}) for the chunks c < nfull, as a
// matrix product on the fp32 matrix cores per channel:
// y[m][tau] += sum_k A[m][k] Bt[k][tau] over the rows m = (b, c),
// c < nfull, with k = 2n + p interleaving the parts,
//   A[m][2n] = Re s_{b,c}[n],  A[m][2n+1] = -Im s_{b,c}[n],
//   Bt[2n][tau] = Re c_tau[n], Bt[2n+1][tau] = Im c_tau[n].
// Block (32 steps tau, 128 rows m, channel h): the 128 x 32 tile of Bt in
// LDS, wave w the rows [32 w, 32 w + 32) of the group, one 32 x 32 tile of
// v_mfma_f32_32x32x2_f32 products (lane l feeds A[l % 32][k0 + l / 32] and
// Bt[k0 + l / 32][l % 32]; accumulator register r holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32).
typedef float v16f_r __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void recurrent_correct_mfma_kernel(
    const float2* __restrict__ ct, const float2* __restrict__ cst, float* __restrict__ y, int H,
    int batch, int N, int T, int C, int nc, int nfull) {
  constexpr int D = kPowDim;
  __shared__ float sb[2 * D][32];
  const int h = blockIdx.z, tau0 = blockIdx.x * 32, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int M = batch * nfull;
  // Bt tile: k in [0, 128), tau in [tau0, tau0 + 32)
  for (int idx = tid; idx < 2 * D * 32; idx += 256) {
    const int kk = idx >> 5, tt = idx & 31, n = kk >> 1, tau = tau0 + tt;
    float v = 0.f;
    if (n < N && tau < C) {
      const float2 c = ct[((size_t)h * C + tau) * N + n];
      v = (kk & 1) ? c.y : c.x;
    }
    sb[kk][tt] = v;
  }
  // A rows of this wave: m = m0 + lane % 32
  const int m0 = (blockIdx.y * 4 + w) * 32;
  const int m = m0 + (lane & 31), part = lane >> 5;
  const bool mon = m < M;
  const int bm = mon ? m / nfull : 0, cm = mon ? m - bm * nfull : 0;
  const float* sr = reinterpret_cast<const float*>(cst + (((size_t)bm * H + h) * nc + cm) * D);
  float av[D];
#pragma unroll
  for (int n = 0; n < D; ++n) {
    const float v = mon ? sr[2 * n + part] : 0.f;
    av[n] = part ? -v : v;
  }
  __syncthreads();
  v16f_r acc = {};
#pragma unroll
  for (int n = 0; n < D; ++n)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[n], sb[2 * n + part][lane & 31], acc, 0, 0, 0);
  const int tau = tau0 + (lane & 31);
  if (tau >= C) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int mr = m0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (mr >= M) continue;
    const int b = mr / nfull, c = mr - b * nfull;
    y[((size_t)b * H + h) * T + (size_t)c * C + tau] += acc[r];
  }
}


hipError_t launch_recurrent_prepare(const s4dplr_plan* p, const float* lam, const float* P,
                                    const float* Q, const float* B, const float* C,
                                    const float* dt, unsigned char* ws, hipStream_t s) {
  const int diag = (p->flags & S4DPLR_DIAGONAL) ? 1 : 0;
  const int zoh = (p->flags & S4DPLR_ZOH) ? 1 : 0;
  recurrent_prepare_kernel<<<p->H, 64, 0, s>>>(
      reinterpret_cast<const float2*>(lam), reinterpret_cast<const float2*>(P),
      reinterpret_cast<const float2*>(Q), reinterpret_cast<const float2*>(B),
      reinterpret_cast<const float2*>(C), dt, reinterpret_cast<float4*>(ws + p->off_rrec),
      reinterpret_cast<float4*>(ws + p->off_rchan), p->N, diag, zoh);
  if (p->rchunk > 0) {
    int log2C = 0;
    while ((1 << log2C) < p->rchunk) ++log2C;
    recurrent_power_kernel<<<p->H, 256, 0, s>>>(
        reinterpret_cast<const float2*>(lam), reinterpret_cast<const float2*>(P),
        reinterpret_cast<const float2*>(Q), dt, reinterpret_cast<float2*>(ws + p->off_rpow), p->N,
        diag, zoh, log2C);
    recurrent_ctab_kernel<<<p->H, 64, 0, s>>>(
        reinterpret_cast<const float2*>(lam), reinterpret_cast<const float2*>(P),
        reinterpret_cast<const float2*>(Q), reinterpret_cast<const float2*>(C), dt,
        reinterpret_cast<float2*>(ws + p->off_rct), p->N, diag, zoh, p->rchunk);
  }
  return hipGetLastError();
}

namespace {

// One launch of the scan kernel over vrows = rows * ncl groups (chunks
// [c0, c0 + ncl) of the nc chunks of every row).
struct ScanArgs {
  const float* D;
  const float* u;
  float* state;
  float* y;
  int T, C, nc, c0, ncl, mode;
  float2* cst;
};

template <int PPL, int LOG2G>
void scan_launch(const s4dplr_plan* p, const ScanArgs& a, unsigned char* ws, hipStream_t s) {
  const int vrows = p->batch * p->H * a.ncl;
  const float4* rec = reinterpret_cast<const float4*>(ws + p->off_rrec);
  const float4* chan = reinterpret_cast<const float4*>(ws + p->off_rchan);
  float2* st = reinterpret_cast<float2*>(a.state);
  const long threads = (long)vrows << LOG2G;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (p->flags & S4DPLR_DIAGONAL)
    recurrent_scan_kernel<PPL, LOG2G, true><<<blocks, 256, 0, s>>>(
        rec, chan, a.D, a.u, st, a.y, p->H, vrows, p->N, a.T, a.C, a.nc, a.c0, a.ncl, a.mode,
        a.cst);
  else
    recurrent_scan_kernel<PPL, LOG2G, false><<<blocks, 256, 0, s>>>(
        rec, chan, a.D, a.u, st, a.y, p->H, vrows, p->N, a.T, a.C, a.nc, a.c0, a.ncl, a.mode,
        a.cst);
}

template <int PPL>
bool scan_dispatch_g(int lg, const s4dplr_plan* p, const ScanArgs& a, unsigned char* ws,
                     hipStream_t s) {
  switch (lg) {
    case 0: scan_launch<PPL, 0>(p, a, ws, s); return true;
    case 1: scan_launch<PPL, 1>(p, a, ws, s); return true;
    case 2: scan_launch<PPL, 2>(p, a, ws, s); return true;
    case 3: scan_launch<PPL, 3>(p, a, ws, s); return true;
    case 4: scan_launch<PPL, 4>(p, a, ws, s); return true;
    case 5: scan_launch<PPL, 5>(p, a, ws, s); return true;
    default: return false;
  }
}

bool scan_dispatch(const s4dplr_plan* p, const ScanArgs& a, unsigned char* ws, hipStream_t s) {
  int ppl, lg;
  recurrent_shape(p->N, (long)p->batch * p->H * a.ncl, &ppl, &lg);
  switch (ppl) {
    case 1: return scan_dispatch_g<1>(lg, p, a, ws, s);
    case 2: return scan_dispatch_g<2>(lg, p, a, ws, s);
    case 4: return scan_dispatch_g<4>(lg, p, a, ws, s);
    case 8: return scan_dispatch_g<8>(lg, p, a, ws, s);
    default: return false;
  }
}

}  // namespace

// Sequences alone give few lanes when batch * H is small, and each lane then
// walks all T steps in order.  With the plan's chunk length C (N <= 64, few
// sequences) a scan of at least two chunks runs as three or four launches,
// the same linear recurrence:
//   1. every chunk from a zero state: its zero-state output and final state f_c;
//   2. the carries s_{c+1} = A-bar^C s_c + f_c of every row (s_0 = state);
//   3. y += Re(c_tau . s_c) on every full chunk (c_tau = C A-bar^(tau+1));
//   4. a shorter last chunk again from its carry, writing y and the final
//      state (with a full last chunk the carries give the final state).
hipError_t launch_recurrent_scan(const s4dplr_plan* p, const float* D, const float* u,
                                 float* state, float* y, int T, unsigned char* ws,
                                 hipStream_t s) {
  const int C = p->rchunk;
  const int nc = C > 0 ? (T + C - 1) / C : 1;
  if (C > 0 && nc >= 2 && nc <= p->rnc) {
    float2* cst = reinterpret_cast<float2*>(ws + p->off_rcs);
    const ScanArgs local{D, u, state, y, T, C, nc, 0, nc, kScanLocal, cst};
    if (!scan_dispatch(p, local, ws, s)) return hipErrorInvalidValue;
    const int full = T % C == 0;
    recurrent_carry_kernel<<<p->batch * p->H, 64, 0, s>>>(
        reinterpret_cast<const float2*>(ws + p->off_rpow), reinterpret_cast<float2*>(state), cst,
        p->H, p->N, nc, full);
    const int nfull = full ? nc : nc - 1;
    const int mrows = p->batch * nfull;
    recurrent_correct_mfma_kernel<<<dim3((C + 31) / 32, (mrows + 127) / 128, p->H), 256, 0, s>>>(
        reinterpret_cast<const float2*>(ws + p->off_rct), cst, y, p->H, p->batch, p->N, T, C, nc,
        nfull);
    if (!full) {   // a shorter last chunk: scanned again from its carry
      const ScanArgs last{D, u, state, y, T, C, nc, nc - 1, 1, kScanCarried, cst};
      if (!scan_dispatch(p, last, ws, s)) return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const ScanArgs whole{D, u, state, y, T, T, 1, 0, 1, kScanWhole, nullptr};
  if (!scan_dispatch(p, whole, ws, s)) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace s4
