// Long sequences (L = 32768, 65536): the row no longer fits in LDS, so the
// transforms of M = L complex points are split four-step, M = M1 x M2 with
// M2 = 256 ("The S4 kernel, from scratch", section 5: the convolution is
// applied by FFT, zero-padded to 2L; the split only changes the order of the
// same DFT sums).
//
// Index maps: time n = M2 n1 + n2, frequency k = k1 + M1 k2.
//   forward: column DFTs over n1 (-> k1), twiddle W_M^{n2 k1}, row DFTs over
//            n2 (-> k2); the spectrum is stored row-major by k1, i.e. bin
//            k1 + M1 k2 sits at position k1 M2 + k2 ("permuted" layout).
//   inverse: row DFTs over k2 (-> n2), twiddle W_M^{-n2 k1}, column DFTs over
//            k1 (-> n1).
// Bin k pairs with M - k (the real-FFT pairing): rows k1 and M1 - k1, with
// k2 -> M2-1-k2, except row 0, which pairs with itself through k2 -> -k2.
#include <hip/hip_runtime.h>

#include "device_fft.h"
#include "internal.h"

namespace s4 {

constexpr int kBigThreads = 256;

template <int LOG2M>
struct BigShape {
  static constexpr int M = 1 << LOG2M;
  static constexpr int LOG2M2 = 8, M2 = 256;
  static constexpr int LOG2M1 = LOG2M - 8, M1 = M / 256;
  static constexpr int CT = kBigThreads / (M1 / 16);   // columns per block (16 threads each)
  static constexpr int CP = lds_padded_size(M1);        // padded column length
  static constexpr int RP = lds_padded_size(M2);        // padded row length
  static constexpr int RT = kBigThreads / (M2 / 16);   // rows per block (16)
  static_assert(LOG2M >= 15 && LOG2M <= 16, "four-step range");
};

// The four-step twiddles W_M^m (m = n2 k1 < M) from two 256-entry tables
// held in LDS: W_M^m = W_M^{256 (m >> 8)} * W_M^{m & 255}.  tw4 in the
// workspace holds [lo: W_M^b, b < 256][hi: W_M^{256 a}, a < 256].
struct TwM {
  float2 lo[256];
  float2 hi[256];
};
__device__ __forceinline__ void load_twM(TwM& t, const float2* __restrict__ tw4, int tid,
                                         int nthr) {
  for (int i = tid; i < 512; i += nthr) (i < 256 ? t.lo[i] : t.hi[i - 256]) = tw4[i];
}
__device__ __forceinline__ float2 w_M(const TwM& t, int m) {
  return cmul(t.hi[m >> 8], t.lo[m & 255]);
}

// (1 -+ i W_{2M}^j)/2 applied to the pair (Z_j, Z_{M-j}): the bin X_j of the
// real transform of length 2M; csj = (cos, sin)(pi j / M).
__device__ __forceinline__ float2 big_rfft_x(float2 zj, float2 zmj, float2 csj) {
  const float2 p = make_float2(0.5f * (1.0f - csj.y), -0.5f * csj.x);
  const float2 q = make_float2(0.5f * (1.0f + csj.y), 0.5f * csj.x);
  return cadd(cmul(p, zj), cmul(q, cconj(zmj)));
}

// ---------------------------------------------------------------------------
// Forward column step on real rows x (L floats, packed z_k = x_2k + i x_2k+1,
// z zero for k >= M/2): Y[row][k1][n2] = W_M^{n2 k1} sum_{n1} z[M2 n1 + n2] W_M1^{n1 k1}
// ---------------------------------------------------------------------------
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_cols_fwd_kernel(
    const float* __restrict__ x, float2* __restrict__ Y, const float2* __restrict__ tw1,
    const float2* __restrict__ tw4) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, CT = S::CT, CP = S::CP;
  __shared__ float2 lds[CT * CP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, row = blockIdx.y, c0 = blockIdx.x * CT;
  load_twM(twm, tw4, tid, kBigThreads);
  const float2* __restrict__ z = reinterpret_cast<const float2*>(x + (size_t)row * M);
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int n1 = idx / CT, c = idx % CT;
    lds[c * CP + lds_pad(n1)] = (n1 < M1 / 2) ? z[M2 * n1 + c0 + c] : make_float2(0.f, 0.f);
  }
  __syncthreads();
  lds_fft<S::LOG2M1, false>(lds + (tid / (M1 / 16)) * CP, tid % (M1 / 16), true, tw1);
  float2* __restrict__ Yr = Y + (size_t)row * M;
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int k1 = idx / CT, c = idx % CT, n2 = c0 + c;
    Yr[k1 * M2 + n2] = cmul(lds[c * CP + lds_pad(k1)], w_M(twm, n2 * k1));
  }
}

// ---------------------------------------------------------------------------
// Inverse column step: x[M2 n1 + n2] = sum_{k1} Y[k1][n2] W_M1^{-n1 k1}.
// MODE 0: outputs n < M/2 as (y_2n, y_2n+1) (the kept half of the causal
// convolution).  MODE 1: all n, real part times `scale` (time-domain kernel).
// ---------------------------------------------------------------------------
template <int LOG2M, int MODE>
__global__ __launch_bounds__(kBigThreads) void big_cols_inv_kernel(
    const float2* __restrict__ Y, float* __restrict__ out, const float2* __restrict__ tw1,
    float scale) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, CT = S::CT, CP = S::CP;
  __shared__ float2 lds[CT * CP];
  const int tid = threadIdx.x, row = blockIdx.y, c0 = blockIdx.x * CT;
  const float2* __restrict__ Yr = Y + (size_t)row * M;
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int k1 = idx / CT, c = idx % CT;
    lds[c * CP + lds_pad(k1)] = Yr[k1 * M2 + c0 + c];
  }
  __syncthreads();
  lds_fft<S::LOG2M1, true>(lds + (tid / (M1 / 16)) * CP, tid % (M1 / 16), true, tw1);
  if constexpr (MODE == 0) {
    float2* __restrict__ yr = reinterpret_cast<float2*>(out + (size_t)row * M);
    for (int idx = tid; idx < (M1 / 2) * CT; idx += kBigThreads) {
      const int n1 = idx / CT, c = idx % CT;
      yr[M2 * n1 + c0 + c] = lds[c * CP + lds_pad(n1)];
    }
  } else {
    float* __restrict__ kr = out + (size_t)row * M;
    for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
      const int n1 = idx / CT, c = idx % CT;
      kr[M2 * n1 + c0 + c] = lds[c * CP + lds_pad(n1)].x * scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Row step of the inverse transform alone (time-domain kernel from the
// generating function, stored in the permuted layout by the Cauchy kernel):
// Y[k1][n2] = W_M^{-n2 k1} sum_{k2} X[k1][k2] W_M2^{-n2 k2}
// ---------------------------------------------------------------------------
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_rows_inv_kernel(
    const float2* __restrict__ X, float2* __restrict__ Y, const float2* __restrict__ tw2,
    const float2* __restrict__ tw4) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M2 = S::M2, RT = S::RT, RP = S::RP;
  __shared__ float2 lds[RT * RP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, row = blockIdx.y, r0 = blockIdx.x * RT;
  load_twM(twm, tw4, tid, kBigThreads);
  const float2* __restrict__ Xr = X + (size_t)row * M;
  for (int idx = tid; idx < RT * M2; idx += kBigThreads) {
    const int s = idx / M2, k2 = idx % M2;
    lds[s * RP + lds_pad(k2)] = Xr[(r0 + s) * M2 + k2];
  }
  __syncthreads();
  lds_fft<S::LOG2M2, true>(lds + (tid / 16) * RP, tid % 16, true, tw2);
  float2* __restrict__ Yr = Y + (size_t)row * M;
  for (int idx = tid; idx < RT * M2; idx += kBigThreads) {
    const int s = idx / M2, n2 = idx % M2, k1 = r0 + s;
    Yr[k1 * M2 + n2] = cmulc(lds[s * RP + lds_pad(n2)], w_M(twm, n2 * k1));
  }
}

// ---------------------------------------------------------------------------
// Paired row steps.  A block takes 8 pair tasks t (rows k1 = t and M1 - t,
// t = 0 .. M1/2) into 16 LDS slots and runs the forward row DFTs.
//   CONV:  spectral weights Z'_k = alpha_k Z_k + beta_k conj(Z_{M-k}), the
//          inverse row DFTs and the inverse twiddle, back into Y.
//   !CONV: the spectrum of (K + D delta) padded to 2L and the weights
//          alpha, beta of every bin, written in the permuted layout.
// ---------------------------------------------------------------------------
template <int LOG2M, bool CONV>
__global__ __launch_bounds__(kBigThreads) void big_rows_pair_kernel(
    float2* __restrict__ Y, float4* __restrict__ coefp, const float* __restrict__ D,
    const float2* __restrict__ tw2, const float2* __restrict__ cs,
    const float2* __restrict__ tw4, int batch, int conj) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, RP = S::RP;
  constexpr int TASKS = 8;
  __shared__ float2 lds[2 * TASKS * RP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, row = blockIdx.y, t0 = blockIdx.x * TASKS;
  if constexpr (CONV) load_twM(twm, tw4, tid, kBigThreads);
  const int h = CONV ? row / batch : row;     // logical rows: h*batch + b
  float2* __restrict__ Yr = Y + (size_t)row * M;
  auto slot_row = [&](int s) -> int {
    const int t = t0 + s / 2;
    return (s & 1) ? ((M1 - t) & (M1 - 1)) : t;
  };
  auto task_valid = [&](int s) -> bool { return t0 + s / 2 <= M1 / 2; };
  for (int idx = tid; idx < 2 * TASKS * M2; idx += kBigThreads) {
    const int s = idx / M2, k = idx % M2;
    lds[s * RP + lds_pad(k)] = task_valid(s) ? Yr[slot_row(s) * M2 + k] : make_float2(0.f, 0.f);
  }
  __syncthreads();
  lds_fft<S::LOG2M2, false>(lds + (tid / 16) * RP, tid % 16, true, tw2);
  // pairs: every item (task i, k2) of slot a = 2i meets (slot b = 2i+1, k2p)
  const float4* __restrict__ cfh = coefp + (size_t)h * M;
  const float sc = 0.5f / (float)M;
  const float Dh = (!CONV && D) ? D[h] : 0.f;
  for (int idx = tid; idx < TASKS * M2; idx += kBigThreads) {
    const int i = idx / M2, k2 = idx % M2, t = t0 + i;
    if (t > M1 / 2) continue;
    const int ka = t, kb = (M1 - t) & (M1 - 1);
    const bool self = (ka == kb);
    const int k2p = (ka == 0) ? ((M2 - k2) & (M2 - 1)) : (M2 - 1 - k2);
    if (self && k2p < k2) continue;
    float2* A = lds + (2 * i) * RP;
    float2* B = self ? A : lds + (2 * i + 1) * RP;
    const float2 za = A[lds_pad(k2)], zb = B[lds_pad(k2p)];
    if constexpr (CONV) {
      const float4 ca = cfh[ka * M2 + k2], cb = cfh[kb * M2 + k2p];
      const float2 oa = cadd(cmul(make_float2(ca.x, ca.y), za), cmul(make_float2(ca.z, ca.w), cconj(zb)));
      const float2 ob = cadd(cmul(make_float2(cb.x, cb.y), zb), cmul(make_float2(cb.z, cb.w), cconj(za)));
      A[lds_pad(k2)] = oa;
      if (!(self && k2p == k2)) B[lds_pad(k2p)] = ob;
    } else {
      const int kk = ka + M1 * k2;          // bin of slot a
      const int km = M - kk;                // its partner, in [1, M]
      const float2 csa = cs[kk], csb = cs[km];
      float2 sa = big_rfft_x(za, zb, csa), sb = big_rfft_x(zb, za, csb);
      sa.x += Dh;
      sb.x += Dh;
      if (conj) {   // weights of the correlation with (K + D delta)
        sa.y = -sa.y;
        sb.y = -sb.y;
      }
      {
        const float a = sc * (1.0f - csa.y), b = sc * (1.0f + csa.y), c = sc * csa.x;
        const float2 al = make_float2(fmaf(a, sa.x, b * sb.x), fmaf(a, sa.y, -b * sb.y));
        const float2 df = make_float2(sa.x - sb.x, sa.y + sb.y);
        coefp[(size_t)h * M + ka * M2 + k2] = make_float4(al.x, al.y, -c * df.y, c * df.x);
      }
      if (km < M && km != kk) {
        const float a = sc * (1.0f - csb.y), b = sc * (1.0f + csb.y), c = sc * csb.x;
        const float2 al = make_float2(fmaf(a, sb.x, b * sa.x), fmaf(a, sb.y, -b * sa.y));
        const float2 df = make_float2(sb.x - sa.x, sb.y + sa.y);
        coefp[(size_t)h * M + kb * M2 + k2p] = make_float4(al.x, al.y, -c * df.y, c * df.x);
      }
    }
  }
  if constexpr (CONV) {
    __syncthreads();
    lds_fft<S::LOG2M2, true>(lds + (tid / 16) * RP, tid % 16, true, tw2);
    for (int idx = tid; idx < 2 * TASKS * M2; idx += kBigThreads) {
      const int s = idx / M2, n2 = idx % M2;
      if (!task_valid(s)) continue;
      const int k1 = slot_row(s);
      if ((s & 1) && k1 == slot_row(s - 1)) continue;    // self-paired task: slot a only
      Yr[k1 * M2 + n2] = cmulc(lds[s * RP + lds_pad(n2)], w_M(twm, n2 * k1));
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.  Intermediate rows live in the workspace's big buffer, in
// logical row order (channel-major for the convolution: row = h*batch + b),
// while u and y stay in their [batch][H][L] layout: the column kernels map a
// logical row to its memory row.
// ---------------------------------------------------------------------------
template <typename T>
static T* wat(unsigned char* ws, size_t off) { return reinterpret_cast<T*>(ws + off); }

template <int LOG2M>
static void big_spectrum_from_time(const s4dplr_plan* p, const float* Ktime, const float* D,
                                   unsigned char* ws, hipStream_t s, int conj) {
  using S = BigShape<LOG2M>;
  float2* Y = wat<float2>(ws, p->off_big);
  const float2* cs = wat<const float2>(ws, p->off_cs);
  const float2* tw4 = wat<const float2>(ws, p->off_tw4);
  big_cols_fwd_kernel<LOG2M><<<dim3(S::M2 / S::CT, p->H), kBigThreads, 0, s>>>(
      Ktime, Y, wat<const float2>(ws, p->off_tw1), tw4);
  big_rows_pair_kernel<LOG2M, false><<<dim3((S::M1 / 2 + 1 + 7) / 8, p->H), kBigThreads, 0, s>>>(
      Y, wat<float4>(ws, p->off_coef), D, wat<const float2>(ws, p->off_tw2), cs, tw4, 1, conj);
}

template <int LOG2M>
static void big_kspec(const s4dplr_plan* p, const float* Ktime, const float* D, float* Kout,
                      unsigned char* ws, hipStream_t s, int conj) {
  using S = BigShape<LOG2M>;
  if (!Ktime) {
    // inverse transform of the generating function (permuted layout) -> K
    float2* Y = wat<float2>(ws, p->off_big);
    float* K = Kout ? Kout : wat<float>(ws, p->off_kbuf);
    big_rows_inv_kernel<LOG2M><<<dim3(S::M1 / S::RT, p->H), kBigThreads, 0, s>>>(
        wat<const float2>(ws, p->off_khat), Y, wat<const float2>(ws, p->off_tw2),
        wat<const float2>(ws, p->off_tw4));
    big_cols_inv_kernel<LOG2M, 1><<<dim3(S::M2 / S::CT, p->H), kBigThreads, 0, s>>>(
        Y, K, wat<const float2>(ws, p->off_tw1), 1.0f / (float)S::M);
    Ktime = K;
  }
  big_spectrum_from_time<LOG2M>(p, Ktime, D, ws, s, conj);
}

hipError_t launch_big_kspec(const s4dplr_plan* p, const float* Ktime, const float* D,
                            float* Kout, unsigned char* ws, hipStream_t s, int conj) {
  if (p->log2L == 15) big_kspec<15>(p, Ktime, D, Kout, ws, s, conj);
  else if (p->log2L == 16) big_kspec<16>(p, Ktime, D, Kout, ws, s, conj);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Column kernels for the convolution need the memory row of a logical row;
// they are instantiated over a row-remapping wrapper below.
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_conv_cols_fwd_kernel(
    const float* __restrict__ u, float2* __restrict__ Y, const float2* __restrict__ tw1,
    const float2* __restrict__ tw4, int H, int batch) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, CT = S::CT, CP = S::CP;
  __shared__ float2 lds[CT * CP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, lrow = blockIdx.y, c0 = blockIdx.x * CT;
  load_twM(twm, tw4, tid, kBigThreads);
  const int h = lrow / batch, b = lrow - h * batch;
  const float2* __restrict__ z = reinterpret_cast<const float2*>(u + ((size_t)b * H + h) * M);
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int n1 = idx / CT, c = idx % CT;
    lds[c * CP + lds_pad(n1)] = (n1 < M1 / 2) ? z[M2 * n1 + c0 + c] : make_float2(0.f, 0.f);
  }
  __syncthreads();
  lds_fft<S::LOG2M1, false>(lds + (tid / (M1 / 16)) * CP, tid % (M1 / 16), true, tw1);
  float2* __restrict__ Yr = Y + (size_t)lrow * M;
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int k1 = idx / CT, c = idx % CT, n2 = c0 + c;
    Yr[k1 * M2 + n2] = cmul(lds[c * CP + lds_pad(k1)], w_M(twm, n2 * k1));
  }
}

template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_conv_cols_inv_kernel(
    const float2* __restrict__ Y, float* __restrict__ y, const float2* __restrict__ tw1, int H,
    int batch) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, CT = S::CT, CP = S::CP;
  __shared__ float2 lds[CT * CP];
  const int tid = threadIdx.x, lrow = blockIdx.y, c0 = blockIdx.x * CT;
  const int h = lrow / batch, b = lrow - h * batch;
  const float2* __restrict__ Yr = Y + (size_t)lrow * M;
  for (int idx = tid; idx < M1 * CT; idx += kBigThreads) {
    const int k1 = idx / CT, c = idx % CT;
    lds[c * CP + lds_pad(k1)] = Yr[k1 * M2 + c0 + c];
  }
  __syncthreads();
  lds_fft<S::LOG2M1, true>(lds + (tid / (M1 / 16)) * CP, tid % (M1 / 16), true, tw1);
  float2* __restrict__ yr = reinterpret_cast<float2*>(y + ((size_t)b * H + h) * M);
  for (int idx = tid; idx < (M1 / 2) * CT; idx += kBigThreads) {
    const int n1 = idx / CT, c = idx % CT;
    yr[M2 * n1 + c0 + c] = lds[c * CP + lds_pad(n1)];
  }
}

template <int LOG2M>
static void big_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                     hipStream_t s) {
  using S = BigShape<LOG2M>;
  const int rows = p->batch * p->H;
  float2* Y = wat<float2>(ws, p->off_big);
  const float2* cs = wat<const float2>(ws, p->off_cs);
  const float2* tw4 = wat<const float2>(ws, p->off_tw4);
  big_conv_cols_fwd_kernel<LOG2M><<<dim3(S::M2 / S::CT, rows), kBigThreads, 0, s>>>(
      u, Y, wat<const float2>(ws, p->off_tw1), tw4, p->H, p->batch);
  big_rows_pair_kernel<LOG2M, true><<<dim3((S::M1 / 2 + 1 + 7) / 8, rows), kBigThreads, 0, s>>>(
      Y, wat<float4>(ws, p->off_coef), nullptr, wat<const float2>(ws, p->off_tw2), cs, tw4,
      p->batch, 0);
  big_conv_cols_inv_kernel<LOG2M><<<dim3(S::M2 / S::CT, rows), kBigThreads, 0, s>>>(
      Y, y, wat<const float2>(ws, p->off_tw1), p->H, p->batch);
}

// ---------------------------------------------------------------------------
// Backward pass for the long path.  Row step of the forward transform alone:
// Z[k1][k2] = sum_{n2} Y[k1][n2] W_M2^{n2 k2}, in place (the column step has
// already applied the twiddle), leaving bin k1 + M1 k2 at k1 M2 + k2.
// ---------------------------------------------------------------------------
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_rows_fwd_kernel(
    float2* __restrict__ Y, const float2* __restrict__ tw2) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M2 = S::M2, RT = S::RT, RP = S::RP;
  __shared__ float2 lds[RT * RP];
  const int tid = threadIdx.x, row = blockIdx.y, r0 = blockIdx.x * RT;
  float2* __restrict__ Yr = Y + (size_t)row * M;
  for (int idx = tid; idx < RT * M2; idx += kBigThreads) {
    const int s = idx / M2, n2 = idx % M2;
    lds[s * RP + lds_pad(n2)] = Yr[(r0 + s) * M2 + n2];
  }
  __syncthreads();
  lds_fft<S::LOG2M2, false>(lds + (tid / 16) * RP, tid % 16, true, tw2);
  for (int idx = tid; idx < RT * M2; idx += kBigThreads) {
    const int s = idx / M2, k2 = idx % M2;
    Yr[(r0 + s) * M2 + k2] = lds[s * RP + lds_pad(k2)];
  }
}

// position of bin k in the permuted layout
template <int LOG2M>
__device__ __forceinline__ int big_pos(int k) {
  using S = BigShape<LOG2M>;
  return (k & (S::M1 - 1)) * S::M2 + (k >> S::LOG2M1);
}

// dK: per channel h and bin k, the batch sums S_k and S_{M-k} of
// conj(U_j) G_j over the spectra of the zero-padded u and dy rows
// (X_j = big_rfft_x(Z_j, Z_{M-j}), Z_M = Z_0), and the packed inverse input
//   W_k = (S_k + conj S_{M-k}) / 2 + i e^{i pi k/M} (S_k - conj S_{M-k}) / 2,
// scaled by 1/M, at the bin's position in the permuted layout.  Thread i takes
// position i, so the reads of bin k and of its partner M - k (rows k1 and
// M1 - k1 read backwards, or row 0 with k2 -> -k2) are both contiguous.
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_corr_kernel(
    const float2* __restrict__ Zu, const float2* __restrict__ Zg, float2* __restrict__ W,
    const float2* __restrict__ cs, int batch) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2;
  const int h = blockIdx.y;
  const int pk = blockIdx.x * kBigThreads + threadIdx.x;     // < M (grid is exact)
  const int k1 = pk / M2, k2 = pk % M2;
  const int k = k1 + M1 * k2;
  const int km = M - k;                                       // in [1, M]
  const int pm = big_pos<LOG2M>(km & (M - 1));
  const float2 ck = cs[k], cm = cs[km];
  float2 sk = make_float2(0.f, 0.f), sm = sk;
  for (int b = 0; b < batch; ++b) {
    const size_t r = ((size_t)h * batch + b) * M;
    const float2 uk = Zu[r + pk], um = Zu[r + pm], gk = Zg[r + pk], gm = Zg[r + pm];
    const float2 Uk = big_rfft_x(uk, um, ck), Gk = big_rfft_x(gk, gm, ck);
    const float2 Um = big_rfft_x(um, uk, cm), Gm = big_rfft_x(gm, gk, cm);
    sk = cadd(sk, cmul(cconj(Uk), Gk));
    sm = cadd(sm, cmul(cconj(Um), Gm));
  }
  const float sc = 0.5f / (float)M;
  const float2 ek = make_float2(sk.x + sm.x, sk.y - sm.y);
  const float2 dk = make_float2(sk.x - sm.x, sk.y + sm.y);
  const float2 wk = cadd(ek, cmul(make_float2(-ck.y, ck.x), dk));
  W[(size_t)h * M + pk] = make_float2(sc * wk.x, sc * wk.y);
}

// Ghat_l = FFT_L(dK)_l / L = X_{2l} / L, X the spectrum of dK zero-padded to
// 2L (from Z in the permuted layout); X_{2M - j} = conj(X_j).
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_ghat_kernel(
    const float2* __restrict__ Z, float2* __restrict__ ghat, const float2* __restrict__ cs) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M;
  const int h = blockIdx.y;
  const int l = blockIdx.x * kBigThreads + threadIdx.x;
  if (l >= M) return;
  int j = 2 * l;
  const bool mirror = j > M;
  if (mirror) j = 2 * M - j;
  const float2* __restrict__ Zh = Z + (size_t)h * M;
  const float2 zj = Zh[big_pos<LOG2M>(j & (M - 1))], zm = Zh[big_pos<LOG2M>((M - j) & (M - 1))];
  float2 x = big_rfft_x(zj, zm, cs[j]);
  if (mirror) x = cconj(x);
  const float inv = 1.0f / (float)M;
  ghat[(size_t)h * M + l] = make_float2(x.x * inv, x.y * inv);
}

__global__ void big_first_col_kernel(const float* __restrict__ K, float* __restrict__ d, int H,
                                     int L) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h < H) d[h] = K[(size_t)h * L];
}

template <int LOG2M>
static void big_corr(const s4dplr_plan* p, const float* u, const float* dy, float* dK, float* dD,
                     unsigned char* ws, hipStream_t s) {
  using S = BigShape<LOG2M>;
  const int rows = p->batch * p->H;
  float2* Yu = wat<float2>(ws, p->off_big);
  float2* Yg = wat<float2>(ws, p->off_big2);
  const float2* tw1 = wat<const float2>(ws, p->off_tw1);
  const float2* tw2 = wat<const float2>(ws, p->off_tw2);
  const float2* tw4 = wat<const float2>(ws, p->off_tw4);
  const float2* cs = wat<const float2>(ws, p->off_cs);
  const dim3 cgrid(S::M2 / S::CT, rows), rgrid(S::M1 / S::RT, rows);
  big_conv_cols_fwd_kernel<LOG2M><<<cgrid, kBigThreads, 0, s>>>(u, Yu, tw1, tw4, p->H, p->batch);
  big_conv_cols_fwd_kernel<LOG2M><<<cgrid, kBigThreads, 0, s>>>(dy, Yg, tw1, tw4, p->H, p->batch);
  big_rows_fwd_kernel<LOG2M><<<rgrid, kBigThreads, 0, s>>>(Yu, tw2);
  big_rows_fwd_kernel<LOG2M><<<rgrid, kBigThreads, 0, s>>>(Yg, tw2);
  float2* Wb = wat<float2>(ws, p->off_khat);
  big_corr_kernel<LOG2M><<<dim3(S::M / kBigThreads, p->H), kBigThreads, 0, s>>>(Yu, Yg, Wb, cs,
                                                                               p->batch);
  // inverse: rows then columns, the first M/2 outputs as (c_2n, c_2n+1)
  float* out = dK ? dK : wat<float>(ws, p->off_kbuf);
  big_rows_inv_kernel<LOG2M><<<dim3(S::M1 / S::RT, p->H), kBigThreads, 0, s>>>(Wb, Yu, tw2, tw4);
  big_cols_inv_kernel<LOG2M, 0><<<dim3(S::M2 / S::CT, p->H), kBigThreads, 0, s>>>(Yu, out, tw1,
                                                                                 1.0f);
  if (dD) big_first_col_kernel<<<(p->H + 255) / 256, 256, 0, s>>>(out, dD, p->H, p->L);
}

template <int LOG2M>
static void big_ghat(const s4dplr_plan* p, const float* dK, float2* ghat, unsigned char* ws,
                     hipStream_t s) {
  using S = BigShape<LOG2M>;
  float2* Y = wat<float2>(ws, p->off_big);
  big_cols_fwd_kernel<LOG2M><<<dim3(S::M2 / S::CT, p->H), kBigThreads, 0, s>>>(
      dK, Y, wat<const float2>(ws, p->off_tw1), wat<const float2>(ws, p->off_tw4));
  big_rows_fwd_kernel<LOG2M><<<dim3(S::M1 / S::RT, p->H), kBigThreads, 0, s>>>(
      Y, wat<const float2>(ws, p->off_tw2));
  big_ghat_kernel<LOG2M><<<dim3(S::M / kBigThreads, p->H), kBigThreads, 0, s>>>(
      Y, ghat, wat<const float2>(ws, p->off_cs));
}

hipError_t launch_big_corr(const s4dplr_plan* p, const float* u, const float* dy, float* dK,
                           float* dD, unsigned char* ws, hipStream_t s) {
  if (p->log2L == 15) big_corr<15>(p, u, dy, dK, dD, ws, s);
  else if (p->log2L == 16) big_corr<16>(p, u, dy, dK, dD, ws, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_big_ghat(const s4dplr_plan* p, const float* dK, unsigned char* ws,
                           hipStream_t s) {
  float2* ghat = wat<float2>(ws, p->off_bghat);
  if (p->log2L == 15) big_ghat<15>(p, dK, ghat, ws, s);
  else if (p->log2L == 16) big_ghat<16>(p, dK, ghat, ws, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_big_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                           hipStream_t s) {
  if (p->log2L == 15) big_conv<15>(p, u, y, ws, s);
  else if (p->log2L == 16) big_conv<16>(p, u, y, ws, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace s4
