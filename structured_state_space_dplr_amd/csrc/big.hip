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
  static_assert(LOG2M >= 14 && LOG2M <= 16, "four-step range");
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
// Column steps.  A task is CT = 256/T adjacent columns n2 of one logical row,
// T = M1/16 lanes per column, 16 points per lane:
//   * global reads with the column index fastest (whole cache lines), straight
//     into the first radix-16 pass (input n1 = la + T r in lane la);
//   * LDS, then the remaining pass with the T lanes of a column inside one
//     wave; its outputs go back to LDS in natural order;
//   * global writes with the column index fastest.
// Blocks are persistent (a few per CU) and the next task's input is in flight
// while the current one is transformed.  Logical row h*batch + b reads or
// writes memory row b*H + h of the [batch][H][L] arrays (batch = 1: row h).
// ---------------------------------------------------------------------------
template <int LOG2M, int NTHR = kBigThreads>
struct ColShape {
  using S = BigShape<LOG2M>;
  static constexpr int LOG2M1 = S::LOG2M1, M1 = S::M1, M2 = S::M2;
  static constexpr int T = M1 / 16;                  // lanes per column
  static constexpr int CT = NTHR / T;                // columns per task
  static constexpr int NG = M2 / CT;                 // tasks per logical row
  static constexpr int CP = lds_padded_size(M1);
  static_assert(fft_num_passes(LOG2M1) == 2 && fft_radix_log(LOG2M1, 0) == 4, "two passes");
};
constexpr int kColBlocks = 256 * 4;   // four resident blocks per CU (LDS-bound)

template <int LOG2M, int NTHR = kBigThreads>
static int col_blocks(int rows) {
  const int ntask = rows * ColShape<LOG2M, NTHR>::NG;
  return ntask < kColBlocks ? ntask : kColBlocks;
}

__device__ __forceinline__ size_t mem_row(int lrow, int H, int batch) {
  const int h = lrow / batch, b = lrow - h * batch;
  return (size_t)b * H + h;
}

// Forward column step on real rows x (L floats, packed z_k = x_2k + i x_2k+1,
// z zero for k >= M/2): Y[row][k1][n2] = W_M^{n2 k1} sum_{n1} z[M2 n1 + n2] W_M1^{n1 k1}
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads, 4) void big_cols_fwd_kernel(
    const float* __restrict__ x, float2* __restrict__ Y, const float2* __restrict__ tw1,
    const float2* __restrict__ tw4, int rows, int H, int batch) {
  using C = ColShape<LOG2M>;
  using P0 = WPass<C::LOG2M1, 0>;
  using P1 = WPass<C::LOG2M1, 1>;
  constexpr int M = BigShape<LOG2M>::M, M2 = C::M2, T = C::T, CT = C::CT, NG = C::NG,
                CP = C::CP;
  __shared__ float2 lds[CT * CP];
  __shared__ TwM twm;
  const int tid = threadIdx.x;
  const int ca = tid % CT, la = tid / CT;    // global side: column fastest
  const int cb = tid / T, lb = tid % T;      // transform side: a column's lanes in one wave
  load_twM(twm, tw4, tid, kBigThreads);
  PassTwiddles<C::LOG2M1, 1> pt;
  pt.load(tw1, lb);
  const int ntask = rows * NG;
  float2 pre[8];
  auto fetch = [&](int task) {
    const int lrow = task / NG, g = task - lrow * NG;
    const float2* __restrict__ z =
        reinterpret_cast<const float2*>(x + mem_row(lrow, H, batch) * M) + g * CT + ca;
#pragma unroll
    for (int r = 0; r < 8; ++r) pre[r] = load_stream(&z[M2 * (la + T * r)]);   // n1 < M1/2
  };
  int task = blockIdx.x;
  if (task < ntask) fetch(task);
  __syncthreads();
  for (; task < ntask; task += gridDim.x) {
    float2 v[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = pre[r];
    if (task + (int)gridDim.x < ntask) fetch(task + gridDim.x);
    dft16_fwd_half_input(v);
    P0::store(v, lds + ca * CP, la);
    __syncthreads();
    P1::load(v, lds + cb * CP, lb);
    {
      float2 w1[16];
      pt.expand(w1);
      P1::template compute<false>(v, w1);
    }
    wave_sync();
    P1::store(v, lds + cb * CP, lb);
    __syncthreads();
    const int lrow = task / NG, n2 = (task - lrow * NG) * CT + ca;
    float2* __restrict__ Yr = Y + (size_t)lrow * M + n2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k1 = la + T * r;
      Yr[k1 * M2] = cmul(lds[ca * CP + lds_pad(k1)], w_M(twm, n2 * k1));
    }
    __syncthreads();
  }
}

// Inverse column step: x[M2 n1 + n2] = sum_{k1} Y[k1][n2] W_M1^{-n1 k1}.
// MODE 0: outputs n < M/2 as (y_2n, y_2n+1) (the kept half of the causal
// convolution).  MODE 1: all n, real part times `scale` (time-domain kernel).
template <int LOG2M, int MODE>
__global__ __launch_bounds__(kBigThreads, 4) void big_cols_inv_kernel(
    const float2* __restrict__ Y, float* __restrict__ out, const float2* __restrict__ tw1,
    int rows, int H, int batch, float scale) {
  using C = ColShape<LOG2M>;
  using P0 = WPass<C::LOG2M1, 0>;
  using P1 = WPass<C::LOG2M1, 1>;
  constexpr int M = BigShape<LOG2M>::M, M2 = C::M2, T = C::T, CT = C::CT, NG = C::NG,
                CP = C::CP;
  __shared__ float2 lds[CT * CP];
  const int tid = threadIdx.x;
  const int ca = tid % CT, la = tid / CT;
  const int cb = tid / T, lb = tid % T;
  PassTwiddles<C::LOG2M1, 1> pt;
  pt.load(tw1, lb);
  const int ntask = rows * NG;
  float2 pre[16];
  auto fetch = [&](int task) {
    const int lrow = task / NG, g = task - lrow * NG;
    const float2* __restrict__ Yr = Y + (size_t)lrow * M + g * CT + ca;
#pragma unroll
    for (int r = 0; r < 16; ++r) pre[r] = Yr[M2 * (la + T * r)];
  };
  int task = blockIdx.x;
  if (task < ntask) fetch(task);
  for (; task < ntask; task += gridDim.x) {
    float2 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = pre[r];
    if (task + (int)gridDim.x < ntask) fetch(task + gridDim.x);
    dft_dif<16, true>(v);
    P0::store(v, lds + ca * CP, la);
    __syncthreads();
    P1::load(v, lds + cb * CP, lb);
    {
      float2 w1[16];
      pt.expand(w1);
      P1::template compute<true>(v, w1);
    }
    wave_sync();
    P1::store(v, lds + cb * CP, lb);
    __syncthreads();
    const int lrow = task / NG, n2 = (task - lrow * NG) * CT + ca;
    if constexpr (MODE == 0) {
      float2* __restrict__ yr =
          reinterpret_cast<float2*>(out + mem_row(lrow, H, batch) * M) + n2;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int n1 = la + T * r;     // < M1/2
        store_stream(&yr[M2 * n1], lds[ca * CP + lds_pad(n1)]);
      }
    } else {
      float* __restrict__ kr = out + mem_row(lrow, H, batch) * M + n2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n1 = la + T * r;
        kr[M2 * n1] = lds[ca * CP + lds_pad(n1)].x * scale;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Row step alone, one 256-point row per 16-lane group (no workgroup barrier
// after the twiddle table is in LDS):
//   forward (!INV): Z[k1][k2] = sum_{n2} Y[k1][n2] W_M2^{n2 k2}, in place (the
//                   column step has applied the twiddle); bin k1 + M1 k2 is
//                   left at k1 M2 + k2;
//   inverse (INV):  Y[k1][n2] = W_M^{-n2 k1} sum_{k2} X[k1][k2] W_M2^{-n2 k2}
//                   (X in the permuted layout, e.g. the generating function).
// Every lane reads and writes the same 16 points of its row, so X may be Y.
// TWS = 2 takes the four-step twiddles W_M^m of an M-point transform from the
// table of a 2M-point one (W_M^m = W_2M^(2m)).
// ---------------------------------------------------------------------------
template <int LOG2M, bool INV, int TWS = 1>
__global__ __launch_bounds__(kBigThreads) void big_rows_kernel(
    const float2* X, float2* Y, const float2* __restrict__ tw2, const float2* __restrict__ tw4,
    int rows) {
  using S = BigShape<LOG2M>;
  using P0 = WPass<8, 0>;
  using P1 = WPass<8, 1>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, MP = lds_padded_size(M2);
  constexpr int G = kBigThreads / 16;
  __shared__ float2 lds[G * MP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, grp = tid >> 4, lt = tid & 15;
  if constexpr (INV) {
    load_twM(twm, tw4, tid, kBigThreads);
    __syncthreads();
  }
  const int task = blockIdx.x * G + grp;
  if (task >= rows * M1) return;
  const int lrow = task / M1, k1 = task - lrow * M1;
  const float2* Xr = X + (size_t)lrow * M + k1 * M2;
  float2 v[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = Xr[lt + 16 * r];
  PassTwiddles<8, 1> pt;
  pt.load(tw2, lt);
  float2* buf = lds + grp * MP;
  dft_dif<16, INV>(v);
  P0::store(v, buf, lt);
  wave_sync();
  P1::load(v, buf, lt);
  {
    float2 w[16];
    pt.expand(w);
    P1::template compute<INV>(v, w);
  }
  float2* Yr = Y + (size_t)lrow * M + k1 * M2;
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) {
    const int n = lt + 16 * s2;
    float2 o = v[bitrev<4>(s2)];
    if constexpr (INV) o = cmulc(o, w_M(twm, TWS * n * k1));
    Yr[n] = o;
  }
}

template <int LOG2M>
static int rows_blocks(int rows) {
  return (rows * BigShape<LOG2M>::M1 + kBigThreads / 16 - 1) / (kBigThreads / 16);
}

// ---------------------------------------------------------------------------
// Paired row steps, one pair task per 16-lane group and no workgroup barrier
// after the twiddle table is in LDS.  Task (h, t, b), t = 0 .. M1/2, takes
// rows ka = t and kb = M1 - t (mod M1) of logical row h*batch + b; the
// tasks are numbered with b fastest, so the groups of one wave that share a
// channel read the same weights in the same instructions.
// Lane lt runs the 256-point transforms of row ka as transform lane lt and of
// row kb as transform lane lb = 15 - lt (t = 0: lb = -lt mod 16).  After the
// forward passes the lane holds bins k2 = lt + 16 s of row ka, and the
// real-FFT partner of each, bin M2-1-k2 (row 0: -k2) of row kb, is bin
// lb + 16 (15 - s) of row kb in the same lane (t = 0, lt = 0: bin
// 16 ((16 - s) mod 16) of row 0 itself).  Tasks t = 0 and t = M1/2 pair a row
// with itself: the lane's row-ka bins are then the whole row and only they
// are kept.
//   CONV:  spectral weights Z'_k = alpha_k Z_k + beta_k conj(Z_{M-k}), the
//          inverse row DFTs (the lane's bins are exactly its first inverse
//          pass input) and the inverse twiddle, back into Y.  The weights of a
//          bin come from the stored spectrum at the bin and at its partner,
//          which the lane holds for both of its rows:
//            alpha_k = ((1 - s_k) S_k + (1 + s_k) conj(S_{M-k})) / (2M),
//            beta_k  = i c_k (S_k - conj(S_{M-k})) / (2M),
//          (c_k, s_k) = (cos, sin)(pi k / M).
//   !CONV: the spectrum S of (K + D delta) padded to 2M (conjugated for the
//          correlation), one float2 per bin in the permuted layout; bin 0's
//          slot holds the two real values (S_0, S_M).
// Storing S (8 B per bin) rather than alpha and beta (16 B) halves the
// spectrum's traffic in both kernels.
// Registers and LDS: the two rows go through one LDS buffer per group in
// turn, and S is read inside the weighting loop, two values per bin pair,
// so that the kernel stays under 168 VGPRs and 40 KB of LDS per block: three
// waves per SIMD instead of two.
// ---------------------------------------------------------------------------
template <int LOG2M, bool CONV>
__global__ __launch_bounds__(kBigThreads) void big_rows_pair_kernel(
    float2* __restrict__ Y, float2* __restrict__ specp, const float* __restrict__ D,
    const float2* __restrict__ tw2, const float2* __restrict__ cs,
    const float2* __restrict__ tw4, int nh, int batch, int conj) {
  using S = BigShape<LOG2M>;
  using P0 = WPass<8, 0>;
  using P1 = WPass<8, 1>;
  static_assert(S::M2 == 256 && P0::T == 16 && P1::NS == 16, "256-point rows, 16 lanes");
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2;
  constexpr int MP = lds_padded_size(M2);
  constexpr int G = kBigThreads / 16;      // pair tasks per block
  constexpr int TP = M1 / 2 + 1;           // pair tasks per logical row
  __shared__ float2 lds[G * MP];
  __shared__ TwM twm;
  const int tid = threadIdx.x, grp = tid >> 4, lt = tid & 15;
  if constexpr (CONV) {
    load_twM(twm, tw4, tid, kBigThreads);
    __syncthreads();
  }
  const int task = blockIdx.x * G + grp;
  if (task >= nh * TP * batch) return;
  const int b = task % batch, ht = task / batch, t = ht % TP, h = ht / TP;
  const int ka = t, kb = (M1 - t) & (M1 - 1);
  const bool self = ka == kb;
  const int lb = (t == 0) ? ((16 - lt) & 15) : 15 - lt;
  const bool sp = (t == 0) && (lt == 0);
  float2* __restrict__ Yr = Y + (size_t)(h * batch + b) * M;
  float2* __restrict__ bufA = lds + grp * MP;
  float2 za[16], zb[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    za[r] = Yr[ka * M2 + lt + 16 * r];
    zb[r] = Yr[kb * M2 + lb + 16 * r];
  }
  PassTwiddles<8, 1> pta, ptb;
  pta.load(tw2, lt);
  ptb.load(tw2, lb);
  // forward pass 0 (span 1, no twiddles), then pass 1 through LDS
  dft_dif<16, false>(za);
  dft_dif<16, false>(zb);
  P0::store(za, bufA, lt);
  const float2 cs0 = cs[ka + M1 * lt];
  wave_sync();
  P1::load(za, bufA, lt);
  wave_sync();
  P0::store(zb, bufA, lb);
  wave_sync();
  P1::load(zb, bufA, lb);
  {
    float2 w[16];
    pta.expand(w);
    P1::template compute<false>(za, w);
    ptb.expand(w);
    P1::template compute<false>(zb, w);
  }
  // bin lt + 16 s of row ka is za[bitrev(s)]; its partner is pz[s]
  float2 pz[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2)
    pz[s2] = sp ? zb[bitrev<4>((16 - s2) & 15)] : zb[bitrev<4>(15 - s2)];
  // cs_k = (cos, sin)(pi k / M) for k = ka + M1 (lt + 16 s) is cs of the
  // lane's first bin turned by pi s / 16; cs_{M-k} = (-cos, sin)(pi k / M)
  float2 csa[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) csa[s2] = cmul(cs0, make_float2(kCos32[s2], kSin32[s2]));
  if constexpr (CONV) {
    // weighted bins in natural order: oa[s] = Z'(lt + 16 s) of row ka,
    // ob[s] = Z'(lb + 16 s) of row kb (whose partners, for the tasks that
    // keep row kb, are the row-ka bins lt + 16 (15 - s))
    const float sc = 0.5f / (float)M;
    // Z'_k from the bin, its partner's bin, S at both and (c, s) of k
    auto weigh = [sc](float2 z, float2 zp, float2 S, float2 Sp, float2 c) {
      const float a = sc * (1.0f - c.y), b = sc * (1.0f + c.y), cc = sc * c.x;
      const float2 al = make_float2(fmaf(a, S.x, b * Sp.x), fmaf(a, S.y, -b * Sp.y));
      const float2 df = make_float2(S.x - Sp.x, S.y + Sp.y);           // S_k - conj(S_{M-k})
      const float2 be = make_float2(-cc * df.y, cc * df.x);            // i c (S_k - conj S_{M-k})
      return cadd(cmul(al, z), cmul(be, cconj(zp)));
    };
    float2 oa[16], ob[16];
    const float2* __restrict__ spa = specp + (size_t)h * M + ka * M2 + lt;
    const float2* __restrict__ spb = specp + (size_t)h * M + kb * M2 + lb;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      // row-ka bin s2 and its partner, row-kb bin 15 - s2, give oa[s2] and
      // ob[15 - s2] from the same four values.  The sp lane's partner of
      // bin s2 is its own bin (16 - s2) mod 16 of row 0 instead; that task
      // keeps only row ka, so its ob may take that S value as well.
      const int ps = sp ? ((16 - s2) & 15) : 15 - s2;
      const float2 Sa = spa[16 * s2], Sb = spb[16 * ps];
      const float2 ca = cmul(cs0, make_float2(kCos32[s2], kSin32[s2]));
      float2 S = Sa, Sp = Sb;
      if (sp && s2 == 0) {   // bin 0: the slot holds (S_0, S_M), both real
        S = make_float2(Sa.x, 0.f);
        Sp = make_float2(Sa.y, 0.f);
      }
      oa[s2] = weigh(za[bitrev<4>(s2)], pz[s2], S, Sp, ca);
      ob[15 - s2] = weigh(zb[bitrev<4>(15 - s2)], za[bitrev<4>(s2)], Sb, Sa,
                          make_float2(-ca.x, ca.y));
    }
    // inverse pass 0: input x[lt + 16 r] = bin lt + 16 r, already in this lane
    dft_dif<16, true>(oa);
    dft_dif<16, true>(ob);
    wave_sync();
    P0::store(oa, bufA, lt);
    wave_sync();
    P1::load(oa, bufA, lt);
    wave_sync();
    P0::store(ob, bufA, lb);
    wave_sync();
    P1::load(ob, bufA, lb);
    {
      float2 w[16];
      pta.expand(w);
      P1::template compute<true>(oa, w);
      ptb.expand(w);
      P1::template compute<true>(ob, w);
    }
    // output n2 = lt + 16 s (row kb: lb + 16 s) in [bitrev(s)]
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const int n2 = lt + 16 * s2;
      Yr[ka * M2 + n2] = cmulc(oa[bitrev<4>(s2)], w_M(twm, n2 * ka));
    }
    if (!self) {
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        const int n2 = lb + 16 * s2;
        Yr[kb * M2 + n2] = cmulc(ob[bitrev<4>(s2)], w_M(twm, n2 * kb));
      }
    }
  } else {
    const float Dh = D ? D[h] : 0.f;
    float2* __restrict__ sph = specp + (size_t)h * M;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const int k2 = lt + 16 * s2;
      const int k2p = sp ? ((16 - s2) & 15) * 16 : lb + 16 * (15 - s2);   // partner's k2
      const float2 za_ = za[bitrev<4>(s2)], zb_ = pz[s2];
      const float2 csb = make_float2(-csa[s2].x, csa[s2].y);
      float2 sa = big_rfft_x(za_, zb_, csa[s2]), sb = big_rfft_x(zb_, za_, csb);
      sa.x += Dh;
      sb.x += Dh;
      if (conj) {   // the spectrum of the correlation with (K + D delta)
        sa.y = -sa.y;
        sb.y = -sb.y;
      }
      if (sp && s2 == 0) {
        sph[0] = make_float2(sa.x, sb.x);     // (S_0, S_M): both real
      } else {
        sph[ka * M2 + k2] = sa;
        if (!self) sph[kb * M2 + k2p] = sb;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 1 from the half-length spectrum Y (rank 1): the packed kernel
// z_n = K_2n + i K_2n+1 = IDFT_{L/2}(Y)_n / L (n < L/2) and the padded
// spectrum S_k = sum_{n<L} K_n W_2L^{kn} + D (k <= L).  The even bins are
// the Hermitian part of the generating function, S_2m = Xh_m + D, written by
// the Cauchy kernel.  For the odd bins, with a = K_even, b = K_odd,
//   S_{2j+1} = E_j + W_2L^{2j+1} O_j + D,
//   E = DFT_{L/2}(a_m W_L^m),  O = DFT_{L/2}(b_m W_L^m),
// and F = DFT_{L/2}(z_m W_L^m) = E + i O; a and b are real, so
// E_{L/2-1-j} = conj E_j (likewise O), which separates the two:
//   E_j = (F_j + conj F_p) / 2,  O_j = (F_j - conj F_p) / (2i),  p = L/2 - 1 - j.
// So one L/2-point transform gives all odd bins, where the padded transform
// of K takes an L-point one ("The S4 kernel, from scratch", section 5: the
// spectrum of the kernel zero-padded to 2L).
// ---------------------------------------------------------------------------

// Column step (M = L/2 points per row, four-step M1 x 256): the inverse
// column DFTs after big_rows_kernel, z times `scale` out as K (natural
// order), then z_n W_L^n through the forward column DFTs, times the four-step
// twiddle W_M^{n2 k1}, into F[row][k1][n2].  One-wave blocks, one task each
// (a quarter of the columns per task of the other column steps; the
// waveform workload's 64 rows give 2048): at waveform 16.8 us against
// 17.1-17.2 with 128 threads and 20.9 with 256.
template <int LOG2M>
__global__ __launch_bounds__(64) void big_cols_invfwd_kernel(
    const float2* __restrict__ X, float* __restrict__ K, float2* __restrict__ F,
    const float2* __restrict__ tw1, const float2* __restrict__ tw4, int rows, float scale) {
  using C = ColShape<LOG2M, 64>;
  using P0 = WPass<C::LOG2M1, 0>;
  using P1 = WPass<C::LOG2M1, 1>;
  constexpr int M = BigShape<LOG2M>::M, M2 = C::M2, T = C::T, CT = C::CT, NG = C::NG,
                CP = C::CP;
  __shared__ float2 lds[CT * CP];
  __shared__ TwM twm;   // W_L^m, L = 2M: the twist W_L^n and, at even powers, W_M
  const int tid = threadIdx.x;
  const int ca = tid % CT, la = tid / CT;
  const int cb = tid / T, lb = tid % T;
  load_twM(twm, tw4, tid, 64);
  PassTwiddles<C::LOG2M1, 1> pt;
  pt.load(tw1, lb);
  const int ntask = rows * NG;
  float2 pre[16];
  auto fetch = [&](int task) {
    const int lrow = task / NG, g = task - lrow * NG;
    const float2* __restrict__ Xr = X + (size_t)lrow * M + g * CT + ca;
#pragma unroll
    for (int r = 0; r < 16; ++r) pre[r] = Xr[M2 * (la + T * r)];
  };
  int task = blockIdx.x;
  if (task < ntask) fetch(task);
  __syncthreads();
  for (; task < ntask; task += gridDim.x) {
    float2 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = pre[r];
    if (task + (int)gridDim.x < ntask) fetch(task + gridDim.x);
    // inverse column DFT
    dft_dif<16, true>(v);
    P0::store(v, lds + ca * CP, la);
    __syncthreads();
    P1::load(v, lds + cb * CP, lb);
    {
      float2 w1[16];
      pt.expand(w1);
      P1::template compute<true>(v, w1);
    }
    wave_sync();
    P1::store(v, lds + cb * CP, lb);
    __syncthreads();
    const int lrow = task / NG, n2 = (task - lrow * NG) * CT + ca;
    float2* __restrict__ zr = reinterpret_cast<float2*>(K + (size_t)lrow * (2 * (size_t)M)) + n2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n1 = la + T * r;
      const float2 zv = lds[ca * CP + lds_pad(n1)];
      const float2 zs = make_float2(zv.x * scale, zv.y * scale);
      zr[M2 * n1] = zs;
      v[r] = cmul(zs, w_M(twm, M2 * n1 + n2));        // z_n W_L^n, the input n1 = la + T r
    }
    __syncthreads();                                   // the column is read; reuse its LDS
    // forward column DFT of the twisted sequence
    dft_dif<16, false>(v);
    P0::store(v, lds + ca * CP, la);
    __syncthreads();
    P1::load(v, lds + cb * CP, lb);
    {
      float2 w1[16];
      pt.expand(w1);
      P1::template compute<false>(v, w1);
    }
    wave_sync();
    P1::store(v, lds + cb * CP, lb);
    __syncthreads();
    float2* __restrict__ Fr = F + (size_t)lrow * M + n2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k1 = la + T * r;
      Fr[k1 * M2] = cmul(lds[ca * CP + lds_pad(k1)], w_M(twm, 2 * n2 * k1));
    }
    __syncthreads();
  }
}

// Row step: the row DFTs of F, one row per 16-lane group, rows k1 and
// M1 - 1 - k1 in the two groups of a pair in one wave.  Bin j = k1 + M1 k2
// and its mirror p = L/2 - 1 - j = (M1 - 1 - k1) + M1 (255 - k2) are then in
// the two groups' LDS rows, so each group forms the odd bins S_{2j+1} of its
// own row into the padded spectrum's permuted layout (bin k at
// (k mod L/256) 256 + k div (L/256): row 2 k1 + 1, column k2).  One-wave
// blocks, 74 VGPRs: at waveform 8.2 us against 9.2 us for two rows per
// group with mirrored lane indices (one wave per SIMD).
template <int LOG2M>
__global__ __launch_bounds__(64) void big_rows_odd_kernel(
    const float2* __restrict__ F, float2* __restrict__ spec, const float* __restrict__ D,
    const float2* __restrict__ tw2, const float2* __restrict__ cs, int nh) {
  using S = BigShape<LOG2M>;
  using P0 = WPass<8, 0>;
  using P1 = WPass<8, 1>;
  static_assert(S::M2 == 256 && P0::T == 16 && P1::NS == 16, "256-point rows, 16 lanes");
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2, L = 2 * M;
  constexpr int MP = lds_padded_size(M2);
  constexpr int NT = 64, G = NT / 16;
  __shared__ float2 lds[G * MP];
  const int tid = threadIdx.x, grp = tid >> 4, lt = tid & 15;
  const int q = blockIdx.x * G + grp;               // groups 2i, 2i+1: rows t, M1-1-t
  if (q >= nh * M1) return;                         // uniform over pairs of groups
  const int side = q & 1, pi = q >> 1;
  const int h = pi / (M1 / 2), t = pi - h * (M1 / 2);
  const int r = side ? M1 - 1 - t : t;
  const float2* __restrict__ Fr = F + (size_t)h * M + r * M2;
  float2* __restrict__ buf = lds + grp * MP;
  const float2* __restrict__ pbuf = lds + (grp ^ 1) * MP;
  float2 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = Fr[lt + 16 * k];
  PassTwiddles<8, 1> pt;
  pt.load(tw2, lt);
  const float2 cs0 = cs[2 * r + 1 + 2 * M1 * lt];
  const float Dh = D ? D[h] : 0.f;
  dft_dif<16, false>(v);
  P0::store(v, buf, lt);
  wave_sync();
  P1::load(v, buf, lt);
  {
    float2 w[16];
    pt.expand(w);
    P1::template compute<false>(v, w);
  }
  // bins k2 = lt + 16 s of row r in v[bitrev(s)], natural order into LDS
  wave_sync();
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) buf[lds_pad(lt + 16 * s2)] = v[bitrev<4>(s2)];
  wave_sync();
  float2* __restrict__ sph = spec + (size_t)h * L + (2 * r + 1) * M2;
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) {
    const int k2 = lt + 16 * s2;
    // bin j = r + M1 k2 and its mirror L/2 - 1 - j = (M1 - 1 - r) + M1 (255 - k2)
    const float2 fj = v[bitrev<4>(s2)], fp = pbuf[lds_pad(255 - k2)];
    const float2 e = make_float2(0.5f * (fj.x + fp.x), 0.5f * (fj.y - fp.y));
    const float2 o = make_float2(0.5f * (fj.y + fp.y), -0.5f * (fj.x - fp.x));
    const float2 c = cmul(cs0, make_float2(kCos32[s2], kSin32[s2]));
    const float2 sj = cmul(make_float2(c.x, -c.y), o);   // W_2L^{2j+1} = (cos, -sin)
    sph[k2] = make_float2(e.x + sj.x + Dh, e.y + sj.y);
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

// blocks of the paired row step: M1/2 + 1 pair tasks per logical row, one per
// 16-lane group
template <int LOG2M>
static int pair_blocks(int rows) {
  constexpr int TP = BigShape<LOG2M>::M1 / 2 + 1, G = kBigThreads / 16;
  return (rows * TP + G - 1) / G;
}

template <int LOG2M>
static void big_spectrum_from_time(const s4dplr_plan* p, const float* Ktime, const float* D,
                                   unsigned char* ws, hipStream_t s, int conj) {
  float2* Y = wat<float2>(ws, p->off_big);
  const float2* cs = wat<const float2>(ws, p->off_cs);
  const float2* tw4 = wat<const float2>(ws, p->off_tw4);
  big_cols_fwd_kernel<LOG2M><<<col_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
      Ktime, Y, wat<const float2>(ws, p->off_tw1), tw4, p->H, p->H, 1);
  big_rows_pair_kernel<LOG2M, false><<<pair_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
      Y, wat<float2>(ws, p->off_coef), D, wat<const float2>(ws, p->off_tw2), cs, tw4, p->H, 1,
      conj);
}

template <int LOG2M>
static void big_kspec(const s4dplr_plan* p, const float* Ktime, const float* D, float* Kout,
                      unsigned char* ws, hipStream_t s, int conj, bool half) {
  using S = BigShape<LOG2M>;
  if (!Ktime && half) {
    // The workspace holds Y (M/2 points, the four-step order of an M/2-point
    // transform) and the even bins of S; the inverse transform of Y, times
    // 1/M, is the packed kernel z_n = K_2n + i K_2n+1 (K in natural order),
    // and one more M/2-point transform of it gives the odd bins.
    float2* Xr = wat<float2>(ws, p->off_big);
    float2* F = wat<float2>(ws, p->off_khat);   // Y is consumed by the row step
    float* K = Kout ? Kout : wat<float>(ws, p->off_kbuf);
    const float2* tw4 = wat<const float2>(ws, p->off_tw4);
    big_rows_kernel<LOG2M - 1, true, 2><<<rows_blocks<LOG2M - 1>(p->H), kBigThreads, 0, s>>>(
        wat<const float2>(ws, p->off_khat), Xr, wat<const float2>(ws, p->off_tw2), tw4, p->H);
    big_cols_invfwd_kernel<LOG2M - 1><<<(p->H * ColShape<LOG2M - 1, 64>::NG), 64, 0, s>>>(
        Xr, K, F, wat<const float2>(ws, p->off_tw1h), tw4, p->H, 1.0f / (float)S::M);
    constexpr int G = 64 / 16, NR = BigShape<LOG2M - 1>::M1;
    big_rows_odd_kernel<LOG2M - 1><<<(p->H * NR + G - 1) / G, 64, 0, s>>>(
        F, wat<float2>(ws, p->off_coef), D, wat<const float2>(ws, p->off_tw2),
        wat<const float2>(ws, p->off_cs), p->H);
    return;
  }
  if (!Ktime) {
    // inverse transform of the generating function (permuted layout) -> K
    float2* Y = wat<float2>(ws, p->off_big);
    float* K = Kout ? Kout : wat<float>(ws, p->off_kbuf);
    big_rows_kernel<LOG2M, true><<<rows_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
        wat<const float2>(ws, p->off_khat), Y, wat<const float2>(ws, p->off_tw2),
        wat<const float2>(ws, p->off_tw4), p->H);
    big_cols_inv_kernel<LOG2M, 1><<<col_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
        Y, K, wat<const float2>(ws, p->off_tw1), p->H, p->H, 1, 1.0f / (float)S::M);
    Ktime = K;
  }
  big_spectrum_from_time<LOG2M>(p, Ktime, D, ws, s, conj);
}

hipError_t launch_big_kspec(const s4dplr_plan* p, const float* Ktime, const float* D,
                            float* Kout, unsigned char* ws, hipStream_t s, int conj, bool half) {
  if (p->log2L == 15) big_kspec<15>(p, Ktime, D, Kout, ws, s, conj, half);
  else if (p->log2L == 16) big_kspec<16>(p, Ktime, D, Kout, ws, s, conj, half);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int LOG2M>
static void big_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                     hipStream_t s) {
  const int rows = p->batch * p->H;
  float2* Y = wat<float2>(ws, p->off_big);
  const float2* cs = wat<const float2>(ws, p->off_cs);
  const float2* tw4 = wat<const float2>(ws, p->off_tw4);
  big_cols_fwd_kernel<LOG2M><<<col_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(
      u, Y, wat<const float2>(ws, p->off_tw1), tw4, rows, p->H, p->batch);
  big_rows_pair_kernel<LOG2M, true><<<pair_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(
      Y, wat<float2>(ws, p->off_coef), nullptr, wat<const float2>(ws, p->off_tw2), cs, tw4,
      p->H, p->batch, 0);
  big_cols_inv_kernel<LOG2M, 0><<<col_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(
      Y, y, wat<const float2>(ws, p->off_tw1), rows, p->H, p->batch, 1.0f);
}

// ---------------------------------------------------------------------------
// Backward pass for the long path.
// ---------------------------------------------------------------------------

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
// scaled by 1/M, at the bin's position in the permuted layout.  Block t takes
// rows k1 = t and M1 - t (t = 0 .. M1/2), thread i the bin at position i of
// row t and its partner M - k (row M1 - t read backwards, or row 0 with
// k2 -> -k2), so every spectrum value is read once and both reads are
// contiguous; the thread writes W at both bins (rows 0 and M1/2 pair with
// themselves and write only their own bin).
template <int LOG2M>
__global__ __launch_bounds__(kBigThreads) void big_corr_kernel(
    const float2* __restrict__ Zu, const float2* __restrict__ Zg, float2* __restrict__ W,
    const float2* __restrict__ cs, int batch) {
  using S = BigShape<LOG2M>;
  constexpr int M = S::M, M1 = S::M1, M2 = S::M2;
  static_assert(M2 == kBigThreads, "one thread per bin of a row");
  const int h = blockIdx.y, t = blockIdx.x, k2 = threadIdx.x;
  const bool self = t == 0 || t == M1 / 2;
  const int pk = t * M2 + k2;
  const int k = t + M1 * k2;
  const int km = M - k;                                       // in [1, M]
  const int pm = big_pos<LOG2M>(km & (M - 1));
  // cs_{M-k} = (cos, sin)(pi - pi k/M) = (-cos, sin)(pi k/M)
  const float2 ck = cs[k], cm = make_float2(-ck.x, ck.y);
  float2 sk = make_float2(0.f, 0.f), sm = sk;
  // four batch rows per round, all their loads issued before the products
  for (int b0 = 0; b0 < batch; b0 += 4) {
    float2 uk[4], um[4], gk[4], gm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = b0 + i < batch ? b0 + i : batch - 1;
      const size_t r = ((size_t)h * batch + b) * M;
      uk[i] = Zu[r + pk];
      um[i] = Zu[r + pm];
      gk[i] = Zg[r + pk];
      gm[i] = Zg[r + pm];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (b0 + i >= batch) break;
      const float2 Uk = big_rfft_x(uk[i], um[i], ck), Gk = big_rfft_x(gk[i], gm[i], ck);
      const float2 Um = big_rfft_x(um[i], uk[i], cm), Gm = big_rfft_x(gm[i], gk[i], cm);
      sk = cadd(sk, cmul(cconj(Uk), Gk));
      sm = cadd(sm, cmul(cconj(Um), Gm));
    }
  }
  const float sc = 0.5f / (float)M;
  float2* __restrict__ Wh = W + (size_t)h * M;
  {
    const float2 e = make_float2(sk.x + sm.x, sk.y - sm.y);
    const float2 d = make_float2(sk.x - sm.x, sk.y + sm.y);
    const float2 w = cadd(e, cmul(make_float2(-ck.y, ck.x), d));
    Wh[pk] = make_float2(sc * w.x, sc * w.y);
  }
  if (!self) {
    const float2 e = make_float2(sm.x + sk.x, sm.y - sk.y);
    const float2 d = make_float2(sm.x - sk.x, sm.y + sk.y);
    const float2 w = cadd(e, cmul(make_float2(-cm.y, cm.x), d));
    Wh[pm] = make_float2(sc * w.x, sc * w.y);
  }
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
  big_cols_fwd_kernel<LOG2M><<<col_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(u, Yu, tw1, tw4,
                                                                             rows, p->H, p->batch);
  big_cols_fwd_kernel<LOG2M><<<col_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(dy, Yg, tw1, tw4,
                                                                             rows, p->H, p->batch);
  big_rows_kernel<LOG2M, false><<<rows_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(Yu, Yu, tw2,
                                                                                tw4, rows);
  big_rows_kernel<LOG2M, false><<<rows_blocks<LOG2M>(rows), kBigThreads, 0, s>>>(Yg, Yg, tw2,
                                                                                tw4, rows);
  float2* Wb = wat<float2>(ws, p->off_khat);
  big_corr_kernel<LOG2M><<<dim3(S::M1 / 2 + 1, p->H), kBigThreads, 0, s>>>(Yu, Yg, Wb, cs,
                                                                           p->batch);
  // inverse: rows then columns, the first M/2 outputs as (c_2n, c_2n+1)
  float* out = dK ? dK : wat<float>(ws, p->off_kbuf);
  big_rows_kernel<LOG2M, true><<<rows_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(Wb, Yu, tw2, tw4,
                                                                               p->H);
  big_cols_inv_kernel<LOG2M, 0><<<col_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
      Yu, out, tw1, p->H, p->H, 1, 1.0f);
  if (dD) big_first_col_kernel<<<(p->H + 255) / 256, 256, 0, s>>>(out, dD, p->H, p->L);
}

template <int LOG2M>
static void big_ghat(const s4dplr_plan* p, const float* dK, float2* ghat, unsigned char* ws,
                     hipStream_t s) {
  using S = BigShape<LOG2M>;
  float2* Y = wat<float2>(ws, p->off_big);
  big_cols_fwd_kernel<LOG2M><<<col_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
      dK, Y, wat<const float2>(ws, p->off_tw1), wat<const float2>(ws, p->off_tw4), p->H, p->H, 1);
  big_rows_kernel<LOG2M, false><<<rows_blocks<LOG2M>(p->H), kBigThreads, 0, s>>>(
      Y, Y, wat<const float2>(ws, p->off_tw2), wat<const float2>(ws, p->off_tw4), p->H);
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
