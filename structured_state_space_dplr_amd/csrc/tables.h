// The plan's table region as formulas: the frequency nodes tan(pi l / L), the
// two-float nodes of rank > 1 plans, (cos, sin)(pi j / L), and the FFT
// twiddles of the transform sizes the plan uses, each computed in fp64 and
// rounded once to fp32.  One entry per call, so the same code fills the
// tables on the device (the no-allocation path) and is checked on the host
// against the plan's own tables.  The frequency nodes follow "The S4 kernel,
// from scratch", section 4 (g(z) = (2/dt)(1 - z)/(1 + z) at the roots of
// unity is i (2/dt) tan(pi l / L)).
#pragma once

#include <cmath>

#include "fft_sched.h"

namespace s4 {

struct TableSpec {
  float* tan;
  float* tan2;      // NULL unless rank > 1
  float* cs;
  float* tw_a;      // L <= 16384: twiddles of L-point transforms; else of L/256 points
  float* tw_b;      // L <= 16384: of L/2-point transforms; else of 256 points
  float* tw4;       // L >= 32768: W_L^b (b < 256), then W_L^(256 a) (a < 256); else NULL
  float* tw_c;      // L >= 32768: twiddles of L/512-point transforms; else NULL
  int L, log2a, log2b, log2c;
};

constexpr double kTablePi = 3.14159265358979323846;

S4_HD inline long table_entries(const TableSpec& a) {
  return 2L * a.L + (a.L + 1) + fft_tw_size(a.log2a) + fft_tw_size(a.log2b) +
         (a.tw4 ? 512 + fft_tw_size(a.log2c) : 0);
}

// entry e of the pass twiddle table of a 2^log2n-point transform: pass p >= 1
// holds W_{ns R}^{(r k) mod (ns R)} at k R + r, k < ns = 16^p, r < R
S4_HD inline void table_twiddle(float* t, int log2n, int e) {
  int p = 1;
  while (p + 1 < fft_num_passes(log2n) && e >= fft_tw_offset(log2n, p + 1)) ++p;
  const int i = e - fft_tw_offset(log2n, p);
  const int R = 1 << fft_radix_log(log2n, p);
  const int k = i / R, r = i - k * R;
  const long span = (long)(1 << fft_ns_log(log2n, p)) * R;
  const long m = ((long)r * k) % span;
  const double ang = -2.0 * kTablePi * (double)m / (double)span;
  t[2 * e + 0] = (float)cos(ang);
  t[2 * e + 1] = (float)sin(ang);
}

// entry g of the concatenation tan | tan2 | cs | tw_a | tw_b | tw4 | tw_c
S4_HD inline void table_entry(const TableSpec& a, long g) {
  const int L = a.L;
  if (g < L) {
    const int l = (int)g;
    a.tan[l] = (2 * l == L) ? 0.0f : (float)tan(kTablePi * (double)l / (double)L);
    return;
  }
  g -= L;
  if (g < L) {
    if (a.tan2) {
      const int l = (int)g;
      const double t = (2 * l == L) ? 0.0 : tan(kTablePi * (double)l / (double)L);
      const float hi = (float)t;
      a.tan2[2 * l + 0] = hi;
      a.tan2[2 * l + 1] = (float)(t - (double)hi);
    }
    return;
  }
  g -= L;
  if (g <= L) {
    const int j = (int)g;
    const double x = kTablePi * (double)j / (double)L;
    float c = (float)cos(x), sn = (float)sin(x);
    if (j == L) sn = 0.0f;          // sin(pi) exactly
    if (2 * j == L) c = 0.0f;       // cos(pi/2) exactly
    a.cs[2 * j + 0] = c;
    a.cs[2 * j + 1] = sn;
    return;
  }
  g -= L + 1;
  const int na = fft_tw_size(a.log2a), nb = fft_tw_size(a.log2b);
  if (g < na) {
    table_twiddle(a.tw_a, a.log2a, (int)g);
    return;
  }
  g -= na;
  if (g < nb) {
    table_twiddle(a.tw_b, a.log2b, (int)g);
    return;
  }
  g -= nb;
  if (g < 512) {
    const int q = (int)g;
    const long m = q < 256 ? q : 256L * (q - 256);
    const double ang = -2.0 * kTablePi * (double)(m % L) / (double)L;
    a.tw4[2 * q + 0] = (float)cos(ang);
    a.tw4[2 * q + 1] = (float)sin(ang);
    return;
  }
  g -= 512;
  table_twiddle(a.tw_c, a.log2c, (int)g);
}

}  // namespace s4
