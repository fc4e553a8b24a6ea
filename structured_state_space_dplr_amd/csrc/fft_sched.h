// Pass schedule of the workgroup FFTs, shared by the host (which builds the
// twiddle tables in fp64) and the device (which consumes them).
//
// A transform of n = 2^log2n points is done as Stockham autosort passes of
// radix 16, with one shorter pass (radix 2, 4 or 8) last when log2n is not a
// multiple of 4.  Each thread owns E = min(16, n) points, so n/E threads work
// on one transform.  Pass p has span Ns = 16^p; its twiddles are
// W_{Ns R}^{r k} for k < Ns, r < R, stored at table[offset(p) + k*R + r].
#pragma once

#if defined(__HIPCC__)
#define S4_HD __host__ __device__
#else
#define S4_HD
#endif

namespace s4 {

S4_HD constexpr int fft_elems_log(int log2n) { return log2n < 4 ? log2n : 4; }
S4_HD constexpr int fft_num_passes(int log2n) { return (log2n + 3) / 4; }
S4_HD constexpr int fft_radix_log(int log2n, int p) {
  return (log2n - 4 * p) >= 4 ? 4 : (log2n - 4 * p);
}
S4_HD constexpr int fft_ns_log(int /*log2n*/, int p) { return 4 * p; }

// Twiddle entries of pass p (pass 0 needs none).
S4_HD constexpr int fft_tw_entries(int log2n, int p) {
  return p == 0 ? 0 : (1 << (fft_ns_log(log2n, p) + fft_radix_log(log2n, p)));
}
S4_HD constexpr int fft_tw_offset(int log2n, int p) {
  int off = 0;
  for (int q = 0; q < p; ++q) off += fft_tw_entries(log2n, q);
  return off;
}
S4_HD constexpr int fft_tw_size(int log2n) {
  return fft_tw_offset(log2n, fft_num_passes(log2n));
}

// Padded LDS index: one spare slot every 16 points spreads the strided
// stores of the early passes over the LDS banks.
S4_HD constexpr int lds_pad(int i) { return i + (i >> 4); }
S4_HD constexpr int lds_padded_size(int n) { return n + (n >> 4) + 1; }

}  // namespace s4
