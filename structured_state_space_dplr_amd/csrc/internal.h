// Internal plan structure and kernel launchers of libs4dplr.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "s4dplr.h"

// Largest L handled by the single-workgroup (LDS-resident) kernels; longer
// sequences use the multi-pass path.
#define S4DPLR_LDS_MAX_LOG2L 14

struct s4dplr_plan {
  int H, N, NP, L, log2L, batch;   // NP: N rounded up to the Cauchy loop unroll (4)
  int rank;                        // columns of the low-rank factors P, Q (1 .. 4)
  unsigned flags;
  // Workspace layout, byte offsets from the 256-byte aligned base.
  size_t off_tan;    // [L] float: tan(pi l / L), 0 at l = L/2
  size_t off_tan2;   // rank > 1: [L] float2 (hi, lo): tan(pi l / L) = hi + lo to ~48 bits
  size_t off_cs;     // [L+1] float2: (cos(pi j / L), sin(pi j / L))
  size_t off_twL;    // FFT twiddles for transforms of L points
  size_t off_twH;    // FFT twiddles for transforms of L/2 points
  size_t off_tw1;    // long path: FFT twiddles for the column transforms (L/256 points)
  size_t off_tw2;    // long path: FFT twiddles for the row transforms (256 points)
  size_t off_tw4;    // long path: [512] float2, W_L^b (b < 256) then W_L^(256 a) (a < 256)
  size_t off_tw1h;   // long path: FFT twiddles for the column transforms of L/2 points
                     // (L/512 points), the half-length inverse of stage 1
  size_t tables_bytes;
  size_t off_khat;   // [H][L] float2: generating function at the roots of unity
  size_t off_coef;   // [H][L] float4: spectral weights (alpha, beta) of bin j
  size_t off_kbuf;   // [H][L] float time-domain kernel when not written out (long path, ZOH)
  size_t off_big;    // long path: [batch*H][L] float2 intermediate rows
  size_t off_big2;   // long path, backward: a second [batch*H][L] float2 buffer
  size_t off_rrec;   // recurrent view: [H][N] x 4 float4 per-pole step records
  size_t off_rchan;  // recurrent view: [H] float4 per-channel sums (S1, S2)
  int rchunk;        // recurrent view: chunk length C of the chunked scan (0: whole sequences)
  int rnc;           // recurrent view: chunks per sequence the chunk-state buffer holds
  size_t off_rpow;   // recurrent view, chunked: [H][64][64] float2 A-bar^C
  size_t off_rcs;    // recurrent view, chunked: [batch*H][rnc][64] float2 chunk states
  size_t off_rct;    // recurrent view, chunked: [H][C][N] float2 rows C A-bar^tau, tau < C
  // Backward pass:
  size_t off_bghat;  // [H][L] float2: FFT_L(dK) / L
  size_t off_bpart;  // partial sums: correlation spectra [ceil(B/kCorrRows) + 1][H][L+1] float2,
                     // or per-pole sums [H][ceil(L/kBwdChunk)][N] x 5 fp64 complex
  size_t off_bz;     // block (S4DPLR_BLOCK): [batch][H][L] float normalized input
  size_t off_bs;     // block (S4DPLR_BLOCK): [batch][H][L] float layer output
  size_t off_bw;     // block (S4DPLR_BLOCK): [2][2H][H] bf16: W split into hi and lo parts
  size_t fwd_bytes;  // prefix of the workspace the forward pass touches (tables .. off_big2)
  size_t total;
  std::vector<unsigned char> tables;  // exact bytes of the table region
};

namespace s4 {

constexpr int kCorrRows = 4;     // batch rows per block of the dK correlation
constexpr int kBwdChunk = 256;   // frequencies per block of the per-pole backward sums

bool lds_path(const s4dplr_plan* p);

// Stage 1: the time-domain kernel K (written to Kout when not null) and the
// convolution weights of the spectrum of (K + D delta) padded to 2L (D may be
// null) in the workspace.
hipError_t launch_kernel_gen(const s4dplr_plan* p, const float* lam, const float* P,
                             const float* Q, const float* B, const float* C, const float* dt,
                             const float* D, float* Kout, unsigned char* ws, hipStream_t s);
// The generating function at the L roots of unity into khat [H][L], natural
// order.
hipError_t launch_generating_function(const s4dplr_plan* p, const float* lam, const float* P,
                                      const float* Q, const float* B, const float* C,
                                      const float* dt, float* khat, unsigned char* ws,
                                      hipStream_t s);
// The convolution weights from a given time-domain kernel; with conj set, the
// weights of the correlation with (K + D delta) instead (the input gradient).
hipError_t launch_spectrum_from_time(const s4dplr_plan* p, const float* Ktime, const float* D,
                                     unsigned char* ws, hipStream_t s, int conj);
hipError_t launch_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                       hipStream_t s);
// Long sequences (log2 L = 15, 16): four-step transforms through the workspace.
// Without Ktime the workspace's generating-function region is the input: K-hat
// (L points, four-step order) or, with `half`, the L/2-point spectrum Y of the
// packed kernel that the rank-1 Cauchy kernel writes for this path.
hipError_t launch_big_kspec(const s4dplr_plan* p, const float* Ktime, const float* D,
                            float* Kout, unsigned char* ws, hipStream_t s, int conj, bool half);
hipError_t launch_big_conv(const s4dplr_plan* p, const float* u, float* y, unsigned char* ws,
                           hipStream_t s);
// Long path backward: dK, dD of the convolution, and Ghat = FFT_L(dK) / L into
// the workspace.
hipError_t launch_big_corr(const s4dplr_plan* p, const float* u, const float* dy, float* dK,
                           float* dD, unsigned char* ws, hipStream_t s);
hipError_t launch_big_ghat(const s4dplr_plan* p, const float* dK, unsigned char* ws,
                           hipStream_t s);

// The library's own device scratch for s4dplr_forward_noalloc: its size, and
// its address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
// The plan's table region computed on the device into w (noalloc.hip).
hipError_t launch_plan_tables(const s4dplr_plan* p, unsigned char* w, hipStream_t s);
// Where the entries of the plan's tables go in a buffer laid out like the
// workspace (tables.h); defined in api.cpp.
struct TableSpec;
TableSpec plan_table_spec(const s4dplr_plan* p, unsigned char* w);
hipError_t noalloc_scratch(unsigned char** out);

// Recurrent view: per-pole step records from the parameters, then T steps of
// every (batch, channel) sequence from the carried state.
hipError_t launch_recurrent_prepare(const s4dplr_plan* p, const float* lam, const float* P,
                                    const float* Q, const float* B, const float* C,
                                    const float* dt, unsigned char* ws, hipStream_t s);
hipError_t launch_recurrent_scan(const s4dplr_plan* p, const float* D, const float* u,
                                 float* state, float* y, int T, unsigned char* ws,
                                 hipStream_t s);
// Backward pass.  dK (may be null) and dD (may be null) of the convolution:
// the batch sum of the correlation of dy with u.
hipError_t launch_corr(const s4dplr_plan* p, const float* u, const float* dy, float* dK,
                       float* dD, unsigned char* ws, hipStream_t s);
// Parameter gradients of kernel generation from dK (each output may be null).
hipError_t launch_kernel_gen_bwd(const s4dplr_plan* p, const float* lam, const float* P,
                                 const float* Q, const float* B, const float* C, const float* dt,
                                 const float* dK, float* dlam, float* dP, float* dQ, float* dB,
                                 float* dC, float* ddt, unsigned char* ws, hipStream_t s);
// Zero-order hold, diagonal: the Vandermonde kernel K [H][L] (all L), and its
// parameter gradients from dK (outputs may be null).
hipError_t launch_vandermonde(const s4dplr_plan* p, const float* lam, const float* B,
                              const float* C, const float* dt, float* K, hipStream_t s);
hipError_t launch_vandermonde_bwd(const s4dplr_plan* p, const float* lam, const float* B,
                                  const float* C, const float* dt, const float* dK, float* dlam,
                                  float* dB, float* dC, float* ddt, unsigned char* ws,
                                  hipStream_t s);
// The block: layer norm over channels into z, and the fused GLU projection
// with bias and residual.
hipError_t launch_layer_norm(const s4dplr_plan* p, const float* x, const float* gamma,
                             const float* beta, float* z, hipStream_t s);
hipError_t launch_block_epilogue(const s4dplr_plan* p, const float* x, const float* s,
                                 const float* W, const float* bias, float* out,
                                 unsigned char* ws, hipStream_t st);
// Work split of the scan: poles per lane (1, 2, 4 or 8) and log2 of the lanes
// per sequence (0..5), chosen from N and the number of sequences.
void recurrent_shape(int N, long rows, int* ppl, int* log2g);

}  // namespace s4
