// Host side of libs4dplr: argument validation, plans, workspace layout, the
// fp64 constant tables, and the order of kernel launches.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "fft_sched.h"
#include "internal.h"
#include "s4dplr.h"
#include "tables.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(long v) {
  int r = 0;
  while ((1L << r) < v) ++r;
  return r;
}

s4dplr_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return S4DPLR_ERR_HIP;
}

// The kernels read and write complex values and pairs of real samples as
// 8-byte words, so every device buffer must be 8-byte aligned (NULL passes).
template <typename... Ts>
static bool misaligned(const Ts*... ps) {
  return ((ps != nullptr && (reinterpret_cast<uintptr_t>(ps) & 7u) != 0) || ...);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Twiddles of the workgroup FFT of 2^log2n points, pass by pass, as the
// schedule in fft_sched.h lays them out: W_{Ns R}^{r k} = e^{-2 pi i r k/(Ns R)}.
void fft_twiddles(int log2n, float* out) {
  const int P = s4::fft_num_passes(log2n);
  for (int p = 1; p < P; ++p) {
    const int ns = 1 << s4::fft_ns_log(log2n, p);
    const int R = 1 << s4::fft_radix_log(log2n, p);
    const long span = (long)ns * R;
    float* t = out + 2 * s4::fft_tw_offset(log2n, p);
    for (int k = 0; k < ns; ++k)
      for (int r = 0; r < R; ++r) {
        const long m = ((long)r * k) % span;
        const double ang = -2.0 * M_PI * (double)m / (double)span;
        t[2 * (k * R + r) + 0] = (float)std::cos(ang);
        t[2 * (k * R + r) + 1] = (float)std::sin(ang);
      }
  }
}

bool valid_plan(const s4dplr_plan* p) { return p != nullptr; }

}  // namespace

namespace s4 {

TableSpec plan_table_spec(const s4dplr_plan* p, unsigned char* w) {
  const bool lds = p->log2L <= S4DPLR_LDS_MAX_LOG2L;
  TableSpec a;
  a.tan = reinterpret_cast<float*>(w + p->off_tan);
  a.tan2 = p->rank > 1 ? reinterpret_cast<float*>(w + p->off_tan2) : nullptr;
  a.cs = reinterpret_cast<float*>(w + p->off_cs);
  a.tw_a = reinterpret_cast<float*>(w + (lds ? p->off_twL : p->off_tw1));
  a.tw_b = reinterpret_cast<float*>(w + (lds ? p->off_twH : p->off_tw2));
  a.tw4 = lds ? nullptr : reinterpret_cast<float*>(w + p->off_tw4);
  a.tw_c = lds ? nullptr : reinterpret_cast<float*>(w + p->off_tw1h);
  a.log2c = lds ? 0 : p->log2L - 9;
  a.L = p->L;
  a.log2a = lds ? p->log2L : p->log2L - 8;
  a.log2b = lds ? (p->log2L > 0 ? p->log2L - 1 : 0) : 8;
  return a;
}

void recurrent_shape(int N, long rows, int* ppl_out, int* log2g_out) {
  auto groups_log2 = [N](int ppl) {
    const int need = (N + ppl - 1) / ppl;
    int lg = 0;
    while ((1 << lg) < need) ++lg;
    return lg;
  };
  int ppl = 1;
  while (ppl < 8 && ppl < N) ppl <<= 1;
  int lg = groups_log2(ppl);
  // More lanes per sequence (fewer poles per lane) while the launch is short
  // of about two waves per SIMD (256 CUs x 4 SIMDs).
  constexpr long kTargetWaves = 2048;
  while (ppl > 1) {
    const int lg2 = groups_log2(ppl >> 1);
    if (lg2 > 5) break;
    const long waves = ((rows << lg) + 63) / 64;
    if (waves >= kTargetWaves) break;
    ppl >>= 1;
    lg = lg2;
  }
  *ppl_out = ppl;
  *log2g_out = lg;
}

}  // namespace s4

extern "C" {

int s4dplr_abi_version(void) { return S4DPLR_ABI_VERSION; }

int s4dplr_last_hip_error(void) { return g_last_hip_error; }

const char* s4dplr_status_string(s4dplr_status s) {
  switch (s) {
    case S4DPLR_OK: return "success";
    case S4DPLR_ERR_NULL: return "a required pointer is NULL";
    case S4DPLR_ERR_SHAPE: return "a size is outside the supported limits";
    case S4DPLR_ERR_WORKSPACE: return "workspace missing or not 256-byte aligned";
    case S4DPLR_ERR_UNSUPPORTED: return "unsupported flags";
    case S4DPLR_ERR_HIP: return "HIP runtime error while enqueueing";
    case S4DPLR_ERR_ALIAS: return "an output buffer overlaps an input or the workspace";
    case S4DPLR_ERR_TOO_LARGE:
      return "the plan needs more scratch than the library's static device array holds";
    case S4DPLR_ERR_ALIGN: return "a device buffer is not 8-byte aligned";
  }
  return "unknown status";
}

s4dplr_status s4dplr_plan_create(s4dplr_plan** out, int H, int N, int L, int batch,
                                 unsigned flags) {
  if (!out) return S4DPLR_ERR_NULL;
  *out = nullptr;
  if (flags & ~(S4DPLR_DIAGONAL | S4DPLR_ZOH | S4DPLR_BLOCK | S4DPLR_RANK_MASK))
    return S4DPLR_ERR_UNSUPPORTED;
  if ((flags & S4DPLR_ZOH) && !(flags & S4DPLR_DIAGONAL)) return S4DPLR_ERR_UNSUPPORTED;
  const unsigned rank_field = (flags & S4DPLR_RANK_MASK) >> S4DPLR_RANK_SHIFT;
  const int rank = rank_field ? (int)rank_field : 1;
  if (rank > 4) return S4DPLR_ERR_UNSUPPORTED;
  if (rank > 1 && (flags & S4DPLR_DIAGONAL)) return S4DPLR_ERR_UNSUPPORTED;
  const bool zoh = (flags & S4DPLR_ZOH) != 0;
  if (H < 1 || batch < 1 || N < 1 || N > 256) return S4DPLR_ERR_SHAPE;
  if (!is_pow2(L) || L < 2 || L > 65536) return S4DPLR_ERR_SHAPE;
  if ((long long)batch * H * L >= (1LL << 31)) return S4DPLR_ERR_SHAPE;
  const int log2L = ilog2(L);

  s4dplr_plan* p = new (std::nothrow) s4dplr_plan();
  if (!p) return S4DPLR_ERR_SHAPE;
  p->H = H;
  p->N = N;
  p->NP = (N + 3) / 4 * 4;
  p->L = L;
  p->log2L = log2L;
  p->batch = batch;
  p->rank = rank;
  p->flags = flags;

  // Table region.
  size_t off = 0;
  p->off_tan = off;
  off = align_up(off + sizeof(float) * L);
  p->off_tan2 = off;
  if (rank > 1) off = align_up(off + 2 * sizeof(float) * L);
  p->off_cs = off;
  off = align_up(off + 2 * sizeof(float) * (L + 1));
  const bool lds = log2L <= S4DPLR_LDS_MAX_LOG2L;
  p->off_twL = off;
  if (lds) off = align_up(off + 2 * sizeof(float) * (size_t)s4::fft_tw_size(log2L));
  p->off_twH = off;
  if (lds) off = align_up(off + 2 * sizeof(float) * (size_t)s4::fft_tw_size(log2L - 1));
  p->off_tw1 = off;
  if (!lds) off = align_up(off + 2 * sizeof(float) * (size_t)s4::fft_tw_size(log2L - 8));
  p->off_tw2 = off;
  if (!lds) off = align_up(off + 2 * sizeof(float) * (size_t)s4::fft_tw_size(8));
  p->off_tw4 = off;
  if (!lds) off = align_up(off + 2 * sizeof(float) * 512);
  p->off_tw1h = off;
  if (!lds) off = align_up(off + 2 * sizeof(float) * (size_t)s4::fft_tw_size(log2L - 9));
  p->tables_bytes = off;
  // Scratch region.
  p->off_khat = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)H * L);
  p->off_coef = off;
  off = align_up(off + sizeof(float) * 4 * (size_t)H * L);
  p->off_kbuf = off;
  if (!lds || zoh) off = align_up(off + sizeof(float) * (size_t)H * L);
  p->off_big = off;
  if (!lds) off = align_up(off + sizeof(float) * 2 * (size_t)batch * H * L);
  p->off_big2 = off;
  p->fwd_bytes = off;   // the forward pass uses nothing past this point
  if (!lds) off = align_up(off + sizeof(float) * 2 * (size_t)batch * H * L);
  p->off_rrec = off;
  off = align_up(off + sizeof(float) * 16 * (size_t)H * N);
  p->off_rchan = off;
  off = align_up(off + sizeof(float) * 4 * (size_t)H);
  // Chunked scan: when the batch * H sequences alone would give under about
  // two waves per SIMD, each sequence of L steps is cut into rnc chunks of C
  // steps (C >= 64, a power of two) so that sequences x chunks reach 16384.
  p->rchunk = 0;
  p->rnc = 0;
  {
    const long rows = (long)batch * H;
    if (N <= 64 && rows < 4096 && L >= 128) {
      int nc = 2;
      while ((long)nc * rows < 16384 && L / (2 * nc) >= 64) nc *= 2;
      p->rchunk = L / nc;
      p->rnc = nc;
    }
  }
  p->off_rpow = off;
  if (p->rchunk) off = align_up(off + sizeof(float) * 2 * (size_t)H * 64 * 64);
  p->off_rcs = off;
  if (p->rchunk) off = align_up(off + sizeof(float) * 2 * (size_t)batch * H * p->rnc * 64);
  p->off_rct = off;
  if (p->rchunk) off = align_up(off + sizeof(float) * 2 * (size_t)H * p->rchunk * N);
  p->off_bghat = off;
  off = align_up(off + sizeof(float) * 2 * (size_t)H * L);
  p->off_bpart = off;
  {
    const size_t nchunks = (L + s4::kBwdChunk - 1) / s4::kBwdChunk;
    size_t need = sizeof(double) * 10 * (size_t)H * nchunks * N;   // 5 fp64 complex per-pole sums
    if (lds) {
      // the partial spectra of the batch-row groups, plus one row for their sum
      const size_t corr = sizeof(float) * 2 *
                          (size_t)((batch + s4::kCorrRows - 1) / s4::kCorrRows + 1) * H * (L + 1);
      if (corr > need) need = corr;
    }
    if (zoh) {
      const size_t vpart = sizeof(float) * 4 * (size_t)H * nchunks * N;
      if (vpart > need) need = vpart;
    }
    off = align_up(off + need);
  }
  p->off_bz = off;
  if (flags & S4DPLR_BLOCK) off = align_up(off + sizeof(float) * (size_t)batch * H * L);
  p->off_bs = off;
  if (flags & S4DPLR_BLOCK) off = align_up(off + sizeof(float) * (size_t)batch * H * L);
  p->off_bw = off;
  if (flags & S4DPLR_BLOCK) off = align_up(off + sizeof(unsigned short) * 4 * (size_t)H * H);
  p->total = off;

  // fp64 tables, rounded once to fp32.
  p->tables.assign(p->tables_bytes, 0);
  float* tanT = reinterpret_cast<float*>(p->tables.data() + p->off_tan);
  for (int l = 0; l < L; ++l)
    tanT[l] = (2 * l == L) ? 0.0f : (float)std::tan(M_PI * (double)l / (double)L);
  if (rank > 1) {
    // the nodes as two floats: the rank-r Woodbury solve amplifies the
    // rounding of a single-float node near a sharp pole
    float* t2 = reinterpret_cast<float*>(p->tables.data() + p->off_tan2);
    for (int l = 0; l < L; ++l) {
      const double t = (2 * l == L) ? 0.0 : std::tan(M_PI * (double)l / (double)L);
      const float hi = (float)t;
      t2[2 * l + 0] = hi;
      t2[2 * l + 1] = (float)(t - (double)hi);
    }
  }
  float* cs = reinterpret_cast<float*>(p->tables.data() + p->off_cs);
  for (int j = 0; j <= L; ++j) {
    cs[2 * j + 0] = (float)std::cos(M_PI * (double)j / (double)L);
    cs[2 * j + 1] = (float)std::sin(M_PI * (double)j / (double)L);
  }
  cs[2 * L + 1] = 0.0f;      // sin(pi) exactly
  if (L % 2 == 0) cs[L + 0] = 0.0f;  // cos(pi/2) exactly, at j = L/2
  if (lds) {
    fft_twiddles(log2L, reinterpret_cast<float*>(p->tables.data() + p->off_twL));
    fft_twiddles(log2L - 1, reinterpret_cast<float*>(p->tables.data() + p->off_twH));
  } else {
    fft_twiddles(log2L - 8, reinterpret_cast<float*>(p->tables.data() + p->off_tw1));
    fft_twiddles(8, reinterpret_cast<float*>(p->tables.data() + p->off_tw2));
    fft_twiddles(log2L - 9, reinterpret_cast<float*>(p->tables.data() + p->off_tw1h));
    float* t4 = reinterpret_cast<float*>(p->tables.data() + p->off_tw4);
    for (int i = 0; i < 512; ++i) {
      const long m = i < 256 ? i : 256L * (i - 256);      // W_L^m
      const double ang = -2.0 * M_PI * (double)(m % L) / (double)L;
      t4[2 * i + 0] = (float)std::cos(ang);
      t4[2 * i + 1] = (float)std::sin(ang);
    }
  }
  *out = p;
  return S4DPLR_OK;
}

void s4dplr_plan_destroy(s4dplr_plan* p) { delete p; }

s4dplr_status s4dplr_plan_workspace_bytes(const s4dplr_plan* p, size_t* bytes) {
  if (!valid_plan(p) || !bytes) return S4DPLR_ERR_NULL;
  *bytes = p->total;
  return S4DPLR_OK;
}

static s4dplr_status check_ws(const void* ws) {
  if (!ws) return S4DPLR_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return S4DPLR_ERR_WORKSPACE;
  return S4DPLR_OK;
}

s4dplr_status s4dplr_plan_init(const s4dplr_plan* p, void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  hipError_t e = hipMemcpyAsync(ws, p->tables.data(), p->tables_bytes, hipMemcpyHostToDevice,
                                stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

static s4dplr_status check_params(const s4dplr_plan* p, const float* lambda, const float* P,
                                  const float* B, const float* C, const float* dt) {
  if (!lambda || !B || !C || !dt) return S4DPLR_ERR_NULL;
  if (!(p->flags & S4DPLR_DIAGONAL) && !P) return S4DPLR_ERR_NULL;
  return S4DPLR_OK;
}

s4dplr_status s4dplr_kernel_gen(const s4dplr_plan* p, const float* lambda, const float* P,
                                const float* Q, const float* B, const float* C,
                                const float* dt, float* K, void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!K) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  if (overlaps(K, kb, ws, p->total)) return S4DPLR_ERR_ALIAS;
  if (misaligned(lambda, P, Q, B, C, dt, K)) return S4DPLR_ERR_ALIGN;
  unsigned char* w = static_cast<unsigned char*>(ws);
  hipError_t e;
  if ((e = s4::launch_kernel_gen(p, lambda, P, Q, B, C, dt, nullptr, K, w, stream)) != hipSuccess)
    return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_generating_function(const s4dplr_plan* p, const float* lambda,
                                         const float* P, const float* Q, const float* B,
                                         const float* C, const float* dt, float* khat, void* ws,
                                         hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!khat) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  if (p->flags & S4DPLR_ZOH) return S4DPLR_ERR_UNSUPPORTED;
  const size_t kb = 2 * sizeof(float) * (size_t)p->H * p->L;
  const size_t cb = 2 * sizeof(float) * (size_t)p->H * p->N;
  const size_t rb = cb * (size_t)p->rank;   // P and Q: [H][rank][N] complex
  const size_t hb = sizeof(float) * (size_t)p->H;
  if (overlaps(khat, kb, ws, p->total) || overlaps(khat, kb, lambda, cb) ||
      overlaps(khat, kb, P, rb) || overlaps(khat, kb, Q, rb) || overlaps(khat, kb, B, cb) ||
      overlaps(khat, kb, C, cb) || overlaps(khat, kb, dt, hb))
    return S4DPLR_ERR_ALIAS;
  if (misaligned(lambda, P, Q, B, C, dt, khat)) return S4DPLR_ERR_ALIGN;
  hipError_t e = s4::launch_generating_function(p, lambda, P, Q, B, C, dt, khat,
                                                static_cast<unsigned char*>(ws), stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_conv_fwd(const s4dplr_plan* p, const float* u, const float* K,
                              const float* D, float* y, void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (!u || !K || !y) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  if (overlaps(y, ub, u, ub) || overlaps(y, ub, K, kb) || overlaps(y, ub, ws, p->total))
    return S4DPLR_ERR_ALIAS;
  if (misaligned(u, K, D, y)) return S4DPLR_ERR_ALIGN;
  unsigned char* w = static_cast<unsigned char*>(ws);
  hipError_t e;
  if ((e = s4::launch_spectrum_from_time(p, K, D, w, stream, 0)) != hipSuccess) return hip_fail(e);
  if ((e = s4::launch_conv(p, u, y, w, stream)) != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_forward(const s4dplr_plan* p, const float* lambda, const float* P,
                             const float* Q, const float* B, const float* C, const float* dt,
                             const float* D, const float* u, float* K, float* y, void* ws,
                             hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!u || !y) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  if (overlaps(y, ub, u, ub) || overlaps(y, ub, ws, p->total)) return S4DPLR_ERR_ALIAS;
  if (K && (overlaps(K, kb, u, ub) || overlaps(K, kb, y, ub) || overlaps(K, kb, ws, p->total)))
    return S4DPLR_ERR_ALIAS;
  if (misaligned(lambda, P, Q, B, C, dt, D, u, K, y)) return S4DPLR_ERR_ALIGN;
  unsigned char* w = static_cast<unsigned char*>(ws);
  hipError_t e;
  if ((e = s4::launch_kernel_gen(p, lambda, P, Q, B, C, dt, D, K, w, stream)) != hipSuccess)
    return hip_fail(e);
  if ((e = s4::launch_conv(p, u, y, w, stream)) != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_forward_noalloc(const s4dplr_plan* p, const float* lambda, const float* P,
                                     const float* Q, const float* B, const float* C,
                                     const float* dt, const float* D, const float* u, float* K,
                                     float* y, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!u || !y) return S4DPLR_ERR_NULL;
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  if (overlaps(y, ub, u, ub)) return S4DPLR_ERR_ALIAS;
  if (K && (overlaps(K, kb, u, ub) || overlaps(K, kb, y, ub))) return S4DPLR_ERR_ALIAS;
  if (misaligned(lambda, P, Q, B, C, dt, D, u, K, y)) return S4DPLR_ERR_ALIGN;
  if (p->fwd_bytes > s4::noalloc_scratch_bytes()) return S4DPLR_ERR_TOO_LARGE;
  unsigned char* w = nullptr;
  hipError_t e = s4::noalloc_scratch(&w);
  if (e != hipSuccess) return hip_fail(e);
  // the array keeps whatever the last call on this device left in it: the
  // tables of this plan are computed into it again by every call, on the
  // device (no copy from host memory)
  if ((e = s4::launch_plan_tables(p, w, stream)) != hipSuccess) return hip_fail(e);
  if ((e = s4::launch_kernel_gen(p, lambda, P, Q, B, C, dt, D, K, w, stream)) != hipSuccess)
    return hip_fail(e);
  if ((e = s4::launch_conv(p, u, y, w, stream)) != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_conv_apply(const s4dplr_plan* p, const float* u, float* y, void* ws,
                                hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (!u || !y) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  if (overlaps(y, ub, u, ub) || overlaps(y, ub, ws, p->total)) return S4DPLR_ERR_ALIAS;
  if (misaligned(u, y)) return S4DPLR_ERR_ALIGN;
  hipError_t e = s4::launch_conv(p, u, y, static_cast<unsigned char*>(ws), stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_recurrent_prepare(const s4dplr_plan* p, const float* lambda,
                                       const float* P, const float* Q, const float* B,
                                       const float* C, const float* dt, void* ws,
                                       hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (s4dplr_status st = check_ws(ws)) return st;
  if (p->rank > 1) return S4DPLR_ERR_UNSUPPORTED;   // the O(N) step is rank 1
  if (misaligned(lambda, P, Q, B, C, dt)) return S4DPLR_ERR_ALIGN;
  hipError_t e = s4::launch_recurrent_prepare(p, lambda, P, Q, B, C, dt,
                                              static_cast<unsigned char*>(ws), stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_recurrent_scan(const s4dplr_plan* p, const float* D, const float* u, int T,
                                    float* state, float* y, void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (T < 0) return S4DPLR_ERR_SHAPE;
  const long long rows = (long long)p->batch * p->H;
  if (rows * T >= (1LL << 31)) return S4DPLR_ERR_SHAPE;
  if (!state) return S4DPLR_ERR_NULL;
  if (T > 0 && (!u || !y)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t ub = sizeof(float) * (size_t)rows * T;
  const size_t sb = sizeof(float) * 2 * (size_t)rows * p->N;
  if (overlaps(y, ub, u, ub) || overlaps(y, ub, state, sb) || overlaps(y, ub, ws, p->total) ||
      overlaps(state, sb, u, ub) || overlaps(state, sb, ws, p->total))
    return S4DPLR_ERR_ALIAS;
  if (misaligned(D, u, state, y)) return S4DPLR_ERR_ALIGN;
  if (T == 0) return S4DPLR_OK;
  hipError_t e = s4::launch_recurrent_scan(p, D, u, state, y, T,
                                           static_cast<unsigned char*>(ws), stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_conv_bwd(const s4dplr_plan* p, const float* u, const float* K,
                              const float* D, const float* dy, float* du, float* dK, float* dD,
                              void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (!dy) return S4DPLR_ERR_NULL;
  if (du && !K) return S4DPLR_ERR_NULL;
  if ((dK || dD) && !u) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  const size_t db = sizeof(float) * (size_t)p->H;
  if (du && (overlaps(du, ub, dy, ub) || overlaps(du, ub, u, ub) || overlaps(du, ub, K, kb) ||
             overlaps(du, ub, D, db) || overlaps(du, ub, ws, p->total)))
    return S4DPLR_ERR_ALIAS;
  if (dK && (overlaps(dK, kb, dy, ub) || overlaps(dK, kb, u, ub) || overlaps(dK, kb, du, ub) ||
             overlaps(dK, kb, K, kb) || overlaps(dK, kb, ws, p->total)))
    return S4DPLR_ERR_ALIAS;
  if (dD && (overlaps(dD, db, dy, ub) || overlaps(dD, db, u, ub) || overlaps(dD, db, du, ub) ||
             overlaps(dD, db, dK, kb) || overlaps(dD, db, ws, p->total)))
    return S4DPLR_ERR_ALIAS;
  if (misaligned(u, K, D, dy, du, dK, dD)) return S4DPLR_ERR_ALIGN;
  unsigned char* w = static_cast<unsigned char*>(ws);
  hipError_t e;
  if (du) {
    if ((e = s4::launch_spectrum_from_time(p, K, D, w, stream, 1)) != hipSuccess) return hip_fail(e);
    if ((e = s4::launch_conv(p, dy, du, w, stream)) != hipSuccess) return hip_fail(e);
  }
  if (dK || dD) {
    if ((e = s4::launch_corr(p, u, dy, dK, dD, w, stream)) != hipSuccess) return hip_fail(e);
  }
  return S4DPLR_OK;
}

s4dplr_status s4dplr_kernel_gen_bwd(const s4dplr_plan* p, const float* lambda, const float* P,
                                    const float* Q, const float* B, const float* C,
                                    const float* dt, const float* dK, float* dlambda, float* dP,
                                    float* dQ, float* dB, float* dC, float* ddt, void* ws,
                                    hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!dK) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  if (p->rank > 1) return S4DPLR_ERR_UNSUPPORTED;   // gradients are built for rank 1
  const bool zoh = (p->flags & S4DPLR_ZOH) != 0;
  const bool diag = (p->flags & S4DPLR_DIAGONAL) != 0;
  if (diag) dP = dQ = nullptr;
  if (!Q) dQ = nullptr;
  const size_t cb = sizeof(float) * 2 * (size_t)p->H * p->N;
  const size_t hb = sizeof(float) * (size_t)p->H;
  const size_t kb = sizeof(float) * (size_t)p->H * p->L;
  // every output is disjoint from every input, from the workspace and from the other outputs
  const void* ins[] = {lambda, P, Q, B, C, dK, dt};
  const size_t inb[] = {cb, cb, cb, cb, cb, kb, hb};
  void* outs[] = {dlambda, dP, dQ, dB, dC, ddt};
  const size_t outb[] = {cb, cb, cb, cb, cb, hb};
  for (int i = 0; i < 6; ++i) {
    if (!outs[i]) continue;
    if (overlaps(outs[i], outb[i], ws, p->total)) return S4DPLR_ERR_ALIAS;
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], outb[i], ins[j], inb[j])) return S4DPLR_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outb[i], outs[j], outb[j])) return S4DPLR_ERR_ALIAS;
  }
  if (misaligned(lambda, P, Q, B, C, dt, dK) || misaligned(dlambda, dP, dQ, dB, dC, ddt))
    return S4DPLR_ERR_ALIGN;
  hipError_t e = zoh ? s4::launch_vandermonde_bwd(p, lambda, B, C, dt, dK, dlambda, dB, dC, ddt,
                                                  static_cast<unsigned char*>(ws), stream)
                     : s4::launch_kernel_gen_bwd(p, lambda, P, Q, B, C, dt, dK, dlambda, dP, dQ,
                                                 dB, dC, ddt, static_cast<unsigned char*>(ws),
                                                 stream);
  if (e != hipSuccess) return hip_fail(e);
  return S4DPLR_OK;
}

s4dplr_status s4dplr_block_forward(const s4dplr_plan* p, const float* x, const float* gamma,
                                   const float* beta, const float* lambda, const float* P,
                                   const float* Q, const float* B, const float* C,
                                   const float* dt, const float* D, const float* W,
                                   const float* bias, float* out, void* ws, hipStream_t stream) {
  if (!valid_plan(p)) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_params(p, lambda, P, B, C, dt)) return st;
  if (!x || !gamma || !beta || !W || !bias || !out) return S4DPLR_ERR_NULL;
  if (s4dplr_status st = check_ws(ws)) return st;
  if (!(p->flags & S4DPLR_BLOCK)) return S4DPLR_ERR_UNSUPPORTED;
  if (p->batch > 65535) return S4DPLR_ERR_SHAPE;   // one grid row per batch row
  const size_t ub = sizeof(float) * (size_t)p->batch * p->H * p->L;
  const size_t hb = sizeof(float) * (size_t)p->H;
  const size_t cb = 2 * sizeof(float) * (size_t)p->H * p->N;
  const size_t wb = 2 * sizeof(float) * (size_t)p->H * p->H;
  if (out != x && overlaps(out, ub, x, ub)) return S4DPLR_ERR_ALIAS;
  const size_t rb = cb * (size_t)p->rank;   // P and Q: [H][rank][N] complex
  const void* ins[] = {gamma, beta, lambda, P, Q, B, C, dt, D, W, bias};
  const size_t inb[] = {hb, hb, cb, rb, rb, cb, cb, hb, hb, wb, 2 * hb};
  for (int i = 0; i < 11; ++i)
    if (overlaps(out, ub, ins[i], inb[i])) return S4DPLR_ERR_ALIAS;
  if (overlaps(out, ub, ws, p->total) || overlaps(x, ub, ws, p->total)) return S4DPLR_ERR_ALIAS;
  if (misaligned(x, gamma, beta, lambda, P, Q, B, C, dt, D, W, bias, out))
    return S4DPLR_ERR_ALIGN;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* z = reinterpret_cast<float*>(w + p->off_bz);
  float* sv = reinterpret_cast<float*>(w + p->off_bs);
  hipError_t e;
  if ((e = s4::launch_layer_norm(p, x, gamma, beta, z, stream)) != hipSuccess) return hip_fail(e);
  if ((e = s4::launch_kernel_gen(p, lambda, P, Q, B, C, dt, D, nullptr, w, stream)) != hipSuccess)
    return hip_fail(e);
  if ((e = s4::launch_conv(p, z, sv, w, stream)) != hipSuccess) return hip_fail(e);
  if ((e = s4::launch_block_epilogue(p, x, sv, W, bias, out, w, stream)) != hipSuccess)
    return hip_fail(e);
  return S4DPLR_OK;
}

}  // extern "C"
