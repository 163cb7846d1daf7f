// Host side of the C ABI declared in include/rdfocus.h: parameter validation, plan construction
// (float64 matched filter and tables, rounded to float32 once), launch sequences.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <vector>

#include "../../include/rdfocus.h"
#include "rd_host.hpp"
#include "rd_kernels.hpp"

namespace {

using rdf::host::kC;
using rdf::host::azimuth_five;
using rdf::host::azimuth_pow2;
using rdf::host::bluestein_m;
using rdf::host::partial_overlap;
using rdf::host::persistent_grid;
using rdf::host::pow2_split;
using rdf::host::roots_table;

thread_local std::string g_last_error;

rd_status fail(rd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

std::mutex g_plans_mu;
std::set<const rd_plan*> g_plans;  // live plans, so a destroyed plan is recognised

}  // namespace

struct rd_plan {
  rd_params p{};
  int device = 0;
  int cus = 0;
  int L = 0;           // replica length
  double dr = 0.0;     // range-bin spacing
  bool azimuth = false;
  const rdf::LineOps* rops = nullptr;  // range-length kernels
  const rdf::LineOps* aops = nullptr;  // azimuth-length kernels
  int rc_variant = 0;   // 0 table loads, 1 register-cached (pf)
  int pad_m = 0;        // > 0: Nr has no built transform; range compression runs as a zero-padded
                        // circular convolution of length pad_m >= Nr + L - 1 (power of two), and
                        // RCMC runs on rows of run-time length
  int rcmc_margin = 0;  // samples the RCMC kernel stages after a chunk (shifts up to margin - 5)
  int cached = 0;       // image passes use ordinary (cacheable) accesses: image fits the cache
  int rc_grid = 0;      // persistent grid of the range kernels
  int A = 0, B = 0;     // Doppler row order after the forward azimuth transform: row r holds bin
                        // r / B + A (r % B) (digit order of the two steps; A = 1, B = Na when the
                        // transform is the Bluestein form, whose output is in natural order)
  int ca = 0, cb = 0;   // the column transform steps: lengths ca (strided) and cb (block)
  int col_n = 0;        // their transform length ca cb: Na, or M for the Bluestein form
  int bs_m = 0;         // > 0: the azimuth transform is Bluestein's, through columns of length M
  float2* bs_ws = nullptr;   // [M][Nr] Bluestein workspace
  float2* bs_fb = nullptr;   // [2][M] spectra of the two chirps / M, in the column steps' row order
  float2* H = nullptr;       // [Nr] conj(FFT(h)) / Nr
  float2* tw_r = nullptr;    // [Nr] e^{-j 2 pi k / Nr}
  float2* rc_tab = nullptr;  // per-thread constants of the range kernel (null if it has none)
  float2* tw_a = nullptr;    // [Na] e^{-j 2 pi k / Na} (line-transform test hook)
  float2* tw_A = nullptr;    // [A] e^{-j 2 pi k / A}
  float2* tw_B = nullptr;    // [B] e^{-j 2 pi k / B}
  double* rowc = nullptr;    // [Na][4] RCMC shift and filter phase coefficients per Doppler bin
  float2* work = nullptr;    // [Na * Nr] workspace (stage test hook only, allocated on first use)
  rdf::AzRowConst az{};
  double rd_max_shift = 0.0;  // largest RCMC shift (samples); must stay below margin - 5
  int wk_halo = -1;     // omega-k: zero samples staged after a row (-1: geometry not supported)
  int wk_grid = 0;      // omega-k row-stage grid
  int f16_grid = 0;     // grid of the binary16-storage range kernel (0: not available)
};

namespace {

bool live_plan(const rd_plan* p) {
  std::lock_guard<std::mutex> g(g_plans_mu);
  return g_plans.count(p) != 0;
}

void free_plan(rd_plan* p) {
  (void)hipFree(p->H);
  (void)hipFree(p->tw_r);
  (void)hipFree(p->rc_tab);
  (void)hipFree(p->tw_a);
  (void)hipFree(p->tw_A);
  (void)hipFree(p->tw_B);
  (void)hipFree(p->rowc);
  (void)hipFree(p->work);
  (void)hipFree(p->bs_ws);
  (void)hipFree(p->bs_fb);
  delete p;
}

template <class T>
rd_status upload(T** dst, const std::vector<T>& src, const char* what) {
  if (hipMalloc(dst, src.size() * sizeof(T)) != hipSuccess) {
    *dst = nullptr;
    return fail(RD_ERR_OUT_OF_MEMORY, "hipMalloc of %s (%zu bytes) failed", what,
                src.size() * sizeof(T));
  }
  if (hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess)
    return fail(RD_ERR_DEVICE, "upload of %s failed", what);
  return RD_OK;
}

// host complex tables (rd_c64) into the kernels' float2 arrays: the same 8-byte layout
static_assert(sizeof(rd_c64) == sizeof(float2), "rd_c64 and float2 must share a layout");
rd_status upload(float2** dst, const std::vector<rd_c64>& src, const char* what) {
  return upload(reinterpret_cast<rd_c64**>(dst), src, what);
}

rd_status check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return RD_OK;
  return fail(RD_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
}

rd_status check_call(rd_plan* plan) {
  if (!plan || !live_plan(plan)) return fail(RD_ERR_INVALID_ARG, "null or destroyed plan");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
    return fail(RD_ERR_DEVICE, "the plan was created on device %d but device %d is current",
                plan->device, dev);
  return RD_OK;
}

// RD_DEBUG builds check each launch's geometry against the plan before launching and refuse the
// launch (RD_ERR_LAUNCH, naming the failed condition) instead of running a kernel on a shape it
// was not built for; other builds compile the checks away.
#ifdef RD_DEBUG
#define RD_EXPECT(cond)                                                                        \
  do {                                                                                         \
    if (!(cond)) return fail(RD_ERR_LAUNCH, "debug check failed (%s:%d): %s", __FILE__, __LINE__, #cond); \
  } while (0)
#else
#define RD_EXPECT(cond) \
  do {                  \
  } while (0)
#endif

bool aligned8(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// -------------------------------------------------------------------------- launch sequences
// chained: the output feeds the azimuth chain (stored cacheable where the image fits the cache)
rd_status run_range_compress(rd_plan* P, const float2* in, float2* out, bool chained, hipStream_t s) {
  RD_EXPECT(in && out && P->H && P->tw_r && P->rc_grid >= 1);
  RD_EXPECT(P->rops->n == (P->pad_m ? P->pad_m : P->p.Nr));
  RD_EXPECT(!P->pad_m || P->p.Nr + P->L - 1 <= P->pad_m);
  RD_EXPECT(P->pad_m || P->rops->rc_tab_len() == 0 || P->rc_tab);
  if (P->rc_variant == 1)
    return check_hip(P->rops->range_compress_pf(in, out, P->H, P->tw_r, P->rc_tab, P->p.Na,
                                                P->rc_grid, chained ? P->cached : 0, P->p.Nr,
                                                P->pad_m ? P->L - 1 : 0, s),
                     "range compression launch");
  return check_hip(P->rops->range_compress(in, out, P->H, P->tw_r, P->p.Na, P->rc_grid, s),
                   "range compression launch");
}

rd_status run_range_compress_f16(rd_plan* P, const void* in, void* out, bool chained, hipStream_t s) {
  RD_EXPECT(in && out && P->f16_grid >= 1 && P->rops->range_compress_f16);
  RD_EXPECT(!P->pad_m || P->p.Nr + P->L - 1 <= P->pad_m);
  return check_hip(P->rops->range_compress_f16(in, out, P->H, P->tw_r, P->rc_tab, P->p.Na, P->f16_grid,
                                               chained ? P->cached : 0, P->p.Nr, P->pad_m ? P->L - 1 : 0, s),
                   "binary16 range compression launch");
}

// Azimuth processing in place on [Na][Nr] (no corner turns):
//   forward transform, strided step (reads `src`, writes `dst`) then block step;
//   RCMC + filter per Doppler row; inverse transform, block step then strided step.
rdf::ColStep col_step(const rd_plan* P, bool forward, bool strided) {
  rdf::ColStep st{};
  st.dir = forward ? -1 : +1;
  if (strided) {
    st.L = P->ca;
    st.base_mul = 1;
    st.stride = P->cb;
    st.sets = P->cb;
    st.twiddle = forward ? 1 : 0;
  } else {
    st.L = P->cb;
    st.base_mul = P->cb;
    st.stride = 1;
    st.sets = P->ca;
    st.twiddle = forward ? 0 : 1;
  }
  return st;
}

// half: binary16 storage, each step scaled by 1 / (its length) so that no intermediate exceeds
// the largest magnitude of the step's input (the binary16 range ends at 65504)
rd_status run_col(rd_plan* P, const void* src, void* dst, bool forward, bool strided, bool half,
                  hipStream_t s) {
  rdf::ColStep st = col_step(P, forward, strided);
  RD_EXPECT(src && dst && P->ca * P->cb == P->col_n && P->col_n == (P->bs_m ? P->bs_m : P->p.Na));
  RD_EXPECT((strided ? P->tw_A : P->tw_B) && st.L * st.sets == P->col_n);
  st.half = half ? 1 : 0;
  st.scale = 1.0f / float(st.L);
  return check_hip(rdf::launch_col_fft(src, dst, strided ? P->tw_A : P->tw_B, st, P->p.Nr, P->col_n,
                                       P->cached, s),
                   "azimuth transform launch");
}

// Bluestein form of an azimuth DFT of length Na (sign -1 forward, +1 inverse unnormalised):
// X[k] = c[k] sum_m (x[m] c[m]) conj(c[k - m]) with c[n] = exp(sign j pi n^2 / Na), the sum a
// linear convolution done as a length-M circular one (M >= 2 Na - 1) by the column steps.
// half: src and dst in binary16 (the workspace stays float32) and the result scaled by 1 / Na.
rd_status run_bluestein(rd_plan* P, const void* src, void* dst, int sign, bool half, float2* W, hipStream_t s) {
  const int Na = P->p.Na, M = P->bs_m;
  const int64_t Nr = P->p.Nr;
  const int h = half ? 1 : 0;
  RD_EXPECT(src && dst && W && P->bs_fb && M >= 2 * Na - 1 && P->A == 1 && P->B == Na);
  rd_status st;
  if ((st = check_hip(rdf::launch_chirp_rows(src, W, Nr, Na, M, Na, sign, h, 0, 1.0f, s), "chirp launch")) != RD_OK)
    return st;
  if ((st = run_col(P, W, W, true, true, false, s)) != RD_OK) return st;
  if ((st = run_col(P, W, W, true, false, false, s)) != RD_OK) return st;
  if ((st = check_hip(rdf::launch_scale_rows(W, P->bs_fb + (sign < 0 ? 0 : M), Nr, M, s), "scale launch")) != RD_OK)
    return st;
  if ((st = run_col(P, W, W, false, false, false, s)) != RD_OK) return st;
  if ((st = run_col(P, W, W, false, true, false, s)) != RD_OK) return st;
  return check_hip(rdf::launch_chirp_rows(W, dst, Nr, Na, Na, Na, sign, 0, h, half ? 1.0f / float(Na) : 1.0f, s),
                   "chirp launch");
}

// The azimuth transform: src [Na][Nr] (pulses) -> dst, row r holding Doppler bin r / B + A (r % B)
// (half: binary16 storage, transform scaled by 1 / Na; ws: the Bluestein form's [M][Nr] workspace)
rd_status az_forward(rd_plan* P, const void* src, void* dst, bool half, hipStream_t s, float2* ws = nullptr) {
  if (P->bs_m) return run_bluestein(P, src, dst, -1, half, ws ? ws : P->bs_ws, s);
  rd_status st;
  if ((st = run_col(P, src, dst, true, true, half, s)) != RD_OK) return st;
  return run_col(P, dst, dst, true, false, half, s);
}

// Its inverse, in place, back to pulse order: unnormalised (1/Na is folded into the row stage),
// or with binary16 storage scaled by 1 / Na like the forward transform
rd_status az_inverse(rd_plan* P, void* io, bool half, hipStream_t s, float2* ws = nullptr) {
  if (P->bs_m) return run_bluestein(P, io, io, +1, half, ws ? ws : P->bs_ws, s);
  rd_status st;
  if ((st = run_col(P, io, io, false, false, half, s)) != RD_OK) return st;
  return run_col(P, io, io, false, true, half, s);
}

// The row stage with the constants c (rows in c's Doppler order); in place allowed
rd_status run_rows_c(rd_plan* P, const void* src, void* dst, const rdf::AzRowConst& c, bool half, hipStream_t s) {
  RD_EXPECT(src && dst && c.row && int64_t(c.A) * c.B == P->p.Na);
  RD_EXPECT(c.halo >= 0 && c.halo <= P->rcmc_margin);
  if (P->pad_m)
    return check_hip(rdf::launch_rcmc_mf_any(src, dst, c, P->p.Na, P->p.Nr, P->cached, half, s), "RCMC launch");
  return check_hip(P->rops->rcmc_mf(src, dst, c, P->p.Na, 0, P->cached, half, s), "RCMC launch");
}

// RCMC and (filter) the azimuth filter per Doppler row; half: binary16 rows, whose forward
// transform already carries 1 / Na
rd_status run_rows(rd_plan* P, const void* src, void* dst, bool filter, bool half, hipStream_t s) {
  rdf::AzRowConst c = P->az;
  c.filter = filter ? 1 : 0;
  if (half) c.inv_na = 1.0f;
  return run_rows_c(P, src, dst, c, half, s);
}

rd_status check_rcmc_margin(const rd_plan* P) {
  if (std::floor(P->rd_max_shift) + 5 > double(P->rcmc_margin))
    return fail(RD_ERR_UNSUPPORTED_LENGTH,
                "range migration of %.1f samples exceeds the %d-sample margin built for Nr=%d",
                P->rd_max_shift, P->rcmc_margin - 5, P->p.Nr);
  return RD_OK;
}

rd_status run_azimuth(rd_plan* P, const void* rc, void* img, bool half, hipStream_t s, float2* ws = nullptr) {
  // rc is read only by the first step, so img may alias it
  rd_status st;
  if ((st = az_forward(P, rc, img, half, s, ws)) != RD_OK) return st;
  if ((st = run_rows(P, img, img, true, half, s)) != RD_OK) return st;
  return az_inverse(P, img, half, s, ws);
}

// omega-k: the azimuth transform first (the 2-D transform's order is free), then one row stage
// per Doppler row, then the inverse azimuth transform; echo is read only by the first step.
// half: binary16 storage of echo, intermediates and image (the azimuth steps scaled by 1/L, the
// row stage without its 1/Na: the image divided by Na)
rd_status run_omega_k(rd_plan* plan, const void* echo, void* img, int32_t ref_bin, bool half, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  const rd_params& p = plan->p;
  if (ref_bin < 0 || ref_bin >= p.Nr) return fail(RD_ERR_INVALID_ARG, "ref_bin=%d must be in [0, Nr=%d)", ref_bin, p.Nr);
  if (!plan->rops->omega_k_rows || plan->pad_m)
    return fail(RD_ERR_UNSUPPORTED_LENGTH, "omega-k needs a built transform of length Nr=%d", p.Nr);
  if (plan->wk_halo < 0)
    return fail(RD_ERR_INVALID_ARG, "f0 - Fs/2 must exceed c PRF / (4 V) for the Stolt mapping");
  if (plan->wk_halo > plan->rops->wk_cap)
    return fail(RD_ERR_UNSUPPORTED_LENGTH, "Stolt shift of %d samples exceeds the %d-sample margin built for Nr=%d",
                plan->wk_halo - 5, plan->rops->wk_cap - 5, p.Nr);
  if (half ? !aligned4(echo) || !aligned4(img) : !aligned8(echo) || !aligned8(img))
    return fail(RD_ERR_INVALID_ARG, "echo and img must be non-NULL and %d-byte aligned", half ? 4 : 8);
  const size_t bytes = size_t(p.Na) * p.Nr * (half ? sizeof(rd_c32h) : sizeof(rd_c64));
  if (partial_overlap(echo, img, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and img overlap without being equal");
  rdf::OkConst c{};
  c.f0 = p.carrier_hz;
  c.df = p.fs_hz / p.Nr;
  c.inv_df = p.Nr / p.fs_hz;
  c.bstep = kC * p.prf_hz / (2.0 * p.velocity_mps * p.Na);
  const double r_ref = p.range_bin0_m + ref_bin * plan->dr;
  c.k1 = 2.0 * r_ref / kC;
  const double turns = c.k1 * p.carrier_hz;
  c.k0 = turns - std::floor(turns);
  c.ref = ref_bin;
  c.A = plan->A;
  c.B = plan->B;
  c.halo = plan->wk_halo;
  c.inv_na = half ? 1.0f : float(1.0 / double(p.Na));
  hipStream_t s = static_cast<hipStream_t>(stream);
  RD_EXPECT(c.halo >= 5 && c.halo <= plan->rops->wk_cap && int64_t(c.A) * c.B == p.Na && plan->wk_grid >= 1);
  if ((st = az_forward(plan, echo, img, half, s)) != RD_OK) return st;
  if ((st = check_hip(plan->rops->omega_k_rows(img, img, plan->H, plan->tw_r, c, plan->az.w, p.Na, plan->wk_grid,
                                               plan->cached, half ? 1 : 0, s),
                      "omega-k row stage launch")) != RD_OK)
    return st;
  return az_inverse(plan, img, half, s);
}

}  // namespace

// ------------------------------------------------------------------------------- static scratch
// Workspace of rd_focus_noalloc: a file-scope device array, so that the entry point allocates
// nothing.  Every GPU the library runs on holds its own copy (at its own address) until the
// process ends.  Host code never uses the array's name as an address: the device address is
// looked up once per device with hipGetSymbolAddress and passed to the kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float2 scratch[kScratchBytes / sizeof(float2)];

namespace {

std::mutex g_scratch_mu;
float2* g_scratch_ptr[64] = {};  // per device index

// Device address of `scratch` on device `dev`, which must be current (looked up on the first
// call per device).
rd_status scratch_address(int dev, float2** out) {
  if (dev < 0 || dev >= 64) return fail(RD_ERR_DEVICE, "device %d out of range for the static scratch", dev);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RD_ERR_DEVICE, "hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float2*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return RD_OK;
}

}  // namespace

extern "C" {

int rd_length_supported(int32_t n) { return rdf::line_ops(n) != nullptr ? 1 : 0; }

const char* rd_status_string(rd_status st) {
  switch (st) {
    case RD_OK: return "ok";
    case RD_ERR_INVALID_ARG: return "invalid argument";
    case RD_ERR_UNSUPPORTED_LENGTH: return "unsupported transform length";
    case RD_ERR_OUT_OF_MEMORY: return "out of device memory";
    case RD_ERR_DEVICE: return "device error";
    case RD_ERR_LAUNCH: return "kernel launch failed";
    case RD_ERR_NOT_CONFIGURED: return "azimuth processing not configured (range-only plan)";
  }
  return "unknown status";
}

const char* rd_last_error(void) { return g_last_error.c_str(); }

rd_status rd_plan_create(const rd_params* params, rd_plan** out) {
  if (!out) return fail(RD_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!params) return fail(RD_ERR_INVALID_ARG, "params is NULL");
  const rd_params p = *params;
  if (p.Na <= 0 || p.Nr <= 0) return fail(RD_ERR_INVALID_ARG, "Na=%d and Nr=%d must be > 0", p.Na, p.Nr);
  if (int64_t(p.Na) * p.Nr > (int64_t(1) << 32))
    return fail(RD_ERR_INVALID_ARG, "Na*Nr = %lld exceeds 2^32 samples", (long long)p.Na * p.Nr);
  if (!(p.pulse_s > 0) || !(p.bandwidth_hz > 0) || !(p.fs_hz > 0) || !std::isfinite(p.pulse_s) ||
      !std::isfinite(p.bandwidth_hz) || !std::isfinite(p.fs_hz))
    return fail(RD_ERR_INVALID_ARG, "pulse_s, bandwidth_hz and fs_hz must be finite and > 0");
  if (p.range_window != RD_WINDOW_RECT && p.range_window != RD_WINDOW_HAMMING)
    return fail(RD_ERR_INVALID_ARG, "range_window %d is not RD_WINDOW_RECT or RD_WINDOW_HAMMING",
                p.range_window);
  if (p.flags != 0) return fail(RD_ERR_INVALID_ARG, "flags must be 0");
  const double Lf = std::ceil(p.pulse_s * p.fs_hz - 1e-6);
  if (Lf < 1 || Lf > p.Nr)
    return fail(RD_ERR_INVALID_ARG, "replica length ceil(Tp*Fs) = %.0f must be in [1, Nr=%d]", Lf, p.Nr);
  const bool any_az = p.carrier_hz != 0 || p.prf_hz != 0 || p.velocity_mps != 0;
  const bool all_az = p.carrier_hz > 0 && p.prf_hz > 0 && p.velocity_mps > 0 &&
                      std::isfinite(p.carrier_hz) && std::isfinite(p.prf_hz) &&
                      std::isfinite(p.velocity_mps);
  if (any_az && !all_az)
    return fail(RD_ERR_INVALID_ARG,
                "carrier_hz, prf_hz, velocity_mps must all be > 0 (full chain) or all 0 (range only)");
  const rdf::LineOps* rops = rdf::line_ops(p.Nr);
  int pad_m = 0;
  if (!rops) {
    // any line length up to 8192: range compression as a zero-padded convolution of length
    // M = the smallest built power of two >= Nr + L - 1 (the azimuth steps and the RCMC take the
    // row length at run time)
    if (p.Nr > 8192) return fail(RD_ERR_UNSUPPORTED_LENGTH, "no transform of length Nr=%d is built, and Nr > 8192", p.Nr);
    pad_m = 256;
    while (pad_m < p.Nr + int(Lf) - 1) pad_m *= 2;
    rops = rdf::line_ops(pad_m);
    if (!rops || !rops->range_compress_pf) return fail(RD_ERR_UNSUPPORTED_LENGTH, "no padded transform for Nr=%d", p.Nr);
  }
  const rdf::LineOps* aops = nullptr;
  if (all_az) {
    aops = rdf::line_ops(p.Na);  // (only the line-transform test hook needs one)
    const bool bluestein = !azimuth_pow2(p.Na) && !azimuth_five(p.Na);
    if (bluestein && (p.Na < 16 || p.Na > 8192))
      return fail(RD_ERR_UNSUPPORTED_LENGTH,
                  "full-chain plans need Na a power of two in [256, 16384], 25 * 2^k in [400, 3200], or "
                  "16..8192 for the Bluestein form (Na=%d)", p.Na);
    if (int64_t(bluestein ? bluestein_m(p.Na) : p.Na) * p.Nr * 8 > int64_t(0xFFFFFFF0))
      return fail(RD_ERR_INVALID_ARG, "full-chain plans need Na*Nr*8 (M*Nr*8 for the Bluestein form) < 4 GiB");
    if (p.rcmc_taps != 8)
      return fail(RD_ERR_INVALID_ARG, "rcmc_taps=%d: only the 8-tap interpolator is built", p.rcmc_taps);
    if (!(p.kaiser_beta >= 0.0 && p.kaiser_beta <= 12.0))
      return fail(RD_ERR_INVALID_ARG, "kaiser_beta=%g must be in [0, 12]", p.kaiser_beta);
    const double lam = kC / p.carrier_hz;
    const double umax = std::pow(lam * (p.prf_hz / 2.0) / (2.0 * p.velocity_mps), 2);
    if (!(umax < 1.0))
      return fail(RD_ERR_INVALID_ARG, "Doppler band exceeds 2V/lambda ((lambda PRF / 4V)^2 = %g)", umax);
    if (!std::isfinite(p.range_bin0_m) || p.range_bin0_m <= 0)
      return fail(RD_ERR_INVALID_ARG, "range_bin0_m must be finite and > 0");
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RD_ERR_DEVICE, "no current HIP device");
  rd_plan* P = new (std::nothrow) rd_plan();
  if (!P) return fail(RD_ERR_OUT_OF_MEMORY, "host allocation failed");
  P->p = p;
  P->device = dev;
  P->L = int(Lf);
  P->dr = kC / (2.0 * p.fs_hz);
  P->azimuth = all_az;
  P->rops = rops;
  P->pad_m = pad_m;
  P->rcmc_margin = pad_m ? rdf::rcmc_any_margin() : rops->margin;
  P->aops = aops;
  if (hipDeviceGetAttribute(&P->cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    P->cus = 256;

  rd_status st = RD_OK;
  auto bail = [&](rd_status s) {
    free_plan(P);
    return s;
  };
  {
    const int n_tf = pad_m ? pad_m : p.Nr;
    const std::vector<rd_c64> Hh =
        pad_m ? rdf::host::padded_filter(p, P->L, pad_m) : rdf::host::matched_filter(p, P->L);
    const std::vector<rd_c64> roots = roots_table(n_tf);
    if ((st = upload(&P->H, Hh, "matched filter")) != RD_OK) return bail(st);
    if ((st = upload(&P->tw_r, roots, "range twiddles")) != RD_OK) return bail(st);
    if (const int n = rops->rc_tab_len(); n > 0 && !pad_m) {
      std::vector<float2> tab(static_cast<size_t>(n));
      rops->rc_tab_fill(reinterpret_cast<const float2*>(Hh.data()), reinterpret_cast<const float2*>(roots.data()), tab.data());
      if ((st = upload(&P->rc_tab, tab, "range kernel table")) != RD_OK) return bail(st);
    }
  }
  int occ_rc = 0, occ_fft = 0, occ_azc = 0;
  if (rops->occupancy(&occ_rc, &occ_fft, &occ_azc) != hipSuccess)
    return bail(fail(RD_ERR_DEVICE, "occupancy query failed"));
  P->rc_grid = persistent_grid(occ_rc, P->cus, p.Na, rops->lpw);
  // Kernel variant for range compression: RD_RC_VARIANT=table keeps twiddle/filter loads in
  // the line loop (a slower reference variant kept for measurement), otherwise the
  // register-cached kernel (pf) runs wherever it is built.
  {
    const char* v = std::getenv("RD_RC_VARIANT");
    const std::string want = v ? v : "";
    int occ = 0;
    if (rops->range_compress_pf && (want != "table" || pad_m)) {
      if (rops->occupancy_pf(&occ, pad_m ? 1 : 0) != hipSuccess)
        return bail(fail(RD_ERR_DEVICE, "occupancy query failed"));
      P->rc_variant = 1;
      P->rc_grid = persistent_grid(occ, P->cus, p.Na, rops->lpw);
    }
    if (rops->range_compress_f16) {
      int occ16 = 0;
      if (rops->occupancy_f16(&occ16, pad_m ? 1 : 0) != hipSuccess)
        return bail(fail(RD_ERR_DEVICE, "occupancy query failed"));
      P->f16_grid = persistent_grid(occ16, P->cus, p.Na, rops->lpw);
    }
    const char* g = std::getenv("RD_RC_GRID");  // workgroups of the range kernel (tuning)
    if (g && std::atoi(g) > 0) P->rc_grid = std::atoi(g);
  }

  if ((st = upload(&P->tw_a, roots_table(rdf::line_ops(p.Na) ? p.Na : 1), "azimuth twiddles")) != RD_OK)
    return bail(st);
  if (all_az) {
    const int Na = p.Na;
    // Na = A B: A the largest power of two <= sqrt(Na) for powers of two; else A = Na / 25,
    // B = 25 (both steps are built column transform lengths)
    if (azimuth_five(Na)) {
      P->ca = Na / 25;
      P->cb = 25;
      P->col_n = Na;
    } else if (azimuth_pow2(Na)) {
      pow2_split(Na, &P->ca, &P->cb);
      P->col_n = Na;
    } else {
      // Bluestein: columns of length M; the transform's output rows are in natural order
      P->bs_m = bluestein_m(Na);
      pow2_split(P->bs_m, &P->ca, &P->cb);
      P->col_n = P->bs_m;
    }
    P->A = P->bs_m ? 1 : P->ca;
    P->B = P->bs_m ? Na : P->cb;
    std::vector<double> rowc;
    const double max_shift = rdf::host::doppler_row_coefficients(p, P->dr, &rowc);
    // taps reach floor(shift) + 4 samples past the output (one more for rounding differences
    // between this bound and the kernel's float64 shift)
    // (a plan whose migration exceeds the RCMC margin still serves omega-k and back-projection;
    // the range-Doppler entry points report it)
    P->rd_max_shift = max_shift;
    P->az.halo = std::min(int(std::floor(max_shift)) + 5, P->rcmc_margin);
    // omega-k (where the geometry gives a real wavenumber at every sample)
    {
      const int halo = rdf::host::stolt_halo(p);
      if (rops->omega_k_rows && !pad_m && halo >= 0) {
        P->wk_halo = halo;
        int occ = 0;
        if (rops->occupancy_wk(&occ) != hipSuccess) return bail(fail(RD_ERR_DEVICE, "occupancy query failed"));
        P->wk_grid = persistent_grid(occ, P->cus, Na, rops->lpw);
      }
    }
    if ((st = upload(&P->tw_A, roots_table(P->ca), "azimuth step twiddles")) != RD_OK) return bail(st);
    if ((st = upload(&P->tw_B, roots_table(P->cb), "azimuth step twiddles")) != RD_OK) return bail(st);
    if (P->bs_m) {
      if ((st = upload(&P->bs_fb, rdf::host::bluestein_spectra(Na, P->bs_m, P->ca, P->cb), "Bluestein chirp spectra")) != RD_OK)
        return bail(st);
      if (hipMalloc(&P->bs_ws, size_t(P->bs_m) * size_t(p.Nr) * sizeof(float2)) != hipSuccess) {
        P->bs_ws = nullptr;
        return bail(fail(RD_ERR_OUT_OF_MEMORY, "hipMalloc of the Bluestein workspace failed"));
      }
    }
    if ((st = upload(&P->rowc, rowc, "azimuth row coefficients")) != RD_OK) return bail(st);
    P->az.row = P->rowc;
    P->az.A = P->A;
    P->az.B = P->B;
    P->az.inv_na = float(1.0 / double(Na));
    P->az.filter = 1;
    rdf::host::rcmc_weight_polys(p.kaiser_beta, &P->az.w);
    // The image passes run cacheable when the image fits well inside the 256 MB Infinity
    // Cache (RD_AZ_CACHE=0/1 overrides, for measurement).
    P->cached = int64_t(Na) * p.Nr * 8 <= (int64_t(160) << 20) ? 1 : 0;
    if (const char* ce = std::getenv("RD_AZ_CACHE")) P->cached = std::atoi(ce) ? 1 : 0;
  }
  {
    std::lock_guard<std::mutex> g(g_plans_mu);
    g_plans.insert(P);
  }
  *out = P;
  return RD_OK;
}

rd_status rd_plan_destroy(rd_plan* plan) {
  if (!plan) return RD_OK;
  {
    std::lock_guard<std::mutex> g(g_plans_mu);
    if (!g_plans.erase(plan)) return fail(RD_ERR_INVALID_ARG, "plan is not live (destroyed twice?)");
  }
  free_plan(plan);
  return RD_OK;
}

rd_status rd_range_compress(rd_plan* plan, const rd_c64* echo, rd_c64* rc, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!aligned8(echo) || !aligned8(rc)) return fail(RD_ERR_INVALID_ARG, "echo and rc must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  if (partial_overlap(echo, rc, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and rc overlap without being equal");
  return run_range_compress(plan, reinterpret_cast<const float2*>(echo),
                            reinterpret_cast<float2*>(rc), false, static_cast<hipStream_t>(stream));
}

rd_status rd_range_compress_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* rc, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (plan->f16_grid <= 0)
    return fail(RD_ERR_UNSUPPORTED_LENGTH, "no binary16 range kernel for Nr=%d", plan->p.Nr);
  if (!aligned4(echo) || !aligned4(rc)) return fail(RD_ERR_INVALID_ARG, "echo and rc must be non-NULL and 4-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c32h);
  if (partial_overlap(echo, rc, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and rc overlap without being equal");
  return run_range_compress_f16(plan, echo, rc, false, static_cast<hipStream_t>(stream));
}

rd_status rd_azimuth_focus(rd_plan* plan, const rd_c64* rc, rd_c64* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned8(rc) || !aligned8(img)) return fail(RD_ERR_INVALID_ARG, "rc and img must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  if (partial_overlap(rc, img, bytes)) return fail(RD_ERR_INVALID_ARG, "rc and img overlap without being equal");
  return run_azimuth(plan, rc, img, false, static_cast<hipStream_t>(stream));
}

rd_status rd_focus(rd_plan* plan, const rd_c64* echo, rd_c64* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned8(echo) || !aligned8(img)) return fail(RD_ERR_INVALID_ARG, "echo and img must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  if (partial_overlap(echo, img, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and img overlap without being equal");
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* I = reinterpret_cast<float2*>(img);
  st = run_range_compress(plan, reinterpret_cast<const float2*>(echo), I, true, s);
  if (st != RD_OK) return st;
  return run_azimuth(plan, I, I, false, s);
}

rd_status rd_focus_noalloc(rd_plan* plan, const rd_c64* echo, rd_c64* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned8(echo) || !aligned8(img)) return fail(RD_ERR_INVALID_ARG, "echo and img must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  if (partial_overlap(echo, img, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and img overlap without being equal");
  float2* ws = nullptr;
  if (plan->bs_m) {
    const size_t need = size_t(plan->bs_m) * size_t(plan->p.Nr) * sizeof(float2);
    if (need > kScratchBytes)
      return fail(RD_ERR_INVALID_ARG,
                  "the Bluestein workspace of this plan (%zu bytes: M=%d x Nr=%d) exceeds the %zu-byte static scratch",
                  need, plan->bs_m, plan->p.Nr, kScratchBytes);
    if ((st = scratch_address(plan->device, &ws)) != RD_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* I = reinterpret_cast<float2*>(img);
  st = run_range_compress(plan, reinterpret_cast<const float2*>(echo), I, true, s);
  if (st != RD_OK) return st;
  return run_azimuth(plan, I, I, false, s, ws);
}

rd_status rd_azimuth_focus_f16(rd_plan* plan, const rd_c32h* rc, rd_c32h* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned4(rc) || !aligned4(img)) return fail(RD_ERR_INVALID_ARG, "rc and img must be non-NULL and 4-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c32h);
  if (partial_overlap(rc, img, bytes)) return fail(RD_ERR_INVALID_ARG, "rc and img overlap without being equal");
  return run_azimuth(plan, rc, img, true, static_cast<hipStream_t>(stream));
}

rd_status rd_focus_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if (plan->f16_grid <= 0)
    return fail(RD_ERR_UNSUPPORTED_LENGTH, "no binary16 range kernel for Nr=%d", plan->p.Nr);
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned4(echo) || !aligned4(img)) return fail(RD_ERR_INVALID_ARG, "echo and img must be non-NULL and 4-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c32h);
  if (partial_overlap(echo, img, bytes)) return fail(RD_ERR_INVALID_ARG, "echo and img overlap without being equal");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_range_compress_f16(plan, echo, img, true, s)) != RD_OK) return st;
  return run_azimuth(plan, img, img, true, s);
}

rd_status rd_omega_k(rd_plan* plan, const rd_c64* echo, rd_c64* img, int32_t ref_bin, void* stream) {
  return run_omega_k(plan, echo, img, ref_bin, false, stream);
}

rd_status rd_omega_k_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* img, int32_t ref_bin, void* stream) {
  return run_omega_k(plan, echo, img, ref_bin, true, stream);
}

rd_status rd_debug_azimuth_stages(rd_plan* plan, const rd_c64* rc, rd_c64* azfft, rd_c64* rcmc,
                                  rd_c64* img, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned8(rc) || !aligned8(azfft) || !aligned8(rcmc) || !aligned8(img))
    return fail(RD_ERR_INVALID_ARG, "all buffers must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  const void* bufs[4] = {rc, azfft, rcmc, img};
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b) {
      const bool same_ok = (a == 0 && b == 3);  // img may equal rc
      const char* x = static_cast<const char*>(bufs[a]);
      const char* y = static_cast<const char*>(bufs[b]);
      const bool overlap = x < y + bytes && y < x + bytes;
      if (overlap && !(same_ok && x == y))
        return fail(RD_ERR_INVALID_ARG, "debug buffers %d and %d overlap", a, b);
    }
  if (!plan->work && hipMalloc(&plan->work, bytes) != hipSuccess) {
    plan->work = nullptr;
    return fail(RD_ERR_OUT_OF_MEMORY, "hipMalloc of the %zu-byte stage workspace failed", bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* I = reinterpret_cast<float2*>(img);
  float2* W = plan->work;
  const int64_t Nr = plan->p.Nr;
  if ((st = az_forward(plan, rc, I, false, s)) != RD_OK) return st;
  if ((st = run_rows(plan, I, W, false, false, s)) != RD_OK) return st;  // RCMC alone
  if ((st = check_hip(rdf::launch_row_unpermute(I, reinterpret_cast<float2*>(azfft), plan->A, plan->B,
                                                Nr, s), "row order launch")) != RD_OK)
    return st;
  if ((st = check_hip(rdf::launch_row_unpermute(W, reinterpret_cast<float2*>(rcmc), plan->A, plan->B,
                                                Nr, s), "row order launch")) != RD_OK)
    return st;
  if ((st = run_rows(plan, I, I, true, false, s)) != RD_OK) return st;
  return az_inverse(plan, I, false, s);
}

rd_status rd_debug_rcmc(rd_plan* plan, const rd_c64* in, rd_c64* out, int32_t filter, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "range-only plan");
  if ((st = check_rcmc_margin(plan)) != RD_OK) return st;
  if (!aligned8(in) || !aligned8(out)) return fail(RD_ERR_INVALID_ARG, "in and out must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(plan->p.Na) * plan->p.Nr * sizeof(rd_c64);
  if (partial_overlap(in, out, bytes)) return fail(RD_ERR_INVALID_ARG, "in and out overlap without being equal");
  rdf::AzRowConst c = plan->az;
  c.filter = filter ? 1 : 0;
  c.A = 1;  // row k holds Doppler bin k
  c.B = plan->p.Na;
  return run_rows_c(plan, in, out, c, false, static_cast<hipStream_t>(stream));
}

rd_status rd_debug_line_fft(rd_plan* plan, int32_t axis, int32_t inverse, const rd_c64* in,
                            rd_c64* out, int64_t lines, void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (axis != 0 && axis != 1) return fail(RD_ERR_INVALID_ARG, "axis must be 0 (Na) or 1 (Nr)");
  const int n = axis == 0 ? plan->p.Na : plan->p.Nr;
  const rdf::LineOps* ops = rdf::line_ops(n);
  if (!ops) return fail(RD_ERR_UNSUPPORTED_LENGTH, "no transform of length %d is built", n);
  if (lines < 0) return fail(RD_ERR_INVALID_ARG, "lines must be >= 0");
  if (lines == 0) return RD_OK;
  if (!aligned8(in) || !aligned8(out)) return fail(RD_ERR_INVALID_ARG, "in and out must be non-NULL and 8-byte aligned");
  if (partial_overlap(in, out, size_t(lines) * n * sizeof(rd_c64)))
    return fail(RD_ERR_INVALID_ARG, "in and out overlap without being equal");
  int occ_rc = 0, occ_fft = 0, occ_azc = 0;
  if (ops->occupancy(&occ_rc, &occ_fft, &occ_azc) != hipSuccess)
    return fail(RD_ERR_DEVICE, "occupancy query failed");
  const int grid = persistent_grid(occ_fft, plan->cus, lines, ops->lpw);
  const float2* tw = axis == 0 ? plan->tw_a : plan->tw_r;
  return check_hip(ops->fft(reinterpret_cast<const float2*>(in), reinterpret_cast<float2*>(out), tw,
                            lines, inverse ? 1 : 0, inverse ? float(1.0 / n) : 1.0f, grid,
                            static_cast<hipStream_t>(stream)),
                   "line FFT launch");
}

rd_status rd_backproject(rd_plan* plan, const rd_c64* rc, rd_c64* img, const rd_bp_grid* grid,
                         void* stream) {
  rd_status st = check_call(plan);
  if (st != RD_OK) return st;
  if (!plan->azimuth) return fail(RD_ERR_NOT_CONFIGURED, "back-projection needs a full-chain plan (carrier, PRF, velocity)");
  if (!grid) return fail(RD_ERR_INVALID_ARG, "grid must not be NULL");
  const rd_bp_grid g = *grid;
  if (g.nx < 0 || g.ny < 0) return fail(RD_ERR_INVALID_ARG, "nx and ny must be >= 0");
  if (g.nx == 0 || g.ny == 0) return RD_OK;
  if (g.nx > 65535 * 4) return fail(RD_ERR_INVALID_ARG, "nx=%d exceeds %d", g.nx, 65535 * 4);
  if (!std::isfinite(g.x0_m) || !std::isfinite(g.dx_m) || !std::isfinite(g.r0_m) || !std::isfinite(g.dr_m))
    return fail(RD_ERR_INVALID_ARG, "grid origin and spacings must be finite");
  if (!(g.r0_m > 0.0) || !(g.r0_m + double(g.ny - 1) * g.dr_m > 0.0))
    return fail(RD_ERR_INVALID_ARG, "pixel slant ranges must be > 0");
  if (!aligned8(rc) || !aligned8(img)) return fail(RD_ERR_INVALID_ARG, "rc and img must be non-NULL and 8-byte aligned");
  const size_t in_bytes = size_t(plan->p.Na) * size_t(plan->p.Nr) * sizeof(rd_c64);
  const size_t out_bytes = size_t(g.nx) * size_t(g.ny) * sizeof(rd_c64);
  const uintptr_t a = reinterpret_cast<uintptr_t>(rc), b = reinterpret_cast<uintptr_t>(img);
  if (a < b + out_bytes && b < a + in_bytes) return fail(RD_ERR_INVALID_ARG, "rc and img overlap");
  rdf::BpConst c{};
  c.nx = g.nx;
  c.ny = g.ny;
  c.Na = plan->p.Na;
  c.Nr = plan->p.Nr;
  c.x0 = g.x0_m;
  c.dx = g.dx_m;
  c.r0 = g.r0_m;
  c.drp = g.dr_m;
  c.step = plan->p.velocity_mps / plan->p.prf_hz;
  c.rb0 = plan->p.range_bin0_m;
  c.inv_dr = 1.0 / plan->dr;
  c.two_over_lam = 2.0 * plan->p.carrier_hz / kC;
  // Hardware sin/cos (turns in, ~1e-6 absolute error) unless RD_BP_SINCOS=accurate selects the
  // library sincospi (a measurement variant).
  const char* v = std::getenv("RD_BP_SINCOS");
  const int native = (v && std::string(v) == "accurate") ? 0 : 1;
  RD_EXPECT(c.nx > 0 && c.ny > 0 && c.Na > 0 && c.Nr > 0 && std::isfinite(c.step) && c.inv_dr > 0);
  return check_hip(rdf::launch_backproject(reinterpret_cast<const float2*>(rc), reinterpret_cast<float2*>(img),
                                           c, native, static_cast<hipStream_t>(stream)),
                   "back-projection launch");
}

rd_status rd_corner_turn(const rd_c64* in, rd_c64* out, int64_t rows, int64_t cols,
                         void* stream) {
  if (rows < 0 || cols < 0) return fail(RD_ERR_INVALID_ARG, "rows and cols must be >= 0");
  if (rows == 0 || cols == 0) return RD_OK;
  if (cols > (int64_t(1) << 40) / rows)
    return fail(RD_ERR_INVALID_ARG, "rows * cols exceeds 2^40 elements");
  if (((rows + 63) / 64) * ((cols + 63) / 64) > int64_t(0x7fffffff))
    return fail(RD_ERR_INVALID_ARG, "more than 2^31 - 1 tiles of 64 x 64");
  if (!aligned8(in) || !aligned8(out)) return fail(RD_ERR_INVALID_ARG, "in and out must be non-NULL and 8-byte aligned");
  const size_t bytes = size_t(rows) * size_t(cols) * sizeof(rd_c64);
  const uintptr_t a = reinterpret_cast<uintptr_t>(in), b = reinterpret_cast<uintptr_t>(out);
  if (a < b + bytes && b < a + bytes) return fail(RD_ERR_INVALID_ARG, "in and out overlap (the corner turn is out of place)");
  // arrays beyond the 256 MB Infinity Cache stream with the non-temporal hint
  const int streaming = bytes > (size_t(160) << 20) ? 1 : 0;
  return check_hip(rdf::launch_corner_turn(reinterpret_cast<const float2*>(in), reinterpret_cast<float2*>(out),
                                           rows, cols, streaming, static_cast<hipStream_t>(stream)),
                   "corner turn launch");
}

}  // extern "C"
