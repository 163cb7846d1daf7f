// Launch interface of the focusing kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rd_host.hpp"

namespace rdf {

// RCMC + azimuth filter on one Doppler row k of the [Na][Nr] array (range along the row):
//   Delta(n) = alpha_k + n beta_k   (= R(n) (1/D_k - 1) / dr, samples)
//   T[n]     = sum_{j=-3..4} w_j(f) S[floor(n + Delta) + j],  f = frac(n + Delta)
//   out[n]   = T[n] exp(+j 2 pi (gamma_k + n delta_k)) / Na   (= 4 pi R(n) D_k / lambda)
// w_j(f): the interpolator weights of RcmcPoly (rd_host.hpp), from polynomials fitted on the host.
struct AzRowConst {
  const double* row;   // [Na][4]: alpha, beta, gamma, delta per Doppler bin (FFT order)
  int A, B;            // Na = A B; row r holds Doppler bin (r / B) + A (r % B)
  float inv_na;
  int filter;          // 0: RCMC only (no filter, no 1/Na), for the stage test hook
  int halo;            // samples staged after a chunk: floor(max shift) + 5 <= margin
  RcmcPoly w;
};

// omega-k: range FFT, range filter x reference function, Stolt interpolation and range IFFT of
// one Doppler row (the row's azimuth transform done before, its inverse after).  Frequencies
// in Hz, times in s; range bin js (signed, FFT order) lies at js df.
struct OkConst {
  double f0;      // carrier
  double df;      // range-frequency bin spacing Fs / Nr
  double inv_df;  // Nr / Fs
  double bstep;   // c PRF / (2 V Na): Doppler bin kk (signed) has b = kk bstep
  double k1;      // 2 Rref / c
  double k0;      // fractional part of 2 Rref f0 / c (turns)
  int ref;        // reference range bin: the line is read rotated by ref and stored back
  int A, B;       // Na = A B; row r holds Doppler bin (r / B) + A (r % B)
  int halo;       // zero samples staged after the row: floor(max Stolt shift) + 5 <= wk_cap
  float inv_na;   // 1 / Na (the inverse azimuth transform's scale)
};

struct LineOps {
  int n;       // transform length
  int wg;      // threads per workgroup
  int lpw;     // lines per workgroup
  hipError_t (*range_compress)(const float2* in, float2* out, const float2* H, const float2* tw,
                               int64_t lines, int grid, hipStream_t s);
  hipError_t (*fft)(const float2* in, float2* out, const float2* tw, int64_t lines, int inverse,
                    float scale, int grid, hipStream_t s);
  // workgroups of each persistent kernel that fit on one CU
  hipError_t (*occupancy)(int* rc, int* fft, int* azc);
  // register-cached, prefetching range compression (nullptr where the forward and inverse
  // radix lists differ) and its occupancy
  // (cached: ordinary stores, for output that the next pass re-reads from the cache; else
  // non-temporal stores)
  // n_line: samples per line in memory; n_line == n is the transform itself, a shorter
  // n_line (skip < n_line, n_line + skip <= n) is the fast-convolution form: lines extended
  // periodically by skip samples and zero-padded to n, H the plan's padded filter, and the
  // output window [skip, skip + n_line)
  hipError_t (*range_compress_pf)(const float2* in, float2* out, const float2* H,
                                  const float2* tw, const float2* tab, int64_t lines, int grid,
                                  int cached, int n_line, int skip, hipStream_t s);
  hipError_t (*occupancy_pf)(int* rc, int pad);
  // Per-thread constant table of the register-cached kernel (twiddles and filter in the order
  // each thread holds them, so that a workgroup loads it with contiguous wave accesses):
  // element count (0: the kernel reads H and tw directly) and host-side fill from the
  // natural-order filter H[n] and roots e^{-j 2 pi k / n} (a permutation, no arithmetic).
  int (*rc_tab_len)();
  void (*rc_tab_fill)(const float2* H, const float2* roots, float2* out);
  // RCMC + azimuth filter over rows of this length (in == out allowed; grid 0 = one row per
  // thread group, the row's chunks in order); margin = samples staged after a chunk, so the largest shift the kernel
  // accepts is margin - 5
  // (half: binary16 rows, 4 bytes a sample, float32 arithmetic)
  hipError_t (*rcmc_mf)(const void* in, void* out, const AzRowConst& c, int64_t rows, int grid,
                        int cached, int half, hipStream_t s);
  int margin;
  // omega-k row stage over `rows` Doppler rows (in == out allowed); wk_cap = the largest halo
  // the kernel stages, occupancy_wk = its workgroups per CU
  // (half: binary16 rows, float32 arithmetic)
  hipError_t (*omega_k_rows)(const void* in, void* out, const float2* H, const float2* tw,
                             const OkConst& c, const RcmcPoly& w, int64_t rows, int grid,
                             int cached, int half, hipStream_t s);
  hipError_t (*occupancy_wk)(int* wgs);
  int wk_cap;
  // range compression with binary16 line storage (4 bytes a sample in and out, float32
  // arithmetic; tab, cached, n_line and skip as for range_compress_pf) and its occupancy
  hipError_t (*range_compress_f16)(const void* in, void* out, const float2* H, const float2* tw,
                                   const float2* tab, int64_t lines, int grid, int cached, int n_line,
                                   int skip, hipStream_t s);
  hipError_t (*occupancy_f16)(int* wgs, int pad);
};

// nullptr if the length has no built transform
const LineOps* line_ops(int n);

// RCMC + azimuth filter over rows of any length n (512-sample chunks; halo up to
// rcmc_any_margin(), so shifts up to rcmc_any_margin() - 5); in == out allowed; half as for
// LineOps::rcmc_mf
hipError_t launch_rcmc_mf_any(const void* in, void* out, const AzRowConst& c, int64_t rows, int n,
                              int cached, int half, hipStream_t s);
int rcmc_any_margin();

// In-place four-step azimuth transforms on [rows][cols]; see rd_kernels.hip.
struct ColStep {
  int L;          // transform length of this step
  int dir;        // -1 forward, +1 inverse
  int base_mul;   // first row of set g is g * base_mul
  int stride;     // row stride within a set
  int sets;       // number of row sets
  int twiddle;    // apply the inter-step twiddle W_Na^{dir g t}
  int half;       // binary16 storage (4 bytes a sample), float32 arithmetic
  float scale;    // binary16 storage only: every output times scale
};
// cached: ordinary loads and stores (image held by the Infinity Cache), else non-temporal
hipError_t launch_col_fft(const void* in, void* out, const float2* tw_L, const ColStep& st,
                          int64_t cols, int na, int cached, hipStream_t s);

// Back-projection constants (see k_backproject): pixel (i, j) lies at along-track x0 + i dx and
// closest-approach slant range r0 + j drp; pulse m at along-track m * step (= V / PRF).
struct BpConst {
  int nx, ny, Na, Nr;
  double x0, dx, r0, drp;
  double step;          // V / PRF
  double rb0, inv_dr;   // slant range of bin 0, 1 / bin spacing
  double two_over_lam;  // 2 / lambda: turns of the two-way carrier phase per metre
};
// img[i][j] for i < nx, j < ny from rc [Na][Nr]; hipErrorInvalidValue if the grid does not fit
hipError_t launch_backproject(const float2* rc, float2* img, const BpConst& c, int native_sincos,
                              hipStream_t s);

// out[c][r] = in[r][c] for a row-major [rows][cols] array (streaming: non-temporal accesses);
// hipErrorInvalidValue beyond 2^31 - 1 tiles of 64 x 64
hipError_t launch_corner_turn(const float2* in, float2* out, int64_t rows, int64_t cols,
                              int streaming, hipStream_t s);

// out[k] = in[(k % A) B + k / A] for rows of `cols` samples: Doppler-digit row order to natural
// Bluestein row passes (see rd_kernels.hip): chirp multiply with zero fill, and a per-row scale
// hin / hout: binary16 input / output (not both); scale multiplies every output
hipError_t launch_chirp_rows(const void* in, void* out, int64_t cols, int rows_in, int rows_out, int na,
                             int sign, int hin, int hout, float scale, hipStream_t s);
hipError_t launch_scale_rows(float2* io, const float2* f, int64_t cols, int rows, hipStream_t s);
hipError_t launch_row_unpermute(const float2* in, float2* out, int A, int B, int64_t cols,
                                hipStream_t s);

}  // namespace rdf
