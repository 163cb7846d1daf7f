// Launch interface of the focusing kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rdf {

// Azimuth matched filter exp(+j 4 pi R(n) D_k / lambda) / Na, R(n) = rb0 + n dr.
struct AzFilterConst {
  double rb0;             // slant range of range bin 0
  double dr;              // range-bin spacing
  double two_over_lambda; // 2 / lambda: cycles of the two-way path per metre
  float inv_na;           // 1 / Na (inverse-transform scale)
};

// RCMC: output bin n of Doppler bin k reads x = n + R(n) Q_k with Q_k = u/(D(1+D))/dr;
// weights are the Kaiser-windowed sinc, evaluated as (-1)^j I0-series(y_j) / (f - j) and
// normalised by their sum (the common factor sin(pi f)/(pi I0(beta)) cancels).
constexpr int kRcmcMaxTerms = 32;
struct RcmcConst {
  double rb0;
  double dr;
  float y0;          // (beta/2)^2
  float y1;          // (beta/2)^2 / (taps/2)^2:  y_j = y0 - y1 t_j^2
  int nterm;         // series terms kept
  float coef[kRcmcMaxTerms];  // 1/(m!)^2, highest order first
};

struct LineOps {
  int n;       // transform length
  int wg;      // threads per workgroup
  int lpw;     // lines per workgroup
  hipError_t (*range_compress)(const float2* in, float2* out, const float2* H, const float2* tw,
                               int64_t lines, int grid, hipStream_t s);
  hipError_t (*fft)(const float2* in, float2* out, const float2* tw, int64_t lines, int inverse,
                    float scale, int grid, hipStream_t s);
  hipError_t (*az_compress)(const float2* in, float2* out, const float2* tw, const double* Dk,
                            AzFilterConst c, int64_t lines, int grid, hipStream_t s);
  // workgroups of each persistent kernel that fit on one CU
  hipError_t (*occupancy)(int* rc, int* fft, int* azc);
  // register-cached, prefetching range compression (nullptr where the forward and inverse
  // radix lists differ) and its occupancy
  hipError_t (*range_compress_pf)(const float2* in, float2* out, const float2* H,
                                  const float2* tw, int64_t lines, int grid, hipStream_t s);
  hipError_t (*occupancy_pf)(int* rc);
  // two lines per trip with alternating register sets (one line per workgroup only)
  hipError_t (*range_compress_pf2)(const float2* in, float2* out, const float2* H,
                                   const float2* tw, int64_t lines, int grid, hipStream_t s);
  hipError_t (*occupancy_pf2)(int* rc);
};

// nullptr if the length has no built transform
const LineOps* line_ops(int n);

// out[c][r] = in[r][c] for an R x C row-major complex array
hipError_t launch_corner_turn(const float2* in, float2* out, int64_t rows, int64_t cols,
                              hipStream_t s);

// 8-tap RCMC on the corner-turned layout: in/out [Nr][Na] (row = range bin, column = Doppler)
hipError_t launch_rcmc8(const float2* in, float2* out, const double* Qk, const RcmcConst& c,
                        int Nr, int Na, hipStream_t s);

}  // namespace rdf
