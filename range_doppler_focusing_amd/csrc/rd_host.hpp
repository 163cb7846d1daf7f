// Host arithmetic of plan construction: the float64 tables the kernels read (matched filter,
// roots, Bluestein chirp spectra, RCMC interpolator polynomials, per-Doppler coefficients) and
// the integer geometry of the launches.  No HIP types or calls, so the same source also builds
// with a plain host compiler (and its address / undefined-behaviour sanitizers) for checks that
// need no GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/rdfocus.h"

namespace rdf {

// RCMC interpolator (nxmr.cn/news/101525 §2.2: interpolation along the migrated slant range;
// an 8-tap Kaiser-windowed sinc).  For fraction f in [0, 1) an output reads samples
// floor(x) - 3 .. floor(x) + 4 with weights w_j = b_j(f) / sum_i b_i(f), where
//   b_j(f) = (-1)^j K(f - j) prod_{i != j} (f - i)
// is sinc(f - j) K(f - j) times a factor common to all taps (pi prod_i (f - i) / sin(pi f)),
// smooth in f.  By the symmetry b_{1-j}(x) = b_j(-x) with x = f - 1/2, taps j = -q and 1 + q
// (q = 0..3) come from one degree-7 polynomial p_q(x) = E_q(x^2) + x O_q(x^2):
// b_{-q}(x) = E + x O and b_{1+q}(x) = E - x O.  (Degree 7 keeps the normalised weights within
// 1e-7 of the windowed sinc for beta = 2.5 and 5e-7 for beta = 8; degree 8 cost one more FMA
// per tap pair, degree 6 is off by up to 7e-6.)
constexpr int kRcmcTaps = 8;
constexpr int kRcmcDeg = 7;
constexpr int kRcmcEven = kRcmcDeg / 2 + 1;    // coefficients of E_q
constexpr int kRcmcOdd = (kRcmcDeg + 1) / 2;   // coefficients of O_q
struct RcmcPoly {
  float even[kRcmcTaps / 2][kRcmcEven];  // E_q, ascending powers of x^2
  float odd[kRcmcTaps / 2][kRcmcOdd];    // O_q, ascending powers of x^2
};

namespace host {

constexpr double kC = 299792458.0;
constexpr double kTwoPi = 6.283185307179586476925286766559;

// e^{-j 2 pi k / N}, k < N, evaluated in float64 and rounded once
std::vector<rd_c64> roots_table(int N);

// H[k] = conj(sum_{n < L} h[n] e^{-j 2 pi k n / Nr}) / Nr with the replica
// h[n] = w[n] exp(j pi Kr (n/Fs - Tp/2)^2) (nxmr.cn/news/101525 §2.1: the chirp spectrum
// precomputed on the host), by direct summation in float64, rounded to float32 once.
std::vector<rd_c64> matched_filter(const rd_params& p, int L);

// In-place radix-2 float64 FFT (forward, e^{-j...}) of a power-of-two length.
void fft_pow2(std::vector<double>& re, std::vector<double>& im);

// FFT_M(g) / M of g[k] = conj(h[L - 1 - k]) (k < L, zero up to M): the filter of a line of any
// length N <= M - L + 1 range-compressed as one zero-padded circular convolution of length M.
std::vector<rd_c64> padded_filter(const rd_params& p, int L, int M);

// Spectra / M of the Bluestein chirps b[n] = exp(-sign j pi n^2 / Na) (|n| < Na, circular in
// M), forward (sign -1) then inverse (sign +1), each in the column steps' output row order
// (row r holds bin r / cb + ca (r % cb)).  2 M values.
std::vector<rd_c64> bluestein_spectra(int na, int m, int ca, int cb);

// Modified Bessel function of the first kind, order 0 (power series).
double bessel_i0(double z);

// Degree-kRcmcDeg Chebyshev fits of the interpolator taps b_j for Kaiser parameter beta, as monomials.
void rcmc_weight_polys(double beta, RcmcPoly* out);

// Azimuth lengths of full-chain plans.
bool azimuth_pow2(int na);          // a power of two in [256, 16384]
bool azimuth_five(int na);          // 25 * 2^k with 2^k in [16, 128]
int bluestein_m(int na);            // power of two >= 2 Na - 1, at least 256
void pow2_split(int n, int* a, int* b);  // n = a b, a the largest power of two <= sqrt(n)

// Workgroups of a persistent kernel over `lines` lines: all resident slots, or fewer if there
// are fewer line groups.
int persistent_grid(int occ, int cus, int64_t lines, int lpw);

// [a, a + n) and [b, b + n) overlap but are not the same buffer.
bool partial_overlap(const void* a, const void* b, size_t n);

// Per-Doppler-bin RCMC shift and azimuth filter phase (nxmr.cn/news/101525 §2.2), for bins in
// FFT order: rowc[4k..4k+3] = alpha, beta, gamma, delta with shift(n) = alpha + n beta samples
// and phase(n) = gamma + n delta cycles.  Returns the largest shift over the row.
double doppler_row_coefficients(const rd_params& p, double dr, std::vector<double>* rowc);

// omega-k: samples staged past a row for the Stolt mapping's largest shift, or -1 when the
// geometry has no real wavenumber at every sample.
int stolt_halo(const rd_params& p);

}  // namespace host
}  // namespace rdf
