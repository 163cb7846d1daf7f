// Host arithmetic of plan construction (declarations and citations in rd_host.hpp).
#include "rd_host.hpp"

#include <algorithm>
#include <cmath>
#include <utility>

namespace rdf {
namespace host {

std::vector<rd_c64> roots_table(int N) {
  std::vector<rd_c64> t(static_cast<size_t>(N > 0 ? N : 0));
  for (int k = 0; k < N; ++k) {
    const double a = kTwoPi * double(k) / double(N);
    t[size_t(k)] = rd_c64{float(std::cos(a)), float(-std::sin(a))};
  }
  return t;
}

namespace {
// the replica's samples h[n], n < L
void replica(const rd_params& p, int L, std::vector<double>* hr, std::vector<double>* hi) {
  const double Kr = p.bandwidth_hz / p.pulse_s;
  hr->assign(size_t(L), 0.0);
  hi->assign(size_t(L), 0.0);
  for (int n = 0; n < L; ++n) {
    const double t = double(n) / p.fs_hz - p.pulse_s / 2.0;
    double w = 1.0;
    if (p.range_window == RD_WINDOW_HAMMING && L > 1) w = 0.54 - 0.46 * std::cos(kTwoPi * n / (L - 1));
    const double ph = M_PI * Kr * t * t;
    (*hr)[size_t(n)] = w * std::cos(ph);
    (*hi)[size_t(n)] = w * std::sin(ph);
  }
}
}  // namespace

std::vector<rd_c64> matched_filter(const rd_params& p, int L) {
  const int Nr = p.Nr;
  std::vector<double> hr, hi;
  replica(p, L, &hr, &hi);
  std::vector<double> c(static_cast<size_t>(Nr)), s(static_cast<size_t>(Nr));
  for (int m = 0; m < Nr; ++m) {
    c[size_t(m)] = std::cos(kTwoPi * m / Nr);
    s[size_t(m)] = std::sin(kTwoPi * m / Nr);
  }
  std::vector<rd_c64> H(static_cast<size_t>(Nr));
  for (int k = 0; k < Nr; ++k) {
    double re = 0.0, im = 0.0;
    int64_t idx = 0;  // (k * n) mod Nr
    for (int n = 0; n < L; ++n) {
      // h[n] e^{-j 2 pi idx / Nr}
      re += hr[size_t(n)] * c[size_t(idx)] + hi[size_t(n)] * s[size_t(idx)];
      im += hi[size_t(n)] * c[size_t(idx)] - hr[size_t(n)] * s[size_t(idx)];
      idx += k;
      if (idx >= Nr) idx -= Nr;
    }
    H[size_t(k)] = rd_c64{float(re / Nr), float(-im / Nr)};  // conjugate, 1/Nr
  }
  return H;
}

void fft_pow2(std::vector<double>& re, std::vector<double>& im) {
  const size_t n = re.size();
  for (size_t i = 1, j = 0; i < n; ++i) {
    size_t bit = n >> 1;
    for (; j & bit; bit >>= 1) j ^= bit;
    j ^= bit;
    if (i < j) {
      std::swap(re[i], re[j]);
      std::swap(im[i], im[j]);
    }
  }
  for (size_t len = 2; len <= n; len <<= 1) {
    const size_t half = len / 2;
    for (size_t k = 0; k < half; ++k) {
      const double a = -kTwoPi * double(k) / double(len);
      const double wr = std::cos(a), wi = std::sin(a);
      for (size_t b = 0; b < n; b += len) {
        const size_t u = b + k, v = u + half;
        const double xr = re[v] * wr - im[v] * wi, xi = re[v] * wi + im[v] * wr;
        re[v] = re[u] - xr;
        im[v] = im[u] - xi;
        re[u] += xr;
        im[u] += xi;
      }
    }
  }
}

// Range compression of a line of any length N as one zero-padded circular convolution of length
// M >= N + L - 1 (L = replica length).  The length-N circular correlation
//   rc[n] = sum_{i < L} x[(n + i) mod N] conj(h[i])
// reads x[0 .. N + L - 2] of the periodically extended line; with g[k] = conj(h[L - 1 - k]) for
// k < L (zero up to M), the linear convolution of that extended line with g holds rc[n] at
// n + L - 1, and a length-M circular convolution aliases nothing onto [L - 1, N + L - 1) when
// M >= N + L - 1.
std::vector<rd_c64> padded_filter(const rd_params& p, int L, int M) {
  std::vector<double> hr, hi;
  replica(p, L, &hr, &hi);
  std::vector<double> re(static_cast<size_t>(M), 0.0), im(static_cast<size_t>(M), 0.0);
  for (int n = 0; n < L; ++n) {
    re[size_t(L - 1 - n)] = hr[size_t(n)];
    im[size_t(L - 1 - n)] = -hi[size_t(n)];
  }
  fft_pow2(re, im);
  std::vector<rd_c64> out(static_cast<size_t>(M));
  for (int k = 0; k < M; ++k) out[size_t(k)] = rd_c64{float(re[size_t(k)] / M), float(im[size_t(k)] / M)};
  return out;
}

std::vector<rd_c64> bluestein_spectra(int na, int m, int ca, int cb) {
  std::vector<rd_c64> out(size_t(2) * size_t(m));
  for (int d = 0; d < 2; ++d) {
    const double sign = d == 0 ? -1.0 : 1.0;
    std::vector<double> re(static_cast<size_t>(m), 0.0), im(static_cast<size_t>(m), 0.0);
    for (int n = 0; n < na; ++n) {
      const int64_t q = (int64_t(n) * n) % (2 * int64_t(na));
      const double ph = -sign * M_PI * double(q) / double(na);
      re[size_t(n)] = std::cos(ph);
      im[size_t(n)] = std::sin(ph);
      if (n > 0) {
        re[size_t(m - n)] = re[size_t(n)];
        im[size_t(m - n)] = im[size_t(n)];
      }
    }
    fft_pow2(re, im);
    for (int r = 0; r < m; ++r) {
      const int bin = r / cb + ca * (r % cb);
      out[size_t(d) * size_t(m) + size_t(r)] = rd_c64{float(re[size_t(bin)] / m), float(im[size_t(bin)] / m)};
    }
  }
  return out;
}

double bessel_i0(double z) {
  const double y = 0.25 * z * z;
  double term = 1.0, sum = 1.0;
  for (int m = 1; m < 200 && term > 1e-18 * sum; ++m) {
    term *= y / (double(m) * double(m));
    sum += term;
  }
  return sum;
}

// Each b_j is interpolated at kRcmcDeg + 1 Chebyshev points of [0, 1] and expanded in monomials
// of x = f - 1/2; only taps j = 0, -1, -2, -3 are fitted, their even and odd parts serving the
// mirrored taps too.
void rcmc_weight_polys(double beta, RcmcPoly* out) {
  constexpr int D = kRcmcDeg, M = D + 1;
  const double half = kRcmcTaps / 2.0;
  const double i0b = bessel_i0(beta);
  for (int q = 0; q < kRcmcTaps / 2; ++q) {
    const int j = -q;
    auto b = [&](double f) {
      const double tt = f - j;
      const double a = 1.0 - (tt / half) * (tt / half);
      double v = bessel_i0(beta * std::sqrt(a > 0 ? a : 0.0)) / i0b;
      for (int i = -(kRcmcTaps / 2 - 1); i <= kRcmcTaps / 2; ++i)
        if (i != j) v *= (f - i);
      return (j & 1) ? -v : v;
    };
    double cheb[M] = {};
    for (int k = 0; k < M; ++k) {
      double acc = 0.0;
      for (int i = 0; i < M; ++i) {
        const double th = M_PI * (i + 0.5) / M;
        acc += b(0.5 + 0.5 * std::cos(th)) * std::cos(k * th);
      }
      cheb[k] = acc * 2.0 / M;
    }
    cheb[0] *= 0.5;
    // sum_k cheb[k] T_k(u) -> monomials in u, then u = 2x
    double mono[M] = {}, tkm1[M] = {}, tk[M] = {};
    tkm1[0] = 1.0;  // T_0
    tk[1] = 1.0;    // T_1
    mono[0] += cheb[0];
    for (int m = 0; m < M; ++m) mono[m] += cheb[1] * tk[m];
    for (int k = 2; k < M; ++k) {
      double tn[M] = {};
      for (int m = 0; m < M; ++m) {
        if (m > 0) tn[m] += 2.0 * tk[m - 1];
        tn[m] -= tkm1[m];
      }
      for (int m = 0; m < M; ++m) {
        mono[m] += cheb[k] * tn[m];
        tkm1[m] = tk[m];
        tk[m] = tn[m];
      }
    }
    double p2 = 1.0;
    for (int m = 0; m < M; ++m) {
      const double cm = mono[m] * p2;  // coefficient of x^m
      if (m % 2 == 0)
        out->even[q][m / 2] = float(cm);
      else
        out->odd[q][m / 2] = float(cm);
      p2 *= 2.0;
    }
  }
}

bool azimuth_pow2(int na) { return na >= 256 && na <= 16384 && (na & (na - 1)) == 0; }

bool azimuth_five(int na) {
  if (na <= 0 || na % 25 != 0) return false;
  const int a = na / 25;
  return a >= 16 && a <= 128 && (a & (a - 1)) == 0;
}

int bluestein_m(int na) {
  int m = 256;
  while (m < 2 * na - 1) m *= 2;
  return m;
}

void pow2_split(int n, int* a, int* b) {
  *a = 1;
  while (*a * *a * 4 <= n) *a *= 2;
  *b = n / *a;
}

int persistent_grid(int occ, int cus, int64_t lines, int lpw) {
  const int64_t l = lpw > 0 ? lpw : 1;
  const int64_t need = (lines + l - 1) / l;
  const int64_t resident = int64_t(occ > 0 ? occ : 1) * int64_t(cus > 0 ? cus : 1);
  const int64_t g = need < resident ? need : resident;
  return int(g > 0 ? g : 1);
}

bool partial_overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  const uintptr_t y = reinterpret_cast<uintptr_t>(b);
  return x != y && x < y + n && y < x + n;
}

double doppler_row_coefficients(const rd_params& p, double dr, std::vector<double>* rowc) {
  const int Na = p.Na;
  const double lam = kC / p.carrier_hz;
  rowc->assign(size_t(Na) * 4, 0.0);
  double max_shift = 0.0;
  for (int k = 0; k < Na; ++k) {
    const int kk = (k <= (Na - 1) / 2) ? k : k - Na;  // FFT bin order
    const double f = double(kk) * p.prf_hz / double(Na);
    const double u = std::pow(lam * f / (2.0 * p.velocity_mps), 2);
    const double D = std::sqrt(1.0 - u);
    const double Q = u / (D * (1.0 + D)) / dr;  // shift per metre of slant range, samples
    double* r = rowc->data() + size_t(4) * size_t(k);
    r[0] = p.range_bin0_m * Q;  // shift(n) = alpha + n beta
    r[1] = dr * Q;
    r[2] = 2.0 * D * p.range_bin0_m / lam;  // phase cycles = gamma + n delta
    r[3] = 2.0 * D * dr / lam;
    max_shift = std::max(max_shift, r[0] + double(p.Nr - 1) * r[1]);
  }
  return max_shift;
}

// The Stolt shift (sqrt(a^2 + b^2) - a) / df is largest at the lowest range frequency
// a = f0 - Fs/2 and the Doppler band edge b = c PRF / (4 V); the mapping needs a > b there.
int stolt_halo(const rd_params& p) {
  const double df = p.fs_hz / p.Nr;
  const double amin = p.carrier_hz - double(p.Nr / 2) * df;
  const double bmax = kC * p.prf_hz / (4.0 * p.velocity_mps);
  if (!(amin > bmax)) return -1;
  return int(std::floor((std::sqrt(amin * amin + bmax * bmax) - amin) / df)) + 5;
}

}  // namespace host
}  // namespace rdf
