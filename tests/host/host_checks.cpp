// Checks of the library's host arithmetic (rd_host.cpp), built by a plain host compiler with the
// address and undefined-behaviour sanitizers: every table a plan uploads is compared with an
// independent computation (a naive DFT, Parseval's identity, a Bluestein transform run through
// the table, the C++ library's Bessel function, the interpolator's zero crossings), and the
// launch-geometry helpers with their invariants.  Prints "host checks passed" and exits 0, or
// names the first failed check and exits 1.
#include <cmath>
#include <complex>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "rd_host.hpp"

using cd = std::complex<double>;
using namespace rdf::host;

static int g_fail = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::printf("FAILED %s:%d: ", __FILE__, __LINE__);   \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
      ++g_fail;                                            \
    }                                                      \
  } while (0)

static std::vector<cd> naive_dft(const std::vector<cd>& x, int sign) {
  const size_t n = x.size();
  std::vector<cd> y(n);
  for (size_t k = 0; k < n; ++k) {
    cd acc = 0;
    for (size_t m = 0; m < n; ++m) {
      const double a = sign * kTwoPi * double((k * m) % n) / double(n);
      acc += x[m] * cd(std::cos(a), std::sin(a));
    }
    y[k] = acc;
  }
  return y;
}

static cd c(const rd_c64& v) { return cd(v.re, v.im); }

static rd_params chirp_params(int nr, double pulse_s, double bw, double fs, int window) {
  rd_params p{};
  p.Na = 1;
  p.Nr = nr;
  p.pulse_s = pulse_s;
  p.bandwidth_hz = bw;
  p.fs_hz = fs;
  p.range_window = window;
  return p;
}

static void check_roots() {
  for (int n : {1, 2, 3, 5, 16, 25, 256, 4096, 6000}) {
    const std::vector<rd_c64> w = roots_table(n);
    CHECK(w.size() == size_t(n), "roots_table(%d) size", n);
    CHECK(w[0].re == 1.0f && w[0].im == 0.0f, "roots_table(%d)[0] != 1", n);
    for (int k = 0; k < n; ++k) CHECK(std::abs(std::abs(c(w[k])) - 1.0) < 2e-7, "|w_%d^%d| != 1", n, k);
    // group law w^a w^b = w^(a+b)
    for (int a = 0; a < n; a += 1 + n / 7)
      for (int b = 0; b < n; b += 1 + n / 5)
        CHECK(std::abs(c(w[a]) * c(w[b]) - c(w[(a + b) % n])) < 4e-7, "w_%d^%d w^%d", n, a, b);
    if (n % 4 == 0) CHECK(std::abs(c(w[n / 4]) - cd(0, -1)) < 1e-7, "w_%d^(N/4) != -j", n);
  }
}

static void check_fft(std::mt19937_64& rng) {
  std::normal_distribution<double> g;
  for (int n : {1, 2, 4, 8, 64, 256, 1024}) {
    std::vector<cd> x(static_cast<size_t>(n));
    std::vector<double> re(static_cast<size_t>(n)), im(static_cast<size_t>(n));
    for (int i = 0; i < n; ++i) {
      x[size_t(i)] = cd(g(rng), g(rng));
      re[size_t(i)] = x[size_t(i)].real();
      im[size_t(i)] = x[size_t(i)].imag();
    }
    fft_pow2(re, im);
    const std::vector<cd> y = naive_dft(x, -1);
    double err = 0, ref = 0;
    for (int i = 0; i < n; ++i) {
      err = std::max(err, std::abs(cd(re[size_t(i)], im[size_t(i)]) - y[size_t(i)]));
      ref = std::max(ref, std::abs(y[size_t(i)]));
    }
    CHECK(err <= 1e-12 * (ref + 1) * std::log2(n + 1.0) * 4, "fft_pow2(%d) error %g", n, err);
  }
}

static void check_filters() {
  // Parseval: sum_k |Nr H[k]|^2 = Nr sum_n |h[n]|^2 = Nr sum_n w[n]^2 (a unit-modulus chirp)
  for (int window : {RD_WINDOW_RECT, RD_WINDOW_HAMMING})
    for (int nr : {64, 100, 256, 1000}) {
      const int L = nr / 3 + 1;
      const rd_params p = chirp_params(nr, L / 50e6, 20e6, 50e6, window);
      const std::vector<rd_c64> H = matched_filter(p, L);
      CHECK(H.size() == size_t(nr), "matched_filter size");
      double e = 0;
      for (const rd_c64& v : H) e += std::norm(c(v)) * double(nr) * double(nr);
      double w2 = 0;
      for (int n = 0; n < L; ++n) {
        const double w = window == RD_WINDOW_HAMMING && L > 1 ? 0.54 - 0.46 * std::cos(kTwoPi * n / (L - 1)) : 1.0;
        w2 += w * w;
      }
      CHECK(std::abs(e / (nr * w2) - 1.0) < 1e-5, "Parseval of H (Nr=%d, window %d): %g", nr, window, e / (nr * w2));
    }
  // the padded filter (an FFT of the reversed, conjugated replica) against the direct-sum
  // matched filter at M = Nr: DFT(g)[k] = e^{-j 2 pi k (L - 1) / M} conj(DFT(h)[k])
  for (int m : {64, 256, 2048}) {
    const int L = m / 5 + 3;
    const rd_params p = chirp_params(m, L / 120e6, 100e6, 120e6, RD_WINDOW_HAMMING);
    const std::vector<rd_c64> H = matched_filter(p, L);
    const std::vector<rd_c64> G = padded_filter(p, L, m);
    double err = 0, ref = 0;
    for (int k = 0; k < m; ++k) {
      const double a = -kTwoPi * double((int64_t(k) * (L - 1)) % m) / m;
      err = std::max(err, std::abs(c(G[size_t(k)]) - cd(std::cos(a), std::sin(a)) * c(H[size_t(k)])));
      ref = std::max(ref, std::abs(c(H[size_t(k)])));
    }
    CHECK(err < 1e-6 * ref, "padded_filter vs matched_filter at M=%d: %g of %g", m, err, ref);
  }
}

static void check_bluestein(std::mt19937_64& rng) {
  std::normal_distribution<double> g;
  for (int na : {16, 17, 100, 257, 997}) {
    const int m = bluestein_m(na);
    int ca = 0, cb = 0;
    pow2_split(m, &ca, &cb);
    const std::vector<rd_c64> spec = bluestein_spectra(na, m, ca, cb);
    CHECK(spec.size() == size_t(2) * size_t(m), "bluestein_spectra size");
    std::vector<cd> x(static_cast<size_t>(na));
    for (cd& v : x) v = cd(g(rng), g(rng));
    for (int d = 0; d < 2; ++d) {
      const int sign = d == 0 ? -1 : 1;
      // spectrum in natural bin order (row r holds bin r / cb + ca (r % cb))
      std::vector<cd> B(static_cast<size_t>(m));
      for (int r = 0; r < m; ++r) B[size_t(r / cb + ca * (r % cb))] = c(spec[size_t(d) * size_t(m) + size_t(r)]);
      // X[k] = c_k sum_n (x_n c_n) conj(c_{k-n}), c_n = exp(sign j pi n^2 / Na)
      std::vector<cd> y(static_cast<size_t>(m), 0.0);
      auto chirp = [&](int64_t n) {
        const double a = sign * M_PI * double((n * n) % (2 * int64_t(na))) / na;
        return cd(std::cos(a), std::sin(a));
      };
      for (int n = 0; n < na; ++n) y[size_t(n)] = x[size_t(n)] * chirp(n);
      std::vector<cd> Y = naive_dft(y, -1);
      for (int k = 0; k < m; ++k) Y[size_t(k)] *= B[size_t(k)];
      const std::vector<cd> z = naive_dft(Y, +1);  // the 1/M is inside B
      const std::vector<cd> X = naive_dft(x, sign);
      double err = 0, ref = 0;
      for (int k = 0; k < na; ++k) {
        err = std::max(err, std::abs(chirp(k) * z[size_t(k)] - X[size_t(k)]));
        ref = std::max(ref, std::abs(X[size_t(k)]));
      }
      CHECK(err < 2e-5 * ref, "Bluestein transform Na=%d sign %d: %g of %g", na, sign, err, ref);
    }
  }
}

static void check_interpolator() {
  for (double z = 0; z <= 30; z += 0.37)
    CHECK(std::abs(bessel_i0(z) / std::cyl_bessel_i(0.0, z) - 1) < 1e-13, "bessel_i0(%g)", z);
  for (double beta : {0.0, 2.5, 5.0, 8.0}) {
    rdf::RcmcPoly P{};
    rcmc_weight_polys(beta, &P);
    auto poly = [&](int q, double x, bool mirror) {
      double e = 0, o = 0, x2 = x * x, pw = 1;
      for (int i = 0; i < rdf::kRcmcEven; ++i, pw *= x2) e += P.even[q][i] * pw;
      pw = 1;
      for (int i = 0; i < rdf::kRcmcOdd; ++i, pw *= x2) o += P.odd[q][i] * pw;
      return mirror ? e - x * o : e + x * o;
    };
    for (int s = 0; s <= 64; ++s) {
      const double f = s / 64.0, x = f - 0.5;
      double w[8], sum = 0;  // taps j = -3..4 at index j + 3
      for (int q = 0; q < 4; ++q) {
        w[3 - q] = poly(q, x, false);  // j = -q
        w[4 + q] = poly(q, x, true);   // j = 1 + q
      }
      for (double v : w) sum += v;
      // the windowed sinc with the C++ library's Bessel function
      double r[8], rs = 0;
      for (int j = -3; j <= 4; ++j) {
        const double t = f - j;
        const double sinc = std::abs(t) < 1e-15 ? 1.0 : std::sin(M_PI * t) / (M_PI * t);
        const double a = 1 - (t / 4) * (t / 4);
        r[j + 3] = sinc * std::cyl_bessel_i(0.0, beta * std::sqrt(a > 0 ? a : 0)) / std::cyl_bessel_i(0.0, beta);
        rs += r[j + 3];
      }
      for (int i = 0; i < 8; ++i)
        CHECK(std::abs(w[i] / sum - r[i] / rs) < 2e-6, "interpolator beta=%g f=%g tap %d: %g vs %g", beta, f,
              i - 3, w[i] / sum, r[i] / rs);
      if (s == 0)
        for (int i = 0; i < 8; ++i) CHECK(std::abs(w[i] / sum - (i == 3 ? 1.0 : 0.0)) < 1e-6, "f=0 tap %d", i - 3);
    }
  }
}

static void check_geometry() {
  for (int n = 16; n <= 65536; n *= 2) {
    int a = 0, b = 0;
    pow2_split(n, &a, &b);
    CHECK(a * b == n && a <= b && b <= 4 * a && (a & (a - 1)) == 0, "pow2_split(%d) = %d x %d", n, a, b);
  }
  for (int na = 1; na <= 8192; na += 37) {
    const int m = bluestein_m(na);
    CHECK(m >= 256 && (m & (m - 1)) == 0 && m >= 2 * na - 1 && (m == 256 || m / 2 < 2 * na - 1),
          "bluestein_m(%d) = %d", na, m);
  }
  CHECK(azimuth_pow2(256) && azimuth_pow2(16384) && !azimuth_pow2(128) && !azimuth_pow2(32768) && !azimuth_pow2(3000),
        "azimuth_pow2");
  CHECK(azimuth_five(400) && azimuth_five(3200) && !azimuth_five(375) && !azimuth_five(6400) && !azimuth_five(0) &&
            !azimuth_five(-400),
        "azimuth_five");
  CHECK(persistent_grid(3, 256, 4096, 1) == 768 && persistent_grid(4, 256, 100, 1) == 100 &&
            persistent_grid(0, 0, 0, 0) == 1 && persistent_grid(2, 256, 8193, 2) == 512 &&
            persistent_grid(4, 256, int64_t(1) << 40, 1) == 1024,
        "persistent_grid");
  char buf[64];
  CHECK(!partial_overlap(buf, buf, 64) && partial_overlap(buf, buf + 8, 16) && !partial_overlap(buf, buf + 16, 16),
        "partial_overlap");
}

static void check_doppler_rows() {
  rd_params p{};
  p.Na = 1000;
  p.Nr = 600;
  p.fs_hz = 360e6;
  p.carrier_hz = 9.6e9;
  p.prf_hz = 1500;
  p.velocity_mps = 150;
  p.range_bin0_m = 10e3;
  const double dr = kC / (2 * p.fs_hz), lam = kC / p.carrier_hz;
  std::vector<double> rowc;
  const double mx = doppler_row_coefficients(p, dr, &rowc);
  CHECK(rowc.size() == size_t(4) * size_t(p.Na), "rowc size");
  // zero Doppler: no migration, phase 2 R / lambda cycles
  CHECK(rowc[0] == 0 && rowc[1] == 0 && std::abs(rowc[2] - 2 * p.range_bin0_m / lam) < 1e-6 &&
            std::abs(rowc[3] - 2 * dr / lam) < 1e-12,
        "zero-Doppler row");
  double m2 = 0;
  for (int k = 1; k < p.Na; ++k) {
    // +f and -f migrate alike
    for (int i = 0; i < 4; ++i) CHECK(rowc[4 * k + i] == rowc[4 * (p.Na - k) + i], "bins %d and %d differ", k, p.Na - k);
    // R (1 / D - 1) / dr with D = sqrt(1 - (lambda f / 2V)^2), written as D directly
    const int kk = k <= (p.Na - 1) / 2 ? k : k - p.Na;
    const double f = kk * p.prf_hz / p.Na, D = std::sqrt(1 - std::pow(lam * f / (2 * p.velocity_mps), 2));
    CHECK(std::abs(rowc[4 * k] - p.range_bin0_m * (1 / D - 1) / dr) < 1e-9 * (1 + rowc[4 * k]), "shift of bin %d", k);
    m2 = std::max(m2, rowc[4 * k] + (p.Nr - 1) * rowc[4 * k + 1]);
  }
  CHECK(mx == m2, "max shift");
  CHECK(stolt_halo(p) >= 5, "stolt halo of an X-band scene");
  rd_params q = p;
  q.carrier_hz = 1e6;  // below the Doppler band edge in wavenumber: no real mapping
  CHECK(stolt_halo(q) == -1, "stolt halo of an impossible geometry");
}

int main() {
  std::mt19937_64 rng(12345);
  check_roots();
  check_fft(rng);
  check_filters();
  check_bluestein(rng);
  check_interpolator();
  check_geometry();
  check_doppler_rows();
  if (g_fail) {
    std::printf("%d host checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
