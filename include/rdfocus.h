/*
 * rdfocus -- Range-Doppler SAR focusing on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The library focuses a raw SAR echo with the Range-Doppler chain:
 *   range compression per pulse  : FFT along range, multiply by the precomputed matched filter
 *                                  H(f), inverse FFT (one fused kernel, line resident in LDS);
 *   azimuth processing           : azimuth FFT down every range bin, range cell migration
 *                                  correction (RCMC, 8-tap Kaiser-windowed sinc) along range in
 *                                  every Doppler row, azimuth matched filter, azimuth inverse
 *                                  FFT -- all on the [Na][Nr] array in place, without corner
 *                                  turns (the azimuth transforms run as two passes of short
 *                                  transforms over strided / contiguous row sets).
 * Sources: cf-1.com/news/2323550 ("SAR imaging acceleration on Apple Silicon") §2.1 (the RD
 * steps), §3.1 (fused FFT -> filter -> IFFT per range line), §3.2 (inverse transform by
 * conj-FFT-conj), §5.1 (azimuth FFT, sinc RCMC, azimuth filter + IFFT); nxmr.cn/news/101525
 * ("ultra-high-resolution airborne SAR imaging on GPU") §2.1 (echo float2 [Na][Nr] and a chirp
 * spectrum [Nr] precomputed on the host), §2.2 (RCMC along the hyperbolic slant range), §3.1
 * (interleaved complex layout).
 *
 * Conventions (every call):
 *  - Complex samples are interleaved float32 pairs (rd_c64), row-major [Na][Nr]: row m is the
 *    m-th pulse (range line), column n the n-th range sample.  Outputs use the same layout.
 *  - Data pointers are DEVICE pointers on the plan's device, 8-byte aligned, owned by the
 *    caller; the library never frees them.  The plan owns its filter, twiddle and coefficient
 *    tables (a few hundred KB); focusing needs no further workspace.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work and return:
 *    results are ready once the stream is synchronised.  Argument errors are reported
 *    synchronously before anything is enqueued; launch errors are reported by the call;
 *    faults inside a kernel surface at the caller's next synchronisation.
 *  - A plan may be used by one stream at a time (it holds one workspace).  Calls must be made
 *    with the plan's device current.
 *  - No call aborts or throws; every call returns an rd_status.  rd_last_error() returns a
 *    thread-local message describing the last failure on the calling thread.
 *
 * Forward transforms are unnormalised with kernel e^{-j 2 pi k n / N}; inverse transforms
 * carry 1/N (folded into the filters).
 */
#ifndef RDFOCUS_H
#define RDFOCUS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Interleaved complex float32 sample (nxmr.cn/news/101525 §3.1: real/imag adjacent). */
typedef struct {
  float re, im;
} rd_c64;

/* Interleaved complex sample in IEEE 754 binary16 (half precision): the bit patterns of the
 * real and imaginary parts, 4 bytes a sample (cf-1.com/news/2323550 §7: FP16 storage with FP32
 * arithmetic). */
typedef struct {
  uint16_t re, im;
} rd_c32h;

typedef enum {
  RD_OK = 0,
  RD_ERR_INVALID_ARG = -1,        /* bad pointer, size, alignment, aliasing or parameter   */
  RD_ERR_UNSUPPORTED_LENGTH = -2, /* Na or Nr out of the supported lengths (see rd_length_supported) */
  RD_ERR_OUT_OF_MEMORY = -3,      /* device allocation for the plan failed                  */
  RD_ERR_DEVICE = -4,             /* HIP runtime error, or the plan's device is not current  */
  RD_ERR_LAUNCH = -5,             /* a kernel launch failed                                  */
  RD_ERR_NOT_CONFIGURED = -6      /* azimuth call on a range-only plan                       */
} rd_status;

/* Weighting of the replica before its spectrum is taken (framerc.cn/news/4459478 §3.1:
 * unweighted filters leave ~-13 dB sidelobes; Hamming lowers them and widens the mainlobe). */
enum { RD_WINDOW_RECT = 0, RD_WINDOW_HAMMING = 1 };

/* Problem statement (nxmr.cn/news/101525 §2.1: the echo float2 [Na][Nr] with Na pulses of Nr
 * range samples, and a chirp spectrum [Nr] precomputed on the host; §2.2: the platform and
 * slant-range geometry of RCMC; cf-1.com/news/2323550 §2.1: chirp parameters, range compression
 * by a matched filter, azimuth processing).  Range: linear-FM up-chirp of duration pulse_s and bandwidth
 * bandwidth_hz sampled at fs_hz; the replica holds L = ceil(pulse_s * fs_hz) samples at
 * indices [0, L) of a range line, h[n] = w[n] exp(j pi (B/Tp) (n/Fs - Tp/2)^2), and
 * H = conj(FFT_Nr(h)) is built in float64 on the host and rounded to float32 once.
 * Azimuth (zero squint, Doppler centroid 0): carrier_hz, prf_hz and velocity_mps all > 0
 * make a full-chain plan; all three == 0 make a range-only plan.  range_bin0_m is the slant
 * range of range sample 0, so bin n lies at R(n) = range_bin0_m + n * c / (2 fs_hz).
 * RCMC: rcmc_taps-point Kaiser(kaiser_beta)-windowed sinc, weights normalised to sum 1,
 * samples outside the line taken as 0. */
typedef struct {
  int32_t Na;            /* pulses (azimuth lines) >= 1; full-chain plans: see               *
                          * rd_length_supported                                              */
  int32_t Nr;            /* range samples per pulse: a supported transform length, or any    *
                          * length 1..8192 (see rd_range_compress, rd_length_supported)      */
  double pulse_s;        /* Tp  > 0                                                          */
  double bandwidth_hz;   /* B   > 0 (chirp rate +B/Tp)                                       */
  double fs_hz;          /* Fs  > 0; requires L <= Nr                                        */
  int32_t range_window;  /* RD_WINDOW_RECT or RD_WINDOW_HAMMING                              */
  double carrier_hz;     /* f0 (wavelength c/f0), or 0 for a range-only plan                 */
  double prf_hz;         /* pulse repetition frequency, or 0                                 */
  double velocity_mps;   /* platform speed, or 0; requires (c/f0 * PRF / (4 V))^2 < 1        */
  double range_bin0_m;   /* slant range of range sample 0 (ignored by range-only plans)      */
  int32_t rcmc_taps;     /* 8 (the only interpolator length built)                           */
  double kaiser_beta;    /* Kaiser window shape, 0 <= beta <= 12                             */
  uint32_t flags;        /* reserved, must be 0                                              */
} rd_params;

typedef struct rd_plan rd_plan;

/* Returns 1 if `n` is a transform length the library builds (256..16384 powers of two, and
 * 6000 = 2^4 * 3 * 5^3), else 0.  Plans also accept any other Nr in 1..8192: range compression
 * then runs as a zero-padded convolution (see rd_range_compress) and the RCMC of the
 * range-Doppler chain on rows of that length; rd_omega_k and rd_debug_line_fft along range need
 * a built length.  Full-chain plans also need Na a power of two in [256, 16384], 25 * 2^k in
 * [400, 3200] (nxmr.cn/news/101525 §5.3 images 1200 x 800), or any other Na in [16, 8192]: the
 * azimuth transform then takes the Bluestein (chirp-z) form of §5.1 through column transforms
 * of length M = the smallest power of two >= max(256, 2 Na - 1), with a plan-owned workspace of
 * M*Nr*8 bytes; and Na*Nr*8 (M*Nr*8) < 4 GiB (checked by rd_plan_create).  The range-Doppler entry points
 * (rd_azimuth_focus, rd_focus and the stage hook) further need a range migration
 * R(n)(1/D_k - 1)/dr below Nr/8 - 5 samples (1019 samples at lengths with no built transform)
 * over the whole Doppler band; beyond it they return RD_ERR_UNSUPPORTED_LENGTH, while the plan
 * still serves rd_omega_k and rd_backproject. */
int rd_length_supported(int32_t n);

/* Validates `params`, builds the matched filter H (float64 -> float32), the twiddle and
 * azimuth tables and the workspace on the current HIP device, and returns the plan in *out
 * (nxmr.cn/news/101525 §2.1: the chirp spectrum is computed once on the host, ahead of the
 * per-line kernels).  The plan owns its tables; rd_plan_destroy releases them.
 * On error *out is set to NULL and nothing is leaked. */
rd_status rd_plan_create(const rd_params* params, rd_plan** out);

/* Releases everything the plan owns; waits for the plan's outstanding work on the device.
 * NULL is a no-op.  A destroyed plan must not be used again (detected where possible). */
rd_status rd_plan_destroy(rd_plan* plan);

/* Range compression of every pulse (cf-1.com/news/2323550 §3.1, §3.2; nxmr.cn/news/101525
 * §2.1):  rc[m] = IFFT_Nr( FFT_Nr(echo[m]) * H ).  One fused kernel: each line is read from
 * HBM once and written once.  echo == rc (in place) is allowed; other overlap is an error.
 * Any line length: nxmr.cn/news/101525 §4.1 names Nr = 1200 as a usual airborne length and
 * §5.1 asks for transforms of lengths that are not powers of two.  Where Nr has no built
 * transform (Nr <= 8192), the same length-Nr circular correlation
 *   rc[m][n] = sum_i echo[m][(n + i) mod Nr] conj(h[i])
 * is computed exactly (up to float32 rounding) as one zero-padded circular convolution of
 * length M = the smallest power of two >= max(256, Nr + L - 1): the kernel reads the line,
 * extended periodically by L - 1 samples and zero-padded to M, into registers, multiplies its
 * spectrum by the M-point spectrum of the reversed, conjugated replica, and stores outputs
 * [L - 1, L - 1 + Nr) of the inverse transform.  The line is still read and written once. */
rd_status rd_range_compress(rd_plan* plan, const rd_c64* echo, rd_c64* rc, void* stream);

/* rd_range_compress with binary16 storage (cf-1.com/news/2323550 §7: FP16 storage, FP32
 * arithmetic): echo and rc are [Na][Nr] rd_c32h.  Each sample is converted exactly to float32 on
 * load, the whole line is processed in float32 as in rd_range_compress (same filter, same
 * transforms), and each output is rounded to the nearest binary16 value (ties to even) on
 * store; magnitudes beyond 65504 become infinities.  HBM traffic is 8 bytes a sample instead of
 * 16.  echo == rc (in place) is allowed; other overlap is an error.  Pointers must be 4-byte
 * aligned.  Every line length rd_range_compress takes is supported (the padded form too). */
rd_status rd_range_compress_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* rc, void* stream);

/* Azimuth processing of range-compressed data rc [Na][Nr] into the focused image img
 * [Na][Nr] (cf-1.com/news/2323550 §2.1, §5.1; nxmr.cn/news/101525 §2.2):
 *   S[k][n]   = sum_m rc[m][n] e^{-j 2 pi k m / Na}                (azimuth FFT)
 *   T[k][n]   = sum_{j=-3..4} w_j S[k][floor(x)+j],  x = n + R(n) (1/D_k - 1)/dr   (RCMC)
 *   img[m][n] = (1/Na) sum_k T[k][n] exp(+j 4 pi R(n) D_k / lambda) e^{+j 2 pi k m / Na}
 * with f_k the Doppler of bin k (FFT order), D_k = sqrt(1 - (lambda f_k / (2V))^2).
 * rc == img is allowed.  RD_ERR_NOT_CONFIGURED on a range-only plan. */
rd_status rd_azimuth_focus(rd_plan* plan, const rd_c64* rc, rd_c64* img, void* stream);

/* rd_range_compress followed by rd_azimuth_focus: raw echo to focused image.  echo == img is
 * allowed.  RD_ERR_NOT_CONFIGURED on a range-only plan. */
rd_status rd_focus(rd_plan* plan, const rd_c64* echo, rd_c64* img, void* stream);

/* rd_focus with binary16 storage of the echo, of every intermediate and of the image
 * (cf-1.com/news/2323550 §7: FP16 storage, FP32 arithmetic): echo and img are [Na][Nr]
 * rd_c32h and the chain runs in place in img.  Every kernel converts its input exactly to
 * float32, computes as rd_focus does, and rounds its output to the nearest binary16 value (ties
 * to even).  The unnormalised azimuth sums of rd_focus leave the binary16 range (65504): on a
 * 4096 x 4096 airborne scene whose range-compressed peak is 2.7e3, the azimuth spectrum reaches
 * 3.0e5 and the image 3.0e4.  Here each azimuth transform step is therefore scaled by
 * 1/(its length), the forward and the inverse transform each by 1/Na in all, and the row stage
 * omits its 1/Na:
 *   img_f16 = img / Na,  img = rd_focus's image of the same echo,
 * and no intermediate exceeds the largest magnitude of the range-compressed data.  Magnitudes
 * beyond 65504 still become infinities.  HBM traffic is 8 bytes a sample per pass instead of 16
 * (the Bluestein form's workspace stays float32).  echo == img is allowed; other overlap is an
 * error; pointers must be 4-byte aligned.  Every plan rd_focus takes is supported.
 * RD_ERR_NOT_CONFIGURED on a range-only plan; RD_ERR_UNSUPPORTED_LENGTH where rd_focus would
 * refuse the plan (range migration beyond the RCMC margin). */
rd_status rd_focus_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* img, void* stream);

/* rd_focus for callers that cannot allocate device memory while they run (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same result as rd_focus,
 * bit for bit, with the same arguments and errors, and no allocation of any kind (no hipMalloc,
 * hipFree or allocating library routine).  The one scratch buffer of the chain -- the [M][Nr]
 * float32 workspace of the Bluestein azimuth form (azimuth lengths that are neither a power of
 * two nor 25 * 2^k) -- is the library's static device scratch of 64 MiB instead of the plan's
 * workspace, so plans with M * Nr * 8 > 64 MiB return RD_ERR_INVALID_ARG; other plans use no
 * scratch.  Every GPU holds one such scratch for the life of the process, shared by every call
 * on that GPU: calls of rd_focus_noalloc that overlap on one GPU (different streams, or host
 * threads) race on it and must be serialised by the caller.  Nothing in it needs to start at
 * zero (each call writes every workspace sample before reading it); it keeps the last call's
 * contents. */
rd_status rd_focus_noalloc(rd_plan* plan, const rd_c64* echo, rd_c64* img, void* stream);

/* The azimuth half of rd_focus_f16 (cf-1.com/news/2323550 §7): range-compressed data rc
 * [Na][Nr] rd_c32h to img [Na][Nr] rd_c32h, img = (rd_azimuth_focus's image of the same rc) / Na,
 * with the same binary16 storage and scaling of every intermediate.  rd_focus_f16 equals
 * rd_range_compress_f16 followed by this call, bit for bit.  rc == img is allowed; other overlap
 * is an error; pointers must be 4-byte aligned.  RD_ERR_NOT_CONFIGURED on a range-only plan;
 * RD_ERR_UNSUPPORTED_LENGTH where rd_azimuth_focus would refuse the plan. */
rd_status rd_azimuth_focus_f16(rd_plan* plan, const rd_c32h* rc, rd_c32h* img, void* stream);

/* omega-k focusing with Stolt interpolation (nxmr.cn/news/101525 §3: the migration correction
 * becomes a frequency-domain mapping; forward and inverse 2-D transforms and two large complex
 * multiplies; §3.2: a phase built from the range and Doppler frequencies).  Raw echo [Na][Nr]
 * to image [Na][Nr] on the same grid as rd_focus (row m = pulse m, bin n at R(n)):
 *   S[k][j]  = 2-D DFT of echo (range bin j, Doppler bin k, FFT order)
 *   S       *= H[j] exp(+j 2 pi [(2 Rref / c) Q(f_j, f_k) - f_j tau0]),
 *              Q = sqrt((f0 + f_j)^2 - (c f_k / (2V))^2), tau0 = 2 range_bin0 / c,
 *              Rref = R(ref_bin) (the reference range)
 *   T[k][f'] = S[k] read at f = sqrt((f0 + f')^2 + (c f_k / (2V))^2) - f0 (Stolt mapping) with
 *              the 8-tap Kaiser(kaiser_beta)-windowed sinc of the RCMC, normalised weights,
 *              zero outside the sampled band [-Fs/2, Fs/2)
 *   T       *= exp(-j 2 pi f' 2 (Rref - range_bin0) / c);  img = inverse 2-D DFT (1/(Na Nr)).
 * Device work: azimuth transform steps, one fused kernel per Doppler row (range FFT, multiply,
 * Stolt mapping from LDS, range IFFT), inverse azimuth steps; echo == img allowed.
 * RD_ERR_NOT_CONFIGURED on a range-only plan; RD_ERR_INVALID_ARG if ref_bin is outside
 * [0, Nr) or f0 - Fs/2 <= c PRF / (4 V); RD_ERR_UNSUPPORTED_LENGTH if Nr has no built
 * transform (see rd_length_supported), or if the largest Stolt shift
 * (at f' = -Fs/2 and the Doppler band edge) plus 5 samples exceeds Nr/2 (Nr/8 at 16384). */
rd_status rd_omega_k(rd_plan* plan, const rd_c64* echo, rd_c64* img, int32_t ref_bin, void* stream);

/* rd_omega_k with binary16 storage of the echo, of every intermediate and of the image
 * (cf-1.com/news/2323550 §7: FP16 storage, FP32 arithmetic): echo and img are [Na][Nr] rd_c32h,
 * the chain runs in place in img, every kernel converts its input exactly to float32 and
 * rounds its output to the nearest binary16 value (ties to even).  As in rd_focus_f16, each
 * azimuth transform step is scaled by 1/(its length) and the row stage omits its 1/Na, so
 *   img_f16 = img / Na,  img = rd_omega_k's image of the same echo and ref_bin.
 * Arguments, conditions and errors as rd_omega_k, with 4-byte alignment. */
rd_status rd_omega_k_f16(rd_plan* plan, const rd_c32h* echo, rd_c32h* img, int32_t ref_bin, void* stream);

/* Test hook: the azimuth chain with its intermediates exposed.  azfft and rcmc receive the
 * azimuth spectrum S[k][n] and the RCMC output T[k][n], [Na][Nr] with row k = Doppler bin in
 * FFT order; img receives the image [Na][Nr].  azfft, rcmc and img must be distinct from each
 * other and from rc (img may equal rc).  The first call allocates a stage workspace of one
 * image (Na*Nr*8 bytes) owned by the plan. */
rd_status rd_debug_azimuth_stages(rd_plan* plan, const rd_c64* rc, rd_c64* azfft, rd_c64* rcmc,
                                  rd_c64* img, void* stream);

/* Test hook: the row stage of the range-Doppler chain on its own (cf-1.com/news/2323550 §5.1:
 * RCMC by sinc interpolation and the azimuth filter; nxmr.cn/news/101525 §2.2: the migrated
 * slant range along each range line of the range-Doppler domain).  in and out are [Na][Nr] with
 * row k holding Doppler bin k (FFT order) and range along the row:
 *   out[k][n] = sum_{j=-3..4} w_j in[k][floor(x)+j],  x = n + R(n) (1/D_k - 1)/dr
 * (the RCMC of rd_azimuth_focus), times exp(+j 4 pi R(n) D_k / lambda) / Na if filter != 0.
 * The chain runs this stage in place, so in == out is allowed (and gives the same bits as out of
 * place); other overlap is an error.  RD_ERR_NOT_CONFIGURED on a range-only plan;
 * RD_ERR_UNSUPPORTED_LENGTH where rd_azimuth_focus refuses the plan. */
rd_status rd_debug_rcmc(rd_plan* plan, const rd_c64* in, rd_c64* out, int32_t filter, void* stream);

/* Test hook: `lines` independent transforms of length Na (axis = 0) or Nr (axis = 1), from
 * in[lines][len] to out[lines][len] (in == out allowed): forward if inverse == 0, else the
 * inverse including 1/len.  Uses the same LDS-resident transform as the focusing kernels. */
rd_status rd_debug_line_fft(rd_plan* plan, int32_t axis, int32_t inverse, const rd_c64* in,
                            rd_c64* out, int64_t lines, void* stream);

/* Back-projection image grid (framerc.cn/news/4459478 §3.2: the imaging grid and the
 * observation geometry).  Slant-plane geometry of the focusing scenes: the platform flies a
 * straight track along x and is at x = V m / PRF at pulse m; pixel (i, j) lies at along-track
 * position x0_m + i dx_m and closest-approach slant range r0_m + j dr_m (metres). */
typedef struct {
  int32_t nx;    /* along-track pixels: rows of the image, >= 0                     */
  int32_t ny;    /* slant-range pixels: columns of the image, >= 0                  */
  double x0_m;   /* along-track position of row 0                                   */
  double dx_m;   /* row spacing                                                     */
  double r0_m;   /* closest-approach slant range of column 0 (> 0)                   */
  double dr_m;   /* column spacing (every column's range must stay > 0)             */
} rd_bp_grid;

/* Back-projection of range-compressed data (framerc.cn/news/4459478 §1.1, §2.2, §4.2):
 *   img[i][j] = sum_{m < Na} s_m(d) exp(+j 4 pi d / lambda),  d = sqrt(r_j^2 + (x_i - V m/PRF)^2),
 * where s_m(d) is range line m of rc [Na][Nr] (the output of rd_range_compress) linearly
 * interpolated at bin (d - range_bin0_m) / dr, samples outside the line taken as zero, and
 * lambda = c / carrier_hz.  img is [nx][ny] complex (row-major), device memory owned by the
 * caller; it must not overlap rc.  nx = 0 or ny = 0 is a no-op.  RD_ERR_NOT_CONFIGURED on a
 * range-only plan; RD_ERR_INVALID_ARG for a NULL grid, negative sizes, nx > 262140, non-finite
 * or non-positive ranges, bad or overlapping pointers.  Arithmetic: float32 per pulse (range
 * excess without cancellation, hardware sin/cos), float64 per-pixel constants and accumulation
 * over blocks of 32 pulses. */
rd_status rd_backproject(rd_plan* plan, const rd_c64* rc, rd_c64* img, const rd_bp_grid* grid,
                         void* stream);

/* Corner turn (cf-1.com/news/2323550 §5.1-§5.2: the transposes between range lines and azimuth
 * lines; nxmr.cn/news/101525 §2.2.1: padded shared-memory tiles):  out[c][r] = in[r][c] for a
 * row-major complex array in[rows][cols] (for example [Na][Nr] -> [Nr][Na]); out is [cols][rows].
 * Device pointers, 8-byte aligned, owned by the caller; the two buffers must not overlap (out of
 * place only).  rows = 0 or cols = 0 is a no-op.  RD_ERR_INVALID_ARG for negative sizes,
 * rows * cols > 2^40, more than 2^31 - 1 tiles of 64 x 64, or bad or overlapping pointers.
 * The work is 64 x 64 tiles through LDS on a persistent grid.  No plan is needed:
 * the work runs on the current device.  rd_focus does not use it (its azimuth transforms run
 * in place on [Na][Nr]); it serves callers that want the azimuth-major layout. */
rd_status rd_corner_turn(const rd_c64* in, rd_c64* out, int64_t rows, int64_t cols, void* stream);

/* Static description of a status code. */
const char* rd_status_string(rd_status status);

/* Message of the last failure on the calling thread ("" if none). */
const char* rd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RDFOCUS_H */
