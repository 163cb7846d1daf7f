// Focusing kernels for gfx950.
//
// Range compression (cf-1.com/news/2323550 §3.1; nxmr.cn/news/101525 §2.1): one workgroup per
// range line (or LPW short lines), whole line resident in LDS/VGPRs, so each sample crosses HBM
// once in and once out.  The grid is persistent: workgroups loop over lines, which keeps H and
// the twiddles hot in the CU's cache and avoids a launch tail of one-line workgroups.
//
// Azimuth processing (cf-1.com/news/2323550 §5.1): corner turn to [Nr][Na], per-row FFT, RCMC
// along the range axis (nxmr.cn/news/101525 §2.2: a workgroup covers contiguous range rows so
// neighbouring rows are reused from cache), azimuth filter multiply fused with the inverse FFT.
#include "fft_core.hpp"
#include "rd_kernels.hpp"

#ifndef RD_PF_WAVES
#define RD_PF_WAVES 1
#endif
namespace rdf {

// ------------------------------------------------------------------------------------------
// fused range compression: load -> FFT -> x H (H already carries 1/N) -> IFFT -> store.
// Table variant: twiddles and H are read from global tables inside the line loop.
template <int N>
__global__ void __launch_bounds__(LineCfg<N>::WG)
    k_range_compress(const float2* in, float2* out, const float2* __restrict__ H,
                     const float2* __restrict__ tw, int64_t lines) {
  using C = LineCfg<N>;
  constexpr int T = C::T;
  constexpr int R0 = ListInfo<typename C::Fwd>::first;
  constexpr int RL = ListInfo<typename C::Fwd>::last;
  __shared__ float2 lds[C::LPW * C::LDS];
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += int64_t(gridDim.x) * C::LPW) {
    const LineIO src(in, N, l0, C::LPW, lines), dst(out, N, l0, C::LPW, lines);
    float2 v[C::P];
    load_line<N, T, R0>(v, src, grp * N, tid);
    Passes<N, T, -1, 1, typename C::Fwd>::run(v, my, tw, tid);
    {
      using G = Geom<N, T, RL>;
      const float2* Hl = opaque(H);
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        const int j = tid + b * T;
        if (G::live(j)) {
#pragma unroll
          for (int r = 0; r < RL; ++r) v[b * RL + r] = cmul(v[b * RL + r], Hl[j + r * G::NB]);
        }
      }
    }
    Passes<N, T, +1, 1, typename C::Inv>::run(v, my, tw, tid);
    store_line<N, T, R0>(v, dst, grp * N, tid);
  }
}

// Register-cached variant: the twiddles (small sets in LDS) and H are loaded once for the
// workgroup's lifetime, so the line loop issues no table loads; with PREFETCH the next line's
// samples are loaded into a second register set while the current line is transformed.  Needs
// Fwd == Inv (one twiddle cache serves both directions).
template <int N>
__device__ __forceinline__ void rc_line(float2* v, float2* lds,
                                        const TwCache<N, LineCfg<N>::T, 1, typename LineCfg<N>::Fwd>& twc,
                                        const float2* h, int tid) {
  using C = LineCfg<N>;
  using L = typename C::Fwd;
  constexpr int T = C::T;
  constexpr int RL = ListInfo<L>::last;
  using GL = Geom<N, T, RL>;
  PassesCached<N, T, -1, 1, L>::run(v, lds, twc, tid);
#pragma unroll
  for (int b = 0; b < GL::B; ++b) {
    if (GL::live(tid + b * T)) {
#pragma unroll
      for (int r = 0; r < RL; ++r) v[b * RL + r] = cmul(v[b * RL + r], h[b * RL + r]);
    }
  }
  PassesCached<N, T, +1, 1, L>::run(v, lds, twc, tid);
}

template <int N>
__device__ __forceinline__ void load_filter(float2* h, const float2* __restrict__ H, int tid) {
  using C = LineCfg<N>;
  constexpr int RL = ListInfo<typename C::Fwd>::last;
  using GL = Geom<N, C::T, RL>;
#pragma unroll
  for (int b = 0; b < GL::B; ++b) {
    const int j = tid + b * C::T;
#pragma unroll
    for (int r = 0; r < RL; ++r) h[b * RL + r] = GL::live(j) ? H[j + r * GL::NB] : make_float2(0.f, 0.f);
  }
}

template <int N, bool PREFETCH>
__global__ void __launch_bounds__(LineCfg<N>::WG)
    k_range_compress_pf(const float2* in, float2* out, const float2* __restrict__ H,
                        const float2* __restrict__ tw, int64_t lines) {
  using C = LineCfg<N>;
  using L = typename C::Fwd;
  static_assert(std::is_same<typename C::Fwd, typename C::Inv>::value, "needs Fwd == Inv");
  constexpr int T = C::T;
  constexpr int R0 = ListInfo<L>::first;
  constexpr int RL = ListInfo<L>::last;
  using TC = TwCache<N, T, 1, L>;
  __shared__ float2 lds[C::LPW * C::LDS + (TC::LDS > 0 ? TC::LDS : 1)];
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  TC twc;
  twc.load_all(tw, lds + C::LPW * C::LDS, tid, threadIdx.x, C::WG);
  // (the first pass's barrier orders the LDS twiddle table before its first use)
  float2 h[Geom<N, T, RL>::B * RL];
  load_filter<N>(h, H, tid);
  const int64_t stride = int64_t(gridDim.x) * C::LPW;
  float2 nxt[C::P];
  if (PREFETCH) {
    load_line<N, T, R0>(nxt, LineIO(in, N, int64_t(blockIdx.x) * C::LPW, C::LPW, lines), grp * N, tid);
    touch<C::P>(nxt);
  }
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += stride) {
    float2 v[C::P];
    if (PREFETCH) {
#pragma unroll
      for (int i = 0; i < C::P; ++i) v[i] = nxt[i];
      load_line<N, T, R0>(nxt, LineIO(in, N, l0 + stride, C::LPW, lines), grp * N, tid);
    } else {
      load_line<N, T, R0>(v, LineIO(in, N, l0, C::LPW, lines), grp * N, tid);
    }
    rc_line<N>(v, my, twc, h, tid);
    store_line<N, T, R0>(v, LineIO(out, N, l0, C::LPW, lines), grp * N, tid);
    // Wait for the prefetch here, where the stores just issued are younger than it and need not
    // complete; a wait at the loop head would merge with the loop entry and drain the stores.
    if (PREFETCH) touch<C::P>(nxt);
  }
}

// Two lines per loop trip with alternating register sets: line A's output registers stay
// untouched while line B is transformed (a pending store pins its data registers until it
// completes), and the next line is prefetched into a third set.  One line per workgroup.
template <int N>
__global__ void __launch_bounds__(LineCfg<N>::WG)
    k_range_compress_pf2(const float2* in, float2* out, const float2* __restrict__ H,
                         const float2* __restrict__ tw, int64_t lines) {
  using C = LineCfg<N>;
  using L = typename C::Fwd;
  static_assert(std::is_same<typename C::Fwd, typename C::Inv>::value, "needs Fwd == Inv");
  static_assert(C::LPW == 1, "one line per workgroup");
  constexpr int T = C::T;
  constexpr int P = C::P;
  constexpr int R0 = ListInfo<L>::first;
  constexpr int RL = ListInfo<L>::last;
  using TC = TwCache<N, T, 1, L>;
  __shared__ float2 lds[C::LDS + (TC::LDS > 0 ? TC::LDS : 1)];
  const int tid = threadIdx.x;
  TC twc;
  twc.load_all(tw, lds + C::LDS, tid, tid, C::WG);
  float2 h[Geom<N, T, RL>::B * RL];
  load_filter<N>(h, H, tid);
  const int64_t stride = gridDim.x;
  int64_t line = blockIdx.x;
  float2 pf[P], a[P], b[P];
#pragma unroll
  for (int i = 0; i < P; ++i) b[i] = make_float2(0.f, 0.f);
  load_line<N, T, R0>(pf, LineIO(in, N, line, 1, lines), 0, tid);
  touch<P>(pf);
  for (; line + stride < lines; line += 2 * stride) {
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = pf[i];
    load_line<N, T, R0>(pf, LineIO(in, N, line + stride, 1, lines), 0, tid);
    rc_line<N>(a, lds, twc, h, tid);
    store_line<N, T, R0>(a, LineIO(out, N, line, 1, lines), 0, tid);
    touch<P>(pf);
    touch<P>(b);
#pragma unroll
    for (int i = 0; i < P; ++i) b[i] = pf[i];
    load_line<N, T, R0>(pf, LineIO(in, N, line + 2 * stride, 1, lines), 0, tid);
    rc_line<N>(b, lds, twc, h, tid);
    store_line<N, T, R0>(b, LineIO(out, N, line + stride, 1, lines), 0, tid);
    touch<P>(pf);
    touch<P>(a);
  }
  if (line < lines) {  // odd tail
#pragma unroll
    for (int i = 0; i < P; ++i) a[i] = pf[i];
    rc_line<N>(a, lds, twc, h, tid);
    store_line<N, T, R0>(a, LineIO(out, N, line, 1, lines), 0, tid);
  }
}

// ------------------------------------------------------------------------------------------
// independent line transforms (azimuth FFT and the transform test hook); in == out allowed
template <int N, int DIR>
__global__ void __launch_bounds__(LineCfg<N>::WG)
    k_line_fft(const float2* in, float2* out, const float2* __restrict__ tw, int64_t lines,
               float scale) {
  using C = LineCfg<N>;
  using L = typename std::conditional<(DIR < 0), typename C::Fwd, typename C::Inv>::type;
  constexpr int T = C::T;
  constexpr int RI = ListInfo<L>::first;
  constexpr int RO = ListInfo<L>::last;
  __shared__ float2 lds[C::LPW * C::LDS];
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += int64_t(gridDim.x) * C::LPW) {
    float2 v[C::P];
    load_line<N, T, RI>(v, LineIO(in, N, l0, C::LPW, lines), grp * N, tid);
    Passes<N, T, DIR, 1, L>::run(v, my, tw, tid);
    if (scale != 1.0f) {
#pragma unroll
      for (int i = 0; i < C::P; ++i) v[i] = cscale(v[i], scale);
    }
    store_line<N, T, RO>(v, LineIO(out, N, l0, C::LPW, lines), grp * N, tid);
  }
}

// ------------------------------------------------------------------------------------------
// azimuth filter + inverse azimuth FFT, one row (range bin n) of the [Nr][Na] layout per line:
//   out[n][m] = (1/Na) sum_k in[n][k] exp(+j 4 pi R(n) D_k / lambda) e^{+j 2 pi k m / Na}
// The filter phase is formed in float64 (4 pi R D / lambda reaches ~1e7 rad), reduced to the
// nearest whole cycle, and only the residual (|frac| <= 1/2 cycle) is taken to float32.
template <int N>
__global__ void __launch_bounds__(LineCfg<N>::WG)
    k_az_compress(const float2* in, float2* out, const float2* __restrict__ tw,
                  const double* __restrict__ Dk, AzFilterConst c, int64_t lines) {
  using C = LineCfg<N>;
  using L = typename C::Inv;
  constexpr int T = C::T;
  constexpr int RI = ListInfo<L>::first;
  constexpr int RO = ListInfo<L>::last;
  __shared__ float2 lds[C::LPW * C::LDS];
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += int64_t(gridDim.x) * C::LPW) {
    const int64_t line = l0 + grp;
    float2 v[C::P];
    load_line<N, T, RI>(v, LineIO(in, N, l0, C::LPW, lines), grp * N, tid);
    const double* Dl = opaque(Dk);
    const double a = c.two_over_lambda * (c.rb0 + double(line) * c.dr);
    using G = Geom<N, T, RI>;
#pragma unroll
    for (int b = 0; b < G::B; ++b) {
      const int j = tid + b * T;
      if (G::live(j)) {
#pragma unroll
        for (int r = 0; r < RI; ++r) {
          const double cyc = a * Dl[j + r * G::NB];
          const float f = float(cyc - rint(cyc));
          float s, co;
          sincospif(2.0f * f, &s, &co);
          v[b * RI + r] = cmul(v[b * RI + r], make_float2(co * c.inv_na, s * c.inv_na));
        }
      }
    }
    Passes<N, T, +1, 1, L>::run(v, my, tw, tid);
    store_line<N, T, RO>(v, LineIO(out, N, l0, C::LPW, lines), grp * N, tid);
  }
}

// ------------------------------------------------------------------------------------------
// RCMC, 8 taps, on [Nr][Na]: out[n][k] = sum_{j=-3..4} w_j in[i0 + j][k], x = n + R(n) Q_k,
// i0 = floor(x), f = x - i0, w_j = kaiser-sinc(f - j) / sum.  The shift is formed in float64
// and only its fraction goes to float32, so large range indices cost no precision.
// Workgroups of consecutive rows run on the same XCD (blocks are dealt to the 8 XCDs
// round-robin), so the 8-row neighbourhood of a row is mostly served from that XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int b, int G) {
  const int q = G / 8, r = G % 8;
  const int x = b % 8, i = b / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

__global__ void __launch_bounds__(256)
    k_rcmc8(const float2* __restrict__ in, float2* __restrict__ out,
            const double* __restrict__ Qk, RcmcConst c, int Nr, int Na, int kblocks) {
  const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int n = logical / kblocks;
  const int k = (logical - n * kblocks) * 256 + threadIdx.x;
  if (k >= Na) return;
  const double x = (c.rb0 + double(n) * c.dr) * Qk[k];
  const double fl = floor(x);
  const int i0 = n + int(fl);
  const float f = float(x - fl);
  float2 acc = make_float2(0.f, 0.f);
  if (f == 0.0f) {
    if (i0 >= 0 && i0 < Nr) acc = in[int64_t(i0) * Na + k];
  } else {
    float wsum = 0.f;
#pragma unroll
    for (int j = -3; j <= 4; ++j) {
      const float t = f - float(j);
      const float y = c.y0 - c.y1 * t * t;
      float p = c.coef[0];
      for (int m = 1; m < c.nterm; ++m) p = fmaf(p, y, c.coef[m]);
      const float a = ((j & 1) ? -p : p) / t;
      wsum += a;
      const int i = i0 + j;
      if (i >= 0 && i < Nr) {
        const float2 s = in[int64_t(i) * Na + k];
        acc.x = fmaf(a, s.x, acc.x);
        acc.y = fmaf(a, s.y, acc.y);
      }
    }
    const float inv = 1.0f / wsum;
    acc = cscale(acc, inv);
  }
  out[int64_t(n) * Na + k] = acc;
}

// ------------------------------------------------------------------------------------------
// corner turn: out[c][r] = in[r][c] through a 64 x 64 LDS tile padded by one element per row
// (nxmr.cn/news/101525 §2.2.1: the pad moves consecutive rows onto different banks).
__global__ void __launch_bounds__(256)
    k_corner_turn(const float2* __restrict__ in, float2* __restrict__ out, int64_t rows,
                  int64_t cols) {
  __shared__ float2 tile[64][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + ty + 4 * i, c = c0 + tx;
    if (r < rows && c < cols) tile[ty + 4 * i][tx] = in[r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t c = c0 + ty + 4 * i, r = r0 + tx;
    if (r < rows && c < cols) out[c * rows + r] = tile[tx][ty + 4 * i];
  }
}

// ------------------------------------------------------------------------------------------
// launchers
template <int N>
hipError_t launch_rc(const float2* in, float2* out, const float2* H, const float2* tw,
                     int64_t lines, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_range_compress<N>, dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H, tw,
                     lines);
  return hipGetLastError();
}

template <int N>
hipError_t launch_fft(const float2* in, float2* out, const float2* tw, int64_t lines, int inverse,
                      float scale, int grid, hipStream_t s) {
  if (inverse)
    hipLaunchKernelGGL((k_line_fft<N, +1>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, tw,
                       lines, scale);
  else
    hipLaunchKernelGGL((k_line_fft<N, -1>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, tw,
                       lines, scale);
  return hipGetLastError();
}

template <int N>
hipError_t launch_azc(const float2* in, float2* out, const float2* tw, const double* Dk,
                      AzFilterConst c, int64_t lines, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_az_compress<N>, dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, tw, Dk, c,
                     lines);
  return hipGetLastError();
}

template <int N>
hipError_t occupancy(int* rc, int* fft, int* azc) {
  hipError_t e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress<N>, LineCfg<N>::WG, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(fft, k_line_fft<N, -1>, LineCfg<N>::WG, 0);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(azc, k_az_compress<N>, LineCfg<N>::WG, 0);
}

#ifndef RD_RC_PREFETCH
#define RD_RC_PREFETCH true
#endif
template <int N>
hipError_t launch_rc_pf(const float2* in, float2* out, const float2* H, const float2* tw,
                        int64_t lines, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_range_compress_pf<N, RD_RC_PREFETCH>), dim3(grid), dim3(LineCfg<N>::WG), 0,
                     s, in, out, H, tw, lines);
  return hipGetLastError();
}

template <int N>
hipError_t launch_rc_pf2(const float2* in, float2* out, const float2* H, const float2* tw,
                         int64_t lines, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_range_compress_pf2<N>, dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H,
                     tw, lines);
  return hipGetLastError();
}

template <int N>
hipError_t occupancy_pf(int* rc) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_pf<N, RD_RC_PREFETCH>,
                                                      LineCfg<N>::WG, 0);
}

template <int N>
hipError_t occupancy_pf2(int* rc) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_pf2<N>, LineCfg<N>::WG,
                                                      0);
}

template <int N>
constexpr LineOps make_ops() {
  constexpr bool sym = std::is_same<typename LineCfg<N>::Fwd, typename LineCfg<N>::Inv>::value;
  if constexpr (sym && LineCfg<N>::LPW == 1) {
    return LineOps{N, LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>, &launch_fft<N>,
                   &launch_azc<N>, &occupancy<N>, &launch_rc_pf<N>, &occupancy_pf<N>,
                   &launch_rc_pf2<N>, &occupancy_pf2<N>};
  } else if constexpr (sym) {
    return LineOps{N, LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>, &launch_fft<N>,
                   &launch_azc<N>, &occupancy<N>, &launch_rc_pf<N>, &occupancy_pf<N>,
                   nullptr, nullptr};
  } else {
    return LineOps{N, LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>, &launch_fft<N>,
                   &launch_azc<N>, &occupancy<N>, nullptr, nullptr, nullptr, nullptr};
  }
}

static const LineOps kOps[] = {make_ops<256>(),  make_ops<512>(),  make_ops<1024>(),
                               make_ops<2048>(), make_ops<4096>(), make_ops<8192>(),
                               make_ops<16384>(), make_ops<6000>()};

const LineOps* line_ops(int n) {
  for (const LineOps& o : kOps)
    if (o.n == n) return &o;
  return nullptr;
}

hipError_t launch_corner_turn(const float2* in, float2* out, int64_t rows, int64_t cols,
                              hipStream_t s) {
  const dim3 grid(unsigned((cols + 63) / 64), unsigned((rows + 63) / 64));
  hipLaunchKernelGGL(k_corner_turn, grid, dim3(256), 0, s, in, out, rows, cols);
  return hipGetLastError();
}

hipError_t launch_rcmc8(const float2* in, float2* out, const double* Qk, const RcmcConst& c,
                        int Nr, int Na, hipStream_t s) {
  const int kblocks = (Na + 255) / 256;
  const int64_t blocks = int64_t(kblocks) * Nr;
  hipLaunchKernelGGL(k_rcmc8, dim3(unsigned(blocks)), dim3(256), 0, s, in, out, Qk, c, Nr, Na,
                     kblocks);
  return hipGetLastError();
}

}  // namespace rdf
