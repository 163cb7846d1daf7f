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

namespace rdf {

// ------------------------------------------------------------------------------------------
// fused range compression: load -> FFT -> x H (H already carries 1/N) -> IFFT -> store
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
    const int64_t line = l0 + grp;
    const bool live = line < lines;
    float2 v[C::P];
#pragma unroll
    for (int i = 0; i < C::P; ++i) v[i] = make_float2(0.f, 0.f);
    if (live) load_global<N, T, R0>(v, in + line * N, tid);
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
    if (live) store_global<N, T, R0>(v, out + line * N, tid);
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
    const int64_t line = l0 + grp;
    const bool live = line < lines;
    float2 v[C::P];
#pragma unroll
    for (int i = 0; i < C::P; ++i) v[i] = make_float2(0.f, 0.f);
    if (live) load_global<N, T, RI>(v, in + line * N, tid);
    Passes<N, T, DIR, 1, L>::run(v, my, tw, tid);
    if (scale != 1.0f) {
#pragma unroll
      for (int i = 0; i < C::P; ++i) v[i] = cscale(v[i], scale);
    }
    if (live) store_global<N, T, RO>(v, out + line * N, tid);
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
    const bool live = line < lines;
    float2 v[C::P];
#pragma unroll
    for (int i = 0; i < C::P; ++i) v[i] = make_float2(0.f, 0.f);
    const double* Dl = opaque(Dk);
    if (live) {
      load_global<N, T, RI>(v, in + line * N, tid);
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
    }
    Passes<N, T, +1, 1, L>::run(v, my, tw, tid);
    if (live) store_global<N, T, RO>(v, out + line * N, tid);
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

template <int N>
constexpr LineOps make_ops() {
  return LineOps{N,           LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>,
                 &launch_fft<N>, &launch_azc<N>, &occupancy<N>};
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
