// Focusing kernels for gfx950.
//
// Range compression (cf-1.com/news/2323550 §3.1; nxmr.cn/news/101525 §2.1): each range line is
// transformed, multiplied by H and inverse transformed in one kernel with the whole line in
// registers and LDS, so each sample crosses HBM once in and once out.  Persistent grids:
// workgroups loop over lines with the next line prefetched into registers.  Variants: the
// 4096-sample DIF/DIT kernel, the register-cached kernel for the other built lengths, the
// zero-padded form for any length up to 8192, and binary16 line storage.
//
// Azimuth processing (cf-1.com/news/2323550 §5.1; nxmr.cn/news/101525 §2.2) in place on
// [Na][Nr], with no corner turn: the azimuth transform as strided and block column steps, RCMC
// fused with the azimuth filter per Doppler row from LDS, and the inverse column steps.  Other
// azimuth lengths take the Bluestein form (nxmr.cn/news/101525 §5.1): chirp passes around
// column steps of a power-of-two length.  omega-k (nxmr.cn/news/101525 §3) reuses the column
// steps around one fused row stage.  The column steps, both row stages and the chirp passes
// also have binary16-storage variants (cf-1.com/news/2323550 §7), float32 arithmetic inside.
// Also here: the corner turn (an entry point of its own), back-projection
// (framerc.cn/news/4459478), and the line-transform test hook.
#include <atomic>

#include "fft_core.hpp"
#include "rd_kernels.hpp"

#ifndef RD_PF_WAVES
#define RD_PF_WAVES 1
#endif
namespace rdf {
// Cache policy of the image passes (an instruction's cache-policy bits): the azimuth chain
// re-reads what the previous pass wrote, which the 256 MB Infinity Cache holds when the image
// fits there -- ordinary (cacheable) accesses then (measured ~5% faster on the 4096 x 4096
// chain); a larger image would only churn the cache, so its passes stream with the
// non-temporal hint (measured ~5% faster on the 16384 x 16384 chain).
constexpr int kAuxCached = 0;
constexpr int kAuxStream = kBufNonTemporal;

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
  RD_POISON_LDS(lds);
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += int64_t(gridDim.x) * C::LPW) {
    const LineIO src(in, N, l0, C::LPW, lines), dst(out, N, l0, C::LPW, lines);
    float2 v[C::P];
    load_line<N, T, R0>(v, src, grp * N, tid);
    Passes<N, T, -1, 1, typename C::Fwd, C::WAVE>::run(v, my, tw, tid);
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
    Passes<N, T, +1, 1, typename C::Inv, C::WAVE>::run(v, my, tw, tid);
    store_line<N, T, R0>(v, dst, grp * N, tid);
  }
}

// Register-cached variant: the twiddles (small sets in LDS, larger ones in registers) are
// loaded once for the workgroup's lifetime, so the line loop issues no twiddle loads.  Needs
// Fwd == Inv (one twiddle cache serves both directions).  The filter H is either held in
// registers for the kernel's lifetime (HREG) or read per line from the global table (cache
// resident) at the multiply.  With prefetch (PF), the next line is loaded into a second register
// set at the start of the current one.  (Measured on the 4096-point line: a prefetch issued
// after the multiply, with H read per line so the two never hold registers together, reaches
// occupancy 4 but is slower -- the exposed filter loads cost more than the occupancy gains.)
template <int N>
constexpr int filter_regs() {
  using C = LineCfg<N>;
  return Geom<N, C::T, ListInfo<typename C::Fwd>::last>::B * ListInfo<typename C::Fwd>::last;
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

// v *= H: from the registers h (HREG) or from the global table Hg
template <int N>
__device__ __forceinline__ void filter_multiply(float2* v, const float2* h,
                                                const float2* __restrict__ Hg, int tid) {
  using C = LineCfg<N>;
  constexpr int RL = ListInfo<typename C::Fwd>::last;
  using GL = Geom<N, C::T, RL>;
  if constexpr (!C::HREG) {
    // Issue every filter load before the first use: left to itself the compiler serialises
    // them (load, wait, multiply) to save registers, one cache round trip per sample.
    float2 hv[GL::B * RL];
    load_filter<N>(hv, Hg, tid);
    touch<GL::B * RL>(hv);
#pragma unroll
    for (int b = 0; b < GL::B; ++b) {
      if (GL::live(tid + b * C::T)) {
#pragma unroll
        for (int r = 0; r < RL; ++r) v[b * RL + r] = cmul(v[b * RL + r], hv[b * RL + r]);
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < GL::B; ++b) {
    const int j = tid + b * C::T;
    if (GL::live(j)) {
#pragma unroll
      for (int r = 0; r < RL; ++r)
        v[b * RL + r] = cmul(v[b * RL + r], C::HREG ? h[b * RL + r] : Hg[j + r * GL::NB]);
    }
  }
}

// Line I/O of the range kernels: natural (n_line == N) or zero-padded (PAD, see below).
template <int N, bool PAD, bool HALF>
__device__ __forceinline__ void rc_load(float2* v, const void* in, int64_t l0, int64_t lines, int grp,
                                        int tid, int n_line, int skip) {
  using C = LineCfg<N>;
  constexpr int R0 = ListInfo<typename C::Fwd>::first;
  const float2* src = static_cast<const float2*>(in);
  if constexpr (PAD && HALF)
    load_line_pad_h<N, C::T, R0>(v, LineIOh(in, n_line, l0, C::LPW, lines), grp * n_line, tid, n_line,
                                 n_line + skip);
  else if constexpr (PAD)
    load_line_pad<N, C::T, R0>(v, LineIO(src, n_line, l0, C::LPW, lines), grp * n_line, tid, n_line,
                               n_line + skip);
  else if constexpr (HALF)
    load_line_h<N, C::T, R0>(v, LineIOh(in, N, l0, C::LPW, lines), grp * N, tid);
  else
    load_line<N, C::T, R0>(v, LineIO(src, N, l0, C::LPW, lines), grp * N, tid);
}
template <int N, bool PAD, bool HALF, int SAUX>
__device__ __forceinline__ void rc_store(const float2* v, void* out, int64_t l0, int64_t lines, int grp,
                                         int tid, int n_line, int skip) {
  using C = LineCfg<N>;
  constexpr int R0 = ListInfo<typename C::Fwd>::first;
  float2* dst = static_cast<float2*>(out);
  if constexpr (PAD && HALF)
    store_line_pad_h<N, C::T, R0, SAUX>(v, LineIOh(out, n_line, l0, C::LPW, lines), grp * n_line, tid,
                                        n_line, skip);
  else if constexpr (PAD)
    store_line_pad<N, C::T, R0, SAUX>(v, LineIO(dst, n_line, l0, C::LPW, lines), grp * n_line, tid, n_line,
                                      skip);
  else if constexpr (HALF)
    store_line_h<N, C::T, R0, SAUX>(v, LineIOh(out, N, l0, C::LPW, lines), grp * N, tid);
  else
    store_line<N, C::T, R0, SAUX>(v, LineIO(dst, N, l0, C::LPW, lines), grp * N, tid);
}

// PAD: lines of n_line < N samples (any length): each is extended periodically by skip samples
// and zero-padded to N; with the plan's filter (the N-point spectrum of the reversed, conjugated
// replica of skip + 1 samples) the N-point circular convolution holds the length-n_line circular
// correlation at positions [skip, skip + n_line), exactly when N >= n_line + skip.
template <int N, bool PF, int SAUX, bool PAD = false, bool HALF = false>
__global__ void __launch_bounds__(LineCfg<N>::WG, LineCfg<N>::WPE)
    k_range_compress_pf(const void* in, void* out, const float2* __restrict__ H,
                        const float2* __restrict__ tw, int64_t lines, int n_line, int skip) {
  using C = LineCfg<N>;
  using L = typename C::Fwd;
  static_assert(std::is_same<typename C::Fwd, typename C::Inv>::value, "needs Fwd == Inv");
  constexpr int T = C::T;
  using TC = TwCache<N, T, 1, L>;
  constexpr bool LATE = PF && PfLate<N>::value && !C::HREG;
  constexpr bool DB = LdsDouble<N>::value;          // two line buffers, one barrier per exchange
  constexpr int LBUF = C::LDS * (DB ? 2 : 1);
  constexpr bool SWAP = DB && (ListInfo<L>::count - 1) % 2 == 1;  // inverse starts on buffer b
  __shared__ float2 lds[C::LPW * LBUF + (TC::LDS > 0 ? TC::LDS : 1)];
  RD_POISON_LDS(lds);
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * LBUF;
  float2* my2 = my + (DB ? C::LDS : 0);
  const int64_t stride = int64_t(gridDim.x) * C::LPW;
  // The first line's loads go out before the table loads, so the line's HBM latency overlaps
  // the table reads instead of following them.
  float2 nxt[C::P];
  if constexpr (PF)
    rc_load<N, PAD, HALF>(nxt, in, int64_t(blockIdx.x) * C::LPW, lines, grp, tid, n_line, skip);
  TC twc;
  twc.load_all(tw, lds + C::LPW * LBUF, tid, threadIdx.x, C::WG);
  // (the first pass's barrier orders the LDS twiddle table before its first use, unless a line's
  // exchanges are wave-local or double-buffered: then an explicit barrier does)
  if constexpr ((C::WAVE || DB) && TC::LDS > 0) __syncthreads();
  float2 h[C::HREG ? filter_regs<N>() : 1];
  if constexpr (C::HREG) load_filter<N>(h, H, tid);
  // Wait for the filter and twiddle registers before the line loop (see touch): a wait for them
  // inside the loop would also wait for the previous line's stores on every iteration.
  if constexpr (C::HREG) touch<filter_regs<N>()>(h);
  twc.touch_all();
  if constexpr (PF) touch<C::P>(nxt);
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += stride) {
    float2 v[C::P];
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < C::P; ++i) v[i] = nxt[i];
      if constexpr (!LATE) rc_load<N, PAD, HALF>(nxt, in, l0 + stride, lines, grp, tid, n_line, skip);
    } else {
      rc_load<N, PAD, HALF>(v, in, l0, lines, grp, tid, n_line, skip);
    }
    if constexpr (DB)
      PassesCached<N, T, -1, 1, L, C::WAVE>::run2(v, my, my2, twc, tid);
    else
      PassesCached<N, T, -1, 1, L, C::WAVE>::run(v, my, twc, tid);
    filter_multiply<N>(v, h, opaque(H), tid);
    if constexpr (LATE) rc_load<N, PAD, HALF>(nxt, in, l0 + stride, lines, grp, tid, n_line, skip);
    if constexpr (DB)
      PassesCached<N, T, +1, 1, L, C::WAVE>::run2(v, SWAP ? my2 : my, SWAP ? my : my2, twc, tid);
    else
      PassesCached<N, T, +1, 1, L, C::WAVE>::run(v, my, twc, tid);
    rc_store<N, PAD, HALF, SAUX>(v, out, l0, lines, grp, tid, n_line, skip);
    // Wait for the prefetch here, where the stores just issued are younger than it and need not
    // complete; a wait at the loop head would merge with the loop entry and drain the stores.
    if constexpr (PF) touch<C::P>(nxt);
  }
}

// ------------------------------------------------------------------------------------------
// Range compression of 4096-sample lines with two barriers per line.  With n = t + 256 n2
// (t = n0 + 16 n1 < 256) and k = k0 + 16 k1 + 256 k2, the forward transform runs in the
// decimation-in-frequency order
//   a: DFT16 over n2 -> k0, times W_4096^{t k0}            (thread t = n0 + 16 n1)
//   b: DFT16 over n1 -> k1, times W_256^{n0 k1}             (thread 16 k0 + n0)
//   c: DFT16 over n0 -> k2                                   (thread 16 k0 + k1)
// and leaves X[k0 + 16 k1 + 256 k2] in thread 16 k0 + k1, which multiplies it by the filter
// (held in registers in that permuted order for all the workgroup's lines) and runs the inverse
// as the mirror image in
// decimation-in-time order (c, b, a with conjugate roots, the twiddles before the DFTs), ending
// with y[t + 256 n2] in thread t.  Steps b -> c and their mirror exchange data only inside a
// group of 16 lanes (one wave), so they need no workgroup barrier; a -> b and its mirror are
// workgroup exchanges, one barrier each (two per line).  Both directions use the same twiddles:
// W_4096^{t k0} in registers (the powers k0 = 1, 2, 4, 8, the others formed as products; the
// matrix-core variant, which reads the plan's full table, holds all fifteen) and W_256^{n0 k1} in
// an LDS table.  LDS layout: region g = 0..15 of 272 elements (rows of 256 or
// 16 x 17, padded so that two 16-lane groups of a half-wave fall on complementary banks):
// every exchange is free of bank conflicts under the gfx950 geometry (8-byte reads: 32 lanes
// over 64 banks; 8-byte writes: 16 lanes over 32 banks).
// The filter in the order the threads hold it, so that every wave reads it with contiguous
// accesses: tab[r 256 + t] = H[g + 16 l + 256 r] (g = t / 16, l = t % 16, r = 0..15), followed by
// the twiddles in the same thread-major order, so every start-up table read is a contiguous wave
// access (strided start-up table reads by every workgroup at once were measured to cost 2-9 us
// per launch).
#ifndef RD_RC4096_TWTAB
#define RD_RC4096_TWTAB 1
#endif
// The twiddles W_4096^{t k} and the W_256 table are read from the same thread-major table
// (rounded once from float64), not evaluated by every workgroup with sincospi: measured on MI355X
// 0.3-0.5 us faster per 4096-line launch (RD_RC4096_TWTAB=0 builds the evaluated form).
constexpr int kRc4096Tab = 16 * 256 + (RD_RC4096_TWTAB ? 16 * 256 : 0);
void rc4096_tab_fill(const float2* H, const float2* roots, float2* out) {
  for (int r = 0; r < 16; ++r)
    for (int t = 0; t < 256; ++t) out[r * 256 + t] = H[(t >> 4) + 16 * (t & 15) + 256 * r];
  if (RD_RC4096_TWTAB) {
    for (int k = 1; k < 16; ++k)
      for (int t = 0; t < 256; ++t) out[4096 + (k - 1) * 256 + t] = roots[(t * k) & 4095];
    for (int t = 0; t < 240; ++t) out[4096 + 15 * 256 + t] = roots[16 * (((t & 15) * (t / 16 + 1)) & 255)];
  }
}

// Occupancy: four workgroups per CU (four waves per SIMD, 1024 workgroups, exactly four lines
// each at 4096 lines) need at most 128 VGPRs.  Live across every line: the line (32 registers),
// the filter (32, loaded once), four of the fifteen twiddles W_4096^{t k} (8; the other eleven are
// formed as products where they are applied) and, from the filter multiply on, the next line's
// prefetch (32): 126 VGPRs (binary16: 111, its prefetch packed at one register a sample).
// Measured on MI355X (interleaved runs, 200 launches each): 52.7-53.3 us per launch against
// 55.6-56.1 us when the fifteen twiddles are held and the filter is reloaded from the table before
// stage c of every line (114 VGPRs), whose reads cost 128 MB of L2 traffic per launch; 56.8 us for
// the three-wave form that held the filter and fifteen twiddles (166 VGPRs).  Issuing the prefetch
// earlier (after the first exchange, or before stage a) measured 1.5-4 us slower.
#ifndef RD_RC4096_MFMA
#define RD_RC4096_MFMA 0
#endif

typedef float rdf_v4f __attribute__((ext_vector_type(4)));
// x[k] *= w^k (CONJ: conj(w)^k), k = 1..K-1 (K <= 16), with w^k formed from w^1, w^2, w^4, w^8 in
// w2[0..3]
// (the base roots pass through an empty asm statement, so the products are formed at every
// application instead of being hoisted out of a line loop into fifteen live registers)
template <bool CONJ, int K = 16>
__device__ __forceinline__ void twiddles_from_powers(float2* x, const float2* w2) {
  float2 p[K];
#pragma unroll
  for (int k = 1; k < K; ++k) {
    const int hb = 1 << ilog2(k);
    if (hb == k) {
      p[k] = w2[ilog2(k)];
      asm volatile("" : "+v"(p[k].x), "+v"(p[k].y));
    } else {
      p[k] = cmul(p[hb], p[k - hb]);
    }
    float2 w = p[k];
    if (CONJ) w.y = -w.y;
    x[k] = cmul(x[k], w);
  }
}

template <int SAUX, bool HALF = false>
__global__ void __launch_bounds__(256, 4)
    k_range_compress_4096(const void* in, void* out, const float2* __restrict__ tab,
                          int64_t lines) {
  constexpr int N = 4096, T = 256, REG = 272;
  __shared__ float2 lds[16 * REG + 15 * 16];
  RD_POISON_LDS(lds);
  float2* tw2 = lds + 16 * REG;  // W_256^{n0 k}: tw2[(k - 1) 16 + n0], k = 1..15
  const int t = threadIdx.x;
  const int g = t >> 4, l = t & 15;
  const int64_t stride = gridDim.x;
  // The first line's loads go out before the table loads, so the line's HBM latency overlaps
  // the table reads instead of following them.
  // line I/O: float32 or binary16 storage.  A binary16 prefetch stays packed (one register a
  // sample) until it becomes the working line.
  using Pre = typename std::conditional<HALF, unsigned int, float2>::type;
  auto load = [&](Pre* dst, int64_t line) {
    if constexpr (HALF)
      load_line_h_packed<N, T, 16>(dst, LineIOh(in, N, line, 1, lines), 0, t);
    else
      load_line<N, T, 16>(dst, LineIO(static_cast<const float2*>(in), N, line, 1, lines), 0, t);
  };
  Pre nxt[16];
  load(nxt, blockIdx.x);
  // W_4096^{t k}, k = 1..15: only k = 1, 2, 4, 8 are held and the others are formed as products
  // where they are applied, which leaves the registers to hold the filter across lines
  constexpr bool DER = !RD_RC4096_MFMA;
  float2 w1[15];
  if constexpr (DER) {
    if (t < 240) tw2[t] = tab[4096 + 15 * 256 + t];
#pragma unroll
    for (int i = 0; i < 4; ++i) w1[i] = tab[4096 + ((1 << i) - 1) * 256 + t];
  } else if constexpr (RD_RC4096_TWTAB) {
    if (t < 240) tw2[t] = tab[4096 + 15 * 256 + t];
#pragma unroll
    for (int k = 1; k < 16; ++k) w1[k - 1] = tab[4096 + (k - 1) * 256 + t];
  } else {
    if (t < 240) tw2[t] = root_of<256>(((t & 15) * (t / 16 + 1)) & 255);
#pragma unroll
    for (int k = 1; k < 16; ++k) w1[k - 1] = root_of<4096>((t * k) & 4095);
  }
#if !RD_RC4096_MFMA
  // the filter H[k0 + 16 k1 + 256 r] for this thread's (k0, k1) = (g, l), held for every line
  float2 h[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) h[r] = tab[r * 256 + t];
#endif
  __syncthreads();
  for (int64_t line = blockIdx.x; line < lines; line += stride) {
    float2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (HALF)
        v[i] = h2_to_f2(nxt[i]);
      else
        v[i] = nxt[i];
    }
    // ---- forward
    Dft<16, -1>::run(v);
    if constexpr (DER) {
      twiddles_from_powers<false>(v, w1);
    } else {
#pragma unroll
      for (int k = 1; k < 16; ++k) v[k] = cmul(v[k], w1[k - 1]);
    }
    // No barrier before these writes: thread t writes element t of every region, exactly the
    // elements it alone read in the previous line's last exchange (its LDS accesses execute in
    // order), and every other access to them lies on the far side of the barriers below.
#pragma unroll
    for (int k = 0; k < 16; ++k) lds[REG * k + t] = v[k];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n1 = dft_input_order<16>(i);
      v[n1] = lds[REG * g + l + 16 * n1];
    }
    Dft<16, -1>::run(v);
#pragma unroll
    for (int k = 1; k < 16; ++k) v[k] = cmul(v[k], tw2[(k - 1) * 16 + l]);
#if RD_RC4096_MFMA
    // Stage c, the filter and the mirror stage c as matrix products on the matrix cores: for each
    // of this wave's four regions k0 (a batch of 16 vectors k1, 16 points n0 each),
    // Y = F X (F the 16-point DFT matrix, X[n0][k1]), Y times the filter, Z = conj(F) Y.
    {
      exchange_sync<true>();
#pragma unroll
      for (int k = 0; k < 16; ++k) lds[REG * g + 17 * k + l] = v[k];
      exchange_sync<true>();
      const int w4 = (t >> 6) * 4, lq = t & 15, lg = (t >> 4) & 3;
      // k step s takes the points n0 = 4 lg + s of lane group lg: X in the B layout (column k1 =
      // lane % 16), F in the A layout (row = lane % 16), and the product's rows 4 lg + i
      // (i = 0..3) in the same lane group, ready as the next product's B operand.
      float fr[4], fi[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float2 e = root_of<16>((lq * (4 * lg + st)) & 15);  // e^{-j 2 pi row k / 16}
        fr[st] = e.x;
        fi[st] = e.y;
      }
      const float2* hl = opaque(tab);
      rdf_v4f yr[4], yi[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        rdf_v4f ar = {0.f, 0.f, 0.f, 0.f}, ai = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float2 x = lds[REG * (w4 + b) + 17 * lq + 4 * lg + st];
          ar = __builtin_amdgcn_mfma_f32_16x16x4f32(fr[st], x.x, ar, 0, 0, 0);
          ar = __builtin_amdgcn_mfma_f32_16x16x4f32(fi[st], -x.y, ar, 0, 0, 0);
          ai = __builtin_amdgcn_mfma_f32_16x16x4f32(fi[st], x.x, ai, 0, 0, 0);
          ai = __builtin_amdgcn_mfma_f32_16x16x4f32(fr[st], x.y, ai, 0, 0, 0);
        }
        // the filter (carries 1/N) at X[k0 + 16 k1 + 256 k2], k2 = 4 lg + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 y = cmul(make_float2(ar[i], ai[i]), hl[(4 * lg + i) * 256 + 16 * (w4 + b) + lq]);
          ar[i] = y.x;
          ai[i] = y.y;
        }
        yr[b] = ar;
        yi[b] = ai;
      }
      exchange_sync<true>();
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        rdf_v4f zr = {0.f, 0.f, 0.f, 0.f}, zi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          zr = __builtin_amdgcn_mfma_f32_16x16x4f32(fr[st], yr[b][st], zr, 0, 0, 0);
          zr = __builtin_amdgcn_mfma_f32_16x16x4f32(fi[st], yi[b][st], zr, 0, 0, 0);
          zi = __builtin_amdgcn_mfma_f32_16x16x4f32(fi[st], -yr[b][st], zi, 0, 0, 0);
          zi = __builtin_amdgcn_mfma_f32_16x16x4f32(fr[st], yi[b][st], zi, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lds[REG * (w4 + b) + 17 * lq + 4 * lg + i] = make_float2(zr[i], zi[i]);
      }
      // The next line's loads go out here, once the products' registers are free.
      load(nxt, line + stride);
      exchange_sync<true>();
    }
#else
    exchange_sync<true>();
#pragma unroll
    for (int k = 0; k < 16; ++k) lds[REG * g + 17 * k + l] = v[k];
    exchange_sync<true>();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n0 = dft_input_order<16>(i);
      v[n0] = lds[REG * g + 17 * l + n0];
    }
    Dft<16, -1>::run(v);
    // ---- filter (carries 1/N)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = cmul(v[r], h[r]);
    // The next line's loads go out here, once the filter registers are free.
    load(nxt, line + stride);
    // ---- inverse
    Dft<16, +1>::run(v);
    exchange_sync<true>();
#pragma unroll
    for (int n0 = 0; n0 < 16; ++n0) lds[REG * g + 17 * l + n0] = v[n0];
    exchange_sync<true>();
#endif
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = dft_input_order<16>(i);
      v[k] = lds[REG * g + 17 * k + l];
    }
#pragma unroll
    for (int k = 1; k < 16; ++k) {
      float2 w = tw2[(k - 1) * 16 + l];
      w.y = -w.y;
      v[k] = cmul(v[k], w);
    }
    Dft<16, +1>::run(v);
    exchange_sync<true>();
#pragma unroll
    for (int n1 = 0; n1 < 16; ++n1) lds[REG * g + l + 16 * n1] = v[n1];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = dft_input_order<16>(i);
      v[k] = lds[REG * k + t];
    }
    if constexpr (DER) {
      twiddles_from_powers<true>(v, w1);
    } else {
#pragma unroll
      for (int k = 1; k < 16; ++k) {
        float2 w = w1[k - 1];
        w.y = -w.y;
        v[k] = cmul(v[k], w);
      }
    }
    Dft<16, +1>::run(v);
    if constexpr (HALF)
      store_line_h<N, T, 16, SAUX>(v, LineIOh(out, N, line, 1, lines), 0, t);
    else
      store_line<N, T, 16, SAUX>(v, LineIO(static_cast<float2*>(out), N, line, 1, lines), 0, t);
    touch<16>(nxt);
  }
}

// ------------------------------------------------------------------------------------------
// Range compression of 16384-sample lines as four steps inside one workgroup of 16 waves, two
// barriers per line.  With n = t + 1024 n_a (t < 1024, thread t) and k = k_a + 16 k_m:
//   a: DFT16 over n_a -> k_a, times W_16384^{t k_a}                  (thread t, registers)
//   exchange: sub-line k_a (element t) to wave k_a                    (workgroup barrier)
//   m: 1024-point transform over t -> k_m in wave k_a: passes 16, 4, 16 with wave-local
//      exchanges in the wave's own LDS row (lane l ends holding k_m = l + 64 r)
// then the filter H[k_a + 16 k_m], the 1024-point inverse of each sub-line in its wave, the
// sub-lines back to columns (the second barrier), the conjugate twiddles and the inverse DFT16,
// leaving y[t + 1024 n_a] in thread t.  A wave reads and writes only its own LDS row between the
// two barriers, and the next line's first exchange writes exactly the elements each thread read
// in the last one, so no other barrier is needed.  The filter (in the order the threads hold it)
// and the twiddles W_16384^{t k} come from the plan's table; the 1024-point pass twiddles live
// in LDS.  The earlier form (Stockham passes 8, 16, 16, 8 over all 1024 threads) made three
// workgroup exchanges per direction, twelve barriers per line.  Only the twiddles W^t, W^2t, W^4t,
// W^8t are held, the others formed as products; the binary16 form keeps its prefetch packed.
#ifndef RD_RC_16384
#define RD_RC_16384 1
#endif
#ifndef RD_RC_16384_HALF
#define RD_RC_16384_HALF 1  // binary16 storage through the same kernel (else the Stockham kernel)
#endif
// the filter in the order the threads hold it, then W_16384^{t k} for k = 1, 2, 4, 8 (the kernel
// forms the other eleven stage-a twiddles as products)
constexpr int kRc16kTab = 16 * 1024 + 4 * 1024;
void rc16k_tab_fill(const float2* H, const float2* roots, float2* out) {
  for (int r = 0; r < 16; ++r)
    for (int t = 0; t < 1024; ++t) out[r * 1024 + t] = H[(t >> 6) + 16 * (t & 63) + 1024 * r];
  for (int i = 0; i < 4; ++i)
    for (int t = 0; t < 1024; ++t) out[16384 + i * 1024 + t] = roots[(t << i) & 16383];
}

template <int SAUX, bool HALF = false>
__global__ void __launch_bounds__(1024)
    k_range_compress_16384(const void* in, void* out, const float2* __restrict__ tab, int64_t lines) {
  constexpr int N = 16384, T = 1024, M = 1024, ROW = lds_len(M);
  using SL = L_16_4_16;  // palindromic: the forward output layout is the inverse input layout
  using TC = TwCache<M, 64, 1, SL>;
  static_assert(TC::LDS > 0 && 16 * ROW + TC::LDS <= 163840 / 8, "LDS budget");
  __shared__ float2 lds[16 * ROW + TC::LDS];
  RD_POISON_LDS(lds);
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  float2* row = lds + wv * ROW;  // this wave's sub-line and exchange buffer
  const int64_t stride = gridDim.x;
  using Pre = typename std::conditional<HALF, unsigned int, float2>::type;
  auto load = [&](Pre* dst, int64_t line) {
    if constexpr (HALF)
      load_line_h_packed<N, T, 16>(dst, LineIOh(in, N, line, 1, lines), 0, t);
    else
      load_line<N, T, 16>(dst, LineIO(static_cast<const float2*>(in), N, line, 1, lines), 0, t);
  };
  Pre nxt[16];
  load(nxt, blockIdx.x);
  TC twc;
  twc.load_all(tab, lds + 16 * ROW, lane, t, T);
  // W_16384^{t k}: only k = 1, 2, 4, 8 are held and the other eleven are formed as products where
  // they are applied.  The registers this frees let the next line's loads go out earlier: after
  // the filter multiply (float32: 115 VGPRs; holding all fifteen took 125 and put the loads after
  // the inverse sub-line transform, 1.8% slower) or, with the binary16 prefetch packed, right
  // after the first exchange (117 VGPRs; 4% faster than after the inverse sub-line transform).
  constexpr int NW = 4;
  float2 w1[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) w1[i] = tab[16384 + i * 1024 + t];
  __syncthreads();
  for (int64_t line = blockIdx.x; line < lines; line += stride) {
    float2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (HALF)
        v[i] = h2_to_f2(nxt[i]);
      else
        v[i] = nxt[i];
    }
    // ---- forward: stage a
    Dft<16, -1>::run(v);
    twiddles_from_powers<false>(v, w1);
#pragma unroll
    for (int k = 0; k < 16; ++k) lds[k * ROW + t] = v[k];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = dft_input_order<16>(i);
      v[r] = row[lane + 64 * r];
    }
    if constexpr (HALF) load(nxt, line + stride);
    // the filter for this thread's outputs: float32 issues its loads before the forward sub-line
    // transform, which then covers their cache latency (915 -> 910 us per 16384^2 launch); the
    // binary16 form, whose prefetch is in flight there, loads it after (earlier, it spills)
    constexpr bool HEARLY = !HALF;
    float2 h[16];
    if constexpr (HEARLY) {
      const float2* hl = opaque(tab);
#pragma unroll
      for (int r = 0; r < 16; ++r) h[r] = hl[r * 1024 + t];
    }
    PassesCached<M, 64, -1, 1, SL, true>::run(v, row, twc, lane);
    if constexpr (!HEARLY) {
      const float2* hl = opaque(tab);
#pragma unroll
      for (int r = 0; r < 16; ++r) h[r] = hl[r * 1024 + t];
    }
    // ---- filter (carries 1/N)
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = cmul(v[r], h[r]);
    if constexpr (!HALF) load(nxt, line + stride);
    // ---- inverse
    PassesCached<M, 64, +1, 1, SL, true>::run(v, row, twc, lane);
    exchange_sync<true>();
#pragma unroll
    for (int r = 0; r < 16; ++r) row[lane + 64 * r] = v[r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = dft_input_order<16>(i);
      v[k] = lds[k * ROW + t];
    }
    twiddles_from_powers<true>(v, w1);
    Dft<16, +1>::run(v);
    if constexpr (HALF)
      store_line_h<N, T, 16, SAUX>(v, LineIOh(out, N, line, 1, lines), 0, t);
    else
      store_line<N, T, 16, SAUX>(v, LineIO(static_cast<float2*>(out), N, line, 1, lines), 0, t);
    touch<16>(nxt);
  }
}

// ------------------------------------------------------------------------------------------
// Range compression of 6000-sample lines as four steps inside one workgroup of 10 waves, two
// barriers per line.  With n = t + 600 n_a (thread t < 600: every wave's line accesses are whole
// 512-byte segments, 64-byte aligned; threads 600..639 idle outside the sub-line transforms) and
// k = k_a + 10 k_m:
//   a: DFT10 over n_a -> k_a, times W_6000^{t k_a}                  (thread t, registers)
//   exchange: sub-line k_a (element t) to wave k_a                    (workgroup barrier)
//   m: 600-point transform over t -> k_m in wave k_a: passes 10, 6, 10 (prime-factor DFT10 and
//      DFT6) with wave-local exchanges in the wave's own LDS row (lane l < 60 ends holding
//      k_m = l + 60 r)
// then the filter H[k_a + 10 k_m], the inverse of each sub-line in its wave, the sub-lines back
// to columns (the second barrier), the conjugate twiddles and the inverse DFT10, leaving
// y[t + 600 n_a] in thread t.  The hazards are those of the 16384-point kernel.  About 56 KB of
// LDS, so two workgroups share a CU.  The earlier form (passes 10, 6, 10, 10 over 600 threads)
// made three workgroup exchanges per direction.
#ifndef RD_RC_6000
#define RD_RC_6000 1
#endif
#ifndef RD_RC6000_WPE
#define RD_RC6000_WPE 5
#endif
// the filter in the order the threads hold it, then W_6000^{t k} for k = 1, 2, 4, 8 (the kernel
// forms the other five stage-a twiddles as products)
constexpr int kRc6kTab = 10 * 640 + 4 * 640;
void rc6k_tab_fill(const float2* H, const float2* roots, float2* out) {
  for (int r = 0; r < 10; ++r)
    for (int t = 0; t < 640; ++t) {
      const int w = t >> 6, l = t & 63;
      out[r * 640 + t] = l < 60 ? H[w + 10 * (l + 60 * r)] : make_float2(0.f, 0.f);
    }
  for (int i = 0; i < 4; ++i)
    for (int t = 0; t < 640; ++t) out[6400 + i * 640 + t] = t < 600 ? roots[(t << i) % 6000] : make_float2(1.f, 0.f);
}

template <int SAUX, bool HALF = false>
__global__ void __launch_bounds__(640, RD_RC6000_WPE)
    k_range_compress_6000(const void* in, void* out, const float2* __restrict__ tab, int64_t lines) {
  constexpr int M = 600, ROW = lds_len(M), W = 10;
  using SL = L_10_6_10;
  using TC = TwCache<M, 64, 1, SL>;
  static_assert(TC::LDS > 0, "pass twiddles in LDS");
  __shared__ float2 lds[W * ROW + TC::LDS];
  RD_POISON_LDS(lds);
  const int thr = threadIdx.x, wv = thr >> 6, lane = thr & 63;
  const bool act = thr < 600;    // stage-a column t = thr
  const bool lact = lane < 60;   // lanes of the 600-point sub-line transform
  const int t = thr;
  float2* row = lds + wv * ROW;
  const int64_t stride = gridDim.x;
  constexpr int ES = HALF ? 4 : 8;
  // element t + 600 n_a of a line: lane offset t * ES (past the resource for idle lanes, so their
  // loads read zero and their stores are dropped), pass offset n_a * 600 * ES (scalar)
  const uint32_t off = act ? uint32_t(t) * ES : kBufOff;
  auto rsrc = [&](const void* base, int64_t line) {
    const int64_t n = line < lines ? 1 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base) + line * 6000 * ES), 0,
                                             int(n * 6000 * ES), kBufDword3);
  };
  using Pre = typename std::conditional<HALF, unsigned int, float2>::type;
  auto load = [&](Pre* dst, int64_t line) {
    const __amdgpu_buffer_rsrc_t rs = rsrc(in, line < lines ? line : 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int r = dft_input_order<10>(i);
      if constexpr (HALF)
        dst[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, line < lines ? off : kBufOff, r * 600 * ES, kBufNonTemporal);
      else
        dst[r] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs, line < lines ? off : kBufOff,
                                                                                 r * 600 * ES, kBufNonTemporal));
    }
  };
  Pre nxt[10];
  load(nxt, blockIdx.x);
  TC twc;
  twc.load_all(tab, lds + W * ROW, lane, thr, 640);
  // W_6000^{t k}, k = 1..9: only k = 1, 2, 4, 8 are held and the others are formed as products
  // where they are applied, which leaves the registers to hold the filter H[k_a + 10 k_m] (this
  // thread's outputs) across lines: 96 VGPRs, still two workgroups per CU
  float2 w1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w1[i] = tab[6400 + i * 640 + thr];
  float2 h[10];
#pragma unroll
  for (int r = 0; r < 10; ++r) h[r] = tab[r * 640 + thr];
  __syncthreads();
  for (int64_t line = blockIdx.x; line < lines; line += stride) {
    float2 v[MaxRegs<M, 64, SL>::value];  // 12: the radix-6 pass gives some lanes two butterflies
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      if constexpr (HALF)
        v[i] = h2_to_f2(nxt[i]);
      else
        v[i] = nxt[i];
    }
    // ---- forward: stage a
    Dft<10, -1>::run(v);
    twiddles_from_powers<false, 10>(v, w1);
    if (act) {
#pragma unroll
      for (int k = 0; k < 10; ++k) lds[k * ROW + t] = v[k];
    }
    __syncthreads();
    if (lact) {
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int r = dft_input_order<10>(i);
        v[r] = row[lane + 60 * r];
      }
    }
    PassesCached<M, 64, -1, 1, SL, true>::run(v, row, twc, lane);
    // ---- filter (carries 1/N)
#pragma unroll
    for (int r = 0; r < 10; ++r) v[r] = cmul(v[r], h[r]);
    // ---- inverse
    PassesCached<M, 64, +1, 1, SL, true>::run(v, row, twc, lane);
    load(nxt, line + stride);
    exchange_sync<true>();
    if (lact) {
#pragma unroll
      for (int r = 0; r < 10; ++r) row[lane + 60 * r] = v[r];
    }
    __syncthreads();
    if (act) {
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int k = dft_input_order<10>(i);
        v[k] = lds[k * ROW + t];
      }
    }
    twiddles_from_powers<true, 10>(v, w1);
    Dft<10, +1>::run(v);
    {
      const __amdgpu_buffer_rsrc_t rs = rsrc(out, line);
#pragma unroll
      for (int r = 0; r < 10; ++r) {
        if constexpr (HALF)
          __builtin_amdgcn_raw_buffer_store_b32(f2_to_h2(v[r]), rs, off, r * 600 * ES, SAUX);
        else
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(rdf_v2u, v[r]), rs, off, r * 600 * ES, SAUX);
      }
    }
    touch<10>(nxt);
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
  RD_POISON_LDS(lds);
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * C::LDS;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < lines; l0 += int64_t(gridDim.x) * C::LPW) {
    float2 v[C::P];
    load_line<N, T, RI>(v, LineIO(in, N, l0, C::LPW, lines), grp * N, tid);
    Passes<N, T, DIR, 1, L, C::WAVE>::run(v, my, tw, tid);
    if (scale != 1.0f) {
#pragma unroll
      for (int i = 0; i < C::P; ++i) v[i] = cscale(v[i], scale);
    }
    store_line<N, T, RO>(v, LineIO(out, N, l0, C::LPW, lines), grp * N, tid);
  }
}

// ------------------------------------------------------------------------------------------
// Azimuth transforms without corner turns (four-step over the rows of the [Na][Nr] array).
// With Na = A B, row m = B m1 + m2 and Doppler k = k1 + A k2:
//   forward step 1 (strided): for each m2, DFT_A over rows B m1 + m2, then x W_Na^{m2 k1};
//                              row B k1 + m2 then holds Y[k1][m2]
//   forward step 2 (block):    for each k1, DFT_B over the contiguous rows B k1 + m2;
//                              row B k1 + k2 then holds X[k1 + A k2]  (Doppler-digit order)
//   inverse step 1 (block):    for each k1, DFT_B^-1 over rows B k1 + k2, then x W_Na^{-m2 k1}
//   inverse step 2 (strided):  for each m2, DFT_A^-1 over rows B k1 + m2 -> row B m1 + m2.
// A workgroup takes one row set (L rows) x 64 columns; each lane owns one column, so every
// global access of a wave is one contiguous 512-byte row segment (256 bytes with binary16
// storage, whose steps also scale every output by `scale` to keep the values in range).  In
// place (out may equal in).
struct ColGeom {
  int64_t cols;      // row length (elements)
  int base_mul;      // first row of row set g = g * base_mul
  int stride;        // row stride inside a set
  int chunks;        // column chunks of 64
  int na;            // total transform length (for the inter-step twiddle), power of two
  int twiddle;       // multiply output t by W_Na^{DIR g t} after the transform
  float scale;       // binary16 storage only: every output times scale
};

template <int L, int DIR, int AUX, bool HALF = false>
__global__ void __launch_bounds__(ColCfg<L>::WG)
    k_col_fft(const void* in, void* out, const float2* __restrict__ tw, ColGeom cg, uint32_t bytes) {
  using C = ColCfg<L>;
  using LST = typename std::conditional<(DIR < 0), typename C::Fwd, typename C::Inv>::type;
  constexpr int T = C::T;
  constexpr int RI = ListInfo<LST>::first;
  constexpr int RO = ListInfo<LST>::last;
  using TC = TwCache<L, T, 1, LST>;
  static_assert(Geom<L, T, RI>::FULL && Geom<L, T, RO>::FULL,
                "the column loads and stores below assume every lane's butterflies are live");
  __shared__ float2 lds[C::COLS * C::LDS + (TC::LDS > 0 ? TC::LDS : 1)];
  __shared__ float2 step_tw[L];  // inter-step twiddles W_Na^{DIR g t}, t < L
  RD_POISON_LDS(lds);
  RD_POISON_LDS(step_tw);
  const int col = threadIdx.x & 63;
  const int tid = threadIdx.x >> 6;
  float2* my = lds + col * C::LDS;
  TC twc;
  twc.load_all(tw, lds + C::COLS * C::LDS, tid, threadIdx.x, C::WG);
  const int g = blockIdx.x / cg.chunks;
  if (cg.twiddle && threadIdx.x < L) {
    // exact argument: (g t mod Na) / Na; read after the passes' barriers
    const int gt = g * int(threadIdx.x);
    const int m = (cg.na & (cg.na - 1)) == 0 ? gt & (cg.na - 1) : gt % cg.na;
    float sn, cs;
    sincospif(float(m) * (2.0f / float(cg.na)), &sn, &cs);
    step_tw[threadIdx.x] = make_float2(cs, DIR > 0 ? sn : -sn);
  }
  const int64_t c = int64_t(blockIdx.x - g * cg.chunks) * 64 + col;
  const bool live = c < cg.cols;
  // Element t of this lane's column lies at byte base + t * rowstep (32-bit: the array is
  // below 4 GiB).  Lanes past the last column read the last column and store nothing.  (The
  // same offsets split into a per-lane base and a wave-uniform scalar part measured ~5% slower
  // on the 16384-row steps.)
  constexpr int ES = HALF ? 4 : 8;  // bytes per element
  const uint32_t base = uint32_t((int64_t(g) * cg.base_mul * cg.cols + (live ? c : cg.cols - 1)) * ES);
  const uint32_t rowstep = uint32_t(int64_t(cg.stride) * cg.cols * ES);
  const __amdgpu_buffer_rsrc_t rin =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(in), 0, int(bytes), kBufDword3);
  const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(out, 0, int(bytes), kBufDword3);
  float2 v[C::P];
  {
    using G = Geom<L, T, RI>;
#pragma unroll
    for (int b = 0; b < G::B; ++b) {
      const int j = tid + b * T;
#pragma unroll
      for (int r = 0; r < RI; ++r) {
        const uint32_t off = base + uint32_t(j + r * G::NB) * rowstep;
        if constexpr (HALF)
          v[b * RI + r] = h2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(rin, off, 0, AUX));
        else
          v[b * RI + r] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rin, off, 0, AUX));
      }
    }
  }
  PassesCached<L, T, DIR, 1, LST>::run(v, my, twc, tid);
  {
    using G = Geom<L, T, RO>;
#pragma unroll
    for (int b = 0; b < G::B; ++b) {
      const int j = tid + b * T;
#pragma unroll
      for (int r = 0; r < RO; ++r) {
        float2 x = v[b * RO + r];
        if (cg.twiddle) x = cmul(x, step_tw[j + r * G::NB]);
        const uint32_t off = base + uint32_t(j + r * G::NB) * rowstep;
        if constexpr (HALF) {
          if (live) __builtin_amdgcn_raw_buffer_store_b32(f2_to_h2(cscale(x, cg.scale)), rout, off, 0, AUX);
        } else {
          if (live) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(rdf_v2u, x), rout, off, 0, AUX);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// RCMC + azimuth filter per Doppler row (constants in rd_kernels.hpp).  A row is processed in
// chunks of CH outputs; a chunk's input window (3 samples before it, CH samples, and `halo`
// samples after it, zero outside the row) is staged in LDS, so every tap is a plain LDS read.
// Rows up to 4096 samples are one chunk, staged between zero margins written once; longer rows
// split into 4096-sample chunks, which keeps the staging buffer small enough for several
// workgroups per CU.  The chunks of one row are processed in order by one thread group, which
// makes the stage safe in place (out == in): a chunk's window reads only samples at or after
// its own start from memory (nothing this group has stored yet, and no other group touches the
// row), and the 3 samples before it come from the previous chunk's staged input in LDS.  Shift
// and filter phase are formed in float64 (the phase reaches ~1e7 rad) and reduced before they
// are taken to float32.  HALF: binary16 rows (4 bytes a sample) in and out, float32 arithmetic.
template <int N>
struct RowStage {
  static constexpr int CH = (N > 4096 && N % 4096 == 0) ? 4096 : N;  // outputs per chunk
  static constexpr int CHUNKS = N / CH;
  static constexpr int T = CHUNKS == 1 ? LineCfg<N>::T : 256;          // threads per row
  static constexpr int LPW = CHUNKS == 1 ? LineCfg<N>::LPW : 1;        // rows per workgroup
  static constexpr int WG = T * LPW;
  static constexpr int MARGIN = N / 8;       // staged samples after a chunk (shift + 5 <= MARGIN)
  static constexpr int LEN = 3 + CH + MARGIN;
  static constexpr int P = LineCfg<N>::P;    // registers per thread for a chunk
};
// Rows of any length (given at run time): 512-sample chunks with up to 1024 staged samples after
// each, two rows per workgroup; the row's buffer resource reads zero past its end and drops
// stores there.
template <>
struct RowStage<0> {
  static constexpr int CH = 512;
  static constexpr int CHUNKS = 0;  // run time
  static constexpr int T = 128;
  static constexpr int LPW = 2;
  static constexpr int WG = T * LPW;
  static constexpr int MARGIN = 1024;
  static constexpr int LEN = 3 + CH + MARGIN;
  static constexpr int P = CH / T;
};

// row I/O of the row stage: float32 or binary16 storage
template <bool HALF>
struct RowIO;
template <>
struct RowIO<false> {
  using IO = LineIO;
  __device__ static IO make(const void* b, int n, int64_t first, int count, int64_t total) {
    return LineIO(static_cast<const float2*>(b), n, first, count, total);
  }
  template <int AUX>
  __device__ static float2 one(const IO& io, int i) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(io.rsrc, i * 8, 0, AUX));
  }
  template <int N, int T, int R, int AUX>
  __device__ static void load(float2* v, const IO& io, int e0, int tid) { load_line<N, T, R, AUX>(v, io, e0, tid); }
  template <int N, int T, int R, int AUX>
  __device__ static void store(const float2* v, const IO& io, int e0, int tid) {
    store_line<N, T, R, AUX>(v, io, e0, tid);
  }
};
template <>
struct RowIO<true> {
  using IO = LineIOh;
  __device__ static IO make(const void* b, int n, int64_t first, int count, int64_t total) {
    return LineIOh(b, n, first, count, total);
  }
  template <int AUX>
  __device__ static float2 one(const IO& io, int i) {
    return h2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(io.rsrc, i * 4, 0, AUX));
  }
  template <int N, int T, int R, int AUX>
  __device__ static void load(float2* v, const IO& io, int e0, int tid) { load_line_h<N, T, R, AUX>(v, io, e0, tid); }
  template <int N, int T, int R, int AUX>
  __device__ static void store(const float2* v, const IO& io, int e0, int tid) {
    store_line_h<N, T, R, AUX>(v, io, e0, tid);
  }
};

// The outputs of one staged chunk (starting at row sample n0) into v: thread tid computes chunk
// positions j + r NB (the layout of the chunk's loads and stores).
template <int CH, int T, int R0>
__device__ __forceinline__ void rcmc_chunk(float2* v, const float2* my, const AzRowConst& c, int n0,
                                           double alpha, double beta, double gamma, double delta, int tid) {
  using G = Geom<CH, T, R0>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
      // filter phasor exp(j 2 pi (gamma + n delta)) for n = n0 + j + r NB: exact at r = 0
      // (phase reduced in float64), then advanced by the exact step rotation
      float2 z = make_float2(1.f, 0.f), rot = make_float2(1.f, 0.f);
      if (c.filter) {
        const double c0 = gamma + double(n0 + j) * delta;
        const double c1 = double(G::NB) * delta;
        float sn, cs;
        sincospif(2.0f * float(c0 - rint(c0)), &sn, &cs);
        z = make_float2(cs * c.inv_na, sn * c.inv_na);
        sincospif(2.0f * float(c1 - rint(c1)), &sn, &cs);
        rot = make_float2(cs, sn);
      }
      // the shift x = alpha + n beta (n = n0 + j + r NB; x >= 0) in 32.32 fixed point: rounded
      // once from float64 at r = 0, then advanced by the rounded step NB beta (accumulated error
      // below 1e-8 samples over a thread's outputs); the high word is floor(x), the low word the
      // fraction
      int64_t X = static_cast<int64_t>(rint((alpha + double(n0 + j) * beta) * 4294967296.0));
      const int64_t S = static_cast<int64_t>(rint(double(G::NB) * beta * 4294967296.0));
#pragma unroll
      for (int r = 0; r < R0; ++r, X += S) {
        const int m = j + r * G::NB;  // position in the chunk
        const int fl = static_cast<int>(X >> 32);
        const float xf = fmaf(float(static_cast<uint32_t>(X)), 0x1p-32f, -0.5f);
        const float y = xf * xf;
        const float2* tap = my + (m + fl);  // tap t reads sample n0 + m + fl + t - 3
        float2 acc = make_float2(0.f, 0.f);
        float es = 0.f;  // sum of the even parts: the weights sum to 2 es
#pragma unroll
        for (int q = 0; q < kRcmcTaps / 2; ++q) {
          float e = c.w.even[q][kRcmcEven - 1];
#pragma unroll
          for (int mm = kRcmcEven - 2; mm >= 0; --mm) e = fmaf(e, y, c.w.even[q][mm]);
          float o = c.w.odd[q][kRcmcOdd - 1];
#pragma unroll
          for (int mm = kRcmcOdd - 2; mm >= 0; --mm) o = fmaf(o, y, c.w.odd[q][mm]);
          const float wa = fmaf(xf, o, e);    // tap j = -q   (t = 3 - q)
          const float wb = fmaf(-xf, o, e);   // tap j = 1 + q (t = 4 + q)
          const float2 sa = tap[3 - q], sb = tap[4 + q];
          acc.x = fmaf(wa, sa.x, fmaf(wb, sb.x, acc.x));
          acc.y = fmaf(wa, sa.y, fmaf(wb, sb.y, acc.y));
          es += e;
        }
        const float sc = 0.5f * __builtin_amdgcn_rcpf(es);
        float2 o = make_float2(acc.x * sc, acc.y * sc);
        if (c.filter) {
          o = cmul(o, z);
          z = cmul(z, rot);
        }
        v[b * R0 + r] = o;
      }
    }
  }
}

template <int N, int AUX, bool HALF = false>
__global__ void __launch_bounds__(RowStage<N>::WG)
    k_rcmc_mf(const void* in, void* out, AzRowConst c, int64_t rows, int n_rt) {
  using RIO = RowIO<HALF>;
  using RS = RowStage<N>;
  constexpr bool RT = RS::CHUNKS == 0;        // row length n_rt at run time
  const int nl = RT ? n_rt : N;              // samples per row
  const int chunks = RT ? (n_rt + RS::CH - 1) / RS::CH : RS::CHUNKS;
  constexpr int T = RS::T;
  constexpr int CH = RS::CH;
  constexpr int R0 = CH / T;  // each thread holds chunk samples j + r T, r < CH/T
  static_assert(CH % T == 0 && R0 <= RS::P, "row layout");
  using G = Geom<CH, T, R0>;
  __shared__ float2 lds[RS::LPW * RS::LEN];
  RD_POISON_LDS(lds);
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * RS::LEN;
  for (int i = threadIdx.x; i < RS::LPW * RS::LEN; i += RS::WG) lds[i] = make_float2(0.f, 0.f);
  // one row per thread group: rows [r0, r0 + LPW) per workgroup pass
  for (int64_t r0 = int64_t(blockIdx.x) * RS::LPW; r0 < rows; r0 += int64_t(gridDim.x) * RS::LPW) {
    const bool live_row = r0 + grp < rows;
    const int64_t row = live_row ? r0 + grp : rows - 1;
    const int k = int(row / c.B) + c.A * int(row % c.B);
    const double alpha = c.row[4 * k], beta = c.row[4 * k + 1];
    const double gamma = c.row[4 * k + 2], delta = c.row[4 * k + 3];
    float2 v[RS::P];
    if constexpr (RS::CHUNKS == 1) {
      // the whole row is the chunk; the zero margins around it are never written
      RIO::template load<CH, T, R0, AUX>(v, RIO::make(in, N, r0, RS::LPW, rows), grp * N, tid);
      __syncthreads();  // the previous row's taps have been read
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        const int j = tid + b * T;
        if (G::live(j)) {
#pragma unroll
          for (int r = 0; r < R0; ++r) my[3 + j + r * G::NB] = v[b * R0 + r];
        }
      }
      __syncthreads();
      rcmc_chunk<CH, T, R0>(v, my, c, 0, alpha, beta, gamma, delta, tid);
      RIO::template store<CH, T, R0, AUX>(v, RIO::make(out, N, r0, RS::LPW, rows), grp * N, tid);
    } else {
      // rows past the end: an empty resource (loads read zero, stores are dropped)
      const typename RIO::IO src = RIO::make(in, nl, live_row ? row : rows, 1, rows);
      const typename RIO::IO dst = RIO::make(out, nl, live_row ? row : rows, 1, rows);
      for (int ch = 0; ch < chunks; ++ch) {
        const int n0 = ch * CH;
        RIO::template load<CH, T, R0, AUX>(v, src, n0, tid);
        // Window edges: slots 0..2 hold the 3 samples before the chunk -- zero before the row,
        // else the previous chunk's last 3 input samples, still staged at my[CH..CH+2] (read
        // before the barrier below, after which the slots are overwritten); slots after the
        // chunk hold the first `halo` samples that follow it (zero past the row), the first
        // pass of them loaded with the chunk.
        float2 pre = make_float2(0.f, 0.f);
        int hs = -1;  // this thread's window slot, if any
        if (tid < 3) {
          hs = tid;
          if (ch > 0) pre = my[CH + tid];
        } else if (tid < 3 + c.halo) {
          const int sidx = n0 + CH + (tid - 3);
          hs = CH + tid;
          if (sidx < nl) pre = RIO::template one<AUX>(src, sidx);
        }
        __syncthreads();  // the previous chunk's taps and edge samples have been read
#pragma unroll
        for (int b = 0; b < G::B; ++b) {
          const int j = tid + b * T;
          if (G::live(j)) {
#pragma unroll
            for (int r = 0; r < R0; ++r) my[3 + j + r * G::NB] = v[b * R0 + r];
          }
        }
        if (hs >= 0) my[hs] = pre;
        for (int i = tid + T; i < 3 + c.halo; i += T) {  // halos longer than one pass
          const int sidx = n0 + CH + (i - 3);
          my[CH + i] = sidx < nl ? RIO::template one<AUX>(src, sidx) : make_float2(0.f, 0.f);
        }
        __syncthreads();
        rcmc_chunk<CH, T, R0>(v, my, c, n0, alpha, beta, gamma, delta, tid);
        RIO::template store<CH, T, R0, AUX>(v, dst, n0, tid);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// omega-k row stage (nxmr.cn/news/101525 §3, §3.2): one workgroup group per Doppler row of the
// azimuth-transformed echo.  The row is read rotated by the reference bin, transformed along
// range in registers, multiplied by H times the reference function, staged in LDS in centred
// frequency order, read back through the Stolt mapping with the 8-tap interpolator, inverse
// transformed, and stored rotated back.  The two rotations are the exact forms of the linear
// phase terms exp(+-j 2 pi f 2 (Rref - range_bin0) / c) of the reference function and of the
// registration that follows the mapping (f 2 (Rref - range_bin0) / c = js ref / Nr).
template <int N>
struct OkRow {
  using C = LineCfg<N>;
  static constexpr int CAP = N >= 16384 ? N / 8 : N / 2;  // zero samples staged after a row
  static constexpr int STG = 3 + N + CAP;                  // staging: 3 zeros, the row, CAP zeros
  static constexpr int REG = C::LDS > STG ? C::LDS : STG;  // per line: transform scratch / staging
};

// line I/O rotated by rot (0 <= rot < N): slot e of the line holds sample (e + rot) mod N
// (HALF: binary16 storage through a LineIOh resource)
template <int N, int T, int R, int AUX, bool HALF = false, class IO>
__device__ __forceinline__ void load_line_rot(float2* v, const IO& io, int elem0, int tid, int rot) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        int e = j + r * G::NB + rot;
        e -= e >= N ? N : 0;
        if constexpr (HALF)
          v[b * R + r] = h2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(io.rsrc, uint32_t(elem0 + e) * 4u, 0, AUX));
        else
          v[b * R + r] = __builtin_bit_cast(
              float2, __builtin_amdgcn_raw_buffer_load_b64(io.rsrc, uint32_t(elem0 + e) * 8u, 0, AUX));
      }
    }
  }
}
template <int N, int T, int R, int AUX, bool HALF = false, class IO>
__device__ __forceinline__ void store_line_rot(const float2* v, const IO& io, int elem0, int tid, int rot) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int e = j + r * G::NB + rot;
        e -= e >= N ? N : 0;
        if constexpr (HALF)
          __builtin_amdgcn_raw_buffer_store_b32(f2_to_h2(v[b * R + r]), io.rsrc, uint32_t(elem0 + e) * 4u, 0, AUX);
        else
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(rdf_v2u, v[b * R + r]), io.rsrc,
                                                uint32_t(elem0 + e) * 8u, 0, AUX);
      }
    }
  }
}

// sqrt of a positive normal double (the wavenumbers here are ~1e18..1e21 Hz^2): the hardware
// reciprocal square root refined by one Newton-Raphson step in Goldschmidt form and a final
// residual correction, which leaves an error of a few ulp (the library form adds range scaling
// and special-case handling that these arguments never need).
__device__ __forceinline__ double sqrt_pos(double x) {
  const double y = __builtin_amdgcn_rsq(x);
  double s = x * y, h = 0.5 * y;
  const double e = fma(-h, s, 0.5);
  s = fma(s, e, s);
  h = fma(h, e, h);
  return fma(fma(-s, s, x), h, s);
}

// At 2048 and 4096 three workgroups share a CU (LDS 50-51 KB each) when the kernel fits 168 VGPRs:
// with the per-sample loops fenced (TIGHT below) and the last pass's twiddles formed from powers
// it does, spilling 28-40 B.  Whole omega-k, against two workgroups per CU (207-228 VGPRs):
// 4096^2 277.5-277.9 against 282.5-283.1 us, 4096 x 2048 143.6-143.8 against 146.9-147.0 us.
template <int N, int AUX, bool HALF = false>
__global__ void __launch_bounds__(LineCfg<N>::WG, (N == 2048 || N == 4096 ? 3 : 1))
    k_omega_k_row(const void* in, void* out, const float2* __restrict__ H,
                  const float2* __restrict__ tw, OkConst c, RcmcPoly w, int64_t rows) {
  using RIO = RowIO<HALF>;
  using C = LineCfg<N>;
  using L = typename C::Fwd;
  static_assert(std::is_same<typename C::Fwd, typename C::Inv>::value, "needs Fwd == Inv");
  constexpr int T = C::T;
  constexpr int R0 = ListInfo<L>::first;
  static_assert(R0 == ListInfo<L>::last, "palindromic radix list: spectrum layout = inverse input layout");
  using G = Geom<N, T, R0>;
  using TC = TwCache<N, T, 1, L>;
  constexpr int REG = OkRow<N>::REG;
  __shared__ float2 lds[C::LPW * REG + (TC::LDS > 0 ? TC::LDS : 1)];
  RD_POISON_LDS(lds);
  const int grp = threadIdx.x / T;
  const int tid = threadIdx.x - grp * T;
  float2* my = lds + grp * REG;
  TC twc;
  twc.load_all(tw, lds + C::LPW * REG, tid, threadIdx.x, C::WG);
  if constexpr (C::WAVE && TC::LDS > 0) __syncthreads();
  twc.touch_all();
  const int na = c.A * c.B;
  for (int64_t l0 = int64_t(blockIdx.x) * C::LPW; l0 < rows; l0 += int64_t(gridDim.x) * C::LPW) {
    const int64_t row = l0 + grp < rows ? l0 + grp : rows - 1;  // lines past the end: loads read
                                                                 // zero, stores are dropped
    const int k = int(row / c.B) + c.A * int(row % c.B);
    const double b = double(2 * k < na ? k : k - na) * c.bstep;
    const double b2 = b * b;
    float2 v[C::P];
    // Where registers are tight, the rotation is hidden from the compiler once per row, so the
    // rotated offsets are formed where they are used instead of being hoisted out of the loop
    // (32 registers for the whole kernel otherwise): that buys a wave per SIMD at 256, 512, 2048
    // and 4096 and cuts the spills at 6000 and 16384; elsewhere it only costs ~4% more instructions.
    constexpr bool TIGHT = N <= 512 || N == 2048 || N == 4096 || N == 6000 || N >= 16384;
    int rot = c.ref;
    if constexpr (TIGHT) asm volatile("" : "+s"(rot));
    // At 16384 (1024 threads: at most 128 registers) the per-sample loops below use a copy of
    // the thread index hidden from the compiler once per row, so the values derived from it
    // (bin indices in float64, filter addresses) are formed in the row loop rather than hoisted
    // into registers that then spill.
    int tid_s = tid;
    if constexpr (N >= 16384) asm volatile("" : "+v"(tid_s));
    const typename RIO::IO io_in = RIO::make(in, N, l0, C::LPW, rows);
    load_line_rot<N, T, R0, AUX, HALF>(v, io_in, grp * N, tid, rot);
    PassesCached<N, T, -1, 1, L, C::WAVE>::run(v, my, twc, tid);
    // v = X[kx] H[kx] exp(j 2 pi (k0 - k1 (a - Q))) / Na at range bin kx = j + r NB,
    // a = f0 + js df, Q = sqrt(a^2 - b^2) (float64: the phase reaches ~1e4 turns)
#pragma unroll
    for (int bb = 0; bb < G::B; ++bb) {
      const int j = tid_s + bb * T;
      if (G::live(j)) {
#pragma unroll
        for (int r = 0; r < R0; ++r) {
          const int kx = j + r * G::NB;
          const int js = 2 * kx < N ? kx : kx - N;
          const double a = c.f0 + double(js) * c.df;
          const double q = sqrt_pos(fma(a, a, -b2));
          const double t = fma(-c.k1, a - q, c.k0);
          const float f = float(t - floor(t));     // hardware sin/cos take turns
          const float sn = __builtin_amdgcn_sinf(f), cs = __builtin_amdgcn_cosf(f);
          const float2 h = H[kx];
          const float2 z = make_float2((h.x * cs - h.y * sn) * c.inv_na, (h.x * sn + h.y * cs) * c.inv_na);
          v[bb * R0 + r] = cmul(v[bb * R0 + r], z);
          if constexpr (TIGHT) group_fence();  // one sample's float64 temporaries at a time
        }
      }
    }
    __syncthreads();  // the forward transform's last reads of this line's scratch are done
    // staging: my[3 + u] = spectrum at centred position u = (kx + N/2) mod N, zero around it
#pragma unroll
    for (int bb = 0; bb < G::B; ++bb) {
      const int j = tid_s + bb * T;
      if (G::live(j)) {
#pragma unroll
        for (int r = 0; r < R0; ++r) {
          int u = j + r * G::NB + N / 2;
          u -= u >= N ? N : 0;
          my[3 + u] = v[bb * R0 + r];
        }
      }
    }
    if (tid < 3) my[tid] = make_float2(0.f, 0.f);
    for (int i = tid; i < c.halo; i += T) my[3 + N + i] = make_float2(0.f, 0.f);
    __syncthreads();
    // Stolt mapping: output at centred position u reads the staged spectrum at
    // x = u + (sqrt(a'^2 + b^2) - a') / df, a' = f0 + (u - N/2) df; x >= u and x <= N - 1 + halo - 5
#pragma unroll
    for (int bb = 0; bb < G::B; ++bb) {
      const int j = tid_s + bb * T;
      if (G::live(j)) {
#pragma unroll
        for (int r = 0; r < R0; ++r) {
          int u = j + r * G::NB + N / 2;
          u -= u >= N ? N : 0;
          const double a = c.f0 + double(u - N / 2) * c.df;
          const double x = double(u) + (sqrt_pos(fma(a, a, b2)) - a) * c.inv_df;
          const double fl = floor(x);
          const float xf = float(x - fl) - 0.5f;
          const float y = xf * xf;
          const float2* tap = my + int(fl);  // tap t reads centred sample fl + t - 3
          float2 acc = make_float2(0.f, 0.f);
          float es = 0.f;
#pragma unroll
          for (int q = 0; q < kRcmcTaps / 2; ++q) {
            float e = w.even[q][kRcmcEven - 1];
#pragma unroll
            for (int mm = kRcmcEven - 2; mm >= 0; --mm) e = fmaf(e, y, w.even[q][mm]);
            float o = w.odd[q][kRcmcOdd - 1];
#pragma unroll
            for (int mm = kRcmcOdd - 2; mm >= 0; --mm) o = fmaf(o, y, w.odd[q][mm]);
            const float wa = fmaf(xf, o, e);
            const float wb = fmaf(-xf, o, e);
            const float2 sa = tap[3 - q], sb = tap[4 + q];
            acc.x = fmaf(wa, sa.x, fmaf(wb, sb.x, acc.x));
            acc.y = fmaf(wa, sa.y, fmaf(wb, sb.y, acc.y));
            es += e;
          }
          const float sc = 0.5f * __builtin_amdgcn_rcpf(es);
          v[bb * R0 + r] = make_float2(acc.x * sc, acc.y * sc);
          if constexpr (TIGHT) group_fence();
        }
      }
    }
    // (the inverse transform's first exchange begins with a barrier: the staging reads are done)
    PassesCached<N, T, +1, 1, L, C::WAVE>::run(v, my, twc, tid);
    if constexpr (TIGHT) asm volatile("" : "+s"(rot));
    store_line_rot<N, T, R0, AUX, HALF>(v, RIO::make(out, N, l0, C::LPW, rows), grp * N, tid, rot);
  }
}

// ------------------------------------------------------------------------------------------
// Corner turn out[c][r] = in[r][c] of a row-major [rows][cols] complex array (the transpose
// between range lines and azimuth lines in cf-1.com/news/2323550 §5.1-§5.2 and the padded
// shared-memory tiles of nxmr.cn/news/101525 §2.2.1).  A workgroup moves one 64 x 64 tile:
// each wave reads whole 512-byte row segments of the input, the tile passes through LDS with a
// row pitch of 65 elements, and each wave writes whole 512-byte row segments of the output.
// Bank geometry of gfx950 (8-byte writes: 16 lanes over 32 banks; 8-byte reads: 32 lanes over
// 64 banks): the tile writes are runs of consecutive elements and the transposed reads step by
// 65 elements (an odd count), so neither meets a bank conflict.  Edges of ragged shapes are
// masked.  Every element is read once and written once (16 bytes per element).
constexpr int kTurnTile = 64, kTurnPitch = 65;
typedef float rdf_v2f __attribute__((ext_vector_type(2)));

template <int AUX>
__device__ __forceinline__ void turn_load(float2* v, const float2* __restrict__ in, int64_t rows, int64_t cols,
                                          int64_t r0, int64_t c0, int lane, int w) {
  const int64_t c = c0 + lane;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t r = r0 + w + 4 * k;
    float2 x = make_float2(0.f, 0.f);
    if (r < rows && c < cols) {
      const rdf_v2f* src = reinterpret_cast<const rdf_v2f*>(in + r * cols + c);
      const rdf_v2f y = AUX ? __builtin_nontemporal_load(src) : *src;
      x = make_float2(y.x, y.y);
    }
    v[k] = x;
  }
}

// Persistent form: workgroup b moves tiles b, b + G, b + 2G, ... (row-major tile order), and the
// next tile's loads are issued as soon as the current tile is in LDS, so they are in flight
// during the transposed reads and the stores (loads and stores complete in order, so the wait
// for the prefetch does not wait for the stores).
template <int AUX>
__global__ void __launch_bounds__(256)
    k_corner_turn(const float2* __restrict__ in, float2* __restrict__ out, int64_t rows,
                  int64_t cols, int tiles_x, int tiles) {
  __shared__ float2 tile[kTurnTile * kTurnPitch];
  RD_POISON_LDS(tile);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float2 cur[16];
  int t = blockIdx.x;
  if (t < tiles) {
    const int ty = t / tiles_x;
    turn_load<AUX>(cur, in, rows, cols, int64_t(ty) * kTurnTile, int64_t(t - ty * tiles_x) * kTurnTile, lane, w);
  }
  for (; t < tiles; t += gridDim.x) {
    const int ty = t / tiles_x;
    const int64_t r0 = int64_t(ty) * kTurnTile, c0 = int64_t(t - ty * tiles_x) * kTurnTile;
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[(w + 4 * k) * kTurnPitch + lane] = cur[k];
    __syncthreads();
    const int tn = t + int(gridDim.x);
    if (tn < tiles) {
      const int tyn = tn / tiles_x;
      turn_load<AUX>(cur, in, rows, cols, int64_t(tyn) * kTurnTile, int64_t(tn - tyn * tiles_x) * kTurnTile,
                     lane, w);
    }
    const int64_t r = r0 + lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int cc = w + 4 * k;
      const int64_t c = c0 + cc;
      if (c < cols && r < rows) {
        rdf_v2f* dst = reinterpret_cast<rdf_v2f*>(out + c * rows + r);
        const float2 v = tile[lane * kTurnPitch + cc];
        const rdf_v2f y = {v.x, v.y};
        if (AUX)
          __builtin_nontemporal_store(y, dst);
        else
          *dst = y;
      }
    }
    __syncthreads();  // the tile's LDS reads are done before the next tile is written
  }
}

hipError_t launch_corner_turn(const float2* in, float2* out, int64_t rows, int64_t cols,
                              int streaming, hipStream_t s) {
  const int64_t gx = (cols + kTurnTile - 1) / kTurnTile, gy = (rows + kTurnTile - 1) / kTurnTile;
  if (gx * gy > 0x7fffffff) return hipErrorInvalidValue;
  const int tiles = int(gx * gy);
  // persistent grid: the resident workgroups of the whole device (queried once per device)
  // (several host threads may race to fill an entry: they store the same value)
  static std::atomic<int> resident[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int res = resident[dev].load(std::memory_order_relaxed);
  if (res == 0) {
    int occ = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_corner_turn<1>, 256, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidValue;
    res = (occ > 0 ? occ : 1) * (cus > 0 ? cus : 1);
    resident[dev].store(res, std::memory_order_relaxed);
  }
  const int grid = tiles < res ? tiles : res;
  if (streaming)
    hipLaunchKernelGGL(k_corner_turn<1>, dim3(grid), dim3(256), 0, s, in, out, rows, cols, int(gx), tiles);
  else
    hipLaunchKernelGGL(k_corner_turn<0>, dim3(grid), dim3(256), 0, s, in, out, rows, cols, int(gx), tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Back-projection (framerc.cn/news/4459478 §1.1, §2.2, §4.2): for every pixel (along-track x,
// closest-approach slant range r) and every pulse m, the range d = sqrt(r^2 + (x - V m/PRF)^2),
// the range-compressed line m linearly interpolated at bin (d - range_bin0)/dr (zero outside the
// line), times exp(+j 4 pi d / lambda), summed over all pulses.  One lane per pixel; a wave holds
// 64 consecutive range pixels of one along-track row, a workgroup 4 rows, so the pulse loop is
// uniform and each pulse's gathers fall in one short, nearly contiguous stretch of its line
// (read through the cache; the line is a buffer resource, so bins outside it read zero).
// Precision: d = r + delta with delta = a^2 / (r + d) evaluated in float32 without cancellation
// (a = x - V m/PRF formed in float64); the pixel's constant phase 2 r / lambda (turns) and its
// bin offset (r - range_bin0)/dr are split in float64 once per pixel, so the per-pulse float32
// quantities (delta / dr, 2 delta / lambda) stay small; partial sums of 32 pulses go to float64.
// One pulse's contribution to a pixel, added to (sr, si).  xa is the pixel's along-track offset
// from the platform at this pulse, x - V m / PRF, carried in float64 from pulse to pulse (one add
// instead of forming it from m).  ib8 is 8 times the pixel's integer bin offset (clamped to
// [-4 Nr, 4 Nr]); the bin t is clamped to 5 Nr + 2, so every index past the line stays past it
// (ib + t >= Nr + 2) without overflowing 32 bits.
template <bool NATIVE_SINCOS>
__device__ __forceinline__ void bp_pulse(const float2* __restrict__ rc, const BpConst& c, int m, double& xa,
                                         float rf, float fb, int ib8, float k_bin, float k_turn, float t_max,
                                         uint32_t line_bytes, float& sr, float& si) {
  const float a = float(xa);
  xa -= c.step;
  const float a2 = a * a;
  const float d = __builtin_amdgcn_sqrtf(fmaf(rf, rf, a2));   // only in the denominator below
  const float delta = a2 * __builtin_amdgcn_rcpf(rf + d);     // d - r without cancellation
  const float t = fminf(fmaf(delta, k_bin, fb), t_max);       // >= 0: delta >= 0, fb in [0, 1)
  const float fl = floorf(t);
  const float w = t - fl;
  const __amdgpu_buffer_rsrc_t line = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float2*>(rc + int64_t(m) * c.Nr), 0, int(line_bytes), kBufDword3);
  // Two 8-byte loads at bins idx and idx + 1 (idx = ib + fl), each range-checked on its own: a
  // negative idx wraps to an offset far past the line (>= 2^32 - 32 Nr) and reads zero, so idx = -1
  // reads zero and bin 0; idx >= Nr reads zero twice.  The second offset is hidden from the
  // compiler, which would otherwise fuse the pair into one 16-byte load whose range check is
  // all-or-nothing and would drop the last in-line sample.
  const uint32_t off = uint32_t(ib8) + (uint32_t(int(fl)) << 3);
  uint32_t off1 = off + 8u;
  asm volatile("" : "+v"(off1));
  const float2 s0 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(line, off, 0, 0));
  const float2 s1 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(line, off1, 0, 0));
  const float vr = fmaf(w, s1.x - s0.x, s0.x), vi = fmaf(w, s1.y - s0.y, s0.y);
  const float turns = delta * k_turn;
  float sn, cs;
  if constexpr (NATIVE_SINCOS) {
    const float f = __builtin_amdgcn_fractf(turns);   // hardware sin/cos take turns
    sn = __builtin_amdgcn_sinf(f);
    cs = __builtin_amdgcn_cosf(f);
  } else {
    sincospif(2.0f * (turns - rintf(turns)), &sn, &cs);
  }
  sr = fmaf(vr, cs, fmaf(-vi, sn, sr));
  si = fmaf(vr, sn, fmaf(vi, cs, si));
}

template <bool NATIVE_SINCOS>
__global__ void __launch_bounds__(256)
    k_backproject(const float2* __restrict__ rc, float2* __restrict__ img, BpConst c) {
  const int j = int(blockIdx.x) * 64 + int(threadIdx.x & 63);
  const int i = int(blockIdx.y) * 4 + int(threadIdx.x >> 6);
  const double r = c.r0 + double(j) * c.drp;
  double xa = c.x0 + double(i) * c.dx;
  // bin offset of the pixel's closest approach: integer part ib and fraction fb.  ib is clamped to
  // [-4 Nr, 4 Nr] so that the index arithmetic stays in 32 bits; a pixel beyond the clamp reads zero,
  // which is the definition's value unless its range curve still reaches the line, a range excess
  // of more than 3 Nr bins, far outside the float32 domain of the excess and its phase.
  double b0 = (r - c.rb0) * c.inv_dr;
  b0 = b0 < -4.0 * c.Nr ? -4.0 * c.Nr : (b0 > 4.0 * c.Nr ? 4.0 * c.Nr : b0);
  const double ibd = floor(b0);
  const int ib8 = int(ibd) * 8;
  const float fb = float(b0 - ibd);
  const float rf = float(r);
  const float k_bin = float(c.inv_dr), k_turn = float(c.two_over_lam);
  const float t_max = float(5 * c.Nr + 2);
  const uint32_t line_bytes = uint32_t(c.Nr) * 8u;
  double acc_r = 0.0, acc_i = 0.0;
  constexpr int BLK = 32;  // pulses summed in float32 before each float64 accumulation
  int m0 = 0;
  for (; m0 + BLK <= c.Na; m0 += BLK) {
    float sr = 0.f, si = 0.f;
#pragma unroll
    for (int k = 0; k < BLK; ++k)
      bp_pulse<NATIVE_SINCOS>(rc, c, m0 + k, xa, rf, fb, ib8, k_bin, k_turn, t_max, line_bytes, sr, si);
    acc_r += double(sr);
    acc_i += double(si);
  }
  {
    float sr = 0.f, si = 0.f;
    for (int m = m0; m < c.Na; ++m)
      bp_pulse<NATIVE_SINCOS>(rc, c, m, xa, rf, fb, ib8, k_bin, k_turn, t_max, line_bytes, sr, si);
    acc_r += double(sr);
    acc_i += double(si);
  }
  if (i < c.nx && j < c.ny) {
    const double turns0 = r * c.two_over_lam;
    float sn, cs;
    sincospif(float(2.0 * (turns0 - rint(turns0))), &sn, &cs);
    const float ar = float(acc_r), ai = float(acc_i);
    img[int64_t(i) * c.ny + j] = make_float2(ar * cs - ai * sn, ar * sn + ai * cs);
  }
}

hipError_t launch_backproject(const float2* rc, float2* img, const BpConst& c, int native_sincos,
                              hipStream_t s) {
  const int64_t gx = (int64_t(c.ny) + 63) / 64, gy = (int64_t(c.nx) + 3) / 4;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidValue;
  const dim3 grid{unsigned(gx), unsigned(gy), 1u};
  if (native_sincos)
    hipLaunchKernelGGL(k_backproject<true>, grid, dim3(256), 0, s, rc, img, c);
  else
    hipLaunchKernelGGL(k_backproject<false>, grid, dim3(256), 0, s, rc, img, c);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Doppler-digit row order -> natural order (stage test hook only)
__global__ void __launch_bounds__(256)
    k_row_unpermute(const float2* __restrict__ in, float2* __restrict__ out, int A, int B,
                    int64_t cols) {
  const int k = blockIdx.x;
  const int64_t src = int64_t(k % A) * B + k / A;
  for (int64_t i = threadIdx.x; i < cols; i += 256) out[int64_t(k) * cols + i] = in[src * cols + i];
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
hipError_t occupancy(int* rc, int* fft, int* azc) {
  hipError_t e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress<N>, LineCfg<N>::WG, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(fft, k_line_fft<N, -1>, LineCfg<N>::WG, 0);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(azc, k_rcmc_mf<N, kAuxCached>, RowStage<N>::WG, 0);
}

#ifndef RD_RC_PREFETCH
#define RD_RC_PREFETCH true
#endif
#ifndef RD_RC_4096
#define RD_RC_4096 1
#endif
template <int N>
hipError_t launch_rc_pf(const float2* in, float2* out, const float2* H, const float2* tw,
                        const float2* tab, int64_t lines, int grid, int cached, int n_line,
                        int skip, hipStream_t s) {
  constexpr bool PF = RD_RC_PREFETCH && LineCfg<N>::PF;
  const dim3 g(grid), b(LineCfg<N>::WG);
  if (n_line != N) {
    if (n_line <= 0 || skip < 0 || skip >= n_line || n_line + skip > N) return hipErrorInvalidValue;
    if (cached)
      hipLaunchKernelGGL((k_range_compress_pf<N, PF, kAuxCached, true>), g, b, 0, s, in, out, H, tw, lines,
                         n_line, skip);
    else
      hipLaunchKernelGGL((k_range_compress_pf<N, PF, kAuxStream, true>), g, b, 0, s, in, out, H, tw, lines,
                         n_line, skip);
    return hipGetLastError();
  }
  if constexpr (N == 4096 && RD_RC_4096) {
    if (cached)
      hipLaunchKernelGGL(k_range_compress_4096<kAuxCached>, dim3(grid), dim3(256), 0, s, in, out, tab, lines);
    else
      hipLaunchKernelGGL(k_range_compress_4096<kAuxStream>, dim3(grid), dim3(256), 0, s, in, out, tab, lines);
    return hipGetLastError();
  }
  if constexpr (N == 6000 && RD_RC_6000) {
    if (cached)
      hipLaunchKernelGGL(k_range_compress_6000<kAuxCached>, dim3(grid), dim3(640), 0, s, in, out, tab, lines);
    else
      hipLaunchKernelGGL(k_range_compress_6000<kAuxStream>, dim3(grid), dim3(640), 0, s, in, out, tab, lines);
    return hipGetLastError();
  }
  if constexpr (N == 16384 && RD_RC_16384) {
    if (cached)
      hipLaunchKernelGGL(k_range_compress_16384<kAuxCached>, dim3(grid), dim3(1024), 0, s, in, out, tab, lines);
    else
      hipLaunchKernelGGL(k_range_compress_16384<kAuxStream>, dim3(grid), dim3(1024), 0, s, in, out, tab, lines);
    return hipGetLastError();
  }
  if (cached)
    hipLaunchKernelGGL((k_range_compress_pf<N, PF, kAuxCached>), g, b, 0, s, in, out, H, tw, lines, N, 0);
  else
    hipLaunchKernelGGL((k_range_compress_pf<N, PF, kAuxStream>), g, b, 0, s, in, out, H, tw, lines, N, 0);
  return hipGetLastError();
}

// binary16 storage (4 bytes a sample in and out), float32 arithmetic: the same kernels with
// 32-bit line I/O; streaming stores
template <int N, int SAUX>
void launch_rc_f16_aux(const void* in, void* out, const float2* H, const float2* tw, const float2* tab,
                       int64_t lines, int grid, int n_line, int skip, hipStream_t s) {
  constexpr bool PF = RD_RC_PREFETCH && LineCfg<N>::PF;
  if (n_line != N)
    hipLaunchKernelGGL((k_range_compress_pf<N, PF, SAUX, true, true>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in,
                       out, H, tw, lines, n_line, skip);
  else if constexpr (N == 4096 && RD_RC_4096)
    hipLaunchKernelGGL((k_range_compress_4096<SAUX, true>), dim3(grid), dim3(256), 0, s, in, out, tab, lines);
  else if constexpr (N == 6000 && RD_RC_6000)
    hipLaunchKernelGGL((k_range_compress_6000<SAUX, true>), dim3(grid), dim3(640), 0, s, in, out, tab, lines);
  else if constexpr (N == 16384 && RD_RC_16384 && RD_RC_16384_HALF)
    hipLaunchKernelGGL((k_range_compress_16384<SAUX, true>), dim3(grid), dim3(1024), 0, s, in, out, tab, lines);
  else
    hipLaunchKernelGGL((k_range_compress_pf<N, PF, SAUX, false, true>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in,
                       out, H, tw, lines, N, 0);
}

template <int N>
hipError_t launch_rc_f16(const void* in, void* out, const float2* H, const float2* tw, const float2* tab,
                         int64_t lines, int grid, int cached, int n_line, int skip, hipStream_t s) {
  if (n_line != N && (n_line <= 0 || skip < 0 || skip >= n_line || n_line + skip > N)) return hipErrorInvalidValue;
  if (cached)
    launch_rc_f16_aux<N, kAuxCached>(in, out, H, tw, tab, lines, grid, n_line, skip, s);
  else
    launch_rc_f16_aux<N, kAuxStream>(in, out, H, tw, tab, lines, grid, n_line, skip, s);
  return hipGetLastError();
}

template <int N>
hipError_t occupancy_f16(int* rc, int pad) {
  if (pad)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        rc, k_range_compress_pf<N, RD_RC_PREFETCH && LineCfg<N>::PF, kAuxStream, true, true>, LineCfg<N>::WG, 0);
  if constexpr (N == 4096 && RD_RC_4096)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_4096<kAuxStream, true>, 256, 0);
  if constexpr (N == 6000 && RD_RC_6000)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_6000<kAuxStream, true>, 640, 0);
  if constexpr (N == 16384 && RD_RC_16384 && RD_RC_16384_HALF)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_16384<kAuxStream, true>, 1024, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      rc, k_range_compress_pf<N, RD_RC_PREFETCH && LineCfg<N>::PF, kAuxStream, false, true>, LineCfg<N>::WG, 0);
}

template <int N>
hipError_t occupancy_pf(int* rc, int pad) {
  if (pad)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        rc, k_range_compress_pf<N, RD_RC_PREFETCH && LineCfg<N>::PF, kAuxStream, true>, LineCfg<N>::WG, 0);
  if constexpr (N == 4096 && RD_RC_4096)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_4096<kAuxStream>, 256, 0);
  if constexpr (N == 16384 && RD_RC_16384)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_16384<kAuxStream>, 1024, 0);
  if constexpr (N == 6000 && RD_RC_6000)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_6000<kAuxStream>, 640, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(rc, k_range_compress_pf<N, RD_RC_PREFETCH && LineCfg<N>::PF, kAuxStream>,
                                                      LineCfg<N>::WG, 0);
}

template <int N>
hipError_t launch_rcmc_mf(const void* in, void* out, const AzRowConst& c, int64_t rows, int grid,
                          int cached, int half, hipStream_t s) {
  const int64_t wgs = (rows + RowStage<N>::LPW - 1) / RowStage<N>::LPW;  // one row per thread group
  if (grid <= 0 || grid > wgs) grid = int(wgs);
  const dim3 g(grid), b(RowStage<N>::WG);
  if (half && cached)
    hipLaunchKernelGGL((k_rcmc_mf<N, kAuxCached, true>), g, b, 0, s, in, out, c, rows, N);
  else if (half)
    hipLaunchKernelGGL((k_rcmc_mf<N, kAuxStream, true>), g, b, 0, s, in, out, c, rows, N);
  else if (cached)
    hipLaunchKernelGGL((k_rcmc_mf<N, kAuxCached>), g, b, 0, s, in, out, c, rows, N);
  else
    hipLaunchKernelGGL((k_rcmc_mf<N, kAuxStream>), g, b, 0, s, in, out, c, rows, N);
  return hipGetLastError();
}

template <int N>
hipError_t launch_omega_k_rows(const void* in, void* out, const float2* H, const float2* tw,
                               const OkConst& c, const RcmcPoly& w, int64_t rows, int grid,
                               int cached, int half, hipStream_t s) {
  if (c.halo < 0 || c.halo > OkRow<N>::CAP || c.ref < 0 || c.ref >= N) return hipErrorInvalidValue;
  const int64_t wgs = (rows + LineCfg<N>::LPW - 1) / LineCfg<N>::LPW;
  if (grid <= 0 || grid > wgs) grid = int(wgs);
  if (half && cached)
    hipLaunchKernelGGL((k_omega_k_row<N, kAuxCached, true>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H,
                       tw, c, w, rows);
  else if (half)
    hipLaunchKernelGGL((k_omega_k_row<N, kAuxStream, true>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H,
                       tw, c, w, rows);
  else if (cached)
    hipLaunchKernelGGL((k_omega_k_row<N, kAuxCached>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H, tw,
                       c, w, rows);
  else
    hipLaunchKernelGGL((k_omega_k_row<N, kAuxStream>), dim3(grid), dim3(LineCfg<N>::WG), 0, s, in, out, H, tw,
                       c, w, rows);
  return hipGetLastError();
}

template <int N>
hipError_t occupancy_wk(int* wgs) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs, k_omega_k_row<N, kAuxCached>, LineCfg<N>::WG, 0);
}

// RCMC + azimuth filter over rows of n samples, any n >= 1 (run-time length; shifts up to
// RowStage<0>::MARGIN - 5)
hipError_t launch_rcmc_mf_any(const void* in, void* out, const AzRowConst& c, int64_t rows, int n,
                              int cached, int half, hipStream_t s) {
  using RS = RowStage<0>;
  if (n <= 0 || c.halo < 0 || c.halo > RS::MARGIN) return hipErrorInvalidValue;
  const int64_t wgs = (rows + RS::LPW - 1) / RS::LPW;  // one row per thread group
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  const int grid = int(wgs);
  if (half && cached)
    hipLaunchKernelGGL((k_rcmc_mf<0, kAuxCached, true>), dim3(grid), dim3(RS::WG), 0, s, in, out, c, rows, n);
  else if (half)
    hipLaunchKernelGGL((k_rcmc_mf<0, kAuxStream, true>), dim3(grid), dim3(RS::WG), 0, s, in, out, c, rows, n);
  else if (cached)
    hipLaunchKernelGGL((k_rcmc_mf<0, kAuxCached>), dim3(grid), dim3(RS::WG), 0, s, in, out, c, rows, n);
  else
    hipLaunchKernelGGL((k_rcmc_mf<0, kAuxStream>), dim3(grid), dim3(RS::WG), 0, s, in, out, c, rows, n);
  return hipGetLastError();
}
int rcmc_any_margin() { return RowStage<0>::MARGIN; }

template <int N>
int rc_tab_len() {
  if constexpr (N == 4096 && RD_RC_4096) return kRc4096Tab;
  if constexpr (N == 16384 && RD_RC_16384) return kRc16kTab;
  if constexpr (N == 6000 && RD_RC_6000) return kRc6kTab;
  return 0;
}
template <int N>
void rc_tab_fill(const float2* H, const float2* roots, float2* out) {
  if constexpr (N == 4096 && RD_RC_4096) rc4096_tab_fill(H, roots, out);
  if constexpr (N == 16384 && RD_RC_16384) rc16k_tab_fill(H, roots, out);
  if constexpr (N == 6000 && RD_RC_6000) rc6k_tab_fill(H, roots, out);
}

template <int N>
constexpr LineOps make_ops() {
  constexpr bool sym = std::is_same<typename LineCfg<N>::Fwd, typename LineCfg<N>::Inv>::value;
  if constexpr (sym) {
    return LineOps{N, LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>, &launch_fft<N>,
                   &occupancy<N>, &launch_rc_pf<N>, &occupancy_pf<N>, &rc_tab_len<N>,
                   &rc_tab_fill<N>, &launch_rcmc_mf<N>, RowStage<N>::MARGIN,
                   &launch_omega_k_rows<N>, &occupancy_wk<N>, OkRow<N>::CAP, &launch_rc_f16<N>,
                   &occupancy_f16<N>};
  } else {
    return LineOps{N, LineCfg<N>::WG, LineCfg<N>::LPW, &launch_rc<N>, &launch_fft<N>,
                   &occupancy<N>, nullptr, nullptr, &rc_tab_len<N>, &rc_tab_fill<N>,
                   &launch_rcmc_mf<N>, RowStage<N>::MARGIN, nullptr, nullptr, 0, nullptr, nullptr};
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

template <int L, int DIR, int AUX>
void launch_col3(const void* in, void* out, const float2* tw_L, const ColGeom& cg, dim3 grid,
                 uint32_t bytes, int half, hipStream_t s) {
  if (half)
    hipLaunchKernelGGL((k_col_fft<L, DIR, AUX, true>), grid, dim3(ColCfg<L>::WG), 0, s, in, out, tw_L, cg, bytes);
  else
    hipLaunchKernelGGL((k_col_fft<L, DIR, AUX>), grid, dim3(ColCfg<L>::WG), 0, s, in, out, tw_L, cg, bytes);
}

template <int L>
hipError_t launch_col(const void* in, void* out, const float2* tw_L, const ColStep& st,
                      int64_t cols, int na, int cached, hipStream_t s) {
  ColGeom cg;
  cg.cols = cols;
  cg.base_mul = st.base_mul;
  cg.stride = st.stride;
  cg.chunks = int((cols + 63) / 64);
  cg.na = na;
  cg.twiddle = st.twiddle;
  cg.scale = st.scale;
  const uint64_t bytes = uint64_t(na) * uint64_t(cols) * (st.half ? 4u : 8u);
  if (bytes > 0xFFFFFFF0ull) return hipErrorInvalidValue;
  const dim3 grid(unsigned(int64_t(st.sets) * cg.chunks));
  if (st.dir < 0) {
    if (cached) launch_col3<L, -1, kAuxCached>(in, out, tw_L, cg, grid, uint32_t(bytes), st.half, s);
    else launch_col3<L, -1, kAuxStream>(in, out, tw_L, cg, grid, uint32_t(bytes), st.half, s);
  } else {
    if (cached) launch_col3<L, +1, kAuxCached>(in, out, tw_L, cg, grid, uint32_t(bytes), st.half, s);
    else launch_col3<L, +1, kAuxStream>(in, out, tw_L, cg, grid, uint32_t(bytes), st.half, s);
  }
  return hipGetLastError();
}

hipError_t launch_col_fft(const void* in, void* out, const float2* tw_L, const ColStep& st,
                          int64_t cols, int na, int cached, hipStream_t s) {
  switch (st.L) {
    case 16: return launch_col<16>(in, out, tw_L, st, cols, na, cached, s);
    case 32: return launch_col<32>(in, out, tw_L, st, cols, na, cached, s);
    case 64: return launch_col<64>(in, out, tw_L, st, cols, na, cached, s);
    case 128: return launch_col<128>(in, out, tw_L, st, cols, na, cached, s);
    case 25: return launch_col<25>(in, out, tw_L, st, cols, na, cached, s);
    default: return hipErrorInvalidValue;
  }
}

// Bluestein (chirp-z) transforms along the azimuth axis (nxmr.cn/news/101525 §5.1: any length):
// the two elementwise row passes.  out[r][c] = scale in[r][c] exp(sign j pi r^2 / na) for
// r < rows_in and 0 for rows_in <= r < rows_out (r^2 reduced modulo 2 na in integers, so the
// argument of sincospi is exact and below 2); io[r][c] *= f[r].  HIN / HOUT: binary16 storage
// of the input / output (the image side of a binary16 chain; the workspace stays float32).
template <bool HIN, bool HOUT>
__global__ void __launch_bounds__(256)
    k_chirp_rows(const void* __restrict__ in, void* __restrict__ out, int64_t cols, int rows_in, int na,
                 int sign, float scale) {
  const int r = blockIdx.y;
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c >= cols) return;
  const int64_t e = int64_t(r) * cols + c;
  float2 v = make_float2(0.f, 0.f);
  if (r < rows_in) {
    const int64_t q = (int64_t(r) * r) % (2 * int64_t(na));
    float sn, cs;
    sincospif(float(q) / float(na), &sn, &cs);
    const float2 x = HIN ? h2_to_f2(static_cast<const unsigned int*>(in)[e]) : static_cast<const float2*>(in)[e];
    v = cmul(x, make_float2(cs * scale, (sign > 0 ? sn : -sn) * scale));
  }
  if constexpr (HOUT)
    static_cast<unsigned int*>(out)[e] = f2_to_h2(v);
  else
    static_cast<float2*>(out)[e] = v;
}

__global__ void __launch_bounds__(256)
    k_scale_rows(float2* __restrict__ io, const float2* __restrict__ f, int64_t cols) {
  const int r = blockIdx.y;
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (c < cols) io[int64_t(r) * cols + c] = cmul(io[int64_t(r) * cols + c], f[r]);
}

hipError_t launch_chirp_rows(const void* in, void* out, int64_t cols, int rows_in, int rows_out, int na,
                             int sign, int hin, int hout, float scale, hipStream_t s) {
  const int64_t gx = (cols + 255) / 256;
  if (gx > 0x7fffffff || rows_out <= 0 || rows_out > 65535 || rows_in > rows_out || na <= 0 || (hin && hout))
    return hipErrorInvalidValue;
  const dim3 g{static_cast<uint32_t>(gx), static_cast<uint32_t>(rows_out)}, b{256};
  if (hin)
    hipLaunchKernelGGL((k_chirp_rows<true, false>), g, b, 0, s, in, out, cols, rows_in, na, sign, scale);
  else if (hout)
    hipLaunchKernelGGL((k_chirp_rows<false, true>), g, b, 0, s, in, out, cols, rows_in, na, sign, scale);
  else
    hipLaunchKernelGGL((k_chirp_rows<false, false>), g, b, 0, s, in, out, cols, rows_in, na, sign, scale);
  return hipGetLastError();
}

hipError_t launch_scale_rows(float2* io, const float2* f, int64_t cols, int rows, hipStream_t s) {
  const int64_t gx = (cols + 255) / 256;
  if (gx > 0x7fffffff || rows <= 0 || rows > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_scale_rows, dim3(unsigned(gx), unsigned(rows)), dim3(256), 0, s, io, f, cols);
  return hipGetLastError();
}

hipError_t launch_row_unpermute(const float2* in, float2* out, int A, int B, int64_t cols,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_row_unpermute, dim3(unsigned(A * B)), dim3(256), 0, s, in, out, A, B, cols);
  return hipGetLastError();
}

}  // namespace rdf
