// LDS-resident line FFT for gfx950 (wave64, 160 KB LDS per CU).
//
// A line of N complex float32 points is transformed by a group of T threads.  Each pass is a
// radix-R Stockham decimation-in-time step (the auto-sorting form, so no bit reversal):
//   butterfly j (0 <= j < N/R) takes x[j + r N/R] (r < R), multiplies input r by
//   W_{Ns R}^{(j mod Ns) r}, runs a length-R DFT and writes element r to
//   (j / Ns) Ns R + (j mod Ns) + r Ns,  where Ns is the product of the earlier radices.
// Between passes the line goes through one bank-padded LDS buffer; the first pass reads its
// inputs straight from global memory and the last pass leaves its outputs in registers in
// natural order (element j + r N/R_last), so a pointwise multiply and a second transform with
// the radix list reversed can follow without another exchange.
//
// The inverse transform uses the same passes with the conjugate kernel e^{+j...}; in exact and
// in round-to-nearest arithmetic this equals conj(FFT(conj(x))), the identity that
// cf-1.com/news/2323550 §3.2 uses to share the forward code path.  1/N is folded into the
// caller's filter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rdf {

// ---------------------------------------------------------------------------- complex helpers
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
// a * (S j) for S = +1 / -1
template <int S>
__device__ __forceinline__ float2 mul_j(float2 a) {
  return S > 0 ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
}

// The same global pointer, offset by an amount the compiler cannot see (always zero): table
// loads behind it stay where they are written instead of being hoisted out of a line loop
// into registers (hoisting H and every twiddle costs ~100 VGPRs and halves the occupancy).
// Offsetting, rather than laundering the pointer itself, keeps its global address space.
template <class T>
__device__ __forceinline__ const T* opaque(const T* p) {
  int zero = 0;
  asm volatile("" : "+s"(zero));
  return p + zero;
}

// Debug builds (RD_DEBUG) fill a kernel's LDS array with quiet NaNs before first use, so a read of
// an element that no thread has written shows up as NaN in the output; other builds do nothing.
template <size_t BYTES>
__device__ __forceinline__ void debug_poison_lds(void* lds) {
#ifdef RD_DEBUG
  const unsigned n = blockDim.x * blockDim.y * blockDim.z;
  const unsigned t = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
  unsigned* w = static_cast<unsigned*>(lds);
  for (unsigned i = t; i < BYTES / 4; i += n) w[i] = 0x7fc00000u;
  __syncthreads();
#else
  (void)lds;
#endif
}
#define RD_POISON_LDS(a) debug_poison_lds<sizeof(a)>(a)

// Marks registers as read here.  Placed after a line's stores, it makes the compiler wait for
// prefetched registers at that point, where the outstanding stores are younger than the
// prefetch and need not complete; otherwise the wait lands at the loop head, whose merged
// state (loop entry: the prefetch is the youngest access) forces every store to complete first.
template <int K>
__device__ __forceinline__ void touch(const float2* v) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" ::"v"(v[i].x), "v"(v[i].y));
}
template <int K>
__device__ __forceinline__ void touch(const unsigned int* v) {
#pragma unroll
  for (int i = 0; i < K; ++i) asm volatile("" ::"v"(v[i]));
}

// ---------------------------------------------------------------------------- compile-time roots
// cos / sin of 2 pi p / q in double precision, evaluated by the compiler: the angle is reduced
// exactly (integer arithmetic) to [0, pi/4] and expanded in Taylor series there.
constexpr double kPi = 3.141592653589793238462643383279502884;

constexpr double ct_sin_small(double x) {
  double term = x, sum = x;
  for (int n = 1; n < 16; ++n) {
    term *= -x * x / double((2 * n) * (2 * n + 1));
    sum += term;
  }
  return sum;
}
constexpr double ct_cos_small(double x) {
  double term = 1.0, sum = 1.0;
  for (int n = 1; n < 16; ++n) {
    term *= -x * x / double((2 * n - 1) * (2 * n));
    sum += term;
  }
  return sum;
}
// (cos, sin) of 2 pi p / q
struct CS {
  double c, s;
};
constexpr CS ct_root(long p, long q) {
  p %= q;
  if (p < 0) p += q;
  const long quad = (4 * p) / q;   // quadrant of the angle
  const long rem = 4 * p - quad * q; // angle within the quadrant = (pi/2) rem / q
  double c0 = 1.0, s0 = 0.0;
  if (rem != 0) {
    if (2 * rem <= q) {              // <= pi/4
      const double x = (kPi / 2.0) * double(rem) / double(q);
      c0 = ct_cos_small(x);
      s0 = ct_sin_small(x);
    } else {                         // use the complement angle
      const double x = (kPi / 2.0) * double(q - rem) / double(q);
      c0 = ct_sin_small(x);
      s0 = ct_cos_small(x);
    }
  }
  switch (quad) {
    case 0: return {c0, s0};
    case 1: return {-s0, c0};
    case 2: return {-c0, -s0};
    default: return {s0, -c0};
  }
}

template <int N>
struct Roots {
  float c[N];
  float s[N];
  constexpr Roots() : c(), s() {
    for (int k = 0; k < N; ++k) {
      const CS v = ct_root(k, N);
      c[k] = float(v.c);
      s[k] = float(v.s);
    }
  }
};
template <int N>
inline constexpr Roots<N> kRoots{};

// x * W_N^e with W_N = e^{DIR j 2 pi / N}; e is a compile-time constant after unrolling, so
// the branches fold and the root is an immediate.
template <int N, int DIR>
__device__ __forceinline__ float2 rot_const(float2 x, int e) {
  e %= N;
  if (e == 0) return x;
  if (4 * e == N) return mul_j<DIR>(x);
  if (2 * e == N) return make_float2(-x.x, -x.y);
  if (4 * e == 3 * N) return mul_j<-DIR>(x);
  const float c = kRoots<N>.c[e];
  const float s = DIR > 0 ? kRoots<N>.s[e] : -kRoots<N>.s[e];
  return cmul(x, make_float2(c, s));
}

// ---------------------------------------------------------------------------- small DFTs
// In-place length-R DFT of v[0..R-1], natural order in and out, kernel e^{DIR j 2 pi kn/R}.
template <int R, int DIR>
struct Dft;

template <int A, int B, int DIR>
__device__ __forceinline__ void dft_ct(float2* v);

template <int DIR>
struct Dft<1, DIR> {
  static __device__ __forceinline__ void run(float2*) {}
};

template <int DIR>
struct Dft<2, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    const float2 a = v[0], b = v[1];
    v[0] = cadd(a, b);
    v[1] = csub(a, b);
  }
};

template <int DIR>
struct Dft<3, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    constexpr float h = 0.866025403784438646763723170752936183f;  // sin(2 pi / 3)
    const float2 t = cadd(v[1], v[2]);
    const float2 d = csub(v[1], v[2]);
    const float2 m = make_float2(v[0].x - 0.5f * t.x, v[0].y - 0.5f * t.y);
    const float2 jd = mul_j<DIR>(cscale(d, h));
    v[0] = cadd(v[0], t);
    v[1] = cadd(m, jd);
    v[2] = csub(m, jd);
  }
};

template <int DIR>
struct Dft<4, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    const float2 t0 = cadd(v[0], v[2]), t1 = csub(v[0], v[2]);
    const float2 t2 = cadd(v[1], v[3]), t3 = mul_j<DIR>(csub(v[1], v[3]));
    v[0] = cadd(t0, t2);
    v[2] = csub(t0, t2);
    v[1] = cadd(t1, t3);
    v[3] = csub(t1, t3);
  }
};

template <int DIR>
struct Dft<5, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    constexpr float c1 = 0.309016994374947424102293417182819059f;   // cos(2 pi / 5)
    constexpr float c2 = -0.809016994374947424102293417182819059f;  // cos(4 pi / 5)
    constexpr float s1 = 0.951056516295153572116439333379382143f;   // sin(2 pi / 5)
    constexpr float s2 = 0.587785252292473129168705954639072769f;   // sin(4 pi / 5)
    const float2 t1 = cadd(v[1], v[4]), d1 = csub(v[1], v[4]);
    const float2 t2 = cadd(v[2], v[3]), d2 = csub(v[2], v[3]);
    const float2 x0 = v[0];
    const float2 a1 = make_float2(x0.x + c1 * t1.x + c2 * t2.x, x0.y + c1 * t1.y + c2 * t2.y);
    const float2 a2 = make_float2(x0.x + c2 * t1.x + c1 * t2.x, x0.y + c2 * t1.y + c1 * t2.y);
    const float2 b1 = mul_j<DIR>(make_float2(s1 * d1.x + s2 * d2.x, s1 * d1.y + s2 * d2.y));
    const float2 b2 = mul_j<DIR>(make_float2(s2 * d1.x - s1 * d2.x, s2 * d1.y - s1 * d2.y));
    v[0] = make_float2(x0.x + t1.x + t2.x, x0.y + t1.y + t2.y);
    v[1] = cadd(a1, b1);
    v[4] = csub(a1, b1);
    v[2] = cadd(a2, b2);
    v[3] = csub(a2, b2);
  }
};

// Composite lengths run as one Cooley-Tukey split R = A * B (dft_ct below); others directly.
template <int R>
struct DftSplit {
  static constexpr int A = 1, B = R;
};
template <> struct DftSplit<6> { static constexpr int A = 2, B = 3; };
template <> struct DftSplit<8> { static constexpr int A = 2, B = 4; };
template <> struct DftSplit<10> { static constexpr int A = 2, B = 5; };
template <> struct DftSplit<15> { static constexpr int A = 3, B = 5; };
template <> struct DftSplit<16> { static constexpr int A = 4, B = 4; };
template <> struct DftSplit<20> { static constexpr int A = 4, B = 5; };
template <> struct DftSplit<25> { static constexpr int A = 5, B = 5; };

constexpr int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }
// A split with coprime factors runs as a prime-factor (Good-Thomas) DFT: no twiddles.
template <int R>
constexpr bool dft_pfa() { return DftSplit<R>::A > 1 && gcd_i(DftSplit<R>::A, DftSplit<R>::B) == 1; }

// The i-th input a length-R DFT consumes: a split DFT starts with the A inputs of its first
// sub-DFT (B n1 + 0, or (B n1) mod R for a prime-factor split), then those of the second, ...
// Loading a butterfly's inputs in this order lets its first sub-DFT start as soon as the first A
// loads have returned (memory counters complete in order).
template <int R>
constexpr int dft_input_order(int i) {
  constexpr int A = DftSplit<R>::A, B = DftSplit<R>::B;
  if constexpr (A == 1) return i;
  else if constexpr (dft_pfa<R>()) return (B * (i % A) + A * (i / A)) % R;
  else return B * (i % A) + i / A;
}

template <int A, int B, int DIR>
__device__ __forceinline__ void dft_pfa_run(float2* v);

template <int R, int DIR>
struct Dft {
  static_assert(DftSplit<R>::A > 1, "no DFT of this length");
  static __device__ __forceinline__ void run(float2* v) {
    if constexpr (dft_pfa<R>())
      dft_pfa_run<DftSplit<R>::A, DftSplit<R>::B, DIR>(v);
    else
      dft_ct<DftSplit<R>::A, DftSplit<R>::B, DIR>(v);
  }
};

// Length A*B DFT in registers with gcd(A, B) = 1 (Good-Thomas prime-factor algorithm): input
// n = (B n1 + A n2) mod N, output k the residue with k = k1 (mod A) and k = k2 (mod B).  Then
// W_N^{n k} = W_A^{n1 k1} W_B^{n2 k2}, so the DFT is DFT_A over n1 followed by DFT_B over n2 with
// no twiddle multiplies between them; both index maps are compile-time register renamings.
template <int A, int B>
struct PfaMap {
  int in[A * B];   // in[n1 + A n2] = (B n1 + A n2) mod N
  int out[A * B];  // out[k1 + A k2] = the k in [0, N) with k = k1 (mod A), k = k2 (mod B)
  constexpr PfaMap() : in(), out() {
    for (int n2 = 0; n2 < B; ++n2)
      for (int n1 = 0; n1 < A; ++n1) in[n1 + A * n2] = (B * n1 + A * n2) % (A * B);
    for (int k = 0; k < A * B; ++k) out[(k % A) + A * (k % B)] = k;
  }
};
template <int A, int B>
inline constexpr PfaMap<A, B> kPfaMap{};

template <int A, int B, int DIR>
__device__ __forceinline__ void dft_pfa_run(float2* v) {
  constexpr int N = A * B;
  float2 t[N];
#pragma unroll
  for (int n2 = 0; n2 < B; ++n2) {
    float2 u[A];
#pragma unroll
    for (int n1 = 0; n1 < A; ++n1) u[n1] = v[kPfaMap<A, B>.in[n1 + A * n2]];
    Dft<A, DIR>::run(u);
#pragma unroll
    for (int k1 = 0; k1 < A; ++k1) t[k1 * B + n2] = u[k1];
  }
#pragma unroll
  for (int k1 = 0; k1 < A; ++k1) {
    float2 u[B];
#pragma unroll
    for (int n2 = 0; n2 < B; ++n2) u[n2] = t[k1 * B + n2];
    Dft<B, DIR>::run(u);
#pragma unroll
    for (int k2 = 0; k2 < B; ++k2) v[kPfaMap<A, B>.out[k1 + A * k2]] = u[k2];
  }
}

// Length-8 and length-16 DFTs with the internal rotations folded into fused multiply-adds.
// Each rotation by a constant root is written as scale * (unit-diagonal factor): the roots at
// odd multiples of pi/4 are h (+-1 +- j) with h = sqrt(1/2), and those at odd multiples of pi/8
// are c (1 +- j tau) times a power of j, with c = cos(pi/8), tau = tan(pi/8) (|tau| < 1, so
// the factored form loses no accuracy).  The factor costs two additions (or two FMAs), and the
// common scale of the two inputs that meet in the following radix-2 step multiplies their
// combination inside that step's FMAs, so no separate multiplication remains: 144 instead of
// 160 VALU operations for a length-16 DFT, 52 instead of 56 for length 8.  Same split as
// dft_ct (input n = B n1 + n2, output k = k1 + A k2), so dft_input_order is unchanged.
constexpr float kSqrtHalf = 0.707106781186547524400844362104849039f;  // cos(pi/4)
constexpr float kCosPi8 = 0.923879532511286756128183189396788933f;    // cos(pi/8)
constexpr float kTanPi8 = 0.414213562373095048801688724209698079f;    // tan(pi/8)

// Keeps the scheduler from interleaving the output groups of one DFT: each group's
// temporaries die before the next group starts (interleaved, the length-16 DFT needs ~10 more
// registers, which costs a wave per SIMD or spills in the range-compression kernel).
__device__ __forceinline__ void group_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ float2 cfma(float s, float2 q, float2 a) {
  return make_float2(fmaf(s, q.x, a.x), fmaf(s, q.y, a.y));
}
// (1 + D j) u and (-1 + D j) u
template <int D>
__device__ __forceinline__ float2 mul_1pj(float2 u) {
  return D > 0 ? make_float2(u.x - u.y, u.y + u.x) : make_float2(u.x + u.y, u.y - u.x);
}
template <int D>
__device__ __forceinline__ float2 mul_m1pj(float2 u) {
  return D > 0 ? make_float2(-u.x - u.y, u.x - u.y) : make_float2(u.y - u.x, -u.y - u.x);
}
// (1 + S j tau) u, S = +1 / -1
template <int S>
__device__ __forceinline__ float2 mul_1ptau(float2 u) {
  return make_float2(fmaf(-float(S) * kTanPi8, u.y, u.x), fmaf(float(S) * kTanPi8, u.x, u.y));
}

// k1 = odd group of a split-radix step: inputs already multiplied by W^{n2 k1} except for the
// scales; returns the four outputs k2 = 0..3 of the length-4 DFT over n2 in o[0..3].
template <int DIR>
__device__ __forceinline__ void dft8_odd(const float2* u, float2* o) {
  // W8^0, W8^1 = h (1 + D j), W8^2 = D j, W8^3 = h (-1 + D j)
  const float2 p1 = mul_1pj<DIR>(u[1]), p3 = mul_m1pj<DIR>(u[3]);
  const float2 t2 = mul_j<DIR>(u[2]);
  const float2 a0 = cadd(u[0], t2), a1 = csub(u[0], t2);
  const float2 q2 = cadd(p1, p3), q3 = mul_j<DIR>(csub(p1, p3));
  o[0] = cfma(kSqrtHalf, q2, a0);
  o[2] = cfma(-kSqrtHalf, q2, a0);
  o[1] = cfma(kSqrtHalf, q3, a1);
  o[3] = cfma(-kSqrtHalf, q3, a1);
}

template <int DIR>
struct Dft<8, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    // n = 4 n1 + n2, k = k1 + 2 k2
    float2 e[4], d[4];
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {
      e[n2] = cadd(v[n2], v[4 + n2]);
      d[n2] = csub(v[n2], v[4 + n2]);
    }
    Dft<4, DIR>::run(e);
    float2 o[4];
    dft8_odd<DIR>(d, o);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      v[2 * k2] = e[k2];
      v[1 + 2 * k2] = o[k2];
    }
  }
};

template <int DIR>
struct Dft<16, DIR> {
  static __device__ __forceinline__ void run(float2* v) {
    // n = 4 n1 + n2, k = k1 + 4 k2; U[k1][n2] = DFT4 over n1 of v[4 n1 + n2]
    float2 U[4][4];
#pragma unroll
    for (int n2 = 0; n2 < 4; ++n2) {
      float2 u[4] = {v[n2], v[4 + n2], v[8 + n2], v[12 + n2]};
      Dft<4, DIR>::run(u);
#pragma unroll
      for (int k1 = 0; k1 < 4; ++k1) U[k1][n2] = u[k1];
    }
    // k1 = 0: no rotations
    Dft<4, DIR>::run(U[0]);
    group_fence();
    // k1 = 2: W16^{0,2,4,6} = 1, h(1 + D j), D j, h(-1 + D j)
    float2 o2[4];
    dft8_odd<DIR>(U[2], o2);
    group_fence();
    // k1 = 1: W16^{0,1,2,3} = 1, c (1 + D j tau), h (1 + D j), c (D j)(1 - D j tau)
    float2 o1[4], o3[4];
    {
      const float2* u = U[1];
      const float2 p2 = mul_1pj<DIR>(u[2]);
      const float2 y1 = mul_1ptau<DIR>(u[1]), y3 = mul_1ptau<-DIR>(u[3]);
      const float2 a0 = cfma(kSqrtHalf, p2, u[0]), a1 = cfma(-kSqrtHalf, p2, u[0]);
      const float2 s2 = cadd(y1, mul_j<DIR>(y3));
      const float2 d3 = mul_j<DIR>(csub(y1, mul_j<DIR>(y3)));
      o1[0] = cfma(kCosPi8, s2, a0);
      o1[2] = cfma(-kCosPi8, s2, a0);
      o1[1] = cfma(kCosPi8, d3, a1);
      o1[3] = cfma(-kCosPi8, d3, a1);
    }
    group_fence();
    // k1 = 3: W16^{0,3,6,9} = 1, c (D j)(1 - D j tau), h (-1 + D j), -c (1 + D j tau)
    {
      const float2* u = U[3];
      const float2 p2 = mul_m1pj<DIR>(u[2]);
      const float2 y1 = mul_1ptau<-DIR>(u[1]), y3 = mul_1ptau<DIR>(u[3]);
      const float2 a0 = cfma(kSqrtHalf, p2, u[0]), a1 = cfma(-kSqrtHalf, p2, u[0]);
      const float2 jy1 = mul_j<DIR>(y1);
      const float2 s2 = csub(jy1, y3);
      const float2 d3 = mul_j<DIR>(cadd(jy1, y3));
      o3[0] = cfma(kCosPi8, s2, a0);
      o3[2] = cfma(-kCosPi8, s2, a0);
      o3[1] = cfma(kCosPi8, d3, a1);
      o3[3] = cfma(-kCosPi8, d3, a1);
    }
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) {
      v[0 + 4 * k2] = U[0][k2];
      v[1 + 4 * k2] = o1[k2];
      v[2 + 4 * k2] = o2[k2];
      v[3 + 4 * k2] = o3[k2];
    }
  }
};

// ---------------------------------------------------------------------------- pass machinery
template <int... Rs>
struct IntList {};

template <class L>
struct ListInfo;
template <int R>
struct ListInfo<IntList<R>> {
  static constexpr int first = R, last = R, product = R, count = 1;
};
template <int R, int R2, int... Rs>
struct ListInfo<IntList<R, R2, Rs...>> {
  static constexpr int first = R;
  static constexpr int last = ListInfo<IntList<R2, Rs...>>::last;
  static constexpr int product = R * ListInfo<IntList<R2, Rs...>>::product;
  static constexpr int count = 1 + ListInfo<IntList<R2, Rs...>>::count;
};

// Exchange layout in LDS.  Measured on gfx950 (SQ_LDS_BANK_CONFLICT on single-pattern
// kernels): 8-byte LDS reads are served 32 lanes at a time over 64 four-byte banks, 8-byte writes
// 16 lanes at a time over 32 banks.  The exchange after a pass whose earlier radices multiply to
// NS writes element (j/NS) NS R + j%NS + r NS and the next pass reads j + r N/R2; both are
// stored at i + P floor(i/Q) (P pad elements after every Q), with (P, Q) chosen per line length
// and exchange.  The default, one pad after every 16, keeps the stride-R writes of the first
// exchange on distinct banks (its contiguous reads then meet one two-way conflict per half-wave,
// which no block padding avoids); an exchange whose writes are already contiguous runs of 16
// needs no padding at all (P = 0).  The choices were found by enumerating (P, Q) against that
// bank model.
template <int N, int NS>
struct XPad {
  static constexpr int P = 1, Q = 16;
};
template <> struct XPad<512, 8> { static constexpr int P = 0, Q = 512; };
template <> struct XPad<1024, 16> { static constexpr int P = 0, Q = 1024; };
template <> struct XPad<2048, 16> { static constexpr int P = 0, Q = 2048; };
template <> struct XPad<4096, 16> { static constexpr int P = 0, Q = 4096; };
template <> struct XPad<8192, 8> { static constexpr int P = 0, Q = 8192; };
template <> struct XPad<8192, 32> { static constexpr int P = 0, Q = 8192; };
template <> struct XPad<8192, 256> { static constexpr int P = 0, Q = 8192; };
// 6000 = 10 * 6 * 10 * 10: periods that divide the exchange strides, so every access stays a
// per-thread base plus a constant (model: 670 instead of 2707 conflict cycles a line and direction;
// measured 45.4 M cycles per 8192-line launch with one pad per 16, as the model predicts)
template <> struct XPad<6000, 1> { static constexpr int P = 1, Q = 200; };
template <> struct XPad<6000, 10> { static constexpr int P = 2, Q = 300; };
template <> struct XPad<6000, 60> { static constexpr int P = 4, Q = 600; };
// 600 = 10 * 6 * 10 on one wave (the sub-line transform of the four-step 6000 kernel): model 30
// and 36 conflict cycles for the two exchanges, against 168 and 46 with one pad per 16
template <> struct XPad<600, 1> { static constexpr int P = 1, Q = 100; };
template <> struct XPad<600, 10> { static constexpr int P = 1, Q = 60; };

template <int N, int NS>
__device__ __forceinline__ int xpad(int i) {
  using X = XPad<N, NS>;
  return i + X::P * (i / X::Q);
}
// LDS elements of a line buffer: the unpadded length plus at most one pad per 16 elements
// (every XPad choice must stay within this; checked where it is used).
constexpr int lds_len(int n) { return n + n / 16 + 1; }
// xpad(base + r * STRIDE) written so that, for the strides that occur, it is one per-thread
// base plus a compile-time offset (an LDS instruction's immediate), not a fresh shift-and-add
// per element.  Exact when STRIDE % Q == 0, or when base % Q + r * STRIDE < Q (FITS).
template <int N, int NS, int STRIDE, bool FITS>
__device__ __forceinline__ int xpad_step(int padded_base, int base, int r) {
  using X = XPad<N, NS>;
  static_assert(X::P * ((N - 1) / X::Q) <= N / 16, "exchange padding exceeds the line buffer");
  if constexpr (X::P == 0) {
    return padded_base + r * STRIDE;
  } else if constexpr (STRIDE % X::Q == 0) {
    return padded_base + r * (STRIDE + STRIDE / X::Q * X::P);
  } else if constexpr (FITS) {
    return padded_base + r * STRIDE;
  } else {
    return xpad<N, NS>(base + r * STRIDE);
  }
}

// Registers a thread needs for a radix-R pass: ceil(N/R / T) butterflies of R points.
constexpr int pass_regs(int N, int T, int R) { return ((N / R + T - 1) / T) * R; }
template <int N, int T, class L>
struct MaxRegs;
template <int N, int T, int R>
struct MaxRegs<N, T, IntList<R>> {
  static constexpr int value = pass_regs(N, T, R);
};
template <int N, int T, int R, int R2, int... Rs>
struct MaxRegs<N, T, IntList<R, R2, Rs...>> {
  static constexpr int a = pass_regs(N, T, R), b = MaxRegs<N, T, IntList<R2, Rs...>>::value;
  static constexpr int value = a > b ? a : b;
};

// Register layout of a radix-R pass: v[b*R + r] holds element j + r*N/R, j = tid + b*T.
template <int N, int T, int R>
struct Geom {
  static constexpr int NB = N / R;
  static constexpr int B = (NB + T - 1) / T;
  static constexpr bool FULL = (NB % T) == 0;
  static __device__ __forceinline__ bool live(int j) { return FULL || j < NB; }
};

// Line data streams through once (HBM in, HBM out).  Its loads and stores are buffer
// instructions on a resource covering the workgroup's lines: the line base lives in scalar
// registers, each lane's offset j*8 is one loop-invariant VGPR and the pass stride r*N/R*8 is a
// scalar offset, so no per-line 64-bit address arithmetic (and no address registers that a
// pending store would pin) exists.  The resource's size bounds every access: lanes past the end
// read zeros and their stores are dropped, which makes ragged tails branch-free.  Accesses carry
// the non-temporal hint so they do not displace the filter and twiddle tables from the caches.
typedef unsigned int rdf_v2u __attribute__((ext_vector_type(2)));
constexpr int kBufNonTemporal = 2;
constexpr int kBufDword3 = 0x00020000;  // raw (untyped) 32-bit data format

struct LineIO {
  __amdgpu_buffer_rsrc_t rsrc;
  // lines [first, first + count) of a row-major [*][N] complex array, clipped to `total` lines
  __device__ __forceinline__ LineIO(const float2* base, int N, int64_t first, int count,
                                    int64_t total) {
    int64_t n = total - first;
    n = n < 0 ? 0 : (n > count ? count : n);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(base + first * N), 0,
                                             int(n * N * 8), kBufDword3);
  }
};

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void load_line(float2* v, const LineIO& io, int elem0, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        const rdf_v2u x = __builtin_amdgcn_raw_buffer_load_b64(io.rsrc, (elem0 + j) * 8,
                                                               r * G::NB * 8, AUX);
        v[b * R + r] = __builtin_bit_cast(float2, x);
      }
    }
  }
}

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void store_line(const float2* v, const LineIO& io, int elem0, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(rdf_v2u, v[b * R + r]), io.rsrc,
                                              (elem0 + j) * 8, r * G::NB * 8, AUX);
    }
  }
}

// binary16 line storage: interleaved complex, 4 bytes a sample (real, imaginary), float32 in
// registers.  Loads convert exactly; stores round to nearest even (the IEEE conversion: values
// beyond the binary16 range become infinities).  Same resource scheme as LineIO.
typedef _Float16 rdf_h2 __attribute__((ext_vector_type(2)));
struct LineIOh {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ LineIOh(const void* base, int N, int64_t first, int count, int64_t total) {
    int64_t n = total - first;
    n = n < 0 ? 0 : (n > count ? count : n);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(base)) + first * N * 4, 0, int(n * N * 4), kBufDword3);
  }
};

__device__ __forceinline__ float2 h2_to_f2(unsigned int u) {
  const rdf_h2 h = __builtin_bit_cast(rdf_h2, u);
  return make_float2(float(h.x), float(h.y));
}
__device__ __forceinline__ unsigned int f2_to_h2(float2 v) {
  rdf_h2 h;
  h.x = static_cast<_Float16>(v.x);
  h.y = static_cast<_Float16>(v.y);
  return __builtin_bit_cast(unsigned int, h);
}

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void load_line_h(float2* v, const LineIOh& io, int elem0, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        v[b * R + r] = h2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(io.rsrc, (elem0 + j) * 4, r * G::NB * 4, AUX));
      }
    }
  }
}

// The same loads, the samples left packed (real half in the low 16 bits); h2_to_f2 unpacks one.
template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void load_line_h_packed(unsigned int* v, const LineIOh& io, int elem0,
                                                   int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        v[b * R + r] = __builtin_amdgcn_raw_buffer_load_b32(io.rsrc, (elem0 + j) * 4, r * G::NB * 4, AUX);
      }
    }
  }
}

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void store_line_h(const float2* v, const LineIOh& io, int elem0, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(f2_to_h2(v[b * R + r]), io.rsrc, (elem0 + j) * 4,
                                              r * G::NB * 4, AUX);
    }
  }
}

// Zero-padded line I/O: a line of n_line < N samples (consecutive lines n_line apart) enters an
// N-point transform, and the outputs at positions [skip, skip + n_line) of the transform are
// stored as the line.  An access that falls outside its window gets an offset past the
// resource's size, so the hardware range check reads zero or drops the store (no branch).
constexpr uint32_t kBufOff = 0x80000000u;  // past any line resource of this library

// A line of n_line samples, periodically extended to n_ext (n_line <= n_ext < 2 n_line) and
// zero-padded to N: element e reads x[e] for e < n_line, x[e - n_line] for e < n_ext, else 0
// (an offset past the resource, which the hardware range check turns into zero).
template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void load_line_pad(float2* v, const LineIO& io, int elem0, int tid,
                                              int n_line, int n_ext) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        const int e = j + r * G::NB;
        const int w = e < n_line ? e : e - n_line;
        const uint32_t off = e < n_ext ? uint32_t(elem0 + w) * 8u : kBufOff;
        v[b * R + r] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(io.rsrc, off, 0, AUX));
      }
    }
  }
}

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void store_line_pad(const float2* v, const LineIO& io, int elem0, int tid,
                                               int n_line, int skip) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int o = j + r * G::NB - skip;
        const uint32_t off = uint32_t(o) < uint32_t(n_line) ? uint32_t(elem0 + o) * 8u : kBufOff;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(rdf_v2u, v[b * R + r]), io.rsrc, off, 0, AUX);
      }
    }
  }
}

// binary16 forms of the padded line I/O above (4-byte elements; same windows)
template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void load_line_pad_h(float2* v, const LineIOh& io, int elem0, int tid,
                                                int n_line, int n_ext) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        const int e = j + r * G::NB;
        const int w = e < n_line ? e : e - n_line;
        const uint32_t off = e < n_ext ? uint32_t(elem0 + w) * 4u : kBufOff;
        v[b * R + r] = h2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(io.rsrc, off, 0, AUX));
      }
    }
  }
}

template <int N, int T, int R, int AUX = kBufNonTemporal>
__device__ __forceinline__ void store_line_pad_h(const float2* v, const LineIOh& io, int elem0, int tid,
                                                 int n_line, int skip) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int o = j + r * G::NB - skip;
        const uint32_t off = uint32_t(o) < uint32_t(n_line) ? uint32_t(elem0 + o) * 4u : kBufOff;
        __builtin_amdgcn_raw_buffer_store_b32(f2_to_h2(v[b * R + r]), io.rsrc, off, 0, AUX);
      }
    }
  }
}

// Reads of the pass after the exchange keyed NS (the product of the radices before it).
template <int N, int T, int R, int NS>
__device__ __forceinline__ void load_lds(float2* v, const float2* lds, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
      const int pj = xpad<N, NS>(j);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = dft_input_order<R>(i);
        v[b * R + r] = lds[xpad_step<N, NS, G::NB, false>(pj, j, r)];
      }
    }
  }
}

template <int N, int T, int R, int NS>
__device__ __forceinline__ void store_lds(const float2* v, float2* lds, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    const int j = tid + b * T;
    if (G::live(j)) {
      const int base = (j / NS) * (NS * R) + (j % NS);
      const int pb = xpad<N, NS>(base);
      // a pad period that is a multiple of NS R keeps a thread's R outputs inside one period
      constexpr bool fits = XPad<N, NS>::Q % (NS * R) == 0;
#pragma unroll
      for (int r = 0; r < R; ++r) lds[xpad_step<N, NS, NS, fits>(pb, base, r)] = v[b * R + r];
    }
  }
}

// Inter-pass twiddles W_{NS R}^{(j mod NS) r} = tw[(j mod NS) r N/(NS R)], tw[k] = e^{-j2pi k/N}.
template <int N, int T, int R, int NS, int DIR>
__device__ __forceinline__ void twiddle(float2* v, const float2* __restrict__ tw, int tid) {
  if constexpr (NS > 1) {
    using G = Geom<N, T, R>;
    constexpr int STEP = N / (NS * R);
#pragma unroll
    for (int b = 0; b < G::B; ++b) {
      const int j = tid + b * T;
      if (G::live(j)) {
        const int e = (j % NS) * STEP;
#pragma unroll
        for (int r = 1; r < R; ++r) {
          float2 w = tw[e * r];
          if (DIR > 0) w.y = -w.y;
          v[b * R + r] = cmul(v[b * R + r], w);
        }
      }
    }
  }
}

template <int N, int T, int R, int DIR>
__device__ __forceinline__ void butterflies(float2* v, int tid) {
  using G = Geom<N, T, R>;
#pragma unroll
  for (int b = 0; b < G::B; ++b) {
    if (G::live(tid + b * T)) Dft<R, DIR>::run(v + b * R);
  }
}

// Ordering of an exchange through LDS.  When every thread of a transform lies in one wave
// (WAVE), the wave's LDS accesses execute in program order, so the exchange needs only to keep
// the compiler from moving accesses across it; otherwise it is a workgroup barrier.
template <bool WAVE>
__device__ __forceinline__ void exchange_sync() {
  if constexpr (WAVE) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// The passes of one transform.  Every thread of the workgroup must call run() (it contains
// workgroup barriers unless WAVE); threads whose butterflies fall past N/R idle through a pass.
template <int N, int T, int DIR, int NS, class L, bool WAVE = false>
struct Passes;

template <int N, int T, int DIR, int NS, int R, bool WAVE>
struct Passes<N, T, DIR, NS, IntList<R>, WAVE> {
  static __device__ __forceinline__ void run(float2* v, float2* lds, const float2* __restrict__ tw,
                                             int tid) {
    twiddle<N, T, R, NS, DIR>(v, opaque(tw), tid);
    butterflies<N, T, R, DIR>(v, tid);
  }
};

template <int N, int T, int DIR, int NS, int R, int R2, int... Rs, bool WAVE>
struct Passes<N, T, DIR, NS, IntList<R, R2, Rs...>, WAVE> {
  static __device__ __forceinline__ void run(float2* v, float2* lds, const float2* __restrict__ tw,
                                             int tid) {
    twiddle<N, T, R, NS, DIR>(v, opaque(tw), tid);
    butterflies<N, T, R, DIR>(v, tid);
    exchange_sync<WAVE>();  // the line buffer may still be read by the previous exchange
    store_lds<N, T, R, NS>(v, lds, tid);
    exchange_sync<WAVE>();
    load_lds<N, T, R2, NS>(v, lds, tid);
    Passes<N, T, DIR, NS * R, IntList<R2, Rs...>, WAVE>::run(v, lds, tw, tid);
  }
};

// ---------------------------------------------------------------------------- exact roots
// W_N^m = e^{-j 2 pi m / N} (m >= 0) evaluated on the device.  The index is reduced to its
// quadrant in integer arithmetic, so the float32 argument 2 r / N of sincospi is below 1/2 and
// rounded once (exact for N a power of two); the quadrant turn is a sign/swap.  Used for
// twiddle sets that a workgroup builds once: reading them from a global table with strided
// lane addresses (every workgroup at once) was measured to cost microseconds per launch.
template <int N>
__device__ __forceinline__ float2 root_of(int m) {
  if constexpr (N % 4 != 0) {
    // no exact quadrants: reduce m to (-N/2, N/2], so the argument of sincospi is in (-1, 1]
    m %= N;
    if (2 * m > N) m -= N;
    float sn, cs;
    sincospif(float(2 * m) / float(N), &sn, &cs);
    return make_float2(cs, -sn);
  }
  m %= N;
  const int q = (4 * m) / N;
  const int r = m - q * (N / 4);
  float sn, cs;
  sincospif(float(2 * r) / float(N), &sn, &cs);
  switch (q) {  // (cs - j sn) (-j)^q
    case 0: return make_float2(cs, -sn);
    case 1: return make_float2(-sn, -cs);
    case 2: return make_float2(-cs, sn);
    default: return make_float2(sn, cs);
  }
}

// ---------------------------------------------------------------------------- register-cached twiddles
// The inter-pass twiddles of a whole transform, loaded once into registers.  A persistent
// workgroup that transforms many lines then issues no table loads inside its line loop, so the
// only global loads in flight are line data (which can be prefetched a line ahead: vector
// memory counters complete in order, so any table load waited on mid-line would also wait for
// the prefetch).
template <int N, int T, int NS, class L>
struct TwCache;

// A pass whose twiddle set is small (NS (R-1) entries, at most TwLdsBudget<N>::bytes) keeps it
// in LDS, stored r-major so the lanes of a wave read consecutive entries; larger sets (one per
// thread) stay in registers.  tw_lds points at this pass's slice of the workgroup's twiddle LDS.
// The budget is 4 KB unless a line configuration below raises it for its length (where the
// line leaves LDS unused but registers are scarce).
template <int N>
struct TwLdsBudget {
  static constexpr int bytes = 4096;
};
template <int N, int NS, int R>
constexpr bool tw_in_lds() { return NS > 1 && NS * (R - 1) * 8 <= TwLdsBudget<N>::bytes; }
// A register-held twiddle set of a power-of-two radix may keep only the powers w^(2^i) of each
// butterfly's base root w and form the others as products when applied (log2 R instead of R - 1
// registers per butterfly, for R - 1 - log2 R extra complex multiplies per application).
template <int N>
struct TwDerive {
  static constexpr bool value = false;
};
// Range compression of a line whose filter is not held in registers may issue the next line's
// prefetch after the filter multiply (the prefetch then overlaps the inverse transform only, and
// the filter loads do not wait for it).
template <int N>
struct PfLate {
  static constexpr bool value = false;
};
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
template <int N, int NS, int R>
constexpr int tw_lds_len() { return tw_in_lds<N, NS, R>() ? NS * (R - 1) : 0; }

template <int N, int T, int NS, int R>
struct TwCacheBase {
  using G = Geom<N, T, R>;
  static constexpr bool IN_LDS = tw_in_lds<N, NS, R>();
  static constexpr bool DERIVE = NS > 1 && !IN_LDS && TwDerive<N>::value && R > 2;
  static constexpr int KB = DERIVE ? ilog2(R - 1) + 1 : R - 1;  // registers per butterfly
  static constexpr int K = (NS > 1 && !IN_LDS) ? G::B * KB : 1;
  float2 w[K];
  const float2* lw = nullptr;
  // every thread of the workgroup calls this; the caller synchronises before first use
  __device__ __forceinline__ void load(const float2* __restrict__ tw, float2* tw_lds, int tid,
                                       int wg_tid, int wg_size) {
    constexpr int STEP = N / (NS * R);
    if constexpr (IN_LDS) {
      for (int i = wg_tid; i < NS * (R - 1); i += wg_size) {
        const int r = i / NS + 1, m = i % NS;     // entry (r, m) = W_N^{m STEP r}
        tw_lds[i] = root_of<N>(m * STEP * r);
      }
      lw = tw_lds;
    } else if constexpr (DERIVE) {
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        const int j = tid + b * T;
        const int e = (j % NS) * STEP;
#pragma unroll
        for (int i = 0; i < KB; ++i)
          w[b * KB + i] = G::live(j) ? root_of<N>(e << i) : make_float2(1.f, 0.f);
      }
    } else if constexpr (NS > 1) {
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        const int j = tid + b * T;
        const int e = (j % NS) * STEP;
#pragma unroll
        for (int r = 1; r < R; ++r)
          w[b * (R - 1) + r - 1] = G::live(j) ? root_of<N>(e * r) : make_float2(1.f, 0.f);
      }
    }
  }
  // Marks the register-held set as used here (see touch): placed before a line loop, it makes
  // the wait for its loads happen there, once, instead of inside the loop, where the wait would
  // also cover the stores of the previous line.
  __device__ __forceinline__ void touch_regs() const {
    if constexpr (NS > 1 && !IN_LDS) touch<K>(w);
  }
  template <int DIR>
  __device__ __forceinline__ void apply(float2* v, int tid) const {
    if constexpr (DERIVE) {
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        if (G::live(tid + b * T)) {
          // p[r] = w^r: powers of two from the registers, the rest as w^(2^k) * w^(r - 2^k)
          // (the base roots pass through an empty asm statement, so the products are formed
          // here at every application instead of being hoisted out of a line loop into R - 1
          // live registers)
          float2 p[R];
#pragma unroll
          for (int r = 1; r < R; ++r) {
            const int hb = 1 << ilog2(r);
            if (hb == r) {
              p[r] = w[b * KB + ilog2(r)];
              asm volatile("" : "+v"(p[r].x), "+v"(p[r].y));
            } else {
              p[r] = cmul(p[hb], p[r - hb]);
            }
            float2 x = p[r];
            if (DIR > 0) x.y = -x.y;
            v[b * R + r] = cmul(v[b * R + r], x);
          }
        }
      }
    } else if constexpr (NS > 1) {
#pragma unroll
      for (int b = 0; b < G::B; ++b) {
        const int j = tid + b * T;
        if (G::live(j)) {
#pragma unroll
          for (int r = 1; r < R; ++r) {
            float2 x = IN_LDS ? lw[(r - 1) * NS + (j % NS)] : w[b * (R - 1) + r - 1];
            if (DIR > 0) x.y = -x.y;
            v[b * R + r] = cmul(v[b * R + r], x);
          }
        }
      }
    }
  }
};

template <int N, int T, int NS, int R>
struct TwCache<N, T, NS, IntList<R>> : TwCacheBase<N, T, NS, R> {
  static constexpr int LDS = tw_lds_len<N, NS, R>();
  __device__ __forceinline__ void load_all(const float2* __restrict__ tw, float2* tw_lds, int tid,
                                           int wg_tid, int wg_size) {
    this->load(tw, tw_lds, tid, wg_tid, wg_size);
  }
  __device__ __forceinline__ void touch_all() const { this->touch_regs(); }
};

template <int N, int T, int NS, int R, int R2, int... Rs>
struct TwCache<N, T, NS, IntList<R, R2, Rs...>> : TwCacheBase<N, T, NS, R> {
  using Next = TwCache<N, T, NS * R, IntList<R2, Rs...>>;
  static constexpr int LDS = tw_lds_len<N, NS, R>() + Next::LDS;  // twiddle LDS entries, all passes
  Next next;
  __device__ __forceinline__ void load_all(const float2* __restrict__ tw, float2* tw_lds, int tid,
                                           int wg_tid, int wg_size) {
    this->load(tw, tw_lds, tid, wg_tid, wg_size);
    next.load_all(tw, tw_lds + tw_lds_len<N, NS, R>(), tid, wg_tid, wg_size);
  }
  __device__ __forceinline__ void touch_all() const {
    this->touch_regs();
    next.touch_all();
  }
};

// The passes of one transform with twiddles from a TwCache (same contract as Passes).
template <int N, int T, int DIR, int NS, class L, bool WAVE = false>
struct PassesCached;

// run2: the double-buffered form.  Consecutive exchanges alternate between two line buffers a and
// b, so an exchange's writes cannot meet the previous exchange's reads (those complete before the
// barrier of the exchange in between) and need no barrier before them: one barrier per exchange
// instead of two.  A caller chaining transforms continues with the buffer the last exchange did
// not use (see LdsDouble).
template <int N, int T, int DIR, int NS, int R, bool WAVE>
struct PassesCached<N, T, DIR, NS, IntList<R>, WAVE> {
  static __device__ __forceinline__ void run(float2* v, float2* lds,
                                             const TwCache<N, T, NS, IntList<R>>& c, int tid) {
    c.template apply<DIR>(v, tid);
    butterflies<N, T, R, DIR>(v, tid);
  }
  static __device__ __forceinline__ void run2(float2* v, float2*, float2*,
                                              const TwCache<N, T, NS, IntList<R>>& c, int tid) {
    c.template apply<DIR>(v, tid);
    butterflies<N, T, R, DIR>(v, tid);
  }
};

template <int N, int T, int DIR, int NS, int R, int R2, int... Rs, bool WAVE>
struct PassesCached<N, T, DIR, NS, IntList<R, R2, Rs...>, WAVE> {
  static __device__ __forceinline__ void run(float2* v, float2* lds,
                                             const TwCache<N, T, NS, IntList<R, R2, Rs...>>& c,
                                             int tid) {
    c.template apply<DIR>(v, tid);
    butterflies<N, T, R, DIR>(v, tid);
    exchange_sync<WAVE>();
    store_lds<N, T, R, NS>(v, lds, tid);
    exchange_sync<WAVE>();
    load_lds<N, T, R2, NS>(v, lds, tid);
    PassesCached<N, T, DIR, NS * R, IntList<R2, Rs...>, WAVE>::run(v, lds, c.next, tid);
  }
  static __device__ __forceinline__ void run2(float2* v, float2* a, float2* b,
                                              const TwCache<N, T, NS, IntList<R, R2, Rs...>>& c,
                                              int tid) {
    c.template apply<DIR>(v, tid);
    butterflies<N, T, R, DIR>(v, tid);
    store_lds<N, T, R, NS>(v, a, tid);
    exchange_sync<WAVE>();
    load_lds<N, T, R2, NS>(v, a, tid);
    PassesCached<N, T, DIR, NS * R, IntList<R2, Rs...>, WAVE>::run2(v, b, a, c.next, tid);
  }
};

// Range compression of a length whose kernel fits only one workgroup per CU may hold two line
// buffers in LDS and run its exchanges double-buffered (PassesCached::run2).  A transform of
// `count` passes makes count - 1 exchanges; starting with buffer a, its last exchange used a when
// that number is odd, so the next transform starts with b (and, the inverse making as many
// exchanges, the following line's forward transform starts with a again).
template <int N>
struct LdsDouble {
  static constexpr bool value = false;
};
template <>
struct LdsDouble<6000> {
  static constexpr bool value = true;
};

// ---------------------------------------------------------------------------- line configurations
// T threads per line (16 points per thread in radix-16 passes), LPW lines per workgroup.  The
// forward and inverse transforms run the same list of passes (a list that starts and ends with
// the same radix: the forward transform's output layout is then the inverse transform's input
// layout), so one twiddle cache serves both.  PF: the range-compression kernel holds
// a prefetched second line in registers.  HREG: the filter H is held in registers for the
// kernel's lifetime (else read from the cached global table per line, all of a thread's filter
// loads issued together).  TWB: twiddle sets up to TWB bytes live in LDS.  WPE: waves per SIMD
// the range-compression kernel's registers are sized for (the second launch bound: at most
// 512 / WPE registers per lane).  TWD: register-held twiddle sets keep only the power-of-two
// powers of each root (PfLate/TwDerive above).  LATE: the prefetch is issued after the filter
// multiply.  The long lines (8192, 16384: 512 / 1024 threads, at most 128 registers) need TWD
// to fit a prefetch; measured on MI355X, prefetch + TWD + LATE is 5-7% faster there than no
// prefetch.  At 2048 and 4096 TWD takes the padded range kernels (lines of any length) from two to
// three workgroups per CU, or out of spilling (2048: 202 -> 163 registers, 16384 lines of 1200
// samples 93 -> 90 us), and lets the omega-k row stage at 4096 fit three workgroups per CU.
// (The 4096-point range kernel of the headline is a kernel of its own.)  6000 = 10 * 6 * 10 * 10 on 600 threads (at
// most 12 points a thread) with the prefetch after the filter multiply and the filter read per
// line: 142 registers and no spills, against 255 for 20 * 15 * 20 on 400 threads with the filter
// in registers (measured on MI355X, 8192 lines: 301 against 335 us; the radix-20 butterflies
// alone need ~80 registers, and every 128-register form of either list spills).
template <int N>
struct LineCfg;

#define RDF_LINE_CFG(N_, T_, FWD, INV, PF_, HREG_, TWB_, WPE_, TWD_, LATE_)      \
  template <>                                                                     \
  struct PfLate<N_> {                                                             \
    static constexpr bool value = LATE_;                                          \
  };                                                                              \
  template <>                                                                     \
  struct TwLdsBudget<N_> {                                                        \
    static constexpr int bytes = TWB_;                                            \
  };                                                                              \
  template <>                                                                     \
  struct TwDerive<N_> {                                                           \
    static constexpr bool value = TWD_;                                           \
  };                                                                              \
  template <>                                                                     \
  struct LineCfg<N_> {                                                            \
    static constexpr int N = N_;                                                  \
    static constexpr int T = T_;                                                  \
    using Fwd = FWD;                                                              \
    using Inv = INV;                                                              \
    static constexpr bool PF = PF_;                                               \
    static constexpr bool HREG = HREG_;                                           \
    static constexpr int WPE = WPE_;                                              \
    static constexpr int LPW = T_ >= 256 ? 1 : 256 / T_;                          \
    static constexpr bool WAVE = 64 % T_ == 0; /* a line's threads share one wave */ \
    static constexpr int WG = T_ * LPW;                                           \
    static constexpr int LDS = lds_len(N_);                                       \
    static constexpr int P = MaxRegs<N_, T_, FWD>::value > MaxRegs<N_, T_, INV>::value \
                                 ? MaxRegs<N_, T_, FWD>::value                    \
                                 : MaxRegs<N_, T_, INV>::value;                   \
    static_assert(ListInfo<FWD>::product == N_ && ListInfo<INV>::product == N_,   \
                  "radix list must multiply to N");                               \
    static_assert(ListInfo<FWD>::first == ListInfo<INV>::last &&                  \
                      ListInfo<FWD>::last == ListInfo<INV>::first,                \
                  "inverse list must be the forward list reversed at its ends");  \
  };

using L_16_16 = IntList<16, 16>;
using L_8_8_8 = IntList<8, 8, 8>;
using L_16_4_16 = IntList<16, 4, 16>;
using L_16_8_16 = IntList<16, 8, 16>;
using L_16_16_16 = IntList<16, 16, 16>;
using L_8_4_8_4_8 = IntList<8, 4, 8, 4, 8>;
using L_8_16_16_8 = IntList<8, 16, 16, 8>;
using L_20_15_20 = IntList<20, 15, 20>;  // the earlier 6000-point list (RD_CFG6000 selects it)
using L_10_6_10_10 = IntList<10, 6, 10, 10>;
using L_10_6_10 = IntList<10, 6, 10>;  // the 600-point sub-line transform of the four-step 6000 kernel
template <>
struct TwLdsBudget<600> {
  static constexpr int bytes = 8192;  // both inter-pass twiddle sets of 10 * 6 * 10 in LDS
};

RDF_LINE_CFG(256, 16, L_16_16, L_16_16, true, true, 4096, 1, false, false)
RDF_LINE_CFG(512, 64, L_8_8_8, L_8_8_8, true, true, 4096, 1, false, false)
RDF_LINE_CFG(1024, 64, L_16_4_16, L_16_4_16, true, true, 8192, 1, false, false)
RDF_LINE_CFG(2048, 128, L_16_8_16, L_16_8_16, true, true, 4096, 1, true, false)
RDF_LINE_CFG(4096, 256, L_16_16_16, L_16_16_16, true, true, 4096, 3, true, false)
RDF_LINE_CFG(8192, 512, L_8_4_8_4_8, L_8_4_8_4_8, true, false, 8192, 4, true, true)
RDF_LINE_CFG(16384, 1024, L_8_16_16_8, L_8_16_16_8, true, false, 16384, 1, true, true)
#ifndef RD_CFG6000
#define RD_CFG6000 600, L_10_6_10_10, L_10_6_10_10, true, false, 8192, 2, false, true
#endif
#define RDF_LINE_CFG_X(...) RDF_LINE_CFG(__VA_ARGS__)
RDF_LINE_CFG_X(6000, RD_CFG6000)
#undef RDF_LINE_CFG_X

#undef RDF_LINE_CFG

// ---------------------------------------------------------------------------- column configurations
// Length-L transforms along the rows of a row-major array (one column per lane, 64 columns per
// workgroup).  T = L/16 threads per column hold 16 points each in radix-16 passes.
template <int L>
struct ColCfg;

#define RDF_COL_CFG(L_, FWD, INV)                                                 \
  template <>                                                                     \
  struct ColCfg<L_> {                                                             \
    static constexpr int L = L_;                                                  \
    static constexpr int T = L_ / 16;                                             \
    static constexpr int COLS = 64;                                               \
    static constexpr int WG = T * COLS;                                           \
    using Fwd = FWD;                                                              \
    using Inv = INV;                                                              \
    static constexpr int LDS = lds_len(L_) | 1;                                   \
    static constexpr int P = MaxRegs<L_, T, FWD>::value > MaxRegs<L_, T, INV>::value \
                                 ? MaxRegs<L_, T, FWD>::value                     \
                                 : MaxRegs<L_, T, INV>::value;                    \
    static_assert(ListInfo<FWD>::product == L_ && ListInfo<INV>::product == L_,   \
                  "radix list must multiply to L");                               \
  };

using L_16 = IntList<16>;
using L_5_5 = IntList<5, 5>;
using L_16_2 = IntList<16, 2>;
using L_2_16 = IntList<2, 16>;
using L_16_4 = IntList<16, 4>;
using L_4_16 = IntList<4, 16>;
using L_16_8 = IntList<16, 8>;
using L_8_16 = IntList<8, 16>;

RDF_COL_CFG(16, L_16, L_16)
RDF_COL_CFG(32, L_16_2, L_2_16)
RDF_COL_CFG(64, L_16_4, L_4_16)
RDF_COL_CFG(128, L_16_8, L_8_16)
RDF_COL_CFG(256, L_16_16, L_16_16)
RDF_COL_CFG(25, L_5_5, L_5_5)

#undef RDF_COL_CFG

}  // namespace rdf
