// hq_device.h — device building blocks of the HyperQuant HIP kernels (gfx950).
//
// Source of the method: "HyperQuant: A Rate-Distortion-Optimal Quantization
// Pipeline for Large Language and Diffusion Models", gist.science explainer,
// section "Methodology: The HyperQuant Pipeline" (cited below as Methodology
// 1-4).  Every floating-point step is one IEEE binary32 operation in a fixed
// order (the library is built with -ffp-contract=off and without fast-math),
// so that the output is a pure function of the input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kChunkTiles = 64;   // tiles per chunk of the stream
constexpr int kLaneElems = 32;    // tile elements held by one lane
// 1/sqrt(n) is a power of two (n = 64, 256): scaling by it is exact wherever
// the scaled value is representable
template <int N>
constexpr bool kPow2Scale = (N == 64 || N == 256);
constexpr int kMaxGroupChunks = 4;   // most chunks an encode workgroup stages per ticket (one look-back each)

// --------------------------------------------------------------------------
// Counter-based generator: the "pcg" hash of Jarzynski & Olano (JCGT 9(3),
// 2020): one PCG LCG step followed by PCG's RXS-M-XS output permutation.
// --------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pcg_hash(uint32_t v) {
  uint32_t state = v * 747796405u + 2891336453u;
  uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// bf16 round-to-nearest-even of a finite value (bit arithmetic)
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = as_u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// two floats -> packed bf16 pair (low half = lo), round to nearest even
// (v_cvt_pk_bf16_f32); the same bits as bf16_rne_bits for finite values
typedef __bf16 hq_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hq_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const hq_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hq_bf16x2));
}

__device__ __forceinline__ uint32_t zigzag(int32_t v) {
  return ((uint32_t)v << 1) ^ (uint32_t)(v >> 31);
}
__device__ __forceinline__ int32_t unzigzag(uint32_t u) {
  return (int32_t)(u >> 1) ^ -(int32_t)(u & 1u);
}

template <int LAT> struct LatticeTraits;
template <> struct LatticeTraits<1> { static constexpr int dim = 1, coset = 0; };
template <> struct LatticeTraits<2> { static constexpr int dim = 2, coset = 1; };
template <> struct LatticeTraits<4> { static constexpr int dim = 4, coset = 0; };
template <> struct LatticeTraits<8> { static constexpr int dim = 8, coset = 1; };

struct A2Consts { float sqrt3, inv_sqrt3; };

// --------------------------------------------------------------------------
// Nearest lattice points (Methodology 2).  t: d coordinates; writes the
// integer code d[] and coset bit p.  Tie rules: round half to even; the
// moved coordinate of a D_n candidate is the one with the largest |t - rint t|
// (smallest index on ties), moved towards t; E8 picks the half-integer coset
// only when it is strictly nearer.
// --------------------------------------------------------------------------
__device__ __forceinline__ void nearest_z(const float* t, int32_t* d, uint32_t& p) {
  d[0] = (int32_t)__builtin_rintf(t[0]);
  p = 0;
}

__device__ __forceinline__ void nearest_d4(const float* t, int32_t* d, uint32_t& p) {
  float f[4], ad[4];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = __builtin_rintf(t[i]);
    ad[i] = __builtin_fabsf(t[i] - f[i]);
    s += (int32_t)f[i];
  }
  int j = 0;
  float mx = ad[0];
#pragma unroll
  for (int i = 1; i < 4; i++)
    if (ad[i] > mx) { mx = ad[i]; j = i; }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    int32_t a = (int32_t)f[i];
    if ((s & 1) && i == j) a += (t[i] >= f[i]) ? 1 : -1;
    d[i] = a;
  }
  p = 0;
}

// E8 = D8 u (D8 + 1/2) (Methodology 2): the nearer of the two cosets'
// nearest points A (D8) and B (D8 + 1/2).  With delta = t - rint(t) (exact),
//   |t-A|^2 - |t-B|^2 = sum|delta| - 2 + [A moved](1 - 2 max|delta|) - [B moved] 2 min|delta|
// in exact arithmetic (B's moved coordinate is the one of smallest |delta|),
// evaluated in fp32 in this order; B iff it is > 0.
//
// The encoder goes straight to Rice symbols (nearest_e8_symbols), arranged
// for fewer operations.  With f = rint(t) and delta = t - f:
//  - floor(t) = f - [delta < 0], so the half-integer candidate's coset parity
//    is f's parity flipped by the number of negative deltas;
//  - the moved coordinate is the first one whose |delta| equals the max (A)
//    or the min (B); A moves it by +1 if delta >= 0 else -1; B moves
//    floor(t) by +1 if t >= floor(t) + 1/2, i.e. if delta < 0 or
//    delta == 1/2, else by -1.
// Every integer code is d = f + adj: adj = -[B and delta < 0] (the floor)
// for the coordinates that do not move, and that plus the move for the one
// that does.  The symbol zz(d) = |2 d + 1/2| - 1/2 is the truncation of
// |fma(f, 2, 1/2 + 2 adj)| to an integer (exact: small integers and halves).
// The per-coordinate conditions are lane masks ("first equal" and the parity
// of the negative deltas are scalar mask operations), and the moved
// coordinate's 1/2 + 2 adj is one per-lane value, so each coordinate costs two
// selects, an fma and a conversion.
struct E8Choice {
  float f[8];        // rint(t)
  float dl[8];       // t - rint(t) (exact)
  bool neg[8];       // t - rint(t) < 0
  bool first[8];     // the moved coordinate, if any moves (at most one)
  bool useB;         // half-integer coset
  bool negj;         // the first coordinate's delta is negative
  float mvh;         // the move: +1, -1, or 0 when no coordinate moves
};

__device__ __forceinline__ void e8_choose(const float* t, E8Choice& c) {
  float ad[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    c.f[i] = __builtin_rintf(t[i]);
    c.dl[i] = t[i] - c.f[i];
    ad[i] = __builtin_fabsf(c.dl[i]);
    c.neg[i] = c.dl[i] < 0.0f;
  }
  const float sf = ((c.f[0] + c.f[1]) + (c.f[2] + c.f[3])) + ((c.f[4] + c.f[5]) + (c.f[6] + c.f[7]));   // exact
  const bool oddA = ((int32_t)sf & 1) != 0;
  bool nneg = false;
#pragma unroll
  for (int i = 0; i < 8; i++) nneg = nneg ^ c.neg[i];
  const bool oddB = oddA != nneg;
  // (max and min are exact and order-free on these finite values: grouped
  // for three-operand instructions)
  const float mx = __builtin_fmaxf(
      __builtin_fmaxf(__builtin_fmaxf(ad[0], __builtin_fmaxf(ad[1], ad[2])), __builtin_fmaxf(ad[3], __builtin_fmaxf(ad[4], ad[5]))),
      __builtin_fmaxf(ad[6], ad[7]));
  const float mn = __builtin_fminf(
      __builtin_fminf(__builtin_fminf(ad[0], __builtin_fminf(ad[1], ad[2])), __builtin_fminf(ad[3], __builtin_fminf(ad[4], ad[5]))),
      __builtin_fminf(ad[6], ad[7]));
  const float sabs = ((ad[0] + ad[1]) + (ad[2] + ad[3])) + ((ad[4] + ad[5]) + (ad[6] + ad[7]));
  // (2 mx and 2 mn are exact, so each fused multiply-add below rounds once,
  // as the two-operation forms 1 - 2 mx and diff - 2 mn do)
  float diff = sabs - 2.0f;
  if (oddA) diff = diff + __builtin_fmaf(-2.0f, mx, 1.0f);
  if (oddB) diff = __builtin_fmaf(-2.0f, mn, diff);
  c.useB = diff > 0.0f;
  const float target = c.useB ? mn : mx;
  // (bitwise operators on the conditions: they stay lane masks)
  bool seen = false, negj = false;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const bool eq = ad[i] == target;
    c.first[i] = eq & !seen;
    seen = seen | eq;
    negj = negj | (c.first[i] & c.neg[i]);
  }
  c.negj = negj;
  const bool odd = c.useB ? oddB : oddA;
  const bool up = c.useB ? (negj | (target == 0.5f)) : !negj;
  c.mvh = odd ? (up ? 1.0f : -1.0f) : 0.0f;
}

__device__ __forceinline__ void nearest_e8_symbols(const float* t, uint32_t* u, uint32_t& p) {
  E8Choice c;
  e8_choose(t, c);
  // 1/2 + 2 adj of the moved coordinate
  const float K = ((c.useB & c.negj) ? -1.5f : 0.5f) + 2.0f * c.mvh;
#pragma unroll
  for (int i = 0; i < 7; i++) {
    const float x = (c.useB & c.neg[i]) ? -1.5f : 0.5f;
    const float cc = c.first[i] ? K : x;
    u[i] = (uint32_t)__builtin_fabsf(__builtin_fmaf(c.f[i], 2.0f, cc));
  }
  {
    // the last coordinate is stored halved (floor), its parity being the others' sum's:
    // floor((f + adj) / 2) with adj / 2 = (cc - 1/2) / 4
    const float x = (c.useB & c.neg[7]) ? -0.5f : 0.0f;
    const float ch = c.first[7] ? __builtin_fmaf(K, 0.25f, -0.125f) : x;
    const float h = __builtin_floorf(__builtin_fmaf(c.f[7], 0.5f, ch));
    u[7] = (uint32_t)__builtin_fabsf(__builtin_fmaf(h, 2.0f, 0.5f));
  }
  p = c.useB ? 1u : 0u;
}

// The nearest E8 point itself (same choice): f + adj, plus 1/2 in coset B.
__device__ __forceinline__ void nearest_e8_point(const float* t, float* pt) {
  E8Choice c;
  e8_choose(t, c);
  const float base = c.useB ? 0.5f : 0.0f;
  const float Kp = ((c.useB & c.negj) ? -0.5f : base) + c.mvh;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float x = (c.useB & c.neg[i]) ? -0.5f : base;
    pt[i] = c.f[i] + (c.first[i] ? Kp : x);
  }
}

// t - (its nearest E8 point), for t a multiple of 2^-23 in [-1, 1) (the
// dither's box sample): (t - f) - (adj + p/2) with the point never formed.
// Both ways are exact for such t (every value is a multiple of 2^-23 below 2
// in magnitude), so this equals t - nearest_e8_point(t).
__device__ __forceinline__ void e8_box_residual(const float* t, float* u) {
  E8Choice c;
  e8_choose(t, c);
  const float base = c.useB ? 0.5f : 0.0f;
  const float Kp = ((c.useB & c.negj) ? -0.5f : base) + c.mvh;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float x = (c.useB & c.neg[i]) ? -0.5f : base;
    u[i] = c.dl[i] - (c.first[i] ? Kp : x);
  }
}

// A2 = R u (R + (1/2, sqrt3/2)), R = Z x sqrt3 Z; code (p, m, n') with point
// (m + p/2, sqrt3 (n' + p/2)).
__device__ __forceinline__ void nearest_a2(const float* t, int32_t* d, uint32_t& p, A2Consts k) {
  float s1 = t[1] * k.inv_sqrt3;
  float am = __builtin_rintf(t[0]), an = __builtin_rintf(s1);
  float bm = __builtin_floorf(t[0]), bn = __builtin_floorf(s1);
  float a1 = k.sqrt3 * an;
  float b0 = bm + 0.5f, b1 = k.sqrt3 * (bn + 0.5f);
  float ea0 = t[0] - am, ea1 = t[1] - a1;
  float eb0 = t[0] - b0, eb1 = t[1] - b1;
  float da = ea0 * ea0 + ea1 * ea1;
  float db = eb0 * eb0 + eb1 * eb1;
  const bool useB = db < da;
  d[0] = (int32_t)(useB ? bm : am);
  d[1] = (int32_t)(useB ? bn : an);
  p = useB ? 1u : 0u;
}

// Z, A2 and D4 (E8 goes through e8_choose)
template <int LAT>
__device__ __forceinline__ void nearest(const float* t, int32_t* d, uint32_t& p, A2Consts k) {
  static_assert(LAT != 8, "E8: nearest_e8_symbols / nearest_e8_point");
  if constexpr (LAT == 1) nearest_z(t, d, p);
  else if constexpr (LAT == 2) nearest_a2(t, d, p, k);
  else nearest_d4(t, d, p);
}

// lattice point (as floats) of a code (used for the dither reduction)
template <int LAT>
__device__ __forceinline__ void code_point(const int32_t* d, uint32_t p, float* pt, A2Consts k) {
  constexpr int D = LatticeTraits<LAT>::dim;
  if constexpr (LAT == 2) {
    float h = p ? 0.5f : 0.0f;
    pt[0] = (float)d[0] + h;
    pt[1] = k.sqrt3 * ((float)d[1] + h);
  } else {
#pragma unroll
    for (int i = 0; i < D; i++) pt[i] = (LAT == 8 && p) ? (float)d[i] + 0.5f : (float)d[i];
  }
}

// Bit-stripping + zigzag (Methodology 3): the last coordinate of a D4/E8
// block is stored halved (its parity equals that of the other coordinates'
// sum); everything else is zigzag-mapped.
template <int LAT>
__device__ __forceinline__ void block_symbols(const int32_t* d, uint32_t* u) {
  constexpr int D = LatticeTraits<LAT>::dim;
#pragma unroll
  for (int i = 0; i < D; i++) {
    int32_t v = d[i];
    if ((LAT == 4 || LAT == 8) && i == D - 1) v = v >> 1;   // arithmetic shift: floor(v / 2)
    u[i] = zigzag(v);
  }
}

// Subtractive dither (Methodology 4): v uniform on a box that is a
// fundamental region of a sublattice (E8, D4: [-1,1)^d of 2Z^d; Z: [-1/2,1/2);
// A2: [-1/2,1/2) x sqrt3 [-1/2,1/2) of Z x sqrt3 Z), reduced into the Voronoi
// cell: u = v - Q(v).  24 uniform bits per coordinate g.
template <int LAT>
__device__ __forceinline__ void dither_block(uint32_t key_dither, uint32_t g0, float* u, A2Consts k) {
  constexpr int D = LatticeTraits<LAT>::dim;
  float v[D];
#pragma unroll
  for (int i = 0; i < D; i++) {
    // (a < 2^24: the product and the difference are exact, so one fused
    // multiply-add gives the same value as the two operations)
    float a = (float)(pcg_hash(key_dither + g0 + (uint32_t)i) >> 8);
    if constexpr (LAT == 8 || LAT == 4) v[i] = __builtin_fmaf(a, 0x1p-23f, -1.0f);
    else v[i] = __builtin_fmaf(a, 0x1p-24f, -0.5f);
  }
  if constexpr (LAT == 2) v[1] = k.sqrt3 * v[1];
  if constexpr (LAT == 8) {
    e8_box_residual(v, u);
  } else {
    float pt[D];
    int32_t d[D];
    uint32_t p;
    nearest<LAT>(v, d, p, k);
    code_point<LAT>(d, p, pt, k);
#pragma unroll
    for (int i = 0; i < D; i++) u[i] = v[i] - pt[i];
  }
}

// This wave's LDS writes made visible to its own later LDS reads (for data
// exchanged among lanes of one wave, such as a tile's lanes): the writes are
// waited for, and neither the compiler nor the scheduler moves accesses
// across.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave votes over the active lanes, straight from the comparison's lane mask
// (a ballot of the condition, then a scalar test).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0ull; }
__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0ull; }

// Index of the lowest set bit of w, all ones when w is 0 (v_ffbl_b32).  Written
// as the instruction itself: the C builtin leaves w == 0 undefined, and the
// compiler then folds the range checks that the fast unary path relies on.
__device__ __forceinline__ uint32_t ffbl(uint32_t w) {
  uint32_t r;
  asm("v_ffbl_b32 %0, %1" : "=v"(r) : "v"(w));
  return r;
}

// Unary codes of an LDS bit array, read through a 64-bit window {hi:lo}
// that holds the next nb valid bits (bits past nb are zero).  take() is the
// straight-line path: the next code is the lowest one bit of lo, found only
// when the run of zeros is shorter than 31 bits; any other case (longer run,
// window exhausted) shows up as z >= 31 in the group's running maximum, and
// the group is then read again from its saved state with next_exact().
// pos() = idx * 32 - nb is the bit index of the window's first bit.
struct UnaryWindow {
  const uint32_t* s;
  uint32_t lo, hi, nb, idx;
  __device__ __forceinline__ void init(const uint32_t* words, uint32_t p0) {
    s = words;
    const uint32_t i = p0 >> 5, sh = p0 & 31u;
    const uint32_t w0 = s[i], w1 = s[i + 1];
    lo = __builtin_amdgcn_alignbit(w1, w0, sh);
    hi = sh ? (w1 >> sh) : w1;
    nb = 64u - sh;
    idx = i + 2u;
  }
  __device__ __forceinline__ uint32_t pos() const { return idx * 32u - nb; }
  // top the window up to more than 32 bits (one word)
  __device__ __forceinline__ void refill() {
    if (nb <= 32u) {
      const uint64_t W = (((uint64_t)hi << 32) | lo) | ((uint64_t)s[idx] << nb);
      lo = (uint32_t)W;
      hi = (uint32_t)(W >> 32);
      idx++;
      nb += 32u;
    }
  }
  // the next 8 codes on the fast path, read at increasing offsets into the
  // unchanged window (each from the 32 bits at its offset), then the window
  // advances once.  The read is exact while every offset and every code stays
  // below 31 (an offset past 30 would wrap the funnel shift).  Offsets grow
  // by code + 1, so that is the last offset and the last code below 31: a
  // slice with no one gives the code 0xFFFFFFFF, which leaves the offset
  // where it was, so every later code reads the same slice and the last code
  // is 0xFFFFFFFF too.  zmax = max(last offset, last code): >= 31 means the
  // fast read is not exact.
  __device__ __forceinline__ void take8(uint32_t (&z)[8], uint32_t& zmax) {
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < 7; i++) {
      z[i] = ffbl(__builtin_amdgcn_alignbit(hi, lo, off));
      off = off + z[i] + 1u;
    }
    z[7] = ffbl(__builtin_amdgcn_alignbit(hi, lo, off));
    zmax = off > z[7] ? off : z[7];
    off = off + z[7] + 1u;
    const uint64_t W = (((uint64_t)hi << 32) | lo) >> (off & 63u);
    lo = (uint32_t)W;
    hi = (uint32_t)(W >> 32);
    nb -= off;
  }
  // next code, any length; returns 0xFFFFFFFF if the run reaches `limit`
  __device__ __forceinline__ uint32_t next_exact(uint32_t limit) {
    uint64_t W = ((uint64_t)hi << 32) | lo;
    uint32_t q = 0;
    while (W == 0ull) {
      q += nb;
      if (idx * 32u >= limit) return 0xFFFFFFFFu;
      W = ((uint64_t)s[idx + 1] << 32) | s[idx];
      idx += 2u;
      nb = 64u;
    }
    const uint32_t l = (uint32_t)W, h = (uint32_t)(W >> 32);
    const uint32_t z = l != 0u ? (uint32_t)__builtin_ctz(l) : 32u + (uint32_t)__builtin_ctz(h);
    W = (W >> z) >> 1;
    nb -= z + 1u;
    lo = (uint32_t)W;
    hi = (uint32_t)(W >> 32);
    return q + z;
  }
};

// Bits [o, o + w) of the little-endian bit string seg[] (w <= 32).  Called
// with o and w fixed by fully unrolled loops, so seg[] is indexed statically.
__device__ __forceinline__ uint32_t seg_bits(const uint32_t* seg, int o, int w) {
  const int j = o >> 5, b = o & 31;
  if (b + w <= 32) return __builtin_amdgcn_ubfe(seg[j], b, w);
  return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(seg[j + 1], seg[j], b), 0, w);
}

// Parity of the first D - 1 coordinates of block b for K >= 2: a coordinate's
// low bit is bit 1 xor bit 0 of its remainder field (bit 1 is the magnitude's
// low bit, bit 0 the zigzag sign, which complements it), so the parity is that
// of the count of those two bits over the block's first D - 1 fields (static
// offsets; chunks of at most 31 bits).
template <int K, int D>
__device__ __forceinline__ uint32_t block_low_parity(const uint32_t* seg, int b) {
  constexpr int F = 31 / K;                                 // fields per chunk
  uint32_t cnt = 0;
#pragma unroll
  for (int f0 = 0; f0 < D - 1; f0 += F) {
    const int nf = (D - 1 - f0) < F ? (D - 1 - f0) : F;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < nf; i++) m |= 3u << (i * K);
    cnt += __builtin_popcount(seg_bits(seg, (b * D + f0) * K, nf * K) & m);
  }
  return cnt & 1u;
}

// Signed coordinate of the e-th code of a lane: unzigzag((q << K) | r) with r
// the e-th K-bit field of the remainder plane.  The zigzag sign is r's low
// bit (as 0 / -1); the magnitude is q above r's upper K-1 bits.
template <int K>
__device__ __forceinline__ int32_t code_coord(const uint32_t* seg, int e, uint32_t qz) {
  if constexpr (K == 0) {
    return (int32_t)(qz >> 1) ^ -(int32_t)(qz & 1u);
  } else {
    const int o = e * K;
    const int32_t neg = __builtin_amdgcn_sbfe((int32_t)seg[o >> 5], o & 31, 1);
    if constexpr (K == 1) return (int32_t)qz ^ neg;
    else return (int32_t)((qz << (K - 1)) | seg_bits(seg, o + 1, K - 1)) ^ neg;
  }
}

// position (0..31) of the r-th set bit (r counted from 0) of w; w has > r ones
// (otherwise the result is some position): a binary search, each level
// counting the ones of the next half-width field at the current position
__device__ __forceinline__ uint32_t select_bit(uint32_t w, uint32_t r) {
  uint32_t pos = 0;
#pragma unroll
  for (uint32_t half = 16; half >= 1; half >>= 1) {
    const uint32_t c = __builtin_popcount(__builtin_amdgcn_ubfe(w, pos, half));
    const uint32_t d = r - c;
    const bool up = (int32_t)d >= 0;                        // r >= c (both below 64)
    r = up ? d : r;
    pos = up ? pos + half : pos;
  }
  return pos;
}

// Sign diagonal on packed bf16 pairs.  For a lane's 32-bit sign mask sgn
// (bit i = sign of element i), pair_sign_words() spreads each 16-element half
// h into W[h]: sign of element 2k at bit 2k, of element 2k + 1 at bit 2k + 16
// (k = 0..7).  pair_sign_mask() shifts pair p's two bits to 15 and 31, the
// sign bits of the packed pair (element 2p low, 2p + 1 high).
__device__ __forceinline__ void pair_sign_words(uint32_t sgn, uint32_t (&W)[2]) {
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const uint32_t sg = (sgn >> (16 * h)) & 0xFFFFu;
    W[h] = (sg & 0x5555u) | ((sg & 0xAAAAu) << 15);
  }
}
__device__ __forceinline__ uint32_t pair_sign_mask(const uint32_t (&W)[2], int p) {
  return (W[p >> 3] << (15 - 2 * (p & 7))) & 0x80008000u;
}
// The same values hidden from loop-invariant code motion: the 32 per-element
// masks would otherwise be hoisted out of the chunk loop and held in 32 VGPRs.
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

// gfx950's global -> LDS load, 16 bytes a lane: from base + voff (bytes) to
// the wave's LDS block at byte address lds (m0), lane i's 16 bytes at
// lds + 16 i.  Written as the instruction: the compiler cannot tell a
// kernel's stage buffers apart and would otherwise wait for it before every
// later LDS access; the callers wait for it themselves (vmcnt, then a
// barrier) before the buffer is read.  It writes no vector register; m0 is
// restored after the issue.
__device__ __forceinline__ void lds_load16(const uint32_t* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}

// The same for one 16-bit value a lane, zero-extended to a 32-bit LDS word
// (lane i's at lds + 4 i).
__device__ __forceinline__ void lds_load_u16(const uint16_t* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}

// The same for one 32-bit word a lane (lane i's at lds + 4 i).
__device__ __forceinline__ void lds_load4(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}

// The same for one 32-bit word a lane (lane i's at lds + 4 i), read coherently
// at device scope (sc1: not from a stale line of this XCD's L2), for words
// that workgroups on other XCDs update with atomics.
__device__ __forceinline__ void lds_load_u32_coherent(const uint32_t* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %2, %3 sc1\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}

// LDS byte address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// v of the lane at physical xor distance px (1, 2, or the half-row mirror
// 7) within its 8-lane group, by DPP (no LDS round trip); other distances
// through the crossbar.  px folds to a constant in the unrolled callers.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int px) {
  if (px == 1) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  if (px == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  if (px == 7) return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  return (uint32_t)__shfl_xor((int)v, px);
}
__device__ __forceinline__ float lane_xor(float v, int px) {
  return __builtin_bit_cast(float, lane_xor(__builtin_bit_cast(uint32_t, v), px));
}

// Inclusive prefix sum of v over a whole wave (all 64 lanes active), in DPP:
// shifts by 1, 2, 4, 8 within each 16-lane row (lanes with no source add 0),
// then row 0's last value into row 1 and row 2's into row 3 (row_bcast:15),
// then row 1's last into rows 2 and 3 (row_bcast:31).
static_assert(kChunkTiles == 64, "a chunk's tiles are scanned by one 64-lane wave");
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Inclusive prefix sum and total of v over the LPT consecutive physical
// lanes of a tile (lanes p = 0..LPT-1 of an aligned group), all in DPP: row
// shifts with the group's edge masked (the shift by 4 writes banks 1 and 3
// only, the upper halves of 8-lane groups), and the total by a butterfly
// (quad swaps, then the half-row mirror).
template <int LPT>
__device__ __forceinline__ void tile_scan(uint32_t v, int p, uint32_t& incl, uint32_t& total) {
  uint32_t inc = v, s = v;
  if constexpr (LPT >= 2) {
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, inc, 0x111, 0xF, 0xF, false);   // row_shr:1
    inc = p >= 1 ? inc + t : inc;
    s += __builtin_amdgcn_update_dpp(0u, s, 0xB1, 0xF, 0xF, false);                    // quad_perm [1,0,3,2]
  }
  if constexpr (LPT >= 4) {
    const uint32_t t = __builtin_amdgcn_update_dpp(0u, inc, 0x112, 0xF, 0xF, false);   // row_shr:2
    inc = p >= 2 ? inc + t : inc;
    s += __builtin_amdgcn_update_dpp(0u, s, 0x4E, 0xF, 0xF, false);                    // quad_perm [2,3,0,1]
  }
  if constexpr (LPT >= 8) {
    inc += __builtin_amdgcn_update_dpp(0u, inc, 0x114, 0xF, 0xA, false);               // row_shr:4, p >= 4
    s += __builtin_amdgcn_update_dpp(0u, s, 0x141, 0xF, 0xF, false);                   // row_half_mirror
  }
  incl = inc;
  total = s;
}

// Issue priority of the calling wave (the hardware's four levels, 0..3).
// Among ready waves the arbiter picks the highest priority, then the oldest:
// with equal priorities the workgroup dispatched first on a CU races ahead
// and the CU ends half empty.  The kernels lower a wave's priority as its
// workgroup's share of the work shrinks, so whichever is behind catches up.
__device__ __forceinline__ void wave_priority(uint32_t p) {
  if (p == 0) __builtin_amdgcn_s_setprio(0);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
}

// Lanes of a tile.  At n = 256 (8 lanes per tile) physical lanes 4..7 hold
// logical lanes 7..4, so that the stride-128 butterfly partner q ^ 4 is the
// half-row mirror p ^ 7, a DPP pattern; the partners q ^ 1 and q ^ 2 stay
// p ^ 1 and p ^ 2 (quad permutes).  Everything that depends on a lane's
// place in the tile uses the logical lane q.
template <int LPT>
__device__ __forceinline__ int tile_lane(int p) { return (LPT == 8 && p >= 4) ? (p ^ 3) : p; }
// physical xor distance to the logical partner q ^ m
template <int LPT>
__device__ __forceinline__ constexpr int partner_xor(int m) { return (LPT == 8 && m == 4) ? 7 : m; }

// One cross-lane stage on eight elements: a[o + i] += f * partner's a[o + i]
// as v_fmac_f32_dpp, the partner selected by the DPP control.  One fused
// multiply-add with a +-1 factor rounds once, like the butterfly's add.
// s_nop 4: a VGPR written by a VALU op (or EXEC written by SALU) right
// before must not be read through DPP within 2 (5) wait states.
#define HQ_FMAC_DPP8(CTRL, a, o, f)                                                               \
  asm("s_nop 4\n"                                                                                \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                           \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                              \
      : "+v"(a[(o) + 0]), "+v"(a[(o) + 1]), "+v"(a[(o) + 2]), "+v"(a[(o) + 3]), "+v"(a[(o) + 4]),  \
        "+v"(a[(o) + 5]), "+v"(a[(o) + 6]), "+v"(a[(o) + 7])                                       \
      : "v"(f))

// Lane sign of the presigned butterfly: (-1)^popcount(q) for logical lane q.
__device__ __forceinline__ bool lane_sign_odd(int q) { return (__builtin_popcount((uint32_t)q) & 1) != 0; }

// The butterfly with the cross-lane stages as one fused multiply-add per
// element, for inputs presigned per lane: lane q must hold (-1)^popcount(q)
// times its elements.  A cross-lane stage pairs lanes whose signs differ, so
// the lane with the stage bit clear computes own - partner (the pair's sum)
// and the other own + partner (the pair's difference, with the sign of its
// partner); every lane's sign thus flips once per set bit of q, and on return
// every lane holds the butterfly's exact values.  The sign of an exact zero is
// +0 wherever no -0 was among the inputs (no sum or difference of such values
// rounds to -0); with -0 inputs it may differ from the plain butterfly's.
template <int LPT>
__device__ __forceinline__ void fwht_tile_signed(float (&a)[kLaneElems], int q) {
#pragma unroll
  for (int h = 1; h < kLaneElems; h <<= 1) {
#pragma unroll
    for (int j = 0; j < kLaneElems; j++) {
      if (j & h) continue;
      float lo = a[j], hi = a[j + h];
      a[j] = lo + hi;
      a[j + h] = lo - hi;
    }
  }
#pragma unroll
  for (int m = 1; m < LPT; m <<= 1) {
    const float f = (q & m) ? 1.0f : -1.0f;
    if (m == 1) {                                            // partner lane ^ 1: quad_perm 1,0,3,2
#pragma unroll
      for (int o = 0; o < kLaneElems; o += 8) HQ_FMAC_DPP8("quad_perm:[1,0,3,2]", a, o, f);
    } else if (m == 2) {                                     // partner lane ^ 2: quad_perm 2,3,0,1
#pragma unroll
      for (int o = 0; o < kLaneElems; o += 8) HQ_FMAC_DPP8("quad_perm:[2,3,0,1]", a, o, f);
    } else {                                                 // partner q ^ 4 = lane p ^ 7: half-row mirror
#pragma unroll
      for (int o = 0; o < kLaneElems; o += 8) HQ_FMAC_DPP8("row_half_mirror", a, o, f);
    }
  }
}

// Signs of the butterfly's outputs when every input is a signed zero (bit i
// of z: element 32 q + i is -0): under IEEE rounding to nearest, lo + hi is
// -0 only for -0 + -0, and lo - hi only for -0 - (+0).  Same stage order and
// lane pairing as the butterfly.
template <int LPT>
__device__ __forceinline__ uint32_t zero_sign_butterfly(uint32_t z, int q) {
  constexpr uint32_t lo_mask[5] = {0x55555555u, 0x33333333u, 0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
#pragma unroll
  for (int st = 0; st < 5; st++) {
    const int h = 1 << st;
    const uint32_t lo = z & lo_mask[st], hi = (z >> h) & lo_mask[st];
    z = (lo & hi) | ((lo & ~hi) << h);
  }
  // (q through an opaque copy: its bit masks are formed on this rare path,
  // not hoisted into registers held across the caller's loop)
  uint32_t qo = (uint32_t)q;
  opaque(qo);
#pragma unroll
  for (int m = 1; m < LPT; m <<= 1) {
    const uint32_t p = lane_xor(z, partner_xor<LPT>(m));
    z = (qo & (uint32_t)m) ? (p & ~z) : (z & p);
  }
  return z;
}

// read 32 bits starting at bit `pos` of an LDS word array (needs one guard word)
__device__ __forceinline__ uint32_t lds_read32(const uint32_t* w, uint32_t pos) {
  uint32_t i = pos >> 5, s = pos & 31u;
  uint64_t v = ((uint64_t)w[i + 1] << 32) | w[i];
  return (uint32_t)(v >> s);
}

// OR an nbits-wide field (nbits <= 32) into an LDS bit array at bit `pos`
__device__ __forceinline__ void lds_or_bits(uint32_t* w, uint32_t pos, uint32_t field, uint32_t nbits) {
  uint32_t i = pos >> 5, s = pos & 31u;
  atomicOr(&w[i], field << s);
  if (s + nbits > 32u) atomicOr(&w[i + 1], field >> (32u - s));
}

}  // namespace hq
