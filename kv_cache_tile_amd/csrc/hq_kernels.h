// hq_kernels.h — the HyperQuant encode and decode kernels for gfx950.
//
// Method: "HyperQuant: A Rate-Distortion-Optimal Quantization Pipeline for
// Large Language and Diffusion Models", gist.science explainer, section
// "Methodology: The HyperQuant Pipeline", components 1-4 (RHT, lattice,
// bit-stripping + Rice, KV dither).
//
// Encode: one workgroup = one chunk of 64 tiles at a time (persistent
// workgroups take chunks from an atomic ticket).  Lane q of a tile holds its
// elements 32q..32q+31: load, sign flip, butterfly, scale, lattice search,
// symbols and the Rice parameter are all in registers; tile lengths are
// scanned within the chunk, the chunk's word offset in the stream comes from
// a decoupled look-back over earlier chunks' published sizes, and the bits
// are packed into LDS and written out with coalesced stores.
// Decode: one workgroup per unit of tiles of a chunk (grid-strided): the
// unit's bits are staged in LDS, each lane finds where its unary codes start
// (a popcount scan), parses its 32 codes with a reader specialised on the
// tile's Rice parameter, rebuilds the lattice points, runs the butterfly and
// stores.
//
// The templates are instantiated once per lattice, in hq_kern_<lattice>.hip
// (separate translation units, built in parallel); hq_lib.hip holds the host
// side and reaches the kernels through the tables declared at the end.
#pragma once
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "hq.h"
#include "hq_device.h"

namespace hq {

// Look-back words: (epoch << 34) | (flag << 32) | value.  The value travels
// inside the atomic word itself, so relaxed agent-scope atomics suffice: no
// other memory is published through them (release/acquire at agent scope
// would write back / invalidate the whole L2 of the XCD on every chunk).
constexpr uint32_t kFlagAgg = 1u, kFlagIncl = 2u;
constexpr uint32_t kEpochMask = 0x3FFFFFFFu;
constexpr int kLookJ = 4;                                   // look-back predecessors per lane per round

// One step of a group's unary codes, built last symbol first:
// G = ((G << 1) | 1) << (byte n of q) when `one`, else G << (byte n of q).
// The shift takes the byte straight from q (SDWA operand select); only its
// low 5 bits count, which is the whole quotient wherever G is kept.
template <int n>
__device__ __forceinline__ void unary_step(uint32_t& G, uint32_t q, bool one) {
  if (one) asm("v_lshl_or_b32 %0, %0, 1, 1" : "+v"(G));
  if constexpr (n == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
        : "+v"(G) : "v"(q));
  else if constexpr (n == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "+v"(G) : "v"(q));
  else if constexpr (n == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
        : "+v"(G) : "v"(q));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "+v"(G) : "v"(q));
}

// Rice fields of one lane (32 symbols, parameter K) into the staging bits of
// its tile starting at bit t0, from the byte-packed symbols P (symbol 4j + m
// is byte m of P[j]; every symbol of the wave is below 256).
//  - Remainder plane: the K-bit remainders of 4 symbols become one 4K-bit
//    field with byte dot products (weights 1, 2^K, 4^K, 8^K), the 8 fields
//    are assembled at static offsets in K registers, then written as K or K+1
//    words at the lane's bit alignment: plain stores for the words the lane
//    owns, OR for the two it may share with its neighbours.
//  - Unary plane: the codes (q zeros, then a one) of 8 symbols are gathered
//    in one register and ORed in at once; a group longer than 32 bits sets
//    its bits one by one.
template <int K, int N, uint32_t B>
__device__ __forceinline__ void pack_lane_bytes(uint32_t* stage, uint32_t t0, int q,
                                                const uint32_t (&P)[kLaneElems / 2], uint32_t lane_excl) {
  if constexpr (K > 0) {
    constexpr uint32_t rmask4 = 0x01010101u * ((1u << K) - 1u);
    uint32_t w[K + 1];
#pragma unroll
    for (int j = 0; j <= K; j++) w[j] = 0u;
#pragma unroll
    for (int j = 0; j < kLaneElems / 4; j++) {
      const uint32_t x = P[j] & rmask4;
      uint32_t f;
      if constexpr (3 * K <= 7) {
        f = __builtin_amdgcn_udot4(x, 1u | (1u << (K + 8)) | (1u << (2 * K + 16)) | (1u << (3 * K + 24)), 0u, false);
      } else {
        const uint32_t hi = __builtin_amdgcn_udot4(x, (1u << 16) | (1u << (K + 24)), 0u, false);
        f = __builtin_amdgcn_udot4(x, 1u | (1u << (K + 8)), hi << (2 * K), false);
      }
      const int o = j * 4 * K, wj = o >> 5, b = o & 31;
      w[wj] |= f << b;
      if (b + 4 * K > 32) w[wj + 1] |= f >> (32 - b);
    }
    // (q through an opaque copy: the lane's offset is formed here, not
    // hoisted out of the chunk loop as eight per-k constants held in
    // registers, which the 6-wave encode would spill)
    uint32_t qo = (uint32_t)q;
    opaque(qo);
    const uint32_t rpos = t0 + B + qo * (uint32_t)(kLaneElems * K);
    const uint32_t wi = rpos >> 5, sh = rpos & 31u;
    if (sh == 0u) {
      // starts and ends on word boundaries: every word is this lane's own
#pragma unroll
      for (int j = 0; j < K; j++) stage[wi + j] = w[j];
    } else {
      atomicOr(&stage[wi], w[0] << sh);
#pragma unroll
      for (int j = 1; j < K; j++) stage[wi + j] = (w[j] << sh) | (w[j - 1] >> (32u - sh));
      atomicOr(&stage[wi + K], w[K - 1] >> (32u - sh));
    }
  }
  uint32_t upos = t0 + B + (uint32_t)N * (uint32_t)K + lane_excl;
  constexpr uint32_t qmask4 = 0x01010101u * (0xFFu >> K);
#pragma unroll
  for (int g = 0; g < kLaneElems / 8; g++) {
    // quotients of the group's 8 symbols, 4 bytes per register; the group's
    // code bits tb = sum (q + 1) by byte sums (G is exact when tb <= 32)
    const uint32_t Qa = K > 0 ? (P[2 * g] >> K) & qmask4 : P[2 * g];
    const uint32_t Qb = K > 0 ? (P[2 * g + 1] >> K) & qmask4 : P[2 * g + 1];
    const uint32_t tb = __builtin_amdgcn_sad_u8(Qa, 0u, __builtin_amdgcn_sad_u8(Qb, 0u, 8u));
    // the group's codes, last symbol first: each step makes room for the
    // codes so far after a one (the next symbol's terminating one) and then
    // shifts by that symbol's quotient (its leading zeros)
    uint32_t G = 1u;
    unary_step<3>(G, Qb, false);
    unary_step<2>(G, Qb, true);
    unary_step<1>(G, Qb, true);
    unary_step<0>(G, Qb, true);
    unary_step<3>(G, Qa, true);
    unary_step<2>(G, Qa, true);
    unary_step<1>(G, Qa, true);
    unary_step<0>(G, Qa, true);
    if (tb <= 32u) {
      // the group's bits at upos: the low word, and the spill into the next
      // one, (G >> 1) >> (31 - sh), which is 0 for sh = 0 (shift counts
      // taken mod 32 as the hardware does)
      const uint32_t wi = upos >> 5;
      atomicOr(&stage[wi], G << (upos & 31u));
      atomicOr(&stage[wi + 1], (G >> 1) >> (~upos & 31u));
    } else {
      uint32_t pos = upos;
#pragma unroll 1
      for (int i = 0; i < 8; i++) {
        const int e = 8 * g + i;
        pos += __builtin_amdgcn_ubfe(P[e >> 2], 8 * (e & 3) + K, 8 - K);
        atomicOr(&stage[pos >> 5], 1u << (pos & 31u));
        pos += 1u;
      }
    }
    upos += tb;
  }
}

// The same fields from 16-bit symbol pairs (R[i / 2], half i % 2) with a
// runtime k, for waves with a symbol of 256 or more: remainders four at a
// time, one OR per unary code.
template <int N, uint32_t B>
__device__ __forceinline__ void pack_lane_pairs(uint32_t* stage, uint32_t t0, int q,
                                                const uint32_t (&R)[kLaneElems / 2], uint32_t k, uint32_t lane_excl) {
  if (k > 0) {
    const uint32_t rmask = (1u << k) - 1u;
    uint32_t rpos = t0 + B + (uint32_t)q * kLaneElems * k;
#pragma unroll
    for (int g = 0; g < kLaneElems / 4; g++) {
      const uint32_t lo = R[2 * g], hi = R[2 * g + 1];
      const uint32_t f = (lo & rmask) | (((lo >> 16) & rmask) << k) | ((hi & rmask) << (2u * k)) |
                         (((hi >> 16) & rmask) << (3u * k));
      lds_or_bits(stage, rpos, f, 4u * k);
      rpos += 4u * k;
    }
  }
  uint32_t upos = t0 + B + (uint32_t)N * k + lane_excl;
#pragma unroll
  for (int i = 0; i < kLaneElems; i++) {
    upos += __builtin_amdgcn_ubfe(R[i >> 1], 16 * (i & 1), 16) >> k;
    atomicOr(&stage[upos >> 5], 1u << (upos & 31u));
    upos += 1u;
  }
}

// Group tickets.  Workspace (32-bit words): [0..1] the event word (low
// half: draws, high half: early exits), [2] the epoch, [64..128) and
// [128..192) two bit arrays of started workgroups (a call of epoch e uses
// array e & 1), then the look-back words.  Workgroup b's first group is
// group b, with no contended atomic at start-up: it only sets its bit in the
// started array (32 workgroups share a word).  After its first group a
// workgroup checks the array (loaded ahead, during its group's last chunk):
// if every workgroup of the grid has started, it draws the following groups
// from the counter (draw v is group grid + v); if not, it leaves (an early
// exit), so that the workgroups still waiting for room can start.  Either
// way every group is held by a workgroup that is running, and a look-back
// waits only for groups numbered below its own: the encode progresses
// whatever part of the grid is resident, and next to any other kernel.
// Each workgroup ends with exactly one terminal event, a failing draw or an
// early exit, so the event whose result makes (exits + failing draws) equal
// to the grid is the last use of the workspace in this call: its holder
// resets the event word, clears the other started array for the next call
// and moves the epoch on.  Returns the group, or 0xFFFFFFFF when the
// workgroup is done.
constexpr uint32_t kStartedWords = 64;                      // bits for up to 2048 workgroups
constexpr uint32_t kStartedBase = 64, kLookBase = 192;      // word offsets in the workspace
constexpr uint32_t kLengthWord = 4;                          // (words 4, 5) the rate search's length count
__device__ __forceinline__ uint32_t take_ticket(uint32_t* ws, uint64_t CG, uint32_t epoch, bool all_started) {
  const uint32_t grid = gridDim.x;
  const uint64_t dyn = CG - grid;                            // groups handed out by draws
  const uint64_t add = all_started ? 1ull : (1ull << 32);
  uint64_t* evw = reinterpret_cast<uint64_t*>(ws);
  const uint64_t post = __hip_atomic_fetch_add(evw, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
  const uint64_t draws = (uint32_t)post, exits = post >> 32;
  if (exits + (draws > dyn ? draws - dyn : 0ull) == grid) {
    __hip_atomic_store(evw, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t* other = ws + kStartedBase + ((epoch + 1u) & 1u) * kStartedWords;
    for (uint32_t i = 0; i < kStartedWords; i++) __hip_atomic_store(&other[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t next = (epoch + 1u) & kEpochMask;
    asm volatile("" : "+s"(next));                          // (formed here, not held across the loop)
    __hip_atomic_store(&ws[2], next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return (all_started && draws - 1 < dyn) ? grid + (uint32_t)(draws - 1) : 0xFFFFFFFFu;
}

// Sign diagonal (Methodology 1): bit i of lane q's mask is the sign of tile
// element 32 q + i.  Threads 0..N-1 hash one element each, a ballot gathers
// 64 bits per wave into LDS (the workgroup has at least N threads).
template <int N>
__device__ __forceinline__ uint32_t sign_mask(uint32_t* smask, uint32_t key_sign, int tid, int q) {
  const uint32_t bit = tid < N ? (pcg_hash(key_sign + (uint32_t)tid) >> 31) : 0u;
  const uint64_t bal = __ballot(bit);
  if (tid < N && (tid & 63) == 0) {
    smask[tid >> 5] = (uint32_t)bal;
    if (N > 32) smask[(tid >> 5) + 1] = (uint32_t)(bal >> 32);
  }
  __syncthreads();
  return smask[q];
}

// The encoder's work on one tile up to its length, shared by the encoder and
// the length pass: load and sign diagonal, butterfly, step, nearest lattice
// points, symbols and the Rice parameter.  The lane's symbols come back in R
// (bytes, four a register, when `bytes`; else 16-bit pairs), its blocks'
// coset bits in cb, the tile's bf16 step bits in sbits (nonfinite: a
// non-finite tile, coded as zero), the Rice parameter in k, the tile's
// Rice-coded length without its coset bits in best_c, and this lane's sum of
// quotients in lane_sum.  k_prev carries the lane's previous Rice parameter.
template <int LAT, int N, bool DITHER, bool BF16>
__device__ __forceinline__ void encode_tile(const void* __restrict__ x, const uint4 (&pre)[4], const uint32_t* emask,
                                            uint32_t sgn, uint64_t T, uint64_t t, bool active, int q, float c,
                                            float inv_sqrtn, float inv_n, uint32_t key_dither, A2Consts a2,
                                            uint32_t& k_prev, uint32_t (&R)[kLaneElems / 2], uint32_t& cb,
                                            uint32_t& sbits, bool& nonfinite, bool& bytes, uint32_t& k,
                                            uint32_t& best_c, uint32_t& lane_sum) {
  constexpr int LPT = N / kLaneElems;
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;
  constexpr bool bf16 = BF16;
  // ---- load + sign diagonal (bf16 -> fp32 is exact; the sign bits are
  // flipped on the packed pairs) ----
  float a[kLaneElems];
  uint32_t sg = sgn;
  opaque(sg);
  // (an inactive tile works on the last tile's data and stores nothing)
  if (bf16) {
    const uint4* em = reinterpret_cast<const uint4*>(emask + 16 * q);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const uint4 w = pre[v], m = em[v];
      uint32_t ww[4] = {w.x, w.y, w.z, w.w}, mm[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
      for (int h = 0; h < 4; h++) {
        uint32_t pw = ww[h] ^ mm[h];
        opaque(pw);                                       // one xor per pair, then the two halves
        a[v * 8 + 2 * h] = as_f(pw << 16);
        a[v * 8 + 2 * h + 1] = as_f(pw & 0xFFFF0000u);
      }
    }
  } else {
    const uint64_t base = (active ? t : T - 1) * N + (uint64_t)q * kLaneElems;
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + base);
#pragma unroll
    for (int v = 0; v < 8; v++) {
      float4 w = p[v];
      a[v * 4] = w.x; a[v * 4 + 1] = w.y; a[v * 4 + 2] = w.z; a[v * 4 + 3] = w.w;
    }
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) a[i] = as_f(as_u(a[i]) ^ ((sg << (31 - i)) & 0x80000000u));
  }

  // ---- RHT: the butterfly (exact values in every lane), then y = z fl(1/sqrt(n)).
  // When 1/sqrt(n) is a power of two and the input is bf16 the scale is
  // exact: every butterfly value z is a multiple of 2^-133 (the finest bf16
  // unit; sums round to coarser multiples), so z / sqrt(n) is representable
  // even below the normal range.  Then the lane keeps z and the scale is
  // folded into the quantiser's factor (ydom false). ----
  fwht_tile_signed<LPT>(a, q);
  constexpr bool ydom = !kPow2Scale<N> || !bf16;
  if (ydom) {
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) a[i] = a[i] * inv_sqrtn;
  }

  // ---- tile energy and step = bf16(sqrt(ss / n) * c), ss the pinned
  // pairwise sum of y^2.  An estimate from fused multiply-add chains decides
  // the step unless it lies within 64 units in the last place of a bf16
  // rounding tie: the pinned sum and the estimate are each within 9 and 13
  // roundings of the exact sum of squares, so their two values of
  // sqrt(ss / n) * c (the estimate's square root by the hardware
  // instruction, within 1 ulp) differ by less than 16 units in the last
  // place.  A wave
  // with such a tile, or with an estimate outside [2^-90, 2^100] (where
  // subnormal terms, overflow, a flushed or an infinite step could enter),
  // computes the pinned sum (steps below 2^-124 are stored as 0). ----
  float e4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kLaneElems; i++) e4[i & 3] = __builtin_fmaf(a[i], a[i], e4[i & 3]);
  float est = (e4[0] + e4[1]) + (e4[2] + e4[3]);
#pragma unroll
  for (int m = 1; m < LPT; m <<= 1) est = est + lane_xor(est, partner_xor<LPT>(m));
  if (!ydom) est = est * inv_n;                            // sum of z^2 / n (exact power-of-two scale)
  const float r_est = __builtin_amdgcn_sqrtf(est * inv_n) * c;   // v_sqrt_f32: within 1 ulp
  const bool near_tie = ((as_u(r_est) & 0xFFFFu) - 0x7FC0u) <= 0x80u;
  const bool in_range = est >= 0x1p-90f && est <= 0x1p100f && r_est >= 0x1p-100f && r_est <= 0x1p100f;
  nonfinite = false;
  if (wave_any(near_tie || !in_range)) {
    asm volatile("");                                     // (rare: stays a branch)
    // the pinned tree as a running stack of partial sums: part[l] holds
    // the sum of the last complete block of 2^l squares
    float part[6];
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) {
      const float y = ydom ? a[i] : a[i] * inv_sqrtn;
      float v = y * y;
      int l = 0;
#pragma unroll
      for (; (i >> l) & 1; l++) v = part[l] + v;
      part[l] = v;
    }
    float ss = part[5];
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) ss = ss + lane_xor(ss, partner_xor<LPT>(m));
    nonfinite = (as_u(ss) & 0x7F800000u) == 0x7F800000u;
    sbits = 0;
    if (!nonfinite) {
      const float rms = sqrtf(ss * inv_n);
      const float r = rms * c;
      sbits = bf16_rne_bits(r);
      if ((sbits & 0x7F80u) == 0x7F80u) { nonfinite = true; sbits = 0; }
      else if ((sbits & 0x7F80u) < 0x0180u) sbits = 0;    // below 2^-124: stored as 0
    }
  } else {
    sbits = bf16_rne_bits(r_est);
  }
  // fl(1 / s) from the hardware reciprocal r0 (within 1 ulp) and one
  // correction: e = 1 - s r0 is exact (s has 8 significant bits), r0 + r0 e
  // differs from 1 / s by e^2 / s (below 2^-22 ulp), and 1 / s = 2^-j / M
  // (s = M 2^j, M < 256 an integer) lies at least 2^-9 ulp from every
  // rounding midpoint, so the fused multiply-add rounds to fl(1 / s).  s is
  // in [2^-124, 2^61 c]: r0 and 1 / s are normal.
  const float s = as_f(sbits << 16);
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  const float inv = sbits == 0u ? 0.0f : __builtin_fmaf(e, r0, r0);
  // t = y / s; with z kept, z * (inv / sqrt(n)) is the same product: both
  // scalings are exact (a finite tile energy bounds the step by
  // sqrt(FLT_MAX / n) * c < 2^61 c, far below 2^122 for the table's rate
  // constants, so inv / sqrt(n) is a normal number)
  const float qf = ydom ? inv : inv * inv_sqrtn;
#pragma unroll
  for (int i = 0; i < kLaneElems; i++) a[i] = a[i] * qf;
  if (wave_any(nonfinite)) {                                 // rare: a non-finite tile is coded as zero
    asm volatile("");                                     // (stays a branch, not 32 selects)
    if (nonfinite) {
#pragma unroll
      for (int i = 0; i < kLaneElems; i++) a[i] = 0.0f;
    }
  }


  // ---- nearest lattice point, strip, zigzag: symbols as 16-bit pairs
  // (every symbol is below 2^12: |t| <= sqrt(n) / c' for the table's c) ----
  uint32_t S2[kLaneElems / 2];
  cb = 0;
#pragma unroll
  for (int i = 0; i < kLaneElems / 2; i++) S2[i] = 0u;
#pragma unroll
  for (int b = 0; b < BPL; b++) {
    uint32_t p;
    uint32_t u[D];
    if constexpr (DITHER) {
      // KV: add the dither (Methodology 4), block by block
      float du[D];
      dither_block<LAT>(key_dither, (uint32_t)(t * N) + (uint32_t)(q * kLaneElems + b * D), du, a2);
#pragma unroll
      for (int i = 0; i < D; i++) a[b * D + i] = a[b * D + i] + du[i];
    }
    if constexpr (LAT == 8) {
      if (b > 0) {
        // one 8-block at a time: its inputs are released together with the
        // previous block's symbols (keeps four blocks' temporaries from
        // being live at once)
        asm volatile("" : "+v"(S2[4 * b - 4]), "+v"(S2[4 * b - 3]), "+v"(S2[4 * b - 2]), "+v"(S2[4 * b - 1]),
                          "+v"(a[8 * b + 0]), "+v"(a[8 * b + 1]), "+v"(a[8 * b + 2]), "+v"(a[8 * b + 3]),
                          "+v"(a[8 * b + 4]), "+v"(a[8 * b + 5]), "+v"(a[8 * b + 6]), "+v"(a[8 * b + 7]));
      }
      nearest_e8_symbols(&a[b * D], u, p);
    } else {
      int32_t d[D];
      nearest<LAT>(&a[b * D], d, p, a2);
      block_symbols<LAT>(d, u);
    }
#pragma unroll
    for (int i = 0; i < D; i++) {
      const int e = b * D + i;
      S2[e >> 1] |= u[i] << (16 * (e & 1));
    }
    cb |= p << b;
  }

  // ---- Rice parameter: smallest k in 0..7 minimising the tile's length ----
  // cost(k) = S(k) + n (1 + k) with S(k) = sum of sym >> k is convex in k
  // (S(k) - S(k+1) = sum ceil((sym >> k) / 2) does not grow with k), so the
  // smallest minimiser is the first k with S(k) - S(k+1) <= n (7 if none).
  // Three sums around the tile's previous k settle it when k has not moved;
  // otherwise the wave computes all eight.  When every symbol of the wave
  // fits a byte, four symbols share a register and one shift, one mask and
  // one byte-sum (v_sad_u8) add four terms.
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < kLaneElems / 2; i++) mx |= S2[i];
  bytes = wave_all((mx & 0xFF00FF00u) == 0u);
  // R: the byte-packed symbols (R[j], byte m = symbol 4j + m) when every
  // symbol of the wave fits a byte, else the 16-bit pairs
  if (bytes) {
#pragma unroll
    for (int j = 0; j < kLaneElems / 4; j++) R[j] = __builtin_amdgcn_perm(S2[2 * j + 1], S2[2 * j], 0x06040200u);
#pragma unroll
    for (int j = kLaneElems / 4; j < kLaneElems / 2; j++) R[j] = S2[j];   // (unread: no copies)
  } else {
#pragma unroll
    for (int j = 0; j < kLaneElems / 2; j++) R[j] = S2[j];
  }
  k = 0;
  best_c = 0;
  lane_sum = 0;
  bool settled = false;
  if (bytes && k_prev < 8u) {
    const uint32_t kb = k_prev == 0u ? 0u : (k_prev >= 6u ? 5u : k_prev - 1u);
    uint32_t L[3], Tt[3];
#pragma unroll
    for (int jj = 0; jj < 3; jj++) {
      // sum of (sym >> k) = (sum of sym with its low k bits cleared) >> k
      const uint32_t kk = kb + (uint32_t)jj;
      const uint32_t bmask = 0x01010100u - (0x01010101u << kk);   // bytes 256 - 2^kk
      uint32_t acc = 0;
#pragma unroll
      for (int j = 0; j < kLaneElems / 4; j++) acc = __builtin_amdgcn_sad_u8(R[j] & bmask, 0u, acc);
      acc >>= kk;
      L[jj] = acc;
      uint32_t tot = acc;
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) tot += lane_xor(tot, partner_xor<LPT>(m));
      Tt[jj] = tot;
    }
    const bool drop0 = Tt[0] - Tt[1] > (uint32_t)N, drop1 = Tt[1] - Tt[2] > (uint32_t)N;
    int pick = -1;
    if (kb == 0u && !drop0) pick = 0;
    else if (drop0 && !drop1) pick = 1;
    else if (kb == 5u && drop0 && drop1) pick = 2;
    if (pick >= 0) {
      settled = true;
      k = kb + (uint32_t)pick;
      const uint32_t tot = pick == 0 ? Tt[0] : (pick == 1 ? Tt[1] : Tt[2]);
      lane_sum = pick == 0 ? L[0] : (pick == 1 ? L[1] : L[2]);
      best_c = tot + (uint32_t)N * (1u + k);
    }
  }
  if (wave_any(!settled)) {
    // rare: all eight sums, one k per (rolled) iteration, running minimum
    uint32_t bk = 0, bc = 0xFFFFFFFFu, bsum = 0;
#pragma unroll 1
    for (uint32_t kk = 0; kk < 8u; kk++) {
      uint32_t acc = 0;
      if (bytes) {
        const uint32_t bmask = 0x01010100u - (0x01010101u << kk);   // bytes 256 - 2^kk
#pragma unroll
        for (int j = 0; j < kLaneElems / 4; j++) acc = __builtin_amdgcn_sad_u8(R[j] & bmask, 0u, acc);
        acc >>= kk;
      } else {
        // 16-bit halves: each half's sum stays below 2^16 (16 symbols < 2^12)
        const uint32_t hmask = 0x00010001u * (0xFFFFu >> kk);
        uint32_t a2acc = 0;
#pragma unroll
        for (int j = 0; j < kLaneElems / 2; j++) a2acc += (R[j] >> kk) & hmask;
        acc = (a2acc & 0xFFFFu) + (a2acc >> 16);
      }
      uint32_t tot = acc;
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) tot += lane_xor(tot, partner_xor<LPT>(m));
      const uint32_t cost = tot + (uint32_t)N * (1u + kk);
      if (cost < bc) { bc = cost; bk = kk; bsum = acc; }
    }
    if (!settled) {
      k = bk;
      best_c = bc;
      lane_sum = bsum;
    }
  }
  k_prev = k;
}

// --------------------------------------------------------------------------
// Encode kernel
// --------------------------------------------------------------------------
// Occupancy: the E8 encode at n = 128 and 256 runs 6 waves per SIMD (three
// 512-thread or six 256-thread workgroups a CU, at most 80 VGPRs): the
// chunk's input is then loaded at the top of its own iteration (the other
// workgroups hide the latency) rather than prefetched into 16 registers
// during the previous chunk.  Measured on one box, bit-identical streams:
// 3.5% fewer cycles for a 4096 x 16384 layer at n = 256, 6.5% less time for
// 11008 x 4096 at n = 128.  Z and D4 at n = 128 measured no faster (D4 4%
// slower), A2 would spill at 80 VGPRs, and the dither adds registers: they,
// and n = 64, keep 4 waves and the prefetch.
template <int LAT, int N, bool DITHER>
constexpr bool kEncodePrefetch = !(LAT == 8 && N >= 128 && !DITHER);

template <int LAT, int N, bool DITHER, bool BF16>
__global__ void __launch_bounds__(kChunkTiles * (N / kLaneElems)) __attribute__((amdgpu_waves_per_eu(kEncodePrefetch<LAT, N, DITHER> ? 4 : 6)))
encode_kernel(const void* __restrict__ x, uint32_t /* input is bf16: BF16 */, uint64_t T, uint64_t C, float c, float inv_sqrtn, float inv_n,
              uint32_t key_sign, uint32_t key_dither, A2Consts a2,
              uint32_t* __restrict__ payload, uint64_t cap_words,
              uint16_t* __restrict__ step_out, uint16_t* __restrict__ meta_out,
              uint32_t* __restrict__ chunk_off, uint32_t* __restrict__ status,
              uint32_t* __restrict__ ws, uint32_t stage_words, uint32_t grp_words, uint32_t group_chunks,
              uint32_t spin_limit) {
  constexpr int LPT = N / kLaneElems;                       // lanes per tile
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;                       // lattice blocks per lane
  constexpr uint32_t CB_LANE = LatticeTraits<LAT>::coset * BPL;   // coset bits per lane
  constexpr uint32_t B = CB_LANE * LPT;                     // coset bits per tile
  constexpr bool bf16 = BF16;                               // input dtype (else fp32)

  extern __shared__ uint32_t smem[];
  uint32_t* stage = smem;                                   // [stage_words]: two group areas
  uint32_t* tile_len = smem + stage_words;                  // [64]
  uint32_t* tile_off = tile_len + kChunkTiles;              // [64]
  uint32_t* misc = tile_off + kChunkTiles;                  // [4]
  uint32_t* smask = misc + 4;                               // [N / 32] sign diagonal bits
  uint32_t* goff = smask + 8;                               // [2][kMaxGroupChunks] chunk word offsets per half
  uint32_t* started_copy = goff + 2 * kMaxGroupChunks;      // [kStartedWords] the started array, read ahead
  uint32_t* emask = started_copy + kStartedWords;           // [LPT][16] per-pair sign masks of each lane

  const int tid = threadIdx.x;
  const int tau = tid / LPT;
  const int p_lane = tid % LPT;                            // physical lane in the tile
  const int q = tile_lane<LPT>(p_lane);                     // logical lane
  uint64_t* look = reinterpret_cast<uint64_t*>(ws + kLookBase);   // one word per group

  // Tickets number groups of group_chunks consecutive chunks (take_ticket).
  // Chunk and group numbers are 32-bit (the plan admits fewer than 2^32
  // scalars, so fewer than 2^20 chunks): scalar registers are scarce here.
  const uint32_t C32 = (uint32_t)C;
  const uint32_t CG = (C32 + group_chunks - 1) / group_chunks;
  if (tid == 0)
    misc[2] = __hip_atomic_load(&ws[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kEpochMask;

  // sign diagonal entries of this lane's 32 positions (Methodology 1), with
  // the butterfly's lane sign folded in (inputs presigned per lane); the
  // barrier inside also publishes the epoch
  const uint32_t sgn = sign_mask<N>(smask, key_sign, tid, q) ^ (lane_sign_odd(q) ? 0xFFFFFFFFu : 0u);
  // the packed-pair form of every logical lane's mask, read back from LDS
  // where the pairs are loaded (one xor a pair)
  if (tid < 16 * LPT) {
    const int qq = tid >> 4;
    uint32_t W[2];
    pair_sign_words(smask[qq] ^ (lane_sign_odd(qq) ? 0xFFFFFFFFu : 0u), W);
    emask[tid] = pair_sign_mask(W, tid & 15);
  }
  uint32_t k_prev = 0xFFu;                                  // Rice parameter of this lane's previous tile
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(misc[2]);   // (uniform: a scalar)
  uint32_t* started = ws + kStartedBase + (epoch & 1u) * kStartedWords;
  // with no group left to draw (a grid as large as the group count) every
  // draw fails: no started bits are set or read
  bool checked = CG == gridDim.x, all_started = false;      // wave 1: the started array was read, and its verdict
  const uint32_t started_copy_lds = __builtin_amdgcn_readfirstlane(lds_addr(started_copy));
  for (uint32_t i = tid; i < stage_words; i += blockDim.x) stage[i] = 0u;
  __syncthreads();
  uint32_t grp = blockIdx.x;
  uint32_t chunk = grp * group_chunks;
  uint32_t gi = 0, gw = 0;                                  // chunk of the group, group words staged so far
  bool gfits = true;

  // bf16 input of the chunk about to be processed, loaded one phase ahead
  // (the next chunk of a group during this one's scan and packing; a new
  // group's first chunk as soon as its ticket is known), or at the top of
  // its own iteration where kEncodePrefetch is false.
  // A tile past the end (ragged last chunk, or no chunk left) loads the last
  // tile instead: its results are never stored, and the registers need no
  // clearing.
  uint4 pre[4];
  auto prefetch = [&](uint64_t ch) {
    if (bf16) {
      uint64_t tt = ch * kChunkTiles + (uint64_t)tau;
      tt = tt < T ? tt : T - 1;
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + tt * N +
                                                      (uint64_t)q * kLaneElems);
#pragma unroll
      for (int v = 0; v < 4; v++) pre[v] = p[v];
    }
  };
  if (kEncodePrefetch<LAT, N, DITHER>) prefetch(chunk);
  // this workgroup has started (after the loads above, so that waiting for
  // them does not wait for this contended atomic)
  if (tid == 64 && !checked)
    (void)__hip_atomic_fetch_or(&started[blockIdx.x >> 5], 1u << (blockIdx.x & 31u), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);

  // The staging area holds two group areas of grp_words (a group's worst
  // case), at 0 and at stage_words - grp_words; consecutive groups of a
  // workgroup alternate between them.  A finished group stays in its area
  // while the next group computes and packs into the other, and is placed at
  // the start of that group's last chunk: wave 0 runs its look-back (its
  // predecessors have published long since) while the other waves compute,
  // and its words are copied out after that chunk's compute barrier.  When
  // the two areas overlap (less LDS than two worst cases) and the words
  // actually written would meet, the finished group is placed at once.
  const uint32_t base1 = stage_words - grp_words;          // the second area's first word
  uint32_t h = 0;                                           // the current group's area
  bool pend = false, pgfits = true;
  uint32_t pgrp = 0, pchunk = 0;
  uint32_t pgtotal = 0, pgi = 0, ph = 0;

  // wave 0: decoupled look-back over groups.  A round loads kLookJ
  // predecessors per lane at once (distance d = 64 jj + lane, all loads in
  // flight together), waits until each has published, and sums the values up
  // to the nearest inclusive prefix.  Then the group's inclusive prefix, its
  // chunks' offsets and its status; misc[3] = its first word.  The wait is
  // bounded (spin_limit polls): past it the group is published with the
  // prefix found so far and HQ_FLAG_STALL, so that every later group, and
  // the kernel, still end.
  auto place = [&]() {
    uint32_t excl = 0;
    bool stalled = false;
    if (pgrp > 0) {
      int64_t base = (int64_t)pgrp - 1;
      uint32_t polls = 0;
      uint32_t lt = (uint32_t)tid;
      opaque(lt);                                           // (lane offsets formed here, not held across the loop)
      for (;;) {
        uint64_t v[kLookJ];
#pragma unroll
        for (int jj = 0; jj < kLookJ; jj++) {
          const int64_t j = base - (int64_t)(64 * jj + lt);
          v[jj] = j < 0 ? ((uint64_t)((epoch << 2) | kFlagIncl) << 32)   // before group 0: prefix 0
                        : __hip_atomic_load(&look[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        for (;;) {
          bool done = true;
#pragma unroll
          for (int jj = 0; jj < kLookJ; jj++) {
            const uint32_t hi = (uint32_t)(v[jj] >> 32);
            if ((hi >> 2) != epoch || (hi & 3u) == 0) {
              const int64_t j = base - (int64_t)(64 * jj + lt);
              v[jj] = __hip_atomic_load(&look[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              const uint32_t h2 = (uint32_t)(v[jj] >> 32);
              done = done & ((h2 >> 2) == epoch) & ((h2 & 3u) != 0);
            }
          }
          if (wave_all(done)) break;
          if (++polls > spin_limit) { stalled = true; break; }
          __builtin_amdgcn_s_sleep(1);
        }
        if (stalled) break;
        uint32_t first = 0xFFFFFFFFu;                        // distance of the nearest inclusive prefix
#pragma unroll
        for (int jj = kLookJ - 1; jj >= 0; jj--) {
          const uint64_t m = __ballot(((uint32_t)(v[jj] >> 32) & 3u) == kFlagIncl);
          if (m) first = 64u * (uint32_t)jj + (uint32_t)__builtin_ctzll(m);
        }
        uint32_t part = 0;
#pragma unroll
        for (int jj = 0; jj < kLookJ; jj++)
          part += (64u * (uint32_t)jj + (uint32_t)tid <= first) ? (uint32_t)v[jj] : 0u;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m);
        excl += part;
        if (first != 0xFFFFFFFFu) break;
        base -= 64 * kLookJ;
      }
    }
    if (tid == 0) {
      if (pgrp > 0) {
        uint64_t tag = (uint64_t)((epoch << 2) | kFlagIncl);
        __hip_atomic_store(&look[pgrp], (tag << 32) | (uint64_t)(excl + pgtotal), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      misc[3] = excl;
      const uint32_t c0 = pgrp * group_chunks;
      for (uint32_t i = 0; i <= pgi; i++) chunk_off[c0 + i] = excl + goff[ph * kMaxGroupChunks + i];
      if (pchunk == C32 - 1) chunk_off[C32] = excl + pgtotal;
      if (!pgfits || (uint64_t)excl + pgtotal > cap_words) atomicOr(status, HQ_FLAG_NOSPACE);
      if (stalled) atomicOr(status, HQ_FLAG_STALL);
    }
  };
  // all threads, after place() and a barrier: the placed group's words out
  // (16-byte stores at 16-byte payload offsets; the up to 3 words before the
  // first and after the last one by one), then its area cleared (the group
  // areas are 16-byte aligned, whole vectors)
  auto copy_out = [&]() {
    const uint32_t excl = misc[3];
    const bool store = pgfits && (uint64_t)excl + pgtotal <= cap_words;
    const uint32_t zw = pgtotal + 2 < grp_words ? pgtotal + 2 : grp_words;
    uint32_t* src = stage + (ph ? base1 : 0u);
    if (store) {
      const uint32_t e = excl + pgtotal;
      const uint32_t a0 = (excl + 3u) & ~3u, a1 = e & ~3u;
      const uint32_t nv = a1 > a0 ? (a1 - a0) >> 2 : 0u;
      for (uint32_t v = tid; v < nv; v += blockDim.x) {
        const uint32_t s0 = a0 - excl + 4u * v;
        *reinterpret_cast<uint4*>(payload + a0 + 4u * v) = make_uint4(src[s0], src[s0 + 1], src[s0 + 2], src[s0 + 3]);
      }
      if (tid < 8) {
        const uint32_t lo = tid < 4 ? excl : (a1 > a0 ? a1 : a0);
        const uint32_t hi = tid < 4 ? (a0 < e ? a0 : e) : e;
        const uint32_t i = lo + (uint32_t)(tid & 3);
        if (i < hi) payload[i] = src[i - excl];
      }
    }
    __syncthreads();                                        // (every read of the area is done)
    uint4* src4 = reinterpret_cast<uint4*>(src);
    for (uint32_t v = tid; v < (zw + 3u) >> 2; v += blockDim.x) src4[v] = make_uint4(0u, 0u, 0u, 0u);
  };

  // this workgroup's expected share of chunks; priority falls by quarters of it
  const uint32_t share = (uint32_t)((C + gridDim.x - 1) / gridDim.x);
  uint32_t done = 0;
  for (;;) {
    if (grp >= CG) break;
    const uint32_t quarters = 4u * done++ / share;
    wave_priority(quarters >= 3u ? 0u : 3u - quarters);
    const bool last = (gi + 1 == group_chunks) || (chunk + 1 >= C32);
    if (pend && last && tid < 64) place();
    // before the first draw: wave 1 loads the started array into LDS now
    // (no register held through the compute), to read it after this chunk's
    // compute
    if (last && !checked && tid >= 64 && tid < 128) {
      uint32_t so = 4u * (uint32_t)(tid - 64);
      opaque(so);                                           // (formed here, not held across the loop)
      lds_load_u32_coherent(started, so, started_copy_lds);
    }

    const uint64_t t = (uint64_t)chunk * kChunkTiles + (uint64_t)tau;
    const bool active = t < T;
    if (!kEncodePrefetch<LAT, N, DITHER>) prefetch(chunk);

    uint32_t R[kLaneElems / 2];
    uint32_t cb, sbits, k, best_c, lane_sum;
    bool nonfinite, bytes;
    encode_tile<LAT, N, DITHER, BF16>(x, pre, emask, sgn, T, t, active, q, c, inv_sqrtn, inv_n, key_dither, a2,
                                      k_prev, R, cb, sbits, nonfinite, bytes, k, best_c, lane_sum);
    // this lane's unary quotients: sum (q_i + 1) bits; exclusive prefix over the tile's lanes
    const uint32_t lane_unary = lane_sum + (uint32_t)kLaneElems;
    uint32_t lane_excl = 0, span = lane_unary;              // exclusive prefix in logical lane order
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) {
      const uint32_t other = lane_xor(span, partner_xor<LPT>(m));
      if (q & m) lane_excl += other;
      span += other;
    }
    const uint32_t tlen = B + best_c;
    if (q == 0) {
      uint32_t to = (uint32_t)tau;
      opaque(to);                                           // (formed here, not held across the loop)
      tile_len[to] = active ? tlen : 0u;
      if (active) {
        step_out[t] = (uint16_t)sbits;
        meta_out[t] = (uint16_t)((tlen << 3) | k);
        if (nonfinite) atomicOr(status, HQ_FLAG_NONFINITE);
      }
    }
    __syncthreads();
    if (pend && last) {
      copy_out();
      pend = false;
    }

    // the group's next chunk: load its input during this one's scan and packing
    if (kEncodePrefetch<LAT, N, DITHER> && !last) prefetch(chunk + 1);

    // ---- chunk scan: bit offset of every tile inside the chunk; after the
    // group's last chunk, publish the group's size at once so later groups
    // can look back past it ----
    if (tid < kChunkTiles) {
      const uint32_t v = tile_len[tid], inc = wave_incl_scan(v);
      tile_off[tid] = inc - v;
      if (tid == kChunkTiles - 1) {
        misc[1] = inc;
        if (last) {
          const uint64_t tag = (uint64_t)((epoch << 2) | (grp == 0 ? kFlagIncl : kFlagAgg));
          __hip_atomic_store(&look[grp], (tag << 32) | (gw + ((inc + 31u) >> 5)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
    const uint32_t total_bits = misc[1];
    const uint32_t W = (total_bits + 31u) >> 5;
    const bool fits = gw + W + 2 <= grp_words;
    gfits = gfits && fits;
    if (tid == 0) goff[h * kMaxGroupChunks + gi] = gw;      // this chunk's word offset in the group
    // after the group's last chunk: the next ticket now (its reply arrives
    // during the packing)
    uint32_t next_ticket = 0;
    if (last && tid >= 64 && tid < 128) {
      // every workgroup of the grid has started (wave 1: lane i checks word i)
      if (!checked) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // (this wave's load of the started array)
        uint32_t i = (uint32_t)(tid - 64);
        opaque(i);                                          // (formed here, not held across the loop)
        const uint32_t g = gridDim.x;
        const uint32_t want = 32u * i >= g ? 0u : (32u * (i + 1u) <= g ? 0xFFFFFFFFu : (1u << (g & 31u)) - 1u);
        all_started = wave_all((started_copy[i] & want) == want);
        if (!all_started) {
          // the copy was taken at the top of this chunk, with one-chunk groups
          // a few microseconds after the launch, when some starts may not have
          // landed yet: read the array again before leaving
          const uint32_t v = __hip_atomic_load(&started[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          all_started = wave_all((v & want) == want);
        }
        checked = true;
      }
      if (tid == 64) next_ticket = take_ticket(ws, CG, epoch, all_started);
    }

    // the words about to be written would meet the finished group's: place it now
    if (pend && (h ? pgtotal + 2 > base1 : gw + W + 2 > base1)) {
      if (tid < 64) place();
      __syncthreads();
      copy_out();
      pend = false;
      __syncthreads();
    }

    // ---- pack: coset bits | remainder plane (k bits per symbol) | unary plane,
    // at the chunk's word offset in the group's area of the staging area
    // (zero: cleared at the start and after each copy) ----
    if (active && fits) {
      uint32_t* stage_h = stage + (h ? base1 : 0u);
      const uint32_t t0 = gw * 32u + tile_off[tau];
      if constexpr (CB_LANE > 0) lds_or_bits(stage_h, t0 + (uint32_t)q * CB_LANE, cb, CB_LANE);
      if (bytes) {
        switch (k) {
#define HQ_PACK_CASE(KK) \
          case KK: pack_lane_bytes<KK, N, B>(stage_h, t0, q, R, lane_excl); break;
          HQ_PACK_CASE(0) HQ_PACK_CASE(1) HQ_PACK_CASE(2) HQ_PACK_CASE(3)
          HQ_PACK_CASE(4) HQ_PACK_CASE(5) HQ_PACK_CASE(6)
          default: pack_lane_bytes<7, N, B>(stage_h, t0, q, R, lane_excl); break;
#undef HQ_PACK_CASE
        }
      } else {
        pack_lane_pairs<N, B>(stage_h, t0, q, R, k, lane_excl);
      }
    }
    if (last && tid == 64) misc[0] = next_ticket;
    __syncthreads();
    if (!last) {
      gw += W;
      gi++;
      chunk++;
      continue;
    }
    pend = true;
    pgrp = grp;
    pchunk = chunk;
    pgtotal = gw + W;                                       // the group's words
    pgi = gi;
    pgfits = gfits;
    ph = h;
    h ^= 1u;
    grp = misc[0];
    chunk = grp * group_chunks;
    if (kEncodePrefetch<LAT, N, DITHER>) prefetch(chunk);
    gi = 0;
    gw = 0;
    gfits = true;
  }
  if (pend) {                                               // the workgroup's last group
    if (tid < 64) place();
    __syncthreads();
    copy_out();
  }
}

// --------------------------------------------------------------------------
// Length pass: the payload size, in words, that the encoder would write at
// rate constant c (each chunk's tile lengths summed and rounded up to a
// whole word, over every chunk), with nothing packed, placed or stored.  The
// closed-loop rate search (Methodology 3) runs it as its trial.  Each
// workgroup takes chunks blockIdx.x, blockIdx.x + grid, ... and adds its
// total to *words once at the end; no workgroup waits for another.
// --------------------------------------------------------------------------
template <int LAT, int N, bool DITHER, bool BF16>
__global__ void __launch_bounds__(kChunkTiles * (N / kLaneElems)) __attribute__((amdgpu_waves_per_eu(4)))
length_kernel(const void* __restrict__ x, uint64_t T, uint64_t C, float c, float inv_sqrtn, float inv_n,
              uint32_t key_sign, uint32_t key_dither, A2Consts a2, unsigned long long* __restrict__ words) {
  constexpr int LPT = N / kLaneElems;
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr uint32_t B = LatticeTraits<LAT>::coset * (kLaneElems / D) * LPT;   // coset bits per tile
  __shared__ uint32_t smask[8];                             // [N / 32] sign diagonal bits
  __shared__ uint32_t emask[16 * LPT];                      // per-pair sign masks of each lane
  __shared__ uint32_t tile_len[2][kChunkTiles];             // alternate chunks' tile lengths

  const int tid = threadIdx.x;
  const int tau = tid / LPT;
  const int q = tile_lane<LPT>(tid % LPT);
  const uint32_t sgn = sign_mask<N>(smask, key_sign, tid, q) ^ (lane_sign_odd(q) ? 0xFFFFFFFFu : 0u);
  if (tid < 16 * LPT) {
    const int qq = tid >> 4;
    uint32_t W[2];
    pair_sign_words(smask[qq] ^ (lane_sign_odd(qq) ? 0xFFFFFFFFu : 0u), W);
    emask[tid] = pair_sign_mask(W, tid & 15);
  }
  __syncthreads();

  // the next chunk's bf16 input is loaded during this one's work; a tile
  // past the end loads the last tile (its length is not counted)
  uint4 pre[4];
  auto prefetch = [&](uint64_t ch) {
    if (BF16) {
      uint64_t tt = ch * kChunkTiles + (uint64_t)tau;
      tt = tt < T ? tt : T - 1;
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + tt * N +
                                                      (uint64_t)q * kLaneElems);
#pragma unroll
      for (int v = 0; v < 4; v++) pre[v] = p[v];
    }
  };
  uint32_t k_prev = 0xFFu;
  unsigned long long total = 0;                             // (lane 63 of wave 0) this workgroup's words
  uint32_t buf = 0;
  uint64_t chunk = blockIdx.x;
  prefetch(chunk);
  for (; chunk < C; chunk += gridDim.x) {
    const uint64_t t = chunk * kChunkTiles + (uint64_t)tau;
    const bool active = t < T;
    uint32_t R[kLaneElems / 2];
    uint32_t cb, sbits, k, best_c, lane_sum;
    bool nonfinite, bytes;
    encode_tile<LAT, N, DITHER, BF16>(x, pre, emask, sgn, T, t, active, q, c, inv_sqrtn, inv_n, key_dither, a2,
                                      k_prev, R, cb, sbits, nonfinite, bytes, k, best_c, lane_sum);
    if (chunk + gridDim.x < C) prefetch(chunk + gridDim.x);
    if (q == 0) tile_len[buf][tau] = active ? B + best_c : 0u;
    // one barrier a chunk: the buffer written next was last read before it
    __syncthreads();
    if (tid < kChunkTiles) {
      const uint32_t inc = wave_incl_scan(tile_len[buf][tid]);
      if (tid == kChunkTiles - 1) total += (inc + 31u) >> 5;
    }
    buf ^= 1u;
  }
  if (tid == kChunkTiles - 1 && total) atomicAdd(words, total);
}

// --------------------------------------------------------------------------
// Decode kernel
// --------------------------------------------------------------------------
// decode work unit: TPW tiles of a chunk (a half chunk at n = 256, so that
// workgroups stay at 256 threads and several fit on a CU)
template <int N>
struct DecodeGeom {
  static constexpr int LPT = N / kLaneElems;
  static constexpr int TPW = (256 / LPT) < kChunkTiles ? (256 / LPT) : kChunkTiles;
  static constexpr int SUB = kChunkTiles / TPW;
  static constexpr int THREADS = TPW * LPT;
};

// Rice parse of one lane's 32 codes for Rice parameter K, each block's
// integer code (d, p) handed to sink.block(b, d, p) as it is read, and
// sink.group_done(g) after the 8 codes of group g.  Remainders come from the
// lane's K-bit fields (static offsets), quotients from the unary window, 8
// codes per group; a group whose fast read saw a run of 31+ zeros (or ran out
// of window) is read again exactly.  Returns false if the codes are not a
// valid stream (a symbol above 16 bits, or a run past `end`); `upos` is left
// at the bit after the lane's last code.
template <int LAT, int K, class Sink>
__device__ __forceinline__ bool parse_codes(const uint32_t* stage, uint32_t rb, uint32_t u0, uint32_t end,
                                            uint32_t cbits, Sink& sink, uint32_t& upos) {
  constexpr int D = LatticeTraits<LAT>::dim;
  uint32_t seg[K + 1];
  seg[K] = 0u;
  if constexpr (K > 0) {
    const uint32_t base = rb >> 5, sh = rb & 31u;
    uint32_t raw[K + 1];
#pragma unroll
    for (int j = 0; j <= K; j++) raw[j] = stage[base + j];
#pragma unroll
    for (int j = 0; j < K; j++) seg[j] = __builtin_amdgcn_alignbit(raw[j + 1], raw[j], sh);
  }
  UnaryWindow uw;
  uw.init(stage, u0);
  bool ok = true;
#pragma unroll
  for (int g = 0; g < kLaneElems / 8; g++) {
    uw.refill();
    const uint32_t saved = uw.pos();                        // the group's first bit, for a re-read
    uint32_t z[8], zmax = 0;
    uw.take8(z, zmax);
    if (wave_any(zmax >= 31u)) {
      if (zmax >= 31u) {
        // rare: read the group again exactly (a rolled loop; codes shift in from the top)
        uw.init(stage, saved);
#pragma unroll 1
        for (int i = 0; i < 8; i++) {
          uint32_t qv = uw.next_exact(end);
          if (qv > (0xFFFFu >> K)) { ok = false; qv = 0u; }
#pragma unroll
          for (int j = 0; j < 7; j++) z[j] = z[j + 1];
          z[7] = qv;
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < 8 / D; bb++) {
      const int b = g * (8 / D) + bb;                       // block index in the lane
      int32_t d[D];
#pragma unroll
      for (int i = 0; i < D; i++) d[i] = code_coord<K>(seg, b * D + i, z[bb * D + i]);
      if constexpr (LAT == 4 || LAT == 8) {
        uint32_t par = 0;
        if constexpr (K >= 2) {
          par = block_low_parity<K, D>(seg, b);
        } else {
#pragma unroll
          for (int i = 0; i < D - 1; i++) par ^= (uint32_t)d[i];
        }
        d[D - 1] = (int32_t)(((uint32_t)d[D - 1] << 1) | (par & 1u));
      }
      sink.block(b, d, (cbits >> b) & 1u);
    }
    sink.group_done(g);
  }
  upos = uw.pos();
  return ok;
}

// The decoder's sink: a[e] = (lattice point - dither) * s, every zero +0 (a
// product with +0 added, one fused multiply-add; no nonzero product rounds
// to zero for the steps the caller passes).
template <int LAT, bool DITHER>
struct RebuildSink {
  static constexpr int D = LatticeTraits<LAT>::dim;
  float (&a)[kLaneElems];
  float s;
  uint32_t key_dither, g_lane;
  A2Consts a2;
  __device__ __forceinline__ void block(int b, const int32_t (&d)[D], uint32_t p) {
    if constexpr (LAT == 8 && !DITHER) {
      // E8 without dither: (d + p/2) * s as one fma, exact (13 and 8
      // significant bits) for normal products
      const float add = p ? 0.5f * s : 0.0f;
#pragma unroll
      for (int i = 0; i < D; i++) a[b * D + i] = __builtin_fmaf((float)d[i], s, add);
    } else {
      float pt[D];
      code_point<LAT>(d, p, pt, a2);
      if constexpr (DITHER) {
        float du[D];
        dither_block<LAT>(key_dither, g_lane + (uint32_t)(b * D), du, a2);
#pragma unroll
        for (int i = 0; i < D; i++) pt[i] = pt[i] - du[i];
      }
#pragma unroll
      for (int i = 0; i < D; i++) a[b * D + i] = __builtin_fmaf(pt[i], s, 0.0f);
    }
  }
  // the group's values are final here: keeps the compiler from holding all
  // 32 quotients and rebuilding every block at the end (register pressure)
  __device__ __forceinline__ void group_done(int g) {
    asm volatile("" : "+v"(a[8 * g + 0]), "+v"(a[8 * g + 1]), "+v"(a[8 * g + 2]), "+v"(a[8 * g + 3]),
                      "+v"(a[8 * g + 4]), "+v"(a[8 * g + 5]), "+v"(a[8 * g + 6]), "+v"(a[8 * g + 7]));
  }
};

template <int LAT, bool DITHER, int K>
__device__ __forceinline__ bool parse_lane(const uint32_t* stage, uint32_t rb, uint32_t u0, uint32_t end,
                                           uint32_t cbits, float s, uint32_t key_dither, uint32_t g_lane,
                                           A2Consts a2, float (&a)[kLaneElems], uint32_t& upos) {
  RebuildSink<LAT, DITHER> sink{a, s, key_dither, g_lane, a2};
  return parse_codes<LAT, K>(stage, rb, u0, end, cbits, sink, upos);
}

// The int8 product's sink (Z, D4, E8 without dither): the integer codes 2P
// = 2 d + p (p the E8 coset bit; 0 for Z and D4), saturated to [-127, 127]
// and packed four to a word (w[j], byte m = code 4 j + m); lo and hi track
// the least and greatest code before saturation.
template <int LAT>
struct CodesSink {
  static constexpr int D = LatticeTraits<LAT>::dim;
  uint32_t w[kLaneElems / 4];
  int32_t c[8];
  int32_t lo = 0, hi = 0;
  __device__ __forceinline__ void block(int b, const int32_t (&d)[D], uint32_t p) {
    static_assert(LAT != 2, "integer codes: Z, D4 or E8");
    const int o = (b * D) & 7;
#pragma unroll
    for (int i = 0; i < D; i++) c[o + i] = LAT == 8 ? (int32_t)(((uint32_t)d[i] << 1) | p) : (int32_t)((uint32_t)d[i] << 1);
  }
  __device__ __forceinline__ void group_done(int g) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      lo = c[i] < lo ? c[i] : lo;
      hi = c[i] > hi ? c[i] : hi;
      c[i] = c[i] < -127 ? -127 : (c[i] > 127 ? 127 : c[i]);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint32_t x = __builtin_amdgcn_perm((uint32_t)c[4 * h + 1], (uint32_t)c[4 * h], 0x0c0c0400u);
      const uint32_t y = __builtin_amdgcn_perm((uint32_t)c[4 * h + 3], (uint32_t)c[4 * h + 2], 0x04000c0cu);
      w[2 * g + h] = x | y;
    }
    asm volatile("" : "+v"(w[2 * g]), "+v"(w[2 * g + 1]));
  }
  __device__ __forceinline__ bool over() const { return lo < -127 || hi > 127; }
};

// Occupancy target: 7 waves per SIMD (72 VGPRs) without dither, 5 with it;
// 8 (64 VGPRs, no spill) for Z and D4, which measured 4.5% faster there on
// the 11008 x 4096 weight while E8 was 2% and A2 4% slower (bit-identical).
template <int LAT, bool DITHER, bool CODES>
constexpr int kDecodeWaves = DITHER ? 5 : ((CODES || LAT == 8 || LAT == 2) ? 7 : 8);
// CODES: write each tile's integer codes 2P (int8, saturated to [-127, 127]
// with HQ_FLAG_RANGE) instead of the reconstruction, for an int8 product
// (Z, D4, E8 without dither): the rebuild takes the step 2, and the inverse
// RHT and the store below are skipped.
template <int LAT, int N, bool DITHER, bool CODES = false>
__global__ void __launch_bounds__(DecodeGeom<N>::THREADS) __attribute__((amdgpu_waves_per_eu(kDecodeWaves<LAT, DITHER, CODES>)))
decode_kernel(const uint32_t* __restrict__ payload, uint64_t payload_words,
              const uint16_t* __restrict__ step, const uint16_t* __restrict__ meta,
              const uint32_t* __restrict__ chunk_off, uint64_t T, uint64_t C, float inv_sqrtn,
              uint32_t key_sign, uint32_t key_dither, A2Consts a2, void* __restrict__ out, uint32_t bf16,
              uint32_t* __restrict__ status, uint32_t stage_words, uint32_t chunk_cap_words,
              uint32_t tile_bound) {
  constexpr int LPT = N / kLaneElems;
  constexpr int TPW = DecodeGeom<N>::TPW;
  constexpr int SUB = DecodeGeom<N>::SUB;
  constexpr int THREADS = DecodeGeom<N>::THREADS;
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;
  constexpr uint32_t CB_LANE = LatticeTraits<LAT>::coset * BPL;
  constexpr uint32_t B = CB_LANE * LPT;

  // Two stage buffers, used by alternate units: while a unit is decoded from
  // one, the next unit's words stream into the other (global -> LDS loads in
  // flight during the decode), and wave 0 has scanned its chunk from tile
  // metadata it loaded a unit earlier.  The scan's tables rotate over three
  // sets: wave 0 writes the next unit's before the unit's barrier, while
  // another wave may still be a unit behind it, reading its own unit's set
  // (the barrier keeps every wave within one unit of the others).  No global
  // load is waited for on the critical path; one barrier per unit.
  extern __shared__ uint32_t smem[];
  uint32_t* stage0 = smem;                                  // [2][stage_words] a unit's words + guard
  uint32_t* tile_off0 = smem + 2 * stage_words;             // [3][64] bit offset of each tile in the chunk
  uint32_t* tile_ok0 = tile_off0 + 3 * kChunkTiles;         // [3][64]
  uint32_t* tile_ms0 = tile_ok0 + 3 * kChunkTiles;          // [3][64] meta | step << 16
  uint32_t* misc0 = tile_ms0 + 3 * kChunkTiles;             // [3][4] see scan()
  uint32_t* pmeta0 = misc0 + 12;                            // [2][64] a chunk's meta, loaded ahead
  uint32_t* pstep0 = pmeta0 + 2 * kChunkTiles;              // [2][64] and its steps
  uint32_t* ustart = pstep0 + 2 * kChunkTiles;              // [TPW * LPT] first unary bit per lane
  uint32_t* smask = ustart + TPW * LPT;                     // [N / 32] sign diagonal bits

  const int tid = threadIdx.x;
  const int tau = tid / LPT;
  const int p_lane = tid % LPT;                            // physical lane in the tile
  const int q = tile_lane<LPT>(p_lane);                     // logical lane

  // the lane's sign diagonal bits stay in LDS (smask[q]), read where needed
  (void)sign_mask<N>(smask, key_sign, tid, q);

  // tile metadata of a unit's chunk, loaded one unit before its scan by
  // wave 0 straight into LDS slot `slot` (no registers held; a tile past the
  // end reads the last one, the scan masks it), and the chunk offsets
  // (every wave: uniform values)
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  uint64_t pw0 = 0, pw1 = 0;
  auto fetch = [&](uint64_t un, int slot) {
    const uint64_t ch = un / SUB;
    if (tid < 64) {
      const uint64_t t0 = ch * kChunkTiles;
      const uint32_t i = t0 + (uint64_t)tid < T ? (uint32_t)tid : (uint32_t)(T - 1 - t0);
      lds_load_u16(meta + t0, 2u * i, smem_lds + 4u * (uint32_t)(pmeta0 - smem + slot * kChunkTiles));
      lds_load_u16(step + t0, 2u * i, smem_lds + 4u * (uint32_t)(pstep0 - smem + slot * kChunkTiles));
    }
    pw0 = chunk_off[ch];
    pw1 = chunk_off[ch + 1];
  };
  // wave 0: tile offsets inside the chunk (a chunk whose size disagrees with
  // its tiles is dropped) and the unit's word range.  misc: [0] 32 (L - w0)
  // (mod 2^32), where stage word 0 is payload word L, the unit's first word
  // aligned down to 4; [1] 16-byte vectors to stage; [2], [3] L.
  auto scan = [&](uint64_t un, int set, int slot) {
    const int first = (int)(un % SUB) * TPW;
    const bool range_ok = pw1 >= pw0 && pw1 <= payload_words && (pw1 - pw0) <= chunk_cap_words;
    const bool exists = (un / SUB) * kChunkTiles + (uint64_t)tid < T;
    const uint32_t mt = exists ? pmeta0[slot * kChunkTiles + tid] : 0u;
    const uint32_t st_ = exists ? pstep0[slot * kChunkTiles + tid] : 0u;
    const uint32_t len = mt >> 3, kk = mt & 7u;
    const uint32_t inc = wave_incl_scan(len);
    tile_off0[set * kChunkTiles + tid] = inc - len;
    const uint32_t total = __builtin_amdgcn_readlane(inc, kChunkTiles - 1);
    const bool too_long = wave_any(len > tile_bound);          // longer than any valid tile can be
    const bool chunk_ok = range_ok && !too_long && (uint64_t)((total + 31u) >> 5) == pw1 - pw0;
    tile_ok0[set * kChunkTiles + tid] = (chunk_ok && len >= B + (uint32_t)N * (kk + 1u)) ? 1u : 0u;
    tile_ms0[set * kChunkTiles + tid] = mt | (st_ << 16);
    // this unit's bits [tile_off[first], tile_off[first + TPW - 1] + len)
    const uint32_t f0 = __builtin_amdgcn_readlane(inc - len, first);
    const uint32_t f1 = __builtin_amdgcn_readlane(inc, first + TPW - 1);
    if (tid == 0) {
      uint64_t L = pw0;
      uint32_t nvec = 0;
      if (chunk_ok) {
        const uint64_t wa = pw0 + (f0 >> 5), we = pw0 + ((f1 + 31u) >> 5);
        L = wa & ~3ull;
        nvec = (uint32_t)((we - L + 3u) >> 2);
      }
      misc0[set * 4 + 0] = (uint32_t)(L - pw0) * 32u;
      misc0[set * 4 + 1] = nvec;
      misc0[set * 4 + 2] = (uint32_t)L;
      misc0[set * 4 + 3] = (uint32_t)(L >> 32);
    }
  };
  // all threads: start the unit's words (its scan in table set ts) streaming
  // into stage buffer buf (16 bytes a lane, straight to LDS; the stream's
  // last, partial vector by plain loads) and zero the guard words behind them
  auto stage_in = [&](int buf, int ts) {
    const uint32_t nvec = __builtin_amdgcn_readfirstlane(misc0[ts * 4 + 1]);
    const uint64_t L = (uint64_t)__builtin_amdgcn_readfirstlane(misc0[ts * 4 + 2]) |
                       ((uint64_t)__builtin_amdgcn_readfirstlane(misc0[ts * 4 + 3]) << 32);
    const int set = buf;
    uint32_t* st = stage0 + set * stage_words;
    uint32_t lt = (uint32_t)tid;
    opaque(lt);                                             // (recomputed here, not held across the unit)
    const uint32_t wave0 = __builtin_amdgcn_readfirstlane(lt & ~63u);   // this wave's first thread
    for (uint32_t r = 0; r * (uint32_t)THREADS < nvec; r++) {
      const uint32_t j = r * (uint32_t)THREADS + lt;
      if (j < nvec) {
        const uint64_t g = L + 4ull * j;
        if (g + 4u <= payload_words) {
          // this wave's 1 KB of the stage
          const uint32_t dst = smem_lds + 4u * ((uint32_t)set * stage_words + 4u * (r * (uint32_t)THREADS + wave0));
          lds_load16(payload + L, 16u * j, dst);
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) st[4u * j + (uint32_t)e] = g + (uint64_t)e < payload_words ? payload[g + e] : 0u;
        }
      }
    }
    if (lt < 8u) st[4u * nvec + lt] = 0u;
  };

  const uint64_t units = C * SUB;
  // priority by the units this workgroup has left (the current one included)
  uint64_t left = blockIdx.x < units ? (units - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  // unit k (k-th of this workgroup) uses stage buffer k & 1, metadata slot
  // k & 1 and table set k mod 3
  if (blockIdx.x < units) {
    fetch(blockIdx.x, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < 64) scan(blockIdx.x, 0, 0);
    if (blockIdx.x + gridDim.x < units) fetch(blockIdx.x + gridDim.x, 1);
    __syncthreads();
    stage_in(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  int cur = 0, ts = 0;
  for (uint64_t unit = blockIdx.x; unit < units; unit += gridDim.x, cur ^= 1, ts = ts == 2 ? 0 : ts + 1) {
    wave_priority(left >= 4u ? 3u : (uint32_t)left - 1u);
    left--;
    const uint64_t un = unit + gridDim.x;
    const int tn = ts == 2 ? 0 : ts + 1;                    // the next unit's table set
    // this unit's words have landed (each wave waited for its own loads
    // before its previous stores, the barrier waits for everyone's); wave 0
    // scans the next unit
    if (un < units) {
      if (tid < 64) scan(un, tn, cur ^ 1);
      if (un + gridDim.x < units) fetch(un + gridDim.x, cur);   // (issued before the stage loads)
    }
    __syncthreads();
    if (un < units) stage_in(cur ^ 1, tn);

    const uint32_t* stage = stage0 + cur * stage_words;
    const uint64_t chunk = unit / SUB;
    const int first = (int)(unit % SUB) * TPW;              // first tile of this unit in the chunk
    const int ct = first + tau;                             // tile index in the chunk
    const uint64_t t = chunk * kChunkTiles + (uint64_t)ct;
    const bool active = t < T;
    const uint32_t ms = tile_ms0[ts * kChunkTiles + ct];
    const uint32_t m = active ? (ms & 0xFFFFu) : 0u;
    const uint32_t len = m >> 3, k = m & 7u;
    const uint32_t sraw = active ? (ms >> 16) : 0u;
    // the encoder writes +0 or a finite step of at least 2^-124, nothing
    // else: any other step marks a corrupt tile
    bool ok = active && tile_ok0[ts * kChunkTiles + ct] != 0u && (sraw == 0u || sraw - 0x180u < 0x7E00u);
    const uint32_t start = tile_off0[ts * kChunkTiles + ct] - misc0[ts * 4 + 0], end = start + len;
    const uint32_t ub = start + B + (uint32_t)N * k;        // unary plane

    // ---- where does each lane's first unary code start?  Every codeword has
    // exactly one 1 in the unary plane [ub, end): count ones over the aligned
    // stage words that cover it (the first masked below ub, the last at
    // end), kUW consecutive words per physical lane per round, so the usual
    // tile takes one round.  The lane whose word holds the (32 q)-th one
    // records that word's index and the one's rank in it for logical lane q
    // (index < 2^27, rank < 32: one word), and after a wave-level sync (a
    // tile's lanes share a wave) lane q finds the bit itself: one select per
    // lane. ----
    constexpr uint32_t kUW = 3;
    const uint32_t a0 = ub >> 5;
    const uint32_t nw = ok ? ((end - 1u) >> 5) - a0 + 1u : 0u;   // ok: end - ub >= N
    const uint32_t lo_mask = ~0u << (ub & 31u);
    const uint32_t hi_keep = end & 31u;                       // counted bits of the last word (0: all)
    uint32_t carry = 0;
    for (uint32_t r = 0;; r++) {
      const bool more = r * kUW * (uint32_t)LPT < nw;
      if (!wave_any(more)) break;
      const uint32_t j0 = (r * (uint32_t)LPT + (uint32_t)p_lane) * kUW;
      uint32_t c[kUW], cs = 0;
#pragma unroll
      for (uint32_t i = 0; i < kUW; i++) {
        const uint32_t j = j0 + i;
        uint32_t x = j < nw ? stage[a0 + j] : 0u;
        if (j == 0u) x &= lo_mask;
        if (j + 1u == nw && hi_keep != 0u) x &= (1u << hi_keep) - 1u;
        c[i] = __builtin_popcount(x);
        cs += c[i];
      }
      uint32_t inc, tot;
      tile_scan<LPT>(cs, p_lane, inc, tot);
      uint32_t before = carry + inc - cs;
#pragma unroll
      for (uint32_t i = 0; i < kUW; i++) {
        const uint32_t after = before + c[i];
        const uint32_t mm = before / 32u + 1u;
        if (c[i] != 0u && mm < (uint32_t)LPT && 32u * mm <= after)
          ustart[tau * LPT + mm] = ((a0 + j0 + i) << 5) | (32u * mm - before - 1u);
        before = after;
      }
      carry += tot;
    }
    ok = ok && carry == (uint32_t)N;
    wave_lds_sync();                                        // (a tile's lanes are in one wave)

    // ---- parse and rebuild, specialised on the tile's Rice parameter; a lane
    // of an invalid tile reads from bit 0 with no run limit (in bounds, result
    // discarded).  The values reach the oracle's in one of two ways:
    //  - a step of at least 2^-124 (every other nonzero one is corrupt): the
    //    rebuild takes the step times the butterfly's lane sign (and, for E8,
    //    D4 and Z without dither, times 1/sqrt(n) where that is a power of
    //    two), every zero is +0, and the presigned butterfly ends with the
    //    exact values (the rest of the scale follows it).  E8, D4 and Z points
    //    are multiples of 1/2 with at most 14 significant bits, so every
    //    product and butterfly value is a multiple of 2^-134 (2^-138 scaled),
    //    representable wherever it falls.  A2's sqrt3 coordinate and dithered
    //    ones are rounded, so their products are not scaled; a product rounded
    //    once is the same product negated, and it is not zero (a dithered
    //    coordinate is at least 2^-25 from zero, 2^-25 * 2^-124 is the least
    //    subnormal).  No value is ever -0.
    //  - a +0 step: every value is a signed zero.  The rebuild takes the step
    //    1 to see each value's sign, and the signs go through the butterfly's
    //    rules for zeros (at the store). ----
    static_assert(!CODES || (!DITHER && LAT != 2), "integer codes: Z, D4 or E8 without dither");
    constexpr bool kFoldScale = kPow2Scale<N> && LAT != 2 && !DITHER && !CODES;
    float a[kLaneElems];
    CodesSink<LAT == 2 ? 8 : LAT> codes;                    // (CODES only)
    bool lane_ok;
    const bool zero_step = sraw == 0u;
    {
      const float s = as_f(sraw << 16);
      uint32_t cbits = 0;
      if constexpr (CB_LANE > 0) cbits = lds_read32(stage, ok ? start + (uint32_t)q * CB_LANE : 0u);
      const float s_lane = CODES ? 2.0f
                                 : zero_step ? 1.0f : (lane_sign_odd(q) ? -s : s) * (kFoldScale ? inv_sqrtn : 1.0f);
      const uint32_t rb = ok ? start + B + (uint32_t)q * kLaneElems * k : 0u;
      uint32_t lt = (uint32_t)tid;
      opaque(lt);                                           // (an address recomputed, not spilled)
      uint32_t u0 = ub;
      if (q != 0) {
        // the recorded word, masked as when counted (bits past the tile's end
        // cannot hold a rank below its count of ones), and the bit after its
        // rank-th one
        const uint32_t rec = ok ? ustart[(lt & ~(uint32_t)(LPT - 1)) + (uint32_t)q] : 0u;
        const uint32_t wa = rec >> 5;
        uint32_t x = stage[wa];
        if (wa == a0) x &= lo_mask;
        u0 = 32u * wa + select_bit(x, rec & 31u) + 1u;
      }
      u0 = ok ? u0 : 0u;
      const uint32_t lim = ok ? end : 0u;
      const uint32_t g_lane = (uint32_t)(t * N) + (uint32_t)(q * kLaneElems);
      uint32_t upos = 0;
      bool pok;
      if constexpr (CODES) {
        switch (k) {
#define HQ_PARSE_CASE(KK) \
          case KK: pok = parse_codes<LAT, KK>(stage, rb, u0, lim, cbits, codes, upos); break;
          HQ_PARSE_CASE(0) HQ_PARSE_CASE(1) HQ_PARSE_CASE(2) HQ_PARSE_CASE(3)
          HQ_PARSE_CASE(4) HQ_PARSE_CASE(5) HQ_PARSE_CASE(6)
          default: pok = parse_codes<LAT, 7>(stage, rb, u0, lim, cbits, codes, upos); break;
#undef HQ_PARSE_CASE
        }
      } else {
        switch (k) {
#define HQ_PARSE_CASE(KK) \
          case KK: pok = parse_lane<LAT, DITHER, KK>(stage, rb, u0, lim, cbits, s_lane, key_dither, g_lane, a2, a, upos); break;
          HQ_PARSE_CASE(0) HQ_PARSE_CASE(1) HQ_PARSE_CASE(2) HQ_PARSE_CASE(3)
          HQ_PARSE_CASE(4) HQ_PARSE_CASE(5) HQ_PARSE_CASE(6)
          default: pok = parse_lane<LAT, DITHER, 7>(stage, rb, u0, lim, cbits, s_lane, key_dither, g_lane, a2, a, upos); break;
#undef HQ_PARSE_CASE
        }
      }
      lane_ok = ok && pok;
      if (q == LPT - 1 && upos != end) lane_ok = false;      // the last one ends the tile
    }

    // tile-wide AND; every lane takes part in the shuffles (no short-circuit)
    int all_ok = lane_ok ? 1 : 0;
#pragma unroll
    for (int s2 = 1; s2 < LPT; s2 <<= 1) all_ok &= (int)lane_xor((uint32_t)all_ok, partner_xor<LPT>(s2));
    lane_ok = all_ok != 0;

    // the next unit's stage loads, a unit old by now, are complete before
    // this unit's stores are issued (vector memory operations retire in
    // order: the next wait needs no store to finish)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (CODES) {
      // 2P is an exact integer; an invalid tile's codes are zeros
      if (active) {
        if (!lane_ok && q == 0) atomicOr(status, HQ_FLAG_CORRUPT);
        uint32_t w[8];
#pragma unroll
        for (int v = 0; v < 8; v++) w[v] = lane_ok ? codes.w[v] : 0u;
        if (lane_ok && codes.over()) atomicOr(status, HQ_FLAG_RANGE);
        uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<int8_t*>(out) + t * N + (uint64_t)q * kLaneElems);
        p[0] = make_uint4(w[0], w[1], w[2], w[3]);
        p[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
      continue;
    }
    // ---- inverse RHT and store (an invalid tile decodes to zeros) ----
    if (active) {
      if (!lane_ok) {
        if (q == 0) atomicOr(status, HQ_FLAG_CORRUPT);
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) a[i] = 0.0f;
      }
      // a +0 step: the outputs' signs (bit i for element i) from the rebuilt
      // values' signs; the values themselves become +0
      uint32_t zsign = 0;
      if (wave_any(zero_step && lane_ok)) {
        asm volatile("");                                   // (rare: kept out of line)
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) m |= (as_u(a[i]) >> 31) << i;
        zsign = zero_sign_butterfly<LPT>(zero_step && lane_ok ? m : 0u, q);
        if (zero_step) {
#pragma unroll
          for (int i = 0; i < kLaneElems; i++) a[i] = 0.0f;
        }
      }
      // then y = z fl(1/sqrt(n)) (already in the presigned values where it
      // was folded there), and the sign diagonal (on the packed bf16 pairs:
      // rounding to nearest even commutes with a sign flip)
      fwht_tile_signed<LPT>(a, q);
      if constexpr (!kFoldScale) {
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) a[i] = a[i] * inv_sqrtn;
      }
      uint32_t qs = (uint32_t)q;
      opaque(qs);                                           // (the address formed here, not held across the loop)
      const uint32_t sg = smask[qs] ^ zsign;
      const uint64_t base = t * N + (uint64_t)q * kLaneElems;
      if (bf16) {
        uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + base);
        uint32_t sw[2];
        pair_sign_words(sg, sw);
#pragma unroll
        for (int v = 0; v < 4; v++) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; h++)
            w[h] = bf16x2_rne(a[v * 8 + 2 * h], a[v * 8 + 2 * h + 1]) ^ pair_sign_mask(sw, 4 * v + h);
          p[v] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) a[i] = as_f(as_u(a[i]) ^ ((sg << (31 - i)) & 0x80000000u));
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base);
#pragma unroll
        for (int v = 0; v < 8; v++) p[v] = make_float4(a[v * 4], a[v * 4 + 1], a[v * 4 + 2], a[v * 4 + 3]);
      }
    }
  }
}

// --------------------------------------------------------------------------
// The quantiser alone (Methodology 2): the nearest lattice point of each
// d-block of t, with the encoder's own decision and tie rules, one block per
// thread (grid-strided).
// --------------------------------------------------------------------------
template <int LAT>
__global__ void __launch_bounds__(256) nearest_kernel(const float* __restrict__ t, uint64_t nblocks,
                                                      float* __restrict__ pt, A2Consts a2) {
  constexpr int D = LatticeTraits<LAT>::dim;
  for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += (uint64_t)gridDim.x * blockDim.x) {
    float v[D], p[D];
#pragma unroll
    for (int i = 0; i < D; i++) v[i] = t[b * D + i];
    if constexpr (LAT == 8) {
      nearest_e8_point(v, p);
    } else {
      int32_t d[D];
      uint32_t c;
      nearest<LAT>(v, d, c, a2);
      code_point<LAT>(d, c, p, a2);
    }
#pragma unroll
    for (int i = 0; i < D; i++) pt[b * D + i] = p[i];
  }
}
using NearFn = void (*)(const float*, uint64_t, float*, A2Consts);

// ---- per-lattice kernel tables (defined in hq_kern_<lattice>.hip) ----------
using EncFn = void (*)(const void*, uint32_t, uint64_t, uint64_t, float, float, float, uint32_t, uint32_t,
                       A2Consts, uint32_t*, uint64_t, uint16_t*, uint16_t*, uint32_t*, uint32_t*, uint32_t*,
                       uint32_t, uint32_t, uint32_t, uint32_t);
using DecFn = void (*)(const uint32_t*, uint64_t, const uint16_t*, const uint16_t*, const uint32_t*, uint64_t,
                       uint64_t, float, uint32_t, uint32_t, A2Consts, void*, uint32_t, uint32_t*, uint32_t,
                       uint32_t, uint32_t);

template <int LAT, int N>
EncFn enc_table_n(bool dither, bool bf16) {
  if (dither) return bf16 ? encode_kernel<LAT, N, true, true> : encode_kernel<LAT, N, true, false>;
  return bf16 ? encode_kernel<LAT, N, false, true> : encode_kernel<LAT, N, false, false>;
}
template <int LAT>
EncFn enc_table(uint32_t n, bool dither, bool bf16) {
  if (n == 64) return enc_table_n<LAT, 64>(dither, bf16);
  if (n == 128) return enc_table_n<LAT, 128>(dither, bf16);
  return enc_table_n<LAT, 256>(dither, bf16);
}
using LenFn = void (*)(const void*, uint64_t, uint64_t, float, float, float, uint32_t, uint32_t, A2Consts,
                       unsigned long long*);
template <int LAT, int N>
LenFn len_table_n(bool dither, bool bf16) {
  if (dither) return bf16 ? length_kernel<LAT, N, true, true> : length_kernel<LAT, N, true, false>;
  return bf16 ? length_kernel<LAT, N, false, true> : length_kernel<LAT, N, false, false>;
}
template <int LAT>
LenFn len_table(uint32_t n, bool dither, bool bf16) {
  if (n == 64) return len_table_n<LAT, 64>(dither, bf16);
  if (n == 128) return len_table_n<LAT, 128>(dither, bf16);
  return len_table_n<LAT, 256>(dither, bf16);
}
template <int LAT>
DecFn dec_codes_table(uint32_t n) {
  if (n == 64) return decode_kernel<LAT, 64, false, true>;
  if (n == 128) return decode_kernel<LAT, 128, false, true>;
  return decode_kernel<LAT, 256, false, true>;
}
template <int LAT>
DecFn dec_table(uint32_t n, bool dither) {
  if (n == 64) return dither ? decode_kernel<LAT, 64, true> : decode_kernel<LAT, 64, false>;
  if (n == 128) return dither ? decode_kernel<LAT, 128, true> : decode_kernel<LAT, 128, false>;
  return dither ? decode_kernel<LAT, 256, true> : decode_kernel<LAT, 256, false>;
}

EncFn enc_fn_z(uint32_t n, bool dither, bool bf16);
EncFn enc_fn_a2(uint32_t n, bool dither, bool bf16);
EncFn enc_fn_d4(uint32_t n, bool dither, bool bf16);
EncFn enc_fn_e8(uint32_t n, bool dither, bool bf16);
LenFn len_fn_z(uint32_t n, bool dither, bool bf16);
LenFn len_fn_a2(uint32_t n, bool dither, bool bf16);
LenFn len_fn_d4(uint32_t n, bool dither, bool bf16);
LenFn len_fn_e8(uint32_t n, bool dither, bool bf16);
DecFn dec_fn_z(uint32_t n, bool dither);
DecFn dec_fn_a2(uint32_t n, bool dither);
DecFn dec_fn_d4(uint32_t n, bool dither);
DecFn dec_fn_e8(uint32_t n, bool dither);
NearFn near_fn_z();
NearFn near_fn_a2();
NearFn near_fn_d4();
NearFn near_fn_e8();
DecFn dec_codes_fn_z(uint32_t n);
DecFn dec_codes_fn_d4(uint32_t n);
DecFn dec_codes_fn_e8(uint32_t n);

}  // namespace hq
