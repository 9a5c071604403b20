// hq_lib.hip — HyperQuant encode/decode kernels for gfx950 and the C ABI of
// libhq.so (declared in include/hq.h).
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
// Decode: one workgroup per chunk (grid-strided): payload staged in LDS, one
// lane per tile parses its Rice codewords into LDS, then every lane rebuilds
// its 32 elements, runs the butterfly and stores.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "hq.h"
#include "hq_device.h"

using namespace hq;

namespace {

struct RateEntry { uint8_t lattice, dither; uint16_t tile; uint16_t bps_q; uint32_t c_bits; };
#include "hq_rate_table.inc"   // kRateTable[], generated from rate_table.json

// Look-back words: (epoch << 34) | (flag << 32) | value.  The value travels
// inside the atomic word itself, so relaxed agent-scope atomics suffice: no
// other memory is published through them (release/acquire at agent scope
// would write back / invalidate the whole L2 of the XCD on every chunk).
constexpr uint32_t kFlagAgg = 1u, kFlagIncl = 2u;
constexpr uint32_t kEpochMask = 0x3FFFFFFFu;

// --------------------------------------------------------------------------
// Encode kernel
// --------------------------------------------------------------------------
template <int LAT, int N, bool BF16, bool DITHER>
__global__ void __launch_bounds__(kChunkTiles * (N / kLaneElems)) __attribute__((amdgpu_waves_per_eu(4)))
encode_kernel(const void* __restrict__ x, uint64_t T, uint64_t C, float c, float inv_sqrtn, float inv_n,
              uint32_t key_sign, uint32_t key_dither, A2Consts a2,
              uint32_t* __restrict__ payload, uint64_t cap_words,
              uint16_t* __restrict__ step_out, uint16_t* __restrict__ meta_out,
              uint32_t* __restrict__ chunk_off, uint32_t* __restrict__ status,
              uint32_t* __restrict__ ws, uint32_t stage_words) {
  constexpr int LPT = N / kLaneElems;                       // lanes per tile
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;                       // lattice blocks per lane
  constexpr uint32_t CB_LANE = LatticeTraits<LAT>::coset * BPL;   // coset bits per lane
  constexpr uint32_t B = CB_LANE * LPT;                     // coset bits per tile

  extern __shared__ uint32_t smem[];
  uint32_t* stage = smem;                                   // [stage_words]
  uint32_t* tile_len = smem + stage_words;                  // [64]
  uint32_t* tile_off = tile_len + kChunkTiles;              // [64]
  uint32_t* misc = tile_off + kChunkTiles;                  // [4]

  const int tid = threadIdx.x;
  const int tau = tid / LPT;
  const int q = tid % LPT;
  uint64_t* look = reinterpret_cast<uint64_t*>(ws + 2);

  // sign diagonal entries of this lane's 32 positions (Methodology 1)
  uint32_t sgn = 0;
#pragma unroll
  for (int i = 0; i < kLaneElems; i++) sgn |= (pcg_hash(key_sign + (uint32_t)(q * kLaneElems + i)) >> 31) << i;

  const float lane_scale = (__builtin_popcount((uint32_t)q) & 1) ? -inv_sqrtn : inv_sqrtn;

  if (tid == 0) misc[2] = __hip_atomic_load(&ws[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t epoch = misc[2] & kEpochMask;

  for (;;) {
    if (tid == 0) {
      uint32_t tk = __hip_atomic_fetch_add(&ws[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      misc[0] = tk;
      if ((uint64_t)tk == C + gridDim.x - 1) {               // last ticket: all taken, reset for next call
        __hip_atomic_store(&ws[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ws[1], (epoch + 1u) & kEpochMask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    const uint64_t chunk = misc[0];
    if (chunk >= C) break;

    const uint64_t t = chunk * kChunkTiles + (uint64_t)tau;
    const bool active = t < T;

    // ---- load + sign (bf16 -> fp32 is exact) ----
    float a[kLaneElems];
    if (active) {
      const uint64_t base = t * N + (uint64_t)q * kLaneElems;
      if constexpr (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + base);
#pragma unroll
        for (int v = 0; v < 4; v++) {
          uint4 w = p[v];
          uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int h = 0; h < 4; h++) {
            a[v * 8 + 2 * h] = as_f(ww[h] << 16);
            a[v * 8 + 2 * h + 1] = as_f(ww[h] & 0xFFFF0000u);
          }
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + base);
#pragma unroll
        for (int v = 0; v < 8; v++) {
          float4 w = p[v];
          a[v * 4] = w.x; a[v * 4 + 1] = w.y; a[v * 4 + 2] = w.z; a[v * 4 + 3] = w.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLaneElems; i++) a[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) a[i] = as_f(as_u(a[i]) ^ (((sgn >> i) & 1u) << 31));

    // ---- RHT: butterfly, then 1/sqrt(n) (with the lane's butterfly sign) ----
    fwht_tile_signed<LPT>(a, q);
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) a[i] = a[i] * lane_scale;

    // ---- tile energy: pairwise tree over the tile, step = bf16(rms * c) ----
    float sq[kLaneElems];
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) sq[i] = a[i] * a[i];
#pragma unroll
    for (int m = kLaneElems; m > 1; m >>= 1) {
#pragma unroll
      for (int i = 0; i < m / 2; i++) sq[i] = sq[2 * i] + sq[2 * i + 1];
    }
    float ss = sq[0];
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) ss = ss + __shfl_xor(ss, m);
    bool nonfinite = (as_u(ss) & 0x7F800000u) == 0x7F800000u;
    float s = 0.0f;
    uint32_t sbits = 0;
    if (!nonfinite) {
      float rms = sqrtf(ss * inv_n);
      float r = rms * c;
      sbits = bf16_rne_bits(r);
      if ((sbits & 0x7F80u) == 0x7F80u) { nonfinite = true; sbits = 0; }
      else if ((sbits & 0x7F80u) == 0) sbits = 0;
      s = as_f(sbits << 16);
    }
    const float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) a[i] = nonfinite ? 0.0f : a[i] * inv;

    // ---- KV: add the dither (Methodology 4) ----
    if constexpr (DITHER) {
      const uint32_t g_lane = (uint32_t)(t * N) + (uint32_t)(q * kLaneElems);
#pragma unroll
      for (int b = 0; b < BPL; b++) {
        float u[D];
        dither_block<LAT>(key_dither, g_lane + (uint32_t)(b * D), u, a2);
#pragma unroll
        for (int i = 0; i < D; i++) a[b * D + i] = a[b * D + i] + u[i];
      }
    }

    // ---- nearest lattice point, strip, zigzag ----
    uint32_t sym[kLaneElems];
    uint32_t cb = 0;
#pragma unroll
    for (int b = 0; b < BPL; b++) {
      int32_t d[D];
      uint32_t p;
      nearest<LAT>(&a[b * D], d, p, a2);
      block_symbols<LAT>(d, &sym[b * D]);
      cb |= p << b;
    }

    // ---- Rice parameter: smallest k in 0..7 minimising the tile's length ----
    // S[k] = sum of sym >> k over this lane.  When every symbol of the wave
    // fits a byte, four symbols share a register and one shift, one mask and
    // one byte-sum (v_sad_u8) add four terms.
    uint32_t S[8];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kLaneElems; i++) mx |= sym[i];
    if (__all(mx < 256u)) {
      uint32_t P[kLaneElems / 4];
#pragma unroll
      for (int j = 0; j < kLaneElems / 4; j++)
        P[j] = sym[4 * j] | (sym[4 * j + 1] << 8) | (sym[4 * j + 2] << 16) | (sym[4 * j + 3] << 24);
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const uint32_t bmask = 0x01010101u * (0xFFu >> k);
        uint32_t acc = 0;
#pragma unroll
        for (int j = 0; j < kLaneElems / 4; j++) acc = __builtin_amdgcn_sad_u8((P[j] >> k) & bmask, 0u, acc);
        S[k] = acc;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; k++) {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) acc += sym[i] >> k;
        S[k] = acc;
      }
    }
    uint32_t best_k = 0, best_c = 0xFFFFFFFFu;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      uint32_t tot = S[k];
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) tot += __shfl_xor(tot, m);
      uint32_t cost = tot + (uint32_t)N * (1u + k);
      if (cost < best_c) { best_c = cost; best_k = k; }
    }
    const uint32_t k = best_k;
    // this lane's unary quotients: sum (q_i + 1) bits; exclusive prefix over the tile's lanes
    uint32_t lane_unary = 0;
#pragma unroll
    for (int kk = 0; kk < 8; kk++) if (kk == (int)k) lane_unary = S[kk];
    lane_unary += (uint32_t)kLaneElems;
    uint32_t incl = lane_unary;
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) {
      uint32_t v = __shfl_up(incl, m, LPT);
      if (q >= m) incl += v;
    }
    const uint32_t lane_excl = incl - lane_unary;
    const uint32_t tlen = B + best_c;
    if (q == 0) tile_len[tau] = active ? tlen : 0u;
    __syncthreads();

    // ---- chunk scan: bit offset of every tile inside the chunk ----
    if (tid < kChunkTiles) {
      uint32_t v = tile_len[tid], inc = v;
#pragma unroll
      for (int m = 1; m < kChunkTiles; m <<= 1) {
        uint32_t o = __shfl_up(inc, m, kChunkTiles);
        if (tid >= m) inc += o;
      }
      tile_off[tid] = inc - v;
      if (tid == kChunkTiles - 1) misc[1] = inc;
    }
    __syncthreads();
    const uint32_t total_bits = misc[1];
    uint32_t W = (total_bits + 31u) >> 5;
    const bool fits = W + 2 <= stage_words;

    // publish this chunk's size early so later chunks can look back past it
    if (tid == 0) {
      uint64_t tag = (uint64_t)((epoch << 2) | (chunk == 0 ? kFlagIncl : kFlagAgg));
      __hip_atomic_store(&look[chunk], (tag << 32) | W, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (uint32_t i = tid; i < W + 2 && i < stage_words; i += blockDim.x) stage[i] = 0u;
    __syncthreads();

    // ---- pack: coset bits | remainder plane (k bits per symbol) | unary plane ----
    if (active && fits) {
      const uint32_t t0 = tile_off[tau];
      if constexpr (CB_LANE > 0) lds_or_bits(stage, t0 + (uint32_t)q * CB_LANE, cb, CB_LANE);
      if (k > 0) {
        // four k-bit remainders (at most 28 bits) per OR into the staging bits
        const uint32_t rmask = (1u << k) - 1u;
        uint32_t rpos = t0 + B + (uint32_t)q * kLaneElems * k;
#pragma unroll
        for (int g = 0; g < kLaneElems / 4; g++) {
          const uint32_t f = (sym[4 * g] & rmask) | ((sym[4 * g + 1] & rmask) << k) |
                             ((sym[4 * g + 2] & rmask) << (2u * k)) | ((sym[4 * g + 3] & rmask) << (3u * k));
          lds_or_bits(stage, rpos, f, 4u * k);
          rpos += 4u * k;
        }
      }
      uint32_t upos = t0 + B + (uint32_t)N * k + lane_excl;
#pragma unroll
      for (int i = 0; i < kLaneElems; i++) {
        upos += sym[i] >> k;
        atomicOr(&stage[upos >> 5], 1u << (upos & 31u));
        upos += 1u;
      }
    }
    __syncthreads();

    // ---- decoupled look-back, one predecessor per lane of wave 0 ----
    if (tid < 64) {
      uint32_t excl = 0;
      if (chunk > 0) {
        int64_t base = (int64_t)chunk - 1;
        for (;;) {
          const int64_t j = base - tid;
          uint64_t v;
          uint32_t flag;
          if (j < 0) {
            v = 0;
            flag = kFlagIncl;                                // before chunk 0: prefix 0
          } else {
            for (;;) {
              v = __hip_atomic_load(&look[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              const uint32_t hi = (uint32_t)(v >> 32);
              if ((hi >> 2) == epoch && (hi & 3u) != 0) { flag = hi & 3u; break; }
              __builtin_amdgcn_s_sleep(1);
            }
          }
          const uint64_t incl_mask = __ballot(flag == kFlagIncl);
          const int first = incl_mask ? __builtin_ctzll(incl_mask) : 64;
          uint32_t part = (tid <= first) ? (uint32_t)v : 0u;
#pragma unroll
          for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m);
          excl += part;
          if (incl_mask) break;
          base -= 64;
        }
      }
      if (tid == 0) {
        if (chunk > 0) {
          uint64_t tag = (uint64_t)((epoch << 2) | kFlagIncl);
          __hip_atomic_store(&look[chunk], (tag << 32) | (uint64_t)(excl + W), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
        misc[3] = excl;
        chunk_off[chunk] = excl;
        if (chunk == C - 1) chunk_off[C] = excl + W;
        if (!fits || (uint64_t)excl + W > cap_words) atomicOr(status, HQ_FLAG_NOSPACE);
      }
    }
    __syncthreads();
    const uint32_t excl = misc[3];
    if (fits && (uint64_t)excl + W <= cap_words) {
      for (uint32_t i = tid; i < W; i += blockDim.x) payload[excl + i] = stage[i];
    }
    if (active && q == 0) {
      step_out[t] = (uint16_t)sbits;
      meta_out[t] = (uint16_t)((tlen << 3) | k);
      if (nonfinite) atomicOr(status, HQ_FLAG_NONFINITE);
    }
    __syncthreads();
  }
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

template <int LAT, int N, bool BF16, bool DITHER>
__global__ void __launch_bounds__(DecodeGeom<N>::THREADS)
decode_kernel(const uint32_t* __restrict__ payload, uint64_t payload_words,
              const uint16_t* __restrict__ step, const uint16_t* __restrict__ meta,
              const uint32_t* __restrict__ chunk_off, uint64_t T, uint64_t C, float inv_sqrtn,
              uint32_t key_sign, uint32_t key_dither, A2Consts a2, void* __restrict__ out,
              uint32_t* __restrict__ status, uint32_t stage_words, uint32_t chunk_cap_words,
              uint32_t tile_bound) {
  constexpr int LPT = N / kLaneElems;
  constexpr int TPW = DecodeGeom<N>::TPW;
  constexpr int SUB = DecodeGeom<N>::SUB;
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;
  constexpr uint32_t CB_LANE = LatticeTraits<LAT>::coset * BPL;
  constexpr uint32_t B = CB_LANE * LPT;

  extern __shared__ uint32_t smem[];
  uint32_t* stage = smem;                                   // [stage_words] this unit's bits + guard
  uint32_t* tile_off = stage + stage_words;                 // [64] bit offset of each tile in the chunk
  uint32_t* tile_ok = tile_off + kChunkTiles;               // [64]
  uint32_t* ustart = tile_ok + kChunkTiles;                 // [TPW * LPT] first unary bit per lane
  uint32_t* misc = ustart + TPW * LPT;                      // [4]

  const int tid = threadIdx.x;
  const int tau = tid / LPT;
  const int q = tid % LPT;

  uint32_t sgn = 0;
#pragma unroll
  for (int i = 0; i < kLaneElems; i++) sgn |= (pcg_hash(key_sign + (uint32_t)(q * kLaneElems + i)) >> 31) << i;
  const float lane_scale = (__builtin_popcount((uint32_t)q) & 1) ? -inv_sqrtn : inv_sqrtn;

  const uint64_t units = C * SUB;
  for (uint64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const uint64_t chunk = unit / SUB;
    const int first = (int)(unit % SUB) * TPW;              // first tile of this unit in the chunk
    const uint64_t w0 = chunk_off[chunk], w1 = chunk_off[chunk + 1];
    const bool range_ok = w1 >= w0 && w1 <= payload_words && (w1 - w0) <= chunk_cap_words;

    // tile offsets inside the chunk; a chunk whose size disagrees with its tiles is dropped
    if (tid < kChunkTiles) {
      const uint64_t tt = chunk * kChunkTiles + (uint64_t)tid;
      const uint32_t m = tt < T ? (uint32_t)meta[tt] : 0u;
      const uint32_t len = m >> 3, kk = m & 7u;
      uint32_t inc = len;
#pragma unroll
      for (int s2 = 1; s2 < kChunkTiles; s2 <<= 1) {
        uint32_t o = __shfl_up(inc, s2, kChunkTiles);
        if (tid >= s2) inc += o;
      }
      tile_off[tid] = inc - len;
      const uint32_t total = __shfl(inc, kChunkTiles - 1, kChunkTiles);
      const bool too_long = __any(len > tile_bound);        // longer than any valid tile can be
      const bool chunk_ok = range_ok && !too_long && (uint64_t)((total + 31u) >> 5) == w1 - w0;
      tile_ok[tid] = (chunk_ok && len >= B + (uint32_t)N * (kk + 1u)) ? 1u : 0u;
      // this unit's bit range [tile_off[first], tile_off[first + TPW]) in whole words
      if (tid == first) misc[0] = chunk_ok ? (inc - len) : 0u;
      if (tid == first + TPW - 1) misc[1] = chunk_ok ? inc : 0u;
    }
    __syncthreads();
    const uint32_t sw = misc[0] >> 5;                       // first staged word (chunk-relative)
    const uint32_t WL = ((misc[1] + 31u) >> 5) - sw;        // words staged
    const uint32_t base_bit = sw * 32u;
    for (uint32_t i = tid; i < WL; i += blockDim.x) stage[i] = payload[w0 + sw + i];
    if (tid < 4) stage[WL + tid] = 0u;
    __syncthreads();

    const int ct = first + tau;                             // tile index in the chunk
    const uint64_t t = chunk * kChunkTiles + (uint64_t)ct;
    const bool active = t < T;
    const uint32_t m = active ? (uint32_t)meta[t] : 0u;
    const uint32_t len = m >> 3, k = m & 7u;
    bool ok = active && tile_ok[ct] != 0u;
    const uint32_t start = tile_off[ct] - base_bit, end = start + len;
    const uint32_t ub = start + B + (uint32_t)N * k;        // unary plane

    // ---- where does each lane's first unary code start?  Every codeword has
    // exactly one 1 in the unary plane: count ones word by word (lane q takes
    // words q, q+LPT, ...) and mark the bit after the (32 q)-th one. ----
    const uint32_t words = ok ? (end - ub + 31u) >> 5 : 0u;
    uint32_t carry = 0;
    for (uint32_t r = 0;; r++) {
      const bool more = r * LPT < words;
      if (!__any(more)) break;
      const uint32_t j = r * LPT + (uint32_t)q;
      uint32_t w = 0;
      if (j < words) {
        const uint32_t p = ub + 32u * j;
        w = lds_read32(stage, p);
        const uint32_t valid = end - p;
        if (valid < 32u) w &= (1u << valid) - 1u;
      }
      const uint32_t c = __builtin_popcount(w);
      uint32_t inc = c;
#pragma unroll
      for (int s2 = 1; s2 < LPT; s2 <<= 1) {
        uint32_t o = __shfl_up(inc, s2, LPT);
        if (q >= s2) inc += o;
      }
      const uint32_t before = carry + inc - c, after = carry + inc;
      const uint32_t mm = before / 32u + 1u;
      if (c != 0u && mm < (uint32_t)LPT && 32u * mm <= after)
        ustart[tau * LPT + mm] = ub + 32u * j + select_bit(w, 32u * mm - before - 1u) + 1u;
      carry += __shfl(inc, LPT - 1, LPT);
    }
    ok = ok && carry == (uint32_t)N;
    __syncthreads();

    // ---- parse and rebuild block by block: remainder and unary readers
    // advance together; each block becomes lattice point (- dither) * step ----
    float a[kLaneElems];
    bool lane_ok = ok;
    {
      const float s = active ? as_f((uint32_t)step[t] << 16) : 0.0f;
      uint32_t cbits = 0;
      if constexpr (CB_LANE > 0) {
        if (ok) cbits = lds_read32(stage, start + (uint32_t)q * CB_LANE);
      }
      uint32_t rpk[8];
      UnaryReader ud;
      if (ok) {
        extract_remainders(stage, start + B + (uint32_t)q * kLaneElems * k, k, rpk);
        ud.init(stage, q == 0 ? ub : ustart[tau * LPT + q]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; j++) rpk[j] = 0u;
      }
#pragma unroll
      for (int b = 0; b < BPL; b++) {
        uint32_t u[D];
#pragma unroll
        for (int i = 0; i < D; i++) {
          const int e = b * D + i;
          uint32_t qv = 0;
          if (ok) {
            if ((e & 7) == 0) ud.refill();
            qv = ud.next(end);
          }
          const uint32_t r = (rpk[e >> 2] >> (8 * (e & 3))) & 0xFFu;
          if (qv > 0xFFFFu) lane_ok = false;
          const uint32_t uu = (qv << k) | r;
          if (uu > 0xFFFFu) lane_ok = false;
          u[i] = uu;
        }
        float pt[D];
        block_point<LAT>(u, (cbits >> b) & 1u, pt, a2);
        if constexpr (DITHER) {
          float du[D];
          dither_block<LAT>(key_dither, (uint32_t)(t * N) + (uint32_t)(q * kLaneElems + b * D), du, a2);
#pragma unroll
          for (int i = 0; i < D; i++) pt[i] = pt[i] - du[i];
        }
#pragma unroll
        for (int i = 0; i < D; i++) a[b * D + i] = pt[i] * s;
      }
      if (ok && q == LPT - 1 && ud.pos != end) lane_ok = false;   // the last one ends the tile
    }
    // tile-wide AND; every lane takes part in the shuffles (no short-circuit)
    int all_ok = lane_ok ? 1 : 0;
#pragma unroll
    for (int s2 = 1; s2 < LPT; s2 <<= 1) all_ok &= __shfl_xor(all_ok, s2);
    lane_ok = all_ok != 0;

    // ---- inverse RHT and store (an invalid tile decodes to zeros) ----
    if (active) {
      if (!lane_ok) {
        if (q == 0) atomicOr(status, HQ_FLAG_CORRUPT);
#pragma unroll
        for (int i = 0; i < kLaneElems; i++) a[i] = 0.0f;
      }
      fwht_tile_signed<LPT>(a, q);
      // lane q holds (-1)^popcount(q) times the butterfly output: fold that
      // sign into the scale; + 0.0f turns a -0 into +0 (every zero of the
      // exact butterfly is +0), then apply the sign diagonal
#pragma unroll
      for (int i = 0; i < kLaneElems; i++) {
        const float o = a[i] * lane_scale + 0.0f;
        a[i] = as_f(as_u(o) ^ (((sgn >> i) & 1u) << 31));
      }
      const uint64_t base = t * N + (uint64_t)q * kLaneElems;
      if constexpr (BF16) {
        uint4* p = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + base);
#pragma unroll
        for (int v = 0; v < 4; v++) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; h++)
            w[h] = bf16_rne_bits(a[v * 8 + 2 * h]) | (bf16_rne_bits(a[v * 8 + 2 * h + 1]) << 16);
          p[v] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
        float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + base);
#pragma unroll
        for (int v = 0; v < 8; v++) p[v] = make_float4(a[v * 4], a[v * 4 + 1], a[v * 4 + 2], a[v * 4 + 3]);
      }
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------
// Host side
// --------------------------------------------------------------------------
uint32_t lattice_dim(uint32_t lat) {
  switch (lat) { case HQ_Z: return 1; case HQ_A2: return 2; case HQ_D4: return 4; case HQ_E8: return 8; }
  return 0;
}

uint32_t host_pcg(uint32_t v) {
  uint32_t state = v * 747796405u + 2891336453u;
  uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}
// stream keys of the sign diagonal ("SIGN") and of the dither ("DITH")
uint32_t derive_key(uint64_t seed, uint32_t domain) {
  return host_pcg(host_pcg((uint32_t)(seed & 0xFFFFFFFFu) ^ domain) ^ (uint32_t)(seed >> 32));
}

bool rate_constant(uint32_t lat, uint32_t tile, uint32_t dither, float bps, float* c) {
  float q4 = bps * 4.0f;
  if (!(q4 == floorf(q4))) return false;
  uint32_t bq = (uint32_t)q4;
  for (const RateEntry& e : kRateTable) {
    if (e.lattice == lat && e.tile == tile && e.dither == dither && e.bps_q == bq) {
      memcpy(c, &e.c_bits, 4);
      return true;
    }
  }
  return false;
}

// Worst-case tile length: |t|_2 <= sqrt(n)/c' (c' = c less the bf16 rounding
// margin), so sum|t_i| <= n/c'; every code integer is within 3/2 of its t_i,
// so the symbols sum to at most 2n/c' + 3n (+2n with the dither); the chosen
// k codes at most as long as any fixed k.
uint32_t tile_bound_bits(uint32_t n, uint32_t lat, uint32_t dither, float c) {
  double cp = (double)c * (1.0 - 1.0 / 128.0);
  double S = 2.0 * n / cp + 3.0 * n + (dither ? 2.0 * n : 0.0);
  double best = 1e300;
  for (int k = 0; k < 8; k++) {
    double L = floor(S / (double)(1u << k)) + (double)n * (1 + k);
    if (L < best) best = L;
  }
  uint32_t d = lattice_dim(lat);
  double B = (lat == HQ_E8 || lat == HQ_A2) ? (double)(n / d) : 0.0;
  double bound = B + best;
  return bound > 8191.0 ? 0u : (uint32_t)bound;
}

struct Plan {
  uint64_t T, C, cap_words, ws_bytes;
  uint32_t bound, stage_words;
  float c;
};

int make_plan(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lat, float bps,
              uint32_t kv, Plan* P) {
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_EINVAL;
  if (tile != 64 && tile != 128 && tile != 256) return HQ_EINVAL;
  if (!lattice_dim(lat) || kv > 1) return HQ_EINVAL;
  if (rows == 0 || cols == 0 || cols % tile) return HQ_EINVAL;
  if (rows > (1ull << 32) || cols > (1ull << 32) || rows * cols >= (1ull << 32)) return HQ_EINVAL;
  float c;
  if (!rate_constant(lat, tile, kv, bps, &c)) return HQ_EINVAL;
  uint32_t bound = tile_bound_bits(tile, lat, kv, c);
  if (!bound) return HQ_EINVAL;
  P->T = rows * cols / tile;
  P->C = (P->T + kChunkTiles - 1) / kChunkTiles;
  P->bound = bound;
  P->c = c;
  P->stage_words = (uint32_t)(((uint64_t)kChunkTiles * bound + 31) / 32) + 4;
  P->cap_words = (P->T * bound + 31) / 32 + P->C;
  P->ws_bytes = 8 + 8 * P->C;
  return HQ_OK;
}

// ---- dispatch tables -------------------------------------------------------
using EncFn = void (*)(const void*, uint64_t, uint64_t, float, float, float, uint32_t, uint32_t, A2Consts,
                       uint32_t*, uint64_t, uint16_t*, uint16_t*, uint32_t*, uint32_t*, uint32_t*, uint32_t);
using DecFn = void (*)(const uint32_t*, uint64_t, const uint16_t*, const uint16_t*, const uint32_t*, uint64_t,
                       uint64_t, float, uint32_t, uint32_t, A2Consts, void*, uint32_t*, uint32_t, uint32_t, uint32_t);

template <int LAT, int N>
EncFn enc_pick(bool bf16, bool dither) {
  if (bf16) return dither ? encode_kernel<LAT, N, true, true> : encode_kernel<LAT, N, true, false>;
  return dither ? encode_kernel<LAT, N, false, true> : encode_kernel<LAT, N, false, false>;
}
template <int LAT, int N>
DecFn dec_pick(bool bf16, bool dither) {
  if (bf16) return dither ? decode_kernel<LAT, N, true, true> : decode_kernel<LAT, N, true, false>;
  return dither ? decode_kernel<LAT, N, false, true> : decode_kernel<LAT, N, false, false>;
}
template <int LAT>
EncFn enc_by_tile(uint32_t n, bool bf16, bool dither) {
  if (n == 64) return enc_pick<LAT, 64>(bf16, dither);
  if (n == 128) return enc_pick<LAT, 128>(bf16, dither);
  return enc_pick<LAT, 256>(bf16, dither);
}
template <int LAT>
DecFn dec_by_tile(uint32_t n, bool bf16, bool dither) {
  if (n == 64) return dec_pick<LAT, 64>(bf16, dither);
  if (n == 128) return dec_pick<LAT, 128>(bf16, dither);
  return dec_pick<LAT, 256>(bf16, dither);
}
EncFn enc_fn(uint32_t lat, uint32_t n, bool bf16, bool dither) {
  switch (lat) {
    case HQ_Z: return enc_by_tile<1>(n, bf16, dither);
    case HQ_A2: return enc_by_tile<2>(n, bf16, dither);
    case HQ_D4: return enc_by_tile<4>(n, bf16, dither);
    default: return enc_by_tile<8>(n, bf16, dither);
  }
}
DecFn dec_fn(uint32_t lat, uint32_t n, bool bf16, bool dither) {
  switch (lat) {
    case HQ_Z: return dec_by_tile<1>(n, bf16, dither);
    case HQ_A2: return dec_by_tile<2>(n, bf16, dither);
    case HQ_D4: return dec_by_tile<4>(n, bf16, dither);
    default: return dec_by_tile<8>(n, bf16, dither);
  }
}

int grid_for(const void* fn, int block, size_t lds, uint64_t chunks, int* grid) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HQ_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return HQ_EHIP;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, block, lds) != hipSuccess) return HQ_EHIP;
  if (per < 1) return HQ_EINVAL;
  uint64_t g = (uint64_t)cus * (uint64_t)per;
  if (g > chunks) g = chunks;
  *grid = (int)(g < 1 ? 1 : g);
  return HQ_OK;
}

int do_encode(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lat,
              float bps, uint64_t seed, uint32_t kv, uint32_t* payload, uint64_t cap, uint16_t* step,
              uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* ws, uint64_t ws_bytes,
              void* stream) {
  Plan P;
  int rc = make_plan(dtype, rows, cols, tile, lat, bps, kv, &P);
  if (rc) return rc;
  if (!x || !payload || !step || !meta || !chunk_off || !status || !ws) return HQ_EINVAL;
  if (cap < P.cap_words || ws_bytes < P.ws_bytes) return HQ_ENOSPC;
  if (((uintptr_t)x & 15) || ((uintptr_t)ws & 7)) return HQ_EINVAL;
  EncFn fn = enc_fn(lat, tile, dtype == HQ_BF16, kv != 0);
  const int block = kChunkTiles * (int)(tile / kLaneElems);
  const size_t lds = (size_t)(P.stage_words + 2 * kChunkTiles + 4) * 4;
  int grid;
  rc = grid_for((const void*)fn, block, lds, P.C, &grid);
  if (rc) return rc;
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  const float inv_sqrtn = (float)(1.0 / sqrt((double)tile));
  const float inv_n = 1.0f / (float)tile;   // exact: tile is a power of two
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, (hipStream_t)stream, x, P.T, P.C, P.c, inv_sqrtn, inv_n,
                     derive_key(seed, 0x5349474Eu), derive_key(seed, 0x44495448u), a2, payload, cap, step, meta,
                     chunk_off, status, (uint32_t*)ws, P.stage_words);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

int do_decode(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
              const uint32_t* chunk_off, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
              uint32_t lat, float bps, uint64_t seed, uint32_t kv, void* out, uint32_t* status, void* stream) {
  Plan P;
  int rc = make_plan(dtype, rows, cols, tile, lat, bps, kv, &P);
  if (rc) return rc;
  if (!payload || !step || !meta || !chunk_off || !status || !out) return HQ_EINVAL;
  if ((uintptr_t)out & 15) return HQ_EINVAL;
  DecFn fn = dec_fn(lat, tile, dtype == HQ_BF16, kv != 0);
  const uint32_t lpt = tile / kLaneElems;
  const uint32_t tpw = (256 / lpt) < (uint32_t)kChunkTiles ? 256 / lpt : (uint32_t)kChunkTiles;
  const int block = (int)(tpw * lpt);
  const uint32_t chunk_cap = (uint32_t)(((uint64_t)kChunkTiles * P.bound + 31) / 32);
  // a unit's bits start anywhere in a word: one extra word, plus the readers' guard
  const uint32_t stage_words = (uint32_t)(((uint64_t)tpw * P.bound + 31) / 32) + 1 + 4;
  const size_t lds = (size_t)(stage_words + 2 * kChunkTiles + tpw * lpt + 4) * 4;
  int grid;
  rc = grid_for((const void*)fn, block, lds, P.C * (kChunkTiles / tpw), &grid);
  if (rc) return rc;
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  const float inv_sqrtn = (float)(1.0 / sqrt((double)tile));
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, (hipStream_t)stream, payload, payload_words, step, meta,
                     chunk_off, P.T, P.C, inv_sqrtn, derive_key(seed, 0x5349474Eu),
                     derive_key(seed, 0x44495448u), a2, out, status, stage_words, chunk_cap, P.bound);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

int hq_plan(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice, float bps,
            uint32_t kv, uint64_t* tiles, uint64_t* chunks, uint64_t* payload_cap_words,
            uint64_t* workspace_bytes, uint32_t* tile_bound, float* rate_c) {
  Plan P;
  int rc = make_plan(dtype, rows, cols, tile, lattice, bps, kv, &P);
  if (rc) return rc;
  if (tiles) *tiles = P.T;
  if (chunks) *chunks = P.C;
  if (payload_cap_words) *payload_cap_words = P.cap_words;
  if (workspace_bytes) *workspace_bytes = P.ws_bytes;
  if (tile_bound) *tile_bound = P.bound;
  if (rate_c) *rate_c = P.c;
  return HQ_OK;
}

int hq_encode(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
              float bps, uint64_t seed, uint32_t* payload, uint64_t payload_cap_words, uint16_t* step,
              uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* workspace,
              uint64_t workspace_bytes, void* stream) {
  return do_encode(x, dtype, rows, cols, tile, lattice, bps, seed, 0, payload, payload_cap_words, step, meta,
                   chunk_off, status, workspace, workspace_bytes, stream);
}

int hq_decode(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
              const uint32_t* chunk_off, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
              uint32_t lattice, float bps, uint64_t seed, void* x_out, uint32_t* status, void* stream) {
  return do_decode(payload, payload_words, step, meta, chunk_off, dtype, rows, cols, tile, lattice, bps, seed,
                   0, x_out, status, stream);
}

int hq_kv_encode(const void* x, uint32_t dtype, uint64_t tokens, uint32_t head_dim, uint32_t lattice,
                 float bps, uint64_t seed, uint32_t* payload, uint64_t payload_cap_words, uint16_t* step,
                 uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* workspace,
                 uint64_t workspace_bytes, void* stream) {
  return do_encode(x, dtype, tokens, head_dim, head_dim, lattice, bps, seed, 1, payload, payload_cap_words,
                   step, meta, chunk_off, status, workspace, workspace_bytes, stream);
}

int hq_kv_decode(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
                 const uint32_t* chunk_off, uint32_t dtype, uint64_t tokens, uint32_t head_dim,
                 uint32_t lattice, float bps, uint64_t seed, void* x_out, uint32_t* status, void* stream) {
  return do_decode(payload, payload_words, step, meta, chunk_off, dtype, tokens, head_dim, head_dim, lattice,
                   bps, seed, 1, x_out, status, stream);
}

const char* hq_strerror(int code) {
  switch (code) {
    case HQ_OK: return "ok";
    case HQ_EINVAL: return "invalid argument (shape, tile, lattice, dtype, bps or alignment)";
    case HQ_EHIP: return "HIP runtime or launch error";
    case HQ_ENOSPC: return "buffer capacity below the planned size";
    case HQ_ENONFINITE: return "non-finite input";
    case HQ_ECORRUPT: return "corrupt compressed stream";
  }
  return "unknown error";
}

uint32_t hq_version(void) { return (1u << 16) | 0u; }

}  // extern "C"
