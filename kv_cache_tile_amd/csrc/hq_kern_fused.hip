// hq_kern_fused.hip — the int8 product read straight from the compressed
// stream, in one launch (gist.science explainer of HyperQuant, "Significance
// and Claims": decoding fused with the matrix product is the route to a
// wall-clock gain; Key Contributions, "Hardware Integration": int8 matrix-core
// products on the post-RHT lattice output).
//
// A weight row times an activation x is the sum over the row's tiles of
// s_t <P_t, RHT(x)_t> (the weight tile decodes to D H (s P) / sqrt(n)).  With
// the activation tiles quantized to int8 (act_quant_kernel) and the codes 2P
// of a tile (integers for Z, D4 and E8):
//   y[b][r] = 0.5 * fma chain over tiles t ascending, from +0, of
//             (float) I_t * fl(s_t * a_t),   I_t = <2P_t, q_t> (exact int32),
// the same value as the two-pass path, without its int8 code tensor or its
// int32 scratch in HBM.
//
// A workgroup owns ROWS = 8 weight rows and walks their tiles in ascending
// column order, TC = 8 columns at a time (a unit of 64 tiles, LPT lanes a
// tile as in the decoder).  Each row is a whole number of 64-tile chunks of
// the stream; entering a chunk column, one wave per row checks the chunk
// (the decoder's rules) and scans its tile lengths, and the column's
// activation scales are staged.  Per unit:
//   1. the unit's bits (8 contiguous runs, one per row) stream into one of
//      two LDS buffers, the next unit's during this unit's work;
//   2. each tile's lanes find their first unary code and parse their 32
//      codes (the decoder's reader, parse_codes) straight to the integers
//      2P, saturated to int8 in LDS;
//   3. one wave per tile column forms the 8 rows x 32 activations of int32
//      products with v_mfma_i32_32x32x32_i8 (rows 8..31 of the operand are
//      zero; the activation operand read from hq_act_quant_blocked's layout,
//      1 KB of contiguous memory a load), written to LDS;
//   4. each (activation b, row j) takes the unit's chain steps in order, in
//      registers of one thread.
#include "hq_kernels.h"

namespace hq {

typedef int fz_i32x16 __attribute__((ext_vector_type(16)));
typedef int fz_i32x4 __attribute__((ext_vector_type(4)));

constexpr int kFusedRows = 8;      // weight rows per workgroup
constexpr int kFusedCols = 8;      // tile columns per unit
constexpr int kFusedBatch = 32;    // activations per launch row of workgroups

// Tile products live in the codes rows of their column once the column's
// products are formed (n >= 128: a column's rows hold 2n >= 256 words);
// at n = 64 they have a buffer of their own.
template <int N>
constexpr bool kProductsInCodes = N >= 128;

template <int LAT, int N>
__global__ void __launch_bounds__(kFusedRows * kFusedCols * (N / kLaneElems))
fused_product_kernel(const uint32_t* __restrict__ payload, uint64_t payload_words,
                     const uint16_t* __restrict__ step, const uint16_t* __restrict__ meta,
                     const uint32_t* __restrict__ chunk_off, uint64_t rows, uint32_t tpr,
                     const int8_t* __restrict__ qa, const float* __restrict__ scale, uint64_t batch,
                     float* __restrict__ y, uint32_t* __restrict__ status, uint32_t seg_words,
                     uint32_t chunk_cap_words, uint32_t tile_bound) {
  constexpr int LPT = N / kLaneElems;
  constexpr int ROWS = kFusedRows, TC = kFusedCols, TPW = ROWS * TC;
  constexpr int THREADS = TPW * LPT, WAVES = THREADS / 64;
  constexpr int D = LatticeTraits<LAT>::dim;
  constexpr int BPL = kLaneElems / D;
  constexpr uint32_t CB_LANE = LatticeTraits<LAT>::coset * BPL;
  constexpr uint32_t B = CB_LANE * LPT;
  static_assert(LAT != 2, "integer codes: Z, D4 or E8");
  static_assert(WAVES >= 2, "at least two waves");
  static_assert(ROWS == 8, "the products buffer holds rows in two 16-byte halves");

  // LDS; row strides padded against bank conflicts (MS: one word; CRS: two
  // 16-byte vectors) and each tile's 32-byte code chunks rotated by its column
  constexpr int MS = kChunkTiles + 1;                       // words per row of the tile tables
  constexpr int CRS = TC * N / 4 + 8;                       // words per row of codes
  extern __shared__ uint32_t smem[];
  uint32_t* stage0 = smem;                                  // [2][ROWS][seg_words] units' bits + guard
  uint32_t* toff = stage0 + 2 * ROWS * seg_words;           // [ROWS][MS] tile bit offsets in the chunk
  uint32_t* tms = toff + ROWS * MS;                         // [ROWS][MS] meta | step << 16
  uint32_t* tok = tms + ROWS * MS;                          // [ROWS][MS] tile valid
  uint32_t* cinfo = tok + ROWS * MS;                        // [ROWS][4] chunk's first word (lo, hi), valid
  uint32_t* adj = cinfo + 4 * ROWS;                         // [2][ROWS] stage bit of a chunk's bit 0
  float* sscale = reinterpret_cast<float*>(adj + 2 * ROWS);  // [TC][32] activation scales of the unit
  uint32_t* ustart = reinterpret_cast<uint32_t*>(sscale + kFusedBatch * TC);   // [THREADS]
  uint32_t* codes = ustart + THREADS;                       // [ROWS][CRS] int8 codes 2P
  int32_t* ibuf = reinterpret_cast<int32_t*>(codes + ROWS * CRS);   // [TC][32][ROWS] tile products (n = 64)
  // word of the product (activation b, row j) of column c: in the column's
  // codes rows, row segment b % 8 at (b / 8) 8 + j, the row halves swapped
  // for b / 8 odd (n >= 128); else in ibuf, (c 32 + b) 8 + j, halves swapped
  // the same way.  Either way a 16-byte store of a row half by 16 lanes, and
  // a word read by 64 lanes, find distinct banks.
  auto prod_word = [&](int c, int b, int j) -> int32_t* {
    const int js = (((j >> 2) ^ ((b >> 3) & 1)) << 2) | (j & 3);
    if constexpr (kProductsInCodes<N>)
      return reinterpret_cast<int32_t*>(codes) + (b & 7) * CRS + c * (N / 4) + (b >> 3) * 8 + js;
    else
      return ibuf + (c * kFusedBatch + b) * ROWS + js;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tau = tid / LPT;                                // tile of the unit
  const int p_lane = tid % LPT;
  const int q = tile_lane<LPT>(p_lane);                     // logical lane
  // tiles column-major in the unit: wave w holds the CPW whole columns
  // w CPW .. w CPW + CPW - 1 (all ROWS rows), which it also multiplies
  constexpr int CPW = TC / WAVES;
  static_assert(CPW * WAVES == TC && ROWS * LPT * CPW == 64, "a wave holds whole columns");
  const int jrow = tau % ROWS, tcol = tau / ROWS;           // its row and column in the unit
  const uint64_t r0 = (uint64_t)blockIdx.x * ROWS;
  const uint64_t b0 = (uint64_t)blockIdx.y * kFusedBatch;
  const uint32_t cpr = tpr / kChunkTiles;                   // chunks per row
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // chain accumulators: pair e = tid + i THREADS is (activation e / ROWS, row e % ROWS)
  constexpr int PAIRS = ROWS * kFusedBatch, CPT = (PAIRS + THREADS - 1) / THREADS;
  float acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; i++) acc[i] = 0.0f;

  // start streaming the bits of the unit at column tn into buffer buf: wave
  // w takes rows w, w + waves, ...; a row's run of words, from the 16-byte
  // vector holding its first bit, goes straight to LDS (the stream's last,
  // partial vector by plain loads), with eight zero guard words after it
  auto stage_in = [&](uint32_t tn, int buf) {
    const uint32_t pn = tn % kChunkTiles;
    for (int j = wave; j < ROWS; j += WAVES) {
      const bool cok = __builtin_amdgcn_readfirstlane(cinfo[4 * j + 2]) != 0u;
      const uint32_t first = __builtin_amdgcn_readfirstlane(toff[j * MS + pn]);
      const uint32_t lastm = __builtin_amdgcn_readfirstlane(tms[j * MS + pn + TC - 1]) & 0xFFFFu;
      const uint32_t endb = __builtin_amdgcn_readfirstlane(toff[j * MS + pn + TC - 1]) + (lastm >> 3);
      const uint64_t cw0 = ((uint64_t)__builtin_amdgcn_readfirstlane(cinfo[4 * j + 1]) << 32) |
                           __builtin_amdgcn_readfirstlane(cinfo[4 * j]);
      const uint64_t L = (cw0 + (first >> 5)) & ~3ull;
      const uint32_t nvec = cok ? (uint32_t)((cw0 + ((endb + 31u) >> 5) - L + 3u) >> 2) : 0u;
      const uint32_t segw = (uint32_t)(buf * ROWS + j) * seg_words;
      uint32_t* seg = stage0 + segw;
      for (uint32_t v0 = 0; v0 < nvec; v0 += 64) {
        const uint32_t v = v0 + (uint32_t)lane;
        if (v < nvec) {
          const uint64_t g = L + 4ull * v;
          if (g + 4u <= payload_words) {
            lds_load16(payload + L, 16u * v, smem_lds + 4u * (segw + 4u * v0));
          } else {
#pragma unroll
            for (int e = 0; e < 4; e++) seg[4u * v + (uint32_t)e] = g + (uint64_t)e < payload_words ? payload[g + e] : 0u;
          }
        }
      }
      if (lane < 8) seg[4u * nvec + (uint32_t)lane] = 0u;
      if (lane == 0) adj[buf * ROWS + j] = segw * 32u + (uint32_t)(32 * ((int64_t)cw0 - (int64_t)L));
    }
  };

  int cur = 0;
  for (uint32_t t0 = 0; t0 < tpr; t0 += TC, cur ^= 1) {
    const uint32_t p0 = t0 % kChunkTiles;                   // the unit's first position in its chunk
    if (p0 == 0) {
      // a new chunk column: wave w checks rows w, w + waves, ...: each chunk
      // and its tile offsets; every thread loads a share of the column's
      // activation scales
      __syncthreads();                                      // (the previous unit's reads are done)
      for (int wr = wave; wr < ROWS; wr += WAVES) {
        const uint64_t row = r0 + (uint64_t)wr;
        const bool exists = row < rows;
        const uint64_t c = exists ? row * cpr + t0 / kChunkTiles : 0;
        const uint32_t mt = exists ? meta[c * kChunkTiles + lane] : 0u;
        const uint32_t st = exists ? step[c * kChunkTiles + lane] : 0u;
        const uint32_t len = mt >> 3, kk = mt & 7u;
        const uint32_t inc = wave_incl_scan(len);
        toff[wr * MS + lane] = inc - len;
        const uint32_t total = __builtin_amdgcn_readlane(inc, kChunkTiles - 1);
        const uint64_t pw0 = exists ? chunk_off[c] : 0, pw1 = exists ? chunk_off[c + 1] : 0;
        const bool range_ok = pw1 >= pw0 && pw1 <= payload_words && (pw1 - pw0) <= chunk_cap_words;
        const bool too_long = wave_any(len > tile_bound);
        const bool chunk_ok = exists && range_ok && !too_long && (uint64_t)((total + 31u) >> 5) == pw1 - pw0;
        tok[wr * MS + lane] =
            (chunk_ok && len >= B + (uint32_t)N * (kk + 1u) && (st == 0u || st - 0x180u < 0x7E00u)) ? 1u : 0u;
        tms[wr * MS + lane] = mt | (st << 16);
        if (lane == 0) {
          cinfo[4 * wr] = (uint32_t)pw0;
          cinfo[4 * wr + 1] = (uint32_t)(pw0 >> 32);
          cinfo[4 * wr + 2] = chunk_ok ? 1u : 0u;
        }
      }
      __syncthreads();
      stage_in(t0, cur);                                    // (the first unit of the column: not ahead)
    }
    // this unit's bits have landed (each wave waits for its own loads, the
    // barrier for everyone's); then the next unit's, if in this column, start
    // streaming into the other buffer during this unit's parse
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the unit's activation scales stream into LDS (sscale[c 32 + b]; an
    // activation past the batch reads activation 0's, and its chain is never
    // stored), read by the chain after the unit's products
    for (int i0 = wave * 64; i0 < TC * kFusedBatch; i0 += WAVES * 64) {
      const uint32_t i = (uint32_t)(i0 + lane);
      const uint64_t bb = b0 + (uint64_t)(i % kFusedBatch);
      const uint64_t src = (bb < batch ? bb : 0) * tpr + t0 + i / kFusedBatch;
      lds_load4(scale, (uint32_t)(4 * src), smem_lds + 4u * (uint32_t)((sscale - reinterpret_cast<float*>(smem)) + i0));
    }
    if (t0 + TC < tpr && (t0 + TC) % kChunkTiles != 0) stage_in(t0 + TC, cur ^ 1);
    const uint32_t* stage = stage0;

    // ---- parse: the tile of (row jrow, column tcol) ----
    const uint32_t pos = p0 + (uint32_t)tcol;
    const uint32_t ms = tms[jrow * MS + pos];
    const uint32_t len = (ms & 0xFFFFu) >> 3, k = ms & 7u;
    bool ok = tok[jrow * MS + pos] != 0u && r0 + (uint64_t)jrow < rows;
    const uint32_t start = adj[cur * ROWS + jrow] + toff[jrow * MS + pos];
    const uint32_t end = start + len;
    const uint32_t ub = start + B + (uint32_t)N * k;        // unary plane
    // where each lane's first unary code starts (the decoder's search: ones
    // counted over the aligned words of the unary plane, the (32 q)-th one
    // recorded for lane q)
    constexpr uint32_t kUW = 3;
    const uint32_t a0 = ub >> 5;
    const uint32_t nwu = ok ? ((end - 1u) >> 5) - a0 + 1u : 0u;
    const uint32_t lo_mask = ~0u << (ub & 31u);
    const uint32_t hi_keep = end & 31u;
    uint32_t carry = 0;
    for (uint32_t r = 0;; r++) {
      const bool more = r * kUW * (uint32_t)LPT < nwu;
      if (!wave_any(more)) break;
      const uint32_t j0 = (r * (uint32_t)LPT + (uint32_t)p_lane) * kUW;
      uint32_t c[kUW], cs = 0;
#pragma unroll
      for (uint32_t i = 0; i < kUW; i++) {
        const uint32_t j = j0 + i;
        uint32_t x = j < nwu ? stage[a0 + j] : 0u;
        if (j == 0u) x &= lo_mask;
        if (j + 1u == nwu && hi_keep != 0u) x &= (1u << hi_keep) - 1u;
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

    CodesSink<LAT> csink;
    bool lane_ok;
    {
      uint32_t cbits = 0;
      if constexpr (CB_LANE > 0) cbits = lds_read32(stage, ok ? start + (uint32_t)q * CB_LANE : 0u);
      const uint32_t rb = ok ? start + B + (uint32_t)q * kLaneElems * k : 0u;
      uint32_t u0 = ub;
      if (q != 0) {
        const uint32_t rec = ok ? ustart[tau * LPT + q] : 0u;
        const uint32_t wa = rec >> 5;
        uint32_t x = stage[wa];
        if (wa == a0) x &= lo_mask;
        u0 = 32u * wa + select_bit(x, rec & 31u) + 1u;
      }
      u0 = ok ? u0 : 0u;
      const uint32_t lim = ok ? end : 0u;
      uint32_t upos = 0;
      bool pok;
      switch (k) {
#define HQ_FPARSE_CASE(KK) \
        case KK: pok = parse_codes<LAT, KK>(stage, rb, u0, lim, cbits, csink, upos); break;
        HQ_FPARSE_CASE(0) HQ_FPARSE_CASE(1) HQ_FPARSE_CASE(2) HQ_FPARSE_CASE(3)
        HQ_FPARSE_CASE(4) HQ_FPARSE_CASE(5) HQ_FPARSE_CASE(6)
        default: pok = parse_codes<LAT, 7>(stage, rb, u0, lim, cbits, csink, upos); break;
#undef HQ_FPARSE_CASE
      }
      lane_ok = ok && pok;
      if (q == LPT - 1 && upos != end) lane_ok = false;
    }
    int all_ok = lane_ok ? 1 : 0;
#pragma unroll
    for (int s2 = 1; s2 < LPT; s2 <<= 1) all_ok &= (int)lane_xor((uint32_t)all_ok, partner_xor<LPT>(s2));
    lane_ok = all_ok != 0;

    // the tile's codes 2P (exact integers), saturated to int8; an invalid
    // tile's codes are zeros
    {
      const bool real = r0 + (uint64_t)jrow < rows;
      if (real && !lane_ok && q == 0) atomicOr(status, HQ_FLAG_CORRUPT);
      uint32_t w[8];
#pragma unroll
      for (int v = 0; v < 8; v++) w[v] = lane_ok ? csink.w[v] : 0u;
      if (real && lane_ok && csink.over()) atomicOr(status, HQ_FLAG_RANGE);
      uint4* dst = reinterpret_cast<uint4*>(codes + jrow * CRS + tcol * (N / 4) + ((q + tcol) % LPT) * 8);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }

    // ---- the tile products on the matrix cores: each wave takes the columns
    // it parsed (no block barrier); operand A = codes (lane l: row l % 32, zero past ROWS),
    // B = activations (lane l: activation l % 32), 16 bytes each at the
    // 16-byte half l / 32 of every 32-code step; output register i of lane l
    // holds row (i / 4) 8 + (l / 32) 4 + i % 4, activation l % 32. ----
    wave_lds_sync();                                        // (this wave's columns' codes are in LDS)
    constexpr int KS = N / 32;
    const fz_i32x4 zero4 = {0, 0, 0, 0};
    const int half = (lane >> 5) * 16;
    const uint64_t bbl = b0 + (uint64_t)(lane & 31);
    for (int cc = 0; cc < CPW; cc++) {
      const int c = wave * CPW + cc;
      const uint32_t t = t0 + (uint32_t)c;
      const int arow = lane & 31;
      // the activations' 32-code steps of tile t, 1 KB each (the blocked layout)
      const int8_t* bstep = qa + ((uint64_t)blockIdx.y * tpr + t) * (uint64_t)(KS * 1024) + (lane & 31) * 32 + half;
      fz_i32x4 bv[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        bv[ks] = bbl < batch ? *reinterpret_cast<const fz_i32x4*>(bstep + 1024 * ks) : zero4;
      fz_i32x16 I = {};
#pragma unroll
      for (int ks = 0; ks < N / 32; ks++) {
        const fz_i32x4 av = arow < ROWS
            ? *reinterpret_cast<const fz_i32x4*>(codes + arow * CRS + c * (N / 4) + ((ks + c) % LPT) * 8 + half / 4)
            : zero4;
        I = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv[ks], I, 0, 0, 0);
      }
      // rows 4h .. 4h + 3 of activation b as one 16-byte store (the column's
      // codes are read: each MFMA above waited for its operands)
      *reinterpret_cast<fz_i32x4*>(prod_word(c, lane & 31, (lane >> 5) * 4)) = fz_i32x4{I[0], I[1], I[2], I[3]};
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");        // (this wave's scale loads)
    __syncthreads();

    // ---- 4. the chain steps of the unit, in column order ----
#pragma unroll
    for (int i = 0; i < CPT; i++) {
      const int e = tid + i * THREADS;
      if (e < PAIRS) {
        const int cb = e / ROWS, cj = e % ROWS;
#pragma unroll
        for (int c = 0; c < TC; c++) {
          const float s = as_f((tms[cj * MS + p0 + c] >> 16) << 16);
          const float av = sscale[c * kFusedBatch + cb];
          acc[i] = __builtin_fmaf((float)*prod_word(c, cb, cj), s * av, acc[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; i++) {
    const int e = tid + i * THREADS;
    const uint64_t row = r0 + (uint64_t)(e % ROWS), bb = b0 + (uint64_t)(e / ROWS);
    if (e < PAIRS && row < rows && bb < batch) y[bb * rows + row] = 0.5f * acc[i];
  }
}

using FusedFn = void (*)(const uint32_t*, uint64_t, const uint16_t*, const uint16_t*, const uint32_t*, uint64_t,
                         uint32_t, const int8_t*, const float*, uint64_t, float*, uint32_t*, uint32_t, uint32_t,
                         uint32_t);

template <int LAT>
FusedFn fused_table(uint32_t n) {
  if (n == 64) return fused_product_kernel<LAT, 64>;
  if (n == 128) return fused_product_kernel<LAT, 128>;
  return fused_product_kernel<LAT, 256>;
}

// the fused product for (lattice, n), its threads and LDS bytes for a
// segment of seg_words (null for an unsupported lattice)
const void* fused_fn(uint32_t lattice, uint32_t n, uint32_t seg_words, uint32_t* threads, size_t* lds) {
  FusedFn f = lattice == 8 ? fused_table<8>(n) : lattice == 4 ? fused_table<4>(n) : lattice == 1 ? fused_table<1>(n)
                                                                                                   : nullptr;
  if (!f) return nullptr;
  const uint32_t th = (uint32_t)(kFusedRows * kFusedCols) * (n / kLaneElems);
  *threads = th;
  *lds = 4 * (2 * (size_t)kFusedRows * seg_words + 3 * kFusedRows * (kChunkTiles + 1) + 4 * kFusedRows +
              2 * kFusedRows + kFusedBatch * kFusedCols + th + (size_t)kFusedRows * (kFusedCols * n / 4 + 8) +
              (n >= 128 ? 0 : (size_t)kFusedCols * kFusedBatch * kFusedRows));
  return (const void*)f;
}

}  // namespace hq
