/*
 * hq.h — C ABI of the HyperQuant encode/decode library (libhq.so, HIP, gfx950).
 *
 * The library compresses a row-major 2-D tensor (LLM weights, or KV-cache
 * vectors) with the HyperQuant pipeline as described in "HyperQuant: A
 * Rate-Distortion-Optimal Quantization Pipeline for Large Language and
 * Diffusion Models" (gist.science explainer, section "Methodology: The
 * HyperQuant Pipeline"):
 *   1. per-tile Randomized Hadamard Transform  y = H_n D x / sqrt(n)  (tile n
 *      contiguous elements of a row, seeded sign diagonal D)        [Methodology 1]
 *   2. per-tile scale (step = bf16(RMS(y) * c(bps))) and nearest point of the
 *      E8 (D8 u D8+1/2), D4, A2 or Z lattice, block by block           [Methodology 2]
 *   3. lossless bit-stripping of the lattice code and Rice coding with one
 *      parameter k in 0..7 per tile (the shortest)                   [Methodology 3]
 *   4. KV variant: a subtractive dither U ~ Uniform(Voronoi cell), added
 *      before quantization and subtracted after, regenerated from the seed
 *      at decode; the sign diagonal is the per-layer rotation         [Methodology 4]
 * and the inverse (decode).
 *
 * Conventions
 *  - All tensor/buffer pointers are DEVICE pointers (hipMalloc'd or
 *    torch-owned); descriptors and sizes are host values.  `stream` is a
 *    hipStream_t passed as void* (NULL = default stream).  Every compute call
 *    but hq_encode_rate (which synchronises `stream` after each trial) is
 *    asynchronous on `stream`; buffers must stay alive until it is
 *    synchronised.  The library allocates no device memory and keeps no
 *    pointer after returning.
 *  - Return value: 0 (HQ_OK) or a negative hq_status for argument errors
 *    (synchronous, nothing launched) and HIP launch errors.  Data-dependent
 *    conditions found while the kernels run are OR-ed as HQ_FLAG_* bits into
 *    the device word *status (the caller zeroes it before the call and reads
 *    it after synchronising).
 *  - Input is never modified.
 *
 * Compressed layout (all produced by hq_encode, consumed by hq_decode):
 *  - T = rows*cols/tile tiles in row-major order; C = ceil(T/64) chunks.
 *  - step[T]      uint16 bf16 bits of the per-tile step (0 = zero tile)
 *  - meta[T]      uint16 (len << 3) | k : tile bit length and Rice parameter
 *  - chunk_off[C+1] uint32 word offset of each chunk in payload; last = total
 *  - payload[]    uint32 words; bit b of a chunk = bit (b & 31) of its word
 *                 b >> 5.  A tile is its coset bits (E8: n/8, A2: n/2) then n
 *                 Rice codewords (q zeros, a one, k remainder bits LSB first);
 *                 tiles are bit-contiguous within a chunk; each chunk starts
 *                 on a word and its tail bits are zero.
 */
#ifndef HQ_H
#define HQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HQ_OK = 0,
    HQ_EINVAL = -1,      /* bad shape, tile, lattice, dtype, or bps not on the rate grid */
    HQ_EHIP = -2,        /* HIP runtime / launch error */
    HQ_ENOSPC = -3,      /* a capacity argument is below what hq_plan reported */
    HQ_ENONFINITE = -4,  /* (status flag) non-finite input tile */
    HQ_ECORRUPT = -5     /* (status flag) inconsistent compressed stream */
} hq_status;

/* bits OR-ed into *status by the kernels */
#define HQ_FLAG_NONFINITE 1u   /* encode: a tile had a non-finite energy; it was coded as zero */
#define HQ_FLAG_CORRUPT   2u   /* decode: a tile's parsed length disagreed with meta (tile -> 0) */
#define HQ_FLAG_NOSPACE   4u   /* encode: payload capacity exceeded (nothing written past it) */
#define HQ_FLAG_RANGE     8u   /* decode to codes: a code 2P beyond [-127, 127] (saturated) */
#define HQ_FLAG_STALL    16u   /* encode: a chunk-offset look-back gave up waiting (about a
                                  second); the stream is not valid.  Not reached unless the
                                  device stops running the encode's workgroups. */

typedef enum { HQ_F32 = 0, HQ_BF16 = 1 } hq_dtype;
typedef enum { HQ_Z = 1, HQ_A2 = 2, HQ_D4 = 4, HQ_E8 = 8 } hq_lattice;

/*
 * hq_plan — host-only, synchronous.  Validates a configuration and returns
 * the sizes of the buffers the caller must allocate.
 *   dtype    HQ_F32 or HQ_BF16 (encode input and decode output element type)
 *   rows, cols  tensor shape, cols % tile == 0, rows*cols < 2^32
 *   tile     64, 128 or 256 (the RHT size n; the pages' example tile is 128,
 *            gist.science explainer of HyperQuant, Methodology section 1)
 *   lattice  HQ_Z, HQ_A2, HQ_D4, HQ_E8 (Methodology 2)
 *   bps      target payload bits per scalar on the grid 1.5, 1.75, ..., 8
 *            (the realized-rate claim of Methodology section 3)
 *   kv       0 for weights (hq_encode), 1 for the dithered KV variant
 * Outputs (any may be NULL): tiles T, chunks C, payload capacity in words
 * (worst case over all inputs), workspace bytes for hq_encode / hq_kv_encode,
 * the worst-case tile length in bits, and the rate constant c used.
 */
int hq_plan(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
            float bps, uint32_t kv,
            uint64_t *tiles, uint64_t *chunks, uint64_t *payload_cap_words,
            uint64_t *workspace_bytes, uint32_t *tile_bound_bits, float *rate_constant);

/*
 * hq_encode — weights.  Methodology 1-3.
 *   x          device, [rows][cols] of dtype, row-major, read only, 16-byte
 *              aligned
 *   seed       selects the sign diagonal D
 *   payload    device, payload_cap_words uint32 (>= hq_plan's capacity)
 *   step, meta device, T uint16 each
 *   chunk_off  device, C+1 uint32
 *   status     device, one uint32 (flags OR-ed in)
 *   workspace  device, 8-byte aligned, workspace_bytes (>= hq_plan's: 768 + 8 C)
 *              zero-filled ONCE before its first use; the kernels leave it
 *              ready for the next call.  Calls that overlap in time must not
 *              share a workspace.
 * The bit stream is a pure function of (x, shape, tile, lattice, bps, seed).
 * The encode's workgroups take groups of chunks in order (a first one each,
 * then from a counter in the workspace once all have started), and each
 * waits only for the chunk offsets of groups taken before its own, by
 * workgroups already running: it needs no part of its grid to be resident
 * at once, and may run next to any other kernel, other encodes included
 * (each with its own workspace).  A wait that lasts past about a second gives
 * up and sets HQ_FLAG_STALL.
 */
int hq_encode(const void *x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
              uint32_t lattice, float bps, uint64_t seed,
              uint32_t *payload, uint64_t payload_cap_words, uint16_t *step, uint16_t *meta,
              uint32_t *chunk_off, uint32_t *status, void *workspace, uint64_t workspace_bytes,
              void *stream);

/*
 * hq_decode — inverse of hq_encode: Rice parse, lattice point, step, inverse
 * RHT.  Same shape arguments and seed as the encode; writes x_out
 * ([rows][cols] of dtype, device, 16-byte aligned).  payload (device) is
 * 16-byte aligned; payload_words is at least chunk_off[C] of the stream (the
 * valid words; the buffer's capacity may be passed); reads never go beyond it.
 * Errors (HQ_EINVAL for a NULL or misaligned pointer, a bad shape or rate)
 * are returned before any device work; a stream inconsistent with its
 * metadata is not an error: its tiles decode to zero and HQ_FLAG_CORRUPT is
 * OR-ed into *status.
 */
int hq_decode(const uint32_t *payload, uint64_t payload_words, const uint16_t *step,
              const uint16_t *meta, const uint32_t *chunk_off,
              uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
              float bps, uint64_t seed, void *x_out, uint32_t *status, void *stream);

/*
 * hq_kv_encode / hq_kv_decode — KV cache (Methodology 4).  x is [tokens][head_dim]
 * (e.g. a [B, H, S, D] cache viewed as B*H*S rows), one tile per (token, head)
 * vector: tile = head_dim.  seed selects the per-layer sign diagonal and the
 * dither; the dither of coordinate g (row-major index in the call) is
 * regenerated at decode, so decode must use the same seed and shape.
 * Other arguments as hq_encode / hq_decode.
 */
int hq_kv_encode(const void *x, uint32_t dtype, uint64_t tokens, uint32_t head_dim,
                 uint32_t lattice, float bps, uint64_t seed,
                 uint32_t *payload, uint64_t payload_cap_words, uint16_t *step, uint16_t *meta,
                 uint32_t *chunk_off, uint32_t *status, void *workspace, uint64_t workspace_bytes,
                 void *stream);
int hq_kv_decode(const uint32_t *payload, uint64_t payload_words, const uint16_t *step,
                 const uint16_t *meta, const uint32_t *chunk_off,
                 uint32_t dtype, uint64_t tokens, uint32_t head_dim, uint32_t lattice,
                 float bps, uint64_t seed, void *x_out, uint32_t *status, void *stream);

/*
 * Closed-loop rate control (gist.science explainer of HyperQuant,
 * Methodology section 3: the realized rate lands within about 0.01 bits per
 * scalar of the target).  The table's constants c reach that on Gaussian
 * data; these calls take an explicit c, or search for the c at which a given
 * tensor's stored stream, 32 * chunk_off[C] / (rows * cols) bits per scalar
 * (coset and Rice bits plus each chunk's word alignment), is within 0.01 of
 * the target.
 *
 * hq_plan_c — as hq_plan, for an explicit rate constant c (finite, > 0).
 *   Returns HQ_EINVAL where c is so small that a tile could exceed 8191 bits.
 * hq_encode_c / hq_decode_c — as hq_encode / hq_decode (kv = 0) or
 *   hq_kv_encode / hq_kv_decode (kv = 1, then cols == tile == head_dim), with
 *   the step s = bf16(rms * c) of an explicit c.  A stream must be decoded
 *   with the c it was encoded with (the decoder sizes its staging from it).
 * hq_rate_bracket — host only.  The search interval for a target in [1, 8]
 *   bits per scalar: K 2^-(floor(R) + 3) and K 2^-(floor(R) - 2), where
 *   K = fl32(sqrt(2 pi e) V^(-1/d)) is the high-rate step constant of an
 *   entropy-coded lattice quantiser (V the covolume: Z 1, A2 sqrt3/2, D4 2,
 *   E8 1).
 * hq_encode_length_c — the length pass: adds to *words (a device uint64,
 *   8-byte aligned; the caller zeroes it first) the payload size in words,
 *   chunk_off[C], that hq_encode_c with the same arguments would produce,
 *   without writing a stream: the same per-tile steps, lattice points,
 *   symbols and Rice parameters, each chunk's tile lengths summed and
 *   rounded up to a word.  Asynchronous on `stream`; needs no workspace;
 *   sets no status flags (a non-finite tile counts as the zero tile the
 *   encoder writes).  Arguments and errors as hq_encode_c.
 * hq_encode_rate — synchronous: bisection on c over that bracket, at the
 *   geometric midpoint fl32(sqrt(lo * hi)); each trial is one length pass
 *   on `stream`, counting into workspace bytes 16..23, followed by an
 *   8-byte read and a stream synchronisation.  A trial with more bits than
 *   the target raises lo, one with fewer lowers hi.  It stops when the rate
 *   is within 0.01 of the target, when the midpoint equals an end of the
 *   interval (fp32 resolution), or after 30 trials, and then encodes the
 *   stream once, with hq_encode_c at *c_out (pass it to hq_decode_c): its
 *   rate is *bps_out bits per scalar, found after *encodes_out trials (the
 *   outputs may be NULL).  Buffers are sized by hq_plan_c at the bracket's
 *   low end (its tiles are the longest); smaller capacities and null or
 *   misaligned buffers give their errors before any device work.  Other
 *   arguments and errors as hq_encode_c.
 */
int hq_plan_c(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
              float c, uint32_t kv,
              uint64_t *tiles, uint64_t *chunks, uint64_t *payload_cap_words,
              uint64_t *workspace_bytes, uint32_t *tile_bound_bits);
int hq_encode_c(const void *x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                uint32_t lattice, float c, uint64_t seed, uint32_t kv,
                uint32_t *payload, uint64_t payload_cap_words, uint16_t *step, uint16_t *meta,
                uint32_t *chunk_off, uint32_t *status, void *workspace, uint64_t workspace_bytes,
                void *stream);
int hq_decode_c(const uint32_t *payload, uint64_t payload_words, const uint16_t *step,
                const uint16_t *meta, const uint32_t *chunk_off,
                uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
                float c, uint64_t seed, uint32_t kv, void *x_out, uint32_t *status, void *stream);
int hq_rate_bracket(uint32_t lattice, float target_bps, float *c_lo, float *c_hi);
int hq_encode_length_c(const void *x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                       uint32_t lattice, float c, uint64_t seed, uint32_t kv, unsigned long long *words,
                       void *stream);

/*
 * hq_encode_c_noalloc — hq_encode_c without the workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The workspace is a
 * static 1 MiB device array in the library, one per GPU, held until the
 * process ends; the first call on a GPU takes its address and clears it with
 * a kernel on `stream`.  The call allocates nothing (no hipMalloc, no
 * library allocation); the caller still passes every input and output.
 * Limit: the workspace hq_plan_c reports (768 + 8 C bytes) must fit 1 MiB,
 * i.e. at most 130976 chunks of 64 tiles; larger tensors get HQ_ENOSPC
 * before any device work.  Every call on one GPU shares its array, and each
 * call leaves it ready for the next: calls issued on one stream follow one
 * another safely, but calls that overlap in time on one GPU (different
 * streams, or threads) race and must not be made.  Other arguments, errors
 * and the stream are hq_encode_c's.
 */
int hq_encode_c_noalloc(const void *x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                        uint32_t lattice, float c, uint64_t seed, uint32_t kv,
                        uint32_t *payload, uint64_t payload_cap_words, uint16_t *step, uint16_t *meta,
                        uint32_t *chunk_off, uint32_t *status, void *stream);
int hq_encode_rate(const void *x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                   uint32_t lattice, float target_bps, uint64_t seed, uint32_t kv,
                   uint32_t *payload, uint64_t payload_cap_words, uint16_t *step, uint16_t *meta,
                   uint32_t *chunk_off, uint32_t *status, void *workspace, uint64_t workspace_bytes,
                   float *c_out, double *bps_out, uint32_t *encodes_out, void *stream);

/*
 * hq_rotate — the KV path's per-layer Haar rotation (gist.science explainer
 * of HyperQuant, Methodology section 4, "Bias Correction for KV Cache": a
 * Haar-uniform rotation as the alternative to the sign diagonal).  For each
 * of `rows` d-vectors (d = 64 or 128), y = Q x (transpose = 0) or Q^T x
 * (transpose = 1), each output one fused multiply-add chain over j = 0 ..
 * d-1 in ascending order from +0 (bf16 output: that value rounded to nearest
 * even).  The rotation runs before hq_kv_encode (whose RHT then applies
 * H D; H D Q is Haar-uniform whenever Q is) and, transposed, after
 * hq_kv_decode.
 *   Q   device, [d][d] fp32 row-major, 4-byte aligned, drawn by the caller
 *   x   device, [rows][d] of x_dtype (HQ_F32 or HQ_BF16), 16-byte aligned
 *   y   device, [rows][d] of y_dtype, 16-byte aligned, not overlapping x
 * Asynchronous on `stream`; HQ_EINVAL for another d, a bad dtype, a NULL or
 * misaligned pointer, or rows >= 2^32 (before any device work).
 */
int hq_rotate(const float *Q, uint32_t d, uint32_t transpose, const void *x, uint32_t x_dtype,
              uint64_t rows, void *y, uint32_t y_dtype, void *stream);

/*
 * int8 product path (gist.science explainer of HyperQuant, Key Contributions,
 * "Hardware Integration": int8 matrix-core products on the post-RHT lattice
 * output; Methodology section 2: the lattice's integer embedding).  A weight
 * tile decodes to D H (s P) / sqrt(n), so a weight row times an activation x
 * is the sum over tiles of s_t <P_t, RHT(x)_t>; these calls compute it with
 * int8 operands.
 *
 * hq_decode_codes — as hq_decode_c (weights, kv = 0) but writes each tile's
 *   integer codes 2P, int8 [rows][cols] (device, 16-byte aligned), for Z, D4
 *   and E8 only (HQ_EINVAL otherwise).  Codes beyond [-127, 127] are
 *   saturated and HQ_FLAG_RANGE is OR-ed into *status; a corrupt tile's codes
 *   are 0 (HQ_FLAG_CORRUPT).  The tile steps stay in `step`.
 * hq_act_quant — activations x [batch][cols] (HQ_F32 or HQ_BF16, device):
 *   per tile of n (the weights' tile size and seed), y = the codec's RHT of
 *   the tile, a = fl(max |y| / 127), q = rint(fl(y / a)) (0 where a = 0),
 *   clamped to [-127, 127]; q int8 [batch][cols], a fp32 [batch][cols / n].
 *   A tile with a NaN gets a = NaN and one with an infinity a = inf (max |y|
 *   lets a NaN through); a code whose quotient y / a is NaN is 0.  Such a
 *   tile's products are then NaN, so the non-finite input shows in y.
 * hq_codes_matmul — y[b][r] = 0.5 * (fma chain over the row's tiles t in
 *   ascending order, from +0, of (float) I * fl(s_t * a_bt)), I the exact
 *   int32 <codes tile, q tile> (matrix cores, all tiles in parallel; the
 *   chain in a second pass).  codes and q 16-byte aligned; y fp32
 *   [batch][rows]; work: device int32 scratch of at least
 *   4 * batch * rows * (cols / n) bytes (HQ_ENOSPC otherwise).
 * All three are asynchronous on `stream`; argument errors return HQ_EINVAL
 * before any device work.
 */
int hq_decode_codes(const uint32_t *payload, uint64_t payload_words, const uint16_t *step,
                    const uint16_t *meta, const uint32_t *chunk_off, uint64_t rows, uint64_t cols,
                    uint32_t tile, uint32_t lattice, float c, uint64_t seed, int8_t *codes,
                    uint32_t *status, void *stream);
int hq_act_quant(const void *x, uint32_t x_dtype, uint64_t batch, uint64_t cols, uint32_t tile,
                 uint64_t seed, int8_t *q, float *scale, void *stream);
int hq_codes_matmul(const int8_t *codes, const uint16_t *step, uint64_t rows, uint64_t cols,
                    uint32_t tile, const int8_t *q, const float *scale, uint64_t batch, float *y,
                    int32_t *work, uint64_t work_bytes, void *stream);

/*
 * hq_act_quant_blocked — hq_act_quant (the same codes and scales) with q in
 * the matrix cores' operand order, for hq_codes_matmul_fused: with T = cols /
 * n tiles a row, the code of activation b, column t n + 32 k + j (j < 32) is
 * q[(((b / 32) T + t) (n / 32) + k) 1024 + (b % 32) 32 + j], so that q holds
 * ceil(batch / 32) * 32 * cols bytes (the entries of activations at or past
 * batch are neither written nor read).  scale fp32 [batch][cols / n] as for
 * hq_act_quant.  Asynchronous on `stream`; HQ_EINVAL before any device work
 * as for hq_act_quant.
 */
int hq_act_quant_blocked(const void *x, uint32_t x_dtype, uint64_t batch, uint64_t cols, uint32_t tile,
                         uint64_t seed, int8_t *q, float *scale, void *stream);

/*
 * hq_codes_matmul_fused — hq_decode_codes followed by hq_codes_matmul in one
 * launch, straight from the compressed stream (gist.science explainer of
 * HyperQuant, "Significance and Claims": decoding fused with the matrix
 * product): the same y, bit for bit, with no code tensor and no scratch in
 * device memory.  Each tile's bits are parsed into its codes 2P in on-chip
 * memory and multiplied there on the matrix cores; the fp32 chain over a
 * row's tiles runs in ascending order.
 *   payload .. chunk_off, rows, cols, tile, lattice, c: a weight stream as
 *              for hq_decode_codes (Z, D4 or E8 without dither); every row
 *              must be a whole number of 64-tile chunks: cols % (64 tile) == 0;
 *              payload 16-byte aligned (it is read in 16-byte vectors)
 *   q, scale   hq_act_quant_blocked's output for [batch][cols] activations
 *              (q in its blocked order, 16-byte aligned)
 *   y          fp32 [batch][rows]
 *   status     device word: HQ_FLAG_CORRUPT (a tile's codes taken as 0) and
 *              HQ_FLAG_RANGE (a code saturated) are OR-ed in, as by
 *              hq_decode_codes
 * Asynchronous on `stream`; HQ_EINVAL for another lattice or shape, or a NULL
 * or misaligned pointer, before any device work.
 */
int hq_codes_matmul_fused(const uint32_t *payload, uint64_t payload_words, const uint16_t *step,
                          const uint16_t *meta, const uint32_t *chunk_off, uint64_t rows, uint64_t cols,
                          uint32_t tile, uint32_t lattice, float c, const int8_t *q, const float *scale,
                          uint64_t batch, float *y, uint32_t *status, void *stream);

/*
 * hq_nearest — the lattice quantiser alone (gist.science explainer of
 * HyperQuant, Methodology section 2): for each of nblocks blocks of d = 1,
 * 2, 4 or 8 coordinates (Z, A2, D4, E8) of t (device, fp32, [nblocks][d]),
 * the nearest lattice point, with the encoder's own decision and tie rules
 * (round half to even; a D_n candidate moves its first coordinate of largest
 * rounding error towards t; E8 and A2 take the second coset only when it is
 * strictly nearer), written as fp32 to points (device, [nblocks][d]; E8:
 * d + p/2, A2: (m + p/2, sqrt3 (n' + p/2))).  Asynchronous on `stream`;
 * HQ_EINVAL for another lattice, a NULL or misaligned pointer, or nblocks >=
 * 2^40.
 */
int hq_nearest(uint32_t lattice, const float *t, uint64_t nblocks, float *points, void *stream);

/* message for a hq_status code (static storage) */
const char *hq_strerror(int code);
/* (major << 16) | minor of the library; the stream layout above is version 1 */
uint32_t hq_version(void);

#ifdef __cplusplus
}
#endif
#endif
