/*
 * hq_oracle.h — CPU oracle of the HyperQuant encode/decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library: the format and arithmetic are re-derived here from the method's
 * description, in plain single-threaded C, fp32 operations one at a time
 * (built with -ffp-contract=off, no fast-math).
 *
 * Method source: "HyperQuant: A Rate-Distortion-Optimal Quantization
 * Pipeline for Large Language and Diffusion Models" — the English abstract
 * (paperdance.org card) and the gist.science explainer, section
 * "Methodology: The HyperQuant Pipeline", components 1 (per-tile RHT),
 * 2 (lattice quantization), 3 (bit-stripping and Rice coding) and
 * 4 (bias correction for the KV cache).
 */
#ifndef HQ_ORACLE_H
#define HQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { HQO_OK = 0, HQO_EINVAL = -1, HQO_ENOSPC = -3, HQO_ENONFINITE = -4, HQO_ECORRUPT = -5 };
enum { HQO_F32 = 0, HQO_BF16 = 1 };
enum { HQO_Z = 1, HQO_A2 = 2, HQO_D4 = 4, HQO_E8 = 8 };

#define HQO_CHUNK_TILES 64u

typedef struct {
    uint32_t dtype;    /* HQO_F32 or HQO_BF16 (input of encode, output of decode) */
    uint32_t tile;     /* n: 64, 128 or 256 */
    uint64_t rows;
    uint64_t cols;     /* cols % tile == 0 */
    uint32_t lattice;  /* HQO_Z, HQO_A2, HQO_D4, HQO_E8 */
    uint32_t dither;   /* 0: weights, 1: KV subtractive dither */
    float    c;        /* rate constant: step = bf16(rms * c) */
    uint32_t pad_;
    uint64_t seed;
    uint64_t tile_base; /* global index of the first tile: the dither of a KV
                           coordinate is indexed by its place in the whole
                           tensor, so a slice of tiles [b, b + T) of a larger
                           tensor is encoded (or decoded) as a tensor of its
                           own with tile_base = b; 0 for a whole tensor */
} hqo_params;

/* ---- generator ---------------------------------------------------------- */
uint32_t hqo_pcg_hash(uint32_t v);
uint32_t hqo_key(uint64_t seed, uint32_t domain);
uint32_t hqo_sign_bit(uint64_t seed, uint32_t i);           /* sigma_i in {0,1} */
uint32_t hqo_dither_bits(uint64_t seed, uint32_t g);        /* 24-bit uniform of coordinate g */

/* ---- single steps (exposed for the pin tests) -------------------------- */
void  hqo_rht_forward(const float *x, uint32_t n, uint64_t seed, float *y);
void  hqo_rht_inverse(const float *y, uint32_t n, uint64_t seed, float *x);
float hqo_tile_step(const float *y, uint32_t n, float c, int *nonfinite);
/* nearest lattice point of one block t[d]; writes the integer code
 * (code[0] = coset bit p, code[1..d] = integer coordinates) and the point */
void  hqo_nearest(uint32_t lattice, const float *t, int32_t *code, float *point);
/* the same for nblocks consecutive blocks; codes has d+1 entries per block */
void  hqo_nearest_batch(uint32_t lattice, const float *t, uint64_t nblocks, int32_t *codes, float *points);
/* dither vector (already reduced into the Voronoi cell) of one block whose
 * first coordinate has global index g0 */
void  hqo_dither_block(uint32_t lattice, uint64_t seed, uint32_t g0, float *u);
uint32_t hqo_zigzag(int32_t v);
int32_t  hqo_unzigzag(uint32_t u);
uint32_t hqo_rice_k(const uint32_t *u, uint32_t n);          /* smallest argmin of coded length */
uint64_t hqo_rice_cost(const uint32_t *u, uint32_t n, uint32_t k);

/* ---- the path ----------------------------------------------------------- */
/* worst-case tile length in bits (0 if the configuration is not encodable) */
uint32_t hqo_tile_bound_bits(const hqo_params *p);
uint64_t hqo_payload_cap_words(const hqo_params *p);
int hqo_encode(const void *x, const hqo_params *p,
               uint16_t *step, uint16_t *meta, uint32_t *chunk_off,
               uint32_t *payload, uint64_t payload_cap_words);
int hqo_decode(const uint16_t *step, const uint16_t *meta, const uint32_t *chunk_off,
               const uint32_t *payload, uint64_t payload_words,
               const hqo_params *p, void *x_out);
/* encode/decode of a tile range [t0, t1) only (sampled parity at full size):
 * tile-local outputs are the same as the full encode's; bits[] receives the
 * concatenated bitstreams of the tiles, starting at bit 0. */
/* decode tiles [t0, t1) from their concatenated bitstreams (bit 0 = start of
 * tile t0); x_out receives the range only ((t1 - t0) * tile elements) */
int hqo_decode_tiles(const uint16_t *step, const uint16_t *meta, const uint32_t *bits, uint64_t bits_words,
                     const hqo_params *p, uint64_t t0, uint64_t t1, void *x_out);
int hqo_encode_tiles(const void *x, const hqo_params *p, uint64_t t0, uint64_t t1,
                     uint16_t *step, uint16_t *meta, uint32_t *bits, uint64_t bits_cap_words);

/* KV rotation y = Q x (transpose = 0) or Q^T x per d-vector, one ascending
 * fused multiply-add chain per output; x, y fp32 or bf16 bits, [rows][d] */
void hqo_rotate(const float *Q, uint32_t d, uint32_t transpose, const void *x, uint32_t x_dtype,
                uint64_t rows, void *y, uint32_t y_dtype);

/* int8 product path: a stream's codes 2P (Z, D4, E8 without dither; int8,
 * saturated, *range_flag set if any was), the activation's per-tile RHT in
 * int8 with fp32 scales, and y[b][r] = 0.5 * (ascending fma chain over the
 * row's tiles of (float)<codes, q> * fl(step * scale)) */
int hqo_decode_codes(const uint16_t *step, const uint16_t *meta, const uint32_t *chunk_off,
                     const uint32_t *payload, uint64_t payload_words, const hqo_params *p, int8_t *codes,
                     uint32_t *range_flag);
void hqo_act_quant(const float *x, uint64_t batch, uint64_t cols, uint32_t n, uint64_t seed, int8_t *q,
                   float *scale);
void hqo_codes_matmul(const int8_t *codes, const uint16_t *step, uint64_t rows, uint64_t cols, uint32_t n,
                      const int8_t *q, const float *scale, uint64_t batch, float *y);

#ifdef __cplusplus
}
#endif
#endif
