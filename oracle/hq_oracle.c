/*
 * hq_oracle.c — plain, slow, single-threaded CPU oracle of the HyperQuant
 * encode/decode path.  TEST INFRASTRUCTURE ONLY (see hq_oracle.h).
 *
 * Every floating-point step is one IEEE binary32 operation, round to
 * nearest even, written out one at a time; the file must be compiled with
 * -ffp-contract=off and without fast-math so that the compiler neither
 * fuses nor reorders them.  No SIMD, no threads, no lookup tables.
 *
 * Citations name the source page and its section:
 *   [Abs]  paperdance.org card of the paper, English abstract.
 *   [M1]   gist.science explainer (English), "Methodology: The HyperQuant
 *          Pipeline", 1. Per-Tile Randomized Hadamard Transform.
 *   [M2]   same section, 2. Lattice Quantization.
 *   [M3]   same section, 3. Bit-Stripping and Rice Coding.
 *   [M4]   same section, 4. Bias Correction for KV Cache.
 * Where the pages leave a step open the reading taken is stated at the step.
 */
#include "hq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Counter-based generator: the "pcg" hash of Jarzynski & Olano, "Hash      */
/* Functions for GPU Rendering", JCGT 9(3), 2020 — one LCG step of PCG      */
/* followed by PCG's RXS-M-XS output permutation (O'Neill 2014).            */
/* The pages name no generator; this one is a bijection on 32-bit words and */
/* needs no state, so encoder and decoder regenerate the same numbers.      */
/* ------------------------------------------------------------------------ */
uint32_t hqo_pcg_hash(uint32_t v)
{
    uint32_t state = v * 747796405u + 2891336453u;
    uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
    return (word >> 22u) ^ word;
}

#define DOMAIN_SIGN   0x5349474Eu   /* "SIGN" */
#define DOMAIN_DITHER 0x44495448u   /* "DITH" */

uint32_t hqo_key(uint64_t seed, uint32_t domain)
{
    uint32_t lo = (uint32_t)(seed & 0xFFFFFFFFu);
    uint32_t hi = (uint32_t)(seed >> 32);
    return hqo_pcg_hash(hqo_pcg_hash(lo ^ domain) ^ hi);
}

/* [M1]: D is a random sign diagonal.  Reading: one D per call (per layer for
 * the KV cache: [M4] rotates each layer's vectors with a random +-1
 * diagonal), entry i negative iff the top bit of hash(key + i) is set. */
uint32_t hqo_sign_bit(uint64_t seed, uint32_t i)
{
    return hqo_pcg_hash(hqo_key(seed, DOMAIN_SIGN) + i) >> 31;
}

/* [M4]: the dither is fresh per vector; coordinate g of the call (row-major
 * flat index) draws 24 uniform bits. */
uint32_t hqo_dither_bits(uint64_t seed, uint32_t g)
{
    return hqo_pcg_hash(hqo_key(seed, DOMAIN_DITHER) + g) >> 8;
}

/* ------------------------------------------------------------------------ */
/* Scalar helpers                                                           */
/* ------------------------------------------------------------------------ */
static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 round-to-nearest-even of a finite fp32 value, returned as bits */
static uint16_t bf16_rne(float f)
{
    uint32_t u = f32_to_bits(f);
    u = u + 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

static uint32_t log2u(uint32_t n) { uint32_t l = 0; while ((1u << l) < n) l++; return l; }

static float inv_sqrt_n(uint32_t n) { return (float)(1.0 / sqrt((double)n)); }
static float sqrt3_f(void) { return (float)sqrt(3.0); }
static float inv_sqrt3_f(void) { return (float)(1.0 / sqrt(3.0)); }

uint32_t hqo_zigzag(int32_t v) { return v >= 0 ? 2u * (uint32_t)v : 2u * (uint32_t)(-(int64_t)v) - 1u; }
int32_t hqo_unzigzag(uint32_t u) { return (u & 1u) ? -(int32_t)((u >> 1) + 1u) : (int32_t)(u >> 1); }

/* floor(v / 2) for a 32-bit integer, without relying on signed shifts */
static int32_t floor_half(int32_t v) { return (v - (v & 1)) / 2; }

static uint32_t lattice_dim(uint32_t lat)
{
    switch (lat) { case HQO_Z: return 1; case HQO_A2: return 2; case HQO_D4: return 4; case HQO_E8: return 8; }
    return 0;
}
/* coset bits per block: E8 = D8 u (D8 + 1/2), A2 = R u (R + (1/2, sqrt3/2)) */
static uint32_t coset_bits_per_block(uint32_t lat) { return (lat == HQO_E8 || lat == HQO_A2) ? 1u : 0u; }

/* ------------------------------------------------------------------------ */
/* [M1] RHT_n(x) = H_n D x, scaled by 1/sqrt(n) so that it is orthogonal     */
/* (the pages call the transform orthogonal).  H_n is the Sylvester-ordered */
/* Walsh-Hadamard matrix, H_ij = (-1)^popcount(i & j), applied by the fast   */
/* butterfly with strides h = 1, 2, 4, ..., n/2 in that order.              */
/* ------------------------------------------------------------------------ */
static void fwht(float *a, uint32_t n)
{
    for (uint32_t h = 1; h < n; h <<= 1) {
        for (uint32_t j = 0; j < n; j++) {
            if (j & h) continue;
            float lo = a[j], hi = a[j + h];
            a[j]     = lo + hi;
            a[j + h] = lo - hi;
        }
    }
}

void hqo_rht_forward(const float *x, uint32_t n, uint64_t seed, float *y)
{
    float a[256];
    float s = inv_sqrt_n(n);
    for (uint32_t i = 0; i < n; i++) a[i] = hqo_sign_bit(seed, i) ? -x[i] : x[i];
    fwht(a, n);
    for (uint32_t i = 0; i < n; i++) y[i] = a[i] * s;
}

/* inverse: x = D H y / sqrt(n)  (H symmetric, H H = n I, D D = I) */
void hqo_rht_inverse(const float *y, uint32_t n, uint64_t seed, float *x)
{
    float a[256];
    float s = inv_sqrt_n(n);
    for (uint32_t i = 0; i < n; i++) a[i] = y[i];
    fwht(a, n);
    for (uint32_t i = 0; i < n; i++) {
        float v = a[i] * s;
        x[i] = hqo_sign_bit(seed, i) ? -v : v;
    }
}

/* ------------------------------------------------------------------------ */
/* [M2] per-tile scale alpha.  Reading: step = bf16_rne(RMS(y) * c), where   */
/* c is the rate constant for the target bps; the sum of squares is the     */
/* pairwise tree ((y0^2 + y1^2) + (y2^2 + y3^2)) + ...  A step below 2^-124 */
/* (zero, a bf16 subnormal, or one of the two lowest normal binades) is     */
/* stored as 0 and the tile decodes to zeros: a dithered coordinate can be  */
/* as small as 2^-25, and below 2^-124 its product with the step could      */
/* round to zero when decoded.                                              */
/* ------------------------------------------------------------------------ */
float hqo_tile_step(const float *y, uint32_t n, float c, int *nonfinite)
{
    float sq[256];
    for (uint32_t i = 0; i < n; i++) sq[i] = y[i] * y[i];
    for (uint32_t m = n; m > 1; m >>= 1)
        for (uint32_t i = 0; i < m / 2; i++) sq[i] = sq[2 * i] + sq[2 * i + 1];
    float ss = sq[0];
    *nonfinite = 0;
    if (!isfinite(ss)) { *nonfinite = 1; return 0.0f; }
    float mean = ss * ldexpf(1.0f, -(int)log2u(n));     /* exact power-of-two scale */
    float rms = sqrtf(mean);
    float r = rms * c;
    uint16_t sb = bf16_rne(r);
    if ((sb & 0x7F80u) == 0x7F80u) { *nonfinite = 1; return 0.0f; }
    if ((sb & 0x7F80u) < 0x0180u) return 0.0f;           /* below 2^-124 */
    return bf16_to_f32(sb);
}

/* ------------------------------------------------------------------------ */
/* [M2] nearest lattice points.                                             */
/* ------------------------------------------------------------------------ */

/* Z: coordinate-wise round half to even */
static void nearest_Z(const float *t, int32_t *code, float *pt)
{
    float f = rintf(t[0]);
    code[0] = 0; code[1] = (int32_t)f; pt[0] = f;
}

/* D4 = {x in Z^4 : sum x even} (Conway & Sloane's decoder): round every
 * coordinate; if the sum is odd, move the coordinate with the largest
 * rounding error (smallest index on ties) to its second-nearest integer. */
static void nearest_D4(const float *t, int32_t *code, float *pt)
{
    float f[4], dl[4];
    int32_t s = 0;
    for (int i = 0; i < 4; i++) { f[i] = rintf(t[i]); dl[i] = t[i] - f[i]; s += (int32_t)f[i]; }
    if (s & 1) {
        int j = 0;
        for (int i = 1; i < 4; i++) if (fabsf(dl[i]) > fabsf(dl[j])) j = i;
        f[j] = (t[j] >= f[j]) ? f[j] + 1.0f : f[j] - 1.0f;
    }
    code[0] = 0;
    for (int i = 0; i < 4; i++) { code[1 + i] = (int32_t)f[i]; pt[i] = f[i]; }
}

/* The nearest point of D8 + h (h = 0 or 1/2 in every coordinate), Conway &
 * Sloane's D_n decoder on the shifted coset.  Start from the nearest point of
 * Z^8 + h: rint(t) (ties to even) or floor(t) + 1/2.  If the coordinates'
 * integer parts sum to an odd number, move the coordinate farthest from that
 * start, smallest index on ties, one step towards t (t >= P: +1, else -1).
 * Distances are compared exactly: with delta = t - rint(t) (exact in fp32),
 * |t - rint t| = |delta| and |t - (floor t + 1/2)| = 1/2 - |delta|, so the
 * farthest coordinate is the one of largest |delta| for h = 0 and of
 * smallest |delta| for h = 1/2 (t - (floor t + 1/2) itself can round in fp32
 * when |t| < 1/4).  P[] gets the point, d[] its integer parts. */
static void nearest_D8_coset(const float *t, int half, float *P, int32_t *d)
{
    float ad[8];
    int32_t s = 0;
    for (int i = 0; i < 8; i++) {
        float f = rintf(t[i]);
        ad[i] = fabsf(t[i] - f);
        float base = half ? floorf(t[i]) : f;
        d[i] = (int32_t)base;
        P[i] = half ? base + 0.5f : base;
        s += d[i];
    }
    if (s & 1) {
        int j = 0;
        for (int i = 1; i < 8; i++)
            if (half ? ad[i] < ad[j] : ad[i] > ad[j]) j = i;
        float step = (t[j] >= P[j]) ? 1.0f : -1.0f;
        P[j] = P[j] + step;
        d[j] += (int32_t)step;
    }
}

/* E8 = D8 u (D8 + 1/2) ([M2]: E8 has a closed-form decoder of fixed cost).
 * Conway & Sloane's E8 decoder: the nearest point A of D8 and B of D8 + 1/2
 * (nearest_D8_coset), then the nearer of the two.  Reading: the pages fix no
 * arithmetic for the comparison.  With delta = t - rint(t), exact in fp32,
 * the difference of the squared distances is, in exact arithmetic,
 *   |t-A|^2 - |t-B|^2 = sum|delta| - 2 + [A moved](1 - 2 max|delta|)
 *                                       - [B moved](2 min|delta|)
 * (every coordinate is |delta| from rint(t) and 1/2 - |delta| from
 * floor(t) + 1/2; a moved coordinate is 1 - |delta| or 1/2 + |delta| away).
 * B is taken iff this, evaluated in fp32 in the order written, is > 0 (ties
 * go to D8): a fixed cost, and within 10 * 2^-23 of the exact difference,
 * which the tests check against both candidates' fp64 distances. */
static void nearest_E8(const float *t, int32_t *code, float *pt)
{
    float A[8], B[8];
    int32_t dA[8], dB[8], sf = 0, sg = 0;
    nearest_D8_coset(t, 0, A, dA);
    nearest_D8_coset(t, 1, B, dB);
    float ad[8];
    for (int i = 0; i < 8; i++) {
        ad[i] = fabsf(t[i] - rintf(t[i]));
        sf += (int32_t)rintf(t[i]);
        sg += (int32_t)floorf(t[i]);
    }
    float mx = ad[0], mn = ad[0];
    for (int i = 1; i < 8; i++) {
        if (ad[i] > mx) mx = ad[i];
        if (ad[i] < mn) mn = ad[i];
    }
    float sabs = ((ad[0] + ad[1]) + (ad[2] + ad[3])) + ((ad[4] + ad[5]) + (ad[6] + ad[7]));
    float diff = sabs - 2.0f;
    if (sf & 1) diff = diff + (1.0f - 2.0f * mx);
    if (sg & 1) diff = diff - 2.0f * mn;
    int useB = diff > 0.0f;
    code[0] = useB;
    for (int i = 0; i < 8; i++) {
        code[1 + i] = useB ? dB[i] : dA[i];
        pt[i] = useB ? B[i] : A[i];
    }
}

/* A2 (hexagonal, minimal distance 1) = R u (R + (1/2, sqrt3/2)) with
 * R = Z x sqrt3 Z: the nearer of the two rectangular-coset roundings,
 * squared distances in fp32, ties to R.  Code: p, m, n' with point
 * (m + p/2, sqrt3 (n' + p/2)). */
static void nearest_A2(const float *t, int32_t *code, float *pt)
{
    const float S3 = sqrt3_f(), IS3 = inv_sqrt3_f();
    float s1 = t[1] * IS3;
    float am = rintf(t[0]), an = rintf(s1);
    float bm = floorf(t[0]), bn = floorf(s1);
    float a0 = am, a1 = S3 * an;
    float b0 = bm + 0.5f, b1 = S3 * (bn + 0.5f);
    float ea0 = t[0] - a0, ea1 = t[1] - a1;
    float eb0 = t[0] - b0, eb1 = t[1] - b1;
    float da = ea0 * ea0 + ea1 * ea1;
    float db = eb0 * eb0 + eb1 * eb1;
    if (db < da) { code[0] = 1; code[1] = (int32_t)bm; code[2] = (int32_t)bn; pt[0] = b0; pt[1] = b1; }
    else         { code[0] = 0; code[1] = (int32_t)am; code[2] = (int32_t)an; pt[0] = a0; pt[1] = a1; }
}

void hqo_nearest(uint32_t lattice, const float *t, int32_t *code, float *point)
{
    switch (lattice) {
    case HQO_Z:  nearest_Z(t, code, point); break;
    case HQO_A2: nearest_A2(t, code, point); break;
    case HQO_D4: nearest_D4(t, code, point); break;
    case HQO_E8: nearest_E8(t, code, point); break;
    }
}

void hqo_nearest_batch(uint32_t lattice, const float *t, uint64_t nblocks, int32_t *codes, float *points)
{
    uint32_t d = lattice_dim(lattice);
    for (uint64_t b = 0; b < nblocks; b++)
        hqo_nearest(lattice, t + b * d, codes + b * (d + 1), points + b * d);
}

/* ------------------------------------------------------------------------ */
/* [M4] subtractive dither U ~ Uniform(V(Lambda)).  Draw v uniformly on a    */
/* box that is a fundamental region of a sublattice of Lambda (E8, D4:       */
/* [-1,1)^d of 2Z^d; Z: [-1/2,1/2); A2: [-1/2,1/2) x sqrt3[-1/2,1/2) of R),  */
/* then reduce into the Voronoi cell: u = v - Q(v).                          */
/* ------------------------------------------------------------------------ */
void hqo_dither_block(uint32_t lattice, uint64_t seed, uint32_t g0, float *u)
{
    uint32_t d = lattice_dim(lattice);
    float v[8] = {0}, pt[8];
    int32_t code[9];
    for (uint32_t i = 0; i < d; i++) {
        float a = (float)hqo_dither_bits(seed, g0 + i);       /* exact: 24 bits */
        if (lattice == HQO_E8 || lattice == HQO_D4) v[i] = a * 0x1p-23f - 1.0f;
        else v[i] = a * 0x1p-24f - 0.5f;
    }
    if (lattice == HQO_A2) v[1] = sqrt3_f() * v[1];
    hqo_nearest(lattice, v, code, pt);
    for (uint32_t i = 0; i < d; i++) u[i] = v[i] - pt[i];
}

/* ------------------------------------------------------------------------ */
/* [M3] bit-stripping and Rice coding.                                      */
/* ------------------------------------------------------------------------ */
uint64_t hqo_rice_cost(const uint32_t *u, uint32_t n, uint32_t k)
{
    uint64_t c = 0;
    for (uint32_t i = 0; i < n; i++) c += (uint64_t)(u[i] >> k) + 1u + k;
    return c;
}

/* Reading: the per-tile Rice parameter is the k in 0..7 of smallest coded
 * length, the smallest such k on ties. */
uint32_t hqo_rice_k(const uint32_t *u, uint32_t n)
{
    uint32_t best = 0;
    uint64_t bc = hqo_rice_cost(u, n, 0);
    for (uint32_t k = 1; k < 8; k++) {
        uint64_t c = hqo_rice_cost(u, n, k);
        if (c < bc) { bc = c; best = k; }
    }
    return best;
}

/* Bit-stripping ([M3]: membership constraints fix some bits of the integer
 * code): E8 keeps its coset bit raw and drops the parity of d7, which equals
 * the parity of d0+...+d6 (D8 has even coordinate sum); D4 likewise drops the
 * parity of w3.  Every other integer is zigzag-mapped to a non-negative
 * symbol.  Symbols are in block order, coordinate order inside a block. */
static void block_symbols(uint32_t lattice, const int32_t *code, uint32_t *sym)
{
    switch (lattice) {
    case HQO_Z:  sym[0] = hqo_zigzag(code[1]); break;
    case HQO_A2: sym[0] = hqo_zigzag(code[1]); sym[1] = hqo_zigzag(code[2]); break;
    case HQO_D4:
        for (int i = 0; i < 3; i++) sym[i] = hqo_zigzag(code[1 + i]);
        sym[3] = hqo_zigzag(floor_half(code[4]));
        break;
    case HQO_E8:
        for (int i = 0; i < 7; i++) sym[i] = hqo_zigzag(code[1 + i]);
        sym[7] = hqo_zigzag(floor_half(code[8]));
        break;
    }
}

/* inverse of block_symbols + point reconstruction (decode) */
static void block_point(uint32_t lattice, uint32_t p, const uint32_t *sym, float *pt)
{
    switch (lattice) {
    case HQO_Z: pt[0] = (float)hqo_unzigzag(sym[0]); break;
    case HQO_A2: {
        float h = p ? 0.5f : 0.0f;
        pt[0] = (float)hqo_unzigzag(sym[0]) + h;
        pt[1] = sqrt3_f() * ((float)hqo_unzigzag(sym[1]) + h);
        break;
    }
    case HQO_D4: {
        int32_t w[4], s = 0;
        for (int i = 0; i < 3; i++) { w[i] = hqo_unzigzag(sym[i]); s += w[i]; }
        w[3] = 2 * hqo_unzigzag(sym[3]) + (s & 1);
        for (int i = 0; i < 4; i++) pt[i] = (float)w[i];
        break;
    }
    case HQO_E8: {
        int32_t d[8], s = 0;
        for (int i = 0; i < 7; i++) { d[i] = hqo_unzigzag(sym[i]); s += d[i]; }
        d[7] = 2 * hqo_unzigzag(sym[7]) + (s & 1);
        for (int i = 0; i < 8; i++) pt[i] = p ? (float)d[i] + 0.5f : (float)d[i];
        break;
    }
    }
}

/* ---- bit I/O: bit b of a stream is bit (b & 31) of 32-bit word b >> 5 ---- */
static void put_bit(uint32_t *w, uint64_t b, uint32_t v) { if (v) w[b >> 5] |= 1u << (b & 31); }
static uint32_t get_bit(const uint32_t *w, uint64_t b) { return (w[b >> 5] >> (b & 31)) & 1u; }

/* Rice_k(u) is the k low bits of u (the remainder) plus the quotient
 * q = u >> k in unary: q zero bits, then a one bit.  Reading: the pages fix
 * neither polarity nor bit order nor where the two fields sit; a tile stores
 * the remainders of all n symbols first (a fixed-width plane, symbol i at
 * bits i*k .. i*k+k-1, least significant first) and then the n unary
 * quotients in symbol order.  Each codeword keeps its Rice length q + 1 + k. */
static uint64_t put_remainder(uint32_t *w, uint64_t b, uint32_t u, uint32_t k)
{
    for (uint32_t i = 0; i < k; i++) put_bit(w, b++, (u >> i) & 1u);
    return b;
}

static uint64_t put_unary(uint32_t *w, uint64_t b, uint32_t u, uint32_t k)
{
    b += u >> k;                  /* zeros: buffer is zero-initialised */
    put_bit(w, b++, 1);
    return b;
}

/* ------------------------------------------------------------------------ */
/* Capacity: a bound on any tile's length from the per-tile scale.          */
/* |t|_2 <= sqrt(n)/c' (c' = c with bf16 rounding margin), so               */
/* sum|t_i| <= n/c'; every code integer is within 3/2 of t_i (covering      */
/* radius <= 1, plus the coset half), so sum of symbols <= 2n/c' + 3n       */
/* (+2n with the dither, |u_i| <= 1); C(k*) <= C(k) for every k.             */
/* ------------------------------------------------------------------------ */
uint32_t hqo_tile_bound_bits(const hqo_params *p)
{
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    if (!d || !(p->c > 0.0f) || !isfinite(p->c)) return 0;
    double cp = (double)p->c * (1.0 - 1.0 / 128.0);
    double S = 2.0 * n / cp + 3.0 * n + (p->dither ? 2.0 * n : 0.0);
    double best = 1e300;
    for (int k = 0; k < 8; k++) {
        double L = floor(S / (double)(1u << k)) + (double)n * (1 + k);
        if (L < best) best = L;
    }
    double B = (double)(n / d) * coset_bits_per_block(p->lattice);
    double bound = B + best;
    if (bound > 8191.0) return 0;
    return (uint32_t)bound;
}

static int check_params(const hqo_params *p)
{
    if (p->dtype != HQO_F32 && p->dtype != HQO_BF16) return HQO_EINVAL;
    if (p->tile != 64 && p->tile != 128 && p->tile != 256) return HQO_EINVAL;
    if (!lattice_dim(p->lattice)) return HQO_EINVAL;
    if (p->dither > 1) return HQO_EINVAL;
    if (p->rows == 0 || p->cols == 0 || p->cols % p->tile) return HQO_EINVAL;
    if (p->rows * p->cols >= (1ull << 32)) return HQO_EINVAL;
    if (p->tile_base > (1ull << 32) || p->tile_base * p->tile + p->rows * p->cols > (1ull << 32)) return HQO_EINVAL;
    if (!hqo_tile_bound_bits(p)) return HQO_EINVAL;
    return HQO_OK;
}

uint64_t hqo_payload_cap_words(const hqo_params *p)
{
    if (check_params(p) != HQO_OK) return 0;
    uint64_t T = p->rows * p->cols / p->tile;
    uint64_t C = (T + HQO_CHUNK_TILES - 1) / HQO_CHUNK_TILES;
    return (T * hqo_tile_bound_bits(p) + 31) / 32 + C;
}

/* ------------------------------------------------------------------------ */
/* Encode one tile: symbols, coset bits, k, length.                         */
/* ------------------------------------------------------------------------ */
typedef struct {
    uint16_t step;
    uint32_t k, len, nonfinite;
    uint32_t nb;            /* number of coset bits */
    uint32_t cos[256];      /* coset bits in block order */
    uint32_t sym[256];
} tile_code;

static void load_tile(const void *x, const hqo_params *p, uint64_t t, float *xt)
{
    uint64_t base = t * p->tile;
    for (uint32_t i = 0; i < p->tile; i++) {
        if (p->dtype == HQO_F32) xt[i] = ((const float *)x)[base + i];
        else xt[i] = bf16_to_f32(((const uint16_t *)x)[base + i]);
    }
}

static void encode_tile(const void *x, const hqo_params *p, uint64_t t, tile_code *tc)
{
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    float xt[256], y[256], tt[256];
    load_tile(x, p, t, xt);
    hqo_rht_forward(xt, n, p->seed, y);                       /* [M1] */
    int nf;
    float s = hqo_tile_step(y, n, p->c, &nf);                 /* [M2] alpha */
    tc->nonfinite = nf;
    tc->step = bf16_rne(s);
    float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
    /* a tile with a non-finite energy is reported and coded as a zero tile */
    for (uint32_t i = 0; i < n; i++) tt[i] = nf ? 0.0f : y[i] * inv;
    if (p->dither) {                                          /* [M4] t + U */
        for (uint32_t b = 0; b < n; b += d) {
            float u[8];
            hqo_dither_block(p->lattice, p->seed, (uint32_t)((p->tile_base + t) * n + b), u);
            for (uint32_t i = 0; i < d; i++) tt[b + i] = tt[b + i] + u[i];
        }
    }
    tc->nb = 0;
    for (uint32_t b = 0; b < n; b += d) {                     /* [M2] nearest point */
        int32_t code[9];
        float pt[8];
        hqo_nearest(p->lattice, tt + b, code, pt);
        if (coset_bits_per_block(p->lattice)) tc->cos[tc->nb++] = (uint32_t)code[0];
        block_symbols(p->lattice, code, tc->sym + b);         /* [M3] strip */
    }
    tc->k = hqo_rice_k(tc->sym, n);                           /* [M3] Rice */
    tc->len = tc->nb + (uint32_t)hqo_rice_cost(tc->sym, n, tc->k);
}

/* tile = coset bits (block order), remainder plane, unary plane */
static uint64_t write_tile(uint32_t *w, uint64_t b, const tile_code *tc, uint32_t n)
{
    for (uint32_t i = 0; i < tc->nb; i++) put_bit(w, b++, tc->cos[i]);
    for (uint32_t i = 0; i < n; i++) b = put_remainder(w, b, tc->sym[i], tc->k);
    for (uint32_t i = 0; i < n; i++) b = put_unary(w, b, tc->sym[i], tc->k);
    return b;
}

/* Stream layout (reading; the pages give none): tiles in row-major order,
 * each tile = its coset bits then its n Rice codewords (remainder plane,
 * then unary plane, see put_remainder/put_unary); tiles are
 * bit-contiguous inside a chunk of 64 tiles; every chunk starts on a 32-bit
 * word (chunk_off[c] = its first word, chunk_off[C] = total words) and its
 * tail is zero-padded.  meta[t] = len << 3 | k; step[t] = bf16 bits. */
int hqo_encode(const void *x, const hqo_params *p,
               uint16_t *step, uint16_t *meta, uint32_t *chunk_off,
               uint32_t *payload, uint64_t payload_cap_words)
{
    int rc = check_params(p);
    if (rc) return rc;
    uint64_t T = p->rows * p->cols / p->tile;
    uint64_t C = (T + HQO_CHUNK_TILES - 1) / HQO_CHUNK_TILES;
    tile_code *tc = (tile_code *)malloc(sizeof(tile_code));
    if (!tc) return HQO_ENOSPC;
    int status = HQO_OK;
    uint64_t word = 0;
    for (uint64_t c = 0; c < C; c++) {
        chunk_off[c] = (uint32_t)word;
        uint64_t t0 = c * HQO_CHUNK_TILES, t1 = t0 + HQO_CHUNK_TILES;
        if (t1 > T) t1 = T;
        uint64_t bit = word * 32;
        for (uint64_t t = t0; t < t1; t++) {
            encode_tile(x, p, t, tc);
            if (tc->nonfinite) status = HQO_ENONFINITE;
            step[t] = tc->step;
            meta[t] = (uint16_t)((tc->len << 3) | tc->k);
            uint64_t need = (bit + tc->len + 31) / 32;
            if (need > payload_cap_words) { free(tc); return HQO_ENOSPC; }
            for (uint64_t w = bit / 32 + 1; w < need; w++) payload[w] = 0;
            if (bit % 32 == 0) payload[bit / 32] = 0;
            bit = write_tile(payload, bit, tc, p->tile);
        }
        word = (bit + 31) / 32;
    }
    chunk_off[C] = (uint32_t)word;
    free(tc);
    return status;
}

int hqo_encode_tiles(const void *x, const hqo_params *p, uint64_t t0, uint64_t t1,
                     uint16_t *step, uint16_t *meta, uint32_t *bits, uint64_t bits_cap_words)
{
    int rc = check_params(p);
    if (rc) return rc;
    uint64_t T = p->rows * p->cols / p->tile;
    if (t0 > t1 || t1 > T) return HQO_EINVAL;
    tile_code *tc = (tile_code *)malloc(sizeof(tile_code));
    if (!tc) return HQO_ENOSPC;
    memset(bits, 0, bits_cap_words * 4);
    int status = HQO_OK;
    uint64_t bit = 0;
    for (uint64_t t = t0; t < t1; t++) {
        encode_tile(x, p, t, tc);
        if (tc->nonfinite) status = HQO_ENONFINITE;
        step[t - t0] = tc->step;
        meta[t - t0] = (uint16_t)((tc->len << 3) | tc->k);
        if ((bit + tc->len + 31) / 32 > bits_cap_words) { free(tc); return HQO_ENOSPC; }
        bit = write_tile(bits, bit, tc, p->tile);
    }
    free(tc);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Decode: parse, rebuild lattice points, undo dither, scale, inverse RHT.  */
/* Corrupt input (reading; the pages are silent): a tile whose n codewords  */
/* do not span exactly its meta length, or that holds a symbol above 16     */
/* bits, and every tile of a chunk whose word count disagrees with its      */
/* tiles' lengths, exceeds the capacity bound or holds a tile longer than   */
/* the per-tile bound, decode to zero (+0 with                              */
/* the sign diagonal applied, no dither) and are reported.  So does a tile  */
/* whose step is neither +0 nor a finite bf16 of at least 2^-124: the      */
/* encoder stores the bf16 of a non-negative RMS times c > 0, with results  */
/* below 2^-124 flushed to +0, so a negative (or -0), smaller or non-finite */
/* step cannot come from encoding.  Valid streams never meet these          */
/* conditions.                                                              */
/* ------------------------------------------------------------------------ */

static int step_bad(uint16_t step) { return step != 0 && (step < 0x0180u || step > 0x7F7Fu); }

/* parse one tile starting at bit b (reads never reach bend); 0 = ok */

static int parse_tile(const uint32_t *w, uint64_t b, uint64_t bend, uint32_t len, uint32_t k,
                      uint32_t n, uint32_t nb, uint32_t *cos, uint32_t *sym)
{
    uint64_t tb = b;
    if (len < nb + n * (k + 1)) return 1;
    if (tb + len > bend) return 1;
    bend = tb + len;                  /* a tile's fields never leave the tile */
    for (uint32_t i = 0; i < nb; i++) cos[i] = get_bit(w, b++);
    for (uint32_t i = 0; i < n; i++) {
        uint32_t r = 0;
        for (uint32_t j = 0; j < k; j++) r |= get_bit(w, b++) << j;
        sym[i] = r;
    }
    for (uint32_t i = 0; i < n; i++) {
        uint64_t q = 0;
        while (b < bend && !get_bit(w, b)) { q++; b++; }
        if (b >= bend) return 1;
        b++;                                  /* the terminating one */
        uint64_t u = (q << k) | sym[i];
        if (u > 0xFFFFu) return 1;
        sym[i] = (uint32_t)u;
    }
    return (b - tb == len) ? 0 : 1;
}

/* points -> (dither) -> step -> inverse RHT of tile t; stores at out[slot] */
static void rebuild_tile(const hqo_params *p, uint64_t t, int bad, uint16_t step,
                         const uint32_t *cos, const uint32_t *sym, void *out, uint64_t slot)
{
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    float s = bad ? 0.0f : bf16_to_f32(step);
    float v[256], xo[256];
    uint32_t zero[8] = {0};
    for (uint32_t blk = 0; blk < n / d; blk++) {
        float pt[8];
        uint32_t pc = (coset_bits_per_block(p->lattice) && !bad) ? cos[blk] : 0;
        block_point(p->lattice, pc, bad ? zero : sym + blk * d, pt);
        if (p->dither && !bad) {
            float u[8];
            hqo_dither_block(p->lattice, p->seed, (uint32_t)((p->tile_base + t) * n + blk * d), u);
            for (uint32_t i = 0; i < d; i++) pt[i] = pt[i] - u[i];
        }
        for (uint32_t i = 0; i < d; i++) v[blk * d + i] = pt[i] * s;
    }
    hqo_rht_inverse(v, n, p->seed, xo);
    for (uint32_t i = 0; i < n; i++) {
        if (p->dtype == HQO_F32) ((float *)out)[slot * n + i] = xo[i];
        else ((uint16_t *)out)[slot * n + i] = bf16_rne(xo[i]);
    }
}

int hqo_decode(const uint16_t *step, const uint16_t *meta, const uint32_t *chunk_off,
               const uint32_t *payload, uint64_t payload_words,
               const hqo_params *p, void *x_out)
{
    int rc = check_params(p);
    if (rc) return rc;
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    uint32_t nb = (n / d) * coset_bits_per_block(p->lattice);
    uint64_t T = p->rows * p->cols / n;
    uint64_t C = (T + HQO_CHUNK_TILES - 1) / HQO_CHUNK_TILES;
    uint64_t chunk_cap = ((uint64_t)HQO_CHUNK_TILES * hqo_tile_bound_bits(p) + 31) / 32;
    int status = HQO_OK;
    uint32_t cos[256], sym[256];
    for (uint64_t c = 0; c < C; c++) {
        uint64_t w0 = chunk_off[c], w1 = chunk_off[c + 1];
        uint64_t t0 = c * HQO_CHUNK_TILES, t1 = t0 + HQO_CHUNK_TILES;
        if (t1 > T) t1 = T;
        uint64_t total = 0;
        int too_long = 0;
        for (uint64_t t = t0; t < t1; t++) {
            total += meta[t] >> 3;
            if ((uint32_t)(meta[t] >> 3) > hqo_tile_bound_bits(p)) too_long = 1;
        }
        int chunk_bad = !(w1 >= w0 && w1 <= payload_words && w1 - w0 <= chunk_cap)
                        || too_long || (total + 31) / 32 != w1 - w0;
        uint64_t b = w0 * 32, bend = w1 * 32;
        for (uint64_t t = t0; t < t1; t++) {
            uint32_t len = meta[t] >> 3, k = meta[t] & 7u;
            int bad = chunk_bad || step_bad(step[t]) || parse_tile(payload, b, bend, len, k, n, nb, cos, sym);
            if (bad) status = HQO_ECORRUPT;
            rebuild_tile(p, t, bad, step[t], cos, sym, x_out, t);
            b += len;
        }
    }
    return status;
}

int hqo_decode_tiles(const uint16_t *step, const uint16_t *meta, const uint32_t *bits, uint64_t bits_words,
                     const hqo_params *p, uint64_t t0, uint64_t t1, void *x_out)
{
    int rc = check_params(p);
    if (rc) return rc;
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    uint32_t nb = (n / d) * coset_bits_per_block(p->lattice);
    int status = HQO_OK;
    uint32_t cos[256], sym[256];
    uint64_t b = 0;
    for (uint64_t t = t0; t < t1; t++) {
        uint32_t len = meta[t - t0] >> 3, k = meta[t - t0] & 7u;
        int bad = step_bad(step[t - t0]) || parse_tile(bits, b, bits_words * 32, len, k, n, nb, cos, sym);
        if (bad) status = HQO_ECORRUPT;
        rebuild_tile(p, t, bad, step[t - t0], cos, sym, x_out, t - t0);
        b += len;
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* [M4] The per-layer rotation of KV vectors by a Haar-uniform orthogonal   */
/* matrix, the alternative to the sign diagonal (gist.science explainer of  */
/* HyperQuant, Methodology section 4, "Bias Correction for KV Cache").      */
/* Reading: the vector is rotated, y = Q x, before the codec's own per-tile */
/* RHT; H D Q is Haar-uniform whenever Q is, so the composite is the pages' */
/* Haar rotation.  Decode applies Q^T after the codec's inverse.  Q is an   */
/* input (the caller draws it).  Each output is one fused multiply-add      */
/* chain over j = 0 .. d-1 in ascending order, starting from +0:            */
/*   y_i = fma(M_i,d-1, x_d-1, ... fma(M_i,1, x_1, fma(M_i,0, x_0, 0))),     */
/* with M = Q (transpose = 0) or Q^T (transpose = 1), Q row-major [d][d].   */
/* x and y are [rows][d], fp32 or bf16 bits (y rounded to nearest even).    */
/* ------------------------------------------------------------------------ */
void hqo_rotate(const float *Q, uint32_t d, uint32_t transpose, const void *x, uint32_t x_dtype,
                uint64_t rows, void *y, uint32_t y_dtype)
{
    float *xv = (float *)malloc(sizeof(float) * d);
    for (uint64_t r = 0; r < rows; r++) {
        for (uint32_t j = 0; j < d; j++)
            xv[j] = x_dtype == HQO_BF16 ? bf16_to_f32(((const uint16_t *)x)[r * d + j])
                                        : ((const float *)x)[r * d + j];
        for (uint32_t i = 0; i < d; i++) {
            float acc = 0.0f;
            for (uint32_t j = 0; j < d; j++) {
                const float m = transpose ? Q[(uint64_t)j * d + i] : Q[(uint64_t)i * d + j];
                acc = fmaf(m, xv[j], acc);
            }
            if (y_dtype == HQO_BF16) ((uint16_t *)y)[r * d + i] = bf16_rne(acc);
            else ((float *)y)[r * d + i] = acc;
        }
    }
    free(xv);
}

/* ------------------------------------------------------------------------ */
/* Decode into integer codes for an int8 matrix product (the pages name     */
/* int8 matrix-core paths on the post-RHT lattice output, the lattice's     */
/* integer embedding fitting 8 bits; gist.science explainer of HyperQuant,  */
/* Key Contributions, "Hardware Integration", and Methodology section 2).   */
/* Reading: a tile's codes are 2 P (P its lattice point, so 2 P is an       */
/* integer vector for Z, D4 and E8), saturated to [-127, 127] (flagged);    */
/* its weights are then D H (s P) / sqrt(n), so a row of the weight matrix  */
/* times an activation x is sum over tiles of s_t <P_t, RHT(x)_t>.  The     */
/* activation's RHT is quantized per tile to int8 with scale a_t =          */
/* fl(max|RHT(x)_t| / 127), q = rint(fl(RHT(x)_i / a_t)), and              */
/*   y[b][r] = 0.5 * (fma chain over tiles t ascending, from +0, of          */
/*             (float) I_t * fl(s_t * a_t)),  I_t = <codes_t, q_t> (exact).  */
/* ------------------------------------------------------------------------ */
int hqo_decode_codes(const uint16_t *step, const uint16_t *meta, const uint32_t *chunk_off,
                     const uint32_t *payload, uint64_t payload_words, const hqo_params *p, int8_t *codes,
                     uint32_t *range_flag)
{
    int rc = check_params(p);
    if (rc) return rc;
    if (p->dither || p->lattice == HQO_A2) return HQO_EINVAL;
    uint32_t n = p->tile, d = lattice_dim(p->lattice);
    uint32_t nb = (n / d) * coset_bits_per_block(p->lattice);
    uint64_t T = p->rows * p->cols / n;
    uint64_t C = (T + HQO_CHUNK_TILES - 1) / HQO_CHUNK_TILES;
    uint64_t chunk_cap = ((uint64_t)HQO_CHUNK_TILES * hqo_tile_bound_bits(p) + 31) / 32;
    int status = HQO_OK;
    uint32_t cos[256], sym[256], zero[8] = {0};
    *range_flag = 0;
    for (uint64_t c = 0; c < C; c++) {
        uint64_t w0 = chunk_off[c], w1 = chunk_off[c + 1];
        uint64_t t0 = c * HQO_CHUNK_TILES, t1 = t0 + HQO_CHUNK_TILES;
        if (t1 > T) t1 = T;
        uint64_t total = 0;
        int too_long = 0;
        for (uint64_t t = t0; t < t1; t++) {
            total += meta[t] >> 3;
            if ((uint32_t)(meta[t] >> 3) > hqo_tile_bound_bits(p)) too_long = 1;
        }
        int chunk_bad = !(w1 >= w0 && w1 <= payload_words && w1 - w0 <= chunk_cap)
                        || too_long || (total + 31) / 32 != w1 - w0;
        uint64_t b = w0 * 32, bend = w1 * 32;
        for (uint64_t t = t0; t < t1; t++) {
            uint32_t len = meta[t] >> 3, k = meta[t] & 7u;
            int bad = chunk_bad || step_bad(step[t]) || parse_tile(payload, b, bend, len, k, n, nb, cos, sym);
            if (bad) status = HQO_ECORRUPT;
            for (uint32_t blk = 0; blk < n / d; blk++) {
                float pt[8];
                uint32_t pc = (coset_bits_per_block(p->lattice) && !bad) ? cos[blk] : 0;
                block_point(p->lattice, pc, bad ? zero : sym + blk * d, pt);
                for (uint32_t i = 0; i < d; i++) {
                    long v = lrintf(2.0f * pt[i]);
                    if (v > 127) { v = 127; *range_flag = 1; }
                    if (v < -127) { v = -127; *range_flag = 1; }
                    codes[t * n + blk * d + i] = (int8_t)v;
                }
            }
            b += len;
        }
    }
    return status;
}

void hqo_act_quant(const float *x, uint64_t batch, uint64_t cols, uint32_t n, uint64_t seed, int8_t *q,
                   float *scale)
{
    float y[256];
    for (uint64_t b = 0; b < batch; b++)
        for (uint64_t t = 0; t < cols / n; t++) {
            hqo_rht_forward(x + b * cols + t * n, n, seed, y);
            /* max |y|, a NaN kept (reading: the pages are silent on
             * non-finite activations; a NaN or an infinity makes the tile's
             * scale non-finite, every code whose quotient is NaN is 0, and the
             * product over the tile is then NaN) */
            float m = 0.0f;
            for (uint32_t i = 0; i < n; i++) {
                float v = fabsf(y[i]);
                if (isnan(v) || v > m) m = v;
            }
            float a = m / 127.0f;
            scale[b * (cols / n) + t] = a;
            for (uint32_t i = 0; i < n; i++) {
                long v = 0;
                if (a != 0.0f) {
                    float r = y[i] / a;
                    v = isnan(r) ? 0 : lrintf(r);
                }
                q[b * cols + t * n + i] = (int8_t)(v > 127 ? 127 : (v < -127 ? -127 : v));
            }
        }
}

void hqo_codes_matmul(const int8_t *codes, const uint16_t *step, uint64_t rows, uint64_t cols, uint32_t n,
                      const int8_t *q, const float *scale, uint64_t batch, float *y)
{
    uint64_t tr = cols / n;
    for (uint64_t b = 0; b < batch; b++)
        for (uint64_t r = 0; r < rows; r++) {
            float acc = 0.0f;
            for (uint64_t t = 0; t < tr; t++) {
                int32_t I = 0;
                for (uint32_t i = 0; i < n; i++)
                    I += (int32_t)codes[r * cols + t * n + i] * (int32_t)q[b * cols + t * n + i];
                float w = bf16_to_f32(step[r * tr + t]) * scale[b * tr + t];
                acc = fmaf((float)I, w, acc);
            }
            y[b * rows + r] = 0.5f * acc;
        }
}
