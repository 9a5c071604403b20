// hq_kern_e8.hip — the E8 lattice's encode, length-pass, decode and
// quantiser kernels (every tile size, with and without the KV dither),
// instantiated in a translation unit of their own so that the four
// lattices compile in parallel.
#include "hq_kernels.h"

namespace hq {
EncFn enc_fn_e8(uint32_t n, bool dither, bool bf16) { return enc_table<8>(n, dither, bf16); }
LenFn len_fn_e8(uint32_t n, bool dither, bool bf16) { return len_table<8>(n, dither, bf16); }
DecFn dec_fn_e8(uint32_t n, bool dither) { return dec_table<8>(n, dither); }
NearFn near_fn_e8() { return nearest_kernel<8>; }
DecFn dec_codes_fn_e8(uint32_t n) { return dec_codes_table<8>(n); }
}  // namespace hq
