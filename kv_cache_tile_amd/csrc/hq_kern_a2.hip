// hq_kern_a2.hip — the A2 lattice's encode, length-pass, decode and
// quantiser kernels (every tile size, with and without the KV dither),
// instantiated in a translation unit of their own so that the four
// lattices compile in parallel.
#include "hq_kernels.h"

namespace hq {
EncFn enc_fn_a2(uint32_t n, bool dither, bool bf16) { return enc_table<2>(n, dither, bf16); }
LenFn len_fn_a2(uint32_t n, bool dither, bool bf16) { return len_table<2>(n, dither, bf16); }
DecFn dec_fn_a2(uint32_t n, bool dither) { return dec_table<2>(n, dither); }
NearFn near_fn_a2() { return nearest_kernel<2>; }
}  // namespace hq
