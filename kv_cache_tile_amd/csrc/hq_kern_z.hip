// hq_kern_z.hip — the Z lattice's encode, length-pass, decode and
// quantiser kernels (every tile size, with and without the KV dither),
// instantiated in a translation unit of their own so that the four
// lattices compile in parallel.
#include "hq_kernels.h"

namespace hq {
EncFn enc_fn_z(uint32_t n, bool dither, bool bf16) { return enc_table<1>(n, dither, bf16); }
LenFn len_fn_z(uint32_t n, bool dither, bool bf16) { return len_table<1>(n, dither, bf16); }
DecFn dec_fn_z(uint32_t n, bool dither) { return dec_table<1>(n, dither); }
NearFn near_fn_z() { return nearest_kernel<1>; }
DecFn dec_codes_fn_z(uint32_t n) { return dec_codes_table<1>(n); }
}  // namespace hq
