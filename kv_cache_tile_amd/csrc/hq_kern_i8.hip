// hq_kern_i8.hip — the int8 product path on the matrix cores (gist.science
// explainer of HyperQuant, Key Contributions, "Hardware Integration": int8
// matrix-core products on the post-RHT lattice output; Methodology section 2:
// the lattice's integer embedding fits 8 bits).
//
// A weight tile decodes to D H (s P) / sqrt(n), so a weight row times an
// activation x is the sum over the row's tiles of s_t <P_t, RHT(x)_t>.  The
// decoder writes the integer codes 2P (int8); act_quant_kernel rotates each
// activation tile with the codec's RHT and quantizes it to int8 with scale
// a_t = fl(max |RHT(x)_t| / 127); the product forms the exact int32 tile
// products on the matrix cores and accumulates
//   y[b][r] = 0.5 * fma chain over tiles t ascending, from +0, of
//             (float) I_t * fl(s_t * a_t)
// in that order, so every output is bit-exact against a plain loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq_device.h"

namespace hq {

// One workgroup of N / 2 threads per activation tile: sign diagonal (the
// codec's sign bits of positions 0 .. n-1), the butterfly with strides 1, 2,
// ..., n/2 in LDS, the scale fl(1/sqrt(n)), then max |y| and the int8 codes.
// BLOCKED: the codes in the matrix cores' operand order, so that one 16-byte
// load a lane brings a whole 32-code step of 32 activations from 1 KB of
// contiguous memory: code (b, column t n + 32 k + j) at
// (((b / 32) T + t) (n / 32) + k) 1024 + (b % 32) 32 + j, T = tiles a row.
template <int N, bool BLOCKED>
__global__ void __launch_bounds__(N / 2)
act_quant_kernel(const void* __restrict__ x, uint32_t xbf16, uint64_t tiles_per_row, uint32_t key_sign,
                 float inv_sqrtn, int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float y[N];
  __shared__ float red[N / 2];
  const int k = threadIdx.x;
  const uint64_t tile = blockIdx.x;                         // (b, t) row-major: tile index in the activations
  const uint64_t base = tile * N;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int i = k + h * (N / 2);
    float v = xbf16 ? as_f((uint32_t)reinterpret_cast<const uint16_t*>(x)[base + i] << 16)
                    : reinterpret_cast<const float*>(x)[base + i];
    if (pcg_hash(key_sign + (uint32_t)i) >> 31) v = -v;
    y[i] = v;
  }
  __syncthreads();
  for (int h = 1; h < N; h <<= 1) {
    const int j = (k / h) * 2 * h + (k % h);
    const float lo = y[j], hi = y[j + h];
    __syncthreads();
    y[j] = lo + hi;
    y[j + h] = lo - hi;
    __syncthreads();
  }
  const float v0 = y[k] * inv_sqrtn, v1 = y[k + N / 2] * inv_sqrtn;
  // max |y| with a NaN kept (a NaN or an infinity in the tile makes its scale
  // non-finite; a code whose quotient is NaN is 0, so the tile's products are
  // NaN downstream)
  auto nan_max = [](float u, float v) { return (u != u || v != v) ? u + v : fmaxf(u, v); };
  red[k] = nan_max(fabsf(v0), fabsf(v1));
  __syncthreads();
  for (int m = N / 4; m > 0; m >>= 1) {
    if (k < m) red[k] = nan_max(red[k], red[k + m]);
    __syncthreads();
  }
  const float a = red[0] / 127.0f;
  auto code = [&](float v) -> int8_t {
    if (a == 0.0f) return 0;
    float r = rintf(v / a);
    if (r != r) return 0;
    r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
    return (int8_t)(int)r;
  };
  if constexpr (BLOCKED) {
    const uint64_t b = tile / tiles_per_row, t = tile % tiles_per_row;
    int8_t* qt = q + (((b >> 5) * tiles_per_row + t) * (N / 32)) * 1024 + (b & 31) * 32;
    qt[(k >> 5) * 1024 + (k & 31)] = code(v0);
    qt[((k + N / 2) >> 5) * 1024 + (k & 31)] = code(v1);
  } else {
    q[base + k] = code(v0);
    q[base + k + N / 2] = code(v1);
  }
  if (k == 0) scale[tile] = a;
}

// The product in two passes, so that the tiles' exact int32 products run in
// parallel and only the fp32 chain is sequential.
// Pass 1: one wave per (32 rows, one tile, 32 activations), four waves to a
// workgroup.
// v_mfma_i32_32x32x32_i8 takes 16 codes per lane from each operand (lane
// l: row / activation l % 32, the 16-byte half l / 32 of the 32-code step;
// both operands use the same split, so every product is summed once), exact
// in int32.  Output layout: register r of lane l holds row
// (r / 4) 8 + (l / 32) 4 + r % 4, activation l % 32.  I goes to
// work[t][r][b] (a store of one register is two 128-byte runs).
typedef int i8_i32x16 __attribute__((ext_vector_type(16)));
typedef int i8_i32x4 __attribute__((ext_vector_type(4)));

template <int N>
__global__ void __launch_bounds__(256)
codes_tile_products_kernel(const int8_t* __restrict__ codes, uint64_t rows, uint64_t cols,
                           const int8_t* __restrict__ q, uint64_t batch, int32_t* __restrict__ work) {
  // a workgroup: 128 rows (a wave per 32) x one tile x 32 activations; the
  // tile's codes and activation codes are staged in LDS with coalesced
  // 16-byte loads (rows padded by 16 bytes against bank conflicts), the
  // activations once for the four waves
  constexpr int RS = N + 16;                                // LDS row stride in bytes
  __shared__ __attribute__((aligned(16))) int8_t sa[128 * RS];
  __shared__ __attribute__((aligned(16))) int8_t sb[32 * RS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t r0 = (uint64_t)blockIdx.x * 128, t = blockIdx.y, b0 = (uint64_t)blockIdx.z * 32;
  const uint64_t tr = cols / N;
  constexpr int CH = N / 16;                                // 16-byte chunks per row
  const i8_i32x4 zero4 = {0, 0, 0, 0};
  for (int e = tid; e < 128 * CH; e += 256) {
    const int r = e / CH, ch = e % CH;
    const uint64_t row = r0 + (uint64_t)r;
    *reinterpret_cast<i8_i32x4*>(sa + r * RS + 16 * ch) =
        row < rows ? *reinterpret_cast<const i8_i32x4*>(codes + row * cols + t * N + 16 * ch) : zero4;
  }
  for (int e = tid; e < 32 * CH; e += 256) {
    const int r = e / CH, ch = e % CH;
    const uint64_t bb = b0 + (uint64_t)r;
    *reinterpret_cast<i8_i32x4*>(sb + r * RS + 16 * ch) =
        bb < batch ? *reinterpret_cast<const i8_i32x4*>(q + bb * cols + t * N + 16 * ch) : zero4;
  }
  __syncthreads();
  const int arow = 32 * wave + (lane & 31), bcol = lane & 31;
  const int half = (lane >> 5) * 16;
  i8_i32x16 I = {};
#pragma unroll
  for (int ks = 0; ks < N / 32; ks++) {
    const i8_i32x4 av = *reinterpret_cast<const i8_i32x4*>(sa + arow * RS + 32 * ks + half);
    const i8_i32x4 bv = *reinterpret_cast<const i8_i32x4*>(sb + bcol * RS + 32 * ks + half);
    I = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, I, 0, 0, 0);
  }
  const uint64_t bg = b0 + (uint64_t)bcol;
  if (bg >= batch) return;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const uint64_t row = r0 + (uint64_t)(32 * wave + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3));
    if (row < rows) work[(t * rows + row) * batch + bg] = I[i];
  }
}

// Pass 2: one thread per output (activation index fastest, so each tile's
// reads are contiguous), the fp32 chain over the row's tiles in ascending
// order.
__global__ void __launch_bounds__(256)
codes_chain_kernel(const int32_t* __restrict__ work, const uint16_t* __restrict__ step, uint64_t rows, uint64_t tr,
                   const float* __restrict__ scale, uint64_t batch, float* __restrict__ y) {
  const uint64_t o = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= rows * batch) return;
  const uint64_t r = o / batch, b = o % batch;
  float acc = 0.0f;
  // (the loads of 8 tiles issued ahead of their chain steps)
#pragma unroll 8
  for (uint64_t t = 0; t < tr; t++) {
    const float w = as_f((uint32_t)step[r * tr + t] << 16) * scale[b * tr + t];
    acc = __builtin_fmaf((float)work[(t * rows + r) * batch + b], w, acc);
  }
  y[b * rows + r] = 0.5f * acc;
}

const void* act_quant_fn(uint32_t n, bool blocked) {
  if (n == 64) return blocked ? (const void*)act_quant_kernel<64, true> : (const void*)act_quant_kernel<64, false>;
  if (n == 128) return blocked ? (const void*)act_quant_kernel<128, true> : (const void*)act_quant_kernel<128, false>;
  if (n == 256) return blocked ? (const void*)act_quant_kernel<256, true> : (const void*)act_quant_kernel<256, false>;
  return nullptr;
}
// both passes on `stream` (shapes checked by the caller); false on a launch error
bool launch_codes_matmul(const int8_t* codes, const uint16_t* step, uint64_t rows, uint64_t cols, uint32_t n,
                         const int8_t* q, const float* scale, uint64_t batch, float* y, int32_t* work,
                         hipStream_t stream) {
  const uint64_t tr = cols / n;
  const dim3 grid((uint32_t)((rows + 127) / 128), (uint32_t)tr, (uint32_t)((batch + 31) / 32));
  if (n == 64) hipLaunchKernelGGL(codes_tile_products_kernel<64>, grid, dim3(256), 0, stream, codes, rows, cols, q, batch, work);
  else if (n == 128) hipLaunchKernelGGL(codes_tile_products_kernel<128>, grid, dim3(256), 0, stream, codes, rows, cols, q, batch, work);
  else hipLaunchKernelGGL(codes_tile_products_kernel<256>, grid, dim3(256), 0, stream, codes, rows, cols, q, batch, work);
  if (hipGetLastError() != hipSuccess) return false;
  hipLaunchKernelGGL(codes_chain_kernel, dim3((uint32_t)((rows * batch + 255) / 256)), dim3(256), 0, stream, work,
                     step, rows, tr, scale, batch, y);
  return hipGetLastError() == hipSuccess;
}

}  // namespace hq
