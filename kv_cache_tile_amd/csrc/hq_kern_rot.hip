// hq_kern_rot.hip — the KV path's per-layer rotation by a Haar-uniform
// orthogonal matrix (gist.science explainer of HyperQuant, Methodology
// section 4, "Bias Correction for KV Cache": a Haar rotation as the
// alternative to the sign diagonal).  The vectors are rotated, y = Q x,
// before the codec's own per-tile RHT, and decode applies Q^T after the
// codec's inverse; H D Q is Haar-uniform whenever Q is.
//
// Every output is one fused multiply-add chain over j = 0 .. D-1 in
// ascending order from +0, so the result is a pure function of (Q, x) and
// bit-exact across implementations.  The contraction runs on the matrix
// cores with one product per output per instruction (below), which keeps
// that order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq_device.h"

namespace hq {

// v_mfma_f32_32x32x1_2b_f32 adds one product to each output of two 32 x 32
// blocks per instruction, rounded once like a fused multiply-add (bit-equal
// to fmaf over normal, subnormal and cancelling operands, and pinned by the
// parity tests against the oracle's chains), so issuing it for j = 0 .. D-1
// in order gives each output exactly the ascending chain.  A wave owns 32
// rows and all D outputs: both blocks take the same 32 rows (lanes l and
// l + 32 supply the x of row l % 32 of the wave's slab) and instruction t
// covers outputs 64 t .. 64 t + 63 (block b the 32 from 64 t + 32 b), D / 64
// instructions per j.  That keeps 64 accumulators per lane for D = 128, so
// several waves share a SIMD.  x streams from global memory 8 values at a
// time (the next 8 in flight); the matrix sits in LDS as Mt[j][i].  Output
// layout of a block: register r of lane l holds row (r / 4) 8 + (l / 32) 4 +
// r % 4, column l % 32.
typedef float rot_f32x32 __attribute__((ext_vector_type(32)));
constexpr int kRotMfmaWaves = 8;

template <int D, bool XBF16, bool YBF16>
__global__ void __launch_bounds__(64 * kRotMfmaWaves)
rotate_mfma_kernel(const float* __restrict__ Q, uint32_t transpose, const void* __restrict__ x, uint64_t rows,
                   void* __restrict__ y) {
  constexpr int IT = D / 64;
  extern __shared__ float rsm[];
  float* Mt = rsm;                       // [D][D]
  const int tid = threadIdx.x;
  for (int e = tid; e < D * D; e += 64 * kRotMfmaWaves) {
    const int a = e / D, b = e % D;
    const float v = Q[e];
    if (transpose) Mt[a * D + b] = v;
    else Mt[b * D + a] = v;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t nblk = (rows + 31) / 32;                  // 32-row slabs, one per wave at a time
  for (uint64_t blk = (uint64_t)blockIdx.x * kRotMfmaWaves + wave; blk < nblk;
       blk += (uint64_t)gridDim.x * kRotMfmaWaves) {
    const uint64_t row = blk * 32 + (uint64_t)(lane & 31);
    const bool live = row < rows;
    rot_f32x32 acc[IT];
#pragma unroll
    for (int t = 0; t < IT; t++)
#pragma unroll
      for (int r = 0; r < 32; r++) acc[t][r] = 0.0f;
    // x of this lane's row, 8 values per step, the next step's load in flight
    // while the current one feeds the matrix cores
    auto load8 = [&](int j0, uint32_t (&w)[8]) {
      if (XBF16) {
        const uint4 v = live ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + row * D + j0)
                             : make_uint4(0u, 0u, 0u, 0u);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + row * D + j0);
        const float4 a0 = live ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 a1 = live ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
        w[0] = as_u(a0.x); w[1] = as_u(a0.y); w[2] = as_u(a0.z); w[3] = as_u(a0.w);
        w[4] = as_u(a1.x); w[5] = as_u(a1.y); w[6] = as_u(a1.z); w[7] = as_u(a1.w);
      }
    };
    uint32_t wn[8];
    load8(0, wn);
#pragma unroll 1
    for (int j0 = 0; j0 < D; j0 += 8) {
      uint32_t w[8];
#pragma unroll
      for (int k = 0; k < 8; k++) w[k] = wn[k];
      if (j0 + 8 < D) load8(j0 + 8, wn);
      float xv[8];
      if (XBF16) {
#pragma unroll
        for (int h = 0; h < 4; h++) {
          xv[2 * h] = as_f(w[h] << 16);
          xv[2 * h + 1] = as_f(w[h] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 8; k++) xv[k] = as_f(w[k]);
      }
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const float* mrow = Mt + (j0 + jj) * D + lane;
#pragma unroll
        for (int t = 0; t < IT; t++)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x1f32(xv[jj], mrow[64 * t], acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < IT; t++) {
#pragma unroll
      for (int r = 0; r < 32; r++) {
        const int b = r >> 4, rr = r & 15;
        const int col = 64 * t + 32 * b + (lane & 31);
        const uint64_t orow = blk * 32 + (uint64_t)((rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3));
        if (orow < rows) {
          if (YBF16) {
            const uint32_t h = bf16x2_rne(acc[t][r], 0.0f) & 0xFFFFu;
            reinterpret_cast<uint16_t*>(y)[orow * D + col] = (uint16_t)h;
          } else {
            reinterpret_cast<float*>(y)[orow * D + col] = acc[t][r];
          }
        }
      }
    }
  }
}

using RotFn = void (*)(const float*, uint32_t, const void*, uint64_t, void*);

template <int D>
RotFn rot_mfma_table_d(bool xbf16, bool ybf16) {
  if (xbf16) return ybf16 ? rotate_mfma_kernel<D, true, true> : rotate_mfma_kernel<D, true, false>;
  return ybf16 ? rotate_mfma_kernel<D, false, true> : rotate_mfma_kernel<D, false, false>;
}

// the matrix-core kernel for (d, input dtype, output dtype), its LDS bytes,
// threads and rows per workgroup pass; null for an unsupported d
const void* rot_mfma_fn(uint32_t d, bool xbf16, bool ybf16, size_t* lds, uint32_t* threads, uint32_t* rows_per_block) {
  *threads = 64 * kRotMfmaWaves;
  *rows_per_block = 32 * kRotMfmaWaves;
  if (d == 64) { *lds = 64 * 64 * 4; return (const void*)rot_mfma_table_d<64>(xbf16, ybf16); }
  if (d == 128) { *lds = 128 * 128 * 4; return (const void*)rot_mfma_table_d<128>(xbf16, ybf16); }
  return nullptr;
}

}  // namespace hq
