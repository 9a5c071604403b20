// hq_lib.hip — host side and C ABI of libhq.so (declared in include/hq.h):
// argument checks, the frozen rate table, worst-case sizes, and the launches
// of the encode/decode kernels (hq_kernels.h, one translation unit per
// lattice).
//
// Method: "HyperQuant: A Rate-Distortion-Optimal Quantization Pipeline for
// Large Language and Diffusion Models", gist.science explainer, section
// "Methodology: The HyperQuant Pipeline".
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "hq.h"
#include "hq_kernels.h"

namespace hq {
// hq_kern_rot.hip: the rotation kernel for (d, input, output dtype), its LDS
// bytes, threads and rows per workgroup pass (null for an unsupported d)
const void* rot_mfma_fn(uint32_t d, bool xbf16, bool ybf16, size_t* lds, uint32_t* threads,
                        uint32_t* rows_per_block);
// hq_kern_i8.hip: the int8 product path's kernels for tile size n (null otherwise)
const void* act_quant_fn(uint32_t n, bool blocked);
bool launch_codes_matmul(const int8_t* codes, const uint16_t* step, uint64_t rows, uint64_t cols, uint32_t n,
                         const int8_t* q, const float* scale, uint64_t batch, float* y, int32_t* work,
                         hipStream_t stream);
// hq_kern_fused.hip: the product read from the stream, for (lattice, n); its
// threads and LDS bytes for segments of seg_words (null if unsupported)
const void* fused_fn(uint32_t lattice, uint32_t n, uint32_t seg_words, uint32_t* threads, size_t* lds);
constexpr int kFusedRowsHost = 8, kFusedColsHost = 8, kFusedBatchHost = 32;   // as in hq_kern_fused.hip
}  // namespace hq

using namespace hq;

namespace {

struct RateEntry { uint8_t lattice, dither; uint16_t tile; uint16_t bps_q; uint32_t c_bits; };
#include "hq_rate_table.inc"   // kRateTable[], generated from rate_table.json

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
  uint32_t bound, chunk_words;
  float c;
};

// the encode look-back's bound on polls of an unpublished predecessor
constexpr uint32_t kSpinLimit = 1u << 20;

// closed-loop rate: targets accepted, tolerance in bits per scalar, most encodes
constexpr float kRateMin = 1.0f, kRateMax = 8.0f;
constexpr double kRateTol = 0.01;
constexpr uint32_t kRateIters = 30;

// sizes for an explicit rate constant c (finite and positive)
int plan_for_c(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lat, float c,
               uint32_t kv, Plan* P) {
  if (dtype != HQ_F32 && dtype != HQ_BF16) return HQ_EINVAL;
  if (tile != 64 && tile != 128 && tile != 256) return HQ_EINVAL;
  if (!lattice_dim(lat) || kv > 1) return HQ_EINVAL;
  if (rows == 0 || cols == 0 || cols % tile) return HQ_EINVAL;
  if (rows > (1ull << 32) || cols > (1ull << 32) || rows * cols >= (1ull << 32)) return HQ_EINVAL;
  if (!(c > 0.0f) || !(c <= 3.0e38f)) return HQ_EINVAL;
  uint32_t bound = tile_bound_bits(tile, lat, kv, c);
  if (!bound) return HQ_EINVAL;
  P->T = rows * cols / tile;
  P->C = (P->T + kChunkTiles - 1) / kChunkTiles;
  P->bound = bound;
  P->c = c;
  P->chunk_words = (uint32_t)(((uint64_t)kChunkTiles * bound + 31) / 32) + 1;   // one chunk, word-aligned
  P->cap_words = (P->T * bound + 31) / 32 + P->C;
  P->ws_bytes = 4 * kLookBase + 8 * P->C;
  return HQ_OK;
}

// sizes for a target rate on the frozen table's grid
int make_plan(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lat, float bps,
              uint32_t kv, Plan* P) {
  float c;
  if (!lattice_dim(lat) || kv > 1 || !rate_constant(lat, tile, kv, bps, &c)) return HQ_EINVAL;
  return plan_for_c(dtype, rows, cols, tile, lat, c, kv, P);
}

EncFn enc_fn(uint32_t lat, uint32_t n, bool dither, bool bf16) {
  switch (lat) {
    case HQ_Z: return enc_fn_z(n, dither, bf16);
    case HQ_A2: return enc_fn_a2(n, dither, bf16);
    case HQ_D4: return enc_fn_d4(n, dither, bf16);
    default: return enc_fn_e8(n, dither, bf16);
  }
}
LenFn len_fn(uint32_t lat, uint32_t n, bool dither, bool bf16) {
  switch (lat) {
    case HQ_Z: return len_fn_z(n, dither, bf16);
    case HQ_A2: return len_fn_a2(n, dither, bf16);
    case HQ_D4: return len_fn_d4(n, dither, bf16);
    default: return len_fn_e8(n, dither, bf16);
  }
}
DecFn dec_fn(uint32_t lat, uint32_t n, bool dither) {
  switch (lat) {
    case HQ_Z: return dec_fn_z(n, dither);
    case HQ_A2: return dec_fn_a2(n, dither);
    case HQ_D4: return dec_fn_d4(n, dither);
    default: return dec_fn_e8(n, dither);
  }
}

// LDS is granted to a workgroup in blocks of a few hundred bytes: on MI355X
// five workgroups of exactly a fifth of a CU's 160 KB (32768 bytes) do not fit
// together, although the occupancy query counts five; five of 32000 bytes do.
// Per-workgroup LDS budgets derived from a CU share are rounded down to this
// grain (a multiple of 320, 640 and 1280 bytes).
constexpr size_t kLdsGrain = 1280;

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

int do_encode(const Plan& P, const void* x, uint32_t dtype, uint32_t tile, uint32_t lat, uint64_t seed,
              uint32_t kv, uint32_t* payload, uint64_t cap, uint16_t* step, uint16_t* meta, uint32_t* chunk_off,
              uint32_t* status, void* ws, uint64_t ws_bytes, void* stream) {
  int rc;
  if (!x || !payload || !step || !meta || !chunk_off || !status || !ws) return HQ_EINVAL;
  if (cap < P.cap_words || ws_bytes < P.ws_bytes) return HQ_ENOSPC;
  if (((uintptr_t)x & 15) || ((uintptr_t)ws & 7)) return HQ_EINVAL;
  EncFn fn = enc_fn(lat, tile, kv != 0, dtype == HQ_BF16);
  const int block = kChunkTiles * (int)(tile / kLaneElems);
  // chunks staged per ticket: as many (up to kMaxGroupChunks) as fit the LDS
  // share of a workgroup at the occupancy its registers allow; the staging
  // area takes the whole share, room for a second group's words
  int dev = 0, max_lds = 0, lds_cu = 0, per_regs = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_regs, (const void*)fn, block, 0) != hipSuccess)
    return HQ_EHIP;
  size_t lds_cap = per_regs > 0 ? (size_t)lds_cu / (size_t)per_regs : (size_t)max_lds;
  if (lds_cap > (size_t)max_lds) lds_cap = (size_t)max_lds;
  lds_cap = lds_cap / kLdsGrain * kLdsGrain;
  const size_t fixed_words = 2 * kChunkTiles + 4 + 8 + 2 * kMaxGroupChunks + kStartedWords + 16 * 8;
  const size_t avail = lds_cap / 4 > fixed_words ? lds_cap / 4 - fixed_words : 0;
  uint32_t group = kMaxGroupChunks, grp_words = 0;
  // (group areas start on 16-byte boundaries: both sizes multiples of 4 words)
  for (;; group--) {
    grp_words = (group * P.chunk_words + 4 + 3) & ~3u;
    if (grp_words <= (avail & ~(size_t)3) || group == 1) break;
  }
  const uint32_t stage_words = (avail & ~(size_t)3) > grp_words ? (uint32_t)(avail & ~(size_t)3) : grp_words;
  const size_t lds = (stage_words + fixed_words) * 4;
  if (lds > (size_t)max_lds) return HQ_EINVAL;
  int grid_full;
  rc = grid_for((const void*)fn, block, lds, UINT64_MAX, &grid_full);
  if (rc) return rc;
  // a smaller grid on request (tests use it so that few chunks still give a
  // workgroup several groups, alternating between the staging halves)
  if (const char* e = getenv("HQ_ENCODE_GRID_CAP")) {
    const long v = strtol(e, nullptr, 10);
    if (v > 0 && v < grid_full) grid_full = (int)v;
  }
  // Chunks per group, at most the size that fits: a workgroup runs its
  // groups' chunks one after another, so the last to finish has run about
  // ceil(groups / grid) groups of `group` chunks.  Every group past the
  // grid's first ones is drawn from one atomic counter, whose draws are
  // served one at a time: 9984 single-chunk draws (11008 chunks over 1024
  // workgroups) took milliseconds.  So each round of draws (grid draws) is
  // charged half a chunk, and the size of least cost, the largest (fewest
  // look-backs) on a tie, is taken: 4096 chunks over 512 workgroups (4 waves a
  // SIMD) keep groups of 4, 5504 over 1024 take groups of 3 (2 rounds of 3 chunks
  // rather than 2 of 4), 2048 over 1024 groups of 2, and 11008 over 1024
  // groups of 4 (12 chunks a workgroup, 1728 draws) rather than 1 (11 chunks,
  // 9984 draws).  The cost below is in units of 1 / (2 grid) chunks.
  // A workgroup that runs more than one group places each finished group
  // while packing the next into the other area; where the two areas overlap
  // so far that a group's words (taken as 7/8 of its worst case) would reach
  // the other area, the placement is forced early and its look-back waits
  // on the critical path, so such sizes are passed over.  The DiT layer at 6
  // waves a SIMD (4096 chunks over 768 workgroups, 13100 staging words)
  // takes groups of 2 instead of 3: 82.1 against 84.2 us, interleaved runs.
  const uint32_t gmax = group;
  uint64_t best = UINT64_MAX;
  for (uint32_t g = gmax; g >= 1u; g--) {
    const uint64_t groups = (P.C + g - 1) / g;
    const uint64_t span = (groups + (uint64_t)grid_full - 1) / (uint64_t)grid_full * g;
    const uint64_t cost = 2 * span * (uint64_t)grid_full + (groups > (uint64_t)grid_full ? groups - grid_full : 0);
    const uint64_t gw_g = ((uint64_t)g * P.chunk_words + 4 + 3) & ~3ull;
    const bool overlaps = 2 * gw_g * 7 > 8 * (uint64_t)stage_words;
    if (g > 1u && groups > (uint64_t)grid_full && overlaps) continue;
    if (cost < best) { best = cost; group = g; }
  }
  if (const char* e = getenv("HQ_ENCODE_GROUP_CHUNKS")) {   // (tests: a fixed group size)
    const long v = strtol(e, nullptr, 10);
    if (v > 0 && (uint32_t)v <= gmax) group = (uint32_t)v;
  }
  grp_words = group * P.chunk_words + 4;
  const uint64_t groups = (P.C + group - 1) / group;
  if (grid_full > (int)(32 * kStartedWords)) grid_full = (int)(32 * kStartedWords);   // the started array's size
  int grid = groups < (uint64_t)grid_full ? (int)groups : grid_full;
  // a grid of a given size, up to the group count, on request (tests use
  // one several times larger than can be resident at once)
  if (const char* e = getenv("HQ_ENCODE_GRID")) {
    const long v = strtol(e, nullptr, 10);
    if (v > 0) grid = (uint64_t)v < groups ? (int)v : (int)groups;
    if (grid > (int)(32 * kStartedWords)) grid = (int)(32 * kStartedWords);
  }
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  const float inv_sqrtn = (float)(1.0 / sqrt((double)tile));
  const float inv_n = 1.0f / (float)tile;   // exact: tile is a power of two
  // polls of a look-back before it gives up (HQ_FLAG_STALL): each poll waits
  // on a device-scope load, so the default is about a second, far beyond any
  // wait for a running predecessor; tests lower it to reach the flag
  uint32_t spin_limit = kSpinLimit;
  if (const char* e = getenv("HQ_ENCODE_SPIN_LIMIT")) {
    const long v = strtol(e, nullptr, 10);
    if (v >= 0 && v < (long)kSpinLimit) spin_limit = (uint32_t)v;
  }
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, (hipStream_t)stream, x, (uint32_t)(dtype == HQ_BF16), P.T, P.C, P.c, inv_sqrtn, inv_n,
                     derive_key(seed, 0x5349474Eu), derive_key(seed, 0x44495448u), a2, payload, cap, step, meta,
                     chunk_off, status, (uint32_t*)ws, stage_words, grp_words, group, spin_limit);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

// the length pass: adds to *words (device) the payload words an encode with
// plan P would write
int do_length(const Plan& P, const void* x, uint32_t dtype, uint32_t tile, uint32_t lat, uint64_t seed,
              uint32_t kv, unsigned long long* words, void* stream) {
  if (!x || !words) return HQ_EINVAL;
  if (((uintptr_t)x & 15) || ((uintptr_t)words & 7)) return HQ_EINVAL;
  if (P.C == 0) return HQ_OK;
  LenFn fn = len_fn(lat, tile, kv != 0, dtype == HQ_BF16);
  const int block = kChunkTiles * (int)(tile / kLaneElems);
  int grid;
  int rc = grid_for((const void*)fn, block, 0, P.C, &grid);
  if (rc) return rc;
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  const float inv_sqrtn = (float)(1.0 / sqrt((double)tile));
  const float inv_n = 1.0f / (float)tile;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), 0, (hipStream_t)stream, x, P.T, P.C, P.c, inv_sqrtn, inv_n,
                     derive_key(seed, 0x5349474Eu), derive_key(seed, 0x44495448u), a2, words);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

int do_decode(const Plan& P, const uint32_t* payload, uint64_t payload_words, const uint16_t* step,
              const uint16_t* meta, const uint32_t* chunk_off, uint32_t dtype, uint32_t tile, uint32_t lat,
              uint64_t seed, uint32_t kv, void* out, uint32_t* status, void* stream, DecFn kernel = nullptr) {
  int rc;
  if (!payload || !step || !meta || !chunk_off || !status || !out) return HQ_EINVAL;
  if (((uintptr_t)out & 15) || ((uintptr_t)payload & 15)) return HQ_EINVAL;
  DecFn fn = kernel ? kernel : dec_fn(lat, tile, kv != 0);
  const uint32_t lpt = tile / kLaneElems;
  const uint32_t tpw = (256 / lpt) < (uint32_t)kChunkTiles ? 256 / lpt : (uint32_t)kChunkTiles;
  const int block = (int)(tpw * lpt);
  const uint32_t chunk_cap = (uint32_t)(((uint64_t)kChunkTiles * P.bound + 31) / 32);
  // a unit's bits start anywhere in a word (one extra word), its first word
  // is aligned down and its last rounded up to 16 bytes (3 + 3), plus the
  // readers' guard (8); each of the two stages a multiple of 16 bytes
  const uint32_t stage_words =
      ((uint32_t)(((uint64_t)tpw * P.bound + 31) / 32) + 1 + 3 + 3 + 8 + 3) & ~3u;
  // stages, 3 table sets (offsets, flags, meta|step) + 3 x 4 words, 2
  // metadata slots (meta, step), the lanes' unary starts, the sign words
  const size_t lds = (size_t)(2 * stage_words + 3 * 3 * kChunkTiles + 12 + 2 * 2 * kChunkTiles + tpw * lpt + 8) * 4;
  int grid;
  const uint64_t units = P.C * (kChunkTiles / tpw);
  rc = grid_for((const void*)fn, block, lds, units, &grid);
  if (rc) return rc;
  // between one and two resident grids of units: two units a workgroup (the
  // second one's words stream in during the first) instead of a second round
  // of units for some workgroups (4096 x 4096 bf16 at n = 128: 2048 units,
  // 23.3 -> 22.1 us); more rounds keep the full grid (balancing them with a
  // smaller one measured slower)
  if (units > (uint64_t)grid && units <= 2 * (uint64_t)grid) grid = (int)((units + 1) / 2);
  // a grid of a given size, up to the unit count, on request (for timing
  // sweeps: units are grid-strided, so any grid decodes the same stream)
  if (const char* e = getenv("HQ_DECODE_GRID")) {
    const unsigned long long v = strtoull(e, nullptr, 10);
    if (v > 0) grid = (int)(v < units ? v : units);
  }
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  const float inv_sqrtn = (float)(1.0 / sqrt((double)tile));
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, (hipStream_t)stream, payload, payload_words, step, meta,
                     chunk_off, P.T, P.C, inv_sqrtn, derive_key(seed, 0x5349474Eu),
                     derive_key(seed, 0x44495448u), a2, out, (uint32_t)(dtype == HQ_BF16), status, stage_words,
                     chunk_cap, P.bound);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

// --------------------------------------------------------------------------
// The encode workspace of hq_encode_c_noalloc: a file-scope device array, one
// copy per GPU for the life of the process.  In host code its name stands for
// a host-side symbol, not a device address: each device's address is taken
// once with hipGetSymbolAddress (with that device current) and kept, and only
// that address is passed to kernels.
// --------------------------------------------------------------------------
constexpr uint64_t kScratchBytes = 1ull << 20;             // 768 + 8 C bytes: up to 130976 chunks
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];                              // device address, set up once per device

__global__ void clear_words(uint32_t* w, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

// the current device's scratch address; on its first use on a device the
// array is cleared by a kernel on `stream` (zero is the workspace's initial
// state), ahead of the encode on the same stream
int scratch_for_current_device(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HQ_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return HQ_EHIP;
    hipLaunchKernelGGL(clear_words, dim3(256), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ptr,
                       (uint32_t)(kScratchBytes / 4));
    if (hipGetLastError() != hipSuccess) return HQ_EHIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return HQ_OK;
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

int hq_plan_c(uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice, float c,
              uint32_t kv, uint64_t* tiles, uint64_t* chunks, uint64_t* payload_cap_words,
              uint64_t* workspace_bytes, uint32_t* tile_bound) {
  Plan P;
  int rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &P);
  if (rc) return rc;
  if (tiles) *tiles = P.T;
  if (chunks) *chunks = P.C;
  if (payload_cap_words) *payload_cap_words = P.cap_words;
  if (workspace_bytes) *workspace_bytes = P.ws_bytes;
  if (tile_bound) *tile_bound = P.bound;
  return HQ_OK;
}

int hq_encode(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
              float bps, uint64_t seed, uint32_t* payload, uint64_t payload_cap_words, uint16_t* step,
              uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* workspace,
              uint64_t workspace_bytes, void* stream) {
  Plan P;
  int rc = make_plan(dtype, rows, cols, tile, lattice, bps, 0, &P);
  if (rc) return rc;
  return do_encode(P, x, dtype, tile, lattice, seed, 0, payload, payload_cap_words, step, meta, chunk_off, status,
                   workspace, workspace_bytes, stream);
}

int hq_decode(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
              const uint32_t* chunk_off, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
              uint32_t lattice, float bps, uint64_t seed, void* x_out, uint32_t* status, void* stream) {
  Plan P;
  int rc = make_plan(dtype, rows, cols, tile, lattice, bps, 0, &P);
  if (rc) return rc;
  return do_decode(P, payload, payload_words, step, meta, chunk_off, dtype, tile, lattice, seed, 0, x_out,
                   status, stream);
}

int hq_kv_encode(const void* x, uint32_t dtype, uint64_t tokens, uint32_t head_dim, uint32_t lattice,
                 float bps, uint64_t seed, uint32_t* payload, uint64_t payload_cap_words, uint16_t* step,
                 uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* workspace,
                 uint64_t workspace_bytes, void* stream) {
  Plan P;
  int rc = make_plan(dtype, tokens, head_dim, head_dim, lattice, bps, 1, &P);
  if (rc) return rc;
  return do_encode(P, x, dtype, head_dim, lattice, seed, 1, payload, payload_cap_words, step, meta, chunk_off,
                   status, workspace, workspace_bytes, stream);
}

int hq_kv_decode(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
                 const uint32_t* chunk_off, uint32_t dtype, uint64_t tokens, uint32_t head_dim,
                 uint32_t lattice, float bps, uint64_t seed, void* x_out, uint32_t* status, void* stream) {
  Plan P;
  int rc = make_plan(dtype, tokens, head_dim, head_dim, lattice, bps, 1, &P);
  if (rc) return rc;
  return do_decode(P, payload, payload_words, step, meta, chunk_off, dtype, head_dim, lattice, seed, 1, x_out,
                   status, stream);
}

int hq_encode_c(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
                float c, uint64_t seed, uint32_t kv, uint32_t* payload, uint64_t payload_cap_words,
                uint16_t* step, uint16_t* meta, uint32_t* chunk_off, uint32_t* status, void* workspace,
                uint64_t workspace_bytes, void* stream) {
  Plan P;
  int rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &P);
  if (rc) return rc;
  if (kv && cols != tile) return HQ_EINVAL;
  return do_encode(P, x, dtype, tile, lattice, seed, kv, payload, payload_cap_words, step, meta, chunk_off,
                   status, workspace, workspace_bytes, stream);
}

int hq_encode_c_noalloc(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                        uint32_t lattice, float c, uint64_t seed, uint32_t kv, uint32_t* payload,
                        uint64_t payload_cap_words, uint16_t* step, uint16_t* meta, uint32_t* chunk_off,
                        uint32_t* status, void* stream) {
  Plan P;
  int rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &P);
  if (rc) return rc;
  if (kv && cols != tile) return HQ_EINVAL;
  if (P.ws_bytes > kScratchBytes) return HQ_ENOSPC;
  void* ws = nullptr;
  rc = scratch_for_current_device(stream, &ws);
  if (rc) return rc;
  return do_encode(P, x, dtype, tile, lattice, seed, kv, payload, payload_cap_words, step, meta, chunk_off, status,
                   ws, kScratchBytes, stream);
}

int hq_decode_c(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
                const uint32_t* chunk_off, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                uint32_t lattice, float c, uint64_t seed, uint32_t kv, void* x_out, uint32_t* status,
                void* stream) {
  Plan P;
  int rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &P);
  if (rc) return rc;
  if (kv && cols != tile) return HQ_EINVAL;
  return do_decode(P, payload, payload_words, step, meta, chunk_off, dtype, tile, lattice, seed, kv, x_out,
                   status, stream);
}

int hq_rate_bracket(uint32_t lattice, float target_bps, float* c_lo, float* c_hi) {
  // fl32(sqrt(2 pi e) V^(-1/d)), V the lattice's covolume (Z 1, A2 sqrt3/2,
  // D4 2, E8 1): the high-rate step constant of an entropy-coded lattice
  // quantiser is that times 2^-R
  uint32_t kb;
  switch (lattice) {
    case HQ_Z: kb = 0x40843F56u; break;
    case HQ_A2: kb = 0x408E1BEDu; break;
    case HQ_D4: kb = 0x405E69A9u; break;
    case HQ_E8: kb = 0x40843F56u; break;
    default: return HQ_EINVAL;
  }
  if (!(target_bps >= kRateMin && target_bps <= kRateMax) || !c_lo || !c_hi) return HQ_EINVAL;
  float k;
  memcpy(&k, &kb, 4);
  const int e = (int)floorf(target_bps);
  *c_lo = ldexpf(k, -e - 3);
  *c_hi = ldexpf(k, -e + 2);
  return HQ_OK;
}

int hq_encode_length_c(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                       uint32_t lattice, float c, uint64_t seed, uint32_t kv, unsigned long long* words,
                       void* stream) {
  Plan P;
  int rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &P);
  if (rc) return rc;
  if (kv && cols != tile) return HQ_EINVAL;
  return do_length(P, x, dtype, tile, lattice, seed, kv, words, stream);
}

int hq_encode_rate(const void* x, uint32_t dtype, uint64_t rows, uint64_t cols, uint32_t tile,
                   uint32_t lattice, float target_bps, uint64_t seed, uint32_t kv, uint32_t* payload,
                   uint64_t payload_cap_words, uint16_t* step, uint16_t* meta, uint32_t* chunk_off,
                   uint32_t* status, void* workspace, uint64_t workspace_bytes, float* c_out, double* bps_out,
                   uint32_t* encodes_out, void* stream) {
  float lo, hi;
  int rc = hq_rate_bracket(lattice, target_bps, &lo, &hi);
  if (rc) return rc;
  if (kv && cols != tile) return HQ_EINVAL;
  // the lowest constant has the longest tiles: its plan bounds every trial
  Plan P;
  rc = plan_for_c(dtype, rows, cols, tile, lattice, lo, kv, &P);
  if (rc) return rc;
  if (!x || !payload || !step || !meta || !chunk_off || !status || !workspace) return HQ_EINVAL;
  if (payload_cap_words < P.cap_words || workspace_bytes < P.ws_bytes) return HQ_ENOSPC;
  if (((uintptr_t)x & 15) || ((uintptr_t)workspace & 7)) return HQ_EINVAL;
  // each trial is a length pass counting into the workspace's length word
  // (no encoder reads it); the stream is encoded once, at the chosen constant
  unsigned long long* count = reinterpret_cast<unsigned long long*>(static_cast<uint32_t*>(workspace) + kLengthWord);
  const double numel = (double)rows * (double)cols;
  float c = lo;
  double r = 0.0;
  uint32_t it = 0;
  while (it < kRateIters) {
    c = (float)sqrt((double)lo * (double)hi);        // geometric midpoint (the product is exact)
    Plan Q;
    rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &Q);
    if (rc) return rc;
    if (hipMemsetAsync(count, 0, sizeof(*count), (hipStream_t)stream) != hipSuccess) return HQ_EHIP;
    rc = do_length(Q, x, dtype, tile, lattice, seed, kv, count, stream);
    if (rc) return rc;
    unsigned long long words = 0;
    if (hipMemcpyAsync(&words, count, sizeof(words), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
        hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
      return HQ_EHIP;
    it++;
    r = 32.0 * (double)words / numel;
    if (fabs(r - (double)target_bps) <= kRateTol || c == lo || c == hi) break;
    if (r > (double)target_bps) lo = c;              // too many bits: a larger step
    else hi = c;
  }
  Plan Q;
  rc = plan_for_c(dtype, rows, cols, tile, lattice, c, kv, &Q);
  if (rc) return rc;
  rc = do_encode(Q, x, dtype, tile, lattice, seed, kv, payload, payload_cap_words, step, meta, chunk_off, status,
                 workspace, workspace_bytes, stream);
  if (rc) return rc;
  if (c_out) *c_out = c;
  if (bps_out) *bps_out = r;
  if (encodes_out) *encodes_out = it;
  return HQ_OK;
}

int hq_rotate(const float* Q, uint32_t d, uint32_t transpose, const void* x, uint32_t x_dtype, uint64_t rows,
              void* y, uint32_t y_dtype, void* stream) {
  if ((x_dtype != HQ_F32 && x_dtype != HQ_BF16) || (y_dtype != HQ_F32 && y_dtype != HQ_BF16) || transpose > 1)
    return HQ_EINVAL;
  size_t lds = 0;
  uint32_t rb = 0, threads = 0;
  const void* fn = rot_mfma_fn(d, x_dtype == HQ_BF16, y_dtype == HQ_BF16, &lds, &threads, &rb);
  if (!fn || !Q || !x || !y || rows >= (1ull << 32)) return HQ_EINVAL;
  if (((uintptr_t)x & 15) || ((uintptr_t)y & 15) || ((uintptr_t)Q & 3)) return HQ_EINVAL;
  if (rows == 0) return HQ_OK;
  int grid;
  int rc = grid_for(fn, (int)threads, lds, (rows + rb - 1) / rb, &grid);
  if (rc) return rc;
  hipLaunchKernelGGL((void (*)(const float*, uint32_t, const void*, uint64_t, void*))fn, dim3(grid), dim3(threads),
                     lds, (hipStream_t)stream, Q, transpose, x, rows, y);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

int hq_decode_codes(const uint32_t* payload, uint64_t payload_words, const uint16_t* step, const uint16_t* meta,
                    const uint32_t* chunk_off, uint64_t rows, uint64_t cols, uint32_t tile, uint32_t lattice,
                    float c, uint64_t seed, int8_t* codes, uint32_t* status, void* stream) {
  Plan P;
  int rc = plan_for_c(HQ_F32, rows, cols, tile, lattice, c, 0, &P);
  if (rc) return rc;
  DecFn fn = lattice == HQ_E8 ? dec_codes_fn_e8(tile) : lattice == HQ_D4 ? dec_codes_fn_d4(tile)
                             : lattice == HQ_Z ? dec_codes_fn_z(tile) : nullptr;
  if (!fn) return HQ_EINVAL;
  return do_decode(P, payload, payload_words, step, meta, chunk_off, HQ_F32, tile, lattice, seed, 0, codes, status,
                   stream, fn);
}

static int act_quant(const void* x, uint32_t x_dtype, uint64_t batch, uint64_t cols, uint32_t tile,
                     uint64_t seed, int8_t* q, float* scale, void* stream, bool blocked) {
  const void* fn = act_quant_fn(tile, blocked);
  if (!fn || (x_dtype != HQ_F32 && x_dtype != HQ_BF16) || !x || !q || !scale || cols % tile ||
      (blocked ? (batch + 31) & ~31ull : batch) * cols >= (1ull << 32))
    return HQ_EINVAL;
  const uint64_t tiles = batch * (cols / tile);
  if (tiles == 0) return HQ_OK;
  hipLaunchKernelGGL((void (*)(const void*, uint32_t, uint64_t, uint32_t, float, int8_t*, float*))fn,
                     dim3((uint32_t)tiles), dim3(tile / 2), 0, (hipStream_t)stream, x, (uint32_t)(x_dtype == HQ_BF16),
                     cols / tile, derive_key(seed, 0x5349474Eu), (float)(1.0 / sqrt((double)tile)), q, scale);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

int hq_act_quant(const void* x, uint32_t x_dtype, uint64_t batch, uint64_t cols, uint32_t tile, uint64_t seed,
                 int8_t* q, float* scale, void* stream) {
  return act_quant(x, x_dtype, batch, cols, tile, seed, q, scale, stream, false);
}

int hq_act_quant_blocked(const void* x, uint32_t x_dtype, uint64_t batch, uint64_t cols, uint32_t tile,
                         uint64_t seed, int8_t* q, float* scale, void* stream) {
  return act_quant(x, x_dtype, batch, cols, tile, seed, q, scale, stream, true);
}

int hq_codes_matmul(const int8_t* codes, const uint16_t* step, uint64_t rows, uint64_t cols, uint32_t tile,
                    const int8_t* q, const float* scale, uint64_t batch, float* y, int32_t* work,
                    uint64_t work_bytes, void* stream) {
  if ((tile != 64 && tile != 128 && tile != 256) || !codes || !step || !q || !scale || !y || !work || cols % tile ||
      rows * cols >= (1ull << 32) || batch * cols >= (1ull << 32) || ((uintptr_t)codes & 15) ||
      ((uintptr_t)q & 15) || ((uintptr_t)work & 3))
    return HQ_EINVAL;
  const uint64_t tr = cols / tile;
  if (work_bytes < 4 * batch * rows * tr) return HQ_ENOSPC;
  if (rows == 0 || batch == 0) return HQ_OK;
  if ((rows + 127) / 128 > 0x7FFFFFFFull || tr > 65535 || (batch + 31) / 32 > 65535) return HQ_EINVAL;
  return launch_codes_matmul(codes, step, rows, cols, tile, q, scale, batch, y, work, (hipStream_t)stream) ? HQ_OK
                                                                                                           : HQ_EHIP;
}

int hq_nearest(uint32_t lattice, const float* t, uint64_t nblocks, float* points, void* stream) {
  NearFn fn = lattice == HQ_Z ? near_fn_z() : lattice == HQ_A2 ? near_fn_a2() : lattice == HQ_D4 ? near_fn_d4()
            : lattice == HQ_E8 ? near_fn_e8() : nullptr;
  if (!fn || !t || !points || ((uintptr_t)t & 3) || ((uintptr_t)points & 3) || nblocks >= (1ull << 40))
    return HQ_EINVAL;
  if (nblocks == 0) return HQ_OK;
  int grid;
  int rc = grid_for((const void*)fn, 256, 0, (nblocks + 255) / 256, &grid);
  if (rc) return rc;
  A2Consts a2{(float)sqrt(3.0), (float)(1.0 / sqrt(3.0))};
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), 0, (hipStream_t)stream, t, nblocks, points, a2);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
}

int hq_codes_matmul_fused(const uint32_t* payload, uint64_t payload_words, const uint16_t* step,
                          const uint16_t* meta, const uint32_t* chunk_off, uint64_t rows, uint64_t cols,
                          uint32_t tile, uint32_t lattice, float c, const int8_t* q, const float* scale,
                          uint64_t batch, float* y, uint32_t* status, void* stream) {
  Plan P;
  int rc = plan_for_c(HQ_BF16, rows, cols, tile, lattice, c, 0, &P);
  if (rc) return rc;
  if (lattice == HQ_A2 || cols % ((uint64_t)kChunkTiles * tile) != 0) return HQ_EINVAL;
  if (!payload || !step || !meta || !chunk_off || !q || !scale || !y || !status) return HQ_EINVAL;
  if (((uintptr_t)payload & 15) || ((uintptr_t)q & 15) || ((batch + 31) & ~31ull) * cols >= (1ull << 32))
    return HQ_EINVAL;
  if (batch == 0) return HQ_OK;
  // a row's run of a unit: its words, 3 before and 3 after for the 16-byte
  // vectors it is streamed in, and 8 zero guard words
  const uint32_t seg_words = ((kFusedColsHost * P.bound + 31) / 32 + 1 + 3 + 3 + 8 + 3) & ~3u;
  const uint32_t chunk_cap = (uint32_t)(((uint64_t)kChunkTiles * P.bound + 31) / 32);
  uint32_t threads = 0;
  size_t lds = 0;
  const void* fn = fused_fn(lattice, tile, seg_words, &threads, &lds);
  if (!fn) return HQ_EINVAL;
  const uint64_t gx = (rows + kFusedRowsHost - 1) / kFusedRowsHost, gy = (batch + kFusedBatchHost - 1) / kFusedBatchHost;
  if (gx > 0x7FFFFFFFull || gy > 65535) return HQ_EINVAL;
  hipLaunchKernelGGL((void (*)(const uint32_t*, uint64_t, const uint16_t*, const uint16_t*, const uint32_t*, uint64_t,
                               uint32_t, const int8_t*, const float*, uint64_t, float*, uint32_t*, uint32_t, uint32_t,
                               uint32_t))fn,
                     dim3((uint32_t)gx, (uint32_t)gy), dim3(threads), lds, (hipStream_t)stream, payload, payload_words,
                     step, meta, chunk_off, rows, (uint32_t)(cols / tile), q, scale, batch, y, status, seg_words,
                     chunk_cap, P.bound);
  return hipGetLastError() == hipSuccess ? HQ_OK : HQ_EHIP;
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
