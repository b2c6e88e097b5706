// Measured ceilings of this part, for the roofline fractions the benchmark
// reports next to the published peaks (HBM 8 TB/s, dense MXFP8 MFMA
// 5.0 PFLOP/s): a streaming device copy (the HBM-bound kernels' read + write
// traffic), the tile quantizer's access pattern with no arithmetic (what a
// quantizer that writes both orientations can reach), and a loop of scaled
// FP8 MFMAs on register operands (the grouped GEMMs' instruction at their
// occupancy, with no memory traffic).  None is part of the MXFP8 path; they
// measure what it runs on.

#include "mx_device.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Thread t of block b copies the 16-byte chunk 256 b + t with non-temporal
// loads and stores.  Of the patterns timed on this part (1, 2, 4 or 8
// chunks per thread, default or non-temporal policy on either side, 256- or
// 1024-thread blocks), one chunk per thread in 256-thread blocks with both
// sides non-temporal is the fastest.
__global__ void __launch_bounds__(256) k_copy(const v4u* __restrict__ src, v4u* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// The tile quantizer's memory traffic without its arithmetic: block
// (tr, tc), column tiles of a row band consecutive, reads the 128 x 128 bf16
// tile at rows 128 tr, columns 128 tc of x [rows, cols] with the
// quantizer's thread map (wave w, lane 16 ry + ch: rows 32 w + 8 ry ... +7,
// 16 bytes at column 8 ch each), writes 8 bytes per tile row and thread to
// row_out [rows, cols] (the rowwise codes' runs of 128 bytes per row) and
// the tile's columns as 128-byte runs to col_out [cols, rows] (8 lanes per
// column, the columnwise codes' lines).  The values written are XORs of the
// loaded ones, so every load is used.  Loads are non-temporal: of the
// policies timed on this pattern that is the faster one (the quantizer
// itself measured faster with default loads).
__global__ void __launch_bounds__(256) k_tile_pattern(const uint8_t* __restrict__ x, uint8_t* __restrict__ row_out,
                                                       uint8_t* __restrict__ col_out, int64_t rows, int64_t cols,
                                                       int32_t n_tc) {
  const int32_t tc = (int32_t)(blockIdx.x % (uint32_t)n_tc), tr = (int32_t)(blockIdx.x / (uint32_t)n_tc);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, ch = lane & 15, ry = lane >> 4;
  const int64_t r0 = (int64_t)tr * 128 + 32 * w + 8 * ry, c0 = (int64_t)tc * 128;
  v4u v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x + ((r0 + i) * cols + c0 + 8 * ch) * 2));
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint2*>(row_out + (r0 + i) * cols + c0 + 8 * ch) =
        make_uint2(v[i].x ^ v[i].y, v[i].z ^ v[i].w);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int q = 256 * s + t;   // column q / 8 of the tile, 16-byte piece q % 8 of its 128-row run
    *reinterpret_cast<v4u*>(col_out + (c0 + (q >> 3)) * rows + (int64_t)tr * 128 + 16 * (q & 7)) =
        v[2 * s] ^ v[2 * s + 1];
  }
}

// A random E4M3 code in every byte (no NaN code), random signs.
__device__ __forceinline__ int random_codes(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    uint32_t c = (x >> (8 * b)) & 0xFF;
    if ((c & 0x7F) >= 0x7E) c &= 0xF7;
    out |= c << (8 * b);
  }
  return (int)out;
}

// One 256-thread workgroup per CU (one wave per SIMD, as the grouped GEMM
// runs), the GEMM step's register pattern: 4 A and 4 B fragments and their
// scale bytes, 4 x 4 accumulators of 32 x 32, `iters` rounds of 16 scaled
// MFMAs with no memory traffic.  With kRandom the fragments hold random
// codes and scales (the power the GEMMs draw on real data, which sets the
// clock the part holds); otherwise near-constant codes.
template <bool kRandom>
__global__ void __launch_bounds__(256) k_mfma_loop(float* __restrict__ out, int32_t iters) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 977u;
  v8i a[4], b[4];
  int sa[4], sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[i][q] = kRandom ? random_codes(seed + 16 * i + q) : 0x38383838 ^ ((lane + q) & 7);
      b[i][q] = kRandom ? random_codes(seed + 16 * i + q + 1000003u) : 0x30303030 ^ ((lane * 3 + q) & 7);
    }
    sa[i] = kRandom ? 118 + (int)(seed * (i + 3) >> 28) : 127;
    sb[i] = kRandom ? 118 + (int)(seed * (i + 7) >> 28) : 100;
  }
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, sb[j], 0, sa[i]);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[i][j][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace mx

using namespace mx;

extern "C" int mx_ceiling_copy(const void* src, void* dst, int64_t bytes, mx_stream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 4096) return MX_EINVAL;
  if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) return MX_EINVAL;
  const int64_t blocks = bytes / 4096;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const v4u*>(src), static_cast<v4u*>(dst));
  return launch_status();
}

extern "C" int mx_ceiling_tile_pattern(const void* x, void* row_out, void* col_out, int64_t rows, int64_t cols,
                                       mx_stream_t stream) {
  if (!x || !row_out || !col_out || rows <= 0 || cols <= 0 || rows % 128 || cols % 128) return MX_EINVAL;
  if ((((uintptr_t)x) | ((uintptr_t)row_out) | ((uintptr_t)col_out)) & 15) return MX_EINVAL;
  const int64_t n_tc = cols / 128, blocks = (rows / 128) * n_tc;
  if (n_tc > 0x7FFFFFFF || blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_tile_pattern, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(x), static_cast<uint8_t*>(row_out), static_cast<uint8_t*>(col_out),
                     rows, cols, (int32_t)n_tc);
  return launch_status();
}

extern "C" int mx_ceiling_mfma(float* out, int32_t workgroups, int32_t iters, int32_t random_operands,
                               mx_stream_t stream) {
  if (!out || workgroups < 1 || iters < 1) return MX_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (random_operands)
    hipLaunchKernelGGL(k_mfma_loop<true>, dim3((unsigned)workgroups), dim3(256), 0, st, out, iters);
  else
    hipLaunchKernelGGL(k_mfma_loop<false>, dim3((unsigned)workgroups), dim3(256), 0, st, out, iters);
  return launch_status();
}
