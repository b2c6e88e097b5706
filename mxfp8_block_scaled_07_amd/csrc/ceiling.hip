// Measured ceilings of this part, for the roofline fractions the benchmark
// reports next to the published peaks (HBM 8 TB/s, dense MXFP8 MFMA
// 5.0 PFLOP/s): a streaming device copy (the HBM-bound kernels' read + write
// traffic) and a loop of scaled FP8 MFMAs on register operands (the
// grouped GEMMs' instruction at their occupancy, with no memory traffic).
// Neither is part of the MXFP8 path; they measure what it runs on.

#include "mx_device.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Block b copies the 16-byte chunks [1024 b, 1024 (b + 1)): four loads per
// thread in flight, then four stores (the dequantize's access pattern).
__global__ void __launch_bounds__(256) k_copy(const v4u* __restrict__ src, v4u* __restrict__ dst) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  v4u v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(src + base + 256 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(v[i], dst + base + 256 * i);
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
  if (!src || !dst || bytes <= 0 || bytes % 16384) return MX_EINVAL;
  if ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) return MX_EINVAL;
  const int64_t blocks = bytes / 16384;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const v4u*>(src), static_cast<v4u*>(dst));
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
