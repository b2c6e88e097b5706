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

// One 256-thread workgroup per CU (one wave per SIMD, as the grouped GEMM
// runs), 16 independent 32x32x64 accumulators per wave (the GEMM's 4 x 4
// tiles), `iters` rounds of 16 scaled MFMAs on operands held in registers.
__global__ void __launch_bounds__(256) k_mfma_loop(float* __restrict__ out, int32_t iters) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((lane + i) & 7);      // E4M3 codes near 1.0
    b[i] = 0x30303030 ^ ((lane * 3 + i) & 7);  // near 0.25
  }
  v16f acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 100);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
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

extern "C" int mx_ceiling_mfma(float* out, int32_t workgroups, int32_t iters, mx_stream_t stream) {
  if (!out || workgroups < 1 || iters < 1) return MX_EINVAL;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)workgroups), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     out, iters);
  return launch_status();
}
