// bf16 baseline layout pass (gfx950): row gather and transpose of bf16
// tensors, the bf16 counterpart of the MX quantize.
//
// The digest page (Overview, "What You'll Learn") measures MXFP8 against a
// BF16 MoE layer.  The BF16 expert step moves the same tensors as the MXFP8
// one, two bytes per element instead of one byte plus a scale byte per 32:
// tokens are gathered into expert order (the permute), and the operands the
// grouped GEMM reads along the other axis (W for dgrad, dY and X_perm for
// wgrad) are transposed so every product stays "NT".  One kernel does both:
// a 64-row x 64-column tile is read once (128-byte row segments), written
// straight out as rows, and written transposed through LDS.

#include "mx_device.h"

namespace mx {
namespace {

constexpr int kT = 64;          // tile rows and columns
constexpr int kPitch = kT + 2;  // LDS row pitch in bf16 (33 dwords: rows fall on shifted banks)

// Block (x, y, z) = (row tile of the output, column tile, batch item).
// Thread t covers 8 consecutive columns (16 B) of rows t / 8 and t / 8 + 32
// on the read side, and 8 consecutive output rows of columns t / 8 and
// t / 8 + 32 on the transposed side.
__global__ void __launch_bounds__(256) k_bf16_gather(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                     const int32_t* __restrict__ gather, int64_t rows_out,
                                                     uint16_t* __restrict__ out_rows, uint16_t* __restrict__ out_cols) {
  __shared__ uint16_t tile[kT * kPitch];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kT;
  const int64_t c0 = (int64_t)blockIdx.y * kT;
  const int64_t b = blockIdx.z;
  const uint16_t* xb = x + b * rows * cols;
  const int ch = t & 7;
  const int64_t c = c0 + 8 * ch;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rl = (t >> 3) + 32 * i;
    const int64_t r = r0 + rl;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows_out && c < cols) {
      const int64_t src = gather ? (int64_t)gather[r] : r;
      if (src >= 0 && src < rows) v = *reinterpret_cast<const uint4*>(xb + src * cols + c);
      if (out_rows) *reinterpret_cast<uint4*>(out_rows + (b * rows_out + r) * cols + c) = v;
    }
    if (out_cols) {
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + rl * kPitch + 8 * ch);
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
  }
  if (!out_cols) return;
  __syncthreads();
  const int rg = t & 7;  // output rows 8 rg .. 8 rg + 7 of the tile
  const int64_t ro = r0 + 8 * rg;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int cl = (t >> 3) + 32 * i;
    const int64_t cc = c0 + cl;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[(8 * rg + 2 * j) * kPitch + cl] | ((uint32_t)tile[(8 * rg + 2 * j + 1) * kPitch + cl] << 16);
    if (cc < cols && ro < rows_out)
      *reinterpret_cast<uint4*>(out_cols + (b * cols + cc) * rows_out + ro) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace
}  // namespace mx

using namespace mx;

extern "C" int mx_bf16_gather(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* gather,
                              int64_t rows_out, uint16_t* out_rows, uint16_t* out_cols, mx_stream_t stream) {
  if (!x || (!out_rows && !out_cols)) return MX_EINVAL;
  if (batch < 1 || rows < 0 || cols <= 0 || rows_out < 0 || cols % 32 || rows_out % 32) return MX_EINVAL;
  if (gather && batch != 1) return MX_EINVAL;
  if (!gather && rows_out < rows) return MX_EINVAL;
  if ((((uintptr_t)x | (uintptr_t)out_rows | (uintptr_t)out_cols) & 15)) return MX_EINVAL;  // 16-byte accesses
  if (rows_out == 0) return MX_OK;
  const int64_t row_tiles = (rows_out + kT - 1) / kT, col_tiles = (cols + kT - 1) / kT;
  if (row_tiles >= (1ll << 31) || col_tiles > 65535 || batch > 65535) return MX_EUNSUPPORTED;
  hipLaunchKernelGGL(k_bf16_gather, dim3((uint32_t)row_tiles, (uint32_t)col_tiles, (uint32_t)batch), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), x, rows, cols, gather, rows_out, out_rows, out_cols);
  return launch_status();
}
