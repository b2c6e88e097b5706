// MXFP8 quantize and dequantize kernels (gfx950) and their C-ABI entry points.
//
// Quantize: per 32-element block, amax -> E8M0 scale byte (floor(log2 amax)
// - 8, clamped) -> E4M3 codes of x / 2^scale, RNE, saturating (digest "Key
// Questions Answered": one scale per fine-grained sub-block; pytorch/ao PR
// #3203 stacked list: MXFP8 quantization kernel).  Dequantize: RNE bf16 of
// code * 2^(byte-127) (same PR list: dequantization kernel, e8m0 -> fp32).
//
// All three kernels are HBM-bound streams.  The element conversions use the
// gfx950 scaled converts (v_cvt_scalef32_pk_fp8_bf16 / _pk_bf16_fp8, two
// elements per instruction, exact RNE); the block amax is an integer max on
// packed bf16 magnitudes, reduced across the 4 lanes of a block with DPP.

#include "mx_device.h"

namespace mx {
namespace {

// ---------------------------------------------------------------------------
// Rowwise: one thread = 8 consecutive bf16 (16 B) of a row; 4 lanes = 1 block.
// Block of 256 threads = 4 output rows x 64 chunks (512 columns).
// grid.x: output rows / 4 (over batch * rows_out), grid.y: column chunks / 64.
// ---------------------------------------------------------------------------
template <bool kGather>
__global__ void __launch_bounds__(256) k_quant_rows(const uint16_t* __restrict__ x, const int32_t* __restrict__ gather,
                                                    int64_t rows_in, int64_t rows_out, int64_t total_rows, int64_t cols,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ch = (int64_t)blockIdx.y * 64 + (threadIdx.x & 63);
  const int64_t cpr = cols >> 3;
  // quads stay whole: cpr is a multiple of 4 and 64 is too
  if (row >= total_rows || ch >= cpr) return;
  int64_t src;
  if (kGather) {
    const int32_t g = gather[row];
    src = (g >= 0 && g < rows_in) ? (int64_t)g : -1;
  } else {
    const int64_t b = row / rows_out;
    const int64_t r = row - b * rows_out;
    src = r < rows_in ? b * rows_in + r : -1;
  }
  uint4 v = make_uint4(0, 0, 0, 0);
  if (src >= 0) v = *reinterpret_cast<const uint4*>(x + src * cols + ch * 8);
  v2u16 m = vmax(vmax(absbits(v.x), absbits(v.y)), vmax(absbits(v.z), absbits(v.w)));
  const uint32_t amax = quad_max(hmax(m));
  const uint32_t sb = scale_byte_from_amax(amax);
  const float sc = e8m0_to_f32(sb);
  const uint2 out = make_uint2(cvt4_e4m3(v.x, v.y, sc), cvt4_e4m3(v.z, v.w, sc));
  *reinterpret_cast<uint2*>(q + row * cols + ch * 8) = out;
  if ((ch & 3) == 0) put_scale(s, total_rows, row, ch >> 2, cols >> 5, sb);
}

// ---------------------------------------------------------------------------
// Columnwise (optionally fused with rowwise): tile of 128 output rows x 64
// columns, 256 threads.  Each thread loads 4 x 16 B (rows rr + 32i, chunk ch),
// emits the rowwise codes of its chunk, and parks the raw bf16 in LDS.  Then
// thread (column c, row block rb) walks its 32 rows down the LDS column,
// reduces the block amax and writes 32 codes contiguously into the
// transposed output.
// grid.x: row tiles, grid.y: column tiles, grid.z: batch.
// ---------------------------------------------------------------------------
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 64;
constexpr int kLdsStride = kColTileCols + 8;  // bf16 per LDS row (144 B)

template <bool kGather, bool kRow>
__global__ void __launch_bounds__(256) k_quant_cols(const uint16_t* __restrict__ x, const int32_t* __restrict__ gather,
                                                    int64_t rows_in, int64_t rows_out, int64_t cols,
                                                    uint8_t* __restrict__ row_q, uint8_t* __restrict__ row_s,
                                                    uint8_t* __restrict__ col_q, uint8_t* __restrict__ col_s) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kColTileRows * kLdsStride];
  const int t = threadIdx.x;
  const int ch = t & 7;
  const int rr = t >> 3;
  const int64_t r0 = (int64_t)blockIdx.x * kColTileRows;
  const int64_t c0 = (int64_t)blockIdx.y * kColTileCols;
  const int64_t b = blockIdx.z;
  const bool col_ok = c0 + ch * 8 < cols;  // cols % 32 == 0: a chunk is all in or all out
  const uint16_t* xb = x + b * rows_in * cols;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = rr + 32 * i;
    const int64_t r = r0 + lr;
    int64_t src = -1;
    if (r < rows_out) {
      if (kGather) {
        const int32_t g = gather[r];
        src = (g >= 0 && g < rows_in) ? (int64_t)g : -1;
      } else {
        src = r < rows_in ? r : -1;
      }
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src >= 0 && col_ok) v = *reinterpret_cast<const uint4*>(xb + src * cols + c0 + ch * 8);
    if (kRow) {
      v2u16 m = vmax(vmax(absbits(v.x), absbits(v.y)), vmax(absbits(v.z), absbits(v.w)));
      const uint32_t amax = quad_max(hmax(m));
      const uint32_t sb = scale_byte_from_amax(amax);
      const float sc = e8m0_to_f32(sb);
      if (r < rows_out && col_ok) {
        const int64_t orow = b * rows_out + r;
        *reinterpret_cast<uint2*>(row_q + orow * cols + c0 + ch * 8) =
            make_uint2(cvt4_e4m3(v.x, v.y, sc), cvt4_e4m3(v.z, v.w, sc));
        if ((ch & 3) == 0) put_scale(row_s, (int64_t)gridDim.z * rows_out, orow, (c0 + ch * 8) >> 5, cols >> 5, sb);
      }
    }
    *reinterpret_cast<uint4*>(&tile[lr * kLdsStride + ch * 8]) = v;
  }
  __syncthreads();
  const int c = t & 63;
  const int rb = t >> 6;
  const int64_t gc = c0 + c;
  const int64_t gr = r0 + 32 * rb;
  if (gc >= cols || gr >= rows_out) return;
  uint32_t w[16];
  v2u16 m = {0, 0};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t lo = tile[(32 * rb + 2 * j) * kLdsStride + c];
    const uint32_t hi = tile[(32 * rb + 2 * j + 1) * kLdsStride + c];
    w[j] = lo | (hi << 16);
    m = vmax(m, absbits(w[j]));
  }
  const uint32_t sb = scale_byte_from_amax(hmax(m));
  const float sc = e8m0_to_f32(sb);
  uint4 o0, o1;
  o0.x = cvt4_e4m3(w[0], w[1], sc);
  o0.y = cvt4_e4m3(w[2], w[3], sc);
  o0.z = cvt4_e4m3(w[4], w[5], sc);
  o0.w = cvt4_e4m3(w[6], w[7], sc);
  o1.x = cvt4_e4m3(w[8], w[9], sc);
  o1.y = cvt4_e4m3(w[10], w[11], sc);
  o1.z = cvt4_e4m3(w[12], w[13], sc);
  o1.w = cvt4_e4m3(w[14], w[15], sc);
  uint8_t* dst = col_q + (b * cols + gc) * rows_out + gr;
  *reinterpret_cast<uint4*>(dst) = o0;
  *reinterpret_cast<uint4*>(dst + 16) = o1;
  put_scale(col_s, (int64_t)gridDim.z * cols, b * cols + gc, gr >> 5, rows_out >> 5, sb);
}

// ---------------------------------------------------------------------------
// Dequantize: one thread = 16 codes (one half block); 256 threads = 4 rows x
// 64 chunks.  grid.x: rows / 4, grid.y: column chunks / 64.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                 int64_t rows, int64_t cols, uint16_t* __restrict__ y) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t ch = (int64_t)blockIdx.y * 64 + (threadIdx.x & 63);
  if (row >= rows || ch >= (cols >> 4)) return;
  const uint4 c = *reinterpret_cast<const uint4*>(q + row * cols + ch * 16);
  const uint32_t sb = s[scale_index(rows, row, ch >> 1)];
  uint4 o0, o1;
  if (sb == 255u) {  // E8M0 NaN scale: the whole block is NaN
    o0 = o1 = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  } else {
    const float sc = e8m0_to_f32(sb);
    uint2 p;
    p = cvt4_bf16(c.x, sc); o0.x = p.x; o0.y = p.y;
    p = cvt4_bf16(c.y, sc); o0.z = p.x; o0.w = p.y;
    p = cvt4_bf16(c.z, sc); o1.x = p.x; o1.y = p.y;
    p = cvt4_bf16(c.w, sc); o1.z = p.x; o1.w = p.y;
  }
  uint16_t* dst = y + row * cols + ch * 16;
  *reinterpret_cast<uint4*>(dst) = o0;
  *reinterpret_cast<uint4*>(dst + 8) = o1;
}

}  // namespace
}  // namespace mx

using namespace mx;

extern "C" int mx_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const int32_t* gather,
                           int64_t rows_out, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s,
                           mx_stream_t stream) {
  const bool want_row = row_q || row_s;
  const bool want_col = col_q || col_s;
  if (!x || batch < 1 || rows < 0 || cols <= 0 || cols % 32 || rows_out < 0) return MX_EINVAL;
  if ((row_q == nullptr) != (row_s == nullptr) || (col_q == nullptr) != (col_s == nullptr)) return MX_EINVAL;
  if (!want_row && !want_col) return MX_EINVAL;
  if (gather && batch != 1) return MX_EINVAL;
  if (want_col && rows_out % 32) return MX_EINVAL;
  if (rows_out == 0) return MX_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (want_col) {
    const dim3 grid((unsigned)((rows_out + kColTileRows - 1) / kColTileRows),
                    (unsigned)((cols + kColTileCols - 1) / kColTileCols), (unsigned)batch);
    if (grid.y > 65535u || grid.z > 65535u) return MX_EINVAL;
    if (gather) {
      if (want_row)
        hipLaunchKernelGGL((k_quant_cols<true, true>), grid, dim3(256), 0, st, x, gather, rows, rows_out, cols, row_q,
                           row_s, col_q, col_s);
      else
        hipLaunchKernelGGL((k_quant_cols<true, false>), grid, dim3(256), 0, st, x, gather, rows, rows_out, cols,
                           row_q, row_s, col_q, col_s);
    } else {
      if (want_row)
        hipLaunchKernelGGL((k_quant_cols<false, true>), grid, dim3(256), 0, st, x, gather, rows, rows_out, cols,
                           row_q, row_s, col_q, col_s);
      else
        hipLaunchKernelGGL((k_quant_cols<false, false>), grid, dim3(256), 0, st, x, gather, rows, rows_out, cols,
                           row_q, row_s, col_q, col_s);
    }
    return launch_status();
  }
  const int64_t total_rows = batch * rows_out;
  const int64_t cpr = cols / 8;
  const dim3 grid((unsigned)((total_rows + 3) / 4), (unsigned)((cpr + 63) / 64));
  if ((total_rows + 3) / 4 > 0x7FFFFFFF || grid.y > 65535u) return MX_EINVAL;
  if (gather)
    hipLaunchKernelGGL((k_quant_rows<true>), grid, dim3(256), 0, st, x, gather, rows, rows_out, total_rows, cols, row_q,
                       row_s);
  else
    hipLaunchKernelGGL((k_quant_rows<false>), grid, dim3(256), 0, st, x, gather, rows, rows_out, total_rows, cols,
                       row_q, row_s);
  return launch_status();
}

extern "C" int mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, uint16_t* y,
                             mx_stream_t stream) {
  if (!q || !s || !y || rows < 0 || cols <= 0 || cols % 32) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  const dim3 grid((unsigned)((rows + 3) / 4), (unsigned)((cols / 16 + 63) / 64));
  if ((rows + 3) / 4 > 0x7FFFFFFF || grid.y > 65535u) return MX_EINVAL;
  hipLaunchKernelGGL(k_dequant, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream), q, s, rows, cols, y);
  return launch_status();
}

extern "C" const char* mx_status_string(int status) {
  switch (status) {
    case MX_OK: return "MX_OK";
    case MX_EINVAL: return "MX_EINVAL: invalid argument";
    case MX_EUNSUPPORTED: return "MX_EUNSUPPORTED: not supported";
    case MX_EHIP: return "MX_EHIP: HIP launch error";
    default: return "unknown mx status";
  }
}
