// MXFP8 quantize and dequantize kernels (gfx950) and their C-ABI entry points.
//
// Quantize: per 32-element block, amax -> E8M0 scale byte (floor(log2 amax)
// - 8, clamped) -> E4M3 codes of x / 2^scale, RNE, saturating (digest "Key
// Questions Answered": one scale per fine-grained sub-block; pytorch/ao PR
// #3203 stacked list: MXFP8 quantization kernel).  Dequantize: RNE bf16 of
// code * 2^(byte-127) (same PR list: dequantization kernel, e8m0 -> fp32).
//
// Quantize and dequantize are HBM-bound streams.  The quantize is the
// 128 x 128 tile quantizer of tile_quant.h (one read of x for the rowwise
// and the columnwise result); the element conversions use the gfx950 scaled
// converts (v_cvt_scalef32_pk_fp8_bf16 / _pk_bf16_fp8, two elements per
// instruction, exact RNE), the block amax is an integer max on packed bf16
// magnitudes.

#include "tile_quant.h"

namespace mx {
namespace {

// Sources of the tile quantizer: the rows of x itself (batched, zero rows
// past the end), or rows picked by a gather index.
struct SrcPlain {
  const uint16_t* x;
  int64_t rows_in, cols;
  struct Table {};
  static constexpr bool kTable = false;
  static constexpr bool kGathered = false;
  static constexpr int kSub = 1;
  static constexpr bool kFetchAll = false;
  __device__ void fill_table(Table&, int64_t, int64_t, int64_t) const {}
  struct Row {
    bool ok;
    const uint16_t* p;
  };
  __device__ Row row(const Table&, int64_t b, int64_t r, int, bool in_range) const {
    Row w;
    w.ok = in_range && r < rows_in;
    w.p = x + (b * rows_in + r) * cols;
    return w;
  }
  typedef uint4 Raw;
  __device__ Raw fetch(const Row& w, int64_t col, bool) const { return *reinterpret_cast<const uint4*>(w.p + col); }
  __device__ uint4 finish(const Raw& v, const Row&, int64_t) const { return v; }
};

struct SrcGather {
  const uint16_t* x;
  const int32_t* gather;
  int64_t rows_in, cols;
  struct Table {
    int32_t src[kTq];
  };
  static constexpr bool kTable = true;
  static constexpr bool kGathered = true;
  static constexpr int kSub = 1;
  static constexpr bool kFetchAll = false;
  __device__ void fill_table(Table& tb, int64_t, int64_t r0, int64_t rows_out) const {
    const int t = threadIdx.x;
    if (t < kTq) {
      const int64_t r = r0 + t;
      int32_t g = -1;
      if (r < rows_out) {
        g = gather[r];
        if (g < 0 || g >= rows_in) g = -1;
      }
      tb.src[t] = g;
    }
  }
  struct Row {
    bool ok;
    const uint16_t* p;
  };
  __device__ Row row(const Table& tb, int64_t, int64_t, int lr, bool in_range) const {
    const int32_t g = tb.src[lr];
    Row w;
    w.ok = in_range && g >= 0;
    w.p = x + (int64_t)g * cols;
    return w;
  }
  typedef uint4 Raw;
  __device__ Raw fetch(const Row& w, int64_t col, bool) const { return *reinterpret_cast<const uint4*>(w.p + col); }
  __device__ uint4 finish(const Raw& v, const Row&, int64_t) const { return v; }
};

// ---------------------------------------------------------------------------
// Dequantize: one thread = 16 codes (half a block), 256 threads per block over
// consecutive 16-code chunks of the row-major tensor (rows run into each
// other, so every block reads and writes one contiguous stretch).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                 int64_t rows, int64_t cols, uint16_t* __restrict__ y) {
  const int64_t cpr = cols >> 4;  // chunks per row
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= rows * cpr) return;
  const int64_t row = g / cpr;
  const int64_t ch = g - row * cpr;
  const uint4 c = *reinterpret_cast<const uint4*>(q + g * 16);
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
  uint16_t* dst = y + g * 16;
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
  if ((row_s && (reinterpret_cast<uintptr_t>(row_s) & 3)) || (col_s && (reinterpret_cast<uintptr_t>(col_s) & 3)))
    return MX_EINVAL;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (row_q && (reinterpret_cast<uintptr_t>(row_q) & 7)) ||
      (col_q && (reinterpret_cast<uintptr_t>(col_q) & 15)))
    return MX_EINVAL;
  if (rows_out == 0) return MX_OK;
  TqShape sh;
  unsigned grid;
  if (!tq_shape(batch, rows_out, cols, sh, grid)) return MX_EINVAL;
  const TqOut o = {row_q, row_s, col_q, col_s, nullptr};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (gather) return tq_launch(SrcGather{x, gather, rows, cols}, sh, grid, o, st);
  return tq_launch(SrcPlain{x, rows, cols}, sh, grid, o, st);
}

extern "C" int mx_dequantize(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t cols, uint16_t* y,
                             mx_stream_t stream) {
  if (!q || !s || !y || rows < 0 || cols <= 0 || cols % 32) return MX_EINVAL;
  // 16 codes in and 16 bf16 out per thread (16-byte accesses); scale dwords
  if ((((uintptr_t)q | (uintptr_t)y) & 15) || ((uintptr_t)s & 3)) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  const int64_t blocks = (rows * (cols / 16) + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), q, s,
                     rows, cols, y);
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
