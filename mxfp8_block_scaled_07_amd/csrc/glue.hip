// The glue of the SwiGLU expert FFN around the grouped GEMMs (gfx950):
// SwiGLU and its backward with the requantize of their results fused in, and
// the weighted unpermute-combine with its backward (the backward fused with
// the quantize of the permuted gradient).
//
// The expert computation stays in MXFP8 between the GEMMs (digest "Key
// Questions Answered"; pytorch/ao PR #3203 "Next steps": the token shuffle
// stays in MXFP8 and the grouped GEMM takes pre-quantized operands), so each
// glue step that produces a GEMM operand writes it directly as MX codes and
// scales, rowwise and columnwise, through the tile quantizer.
//
// Arithmetic is fp32 with one bf16 rounding (RNE) per result:
//   A  = silu(g) u,  silu(g) = g sigmoid(g)                 (H = [g | u])
//   dg = dA u sigmoid(g) (1 + g (1 - sigmoid(g))),  du = dA silu(g)
//   out[t] = sum_j w[t,j] Y[dst_row[t k + j]]  (fma, j ascending)
//   dY[dst_row[i]] = w[i] dOut[i / k]          (one fp32 product)
// sigmoid uses e = exp(-|g|) in (0, 1]: sigmoid(|g|) = 1 / (1 + e) and
// sigmoid(-|g|) = e / (1 + e), so neither 1 - sigmoid nor a large exponent
// is ever formed.  1 + e lies in (1, 2], so its reciprocal is the hardware
// one (V_RCP_F32, within 1 ulp; no denormal can occur) instead of a
// correctly rounded division sequence.

#include "tile_quant.h"

namespace mx {
namespace {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// silu(g) and the two sigmoids sigmoid(g), sigmoid(-g).
__device__ __forceinline__ float silu_parts(float g, float& s, float& sm) {
  const float e = expf(-fabsf(g));
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float er = e * r;
  s = g >= 0.0f ? r : er;
  sm = g >= 0.0f ? er : r;
  return g * s;
}

__device__ __forceinline__ float swiglu1(float g, float u) {
  float s, sm;
  return silu_parts(g, s, sm) * u;
}

// SwiGLU forward: output [rows, F] from H [rows, 2F].
struct SrcSwiglu {
  const uint16_t* h;
  int64_t F;
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
  __device__ Row row(const Table&, int64_t, int64_t r, int, bool in_range) const {
    Row w;
    w.ok = in_range;
    w.p = h + r * 2 * F;
    return w;
  }
  struct Raw {
    uint4 g, u;
  };
  __device__ Raw fetch(const Row& w, int64_t col, bool) const {
    Raw x;
    x.g = *reinterpret_cast<const uint4*>(w.p + col);
    x.u = *reinterpret_cast<const uint4*>(w.p + F + col);
    return x;
  }
  __device__ uint4 finish(const Raw& x, const Row&, int64_t) const {
    uint4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t g = tq_comp(x.g, k), u = tq_comp(x.u, k);
      const uint32_t v = bf16x2_rne(swiglu1(bf_lo(g), bf_lo(u)), swiglu1(bf_hi(g), bf_hi(u)));
      if (k == 0) o.x = v; else if (k == 1) o.y = v; else if (k == 2) o.z = v; else o.w = v;
    }
    return o;
  }
};

// SwiGLU backward: output dH [rows, 2F] = [dg | du] from H [rows, 2F] and
// dA [rows, F].  An 8-column chunk lies wholly in dg or in du (F % 32 == 0).
struct SrcSwigluBwd {
  const uint16_t* h;
  const uint16_t* da;
  int64_t F;
  struct Table {};
  static constexpr bool kTable = false;
  static constexpr bool kGathered = false;
  static constexpr int kSub = 1;
  static constexpr bool kFetchAll = false;
  __device__ void fill_table(Table&, int64_t, int64_t, int64_t) const {}
  struct Row {
    bool ok;
    const uint16_t* ph;
    const uint16_t* pd;
  };
  __device__ Row row(const Table&, int64_t, int64_t r, int, bool in_range) const {
    Row w;
    w.ok = in_range;
    w.ph = h + r * 2 * F;
    w.pd = da + r * F;
    return w;
  }
  struct Raw {
    uint4 g, u, d;
  };
  __device__ Raw fetch(const Row& w, int64_t col, bool) const {
    const bool gate = col < F;  // du needs no u
    const int64_t c = gate ? col : col - F;
    Raw x;
    x.g = *reinterpret_cast<const uint4*>(w.ph + c);
    x.u = gate ? *reinterpret_cast<const uint4*>(w.ph + F + c) : make_uint4(0, 0, 0, 0);
    x.d = *reinterpret_cast<const uint4*>(w.pd + c);
    return x;
  }
  __device__ static float dgate(float g, float u, float d) {
    float s, sm;
    silu_parts(g, s, sm);
    return d * u * s * (1.0f + g * sm);
  }
  __device__ static float dup(float g, float d) {
    float s, sm;
    return d * silu_parts(g, s, sm);
  }
  __device__ uint4 finish(const Raw& x, const Row&, int64_t col) const {
    const bool gate = col < F;
    uint4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t g = tq_comp(x.g, k), u = tq_comp(x.u, k), d = tq_comp(x.d, k);
      const float lo = gate ? dgate(bf_lo(g), bf_lo(u), bf_lo(d)) : dup(bf_lo(g), bf_lo(d));
      const float hi = gate ? dgate(bf_hi(g), bf_hi(u), bf_hi(d)) : dup(bf_hi(g), bf_hi(d));
      const uint32_t v = bf16x2_rne(lo, hi);
      if (k == 0) o.x = v; else if (k == 1) o.y = v; else if (k == 2) o.z = v; else o.w = v;
    }
    return o;
  }
};

// Combine backward as a gather over the permuted rows: row r takes token
// t = src_row[r] and the weight of the pair (t, j) with dst_row[t k + j] == r.
struct SrcCombineBwd {
  const uint16_t* dout;
  const float* weights;
  const int32_t* dst_row;
  const int32_t* src_row;
  int64_t tokens;
  int32_t topk;
  int64_t cols;
  bool vec;   // topk is 4 or 8, dst_row and weights 16-byte aligned: a token's slots load as vectors
  struct Table {
    int32_t tok[kTq];
    float w[kTq];
  };
  static constexpr bool kTable = true;
  static constexpr bool kGathered = true;
  static constexpr int kSub = 4;   // the pair table is built once for 4 column tiles
  __device__ void fill_table(Table& tb, int64_t, int64_t r0, int64_t rows_out) const {
    const int t = threadIdx.x;
    if (t < kTq) {
      const int64_t r = r0 + t;
      int32_t tok = -1;
      float w = 0.0f;
      if (r < rows_out) {
        const int32_t s = src_row[r];
        if (s >= 0 && s < tokens) {
          const int64_t p0 = (int64_t)s * topk;
          if (vec) {
            // the token's slots and weights are contiguous and 16-byte
            // aligned: loaded together as 16-byte vectors, in one round trip
            // instead of a chain of dependent loads
            const int4* d4 = reinterpret_cast<const int4*>(dst_row + p0);
            const float4* w4 = reinterpret_cast<const float4*>(weights + p0);
#pragma unroll
            for (int q = 1; q >= 0; --q) {   // the smallest matching slot wins
              if (q == 1 && topk == 4) continue;
              const int4 d = d4[q];
              const float4 wq = w4[q];
              if (d.w == r) { tok = s; w = wq.w; }
              if (d.z == r) { tok = s; w = wq.z; }
              if (d.y == r) { tok = s; w = wq.y; }
              if (d.x == r) { tok = s; w = wq.x; }
            }
          } else {
            for (int32_t j = 0; j < topk; ++j)
              if (dst_row[p0 + j] == r) {
                tok = s;
                w = weights[p0 + j];
                break;
              }
          }
        }
      }
      tb.tok[t] = tok;
      tb.w[t] = w;
    }
  }
  // kept for several column tiles: the token index, not a 64-bit pointer
  struct Row {
    bool ok;
    int32_t tok;
    float w;
  };
  __device__ Row row(const Table& tb, int64_t, int64_t, int lr, bool in_range) const {
    Row x;
    x.tok = tb.tok[lr];
    x.ok = in_range && x.tok >= 0;
    x.w = tb.w[lr];
    return x;
  }
  typedef uint4 Raw;
  // Called for every row, valid or not (no divergent loads in the column-tile
  // loop): invalid rows read token 0's row, a chunk past the last column
  // reads column 0, and the tile code discards both.  Without tokens, dout
  // may be null and nothing is read.
  static constexpr bool kFetchAll = true;
  __device__ Raw fetch(const Row& x, int64_t col, bool col_ok) const {
    if (tokens == 0) return make_uint4(0, 0, 0, 0);
    const int64_t t = x.ok ? x.tok : 0;
    return *reinterpret_cast<const uint4*>(dout + t * cols + (col_ok ? col : 0));
  }
  __device__ uint4 finish(const Raw& v, const Row& x, int64_t) const {
    uint4 o;
    o.x = bf16x2_rne(x.w * bf_lo(v.x), x.w * bf_hi(v.x));
    o.y = bf16x2_rne(x.w * bf_lo(v.y), x.w * bf_hi(v.y));
    o.z = bf16x2_rne(x.w * bf_lo(v.z), x.w * bf_hi(v.z));
    o.w = bf16x2_rne(x.w * bf_lo(v.w), x.w * bf_hi(v.w));
    return o;
  }
};

// ---------------------------------------------------------------------------
// Combine: one wave per (token, 512-column slab), 4 waves per workgroup;
// lane = 8 columns.  Up to 8 routed rows are loaded at once, then
// accumulated in pair order with fma.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_combine(const uint16_t* __restrict__ y, int64_t y_rows, int64_t H,
                                                 const int32_t* __restrict__ dst_row,
                                                 const float* __restrict__ weights, int64_t tokens, int32_t topk,
                                                 int32_t slabs, uint16_t* __restrict__ out) {
  const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = gw / slabs;
  const int32_t slab = (int32_t)(gw - t * slabs);
  if (t >= tokens) return;
  const int64_t col = (int64_t)slab * 512 + 8 * (threadIdx.x & 63);
  if (col >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int32_t* dr = dst_row + t * topk;
  const float* wr = weights ? weights + t * topk : nullptr;
  for (int32_t j0 = 0; j0 < topk; j0 += 8) {
    uint4 v[8];
    float wj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t j = j0 + u;
      v[u] = make_uint4(0, 0, 0, 0);
      wj[u] = 0.0f;
      if (j < topk) {
        const int32_t r = dr[j];
        if (r >= 0 && r < y_rows) {
          v[u] = *reinterpret_cast<const uint4*>(y + (int64_t)r * H + col);
          wj[u] = wr ? wr[j] : 1.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < topk) {
        acc[0] = fmaf(wj[u], bf_lo(v[u].x), acc[0]);
        acc[1] = fmaf(wj[u], bf_hi(v[u].x), acc[1]);
        acc[2] = fmaf(wj[u], bf_lo(v[u].y), acc[2]);
        acc[3] = fmaf(wj[u], bf_hi(v[u].y), acc[3]);
        acc[4] = fmaf(wj[u], bf_lo(v[u].z), acc[4]);
        acc[5] = fmaf(wj[u], bf_hi(v[u].z), acc[5]);
        acc[6] = fmaf(wj[u], bf_lo(v[u].w), acc[6]);
        acc[7] = fmaf(wj[u], bf_hi(v[u].w), acc[7]);
      }
    }
  }
  *reinterpret_cast<uint4*>(out + t * H + col) = make_uint4(bf16x2_rne(acc[0], acc[1]), bf16x2_rne(acc[2], acc[3]),
                                                            bf16x2_rne(acc[4], acc[5]), bf16x2_rne(acc[6], acc[7]));
}

inline bool misaligned(const void* p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) & (a - 1)); }

// Shared argument checks of the fused quantize outputs.
inline bool bad_quant_outputs(uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s, int64_t rows) {
  if ((row_q == nullptr) != (row_s == nullptr) || (col_q == nullptr) != (col_s == nullptr)) return true;
  if (col_q && rows % 32) return true;
  return misaligned(row_q, 8) || misaligned(row_s, 4) || misaligned(col_q, 16) || misaligned(col_s, 4);
}

}  // namespace
}  // namespace mx

using namespace mx;

extern "C" int mx_swiglu_quantize(const uint16_t* h, int64_t rows, int64_t F, uint16_t* a, uint8_t* row_q,
                                  uint8_t* row_s, uint8_t* col_q, uint8_t* col_s, mx_stream_t stream) {
  if (!h || rows < 0 || F <= 0 || F % 32) return MX_EINVAL;
  if (bad_quant_outputs(row_q, row_s, col_q, col_s, rows) || misaligned(h, 16) || misaligned(a, 16)) return MX_EINVAL;
  if (!a && !row_q && !col_q) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  TqShape sh;
  unsigned grid;
  if (!tq_shape(1, rows, F, sh, grid)) return MX_EINVAL;
  return tq_launch(SrcSwiglu{h, F}, sh, grid, TqOut{row_q, row_s, col_q, col_s, a},
                   reinterpret_cast<hipStream_t>(stream));
}

extern "C" int mx_swiglu_bwd_quantize(const uint16_t* h, const uint16_t* da, int64_t rows, int64_t F, uint16_t* dh,
                                      uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, uint8_t* col_s,
                                      mx_stream_t stream) {
  if (!h || !da || rows < 0 || F <= 0 || F % 32) return MX_EINVAL;
  if (bad_quant_outputs(row_q, row_s, col_q, col_s, rows) || misaligned(h, 16) || misaligned(da, 16) ||
      misaligned(dh, 16))
    return MX_EINVAL;
  if (!dh && !row_q && !col_q) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  TqShape sh;
  unsigned grid;
  if (!tq_shape(1, rows, 2 * F, sh, grid)) return MX_EINVAL;
  return tq_launch(SrcSwigluBwd{h, da, F}, sh, grid, TqOut{row_q, row_s, col_q, col_s, dh},
                   reinterpret_cast<hipStream_t>(stream));
}

extern "C" int mx_combine(const uint16_t* y, int64_t y_rows, int64_t H, const int32_t* dst_row,
                          const float* weights, int64_t tokens, int32_t topk, uint16_t* out, mx_stream_t stream) {
  if (!y || !dst_row || !out || y_rows < 0 || H <= 0 || H % 32 || tokens < 0 || topk < 1) return MX_EINVAL;
  if (misaligned(y, 16) || misaligned(out, 16)) return MX_EINVAL;
  if (tokens == 0) return MX_OK;
  const int64_t slabs = (H + 511) / 512;
  const int64_t blocks = (tokens * slabs + 3) / 4;
  if (blocks > 0x7FFFFFFF || slabs > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), y,
                     y_rows, H, dst_row, weights, tokens, topk, (int32_t)slabs, out);
  return launch_status();
}

extern "C" int mx_combine_bwd_quantize(const uint16_t* dout, const float* weights, const int32_t* dst_row,
                                       const int32_t* src_row, int64_t tokens, int32_t topk, int64_t rows,
                                       int64_t H, uint16_t* dy, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q,
                                       uint8_t* col_s, mx_stream_t stream) {
  if (!src_row || tokens < 0 || topk < 1 || rows < 0 || H <= 0 || H % 32) return MX_EINVAL;
  if (tokens > 0 && (!dout || !weights || !dst_row)) return MX_EINVAL;  // no tokens: every row is zero
  if (bad_quant_outputs(row_q, row_s, col_q, col_s, rows) || misaligned(dout, 16) || misaligned(dy, 16))
    return MX_EINVAL;
  if (!dy && !row_q && !col_q) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  TqShape sh;
  unsigned grid;
  if (!tq_shape(1, rows, H, sh, grid)) return MX_EINVAL;
  const bool vec = (topk == 4 || topk == 8) && !misaligned(dst_row, 16) && !misaligned(weights, 16);
  return tq_launch(SrcCombineBwd{dout, weights, dst_row, src_row, tokens, topk, H, vec}, sh, grid,
                   TqOut{row_q, row_s, col_q, col_s, dy}, reinterpret_cast<hipStream_t>(stream));
}
