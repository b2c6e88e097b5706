// The router in front of the MXFP8 token shuffle (gfx950): top-k expert choice
// with softmax weights, and its backward through the weighted combine.
//
// The pages run the MoE layer in MXFP8 (digest "Overview") without a router
// formula; the reading used throughout: a token's experts are its k largest
// logits (equal logits to the lower expert id), weighted by the softmax of
// the k chosen logits.  With out[t] = sum_j w[t,j] Y[dst_row[t k + j]], the
// backward is dw[t,j] = <dOut[t], Y[dst_row[t k + j]]> and, through the
// softmax, dlogit[t, e_j] = w_j (dw_j - sum_i w_i dw_i), zero elsewhere.
//
// Both kernels give one wave to a token.  Top-k runs k rounds of a wave-wide
// argmax (butterfly over the 64 lanes, key = (logit, -expert)); each lane
// keeps its E/64 logits in registers.  The backward streams dOut[t] and the
// k routed rows of Y, 8 bf16 per lane per load, with fp32 fused multiply-adds,
// then reduces the k partial sums across the wave.

#include "mx_device.h"

namespace mx {
namespace {

constexpr int kMaxPerLane = 16;   // experts per lane: E <= 1024
constexpr int kMaxTopk = 64;

// Wave-wide argmax of (v, -e): every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float ov = __shfl_xor(v, d, 64);
    const int oe = __shfl_xor(e, d, 64);
    if (ov > v || (ov == v && oe < e)) {
      v = ov;
      e = oe;
    }
  }
}

__global__ void __launch_bounds__(256) k_route_topk(const float* __restrict__ logits, int64_t tokens, int32_t E,
                                                    int32_t topk, int32_t* __restrict__ ids,
                                                    float* __restrict__ weights) {
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= tokens) return;
  const int lane = threadIdx.x & 63;
  const float* row = logits + t * E;
  float v[kMaxPerLane];
  uint32_t used = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
    if (e >= E) used |= 1u << i;
  }
  float z0 = 0.0f, sum = 0.0f, my_z = 0.0f;
  int my_e = -1;
  for (int j = 0; j < topk; ++j) {
    // the lane's best unused expert: largest logit, lowest index on ties
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (!(used >> i & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
    wave_argmax(bv, be);
    if ((be & 63) == lane) used |= 1u << (be >> 6);
    if (j == 0) z0 = bv;
    const float p = expf(bv - z0);
    sum += p;
    if (lane == j) {
      my_e = be;
      my_z = bv;
    }
  }
  if (lane < topk) {
    ids[t * topk + lane] = my_e;
    weights[t * topk + lane] = expf(my_z - z0) / sum;
  }
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
  acc = fmaf(bf_lo(a.x), bf_lo(b.x), acc);
  acc = fmaf(bf_hi(a.x), bf_hi(b.x), acc);
  acc = fmaf(bf_lo(a.y), bf_lo(b.y), acc);
  acc = fmaf(bf_hi(a.y), bf_hi(b.y), acc);
  acc = fmaf(bf_lo(a.z), bf_lo(b.z), acc);
  acc = fmaf(bf_hi(a.z), bf_hi(b.z), acc);
  acc = fmaf(bf_lo(a.w), bf_lo(b.w), acc);
  acc = fmaf(bf_hi(a.w), bf_hi(b.w), acc);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// One wave per token; routed rows in groups of 8 (their loads in flight
// together), H in slabs of 512 columns.
__global__ void __launch_bounds__(256) k_router_bwd(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y,
                                                    int64_t y_rows, int64_t H, const int32_t* __restrict__ dst_row,
                                                    const int32_t* __restrict__ ids, const float* __restrict__ weights,
                                                    int64_t tokens, int32_t E, int32_t topk, float* __restrict__ dw,
                                                    float* __restrict__ dlogits) {
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= tokens) return;
  const int lane = threadIdx.x & 63;
  float my_dw = 0.0f;   // lane j < topk keeps dw[t, j]
  for (int32_t j0 = 0; j0 < topk; j0 += 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int64_t r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t j = j0 + u;
      r[u] = -1;
      if (j < topk) {
        const int32_t d = dst_row[t * topk + j];
        if (d >= 0 && d < y_rows) r[u] = d;
      }
    }
    for (int64_t col = 8 * lane; col < H; col += 512) {
      const uint4 g = *reinterpret_cast<const uint4*>(dout + t * H + col);
      uint4 yv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        yv[u] = r[u] >= 0 ? *reinterpret_cast<const uint4*>(y + r[u] * H + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = dot8(g, yv[u], acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float s = wave_sum(acc[u]);
      if (lane == j0 + u) my_dw = s;
    }
  }
  const bool mine = lane < topk;
  const float w = mine ? weights[t * topk + lane] : 0.0f;
  if (dw && mine) dw[t * topk + lane] = my_dw;
  if (dlogits) {
    // lane j holds the gradient of its chosen logit; every lane then writes
    // the full entries of its experts (a repeated expert sums its terms)
    const float inner = wave_sum(w * my_dw);
    const float gsel = mine ? w * (my_dw - inner) : 0.0f;
    const int32_t esel = mine ? ids[t * topk + lane] : -1;
    for (int e = lane; e < E; e += 64) {
      float val = 0.0f;
      for (int32_t j = 0; j < topk; ++j) {
        const int32_t ej = __shfl(esel, j, 64);
        const float gj = __shfl(gsel, j, 64);
        if (ej == e) val += gj;
      }
      dlogits[t * E + e] = val;
    }
  }
}

inline bool misaligned(const void* p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) & (a - 1)); }

}  // namespace
}  // namespace mx

using namespace mx;

extern "C" int mx_route_topk(const float* logits, int64_t tokens, int32_t num_experts, int32_t topk,
                             int32_t* expert_ids, float* weights, mx_stream_t stream) {
  if (!logits || !expert_ids || !weights || tokens < 0) return MX_EINVAL;
  if (num_experts < 1 || topk < 1 || topk > num_experts) return MX_EINVAL;
  if (num_experts > 64 * kMaxPerLane || topk > kMaxTopk) return MX_EUNSUPPORTED;
  if (tokens == 0) return MX_OK;
  const int64_t blocks = (tokens + 3) / 4;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_route_topk, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     logits, tokens, num_experts, topk, expert_ids, weights);
  return launch_status();
}

extern "C" int mx_router_bwd(const uint16_t* dout, const uint16_t* y, int64_t y_rows, int64_t H,
                             const int32_t* dst_row, const int32_t* expert_ids, const float* weights, int64_t tokens,
                             int32_t num_experts, int32_t topk, float* dw, float* dlogits, mx_stream_t stream) {
  if (!dout || !y || !dst_row || !weights || tokens < 0 || y_rows < 0 || H <= 0 || H % 32) return MX_EINVAL;
  if (num_experts < 1 || topk < 1 || topk > 64) return MX_EINVAL;
  if (!dw && !dlogits) return MX_EINVAL;
  if (dlogits && !expert_ids) return MX_EINVAL;
  if (misaligned(dout, 16) || misaligned(y, 16)) return MX_EINVAL;
  if (tokens == 0) return MX_OK;
  const int64_t blocks = (tokens + 3) / 4;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipLaunchKernelGGL(k_router_bwd, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), dout,
                     y, y_rows, H, dst_row, expert_ids, weights, tokens, num_experts, topk, dw, dlogits);
  return launch_status();
}
