// Routing metadata and the MXFP8 token permute (gfx950).
//
// pytorch/ao PR #3203, "Next steps": shuffle tokens by expert while they stay
// in MXFP8 so no dequantize is needed before the grouped GEMM.
// NVIDIA/TransformerEngine issue #556, first maintainer reply: fp8 data moves
// as plain bytes as long as the scales move with them -- the copy below moves
// each token's E4M3 codes and E8M0 scales together, untouched.
//
// Deterministic, stable ranks without ordering atomics:
//   1. k_route_hist   per routing tile (512 flat pairs; 4096 above 1024
//                     experts), an expert histogram
//   2. k_route_scan   counts, padded exclusive scan -> group_offsets, the
//                     first row of every (tile, expert), and src_row -1 for
//                     the pad rows and the rows past the last group
//   3. k_route_rank   one wave per tile walks its pairs in flat order; a pair's
//                     row is its tile base + the number of earlier pairs of the
//                     same expert (wave ballots give the in-chunk part)
//   4. k_permute_tokens copies each token's q/s row once to its topk rows,
//                     16 B per lane, and zeroes the pad rows.

#include <mutex>

#include "mx_device.h"

namespace mx {
namespace {

// Flat (token, slot) pairs per routing tile: small tiles keep many waves
// ranking at once; with many experts the per-tile tables (hist, base: tiles x
// experts) would grow, so large expert counts use larger tiles.
inline int32_t route_tile(int32_t num_experts) { return num_experts <= 1024 ? 512 : 4096; }

// The routing kernels keep one int32 per expert in LDS (64 KB at most).
constexpr int32_t kMaxExperts = 16384;

__global__ void __launch_bounds__(256) k_route_hist(const int32_t* __restrict__ ids, int64_t n, int32_t E,
                                                    int32_t tile, int32_t* __restrict__ hist) {
  extern __shared__ int32_t lh[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) lh[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * tile;
  for (int i = threadIdx.x; i < tile; i += blockDim.x) {
    const int64_t f = base + i;
    if (f < n) {
      const int32_t e = ids[f];
      if (e >= 0 && e < E) atomicAdd(&lh[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = lh[e];
}

// One block of 1024 threads = 32 experts x 32 tile groups at a time: each
// thread sums (then prefix-sums) its group's tiles for its expert.  Pass 1
// gives every expert's count; the padded exclusive scan over experts gives
// group_offsets; pass 2 writes, for every (tile, expert), the first row of
// that tile's pairs of that expert, and marks the rows no pair will take
// (each group's pad rows and the rows past the last group) with src_row -1.
// k_route_rank writes every other src_row entry: each is written once.
__global__ void __launch_bounds__(1024) k_route_scan(const int32_t* __restrict__ hist, int32_t ntiles, int32_t E,
                                                     int32_t* __restrict__ base, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ src_row, int64_t capacity) {
  extern __shared__ int32_t padded[];       // E entries
  __shared__ int32_t part[32][33];          // [expert in chunk][tile group]
  __shared__ int32_t used;                  // rows of all groups, padding included
  const int le = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int32_t per = (ntiles + 31) / 32;
  const int32_t t0 = grp * per, t1 = t0 + per < ntiles ? t0 + per : ntiles;
  for (int32_t e0 = 0; e0 < E; e0 += 32) {
    const int32_t e = e0 + le;
    int32_t c = 0;
    if (e < E)
      for (int32_t t = t0; t < t1; ++t) c += hist[(int64_t)t * E + e];
    part[le][grp] = c;
    __syncthreads();
    if (grp == 0 && e < E) {
      int32_t tot = 0;
      for (int g = 0; g < 32; ++g) tot += part[le][g];
      padded[e] = (tot + 31) & ~31;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {  // padded exclusive scan over experts
    int32_t acc = 0;
    for (int e = 0; e < E; ++e) {
      const int32_t p = padded[e];
      padded[e] = acc;
      offsets[e] = acc;
      acc += p;
    }
    offsets[E] = acc;
    used = acc;
  }
  __syncthreads();
  for (int64_t r = used + threadIdx.x; r < capacity; r += blockDim.x) src_row[r] = -1;
  for (int32_t e0 = 0; e0 < E; e0 += 32) {
    const int32_t e = e0 + le;
    int32_t c = 0;
    if (e < E)
      for (int32_t t = t0; t < t1; ++t) c += hist[(int64_t)t * E + e];
    part[le][grp] = c;
    __syncthreads();
    if (e < E) {
      int32_t acc = padded[e];
      for (int g = 0; g < grp; ++g) acc += part[le][g];
      for (int32_t t = t0; t < t1; ++t) {
        base[(int64_t)t * E + e] = acc;
        acc += hist[(int64_t)t * E + e];
      }
      if (grp == 31) {  // acc is now the group's first pad row
        const int32_t end = e + 1 < E ? padded[e + 1] : used;
        for (int32_t r = acc; r < end; ++r) src_row[r] = -1;
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// One wave (64 lanes) per tile.
__global__ void __launch_bounds__(64) k_route_rank(const int32_t* __restrict__ ids, int64_t n, int32_t topk, int32_t E,
                                                   int32_t tile, const int32_t* __restrict__ base,
                                                   int32_t* __restrict__ dst_row, int32_t* __restrict__ src_row,
                                                   int64_t capacity) {
  extern __shared__ int32_t next_row[];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) next_row[e] = base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t t0 = (int64_t)blockIdx.x * tile;
  for (int c = 0; c < tile; c += 64) {
    const int64_t f = t0 + c + lane;
    int32_t e = -1;
    if (f < n) e = ids[f];
    const bool valid = (e >= 0 && e < E);
    // lanes holding the same (valid) expert id
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? ones : ~ones;
    }
    int32_t row = -1;
    if (valid) row = next_row[e] + __popcll(peers & lt_mask);
    __syncthreads();
    if (valid) {
      // the last lane of each expert's peer group advances the cursor
      const uint64_t gt = peers & ~lt_mask & ~(1ull << lane);
      if (gt == 0) next_row[e] += __popcll(peers);
    }
    __syncthreads();
    if (f < n) {
      dst_row[f] = row;
      if (row >= 0 && row < capacity) src_row[row] = (int32_t)(f / topk);
    }
  }
}

// Token-major copy: block t < tokens reads token t's code row and scale
// dwords once and writes them to its topk rows dst_row[t*topk + j] (ids out
// of range have dst -1 and are skipped), so each source byte is read once
// however many experts the token goes to.  The block has one thread per
// 16-byte chunk of a row (rounded up to whole waves, at most 1024), so in
// rows up to 16 KB every thread moves one chunk.  Up to kDirectK
// destinations are read with uniform loads that are in flight together with
// the first code loads; larger topk stage them through LDS in chunks of
// kMaxK.  Blocks past the tokens zero the pad rows (src_row < 0): each wave
// checks kPadRows consecutive rows with one ballot and zeroes the pad rows
// among them (rows past the last group are all pad, so few rows per wave
// keep that work spread).  Every output row is written by exactly one block.
constexpr int kDirectK = 8;
constexpr int kPadRows = 4;

// Threads per block of k_permute_tokens for rows of `cols` codes.
inline int copy_threads(int64_t cols) {
  const int64_t nq = cols >> 4;
  return nq >= 1024 ? 1024 : nq <= 64 ? 64 : (int)((nq + 63) & ~int64_t(63));
}

// Its grid: one block per token, then blocks of (threads / 64) waves of
// kPadRows rows over the capacity.
inline int64_t copy_grid(int64_t tokens, int64_t capacity, int64_t cols) {
  const int64_t rows_per_block = (int64_t)(copy_threads(cols) / 64) * kPadRows;
  return tokens + (capacity + rows_per_block - 1) / rows_per_block;
}

__global__ void __launch_bounds__(1024) k_permute_tokens(const uint8_t* __restrict__ q, const uint8_t* __restrict__ s,
                                                        int64_t tokens, int64_t cols, int32_t topk,
                                                        const int32_t* __restrict__ dst_row,
                                                        const int32_t* __restrict__ src_row, int64_t capacity,
                                                        uint8_t* __restrict__ q_out, uint8_t* __restrict__ s_out) {
  constexpr int kMaxK = 64;
  __shared__ int32_t dl[kMaxK];
  const int64_t nq = cols >> 4;          // 16-B chunks of codes (cols % 32 == 0)
  const int64_t np = (cols + 127) >> 7;  // scale dwords: one per 128-column panel (panel-major)
  const uint32_t* ss = reinterpret_cast<const uint32_t*>(s);
  uint32_t* sd = reinterpret_cast<uint32_t*>(s_out);
  const int64_t blk = blockIdx.x;
  if (blk < tokens) {
    const int64_t t = blk;
    const uint4* qs = reinterpret_cast<const uint4*>(q + t * cols);
    if (topk <= kDirectK) {
      int32_t d[kDirectK];
#pragma unroll
      for (int j = 0; j < kDirectK; ++j) {
        d[j] = -1;
        if (j < topk) {
          const int32_t x = dst_row[t * topk + j];
          d[j] = x >= 0 && x < capacity ? x : -1;
        }
      }
      for (int64_t i = threadIdx.x; i < nq; i += blockDim.x) {
        const uint4 v = qs[i];
#pragma unroll
        for (int j = 0; j < kDirectK; ++j)
          if (d[j] >= 0) reinterpret_cast<uint4*>(q_out + (int64_t)d[j] * cols)[i] = v;
      }
      for (int64_t p = threadIdx.x; p < np; p += blockDim.x) {
        const uint32_t v = ss[p * tokens + t];
#pragma unroll
        for (int j = 0; j < kDirectK; ++j)
          if (d[j] >= 0) sd[p * capacity + d[j]] = v;
      }
      return;
    }
    // slots in chunks of kMaxK
    for (int32_t j0 = 0; j0 < topk; j0 += kMaxK) {
      const int32_t nk = topk - j0 < kMaxK ? topk - j0 : kMaxK;
      __syncthreads();  // the previous chunk's readers are done with dl
      for (int j = threadIdx.x; j < nk; j += blockDim.x) {
        const int32_t d = dst_row[t * topk + j0 + j];
        dl[j] = d >= 0 && d < capacity ? d : -1;
      }
      __syncthreads();
      for (int64_t i = threadIdx.x; i < nq; i += blockDim.x) {
        const uint4 v = qs[i];
        for (int j = 0; j < nk; ++j) {
          const int32_t d = dl[j];
          if (d >= 0) reinterpret_cast<uint4*>(q_out + (int64_t)d * cols)[i] = v;
        }
      }
      for (int64_t p = threadIdx.x; p < np; p += blockDim.x) {
        const uint32_t v = ss[p * tokens + t];
        for (int j = 0; j < nk; ++j) {
          const int32_t d = dl[j];
          if (d >= 0) sd[p * capacity + d] = v;
        }
      }
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((blk - tokens) * (int64_t)(blockDim.x >> 6) + (threadIdx.x >> 6)) * kPadRows;
  if (r0 >= capacity) return;
  bool pad = false;
  if (lane < kPadRows && r0 + lane < capacity) {
    const int32_t src = src_row[r0 + lane];
    pad = !(src >= 0 && src < tokens);
  }
  for (uint64_t m = __ballot(pad); m != 0; m &= m - 1) {
    const int64_t r = r0 + __builtin_ctzll(m);
    uint4* qd = reinterpret_cast<uint4*>(q_out + r * cols);
    for (int64_t i = lane; i < nq; i += 64) qd[i] = make_uint4(0, 0, 0, 0);
    for (int64_t p = lane; p < np; p += 64) sd[p * capacity + r] = 0u;
  }
}

}  // namespace
}  // namespace mx

using namespace mx;

static int64_t route_tiles(int64_t n, int32_t num_experts) {
  const int32_t t = route_tile(num_experts);
  return (n + t - 1) / t;
}

extern "C" size_t mx_permute_workspace_size(int64_t tokens, int32_t topk, int32_t num_experts) {
  if (tokens < 0 || topk < 1 || num_experts < 1) return 0;
  const int64_t nt = route_tiles(tokens * topk, num_experts);
  return (size_t)(2 * (nt > 0 ? nt : 1) * num_experts) * sizeof(int32_t);
}

// Host-side checks of a permute request: the status mx_permute returns
// before touching the GPU.  Scratch bytes are checked by the callers.
static int permute_check(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols,
                         const int32_t* expert_ids, int32_t topk, int32_t num_experts, int64_t capacity_rows,
                         const uint8_t* q_out, const uint8_t* s_out, const int32_t* group_offsets,
                         const int32_t* dst_row, const int32_t* src_row) {
  const bool copy = q || s || q_out || s_out;
  if (tokens < 0 || topk < 1 || num_experts < 1) return MX_EINVAL;
  if (num_experts > kMaxExperts) return MX_EUNSUPPORTED;
  if (!group_offsets || !src_row || (tokens > 0 && (!expert_ids || !dst_row))) return MX_EINVAL;
  if (copy && (!q || !s || !q_out || !s_out || cols <= 0 || cols % 32)) return MX_EINVAL;
  if (copy && (((uintptr_t)s | (uintptr_t)s_out) & 3)) return MX_EINVAL;  // scale dwords
  if (copy && (((uintptr_t)q | (uintptr_t)q_out) & 15)) return MX_EINVAL;  // 16-byte code copies
  const int64_t n = tokens * topk;
  if (capacity_rows < n + 31 * (int64_t)num_experts || capacity_rows > 0x7FFFFFFF) return MX_EINVAL;
  if (route_tiles(n, num_experts) > 0x7FFFFFFF) return MX_EINVAL;
  if (copy && copy_grid(tokens, capacity_rows, cols) > 0x7FFFFFFF) return MX_EINVAL;  // k_permute_tokens grid
  return MX_OK;
}

// The routing kernels and the copy on a checked request; `workspace` holds
// mx_permute_workspace_size(...) bytes (every byte is written before it is read).
static int permute_launch(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols,
                          const int32_t* expert_ids, int32_t topk, int32_t num_experts, int64_t capacity_rows,
                          uint8_t* q_out, uint8_t* s_out, int32_t* group_offsets, int32_t* dst_row, int32_t* src_row,
                          int32_t* workspace, hipStream_t st) {
  const bool copy = q || s || q_out || s_out;
  const int64_t n = tokens * topk;
  const int32_t tile = route_tile(num_experts);
  const int64_t nt = route_tiles(n, num_experts) > 0 ? route_tiles(n, num_experts) : 1;
  const int64_t copy_blocks = copy_grid(tokens, capacity_rows, cols);
  int32_t* hist = workspace;
  int32_t* base = hist + nt * num_experts;
  const size_t lds = (size_t)num_experts * sizeof(int32_t);  // <= 64 KB (kMaxExperts)
  if (n > 0) {
    hipLaunchKernelGGL(k_route_hist, dim3((unsigned)nt), dim3(256), lds, st, expert_ids, n, num_experts, tile, hist);
  } else {
    hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, st, hist, (int64_t)num_experts, 0);
  }
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), lds, st, hist, (int32_t)nt, num_experts, base,
                     group_offsets, src_row, capacity_rows);
  if (n > 0)
    hipLaunchKernelGGL(k_route_rank, dim3((unsigned)nt), dim3(64), lds, st, expert_ids, n, topk, num_experts, tile,
                       base, dst_row, src_row, capacity_rows);
  if (copy && capacity_rows > 0)
    hipLaunchKernelGGL(k_permute_tokens, dim3((unsigned)copy_blocks), dim3(copy_threads(cols)), 0, st, q, s, tokens,
                       cols, topk, dst_row, src_row, capacity_rows, q_out, s_out);
  return launch_status();
}

extern "C" int mx_permute(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols, const int32_t* expert_ids,
                          int32_t topk, int32_t num_experts, int64_t capacity_rows, uint8_t* q_out, uint8_t* s_out,
                          int32_t* group_offsets, int32_t* dst_row, int32_t* src_row, void* workspace,
                          size_t workspace_bytes, mx_stream_t stream) {
  const int rc = permute_check(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out,
                               group_offsets, dst_row, src_row);
  if (rc != MX_OK) return rc;
  if (!workspace || workspace_bytes < mx_permute_workspace_size(tokens, topk, num_experts)) return MX_EINVAL;
  return permute_launch(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out, group_offsets,
                        dst_row, src_row, static_cast<int32_t*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// mx_permute without a caller workspace: the routing tables live in a
// file-scope device array.  Each GPU holds its own copy; its device address
// is looked up once per device with hipGetSymbolAddress (the array's name in
// host code is only a host-side stand-in and is never passed to a kernel).

namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;  // MX_PERMUTE_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MX_PERMUTE_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;

__device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (set-up on the first call
// per device), or nullptr with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int mx_permute_noalloc(const uint8_t* q, const uint8_t* s, int64_t tokens, int64_t cols,
                                  const int32_t* expert_ids, int32_t topk, int32_t num_experts, int64_t capacity_rows,
                                  uint8_t* q_out, uint8_t* s_out, int32_t* group_offsets, int32_t* dst_row,
                                  int32_t* src_row, mx_stream_t stream) {
  const int rc = permute_check(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out,
                               group_offsets, dst_row, src_row);
  if (rc != MX_OK) return rc;
  if (mx_permute_workspace_size(tokens, topk, num_experts) > kScratchBytes) return MX_EUNSUPPORTED;
  hipError_t err = hipSuccess;
  void* ws = scratch_ptr(&err);
  if (!ws) return MX_EHIP;
  return permute_launch(q, s, tokens, cols, expert_ids, topk, num_experts, capacity_rows, q_out, s_out, group_offsets,
                        dst_row, src_row, static_cast<int32_t*>(ws), reinterpret_cast<hipStream_t>(stream));
}
