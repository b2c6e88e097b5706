// Block-scaled MXFP8 grouped GEMMs (gfx950): expert forward, dgrad and wgrad.
//
// digest "Key Questions Answered": the block-scaled matrix multiply applies the
// per-block scales inside the matrix instruction (the Blackwell design
// dequantizes through tensor memory; on CDNA4 the scales go straight into
// V_MFMA_SCALE_F32_16X16X128_F8F6F4, so there is no dequantize step at all).
// pytorch/ao PR #3203, "Next steps": the grouped GEMM takes pre-quantized
// MXFP8 tensors (codes + scales).
//
// Every product is "NT": C[m, n] = sum_k A[m, k] B[n, k], both operands
// contiguous along k, E8M0 scales [rows, k/32].  One kernel body serves
//   fwd / dgrad : rows of A grouped by expert (group e multiplies B_e)
//   wgrad       : the contraction axis grouped by expert (dW_e = A_e . B_e^T)
//
// Scaled MFMA operand layout (16x16x128, E4M3 x E4M3, measured on gfx950):
//   operand rows: lane l holds row (l & 15); with g = l >> 4 its bytes 0..15
//      are k = 16g .. 16g+15 and bytes 16..31 are k = 64+16g .. 64+16g+15.
//   scale: lane l supplies the E8M0 byte of (its row, 32-block g) of the
//      128-wide k step (op_sel 0 reads bits 7:0 of the scale operand).
//   D[i][j] = sum_k first[i][k] second[j][k]: lane l, register r holds
//      D[4*(l >> 4) + r][l & 15].
// The kernel passes the B tile as the first operand, so each lane ends up
// holding 4 consecutive output columns of one output row.
//
// Tiling: 256 x 256 output tile per 256-thread workgroup (one per CU), 2 x 2
// waves of 128 x 128 (8 x 8 MFMA tiles each), k steps of 128.  Tiles are
// staged in LDS by buffer loads that write LDS directly (no register round
// trip); a load past a row or contraction bound returns zeros, which pads
// ragged tiles for free.  Two LDS stages (2 x 66 KB): the loads of step s+1
// fly while step s computes.  LDS rows are 128 B with the 16-byte chunks
// XOR-swizzled by row so the 16 rows read by a lane group hit distinct banks.
// Tiles are ordered so that the tiles running at the same time on one XCD
// (blocks are dealt round-robin over the 8 XCDs) share operand rows in that
// XCD's L2.

#include "mx_device.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * BK;                          // one operand, one stage
constexpr int kStageBytes = 2 * kTileBytes + 2 * BM * 4;     // A, B, A scales, B scales
constexpr int kXcds = 8;
constexpr uint32_t kOob = 0x80000000u;                       // voffset that reads as zero

__device__ __forceinline__ int swz(int r) { return (r + (r >> 3)) & 7; }

// One operand tile: rows [0, rows) of a matrix starting at the tile's first
// row, ld bytes per row, scales ld/32 bytes per row.
struct TileSrc {
  __amdgpu_buffer_rsrc_t q, s;
  const uint8_t* sp;
  int64_t ld;
  int rows;
};

__device__ __forceinline__ TileSrc make_src(const uint8_t* q, const uint8_t* s, int64_t ld, int64_t row0, int64_t rows) {
  TileSrc t;
  const int64_t span = (int64_t)BM * ld;  // < 2^31 (checked on the host)
  t.q = __builtin_amdgcn_make_buffer_rsrc((void*)(q + row0 * ld), (short)0, (int)span, 0x00020000);
  t.s = __builtin_amdgcn_make_buffer_rsrc((void*)(s + row0 * (ld >> 5)), (short)0, (int)(span >> 5), 0x00020000);
  t.sp = s + row0 * (ld >> 5);
  t.ld = ld;
  t.rows = rows < BM ? (int)rows : BM;
  return t;
}

// Codes of one operand tile, k window [k0, k0+128) with valid k in [k_lo, k_hi).
// Wave w fills 8 LDS blocks of 1 KB (8 rows each); lane l writes slot l.
__device__ __forceinline__ void load_codes(const TileSrc& t, uint8_t* lds_tile, int64_t k0, int64_t k_lo, int64_t k_hi) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = 8 * w + i;
    const int row = 8 * blk + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    const int64_t k = k0 + 16 * c;
    const bool ok = row < t.rows && k >= k_lo && k < k_hi;
    const uint32_t voff = ok ? (uint32_t)(row * t.ld + k) : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(t.q, (lds_void*)(lds_tile + blk * 1024), 16, voff, 0, 0, 0);
  }
}

// The 4 scale bytes of the k step for each of the tile's 256 rows -> one
// dword per row.  Direct path: ld is a multiple of 128 so the dword is aligned.
__device__ __forceinline__ void load_scales_direct(const TileSrc& t, uint8_t* lds_sc, int64_t k0) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = 64 * w + lane;
  const uint32_t voff = row < t.rows ? (uint32_t)(row * (t.ld >> 5) + (k0 >> 5)) : kOob;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(t.s, (lds_void*)(lds_sc + w * 256), 4, voff, 0, 0, 0);
}

// Byte path (ld not a multiple of 128): gather the 4 bytes into a register.
__device__ __forceinline__ uint32_t load_scales_bytes(const TileSrc& t, int64_t k0) {
  const int row = threadIdx.x;
  uint32_t v = 0;
  if (row < t.rows) {
    const int64_t nb = t.ld >> 5;
    const uint8_t* p = t.sp + row * nb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = (k0 >> 5) + j;
      if (b >= 0 && b < nb) v |= (uint32_t)p[b] << (8 * j);
    }
  }
  return v;
}

__device__ __forceinline__ v8i frag(const uint8_t* tile, int row, int g) {
  const int c = g ^ swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * BK + 16 * c);
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * BK + 16 * (c ^ 4));
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// 64 MFMAs: acc[i][j] (A rows 16i.., B rows 16j.. of the wave's 128 x 128).
__device__ __forceinline__ void mma_step(const uint8_t* st, v4f (&acc)[8][8], int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const uint8_t* At = st;
  const uint8_t* Bt = st + kTileBytes;
  const uint32_t* Sa = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
  const uint32_t* Sb = Sa + BM;
  v8i bf[8];
  int sb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rb = wn * 128 + 16 * j + r;
    bf[j] = frag(Bt, rb, g);
    sb[j] = (int)(Sb[rb] >> (8 * g));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ra = wm * 128 + 16 * i + r;
    const v8i af = frag(At, ra, g);
    const int sa = (int)(Sa[ra] >> (8 * g));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0, sb[j], 0, sa);
  }
}

// Accumulate C over k in [k_lo, k_hi); k steps start at k_begin (a multiple of 128).
template <bool kScaleDirect>
__device__ __forceinline__ void mainloop(uint8_t* smem, const TileSrc& A, const TileSrc& B, int64_t k_begin,
                                         int64_t k_lo, int64_t k_hi, v4f (&acc)[8][8], int wm, int wn) {
  if (k_hi <= k_lo) return;
  const int steps = (int)((k_hi - k_begin + BK - 1) / BK);
  auto issue = [&](int stage, int64_t k0, uint32_t& sa_reg, uint32_t& sb_reg) {
    uint8_t* st = smem + stage * kStageBytes;
    load_codes(A, st, k0, k_lo, k_hi);
    load_codes(B, st + kTileBytes, k0, k_lo, k_hi);
    if (kScaleDirect) {
      load_scales_direct(A, st + 2 * kTileBytes, k0);
      load_scales_direct(B, st + 2 * kTileBytes + BM * 4, k0);
    } else {
      sa_reg = load_scales_bytes(A, k0);
      sb_reg = load_scales_bytes(B, k0);
    }
  };
  auto park = [&](int stage, uint32_t sa_reg, uint32_t sb_reg) {
    if (!kScaleDirect) {
      uint32_t* sc = reinterpret_cast<uint32_t*>(smem + stage * kStageBytes + 2 * kTileBytes);
      sc[threadIdx.x] = sa_reg;
      sc[BM + threadIdx.x] = sb_reg;
    }
  };
  uint32_t sa_reg = 0, sb_reg = 0;
  issue(0, k_begin, sa_reg, sb_reg);
  park(0, sa_reg, sb_reg);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    const bool more = s + 1 < steps;
    if (more) issue((s + 1) & 1, k_begin + (int64_t)(s + 1) * BK, sa_reg, sb_reg);
    mma_step(smem + (s & 1) * kStageBytes, acc, wm, wn);
    if (more) park((s + 1) & 1, sa_reg, sb_reg);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// Rows [m0, m0 + rows) x cols [n0, n_end) of an output with ldc elements per row.
template <bool kF32>
__device__ __forceinline__ void store_tile(void* out, int64_t ldc, int64_t m0, int rows, int64_t n0, int64_t n_end,
                                           const v4f (&acc)[8][8], int wm, int wn) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ml = wm * 128 + 16 * i + (lane & 15);
    if (ml >= rows) continue;
    const int64_t m = m0 + ml;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + wn * 128 + 16 * j + 4 * (lane >> 4);
      if (n >= n_end) continue;  // n_end % 32 == 0: the 4 columns are all in or all out
      const v4f v = acc[i][j];
      if (kF32) {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + m * ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        const uint2 p = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                   f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + m * ldc + n) = p;
      }
    }
  }
}

__device__ __forceinline__ int64_t clamp_off(const int32_t* off, int e, int64_t limit) {
  const int64_t v = off[e];
  return v < 0 ? 0 : (v > limit ? limit : v);
}

// Block -> logical tile: blocks are dealt round-robin over the XCDs, so give
// each XCD a contiguous range of logical tiles.  Returns -1 for idle blocks.
__device__ __forceinline__ int64_t logical_tile(int64_t total) {
  const int64_t per = (total + kXcds - 1) / kXcds;
  const int64_t x = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
  if (s >= per) return -1;
  const int64_t L = x * per + s;
  return L < total ? L : -1;
}

// fwd / dgrad: rows grouped.  Within a group tiles run n-tile major, m-tile
// minor, so the m tiles of a group (a few) reuse each B tile back to back.
template <bool kF32, bool kScaleDirect>
__global__ void __launch_bounds__(kThreads) k_gemm_rows(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
                                                        const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
                                                        const int32_t* __restrict__ offsets, int32_t E, int64_t m_cap,
                                                        int64_t N, int64_t K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  const int64_t n_tiles = (N + BN - 1) / BN;
  int64_t total = 0;
  {
    int64_t lo = clamp_off(offsets, 0, m_cap);
    for (int g = 0; g < E; ++g) {
      int64_t hi = clamp_off(offsets, g + 1, m_cap);
      hi = hi < lo ? lo : hi;
      total += (hi - lo + BM - 1) / BM * n_tiles;
      lo = hi;
    }
  }
  const int64_t L = logical_tile(total);
  if (L < 0) return;
  int64_t lo = clamp_off(offsets, 0, m_cap), base = 0;
  int e = 0;
  int64_t hi = lo, mt_e = 0;
  for (; e < E; ++e) {
    hi = clamp_off(offsets, e + 1, m_cap);
    hi = hi < lo ? lo : hi;
    mt_e = (hi - lo + BM - 1) / BM;
    if (L < base + mt_e * n_tiles) break;
    base += mt_e * n_tiles;
    lo = hi;
  }
  const int64_t rem = L - base;
  const int64_t nt = rem / mt_e;
  const int64_t mt = rem - nt * mt_e;
  const int64_t row0 = lo + mt * BM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const TileSrc A = make_src(a_q, a_s, K, row0, hi - row0);
  const TileSrc B = make_src(b_q + (int64_t)e * N * K, b_s + (int64_t)e * N * (K >> 5), K, nt * BN, N - nt * BN);
  mainloop<kScaleDirect>(smem, A, B, 0, 0, K, acc, wm, wn);
  store_tile<kF32>(out, N, row0, A.rows, nt * BN, N, acc, wm, wn);
}

// wgrad: contraction grouped.  Within an expert, tiles are walked in bands of
// 4 m tiles (n-tile major inside a band) so concurrent tiles share A and B.
template <bool kF32, bool kScaleDirect>
__global__ void __launch_bounds__(kThreads) k_gemm_wgrad(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
                                                         const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
                                                         const int32_t* __restrict__ offsets, int32_t E, int64_t m_cap,
                                                         int64_t N, int64_t K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];
  const int64_t m_tiles = (N + BM - 1) / BM;
  const int64_t n_tiles = (K + BN - 1) / BN;
  const int64_t per = m_tiles * n_tiles;
  const int64_t L = logical_tile((int64_t)E * per);
  if (L < 0) return;
  const int64_t e = L / per;
  const int64_t rem = L - e * per;
  constexpr int64_t kBand = 4;
  const int64_t band = rem / (kBand * n_tiles);
  const int64_t first_m = band * kBand;
  const int64_t band_m = (m_tiles - first_m) < kBand ? (m_tiles - first_m) : kBand;
  const int64_t in_band = rem - band * kBand * n_tiles;
  const int64_t mt = first_m + in_band % band_m;
  const int64_t nt = in_band / band_m;
  // group e contracts over [lo, hi): clamped, monotone, whole 32-blocks
  int64_t lo = 0;
  for (int g = 0; g <= e; ++g) {
    const int64_t v = clamp_off(offsets, g, m_cap);
    lo = v > lo ? v : lo;
  }
  int64_t hi = clamp_off(offsets, (int)e + 1, m_cap);
  lo &= ~(int64_t)31;
  hi &= ~(int64_t)31;
  hi = hi < lo ? lo : hi;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const TileSrc A = make_src(a_q, a_s, m_cap, mt * BM, N - mt * BM);
  const TileSrc B = make_src(b_q, b_s, m_cap, nt * BN, K - nt * BN);
  mainloop<kScaleDirect>(smem, A, B, lo & ~(int64_t)(BK - 1), lo, hi, acc, wm, wn);
  void* dst = kF32 ? (void*)(static_cast<float*>(out) + e * N * K) : (void*)(static_cast<uint16_t*>(out) + e * N * K);
  store_tile<kF32>(dst, K, mt * BM, A.rows, nt * BN, K, acc, wm, wn);
}

template <bool kF32, bool kDirect>
void launch_rows(dim3 grid, hipStream_t st, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                 const uint8_t* b_s, const int32_t* off, int32_t E, int64_t m_cap, int64_t N, int64_t K, void* out) {
  hipLaunchKernelGGL((k_gemm_rows<kF32, kDirect>), grid, dim3(kThreads), 0, st, a_q, a_s, b_q, b_s, off, E, m_cap, N,
                     K, out);
}

template <bool kF32, bool kDirect>
void launch_wgrad(dim3 grid, hipStream_t st, const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q,
                  const uint8_t* b_s, const int32_t* off, int32_t E, int64_t m_cap, int64_t N, int64_t K, void* out) {
  hipLaunchKernelGGL((k_gemm_wgrad<kF32, kDirect>), grid, dim3(kThreads), 0, st, a_q, a_s, b_q, b_s, off, E, m_cap,
                     N, K, out);
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace
}  // namespace mx

using namespace mx;

static int gemm_rows(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                     const int32_t* offsets, int32_t E, int64_t m_cap, int64_t N, int64_t K, void* out,
                     int32_t out_dtype, mx_stream_t stream) {
  if (!a_q || !a_s || !b_q || !b_s || !offsets || !out) return MX_EINVAL;
  if (E < 1 || m_cap < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * K >= (1ll << 31)) return MX_EINVAL;  // buffer-resource span of one tile
  if (m_cap == 0) return MX_OK;
  const int64_t n_tiles = (N + BN - 1) / BN;
  const int64_t blocks = round_up(((m_cap + BM - 1) / BM + E) * n_tiles, kXcds);
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks);
  const bool direct = K % 128 == 0;
  if (out_dtype == MX_OUT_F32) {
    if (direct) launch_rows<true, true>(grid, st, a_q, a_s, b_q, b_s, offsets, E, m_cap, N, K, out);
    else launch_rows<true, false>(grid, st, a_q, a_s, b_q, b_s, offsets, E, m_cap, N, K, out);
  } else {
    if (direct) launch_rows<false, true>(grid, st, a_q, a_s, b_q, b_s, offsets, E, m_cap, N, K, out);
    else launch_rows<false, false>(grid, st, a_q, a_s, b_q, b_s, offsets, E, m_cap, N, K, out);
  }
  return launch_status();
}

extern "C" int mx_grouped_gemm_fwd(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                                   const int32_t* group_offsets, int32_t num_groups, int64_t m_cap, int64_t n,
                                   int64_t k, void* out, int32_t out_dtype, mx_stream_t stream) {
  return gemm_rows(a_q, a_s, b_q, b_s, group_offsets, num_groups, m_cap, n, k, out, out_dtype, stream);
}

extern "C" int mx_grouped_gemm_dgrad(const uint8_t* dy_q, const uint8_t* dy_s, const uint8_t* wt_q,
                                     const uint8_t* wt_s, const int32_t* group_offsets, int32_t num_groups,
                                     int64_t m_cap, int64_t n_out, int64_t k_contract, void* dx, int32_t out_dtype,
                                     mx_stream_t stream) {
  return gemm_rows(dy_q, dy_s, wt_q, wt_s, group_offsets, num_groups, m_cap, n_out, k_contract, dx, out_dtype,
                   stream);
}

extern "C" int mx_grouped_gemm_wgrad(const uint8_t* dyt_q, const uint8_t* dyt_s, const uint8_t* xt_q,
                                     const uint8_t* xt_s, const int32_t* group_offsets, int32_t num_groups,
                                     int64_t m_cap, int64_t n, int64_t k, void* dw, int32_t out_dtype,
                                     mx_stream_t stream) {
  if (!dyt_q || !dyt_s || !xt_q || !xt_s || !group_offsets || !dw) return MX_EINVAL;
  if (num_groups < 1 || m_cap < 0 || m_cap % 32 || n <= 0 || k <= 0 || n % 32 || k % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * m_cap >= (1ll << 31)) return MX_EINVAL;  // buffer-resource span of one tile
  const int64_t blocks = round_up((int64_t)num_groups * ((n + BM - 1) / BM) * ((k + BN - 1) / BN), kXcds);
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks);
  const bool direct = m_cap % 128 == 0;
  if (out_dtype == MX_OUT_F32) {
    if (direct) launch_wgrad<true, true>(grid, st, dyt_q, dyt_s, xt_q, xt_s, group_offsets, num_groups, m_cap, n, k, dw);
    else launch_wgrad<true, false>(grid, st, dyt_q, dyt_s, xt_q, xt_s, group_offsets, num_groups, m_cap, n, k, dw);
  } else {
    if (direct) launch_wgrad<false, true>(grid, st, dyt_q, dyt_s, xt_q, xt_s, group_offsets, num_groups, m_cap, n, k, dw);
    else launch_wgrad<false, false>(grid, st, dyt_q, dyt_s, xt_q, xt_s, group_offsets, num_groups, m_cap, n, k, dw);
  }
  return launch_status();
}
