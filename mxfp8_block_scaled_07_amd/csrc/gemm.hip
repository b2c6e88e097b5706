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
// contiguous along k, E8M0 scales [rows, k/32].  One kernel template serves
//   fwd / dgrad : rows of A grouped by expert (group e multiplies B_e)
//   wgrad       : the contraction axis grouped by expert (dW_e = A_e . B_e^T)
//
// Scaled MFMA operand layout (16x16x128, E4M3 x E4M3, measured on gfx950):
//   A: lane l holds row (l & 15); with g = l >> 4 its bytes 0..15 are
//      k = 16g .. 16g+15 and bytes 16..31 are k = 64+16g .. 64+16g+15.
//   B: the same with columns for rows.
//   scale: lane l supplies the E8M0 byte of (its row, 32-block g) of the
//      128-wide k step (op_sel 0 reads bits 7:0 of the scale operand).
//   D: lane l, register r holds C[4*(l >> 4) + r][l & 15].
//
// Tiling: 128 x 128 output tile per 256-thread workgroup, 2 x 2 waves of
// 64 x 64 (4 x 4 MFMA tiles each), k steps of 128 bytes, A/B tiles staged in
// LDS (double buffered, rows padded to 144 B so the 16 rows read by one
// 16-lane group hit distinct banks).

#include "mx_device.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDK = BK + 16;  // LDS bytes per staged row
constexpr int kThreads = 256;

struct Smem {
  uint8_t a[2][BM * LDK];
  uint8_t b[2][BN * LDK];
  uint32_t sa[2][BM];  // 4 scale bytes (the 4 32-blocks of the k step) per row
  uint32_t sb[2][BN];
};

// Staging registers for one k step: A and B 4 x 16 B each per thread, plus
// one scale word (threads 0..127 carry A rows, 128..255 B rows).
struct Stage {
  uint4 a[4], b[4];
  uint32_t s;
};

// Source of one operand tile: rows [row0, row0 + 128) of a [rows, ld] code
// matrix with [rows, ld/32] scales, rows valid below row_end, contraction
// valid below k_end.
struct Operand {
  const uint8_t* q;
  const uint8_t* s;
  int64_t ld;  // bytes per row (= contraction length of the whole matrix)
  int64_t row0, row_end;
};

__device__ __forceinline__ void load_stage(Stage& st, const Operand& A, const Operand& B, int64_t k0, int64_t k_end) {
  const int t = threadIdx.x;
  const int ch = t & 7;
  const int rr = t >> 3;
  const int64_t kc = k0 + 16 * ch;
  const bool kin = kc < k_end;  // k_end % 32 == 0 and 16-B chunks are aligned
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t ra = A.row0 + rr + 32 * i;
    const int64_t rb = B.row0 + rr + 32 * i;
    st.a[i] = (kin && ra < A.row_end) ? *reinterpret_cast<const uint4*>(A.q + ra * A.ld + kc) : make_uint4(0, 0, 0, 0);
    st.b[i] = (kin && rb < B.row_end) ? *reinterpret_cast<const uint4*>(B.q + rb * B.ld + kc) : make_uint4(0, 0, 0, 0);
  }
  const Operand& O = (t < 128) ? A : B;
  const int64_t r = O.row0 + (t & 127);
  uint32_t w = 0;
  if (r < O.row_end) {
    const uint8_t* sp = O.s + r * (O.ld >> 5) + (k0 >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (k0 + 32 * j < k_end) w |= (uint32_t)sp[j] << (8 * j);
  }
  st.s = w;
}

__device__ __forceinline__ void store_stage(Smem& sm, int buf, const Stage& st) {
  const int t = threadIdx.x;
  const int ch = t & 7;
  const int rr = t >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint4*>(&sm.a[buf][(rr + 32 * i) * LDK + 16 * ch]) = st.a[i];
    *reinterpret_cast<uint4*>(&sm.b[buf][(rr + 32 * i) * LDK + 16 * ch]) = st.b[i];
  }
  if (t < 128)
    sm.sa[buf][t] = st.s;
  else
    sm.sb[buf][t - 128] = st.s;
}

__device__ __forceinline__ v8i frag(const uint8_t* base, int row, int g) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + row * LDK + 16 * g);
  const uint4 hi = *reinterpret_cast<const uint4*>(base + row * LDK + 64 + 16 * g);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// acc[i][j] += A rows (wm*64 + 16i ..) x B rows (wn*64 + 16j ..) for one k step.
__device__ __forceinline__ void mma_step(const Smem& sm, int buf, v4f (&acc)[4][4], int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  v8i af[4], bf[4];
  int sa[4], sb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 64 + 16 * i + r;
    const int rb = wn * 64 + 16 * i + r;
    af[i] = frag(sm.a[buf], ra, g);
    bf[i] = frag(sm.b[buf], rb, g);
    sa[i] = (int)(sm.sa[buf][ra] >> (8 * g));
    sb[i] = (int)(sm.sb[buf][rb] >> (8 * g));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
}

// Output tile: rows [m0, m_end) x cols [n0, n_end) of a [*, ldc] matrix.
template <bool kF32>
__device__ __forceinline__ void store_tile(void* out, int64_t ldc, int64_t m0, int64_t m_end, int64_t n0, int64_t n_end,
                                           const v4f (&acc)[4][4], int wm, int wn) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + 16 * j + (lane & 15);
      if (col >= n_end) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + r;
        if (row >= m_end) continue;
        if (kF32)
          static_cast<float*>(out)[row * ldc + col] = acc[i][j][r];
        else
          static_cast<uint16_t*>(out)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
      }
    }
}

// Main loop over [k_begin, k_end) in steps of 128, double buffered.
__device__ __forceinline__ void mainloop(Smem& sm, const Operand& A, const Operand& B, int64_t k_begin, int64_t k_end,
                                         v4f (&acc)[4][4], int wm, int wn) {
  Stage st;
  if (k_begin >= k_end) return;
  load_stage(st, A, B, k_begin, k_end);
  store_stage(sm, 0, st);
  __syncthreads();
  int buf = 0;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += BK) {
    const bool more = k0 + BK < k_end;
    if (more) load_stage(st, A, B, k0 + BK, k_end);
    mma_step(sm, buf, acc, wm, wn);
    if (more) store_stage(sm, buf ^ 1, st);
    __syncthreads();
    buf ^= 1;
  }
}

// Clamp group offsets into [0, limit] and make them monotone.
__device__ __forceinline__ int64_t group_bound(const int32_t* off, int e, int64_t limit) {
  int64_t v = off[e];
  return v < 0 ? 0 : (v > limit ? limit : v);
}

// fwd / dgrad: rows grouped.  Tile index -> (group, m tile, n tile).
template <bool kF32>
__global__ void __launch_bounds__(kThreads) k_gemm_rows(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
                                                        const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
                                                        const int32_t* __restrict__ offsets, int32_t E, int64_t m_cap,
                                                        int64_t N, int64_t K, void* __restrict__ out) {
  __shared__ Smem sm;
  const int64_t n_tiles = (N + BN - 1) / BN;
  const int64_t mt = (int64_t)blockIdx.x / n_tiles;
  const int64_t nt = (int64_t)blockIdx.x - mt * n_tiles;
  // find the group owning m tile mt (uniform across the workgroup)
  int64_t lo = group_bound(offsets, 0, m_cap), acc_tiles = 0;
  int e = -1;
  int64_t row0 = 0, row_end = 0;
  for (int g = 0; g < E; ++g) {
    int64_t hi = group_bound(offsets, g + 1, m_cap);
    if (hi < lo) hi = lo;
    const int64_t tiles = (hi - lo + BM - 1) / BM;
    if (mt < acc_tiles + tiles) {
      e = g;
      row0 = lo + (mt - acc_tiles) * BM;
      row_end = hi;
      break;
    }
    acc_tiles += tiles;
    lo = hi;
  }
  if (e < 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const Operand A{a_q, a_s, K, row0, row_end};
  const Operand B{b_q + (int64_t)e * N * K, b_s + (int64_t)e * N * (K >> 5), K, nt * BN, N};
  mainloop(sm, A, B, 0, K, acc, wm, wn);
  store_tile<kF32>(out, N, row0, row_end, nt * BN, N, acc, wm, wn);
}

// wgrad: contraction grouped.  Tile index -> (group, m tile over N, n tile over K).
template <bool kF32>
__global__ void __launch_bounds__(kThreads) k_gemm_wgrad(const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_s,
                                                         const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_s,
                                                         const int32_t* __restrict__ offsets, int32_t E, int64_t m_cap,
                                                         int64_t N, int64_t K, void* __restrict__ out) {
  __shared__ Smem sm;
  const int64_t m_tiles = (N + BM - 1) / BM;
  const int64_t n_tiles = (K + BN - 1) / BN;
  const int64_t per = m_tiles * n_tiles;
  const int64_t e = (int64_t)blockIdx.x / per;
  const int64_t rem = (int64_t)blockIdx.x - e * per;
  const int64_t mt = rem / n_tiles;
  const int64_t nt = rem - mt * n_tiles;
  // group e contracts over [lo, hi) (monotone after clamping)
  int64_t lo = 0;
  for (int g = 0; g <= e; ++g) {
    const int64_t v = group_bound(offsets, g, m_cap);
    lo = v > lo ? v : lo;
  }
  int64_t hi = group_bound(offsets, (int)e + 1, m_cap);
  lo &= ~(int64_t)31;  // contraction blocks start at multiples of 32
  hi &= ~(int64_t)31;
  if (hi < lo) hi = lo;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const Operand A{a_q, a_s, m_cap, mt * BM, N};
  const Operand B{b_q, b_s, m_cap, nt * BN, K};
  mainloop(sm, A, B, lo, hi, acc, wm, wn);
  void* dst = kF32 ? (void*)(static_cast<float*>(out) + e * N * K) : (void*)(static_cast<uint16_t*>(out) + e * N * K);
  store_tile<kF32>(dst, K, mt * BM, N, nt * BN, K, acc, wm, wn);
}

}  // namespace
}  // namespace mx

using namespace mx;

static int gemm_rows(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                     const int32_t* offsets, int32_t E, int64_t m_cap, int64_t N, int64_t K, void* out,
                     int32_t out_dtype, mx_stream_t stream) {
  if (!a_q || !a_s || !b_q || !b_s || !offsets || !out) return MX_EINVAL;
  if (E < 1 || m_cap < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if (m_cap == 0) return MX_OK;
  const int64_t n_tiles = (N + BN - 1) / BN;
  const int64_t m_tiles = (m_cap + BM - 1) / BM + E;  // bound on sum_e ceil(rows_e / BM)
  const int64_t blocks = n_tiles * m_tiles;
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (out_dtype == MX_OUT_F32)
    hipLaunchKernelGGL((k_gemm_rows<true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a_q, a_s, b_q, b_s, offsets,
                       E, m_cap, N, K, out);
  else
    hipLaunchKernelGGL((k_gemm_rows<false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a_q, a_s, b_q, b_s,
                       offsets, E, m_cap, N, K, out);
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
  const int64_t blocks = (int64_t)num_groups * ((n + BM - 1) / BM) * ((k + BN - 1) / BN);
  if (blocks > 0x7FFFFFFF) return MX_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (out_dtype == MX_OUT_F32)
    hipLaunchKernelGGL((k_gemm_wgrad<true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, dyt_q, dyt_s, xt_q, xt_s,
                       group_offsets, num_groups, m_cap, n, k, dw);
  else
    hipLaunchKernelGGL((k_gemm_wgrad<false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, dyt_q, dyt_s, xt_q, xt_s,
                       group_offsets, num_groups, m_cap, n, k, dw);
  return launch_status();
}
