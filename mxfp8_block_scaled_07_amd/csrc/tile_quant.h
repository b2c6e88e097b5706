// The 128 x 128 tile quantizer behind every MXFP8 quantize of the library:
// the plain quantize, the quantize of gathered (permuted) rows, and the
// quantizes fused into the SwiGLU and combine glue.  A tile of bf16 values
// is produced by a source (a load, a gather, or an element-wise function of
// other tensors), and written as any of: its rowwise MX codes and scales, its
// columnwise MX codes and scales (transposed), and the bf16 values
// themselves.
//
// MX rule (digest "Key Questions Answered": one scale per fine-grained
// sub-block; pytorch/ao PR #3203 stacked list: MXFP8 quantization kernel):
// per 32-element block, scale byte = floor(log2 amax) - 8 clamped to the
// E8M0 range, codes = E4M3 of x / 2^scale, RNE, saturating.
//
// Work split (256 threads = 4 waves).  Thread (wave w, lane = 16 ry + ch)
// owns the 8 consecutive tile rows 32w + 8ry .. +7 at the 8 columns
// 8ch .. 8ch+7: eight 16-byte loads, each wave instruction covering four
// full 256-byte tile rows.
// * Rowwise: the 4 lanes of a quad hold one 32-column block of a row; the
//   amax is reduced with DPP quad permutes.  The 4 scale bytes of a row (one
//   128-column panel) are merged into one dword with DPP row shifts and
//   stored by one lane, so panel dwords are whole.
// * Columnwise: the thread transposes its 8 x 8 block in registers and
//   writes 8 columns x 16 bytes into an LDS tile kept column-major (a column
//   = 128 rows = 256 bytes = 16 slots of 16 bytes; slot s of column c sits
//   at slot s ^ ((c ^ (c >> 3)) & 15), which keeps both the write and the
//   read pattern spread over all banks).  Then 8 lanes take a column, 16
//   rows each: a lane pair shares a 32-row block (amax exchanged with a DPP
//   quad permute), and the 8 lanes store the column's 128 code bytes as one
//   whole line, so a wave's store writes 8 whole lines (lanes holding 64
//   bytes of two 32-row blocks each wrote 16-byte pieces of 32 lines per
//   store, 4-15% slower).  The column's 4 scale bytes are merged into one
//   panel dword with DPP row shifts.
#pragma once

#include "mx_device.h"

namespace mx {

constexpr int kTq = 128;
constexpr int kTqThreads = 256;

struct TqShape {
  int64_t rows_out;  // output rows per batch item
  int64_t cols;      // output columns
  int32_t n_tr;      // row tiles per batch item
  int32_t n_tc;      // column tiles
  int32_t batch;
};

struct TqOut {
  uint8_t* row_q;  // rowwise codes [batch * rows_out, cols] (or null)
  uint8_t* row_s;  // rowwise scales, panel layout over batch * rows_out rows
  uint8_t* col_q;  // columnwise codes [batch, cols, rows_out] (or null)
  uint8_t* col_s;  // columnwise scales, panel layout over batch * cols rows
  uint16_t* y;     // bf16 values [batch * rows_out, cols] (or null)
};

__device__ __forceinline__ uint32_t tq_comp(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ int tq_swz(int c) { return (c ^ (c >> 3)) & 15; }

__device__ __forceinline__ uint32_t dpp_row_shr(uint32_t v, int n4or8) {
  return n4or8 == 4 ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true)
                    : (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t amax8(const uint4& v) {
  const v2u16 m = vmax(vmax(absbits(v.x), absbits(v.y)), vmax(absbits(v.z), absbits(v.w)));
  return hmax(m);
}

// Source concept:
//   struct Table;                          LDS table filled once per tile (may be empty)
//   static constexpr bool kTable;          whether fill_table must run
//   static constexpr bool kGathered;       rows gathered from a source that other rows read again
//   __device__ void fill_table(Table&, int64_t b, int64_t r0, int64_t rows_out) const;
//   struct Row { bool ok; ... };
//   __device__ Row row(const Table&, int64_t b, int64_t r, int local_r, bool in_range) const;
//   struct Raw;
//   __device__ Raw fetch(const Row&, int64_t col, bool col_ok) const;  only for row.ok && col_ok
//     unless kFetchAll (then for every row, and it must stay in bounds)
//   static constexpr int kSub;             column tiles per workgroup
//   static constexpr bool kFetchAll;
//   __device__ uint4 finish(const Raw&, const Row&, int64_t col) const;   8 bf16
// Rows or columns outside the output, and rows the source marks !ok, are
// zero: they raise no amax and produce zero codes (and zero pad scales).
//
// Tile order: consecutive blocks walk the column tiles of a row band (rows
// stream through in order); for gathered sources, where each source row is
// read again by other output rows (a token's k routed copies), they walk the
// row bands of a column tile, so the re-reads of a source row's 256-byte
// slice fall within the window of one column tile (all tokens x 256 B, a few
// MB) and hit in the caches instead of HBM.
template <class Src, bool kRow, bool kCol, bool kY>
__global__ void __launch_bounds__(kTqThreads) k_tile_quant(const Src src, const TqShape sh, const TqOut o) {
  // The source's row table is only read before the first column phase writes
  // the LDS tile: it shares the tile's first bytes, so a gathered tile needs
  // no more LDS than a plain one (5 workgroups per CU).
  typedef typename Src::Table Table;
  constexpr int kTile = kCol ? kTq * kTq * 2 : 16;
  constexpr int kLds = kTile > (int)sizeof(Table) ? kTile : (int)sizeof(Table);
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  Table& table = *reinterpret_cast<Table*>(lds);
  // A workgroup takes kSub consecutive column tiles of one row band: the
  // source's row table and the threads' row descriptors are built once.
  constexpr int kSub = Src::kSub;
  const uint32_t n_tcg = ((uint32_t)sh.n_tc + kSub - 1) / kSub;
  uint32_t idx = blockIdx.x;
  int32_t tcg, tr;
  if (Src::kGathered) {
    tr = (int32_t)(idx % (uint32_t)sh.n_tr);
    idx /= (uint32_t)sh.n_tr;
    tcg = (int32_t)(idx % n_tcg);
    idx /= n_tcg;
  } else {
    tcg = (int32_t)(idx % n_tcg);
    idx /= n_tcg;
    tr = (int32_t)(idx % (uint32_t)sh.n_tr);
    idx /= (uint32_t)sh.n_tr;
  }
  const int32_t b = (int32_t)idx;
  const int64_t r0 = (int64_t)tr * kTq;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int ch = lane & 15, ry = lane >> 4;
  const int lr0 = 32 * w + 8 * ry;
  if (Src::kTable) {
    src.fill_table(table, b, r0, sh.rows_out);
    __syncthreads();
  }
  typename Src::Row rw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + lr0 + i;
    rw[i] = src.row(table, b, r, lr0 + i, r < sh.rows_out);
  }

#pragma unroll 1
  for (int sub = 0; sub < kSub; ++sub) {
    const int32_t tc = tcg * kSub + sub;
    if (tc >= sh.n_tc) break;   // uniform over the workgroup
    const int64_t c0 = (int64_t)tc * kTq;
    const int64_t col = c0 + 8 * ch;
    const bool col_ok = col < sh.cols;  // cols % 32 == 0: a chunk is all in or all out

    uint4 v[8];
    {
      typename Src::Raw raw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (Src::kFetchAll) raw[i] = src.fetch(rw[i], col, col_ok);
        else if (rw[i].ok && col_ok) raw[i] = src.fetch(rw[i], col, true);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = rw[i].ok && col_ok ? src.finish(raw[i], rw[i], col) : make_uint4(0, 0, 0, 0);
    }

    if (kRow || kY) {
      const int64_t R = (int64_t)sh.batch * sh.rows_out;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + lr0 + i;
        const bool r_ok = r < sh.rows_out;
        const int64_t orow = (int64_t)b * sh.rows_out + r;
        if (kY && r_ok && col_ok) *reinterpret_cast<uint4*>(o.y + orow * sh.cols + col) = v[i];
        if (kRow) {
          const uint32_t sb = scale_byte_from_amax(quad_max(amax8(v[i])));
          const float sc = e8m0_to_f32(sb);
          if (r_ok && col_ok)
            *reinterpret_cast<uint2*>(o.row_q + orow * sh.cols + col) =
                make_uint2(cvt4_e4m3(v[i].x, v[i].y, sc), cvt4_e4m3(v[i].z, v[i].w, sc));
          uint32_t d = sb << (8 * (ch >> 2));
          d |= dpp_row_shr(d, 4);
          d |= dpp_row_shr(d, 8);
          if (r_ok && ch == 12) *reinterpret_cast<uint32_t*>(o.row_s + ((c0 >> 7) * R + orow) * 4) = d;
        }
      }
    }

    if (kCol) {
      // every wave is done with the row table (it shares the LDS tile) and with
      // the previous column tile's reads
      if (Src::kTable || kSub > 1) __syncthreads();
      const int slot = lr0 >> 3;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int cc = 8 * ch + j;
        const int k = j >> 1;
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a = tq_comp(v[2 * p], k), bb = tq_comp(v[2 * p + 1], k);
          d[p] = (j & 1) ? (a >> 16) | (bb & 0xFFFF0000u) : (a & 0xFFFFu) | (bb << 16);
        }
        *reinterpret_cast<uint4*>(lds + cc * 256 + 16 * (slot ^ tq_swz(cc))) = make_uint4(d[0], d[1], d[2], d[3]);
      }
      __syncthreads();
      // 8 lanes per column, 16 rows each (two slots): the 8 lanes of a column
      // store its 128 code bytes as one whole line.  Lanes 2q and 2q + 1 share
      // the 32-row block q (amax exchanged with a DPP quad permute); the
      // column's 4 scale bytes (lanes 0, 2, 4, 6 of the group) are merged with
      // row shifts into lane 6, which stores the panel dword.
      const int p = t & 7;
      const int64_t C = (int64_t)sh.batch * sh.cols;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int c = 32 * it + (t >> 3);
        const int64_t gc = c0 + c;
        const uint4 q0 = *reinterpret_cast<const uint4*>(lds + c * 256 + 16 * ((2 * p) ^ tq_swz(c)));
        const uint4 q1 = *reinterpret_cast<const uint4*>(lds + c * 256 + 16 * ((2 * p + 1) ^ tq_swz(c)));
        const uint32_t m0 = amax8(q0), m1 = amax8(q1);
        uint32_t m = m0 > m1 ? m0 : m1;
        const uint32_t mo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, true);  // lane ^ 1
        m = m > mo ? m : mo;
        const uint32_t sb = scale_byte_from_amax(m);
        const float sc = e8m0_to_f32(sb);
        const int64_t gr = r0 + 16 * p;   // rows_out % 32 == 0: the 16 rows are all in or all out
        if (gc < sh.cols && gr < sh.rows_out) {
          typedef unsigned int v4u_ __attribute__((ext_vector_type(4)));
          const v4u_ cw = {cvt4_e4m3(q0.x, q0.y, sc), cvt4_e4m3(q0.z, q0.w, sc), cvt4_e4m3(q1.x, q1.y, sc),
                           cvt4_e4m3(q1.z, q1.w, sc)};
          v4u_* dst = reinterpret_cast<v4u_*>(o.col_q + ((int64_t)b * sh.cols + gc) * sh.rows_out + gr);
          // Gathered sources walk the row bands of a column tile, so their
          // columnwise lines are written front to back: streamed (non-temporal)
          // stores are faster there (measured 7% on the gathered columnwise
          // quantize) and slightly slower for the plain order.
          if constexpr (Src::kGathered) __builtin_nontemporal_store(cw, dst);
          else *dst = cw;
        }
        uint32_t d = (p & 1) ? 0u : sb << (8 * (p >> 1));
        const uint32_t d2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d, 0x112, 0xF, 0xF, true);  // lane - 2
        d |= p >= 2 ? d2 : 0u;
        const uint32_t d4 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)d, 0x114, 0xF, 0xF, true);  // lane - 4
        d |= p >= 4 ? d4 : 0u;
        if (p == 6 && gc < sh.cols)
          *reinterpret_cast<uint32_t*>(o.col_s + ((r0 >> 7) * C + (int64_t)b * sh.cols + gc) * 4) = d;
      }
    }
  }
}

// Host side: the tile grid of a quantize, checked against its limits.
inline bool tq_shape(int64_t batch, int64_t rows_out, int64_t cols, TqShape& sh, unsigned& grid) {
  sh.rows_out = rows_out;
  sh.cols = cols;
  const int64_t ntr = (rows_out + kTq - 1) / kTq, ntc = (cols + kTq - 1) / kTq;
  const int64_t n = batch * ntr * ntc;
  if (n <= 0 || n > 0x7FFFFFFF || batch > 0x7FFFFFFF) return false;
  sh.n_tr = (int32_t)ntr;
  sh.n_tc = (int32_t)ntc;
  sh.batch = (int32_t)batch;
  grid = (unsigned)n;
  return true;
}

// Launch k_tile_quant with the outputs the caller asked for (row and/or col
// and/or the bf16 copy).  Returns the launch status.
template <class Src>
inline int tq_launch(const Src& src, const TqShape& sh, unsigned grid, const TqOut& o, hipStream_t st) {
  const bool r = o.row_q != nullptr, c = o.col_q != nullptr, y = o.y != nullptr;
  // grid: tiles, or groups of Src::kSub column tiles
  const dim3 g(Src::kSub == 1 ? grid
                              : (unsigned)((int64_t)sh.batch * sh.n_tr * ((sh.n_tc + Src::kSub - 1) / Src::kSub))),
      bl(kTqThreads);
  if (r && c && y) hipLaunchKernelGGL((k_tile_quant<Src, true, true, true>), g, bl, 0, st, src, sh, o);
  else if (r && c) hipLaunchKernelGGL((k_tile_quant<Src, true, true, false>), g, bl, 0, st, src, sh, o);
  else if (r && y) hipLaunchKernelGGL((k_tile_quant<Src, true, false, true>), g, bl, 0, st, src, sh, o);
  else if (r) hipLaunchKernelGGL((k_tile_quant<Src, true, false, false>), g, bl, 0, st, src, sh, o);
  else if (c && y) hipLaunchKernelGGL((k_tile_quant<Src, false, true, true>), g, bl, 0, st, src, sh, o);
  else if (c) hipLaunchKernelGGL((k_tile_quant<Src, false, true, false>), g, bl, 0, st, src, sh, o);
  else if (y) hipLaunchKernelGGL((k_tile_quant<Src, false, false, true>), g, bl, 0, st, src, sh, o);
  else return MX_EINVAL;
  return launch_status();
}

}  // namespace mx
