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
// XOR-swizzled by row so fragment reads are free of bank conflicts.
// Workgroups are persistent (one per CU) and walk the output tiles of their
// XCD's share in an order where concurrently running tiles share operand rows
// in that XCD's L2.

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
constexpr int kMaxGroups = 2048;                            // experts per grouped GEMM call
constexpr uint32_t kOob = 0x80000000u;                       // voffset that reads as zero

// 16-byte chunk swizzle of LDS row r.  ds_read_b128 serves 8 lanes (128 B)
// at a time; the 8 rows read by one such group must hit 8 distinct chunk
// columns.  Measured on gfx950: this XOR keeps fragment reads at the full
// LDS rate (~240 B/clk/CU), where (r + r/8) & 7 reaches only ~150.  It
// depends on r mod 16 only, so all fragments a lane reads share one chunk
// column and differ by a constant (immediate) offset.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// One operand tile: rows [0, rows) of a matrix starting at the tile's first
// row, ld bytes per row.  Scales in the panel layout: the dword of (panel p,
// tile row r) sits at p * pstride + 4 r from the tile's first scale dword.
struct TileSrc {
  __amdgpu_buffer_rsrc_t q, s;
  int64_t ld;
  int32_t pstride;
  int rows;
};

// q, s: codes and scale dword of the matrix's row 0; pstride = 4 x the rows
// of the whole scale panel (all groups / experts).
__device__ __forceinline__ TileSrc make_src(const uint8_t* q, const uint8_t* s, int64_t ld, int64_t pstride,
                                            int64_t row0, int64_t rows) {
  TileSrc t;
  const int64_t span = (int64_t)BM * ld;  // < 2^31 (checked on the host)
  t.q = __builtin_amdgcn_make_buffer_rsrc((void*)(q + row0 * ld), (short)0, (int)span, 0x00020000);
  // every panel of the tile's rows: < 2^31 bytes (checked on the host)
  const int64_t sspan = ((ld + 127) >> 7) * pstride;
  t.s = __builtin_amdgcn_make_buffer_rsrc((void*)(s + row0 * 4), (short)0, (int)sspan, 0x00020000);
  t.ld = ld;
  t.pstride = (int32_t)pstride;
  t.rows = rows < BM ? (int)rows : BM;
  return t;
}

// Codes of one operand tile, k window [k0, k0+128) with valid k in [k_lo, k_hi):
// block i (of 8) of wave w, i.e. LDS block 8w+i of 1 KB (8 rows); lane l
// writes slot l.
__device__ __forceinline__ void load_codes_blk(const TileSrc& t, uint8_t* lds_tile, int64_t k0, int64_t k_lo,
                                               int64_t k_hi, int i) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = 8 * w + i;
  const int row = 8 * blk + (lane >> 3);
  const int c = (lane & 7) ^ swz(row);
  // branch-free, 32-bit (tile spans are below 2^31): a lane-dependent branch
  // here would split the step into divergent blocks and stop the scheduler
  // from interleaving the loads with the MFMAs
  const int32_t k = (int32_t)k0 + 16 * c;
  const bool ok = (row < t.rows) & (k >= (int32_t)k_lo) & (k < (int32_t)k_hi);
  const uint32_t voff = ok ? (uint32_t)row * (uint32_t)t.ld + (uint32_t)k : kOob;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(t.q, (lds_void*)(lds_tile + blk * 1024), 16, voff, 0, 0, 0);
}

// The scale dword of the k step (panel k0 / 128) for each of the tile's 256
// rows: the rows' dwords are contiguous in the panel layout.
__device__ __forceinline__ void load_scales(const TileSrc& t, uint8_t* lds_sc, int64_t k0) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = 64 * w + lane;
  const uint32_t voff = row < t.rows ? (uint32_t)(k0 >> 7) * (uint32_t)t.pstride + 4u * (uint32_t)row : kOob;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(t.s, (lds_void*)(lds_sc + w * 256), 4, voff, 0, 0, 0);
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
        const uint2 p = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + m * ldc + n) = p;
      }
    }
  }
}

// One output tile's work: operand sources, contraction window, destination.
struct Tile {
  TileSrc A, B;
  int64_t k_begin, k_lo, k_hi;  // k steps start at k_begin; valid k in [k_lo, k_hi)
  int steps;
  void* out;
  int64_t ldc, m0, n0, n_end;
};

// Group schedule shared by the workgroup: clamped, monotone group bounds and
// (row-grouped problems) the running count of tiles before each group.
struct Sched {
  int32_t bound[kMaxGroups + 1];
  int32_t tiles_before[kMaxGroups + 1];
};

// Inclusive wave scan (sum or max) over the 64 lanes.
template <bool kMax>
__device__ __forceinline__ int32_t wave_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v = kMax ? (o > v ? o : v) : v + o;
  }
  return v;
}

// Wave 0 builds the schedule for E groups; tiles per group = ceil(len / BM) * n_tiles
// (n_tiles = 0 skips the tile counts).
__device__ void build_schedule(Sched& sc, const int32_t* offsets, int E, int64_t m_cap, int32_t n_tiles, bool align32) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int32_t carry_max = 0, carry_sum = 0, prev_last = 0;
    for (int base = 0; base <= E; base += 64) {
      const int i = base + lane;
      int32_t v = 0;
      if (i <= E) {
        const int64_t o = offsets[i];
        v = (int32_t)(o < 0 ? 0 : (o > m_cap ? m_cap : o));
        if (align32) v &= ~31;
      }
      v = wave_scan<true>(v);
      v = v > carry_max ? v : carry_max;
      if (i <= E) sc.bound[i] = v;
      // tiles of group i-1 = [bound[i-1], bound[i])
      const int32_t left = __shfl_up(v, 1, 64);
      const int32_t lo = lane == 0 ? prev_last : left;
      int32_t t = 0;
      if (i >= 1 && i <= E && n_tiles > 0) t = (v - lo + BM - 1) / BM * n_tiles;
      int32_t ps = wave_scan<false>(t) + carry_sum;
      if (i <= E) sc.tiles_before[i] = ps;
      carry_max = __shfl(v, 63, 64);
      carry_sum = __shfl(ps, 63, 64);
      prev_last = carry_max;
    }
  }
  __syncthreads();
}

// Schedule entries are the same for every lane: read them into scalar registers.
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Largest e in [0, E) with tiles_before[e] <= L (skips groups without tiles).
__device__ __forceinline__ int find_group(const Sched& sc, int E, int64_t L) {
  int lo = 0, hi = E;  // tiles_before[lo] <= L < tiles_before[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(sc.tiles_before[mid]) <= L) lo = mid; else hi = mid;
  }
  return lo;
}

struct RowsProblem {
  const uint8_t *a_q, *a_s, *b_q, *b_s;
  int64_t m_cap, N, K;
  void* out;
  bool f32;
};

__device__ __forceinline__ Tile rows_tile(const RowsProblem& p, const Sched& sc, int E, int64_t n_tiles, int64_t L) {
  Tile t;
  const int e = find_group(sc, E, L);
  const int64_t lo = uni(sc.bound[e]), hi = uni(sc.bound[e + 1]);
  const int64_t mt_e = (hi - lo + BM - 1) / BM;
  const int64_t rem = L - uni(sc.tiles_before[e]);
  const int64_t nt = rem / mt_e;
  const int64_t mt = rem - nt * mt_e;
  const int64_t row0 = lo + mt * BM;
  t.A = make_src(p.a_q, p.a_s, p.K, 4 * p.m_cap, row0, hi - row0);
  t.B = make_src(p.b_q + (int64_t)e * p.N * p.K, p.b_s + (int64_t)e * p.N * 4, p.K, 4 * (int64_t)E * p.N, nt * BN,
                 p.N - nt * BN);
  t.k_begin = 0;
  t.k_lo = 0;
  t.k_hi = p.K;
  t.steps = (int)((p.K + BK - 1) / BK);
  t.out = p.out;
  t.ldc = p.N;
  t.m0 = row0;
  t.n0 = nt * BN;
  t.n_end = p.N;
  return t;
}

// wgrad: tiles of an expert walked in bands of 4 m tiles, n-tile major inside
// a band, so concurrently running tiles share A and B rows.
__device__ __forceinline__ Tile wgrad_tile(const RowsProblem& p, const Sched& sc, int64_t m_tiles, int64_t n_tiles,
                                           int64_t L) {
  Tile t;
  const int64_t per = m_tiles * n_tiles;
  const int64_t e = L / per;
  const int64_t rem = L - e * per;
  constexpr int64_t kBand = 4;
  const int64_t band = rem / (kBand * n_tiles);
  const int64_t first_m = band * kBand;
  const int64_t band_m = (m_tiles - first_m) < kBand ? (m_tiles - first_m) : kBand;
  const int64_t in_band = rem - band * kBand * n_tiles;
  const int64_t mt = first_m + in_band % band_m;
  const int64_t nt = in_band / band_m;
  const int64_t lo = uni(sc.bound[e]), hi = uni(sc.bound[e + 1]);  // whole 32-blocks
  // here p.N is the dW row count and p.K its column count; the contraction runs over m_cap
  t.A = make_src(p.a_q, p.a_s, p.m_cap, 4 * p.N, mt * BM, p.N - mt * BM);
  t.B = make_src(p.b_q, p.b_s, p.m_cap, 4 * p.K, nt * BN, p.K - nt * BN);
  t.k_begin = lo & ~(int64_t)(BK - 1);
  t.k_lo = lo;
  t.k_hi = hi;
  t.steps = hi > lo ? (int)((hi - t.k_begin + BK - 1) / BK) : 0;
  t.out = p.f32 ? (void*)(static_cast<float*>(p.out) + e * p.N * p.K) : (void*)(static_cast<uint16_t*>(p.out) + e * p.N * p.K);
  t.ldc = p.K;
  t.m0 = mt * BM;
  t.n0 = nt * BN;
  t.n_end = p.K;
  return t;
}

// The loads of one k stage (A and B codes plus scales) into LDS stage dst,
// issued in 8 parts so they can be spread between MFMAs.
struct StageLoad {
  TileSrc A, B;
  uint8_t* dst;
  int64_t k0, k_lo, k_hi;
  bool active;
};

__device__ __forceinline__ void issue_part(const StageLoad& sl, int i) {
  load_codes_blk(sl.A, sl.dst, sl.k0, sl.k_lo, sl.k_hi, i);
  load_codes_blk(sl.B, sl.dst + kTileBytes, sl.k0, sl.k_lo, sl.k_hi, i);
  if (i == 0) {
    load_scales(sl.A, sl.dst + 2 * kTileBytes, sl.k0);
    load_scales(sl.B, sl.dst + 2 * kTileBytes + BM * 4, sl.k0);
  }
}

__device__ __forceinline__ void issue_stage(const StageLoad& sl) {
#pragma unroll
  for (int i = 0; i < 8; ++i) issue_part(sl, i);
}

// One k step of the wave's 128 x 128 sub-tile: 64 MFMAs, acc[i][j] covering
// A rows 16i.. and B rows 16j...  All 8 B fragments stay in registers; the A
// fragments are double buffered so row i+1 is read while row i multiplies.
// The next stage's loads are issued two at a time between the MFMA rows:
// issued back to back they stall the wave for thousands of cycles (memory
// pipeline back-pressure) before the first MFMA.
__device__ __forceinline__ void mma_step(const uint8_t* st, v4f (&acc)[8][8], int wm, int wn, const StageLoad& sl) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int g = lane >> 4;
  const uint8_t* At = st;
  const uint8_t* Bt = st + kTileBytes;
  const uint32_t* Sa = reinterpret_cast<const uint32_t*>(st + 2 * kTileBytes);
  const uint32_t* Sb = Sa + BM;
  v8i bf[8], af[2];
  int sb[8], sa[2];
  af[0] = frag(At, wm * 128 + r, g);
  sa[0] = (int)(Sa[wm * 128 + r] >> (8 * g));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int rb = wn * 128 + 16 * j + r;
    bf[j] = frag(Bt, rb, g);
    sb[j] = (int)(Sb[rb] >> (8 * g));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    issue_part(sl, i);
    if (i < 7) {
      const int ra = wm * 128 + 16 * (i + 1) + r;
      af[(i + 1) & 1] = frag(At, ra, g);
      sa[(i + 1) & 1] = (int)(Sa[ra] >> (8 * g));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i & 1], acc[i][j], 0, 0, 0, sb[j], 0,
                                                                   sa[i & 1]);
  }
  // Instruction order for the machine scheduler (the MFMA builtins are pure
  // and would otherwise all sink below the loads): the fragment reads first,
  // then per row: its share of the next stage's loads, the next A fragment,
  // and the row's 8 MFMAs.
#define MX_ROW(nvmem, nds)                                                   \
  __builtin_amdgcn_sched_group_barrier(0x020, nvmem, 0); /* VMEM read */     \
  __builtin_amdgcn_sched_group_barrier(0x100, nds, 0);   /* DS read */       \
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);     /* MFMA */
  __builtin_amdgcn_sched_group_barrier(0x100, 27, 0);  // A0, its scale, 8 B fragments and their scales
  MX_ROW(4, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 3)
  MX_ROW(2, 0)
#undef MX_ROW
  __builtin_amdgcn_sched_barrier(0);
  // The MFMA results are only consumed steps later, so the compiler would sink
  // the whole step's MFMAs below the step's s_waitcnt / s_barrier and they
  // would stop hiding the load latency.  An empty asm that claims to update
  // the accumulators keeps them above it.
#pragma unroll
  for (int i = 0; i < 8; ++i)
    asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                 "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
}

__device__ __forceinline__ void zero_acc(v4f (&acc)[8][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
}

// Tile source of the persistent loop (row-grouped or wgrad problems).
template <bool kWgrad>
struct TileGen {
  const RowsProblem& p;
  const Sched& sc;
  int E;
  int64_t m_tiles, n_tiles;
  __device__ __forceinline__ Tile operator()(int64_t l) const {
    return kWgrad ? wgrad_tile(p, sc, m_tiles, n_tiles, l) : rows_tile(p, sc, E, n_tiles, l);
  }
};

// One k step: MFMAs on LDS stage CUR while the next stage (the next k window
// of this tile, or the first one of the next tile) streams into the other.
// The two stages are distinct LDS objects and each step names them
// statically, so the compiler sees that the reads of one never alias the
// in-flight DMA writes of the other and does not wait for those loads
// before reading.
template <int CUR, typename Gen>
__device__ __forceinline__ void k_step(uint8_t* st0, uint8_t* st1, const Tile& cur, int s, bool has_next, int64_t Ln,
                                       const Gen& gen, bool& staged, v4f (&acc)[8][8], int wm, int wn) {
  uint8_t* comp = CUR ? st1 : st0;
  uint8_t* pre = CUR ? st0 : st1;
  __builtin_amdgcn_sched_barrier(0);  // keep each step's fragment reads inside the step
  StageLoad sl{cur.A, cur.B, pre, cur.k_begin + (int64_t)(s + 1) * BK, cur.k_lo, cur.k_hi, s + 1 < cur.steps};
  if (!sl.active && has_next) {
    const Tile nxt = gen(Ln);
    if (nxt.steps > 0) {
      sl = StageLoad{nxt.A, nxt.B, pre, nxt.k_begin, nxt.k_lo, nxt.k_hi, true};
      staged = true;
    }
  }
  if (!sl.active) {  // nothing to prefetch: every load of the stage becomes a zero read
    sl.A.rows = sl.B.rows = 0;
    sl.k_hi = sl.k_lo;
  }
  mma_step(comp, acc, wm, wn, sl);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Persistent workgroup: one per CU.  Logical tiles are split into 8 contiguous
// ranges, one per XCD (workgroup b runs on XCD b % 8); the workgroups of an
// XCD walk their range round robin.  The first k stage of the next tile is
// loaded during the last k step of the current one, so tile changes cost no
// exposed load latency and the epilogue stores overlap the next loads.
template <bool kF32, bool kWgrad>
__global__ void __launch_bounds__(kThreads) k_gemm(RowsProblem p, const int32_t* __restrict__ offsets, int32_t E) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStageBytes];
  __shared__ Sched sc;
  const int64_t m_tiles = (p.N + BM - 1) / BM;  // wgrad only
  const int64_t n_tiles = kWgrad ? (p.K + BN - 1) / BN : (p.N + BN - 1) / BN;
  build_schedule(sc, offsets, E, p.m_cap, kWgrad ? 0 : (int32_t)n_tiles, kWgrad);
  const int64_t total = kWgrad ? (int64_t)E * m_tiles * n_tiles : (int64_t)uni(sc.tiles_before[E]);
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t ctas_per_xcd = gridDim.x / kXcds;
  const int64_t x = blockIdx.x % kXcds;
  const int64_t L_end = (x + 1) * per_xcd < total ? (x + 1) * per_xcd : total;
  int64_t L = x * per_xcd + blockIdx.x / kXcds;
  if (L >= L_end) return;
  const TileGen<kWgrad> gen{p, sc, E, m_tiles, n_tiles};
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[8][8];
  zero_acc(acc);
  Tile cur = gen(L);
  int buf = 0;  // stage holding the current tile's first k window
  bool staged = false;
  while (true) {
    if (cur.steps > 0 && !staged) {
      uint8_t* st = buf ? st1 : st0;
      const StageLoad sl{cur.A, cur.B, st, cur.k_begin, cur.k_lo, cur.k_hi, true};
      issue_stage(sl);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int64_t Ln = L + ctas_per_xcd;
    const bool has_next = Ln < L_end;
    staged = false;
    int s = 0;
    if (buf && s < cur.steps) k_step<1>(st0, st1, cur, s++, has_next, Ln, gen, staged, acc, wm, wn);
    while (s + 1 < cur.steps) {
      k_step<0>(st0, st1, cur, s, has_next, Ln, gen, staged, acc, wm, wn);
      k_step<1>(st0, st1, cur, s + 1, has_next, Ln, gen, staged, acc, wm, wn);
      s += 2;
    }
    if (s < cur.steps) k_step<0>(st0, st1, cur, s++, has_next, Ln, gen, staged, acc, wm, wn);
    buf = (buf + cur.steps) & 1;
    store_tile<kF32>(cur.out, cur.ldc, cur.m0, cur.A.rows, cur.n0, cur.n_end, acc, wm, wn);
    zero_acc(acc);
    if (!has_next) break;
    cur = gen(Ln);
    L = Ln;
  }
}

template <bool kF32, bool kWgrad>
void launch(int ctas, hipStream_t st, const RowsProblem& p, const int32_t* off, int32_t E) {
  hipLaunchKernelGGL((k_gemm<kF32, kWgrad>), dim3(ctas), dim3(kThreads), 0, st, p, off, E);
}

template <bool kWgrad>
int launch_any(const RowsProblem& p, const int32_t* off, int32_t E, hipStream_t st) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MX_EHIP;
  const int ctas = (cus > 0 ? (cus + kXcds - 1) / kXcds : 1) * kXcds;
  if (p.f32) launch<true, kWgrad>(ctas, st, p, off, E);
  else launch<false, kWgrad>(ctas, st, p, off, E);
  return launch_status();
}

}  // namespace
}  // namespace mx

using namespace mx;

static int gemm_rows(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* b_q, const uint8_t* b_s,
                     const int32_t* offsets, int32_t E, int64_t m_cap, int64_t N, int64_t K, void* out,
                     int32_t out_dtype, mx_stream_t stream) {
  if (!a_q || !a_s || !b_q || !b_s || !offsets || !out) return MX_EINVAL;
  if (((uintptr_t)a_s | (uintptr_t)b_s) & 3) return MX_EINVAL;  // scale dwords
  if (E < 1 || m_cap < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * K >= (1ll << 31) || m_cap >= (1ll << 31)) return MX_EINVAL;  // 32-bit tile spans and bounds
  if (E > kMaxGroups) return MX_EUNSUPPORTED;
  if (m_cap == 0) return MX_OK;
  if (((m_cap + BM - 1) / BM + E) * ((N + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  const int64_t panels = (K + 127) / 128;  // scale spans addressed with 32-bit offsets
  if (panels * 4 * m_cap >= (1ll << 31) || panels * 4 * (int64_t)E * N >= (1ll << 31)) return MX_EINVAL;
  const RowsProblem p{a_q, a_s, b_q, b_s, m_cap, N, K, out, out_dtype == MX_OUT_F32};
  return launch_any<false>(p, offsets, E, reinterpret_cast<hipStream_t>(stream));
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
  if (((uintptr_t)dyt_s | (uintptr_t)xt_s) & 3) return MX_EINVAL;  // scale dwords
  if (num_groups < 1 || m_cap < 0 || m_cap % 32 || n <= 0 || k <= 0 || n % 32 || k % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * m_cap >= (1ll << 31)) return MX_EINVAL;  // buffer-resource span of one tile
  if (num_groups > kMaxGroups) return MX_EUNSUPPORTED;
  if ((int64_t)num_groups * ((n + BM - 1) / BM) * ((k + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  const int64_t panels = (m_cap + 127) / 128;
  if (panels * 4 * n >= (1ll << 31) || panels * 4 * k >= (1ll << 31)) return MX_EINVAL;
  const RowsProblem p{dyt_q, dyt_s, xt_q, xt_s, m_cap, n, k, dw, out_dtype == MX_OUT_F32};
  return launch_any<true>(p, group_offsets, num_groups, reinterpret_cast<hipStream_t>(stream));
}
