// Block-scaled MXFP8 grouped GEMMs (gfx950): expert forward, dgrad and wgrad.
//
// digest "Key Questions Answered": the block-scaled matrix multiply applies the
// per-block scales inside the matrix instruction (the Blackwell design
// dequantizes through tensor memory; on CDNA4 the scales go straight into
// V_MFMA_SCALE_F32_32X32X64_F8F6F4, so there is no dequantize step at all).
// pytorch/ao PR #3203, "Next steps": the grouped GEMM takes pre-quantized
// MXFP8 tensors (codes + scales).
//
// Every product is "NT": C[m, n] = sum_k A[m, k] B[n, k], both operands
// contiguous along k, scales in the panel layout of mx_device.h.  One kernel
// body serves
//   fwd / dgrad : rows of A grouped by expert (group e multiplies B_e)
//   wgrad       : the contraction axis grouped by expert (dW_e = A_e . B_e^T)
//
// Scaled MFMA operand layout (32x32x64, E4M3 x E4M3, measured on gfx950):
//   operand rows: lane l holds row (l & 31); with h = l >> 5 its bytes 0..15
//      are k = 16h .. 16h+15 and bytes 16..31 are k = 32+16h .. 32+16h+15.
//   scale: lane l supplies the E8M0 byte of (its row, 32-block h) of the
//      64-wide k step (op_sel 0 reads bits 7:0 of the scale operand).
//   D[i][j] = sum_k first[i][k] second[j][k]: lane l, register r holds
//      D[8 (r >> 2) + 4 h + (r & 3)][l & 31].
// The kernel passes the B tile as the first operand, so each lane holds runs
// of 4 consecutive output columns of one output row.
//
// Tiling: 256 x 256 output tile per 256-thread workgroup (one per CU), 2 x 2
// waves of 128 x 128 (4 x 4 MFMA tiles of 32 x 32 each), k steps of 64.
// Operands are loaded in k lines of 128 bytes per row (two k steps): each
// buffer load writes 8 rows x 128 bytes straight into LDS, so every request
// is a whole 128-byte line (a 16-row x 64-byte load moves the same bytes in
// twice as many half-line requests, and the load stream is what bounds this
// kernel).  A load past a row or contraction bound returns zeros, which pads
// ragged tiles for free.  Two LDS slots of one k line each: while the steps
// of k line j run on one slot, k line j + 1 is loaded into the other.  The
// even step of a k line reads the odd step's fragments too, so the odd step
// frees its slot with a barrier at its start and loads the k line after next
// into it, one load per MFMA slot; at its middle it waits for k line j + 1
// (one wait and two barriers per k line).  The next step's fragments are
// always read during the second half of a step, so a step never starts on
// an LDS read.  Both steps of a k line use the same 128-wide scale panel
// dword, read once.  LDS rows (128 B) are XOR-swizzled by 16-byte chunk
// (conflict free for the fragment reads).  Workgroups are persistent (one
// per CU) and walk the output tiles of their XCD's share in an order where
// concurrently running tiles share operand rows in that XCD's L2; the loads
// run ahead across tile boundaries.

#include "mx_device.h"

// The LDS-direct loads below set M0 in inline asm (see dma16).
#pragma clang diagnostic ignored "-Winline-asm"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxGroups = 2048;                        // experts per grouped GEMM call
constexpr uint32_t kOob = 0x80000000u;                  // voffset that reads as zero
// k lines: 128 bytes of each operand row (two k steps), loaded as whole
// lines.  An LDS slot holds one k line of the tile: A rows 0-127, B rows
// 0-127, A rows 128-255, B rows 128-255 (16 KB each, 128-byte rows), then
// the A and B scale dwords.
constexpr int kLine = 2 * BK;
constexpr int kRegion = 128 * kLine;
constexpr int kSlotScale = 4 * kRegion;
constexpr int kSlotBytes = 4 * kRegion + 2 * BM * 4;
constexpr int kEpiOff = 2 * kRegion;   // the epilogue stages through rows 128-255 and the scales

// The bf16 baseline runs the same kernel with bf16 operands: 64 bytes of a
// row hold 32 bf16, so a k step contracts 32 elements with two
// V_MFMA_F32_32X32X16_BF16 per 32 x 32 tile (the same MFMA cycles and LDS
// bytes per step as one scaled FP8 MFMA of 64), and there are no scales.
template <bool kBf16>
struct Elt {
  static constexpr int kBytes = kBf16 ? 2 : 1;          // bytes per operand element
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in
// bits 15:14, expcnt in 6:4, lgkmcnt in 11:8).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// 16-byte chunk swizzle of a 128-byte LDS row: 16 consecutive rows read at
// one chunk column fall in 16 distinct bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// Group schedule shared by the workgroup: clamped, monotone group bounds and
// (row-grouped problems) the running count of tiles before each group.
struct Sched {
  int32_t bound[kMaxGroups + 1];
  int32_t tiles_before[kMaxGroups + 1];
  int64_t split[2];   // wgrad: the bounds of the workgroup's XCD range of tiles
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

// wgrad work per tile of group e, in k steps: the ring steps of the group's
// contraction range plus an allowance of 4 for the epilogue (an empty
// group's tiles only store zeros).
template <bool kBf16>
__device__ __forceinline__ int64_t wgrad_unit(const Sched& sc, int e) {
  const int32_t lo = sc.bound[e], hi = sc.bound[e + 1];
  constexpr int32_t eb = kBf16 ? 2 : 1;
  const int32_t kb = (lo * eb) & ~127;
  const int32_t steps = hi > lo ? (hi * eb - kb + 63) / 64 : 0;
  return ((steps + 3) & ~3) + 4;
}

// Wave 0 splits the wgrad tiles (T per group, group-major) into 8 ranges of
// about equal work, one per XCD, and stores the bounds of XCD x's range:
// the first tile L at which the work of the tiles before L reaches x/8 (and
// (x+1)/8) of the total.
template <bool kBf16>
__device__ void wgrad_split(Sched& sc, int E, int64_t T, int x) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t total = 0;
    for (int base = 0; base < E; base += 64) {
      int64_t u = base + lane < E ? wgrad_unit<kBf16>(sc, base + lane) : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = __shfl_xor(u, d, 64);
        u += o;
      }
      total += u;
    }
    const int64_t W = total * T;                 // all lanes hold the same total
    const int64_t goal0 = (int64_t)x * W, goal1 = (int64_t)(x + 1) * W;   // compared with 8 x work
    int64_t carry = 0;
    if (lane == 0) {
      sc.split[0] = x == 0 ? 0 : (int64_t)E * T;
      sc.split[1] = (int64_t)E * T;
    }
    __builtin_amdgcn_wave_barrier();
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const int64_t u = e < E ? wgrad_unit<kBf16>(sc, e) : 0;
      int64_t S = u;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = __shfl_up(S, d, 64);
        if (lane >= d) S += o;
      }
      S += carry;
      const int64_t P = S - u;
      if (e < E) {
        if (x > 0 && 8 * T * P <= goal0 && goal0 < 8 * T * S)
          sc.split[0] = (int64_t)e * T + (goal0 - 8 * T * P + 8 * u - 1) / (8 * u);
        if (x + 1 < 8 && 8 * T * P <= goal1 && goal1 < 8 * T * S)
          sc.split[1] = (int64_t)e * T + (goal1 - 8 * T * P + 8 * u - 1) / (8 * u);
      }
      carry = __shfl(S, 63, 64);
    }
  }
  __syncthreads();
}

struct Problem {
  const uint8_t *a_q, *a_s, *b_q, *b_s;
  int64_t m_cap, N, K;
  void* out;
  bool f32;
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (the four dwords of a V#): base, stride 0,
// num_records bytes, the same flags as __builtin_amdgcn_make_buffer_rsrc uses.
__device__ __forceinline__ v4u rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4u{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)bytes, 0x00020000u};
}

// Where a tile's operands come from (the loader's view).
struct LoadTile {
  v4u aq, as, bq, bs;                      // codes / scales from the tile's first A and B rows
  int32_t rows_a, rows_b;                  // valid rows (<= 256) of the two operand tiles
  int32_t k_begin, k_lo, k_hi;             // k steps start at k_begin (a multiple of 128); valid k in [k_lo, k_hi)
  int32_t steps;
};

// Where a tile's result goes (the compute side's view).
struct OutTile {
  void* out;
  int64_t ldc, m0, n0, n_end;
  int32_t rows;   // valid output rows
  int32_t steps;
  int32_t blk_lo, blk_hi;   // valid 32-blocks of the contraction, counted from k_begin
};

// Tile coordinates of logical tile L.
struct Coord {
  int64_t e, row_a, row_b;  // group, first A row, first B row (within B_e for row problems)
  int32_t rows_a, rows_b, k_begin, k_lo, k_hi, steps;
};

// (32-bit tile arithmetic: tile counts are below 2^31, checked on the host;
// 32-bit divisions are much shorter than 64-bit ones)
template <bool kWgrad, bool kBf16>
__device__ __forceinline__ Coord coord(const Problem& p, const Sched& sc, int E, int64_t m_tiles, int64_t n_tiles,
                                       int64_t L64) {
  Coord c;
  const uint32_t L = (uint32_t)L64;
  if (!kWgrad) {
    // rows of group e in tiles of 256; a group's tiles walked in bands of b
    // m tiles, n-tile major inside a band.  The 32 tiles an XCD runs at once
    // then form a b x 32/b block sharing b A and 32/b B row panels in its
    // L2.  Over the group, A panels are fetched about n_tiles * b / 32 times
    // and B panels once per band, so b minimizes mt_e * b + 32 * ceil(mt_e / b)
    // (b = mt_e, one band, for small groups).
    const int e = find_group(sc, E, L64);
    const int32_t lo = uni(sc.bound[e]), hi = uni(sc.bound[e + 1]);
    const uint32_t mt_e = (uint32_t)(hi - lo + BM - 1) / BM;
    const uint32_t rem = L - (uint32_t)uni(sc.tiles_before[e]);
    uint32_t kBand = 1, best = ~0u;
    for (uint32_t b = 1; b <= 8 && b <= mt_e; ++b) {
      const uint32_t cost = mt_e * b + 32 * ((mt_e + b - 1) / b);
      if (cost <= best) {
        best = cost;
        kBand = b;
      }
    }
    const uint32_t per_band = kBand * (uint32_t)n_tiles;
    const uint32_t band = rem / per_band;
    const uint32_t first_m = band * kBand;
    const uint32_t band_m = (mt_e - first_m) < kBand ? (mt_e - first_m) : kBand;
    const uint32_t in_band = rem - band * per_band;
    const uint32_t nt = in_band / band_m;
    const uint32_t mt = first_m + (in_band - nt * band_m);
    c.e = e;
    c.row_a = lo + (int64_t)mt * BM;
    c.row_b = (int64_t)nt * BN;
    c.rows_a = (int32_t)(hi - c.row_a < BM ? hi - c.row_a : BM);
    c.rows_b = (int32_t)(p.N - c.row_b < BN ? p.N - c.row_b : BN);
    // k in bytes of an operand row
    c.k_begin = 0;
    c.k_lo = 0;
    c.k_hi = (int32_t)(p.K * Elt<kBf16>::kBytes);
    c.steps = (int32_t)((p.K * Elt<kBf16>::kBytes + BK - 1) / BK);
  } else {
    // dW_e tiles walked in bands of 4 m tiles, n-tile major inside a band, so
    // concurrently running tiles share A and B rows
    const uint32_t mtl = (uint32_t)m_tiles, ntl = (uint32_t)n_tiles;
    const uint32_t per = mtl * ntl;
    const uint32_t e = L / per;
    const uint32_t rem = L - e * per;
    constexpr uint32_t kBand = 4;
    const uint32_t band = rem / (kBand * ntl);
    const uint32_t first_m = band * kBand;
    const uint32_t band_m = (mtl - first_m) < kBand ? (mtl - first_m) : kBand;
    const uint32_t in_band = rem - band * kBand * ntl;
    const uint32_t nt = in_band / band_m;
    const uint32_t mt = first_m + (in_band - nt * band_m);
    const int32_t lo = uni(sc.bound[e]), hi = uni(sc.bound[e + 1]);  // whole 32-blocks
    // p.N is the dW row count, p.K its column count; the contraction runs over m_cap
    c.e = e;
    c.row_a = (int64_t)mt * BM;
    c.row_b = (int64_t)nt * BN;
    c.rows_a = (int32_t)(p.N - c.row_a < BM ? p.N - c.row_a : BM);
    c.rows_b = (int32_t)(p.K - c.row_b < BN ? p.K - c.row_b : BN);
    // k in bytes of an operand row; MX steps start at the group's 128-row
    // scale panel, bf16 steps at the group's first row
    constexpr int32_t eb = Elt<kBf16>::kBytes;
    c.k_begin = (lo * eb) & ~127;
    c.k_lo = lo * eb;
    c.k_hi = hi * eb;
    c.steps = hi > lo ? (c.k_hi - c.k_begin + BK - 1) / BK : 0;
  }
  return c;
}

template <bool kWgrad, bool kBf16>
__device__ __forceinline__ LoadTile load_tile(const Problem& p, const Coord& c, int E) {
  LoadTile t;
  const int64_t ld = (kWgrad ? p.m_cap : p.K) * Elt<kBf16>::kBytes;  // bytes per operand row
  const int64_t pa = kWgrad ? 4 * p.N : 4 * p.m_cap;      // scale panel strides
  const int64_t pb = kWgrad ? 4 * p.K : 4 * (int64_t)E * p.N;
  const int64_t panels = (ld + 127) >> 7;
  const uint8_t* bq = kWgrad ? p.b_q : p.b_q + c.e * p.N * p.K * Elt<kBf16>::kBytes;
  const uint8_t* bs = kWgrad ? p.b_s : p.b_s + c.e * p.N * 4;
  // num_records: rows past the valid ones read as zero; every span is below
  // 2^31 (checked on the host)
  t.aq = rsrc(p.a_q + c.row_a * ld, c.rows_a * ld);
  t.bq = rsrc(bq + c.row_b * ld, c.rows_b * ld);
  t.as = rsrc(p.a_s + c.row_a * 4, panels * pa);
  t.bs = rsrc(bs + c.row_b * 4, panels * pb);
  t.rows_a = c.rows_a;
  t.rows_b = c.rows_b;
  t.k_begin = c.k_begin;
  t.k_lo = c.k_lo;
  t.k_hi = c.k_hi;
  t.steps = c.steps;
  return t;
}

template <bool kWgrad>
__device__ __forceinline__ OutTile out_tile(const Problem& p, const Coord& c) {
  OutTile o;
  if (!kWgrad) {
    o.out = p.out;
    o.ldc = p.N;
    o.n_end = p.N;
  } else {
    o.out = p.f32 ? (void*)(static_cast<float*>(p.out) + c.e * p.N * p.K)
                  : (void*)(static_cast<uint16_t*>(p.out) + c.e * p.N * p.K);
    o.ldc = p.K;
    o.n_end = p.K;
  }
  o.m0 = c.row_a;
  o.n0 = c.row_b;
  o.rows = c.rows_a;
  o.steps = c.steps;
  o.blk_lo = (c.k_lo - c.k_begin) >> 5;
  o.blk_hi = (c.k_hi - c.k_begin) >> 5;
  return o;
}

// Everything needed to walk the workgroup's tiles.
template <bool kWgrad, bool kBf16>
struct Walk {
  const Problem& p;
  const Sched& sc;
  int E;
  int64_t m_tiles, n_tiles, stride, L_end;
  __device__ __forceinline__ Coord at(int64_t L) const { return coord<kWgrad, kBf16>(p, sc, E, m_tiles, n_tiles, L); }
};

// Per-lane constants of the loads.  Code load i (0..7) of wave w covers 8
// rows x 128 bytes: tile rows 128 (i >> 2) + 8 (4 (i & 3) + w) + l / 8, LDS
// chunk l & 7 holding the global chunk (l & 7) ^ swz8(row).  The chunk is
// the same for all 8 loads of a lane.  Scale loads: lane l of wave w fetches
// the dword of tile row 64 w + l.
struct LaneLoads {
  uint32_t voff[8];   // row * ld + 16 * chunk
  int32_t kc;         // 16 * chunk
  int32_t srow;       // 64 w + l
};

// k steps a tile occupies in the ring: its own rounded up to a multiple of 4
// (two k lines per LDS slot pair), so every tile starts on slot 0 and the
// ring can be unrolled with a single loop exit; the padding steps load
// zeros and add zeros.
__device__ __forceinline__ int32_t ring_steps(int32_t steps) { return (steps + 3) & ~3; }

// The loader walks the same tiles as the compute side, two k lines ahead,
// skipping tiles without k steps.  s counts k steps (2 per k line).
struct Loader {
  LoadTile t;
  int64_t L;
  int32_t s;
  bool valid;
};

template <bool kWgrad, bool kBf16>
__device__ __forceinline__ void loader_seek(Loader& ld, const Walk<kWgrad, kBf16>& w) {
  while (ld.valid && ld.s >= ring_steps(ld.t.steps)) {
    ld.L += w.stride;
    if (ld.L >= w.L_end) {
      ld.valid = false;
    } else {
      ld.t = load_tile<kWgrad, kBf16>(w.p, w.at(ld.L), w.E);
      ld.s = 0;
    }
  }
}

// One LDS-direct buffer load (16 B or 4 B per lane) into LDS at byte lds
// (+ 16 or 4 x lane).  Written as inline asm so the compiler neither tracks
// it nor adds waits for it: every wait on these loads is explicit (vmcnt in
// stage_barrier), and the slot a load writes is never read before that
// wait and a barrier.  M0 holds the LDS address; nothing else in these
// kernels uses M0 (gfx9 LDS instructions do not read it).
__device__ __forceinline__ void dma16(const v4u& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "m0");
}

__device__ __forceinline__ void dma4(const v4u& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// The loads of one k line into one LDS slot: 18 instructions per wave, in
// this order: 0..7 rows 0-127 of A and B (A0 B0 A1 B1 A2 B2 A3 B3), 8..15
// rows 128-255 (A4 B4 .. A7 B7), 16 and 17 the A and B scale dwords.  An odd
// step issues the first 8 or 10 of them, the next even step the rest (see
// k_step).  A loader past its last tile issues the same instructions with
// out-of-range offsets (they read zeros).
struct LoadPlan {
  v4u aq, bq, as, bs;
  uint32_t v[8];       // code voffsets (out of range where the lane's chunk is outside [k_lo, k_hi))
  uint32_t soff;       // k line start
  uint32_t sa, sb;     // scale voffsets
  uint32_t pa, pb;     // scale panel offsets
  uint32_t dst;        // LDS address of the slot + this wave's first 1 KB block
  uint32_t sdst;       // LDS address of the slot's scales + this wave's rows
};

__device__ __forceinline__ LoadPlan plan_line(const Loader& ld, const LaneLoads& ll, const uint8_t* slot,
                                              int64_t pstride_a, int64_t pstride_b) {
  LoadPlan pl;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t kl = ld.t.k_begin + BK * ld.s;   // a multiple of 128 bytes
  const int32_t k = kl + ll.kc;
  const bool ok = ld.valid & (k >= ld.t.k_lo) & (k < ld.t.k_hi);
#pragma unroll
  for (int i = 0; i < 8; ++i) pl.v[i] = ok ? ll.voff[i] : kOob;
  pl.aq = ld.t.aq;
  pl.bq = ld.t.bq;
  pl.as = ld.t.as;
  pl.bs = ld.t.bs;
  pl.soff = ld.valid ? (uint32_t)kl : 0u;
  // a k line with no valid k (ring padding) reads no scales: its panel
  // offset may lie past the scale tensor
  const bool kin = ld.valid & (kl < ld.t.k_hi) & (kl + kLine > ld.t.k_lo);
  pl.sa = (kin & (ll.srow < ld.t.rows_a)) ? 4u * (uint32_t)ll.srow : kOob;
  pl.sb = (kin & (ll.srow < ld.t.rows_b)) ? 4u * (uint32_t)ll.srow : kOob;
  pl.pa = ld.valid ? (uint32_t)(kl >> 7) * (uint32_t)pstride_a : 0u;
  pl.pb = ld.valid ? (uint32_t)(kl >> 7) * (uint32_t)pstride_b : 0u;
  pl.dst = lds_addr(slot) + (uint32_t)(w * 1024);
  pl.sdst = lds_addr(slot) + (uint32_t)(kSlotScale + w * 256);
  return pl;
}

// Load number n (0..17) of a plan; the bf16 operands have no scale loads.
template <bool kBf16>
__device__ __forceinline__ void load_n(const LoadPlan& pl, int n) {
  if (n < 16) {
    const int i = (n < 8 ? 0 : 4) + ((n & 7) >> 1);   // code load i: rows 128 (i >> 2) + ...
    const uint32_t off = (uint32_t)((2 * (i >> 2) + (n & 1)) * kRegion + 4 * (i & 3) * 1024);
    dma16((n & 1) ? pl.bq : pl.aq, pl.dst + off, pl.v[i], pl.soff);
  } else if (kBf16) {
  } else if (n == 16) {
    dma4(pl.as, pl.sdst, pl.sa, pl.pa);
  } else {
    dma4(pl.bs, pl.sdst + BM * 4, pl.sb, pl.pb);
  }
}

// The MFMA operands of one k step for one wave.  Scales hold the raw panel
// dwords until shifted at the start of the step that uses them.
struct Frags {
  v8i a[4], b[4];
  int sa[4], sb[4];
};

// Lane offsets of a fragment inside a 32-row block of 128-byte rows, for the
// first (p = 0) and second (p = 1) k step of the line: row r = l & 31,
// chunks 4 p + h and 4 p + 2 + h (h = l >> 5), swizzled.  swz8 depends on
// the row's bits 1..3 only, so rows 32 i + r of any block share these
// offsets and a fragment is read at (block base) + offset with the block
// base an immediate.
struct FragOff {
  int lo[2], hi[2], sc;   // code chunk offsets per step parity, scale dword offset
};

__device__ __forceinline__ FragOff frag_off() {
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
  FragOff f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    f.lo[p] = r * kLine + 16 * ((4 * p + h) ^ swz8(r));
    f.hi[p] = r * kLine + 16 * ((4 * p + 2 + h) ^ swz8(r));
  }
  f.sc = 4 * r;
  return f;
}

template <int P>
__device__ __forceinline__ v8i frag(const uint8_t* blk, const FragOff& fo) {
  const uint4 lo = *reinterpret_cast<const uint4*>(blk + fo.lo[P]);
  const uint4 hi = *reinterpret_cast<const uint4*>(blk + fo.hi[P]);
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// Base of a wave's 128 rows of A (wm) or B (wn) in a slot.
__device__ __forceinline__ const uint8_t* a_base(const uint8_t* slot, int wm) { return slot + 2 * wm * kRegion; }
__device__ __forceinline__ const uint8_t* b_base(const uint8_t* slot, int wn) { return slot + (2 * wn + 1) * kRegion; }

// The E8M0 byte a lane passes to the MFMA (bits 7:0 of the operand): byte
// sel / 8 of the panel dword, or 0 (2^-127, applied to zero codes) when the
// width is 0.
__device__ __forceinline__ int scale_byte(int v, int sel, uint32_t width) {
  return (int)__builtin_amdgcn_ubfe((uint32_t)v, (uint32_t)sel, width);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

// One k step of one 32 x 32 tile: a scaled FP8 MFMA over 64 k, or for bf16
// operands two bf16 MFMAs over the lane's two 16-byte chunks (A and B
// fragments share the lane -> k layout, so the k order of the two halves
// does not matter).
template <bool kBf16>
__device__ __forceinline__ v16f mma(const v8i& b, const v8i& a, const v16f& c, int sb, int sa) {
  if constexpr (kBf16) {
    const v8bf b0 = __builtin_bit_cast(v8bf, v4i{b[0], b[1], b[2], b[3]});
    const v8bf a0 = __builtin_bit_cast(v8bf, v4i{a[0], a[1], a[2], a[3]});
    const v8bf b1 = __builtin_bit_cast(v8bf, v4i{b[4], b[5], b[6], b[7]});
    const v8bf a1 = __builtin_bit_cast(v8bf, v4i{a[4], a[5], a[6], a[7]});
    const v16f t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, a0, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, a1, t, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, sb, 0, sa);
  }
}

// The MFMA results are only consumed tiles later, so the compiler would sink
// MFMAs below the step's waits and barrier; an empty asm that claims to update
// the accumulators keeps each half in place.
__device__ __forceinline__ void pin(v16f (&acc)[4][4], int i0) {
#pragma unroll
  for (int i = i0; i < i0 + 2; ++i)
    asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
}

__device__ __forceinline__ void zero_acc(v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Tile epilogue, staged through LDS so that every global store writes whole
// 128-byte lines.  Each wave owns a quarter of the staging area (rows
// 128-255 and the scales of LDS slot 1), 32 rows x 272 B
// (64 fp32 columns + 16 B of padding, which puts the 32 rows written by one
// ds_write_b128 in distinct bank groups).  For each 32 x 64 part of its
// 128 x 128 result, a wave writes the fp32 accumulators (straight from the
// accumulator registers), reads them back 8 consecutive columns per lane,
// converts, and stores 8 rows x 64 columns per instruction.  Rows and
// columns outside the tile get out-of-range offsets and are dropped.
constexpr int kEpiPitch = 272;
// cache policy of the output stores: non-temporal (streamed; the output is
// not read again by this kernel)
constexpr int kStoreNt = 2;
constexpr int kEpiSlice = 32 * kEpiPitch;
static_assert(4 * kEpiSlice == kSlotBytes - kEpiOff, "the epilogue uses rows 128-255 and the scales of a slot");

template <bool kF32>
__device__ __forceinline__ void store_tile(const OutTile& o, const v16f (&acc)[4][4], int wm, int wn,
                                           uint8_t* stage) {
  typedef unsigned int v4u_ __attribute__((ext_vector_type(4)));
  constexpr int kEs = kF32 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* slice = stage + wave * kEpiSlice;
  const int64_t pitch = o.ldc * kEs;  // bytes per output row, < 2^23 (checked on the host)
  char* base = static_cast<char*>(o.out) + (o.m0 * o.ldc + o.n0) * kEs;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)(o.rows * pitch), 0x00020000);
  const int wr = lane & 31, h = lane >> 5;      // write side: accumulator layout
  const int rr = lane >> 3, c8 = lane & 7;      // read side: 8 lanes per row, 8 columns each
  const int32_t cols = (int32_t)(o.n_end - o.n0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v16f& v = acc[i][2 * jp + jj];
          *reinterpret_cast<float4*>(slice + wr * kEpiPitch + (32 * jj + 8 * q + 4 * h) * 4) =
              make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      // The slice is exchanged between lanes of the wave.  The wave's LDS
      // accesses execute in order, but the compiler reasons per lane: without
      // this clobber it may reuse an earlier read of the same address or move
      // a read across another lane's write.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int row = 8 * it + rr;
        const float4 a = *reinterpret_cast<const float4*>(slice + row * kEpiPitch + 32 * c8);
        const float4 b = *reinterpret_cast<const float4*>(slice + row * kEpiPitch + 32 * c8 + 16);
        const int ml = wm * 128 + 32 * i + row;
        const int col = wn * 128 + 64 * jp + 8 * c8;  // n_end % 32 == 0: the 8 columns are all in or all out
        const uint32_t voff =
            (ml < o.rows) & (col < cols) ? (uint32_t)ml * (uint32_t)pitch + (uint32_t)(col * kEs) : kOob;
        if (kF32) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u_, a), r, voff, 0, kStoreNt);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u_, b), r, voff + 16, 0, kStoreNt);
        } else {
          const v4u_ d = {bf16x2_rne(a.x, a.y), bf16x2_rne(a.z, a.w), bf16x2_rne(b.x, b.y), bf16x2_rne(b.z, b.w)};
          __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, 0, kStoreNt);
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

// Compute-side cursor.
struct Cursor {
  OutTile t;
  int64_t L;
  int32_t s;      // k step within the tile (padding steps included)
};

// After the last step of a tile: store it and move on to the next tile with k
// steps, storing exact zeros for tiles without any (wgrad of an empty group).
// Returns false when the workgroup has no tiles left.
//
// Vector memory operations complete in issue order, stores included: the
// next odd step's wait covers the tile's stores too.  The epilogue stages
// through rows 128-255 and the scales of slot 1 (the loads in flight at a
// tile end write its rows 0-127); the next even step's loads overwrite the
// staging area, and a barrier after the epilogue keeps every wave's reads
// ahead of them.
template <bool kF32, bool kWgrad, bool kBf16>
__device__ __forceinline__ bool finish_tile(Cursor& c, const Walk<kWgrad, kBf16>& w, v16f (&acc)[4][4], int wm, int wn,
                                            uint8_t* stage) {
  store_tile<kF32>(c.t, acc, wm, wn, stage);
  zero_acc(acc);
  c.s = 0;
  bool more = true;
  while (true) {
    c.L += w.stride;
    if (c.L >= w.L_end) {
      more = false;
      break;
    }
    c.t = out_tile<kWgrad>(w.p, w.at(c.L));
    if (c.t.steps > 0) break;
    store_tile<kF32>(c.t, acc, wm, wn, stage);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  return more;
}

// Wait until the own loads of the next k line are complete (kVm younger
// vector memory operations may stay in flight), then a workgroup barrier.
// The barrier is a bare s_barrier: the fence of __syncthreads would also wait
// for the loads of the k line after it.  Compiler-level memory clobbers keep
// LDS accesses from moving across it.
template <int kVm>
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(kVm));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One k step: the first (ODD = false) or second half of the k line in slot
// SLOT.  Even step: on entry `cur` holds the step's B fragments and A
// fragments 0, 1; A fragments 2, 3 are read during the first half, and all
// eight fragments of the odd step (same slot, other k half) during the
// second half.  Odd step: everything is in registers; a barrier at the start
// frees the slot (every wave has read it), the loads of the k line after
// next go into it from the step's first MFMA slot, the mid-step wait
// (vmcnt(8): the 8 loads issued before it may
// still be in flight) and barrier make the next k line visible, and the
// second half reads the next even step's fragments from the other slot.
// LOADS: which loads of the current plan the step issues: even steps 8..17
// (kE8) or 10..17 (kE10), two in every three MFMA slots from the first; odd
// steps 0..7 (kO8) or 0..9 (kO10), one per slot from the first.
constexpr int kE8 = 0, kE10 = 1, kO8 = 2, kO10 = 3;
template <int SLOT, bool ODD, int LOADS, bool kWgrad, bool kBf16>
__device__ __forceinline__ void k_step(uint8_t* s0, uint8_t* s1, Frags& cur, Frags& nxt, v16f (&acc)[4][4],
                                       Loader& ld, LoadPlan& plan, const LaneLoads& ll, Cursor& c,
                                       const Walk<kWgrad, kBf16>& w, int wm, int wn, int64_t pa, int64_t pb,
                                       const FragOff& fo) {
  uint8_t* const cst = SLOT == 0 ? s0 : s1;
  uint8_t* const ost = SLOT == 0 ? s1 : s0;
  constexpr int P = ODD ? 1 : 0;
  const int h = (threadIdx.x >> 5) & 1;
  const int sel = 8 * (2 * P + h);
  const int32_t bi = 2 * c.s + h;
  const uint32_t bok = (bi >= c.t.blk_lo) & (bi < c.t.blk_hi) ? 8u : 0u;
  const uint8_t* A = a_base(cst, wm);
  const uint8_t* B = b_base(cst, wn);
  const uint8_t* SA = cst + kSlotScale + wm * 128 * 4;
  const uint8_t* nA = a_base(ost, wm);
  const uint8_t* nB = b_base(ost, wn);
  const uint8_t* nSA = ost + kSlotScale + wm * 128 * 4;
  const uint8_t* nSB = ost + kSlotScale + BM * 4 + wn * 128 * 4;
  if constexpr (ODD) {
    plan = plan_line(ld, ll, cst, pa, pb);
    ld.s += 2;
    loader_seek<kWgrad, kBf16>(ld, w);
    // every wave has read this slot (the reads completed at the end of the
    // even step): the loads below may overwrite it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  int xa[4] = {0, 0, 0, 0}, xb[4] = {0, 0, 0, 0};   // the step's scale bytes
  if constexpr (!kBf16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) xb[j] = scale_byte(cur.sb[j], sel, bok);
    xa[0] = scale_byte(cur.sa[0], sel, bok);
    xa[1] = scale_byte(cur.sa[1], sel, bok);
    if constexpr (ODD) {
      xa[2] = scale_byte(cur.sa[2], sel, bok);
      xa[3] = scale_byte(cur.sa[3], sel, bok);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int L0 = LOADS == kE8 ? 8 : LOADS == kE10 ? 10 : 0;
  constexpr int LN = LOADS == kE8 ? 10 : LOADS == kE10 ? 8 : LOADS == kO8 ? 8 : 10;
#define MX_MFMA(i, j) acc[i][j] = mma<kBf16>(cur.b[j], cur.a[i], acc[i][j], xb[j], xa[i]);
#define MX_FENCE __builtin_amdgcn_sched_barrier(0);
// odd steps: load t in MFMA slot t; even steps: load t in slot 3 (t / 2) + t % 2
#define MX_L(t)                                                                                   \
  if constexpr (ODD) {                                                                            \
    if constexpr ((t) < LN) load_n<kBf16>(plan, L0 + (t));                                        \
  } else if constexpr ((t) % 3 != 2 && 2 * ((t) / 3) + (t) % 3 < LN) {                           \
    load_n<kBf16>(plan, L0 + 2 * ((t) / 3) + (t) % 3);                                            \
  }
#define MX_E(x) if constexpr (!ODD) { x; }
#define MX_SE(x) if constexpr (!kBf16 && !ODD) { x; }
#define MX_SO(x) if constexpr (!kBf16 && ODD) { x; }
  // first half: MFMAs of A fragments 0, 1; an even step reads A fragments 2, 3
  MX_MFMA(0, 0) MX_L(0) MX_E(cur.a[2] = frag<0>(A + 64 * kLine, fo))                               MX_FENCE
  MX_MFMA(0, 1) MX_L(1) MX_SE(cur.sa[2] = *reinterpret_cast<const int*>(SA + 256 + fo.sc))         MX_FENCE
  MX_MFMA(0, 2) MX_L(2) MX_E(cur.a[3] = frag<0>(A + 96 * kLine, fo))                               MX_FENCE
  MX_MFMA(0, 3) MX_L(3) MX_SE(cur.sa[3] = *reinterpret_cast<const int*>(SA + 384 + fo.sc))         MX_FENCE
  MX_MFMA(1, 0) MX_L(4)                                                                            MX_FENCE
  MX_MFMA(1, 1) MX_L(5)                                                                            MX_FENCE
  MX_MFMA(1, 2) MX_L(6)                                                                            MX_FENCE
  MX_MFMA(1, 3) MX_L(7)                                                                            MX_FENCE
  pin(acc, 0);
  if constexpr (ODD) stage_barrier<8>();   // the next k line complete (8 younger loads may remain)
  MX_FENCE
  if constexpr (!kBf16 && !ODD) {
    xa[2] = scale_byte(cur.sa[2], sel, bok);
    xa[3] = scale_byte(cur.sa[3], sel, bok);
  }
  // second half: MFMAs of A fragments 2, 3; the next step's fragments (even:
  // all eight, same slot, k half 1; odd: B0-3, A0, A1 and scales, other slot, k half 0)
  MX_MFMA(2, 0) MX_L(8)  if constexpr (ODD) { nxt.b[0] = frag<0>(nB, fo); } else { nxt.b[0] = frag<1>(B, fo); } MX_SO(nxt.sb[0] = *reinterpret_cast<const int*>(nSB + fo.sc))       MX_FENCE
  MX_MFMA(2, 1) MX_L(9)  if constexpr (ODD) { nxt.b[1] = frag<0>(nB + 32 * kLine, fo); } else { nxt.b[1] = frag<1>(B + 32 * kLine, fo); } MX_SO(nxt.sb[1] = *reinterpret_cast<const int*>(nSB + 128 + fo.sc)) MX_FENCE
  MX_MFMA(2, 2) MX_L(10) if constexpr (ODD) { nxt.b[2] = frag<0>(nB + 64 * kLine, fo); } else { nxt.b[2] = frag<1>(B + 64 * kLine, fo); } MX_SO(nxt.sb[2] = *reinterpret_cast<const int*>(nSB + 256 + fo.sc)) MX_FENCE
  MX_MFMA(2, 3) MX_L(11) if constexpr (ODD) { nxt.b[3] = frag<0>(nB + 96 * kLine, fo); } else { nxt.b[3] = frag<1>(B + 96 * kLine, fo); } MX_SO(nxt.sb[3] = *reinterpret_cast<const int*>(nSB + 384 + fo.sc)) MX_FENCE
  MX_MFMA(3, 0) MX_L(12) if constexpr (ODD) { nxt.a[0] = frag<0>(nA, fo); } else { nxt.a[0] = frag<1>(A, fo); } MX_SO(nxt.sa[0] = *reinterpret_cast<const int*>(nSA + fo.sc))       MX_FENCE
  MX_MFMA(3, 1) MX_L(13) if constexpr (ODD) { nxt.a[1] = frag<0>(nA + 32 * kLine, fo); } else { nxt.a[1] = frag<1>(A + 32 * kLine, fo); } MX_SO(nxt.sa[1] = *reinterpret_cast<const int*>(nSA + 128 + fo.sc)) MX_FENCE
  MX_MFMA(3, 2) MX_L(14) MX_E(nxt.a[2] = frag<1>(A + 64 * kLine, fo))                                                                       MX_FENCE
  MX_MFMA(3, 3) MX_L(15) MX_E(nxt.a[3] = frag<1>(A + 96 * kLine, fo))                                                                       MX_FENCE
#undef MX_MFMA
#undef MX_FENCE
#undef MX_L
#undef MX_E
#undef MX_SE
#undef MX_SO
  if constexpr (!kBf16 && !ODD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nxt.sa[i] = cur.sa[i];
      nxt.sb[i] = cur.sb[i];
    }
  }
  pin(acc, 2);
  // the next step's fragments are in registers before this wave reaches the
  // next barrier, after which other waves may overwrite their slot
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);
  ++c.s;
}

// Persistent workgroup: one per CU.  Logical tiles are split into 8 contiguous
// ranges, one per XCD (workgroup b runs on XCD b % 8); the workgroups of an
// XCD walk their range round robin.  Forward and dgrad tiles all have K / 64
// steps: the ranges hold equal tile counts.  A wgrad tile's steps follow its
// group's size (an empty group's tiles only store zeros): the ranges hold
// equal work (wgrad_split).
template <bool kF32, bool kWgrad, bool kBf16>
__global__ void __launch_bounds__(kThreads) k_gemm(Problem p, const int32_t* __restrict__ offsets, int32_t E) {
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kSlotBytes];
  __shared__ Sched sc;
  const int64_t m_tiles = (p.N + BM - 1) / BM;  // wgrad only
  const int64_t n_tiles = kWgrad ? (p.K + BN - 1) / BN : (p.N + BN - 1) / BN;
  build_schedule(sc, offsets, E, p.m_cap, kWgrad ? 0 : (int32_t)n_tiles, kWgrad);
  const int64_t total = kWgrad ? (int64_t)E * m_tiles * n_tiles : (int64_t)uni(sc.tiles_before[E]);
  const int64_t x = blockIdx.x % kXcds;
  int64_t L_begin, L_end;
  if (kWgrad) {
    // tiles differ in work (the groups' contraction lengths): ranges of equal work
    wgrad_split<kBf16>(sc, E, m_tiles * n_tiles, (int)x);
    L_begin = sc.split[0];
    L_end = sc.split[1];
  } else {
    const int64_t per_xcd = (total + kXcds - 1) / kXcds;
    L_begin = x * per_xcd;
    L_end = (x + 1) * per_xcd < total ? (x + 1) * per_xcd : total;
  }
  const int64_t L0 = L_begin + blockIdx.x / kXcds;
  if (L0 >= L_end) return;
  const Walk<kWgrad, kBf16> w{p, sc, E, m_tiles, n_tiles, (int64_t)(gridDim.x / kXcds), L_end};
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lane = threadIdx.x & 63;
  const int64_t ldb = (kWgrad ? p.m_cap : p.K) * Elt<kBf16>::kBytes;  // bytes per operand row
  const int64_t pa = kWgrad ? 4 * p.N : 4 * p.m_cap;
  const int64_t pb = kWgrad ? 4 * p.K : 4 * (int64_t)E * p.N;
  LaneLoads ll;
  {
    const int rr = 8 * wave + (lane >> 3);   // region row of load 0 (load i adds 32 (i & 3))
    const int ch = (lane & 7) ^ swz8(rr);
    ll.kc = 16 * ch;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 128 * (i >> 2) + 32 * (i & 3) + rr;
      ll.voff[i] = (uint32_t)row * (uint32_t)ldb + 16u * (uint32_t)ch;
    }
  }
  ll.srow = 64 * wave + lane;
  v16f acc[4][4];
  zero_acc(acc);
  // compute cursor: leading tiles without k steps are stored as zeros
  Cursor c;
  c.L = L0;
  c.s = 0;
  c.t = out_tile<kWgrad>(p, w.at(L0));
  while (c.t.steps == 0) {
    store_tile<kF32>(c.t, acc, wm, wn, st1 + kEpiOff);
    c.L += w.stride;
    if (c.L >= L_end) return;
    c.t = out_tile<kWgrad>(p, w.at(c.L));
  }
  // loader: starts at the same tile; the prologue loads k line 0 into slot 0
  // and issues loads 0..7 of k line 1 (slot 1), as the odd step before the
  // first even step would
  Loader ld;
  ld.L = c.L;
  ld.t = load_tile<kWgrad, kBf16>(p, w.at(c.L), E);
  ld.s = 0;
  ld.valid = true;
  LoadPlan plan = plan_line(ld, ll, st0, pa, pb);
#pragma unroll
  for (int n = 0; n < 18; ++n) load_n<kBf16>(plan, n);
  ld.s += 2;
  loader_seek<kWgrad, kBf16>(ld, w);
  stage_barrier<0>();
  const FragOff fo = frag_off();
  Frags fa, fb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    fa.b[j] = frag<0>(b_base(st0, wn) + 32 * j * kLine, fo);
    fa.sb[j] = *reinterpret_cast<const int*>(st0 + kSlotScale + BM * 4 + (wn * 128 + 32 * j) * 4 + fo.sc);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    fa.a[i] = frag<0>(a_base(st0, wm) + 32 * i * kLine, fo);
    fa.sa[i] = *reinterpret_cast<const int*>(st0 + kSlotScale + (wm * 128 + 32 * i) * 4 + fo.sc);
  }
  plan = plan_line(ld, ll, st1, pa, pb);
#pragma unroll
  for (int n = 0; n < 8; ++n) load_n<kBf16>(plan, n);
  ld.s += 2;
  loader_seek<kWgrad, kBf16>(ld, w);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  // Loads per k line (18 per wave): the odd step of slot 0 issues 0..9 of
  // its plan and the next even step 10..17; the odd step of slot 1 issues
  // 0..7 only (it may end a tile, whose epilogue stages through its slot's
  // rows 128-255) and the next even step 8..17.  Tiles hold a multiple of 4
  // steps, so a tile always ends on the odd step of slot 1.
  do {
    k_step<0, false, kE8, kWgrad, kBf16>(st0, st1, fa, fb, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
    k_step<0, true, kO10, kWgrad, kBf16>(st0, st1, fb, fa, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
    k_step<1, false, kE10, kWgrad, kBf16>(st0, st1, fa, fb, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
    k_step<1, true, kO8, kWgrad, kBf16>(st0, st1, fb, fa, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
    while (c.s < c.t.steps) {
      k_step<0, false, kE8, kWgrad, kBf16>(st0, st1, fa, fb, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
      k_step<0, true, kO10, kWgrad, kBf16>(st0, st1, fb, fa, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
      k_step<1, false, kE10, kWgrad, kBf16>(st0, st1, fa, fb, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
      k_step<1, true, kO8, kWgrad, kBf16>(st0, st1, fb, fa, acc, ld, plan, ll, c, w, wm, wn, pa, pb, fo);
    }
  } while (finish_tile<kF32, kWgrad, kBf16>(c, w, acc, wm, wn, st1 + kEpiOff));
  // loads past the last tile may still be writing LDS
  __builtin_amdgcn_s_waitcnt(0);
}

template <bool kF32, bool kWgrad, bool kBf16>
void launch(int ctas, hipStream_t st, const Problem& p, const int32_t* off, int32_t E) {
  hipLaunchKernelGGL((k_gemm<kF32, kWgrad, kBf16>), dim3(ctas), dim3(kThreads), 0, st, p, off, E);
}

template <bool kWgrad, bool kBf16>
int launch_any(const Problem& p, const int32_t* off, int32_t E, hipStream_t st) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MX_EHIP;
  const int ctas = (cus > 0 ? (cus + kXcds - 1) / kXcds : 1) * kXcds;
  if (p.f32) launch<true, kWgrad, kBf16>(ctas, st, p, off, E);
  else launch<false, kWgrad, kBf16>(ctas, st, p, off, E);
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
  // 16-byte LDS-direct operand loads and 16-byte output stores
  if (((uintptr_t)a_q | (uintptr_t)b_q | (uintptr_t)out) & 15) return MX_EINVAL;
  if (E < 1 || m_cap < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * K >= (1ll << 31) || m_cap >= (1ll << 31)) return MX_EINVAL;  // 32-bit tile spans and bounds
  if (E > kMaxGroups) return MX_EUNSUPPORTED;
  if (m_cap == 0) return MX_OK;
  if (((m_cap + BM - 1) / BM + E) * ((N + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  const int64_t panels = (K + 127) / 128;  // scale spans addressed with 32-bit offsets
  if (panels * 4 * m_cap >= (1ll << 31) || panels * 4 * (int64_t)E * N >= (1ll << 31)) return MX_EINVAL;
  if (N >= (1 << 21)) return MX_EINVAL;  // output tile spans 256 rows x N x 4 bytes < 2^31
  const Problem p{a_q, a_s, b_q, b_s, m_cap, N, K, out, out_dtype == MX_OUT_F32};
  return launch_any<false, false>(p, offsets, E, reinterpret_cast<hipStream_t>(stream));
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
  // 16-byte LDS-direct operand loads and 16-byte output stores
  if (((uintptr_t)dyt_q | (uintptr_t)xt_q | (uintptr_t)dw) & 15) return MX_EINVAL;
  if (num_groups < 1 || m_cap < 0 || m_cap % 32 || n <= 0 || k <= 0 || n % 32 || k % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * m_cap >= (1ll << 31)) return MX_EINVAL;  // buffer-resource span of one tile
  if (num_groups > kMaxGroups) return MX_EUNSUPPORTED;
  if ((int64_t)num_groups * ((n + BM - 1) / BM) * ((k + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  const int64_t panels = (m_cap + 127) / 128;
  if (panels * 4 * n >= (1ll << 31) || panels * 4 * k >= (1ll << 31)) return MX_EINVAL;
  if (k >= (1 << 21)) return MX_EINVAL;  // output tile spans 256 rows x k x 4 bytes < 2^31
  const Problem p{dyt_q, dyt_s, xt_q, xt_s, m_cap, n, k, dw, out_dtype == MX_OUT_F32};
  return launch_any<true, false>(p, group_offsets, num_groups, reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// bf16 baseline: the same grouped products with bf16 operands and no scales.
// Operand rows are 2 * K (or 2 * M_cap) bytes; the scale pointers of the
// problem are never read (the operand pointers stand in for them).

static int bf16_rows(const uint16_t* a, const uint16_t* b, const int32_t* offsets, int32_t E, int64_t m_cap,
                     int64_t N, int64_t K, void* out, int32_t out_dtype, mx_stream_t stream) {
  if (!a || !b || !offsets || !out) return MX_EINVAL;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)out) & 15) return MX_EINVAL;  // 16-byte operand loads and stores
  if (E < 1 || m_cap < 0 || N <= 0 || K <= 0 || N % 32 || K % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * 2 * K >= (1ll << 31) || m_cap >= (1ll << 31)) return MX_EINVAL;  // 32-bit tile spans and bounds
  if (E > kMaxGroups) return MX_EUNSUPPORTED;
  if (m_cap == 0) return MX_OK;
  if (((m_cap + BM - 1) / BM + E) * ((N + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  if (N >= (1 << 21)) return MX_EINVAL;  // output tile spans 256 rows x N x 4 bytes < 2^31
  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(a);
  const uint8_t* b8 = reinterpret_cast<const uint8_t*>(b);
  const Problem p{a8, a8, b8, b8, m_cap, N, K, out, out_dtype == MX_OUT_F32};
  return launch_any<false, true>(p, offsets, E, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int mx_bf16_grouped_gemm_fwd(const uint16_t* a, const uint16_t* b, const int32_t* group_offsets,
                                        int32_t num_groups, int64_t m_cap, int64_t n, int64_t k, void* out,
                                        int32_t out_dtype, mx_stream_t stream) {
  return bf16_rows(a, b, group_offsets, num_groups, m_cap, n, k, out, out_dtype, stream);
}

extern "C" int mx_bf16_grouped_gemm_dgrad(const uint16_t* dy, const uint16_t* wt, const int32_t* group_offsets,
                                          int32_t num_groups, int64_t m_cap, int64_t n_out, int64_t k_contract,
                                          void* dx, int32_t out_dtype, mx_stream_t stream) {
  return bf16_rows(dy, wt, group_offsets, num_groups, m_cap, n_out, k_contract, dx, out_dtype, stream);
}

extern "C" int mx_bf16_grouped_gemm_wgrad(const uint16_t* dyt, const uint16_t* xt, const int32_t* group_offsets,
                                          int32_t num_groups, int64_t m_cap, int64_t n, int64_t k, void* dw,
                                          int32_t out_dtype, mx_stream_t stream) {
  if (!dyt || !xt || !group_offsets || !dw) return MX_EINVAL;
  if (((uintptr_t)dyt | (uintptr_t)xt | (uintptr_t)dw) & 15) return MX_EINVAL;  // 16-byte operand loads and stores
  if (num_groups < 1 || m_cap < 0 || m_cap % 32 || n <= 0 || k <= 0 || n % 32 || k % 32) return MX_EINVAL;
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32) return MX_EINVAL;
  if ((int64_t)BM * 2 * m_cap >= (1ll << 31)) return MX_EINVAL;  // buffer-resource span of one tile
  if (num_groups > kMaxGroups) return MX_EUNSUPPORTED;
  if ((int64_t)num_groups * ((n + BM - 1) / BM) * ((k + BN - 1) / BN) >= (1ll << 31)) return MX_EINVAL;
  if (k >= (1 << 21)) return MX_EINVAL;  // output tile spans 256 rows x k x 4 bytes < 2^31
  const uint8_t* a8 = reinterpret_cast<const uint8_t*>(dyt);
  const uint8_t* b8 = reinterpret_cast<const uint8_t*>(xt);
  const Problem p{a8, a8, b8, b8, m_cap, n, k, dw, out_dtype == MX_OUT_F32};
  return launch_any<true, true>(p, group_offsets, num_groups, reinterpret_cast<hipStream_t>(stream));
}
