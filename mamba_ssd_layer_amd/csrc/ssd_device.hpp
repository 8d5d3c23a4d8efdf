// Device-side helpers shared by the libssd kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------- chunk geometry
// A chunk is at most Q consecutive tokens of one sequence.  Fixed-length
// batches: row b has nc_row = ceil(L/Q) chunks, chunk c = b*nc_row + k starts
// at token b*L + k*Q.  Packed batches: a table built on the device lists
// (sequence, first token, length) per chunk; unused entries have length 0.
struct ChunkGeom {
  int64_t L;             // tokens per row (fixed length)
  int32_t nc_row;        // chunks per row (fixed length)
  int32_t Q;             // chunk length
  const int32_t *table;  // packed: [nc_max][4]; nullptr for fixed length
};

struct ChunkInfo {
  int seq;
  int len;
  int64_t t0;
};

__device__ __forceinline__ ChunkInfo chunk_info(const ChunkGeom &g, int c) {
  ChunkInfo ci;
  if (g.table) {
    const int4 e = reinterpret_cast<const int4 *>(g.table)[c];
    ci.seq = e.x;
    ci.t0 = e.y;
    ci.len = e.z;
  } else {
    const int b = c / g.nc_row;
    const int k = c - b * g.nc_row;
    ci.seq = b;
    ci.t0 = (int64_t)b * g.L + (int64_t)k * g.Q;
    const int64_t rem = g.L - (int64_t)k * g.Q;
    ci.len = rem < g.Q ? (int)rem : g.Q;
  }
  return ci;
}

// XCD-aware block order for the (chunk, head) grids.  Workgroups are handed
// to the 8 XCDs round-robin by linear id, and each XCD has its own L2.  Block
// b runs chunk c = (b / (8 H)) * 8 + b % 8 and head h = (b / 8) % H, so every
// head of a chunk lands on the same XCD (the chunk's B and C are fetched into
// one L2 once and reused by all heads) and each XCD walks the heads of a chunk
// back to back (the chunk's token rows of x are read as contiguous runs).
// The grid has 8 * H * ceil(nc / 8) blocks; those with c >= nc exit.
constexpr int kXcds = 8;

__device__ __forceinline__ void xcd_chunk_head(int H, int &c, int &h) {
  const int b = blockIdx.x;
  const int r = b / kXcds;
  h = r % H;
  c = (r / H) * kXcds + (b % kXcds);
}

inline unsigned xcd_grid(int64_t nc, int H) {
  return (unsigned)(((nc + kXcds - 1) / kXcds) * kXcds * H);
}

// ----------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Word holding element (lo of a, lo of b) or (hi of a, hi of b): byte selects
// for v_perm_b32, which picks bytes of {a (bytes 4..7), b (bytes 0..3)}.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  // result = [b.lo16 (low half)?]  we want low half = a.lo, high half = b.lo
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  // low half = a.hi, high half = b.hi
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ----------------------------------------------------------------- MFMA wrappers
// v_mfma_f32_32x32x16_bf16: D(32x32) += A(32x16) * B(16x32), wave64.
// Operand layout: lane i holds A[row i%32][k = 8*(i/32) .. +7] and
// B[k = 8*(i/32) .. +7][col i%32].  Result: lane i, register r holds
// D[row 8*(r/4) + 4*(i/32) + r%4][col i%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of result register r for the lane group g = lane/32 (32x32 tiles).
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ----------------------------------------------------------------- direct-to-LDS loads
// gfx950 global_load_lds_dwordx4 / _dword: each lane fetches 16 (4) bytes from
// its own global address; the wavefront's 64 pieces land contiguously in LDS
// at the wave-uniform destination, lane i at +16i (+4i).  M0 carries the LDS
// byte offset, with the one wait state its write needs before the load.
//
// Issued from inline assembly on purpose: the compiler's wait insertion does
// not see these loads, so it adds no vmcnt wait in front of later LDS reads
// (for the builtin form it puts a full vmcnt(0) before every transposing LDS
// read that follows one, which drains any prefetch in flight).  Completion is
// tracked by explicit wait_vmcnt only, and every use of the data is preceded
// by one and, across wavefronts, by a barrier.
__device__ __forceinline__ uint32_t lds_off(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}
__device__ __forceinline__ void dma_lds16(const void *gsrc, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
               : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(const void *gsrc, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
               : "memory", "m0");
}
// Same, addressed as a wave-uniform 64-bit base (SGPRs) plus a per-lane
// 32-bit byte offset.
__device__ __forceinline__ void dma_lds16_sb(uint32_t voff, const void *sbase, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
               : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4_sb(uint32_t voff, const void *sbase, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_dst))
               : "memory", "m0");
}
__device__ __forceinline__ void load_lds16(const void *gsrc, unsigned char *lds_dst) {
  dma_lds16(gsrc, lds_off(lds_dst));
}

// s_waitcnt vmcnt(n) leaving expcnt and lgkmcnt alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) leaving vmcnt and expcnt alone.  Written out before a
// barrier that publishes LDS writes to the other wavefronts: at a loop's back
// edge, where the barrier follows an explicit vmcnt wait, the compiler has
// been seen to emit the barrier without waiting for an LDS write just
// before it (gfx950, ROCm 7.2 hipcc).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// s_waitcnt vmcnt(n) for a run-time n (a switch over the immediates); counts
// above 47 wait for everything.
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define SSD_W(i) case i: wait_vmcnt<i>(); break;
    SSD_W(0) SSD_W(1) SSD_W(2) SSD_W(3) SSD_W(4) SSD_W(5) SSD_W(6) SSD_W(7)
    SSD_W(8) SSD_W(9) SSD_W(10) SSD_W(11) SSD_W(12) SSD_W(13) SSD_W(14) SSD_W(15)
    SSD_W(16) SSD_W(17) SSD_W(18) SSD_W(19) SSD_W(20) SSD_W(21) SSD_W(22) SSD_W(23)
    SSD_W(24) SSD_W(25) SSD_W(26) SSD_W(27) SSD_W(28) SSD_W(29) SSD_W(30) SSD_W(31)
    SSD_W(32) SSD_W(33) SSD_W(34) SSD_W(35) SSD_W(36) SSD_W(37) SSD_W(38) SSD_W(39)
    SSD_W(40) SSD_W(41) SSD_W(42) SSD_W(43) SSD_W(44) SSD_W(45) SSD_W(46) SSD_W(47)
#undef SSD_W
    default: wait_vmcnt<0>(); break;
  }
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4i+j receives
// element j of the 4-element (8-byte) chunks addressed by lanes i, i+4, i+8,
// i+12 of the group -- a 16 x 4 transpose of bf16 data in LDS.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *lds_src) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(lds_src));
  return __builtin_bit_cast(u32x2, v);
}

// 16-byte chunk swizzle of an LDS tile row of `nc` chunks (XOR on the chunk
// index), so that 16 lanes reading the same chunk column of 16 consecutive
// rows hit distinct banks.
__device__ __forceinline__ constexpr int chunk_swz(int row, int nc) {
  return nc >= 16 ? (row & 15) : ((row >> 1) & (nc - 1));
}

template <typename T>
__device__ __forceinline__ T wave_bcast(T v, int src) { return __shfl(v, src, 64); }

// Token range of sequence s: fixed rows of L tokens, or cu_seqlens clamped to
// [0, T] (an inverted range is empty).
__device__ __forceinline__ void seq_range(const int32_t *cu, int s, int64_t L, int64_t T,
                                          int64_t &tb, int64_t &len) {
  if (cu) {
    tb = cu[s];
    const int64_t te = cu[s + 1];
    tb = tb < 0 ? 0 : (tb > T ? T : tb);
    len = (te > T ? T : te) - tb;
    if (len < 0) len = 0;
  } else {
    tb = (int64_t)s * L;
    len = L;
  }
}

// v plus its value in lane ^ 16 (lane ^ 32): gfx950's permlane swaps exchange
// the halves of a register pair without going through LDS; with both
// operands v, lane i receives {v_i, v_partner} in some order, and both lanes
// of a pair form the same sum.
__device__ __forceinline__ float xsum16(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float xsum32(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Sum over aligned groups of W consecutive lanes (W a power of two up to 64),
// every lane of a group receiving it: within 16-lane rows by DPP (quad swaps,
// half-row and row mirrors), across rows by permlane swaps.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "power of two");
  auto dpp = [](float a, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  if (W >= 2) v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
  if (W >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  if (W >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if (W >= 16) v += dpp(v, std::integral_constant<int, 0x140>{}); // row_mirror
  if (W >= 32) v = xsum16(v);
  if (W >= 64) v = xsum32(v);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Stores 16 rows of a bf16 tile, 8 * KQ 16-byte chunks a row, held as lane
// (c16 = lane % 16, g4 = lane / 16) owning chunk 4q + g4 of row c16 in v[q].
// Storing v[q] as it stands writes 64-byte pieces of 16 rows; instead the
// lanes of rows c16 and c16 + 8 trade the halves of each pair v[2m], v[2m+1]
// (a DPP rotate by 8 lanes within each 16-lane row), so that each store
// writes whole 128-byte segments of 8 rows.  The same number of stores is
// issued.  row0 points at the first of the 16 rows; ld is the row pitch in
// elements.
template <int KQ>
__device__ __forceinline__ void store_rows128(uint16_t *row0, int64_t ld, const u32x4 (&v)[KQ],
                                              int c16, int g4) {
  static_assert(KQ % 2 == 0, "pairs of 64-byte pieces");
  auto ror8 = [](uint32_t a) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(a), 0x128, 0xF, 0xF, false));
  };
  const bool lo = c16 < 8;
  const int r = c16 & 7, ch = g4 + 4 * (c16 >> 3);
#pragma unroll
  for (int m = 0; m < KQ / 2; ++m) {
    const u32x4 x = v[2 * m], y = v[2 * m + 1];
    const u32x4 rx{ror8(x.x), ror8(x.y), ror8(x.z), ror8(x.w)};
    const u32x4 ry{ror8(y.x), ror8(y.y), ror8(y.z), ror8(y.w)};
    // rows 0-7: own piece (chunk g4) or row c16 - 8's second piece (chunk 4 + g4);
    // rows 8-15 likewise from the first pieces
    const u32x4 a = lo ? x : ry, b = lo ? rx : y;
    *reinterpret_cast<u32x4 *>(row0 + r * ld + 8 * (8 * m + ch)) = a;
    *reinterpret_cast<u32x4 *>(row0 + (8 + r) * ld + 8 * (8 * m + ch)) = b;
  }
}

// Packed batches (cu_seqlens): wave-parallel walks over the sequences, 64 a
// step (lane i reads sequence i0 + i), so a block finds its place in a few
// rounds of loads instead of one dependent load per sequence.  Every lane of
// the wavefront must make the call (shuffles and ballots).

// A value equal on every lane, moved to a scalar register (so that addresses
// built from it stay wave-uniform).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// ceil(len_i / u) for sequence i (0 past the last sequence).
__device__ __forceinline__ int64_t seq_units(const int32_t *cu, int i, int rows, int64_t T, int u) {
  if (i >= rows) return 0;
  int64_t tb, len;
  seq_range(cu, i, 0, T, tb, len);
  return (len + u - 1) / u;
}

// Inclusive prefix sum over the wavefront's 64 lanes.
__device__ __forceinline__ int64_t wave_scan_incl(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Sum over the sequences i < s of ceil(len_i / u).
__device__ inline int64_t units_before(const int32_t *cu, int s, int64_t T, int u) {
  int64_t acc = 0;
  for (int i0 = 0; i0 < s; i0 += 64) {
    const int64_t v = seq_units(cu, i0 + (threadIdx.x & 63), s, T, u);
    acc += __shfl(wave_scan_incl(v), 63, 64);
  }
  return uniform64(acc);
}

// Units of u tokens listed sequence-major (sequence i holds ceil(len_i / u)
// of them): the sequence holding unit c, and in `before` the units of the
// sequences ahead of it; -1 if c is past the last unit.
__device__ inline int locate_unit(const int32_t *cu, int rows, int64_t T, int64_t c, int u,
                                  int64_t &before) {
  int64_t acc = 0;
  for (int i0 = 0; i0 < rows; i0 += 64) {
    const int64_t v = seq_units(cu, i0 + (threadIdx.x & 63), rows, T, u);
    const int64_t incl = wave_scan_incl(v);
    // the first lane whose running total passes c holds a nonempty sequence
    const unsigned long long m = __ballot(acc + incl > c);
    if (m) {
      const int f = __builtin_ctzll(m);
      before = uniform64(acc + __shfl(incl - v, f, 64));
      return __builtin_amdgcn_readfirstlane(i0 + f);
    }
    acc += __shfl(incl, 63, 64);
  }
  before = uniform64(acc);
  return -1;
}

// Index of sequence s's first 64-token pair of chunks in the sequence-major
// list of the batch's pairs (the layout of the saved per-pair states).
__device__ inline int64_t pair_base64(const int32_t *cu, int s, int64_t L, int64_t T) {
  if (!cu) return (int64_t)s * ((L + 63) / 64);
  return units_before(cu, s, T, 64);
}

}  // namespace ssd
