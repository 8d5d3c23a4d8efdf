// libssd: the whole SSD forward in one pass per (sequence, head), the state
// kept on chip across chunks (the blockwise evaluation of page "Mamba-2
// Architecture: State Space Duality Explained", "2. The Chunked SSD
// Algorithm", with the three chunk-level steps -- chunk state, hand-off,
// output -- done back to back for each chunk instead of as separate passes
// over all chunks).  Chunking is exact, so the chunk length is a free choice:
// this kernel walks 32-token chunks, for which the intra-chunk product is one
// 32 x 32 causal tile.
//
// Design.  Block = (sequence, HPB heads of one group) in XCD-aware order (all
// heads of a sequence on one XCD, so its B and C rows come from one L2),
// 2 HPB wavefronts: wavefront (head hh, half ph) owns state rows p in
// [32 ph, 32 ph + 32) of head hh, held transposed (h^T, rows n, columns p) as
// 2 x N/16 fp32 tiles of the 16x16x32 bf16 MFMA.  The block's heads share
// their B and C tiles in LDS.  The launch uses HPB = 2 (two or three blocks a
// CU); four heads a block (one block a CU) cut the B/C traffic further but
// measured no faster, since each wavefront's chunk latency dominates.
//
// Data movement.  An R-slot LDS ring per block holds chunk k's x (a 32 x 64
// tile per head), B, C and dt while chunks k+1 .. k+R-2 are in flight
// (direct-to-LDS loads; wavefront (hh, ph) fetches rows [16 ph, 16 ph + 16)
// of head hh's x, whole 128-byte rows).  Vector-memory operations complete in
// issue order, so a wavefront knows chunk k has landed once at most the
// operations it issued after that chunk are pending; it waits for exactly
// that count, then one barrier per chunk publishes the tiles.  Each
// wavefront stages its y (bf16) over its own columns of the chunk's x tile
// once it has read them; at the next chunk's top, after the barrier,
// wavefront (hh, ph) stores rows [16 ph, 16 ph + 16) of head hh's y as whole
// rows and then refills exactly those LDS rows with a later chunk's x.  No
// workspace: nothing but x, B, C, dt and y crosses HBM.
//
// Per chunk and wavefront (a_l = cumulative sum of dt A within the chunk,
// from a DPP scan of the 32 dt values):
//   1. inter term: Y^T = h C^T on MFMA, the A-operand being the state rows
//      rounded to bf16 in their accumulator order (C read in the same order),
//      then scaled by exp(a_l);
//   2. intra term: Z^T = B C^T for the three nonzero 16 x 16 tiles of the
//      causal 32 x 32 block (same K order), the decay exp(a_l - a_s) dt_s
//      applied per element in the log2 domain and the tile above the diagonal
//      masked, then Y^T += X^T G^T with the accumulators as B-operands and
//      X^T from transposing LDS reads in the matching token order; plus D x;
//   3. state: h^T = exp(a_last) h^T + B^T (w x) with w_s = exp(a_last - a_s)
//      dt_s, from transposing reads of B and the same X^T registers.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// v_mfma_f32_16x16x32_bf16: D(16x16) += A(16x32) * B(32x16), wave64.  Lane i
// holds A[row i%16][k = 8(i/16) .. +7] and B[k = 8(i/16) .. +7][col i%16];
// result register r of lane i is D[row 4(i/16) + r][col i%16].
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// DPP move of v across lanes (0 where the source lane is outside the row or
// the destination row is masked off).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// Inclusive prefix sum over lanes 0..31 and, independently, over 32..63:
// shifts 1, 2, 4, 8 within each 16-lane row, then row 15's total carried
// into rows 1 and 3.
__device__ __forceinline__ float scan32(float a) {
  a += dpp<0x111, 0xF>(a);
  a += dpp<0x112, 0xF>(a);
  a += dpp<0x114, 0xF>(a);
  a += dpp<0x118, 0xF>(a);
  a += dpp<0x142, 0xA>(a);
  return a;
}

// XOR swizzle of the 16-byte chunks of an LDS tile row (NC = 8 or 16 chunks a
// row).  The transposing reads take 4 consecutive rows x 4 consecutive
// chunks per 16 lanes, and the row operands 16 consecutive rows x 1 chunk:
// swapping the row's two low bit pairs into the chunk index (16 chunks), or
// the row-pair index's (8 chunks), keeps both patterns on distinct banks.
template <int NC>
__device__ __forceinline__ int rot_swz(int r) {
  return NC == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Geometry of one kernel instance: N state size, HPB heads per block, R ring slots.
template <int N, int HPB, int R>
struct FusedCfg {
  static constexpr int P = 64, CQ = 32, WAVES = 2 * HPB, THREADS = 64 * WAVES;
  static constexpr int XH = CQ * P * 2;          // x of one head and chunk: 32 rows x 128 B
  static constexpr int BT = CQ * N * 2;          // B (or C) of a chunk
  static constexpr int DW = 64 * 4;              // one wavefront's dt piece
  static constexpr int OX = 0, OB = HPB * XH, OC = OB + BT, OD = OC + BT;
  static constexpr int SLOT = OD + WAVES * DW;
  static constexpr int AD = R * SLOT;            // per wavefront: [al2 | bs2 | w], 32 floats each
  static constexpr int ADW = 3 * CQ * 4;
  static constexpr int TOTAL = AD + WAVES * ADW;
  static constexpr int BCI = 2 * BT / 1024 / WAVES;  // 1 KB pieces of B and C per wavefront
  static constexpr int LDC = 2 + BCI + 1;        // vector-memory ops a wavefront issues per chunk load
  static constexpr int STC = 2;                  // ... per chunk of y it stores
  static constexpr int BLOCKS_PER_CU = (160 * 1024) / TOTAL;
  static constexpr int WAVES_PER_SIMD = BLOCKS_PER_CU * WAVES / 4;
  static_assert(BCI * WAVES * 1024 == 2 * BT, "B and C split evenly over the wavefronts");
  static_assert(32 * HPB <= 64 * WAVES, "dt pieces");
  static constexpr int SVC = N / 16;             // ... per saved chunk-start state
  static_assert(R >= 3 && (R - 2) * (LDC + STC + SVC) <= 47, "wait counts");
  static_assert(BLOCKS_PER_CU >= 1 && WAVES_PER_SIMD >= 2, "occupancy");
};

template <int N, int HPB, int R, bool SAVE>
__global__ __launch_bounds__((FusedCfg<N, HPB, R>::THREADS), (FusedCfg<N, HPB, R>::WAVES_PER_SIMD))
void k_ssd_fused(
    const uint16_t *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
    const float *__restrict__ h0, const int32_t *__restrict__ cu, int64_t L, int64_t T, int rows,
    int H, int G, uint16_t *__restrict__ y, float *__restrict__ hfin,
    uint16_t *__restrict__ hsave) {
  using F = FusedCfg<N, HPB, R>;
  constexpr int P = F::P, CQ = F::CQ;
  constexpr int NT = N / 16;   // state tiles per p-tile (over n)
  constexpr int KQ = N / 32;   // K steps over n
  constexpr int NCB = N / 8;   // 16-byte chunks per B / C row
  constexpr int XH = F::XH, BT = F::BT, DW = F::DW, OX = F::OX, OB = F::OB, OC = F::OC, OD = F::OD;
  constexpr int SLOT = F::SLOT, AD = F::AD, ADW = F::ADW, BCI = F::BCI, LDC = F::LDC, STC = F::STC,
                SVC = F::SVC;
  __shared__ __align__(16) unsigned char smem[F::TOTAL];

  int s, hb;
  xcd_chunk_head(H / HPB, s, hb);
  if (s >= rows) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int hh = wave >> 1, ph = wave & 1;
  const int h0b = HPB * hb;  // the block's first head
  const int h = h0b + hh;
  const int g = h0b / (H / G);
  int64_t tb, len;
  seq_range(cu, s, L, T, tb, len);
  const int64_t sh = (int64_t)s * H + h;
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const float Ah = A[h];
  const float Dh = Dv ? Dv[h] : 0.f;
  float *adw = reinterpret_cast<float *>(smem + AD + wave * ADW);

  // state h^T: hst[pt][j] holds column p = 32 ph + 16 pt + c16 and rows
  // n = nrow(j) + r, nrow(j) = 32 (j/2) + 8 g4 + 4 (j%2): tiles 2q and 2q+1
  // together give lane group g4 the 8 consecutive n = 32q + 8 g4 + 0..7, so a
  // K step of the inter term reads its C operand as one 16-byte piece
  auto nrow = [&](int j) { return 32 * (j >> 1) + 8 * g4 + 4 * (j & 1); };
  f32x4 hst[2][NT];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    const int64_t prow = (sh * P + 32 * ph + 16 * pt + c16) * N;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      hst[pt][j] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + prow + nrow(j)) : f32x4{};
  }
  const int nck = static_cast<int>((len + CQ - 1) / CQ);
  const int64_t pbase = SAVE ? pair_base64(cu, s, L, T) : 0;
  // The registers hold S = h / 2^lam: the decay of a chunk goes into lam
  // (wave-uniform) instead of into 2 N/16 x 4 multiplies a lane; S is
  // rescaled only when lam drops below -32, or before a chunk whose own
  // decay exceeds 2^-40 (there the exact per-chunk form is used).
  float lam = 0.f;

  // chunk k's loads into ring slot sl: LDC vector-memory ops per wavefront.
  // Each load is a wave-uniform base (the chunk's first row) plus a per-lane
  // byte offset fixed for the whole sequence; only a partial last chunk
  // recomputes the offsets with its rows clamped.
  uint32_t xoff[2], bcoff[BCI], dtoff;
  auto lane_offsets = [&](int last) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // rows 16 ph .. 16 ph + 15 of head hh's x, 8 chunks each
      const int m = i * 64 + lane, r = 16 * ph + (m >> 3), cc = (m & 7) ^ rot_swz<8>(r);
      xoff[i] = static_cast<uint32_t>((min(r, last) * ldx + (int64_t)h * P + 8 * cc) * 2);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {  // B and C pieces
      const int u = wave * BCI + i, pi = u % (BT / 1024);
      const int m = pi * 64 + lane, r = m / NCB, cc = (m % NCB) ^ rot_swz<NCB>(r);
      bcoff[i] = static_cast<uint32_t>((min(r, last) * ldb + (int64_t)g * N + 8 * cc) * 2);
    }
    // dt of the block's heads: entry e = token * HPB + head, 64 entries a
    // wavefront (past the last entry every lane reads that one)
    const int e = min(wave * 64 + lane, CQ * HPB - 1);
    dtoff = static_cast<uint32_t>((min(e / HPB, last) * H + h0b + e % HPB) * 4);
  };
  lane_offsets(CQ - 1);
  auto issue = [&](int k, int sl) {
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;
    if (last < CQ - 1) lane_offsets(last);
    const uint32_t base = lds_off(smem) + sl * SLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma_lds16_sb(xoff[i], x + t0 * ldx, base + OX + hh * XH + 16 * ph * 128 + i * 1024);
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int u = wave * BCI + i, tile = u / (BT / 1024), pi = u % (BT / 1024);
      dma_lds16_sb(bcoff[i], (tile ? Cm : Bm) + t0 * ldb, base + (tile ? OC : OB) + pi * 1024);
    }
    dma_lds4_sb(dtoff, dt + t0 * H, base + OD + wave * DW);
  };
  // rows 16 ph .. 16 ph + 15 of head hh's y of chunk k (staged in slot sl): STC stores
  auto store_y = [&](int k, int sl) {
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int rem = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ));
    const unsigned char *ys = smem + sl * SLOT + OX + hh * XH;
    u32x4 v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = i * 64 + lane, r = 16 * ph + (m >> 3), cc = m & 7;
      v[i] = *reinterpret_cast<const u32x4 *>(ys + r * 128 + ((cc ^ rot_swz<8>(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = i * 64 + lane, r = 16 * ph + (m >> 3), cc = m & 7;
      if (r < rem) *reinterpret_cast<u32x4 *>(y + (t0 + r) * ldx + (int64_t)h * P + 8 * cc) = v[i];
    }
  };
  // row operand of a B or C tile in the state's K order: K step q gives lane
  // group g4 n = 32q + 8 g4 + {0..7}, one 16-byte chunk
  auto row_op = [&](const unsigned char *tile, int row, int q) {
    return *reinterpret_cast<const u32x4 *>(tile + row * (N * 2) + (((4 * q + g4) ^ rot_swz<NCB>(row)) << 4));
  };
  // B^T operand of state tile j: transposing read of token rows row0 + {0..3};
  // lane (c16, g4) receives column nrow-order n = 32 (j/2) + 8 (c16/4) +
  // 4 (j%2) + c16 % 4 (each 4-lane group addresses its own 4-column piece)
  auto trb = [&](const unsigned char *tile, int row0, int j) {
    const int row = row0 + (c16 >> 2), col = 32 * (j >> 1) + 8 * (c16 & 3) + 4 * (j & 1);
    const int cc = (col >> 3) ^ rot_swz<NCB>(row);
    return lds_read_tr16(tile + row * (N * 2) + (cc << 4) + (col & 7) * 2);
  };
  // transposing read of 4 token rows row0 + {0..3} at column col0 + c16 of a
  // row-major tile (ncc chunks a row, row bytes rb)
  auto tr4 = [&](const unsigned char *tile, int rb, int ncc, int row0, int col0) {
    const int row = row0 + (c16 >> 2), col = col0 + 4 * (c16 & 3);
    const int cc = (col >> 3) ^ rot_swz<8>(row);
    return lds_read_tr16(tile + row * rb + (cc << 4) + (col & 7) * 2);
  };

  constexpr int D = R - 1;  // chunks in flight ahead of the one being computed
#pragma unroll
  for (int c = 0; c < D; ++c)
    if (c < nck) issue(c, c);
  int sl = 0;
#pragma unroll 1
  for (int k = 0; k < nck; ++k) {
    // chunk k has landed once at most the ops this wavefront issued after its
    // loads are pending: loads of later chunks (prologue, then one chunk per
    // iteration) and the y stores of the iterations in between
    // (and, when saving, the state stores of the even ones: SVC each)
    {
      int n = k < D ? (min(D, nck) - 1 - k) * LDC : 0;
      for (int j = k < D ? 0 : k - D + 1; j < k; ++j)
        n += (SAVE && !(j & 1) ? SVC : 0) + (j >= 1 ? STC : 0) + (j + D < nck ? LDC : 0);
      wait_vmcnt_dyn(n);
    }
    __syncthreads();  // every wavefront's share of chunk k is in; chunk k-1 is done everywhere
    if (SAVE && !(k & 1)) {  // the state entering the 64-token pair, h = S 2^lam, rounded to bf16
      const float e = exp2_fast(lam);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        u32x4 pk[KQ];  // row p = 32 ph + 16 pt + c16, n = 32 q + 8 g4 + 0..7
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
          const f32x4 u = hst[pt][2 * q] * e, v = hst[pt][2 * q + 1] * e;
          pk[q] = u32x4{pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                        pack_bf16x2(v.z, v.w)};
        }
        store_rows128(hsave + ((pbase + (k >> 1)) * H + h) * (int64_t)(P * N) +
                          (int64_t)(32 * ph + 16 * pt) * N,
                      N, pk, c16, g4);
      }
    }
    const int slp = sl == 0 ? R - 1 : sl - 1;  // slot of chunk k-1, and of chunk k+D
    if (k >= 1) store_y(k - 1, slp);
    if (k + D < nck) issue(k + D, slp);

    unsigned char *xh = smem + sl * SLOT + OX + hh * XH;  // head hh's x tile (this wavefront: columns 32 ph ..)
    const unsigned char *bs = smem + sl * SLOT + OB;
    const unsigned char *cs = smem + sl * SLOT + OC;
    const float *dts = reinterpret_cast<const float *>(smem + sl * SLOT + OD);
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;

    // cumulative decay (lanes l and 32 + l hold token l) and per-token tables
    const int tl = lane & 31;
    const float dtv = tl <= last ? dts[tl * HPB + hh] : 0.f;
    const float a = scan32(dtv * Ah);
    const float alast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 31));
    const float a2last = alast * kLog2e;
    const bool steep = a2last < -40.f;          // exact per-chunk form for this chunk
    const float wshift = steep ? a2last : -lam;  // log2 of w_s / (dt_s exp(-a_s))
    if (lane < 32) {
      const float al = a * kLog2e;
      const float bs = __builtin_amdgcn_logf(dtv) - al;
      adw[tl] = al;                              // log2 exp(a_l)
      adw[CQ + tl] = bs;                         // log2(dt_s exp(-a_s))
      adw[2 * CQ + tl] = exp2_fast(bs + wshift);  // the state update's token weight
    }
    wave_sync();

    // 1. inter term
    u32x4 cop[2][KQ];
#pragma unroll
    for (int lt = 0; lt < 2; ++lt)
#pragma unroll
      for (int q = 0; q < KQ; ++q) cop[lt][q] = row_op(cs, 16 * lt + c16, q);
    f32x4 ya[2][2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = f32x4{};
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const f32x4 u = hst[pt][2 * q], v = hst[pt][2 * q + 1];
        const u32x4 sop{pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                        pack_bf16x2(v.z, v.w)};
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = mfma16(sop, cop[lt][q], ya[pt][lt]);
      }
    }
    const float al0 = adw[c16], al1 = adw[16 + c16];
    const float f0 = exp2_fast(al0 + lam), f1 = exp2_fast(al1 + lam);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      ya[pt][0] *= f0;
      ya[pt][1] *= f1;
    }

    // 2. intra term: Z^T tiles (s-block, l-block) = (0,0), (1,1), (0,1)
    u32x4 gop[2];
    {
      f32x4 z00{}, z11{}, z01{};
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
        const u32x4 b0 = row_op(bs, c16, q), b1 = row_op(bs, 16 + c16, q);
        z00 = mfma16(b0, cop[0][q], z00);
        z01 = mfma16(b0, cop[1][q], z01);
        z11 = mfma16(b1, cop[1][q], z11);
      }
      // lane holds s = 16 sb + 4 g4 + r, l = 16 lb + c16
      const f32x4 bs0 = *reinterpret_cast<const f32x4 *>(adw + CQ + 4 * g4);
      const f32x4 bs1 = *reinterpret_cast<const f32x4 *>(adw + CQ + 16 + 4 * g4);
      float g00[4], g11[4], g01[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float keep = 4 * g4 + r <= c16 ? 1.f : 0.f;
        // for s > l the exponent may be large; min() keeps it finite so the
        // 0 mask wins
        g00[r] = z00[r] * (exp2_fast(fminf(al0 + bs0[r], 64.f)) * keep);
        g11[r] = z11[r] * (exp2_fast(fminf(al1 + bs1[r], 64.f)) * keep);
        g01[r] = z01[r] * exp2_fast(al1 + bs0[r]);
      }
      gop[0] = u32x4{pack_bf16x2(g00[0], g00[1]), pack_bf16x2(g00[2], g00[3]), 0u, 0u};
      gop[1] = u32x4{pack_bf16x2(g01[0], g01[1]), pack_bf16x2(g01[2], g01[3]),
                     pack_bf16x2(g11[0], g11[1]), pack_bf16x2(g11[2], g11[3])};
    }
    // X^T in the same token order: s = 4 g4 + {0..3}, 16 + 4 g4 + {0..3}
    u32x4 xop[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const u32x2 t0 = tr4(xh, 128, 8, 4 * g4, 32 * ph + 16 * pt);
      const u32x2 t1 = tr4(xh, 128, 8, 16 + 4 * g4, 32 * ph + 16 * pt);
      xop[pt] = u32x4{t0.x, t0.y, t1.x, t1.y};
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = mfma16(xop[pt], gop[lt], ya[pt][lt]);
    }
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {  // D x: rows p = 16 pt + 4 g4 + r of token l
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) {
        const int l = 16 * lt + c16, col = 32 * ph + 16 * pt + 4 * g4;
        const u32x2 v = *reinterpret_cast<const u32x2 *>(
            xh + l * 128 + (((col >> 3) ^ rot_swz<8>(l)) << 4) + (col & 7) * 2);
        ya[pt][lt].x += Dh * bf16lo(v.x);
        ya[pt][lt].y += Dh * bf16hi(v.x);
        ya[pt][lt].z += Dh * bf16lo(v.y);
        ya[pt][lt].w += Dh * bf16hi(v.y);
      }
    }

    // 3. state: h = exp(a_last) h + B^T (w x), as S = h / 2^lam: normally
    // lam += a_last log2(e) and S += B^T (w' x) with w'_s = w_s / 2^lam_new;
    // for a steep chunk S is first turned into exp(a_last) h and lam = 0
    {
      if (steep) {
        const float e = exp2_fast(lam + a2last);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int j = 0; j < NT; ++j) hst[pt][j] *= e;
      }
      lam = steep ? 0.f : lam + a2last;
      const f32x4 w0 = *reinterpret_cast<const f32x4 *>(adw + 2 * CQ + 4 * g4);
      const f32x4 w1 = *reinterpret_cast<const f32x4 *>(adw + 2 * CQ + 16 + 4 * g4);
      u32x4 xw[2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        const u32x4 q = xop[pt];
        xw[pt] = u32x4{pack_bf16x2(bf16lo(q.x) * w0.x, bf16hi(q.x) * w0.y),
                       pack_bf16x2(bf16lo(q.y) * w0.z, bf16hi(q.y) * w0.w),
                       pack_bf16x2(bf16lo(q.z) * w1.x, bf16hi(q.z) * w1.y),
                       pack_bf16x2(bf16lo(q.w) * w1.z, bf16hi(q.w) * w1.w)};
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x2 t0 = trb(bs, 4 * g4, j), t1 = trb(bs, 16 + 4 * g4, j);
        const u32x4 bt{t0.x, t0.y, t1.x, t1.y};
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) hst[pt][j] = mfma16(bt, xw[pt], hst[pt][j]);
      }
      if (lam < -32.f) {
        const float e = exp2_fast(lam);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
          for (int j = 0; j < NT; ++j) hst[pt][j] *= e;
        lam = 0.f;
      }
    }

    // y staged (bf16) over this wavefront's columns of the x tile, now fully read
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) {
        const int l = 16 * lt + c16, col = 32 * ph + 16 * pt + 4 * g4;
        const u32x2 o{pack_bf16x2(ya[pt][lt].x, ya[pt][lt].y), pack_bf16x2(ya[pt][lt].z, ya[pt][lt].w)};
        *reinterpret_cast<u32x2 *>(xh + l * 128 + (((col >> 3) ^ rot_swz<8>(l)) << 4) + (col & 7) * 2) = o;
      }
    }
    sl = sl == R - 1 ? 0 : sl + 1;
  }
  if (nck > 0) {
    __syncthreads();  // both halves of the last chunk's y are staged
    store_y(nck - 1, (nck - 1) % R);
  }
  if (hfin) {
    const float e = exp2_fast(lam);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int64_t prow = (sh * P + 32 * ph + 16 * pt + c16) * N;
#pragma unroll
      for (int j = 0; j < NT; ++j) *reinterpret_cast<f32x4 *>(hfin + prow + nrow(j)) = hst[pt][j] * e;
    }
  }
}

}  // namespace

bool fused_supported(int H, int P, int N, int G) {
  return P == 64 && (N == 64 || N == 128) && (H / G) % 2 == 0;
}

namespace {
template <int N, int HPB, int R, bool SAVE>
void launch_fused_t(const uint16_t *x, const float *dt, const float *A, const uint16_t *B,
                    const uint16_t *C, const float *D, const float *h0, const int32_t *cu, int64_t L,
                    int64_t T, int rows, int H, int G, uint16_t *y, float *hfin, uint16_t *hsave,
                    hipStream_t stream) {
  hipLaunchKernelGGL((k_ssd_fused<N, HPB, R, SAVE>), dim3(xcd_grid(rows, H / HPB)),
                     dim3(FusedCfg<N, HPB, R>::THREADS), 0, stream, x, dt, A, B, C, D, h0, cu, L, T,
                     rows, H, G, y, hfin, hsave);
}
}  // namespace

hipError_t launch_fused(const void *x, const float *dt, const float *A, const void *B, const void *C,
                        const float *D, const float *h0, const int32_t *cu, int64_t L, int64_t T,
                        int rows, int H, int P, int N, int G, void *y, float *hfin, void *hsave,
                        hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!fused_supported(H, P, N, G)) return hipErrorInvalidValue;
  const uint16_t *xi = static_cast<const uint16_t *>(x);
  const uint16_t *bi = static_cast<const uint16_t *>(B);
  const uint16_t *ci = static_cast<const uint16_t *>(C);
  uint16_t *yo = static_cast<uint16_t *>(y);
  uint16_t *hs = static_cast<uint16_t *>(hsave);
  if (N == 64) {
    if (hs) launch_fused_t<64, 2, 3, true>(xi, dt, A, bi, ci, D, h0, cu, L, T, rows, H, G, yo, hfin, hs, stream);
    else launch_fused_t<64, 2, 3, false>(xi, dt, A, bi, ci, D, h0, cu, L, T, rows, H, G, yo, hfin, hs, stream);
  } else {
    if (hs) launch_fused_t<128, 2, 3, true>(xi, dt, A, bi, ci, D, h0, cu, L, T, rows, H, G, yo, hfin, hs, stream);
    else launch_fused_t<128, 2, 3, false>(xi, dt, A, bi, ci, D, h0, cu, L, T, rows, H, G, yo, hfin, hs, stream);
  }
  return hipGetLastError();
}

}  // namespace ssd
