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
//      applied per element as exp(a_l) times a per-token table of
//      dt_s exp(-a_s) (per element in the log2 domain for a chunk that decays
//      below 2^-96) and the tile above the diagonal masked, then Y^T += X^T G^T
//      with the accumulators as B-operands and X^T from transposing LDS reads
//      in the matching token order; plus D x as X^T diag(D), D split into two
//      bf16 parts;
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

// Geometry of one kernel instance: N state size, HPB heads per block, PW
// state rows p per wavefront (32 or 16: 64 / PW wavefronts per head), R ring
// slots; ST: the state-only pass (no C, no y).
template <int N, int HPB, int PW, int R, bool ST = false>
struct FusedCfg {
  static constexpr int P = 64, CQ = 32, WPH = P / PW, WAVES = WPH * HPB, THREADS = 64 * WAVES;
  static constexpr int PT = PW / 16;             // 16-column state tiles per wavefront
  static constexpr int XR = CQ / WPH;            // x / y rows of a chunk a wavefront moves
  static constexpr int XI = XR * P * 2 / 1024;   // ... in 1 KB direct-to-LDS loads / row stores
  static constexpr int XH = CQ * P * 2;          // x of one head and chunk: 32 rows x 128 B
  static constexpr int BT = CQ * N * 2;          // B (or C) of a chunk
  static constexpr int DTP = (CQ * HPB + 63) / 64;  // 64-entry dt pieces of a chunk
  static constexpr int DW = 64 * 4;              // one dt piece (wavefront i < DTP loads piece i)
  static constexpr int OX = 0, OB = HPB * XH, OC = OB + BT, OD = OC + (ST ? 0 : BT);
  static constexpr int SLOT = OD + DTP * DW;
  static constexpr int AD = R * SLOT;            // per wavefront: [al2 | bs2 | w | vs], 32 floats each
  static constexpr int ADW = 4 * CQ * 4;
  static constexpr int TOTAL = AD + WAVES * ADW;
  static constexpr int NBC = ST ? 1 : 2;         // B (and C) tiles a chunk loads
  static constexpr int NPC = NBC * BT / 1024;    // 1 KB pieces of B and C
  static constexpr int BCI = (NPC + WAVES - 1) / WAVES;  // ... at most per wavefront (piece
                                                 // u goes to wavefront u % WAVES)
  static constexpr int LDC = XI + BCI;           // vector-memory ops a wavefront issues per chunk
                                                 // load, at most (+1 with a dt piece)
  static constexpr int STC = ST ? 0 : XI;        // ... per chunk of y it stores
  static constexpr int BLOCKS_PER_CU = (160 * 1024) / TOTAL;
  // waves a SIMD must hold for BLOCKS_PER_CU blocks (at most 3: the kernel
  // needs ~140-200 VGPRs, so more would spill)
  static constexpr int WAVES_PER_SIMD_LDS = (BLOCKS_PER_CU * WAVES + 3) / 4;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_LDS < 3 ? WAVES_PER_SIMD_LDS : 3;
  static_assert(PW == 16 || PW == 32, "state rows per wavefront");
  static_assert(XI >= 1 && XI * 1024 == XR * P * 2, "x rows in 1 KB pieces");
  static_assert(BCI >= 1 && NPC * 1024 == NBC * BT, "B and C in 1 KB pieces");
  static_assert(DTP <= WAVES, "a wavefront per dt piece");
  static constexpr int SVC = PT * N / 32;        // ... per saved chunk-start state
  static_assert(R >= 2 && (R - 2) * (LDC + 1 + STC + SVC) <= 47, "wait counts");
  static_assert(BLOCKS_PER_CU >= 1 && WAVES_PER_SIMD >= 1, "occupancy");
};

// What a launch walks: rows of tokens (sequences, or segments of them), each
// from a given state.
struct FusedArgs {
  const uint16_t *x;
  const float *dt, *A;
  const uint16_t *B, *C;
  const float *D;
  const float *h0;       // initial state of each sequence [rows0, H, P, N], or NULL
  const int32_t *cu;     // packed sequences (then S = L, nsr = 1), or NULL
  int64_t L, T;          // tokens per sequence (fixed length), total tokens
  int64_t S;             // tokens per segment (L when not split)
  int nsr;               // segments of a sequence this launch walks
  int rows;              // blocks' rows: sequences x nsr
  int H, G, hr;
  uint16_t *y;
  float *hfin;           // final state of each sequence (last segment), or NULL
  uint16_t *hsave;       // SAVE: bf16 state entering every 64-token pair
  const float *hin;      // split forward: the state entering each segment,
                         // [seq][nsr][H][P][N] (then h0 is not read)
  float *sseg;           // state-only pass: segment j's end state from 0 into
                         // [seq][j + 1] of a [seq][nsr + 1][H][P][N] buffer ...
  float *lseg;           // ... and its total log2 decay into [seq][nsr][H]
};

enum FusedMode { kFwd = 0, kFwdSave = 1, kState = 2 };

template <int N, int HPB, int PW, int R, int MODE>
__global__ __launch_bounds__((FusedCfg<N, HPB, PW, R, MODE == kState>::THREADS),
                             (FusedCfg<N, HPB, PW, R, MODE == kState>::WAVES_PER_SIMD))
void k_ssd_fused(const FusedArgs args) {
  constexpr bool SAVE = MODE == kFwdSave, ST = MODE == kState;
  using F = FusedCfg<N, HPB, PW, R, ST>;
  const uint16_t *__restrict__ x = args.x;
  const float *__restrict__ dt = args.dt;
  const float *__restrict__ A = args.A;
  const uint16_t *__restrict__ Bm = args.B;
  const uint16_t *__restrict__ Cm = args.C;
  const float *__restrict__ Dv = args.D;
  const int32_t *__restrict__ cu = args.cu;
  const int64_t L = args.L, T = args.T;
  const int H = args.H, G = args.G, hr = args.hr;
  uint16_t *__restrict__ y = args.y;
  uint16_t *__restrict__ hsave = args.hsave;
  constexpr int P = F::P, CQ = F::CQ, WPH = F::WPH, PT = F::PT, XR = F::XR, XI = F::XI;
  constexpr int NT = N / 16;   // state tiles per p-tile (over n)
  constexpr int KQ = N / 32;   // K steps over n
  constexpr int NCB = N / 8;   // 16-byte chunks per B / C row
  constexpr int XH = F::XH, BT = F::BT, DW = F::DW, OX = F::OX, OB = F::OB, OC = F::OC, OD = F::OD;
  constexpr int SLOT = F::SLOT, AD = F::AD, ADW = F::ADW, BCI = F::BCI, STC = F::STC, WAVES = F::WAVES,
                SVC = F::SVC;
  __shared__ __align__(16) unsigned char smem[F::TOTAL];

  int s, hb;
  xcd_chunk_head(H / HPB, s, hb);
  if (s >= args.rows) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int hh = wave / WPH, pq = wave % WPH;  // head of the block, state-row slice
  const int p0 = PW * pq;                       // the slice's first row p
  const int h0b = HPB * hb;  // the block's first head
  const int h = h0b + hh;
  const int g = h0b / (H / G);
  // row s: segment seg of sequence sq (packed sequences are never split)
  int64_t tb, len;
  int sq = s, seg = 0;
  if (cu) {
    seq_range(cu, s, L, T, tb, len);
  } else {
    sq = s / args.nsr;
    seg = s - sq * args.nsr;
    tb = (int64_t)sq * L + (int64_t)seg * args.S;
    len = min(args.S, L - (int64_t)seg * args.S);
  }
  constexpr int64_t PN = (int64_t)P * N;
  // the state entering the row, and where the state leaving it goes
  const float *h0p;
  float *hfp;
  if (ST) {
    h0p = nullptr;
    hfp = args.sseg + (((int64_t)sq * (args.nsr + 1) + seg + 1) * H + h) * PN;
  } else {
    h0p = args.hin ? args.hin + ((int64_t)s * H + h) * PN
                   : args.h0 ? args.h0 + ((int64_t)sq * H + h) * PN : nullptr;
    hfp = seg == args.nsr - 1 && args.hfin ? args.hfin + ((int64_t)sq * H + h) * PN : nullptr;
  }
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const int Hd = H / hr;  // heads of dt, A and D: kernel head h takes those of h / hr
  const float Ah = A[h / hr];
  const float Dh = Dv ? Dv[h / hr] : 0.f;
  float *adw = reinterpret_cast<float *>(smem + AD + wave * ADW);

  // state h^T: hst[pt][j] holds column p = p0 + 16 pt + c16 and rows
  // n = nrow(j) + r, nrow(j) = 32 (j/2) + 8 g4 + 4 (j%2): tiles 2q and 2q+1
  // together give lane group g4 the 8 consecutive n = 32q + 8 g4 + 0..7, so a
  // K step of the inter term reads its C operand as one 16-byte piece
  auto nrow = [&](int j) { return 32 * (j >> 1) + 8 * g4 + 4 * (j & 1); };
  f32x4 hst[PT][NT];
#pragma unroll
  for (int pt = 0; pt < PT; ++pt) {
    const int64_t prow = (int64_t)(p0 + 16 * pt + c16) * N;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      hst[pt][j] = h0p ? *reinterpret_cast<const f32x4 *>(h0p + prow + nrow(j)) : f32x4{};
  }
  const int nck = static_cast<int>((len + CQ - 1) / CQ);
  // the row's first 64-token pair in the saved states' layout: a segment of a
  // split sequence starts seg S / 64 pairs into its sequence (S a multiple of
  // 64 when saving)
  const int64_t pbase = !SAVE ? 0
                        : cu  ? pair_base64(cu, s, L, T)
                              : (int64_t)sq * ((L + 63) / 64) + (int64_t)seg * (args.S / 64);
  // The registers hold S = h / 2^lam: the decay of a chunk goes into lam
  // (wave-uniform) instead of into 2 N/16 x 4 multiplies a lane; S is
  // rescaled only when lam drops below -32, or before a chunk whose own
  // decay exceeds 2^-40 (there the exact per-chunk form is used).
  float lam = 0.f;
  float lsum = 0.f;  // state-only pass: the row's total log2 decay

  // a chunk's loads into its ring slot: LDC vector-memory ops per wavefront.
  // Each load is a wave-uniform base (the chunk's first row) plus a per-lane
  // byte offset fixed for the whole sequence; only a partial last chunk
  // recomputes the offsets with its rows clamped.
  uint32_t xoff[XI], bcoff[BCI], dtoff;
  auto lane_offsets = [&](int last) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {  // rows XR pq .. XR pq + XR - 1 of head hh's x, 8 chunks each
      const int m = i * 64 + lane, r = XR * pq + (m >> 3), cc = (m & 7) ^ rot_swz<8>(r);
      xoff[i] = static_cast<uint32_t>((min(r, last) * ldx + (int64_t)h * P + 8 * cc) * 2);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {  // B and C pieces
      const int u = wave + i * WAVES, pi = u % (BT / 1024);
      const int m = pi * 64 + lane, r = m / NCB, cc = (m % NCB) ^ rot_swz<NCB>(r);
      bcoff[i] = static_cast<uint32_t>((min(r, last) * ldb + (int64_t)g * N + 8 * cc) * 2);
    }
    // dt of the block's heads: entry e = token * HPB + head, 64-entry pieces
    // (past the last entry every lane reads that one)
    const int e = min(wave * 64 + lane, CQ * HPB - 1);
    dtoff = static_cast<uint32_t>((min(e / HPB, last) * Hd + (h0b + e % HPB) / hr) * 4);
  };
  lane_offsets(CQ - 1);
  const uint32_t smem0 = __builtin_amdgcn_readfirstlane(lds_off(smem));
  // y row pieces this wavefront stores: byte offsets from a chunk's first row
  uint32_t yoff[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int m = i * 64 + lane, r = XR * pq + (m >> 3), cc = m & 7;
    yoff[i] = static_cast<uint32_t>((r * ldx + (int64_t)h * P + 8 * cc) * 2);
  }
  // Chunks are loaded and their y stored in order, so each side keeps running
  // wave-uniform pointers that advance by one chunk per call; only the last
  // chunk can be partial (lastlen tokens).
  const int lastlen = static_cast<int>(len - (int64_t)(nck - 1) * CQ);
  const uint16_t *xg = x + tb * ldx, *bg = Bm + tb * ldb, *cg = Cm + tb * ldb;
  const float *dg = dt + tb * Hd;
  uint16_t *yg = y + tb * ldx;
  // this wavefront's LDS destinations within a slot
  const uint32_t ldsx = smem0 + OX + hh * XH + XR * pq * 128;
  auto issue = [&](int k, uint32_t soff) {
    if (k == nck - 1 && lastlen < CQ) lane_offsets(lastlen - 1);
#pragma unroll
    for (int i = 0; i < XI; ++i) dma_lds16_sb(xoff[i], xg, ldsx + soff + i * 1024);
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int u = wave + i * WAVES, tile = u / (BT / 1024), pi = u % (BT / 1024);
      if (F::NPC % WAVES != 0 && u >= F::NPC) break;  // wave-uniform
      dma_lds16_sb(bcoff[i], tile ? cg : bg, smem0 + soff + (tile ? OC : OB) + pi * 1024);
    }
    if (wave < F::DTP) dma_lds4_sb(dtoff, dg, smem0 + soff + OD + wave * DW);
    xg += CQ * ldx;
    bg += CQ * ldb;
    cg += CQ * ldb;
    dg += CQ * Hd;
  };
  // rows XR pq .. XR pq + XR - 1 of head hh's y of chunk k (staged in the
  // slot at byte offset soff): STC stores
  auto store_y = [&](int k, uint32_t soff) {
    const int rem = k == nck - 1 ? lastlen : CQ;
    const unsigned char *ys = smem + soff + OX + hh * XH;
    u32x4 v[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int m = i * 64 + lane, r = XR * pq + (m >> 3), cc = m & 7;
      v[i] = *reinterpret_cast<const u32x4 *>(ys + r * 128 + ((cc ^ rot_swz<8>(r)) << 4));
    }
    unsigned char *yb = reinterpret_cast<unsigned char *>(yg);  // wave-uniform
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = XR * pq + ((i * 64 + lane) >> 3);
      if (r < rem) *reinterpret_cast<u32x4 *>(yb + yoff[i]) = v[i];
    }
    yg += CQ * ldx;
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
  // vector-memory ops this wavefront issues per chunk load: x rows, its B/C
  // pieces, and dt piece `wave` for wavefronts below DTP
  const int ldc = XI + (F::NPC - wave + WAVES - 1) / WAVES + (wave < F::DTP ? 1 : 0);
  // ... the same as constants, where every wavefront has NPC / WAVES B/C pieces
  constexpr bool EVEN_BC = F::NPC % WAVES == 0;
  constexpr int LD0 = XI + F::NPC / WAVES, LD1 = LD0 + 1;  // without / with a dt piece
  constexpr int SLOTS = R * SLOT;
  // wait counts known at compile time in the steady state (with saving, only
  // for at most two slots in flight, where the parity of k - 1 decides)
  constexpr bool STATIC_WAIT = EVEN_BC && (D <= 2 || !SAVE);
#pragma unroll
  for (int c = 0; c < D; ++c)
    if (c < nck) issue(c, c * SLOT);
  uint32_t soff = 0;  // byte offset of chunk k's slot
#pragma unroll 1
  for (int k = 0; k < nck; ++k) {
    // chunk k has landed once at most the ops this wavefront issued after its
    // loads are pending: loads of later chunks (prologue, then one chunk per
    // iteration) and the y stores of the iterations in between
    // (and, when saving, the state stores of the even ones: SVC each)
    if (STATIC_WAIT && k >= D && k + D <= nck) {
      // steady state: the last D - 1 iterations each issued STC stores and
      // one chunk load (and, when saving, iteration k - 1 its state if even)
      const bool dtw = wave < F::DTP, sv = SAVE && D == 2 && !((k - 1) & 1);
      if (dtw) {
        if (sv) wait_vmcnt<(D - 1) * (STC + LD1) + SVC>();
        else wait_vmcnt<(D - 1) * (STC + LD1)>();
      } else {
        if (sv) wait_vmcnt<(D - 1) * (STC + LD0) + SVC>();
        else wait_vmcnt<(D - 1) * (STC + LD0)>();
      }
    } else {
      int n = k < D ? (min(D, nck) - 1 - k) * ldc : 0;
      for (int j = k < D ? 0 : k - D + 1; j < k; ++j)
        n += (SAVE && !(j & 1) ? SVC : 0) + (j >= 1 ? STC : 0) + (j + D < nck ? ldc : 0);
      wait_vmcnt_dyn(n);
    }
    wait_lgkmcnt0();  // this wavefront's y staging of chunk k-1 is in LDS
    __syncthreads();  // every wavefront's share of chunk k is in; chunk k-1 is done everywhere
    if (SAVE && !(k & 1)) {  // the state entering the 64-token pair, h = S 2^lam, rounded to bf16
      const float e = exp2_fast(lam);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        u32x4 pk[KQ];  // row p = p0 + 16 pt + c16, n = 32 q + 8 g4 + 0..7
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
          const f32x4 u = hst[pt][2 * q] * e, v = hst[pt][2 * q + 1] * e;
          pk[q] = u32x4{pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                        pack_bf16x2(v.z, v.w)};
        }
        store_rows128(hsave + ((pbase + (k >> 1)) * H + h) * (int64_t)(P * N) +
                          (int64_t)(p0 + 16 * pt) * N,
                      N, pk, c16, g4);
      }
    }
    const uint32_t sprev = soff == 0 ? SLOTS - SLOT : soff - SLOT;  // chunk k-1's slot, and k+D's
    if (!ST && k >= 1) store_y(k - 1, sprev);
    if (k + D < nck) issue(k + D, sprev);

    unsigned char *xh = smem + soff + OX + hh * XH;  // head hh's x tile (this wavefront: columns p0 ..)
    const unsigned char *bs = smem + soff + OB;
    const unsigned char *cs = smem + soff + OC;
    const float *dts = reinterpret_cast<const float *>(smem + soff + OD);
    const int last = k == nck - 1 ? lastlen - 1 : CQ - 1;
    // cumulative decay (lanes l and 32 + l hold token l) and per-token tables
    const int tl = lane & 31;
    const float dtv = tl <= last ? dts[tl * HPB + hh] : 0.f;
    const float a = scan32(dtv * Ah);
    const float alast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 31));
    const float a2last = alast * kLog2e;
    const bool steep = a2last < -40.f;          // exact per-chunk state update for this chunk
    const bool gsep = a2last >= -96.f;          // separable intra-chunk decay (see below)
    const float wshift = steep ? a2last : -lam;  // log2 of w_s / (dt_s exp(-a_s))
    if (lane < 32) {
      const float al = a * kLog2e;
      const float bs = __builtin_amdgcn_logf(dtv) - al;
      adw[tl] = al;                              // log2 exp(a_l)
      adw[CQ + tl] = bs;                         // log2(dt_s exp(-a_s))
      adw[2 * CQ + tl] = exp2_fast(bs + wshift);  // the state update's token weight
      // dt_s exp(-a_s) itself, at most dt_s 2^96 where gsep holds
      adw[3 * CQ + tl] = exp2_fast(fminf(bs, 126.f));
    }
    wave_sync();

    // X^T in the token order of the intra term's K steps and of the state
    // update: s = 4 g4 + {0..3}, 16 + 4 g4 + {0..3}
    u32x4 xop[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const u32x2 t0 = tr4(xh, 128, 8, 4 * g4, p0 + 16 * pt);
      const u32x2 t1 = tr4(xh, 128, 8, 16 + 4 * g4, p0 + 16 * pt);
      xop[pt] = u32x4{t0.x, t0.y, t1.x, t1.y};
    }
    f32x4 ya[PT][2];
    if constexpr (!ST) {
      // 1. inter term
      u32x4 cop[2][KQ];
#pragma unroll
      for (int lt = 0; lt < 2; ++lt)
#pragma unroll
        for (int q = 0; q < KQ; ++q) cop[lt][q] = row_op(cs, 16 * lt + c16, q);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = f32x4{};
#pragma unroll
      for (int q = 0; q < KQ; ++q) {
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const f32x4 u = hst[pt][2 * q], v = hst[pt][2 * q + 1];
          const u32x4 sop{pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                          pack_bf16x2(v.z, v.w)};
#pragma unroll
          for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = mfma16(sop, cop[lt][q], ya[pt][lt]);
        }
      }
      const float al0 = adw[c16], al1 = adw[16 + c16];
      // exp(a_l) for the lane's tokens l = c16, 16 + c16
      const float u0 = exp2_fast(al0), u1 = exp2_fast(al1);
      const float el = exp2_fast(lam);
      const float f0 = u0 * el, f1 = u1 * el;
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        ya[pt][0] *= f0;
        ya[pt][1] *= f1;
      }

      // 2. intra term: Z^T tiles (s-block, l-block) = (0,0), (1,1), (0,1);
      // G^T = Z^T exp(a_l - a_s) dt_s on s <= l
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
        float g00[4], g11[4], g01[4];
        if (gsep) {
          // exp(a_l - a_s) dt_s = exp(a_l) (dt_s exp(-a_s)): both factors normal
          // floats when the chunk decays by less than 2^-96 (and their product
          // finite on the masked s > l side too)
          const f32x4 v0 = *reinterpret_cast<const f32x4 *>(adw + 3 * CQ + 4 * g4);
          const f32x4 v1 = *reinterpret_cast<const f32x4 *>(adw + 3 * CQ + 16 + 4 * g4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float keep = 4 * g4 + r <= c16 ? 1.f : 0.f;
            g00[r] = z00[r] * (u0 * v0[r] * keep);
            g11[r] = z11[r] * (u1 * v1[r] * keep);
            g01[r] = z01[r] * (u1 * v0[r]);
          }
        } else {
          const f32x4 bs0 = *reinterpret_cast<const f32x4 *>(adw + CQ + 4 * g4);
          const f32x4 bs1 = *reinterpret_cast<const f32x4 *>(adw + CQ + 16 + 4 * g4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float keep = 4 * g4 + r <= c16 ? 1.f : 0.f;
            // for s > l the exponent may be large; min() keeps it finite so the
            // 0 mask wins
            g00[r] = z00[r] * (exp2_fast(fminf(al0 + bs0[r], 64.f)) * keep);
            g11[r] = z11[r] * (exp2_fast(fminf(al1 + bs1[r], 64.f)) * keep);
            g01[r] = z01[r] * exp2_fast(al1 + bs0[r]);
          }
        }
        gop[0] = u32x4{pack_bf16x2(g00[0], g00[1]), pack_bf16x2(g00[2], g00[3]), 0u, 0u};
        gop[1] = u32x4{pack_bf16x2(g01[0], g01[1]), pack_bf16x2(g01[2], g01[3]),
                       pack_bf16x2(g11[0], g11[1]), pack_bf16x2(g11[2], g11[3])};
      }
#pragma unroll
      for (int pt = 0; pt < PT; ++pt)
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = mfma16(xop[pt], gop[lt], ya[pt][lt]);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {  // D x in fp32: rows p = 16 pt + 4 g4 + r of token l
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
          const int l = 16 * lt + c16, col = p0 + 16 * pt + 4 * g4;
          const u32x2 v = *reinterpret_cast<const u32x2 *>(
              xh + l * 128 + (((col >> 3) ^ rot_swz<8>(l)) << 4) + (col & 7) * 2);
          ya[pt][lt].x += Dh * bf16lo(v.x);
          ya[pt][lt].y += Dh * bf16hi(v.x);
          ya[pt][lt].z += Dh * bf16lo(v.y);
          ya[pt][lt].w += Dh * bf16hi(v.y);
        }
      }

    }

    // 3. state: h = exp(a_last) h + B^T (w x), as S = h / 2^lam: normally
    // lam += a_last log2(e) and S += B^T (w' x) with w'_s = w_s / 2^lam_new;
    // for a steep chunk S is first turned into exp(a_last) h and lam = 0
    {
      if (steep) {
        const float e = exp2_fast(lam + a2last);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int j = 0; j < NT; ++j) hst[pt][j] *= e;
      }
      lam = steep ? 0.f : lam + a2last;
      if (ST) lsum += a2last;
      const f32x4 w0 = *reinterpret_cast<const f32x4 *>(adw + 2 * CQ + 4 * g4);
      const f32x4 w1 = *reinterpret_cast<const f32x4 *>(adw + 2 * CQ + 16 + 4 * g4);
      u32x4 xw[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
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
        for (int pt = 0; pt < PT; ++pt) hst[pt][j] = mfma16(bt, xw[pt], hst[pt][j]);
      }
      if (lam < -32.f) {
        const float e = exp2_fast(lam);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
#pragma unroll
          for (int j = 0; j < NT; ++j) hst[pt][j] *= e;
        lam = 0.f;
      }
    }

    // y staged (bf16) over this wavefront's columns of the x tile, now fully read
#pragma unroll
    for (int pt = 0; pt < (ST ? 0 : PT); ++pt) {
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) {
        const int l = 16 * lt + c16, col = p0 + 16 * pt + 4 * g4;
        const u32x2 o{pack_bf16x2(ya[pt][lt].x, ya[pt][lt].y), pack_bf16x2(ya[pt][lt].z, ya[pt][lt].w)};
        *reinterpret_cast<u32x2 *>(xh + l * 128 + (((col >> 3) ^ rot_swz<8>(l)) << 4) + (col & 7) * 2) = o;
      }
    }
    soff = soff == SLOTS - SLOT ? 0 : soff + SLOT;
  }
  if (!ST && nck > 0) {
    wait_lgkmcnt0();
    __syncthreads();  // every wavefront's part of the last chunk's y is staged
    store_y(nck - 1, ((nck - 1) % R) * SLOT);
  }
  if (hfp) {
    const float e = exp2_fast(lam);
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      const int64_t prow = (int64_t)(p0 + 16 * pt + c16) * N;
#pragma unroll
      for (int j = 0; j < NT; ++j) *reinterpret_cast<f32x4 *>(hfp + prow + nrow(j)) = hst[pt][j] * e;
    }
  }
  if (ST && pq == 0 && lane == 0) args.lseg[(int64_t)s * H + h] = lsum;
}

}  // namespace

bool fused_supported(int H, int P, int N, int G) {
  return P == 64 && (N == 64 || N == 128 || N == 256) && H % G == 0;
}

namespace {
template <int N, int HPB, int PW, int R, int MODE>
void launch_fused_t(const FusedArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((k_ssd_fused<N, HPB, PW, R, MODE>), dim3(xcd_grid(a.rows, a.H / HPB)),
                     dim3(FusedCfg<N, HPB, PW, R, MODE == kState>::THREADS), 0, stream, a);
}

// Instances: two heads a block (four wavefronts of 32 state rows, a three-slot
// ring) where the heads of a group pair up and the (row, head pair) blocks
// fill the GPU, three where they divide by three and those fill it; else one
// head a block (two wavefronts, a two-slot ring, up to three blocks a CU),
// which doubles the blocks of few long sequences.  N = 256 takes one head a
// block in four wavefronts of 16 rows (the state of a wavefront stays at 64
// registers).
template <int N, int MODE>
void launch_fused_n(int hpb, const FusedArgs &a, hipStream_t stream) {
  if constexpr (N == 256) {
    launch_fused_t<N, 1, 16, 2, MODE>(a, stream);
  } else {
    if (hpb == 3) launch_fused_t<N, 3, 32, 3, MODE>(a, stream);
    else if (hpb == 2) launch_fused_t<N, 2, 32, 3, MODE>(a, stream);
    else launch_fused_t<N, 1, 32, 2, MODE>(a, stream);
  }
}

hipError_t launch_any(const FusedArgs &a, int N, int mode, hipStream_t stream) {
  const int cus = device_cus();
  const int HG = a.H / a.G;
  const int hpb = HG % 3 == 0 && (int64_t)a.rows * (a.H / 3) >= cus ? 3
                  : HG % 2 == 0 && (int64_t)a.rows * (a.H / 2) >= cus ? 2 : 1;
#define SSD_FUSED_N(NN)                                                  \
  if (mode == kFwdSave) launch_fused_n<NN, kFwdSave>(hpb, a, stream);    \
  else if (mode == kState) launch_fused_n<NN, kState>(hpb, a, stream);   \
  else launch_fused_n<NN, kFwd>(hpb, a, stream);
  switch (N) {
    case 64: SSD_FUSED_N(64) break;
    case 128: SSD_FUSED_N(128) break;
    default: SSD_FUSED_N(256) break;
  }
#undef SSD_FUSED_N
  return hipGetLastError();
}

// Hand-off over the segments (the inter-chunk recurrence one level up): per
// (sequence, kernel head) and 4 consecutive state elements a thread, the
// state entering segment 0 (h0, or 0) into hbuf[sq][0], then
// h <- 2^lseg[sq][j] h + hbuf[sq][j + 1] in place along j = 0 .. nseg-2, so
// that hbuf[sq][j] ends as the state entering segment j.
__global__ __launch_bounds__(256) void k_seg_pass(float *__restrict__ hbuf,
                                                  const float *__restrict__ lseg,
                                                  const float *__restrict__ h0, int nseq, int nseg,
                                                  int H, int PN4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (sq, h, e4)
  if (i >= (int64_t)nseq * H * PN4) return;
  const int64_t e4 = i % PN4, sh = i / PN4;
  const int64_t sq = sh / H, h = sh % H;
  f32x4 v = h0 ? reinterpret_cast<const f32x4 *>(h0)[sh * PN4 + e4] : f32x4{};
  f32x4 *hb = reinterpret_cast<f32x4 *>(hbuf) + (sq * nseg * H + h) * PN4 + e4;
  *hb = v;
  for (int j = 0; j + 1 < nseg; ++j) {
    f32x4 *p = hb + (int64_t)(j + 1) * H * PN4;
    v = v * __builtin_amdgcn_exp2f(lseg[(sq * (nseg - 1) + j) * H + h]) + *p;
    *p = v;
  }
}
}  // namespace

hipError_t launch_fused(const void *x, const float *dt, const float *A, const void *B, const void *C,
                        const float *D, const float *h0, const int32_t *cu, int64_t L, int64_t T,
                        int rows, int H, int P, int N, int G, int hr, void *y, float *hfin,
                        void *hsave, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!fused_supported(H, P, N, G) || hr < 1 || H % hr != 0) return hipErrorInvalidValue;
  FusedArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.dt = dt;
  a.A = A;
  a.B = static_cast<const uint16_t *>(B);
  a.C = static_cast<const uint16_t *>(C);
  a.D = D;
  a.h0 = h0;
  a.cu = cu;
  a.L = L;
  a.T = T;
  a.S = L;
  a.nsr = 1;
  a.rows = rows;
  a.H = H;
  a.G = G;
  a.hr = hr;
  a.y = static_cast<uint16_t *>(y);
  a.hfin = hfin;
  a.hsave = static_cast<uint16_t *>(hsave);
  return launch_any(a, N, hsave ? kFwdSave : kFwd, stream);
}

hipError_t launch_fused_split(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *h0, int64_t L,
                              int nseq, int64_t S, int H, int P, int N, int G, int hr, void *y,
                              float *hfin, float *sseg, float *lseg, void *hsave,
                              hipStream_t stream) {
  if (nseq == 0 || L == 0) return hipSuccess;
  if (!fused_supported(H, P, N, G) || hr < 1 || H % hr != 0 || S <= 0 || S % 32 != 0 ||
      (hsave && S % 64 != 0))
    return hipErrorInvalidValue;
  const int nseg = static_cast<int>((L + S - 1) / S);
  FusedArgs a{};
  a.x = static_cast<const uint16_t *>(x);
  a.dt = dt;
  a.A = A;
  a.B = static_cast<const uint16_t *>(B);
  a.C = static_cast<const uint16_t *>(C);
  a.D = D;
  a.L = L;
  a.T = L * nseq;
  a.S = S;
  a.H = H;
  a.G = G;
  a.hr = hr;
  hipError_t e;
  if (nseg > 1) {
    // 1. every segment but the last, from a zero state: its end state and decay
    a.nsr = nseg - 1;
    a.rows = nseq * (nseg - 1);
    a.sseg = sseg;
    a.lseg = lseg;
    if ((e = launch_any(a, N, kState, stream)) != hipSuccess) return e;
    // 2. the states entering the segments (so that step 3 does not read h0,
    // which final_state may alias)
    const int PN4 = P * N / 4;
    const int64_t n = (int64_t)nseq * H * PN4;
    hipLaunchKernelGGL(k_seg_pass, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, sseg,
                       lseg, h0, nseq, nseg, H, PN4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 3. every segment from its entering state: y, and the final state (and,
  // when saving, the state entering every 64-token pair)
  a.nsr = nseg;
  a.rows = nseq * nseg;
  a.h0 = h0;
  a.hin = nseg > 1 ? sseg : nullptr;
  a.sseg = nullptr;
  a.lseg = nullptr;
  a.y = static_cast<uint16_t *>(y);
  a.hfin = hfin;
  a.hsave = static_cast<uint16_t *>(hsave);
  return launch_any(a, N, hsave ? kFwdSave : kFwd, stream);
}

}  // namespace ssd
