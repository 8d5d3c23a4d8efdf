// libssd: chunk_scan on bf16 MFMA (gfx950).
//
// For chunk c, head h and every token l of the chunk:
//   y_l = sum_{s<=l} (C_l . B_s) exp(acum_l - acum_s) dt_s x_s     (intra-chunk)
//       + exp(acum_l) C_l hprev^T                                   (state handed in)
//       + D_h x_l                                                   (skip)
// The first term is the masked product (C B^T o L) X with the causal
// 1-semiseparable decay mask L (page "State Space Duality and Mamba-2 ...",
// section "The Scalar-Identity Structural Constraint"; page "Mamba-2
// Architecture: State Space Duality Explained", "2. The Chunked SSD
// Algorithm", item 1); the second is the inter-chunk hand-off of item 2, with
// the in-chunk decay exp(acum_l) that the page's listing leaves out.
//
// Shared design.  The output is formed transposed, Y^T [P x Q], as 32x32
// MFMA tiles (M = p, N = l), the chunk cut into Q/32 token tiles:
//   * inter term: Y^T += Hprev . C^T over K = n, then each lane scales by the
//     decay of its token -- a lane owns one output column l;
//   * intra term, per source tile k <= j: Z = B_k . C_j^T on MFMA, the decay
//     mask applied to Z in registers, the fp32 accumulator rounded to bf16 and
//     used directly as the B-operand of Y^T += X_k^T . G^T: that MFMA's K order
//     is permuted to the accumulator's row order and X^T is read from LDS in
//     the same order (a transposing LDS read), so no cross-lane shuffle is
//     needed;
//   * decay: off the diagonal (k < j) exp(acum_l - acum_s) is split at
//     m = acum at the token tile's first token into u_l = exp(acum_l - m) (one
//     per lane, taken out of the sum over off-diagonal tiles) and
//     v_s = exp(m - acum_s) dt_s (a per-chunk table in LDS); both are <= 1 for
//     non-increasing acum, so nothing overflows.  Diagonal tiles take
//     exp(acum_l - acum_s) per element, masked to s <= l before the exponent
//     is formed.
//
// One kernel, k_chunk_scan_hb (P = 64, Q in {64, 128, 256}, N in {64, 128,
// 256}): a block walks a run of heads of one chunk; Z is formed once and kept
// in registers, and x / hprev of the next head stream in while the current
// one computes.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

template <int KN>
__device__ __forceinline__ void load_rows(u32x4 (&dst)[KN], const uint16_t *row, bool valid) {
#pragma unroll
  for (int q = 0; q < KN; ++q)
    dst[q] = valid ? *reinterpret_cast<const u32x4 *>(row + q * 16) : u32x4{0u, 0u, 0u, 0u};
}

// Off-diagonal decay with the per-lane factor taken out of the sum: g = z * v[s].
__device__ __forceinline__ void decay_offdiag_v(const f32x16 &z, const float *vrow, int kg,
                                                float (&gv)[16]) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(vrow + 8 * rb + 4 * kg);
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[rb * 4 + e] = z[rb * 4 + e] * v[e];
  }
}

// Diagonal decay: g = z * exp(acum_l - acum_s) * dt_s for s <= l, else 0.  The
// lane's 16 rows are 4 runs of 4 consecutive s, read as 16-byte vectors; the
// mask is applied to the exponent's argument before exp is taken.
__device__ __forceinline__ void decay_diag(const f32x16 &z, float al, int l, int s0, int kg,
                                           const float *sa, const float *sd, float (&gv)[16]) {
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int sb = s0 + 8 * rb + 4 * kg;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(sa + sb);
    const f32x4 d = *reinterpret_cast<const f32x4 *>(sd + sb);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool keep = sb + e <= l;
      const float arg = keep ? (al - a[e]) : -__builtin_inff();
      gv[rb * 4 + e] = keep ? z[rb * 4 + e] * __expf(arg) * d[e] : 0.f;
    }
  }
}

__device__ __forceinline__ void pack_g(const float (&gv)[16], u32x4 &g0, u32x4 &g1) {
  g0.x = pack_bf16x2(gv[0], gv[1]);
  g0.y = pack_bf16x2(gv[2], gv[3]);
  g0.z = pack_bf16x2(gv[4], gv[5]);
  g0.w = pack_bf16x2(gv[6], gv[7]);
  g1.x = pack_bf16x2(gv[8], gv[9]);
  g1.y = pack_bf16x2(gv[10], gv[11]);
  g1.z = pack_bf16x2(gv[12], gv[13]);
  g1.w = pack_bf16x2(gv[14], gv[15]);
}

// ============================================================ head-batched kernel
// P = 64, Q in {64, 128, 256}.  The heads of a group share B and C, so Z = B C^T
// of a chunk is the same for all of them: block = (chunk, group, run of hb
// heads), NW = Q/32 wavefronts, one token tile each: with W = NW/2, wavefront
// w < W owns tile w and wavefront w >= W tile NW-1-(w-W), so tiles j and
// NW-1-j share a SIMD.  The causal work is balanced by handing pairs over:
// wavefront s < W also forms the off-diagonal pairs (NW-1-s, i < W-s) and
// passes their sum to the owner of tile NW-1-s through LDS, so every
// wavefront has W-1 or W off-diagonal pairs and one diagonal pair (Q 256: 3
// or 4).  Its W+1 Z tiles (pairs formed once per block from the chunk's B
// staged in LDS) and the C rows of its tile stay in registers.  The block then walks its heads; x, acum, dt and hprev
// of head i+1 stream into the other half of two-slot LDS rings while head i
// computes, and y of head i, staged over its x as bf16, goes out at the top of
// head i+1 in 128-byte row segments.  Per head:
//   1. y of the previous head is stored; the v table of this head is built;
//   2. the next head's loads go out;
//   3. handed-over pairs (wavefronts 0 .. W-1), summed and written to LDS;
//   4. inter term Y^T = exp(acum at the tile's first token) Hprev C^T, then
//      the tile's own off-diagonal pairs;
//   5. (barrier) the handed-over sum is added, u_l applied, then the diagonal
//      pair and the skip term;
//   6. (barrier) the tile is rounded to bf16 and staged over this head's x.
// LDS bytes of k_chunk_scan_hb<Q, N> with P = 64 (hs: hprev slots).
constexpr int hb_hprev_slots(int Q, int N) { return N > 128 || (Q < 256 && N > 64) ? 1 : 2; }
constexpr int hb_lds_bytes(int Q, int N) {
  return 2 * (Q * 64 * 2) + hb_hprev_slots(Q, N) * (64 * N * 2) + 2 * (2 * Q * 4) +
         (Q / 32) * Q * 4 + (Q / 64) * (32 * 64 * 4);
}

// Blocks a CU holds (LDS-bound) and the waves a SIMD then holds.
constexpr int hb_blocks_per_cu(int Q, int N) { return (160 * 1024) / hb_lds_bytes(Q, N); }
constexpr int hb_waves_per_simd(int Q, int N) {
  return (hb_blocks_per_cu(Q, N) * (Q / 32) + 3) / 4;
}

template <int Q, int N>
__global__ __launch_bounds__(2 * Q, hb_waves_per_simd(Q, N)) void k_chunk_scan_hb(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ Dv, const float *__restrict__ acum,
    const float *__restrict__ dtq, const uint16_t *__restrict__ hprev, ChunkGeom geom, int nc,
    int H, int G, int hb, int nkb, int hr, uint16_t *__restrict__ y) {
  constexpr int P = 64;
  static_assert(N == 64 || N == 128 || N == 256, "head-batched tile shape");
  static_assert(Q == 64 || Q == 128 || Q == 256, "chunk length");
  // N 256: B is staged in two 128-column halves for the Z phase.  hprev has
  // one LDS slot (loaded once the previous head's inter term is done) at
  // N 256, and at N 128 for Q < 256 (so that two blocks fit a CU)
  constexpr int NH = N > 128 ? 2 : 1;  // B halves
  constexpr int NBH = N / NH;          // columns of a staged B half
  constexpr int NCBH = NBH / 8;        // its 16-byte chunks per row
  constexpr int HSL = hb_hprev_slots(Q, N);  // hprev slots
  constexpr int NT = 2 * Q;           // threads
  constexpr int NW = Q / 32;          // wavefronts
  constexpr int W = NW / 2;           // donors (and receivers)
  constexpr int NLT = Q / 32;         // token tiles
  constexpr int TP = P / 32;          // p tiles
  constexpr int KN = N / 16;          // K steps over n
  constexpr int NCB = N / 8;          // 16-byte chunks per B / hprev row
  constexpr int NCX = P / 8;          // 16-byte chunks per x / y row
  constexpr int XB = Q * P * 2;       // x (then y) of one head
  constexpr int HB = P * N * 2;       // hprev of one head
  constexpr int ADB = 2 * Q * 4;      // acum and dt of one head
  constexpr int BB = Q * NBH * 2;     // B of the chunk (a half at N 256), Z phase only
  constexpr int PSB = 32 * P * 4;     // one handed-over partial sum (fp32)
  constexpr int XI = XB / 1024 / NW;  // 1 KB direct loads per wavefront
  constexpr int HI = HB / 1024 / NW;
  constexpr int BI = BB / 1024 / NW;
  static_assert(XI * NW * 1024 == XB && HI * NW * 1024 == HB && BI * NW * 1024 == BB, "1 KB loads");
  // [XS0][XS1][HS0][HS1][AD0][AD1][VT][PS0..PS3]; B is staged over XS0 + XS1
  constexpr int XS0 = 0, XS1 = XB, HS0 = 2 * XB, HS1 = HS0 + (HSL - 1) * HB, AD0 = HS1 + HB,
                AD1 = AD0 + ADB;
  constexpr int VT = AD1 + ADB, PS = VT + NLT * Q * 4, TOTAL = PS + W * PSB;
  static_assert(2 * XB >= BB, "B staging fits over the x ring");
  static_assert(TOTAL == hb_lds_bytes(Q, N) && TOTAL <= 160 * 1024, "LDS");
  static_assert(NLT == NW && NT == 64 * NW, "one token tile a wavefront");
  __shared__ __align__(16) unsigned char smem[TOTAL];

  int c, hk;
  xcd_chunk_head(G * nkb, c, hk);
  if (c >= nc) return;
  const int g = hk / nkb;
  const int kb = hk - g * nkb;
  const int HG = H / G;
  const int hfirst = g * HG + kb * hb;
  const int nh = min(hb, HG - kb * hb);
  if (nh <= 0) return;
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;

  // Lane indices.  Inside the head loop they are re-read from an opaque copy
  // each head, so the compiler forms lane-dependent addresses where they are
  // used instead of keeping dozens of them live across heads.
  struct Lane {
    int tid, lane, col, kg;
    __device__ explicit Lane(int t) : tid(t), lane(t & 63), col(t & 31), kg((t >> 5) & 1) {}
  };
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lane L0(tid);
  const int lane = L0.lane;
  const int col = L0.col;
  const int kg = L0.kg;
  const int s4 = wave % W;
  const bool donor = wave < W;
  const int T = donor ? s4 : NLT - 1 - s4;  // own token tile
  const int TD = NLT - 1 - s4;              // tile of the handed-over pairs
  const int nd = donor ? W - s4 : 0;        // handed-over pairs: source tiles 0 .. nd-1 of TD
  const int l = T * 32 + col;               // this lane's token (output column)
  const int64_t ldx = (int64_t)H * P;
  const int64_t ldb = (int64_t)G * N;
  const int64_t xrow0 = ci.t0 * ldx;
  const int ldx32 = H * P;  // row offsets inside a chunk: Q * H * P < 2^31 (H < 2^16)

  // Direct loads, 16-byte chunks XOR-swizzled per row.  Token rows past the
  // chunk's end repeat its last row: finite data that dt = 0 cancels, in rows
  // of y that are never stored.
  auto issue_head = [&](const Lane &Ln, int hh, int slot, bool with_h) {
    const int lane = Ln.lane;
    const uint16_t *xb = x + xrow0 + (int64_t)hh * P;
    unsigned char *xs = smem + (slot ? XS1 : XS0);
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const unsigned m = (wave * XI + i) * 64 + lane, r = m / NCX;
      const unsigned cc = (m % NCX) ^ chunk_swz(r, NCX);
      load_lds16(xb + min((int)r, ci.len - 1) * ldx32 + cc * 8, xs + (wave * XI + i) * 1024);
    }
    const int64_t ch = (int64_t)c * H + hh;
    const uint16_t *hp = hprev + ch * (P * N);
    unsigned char *hs = smem + (slot ? HS1 : HS0);
#pragma unroll
    for (int i = 0; i < (with_h ? HI : 0); ++i) {
      const unsigned m = (wave * HI + i) * 64 + lane, r = m / NCB;
      const unsigned cc = (m % NCB) ^ chunk_swz(r, NCB);
      load_lds16(hp + r * N + cc * 8, hs + (wave * HI + i) * 1024);
    }
    if constexpr (Q == 256) {
      if (wave < 2)  // wavefront 0: acum, 1: dt
        load_lds16((wave == 0 ? acum : dtq) + ch * Q + lane * 4, smem + (slot ? AD1 : AD0) + wave * 1024);
    } else if (wave == 0 && lane < Q / 2) {  // lanes Q/4 apart: acum, then dt
      constexpr int HQ = Q / 4;
      load_lds16((lane < HQ ? acum + ch * Q + lane * 4 : dtq + ch * Q + (lane - HQ) * 4),
                 smem + (slot ? AD1 : AD0));
    }
  };
  auto issue_hprev = [&](const Lane &Ln, int hh) {  // one-slot hprev (N 256)
    const int lane = Ln.lane;
    const uint16_t *hp = hprev + ((int64_t)c * H + hh) * (P * N);
#pragma unroll
    for (int i = 0; i < HI; ++i) {
      const unsigned m = (wave * HI + i) * 64 + lane, r = m / NCB;
      const unsigned cc = (m % NCB) ^ chunk_swz(r, NCB);
      load_lds16(hp + r * N + cc * 8, smem + HS0 + (wave * HI + i) * 1024);
    }
  };
  auto store_y = [&](const Lane &Ln, int hh, const unsigned char *ys) {
    const unsigned tid = Ln.tid;
    uint16_t *yb = y + xrow0 + (int64_t)hh * P;
    constexpr int NI = Q * NCX / NT;
    u32x4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {  // all LDS reads first, then the stores
      const unsigned u = tid + i * NT, r = u / NCX, gp = u % NCX;
      v[i] = *reinterpret_cast<const u32x4 *>(ys + r * (P * 2) + (gp ^ chunk_swz(r, NCX)) * 16);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const unsigned u = tid + i * NT, r = u / NCX, gp = u % NCX;
      // streaming stores: nothing in this pass reads y again
      if ((int)r < ci.len) __builtin_nontemporal_store(v[i], reinterpret_cast<u32x4 *>(yb + r * ldx32 + gp * 8));
    }
  };

  // ---- Z phase: the chunk's B (in NH column halves), head 0's data, and the
  // C rows of the lane's own and handed-over tiles (registers)
  const uint16_t *cbase = Cm + ci.t0 * ldb + (int64_t)g * N + kg * 8;
  u32x4 cown[KN], cdon[KN];
  f32x16 z[W + 1];
#pragma unroll
  for (int k = 0; k <= W; ++k) z[k] = f32x16{};
#pragma unroll
  for (int half = 0; half < NH; ++half) {
    if (half > 0) __syncthreads();  // the previous half is consumed
    {
      const uint16_t *bb = Bm + ci.t0 * ldb + (int64_t)g * N + half * NBH;
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int m = (wave * BI + i) * 64 + lane;
        const int r = m / NCBH, cc = (m % NCBH) ^ chunk_swz(m / NCBH, NCBH);
        load_lds16(bb + (int64_t)min(r, ci.len - 1) * ldb + cc * 8, smem + XS0 + (wave * BI + i) * 1024);
      }
    }
    if (half == 0) {
      load_rows<KN>(cown, cbase + (int64_t)l * ldb, l < ci.len);
      load_rows<KN>(cdon, cbase + (int64_t)(TD * 32 + col) * ldb, TD * 32 + col < ci.len);
    }
    wait_vmcnt<0>();
    __syncthreads();
    // slot k < W: handed-over pair (TD, k) for k < nd, else own off-diagonal
    // pair (T, k - nd) on a donor and (T, T - (W-1) + k) on a receiver (k =
    // W-1 unused there); slot W: the diagonal pair (T, T).  Operands are
    // picked by value, with no branches, so each tile is formed in the
    // registers it stays in.
#pragma unroll
    for (int k = 0; k <= W; ++k) {
      const bool dk = k < nd;
      const int zi = k == W ? T : (donor ? (dk ? k : k - nd) : min(T - (W - 1) + k, T));
      const unsigned char *brow = smem + XS0 + (32 * zi + col) * (NBH * 2);
      f32x16 acc = z[k];
#pragma unroll
      for (int q = 0; q < KN / NH; ++q) {
        const int cc = (2 * q + kg) ^ chunk_swz(col, NCBH);
        const u32x4 bq = *reinterpret_cast<const u32x4 *>(brow + cc * 16);
        const u32x4 cq = dk ? cdon[half * (KN / NH) + q] : cown[half * (KN / NH) + q];
        acc = mfma32x32x16(as_bf16x8(bq), as_bf16x8(cq), acc);
      }
      z[k] = acc;
    }
  }
  __syncthreads();  // B consumed: the x ring is free
  issue_head(L0, hfirst, 0, true);

  // X^T operands of source tile i by transposing LDS reads: lane (gq = lane/16,
  // d = lane%16) addresses token row 32i + 8h4 + 4kg + d/4, columns 4(d%4)..,
  // and receives p = 32t + 16(gq%2) + d of 4 consecutive tokens -- the K order
  // of the accumulator rows of G (offsets 4kg.., 8+4kg.., 16+4kg.., 24+4kg..)
  auto x_ops = [&](const Lane &Ln, const unsigned char *xs, int i, int t, u32x4 &xa, u32x4 &xb) {
    const int kg = Ln.kg;
    const int gq = Ln.lane >> 4, d = Ln.lane & 15;
    const int p0 = t * 32 + 16 * (gq & 1) + 4 * (d & 3);
    u32x2 part[4];
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {
      const int row = 32 * i + 8 * h4 + 4 * kg + (d >> 2);
      const int cc = (p0 >> 3) ^ chunk_swz(row, NCX);
      part[h4] = lds_read_tr16(xs + row * (P * 2) + cc * 16 + (p0 & 7) * 2);
    }
    xa = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
    xb = u32x4{part[2].x, part[2].y, part[3].x, part[3].y};
  };
  // acc += X_i^T G^T with G = the decayed, bf16-rounded Z tile
  auto pair_xg = [&](const Lane &Ln, f32x16 (&acc)[TP], const unsigned char *xs, int i,
                     const float (&gv)[16]) {
    u32x4 g0, g1;
    pack_g(gv, g0, g1);
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      u32x4 xa, xb;
      x_ops(Ln, xs, i, t, xa, xb);
      acc[t] = mfma32x32x16(as_bf16x8(xa), as_bf16x8(g0), acc[t]);
      acc[t] = mfma32x32x16(as_bf16x8(xb), as_bf16x8(g1), acc[t]);
    }
  };

#pragma unroll 1
  for (int hi = 0; hi < nh; ++hi) {
    const int hh = hfirst + hi;
    const int slot = hi & 1;
    unsigned char *xs = smem + (slot ? XS1 : XS0);
    const unsigned char *hs = smem + (slot ? HS1 : HS0);
    const float *sa = reinterpret_cast<const float *>(smem + (slot ? AD1 : AD0));
    const float *sd = sa + Q;
    float *vt = reinterpret_cast<float *>(smem + VT);  // vt[j][s] = exp(acum[32j] - acum[s]) dt[s]

    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    const Lane Lh(tid_o);
    const int lane = Lh.lane, col = Lh.col, kg = Lh.kg;
    const int l = T * 32 + col;

    wait_vmcnt<0>();  // this head's loads; the stores of y two heads back
    wait_lgkmcnt0();  // this wavefront's y staging of the previous head
    __syncthreads();  // ... for every thread; the previous head is done everywhere
    if (hi > 0) store_y(Lh, hh - 1, smem + (slot ? XS0 : XS1));
    {  // column s = tid % Q; rows 1..3 (first half of the block) or 4..7
      const unsigned s = tid_o & (Q - 1);
      const int j0 = tid_o < Q ? 1 : NLT / 2;
      const int jend = tid_o < Q ? NLT / 2 : NLT;
      const float as = sa[s], ds = sd[s];
      float e[NLT / 2];
#pragma unroll
      for (int jj = 0; jj < NLT / 2; ++jj) e[jj] = __expf(sa[32 * (j0 + jj)] - as) * ds;
#pragma unroll
      for (int jj = 0; jj < NLT / 2; ++jj)
        if (j0 + jj < jend && (int)s < 32 * (j0 + jj)) vt[(j0 + jj) * Q + s] = e[jj];
    }
    __syncthreads();  // v table ready; the other slot's y has been read out
    if (hi + 1 < nh) issue_head(Lh, hh + 1, slot ^ 1, HSL == 2);

    f32x16 acc[TP];
    // 3. handed-over pairs (donors): sum over source tiles 0 .. nd-1 of tile TD
    if (donor) {
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[t] = f32x16{};
#pragma unroll
      for (int k = 0; k < W; ++k) {
        if (k < nd) {
          float gv[16];
          decay_offdiag_v(z[k], vt + TD * Q + 32 * k, kg, gv);
          pair_xg(Lh, acc, xs, k, gv);
        }
      }
      float *ps = reinterpret_cast<float *>(smem + PS + s4 * PSB);
#pragma unroll
      for (int t = 0; t < TP; ++t)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          *reinterpret_cast<f32x4 *>(ps + ((t * 4 + rb) * 64 + lane) * 4) =
              f32x4{acc[t][rb * 4], acc[t][rb * 4 + 1], acc[t][rb * 4 + 2], acc[t][rb * 4 + 3]};
    }
    // 4. inter term, scaled by exp(acum at the tile's first token), then the
    // tile's own off-diagonal pairs
    const float al = sa[l];
    const float m0 = sa[32 * T];
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int q = 0; q < KN; ++q) {
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        const int row = t * 32 + col;
        const int cc = (2 * q + kg) ^ chunk_swz(row, NCB);
        const u32x4 hq = *reinterpret_cast<const u32x4 *>(hs + row * (N * 2) + cc * 16);
        acc[t] = mfma32x32x16(as_bf16x8(hq), as_bf16x8(cown[q]), acc[t]);
      }
    }
    {
      const float em = __expf(m0);
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[t] *= em;
    }
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const bool own = donor ? k >= nd : k < W - 1;
      if (own) {
        const int i = donor ? k - nd : T - (W - 1) + k;
        float gv[16];
        decay_offdiag_v(z[k], vt + T * Q + 32 * i, kg, gv);
        pair_xg(Lh, acc, xs, i, gv);
      }
    }
    __syncthreads();  // handed-over sums are in LDS; every inter term has read hprev
    if (HSL == 1 && hi + 1 < nh) issue_hprev(Lh, hh + 1);
    // 5. handed-over sum (receivers), u_l, the diagonal pair, the skip term
    if (!donor) {
      const float *ps = reinterpret_cast<const float *>(smem + PS + s4 * PSB);
#pragma unroll
      for (int t = 0; t < TP; ++t)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 v = *reinterpret_cast<const f32x4 *>(ps + ((t * 4 + rb) * 64 + lane) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][rb * 4 + e] += v[e];
        }
    }
    {
      const float u = __expf(al - m0);  // <= 1
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[t] *= u;
    }
    {
      float gv[16];
      decay_diag(z[W], al, l, 32 * T, kg, sa, sd, gv);
      pair_xg(Lh, acc, xs, T, gv);
    }
    {  // D x_l in fp32: rows p = 32t + 8rb + 4kg + e of column l are 4
       // consecutive elements of x row l
      const float Dh = Dv ? Dv[hh / hr] : 0.f;
#pragma unroll
      for (int t = 0; t < TP; ++t) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int p = t * 32 + rb * 8 + kg * 4;
          const int cc = (p >> 3) ^ chunk_swz(l, NCX);
          const u32x2 xv = *reinterpret_cast<const u32x2 *>(xs + l * (P * 2) + cc * 16 + (p & 7) * 2);
          acc[t][rb * 4 + 0] += Dh * bf16lo(xv.x);
          acc[t][rb * 4 + 1] += Dh * bf16hi(xv.x);
          acc[t][rb * 4 + 2] += Dh * bf16lo(xv.y);
          acc[t][rb * 4 + 3] += Dh * bf16hi(xv.y);
        }
      }
    }
    __syncthreads();  // this head's x and the handed-over sums read by everyone
    // 6. stage y over this head's x
#pragma unroll
    for (int t = 0; t < TP; ++t) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int p = t * 32 + rb * 8 + kg * 4;
        u32x2 o;
        o.x = pack_bf16x2(acc[t][rb * 4 + 0], acc[t][rb * 4 + 1]);
        o.y = pack_bf16x2(acc[t][rb * 4 + 2], acc[t][rb * 4 + 3]);
        *reinterpret_cast<u32x2 *>(xs + l * (P * 2) + ((p >> 3) ^ chunk_swz(l, NCX)) * 16 + (p & 7) * 2) = o;
      }
    }
  }
  __syncthreads();
  store_y(L0, hfirst + nh - 1, smem + (((nh - 1) & 1) ? XS1 : XS0));
}

}  // namespace

bool chunk_scan_bf16_supported(int P, int N, int Q) {
  return P == 64 && (N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

template <int Q, int P, int N>
static void launch_sc(const void *x, const void *B, const void *C, const float *D,
                      const float *acum, const float *dtq, const void *hprev, void *y,
                      const Geometry &geo, hipStream_t stream) {
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  static_assert(P == 64, "head dim 64 (wider heads run as 64-row kernel heads)");
  int nkb = 1;
  const int slots = hb_blocks_per_cu(Q, N) * device_cus();
  const int hb = pick_heads_per_block(geo.nc_max, geo.H, geo.G, slots, 1.5, nkb);
  hipLaunchKernelGGL((k_chunk_scan_hb<Q, N>), dim3(xcd_grid(geo.nc_max, geo.G * nkb)),
                     dim3(2 * Q), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(C), D, acum,
                     dtq, static_cast<const uint16_t *>(hprev), cg, (int)geo.nc_max, geo.H, geo.G,
                     hb, nkb, geo.hr, static_cast<uint16_t *>(y));
}

template <int Q>
static bool dispatch_sc_n(const void *x, const void *B, const void *C, const float *D,
                          const float *acum, const float *dtq, const void *hprev, void *y,
                          const Geometry &geo, hipStream_t stream) {
  switch (geo.N) {
    case 64: launch_sc<Q, 64, 64>(x, B, C, D, acum, dtq, hprev, y, geo, stream); return true;
    case 128: launch_sc<Q, 64, 128>(x, B, C, D, acum, dtq, hprev, y, geo, stream); return true;
    case 256: launch_sc<Q, 64, 256>(x, B, C, D, acum, dtq, hprev, y, geo, stream); return true;
    default: return false;
  }
}

hipError_t launch_chunk_scan_bf16(const void *x, const void *B, const void *C, const float *D,
                                  const float *acum, const float *dtq, const void *hprev, void *y,
                                  const Geometry &geo, hipStream_t stream) {
  if (geo.nc_max == 0) return hipSuccess;
  if (!chunk_scan_bf16_supported(geo.P, geo.N, geo.Q)) return hipErrorInvalidValue;
  bool ok = false;
  switch (geo.Q) {
    case 64: ok = dispatch_sc_n<64>(x, B, C, D, acum, dtq, hprev, y, geo, stream); break;
    case 128: ok = dispatch_sc_n<128>(x, B, C, D, acum, dtq, hprev, y, geo, stream); break;
    case 256: ok = dispatch_sc_n<256>(x, B, C, D, acum, dtq, hprev, y, geo, stream); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssd
