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
// Two kernels share this arithmetic:
//   * k_chunk_scan_hb (Q = 256, P = 64, N <= 128): one block per CU walks a
//     run of heads of one chunk; Z is formed once and kept in registers, and
//     x / hprev of the next head stream in while the current one computes.
//   * k_chunk_scan_lds (other shapes): block = (chunk, head) in XCD-aware
//     order; B and x tiles stream through LDS rings filled by direct-to-LDS
//     loads, Z is formed per head.
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

// ============================================================ LDS-staged kernel
// Block = (chunk, head), Q/64 wavefronts; wavefront w owns token tiles w and
// Q/32-1-w (balanced causal work) and keeps their C rows in registers.  The
// source tiles go by in lockstep: B and x tiles of 32 tokens stream through
// DEPTH-slot LDS rings filled by direct-to-LDS loads issued DEPTH-1 tiles
// ahead; each step waits for its own tile only, then a block barrier.  When a
// wavefront has both token tiles in play their MFMA chains share the operand
// reads.  hprev is staged once; the inter term and D x are added after the
// loop, and each wavefront writes its tiles through an LDS slice as 16-byte
// row segments.
template <int Q, int P, int N>
__global__ __launch_bounds__(Q, Q >= 128 ? 2 : 1) void k_chunk_scan_lds(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ Dv, const float *__restrict__ acum,
    const float *__restrict__ dtq, const uint16_t *__restrict__ hprev, ChunkGeom geom, int nc,
    int H, int G, int hr, uint16_t *__restrict__ y) {
  static_assert(P == 64 && N % 64 == 0 && Q % 64 == 0, "tile shape");
  constexpr int NT = Q;          // threads
  constexpr int NW = Q / 64;     // wavefronts
  constexpr int NLT = Q / 32;    // token tiles
  constexpr int TP = P / 32;     // p tiles
  constexpr int KN = N / 16;     // K steps over n
  constexpr int NCB = N / 8;     // 16-byte chunks per B / hprev row
  constexpr int NCX = P / 8;     // 16-byte chunks per x row
  constexpr int BT = 32 * N * 2;   // B tile bytes
  constexpr int XT = 32 * P * 2;   // x tile bytes
  constexpr int DEPTH = N <= 128 ? 4 : 2;  // ring slots: tiles k .. k+DEPTH-1
  constexpr int BI = BT / 1024 / NW;       // 1 KB direct loads per wave per B tile
  constexpr int XI = XT / 1024 / NW;       // ... per x tile
  constexpr int HI = P * N * 2 / 1024 / NW;
  constexpr int LPT = BI + XI;             // loads per thread per source tile
  static_assert(BI * NW * 1024 == BT && XI * NW * 1024 == XT && HI * NW * 1024 == P * N * 2,
                "tiles split evenly into 1 KB wave loads");
  constexpr int RB = 0;                    // ring of B tiles
  constexpr int RX = DEPTH * BT;           // ring of x tiles
  constexpr int HS = RX + DEPTH * XT;      // hprev [P][N]
  constexpr int LYB = P + 4;               // output staging row (fp32) + pad
  constexpr int YS = NW * 32 * LYB * 4;    // output staging, after everything else
  constexpr int MAIN = HS + P * N * 2 > YS ? HS + P * N * 2 : YS;

  __shared__ __align__(16) unsigned char smem[MAIN];
  __shared__ __align__(16) float sa[Q];
  __shared__ __align__(16) float sd[Q];
  __shared__ __align__(16) float vt[NLT][Q];  // vt[j][s] = exp(acum[32j] - acum[s]) dt[s], s < 32j

  int c, h;
  xcd_chunk_head(H, c, h);
  if (c >= nc) return;
  const int g = h / (H / G);
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;
  const int64_t ch = (int64_t)c * H + h;
  const int nk = (ci.len + 31) >> 5;  // token tiles that hold tokens
  const int64_t ldx = (int64_t)H * P;
  const int64_t ldb = (int64_t)G * N;
  const uint16_t *xbase = x + ci.t0 * ldx + (int64_t)h * P;
  const uint16_t *bbase = Bm + ci.t0 * ldb + (int64_t)g * N;
  const uint16_t *cbase = Cm + ci.t0 * ldb + (int64_t)g * N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int col = lane & 31;
  const int kg = lane >> 5;
  const int j1 = wave;
  const int j2 = NLT - 1 - wave;  // > j1
  const int l1 = j1 * 32 + col;
  const int l2 = j2 * 32 + col;
  const bool act1 = j1 < nk;
  const bool act2 = j2 < nk;

  // ---- register loads first (acum, dt, the C operands of both token tiles),
  // so the compiler's waits for them leave the direct loads below in flight
  for (int l = tid; l < Q; l += NT) {
    sa[l] = acum[ch * Q + l];
    sd[l] = dtq[ch * Q + l];
  }
  u32x4 c1[KN], c2[KN];
  load_rows<KN>(c1, cbase + (int64_t)l1 * ldb + kg * 8, l1 < ci.len);
  load_rows<KN>(c2, cbase + (int64_t)l2 * ldb + kg * 8, l2 < ci.len);

  // ---- direct loads: hprev, then source tiles 0 .. DEPTH-2.  Rows past the
  // chunk's end read its last row (finite data the zero dt then cancels).
  {
    const uint16_t *hp = hprev + ch * (int64_t)P * N;
#pragma unroll
    for (int i = 0; i < HI; ++i) {
      const int m = (wave * HI + i) * 64 + lane;
      const int r = m / NCB, cc = (m % NCB) ^ chunk_swz(m / NCB, NCB);
      load_lds16(hp + (int64_t)r * N + cc * 8, smem + HS + (wave * HI + i) * 1024);
    }
  }
  auto issue_tile = [&](int k) {
    const int slot = k % DEPTH;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int m = (wave * BI + i) * 64 + lane;
      const int r = m / NCB, cc = (m % NCB) ^ chunk_swz(m / NCB, NCB);
      const int s = min(32 * k + r, ci.len - 1);
      load_lds16(bbase + (int64_t)s * ldb + cc * 8, smem + RB + slot * BT + (wave * BI + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int m = (wave * XI + i) * 64 + lane;
      const int r = m / NCX, cc = (m % NCX) ^ chunk_swz(m / NCX, NCX);
      const int s = min(32 * k + r, ci.len - 1);
      load_lds16(xbase + (int64_t)s * ldx + cc * 8, smem + RX + slot * XT + (wave * XI + i) * 1024);
    }
  };
#pragma unroll
  for (int k = 0; k < DEPTH - 1; ++k) {
    if (k < nk) issue_tile(k);
  }

  __syncthreads();  // sa, sd
  for (int idx = tid; idx < NLT * Q; idx += NT) {
    const int j = idx / Q;
    const int s = idx - j * Q;
    if (s < 32 * j) vt[j][s] = __expf(sa[32 * j] - sa[s]) * sd[s];
  }
  const float al1 = sa[l1], al2 = sa[l2];
  const float u1 = __expf(al1 - sa[32 * j1]);  // <= 1: exp(acum_l - acum at the tile's start)
  const float u2 = __expf(al2 - sa[32 * j2]);
  const float Dh = Dv ? Dv[h / hr] : 0.f;

  f32x16 acc1[TP], acc2[TP];
#pragma unroll
  for (int t = 0; t < TP; ++t) {
    acc1[t] = f32x16{};
    acc2[t] = f32x16{};
  }

  auto scale_rows = [&](f32x16 (&acc)[TP], float u) {
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[t] *= u;
  };
  // Z = B_k C_j^T (8 chained MFMAs); B rows from the ring slot
  auto tile_z = [&](const u32x4 (&creg)[KN], int slot) {
    const unsigned char *bt = smem + RB + slot * BT + col * (N * 2);
    f32x16 z = f32x16{};
#pragma unroll
    for (int q = 0; q < KN; ++q) {
      const int cc = (2 * q + kg) ^ chunk_swz(col, NCB);
      const u32x4 b = *reinterpret_cast<const u32x4 *>(bt + cc * 16);
      z = mfma32x32x16(as_bf16x8(b), as_bf16x8(creg[q]), z);
    }
    return z;
  };
  auto g_off = [&](const u32x4 (&creg)[KN], int j, int k, u32x4 &g0, u32x4 &g1) {
    const f32x16 z = tile_z(creg, k % DEPTH);
    float gv[16];
    decay_offdiag_v(z, &vt[j][32 * k], kg, gv);
    pack_g(gv, g0, g1);
  };
  auto g_diag = [&](const u32x4 (&creg)[KN], int l, float al, int k, u32x4 &g0, u32x4 &g1) {
    const f32x16 z = tile_z(creg, k % DEPTH);
    float gv[16];
    decay_diag(z, al, l, 32 * k, kg, sa, sd, gv);
    pack_g(gv, g0, g1);
  };
  // X^T operands of source tile k straight from the row-major x tile by a
  // transposing LDS read: lane (group gq = lane/16, d = lane%16) addresses
  // token row sb + d/4, columns 4(d%4).., and receives p = 16(gq%2) + d of
  // tokens sb .. sb+3.  sb follows the accumulator row order of G.
  auto x_ops = [&](int k, int t, u32x4 &xa, u32x4 &xb) {
    const unsigned char *xtile = smem + RX + (k % DEPTH) * XT;
    const int gq = lane >> 4, d = lane & 15;
    const int p0 = t * 32 + 16 * (gq & 1) + 4 * (d & 3);
    u32x2 part[4];
#pragma unroll
    for (int h4 = 0; h4 < 4; ++h4) {  // s offsets 4kg, 8+4kg, 16+4kg, 24+4kg
      const int row = 8 * h4 + 4 * kg + (d >> 2);
      const int cc = (p0 >> 3) ^ chunk_swz(row, NCX);
      part[h4] = lds_read_tr16(xtile + row * (P * 2) + cc * 16 + (p0 & 7) * 2);
    }
    xa = u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
    xb = u32x4{part[2].x, part[2].y, part[3].x, part[3].y};
  };
  auto xg_one = [&](f32x16 (&acc)[TP], int k, const u32x4 &g0, const u32x4 &g1) {
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      u32x4 xa, xb;
      x_ops(k, t, xa, xb);
      acc[t] = mfma32x32x16(as_bf16x8(xa), as_bf16x8(g0), acc[t]);
      acc[t] = mfma32x32x16(as_bf16x8(xb), as_bf16x8(g1), acc[t]);
    }
  };
  auto xg_two = [&](int k, const u32x4 &g10, const u32x4 &g11, const u32x4 &g20,
                    const u32x4 &g21) {
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      u32x4 xa, xb;
      x_ops(k, t, xa, xb);
      acc1[t] = mfma32x32x16(as_bf16x8(xa), as_bf16x8(g10), acc1[t]);
      acc2[t] = mfma32x32x16(as_bf16x8(xa), as_bf16x8(g20), acc2[t]);
      acc1[t] = mfma32x32x16(as_bf16x8(xb), as_bf16x8(g11), acc1[t]);
      acc2[t] = mfma32x32x16(as_bf16x8(xb), as_bf16x8(g21), acc2[t]);
    }
  };
  // skip term D x_l in fp32 at the token tile's diagonal step: the lane's
  // accumulator rows p = 32t + 8rb + 4kg + e of column l are 4 consecutive
  // elements of x row l, one 8-byte LDS read each
  auto add_skip = [&](f32x16 (&acc)[TP], int k) {
    const unsigned char *xtile = smem + RX + (k % DEPTH) * XT;
#pragma unroll
    for (int t = 0; t < TP; ++t) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int p = t * 32 + rb * 8 + kg * 4;
        const int cc = (p >> 3) ^ chunk_swz(col, NCX);
        const u32x2 xv = *reinterpret_cast<const u32x2 *>(xtile + col * (P * 2) + cc * 16 + (p & 7) * 2);
        acc[t][rb * 4 + 0] += Dh * bf16lo(xv.x);
        acc[t][rb * 4 + 1] += Dh * bf16hi(xv.x);
        acc[t][rb * 4 + 2] += Dh * bf16lo(xv.y);
        acc[t][rb * 4 + 3] += Dh * bf16hi(xv.y);
      }
    }
  };
  // top of step k: this thread's loads of tile k are done (the loads of the
  // tiles issued after it may stay in flight), then the whole block is
  // (everyone's tile k landed, everyone left step k-1), then tile k+DEPTH-1
  // goes into the slot step k-1 used
  auto begin_step = [&](int k) {
    const int after = min(DEPTH - 2, nk - 1 - k);
    if (after >= 2) {
      wait_vmcnt<2 * LPT>();
    } else if (after == 1) {
      wait_vmcnt<LPT>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (k + DEPTH - 1 < nk) issue_tile(k + DEPTH - 1);
  };
  static_assert(DEPTH <= 4, "begin_step waits for at most two later tiles");

  // ---- intra-chunk term: source tiles in lockstep, in phases uniform per
  // wavefront (j1 < j2): both tiles off-diagonal, tile 1 on its diagonal,
  // tile 2 alone off-diagonal, tile 2 on its diagonal, then idle.  Each
  // token tile accumulates u_l-free until its diagonal step multiplies by u_l.
  int k = 0;
  if (act2) {
#pragma unroll 1
    for (; k < j1; ++k) {
      begin_step(k);
      u32x4 g10, g11, g20, g21;
      g_off(c1, j1, k, g10, g11);
      g_off(c2, j2, k, g20, g21);
      xg_two(k, g10, g11, g20, g21);
    }
    {  // k == j1
      begin_step(k);
      u32x4 g10, g11, g20, g21;
      g_diag(c1, l1, al1, k, g10, g11);
      g_off(c2, j2, k, g20, g21);
      scale_rows(acc1, u1);
      add_skip(acc1, k);
      xg_two(k, g10, g11, g20, g21);
      ++k;
    }
#pragma unroll 1
    for (; k < j2; ++k) {
      begin_step(k);
      u32x4 g0, g1;
      g_off(c2, j2, k, g0, g1);
      xg_one(acc2, k, g0, g1);
    }
    {  // k == j2
      begin_step(k);
      u32x4 g0, g1;
      g_diag(c2, l2, al2, k, g0, g1);
      scale_rows(acc2, u2);
      add_skip(acc2, k);
      xg_one(acc2, k, g0, g1);
      ++k;
    }
  } else if (act1) {
#pragma unroll 1
    for (; k < j1; ++k) {
      begin_step(k);
      u32x4 g0, g1;
      g_off(c1, j1, k, g0, g1);
      xg_one(acc1, k, g0, g1);
    }
    {  // k == j1
      begin_step(k);
      u32x4 g0, g1;
      g_diag(c1, l1, al1, k, g0, g1);
      scale_rows(acc1, u1);
      add_skip(acc1, k);
      xg_one(acc1, k, g0, g1);
      ++k;
    }
  }
#pragma unroll 1
  for (; k < nk; ++k) begin_step(k);
  __syncthreads();  // every wavefront is done with the rings

  // ---- inter-chunk term, added last: exp(acum_l) C_l hprev^T (hprev landed
  // before tile 0 did)
  auto add_inter = [&](f32x16 (&acc)[TP], const u32x4 (&creg)[KN], float al) {
    const float el = __expf(al);
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const int row = t * 32 + col;
      const unsigned char *hrow = smem + HS + row * (N * 2);
      f32x16 v = f32x16{};
#pragma unroll
      for (int q = 0; q < KN; ++q) {
        const int cc = (2 * q + kg) ^ chunk_swz(row, NCB);
        const u32x4 a = *reinterpret_cast<const u32x4 *>(hrow + cc * 16);
        v = mfma32x32x16(as_bf16x8(a), as_bf16x8(creg[q]), v);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] += el * v[r];
    }
  };
  if (act1) add_inter(acc1, c1, al1);
  if (act2) add_inter(acc2, c2, al2);
  __syncthreads();  // hprev consumed: all of smem becomes output staging

  // ---- epilogue: each wave stages its token tiles through its own LDS slice
  // as fp32 [token][p], rounds, and stores 16-byte row segments
  float(*yb)[LYB] = reinterpret_cast<float(*)[LYB]>(smem + wave * 32 * LYB * 4);
  auto epilogue = [&](const f32x16 (&acc)[TP], int j) {
#pragma unroll
    for (int t = 0; t < TP; ++t) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 v{acc[t][rb * 4 + 0], acc[t][rb * 4 + 1], acc[t][rb * 4 + 2], acc[t][rb * 4 + 3]};
        *reinterpret_cast<f32x4 *>(&yb[col][t * 32 + rb * 8 + kg * 4]) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int G8 = P / 8;
#pragma unroll
    for (int it = lane; it < 32 * G8; it += 64) {
      const int r = it / G8;
      const int gp = it - r * G8;
      const int l = j * 32 + r;
      if (l < ci.len) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(&yb[r][gp * 8]);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(&yb[r][gp * 8 + 4]);
        u32x4 o;
        o.x = pack_bf16x2(v0.x, v0.y);
        o.y = pack_bf16x2(v0.z, v0.w);
        o.z = pack_bf16x2(v1.x, v1.y);
        o.w = pack_bf16x2(v1.z, v1.w);
        *reinterpret_cast<u32x4 *>(y + (ci.t0 + l) * ldx + (int64_t)h * P + gp * 8) = o;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (act1) epilogue(acc1, j1);
  if (act2) epilogue(acc2, j2);
}

// ============================================================ head-batched kernel
// Q = 256, P = 64, N <= 128.  The heads of a group share B and C, so Z = B C^T
// of a chunk is the same for all of them: block = (chunk, group, run of hb
// heads), one block of 8 wavefronts per CU.  Each wavefront owns one token
// tile: wavefront w < 4 tile w, wavefront w >= 4 tile 11-w, so tiles j and 7-j
// share a SIMD.  The causal work is balanced by handing pairs over: wavefront
// s < 4 also forms the off-diagonal pairs (7-s, i < 4-s) and passes their sum
// to the owner of tile 7-s through LDS, so every wavefront has 3 or 4
// off-diagonal pairs and one diagonal pair.  Its five Z tiles (pairs formed
// once per block from the chunk's B staged in LDS) and the C rows of its tile
// stay in registers.  The block then walks its heads; x, acum, dt and hprev
// of head i+1 stream into the other half of two-slot LDS rings while head i
// computes, and y of head i, staged over its x as bf16, goes out at the top of
// head i+1 in 128-byte row segments.  Per head:
//   1. y of the previous head is stored; the v table of this head is built;
//   2. the next head's loads go out;
//   3. handed-over pairs (wavefronts 0-3), summed and written to LDS;
//   4. inter term Y^T = exp(acum at the tile's first token) Hprev C^T, then
//      the tile's own off-diagonal pairs;
//   5. (barrier) the handed-over sum is added, u_l applied, then the diagonal
//      pair and the skip term;
//   6. (barrier) the tile is rounded to bf16 and staged over this head's x.
template <int N>
__global__ __launch_bounds__(512, 1) void k_chunk_scan_hb(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ Dv, const float *__restrict__ acum,
    const float *__restrict__ dtq, const uint16_t *__restrict__ hprev, ChunkGeom geom, int nc,
    int H, int G, int hb, int nkb, int hr, uint16_t *__restrict__ y) {
  constexpr int Q = 256, P = 64;
  static_assert(N == 64 || N == 128 || N == 256, "head-batched tile shape");
  // N 256: B is staged in two 128-column halves for the Z phase, and hprev
  // has one LDS slot (loaded once the previous head's inter term is done)
  constexpr int NH = N > 128 ? 2 : 1;  // B halves
  constexpr int NBH = N / NH;          // columns of a staged B half
  constexpr int NCBH = NBH / 8;        // its 16-byte chunks per row
  constexpr int HSL = N > 128 ? 1 : 2; // hprev slots
  constexpr int NT = 512;             // threads
  constexpr int NW = 8;               // wavefronts
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
  constexpr int VT = AD1 + ADB, PS = VT + NLT * Q * 4, TOTAL = PS + 4 * PSB;
  static_assert(2 * XB >= BB, "B staging fits over the x ring");
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
  const int s4 = wave & 3;
  const bool donor = wave < 4;
  const int T = donor ? s4 : NLT - 1 - s4;  // own token tile
  const int TD = NLT - 1 - s4;              // tile of the handed-over pairs
  const int nd = donor ? 4 - s4 : 0;        // handed-over pairs: source tiles 0 .. nd-1 of TD
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
    if (wave < 2)  // wavefront 0: acum, 1: dt
      load_lds16((wave == 0 ? acum : dtq) + ch * Q + lane * 4, smem + (slot ? AD1 : AD0) + wave * 1024);
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
  f32x16 z[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) z[k] = f32x16{};
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
    // slot k < 4: handed-over pair (TD, k) for k < nd, else own off-diagonal
    // pair (T, k - nd) on a donor and (T, T - 3 + k) on a receiver (k = 3 unused
    // there); slot 4: the diagonal pair (T, T).  Operands are picked by value,
    // with no branches, so each tile is formed in the registers it stays in.
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const bool dk = k < nd;
      const int zi = k == 4 ? T : (donor ? (dk ? k : k - nd) : min(T - 3 + k, T));
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
      for (int k = 0; k < 4; ++k) {
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
    for (int k = 0; k < 4; ++k) {
      const bool own = donor ? k >= nd : k < 3;
      if (own) {
        const int i = donor ? k - nd : T - 3 + k;
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
      decay_diag(z[4], al, l, 32 * T, kg, sa, sd, gv);
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
  const dim3 grid(xcd_grid(geo.nc_max, geo.H));
  if constexpr (Q == 256 && P == 64) {
    int nkb = 1;
    const int hb = pick_heads_per_block(geo.nc_max, geo.H, geo.G, device_cus(), 1.5, nkb);
    hipLaunchKernelGGL((k_chunk_scan_hb<N>), dim3(xcd_grid(geo.nc_max, geo.G * nkb)), dim3(512), 0,
                       stream, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                       static_cast<const uint16_t *>(C), D, acum, dtq,
                       static_cast<const uint16_t *>(hprev), cg, (int)geo.nc_max, geo.H, geo.G, hb,
                       nkb, geo.hr, static_cast<uint16_t *>(y));
  } else {
    hipLaunchKernelGGL((k_chunk_scan_lds<Q, P, N>), grid, dim3(Q), 0, stream,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                       static_cast<const uint16_t *>(C), D, acum, dtq,
                       static_cast<const uint16_t *>(hprev), cg, (int)geo.nc_max, geo.H, geo.G,
                       geo.hr, static_cast<uint16_t *>(y));
  }
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
