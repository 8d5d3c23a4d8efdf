// libssd: the whole SSD forward in one pass per (sequence, head), the state
// kept on chip across chunks (the blockwise evaluation of page "Mamba-2
// Architecture: State Space Duality Explained", "2. The Chunked SSD
// Algorithm", with the three chunk-level steps -- chunk state, hand-off,
// output -- done back to back for each chunk instead of as separate passes
// over all chunks).  Chunking is exact, so the chunk length is a free choice:
// this kernel walks 32-token chunks, for which the intra-chunk product is one
// 32 x 32 causal tile.
//
// Design.  Block = (sequence, two heads of one group) in XCD-aware order (all
// heads of a sequence on one XCD, so its B and C rows come from one L2), 4
// wavefronts: wavefront (head hh, half ph) owns state rows p in
// [32 ph, 32 ph + 32) of head hh, held transposed (h^T, rows n, columns p) as
// 2 x N/16 fp32 tiles of the 16x16x32 bf16 MFMA.  The two heads share their B
// and C tiles in LDS.
//
// Data movement.  A three-slot LDS ring per block holds chunk k's x (each
// wavefront's own 32 x 32 slice), B, C and dt (each wavefront's head) while
// chunk k + 2 is in flight (direct-to-LDS loads).  Vector-memory operations
// complete in issue order, so a wavefront knows chunk k has landed once at
// most the operations it issued after that chunk are pending; it waits for
// exactly that count, then one barrier per chunk publishes the tiles.  y of a
// chunk is staged (bf16) in the wavefront's own x slice of that chunk and
// stored in 16-byte row segments at the next chunk's top, before that slot is
// refilled.  No workspace: nothing but x, B, C, dt and y crosses HBM.
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

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int N>
__global__ __launch_bounds__(256, N == 64 ? 3 : 2) void k_ssd_fused(
    const uint16_t *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
    const float *__restrict__ h0, const int32_t *__restrict__ cu, int64_t L, int64_t T, int rows,
    int H, int G, uint16_t *__restrict__ y, float *__restrict__ hfin) {
  constexpr int P = 64, CQ = 32;
  constexpr int NT = N / 16;   // state tiles per p-tile (over n)
  constexpr int KQ = N / 32;   // K steps over n
  constexpr int NCB = N / 8;   // 16-byte chunks per B / C row
  constexpr int XW = CQ * 32 * 2;            // a wavefront's x slice of a chunk: 32 tokens x 32 p
  constexpr int BT = CQ * N * 2;             // B (or C) of a chunk
  constexpr int DW = 64 * 4;                 // a wavefront's dt of a chunk (lanes 32..63 repeat)
  constexpr int OX = 0, OB = 4 * XW, OC = OB + BT, OD = OC + BT;
  constexpr int SLOT = OD + 4 * DW;
  constexpr int AD = 3 * SLOT;               // per wavefront: [al2 | bs2 | w], 32 floats each
  constexpr int ADW = 3 * CQ * 4;
  constexpr int TOTAL = AD + 4 * ADW;
  constexpr int BCI = 2 * BT / 1024 / 4;     // 1 KB pieces of B and C per wavefront
  constexpr int LDC = 2 + BCI + 1;           // vector-memory ops a wavefront issues per chunk load
  constexpr int STC = 2;                     // ... per chunk of y it stores
  static_assert(BCI * 4 * 1024 == 2 * BT, "B and C split evenly over 4 wavefronts");
  static_assert(TOTAL <= 160 * 1024 / (N == 64 ? 3 : 2), "blocks per CU");
  __shared__ __align__(16) unsigned char smem[TOTAL];

  int s, pr;
  xcd_chunk_head(H >> 1, s, pr);
  if (s >= rows) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int hh = wave >> 1, ph = wave & 1;
  const int h = 2 * pr + hh;
  const int g = (2 * pr) / (H / G);
  int64_t tb, len;
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
  const int64_t sh = (int64_t)s * H + h;
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const float Ah = A[h];
  const float Dh = Dv ? Dv[h] : 0.f;
  float *adw = reinterpret_cast<float *>(smem + AD + wave * ADW);

  // state h^T: hst[pt][j] holds rows n = 16 j + 4 g4 + r, column
  // p = 32 ph + 16 pt + c16
  f32x4 hst[2][NT];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    const int64_t prow = (sh * P + 32 * ph + 16 * pt + c16) * N + 4 * g4;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      hst[pt][j] = h0 ? *reinterpret_cast<const f32x4 *>(h0 + prow + 16 * j) : f32x4{};
  }
  const int nck = static_cast<int>((len + CQ - 1) / CQ);

  // chunk k's loads into ring slot sl: LDC vector-memory ops per wavefront
  auto issue = [&](int k, int sl) {
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;
    const uint32_t base = lds_off(smem) + sl * SLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // this wavefront's x slice: 32 rows of 4 chunks
      const int m = i * 64 + lane, r = m >> 2, cc = (m & 3) ^ chunk_swz(r, 4);
      dma_lds16(x + (t0 + min(r, last)) * ldx + (int64_t)h * P + 32 * ph + 8 * cc,
                base + OX + wave * XW + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {  // B and C pieces
      const int u = wave * BCI + i, tile = u / (BT / 1024), pi = u % (BT / 1024);
      const int m = pi * 64 + lane, r = m / NCB, cc = (m % NCB) ^ chunk_swz(r, NCB);
      dma_lds16((tile ? Cm : Bm) + (t0 + min(r, last)) * ldb + (int64_t)g * N + 8 * cc,
                base + (tile ? OC : OB) + pi * 1024);
    }
    // dt of this wavefront's head, 4 bytes a lane
    dma_lds4(dt + (t0 + min(lane & 31, last)) * H + h, base + OD + wave * DW);
  };
  // y of chunk k from its staging (the wavefront's x slice of slot sl): STC stores
  auto store_y = [&](int k, int sl) {
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int rem = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ));
    const unsigned char *ys = smem + sl * SLOT + OX + wave * XW;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = i * 64 + lane, r = m >> 2, cc = m & 3;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(ys + r * 64 + ((cc ^ chunk_swz(r, 4)) << 4));
      if (r < rem)
        *reinterpret_cast<u32x4 *>(y + (t0 + r) * ldx + (int64_t)h * P + 32 * ph + 8 * cc) = v;
    }
  };
  // row operand of a B or C tile in the state's K order: K step q covers
  // n = 32q + 4 g4 + {0..3} and 32q + 16 + 4 g4 + {0..3}
  auto row_op = [&](const unsigned char *tile, int row, int q) {
    const unsigned char *rp = tile + row * (N * 2);
    const int sw = chunk_swz(row, NCB);
    const int c0 = 4 * q + (g4 >> 1), off = 8 * (g4 & 1);
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(rp + ((c0 ^ sw) << 4) + off);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(rp + (((c0 + 2) ^ sw) << 4) + off);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };
  // transposing read of 4 token rows row0 + {0..3} at column col0 + c16 of a
  // row-major tile (ncc chunks a row, row bytes rb)
  auto tr4 = [&](const unsigned char *tile, int rb, int ncc, int row0, int col0) {
    const int row = row0 + (c16 >> 2), col = col0 + 4 * (c16 & 3);
    const int cc = (col >> 3) ^ chunk_swz(row, ncc);
    return lds_read_tr16(tile + row * rb + (cc << 4) + (col & 7) * 2);
  };

  if (nck > 0) issue(0, 0);
  if (nck > 1) issue(1, 1);
  int sl = 0;
#pragma unroll 1
  for (int k = 0; k < nck; ++k) {
    // chunk k has landed once at most the later ops of this wavefront are
    // pending: the y stores of iteration k-1 (k >= 2) and chunk k+1's loads
    const bool more = k + 1 < nck;
    if (k >= 2) {
      if (more) wait_vmcnt<STC + LDC>(); else wait_vmcnt<STC>();
    } else {
      if (more) wait_vmcnt<LDC>(); else wait_vmcnt<0>();
    }
    __syncthreads();  // every wavefront's share of chunk k is in; chunk k-1 is done everywhere
    const int slp = sl == 0 ? 2 : sl - 1;  // slot of chunk k-1, and of chunk k+2
    if (k >= 1) store_y(k - 1, slp);
    if (k + 2 < nck) issue(k + 2, slp);

    unsigned char *xs = smem + sl * SLOT + OX + wave * XW;
    const unsigned char *bs = smem + sl * SLOT + OB;
    const unsigned char *cs = smem + sl * SLOT + OC;
    const float *dts = reinterpret_cast<const float *>(smem + sl * SLOT + OD + wave * DW);
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;

    // cumulative decay (lanes l and 32 + l hold token l) and per-token tables
    const int tl = lane & 31;
    const float dtv = tl <= last ? dts[lane] : 0.f;
    const float a = scan32(dtv * Ah);
    const float alast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 31));
    if (lane < 32) {
      const float al = a * kLog2e;
      adw[tl] = al;                                            // log2 exp(a_l)
      adw[CQ + tl] = __builtin_amdgcn_logf(dtv) - al;          // log2(dt_s exp(-a_s))
      adw[2 * CQ + tl] = exp2_fast((alast - a) * kLog2e) * dtv;  // w_s
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
    const float f0 = exp2_fast(al0), f1 = exp2_fast(al1);
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
      const u32x2 t0 = tr4(xs, 64, 4, 4 * g4, 16 * pt), t1 = tr4(xs, 64, 4, 16 + 4 * g4, 16 * pt);
      xop[pt] = u32x4{t0.x, t0.y, t1.x, t1.y};
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) ya[pt][lt] = mfma16(xop[pt], gop[lt], ya[pt][lt]);
    }
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {  // D x: rows p = 16 pt + 4 g4 + r of token l
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) {
        const int l = 16 * lt + c16, col = 16 * pt + 4 * g4;
        const u32x2 v = *reinterpret_cast<const u32x2 *>(
            xs + l * 64 + (((col >> 3) ^ chunk_swz(l, 4)) << 4) + (col & 7) * 2);
        ya[pt][lt].x += Dh * bf16lo(v.x);
        ya[pt][lt].y += Dh * bf16hi(v.x);
        ya[pt][lt].z += Dh * bf16lo(v.y);
        ya[pt][lt].w += Dh * bf16hi(v.y);
      }
    }

    // 3. state: h^T = exp(a_last) h^T + B^T (w x)
    {
      const float e = exp2_fast(alast * kLog2e);
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
#pragma unroll
        for (int j = 0; j < NT; ++j) hst[pt][j] *= e;
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x2 t0 = tr4(bs, N * 2, NCB, 4 * g4, 16 * j), t1 = tr4(bs, N * 2, NCB, 16 + 4 * g4, 16 * j);
        const u32x4 bt{t0.x, t0.y, t1.x, t1.y};
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) hst[pt][j] = mfma16(bt, xw[pt], hst[pt][j]);
      }
    }

    // y staged (bf16) in this wavefront's x slice, now fully read
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int lt = 0; lt < 2; ++lt) {
        const int l = 16 * lt + c16, col = 16 * pt + 4 * g4;
        const u32x2 o{pack_bf16x2(ya[pt][lt].x, ya[pt][lt].y), pack_bf16x2(ya[pt][lt].z, ya[pt][lt].w)};
        *reinterpret_cast<u32x2 *>(xs + l * 64 + (((col >> 3) ^ chunk_swz(l, 4)) << 4) + (col & 7) * 2) = o;
      }
    }
    sl = sl == 2 ? 0 : sl + 1;
  }
  if (nck > 0) {
    wave_sync();
    store_y(nck - 1, (nck - 1) % 3);
  }
  if (hfin) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int64_t prow = (sh * P + 32 * ph + 16 * pt + c16) * N + 4 * g4;
#pragma unroll
      for (int j = 0; j < NT; ++j) *reinterpret_cast<f32x4 *>(hfin + prow + 16 * j) = hst[pt][j];
    }
  }
}

}  // namespace

bool fused_supported(int H, int P, int N, int G) {
  return P == 64 && (N == 64 || N == 128) && (H / G) % 2 == 0;
}

hipError_t launch_fused(const void *x, const float *dt, const float *A, const void *B, const void *C,
                        const float *D, const float *h0, const int32_t *cu, int64_t L, int64_t T,
                        int rows, int H, int P, int N, int G, void *y, float *hfin,
                        hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!fused_supported(H, P, N, G)) return hipErrorInvalidValue;
  const dim3 grid(xcd_grid(rows, H / 2));
  const uint16_t *xi = static_cast<const uint16_t *>(x);
  const uint16_t *bi = static_cast<const uint16_t *>(B);
  const uint16_t *ci = static_cast<const uint16_t *>(C);
  uint16_t *yo = static_cast<uint16_t *>(y);
  if (N == 64)
    hipLaunchKernelGGL(k_ssd_fused<64>, grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, h0, cu, L,
                       T, rows, H, G, yo, hfin);
  else
    hipLaunchKernelGGL(k_ssd_fused<128>, grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, h0, cu,
                       L, T, rows, H, G, yo, hfin);
  return hipGetLastError();
}

}  // namespace ssd
