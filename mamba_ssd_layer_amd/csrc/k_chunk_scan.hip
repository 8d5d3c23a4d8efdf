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
// Design (per block = (chunk, head), Q/64 wavefronts).  The output is formed
// transposed, Y^T [P x Q], as 32x32 MFMA tiles (M = p, N = l):
//   * wavefront w owns the token tiles w and Q/32-1-w (balanced causal work);
//   * for its token tile it keeps the C rows as MFMA B-operands in registers;
//   * inter term: Y^T += Hprev . C^T over K = n (Hprev read as bf16 A-operands),
//     then each lane scales by exp(acum_l) -- one factor per lane because a lane
//     owns one output column l;
//   * intra term, for every source tile s <= l: Z = B_s . C^T over K = n on MFMA,
//     then the decay mask is applied to Z in registers (masking before the exp
//     argument can overflow), the fp32 accumulator is rounded to bf16 and used
//     directly as the B-operand of Y^T += X^T . G^T: the K-order of that MFMA
//     is permuted to the accumulator's row order, and X^T is read from LDS in
//     the same order, so no cross-lane shuffle is needed;
//   * X^T for the whole chunk is staged once in LDS (transposed on the way in).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

template <int Q, int P, int N>
__global__ __launch_bounds__(Q) void k_chunk_scan_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm,
    const uint16_t *__restrict__ Cm, const float *__restrict__ Dv, const float *__restrict__ acum,
    const float *__restrict__ dtq, const uint16_t *__restrict__ hprev, ChunkGeom geom, int H,
    int G, uint16_t *__restrict__ y) {
  static_assert(P % 32 == 0 && N % 16 == 0 && Q % 64 == 0, "tile shape");
  constexpr int NT = Q;          // threads
  constexpr int NLT = Q / 32;    // token tiles
  constexpr int TP = P / 32;     // p tiles
  constexpr int KN = N / 16;     // K steps over n
  constexpr int LDX = Q + 4;     // padded LDS row of X^T (bf16 elements)

  __shared__ __align__(16) uint16_t xt[P][LDX];
  __shared__ float sa[Q];
  __shared__ float sd[Q];

  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int g = h / (H / G);
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;
  const int64_t ch = (int64_t)c * H + h;

  // ---- stage acum, dt and X^T
  for (int l = threadIdx.x; l < Q; l += NT) {
    sa[l] = acum[ch * Q + l];
    sd[l] = dtq[ch * Q + l];
  }
  const int64_t ldx = (int64_t)H * P;
  const uint16_t *xbase = x + ci.t0 * ldx + (int64_t)h * P;
  {
    constexpr int RQ = Q / 4;
    constexpr int UNITS = RQ * (P / 8);
    for (int u = threadIdx.x; u < UNITS; u += NT) {
      const int rq = u % RQ;
      const int cb = u / RQ;
      const int l0 = rq * 4;
      u32x4 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (l0 + i < ci.len) {
          r[i] = *reinterpret_cast<const u32x4 *>(xbase + (int64_t)(l0 + i) * ldx + cb * 8);
        } else {
          r[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x2 lo, hi;
        lo.x = pair_lo(r[0][m], r[1][m]);
        lo.y = pair_lo(r[2][m], r[3][m]);
        hi.x = pair_hi(r[0][m], r[1][m]);
        hi.y = pair_hi(r[2][m], r[3][m]);
        *reinterpret_cast<u32x2 *>(&xt[cb * 8 + 2 * m][l0]) = lo;
        *reinterpret_cast<u32x2 *>(&xt[cb * 8 + 2 * m + 1][l0]) = hi;
      }
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int kg = lane >> 5;
  const float Dh = Dv ? Dv[h] : 0.f;
  const uint16_t *hp = hprev + ch * (int64_t)P * N;
  const int64_t ldb = (int64_t)G * N;
  const uint16_t *bbase = Bm + ci.t0 * ldb + (int64_t)g * N;
  const uint16_t *cbase = Cm + ci.t0 * ldb + (int64_t)g * N;

#pragma unroll 1
  for (int jj = 0; jj < 2; ++jj) {
    const int j = jj == 0 ? wave : NLT - 1 - wave;
    const int l = j * 32 + col;
    const bool lvalid = l < ci.len;

    // C rows of this token tile as B-operands: lane holds C[l][16q + 8kg .. +8]
    u32x4 creg[KN];
#pragma unroll
    for (int q = 0; q < KN; ++q) {
      creg[q] = lvalid ? *reinterpret_cast<const u32x4 *>(cbase + (int64_t)l * ldb + q * 16 + kg * 8)
                       : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 acc[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[t] = f32x16{};

    // ---- inter-chunk term: Y^T[p][l] = sum_n Hprev[p][n] C[l][n]
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const uint16_t *hrow = hp + (int64_t)(t * 32 + col) * N + kg * 8;
#pragma unroll
      for (int q = 0; q < KN; ++q) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(hrow + q * 16);
        acc[t] = mfma32x32x16(as_bf16x8(a), as_bf16x8(creg[q]), acc[t]);
      }
    }
    const float al = sa[l];
    const float el = __expf(al);
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[t] *= el;

    // ---- intra-chunk term over source tiles k <= j
#pragma unroll 1
    for (int k = 0; k <= j; ++k) {
      const int s0 = k * 32;
      const bool svalid = s0 + col < ci.len;
      const uint16_t *brow = bbase + (int64_t)(s0 + col) * ldb + kg * 8;
      f32x16 z = f32x16{};
#pragma unroll
      for (int q = 0; q < KN; ++q) {
        const u32x4 b = svalid ? *reinterpret_cast<const u32x4 *>(brow + q * 16)
                               : u32x4{0u, 0u, 0u, 0u};
        z = mfma32x32x16(as_bf16x8(b), as_bf16x8(creg[q]), z);
      }
      // z[r] = Z[s = s0 + acc_row(r, kg)][l] = C_l . B_s ; apply the decay mask
      float gv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s = s0 + acc_row(r, kg);
        const bool keep = (k < j) || (s <= l);
        const float arg = keep ? (al - sa[s]) : -__builtin_inff();
        const float v = z[r] * __expf(arg) * sd[s];
        gv[r] = keep ? v : 0.f;
      }
      u32x4 g0, g1;
      g0.x = pack_bf16x2(gv[0], gv[1]);
      g0.y = pack_bf16x2(gv[2], gv[3]);
      g0.z = pack_bf16x2(gv[4], gv[5]);
      g0.w = pack_bf16x2(gv[6], gv[7]);
      g1.x = pack_bf16x2(gv[8], gv[9]);
      g1.y = pack_bf16x2(gv[10], gv[11]);
      g1.z = pack_bf16x2(gv[12], gv[13]);
      g1.w = pack_bf16x2(gv[14], gv[15]);
      // X^T operands in the same K order: MFMA 0 covers s-offsets
      // {4kg..4kg+3, 8+4kg..8+4kg+3}, MFMA 1 the same plus 16.
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        const uint16_t *xr = &xt[t * 32 + col][s0 + 4 * kg];
        const u32x2 a0 = *reinterpret_cast<const u32x2 *>(xr);
        const u32x2 a1 = *reinterpret_cast<const u32x2 *>(xr + 8);
        const u32x2 b0 = *reinterpret_cast<const u32x2 *>(xr + 16);
        const u32x2 b1 = *reinterpret_cast<const u32x2 *>(xr + 24);
        const u32x4 xa{a0.x, a0.y, a1.x, a1.y};
        const u32x4 xb{b0.x, b0.y, b1.x, b1.y};
        acc[t] = mfma32x32x16(as_bf16x8(xa), as_bf16x8(g0), acc[t]);
        acc[t] = mfma32x32x16(as_bf16x8(xb), as_bf16x8(g1), acc[t]);
      }
    }

    // ---- epilogue: + D x_l, round to bf16, store y[t0 + l][h][p]
    if (lvalid) {
      const uint16_t *xrow = xbase + (int64_t)l * ldx;
      uint16_t *yrow = y + (ci.t0 + l) * ldx + (int64_t)h * P;
#pragma unroll
      for (int t = 0; t < TP; ++t) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int p = t * 32 + rb * 8 + kg * 4;
          const u32x2 xv = *reinterpret_cast<const u32x2 *>(xrow + p);
          const float v0 = acc[t][rb * 4 + 0] + Dh * bf16lo(xv.x);
          const float v1 = acc[t][rb * 4 + 1] + Dh * bf16hi(xv.x);
          const float v2 = acc[t][rb * 4 + 2] + Dh * bf16lo(xv.y);
          const float v3 = acc[t][rb * 4 + 3] + Dh * bf16hi(xv.y);
          u32x2 o;
          o.x = pack_bf16x2(v0, v1);
          o.y = pack_bf16x2(v2, v3);
          *reinterpret_cast<u32x2 *>(yrow + p) = o;
        }
      }
    }
  }
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
  hipLaunchKernelGGL((k_chunk_scan_bf16<Q, P, N>), dim3((unsigned)geo.nc_max, (unsigned)geo.H),
                     dim3(Q), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint16_t *>(B), static_cast<const uint16_t *>(C), D, acum,
                     dtq, static_cast<const uint16_t *>(hprev), cg, geo.H, geo.G,
                     static_cast<uint16_t *>(y));
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
