// libssd: the whole SSD forward in one pass per (sequence, head), the state
// kept on chip across chunks (the blockwise evaluation of page "Mamba-2
// Architecture: State Space Duality Explained", "2. The Chunked SSD
// Algorithm", with the three chunk-level steps -- chunk state, hand-off,
// output -- done back to back for each chunk instead of as separate passes
// over all chunks).  Chunking is exact, so the chunk length is a free choice:
// this kernel walks 32-token chunks (one MFMA tile), for which the intra-chunk
// product is a single diagonal tile.
//
// Design.  Block = (sequence, head) in XCD-aware order (all heads of a
// sequence on one XCD, so its B and C rows are read from one L2), 2
// wavefronts; wavefront w owns rows p in [32w, 32w + 32) of the P x N state,
// held transposed (h^T, rows n, columns p) as N/32 fp32 MFMA accumulator
// tiles.  Per 32-token chunk, with the next chunk's x and B arriving in the
// other half of a two-slot LDS ring (direct-to-LDS loads) and its C rows and
// dt in registers:
//   1. acum_l = inclusive cumulative sum of dt A over the chunk (a wavefront
//      scan), and the weights w_l = exp(acum_last - acum_l) dt_l;
//   2. inter term: Y^T = exp(acum_l) Hprev . C^T on MFMA, the A-operand being
//      the state registers rounded to bf16 (their row order is the K order;
//      C is read in the same order);
//   3. intra term: Z^T = B . C^T on MFMA (same K order), the causal decay
//      mask exp(acum_l - acum_s) dt_s applied in registers (masked before the
//      exponent), then Y^T += X^T . G^T with the accumulator as the B-operand
//      (X^T from transposing LDS reads in the accumulator's row order); plus
//      D x in fp32;
//   4. state: h^T = exp(acum_last) h^T + B^T . (w x) on MFMA, from
//      transposing LDS reads of B and x (x scaled by w_l in fp32, rounded
//      once);
//   5. y, rounded to bf16, is staged in LDS and stored at the next chunk's
//      top in 16-byte row segments.
// No workspace: nothing but x, B, C, dt (and y) crosses HBM.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

// Transposing read of a 16-token K step: lane (col, kg) receives element
// [r0 + 8kg + j][c0 + col], j = 0..7, of a row-major bf16 tile with `ncc`
// 16-byte chunks per row (chunk-swizzled), as 4 words in K order.
__device__ __forceinline__ u32x4 tr_k16(int lane, const unsigned char *tile, int ncc, int r0, int c0) {
  const int kg = lane >> 5, gq = lane >> 4, d = lane & 15;
  const int cidx = c0 + 16 * (gq & 1) + 4 * (d & 3);
  u32x2 part[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int row = r0 + 8 * kg + 4 * hf + (d >> 2);
    const int cc = (cidx >> 3) ^ chunk_swz(row, ncc);
    part[hf] = lds_read_tr16(tile + row * (ncc * 16) + cc * 16 + (cidx & 7) * 2);
  }
  return u32x4{part[0].x, part[0].y, part[1].x, part[1].y};
}

template <int N>
__global__ __launch_bounds__(128) void k_ssd_fused(
    const uint16_t *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
    const float *__restrict__ h0, const int32_t *__restrict__ cu, int64_t L, int64_t T, int rows,
    int H, int G, uint16_t *__restrict__ y, float *__restrict__ hfin) {
  constexpr int P = 64, CQ = 32;           // head dim, chunk length
  constexpr int NT = N / 32;               // state tiles per wavefront (over n)
  constexpr int KN = N / 16;               // K steps over n
  constexpr int NCX = P / 8, NCB = N / 8;  // 16-byte chunks per x / B row
  constexpr int XB = CQ * P * 2;           // x of a chunk
  constexpr int BB = CQ * N * 2;           // B of a chunk
  constexpr int LYS = 32 + 8;              // y staging row (bf16 elements)
  constexpr int XI = XB / 1024 / 2, BI = BB / 1024 / 2;  // 1 KB direct loads per wavefront
  static_assert(XI * 2048 == XB && BI * 2048 == BB, "1 KB loads");
  // [XS0][XS1][BS0][BS1][CS0][CS1][YS w0][YS w1][AD w0][AD w1]
  constexpr int XS0 = 0, XS1 = XB, BS0 = 2 * XB, BS1 = BS0 + BB, CS0 = BS1 + BB, CS1 = CS0 + BB;
  constexpr int YS = CS1 + BB;
  constexpr int YSB = CQ * LYS * 2, AD = YS + 2 * YSB, ADB = 3 * CQ * 4;
  constexpr int TOTAL = AD + 2 * ADB + 2 * CQ * 4;
  __shared__ __align__(16) unsigned char smem[TOTAL];

  int s, h;
  xcd_chunk_head(H, s, h);
  if (s >= rows) return;
  const int g = h / (H / G);
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

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;
  const int kg = lane >> 5;
  const int ldx = H * P;
  const int ldb = G * N;
  const float Ah = A[h];
  const float Dh = Dv ? Dv[h] : 0.f;
  float *ad = reinterpret_cast<float *>(smem + AD + wave * ADB);  // [a | dt | w] of the chunk

  // state h^T: tile j holds rows n = 32j + acc_row(r, kg), column p = 32w + col
  f32x16 hst[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      hst[j][r] = h0 ? h0[sh * (P * N) + (int64_t)(32 * wave + col) * N + 32 * j + acc_row(r, kg)] : 0.f;
  }
  const int nck = static_cast<int>((len + CQ - 1) / CQ);

  float dtn = 0.f;  // dt of the chunk being loaded (wavefront 0, lanes < 32)
  auto issue_chunk = [&](int k, int slot) {  // x, B and C rows of chunk k into the ring
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;
    unsigned char *xs = smem + (slot ? XS1 : XS0);
    unsigned char *bs = smem + (slot ? BS1 : BS0);
    unsigned char *cs = smem + (slot ? CS1 : CS0);
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const unsigned m = (wave * XI + i) * 64 + lane, r = m / NCX;
      const unsigned cc = (m % NCX) ^ chunk_swz(r, NCX);
      load_lds16(x + (t0 + min((int)r, last)) * ldx + (int64_t)h * P + cc * 8, xs + (wave * XI + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const unsigned m = (wave * BI + i) * 64 + lane, r = m / NCB;
      const unsigned cc = (m % NCB) ^ chunk_swz(r, NCB);
      load_lds16(Bm + (t0 + min((int)r, last)) * ldb + (int64_t)g * N + cc * 8, bs + (wave * BI + i) * 1024);
      load_lds16(Cm + (t0 + min((int)r, last)) * ldb + (int64_t)g * N + cc * 8, cs + (wave * BI + i) * 1024);
    }
    if (wave == 0 && lane < CQ)  // dt of the chunk (0 past the sequence's end)
      dtn = lane <= last ? dt[(t0 + lane) * H + h] : 0.f;
  };
  // C operands in the state's K order: k-step q covers n-offsets
  // 16q + {4kg .. 4kg+3} and 16q + 8 + {4kg .. 4kg+3} of token row col (the
  // same order serves the B rows of Z)
  auto row_op = [&](const unsigned char *tile, int row, int q) {
    const unsigned char *rp = tile + row * (N * 2);
    const int sw = chunk_swz(row, NCB);
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(rp + ((2 * q) ^ sw) * 16 + 8 * kg);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(rp + ((2 * q + 1) ^ sw) * 16 + 8 * kg);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  };
  auto store_y = [&](int k, const unsigned char *ys) {  // the wavefront's 32 p of chunk k
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int rem = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = lane + 64 * i, r = u >> 2, c4 = u & 3;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(ys + (r * LYS + 8 * c4) * 2);
      if (r < rem) *reinterpret_cast<u32x4 *>(y + (t0 + r) * ldx + (int64_t)h * P + 32 * wave + 8 * c4) = v;
    }
  };
  auto wave_sync = []() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  unsigned char *ysw = smem + YS + wave * YSB;
  float *dts = reinterpret_cast<float *>(smem + AD + 2 * ADB);  // dt of the next chunk (wave 0 writes)
  if (nck > 0) issue_chunk(0, 0);

#pragma unroll 1
  for (int k = 0; k < nck; ++k) {
    const int slot = k & 1;
    const unsigned char *xs = smem + (slot ? XS1 : XS0);
    const unsigned char *bs = smem + (slot ? BS1 : BS0);
    const unsigned char *cs = smem + (slot ? CS1 : CS0);
    wait_vmcnt<0>();  // chunk k's x, B, C, dt; the y stores of chunk k-2
    if (wave == 0 && lane < CQ) dts[slot * CQ + lane] = dtn;
    __syncthreads();  // ... for every thread; chunk k-1 is done everywhere
    const float dtv = dts[slot * CQ + col];
    if (k > 0) store_y(k - 1, ysw);
    if (k + 1 < nck) issue_chunk(k + 1, slot ^ 1);
    u32x4 cop[KN];
#pragma unroll
    for (int q = 0; q < KN; ++q) cop[q] = row_op(cs, col, q);

    // 1. cumulative decay over the chunk (both halves of the wavefront hold
    // the same 32 values), weights of the chunk state
    float a = dtv * Ah;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const float t = __shfl_up(a, off, 32);
      if (col >= off) a += t;
    }
    const float alast = __shfl(a, 31, 32);
    if (kg == 0) {
      ad[col] = a;
      ad[CQ + col] = dtv;
      ad[2 * CQ + col] = __expf(alast - a) * dtv;
    }
    wave_sync();

    // 2. inter term
    f32x16 ya = f32x16{};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const u32x4 hq{pack_bf16x2(hst[j][8 * hf + 0], hst[j][8 * hf + 1]),
                       pack_bf16x2(hst[j][8 * hf + 2], hst[j][8 * hf + 3]),
                       pack_bf16x2(hst[j][8 * hf + 4], hst[j][8 * hf + 5]),
                       pack_bf16x2(hst[j][8 * hf + 6], hst[j][8 * hf + 7])};
        ya = mfma32x32x16(as_bf16x8(hq), as_bf16x8(cop[2 * j + hf]), ya);
      }
    }
    ya *= __expf(a);

    // 3. intra term (the diagonal tile) and the skip term
    f32x16 za = f32x16{};
#pragma unroll
    for (int q = 0; q < KN; ++q) za = mfma32x32x16(as_bf16x8(row_op(bs, col, q)), as_bf16x8(cop[q]), za);
    {
      float gv[16];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int sb = 8 * rb + 4 * kg;
        const f32x4 as = *reinterpret_cast<const f32x4 *>(ad + sb);
        const f32x4 ds = *reinterpret_cast<const f32x4 *>(ad + CQ + sb);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = sb + e <= col;
          const float arg = keep ? (a - as[e]) : -__builtin_inff();
          gv[rb * 4 + e] = keep ? za[rb * 4 + e] * __expf(arg) * ds[e] : 0.f;
        }
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
      // X^T operands in the accumulator's row order (s offsets 4kg.., 8+4kg..,
      // 16+4kg.., 24+4kg..) by transposing reads: lane (gq, d) addresses row
      // 8h4 + 4kg + d/4, columns p0 .. p0+3
      const int gq = lane >> 4, d = lane & 15;
      const int p0 = 32 * wave + 16 * (gq & 1) + 4 * (d & 3);
      u32x2 part[4];
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) {
        const int row = 8 * h4 + 4 * kg + (d >> 2);
        const int cc = (p0 >> 3) ^ chunk_swz(row, NCX);
        part[h4] = lds_read_tr16(xs + row * (P * 2) + cc * 16 + (p0 & 7) * 2);
      }
      ya = mfma32x32x16(as_bf16x8(u32x4{part[0].x, part[0].y, part[1].x, part[1].y}),
                        as_bf16x8(g0), ya);
      ya = mfma32x32x16(as_bf16x8(u32x4{part[2].x, part[2].y, part[3].x, part[3].y}),
                        as_bf16x8(g1), ya);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {  // D x_l: rows p = 32w + 8rb + 4kg + e of column l = col
      const int p = 32 * wave + 8 * rb + 4 * kg;
      const int cc = (p >> 3) ^ chunk_swz(col, NCX);
      const u32x2 xv = *reinterpret_cast<const u32x2 *>(xs + col * (P * 2) + cc * 16 + (p & 7) * 2);
      ya[rb * 4 + 0] += Dh * bf16lo(xv.x);
      ya[rb * 4 + 1] += Dh * bf16hi(xv.x);
      ya[rb * 4 + 2] += Dh * bf16lo(xv.y);
      ya[rb * 4 + 3] += Dh * bf16hi(xv.y);
    }

    // 4. state: h^T = exp(acum_last) h^T + B^T . (w x)
    {
      const float ed = __expf(alast);
#pragma unroll
      for (int j = 0; j < NT; ++j) hst[j] *= ed;
#pragma unroll
      for (int ks = 0; ks < CQ / 16; ++ks) {
        const u32x4 xq = tr_k16(lane, xs, NCX, 16 * ks, 32 * wave);
        const float *wl = ad + 2 * CQ + 16 * ks + 8 * kg;
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(wl);
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(wl + 4);
        const u32x4 xw{pack_bf16x2(bf16lo(xq.x) * w0.x, bf16hi(xq.x) * w0.y),
                       pack_bf16x2(bf16lo(xq.y) * w0.z, bf16hi(xq.y) * w0.w),
                       pack_bf16x2(bf16lo(xq.z) * w1.x, bf16hi(xq.z) * w1.y),
                       pack_bf16x2(bf16lo(xq.w) * w1.z, bf16hi(xq.w) * w1.w)};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const u32x4 bq = tr_k16(lane, bs, NCB, 16 * ks, 32 * j);
          hst[j] = mfma32x32x16(as_bf16x8(bq), as_bf16x8(xw), hst[j]);
        }
      }
    }

    // 5. y of this chunk staged (bf16) for the store at the next top
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int p = 8 * rb + 4 * kg;
      u32x2 o;
      o.x = pack_bf16x2(ya[rb * 4 + 0], ya[rb * 4 + 1]);
      o.y = pack_bf16x2(ya[rb * 4 + 2], ya[rb * 4 + 3]);
      *reinterpret_cast<u32x2 *>(ysw + (col * LYS + p) * 2) = o;
    }
    wave_sync();
  }
  if (nck > 0) store_y(nck - 1, ysw);
  if (hfin) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        hfin[sh * (P * N) + (int64_t)(32 * wave + col) * N + 32 * j + acc_row(r, kg)] = hst[j][r];
    }
  }
}

}  // namespace

bool fused_supported(int P, int N) { return P == 64 && (N == 64 || N == 128); }

hipError_t launch_fused(const void *x, const float *dt, const float *A, const void *B, const void *C,
                        const float *D, const float *h0, const int32_t *cu, int64_t L, int64_t T,
                        int rows, int H, int P, int N, int G, void *y, float *hfin,
                        hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (!fused_supported(P, N)) return hipErrorInvalidValue;
  const dim3 grid(xcd_grid(rows, H));
  const uint16_t *xi = static_cast<const uint16_t *>(x);
  const uint16_t *bi = static_cast<const uint16_t *>(B);
  const uint16_t *ci = static_cast<const uint16_t *>(C);
  uint16_t *yo = static_cast<uint16_t *>(y);
  if (N == 64)
    hipLaunchKernelGGL(k_ssd_fused<64>, grid, dim3(128), 0, stream, xi, dt, A, bi, ci, D, h0, cu, L,
                       T, rows, H, G, yo, hfin);
  else
    hipLaunchKernelGGL(k_ssd_fused<128>, grid, dim3(128), 0, stream, xi, dt, A, bi, ci, D, h0, cu,
                       L, T, rows, H, G, yo, hfin);
  return hipGetLastError();
}

}  // namespace ssd
