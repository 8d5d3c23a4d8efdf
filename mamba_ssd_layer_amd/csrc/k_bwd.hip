// libssd: the backward pass of the SSD forward (its gradients), in 32-token
// chunks, for bf16 io, P = 64, N in {64, 128}.
//
// The pages state no backward pass; it follows from the recurrence by the
// chain rule (page "State Space Duality and Mamba-2: Unifying Transformers and
// Semiseparable Matrices", section "Mathematical Foundations", with the
// scalar-identity transition of "The Scalar-Identity Structural Constraint"
// and the decay exp(dt A) of page "Mamba-2 Architecture: State Space Duality
// Explained", Step 1).  With a_t = exp(dt_t A), h_t = a_t h_{t-1} + dt_t x_t
// B_t^T, y_t = h_t C_t + D x_t and g_t = dL/dh_t:
//   g_t = dy_t C_t^T + a_{t+1} g_{t+1}
//   dx_t = D dy_t + dt_t g_t B_t,   dB_t = dt_t g_t^T x_t,   dC_t = h_t^T dy_t
//   ddt_t = x_t^T g_t B_t + A a_t <g_t, h_{t-1}>,   dA = sum_t dt_t a_t <g_t, h_{t-1}>
// Inside a chunk (tokens l, s; a_l the cumulative dt A from the chunk's start,
// L_ls = exp(a_l - a_s) for s <= l; h_s the state at the chunk's start, g_e
// the gradient flowing in from the next chunk) these become the blockwise
// products the forward uses, transposed:
//   Z_ls = C_l.B_s, E_ls = dy_l.x_s, M = Z o L dt_s, EL = E o L dt_s
//   dx^T = dy^T M + (g_e B^T) w_s + D dy^T           w_s = exp(a_last - a_s) dt_s
//   dB^T = C^T EL + (g_e^T x^T) w_s   (summed over the heads of a group)
//   dC^T = B^T EL^T + (h_s^T dy^T) exp(a_l)
//   ddt_t = sum_{l>=t} (E o Z o L)_lt + exp(a_last - a_t) q_t
//           + A (R_t + V_t + U_t),   dA = sum_t dt_t (R_t + V_t + U_t)
// with q_s = x_s^T g_e B_s, v_l = exp(a_l) dy_l.(h_s C_l), K = E o Z o L dt_s,
// R_t = sum over l >= t > s of K_ls (a suffix sum of row sums minus column
// sums of K's strict lower part), V_t = sum_{l>=t} v_l and
// U_t = exp(a_last) <g_e, h_s> + sum_{s<t} w_s q_s.
//
// Three passes:
//   1. the one-pass forward saves h_s of every chunk (k_ssd_fused, SAVE);
//   2. k_bwd_reverse walks each (sequence, two heads) backwards, keeping g on
//      chip like the forward keeps h (g <- exp(a_last) g + C^T (exp(a_l) dy)),
//      saving g_e of every chunk and writing dL/dh0;
//   3. k_bwd_chunk, one block of 16 wavefronts per (chunk, group), walks the
//      group's heads: the chunk's B and C stay in LDS, each head's x, dy, h_s
//      and g_e stream through an LDS ring; dx and ddt are written per head, dB
//      and dC accumulate over the heads in registers and are written once, dA
//      and dD are added atomically per head.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr float kLog2eB = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16b(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ float exp2b(float v) { return __builtin_amdgcn_exp2f(v); }
template <int CTRL, int ROWS>
__device__ __forceinline__ float dppb(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
// inclusive prefix sum over lanes 0..31 (and independently 32..63)
__device__ __forceinline__ float scan32b(float a) {
  a += dppb<0x111, 0xF>(a);
  a += dppb<0x112, 0xF>(a);
  a += dppb<0x114, 0xF>(a);
  a += dppb<0x118, 0xF>(a);
  a += dppb<0x142, 0xA>(a);
  return a;
}
// sum over the 16 lanes of each row of the wavefront (every lane gets it)
__device__ __forceinline__ float rowsum16(float v) {
  v += dppb<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v += dppb<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v += dppb<0x141, 0xF>(v);  // row_half_mirror
  v += dppb<0x140, 0xF>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float lane31(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
}
__device__ __forceinline__ void wsync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// XOR swizzle of the 16-byte chunk index of an LDS tile row of NC chunks by
// the row (a bit-pair rotation of the row's low bits), so that 16 lanes
// reading one chunk column of consecutive rows, and the transposing reads of
// 4 rows, spread over the LDS banks
template <int NC>
__device__ __forceinline__ int swz(int r) {
  return NC == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// A second XOR swizzle, chosen for the access patterns of the x / dy tiles
// (both passes) and the chunk pass's other tiles: row reads of 16 consecutive rows (one chunk column), transposing
// reads of 8 consecutive rows x 2 chunks per 32 lanes, and transposing reads
// of rows {0..3, 8..11} (+ 4, + 32 k) x 2 chunks.  The pair of chunks {c, c^1}
// a row maps to is set by chunk bits 1 and up, which take (16 chunks) the
// row's bits 0-1 and bit 2 XOR bit 3, or (8 chunks, 128-byte rows whose banks
// repeat every other row) its bit 1 and bit 2 XOR bit 3; chunk bit 0 takes
// the row's bit 3.  Every pattern then touches distinct banks.
template <int NC>
__device__ __forceinline__ int swz2(int r) {
  return NC == 16 ? ((((r & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2)) << 1) | ((r >> 3) & 1))
                  : (((((r >> 1) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1)) << 1) | ((r >> 3) & 1));
}

// ---------------------------------------------------------------- pass 2
// Block = (sequence or segment of one, two heads of a group), 4
// wavefronts (head hh, half ph); wavefront (hh, ph) keeps rows p in
// [32 ph, 32 ph + 32) of head hh's g, held transposed like the forward's state
// (tiles 2q, 2q+1 give lane group g4 the n = 32q + 8 g4 + 0..7).  Chunks in
// reverse order through an R-slot ring of dy (per head), C and dt, R - 1
// chunks in flight ahead of the one being computed.
// MODE: RV_FULL walks a whole sequence from dfinal, saves g where each 64-token
// pair ends and writes dL/dh0; for few (sequence, head-pair) blocks the sweep is
// split into segments of segc 32-token chunks: RV_SEGSUM walks a segment from
// g = 0 and writes its sum G_seg and its total decay (log) A_seg, k_bwd_gpass
// chains them, and RV_SEG walks each segment again from the gradient entering
// it from the right (gin) and saves g at its pair ends.
enum { RV_FULL = 0, RV_SEGSUM = 1, RV_SEG = 2 };
// ring slots: kRevSlots - 1 chunks in flight (a fourth slot measured no faster:
// the sweep is bound by its state-gradient stores, not by load latency)
constexpr int kRevSlots = 3;

template <int N, int MODE, int R>
__global__ __launch_bounds__(256, 2) void k_bwd_reverse(
    const uint16_t *__restrict__ dy, const float *__restrict__ dt, const float *__restrict__ A,
    const uint16_t *__restrict__ Cm, const float *__restrict__ gstart,
    const int32_t *__restrict__ cu, int64_t L, int64_t T, int rows, int H, int G, int segc,
    uint16_t *__restrict__ gsave, float *__restrict__ gout, float *__restrict__ aseg) {
  constexpr int P = 64, CQ = 32, D = R - 1;  // D chunks in flight ahead
  constexpr int NT = N / 16, KQ = N / 32, NCB = N / 8;
  constexpr int XH = CQ * P * 2, BT = CQ * N * 2, DW = 256;
  constexpr int OY = 0, OC = 2 * XH, OD = OC + BT, SLOT = OD + 4 * DW;
  constexpr int AD = R * SLOT, ADW = 2 * CQ * 4;
  constexpr int BCI = BT / 1024 / 4;  // 1 KB pieces of C per wavefront
  static_assert(BCI * 4 * 1024 == BT, "C split over 4 wavefronts");
  constexpr int LDR = 2 + BCI + 1;  // vector-memory ops a wavefront issues per chunk load
  constexpr int SV = 2 * KQ;        // state-gradient stores a wavefront issues per chunk
  static_assert(R >= 3 && D * SV + (D - 1) * LDR <= 47, "wait counts");
  __shared__ __align__(16) unsigned char smem[AD + 4 * ADW];

  int s = -1, hb;
  int64_t tb = 0, len = 0, gs = 0;  // gs: the segment's index in the batch's segment list
  int kb = 0, ke = 0;               // the block's chunks [kb, ke) of its sequence
  if (MODE == RV_FULL) {
    xcd_chunk_head(H / 2, s, hb);
    if (s >= rows) return;
    seq_range(cu, s, L, T, tb, len);
    ke = static_cast<int>((len + CQ - 1) / CQ);
  } else {
    int gsi;
    xcd_chunk_head(H / 2, gsi, hb);
    gs = gsi;
    int64_t seg = -1;
    if (!cu) {
      const int64_t nsr = (L + (int64_t)segc * CQ - 1) / ((int64_t)segc * CQ);
      if (nsr == 0) return;
      s = static_cast<int>(gs / nsr);
      seg = gs % nsr;
      if (s >= rows) return;
      seq_range(cu, s, L, T, tb, len);
    } else {
      int64_t before;
      s = locate_unit(cu, rows, T, gs, segc * CQ, before);
      if (s < 0) return;
      seg = gs - before;
      seq_range(cu, s, L, T, tb, len);
    }
    kb = static_cast<int>(seg) * segc;
    ke = min(kb + segc, static_cast<int>((len + CQ - 1) / CQ));
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int hh = wave >> 1, ph = wave & 1;
  const int h = 2 * hb + hh, g = 2 * hb / (H / G);
  const int nck = static_cast<int>((len + CQ - 1) / CQ);
  const int nk = ke - kb;
  const int64_t pbase = MODE == RV_SEGSUM ? 0 : pair_base64(cu, s, L, T);
  const int64_t sh = (int64_t)s * H + h;
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const float Ah = A[h];
  float *adw = reinterpret_cast<float *>(smem + AD + wave * ADW);
  auto nrow = [&](int j) { return 32 * (j >> 1) + 8 * g4 + 4 * (j & 1); };

  // the state rows of (sequence, head) or (segment, head) in [P][N] fp32 buffers
  const int64_t srow0 = (MODE == RV_FULL ? sh : gs * H + h) * P;
  f32x4 gst[2][NT];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
    const int64_t prow = (srow0 + 32 * ph + 16 * pt + c16) * N;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      gst[pt][j] = MODE == RV_SEGSUM || !gstart ? f32x4{}
                                                : *reinterpret_cast<const f32x4 *>(gstart + prow + nrow(j));
  }

  auto issue = [&](int k, int sl) {
    const int64_t t0 = tb + (int64_t)k * CQ;
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;
    const uint32_t base = lds_off(smem) + sl * SLOT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // rows 16 ph .. +15 of head hh's dy
      const int m = i * 64 + lane, r = 16 * ph + (m >> 3), cc = (m & 7) ^ swz2<8>(r);
      dma_lds16(dy + (t0 + min(r, last)) * ldx + (int64_t)h * P + 8 * cc,
                base + OY + hh * XH + 16 * ph * 128 + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < BCI; ++i) {
      const int pi = wave * BCI + i, m = pi * 64 + lane, r = m / NCB;
      const int cc = (m % NCB) ^ swz<NCB>(r);
      dma_lds16(Cm + (t0 + min(r, last)) * ldb + (int64_t)g * N + 8 * cc, base + OC + pi * 1024);
    }
    dma_lds4(dt + (t0 + min(lane & 31, last)) * H + h, base + OD + wave * DW);
  };

  // the gradient flowing into chunk k from the later chunks is kept where it
  // leaves a 64-token pair (k odd, or the sequence's last chunk)
  auto saves = [&](int k) { return MODE != RV_SEGSUM && ((k & 1) || k == nck - 1); };
  // reverse order: iteration i handles chunk ke - 1 - i in slot i % R
#pragma unroll
  for (int c = 0; c < D; ++c)
    if (c < nk) issue(ke - 1 - c, c);
  int sl = 0;
  float asum = 0.f;  // the block's chunks' total decay exponent (RV_SEGSUM)
#pragma unroll 1
  for (int i = 0; i < nk; ++i) {
    const int k = ke - 1 - i;
    // chunk k's loads have landed once at most the later ops are pending
    // (completion in issue order): the prologue's later loads, then per
    // iteration m < i the loads of iteration m + D (LDR) and m's
    // state-gradient stores (SV where one is stored)
    {
      auto sv = [&](int m) { return saves(ke - 1 - m) ? SV : 0; };
      int n = i < D ? (min(D, nk) - 1 - i) * LDR : sv(i - D);
      for (int m = i < D ? 0 : i - D + 1; m < i; ++m) n += (m + D < nk ? LDR : 0) + sv(m);
      wait_vmcnt_dyn(n);
    }
    __syncthreads();
    const int slp = sl == 0 ? R - 1 : sl - 1;  // slot of iteration i-1, and of i+D
    if (k - D >= kb) issue(k - D, slp);
    if (saves(k)) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        u32x4 pk[KQ];  // row p = 32 ph + 16 pt + c16, n = 32 q + 8 g4 + 0..7
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
          const f32x4 u = gst[pt][2 * q], v = gst[pt][2 * q + 1];
          pk[q] = u32x4{pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                        pack_bf16x2(v.z, v.w)};
        }
        store_rows128(gsave + ((pbase + (k >> 1)) * H + h) * (int64_t)(P * N) +
                          (int64_t)(32 * ph + 16 * pt) * N,
                      N, pk, c16, g4);
      }
    }
    const unsigned char *ys = smem + sl * SLOT + OY + hh * XH;
    const unsigned char *cs = smem + sl * SLOT + OC;
    const float *dts = reinterpret_cast<const float *>(smem + sl * SLOT + OD + wave * DW);
    const int last = static_cast<int>(min((int64_t)CQ, len - (int64_t)k * CQ)) - 1;
    const int tl = lane & 31;
    const float dtv = tl <= last ? dts[lane] : 0.f;
    const float a = scan32b(dtv * Ah);
    const float alast = lane31(a);
    asum += alast;
    // exp(a_l); 0 for the rows past a partial chunk's end (they repeat its last row)
    if (lane < 32) adw[tl] = tl <= last ? exp2b(a * kLog2eB) : 0.f;
    wsync();
    // g <- exp(a_last) g + C^T (exp(a_l) dy)
    const float e = exp2b(alast * kLog2eB);
    u32x4 fy[2];
    {
      const f32x4 f0 = *reinterpret_cast<const f32x4 *>(adw + 4 * g4);
      const f32x4 f1 = *reinterpret_cast<const f32x4 *>(adw + 16 + 4 * g4);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        u32x2 t[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int row = 16 * hf + 4 * g4 + (c16 >> 2), col = 32 * ph + 16 * pt + 4 * (c16 & 3);
          const int cc = (col >> 3) ^ swz2<8>(row);
          t[hf] = lds_read_tr16(ys + row * 128 + (cc << 4) + (col & 7) * 2);
        }
        fy[pt] = u32x4{pack_bf16x2(bf16lo(t[0].x) * f0.x, bf16hi(t[0].x) * f0.y),
                       pack_bf16x2(bf16lo(t[0].y) * f0.z, bf16hi(t[0].y) * f0.w),
                       pack_bf16x2(bf16lo(t[1].x) * f1.x, bf16hi(t[1].x) * f1.y),
                       pack_bf16x2(bf16lo(t[1].y) * f1.z, bf16hi(t[1].y) * f1.w)};
#pragma unroll
        for (int j = 0; j < NT; ++j) gst[pt][j] *= e;
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      u32x2 t[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int row = 16 * hf + 4 * g4 + (c16 >> 2);
        const int col = 32 * (j >> 1) + 8 * (c16 & 3) + 4 * (j & 1);
        const int cc = (col >> 3) ^ swz<NCB>(row);
        t[hf] = lds_read_tr16(cs + row * (N * 2) + (cc << 4) + (col & 7) * 2);
      }
      const u32x4 ct{t[0].x, t[0].y, t[1].x, t[1].y};
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) gst[pt][j] = mfma16b(ct, fy[pt], gst[pt][j]);
    }
    sl = sl == R - 1 ? 0 : sl + 1;
  }
  // RV_FULL: dL/dh0; RV_SEGSUM: the segment's G_seg and A_seg
  if (MODE != RV_SEG && gout) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int64_t prow = (srow0 + 32 * ph + 16 * pt + c16) * N;
#pragma unroll
      for (int j = 0; j < NT; ++j) *reinterpret_cast<f32x4 *>(gout + prow + nrow(j)) = gst[pt][j];
    }
  }
  if (MODE == RV_SEGSUM && ph == 0 && lane == 0) aseg[gs * H + h] = asum;
}

// The sweep over segments, per (sequence, head) and 4 elements of the P x N
// gradient a thread: gin[seg] = g; g = exp(A_seg) g + G_seg, from dfinal (or 0)
// down to the first segment; then dL/dh0 = g.
__global__ __launch_bounds__(256) void k_bwd_gpass(
    const float *__restrict__ gseg, const float *__restrict__ aseg,
    const float *__restrict__ dfinal, const int32_t *__restrict__ cu, int64_t L, int64_t T,
    int rows, int H, int PN, int segt, float *__restrict__ gin, float *__restrict__ dinit) {
  const int s = blockIdx.z, h = blockIdx.y;
  const int e = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (s >= rows) return;
  // segt: tokens per segment (all lanes take part in the walk over the
  // sequences before returning)
  const int64_t base = cu ? units_before(cu, s, T, segt) : (int64_t)s * ((L + segt - 1) / segt);
  if (e >= PN) return;
  int64_t tb, len;
  seq_range(cu, s, L, T, tb, len);
  const int nseg = static_cast<int>((len + segt - 1) / segt);
  const int64_t sh = (int64_t)s * H + h;
  f32x4 gv = dfinal ? *reinterpret_cast<const f32x4 *>(dfinal + sh * PN + e) : f32x4{};
#pragma unroll 1
  for (int k = nseg - 1; k >= 0; --k) {
    const int64_t o = ((base + k) * H + h) * (int64_t)PN + e;
    const f32x4 gsum = *reinterpret_cast<const f32x4 *>(gseg + o);
    const float d = exp2b(aseg[(base + k) * H + h] * kLog2eB);
    *reinterpret_cast<f32x4 *>(gin + o) = gv;
    gv = gv * d + gsum;
  }
  if (dinit) *reinterpret_cast<f32x4 *>(dinit + sh * PN + e) = gv;
}

// ---------------------------------------------------------------- pass 3
// Block = (32-token chunk, group), 16 wavefronts (four per SIMD), walking the
// group's heads.  LDS: the chunk's B and C (rows = tokens) and the neighbour
// chunk's B or C; an R-slot ring per head of x and dy (rows = tokens, 8 chunks
// a row), the pair's saved h_s and g_e (rows = p, N/8 chunks a row), dt, and
// the neighbour chunk's x or dy and dt; the head's masked products as ready
// MFMA operands; per-wavefront tables and cross-wavefront partial sums (two
// buffers, by head parity, since a head's sums are finished one head later).
// Tile conventions (16x16x32 MFMA): an "E-layout" tile (lt, st) holds
// matrix[l][s] with lane (c16 = s, g4) rows l = 16 lt + 4 g4 + r; the tiles
// lt = 0, 1 of one st together form a B operand with K = l in the order
// {4 g4 + 0..3, 16 + 4 g4 + 0..3} (8 bytes of each tile per lane), matched by
// transposing reads of token rows in that order for the A operand.  An
// "ET-layout" tile (st, lt) holds matrix[s][l] the same way.
// Per head: wavefronts 0-3 form one E-layout tile each of E = dy x^T and from
// it M = Z o L dt_s, EL = E o L dt_s and the sums of K = E o Z o L dt_s,
// wavefronts 4-7 one ET-layout tile each of E^T and EL^T, and wavefronts 8-15
// derive N/32 tiles each of the state the pair does not hold for this chunk
// (in place).  After a barrier wavefront w < 8 takes the g_e side: one 16 x 16
// tile of dx (p-tile w/2, s-tile w%2), its q_s partial and N/64 tiles of dB;
// wavefront 8 + w the h_s side: the matching tile of h_s C^T for v_l,
// <g_e, h_s> over p-tile w/2 (w even) and N/64 tiles of dC.  Wavefront 4
// finishes the previous head's per-token scalars.  (Eight wavefronts, two a
// SIMD, each doing both sides, measured 6-8% slower.)
template <int N, int R, bool ACC = false>
struct BwdCfg {
  static constexpr int P = 64, CQ = 32, NCB = N / 8, WAVES = 16;
  static constexpr int XT = CQ * P * 2;      // x or dy of a head: 32 rows x 128 B
  static constexpr int ST = P * N * 2;       // h_s or g_e of a head: 64 rows x N bf16
  static constexpr int BT = CQ * N * 2;      // B or C of a chunk
  // a ring slot: x, dy, h_s, g_e, dt of the chunk; x or dy, dt of the neighbour chunk
  static constexpr int OX = 0, OY = XT, OH = 2 * XT, OG = OH + ST, ODT = OG + ST;
  static constexpr int ONX = ODT + 256, ONDT = ONX + XT;
  // ACC: the dx already written for the head (rows = tokens, like x), which
  // this pass adds its own to
  static constexpr int OAX = ONDT + 256;
  static constexpr int HSLOT = OAX + (ACC ? XT : 0);
  static constexpr int OB = R * HSLOT, OCC = OB + BT;   // R ring slots of a head's tiles
  static constexpr int ONBC = OCC + BT;                  // B or C of the neighbour chunk
  static constexpr int OOP = ONBC + BT;                  // operands M, EL, ELT: [2][64 lanes][16 B] each
  static constexpr int OTAB = OOP + 3 * 2048;            // per wavefront and buffer: 6 tables of 32 floats
  static constexpr int TABW = 6 * CQ * 4;
  static constexpr int OPART = OTAB + 2 * WAVES * TABW;  // per buffer: the partial sums below
  static constexpr int PARTW = 512 * 4;
  static constexpr int TOTAL = OPART + 2 * PARTW;
  static constexpr int KP = ST / 1024 / WAVES;           // h_s (and g_e) pieces per wavefront; 0:
                                                         // one piece a wavefront, h_s for the
                                                         // first half of them, g_e for the rest
  static constexpr int NTW = N / 64;                     // tiles of dB (or of dC) per wavefront
  static constexpr int DTW = N / 32;                     // tiles of the derived state per wavefront
                                                         // of the eight that derive
  static_assert((KP >= 1 && KP * WAVES * 1024 == ST) || (KP == 0 && 2 * ST == WAVES * 1024),
                "state pieces");
  static_assert(TOTAL <= 160 * 1024, "LDS");
};

template <int N, int R, bool ACC = false>
__global__ __launch_bounds__(1024, 1) void k_bwd_chunk(
    const uint16_t *__restrict__ x, const float *__restrict__ dt, const float *__restrict__ A,
    const uint16_t *__restrict__ Bm, const uint16_t *__restrict__ Cm, const float *__restrict__ Dv,
    const uint16_t *__restrict__ dy, const uint16_t *__restrict__ hsave, int hsld,
    const uint16_t *__restrict__ gsave, const int32_t *__restrict__ cu, int64_t L, int64_t T,
    int rows, int64_t nchunks, int H, int G, const uint16_t *dxacc, uint16_t *dx,
    float *__restrict__ ddt, float *__restrict__ dA, float *__restrict__ dB,
    float *__restrict__ dC, float *__restrict__ dD) {
  using F = BwdCfg<N, R, ACC>;
  constexpr int P = F::P, CQ = F::CQ, NCB = F::NCB, KP = F::KP, NTW = F::NTW;
  constexpr int W = F::WAVES, NT = 64 * W;  // wavefronts, threads
  constexpr int KQ = N / 32;  // K steps over n
  __shared__ __align__(16) unsigned char smem[F::TOTAL];

  // XCD-aware order: block b runs on XCD b % 8, which takes a contiguous range
  // of (chunk, group) indices, so the two chunks of a 64-token pair (which
  // read the same saved tiles) run on one XCD at about the same time and the
  // second read is served by its L2
  const int64_t nblk = nchunks * G, per = (nblk + 7) / 8;
  const int64_t lb = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (lb >= nblk) return;
  const int64_t c = lb / G;
  const int g = static_cast<int>(lb % G);
  // chunk c of the sequence-major list -> (sequence, chunk within it), and the
  // index of the sequence's first 64-token pair (the saved states' layout)
  int s = -1;
  int64_t k = 0, tb = 0, len = 0, pb0 = 0;
  if (!cu) {
    const int64_t nckr = (L + CQ - 1) / CQ;
    if (nckr == 0) return;
    s = static_cast<int>(c / nckr);
    k = c % nckr;
    if (s >= rows) return;
    seq_range(cu, s, L, T, tb, len);
    pb0 = (int64_t)s * ((L + 63) / 64);
  } else {
    int64_t before;
    s = locate_unit(cu, rows, T, c, CQ, before);
    if (s < 0) return;
    k = c - before;
    seq_range(cu, s, L, T, tb, len);
    pb0 = units_before(cu, s, T, 64);
  }
  // The saved states are kept per 64-token pair of chunks: h_s entering the
  // pair, g_e leaving it.  An even chunk reads its h_s; its g_e is derived
  // from the pair's and the next chunk (unless it ends the sequence); an odd
  // chunk reads its g_e and derives h_s from the pair's and the chunk before.
  enum { NONE = 0, DG = 1, DH = 2 };
  const int nck = static_cast<int>((len + CQ - 1) / CQ);
  const int mode = (k & 1) ? DH : (k + 1 < nck ? DG : NONE);
  const int64_t pidx = pb0 + (k >> 1);
  const int64_t tn0 = tb + (k + (mode == DG ? 1 : -1)) * CQ;  // the neighbour chunk's first token
  const int lastn = mode == NONE ? 0 : static_cast<int>(min((int64_t)CQ, tb + len - tn0)) - 1;
  const int64_t t0 = tb + k * CQ;
  const int last = static_cast<int>(min((int64_t)CQ, len - k * CQ)) - 1;
  const bool full = last == CQ - 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g4 = lane >> 4, tl = lane & 31;
  const int hpg = H / G;
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const uint32_t lbase = lds_off(smem);
  const unsigned char *bsm = smem + F::OB;
  const unsigned char *csm = smem + F::OCC;
  unsigned char *opm = smem + F::OOP, *opel = opm + 2048, *opelt = opm + 4096;
  auto tab_of = [&](int b) { return reinterpret_cast<float *>(smem + F::OTAB + (b * W + wave) * F::TABW); };
  auto part_of = [&](int b) { return reinterpret_cast<float *>(smem + F::OPART + b * F::PARTW); };
  // tables: a_l log2(e), exp(a_l), w_s, dt_s, exp(a_last - a_s), and the
  // neighbour chunk's token factors (w'_s for h_s, exp(a'_l) for g_e)
  enum { TA2 = 0, TF = 32, TW = 64, TDT = 96, TEL = 128, TNW = 160 };
  // partial sums: q_s [p-tile][s], v_l [p-tile][l], <g_e, h_s> [p-tile], column
  // sums of E o Z o L [lt][s] (all l >= s) and of K [lt][s] (l > s), row sums
  // of K [st][l] (s < l), diagonal of E [s]
  enum { PQ = 0, PV = 128, PGH = 256, PC1 = 264, PCK = 328, PRK = 392, PDE = 456 };

  // ---- operand reads ----
  // 16 bytes of a token row of x / dy (8 chunks): p = 32 kq + 8 g4 + 0..7
  auto rowx = [&](const unsigned char *t, int row, int kq) {
    return *reinterpret_cast<const u32x4 *>(t + row * 128 + (((4 * kq + g4) ^ swz2<8>(row)) << 4));
  };
  // 16 bytes of a row of an N-wide tile (B, C, h_s, g_e): n = 32 q + 8 g4 + 0..7
  auto rown = [&](const unsigned char *t, int row, int q) {
    return *reinterpret_cast<const u32x4 *>(t + row * (N * 2) + (((4 * q + g4) ^ swz2<NCB>(row)) << 4));
  };
  // transposing read: lane (c16, g4) gets column col0 + c16 of rows r0 + 0..3
  // and r1 + 0..3 (r0, r1 per lane group)
  auto trn = [&](const unsigned char *t, int rb, int r0, int r1, int col0, bool wide) {
    u32x2 v[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = (hf ? r1 : r0) + (c16 >> 2), col = col0 + 4 * (c16 & 3);
      const int cc = (col >> 3) ^ (wide ? swz2<NCB>(row) : swz2<8>(row));
      v[hf] = lds_read_tr16(t + row * rb + (cc << 4) + (col & 7) * 2);
    }
    return u32x4{v[0].x, v[0].y, v[1].x, v[1].y};
  };

  // Per-lane byte offsets of this wavefront's DMA pieces, fixed for the block:
  // x (wavefronts 0-3) or dy (4-7) piece wave % 4 (rows 8 (wave % 4) .. +7,
  // clamped to the chunk's end); h_s and g_e pieces wave + W k (the swizzle
  // repeats every 16 rows, so piece k's offsets are piece 0's plus 8 KB k); dt;
  // the neighbour chunk's x or dy piece wave % 4 (wavefronts 8-11).
  uint32_t xoff, hoff, hsoff, dtoff, nxoff, ndtoff;
  {
    const int m = (wave & 3) * 64 + lane, r = m >> 3, cc = (m & 7) ^ swz2<8>(r);
    xoff = static_cast<uint32_t>((min(r, last) * ldx + 8 * cc) * 2);
    const int mh = (KP ? wave : wave % (W / 2)) * 64 + lane, rh = mh / NCB,
              ch = (mh % NCB) ^ swz2<NCB>(rh);
    hoff = static_cast<uint32_t>((rh * N + 8 * ch) * 2);
    hsoff = static_cast<uint32_t>((rh * hsld + 8 * ch) * 2);
    dtoff = static_cast<uint32_t>(min(tl, last) * H * 4);
    nxoff = static_cast<uint32_t>((min(r, lastn) * ldx + 8 * cc) * 2);
    ndtoff = static_cast<uint32_t>(min(tl, lastn) * H * 4);
  }
  // the wavefronts that load the neighbour chunk's x / dy pieces and its dt
  const bool nxw = wave >= 8 && wave < 12;
  const int ndtw = 12;
  // head j's x, dy, h_s, g_e and dt into ring slot sl: scalar bases, fixed lane offsets
  auto issue_head = [&](int j, int sl) {
    const int h = g * hpg + j;
    const uint32_t base = lbase + sl * F::HSLOT;
    if (wave < 8)
      dma_lds16_sb(xoff, (wave < 4 ? x : dy) + t0 * ldx + (int64_t)h * P,
                   base + (wave < 4 ? F::OX : F::OY) + (wave & 3) * 1024);
    const int64_t st0 = (pidx * H + h) * (int64_t)(P * N);
    const int64_t sh0 = (pidx * H + h) * (int64_t)P * hsld;
    if constexpr (KP == 0) {
      if (wave < W / 2)
        dma_lds16_sb(hsoff, hsave + sh0, base + F::OH + wave * 1024);
      else
        dma_lds16_sb(hoff, gsave + st0, base + F::OG + (wave - W / 2) * 1024);
    } else {
#pragma unroll
      for (int kk = 0; kk < KP; ++kk)
        dma_lds16_sb(hsoff, hsave + sh0 + (int64_t)(512 * W / N) * hsld * kk,
                     base + F::OH + (wave + W * kk) * 1024);
#pragma unroll
      for (int kk = 0; kk < KP; ++kk)
        dma_lds16_sb(hoff, gsave + st0 + 512 * W * kk, base + F::OG + (wave + W * kk) * 1024);
    }
    if (wave == 0) dma_lds4_sb(dtoff, dt + t0 * H + h, base + F::ODT);
    if (mode != NONE) {  // the neighbour chunk's x (for h_s) or dy (for g_e), and dt
      if (nxw)
        dma_lds16_sb(nxoff, (mode == DH ? x : dy) + tn0 * ldx + (int64_t)h * P,
                     base + F::ONX + (wave & 3) * 1024);
      if (wave == ndtw) dma_lds4_sb(ndtoff, dt + tn0 * H + h, base + F::ONDT);
    }
    if (ACC && wave >= 12)  // piece wave % 4 of the dx to add to (rows as for x)
      dma_lds16_sb(xoff, dxacc + t0 * ldx + (int64_t)h * P, base + F::OAX + (wave & 3) * 1024);
  };

  // ---- the chunk's B and C, then heads 0 .. R-2 ahead ----
  {
    // pieces u = wave, wave + W, ... of the 2 BT / 1024 of B and C
    constexpr int NBCP = 2 * F::BT / 1024;
#pragma unroll
    for (int i = 0; i < (NBCP + W - 1) / W; ++i) {
      const int u = wave + W * i, tile = u / (F::BT / 1024), pi = u % (F::BT / 1024);
      if (u >= NBCP) break;
      const int m = pi * 64 + lane, r = m / NCB, cc = (m % NCB) ^ swz2<NCB>(r);
      dma_lds16((tile ? Cm : Bm) + (t0 + min(r, last)) * ldb + (int64_t)g * N + 8 * cc,
                lbase + (tile ? F::OCC : F::OB) + pi * 1024);
    }
    // the neighbour chunk's B (for h_s) or C (for g_e)
    if (mode != NONE && wave < F::BT / 1024) {
      const int m = wave * 64 + lane, r = m / NCB, cc = (m % NCB) ^ swz2<NCB>(r);
      dma_lds16((mode == DH ? Bm : Cm) + (tn0 + min(r, lastn)) * ldb + (int64_t)g * N + 8 * cc,
                lbase + F::ONBC + wave * 1024);
    }
  }
  // vector-memory ops a wavefront issues per head: its x or dy piece, the
  // h_s and g_e pieces, dt, the neighbour chunk's piece and dt
  const int LDW = (wave < 8 ? 1 : 0) + (KP ? 2 * KP : 1) + (wave == 0 ? 1 : 0) +
                  (mode != NONE ? (nxw ? 1 : 0) + (wave == ndtw ? 1 : 0) : 0) +
                  (ACC && wave >= 12 ? 1 : 0);
  // stores and atomics a wavefront issues in iteration m: its dx tile of head
  // m (wavefronts 0-7); wavefront 4 also ddt, dA, dD of head m - 1
  const int dxw = wave < 8 ? 1 : 0;
  auto stw = [&](int m) { return dxw + (wave == 4 && m >= 1 ? 2 + (dD ? 1 : 0) : 0); };
#pragma unroll
  for (int jj = 0; jj < R - 1; ++jj)
    if (jj < hpg) issue_head(jj, jj);
  wait_vmcnt_dyn(min(R - 1, hpg) * LDW);  // B and C are in (the head loads issued after them may not be)
  __syncthreads();

  // this wavefront's roles
  const bool etile = wave < 4;               // E-layout tile (lt, st) = (wave / 2, wave % 2)
  const int qa = (wave >> 1) & 1, qb = wave & 1;  // E: (lt, st) = (qa, qb); ET: (st, lt) = (qa, qb)
  const int pt = (wave & 7) >> 1, sh = wave & 1;  // dx / h_s C^T tile (p-tile, s- or l-tile)
  // the wavefront that finishes a head's per-token scalars
  const bool fin = wave == 4;
  // Z = C B^T, the E-layout tile (qa, qb) (wavefronts 0-3)
  f32x4 z{};
  if (etile) {
#pragma unroll
    for (int q = 0; q < KQ; ++q) z = mfma16b(rown(csm, 16 * qa + c16, q), rown(bsm, 16 * qb + c16, q), z);
  }

  f32x4 dBa[NTW];  // this wavefront's tiles of dB (wavefronts 0-7) or dC (8-15)
#pragma unroll
  for (int i = 0; i < NTW; ++i) dBa[i] = f32x4{};

  // ---- per-token scalars of head jj (its partials complete): computed by
  // wavefront 4 at the top of the next head's iteration, before its ET tile
  // (0-3 start that head's heavier E tiles meanwhile); it writes ddt and adds
  // dA, dD ----
  auto finish = [&](int jj, float Ah, float alast) {
    const int h = g * hpg + jj;
    const float *tab = tab_of(jj & 1);
    const float *part = part_of(jj & 1);
    float q = 0.f, v = 0.f, gh = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q += part[PQ + 32 * w + tl];
      v += part[PV + 32 * w + tl];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) gh += part[PGH + w];
    const float t1 = part[PC1 + tl] + part[PC1 + 32 + tl];
    const float ck = part[PCK + tl] + part[PCK + 32 + tl];
    const float rkr = part[PRK + tl] + part[PRK + 32 + tl];
    v *= tab[TF + tl];
    const float u = tab[TW + tl] * q;
    const float uin = scan32b(u);
    const float vin = scan32b(v);
    const float rkv = rkr - ck;
    const float rin = scan32b(rkv);
    const float U = exp2b(alast * kLog2eB) * gh + (uin - u);
    const float V = lane31(vin) - vin + v;
    const float Rr = lane31(rin) - rin + rkv;
    const float term1 = t1 + tab[TEL + tl] * q;
    const float dd = term1 + Ah * (Rr + V + U);
    const bool ok = lane < 32 && tl <= last;
    const float da = lane31(scan32b(ok ? tab[TDT + tl] * (Rr + V + U) : 0.f));
    const float dsum = lane31(scan32b(ok ? part[PDE + tl] : 0.f));
    if (wave == 4) {
      if (ok) ddt[(t0 + tl) * H + h] = dd;
      if (lane == 0) {
        atomicAdd(dA + h, da);
        if (dD) atomicAdd(dD + h, dsum);
      }
    }
  };
  float pAh = 0.f, palast = 0.f;  // of the previous head

#pragma unroll 1
  for (int j = 0; j < hpg; ++j) {
    const int sl = j % R;
    const int h = g * hpg + j;
    {
      // Head j's loads have landed once at most the ops this wavefront issued
      // after them are pending (completion in issue order): the later
      // prologue loads, then per head m < j the loads of head m + R - 1 and
      // m's stores.  A partial chunk may skip stores: there wait for all.
      int n = 0;
      if (full) {
        const int m0 = j - (R - 1);
        if (m0 < 0) {
          n = (min(R - 2, hpg - 1) - j) * LDW;
          for (int m = 0; m < j; ++m) n += (m + R - 1 < hpg ? LDW : 0) + stw(m);
        } else {
          n = stw(m0);
          for (int m = m0 + 1; m < j; ++m) n += (m + R - 1 < hpg ? LDW : 0) + stw(m);
        }
      }
      wait_vmcnt_dyn(n);
      __syncthreads();  // head j is in everywhere; head j-1 and its partials are done everywhere
    }
    if (j + R - 1 < hpg) issue_head(j + R - 1, (j + R - 1) % R);
    if (j > 0 && fin) finish(j - 1, pAh, palast);
    const int pb = j & 1;
    float *tab = tab_of(pb);
    float *part = part_of(pb);
    unsigned char *hsl = smem + sl * F::HSLOT;
    const unsigned char *xs = hsl + F::OX;
    unsigned char *ys = hsl + F::OY;
    const unsigned char *hss = hsl + F::OH;
    const unsigned char *gss = hsl + F::OG;
    const float *dts = reinterpret_cast<const float *>(hsl + F::ODT);
    if (!full) {  // dy of tokens past the sequence's end is zero
      for (int i = threadIdx.x; i < (CQ - 1 - last) * 8; i += NT) {
        const int row = last + 1 + (i >> 3);
        *reinterpret_cast<u32x4 *>(ys + row * 128 + ((i & 7) << 4)) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    const float Ah = A[h];
    // per-token tables: a_l (log2), exp(a_l), w_s, dt_s, exp(a_last - a_s)
    const float dtv = tl <= last ? dts[tl] : 0.f;
    const float a = scan32b(dtv * Ah);
    const float alast = lane31(a);
    if (lane < 32) {
      tab[TA2 + tl] = a * kLog2eB;
      tab[TF + tl] = exp2b(a * kLog2eB);
      tab[TW + tl] = exp2b((alast - a) * kLog2eB) * dtv;
      tab[TDT + tl] = dtv;
      tab[TEL + tl] = exp2b((alast - a) * kLog2eB);
    }
    // the neighbour chunk's cumulative decay a' and its token factors
    float enl = 0.f;  // exp(a'_last)
    if (mode != NONE) {
      const float *ndts = reinterpret_cast<const float *>(hsl + F::ONDT);
      const float dtn = tl <= lastn ? ndts[tl] : 0.f;
      const float an = scan32b(dtn * Ah);
      const float anl = lane31(an);
      enl = exp2b(anl * kLog2eB);
      if (lane < 32)
        tab[TNW + tl] = mode == DH ? exp2b((anl - an) * kLog2eB) * dtn
                                   : (tl <= lastn ? exp2b(an * kLog2eB) : 0.f);
    }
    wsync();

    // ---- phase 1: one tile of the masked products per wavefront ----
    if (etile) {
      // E-layout (lt, st) = (qa, qb): l = 16 qa + 4 g4 + r, s = 16 qb + c16
      f32x4 e{};
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) e = mfma16b(rowx(ys, 16 * qa + c16, kq), rowx(xs, 16 * qb + c16, kq), e);
      const int sx = 16 * qb + c16;
      const f32x4 al = *reinterpret_cast<const f32x4 *>(tab + TA2 + 16 * qa + 4 * g4);
      const float as = tab[TA2 + sx], ds = tab[TDT + sx];
      float mv[4], elv[4], t1 = 0.f, ck = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = 16 * qa + 4 * g4 + r;
        const float lf = sx <= l ? exp2b(fminf(al[r] - as, 0.f)) : 0.f;
        mv[r] = z[r] * lf * ds;
        elv[r] = e[r] * lf * ds;
        const float pvr = e[r] * z[r] * lf;
        t1 += pvr;
        if (l > sx) ck += pvr * ds;
        float rk = sx < l ? pvr * ds : 0.f;
        rk = rowsum16(rk);
        if (c16 == 0) part[PRK + 32 * qb + l] = rk;
      }
      *reinterpret_cast<u32x2 *>(opm + qb * 1024 + lane * 16 + qa * 8) =
          u32x2{pack_bf16x2(mv[0], mv[1]), pack_bf16x2(mv[2], mv[3])};
      *reinterpret_cast<u32x2 *>(opel + qb * 1024 + lane * 16 + qa * 8) =
          u32x2{pack_bf16x2(elv[0], elv[1]), pack_bf16x2(elv[2], elv[3])};
      t1 = xsum32(xsum16(t1));
      ck = xsum32(xsum16(ck));
      if (lane < 16) {
        part[PC1 + 32 * qa + sx] = t1;
        part[PCK + 32 * qa + sx] = ck;
      }
      if (qa == qb && (c16 >> 2) == g4) {  // the diagonal E_ss
        const int r = c16 & 3;
        part[PDE + sx] = r == 0 ? e.x : r == 1 ? e.y : r == 2 ? e.z : e.w;
      }
    } else if (wave < 8) {
      // ET-layout (st, lt) = (qa, qb): s = 16 qa + 4 g4 + r, l = 16 qb + c16
      f32x4 et{};
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) et = mfma16b(rowx(xs, 16 * qa + c16, kq), rowx(ys, 16 * qb + c16, kq), et);
      const int lx = 16 * qb + c16;
      const f32x4 as = *reinterpret_cast<const f32x4 *>(tab + TA2 + 16 * qa + 4 * g4);
      const f32x4 ds = *reinterpret_cast<const f32x4 *>(tab + TDT + 16 * qa + 4 * g4);
      const float al = tab[TA2 + lx];
      float ev[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sx = 16 * qa + 4 * g4 + r;
        const float lf = sx <= lx ? exp2b(fminf(al - as[r], 0.f)) : 0.f;
        ev[r] = et[r] * lf * ds[r];
      }
      *reinterpret_cast<u32x2 *>(opelt + qb * 1024 + lane * 16 + qa * 8) =
          u32x2{pack_bf16x2(ev[0], ev[1]), pack_bf16x2(ev[2], ev[3])};
    }
    if (mode != NONE && wave >= 8) {
      // the derived state, in place over the loaded one: h_s = exp(a'_last)
      // h_s' + B'^T (w' x') (the chunk before), or g_e = exp(a'_last) g_e' +
      // C'^T (exp(a') dy') (the chunk after); tiles (p-tile, n-tile nd) with
      // lane (c16 = p, g4) holding n = 16 nd + 4 g4 + 0..3
      unsigned char *stile = mode == DH ? hsl + F::OH : hsl + F::OG;
      const unsigned char *ntile = hsl + F::ONX;
      const unsigned char *nbc = smem + F::ONBC;
      const int dw = wave & 7;  // this wavefront's place among those that derive
      const int nd = (F::DTW * dw) >> 2, pt0 = (F::DTW * dw) & 3;
      // B'^T (or C'^T) rows n, K = token s, scaled by the token factors once
      const u32x4 t = trn(nbc, N * 2, 4 * g4, 16 + 4 * g4, 16 * nd, true);
      const f32x4 f0 = *reinterpret_cast<const f32x4 *>(tab + TNW + 4 * g4);
      const f32x4 f1 = *reinterpret_cast<const f32x4 *>(tab + TNW + 16 + 4 * g4);
      const u32x4 aop{pack_bf16x2(bf16lo(t.x) * f0.x, bf16hi(t.x) * f0.y),
                      pack_bf16x2(bf16lo(t.y) * f0.z, bf16hi(t.y) * f0.w),
                      pack_bf16x2(bf16lo(t.z) * f1.x, bf16hi(t.z) * f1.y),
                      pack_bf16x2(bf16lo(t.w) * f1.z, bf16hi(t.w) * f1.w)};
#pragma unroll
      for (int i = 0; i < F::DTW; ++i) {
        const int ptd = pt0 + i;
        const u32x4 bop = trn(ntile, 128, 4 * g4, 16 + 4 * g4, 16 * ptd, false);
        const f32x4 d = mfma16b(aop, bop, f32x4{});
        const int p = 16 * ptd + c16, n = 16 * nd + 4 * g4;
        u32x2 *dst = reinterpret_cast<u32x2 *>(stile + p * (N * 2) + (((n >> 3) ^ swz2<NCB>(p)) << 4) + (n & 7) * 2);
        const u32x2 o = *dst;
        *dst = u32x2{pack_bf16x2(enl * bf16lo(o.x) + d.x, enl * bf16hi(o.x) + d.y),
                     pack_bf16x2(enl * bf16lo(o.y) + d.z, enl * bf16hi(o.y) + d.w)};
      }
    }
    __syncthreads();  // the head's operands, sums of phase 1 and derived state are in LDS

    // ---- phase 2 ----
    const float Dh = Dv ? Dv[h] : 0.f;
    {
      // wavefronts 0-7 on the g_e side, 8-15 on the h_s side; dBa holds this
      // wavefront's tiles of dB (g_e side) or dC
      // n-tile of dB or dC, s-tiles t0d .. t0d + NTW - 1
      const int nt = (NTW * (wave & 7)) >> 1, t0d = (NTW * (wave & 7)) & 1;
      const int sx = 16 * sh + c16, col = 16 * pt + 4 * g4;
      const int ro = sx * 128 + (((col >> 3) ^ swz2<8>(sx)) << 4) + (col & 7) * 2;
      const u32x2 dv = *reinterpret_cast<const u32x2 *>(ys + ro);
      if (wave < 8) {
        u32x4 gr[KQ];
#pragma unroll
        for (int q = 0; q < KQ; ++q) gr[q] = rown(gss, 16 * pt + c16, q);
        // dx tile (p-tile pt, s-tile sh): dy^T M + w_s g_e B^T + D dy; q_s partial
        const u32x4 dyt = trn(ys, 128, 4 * g4, 16 + 4 * g4, 16 * pt, false);
        const u32x4 mop = *reinterpret_cast<const u32x4 *>(opm + sh * 1024 + lane * 16);
        f32x4 acc = mfma16b(dyt, mop, f32x4{});
        f32x4 gb{};
#pragma unroll
        for (int q = 0; q < KQ; ++q) gb = mfma16b(gr[q], rown(bsm, 16 * sh + c16, q), gb);
        const float ws = tab[TW + sx];
        const u32x2 xv = *reinterpret_cast<const u32x2 *>(xs + ro);
        float o0 = acc.x + ws * gb.x + Dh * bf16lo(dv.x);
        float o1 = acc.y + ws * gb.y + Dh * bf16hi(dv.x);
        float o2 = acc.z + ws * gb.z + Dh * bf16lo(dv.y);
        float o3 = acc.w + ws * gb.w + Dh * bf16hi(dv.y);
        if constexpr (ACC) {
          const u32x2 av = *reinterpret_cast<const u32x2 *>(hsl + F::OAX + ro);
          o0 += bf16lo(av.x);
          o1 += bf16hi(av.x);
          o2 += bf16lo(av.y);
          o3 += bf16hi(av.y);
        }
        if (sx <= last)
          *reinterpret_cast<u32x2 *>(dx + (t0 + sx) * ldx + (int64_t)h * P + col) =
              u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        float qv = bf16lo(xv.x) * gb.x + bf16hi(xv.x) * gb.y + bf16lo(xv.y) * gb.z + bf16hi(xv.y) * gb.w;
        qv = xsum32(xsum16(qv));
        if (lane < 16) part[PQ + 32 * pt + sx] = qv;
        // dB tiles: C^T EL + (g_e^T x^T) w_s
        const u32x4 ct = trn(csm, N * 2, 4 * g4, 16 + 4 * g4, 16 * nt, true);
        u32x4 gsT[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
          gsT[kq] = trn(gss, N * 2, 32 * kq + 8 * g4, 32 * kq + 8 * g4 + 4, 16 * nt, true);
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int t = t0d + i;
          const u32x4 elop = *reinterpret_cast<const u32x4 *>(opel + t * 1024 + lane * 16);
          dBa[i] = mfma16b(ct, elop, dBa[i]);
          f32x4 gx{};
#pragma unroll
          for (int kq = 0; kq < 2; ++kq) gx = mfma16b(gsT[kq], rowx(xs, 16 * t + c16, kq), gx);
          dBa[i] += gx * tab[TW + 16 * t + c16];
        }
      } else {
        u32x4 hr[KQ];
#pragma unroll
        for (int q = 0; q < KQ; ++q) hr[q] = rown(hss, 16 * pt + c16, q);
        f32x4 hc{};
#pragma unroll
        for (int q = 0; q < KQ; ++q) hc = mfma16b(hr[q], rown(csm, 16 * sh + c16, q), hc);
        // v_l partial dy_l . (h_s C_l)
        float vv = bf16lo(dv.x) * hc.x + bf16hi(dv.x) * hc.y + bf16lo(dv.y) * hc.z + bf16hi(dv.y) * hc.w;
        vv = xsum32(xsum16(vv));
        if (lane < 16) part[PV + 32 * pt + sx] = vv;
        if (sh == 0) {  // <g_e, h_s> over p-tile pt: the trace of (g_e h_s^T) on that tile
          f32x4 gh4{};
#pragma unroll
          for (int q = 0; q < KQ; ++q) gh4 = mfma16b(rown(gss, 16 * pt + c16, q), hr[q], gh4);
          const int r = c16 - 4 * g4;
          float gh = r == 0 ? gh4.x : r == 1 ? gh4.y : r == 2 ? gh4.z : r == 3 ? gh4.w : 0.f;
          gh = rowsum16(gh);
          gh = xsum32(xsum16(gh));
          if (lane == 0) part[PGH + pt] = gh;
        }
        // dC tiles: B^T EL^T + (h_s^T dy^T) exp(a_l)
        const u32x4 bt = trn(bsm, N * 2, 4 * g4, 16 + 4 * g4, 16 * nt, true);
        u32x4 hsT[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
          hsT[kq] = trn(hss, N * 2, 32 * kq + 8 * g4, 32 * kq + 8 * g4 + 4, 16 * nt, true);
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int t = t0d + i;
          const u32x4 eltop = *reinterpret_cast<const u32x4 *>(opelt + t * 1024 + lane * 16);
          dBa[i] = mfma16b(bt, eltop, dBa[i]);
          f32x4 hy{};
#pragma unroll
          for (int kq = 0; kq < 2; ++kq) hy = mfma16b(hsT[kq], rowx(ys, 16 * t + c16, kq), hy);
          dBa[i] += hy * tab[TF + 16 * t + c16];
        }
      }
    }
    pAh = Ah;
    palast = alast;
  }
  __syncthreads();  // the last head's partials are in everywhere
  if (fin) finish(hpg - 1, pAh, palast);

  // ---- dB, dC of the chunk's rows: lane column s, rows n = 16 nt + 4 g4 + r ----
  {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = (NTW * (wave & 7)) >> 1, t = ((NTW * (wave & 7)) & 1) + i;
      const int sx = 16 * t + c16;
      if (sx <= last)
        *reinterpret_cast<f32x4 *>((wave < 8 ? dB : dC) + (t0 + sx) * ldb + (int64_t)g * N +
                                   16 * nt + 4 * g4) = dBa[i];
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_f32(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_bwd_reverse(const void *dy, const float *dt, const float *A, const void *C,
                              const float *dfinal, const int32_t *cu, int64_t L, int64_t T,
                              int rows, int H, int N, int G, void *gsave, float *dinit,
                              int64_t nseg, int seg_len, float *gseg, float *aseg, float *gin,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if ((N != 64 && N != 128) || (nseg > 0 && (seg_len < 32 || seg_len % 32 != 0)))
    return hipErrorInvalidValue;
  const int segc = seg_len / 32;
  const uint16_t *d = static_cast<const uint16_t *>(dy);
  const uint16_t *c = static_cast<const uint16_t *>(C);
  uint16_t *gs = static_cast<uint16_t *>(gsave);
  auto rev = [&](auto kern, int64_t units, const float *gstart, float *gout) {
    hipLaunchKernelGGL(kern, dim3(xcd_grid(units, H / 2)), dim3(256), 0, stream, d, dt, A, c, gstart,
                       cu, L, T, rows, H, G, segc, gs, gout, aseg);
    return hipGetLastError();
  };
  if (nseg == 0) {
    return N == 64 ? rev(k_bwd_reverse<64, RV_FULL, kRevSlots>, rows, dfinal, dinit)
                   : rev(k_bwd_reverse<128, RV_FULL, kRevSlots>, rows, dfinal, dinit);
  }
  hipError_t e = N == 64 ? rev(k_bwd_reverse<64, RV_SEGSUM, kRevSlots>, nseg, nullptr, gseg)
                         : rev(k_bwd_reverse<128, RV_SEGSUM, kRevSlots>, nseg, nullptr, gseg);
  if (e != hipSuccess) return e;
  const int PN = 64 * N;
  hipLaunchKernelGGL(k_bwd_gpass, dim3(PN / 1024, H, rows), dim3(256), 0, stream, gseg, aseg,
                     dfinal, cu, L, T, rows, H, PN, seg_len, gin, dinit);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return N == 64 ? rev(k_bwd_reverse<64, RV_SEG, kRevSlots>, nseg, gin, nullptr)
                 : rev(k_bwd_reverse<128, RV_SEG, kRevSlots>, nseg, gin, nullptr);
}

hipError_t launch_bwd_chunk(const void *x, const float *dt, const float *A, const void *B,
                            const void *C, const float *D, const void *dy, const void *hsave,
                            int hsld, const void *gsave, const int32_t *cu, int64_t L, int64_t T,
                            int rows, int64_t nchunks, int H, int N, int G, const void *dxacc,
                            void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                            hipStream_t stream) {
  if (nchunks == 0) return hipSuccess;
  if (dxacc && N != 128) return hipErrorInvalidValue;
  if (hsld < N || hsld % 8) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((nchunks * G + 7) / 8 * 8));
  const uint16_t *xi = static_cast<const uint16_t *>(x);
  const uint16_t *bi = static_cast<const uint16_t *>(B);
  const uint16_t *ci = static_cast<const uint16_t *>(C);
  const uint16_t *di = static_cast<const uint16_t *>(dy);
  const uint16_t *hs = static_cast<const uint16_t *>(hsave);
  const uint16_t *gs = static_cast<const uint16_t *>(gsave);
  uint16_t *dxo = static_cast<uint16_t *>(dx);
  // two ring slots (one head in flight ahead); one block a CU (the LDS holds
  // one), of 16 wavefronts: four a SIMD hide more of each head's chain of
  // dependent steps than two did
  // (dxacc: dx adds into what dxacc holds, read tile by tile before each is
  // written, so dxacc may be dx itself)
  const uint16_t *dxa = static_cast<const uint16_t *>(dxacc);
  if (N == 64)
    hipLaunchKernelGGL((k_bwd_chunk<64, 2>), grid, dim3(1024), 0, stream, xi, dt, A, bi, ci, D,
                       di, hs, hsld, gs, cu, L, T, rows, nchunks, H, G, dxa, dxo, ddt, dA, dB, dC,
                       dD);
  else if (N == 128 && dxa)
    hipLaunchKernelGGL((k_bwd_chunk<128, 2, true>), grid, dim3(1024), 0, stream, xi, dt, A, bi, ci,
                       D, di, hs, hsld, gs, cu, L, T, rows, nchunks, H, G, dxa, dxo, ddt, dA, dB,
                       dC, dD);
  else if (N == 128)
    hipLaunchKernelGGL((k_bwd_chunk<128, 2>), grid, dim3(1024), 0, stream, xi, dt, A, bi, ci, D,
                       di, hs, hsld, gs, cu, L, T, rows, nchunks, H, G, dxa, dxo, ddt, dA, dB, dC,
                       dD);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {
// rows x units 16-byte pieces from rows src_ld bytes apart to rows dst_ld
// bytes apart (a column block of a row-major tensor into a packed one, or back)
__global__ __launch_bounds__(256) void k_copy2d16(const unsigned char *__restrict__ src,
                                                  int64_t src_ld, unsigned char *__restrict__ dst,
                                                  int64_t dst_ld, int64_t rows, int units) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * units) return;
  const int64_t r = i / units, u = i - r * units;
  *reinterpret_cast<u32x4 *>(dst + r * dst_ld + u * 16) =
      *reinterpret_cast<const u32x4 *>(src + r * src_ld + u * 16);
}
// acc += add (fp32)
__global__ __launch_bounds__(256) void k_add_f32(float *__restrict__ acc,
                                                 const float *__restrict__ add, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) acc[i] += add[i];
}
}  // namespace

hipError_t launch_copy2d16(const void *src, int64_t src_ld, void *dst, int64_t dst_ld,
                           int64_t rows, int units, hipStream_t stream) {
  const int64_t n = rows * units;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy2d16, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const unsigned char *>(src), src_ld,
                     static_cast<unsigned char *>(dst), dst_ld, rows, units);
  return hipGetLastError();
}

hipError_t launch_add_f32(float *acc, const float *add, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_add_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     acc, add, n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     p, n);
  return hipGetLastError();
}

}  // namespace ssd
