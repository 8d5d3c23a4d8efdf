// libssd: chunk_state on bf16 MFMA (gfx950).
//
// For chunk c and head h:  S[p][n] = sum_l x_l[p] * w_l * B_l[n],
//   w_l = exp(acum_last - acum_l) * dt_l,
// the state a chunk leaves behind when it starts from zero (page "Mamba-2
// Architecture: State Space Duality Explained", "2. The Chunked SSD
// Algorithm", item 2; the page's listing omits the decay and step-size
// weights, which the recurrence implies).  It is a [P x Q] . [Q x N]
// contraction over the chunk's tokens.
//
// Design.  The heads of a group share B, so a block takes a run of heads of
// one chunk (block = (chunk, group, run of hb heads), 8 wavefronts, XCD-aware
// order).  The chunk's B is staged in LDS once and each wavefront keeps its
// MFMA B-operands in registers: its 32x32 output tile's 32 columns n over all
// Q tokens, read by transposing LDS reads (ds_read_b64_tr_b16) so the
// contracted token index runs along each lane's registers.  Per head:
//   1. S of the previous head, staged in LDS, is rounded to bf16 (the io
//      precision, like the hprev the hand-off writes) and stored;
//      this head's x, already in its ring slot, is scaled in place by w_l in
//      fp32 and rounded once to bf16;
//   2. a later head's x, acum and dt go into the slot the previous head
//      freed by direct-to-LDS loads (a three-slot ring keeps two heads in
//      flight where the LDS allows, else two slots one head); each wavefront
//      waits for exactly the operations it issued after a head's loads;
//   3. each wavefront forms its tile(s) on v_mfma_f32_32x32x16_bf16 from
//      transposing reads of the scaled x, and stages them in LDS (fp32).
// With N = 64 the four tiles are split over K between wavefront pairs and the
// two halves are added when S is stored; with N = 256 a wavefront owns two
// tiles.  Token rows past a partial chunk's end repeat its last row, which the
// zero dt there cancels.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

// LDS bytes of k_chunk_state_hb<Q, N, R> (P = 64, 8 wavefronts): R slots of a
// head's x and its acum/dt, the S staging (split over K when there are fewer
// 32x32 tiles than wavefronts); B is staged over the same space first.
constexpr int cs_lds_bytes(int Q, int N, int R) {
  const int tiles = 2 * (N / 32), ksplit = tiles < 8 ? 8 / tiles : 1;
  const int main = R * (Q * 64 * 2) + R * (2 * Q * 4) + ksplit * 64 * (N + 8) * 4;
  return main > Q * N * 2 ? main : Q * N * 2;
}

template <int Q, int N, int R>
__global__ __launch_bounds__(512, 1) void k_chunk_state_hb(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm, const float *__restrict__ acum,
    const float *__restrict__ dtq, ChunkGeom geom, int nc, int H, int G, int hb, int nkb,
    uint16_t *__restrict__ states) {
  constexpr int P = 64;
  constexpr int NT = 512, NW = 8;
  constexpr int TPN = P / 32;                            // p tiles
  constexpr int TILES = TPN * (N / 32);                  // 32x32 output tiles
  constexpr int TPW = TILES > NW ? TILES / NW : 1;       // tiles per wavefront
  constexpr int KSPLIT = TILES < NW ? NW / TILES : 1;    // wavefronts per tile (split over K)
  constexpr int TG = NW / KSPLIT;                        // wavefronts over distinct tiles
  constexpr int KS = Q / 16 / KSPLIT;                    // K steps per wavefront
  static_assert(TG * TPW == TILES && KS * 16 * KSPLIT == Q, "work split");
  constexpr int NCX = P / 8, NCB = N / 8;                // 16-byte chunks per x / B row
  constexpr int XB = Q * P * 2, BB = Q * N * 2, ADB = 2 * Q * 4;
  constexpr int LSS = N + 8;                             // S staging row (fp32) + pad
  constexpr int SSB = P * LSS * 4;
  constexpr int XI = XB / 1024 / NW, BI = BB / 1024 / NW;
  static_assert(XI * NW * 1024 == XB && BI * NW * 1024 == BB, "1 KB loads");
  // [XS x R][AD x R][SS x KSPLIT]; B is staged over all of it first.  R ring
  // slots: the loads of R - 1 heads are in flight while a head computes.
  constexpr int AD = R * XB, SS = AD + R * ADB;
  constexpr int MAIN = SS + KSPLIT * SSB;
  constexpr int SC = P * N / 4 / NT;  // S stores a thread issues per head
  static_assert(R >= 2 && SC * NT * 4 == P * N, "ring, S stores");
  constexpr int TOTAL = MAIN > BB ? MAIN : BB;
  static_assert(TOTAL == cs_lds_bytes(Q, N, R) && TOTAL <= 160 * 1024, "LDS");
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

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = wave % TG;  // tile group
  const int kp = wave / TG;  // K part
  const int ldx32 = H * P;   // row offsets inside a chunk: Q * H * P < 2^31
  const int64_t xrow0 = ci.t0 * (int64_t)ldx32;

  // Transposing read of a 16-token K step for MFMA operands: lane (col, kg)
  // receives element [r0 + 8kg + j][c0 + col], j = 0..7, of a row-major bf16
  // tile with `ncc` 16-byte chunks per row (chunk-swizzled), as 4 words in K
  // order.
  auto tr_op = [](int lane, const unsigned char *tile, int ncc, int r0, int c0) {
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
  };
  auto issue_head = [&](int lane, int hh, int slot) {
    const uint16_t *xb = x + xrow0 + (int64_t)hh * P;
    unsigned char *xs = smem + slot * XB;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int m = (wave * XI + i) * 64 + lane;
      const int r = m / NCX, cc = (m % NCX) ^ chunk_swz(m / NCX, NCX);
      load_lds16(xb + min(r, ci.len - 1) * ldx32 + cc * 8, xs + (wave * XI + i) * 1024);
    }
    if (wave < 2 && lane < Q / 4)  // wavefront 0: acum, 1: dt
      load_lds16((wave == 0 ? acum : dtq) + ((int64_t)c * H + hh) * Q + lane * 4,
                 smem + AD + slot * ADB + wave * (Q * 4));
  };
  // vector-memory ops a wavefront issues per head load (x pieces, plus acum
  // or dt for wavefronts 0 and 1)
  const int LC = XI + (wave < 2 ? 1 : 0);
  auto store_s = [&](int t, int hh) {
    uint16_t *out = states + ((int64_t)c * H + hh) * (P * N);
#pragma unroll
    for (int i = 0; i < P * N / 4 / NT; ++i) {
      const int u = t + i * NT;
      const int p = u / (N / 4), c4 = u % (N / 4);
      f32x4 v = *reinterpret_cast<const f32x4 *>(smem + SS + (p * LSS + 4 * c4) * 4);
#pragma unroll
      for (int k = 1; k < KSPLIT; ++k)
        v += *reinterpret_cast<const f32x4 *>(smem + SS + k * SSB + (p * LSS + 4 * c4) * 4);
      // streaming stores: the next pass reads S once, from HBM
      __builtin_nontemporal_store(u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)},
                                  reinterpret_cast<u32x2 *>(out + p * N + 4 * c4));
    }
  };

  // ---- B operands, once per block
  {
    const uint16_t *bb = Bm + ci.t0 * (int64_t)G * N + (int64_t)g * N;
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int m = (wave * BI + i) * 64 + lane;
      const int r = m / NCB, cc = (m % NCB) ^ chunk_swz(m / NCB, NCB);
      load_lds16(bb + (int64_t)min(r, ci.len - 1) * G * N + cc * 8, smem + (wave * BI + i) * 1024);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  u32x4 bop[TPW][KS];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tn = (tg * TPW + i) / TPN;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bop[i][ks] = tr_op(tid & 63, smem, NCB, 16 * (kp * KS + ks), 32 * tn);
  }
  __syncthreads();  // B consumed: the rings are free
#pragma unroll
  for (int j = 0; j < R - 1; ++j)
    if (j < nh) issue_head(tid & 63, hfirst + j, j);

  int slot = 0;
#pragma unroll 1
  for (int hi = 0; hi < nh; ++hi) {
    const int hh = hfirst + hi;
    // lane indices re-read per head, so lane-dependent addresses are formed
    // where they are used rather than kept live across heads
    int t = tid;
    asm volatile("" : "+v"(t));
    const int lane = t & 63, col = lane & 31, kg = lane >> 5;
    unsigned char *xs = smem + slot * XB;
    const float *sa = reinterpret_cast<const float *>(smem + AD + slot * ADB);
    const float *sd = sa + Q;

    {
      // this head's loads have landed once at most the ops issued after them
      // are pending (completion in issue order): the prologue's later loads,
      // then per head m < hi the S stores of head m - 1 and the loads of head
      // m + R - 1
      int n = 0;
      if (hi < R - 1) {
        n = (min(R - 1, nh) - 1 - hi) * LC;
        for (int m = 0; m < hi; ++m) n += (m > 0 ? SC : 0) + (m + R - 1 < nh ? LC : 0);
      } else {
        for (int m = hi - R + 2; m < hi; ++m) n += SC + (m + R - 1 < nh ? LC : 0);
      }
      wait_vmcnt_dyn(n);
    }
    // the previous head's S tile (LDS writes) complete before the barrier: the
    // compiler does not always add this wait at the loop's back edge
    wait_lgkmcnt0();
    __syncthreads();  // ... for every thread; the previous head is done everywhere
    if (hi > 0) store_s(t, hh - 1);
    {  // x_l *= w_l in place (fp32, one rounding)
      const float alast = sa[Q - 1];
#pragma unroll
      for (int i = 0; i < Q * NCX / NT; ++i) {
        const int m = t + i * NT;
        const int l = m / NCX;
        const float w = __expf(alast - sa[l]) * sd[l];
        u32x4 *pc = reinterpret_cast<u32x4 *>(xs + m * 16);
        const u32x4 v = *pc;
        u32x4 o;
        o.x = pack_bf16x2(bf16lo(v.x) * w, bf16hi(v.x) * w);
        o.y = pack_bf16x2(bf16lo(v.y) * w, bf16hi(v.y) * w);
        o.z = pack_bf16x2(bf16lo(v.z) * w, bf16hi(v.z) * w);
        o.w = pack_bf16x2(bf16lo(v.w) * w, bf16hi(v.w) * w);
        *pc = o;
      }
    }
    __syncthreads();  // scaled x ready; staged S read out
    const int slp = slot == 0 ? R - 1 : slot - 1;  // head hi - 1's slot, free now
    if (hi + R - 1 < nh) issue_head(lane, hh + R - 1, slp);

#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = tg * TPW + i;
      const int tp = tt % TPN, tn = tt / TPN;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 a = tr_op(lane, xs, NCX, 16 * (kp * KS + ks), 32 * tp);
        acc = mfma32x32x16(as_bf16x8(a), as_bf16x8(bop[i][ks]), acc);
      }
      float *ss = reinterpret_cast<float *>(smem + SS + kp * SSB);
#pragma unroll
      for (int r = 0; r < 16; ++r) ss[(tp * 32 + acc_row(r, kg)) * LSS + tn * 32 + col] = acc[r];
    }
    slot = slot == R - 1 ? 0 : slot + 1;
  }
  __syncthreads();
  store_s(tid, hfirst + nh - 1);
}

}  // namespace

bool chunk_state_bf16_supported(int P, int N, int Q) {
  return P == 64 && (N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

template <int Q, int P, int N>
static void launch_cs(const void *x, const void *B, const float *acum, const float *dtq,
                      uint16_t *states, const Geometry &geo, hipStream_t stream) {
  static_assert(P == 64, "head dimension");
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  int nkb = 1;
  const int hb = pick_heads_per_block(geo.nc_max, geo.H, geo.G, device_cus(), 1.0, nkb);
  // three ring slots where the LDS allows (two heads' loads in flight)
  constexpr int R = cs_lds_bytes(Q, N, 3) <= 160 * 1024 ? 3 : 2;
  hipLaunchKernelGGL((k_chunk_state_hb<Q, N, R>), dim3(xcd_grid(geo.nc_max, geo.G * nkb)), dim3(512),
                     0, stream, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                     acum, dtq, cg, (int)geo.nc_max, geo.H, geo.G, hb, nkb, states);
}

template <int Q>
static bool dispatch_cs_n(const void *x, const void *B, const float *acum, const float *dtq,
                          uint16_t *states, const Geometry &geo, hipStream_t stream) {
  switch (geo.N) {
    case 64: launch_cs<Q, 64, 64>(x, B, acum, dtq, states, geo, stream); return true;
    case 128: launch_cs<Q, 64, 128>(x, B, acum, dtq, states, geo, stream); return true;
    case 256: launch_cs<Q, 64, 256>(x, B, acum, dtq, states, geo, stream); return true;
    default: return false;
  }
}

hipError_t launch_chunk_state_bf16(const void *x, const void *B, const float *acum,
                                   const float *dtq, void *states_v, const Geometry &geo,
                                   hipStream_t stream) {
  uint16_t *states = static_cast<uint16_t *>(states_v);
  if (geo.nc_max == 0) return hipSuccess;
  if (!chunk_state_bf16_supported(geo.P, geo.N, geo.Q)) return hipErrorInvalidValue;
  bool ok = false;
  switch (geo.Q) {
    case 64: ok = dispatch_cs_n<64>(x, B, acum, dtq, states, geo, stream); break;
    case 128: ok = dispatch_cs_n<128>(x, B, acum, dtq, states, geo, stream); break;
    case 256: ok = dispatch_cs_n<256>(x, B, acum, dtq, states, geo, stream); break;
  }
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssd
