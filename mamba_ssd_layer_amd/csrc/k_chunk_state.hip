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
// Design.  x [T,H,P] and B [T,G,N] keep the token index strided, while an MFMA
// operand needs runs along the contracted (token) index, so both tiles are
// transposed on their way into LDS: each thread loads 4 token rows x 8
// columns (four 16-byte loads), scales x by w_l in fp32, repacks column-wise
// into bf16 pairs and writes 8-byte runs of 4 tokens.  The chunk goes through
// in stages of 64 tokens; a stage's global loads are issued before the
// previous stage's MFMAs, so only the first one waits on memory.  The MFMA then reads
// 16-byte K-runs (8 tokens) per lane.  Padded LDS rows (K + 8 elements,
// 144 bytes) keep the 16-byte column reads of 16 consecutive rows on distinct
// banks.  Block = (chunk, head) in XCD-aware order, 4 wavefronts; the (P/32) x (N/32) output tiles
// of 32x32 are split evenly over the wavefronts; fp32 accumulation, fp32 S.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kStateThreads = 256;
constexpr int kKT = 64;         // tokens per LDS stage
constexpr int kLDK = kKT + 8;   // padded LDS row (bf16 elements)

// A stage is kKT token rows of a [tokens x D] bf16 matrix (row stride `ld`
// elements), moved in units of 4 rows x 8 columns: four 16-byte loads per
// unit, row quad fastest across threads.  Rows at or past `len` are zeros and
// never read from global memory.
template <int D>
struct Stage {
  static constexpr int RQ = kKT / 4;  // row quads per stage
  static constexpr int UNITS = RQ * (D / 8);
  static constexpr int PER_THREAD = (UNITS + kStateThreads - 1) / kStateThreads;
  u32x4 r[PER_THREAD][4];

  __device__ __forceinline__ void load(const uint16_t *__restrict__ src, int64_t ld, int kt,
                                       int len) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int u = threadIdx.x + i * kStateThreads;
      const int rq = u % RQ;
      const int cb = u / RQ;
      const int l0 = kt + rq * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[i][e] = (u < UNITS && l0 + e < len)
                      ? *reinterpret_cast<const u32x4 *>(src + (int64_t)(l0 + e) * ld + cb * 8)
                      : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // Writes the stage transposed, dst[d][l] with row length kLDK: column-wise
  // bf16 pairs, 8-byte runs of 4 tokens.  If `wt` is given, row l is scaled by
  // wt[l] in fp32 and rounded once to bf16.
  __device__ __forceinline__ void store(const float *wt, int kt, uint16_t (*dst)[kLDK]) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int u = threadIdx.x + i * kStateThreads;
      if (u >= UNITS) continue;
      const int rq = u % RQ;
      const int cb = u / RQ;
      u32x2 out[8];
      if (wt) {
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = wt[kt + rq * 4 + e];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // columns 2m (low halves) and 2m+1 (high halves) of word m
          out[2 * m].x = pack_bf16x2(bf16lo(r[i][0][m]) * w[0], bf16lo(r[i][1][m]) * w[1]);
          out[2 * m].y = pack_bf16x2(bf16lo(r[i][2][m]) * w[2], bf16lo(r[i][3][m]) * w[3]);
          out[2 * m + 1].x = pack_bf16x2(bf16hi(r[i][0][m]) * w[0], bf16hi(r[i][1][m]) * w[1]);
          out[2 * m + 1].y = pack_bf16x2(bf16hi(r[i][2][m]) * w[2], bf16hi(r[i][3][m]) * w[3]);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          out[2 * m].x = pair_lo(r[i][0][m], r[i][1][m]);
          out[2 * m].y = pair_lo(r[i][2][m], r[i][3][m]);
          out[2 * m + 1].x = pair_hi(r[i][0][m], r[i][1][m]);
          out[2 * m + 1].y = pair_hi(r[i][2][m], r[i][3][m]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        *reinterpret_cast<u32x2 *>(&dst[cb * 8 + jj][rq * 4]) = out[jj];
      }
    }
  }
};

template <int Q, int P, int N>
__global__ __launch_bounds__(kStateThreads) void k_chunk_state_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ Bm, const float *__restrict__ acum,
    const float *__restrict__ dtq, ChunkGeom geom, int nc, int H, int G,
    float *__restrict__ states) {
  static_assert(P % 32 == 0 && N % 32 == 0, "tile shape");
  constexpr int TP = P / 32;
  constexpr int TN = N / 32;
  constexpr int NT = TP * TN;
  static_assert(NT % 4 == 0, "tiles must split evenly over 4 wavefronts");
  constexpr int TPW = NT / 4;

  __shared__ __align__(16) uint16_t xs[P][kLDK];
  __shared__ __align__(16) uint16_t bs[N][kLDK];
  __shared__ float sw[Q];

  int c, h;
  xcd_chunk_head(H, c, h);
  if (c >= nc) return;
  const int g = h / (H / G);
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;

  const int64_t ch = (int64_t)c * H + h;
  const uint16_t *xbase = x + ci.t0 * (int64_t)H * P + (int64_t)h * P;
  const uint16_t *bbase = Bm + ci.t0 * (int64_t)G * N + (int64_t)g * N;
  Stage<P> xst;
  Stage<N> bst;
  // the first stage's loads go out before anything waits
  xst.load(xbase, (int64_t)H * P, 0, ci.len);
  bst.load(bbase, (int64_t)G * N, 0, ci.len);
  {
    const float *ac = acum + ch * Q;
    const float *dq = dtq + ch * Q;
    const float alast = ac[Q - 1];
    for (int l = threadIdx.x; l < Q; l += kStateThreads) sw[l] = __expf(alast - ac[l]) * dq[l];
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int kg = lane >> 5;

  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};

#pragma unroll 1
  for (int kt = 0; kt < ci.len; kt += kKT) {
    xst.store(sw, kt, xs);
    bst.store(nullptr, kt, bs);
    __syncthreads();
    if (kt + kKT < ci.len) {  // next stage's loads overlap this stage's MFMAs
      xst.load(xbase, (int64_t)H * P, kt + kKT, ci.len);
      bst.load(bbase, (int64_t)G * N, kt + kKT, ci.len);
    }
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = wave * TPW + i;
        const int tp = t % TP;
        const int tn = t / TP;
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&xs[tp * 32 + col][ks * 16 + kg * 8]);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(&bs[tn * 32 + col][ks * 16 + kg * 8]);
        acc[i] = mfma32x32x16(as_bf16x8(a), as_bf16x8(b), acc[i]);
      }
    }
    __syncthreads();
  }

  float *out = states + ch * (int64_t)P * N;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave * TPW + i;
    const int tp = t % TP;
    const int tn = t / TP;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = tp * 32 + acc_row(r, kg);
      out[p * N + tn * 32 + col] = acc[i][r];
    }
  }
}

}  // namespace

bool chunk_state_bf16_supported(int P, int N, int Q) {
  return P == 64 && (N == 64 || N == 128 || N == 256) && (Q == 64 || Q == 128 || Q == 256);
}

template <int Q, int P, int N>
static void launch_cs(const void *x, const void *B, const float *acum, const float *dtq,
                      float *states, const Geometry &geo, hipStream_t stream) {
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  hipLaunchKernelGGL((k_chunk_state_bf16<Q, P, N>), dim3(xcd_grid(geo.nc_max, geo.H)),
                     dim3(kStateThreads), 0, stream, static_cast<const uint16_t *>(x),
                     static_cast<const uint16_t *>(B), acum, dtq, cg, (int)geo.nc_max, geo.H,
                     geo.G, states);
}

template <int Q>
static bool dispatch_cs_n(const void *x, const void *B, const float *acum, const float *dtq,
                          float *states, const Geometry &geo, hipStream_t stream) {
  switch (geo.N) {
    case 64: launch_cs<Q, 64, 64>(x, B, acum, dtq, states, geo, stream); return true;
    case 128: launch_cs<Q, 64, 128>(x, B, acum, dtq, states, geo, stream); return true;
    case 256: launch_cs<Q, 64, 256>(x, B, acum, dtq, states, geo, stream); return true;
    default: return false;
  }
}

hipError_t launch_chunk_state_bf16(const void *x, const void *B, const float *acum,
                                   const float *dtq, float *states, const Geometry &geo,
                                   hipStream_t stream) {
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
