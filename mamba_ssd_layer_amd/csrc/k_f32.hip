// libssd: chunk_state and chunk_scan for fp32 inputs, on the fp32 vector ALU
// (gfx950).  Same arithmetic as the bf16 MFMA kernels but every product and
// sum in fp32, for any head dim / state size that is a multiple of 16 up to
// 256.  Meant for small problems and fp32 checking; the bf16 path is the
// throughput path.
//
//   chunk_state: S[p][n] = sum_l x_l[p] exp(acum_last - acum_l) dt_l B_l[n]
//   chunk_scan:  y_l = sum_{s<=l} (C_l . B_s) exp(acum_l - acum_s) dt_s x_s
//                      + exp(acum_l) C_l hprev^T + D x_l
// (page "Mamba-2 Architecture: State Space Duality Explained", "2. The Chunked
// SSD Algorithm", items 1-2, with the decay weights the recurrence implies).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kF32Threads = 256;
constexpr int kRowTile = 16;  // output tokens per pass in chunk_scan

// Block = (chunk, head).  Thread = output elements (p, n), n fastest.
__global__ __launch_bounds__(kF32Threads) void k_chunk_state_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ acum,
    const float *__restrict__ dtq, ChunkGeom geom, int H, int G, int P, int N,
    float *__restrict__ states) {
  extern __shared__ float sw[];  // [Q]
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int g = h / (H / G);
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;
  const int Q = geom.Q;
  const int64_t ch = (int64_t)c * H + h;
  const float alast = acum[ch * Q + Q - 1];
  for (int l = threadIdx.x; l < Q; l += kF32Threads)
    sw[l] = __expf(alast - acum[ch * Q + l]) * dtq[ch * Q + l];
  __syncthreads();
  const int64_t ldx = (int64_t)H * P;
  const int64_t ldb = (int64_t)G * N;
  const float *xb = x + ci.t0 * ldx + (int64_t)h * P;
  const float *bb = Bm + ci.t0 * ldb + (int64_t)g * N;
  float *out = states + ch * (int64_t)P * N;
  for (int e = threadIdx.x; e < P * N; e += kF32Threads) {
    const int p = e / N;
    const int n = e - p * N;
    float acc = 0.f;
    for (int l = 0; l < ci.len; ++l) acc += xb[l * ldx + p] * sw[l] * bb[l * ldb + n];
    out[e] = acc;
  }
}

// Block = (chunk, head, 16-token row tile).  Pass 1 fills
// gm[li][s] = (C_l . B_s) exp(acum_l - acum_s) dt_s for s <= l (0 otherwise);
// pass 2 forms y for the tile's tokens.
__global__ __launch_bounds__(kF32Threads) void k_chunk_scan_f32(
    const float *__restrict__ x, const float *__restrict__ Bm, const float *__restrict__ Cm,
    const float *__restrict__ Dv, const float *__restrict__ acum, const float *__restrict__ dtq,
    const float *__restrict__ hprev, ChunkGeom geom, int H, int G, int P, int N,
    float *__restrict__ y) {
  extern __shared__ float smem[];
  const int Q = geom.Q;
  float *sa = smem;               // [Q]
  float *sd = smem + Q;           // [Q]
  float *gm = smem + 2 * Q;       // [kRowTile][Q]
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int g = h / (H / G);
  const ChunkInfo ci = chunk_info(geom, c);
  const int lt = blockIdx.z * kRowTile;
  if (lt >= ci.len) return;
  const int64_t ch = (int64_t)c * H + h;
  for (int l = threadIdx.x; l < Q; l += kF32Threads) {
    sa[l] = acum[ch * Q + l];
    sd[l] = dtq[ch * Q + l];
  }
  __syncthreads();
  const int64_t ldx = (int64_t)H * P;
  const int64_t ldb = (int64_t)G * N;
  const float *xb = x + ci.t0 * ldx + (int64_t)h * P;
  const float *bb = Bm + ci.t0 * ldb + (int64_t)g * N;
  const float *cb = Cm + ci.t0 * ldb + (int64_t)g * N;
  const float *hp = hprev + ch * (int64_t)P * N;
  float *yb = y + ci.t0 * ldx + (int64_t)h * P;
  const float Dh = Dv ? Dv[h] : 0.f;
  {
    const int rows = min(kRowTile, ci.len - lt);
    const int span = lt + rows;  // sources s < span can be reached
    for (int idx = threadIdx.x; idx < rows * span; idx += kF32Threads) {
      const int li = idx / span;
      const int s = idx - li * span;
      const int l = lt + li;
      float v = 0.f;
      if (s <= l) {
        float dot = 0.f;
        for (int n = 0; n < N; ++n) dot += cb[l * ldb + n] * bb[s * ldb + n];
        v = dot * __expf(sa[l] - sa[s]) * sd[s];
      }
      gm[li * Q + s] = v;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < rows * P; idx += kF32Threads) {
      const int li = idx / P;
      const int p = idx - li * P;
      const int l = lt + li;
      float intra = 0.f;
      for (int s = 0; s <= l; ++s) intra += gm[li * Q + s] * xb[s * ldx + p];
      float inter = 0.f;
      for (int n = 0; n < N; ++n) inter += cb[l * ldb + n] * hp[p * N + n];
      const float xl = xb[l * ldx + p];
      yb[l * ldx + p] = intra + __expf(sa[l]) * inter + Dh * xl;
    }
  }
}

}  // namespace

hipError_t launch_chunk_state_f32(const float *x, const float *B, const float *acum,
                                  const float *dtq, float *states, const Geometry &geo,
                                  hipStream_t stream) {
  if (geo.nc_max == 0) return hipSuccess;
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  hipLaunchKernelGGL(k_chunk_state_f32, dim3((unsigned)geo.nc_max, (unsigned)geo.H),
                     dim3(kF32Threads), geo.Q * sizeof(float), stream, x, B, acum, dtq, cg,
                     geo.H, geo.G, geo.P, geo.N, states);
  return hipGetLastError();
}

hipError_t launch_chunk_scan_f32(const float *x, const float *B, const float *C, const float *D,
                                 const float *acum, const float *dtq, const float *hprev, float *y,
                                 const Geometry &geo, hipStream_t stream) {
  if (geo.nc_max == 0) return hipSuccess;
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  const size_t smem = (size_t)(2 + kRowTile) * geo.Q * sizeof(float);
  hipLaunchKernelGGL(k_chunk_scan_f32,
                     dim3((unsigned)geo.nc_max, (unsigned)geo.H,
                          (unsigned)((geo.Q + kRowTile - 1) / kRowTile)),
                     dim3(kF32Threads), smem, stream, x, B, C, D, acum, dtq, hprev, cg, geo.H,
                     geo.G, geo.P, geo.N, y);
  return hipGetLastError();
}

}  // namespace ssd
