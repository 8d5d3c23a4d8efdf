// libssd: the backward pass of the chunked forward on the fp32 vector ALU
// (gfx950), for every shape the forward takes (fp32 or bf16 io, head dims and
// state sizes multiples of 16 up to 256): the general path, where the MFMA
// backward (bf16, P = 64, N <= 128) does not apply.  Correct, not tuned.
//
// The pages state no backward pass; it is the chain rule through the
// recurrence (page "State Space Duality and Mamba-2: Unifying Transformers and
// Semiseparable Matrices", "Mathematical Foundations", with the scalar-identity
// transition of "The Scalar-Identity Structural Constraint"), evaluated
// blockwise like the forward (page "Mamba-2 Architecture: State Space Duality
// Explained", "2. The Chunked SSD Algorithm").  With a_l the cumulative sum of
// dt A from the chunk's start (inclusive), h_s the state entering the chunk
// and ge the gradient w.r.t. the state leaving it (what the later chunks pass
// back), per chunk and head, for tokens t, l, s of the chunk:
//   g_t   = sum_{l>=t} e^{a_l - a_t} dy_l C_l^T + e^{a_last - a_t} ge
//   h_t   = e^{a_t} h_s + sum_{s<=t} e^{a_t - a_s} dt_s x_s B_s^T
//   dx_t  = D dy_t + dt_t g_t B_t
//   dB_t  = dt_t g_t^T x_t,   dC_t = h_t^T dy_t      (summed over a group's heads)
//   ddt_t = x_t^T g_t B_t + A e^{dt_t A} <g_t, h_{t-1}>,
//   dA    = sum_t dt_t e^{dt_t A} <g_t, h_{t-1}>,   dD = sum_t <dy_t, x_t>
// and between chunks ge_{c-1} = e^{a_last} ge_c + sum_l e^{a_l} dy_l C_l^T,
// from d(final_state) at the sequence's end down to d(init_state).  With
// E_ls = dy_l . x_s and Z_ls = C_l . B_s, e^{dt_t A} <g_t, h_{t-1}> expands
// (the e^{+-a_t} factors cancel) into R_t + V_t + U_t:
//   R_t = sum_{l>=t>s} e^{a_l - a_s} dt_s E_ls Z_ls
//   V_t = sum_{l>=t} e^{a_l} dy_l^T h_s C_l
//   U_t = e^{a_last} <ge, h_s> + sum_{s<t} e^{a_last - a_s} dt_s x_s^T ge B_s
// Every exponent is <= 0 for A <= 0, so nothing overflows.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int kVT = 256;    // threads a block
constexpr int kVQ = 64;     // chunk length of this path
constexpr int kTB = 8;      // tokens a thread takes together (operands loaded once for them)

__device__ __forceinline__ float vld(const float *p) { return *p; }
__device__ __forceinline__ float vld(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ void vst(float *p, float v) { *p = v; }
__device__ __forceinline__ void vst(uint16_t *p, float v) {
  *p = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
}

// R_c = sum_l e^{a_l} dy_l C_l^T per (chunk, head): block = (chunk, head),
// thread = state elements (p, n).
template <typename IO>
__global__ __launch_bounds__(kVT) void k_bwd_rsum_vec(const IO *__restrict__ dy,
                                                     const IO *__restrict__ Cm,
                                                     const float *__restrict__ acum, ChunkGeom geom,
                                                     int H, int G, int P, int N,
                                                     float *__restrict__ R) {
  __shared__ float sw[kVQ];
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;
  const int64_t ch = (int64_t)c * H + h;
  if (threadIdx.x < kVQ)
    sw[threadIdx.x] = (int)threadIdx.x < ci.len ? __expf(acum[ch * kVQ + threadIdx.x]) : 0.f;
  __syncthreads();
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const IO *yb = dy + ci.t0 * ldx + (int64_t)h * P;
  const IO *cb = Cm + ci.t0 * ldb + (int64_t)(h / (H / G)) * N;
  float *out = R + ch * (int64_t)P * N;
  for (int e = threadIdx.x; e < P * N; e += kVT) {
    const int p = e / N, n = e - p * N;
    float acc = 0.f;
    for (int l = 0; l < ci.len; ++l) acc += vld(yb + l * ldx + p) * sw[l] * vld(cb + l * ldb + n);
    out[e] = acc;
  }
}

// ge entering each chunk from the right, per (sequence, head) and 4 state
// elements a thread, the sequence's chunks in reverse: GE[c] = ge;
// ge = e^{a_last(c)} ge + R[c]; then d(init_state) = ge.
__global__ __launch_bounds__(kVT) void k_bwd_pass_vec(const float *__restrict__ R,
                                                     float *__restrict__ GE,
                                                     const float *__restrict__ acum,
                                                     const float *__restrict__ dfinal,
                                                     float *__restrict__ dinit, int H, int PN,
                                                     int nc_row, const int32_t *__restrict__ dir) {
  const int e0 = (blockIdx.x * kVT + threadIdx.x) * 4;
  if (e0 >= PN) return;
  const int h = blockIdx.y, s = blockIdx.z;
  const int cb = dir ? dir[s] : s * nc_row;
  const int ce = dir ? dir[s + 1] : cb + nc_row;
  const int64_t soff = ((int64_t)s * H + h) * PN + e0;
  f32x4 ge = dfinal ? *reinterpret_cast<const f32x4 *>(dfinal + soff) : f32x4{};
  for (int c = ce - 1; c >= cb; --c) {
    const int64_t ch = (int64_t)c * H + h;
    *reinterpret_cast<f32x4 *>(GE + ch * PN + e0) = ge;
    ge = __expf(acum[ch * kVQ + kVQ - 1]) * ge + *reinterpret_cast<const f32x4 *>(R + ch * PN + e0);
  }
  if (dinit) *reinterpret_cast<f32x4 *>(dinit + soff) = ge;
}

// Per (chunk, group): Z once, then per head of the group E, the per-token
// scalars and dx, ddt; dB and dC summed over the heads (each of their elements
// is owned by one thread of the one block of its chunk and group: the first
// head writes it, the others add); dA and dD added atomically per head.
template <typename IO>
__global__ __launch_bounds__(kVT) void k_bwd_chunk_vec(
    const IO *__restrict__ x, const float *__restrict__ A, const IO *__restrict__ Bm,
    const IO *__restrict__ Cm, const float *__restrict__ Dv, const IO *__restrict__ dy,
    const float *__restrict__ acum, const float *__restrict__ dtq, const IO *__restrict__ hprev,
    const float *__restrict__ GE, ChunkGeom geom, int H, int G, int P, int N,
    IO *__restrict__ dx, float *__restrict__ ddt, float *__restrict__ dA, float *__restrict__ dB,
    float *__restrict__ dC, float *__restrict__ dD) {
  __shared__ float Z[kVQ][kVQ + 1];  // C_l . B_s (s <= l), the block's
  __shared__ float E[kVQ][kVQ + 1];  // dy_l . x_s, then (dy_l . x_s) e^{a_l - a_s}
  __shared__ float M[kVQ][kVQ + 1];  // (C_l . B_s) e^{a_l - a_s}
  __shared__ float sa[kVQ], sd[kVQ], sq[kVQ], sv[kVQ];
  __shared__ float red[3];  // <ge, h_s>, dA, dD of the head
  const int c = blockIdx.x, g = blockIdx.y;
  const ChunkInfo ci = chunk_info(geom, c);
  const int len = ci.len;
  if (len <= 0) return;
  const int tid = threadIdx.x;
  const int HG = H / G;
  const int64_t ldx = (int64_t)H * P, ldb = (int64_t)G * N;
  const IO *bb = Bm + ci.t0 * ldb + (int64_t)g * N;
  const IO *cb = Cm + ci.t0 * ldb + (int64_t)g * N;
  const int64_t PN = (int64_t)P * N;

  for (int i = tid; i < len * len; i += kVT) {
    const int l = i / len, s = i - l * len;
    float z = 0.f;
    if (s <= l)
      for (int n = 0; n < N; ++n) z += vld(cb + l * ldb + n) * vld(bb + s * ldb + n);
    Z[l][s] = z;
  }
  float *dBc = dB + ci.t0 * ldb + (int64_t)g * N;
  float *dCc = dC + ci.t0 * ldb + (int64_t)g * N;

  for (int j = 0; j < HG; ++j) {
    const int h = g * HG + j;
    const int64_t ch = (int64_t)c * H + h;
    const IO *xb = x + ci.t0 * ldx + (int64_t)h * P;
    const IO *yb = dy + ci.t0 * ldx + (int64_t)h * P;
    const IO *hs = hprev + ch * PN;
    const float *ge = GE + ch * PN;
    const float Ah = A[h];
    const float Dh = Dv ? Dv[h] : 0.f;
    __syncthreads();  // the previous head is done with the tables, E and M
    if (tid < kVQ) {
      sa[tid] = acum[ch * kVQ + tid];
      sd[tid] = tid < len ? dtq[ch * kVQ + tid] : 0.f;
      sq[tid] = 0.f;
      sv[tid] = 0.f;
    }
    if (tid < 3) red[tid] = 0.f;
    for (int i = tid; i < len * len; i += kVT) {
      const int l = i / len, s = i - l * len;
      float e = 0.f;
      if (s <= l)
        for (int p = 0; p < P; ++p) e += vld(yb + l * ldx + p) * vld(xb + s * ldx + p);
      E[l][s] = e;
    }
    __syncthreads();
    const float alast = sa[kVQ - 1];
    // the decay L_ls = e^{a_l - a_s} (s <= l) folded in: E <- E o L, M = Z o L
    for (int i = tid; i < len * len; i += kVT) {
      const int l = i / len, s = i - l * len;
      const float dec = s <= l ? __expf(sa[l] - sa[s]) : 0.f;
      E[l][s] *= dec;
      M[l][s] = Z[l][s] * dec;
    }
    // <ge, h_s>
    {
      float part = 0.f;
      for (int64_t e = tid; e < PN; e += kVT) part += ge[e] * vld(hs + e);
      atomicAdd(&red[0], part);
    }
    __syncthreads();
    // (token block of kTB, n): dB and dC of this head, q_t and v_t partial sums;
    // every operand loaded once per block of tokens
    const int ntb = (len + kTB - 1) / kTB;
    for (int i = tid; i < ntb * N; i += kVT) {
      const int t0 = (i / N) * kTB, n = i % N;
      float xge[kTB], dyh[kTB], sB[kTB], sC[kTB];
#pragma unroll
      for (int k = 0; k < kTB; ++k) xge[k] = dyh[k] = sB[k] = sC[k] = 0.f;
      for (int p = 0; p < P; ++p) {
        const float gv = ge[(int64_t)p * N + n], hv = vld(hs + (int64_t)p * N + n);
#pragma unroll
        for (int k = 0; k < kTB; ++k) {
          const int t = min(t0 + k, len - 1);
          xge[k] += vld(xb + t * ldx + p) * gv;
          dyh[k] += vld(yb + t * ldx + p) * hv;
        }
      }
      for (int l = t0; l < len; ++l) {  // sum over l >= t of (E o L)_lt C_l
        const float cv = vld(cb + l * ldb + n);
#pragma unroll
        for (int k = 0; k < kTB; ++k)
          if (t0 + k <= l) sB[k] += E[l][t0 + k] * cv;
      }
      for (int s = 0; s < min(t0 + kTB, len); ++s) {  // sum over s <= t of (E o L)_ts dt_s B_s
        const float bv = sd[s] * vld(bb + s * ldb + n);
#pragma unroll
        for (int k = 0; k < kTB; ++k)
          if (s <= t0 + k && t0 + k < len) sC[k] += E[t0 + k][s] * bv;
      }
#pragma unroll
      for (int k = 0; k < kTB; ++k) {
        const int t = t0 + k;
        if (t >= len) break;
        const float at = sa[t];
        const float vb = sd[t] * (sB[k] + __expf(alast - at) * xge[k]);
        const float vc = __expf(at) * dyh[k] + sC[k];
        const int64_t o = (int64_t)t * ldb + n;
        dBc[o] = j ? dBc[o] + vb : vb;
        dCc[o] = j ? dCc[o] + vc : vc;
        atomicAdd(&sq[t], xge[k] * vld(bb + t * ldb + n));
        atomicAdd(&sv[t], dyh[k] * vld(cb + t * ldb + n));
      }
    }
    // (token block of kTB, p): dx
    for (int i = tid; i < ntb * P; i += kVT) {
      const int t0 = (i / P) * kTB, p = i % P;
      float sz[kTB], gb[kTB];
#pragma unroll
      for (int k = 0; k < kTB; ++k) sz[k] = gb[k] = 0.f;
      for (int l = t0; l < len; ++l) {  // sum over l >= t of (Z o L)_lt dy_l
        const float yv = vld(yb + l * ldx + p);
#pragma unroll
        for (int k = 0; k < kTB; ++k)
          if (t0 + k <= l) sz[k] += M[l][t0 + k] * yv;
      }
      for (int n = 0; n < N; ++n) {
        const float gv = ge[(int64_t)p * N + n];
#pragma unroll
        for (int k = 0; k < kTB; ++k) gb[k] += gv * vld(bb + min(t0 + k, len - 1) * ldb + n);
      }
#pragma unroll
      for (int k = 0; k < kTB; ++k) {
        const int t = t0 + k;
        if (t >= len) break;
        vst(dx + (ci.t0 + t) * ldx + (int64_t)h * P + p,
            Dh * vld(yb + t * ldx + p) + sd[t] * (sz[k] + __expf(alast - sa[t]) * gb[k]));
      }
    }
    __syncthreads();
    // per token: ddt, and this head's dA and dD (E holds E o L, whose
    // diagonal is E's)
    if (tid < len) {
      const int t = tid;
      const float at = sa[t];
      float term1 = 0.f, Rt = 0.f, Vt = 0.f, Ut = __expf(alast) * red[0];
      for (int l = t; l < len; ++l) {
        term1 += E[l][t] * Z[l][t];
        Vt += __expf(sa[l]) * sv[l];
        for (int s = 0; s < t; ++s) Rt += E[l][s] * sd[s] * Z[l][s];
      }
      for (int s = 0; s < t; ++s) Ut += __expf(alast - sa[s]) * sd[s] * sq[s];
      const float w = Rt + Vt + Ut;
      ddt[(ci.t0 + t) * (int64_t)H + h] = term1 + __expf(alast - at) * sq[t] + Ah * w;
      atomicAdd(&red[1], sd[t] * w);
      atomicAdd(&red[2], E[t][t]);
    }
    __syncthreads();
    if (tid == 0) {
      atomicAdd(dA + h, red[1]);
      if (dD) atomicAdd(dD + h, red[2]);
    }
  }
}

template <typename IO>
hipError_t bwd_vec(const void *x, const float *A, const void *B, const void *C, const float *D,
                   const void *dy, const float *dfinal, const float *acum, const float *dtq,
                   const void *hprev, float *R, float *GE, const Geometry &geo, void *dx,
                   float *ddt, float *dA, float *dB, float *dC, float *dD, float *dinit,
                   hipStream_t stream) {
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  const IO *xi = static_cast<const IO *>(x), *bi = static_cast<const IO *>(B),
           *ci = static_cast<const IO *>(C), *yi = static_cast<const IO *>(dy);
  hipError_t e;
  if (geo.nc_max > 0) {
    hipLaunchKernelGGL(k_bwd_rsum_vec<IO>, dim3((unsigned)geo.nc_max, (unsigned)geo.H), dim3(kVT),
                       0, stream, yi, ci, acum, cg, geo.H, geo.G, geo.P, geo.N, R);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // (every sequence, also an empty one: d(init_state) = d(final_state) there)
  const int PN = geo.P * geo.N;
  hipLaunchKernelGGL(k_bwd_pass_vec, dim3((unsigned)((PN / 4 + kVT - 1) / kVT), (unsigned)geo.H,
                                          (unsigned)geo.nrows),
                     dim3(kVT), 0, stream, R, GE, acum, dfinal, dinit, geo.H, PN, geo.nc_row,
                     geo.packed ? geo.dir : nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (geo.nc_max == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_chunk_vec<IO>, dim3((unsigned)geo.nc_max, (unsigned)geo.G), dim3(kVT),
                     0, stream, xi, A, bi, ci, D, yi, acum, dtq, static_cast<const IO *>(hprev),
                     GE, cg, geo.H, geo.G, geo.P, geo.N, static_cast<IO *>(dx), ddt, dA, dB, dC,
                     dD);
  return hipGetLastError();
}

}  // namespace

int bwd_vec_chunk_len() { return kVQ; }

hipError_t launch_bwd_vec(const void *x, const float *A, const void *B, const void *C,
                          const float *D, const void *dy, const float *dfinal, const float *acum,
                          const float *dtq, const void *hprev, float *R, float *GE, bool bf16,
                          const Geometry &geo, void *dx, float *ddt, float *dA, float *dB,
                          float *dC, float *dD, float *dinit, hipStream_t stream) {
  if (geo.Q != kVQ || geo.N > 256 || geo.P > 256) return hipErrorInvalidValue;
  // a packed batch walks its chunks through the table and directory
  if (geo.packed && (!geo.table || !geo.dir)) return hipErrorInvalidValue;
  return bf16 ? bwd_vec<uint16_t>(x, A, B, C, D, dy, dfinal, acum, dtq, hprev, R, GE, geo, dx, ddt,
                                  dA, dB, dC, dD, dinit, stream)
              : bwd_vec<float>(x, A, B, C, D, dy, dfinal, acum, dtq, hprev, R, GE, geo, dx, ddt,
                               dA, dB, dC, dD, dinit, stream);
}

}  // namespace ssd
