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

// 4 consecutive elements of an io tensor as floats (one 16-byte fp32 or
// 8-byte bf16 load; the offsets used here are multiples of 4 elements of rows
// whose lengths are multiples of 16), and the matching store
__device__ __forceinline__ void ld4(const float *p, float (&v)[4]) {
  const f32x4 q = *reinterpret_cast<const f32x4 *>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void ld4(const uint16_t *p, float (&v)[4]) {
  const u32x2 q = *reinterpret_cast<const u32x2 *>(p);
  v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
}
__device__ __forceinline__ void st4(float *p, const float (&v)[4]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ void st4(uint16_t *p, const float (&v)[4]) {
  *reinterpret_cast<u32x2 *>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ float dot4(const float (&a)[4], const float (&b)[4]) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// R_c = sum_l e^{a_l} dy_l C_l^T per (chunk, head): block = (chunk, head);
// each thread forms 4 x 4 tiles (p, n) of the P x N product over the chunk's
// tokens from 4-element loads of dy and C.
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
  const int N4 = N / 4, ntile = (P / 4) * N4;
  for (int tile = threadIdx.x; tile < ntile; tile += kVT) {
    const int p0 = 4 * (tile / N4), n0 = 4 * (tile % N4);
    float acc[4][4] = {};
    for (int l = 0; l < ci.len; ++l) {
      float a[4], b[4];
      ld4(yb + l * ldx + p0, a);
      ld4(cb + l * ldb + n0, b);
      const float w = sw[l];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = a[i] * w;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[i][k] += ai * b[k];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) st4(out + (int64_t)(p0 + i) * N + n0, acc[i]);
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

// Per (chunk, group): Z once, then per head of the group E, dx, dB, dC and the
// per-token scalars; dB and dC summed over the heads (each of their elements
// is owned by one thread of the one block of its chunk and group: the first
// head writes it, the others add); dA and dD added atomically per head.  The
// products over p, n and the chunk's tokens are formed in 4 x 4 register
// tiles from 4-element loads (the chunk's rows of x, dy, B and C, and the
// head's P x N tiles of the state and its gradient, are re-read from the
// caches); the triangular 64 x 64 matrices live in LDS.
template <typename IO>
__global__ __launch_bounds__(kVT) void k_bwd_chunk_vec(
    const IO *__restrict__ x, const float *__restrict__ A, const IO *__restrict__ Bm,
    const IO *__restrict__ Cm, const float *__restrict__ Dv, const IO *__restrict__ dy,
    const float *__restrict__ acum, const float *__restrict__ dtq, const IO *__restrict__ hprev,
    const float *__restrict__ GE, ChunkGeom geom, int H, int G, int P, int N,
    IO *__restrict__ dx, float *__restrict__ ddt, float *__restrict__ dA, float *__restrict__ dB,
    float *__restrict__ dC, float *__restrict__ dD) {
  __shared__ float Zs[kVQ][kVQ + 1];  // C_l . B_s on s <= l (0 elsewhere)
  __shared__ float Es[kVQ][kVQ + 1];  // (dy_l . x_s) e^{a_l - a_s} on s <= l (0 elsewhere)
  __shared__ float Ms[kVQ][kVQ + 1];  // (C_l . B_s) e^{a_l - a_s}; later prefix sums of K
  __shared__ float sa[kVQ], sd[kVQ], sw[kVQ], sq[kVQ], sv[kVQ];
  __shared__ float red[3];  // <ge, h_s>, dA, dD of the head
  // 16-row (or 16-column) slices of the operands of the (t, n) and (t, p)
  // products, 16-byte aligned rows read as 4-element vectors
  __shared__ __align__(16) float Sx[16][kVQ], Sy[16][kVQ], Sg[16][kVQ], Sh[16][kVQ];
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

  // the 4 x 4 tile (l0.., s0..) of the 64 x 64 token matrices this thread forms
  const int l0 = 4 * (tid >> 4), s0 = 4 * (tid & 15);
  const bool tri = s0 <= l0 + 3 && l0 < len;  // the tile meets the chunk's lower triangle
  auto row = [&](int t) { return min(t, len - 1); };  // rows past the end read the last one

  {  // Z = C B^T
    float acc[4][4] = {};
    if (tri) {
      for (int n = 0; n < N; n += 4) {
        float a[4][4], b[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ld4(cb + row(l0 + i) * ldb + n, a[i]);
          ld4(bb + row(s0 + i) * ldb + n, b[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) acc[i][k] += dot4(a[i], b[k]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int l = l0 + i, s = s0 + k;
        Zs[l][s] = s <= l && l < len ? acc[i][k] : 0.f;
      }
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
    __syncthreads();  // the previous head is done with the tables, Es and Ms
    if (tid < kVQ) {
      sa[tid] = acum[ch * kVQ + tid];  // past the chunk's end: its last value
      sd[tid] = tid < len ? dtq[ch * kVQ + tid] : 0.f;
      sq[tid] = 0.f;
      sv[tid] = 0.f;
    }
    if (tid < 3) red[tid] = 0.f;
    __syncthreads();
    const float alast = sa[kVQ - 1];
    if (tid < kVQ) sw[tid] = __expf(alast - sa[tid]);
    {  // E = dy x^T, with the decay L_ls = e^{a_l - a_s} folded in; M = Z o L
      float acc[4][4] = {};
      if (tri) {
        for (int p = 0; p < P; p += 4) {
          float a[4][4], b[4][4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ld4(yb + row(l0 + i) * ldx + p, a[i]);
            ld4(xb + row(s0 + i) * ldx + p, b[i]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[i][k] += dot4(a[i], b[k]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int l = l0 + i, s = s0 + k;
          const float dec = s <= l && l < len ? __expf(sa[l] - sa[s]) : 0.f;
          Es[l][s] = acc[i][k] * dec;
          Ms[l][s] = Zs[l][s] * dec;
        }
    }
    {  // <ge, h_s>
      float part = 0.f;
      for (int64_t e = 4 * (int64_t)tid; e < PN; e += 4 * kVT) {
        float a[4], b[4];
        ld4(ge + e, a);
        ld4(hs + e, b);
        part += dot4(a, b);
      }
      atomicAdd(&red[0], part);
    }
    __syncthreads();
    // (t, n) tiles, 64 columns n at a time: xge = x ge, dyh = dy h_s over p,
    // from 16-row slices of x, dy (transposed), ge and h_s staged in LDS (each
    // read from the caches once per column block instead of once per token
    // tile); sB = (E o L)^T C over l >= t; sC = (E o L) (dt B) over s <= t;
    // then this head's dB, dC and the per-token q_t = sum_n xge B_t,
    // v_t = sum_n dyh C_t.  Thread = (token tile ti, column tile ci) of the block.
    const int ti = tid >> 4, ci4 = 4 * (tid & 15);
    for (int nb = 0; nb < N; nb += 64) {
      const int ncols = min(64, N - nb);  // a multiple of 16
      const int t0 = 4 * ti, n0 = nb + ci4;
      const bool act = ci4 < ncols;
      float xg[4][4] = {}, dh[4][4] = {};
      for (int p0 = 0; p0 < P; p0 += 16) {
        __syncthreads();  // the previous slice (or phase) is done with the buffer
        {  // x, dy rows t, columns p0 .. p0+15 -> [k][t]; ge, h_s rows p0 .. p0+15
          const int t = tid >> 2, k4 = 4 * (tid & 3);
          float xa[4], ya[4];
          ld4(xb + row(t) * ldx + p0 + k4, xa);
          ld4(yb + row(t) * ldx + p0 + k4, ya);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            Sx[k4 + m][t] = xa[m];
            Sy[k4 + m][t] = ya[m];
          }
          const int k = tid >> 4, c4 = 4 * (tid & 15);
          float gv[4] = {}, hv[4] = {};
          if (c4 < ncols) {
            ld4(ge + (int64_t)(p0 + k) * N + nb + c4, gv);
            ld4(hs + (int64_t)(p0 + k) * N + nb + c4, hv);
          }
          st4(&Sg[k][c4], gv);
          st4(&Sh[k][c4], hv);
        }
        __syncthreads();
        if (act) {
#pragma unroll 4
          for (int k = 0; k < 16; ++k) {
            float xa[4], ya[4], gv[4], hv[4];
            ld4(&Sx[k][t0], xa);
            ld4(&Sy[k][t0], ya);
            ld4(&Sg[k][ci4], gv);
            ld4(&Sh[k][ci4], hv);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                xg[i][m] += xa[i] * gv[m];
                dh[i][m] += ya[i] * hv[m];
              }
          }
        }
      }
      if (!act || t0 >= len) continue;
      float sB[4][4] = {}, sC[4][4] = {};
      for (int l = t0; l < len; ++l) {
        float cv[4];
        ld4(cb + l * ldb + n0, cv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = Es[l][t0 + i];
#pragma unroll
          for (int m = 0; m < 4; ++m) sB[i][m] += e * cv[m];
        }
      }
      const int se = min(t0 + 4, len);
      for (int s = 0; s < se; ++s) {
        float bv[4];
        ld4(bb + s * ldb + n0, bv);
        const float ds = sd[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = Es[t0 + i][s] * ds;
#pragma unroll
          for (int m = 0; m < 4; ++m) sC[i][m] += e * bv[m];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        if (t >= len) break;
        const float ea = __expf(sa[t]);
        float vb[4], vc[4], bt[4], ct[4];
        ld4(bb + t * ldb + n0, bt);
        ld4(cb + t * ldb + n0, ct);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          vb[m] = sd[t] * (sB[i][m] + sw[t] * xg[i][m]);
          vc[m] = ea * dh[i][m] + sC[i][m];
        }
        float *ob = dBc + (int64_t)t * ldb + n0, *oc = dCc + (int64_t)t * ldb + n0;
        if (j) {
          float pb[4], pc[4];
          ld4(ob, pb);
          ld4(oc, pc);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            vb[m] += pb[m];
            vc[m] += pc[m];
          }
        }
        st4(ob, vb);
        st4(oc, vc);
        atomicAdd(&sq[t], dot4(xg[i], bt));
        atomicAdd(&sv[t], dot4(dh[i], ct));
      }
    }
    // (t, p) tiles, 64 rows p at a time: dx = D dy + dt (sz + e^{a_last - a_t} gb)
    // with sz = (Z o L)^T dy over l >= t and gb = B ge^T over n, the latter from
    // 16-column slices of B and ge staged (transposed) in LDS
    for (int pb = 0; pb < P; pb += 64) {
      const int prows = min(64, P - pb);  // a multiple of 16
      const int t0 = 4 * ti, p0 = pb + ci4;
      const bool act = ci4 < prows;
      float gb[4][4] = {};
      for (int n0 = 0; n0 < N; n0 += 16) {
        __syncthreads();
        {  // B rows t and ge rows pb + r, columns n0 .. n0+15 -> [k][t], [k][r]
          const int r = tid >> 2, k4 = 4 * (tid & 3);
          float bv[4], gv[4] = {};
          ld4(bb + row(r) * ldb + n0 + k4, bv);
          if (r < prows) ld4(ge + (int64_t)(pb + r) * N + n0 + k4, gv);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            Sx[k4 + m][r] = bv[m];
            Sg[k4 + m][r] = gv[m];
          }
        }
        __syncthreads();
        if (act) {
#pragma unroll 4
          for (int k = 0; k < 16; ++k) {
            float bv[4], gv[4];
            ld4(&Sx[k][t0], bv);
            ld4(&Sg[k][ci4], gv);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int m = 0; m < 4; ++m) gb[i][m] += bv[i] * gv[m];
          }
        }
      }
      if (!act || t0 >= len) continue;
      float sz[4][4] = {};
      for (int l = t0; l < len; ++l) {
        float yv[4];
        ld4(yb + l * ldx + p0, yv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float m = Ms[l][t0 + i];
#pragma unroll
          for (int k = 0; k < 4; ++k) sz[i][k] += m * yv[k];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        if (t >= len) break;
        float yv[4], o[4];
        ld4(yb + t * ldx + p0, yv);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = Dh * yv[k] + sd[t] * (sz[i][k] + sw[t] * gb[i][k]);
        st4(dx + (ci.t0 + t) * ldx + (int64_t)h * P + p0, o);
      }
    }
    __syncthreads();  // sq, sv complete; Ms is free
    // R_t = sum over l >= t > s of K_ls, K_ls = (E o L)_ls dt_s Z_ls: each row's
    // exclusive prefix sums over s (Ms[l][t] = sum_{s<t} K_ls for t <= l) ...
    if (tid < len) {
      const int l = tid;
      float run = 0.f;
      for (int t = 0; t <= l; ++t) {
        const float k = Es[l][t] * sd[t] * Zs[l][t];
        Ms[l][t] = run;
        run += k;
      }
    }
    __syncthreads();
    // ... then per token t the sums down column t, and ddt, dA, dD
    if (tid < len) {
      const int t = tid;
      float term1 = 0.f, Rt = 0.f, Vt = 0.f, Ut = __expf(alast) * red[0];
      for (int l = t; l < len; ++l) {
        term1 += Es[l][t] * Zs[l][t];
        Rt += Ms[l][t];
        Vt += __expf(sa[l]) * sv[l];
      }
      for (int s = 0; s < t; ++s) Ut += sw[s] * sd[s] * sq[s];
      const float w = Rt + Vt + Ut;
      ddt[(ci.t0 + t) * (int64_t)H + h] = term1 + sw[t] * sq[t] + Ah * w;
      atomicAdd(&red[1], sd[t] * w);
      atomicAdd(&red[2], Es[t][t]);
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
