// libssd: the SSD core's neighbours in the Mamba-2 block (page "Mamba-2
// Architecture: State Space Duality Explained", "Step 2: Full Mamba-2 Block
// with Gated Projections"):
//   * before the core, a causal depthwise convolution of width K over the
//     token axis of each channel (bias, left padding K-1, outputs truncated to
//     the sequence) followed by SiLU;
//   * after it, the output gated by SiLU(z) and RMS-normalised over the whole
//     channel width with a learned weight.
// Both are elementwise along channels and HBM-bound: each reads its inputs and
// writes its output once.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

// VEC channels per 16-byte access: 8 bf16 or 4 fp32
template <typename IO> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const u32x4 &q, float (&v)[8]) {
    v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
    v[4] = bf16lo(q.z); v[5] = bf16hi(q.z); v[6] = bf16lo(q.w); v[7] = bf16hi(q.w);
  }
  __device__ static void load(const uint16_t *p, float (&v)[8]) {
    unpack(*reinterpret_cast<const u32x4 *>(p), v);
  }
  __device__ static void store(uint16_t *p, const float (&v)[8]) {
    *reinterpret_cast<u32x4 *>(p) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
  // a streaming (non-temporal) store: output nothing in this kernel reads again
  __device__ static void store_nt(uint16_t *p, const float (&v)[8]) {
    __builtin_nontemporal_store(u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                      pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])},
                                reinterpret_cast<u32x4 *>(p));
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const u32x4 &q, float (&v)[4]) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
  __device__ static void load(const float *p, float (&v)[4]) {
    const f32x4 q = *reinterpret_cast<const f32x4 *>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static void store(float *p, const float (&v)[4]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
  __device__ static void store_nt(float *p, const float (&v)[4]) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
  }
};

// SiLU with the hardware reciprocal (about 1 ulp) in place of an IEEE
// division: the correctly rounded divide is a dozen vector instructions per
// element and made the convolution VALU-bound (195 -> 154 us at 32,768 tokens
// x 5376 channels); the result is rounded to bf16 or kept to ~1e-7 in fp32
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

constexpr int kConvRun = 16;  // tokens per thread

// Thread = (channel group of VEC, run of kConvRun tokens), channel groups
// fastest so a wavefront reads contiguous row segments.  A run inside one
// sequence loads its kConvRun + K - 1 input rows up front (16 bytes each, all
// in flight together; rows before the sequence start read as 0) and then
// forms its outputs, written with streaming stores.  A run that crosses a sequence boundary walks its tokens
// in order instead, keeping the K-1 previous inputs in registers and
// resetting them to 0 at each sequence start.
template <typename IO, int K>
__global__ __launch_bounds__(256) void k_conv1d_silu(const IO *__restrict__ in, int64_t in_stride,
                                                     const float *__restrict__ weight,
                                                     const float *__restrict__ bias,
                                                     IO *__restrict__ out, int64_t out_stride,
                                                     int64_t T, int64_t seqlen, int nseq,
                                                     const int32_t *__restrict__ cu, int groups) {
  constexpr int V = Vec<IO>::N;
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t runs = (T + kConvRun - 1) / kConvRun;
  if (gid >= runs * groups) return;
  const int grp = static_cast<int>(gid % groups);
  const int64_t t0 = (gid / groups) * kConvRun;
  const int64_t t1 = min(T, t0 + kConvRun);
  const int c0 = grp * V;

  float w[V][K], b[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) w[v][k] = weight[(int64_t)(c0 + v) * K + k];
    b[v] = bias ? bias[c0 + v] : 0.f;
  }
  // the sequence holding t0: [s_begin, s_end)
  int64_t s_begin, s_end;
  int s = 0;
  if (cu) {
    int lo = 0, hi = nseq - 1;  // largest s with cu[s] <= t0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t0) lo = mid; else hi = mid - 1;
    }
    s = lo;
    s_begin = cu[s];
    s_end = cu[s + 1];
    while (s_end <= t0 && s + 1 < nseq) {  // skip empty sequences
      ++s;
      s_begin = cu[s];
      s_end = cu[s + 1];
    }
    s_begin = s_begin < 0 ? 0 : s_begin;  // any cu_seqlens: reads stay inside [0, T)
  } else {
    s_begin = (t0 / seqlen) * seqlen;
    s_end = s_begin + seqlen;
  }
  if (t1 <= s_end) {
    constexpr int NR = kConvRun + K - 1;
    u32x4 raw[NR];  // raw[i] = the input row t0 - (K-1) + i
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int64_t src = t0 - (K - 1) + i;
      raw[i] = src >= s_begin && src < t1
                   ? *reinterpret_cast<const u32x4 *>(in + src * in_stride + c0)
                   : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kConvRun; ++i) {
      if (t0 + i < t1) {
        float acc[V], o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = b[v];
#pragma unroll
        for (int j = 0; j < K; ++j) {
          float r[V];
          Vec<IO>::unpack(raw[i + j], r);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[v] += w[v][j] * r[v];
        }
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = silu(acc[v]);
        Vec<IO>::store_nt(out + (t0 + i) * out_stride + c0, o);
      }
    }
    return;
  }
  float win[K > 1 ? K - 1 : 1][V];  // win[j] = input at t - (K-1) + j
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int64_t src = t0 - (K - 1) + j;
    if (src >= s_begin) {
      Vec<IO>::load(in + src * in_stride + c0, win[j]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) win[j][v] = 0.f;
    }
  }
  for (int64_t t = t0; t < t1; ++t) {
    if (t >= s_end) {  // a new sequence starts here: the window empties
      if (cu) {
        while (s + 1 < nseq && cu[s + 1] <= t) ++s;
        s_begin = cu[s] < 0 ? 0 : cu[s];
        s_end = cu[s + 1] > t ? cu[s + 1] : T;  // a malformed table never loops back
      } else {
        s_begin = t;
        s_end = t + seqlen;
      }
#pragma unroll
      for (int j = 0; j < K - 1; ++j)
#pragma unroll
        for (int v = 0; v < V; ++v) win[j][v] = 0.f;
    }
    float cur[V], o[V];
    Vec<IO>::load(in + t * in_stride + c0, cur);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float acc = b[v];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc += w[v][j] * win[j][v];
      acc += w[v][K - 1] * cur[v];
      o[v] = silu(acc);
    }
    Vec<IO>::store(out + t * out_stride + c0, o);
#pragma unroll
    for (int j = 0; j + 1 < K - 1; ++j)
#pragma unroll
      for (int v = 0; v < V; ++v) win[j][v] = win[j + 1][v];
    if (K > 1) {
#pragma unroll
      for (int v = 0; v < V; ++v) win[K > 1 ? K - 2 : 0][v] = cur[v];
    }
  }
}

// Block = ROWS consecutive token rows of `width` channels; thread t owns the
// 16-byte column chunks t, t + 256, ... (up to CACHE of them), whose weights it
// loads once.  The next row's y and z chunks are loaded while the current row
// is reduced and written.  Per row: g = y silu(z) in registers, squares
// summed over the row (DPP and permlane sums in the wavefront, then one LDS slot per wavefront,
// double-buffered so one barrier per row suffices), then
// g * rsqrt(mean + eps) * weight is written; without a weight, g.  Rows wider
// than 256 * CACHE chunks form g again for the chunks past the cache.
template <typename IO, int CACHE, int ROWS>
__global__ __launch_bounds__(256) void k_gate_rmsnorm(const IO *y, const IO *z,
                                                      const float *__restrict__ weight, float eps,
                                                      IO *out, int64_t tokens, int width) {
  constexpr int V = Vec<IO>::N;
  __shared__ float part[2][4];
  const int nvec = width / V;
  const int tid = threadIdx.x;
  float wv[CACHE][V];
#pragma unroll
  for (int k = 0; k < CACHE; ++k) {
    const int i = tid + 256 * k;
#pragma unroll
    for (int v = 0; v < V; ++v) wv[k][v] = (weight && i < nvec) ? weight[i * V + v] : 1.f;
  }
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  // raw 16-byte chunks of y and z of one row (zeros past the row's end)
  auto load_row = [&](int64_t row, u32x4 (&ya)[CACHE], u32x4 (&za)[CACHE]) {
#pragma unroll
    for (int k = 0; k < CACHE; ++k) {
      const int i = tid + 256 * k;
      const bool ok = row < tokens && i < nvec;
      ya[k] = ok ? *reinterpret_cast<const u32x4 *>(y + row * width + (int64_t)i * V) : u32x4{0u, 0u, 0u, 0u};
      za[k] = ok ? *reinterpret_cast<const u32x4 *>(z + row * width + (int64_t)i * V) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 yc[CACHE], zc[CACHE];
  load_row(r0, yc, zc);
  for (int rr = 0; rr < ROWS; ++rr) {
    const int64_t row = r0 + rr;
    if (row >= tokens) break;
    u32x4 yn[CACHE], zn[CACHE];
    if (rr + 1 < ROWS) load_row(row + 1, yn, zn);
    const IO *yr = y + row * width;
    const IO *zr = z + row * width;
    IO *orow = out + row * width;
    float g[CACHE][V];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CACHE; ++k) {
      const int i = tid + 256 * k;
      if (i < nvec) {
        float a[V], c[V];
        Vec<IO>::unpack(yc[k], a);
        Vec<IO>::unpack(zc[k], c);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          g[k][v] = a[v] * silu(c[v]);
          ss += g[k][v] * g[k][v];
        }
      }
    }
    for (int i = tid + 256 * CACHE; i < nvec; i += 256) {
      float a[V], c[V];
      Vec<IO>::load(yr + i * V, a);
      Vec<IO>::load(zr + i * V, c);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float gv = a[v] * silu(c[v]);
        ss += gv * gv;
      }
    }
    float scale = 1.f;
    if (weight) {
      ss = wave_sum(ss);
      if ((tid & 63) == 0) part[rr & 1][tid >> 6] = ss;
      __syncthreads();
      scale = rsqrtf((part[rr & 1][0] + part[rr & 1][1] + part[rr & 1][2] + part[rr & 1][3]) / width + eps);
    }
#pragma unroll
    for (int k = 0; k < CACHE; ++k) {
      const int i = tid + 256 * k;
      if (i < nvec) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = g[k][v] * scale * wv[k][v];
        Vec<IO>::store(orow + i * V, o);
      }
    }
    for (int i = tid + 256 * CACHE; i < nvec; i += 256) {
      float a[V], c[V], o[V];
      Vec<IO>::load(yr + i * V, a);
      Vec<IO>::load(zr + i * V, c);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const float gv = a[v] * silu(c[v]);
        o[v] = weight ? gv * scale * weight[i * V + v] : gv;
      }
      Vec<IO>::store(orow + i * V, o);
    }
    if (rr + 1 < ROWS) {
#pragma unroll
      for (int k = 0; k < CACHE; ++k) {
        yc[k] = yn[k];
        zc[k] = zn[k];
      }
    }
  }
}

template <typename IO>
hipError_t conv_t(const void *in, int64_t in_stride, const float *w, const float *b, int K,
                  void *out, int64_t out_stride, int64_t T, int64_t seqlen, int nseq,
                  const int32_t *cu, int64_t channels, hipStream_t stream) {
  const int groups = static_cast<int>(channels / Vec<IO>::N);
  const int64_t threads = ((T + kConvRun - 1) / kConvRun) * groups;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  const IO *i = static_cast<const IO *>(in);
  IO *o = static_cast<IO *>(out);
  switch (K) {
    case 1: hipLaunchKernelGGL((k_conv1d_silu<IO, 1>), grid, dim3(256), 0, stream, i, in_stride, w, b, o, out_stride, T, seqlen, nseq, cu, groups); break;
    case 2: hipLaunchKernelGGL((k_conv1d_silu<IO, 2>), grid, dim3(256), 0, stream, i, in_stride, w, b, o, out_stride, T, seqlen, nseq, cu, groups); break;
    case 3: hipLaunchKernelGGL((k_conv1d_silu<IO, 3>), grid, dim3(256), 0, stream, i, in_stride, w, b, o, out_stride, T, seqlen, nseq, cu, groups); break;
    case 4: hipLaunchKernelGGL((k_conv1d_silu<IO, 4>), grid, dim3(256), 0, stream, i, in_stride, w, b, o, out_stride, T, seqlen, nseq, cu, groups); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d_silu(const void *in, int64_t in_stride, const float *weight,
                              const float *bias, int K, void *out, int64_t out_stride, int64_t T,
                              int64_t seqlen, int nseq, const int32_t *cu_seqlens,
                              int64_t channels, bool bf16, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  return bf16 ? conv_t<uint16_t>(in, in_stride, weight, bias, K, out, out_stride, T, seqlen, nseq,
                                 cu_seqlens, channels, stream)
              : conv_t<float>(in, in_stride, weight, bias, K, out, out_stride, T, seqlen, nseq,
                              cu_seqlens, channels, stream);
}

hipError_t launch_gate_rmsnorm(const void *y, const void *z, const float *weight, float eps,
                               void *out, int64_t tokens, int width, bool bf16,
                               hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  constexpr int kRows = 16;
  const dim3 grid(static_cast<unsigned>((tokens + kRows - 1) / kRows));
  if (bf16)
    hipLaunchKernelGGL((k_gate_rmsnorm<uint16_t, 3, kRows>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(y), static_cast<const uint16_t *>(z), weight,
                       eps, static_cast<uint16_t *>(out), tokens, width);
  else
    hipLaunchKernelGGL((k_gate_rmsnorm<float, 5, kRows>), grid, dim3(256), 0, stream,
                       static_cast<const float *>(y), static_cast<const float *>(z), weight, eps,
                       static_cast<float *>(out), tokens, width);
  return hipGetLastError();
}

}  // namespace ssd
