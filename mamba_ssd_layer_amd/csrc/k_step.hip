// libssd: ssd_step, one recurrent step per sequence (decoding).
//
//   state <- exp(dt A) state + dt x B^T        y = C state + D x
//
// the scalar-identity recurrence for a single token (page "State Space
// Duality and Mamba-2: Unifying Transformers and Semiseparable Matrices",
// section "The Dual Perspectives of Semiseparable Multiplication", item 1:
// the recurrent mode, constant state per head).
//
// Design.  The step is bound by one read and one write of the fp32 state
// (2 * P * N * 4 bytes per head); everything else is a few hundred bytes.
// Block = (sequence, head), 256 threads.  A state row p (N floats) belongs to
// N/4 consecutive threads, 4 elements each -- one 16-byte load and one store
// per thread and row, so every wavefront moves whole contiguous rows.  The
// block walks its P rows in passes of 1024/N rows; B, C, the decay and dt x_p
// are per-row scalars or per-thread registers.  y_p = C . state_p is reduced
// across the row's threads with cross-lane shuffles; the row's first thread
// adds D x_p and writes y_p.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const uint16_t *p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ void ld4(const float *p, float (&v)[4]) {
  const f32x4 q = *reinterpret_cast<const f32x4 *>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ __forceinline__ void ld4(const uint16_t *p, float (&v)[4]) {
  const u32x2 q = *reinterpret_cast<const u32x2 *>(p);
  v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
}
__device__ __forceinline__ void st1(float *p, float v) { *p = v; }
__device__ __forceinline__ void st1(uint16_t *p, float v) {
  *p = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);  // round to nearest even
}

template <typename IO, int N>
__global__ __launch_bounds__(256) void k_step(const IO *__restrict__ x, const float *__restrict__ dt,
                                              const float *__restrict__ A, const IO *__restrict__ Bm,
                                              const IO *__restrict__ Cm, const float *__restrict__ Dv,
                                              float *__restrict__ state, IO *__restrict__ y, int H,
                                              int P, int G) {
  constexpr int TPR = N / 4;      // threads per state row
  constexpr int RPP = 256 / TPR;  // rows per pass
  static_assert(TPR >= 1 && TPR <= 64 && (64 % TPR) == 0, "a row stays inside one wavefront");
  const int64_t sh = blockIdx.x;  // sequence * H + head
  const int h = static_cast<int>(sh % H);
  const int64_t s = sh / H;
  const int g = h / (H / G);
  const int n4 = threadIdx.x % TPR;
  const int r0 = threadIdx.x / TPR;

  const float dtv = dt[sh];
  const float decay = __expf(dtv * A[h]);
  const float Dh = Dv ? Dv[h] : 0.f;
  float bv[4], cv[4];
  ld4(Bm + (s * G + g) * N + 4 * n4, bv);
  ld4(Cm + (s * G + g) * N + 4 * n4, cv);
  float *st = state + sh * P * N + 4 * n4;
  const IO *xr = x + sh * P;
  IO *yr = y + sh * P;

#pragma unroll 4
  for (int p0 = 0; p0 < P; p0 += RPP) {
    const int p = p0 + r0;
    const bool valid = p < P;
    float part = 0.f, xp = 0.f;
    if (valid) {
      xp = ld1(xr + p);
      const float u = dtv * xp;
      f32x4 hv = *reinterpret_cast<const f32x4 *>(st + (int64_t)p * N);
      hv.x = decay * hv.x + u * bv[0];
      hv.y = decay * hv.y + u * bv[1];
      hv.z = decay * hv.z + u * bv[2];
      hv.w = decay * hv.w + u * bv[3];
      *reinterpret_cast<f32x4 *>(st + (int64_t)p * N) = hv;
      part = cv[0] * hv.x + cv[1] * hv.y + cv[2] * hv.z + cv[3] * hv.w;
    }
    // every lane takes part in the lane exchanges; a row's TPR lanes share `valid`
    part = group_sum<TPR>(part);
    if (valid && n4 == 0) st1(yr + p, part + Dh * xp);
  }
}

template <typename IO>
hipError_t launch_step_t(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, float *state, void *y, int64_t S, int H,
                         int P, int N, int G, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(S * H));
  const IO *xi = static_cast<const IO *>(x);
  const IO *bi = static_cast<const IO *>(B);
  const IO *ci = static_cast<const IO *>(C);
  IO *yo = static_cast<IO *>(y);
  switch (N) {
    case 16: hipLaunchKernelGGL((k_step<IO, 16>), grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, state, yo, H, P, G); break;
    case 32: hipLaunchKernelGGL((k_step<IO, 32>), grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, state, yo, H, P, G); break;
    case 64: hipLaunchKernelGGL((k_step<IO, 64>), grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, state, yo, H, P, G); break;
    case 128: hipLaunchKernelGGL((k_step<IO, 128>), grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, state, yo, H, P, G); break;
    case 256: hipLaunchKernelGGL((k_step<IO, 256>), grid, dim3(256), 0, stream, xi, dt, A, bi, ci, D, state, yo, H, P, G); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool step_supported(int N) { return N == 16 || N == 32 || N == 64 || N == 128 || N == 256; }

hipError_t launch_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
                       const float *D, float *state, void *y, bool bf16, int64_t S, int H, int P,
                       int N, int G, hipStream_t stream) {
  if (S == 0) return hipSuccess;
  return bf16 ? launch_step_t<uint16_t>(x, dt, A, B, C, D, state, y, S, H, P, N, G, stream)
              : launch_step_t<float>(x, dt, A, B, C, D, state, y, S, H, P, N, G, stream);
}

}  // namespace ssd
