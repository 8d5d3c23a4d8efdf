// libssd: the memory-bound stages -- packed-batch chunk table, chunk_cumsum
// and state_passing (gfx950).
//
// chunk_cumsum builds the log-space cumulative decay of each chunk: the
// product of scalar decays between two tokens is exp(s_j - s_i) with s the
// running sum of dt*A (page "State Space Duality and Mamba-2: Unifying
// Transformers and Semiseparable Matrices", section "The Scalar-Identity
// Structural Constraint").  state_passing is the scalar recurrence that hands
// the P x N state from chunk to chunk (page "Mamba-2 Architecture: State Space
// Duality Explained", section "2. The Chunked SSD Algorithm", item 2).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ------------------------------------------------------------------ chunk table
// One block.  For each sequence s (clamped to [0, T]) emits ceil(len_s / Q)
// chunks (sequence, first token, length, 0), numbered by an exclusive prefix
// over sequences; the directory gets the first chunk of every sequence, the
// total, and an error word (nonzero when cu_seqlens is not a non-decreasing
// run from 0 to T).  Entries past the total are (-1, 0, 0, 0).  No access
// leaves [0, nc_max) whatever cu_seqlens holds.
constexpr int kTableThreads = 1024;

__global__ __launch_bounds__(kTableThreads) void k_chunk_table(const int32_t *__restrict__ cu,
                                                              int32_t nseq, int32_t T, int32_t Q,
                                                              int32_t nc_max,
                                                              int32_t *__restrict__ table,
                                                              int32_t *__restrict__ dir) {
  __shared__ int32_t scan[kTableThreads];
  __shared__ int32_t carry_s;
  __shared__ int32_t err_s;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_s = 0;
    err_s = (cu[0] != 0 || cu[nseq] != T) ? 1 : 0;
  }
  __syncthreads();
  for (int base = 0; base < nseq; base += kTableThreads) {
    const int s = base + tid;
    int32_t b = 0, len = 0, nc = 0;
    if (s < nseq) {
      const int32_t lo = cu[s], hi = cu[s + 1];
      if (hi < lo) atomicOr(&err_s, 1);
      b = min(max(lo, 0), T);
      const int32_t e = min(max(hi, 0), T);
      len = max(e - b, 0);
      nc = (len + Q - 1) / Q;
    }
    scan[tid] = nc;
    __syncthreads();
    // Hillis-Steele inclusive scan over the block
    for (int off = 1; off < kTableThreads; off <<= 1) {
      const int32_t v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int32_t first = carry_s + scan[tid] - nc;
    if (s < nseq) {
      dir[s] = min(first, nc_max);
      for (int k = 0; k < nc; ++k) {
        const int32_t idx = first + k;
        if (idx >= nc_max) {
          atomicOr(&err_s, 2);
          break;
        }
        int4 ent;
        ent.x = s;
        ent.y = b + k * Q;
        ent.z = min(Q, len - k * Q);
        ent.w = 0;
        reinterpret_cast<int4 *>(table)[idx] = ent;
      }
    }
    __syncthreads();
    if (tid == kTableThreads - 1) carry_s += scan[tid];
    __syncthreads();
  }
  const int32_t total = min(carry_s, nc_max);
  for (int idx = total + tid; idx < nc_max; idx += kTableThreads) {
    reinterpret_cast<int4 *>(table)[idx] = make_int4(-1, 0, 0, 0);
  }
  if (tid == 0) {
    dir[nseq] = total;
    dir[nseq + 1] = err_s;
  }
}

hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, int32_t *table,
                              int32_t *dir, hipStream_t stream) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(kTableThreads), 0, stream, cu_seqlens,
                     (int32_t)geo.nrows, (int32_t)geo.tokens, geo.Q, (int32_t)geo.nc_max, table,
                     dir);
  return hipGetLastError();
}

// ------------------------------------------------------------------ chunk_cumsum
// Block = (chunk, 16 heads); 4 waves, each scans 4 heads.  A wave scans Q
// values: lane i holds Q/64 consecutive tokens, a serial prefix in registers,
// then an inclusive scan of the lane totals across the wavefront.  Outputs are
// transposed to chunk-major, Q-contiguous rows (acum, dtq), so the contraction
// kernels read them with unit stride.  H heads of dt and A; with hr > 1 each
// head's rows are written for its hr kernel heads h * hr .. h * hr + hr - 1.
constexpr int kCumsumHeads = 16;

template <int Q>
__global__ __launch_bounds__(256) void k_chunk_cumsum(const float *__restrict__ dt,
                                                      const float *__restrict__ A, ChunkGeom geom,
                                                      int H, int hr, float *__restrict__ acum,
                                                      float *__restrict__ dtq) {
  constexpr int E = Q / 64;  // tokens per lane
  __shared__ float sdt[kCumsumHeads][Q + 1];
  const int c = blockIdx.x;
  const int hbase = blockIdx.y * kCumsumHeads;
  const ChunkInfo ci = chunk_info(geom, c);
  if (ci.len <= 0) return;
  for (int idx = threadIdx.x; idx < Q * kCumsumHeads; idx += 256) {
    const int l = idx / kCumsumHeads;
    const int j = idx - l * kCumsumHeads;
    const int h = hbase + j;
    float v = 0.f;
    if (l < ci.len && h < H) v = dt[(ci.t0 + l) * (int64_t)H + h];
    sdt[j][l] = v;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int j = wave; j < kCumsumHeads; j += 4) {
    const int h = hbase + j;
    if (h >= H) break;
    const float a = A[h];
    float v[E], pre[E];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[e] = sdt[j][lane * E + e];
      run += v[e] * a;
      pre[e] = run;
    }
    // inclusive scan of the lane totals over the wavefront by DPP: shifts
    // 1, 2, 4, 8 within each 16-lane row, then row 15's total carried into
    // the next row and lane 31's into the upper half (invalid sources add 0)
    float incl = run;
    auto dpp = [](float x, auto ctrl, auto rows) {
      return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                        decltype(rows)::value, 0xF, false));
    };
    incl += dpp(incl, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xF>{});
    incl += dpp(incl, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xF>{});
    incl += dpp(incl, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xF>{});
    incl += dpp(incl, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xF>{});
    incl += dpp(incl, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});
    incl += dpp(incl, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});
    // exclusive value: the previous lane's inclusive one (DPP wave_shr:1, 0 into lane 0)
    const float excl = dpp(incl, std::integral_constant<int, 0x138>{}, std::integral_constant<int, 0xF>{});
    // positions past a partial chunk's end repeat the value at its last token
    const int last = ci.len - 1;
    float mine = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e == last % E) mine = excl + pre[e];
    }
    const float lastval = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), last / E));
    for (int r = 0; r < hr; ++r) {
      float *ao = acum + ((int64_t)c * H * hr + (int64_t)h * hr + r) * Q + lane * E;
      float *dq = dtq + ((int64_t)c * H * hr + (int64_t)h * hr + r) * Q + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ao[e] = lane * E + e < ci.len ? excl + pre[e] : lastval;
        dq[e] = v[e];
      }
    }
  }
}

hipError_t launch_chunk_cumsum(const float *dt, const float *A, const Geometry &geo, float *acum,
                               float *dtq, hipStream_t stream) {
  if (geo.nc_max == 0) return hipSuccess;
  const ChunkGeom cg{geo.L, geo.nc_row, geo.Q, geo.table};
  const int Hd = geo.H / geo.hr;  // heads of dt and A
  const dim3 grid((unsigned)geo.nc_max, (unsigned)((Hd + kCumsumHeads - 1) / kCumsumHeads));
  switch (geo.Q) {
    case 64:
      hipLaunchKernelGGL(k_chunk_cumsum<64>, grid, dim3(256), 0, stream, dt, A, cg, Hd, geo.hr, acum, dtq);
      break;
    case 128:
      hipLaunchKernelGGL(k_chunk_cumsum<128>, grid, dim3(256), 0, stream, dt, A, cg, Hd, geo.hr, acum, dtq);
      break;
    case 256:
      hipLaunchKernelGGL(k_chunk_cumsum<256>, grid, dim3(256), 0, stream, dt, A, cg, Hd, geo.hr, acum, dtq);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ state_passing
// Thread = 4 consecutive state elements of one (sequence, head); it walks the
// sequence's chunks in order: hprev[c] = h; h = exp(acum_last[c]) * h + S[c].
// Loads of S are issued kBatch chunks ahead so the serial FMA chain does not
// wait on HBM latency one chunk at a time.  S and hprev are bf16 for bf16 io
// (kBf16), fp32 otherwise; the carried state is fp32 either way.
constexpr int kPassThreads = 256;
constexpr int kPassVec = 4;
// chunks whose S loads are in flight together: 128 bytes a thread either way
template <bool kBf16> constexpr int kBatch = kBf16 ? 16 : 8;

template <bool kBf16>
__global__ __launch_bounds__(kPassThreads) void k_state_passing(
    const void *__restrict__ states_v, void *__restrict__ hprev_v, const float *__restrict__ acum,
    const float *init, float *final_state, int H, int PN, int Q, int nc_row,
    const int32_t *__restrict__ dir) {
  const int e0 = (blockIdx.x * kPassThreads + threadIdx.x) * kPassVec;
  if (e0 >= PN) return;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  int cb, ce;
  if (dir) {
    cb = dir[s];
    ce = dir[s + 1];
  } else {
    cb = s * nc_row;
    ce = cb + nc_row;
  }
  f32x4 st = {0.f, 0.f, 0.f, 0.f};
  const int64_t soff = ((int64_t)s * H + h) * PN + e0;
  if (init) st = *reinterpret_cast<const f32x4 *>(init + soff);
  constexpr int NB = kBatch<kBf16>;
  for (int c = cb; c < ce; c += NB) {
    // raw loads only here (bf16 pairs are widened where they are used, so no
    // load waits for another)
    f32x4 sv[NB];
    u32x2 sb[NB];
    float dl[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (c + k < ce) {
        const int64_t ch = (int64_t)(c + k) * H + h;
        if (kBf16)
          sb[k] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(states_v) + ch * PN + e0));
        else
          sv[k] = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4 *>(static_cast<const float *>(states_v) + ch * PN + e0));
        dl[k] = acum[ch * Q + Q - 1];
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (c + k < ce) {
        const int64_t ch = (int64_t)(c + k) * H + h;
        if (kBf16) {
          u32x2 w;
          w.x = pack_bf16x2(st.x, st.y);
          w.y = pack_bf16x2(st.z, st.w);
          *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(hprev_v) + ch * PN + e0) = w;
        } else {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(hprev_v) + ch * PN + e0) = st;
        }
        const float d = __expf(dl[k]);
        if (kBf16)
          st = d * st + f32x4{bf16lo(sb[k].x), bf16hi(sb[k].x), bf16lo(sb[k].y), bf16hi(sb[k].y)};
        else
          st = d * st + sv[k];
      }
    }
  }
  if (final_state) *reinterpret_cast<f32x4 *>(final_state + soff) = st;
}

hipError_t launch_state_passing(const void *states, void *hprev, bool bf16,
                                const float *acum, const float *init, float *final_state,
                                const Geometry &geo, hipStream_t stream) {
  const int PN = geo.P * geo.N;
  if (geo.nrows == 0) return hipSuccess;
  const dim3 grid((unsigned)((PN / kPassVec + kPassThreads - 1) / kPassThreads), (unsigned)geo.H,
                  (unsigned)geo.nrows);
  if (bf16) {
    hipLaunchKernelGGL(k_state_passing<true>, grid, dim3(kPassThreads), 0, stream, states, hprev,
                       acum, init, final_state, geo.H, PN, geo.Q, geo.nc_row,
                       geo.packed ? geo.dir : nullptr);
  } else {
    hipLaunchKernelGGL(k_state_passing<false>, grid, dim3(kPassThreads), 0, stream, states, hprev,
                       acum, init, final_state, geo.H, PN, geo.Q, geo.nc_row,
                       geo.packed ? geo.dir : nullptr);
  }
  return hipGetLastError();
}

}  // namespace ssd
