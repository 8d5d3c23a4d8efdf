// libssd C ABI: argument validation, workspace layout and launch order.
// Every check runs before the first HIP call, so a rejected call leaves all
// device state untouched and can be tested on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "ssd.h"
#include "ssd_launch.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
  ssd::Geometry geo;
  ssd_workspace_layout ws;
  bool bf16;
  bool mfma;  // bf16 on the MFMA stage kernels (else the vector-ALU ones)
  size_t io_size;
};

// Validates dims + chunk length and computes geometry and workspace layout.
// vec: run every stage on the vector-ALU kernels (one kernel head per head)
ssd_status make_plan(const ssd_dims *d, int chunk_len, Plan *plan, bool vec = false) {
  if (!d || !plan) return SSD_ERR_INVALID_ARG;
  if (d->reserved != 0) return SSD_ERR_INVALID_ARG;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
      d->ngroups < 1 || d->nseq < 0)
    return SSD_ERR_INVALID_ARG;
  if (d->nseq > 0 && d->batch != 1) return SSD_ERR_INVALID_ARG;
  if (chunk_len < 1) return SSD_ERR_INVALID_ARG;
  if (chunk_len != 64 && chunk_len != 128 && chunk_len != 256) return SSD_ERR_UNSUPPORTED;
  // heads split evenly over the groups: the only head-to-group map compiled
  if (d->nheads % d->ngroups != 0) return SSD_ERR_UNSUPPORTED;
  const int64_t Hd = d->nheads, Pd = d->headdim, N = d->dstate, G = d->ngroups;
  const bool bf16 = d->io_dtype == SSD_BF16;
  if (Pd % 16 != 0 || N % 16 != 0 || Pd > 256 || N > 256) return SSD_ERR_UNSUPPORTED;
  // bf16: a head dim of 64 hr runs as hr kernel heads of 64 state rows on the
  // MFMA stage kernels; the other bf16 shapes (head dims not a multiple of 64,
  // state sizes other than 64 / 128 / 256) run on the vector-ALU ones
  const bool mfma = !vec && bf16 && Pd % 64 == 0 &&
                    ssd::chunk_state_bf16_supported(64, (int)N, chunk_len) &&
                    ssd::chunk_scan_bf16_supported(64, (int)N, chunk_len);
  const int64_t hr = mfma ? Pd / 64 : 1;
  const int64_t H = Hd * hr, P = Pd / hr;
  // grid limits: heads and rows sit on grid y / z (at most 65535)
  const int64_t nrows = d->nseq > 0 ? d->nseq : d->batch;
  if (H > 65535 || nrows > 65535) return SSD_ERR_UNSUPPORTED;
  const int64_t T = d->nseq > 0 ? d->seqlen : d->batch * d->seqlen;
  if (d->nseq == 0 && d->seqlen > 0 && d->batch > INT64_MAX / d->seqlen) return SSD_ERR_UNSUPPORTED;
  if (T >= ((int64_t)1 << 31)) return SSD_ERR_UNSUPPORTED;
  const int64_t Q = chunk_len;
  const int64_t nc_row = d->nseq > 0 ? 0 : ceil_div(d->seqlen, Q);
  const int64_t nc_max = d->nseq > 0 ? ceil_div(T, Q) + d->nseq : d->batch * nc_row;
  // the (chunk, head) grids launch 8*ceil(nc/8)*H blocks of up to 256 threads
  if ((nc_max + 8) * H >= ((int64_t)1 << 24)) return SSD_ERR_UNSUPPORTED;

  Plan p{};
  p.bf16 = bf16;
  p.mfma = mfma;
  p.io_size = bf16 ? 2 : 4;
  ssd::Geometry &g = p.geo;
  g.tokens = T;
  g.L = d->nseq > 0 ? T : d->seqlen;
  g.nc_row = (int32_t)nc_row;
  g.Q = chunk_len;
  g.nc_max = nc_max;
  g.nrows = nrows;
  g.H = (int32_t)H;
  g.P = (int32_t)P;
  g.N = (int32_t)N;
  g.G = (int32_t)G;
  g.hr = (int32_t)hr;
  g.packed = d->nseq > 0;
  g.table = nullptr;
  g.dir = nullptr;

  ssd_workspace_layout &w = p.ws;
  size_t off = 0;
  const size_t nch = (size_t)nc_max * (size_t)H;
  w.nc_max = nc_max;
  w.acum_offset = off;
  off = align_up(off + nch * Q * sizeof(float));
  w.dtq_offset = off;
  off = align_up(off + nch * Q * sizeof(float));
  w.states_offset = off;
  off = align_up(off + nch * (size_t)(P * N) * p.io_size);
  w.hprev_offset = off;
  off = align_up(off + nch * (size_t)(P * N) * p.io_size);
  if (g.packed) {
    w.chunk_table_offset = off;
    off = align_up(off + (size_t)nc_max * 4 * sizeof(int32_t));
    w.chunk_dir_offset = off;
    off = align_up(off + (size_t)(d->nseq + 2) * sizeof(int32_t));
  } else {
    w.chunk_table_offset = 0;
    w.chunk_dir_offset = 0;
  }
  w.total_bytes = off == 0 ? kAlign : off;
  *plan = p;
  return SSD_OK;
}

// Binds the workspace pointers of the plan; checks size and alignment.
ssd_status bind_workspace(Plan *p, void *workspace, size_t workspace_bytes) {
  if (!workspace || workspace_bytes < p->ws.total_bytes) return SSD_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SSD_ERR_INVALID_ARG;
  if (p->geo.packed) {
    char *base = static_cast<char *>(workspace);
    p->geo.table = reinterpret_cast<const int32_t *>(base + p->ws.chunk_table_offset);
    p->geo.dir = reinterpret_cast<const int32_t *>(base + p->ws.chunk_dir_offset);
  }
  return SSD_OK;
}

template <typename T>
T *ws_ptr(void *workspace, size_t offset) {
  return reinterpret_cast<T *>(static_cast<char *>(workspace) + offset);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

struct Sizes {
  size_t x, bc, dt, state;
};

Sizes tensor_bytes(const Plan &p) {
  const ssd::Geometry &g = p.geo;
  Sizes s;
  s.x = (size_t)g.tokens * g.H * g.P * p.io_size;
  s.bc = (size_t)g.tokens * g.G * g.N * p.io_size;
  s.dt = (size_t)g.tokens * (g.H / g.hr) * sizeof(float);
  s.state = (size_t)g.nrows * g.H * g.P * g.N * sizeof(float);
  return s;
}

// Token tensors may be NULL only when there are no tokens.
bool tok_ptr_ok(const void *ptr, const Plan &p, size_t align) {
  if (p.geo.tokens == 0) return ptr == nullptr || aligned(ptr, align);
  return ptr != nullptr && aligned(ptr, align);
}

ssd_status check_cumsum_args(const float *dt, const float *A, const int32_t *cu, const Plan &p) {
  if (!tok_ptr_ok(dt, p, 4)) return SSD_ERR_INVALID_ARG;
  if (!A || !aligned(A, 4)) return SSD_ERR_INVALID_ARG;
  if (p.geo.packed && (!cu || !aligned(cu, 4))) return SSD_ERR_INVALID_ARG;
  return SSD_OK;
}

ssd_status check_state_args(const void *x, const void *B, const Plan &p) {
  if (!tok_ptr_ok(x, p, 16) || !tok_ptr_ok(B, p, 16)) return SSD_ERR_INVALID_ARG;
  return SSD_OK;
}

ssd_status check_pass_args(const float *init, const float *fin, const Plan &p) {
  const size_t sb = tensor_bytes(p).state;
  if (init && !aligned(init, 16)) return SSD_ERR_INVALID_ARG;
  if (fin && !aligned(fin, 16)) return SSD_ERR_INVALID_ARG;
  if (init && fin && init != fin && overlaps(init, sb, fin, sb)) return SSD_ERR_INVALID_ARG;
  return SSD_OK;
}

ssd_status check_scan_args(const void *x, const void *B, const void *C, const float *D, const void *y,
                           const float *dt, const Plan &p) {
  if (!tok_ptr_ok(x, p, 16) || !tok_ptr_ok(B, p, 16) || !tok_ptr_ok(C, p, 16) ||
      !tok_ptr_ok(y, p, 16))
    return SSD_ERR_INVALID_ARG;
  if (D && !aligned(D, 4)) return SSD_ERR_INVALID_ARG;
  const Sizes s = tensor_bytes(p);
  if (overlaps(y, s.x, x, s.x) || overlaps(y, s.x, B, s.bc) || overlaps(y, s.x, C, s.bc) ||
      overlaps(y, s.x, dt, s.dt))
    return SSD_ERR_INVALID_ARG;
  return SSD_OK;
}

ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

ssd_status run_cumsum(const float *dt, const float *A, const int32_t *cu, const Plan &p,
                      void *ws, hipStream_t st) {
  if (p.geo.packed) {
    hipError_t e = ssd::launch_chunk_table(cu, p.geo, ws_ptr<int32_t>(ws, p.ws.chunk_table_offset),
                                           ws_ptr<int32_t>(ws, p.ws.chunk_dir_offset), st);
    if (e != hipSuccess) return SSD_ERR_HIP;
  }
  return hip_status(ssd::launch_chunk_cumsum(dt, A, p.geo, ws_ptr<float>(ws, p.ws.acum_offset),
                                             ws_ptr<float>(ws, p.ws.dtq_offset), st));
}

ssd_status run_state(const void *x, const void *B, const Plan &p, void *ws, hipStream_t st) {
  const float *acum = ws_ptr<float>(ws, p.ws.acum_offset);
  const float *dtq = ws_ptr<float>(ws, p.ws.dtq_offset);
  void *states = ws_ptr<void>(ws, p.ws.states_offset);
  if (p.mfma)
    return hip_status(ssd::launch_chunk_state_bf16(x, B, acum, dtq, states, p.geo, st));
  return hip_status(ssd::launch_chunk_state_vec(x, B, acum, dtq, states, p.bf16, p.geo, st));
}

ssd_status run_pass(const float *init, float *fin, const Plan &p, void *ws, hipStream_t st) {
  return hip_status(ssd::launch_state_passing(
      ws_ptr<void>(ws, p.ws.states_offset), ws_ptr<void>(ws, p.ws.hprev_offset), p.bf16,
      ws_ptr<float>(ws, p.ws.acum_offset), init, fin, p.geo, st));
}

ssd_status run_scan(const void *x, const void *B, const void *C, const float *D, void *y,
                    const Plan &p, void *ws, hipStream_t st) {
  const float *acum = ws_ptr<float>(ws, p.ws.acum_offset);
  const float *dtq = ws_ptr<float>(ws, p.ws.dtq_offset);
  const void *hprev = ws_ptr<void>(ws, p.ws.hprev_offset);
  if (p.mfma)
    return hip_status(ssd::launch_chunk_scan_bf16(x, B, C, D, acum, dtq, hprev, y, p.geo, st));
  return hip_status(
      ssd::launch_chunk_scan_vec(x, B, C, D, acum, dtq, hprev, y, p.bf16, p.geo, st));
}

}  // namespace

extern "C" {

size_t ssd_workspace_size(const ssd_dims *dims, int chunk_len) {
  Plan p;
  if (make_plan(dims, chunk_len, &p) != SSD_OK) return 0;
  return p.ws.total_bytes;
}

ssd_status ssd_get_workspace_layout(const ssd_dims *dims, int chunk_len, ssd_workspace_layout *out) {
  if (!out) return SSD_ERR_INVALID_ARG;
  Plan p;
  const ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  *out = p.ws;
  return SSD_OK;
}

ssd_status ssd_chunk_cumsum(const float *dt, const float *A, int chunk_len, const int32_t *cu_seqlens,
                            const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                            void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  return run_cumsum(dt, A, cu_seqlens, p, workspace, static_cast<hipStream_t>(stream));
}

ssd_status ssd_chunk_state(const void *x, const void *B, int chunk_len, const ssd_dims *dims,
                           void *workspace, size_t workspace_bytes, void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_state_args(x, B, p)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  return run_state(x, B, p, workspace, static_cast<hipStream_t>(stream));
}

ssd_status ssd_state_passing(const float *init_state, float *final_state, int chunk_len,
                             const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                             void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_pass_args(init_state, final_state, p)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  return run_pass(init_state, final_state, p, workspace, static_cast<hipStream_t>(stream));
}

ssd_status ssd_chunk_scan(const void *x, const void *B, const void *C, const float *D, void *y,
                          int chunk_len, const ssd_dims *dims, void *workspace,
                          size_t workspace_bytes, void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, y, nullptr, p)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  return run_scan(x, B, C, D, y, p, workspace, static_cast<hipStream_t>(stream));
}

ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, int chunk_len,
                              const float *init_state, const int32_t *cu_seqlens, void *y,
                              float *final_state, const ssd_dims *dims, void *workspace,
                              size_t workspace_bytes, void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = check_state_args(x, B, p)) != SSD_OK) return s;
  if ((s = check_pass_args(init_state, final_state, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, y, dt, p)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = run_cumsum(dt, A, cu_seqlens, p, workspace, st)) != SSD_OK) return s;
  if ((s = run_state(x, B, p, workspace, st)) != SSD_OK) return s;
  if ((s = run_pass(init_state, final_state, p, workspace, st)) != SSD_OK) return s;
  return run_scan(x, B, C, D, y, p, workspace, st);
}

}  // extern "C"

// The allocation-free forward's workspace: one fixed array in every device's
// global memory, held until the process ends.  In host code `scratch` only
// names the symbol; its device address (a different one on each device) comes
// from hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
ssd_status current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SSD_ERR_HIP;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return SSD_OK;
}

}  // namespace

extern "C" {

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *B, const void *C, const float *D, int chunk_len,
                                      const float *init_state, const int32_t *cu_seqlens, void *y,
                                      float *final_state, const ssd_dims *dims, void *stream) {
  Plan p;
  ssd_status s = make_plan(dims, chunk_len, &p);
  if (s != SSD_OK) return s;
  if (p.ws.total_bytes > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = check_state_args(x, B, p)) != SSD_OK) return s;
  if ((s = check_pass_args(init_state, final_state, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, y, dt, p)) != SSD_OK) return s;
  void *ws = nullptr;
  if ((s = current_scratch(&ws)) != SSD_OK) return s;
  if ((s = bind_workspace(&p, ws, SSD_NOALLOC_SCRATCH_BYTES)) != SSD_OK) return s;
  // Nothing in the workspace needs clearing: every stage writes what a later
  // one reads (the chunk table included) before it is read.
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = run_cumsum(dt, A, cu_seqlens, p, ws, st)) != SSD_OK) return s;
  if ((s = run_state(x, B, p, ws, st)) != SSD_OK) return s;
  if ((s = run_pass(init_state, final_state, p, ws, st)) != SSD_OK) return s;
  return run_scan(x, B, C, D, y, p, ws, st);
}

ssd_status ssd_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
                    const float *D, float *state, void *y, const ssd_dims *d, void *stream) {
  if (!d) return SSD_ERR_INVALID_ARG;
  if (d->reserved != 0) return SSD_ERR_INVALID_ARG;
  if (d->io_dtype != SSD_F32 && d->io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  if (d->batch < 0 || d->seqlen != 1 || d->nseq != 0 || d->nheads < 1 || d->headdim < 1 ||
      d->dstate < 1 || d->ngroups < 1)
    return SSD_ERR_INVALID_ARG;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_UNSUPPORTED;
  const int64_t S = d->batch, H = d->nheads, P = d->headdim, N = d->dstate, G = d->ngroups;
  if (!ssd::step_supported((int)N)) return SSD_ERR_UNSUPPORTED;
  // one block per (sequence, head); element offsets of the state below 2^62
  if (H > (1 << 20) || P > (1 << 20) || S * H >= ((int64_t)1 << 31)) return SSD_ERR_UNSUPPORTED;
  if (!A || !aligned(A, 4) || (D && !aligned(D, 4))) return SSD_ERR_INVALID_ARG;
  if (S == 0) return SSD_OK;
  const size_t io = d->io_dtype == SSD_BF16 ? 2 : 4;
  const size_t xb = (size_t)S * H * P * io, bcb = (size_t)S * G * N * io, dtb = (size_t)S * H * 4;
  const size_t sb = (size_t)S * H * P * N * 4;
  if (!x || !dt || !B || !C || !state || !y) return SSD_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(dt, 4) || !aligned(B, 16) || !aligned(C, 16) ||
      !aligned(state, 16) || !aligned(y, 16))
    return SSD_ERR_INVALID_ARG;
  if (overlaps(state, sb, x, xb) || overlaps(state, sb, B, bcb) || overlaps(state, sb, C, bcb) ||
      overlaps(state, sb, dt, dtb) || overlaps(state, sb, y, xb) || overlaps(state, sb, A, H * 4) ||
      (D && overlaps(state, sb, D, H * 4)))
    return SSD_ERR_INVALID_ARG;
  if (overlaps(y, xb, x, xb) || overlaps(y, xb, B, bcb) || overlaps(y, xb, C, bcb) ||
      overlaps(y, xb, dt, dtb))
    return SSD_ERR_INVALID_ARG;
  return hip_status(ssd::launch_step(x, dt, A, B, C, D, state, y, io == 2, S, (int)H, (int)P,
                                     (int)N, (int)G, static_cast<hipStream_t>(stream)));
}

ssd_status ssd_conv1d_silu(const void *in, int64_t in_stride, const float *weight,
                           const float *bias, int K, void *out, int64_t out_stride, int64_t batch,
                           int64_t seqlen, int64_t nseq, const int32_t *cu_seqlens,
                           int64_t channels, int32_t io_dtype, void *stream) {
  if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  const int64_t vec = io_dtype == SSD_BF16 ? 8 : 4;
  const size_t io = io_dtype == SSD_BF16 ? 2 : 4;
  if (K < 1 || channels < 1 || batch < 1 || seqlen < 0 || nseq < 0) return SSD_ERR_INVALID_ARG;
  if (K > 4) return SSD_ERR_UNSUPPORTED;
  if (channels % vec || in_stride < channels || out_stride < channels || in_stride % vec ||
      out_stride % vec)
    return SSD_ERR_INVALID_ARG;
  if (nseq > 0 && batch != 1) return SSD_ERR_INVALID_ARG;
  if (nseq == 0 && seqlen > 0 && batch > INT64_MAX / seqlen) return SSD_ERR_UNSUPPORTED;
  const int64_t T = nseq > 0 ? seqlen : batch * seqlen;
  if (T >= ((int64_t)1 << 31) || nseq >= ((int64_t)1 << 31) || channels >= ((int64_t)1 << 31))
    return SSD_ERR_UNSUPPORTED;
  if (!weight || !aligned(weight, 4) || (bias && !aligned(bias, 4))) return SSD_ERR_INVALID_ARG;
  if (nseq > 0 && (!cu_seqlens || !aligned(cu_seqlens, 4))) return SSD_ERR_INVALID_ARG;
  if (T == 0) return SSD_OK;
  if (!in || !out || !aligned(in, 16) || !aligned(out, 16)) return SSD_ERR_INVALID_ARG;
  const size_t inb = ((size_t)(T - 1) * in_stride + channels) * io;
  const size_t outb = ((size_t)(T - 1) * out_stride + channels) * io;
  if (overlaps(in, inb, out, outb)) return SSD_ERR_INVALID_ARG;
  return hip_status(ssd::launch_conv1d_silu(in, in_stride, weight, bias, K, out, out_stride, T,
                                            nseq > 0 ? 0 : seqlen, (int)nseq,
                                            nseq > 0 ? cu_seqlens : nullptr, channels,
                                            io_dtype == SSD_BF16, static_cast<hipStream_t>(stream)));
}

ssd_status ssd_gate_rmsnorm(const void *y, const void *z, const float *weight, float eps, void *out,
                            int64_t tokens, int64_t width, int32_t io_dtype, void *stream) {
  if (io_dtype != SSD_F32 && io_dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  const int64_t vec = io_dtype == SSD_BF16 ? 8 : 4;
  const size_t io = io_dtype == SSD_BF16 ? 2 : 4;
  if (tokens < 0 || width < 1 || width % vec || !(eps >= 0.f)) return SSD_ERR_INVALID_ARG;
  if (tokens >= ((int64_t)1 << 31) || width >= ((int64_t)1 << 30)) return SSD_ERR_UNSUPPORTED;
  if (weight && !aligned(weight, 4)) return SSD_ERR_INVALID_ARG;
  if (tokens == 0) return SSD_OK;
  if (!y || !z || !out || !aligned(y, 16) || !aligned(z, 16) || !aligned(out, 16))
    return SSD_ERR_INVALID_ARG;
  const size_t nb = (size_t)tokens * width * io;
  if ((out != y && overlaps(out, nb, y, nb)) || (out != z && overlaps(out, nb, z, nb)))
    return SSD_ERR_INVALID_ARG;
  return hip_status(ssd::launch_gate_rmsnorm(y, z, weight, eps, out, tokens, (int)width,
                                             io_dtype == SSD_BF16,
                                             static_cast<hipStream_t>(stream)));
}

ssd_status ssd_fused_fwd(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, const float *init_state,
                         const int32_t *cu_seqlens, void *y, float *final_state,
                         const ssd_dims *dims, void *stream) {
  return ssd_fused_fwd_train(x, dt, A, B, C, D, init_state, cu_seqlens, y, final_state, nullptr, 0,
                             dims, stream);
}

}  // extern "C"

namespace {

// Plan of the one-pass forward and its backward: the chunked plan's checks,
// then the one-pass shape limits.
ssd_status make_fused_plan(const ssd_dims *dims, Plan *p) {
  ssd_status s = make_plan(dims, 64, p);  // the chunk length only sizes the (unused) workspace
  if (s != SSD_OK) return s;
  if (!p->bf16 || !ssd::fused_supported(p->geo.H, p->geo.P, p->geo.N, p->geo.G))
    return SSD_ERR_UNSUPPORTED;
  if (p->geo.nrows >= ((int64_t)1 << 24) / p->geo.H) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// The backward's shapes: head dim 64 (no head split), N in {64, 128, 256}, an
// even number of heads per group (its reverse sweep pairs the heads of a
// group).  Its kernels hold N <= 128; N = 256 runs as two halves of 128 state
// columns (split_bwd).
bool bwd_supported(const Plan &p) {
  return p.geo.hr == 1 && (p.geo.N == 64 || p.geo.N == 128 || p.geo.N == 256) &&
         (p.geo.H / p.geo.G) % 2 == 0;
}

// 32-token chunks of the batch (packed: an upper bound, ceil(T/32) + nseq)
int64_t chunks32(const Plan &p) {
  const ssd::Geometry &g = p.geo;
  return g.packed ? ceil_div(g.tokens, 32) + g.nrows : g.nrows * ceil_div(g.L, 32);
}

// 64-token pairs of chunks (packed: an upper bound, ceil(T/64) + nseq)
int64_t pairs64(const Plan &p) {
  const ssd::Geometry &g = p.geo;
  return g.packed ? ceil_div(g.tokens, 64) + g.nrows : g.nrows * ceil_div(g.L, 64);
}

size_t chunk_states_bytes(const Plan &p) {
  return align_up((size_t)pairs64(p) * p.geo.H * p.geo.P * p.geo.N * 2);
}

// The backward's reverse sweep runs one block per (sequence, two heads); with
// fewer such blocks than the GPU has CUs (256 on MI355X) it is split into
// segments instead.  The decisions depend on the dims only.
bool bwd_segmented(const Plan &p) { return p.geo.nrows * (p.geo.H / 2) < 256; }

// Segments of seg_len tokens in the batch (packed: an upper bound,
// ceil(T / seg_len) + nseq)
int64_t bwd_segments(const Plan &p, int64_t seg_len) {
  const ssd::Geometry &g = p.geo;
  return g.packed ? ceil_div(g.tokens, seg_len) + g.nrows : g.nrows * ceil_div(g.L, seg_len);
}

// The segment length: the longest power of two from 256 tokens up that still
// gives at least 1024 (segment, head pair) blocks, four a CU.  Longer segments
// move fewer segment sums and entering gradients (fp32 P x N tiles, written and
// read twice) at the same parallelism.
int64_t bwd_seg_len(const Plan &p) {
  const ssd::Geometry &g = p.geo;
  const int64_t pairs = g.H / 2;
  auto blocks = [&](int64_t S) {
    return (g.packed ? ceil_div(g.tokens, S) : g.nrows * ceil_div(g.L, S)) * pairs;
  };
  int64_t S = 256;
  while (S < ((int64_t)1 << 20) && blocks(2 * S) >= 1024) S *= 2;
  return S;
}

// Backward workspace: the state gradients per pair (bf16), then, when the
// sweep is segmented, the segment sums and incoming gradients (fp32) and the
// segment decays.
struct BwdWorkspace {
  size_t gsave, gseg, gin, aseg, total;
  int64_t nseg, seglen;
  // N = 256, after one half's own workspace: its B, C and d(final_state), its
  // ddt (the second half's, added to the first's), dB, dC and d(init_state)
  size_t bh, ch, dfh, ddth, dbh, dch, dih;
};

BwdWorkspace bwd_workspace(const Plan &p) {
  if (p.geo.N == 256) {
    Plan ph = p;
    ph.geo.N = 128;
    BwdWorkspace w = bwd_workspace(ph);
    const ssd::Geometry &g = p.geo;
    const size_t bc = (size_t)g.tokens * g.G * 128, st = (size_t)g.nrows * g.H * g.P * 128;
    size_t off = w.total;
    auto take = [&](size_t bytes) {
      const size_t o = off;
      off += align_up(bytes);
      return o;
    };
    w.bh = take(bc * 2);
    w.ch = take(bc * 2);
    w.dfh = take(st * 4);
    w.ddth = take((size_t)g.tokens * g.H * 4);
    w.dbh = take(bc * 4);
    w.dch = take(bc * 4);
    w.dih = take(st * 4);
    w.total = off;
    return w;
  }
  BwdWorkspace w{};
  w.gsave = 0;
  size_t off = chunk_states_bytes(p);
  if (bwd_segmented(p)) {
    w.seglen = bwd_seg_len(p);
    w.nseg = bwd_segments(p, w.seglen);
    const size_t tile = (size_t)w.nseg * p.geo.H * p.geo.P * p.geo.N * 4;
    w.gseg = off;
    off += align_up(tile);
    w.gin = off;
    off += align_up(tile);
    w.aseg = off;
    off += align_up((size_t)w.nseg * p.geo.H * 4);
  }
  w.total = off;
  return w;
}

// The backward at N = 256 as two runs of the N = 128 kernels.  The state's
// columns n never mix in the recurrence: the state gradient, dB, dC and
// d(init_state) of columns [128 k, 128 k + 128) come from those columns of B,
// C, the saved states and d(final_state) alone, and dx, ddt and dA are sums
// over n, so each half adds its part (the D dy term and dD only in the first).
// Each half's B, C and d(final_state) are copied out of the 256-column rows
// into packed 128-column buffers in the workspace (the saved states are read
// in place, their rows 256 columns apart), its dB, dC and d(init_state) copied
// back into their columns; the second half's per-chunk pass adds its dx into
// the first's as it writes it, and its ddt is added to the first's after.
hipError_t split_bwd(const Plan &p, const BwdWorkspace &bw, const void *x, const float *dt,
                     const float *A, const void *B, const void *C, const float *D,
                     const int32_t *cu, const void *chunk_states, const void *dy,
                     const float *dfinal, void *dx, float *ddt, float *dA, float *dB, float *dC,
                     float *dD, float *dinit, void *workspace, hipStream_t st) {
  const ssd::Geometry &g = p.geo;
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  void *Bh = ws + bw.bh, *Ch = ws + bw.ch;
  float *dfh = dfinal ? reinterpret_cast<float *>(ws + bw.dfh) : nullptr;
  float *ddth = reinterpret_cast<float *>(ws + bw.ddth);
  float *dBh = reinterpret_cast<float *>(ws + bw.dbh), *dCh = reinterpret_cast<float *>(ws + bw.dch);
  float *dih = dinit ? reinterpret_cast<float *>(ws + bw.dih) : nullptr;
  const int64_t trows = g.tokens * g.G;          // (token, group) rows of B, C, dB, dC
  const int64_t frows = g.nrows * g.H * g.P;     // state rows of d(final), d(init)
  const unsigned char *b = static_cast<const unsigned char *>(B);
  const unsigned char *c = static_cast<const unsigned char *>(C);
  const unsigned char *s = static_cast<const unsigned char *>(chunk_states);
  hipError_t e = ssd::launch_fill_f32(dA, g.H, st);
  if (e == hipSuccess && dD) e = ssd::launch_fill_f32(dD, g.H, st);
  for (int k = 0; k < 2 && e == hipSuccess; ++k) {
    const int64_t o2 = k * 256, o4 = k * 512;  // the half's byte offset in a bf16 / fp32 row
    e = ssd::launch_copy2d16(b + o2, 512, Bh, 256, trows, 16, st);
    if (e == hipSuccess) e = ssd::launch_copy2d16(c + o2, 512, Ch, 256, trows, 16, st);
    if (e == hipSuccess && dfinal)
      e = ssd::launch_copy2d16(reinterpret_cast<const unsigned char *>(dfinal) + o4, 1024, dfh,
                               512, frows, 32, st);
    if (e == hipSuccess)
      e = ssd::launch_bwd_reverse(dy, dt, A, Ch, dfh, cu, g.L, g.tokens, (int)g.nrows, g.H, 128,
                                  g.G, workspace, dih, bw.nseg, (int)bw.seglen,
                                  ws_ptr<float>(workspace, bw.gseg),
                                  ws_ptr<float>(workspace, bw.aseg),
                                  ws_ptr<float>(workspace, bw.gin), st);
    if (e == hipSuccess)
      e = ssd::launch_bwd_chunk(x, dt, A, Bh, Ch, k ? nullptr : D, dy, s + o2, 256, workspace,
                                cu, g.L, g.tokens, (int)g.nrows, chunks32(p), g.H, 128, g.G,
                                k ? dx : nullptr, dx, k ? ddth : ddt, dA, dBh, dCh,
                                k ? nullptr : dD, st);
    if (e == hipSuccess)
      e = ssd::launch_copy2d16(dBh, 512, reinterpret_cast<unsigned char *>(dB) + o4, 1024, trows,
                               32, st);
    if (e == hipSuccess)
      e = ssd::launch_copy2d16(dCh, 512, reinterpret_cast<unsigned char *>(dC) + o4, 1024, trows,
                               32, st);
    if (e == hipSuccess && dinit)
      e = ssd::launch_copy2d16(dih, 512, reinterpret_cast<unsigned char *>(dinit) + o4, 1024,
                               frows, 32, st);
  }
  if (e == hipSuccess) e = ssd::launch_add_f32(ddt, ddth, g.tokens * g.H, st);
  return e;
}

}  // namespace

extern "C" {

size_t ssd_fused_states_size(const ssd_dims *dims) {
  Plan p;
  if (make_fused_plan(dims, &p) != SSD_OK) return 0;
  return chunk_states_bytes(p);
}

ssd_status ssd_fused_fwd_train(const void *x, const float *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *init_state,
                               const int32_t *cu_seqlens, void *y, float *final_state,
                               void *chunk_states, size_t states_bytes, const ssd_dims *dims,
                               void *stream) {
  Plan p;
  ssd_status s = make_fused_plan(dims, &p);
  if (s != SSD_OK) return s;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = check_state_args(x, B, p)) != SSD_OK) return s;
  if ((s = check_pass_args(init_state, final_state, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, y, dt, p)) != SSD_OK) return s;
  if (chunk_states) {
    if (!aligned(chunk_states, 16)) return SSD_ERR_INVALID_ARG;
    if (states_bytes < chunk_states_bytes(p)) return SSD_ERR_WORKSPACE;
    const Sizes z = tensor_bytes(p);
    const size_t hb = chunk_states_bytes(p);
    if (overlaps(chunk_states, hb, x, z.x) || overlaps(chunk_states, hb, y, z.x) ||
        overlaps(chunk_states, hb, B, z.bc) || overlaps(chunk_states, hb, C, z.bc) ||
        overlaps(chunk_states, hb, dt, z.dt) || overlaps(chunk_states, hb, init_state, z.state) ||
        overlaps(chunk_states, hb, final_state, z.state))
      return SSD_ERR_INVALID_ARG;
  }
  const ssd::Geometry &g = p.geo;
  return hip_status(ssd::launch_fused(x, dt, A, B, C, D, init_state,
                                      g.packed ? cu_seqlens : nullptr, g.L, g.tokens, (int)g.nrows,
                                      g.H, g.P, g.N, g.G, g.hr, y, final_state, chunk_states,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The split one-pass forward: fixed-length sequences cut into segments of
// seg_len tokens; its workspace holds the state entering every segment (fp32,
// [nrows][nseg][H][P][N]) and, for every segment but the last, its log2 decay
// (fp32, [nrows][nseg-1][H]).
struct SplitWorkspace {
  size_t sseg, lseg, total;
  int64_t nseg;
};

SplitWorkspace split_workspace(const Plan &p, int64_t seg_len) {
  SplitWorkspace w{};
  w.nseg = ceil_div(p.geo.L, seg_len);
  const int64_t nj = w.nseg > 1 ? w.nseg - 1 : 0;
  if (nj == 0) return w;
  const ssd::Geometry &g = p.geo;
  w.sseg = 0;
  w.lseg = align_up((size_t)g.nrows * w.nseg * g.H * g.P * g.N * 4);
  w.total = w.lseg + align_up((size_t)g.nrows * nj * g.H * 4);
  return w;
}

ssd_status make_split_plan(const ssd_dims *dims, int64_t seg_len, Plan *p) {
  ssd_status s = make_fused_plan(dims, p);
  if (s != SSD_OK) return s;
  if (seg_len < 32 || seg_len % 32 != 0) return SSD_ERR_INVALID_ARG;
  if (p->geo.packed) return SSD_ERR_UNSUPPORTED;
  const int64_t nseg = ceil_div(p->geo.L, seg_len);
  if (p->geo.nrows * nseg >= ((int64_t)1 << 24) / p->geo.H) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_fused_split_workspace_size(const ssd_dims *dims, int64_t seg_len) {
  Plan p;
  if (make_split_plan(dims, seg_len, &p) != SSD_OK) return 0;
  return split_workspace(p, seg_len).total;
}

int64_t ssd_fused_split_seg_len(const ssd_dims *dims) {
  Plan p;
  if (make_fused_plan(dims, &p) != SSD_OK || p.geo.packed) return 0;
  const ssd::Geometry &g = p.geo;
  const int64_t L32 = ceil_div(g.L, 32) * 32;
  const int64_t units = g.nrows * g.H, cus = ssd::device_cus();
  if (L32 == 0 || units >= 2 * cus) return L32;  // enough (sequence, head) rows already
  // about 8 (segment, head) rows a CU, segments a power of two of at least 512 tokens
  const int64_t want = g.nrows * g.L * g.H / (8 * cus);
  int64_t S = 512;
  while (S * 2 <= want) S *= 2;
  return S < L32 ? S : L32;
}

}  // extern "C"

namespace {

// ssd_fused_fwd_split with or without saving the per-pair states
ssd_status split_fwd(const void *x, const float *dt, const float *A, const void *B, const void *C,
                     const float *D, const float *init_state, void *y, float *final_state,
                     void *chunk_states, size_t states_bytes, int64_t seg_len,
                     const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                     void *stream) {
  Plan p;
  ssd_status s = make_split_plan(dims, seg_len, &p);
  if (s != SSD_OK) return s;
  if ((s = check_cumsum_args(dt, A, nullptr, p)) != SSD_OK) return s;
  if ((s = check_state_args(x, B, p)) != SSD_OK) return s;
  if ((s = check_pass_args(init_state, final_state, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, y, dt, p)) != SSD_OK) return s;
  const SplitWorkspace w = split_workspace(p, seg_len);
  const Sizes z = tensor_bytes(p);
  if (w.total > 0) {
    if (!workspace || workspace_bytes < w.total) return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SSD_ERR_INVALID_ARG;
    if (overlaps(workspace, w.total, x, z.x) || overlaps(workspace, w.total, y, z.x) ||
        overlaps(workspace, w.total, B, z.bc) || overlaps(workspace, w.total, C, z.bc) ||
        overlaps(workspace, w.total, dt, z.dt) ||
        overlaps(workspace, w.total, init_state, z.state) ||
        overlaps(workspace, w.total, final_state, z.state))
      return SSD_ERR_INVALID_ARG;
  }
  if (chunk_states) {
    if (seg_len % 64 != 0 || !aligned(chunk_states, 16)) return SSD_ERR_INVALID_ARG;
    const size_t hb = chunk_states_bytes(p);
    if (states_bytes < hb) return SSD_ERR_WORKSPACE;
    if (overlaps(chunk_states, hb, x, z.x) || overlaps(chunk_states, hb, y, z.x) ||
        overlaps(chunk_states, hb, B, z.bc) || overlaps(chunk_states, hb, C, z.bc) ||
        overlaps(chunk_states, hb, dt, z.dt) || overlaps(chunk_states, hb, init_state, z.state) ||
        overlaps(chunk_states, hb, final_state, z.state) ||
        (w.total > 0 && overlaps(chunk_states, hb, workspace, w.total)))
      return SSD_ERR_INVALID_ARG;
  }
  const ssd::Geometry &g = p.geo;
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  return hip_status(ssd::launch_fused_split(
      x, dt, A, B, C, D, init_state, g.L, (int)g.nrows, seg_len, g.H, g.P, g.N, g.G, g.hr, y,
      final_state, w.total ? reinterpret_cast<float *>(ws + w.sseg) : nullptr,
      w.total ? reinterpret_cast<float *>(ws + w.lseg) : nullptr, chunk_states,
      static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ssd_status ssd_fused_fwd_split(const void *x, const float *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *init_state, void *y,
                               float *final_state, int64_t seg_len, const ssd_dims *dims,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return split_fwd(x, dt, A, B, C, D, init_state, y, final_state, nullptr, 0, seg_len, dims,
                   workspace, workspace_bytes, stream);
}

ssd_status ssd_fused_fwd_split_train(const void *x, const float *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const float *init_state, void *y, float *final_state,
                                     void *chunk_states, size_t states_bytes, int64_t seg_len,
                                     const ssd_dims *dims, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (!chunk_states) return SSD_ERR_INVALID_ARG;
  return split_fwd(x, dt, A, B, C, D, init_state, y, final_state, chunk_states, states_bytes,
                   seg_len, dims, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The general backward: the forward's workspace at the vector path's chunk
// length (acum, dtq, chunk states, hprev, chunk table), then per chunk and
// head two fp32 P x N tiles: the dy C^T sums of the reverse hand-off, and the
// state gradient entering each chunk from the right.
struct VecBwdWorkspace {
  size_t rsum, ge, total;
};

// The general backward forms the chunk states again with the forward's stage
// kernels at its 64-token chunks: bf16 with a 64-row head dim and a state size
// the MFMA stage kernels take (one kernel head a head, so the layouts the
// vector backward reads are the same) uses those; every other shape the
// vector-ALU ones.
ssd_status make_vec_bwd_plan(const ssd_dims *dims, Plan *p) {
  const ssd_status s = make_plan(dims, ssd::bwd_vec_chunk_len(), p, false);
  if (s != SSD_OK || (p->mfma && p->geo.P == dims->headdim)) return s;
  return make_plan(dims, ssd::bwd_vec_chunk_len(), p, true);
}

VecBwdWorkspace vec_bwd_workspace(const Plan &p) {
  VecBwdWorkspace w{};
  const size_t tile = (size_t)p.ws.nc_max * p.geo.H * p.geo.P * p.geo.N * 4;
  w.rsum = align_up(p.ws.total_bytes);
  w.ge = w.rsum + align_up(tile);
  w.total = w.ge + align_up(tile);
  return w;
}

}  // namespace

extern "C" {

size_t ssd_chunk_scan_bwd_workspace_size(const ssd_dims *dims) {
  Plan p;
  if (make_vec_bwd_plan(dims, &p) != SSD_OK) return 0;
  return vec_bwd_workspace(p).total;
}

ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *init_state,
                              const int32_t *cu_seqlens, const void *dy, const float *dfinal,
                              void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                              float *dinit, const ssd_dims *dims, void *workspace,
                              size_t workspace_bytes, void *stream) {
  Plan p;
  ssd_status s = make_vec_bwd_plan(dims, &p);
  if (s != SSD_OK) return s;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, dy, dt, p)) != SSD_OK) return s;
  if ((s = check_pass_args(init_state, nullptr, p)) != SSD_OK) return s;
  if (!tok_ptr_ok(dx, p, 16) || !tok_ptr_ok(ddt, p, 4) || !tok_ptr_ok(dB, p, 16) ||
      !tok_ptr_ok(dC, p, 16))
    return SSD_ERR_INVALID_ARG;
  if (!dA || !aligned(dA, 4) || (dD && !aligned(dD, 4))) return SSD_ERR_INVALID_ARG;
  if ((dD != nullptr) != (D != nullptr)) return SSD_ERR_INVALID_ARG;
  if ((dfinal && !aligned(dfinal, 16)) || (dinit && !aligned(dinit, 16))) return SSD_ERR_INVALID_ARG;
  const VecBwdWorkspace vw = vec_bwd_workspace(p);
  if (!workspace || workspace_bytes < vw.total) return SSD_ERR_WORKSPACE;
  // (binds the packed batch's chunk table and directory in the workspace)
  if ((s = bind_workspace(&p, workspace, workspace_bytes)) != SSD_OK) return s;
  // outputs overlap no input and no other output
  const Sizes z = tensor_bytes(p);
  const ssd::Geometry &g = p.geo;
  const size_t bbc32 = (size_t)g.tokens * g.G * g.N * 4, bh = (size_t)g.H * 4;
  const void *ins[] = {x, dt, A, B, C, D, init_state, dy, dfinal, workspace};
  const size_t insz[] = {z.x, z.dt, bh, z.bc, z.bc, bh, z.state, z.x, z.state, vw.total};
  const void *outs[] = {dx, ddt, dA, dB, dC, dD, dinit};
  const size_t outsz[] = {z.x, z.dt, bh, bbc32, bbc32, bh, z.state};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return SSD_ERR_INVALID_ARG;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return SSD_ERR_INVALID_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the forward's chunk states again (the state entering every chunk)
  if ((s = run_cumsum(dt, A, cu_seqlens, p, workspace, st)) != SSD_OK) return s;
  if ((s = run_state(x, B, p, workspace, st)) != SSD_OK) return s;
  if ((s = run_pass(init_state, nullptr, p, workspace, st)) != SSD_OK) return s;
  hipError_t e = ssd::launch_fill_f32(dA, g.H, st);
  if (e == hipSuccess && dD) e = ssd::launch_fill_f32(dD, g.H, st);
  if (e == hipSuccess)
    e = ssd::launch_bwd_vec(x, A, B, C, D, dy, dfinal, ws_ptr<float>(workspace, p.ws.acum_offset),
                            ws_ptr<float>(workspace, p.ws.dtq_offset),
                            ws_ptr<void>(workspace, p.ws.hprev_offset),
                            ws_ptr<float>(workspace, vw.rsum), ws_ptr<float>(workspace, vw.ge),
                            p.bf16, g, dx, ddt, dA, dB, dC, dD, dinit, st);
  return hip_status(e);
}

size_t ssd_fused_bwd_workspace_size(const ssd_dims *dims) {
  Plan p;
  if (make_fused_plan(dims, &p) != SSD_OK || !bwd_supported(p)) return 0;
  return bwd_workspace(p).total;
}

ssd_status ssd_fused_bwd(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, const int32_t *cu_seqlens,
                         const void *chunk_states, size_t states_bytes, const void *dy,
                         const float *dfinal, void *dx, float *ddt, float *dA, float *dB,
                         float *dC, float *dD, float *dinit, const ssd_dims *dims, void *workspace,
                         size_t workspace_bytes, void *stream) {
  Plan p;
  ssd_status s = make_fused_plan(dims, &p);
  if (s != SSD_OK) return s;
  if (!bwd_supported(p)) return SSD_ERR_UNSUPPORTED;
  if ((s = check_cumsum_args(dt, A, cu_seqlens, p)) != SSD_OK) return s;
  if ((s = check_scan_args(x, B, C, D, dy, dt, p)) != SSD_OK) return s;
  if (!tok_ptr_ok(dx, p, 16) || !tok_ptr_ok(ddt, p, 4) || !tok_ptr_ok(dB, p, 16) ||
      !tok_ptr_ok(dC, p, 16))
    return SSD_ERR_INVALID_ARG;
  if (!dA || !aligned(dA, 4) || (dD && !aligned(dD, 4))) return SSD_ERR_INVALID_ARG;
  if ((dD != nullptr) != (D != nullptr)) return SSD_ERR_INVALID_ARG;
  if ((dfinal && !aligned(dfinal, 16)) || (dinit && !aligned(dinit, 16))) return SSD_ERR_INVALID_ARG;
  const size_t hb = chunk_states_bytes(p);
  const BwdWorkspace bw = bwd_workspace(p);
  if (!chunk_states || !aligned(chunk_states, 16)) return SSD_ERR_INVALID_ARG;
  if (states_bytes < hb) return SSD_ERR_WORKSPACE;
  if (!workspace || workspace_bytes < bw.total) return SSD_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SSD_ERR_INVALID_ARG;
  // outputs overlap no input and no other output
  const Sizes z = tensor_bytes(p);
  const ssd::Geometry &g = p.geo;
  const size_t bdt = z.dt, bbc32 = (size_t)g.tokens * g.G * g.N * 4, bh = (size_t)g.H * 4;
  const void *ins[] = {x, dt, A, B, C, D, chunk_states, dy, dfinal, workspace};
  const size_t insz[] = {z.x, bdt, bh, z.bc, z.bc, bh, hb, z.x, z.state, bw.total};
  const void *outs[] = {dx, ddt, dA, dB, dC, dD, dinit};
  const size_t outsz[] = {z.x, bdt, bh, bbc32, bbc32, bh, z.state};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 10; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return SSD_ERR_INVALID_ARG;
    for (int j = i + 1; j < 7; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return SSD_ERR_INVALID_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t *cu = g.packed ? cu_seqlens : nullptr;
  if (g.N == 256)
    return hip_status(split_bwd(p, bw, x, dt, A, B, C, D, cu, chunk_states, dy, dfinal, dx, ddt,
                                dA, dB, dC, dD, dinit, workspace, st));
  hipError_t e = ssd::launch_fill_f32(dA, g.H, st);
  if (e == hipSuccess && dD) e = ssd::launch_fill_f32(dD, g.H, st);
  if (e == hipSuccess)
    e = ssd::launch_bwd_reverse(dy, dt, A, C, dfinal, cu, g.L, g.tokens, (int)g.nrows, g.H, g.N,
                                g.G, workspace, dinit, bw.nseg, (int)bw.seglen,
                                ws_ptr<float>(workspace, bw.gseg), ws_ptr<float>(workspace, bw.aseg),
                                ws_ptr<float>(workspace, bw.gin), st);
  if (e == hipSuccess)
    e = ssd::launch_bwd_chunk(x, dt, A, B, C, D, dy, chunk_states, g.N, workspace, cu, g.L, g.tokens,
                              (int)g.nrows, chunks32(p), g.H, g.N, g.G, nullptr, dx, ddt, dA, dB,
                              dC, dD, st);
  return hip_status(e);
}

const char *ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported shape or chunk length";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int ssd_version(void) { return SSD_VERSION; }

}  // extern "C"
