// Host-side launchers of the libssd kernels (internal; the public ABI is ssd.h).
// Every launcher only enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

struct Geometry {
  int64_t tokens;   // T
  int64_t L;        // tokens per row (fixed length)
  int32_t nc_row;   // chunks per row (fixed length)
  int32_t Q;        // chunk length
  int64_t nc_max;   // chunks laid out in the workspace
  int64_t nrows;    // sequences: batch (fixed) or nseq (packed)
  int32_t H, P, N, G;   // kernel heads and head dim (see hr)
  // Heads split: with bf16 io and a head dim of 64 hr, each head's P x N state
  // runs as hr kernel heads of 64 rows (rows p of the state never interact, and
  // x, y, the states and the workspace have the same memory layout either
  // way); kernel head h takes dt, A and D of head h / hr.  1 otherwise.
  int32_t hr;
  bool packed;
  const int32_t *table;  // packed: chunk table in the workspace
  const int32_t *dir;    // packed: chunk directory in the workspace
};

hipError_t launch_chunk_table(const int32_t *cu_seqlens, const Geometry &geo, int32_t *table,
                              int32_t *dir, hipStream_t stream);
hipError_t launch_chunk_cumsum(const float *dt, const float *A, const Geometry &geo, float *acum,
                               float *dtq, hipStream_t stream);
// states and hprev are bf16 when bf16 is set, else fp32
hipError_t launch_state_passing(const void *states, void *hprev, bool bf16,
                                const float *acum, const float *init, float *final_state,
                                const Geometry &geo, hipStream_t stream);
// bf16 io, MFMA contractions
bool chunk_state_bf16_supported(int P, int N, int Q);
hipError_t launch_chunk_state_bf16(const void *x, const void *B, const float *acum,
                                   const float *dtq, void *states, const Geometry &geo,
                                   hipStream_t stream);
bool chunk_scan_bf16_supported(int P, int N, int Q);
// D is indexed by kernel head / geo.hr
hipError_t launch_chunk_scan_bf16(const void *x, const void *B, const void *C, const float *D,
                                  const float *acum, const float *dtq, const void *hprev, void *y,
                                  const Geometry &geo, hipStream_t stream);
// fp32 vector-ALU contractions, for fp32 io and for the bf16 shapes the MFMA
// kernels do not take (states / hprev in the io precision)
hipError_t launch_chunk_state_vec(const void *x, const void *B, const float *acum,
                                  const float *dtq, void *states, bool bf16, const Geometry &geo,
                                  hipStream_t stream);
hipError_t launch_chunk_scan_vec(const void *x, const void *B, const void *C, const float *D,
                                 const float *acum, const float *dtq, const void *hprev, void *y,
                                 bool bf16, const Geometry &geo, hipStream_t stream);

// single-token recurrent step (decode)
bool step_supported(int N);
hipError_t launch_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
                       const float *D, float *state, void *y, bool bf16, int64_t S, int H, int P,
                       int N, int G, hipStream_t stream);

// the core's block neighbours: causal depthwise conv1d + SiLU, SiLU gate + RMS norm
hipError_t launch_conv1d_silu(const void *in, int64_t in_stride, const float *weight,
                              const float *bias, int K, void *out, int64_t out_stride, int64_t T,
                              int64_t seqlen, int nseq, const int32_t *cu_seqlens,
                              int64_t channels, bool bf16, hipStream_t stream);
hipError_t launch_gate_rmsnorm(const void *y, const void *z, const float *weight, float eps,
                               void *out, int64_t tokens, int width, bool bf16, hipStream_t stream);

// the whole forward in one pass per (sequence, head); H kernel heads of P rows,
// dt, A and D of kernel head h at h / hr
bool fused_supported(int H, int P, int N, int G);
hipError_t launch_fused(const void *x, const float *dt, const float *A, const void *B, const void *C,
                        const float *D, const float *h0, const int32_t *cu, int64_t L, int64_t T,
                        int rows, int H, int P, int N, int G, int hr, void *y, float *hfin,
                        void *hsave, hipStream_t stream);
// the one-pass forward over segments of S tokens (S a multiple of 32) of nseq
// fixed-length sequences: a state-only pass over every segment but the last
// (end state from zero into sseg [nseq][j + 1] of a [nseq][nseg][H][P][N]
// buffer, total log2 decay into lseg [nseq][nseg-1][H]), a hand-off pass
// turning sseg into the states entering every segment, then the forward of
// every segment from its entering state (h0 read only by the hand-off); with
// hsave (S a multiple of 64) the last pass also saves the state entering
// every 64-token pair, in ssd_fused_fwd_train's layout
hipError_t launch_fused_split(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *h0, int64_t L,
                              int nseq, int64_t S, int H, int P, int N, int G, int hr, void *y,
                              float *hfin, float *sseg, float *lseg, void *hsave,
                              hipStream_t stream);
// backward of the one-pass forward (bf16, P == 64, N in {64, 128}, even heads per group)
// nseg > 0: the sweep split into that many segments of seg_len tokens (a
// multiple of 32; gseg, gin [nseg][H][P][N] and aseg [nseg][H] fp32 scratch);
// 0: one pass per sequence
hipError_t launch_bwd_reverse(const void *dy, const float *dt, const float *A, const void *C,
                              const float *dfinal, const int32_t *cu, int64_t L, int64_t T,
                              int rows, int H, int N, int G, void *gsave, float *dinit,
                              int64_t nseg, int seg_len, float *gseg, float *aseg, float *gin,
                              hipStream_t stream);
// hsave: the saved states, rows of hsld >= N elements (N, or 2N when hsave
// points into one half of the columns of N = 256 states)
hipError_t launch_bwd_chunk(const void *x, const float *dt, const float *A, const void *B,
                            const void *C, const float *D, const void *dy, const void *hsave,
                            int hsld, const void *gsave, const int32_t *cu, int64_t L, int64_t T,
                            int rows, int64_t nchunks, int H, int N, int G, const void *dxacc,
                            void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                            hipStream_t stream);
hipError_t launch_fill_f32(float *p, int64_t n, hipStream_t stream);
// rows x units 16-byte pieces between row-major layouts (byte row strides)
hipError_t launch_copy2d16(const void *src, int64_t src_ld, void *dst, int64_t dst_ld,
                           int64_t rows, int units, hipStream_t stream);
// acc += add elementwise: bf16 (n a multiple of 8, 16-byte aligned) and fp32
hipError_t launch_add_f32(float *acc, const float *add, int64_t n, hipStream_t stream);

// the general backward on the vector ALU, from the forward's workspace at chunk
// length bwd_vec_chunk_len() (acum, dtq, hprev in the io precision): the dy C^T
// sums per chunk into R, the state gradient entering every chunk from the
// right into GE (fp32 [nc][H][P][N] each) and d(init_state), then every
// gradient per (chunk, group); dA and dD must be zeroed before
int bwd_vec_chunk_len();
hipError_t launch_bwd_vec(const void *x, const float *A, const void *B, const void *C,
                          const float *D, const void *dy, const float *dfinal, const float *acum,
                          const float *dtq, const void *hprev, float *R, float *GE, bool bf16,
                          const Geometry &geo, void *dx, float *ddt, float *dA, float *dB,
                          float *dC, float *dD, float *dinit, hipStream_t stream);

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

// Heads per block of a head-batched kernel (one block per CU at a time): a
// launch takes ceil(blocks / slots) rounds of (hb heads + a prologue worth
// `prologue` heads' time); pick the run length with the fewest head-times,
// then even out the runs of a group.  Returns hb; nkb = runs per group.
inline int pick_heads_per_block(int64_t nc, int H, int G, int slots, double prologue, int &nkb) {
  const int HG = H / G;
  int best = HG;
  double best_cost = 1e300;
  for (int hb = 1; hb <= HG; ++hb) {
    const int64_t blocks = nc * G * ((HG + hb - 1) / hb);
    const double cost = (double)((blocks + slots - 1) / slots) * (hb + prologue);
    if (cost < best_cost) {
      best_cost = cost;
      best = hb;
    }
  }
  nkb = (HG + best - 1) / best;
  return (HG + nkb - 1) / nkb;
}

}  // namespace ssd
