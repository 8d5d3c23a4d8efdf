/*
 * libssd -- Mamba-2 SSD (structured state space duality) chunked-scan forward
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (per sequence s, head h, group g = floor(h*G/H)):
 *
 *   h_{-1} = init_state[s,h]                          (zeros if init_state == NULL)
 *   h_t    = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t B_t^T     (P x N state)
 *   y_t    = C_t h_t + D_h * x_t                      (D == NULL means D = 0)
 *   final_state[s,h] = h after the sequence's last token
 *
 * i.e. the selective state space recurrence with a scalar-identity transition
 * (page "State Space Duality and Mamba-2: Unifying Transformers and
 * Semiseparable Matrices", sections "Mathematical Foundations" and "The
 * Scalar-Identity Structural Constraint"), evaluated blockwise as on page
 * "Mamba-2 Architecture: State Space Duality Explained", section "2. The
 * Chunked SSD Algorithm": within a chunk of Q tokens the masked product
 * (C B^T o L) X, between chunks a hand-off of the P x N state.  The pages are
 * silent on the input discretisation and the skip term; the library takes the
 * Euler weight dt_t on B_t x_t and adds D_h x_t.  dt is taken as given
 * (already positive, no softplus inside).  Heads in one group share B and C
 * (same page, item 4 of the chunked algorithm).
 *
 * Layouts (row-major, contiguous, last index fastest).  T = batch * seqlen
 * tokens for a fixed-length batch, or the packed total for variable length:
 *   x          [T, H, P]   io dtype        y           [T, H, P] io dtype
 *   B, C       [T, G, N]   io dtype        dt          [T, H]    float
 *   A, D       [H]         float           init/final  [S, H, P, N] float
 * where S = batch (fixed length) or nseq (variable length).
 *
 * Memory and ownership.  Every pointer argument except `dims` and the layout
 * struct is device memory owned by the caller.  The library allocates
 * nothing and never synchronises: every entry point only enqueues kernels on
 * `stream` (a hipStream_t; NULL = the default stream) and returns.  Calls on
 * different streams are independent provided they use distinct workspaces.
 * Its one piece of global state is the fixed scratch array that
 * ssd_chunk_scan_fwd_noalloc uses as its workspace (see there).
 *
 * Alignment.  x, B, C, y, init_state, final_state: 16 bytes; dt, A, D: 4
 * bytes; workspace: 256 bytes.
 *
 * Errors.  Every entry point returns an ssd_status.  Arguments are validated
 * before any HIP call, so a rejected call touches no device state.  A failed
 * kernel launch returns SSD_ERR_HIP; faults inside kernels surface at the
 * caller's next synchronisation, as with any asynchronous HIP work.  Nothing
 * is printed and nothing is thrown.
 *
 * Aliasing.  y must not overlap x, B, C or dt.  final_state may be the same
 * pointer as init_state (the state is read before it is overwritten) but may
 * not otherwise overlap it.
 */
#ifndef LIBSSD_SSD_H_
#define LIBSSD_SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_VERSION 1

typedef enum {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, overlap, bad dims */
  SSD_ERR_UNSUPPORTED = 2, /* valid, but outside the compiled shapes (see below) */
  SSD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than ssd_workspace_size() */
  SSD_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} ssd_status;

/* Element type of x, B, C, y (and of the Hprev workspace buffer). */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef struct {
  int64_t batch;    /* fixed-length rows; must be 1 when nseq > 0 */
  int64_t seqlen;   /* tokens per row; when nseq > 0 the total packed token count T */
  int64_t nheads;   /* H */
  int64_t headdim;  /* P */
  int64_t dstate;   /* N */
  int64_t ngroups;  /* G; H not a multiple of G returns SSD_ERR_UNSUPPORTED */
  int64_t nseq;     /* 0: fixed-length batch; > 0: packed sequences given by cu_seqlens */
  int32_t io_dtype; /* an ssd_dtype */
  int32_t reserved; /* must be 0 */
} ssd_dims;

/* Supported shapes.
 *   chunk_len Q in {64, 128, 256}; nheads a multiple of ngroups; headdim and
 *   dstate multiples of 16, at most 256.
 *   SSD_BF16, headdim P in {64, 128, 192, 256} and dstate N in {64, 128,
 *             256}: every contraction on bf16 MFMA with fp32 accumulation; y
 *             rounded to nearest-even.  A head of P = 64 r runs as r kernel
 *             heads of 64 state rows (rows p of the state never interact),
 *             which share the head's dt, A and D.
 *   SSD_BF16, other shapes: chunk_state and chunk_scan on the fp32 vector
 *             ALU (bf16 widened exactly, fp32 arithmetic, chunk states and
 *             hprev in bf16, y rounded to nearest-even) -- correct, not fast.
 *   SSD_F32:  fp32 throughout, on the vector ALU.
 *   T, nseq and every sequence length below 2^31.
 * Anything else valid returns SSD_ERR_UNSUPPORTED. */

/* Byte offsets of the workspace buffers (all 256-byte aligned).  The
 * per-stage entry points below read and write these; tests read them to check
 * each stage.  H and P below are the kernel heads and rows: with bf16 and a
 * head dim of 64 r, H = r nheads and P = 64 (the same bytes as [nheads][64 r]).
 * nc_max chunks are laid out, numbered sequence-major:
 *   fixed length: nc_max = batch * ceil(seqlen / Q), chunk c = b * ceil(L/Q) + k
 *   packed:       nc_max = ceil(T / Q) + nseq (upper bound; the exact count is
 *                 written to the chunk directory), chunks restart at each
 *                 sequence start.
 *   acum   float [nc_max][H][Q]   inclusive cumulative sum of dt*A from the chunk
 *                                 start; positions past a partial chunk's end hold
 *                                 the chunk's last value
 *   dtq    float [nc_max][H][Q]   dt transposed to chunk-major, 0 past the end
 *   states io    [nc_max][H][P][N] chunk states S_c (decay-weighted sum of
 *                                 dt_l x_l B_l^T over the chunk, summed in fp32
 *                                 and rounded once to the io type)
 *   hprev  io    [nc_max][H][P][N] state entering each chunk
 *   chunk_table  int32 [nc_max][4] (sequence, first token, length, 0)   packed only
 *   chunk_dir    int32 [nseq + 2]  first chunk of each sequence, then the total,
 *                                  then an error word (nonzero: cu_seqlens was not
 *                                  non-decreasing from 0 to T)          packed only
 */
typedef struct {
  size_t total_bytes;
  int64_t nc_max;
  size_t acum_offset;
  size_t dtq_offset;
  size_t states_offset;
  size_t hprev_offset;
  size_t chunk_table_offset; /* 0 and unused for fixed-length batches */
  size_t chunk_dir_offset;   /* 0 and unused for fixed-length batches */
} ssd_workspace_layout;

/* Workspace bytes needed for these dims and chunk length; 0 if they are
 * invalid or unsupported.  Host-only, no HIP call. */
size_t ssd_workspace_size(const ssd_dims *dims, int chunk_len);

/* Fills *out with the workspace layout.  Host-only, no HIP call. */
ssd_status ssd_get_workspace_layout(const ssd_dims *dims, int chunk_len,
                                    ssd_workspace_layout *out);

/* The whole forward: chunk_cumsum, chunk_state, state_passing, chunk_scan, in
 * that order on `stream`.
 *   cu_seqlens: device int32 [nseq + 1] when dims->nseq > 0 (non-decreasing,
 *               cu_seqlens[0] = 0, cu_seqlens[nseq] = T), else NULL.  Values
 *               that break this never cause an out-of-bounds access: lengths
 *               are clamped and the error word of the chunk directory is set.
 *   D, init_state, final_state: may be NULL.
 * Returns after enqueueing. */
ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, int chunk_len,
                              const float *init_state, const int32_t *cu_seqlens, void *y,
                              float *final_state, const ssd_dims *dims, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ssd_chunk_scan_fwd without a workspace argument and without allocating, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * fixed array of SSD_NOALLOC_SCRATCH_BYTES in the global memory of every
 * device the library runs on, reserved for the life of the process; the call
 * uses the current device's (hipGetDevice), which must be the device of
 * `stream`.  Problems whose ssd_workspace_size(dims, chunk_len) exceeds it
 * return SSD_ERR_WORKSPACE (checked before any HIP call; e.g. B 4, L 2048,
 * H 24, P 64, N 128 at chunk 256 needs about 26 MB).  Every call on one
 * device shares that array: calls that overlap in time on one device (other
 * streams, other threads) race and give wrong results.  The array keeps the
 * last call's contents; nothing in it needs clearing, since every stage
 * writes what a later one reads.  Otherwise identical to ssd_chunk_scan_fwd
 * (arguments, layouts, aliasing, errors, results bit for bit).  The first
 * call on a device looks the array's device address up (hipGetSymbolAddress)
 * and keeps it; no call allocates.  Returns after enqueueing. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *B, const void *C, const float *D, int chunk_len,
                                      const float *init_state, const int32_t *cu_seqlens, void *y,
                                      float *final_state, const ssd_dims *dims, void *stream);

/* Stage 1 (chunk_cumsum): for packed batches first builds the chunk table and
 * directory from cu_seqlens; then writes acum and dtq.  The log-space
 * cumulative decay: the product of the scalar decays between tokens i and j
 * is exp(s_j - s_i), page "State Space Duality and Mamba-2 ...", section "The
 * Scalar-Identity Structural Constraint". */
ssd_status ssd_chunk_cumsum(const float *dt, const float *A, int chunk_len,
                            const int32_t *cu_seqlens, const ssd_dims *dims, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Stage 2 (chunk_state): states[c,h] = sum_l exp(acum_last - acum_l) dtq_l
 * x_l^T B_l over the chunk's tokens, the state each chunk would leave from a
 * zero start (page "Mamba-2 Architecture: State Space Duality Explained",
 * "2. The Chunked SSD Algorithm", item 2, with the decay weights the
 * recurrence implies), summed in fp32 and stored in the io precision.  Needs
 * stage 1's output in the same workspace. */
ssd_status ssd_chunk_state(const void *x, const void *B, int chunk_len, const ssd_dims *dims,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Stage 3 (state_passing): per sequence and head, in chunk order,
 * hprev[c] = h; h = exp(acum_last[c]) h + states[c], starting from
 * init_state (or 0); final_state = h at the sequence end (same page and item:
 * the scalar recurrence between chunk boundaries).  Needs stages 1-2. */
ssd_status ssd_state_passing(const float *init_state, float *final_state, int chunk_len,
                             const ssd_dims *dims, void *workspace, size_t workspace_bytes,
                             void *stream);

/* Stage 4 (chunk_scan): per chunk, y_l = sum_{s<=l} (C_l . B_s)
 * exp(acum_l - acum_s) dt_s x_s + exp(acum_l) C_l hprev^T + D x_l -- the
 * masked product (C B^T o L) X plus the state handed in (same page, item 1
 * and the inter-chunk hand-off).  Needs stages 1-3. */
ssd_status ssd_chunk_scan(const void *x, const void *B, const void *C, const float *D, void *y,
                          int chunk_len, const ssd_dims *dims, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Single-token recurrent step, for decoding: one new token per sequence, the
 * state updated in place (page "State Space Duality and Mamba-2: Unifying
 * Transformers and Semiseparable Matrices", section "The Dual Perspectives of
 * Semiseparable Multiplication", item 1, the recurrent mode with a constant
 * state per head; page "Mamba-2 Architecture: State Space Duality
 * Explained", "Step 3: Autoregressive Token Generation without KV Cache"):
 *   state[s,h] <- exp(dt[s,h] A_h) state[s,h] + dt[s,h] x[s,h] B[s,g]^T
 *   y[s,h]      = C[s,g] state[s,h] + D_h x[s,h]
 * i.e. the recurrence at the top of this file for one token.  Calling it for
 * tokens t0, t1, ... continues ssd_chunk_scan_fwd from its final_state: the
 * results agree with one forward over all the tokens up to rounding.
 *   dims: batch = S sequences, seqlen = 1, nseq = 0, other fields as above.
 *   x [S, H, P] io, dt [S, H] float, B and C [S, G, N] io, D [H] float or
 *   NULL, state [S, H, P, N] float (read, then overwritten), y [S, H, P] io.
 * Supported: dstate N in {16, 32, 64, 128, 256}; any headdim P >= 1; both io
 * dtypes; fp32 arithmetic, y rounded to nearest-even for bf16.  Alignment as
 * above; state must not overlap any other argument, y none of the inputs.
 * One pass over the state: it is bound by 2 * S*H*P*N*4 bytes of HBM traffic.
 * Returns after enqueueing. */
ssd_status ssd_step(const void *x, const float *dt, const float *A, const void *B, const void *C,
                    const float *D, float *state, void *y, const ssd_dims *dims, void *stream);

/* The core's neighbours in the Mamba-2 block (page "Mamba-2 Architecture:
 * State Space Duality Explained", "Step 2: Full Mamba-2 Block with Gated
 * Projections").  Both are HBM-bound and take T token rows; the sequences are
 * `batch` rows of `seqlen` tokens (cu_seqlens NULL, nseq 0, T = batch *
 * seqlen) or nseq packed sequences given by the device int32 cu_seqlens
 * [nseq + 1] (batch 1, T = seqlen), as for ssd_chunk_scan_fwd.
 *
 * ssd_conv1d_silu: the causal depthwise convolution over the token axis that
 * precedes the core (width K, left padding K - 1, outputs truncated to the
 * sequence), then SiLU:
 *   out[t, c] = silu(bias[c] + sum_{k<K} weight[c * K + k] * in[t - (K-1) + k, c])
 * where positions before the first token of t's sequence read zero, and
 * silu(v) = v / (1 + exp(-v)).
 *   in:  T rows of in_stride elements; channels 0 .. channels-1 of each row are
 *        read, so one slice (x, B or C) of a packed projection can be read in
 *        place by offsetting the pointer.  out: T rows of out_stride elements.
 *   weight [channels][K] float; bias [channels] float or NULL; 1 <= K <= 4.
 *   channels, in_stride and out_stride multiples of 8 (bf16) / 4 (fp32)
 *   elements; in and out 16-byte aligned; out must not overlap in.
 *   Malformed cu_seqlens never cause an out-of-bounds access (as above).
 *
 * ssd_gate_rmsnorm: the gate and normalisation after the core:
 *   g = y * silu(z);  out = weight ? g / sqrt(mean over the row of g^2 + eps) * weight : g
 * per token row of `width` channels (H * P for the core's output).
 *   y, z, out [T, width] io dtype, 16-byte aligned; out may be y or z itself
 *   but must not otherwise overlap them; weight [width] float or NULL;
 *   width a multiple of 8 (bf16) / 4 (fp32); eps >= 0.
 * fp32 arithmetic, bf16 results rounded to nearest-even.  Return after
 * enqueueing. */
ssd_status ssd_conv1d_silu(const void *in, int64_t in_stride, const float *weight,
                           const float *bias, int kernel_width, void *out, int64_t out_stride,
                           int64_t batch, int64_t seqlen, int64_t nseq, const int32_t *cu_seqlens,
                           int64_t channels, int32_t io_dtype, void *stream);
ssd_status ssd_gate_rmsnorm(const void *y, const void *z, const float *weight, float eps, void *out,
                            int64_t tokens, int64_t width, int32_t io_dtype, void *stream);

/* The same forward in one pass per (sequence, head), the P x N state kept on
 * chip across chunks, so that only x, B, C, dt and y cross HBM (no workspace,
 * no chunk_len: it walks chunks of 32 tokens, and chunking is exact).  The
 * arguments, layouts, aliasing rules and results are those of
 * ssd_chunk_scan_fwd, to rounding.
 * Supported: SSD_BF16, headdim P in {64, 128, 192, 256} (a head of 64 r
 * rows runs as r kernel heads sharing dt, A, D), dstate N in {64, 128, 256},
 * nheads a multiple of ngroups; else SSD_ERR_UNSUPPORTED.  It keeps one block
 * per (sequence, kernel head), or per 2 or 3 heads of a group, busy for the
 * sequence's whole length, so it pays off when sequences x heads fills the
 * GPU (hundreds or more); a single long sequence is better served by the
 * chunk-parallel ssd_chunk_scan_fwd.  Returns after enqueueing. */
ssd_status ssd_fused_fwd(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, const float *init_state,
                         const int32_t *cu_seqlens, void *y, float *final_state,
                         const ssd_dims *dims, void *stream);

/* ssd_fused_fwd that also saves, for the backward pass, the state entering
 * every 64-token pair of chunks (the inter-chunk states of page "Mamba-2
 * Architecture: State Space Duality Explained", "2. The Chunked SSD
 * Algorithm", item 3, kept at every other 32-token chunk), rounded to bf16:
 *   chunk_states  device bf16 [npairs][H][P][N], 16-byte aligned, not
 *                 overlapping any other argument; pair b = the sequence-major
 *                 index of the 64-token pair (sequence s's pairs start at the
 *                 sum of ceil(len_i / 64) over i < s), holding the state
 *                 before the pair's first token; NULL: nothing saved (then
 *                 this is ssd_fused_fwd);
 *   states_bytes  its size, at least ssd_fused_states_size(dims), else
 *                 SSD_ERR_WORKSPACE.
 * Everything else as ssd_fused_fwd.  Returns after enqueueing. */
ssd_status ssd_fused_fwd_train(const void *x, const float *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *init_state,
                               const int32_t *cu_seqlens, void *y, float *final_state,
                               void *chunk_states, size_t states_bytes, const ssd_dims *dims,
                               void *stream);

/* The one-pass forward for few, long fixed-length sequences, where one block
 * per (sequence, head) leaves the GPU idle: each sequence is cut into
 * segments of seg_len tokens and the chunked algorithm of page "Mamba-2
 * Architecture: State Space Duality Explained", "2. The Chunked SSD
 * Algorithm", is applied one level up (blockwise evaluation, glossary page
 * "State Space Duality", "Why it is useful"), with the one-pass kernel as the
 * per-segment step:
 *   1. every segment but the last, from a zero state: its end state and total
 *      decay (a state-only pass: x, B and dt are read, nothing is written but
 *      the workspace);
 *   2. the hand-off h_{j+1} = exp(sum of dt A over segment j) h_j + S_j from
 *      init_state (or 0), giving the state entering every segment;
 *   3. every segment from its entering state: y, and final_state from the
 *      last one.
 * Arguments, layouts and results are ssd_fused_fwd's (cu_seqlens absent:
 * fixed-length batches only, nseq > 0 returns SSD_ERR_UNSUPPORTED), to
 * rounding; final_state may alias init_state.
 *   seg_len    tokens per segment, a positive multiple of 32, else
 *              SSD_ERR_INVALID_ARG; seg_len >= seqlen runs ssd_fused_fwd
 *              (no workspace needed).
 *   workspace  device memory of at least ssd_fused_split_workspace_size(dims,
 *              seg_len) bytes (else SSD_ERR_WORKSPACE), 256-byte aligned,
 *              overlapping no argument: fp32 [batch][nseg][H][P][N] states
 *              entering the segments, then fp32 [batch][nseg-1][H] segment
 *              decays (log2), nseg = ceil(seqlen / seg_len).
 * Supported shapes are ssd_fused_fwd's.  Returns after enqueueing. */
ssd_status ssd_fused_fwd_split(const void *x, const float *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *init_state, void *y,
                               float *final_state, int64_t seg_len, const ssd_dims *dims,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ssd_fused_fwd_split that also saves the state entering every 64-token pair
 * of chunks for the backward pass (ssd_fused_bwd), like ssd_fused_fwd_train:
 * step 3 stores, at the top of every other 32-token chunk of each segment,
 * its state rounded to bf16 (the state entering a segment is the one step 2
 * handed it, so the saved states differ from ssd_fused_fwd_train's by
 * rounding only).
 *   chunk_states  device, [npairs][H][P][N] bf16, ssd_fused_fwd_train's
 *                 layout, 16-byte aligned, overlapping no other argument;
 *                 NULL returns SSD_ERR_INVALID_ARG;
 *   states_bytes  its size, at least ssd_fused_states_size(dims), else
 *                 SSD_ERR_WORKSPACE;
 *   seg_len       a positive multiple of 64 (a segment starts a pair), else
 *                 SSD_ERR_INVALID_ARG.
 * Everything else as ssd_fused_fwd_split.  Returns after enqueueing. */
ssd_status ssd_fused_fwd_split_train(const void *x, const float *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const float *init_state, void *y, float *final_state,
                                     void *chunk_states, size_t states_bytes, int64_t seg_len,
                                     const ssd_dims *dims, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Workspace bytes of ssd_fused_fwd_split for these dims and seg_len (0 when
 * seg_len >= seqlen, or when the arguments are invalid).  Host-only. */
size_t ssd_fused_split_workspace_size(const ssd_dims *dims, int64_t seg_len);

/* A segment length for ssd_fused_fwd_split on the current device: seqlen
 * rounded up to 32 (no split) when sequences x heads already give two blocks
 * per compute unit, else the power of two (at least 512) that gives about 8
 * (segment, head) rows per compute unit; 0 outside ssd_fused_fwd's shapes or
 * for packed sequences.  Host-only (queries the device's compute units). */
int64_t ssd_fused_split_seg_len(const ssd_dims *dims);

/* Bytes of ssd_fused_fwd_train's chunk_states for these dims (npairs =
 * batch * ceil(seqlen / 64), or ceil(T / 64) + nseq for packed sequences);
 * 0 if the dims are invalid or outside ssd_fused_fwd's shapes.  Host-only. */
size_t ssd_fused_states_size(const ssd_dims *dims);

/* Gradients of ssd_chunk_scan_fwd for every shape it takes (fp32 or bf16,
 * head dims and state sizes multiples of 16 up to 256, fixed-length or packed
 * batches): the chain rule through the recurrence (as ssd_fused_bwd below),
 * evaluated blockwise in 64-token chunks on the fp32 vector ALU, with no
 * saved states: it first runs the forward's chunk_cumsum, chunk_state and
 * state_passing again into the workspace (the state entering every chunk),
 * then the reverse hand-off of the state gradient from d(final_state) (the
 * sums of exp(a_l) dy_l C_l^T per chunk), then every gradient per (chunk,
 * group).  The general path: correct, not tuned; ssd_fused_bwd is the fast
 * one where its shapes apply.
 *   x, dt, A, B, C, D, init_state, cu_seqlens, dims: as for the forward;
 *   dy   upstream gradient of y, like y;  dfinal: of final_state, fp32
 *        [rows, H, P, N] 16-byte aligned, or NULL (zero);
 *   dx   like x (io dtype);  ddt float [T, H];  dB, dC float [T, G, N]
 *        (summed over the heads of a group);  dA float [H];  dD float [H],
 *        NULL exactly when D is NULL;  dinit float [rows, H, P, N] or NULL.
 * workspace: device memory of at least ssd_chunk_scan_bwd_workspace_size(dims)
 * bytes (else SSD_ERR_WORKSPACE), 256-byte aligned.  Outputs overlap no input
 * and no other output (else SSD_ERR_INVALID_ARG).  On `stream`: dA and dD are
 * cleared and then added to with float atomics per (chunk, head), so they sum
 * in an unspecified order; every other output is written once.  Returns after
 * enqueueing. */
ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *init_state,
                              const int32_t *cu_seqlens, const void *dy, const float *dfinal,
                              void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                              float *dinit, const ssd_dims *dims, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes of ssd_chunk_scan_bwd (0 if the dims are invalid or
 * unsupported).  Host-only. */
size_t ssd_chunk_scan_bwd_workspace_size(const ssd_dims *dims);

/* Workspace bytes of ssd_fused_bwd: the gradient w.r.t. the state leaving
 * every 64-token pair (bf16, laid out like chunk_states) and, when the sweep
 * is split into segments (sequences x nheads / 2 < 256), two fp32 P x N tiles
 * and a decay per segment and head.  At N = 256 those of N = 128 (each half
 * of the state's columns runs in turn), then one half's B and C (bf16),
 * dfinal, dB, dC and dinit (fp32) and ddt.  Host-only. */
size_t ssd_fused_bwd_workspace_size(const ssd_dims *dims);

/* Gradients of the forward.  The pages give the recurrence h_t = exp(dt_t A)
 * h_{t-1} + dt_t x_t B_t^T, y_t = h_t C_t + D x_t (page "State Space Duality
 * and Mamba-2: Unifying Transformers and Semiseparable Matrices", section
 * "Mathematical Foundations", with the scalar-identity decay of "The
 * Scalar-Identity Structural Constraint"), but no backward pass; this is the
 * chain rule applied to it, for the scalar loss
 *   sum_t <dy_t, y_t> + sum_{s,h} <dfinal[s,h], final_state[s,h]>.
 * Inputs (the forward's, same layouts): x, dt, A, B, C, D (may be NULL),
 * cu_seqlens, and
 *   chunk_states  what ssd_fused_fwd_train saved for these inputs and
 *                 init_state (states_bytes its size); equally the hprev
 *                 buffer of an ssd_chunk_scan_fwd workspace for the same
 *                 inputs with chunk_len 64 (bf16), which holds the same states
 *                 in the same layout: the chunk-parallel forward for a few long
 *                 sequences;
 *   dy            device bf16 [T, H, P], the gradient w.r.t. y;
 *   dfinal        device float [rows, H, P, N] or NULL (zero).
 * Outputs (device, overwritten; none may overlap an input or another output):
 *   dx   bf16  [T, H, P]    16-byte aligned
 *   ddt  float [T, H]
 *   dA   float [H]
 *   dB   float [T, G, N]    summed over the heads of each group, 16-byte aligned
 *   dC   float [T, G, N]    likewise
 *   dD   float [H], NULL exactly when D is NULL
 *   dinit float [rows, H, P, N] (the gradient w.r.t. init_state) or NULL.
 * workspace: device memory of at least ssd_fused_bwd_workspace_size(dims)
 * bytes, 16-byte aligned, else SSD_ERR_WORKSPACE.  Supported: SSD_BF16,
 * headdim 64, dstate N in {64, 128, 256}, an even number of heads per group;
 * else SSD_ERR_UNSUPPORTED (and ssd_fused_bwd_workspace_size returns 0).  On
 * `stream`: dA and dD cleared; the reverse sweep of the
 * state gradient (one pass per (sequence, two heads), or, with fewer such
 * pairs than 256, per segment: segment sums, a chained pass, the segments
 * again; segments of the longest power of two from 256 tokens that still
 * gives 1024 (segment, head pair) blocks); the per-chunk gradients, which add
 * into dA and dD with float atomics, so those two sum in an unspecified order.  N = 256 runs
 * these steps once per half of the state's columns (the columns never mix in
 * the recurrence): each half's B, C, saved states and dfinal are copied into
 * the workspace, its dB, dC and dinit copied back into their columns; the
 * second half adds its dx into the first's (read back as bf16) before its one
 * rounding, and its ddt is added to the first's.  Returns after enqueueing. */
ssd_status ssd_fused_bwd(const void *x, const float *dt, const float *A, const void *B,
                         const void *C, const float *D, const int32_t *cu_seqlens,
                         const void *chunk_states, size_t states_bytes, const void *dy,
                         const float *dfinal, void *dx, float *ddt, float *dA, float *dB,
                         float *dC, float *dD, float *dinit, const ssd_dims *dims, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *ssd_status_string(ssd_status status);

/* SSD_VERSION of the built library. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H_ */
