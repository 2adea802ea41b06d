/*
 * ssd.h -- C ABI of libssd: the Mamba-2 chunked SSD forward pass on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b and head h, with group g = h / (nheads /
 * ngroups), a P x N state s (P = headdim, N = dstate) is carried across the
 * sequence:
 *
 *     s_t = exp(dt_t * A_h) * s_{t-1} + dt_t * x_t (outer) B_t        (P x N)
 *     y_t = s_t C_t + D_h * x_t                                       (length P)
 *
 * The output line is the recurrence y_t = c_t^T h_t + D x_t given in devin.kr
 * "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section "Mamba-2
 * 아키텍처의 핵심 연산" (core operations); the decay a_t = dt_t A_h and its
 * running sum G named there drive the state update, which is the standard
 * discretised Mamba-2 update written above.  The library evaluates it chunk by
 * chunk in three stages, the decomposition described in the same page's
 * section "세 가지 핵심 커널 구현" (three kernels) and in brifing.si
 * "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
 * CUDA Tile", sections 4-9:
 *   1. chunk_cumsum   -- within-chunk running sum of a_t, scaled by log2(e);
 *   2. chunk_state    -- every chunk's own state contribution by the jump
 *                        formula;
 *      state_pass     -- the sequential pass of states across chunks;
 *   3. compute_out    -- causal-masked decayed interaction tile, carried-state
 *                        term and D skip fused, nothing chunk x chunk in HBM.
 * Two builds of these stages exist.  The fused kernel (bf16 io, headdim 64,
 * dstate 128, chunk_size 256, an even number of heads per group) runs all
 * stages per (chunk, head pair) in one pass over x, handing each chunk's
 * state to the next chunk's workgroup through device memory.  The staged
 * kernels (every supported shape) run them as four kernels with the running
 * sums and chunk-start states in the workspace.  ssd_fwd takes the staged
 * kernels, which measure faster on MI355X; ssd_config.fused = 1 selects the
 * fused one and ssd_tune times both.
 * The result equals the token recurrence up to floating-point rounding.
 * ssd_step runs the same recurrence token by token from a resident state
 * (decode).
 *
 * Layouts.  Every tensor is dense, row-major, with no padding:
 *     x, y                [batch, seqlen, nheads, headdim]  io dtype
 *     B, C                [batch, seqlen, ngroups, dstate]  io dtype
 *     dt                  [batch, seqlen, nheads]           fp32, > 0 (used as given;
 *                                                            the _ex entry points and
 *                                                            ssd_step can prepare a raw
 *                                                            one: ssd_dt_transform)
 *     A, D                [nheads]                          fp32
 *     init_state, final_state [batch, nheads, headdim, dstate] fp32
 * io dtype is SSD_BF16 (bf16 operands, fp32 accumulation) or SSD_F32.
 *
 * Ownership and ordering.  Every tensor pointer is DEVICE memory owned by the
 * caller.  The library allocates nothing, frees nothing, never synchronises
 * and keeps no pointer after a call returns (ssd_tune, a measurement tool,
 * is the one exception: it creates HIP events and synchronises).  Work is
 * enqueued on `stream`
 * (a hipStream_t; NULL = the default stream) and its results are valid once
 * the caller has synchronised with that stream; inputs must stay unchanged
 * until then.  y must not overlap any input.  final_state may be the same
 * buffer as init_state (each state tile is read before it is written).
 * Calls are reentrant; the only global state is a thread-local error message
 * and, per kernel, a record of the devices on which its dynamic-LDS limit has
 * been raised (set once, thread-safely).  The forward path can be captured
 * into a HIP graph: it enqueues kernels only.
 *
 * Preconditions that are documented, not checked: dt > 0, A <= 0 (A = 0 is
 * allowed and gives causal linear attention), all inputs finite.
 *
 * Errors.  Every entry point validates on the host before any HIP call and
 * returns the first failing check in this order: SSD_ERR_NULL_POINTER (a
 * required pointer is NULL), SSD_ERR_BAD_SHAPE (a size <= 0, nheads not a
 * multiple of ngroups, or a size product overflowing int64), SSD_ERR_BAD_CHUNK
 * (chunk_size not one of 16, 32, 64, 128, 256; ssd_step does not use it),
 * SSD_ERR_BAD_DTYPE, SSD_ERR_BAD_VALUE (an invalid ssd_dt_transform or
 * ssd_config),
 * SSD_ERR_MISALIGNED (a tensor pointer not 16-byte aligned),
 * SSD_ERR_UNSUPPORTED (headdim or dstate not a multiple of 16, or dstate >
 * 256), SSD_ERR_WORKSPACE (workspace too small).  SSD_ERR_HIP reports a failed
 * kernel launch.  Nothing is enqueued when a call returns an error.  No C++
 * exception crosses this interface.  ssd_last_error_message() describes the
 * last error of the calling thread.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 6

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL_POINTER = 1,
  SSD_ERR_BAD_SHAPE = 2,
  SSD_ERR_BAD_CHUNK = 3,
  SSD_ERR_BAD_DTYPE = 4,
  SSD_ERR_MISALIGNED = 5,
  SSD_ERR_WORKSPACE = 6,
  SSD_ERR_UNSUPPORTED = 7,
  SSD_ERR_HIP = 8,
  SSD_ERR_INTERNAL = 9,
  SSD_ERR_BAD_VALUE = 10
} ssd_status;

/* Problem description.  chunk_size Q splits the sequence into
 * T = ceil(seqlen / Q) chunks; a partial last chunk is allowed.  The chunk
 * size does not change y, the final state or any gradient (the chunked
 * evaluation equals the recurrence for every chunk size, up to rounding),
 * and the matrix-core kernels step through tokens 32 at a time, so the
 * entry points that return only those (ssd_fwd*, ssd_fwd_noalloc, ssd_tune,
 * ssd_bwd) run chunk_size 16 as 32.  ssd_chunk_cumsum restarts its sums
 * every 16 tokens for it; ssd_fwd_states and ssd_compute_out, whose
 * workspace holds per-chunk states, return SSD_ERR_UNSUPPORTED for it. */
typedef struct {
  int64_t batch;
  int64_t seqlen;
  int64_t nheads;
  int64_t headdim;    /* P */
  int64_t dstate;     /* N */
  int64_t ngroups;    /* G */
  int64_t chunk_size; /* Q */
  int32_t io_dtype;   /* ssd_dtype: dtype of x, B, C, y and of the chunk states */
  int32_t reserved;   /* must be 0 */
} ssd_problem;

/* Optional preparation of a raw step size, for the entry points that take
 * one (NULL there = dt is used as given).  A Mamba-2 layer produces its step
 * size from a projection as softplus(dt_raw + dt_bias), optionally clamped;
 * the pages leave this preparation out, and the library applies it where dt is
 * first read (stage 1, or the decode step), so no prepared copy of dt is ever
 * written or read back:
 *     v  = dt[b, t, h] + (dt_bias ? dt_bias[h] : 0)
 *     v  = softplus ? log(1 + exp(v)) : v
 *     dt' = min(max(v, dt_min), dt_max)
 * Every later use of dt (decays, input weights) uses dt'.  dt' must satisfy
 * the positivity precondition; dt_min = 0 and dt_max = INFINITY leave a
 * positive value unclamped.
 * Errors (SSD_ERR_BAD_VALUE): softplus not 0 or 1, reserved not 0, dt_min or
 * dt_max NaN, dt_min > dt_max.  dt_bias, when given, is [nheads] fp32 device
 * memory, 16-byte aligned (else SSD_ERR_MISALIGNED). */
typedef struct {
  const float* dt_bias; /* [nheads] fp32 device, or NULL */
  int32_t softplus;     /* 1: apply softplus after the bias; 0: do not */
  int32_t reserved;     /* must be 0 */
  float dt_min;         /* lower clamp */
  float dt_max;         /* upper clamp */
} ssd_dt_transform;

/* Tile choices of the forward pass's kernels, for shape tuning.  The pages
 * tune block sizes and occupancy per shape; here the alternatives are ones
 * the library compiles, chosen per problem at run time:
 *   fused        : 1 = the single-pass fused kernel (built for bf16 io,
 *                  headdim 64, dstate 128, chunk_size 256 and an even number
 *                  of heads per group), 0 = the staged kernels; the four
 *                  fields below are checked in both cases and used by the
 *                  staged kernels only;
 *   cumsum_heads : 0 = the running sums G and the prepared step sizes are
 *                  formed inside the chunk_state kernel (no launch of their
 *                  own); 4 or 16 = a separate chunk_cumsum launch with that
 *                  many heads per workgroup (the values are bitwise the same
 *                  either way);
 *   state_heads  : heads per chunk_state workgroup (they share the chunk's B
 *                  rows), 1, 2 or 4, dividing the heads of a group;
 *   out_heads    : heads per compute_out workgroup (they share the raw tile
 *                  C B^T), 1, or 2 for bf16 io, dstate <= 128 and an even
 *                  number of heads per group (two heads' accumulators do not
 *                  fit the registers otherwise);
 *   out_resident : 1 = stage 3 as one workgroup per (batch, chunk, run of
 *                  heads of one group) that builds the raw tile C B^T once,
 *                  keeps it in registers and streams only each head's x,
 *                  state and running sums (built for bf16 io, headdim 64,
 *                  dstate <= 128, chunk_size 256 and nheads * headdim <=
 *                  2^22; out_heads is then unused but still checked);
 *                  0 = the head-pair kernel above.  Both give bitwise the
 *                  same y.
 * Every choice computes the same result up to floating-point summation order.
 * ssd_default_config gives the static table the plain entry points use;
 * ssd_tune measures the alternatives. */
typedef struct {
  int32_t cumsum_heads;
  int32_t state_heads;
  int32_t out_heads;
  int32_t fused;        /* 0 or 1 */
  int32_t out_resident; /* 0 or 1 */
} ssd_config;

/* ABI version of the loaded library (SSD_ABI_VERSION at build time). */
int ssd_abi_version(void);

/* Static text for a status code ("unknown status" for other values). */
const char* ssd_status_string(int status);

/* Description of the last error returned on the calling thread ("" if none).
 * The pointer stays valid until the thread's next libssd call. */
const char* ssd_last_error_message(void);

/* Workspace bytes enough for every forward entry point and configuration on
 * `prob`: the larger of the two layouts below.  Every forward workspace
 * starts with a 256-byte header: the status word of ssd_fwd_status and the
 * tag of the latest call.  The staged kernels then use two fp32 [batch,
 * nheads, T*Q] arrays (the base-2 running sums G and dt in [batch, head,
 * token] order) and the chunk-start states [batch, nheads, T, headdim,
 * dstate] in the io dtype (in an internal fragment order, padded to whole
 * 64-row and 32-column tiles); the fused kernel uses one 8-byte flag per
 * (batch, head, 32 x 32 state tile) and, when final_state is NULL, an fp32
 * [batch, nheads, headdim, dstate] state buffer.  Segments are 256-byte
 * aligned.  No part of a workspace needs to hold anything on entry.
 * Writes the size to *bytes.  Errors: NULL_POINTER, BAD_SHAPE, BAD_CHUNK,
 * BAD_DTYPE, UNSUPPORTED. */
ssd_status ssd_fwd_workspace_size(const ssd_problem* prob, size_t* bytes);

/* Workspace bytes that ssd_fwd_config needs with configuration `cfg` (NULL =
 * the default one, what ssd_fwd uses): the header and the layout of that
 * configuration's kernels only.  ssd_fwd_states, ssd_compute_out and
 * ssd_tune need the staged layout (cfg with fused = 0).  Errors: as
 * ssd_fwd_workspace_size, and BAD_VALUE for an invalid configuration. */
ssd_status ssd_fwd_config_workspace_size(const ssd_problem* prob, const ssd_config* cfg,
                                         size_t* bytes);

/* Whether the latest forward call on `workspace` gave up a bounded wait.
 * The forward kernels hand data between workgroups (the fused kernel from
 * chunk to chunk, compute_out between the waves of a workgroup) through waits
 * that cannot deadlock when the kernel's workgroups run concurrently, but
 * are bounded anyway; a wait past its bound marks the call in the workspace
 * header and leaves y and final_state undefined.  This call copies the
 * header to the host after synchronising with `stream` (it SYNCHRONISES) and
 * sets *timed_out to 1 if the latest call that used the workspace timed out,
 * else 0.  workspace: the one given to that call (16-byte aligned, at least
 * 16 bytes), or NULL for the built-in scratch of ssd_fwd_noalloc on the
 * current device (*timed_out = 0 if that entry point has not run there).
 * Errors: NULL_POINTER (timed_out NULL), MISALIGNED, WORKSPACE (fewer than
 * 16 bytes), HIP. */
ssd_status ssd_fwd_status(const void* workspace, size_t workspace_bytes, void* stream,
                          int32_t* timed_out);

/* Full forward pass: chunk_cumsum -> chunk_state -> state_pass -> compute_out.
 *   x, dt, A, B, C : inputs (device), layouts above.
 *   D              : [nheads] fp32 skip weights, or NULL for no skip term.
 *   init_state     : [batch, nheads, headdim, dstate] fp32, or NULL for zeros.
 *   y              : output [batch, seqlen, nheads, headdim] in the io dtype.
 *   final_state    : output state after the last token (fp32), or NULL.
 *   workspace      : device scratch of at least ssd_fwd_config_workspace_size
 *                    (prob, NULL) bytes (ssd_fwd_workspace_size is always
 *                    enough), 16-byte aligned, owned by the caller; its
 *                    contents on entry do not matter.  One workspace serves
 *                    one call at a time.
 *   stream         : hipStream_t to enqueue on (NULL = default stream). */
ssd_status ssd_fwd(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* init_state,
                   void* y, float* final_state, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ssd_fwd with the raw step size prepared inside stage 1 (see
 * ssd_dt_transform; dtx = NULL makes this exactly ssd_fwd).  Same workspace,
 * arguments, outputs and errors as ssd_fwd. */
ssd_status ssd_fwd_ex(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                      const float* dt, const float* A, const void* B, const void* C,
                      const float* D, const float* init_state, void* y, float* final_state,
                      void* workspace, size_t workspace_bytes, void* stream);

/* The tile choices ssd_fwd makes for `prob` (the static table).
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_CHUNK, BAD_DTYPE, UNSUPPORTED. */
ssd_status ssd_default_config(const ssd_problem* prob, ssd_config* cfg);

/* ssd_fwd_ex with the kernels' tile choices given (cfg = NULL: the default,
 * making this exactly ssd_fwd_ex).  An invalid choice is SSD_ERR_BAD_VALUE
 * (checked with the transform, before alignment).  The workspace must hold
 * ssd_fwd_config_workspace_size(prob, cfg) bytes.  Same arguments, outputs
 * and other errors as ssd_fwd. */
ssd_status ssd_fwd_config(const ssd_problem* prob, const ssd_config* cfg,
                          const ssd_dt_transform* dtx, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          const float* init_state, void* y, float* final_state, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ssd_fwd_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library's own scratch takes the
 * workspace's place: one 64 MiB array per GPU, part of the library's code
 * object, held until the process ends; its address is looked up once per
 * device.  This call allocates nothing.  Problems whose default
 * configuration needs more than 64 MiB of workspace (ssd_fwd_config_
 * workspace_size with cfg = NULL) are refused with SSD_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (several streams or threads) race, so the
 * caller serialises them; nothing in the scratch has to hold anything on
 * entry.  ssd_fwd_status(NULL, ...) reads its status word.  Same
 * arguments, outputs and other errors as ssd_fwd_ex. */
ssd_status ssd_fwd_noalloc(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                           const float* dt, const float* A, const void* B, const void* C,
                           const float* D, const float* init_state, void* y,
                           float* final_state, void* stream);

/* Shape tuning: runs the whole forward pass (as ssd_fwd_config, on the
 * caller's inputs and buffers) with every valid tile choice for `prob`, once
 * untimed and then `reps` times between two HIP events on `stream`, and
 * reports the mean time of each and the fastest choice.  The device is first
 * warmed up with the default choice, and every choice is measured twice (in
 * forward, then reverse order; the smaller mean is kept) so that clock or
 * cache drift during the sweep does not favour one end of it.  Unlike every other
 * entry point this one SYNCHRONISES with `stream` (once per choice), creates
 * and destroys two HIP events, and is meant to run once per shape, outside
 * any timed or captured region.  On return y and final_state hold the result
 * of the last run, init_state must not alias final_state (each run reads it),
 * and `workspace` is as for ssd_fwd.
 *   reps      : timed runs per choice, 1 .. 1000;
 *   tried, tried_ms : arrays of max_tried entries receiving the choices in
 *               the order measured and their mean ms (may be NULL when
 *               max_tried is 0);
 *   n_tried   : receives the number of choices measured (all valid ones,
 *               even beyond max_tried);
 *   best, best_ms : the fastest choice and its mean ms (best_ms may be NULL).
 * Errors as for ssd_fwd_ex; SSD_ERR_BAD_VALUE for reps or max_tried out of
 * range or init_state aliasing final_state; SSD_ERR_HIP if an event or
 * launch fails. */
ssd_status ssd_tune(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                    const float* dt, const float* A, const void* B, const void* C, const float* D,
                    const float* init_state, void* y, float* final_state, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t reps, ssd_config* tried,
                    float* tried_ms, int32_t max_tried, int32_t* n_tried, ssd_config* best,
                    float* best_ms);

/* Stage 1 alone (the chunk_cumsum step): for every (b, h) and token t in chunk
 * c = t / Q,
 *     G_out[b, h, t]  = log2(e) * sum_{k = cQ .. t} dt[b, k, h] * A[h]
 *     dt_out[b, h, t] = dt[b, t, h]
 * The within-chunk running sum of the decay a_k in base-2 log space, and dt
 * moved to [batch, head, token] order so later stages read tokens
 * contiguously (devin.kr page above, section "세 가지 핵심 커널 구현",
 * chunk_cumsum, and section "cuTile 기반 성능 최적화 기법" (optimisations),
 * the [batch, head, token] layout).  G_out, dt_out: [batch, nheads, seqlen]
 * fp32 device buffers.  Errors as for ssd_fwd (no workspace). */
ssd_status ssd_chunk_cumsum(const ssd_problem* prob, const float* dt, const float* A,
                            float* G_out, float* dt_out, void* stream);

/* ssd_chunk_cumsum with the step size prepared first (ssd_dt_transform;
 * NULL = ssd_chunk_cumsum): G_out and dt_out are built from dt', and dt_out
 * holds dt' itself. */
ssd_status ssd_chunk_cumsum_ex(const ssd_problem* prob, const ssd_dt_transform* dtx,
                               const float* dt, const float* A, float* G_out, float* dt_out,
                               void* stream);

/* Stages 1 and 2 (chunk_cumsum, chunk_state, state_pass): the state at the start of
 * every chunk and the state after the last token, without computing y
 * (devin.kr page above, section "세 가지 핵심 커널 구현", fwd_pass_state;
 * brifing.si page, sections 4, 5 and 8).  Chunk c's contribution is one matrix
 * product over the chunk's stacked x and B rows, each row weighted by
 * exp2(G_last - G_j) * dt_j; states pass on as
 * H_{c+1} = exp2(G_last) * H_c + S_c, with H_0 = init_state (or zero).
 *   chunk_states : output [batch, nheads, T, headdim, dstate] in the io dtype
 *                  (H_c for c = 0..T-1), or NULL.
 *   final_state  : output [batch, nheads, headdim, dstate] fp32 (required).
 *   workspace    : the staged layout (ssd_fwd_config_workspace_size with
 *                  fused = 0, or ssd_fwd_workspace_size).
 * Other arguments as for ssd_fwd.  These are the staged kernels whatever the
 * shape. */
ssd_status ssd_fwd_states(const ssd_problem* prob, const void* x, const float* dt,
                          const float* A, const void* B, const float* init_state,
                          float* final_state, void* chunk_states, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ssd_fwd_states with the raw step size prepared inside stage 1 (see
 * ssd_dt_transform; dtx = NULL makes this exactly ssd_fwd_states).  A
 * following ssd_compute_out on the same workspace uses the prepared step
 * sizes, so the pair equals ssd_fwd_ex. */
ssd_status ssd_fwd_states_ex(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                             const float* dt, const float* A, const void* B,
                             const float* init_state, float* final_state, void* chunk_states,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Stage 3 alone (compute_out): y from the inputs and from the running sums and
 * chunk-start states that a preceding ssd_fwd_states call left in `workspace`
 * (same problem, same workspace, chunk_states == NULL, enqueued earlier on
 * the same stream or otherwise ordered before this call).  For token i of a
 * chunk: y_i = sum_{j<=i} (C_i . B_j) exp2(G_i - G_j) dt_j x_j
 *            + exp2(G_i) H_c C_i + D_h x_i,
 * the fused carried-state term, causal interaction tile and skip of devin.kr
 * "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section "세 가지 핵심
 * 커널 구현", compute_out, and brifing.si "Accelerating Mamba-2 ...", sections
 * 9 and 11; the chunk x chunk tile is never written to memory.
 * With the staged kernels (ssd_config.fused = 0) ssd_fwd is exactly
 * ssd_fwd_states followed by ssd_compute_out.
 *   x, B, C, D, y : as for ssd_fwd (D may be NULL).
 *   workspace     : the staged layout (ssd_fwd_config_workspace_size with
 *                   fused = 0); its running sums and states are only read,
 *                   its header is written (ssd_fwd_status reports whether
 *                   the kernel's bounded waits all ended in time).
 * Errors as for ssd_fwd. */
ssd_status ssd_compute_out(const ssd_problem* prob, const void* x, const void* B, const void* C,
                           const float* D, void* y, const void* workspace,
                           size_t workspace_bytes, void* stream);

/* Token-sequential mode (decode): advance a resident state through
 * prob->seqlen tokens one at a time, without chunking.  For every (b, h):
 *     s = exp(dt_t A_h) s + dt_t x_t (outer) B_t,   y_t = s C_t + D_h x_t
 * for t = 0 .. seqlen-1, starting from `state` and leaving the state after
 * the last token in `state`.  This is the per-token recurrence that the
 * chunked pass evaluates in bulk (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향
 * 전달 커널 가속화", section "Mamba-2 아키텍처의 핵심 연산": the output line
 * y_t = c_t^T h_t + D x_t, run sequentially at inference); seqlen = 1 is one
 * decode step.  Results equal ssd_fwd over the same tokens with init_state =
 * state, up to rounding.
 *   state   : [batch, nheads, headdim, dstate] fp32 device, read and updated
 *             in place (required).
 *   x, y    : [batch, seqlen, nheads, headdim] io dtype; y must not overlap
 *             any input or the state.
 *   dt      : [batch, seqlen, nheads] fp32 (raw when dtx is given).
 *   A, D    : [nheads] fp32 (D may be NULL: no skip term).
 *   B, C    : [batch, seqlen, ngroups, dstate] io dtype.
 *   dtx     : optional step-size preparation (NULL = dt used as given).
 * prob->chunk_size is not used.  No workspace.  Errors as for ssd_fwd, with
 * the same limits on headdim and dstate; the state must not be read or
 * written by other work until the call has completed on `stream`. */
ssd_status ssd_step(const ssd_problem* prob, const ssd_dt_transform* dtx, float* state,
                    const void* x, const float* dt, const float* A, const void* B, const void* C,
                    const float* D, void* y, void* stream);

/* ------------------------------------------------------------------ backward */

/* Default workspace bytes of ssd_bwd for `prob`, and the least it accepts
 * (errors as for ssd_bwd's shape checks).
 *
 * The largest part of the workspace holds fp32 partial gradients of B and
 * C, one per "part" of kh consecutive heads of a group (the per-chunk
 * kernels sum a part's heads as they go; kh is the largest divisor of the
 * heads per group, up to 8, that leaves batch * chunks * nheads / kh >= 1024
 * workgroups, else 1, and depends on the shape alone).  These are summed
 * over the parts of each group.  ssd_bwd forms them for a batch of parts at
 * a time and folds each batch into running fp32 sums per group before the
 * next, so the workspace it needs shrinks with the parts per batch.  Given
 * workspace_bytes, ssd_bwd considers the batchings into equal batches whose
 * layout fits and takes the one whose per-chunk kernel launches need the
 * fewest rounds of the workgroups the device runs at once (the fewest
 * batches on a tie).  The default size keeps each batch's partial gradients
 * within the room of one fp32 copy of x (all parts in one batch when
 * 2 dstate (nheads / kh) <= nheads headdim), but keeps enough parts per
 * batch for about 1024 workgroups per launch; the minimum is the smallest
 * layout over all part counts.  Larger workspaces allow larger batches, up
 * to all parts.  Results do not depend on the batching: a part adds its
 * heads, and the per-group sums add the parts, in ascending order either
 * way, so they are bitwise identical for any accepted workspace size. */
ssd_status ssd_bwd_workspace_size(const ssd_problem* prob, size_t* bytes);
ssd_status ssd_bwd_workspace_min_size(const ssd_problem* prob, size_t* bytes);

/* Gradients of the scan: given dy = dLoss/dy and, optionally, dfinal =
 * dLoss/d(final state), the gradients of every input of ssd_fwd_ex.
 *
 * The pages stop at the forward pass and name the backward pass as what
 * end-to-end training still needs (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향
 * 전달 커널 가속화", closing remarks; brifing.si "Accelerating Mamba-2 ...",
 * limitations); the operation is the derivative of the forward definition
 * (ssd_fwd), evaluated chunkwise with the forward pass's own decomposition:
 * the chunk-start states are recomputed (stages 1 and 2), the gradients of
 * the chunk-boundary states run through the same two stages backwards
 * (weights exp2(G_i) on dy_i C_i^T, chunks last to first from dfinal), and one
 * pass per chunk forms dx, dB, dC and the per-token terms of the step-size
 * gradient, whose reverse running sum over the sequence gives ddt and dA.
 *
 *   dtx, x, dt, A, B, C, D, init_state : as for ssd_fwd_ex (D, init_state,
 *                 dtx optional).
 *   dy          : [batch, seqlen, nheads, headdim] io dtype.
 *   dfinal      : [batch, nheads, headdim, dstate] fp32, or NULL (zero).
 *   dx          : output, layout of x, io dtype.
 *   ddt         : output [batch, seqlen, nheads] fp32, gradient with respect
 *                 to the `dt` argument (the raw value when dtx is given: the
 *                 chain rule through bias, softplus and clamp, the clamp
 *                 passing the gradient where dt_min <= value <= dt_max).
 *   dA          : output [nheads] fp32.
 *   dB, dC      : outputs, layout of B and C, io dtype (summed over the
 *                 heads of each group).
 *   dD          : output [nheads] fp32, or NULL (not computed).
 *   dinit       : output [batch, nheads, headdim, dstate] fp32, or NULL.
 *   ddt_bias    : output [nheads] fp32, or NULL: the sum of ddt over batch
 *                 and tokens, i.e. the gradient with respect to a per-head
 *                 bias added to the dt argument.
 * Precision: every gradient is formed in fp32 from the io values, with the
 * chunk-boundary states and their gradients kept in fp32 (the step-size
 * gradient sums terms that largely cancel over the whole sequence); for bf16
 * io the chunk x chunk products run on bf16 MFMA (exact operands, fp32 sums)
 * and the products with fp32 weights as two bf16 MFMAs on a hi/lo split of
 * the weights (~16 significant bits); only dx, dB and dC are rounded to the
 * io dtype.  Deterministic: the same call gives bitwise the same results.
 * Outputs must not overlap inputs or each other.  Every pointer 16-byte
 * aligned.  Errors as for ssd_fwd_ex (same order: NULL pointers, shape,
 * chunk, dtype, transform values, alignment, limits, workspace, where
 * SSD_ERR_WORKSPACE means below ssd_bwd_workspace_min_size); in
 * addition SSD_ERR_UNSUPPORTED when headdim exceeds 256 or the per-chunk
 * tiles of headdim x dstate do not fit the LDS.  Enqueued on `stream`
 * without synchronising. */
ssd_status ssd_bwd(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                   const float* dt, const float* A, const void* B, const void* C, const float* D,
                   const float* init_state, const void* dy, const float* dfinal, void* dx,
                   float* ddt, float* dA, void* dB, void* dC, float* dD, float* dinit,
                   float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
