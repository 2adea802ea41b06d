// ssd_api.cpp -- host side of libssd: validation, workspace plan, launches.
//
// Every entry point validates its arguments on the host, in the order the
// public header documents, before making any HIP call; on success it
// enqueues the stage kernels on the caller's stream and returns without
// synchronising.  No exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <exception>
#include <string>

#include "../../include/ssd.h"
#include "ssd_device.hpp"

namespace ssd {
hipError_t launch_chunk_cumsum(const float* dt, const float* A, float* G, float* dtT,
                               int64_t batch, int64_t L, int64_t H, int Q, int64_t ld,
                               int64_t Lw, const DtXform* xf, int heads_tile, hipStream_t stream);
hipError_t launch_step(int io_bf16, float* state, const void* x, const float* dt, const float* A,
                       const void* Bm, const void* Cm, const float* D, void* y,
                       const DtXform* xf, int64_t batch, int64_t L, int64_t H, int64_t P,
                       int64_t N, int64_t G, hipStream_t stream);
hipError_t launch_chunk_state(int io_bf16, const void* x, const void* Bm, float* Gw, float* dtw,
                              void* S, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int Q, int64_t T_, int64_t ldw, int frag_major, int kh,
                              const float* dt_raw, const float* A, const DtXform* xf,
                              hipStream_t stream);
hipError_t launch_state_pass(int io_bf16, void* S, const float* Gw, const float* init_state,
                             float* final_state, int64_t batch, int64_t H, int64_t P, int64_t N,
                             int Q, int64_t T_, int64_t ldw, int frag_major, int reverse,
                             hipStream_t stream);
hipError_t launch_compute_out(int io_bf16, const void* x, const void* Bm, const void* Cm,
                              const float* Gw, const float* dtw, const void* Hc, const float* Dv,
                              void* y, StatusRef status, int64_t batch, int64_t L, int64_t H, int64_t P,
                              int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw,
                              int kh, hipStream_t stream);
int compute_out_smem_bytes(int io_bf16, int Q, int64_t N, int kh);
hipError_t launch_out_resident(const void* x, const void* Bm, const void* Cm, const float* Gw,
                               const float* dtw, const void* Hc, const float* Dv, void* y,
                               StatusRef flag, int64_t batch, int64_t L, int64_t H, int64_t N,
                               int64_t G, int64_t T_, int64_t ldw, hipStream_t stream);
int out_resident_supported(int io_bf16, int64_t H, int64_t P, int64_t N, int Q);
hipError_t launch_fused_fwd(const void* x, const float* dt, const float* A, const void* Bm,
                            const void* Cm, const float* D, const float* init, float* chain,
                            void* y, void* flags, void* status, void* last_gen,
                            const DtXform* xf, int64_t batch, int64_t L, int64_t H, int64_t G,
                            int Q, int64_t T, unsigned int gen, hipStream_t stream);
int fused_fwd_supported(int io_bf16, int64_t H, int64_t G, int64_t P, int64_t N, int Q);
size_t fused_fwd_flag_bytes(int64_t batch, int64_t H, int64_t N);
void* noalloc_scratch_address();
int compute_out_kh_valid(int io_bf16, int64_t H, int64_t G, int64_t N, int kh);
int compute_out_default_kh(int io_bf16, int64_t H, int64_t G, int64_t N);
int chunk_state_default_kh(int64_t H, int64_t G);
int bwd_block_rows(int io_bf16, int Q, int64_t P, int64_t N);
int64_t bwd_chunk_slots(int io_bf16, int64_t P, int64_t N);
hipError_t launch_chunk_state_split(const void* x, const void* Bm, float* Gw, float* dtw,
                                    float* S, int64_t batch, int64_t L, int64_t H, int64_t P,
                                    int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw, int kh,
                                    hipStream_t stream);
hipError_t launch_bwd_prep(const float* Gw, float* w2, float* Gz, int64_t batch, int64_t H,
                           int64_t L, int64_t ldw, hipStream_t stream);
hipError_t launch_bwd_chunks(int io_bf16, int TB, const void* x, const void* Bm, const void* Cm,
                             const void* dy, const float* Gw, const float* dtw, const void* Hc,
                             const void* Lam, const float* Dv, void* dx, float* Pb, float* Qb,
                             float* dBh, float* dCh, float* dDpart, int64_t batch, int64_t L,
                             int64_t H, int64_t P, int64_t N, int64_t G, int Q, int64_t T_,
                             int64_t ldw, int p0, int np, int hbp, int kh, hipStream_t stream);
int bwd_part_heads(int64_t batch, int64_t T_, int64_t H, int64_t G);
hipError_t launch_bwd_group_sum(int io_bf16, const float* dBh, const float* dCh, float* accB,
                                float* accC, void* dB, void* dC, int64_t batch, int64_t L,
                                int64_t H, int64_t N, int64_t G, int h0, int nb, int hb,
                                hipStream_t stream);
hipError_t launch_bwd_finish(const float* Pb, const float* Qb, const float* dtw,
                             const float* dt_in, const float* A, const float* dfinal,
                             const float* fin, const DtXform* xf, float* ddt, double* dApart,
                             double* dbpart, const float* dDpart, float* dA, float* dD,
                             float* dbias, int64_t batch, int64_t L, int64_t H, int64_t P,
                             int64_t N, int64_t T_, int64_t ldw, hipStream_t stream);
}  // namespace ssd

namespace {

constexpr int64_t kMaxLds = 160 * 1024;
// Every forward workspace starts with this header: [0] the status word a
// kernel writes when a bounded wait gives up ((gen << 32) | 1), [1] the gen
// of the latest call that used the workspace.
constexpr size_t kHeaderBytes = 256;
thread_local std::string g_last_error;

// Call generations.  Each forward call takes a fresh 32-bit value; the fused
// kernel tags its chunk-to-chunk flags with it (so flags left by an earlier
// call never match) and both paths tag the status word.  Seeded from the
// clock so that a workspace reused by another process does not repeat them.
unsigned int next_gen() {
  static std::atomic<unsigned int> ctr{0u};
  static std::atomic<bool> seeded{false};
  if (!seeded.load(std::memory_order_acquire)) {
    const auto t = std::chrono::high_resolution_clock::now().time_since_epoch().count();
    unsigned int expect = 0u;
    ctr.compare_exchange_strong(expect, (unsigned int)((uint64_t)t ^ ((uint64_t)t >> 32)) | 1u);
    seeded.store(true, std::memory_order_release);
  }
  unsigned int g = ctr.fetch_add(1u, std::memory_order_relaxed);
  return g ? g : ctr.fetch_add(1u, std::memory_order_relaxed);
}

ssd_status fail(ssd_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ssd_status fail(ssd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ssd_status ok() {
  g_last_error.clear();
  return SSD_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
  // Q: the chunk the kernels run; Qreq: the caller's chunk_size (16 runs as 32)
  int64_t B, L, H, P, N, G, Q, T, Lp, Qreq;
  int bf16;
  size_t esize;
  // staged path: running sums, step sizes, chunk-start states
  size_t g_off, dt_off, hc_off, staged_bytes;
  // stage 3 with the interaction tile resident across heads (out_resident)
  int resident_ok;
  // fused path: chunk-to-chunk flags and the state handed between chunks
  int fused_ok;
  size_t flags_off, chain_off, fused_bytes;
  size_t bytes;   // enough for either path (ssd_fwd_workspace_size)
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Shape checks shared by every entry point (after the NULL checks).  The
// decode step does not chunk, so it skips the chunk-size check.
ssd_status plan_problem(const ssd_problem* prob, Plan* pl, bool need_chunk = true) {
  const ssd_problem& p = *prob;
  if (p.batch <= 0 || p.seqlen <= 0 || p.nheads <= 0 || p.headdim <= 0 || p.dstate <= 0 ||
      p.ngroups <= 0 || (need_chunk && p.chunk_size <= 0))
    return fail(SSD_ERR_BAD_SHAPE, "every size must be positive");
  if (p.nheads % p.ngroups != 0)
    return fail(SSD_ERR_BAD_SHAPE, "nheads (%lld) must be a multiple of ngroups (%lld)",
                (long long)p.nheads, (long long)p.ngroups);
  int64_t t1, t2, t3;
  if (!mul_ok(p.batch, p.seqlen, &t1) || !mul_ok(t1, p.nheads, &t2) ||
      !mul_ok(t2, p.headdim, &t3) || !mul_ok(t1, p.ngroups, &t2) || !mul_ok(t2, p.dstate, &t3))
    return fail(SSD_ERR_BAD_SHAPE, "tensor size overflows int64");
  if (p.seqlen > INT64_MAX / 2 - 256)
    return fail(SSD_ERR_BAD_SHAPE, "seqlen too large");
  const int64_t Qreq = need_chunk ? p.chunk_size : 256;
  if (!(Qreq == 16 || Qreq == 32 || Qreq == 64 || Qreq == 128 || Qreq == 256))
    return fail(SSD_ERR_BAD_CHUNK, "chunk_size must be 16, 32, 64, 128 or 256 (got %lld)",
                (long long)Qreq);
  // The chunk size does not change y, the final state or any gradient (the
  // chunked evaluation equals the recurrence for every chunk size), and the
  // MFMA kernels step through tokens 32 at a time: a chunk of 16 runs as 32.
  // Only the entry points that return per-chunk values (ssd_chunk_cumsum,
  // ssd_fwd_states, ssd_compute_out) depend on it.
  const int64_t Q = Qreq < 32 ? 32 : Qreq;
  if (p.io_dtype != SSD_BF16 && p.io_dtype != SSD_F32)
    return fail(SSD_ERR_BAD_DTYPE, "io_dtype must be SSD_BF16 or SSD_F32 (got %d)", p.io_dtype);
  if (p.reserved != 0) return fail(SSD_ERR_BAD_DTYPE, "reserved field must be 0");
  pl->B = p.batch; pl->L = p.seqlen; pl->H = p.nheads; pl->P = p.headdim; pl->N = p.dstate;
  pl->G = p.ngroups; pl->Q = Q; pl->Qreq = Qreq;
  pl->T = (p.seqlen + Q - 1) / Q;
  pl->Lp = pl->T * Q;
  pl->bf16 = p.io_dtype == SSD_BF16;
  pl->esize = pl->bf16 ? 2 : 4;
  pl->fused_ok = need_chunk && ssd::fused_fwd_supported(pl->bf16, pl->H, pl->G, pl->P, pl->N, (int)Q);
  pl->resident_ok = need_chunk && ssd::out_resident_supported(pl->bf16, pl->H, pl->P, pl->N, (int)Q);
  return SSD_OK;
}

// The optional step-size preparation: value checks (after the dtype check)
// and the device-side description the kernels take.
ssd_status check_dt_transform(const ssd_dt_transform* dtx, ssd::DtXform* xf) {
  if (!dtx) return SSD_OK;
  if (dtx->softplus != 0 && dtx->softplus != 1)
    return fail(SSD_ERR_BAD_VALUE, "dt transform: softplus must be 0 or 1 (got %d)", dtx->softplus);
  if (dtx->reserved != 0) return fail(SSD_ERR_BAD_VALUE, "dt transform: reserved field must be 0");
  if (dtx->dt_min != dtx->dt_min || dtx->dt_max != dtx->dt_max)
    return fail(SSD_ERR_BAD_VALUE, "dt transform: dt_min and dt_max must not be NaN");
  if (dtx->dt_min > dtx->dt_max)
    return fail(SSD_ERR_BAD_VALUE, "dt transform: dt_min (%g) exceeds dt_max (%g)",
                (double)dtx->dt_min, (double)dtx->dt_max);
  xf->bias = dtx->dt_bias;
  xf->softplus = dtx->softplus;
  xf->lo = dtx->dt_min;
  xf->hi = dtx->dt_max;
  return SSD_OK;
}

// The kernels' tile choices (ssd_config): the static table, and the checks a
// caller's choice must pass.
// Heads per workgroup of the stand-alone running-sum kernel.
constexpr int kCumsumHeads = 4;

ssd_config default_config(const Plan& pl) {
  ssd_config c;
  // the running sums inside chunk_state: no launch of their own, and no
  // round trip of the raw step sizes through a kernel boundary
  c.cumsum_heads = 0;
  c.state_heads = ssd::chunk_state_default_kh(pl.H, pl.G);
  c.out_heads = ssd::compute_out_default_kh(pl.bf16, pl.H, pl.G, pl.N);
  // the staged kernels: at the shapes the fused kernel is built for they
  // measure faster on MI355X (2.7B shape, cold cache: 0.29 ms against 0.37
  // ms), so the fused kernel is an explicit choice and a tuning candidate
  c.fused = 0;
  // stage 3 with the interaction tile resident across heads where it is
  // built (2.7B shape, cold cache: 0.22 ms for the whole pass against 0.28 ms
  // with the head-pair kernel)
  c.out_resident = pl.resident_ok ? 1 : 0;
  return c;
}

ssd_status check_config(const Plan& pl, const ssd_config& c) {
  if (c.fused != 0 && c.fused != 1)
    return fail(SSD_ERR_BAD_VALUE, "config: fused must be 0 or 1 (got %d)", c.fused);
  if (c.fused && !pl.fused_ok)
    return fail(SSD_ERR_BAD_VALUE,
                "config: the fused kernel is built for bf16 io, headdim 64, dstate 128, "
                "chunk_size 256 and an even number of heads per group");
  if (c.out_resident != 0 && c.out_resident != 1)
    return fail(SSD_ERR_BAD_VALUE, "config: out_resident must be 0 or 1 (got %d)", c.out_resident);
  if (c.out_resident && !pl.resident_ok)
    return fail(SSD_ERR_BAD_VALUE,
                "config: out_resident is built for bf16 io, headdim 64, dstate <= 128, "
                "chunk_size 256 and nheads * headdim <= 2^22");
  if (c.cumsum_heads != 0 && c.cumsum_heads != 4 && c.cumsum_heads != 16)
    return fail(SSD_ERR_BAD_VALUE, "config: cumsum_heads must be 0, 4 or 16 (got %d)",
                c.cumsum_heads);
  const int64_t hg = pl.H / pl.G;
  if (!(c.state_heads == 1 || c.state_heads == 2 || c.state_heads == 4) || hg % c.state_heads != 0)
    return fail(SSD_ERR_BAD_VALUE,
                "config: state_heads must be 1, 2 or 4 and divide the %lld heads of a group (got %d)",
                (long long)hg, c.state_heads);
  if (!ssd::compute_out_kh_valid(pl.bf16, pl.H, pl.G, pl.N, c.out_heads))
    return fail(SSD_ERR_BAD_VALUE,
                "config: out_heads must be 1, or 2 for bf16 io, dstate <= 128 and an even number "
                "of heads per group (got %d)", c.out_heads);
  return SSD_OK;
}

// Limits of the kernels (checked after alignment, as the header documents).
ssd_status check_supported(const Plan& pl, int out_heads = 0) {
  if (pl.P % 16 != 0 || pl.N % 16 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "headdim (%lld) and dstate (%lld) must be multiples of 16",
                (long long)pl.P, (long long)pl.N);
  if (pl.N > 256) return fail(SSD_ERR_UNSUPPORTED, "dstate must be <= 256 (got %lld)", (long long)pl.N);
  if (pl.B * pl.H > INT32_MAX / 64 || pl.B * pl.T > INT32_MAX / 64 || pl.H > 65535 ||
      pl.B > 65535 || pl.T > INT32_MAX / 8)
    return fail(SSD_ERR_UNSUPPORTED, "grid too large for this build");
  const int okh = out_heads ? out_heads : ssd::compute_out_default_kh(pl.bf16, pl.H, pl.G, pl.N);
  if (ssd::compute_out_smem_bytes(pl.bf16, (int)pl.Q, pl.N, okh) > kMaxLds)
    return fail(SSD_ERR_UNSUPPORTED, "fp32 io with chunk_size %lld and dstate %lld exceeds LDS",
                (long long)pl.Q, (long long)pl.N);
  return SSD_OK;
}

void workspace_plan(Plan* pl) {
  const size_t gsz = size_t(pl->B) * pl->H * pl->Lp * sizeof(float);
  pl->g_off = kHeaderBytes;
  pl->dt_off = pl->g_off + align256(gsz);
  pl->hc_off = pl->dt_off + align256(gsz);
  // chunk-start states, fragment-major (padded to whole 64-row slices and
  // 32-column steps)
  const size_t hcsz = size_t(pl->B) * pl->H * pl->T * size_t(ssd::hc_frag(pl->P, pl->N).state_elems()) *
                      pl->esize;
  pl->staged_bytes = pl->hc_off + align256(hcsz);
  pl->flags_off = kHeaderBytes;
  pl->chain_off = pl->flags_off + align256(ssd::fused_fwd_flag_bytes(pl->B, pl->H, pl->N));
  pl->fused_bytes = pl->chain_off + align256(size_t(pl->B) * pl->H * pl->P * pl->N * sizeof(float));
  pl->bytes = pl->staged_bytes;
  if (pl->fused_ok && pl->fused_bytes > pl->bytes) pl->bytes = pl->fused_bytes;
}

size_t config_bytes(const Plan& pl, const ssd_config& c) {
  return c.fused ? pl.fused_bytes : pl.staged_bytes;
}

// Backward-pass workspace: running sums and step sizes, the reversed-chunk
// weights, per-token P and Qr, chunk-start states H_c and boundary-state
// gradients L_{c+1} ([batch, H, T, P, N] fp32), the final state, the
// per-part dB/dC sums, the per-(b, h) / per-(b, c, h) scalar parts and, with
// more than one batch of parts, the running per-group sums.
struct BwdPlan {
  size_t g_off, dt_off, gz_off, w2_off, pb_off, qb_off, hc_off, lam_off, fin_off, dap_off,
      dbp_off, ddp_off, acb_off, acc_off, dbh_off, dch_off, bytes;
  int TB;
  int kh;    // heads per part: a chunk-kernel workgroup sums their dB/dC contributions
  int np;    // parts, H / kh
  int hb;    // parts per batch of the chunk kernels (their dB/dC sums are rows of hb parts)
};

// Workspace of the backward pass for batches of hb parts.  The fp32 dB/dC
// sums of the parts are the largest item (2 x B L (H / kh) N floats); they
// are produced for hb parts at a time and folded into running per-group sums
// after each batch, so only one batch's parts exist at a time.
BwdPlan bwd_plan(const Plan& pl, int64_t hb) {
  BwdPlan w;
  const size_t tok = align256(size_t(pl.B) * pl.H * pl.Lp * sizeof(float));
  const size_t st = align256(size_t(pl.B) * pl.H * pl.T * pl.P * pl.N * sizeof(float));
  const size_t one_part = size_t(pl.B) * pl.L * pl.N * sizeof(float);   // one part, one of dB/dC
  w.kh = ssd::bwd_part_heads(pl.B, pl.T, pl.H, pl.G);
  w.np = (int)(pl.H / w.kh);
  w.hb = (int)hb;
  const size_t parts = align256(one_part * size_t(hb));
  const size_t acc = hb < w.np ? align256(size_t(pl.B) * pl.L * pl.G * pl.N * sizeof(float)) : 0;
  size_t o = 0;
  w.g_off = o; o += tok;
  w.dt_off = o; o += tok;
  w.gz_off = o; o += tok;
  w.w2_off = o; o += tok;
  w.pb_off = o; o += tok;
  w.qb_off = o; o += tok;
  w.hc_off = o; o += st;
  w.lam_off = o; o += st;
  w.fin_off = o; o += align256(size_t(pl.B) * pl.H * pl.P * pl.N * sizeof(float));
  w.dap_off = o; o += align256(size_t(pl.B) * pl.H * sizeof(double));
  w.dbp_off = o; o += align256(size_t(pl.B) * pl.H * sizeof(double));
  w.ddp_off = o; o += align256(size_t(pl.B) * pl.T * pl.H * sizeof(float));
  w.acb_off = o; o += acc;
  w.acc_off = o; o += acc;
  w.dbh_off = o; o += parts;
  w.dch_off = o; o += parts;
  w.bytes = o;
  w.TB = ssd::bwd_block_rows(pl.bf16, (int)pl.Q, pl.P, pl.N);
  return w;
}

// Batches of at most `cap` parts, balanced: ceil(n / cap) batches of equal
// size but for the last.
int64_t balanced_heads(int64_t n, int64_t cap) {
  const int64_t nbat = (n + cap - 1) / cap;
  return (n + nbat - 1) / nbat;
}

int64_t bwd_parts(const Plan& pl) { return pl.H / ssd::bwd_part_heads(pl.B, pl.T, pl.H, pl.G); }

// The default plan (ssd_bwd_workspace_size): all parts in one batch when
// their dB/dC sums take no more room than an fp32 copy of x would (2 N parts
// <= H P); otherwise the part count that fits that room, but at least enough
// parts for ~1024 workgroups per chunk-kernel launch.
BwdPlan bwd_default_plan(const Plan& pl) {
  const int64_t np = bwd_parts(pl);
  int64_t hb = np;
  if (2 * pl.N * np > pl.H * pl.P) {
    const int64_t fit = std::max<int64_t>(1, pl.H * pl.P / (2 * pl.N));
    const int64_t wg = pl.B * pl.T;
    hb = balanced_heads(np, std::min<int64_t>(np, std::max<int64_t>(fit, (1024 + wg - 1) / wg)));
  }
  return bwd_plan(pl, hb);
}

// The plan for a caller's workspace.  Among the part batchings whose layout
// fits `bytes` (nbat equal batches of hb = ceil(np / nbat) parts), the one
// whose chunk-kernel launches take the fewest rounds of `slots` concurrent
// workgroups (B T hb workgroups per batch), the fewest batches on a tie; with
// slots = 0 (unknown), the most parts per batch that fit.  hb = 0 when not
// even one part per batch fits.
BwdPlan bwd_plan_for(const Plan& pl, size_t bytes, int64_t slots) {
  BwdPlan best{};
  int64_t best_rounds = -1;
  const int64_t np = bwd_parts(pl);
  for (int64_t nbat = 1; nbat <= np; ++nbat) {
    const int64_t hb = (np + nbat - 1) / nbat;
    if ((np + hb - 1) / hb != nbat) continue;    // the same batching as a smaller nbat
    const BwdPlan w = bwd_plan(pl, hb);
    if (w.bytes > bytes) continue;
    if (slots <= 0) return w;
    const int64_t wg = pl.B * pl.T, full = np / hb, rest = np % hb;
    const int64_t rounds = full * ((wg * hb + slots - 1) / slots) + (wg * rest + slots - 1) / slots;
    if (best_rounds < 0 || rounds < best_rounds) {
      best = w;
      best_rounds = rounds;
    }
  }
  if (best_rounds < 0) {
    best = bwd_plan(pl, 1);
    best.hb = 0;
  }
  return best;
}

// The smallest workspace any part batching needs.
size_t bwd_min_bytes(const Plan& pl) {
  size_t m = SIZE_MAX;
  const int64_t np = bwd_parts(pl);
  for (int64_t cap = np; cap >= 1; --cap)
    m = std::min(m, bwd_plan(pl, balanced_heads(np, cap)).bytes);
  return m;
}

ssd_status check_supported_bwd(const Plan& pl) {
  ssd_status st = check_supported(pl);
  if (st != SSD_OK) return st;
  if (pl.P > 256) return fail(SSD_ERR_UNSUPPORTED, "backward: headdim must be <= 256");
  if (ssd::bwd_block_rows(pl.bf16, (int)pl.Q, pl.P, pl.N) == 0)
    return fail(SSD_ERR_UNSUPPORTED, "backward: headdim %lld and dstate %lld exceed LDS",
                (long long)pl.P, (long long)pl.N);
  return SSD_OK;
}

ssd_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

static ssd_status check_fwd(const ssd_problem* prob, const ssd_config* cfg,
                            const ssd_dt_transform* dtx, const void* x, const float* dt,
                            const float* A, const void* B, const void* C, const float* D,
                            const float* init_state, void* y, float* final_state,
                            void* workspace, size_t workspace_bytes, Plan* pl, ssd_config* use,
                            ssd::DtXform* xf);

namespace ssd {

// Argument checks of the forward entry points without the workspace check,
// for the entry point that brings its own scratch; reports the bytes the
// default configuration needs.
ssd_status fwd_check_scratch(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                             const float* dt, const float* A, const void* B, const void* C,
                             const float* D, const float* init_state, void* y,
                             float* final_state, size_t* need) {
  try {
    Plan pl;
    ssd_config use;
    ssd::DtXform xf;
    // any non-NULL, aligned stand-in passes the workspace pointer checks; the
    // size check is made against the scratch by the caller
    alignas(16) static const unsigned char stand_in[16] = {0};
    ssd_status st = check_fwd(prob, nullptr, dtx, x, dt, A, B, C, D, init_state, y, final_state,
                              const_cast<unsigned char*>(stand_in), SIZE_MAX, &pl, &use, &xf);
    if (st != SSD_OK) return st;
    *need = config_bytes(pl, use);
    return SSD_OK;
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status report(ssd_status st, const char* msg) {
  if (st == SSD_OK) return ok();
  return fail(st, "%s", msg);
}

}  // namespace ssd

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL_POINTER: return "required pointer is NULL";
    case SSD_ERR_BAD_SHAPE: return "invalid problem shape";
    case SSD_ERR_BAD_CHUNK: return "unsupported chunk size";
    case SSD_ERR_BAD_DTYPE: return "invalid io dtype";
    case SSD_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case SSD_ERR_WORKSPACE: return "workspace too small";
    case SSD_ERR_UNSUPPORTED: return "shape not supported by this build";
    case SSD_ERR_HIP: return "HIP runtime error";
    case SSD_ERR_INTERNAL: return "internal error";
    case SSD_ERR_BAD_VALUE: return "invalid argument value";
    default: return "unknown status";
  }
}

const char* ssd_last_error_message(void) { return g_last_error.c_str(); }

ssd_status ssd_fwd_workspace_size(const ssd_problem* prob, size_t* bytes) {
  try {
    if (!prob || !bytes) return fail(SSD_ERR_NULL_POINTER, "prob and bytes must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    st = check_supported(pl);
    if (st != SSD_OK) return st;
    workspace_plan(&pl);
    *bytes = pl.bytes;
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_fwd_config_workspace_size(const ssd_problem* prob, const ssd_config* cfg,
                                        size_t* bytes) {
  try {
    if (!prob || !bytes) return fail(SSD_ERR_NULL_POINTER, "prob and bytes must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    workspace_plan(&pl);
    const ssd_config use = cfg ? *cfg : default_config(pl);
    st = check_config(pl, use);
    if (st != SSD_OK) return st;
    st = check_supported(pl, use.out_heads);
    if (st != SSD_OK) return st;
    *bytes = config_bytes(pl, use);
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_fwd_status(const void* workspace, size_t workspace_bytes, void* stream,
                          int32_t* timed_out) {
  try {
    if (!timed_out) return fail(SSD_ERR_NULL_POINTER, "timed_out must not be NULL");
    const void* ws = workspace;
    if (!ws) {
      ws = ssd::noalloc_scratch_address();
      if (!ws) {            // the no-allocation entry point has not run on this device
        *timed_out = 0;
        return ok();
      }
    } else {
      if (!aligned16(ws)) return fail(SSD_ERR_MISALIGNED, "workspace must be 16-byte aligned");
      if (workspace_bytes < 16)
        return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, the header needs 16",
                    workspace_bytes);
    }
    unsigned long long h[2] = {0ull, 0ull};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h, ws, sizeof(h), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "status read");
    // the status word is tagged with the gen of the call that timed out;
    // the latest call recorded its own gen in the next word
    *timed_out = (h[0] & 0xffffffffull) != 0 && (h[0] >> 32) == (h[1] & 0xffffffffull);
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_chunk_cumsum_ex(const ssd_problem* prob, const ssd_dt_transform* dtx,
                               const float* dt, const float* A, float* G_out, float* dt_out,
                               void* stream) {
  try {
    if (!prob || !dt || !A || !G_out || !dt_out)
      return fail(SSD_ERR_NULL_POINTER, "prob, dt, A, G_out and dt_out must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    ssd::DtXform xf;
    st = check_dt_transform(dtx, &xf);
    if (st != SSD_OK) return st;
    if (!aligned16(dt) || !aligned16(A) || !aligned16(G_out) || !aligned16(dt_out) ||
        (dtx && !aligned16(dtx->dt_bias)))
      return fail(SSD_ERR_MISALIGNED, "dt, A, dt_bias, G_out and dt_out must be 16-byte aligned");
    st = check_supported(pl);
    if (st != SSD_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(ssd::launch_chunk_cumsum(dt, A, G_out, dt_out, pl.B, pl.L, pl.H, (int)pl.Qreq,
                                               pl.L, pl.L, dtx ? &xf : nullptr, kCumsumHeads,
                                               s),
                      "chunk_cumsum launch");
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_chunk_cumsum(const ssd_problem* prob, const float* dt, const float* A,
                            float* G_out, float* dt_out, void* stream) {
  return ssd_chunk_cumsum_ex(prob, nullptr, dt, A, G_out, dt_out, stream);
}

static ssd_status run_states(const Plan& pl, const ssd_config& cfg, const void* x, const float* dt,
                             const float* A, const void* B, const float* init_state,
                             float* final_state, void* chunk_states, void* workspace,
                             const ssd::DtXform* xf, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  float* Gw = reinterpret_cast<float*>(ws + pl.g_off);
  float* dtw = reinterpret_cast<float*>(ws + pl.dt_off);
  void* Hc = chunk_states ? chunk_states : static_cast<void*>(ws + pl.hc_off);
  // the running sums: a chunk_cumsum launch, or (cumsum_heads = 0) inside
  // chunk_state, which then writes the same rows
  const bool fold = cfg.cumsum_heads == 0;
  hipError_t e = hipSuccess;
  if (!fold) {
    e = ssd::launch_chunk_cumsum(dt, A, Gw, dtw, pl.B, pl.L, pl.H, (int)pl.Q, pl.Lp, pl.Lp, xf,
                                 cfg.cumsum_heads, s);
    if (e != hipSuccess) return hip_status(e, "chunk_cumsum launch");
  }
  // each chunk's own contribution S_c into the state buffer, then the
  // recurrence turns it, in place, into the chunk-start states H_c
  const int frag_major = chunk_states ? 0 : 1;
  e = ssd::launch_chunk_state(pl.bf16, x, B, Gw, dtw, Hc, pl.B, pl.L, pl.H, pl.P, pl.N, pl.G,
                              (int)pl.Q, pl.T, pl.Lp, frag_major, cfg.state_heads,
                              fold ? dt : nullptr, A, xf, s);
  if (e != hipSuccess) return hip_status(e, "chunk_state launch");
  e = ssd::launch_state_pass(pl.bf16, Hc, Gw, init_state, final_state, pl.B, pl.H, pl.P, pl.N,
                             (int)pl.Q, pl.T, pl.Lp, frag_major, 0, s);
  return hip_status(e, "state_pass launch");
}

ssd_status ssd_fwd_states_ex(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                             const float* dt, const float* A, const void* B,
                             const float* init_state, float* final_state, void* chunk_states,
                             void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!prob || !x || !dt || !A || !B || !final_state || !workspace)
      return fail(SSD_ERR_NULL_POINTER,
                  "prob, x, dt, A, B, final_state and workspace must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    ssd::DtXform xf;
    st = check_dt_transform(dtx, &xf);
    if (st != SSD_OK) return st;
    if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) ||
        !aligned16(init_state) || !aligned16(final_state) || !aligned16(chunk_states) ||
        !aligned16(workspace) || (dtx && !aligned16(dtx->dt_bias)))
      return fail(SSD_ERR_MISALIGNED, "every tensor pointer must be 16-byte aligned");
    st = check_supported(pl);
    if (st != SSD_OK) return st;
    if (pl.Qreq != pl.Q)
      return fail(SSD_ERR_UNSUPPORTED, "chunk_size %lld: the chunk-state kernels are built for "
                  "32..256 (ssd_fwd and ssd_bwd take 16)", (long long)pl.Qreq);
    workspace_plan(&pl);
    if (workspace_bytes < pl.staged_bytes)
      return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  pl.staged_bytes);
    return run_states(pl, default_config(pl), x, dt, A, B, init_state, final_state, chunk_states,
                      workspace, dtx ? &xf : nullptr, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_fwd_states(const ssd_problem* prob, const void* x, const float* dt,
                          const float* A, const void* B, const float* init_state,
                          float* final_state, void* chunk_states, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return ssd_fwd_states_ex(prob, nullptr, x, dt, A, B, init_state, final_state, chunk_states,
                           workspace, workspace_bytes, stream);
}

static ssd_status run_out(const Plan& pl, const ssd_config& cfg, const void* x, const void* B,
                          const void* C, const float* D, void* y, const void* workspace,
                          hipStream_t s) {
  const char* ws = static_cast<const char*>(workspace);
  const float* Gw = reinterpret_cast<const float*>(ws + pl.g_off);
  const float* dtw = reinterpret_cast<const float*>(ws + pl.dt_off);
  const void* Hc = ws + pl.hc_off;
  ssd::StatusRef status{reinterpret_cast<unsigned long long*>(const_cast<char*>(ws)), next_gen()};
  if (cfg.out_resident)
    return hip_status(ssd::launch_out_resident(x, B, C, Gw, dtw, Hc, D, y, status, pl.B, pl.L, pl.H,
                                               pl.N, pl.G, pl.T, pl.Lp, s),
                      "compute_out launch");
  return hip_status(ssd::launch_compute_out(pl.bf16, x, B, C, Gw, dtw, Hc, D, y, status, pl.B, pl.L,
                                            pl.H, pl.P, pl.N, pl.G, (int)pl.Q, pl.T, pl.Lp,
                                            cfg.out_heads, s),
                    "compute_out launch");
}

ssd_status ssd_compute_out(const ssd_problem* prob, const void* x, const void* B, const void* C,
                           const float* D, void* y, const void* workspace,
                           size_t workspace_bytes, void* stream) {
  try {
    if (!prob || !x || !B || !C || !y || !workspace)
      return fail(SSD_ERR_NULL_POINTER, "prob, x, B, C, y and workspace must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(D) || !aligned16(y) ||
        !aligned16(workspace))
      return fail(SSD_ERR_MISALIGNED, "every tensor pointer must be 16-byte aligned");
    st = check_supported(pl);
    if (st != SSD_OK) return st;
    if (pl.Qreq != pl.Q)
      return fail(SSD_ERR_UNSUPPORTED, "chunk_size %lld: the chunk-state kernels are built for "
                  "32..256 (ssd_fwd and ssd_bwd take 16)", (long long)pl.Qreq);
    workspace_plan(&pl);
    if (workspace_bytes < pl.staged_bytes)
      return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  pl.staged_bytes);
    return run_out(pl, default_config(pl), x, B, C, D, y, workspace,
                   static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

// Validation shared by the forward entry points (NULL / shape / chunk / dtype,
// then the transform and the config values, alignment, limits, workspace).
static ssd_status check_fwd(const ssd_problem* prob, const ssd_config* cfg,
                            const ssd_dt_transform* dtx, const void* x, const float* dt,
                            const float* A, const void* B, const void* C, const float* D,
                            const float* init_state, void* y, float* final_state,
                            void* workspace, size_t workspace_bytes, Plan* pl, ssd_config* use,
                            ssd::DtXform* xf) {
  if (!prob || !x || !dt || !A || !B || !C || !y || !workspace)
    return fail(SSD_ERR_NULL_POINTER, "prob, x, dt, A, B, C, y and workspace must not be NULL");
  ssd_status st = plan_problem(prob, pl);
  if (st != SSD_OK) return st;
  st = check_dt_transform(dtx, xf);
  if (st != SSD_OK) return st;
  *use = cfg ? *cfg : default_config(*pl);
  st = check_config(*pl, *use);
  if (st != SSD_OK) return st;
  if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) || !aligned16(C) ||
      !aligned16(D) || !aligned16(init_state) || !aligned16(y) || !aligned16(final_state) ||
      !aligned16(workspace) || (dtx && !aligned16(dtx->dt_bias)))
    return fail(SSD_ERR_MISALIGNED, "every tensor pointer must be 16-byte aligned");
  st = check_supported(*pl, use->out_heads);
  if (st != SSD_OK) return st;
  workspace_plan(pl);
  const size_t need = config_bytes(*pl, *use);
  if (workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return SSD_OK;
}

static ssd_status run_fwd(const Plan& pl, const ssd_config& use, const ssd::DtXform* xf,
                          const void* x, const float* dt, const float* A, const void* B,
                          const void* C, const float* D, const float* init_state, void* y,
                          float* final_state, void* workspace, hipStream_t s) {
  if (use.fused) {
    // one kernel; the state handed from chunk to chunk lives in final_state
    // itself when the caller wants it, else in the workspace
    char* ws = static_cast<char*>(workspace);
    float* chain = final_state ? final_state : reinterpret_cast<float*>(ws + pl.chain_off);
    return hip_status(ssd::launch_fused_fwd(x, dt, A, B, C, D, init_state, chain, y,
                                            ws + pl.flags_off, ws, ws + 8, xf, pl.B, pl.L, pl.H,
                                            pl.G, (int)pl.Q, pl.T, next_gen(), s),
                      "fused forward launch");
  }
  ssd_status st = run_states(pl, use, x, dt, A, B, init_state, final_state, nullptr, workspace,
                             xf, s);
  if (st != SSD_OK) return st;
  return run_out(pl, use, x, B, C, D, y, workspace, s);
}

ssd_status ssd_fwd_config(const ssd_problem* prob, const ssd_config* cfg,
                          const ssd_dt_transform* dtx, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          const float* init_state, void* y, float* final_state, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    Plan pl;
    ssd_config use;
    ssd::DtXform xf;
    ssd_status st = check_fwd(prob, cfg, dtx, x, dt, A, B, C, D, init_state, y, final_state,
                              workspace, workspace_bytes, &pl, &use, &xf);
    if (st != SSD_OK) return st;
    return run_fwd(pl, use, dtx ? &xf : nullptr, x, dt, A, B, C, D, init_state, y, final_state,
                   workspace, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_fwd_ex(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                      const float* dt, const float* A, const void* B, const void* C,
                      const float* D, const float* init_state, void* y, float* final_state,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd_config(prob, nullptr, dtx, x, dt, A, B, C, D, init_state, y, final_state,
                        workspace, workspace_bytes, stream);
}

ssd_status ssd_default_config(const ssd_problem* prob, ssd_config* cfg) {
  try {
    if (!prob || !cfg) return fail(SSD_ERR_NULL_POINTER, "prob and cfg must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    st = check_supported(pl);
    if (st != SSD_OK) return st;
    *cfg = default_config(pl);
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_tune(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                    const float* dt, const float* A, const void* B, const void* C, const float* D,
                    const float* init_state, void* y, float* final_state, void* workspace,
                    size_t workspace_bytes, void* stream, int32_t reps, ssd_config* tried,
                    float* tried_ms, int32_t max_tried, int32_t* n_tried, ssd_config* best,
                    float* best_ms) {
  try {
    if (!best || !n_tried) return fail(SSD_ERR_NULL_POINTER, "best and n_tried must not be NULL");
    Plan pl;
    ssd_config use;
    ssd::DtXform xf;
    ssd_status st = check_fwd(prob, nullptr, dtx, x, dt, A, B, C, D, init_state, y, final_state,
                              workspace, workspace_bytes, &pl, &use, &xf);
    if (st != SSD_OK) return st;
    if (reps < 1 || reps > 1000)
      return fail(SSD_ERR_BAD_VALUE, "reps must be in [1, 1000] (got %d)", reps);
    if (init_state && static_cast<const void*>(init_state) == static_cast<const void*>(final_state))
      return fail(SSD_ERR_BAD_VALUE, "tune: init_state must not alias final_state");
    if (max_tried < 0 || (max_tried > 0 && (!tried || !tried_ms)))
      return fail(SSD_ERR_BAD_VALUE, "max_tried must be >= 0, with tried and tried_ms given when > 0");
    if (workspace_bytes < pl.staged_bytes)
      return fail(SSD_ERR_WORKSPACE, "tune: workspace has %zu bytes, the staged kernels need %zu",
                  workspace_bytes, pl.staged_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[2] = {nullptr, nullptr};
    if (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess) {
      if (ev[0]) (void)hipEventDestroy(ev[0]);
      return fail(SSD_ERR_HIP, "tune: event creation failed");
    }
    const ssd::DtXform* xfp = dtx ? &xf : nullptr;
    // the valid choices, in a fixed order: the fused kernel (where built),
    // then every staged combination
    // (the stage-3 choices: head-pair kernel with 2 or 1 heads, resident tile)
    constexpr int kMaxCand = 1 + 3 * 3 * 3;
    ssd_config cand[kMaxCand];
    int n = 0;
    if (pl.fused_ok) {
      ssd_config c = default_config(pl);
      c.fused = 1;
      cand[n++] = c;
    }
    const int okh = ssd::compute_out_default_kh(pl.bf16, pl.H, pl.G, pl.N);
    for (int ch : {0, 4, 16})
      for (int sh : {4, 2, 1})
        for (int out = 0; out < 3; ++out) {
          const int oh = out == 2 ? okh : 2 - out;
          const ssd_config c{ch, sh, oh, 0, out == 2 ? 1 : 0};
          if (check_config(pl, c) == SSD_OK && check_supported(pl, oh) == SSD_OK) cand[n++] = c;
        }
    // mean ms of `reps` runs of choice c between two events (after one untimed run)
    auto time_one = [&](const ssd_config& c, float* ms) -> ssd_status {
      ssd_status r = run_fwd(pl, c, xfp, x, dt, A, B, C, D, init_state, y, final_state, workspace, s);
      if (r == SSD_OK && hipEventRecord(ev[0], s) != hipSuccess)
        r = fail(SSD_ERR_HIP, "tune: event record failed");
      for (int k = 0; k < reps && r == SSD_OK; ++k)
        r = run_fwd(pl, c, xfp, x, dt, A, B, C, D, init_state, y, final_state, workspace, s);
      if (r == SSD_OK && (hipEventRecord(ev[1], s) != hipSuccess ||
                          hipEventSynchronize(ev[1]) != hipSuccess ||
                          hipEventElapsedTime(ms, ev[0], ev[1]) != hipSuccess))
        r = fail(SSD_ERR_HIP, "tune: event timing failed");
      *ms /= (float)reps;
      return r;
    };
    // warm the device up with the default choice, then measure every choice
    // twice, in forward and in reverse order, keeping the smaller mean, so a
    // drift of clocks or caches during the sweep does not favour one end
    float warm = 0.0f, t_ms[kMaxCand];
    st = time_one(use, &warm);
    for (int i = 0; i < n && st == SSD_OK; ++i) st = time_one(cand[i], &t_ms[i]);
    for (int i = n - 1; i >= 0 && st == SSD_OK; --i) {
      float again = 0.0f;
      st = time_one(cand[i], &again);
      if (st == SSD_OK && again < t_ms[i]) t_ms[i] = again;
    }
    float best_t = 0.0f;
    for (int i = 0; i < n && st == SSD_OK; ++i) {
      if (i < max_tried) {
        tried[i] = cand[i];
        tried_ms[i] = t_ms[i];
      }
      if (i == 0 || t_ms[i] < best_t) {
        best_t = t_ms[i];
        *best = cand[i];
      }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (st != SSD_OK) return st;
    *n_tried = n;
    if (best_ms) *best_ms = best_t;
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_fwd(const ssd_problem* prob, const void* x, const float* dt, const float* A,
                   const void* B, const void* C, const float* D, const float* init_state,
                   void* y, float* final_state, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return ssd_fwd_ex(prob, nullptr, x, dt, A, B, C, D, init_state, y, final_state, workspace,
                    workspace_bytes, stream);
}

ssd_status ssd_step(const ssd_problem* prob, const ssd_dt_transform* dtx, float* state,
                    const void* x, const float* dt, const float* A, const void* B, const void* C,
                    const float* D, void* y, void* stream) {
  try {
    if (!prob || !state || !x || !dt || !A || !B || !C || !y)
      return fail(SSD_ERR_NULL_POINTER, "prob, state, x, dt, A, B, C and y must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl, /*need_chunk=*/false);
    if (st != SSD_OK) return st;
    ssd::DtXform xf;
    st = check_dt_transform(dtx, &xf);
    if (st != SSD_OK) return st;
    if (!aligned16(state) || !aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(B) ||
        !aligned16(C) || !aligned16(D) || !aligned16(y) || (dtx && !aligned16(dtx->dt_bias)))
      return fail(SSD_ERR_MISALIGNED, "every tensor pointer must be 16-byte aligned");
    if (pl.P % 16 != 0 || pl.N % 16 != 0)
      return fail(SSD_ERR_UNSUPPORTED, "headdim (%lld) and dstate (%lld) must be multiples of 16",
                  (long long)pl.P, (long long)pl.N);
    if (pl.N > 256) return fail(SSD_ERR_UNSUPPORTED, "dstate must be <= 256 (got %lld)", (long long)pl.N);
    if (pl.H > 65535 || pl.B > 65535 || pl.P > INT32_MAX / 2)
      return fail(SSD_ERR_UNSUPPORTED, "grid too large for this build");
    return hip_status(ssd::launch_step(pl.bf16, state, x, dt, A, B, C, D, y, dtx ? &xf : nullptr,
                                       pl.B, pl.L, pl.H, pl.P, pl.N, pl.G,
                                       static_cast<hipStream_t>(stream)),
                      "step launch");
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_bwd_workspace_size(const ssd_problem* prob, size_t* bytes) {
  try {
    if (!prob || !bytes) return fail(SSD_ERR_NULL_POINTER, "prob and bytes must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    st = check_supported_bwd(pl);
    if (st != SSD_OK) return st;
    *bytes = bwd_default_plan(pl).bytes;
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_bwd_workspace_min_size(const ssd_problem* prob, size_t* bytes) {
  try {
    if (!prob || !bytes) return fail(SSD_ERR_NULL_POINTER, "prob and bytes must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    st = check_supported_bwd(pl);
    if (st != SSD_OK) return st;
    *bytes = bwd_min_bytes(pl);
    return ok();
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

ssd_status ssd_bwd(const ssd_problem* prob, const ssd_dt_transform* dtx, const void* x,
                   const float* dt, const float* A, const void* B, const void* C, const float* D,
                   const float* init_state, const void* dy, const float* dfinal, void* dx,
                   float* ddt, float* dA, void* dB, void* dC, float* dD, float* dinit,
                   float* ddt_bias, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!prob || !x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC ||
        !workspace)
      return fail(SSD_ERR_NULL_POINTER,
                  "prob, x, dt, A, B, C, dy, dx, ddt, dA, dB, dC and workspace must not be NULL");
    Plan pl;
    ssd_status st = plan_problem(prob, &pl);
    if (st != SSD_OK) return st;
    ssd::DtXform xf;
    st = check_dt_transform(dtx, &xf);
    if (st != SSD_OK) return st;
    const void* ptrs[] = {x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD,
                          dinit, ddt_bias, workspace, dtx ? dtx->dt_bias : nullptr};
    for (const void* p : ptrs)
      if (!aligned16(p)) return fail(SSD_ERR_MISALIGNED, "every tensor pointer must be 16-byte aligned");
    st = check_supported_bwd(pl);
    if (st != SSD_OK) return st;
    if (bwd_plan_for(pl, workspace_bytes, 0).hb == 0)
      return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs at least %zu",
                  workspace_bytes, bwd_min_bytes(pl));
    // every argument checked: the device's workgroup slots pick the batching
    const BwdPlan w =
        bwd_plan_for(pl, workspace_bytes, ssd::bwd_chunk_slots(pl.bf16, pl.P, pl.N));
    char* ws = static_cast<char*>(workspace);
    float* Gw = reinterpret_cast<float*>(ws + w.g_off);
    float* dtw = reinterpret_cast<float*>(ws + w.dt_off);
    float* Gz = reinterpret_cast<float*>(ws + w.gz_off);
    float* w2 = reinterpret_cast<float*>(ws + w.w2_off);
    float* Pb = reinterpret_cast<float*>(ws + w.pb_off);
    float* Qb = reinterpret_cast<float*>(ws + w.qb_off);
    void* Hc = ws + w.hc_off;
    void* Lam = ws + w.lam_off;
    float* fin = reinterpret_cast<float*>(ws + w.fin_off);
    float* dBh = reinterpret_cast<float*>(ws + w.dbh_off);
    float* dCh = reinterpret_cast<float*>(ws + w.dch_off);
    float* acB = reinterpret_cast<float*>(ws + w.acb_off);
    float* acC = reinterpret_cast<float*>(ws + w.acc_off);
    double* dAp = reinterpret_cast<double*>(ws + w.dap_off);
    double* dbp = reinterpret_cast<double*>(ws + w.dbp_off);
    float* dDp = reinterpret_cast<float*>(ws + w.ddp_off);
    const ssd::DtXform* xfp = dtx ? &xf : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const ssd_config cfg = default_config(pl);
    // forward stages: running sums, prepared step sizes, chunk-start states
    hipError_t e = ssd::launch_chunk_cumsum(dt, A, Gw, dtw, pl.B, pl.L, pl.H, (int)pl.Q, pl.Lp,
                                            pl.Lp, xfp, kCumsumHeads, s);
    if (e != hipSuccess) return hip_status(e, "chunk_cumsum launch");
    // fp32 states from the io values: for bf16 io the chunk contributions are
    // formed from the exact bf16 inputs with the weighted x split into three
    // bf16 parts (~24 significant bits); for fp32 io on the fp32 MFMA
    auto states = [&](const void* a, const void* bm, float* g, float* wt, void* out) {
      return pl.bf16 ? ssd::launch_chunk_state_split(a, bm, g, wt, static_cast<float*>(out), pl.B,
                                                     pl.L, pl.H, pl.P, pl.N, pl.G, (int)pl.Q,
                                                     pl.T, pl.Lp, cfg.state_heads, s)
                     : ssd::launch_chunk_state(0, a, bm, g, wt, out, pl.B, pl.L, pl.H, pl.P,
                                               pl.N, pl.G, (int)pl.Q, pl.T, pl.Lp, 0,
                                               cfg.state_heads, nullptr, nullptr, nullptr, s);
    };
    e = states(x, B, Gw, dtw, Hc);
    if (e != hipSuccess) return hip_status(e, "chunk_state launch");
    e = ssd::launch_state_pass(0, Hc, Gw, init_state, dfinal ? fin : nullptr, pl.B, pl.H,
                               pl.P, pl.N, (int)pl.Q, pl.T, pl.Lp, 0, 0, s);
    if (e != hipSuccess) return hip_status(e, "state_pass launch");
    // gradients of the chunk-boundary states: the same two stages run backwards
    e = ssd::launch_bwd_prep(Gw, w2, Gz, pl.B, pl.H, pl.L, pl.Lp, s);
    if (e != hipSuccess) return hip_status(e, "bwd_prep launch");
    e = states(dy, C, Gz, w2, Lam);
    if (e != hipSuccess) return hip_status(e, "chunk_state (reverse) launch");
    e = ssd::launch_state_pass(0, Lam, Gw, dfinal, dinit, pl.B, pl.H, pl.P, pl.N, (int)pl.Q,
                               pl.T, pl.Lp, 0, 1, s);
    if (e != hipSuccess) return hip_status(e, "state_pass (reverse) launch");
    // per-chunk gradients, hb parts (of kh heads) at a time, each batch's
    // dB/dC sums folded into the per-group sums before the next batch
    // overwrites them
    for (int p0 = 0; p0 < w.np; p0 += w.hb) {
      const int nb = std::min(w.hb, w.np - p0);
      e = ssd::launch_bwd_chunks(pl.bf16, w.TB, x, B, C, dy, Gw, dtw, Hc, Lam, D, dx, Pb, Qb,
                                 dBh, dCh, dDp, pl.B, pl.L, pl.H, pl.P, pl.N, pl.G, (int)pl.Q,
                                 pl.T, pl.Lp, p0, nb, w.hb, w.kh, s);
      if (e != hipSuccess) return hip_status(e, "bwd chunk kernels launch");
      e = ssd::launch_bwd_group_sum(pl.bf16, dBh, dCh, acB, acC, dB, dC, pl.B, pl.L, w.np, pl.N,
                                    pl.G, p0, nb, w.hb, s);
      if (e != hipSuccess) return hip_status(e, "bwd group sum launch");
    }
    e = ssd::launch_bwd_finish(Pb, Qb, dtw, dt, A, dfinal, fin, xfp, ddt, dAp, dbp, dDp, dA, dD,
                               ddt_bias, pl.B, pl.L, pl.H, pl.P, pl.N, pl.T, pl.Lp, s);
    return hip_status(e, "bwd finish launch");
  } catch (...) {
    return fail(SSD_ERR_INTERNAL, "unexpected exception");
  }
}

}  // extern "C"
