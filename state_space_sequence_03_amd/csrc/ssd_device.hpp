// ssd_device.hpp -- device-side types and MFMA fragment helpers for gfx950.
//
// Fragment convention used by every kernel here: an MFMA "K-step" covers 32
// values of the contraction index k.  Lane l of a wave (64 lanes) holds 8 of
// them for one row (A operand) or one column (B operand): row/col = l % 16,
// k = 8 * (l / 16) + e, e = 0..7.  The 16x16 fp32 accumulator holds, in lane
// l, column l % 16 and rows 4 * (l / 16) + r, r = 0..3.
//
//   bf16: one v_mfma_f32_16x16x32_bf16 per K-step.
//   fp32: eight v_mfma_f32_16x16x4_f32; in the s-th one lane group g = l / 16
//         supplies k = 8g + s, so the eight together cover the same 32 k's.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace ssd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef floatx8 type; };

__device__ __forceinline__ floatx4 mma(floatx4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(floatx4 c, floatx8 a, floatx8 b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

template <typename T> __device__ __forceinline__ T to_io(float v);
template <> __device__ __forceinline__ bf16 to_io<bf16>(float v) { return static_cast<bf16>(v); }
template <> __device__ __forceinline__ float to_io<float>(float v) { return v; }

__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// Hardware base-2 exponential (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log(1 + e^v) as max(v, 0) + log1p(e^{-|v|}): e^{-|v|} <= 1 never
// overflows, and log1p keeps the small values of strongly negative v.
// log1p(w) comes from the hardware base-2 log with Kahan's correction
// (u = 1 + w; log1p(w) = log(u) * w / (u - 1), or w when u rounds to 1;
// D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, Theorem 4), accurate to a few ulps with
// no table or polynomial of its own; the quotient uses the hardware
// reciprocal (1 ulp), since u - 1 is exact.
__device__ __forceinline__ float softplus_f32(float v) {
  const float w = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
  const float u = 1.0f + w;
  const float lp = u == 1.0f ? w
                             : __builtin_amdgcn_logf(u) * (w * __builtin_amdgcn_rcpf(u - 1.0f)) *
                                   0.6931471805599453f;
  return fmaxf(v, 0.0f) + lp;
}

// Optional preparation of the raw step size, applied where dt is first read
// (chunk_cumsum, or the decode step) so that every later stage sees the
// prepared value:  v = dt + bias[h];  v = softplus(v) when asked;
// v = min(max(v, lo), hi).
struct DtXform {
  const float* bias;   // [H] or nullptr
  int softplus;
  float lo, hi;
};
__device__ __forceinline__ float dt_prepare(const DtXform& f, float v, int h) {
  if (f.bias) v += f.bias[h];
  if (f.softplus) v = softplus_f32(v);
  return fminf(fmaxf(v, f.lo), f.hi);
}
// The same with the head's bias already loaded (`bias` is used when f.bias is
// set): identical arithmetic.
__device__ __forceinline__ float dt_prepare_b(const DtXform& f, float v, float bias) {
  if (f.bias) v += bias;
  if (f.softplus) v = softplus_f32(v);
  return fminf(fmaxf(v, f.lo), f.hi);
}

// Within-chunk running sum of one head by one wave, base 2: lane l holds the
// TPL consecutive tokens l*TPL .. l*TPL + TPL - 1 (raw = prepared dt, 0 on
// padding and on lanes past the chunk), and gets
//   g[e] = log2(e) A sum_{k <= l*TPL + e} raw[k]
// as a serial sum over its own tokens plus an inclusive scan of the lane
// totals across the wave.  chunk_cumsum and chunk_state both call it, so the
// running sums are bitwise the same whichever forms them.  The lane scan runs
// on DPP moves: shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes
// whose source lies before the row's start add zero), then each row's total
// broadcast into the next row (row_bcast:15, rows 1 and 3) and the total of
// rows 0-1 into rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_src(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xf, false));
}
template <int TPL>
__device__ __forceinline__ void wave_chunk_scan(const float (&raw)[TPL], float a2, float (&g)[TPL],
                                                int lane) {
  (void)lane;
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < TPL; ++e) {
    run += raw[e] * a2;
    g[e] = run;
  }
  float incl = run;
  incl += dpp_src<0x111, 0xf>(incl);   // row_shr:1
  incl += dpp_src<0x112, 0xf>(incl);   // row_shr:2
  incl += dpp_src<0x114, 0xf>(incl);   // row_shr:4
  incl += dpp_src<0x118, 0xf>(incl);   // row_shr:8
  incl += dpp_src<0x142, 0xa>(incl);   // row_bcast:15 into rows 1, 3
  incl += dpp_src<0x143, 0xc>(incl);   // row_bcast:31 into rows 2, 3
  const float carry = incl - run;
#pragma unroll
  for (int e = 0; e < TPL; ++e) g[e] = carry + g[e];
}

// 16-byte vector of io elements: 8 bf16 or 4 fp32.
typedef uint4 vec16;
template <typename T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

__device__ __forceinline__ vec16 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

template <typename T>
__device__ __forceinline__ vec16 load16(const T* p) { return *reinterpret_cast<const vec16*>(p); }
template <typename T>
__device__ __forceinline__ void store16(T* p, vec16 v) { *reinterpret_cast<vec16*>(p) = v; }

// Store 4 consecutive io elements converted from fp32 (8 bytes bf16, 16 bytes
// fp32); p must be aligned to that size.
template <typename T> __device__ __forceinline__ void store4(T* p, floatx4 v);
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, floatx4 v) {
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(v[e]);
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float* p, floatx4 v) {
  *reinterpret_cast<floatx4*>(p) = v;
}

// Load one fragment (8 consecutive k values) from memory where k is contiguous.
__device__ __forceinline__ bf16x8 load_frag(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ floatx8 load_frag(const float* p) {
  // two 16-byte halves: rows are only guaranteed 16-byte aligned
  const floatx4 lo = *reinterpret_cast<const floatx4*>(p);
  const floatx4 hi = *reinterpret_cast<const floatx4*>(p + 4);
  floatx8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
// A fragment stored lane-contiguously in LDS (the fragment-major order below):
// lane l's 8 values at f + l * sizeof(fragment).
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type lds_frag(const unsigned char* f, int lane);
template <> __device__ __forceinline__ bf16x8 lds_frag<bf16>(const unsigned char* f, int lane) {
  return *reinterpret_cast<const bf16x8*>(f + lane * 16);
}
template <> __device__ __forceinline__ floatx8 lds_frag<float>(const unsigned char* f, int lane) {
  const floatx4 lo = *reinterpret_cast<const floatx4*>(f + lane * 32);
  const floatx4 hi = *reinterpret_cast<const floatx4*>(f + lane * 32 + 16);
  return floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <typename T> __device__ __forceinline__ typename FragOf<T>::type zero_frag() {
  typename FragOf<T>::type z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = static_cast<T>(0.0f);
  return z;
}


// ---- fragment-major chunk-start states -------------------------------------
// The state stage leaves the chunk-start states H_c in the workspace in the
// order compute_out consumes them as MFMA operands, so that every fragment
// load is one contiguous 1 KiB read for the wave.  For chunk state (b, h, c) [P x N],
// 64-row p slice pb, 16-row tile pt, 32-column step ks and lane l, 8
// consecutive elements H[64 pb + 16 pt + l%16][32 ks + 8 (l/16) + e] are stored
// at element offset (((pb * 4 + pt) * KSW + ks) * 64 + l) * 8 of the state.
// Rows past P and columns past N hold zeros or are never read.
__host__ __device__ inline int nk_class(int64_t N) {   // 32-column steps, rounded to 1/2/4/8
  const int nk = (int)((N + 31) / 32);
  return nk <= 1 ? 1 : nk <= 2 ? 2 : nk <= 4 ? 4 : 8;
}
struct HcFrag {
  int PB, KSW;
  __host__ __device__ int64_t state_elems() const { return (int64_t)PB * 4 * KSW * 512; }
  __host__ __device__ int64_t offset(int pb, int pt, int ks, int lane) const {
    return ((((int64_t)pb * 4 + pt) * KSW + ks) * 64 + lane) * 8;
  }
};
__host__ __device__ inline HcFrag hc_frag(int64_t P, int64_t N) {
  HcFrag f;
  f.PB = (int)((P + 63) / 64);
  f.KSW = nk_class(N);     // chunk_state's n slices cover exactly 32 * KSW columns
  return f;
}
// n-slice width of chunk_state: 32 * KSW columns, at most 128 per workgroup
__host__ __device__ inline int state_nw(int64_t N) {
  const int w = 32 * nk_class(N);
  return w < 128 ? w : 128;
}

// ---- token-major LDS tiles -------------------------------------------------
// A tile [token][feature] (row stride `stride` elements) holds operands whose
// contraction index k is the token.  An MFMA fragment needs 8 tokens of one
// feature per lane.  gfx950's transposing LDS read (ds_read_b64_tr_b16) does
// this for 16-bit data: within each 16-lane group, if lane r addresses the 4
// elements at [t0 + r/4][c0 + 4*(r%4)], lane l receives rows t0..t0+3 of
// column c0 + l.  Two such reads give the 8 tokens {ta..ta+3, tb..tb+3}.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x8 frag_tokens(const bf16* tile, int stride, int ta, int tb,
                                              int c0, int lane) {
  const int r = lane & 15;
  const int off = (r >> 2) * stride + c0 + 4 * (r & 3);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + ta * stride + off));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + tb * stride + off));
  bf16x8 f;
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
  return f;
}
// fp32 tiles: eight scalar reads (used only by the fp32 io path).
__device__ __forceinline__ floatx8 frag_tokens(const float* tile, int stride, int ta, int tb,
                                               int c0, int lane) {
  const int c = c0 + (lane & 15);
  floatx8 f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[e] = tile[(ta + e) * stride + c];
    f[4 + e] = tile[(tb + e) * stride + c];
  }
  return f;
}

// ---- direct global -> LDS loads ------------------------------------------------

// s_waitcnt immediate: wait until at most n vector-memory operations of this
// wave are outstanding (expcnt and lgkmcnt fields at their maxima = no wait).
constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | (((n >> 4) & 3) << 14) | (7 << 4) | (0xF << 8);
}

// One direct global->LDS load (global_load_lds_dwordx4): lane l's 16 bytes at
// `gaddr` land at LDS byte address lds + 16 l (lds is wave-uniform, set in M0).
// `lds` is a generic pointer into shared memory: its low 32 bits are the LDS
// byte address (the shared aperture sits on a 4 GiB boundary), which avoids
// an address-space cast.
// Issued as inline assembly so the compiler's wait-count pass does not treat
// every later LDS read as a possible reader of this write (it cannot tell ring
// slots apart and would drain all loads before each read, defeating the
// prefetch); the kernels' own s_waitcnt vmcnt + barrier order the data
// instead.  Vector-memory operations complete in issue order, so loads the
// compiler does not see only make its own waits stricter.
__device__ __forceinline__ void dma16(const void* gaddr, const void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gaddr), "s"(base)
      : "memory", "m0");
}

// A 4-byte direct load: lane i's dword lands at LDS byte lds + 4 i, so one
// instruction gathers 64 values from any addresses into 64 consecutive
// floats (`lds` must be the same for every active lane).
__device__ __forceinline__ void dma4(const void* gaddr, const void* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(gaddr), "s"(base)
      : "memory", "m0");
}

// The same load with a wave-uniform 64-bit base held in SGPRs and a per-lane
// 32-bit byte offset (the instruction's saddr form): a stream that advances
// by whole rows only moves the base, so its per-lane offsets stay in
// registers and no 64-bit address arithmetic is repeated per load.
__device__ __forceinline__ void dma16_so(const void* base, uint32_t off, const void* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  // the builtin returns a signed int: take each half back as uint32_t before
  // widening, or a low word with bit 31 set would sign-extend into the high word
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(bs), "s"(m)
      : "memory", "m0");
}

// Wait for this wave's loads until at most n (0..3) groups of `per` vector
// memory operations remain outstanding (the immediate must be a constant).
// The loads above write LDS behind the compiler's back, so after the wait a
// compiler fence keeps it from moving the LDS reads of that data above it.
template <int per>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * per));
  else if (n == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * per));
  else if (n == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(per));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __asm__ __volatile__("" ::: "memory");
}

// The same wait when `extra` more vector-memory operations (stores) were
// issued after the awaited group: at most n groups of `per` plus `extra`
// remain outstanding.
template <int per, int extra>
__device__ __forceinline__ void wait_groups_plus(int n) {
  if (n >= 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * per + extra));
  else if (n == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * per + extra));
  else if (n == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(per + extra));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(extra));
  __asm__ __volatile__("" ::: "memory");
}

// Where a kernel reports a bounded wait that gave up: the 64-bit status word
// of the workspace header.  A timeout stores (gen << 32) | 1 there, and the
// kernel records gen in the next word, so the host can tell whether the
// latest call on a workspace timed out without the word ever being cleared.
struct StatusRef {
  unsigned long long* word;   // [0] status, [1] gen of the latest call
  unsigned int gen;
};
__device__ __forceinline__ void report_timeout(const StatusRef& s) {
  __hip_atomic_store(s.word, ((unsigned long long)s.gen << 32) | 1ull, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void record_call(const StatusRef& s) {
  __hip_atomic_store(s.word + 1, (unsigned long long)s.gen, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Hand-offs between the waves of one workgroup through LDS counters that
// only grow.  wait_count waits until a counter reaches `target`; the wait is
// bounded: past the bound the wave goes on and reports the timeout in the
// call's status word rather than hang the workgroup (the protocols using it
// cannot deadlock, so a timeout marks a bug).
constexpr int kSpinLimit = 1 << 16;
__device__ __forceinline__ void wait_count(int* ctr, int target, StatusRef flag, int lane) {
  for (int spins = 0;; ++spins) {
    // an atomic (not volatile) load, so it stays an LDS read
    const int v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (v >= target) break;
    if (spins >= kSpinLimit) {
      if (lane == 0) report_timeout(flag);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __asm__ __volatile__("" ::: "memory");
}

// Add one to an LDS counter after this wave's earlier LDS accesses completed.
__device__ __forceinline__ void bump_count(int* ctr, int lane) {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __asm__ __volatile__("" ::: "memory");
}

// Exchange through LDS between lanes of one wave: every LDS access of this
// wave before the call completes before any after it.  The hardware keeps a
// wave's LDS operations in order; the memory clobber keeps the compiler from
// moving LDS loads above earlier LDS stores whose addresses differ per lane
// (which single-thread alias analysis would otherwise allow).
__device__ __forceinline__ void wave_sync() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Host side: raise kernel Kern's dynamic-LDS limit to `bytes` once per
// device.  The attribute belongs to the current device, and launches may come
// from several host threads at once: each device's first launch sets it (a
// repeated set is harmless), a per-kernel bit mask records the devices done.
template <auto Kern>
inline hipError_t ensure_dyn_lds(int bytes) {
  static std::atomic<uint64_t> done{0};   // bit d: device d (devices 0..63)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace ssd
