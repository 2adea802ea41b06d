// step.hip -- token-sequential mode: the recurrence advanced one token at a
// time from a resident state (decode).
//
// For every (b, h), with g = h / (H / G), starting from the caller's state s
// and for t = 0 .. L-1:
//     s   = exp(dt_t A_h) s + dt_t x_t (outer) B_t          (P x N, fp32)
//     y_t = s C_t + D_h x_t
// and s is written back in place.  This is the per-token recurrence that the
// chunked pass evaluates in bulk; the pages contrast the two modes (devin.kr
// "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section "Mamba-2
// 아키텍처의 핵심 연산": the output line y_t = c_t^T h_t + D x_t, evaluated
// sequentially at inference and chunk-parallel in training).
//
// Work is elementwise in the state plus one dot product per row, and the state
// (4 P N bytes per head) dominates the bytes moved, so the kernel is a
// streaming kernel: each lane owns E = 8 consecutive n of one row p in
// registers for all L tokens (two 16-byte loads and stores of the state in
// total), a row is spread over R lanes (R = the power of two >= N / E), and the row's
// output is a shuffle sum over those R lanes.  One workgroup of 256 threads
// covers 256 / R rows of one head.  The decay is exp2(dt A log2 e) on the
// hardware exp2, as in the chunked stages.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kStepThreads = 256;

// 8 consecutive io elements as fp32; p is 16-byte aligned.
__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 w = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(w[e]);
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}

// 4 consecutive io elements as fp32; p is 8-byte (bf16) or 16-byte (fp32) aligned.
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  const bf16x4 w = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(w[e]);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = a[e];
}
// E consecutive io elements (E = 4 or a multiple of 8)
template <int E, typename T>
__device__ __forceinline__ void load_e(const T* p, float* v) {
  if constexpr (E == 4) {
    load4(p, v);
  } else {
#pragma unroll
    for (int c = 0; c < E; c += 8) load8(p + c, v + c);
  }
}

template <typename T, int R, bool XF, int E>
__global__ void __launch_bounds__(kStepThreads)
step_kernel(float* __restrict__ state, const T* __restrict__ x, const float* __restrict__ dt,
            const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
            const float* __restrict__ D, T* __restrict__ y, DtXform xf, int64_t L, int H, int P,
            int N, int G, int hpg) {
  constexpr int ROWS = kStepThreads / R;
  const int tid = threadIdx.x;
  const int r = tid % R;
  const int p = blockIdx.x * ROWS + tid / R;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int g = h / hpg;
  const int n0 = E * r;
  const bool row_ok = p < P;
  const bool act = row_ok && n0 < N;   // lanes past N only join the row sums

  float s[E];
  float* sp = state + (((b * H + h) * P + (row_ok ? p : 0)) * (int64_t)N + n0);
  if (act) {
    load_e<E>(sp, s);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = 0.0f;
  }
  const float a2 = A[h] * kLog2e;
  const float Dh = D ? D[h] : 0.0f;

  for (int64_t t = 0; t < L; ++t) {
    const int64_t bt = b * L + t;
    float d = dt[bt * H + h];
    if constexpr (XF) d = dt_prepare(xf, d, h);
    const float alpha = fast_exp2(d * a2);
    const float xv = row_ok ? to_f32(x[(bt * H + h) * P + p]) : 0.0f;
    float bv[E], cv[E];
    if (act) {
      const int64_t off = (bt * G + g) * N + n0;
      load_e<E>(Bm + off, bv);
      load_e<E>(Cm + off, cv);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) bv[e] = cv[e] = 0.0f;
    }
    const float dx = d * xv;
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s[e] = fmaf(alpha, s[e], dx * bv[e]);
      part = fmaf(s[e], cv[e], part);
    }
    // sum over the R lanes of the row (aligned groups of R lanes in a wave)
#pragma unroll
    for (int off = R / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
    if (row_ok && r == 0) y[(bt * H + h) * P + p] = to_io<T>(fmaf(Dh, xv, part));
  }

  if (act) {
#pragma unroll
    for (int c = 0; c < E; c += 4)
      *reinterpret_cast<floatx4*>(sp + c) = floatx4{s[c], s[c + 1], s[c + 2], s[c + 3]};
  }
}

// State elements per lane: 8 (two 16-byte pieces of fp32 state).  At batch
// 128 of the 2.7B shape 8 measured 121-123 us per step; 4 and 16 both ~146 us.
#ifndef SSD_STEP_E
#define SSD_STEP_E 8
#endif
template <typename T, int R>
static void launch_r(float* state, const void* x, const float* dt, const float* A, const void* Bm,
                     const void* Cm, const float* D, void* y, const DtXform* xf, int64_t batch,
                     int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, hipStream_t stream) {
  constexpr int ROWS = kStepThreads / R;
  dim3 grid((unsigned)((P + ROWS - 1) / ROWS), (unsigned)H, (unsigned)batch);
  const T* xt = static_cast<const T*>(x);
  const T* bt = static_cast<const T*>(Bm);
  const T* ct = static_cast<const T*>(Cm);
  T* yt = static_cast<T*>(y);
  const int hpg = (int)(H / G);
  if (xf)
    hipLaunchKernelGGL((step_kernel<T, R, true, SSD_STEP_E>), grid, dim3(kStepThreads), 0, stream, state, xt,
                       dt, A, bt, ct, D, yt, *xf, L, (int)H, (int)P, (int)N, (int)G, hpg);
  else
    hipLaunchKernelGGL((step_kernel<T, R, false, SSD_STEP_E>), grid, dim3(kStepThreads), 0, stream, state, xt,
                       dt, A, bt, ct, D, yt, DtXform{nullptr, 0, 0.0f, 0.0f}, L, (int)H, (int)P,
                       (int)N, (int)G, hpg);
}

template <typename T>
static void launch_t(float* state, const void* x, const float* dt, const float* A, const void* Bm,
                     const void* Cm, const float* D, void* y, const DtXform* xf, int64_t batch,
                     int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, hipStream_t stream) {
  const int64_t need = N / SSD_STEP_E;   // N a multiple of 16, at most 256
  if (need <= 1)
    launch_r<T, 1>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else if (need <= 2)
    launch_r<T, 2>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else if (need <= 4)
    launch_r<T, 4>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else if (need <= 8)
    launch_r<T, 8>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else if (need <= 16)
    launch_r<T, 16>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else if (need <= 32)
    launch_r<T, 32>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else
    launch_r<T, 64>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
}

// Host launcher.  Shapes as in ssd_step: state [batch, H, P, N] fp32 (in
// place), x/y [batch, L, H, P], dt [batch, L, H], B/C [batch, L, G, N];
// N a multiple of 16 and at most 256 (checked by the caller).
hipError_t launch_step(int io_bf16, float* state, const void* x, const float* dt, const float* A,
                       const void* Bm, const void* Cm, const float* D, void* y,
                       const DtXform* xf, int64_t batch, int64_t L, int64_t H, int64_t P,
                       int64_t N, int64_t G, hipStream_t stream) {
  if (io_bf16)
    launch_t<bf16>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  else
    launch_t<float>(state, x, dt, A, Bm, Cm, D, y, xf, batch, L, H, P, N, G, stream);
  return hipGetLastError();
}

}  // namespace ssd
