// state_pass.hip -- stage 2b: the sequential state recurrence across chunks.
//
// For every (b, h):   H_0 = init_state (or 0),
//                     H_{c+1} = exp2(G_last(c)) * H_c + S_c,
// where S_c is chunk c's own contribution (chunk_state.hip) and G_last(c) the
// log2-space decay sum over chunk c, so exp2(G_last(c)) is the chunk's total
// decay.  The buffer holding S_c on entry holds H_c (the state at the start of
// chunk c, in the io dtype) on exit; the fp32 state after the last token is
// the final state (brifing.si "Accelerating Mamba-2 ...", section 8; devin.kr
// "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section "세 가지 핵심 커널
// 구현", fwd_pass_state).
//
// With `reverse` set the chunks are visited last to first: then the buffer
// holding S'_c on entry holds, for chunk c, the carry before S'_c is added,
// i.e. L_{c+1} of  L_c = exp2(G_last(c)) * L_{c+1} + S'_c  started from
// `init_state` after the last chunk, and the fp32 carry after the first chunk
// goes to `final_state`.  That is the backward pass's recurrence for the
// gradient of the chunk-boundary states (bwd.hip).
//
// The recurrence is elementwise in the state, so every thread owns 8
// consecutive elements of one head's state (one 16-byte piece in bf16) for
// all chunks, keeps them in fp32 registers, and streams the chunks: the loads
// of S_c do not depend on the recurrence and are issued kSpAhead chunks ahead.
// The element order is whatever order chunk_state wrote (fragment-major for
// the workspace, [P][N] for a caller's buffer); only the initial and final
// states, always [P][N] fp32, need the (p, n) of a piece.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kSpThreads = 256;
constexpr int kSpAhead = 8;     // chunks in flight per thread

template <typename T>
struct Piece8 {                  // 8 io elements
  vec16 v[(8 * sizeof(T)) / 16];
};

template <typename T>
__device__ __forceinline__ Piece8<T> load_piece(const T* p) {
  Piece8<T> r;
#pragma unroll
  for (int i = 0; i < (int)(8 * sizeof(T)) / 16; ++i) r.v[i] = load16(p + i * Vec16<T>::n);
  return r;
}

template <typename T>
__global__ void __launch_bounds__(kSpThreads)
state_pass_kernel(T* __restrict__ S, const float* __restrict__ Gw, const float* __restrict__ init_state,
                  float* __restrict__ final_state, int H, int P, int N, int Q, int T_, int64_t ldw,
                  int64_t SE, int frag_major, int reverse) {
  const int nbs = (int)((SE / 8 + kSpThreads - 1) / kSpThreads);   // blocks per state
  const int bh = blockIdx.x / nbs;
  const int64_t q = (int64_t)(blockIdx.x % nbs) * kSpThreads + threadIdx.x;   // piece index
  if (8 * q >= SE) return;
  // (p, n0) of the piece
  int p, n0;
  if (frag_major) {
    const HcFrag hf = hc_frag(P, N);
    const int ln = (int)(q % 64), ks = (int)(q / 64 % hf.KSW), pt = (int)(q / 64 / hf.KSW % 4);
    const int pb = (int)(q / 64 / hf.KSW / 4);
    p = pb * 64 + pt * 16 + ln % 16;
    n0 = ks * 32 + (ln / 16) * 8;
  } else {
    p = (int)(8 * q / N);
    n0 = (int)(8 * q % N);
  }
  const bool valid = p < P && n0 < N;
  float h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = 0.0f;
  if (init_state && valid) {
    const float* src = init_state + ((int64_t)bh * P + p) * N + n0;
    const floatx4 a = *reinterpret_cast<const floatx4*>(src);
    const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { h[e] = a[e]; h[4 + e] = b[e]; }
  }
  T* base = S + (int64_t)bh * T_ * SE + 8 * q;
  const float* glast = Gw + (int64_t)bh * ldw + (Q - 1);

  for (int c0 = 0; c0 < T_; c0 += kSpAhead) {
    // issue every load of this batch before using any of it
    Piece8<T> in[kSpAhead];
    float dec[kSpAhead];
#pragma unroll
    for (int k = 0; k < kSpAhead; ++k) {
      int c = min(c0 + k, T_ - 1);
      if (reverse) c = T_ - 1 - c;
      in[k] = load_piece<T>(base + (int64_t)c * SE);
      dec[k] = glast[(int64_t)c * Q];
    }
#pragma unroll
    for (int k = 0; k < kSpAhead; ++k) {
      if (c0 + k < T_) {
        Piece8<T> out;
        T* o = reinterpret_cast<T*>(out.v);
        const T* s = reinterpret_cast<const T*>(in[k].v);
        const float a = fast_exp2(dec[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = to_io<T>(h[e]);
          h[e] = a * h[e] + to_f32(s[e]);
        }
        T* dst = base + (int64_t)(reverse ? T_ - 1 - (c0 + k) : c0 + k) * SE;
#pragma unroll
        for (int i = 0; i < (int)(8 * sizeof(T)) / 16; ++i) store16(dst + i * Vec16<T>::n, out.v[i]);
      }
    }
  }
  if (final_state && valid) {
    float* dst = final_state + ((int64_t)bh * P + p) * N + n0;
    *reinterpret_cast<floatx4*>(dst) = floatx4{h[0], h[1], h[2], h[3]};
    *reinterpret_cast<floatx4*>(dst + 4) = floatx4{h[4], h[5], h[6], h[7]};
  }
}

hipError_t launch_state_pass(int io_bf16, void* S, const float* Gw, const float* init_state,
                             float* final_state, int64_t batch, int64_t H, int64_t P, int64_t N,
                             int Q, int64_t T_, int64_t ldw, int frag_major, int reverse,
                             hipStream_t stream) {
  const int64_t SE = frag_major ? hc_frag(P, N).state_elems() : P * N;
  const int64_t pieces = SE / 8;
  const dim3 grid((unsigned)((pieces + kSpThreads - 1) / kSpThreads * batch * H));
  if (io_bf16)
    hipLaunchKernelGGL(state_pass_kernel<bf16>, grid, dim3(kSpThreads), 0, stream,
                       static_cast<bf16*>(S), Gw, init_state, final_state, (int)H, (int)P, (int)N,
                       Q, (int)T_, ldw, SE, frag_major, reverse);
  else
    hipLaunchKernelGGL(state_pass_kernel<float>, grid, dim3(kSpThreads), 0, stream,
                       static_cast<float*>(S), Gw, init_state, final_state, (int)H, (int)P, (int)N,
                       Q, (int)T_, ldw, SE, frag_major, reverse);
  return hipGetLastError();
}

}  // namespace ssd
