// fwd_pass_state.hip -- stage 2: chunk states and the sequential state pass.
//
// For every (b, h) and chunk c (Q tokens, j = 0..Q-1 inside the chunk):
//     w_j  = exp2(G_last - G_j) * dt_j                  (decay from token j to chunk end)
//     S_c  = sum_j (w_j x_j) (outer) B_j = X_c^T diag(w) B_c          (P x N)
//     H_0  = init_state (or 0),   H_{c+1} = exp2(G_last) * H_c + S_c
// and the output is H_c for every chunk (the state at the chunk start, in the
// io dtype) plus the fp32 state after the last token.  S_c is the jump
// formula: the chunk's effect on the state is a single matrix product over
// its stacked x and B rows (brifing.si "Accelerating Mamba-2 ...", section 4),
// with each row multiplied by its exponential decay before the product so the
// product stays a plain GEMM (same page, section 5).  The loop over chunks is
// sequential inside each workgroup, one state slice per workgroup (devin.kr
// "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section "세 가지 핵심
// 커널 구현", fwd_pass_state; brifing.si, section 8).
//
// Mapping (gfx950): one workgroup of 4 waves owns a 64 (p) x 64 (n) slice of
// one head's state for the whole sequence.  The slice lives in MFMA
// accumulators (fp32) across all chunks: each chunk first stores the current
// state (H_c) through LDS as full 128-byte rows, scales the accumulators by
// exp2(G_last), then accumulates X~^T B with v_mfma_f32_16x16x32_bf16 (K =
// tokens).  Both operands are token-contiguous per lane, so the chunk's x
// (weighted by w_j in fp32, rounded once to the io dtype) and B are written
// to LDS transposed, [feature][token]; each thread transposes an 8-token x
// 8-feature block in registers so every LDS write is 16 bytes.  Wave (wp, wn)
// computes rows 32*wp..+32 and columns 32*wn..+32 (2 x 2 tiles of 16x16).
// The workgroups that share one head's x are placed on the same XCD so the
// second n-slice reads x from that XCD's L2.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kStateThreads = 256;
constexpr int kPT = 64;  // p-slice per workgroup
constexpr int kNT = 64;  // n-slice per workgroup

template <typename T>
struct StateSmem {
  static constexpr int kVec = Vec16<T>::n;      // io elements per 16 bytes
  static constexpr int kPad = 16 / sizeof(T);   // 16-byte row padding
  static constexpr int kQMax = 256;
  static constexpr int kRow = kQMax + kPad;     // [feature][token] row length
  T xs[kPT][kRow];
  T bs[kNT][kRow];
  T hs[kPT][kNT + kPad];
};

// Stage a [Q tokens x 64 features] slab of src (row stride `stride` elements,
// features [f0, f0 + 64) valid below fmax, tokens valid below qv) into
// dst[feature][token] transposed, optionally multiplying row j by w[j].
template <typename T, bool kScale>
__device__ __forceinline__ void stage_transposed(T (*dst)[StateSmem<T>::kRow],
                                                 const T* __restrict__ src, int64_t stride,
                                                 int f0, int fmax, int Q, int qv,
                                                 const float* __restrict__ G,
                                                 const float* __restrict__ dtc, float g_last) {
  constexpr int V = Vec16<T>::n;        // features per 16-byte load
  constexpr int FG = 64 / V;            // feature groups per slab
  const int tasks = (Q / 8) * FG;       // each task: 8 tokens x V features
  for (int task = threadIdx.x; task < tasks; task += kStateThreads) {
    const int fg = task % FG, j8 = task / FG;
    const int f = f0 + fg * V;
    float w[8];
    if (kScale) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j8 * 8 + e;
        w[e] = fast_exp2(g_last - G[j]) * dtc[j];
      }
    }
    T in[8][V];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j8 * 8 + e;
      vec16 v = zero16();
      if (j < qv && f < fmax) v = load16(src + (int64_t)j * stride + f);
      const T* pv = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int k = 0; k < V; ++k) in[e][k] = pv[k];
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
      T out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        out[e] = kScale ? to_io<T>(to_f32(in[e][k]) * w[e]) : in[e][k];
      // 8 tokens of one feature: 16 bytes (bf16) or 32 bytes (fp32)
#pragma unroll
      for (int h = 0; h < 8 / V; ++h) {
        vec16 pk;
        T* pp = reinterpret_cast<T*>(&pk);
#pragma unroll
        for (int e = 0; e < V; ++e) pp[e] = out[h * V + e];
        store16(&dst[fg * V + k][j8 * 8 + h * V], pk);
      }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(kStateThreads)
fwd_pass_state_kernel(const T* __restrict__ x, const T* __restrict__ Bm,
                      const float* __restrict__ Gw, const float* __restrict__ dtw,
                      const float* __restrict__ init_state, float* __restrict__ final_state,
                      T* __restrict__ Hc, int64_t L, int H, int P, int N, int G, int Q, int T_,
                      int64_t ldw, int BH, int NB, int PB, int frag_major) {
  typedef typename FragOf<T>::type frag_t;
  __shared__ StateSmem<T> sm;

  // XCD-aware placement: blocks are dealt round-robin to the 8 XCDs, so the
  // NB*PB slices of one head get ids congruent mod 8 and sit on one XCD.
  const int id = blockIdx.x;
  const int xcd = id % 8, slot = id / 8;
  const int per = NB * PB;
  const int bh = (slot / per) * 8 + xcd;
  if (bh >= BH) return;
  const int nb = slot % per % NB, pb = slot % per / NB;
  const int b = bh / H, h = bh % H, g = h / (H / G);
  const int p0 = pb * kPT, n0 = nb * kNT;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wp = wave / 2, wn = wave % 2;   // wave's 32x32 quadrant
  const int lr = lane % 16, lg = lane / 16;

  // accumulators: tile (tp, tn) of 16x16, lane holds column lr, rows 4lg..4lg+3
  floatx4 acc[2][2];
#pragma unroll
  for (int tp = 0; tp < 2; ++tp)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = p0 + wp * 32 + tp * 16 + lg * 4 + r;
        const int n = n0 + wn * 32 + tn * 16 + lr;
        float v = 0.0f;
        if (init_state && p < P && n < N) v = init_state[((int64_t)bh * P + p) * N + n];
        acc[tp][tn][r] = v;
      }

  const float* Grow = Gw + (int64_t)bh * ldw;
  const float* drow = dtw + (int64_t)bh * ldw;
  const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;

  for (int c = 0; c < T_; ++c) {
    const int64_t t0 = (int64_t)c * Q;
    const int qv = (int)min((int64_t)Q, L - t0);
    const float* Gc = Grow + t0;
    const float* dtc = drow + t0;
    const float g_last = Gc[Q - 1];

    // (1) H_c out: accumulators -> LDS (io dtype) -> 16-byte row stores.
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.hs[wp * 32 + tp * 16 + lg * 4 + r][wn * 32 + tn * 16 + lr] = to_io<T>(acc[tp][tn][r]);
    // (2) stage X~^T and B^T for this chunk
    stage_transposed<T, true>(sm.xs, x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P, xstride,
                              p0, P, Q, qv, Gc, dtc, g_last);
    stage_transposed<T, false>(sm.bs, Bm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N, bstride,
                               n0, N, Q, qv, nullptr, nullptr, 0.0f);
    __syncthreads();
    if (frag_major) {
      // workspace: fragment-major order (see ssd_device.hpp); this tile is p slice
      // pb and the two 32-column steps 2 nb, 2 nb + 1; 512 pieces of 8 elements
      const HcFrag hf = hc_frag(P, N);
      T* hbase = Hc + ((int64_t)bh * T_ + c) * hf.state_elems();
      for (int idx = tid; idx < 512; idx += kStateThreads) {
        const int ln = idx % 64, kk = (idx / 64) % 2, pt = idx / 128;
        const T* src = &sm.hs[pt * 16 + ln % 16][kk * 32 + (ln / 16) * 8];
        T* dst = hbase + hf.offset(pb, pt, 2 * nb + kk, ln);
#pragma unroll
        for (int h2 = 0; h2 < (int)(8 * sizeof(T)) / 16; ++h2)
          store16(dst + h2 * Vec16<T>::n, load16(src + h2 * Vec16<T>::n));
      }
    } else {
      // caller's buffer: [P][N] rows
      constexpr int V = Vec16<T>::n;
      constexpr int RV = kNT / V;            // 16-byte pieces per row
      T* hbase = Hc + ((int64_t)bh * T_ + c) * (int64_t)P * N;
      for (int idx = tid; idx < kPT * RV; idx += kStateThreads) {
        const int pr = idx / RV, piece = idx % RV;
        const int p = p0 + pr, n = n0 + piece * V;
        if (p < P && n < N) store16(hbase + (int64_t)p * N + n, load16(&sm.hs[pr][piece * V]));
      }
    }
    // (3) H_{c+1} = exp2(G_last) H_c + X~^T B
    const float decay = fast_exp2(g_last);
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) acc[tp][tn] *= decay;
    for (int ks = 0; ks < Q / 32; ++ks) {
      frag_t a[2], bb[2];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) a[tp] = load_frag(&sm.xs[wp * 32 + tp * 16 + lr][ks * 32 + lg * 8]);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) bb[tn] = load_frag(&sm.bs[wn * 32 + tn * 16 + lr][ks * 32 + lg * 8]);
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) acc[tp][tn] = mma(acc[tp][tn], a[tp], bb[tn]);
    }
    __syncthreads();
  }

  // final state (fp32)
  if (final_state) {
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = p0 + wp * 32 + tp * 16 + lg * 4 + r;
          const int n = n0 + wn * 32 + tn * 16 + lr;
          if (p < P && n < N) final_state[((int64_t)bh * P + p) * N + n] = acc[tp][tn][r];
        }
  }
}

template <typename T>
hipError_t launch_fwd_pass_state_t(const void* x, const void* Bm, const float* Gw, const float* dtw,
                                   const float* init_state, float* final_state, void* Hc,
                                   int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                   int64_t G, int Q, int64_t T_, int64_t ldw, int frag_major,
                                   hipStream_t stream) {
  const int NB = (int)((N + kNT - 1) / kNT), PB = (int)((P + kPT - 1) / kPT);
  const int64_t BH = batch * H;
  const int64_t groups8 = (BH + 7) / 8;
  const int64_t nblocks = groups8 * 8 * NB * PB;
  hipLaunchKernelGGL(fwd_pass_state_kernel<T>, dim3((unsigned)nblocks), dim3(kStateThreads), 0,
                     stream, static_cast<const T*>(x), static_cast<const T*>(Bm), Gw, dtw,
                     init_state, final_state, static_cast<T*>(Hc), L, (int)H, (int)P, (int)N,
                     (int)G, Q, (int)T_, ldw, (int)BH, NB, PB, frag_major);
  return hipGetLastError();
}

hipError_t launch_fwd_pass_state(int io_bf16, const void* x, const void* Bm, const float* Gw,
                                 const float* dtw, const float* init_state, float* final_state,
                                 void* Hc, int64_t batch, int64_t L, int64_t H, int64_t P,
                                 int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw,
                                 int frag_major, hipStream_t stream) {
  if (io_bf16)
    return launch_fwd_pass_state_t<bf16>(x, Bm, Gw, dtw, init_state, final_state, Hc, batch, L, H,
                                         P, N, G, Q, T_, ldw, frag_major, stream);
  return launch_fwd_pass_state_t<float>(x, Bm, Gw, dtw, init_state, final_state, Hc, batch, L, H,
                                        P, N, G, Q, T_, ldw, frag_major, stream);
}

}  // namespace ssd
