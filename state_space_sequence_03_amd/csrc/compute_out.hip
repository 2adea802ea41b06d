// compute_out.hip -- stage 3: chunk outputs with everything fused.
//
// For token i of chunk c of head (b, h) (i, j = 0..Q-1 inside the chunk):
//   y_i = sum_{j<=i} (C_i . B_j) exp2(G_i - G_j) dt_j x_j      (intra-chunk interaction)
//       + exp2(G_i) (H_c C_i)                                  (carried-state term)
//       + D_h x_i                                              (skip)
// The three terms are fused in one tiled kernel that keeps the Q x Q
// interaction tile in registers, builds it with the tensor-core product
// C B^T, masks it causally in place from index comparisons, applies the
// decay with exp2 and masks before exponentiating so no positive exponent is
// evaluated (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화",
// section "세 가지 핵심 커널 구현", compute_out; brifing.si "Accelerating
// Mamba-2 ...", sections 9 and 11).  Nothing Q x Q is written to HBM.
//
// gfx950 design.  One workgroup (4 waves) per (b, h, chunk, 64-wide p slice).
// Rows are processed in row blocks of 16*RB tokens, dealt to the 4 waves in a
// snake order so every wave gets the same causal work.  For a row block with
// first row i0, let jl = 32*floor(i0/32) and r = jl - 1 (the token before the
// block's last full 32-token column pair; G_{-1} = 0).  Because decays are
// negative, G is non-increasing, and for j <= r < i
//     exp2(G_i - G_j) = exp2(G_i - G_r) * exp2(G_r - G_j)
// with both factors <= 1.  So:
//   acc  = exp2(G_r) * (C_i . H_c)                       [MFMA over n, then a scalar]
//   acc += sum_{j<jl} (C_i.B_j) * W_r[j] * x_j          W_r[j] = exp2(G_r - G_j) dt_j from LDS
//   acc *= exp2(G_i - G_r)                               [one exp2 per row]
//   acc += sum_{jl<=j<=i} (C_i.B_j) exp2(G_i - G_j) dt_j x_j   [32-wide band, masked exp2]
// which is the definition above regrouped; the per-element exp2 is only
// evaluated on the 32-token band next to the diagonal.  The skip term D_h x_i
// is added to the diagonal of the interaction tile (S_ii += D_h), so x is not
// read a second time.
//
// MFMA chaining: the interaction tile is produced transposed, S^T = B C^T
// (A operand = B rows, B operand = C rows, both contiguous along n), so each
// lane ends up holding one row i and 4+4 token columns j -- exactly an A
// operand of the next v_mfma_f32_16x16x32_bf16 once the 32 tokens of a pair of
// 16-token blocks are taken in the order {4g..4g+3, 16+4g..16+4g+3} for lane
// group g.  x is staged in LDS transposed ([p][token]) in that same token
// order, so the B operand of S x is one 16-byte read.  The tile never leaves
// registers between the two products.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kOutThreads = 256;
constexpr int kOutP = 64;     // p slice per workgroup

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token held at permuted position k (0..31) of a 32-token pair: position
// 8g + e holds token 4g + e for e < 4 and 16 + 4g + (e - 4) for e >= 4.
__device__ __forceinline__ int pair_token(int k) {
  const int g = k >> 3, e = k & 7;
  return (e < 4) ? (4 * g + e) : (16 + 4 * g + (e - 4));
}

struct OutLayout {
  int xrow, hrow, yrow;     // row lengths (elements)
  int xs_off, hs_off, g_off, d_off, w_off, ys_off, bytes;
};

template <typename T>
__host__ __device__ inline OutLayout out_layout(int Q, int NK, int RB) {
  OutLayout o;
  const int pad = 16 / (int)sizeof(T);
  o.xrow = Q + pad;
  o.hrow = 32 * NK + pad;
  o.yrow = kOutP + pad;
  int off = 0;
  o.xs_off = off; off += kOutP * o.xrow * (int)sizeof(T);
  o.hs_off = off; off += kOutP * o.hrow * (int)sizeof(T);
  o.g_off = off;  off += Q * 4;
  o.d_off = off;  off += Q * 4;
  o.w_off = off;  off += (Q / 32) * Q * 4;
  o.ys_off = off; off += 4 * 16 * RB * o.yrow * (int)sizeof(T);
  o.bytes = off;
  return o;
}

template <typename T, int NK, int RB>
__global__ void __launch_bounds__(kOutThreads)
compute_out_kernel(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                   const float* __restrict__ Gw, const float* __restrict__ dtw,
                   const T* __restrict__ Hc, const float* __restrict__ Dv, T* __restrict__ y,
                   int64_t L, int H, int P, int N, int G, int Q, int T_, int64_t ldw,
                   int nbc, int PB) {
  typedef typename FragOf<T>::type frag_t;
  constexpr int V = Vec16<T>::n;
  extern __shared__ __align__(16) unsigned char smem[];
  const OutLayout lay = out_layout<T>(Q, NK, RB);
  T* xs = reinterpret_cast<T*>(smem + lay.xs_off);
  T* hs = reinterpret_cast<T*>(smem + lay.hs_off);
  float* Gs = reinterpret_cast<float*>(smem + lay.g_off);
  float* ds = reinterpret_cast<float*>(smem + lay.d_off);
  float* Ws = reinterpret_cast<float*>(smem + lay.w_off);
  T* ysall = reinterpret_cast<T*>(smem + lay.ys_off);

  // XCD-aware placement: every head and p slice of one (b, chunk) gets block
  // ids congruent mod 8, so they run on one XCD and share its L2 copy of the
  // chunk's B and C rows.
  const int id = blockIdx.x;
  const int xcd = id % 8, slot = id / 8;
  const int per = H * PB;
  const int bc = (slot / per) * 8 + xcd;
  if (bc >= nbc) return;
  const int hp = slot % per;
  const int h = hp / PB, pb = hp % PB;
  const int b = bc / T_, c = bc % T_;
  const int g = h / (H / G);
  const int p0 = pb * kOutP;
  const int64_t t0 = (int64_t)c * Q;
  const int qv = (int)min((int64_t)Q, L - t0);
  const int bh = b * H + h;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
  const T* xc = x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
  const T* Bc = Bm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;
  const T* Cc = Cm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;
  const float d_h = Dv ? Dv[h] : 0.0f;

  // ---- stage G, dt, x^T (permuted), H_c slice, W table --------------------
  const float* Grow = Gw + (int64_t)bh * ldw + t0;
  const float* drow = dtw + (int64_t)bh * ldw + t0;
  for (int j = tid; j < Q; j += kOutThreads) { Gs[j] = Grow[j]; ds[j] = drow[j]; }
  {
    constexpr int FG = kOutP / V;
    const int tasks = (Q / 8) * FG;
    for (int task = tid; task < tasks; task += kOutThreads) {
      const int fg = task % FG, k8 = task / FG;     // k8: 8 permuted positions
      const int f = p0 + fg * V;
      const int pair = k8 / 4;
      T in[8][V];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = pair * 32 + pair_token((k8 % 4) * 8 + e);
        vec16 v = zero16();
        if (j < qv && f < P) v = load16(xc + (int64_t)j * xstride + f);
        const T* pv = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int k = 0; k < V; ++k) in[e][k] = pv[k];
      }
#pragma unroll
      for (int k = 0; k < V; ++k) {
#pragma unroll
        for (int hh = 0; hh < 8 / V; ++hh) {
          vec16 pk;
          T* pp = reinterpret_cast<T*>(&pk);
#pragma unroll
          for (int e = 0; e < V; ++e) pp[e] = in[hh * V + e][k];
          store16(xs + (fg * V + k) * lay.xrow + k8 * 8 + hh * V, pk);
        }
      }
    }
  }
  {
    const T* hsrc = Hc + ((int64_t)bh * T_ + c) * (int64_t)P * N;
    const int RV = (32 * NK) / V;                  // 16-byte pieces per hs row
    for (int idx = tid; idx < kOutP * RV; idx += kOutThreads) {
      const int pr = idx / RV, piece = idx % RV;
      const int p = p0 + pr, n = piece * V;
      vec16 v = zero16();
      if (p < P && n < N) v = load16(hsrc + (int64_t)p * N + n);
      store16(hs + pr * lay.hrow + n, v);
    }
  }
  __syncthreads();
  {
    const int NQ = Q / 32;
    for (int idx = tid; idx < NQ * Q; idx += kOutThreads) {
      const int q = idx / Q, j = idx % Q;
      float w = 0.0f;
      if (q >= 1 && j < 32 * q) w = fast_exp2(Gs[32 * q - 1] - Gs[j]) * ds[j];
      Ws[idx] = w;
    }
  }
  __syncthreads();

  T* ys = ysall + wave * (16 * RB) * lay.yrow;
  const int NRB = Q / (16 * RB);
  const int npt = min(4, (P - p0 + 15) / 16);   // valid 16-wide p tiles

  for (int k = 0; 4 * k < NRB; ++k) {
    const int rb = (k % 2 == 0) ? 4 * k + wave : 4 * k + 3 - wave;
    if (rb >= NRB) continue;
    const int i0 = rb * 16 * RB;
    if (i0 >= qv) continue;
    const int jl = (i0 / 32) * 32;
    const int q = jl / 32;
    const float g_ref = jl > 0 ? Gs[jl - 1] : 0.0f;

    // C rows of this block as fragments (A operand for C H^T, B operand for B C^T)
    frag_t cf[RB][NK];
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const int i = i0 + ib * 16 + lr, n = ks * 32 + lg * 8;
        cf[ib][ks] = (i < qv && n < N) ? load_frag(Cc + (int64_t)i * bstride + n) : zero_frag<T>();
      }

    // carried-state term
    floatx4 acc[RB][4];
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[ib][pt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt >= npt) break;
        const frag_t hf = load_frag(hs + (pt * 16 + lr) * lay.hrow + ks * 32 + lg * 8);
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) acc[ib][pt] = mma(acc[ib][pt], cf[ib][ks], hf);
      }
    if (jl > 0) {
      const float sref = fast_exp2(g_ref);
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ib][pt] *= sref;
    }

    // off-diagonal token pairs: S = (C B^T) * W_r, rounded once, times x
    const float* Wq = Ws + q * Q;
    for (int jp = 0; jp < q; ++jp) {
      floatx4 s[RB][2];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) { s[ib][0] = floatx4{0.f, 0.f, 0.f, 0.f}; s[ib][1] = s[ib][0]; }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const int n = ks * 32 + lg * 8;
        frag_t b0 = zero_frag<T>(), b1 = zero_frag<T>();
        if (n < N) {
          b0 = load_frag(Bc + (int64_t)(jp * 32 + lr) * bstride + n);
          b1 = load_frag(Bc + (int64_t)(jp * 32 + 16 + lr) * bstride + n);
        }
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) {
          s[ib][0] = mma(s[ib][0], b0, cf[ib][ks]);
          s[ib][1] = mma(s[ib][1], b1, cf[ib][ks]);
        }
      }
      const floatx4 w0 = *reinterpret_cast<const floatx4*>(Wq + jp * 32 + 4 * lg);
      const floatx4 w1 = *reinterpret_cast<const floatx4*>(Wq + jp * 32 + 16 + 4 * lg);
      frag_t af[RB];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          af[ib][r] = to_io<T>(s[ib][0][r] * w0[r]);
          af[ib][4 + r] = to_io<T>(s[ib][1][r] * w1[r]);
        }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt >= npt) break;
        const frag_t xf = load_frag(xs + (pt * 16 + lr) * lay.xrow + jp * 32 + lg * 8);
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) acc[ib][pt] = mma(acc[ib][pt], af[ib], xf);
      }
    }

    // row scale exp2(G_i - G_r); lane rows are i = i0 + 16 ib + 4 lg + r
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = fast_exp2(Gs[i0 + ib * 16 + 4 * lg + r] - g_ref);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ib][pt][r] *= u;
      }

    // band next to the diagonal: tokens jl..jl+31, masked exp2 per element
    {
      floatx4 s[RB][2];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) { s[ib][0] = floatx4{0.f, 0.f, 0.f, 0.f}; s[ib][1] = s[ib][0]; }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const int n = ks * 32 + lg * 8;
        frag_t b0 = zero_frag<T>(), b1 = zero_frag<T>();
        if (n < N) {
          if (jl + lr < qv) b0 = load_frag(Bc + (int64_t)(jl + lr) * bstride + n);
          if (jl + 16 + lr < qv) b1 = load_frag(Bc + (int64_t)(jl + 16 + lr) * bstride + n);
        }
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) {
          // a 16-token block that starts after the row block's last row is fully masked
          s[ib][0] = mma(s[ib][0], b0, cf[ib][ks]);
          if (jl + 16 <= i0 + ib * 16 + 15) s[ib][1] = mma(s[ib][1], b1, cf[ib][ks]);
        }
      }
      frag_t af[RB];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) {
        const int i = i0 + ib * 16 + lr;
        const float gi = Gs[i];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = jl + 16 * t + 4 * lg + r;
            float v = 0.0f;
            if (j <= i) {
              v = s[ib][t][r] * (fast_exp2(gi - Gs[j]) * ds[j]);
              if (j == i) v += d_h;
            }
            af[ib][4 * t + r] = to_io<T>(v);
          }
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt >= npt) break;
        const frag_t xf = load_frag(xs + (pt * 16 + lr) * lay.xrow + q * 32 + lg * 8);
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) acc[ib][pt] = mma(acc[ib][pt], af[ib], xf);
      }
    }

    // store: accumulators -> LDS (io dtype) -> 16-byte row pieces
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ys[(ib * 16 + 4 * lg + r) * lay.yrow + pt * 16 + lr] = to_io<T>(acc[ib][pt][r]);
    wave_sync();
    {
      constexpr int RV = kOutP / V;
      for (int idx = lane; idx < 16 * RB * RV; idx += kWave) {
        const int rr = idx / RV, piece = idx % RV;
        const int i = i0 + rr, p = p0 + piece * V;
        if (i < qv && p < P)
          store16(y + (((int64_t)b * L + t0 + i) * H + h) * P + p, load16(ys + rr * lay.yrow + piece * V));
      }
    }
    wave_sync();
  }
}

template <typename T, int NK, int RB>
static hipError_t launch_out_nk(const void* x, const void* Bm, const void* Cm, const float* Gw,
                                const float* dtw, const void* Hc, const float* Dv, void* y,
                                int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                int64_t G, int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
  const OutLayout lay = out_layout<T>(Q, NK, RB);
  const int PB = (int)((P + kOutP - 1) / kOutP);
  const int64_t nbc = batch * T_;
  const int64_t nblocks = ((nbc + 7) / 8) * 8 * H * PB;
  auto kern = compute_out_kernel<T, NK, RB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lay.bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(kOutThreads), lay.bytes, stream,
                     static_cast<const T*>(x), static_cast<const T*>(Bm), static_cast<const T*>(Cm),
                     Gw, dtw, static_cast<const T*>(Hc), Dv, static_cast<T*>(y), L, (int)H, (int)P,
                     (int)N, (int)G, Q, (int)T_, ldw, (int)nbc, PB);
  return hipGetLastError();
}

template <typename T, int RB>
static hipError_t launch_out_rb(const void* x, const void* Bm, const void* Cm, const float* Gw,
                                const float* dtw, const void* Hc, const float* Dv, void* y,
                                int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                int64_t G, int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
  const int64_t nk = (N + 31) / 32;
  if (nk <= 1) return launch_out_nk<T, 1, RB>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
  if (nk <= 2) return launch_out_nk<T, 2, RB>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
  if (nk <= 4) return launch_out_nk<T, 4, RB>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
  return launch_out_nk<T, 8, RB>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
}

int compute_out_rows_per_block(int Q) { return Q >= 256 ? 2 : 1; }

int compute_out_smem_bytes(int io_bf16, int Q, int64_t N) {
  const int nk = (int)((N + 31) / 32);
  const int NK = nk <= 1 ? 1 : nk <= 2 ? 2 : nk <= 4 ? 4 : 8;
  const int RB = compute_out_rows_per_block(Q);
  return io_bf16 ? out_layout<bf16>(Q, NK, RB).bytes : out_layout<float>(Q, NK, RB).bytes;
}

hipError_t launch_compute_out(int io_bf16, const void* x, const void* Bm, const void* Cm,
                              const float* Gw, const float* dtw, const void* Hc, const float* Dv,
                              void* y, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
  const int RB = compute_out_rows_per_block(Q);
  if (io_bf16) {
    if (RB == 2) return launch_out_rb<bf16, 2>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
    return launch_out_rb<bf16, 1>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
  }
  if (RB == 2) return launch_out_rb<float, 2>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
  return launch_out_rb<float, 1>(x, Bm, Cm, Gw, dtw, Hc, Dv, y, batch, L, H, P, N, G, Q, T_, ldw, stream);
}

}  // namespace ssd
