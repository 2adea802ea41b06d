// chunk_cumsum.hip -- stage 1: within-chunk running sum of the decay, base 2.
//
// For every (b, h) and token t of chunk c:
//     G[b, h, t]   = log2(e) * sum_{k=cQ..t} dt[b, k, h] * A[h]
//     dtT[b, h, t] = dt[b, t, h]
// The running sum restarts at every chunk and is kept in base-2 log space so
// that the later stages evaluate every decay with exp2 (devin.kr "NVIDIA CUDA
// Tile로 Mamba-2 순방향 전달 커널 가속화", section "세 가지 핵심 커널 구현",
// chunk_cumsum; brifing.si "Accelerating Mamba-2 ...", section 7).  Both
// outputs are written in [batch, head, token] order so that consumers read a
// chunk's tokens contiguously (devin.kr, section "cuTile 기반 성능 최적화 기법",
// the transposed dt / decay_cumsum layout).
//
// Mapping: one workgroup of 256 threads per (chunk, HT-head tile, batch), HT
// = 4 by default -- small tiles, so that even one batch of a long sequence
// spreads over many more workgroups than the chip has CUs (the kernel is
// latency-bound: 16-head tiles left 1.25 workgroups per CU at the 2.7B shape
// and took 7.8 us against 6.8 us, 11.0 against 7.1 with the step-size
// preparation); HT = 16 is kept as a tuning alternative.  The [Q tokens x HT
// heads] slab of dt arrives as 16-byte loads (4 heads of one token per lane)
// and is transposed through LDS to [head][token].  Each wave then scans HT/4
// heads: a lane takes Q/64 consecutive tokens, sums them serially, a
// wave-wide inclusive scan over the lane totals adds the carry, and the lane
// writes its tokens' G and dt as one vector store each, so a wave writes a
// whole row contiguously.
//
// Rows are `ld` floats apart in the outputs; tokens in [L, Lw) are padding
// (dt = 0, so G holds the chunk's last running sum), which lets the later
// stages read whole chunks without bounds checks.
//
// With XF set, every real token's dt first goes through the optional step-size
// preparation (bias, softplus, clamp; ssd_device.hpp), and both outputs are
// built from the prepared value: the later stages read dt only from dtT.
// Padding tokens are not prepared and stay 0.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kCumsumThreads = 256;

template <int N>
struct FloatVec;
template <> struct FloatVec<1> { typedef float type; };
template <> struct FloatVec<2> { typedef float type __attribute__((ext_vector_type(2))); };
template <> struct FloatVec<4> { typedef float type __attribute__((ext_vector_type(4))); };

template <int Q, bool XF, int HT>
__global__ void __launch_bounds__(kCumsumThreads)
chunk_cumsum_kernel(const float* __restrict__ dt, const float* __restrict__ A,
                    float* __restrict__ G, float* __restrict__ dtT,
                    int64_t L, int H, int64_t ld, int64_t Lw, DtXform xf) {
  constexpr int TPL = Q >= kWave ? Q / kWave : 1;       // tokens per lane
  constexpr int LANES = Q / TPL;                         // lanes holding tokens
  typedef typename FloatVec<TPL>::type vec_t;
  __shared__ __align__(16) float tile[HT][Q + 4];
  const int c = blockIdx.x;
  const int h0 = blockIdx.y * HT;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)c * Q;

  // [Q x HT] slab: lane loads 4 heads of one token (zero outside [0, L) x [0, H))
  const bool full = h0 + HT <= H && (H % 4) == 0;
#pragma unroll
  for (int idx = tid; idx < Q * (HT / 4); idx += kCumsumThreads) {
    const int t = idx / (HT / 4), h4 = (idx % (HT / 4)) * 4;
    const int64_t tok = t0 + t;
    floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tok < L) {
      const float* src = dt + (b * L + tok) * H + h0 + h4;
      if (full) {
        v = *reinterpret_cast<const floatx4*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = h0 + h4 + e < H ? src[e] : 0.0f;
      }
      if constexpr (XF) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (h0 + h4 + e < H) v[e] = dt_prepare(xf, v[e], h0 + h4 + e);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[h4 + e][t] = v[e];
  }
  __syncthreads();

  const int lane = tid % kWave, wave = tid / kWave;
  const int first = lane * TPL;                         // first token of this lane
  const bool vec_ok = ld % TPL == 0;                    // vector stores stay aligned
#pragma unroll
  for (int k = 0; k < HT / (kCumsumThreads / kWave); ++k) {
    const int hh = wave + k * (kCumsumThreads / kWave);
    const int h = h0 + hh;
    if (h >= H) break;
    const float a2 = A[h] * kLog2e;
    float gs[TPL], raw[TPL];
#pragma unroll
    for (int e = 0; e < TPL; ++e) raw[e] = lane < LANES ? tile[hh][first + e] : 0.0f;
    wave_chunk_scan<TPL>(raw, a2, gs, lane);
    const int64_t row = ((int64_t)b * H + h) * ld + t0 + first;
    if (lane < LANES && vec_ok && t0 + first + TPL <= Lw) {
      vec_t g, d;
      if constexpr (TPL == 1) {
        g = gs[0];
        d = raw[0];
      } else {
#pragma unroll
        for (int e = 0; e < TPL; ++e) {
          g[e] = gs[e];
          d[e] = raw[e];
        }
      }
      *reinterpret_cast<vec_t*>(G + row) = g;
      *reinterpret_cast<vec_t*>(dtT + row) = d;
    } else if (lane < LANES) {
      // rows not vector-aligned, or the end of the row: element by element
#pragma unroll
      for (int e = 0; e < TPL; ++e)
        if (t0 + first + e < Lw) {
          G[row + e] = gs[e];
          dtT[row + e] = raw[e];
        }
    }
  }
}

template <int Q, int HT>
static void launch_q(int64_t T, int64_t batch, const float* dt, const float* A, float* G,
                     float* dtT, int64_t L, int H, int64_t ld, int64_t Lw, const DtXform* xf,
                     hipStream_t stream) {
  dim3 grid((unsigned)T, (unsigned)((H + HT - 1) / HT), (unsigned)batch);
  if (xf)
    hipLaunchKernelGGL((chunk_cumsum_kernel<Q, true, HT>), grid, dim3(kCumsumThreads), 0, stream,
                       dt, A, G, dtT, L, H, ld, Lw, *xf);
  else
    hipLaunchKernelGGL((chunk_cumsum_kernel<Q, false, HT>), grid, dim3(kCumsumThreads), 0, stream,
                       dt, A, G, dtT, L, H, ld, Lw, DtXform{nullptr, 0, 0.0f, 0.0f});
}

template <int HT>
static void launch_ht(int Q, int64_t T, int64_t batch, const float* dt, const float* A, float* G,
                      float* dtT, int64_t L, int H, int64_t ld, int64_t Lw, const DtXform* xf,
                      hipStream_t stream) {
  switch (Q) {
    case 16: launch_q<16, HT>(T, batch, dt, A, G, dtT, L, H, ld, Lw, xf, stream); break;
    case 32: launch_q<32, HT>(T, batch, dt, A, G, dtT, L, H, ld, Lw, xf, stream); break;
    case 64: launch_q<64, HT>(T, batch, dt, A, G, dtT, L, H, ld, Lw, xf, stream); break;
    case 128: launch_q<128, HT>(T, batch, dt, A, G, dtT, L, H, ld, Lw, xf, stream); break;
    default: launch_q<256, HT>(T, batch, dt, A, G, dtT, L, H, ld, Lw, xf, stream); break;
  }
}

// Host launcher.  Q in {16, 32, 64, 128, 256}; grid covers ceil(Lw / Q) chunks;
// rows of G and dtT are `ld` floats apart; xf = nullptr: dt used as given;
// heads_tile (4 or 16) is the number of heads per workgroup.
hipError_t launch_chunk_cumsum(const float* dt, const float* A, float* G, float* dtT,
                               int64_t batch, int64_t L, int64_t H, int Q, int64_t ld,
                               int64_t Lw, const DtXform* xf, int heads_tile, hipStream_t stream) {
  const int64_t T = (Lw + Q - 1) / Q;
  if (heads_tile == 16)
    launch_ht<16>(Q, T, batch, dt, A, G, dtT, L, (int)H, ld, Lw, xf, stream);
  else
    launch_ht<4>(Q, T, batch, dt, A, G, dtT, L, (int)H, ld, Lw, xf, stream);
  return hipGetLastError();
}

}  // namespace ssd
