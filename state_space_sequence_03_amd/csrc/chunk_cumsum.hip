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
// Mapping: one workgroup of 256 threads per (chunk, 16-head tile, batch).
// The [Q tokens x 16 heads] slab of dt is read row by row (16 contiguous
// floats per token) into LDS, then each wave scans 4 heads: every lane sums
// Q/64 consecutive tokens serially, a wave-wide inclusive scan over the lane
// totals (DPP/permute shuffles) adds the carry, and each lane writes its
// tokens contiguously.
//
// Rows are `ld` floats apart in the outputs; tokens in [L, Lw) are padding
// (dt = 0, so G holds the chunk's last running sum), which lets the later
// stages read whole chunks without bounds checks.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kCumsumHeads = 16;
constexpr int kCumsumThreads = 256;

__global__ void __launch_bounds__(kCumsumThreads)
chunk_cumsum_kernel(const float* __restrict__ dt, const float* __restrict__ A,
                    float* __restrict__ G, float* __restrict__ dtT,
                    int64_t L, int H, int Q, int64_t ld, int64_t Lw) {
  __shared__ float tile[256][kCumsumHeads + 1];
  const int c = blockIdx.x;
  const int h0 = blockIdx.y * kCumsumHeads;
  const int64_t b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)c * Q;

  // Coalesced load of the [Q x 16] slab (zero outside [0, L) x [0, H)).
  for (int idx = tid; idx < Q * kCumsumHeads; idx += kCumsumThreads) {
    const int t = idx / kCumsumHeads, hh = idx % kCumsumHeads;
    const int64_t tok = t0 + t;
    const int h = h0 + hh;
    float v = 0.0f;
    if (tok < L && h < H) v = dt[(b * L + tok) * H + h];
    tile[t][hh] = v;
  }
  __syncthreads();

  const int lane = tid % kWave, wave = tid / kWave;
  const int tpl = Q >= kWave ? Q / kWave : 1;      // tokens per lane
  const int first = lane * tpl;                   // first token of this lane
  for (int hh = wave; hh < kCumsumHeads; hh += kCumsumThreads / kWave) {
    const int h = h0 + hh;
    if (h >= H) break;
    const float a2 = A[h] * kLog2e;
    float part[4];
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float v = 0.0f;
      if (k < tpl && first + k < Q) v = tile[first + k][hh] * a2;
      run += v;
      part[k] = run;
    }
    // inclusive scan of lane totals across the wave
    float incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    const float carry = incl - run;
    float* grow = G + ((int64_t)b * H + h) * ld;
    float* drow = dtT + ((int64_t)b * H + h) * ld;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = first + k;
      const int64_t tok = t0 + t;
      if (k < tpl && t < Q && tok < Lw) {
        grow[tok] = carry + part[k];
        drow[tok] = tile[t][hh];
      }
    }
  }
}

// Host launcher.  Q in {32, 64, 128, 256}; grid covers ceil(Lw / Q) chunks.
hipError_t launch_chunk_cumsum(const float* dt, const float* A, float* G, float* dtT,
                               int64_t batch, int64_t L, int64_t H, int Q, int64_t ld,
                               int64_t Lw, hipStream_t stream) {
  const int64_t T = (Lw + Q - 1) / Q;
  dim3 grid((unsigned)T, (unsigned)((H + kCumsumHeads - 1) / kCumsumHeads), (unsigned)batch);
  hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(kCumsumThreads), 0, stream, dt, A, G, dtT,
                     L, (int)H, Q, ld, Lw);
  return hipGetLastError();
}

}  // namespace ssd
