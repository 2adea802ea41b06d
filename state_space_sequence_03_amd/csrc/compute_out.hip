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
// gfx950 design.  One workgroup (4 waves) per (b, chunk, KH heads of one
// group, 64-wide p slice, 128-row part of the chunk).  Heads of one group share
// C, B and therefore the raw tile C B^T, which is computed once for all KH
// heads; only the decay, x, the carried state and the accumulators are per
// head.  Its rows are split into 16-row blocks dealt to
// the waves in a snake order (wave w owns blocks w and 7-w of the part) so
// causal work is balanced; each wave keeps its blocks' C rows (as MFMA
// fragments) and output accumulators in registers for the whole chunk.  The
// workgroup streams the chunk's tokens in pairs of 16-token blocks through a
// ring of LDS slots filled by asynchronous direct global->LDS loads issued
// several pairs ahead (global memory latency under load is far longer than
// one pair's compute); the waves hand slots to each other through LDS
// counters rather than a barrier per pair (see wait_count below).
//
// Decay factorisation.  For a row block starting at i0, let jl = 32*floor(i0/32)
// and r = jl - 1 (G_{-1} = 0).  Decays are negative, so G is non-increasing and
// for j <= r < i
//     exp2(G_i - G_j) = exp2(G_i - G_r) * exp2(G_r - G_j),   both factors <= 1.
// So the accumulator starts as exp2(G_r) (C_i . H_c), every pair p left of jl
// adds (C_i . B_j) exp2(G_r - G_j) dt_j x_j, where the weight is the product of
// a per-token table e_j = exp2(G_e - G_j) dt_j (G_e = running sum at the pair's
// last token e) and one scalar exp2(G_r - G_e) per (block, pair) -- both <= 1;
// at the block's own pair (the band) the accumulator is scaled by
// exp2(G_i - G_r) per row and the band adds the masked per-element
// exp2(G_i - G_j) dt_j terms.  This is the definition above regrouped; exp2 per
// tile element is evaluated only on the 32-token band, and no factor exceeds 1.
// The skip term D_h x_i rides on the tile's diagonal (S_ii += D_h).
//
// MFMA chaining: the tile is produced transposed, S^T = B C^T (A operand = B
// rows, B operand = C rows, both contiguous along n), so each lane ends up
// holding one row i and the 4+4 token columns {4g..4g+3, 16+4g..16+4g+3} of a
// token pair -- exactly an A operand of the next v_mfma_f32_16x16x32_bf16 when
// the pair's tokens are taken in that order.  The matching x operand (8 tokens
// of one p column per lane) comes from the natural-layout x tile through two
// transposing LDS reads.  The tile never leaves registers between the two
// products.  The output product takes the x fragment as its first operand
// (y^T = x^T S^T), so each lane's accumulator holds 4 consecutive p of its
// row i, the band's row rescale is one scalar per lane, and finished rows are
// stored straight from the accumulators.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kOutThreads = 256;
constexpr int kOutWaves = kOutThreads / kWave;
constexpr int kOutP = 64;     // p slice per workgroup
constexpr int kOutStaticLds = 256;   // bound on the kernel's static LDS (the slot counters)

// Waves of a workgroup hand ring slots to each other through LDS counters
// (wait_count / bump_count) instead of a barrier per token pair, so a wave
// that finishes a pair early (no band block in it) moves on to the next one
// while another still works on its band.  Each slot has an arrival count
// (one per wave whose share of the slot's loads has landed) and a release
// count (one per wave done reading it); both only grow, by kOutWaves per use
// of the slot.

// One ring slot holds a token pair (32 tokens): B rows over all of n (padded
// to 32*NK columns) and, for each of the KH heads, x rows over the
// workgroup's 64 p columns, all in natural [token][feature] order, filled by
// gfx950's direct global->LDS loads (global_load_lds_dwordx4: lane l's 16
// bytes land at the wave-uniform LDS base + 16*l, from any global address).
// 16-byte chunks are XOR-swizzled per row so fragment reads hit distinct banks.
template <typename T, int NK, int KH>
struct Slot {
  static constexpr int V = Vec16<T>::n;                        // elements per chunk
  static constexpr int BC = 32 * NK / V;                       // chunks per B row
  static constexpr int BCH = 32 * BC;                          // B chunks per slot
  static constexpr int XC = kOutP / V;                         // chunks per x row
  static constexpr int XCH = 32 * XC;                          // x chunks per head
  static constexpr int BYTES = (BCH + KH * XCH) * 16;
  static constexpr int BINST = (BCH + kOutThreads - 1) / kOutThreads;   // per wave per pair
  static constexpr int XINST = (XCH + kOutThreads - 1) / kOutThreads;   // per wave, head, pair
  static constexpr int LPG = BINST + KH * XINST;               // load instructions per wave per pair
  static constexpr int BSW = BC < 16 ? BC - 1 : 15;
  static_assert(BCH % 64 == 0 && XCH % 64 == 0, "slot parts must be whole 64-chunk blocks");
#ifdef SSD_OUT_FORCE_NSLOT
  static constexpr int NSLOT = SSD_OUT_FORCE_NSLOT;
#else
  static constexpr int NSLOT = BYTES <= 16 * 1024 ? 4 : BYTES <= 28 * 1024 ? 3 : 2;
#endif
  static_assert(NSLOT >= 2 && NSLOT <= 4, "the drain-time waits cover up to two pairs ahead");
  __device__ static int bsw(int r) { return r & BSW; }
  __device__ static int xsw(int r) { return ((r >> 1) & 3) << 1; }
  // byte offsets (within a slot) of element (row r, column col) of B / of head k's x
  __device__ static int boff(int r, int col) {
    return (r * BC + ((col / V) ^ bsw(r))) * 16 + (col % V) * (int)sizeof(T);
  }
  __device__ static int xoff(int k, int r, int col) {
    return (BCH + k * XCH + r * XC + ((col / V) ^ xsw(r))) * 16 + (col % V) * (int)sizeof(T);
  }
};

struct OutLayout {
  int g_off, d_off, e_off, ring_off, bytes, slot_bytes, nslot;
};

template <typename T, int NK, int KH>
__host__ __device__ inline OutLayout out_layout(int Q) {
  OutLayout o;
  o.slot_bytes = Slot<T, NK, KH>::BYTES;
  o.nslot = Slot<T, NK, KH>::NSLOT;
  int off = 0;
  o.g_off = off; off += KH * Q * 4;
  o.d_off = off; off += KH * Q * 4;
  o.e_off = off; off += KH * Q * 4;
  o.ring_off = off; off += o.nslot * o.slot_bytes;
  o.bytes = off;
  return o;
}

// Issue the direct-to-LDS loads of token pair `jp` into `slot`.  Every wave
// issues exactly Slot::LPG instructions (a wave with no block of its own
// reloads an existing block with identical data), so one vmcnt target is
// exact for all waves.  Rows past the chunk's valid tokens and columns past
// N or P read clamped, valid addresses; those values only meet masked tile
// entries, zero C columns or unstored outputs.
template <typename T, int NK, int KH>
__device__ __forceinline__ void issue_pair(unsigned char* slot, const T* __restrict__ Bc,
                                           int64_t bstride, int N, const T* __restrict__ xc,
                                           int64_t xstride, int64_t hstep, int p0, int P, int jp,
                                           int qv, int wave, int lane) {
  typedef Slot<T, NK, KH> S;
  constexpr int V = S::V;
  constexpr int NBB = S::BCH / 64, NXB = S::XCH / 64;   // 64-chunk blocks (whole)
#pragma unroll
  for (int k = 0; k < S::BINST; ++k) {
    const int blk = (k * 4 + wave) % NBB;
    const int q = blk * 64 + lane;
    const int r = q / S::BC, pc = q % S::BC;
    int cl = pc ^ S::bsw(r);
    const int tok = min(jp * 32 + r, qv - 1);
    cl = cl * V < N ? cl : 0;
    dma16(Bc + (int64_t)tok * bstride + cl * V, (slot + blk * 1024));
  }
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int k = 0; k < S::XINST; ++k) {
      const int blk = (k * 4 + wave) % NXB;
      const int q = blk * 64 + lane;
      const int r = q / S::XC, pc = q % S::XC;
      const int cl = pc ^ S::xsw(r);
      const int tok = min(jp * 32 + r, qv - 1);
      int p = p0 + cl * V;
      p = p < P ? p : p0;
      dma16(xc + hh * hstep + (int64_t)tok * xstride + p,
            (slot + (S::BCH + hh * S::XCH) * 16 + blk * 1024));
    }
}

// The same loads for a pair whose 32 tokens all lie inside the sequence: the
// per-lane parts of the addresses (row within the pair, clamped column) do
// not depend on the pair, so they are byte offsets computed once, and each
// pair only moves the wave-uniform row base.
template <typename T, int NK, int KH>
struct PairOffsets {
  uint32_t b[Slot<T, NK, KH>::BINST];
  uint32_t x[KH][Slot<T, NK, KH>::XINST];
};

template <typename T, int NK, int KH>
__device__ __forceinline__ PairOffsets<T, NK, KH> pair_offsets(int64_t bstride, int N,
                                                               int64_t xstride, int64_t hstep,
                                                               int p0, int P, int wave, int lane) {
  typedef Slot<T, NK, KH> S;
  constexpr int V = S::V;
  constexpr int NBB = S::BCH / 64, NXB = S::XCH / 64;
  PairOffsets<T, NK, KH> o;
#pragma unroll
  for (int k = 0; k < S::BINST; ++k) {
    const int q = ((k * 4 + wave) % NBB) * 64 + lane;
    const int r = q / S::BC, pc = q % S::BC;
    int cl = pc ^ S::bsw(r);
    cl = cl * V < N ? cl : 0;
    o.b[k] = (uint32_t)(((int64_t)r * bstride + cl * V) * (int64_t)sizeof(T));
  }
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int k = 0; k < S::XINST; ++k) {
      const int q = ((k * 4 + wave) % NXB) * 64 + lane;
      const int r = q / S::XC, pc = q % S::XC;
      const int cl = pc ^ S::xsw(r);
      int p = p0 + cl * V;
      p = p < P ? p : p0;
      o.x[hh][k] = (uint32_t)((hh * hstep + (int64_t)r * xstride + p) * (int64_t)sizeof(T));
    }
  return o;
}

template <typename T, int NK, int KH>
__device__ __forceinline__ void issue_pair_fast(unsigned char* slot, const PairOffsets<T, NK, KH>& o,
                                                const T* __restrict__ Bc, int64_t bstride,
                                                const T* __restrict__ xc, int64_t xstride, int jp,
                                                int wave) {
  typedef Slot<T, NK, KH> S;
  constexpr int NBB = S::BCH / 64, NXB = S::XCH / 64;
  const T* bb = Bc + (int64_t)jp * 32 * bstride;
  const T* xb = xc + (int64_t)jp * 32 * xstride;
#pragma unroll
  for (int k = 0; k < S::BINST; ++k)
    dma16_so(bb, o.b[k], slot + ((k * 4 + wave) % NBB) * 1024);
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int k = 0; k < S::XINST; ++k)
      dma16_so(xb, o.x[hh][k], slot + (S::BCH + hh * S::XCH) * 16 + ((k * 4 + wave) % NXB) * 1024);
}

// A operand of S^T = B C^T: lane row j of the pair, n = n0 .. n0+7.
template <typename T, int NK, int KH>
__device__ __forceinline__ typename FragOf<T>::type slot_b_frag(const unsigned char* slot, int j,
                                                                int n0) {
  typedef Slot<T, NK, KH> S;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(slot + S::boff(j, n0));
  } else {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(slot + S::boff(j, n0));
    const floatx4 hi = *reinterpret_cast<const floatx4*>(slot + S::boff(j, n0 + 4));
    return floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// B operand of S x for head hh: column p = c0 + lane%16, tokens
// {4 lg .. 4 lg + 3, 16 + 4 lg .. +3} of the pair.
template <typename T, int NK, int KH>
__device__ __forceinline__ typename FragOf<T>::type slot_x_frag(const unsigned char* slot, int hh,
                                                                int c0, int lane) {
  typedef Slot<T, NK, KH> S;
  const int lg = lane / 16;
  if constexpr (sizeof(T) == 2) {
    // transposing reads: lane r of each 16-lane group addresses the 4 elements
    // at [t0 + r/4][c0 + 4 (r%4)]; lane l then holds rows t0..t0+3 of column c0 + l.
    // row ta + 16 has the same swizzle as row ta, 16 rows further on; the
    // head's block sits a whole multiple of rows away, so one lane address
    // serves all four reads of a column tile
    const int r = lane & 15;
    const int col = c0 + 4 * (r & 3);
    const int ta = 4 * lg + (r >> 2);
    const unsigned char* pa = slot + S::xoff(0, ta, col) + hh * S::XCH * 16;
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + 16 * S::XC * 16));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    const int c = c0 + (lane & 15);
    floatx8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = *reinterpret_cast<const float*>(slot + S::xoff(hh, 4 * lg + e, c));
      f[4 + e] = *reinterpret_cast<const float*>(slot + S::xoff(hh, 16 + 4 * lg + e, c));
    }
    return f;
  }
}

// Per-wave state: the wave's row blocks (slot 0 = the later one), their C
// fragments, the KH heads' accumulators and each block's reference running
// sum G_r (r = 32 q - 1, the token before the block's band; 0 for q = 0).
template <typename T, int NK, int IB, int KH>
struct WaveRows {
  typedef typename FragOf<T>::type frag_t;
  int ib[IB], q[IB];
  frag_t cf[IB][NK];
  floatx4 acc[KH][IB][4];
  float gr[KH][IB];
};

// One token pair for the first NS row blocks of the wave; if BAND, the last
// of them is at its own pair (the band next to the diagonal).
template <typename T, int NK, int IB, int KH, int NS, bool BAND>
__device__ __forceinline__ void pair_step(WaveRows<T, NK, IB, KH>& w, const unsigned char* sl,
                                          int jp, const float* Gs, const float* ds,
                                          const float* es, int Q, const float* dh, int lane) {
  typedef typename FragOf<T>::type frag_t;
  const int lr = lane % 16, lg = lane / 16;
  // raw tile S^T = B C^T for the active blocks (shared by all heads)
  floatx4 st[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s) { st[s][0] = floatx4{0.f, 0.f, 0.f, 0.f}; st[s][1] = st[s][0]; }
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    frag_t b0, b1;
    if constexpr (sizeof(T) == 2) {
      // row 16 + lr has the same swizzle as row lr, 16 rows further on
      const unsigned char* bp = sl + Slot<T, NK, KH>::boff(lr, ks * 32 + lg * 8);
      b0 = *reinterpret_cast<const bf16x8*>(bp);
      b1 = *reinterpret_cast<const bf16x8*>(bp + 16 * Slot<T, NK, KH>::BC * 16);
    } else {
      b0 = slot_b_frag<T, NK, KH>(sl, lr, ks * 32 + lg * 8);
      b1 = slot_b_frag<T, NK, KH>(sl, 16 + lr, ks * 32 + lg * 8);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      st[s][0] = mma(st[s][0], b0, w.cf[s][ks]);
      st[s][1] = mma(st[s][1], b1, w.cf[s][ks]);
    }
  }
  const int jb = jp * 32;
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) {
    const float* G = Gs + hh * Q;
    frag_t xf[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) xf[pt] = slot_x_frag<T, NK, KH>(sl, hh, pt * 16, lane);
    const floatx4 e0 = *reinterpret_cast<const floatx4*>(es + hh * Q + jb + 4 * lg);
    const floatx4 e1 = *reinterpret_cast<const floatx4*>(es + hh * Q + jb + 16 + 4 * lg);
    const float g_end = G[jb + 31];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      frag_t af;
      if (!(BAND && s == NS - 1)) {
        // left of the block's band: weight exp2(G_r - G_e) * e_j (both <= 1)
        const float f = fast_exp2(w.gr[hh][s] - g_end);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          af[r] = to_io<T>(st[s][0][r] * (e0[r] * f));
          af[4 + r] = to_io<T>(st[s][1][r] * (e1[r] * f));
        }
      } else {
        // the band: first scale row i = 16 ib + lr (this lane's accumulator
        // column) by exp2(G_i - G_r)
        const int ib = w.ib[s];
        const int i = ib * 16 + lr;
        const float gi = G[i];
        const float u = fast_exp2(gi - w.gr[hh][s]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) w.acc[hh][s][pt] *= u;
        // lane holds row i and tokens j = jb + 16 t + 4 lg + r; the exponent is
        // masked to -inf before exp2, so no positive exponent is ever
        // evaluated; the skip weight D_h rides on the diagonal
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const floatx4 gj = *reinterpret_cast<const floatx4*>(G + jb + 16 * t + 4 * lg);
          const floatx4 dj = *reinterpret_cast<const floatx4*>(ds + hh * Q + jb + 16 * t + 4 * lg);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = jb + 16 * t + 4 * lg + r;
            const float ex = j <= i ? gi - gj[r] : -__builtin_inff();
            float v = st[s][t][r] * (fast_exp2(ex) * dj[r]);
            v = j == i ? v + dh[hh] : v;
            af[4 * t + r] = to_io<T>(v);
          }
        }
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) w.acc[hh][s][pt] = mma(w.acc[hh][s][pt], xf[pt], af);
    }
  }
}

template <typename T, int NK, int IB, int KH>
__global__ void __launch_bounds__(kOutThreads) __attribute__((amdgpu_waves_per_eu(2)))
compute_out_kernel(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                   const float* __restrict__ Gw, const float* __restrict__ dtw,
                   const T* __restrict__ Hc, const float* __restrict__ Dv, T* __restrict__ y,
                   StatusRef flag, int64_t L, int H, int P, int N, int G, int Q, int T_,
                   int64_t ldw, int nbc, int PB, int RS) {
  typedef typename FragOf<T>::type frag_t;
  typedef Slot<T, NK, KH> S;
  constexpr int NSLOT = S::NSLOT;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int arrived[NSLOT], released[NSLOT];
  static_assert(2 * NSLOT * sizeof(int) <= kOutStaticLds, "static LDS bound");
  const OutLayout lay = out_layout<T, NK, KH>(Q);
  float* Gs = reinterpret_cast<float*>(smem + lay.g_off);
  float* ds = reinterpret_cast<float*>(smem + lay.d_off);
  float* es = reinterpret_cast<float*>(smem + lay.e_off);
  unsigned char* ring = smem + lay.ring_off;

  // XCD-aware placement: every head set, p slice and row part of one
  // (b, chunk) gets block ids congruent mod 8, so they run on one XCD and
  // share its L2 copy of the chunk's B and C rows; neighbouring ids take
  // different chunks, so the workgroups running at one time spread their
  // reads over several chunks' rows instead of all reading the same lines.
  const int id = blockIdx.x;
  if (id == 0 && threadIdx.x == 0) record_call(flag);
  const int xcd = id % 8, slot_id = id / 8;
  const int nbx = (nbc + 7) / 8;
  const int bc = (slot_id % nbx) * 8 + xcd;
  if (bc >= nbc) return;
  const int hp = slot_id / nbx;
  const int rsi = hp % RS;
  const int hs = hp / RS / PB, pb = hp / RS % PB;
  const int h0 = hs * KH;                         // first head of the set
  const int b = bc / T_, c = bc % T_;
  const int g = h0 / (H / G);
  const int p0 = pb * kOutP;
  const int64_t t0 = (int64_t)c * Q;
  const int qv = (int)min((int64_t)Q, L - t0);
  // this workgroup's 16-row blocks [ib0, ib0 + nibw) and the token pairs they need
  const int nibw = Q / 16 / RS;
  const int ib0 = rsi * nibw;
  const int rows_end = min(qv, (ib0 + nibw) * 16);
  if (rows_end <= ib0 * 16) return;               // part lies past the sequence end
  const int npairs = (rows_end + 31) / 32;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform (SGPR)
  const int lr = lane % 16, lg = lane / 16;
  if (tid < NSLOT) {
    arrived[tid] = 0;
    released[tid] = 0;
  }
  __syncthreads();                                // counters cleared before any wave bumps one
  const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
  const T* xc = x + ((int64_t)b * L + t0) * xstride + (int64_t)h0 * P;
  const T* Bc = Bm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;
  const T* Cc = Cm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;

  // ---- prologue ----------------------------------------------------------------
  // The chunk-start states of the KH heads are staged once per workgroup in
  // the ring slots the first pairs leave free (slots 2 .. NSLOT-1) when they
  // fit, instead of every wave reading all of them from global memory; the
  // first ring pairs are issued at the same time, and every global load of
  // the prologue is issued before any of it is used.
  constexpr int kFragBytes = 64 * (int)sizeof(frag_t);
  constexpr int kHBytes = KH * 4 * NK * kFragBytes;
  constexpr bool kStageH = NSLOT >= 3 && kHBytes <= (NSLOT - 2) * S::BYTES;
  constexpr int kPro = kStageH ? 2 : NSLOT - 1;    // pairs issued before the states are used
  const int64_t hstep = P;
  const PairOffsets<T, NK, KH> poff =
      pair_offsets<T, NK, KH>(bstride, N, xstride, hstep, p0, P, wave, lane);
  // byte offsets within a pair fit 32 bits (checked once, uniform)
  const bool off32 = (int64_t)32 * (xstride + bstride) * (int64_t)sizeof(T) < ((int64_t)1 << 31);
  auto issue = [&](int jn) {
    unsigned char* sl = ring + (jn % NSLOT) * S::BYTES;
    if (off32 && (jn + 1) * 32 <= qv)
      issue_pair_fast<T, NK, KH>(sl, poff, Bc, bstride, xc, xstride, jn, wave);
    else
      issue_pair<T, NK, KH>(sl, Bc, bstride, N, xc, xstride, hstep, p0, P, jn, qv, wave, lane);
  };

  WaveRows<T, NK, IB, KH> w;
  bool own[IB];
#pragma unroll
  for (int s = 0; s < IB; ++s) {
    const int sn = IB - 1 - s;
    const int ib = ib0 + ((sn % 2 == 0) ? 4 * sn + wave : 4 * sn + 3 - wave);
    own[s] = ib < ib0 + nibw && ib * 16 < qv;
    w.ib[s] = ib;
    w.q[s] = ib / 2;
  }
  // a wave whose later block is not owned (sequence end) moves its earlier one up
  int nown = 0;
#pragma unroll
  for (int s = 0; s < IB; ++s) nown += own[s] ? 1 : 0;
  if (IB == 2 && !own[0] && own[1]) { w.ib[0] = w.ib[IB - 1]; w.q[0] = w.q[IB - 1]; }
  // loads the compiler tracks come first: its own waits for them then never
  // cover the direct-to-LDS loads issued after them
#pragma unroll
  for (int s = 0; s < IB; ++s)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int i = w.ib[s] * 16 + lr, n = ks * 32 + lg * 8;
      w.cf[s][ks] = (s < nown && i < qv && n < N) ? load_frag(Cc + (int64_t)i * bstride + n)
                                                   : zero_frag<T>();
    }
  float gv[2], dv[2];                               // KH * Q <= 2 * kOutThreads
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = tid + u * kOutThreads;
    gv[u] = 0.0f;
    dv[u] = 0.0f;
    if (idx < KH * Q) {
      const int64_t row = (int64_t)(b * H + h0 + idx / Q) * ldw + t0;
      gv[u] = Gw[row + idx % Q];
      dv[u] = dtw[row + idx % Q];
    }
  }
  float dh[KH];
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) dh[hh] = Dv ? Dv[h0 + hh] : 0.0f;
  const HcFrag hcl = hc_frag(P, N);
  // chunk-start states, fragment-major: for one head and p slice the 4 x NK
  // fragments are one contiguous run
  auto hc_src = [&](int hh) {
    return Hc + ((int64_t)(b * H + h0 + hh) * T_ + c) * hcl.state_elems() + hcl.offset(pb, 0, 0, 0);
  };
#pragma unroll
  for (int k = 0; k < kPro; ++k)
    if (k < npairs) issue(k);
  frag_t hf[KH][4][NK];
  if constexpr (kStageH) {
    unsigned char* hstage = ring + 2 * S::BYTES;
    constexpr int kPer = kHBytes / 1024 / 4;        // 1 KiB loads per wave
    constexpr int kHeadK = 4 * NK * kFragBytes / 1024;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int g = k * 4 + wave;
      dma16(reinterpret_cast<const unsigned char*>(hc_src(g / kHeadK)) + (g % kHeadK) * 1024 + lane * 16,
            hstage + g * 1024);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __asm__ __volatile__("" ::: "memory");   // LDS written by the direct loads is read below
    if (npairs > 0) bump_count(&arrived[0], lane);   // this wave's share of pair 0 landed
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (tid + u * kOutThreads < KH * Q) {
        Gs[tid + u * kOutThreads] = gv[u];
        ds[tid + u * kOutThreads] = dv[u];
      }
    __syncthreads();                                // states, G, dt visible
#pragma unroll
    for (int hh = 0; hh < KH; ++hh)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const unsigned char* f = hstage + ((hh * 4 + pt) * NK + ks) * kFragBytes;
          hf[hh][pt][ks] = (ks * 32 + lg * 8 < N) ? lds_frag<T>(f, lane) : zero_frag<T>();
        }
  } else {
#pragma unroll
    for (int hh = 0; hh < KH; ++hh)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
          hf[hh][pt][ks] = (ks * 32 + lg * 8 < N)
                               ? load_frag(hc_src(hh) + hcl.offset(0, pt, ks, lane))
                               : zero_frag<T>();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __asm__ __volatile__("" ::: "memory");   // LDS written by the direct loads is read below
    if (npairs > 0) bump_count(&arrived[0], lane);   // this wave's share of pair 0 landed
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (tid + u * kOutThreads < KH * Q) {
        Gs[tid + u * kOutThreads] = gv[u];
        ds[tid + u * kOutThreads] = dv[u];
      }
    __syncthreads();                                // G, dt visible
  }
  // carried-state term C_i . H_c for every head
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f}, a2 = a;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        a = mma(a, hf[hh][pt][ks], w.cf[0][ks]);
        if (IB == 2) a2 = mma(a2, hf[hh][pt][ks], w.cf[IB - 1][ks]);
      }
      w.acc[hh][0][pt] = a;
      if (IB == 2) w.acc[hh][IB - 1][pt] = a2;
    }
  // e_j = exp2(G_e - G_j) dt_j, e = last token of j's pair (<= dt_j)
  for (int idx = tid; idx < KH * Q; idx += kOutThreads) {
    const int j = idx % Q;
    const int e = (j | 31) < Q ? (j | 31) : Q - 1;
    es[idx] = fast_exp2(Gs[idx - j + e] - Gs[idx]) * ds[idx];
  }
#pragma unroll
  for (int hh = 0; hh < KH; ++hh)
#pragma unroll
    for (int s = 0; s < IB; ++s) {
      const int q = w.q[s];
      w.gr[hh][s] = q >= 1 ? Gs[hh * Q + 32 * q - 1] : 0.0f;
      if (q >= 1) {
        const float sref = fast_exp2(w.gr[hh][s]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) w.acc[hh][s][pt] *= sref;
      }
    }
  if constexpr (kStageH) {
    // every wave has its states: the staging slots go back to the ring
    __syncthreads();
#pragma unroll
    for (int k = kPro; k < NSLOT - 1; ++k)
      if (k < npairs) issue(k);
  }

  const int q0 = nown >= 1 ? w.q[0] : -1;
  const int q1 = nown >= 2 ? w.q[IB - 1] : -1;

  // Token pair jp: refill the slot pair jp-1 used (once every wave released
  // it) with pair jp+NSLOT-1; wait for this wave's own loads of pair jp+1
  // (vector memory operations retire in issue order, and global stores issued
  // since only make the wait stricter) and announce them one pair early, so
  // that a wave reaching pair jp+1 never waits for another wave to reach it;
  // then wait for every wave's share of pair jp.  release_pair(jp) follows
  // the wave's last read of the pair.  A wave can so run one pair ahead of
  // the slowest one.
  auto sync_pair = [&](int jp) {
    const int nxt = jp + NSLOT - 1;
    if (nxt < npairs) {
      if (jp >= 1)
        wait_count(&released[(jp - 1) % NSLOT], kOutWaves * ((jp - 1) / NSLOT + 1), flag, lane);
      issue(nxt);
    }
    if (jp + 1 < npairs) {
      wait_groups<S::LPG>(min(NSLOT - 2, npairs - 2 - jp));
      bump_count(&arrived[(jp + 1) % NSLOT], lane);
    }
    wait_count(&arrived[jp % NSLOT], kOutWaves * (jp / NSLOT + 1), flag, lane);
  };
  auto release_pair = [&](int jp) { bump_count(&released[jp % NSLOT], lane); };
  // a finished block: lane holds row i = 16 ib + lr and the 4 consecutive p
  // columns 16 pt + 4 lg .. +3 of every tile, stored straight from registers
  const bool vec4 = (P % 4) == 0;
  auto store_block = [&](int done) {
    const int i2 = (done == 0 ? w.ib[0] : w.ib[IB - 1]) * 16 + lr;
    if (i2 >= qv) return;
#pragma unroll
    for (int hh = 0; hh < KH; ++hh) {
      T* yrow = y + (((int64_t)b * L + t0 + i2) * H + h0 + hh) * P;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const floatx4 v = done == 0 ? w.acc[hh][0][pt] : w.acc[hh][IB - 1][pt];
        const int p = p0 + pt * 16 + 4 * lg;
        if (vec4 && p + 4 <= P) {
          store4<T>(yrow + p, v);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (p + r < P) yrow[p + r] = to_io<T>(v[r]);
        }
      }
    }
  };

  // ---- stream the token pairs ---------------------------------------------------
  // Phases with one pair step each, so every loop body keeps the accumulators
  // in place: both blocks left of the earlier block's band, that band, the
  // later block alone, its band, then pairs this wave only helps to load.
  int jp = 0;
  if constexpr (IB == 2) {
    if (nown == 2) {
      for (; jp < q1; ++jp) {
        sync_pair(jp);
        pair_step<T, NK, IB, KH, IB, false>(w, ring + (jp % NSLOT) * S::BYTES, jp, Gs, ds, es, Q,
                                            dh, lane);
        release_pair(jp);
      }
      sync_pair(jp);
      pair_step<T, NK, IB, KH, IB, true>(w, ring + (jp % NSLOT) * S::BYTES, jp, Gs, ds, es, Q, dh,
                                         lane);
      release_pair(jp);
      store_block(IB - 1);
      ++jp;
    }
  }
  if (nown >= 1) {
    for (; jp < q0; ++jp) {
      sync_pair(jp);
      pair_step<T, NK, IB, KH, 1, false>(w, ring + (jp % NSLOT) * S::BYTES, jp, Gs, ds, es, Q, dh,
                                         lane);
      release_pair(jp);
    }
    sync_pair(jp);
    pair_step<T, NK, IB, KH, 1, true>(w, ring + (jp % NSLOT) * S::BYTES, jp, Gs, ds, es, Q, dh,
                                      lane);
    release_pair(jp);
    store_block(0);
    ++jp;
  }
  for (; jp < npairs; ++jp) {
    sync_pair(jp);
    release_pair(jp);
  }
  // every load into LDS was waited for inside the loop (the last pair with
  // vmcnt(0)); only global stores may still be in flight here
}

template <typename T, int NK, int IB, int KH>
static hipError_t launch_out(const void* x, const void* Bm, const void* Cm, const float* Gw,
                             const float* dtw, const void* Hc, const float* Dv, void* y, StatusRef flag,
                             int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                             int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
  const OutLayout lay = out_layout<T, NK, KH>(Q);
  const int PB = (int)((P + kOutP - 1) / kOutP);
  const int RS = Q >= 128 ? Q / 128 : 1;   // 128 rows (8 blocks, 2 per wave) per workgroup
  const int64_t nbc = batch * T_;
  const int64_t nblocks = ((nbc + 7) / 8) * 8 * (H / KH) * PB * RS;
  auto kern = compute_out_kernel<T, NK, IB, KH>;
  const hipError_t e = ensure_dyn_lds<compute_out_kernel<T, NK, IB, KH>>(160 * 1024 - kOutStaticLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(kOutThreads), lay.bytes, stream,
                     static_cast<const T*>(x), static_cast<const T*>(Bm), static_cast<const T*>(Cm),
                     Gw, dtw, static_cast<const T*>(Hc), Dv, static_cast<T*>(y), flag, L, (int)H, (int)P,
                     (int)N, (int)G, Q, (int)T_, ldw, (int)nbc, PB, RS);
  return hipGetLastError();
}

// heads per workgroup: two heads of one group share the tile C B^T when the
// group has an even head count and the accumulators of both fit in registers
// next to 2 waves per SIMD (bf16, dstate <= 128); one head otherwise.  Both
// are valid where two are (the caller may choose one).
int compute_out_kh_valid(int io_bf16, int64_t H, int64_t G, int64_t N, int kh) {
  if (kh == 1) return 1;
  return kh == 2 && io_bf16 && nk_class(N) <= 4 && (H / G) % 2 == 0;
}
#ifndef SSD_OUT_MAX_KH
#define SSD_OUT_MAX_KH 2
#endif
int compute_out_default_kh(int io_bf16, int64_t H, int64_t G, int64_t N) {
  return (SSD_OUT_MAX_KH >= 2 && compute_out_kh_valid(io_bf16, H, G, N, 2)) ? 2 : 1;
}

template <typename T, int IB, int KH>
static hipError_t launch_out_nk(int NK, const void* x, const void* Bm, const void* Cm,
                                const float* Gw, const float* dtw, const void* Hc, const float* Dv,
                                void* y, StatusRef flag, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                int64_t G, int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
#define SSD_OUT_ARGS x, Bm, Cm, Gw, dtw, Hc, Dv, y, flag, batch, L, H, P, N, G, Q, T_, ldw, stream
  switch (NK) {
    case 1: return launch_out<T, 1, IB, KH>(SSD_OUT_ARGS);
    case 2: return launch_out<T, 2, IB, KH>(SSD_OUT_ARGS);
    case 4: return launch_out<T, 4, IB, KH>(SSD_OUT_ARGS);
    default: return launch_out<T, 8, IB, KH>(SSD_OUT_ARGS);
  }
#undef SSD_OUT_ARGS
}

template <typename T>
static hipError_t launch_out_t(int kh, const void* x, const void* Bm, const void* Cm, const float* Gw,
                               const float* dtw, const void* Hc, const float* Dv, void* y, StatusRef flag,
                               int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                               int64_t G, int Q, int64_t T_, int64_t ldw, hipStream_t stream) {
#define SSD_OUT_ARGS nk_class(N), x, Bm, Cm, Gw, dtw, Hc, Dv, y, flag, batch, L, H, P, N, G, Q, T_, ldw, stream
  const bool two = kh == 2;
  if (Q >= 128) return two ? launch_out_nk<T, 2, 2>(SSD_OUT_ARGS) : launch_out_nk<T, 2, 1>(SSD_OUT_ARGS);
  return two ? launch_out_nk<T, 1, 2>(SSD_OUT_ARGS) : launch_out_nk<T, 1, 1>(SSD_OUT_ARGS);
#undef SSD_OUT_ARGS
}

template <typename T>
static int smem_bytes_t(int Q, int NK, int KH) {
#define SSD_LAY(nk) (KH == 2 ? out_layout<T, nk, 2>(Q).bytes : out_layout<T, nk, 1>(Q).bytes)
  switch (NK) {
    case 1: return SSD_LAY(1);
    case 2: return SSD_LAY(2);
    case 4: return SSD_LAY(4);
    default: return SSD_LAY(8);
  }
#undef SSD_LAY
}

int compute_out_smem_bytes(int io_bf16, int Q, int64_t N, int kh) {
  const int NK = nk_class(N), KH = kh;
  return kOutStaticLds + (io_bf16 ? smem_bytes_t<bf16>(Q, NK, KH) : smem_bytes_t<float>(Q, NK, KH));
}

hipError_t launch_compute_out(int io_bf16, const void* x, const void* Bm, const void* Cm,
                              const float* Gw, const float* dtw, const void* Hc, const float* Dv,
                              void* y, StatusRef status, int64_t batch, int64_t L, int64_t H,
                              int64_t P, int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw,
                              int kh, hipStream_t stream) {
  if (io_bf16)
    return launch_out_t<bf16>(kh, x, Bm, Cm, Gw, dtw, Hc, Dv, y, status, batch, L, H, P, N, G, Q, T_, ldw, stream);
  return launch_out_t<float>(kh, x, Bm, Cm, Gw, dtw, Hc, Dv, y, status, batch, L, H, P, N, G, Q, T_, ldw, stream);
}

}  // namespace ssd
