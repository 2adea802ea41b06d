// out_resident.hip -- stage 3 with the chunk's interaction tile resident in
// registers while the workgroup walks through many heads.
//
// What it computes is compute_out's (compute_out.hip): for token i of chunk c
// of head (b, h),
//   y_i = sum_{j<=i} (C_i . B_j) exp2(G_i - G_j) dt_j x_j + exp2(G_i) (H_c C_i) + D_h x_i
// (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section
// "세 가지 핵심 커널 구현", compute_out; brifing.si "Accelerating Mamba-2 ...",
// sections 9 and 11), with the same decay factorisation, masking, operand
// order and roundings, so both kernels give bitwise the same y.
//
// Why a second kernel.  All heads of a group share C and B, so the raw tile
// C B^T of a chunk is the same for every one of them; only the decay weights,
// x, the chunk-start state and D are per head.  compute_out rebuilds the tile
// for every pair of heads and streams B, C, x and the states through LDS for
// each (head pair, 128-row half) -- about 3x the bytes the chunk's inputs
// hold.  Here one workgroup takes one (b, chunk) and a run of heads of one
// group: it builds the raw tile once and keeps it in registers, then streams
// only each head's x rows, state, running sums and step sizes, so every input
// byte crosses into the CU once.
//
// gfx950 layout.  8 waves (512 threads), one workgroup per CU: all 256 rows
// of the chunk as 16 blocks of 16 rows, wave w owning blocks w and 15 - w, so
// causal work is the same for every wave.  Block ib needs the 32-token pairs
// 0 .. ib/2; the wave's two blocks need 9 pair tiles between them (w/2 + 1
// and (15 - w)/2 + 1), kept as fp32 MFMA accumulators (8 registers each) in
// slots 0..8: the early block's pair jp in slot jp, the late block's in slot
// 8 - jp -- the two ranges never meet, and both indices are compile-time
// constants in the unrolled pair loop.  The tile is produced transposed
// (S^T = B C^T, lane = row i, 4 + 4 token columns), which is exactly the A
// operand of the output product once weighted and rounded to bf16.
//
// Streaming.  Two head buffers in LDS (x rows with XOR-swizzled 16-byte
// chunks, the fragment-major state slice, G, dt and the off-band weight
// tables), filled by direct global->LDS loads one head ahead; a workgroup
// barrier per head hands buffers on.  Every wave issues exactly kLoadsPerHead loads
// per head and kStoresPerHead stores, so one vmcnt target per head is exact.
// y is written with buffer stores whose range ends at the chunk's last valid
// row: rows past the sequence end are dropped by the hardware range check,
// so the stores are never branched around and their count stays fixed.
#include <type_traits>

#include "ssd_device.hpp"

namespace ssd {

namespace {

constexpr int kRsWaves = 8;
constexpr int kRsThreads = kRsWaves * kWave;   // 512
constexpr int kRsQ = 256;                      // chunk rows (16 blocks, 8 pairs)
constexpr int kRsP = 64;                       // headdim
constexpr int kRsNK = 4;                       // most 32-column steps over n (dstate <= 128)

// one head buffer
constexpr int kBufX = 0;                                // 256 rows x 128 B
constexpr int kBufH = kBufX + kRsQ * kRsP * 2;          // fragment-major state, 16 KiB
constexpr int kBufG = kBufH + kRsP * kRsNK * 32 * 2;    // G (fp32 x 256)
constexpr int kBufD = kBufG + kRsQ * 4;                 // dt
constexpr int kBufE = kBufD + kRsQ * 4;                 // off-band weights E_q, q = 1..7
constexpr int kEElems = 16 * 8 * 7;                     // sum of 32 q over q = 1..7
constexpr int kBufBytes = kBufE + kEElems * 4;          // 54784
constexpr int kNBuf = 2;
// each wave's y rows (its two blocks, 32 rows x 128 B) on their way out
constexpr int kYStage = kNBuf * kBufBytes;
constexpr int kYStageBytes = kRsWaves * 32 * 128;
// B rows (256 x 256 B) are staged once, from the start of buffer 1 (before
// any y row is)
constexpr int kBOff = kBufBytes;
constexpr int kBBytes = kRsQ * kRsNK * 32 * 2;
constexpr int kRsLds = kYStage + kYStageBytes > kBOff + kBBytes ? kYStage + kYStageBytes
                                                                : kBOff + kBBytes;
static_assert(kRsLds <= 160 * 1024, "LDS of one CU");

// Row q of the off-band weight tables: tokens 0 .. 32 q - 1.
__host__ __device__ constexpr int e_row(int q) { return 16 * q * (q - 1); }

// Per head and wave: 4 of the 32 x blocks of 1 KiB, 2 of the (up to 16)
// state blocks, and the whole G and dt rows (every wave loads these, so each
// can read them once its own loads have landed) -- 8 loads.  Where fewer
// state blocks exist (dstate < 128) the extra loads repeat one (identical
// data to the same place), so the count is fixed.
constexpr int kLoadsPerHead = 8;
constexpr int kStoresPerHead = 4;   // 4 x 8 whole rows of 128 bytes

__device__ __forceinline__ int bsw(int r) { return r & 15; }
__device__ __forceinline__ int xsw(int r) { return ((r >> 1) & 3) << 1; }

// Wait until at most n of this wave's vector-memory operations are
// outstanding, for the few counts the head loop uses; then keep the compiler
// from moving LDS reads of the awaited data above the wait.
template <int N>
__device__ __forceinline__ void wait_vm_ops() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  __asm__ __volatile__("" ::: "memory");
}

// Workgroup barrier that orders LDS only: this wave's LDS writes complete
// before it, and no LDS access moves across it.  Loads and stores in flight
// to or from global memory are not waited for (the head loop counts those
// itself).
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// A wave-uniform value the compiler must take as redefined here: tests of
// it are then made where they are used, as scalar compares, instead of being
// hoisted out of the head loop as dozens of live lane masks (which spill).
__device__ __forceinline__ int opaque_s(int v) {
  __asm__ __volatile__("" : "+s"(v));
  return v;
}

// The same for a per-lane value.
__device__ __forceinline__ int opaque_v(int v) {
  __asm__ __volatile__("" : "+v"(v));
  return v;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct HeadSrc {
  const bf16* x;      // x rows of the chunk for this head: x + ((b L + t0) H + h) P
  const bf16* hc;     // fragment-major chunk-start state
  const float* g;     // G row of (b, h) from t0
  const float* dt;    // dt row of (b, h) from t0
};

// Per-lane byte offsets of a head's loads (the same for every head and
// block): an x row within a group of 8 rows and its swizzled 16-byte chunk,
// and lane * 16 for the contiguous state, G and dt blocks.
struct HeadOffsets {
  uint32_t x;
  uint32_t l16;
};

// The kLoadsPerHead loads of one head into buffer `buf` (load k of this
// wave).  In a chunk cut by the sequence end, x rows past its last valid
// token read that token's row instead (their values meet only masked tile
// entries or rows that are never stored).
template <int NK>
__device__ __forceinline__ void issue_load(int k, unsigned char* buf, const HeadSrc& s,
                                           const HeadOffsets& o, int64_t xstride, int qv,
                                           int wave, int lane) {
  if (k < 4) {
    const int row0 = (wave + 8 * k) * 8;
    unsigned char* dst = buf + kBufX + (wave + 8 * k) * 1024;
    if (qv == kRsQ) {
      dma16_so(s.x + (int64_t)row0 * xstride, o.x, dst);
    } else {
      const int r = row0 + lane / 8;
      const int gc = (lane % 8) ^ xsw(r);
      dma16(s.x + (int64_t)min(r, qv - 1) * xstride + gc * 8, dst);
    }
  } else if (k < 6) {
    const int blk = (wave + 8 * (k - 4)) % (4 * NK);
    dma16_so(s.hc + blk * 512, o.l16, buf + kBufH + blk * 1024);
  } else if (k == 6) {
    dma16_so(s.g, o.l16, buf + kBufG);
  } else {
    dma16_so(s.dt, o.l16, buf + kBufD);
  }
}
template <int NK>
__device__ __forceinline__ void issue_head(unsigned char* buf, const HeadSrc& s,
                                           const HeadOffsets& o, int64_t xstride, int qv,
                                           int wave, int lane) {
#pragma unroll
  for (int k = 0; k < kLoadsPerHead; ++k) issue_load<NK>(k, buf, s, o, xstride, qv, wave, lane);
}

// The off-band weights of one head, seen from each row-block reference
// r = 32 q - 1 (q = 1..7, the last token before the band pair q):
//   E_q(j) = (exp2(G_e - G_j) dt_j) * exp2(G_r - G_e),  j < 32 q,
// e = the last token of j's pair, so both factors are <= 1.  Each is the
// product the tile operand needs (one rounding, the factors formed as the
// head-pair kernel forms them), made once per head here instead of by every
// wave per tile: the 896 entries spread over all 512 threads (entry k and
// k + 512), from G and dt rows that all waves loaded.
__device__ __forceinline__ void weight_table(unsigned char* buf, int tid) {
  const float* Gs = reinterpret_cast<const float*>(buf + kBufG);
  const float* ds = reinterpret_cast<const float*>(buf + kBufD);
  float* Es = reinterpret_cast<float*>(buf + kBufE);
#pragma unroll
  for (int k = tid; k < kEElems; k += kRsThreads) {
    int q = 1;
#pragma unroll
    for (int r = 2; r < 8; ++r) q = k >= e_row(r) ? r : q;
    const int j = k - e_row(q), e = j | 31;
    const float ge = Gs[e];
    Es[k] = (fast_exp2(ge - Gs[j]) * ds[j]) * fast_exp2(Gs[32 * q - 1] - ge);
  }
}

// Weighted tile -> bf16 A operand, left of the block's band: weights E_q of
// the lane's 4 + 4 tokens.
__device__ __forceinline__ bf16x8 offband_operand(const floatx4 (&st)[2], floatx4 e0, floatx4 e1) {
  bf16x8 af;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    af[r] = static_cast<bf16>(st[0][r] * e0[r]);
    af[4 + r] = static_cast<bf16>(st[1][r] * e1[r]);
  }
  return af;
}

}  // namespace

template <int NK>
__global__ void __launch_bounds__(kRsThreads)
out_resident_kernel(const bf16* __restrict__ x, const bf16* __restrict__ Bm,
                    const bf16* __restrict__ Cm, const float* __restrict__ Gw,
                    const float* __restrict__ dtw, const bf16* __restrict__ Hc,
                    const float* __restrict__ Dv, bf16* __restrict__ y, StatusRef flag, int64_t L,
                    int H, int N, int G, int T_, int64_t ldw, int ngrp, int nsplit, int hpw) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int id = blockIdx.x;
  if (id == 0 && threadIdx.x == 0) record_call(flag);
  // XCD-aware placement: block ids congruent mod 8 run on one XCD; the
  // workgroups of one (b, chunk, group) -- which read the same B and C rows --
  // get ids congruent mod 8, so they share that XCD's L2.
  const int xcd = id % 8, k8 = id / 8;
  const int grp = (k8 / nsplit) * 8 + xcd;
  if (grp >= ngrp) return;
  const int split = k8 % nsplit;
  const int g = grp % G, bc = grp / G;
  const int b = bc / T_, c = bc % T_;
  const int hg = H / G;
  const int h_begin = g * hg + split * hpw;
  const int h_end = min(h_begin + hpw, (g + 1) * hg);
  const int nh = h_end - h_begin;
  if (nh <= 0) return;
  const int64_t t0 = (int64_t)c * kRsQ;
  const int qv = (int)min((int64_t)kRsQ, L - t0);

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane % 16, lg = lane / 16;
  const int ib_e = wave, ib_l = 2 * kRsWaves - 1 - wave;   // the wave's two row blocks
  const int q0 = ib_e / 2, q1 = ib_l / 2;                    // their band pairs; q0 + q1 = 7

  const int64_t xstride = (int64_t)H * kRsP, bstride = (int64_t)G * N;
  const bf16* Bc = Bm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;
  const bf16* Cc = Cm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;
  // one fragment-major state: 4 row tiles x NK column steps of 1 KiB
  // (NK = nk_class(dstate): 1, 2 or 4)
  const int64_t helems = (int64_t)kRsP * NK * 32;

  auto head_src = [&](int hh) {
    const int h = h_begin + hh;
    HeadSrc s;
    s.x = x + ((int64_t)b * L + t0) * xstride + (int64_t)h * kRsP;
    s.hc = Hc + ((int64_t)(b * H + h) * T_ + c) * helems;
    s.g = Gw + (int64_t)(b * H + h) * ldw + t0;
    s.dt = dtw + (int64_t)(b * H + h) * ldw + t0;
    return s;
  };
  HeadOffsets ho;
  ho.x = (uint32_t)(((int64_t)(lane / 8) * xstride + ((lane % 8) ^ xsw(lane / 8)) * 8) * 2);
  ho.l16 = (uint32_t)lane * 16u;

  // ---- once per workgroup: C fragments, B rows, the resident tiles --------------
  // loads the compiler tracks first, so its own wait for them stays exact
  bf16x8 cf_e[NK], cf_l[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const int n = ks * 32 + lg * 8;
    const int ie = min(ib_e * 16 + lr, qv - 1), il = min(ib_l * 16 + lr, qv - 1);
    cf_e[ks] = n < N ? load_frag(Cc + (int64_t)ie * bstride + n) : zero_frag<bf16>();
    cf_l[ks] = n < N ? load_frag(Cc + (int64_t)il * bstride + n) : zero_frag<bf16>();
  }
  // B: 64 blocks of 4 rows x 256 B, 8 per wave
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = wave + 8 * i;
    const int r = blk * 4 + lane / 16;
    int gc = (lane % 16) ^ bsw(r);
    gc = gc * 8 < N ? gc : 0;
    const int tok = min(r, qv - 1);
    dma16(Bc + (int64_t)tok * bstride + gc * 8, smem + kBOff + blk * 1024);
  }
  wait_vm_ops<0>();                                          // C and B landed
  lds_barrier();
  // head 0 -> buffer 0 while the tiles are built (issued after the wait: vector
  // memory completes in order, so a wait for C would otherwise wait for it too)
  issue_head<NK>(smem, head_src(0), ho, xstride, qv, wave, lane);

  floatx4 tile[9][2];
#pragma unroll
  for (int s = 0; s < 9; ++s) { tile[s][0] = floatx4{0.f, 0.f, 0.f, 0.f}; tile[s][1] = tile[s][0]; }
#pragma unroll
  for (int jp = 0; jp < 8; ++jp) {
    const int qe = opaque_s(q0), ql = opaque_s(q1);
    if (jp > qe && jp > ql) continue;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      // rows jp*32 + lr and + 16 share the swizzle of row lr
      const unsigned char* bp = smem + kBOff + (jp * 32 + lr) * 256 + (((ks * 4 + lg) ^ bsw(lr)) * 16);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(bp);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(bp + 16 * 256);
      if (jp <= qe) {
        tile[jp][0] = mma(tile[jp][0], b0, cf_e[ks]);
        tile[jp][1] = mma(tile[jp][1], b1, cf_e[ks]);
      }
      if (jp <= ql) {
        tile[8 - jp][0] = mma(tile[8 - jp][0], b0, cf_l[ks]);
        tile[8 - jp][1] = mma(tile[8 - jp][1], b1, cf_l[ks]);
      }
    }
  }
  wait_vm_ops<0>();                                          // this wave's head-0 loads landed
  weight_table(smem, tid);
  lds_barrier();     // B rows no longer read; every wave's head-0 loads and weights in place

  // per-lane store offsets (bytes, relative to row 0 of the chunk, head 0)
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      y + ((int64_t)b * L + t0) * xstride, (short)0, (int)((int64_t)qv * xstride * 2), 0x00020000);

  // Head hh starts after a barrier that follows every wave's wait for its
  // own loads of hh and the weight tables of hh (made by the first four
  // waves), so all of hh is in LDS and every wave is done with head hh-1,
  // whose buffer takes head hh+1: a head's loads are issued one head ahead,
  // ~4 us before they are needed.  (Hand-offs through LDS counters instead
  // of the barrier, letting the older waves, which win the SIMD's issue
  // arbitration, run up to one head ahead, measured 1-2% slower.)
  for (int hh = 0; hh < nh; ++hh) {
    // the loads of head hh+1 are spread over the head (two after the carried
    // term, two in each of the first three pair steps -- every wave has at
    // least five): issued all at once they queue behind one another and
    // stall the later waves
    const bool pre = hh + 1 < nh;
    unsigned char* pbuf = smem + ((hh + 1) % kNBuf) * kBufBytes;
    const HeadSrc psrc = head_src(hh + 1);
    auto prefetch = [&](int k) {
      if (pre) issue_load<NK>(k, pbuf, psrc, ho, xstride, qv, wave, lane);
    };
    unsigned char* buf = smem + (hh % kNBuf) * kBufBytes;
    const float* Gs = reinterpret_cast<const float*>(buf + kBufG);
    const float* ds = reinterpret_cast<const float*>(buf + kBufD);
    const float* Es = reinterpret_cast<const float*>(buf + kBufE);
    const int h = h_begin + hh;
    const float dh = Dv ? Dv[h] : 0.0f;

    // carried-state term C_i . H_c, then the reference scale exp2(G_r)
    floatx4 acc_e[4], acc_l[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      floatx4 a = floatx4{0.f, 0.f, 0.f, 0.f}, a2 = a;
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 hf = lds_frag<bf16>(buf + kBufH + (pt * NK + ks) * 1024, lane);
        a = mma(a, hf, cf_e[ks]);
        a2 = mma(a2, hf, cf_l[ks]);
      }
      acc_e[pt] = a;
      acc_l[pt] = a2;
    }
    prefetch(0);
    prefetch(1);
    const float gr_e = q0 >= 1 ? Gs[32 * q0 - 1] : 0.0f;
    const float gr_l = q1 >= 1 ? Gs[32 * q1 - 1] : 0.0f;
    if (q0 >= 1) {
      const float sref = fast_exp2(gr_e);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc_e[pt] *= sref;
    }
    if (q1 >= 1) {
      const float sref = fast_exp2(gr_l);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc_l[pt] *= sref;
    }

    // the band pair of a block: scale row i by exp2(G_i - G_r), then add the
    // masked per-element weights exp2(G_i - G_j) dt_j (the exponent is masked
    // to -inf before exp2, so no positive exponent is evaluated); D_h rides
    // on the diagonal
    // Of the band pair's two 16-token halves, an even block (rows = the first
    // half) sees the second half masked out entirely, and an odd block sees
    // the first half entirely below its rows (unmasked, no diagonal); only
    // the half on the diagonal needs the per-element mask.  The values are
    // those of the full masked evaluation (masked entries are exact zeros).
    auto band_half = [&](auto oddc, const floatx4 (&st)[2], floatx4 (&acc)[4], int ib, float gr,
                         int jb, const bf16x8 (&xf)[4]) {
      constexpr int ODD = decltype(oddc)::value;
      const int i = ib * 16 + lr;
      const float gi = Gs[i];
      // row minus the lane's first token column of the diagonal half,
      // laundered so the masks below are formed here rather than hoisted out
      // of the head loop
      const int d = opaque_v(i - jb - 16 * ODD - 4 * lg);
      const float u = fast_exp2(gi - gr);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[pt] *= u;
      bf16x8 af;
      const floatx4 gj = *reinterpret_cast<const floatx4*>(Gs + jb + 16 * ODD + 4 * lg);
      const floatx4 dj = *reinterpret_cast<const floatx4*>(ds + jb + 16 * ODD + 4 * lg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ex = r <= d ? gi - gj[r] : -__builtin_inff();
        float v = st[ODD][r] * (fast_exp2(ex) * dj[r]);
        v = r == d ? v + dh : v;
        af[4 * ODD + r] = static_cast<bf16>(v);
      }
      if constexpr (ODD) {
        const floatx4 g0 = *reinterpret_cast<const floatx4*>(Gs + jb + 4 * lg);
        const floatx4 d0 = *reinterpret_cast<const floatx4*>(ds + jb + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) af[r] = static_cast<bf16>(st[0][r] * (fast_exp2(gi - g0[r]) * d0[r]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) af[4 + r] = static_cast<bf16>(0.0f);
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[pt] = mma(acc[pt], xf[pt], af);
    };
    auto band = [&](const floatx4 (&st)[2], floatx4 (&acc)[4], int ib, float gr, int jb,
                    const bf16x8 (&xf)[4]) {
      if (opaque_s(ib) & 1)
        band_half(std::integral_constant<int, 1>{}, st, acc, ib, gr, jb, xf);
      else
        band_half(std::integral_constant<int, 0>{}, st, acc, ib, gr, jb, xf);
    };

    // off-band weights of the lane's tokens {4 lg .. +3, 16 + 4 lg .. +3} of
    // pair jp, seen from reference q
    auto offband_w = [&](int q, int jb, floatx4& e0, floatx4& e1) {
      e0 = *reinterpret_cast<const floatx4*>(Es + e_row(q) + jb + 4 * lg);
      e1 = *reinterpret_cast<const floatx4*>(Es + e_row(q) + jb + 16 + 4 * lg);
    };
    // The pair steps, specialised per wave class: the early block's band
    // pair Q0 = w/2 (0..3) fixes the late block's, 7 - Q0, so with Q0 a
    // constant every step's blocks and kinds are known and the steps form
    // one branch-free stretch the compiler can schedule across.
    auto pair_steps = [&](auto q0c) {
      constexpr int Q0 = decltype(q0c)::value, Q1 = 7 - Q0;
#pragma unroll
      for (int jp = 0; jp <= Q1; ++jp) {
        const int jb = jp * 32;
        // x operand: column p = 16 pt + lane%16, tokens {4 lg .. +3, 16 + 4 lg .. +3}
        // of the pair, by transposing reads (lane r of a 16-lane group addresses
        // row ta = 4 lg + r/4, columns 4 (r%4) .. +3 of the 16-column tile)
        bf16x8 xf[4];
        {
          const int r = lane & 15;
          const int ta = 4 * lg + (r >> 2);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const int col = pt * 16 + 4 * (r & 3);
            const unsigned char* pa =
                buf + kBufX + (jb + ta) * 128 + (((col >> 3) ^ xsw(ta)) * 16) + (col & 7) * 2;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + 16 * 128));
            xf[pt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        if (jp < 3) {
          prefetch(2 + 2 * jp);
          prefetch(3 + 2 * jp);
        }
        if (jp < Q0) {
          floatx4 e0, e1;
          offband_w(Q0, jb, e0, e1);
          const bf16x8 af = offband_operand(tile[jp], e0, e1);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc_e[pt] = mma(acc_e[pt], xf[pt], af);
        } else if (jp == Q0) {
          band(tile[jp], acc_e, ib_e, gr_e, jb, xf);
        }
        if (jp < Q1) {
          floatx4 e0, e1;
          offband_w(Q1, jb, e0, e1);
          const bf16x8 af = offband_operand(tile[8 - jp], e0, e1);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc_l[pt] = mma(acc_l[pt], xf[pt], af);
        } else {
          band(tile[8 - jp], acc_l, ib_l, gr_l, jb, xf);
        }
      }
    };
    switch (opaque_s(q0)) {
      case 0: pair_steps(std::integral_constant<int, 0>{}); break;
      case 1: pair_steps(std::integral_constant<int, 1>{}); break;
      case 2: pair_steps(std::integral_constant<int, 2>{}); break;
      default: pair_steps(std::integral_constant<int, 3>{}); break;
    }

    // y rows of both blocks (lane: row lr of each, p = 16 pt + 4 lg .. +3)
    // through this wave's staging rows -- 0..15 the early block, 16..31 the
    // late one -- so that each store writes 8 whole 128-byte rows instead of
    // 16 scattered 32-byte pieces.  In the staging, the 8-byte piece
    // (row, p) sits in 16-byte chunk (p / 8) ^ (row % 8) and half
    // (p / 4 % 2) ^ (row / 8 % 2): the 16 rows of one write and the 8 chunks
    // of one row in a read meet distinct banks.
    unsigned char* ys = smem + kYStage + wave * (32 * 128);
    {
      const int lrv = opaque_v(lr);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(blk ? acc_l[pt][e] : acc_e[pt][e]);
          const int row = blk * 16 + lrv;
          const int c = (2 * pt + (lg >> 1)) ^ (row & 7), half = (lg & 1) ^ ((row >> 3) & 1);
          *reinterpret_cast<bf16x4*>(ys + row * 128 + c * 16 + half * 8) = v;
        }
    }
    wave_sync();
    {
      // store s: staging rows 8 s + lane / 8, 16-byte chunk lane % 8 of each;
      // rows past the sequence end fall outside the store range and are dropped
      const int rl = opaque_v(lane >> 3), cl = lane & 7;
      const uint32_t col = (uint32_t)h * kRsP * 2 + (uint32_t)cl * 16;
#pragma unroll
      for (int st = 0; st < kStoresPerHead; ++st) {
        const int row = 8 * st + rl;                 // row % 8 = rl, row / 8 % 2 = st % 2
        u32x4 v = *reinterpret_cast<const u32x4*>(ys + row * 128 + ((cl ^ rl) * 16));
        if (st & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        const int grow = st < 2 ? ib_e * 16 + row : ib_l * 16 + row - 16;
        __builtin_amdgcn_raw_buffer_store_b128(v, yr, (int)((uint32_t)(grow * (int)xstride * 2) + col),
                                               0, 0);
      }
    }
    if (hh + 1 < nh) {
      // this wave's loads of head hh+1 landed: after them it issued only the
      // stores of head hh
      wait_vm_ops<kStoresPerHead>();
      weight_table(smem + ((hh + 1) % kNBuf) * kBufBytes, tid);
      lds_barrier();
    }
  }
}

// Built for bf16 io, headdim 64, dstate <= 128 and chunk 256; the store
// range of a chunk (256 rows of H * 64 values) must fit the 32-bit buffer
// offsets.
int out_resident_supported(int io_bf16, int64_t H, int64_t P, int64_t N, int Q) {
  return io_bf16 && P == kRsP && N <= 32 * kRsNK && Q == kRsQ && H * P <= ((int64_t)1 << 22);
}

// Heads per workgroup: the fewest splits of a group's heads that still give
// every CU a workgroup (one workgroup fills a CU).
static int resident_splits(int64_t ngrp, int64_t hg) {
  int64_t k = (256 + ngrp - 1) / ngrp;
  if (k > hg) k = hg;
  if (k < 1) k = 1;
  return (int)k;
}

hipError_t launch_out_resident(const void* x, const void* Bm, const void* Cm, const float* Gw,
                               const float* dtw, const void* Hc, const float* Dv, void* y,
                               StatusRef flag, int64_t batch, int64_t L, int64_t H, int64_t N,
                               int64_t G, int64_t T_, int64_t ldw, hipStream_t stream) {
  const int64_t ngrp = batch * T_ * G;
  const int64_t hg = H / G;
  const int nsplit = resident_splits(ngrp, hg);
  const int hpw = (int)((hg + nsplit - 1) / nsplit);
  const int64_t nblocks = ((ngrp + 7) / 8) * 8 * nsplit;
  const int nk = nk_class(N);
  auto kern = nk == 1 ? out_resident_kernel<1> : nk == 2 ? out_resident_kernel<2> : out_resident_kernel<4>;
  const hipError_t e = nk == 1   ? ensure_dyn_lds<out_resident_kernel<1>>(kRsLds)
                       : nk == 2 ? ensure_dyn_lds<out_resident_kernel<2>>(kRsLds)
                                 : ensure_dyn_lds<out_resident_kernel<4>>(kRsLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(kRsThreads), kRsLds, stream,
                     static_cast<const bf16*>(x), static_cast<const bf16*>(Bm),
                     static_cast<const bf16*>(Cm), Gw, dtw, static_cast<const bf16*>(Hc), Dv,
                     static_cast<bf16*>(y), flag, L, (int)H, (int)N, (int)G, (int)T_, ldw,
                     (int)ngrp, nsplit, hpw);
  return hipGetLastError();
}

}  // namespace ssd
