// bwd.hip -- gradients of the chunked scan (the backward pass).
//
// The pages stop at the forward pass and name the backward pass as what end-
// to-end training still needs (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향
// 전달 커널 가속화", closing remarks; brifing.si "Accelerating Mamba-2 ...",
// limitations).  The gradient itself is fixed by the forward definition; this
// file evaluates it chunkwise, with the same decomposition the forward pass
// uses.  For one (b, h), chunk c, tokens i (reading) and j (read), in-chunk
// log2 running sums G, prepared step sizes dt, a_ij = exp2(G_i - G_j) for
// j <= i, H_c the state entering the chunk and L_{c+1} the gradient of the
// state leaving it (dy = gradient of y):
//
//   dx_j = D dy_j + dt_j [ sum_{i>=j} a_ij (C_i.B_j) dy_i + exp2(G_last-G_j) L_{c+1} B_j ]
//   dB_j = dt_j [ sum_{i>=j} a_ij (dy_i.x_j) C_i + exp2(G_last-G_j) L_{c+1}^T x_j ]  (per head)
//   dC_i = sum_{j<=i} a_ij dt_j (dy_i.x_j) B_j + exp2(G_i) H_c^T dy_i                 (per head)
//   P_i  = <dy_i, y_i - D x_i>,    Qr_j = <x_j, lam_j B_j>
//
// where lam_j is the gradient of the state after token j.  The gradient of
// the log-decay of token k is  dl_k = <dfinal, s_L> + sum_{t>=k} (P_t - dt_t Qr_t)
// over the whole sequence (every pair (source, reader) that token k's decay
// sits between is counted by P at the reader and removed by Q at the source
// when the source is at or after k), so
//
//   ddt_k = A dl_k + Qr_k,     dA = sum_k dt_k dl_k,     dD = sum <dy, x>,
//
// and the gradients through the step-size preparation follow by the chain
// rule.  L_c comes from the forward machinery run backwards: chunk c's own
// part  S'_c = sum_i exp2(G_i) dy_i C_i^T  is chunk_state with weights
// exp2(G_i) (x -> dy, B -> C), and  L_c = exp2(G_last(c)) L_{c+1} + S'_c  is
// state_pass in reverse chunk order, started from dfinal; its last carry is
// the gradient of the initial state.
//
// The states H_c and L_c are computed and kept in fp32 whatever the io dtype
// (for bf16 io chunk_state's split form: the weighted inputs formed in fp32,
// split into three bf16 parts, ~24 significant bits, on bf16 MFMA; then the
// fp32 state_pass): dl is a running sum over the whole sequence of terms that
// largely cancel, and bf16 states would put their rounding, summed over
// thousands of tokens, straight into ddt and dA.  (The carried terms below
// stay on the fp32 MFMA: with the split there, both per-chunk kernels spill
// twice as many registers and the pass measured 5.30 ms against 4.52 ms.)
//
// The per-chunk terms: one workgroup per (chunk, part, batch), a part being
// kh consecutive heads of one group, walks 32-token blocks of the chunk; two
// kernels, one for the reading side (dC, P) and one for the read side (dx,
// dB, Qr), each keeping its outputs in registers across the pairs of blocks
// and, for dB and dC, across the part's heads.  Every product runs on MFMA:
// the chunk x chunk products C B^T and dy x^T from io-dtype LDS tiles (bf16
// operands are exact and the sums fp32; fp32 io uses the fp32 MFMA); the
// products with the fp32 weights W, U, V as split-bf16 MFMAs for bf16 io
// (fp32 MFMA for fp32 io); the carried terms, which feed the step-size
// gradient, on the exact fp32 MFMA.  dB and dC are written per part in fp32
// and summed over the parts of a group by a final pass.
//
// The two kernels are bound by VALU issue more than by MFMA or memory, so
// their loops are written for few vector instructions: tile loads issued all
// at once through buffer resources (zero past the valid rows, no fill or
// branch), row/piece indexes from a 24-bit multiply by a reciprocal (no
// run-time division), 16-lane sums on DPP, the wave index as a scalar, the
// weights split to bf16 once by the wave that forms them, the P and Qr pair
// shares summed across lanes once per block, and outputs staged through LDS
// to leave as whole-row 16-byte pieces.
#include "ssd_device.hpp"

namespace ssd {

constexpr int kBwdThreads = 256;

constexpr int kBwdTB = 32;   // token rows per block of a chunk

// Heads per workgroup of the per-chunk kernels at most: a workgroup takes a
// "part", kh consecutive heads of one group, and sums their dB and dC
// contributions in its accumulators, so the parts written out number H / kh.
constexpr int kBwdPartHeadsMax = 8;

// io-dtype tiles in LDS: rows of K values, K rounded up to whole 32-value MFMA
// K-steps (zero-filled) plus 16 bytes against bank conflicts.
__host__ __device__ inline int round32(int v) { return (v + 31) / 32 * 32; }
template <typename T>
__host__ __device__ inline int tile_ld(int K) { return round32(K) + 16 / (int)sizeof(T); }

// LDS bytes of the tile pair both per-chunk kernels stage (every region a
// multiple of 16 bytes)
template <typename T>
__host__ __device__ inline int bwd_pair_bytes(int P, int N) {   // two io tiles: N- and P-wide
  return kBwdTB * (tile_ld<T>(N) + tile_ld<T>(P)) * (int)sizeof(T);
}

// A block's worth of 16-byte pieces per thread, loaded into registers before
// any is written to LDS: every load of a tile is in flight at once, where a
// loop of load-then-write pays one memory latency per piece.  MAXP bounds the
// pieces of one thread (the tile's widest K is known at compile time).  The
// thread index is taken as redefined at every call, so that each piece's
// offsets are computed where they are used rather than hoisted out of the
// block loops and kept live (which spills).
__device__ __forceinline__ int fresh_tid() {
  int v = threadIdx.x;
  __asm__ __volatile__("" : "+v"(v));
  return v;
}

// Piece e of rows of KC pieces (e < 1024, KC <= 256) is row e / KC, piece
// e % KC.  The quotient is (e m) >> 20 with m = floor(2^20 / KC) + 1: for
// e = q KC + f, e m / 2^20 = q + f / KC + e s / (KC 2^20) with 1 <= s <= KC,
// below q + 1 while e KC < 2^20, so it is exact here, on full-rate 24-bit
// multiplies where a division by a run-time value costs a long sequence of
// quarter-rate ones.  m is kernel-uniform (a scalar, computed once).
struct PieceRows {
  unsigned kc, m;
  __device__ __forceinline__ explicit PieceRows(int KC) : kc((unsigned)KC), m((1u << 20) / (unsigned)KC + 1u) {}
  __device__ __forceinline__ unsigned row(unsigned e) const { return __umul24(e, m) >> 20; }
  __device__ __forceinline__ unsigned col(unsigned e, unsigned r) const { return e - __umul24(r, kc); }
};

// byte offsets from a base pointer: a 32-bit offset from a wave-uniform base
// is one scalar-base memory instruction, with no 64-bit address arithmetic
template <typename T>
__device__ __forceinline__ const T* at_bytes(const T* base, unsigned off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ T* at_bytes(T* base, unsigned off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// Loads through a buffer resource that spans the valid rows: a raw buffer
// load past the resource's range returns zero, so rows past the valid ones,
// the pieces of threads beyond the tile and (given an offset past the range)
// the pad columns come back zero with no zero-fill or branch.
constexpr unsigned kOutOfRange = 0x80000000u;
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ vec16 rsrc_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(vec16, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// kBwdTB rows x K io elements (rows `row_stride` apart), K <= KMAX, in
// registers; rows at or past `rows_valid` and the columns from K to the next
// multiple of 32 are zero.
template <int KMAX, typename T>
struct IoTile {
  static constexpr int V = 16 / sizeof(T);
  static constexpr int MAXP = (kBwdTB * KMAX / V + kBwdThreads - 1) / kBwdThreads;
  vec16 v[MAXP];
  __device__ __forceinline__ void load(const T* src, int64_t row_stride, int rows_valid, int K) {
    const PieceRows pr(round32(K) / V);
    const unsigned t = fresh_tid(), rs = (unsigned)row_stride * sizeof(T);
    const __amdgpu_buffer_rsrc_t rr = rows_rsrc(src, (unsigned)rows_valid * rs);
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const unsigned e = t + k * kBwdThreads, r = pr.row(e), c = pr.col(e, r) * V;
      const bool in = e < kBwdTB * pr.kc && (int)c < K;
      v[k] = rsrc_load16(rr, in ? r * rs + c * sizeof(T) : kOutOfRange);
    }
  }
  // into an LDS tile of row stride ld
  __device__ __forceinline__ void store(T* dst, int ld, int K) const {
    const PieceRows pr(round32(K) / V);
    const unsigned t = fresh_tid();
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const unsigned e = t + k * kBwdThreads, r = pr.row(e), c = pr.col(e, r) * V;
      if (e < kBwdTB * pr.kc) store16(dst + __umul24(r, (unsigned)ld) + c, v[k]);
    }
  }
};

// 32 fp32 state rows (row r at src + r N, N <= NMAX values, N a multiple of
// 4) in registers; rows at or past `rows_valid` and the columns from N to NR
// are zero.
template <int NMAX>
struct StateRows {
  static constexpr int MAXP = (32 * NMAX / 4 + kBwdThreads - 1) / kBwdThreads;
  float4 v[MAXP];
  __device__ __forceinline__ void load(const float* src, int rows_valid, int N, int NR) {
    const PieceRows pr(NR / 4);
    const unsigned t = fresh_tid();
    const __amdgpu_buffer_rsrc_t rr = rows_rsrc(src, (unsigned)(rows_valid < 32 ? rows_valid : 32) * (unsigned)N * 4u);
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const unsigned e = t + k * kBwdThreads, r = pr.row(e), c = pr.col(e, r) * 4;
      const bool in = e < 32 * pr.kc && (int)c < N;
      v[k] = __builtin_bit_cast(float4, rsrc_load16(rr, in ? (__umul24(r, (unsigned)N) + c) * 4 : kOutOfRange));
    }
  }
  // into LDS rows of `lds` floats (padded strides: four scalar writes)
  __device__ __forceinline__ void store(float* dst, int lds, int NR) const {
    const PieceRows pr(NR / 4);
    const unsigned t = fresh_tid();
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const unsigned e = t + k * kBwdThreads, r = pr.row(e), c = pr.col(e, r) * 4;
      if (e < 32 * pr.kc) {
        float* d = dst + __umul24(r, (unsigned)lds) + c;
        d[0] = v[k].x;
        d[1] = v[k].y;
        d[2] = v[k].z;
        d[3] = v[k].w;
      }
    }
  }
};

// Output rows staged in LDS: 32 fp32 rows of K values (K a multiple of 16),
// row stride K.  When a row holds a multiple of 16 four-value pieces, piece c
// of row r sits at c ^ 4 ((r >> 2) & 3): the four row groups of an MFMA
// accumulator (lanes 16 g .. 16 g + 15 hold rows 4 g + r of 16 columns) then
// write to four different 16-bank groups, and a row reads back as whole
// 16-byte pieces.
__device__ __forceinline__ int stage_at(int r, int col, int K) {
  const int sw = ((K / 4) & 15) == 0 ? 4 * ((r >> 2) & 3) : 0;
  return r * K + (((col >> 2) ^ sw) << 2) + (col & 3);
}

// The first rows_valid staged rows to global rows `row_stride` floats apart,
// as 16-byte pieces (K <= KMAX).
template <int KMAX>
__device__ __forceinline__ void stage_to_global(float* dst, int64_t row_stride, const float* st,
                                                int K, int rows_valid) {
  constexpr int MAXP = (32 * KMAX / 4 + kBwdThreads - 1) / kBwdThreads;
  const PieceRows pr(K / 4);
  const unsigned t = fresh_tid(), rs = (unsigned)row_stride * 4u;
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const unsigned e = t + k * kBwdThreads, r = pr.row(e), c = pr.col(e, r);
    if (e < 32 * pr.kc && (int)r < rows_valid)
      *at_bytes(reinterpret_cast<float4*>(dst), r * rs + c * 16) =
          *reinterpret_cast<const float4*>(st + stage_at(r, 4 * c, K));
  }
}

// 16 bytes of io values
template <typename T>
struct Piece16 {
  T v[16 / sizeof(T)];
};

// Sum over aligned groups of 16 lanes on DPP moves (no LDS round trips): the
// partners at lane xor 1 and xor 2 of each quad, then the mirrored lane of
// each half row (i <-> 7 - i: the other quad) and of the row (i <-> 15 - i:
// the other half).  Each step adds two equal partial sums in either order, so
// every lane of the group ends with the same total.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_src<0xB1, 0xf>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_src<0x4E, 0xf>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_src<0x141, 0xf>(v);   // row_half_mirror
  v += dpp_src<0x140, 0xf>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ int valid_rows(int64_t L, int64_t t0, int TB) {
  const int64_t v = L - t0;
  return v <= 0 ? 0 : (v >= TB ? TB : (int)v);
}

// 16x16 tile of  sum_k A[row][k] B[col][k]  over K (a multiple of 32 after
// padding) for one wave: A rows a0.., B rows b0.. of io tiles with row stride
// ld.  The accumulator holds, in lane l, column l % 16 and rows 4 (l / 16) + r.
// K <= KMAX: the K-steps unrolled, each under a uniform test.
template <int KMAX, typename T>
__device__ __forceinline__ floatx4 tile_dot(const T* A, const T* B, int ld, int K, int lane) {
  const T* pa = A + (lane & 15) * ld + 8 * (lane >> 4);
  const T* pb = B + (lane & 15) * ld + 8 * (lane >> 4);
  floatx4 c = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k0 = 0; k0 < KMAX; k0 += 32)
    if (k0 < K) c = mma(c, load_frag(pa + k0), load_frag(pb + k0));
  return c;
}

// Reading side: dC (summed over the part's heads, fp32) and P for every token
// of one chunk.  Block pairs (I, J <= I) of 32 tokens, for each head of the
// part in turn.  Every product is on MFMA: C B^T and dy x^T from the io-dtype
// tiles (one 16x16 tile of each per wave; io values are exact operands, sums
// fp32), then W = mask exp2(G_i - G_j) dt_j (dy.x) through LDS (as bf16 hi
// and lo planes for bf16 io) and dC += W B, each wave owning 16 rows and
// every other 16-column tile of dC in its accumulators for the whole block
// and all the part's heads.  The carried term exp2(G_i) H_c^T dy_i likewise,
// H_c streamed through LDS 32 state rows (one K-step) at a time.
constexpr int kBwdLdW = kBwdTB + 4;   // fp32 weight rows: 16-byte aligned fragments

template <typename T>
__host__ __device__ inline int bwd_target_bytes(int P, int N) {
  const int pair = bwd_pair_bytes<T>(P, N), st = (32 * (N + 1) * 4 + 15) / 16 * 16;
  return pair + (pair > st ? pair : st) + kBwdTB * kBwdLdW * 4 + 6 * kBwdTB * 4;   // Gi Gj Pp Pc
}

// Four fp32 weights w[r] of one column of a 16 x 16 accumulator tile (rows
// 4 (lane / 16) + r) as bf16 hi = bf16(w) and lo = bf16(w - hi), written to
// k-major (transposed) planes: the four values are contiguous there, one
// 8-byte write per plane, and a consumer reads its row of eight k-values
// with the transposing LDS read, as for the token-major io tiles.
constexpr int kBwdLdT = kBwdTB + 4;   // bf16 plane rows: 72 bytes, 8-byte aligned
static_assert(2 * kBwdTB * kBwdLdT * 2 <= kBwdTB * kBwdLdW * 4, "two planes fill an fp32 weight region");
__device__ __forceinline__ void split_to_planes(const float (&w)[4], bf16* hi_at, bf16* lo_at) {
  bf16x4 hi, lo;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hi[r] = static_cast<bf16>(w[r]);
    lo[r] = static_cast<bf16>(w[r] - static_cast<float>(hi[r]));
  }
  *reinterpret_cast<bf16x4*>(hi_at) = hi;
  *reinterpret_cast<bf16x4*>(lo_at) = lo;
}

// 8 io values (k-contiguous) as an fp32 MFMA fragment
__device__ __forceinline__ floatx8 frag32(const bf16* p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
  floatx8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<float>(v[e]);
  return r;
}
__device__ __forceinline__ floatx8 frag32(const float* p) { return load_frag(p); }

// Occupancy: both per-chunk kernels fit four workgroups per CU in LDS but
// need more than 128 VGPRs.  For bf16 io up to dstate 128 / headdim 64 they
// are built for four waves per SIMD (128 VGPRs, a ~100-byte spill per lane,
// mostly outside the pair loops), which measured faster than three waves
// with no spill.  The wider instantiations would spill several hundred bytes
// and keep the default.
template <typename T, int NKN, int NKP>
constexpr int bwd_min_waves() { return sizeof(T) == 2 && NKN <= 8 && NKP <= 4 ? 4 : 1; }

template <typename T, int NKN, int NKP>
__global__ void __launch_bounds__(kBwdThreads, (bwd_min_waves<T, NKN, NKP>()))
bwd_target_kernel(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                  const T* __restrict__ dy, const float* __restrict__ Gw,
                  const float* __restrict__ dtw, const float* __restrict__ Hc,
                  float* __restrict__ Pout, float* __restrict__ dCh, int64_t L, int H, int P,
                  int N, int G, int hpg, int Q, int T_, int64_t ldw, int p0, int hbp, int kh) {
  constexpr int TB = kBwdTB, ldW = kBwdLdW, NT = NKN / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  // part p0 + blockIdx.y of this launch: heads part kh .. part kh + kh - 1,
  // all of one group; the dC parts of the launch are rows of hbp parts
  const int c = blockIdx.x, part = p0 + (int)blockIdx.y, hfirst = part * kh;
  const int64_t b = blockIdx.z;
  const int g = hfirst / hpg;
  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave tile choices become uniform branches
  const int lane = tid % kWave, wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ti2 = wv >> 1, tj2 = wv & 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  // second-stage ownership: rows 16 ib .. +15, column tiles nh, nh + 2, ...
  const int ib = wv & 1, nh = wv >> 1;
  const int ldN = tile_ld<T>(N), ldP = tile_ld<T>(P), NR = round32(N), PR = round32(P);
  const int pair = bwd_pair_bytes<T>(P, N), st = (32 * (N + 1) * 4 + 15) / 16 * 16;
  T* Ct = reinterpret_cast<T*>(smem);
  T* gt = Ct + TB * ldN;
  unsigned char* U = smem + pair;
  T* Bt = reinterpret_cast<T*>(U);
  T* xt = Bt + TB * ldN;
  float* Hs = reinterpret_cast<float*>(U);
  float* Ws = reinterpret_cast<float*>(U + (pair > st ? pair : st));
  float* Gi = Ws + TB * ldW;
  float* Gj = Gi + TB;
  float* Pp = Gj + TB;          // [2][TB]: pair shares of P from the two column-half waves
  float* Pc = Pp + 2 * TB;      // [2][TB]: carried shares of P
  const int nb = Q / TB, ntiles = N / 16;

  for (int I = 0; I < nb; ++I) {
    const int64_t ti0 = (int64_t)c * Q + I * TB;
    const int vi = valid_rows(L, ti0, TB);
    if (vi == 0) break;                       // the rest of the chunk is padding
    // the block's dC, summed over the part's heads in ascending order
    floatx4 dc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) dc[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int hh = 0; hh < kh; ++hh) {
      const int h = hfirst + hh;
      const float* Grow = Gw + (b * H + h) * ldw + (int64_t)c * Q;
      const float* drow = dtw + (b * H + h) * ldw + (int64_t)c * Q;
      const float* Hrow = Hc + ((b * H + h) * T_ + c) * (int64_t)P * N;
      {
        const float gi = tid < TB ? Grow[I * TB + tid] : 0.0f;
        IoTile<16 * NKN, T> tc;            // C rows: the same for every head of the part
        IoTile<16 * NKP, T> tg;
        if (hh == 0) tc.load(Cm + ((b * L + ti0) * G + g) * N, (int64_t)G * N, vi, N);
        tg.load(dy + ((b * L + ti0) * H + h) * P, (int64_t)H * P, vi, P);
        __syncthreads();
        if (hh == 0) tc.store(Ct, ldN, N);
        tg.store(gt, ldP, P);
        if (tid < TB) Gi[tid] = gi;
      }
      // P's pair shares: each lane keeps its rows' products over all the pairs
      // (its rows and column offset are the same in every pair) and the sums
      // over the 16 lanes of a row are taken once, after the pairs
      float pa[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int J = 0; J <= I; ++J) {
        const int64_t tj0 = (int64_t)c * Q + J * TB;
        const int vj = valid_rows(L, tj0, TB);
        const int j = 16 * tj2 + l16;
        const float dj = drow[J * TB + j];
        {
          const float gj = tid < TB ? Grow[J * TB + tid] : 0.0f;
          IoTile<16 * NKN, T> tb;
          IoTile<16 * NKP, T> tx;
          tb.load(Bm + ((b * L + tj0) * G + g) * N, (int64_t)G * N, vj, N);
          tx.load(x + ((b * L + tj0) * H + h) * P, (int64_t)H * P, vj, P);
          __syncthreads();
          tb.store(Bt, ldN, N);
          tx.store(xt, ldP, P);
          if (tid < TB) Gj[tid] = gj;
        }
        __syncthreads();
        // this wave's tile: rows i = 16 ti2 + 4 (lane / 16) + r, column j = 16 tj2 + lane % 16
        const floatx4 cb = tile_dot<16 * NKN>(Ct + 16 * ti2 * ldN, Bt + 16 * tj2 * ldN, ldN, NR, lane);
        const floatx4 gx = tile_dot<16 * NKP>(gt + 16 * ti2 * ldP, xt + 16 * tj2 * ldP, ldP, PR, lane);
        float wr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ti2 + 4 * g4 + r;
          const bool on = J < I || j <= i;
          // every entry is evaluated (the running sums and step sizes are finite
          // on padding tokens too) and the masked ones selected away: a select,
          // where a conditional LDS read would be an exec-mask branch
          const float gi = Gi[i], gj = Gj[j];
          const float w = on ? fast_exp2(gi - gj) * dj * gx[r] : 0.0f;
          wr[r] = w;
          if constexpr (sizeof(T) != 2) Ws[i * ldW + j] = w;
          pa[r] = fmaf(w, cb[r], pa[r]);
        }
        // bf16 io: W as hi and lo planes, k-major (row j, columns i)
        bf16* const Wh = reinterpret_cast<bf16*>(Ws);
        bf16* const Wl = Wh + TB * kBwdLdT;
        if constexpr (sizeof(T) == 2)
          split_to_planes(wr, Wh + j * kBwdLdT + 16 * ti2 + 4 * g4, Wl + j * kBwdLdT + 16 * ti2 + 4 * g4);
        __syncthreads();
        // dC rows 16 ib + .. += W[rows][0..31] B[0..31][tile columns]
        if constexpr (sizeof(T) == 2) {
          // bf16 io: W's hi and lo planes and B's token-major fragment by
          // transposing LDS reads
          const bf16x8 wh = frag_tokens(Wh, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * ib, lane);
          const bf16x8 wl = frag_tokens(Wl, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * ib, lane);
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            const int nt = nh + 2 * q;
            if (nt < ntiles) {
              const bf16x8 bq = frag_tokens(reinterpret_cast<const bf16*>(Bt), ldN, 8 * g4,
                                            8 * g4 + 4, 16 * nt, lane);
              dc[q] = mma(mma(dc[q], wh, bq), wl, bq);
            }
          }
        } else {
          const floatx8 a = load_frag(Ws + (16 * ib + l16) * ldW + 8 * g4);
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            const int nt = nh + 2 * q;
            if (nt < ntiles) {
              floatx8 bq;
#pragma unroll
              for (int e = 0; e < 8; ++e) bq[e] = to_f32(Bt[(8 * g4 + e) * ldN + 16 * nt + l16]);
              dc[q] = mma(dc[q], a, bq);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = sum16(pa[r]);
        if (l16 == 0) Pp[tj2 * TB + 16 * ti2 + 4 * g4 + r] = s;
      }
      // carried term exp2(G_i) H_c^T dy_i: H_c through LDS 32 state rows at a time
      floatx4 hc[NT];
#pragma unroll
      for (int q = 0; q < NT; ++q) hc[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int p0 = 0; p0 < P; p0 += 32) {
        {
          StateRows<16 * NKN> hs;
          hs.load(Hrow + (int64_t)p0 * N, P - p0, N, N);
          __syncthreads();
          hs.store(Hs, N + 1, N);
        }
        __syncthreads();
        const floatx8 a = frag32(gt + (16 * ib + l16) * ldP + p0 + 8 * g4);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          const int nt = nh + 2 * q;
          if (nt < ntiles) {
            floatx8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = Hs[(8 * g4 + e) * (N + 1) + 16 * nt + l16];
            hc[q] = mma(hc[q], a, bq);
          }
        }
      }
      // rows i = 16 ib + 4 (lane / 16) + r, column 16 nt + lane % 16 of each tile
      float pc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ib + 4 * g4 + r;
        const float e = fast_exp2(Gi[i]);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          const int nt = nh + 2 * q;
          if (nt < ntiles) {
            const float v = e * hc[q][r];
            dc[q][r] += v;
            pc[r] = fmaf(v, to_f32(Ct[i * ldN + 16 * nt + l16]), pc[r]);
          }
        }
        pc[r] = sum16(pc[r]);
        if (l16 == 0) Pc[nh * TB + i] = pc[r];
      }
      __syncthreads();
      if (tid < vi) Pout[(b * H + h) * ldw + (int64_t)c * Q + I * TB + tid] =
            (Pp[tid] + Pp[TB + tid]) + (Pc[tid] + Pc[TB + tid]);
    }   // heads of the part
    // the block's dC rows through LDS where the state rows were (every wave
    // is past the last head's carried term), then out as whole-row pieces
    float* Ds = reinterpret_cast<float*>(U);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ib + 4 * g4 + r;
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const int nt = nh + 2 * q;
        if (nt < ntiles) Ds[stage_at(i, 16 * nt + l16, N)] = dc[q][r];
      }
    }
    __syncthreads();
    stage_to_global<16 * NKN>(dCh + ((b * L + ti0) * hbp + (part - p0)) * (int64_t)N,
                              (int64_t)hbp * N, Ds, N, vi);
  }
}

// Read side: dx, dB (summed over the part's heads, fp32), Qr and the chunk's
// share of dD.  Block pairs (J, I >= J) of 32 tokens, for each head of the
// part in turn, every product on MFMA: B C^T and x dy^T from the io-dtype
// tiles, U = mask exp2(G_i - G_j) (C.B) and V = mask exp2(G_i - G_j) dt_j
// (dy.x) through LDS (bf16 hi and lo planes for bf16 io), then dx += U dy
// and dB += V C, each wave owning 16 rows j and every other 16-column tile
// of dx and dB (dB across the part's heads, dx per head).  The carried terms
// come from L_{c+1} streamed through LDS 32 state rows at a time:
// exp2(G_last - G_j) (B_j L^T) into dx and exp2(G_last - G_j) dt_j (x_j L)
// into dB, the factor folded into the row's operand fragment.
template <typename T>
__host__ __device__ inline int bwd_source_bytes(int P, int N) {
  const int pair = bwd_pair_bytes<T>(P, N), st = (32 * (round32(N) + 1) * 4 + 15) / 16 * 16;
  return pair + (pair > st ? pair : st) + 2 * kBwdTB * kBwdLdW * 4 + 8 * kBwdTB * 4 +
         kBwdPartHeadsMax * (kBwdThreads / kWave) * 4;
}

template <typename T, int NKN, int NKP>
__global__ void __launch_bounds__(kBwdThreads, (bwd_min_waves<T, NKN, NKP>()))
bwd_source_kernel(const T* __restrict__ x, const T* __restrict__ Bm, const T* __restrict__ Cm,
                  const T* __restrict__ dy, const float* __restrict__ Gw,
                  const float* __restrict__ dtw, const float* __restrict__ Lam,
                  const float* __restrict__ Dv, T* __restrict__ dx, float* __restrict__ dBh,
                  float* __restrict__ Qout, float* __restrict__ dDpart, int64_t L, int H, int P,
                  int N, int G, int hpg, int Q, int T_, int64_t ldw, int p0, int hbp, int kh) {
  constexpr int TB = kBwdTB, ldW = kBwdLdW, NT = NKN / 2, PT = NKP / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  // part p0 + blockIdx.y of this launch: heads part kh .. part kh + kh - 1,
  // all of one group; the dB parts of the launch are rows of hbp parts
  const int c = blockIdx.x, part = p0 + (int)blockIdx.y, hfirst = part * kh;
  const int64_t b = blockIdx.z;
  const int g = hfirst / hpg;
  const int tid = threadIdx.x;
  // the wave index as a scalar: per-wave tile choices become uniform branches
  const int lane = tid % kWave, wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int tj2 = wv >> 1, ti2 = wv & 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  // second-stage ownership: rows j = 16 jb .. +15, column tiles nh, nh + 2, ...
  const int jb = wv & 1, nh = wv >> 1;
  const int ldN = tile_ld<T>(N), ldP = tile_ld<T>(P), NR = round32(N), PR = round32(P);
  const int lsN = NR + 1;       // state-pass rows, zero-padded to whole K-steps
  const int pair = bwd_pair_bytes<T>(P, N), st = (32 * lsN * 4 + 15) / 16 * 16;
  T* Bt = reinterpret_cast<T*>(smem);
  T* xt = Bt + TB * ldN;
  unsigned char* U = smem + pair;
  T* Ct = reinterpret_cast<T*>(U);
  T* gt = Ct + TB * ldN;
  float* Ls = reinterpret_cast<float*>(U);
  float* Us = reinterpret_cast<float*>(U + (pair > st ? pair : st));
  float* Vs = Us + TB * ldW;
  float* Gi = Vs + TB * ldW;
  float* Gj = Gi + TB;
  float* dj = Gj + TB;
  float* Qp = dj + TB;          // [2][TB]: pair shares of Qr from the two column-half waves
  float* Qc = Qp + 2 * TB;      // [2][TB]: carried shares of Qr
  float* dDw = Qc + 3 * TB;     // [head of the part][wave]: shares of dD
  const int nb = Q / TB, ntn = N / 16, ntp = P / 16;
  if (lane == 0)
    for (int hh = 0; hh < kh; ++hh) dDw[hh * (kBwdThreads / kWave) + wv] = 0.0f;

  for (int J = 0; J < nb; ++J) {
    const int64_t tj0 = (int64_t)c * Q + J * TB;
    const int vj = valid_rows(L, tj0, TB);
    if (vj == 0) break;
    // the block's dB, summed over the part's heads in ascending order, each
    // head's step sizes folded into its operands
    floatx4 dba[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) dba[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int hh = 0; hh < kh; ++hh) {
      const int h = hfirst + hh;
      const float* Grow = Gw + (b * H + h) * ldw + (int64_t)c * Q;
      const float* drow = dtw + (b * H + h) * ldw + (int64_t)c * Q;
      const float* Lrow = Lam + ((b * H + h) * T_ + c) * (int64_t)P * N;
      const float Dh = Dv ? Dv[h] : 0.0f;
      const float Gl = Grow[Q - 1];
      float dsum = 0.0f;
      {
        const float gj = tid < TB ? Grow[J * TB + tid] : 0.0f;
        const float dv = tid < TB ? drow[J * TB + tid] : 0.0f;
        IoTile<16 * NKN, T> tb;            // B rows: the same for every head of the part
        IoTile<16 * NKP, T> tx;
        if (hh == 0) tb.load(Bm + ((b * L + tj0) * G + g) * N, (int64_t)G * N, vj, N);
        tx.load(x + ((b * L + tj0) * H + h) * P, (int64_t)H * P, vj, P);
        __syncthreads();
        if (hh == 0) tb.store(Bt, ldN, N);
        tx.store(xt, ldP, P);
        if (tid < TB) {
          Gj[tid] = gj;
          dj[tid] = dv;
        }
      }
      floatx4 dxa[PT];
#pragma unroll
      for (int q = 0; q < PT; ++q) dxa[q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      // Qr's pair shares: each lane keeps its rows' products over all the
      // pairs, summed over the 16 lanes of a row once, after the pairs
      float qa[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int I = J; I < nb; ++I) {
        const int64_t ti0 = (int64_t)c * Q + I * TB;
        const int vi = valid_rows(L, ti0, TB);
        if (vi == 0) break;
        {
          const float gi = tid < TB ? Grow[I * TB + tid] : 0.0f;
          IoTile<16 * NKN, T> tc;
          IoTile<16 * NKP, T> tg;
          tc.load(Cm + ((b * L + ti0) * G + g) * N, (int64_t)G * N, vi, N);
          tg.load(dy + ((b * L + ti0) * H + h) * P, (int64_t)H * P, vi, P);
          __syncthreads();
          tc.store(Ct, ldN, N);
          tg.store(gt, ldP, P);
          if (tid < TB) Gi[tid] = gi;
        }
        __syncthreads();
        // this wave's tile: rows j = 16 tj2 + 4 (lane / 16) + r, column i = 16 ti2 + lane % 16
        const floatx4 cb = tile_dot<16 * NKN>(Bt + 16 * tj2 * ldN, Ct + 16 * ti2 * ldN, ldN, NR, lane);
        const floatx4 gx = tile_dot<16 * NKP>(xt + 16 * tj2 * ldP, gt + 16 * ti2 * ldP, ldP, PR, lane);
        const int i = 16 * ti2 + l16;
        float ur[4], vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * tj2 + 4 * g4 + r;
          const bool on = I > J || j <= i;
          const float gi = Gi[i], gj = Gj[j];     // read unconditionally: a select, not a branch
          const float a = on ? fast_exp2(gi - gj) : 0.0f;
          const float u = a * cb[r];
          ur[r] = u;
          vr[r] = a * gx[r] * dj[j];              // dB's weights carry dt_j
          if constexpr (sizeof(T) != 2) {
            Us[j * ldW + i] = u;
            Vs[j * ldW + i] = vr[r];
          }
          qa[r] = fmaf(u, gx[r], qa[r]);
        }
        // bf16 io: U and V as hi and lo planes, k-major (row i, columns j)
        bf16* const Uh = reinterpret_cast<bf16*>(Us);
        bf16* const Ul = Uh + TB * kBwdLdT;
        bf16* const Vh = reinterpret_cast<bf16*>(Vs);
        bf16* const Vl = Vh + TB * kBwdLdT;
        if constexpr (sizeof(T) == 2) {
          split_to_planes(ur, Uh + i * kBwdLdT + 16 * tj2 + 4 * g4, Ul + i * kBwdLdT + 16 * tj2 + 4 * g4);
          split_to_planes(vr, Vh + i * kBwdLdT + 16 * tj2 + 4 * g4, Vl + i * kBwdLdT + 16 * tj2 + 4 * g4);
        }
        __syncthreads();
        // rows 16 jb + ..: dB += V[rows][0..31] C[0..31][tiles], dx += U[rows][..] dy[..][tiles]
        if constexpr (sizeof(T) == 2) {
          // bf16 io: U's and V's hi and lo planes, C's and dy's token-major
          // fragments by transposing LDS reads
          const bf16x8 vh = frag_tokens(Vh, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * jb, lane);
          const bf16x8 vl = frag_tokens(Vl, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * jb, lane);
          const bf16x8 uh = frag_tokens(Uh, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * jb, lane);
          const bf16x8 ul = frag_tokens(Ul, kBwdLdT, 8 * g4, 8 * g4 + 4, 16 * jb, lane);
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            const int nt = nh + 2 * q;
            if (nt < ntn) {
              const bf16x8 bq = frag_tokens(reinterpret_cast<const bf16*>(Ct), ldN, 8 * g4,
                                            8 * g4 + 4, 16 * nt, lane);
              dba[q] = mma(mma(dba[q], vh, bq), vl, bq);
            }
          }
#pragma unroll
          for (int q = 0; q < PT; ++q) {
            const int pt = nh + 2 * q;
            if (pt < ntp) {
              const bf16x8 bq = frag_tokens(reinterpret_cast<const bf16*>(gt), ldP, 8 * g4,
                                            8 * g4 + 4, 16 * pt, lane);
              dxa[q] = mma(mma(dxa[q], uh, bq), ul, bq);
            }
          }
        } else {
          const floatx8 av = load_frag(Vs + (16 * jb + l16) * ldW + 8 * g4);
          const floatx8 au = load_frag(Us + (16 * jb + l16) * ldW + 8 * g4);
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            const int nt = nh + 2 * q;
            if (nt < ntn) {
              floatx8 bq;
#pragma unroll
              for (int e = 0; e < 8; ++e) bq[e] = to_f32(Ct[(8 * g4 + e) * ldN + 16 * nt + l16]);
              dba[q] = mma(dba[q], av, bq);
            }
          }
#pragma unroll
          for (int q = 0; q < PT; ++q) {
            const int pt = nh + 2 * q;
            if (pt < ntp) {
              floatx8 bq;
#pragma unroll
              for (int e = 0; e < 8; ++e) bq[e] = to_f32(gt[(8 * g4 + e) * ldP + 16 * pt + l16]);
              dxa[q] = mma(dxa[q], au, bq);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = sum16(qa[r]);
        if (l16 == 0) Qp[ti2 * TB + 16 * tj2 + 4 * g4 + r] = s;
      }
      // carried terms, L_{c+1} through LDS 32 state rows (p0 .. p0+31) at a time;
      // this wave's A-operand row j = 16 jb + lane % 16 carries exp2(G_last - G_j)
      const float erow = fast_exp2(Gl - Gj[16 * jb + l16]);
      const float erow_b = erow * dj[16 * jb + l16];    // dB's rows carry dt_j too
      float qx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int p0 = 0; p0 < P; p0 += 32) {
        {
          StateRows<16 * NKN> ls;
          ls.load(Lrow + (int64_t)p0 * N, P - p0, N, NR);
          __syncthreads();
          ls.store(Ls, lsN, NR);
        }
        __syncthreads();
        // dx tile (rows j, columns p = p0 + 16 nh + lane % 16) += e_j sum_n B[j][n] L[p][n]
        const int q = p0 / 32;
        if (16 * nh + p0 < P) {
          floatx4 cj = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
          for (int k0 = 0; k0 < NR; k0 += 32) {
            floatx8 a = frag32(Bt + (16 * jb + l16) * ldN + k0 + 8 * g4);
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] *= erow;
            floatx8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = Ls[(16 * nh + l16) * lsN + k0 + 8 * g4 + e];
            cj = mma(cj, a, bq);
          }
#pragma unroll
          for (int qq = 0; qq < PT; ++qq)
            if (qq == q) dxa[qq] += cj;
          // Qr's carried share: sum_p x[j][p] (e_j B_j L^T)[p]
          const int p = p0 + 16 * nh + l16;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            qx[r] = fmaf(to_f32(xt[(16 * jb + 4 * g4 + r) * ldP + p]), cj[r], qx[r]);
        }
        // dB tiles (rows j, columns n) += e_j sum_{p in pass} x[j][p] L[p][n]
        floatx8 a = frag32(xt + (16 * jb + l16) * ldP + p0 + 8 * g4);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] *= erow_b;
#pragma unroll
        for (int qq = 0; qq < NT; ++qq) {
          const int nt = nh + 2 * qq;
          if (nt < ntn) {
            floatx8 bq;
#pragma unroll
            for (int e = 0; e < 8; ++e) bq[e] = Ls[(8 * g4 + e) * lsN + 16 * nt + l16];
            dba[qq] = mma(dba[qq], a, bq);
          }
        }
      }
      // rows j = 16 jb + 4 (lane / 16) + r, column 16 tile + lane % 16
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jb + 4 * g4 + r;
        const float qs = sum16(qx[r]);
        if (l16 == 0) Qc[nh * TB + j] = qs;
      }
      // this head's dx 64 columns at a time through LDS where the pair weights
      // were (U and V: 32 x 72 floats; the last pair is behind the carried
      // term's barriers), then out as whole-row pieces; dx = dt_j dxa + D dy
      // with dy read as row pieces alongside, which also gives the dD share
      float* Xs = Us;
      for (int pg = 0; 64 * pg < P; ++pg) {
        if (pg > 0) __syncthreads();                 // the previous group is out
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jb + 4 * g4 + r;
#pragma unroll
          for (int q = 0; q < PT; ++q) {
            const int pt = nh + 2 * q;
            if (pt < ntp && pt / 4 == pg) Xs[stage_at(j, 16 * pt + l16 - 64 * pg, 64)] = dxa[q][r];
          }
        }
        __syncthreads();
        if (pg == 0 && tid < vj)
          Qout[(b * H + h) * ldw + (int64_t)c * Q + J * TB + tid] =
              (Qp[tid] + Qp[TB + tid]) + (Qc[tid] + Qc[TB + tid]);
        // dx pieces of V values: columns 64 pg .. 64 pg + W - 1 of rows j < vj
        constexpr int V = 16 / sizeof(T), MAXP = (32 * 64 / V + kBwdThreads - 1) / kBwdThreads;
        const int W = P - 64 * pg < 64 ? P - 64 * pg : 64;
        const PieceRows pr(W / V);
        const unsigned t = fresh_tid(), rs = (unsigned)(H * P) * sizeof(T);
        const int64_t base = ((b * L + tj0) * H + h) * P + 64 * pg;   // row 0, column 64 pg
#pragma unroll
        for (int k = 0; k < MAXP; ++k) {
          const unsigned e = t + k * kBwdThreads, r = pr.row(e), col = pr.col(e, r) * V;
          if (e < 32 * pr.kc && (int)r < vj) {
            const unsigned off = r * rs + col * sizeof(T);
            const Piece16<T> gv = __builtin_bit_cast(Piece16<T>, load16(at_bytes(dy + base, off)));
            const Piece16<T> xv = __builtin_bit_cast(
                Piece16<T>, load16(xt + __umul24(r, (unsigned)ldP) + 64 * pg + col));
            const float d = dj[r];
            Piece16<T> o;
#pragma unroll
            for (int v4 = 0; v4 < V; v4 += 4) {
              const float4 s = *reinterpret_cast<const float4*>(Xs + stage_at(r, col + v4, 64));
              const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const float g = to_f32(gv.v[v4 + u]);
                o.v[v4 + u] = to_io<T>(fmaf(d, sv[u], Dh * g));
                dsum = fmaf(g, to_f32(xv.v[v4 + u]), dsum);
              }
            }
            store16(at_bytes(dx + base, off), __builtin_bit_cast(vec16, o));
          }
        }
      }
      // this head's share of dD = sum <dy, x> over the block, added to the
      // wave's slot (each wave its own: no race, a fixed order)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off, kWave);
      if (lane == 0) dDw[hh * (kBwdThreads / kWave) + wv] += dsum;
    }   // heads of the part
    // the block's dB rows through LDS where the state rows were (every wave
    // is past the last head's carried term), then out as whole-row pieces
    float* Ds = reinterpret_cast<float*>(U);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * jb + 4 * g4 + r;
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const int nt = nh + 2 * q;
        if (nt < ntn) Ds[stage_at(j, 16 * nt + l16, N)] = dba[q][r];
      }
    }
    __syncthreads();
    stage_to_global<16 * NKN>(dBh + ((b * L + tj0) * hbp + (part - p0)) * (int64_t)N,
                              (int64_t)hbp * N, Ds, N, vj);
  }
  // the chunk's shares of dD, one per head of the part
  __syncthreads();
  if (tid < kh) {
    const float* w = dDw + tid * (kBwdThreads / kWave);
    dDpart[(b * T_ + c) * H + hfirst + tid] = w[0] + w[1] + w[2] + w[3];
  }
}

constexpr int kDtThreads = 512;   // threads of the step-size gradient kernel

// Step-size gradients of one (b, h): the reverse running sum of P - dt Qr over
// the whole sequence (fp64), then ddt, the (b, h) shares of dA and of the
// bias gradient, with the step-size preparation's chain rule when XF is set.
// The sequence is walked in blocks of 2048 tokens from its end.  Each of the
// 512 threads takes 4 contiguous tokens of a block (one 16-byte load per
// array, the wave's loads contiguous; past L they load zero), a suffix scan of the
// threads' sums (within a wave on shuffles, then over the waves) gives each
// thread the sum of every later token of the block, and a carry, started at
// <dfinal, final state>, brings the later blocks' total.
template <bool XF>
__global__ void __launch_bounds__(kDtThreads)
bwd_dt_kernel(const float* __restrict__ Pb, const float* __restrict__ Qb,
              const float* __restrict__ dtw, const float* __restrict__ dt_in,
              const float* __restrict__ A, const float* __restrict__ dfinal,
              const float* __restrict__ fin, DtXform xf, float* __restrict__ ddt,
              double* __restrict__ dApart, double* __restrict__ dbpart, int64_t L, int H,
              int64_t PN, int64_t ldw) {
  constexpr int TPT = 4, NW = kDtThreads / kWave;
  constexpr int BLK = kDtThreads * TPT;
  __shared__ double wsum[NW];
  __shared__ double red[2][NW];
  const int h = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int64_t bh = b * H + h;

  // <dfinal, final state>: every token's decay lies before the final state
  double kf = 0.0;
  if (dfinal)
    for (int64_t e = tid; e < PN; e += kDtThreads) kf += (double)dfinal[bh * PN + e] * fin[bh * PN + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kf += __shfl_xor(kf, off, kWave);
  if (lane == 0) red[0][wv] = kf;
  __syncthreads();
  double carry = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) carry += red[0][w];

  const float a = A[h];
  const unsigned row_bytes = (unsigned)L * 4u;
  const __amdgpu_buffer_rsrc_t rp = rows_rsrc(Pb + bh * ldw, row_bytes);
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(Qb + bh * ldw, row_bytes);
  const __amdgpu_buffer_rsrc_t rd = rows_rsrc(dtw + bh * ldw, row_bytes);
  double da = 0.0, db = 0.0;
  for (int64_t blk = (L + BLK - 1) / BLK - 1; blk >= 0; --blk) {
    const int64_t t0 = blk * BLK + (int64_t)tid * TPT;
    const unsigned off = (unsigned)t0 * 4u;
    float pv[TPT], qv[TPT], dv[TPT], xv[TPT];
#pragma unroll
    for (int k = 0; k < TPT / 4; ++k) {
      const float4 p4 = __builtin_bit_cast(float4, rsrc_load16(rp, off + 16 * k));
      const float4 q4 = __builtin_bit_cast(float4, rsrc_load16(rq, off + 16 * k));
      const float4 d4 = __builtin_bit_cast(float4, rsrc_load16(rd, off + 16 * k));
      pv[4 * k] = p4.x; pv[4 * k + 1] = p4.y; pv[4 * k + 2] = p4.z; pv[4 * k + 3] = p4.w;
      qv[4 * k] = q4.x; qv[4 * k + 1] = q4.y; qv[4 * k + 2] = q4.z; qv[4 * k + 3] = q4.w;
      dv[4 * k] = d4.x; dv[4 * k + 1] = d4.y; dv[4 * k + 2] = d4.z; dv[4 * k + 3] = d4.w;
    }
    // a piece that straddles L is not zeroed dword by dword, and the rows
    // hold stale values past L: tokens from L on are cleared here
#pragma unroll
    for (int e = 0; e < TPT; ++e)
      if (t0 + e >= L) pv[e] = qv[e] = dv[e] = 0.0f;
    if constexpr (XF) {
#pragma unroll
      for (int e = 0; e < TPT; ++e) xv[e] = t0 + e < L ? dt_in[(b * L + t0 + e) * H + h] : 0.0f;
    }
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < TPT; ++e) s += (double)pv[e] - (double)dv[e] * qv[e];
    // inclusive sum over this lane and the later lanes of the wave
    double inc = s;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double v = __shfl_down(inc, o, kWave);
      if (lane + o < kWave) inc += v;
    }
    const double nxt = __shfl_down(inc, 1, kWave);          // every lane takes part
    const double later_lanes = lane + 1 < kWave ? nxt : 0.0;
    if (lane == 0) wsum[wv] = inc;
    __syncthreads();
    double run = carry, tot = 0.0;
#pragma unroll
    for (int w = NW - 1; w >= 0; --w) {
      if (w > wv) run += wsum[w];
      tot += wsum[w];
    }
    __syncthreads();                             // wsum is rewritten by the next block
    run += later_lanes;
    carry += tot;
    // this thread's tokens, last first
#pragma unroll
    for (int e = TPT - 1; e >= 0; --e) {
      const int64_t t = t0 + e;
      run += (double)pv[e] - (double)dv[e] * qv[e];
      if (t < L) {
        const float dl = (float)run;
        float gdt = fmaf(a, dl, qv[e]);
        da += (double)dv[e] * run;
        if constexpr (XF) {
          float v = xv[e];
          if (xf.bias) v += xf.bias[h];
          float w = v, sig = 1.0f;
          if (xf.softplus) {
            w = softplus_f32(v);
            sig = 1.0f / (1.0f + fast_exp2(-v * kLog2e));
          }
          gdt = (w >= xf.lo && w <= xf.hi) ? gdt * sig : 0.0f;
        }
        db += gdt;
        ddt[(b * L + t) * H + h] = gdt;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    da += __shfl_xor(da, off, kWave);
    db += __shfl_xor(db, off, kWave);
  }
  __syncthreads();
  if (lane == 0) {
    red[0][wv] = da;
    red[1][wv] = db;
  }
  __syncthreads();
  if (tid == 0) {
    double sa = 0.0, sb = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sa += red[0][w];
      sb += red[1][w];
    }
    dApart[bh] = sa;
    dbpart[bh] = sb;
  }
}

// weights exp2(G) of the reversed chunk contributions (0 on padding tokens),
// and an all-zero running sum so that chunk_state's exp2(G_last - G_j) is 1
__global__ void __launch_bounds__(kBwdThreads)
bwd_prep_kernel(const float* __restrict__ Gw, float* __restrict__ w2, float* __restrict__ Gz,
                int64_t total, int64_t L, int64_t ldw) {
  for (int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kBwdThreads) {
    w2[e] = e % ldw < L ? fast_exp2(Gw[e]) : 0.0f;
    Gz[e] = 0.0f;
  }
}

// dB and dC: sums over each group of the fp32 parts the chunk kernels write,
// one part per kh consecutive heads of a group (the part's heads already
// summed in ascending order).  Here `H` counts parts and `hpg` parts per
// group; one batch of parts h0 .. h0 + nb - 1 at a time (rows of hb parts).
// Each element adds its group's parts of the batch in ascending order to the
// running fp32 sum (starting from zero at the group's first part) and, at the
// group's last part, stores the io-dtype result: the order of additions is
// that of one pass over all the parts, whatever the batches.  Only the
// groups g0 .. g0 + ng - 1 that the batch touches are visited (total = B L ng N).
template <typename T>
__global__ void __launch_bounds__(kBwdThreads)
bwd_group_sum_kernel(const float* __restrict__ dBh, const float* __restrict__ dCh,
                     float* __restrict__ accB, float* __restrict__ accC, T* __restrict__ dB,
                     T* __restrict__ dC, int64_t total, int H, int G, int N, int h0, int nb,
                     int hb, int g0, int ng) {
  const int hpg = H / G;
  for (int64_t e = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kBwdThreads) {
    const int n = (int)(e % N);
    const int64_t bq = e / N;                 // (b*L + t)*ng + (g - g0)
    const int64_t bt = bq / ng;
    const int g = g0 + (int)(bq % ng);
    const int64_t o = (bt * G + g) * N + n;   // element of dB, dC and the running sums
    const int ha = max(h0, g * hpg), hz = min(h0 + nb, (g + 1) * hpg);
    const bool first = ha == g * hpg, last = hz == (g + 1) * hpg;
    float sb = first ? 0.0f : accB[o], sc = first ? 0.0f : accC[o];
    const int64_t base = (bt * hb + (ha - h0)) * N + n;
    for (int k = 0; k < hz - ha; ++k) {
      sb += dBh[base + (int64_t)k * N];
      sc += dCh[base + (int64_t)k * N];
    }
    if (last) {
      dB[o] = to_io<T>(sb);
      dC[o] = to_io<T>(sc);
    } else {
      accB[o] = sb;
      accC[o] = sc;
    }
  }
}

// dA, dD and the bias gradient: sums of the per-(b, h) and per-(b, c, h)
// parts.  One workgroup per head; thread i adds parts i, i + 256, ... and a
// fixed tree adds the threads' sums, so the result is deterministic.
__global__ void __launch_bounds__(kBwdThreads)
bwd_scalars_kernel(const double* __restrict__ dApart, const double* __restrict__ dbpart,
                   const float* __restrict__ dDpart, float* __restrict__ dA, float* __restrict__ dD,
                   float* __restrict__ dbias, int64_t batch, int H, int T_) {
  __shared__ double red[3][kBwdThreads];
  const int h = blockIdx.x, tid = threadIdx.x;
  double sa = 0.0, sb = 0.0, sd = 0.0;
  for (int64_t b = tid; b < batch; b += kBwdThreads) {
    sa += dApart[b * H + h];
    sb += dbpart[b * H + h];
  }
  for (int64_t bc = tid; bc < batch * T_; bc += kBwdThreads) sd += dDpart[bc * H + h];
  red[0][tid] = sa;
  red[1][tid] = sb;
  red[2][tid] = sd;
  __syncthreads();
  for (int w = kBwdThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
      red[2][tid] += red[2][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    dA[h] = (float)red[0][0];
    if (dD) dD[h] = (float)red[2][0];
    if (dbias) dbias[h] = (float)red[1][0];
  }
}

// ---------------------------------------------------------------- host side

// Heads per part: the largest divisor of the heads per group, at most
// kBwdPartHeadsMax, that still leaves ~1024 workgroups per chunk-kernel launch
// over all the parts (B T (H / kh) >= 1024; four workgroups on each of 256
// CUs), else 1.  It depends on the shape alone, so the parts, and the order
// in which dB and dC are summed, are the same whatever the workspace.
int bwd_part_heads(int64_t batch, int64_t T_, int64_t H, int64_t G) {
  const int64_t hpg = H / G, wg = batch * T_;
  int kh = 1;
  for (int k = 2; k <= kBwdPartHeadsMax && k <= hpg; ++k)
    if (hpg % k == 0 && wg * (H / k) >= 1024) kh = k;
  return kh;
}

// Token-block rows of the per-chunk kernels: 32, or 0 when their LDS plan
// for this headdim and dstate does not fit.  The plans are ~34.5 and ~39 KiB
// at headdim 64 / dstate 128 in bf16, so four workgroups share a CU.
int bwd_block_rows(int io_bf16, int Q, int64_t P, int64_t N) {
  const int lim = 160 * 1024;
  if (Q % kBwdTB != 0 || P > 256 || N > 256) return 0;
  const int a = io_bf16 ? bwd_target_bytes<bf16>((int)P, (int)N) : bwd_target_bytes<float>((int)P, (int)N);
  const int s = io_bf16 ? bwd_source_bytes<bf16>((int)P, (int)N) : bwd_source_bytes<float>((int)P, (int)N);
  return a <= lim && s <= lim ? kBwdTB : 0;
}

// Workgroups of the two per-chunk kernels that the device runs at once: the
// smaller of their resident counts per CU (registers, LDS, waves) times the
// CU count of the current device; 0 if the runtime cannot say.
template <typename T, int NKN, int NKP>
static int64_t chunk_slots_of(int64_t P, int64_t N) {
  int dev = 0, cus = 0, a = 0, b = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (ensure_dyn_lds<bwd_target_kernel<T, NKN, NKP>>(bwd_target_bytes<T>((int)P, (int)N)) != hipSuccess ||
      ensure_dyn_lds<bwd_source_kernel<T, NKN, NKP>>(bwd_source_bytes<T>((int)P, (int)N)) !=
          hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, bwd_target_kernel<T, NKN, NKP>, kBwdThreads,
                                                   bwd_target_bytes<T>((int)P, (int)N)) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, bwd_source_kernel<T, NKN, NKP>,
                                                   kBwdThreads,
                                                   bwd_source_bytes<T>((int)P, (int)N)) !=
          hipSuccess)
    return 0;
  return (int64_t)cus * (a < b ? a : b);
}

template <typename T>
static int64_t chunk_slots_t(int64_t P, int64_t N) {
  if (N <= 128) {
    if (P <= 64) return chunk_slots_of<T, 8, 4>(P, N);
    if (P <= 128) return chunk_slots_of<T, 8, 8>(P, N);
    return chunk_slots_of<T, 8, 16>(P, N);
  }
  if (P <= 64) return chunk_slots_of<T, 16, 4>(P, N);
  if (P <= 128) return chunk_slots_of<T, 16, 8>(P, N);
  return chunk_slots_of<T, 16, 16>(P, N);
}

int64_t bwd_chunk_slots(int io_bf16, int64_t P, int64_t N) {
  const int64_t s = io_bf16 ? chunk_slots_t<bf16>(P, N) : chunk_slots_t<float>(P, N);
  (void)hipGetLastError();   // a failed query leaves no error behind for the launches
  return s;
}

template <typename T, int NKN, int NKP>
static hipError_t launch_chunks(const void* x, const void* Bm, const void* Cm, const void* dy,
                                const float* Gw, const float* dtw, const void* Hc, const void* Lam,
                                const float* Dv, void* dx, float* Pb, float* Qb, float* dBh,
                                float* dCh, float* dDpart, int64_t batch, int64_t L, int64_t H,
                                int64_t P, int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw,
                                int p0, int np, int hbp, int kh, hipStream_t stream) {
  const int ta = bwd_target_bytes<T>((int)P, (int)N);
  const int sb = bwd_source_bytes<T>((int)P, (int)N);
  hipError_t e = ensure_dyn_lds<bwd_target_kernel<T, NKN, NKP>>(ta);
  if (e != hipSuccess) return e;
  e = ensure_dyn_lds<bwd_source_kernel<T, NKN, NKP>>(sb);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)T_, (unsigned)np, (unsigned)batch);
  const int hpg = (int)(H / G);
  if (kh < 1 || kh > kBwdPartHeadsMax || hpg % kh != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_target_kernel<T, NKN, NKP>), grid, dim3(kBwdThreads), ta, stream,
                     static_cast<const T*>(x), static_cast<const T*>(Bm),
                     static_cast<const T*>(Cm), static_cast<const T*>(dy), Gw, dtw,
                     static_cast<const float*>(Hc), Pb, dCh, L, (int)H, (int)P, (int)N, (int)G,
                     hpg, Q, (int)T_, ldw, p0, hbp, kh);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_source_kernel<T, NKN, NKP>), grid, dim3(kBwdThreads), sb, stream,
                     static_cast<const T*>(x), static_cast<const T*>(Bm),
                     static_cast<const T*>(Cm), static_cast<const T*>(dy), Gw, dtw,
                     static_cast<const float*>(Lam), Dv, static_cast<T*>(dx), dBh, Qb, dDpart, L,
                     (int)H, (int)P, (int)N, (int)G, hpg, Q, (int)T_, ldw, p0, hbp, kh);
  return hipGetLastError();
}

template <typename T, int NKN>
static hipError_t launch_chunks_p(int64_t P, const void* x, const void* Bm, const void* Cm,
                                  const void* dy, const float* Gw, const float* dtw,
                                  const void* Hc, const void* Lam, const float* Dv, void* dx,
                                  float* Pb, float* Qb, float* dBh, float* dCh, float* dDpart,
                                  int64_t batch, int64_t L, int64_t H, int64_t N, int64_t G, int Q,
                                  int64_t T_, int64_t ldw, int p0, int np, int hbp, int kh,
                                  hipStream_t stream) {
#define SSD_BWD_ARGS x, Bm, Cm, dy, Gw, dtw, Hc, Lam, Dv, dx, Pb, Qb, dBh, dCh, dDpart, batch, L, H, \
                     P, N, G, Q, T_, ldw, p0, np, hbp, kh, stream
  if (P <= 64) return launch_chunks<T, NKN, 4>(SSD_BWD_ARGS);
  if (P <= 128) return launch_chunks<T, NKN, 8>(SSD_BWD_ARGS);
  return launch_chunks<T, NKN, 16>(SSD_BWD_ARGS);
#undef SSD_BWD_ARGS
}

template <typename T>
static hipError_t launch_chunks_t(int TB, const void* x, const void* Bm, const void* Cm,
                                  const void* dy, const float* Gw, const float* dtw,
                                  const void* Hc, const void* Lam, const float* Dv, void* dx,
                                  float* Pb, float* Qb, float* dBh, float* dCh, float* dDpart,
                                  int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                  int64_t G, int Q, int64_t T_, int64_t ldw, int p0, int np, int hbp,
                                  int kh, hipStream_t stream) {
#define SSD_BWD_ARGS P, x, Bm, Cm, dy, Gw, dtw, Hc, Lam, Dv, dx, Pb, Qb, dBh, dCh, dDpart, batch, L, \
                     H, N, G, Q, T_, ldw, p0, np, hbp, kh, stream
  if (TB != kBwdTB) return hipErrorInvalidValue;
  if (N <= 128) return launch_chunks_p<T, 8>(SSD_BWD_ARGS);
  return launch_chunks_p<T, 16>(SSD_BWD_ARGS);
#undef SSD_BWD_ARGS
}

hipError_t launch_bwd_prep(const float* Gw, float* w2, float* Gz, int64_t batch, int64_t H,
                           int64_t L, int64_t ldw, hipStream_t stream) {
  const int64_t total = batch * H * ldw;
  const int64_t blocks = (total + kBwdThreads - 1) / kBwdThreads;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(kBwdThreads), 0, stream, Gw, w2, Gz, total, L, ldw);
  return hipGetLastError();
}

hipError_t launch_bwd_chunks(int io_bf16, int TB, const void* x, const void* Bm, const void* Cm,
                             const void* dy, const float* Gw, const float* dtw, const void* Hc,
                             const void* Lam, const float* Dv, void* dx, float* Pb, float* Qb,
                             float* dBh, float* dCh, float* dDpart, int64_t batch, int64_t L,
                             int64_t H, int64_t P, int64_t N, int64_t G, int Q, int64_t T_,
                             int64_t ldw, int p0, int np, int hbp, int kh, hipStream_t stream) {
  if (io_bf16)
    return launch_chunks_t<bf16>(TB, x, Bm, Cm, dy, Gw, dtw, Hc, Lam, Dv, dx, Pb, Qb, dBh, dCh,
                                 dDpart, batch, L, H, P, N, G, Q, T_, ldw, p0, np, hbp, kh, stream);
  return launch_chunks_t<float>(TB, x, Bm, Cm, dy, Gw, dtw, Hc, Lam, Dv, dx, Pb, Qb, dBh, dCh,
                                dDpart, batch, L, H, P, N, G, Q, T_, ldw, p0, np, hbp, kh, stream);
}

// `H` counts parts here (kh heads each, the units the chunk kernels write),
// h0 .. h0 + nb - 1 are the batch's parts and hb the parts per row.
hipError_t launch_bwd_group_sum(int io_bf16, const float* dBh, const float* dCh, float* accB,
                                float* accC, void* dB, void* dC, int64_t batch, int64_t L,
                                int64_t H, int64_t N, int64_t G, int h0, int nb, int hb,
                                hipStream_t stream) {
  const int hpg = (int)(H / G);
  const int g0 = h0 / hpg, ng = (h0 + nb - 1) / hpg - g0 + 1;   // the groups the batch touches
  const int64_t total = batch * L * ng * N;
  const int64_t blocks = (total + kBwdThreads - 1) / kBwdThreads;
  const dim3 g2((unsigned)(blocks < 8192 ? blocks : 8192));
  if (io_bf16)
    hipLaunchKernelGGL(bwd_group_sum_kernel<bf16>, g2, dim3(kBwdThreads), 0, stream, dBh, dCh,
                       accB, accC, static_cast<bf16*>(dB), static_cast<bf16*>(dC), total, (int)H,
                       (int)G, (int)N, h0, nb, hb, g0, ng);
  else
    hipLaunchKernelGGL(bwd_group_sum_kernel<float>, g2, dim3(kBwdThreads), 0, stream, dBh, dCh,
                       accB, accC, static_cast<float*>(dB), static_cast<float*>(dC), total,
                       (int)H, (int)G, (int)N, h0, nb, hb, g0, ng);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const float* Pb, const float* Qb, const float* dtw,
                             const float* dt_in, const float* A, const float* dfinal,
                             const float* fin, const DtXform* xf, float* ddt, double* dApart,
                             double* dbpart, const float* dDpart, float* dA, float* dD,
                             float* dbias, int64_t batch, int64_t L, int64_t H, int64_t P,
                             int64_t N, int64_t T_, int64_t ldw, hipStream_t stream) {
  const dim3 g1((unsigned)H, (unsigned)batch);
  if (xf)
    hipLaunchKernelGGL(bwd_dt_kernel<true>, g1, dim3(kDtThreads), 0, stream, Pb, Qb, dtw, dt_in,
                       A, dfinal, fin, *xf, ddt, dApart, dbpart, L, (int)H, P * N, ldw);
  else
    hipLaunchKernelGGL(bwd_dt_kernel<false>, g1, dim3(kDtThreads), 0, stream, Pb, Qb, dtw, dt_in,
                       A, dfinal, fin, DtXform{nullptr, 0, 0.0f, 0.0f}, ddt, dApart, dbpart, L,
                       (int)H, P * N, ldw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scalars_kernel, dim3((unsigned)H), dim3(kBwdThreads), 0, stream, dApart,
                     dbpart, dDpart, dA, dD, dbias, batch, (int)H, (int)T_);
  return hipGetLastError();
}

}  // namespace ssd
