// chunk_state.hip -- stage 2a: every chunk's own contribution to the state.
//
// For chunk c of head (b, h) (tokens j = 0..Q-1 of the chunk):
//     w_j = exp2(G_last - G_j) * dt_j            (decay from token j to the chunk end)
//     S_c = sum_j w_j x_j (outer) B_j  =  X_c^T diag(w) B_c        (P x N)
// the jump formula: a chunk's whole effect on the state is one matrix product
// over its stacked x and B rows, each row first multiplied by its exponential
// decay so the product stays a plain GEMM (brifing.si "Accelerating Mamba-2
// ...", sections 4 and 5).  S_c depends on nothing outside its chunk, so all
// chunks are computed at once here; the sequential recurrence
// H_{c+1} = exp2(G_last) H_c + S_c is the small elementwise pass in
// state_pass.hip.
//
// gfx950 mapping.  One workgroup per (b, chunk, KH heads of one group, 64-row p
// slice, n slice of up to 128 columns): the heads share the chunk's B rows, so
// B is read once per KH heads.  Waves own one head's 64 p rows and 64 (or
// fewer) n columns.  The product is formed transposed, S^T = B^T X~ on
// v_mfma_f32_16x16x32_bf16 (A operand = B columns, B operand = scaled x
// columns, both token-contiguous), so each lane's accumulator holds 4
// consecutive n of one p row and is stored straight to memory with no LDS
// transpose.  The chunk streams through a ring of 32-token slots filled by
// direct global->LDS loads; each wave multiplies the x rows it loaded by w_j
// in place, one barrier per slot publishes them, and both operands are read
// with transposing LDS reads (ds_read_b64_tr_b16).
#include <type_traits>

#include "ssd_device.hpp"

namespace ssd {

constexpr int kCsTok = 32;    // tokens per ring slot (one MFMA K-step)
#ifndef SSD_CS_KH
#define SSD_CS_KH 4
#endif
constexpr int kCsP = 64;      // p rows per head per workgroup

template <typename T, int KH, int NW>
struct CsCfg {
  static constexpr int V = Vec16<T>::n;                 // elements per 16-byte chunk
  static constexpr int WNT = NW / 16 < 4 ? NW / 16 : 4; // 16-column n tiles per wave
  static constexpr int WPN = NW / 16 / WNT;             // waves per head
  static constexpr int NWV = KH * WPN;                  // waves per workgroup
  static constexpr int THREADS = NWV * kWave;
  static constexpr int BC = NW / V;                     // chunks per B row
  static constexpr int BCH = kCsTok * BC;               // B chunks per slot
  static constexpr int XC = kCsP / V;                   // chunks per x row
  static constexpr int XCH = kCsTok * XC;               // x chunks per head per slot
  static constexpr int BYTES = (BCH + KH * XCH) * 16;
  static constexpr int NBB = (BCH + 63) / 64, NXB = KH * XCH / 64;   // 64-chunk blocks
  static constexpr int BINST = (NBB + NWV - 1) / NWV;   // B loads per wave per slot
  static constexpr int XINST = NXB / NWV;               // x loads per wave per slot
  static constexpr int LPG = BINST + XINST;
  // four slots (three in flight) when a slot is at most 16 KiB, three otherwise:
  // either way two workgroups fit a CU's LDS
  static constexpr int NSLOT = BYTES <= 16 * 1024 ? 4 : 3;
  static constexpr int BSW = BC < 16 ? BC - 1 : 15;
  static_assert(BCH % 64 == 0, "B part of a slot must be whole 64-chunk blocks");
  static_assert(NXB % NWV == 0, "x blocks are scaled in place by the wave that loads them");
  static_assert(XC >= 8, "x swizzle needs 8 chunks per row");
  __host__ __device__ static int gd_bytes(int Q) {      // the w rows, whole 1 KiB blocks
    return (KH * Q * 4 + 1023) / 1024 * 1024;
  }
  // the G and dt rows (or the raw dt) are staged in the ring slot the
  // prologue leaves empty
  static_assert(KH * 2 * 256 * 4 <= BYTES, "G and dt rows of a 256-token chunk fit a ring slot");
  __host__ __device__ static int lds_bytes(int Q) { return NSLOT * BYTES + gd_bytes(Q); }
  __device__ static int bsw(int r) { return r & BSW; }
  __device__ static int xsw(int r) { return ((r >> 1) & 3) << 1; }
  __device__ static int boff(int r, int col) {
    return (r * BC + ((col / V) ^ bsw(r))) * 16 + (col % V) * (int)sizeof(T);
  }
  __device__ static int xoff(int k, int r, int col) {
    return (BCH + k * XCH + r * XC + ((col / V) ^ xsw(r))) * 16 + (col % V) * (int)sizeof(T);
  }
};

// Fragment of a token-major slot tile: column c0 + lane%16, the 8 tokens
// {4 lg .. 4 lg + 3, 16 + 4 lg .. 16 + 4 lg + 3} (lg = lane / 16).
// `row16` is the byte distance of the same column 16 rows further on: both
// tiles' swizzles repeat every 16 rows, so the second read reuses the first
// read's lane address with a constant offset.
template <typename T, typename Off>
__device__ __forceinline__ typename FragOf<T>::type slot_tok_frag(const unsigned char* slot, Off off,
                                                                  int row16, int c0, int lane) {
  const int lg = lane / 16;
  if constexpr (sizeof(T) == 2) {
    // transposing reads: lane r of each 16-lane group addresses the 4 elements
    // at [t0 + r/4][c0 + 4 (r%4)]; lane l then holds rows t0..t0+3 of column c0 + l.
    const int r = lane & 15;
    const int col = c0 + 4 * (r & 3);
    const unsigned char* pa = slot + off(4 * lg + (r >> 2), col);
    const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
    const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + row16));
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    const int c = c0 + (lane & 15);
    floatx8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = *reinterpret_cast<const float*>(slot + off(4 * lg + e, c));
      f[4 + e] = *reinterpret_cast<const float*>(slot + off(16 + 4 * lg + e, c));
    }
    return f;
  }
}

// Multiply 16 bytes of io elements by w (fp32 arithmetic, one rounding).  The
// bf16 form works on an 8-vector so the results are packed two per convert.
template <typename T>
__device__ __forceinline__ vec16 scale16(vec16 v, float w);
template <>
__device__ __forceinline__ vec16 scale16<bf16>(vec16 v, float w) {
  const bf16x8 in = __builtin_bit_cast(bf16x8, v);
  bf16x8 out;
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = static_cast<bf16>(static_cast<float>(in[k]) * w);
  return __builtin_bit_cast(vec16, out);
}
template <>
__device__ __forceinline__ vec16 scale16<float>(vec16 v, float w) {
  floatx4 f = __builtin_bit_cast(floatx4, v);
  f *= w;
  return __builtin_bit_cast(vec16, f);
}

// Running sums inside chunk_state (stage 1 folded into stage 2a).  With `fold`
// set the kernel reads the raw step sizes dt [batch, seqlen, nheads] instead
// of G and dt' rows: its KH heads' dt over the chunk arrive by 4-byte direct
// loads straight into the rows of the G / w staging (one load instruction per
// 64 tokens of one head), ahead of the ring's first slots; waves 0..KH-1 then
// form each head's prepared dt' and running sum G with chunk_cumsum's own
// scan (wave_chunk_scan: bitwise the same values), and the workgroups of p
// slice 0 and n slice 0 store both rows for the later stages, which read them
// as they would read chunk_cumsum's.
struct CsFold {
  const float* dt;    // raw dt [batch, seqlen, nheads]
  const float* A;     // [nheads]
  DtXform xf;         // the step-size preparation, used when xf_on
  int xf_on;
  int on;             // 0: G and dt' rows are inputs (Gw, dtw)
};

// Three-part bf16 split of 8 fp32 values: v = hi + mid + lo to ~24
// significant bits (hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid);
// each difference is exact in fp32).  With an exact bf16 operand, three bf16
// MFMAs (mma3) then give the product with the fp32 values to about fp32
// accuracy, at 3 x 16 cycles against 8 x 32 for the fp32 MFMA.
__device__ __forceinline__ void split3(const floatx8& v, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<bf16>(v[e]);
    const float r1 = v[e] - static_cast<float>(hi[e]);
    mid[e] = static_cast<bf16>(r1);
    lo[e] = static_cast<bf16>(r1 - static_cast<float>(mid[e]));
  }
}
__device__ __forceinline__ floatx4 mma3(floatx4 c, bf16x8 a, const bf16x8& hi, const bf16x8& mid,
                                        const bf16x8& lo) {
  return mma(mma(mma(c, a, hi), a, mid), a, lo);
}

// S3 (bf16 io only): the chunk contribution in fp32 from the exact bf16
// inputs, for the backward pass's states.  Each weighted x value w_j x_j is
// formed in fp32 and split into three bf16 parts hi + mid + lo (~24
// significant bits: hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi -
// mid), every difference exact in fp32), and the product with the exact B
// rows runs as three bf16 MFMAs per K-step; S is stored in fp32.
template <typename T, int KH, int NW, bool S3 = false>
__global__ void __launch_bounds__((CsCfg<T, KH, NW>::THREADS))
chunk_state_kernel(const T* __restrict__ x, const T* __restrict__ Bm, float* __restrict__ Gw,
                   float* __restrict__ dtw, std::conditional_t<S3, float, T>* __restrict__ S,
                   int64_t L, int H, int P, int N, int G, int Q, int T_, int64_t ldw, int nbc,
                   int PB, int NSL, int frag_major, CsFold fold) {
  typedef CsCfg<T, KH, NW> C;
  typedef std::conditional_t<S3, float, T> TO;     // stored type of S
  static_assert(!S3 || sizeof(T) == 2, "the split form reads bf16 inputs");
  typedef typename FragOf<T>::type frag_t;
  constexpr int V = C::V;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;
  float* gd = reinterpret_cast<float*>(smem + C::NSLOT * C::BYTES);   // [KH][w row]

  // XCD-aware placement: block ids congruent mod 8 run on one XCD, so the
  // workgroups of one (b, chunk) -- which share its B rows -- are dealt to one
  // XCD and read B from its L2; neighbouring ids take different chunks.
  const int id = blockIdx.x;
  const int xcd = id % 8, sid = id / 8;
  const int nbx = (nbc + 7) / 8;
  const int bc = (sid % nbx) * 8 + xcd;
  if (bc >= nbc) return;
  const int hp = sid / nbx;                        // (head set, p slice, n slice)
  const int nsl = hp % NSL, pb = hp / NSL % PB, hs = hp / NSL / PB;
  const int h0 = hs * KH;
  const int b = bc / T_, c = bc % T_;
  const int g = h0 / (H / G);
  const int p0 = pb * kCsP, n0 = nsl * NW;
  const int64_t t0 = (int64_t)c * Q;
  const int qv = (int)min((int64_t)Q, L - t0);
  const int ns = (qv + kCsTok - 1) / kCsTok;      // slots holding valid tokens

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
  const T* xc = x + ((int64_t)b * L + t0) * xstride + (int64_t)h0 * P;
  // the scanning waves' A and bias, read before any load into LDS (whose asm
  // clobbers memory) so that they stay scalar loads and no wait for them
  // drains the ring's loads
  float a2f = 0.0f, bias_f = 0.0f;
  if (fold.on && wave < KH) {
    a2f = fold.A[h0 + wave] * kLog2e;
    if (fold.xf_on && fold.xf.bias) bias_f = fold.xf.bias[h0 + wave];
  }
  const T* Bc = Bm + ((int64_t)b * L + t0) * bstride + (int64_t)g * N;

  // Loads of slot k into ring slot k % NSLOT.  Every wave issues exactly LPG
  // instructions (B blocks beyond the count are reloaded with identical data;
  // x blocks divide evenly, each loaded by exactly one wave).  Rows past the
  // chunk's valid tokens and columns past N or P read clamped, valid
  // addresses: those rows get weight 0, those columns are outputs that are
  // never consumed.
  // A slot whose 32 tokens all lie inside the sequence: the per-lane parts
  // of the addresses do not depend on the slot, so they are byte offsets
  // computed once and each slot only moves the wave-uniform row base.
  uint32_t ob[C::BINST], ox[C::XINST];
#pragma unroll
  for (int i = 0; i < C::BINST; ++i) {
    const int q = ((i * C::NWV + wave) % C::NBB) * 64 + lane;
    const int r = q / C::BC, pc = q % C::BC;
    int col = n0 + (pc ^ C::bsw(r)) * V;
    col = col < N ? col : 0;
    ob[i] = (uint32_t)(((int64_t)r * bstride + col) * (int64_t)sizeof(T));
  }
#pragma unroll
  for (int i = 0; i < C::XINST; ++i) {
    const int q = (i * C::NWV + wave) * 64 + lane;
    const int hh = q / C::XCH, rq = q % C::XCH;
    const int r = rq / C::XC, pc = rq % C::XC;
    int p = p0 + (pc ^ C::xsw(r)) * V;
    p = p < P ? p : p0;
    ox[i] = (uint32_t)(((int64_t)hh * P + (int64_t)r * xstride + p) * (int64_t)sizeof(T));
  }
  const bool off32 = (int64_t)kCsTok * (xstride + bstride) * (int64_t)sizeof(T) < ((int64_t)1 << 31);
  auto issue = [&](int k) {
    unsigned char* sl = ring + (k % C::NSLOT) * C::BYTES;
    if (off32 && (k + 1) * kCsTok <= qv) {
      const T* bb = Bc + (int64_t)k * kCsTok * bstride;
      const T* xb = xc + (int64_t)k * kCsTok * xstride;
#pragma unroll
      for (int i = 0; i < C::BINST; ++i)
        dma16_so(bb, ob[i], sl + ((i * C::NWV + wave) % C::NBB) * 1024);
#pragma unroll
      for (int i = 0; i < C::XINST; ++i)
        dma16_so(xb, ox[i], sl + C::BCH * 16 + (i * C::NWV + wave) * 1024);
      return;
    }
#pragma unroll
    for (int i = 0; i < C::BINST; ++i) {
      const int blk = (i * C::NWV + wave) % C::NBB;
      const int q = blk * 64 + lane;
      const int r = q / C::BC, pc = q % C::BC;
      const int tok = min(k * kCsTok + r, qv - 1);
      int col = n0 + (pc ^ C::bsw(r)) * V;
      col = col < N ? col : 0;
      dma16(Bc + (int64_t)tok * bstride + col, (sl + blk * 1024));
    }
#pragma unroll
    for (int i = 0; i < C::XINST; ++i) {
      const int blk = i * C::NWV + wave;
      const int q = blk * 64 + lane;
      const int hh = q / C::XCH, rq = q % C::XCH;
      const int r = rq / C::XC, pc = rq % C::XC;
      const int tok = min(k * kCsTok + r, qv - 1);
      int p = p0 + (pc ^ C::xsw(r)) * V;
      p = p < P ? p : p0;
      dma16(xc + hh * P + (int64_t)tok * xstride + p, (sl + C::BCH * 16 + blk * 1024));
    }
  };

  // ---- prologue: G and dt rows of the KH heads (or raw dt), then the first slots
  // All of it is staged in the ring slot the prologue leaves empty (stg), and
  // only the weights w stay (gd).  Raw dt with fold set: with 4 heads per
  // workgroup, a token's 4 values are 16 contiguous bytes, loaded whole as
  // [token][head] (64 tokens per instruction); with fewer heads, 64 tokens of
  // one head per 4-byte gather into its row [hh][.. | dt row].  Rows past the
  // sequence end read its last token (the scan zeroes them).  Without fold,
  // the G and dt rows arrive as [hh][G row | dt row].
  unsigned char* stg = ring + (C::NSLOT - 1) * C::BYTES;
  const float* dtst = reinterpret_cast<const float*>(stg);
  if (fold.on) {
    if constexpr (KH == 4) {
      for (int m = wave; m * 64 < Q; m += C::NWV) {
        const int j = m * 64 + lane;
        const int64_t tok = min(t0 + j, L - 1);
        if (j < Q) dma16(fold.dt + ((int64_t)b * L + tok) * H + h0, dtst + 4 * (j - lane));
      }
    } else {
      const int nins = KH * ((Q + 63) / 64);
      for (int m = wave; m < nins; m += C::NWV) {
        const int hh = m / ((Q + 63) / 64), j = (m % ((Q + 63) / 64)) * 64 + lane;
        const int64_t tok = min(t0 + j, L - 1);
        if (j < Q) dma4(fold.dt + ((int64_t)b * L + tok) * H + h0 + hh,
                        stg + (hh * 2 * Q + Q + j - lane) * 4);
      }
    }
  } else {
    const int nchunk = KH * Q / 2;                 // 16-byte chunks of G + dt
    const int ngb = (nchunk + 63) / 64;
    const int ginst = (ngb + C::NWV - 1) / C::NWV;
    for (int i = 0; i < ginst; ++i) {              // uniform trip count
      const int blk = (i * C::NWV + wave) % ngb;
      int q = blk * 64 + lane;
      q = q < nchunk ? q : nchunk - 1;
      const int hh = q / (Q / 2), r = q % (Q / 2);
      const float* src = (r < Q / 4 ? Gw : dtw) + (int64_t)(b * H + h0 + hh) * ldw + t0 + 4 * (r % (Q / 4));
      dma16(src, stg + blk * 1024);
    }
  }
  const int npro = min(C::NSLOT - 1, ns);
  for (int k = 0; k < npro; ++k) issue(k);
  wait_groups<C::LPG>(npro);                       // this wave's G/dt loads have landed
  __syncthreads();
  // vector stores this wave issues after the prologue's slots (the G and dt'
  // rows, with fold set): the first waits of the slot loop allow for them
  int late_stores = 0;
  if (fold.on) {
    // waves 0..KH-1 each scan one head and write its weights
    //   w_j = exp2(G_last - G_j) dt'_j
    // (padding tokens have dt' = 0, so w = 0), forming exactly the values the
    // unfolded path forms from stored G and dt rows
    if (wave < KH) {
      const int hh = wave, h = h0 + hh;
      const float* srow = dtst + hh * 2 * Q;
      float* wrow = gd + hh * Q;
      // token j's raw dt of this head, from where the prologue put it
      auto raw_dt = [&](int j) { return KH == 4 ? dtst[4 * j + hh] : srow[Q + j]; };
      auto prep = [&](int j, float v) {
        return t0 + j < L ? (fold.xf_on ? dt_prepare_b(fold.xf, v, bias_f) : v) : 0.0f;
      };
      auto lane_of = [](float v, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
      };
      const float a2 = a2f;
      const bool writer = pb == 0 && nsl == 0;
      // the two rows take at least one store instruction each (the compiler
      // may merge a lane's scalar stores), so counting two never lets a wait
      // of the slot loop pass before its loads have landed
      late_stores = writer ? 2 : 0;
      const int64_t grow = (int64_t)(b * H + h) * ldw + t0;
      if (Q == 256) {
        constexpr int TPL = 4;
        float raw[TPL], g4[TPL];
        const int first = lane * TPL;
#pragma unroll
        for (int e = 0; e < TPL; ++e) raw[e] = prep(first + e, raw_dt(first + e));
        wave_chunk_scan<TPL>(raw, a2, g4, lane);
        const float glast = lane_of(g4[TPL - 1], kWave - 1);
        floatx4 w;
#pragma unroll
        for (int e = 0; e < TPL; ++e) w[e] = fast_exp2(glast - g4[e]) * raw[e];
        *reinterpret_cast<floatx4*>(wrow + first) = w;
        if (writer) {
          *reinterpret_cast<floatx4*>(Gw + grow + first) = floatx4{g4[0], g4[1], g4[2], g4[3]};
          *reinterpret_cast<floatx4*>(dtw + grow + first) = floatx4{raw[0], raw[1], raw[2], raw[3]};
        }
      } else if (Q >= kWave) {
        // Q = 64 or 128: 1 or 2 tokens per lane
        const int tpl = Q / kWave;
        float raw2[2] = {0.0f, 0.0f}, g2[2];
        const int first = lane * tpl;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (e < tpl) raw2[e] = prep(first + e, raw_dt(first + e));
        if (tpl == 2) {
          wave_chunk_scan<2>(raw2, a2, g2, lane);
        } else {
          float r1[1] = {raw2[0]}, o1[1];
          wave_chunk_scan<1>(r1, a2, o1, lane);
          g2[0] = o1[0];
        }
        const float glast = lane_of(tpl == 2 ? g2[1] : g2[0], kWave - 1);
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (e < tpl) wrow[first + e] = fast_exp2(glast - g2[e]) * raw2[e];
        if (writer) {
#pragma unroll
          for (int e = 0; e < 2; ++e)
            if (e < tpl) {
              Gw[grow + first + e] = g2[e];
              dtw[grow + first + e] = raw2[e];
            }
        }
      } else {
        // Q = 32: lanes 0..31 hold one token each
        float r1[1] = {0.0f}, g1[1];
        if (lane < Q) r1[0] = prep(lane, raw_dt(lane));
        wave_chunk_scan<1>(r1, a2, g1, lane);
        const float glast = lane_of(g1[0], Q - 1);
        if (lane < Q) wrow[lane] = fast_exp2(glast - g1[0]) * r1[0];
        if (writer) {
          if (lane < Q) {
            Gw[grow + lane] = g1[0];
            dtw[grow + lane] = r1[0];
          }
        }
      }
    }
  } else {
    // w_j = exp2(G_last - G_j) dt_j from the staged rows; padding tokens
    // have dt = 0 and G flat past the sequence end, so they get w = 0
    for (int idx = tid; idx < KH * Q; idx += C::THREADS) {
      const int hh = idx / Q, j = idx % Q;
      const float* srow = dtst + hh * 2 * Q;
      gd[hh * Q + j] = fast_exp2(srow[Q - 1] - srow[j]) * srow[Q + j];
    }
  }
  __syncthreads();

  // ---- stream the slots ---------------------------------------------------------
  const int hh = wave / C::WPN;                   // this wave's head and n columns
  const int nw0 = (wave % C::WPN) * C::WNT * 16;
  floatx4 acc[C::WNT][4];
#pragma unroll
  for (int nt = 0; nt < C::WNT; ++nt)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[nt][pt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k = 0; k < ns; ++k) {
    // this wave's loads of slot k
    if (k < npro && late_stores)
      wait_groups_plus<C::LPG, 2>(min(C::NSLOT - 2, ns - 1 - k));
    else
      wait_groups<C::LPG>(min(C::NSLOT - 2, ns - 1 - k));
    unsigned char* sl = ring + (k % C::NSLOT) * C::BYTES;
    if constexpr (!S3) {
      // scale the x rows this wave loaded by their token's weight, in place
#pragma unroll
      for (int i = 0; i < C::XINST; ++i) {
        const int blk = i * C::NWV + wave;
        const int q = blk * 64 + lane;
        const int hq = q / C::XCH, r = q % C::XCH / C::XC;
        vec16* pch = reinterpret_cast<vec16*>(sl + C::BCH * 16 + q * 16);
        *pch = scale16<T>(*pch, gd[hq * Q + k * kCsTok + r]);
      }
    }
    __syncthreads();                               // slot k complete; slot k-1 free
    if (k + C::NSLOT - 1 < ns) issue(k + C::NSLOT - 1);
    if constexpr (S3) {
      // the lane's 8 tokens {4 lg .. +3, 16 + 4 lg .. +3} of the slot and their weights
      const int lg = lane / 16;
      const floatx4 w0 = *reinterpret_cast<const floatx4*>(gd + hh * Q + k * kCsTok + 4 * lg);
      const floatx4 w1 = *reinterpret_cast<const floatx4*>(gd + hh * Q + k * kCsTok + 16 + 4 * lg);
      frag_t fa[C::WNT];
#pragma unroll
      for (int nt = 0; nt < C::WNT; ++nt)
        fa[nt] = slot_tok_frag<T>(sl, [&](int r, int col) { return C::boff(r, col); },
                                  16 * C::BC * 16, nw0 + nt * 16, lane);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const frag_t xr = slot_tok_frag<T>(sl, [&](int r, int col) { return C::xoff(hh, r, col); },
                                           16 * C::XC * 16, pt * 16, lane);
        floatx8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = to_f32(xr[e]) * (e < 4 ? w0[e] : w1[e - 4]);
        bf16x8 hi, mid, lo;
        split3(v, hi, mid, lo);
#pragma unroll
        for (int nt = 0; nt < C::WNT; ++nt) acc[nt][pt] = mma3(acc[nt][pt], fa[nt], hi, mid, lo);
      }
    } else {
      frag_t fb[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
        fb[pt] = slot_tok_frag<T>(sl, [&](int r, int col) { return C::xoff(hh, r, col); },
                                  16 * C::XC * 16, pt * 16, lane);
#pragma unroll
      for (int nt = 0; nt < C::WNT; ++nt) {
        const frag_t fa = slot_tok_frag<T>(sl, [&](int r, int col) { return C::boff(r, col); },
                                           16 * C::BC * 16, nw0 + nt * 16, lane);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[nt][pt] = mma(acc[nt][pt], fa, fb[pt]);
      }
    }
  }

  // ---- store S_c: lane holds p = 16 pt + lane%16 and n = n_base + 4 lg .. +3 --
  const int h = h0 + hh, lr = lane % 16, lg = lane / 16;
  if (frag_major) {
    const HcFrag hf = hc_frag(P, N);
    TO* base = S + ((int64_t)(b * H + h) * T_ + c) * hf.state_elems();
#pragma unroll
    for (int nt = 0; nt < C::WNT; ++nt) {
      const int n = n0 + nw0 + nt * 16 + 4 * lg;              // multiple of 4
      const int ks = n / 32, q = (n % 32) / 8, e0 = n % 8;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        TO* dst = base + hf.offset(pb, pt, ks, lr + 16 * q) + e0;
        if constexpr (sizeof(TO) == 2) {
          const bf16x4 v{to_io<T>(acc[nt][pt][0]), to_io<T>(acc[nt][pt][1]),
                         to_io<T>(acc[nt][pt][2]), to_io<T>(acc[nt][pt][3])};
          *reinterpret_cast<bf16x4*>(dst) = v;
        } else {
          *reinterpret_cast<floatx4*>(dst) = acc[nt][pt];
        }
      }
    }
  } else {
    TO* base = S + ((int64_t)(b * H + h) * T_ + c) * (int64_t)P * N;
#pragma unroll
    for (int nt = 0; nt < C::WNT; ++nt) {
      const int n = n0 + nw0 + nt * 16 + 4 * lg;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int p = p0 + pt * 16 + lr;
        if (p < P && n < N) {
          TO* dst = base + (int64_t)p * N + n;
          if constexpr (sizeof(TO) == 2) {
            const bf16x4 v{to_io<T>(acc[nt][pt][0]), to_io<T>(acc[nt][pt][1]),
                           to_io<T>(acc[nt][pt][2]), to_io<T>(acc[nt][pt][3])};
            *reinterpret_cast<bf16x4*>(dst) = v;
          } else {
            *reinterpret_cast<floatx4*>(dst) = acc[nt][pt];
          }
        }
      }
    }
  }
}

// Default heads per workgroup: 4 (or 2, or 1) heads of one group share the B
// rows (2 heads, 2560 workgroups in five full rounds with a 4-slot ring,
// measured 71.8 us against 68.4 us at the 2.7B shape: the smaller tail does
// not pay for reading each chunk's B rows twice as often).  Any count that
// divides the heads of a group is valid.
int chunk_state_default_kh(int64_t H, int64_t G) {
  const int64_t hg = H / G;
  return SSD_CS_KH >= 4 && hg % 4 == 0 ? 4 : hg % 2 == 0 ? 2 : 1;
}

template <typename T, int KH, int NW, bool S3 = false>
static hipError_t launch_cs(const void* x, const void* Bm, float* Gw, float* dtw, void* S,
                            int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                            int Q, int64_t T_, int64_t ldw, int frag_major, const CsFold& fold,
                            hipStream_t stream) {
  typedef CsCfg<T, KH, NW> C;
  const int PB = (int)((P + kCsP - 1) / kCsP);
  const int NSL = (int)(32 * nk_class(N) / NW);
  const int64_t nbc = batch * T_;
  const int64_t nblocks = ((nbc + 7) / 8) * 8 * (H / KH) * PB * NSL;
  const int lds = C::lds_bytes(Q);
  typedef std::conditional_t<S3, float, T> TO;
  auto kern = chunk_state_kernel<T, KH, NW, S3>;
  // the attribute is the most any launch of this kernel asks for (chunks of
  // at most 256 tokens), not the CU's whole LDS
  const hipError_t e = ensure_dyn_lds<chunk_state_kernel<T, KH, NW, S3>>(C::lds_bytes(256));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(C::THREADS), lds, stream,
                     static_cast<const T*>(x), static_cast<const T*>(Bm), Gw, dtw,
                     static_cast<TO*>(S), L, (int)H, (int)P, (int)N, (int)G, Q, (int)T_, ldw,
                     (int)nbc, PB, NSL, frag_major, fold);
  return hipGetLastError();
}

template <typename T, int KH, bool S3 = false>
static hipError_t launch_cs_nw(const void* x, const void* Bm, float* Gw, float* dtw, void* S,
                               int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                               int64_t G, int Q, int64_t T_, int64_t ldw, int frag_major,
                               const CsFold& fold, hipStream_t stream) {
#define SSD_CS_ARGS x, Bm, Gw, dtw, S, batch, L, H, P, N, G, Q, T_, ldw, frag_major, fold, stream
  switch (state_nw(N)) {
    case 32: return launch_cs<T, KH, 32, S3>(SSD_CS_ARGS);
    case 64: return launch_cs<T, KH, 64, S3>(SSD_CS_ARGS);
    default: return launch_cs<T, KH, 128, S3>(SSD_CS_ARGS);
  }
#undef SSD_CS_ARGS
}

template <typename T, bool S3 = false>
static hipError_t launch_cs_t(int kh, const void* x, const void* Bm, float* Gw, float* dtw,
                              void* S, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int Q, int64_t T_, int64_t ldw, int frag_major,
                              const CsFold& fold, hipStream_t stream) {
#define SSD_CS_ARGS x, Bm, Gw, dtw, S, batch, L, H, P, N, G, Q, T_, ldw, frag_major, fold, stream
  switch (kh) {
    case 4: return launch_cs_nw<T, 4, S3>(SSD_CS_ARGS);
    case 2: return launch_cs_nw<T, 2, S3>(SSD_CS_ARGS);
    default: return launch_cs_nw<T, 1, S3>(SSD_CS_ARGS);
  }
#undef SSD_CS_ARGS
}

// kh: heads per workgroup (1, 2 or 4, dividing the heads of a group; checked
// by the caller).  dt_raw == NULL: Gw and dtw hold the running sums and
// prepared step sizes (chunk_cumsum's rows, or the backward pass's weights);
// otherwise the kernel forms them from dt_raw, A and the optional
// preparation xf and writes them to Gw and dtw (rows of ldw floats, every
// chunk's Q positions).
hipError_t launch_chunk_state(int io_bf16, const void* x, const void* Bm, float* Gw, float* dtw,
                              void* S, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                              int64_t G, int Q, int64_t T_, int64_t ldw, int frag_major, int kh,
                              const float* dt_raw, const float* A, const DtXform* xf,
                              hipStream_t stream) {
  CsFold fold{dt_raw, A, xf ? *xf : DtXform{nullptr, 0, 0.0f, 0.0f}, xf ? 1 : 0,
              dt_raw ? 1 : 0};
  if (io_bf16)
    return launch_cs_t<bf16>(kh, x, Bm, Gw, dtw, S, batch, L, H, P, N, G, Q, T_, ldw, frag_major,
                             fold, stream);
  return launch_cs_t<float>(kh, x, Bm, Gw, dtw, S, batch, L, H, P, N, G, Q, T_, ldw, frag_major,
                            fold, stream);
}

// The backward pass's states from bf16 inputs: S in fp32 from the exact x and
// B values with the three-part split of the weighted x (S3 above); plain
// [B, H, T, P, N] layout, G and w rows given.
hipError_t launch_chunk_state_split(const void* x, const void* Bm, float* Gw, float* dtw,
                                    float* S, int64_t batch, int64_t L, int64_t H, int64_t P,
                                    int64_t N, int64_t G, int Q, int64_t T_, int64_t ldw, int kh,
                                    hipStream_t stream) {
  CsFold fold{nullptr, nullptr, DtXform{nullptr, 0, 0.0f, 0.0f}, 0, 0};
  return launch_cs_t<bf16, true>(kh, x, Bm, Gw, dtw, S, batch, L, H, P, N, G, Q, T_, ldw, 0, fold,
                                 stream);
}

}  // namespace ssd
