// gla_bwd.hip -- backward kernels of the GLA chunkwise layer for gfx950.
//
// The states S_{n-1} are recomputed (not kept from the forward; zako-mio report
// ch. 2.2, materialise in the forward and recompute in the backward) and the
// state gradient dS_n runs backwards over chunks:
//   dS_{L/C} = dhT,  dS_{n-1} = diag(e^{b_n}) dS_n + (Q ⊙ Lambda)^T dO[n].
// Per chunk, with A the chunk's causal gated score matrix (A[m][r] =
// sum_k q_mk k_rk e^{B_mk - B_rk}, r <= m) and dA = (dO V^T) ⊙ M:
//   dQ = (dO S_{n-1}^T) ⊙ Lambda + sum_r dA[m][r] k_r ⊙ e^{B_m - B_r}
//   dK = (V dS_n^T) ⊙ Gamma     + sum_m dA[m][r] q_m ⊙ e^{B_m - B_r}
//   dV = (K ⊙ Gamma) dS_n       + A^T dO
// (the chain rule through the chunkwise form; the oracle checks these against
// back-propagation through the token recurrence).  The gate gradient uses the
// closed form of the pages (zako-mio report ch. 3.4; papercache.org notes §4.3
// and App. B): dlog b = q ⊙ dq - k ⊙ dk from the fp32 dq, dk, then dlog alpha
// = reverse cumsum of dlog b over the whole sequence, plus rowsum(hT ⊙ dhT)
// when the final state has a gradient.
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"

namespace gla {

// ------------------------------------------------------------------ B3a: A and dA per chunk
// A (the forward's score matrix, fp32) and dA = (dO V^T) ⊙ M, written to the
// workspace as C x C fp32 blocks (zeros above the diagonal).
// fp32 (cum_lo): the decay exponents of A take the cumsum's low part too.
template <typename T, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_attn(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ cum, const float* __restrict__ cum_lo,
    float* __restrict__ Aw, float* __restrict__ dAw, int L, int dk, int dv, int NC) {
  using M = Mma<T>;
  using PB = PBuilder<T, C>;
  constexpr int LDT = PB::LDT, LDF = PB::LDF, KS = PB::KS;
  constexpr int NRT = C / 16, NTRI = NRT * (NRT + 1) / 2;
  constexpr bool LO = sizeof(T) == 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[PB::SLICE_BYTES];
  __shared__ __attribute__((aligned(16))) float bsl[LO ? C * LDF : 1];
  __shared__ float pd[4][16][17];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  float* bs = reinterpret_cast<float*>(ks + C * LDT);
  float* als = bs + C * LDF;

  const int n = blockIdx.x, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  float* Ab = Aw ? Aw + ((size_t)bh * NC + n) * C * C : nullptr;
  float* dAb = dAw + ((size_t)bh * NC + n) * C * C;

  // dA on MFMA over d_v: lower block triangle tiles (ti >= tj)
  for (int t = w; t < NTRI; t += 4) {
    int ti = 0, rem = t;
    while (rem > ti) { rem -= ti + 1; ++ti; }
    const int tj = rem;
    const int ra = ti * 16 + (l & 15), rb = tj * 16 + (l & 15);
    floatx4 acc = zero4();
    // the operands of KG K steps are loaded before their products (rows past
    // the end of the sequence read the last row and are dropped)
    constexpr int KG = 8;
    const int rra = ra < rv ? ra : rv - 1, rrb = rb < rv ? rb : rv - 1;
    for (int kk0 = 0; kk0 < dv; kk0 += KG * M::K) {
      typename M::frag a[KG], b[KG];
#pragma unroll
      for (int gk = 0; gk < KG; ++gk) {
        const int kk = kk0 + gk * M::K;
        if (kk >= dv) break;
        const int c = kk + (l >> 4) * M::KPL;
        a[gk] = load_frag<T>(dout + vo + (size_t)(r0 + rra) * dv + c);
        b[gk] = load_frag<T>(v + vo + (size_t)(r0 + rrb) * dv + c);
        if (ra >= rv) a[gk] = typename M::frag{};
        if (rb >= rv) b[gk] = typename M::frag{};
      }
#pragma unroll
      for (int gk = 0; gk < KG; ++gk) {
        if (kk0 + gk * M::K >= dv) break;
        acc = M::run(a[gk], b[gk], acc);
      }
    }
    const int col = tj * 16 + (l & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = ti * 16 + (l >> 4) * 4 + r;
      dAb[row * C + col] = (col <= row) ? acc[r] : 0.f;
    }
  }
  // zeros above the block diagonal
  for (int it = tid; it < C * C; it += kThreads) {
    const int row = it / C, col = it % C;
    if ((col >> 4) > (row >> 4)) dAb[it] = 0.f;
    if (Aw && col > row) Ab[it] = 0.f;
  }
  if (!Aw) return;  // dA only (the score matrix A is formed elsewhere)

  PB pb;
  pb.init();
  for (int s0 = 0; s0 < dk; s0 += KS) {
    lds_barrier();
    PB::stage(q, k, cum, qo, r0, rv, dk, s0, qs, ks, bs, nullptr);
    if constexpr (LO) PB::stage_lo(cum_lo, qo, r0, rv, dk, s0, bsl);
    lds_barrier();
    PB::template gates<LO>(bs, als, bsl);
    pb.template offdiag<LO>(qs, ks, bs, bsl);
    lds_barrier();
    pb.diag(qs, ks, als);
  }
  lds_barrier();
  pb.finish(pd, [&](int m, int r, float val) { Ab[m * C + r] = val; });
}

// The recurrent backward's first launch, one workgroup per (chunk,
// batch-head), 256 threads (bf16, C = 64):
//  * the chunk-local inclusive cumsum of log alpha into cum (a thread per 4
//    channels and 16 rows, the 16-row totals combined through LDS);
//  * dA = (dO V^T) on the lower block triangle, masked to the causal triangle
//    (zeros above it).  The d_v contraction is split over the four waves (K
//    steps w, w + 4, ...), each wave holding all the triangle's 16 x 16 tiles,
//    so every dO and V element of the chunk is read once; the partial tiles
//    meet in LDS.  Rows past the sequence end read the last row and are
//    zeroed.
template <int C>
__global__ __launch_bounds__(kThreads) void k_chunk_da_cum(
    const bf16* __restrict__ v, const bf16* __restrict__ dout, const float* __restrict__ a,
    float* __restrict__ cum, float* __restrict__ dAw, int L, int dk, int dv, int NC) {
  using M = Mma<bf16>;
  constexpr int NRT = C / 16, NTRI = NRT * (NRT + 1) / 2;
  static_assert(NTRI * 4 * kWave >= kThreads, "cumsum totals fit the reduction buffer");
  __shared__ f32x4 red[4][NTRI][kWave];
  const int n = blockIdx.x, bh = blockIdx.y, w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  {
    f32x4* tot = &red[0][0][0];
    const int quads = dk / 4, per = quads * (C / 16);  // <= 256 for dk <= 256
    const int gq = tid % quads, rg = tid / quads;
    const int rr0 = rg * 16, rr1 = tid < per ? min(rv, rr0 + 16) : rr0;
    const size_t base = ((size_t)bh * L + r0) * dk + 4 * gq;
    f32x4 x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (rr0 + i < rr1) x[i] = *reinterpret_cast<const f32x4*>(a + base + (size_t)(rr0 + i) * dk);
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (rr0 + i < rr1) {
        run += x[i];
        x[i] = run;
      }
    if (tid < per) tot[tid] = run;
    __syncthreads();
    f32x4 off = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < rg; ++g) off += tot[g * quads + gq];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (rr0 + i < rr1) *reinterpret_cast<f32x4*>(cum + base + (size_t)(rr0 + i) * dk) = x[i] + off;
    __syncthreads();  // the totals' buffer is reused below
  }
  floatx4 acc[NTRI];
#pragma unroll
  for (int t = 0; t < NTRI; ++t) acc[t] = zero4();
  const size_t vo = ((size_t)bh * L + r0) * dv;
  for (int ks = w; ks < dv / M::K; ks += 4) {
    const int c = ks * M::K + (l >> 4) * M::KPL;
    M::frag fa[NRT], fb[NRT];
#pragma unroll
    for (int i = 0; i < NRT; ++i) {
      const int row = i * 16 + (l & 15), rr = row < rv ? row : rv - 1;
      fa[i] = load_frag<bf16>(dout + vo + (size_t)rr * dv + c);
      fb[i] = load_frag<bf16>(v + vo + (size_t)rr * dv + c);
      if (row >= rv) {
        fa[i] = M::frag{};
        fb[i] = M::frag{};
      }
    }
    int t = 0;
#pragma unroll
    for (int ti = 0; ti < NRT; ++ti)
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj, ++t) acc[t] = M::run(fa[ti], fb[tj], acc[t]);
  }
#pragma unroll
  for (int t = 0; t < NTRI; ++t) red[w][t][l] = f32x4{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  __syncthreads();
  float* dAb = dAw + ((size_t)bh * NC + n) * C * C;
  for (int t = w; t < NTRI; t += 4) {
    int ti = 0, rem = t;
    while (rem > ti) { rem -= ti + 1; ++ti; }
    const int tj = rem, col = tj * 16 + (l & 15);
    const f32x4 sum = red[0][t][l] + red[1][t][l] + red[2][t][l] + red[3][t][l];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = ti * 16 + (l >> 4) * 4 + r;
      dAb[row * C + col] = (col <= row) ? sum[r] : 0.f;
    }
  }
  for (int it = tid; it < C * C; it += kThreads) {
    const int row = it / C, col = it % C;
    if ((col >> 4) > (row >> 4)) dAb[it] = 0.f;
  }
}

hipError_t launch_chunk_da_cum(const Plan& p, const void* v, const void* dout, const float* a,
                               float* cum, float* dA, hipStream_t s) {
  if (!p.bf16 || p.C != 64 || p.dk % 4 || p.dk > 256 || p.dv % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_chunk_da_cum<64>), dim3(p.NC, p.BH), dim3(kThreads), 0, s,
                     (const bf16*)v, (const bf16*)dout, a, cum, dA, p.L, p.dk, p.dv, p.NC);
  return hipGetLastError();
}

// ------------------------------------------------------------------ B3b: dq, dk, dlog b
// K ranges of the sub-chunk products of k_chunk_dqdk, whole MFMA K steps.
// The dq product of query sub-chunk j runs over key rows [0, KQ(j)) (keys
// [0, 16 j) are used, or [0, 16 j + 16) when the diagonal block is folded in);
// the dk product of key sub-chunk u over query rows [MLO(u), C) (queries
// [16 (u + 1), C), or [16 u, C) folded).
template <int K, int C>
struct OffCols {
  static constexpr int KQ(int j, bool fold) { return ((16 * (j + fold) + K - 1) / K) * K; }
  static constexpr int MLO(int u, bool fold) { return ((16 * (u + !fold)) / K) * K; }
};

// Largest decay (B at a sub-chunk's first row minus B at its last) of a
// channel whose diagonal sub-chunk block k_chunk_dqdk folds into its bf16
// products: e^30 ~ 1e13 leaves fp32 ample range for the gated operands.
constexpr float kFoldSpan = 30.f;

// One workgroup per (batch-head, chunk, d_k tile of TK channels).
// IB: the inter-chunk terms (already scaled by Lambda and Gamma) come in fp32
// from dqi / dki (k_bwd_inter) instead of products with materialised states,
// and dlog alpha is written whole (with the carry over later chunks, from
// cq, ck and crs); without IB it is chunk-local, its chunk totals go to dlt.
// fp32 (cum_lo): every decay exponent takes the cumsum's low part too.
template <typename T, int C, int TK, bool IB>
__global__ __launch_bounds__(kThreads) void k_chunk_dqdk(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ cum, const float* __restrict__ cum_lo,
    const T* __restrict__ st_n,
    const T* __restrict__ st_lo, const T* __restrict__ dst_n, const T* __restrict__ dst_lo,
    const float* __restrict__ dAw, const float* __restrict__ dqi, const float* __restrict__ dki,
    T* __restrict__ dq, T* __restrict__ dkk, float* __restrict__ dla, float* __restrict__ dlt,
    const float* __restrict__ cq, const float* __restrict__ ck, const float* __restrict__ crs,
    int L, int dk, int dv, int NC) {
  using M = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr bool LO = !BF;
  constexpr int PT = 16 / (int)sizeof(T);
  constexpr int LDA = C + PT;            // T rows of length C
  constexpr int LDK = TK + 4;            // fp32 rows of length TK
  constexpr int NRT = C / 16, NCT = TK / 16;
  constexpr int WC = NCT < 4 ? NCT : 4, WR = 4 / WC;
  constexpr int NCW = NCT / WC, NRW = (NRT + WR - 1) / WR;
  __shared__ float dad[C][17];                              // diagonal blocks, fp32
  __shared__ int sharp_w[kThreads / kWave];                 // per wave: a sharp sub-chunk
  // q, k and the cumsum of the tile, channel-major (a channel's tokens are
  // contiguous, so a lane's run of 8 tokens is two 16-byte reads); a row of
  // C + 4 floats puts 16 consecutive channels' 16-byte reads on distinct banks
  constexpr int LDC = C + 4;
  __shared__ __attribute__((aligned(16))) float qf[TK][LDC], kf[TK][LDC], bt[TK][LDC];
  __shared__ __attribute__((aligned(16))) float btl[LO ? TK : 1][LDC];  // the cumsum's low part
  // One region serves, in turn, dA with its diagonal blocks zeroed (rows for
  // the dq blocks, transposed reads for the dk blocks; with its low part for
  // bf16), the diagonal blocks' terms of dq and dk (dgo), and dlog b.
  using OC = OffCols<M::K, C>;
  // bf16: the diagonal blocks may join the matrix-core products (see below)
  constexpr bool FOLD = BF && C % M::K == 0;
  constexpr int DA_BYTES = C * LDA * (int)sizeof(T), DAL_BYTES = BF ? DA_BYTES : 0;
  constexpr int OFF_BYTES = DA_BYTES + DAL_BYTES;
  constexpr int DGO_BYTES = 2 * C * (TK + 4) * 4;
  static_assert(TK * (C + 4) * 4 <= DGO_BYTES, "dlog b fits the region");
  __shared__ __attribute__((aligned(16))) unsigned char ubuf[OFF_BYTES > DGO_BYTES ? OFF_BYTES : DGO_BYTES];
  auto da = reinterpret_cast<T(*)[LDA]>(ubuf);
  auto dal = reinterpret_cast<T(*)[LDA]>(ubuf + DA_BYTES);
  auto dgo = reinterpret_cast<float(*)[C][TK + 4]>(ubuf);

  const int n = blockIdx.x, c0 = blockIdx.y * TK, bh = blockIdx.z;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  const float* dAb = dAw + ((size_t)bh * NC + n) * C * C;
  const int wc = w % WC, wr = w / WC;
  floatx4 aq[NRW][NCW], ak[NRW][NCW];
#pragma unroll
  for (int a = 0; a < NRW; ++a)
#pragma unroll
    for (int b = 0; b < NCW; ++b) aq[a][b] = ak[a][b] = zero4();

  // Operands of the inter-chunk products for KG K steps at kk0: states (and
  // their low halves) of this wave's channels, dO and V of its rows.
  const size_t so = ((size_t)bh * NC + n) * dk * dv;
  const T* sp = st_n + so;
  const T* dsp = dst_n + so;
  const bool lo_s = st_lo != nullptr, lo_d = dst_lo != nullptr;
  constexpr int KG = 4;
  struct InterFrags {
    typename M::frag bs_[KG][NCW], bd_[KG][NCW], bsl[KG][NCW], bdl[KG][NCW];
    typename M::frag ao[KG][NRW], av[KG][NRW];
  };
  auto inter_load = [&](InterFrags& f, int kk0) __attribute__((always_inline)) {
#pragma unroll
    for (int gk = 0; gk < KG; ++gk) {
      const int kk = kk0 + gk * M::K;
      if (kk >= dv) break;
      const int cc = kk + (l >> 4) * M::KPL;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int ch = c0 + (wc + WC * ct) * 16 + (l & 15);
        f.bs_[gk][ct] = load_frag<T>(sp + (size_t)ch * dv + cc);
        f.bd_[gk][ct] = load_frag<T>(dsp + (size_t)ch * dv + cc);
        if (lo_s) f.bsl[gk][ct] = load_frag<T>(st_lo + so + (size_t)ch * dv + cc);
        if (lo_d) f.bdl[gk][ct] = load_frag<T>(dst_lo + so + (size_t)ch * dv + cc);
      }
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) {
        const int rti = wr + WR * rt;
        if (rti >= NRT) continue;
        // rows past the end of the sequence read the last row and drop it
        const int row = rti * 16 + (l & 15), rr = row < rv ? row : rv - 1;
        f.ao[gk][rt] = load_frag<T>(dout + vo + (size_t)(r0 + rr) * dv + cc);
        f.av[gk][rt] = load_frag<T>(v + vo + (size_t)(r0 + rr) * dv + cc);
        if (row >= rv) {
          f.ao[gk][rt] = typename M::frag{};
          f.av[gk][rt] = typename M::frag{};
        }
      }
    }
  };
  auto inter_mma = [&](const InterFrags& f, int gk) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      if (wr + WR * rt >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        aq[rt][ct] = M::run(f.ao[gk][rt], f.bs_[gk][ct], aq[rt][ct]);
        ak[rt][ct] = M::run(f.av[gk][rt], f.bd_[gk][ct], ak[rt][ct]);
        if (lo_s) aq[rt][ct] = M::run(f.ao[gk][rt], f.bsl[gk][ct], aq[rt][ct]);
        if (lo_d) ak[rt][ct] = M::run(f.av[gk][rt], f.bdl[gk][ct], ak[rt][ct]);
      }
    }
  };
  // Loads first: this thread's 4 x 4 block of dA and 8-channel unit of the
  // q, k, cumsum tile (at most one of each per thread), then the first group
  // of inter-chunk operands, which stays in flight while dA, q, k and the
  // gates are staged (loads complete in order, so consuming the earlier ones
  // does not wait for it, and the barriers until its products are LDS-only).
  static_assert((C / 4) * (C / 4) <= kThreads && C * (TK / 8) <= kThreads, "one unit per thread");
  const bool has_da = tid < (C / 4) * (C / 4), has_tile = tid < C * (TK / 8);
  const int m0 = (tid / (C / 4)) * 4, c4 = (tid % (C / 4)) * 4;
  floatx4 xda[4];
  if (has_da)
#pragma unroll
    for (int i = 0; i < 4; ++i) xda[i] = *reinterpret_cast<const f32x4*>(dAb + (m0 + i) * C + c4);
  const int trow = tid / (TK / 8), tc = (tid % (TK / 8)) * 8;
  const bool tvalid = trow < rv;
  const size_t tgi = qo + (size_t)(tvalid ? r0 + trow : r0 + rv - 1) * dk + c0 + tc;
  Raw8<T> tq_, tk_;
  Raw8<float> tb_, tbl_;
  if (has_tile) {
    raw_load(tq_, q + tgi);
    raw_load(tk_, k + tgi);
    raw_load(tb_, cum + tgi);
    if constexpr (LO) raw_load(tbl_, cum_lo + tgi);
  }
  InterFrags f0;
  if constexpr (!IB) {
    inter_load(f0, 0);
  } else {
    // the inter terms of this wave's rows and channels (rows past the end of
    // the sequence are never read; their terms stay 0)
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int rti = wr + WR * rt;
      if (rti >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rti * 16 + (l >> 4) * 4 + r;
          if (row < rv) {
            const size_t gi = qo + (size_t)(r0 + row) * dk + c0 + c;
            aq[rt][ct][r] = dqi[gi];
            ak[rt][ct][r] = dki[gi];
          }
        }
      }
    }
  }
  // IB: dlog alpha's carry into this chunk, rowsum(hT ⊙ dhT) plus the later
  // chunks' totals of q ⊙ dq - k ⊙ dk.  Summed over a chunk, the intra-chunk
  // parts of q ⊙ dq and of k ⊙ dk are the same double sum over the chunk's
  // (query, key) pairs, so a chunk's total is that of the inter terms alone,
  // which k_bwd_inter sums as it walks: an inclusive prefix over chunks of
  // q ⊙ dq_inter (the later chunks' part is the whole sum minus the prefix)
  // and an exclusive suffix of k ⊙ dk_inter, each in two halves of the
  // chunk's rows.  Loaded here, used at the end.
  float cyq[4], cyk[2], cyr = 0.f;
  if constexpr (IB) {
    const int cc = c0 + tid % TK;
    const float* qp = cq + (size_t)bh * NC * 2 * dk + cc;
    const float* kp = ck + ((size_t)bh * NC + n) * 2 * dk + cc;
    cyq[0] = qp[(size_t)(NC - 1) * 2 * dk];
    cyq[1] = qp[((size_t)(NC - 1) * 2 + 1) * dk];
    cyq[2] = qp[(size_t)n * 2 * dk];
    cyq[3] = qp[((size_t)n * 2 + 1) * dk];
    cyk[0] = kp[0];
    cyk[1] = kp[dk];
    cyr = crs[(size_t)bh * dk + cc];
  }

  // dA rows of the block as 4-element vectors (hi / lo split, the diagonal
  // blocks zeroed and kept in fp32 apart)
  auto stage_da = [&]() __attribute__((always_inline)) {
    if (!has_da) return;
    const bool dgb = (m0 >> 4) == (c4 >> 4);  // inside a diagonal 16 x 16 block
    floatx4 hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (dgb) dad[m0 + i][(c4 + e) & 15] = xda[i][e];
        // a folded diagonal block keeps its causal part (key <= query)
        const float xo = dgb && (!FOLD || c4 + e > m0 + i) ? 0.f : xda[i][e];
        hi[i][e] = to_f32(from_f32<T>(xo));
        lo[i][e] = xo - hi[i][e];
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      store4(&da[m0 + i][c4], hi[i]);
      if constexpr (BF) store4(&dal[m0 + i][c4], lo[i]);
    }
  };
  stage_da();
  // q, k (0 past the end of the sequence) and the cumsum of the tile
  if (has_tile) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qf[tc + e][trow] = tvalid ? raw_get(tq_, e) : 0.f;
      kf[tc + e][trow] = tvalid ? raw_get(tk_, e) : 0.f;
      bt[tc + e][trow] = raw_get(tb_, e);
      if constexpr (LO) btl[tc + e][trow] = raw_get(tbl_, e);
    }
  }
  // The diagonal sub-chunk blocks are folded into the products below (their
  // own keys or queries inside the gated operands, the causal mask from dA)
  // when no channel of the tile decays by more than kFoldSpan across any
  // 16-row sub-chunk: the in-block factors e^{z_j - B_s} and e^{B_s - z'_u}
  // then stay below e^kFoldSpan and the outer ones above e^-kFoldSpan.  A
  // wave stages whole sub-chunks (16 rows every 16 TK / 8 lanes), so the
  // lane on a sub-chunk's first row reads the same channels' cumsum on its
  // last row from the lane 15 rows on.
  if constexpr (FOLD) {
    constexpr int LPR = TK / 8;
    static_assert(16 * LPR <= kWave && (C * LPR) % kWave == 0, "whole sub-chunks per wave");
    int sharp = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float b0 = has_tile ? raw_get(tb_, e) : 0.f;
      const float b15 = __shfl_down(b0, 15 * LPR);
      sharp |= has_tile && (trow & 15) == 0 && b0 - b15 > kFoldSpan;
    }
    const bool ws = __ballot(sharp) != 0;
    if (l == 0) sharp_w[w] = ws;
  }
  lds_barrier();
  bool fold = FOLD;
  if constexpr (FOLD) {
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) fold = fold && !sharp_w[i];
  }

  // inter-chunk terms: dO S_{n-1}^T and V dS_n^T, reduction over d_v, in
  // groups of KG K steps whose operands are loaded before their products are
  // issued.  The first group's loads were issued at the start of the kernel.
  if constexpr (!IB) {
#pragma unroll
    for (int gk = 0; gk < KG; ++gk)
      if (gk * M::K < dv) inter_mma(f0, gk);
    for (int kk0 = KG * M::K; kk0 < dv; kk0 += KG * M::K) {
      InterFrags f;
      inter_load(f, kk0);
#pragma unroll
      for (int gk = 0; gk < KG; ++gk)
        if (kk0 + gk * M::K < dv) inter_mma(f, gk);
    }
  }
  if constexpr (!IB) {
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int rti = wr + WR * rt;
      if (rti >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
        const float blast = bt[c][C - 1];
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bt[c][rti * 16 + (l >> 4) * 4]);
        float blastl = 0.f;
        f32x4 bl4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (LO) {
          blastl = btl[c][C - 1];
          bl4 = *reinterpret_cast<const f32x4*>(&btl[c][rti * 16 + (l >> 4) * 4]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          aq[rt][ct][r] *= gexp<T>(b4[r] + bl4[r]);
          ak[rt][ct][r] *= gexp<T>((blast - b4[r]) + (blastl - bl4[r]));
        }
      }
    }
  }

  // intra terms of the off-diagonal sub-chunk blocks (and, folded, of the
  // diagonal ones), with the reference row of each block (off the diagonal
  // both factors are <= 1):
  //   dq rows of sub-chunk j:  e^{B_m - z_j} ⊙ [dA_off (K ⊙ e^{z_j - B})]
  //   dk rows of sub-chunk u:  e^{z'_u - B_r} ⊙ [dA_off^T (Q ⊙ e^{B - z'_u})]
  // Each lane forms its own B operand (its output channel, the K rows its
  // fragment holds) from the staged k or q and the cumsum, with the low part
  // for bf16; the A operand is dA's rows (dq) or, read transposed, its
  // columns (dk).  Nothing is written to LDS here.
  // x = src[tok][c] e^{+-(B_tok - z)} for tok in [t0, t1), else 0
  auto gated = [&](const float (*src)[LDC], int c, int kc, int t0, int t1, float z, float zl,
                   bool up, typename M::frag& fh, typename M::frag& fl)
                   __attribute__((always_inline)) {
    if constexpr (BF) {
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bt[c][kc]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bt[c][kc + 4]);
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(&src[c][kc]);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(&src[c][kc + 4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = kc + e;
        const float bv = e < 4 ? b0[e] : b1[e - 4];
        const float sv = e < 4 ? s0[e] : s1[e - 4];
        const float g = up ? bv - z : z - bv;
        const float x = (tok >= t0 && tok < t1) ? sv * gexp<T>(g) : 0.f;
        fh[e] = static_cast<bf16>(x);
        fl[e] = static_cast<bf16>(x - static_cast<float>(fh[e]));
      }
    } else {
      const float g = up ? (bt[c][kc] - z) + (btl[c][kc] - zl) : (z - bt[c][kc]) + (zl - btl[c][kc]);
      fh = (kc >= t0 && kc < t1) ? src[c][kc] * gexp<T>(g) : 0.f;
      fl = 0.f;
    }
  };
  if constexpr (NRT > 1 || FOLD) {
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int j = wr + WR * rt;
      if (j < !fold || j >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
        const float z = bt[c][16 * j];
        const float zl = LO ? btl[c][16 * j] : 0.f;
        floatx4 t4 = zero4();
        for (int kk = 0; kk < OC::KQ(j, fold); kk += M::K) {
          const int kc = kk + (l >> 4) * M::KPL;
          typename M::frag bh, bl;
          gated(kf, c, kc, 0, 16 * (j + fold), z, zl, false, bh, bl);
          const auto ah = load_frag<T>(&da[j * 16 + (l & 15)][kc]);
          t4 = M::run(ah, bh, t4);
          if constexpr (BF) {
            t4 = M::run(load_frag<T>(&dal[j * 16 + (l & 15)][kc]), bh, t4);
            t4 = M::run(ah, bl, t4);
          }
        }
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bt[c][j * 16 + (l >> 4) * 4]);
        f32x4 bl4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (LO) bl4 = *reinterpret_cast<const f32x4*>(&btl[c][j * 16 + (l >> 4) * 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) aq[rt][ct][r] += gexp<T>((b4[r] - z) + (bl4[r] - zl)) * t4[r];
      }
    }
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int u = wr + WR * rt;
      if (u + !fold >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
        const float z = bt[c][16 * u + 15];
        const float zl = LO ? btl[c][16 * u + 15] : 0.f;
        floatx4 t4 = zero4();
        for (int kk = OC::MLO(u, fold); kk < C; kk += M::K) {
          const int kc = kk + (l >> 4) * M::KPL;
          typename M::frag bh, bl, ah, alo;
          gated(qf, c, kc, 16 * (u + !fold), C, z, zl, true, bh, bl);
          // A[r][m] = dA[m][r] for r in sub-chunk u (the lane's row), m at kc
          if constexpr (BF) {
            ah = col_frag_tr(&da[0][0], LDA, kk, 16 * u, l);
            alo = col_frag_tr(&dal[0][0], LDA, kk, 16 * u, l);
          } else {
            ah = da[kc][16 * u + (l & 15)];
          }
          t4 = M::run(ah, bh, t4);
          if constexpr (BF) {
            t4 = M::run(alo, bh, t4);
            t4 = M::run(ah, bl, t4);
          }
        }
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&bt[c][u * 16 + (l >> 4) * 4]);
        f32x4 bl4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (LO) bl4 = *reinterpret_cast<const f32x4*>(&btl[c][u * 16 + (l >> 4) * 4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) ak[rt][ct][r] += gexp<T>((z - b4[r]) + (zl - bl4[r])) * t4[r];
      }
    }
    lds_barrier();  // the diagonal terms below and dlog b reuse the region
  }
  if (!fold) {
    // diagonal sub-chunk blocks, fp32 VALU with running gate products.  Thread
    // (dq or dk, block b, channel c) keeps the block's 16 gates and its 16 k (or
    // q) values of channel c in registers and forms all 16 rows of the block's
    // term; the terms go through LDS to the waves that own the rows.
    static_assert(2 * NRT * TK <= kThreads || (2 * NRT * TK) % kThreads == 0, "diagonal split");
    for (int it = tid; it < 2 * NRT * TK; it += kThreads) {
      const int which = it / (NRT * TK), b = (it / TK) % NRT, c = it % TK;
      float a[16], x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // the per-row gate alpha of row i in the block (row 0's is not used)
        float d = i ? bt[c][16 * b + i] - bt[c][16 * b + i - 1] : 0.f;
        if constexpr (LO) d += i ? btl[c][16 * b + i] - btl[c][16 * b + i - 1] : 0.f;
        a[i] = i ? gexp<T>(d) : 1.f;
        x[i] = which ? qf[c][16 * b + i] : kf[c][16 * b + i];
      }
      const float* dd = &dad[16 * b][0];  // [16][17]: dA[16 b + m][16 b + s]
      if (which == 0) {
        // dq row m: sum over keys s <= m of dA[m][s] k_s e^{B_m - B_s}
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          float E = 1.f, sum = 0.f;
#pragma unroll
          for (int s2 = m; s2 >= 0; --s2) {
            if (s2 < m) E *= a[s2 + 1];
            sum += dd[m * 17 + s2] * x[s2] * E;
          }
          dgo[0][16 * b + m][c] = sum;
        }
      } else {
        // dk row r: sum over queries s >= r of dA[s][r] q_s e^{B_s - B_r}
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float F = 1.f, sum = 0.f;
#pragma unroll
          for (int s2 = r; s2 < 16; ++s2) {
            if (s2 > r) F *= a[s2];
            sum += dd[s2 * 17 + r] * x[s2] * F;
          }
          dgo[1][16 * b + r][c] = sum;
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int rti = wr + WR * rt;
      if (rti >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = rti * 16 + (l >> 4) * 4 + r;
          aq[rt][ct][r] += dgo[0][row][c];
          ak[rt][ct][r] += dgo[1][row][c];
        }
      }
    }
    lds_barrier();  // everyone is done with bt / the operands
  }
  float* dlb = reinterpret_cast<float*>(ubuf);  // reuse: dlog b of the tile, [TK][LDC]
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int rti = wr + WR * rt;
    if (rti >= NRT) continue;
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct) {
      const int c = (wc + WC * ct) * 16 + (l & 15), row0 = rti * 16 + (l >> 4) * 4;
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(&qf[c][row0]);
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(&kf[c][row0]);
      f32x4 d4;
#pragma unroll
      for (int r = 0; r < 4; ++r) d4[r] = q4[r] * aq[rt][ct][r] - k4[r] * ak[rt][ct][r];
      *reinterpret_cast<f32x4*>(&dlb[c * LDC + row0]) = d4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + r;
        if (row < rv) {
          const size_t gi = qo + (size_t)(r0 + row) * dk + c0 + c;
          dq[gi] = from_f32<T>(aq[rt][ct][r]);
          dkk[gi] = from_f32<T>(ak[rt][ct][r]);
        }
      }
    }
  }
  lds_barrier();
  // chunk-local reverse cumsum of dlog b, and the chunk total: thread
  // (row group g, channel c) sums its RPG rows from the bottom, then adds the
  // totals of the row groups below it
  constexpr int NGR = kThreads / TK, RPG = C / NGR;
  static_assert(NGR * TK == kThreads && RPG * NGR == C, "row groups of the reverse cumsum");
  float* gtot = &bt[0][0];  // reuse: [NGR][TK] group totals
  {
    const int c = tid % TK, g = tid / TK;
    float part[RPG], xv[RPG];
    if constexpr (RPG % 4 == 0) {
#pragma unroll
      for (int i = 0; i < RPG; i += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(&dlb[c * LDC + g * RPG + i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[i + e] = t[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPG; ++i) xv[i] = dlb[c * LDC + g * RPG + i];
    }
    float s = 0.f;
#pragma unroll
    for (int i = RPG - 1; i >= 0; --i) {
      s += g * RPG + i < rv ? xv[i] : 0.f;
      part[i] = s;
    }
    gtot[g * TK + c] = s;
    lds_barrier();
    float off = 0.f;
    for (int g2 = g + 1; g2 < NGR; ++g2) off += gtot[g2 * TK + c];
    if constexpr (IB) off += cyr + ((cyq[0] - cyq[2]) + (cyq[1] - cyq[3])) - (cyk[0] + cyk[1]);
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int row = g * RPG + i;
      if (row < rv) dla[qo + (size_t)(r0 + row) * dk + c0 + c] = part[i] + off;
    }
    // without IB, the chunk total for k_dla_carry
    if (!IB && g == 0) dlt[((size_t)bh * NC + n) * dk + c0 + c] = part[0] + off;
  }
}

// ------------------------------------------------------------------ B3c: dv
// One workgroup per (batch-head, chunk, d_v tile): dV = (K ⊙ Gamma) dS_n + A^T dO.
// fp32 (cum_lo): Gamma's exponents take the cumsum's low part too.
template <typename T, int C, int TVD>
__global__ __launch_bounds__(kThreads) void k_chunk_dv(
    const T* __restrict__ k, const T* __restrict__ dout, const float* __restrict__ cum,
    const float* __restrict__ cum_lo, const T* __restrict__ dst_t, const float* __restrict__ Aw, T* __restrict__ dvv, int L,
    int dk, int dv, int NC) {
  using M = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int PT = 16 / (int)sizeof(T);
  constexpr int LDA = C + PT;
  constexpr int KSL = 64;                 // d_k slice of the staged K ⊙ Gamma
  constexpr int LDKT = KSL + PT;
  constexpr int NRT = C / 16, NCT = TVD / 16;
  constexpr int WC = NCT < 4 ? NCT : 4, WR = 4 / WC;
  constexpr int NCW = NCT / WC, NRW = (NRT + WR - 1) / WR;
  __shared__ __attribute__((aligned(16))) T ath[C][LDA];   // A^T, [r][m]
  __shared__ __attribute__((aligned(16))) T atl[BF ? C : 1][BF ? LDA : 8];
  __shared__ __attribute__((aligned(16))) T dot[TVD][LDA];  // dO^T, [col][m]
  __shared__ __attribute__((aligned(16))) T kt[C][LDKT];    // K ⊙ Gamma slice, [m][ch]

  const int n = blockIdx.x, j0 = blockIdx.y * TVD, bh = blockIdx.z;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  const float* Ab = Aw + ((size_t)bh * NC + n) * C * C;

  // A^T and dO^T, staged in 4 x 4 blocks per thread (4-element writes)
  for (int it = tid; it < (C / 4) * (C / 4); it += kThreads) {
    const int m0 = (it / (C / 4)) * 4, c4 = (it % (C / 4)) * 4;
    floatx4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const f32x4*>(Ab + (m0 + i) * C + c4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      floatx4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = to_f32(from_f32<T>(x[i][e]));
        lo[i] = x[i][e] - hi[i];
      }
      store4(&ath[c4 + e][m0], hi);
      if constexpr (BF) store4(&atl[c4 + e][m0], lo);
    }
  }
  for (int it = tid; it < (C / 4) * (TVD / 4); it += kThreads) {
    const int m0 = (it / (TVD / 4)) * 4, c4 = (it % (TVD / 4)) * 4;
    floatx4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + i < rv ? m0 + i : rv - 1;  // rows past the end: read, then 0
      x[i] = load4(dout + vo + (size_t)(r0 + m) * dv + j0 + c4);
      if (m0 + i >= rv) x[i] = zero4();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      floatx4 t;
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = x[i][e];
      store4(&dot[c4 + e][m0], t);
    }
  }

  const int wc = w % WC, wr = w / WC;
  floatx4 acc[NRW][NCW];
#pragma unroll
  for (int a = 0; a < NRW; ++a)
#pragma unroll
    for (int b = 0; b < NCW; ++b) acc[a][b] = zero4();

  const T* dsp = dst_t + ((size_t)bh * NC + n) * dv * dk;
  const float* blast = cum + qo + (size_t)(r0 + rv - 1) * dk;
  for (int s0 = 0; s0 < dk; s0 += KSL) {
    const int ks = min(KSL, dk - s0);
    lds_barrier();
    for (int it = tid; it < C * (ks / 8); it += kThreads) {
      const int m = it / (ks / 8), c = (it % (ks / 8)) * 8;
      const int mm = m < rv ? m : rv - 1;
      const size_t gi = qo + (size_t)(r0 + mm) * dk + s0 + c;
      float kv[8], bv[8], bl[8], x[8], d[8];
      load8(k + gi, kv);
      load8(cum + gi, bv);
      load8(blast + s0 + c, bl);
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = bl[e] - bv[e];
      if constexpr (!BF) {
        load8(cum_lo + gi, bv);
        load8(cum_lo + (blast - cum) + s0 + c, bl);
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] += bl[e] - bv[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = m < rv ? kv[e] * gexp<T>(d[e]) : 0.f;
      store8(&kt[m][c], x);
    }
    lds_barrier();
    for (int kk = 0; kk < ks; kk += M::K) {
      const int kc = kk + (l >> 4) * M::KPL;
      typename M::frag b[NCW];
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int col = j0 + (wc + WC * ct) * 16 + (l & 15);
        b[ct] = load_frag<T>(dsp + (size_t)col * dk + s0 + kc);
      }
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) {
        const int rti = wr + WR * rt;
        if (rti >= NRT) continue;
        auto a = load_frag<T>(&kt[rti * 16 + (l & 15)][kc]);
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) acc[rt][ct] = M::run(a, b[ct], acc[rt][ct]);
      }
    }
  }
  // A^T dO: rows are keys r, reduction over queries m >= r
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int rti = wr + WR * rt;
    if (rti >= NRT) continue;
    for (int kk = ((rti * 16) / M::K) * M::K; kk < C; kk += M::K) {
      const int kc = kk + (l >> 4) * M::KPL;
      auto ah = load_frag<T>(&ath[rti * 16 + (l & 15)][kc]);
      typename M::frag alo{};
      if constexpr (BF) alo = load_frag<T>(&atl[rti * 16 + (l & 15)][kc]);
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        auto b = load_frag<T>(&dot[(wc + WC * ct) * 16 + (l & 15)][kc]);
        acc[rt][ct] = M::run(ah, b, acc[rt][ct]);
        if constexpr (BF) acc[rt][ct] = M::run(alo, b, acc[rt][ct]);
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int rti = wr + WR * rt;
    if (rti >= NRT) continue;
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct) {
      const int col = j0 + (wc + WC * ct) * 16 + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rti * 16 + (l >> 4) * 4 + r;
        if (row < rv) dvv[vo + (size_t)(r0 + row) * dv + col] = from_f32<T>(acc[rt][ct][r]);
      }
    }
  }
}

// ------------------------------------------------------------------ B4: final-state term and carry
__global__ __launch_bounds__(kWave) void k_rowsum_state(const float* __restrict__ hT,
                                                        const float* __restrict__ dhT,
                                                        float* __restrict__ rs, int dk, int dv) {
  const int i = blockIdx.x, bh = blockIdx.y;
  float s = 0.f;
  if (hT && dhT) {
    const size_t base = ((size_t)bh * dk + i) * dv;
    for (int j = threadIdx.x; j < dv; j += kWave) s += hT[base + j] * dhT[base + j];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (threadIdx.x == 0) rs[(size_t)bh * dk + i] = s;
}

// dlog alpha_t = (chunk-local reverse cumsum of dlog b)_t
//              + sum of the totals of all later chunks + rowsum(hT ⊙ dhT).
// One workgroup per (chunk, batch-head): its first dk / 4 threads form the
// chunk's offsets for 4 channels each (independent vector loads of the later
// chunks' totals), then every thread adds them to 4-channel vectors of the
// chunk's rows.
__global__ __launch_bounds__(kThreads) void k_dla_carry(const float* __restrict__ dlt,
                                                        const float* __restrict__ rs,
                                                        float* __restrict__ dla, int L, int dk,
                                                        int C, int NC) {
  __shared__ f32x4 off4[kThreads];
  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int dk4 = dk / 4;
  for (int c4 = tid; c4 < dk4; c4 += kThreads) {
    f32x4 s = *reinterpret_cast<const f32x4*>(rs + (size_t)bh * dk + 4 * c4);
    const float* base = dlt + (size_t)bh * NC * dk + 4 * c4;
    int m = n + 1;
    for (; m + 7 < NC; m += 8) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const f32x4*>(base + (size_t)(m + u) * dk);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += x[u];
    }
    for (; m < NC; ++m) s += *reinterpret_cast<const f32x4*>(base + (size_t)m * dk);
    off4[c4] = s;
  }
  __syncthreads();
  const int r0 = n * C, rows = min(C, L - r0);
  float* d = dla + ((size_t)bh * L + r0) * dk;
  const int total = rows * dk4;
  for (int e0 = tid; e0 < total; e0 += 4 * kThreads) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kThreads;
      if (e < total) v[u] = *reinterpret_cast<const f32x4*>(d + (size_t)e * 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kThreads;
      if (e < total) *reinterpret_cast<f32x4*>(d + (size_t)e * 4) = v[u] + off4[e % dk4];
    }
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int C>
static hipError_t launch_attn_t(const Plan& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* cum, float* Aw, float* dAw,
                                hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_attn<T, C>), dim3(p.NC, p.BH), dim3(kThreads), 0, s, (const T*)q,
                     (const T*)k, (const T*)v, (const T*)dout, cum, cum_lo_of(p, cum), Aw, dAw,
                     p.L, p.dk, p.dv, p.NC);
  return hipGetLastError();
}

hipError_t launch_chunk_attn(const Plan& p, const void* q, const void* k, const void* v,
                             const void* dout, const float* cum, float* Aw, float* dAw,
                             hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_attn_t<bf16, 64>(p, q, k, v, dout, cum, Aw, dAw, s);
    return launch_attn_t<bf16, 32>(p, q, k, v, dout, cum, Aw, dAw, s);
  }
  if (p.C == 64) return launch_attn_t<float, 64>(p, q, k, v, dout, cum, Aw, dAw, s);
  if (p.C == 32) return launch_attn_t<float, 32>(p, q, k, v, dout, cum, Aw, dAw, s);
  return launch_attn_t<float, 16>(p, q, k, v, dout, cum, Aw, dAw, s);
}

template <typename T, int C, int TK>
static hipError_t launch_dqdk_t(const Plan& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* cum, const void* st_n,
                                const void* st_lo, const void* dst_n, const void* dst_lo,
                                const float* dAw, void* dq, void* dk, float* dla, float* dlt,
                                hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_dqdk<T, C, TK, false>), dim3(p.NC, p.dk / TK, p.BH), dim3(kThreads),
                     0, s, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, cum,
                     cum_lo_of(p, cum), (const T*)st_n, (const T*)st_lo, (const T*)dst_n, (const T*)dst_lo, dAw,
                     nullptr, nullptr, (T*)dq, (T*)dk, dla, dlt, nullptr, nullptr, nullptr, p.L,
                     p.dk, p.dv, p.NC);
  return hipGetLastError();
}

hipError_t launch_chunk_dqdk_inter(const Plan& p, const void* q, const void* k, const float* cum,
                                   const float* dAw, const float* dqi, const float* dki, void* dq,
                                   void* dk, float* dla, const float* qpre, const float* ksuf,
                                   const float* rs, hipStream_t s) {
  if (!p.bf16 || p.C != 64 || p.dk % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_chunk_dqdk<bf16, 64, 32, true>), dim3(p.NC, p.dk / 32, p.BH),
                     dim3(kThreads), 0, s, (const bf16*)q, (const bf16*)k, nullptr, nullptr, cum,
                     nullptr, nullptr, nullptr, nullptr, nullptr, dAw, dqi, dki, (bf16*)dq, (bf16*)dk, dla,
                     nullptr, qpre, ksuf, rs, p.L, p.dk, p.dv, p.NC);
  return hipGetLastError();
}

template <typename T, int C>
static hipError_t launch_dqdk_c(const Plan& p, const void* q, const void* k, const void* v,
                                const void* dout, const float* cum, const void* st_n,
                                const void* st_lo, const void* dst_n, const void* dst_lo,
                                const float* dAw, void* dq, void* dk, float* dla, float* dlt,
                                hipStream_t s) {
  if (p.dk % 32 == 0)
    return launch_dqdk_t<T, C, 32>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
  return launch_dqdk_t<T, C, 16>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
}

hipError_t launch_chunk_dqdk(const Plan& p, const void* q, const void* k, const void* v,
                             const void* dout, const float* cum, const void* st_n,
                             const void* st_lo, const void* dst_n, const void* dst_lo,
                             const float* dAw, void* dq, void* dk, float* dla, float* dlt,
                             hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64)
      return launch_dqdk_c<bf16, 64>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
    return launch_dqdk_c<bf16, 32>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
  }
  if (p.C == 64)
    return launch_dqdk_c<float, 64>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
  if (p.C == 32)
    return launch_dqdk_c<float, 32>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
  return launch_dqdk_c<float, 16>(p, q, k, v, dout, cum, st_n, st_lo, dst_n, dst_lo, dAw, dq, dk, dla, dlt, s);
}

template <typename T, int C, int TVD>
static hipError_t launch_dv_t(const Plan& p, const void* k, const void* dout, const float* cum,
                              const void* dst_t, const float* Aw, void* dv, hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_dv<T, C, TVD>), dim3(p.NC, p.dv / TVD, p.BH), dim3(kThreads), 0, s,
                     (const T*)k, (const T*)dout, cum, cum_lo_of(p, cum), (const T*)dst_t, Aw, (T*)dv, p.L, p.dk,
                     p.dv, p.NC);
  return hipGetLastError();
}

template <typename T, int C>
static hipError_t launch_dv_c(const Plan& p, const void* k, const void* dout, const float* cum,
                              const void* dst_t, const float* Aw, void* dv, hipStream_t s) {
  if (p.dv % 128 == 0) return launch_dv_t<T, C, 128>(p, k, dout, cum, dst_t, Aw, dv, s);
  if (p.dv % 64 == 0) return launch_dv_t<T, C, 64>(p, k, dout, cum, dst_t, Aw, dv, s);
  if (p.dv % 32 == 0) return launch_dv_t<T, C, 32>(p, k, dout, cum, dst_t, Aw, dv, s);
  return launch_dv_t<T, C, 16>(p, k, dout, cum, dst_t, Aw, dv, s);
}

hipError_t launch_chunk_dv(const Plan& p, const void* k, const void* dout, const float* cum,
                           const void* dst_t, const float* Aw, void* dv, hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_dv_c<bf16, 64>(p, k, dout, cum, dst_t, Aw, dv, s);
    return launch_dv_c<bf16, 32>(p, k, dout, cum, dst_t, Aw, dv, s);
  }
  if (p.C == 64) return launch_dv_c<float, 64>(p, k, dout, cum, dst_t, Aw, dv, s);
  if (p.C == 32) return launch_dv_c<float, 32>(p, k, dout, cum, dst_t, Aw, dv, s);
  return launch_dv_c<float, 16>(p, k, dout, cum, dst_t, Aw, dv, s);
}

hipError_t launch_rowsum_state(const Plan& p, const float* hT, const float* dhT, float* rs,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_rowsum_state, dim3(p.dk, p.BH), dim3(kWave), 0, s, hT, dhT, rs, p.dk, p.dv);
  return hipGetLastError();
}

hipError_t launch_dla_carry(const Plan& p, const float* dlt, const float* rs, float* dla,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_dla_carry, dim3(p.NC, p.BH), dim3(kThreads), 0, s, dlt, rs, dla, p.L, p.dk,
                     p.C, p.NC);
  return hipGetLastError();
}

}  // namespace gla
