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
template <typename T, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_attn(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ cum, float* __restrict__ Aw,
    float* __restrict__ dAw, int L, int dk, int dv, int NC) {
  using M = Mma<T>;
  using PB = PBuilder<T, C>;
  constexpr int LDT = PB::LDT, LDF = PB::LDF, KS = PB::KS;
  constexpr int NRT = C / 16, NTRI = NRT * (NRT + 1) / 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[PB::SLICE_BYTES];
  __shared__ float pd[4][16][17];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  float* bs = reinterpret_cast<float*>(ks + C * LDT);
  float* als = bs + C * LDF;

  const int n = blockIdx.x, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  float* Ab = Aw + ((size_t)bh * NC + n) * C * C;
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
    if ((col >> 4) > (row >> 4)) { dAb[it] = 0.f; Ab[it] = 0.f; }
    else if (col > row) Ab[it] = 0.f;
  }

  PB pb;
  pb.init();
  for (int s0 = 0; s0 < dk; s0 += KS) {
    lds_barrier();
    PB::stage(q, k, cum, qo, r0, rv, dk, s0, qs, ks, bs, nullptr);
    lds_barrier();
    PB::gates(bs, als);
    pb.offdiag(qs, ks, bs);
    lds_barrier();
    pb.diag(qs, ks, als);
  }
  lds_barrier();
  pb.finish(pd, [&](int m, int r, float val) { Ab[m * C + r] = val; });
}

// ------------------------------------------------------------------ B3b: dq, dk, dlog b
// Column layout of the off-diagonal intra operands of k_chunk_dqdk.  For query
// sub-chunk j >= 1 the dq operand holds K ⊙ e^{z_j - B} over key rows
// [0, KQ(j)) (z_j = B at row 16 j; rows >= 16 j are 0), at columns
// [OQ(j), OQ(j) + KQ(j)); for key sub-chunk u < NRT - 1 the dk operand holds
// Q ⊙ e^{B - z'_u} over query rows [MLO(u), C) (z'_u = B at row 16 u + 15;
// rows < 16 (u + 1) are 0), at columns [OK(u), OK(u) + C - MLO(u)).  K spans
// are whole MFMA K steps.
template <int K, int C>
struct OffCols {
  static constexpr int NRT = C / 16;
  static constexpr int KQ(int j) { return ((16 * j + K - 1) / K) * K; }
  static constexpr int MLO(int u) { return ((16 * (u + 1)) / K) * K; }
  static constexpr int OQ(int j) {
    int o = 0;
    for (int i = 1; i < j; ++i) o += KQ(i);
    return o;
  }
  static constexpr int OK(int u) {
    int o = 0;
    for (int i = 0; i < u; ++i) o += C - MLO(i);
    return o;
  }
  static constexpr int WQ = OQ(NRT) > 0 ? OQ(NRT) : K;       // dq operand columns
  static constexpr int WK = OK(NRT - 1) > 0 ? OK(NRT - 1) : K;  // dk operand columns
};

// One workgroup per (batch-head, chunk, d_k tile of TK channels).
template <typename T, int C, int TK>
__global__ __launch_bounds__(kThreads) void k_chunk_dqdk(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ cum, const T* __restrict__ st_n,
    const T* __restrict__ st_lo, const T* __restrict__ dst_n, const T* __restrict__ dst_lo,
    const float* __restrict__ dAw, T* __restrict__ dq, T* __restrict__ dkk,
    float* __restrict__ dla, float* __restrict__ dlt, int L, int dk, int dv, int NC) {
  using M = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int PT = 16 / (int)sizeof(T);
  constexpr int LDA = C + PT;            // T rows of length C
  constexpr int LDK = TK + 4;            // fp32 rows of length TK
  constexpr int NRT = C / 16, NCT = TK / 16;
  constexpr int WC = NCT < 4 ? NCT : 4, WR = 4 / WC;
  constexpr int NCW = NCT / WC, NRW = (NRT + WR - 1) / WR;
  __shared__ float dad[C][17];                              // diagonal blocks, fp32
  __shared__ float qf[C][LDK], kf[C][LDK], bt[C][LDK], al[C][LDK];
  // One region serves, in turn, the dq blocks' dA (diagonal blocks zeroed)
  // and operand, the dk blocks' dA^T ([r][m]) and operand, and the diagonal
  // blocks' terms of dq and dk (dgo).  Operands are [ch][column] (OffCols),
  // each with its low part for bf16.
  using OC = OffCols<M::K, C>;
  constexpr int LDO = (OC::WQ > OC::WK ? OC::WQ : OC::WK) + PT;
  constexpr int DA_BYTES = C * LDA * (int)sizeof(T), DAL_BYTES = BF ? DA_BYTES : 0;
  constexpr int OP_BYTES = TK * LDO * (int)sizeof(T), OPL_BYTES = BF ? OP_BYTES : 0;
  constexpr int OFF_BYTES = DA_BYTES + DAL_BYTES + OP_BYTES + OPL_BYTES;
  constexpr int DGO_BYTES = 2 * C * (TK + 4) * 4;
  __shared__ __attribute__((aligned(16))) unsigned char ubuf[OFF_BYTES > DGO_BYTES ? OFF_BYTES : DGO_BYTES];
  auto da = reinterpret_cast<T(*)[LDA]>(ubuf);
  auto dal = reinterpret_cast<T(*)[LDA]>(ubuf + DA_BYTES);
  auto op = reinterpret_cast<T(*)[LDO]>(ubuf + DA_BYTES + DAL_BYTES);
  auto opl = reinterpret_cast<T(*)[LDO]>(ubuf + DA_BYTES + DAL_BYTES + OP_BYTES);
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
  Raw8<float> tb_;
  if (has_tile) {
    raw_load(tq_, q + tgi);
    raw_load(tk_, k + tgi);
    raw_load(tb_, cum + tgi);
  }
  InterFrags f0;
  inter_load(f0, 0);

  // dA rows of the block as 4-element vectors (hi / lo split, the diagonal
  // blocks zeroed and kept in fp32 apart); with transpose, its columns
  auto stage_da = [&](bool transpose) __attribute__((always_inline)) {
    if (!has_da) return;
    const bool dgb = (m0 >> 4) == (c4 >> 4);  // inside a diagonal 16 x 16 block
    floatx4 hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (dgb && !transpose) dad[m0 + i][(c4 + e) & 15] = xda[i][e];
        const float xo = dgb ? 0.f : xda[i][e];
        hi[i][e] = to_f32(from_f32<T>(xo));
        lo[i][e] = xo - hi[i][e];
      }
    if (!transpose) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store4(&da[m0 + i][c4], hi[i]);
        if constexpr (BF) store4(&dal[m0 + i][c4], lo[i]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        floatx4 th, tl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          th[i] = hi[i][e];
          tl[i] = lo[i][e];
        }
        store4(&da[c4 + e][m0], th);
        if constexpr (BF) store4(&dal[c4 + e][m0], tl);
      }
    }
  };
  stage_da(false);
  // q, k (0 past the end of the sequence) and the cumsum of the tile
  if (has_tile) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = tvalid ? raw_get(tq_, e) : 0.f;
    store8(&qf[trow][tc], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = tvalid ? raw_get(tk_, e) : 0.f;
    store8(&kf[trow][tc], x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = raw_get(tb_, e);
    store8(&bt[trow][tc], x);
  }
  lds_barrier();
  for (int it = tid; it < C * TK; it += kThreads) {
    const int row = it / TK, c = it % TK;
    al[row][c] = (row & 15) ? gexp<T>(bt[row][c] - bt[row - 1][c]) : 1.f;
  }

  // inter-chunk terms: dO S_{n-1}^T and V dS_n^T, reduction over d_v, in
  // groups of KG K steps whose operands are loaded before their products are
  // issued.  The first group's loads were issued at the start of the kernel.
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
  lds_barrier();  // al ready
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int rti = wr + WR * rt;
    if (rti >= NRT) continue;
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct) {
      const int c = (wc + WC * ct) * 16 + (l & 15);
      const float blast = bt[C - 1][c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rti * 16 + (l >> 4) * 4 + r;
        aq[rt][ct][r] *= gexp<T>(bt[row][c]);
        ak[rt][ct][r] *= gexp<T>(blast - bt[row][c]);
      }
    }
  }

  // intra terms of the off-diagonal sub-chunk blocks, with the reference row
  // of each block (both factors <= 1):
  //   dq rows of sub-chunk j:  e^{B_m - z_j} ⊙ [dA_off (K ⊙ e^{z_j - B})]
  //   dk rows of sub-chunk u:  e^{z'_u - B_r} ⊙ [dA_off^T (Q ⊙ e^{B - z'_u})]
  // First the dq blocks, then the dk blocks in the same LDS: each operand is
  // formed in one pass, then every wave handles the blocks of its row tiles.
  if constexpr (NRT > 1) {
    // 8 consecutive columns (rows of the chunk) of one channel per unit; the
    // block boundaries of the column layout are multiples of 8
    static_assert(OC::WQ % 8 == 0 && OC::WK % 8 == 0, "8-column units");
    for (int it = tid; it < TK * (OC::WQ / 8); it += kThreads) {
      const int c = it % TK, col = (it / TK) * 8;
      int j = 1;
      while (j + 1 < NRT && col >= OC::OQ(j + 1)) ++j;
      const int r = col - OC::OQ(j);
      const float z = bt[16 * j][c];
      float x[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = r + e < 16 * j ? kf[r + e][c] * gexp<T>(z - bt[r + e][c]) : 0.f;
        lo[e] = x[e] - to_f32(from_f32<T>(x[e]));
      }
      store8(&op[c][col], x);
      if constexpr (BF) store8(&opl[c][col], lo);
    }
    lds_barrier();
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int j = wr + WR * rt;
      if (j < 1 || j >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
        floatx4 t4 = zero4();
        for (int kk = 0; kk < OC::KQ(j); kk += M::K) {
          const int kc = kk + (l >> 4) * M::KPL;
          auto b = load_frag<T>(&op[c][OC::OQ(j) + kc]);
          auto ah = load_frag<T>(&da[j * 16 + (l & 15)][kc]);
          t4 = M::run(ah, b, t4);
          if constexpr (BF) {
            t4 = M::run(load_frag<T>(&dal[j * 16 + (l & 15)][kc]), b, t4);
            t4 = M::run(ah, load_frag<T>(&opl[c][OC::OQ(j) + kc]), t4);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = j * 16 + (l >> 4) * 4 + r;
          aq[rt][ct][r] += gexp<T>(bt[row][c] - bt[16 * j][c]) * t4[r];
        }
      }
    }
    lds_barrier();  // done with dA and the dq operand
    stage_da(true);
    for (int it = tid; it < TK * (OC::WK / 8); it += kThreads) {
      const int c = it % TK, col = (it / TK) * 8;
      int u = 0;
      while (u + 2 < NRT && col >= OC::OK(u + 1)) ++u;
      const int m = OC::MLO(u) + col - OC::OK(u);
      const float z = bt[16 * u + 15][c];
      float x[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = m + e >= 16 * (u + 1) ? qf[m + e][c] * gexp<T>(bt[m + e][c] - z) : 0.f;
        lo[e] = x[e] - to_f32(from_f32<T>(x[e]));
      }
      store8(&op[c][col], x);
      if constexpr (BF) store8(&opl[c][col], lo);
    }
    lds_barrier();
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int u = wr + WR * rt;
      if (u + 1 >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int c = (wc + WC * ct) * 16 + (l & 15);
        floatx4 t4 = zero4();
        for (int kk = OC::MLO(u); kk < C; kk += M::K) {
          const int kc = kk + (l >> 4) * M::KPL;
          const int oc = OC::OK(u) + kc - OC::MLO(u);
          auto b = load_frag<T>(&op[c][oc]);
          auto ah = load_frag<T>(&da[u * 16 + (l & 15)][kc]);
          t4 = M::run(ah, b, t4);
          if constexpr (BF) {
            t4 = M::run(load_frag<T>(&dal[u * 16 + (l & 15)][kc]), b, t4);
            t4 = M::run(ah, load_frag<T>(&opl[c][oc]), t4);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = u * 16 + (l >> 4) * 4 + r;
          ak[rt][ct][r] += gexp<T>(bt[16 * u + 15][c] - bt[row][c]) * t4[r];
        }
      }
    }
    lds_barrier();  // the diagonal terms below reuse the region
  }
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
      a[i] = al[16 * b + i][c];
      x[i] = which ? qf[16 * b + i][c] : kf[16 * b + i][c];
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
  lds_barrier();  // everyone is done with bt / al / the operands
  float* dlb = &al[0][0];  // reuse: dlog b of the tile, [C][LDK]
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
        dlb[row * LDK + c] = qf[row][c] * aq[rt][ct][r] - kf[row][c] * ak[rt][ct][r];
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
    float part[RPG];
    float s = 0.f;
#pragma unroll
    for (int i = RPG - 1; i >= 0; --i) {
      const int row = g * RPG + i;
      s += row < rv ? dlb[row * LDK + c] : 0.f;
      part[i] = s;
    }
    gtot[g * TK + c] = s;
    lds_barrier();
    float off = 0.f;
    for (int g2 = g + 1; g2 < NGR; ++g2) off += gtot[g2 * TK + c];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      const int row = g * RPG + i;
      if (row < rv) dla[qo + (size_t)(r0 + row) * dk + c0 + c] = part[i] + off;
    }
    if (g == 0) dlt[((size_t)bh * NC + n) * dk + c0 + c] = part[0] + off;
  }
}

// ------------------------------------------------------------------ B3c: dv
// One workgroup per (batch-head, chunk, d_v tile): dV = (K ⊙ Gamma) dS_n + A^T dO.
template <typename T, int C, int TVD>
__global__ __launch_bounds__(kThreads) void k_chunk_dv(
    const T* __restrict__ k, const T* __restrict__ dout, const float* __restrict__ cum,
    const T* __restrict__ dst_t, const float* __restrict__ Aw, T* __restrict__ dvv, int L,
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
      float kv[8], bv[8], bl[8], x[8];
      load8(k + gi, kv);
      load8(cum + gi, bv);
      load8(blast + s0 + c, bl);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = m < rv ? kv[e] * gexp<T>(bl[e] - bv[e]) : 0.f;
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
                     (const T*)k, (const T*)v, (const T*)dout, cum, Aw, dAw, p.L, p.dk, p.dv,
                     p.NC);
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
  hipLaunchKernelGGL((k_chunk_dqdk<T, C, TK>), dim3(p.NC, p.dk / TK, p.BH), dim3(kThreads), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, (const T*)dout, cum, (const T*)st_n,
                     (const T*)st_lo, (const T*)dst_n, (const T*)dst_lo, dAw, (T*)dq, (T*)dk, dla,
                     dlt, p.L, p.dk, p.dv, p.NC);
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
                     (const T*)k, (const T*)dout, cum, (const T*)dst_t, Aw, (T*)dv, p.L, p.dk,
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
