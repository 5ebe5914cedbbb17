// gla_fwd.hip -- forward kernels of the GLA chunkwise layer for gfx950.
//
// Method: "Gated Linear Attention Transformers with Hardware-Efficient
// Training" -- chunkwise form (papercache.org notes §4.2), secondary chunking
// (§4.3, Figure 3), materialised chunk states (§3.3, Figure 1b-c).  Per head,
// with B the chunk-local cumsum of a = log alpha, b_n = B at the chunk's last
// row, Lambda = e^B, Gamma = e^{b_n - B}:
//   S_n   = diag(e^{b_n}) S_{n-1} + (K ⊙ Gamma)^T V              (state)
//   O[n]  = (Q ⊙ Lambda) S_{n-1} + P V                           (output)
// where P is the chunk's causal gated score matrix, built from sub-chunk
// blocks: off-diagonal blocks by MFMA with reference-row factors that are all
// <= 1, diagonal blocks in fp32 on the vector ALUs.
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"

namespace gla {

// ------------------------------------------------------------------ K1: chunk cumsum
// Chunk-local inclusive cumsum of log alpha (the App. B listing's "cumsum of
// log decay within a chunk"; its printed loop indexes a[i] where the
// chunk-local position is meant).  One thread per (chunk, key channel).
__global__ __launch_bounds__(kThreads) void k_cumsum(const float* __restrict__ a,
                                                     float* __restrict__ cum, int L, int dk,
                                                     int C, int NC, int cpb) {
  const int sub = threadIdx.x / dk, col = threadIdx.x % dk;
  const int n = blockIdx.x * cpb + sub;
  if (sub >= cpb || n >= NC) return;
  const size_t base = (size_t)blockIdx.y * L * dk + col;
  const int r0 = n * C, r1 = min(L, r0 + C);
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) {
    acc += a[base + (size_t)r * dk];
    cum[base + (size_t)r * dk] = acc;
  }
}

hipError_t launch_cumsum(const Plan& p, const float* a, float* cum, hipStream_t s) {
  const int cpb = kThreads / p.dk;
  dim3 grid((p.NC + cpb - 1) / cpb, p.BH);
  hipLaunchKernelGGL(k_cumsum, grid, dim3(cpb * p.dk), 0, s, a, cum, p.L, p.dk, p.C, p.NC, cpb);
  return hipGetLastError();
}

// ------------------------------------------------------------------ K2: chunk-state recurrence
// One workgroup owns a TS x TS tile of the d_k x d_v state of one (batch, head)
// and walks the chunks of one sequence segment in order (reverse order for the
// backward's dS recurrence).  The tile lives in MFMA accumulators (fp32); each
// chunk's operands are staged transposed through LDS so that both MFMA
// operands read contiguous token runs.
//
// SPLIT (bf16 only): the scaled operand X ⊙ e^{...} is held as a high and a
// low bf16 part (two MFMAs), and st_n_lo receives the low part of every
// written state, so that the backward's gradients see ~16-bit operands.
template <typename T, int TS, int REV, int SPLIT>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    const T* __restrict__ X, const T* __restrict__ Y, const float* __restrict__ cum,
    const float* __restrict__ init, const float* __restrict__ seg_in, T* __restrict__ st_t,
    T* __restrict__ st_n, T* __restrict__ st_n_lo, float* __restrict__ end_out,
    float* __restrict__ seg_out, int L, int dk, int dv, int C, int NC, int NSEG, int seg_chunks,
    int mode) {
  using M = Mma<T>;
  constexpr int NT1 = TS / 16, NTT = NT1 * NT1, NW = (NTT + 3) / 4;
  constexpr int LDC = 64 + 16 / (int)sizeof(T);  // chunk <= 64 tokens, padded rows
  constexpr int CG = TS / 8;
  __shared__ __attribute__((aligned(16))) T xs[TS][LDC];
  __shared__ __attribute__((aligned(16))) T xl[SPLIT ? TS : 1][SPLIT ? LDC : 8];
  __shared__ __attribute__((aligned(16))) T ys[TS][LDC];
  __shared__ float gam[TS];

  const int j0 = blockIdx.x * TS, i0 = blockIdx.y * TS;
  const int bh = blockIdx.z / NSEG, seg = blockIdx.z % NSEG;
  const int w = wave_id(), l = lane_id();
  const size_t xo = (size_t)bh * L * dk, yo = (size_t)bh * L * dv;

  const float* src = nullptr;
  if (mode == SEG_FILL) {
    if (NSEG > 1) src = seg_in + ((size_t)bh * NSEG + seg) * dk * dv;
    else if (init) src = init + (size_t)bh * dk * dv;
  }
  floatx4 acc[NW];
#pragma unroll
  for (int t = 0; t < NW; ++t) {
    acc[t] = zero4();
    const int tt = w + 4 * t;
    if (tt < NTT && src) {
      const int ti = tt / NT1, tj = tt % NT1;
      const int j = j0 + tj * 16 + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + ti * 16 + (l >> 4) * 4 + r;
        acc[t][r] = src[(size_t)i * dv + j];
      }
    }
  }

  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);
  for (int step = 0; step < ne - nb; ++step) {
    const int n = REV ? (ne - 1 - step) : (nb + step);
    const int r0 = n * C, rv = min(C, L - r0);
    const float* glast = cum + xo + (size_t)(r0 + rv - 1) * dk + i0;
    for (int it = threadIdx.x; it < C * CG; it += kThreads) {
      const int row = it / CG, c0 = (it % CG) * 8;
      float xv[8], yv[8];
      if (row < rv) {
        float bv[8], gv[8];
        load8(X + xo + (size_t)(r0 + row) * dk + i0 + c0, xv);
        load8(Y + yo + (size_t)(r0 + row) * dv + j0 + c0, yv);
        load8(cum + xo + (size_t)(r0 + row) * dk + i0 + c0, bv);
        load8(glast + c0, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] *= gexp<T>(REV ? bv[e] : gv[e] - bv[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = yv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const T hi = from_f32<T>(xv[e]);
        xs[c0 + e][row] = hi;
        if constexpr (SPLIT) xl[c0 + e][row] = from_f32<T>(xv[e] - to_f32(hi));
        ys[c0 + e][row] = from_f32<T>(yv[e]);
      }
    }
    if (threadIdx.x < TS) gam[threadIdx.x] = gexp<T>(glast[threadIdx.x]);
    __syncthreads();

    // The state entering this chunk's update: S_{n-1} (forward) or dS_n (reverse).
    if (mode == SEG_FILL && (st_t || st_n)) {
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int tt = w + 4 * t;
        if (tt >= NTT) continue;
        const int ti = tt / NT1, tj = tt % NT1;
        const int j = j0 + tj * 16 + (l & 15);
        const int ib = i0 + ti * 16 + (l >> 4) * 4;
        if (st_t) store4(st_t + (((size_t)bh * NC + n) * dv + j) * dk + ib, acc[t]);
        if (st_n) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const size_t idx = (((size_t)bh * NC + n) * dk + ib + r) * dv + j;
            const T hi = from_f32<T>(acc[t][r]);
            st_n[idx] = hi;
            if (SPLIT && st_n_lo) st_n_lo[idx] = from_f32<T>(acc[t][r] - to_f32(hi));
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int tt = w + 4 * t;
      if (tt >= NTT) continue;
      const int ti = tt / NT1, tj = tt % NT1;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] *= gam[ti * 16 + (l >> 4) * 4 + r];
      for (int kk = 0; kk < C; kk += M::K) {
        auto a = load_frag<T>(&xs[ti * 16 + (l & 15)][kk + (l >> 4) * M::KPL]);
        auto b = load_frag<T>(&ys[tj * 16 + (l & 15)][kk + (l >> 4) * M::KPL]);
        acc[t] = M::run(a, b, acc[t]);
        if constexpr (SPLIT) {
          auto al = load_frag<T>(&xl[ti * 16 + (l & 15)][kk + (l >> 4) * M::KPL]);
          acc[t] = M::run(al, b, acc[t]);
        }
      }
    }
    __syncthreads();
  }

  float* dst = nullptr;
  if (mode == SEG_LOCAL) dst = seg_out + ((size_t)bh * NSEG + seg) * dk * dv;
  else if (NSEG == 1 && end_out) dst = end_out + (size_t)bh * dk * dv;
  if (dst) {
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int tt = w + 4 * t;
      if (tt >= NTT) continue;
      const int ti = tt / NT1, tj = tt % NT1;
      const int j = j0 + tj * 16 + (l & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + ti * 16 + (l >> 4) * 4 + r;
        dst[(size_t)i * dv + j] = acc[t][r];
      }
    }
  }
}

template <typename T, int TS, int REV, int SPLIT>
static hipError_t launch_cs(const Plan& p, int mode, const void* X, const void* Y,
                            const float* cum, const float* init, const float* seg_in,
                            void* st_t, void* st_n, void* st_n_lo, float* end_out,
                            float* seg_out, hipStream_t s) {
  dim3 grid(p.dv / TS, p.dk / TS, p.BH * p.NSEG);
  hipLaunchKernelGGL((k_chunk_state<T, TS, REV, SPLIT>), grid, dim3(kThreads), 0, s,
                     (const T*)X, (const T*)Y, cum, init, seg_in, (T*)st_t, (T*)st_n,
                     (T*)st_n_lo, end_out, seg_out, p.L, p.dk, p.dv, p.C, p.NC, p.NSEG,
                     p.seg_chunks, mode);
  return hipGetLastError();
}

template <typename T, int REV, int SPLIT>
static hipError_t launch_cs_ts(const Plan& p, int mode, const void* X, const void* Y,
                               const float* cum, const float* init, const float* seg_in,
                               void* st_t, void* st_n, void* st_n_lo, float* end_out,
                               float* seg_out, hipStream_t s) {
  switch (p.TS) {
    case 64: return launch_cs<T, 64, REV, SPLIT>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, st_n_lo, end_out, seg_out, s);
    case 32: return launch_cs<T, 32, REV, SPLIT>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, st_n_lo, end_out, seg_out, s);
    default: return launch_cs<T, 16, REV, SPLIT>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, st_n_lo, end_out, seg_out, s);
  }
}

hipError_t launch_chunk_state(const Plan& p, int rev, int mode, int split, const void* X,
                              const void* Y, const float* cum, const float* init,
                              const float* seg_in, void* st_t, void* st_n, void* st_n_lo,
                              float* end_out, float* seg_out, hipStream_t s) {
  if (p.bf16) {
    if (split)
      return rev ? launch_cs_ts<bf16, 1, 1>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, st_n_lo, end_out, seg_out, s)
                 : launch_cs_ts<bf16, 0, 1>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, st_n_lo, end_out, seg_out, s);
    return rev ? launch_cs_ts<bf16, 1, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, nullptr, end_out, seg_out, s)
               : launch_cs_ts<bf16, 0, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, nullptr, end_out, seg_out, s);
  }
  return rev ? launch_cs_ts<float, 1, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, nullptr, end_out, seg_out, s)
             : launch_cs_ts<float, 0, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, nullptr, end_out, seg_out, s);
}

// ------------------------------------------------------------------ segment scan
// Sequence-level parallelism for long sequences: each segment's local state
// (zero start) is combined with the state entering it,
//   S_in(s+1) = e^{G_s} ⊙ S_in(s) + U_s,  G_s = sum of the segment's chunk totals,
// the associative step of the chunk recurrence (papercache.org notes §2.2,
// chunk-level recurrence, applied to groups of chunks).
__global__ __launch_bounds__(kThreads) void k_segment_scan(
    const float* __restrict__ cum, const float* __restrict__ init, const float* __restrict__ seg_u,
    float* __restrict__ seg_in, float* __restrict__ end_out, int L, int dk, int dv, int C, int NC,
    int NSEG, int seg_chunks, int rev) {
  const int i = blockIdx.x, bh = blockIdx.y;
  const float* crow = cum + (size_t)bh * L * dk + i;
  for (int j = threadIdx.x; j < dv; j += blockDim.x) {
    float S = init ? init[((size_t)bh * dk + i) * dv + j] : 0.f;
    for (int t = 0; t < NSEG; ++t) {
      const int seg = rev ? NSEG - 1 - t : t;
      const size_t so = (((size_t)bh * NSEG + seg) * dk + i) * dv + j;
      seg_in[so] = S;
      float G = 0.f;
      const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);
      for (int n = nb; n < ne; ++n) G += crow[(size_t)(min(L, (n + 1) * C) - 1) * dk];
      S = expf(G) * S + seg_u[so];
    }
    if (end_out) end_out[((size_t)bh * dk + i) * dv + j] = S;
  }
}

hipError_t launch_segment_scan(const Plan& p, int rev, const float* cum, const float* init,
                               const float* seg_u, float* seg_in, float* end_out,
                               hipStream_t s) {
  dim3 grid(p.dk, p.BH);
  const int threads = p.dv < kThreads ? p.dv : kThreads;
  hipLaunchKernelGGL(k_segment_scan, grid, dim3(threads), 0, s, cum, init, seg_u, seg_in,
                     end_out, p.L, p.dk, p.dv, p.C, p.NC, p.NSEG, p.seg_chunks, rev);
  return hipGetLastError();
}

// ------------------------------------------------------------------ state copy (L == 0)
__global__ void k_copy_state(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_state(const Plan& p, const float* src, float* dst, hipStream_t s) {
  const size_t n = (size_t)p.BH * p.dk * p.dv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_state, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, src, dst, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ K3: chunk output
// One workgroup per (batch-head, chunk, d_v tile).  Walks d_k in slices:
//  * inter-chunk term (Q ⊙ Lambda) S_{n-1} on MFMA (papercache.org notes §4.2,
//    Lambda carries the decay from the chunk start);
//  * the chunk's gated score matrix P (gla_pblock.h): off-diagonal sub-chunk
//    blocks on MFMA, diagonal blocks in fp32 on the vector ALUs (notes §4.3 /
//    Figure 3).
// Then P V on MFMA and the store.  Off-diagonal P is rounded to the I/O type
// before P V (half-precision inter-sub-chunk products); the diagonal blocks
// are split into a high and a low part so that they keep ~16 mantissa bits.
template <typename T, int C, int TVO>
__global__ __launch_bounds__(kThreads) void k_chunk_output(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ cum, const T* __restrict__ st_t, T* __restrict__ o, int L, int dk,
    int dv, int NC) {
  using M = Mma<T>;
  using PB = PBuilder<T, C>;
  constexpr bool BF = PB::BF;
  constexpr int KS = PB::KS, LDT = PB::LDT, LDF = PB::LDF, PT = PB::PT;
  constexpr int LDP = C + PT, LDV = C + PT;
  constexpr int NRT = C / 16, NCT = TVO / 16;
  constexpr int WC = NCT < 4 ? NCT : 4, WR = 4 / WC;
  constexpr int NCW = NCT / WC, NRW = (NRT + WR - 1) / WR;
  constexpr int SLICE_BYTES = PB::SLICE_BYTES + C * LDT * (int)sizeof(T);
  constexpr int VT_BYTES = TVO * LDV * (int)sizeof(T);
  constexpr int REGION = SLICE_BYTES > VT_BYTES ? SLICE_BYTES : VT_BYTES;

  __shared__ __attribute__((aligned(16))) unsigned char smem[REGION];
  __shared__ __attribute__((aligned(16))) T p_hi[C][LDP];
  __shared__ __attribute__((aligned(16))) T p_lo[BF ? C : 1][BF ? LDP : 8];
  __shared__ float pd[4][16][17];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  float* bs = reinterpret_cast<float*>(ks + C * LDT);
  float* als = bs + C * LDF;
  T* qts = reinterpret_cast<T*>(als + C * LDF);
  T* vt = reinterpret_cast<T*>(smem);

  const int n = blockIdx.x, j0 = blockIdx.y * TVO, bh = blockIdx.z;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;

  for (int it = tid; it < C * LDP; it += kThreads) {
    (&p_hi[0][0])[it] = from_f32<T>(0.f);
    if constexpr (BF) (&p_lo[0][0])[it] = from_f32<T>(0.f);
  }

  PB pb;
  pb.init();
  const int wc = w % WC, wr = w / WC;
  floatx4 acc[NRW][NCW];
#pragma unroll
  for (int a = 0; a < NRW; ++a)
#pragma unroll
    for (int b = 0; b < NCW; ++b) acc[a][b] = zero4();

  const T* stp = st_t + ((size_t)bh * NC + n) * dv * dk;

  for (int s0 = 0; s0 < dk; s0 += KS) {
    __syncthreads();
    PB::stage(q, k, cum, qo, r0, rv, dk, s0, qs, ks, bs, qts);
    __syncthreads();
    PB::gates(bs, als);
    // inter-chunk term
    for (int kk = 0; kk < KS; kk += M::K) {
      typename M::frag bf[NCW];
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int col = j0 + (wc + WC * ct) * 16 + (l & 15);
        bf[ct] = load_frag<T>(stp + (size_t)col * dk + s0 + kk + (l >> 4) * M::KPL);
      }
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) {
        const int rti = wr + WR * rt;
        if (rti >= NRT) continue;
        auto a = load_frag<T>(qts + (rti * 16 + (l & 15)) * LDT + kk + (l >> 4) * M::KPL);
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) acc[rt][ct] = M::run(a, bf[ct], acc[rt][ct]);
      }
    }
    pb.offdiag(qs, ks, bs);
    __syncthreads();
    pb.diag(qs, ks, als);
  }
  __syncthreads();
  pb.finish(pd, [&](int m, int r, float val) {
    const T hi = from_f32<T>(val);
    p_hi[m][r] = hi;
    if constexpr (BF) {
      if ((m >> 4) == (r >> 4)) p_lo[m][r] = from_f32<T>(val - to_f32(hi));
    }
  });
  // V tile, transposed: vt[col][token]
  for (int it = tid; it < C * (TVO / 8); it += kThreads) {
    const int row = it / (TVO / 8), c8 = (it % (TVO / 8)) * 8;
    float vv[8];
    if (row < rv) {
      load8(v + vo + (size_t)(r0 + row) * dv + j0 + c8, vv);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(c8 + e) * LDV + row] = from_f32<T>(vv[e]);
  }
  __syncthreads();

  // P V
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int rti = wr + WR * rt;
    if (rti >= NRT) continue;
    for (int kb = 0; kb < (rti + 1) * 16; kb += M::K) {
      auto a = load_frag<T>(&p_hi[rti * 16 + (l & 15)][kb + (l >> 4) * M::KPL]);
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        auto b = load_frag<T>(vt + ((wc + WC * ct) * 16 + (l & 15)) * LDV + kb + (l >> 4) * M::KPL);
        acc[rt][ct] = M::run(a, b, acc[rt][ct]);
      }
    }
    if constexpr (BF) {
      const int kd = (rti * 16 / M::K) * M::K;
      auto a = load_frag<T>(&p_lo[rti * 16 + (l & 15)][kd + (l >> 4) * M::KPL]);
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        auto b = load_frag<T>(vt + ((wc + WC * ct) * 16 + (l & 15)) * LDV + kd + (l >> 4) * M::KPL);
        acc[rt][ct] = M::run(a, b, acc[rt][ct]);
      }
    }
  }

  // store
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
        if (row < rv) o[vo + (size_t)(r0 + row) * dv + col] = from_f32<T>(acc[rt][ct][r]);
      }
    }
  }
}

template <typename T, int C, int TVO>
static hipError_t launch_co(const Plan& p, const void* q, const void* k, const void* v,
                            const float* cum, const void* st_t, void* o, hipStream_t s) {
  dim3 grid(p.NC, p.dv / TVO, p.BH);
  hipLaunchKernelGGL((k_chunk_output<T, C, TVO>), grid, dim3(kThreads), 0, s, (const T*)q,
                     (const T*)k, (const T*)v, cum, (const T*)st_t, (T*)o, p.L, p.dk, p.dv, p.NC);
  return hipGetLastError();
}

template <typename T, int C>
static hipError_t launch_co_tv(const Plan& p, const void* q, const void* k, const void* v,
                               const float* cum, const void* st_t, void* o, hipStream_t s) {
  switch (p.TVO) {
    case 256: return launch_co<T, C, (sizeof(T) == 2 ? 256 : 128)>(p, q, k, v, cum, st_t, o, s);
    case 128: return launch_co<T, C, 128>(p, q, k, v, cum, st_t, o, s);
    case 64: return launch_co<T, C, 64>(p, q, k, v, cum, st_t, o, s);
    case 32: return launch_co<T, C, 32>(p, q, k, v, cum, st_t, o, s);
    default: return launch_co<T, C, 16>(p, q, k, v, cum, st_t, o, s);
  }
}

hipError_t launch_chunk_output(const Plan& p, const void* q, const void* k, const void* v,
                               const float* cum, const void* st_t, void* o, hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_co_tv<bf16, 64>(p, q, k, v, cum, st_t, o, s);
    return launch_co_tv<bf16, 32>(p, q, k, v, cum, st_t, o, s);
  }
  if (p.C == 64) return launch_co_tv<float, 64>(p, q, k, v, cum, st_t, o, s);
  if (p.C == 32) return launch_co_tv<float, 32>(p, q, k, v, cum, st_t, o, s);
  return launch_co_tv<float, 16>(p, q, k, v, cum, st_t, o, s);
}

}  // namespace gla
