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

namespace gla {

// ------------------------------------------------------------------ helpers

// Load 8 consecutive elements (32-byte or 16-byte aligned) as fp32.
__device__ inline void load8(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[e + 4] = b[e]; }
}
__device__ inline void load8(const bf16* p, float* o) {
  bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(a[e]);
}
__device__ inline void store8(float* p, const float* x) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[e + 4]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ inline void store8(bf16* p, const float* x) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<bf16x8*>(p) = a;
}
// Store 4 consecutive elements from an accumulator column.
__device__ inline void store4(float* p, floatx4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ inline void store4(bf16* p, floatx4 x) {
  bf16x4 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<bf16x4*>(p) = a;
}

// Off-diagonal sub-chunk pair number pi -> (query sub-chunk j, key sub-chunk u < j).
__device__ inline void pair_of(int pi, int& j, int& u) {
  j = 1;
  while (pi >= j) { pi -= j; ++j; }
  u = pi;
}

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
template <typename T, int TS, int REV>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    const T* __restrict__ X, const T* __restrict__ Y, const float* __restrict__ cum,
    const float* __restrict__ init, const float* __restrict__ seg_in, T* __restrict__ st_t,
    T* __restrict__ st_n, float* __restrict__ end_out, float* __restrict__ seg_out, int L,
    int dk, int dv, int C, int NC, int NSEG, int seg_chunks, int mode) {
  using M = Mma<T>;
  constexpr int NT1 = TS / 16, NTT = NT1 * NT1, NW = (NTT + 3) / 4;
  constexpr int LDC = 64 + 16 / (int)sizeof(T);  // chunk <= 64 tokens, padded rows
  constexpr int CG = TS / 8;
  __shared__ __attribute__((aligned(16))) T xs[TS][LDC];
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
        for (int e = 0; e < 8; ++e) xv[e] *= fast_exp(REV ? bv[e] : gv[e] - bv[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = yv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xs[c0 + e][row] = from_f32<T>(xv[e]);
        ys[c0 + e][row] = from_f32<T>(yv[e]);
      }
    }
    if (threadIdx.x < TS) gam[threadIdx.x] = fast_exp(glast[threadIdx.x]);
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
          for (int r = 0; r < 4; ++r)
            st_n[(((size_t)bh * NC + n) * dk + ib + r) * dv + j] = from_f32<T>(acc[t][r]);
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

template <typename T, int TS, int REV>
static hipError_t launch_cs(const Plan& p, int mode, const void* X, const void* Y,
                            const float* cum, const float* init, const float* seg_in,
                            void* st_t, void* st_n, float* end_out, float* seg_out,
                            hipStream_t s) {
  dim3 grid(p.dv / TS, p.dk / TS, p.BH * p.NSEG);
  hipLaunchKernelGGL((k_chunk_state<T, TS, REV>), grid, dim3(kThreads), 0, s,
                     (const T*)X, (const T*)Y, cum, init, seg_in, (T*)st_t, (T*)st_n, end_out,
                     seg_out, p.L, p.dk, p.dv, p.C, p.NC, p.NSEG, p.seg_chunks, mode);
  return hipGetLastError();
}

template <typename T, int REV>
static hipError_t launch_cs_ts(const Plan& p, int mode, const void* X, const void* Y,
                               const float* cum, const float* init, const float* seg_in,
                               void* st_t, void* st_n, float* end_out, float* seg_out,
                               hipStream_t s) {
  switch (p.TS) {
    case 64: return launch_cs<T, 64, REV>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s);
    case 32: return launch_cs<T, 32, REV>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s);
    default: return launch_cs<T, 16, REV>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s);
  }
}

hipError_t launch_chunk_state(const Plan& p, int rev, int mode, const void* X, const void* Y,
                              const float* cum, const float* init, const float* seg_in,
                              void* st_t, void* st_n, float* end_out, float* seg_out,
                              hipStream_t s) {
  if (p.bf16)
    return rev ? launch_cs_ts<bf16, 1>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s)
               : launch_cs_ts<bf16, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s);
  return rev ? launch_cs_ts<float, 1>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s)
             : launch_cs_ts<float, 0>(p, mode, X, Y, cum, init, seg_in, st_t, st_n, end_out, seg_out, s);
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
      S = fast_exp(G) * S + seg_u[so];
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
//    the Lambda factor carries the decay from the chunk start);
//  * off-diagonal sub-chunk blocks of P on MFMA with the query sub-chunk's
//    first row z as reference: (Q_j ⊙ e^{B_j - z}) (K_u ⊙ e^{z - B_u})^T,
//    both factors <= 1 (notes §4.3 / Figure 3, inter-sub-chunk in half
//    precision; App. B listing);
//  * diagonal sub-chunk blocks in fp32 on the vector ALUs (Figure 3, the
//    intra-sub-chunk part in full precision).  The decay between rows
//    r <= m is formed as the running product alpha_{r+1}...alpha_m of
//    per-row gates alpha = e^{B_r - B_{r-1}}, which equals e^{B_m - B_r}
//    up to rounding, never divides and cannot overflow.
// Then P V on MFMA (the diagonal blocks of P split into a bf16 high part and
// a bf16 low part so that they keep ~16 bits) and the result is stored.
template <typename T, int C, int TVO>
__global__ __launch_bounds__(kThreads) void k_chunk_output(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ cum, const T* __restrict__ st_t, T* __restrict__ o, int L, int dk,
    int dv, int NC) {
  using M = Mma<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KS = BF ? 32 : 16;
  constexpr int PT = 16 / (int)sizeof(T);
  constexpr int LDT = KS + PT, LDF = KS + 4, LDP = C + PT, LDV = C + PT;
  constexpr int NRT = C / 16, NCT = TVO / 16;
  constexpr int WC = NCT < 4 ? NCT : 4, WR = 4 / WC;
  constexpr int NCW = NCT / WC, NRW = (NRT + WR - 1) / WR;
  constexpr int NP = NRT * (NRT - 1) / 2, NPW = (NP + 3) / 4;
  constexpr int WPB = 4 / NRT, NG = 8 * WPB;
  constexpr int CPL = KS / NG > 0 ? KS / NG : 1;
  constexpr int SLICE_BYTES = 3 * C * LDT * (int)sizeof(T) + 2 * C * LDF * 4;
  constexpr int VT_BYTES = TVO * LDV * (int)sizeof(T);
  constexpr int REGION = SLICE_BYTES > VT_BYTES ? SLICE_BYTES : VT_BYTES;

  __shared__ __attribute__((aligned(16))) unsigned char smem[REGION];
  __shared__ __attribute__((aligned(16))) T p_hi[C][LDP];
  __shared__ __attribute__((aligned(16))) T p_lo[BF ? C : 1][BF ? LDP : 8];
  __shared__ float pd[4][16][17];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  T* qts = ks + C * LDT;
  float* bs = reinterpret_cast<float*>(qts + C * LDT);
  float* als = bs + C * LDF;
  T* vt = reinterpret_cast<T*>(smem);

  const int n = blockIdx.x, j0 = blockIdx.y * TVO, bh = blockIdx.z;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;

  for (int it = tid; it < C * LDP; it += kThreads) {
    (&p_hi[0][0])[it] = from_f32<T>(0.f);
    if (BF) (&p_lo[0][0])[it] = from_f32<T>(0.f);
  }

  // roles
  const int db = w / WPB, tb = (w % WPB) * kWave + l, dp = tb & 7, dg = tb >> 3;
  const int wc = w % WC, wr = w / WC;
  float dout[17];
#pragma unroll
  for (int i = 0; i < 17; ++i) dout[i] = 0.f;
  floatx4 pacc[NPW > 0 ? NPW : 1];
#pragma unroll
  for (int t = 0; t < (NPW > 0 ? NPW : 1); ++t) pacc[t] = zero4();
  floatx4 acc[NRW][NCW];
#pragma unroll
  for (int a = 0; a < NRW; ++a)
#pragma unroll
    for (int b = 0; b < NCW; ++b) acc[a][b] = zero4();

  const T* stp = st_t + ((size_t)bh * NC + n) * dv * dk;

  for (int s0 = 0; s0 < dk; s0 += KS) {
    __syncthreads();
    for (int it = tid; it < C * (KS / 8); it += kThreads) {
      const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
      const bool valid = row < rv;
      const int crow = valid ? r0 + row : r0 + rv - 1;
      float qv[8], kv[8], bv[8];
      load8(cum + qo + (size_t)crow * dk + s0 + c8, bv);
      if (valid) {
        load8(q + qo + (size_t)crow * dk + s0 + c8, qv);
        load8(k + qo + (size_t)crow * dk + s0 + c8, kv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = kv[e] = 0.f;
      }
      store8(qs + row * LDT + c8, qv);
      store8(ks + row * LDT + c8, kv);
      store8(bs + row * LDF + c8, bv);
      float qt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qt[e] = qv[e] * fast_exp(bv[e]);
      store8(qts + row * LDT + c8, qt);
    }
    __syncthreads();
    for (int it = tid; it < C * KS; it += kThreads) {
      const int row = it / KS, c = it % KS;
      als[row * LDF + c] = (row & 15) ? fast_exp(bs[row * LDF + c] - bs[(row - 1) * LDF + c]) : 1.f;
    }

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

    // off-diagonal sub-chunk blocks of P
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      const int pi = w + 4 * t;
      if (pi >= NP) continue;
      int jq, ju;
      pair_of(pi, jq, ju);
      const int m = l & 15;
      for (int kk = 0; kk < KS; kk += M::K) {
        const int cq = kk + (l >> 4) * M::KPL;
        float sa[M::KPL], sb[M::KPL];
#pragma unroll
        for (int e = 0; e < M::KPL; ++e) {
          const float z = bs[(jq * 16) * LDF + cq + e];
          sa[e] = fast_exp(bs[(jq * 16 + m) * LDF + cq + e] - z);
          sb[e] = fast_exp(z - bs[(ju * 16 + m) * LDF + cq + e]);
        }
        auto a = scaled_frag<T>(qs + (jq * 16 + m) * LDT + cq, sa);
        auto b = scaled_frag<T>(ks + (ju * 16 + m) * LDT + cq, sb);
        pacc[t] = M::run(a, b, pacc[t]);
      }
    }
    __syncthreads();

    // diagonal sub-chunk blocks of P: fp32, running gate products
    if (dg * CPL < KS) {
      const int cb = dg * CPL;
      const int m1 = dp, m2 = 15 - dp;
      float wv[CPL];
#pragma unroll
      for (int i = 0; i < 17; ++i) {
        const bool first = i <= dp;
        const int m = first ? m1 : m2;
        const int r = first ? (dp - i) : (m2 - (i - dp - 1));
        const bool reset = (i == 0) || (i == dp + 1);
        const int R = db * 16 + m, Rk = db * 16 + r;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float qv = to_f32(qs[R * LDT + cb + c]);
          const float al = als[(Rk + 1 < C ? Rk + 1 : Rk) * LDF + cb + c];
          wv[c] = reset ? qv : wv[c] * al;
          part += wv[c] * to_f32(ks[Rk * LDT + cb + c]);
        }
        dout[i] += part;
      }
    }
  }
  __syncthreads();

  // reduce diagonal partials over the 8 channel groups of a wave
#pragma unroll
  for (int i = 0; i < 17; ++i) {
    dout[i] += __shfl_xor(dout[i], 8);
    dout[i] += __shfl_xor(dout[i], 16);
    dout[i] += __shfl_xor(dout[i], 32);
  }
  if ((l >> 3) == 0) {
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      const bool first = i <= dp;
      const int m = first ? dp : 15 - dp;
      const int r = first ? (dp - i) : (15 - dp - (i - dp - 1));
      pd[w][m][r] = dout[i];
    }
  }
  // off-diagonal blocks to LDS (bf16 / fp32)
#pragma unroll
  for (int t = 0; t < NPW; ++t) {
    const int pi = w + 4 * t;
    if (pi >= NP) continue;
    int jq, ju;
    pair_of(pi, jq, ju);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      p_hi[jq * 16 + (l >> 4) * 4 + r][ju * 16 + (l & 15)] = from_f32<T>(pacc[t][r]);
  }
  __syncthreads();
  for (int it = tid; it < NRT * 256; it += kThreads) {
    const int b = it >> 8, m = (it >> 4) & 15, r = it & 15;
    if (r > m) continue;
    float val = 0.f;
#pragma unroll
    for (int ww = 0; ww < WPB; ++ww) val += pd[b * WPB + ww][m][r];
    const T hi = from_f32<T>(val);
    p_hi[b * 16 + m][b * 16 + r] = hi;
    if (BF) p_lo[b * 16 + m][b * 16 + r] = from_f32<T>(val - to_f32(hi));
  }
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
    if (BF) {
      const int kd = (rti * 16 / M::K) * M::K;
      auto a = load_frag<T>(&p_lo[BF ? rti * 16 + (l & 15) : 0][BF ? kd + (l >> 4) * M::KPL : 0]);
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
