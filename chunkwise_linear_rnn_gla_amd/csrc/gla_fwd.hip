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
// chunk-local position is meant).  A thread owns 4 adjacent key channels of
// 16 consecutive rows (16 independent 16-byte loads in flight); the 16-row
// group totals are combined through LDS.  Within a row group the sum runs in
// row order, and group offsets are added in group order.
//
// With cum_lo (the fp32 backward), every sum is compensated (two-sum): cum
// holds the rounded cumsum and cum_lo the rounding error it leaves, so that a
// decay exponent B_m - B_r = (cum_m - cum_r) + (lo_m - lo_r) keeps its
// accuracy relative to its own size however large |B| grows in the chunk.
constexpr int kCumRows = 16;

__device__ inline f32x4 two_sum4(const f32x4& a, const f32x4& b, f32x4& err) {
  f32x4 s;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = a[e] + b[e];
    const float bp = s[e] - a[e];
    err[e] = (a[e] - (s[e] - bp)) + (b[e] - bp);
  }
  return s;
}

__global__ __launch_bounds__(kThreads) void k_cumsum(const float* __restrict__ a,
                                                     float* __restrict__ cum,
                                                     float* __restrict__ cum_lo, int L, int dk,
                                                     int C, int NC, int BH) {
  __shared__ f32x4 tot[kThreads], totl[kThreads];
  const int quads = dk / 4, groups = C / kCumRows;      // per chunk
  const int per_chunk = quads * groups;                 // threads per chunk (<= 256)
  const int cpb = kThreads / per_chunk;                 // chunks per block
  const int t = threadIdx.x, sub = t / per_chunk, rem = t % per_chunk;
  const int gq = rem % quads, rg = rem / quads;
  const long chunk = (long)blockIdx.x * cpb + sub;      // global chunk id over BH * NC
  const bool active = sub < cpb && chunk < (long)BH * NC;
  const int bh = active ? (int)(chunk / NC) : 0, n = active ? (int)(chunk % NC) : 0;
  const int r0 = n * C + rg * kCumRows;
  const int r1 = active ? min(L, r0 + kCumRows) : r0;
  const size_t base = (size_t)bh * L * dk + 4 * gq;
  f32x4 v[kCumRows];
#pragma unroll
  for (int i = 0; i < kCumRows; ++i)
    if (r0 + i < r1) v[i] = *reinterpret_cast<const f32x4*>(a + base + (size_t)(r0 + i) * dk);
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
  if (!cum_lo) {
#pragma unroll
    for (int i = 0; i < kCumRows; ++i) {
      if (r0 + i < r1) {
        run += v[i];
        v[i] = run;
      }
    }
    tot[t] = run;
    __syncthreads();
    f32x4 off = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < rg; ++g) off += tot[sub * per_chunk + g * quads + gq];
#pragma unroll
    for (int i = 0; i < kCumRows; ++i)
      if (r0 + i < r1) *reinterpret_cast<f32x4*>(cum + base + (size_t)(r0 + i) * dk) = v[i] + off;
    return;
  }
  // compensated: (v[i], vl[i]) is the group's running sum as hi + lo
  f32x4 vl[kCumRows], runl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kCumRows; ++i) {
    vl[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r0 + i < r1) {
      f32x4 e;
      run = two_sum4(run, v[i], e);
      runl += e;
      v[i] = run;
      vl[i] = runl;
    }
  }
  tot[t] = run;
  totl[t] = runl;
  __syncthreads();
  f32x4 off = {0.f, 0.f, 0.f, 0.f}, offl = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < rg; ++g) {
    f32x4 e;
    off = two_sum4(off, tot[sub * per_chunk + g * quads + gq], e);
    offl += e + totl[sub * per_chunk + g * quads + gq];
  }
#pragma unroll
  for (int i = 0; i < kCumRows; ++i)
    if (r0 + i < r1) {
      f32x4 e;
      const f32x4 h = two_sum4(v[i], off, e);
      *reinterpret_cast<f32x4*>(cum + base + (size_t)(r0 + i) * dk) = h;
      *reinterpret_cast<f32x4*>(cum_lo + base + (size_t)(r0 + i) * dk) = vl[i] + offl + e;
    }
}

hipError_t launch_cumsum(const Plan& p, const float* a, float* cum, float* cum_lo,
                         hipStream_t s) {
  const int per_chunk = (p.dk / 4) * (p.C / kCumRows);
  const int cpb = kThreads / per_chunk;
  const long chunks = (long)p.BH * p.NC;
  dim3 grid((unsigned)((chunks + cpb - 1) / cpb));
  hipLaunchKernelGGL(k_cumsum, grid, dim3(kThreads), 0, s, a, cum, cum_lo, p.L, p.dk, p.C, p.NC,
                     p.BH);
  return hipGetLastError();
}

// ------------------------------------------------------------------ K2: chunk-state recurrence
// One workgroup owns a TS x TS tile of the d_k x d_v state of one (batch, head)
// and walks the chunks of one sequence segment in order (reverse order for the
// backward's dS recurrence).  The tile lives in MFMA accumulators (fp32); each
// chunk's operands are staged transposed through LDS so that both MFMA
// operands read contiguous token runs.  The next chunk's raw inputs are
// loaded into registers while the current chunk updates the state.
//
// SPLIT (bf16 only): the scaled operand X ⊙ e^{...} is held as a high and a
// low bf16 part (two MFMAs), and st_n_lo receives the low part of every
// written state, so that the backward's gradients see ~16-bit operands.
//
// Workgroups are numbered so that the tiles of one (batch, head) are
// consecutive within one XCD (workgroup w runs on XCD w % 8): the tiles that
// re-read the same k / v / cumsum rows then share an L2.
//
// One launch can run two jobs (the forward recurrence of S and the reverse one
// of dS): workgroups below nblk0 take job0, the rest job1, so that the two
// chains, each mostly waiting on its own latencies, share the compute units.
//
// fp32: the decay exponents also take the cumsum's low part (cum_lo, the
// two-sum compensation of k_cumsum), so that they stay accurate however large
// the chunk-local cumsum grows.
template <typename T, int TS, int SPLIT>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    StateJob job0, StateJob job1, int nblk0, const float* __restrict__ cum,
    const float* __restrict__ cum_lo, int L, int dk, int dv, int C, int NC, int NSEG,
    int seg_chunks) {
  constexpr bool LO = sizeof(T) == 4;
  const bool second = blockIdx.x >= (unsigned)nblk0;
  const StateJob& J = second ? job1 : job0;
  const int bid = second ? (int)blockIdx.x - nblk0 : (int)blockIdx.x;
  const int nblk = second ? (int)gridDim.x - nblk0 : nblk0;
  const int REV = J.rev, mode = J.mode;
  const T* __restrict__ X = static_cast<const T*>(J.X);
  const T* __restrict__ Y = static_cast<const T*>(J.Y);
  const float* __restrict__ init = J.init;
  const float* __restrict__ seg_in = J.seg_in;
  T* __restrict__ st_t = static_cast<T*>(J.st_t);
  T* __restrict__ st_n = static_cast<T*>(J.st_n);
  T* __restrict__ st_n_lo = static_cast<T*>(J.st_n_lo);
  float* __restrict__ end_out = J.end_out;
  float* __restrict__ seg_out = J.seg_out;
  float* __restrict__ seg_g = J.seg_g;
  using M = Mma<T>;
  constexpr int NT1 = TS / 16, NTT = NT1 * NT1, NW = (NTT + 3) / 4;
  constexpr int LDX = TS + gather_pad<T>(TS);    // row-major [token][channel], padded
  constexpr int CG = TS / 8;                     // 8-channel column groups
  constexpr int RS = kThreads / CG;              // row stride between a thread's rows
  constexpr int RPT = (64 + RS - 1) / RS;        // rows per thread (chunk <= 64)
  __shared__ __attribute__((aligned(16))) T xs[64][LDX];
  __shared__ __attribute__((aligned(16))) T xl[SPLIT ? 64 : 1][SPLIT ? LDX : 8];
  __shared__ __attribute__((aligned(16))) T ys[64][LDX];
  __shared__ float gam[TS];
  // The state entering each update, staged for stores of whole row
  // segments: [i][j] (hi, and lo when split) and, for the transposed copy,
  // [j][i].
  constexpr int LDS_ = TS + 16 / (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) T stg[SPLIT ? 2 : 1][TS][LDS_];
  __shared__ __attribute__((aligned(16))) T stgT[TS][LDS_];

  const int ntj = dv / TS, nti = dk / TS;
  const int lid = xcd_logical(bid, nblk);
  const int j0 = (lid % ntj) * TS, i0 = ((lid / ntj) % nti) * TS;
  const int z = lid / (ntj * nti), bh = z / NSEG, seg = z % NSEG;
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int cg = tid % CG, rbase = tid / CG, c0 = cg * 8;
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

  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks), nsteps = max(0, ne - nb);
  // prefetch registers: this thread's rows of X, Y, cumsum and the chunk total
  Raw8<T> rx[RPT], ry[RPT];
  f32x4 rb[RPT][2], rg[2], rbl[RPT][2], rgl[2];
#define GLA_STATE_FETCH(NCH)                                                              \
  do {                                                                                     \
    const int fr0 = (NCH) * C, frv = min(C, L - fr0);                                      \
    const float* glast = cum + xo + (size_t)(fr0 + frv - 1) * dk + i0 + c0;                \
    rg[0] = *reinterpret_cast<const f32x4*>(glast);                                        \
    rg[1] = *reinterpret_cast<const f32x4*>(glast + 4);                                    \
    if constexpr (LO) {                                                                    \
      const float* gll = cum_lo + (glast - cum);                                           \
      rgl[0] = *reinterpret_cast<const f32x4*>(gll);                                       \
      rgl[1] = *reinterpret_cast<const f32x4*>(gll + 4);                                   \
    }                                                                                      \
    _Pragma("unroll") for (int u = 0; u < RPT; ++u) {                                      \
      const int row = rbase + u * RS;                                                      \
      if (row < frv) {                                                                     \
        raw_load(rx[u], X + xo + (size_t)(fr0 + row) * dk + i0 + c0);                      \
        raw_load(ry[u], Y + yo + (size_t)(fr0 + row) * dv + j0 + c0);                      \
        const float* bp = cum + xo + (size_t)(fr0 + row) * dk + i0 + c0;                   \
        rb[u][0] = *reinterpret_cast<const f32x4*>(bp);                                    \
        rb[u][1] = *reinterpret_cast<const f32x4*>(bp + 4);                                \
        if constexpr (LO) {                                                                \
          const float* bpl = cum_lo + (bp - cum);                                          \
          rbl[u][0] = *reinterpret_cast<const f32x4*>(bpl);                                \
          rbl[u][1] = *reinterpret_cast<const f32x4*>(bpl + 4);                            \
        }                                                                                  \
      } else {                                                                             \
        raw_zero(rx[u]);                                                                   \
        raw_zero(ry[u]);                                                                   \
        rb[u][0] = rb[u][1] = f32x4{};                                                     \
        rbl[u][0] = rbl[u][1] = f32x4{};                                                   \
      }                                                                                    \
    }                                                                                      \
  } while (0)
  if (nsteps > 0) GLA_STATE_FETCH(REV ? ne - 1 : nb);
  float gsum[8];  // this segment's total log decay for the thread's 8 channels
#pragma unroll
  for (int e = 0; e < 8; ++e) gsum[e] = 0.f;

  for (int step = 0; step < nsteps; ++step) {
    const int n = REV ? (ne - 1 - step) : (nb + step);
    // stage this chunk (registers -> LDS, row-major, X scaled)
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int row = rbase + u * RS;
      if (row >= C) continue;
      float xv[8], xlo[8], yv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float b = rb[u][e >> 2][e & 3], g = rg[e >> 2][e & 3];
        if constexpr (LO) {
          const float bl = rbl[u][e >> 2][e & 3], gl = rgl[e >> 2][e & 3];
          xv[e] = raw_get(rx[u], e) * (REV ? gexp<T>(b) * gexp<T>(bl) : gexp<T>((g - b) + (gl - bl)));
        } else {
          xv[e] = raw_get(rx[u], e) * gexp<T>(REV ? b : g - b);
        }
        xlo[e] = xv[e] - to_f32(from_f32<T>(xv[e]));
        yv[e] = raw_get(ry[u], e);
      }
      store8_aligned8(&xs[row][c0], xv);
      if constexpr (SPLIT) store8_aligned8(&xl[row][c0], xlo);
      store8_aligned8(&ys[row][c0], yv);
    }
    if (rbase == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gam[c0 + e] = gexp<T>(rg[e >> 2][e & 3]);
        gsum[e] += rg[e >> 2][e & 3];
        if constexpr (LO) {
          gam[c0 + e] *= gexp<T>(rgl[e >> 2][e & 3]);
          gsum[e] += rgl[e >> 2][e & 3];
        }
      }
    }
    // prefetch the next chunk while this one is consumed
    if (step + 1 < nsteps) GLA_STATE_FETCH(REV ? n - 1 : n + 1);

    // The state entering this chunk's update: S_{n-1} (forward) or dS_n
    // (reverse), staged in LDS, then stored as 16-byte units of rows.
    const bool emit = mode == SEG_FILL && (st_t || st_n);
    if (emit) {
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int tt = w + 4 * t;
        if (tt >= NTT) continue;
        const int ti = tt / NT1, tj = tt % NT1;
        const int jl = tj * 16 + (l & 15), il = ti * 16 + (l >> 4) * 4;
        if (st_t) store4(&stgT[jl][il], acc[t]);
        if (st_n) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const T hi = from_f32<T>(acc[t][r]);
            stg[0][il + r][jl] = hi;
            if constexpr (SPLIT) stg[1][il + r][jl] = from_f32<T>(acc[t][r] - to_f32(hi));
          }
        }
      }
    }
    __syncthreads();
    if (emit) {
      constexpr int EPU = 16 / (int)sizeof(T);
      for (int it = tid; it < TS * (TS / EPU); it += kThreads) {
        const int row = it / (TS / EPU), u = (it % (TS / EPU)) * EPU;
        if (st_n) {
          const size_t idx = (((size_t)bh * NC + n) * dk + i0 + row) * dv + j0 + u;
          *reinterpret_cast<f32x4*>(st_n + idx) = *reinterpret_cast<const f32x4*>(&stg[0][row][u]);
          if (SPLIT && st_n_lo)
            *reinterpret_cast<f32x4*>(st_n_lo + idx) =
                *reinterpret_cast<const f32x4*>(&stg[SPLIT ? 1 : 0][row][u]);
        }
        if (st_t)
          *reinterpret_cast<f32x4*>(st_t + (((size_t)bh * NC + n) * dv + j0 + row) * dk + i0 + u) =
              *reinterpret_cast<const f32x4*>(&stgT[row][u]);
      }
    }
    if constexpr (sizeof(T) == 2) {
      // bf16: K runs down the rows (transposed reads), at most two K steps
      // (C <= 64).  Tile t of wave w is (ti, tj) = ((w + 4 t) / NT1, (w + 4 t)
      // % NT1); every fragment of the step is read before the products.
      constexpr int KMAX = 64 / M::K;
      typename M::frag fa[NW][KMAX], fl[NW][KMAX], fb[NW][KMAX];
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int tt = w + 4 * t;
        if (tt >= NTT) continue;
        const int ti = tt / NT1, tj = tt % NT1;
#pragma unroll
        for (int ks = 0; ks < KMAX; ++ks) {
          if (ks * M::K >= C) continue;
          fa[t][ks] = col_frag_tr(&xs[0][0], LDX, ks * M::K, ti * 16, l);
          fb[t][ks] = col_frag_tr(&ys[0][0], LDX, ks * M::K, tj * 16, l);
          if constexpr (SPLIT) fl[t][ks] = col_frag_tr(&xl[0][0], LDX, ks * M::K, ti * 16, l);
        }
      }
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int tt = w + 4 * t;
        if (tt >= NTT) continue;
        const int ti = tt / NT1;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] *= gam[ti * 16 + (l >> 4) * 4 + r];
#pragma unroll
        for (int ks = 0; ks < KMAX; ++ks) {
          if (ks * M::K >= C) continue;
          acc[t] = M::run(fa[t][ks], fb[t][ks], acc[t]);
          if constexpr (SPLIT) acc[t] = M::run(fl[t][ks], fb[t][ks], acc[t]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        const int tt = w + 4 * t;
        if (tt >= NTT) continue;
        const int ti = tt / NT1, tj = tt % NT1;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] *= gam[ti * 16 + (l >> 4) * 4 + r];
        for (int kk = 0; kk < C; kk += M::K) {
          const int kr = kk + (l >> 4) * M::KPL;
          const typename M::frag a = gather_frag<T>(&xs[kr][ti * 16 + (l & 15)], LDX);
          const typename M::frag b = gather_frag<T>(&ys[kr][tj * 16 + (l & 15)], LDX);
          acc[t] = M::run(a, b, acc[t]);
          if constexpr (SPLIT) acc[t] = M::run(gather_frag<T>(&xl[kr][ti * 16 + (l & 15)], LDX), b, acc[t]);
        }
      }
    }
    __syncthreads();
  }

  if (mode == SEG_LOCAL && seg_g && j0 == 0 && rbase == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) seg_g[((size_t)bh * NSEG + seg) * dk + i0 + c0 + e] = gsum[e];
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

#undef GLA_STATE_FETCH

template <typename T, int TS, int SPLIT>
static hipError_t launch_cs(const Plan& p, const StateJob& a, const StateJob* b, hipStream_t s) {
  const int per = (p.dv / TS) * (p.dk / TS) * p.BH * p.NSEG;
  hipLaunchKernelGGL((k_chunk_state<T, TS, SPLIT>), dim3(b ? 2 * per : per), dim3(kThreads), 0, s,
                     a, b ? *b : a, per, cum_of(a), cum_lo_of(p, cum_of(a)), p.L, p.dk, p.dv,
                     p.C, p.NC, p.NSEG, p.seg_chunks);
  return hipGetLastError();
}

template <typename T, int SPLIT>
static hipError_t launch_cs_ts(const Plan& p, const StateJob& a, const StateJob* b,
                               hipStream_t s) {
  switch (p.TS) {
    case 64: return launch_cs<T, 64, SPLIT>(p, a, b, s);
    case 32: return launch_cs<T, 32, SPLIT>(p, a, b, s);
    default: return launch_cs<T, 16, SPLIT>(p, a, b, s);
  }
}

static hipError_t launch_state_jobs(const Plan& p, int split, const StateJob& a,
                                    const StateJob* b, hipStream_t s) {
  if (p.bf16) return split ? launch_cs_ts<bf16, 1>(p, a, b, s) : launch_cs_ts<bf16, 0>(p, a, b, s);
  return launch_cs_ts<float, 0>(p, a, b, s);
}

hipError_t launch_chunk_state(const Plan& p, int rev, int mode, int split, const void* X,
                              const void* Y, const float* cum, const float* init,
                              const float* seg_in, void* st_t, void* st_n, void* st_n_lo,
                              float* end_out, float* seg_out, float* seg_g, hipStream_t s) {
  const StateJob a{rev, mode, X, Y, cum, init, seg_in, st_t, st_n, split ? st_n_lo : nullptr,
                   end_out, seg_out, seg_g};
  return launch_state_jobs(p, split, a, nullptr, s);
}

hipError_t launch_chunk_state_pair(const Plan& p, int split, const StateJob& a, const StateJob& b,
                                   hipStream_t s) {
  if (a.cum != b.cum) return hipErrorInvalidValue;
  return launch_state_jobs(p, split, a, &b, s);
}

// ------------------------------------------------------------------ segment scan
// Sequence-level parallelism for long sequences: each segment's local state
// (zero start) is combined with the state entering it,
//   S_in(s+1) = e^{G_s} ⊙ S_in(s) + U_s,  G_s = the segment's total log decay,
// the associative step of the chunk recurrence (papercache.org notes §2.2,
// chunk-level recurrence, applied to groups of chunks).  A thread owns 4
// adjacent state entries of one row; the U loads of 8 segments are issued
// before they are combined.
__global__ __launch_bounds__(kThreads) void k_segment_scan(
    const float* __restrict__ seg_g, const float* __restrict__ init,
    const float* __restrict__ seg_u, float* __restrict__ seg_in, float* __restrict__ end_out,
    int dk, int dv, int NSEG, int rev, long total4) {
  const long t = (long)blockIdx.x * kThreads + threadIdx.x;
  if (t >= total4) return;
  const int dv4 = dv / 4, j = (int)(t % dv4) * 4;
  const long r = t / dv4;
  const int i = (int)(r % dk), bh = (int)(r / dk);
  const size_t off = ((size_t)bh * dk + i) * dv + j;
  f32x4 S = init ? *reinterpret_cast<const f32x4*>(init + off) : f32x4{};
  for (int t0 = 0; t0 < NSEG; t0 += 8) {
    f32x4 U[8];
    float G[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tt = t0 + u;
      if (tt < NSEG) {
        const int seg = rev ? NSEG - 1 - tt : tt;
        U[u] = *reinterpret_cast<const f32x4*>(seg_u + (((size_t)bh * NSEG + seg) * dk + i) * dv + j);
        G[u] = seg_g[((size_t)bh * NSEG + seg) * dk + i];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tt = t0 + u;
      if (tt < NSEG) {
        const int seg = rev ? NSEG - 1 - tt : tt;
        *reinterpret_cast<f32x4*>(seg_in + (((size_t)bh * NSEG + seg) * dk + i) * dv + j) = S;
        S = expf(G[u]) * S + U[u];
      }
    }
  }
  if (end_out) *reinterpret_cast<f32x4*>(end_out + off) = S;
}

hipError_t launch_segment_scan(const Plan& p, int rev, const float* seg_g, const float* init,
                               const float* seg_u, float* seg_in, float* end_out,
                               hipStream_t s) {
  const long total4 = (long)p.BH * p.dk * (p.dv / 4);
  if (total4 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_segment_scan, dim3((unsigned)((total4 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, seg_g, init, seg_u, seg_in, end_out, p.dk, p.dv,
                     p.NSEG, rev, total4);
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

  // Slice s of (q, k, cumsum) and the state fragments are fetched into
  // registers one slice ahead of their use.
  constexpr int SITEMS = C * (KS / 8);  // 8-element items per slice
  constexpr int KSTEPS = KS / M::K;
  const int srow = tid / (KS / 8), sc8 = (tid % (KS / 8)) * 8;
  const bool sact = tid < SITEMS;
  const bool svalid = sact && srow < rv;
  const int scrow = r0 + (srow < rv ? srow : rv - 1);
  Raw8<T> pq, pk;
  f32x4 pb2[2];
  typename M::frag fnext[KSTEPS][NCW];
#define GLA_SLICE_FETCH(S0)                                                               \
  do {                                                                                     \
    if (sact) {                                                                            \
      const float* bp = cum + qo + (size_t)scrow * dk + (S0) + sc8;                        \
      pb2[0] = *reinterpret_cast<const f32x4*>(bp);                                        \
      pb2[1] = *reinterpret_cast<const f32x4*>(bp + 4);                                    \
      if (svalid) {                                                                        \
        raw_load(pq, q + qo + (size_t)scrow * dk + (S0) + sc8);                            \
        raw_load(pk, k + qo + (size_t)scrow * dk + (S0) + sc8);                            \
      } else {                                                                             \
        raw_zero(pq);                                                                      \
        raw_zero(pk);                                                                      \
      }                                                                                    \
    }                                                                                      \
    _Pragma("unroll") for (int ks = 0; ks < KSTEPS; ++ks)                                  \
    _Pragma("unroll") for (int ct = 0; ct < NCW; ++ct) {                                   \
      const int col = j0 + (wc + WC * ct) * 16 + (l & 15);                                \
      fnext[ks][ct] =                                                                      \
          load_frag<T>(stp + (size_t)col * dk + (S0) + ks * M::K + (l >> 4) * M::KPL);     \
    }                                                                                      \
  } while (0)
  GLA_SLICE_FETCH(0);

  for (int s0 = 0; s0 < dk; s0 += KS) {
    __syncthreads();
    if (sact) {
      float qv[8], kv[8], bv[8], qt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] = raw_get(pq, e);
        kv[e] = raw_get(pk, e);
        bv[e] = pb2[e >> 2][e & 3];
        qt[e] = qv[e] * gexp<T>(bv[e]);
      }
      store8(qs + srow * LDT + sc8, qv);
      store8(ks + srow * LDT + sc8, kv);
      store8(bs + srow * LDF + sc8, bv);
      store8(qts + srow * LDT + sc8, qt);
    }
    __syncthreads();
    PB::gates(bs, als);
    // inter-chunk term
#pragma unroll
    for (int ks2 = 0; ks2 < KSTEPS; ++ks2) {
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) {
        const int rti = wr + WR * rt;
        if (rti >= NRT) continue;
        auto a = load_frag<T>(qts + (rti * 16 + (l & 15)) * LDT + ks2 * M::K + (l >> 4) * M::KPL);
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) acc[rt][ct] = M::run(a, fnext[ks2][ct], acc[rt][ct]);
      }
    }
    // next slice's loads overlap the score-matrix work below
    if (s0 + KS < dk) GLA_SLICE_FETCH(s0 + KS);
    pb.offdiag(qs, ks, bs);
    __syncthreads();
    pb.diag(qs, ks, als);
  }
  // V tile loads in flight while the score matrix is reduced
  constexpr int VITEMS = (C * (TVO / 8) + kThreads - 1) / kThreads;
  Raw8<T> pv[VITEMS];
#pragma unroll
  for (int u = 0; u < VITEMS; ++u) {
    const int it = tid + u * kThreads;
    const int row = it / (TVO / 8), c8 = (it % (TVO / 8)) * 8;
    if (it < C * (TVO / 8) && row < rv) raw_load(pv[u], v + vo + (size_t)(r0 + row) * dv + j0 + c8);
    else raw_zero(pv[u]);
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
#pragma unroll
  for (int u = 0; u < VITEMS; ++u) {
    const int it = tid + u * kThreads;
    if (it >= C * (TVO / 8)) continue;
    const int row = it / (TVO / 8), c8 = (it % (TVO / 8)) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(c8 + e) * LDV + row] = from_f32<T>(raw_get(pv[u], e));
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

#undef GLA_SLICE_FETCH

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
