// gla_recur.hip -- two-pass forward of the GLA chunkwise layer (gfx950).
//
// Pass 1, k_chunk_prep: one workgroup per (batch-head, chunk), all chunks in
// parallel.  From q, k and log alpha of the chunk it forms
//   B      = chunk-local inclusive cumsum of log alpha  (per key channel)
//   Q~     = Q ⊙ e^{B}            (rows of the chunk, I/O type)
//   K~     = K ⊙ e^{b - B}        (b = B at the chunk's last row)
//   b      = the chunk's total log decay
//   P      = the causal gated score matrix of the chunk (gla_pblock.h):
//            P[m][r] = sum_k q_mk k_rk e^{B_mk - B_rk}, r <= m
// (papercache.org notes §4.2 chunkwise form with Lambda, Gamma, gamma; §4.3 /
// Figure 3 for P).  For bf16 I/O, P is stored rounded to bf16 plus the low
// part of its diagonal 16 x 16 blocks.
//
// Pass 2, k_chunk_recur: one workgroup per (batch-head, sequence segment,
// d_v tile), walking the segment's chunks in order with its d_k x d_v_tile
// slice of the state in MFMA accumulators (fp32):
//   O[n]^T = S_{n-1}^T Q~^T + V^T P^T                 (output, transposed)
//   S_n    = diag(e^{b_n}) S_{n-1} + K~^T V           (state)
// (notes §4.2; §3.3 / Figure 1a keeps the state on chip).  Every chunk's
// Q~, K~, P, b and V tile stream into LDS with LDS-DMA (global_load_lds)
// while the previous chunk computes; each wave owns 16 state columns.  In
// its local mode (no output) the same walk starts from zero and leaves each
// segment's own state contribution and total log decay for the segment scan.
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"

namespace gla {

namespace {

// ds_read_b64_tr_b16: within each 16-lane group, lane 4 a + b receives
// element b of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12.
typedef short v4s16 __attribute__((ext_vector_type(4)));
__device__ inline bf16x4 ds_read_tr(const bf16* p) {
  const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s16*)(const_cast<bf16*>(p)));
  bf16x4 o;
  __builtin_memcpy(&o, &r, 8);
  return o;
}
__device__ inline bf16x8 join8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
  return r;
}

// Asynchronous global -> LDS copy of one 16-byte unit per lane: lane i of the
// wave writes LDS bytes [lds_wave_base + 16 i, + 16).  lds_wave_base must be
// the same for the whole wave.
__device__ inline void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                   0, 0);
}
// Wait for this wave's outstanding global memory operations (LDS copies too).
__device__ inline void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- LDS tile swizzles --------------------------------------------------
// Tiles are row-major arrays of 16-byte units; unit u of row r is stored at
// unit slot u ^ swz(r) of that row (an involution within the row, since every
// row holds a power-of-two number of units and the mask stays below it).
// Each mask spreads the rows that one MFMA operand read touches over distinct
// LDS bank windows.  W = 16-element column windows per row.
//
// Row reads (the 16 rows of a tile, one window each): bf16 windows are 32 B,
// fp32 windows 64 B; rows sharing a 256-byte bank span are told apart by the
// row bits below the span, the rest by the XOR.
template <int ES, int W>
__device__ inline int swz_rows(int r) {
  constexpr int WPS = ES == 2 ? 8 : 4;      // windows per 256-byte bank span
  constexpr int RP = W >= WPS ? 1 : WPS / W;  // rows per bank span
  constexpr int MW = W >= WPS ? WPS : W;
  return ((r / RP) & (MW - 1)) * (ES == 2 ? 2 : 4);
}
// Token-run reads: rows 8 g + j (+ 4) for bf16 transposed reads (j < 4, lane
// group g), rows 16 b + 4 g + i for fp32 scalar reads (fixed i).
template <int ES, int W>
__device__ inline int swz_runs(int r) {
  if constexpr (ES == 2) {
    int m = 0;
    if constexpr (W >= 8) m = (r & 3) | (((r >> 3) & 1) << 2);
    else if constexpr (W == 4) m = ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
    else if constexpr (W == 2) m = (r >> 3) & 1;
    return 2 * m;
  } else {
    int m = 0;
    if constexpr (W >= 4) m = (r >> 2) & 3;
    else if constexpr (W == 2) m = (r >> 2) & 1;
    return 4 * m;
  }
}

constexpr int kLdsLimit = 160 * 1024;

// Issue the NW wave copies of one staged tile across the workgroup's NWV
// waves: copy c (64 units of 16 bytes) lands at LDS unit slots off + 64 c ..;
// src(s) is the global address of the unit for slot s.
template <int NW, int NWV, typename F>
__device__ inline void stage_tile(unsigned char* base, int off, int w, int l, F src) {
#pragma unroll
  for (int i = 0; i < (NW + NWV - 1) / NWV; ++i) {
    const int c = w + i * NWV;
    if (NW % NWV != 0 && c >= NW) break;
    dma16(src(c * 64 + l), base + (off + c * 64) * 16);
  }
}

}  // namespace

// =========================================================== pass 1: chunk prep
template <typename T, int C>
__global__ __launch_bounds__(kThreads) void k_chunk_prep(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ la,
    T* __restrict__ qg, T* __restrict__ kg, float* __restrict__ glog, T* __restrict__ ph,
    T* __restrict__ pl, int L, int dk, int NC) {
  using PB = PBuilder<T, C>;
  constexpr bool BF = PB::BF;
  constexpr int KS = PB::KS, LDT = PB::LDT, LDF = PB::LDF;
  constexpr int EPU = 16 / (int)sizeof(T);
  constexpr int RG = kThreads / KS;  // row groups of the slice cumsum
  constexpr int RPT = C / RG;        // rows per thread
  static_assert(RPT >= 1 && C % RG == 0, "cumsum row split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[PB::SLICE_BYTES];
  __shared__ float pd[4][16][17];
  __shared__ float tot[RG][KS];
  __shared__ __attribute__((aligned(16))) T ps[C * C];
  __shared__ __attribute__((aligned(16))) T ls[BF ? C * 16 : EPU];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  float* bs = reinterpret_cast<float*>(ks + C * LDT);
  float* als = bs + C * LDF;

  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const size_t io = (size_t)bh * L * dk;                      // q, k, log alpha
  const size_t cb = (size_t)bh * NC + n;                      // chunk id
  const size_t go = cb * C * dk;                              // Q~, K~ (padded rows)

  for (int it = tid; it < C * C; it += kThreads) ps[it] = from_f32<T>(0.f);
  if constexpr (BF)
    for (int it = tid; it < C * 16; it += kThreads) ls[it] = from_f32<T>(0.f);

  PB pb;
  pb.init();
  const int ch = tid % KS, rg = tid / KS;
  for (int s0 = 0; s0 < dk; s0 += KS) {
    // log alpha of the thread's rows (0 past the end of the sequence)
    float av[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      av[i] = row < rv ? la[io + (size_t)(r0 + row) * dk + s0 + ch] : 0.f;
    }
    __syncthreads();  // previous slice's readers of qs, ks, bs, tot are done
    for (int it = tid; it < C * (KS / 8); it += kThreads) {
      const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
      float qv[8], kv[8];
      if (row < rv) {
        load8(q + io + (size_t)(r0 + row) * dk + s0 + c8, qv);
        load8(k + io + (size_t)(r0 + row) * dk + s0 + c8, kv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = kv[e] = 0.f;
      }
      store8(qs + row * LDT + c8, qv);
      store8(ks + row * LDT + c8, kv);
    }
    // chunk-local cumsum: RPT rows per thread, then the preceding groups' totals
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      run += av[i];
      av[i] = run;
    }
    tot[rg][ch] = run;
    __syncthreads();
    float off = 0.f;
    for (int g = 0; g < rg; ++g) off += tot[g][ch];
#pragma unroll
    for (int i = 0; i < RPT; ++i) bs[(rg * RPT + i) * LDF + ch] = av[i] + off;
    __syncthreads();
    // Q~ = Q ⊙ e^B, K~ = K ⊙ e^{b - B}, b
    for (int it = tid; it < C * (KS / 8); it += kThreads) {
      const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
      float qv[8], kv[8], bv[8], gv[8];
      load8(qs + row * LDT + c8, qv);
      load8(ks + row * LDT + c8, kv);
      load8(bs + row * LDF + c8, bv);
      load8(bs + (C - 1) * LDF + c8, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] *= gexp<T>(bv[e]);
        kv[e] *= gexp<T>(gv[e] - bv[e]);
      }
      store8(qg + go + (size_t)row * dk + s0 + c8, qv);
      store8(kg + go + (size_t)row * dk + s0 + c8, kv);
    }
    if (tid < KS) glog[cb * dk + s0 + tid] = bs[(C - 1) * LDF + tid];
    PB::gates(bs, als);
    pb.offdiag(qs, ks, bs);
    __syncthreads();
    pb.diag(qs, ks, als);
  }
  __syncthreads();
  pb.finish(pd, [&](int m, int r, float val) {
    const T hi = from_f32<T>(val);
    ps[m * C + r] = hi;
    if constexpr (BF) {
      if ((m >> 4) == (r >> 4)) ls[m * 16 + (r & 15)] = from_f32<T>(val - to_f32(hi));
    }
  });
  __syncthreads();
  typedef f32x4 unit_t;
  unit_t* pout = reinterpret_cast<unit_t*>(ph + cb * C * C);
  const unit_t* pin = reinterpret_cast<const unit_t*>(ps);
  for (int it = tid; it < C * C / EPU; it += kThreads) pout[it] = pin[it];
  if constexpr (BF) {
    unit_t* lout = reinterpret_cast<unit_t*>(pl + cb * C * 16);
    const unit_t* lin = reinterpret_cast<const unit_t*>(ls);
    for (int it = tid; it < C * 16 / EPU; it += kThreads) lout[it] = lin[it];
  }
}

// =========================================================== pass 2: recurrence
template <typename T, int C, int DK, int NWV, int OUT>
struct RecurLayout {
  static constexpr int ES = (int)sizeof(T);
  static constexpr bool BF = ES == 2;
  static constexpr int EPU = 16 / ES;           // elements per 16-byte unit
  static constexpr int DVT = 16 * NWV;          // d_v tile: 16 columns per wave
  static constexpr int QUR = DK / EPU;          // units per Q~ / K~ row
  static constexpr int PUR = C / EPU;           // units per P row
  static constexpr int VUR = DVT / EPU;         // units per V row
  static constexpr int QUN = OUT ? C * QUR : 0;
  static constexpr int KUN = C * QUR;
  static constexpr int PUN = OUT ? C * PUR : 0;
  static constexpr int LUN = (OUT && BF) ? C * 16 / EPU : 0;
  static constexpr int GUN = DK / 4 < 64 ? 64 : DK / 4;  // padded to a wave
  static constexpr int VUN = C * VUR;
  static constexpr int oQ = 0, oK = oQ + QUN, oP = oK + KUN, oL = oP + PUN, oG = oL + LUN,
                       oV = oG + GUN, UN = oV + VUN;
  static constexpr int BUF = UN * 16;
  static constexpr int NBUF = 2 * BUF <= kLdsLimit ? 2 : 1;
  static_assert(QUN % 64 == 0 && KUN % 64 == 0 && PUN % 64 == 0 && LUN % 64 == 0 &&
                    GUN % 64 == 0 && VUN % 64 == 0,
                "every staged tile is a whole number of wave copies");
  static_assert(BUF <= kLdsLimit, "staged chunk exceeds LDS");
};

template <typename T, int C, int DK, int NWV, int OUT>
__global__ __launch_bounds__(NWV * kWave) void k_chunk_recur(
    const T* __restrict__ qg, const T* __restrict__ kg, const T* __restrict__ ph,
    const T* __restrict__ pl, const float* __restrict__ glog, const T* __restrict__ v,
    const float* __restrict__ init, T* __restrict__ o, float* __restrict__ fin,
    float* __restrict__ seg_g, int L, int dv, int NC, int NSEG, int seg_chunks) {
  using Lay = RecurLayout<T, C, DK, NWV, OUT>;
  constexpr bool BF = Lay::BF;
  constexpr int EPU = Lay::EPU, DVT = Lay::DVT, NTH = NWV * kWave;
  constexpr int NRT = C / 16, NKT = DK / 16;
  constexpr int WQ = DK / 16, WV = DVT / 16, WP = C / 16;  // 16-column windows per row
  __shared__ __attribute__((aligned(16))) unsigned char lds[Lay::NBUF * Lay::BUF];

  const int ntv = dv / DVT;
  const int lid = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lid % ntv, seg = (lid / ntv) % NSEG, bh = lid / (ntv * NSEG);
  const int j0 = tile * DVT;
  const int w = wave_id(), l = lane_id(), g = l >> 4, ln = l & 15;
  const int col = j0 + 16 * w + ln;  // this lane's state / output column
  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);

  // ---- state slice: lane holds S[16 a + 4 g + r][col]
  floatx4 S[NKT];
  {
    const float* src = nullptr;
    if (OUT) src = NSEG > 1 ? init + ((size_t)bh * NSEG + seg) * DK * dv
                            : (init ? init + (size_t)bh * DK * dv : nullptr);
#pragma unroll
    for (int a = 0; a < NKT; ++a) {
      S[a] = zero4();
      if (src) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][r] = src[(size_t)(a * 16 + 4 * g + r) * dv + col];
      }
    }
  }
  constexpr int NGS = (DK + NTH - 1) / NTH;
  float gsum[NGS];
#pragma unroll
  for (int i = 0; i < NGS; ++i) gsum[i] = 0.f;

  // ---- stage chunk n into buffer b: every tile as whole wave copies
  auto issue = [&](int n, int b) {
    unsigned char* base = lds + b * Lay::BUF;
    const size_t cb = (size_t)bh * NC + n;
    if constexpr (OUT) {
      const T* qb = qg + cb * C * DK;
      stage_tile<Lay::QUN / 64, NWV>(base, Lay::oQ, w, l, [&](int s) {
        const int r = s / Lay::QUR, u = (s % Lay::QUR) ^ swz_rows<Lay::ES, WQ>(r);
        return qb + r * DK + u * EPU;
      });
      const T* pb = ph + cb * C * C;
      stage_tile<Lay::PUN / 64, NWV>(base, Lay::oP, w, l, [&](int s) {
        const int r = s / Lay::PUR, u = (s % Lay::PUR) ^ swz_rows<Lay::ES, WP>(r);
        return pb + r * C + u * EPU;
      });
      if constexpr (BF) {
        const T* lb = pl + cb * C * 16;
        stage_tile<Lay::LUN / 64, NWV>(base, Lay::oL, w, l, [&](int s) { return lb + s * EPU; });
      }
    }
    const T* kb = kg + cb * C * DK;
    stage_tile<Lay::KUN / 64, NWV>(base, Lay::oK, w, l, [&](int s) {
      const int r = s / Lay::QUR, u = (s % Lay::QUR) ^ swz_runs<Lay::ES, WQ>(r);
      return kb + r * DK + u * EPU;
    });
    // chunk log decays: DK / 4 units, the rest of the wave copy repeats unit 0
    const float* gb = glog + cb * DK;
    stage_tile<Lay::GUN / 64, NWV>(base, Lay::oG, w, l,
                                   [&](int s) { return gb + (s < DK / 4 ? s : 0) * 4; });
    // V rows past the end of the sequence repeat the last row (their K~ rows
    // and P columns are zero)
    const int r0 = n * C, last = L - 1;
    const T* vb = v + (size_t)bh * L * dv + j0;
    stage_tile<Lay::VUN / 64, NWV>(base, Lay::oV, w, l, [&](int s) {
      const int r = s / Lay::VUR, u = (s % Lay::VUR) ^ swz_runs<Lay::ES, WV>(r);
      return vb + (size_t)min(r0 + r, last) * dv + u * EPU;
    });
  };

  if (nb < ne) issue(nb, 0);
  for (int n = nb; n < ne; ++n) {
    const int b = Lay::NBUF == 2 ? ((n - nb) & 1) : 0;
    wait_vm();
    __syncthreads();  // chunk n staged; every wave is done with the other buffer
    if (Lay::NBUF == 2 && n + 1 < ne) issue(n + 1, b ^ 1);
    const unsigned char* base = lds + b * Lay::BUF;
    const T* Qs = reinterpret_cast<const T*>(base + Lay::oQ * 16);
    const T* Ks = reinterpret_cast<const T*>(base + Lay::oK * 16);
    const T* Ps = reinterpret_cast<const T*>(base + Lay::oP * 16);
    const T* Ls = reinterpret_cast<const T*>(base + Lay::oL * 16);
    const float* Gs = reinterpret_cast<const float*>(base + Lay::oG * 16);
    const T* Vs = reinterpret_cast<const T*>(base + Lay::oV * 16);
    // element (row, c) of a swizzled tile with RU units per row
    auto qx = [&](int row, int c) {
      return row * DK + (((c / EPU) ^ swz_rows<Lay::ES, WQ>(row)) * EPU) + c % EPU;
    };
    auto kx = [&](int row, int c) {
      return row * DK + (((c / EPU) ^ swz_runs<Lay::ES, WQ>(row)) * EPU) + c % EPU;
    };
    auto px = [&](int row, int c) {
      return row * C + (((c / EPU) ^ swz_rows<Lay::ES, WP>(row)) * EPU) + c % EPU;
    };
    auto vx = [&](int row, int c) {
      return row * DVT + (((c / EPU) ^ swz_runs<Lay::ES, WV>(row)) * EPU) + c % EPU;
    };
    const int vc = 16 * w;  // this wave's first column within the tile

    if constexpr (BF) {
      // V fragments over token runs 32 kt + 8 g + e at column vc + ln
      bf16x8 vf[C / 32];
#pragma unroll
      for (int kt = 0; kt < C / 32; ++kt) {
        const int ra = 32 * kt + 8 * g + (ln >> 2), c = vc + 4 * (ln & 3);
        vf[kt] = join8(ds_read_tr(Vs + vx(ra, c)), ds_read_tr(Vs + vx(ra + 4, c)));
      }
      if constexpr (OUT) {
        floatx4 ot[NRT];
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) ot[jt] = zero4();
        // O^T += S^T Q~^T over pairs of 16-channel tiles; the MFMA's K index
        // 8 g + e maps to channel 32 a2 + 4 g + e (e < 4) or + 16 + 4 g + e - 4
#pragma unroll
        for (int a2 = 0; a2 < NKT / 2; ++a2) {
          bf16x8 A;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            A[r] = static_cast<bf16>(S[2 * a2][r]);
            A[r + 4] = static_cast<bf16>(S[2 * a2 + 1][r]);
          }
#pragma unroll
          for (int jt = 0; jt < NRT; ++jt) {
            const int row = 16 * jt + ln;
            const bf16x4 x0 = *reinterpret_cast<const bf16x4*>(Qs + qx(row, 32 * a2 + 4 * g));
            const bf16x4 x1 = *reinterpret_cast<const bf16x4*>(Qs + qx(row, 32 * a2 + 16 + 4 * g));
            ot[jt] = Mma<bf16>::run(A, join8(x0, x1), ot[jt]);
          }
        }
        // O^T += V^T P^T (P rounded; its diagonal blocks also carry a low part)
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) {
          const int row = 16 * jt + ln;
#pragma unroll
          for (int kt = 0; kt <= (jt >> 1); ++kt) {
            const bf16x8 pf = *reinterpret_cast<const bf16x8*>(Ps + px(row, 32 * kt + 8 * g));
            ot[jt] = Mma<bf16>::run(vf[kt], pf, ot[jt]);
          }
          const int gd = g - 2 * (jt & 1);  // lane group inside the diagonal block
          bf16x8 lf = bf16x8{};
          if (gd == 0 || gd == 1) lf = *reinterpret_cast<const bf16x8*>(Ls + row * 16 + 8 * gd);
          ot[jt] = Mma<bf16>::run(vf[jt >> 1], lf, ot[jt]);
        }
        const int rv = min(C, L - n * C);
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) {
          const int row = 16 * jt + ln;
          if (row < rv)
            store4(o + ((size_t)bh * L + n * C + row) * dv + j0 + vc + 4 * g, ot[jt]);
        }
      }
      // S = diag(e^b) S + K~^T V
#pragma unroll
      for (int a = 0; a < NKT; ++a) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][r] *= gexp<T>(gv[r]);
      }
#pragma unroll
      for (int kt = 0; kt < C / 32; ++kt) {
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
          const int ra = 32 * kt + 8 * g + (ln >> 2), c = 16 * a + 4 * (ln & 3);
          const bf16x8 kf = join8(ds_read_tr(Ks + kx(ra, c)), ds_read_tr(Ks + kx(ra + 4, c)));
          S[a] = Mma<bf16>::run(kf, vf[kt], S[a]);
        }
      }
    } else {
      // fp32: 16x16x4 MFMAs; within each 16-token block b the MFMA i takes
      // tokens 16 b + 4 g + i (K index g)
      float vf[NRT][4];
#pragma unroll
      for (int bb = 0; bb < NRT; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[bb][i] = Vs[vx(16 * bb + 4 * g + i, vc + ln)];
      if constexpr (OUT) {
        floatx4 ot[NRT];
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) ot[jt] = zero4();
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
          for (int jt = 0; jt < NRT; ++jt) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Qs + qx(16 * jt + ln, 16 * a + 4 * g));
#pragma unroll
            for (int r = 0; r < 4; ++r) ot[jt] = Mma<float>::run(S[a][r], x[r], ot[jt]);
          }
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt)
#pragma unroll
          for (int bb = 0; bb <= jt; ++bb) {
            const f32x4 pf = *reinterpret_cast<const f32x4*>(Ps + px(16 * jt + ln, 16 * bb + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i) ot[jt] = Mma<float>::run(vf[bb][i], pf[i], ot[jt]);
          }
        const int rv = min(C, L - n * C);
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) {
          const int row = 16 * jt + ln;
          if (row < rv)
            store4(o + ((size_t)bh * L + n * C + row) * dv + j0 + vc + 4 * g, ot[jt]);
        }
      }
#pragma unroll
      for (int a = 0; a < NKT; ++a) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][r] *= gexp<T>(gv[r]);
      }
#pragma unroll
      for (int bb = 0; bb < NRT; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int a = 0; a < NKT; ++a)
            S[a] = Mma<float>::run(Ks[kx(16 * bb + 4 * g + i, 16 * a + ln)], vf[bb][i], S[a]);
    }
    if constexpr (!OUT) {
#pragma unroll
      for (int i = 0; i < NGS; ++i) {
        const int t = threadIdx.x + i * NTH;
        if (t < DK) gsum[i] += Gs[t];
      }
    }
    if (Lay::NBUF == 1) {
      __syncthreads();  // every wave is done with the buffer
      if (n + 1 < ne) issue(n + 1, 0);
    }
  }

  // ---- end of the segment
  float* dst = nullptr;
  if (OUT) dst = (NSEG == 1 && fin) ? fin + (size_t)bh * DK * dv : nullptr;
  else dst = fin + ((size_t)bh * NSEG + seg) * DK * dv;
  if (dst) {
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(a * 16 + 4 * g + r) * dv + col] = S[a][r];
  }
  if (!OUT && tile == 0) {
#pragma unroll
    for (int i = 0; i < NGS; ++i) {
      const int t = threadIdx.x + i * NTH;
      if (t < DK) seg_g[((size_t)bh * NSEG + seg) * DK + t] = gsum[i];
    }
  }
}

// =========================================================== launchers
template <typename T, int C>
static hipError_t launch_prep_t(const Plan& p, const void* q, const void* k, const float* la,
                                void* qg, void* kg, float* glog, void* ph, void* pl,
                                hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_prep<T, C>), dim3(p.NC, p.BH), dim3(kThreads), 0, s, (const T*)q,
                     (const T*)k, la, (T*)qg, (T*)kg, glog, (T*)ph, (T*)pl, p.L, p.dk, p.NC);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const Plan& p, const void* q, const void* k, const float* la,
                             void* qg, void* kg, float* glog, void* ph, void* pl, hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_prep_t<bf16, 64>(p, q, k, la, qg, kg, glog, ph, pl, s);
    return launch_prep_t<bf16, 32>(p, q, k, la, qg, kg, glog, ph, pl, s);
  }
  if (p.C == 64) return launch_prep_t<float, 64>(p, q, k, la, qg, kg, glog, ph, pl, s);
  if (p.C == 32) return launch_prep_t<float, 32>(p, q, k, la, qg, kg, glog, ph, pl, s);
  return launch_prep_t<float, 16>(p, q, k, la, qg, kg, glog, ph, pl, s);
}

template <typename T, int C, int DK, int NWV>
static hipError_t launch_recur_w(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* glog,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  const dim3 grid(p.BH * p.NSEGR * (p.dv / (16 * NWV)));
  if (out)
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 1>), grid, dim3(NWV * kWave), 0, s,
                       (const T*)qg, (const T*)kg, (const T*)ph, (const T*)pl, glog,
                       (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC, p.NSEGR,
                       p.segr_chunks);
  else
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 0>), grid, dim3(NWV * kWave), 0, s,
                       (const T*)qg, (const T*)kg, (const T*)ph, (const T*)pl, glog,
                       (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC, p.NSEGR,
                       p.segr_chunks);
  return hipGetLastError();
}

template <typename T, int C, int DK>
static hipError_t launch_recur_d(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* glog,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  if (p.NWVR == 4)
    return launch_recur_w<T, C, DK, 4>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  if (p.NWVR == 2)
    return launch_recur_w<T, C, DK, 2>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  if constexpr (recur_min_waves(sizeof(T) == 2, DK) == 1)
    return launch_recur_w<T, C, DK, 1>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  return hipErrorInvalidValue;
}

template <typename T, int C>
static hipError_t launch_recur_c(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* glog,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
#define GLA_RECUR_DK(D) \
  if (p.dk == D) return launch_recur_d<T, C, D>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s)
  if constexpr (sizeof(T) == 2) {
    GLA_RECUR_DK(32);
    GLA_RECUR_DK(64);
    GLA_RECUR_DK(128);
    GLA_RECUR_DK(256);
  } else {
    GLA_RECUR_DK(16);
    GLA_RECUR_DK(32);
    GLA_RECUR_DK(64);
    GLA_RECUR_DK(128);
  }
#undef GLA_RECUR_DK
  return hipErrorInvalidValue;
}

bool recur_supported(int bf16, int C, int dk, int dv) {
  const bool shape = bf16 ? (C == 32 || C == 64) && (dk == 32 || dk == 64 || dk == 128 || dk == 256)
                          : (C == 16 || C == 32 || C == 64) && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
  return shape && dv % (16 * recur_min_waves(bf16, dk)) == 0;
}

hipError_t launch_chunk_recur(const Plan& p, int out, const void* qg, const void* kg,
                              const void* ph, const void* pl, const float* glog, const void* v,
                              const float* init, void* o, float* fin, float* seg_g,
                              hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64)
      return launch_recur_c<bf16, 64>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
    return launch_recur_c<bf16, 32>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  }
  if (p.C == 64)
    return launch_recur_c<float, 64>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  if (p.C == 32)
    return launch_recur_c<float, 32>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
  return launch_recur_c<float, 16>(p, out, qg, kg, ph, pl, glog, v, init, o, fin, seg_g, s);
}

}  // namespace gla
