// gla_prep.hip -- pass 1 of the two-pass forward of the GLA chunkwise layer
// (gfx950).
//
// k_chunk_prep: one workgroup per (batch-head, chunk), all chunks in
// parallel (it also prefetches the chunk's V rows for pass 2).  From q, k and
// log alpha of the chunk it forms
//   B      = chunk-local inclusive cumsum of log alpha  (per key channel)
//   Q~     = Q ⊙ e^{B}            (rows of the chunk, I/O type)
//   K~     = K ⊙ e^{b - B}        (b = B at the chunk's last row)
//   b      = the chunk's total log decay
//   P      = the causal gated score matrix of the chunk (gla_pblock.h):
//            P[m][r] = sum_k q_mk k_rk e^{B_mk - B_rk}, r <= m
// (papercache.org notes §4.2 chunkwise form with Lambda, Gamma, gamma; §4.3 /
// Figure 3 for P).  For bf16 I/O, P is stored rounded to bf16 plus the low
// part of its diagonal 16 x 16 blocks.  The records' layouts are those of
// gla_records.h; pass 2 is gla_recur.hip.
#include "gla_common.h"
#include "gla_dma.h"
#include "gla_internal.h"
#include "gla_pblock.h"
#include "gla_records.h"

namespace gla {

namespace {

// Store one 16-byte unit of EPU values rounded to T.
template <typename T> __device__ inline void store_unit(unsigned char* p, const float* x);
template <> __device__ inline void store_unit<bf16>(unsigned char* p, const float* x) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<bf16x8*>(p) = a;
}
template <> __device__ inline void store_unit<float>(unsigned char* p, const float* x) {
  f32x4 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = x[e];
  *reinterpret_cast<f32x4*>(p) = a;
}

// Copy one 16-byte unit of T from LDS to global memory, with element e
// replaced by 0 where e > last (last < 0: all zero, without reading).
template <typename T>
__device__ inline void store_masked(unsigned char* dst, const T* src, int last) {
  constexpr int EPU = 16 / (int)sizeof(T);
  f32x4 val = f32x4{};
  if (last >= 0) {
    val = *reinterpret_cast<const f32x4*>(src);
    if (last < EPU - 1) {
      T* e = reinterpret_cast<T*>(&val);
#pragma unroll
      for (int i = 0; i < EPU; ++i)
        if (i > last) e[i] = from_f32<T>(0.f);
    }
  }
  *reinterpret_cast<f32x4*>(dst) = val;
}

}  // namespace

// =========================================================== pass 1: chunk prep
// LDS per workgroup stays under a quarter of the CU's 160 KB and registers
// under 128 per lane, so that four workgroups (one wave per SIMD each) are
// resident per CU: the usual grid (one workgroup per chunk, a few per CU) then
// runs in a single round.
//
// REV: the time-reversed sequence, the dv pass of the backward.  Row p of the
// reversed sequence is original row L - 1 - p of q, k and v, and its log gate
// is the next original token's, log alpha[L - p] (0 at p = 0): the gradient
// flows from a token to the tokens before it, decayed by the gates after
// them.  Everything else (records, chunk numbering) refers to the reversed
// sequence.
template <typename T, int C, bool REV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(REV ? 3 : 4))) void k_chunk_prep(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ la,
    const T* __restrict__ v, unsigned char* __restrict__ qrec, unsigned char* __restrict__ krec,
    unsigned char* __restrict__ prec, unsigned char* __restrict__ lrec,
    float* __restrict__ grec, int L, int dk, int dv, int NC) {
  // q, k slices staged in fp32: the diagonal blocks' vector-ALU reads and the
  // scaled MFMA operands then need no conversion
  using PB = PBuilder<T, C, 4, float>;
  using RD = RecDims<T>;
  constexpr bool BF = PB::BF;
  constexpr int KS = PB::KS, LDT = PB::LDT, LDF = PB::LDF;
  constexpr int EPU = RD::EPU;
  static_assert(KS == RD::GW, "one d_k slice is one column group");
  constexpr int RG = kThreads / KS;  // row groups of the slice cumsum
  constexpr int RPT = C / RG;        // rows per thread
  static_assert(RPT >= 1 && C % RG == 0, "cumsum row split");
  // The slice arrays (qs, ks, bs, als) are dead after the last slice; the
  // P staging (ps), the diagonal low parts (ls) and the diagonal partial sums
  // (pd) then reuse their space.
  constexpr int PS_BYTES = C * C * (int)sizeof(T);
  constexpr int LS_BYTES = BF ? C * 16 * (int)sizeof(T) : 0;
  constexpr int PD_BYTES = 4 * 16 * 17 * 4;
  constexpr int TAIL_BYTES = PS_BYTES + LS_BYTES + PD_BYTES;
  constexpr int SMEM_BYTES = PB::SLICE_BYTES > TAIL_BYTES ? PB::SLICE_BYTES : TAIL_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM_BYTES];
  __shared__ float tot[RG][KS];
  __shared__ __attribute__((aligned(16))) unsigned char vtouch[256];
  float* qs = reinterpret_cast<float*>(smem);
  float* ks = qs + C * LDT;
  float* bs = ks + C * LDT;
  float* als = bs + C * LDF;
  T* ps = reinterpret_cast<T*>(smem);
  T* ls = reinterpret_cast<T*>(smem + PS_BYTES);
  auto pd = reinterpret_cast<float(*)[16][17]>(smem + PS_BYTES + LS_BYTES);

  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r0 = n * C, rv = min(C, L - r0);
  const int NG = dk / KS;                                     // column groups per row
  const size_t io = (size_t)bh * L * dk;                      // q, k, log alpha
  const size_t cb = (size_t)bh * NC + n;                      // chunk id
  unsigned char* qr = qrec + cb * C * dk * RD::ES;
  unsigned char* kr = krec + cb * C * dk * RD::ES;
  float* gr = grec + cb * (RD::gbytes(dk) / 4);

  // The recurrence pass reads this chunk's V rows next: bring them from HBM
  // into the caches (the memory-side cache keeps them until then), 8 KB per
  // wave and touch.  Issued in the last slice, when this workgroup's input
  // fetches are done (at the kernel's start they would compete with them),
  // and waited for at the end of the slice loop.
  auto touch_v = [&]() __attribute__((always_inline)) {
    const int vbytes = rv * dv * (int)sizeof(T);
    const size_t vr0 = REV ? (size_t)(L - r0 - rv) : (size_t)r0;  // first row in memory
    const unsigned char* vrow = reinterpret_cast<const unsigned char*>(v + ((size_t)bh * L + vr0) * dv);
    const unsigned dmy = (unsigned)(size_t)(__attribute__((address_space(3))) void*)vtouch;
    for (int p0 = wave_id() * 8192; p0 < vbytes; p0 += (kThreads / kWave) * 8192)
      touch_lines(vrow + p0, min(8192, vbytes - p0), lane_id(), dmy);
  };

  PB pb;
  pb.init();
  const int ch = tid % KS, rg = tid / KS;
  // The next slice's q, k (one 8-element unit each per thread) and log alpha
  // (RPT rows of one channel per thread) are loaded into registers while the
  // current slice is processed.  Rows past the end of the sequence read as 0.
  constexpr int NU = C * (KS / 8);
  static_assert(NU <= kThreads, "one q / k unit per thread");
  const int urow = tid / (KS / 8), uc8 = (tid % (KS / 8)) * 8;
  const bool uld = tid < NU && urow < rv;
  // chunk-uniform bases and 32-bit per-thread offsets (one address register
  // per lane instead of a 64-bit pointer per load)
  // The chunk's rows in memory start at row r0, or (reversed sequence) at
  // row L - r0 - rv, whose rows then run backwards: chunk row p is memory row
  // rv - 1 - p from there, and its log gate memory row rv - p.
  const size_t cbase = io + (size_t)(REV ? L - r0 - rv : r0) * dk;
  const T* qc = q + cbase;
  const T* kc = k + cbase;
  const float* lc = la + cbase;
  const unsigned uoff = (unsigned)((REV ? rv - 1 - urow : urow) * dk + uc8);
  const unsigned aoff = (unsigned)((REV ? rv - rg * RPT : rg * RPT) * dk + ch);
  Raw8<T> rq, rk;
  float ra[RPT];
  auto fetch = [&](int grp) __attribute__((always_inline)) {
    const unsigned s0 = (unsigned)(grp * KS);
    if (uld) {
      raw_load(rq, qc + (uoff + s0));
      raw_load(rk, kc + (uoff + s0));
    } else {
      raw_zero(rq);
      raw_zero(rk);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      if constexpr (REV)  // the first row of the reversed sequence has no gate
        ra[i] = (row < rv && r0 + row > 0) ? lc[aoff - (unsigned)(i * dk) + s0] : 0.f;
      else
        ra[i] = row < rv ? lc[aoff + (unsigned)(i * dk) + s0] : 0.f;
    }
  };
  fetch(0);
  for (int grp = 0; grp < NG; ++grp) {
    const int s0 = grp * KS;
    const Raw8<T> cq = rq, ck = rk;
    float av[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) av[i] = ra[i];
    if (grp + 1 < NG) fetch(grp + 1);
    if (grp == NG - 1) touch_v();
    lds_barrier();  // previous slice's readers of qs, ks, bs, als, tot are done
    if (tid < NU) {
      float qv[8], kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] = raw_get(cq, e);
        kv[e] = raw_get(ck, e);
      }
      store8(qs + urow * LDT + uc8, qv);
      store8(ks + urow * LDT + uc8, kv);
    }
    // per-row gates alpha = e^{log alpha} (1 at a sub-chunk's first row, where
    // the diagonal blocks never use it), from the log gates in registers
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      als[row * LDF + ch] = (row & 15) ? gexp<T>(av[i]) : 1.f;
    }
    // chunk-local cumsum: RPT rows per thread, then the preceding groups' totals
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      run += av[i];
      av[i] = run;
    }
    tot[rg][ch] = run;
    lds_barrier();
    float off = 0.f;
    for (int g = 0; g < rg; ++g) off += tot[g][ch];
#pragma unroll
    for (int i = 0; i < RPT; ++i) bs[(rg * RPT + i) * LDF + ch] = av[i] + off;
    lds_barrier();
    // Q~ = Q ⊙ e^B and K~ = K ⊙ e^{b - B}, one 16-byte unit per thread each.
    // Q~ unit g of a row holds (bf16) columns 4g..4g+3 and 16+4g..16+4g+3 of
    // the group, the channels of the state rows that lane group g holds in
    // its accumulators; (fp32) columns 4g..4g+3.
    for (int it = tid; it < C * 4; it += kThreads) {
      const int row = it >> 2, g = it & 3;
      float x[EPU];
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const int c = BF ? (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4) : 4 * g + e;
        x[e] = to_f32(qs[row * LDT + c]) * gexp<T>(bs[row * LDF + c]);
      }
      store_unit<T>(qr + (((row >> 4) * NG + grp) * 1024 + row_slot(row & 15, g) * 16), x);
      // K~: unit u = columns EPU u .. EPU u + EPU - 1
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const int c = EPU * g + e;
        x[e] = to_f32(ks[row * LDT + c]) * gexp<T>(bs[(C - 1) * LDF + c] - bs[row * LDF + c]);
      }
      int kofs;
      if constexpr (BF) kofs = ((row >> 5) * NG + grp) * 2048 + run_slot<4>(row & 31, g) * 16;
      else kofs = ((row >> 4) * NG + grp) * 1024 + scal_slot<4>(row & 15, g) * 16;
      store_unit<T>(kr + kofs, x);
    }
    if (tid < KS) {
      const float b = bs[(C - 1) * LDF + tid];
      gr[s0 + tid] = gexp<T>(b);  // the chunk's decay of state row s0 + tid
      gr[dk + s0 + tid] = b;      // and its log
    }
    // both read only what the two barriers above published
    pb.offdiag(qs, ks, bs);
    pb.diag(qs, ks, als);
  }
  // no touch may be in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();  // the slice arrays are dead from here on
  pb.finish(pd, [&](int m, int r, float val) {
    const T hi = from_f32<T>(val);
    ps[m * C + r] = hi;
    if constexpr (BF) {
      if ((m >> 4) == (r >> 4)) ls[m * 16 + (r & 15)] = from_f32<T>(val - to_f32(hi));
    }
  });
  lds_barrier();
  // P as row blocks (jt, column group), the groups wholly above the
  // diagonal left out (RecDims::pblock); unit g of a row = its EPU columns.
  // Entries above the diagonal were never written to ps: they are stored as
  // 0 here.
  constexpr int PUR = C / EPU;
  unsigned char* pr = prec + cb * RD::pblocks(C) * 1024;
  for (int it = tid; it < C * PUR; it += kThreads) {
    const int row = it / PUR, uu = it % PUR, jt = row >> 4, cg = uu >> 2;
    if (cg > RD::plast(jt)) continue;
    store_masked<T>(pr + RD::pblock(jt, cg) * 1024 + row_slot(row & 15, uu & 3) * 16,
                    &ps[row * C + uu * EPU], row - uu * EPU);
  }
  if constexpr (BF) {
    unsigned char* lr = lrec + cb * C * 16 * RD::ES;
    for (int it = tid; it < C * 2; it += kThreads) {
      const int row = it >> 1, gd = it & 1;
      store_masked<T>(lr + (row >> 4) * 512 + lo_slot(row & 15, gd) * 16,
                      &ls[row * 16 + 8 * gd], (row & 15) - 8 * gd);
    }
  }
}

// =========================================================== launcher
template <typename T, int C, bool REV = false>
static hipError_t launch_prep_t(const Plan& p, const void* q, const void* k, const float* la,
                                const void* v, void* qg, void* kg, float* grec, void* ph,
                                void* pl, hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_prep<T, C, REV>), dim3(p.NC, p.BH), dim3(kThreads), 0, s,
                     (const T*)q, (const T*)k, la, (const T*)v, (unsigned char*)qg,
                     (unsigned char*)kg, (unsigned char*)ph, (unsigned char*)pl, grec, p.L, p.dk,
                     p.dv, p.NC);
  return hipGetLastError();
}

hipError_t launch_chunk_prep_rev(const Plan& p, const void* q, const void* k, const float* la,
                                 const void* v, void* qg, void* kg, float* grec, void* ph,
                                 void* pl, hipStream_t s) {
  if (!p.bf16 || p.C != 64) return hipErrorInvalidValue;
  return launch_prep_t<bf16, 64, true>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
}

hipError_t launch_chunk_prep(const Plan& p, const void* q, const void* k, const float* la,
                             const void* v, void* qg, void* kg, float* grec, void* ph, void* pl,
                             hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_prep_t<bf16, 64>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
    return launch_prep_t<bf16, 32>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
  }
  if (p.C == 64) return launch_prep_t<float, 64>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
  if (p.C == 32) return launch_prep_t<float, 32>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
  return launch_prep_t<float, 16>(p, q, k, la, v, qg, kg, grec, ph, pl, s);
}

}  // namespace gla
