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
// The same through a buffer resource: 16 bytes at rsrc base + soff + voff
// (voff per lane, soff wave-uniform) into LDS at lds_wave_base + 16 * lane.
// The copy is issued from inline assembly: the instruction writes no
// register, and the compiler, which cannot tell which LDS bytes a copy
// writes, would otherwise wait for every outstanding copy (including the
// prefetch of a later chunk) before the next LDS read.  Completion is waited
// for explicitly (wait_vm) before a staged buffer is read.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 make_rsrc(const void* base) {
  // raw buffer: stride 0, range 2 GiB, 32-bit data format
  const unsigned long long a = (unsigned long long)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
  r[2] = 0x7fffffff;
  r[3] = 0x00020000;
  return r;
}
// lds_wave_base: LDS byte address (wave-uniform).  M0 carries it; no other
// code in the kernels that use this sets or reads M0.
__device__ inline void dma16b(const i32x4& r, unsigned voff, unsigned soff, unsigned lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(voff), "s"(r),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
// LDS byte address of a __shared__ object.
template <typename P>
__device__ inline unsigned lds_addr(P* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) void*)p;
}
// Wait until at most N of this wave's global memory operations are
// outstanding.  Loads complete in issue order, so in a wave that issues only
// loads this waits for all but the last N.
template <int N>
__device__ inline void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory"); }
// Wait for this wave's outstanding global memory operations (LDS copies too).
__device__ inline void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- fragment-blocked layouts ---------------------------------------------
// chunk_prep writes each chunk's Q~, K~, P (and P's diagonal low parts) as
// blocks of 16-byte units laid out the way the recurrence's MFMA operand
// reads want them, so that chunk_recur stages a chunk with contiguous
// 1 KB copies and reads every operand at a lane-constant LDS offset.  The
// unit orders below are involutions (applying one twice gives the identity),
// chosen so that each operand read is free of LDS bank conflicts (64 banks of
// 4 bytes; one 256-byte bank span per pass).
//
// Row block (Q~, P): 16 rows x 4 units.  A 16x16 MFMA operand read has lane
// (g, n) load unit g of row n; the 16 lanes of one g then cover 16 distinct
// units of a 256-byte span.
__device__ inline int row_slot(int n, int g) { return n * 4 + (g ^ ((n >> 2) & 3)); }
// Diagonal-block low part (bf16): 16 rows x 2 units (columns 0-7, 8-15).
__device__ inline int lo_slot(int n, int gd) { return n * 2 + (gd ^ ((n >> 3) & 1)); }
// Token-run block (bf16, transposed reads): 32 rows x UPR units.  A
// ds_read_b64_tr_b16 operand read touches rows 8 g + j (+ 4), j < 4, 32 bytes
// each; half a wave (g = 0, 1) then covers 8 distinct 32-byte windows.
template <int UPR>
__device__ inline int run_slot(int rho, int u) {
  int m;
  if constexpr (UPR == 2) m = ((rho >> 3) & 1) << 3;
  else if constexpr (UPR == 4) m = ((rho >> 3) & 1) << 1;
  else m = (((rho >> 1) & 1) | (((rho >> 3) & 1) << 1)) << 1;
  return (rho * UPR + u) ^ m;
}
// Scalar-read block (fp32): 16 rows x UPR units.  A 16x16x4 operand read has
// lane group g read row 4 g + i (fixed i), 64 bytes; the XOR puts the four
// rows in distinct 64-byte windows of a 256-byte span.
template <int UPR>
__device__ inline int scal_slot(int rho, int u) { return (rho * UPR + u) ^ (((rho >> 2) & 3) << 2); }

// Per-chunk record sizes (bytes).  GW: elements per 64-byte column group
// (one unit of 4 per row of a row block).
template <typename T>
struct RecDims {
  static constexpr int ES = (int)sizeof(T);
  static constexpr bool BF = ES == 2;
  static constexpr int EPU = 16 / ES;
  static constexpr int GW = 64 / ES;
  __host__ __device__ static constexpr int gbytes(int dk) { return ((8 * dk + 1023) / 1024) * 1024; }
};

constexpr int kLdsLimit = 160 * 1024;

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

// Issue copies [w, w + NWV, ...) < NCOPY of a contiguous tile: copy c moves the
// 1 KB at src + 1024 c into LDS at dst + 1024 c.
template <int NCOPY, int NWV>
__device__ inline void copy_tile(const unsigned char* src, unsigned dst, int w, int l) {
  const i32x4 r = make_rsrc(src);
  const unsigned loff = (unsigned)l * 16u;
#pragma unroll
  for (int i = 0; i < (NCOPY + NWV - 1) / NWV; ++i) {
    const int c = w + i * NWV;
    if (NCOPY % NWV != 0 && c >= NCOPY) break;
    dma16b(r, loff, (unsigned)c * 1024u, dst + (unsigned)c * 1024u);
  }
}

}  // namespace

// =========================================================== pass 1: chunk prep
// LDS per workgroup stays under a quarter of the CU's 160 KB and registers
// under 128 per lane, so that four workgroups (one wave per SIMD each) are
// resident per CU: the usual grid (one workgroup per chunk, a few per CU) then
// runs in a single round.
template <typename T, int C>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_chunk_prep(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ la,
    unsigned char* __restrict__ qrec, unsigned char* __restrict__ krec,
    unsigned char* __restrict__ prec, unsigned char* __restrict__ lrec,
    float* __restrict__ grec, int L, int dk, int NC) {
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
  const size_t cbase = io + (size_t)r0 * dk;
  const T* qc = q + cbase;
  const T* kc = k + cbase;
  const float* lc = la + cbase;
  const unsigned uoff = (unsigned)(urow * dk + uc8);
  const unsigned aoff = (unsigned)(rg * RPT * dk + ch);
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
    lds_barrier();  // previous slice's readers of qs, ks, bs, tot are done
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
    PB::gates(bs, als);
    pb.offdiag(qs, ks, bs);
    lds_barrier();
    pb.diag(qs, ks, als);
  }
  lds_barrier();  // the slice arrays are dead from here on
  pb.finish(pd, [&](int m, int r, float val) {
    const T hi = from_f32<T>(val);
    ps[m * C + r] = hi;
    if constexpr (BF) {
      if ((m >> 4) == (r >> 4)) ls[m * 16 + (r & 15)] = from_f32<T>(val - to_f32(hi));
    }
  });
  lds_barrier();
  // P as row blocks (jt, column group); unit g of a row = its EPU columns.
  // Entries above the diagonal were never written to ps: they are stored as
  // 0 here.
  constexpr int PUR = C / EPU, NPG = C / KS;
  unsigned char* pr = prec + cb * C * C * RD::ES;
  for (int it = tid; it < C * PUR; it += kThreads) {
    const int row = it / PUR, uu = it % PUR;
    store_masked<T>(pr + ((row >> 4) * NPG + (uu >> 2)) * 1024 + row_slot(row & 15, uu & 3) * 16,
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

// =========================================================== pass 2: recurrence
template <typename T, int C, int DK, int NWV, int OUT>
struct RecurLayout {
  using RD = RecDims<T>;
  static constexpr int ES = RD::ES;
  static constexpr bool BF = RD::BF;
  static constexpr int DVT = 16 * NWV;          // d_v tile: 16 columns per wave
  static constexpr int NG = DK / RD::GW;        // column groups of a Q~ / K~ row
  static constexpr int NPG = C / RD::GW;        // column groups of a P row
  static constexpr int VUPR = DVT * ES / 16;    // units per V row
  static constexpr int QB = OUT ? C * DK * ES : 0;
  static constexpr int KB = C * DK * ES;
  static constexpr int PB = OUT ? C * C * ES : 0;
  static constexpr int LB = (OUT && BF) ? C * 16 * ES : 0;
  static constexpr int GB = RD::gbytes(DK);
  static constexpr int VB = C * DVT * ES;
  static constexpr int VBLK = BF ? 32 * VUPR * 16 : 16 * VUPR * 16;  // bytes per V block
  static constexpr int oQ = 0, oK = oQ + QB, oP = oK + KB, oL = oP + PB, oG = oL + LB,
                       oV = oG + GB, BUF = oV + VB;
  static constexpr int VCOPY = VB / 1024;       // V copies per chunk
  static constexpr int CPC = BUF / 1024;        // copies per chunk
  // Staging buffers: three (copies run two chunks ahead) when they fit and
  // a chunk's copy count fits the 6-bit vmcnt field, else two, else one.
  static constexpr int NBUF = (CPC <= 63 && 3 * BUF <= kLdsLimit) ? 3 : (2 * BUF <= kLdsLimit ? 2 : 1);
  static_assert(QB % 1024 == 0 && KB % 1024 == 0 && PB % 1024 == 0 && LB % 1024 == 0 &&
                    VB % 1024 == 0,
                "every staged tile is a whole number of 1 KB copies");
  static_assert(BUF <= kLdsLimit, "staged chunk exceeds LDS");
};

// Waves 0 .. NWV-1 compute (16 state columns each); wave NWV only issues the
// LDS copies and waits for them, so that its memory counter holds nothing but
// loads (a partial wait is exact) and the computing waves, which store the
// output, never wait on memory.
template <typename T, int C, int DK, int NWV, int OUT>
__global__ __launch_bounds__((NWV + 1) * kWave) void k_chunk_recur(
    const unsigned char* __restrict__ qrec, const unsigned char* __restrict__ krec,
    const unsigned char* __restrict__ prec, const unsigned char* __restrict__ lrec,
    const float* __restrict__ grec, const T* __restrict__ v, const float* __restrict__ init,
    T* __restrict__ o, float* __restrict__ fin, float* __restrict__ seg_g, int L, int dv, int NC,
    int NSEG, int seg_chunks) {
  using Lay = RecurLayout<T, C, DK, NWV, OUT>;
  constexpr bool BF = Lay::BF;
  constexpr int ES = Lay::ES, DVT = Lay::DVT, NTH = NWV * kWave, VUPR = Lay::VUPR;
  constexpr int NRT = C / 16, NKT = DK / 16, NG = Lay::NG, NPG = Lay::NPG;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Lay::NBUF * Lay::BUF];

  const int ntv = dv / DVT;
  const int lid = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lid % ntv, seg = (lid / ntv) % NSEG, bh = lid / (ntv * NSEG);
  const int j0 = tile * DVT;
  // the wave index as a scalar: copy and column offsets derived from it stay
  // in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const bool loader = w == NWV;
  const int l = lane_id(), g = l >> 4, ln = l & 15;
  const int vc = 16 * (loader ? 0 : w);  // this wave's first column within the tile
  const int col = j0 + vc + ln;          // this lane's state column
  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);

  // ---- state slice: lane holds S[16 a + 4 g + r][col]
  floatx4 S[NKT];
  {
    const float* src = nullptr;
    if (OUT && !loader) src = NSEG > 1 ? init + ((size_t)bh * NSEG + seg) * DK * dv
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

  // ---- V copies: the tile row and 16-byte unit that lane l's slot of copy c
  // holds
  auto vslot = [&](int c, int& rho, int& u) __attribute__((always_inline)) {
    const int s = c * 64 + l;
    if constexpr (BF) {
      const int blk = s / (32 * VUPR);
      const int lg = run_slot<VUPR>((s % (32 * VUPR)) / VUPR, s % VUPR);
      rho = blk * 32 + lg / VUPR;
      u = lg % VUPR;
    } else {
      const int blk = s / (16 * VUPR);
      const int lg = scal_slot<VUPR>((s % (16 * VUPR)) / VUPR, s % VUPR);
      rho = blk * 16 + lg / VUPR;
      u = lg % VUPR;
    }
  };

  const unsigned lds0 = lds_addr(lds);
  // Stage chunk n into buffer b (the loading wave only).
  auto issue = [&](int n, int b) __attribute__((always_inline)) {
    const unsigned base = lds0 + (unsigned)(b * Lay::BUF);
    const size_t cb = (size_t)bh * NC + n;
    if constexpr (OUT) {
      copy_tile<Lay::QB / 1024, 1>(qrec + cb * Lay::QB, base + Lay::oQ, 0, l);
      copy_tile<Lay::PB / 1024, 1>(prec + cb * Lay::PB, base + Lay::oP, 0, l);
      if constexpr (BF) copy_tile<Lay::LB / 1024, 1>(lrec + cb * Lay::LB, base + Lay::oL, 0, l);
    }
    copy_tile<Lay::KB / 1024, 1>(krec + cb * Lay::KB, base + Lay::oK, 0, l);
    copy_tile<Lay::GB / 1024, 1>(reinterpret_cast<const unsigned char*>(grec) + cb * Lay::GB,
                                 base + Lay::oG, 0, l);
    // V rows past the end of the sequence repeat the last row (their K~ rows
    // and P columns are zero)
    const int r0 = n * C;
    const i32x4 vr = make_rsrc(v + ((size_t)bh * L + r0) * dv + j0);
    const bool full = r0 + C <= L;
#pragma unroll
    for (int c = 0; c < Lay::VCOPY; ++c) {
      int rho, u;
      vslot(c, rho, u);
      if (!full) rho = min(rho, L - 1 - r0);
      dma16b(vr, (unsigned)(rho * dv * ES + u * 16), 0u, base + (unsigned)(Lay::oV + c * 1024));
    }
  };

  // ---- lane-constant LDS offsets of the operand reads
  const int qoff = row_slot(ln, g) * 16;                  // Q~ and P row blocks
  const int loff = lo_slot(ln, g & 1) * 16;               // P low part, lanes g = 2 (jt & 1) + gd
  int voff[2], koff[2][2], vsoff[4], ksoff[4];
  if constexpr (BF) {
    const int rho = 8 * g + (ln >> 2), half = (ln & 1) * 8, ub = (ln & 3) >> 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      voff[h] = run_slot<VUPR>(rho + 4 * h, 2 * w + ub) * 16 + half;
#pragma unroll
      for (int ap = 0; ap < 2; ++ap) koff[ap][h] = run_slot<4>(rho + 4 * h, 2 * ap + ub) * 16 + half;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vsoff[i] = scal_slot<VUPR>(4 * g + i, 4 * w + (ln >> 2)) * 16 + (ln & 3) * 4;
      ksoff[i] = scal_slot<4>(4 * g + i, ln >> 2) * 16 + (ln & 3) * 4;
    }
  }

  // One chunk from buffer b: O^T of the chunk into ot (stored by the caller
  // once the next copies are issued), then the state update.
  auto body = [&](int n, int b, floatx4 (&ot)[NRT]) __attribute__((always_inline)) {
    const unsigned char* base = lds + b * Lay::BUF;
    const unsigned char* Qs = base + Lay::oQ;
    const unsigned char* Ks = base + Lay::oK;
    const unsigned char* Ps = base + Lay::oP;
    const unsigned char* Ls = base + Lay::oL;
    const float* Gs = reinterpret_cast<const float*>(base + Lay::oG);
    const unsigned char* Vs = base + Lay::oV;
    if constexpr (BF) {
      // V fragments over token runs 32 kt + 8 g + e at column vc + ln
      bf16x8 vf[C / 32];
#pragma unroll
      for (int kt = 0; kt < C / 32; ++kt) {
        const bf16* vb = reinterpret_cast<const bf16*>(Vs + kt * Lay::VBLK);
        vf[kt] = join8(ds_read_tr(reinterpret_cast<const bf16*>(reinterpret_cast<const unsigned char*>(vb) + voff[0])),
                       ds_read_tr(reinterpret_cast<const bf16*>(reinterpret_cast<const unsigned char*>(vb) + voff[1])));
      }
      if constexpr (OUT) {
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) ot[jt] = zero4();
        // O^T += S^T Q~^T over pairs of 16-channel tiles; the MFMA's K index
        // 8 g + e maps to channel 32 a2 + 4 g + e (e < 4) or + 16 + 4 g + e - 4
        // (the order of the Q~ units)
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
            const bf16x8 B = *reinterpret_cast<const bf16x8*>(Qs + (jt * NG + a2) * 1024 + qoff);
            ot[jt] = Mma<bf16>::run(A, B, ot[jt]);
          }
        }
        // O^T += V^T P^T (P rounded; its diagonal blocks also carry a low part)
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) {
#pragma unroll
          for (int kt = 0; kt <= (jt >> 1); ++kt) {
            const bf16x8 pf = *reinterpret_cast<const bf16x8*>(Ps + (jt * NPG + kt) * 1024 + qoff);
            ot[jt] = Mma<bf16>::run(vf[kt], pf, ot[jt]);
          }
          // every lane reads (a branch would force a wait for the read), the
          // lanes whose K range is not this block's diagonal drop the value
          bf16x8 lf = *reinterpret_cast<const bf16x8*>(Ls + jt * 512 + loff);
          if ((g >> 1) != (jt & 1)) lf = bf16x8{};
          ot[jt] = Mma<bf16>::run(vf[jt >> 1], lf, ot[jt]);
        }
      }
      // S = diag(e^b) S + K~^T V
#pragma unroll
      for (int a = 0; a < NKT; ++a) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][r] *= gv[r];
      }
#pragma unroll
      for (int kt = 0; kt < C / 32; ++kt) {
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
          const unsigned char* kb = Ks + (kt * NG + (a >> 1)) * 2048;
          const bf16x8 kf = join8(ds_read_tr(reinterpret_cast<const bf16*>(kb + koff[a & 1][0])),
                                  ds_read_tr(reinterpret_cast<const bf16*>(kb + koff[a & 1][1])));
          S[a] = Mma<bf16>::run(kf, vf[kt], S[a]);
        }
      }
    } else {
      // fp32: 16x16x4 MFMAs; within each 16-token block bb the MFMA i takes
      // tokens 16 bb + 4 g + i (K index g)
      float vf[NRT][4];
#pragma unroll
      for (int bb = 0; bb < NRT; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vf[bb][i] = *reinterpret_cast<const float*>(Vs + bb * Lay::VBLK + vsoff[i]);
      if constexpr (OUT) {
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) ot[jt] = zero4();
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
          for (int jt = 0; jt < NRT; ++jt) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Qs + (jt * NG + a) * 1024 + qoff);
#pragma unroll
            for (int r = 0; r < 4; ++r) ot[jt] = Mma<float>::run(S[a][r], x[r], ot[jt]);
          }
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt)
#pragma unroll
          for (int bb = 0; bb <= jt; ++bb) {
            const f32x4 pf = *reinterpret_cast<const f32x4*>(Ps + (jt * NPG + bb) * 1024 + qoff);
#pragma unroll
            for (int i = 0; i < 4; ++i) ot[jt] = Mma<float>::run(vf[bb][i], pf[i], ot[jt]);
          }
      }
#pragma unroll
      for (int a = 0; a < NKT; ++a) {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][r] *= gv[r];
      }
#pragma unroll
      for (int bb = 0; bb < NRT; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int a = 0; a < NKT; ++a) {
            const float kv = *reinterpret_cast<const float*>(Ks + (bb * NG + a) * 1024 + ksoff[i]);
            S[a] = Mma<float>::run(kv, vf[bb][i], S[a]);
          }
    }
    if constexpr (!OUT) {
#pragma unroll
      for (int i = 0; i < NGS; ++i) {
        const int t = threadIdx.x + i * NTH;
        if (t < DK) gsum[i] += Gs[DK + t];
      }
    }
  };

  auto store_out = [&](int n, const floatx4 (&ot)[NRT]) __attribute__((always_inline)) {
    if constexpr (OUT) {
      const int rv = min(C, L - n * C);
      T* orow = o + ((size_t)bh * L + n * C + ln) * dv + j0 + vc + 4 * g;
#pragma unroll
      for (int jt = 0; jt < NRT; ++jt)
        if (16 * jt + ln < rv) store4(orow + (size_t)16 * jt * dv, ot[jt]);
    }
  };

  // ---- walk the segment's chunks.  Chunk n + D (D = NBUF - 1) is staged into
  // the buffer that chunk n - 1 used while chunk n computes; before the
  // chunk's closing barrier the loading wave waits until chunk n + 1 has
  // landed (with D = 2 the copies of chunk n + 2 may still be in flight).
  // The computing waves store each chunk's output as soon as it is computed.
  // Buffer indices are literals at every step call.
  constexpr int D = Lay::NBUF - 1;
  // ot: the chunk being computed; op: the previous chunk's output, stored
  // after the next chunk's products are issued so that the stores never wait
  // for the matrix pipeline
  floatx4 ot[NRT], op[NRT];
  int pn = -1;
  auto store_prev = [&]() __attribute__((always_inline)) {
    if (pn >= 0) store_out(pn, op);
  };
  auto keep = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int jt = 0; jt < NRT; ++jt) op[jt] = ot[jt];
    pn = n;
  };
  auto wait_through = [&](int m) __attribute__((always_inline)) {  // chunk m landed
    if constexpr (D == 2) {
      if (m + 1 < ne) wait_vm_le<Lay::CPC>();
      else wait_vm();
    } else {
      wait_vm();
    }
  };
  auto step = [&](int n, int b) __attribute__((always_inline)) {
    if constexpr (D > 0) {
      if (loader) {
        if (n + D < ne) issue(n + D, (b + D) % Lay::NBUF);
        if (n + 1 < ne) wait_through(n + 1);
      } else {
        body(n, b, ot);
        store_prev();
        keep(n);
      }
      lds_barrier();  // chunk n + 1 staged; everyone is done with buffer b
    } else {
      if (!loader) {
        body(n, 0, ot);
        store_prev();
        keep(n);
      }
      lds_barrier();  // everyone is done with the buffer
      if (loader && n + 1 < ne) {
        issue(n + 1, 0);
        wait_vm();
      }
      lds_barrier();  // chunk n + 1 staged
    }
  };

  if (nb < ne) {
    if (loader) {
#pragma unroll
      for (int i = 0; i < (D > 0 ? D : 1); ++i)
        if (nb + i < ne) issue(nb + i, i);
      wait_through(nb);
    }
    lds_barrier();  // chunk nb staged
  }
  for (int n = nb; n < ne; n += Lay::NBUF) {
    step(n, 0);
    if constexpr (Lay::NBUF >= 2) {
      if (n + 1 < ne) step(n + 1, 1);
    }
    if constexpr (Lay::NBUF == 3) {
      if (n + 2 < ne) step(n + 2, 2);
    }
  }

  if (!loader) store_prev();

  // ---- end of the segment
  float* dst = nullptr;
  if (OUT) dst = (NSEG == 1 && fin) ? fin + (size_t)bh * DK * dv : nullptr;
  else dst = fin + ((size_t)bh * NSEG + seg) * DK * dv;
  if (dst && !loader) {
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(a * 16 + 4 * g + r) * dv + col] = S[a][r];
  }
  if (!OUT && tile == 0 && !loader) {
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
                                void* qg, void* kg, float* grec, void* ph, void* pl,
                                hipStream_t s) {
  hipLaunchKernelGGL((k_chunk_prep<T, C>), dim3(p.NC, p.BH), dim3(kThreads), 0, s, (const T*)q,
                     (const T*)k, la, (unsigned char*)qg, (unsigned char*)kg, (unsigned char*)ph,
                     (unsigned char*)pl, grec, p.L, p.dk, p.NC);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(const Plan& p, const void* q, const void* k, const float* la,
                             void* qg, void* kg, float* grec, void* ph, void* pl, hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64) return launch_prep_t<bf16, 64>(p, q, k, la, qg, kg, grec, ph, pl, s);
    return launch_prep_t<bf16, 32>(p, q, k, la, qg, kg, grec, ph, pl, s);
  }
  if (p.C == 64) return launch_prep_t<float, 64>(p, q, k, la, qg, kg, grec, ph, pl, s);
  if (p.C == 32) return launch_prep_t<float, 32>(p, q, k, la, qg, kg, grec, ph, pl, s);
  return launch_prep_t<float, 16>(p, q, k, la, qg, kg, grec, ph, pl, s);
}

template <typename T, int C, int DK, int NWV>
static hipError_t launch_recur_w(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* grec,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  const dim3 grid(p.BH * p.NSEGR * (p.dv / (16 * NWV)));
  const unsigned char *q8 = (const unsigned char*)qg, *k8 = (const unsigned char*)kg,
                      *p8 = (const unsigned char*)ph, *l8 = (const unsigned char*)pl;
  if (out)
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 1>), grid, dim3((NWV + 1) * kWave), 0, s, q8, k8,
                       p8, l8, grec, (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC,
                       p.NSEGR, p.segr_chunks);
  else
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 0>), grid, dim3((NWV + 1) * kWave), 0, s, q8, k8,
                       p8, l8, grec, (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC,
                       p.NSEGR, p.segr_chunks);
  return hipGetLastError();
}

template <typename T, int C, int DK>
static hipError_t launch_recur_d(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* grec,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  if (p.NWVR == 4)
    return launch_recur_w<T, C, DK, 4>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  if (p.NWVR == 2)
    return launch_recur_w<T, C, DK, 2>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  if constexpr (recur_min_waves(sizeof(T) == 2, DK) == 1)
    return launch_recur_w<T, C, DK, 1>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  return hipErrorInvalidValue;
}

template <typename T, int C>
static hipError_t launch_recur_c(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* grec,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
#define GLA_RECUR_DK(D) \
  if (p.dk == D) return launch_recur_d<T, C, D>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s)
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

size_t recur_grec_bytes(int dk) { return RecDims<float>::gbytes(dk); }

bool recur_supported(int bf16, int C, int dk, int dv) {
  const bool shape = bf16 ? (C == 32 || C == 64) && (dk == 32 || dk == 64 || dk == 128 || dk == 256)
                          : (C == 16 || C == 32 || C == 64) && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
  return shape && dv % (16 * recur_min_waves(bf16, dk)) == 0;
}

hipError_t launch_chunk_recur(const Plan& p, int out, const void* qg, const void* kg,
                              const void* ph, const void* pl, const float* grec, const void* v,
                              const float* init, void* o, float* fin, float* seg_g,
                              hipStream_t s) {
  if (p.bf16) {
    if (p.C == 64)
      return launch_recur_c<bf16, 64>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
    return launch_recur_c<bf16, 32>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  }
  if (p.C == 64)
    return launch_recur_c<float, 64>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  if (p.C == 32)
    return launch_recur_c<float, 32>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  return launch_recur_c<float, 16>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
}

}  // namespace gla
