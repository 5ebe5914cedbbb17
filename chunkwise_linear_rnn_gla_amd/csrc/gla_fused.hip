// gla_fused.hip -- fused segment forward of the GLA chunkwise layer (gfx950).
//
// One workgroup (8 waves) owns one (batch-head, sequence segment, d_v tile).
// It starts from the state entering its segment (h0, or the scan of the
// segments' local states) and walks the segment's chunks in order, keeping
// the d_k x d_v state tile in MFMA accumulators (fp32) the whole time:
//   O[n]^T = S_{n-1}^T (Q ⊙ Lambda)^T + V^T P^T          (output, transposed)
//   S_n    = diag(e^{b_n}) S_{n-1} + (K ⊙ Gamma)^T V      (state)
// (papercache.org notes §4.2 chunkwise form; §3.3 / Figure 1a keeps the state
// on chip across chunks; P is the chunk's gated score matrix of §4.3 /
// Figure 3, built by gla_pblock.h).  Per-chunk states never go to memory.
//
// The state tile feeds the next product directly: the fp32 accumulator of a
// 16x16 MFMA holds S[4g + r][n] in lane n + 16 g, which is exactly the A
// operand layout of a 16x16x16 bf16 MFMA computing S^T (Q ⊙ Lambda)^T (and of
// four 16x16x4 fp32 MFMAs on the fp32 path), so no exchange is needed.
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"

namespace gla {

namespace {

// Waves per workgroup: 8 (two per SIMD) for state tiles of up to 64K
// entries; the 128 x 256 and 256 x 128 tiles take 4 waves so that each wave
// may hold its larger share of the tile (up to 512 registers per lane).
constexpr int fused_waves(int DK, int DVT) { return DK * DVT >= 128 * 256 ? 4 : 8; }

// o^T tile += S^T tile x (Q ⊙ Lambda)^T tile over one 16-deep d_k tile.
// s: state accumulator (lane holds S[dk0 + 4g + r][col n]); qrow: pointer to
// (Q ⊙ Lambda)[token n][dk0 + 4g] for this lane (g = lane / 16, n = lane % 16).
__device__ inline floatx4 state_times_q(floatx4 s, const bf16* qrow, floatx4 acc) {
  bf16x4 a;
#pragma unroll
  for (int r = 0; r < 4; ++r) a[r] = static_cast<bf16>(s[r]);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(qrow);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
__device__ inline floatx4 state_times_q(floatx4 s, const float* qrow, floatx4 acc) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(s[r], qrow[r], acc, 0, 0, 0);
  return acc;
}

}  // namespace

// Asynchronous global -> LDS copy of one 16-byte unit per lane: lane i of the
// wave writes LDS bytes [lds_wave_base + 16 i, + 16).  lds_wave_base must be
// the same for the whole wave.
__device__ inline void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                   0, 0);
}
// Wait for this wave's outstanding global loads (including LDS copies).
__device__ inline void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename T, int C, int DK, int DVT, int NWV = fused_waves(DK, DVT),
          int NTH = NWV * kWave>
__global__ __launch_bounds__(NTH) void k_seg_output(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ cum, const float* __restrict__ h0,
    const float* __restrict__ seg_in, T* __restrict__ o, float* __restrict__ hT, int L, int dv,
    int NC, int NSEG, int seg_chunks) {
  using M = Mma<T>;
  using PB = PBuilder<T, C, NWV>;
  constexpr bool BF = PB::BF;
  constexpr int ES = (int)sizeof(T);
  constexpr int KS = PB::KS, LDT = PB::LDT, LDF = PB::LDF, PT = PB::PT;
  constexpr int NRT = C / 16, NKT = DK / 16, NCT = DVT / 16;
  constexpr int NCW = NCT / NWV;  // column tiles per wave
  static_assert(NCW >= 1 && NCT % NWV == 0, "d_v tile must cover the waves");
  // Q ⊙ Lambda rows: d_k + 16 bf16 elements (a stride of 8 mod 16 dwords, so
  // the 16 rows of a state-times-q operand read fall in 8 distinct bank
  // windows); K ⊙ Gamma rows: unpadded and XOR-swizzled (ktx below) for bf16,
  // padded for fp32.
  constexpr int LDQ = DK + (BF ? 16 : 4), LDK = BF ? DK : DK + 4, LDP = C + PT;
  // staging of one slice as 16-byte units: q rows, k rows, cumsum rows
  constexpr int QU = KS * ES / 16;          // units per row of a q / k slice
  constexpr int BU = KS * 4 / 16;           // units per row of a cumsum slice
  constexpr int SU = C * (2 * QU + BU);     // units per slice
  constexpr int SBLK = (SU + NTH - 1) / NTH;
  // V tile: C rows x VU units, unpadded; unit u of row r sits at slot
  // u ^ vsw(r) so that column gathers of rows 8 apart hit different banks
  constexpr int VU = DVT * ES / 16;
  constexpr int VBLK = (C * VU + NTH - 1) / NTH;
  static_assert(SU % kWave == 0 && (C * VU) % kWave == 0, "whole waves per copy");

  // raw slice staging: the next slice's copy is issued only after every wave
  // has unpacked the current one, so one buffer suffices
  __shared__ __attribute__((aligned(16))) unsigned char stg[SU * 16];
  __shared__ __attribute__((aligned(16))) unsigned char smem[PB::SLICE_BYTES];
  __shared__ __attribute__((aligned(16))) T vs[C * DVT];
  __shared__ __attribute__((aligned(16))) T qt[C][LDQ];     // Q ⊙ Lambda
  __shared__ __attribute__((aligned(16))) T kt[C * LDK];    // K ⊙ Gamma
  __shared__ __attribute__((aligned(16))) T p_hi[C][LDP];
  __shared__ __attribute__((aligned(16))) T p_lo[BF ? C : 1][BF ? LDP : 8];
  __shared__ float pd[NWV][16][17];
  __shared__ float gam[DK];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + C * LDT;
  float* bs = reinterpret_cast<float*>(ks + C * LDT);
  float* als = bs + C * LDF;

  const int ntv = dv / DVT;
  const int j0 = (blockIdx.x % ntv) * DVT;
  const int seg = (blockIdx.x / ntv) % NSEG, bh = blockIdx.x / (ntv * NSEG);
  const int w = wave_id(), l = lane_id(), tid = threadIdx.x;
  const int lg = l >> 4, ln = l & 15;
  const size_t qo = (size_t)bh * L * DK, vo = (size_t)bh * L * dv;
  // Swizzles.  An MFMA operand read over tokens touches rows 8 g + j (+ 4) of a
  // tile, g = 0..3 the lane group, j = 0..3.  bf16: each row's part is one
  // 32-byte window; the window index is XORed with wsw(r), which separates
  // the 16 rows of a read into 8 windows (2 passes of the 64 banks, the
  // least for 512 bytes).  fp32: each row's part is 64 bytes; 4 rows.
  auto wsw = [](int r) { return (r & 3) | (((r >> 3) & 1) << 2); };
  // V tile, 16-byte units: unit u of row r sits at slot u ^ vsw(r)
  auto vsw = [&](int r) { return BF ? 2 * wsw(r) : 4 * (r & 3); };
  // K ⊙ Gamma: element (row, col)
  auto ktx = [&](int row, int col) {
    if constexpr (BF) {
      // 16-column windows, XOR-swizzled; d_k = 64 rows span half the banks,
      // so the row parity takes the place of one swizzle bit
      const int f = DK == 64 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : wsw(row);
      return row * DK + (((col >> 4) ^ f) << 4) + (col & 15);
    } else {
      return row * LDK + col;
    }
  };

  for (int it = tid; it < C * LDP; it += NTH) {
    (&p_hi[0][0])[it] = from_f32<T>(0.f);
    if constexpr (BF) (&p_lo[0][0])[it] = from_f32<T>(0.f);
  }

  // state tile: rows kt*16 + 4 lg + r, column j0 + (w * NCW + ct) * 16 + ln
  floatx4 S[NKT][NCW];
  const float* src = NSEG > 1 ? seg_in + ((size_t)bh * NSEG + seg) * DK * dv
                              : (h0 ? h0 + (size_t)bh * DK * dv : nullptr);
#pragma unroll
  for (int a = 0; a < NKT; ++a)
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct) {
      S[a][ct] = zero4();
      if (src) {
        const int col = j0 + (w * NCW + ct) * 16 + ln;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][ct][r] = src[(size_t)(a * 16 + 4 * lg + r) * dv + col];
      }
    }

  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);
  constexpr int NSL = DK / KS;  // slices per chunk

  // DMA one slice (chunk n, channels s0..s0+KS) into staging buffer b.  Rows
  // past the end of the sequence read the last valid row (finite values; q and
  // k of those rows are zeroed when the slice is unpacked).
  auto slice_dma = [&](int n, int s0) {
    const int r0 = n * C, rv = min(C, L - r0);
#pragma unroll
    for (int blk = 0; blk < SBLK; ++blk) {
      const int base = blk * NTH + w * kWave;  // first unit of this wave
      if (base >= SU) break;
      const int u = base + l;
      const char* g;
      if (u < 2 * C * QU) {
        const int which = u / (C * QU), uu = u % (C * QU);
        const int row = min(uu / QU, rv - 1), part = uu % QU;
        const T* p = (which == 0 ? q : k) + qo + (size_t)(r0 + row) * DK + s0;
        g = reinterpret_cast<const char*>(p) + part * 16;
      } else {
        const int uu = u - 2 * C * QU;
        const int row = min(uu / BU, rv - 1), part = uu % BU;
        g = reinterpret_cast<const char*>(cum + qo + (size_t)(r0 + row) * DK + s0) + part * 16;
      }
      dma16(g, &stg[base * 16]);
    }
  };
  auto v_dma = [&](int n) {
    const int r0 = n * C, rv = min(C, L - r0);
#pragma unroll
    for (int blk = 0; blk < VBLK; ++blk) {
      const int base = blk * NTH + w * kWave;
      if (base >= C * VU) break;
      const int slot = base + l, row = slot / VU, us = slot % VU;
      const int unit = us ^ vsw(row);
      const char* g = reinterpret_cast<const char*>(v + vo + (size_t)(r0 + min(row, rv - 1)) * dv + j0) +
                      unit * 16;
      dma16(g, reinterpret_cast<char*>(vs) + base * 16);
    }
  };
  // element (row, col) of the swizzled V tile
  auto vidx = [&](int row, int col) {
    constexpr int EPU = 16 / ES;  // elements per unit
    return row * DVT + (((col / EPU) ^ vsw(row)) * EPU) + col % EPU;
  };

  // MFMA operand (bf16: 8 consecutive tokens kr.. of one column) of the V tile
  // and of K ⊙ Gamma: transposed LDS reads for bf16, a scalar read for fp32.
  auto v_frag = [&](int kr, int cl) -> typename M::frag {
    if constexpr (BF) {
      // lane 4 a + b of each 16-lane group needs tokens kr..kr+7 of column
      // (cl & ~15) + 4 a + b; lane s addresses tokens kr + s / 4 (+ 4) at
      // columns (cl & ~15) + 4 (s % 4) .. + 3
      const int sl = l & 15;
      const int c = (cl & ~15) + 4 * (sl & 3);
      const int ra = kr + (sl >> 2), rb = ra + 4;
      const bf16* pa = reinterpret_cast<const bf16*>(vs) + vidx(ra, c);
      const bf16* pb = reinterpret_cast<const bf16*>(vs) + vidx(rb, c);
      return join8(ds_read_tr(pa), ds_read_tr(pb));
    } else {
      return vs[vidx(kr, cl)];
    }
  };
  auto k_frag = [&](int kr, int a) -> typename M::frag {
    if constexpr (BF) {
      const int sl = l & 15;
      const int ra = kr + (sl >> 2), c = a * 16 + 4 * (sl & 3);
      const bf16* kb = reinterpret_cast<const bf16*>(kt);
      return join8(ds_read_tr(kb + ktx(ra, c)), ds_read_tr(kb + ktx(ra + 4, c)));
    } else {
      return kt[ktx(kr, a * 16 + ln)];
    }
  };

  if (nb < ne) slice_dma(nb, 0);

  for (int n = nb; n < ne; ++n) {
    const int r0 = n * C, rv = min(C, L - r0);
    PB pb;
    pb.init();
    // ---- build P, Q ⊙ Lambda, K ⊙ Gamma and the chunk decay, slice by slice
#pragma unroll 1
    for (int sl = 0; sl < NSL; ++sl) {
      const int s0 = sl * KS;
      wait_dma();
      __syncthreads();  // staging complete; previous users of LDS done
      if (sl == 0) v_dma(n);
      // unpack the slice: padded q, k, cumsum; Q ⊙ Lambda, K ⊙ Gamma; decay
      for (int it = tid; it < C * (KS / 8); it += NTH) {
        const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
        const bool valid = row < rv;
        const T* sq = reinterpret_cast<const T*>(&stg[0]) + row * KS + c8;
        const T* sk = reinterpret_cast<const T*>(&stg[C * QU * 16]) + row * KS + c8;
        const float* sb = reinterpret_cast<const float*>(&stg[2 * C * QU * 16]);
        float qv[8], kv[8], bv[8], qtv[8], ktv[8];
        load8(sq, qv);
        load8(sk, kv);
        load8(sb + row * KS + c8, bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!valid) qv[e] = kv[e] = 0.f;
          const float g = sb[(C - 1) * KS + c8 + e];
          qtv[e] = qv[e] * gexp<T>(bv[e]);
          ktv[e] = kv[e] * gexp<T>(g - bv[e]);
        }
        store8(qs + row * LDT + c8, qv);
        store8(ks + row * LDT + c8, kv);
        store8(bs + row * LDF + c8, bv);
        store8(&qt[row][s0 + c8], qtv);
        store8(&kt[ktx(row, s0 + c8)], ktv);
        if (row == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) gam[s0 + c8 + e] = gexp<T>(sb[(C - 1) * KS + c8 + e]);
        }
      }
      __syncthreads();
      // the next slice (or the next chunk's first) streams in during the P work
      if (sl + 1 < NSL) slice_dma(n, s0 + KS);
      else if (n + 1 < ne) slice_dma(n + 1, 0);
      PB::gates(bs, als);
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
    // V must have landed: wait for the oldest DMA (the V tile) as well
    wait_dma();
    __syncthreads();

    // ---- O^T = S^T (Q ⊙ Lambda)^T for every query tile (S before the update;
    //      each state tile converted once)
    floatx4 ot[NCW][NRT];
#pragma unroll
    for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
      for (int jt = 0; jt < NRT; ++jt) ot[ct][jt] = zero4();
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt)
          ot[ct][jt] = state_times_q(S[a][ct], &qt[jt * 16 + ln][a * 16 + 4 * lg], ot[ct][jt]);
    // ---- O^T += V^T P^T, then store
#pragma unroll
    for (int jt = 0; jt < NRT; ++jt) {
#pragma unroll
      for (int kk = 0; kk < (jt + 1) * 16; kk += M::K) {
        const int kr = kk + lg * M::KPL;
        const auto ph = load_frag<T>(&p_hi[jt * 16 + ln][kr]);
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) {
          const auto vf = v_frag(kr, (w * NCW + ct) * 16 + ln);
          ot[ct][jt] = M::run(vf, ph, ot[ct][jt]);
          if constexpr (BF) {
            if (kk == ((jt * 16) / M::K) * M::K)
              ot[ct][jt] = M::run(vf, load_frag<T>(&p_lo[jt * 16 + ln][kr]), ot[ct][jt]);
          }
        }
      }
      const int row = jt * 16 + ln;
      if (row < rv) {
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct)
          store4(o + vo + (size_t)(r0 + row) * dv + j0 + (w * NCW + ct) * 16 + 4 * lg, ot[ct][jt]);
      }
    }
    // ---- S = diag(e^{b_n}) S + (K ⊙ Gamma)^T V
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[a][ct][r] *= gam[a * 16 + 4 * lg + r];
#pragma unroll 1
    for (int kk = 0; kk < C; kk += M::K) {
      const int kr = kk + lg * M::KPL;
      typename M::frag vf[NCW];
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) vf[ct] = v_frag(kr, (w * NCW + ct) * 16 + ln);
#pragma unroll
      for (int a = 0; a < NKT; ++a) {
        const auto ka = k_frag(kr, a);
#pragma unroll
        for (int ct = 0; ct < NCW; ++ct) S[a][ct] = M::run(ka, vf[ct], S[a][ct]);
      }
    }
  }

  if (NSEG == 1 && hT) {
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int ct = 0; ct < NCW; ++ct) {
        const int col = j0 + (w * NCW + ct) * 16 + ln;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hT[((size_t)bh * DK + a * 16 + 4 * lg + r) * dv + col] = S[a][ct][r];
      }
  }
}

template <typename T, int C, int DK, int DVT>
static hipError_t launch_so(const Plan& p, const void* q, const void* k, const void* v,
                            const float* cum, const float* h0, const float* seg_in, void* o,
                            float* hT, hipStream_t s) {
  dim3 grid(p.BH * p.NSEGF * (p.dv / DVT));
  hipLaunchKernelGGL((k_seg_output<T, C, DK, DVT>), grid, dim3(fused_waves(DK, DVT) * kWave), 0, s,
                     (const T*)q, (const T*)k, (const T*)v, cum, h0, seg_in, (T*)o, hT, p.L,
                     p.dv, p.NC, p.NSEGF, p.segf_chunks);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t launch_so_dv(const Plan& p, const void* q, const void* k, const void* v,
                               const float* cum, const float* h0, const float* seg_in, void* o,
                               float* hT, hipStream_t s) {
  // 256-wide d_v tiles only where the state tile fits the register file and
  // the operand tiles fit LDS (bf16, d_k <= 128)
  if constexpr (sizeof(T) == 2 && DK <= 128) {
    if (p.DVTF == 256) return launch_so<T, 64, DK, 256>(p, q, k, v, cum, h0, seg_in, o, hT, s);
  }
  return launch_so<T, 64, DK, 128>(p, q, k, v, cum, h0, seg_in, o, hT, s);
}

int fused_dv_tile(int bf16, int dk, int dv) { return (bf16 && dk <= 128 && dv % 256 == 0) ? 256 : 128; }

bool fused_supported(int bf16, int C, int dk, int dv) {
  if (C != 64) return false;
  if (dk != 64 && dk != 128 && dk != 256) return false;
  if (dv % 128) return false;
  if (!bf16 && dk == 256) return false;  // fp32 operand tiles would not fit in LDS
  return true;
}

hipError_t launch_seg_output(const Plan& p, const void* q, const void* k, const void* v,
                             const float* cum, const float* h0, const float* seg_in, void* o,
                             float* hT, hipStream_t s) {
  if (p.bf16) {
    if (p.dk == 64) return launch_so_dv<bf16, 64>(p, q, k, v, cum, h0, seg_in, o, hT, s);
    if (p.dk == 128) return launch_so_dv<bf16, 128>(p, q, k, v, cum, h0, seg_in, o, hT, s);
    return launch_so_dv<bf16, 256>(p, q, k, v, cum, h0, seg_in, o, hT, s);
  }
  if (p.dk == 64) return launch_so_dv<float, 64>(p, q, k, v, cum, h0, seg_in, o, hT, s);
  return launch_so_dv<float, 128>(p, q, k, v, cum, h0, seg_in, o, hT, s);
}

}  // namespace gla
