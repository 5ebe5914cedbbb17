// gla_recur.hip -- pass 2 of the two-pass forward of the GLA chunkwise layer
// (gfx950).
//
// k_chunk_recur: one workgroup per (batch-head, sequence segment, d_v tile),
// walking the segment's chunks in order with its d_k x d_v_tile slice of the
// state in MFMA accumulators (fp32):
//   O[n]^T = S_{n-1}^T Q~^T + V^T P^T                 (output, transposed)
//   S_n    = diag(e^{b_n}) S_{n-1} + K~^T V           (state)
// (papercache.org notes §4.2; §3.3 / Figure 1a keeps the state on chip).
// Every chunk's Q~, K~, P, b (written by pass 1, gla_prep.hip, in the layouts
// of gla_records.h) and V tile stream into LDS with LDS-DMA while the
// previous chunk computes; each wave owns 16 state columns.  In its local mode
// (no output) the same walk starts from zero and leaves each segment's own
// state contribution and total log decay for the segment scan.
#include "gla_common.h"
#include "gla_dma.h"
#include "gla_internal.h"
#include "gla_pblock.h"
#include "gla_records.h"

namespace gla {

namespace {

// Loading wave li of NLD issues copies li, li + NLD, ... of a contiguous tile
// of NCOPY copies (all NLD waves issue a one-copy tile); copy c moves the
// 1 KB at src + 1024 c into LDS at dst + 1024 c.
template <int NCOPY, int NLD>
__device__ inline void copy_tile(const unsigned char* src, unsigned dst, int li, int l) {
  static_assert(NCOPY <= 1 || NCOPY % NLD == 0, "uneven split");
  const i32x4 r = make_rsrc(src);
  const unsigned loff = (unsigned)l * 16u;
  if constexpr (NCOPY == 1) {
    dma16b(r, loff, 0u, dst);
  } else {
#pragma unroll
    for (int i = 0; i < NCOPY / NLD; ++i) {
      const int c = li + i * NLD;
      dma16b(r, loff, (unsigned)c * 1024u, dst + (unsigned)c * 1024u);
    }
  }
}

}  // namespace

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
  static constexpr int PB = OUT ? RD::pblocks(C) * 1024 : 0;
  static constexpr int LB = (OUT && BF) ? C * 16 * ES : 0;
  static constexpr int GB = RD::gbytes(DK);
  static constexpr int VB = C * DVT * ES;
  static constexpr int VBLK = BF ? 32 * VUPR * 16 : 16 * VUPR * 16;  // bytes per V block
  // one record buffer: Q~, K~, P, P's low part, gates
  static constexpr int oQ = 0, oK = oQ + QB, oP = oK + KB, oL = oP + PB, oG = oL + LB,
                       RBUF = oG + GB;
  // NLD loading waves share each chunk's copies: a tile of n > 1 copies (a
  // power of two) gives each n / NLD, a one-copy tile is issued by all (the
  // same bytes to the same place), so all issue the same number of copies per
  // chunk and each has its own 6-bit vmcnt of copies in flight.  One is
  // enough where the copies' latency is the limit rather than that counter.
  static constexpr int NLD = 1;
  static constexpr int NWAVES = NWV + NLD;
  static constexpr int per_loader(int bytes) {
    return bytes == 0 ? 0 : (bytes == 1024 ? 1 : bytes / 1024 / NLD);
  }
  static constexpr int VCOPY = per_loader(VB);  // V copies per chunk and loading wave
  static constexpr int RCPC =                   // record copies per chunk and loading wave
      per_loader(QB) + per_loader(KB) + per_loader(PB) + per_loader(LB) + per_loader(GB);
  static constexpr int CPC = RCPC + VCOPY;      // copies per chunk and loading wave
  // Record buffers: three (copies run two chunks ahead) when they fit and a
  // chunk's copy count fits the 6-bit vmcnt field, else two, else one.
  static constexpr int NBUF = (CPC <= 63 && 3 * (RBUF + VB) <= kLdsLimit)
                                  ? 3
                                  : (2 * (RBUF + VB) <= kLdsLimit ? 2 : 1);
  // V buffers: V comes straight from HBM (the records were just written by
  // the prep pass), so its copies run further ahead in a ring of their own
  // while the LDS and the vmcnt field allow (see the loader's waits).
  static constexpr int vnb_max(int n) {
    return (n < 6 && NBUF * RBUF + (n + 1) * VB <= kLdsLimit &&
            (NBUF == 3 ? 2 * VCOPY + RCPC : VCOPY) <= 63)
               ? vnb_max(n + 1)
               : n;
  }
  static constexpr int VNB = NBUF == 1 ? 1 : vnb_max(NBUF);
  static constexpr int oV = NBUF * RBUF;        // V ring after the record buffers
  static constexpr int LDS = oV + VNB * VB;
  static_assert(QB % 1024 == 0 && KB % 1024 == 0 && PB % 1024 == 0 && LB % 1024 == 0 &&
                    VB % 1024 == 0 && GB % 1024 == 0,
                "every staged tile is a whole number of 1 KB copies");
  static constexpr bool split_ok(int bytes) { return bytes <= 1024 || (bytes / 1024) % NLD == 0; }
  static_assert(split_ok(QB) && split_ok(KB) && split_ok(PB) && split_ok(LB) && split_ok(GB) &&
                    split_ok(VB),
                "every tile splits evenly over the loading waves");
  static_assert(LDS <= kLdsLimit, "staged chunk exceeds LDS");
};

// Waves 0 .. NWV-1 compute (16 state columns each); waves NWV .. NWV+NLD-1
// only issue the LDS copies and wait for them, so that their memory counters
// hold nothing but loads (a partial wait is exact) and the computing waves,
// which store the output, never wait on memory.
//
// REV: the time-reversed sequence (the dv pass of the backward): row p of a
// chunk's V and of the output is row L - 1 - p in memory; the records, built
// by the prep pass in its reversed mode, need no change.
template <typename T, int C, int DK, int NWV, int OUT, bool REV = false>
__global__ __launch_bounds__((RecurLayout<T, C, DK, NWV, OUT>::NWAVES * kWave)) void k_chunk_recur(
    const unsigned char* __restrict__ qrec, const unsigned char* __restrict__ krec,
    const unsigned char* __restrict__ prec, const unsigned char* __restrict__ lrec,
    const float* __restrict__ grec, const T* __restrict__ v, const float* __restrict__ init,
    T* __restrict__ o, float* __restrict__ fin, float* __restrict__ seg_g, int L, int dv, int NC,
    int NSEG, int seg_chunks) {
  using Lay = RecurLayout<T, C, DK, NWV, OUT>;
  constexpr bool BF = Lay::BF;
  constexpr int ES = Lay::ES, DVT = Lay::DVT, NTH = NWV * kWave, VUPR = Lay::VUPR;
  constexpr int NRT = C / 16, NKT = DK / 16, NG = Lay::NG, NPG = Lay::NPG;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Lay::LDS];

  const int ntv = dv / DVT;
  const int lid = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lid % ntv, seg = (lid / ntv) % NSEG, bh = lid / (ntv * NSEG);
  const int j0 = tile * DVT;
  // the wave index as a scalar: copy and column offsets derived from it stay
  // in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const bool loader = w >= NWV;
  const bool computer = !loader;
  const int li = (Lay::NLD > 1 && loader) ? w - NWV : 0;  // loading wave index
  const int l = lane_id(), g = l >> 4, ln = l & 15;
  const int vc = computer ? 16 * w : 0;  // this wave's first column within the tile
  const int col = j0 + vc + ln;          // this lane's state column
  const int nb = seg * seg_chunks, ne = min(NC, nb + seg_chunks);

  // ---- state slice: lane holds S[16 a + 4 g + r][col]
  floatx4 S[NKT];
  {
    const float* src = nullptr;
    if (OUT && computer) src = NSEG > 1 ? init + ((size_t)bh * NSEG + seg) * DK * dv
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
  // Stage chunk n's records into record buffer (n - nb) % NBUF (the loading
  // waves only).
  auto issue_r = [&](int n) __attribute__((always_inline)) {
    const unsigned base = lds0 + (unsigned)(((n - nb) % Lay::NBUF) * Lay::RBUF);
    const size_t cb = (size_t)bh * NC + n;
    constexpr int NLD = Lay::NLD;
    if constexpr (OUT) {
      copy_tile<Lay::QB / 1024, NLD>(qrec + cb * Lay::QB, base + Lay::oQ, li, l);
      copy_tile<Lay::PB / 1024, NLD>(prec + cb * Lay::PB, base + Lay::oP, li, l);
      if constexpr (BF) copy_tile<Lay::LB / 1024, NLD>(lrec + cb * Lay::LB, base + Lay::oL, li, l);
    }
    copy_tile<Lay::KB / 1024, NLD>(krec + cb * Lay::KB, base + Lay::oK, li, l);
    copy_tile<Lay::GB / 1024, NLD>(reinterpret_cast<const unsigned char*>(grec) + cb * Lay::GB,
                                   base + Lay::oG, li, l);
  };
  // Stage chunk n's V tile into V buffer n % VNB (the loading waves only).
  auto issue_v = [&](int n) __attribute__((always_inline)) {
    const unsigned base = lds0 + (unsigned)(Lay::oV + (n % Lay::VNB) * Lay::VB);
    // V rows past the end of the sequence repeat the last row (their K~ rows
    // and P columns are zero)
    const int r0 = n * C;
    const i32x4 vr = make_rsrc(REV ? v + (size_t)bh * L * dv + j0 : v + ((size_t)bh * L + r0) * dv + j0);
    const bool full = r0 + C <= L;
    constexpr int NVC = Lay::VB / 1024;
#pragma unroll
    for (int i = 0; i < (NVC == 1 ? 1 : NVC / Lay::NLD); ++i) {
      const int c = NVC == 1 ? 0 : li + i * Lay::NLD;
      int rho, u;
      vslot(c, rho, u);
      if (!full) rho = min(rho, L - 1 - r0);
      const int prow = REV ? L - 1 - r0 - rho : rho;  // row in memory (from r0 unless REV)
      dma16b(vr, (unsigned)(prow * dv * ES + u * 16), 0u, base + (unsigned)(c * 1024));
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

  // Output stores go through a buffer resource spanning the head's L rows:
  // rows past the end of the sequence fall outside it and are dropped by the
  // hardware, so the stores need no branch.
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(OUT ? o + (size_t)bh * L * dv : o, 0, L * dv * ES, 0x00020000);
  // (REV: rows past the end of the sequence map to negative rows, whose
  // offsets, read unsigned, fall outside the resource as well)
  auto store_out = [&](int n, const floatx4 (&ot)[NRT]) __attribute__((always_inline)) {
    if constexpr (OUT) {
#pragma unroll
      for (int jt = 0; jt < NRT; ++jt) {
        const int row = n * C + 16 * jt + ln;
        const int off = ((REV ? L - 1 - row : row) * dv + j0 + vc + 4 * g) * ES;
        if constexpr (BF) {
          bf16x4 h;
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = static_cast<bf16>(ot[jt][r]);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, h), orsrc, off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, ot[jt]), orsrc, off, 0, 0);
        }
      }
    }
  };

  // ot holds the output of chunk pn (-1: none yet), stored at the start of
  // the next chunk's body: its products finished during the barrier, and
  // the stores are then in flight while that body's products run.
  floatx4 ot[NRT];
  int pn = -1;
  auto flush_out = [&](int n) __attribute__((always_inline)) {
    if (pn >= 0) store_out(pn, ot);
    pn = n;
  };

  // One chunk from record buffer b, after the previous chunk's output is
  // stored.  bf16: the state update first (from the bf16 copy of S_{n-1} that
  // the output products use), so that the next chunk's products, which need
  // S_n, never wait for this chunk's output products; then this chunk's
  // output into ot.  fp32: output first, then the update.
  auto body = [&](int n, int b) __attribute__((always_inline)) {
    const unsigned char* base = lds + b * Lay::RBUF;
    const unsigned char* Qs = base + Lay::oQ;
    const unsigned char* Ks = base + Lay::oK;
    const unsigned char* Ps = base + Lay::oP;
    const unsigned char* Ls = base + Lay::oL;
    const float* Gs = reinterpret_cast<const float*>(base + Lay::oG);
    const unsigned char* Vs = lds + Lay::oV + (n % Lay::VNB) * Lay::VB;
    if constexpr (BF) {
      if constexpr (OUT) flush_out(n);
      // V fragments over token runs 32 kt + 8 g + e at column vc + ln
      bf16x8 vf[C / 32];
#pragma unroll
      for (int kt = 0; kt < C / 32; ++kt) {
        const bf16* vb = reinterpret_cast<const bf16*>(Vs + kt * Lay::VBLK);
        vf[kt] = join8(ds_read_tr(reinterpret_cast<const bf16*>(reinterpret_cast<const unsigned char*>(vb) + voff[0])),
                       ds_read_tr(reinterpret_cast<const bf16*>(reinterpret_cast<const unsigned char*>(vb) + voff[1])));
      }
      // S_{n-1}^T as the output products' A operands: the MFMA's K index
      // 8 g + e maps to channel 32 a2 + 4 g + e (e < 4) or + 16 + 4 g + e - 4
      // (the order of the Q~ units)
      bf16x8 A[OUT ? NKT / 2 : 1];
      if constexpr (OUT) {
#pragma unroll
        for (int a2 = 0; a2 < NKT / 2; ++a2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            A[a2][r] = static_cast<bf16>(S[2 * a2][r]);
            A[a2][r + 4] = static_cast<bf16>(S[2 * a2 + 1][r]);
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
      if constexpr (OUT) {
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) ot[jt] = zero4();
        // O^T += S_{n-1}^T Q~^T over pairs of 16-channel tiles
#pragma unroll
        for (int a2 = 0; a2 < NKT / 2; ++a2) {
#pragma unroll
          for (int jt = 0; jt < NRT; ++jt) {
            const bf16x8 B = *reinterpret_cast<const bf16x8*>(Qs + (jt * NG + a2) * 1024 + qoff);
            ot[jt] = Mma<bf16>::run(A[a2], B, ot[jt]);
          }
        }
        // O^T += V^T P^T (P rounded; its diagonal blocks also carry a low part)
#pragma unroll
        for (int jt = 0; jt < NRT; ++jt) {
#pragma unroll
          for (int kt = 0; kt <= (jt >> 1); ++kt) {
            const bf16x8 pf = *reinterpret_cast<const bf16x8*>(Ps + RecDims<T>::pblock(jt, kt) * 1024 + qoff);
            ot[jt] = Mma<bf16>::run(vf[kt], pf, ot[jt]);
          }
          // every lane reads (a branch would force a wait for the read), the
          // lanes whose K range is not this block's diagonal drop the value
          bf16x8 lf = *reinterpret_cast<const bf16x8*>(Ls + jt * 512 + loff);
          if ((g >> 1) != (jt & 1)) lf = bf16x8{};
          ot[jt] = Mma<bf16>::run(vf[jt >> 1], lf, ot[jt]);
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
        flush_out(n);
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
            const f32x4 pf = *reinterpret_cast<const f32x4*>(Ps + RecDims<T>::pblock(jt, bb) * 1024 + qoff);
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

  // ---- walk the segment's chunks.  While chunk n computes, the loading wave
  // stages the records of chunk n + D (D = NBUF - 1) into the record buffer
  // that chunk n - 1 used and the V tile of chunk n + VD (VD = VNB - 1) into
  // the V buffer that chunk n - 1 used, then waits until chunk n + 1 has
  // landed, and the step ends with a barrier.  Record buffer indices are
  // literals at every step call.
  constexpr int D = Lay::NBUF - 1;
  constexpr int VD = Lay::VNB - 1;
  // The copies of step s: chunk s + D's records, then chunk s + VD's V tile
  // (steps before nb issue only what belongs to the segment).
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    if (s + D >= nb && s + D < ne) issue_r(s + D);
    if (s + VD < ne) issue_v(s + VD);
  };
  // At step n, after its copies: wait until chunk n + 1 has landed.  A
  // loading wave issues only loads, which complete in issue order, so each
  // waits until no more of its copies are outstanding than it issued after
  // its last one of chunk n + 1: with VD > D that is its records (issued at
  // step n + 1 - D), followed by that step's V copies and the copies of the
  // steps after it; with VD = D it is its V tile, followed by the later
  // steps' copies.  Copies past the end of the segment are never issued.
  auto wait_next = [&](int n) __attribute__((always_inline)) {
    if constexpr (D == 2 && VD > 2) {
      if (n + VD < ne) wait_vm_le<2 * Lay::VCOPY + Lay::RCPC>();
      else if (n - 1 + VD < ne) wait_vm_le<Lay::VCOPY + Lay::RCPC>();
      else if (n + 2 < ne) wait_vm_le<Lay::RCPC>();
      else wait_vm();
    } else if constexpr (D == 2) {
      if (n + 2 < ne) wait_vm_le<Lay::CPC>();
      else wait_vm();
    } else if constexpr (D == 1 && VD > 1) {
      if (n + VD < ne) wait_vm_le<Lay::VCOPY>();
      else wait_vm();
    } else {
      wait_vm();
    }
  };
  auto step = [&](int n, int b) __attribute__((always_inline)) {
    if constexpr (D > 0) {
      if (loader) {
        issue_step(n);
        if (n + 1 < ne) wait_next(n);
      } else {
        body(n, b);
      }
      lds_barrier();  // chunk n + 1 staged; everyone is done with buffer b
    } else {
      if (computer) body(n, 0);
      lds_barrier();  // everyone is done with the buffer
      if (loader && n + 1 < ne) {
        issue_r(n + 1);
        issue_v(n + 1);
        wait_vm();
      }
      lds_barrier();  // chunk n + 1 staged
    }
  };

  if (nb < ne) {
    if (loader) {
      if constexpr (D > 0) {
        // the copies that steps nb - VD .. nb - 1 would have issued
#pragma unroll
        for (int i = VD; i > 0; --i) issue_step(nb - i);
        wait_next(nb - 1);
      } else {
        issue_r(nb);
        issue_v(nb);
        wait_vm();
      }
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

  if (OUT && computer && pn >= 0) store_out(pn, ot);

  // ---- end of the segment
  float* dst = nullptr;
  if (OUT) dst = (NSEG == 1 && fin) ? fin + (size_t)bh * DK * dv : nullptr;
  else dst = fin + ((size_t)bh * NSEG + seg) * DK * dv;
  if (dst && computer) {
#pragma unroll
    for (int a = 0; a < NKT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)(a * 16 + 4 * g + r) * dv + col] = S[a][r];
  }
  if (!OUT && tile == 0 && computer) {
#pragma unroll
    for (int i = 0; i < NGS; ++i) {
      const int t = threadIdx.x + i * NTH;
      if (t < DK) seg_g[((size_t)bh * NSEG + seg) * DK + t] = gsum[i];
    }
  }
}

// =========================================================== launchers
template <typename T, int C, int DK, int NWV, bool REV>
static hipError_t launch_recur_w(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* grec,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  const dim3 grid(p.BH * p.NSEGR * (p.dv / (16 * NWV)));
  const unsigned char *q8 = (const unsigned char*)qg, *k8 = (const unsigned char*)kg,
                      *p8 = (const unsigned char*)ph, *l8 = (const unsigned char*)pl;
  if (out)
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 1, REV>), grid,
                       dim3(RecurLayout<T, C, DK, NWV, 1>::NWAVES * kWave), 0, s, q8, k8,
                       p8, l8, grec, (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC,
                       p.NSEGR, p.segr_chunks);
  else
    hipLaunchKernelGGL((k_chunk_recur<T, C, DK, NWV, 0, REV>), grid,
                       dim3(RecurLayout<T, C, DK, NWV, 0>::NWAVES * kWave), 0, s, q8, k8,
                       p8, l8, grec, (const T*)v, init, (T*)o, fin, seg_g, p.L, p.dv, p.NC,
                       p.NSEGR, p.segr_chunks);
  return hipGetLastError();
}

template <typename T, int C, int DK, bool REV = false>
static hipError_t launch_recur_d(const Plan& p, int out, const void* qg, const void* kg,
                                 const void* ph, const void* pl, const float* grec,
                                 const void* v, const float* init, void* o, float* fin,
                                 float* seg_g, hipStream_t s) {
  if constexpr (recur_max_waves(sizeof(T) == 2, DK) == 4)
    if (p.NWVR == 4)
      return launch_recur_w<T, C, DK, 4, REV>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  if (p.NWVR == 2)
    return launch_recur_w<T, C, DK, 2, REV>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
  if constexpr (recur_min_waves(sizeof(T) == 2, DK) == 1)
    return launch_recur_w<T, C, DK, 1, REV>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s);
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

hipError_t launch_chunk_recur_rev(const Plan& p, int out, const void* qg, const void* kg,
                                  const void* ph, const void* pl, const float* grec,
                                  const void* v, const float* init, void* o, float* fin,
                                  float* seg_g, hipStream_t s) {
  if (!p.bf16 || p.C != 64) return hipErrorInvalidValue;
#define GLA_RECUR_REV_DK(D)                                                                      \
  if (p.dk == D)                                                                                 \
  return launch_recur_d<bf16, 64, D, true>(p, out, qg, kg, ph, pl, grec, v, init, o, fin, seg_g, s)
  GLA_RECUR_REV_DK(32);
  GLA_RECUR_REV_DK(64);
  GLA_RECUR_REV_DK(128);
  GLA_RECUR_REV_DK(256);
#undef GLA_RECUR_REV_DK
  return hipErrorInvalidValue;
}

size_t recur_grec_bytes(int dk) { return RecDims<float>::gbytes(dk); }
size_t recur_prec_bytes(int is_bf16, int C) {
  return (size_t)(is_bf16 ? RecDims<bf16>::pblocks(C) : RecDims<float>::pblocks(C)) * 1024;
}

bool recur_supported(int bf16, int C, int dk, int dv, int L) {
  const bool shape = bf16 ? (C == 32 || C == 64) && (dk == 32 || dk == 64 || dk == 128 || dk == 256)
                          : (C == 16 || C == 32 || C == 64) && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
  // a head's output must be addressable with 32-bit byte offsets
  const bool range = (long long)L * dv * (bf16 ? 2 : 4) <= 0x7fffffffLL;
  return shape && range && dv % (16 * recur_min_waves(bf16, dk)) == 0;
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
