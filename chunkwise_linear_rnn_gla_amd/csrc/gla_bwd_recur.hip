// gla_bwd_recur.hip -- the backward's inter-chunk gradient terms with the
// states kept on chip (gfx950, bf16 I/O).
//
// The chunkwise backward (chain rule through the chunkwise form of
// papercache.org notes §4.2; the states are recomputed, zako-mio report ch.
// 2.2) needs, per chunk n, the state entering it and the state gradient
// leaving it:
//   dQ_inter[n] = (dO[n] S_{n-1}^T) ⊙ Lambda[n],
//       S_n     = diag(gamma_n) S_{n-1} + (K[n] ⊙ Gamma[n])^T V[n],   S_{-1} = h0
//   dK_inter[n] = (V[n] dS_n^T) ⊙ Gamma[n],
//       dS_{n-1} = diag(gamma_n) dS_n + (Q[n] ⊙ Lambda[n])^T dO[n],  dS_{NC-1} = dhT
// with Lambda = e^{B}, Gamma = e^{b - B}, gamma = e^{b} (B the chunk-local
// cumsum of log alpha, b its last row).  k_bwd_inter computes both without
// writing a single state: a workgroup walks the chunks of one (batch, head)
// with a 32-channel slice of the transposed state U = S^T (dq job, chunks in
// order) or U = dS^T (dk job, chunks in reverse order) in MFMA accumulators,
// all d_v rows of it, one 16-channel column block per computing wave.  Per
// chunk it forms the output product X_y U (X_y = dO or V) scaled by Lambda
// or Gamma, writes it in fp32, and updates U by its column gates and
// X_u^T (Z ⊙ scale) (X_u = V or dO; Z = k ⊙ Gamma or q ⊙ Lambda).
//
// Precision: the closed-form gate gradient subtracts q ⊙ dq - k ⊙ dk, terms
// tens of times larger than their difference, so both products run with the
// fp32 operand (U, and the scaled Z) split into a high and a low bf16 part
// (two MFMAs each); dO, V are exact in bf16.  The dq job also leaves
// rowsum(hT ⊙ dhT) (hT = its final state), the dk job dh0 = dS_{-1}.
//
// Staging: a loading wave copies each chunk's X_y and X_u rows (all d_v
// columns) and the workgroup's 32 columns of Z's input (k or q) and of the
// cumsum into LDS with LDS-DMA, one chunk ahead, into a double buffer.  The X
// rows are stored with a stride of one 16-byte unit more than a row (the
// extra unit is never read), so that every operand read is one per-lane base
// address plus a compile-time offset (no per-tile address registers): the
// output product's row reads (16 rows at one unit) are then free of bank
// conflicts (64 banks x 4 B), the update's transposed reads at most 2-way.
#include "gla_common.h"
#include "gla_dma.h"
#include "gla_internal.h"
#include "gla_pblock.h"
#include "gla_records.h"

namespace gla {

namespace {

constexpr int kBC = 64;   // chunk rows
constexpr int kBW = 32;   // key channels per workgroup (two computing waves)

template <int DV>
struct InterLayout {
  static constexpr int UPR = DV / 8;            // 16-byte units per X row
  static constexpr int RS = UPR + 1;            // units per staged row (one of padding)
  static constexpr int NT = DV / 16;            // 16-row tiles of U (d_v rows)
  static constexpr int TB = kBC * RS * 16;      // one staged X tile
  static constexpr int SB = kBC * kBW * 2;      // the chunk's 32 columns of k or q
  static constexpr int BB = kBC * kBW * 4;      // the chunk's 32 columns of the cumsum
  static constexpr int oY = 0, oU = TB, oS = 2 * TB, oB = 2 * TB + SB, RBUF = 2 * TB + SB + BB;
  static constexpr int LDS = 2 * RBUF;          // double buffer
  static_assert(UPR % 16 == 0, "rows of whole 256-byte bank spans");
  static_assert(LDS <= kLdsLimit, "staged chunk exceeds LDS");
  static_assert(TB % 1024 == 0 && SB % 1024 == 0 && BB % 1024 == 0, "1 KB copies");
};

__device__ inline bf16x4 lds_read8(const unsigned char* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}

}  // namespace

// One job per half of the grid: workgroups [0, nper) run `jf` (dq), the rest
// `jk` (dk).  Three waves: 0 and 1 compute (16 key channels each), 2 loads.
template <int DV>
__global__ __launch_bounds__(3 * kWave) void k_bwd_inter(BwdInterJob jf, BwdInterJob jk,
                                                         const float* __restrict__ cum, int L,
                                                         int dk, int NC, int nper) {
  using Lay = InterLayout<DV>;
  constexpr int UPR = Lay::UPR, NT = Lay::NT;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Lay::LDS];

  const bool second = blockIdx.x >= (unsigned)nper;
  const BwdInterJob& J = second ? jk : jf;
  const int rev = J.rev;
  const int bid = second ? (int)blockIdx.x - nper : (int)blockIdx.x;
  const int ntile = dk / kBW;
  const int lid = xcd_logical(bid, nper);
  const int bh = lid / ntile, i0 = (lid % ntile) * kBW;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const bool loader = w == 2;
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int wc = loader ? 0 : 16 * w;      // this wave's first channel in the slice
  const int icol = i0 + wc + n;            // this lane's state column (key channel)
  const unsigned lds0 = lds_addr(lds);

  // ---- the state slice: lane (g, n) of tile a holds U[16 a + 4 g + r][icol]
  floatx4 U[NT];
#pragma unroll
  for (int a = 0; a < NT; ++a) {
    U[a] = zero4();
    if (J.init && !loader)
      U[a] = *reinterpret_cast<const f32x4*>(J.init + ((size_t)bh * dk + icol) * DV + 16 * a + 4 * g);
  }
  // The state registers are consumed here, before the chunk loop: a load
  // still pending into them at the loop's entry would otherwise make the
  // compiler wait for every outstanding memory operation (including the
  // previous chunk's output stores) at the top of each chunk.
#pragma unroll
  for (int a = 0; a < NT; ++a) asm volatile("" ::"v"(U[a]));

  // ---- the loading wave's copies of one chunk into buffer b
  const unsigned char* xy = reinterpret_cast<const unsigned char*>(J.xy) + (size_t)bh * L * DV * 2;
  const unsigned char* xu = reinterpret_cast<const unsigned char*>(J.xu) + (size_t)bh * L * DV * 2;
  const unsigned char* zs = reinterpret_cast<const unsigned char*>(J.z) + ((size_t)bh * L * dk + i0) * 2;
  const unsigned char* bs = reinterpret_cast<const unsigned char*>(cum + (size_t)bh * L * dk + i0);
  auto issue = [&](int nc, int b) __attribute__((always_inline)) {
    const unsigned base = lds0 + (unsigned)(b * Lay::RBUF);
    const int r0 = nc * kBC;
    const i32x4 ry = make_rsrc(xy), ru = make_rsrc(xu), rz = make_rsrc(zs), rb = make_rsrc(bs);
#pragma unroll 4
    for (int c = 0; c < Lay::TB / 1024; ++c) {
      // staged unit s of the tile: row s / RS, unit s % RS (the padding unit
      // RS - 1 takes a copy of the row's first unit and is never read)
      const int s = 64 * c + l, row = s / Lay::RS, unit = s % Lay::RS;
      const unsigned prow = (unsigned)min(r0 + row, L - 1);
      const unsigned off = prow * (unsigned)(DV * 2) + (unsigned)((unit < UPR ? unit : 0) * 16);
      dma16b(ry, off, 0u, base + Lay::oY + (unsigned)c * 1024u);
      dma16b(ru, off, 0u, base + Lay::oU + (unsigned)c * 1024u);
    }
#pragma unroll
    for (int c = 0; c < Lay::SB / 1024; ++c) {
      const int s = 64 * c + l, row = s / 4, unit = s % 4;
      const unsigned prow = (unsigned)min(r0 + row, L - 1);
      dma16b(rz, prow * (unsigned)(dk * 2) + (unsigned)(unit * 16), 0u, base + Lay::oS + (unsigned)c * 1024u);
    }
#pragma unroll
    for (int c = 0; c < Lay::BB / 1024; ++c) {
      const int s = 64 * c + l, row = s / 8, unit = s % 8;
      const unsigned prow = (unsigned)min(r0 + row, L - 1);
      dma16b(rb, prow * (unsigned)(dk * 4) + (unsigned)(unit * 16), 0u, base + Lay::oB + (unsigned)c * 1024u);
    }
  };

  // Output stores through a buffer resource spanning the head's L rows: rows
  // past the end of the sequence fall outside it and are dropped.
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(J.out + (size_t)bh * L * dk, 0, L * dk * 4, 0x00020000);

  // ---- lane-constant parts of the operand addresses (bytes)
  constexpr int RSB = Lay::RS * 16;                    // staged row stride
  // output product: row m = 16 mb + n, units 4 a2 + (g >> 1) and + 2, half g & 1
  const int yoff = n * RSB + (g >> 1) * 16 + (g & 1) * 8;
  // update: rows 32 kt + 8 g + (n >> 2) and + 4, unit 2 a + ((n & 3) >> 1), half n & 1
  const int uoff = (8 * g + (n >> 2)) * RSB + ((n & 3) >> 1) * 16 + (n & 1) * 8;

  // ---- one chunk from buffer b
  auto body = [&](int nc, int b) __attribute__((always_inline)) {
    const unsigned char* Yt = lds + b * Lay::RBUF + Lay::oY + yoff;
    const unsigned char* Ut = lds + b * Lay::RBUF + Lay::oU + uoff;
    const bf16* Zs = reinterpret_cast<const bf16*>(lds + b * Lay::RBUF + Lay::oS);
    const float* Bs = reinterpret_cast<const float*>(lds + b * Lay::RBUF + Lay::oB);
    const int r0 = nc * kBC, rv = min(kBC, L - r0);
    // chunk totals b of the lane's output channels (4 g + r) and state column
    const f32x4 blast4 = *reinterpret_cast<const f32x4*>(Bs + (rv - 1) * kBW + wc + 4 * g);
    const float bcol = Bs[(rv - 1) * kBW + wc + n];

    // output: Y^T = U^T X_y^T over d_v; the accumulator pair (2 a2, 2 a2 + 1)
    // is the A operand (K index 8 g + e -> row 32 a2 + 4 g + e, or
    // 32 a2 + 16 + 4 g + e - 4), matched by the units read from X_y
    floatx4 Y[kBC / 16];
#pragma unroll
    for (int mb = 0; mb < kBC / 16; ++mb) Y[mb] = zero4();
#pragma unroll
    for (int a2 = 0; a2 < NT / 2; ++a2) {
      bf16x8 bx[kBC / 16];
#pragma unroll
      for (int mb = 0; mb < kBC / 16; ++mb) {
        const unsigned char* p = Yt + mb * 16 * RSB + a2 * 64;
        bx[mb] = join8(lds_read8(p), lds_read8(p + 32));
      }
      bf16x8 ahi, alo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ahi[r] = static_cast<bf16>(U[2 * a2][r]);
        ahi[r + 4] = static_cast<bf16>(U[2 * a2 + 1][r]);
        alo[r] = static_cast<bf16>(U[2 * a2][r] - static_cast<float>(ahi[r]));
        alo[r + 4] = static_cast<bf16>(U[2 * a2 + 1][r] - static_cast<float>(ahi[r + 4]));
      }
#pragma unroll
      for (int mb = 0; mb < kBC / 16; ++mb) {
        Y[mb] = Mma<bf16>::run(ahi, bx[mb], Y[mb]);
        Y[mb] = Mma<bf16>::run(alo, bx[mb], Y[mb]);
      }
    }
    // scale by Lambda = e^{B} (dq) or Gamma = e^{b - B} (dk) and store: lane
    // (g, n) holds rows 16 mb + n, channels wc + 4 g + r
#pragma unroll
    for (int mb = 0; mb < kBC / 16; ++mb) {
      const int m = 16 * mb + n;
      const f32x4 bm = *reinterpret_cast<const f32x4*>(Bs + m * kBW + wc + 4 * g);
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = Y[mb][r] * __expf(rev ? blast4[r] - bm[r] : bm[r]);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), orsrc,
                                             ((r0 + m) * dk + i0 + wc + 4 * g) * 4, 0, 0);
    }

    // update: U <- U diag(e^{b}) + X_u^T Z~, Z~ = k e^{b - B} (dq) or q e^{B}
    // (dk), zero on rows past the end of the sequence
    const float gam = __expf(bcol);
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) U[a][r] *= gam;
#pragma unroll
    for (int kt = 0; kt < kBC / 32; ++kt) {
      const bf16x8 zr = col_frag_tr(Zs, kBW, 32 * kt, wc, l);
      bf16x8 zhi, zlo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // rows past the end (which repeat the last row's cumsum) are zeroed
        // by a select, not a branch
        const int tok = 32 * kt + 8 * g + e;
        const float bt = Bs[tok * kBW + wc + n];
        const float sc = __expf(rev ? bt : bcol - bt);
        const float val = tok < rv ? static_cast<float>(zr[e]) * sc : 0.f;
        zhi[e] = static_cast<bf16>(val);
        zlo[e] = static_cast<bf16>(val - static_cast<float>(zhi[e]));
      }
      constexpr int AG = 4;  // tiles whose operands are read before their products
#pragma unroll
      for (int a0 = 0; a0 < NT; a0 += AG) {
        bf16x8 ax[AG];
#pragma unroll
        for (int i = 0; i < AG; ++i) {
          const unsigned char* p = Ut + kt * 32 * RSB + (a0 + i) * 32;
          ax[i] = join8(ds_read_tr(reinterpret_cast<const bf16*>(p)),
                        ds_read_tr(reinterpret_cast<const bf16*>(p + 4 * RSB)));
        }
#pragma unroll
        for (int i = 0; i < AG; ++i) {
          U[a0 + i] = Mma<bf16>::run(ax[i], zhi, U[a0 + i]);
          U[a0 + i] = Mma<bf16>::run(ax[i], zlo, U[a0 + i]);
        }
      }
    }
  };

  // ---- walk the chunks (in order for dq, backwards for dk); the copies of
  // the next chunk go into the other buffer while this one computes
  auto chunk_of = [&](int st) { return rev ? NC - 1 - st : st; };
  if (loader) {
    issue(chunk_of(0), 0);
    wait_vm();
  }
  lds_barrier();
  for (int st = 0; st < NC; ++st) {
    const int b = st & 1;
    if (loader) {
      if (st + 1 < NC) {
        issue(chunk_of(st + 1), b ^ 1);
        wait_vm();
      }
    } else {
      body(chunk_of(st), b);
    }
    lds_barrier();  // the next chunk has landed; everyone is done with buffer b
  }
  if (loader) return;

  // ---- end of the walk
  if (J.fin_rs) {
    // dq job: U = hT^T; rowsum(hT ⊙ dhT) of the lane's channel
    float part = 0.f;
    if (J.fin_with) {
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        const f32x4 d = *reinterpret_cast<const f32x4*>(J.fin_with + ((size_t)bh * dk + icol) * DV + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) part += U[a][r] * d[r];
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0) J.fin_rs[(size_t)bh * dk + icol] = part;
  }
  if (J.fin_state) {
    // dk job: U = dS_{-1}^T = dh0^T
#pragma unroll
    for (int a = 0; a < NT; ++a)
      *reinterpret_cast<f32x4*>(J.fin_state + ((size_t)bh * dk + icol) * DV + 16 * a + 4 * g) = U[a];
  }
}

bool bwd_inter_supported(int bf16, int C, int dk, int dv, int L) {
  if (!bf16 || C != kBC || dk % kBW || dk < kBW || dk > 256) return false;
  if (dv != 128 && dv != 256) return false;
  // rows addressed with 32-bit byte offsets
  return (long long)L * dv * 2 <= 0x7fffffffLL && (long long)L * dk * 4 <= 0x7fffffffLL;
}

hipError_t launch_bwd_inter(const Plan& p, const BwdInterJob& jq, const BwdInterJob& jk,
                            const float* cum, hipStream_t s) {
  const int nper = p.BH * (p.dk / kBW);
  const dim3 grid(2 * nper), block(3 * kWave);
  if (p.dv == 256)
    hipLaunchKernelGGL(k_bwd_inter<256>, grid, block, 0, s, jq, jk, cum, p.L, p.dk, p.NC, nper);
  else if (p.dv == 128)
    hipLaunchKernelGGL(k_bwd_inter<128>, grid, block, 0, s, jq, jk, cum, p.L, p.dk, p.NC, nper);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gla
