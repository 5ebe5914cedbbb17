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
// cumsum of log alpha, b its last row).
//
// k_bwd_inter computes both without writing a single state: a workgroup
// walks the chunks of one (batch, head) with a 32-channel slice of the
// transposed state U = S^T (dq job, chunks in order) or U = dS^T (dk job,
// chunks in reverse order) in MFMA accumulators.  Per chunk it forms the
// output product X_y U (X_y = dO or V) scaled by Lambda or Gamma, writes it
// in fp32, and updates U by its column gates and X_u^T Z~ (X_u = V or dO;
// Z~ = k ⊙ Gamma or q ⊙ Lambda, formed from the chunk's k or q and cumsum).
//
// Precision: the closed-form gate gradient subtracts q ⊙ dq - k ⊙ dk, terms
// tens of times larger than their difference, so both products run with the
// fp32 operand (U, and Z~) split into a high and a low bf16 part (two MFMAs
// each); dO, V are exact in bf16.  The dq job also leaves rowsum(hT ⊙ dhT)
// (hT = its final state), the dk job dh0 = dS_{-1}.
//
// Gate-gradient sums: summed over the rows of a chunk, the intra-chunk parts
// of q ⊙ dq and k ⊙ dk cancel, so the chunk totals of the closed form come
// from the inter terms alone.  Each job multiplies its finished rows by q
// (dq job) or k (dk job), sums them over the rows and keeps a running sum
// over the chunks it has walked: an inclusive prefix (dq job) or an
// exclusive suffix (dk job), written per chunk and per half of its rows, so
// that the dq/dk kernel adds the carry over later chunks without a pass of
// its own over dlog alpha.
//
// Work split: four waves, each holding a 16-channel column block of U for
// one half of the d_v rows.  The output product is then a sum over d_v of
// two halves: each wave forms its half for all 64 rows, passes the rows its
// partner (the other half of the same column block) finishes through LDS,
// and after the chunk's barrier adds the partner's half of its own rows,
// scales and stores them.  The update needs no exchange (U's rows are
// independent).
//
// Staging: every wave copies its share of the next chunk's X_y and X_u rows
// (all d_v columns) and of the workgroup's 32 columns of Z's input (k or q)
// into LDS with LDS-DMA while it computes the current chunk (a double
// buffer); the cumsum values a lane needs are loaded into registers one
// chunk ahead.  The X rows are stored with a stride of one
// 16-byte unit more than a row (the extra unit is never read), so that every
// operand read is one per-lane base address plus a compile-time offset: the
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
constexpr int kBW = 32;   // key channels per workgroup (two column blocks)

template <int DV>
struct InterLayout {
  static constexpr int UPR = DV / 8;            // 16-byte units per X row
  static constexpr int RS = UPR + 1;            // units per staged row (one of padding)
  static constexpr int NTH = DV / 32;           // 16-row tiles of U per wave (half of d_v)
  static constexpr int TB = kBC * RS * 16;      // one staged X tile
  static constexpr int NCX = TB / 1024;         // 1 KB copies per X tile:
  static constexpr int CPW = DV / 32;           // CPW per wave, and one more by wave 0
  static constexpr int SB = kBC * kBW * 2;      // the chunk's 32 columns of k or q
  static constexpr int oY = 0, oU = TB, oS = 2 * TB, RBUF = 2 * TB + SB;
  // exchange of output halves: per parity, wave and tile 64 lanes x 16 B
  static constexpr int PB = 4 * 2 * 1024;
  static constexpr int oP = 2 * RBUF;
  // q or k at the rows each wave finishes (32 rows x 16 channels per wave)
  static constexpr int oT = 2 * RBUF + 2 * PB;
  static constexpr int LDS = oT + 4 * 1024;
  static_assert(UPR % 16 == 0, "rows of whole 256-byte bank spans");
  static_assert(LDS <= kLdsLimit, "staged chunk exceeds LDS");
  static_assert(TB % 1024 == 0 && NCX == 4 * CPW + 1 && SB == 4 * 1024,
                "1 KB copies, one of Z's input per wave");
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// The sums over the 16 lanes of a DPP row of four values, left in every lane
// of the row: quad permutations [1,0,3,2] and [2,3,0,1] sum each quad, the
// half-row mirror adds the neighbouring quad, the row mirror the other half.
// Written as one asm block rather than with the DPP builtin, which is
// convergent and so keeps the compiler from unrolling the chunk loop.  The
// four values interleave, so every DPP add reads a register written at least
// three instructions earlier; the block opens with the two wait states a
// DPP read of a just-written register needs.
__device__ inline void row16_sum4(f32x4& x) {
  float a = x[0], b = x[1], c = x[2], d = x[3];
#define GLA_DPP4(CTRL)                                                    \
  "v_add_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
  "v_add_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
  "v_add_f32_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
  "v_add_f32_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n"
  asm("s_nop 1\n" GLA_DPP4("quad_perm:[1,0,3,2]") GLA_DPP4("quad_perm:[2,3,0,1]")
          GLA_DPP4("row_half_mirror") GLA_DPP4("row_mirror")
      : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
#undef GLA_DPP4
  x[0] = a;
  x[1] = b;
  x[2] = c;
  x[3] = d;
}

__device__ inline bf16x4 lds_read8(const unsigned char* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}

// The accumulator pair (a, b) as an A operand (a's 4 values, then b's),
// split x = hi + lo: hi = x rounded to bf16, lo = the remainder rounded to
// bf16.  The remainder is formed from hi's bits (a shift or a mask of the
// packed pair), three instructions per value.
__device__ inline void split_pair(const floatx4& a, const floatx4& b, bf16x8& hi, bf16x8& lo) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  u32x4 hw, lw;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x0 = j < 2 ? a[2 * j] : b[2 * j - 4];
    const float x1 = j < 2 ? a[2 * j + 1] : b[2 * j - 3];
    bf16x2 h2;
    h2[0] = static_cast<bf16>(x0);
    h2[1] = static_cast<bf16>(x1);
    const unsigned hb = __builtin_bit_cast(unsigned, h2);
    bf16x2 l2;
    l2[0] = static_cast<bf16>(x0 - __uint_as_float(hb << 16));
    l2[1] = static_cast<bf16>(x1 - __uint_as_float(hb & 0xffff0000u));
    hw[j] = hb;
    lw[j] = __builtin_bit_cast(unsigned, l2);
  }
  hi = __builtin_bit_cast(bf16x8, hw);
  lo = __builtin_bit_cast(bf16x8, lw);
}

// The cumsum values of one chunk that a lane uses: B at the update's tokens
// (32 kt + 8 g + e, the lane's state column), at the last row (the lane's
// output channels and state column) and at the lane's two finished output
// rows (16 mb + n, mb = 2 h + t).
struct CumRegs {
  float bt[2][8];
  f32x4 blast;
  float bcol;
  f32x4 bm[2];
};

__device__ inline float ld_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline f32x4 ld_f32x4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace

// ============================================================ the inter terms
// One wave's walk over the chunks of (batch x head) bh, key channels
// [i0, i0 + 32): wave w holds column block w & 1 (16 key channels) for d_v
// half H = w >> 1; REV walks backwards (the dk job).
template <int DV, int H, bool REV>
__device__ __attribute__((always_inline)) inline void inter_walk(
    const BwdInterJob& J, const float* __restrict__ cum, int L, int dk, int NC, int bh, int i0,
    int w, unsigned char* lds) {
  using Lay = InterLayout<DV>;
  constexpr int UPR = Lay::UPR, NTH = Lay::NTH, CPW = Lay::CPW;
  constexpr int h = H;                     // d_v half: rows [h DV/2, (h + 1) DV/2)
  const int l = lane_id(), g = l >> 4, n = l & 15;
  const int wc = 16 * (w & 1);             // this wave's first channel in the slice
  const int icol = i0 + wc + n;            // this lane's state column (key channel)
  const int dv0 = h * (DV / 2);
  const unsigned lds0 = lds_addr(lds);

  // ---- the state: lane (g, n) of tile a holds U[dv0 + 16 a + 4 g + r][icol]
  floatx4 U[NTH];
#pragma unroll
  for (int a = 0; a < NTH; ++a) {
    U[a] = zero4();
    if (J.init)
      U[a] = *reinterpret_cast<const f32x4*>(J.init + ((size_t)bh * dk + icol) * DV + dv0 + 16 * a + 4 * g);
  }
  // The state registers are consumed here, before the chunk loop: a load
  // still pending into them at the loop's entry would otherwise make the
  // compiler wait for every outstanding memory operation (including the
  // previous chunk's output stores) at the top of each chunk.
#pragma unroll
  for (int a = 0; a < NTH; ++a) asm volatile("" ::"v"(U[a]));

  // ---- this wave's copies of one chunk into buffer b: X units c = w + 4 j
  // (j < CPW) and, in wave 0, c = NCX - 1 (staged unit s = 64 c + l is row
  // s / RS, unit s % RS; the padding unit takes a copy of the row's first
  // unit), and unit w of Z's input.  Rows past the end of the sequence repeat
  // its last row.
  const unsigned char* xy = reinterpret_cast<const unsigned char*>(J.xy) + (size_t)bh * L * DV * 2;
  const unsigned char* xu = reinterpret_cast<const unsigned char*>(J.xu) + (size_t)bh * L * DV * 2;
  const unsigned char* zs = reinterpret_cast<const unsigned char*>(J.z) + ((size_t)bh * L * dk + i0) * 2;
  const float* cs = cum + (size_t)bh * L * dk + i0;
  // the gate-gradient sums' input (q or k): each wave copies the rows it
  // finishes, 16 bytes per lane (row 32 h + l / 2, 8 channels), rows past the
  // end of the sequence repeating its last row (masked where they are used)
  const bool sums = J.tsum != nullptr;
  const unsigned char* ts_in =
      sums ? reinterpret_cast<const unsigned char*>(J.tin) + ((size_t)bh * L * dk + i0 + wc) * 2
           : nullptr;
  const unsigned tlds = lds0 + (unsigned)(Lay::oT + w * 1024);
  int xrow[CPW + 1], xcol[CPW + 1];
#pragma unroll
  for (int j = 0; j <= CPW; ++j) {
    const int s = 64 * (j < CPW ? w + 4 * j : Lay::NCX - 1) + l, unit = s % Lay::RS;
    xrow[j] = s / Lay::RS;
    xcol[j] = (unit < UPR ? unit : 0) * 16;
  }
  const int zrow = (64 * w + l) >> 2, zcol = ((64 * w + l) & 3) * 16;
  auto issue = [&](int nc, int b) __attribute__((always_inline)) {
    const int r0 = nc * kBC, rv = min(kBC, L - r0);
    const unsigned base = lds0 + (unsigned)(b * Lay::RBUF);
    const i32x4 ry = make_rsrc(xy + (size_t)r0 * DV * 2), ru = make_rsrc(xu + (size_t)r0 * DV * 2);
    const i32x4 rz = make_rsrc(zs + (size_t)r0 * dk * 2);
#pragma unroll
    for (int j = 0; j <= CPW; ++j) {
      if (j == CPW && w != 0) break;
      const int c = j < CPW ? w + 4 * j : Lay::NCX - 1;
      const unsigned off = (unsigned)(min(xrow[j], rv - 1) * (DV * 2) + xcol[j]);
      dma16b(ry, off, 0u, base + Lay::oY + (unsigned)c * 1024u);
      dma16b(ru, off, 0u, base + Lay::oU + (unsigned)c * 1024u);
    }
    dma16b(rz, (unsigned)(min(zrow, rv - 1) * dk * 2 + zcol), 0u, base + Lay::oS + (unsigned)w * 1024u);
  };
  // the lane's cumsum values of a chunk, through a buffer resource ending at
  // the chunk's last row (rows past the end of the sequence read 0)
  auto load_cum = [&](int nc, CumRegs& R) __attribute__((always_inline)) {
    const int r0 = nc * kBC, rv = min(kBC, L - r0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(cs + (size_t)r0 * dk), 0, (rv * dk - i0) * 4, 0x00020000);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 8; ++e) R.bt[kt][e] = ld_f32(rs, ((32 * kt + 8 * g + e) * dk + wc + n) * 4);
    R.blast = ld_f32x4(rs, ((rv - 1) * dk + wc + 4 * g) * 4);
    R.bcol = ld_f32(rs, ((rv - 1) * dk + wc + n) * 4);
#pragma unroll
    for (int t = 0; t < 2; ++t) R.bm[t] = ld_f32x4(rs, ((16 * (2 * h + t) + n) * dk + wc + 4 * g) * 4);
  };

  // Output stores through a buffer resource spanning the head's L rows: rows
  // past the end of the sequence fall outside it and are dropped.
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(J.out + (size_t)bh * L * dk, 0, L * dk * 4, 0x00020000);

  // ---- lane-constant parts of the operand addresses (bytes)
  constexpr int RSB = Lay::RS * 16;                    // staged row stride
  // output product: row m = 16 mb + n, units 4 a2 + (g >> 1) and + 2 of the
  // wave's half, half-unit g & 1
  const int yoff = n * RSB + (g >> 1) * 16 + (g & 1) * 8 + dv0 * 2;
  // update: rows 32 kt + 8 g + (n >> 2) and + 4, unit 2 a + ((n & 3) >> 1) of
  // the wave's half, half-unit n & 1
  const int uoff = (8 * g + (n >> 2)) * RSB + ((n & 3) >> 1) * 16 + (n & 1) * 8 + dv0 * 2;
  // exchange: this wave's outgoing tiles, and its partner's (w ^ 2) for it
  const int pout = Lay::oP + w * 2048 + l * 16, pin = Lay::oP + (w ^ 2) * 2048 + l * 16;

  CumRegs R;
  floatx4 Yk[2];  // the previous chunk's own output rows (this wave's half)
  f32x4 sf[2];    // ... and their scale factors
  f32x4 run = zero4();  // running gate-gradient sum of the lane's 4 channels
  int r0prev = 0;

  // add the partner's half to the rows this wave finishes, scale and store:
  // lane (g, n) holds rows 16 (2 h + t) + n, channels wc + 4 g + r
  auto finish = [&](int r0, int par) __attribute__((always_inline)) {
    f32x4 ts = zero4();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(lds + pin + par * Lay::PB + t * 1024);
      f32x4 y;
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = (Yk[t][r] + o[r]) * sf[t][r];
      const int m = 16 * (2 * h + t) + n;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, y), orsrc,
                                             ((r0 + m) * dk + i0 + wc + 4 * g) * 4, 0, 0);
      if (sums && r0 + m < L) {
        const bf16x4 x = lds_read8(lds + Lay::oT + w * 1024 + (16 * t + n) * 32 + 8 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) ts[r] += static_cast<float>(x[r]) * y[r];
      }
    }
    if (sums) {
      // over the 16 rows of the lane group, then into the running sum
      row16_sum4(ts);
      if (!REV) run += ts;
      if (n == 0)
        *reinterpret_cast<f32x4*>(J.tsum + (((size_t)bh * NC + r0 / kBC) * 2 + h) * dk + i0 + wc +
                                  4 * g) = run;
      if (REV) run += ts;
    }
  };

  // ---- walk the chunks (in order for dq, backwards for dk)
  auto chunk_of = [&](int st) { return REV ? NC - 1 - st : st; };
  load_cum(chunk_of(0), R);
  issue(chunk_of(0), 0);
  wait_vm();
  lds_barrier();
  for (int st = 0; st < NC; ++st) {
    const int b = st & 1, nc = chunk_of(st);
    const unsigned char* Yt = lds + b * Lay::RBUF + Lay::oY + yoff;
    const unsigned char* Ut = lds + b * Lay::RBUF + Lay::oU + uoff;
    const int r0 = nc * kBC, rv = min(kBC, L - r0);
    const bf16* Zs = reinterpret_cast<const bf16*>(lds + b * Lay::RBUF + Lay::oS);

    // The chunk's cumsum values were loaded during the previous step (whose
    // end waited for every load): consuming them here, before this step
    // issues its output stores, keeps the compiler's wait for them (it does
    // not see that wait) from also waiting for the stores.
    asm volatile("" ::"v"(R.bcol), "v"(R.blast), "v"(R.bm[0]), "v"(R.bm[1]));
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(R.bt[kt][e]));

    // From the chunk's cumsum: the column gate, the scale factors of the
    // rows this wave finishes (Lambda = e^{B} for dq, Gamma = e^{b - B} for
    // dk), and Z~ = k e^{b - B} (dq) or q e^{B} (dk), zero on rows past the
    // end of the sequence, split into high and low bf16 parts.
    const float gam = __expf(R.bcol);
    f32x4 sfn[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sfn[t][r] = __expf(REV ? R.blast[r] - R.bm[t][r] : R.bm[t][r]);
    bf16x8 zhi[2], zlo[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 zr = col_frag_tr(Zs, kBW, 32 * kt, wc, l);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 32 * kt + 8 * g + e;
        const float sc = __expf(REV ? R.bt[kt][e] : R.bcol - R.bt[kt][e]);
        const float val = tok < rv ? static_cast<float>(zr[e]) * sc : 0.f;
        zhi[kt][e] = static_cast<bf16>(val);
        zlo[kt][e] = static_cast<bf16>(val - static_cast<float>(zhi[kt][e]));
      }
    }

    // the previous chunk's rows (the partner's half came in last step); the
    // copies below (asm with a memory clobber) keep the stores this early,
    // so that they complete during the step
    if (st > 0) finish(r0prev, b ^ 1);

    // this chunk's q or k at the rows this wave finishes (used next step,
    // after finish above has read the previous chunk's: its sums are formed,
    // so those LDS reads have completed)
    if (sums) {
      asm volatile("" ::"v"(run));
      const int tr = min(r0 + 32 * h + (l >> 1), L - 1);
      dma16b(make_rsrc(ts_in), (unsigned)((tr * dk + 8 * (l & 1)) * 2), 0u, tlds);
    }
    // the next chunk's loads, into the other buffer and the cumsum registers
    if (st + 1 < NC) {
      load_cum(chunk_of(st + 1), R);
      issue(chunk_of(st + 1), b ^ 1);
    }

    // output: this wave's half of Y^T = U^T X_y^T over d_v; the accumulator
    // pair (2 a2, 2 a2 + 1) is the A operand (K index 8 g + e -> row
    // dv0 + 32 a2 + 4 g + e, or dv0 + 32 a2 + 16 + 4 g + e - 4), matched by
    // the units read from X_y
    floatx4 Y[kBC / 16];
#pragma unroll
    for (int mb = 0; mb < kBC / 16; ++mb) Y[mb] = zero4();
#pragma unroll
    for (int a2 = 0; a2 < NTH / 2; ++a2) {
      bf16x8 bx[kBC / 16];
#pragma unroll
      for (int mb = 0; mb < kBC / 16; ++mb) {
        const unsigned char* p = Yt + mb * 16 * RSB + a2 * 64;
        bx[mb] = join8(lds_read8(p), lds_read8(p + 32));
      }
      bf16x8 ahi, alo;
      split_pair(U[2 * a2], U[2 * a2 + 1], ahi, alo);
#pragma unroll
      for (int mb = 0; mb < kBC / 16; ++mb) {
        Y[mb] = Mma<bf16>::run(ahi, bx[mb], Y[mb]);
        Y[mb] = Mma<bf16>::run(alo, bx[mb], Y[mb]);
      }
    }
    // the partner's rows go out; this wave's stay for the next step
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      *reinterpret_cast<f32x4*>(lds + pout + b * Lay::PB + t * 1024) = Y[2 * (1 - h) + t];
      Yk[t] = Y[2 * h + t];
      sf[t] = sfn[t];
    }
    r0prev = r0;

    // update: U <- U diag(e^{b}) + X_u^T Z~ over this wave's rows
#pragma unroll
    for (int a = 0; a < NTH; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) U[a][r] *= gam;
#pragma unroll
    for (int kt = 0; kt < kBC / 32; ++kt) {
      constexpr int AG = 4;  // tiles whose operands are read before their products
#pragma unroll
      for (int a0 = 0; a0 < NTH; a0 += AG) {
        bf16x8 ax[AG];
#pragma unroll
        for (int i = 0; i < AG; ++i) {
          const unsigned char* p = Ut + kt * 32 * RSB + (a0 + i) * 32;
          ax[i] = join8(ds_read_tr(reinterpret_cast<const bf16*>(p)),
                        ds_read_tr(reinterpret_cast<const bf16*>(p + 4 * RSB)));
        }
#pragma unroll
        for (int i = 0; i < AG; ++i) {
          U[a0 + i] = Mma<bf16>::run(ax[i], zhi[kt], U[a0 + i]);
          U[a0 + i] = Mma<bf16>::run(ax[i], zlo[kt], U[a0 + i]);
        }
      }
    }

    // the next chunk has landed (this wave's copies), the exchange is
    // written, and everyone is done with buffer b
    wait_vm();
    lds_barrier();
  }
  finish(r0prev, (NC - 1) & 1);

  // ---- end of the walk
  if (J.fin_rs) {
    // dq job: U = hT^T; rowsum(hT ⊙ dhT) of the lane's channel, summed over
    // both halves of d_v (the staging buffers are free after the last
    // barrier)
    float part = 0.f;
    if (J.fin_with) {
#pragma unroll
      for (int a = 0; a < NTH; ++a) {
        const f32x4 d =
            *reinterpret_cast<const f32x4*>(J.fin_with + ((size_t)bh * dk + icol) * DV + dv0 + 16 * a + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) part += U[a][r] * d[r];
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    float* red = reinterpret_cast<float*>(lds);
    if (h == 1 && g == 0) red[wc + n] = part;
    lds_barrier();
    if (h == 0 && g == 0) J.fin_rs[(size_t)bh * dk + icol] = part + red[wc + n];
  }
  if (J.fin_state) {
    // dk job: U = dS_{-1}^T = dh0^T
#pragma unroll
    for (int a = 0; a < NTH; ++a)
      *reinterpret_cast<f32x4*>(J.fin_state + ((size_t)bh * dk + icol) * DV + dv0 + 16 * a + 4 * g) = U[a];
  }
}

// One job per half of the grid: workgroups [0, nper) run `jf` (dq), the rest
// `jk` (dk).
template <int DV>
__global__ __launch_bounds__(4 * kWave) void k_bwd_inter(BwdInterJob jf, BwdInterJob jk,
                                                         const float* __restrict__ cum, int L,
                                                         int dk, int NC, int nper) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[InterLayout<DV>::LDS];
  const bool second = blockIdx.x >= (unsigned)nper;
  const BwdInterJob& J = second ? jk : jf;
  const int bid = second ? (int)blockIdx.x - nper : (int)blockIdx.x;
  const int ntile = dk / kBW;
  const int lid = xcd_logical(bid, nper);
  const int bh = lid / ntile, i0 = (lid % ntile) * kBW;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  if (J.rev) {
    if (w >> 1) inter_walk<DV, 1, true>(J, cum, L, dk, NC, bh, i0, w, lds);
    else inter_walk<DV, 0, true>(J, cum, L, dk, NC, bh, i0, w, lds);
  } else {
    if (w >> 1) inter_walk<DV, 1, false>(J, cum, L, dk, NC, bh, i0, w, lds);
    else inter_walk<DV, 0, false>(J, cum, L, dk, NC, bh, i0, w, lds);
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
  const dim3 grid(2 * nper), block(4 * kWave);
  if (p.dv == 256)
    hipLaunchKernelGGL(k_bwd_inter<256>, grid, block, 0, s, jq, jk, cum, p.L, p.dk, p.NC, nper);
  else if (p.dv == 128)
    hipLaunchKernelGGL(k_bwd_inter<128>, grid, block, 0, s, jq, jk, cum, p.L, p.dk, p.NC, nper);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gla
