// gla_ggate.hip -- the general gate G_t = alpha_t^T beta_t (gfx950).
//
// Recurrence (papercache.org notes on GLA, App. C, general form; the row gate
// alpha acts on the d_k rows of the state, the column gate beta on its d_v
// columns):
//     S_t = (alpha_t^T beta_t) ⊙ S_{t-1} + k_t^T v_t,     o_t = q_t S_t.
// App. C.2 states that the chunkwise form carries over with both gates.  For
// a chunk of C = 16 tokens with chunk-local inclusive cumsums A (of log alpha,
// C x d_k) and Bt (of log beta, C x d_v) and chunk totals a, b:
//     O   = e^{Bt} ⊙ ((Q ⊙ e^{A}) S)                          (inter-chunk)
//         + e^{Bt - b} ⊙ (P (V ⊙ e^{b - Bt}))                 (intra-chunk)
//     S  <- diag(e^{a}) S diag(e^{b}) + (K ⊙ e^{a - A})^T (V ⊙ e^{b - Bt})
// with P[t][s] = sum_i q_t[i] k_s[i] e^{A_t[i] - A_s[i]} for s <= t, formed
// in log space (the notes' §4.3 secondary chunking keeps the diagonal blocks
// in full precision for the same reason).  Every factor is <= 1 except
// e^{Bt - b}, which is at most e^{-b}: the intra term takes the product form
// while a column's decay over the chunk stays under e^{60}, and a log-space
// sum per (t, s) pair for columns that decay faster (sharp beta gates).  The
// same-token term P[t][t] v_t (factor 1) is added separately in fp32: its
// operands need no rounding, and the backward's closed-form gate gradients
// are formed from outputs without it (the same-token parts of q ⊙ dq and
// k ⊙ dk, and of o ⊙ do and v ⊙ dv, are equal and cancel exactly).
//
// Two kernels per pass, as for the row-gated forward:
//   k_gg_prep  (chunk, batch-head): cumsum of log alpha, Q~ = Q e^{A},
//              K~ = K e^{a - A}, e^{a} and P, stored as MFMA fragments;
//   k_gg_recur (16-column tile, batch-head), one or two waves: the state
//              tile stays in MFMA accumulators across the chunks (its rows
//              split over two waves from 64 rows on); per chunk the inter
//              term (Q~ S), the intra term (P V~), the output, the decay and
//              the update (K~^T V~), with the beta cumsum formed across lanes
//              and the next chunks' operands loaded ahead.
// A pass can read its sequence backwards with the gates shifted by one token
// and take its initial state transposed; the backward is built from such
// passes (gla_api.hip).  Gate gradients come from the closed form of App. C
// (k_gg_gate_tot / k_gg_gate_fin).
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"  // xcd_logical

namespace gla {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;

constexpr int kGC = 16;            // tokens per chunk
constexpr float kSafeDecay = 60.f;  // product form while -b <= this
constexpr float kSafeP = 8.f;       // P on MFMA for channels decaying less than this

__device__ inline floatx4 mfma16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sequence position read by pass token u (-1: past the end).
__device__ inline int data_row(int u, int L, int rev) {
  if (u >= L) return -1;
  return rev ? L - 1 - u : u;
}
// Row of the gate applied at pass token u (-1: gate 1).  A reversed pass
// applies at token u the gate of original token L - u, and none at u = 0.
__device__ inline int gate_row(int u, int L, int rev) {
  if (u >= L) return -1;
  if (!rev) return u;
  return u == 0 ? -1 : L - u;
}

// Index of Q~[t][i] in the chunk's Q fragment record.  bf16 (16x16x32 A
// operand): [DKP/32][64 lanes][8]; lane t + 16 g, slot e < 4 holds channel
// 32 p + 4 g + e and slot e >= 4 channel 32 p + 16 + 4 g + e - 4, matching a B
// operand built from two accumulator tiles of the state.  fp32 (16x16x4, four
// steps per 16-row tile): [DKP/16][64][4], lane t + 16 g, slot s = channel
// 16 m + 4 g + s.
template <typename T> __device__ inline int qf_index(int t, int i);
template <> __device__ inline int qf_index<bf16>(int t, int i) {
  const int p = i >> 5, r = i & 31, hi = r >> 4, rr = r & 15;
  return ((p * 64 + t + 16 * (rr >> 2)) << 3) + 4 * hi + (rr & 3);
}
template <> __device__ inline int qf_index<float>(int t, int i) {
  const int m = i >> 4, r = i & 15;
  return ((m * 64 + t + 16 * (r >> 2)) << 2) + (r & 3);
}
// K~[t][i] as the A operand of the state update (rows i, K = tokens):
// [DKP/16][64][4], lane (i % 16) + 16 (t / 4), slot t % 4.
__device__ inline int kf_index(int t, int i) {
  return (((i >> 4) * 64 + (i & 15) + 16 * (t >> 2)) << 2) + (t & 3);
}
// s + err = a + b exactly (Knuth's two-sum).  The chunk-local cumsums are kept
// as hi + lo pairs so that a difference B_t - B_s, the exponent of a decay
// between two tokens, is accurate relative to its own size rather than to
// |B_t|, which sharp gates make hundreds of times larger.
__device__ inline float two_sum(float a, float b, float& err) {
  const float s = a + b, bp = s - a;
  err = (a - (s - bp)) + (b - bp);
  return s;
}
// The compensation serves fp32 operands (the backward's passes, whose gate
// gradients cancel); with bf16 operands it is below their rounding, and the
// lo parts fold away as zeros.
template <typename T> __device__ inline float csum(float a, float b, float& err) {
  if constexpr (sizeof(T) == 4) return two_sum(a, b, err);
  err = 0.f;
  return a + b;
}

// P[t][s] for s < t (zero on and above the diagonal): [64][4] fp32, lane
// t + 16 (s / 4), slot s % 4; then P[t][t], 16 fp32; then e^{a}, DKP fp32.
__device__ inline int pf_index(int t, int s) { return ((t + 16 * (s >> 2)) << 2) + (s & 3); }

}  // namespace

constexpr int kPfFloats = 256 + 16;  // P below the diagonal, then its diagonal

size_t gg_rec_bytes(int is_bf16, int dkp) {
  return (size_t)32 * dkp * (is_bf16 ? 2 : 4) + 4 * kPfFloats + (size_t)4 * dkp;
}

int gg_padded_dim(int is_bf16, int d) {
  for (int p = is_bf16 ? 32 : 16; p <= 256; p *= 2)
    if (d <= p) return p;
  return -1;
}

// grid (NC, BH), 256 threads.  dk: channels of the pass's q and k; dkp: the
// record's (padded) channel count.
// T: the record and arithmetic type; TI: the element type of q and k (bf16
// inputs of an fp32 pass are converted as they are read)
template <typename T, typename TI>
__global__ __launch_bounds__(kThreads) void k_gg_prep(const TI* __restrict__ q,
                                                      const TI* __restrict__ k,
                                                      const float* __restrict__ la,
                                                      uint8_t* __restrict__ rec, size_t rec_bytes,
                                                      int L, int dk, int dkp, int NC, int rev) {
  extern __shared__ float sm[];
  const int ld = dkp + 1;  // odd row stride: the P loop reads 16 rows at one column
  float* qs = sm;
  float* ks = qs + kGC * ld;
  float* cs = ks + kGC * ld;  // cumsum, hi part
  float* cl = cs + kGC * ld;  // lo part
  float* part = cl + kGC * ld;  // the four waves' partial P tiles
  uint32_t* umask = reinterpret_cast<uint32_t*>(part + 1024);  // channels left to the log-space sum
  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  if (tid < 8) umask[tid] = 0u;
  for (int x = tid; x < kGC * dkp; x += kThreads) {
    const int t = x / dkp, i = x - t * dkp, u = n * kGC + t;
    const int dr = data_row(u, L, rev), gr = gate_row(u, L, rev);
    const bool in = i < dk;
    qs[t * ld + i] = (in && dr >= 0) ? to_f32(q[((size_t)bh * L + dr) * dk + i]) : 0.f;
    ks[t * ld + i] = (in && dr >= 0) ? to_f32(k[((size_t)bh * L + dr) * dk + i]) : 0.f;
    cs[t * ld + i] = (in && gr >= 0) ? la[((size_t)bh * L + gr) * dk + i] : 0.f;
  }
  __syncthreads();
  uint8_t* r = rec + ((size_t)bh * NC + n) * rec_bytes;
  T* qf = reinterpret_cast<T*>(r);
  T* kf = qf + kGC * dkp;
  float* pf = reinterpret_cast<float*>(kf + kGC * dkp);
  float* ga = pf + kPfFloats;
  for (int i = tid; i < dkp; i += kThreads) {
    float c = 0.f, e = 0.f;
#pragma unroll
    for (int t = 0; t < kGC; ++t) {
      float err;
      c = csum<T>(c, cs[t * ld + i], err);
      e += err;
      cs[t * ld + i] = c;
      cl[t * ld + i] = e;
    }
    ga[i] = gexp<T>(c + e);
    if (cs[i] - c > kSafeP) atomicOr(&umask[i >> 5], 1u << (i & 31));
#pragma unroll
    for (int t = 0; t < kGC; ++t) {
      const float at = cs[t * ld + i], al = cl[t * ld + i];
      qf[qf_index<T>(t, i)] = from_f32<T>(qs[t * ld + i] * gexp<T>(at + al));
      kf[kf_index(t, i)] = from_f32<T>(ks[t * ld + i] * gexp<T>((c - at) + (e - al)));
    }
  }
  __syncthreads();
  // P[t][s] = sum_i q_t[i] k_s[i] e^{A_t[i] - A_s[i]}.  Channels whose decay
  // over the chunk stays under e^{kSafeP} take one fp32 MFMA tile with the
  // chunk's first row as reference, (q_t e^{A_t - A_0}) (k_s e^{A_0 - A_s}),
  // both exponents under kSafeP so that the product keeps fp32 accuracy;
  // each wave covers a quarter of the channels.  Faster-decaying channels
  // (sharp gates) take the per-pair log-space sum.
  {
    const int w = tid >> 6, l = tid & 63, r16 = l & 15, kk = l >> 4;
    const int span = dkp >> 2;
    floatx4 acc = zero4();
    for (int i0 = w * span; i0 < (w + 1) * span; i0 += 4) {
      const int i = i0 + kk;
      const bool sf = !((umask[i >> 5] >> (i & 31)) & 1u);
      const float c0 = cs[i], l0 = cl[i];
      const float a = sf ? qs[r16 * ld + i] *
                               gexp<T>((cs[r16 * ld + i] - c0) + (cl[r16 * ld + i] - l0))
                         : 0.f;
      const float b = sf ? ks[r16 * ld + i] *
                               gexp<T>((c0 - cs[r16 * ld + i]) + (l0 - cl[r16 * ld + i]))
                         : 0.f;
      acc = mfma4(a, b, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) part[w * 256 + (4 * kk + e) * 16 + r16] = acc[e];
  }
  __syncthreads();
  const int t = tid >> 4, s = tid & 15;
  float acc = 0.f;
  if (s <= t) {
    acc = part[tid] + part[256 + tid] + part[512 + tid] + part[768 + tid];
    const float* qt = qs + t * ld;
    const float* ksr = ks + s * ld;
    const float* ct = cs + t * ld;
    const float* csr = cs + s * ld;
    const float* lt = cl + t * ld;
    const float* lsr = cl + s * ld;
    for (int wd = 0; wd < ((dkp + 31) >> 5); ++wd)
      for (uint32_t m = umask[wd]; m; m &= m - 1) {
        const int i = wd * 32 + __builtin_ctz(m);
        acc += qt[i] * ksr[i] * gexp<T>((ct[i] - csr[i]) + (lt[i] - lsr[i]));
      }
  }
  pf[pf_index(t, s)] = s < t ? acc : 0.f;
  if (s == t) pf[256 + t] = acc;
}

// Fragments of one chunk's records for one lane.
template <typename T, int MT> struct GgFrag;
template <int MT> struct GgFrag<bf16, MT> {
  bf16x8 q[MT / 2];
  bf16x4 k[MT];
};
template <int MT> struct GgFrag<float, MT> {
  f4 q[MT];
  f4 k[MT];
};

template <int MT>
__device__ inline void load_q(GgFrag<bf16, MT>& f, const bf16* qf, int l) {
#pragma unroll
  for (int p = 0; p < MT / 2; ++p) f.q[p] = *reinterpret_cast<const bf16x8*>(qf + ((p * 64 + l) << 3));
}
template <int MT>
__device__ inline void load_q(GgFrag<float, MT>& f, const float* qf, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m) f.q[m] = *reinterpret_cast<const f4*>(qf + ((m * 64 + l) << 2));
}
template <int MT>
__device__ inline void load_k(GgFrag<bf16, MT>& f, const bf16* kf, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m) f.k[m] = *reinterpret_cast<const bf16x4*>(kf + ((m * 64 + l) << 2));
}
template <int MT>
__device__ inline void load_k(GgFrag<float, MT>& f, const float* kf, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m) f.k[m] = *reinterpret_cast<const f4*>(kf + ((m * 64 + l) << 2));
}

// acc += Q~ S (16 tokens x 16 columns), S in accumulator layout.
template <int MT>
__device__ inline floatx4 inter(const GgFrag<bf16, MT>& f, const floatx4 (&S)[MT]) {
  floatx4 acc = zero4();
#pragma unroll
  for (int p = 0; p < MT / 2; ++p) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = static_cast<bf16>(S[2 * p][e]);
      b[4 + e] = static_cast<bf16>(S[2 * p + 1][e]);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.q[p], b, acc, 0, 0, 0);
  }
  return acc;
}
template <int MT>
__device__ inline floatx4 inter(const GgFrag<float, MT>& f, const floatx4 (&S)[MT]) {
  floatx4 acc = zero4();
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma4(f.q[m][s], S[m][s], acc);
  return acc;
}

// P V~ (16 x 16): P in fp32 (hi + lo for bf16 operands), V~ in accumulator
// layout (lane (j, g) holds tokens 4 g .. 4 g + 3 of column j).
__device__ inline floatx4 intra(const f4& p, const floatx4& vt, bf16) {
  bf16x4 hi, lo, vb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = static_cast<bf16>(p[e]);
    lo[e] = static_cast<bf16>(p[e] - static_cast<float>(hi[e]));
    vb[e] = static_cast<bf16>(vt[e]);
  }
  return mfma16(lo, vb, mfma16(hi, vb, zero4()));
}
__device__ inline floatx4 intra(const f4& p, const floatx4& vt, float) {
  floatx4 acc = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma4(p[s], vt[s], acc);
  return acc;
}

// S += K~^T V~
template <int MT>
__device__ inline void update(floatx4 (&S)[MT], const GgFrag<bf16, MT>& f, const floatx4& vt) {
  bf16x4 vb;
#pragma unroll
  for (int e = 0; e < 4; ++e) vb[e] = static_cast<bf16>(vt[e]);
#pragma unroll
  for (int m = 0; m < MT; ++m) S[m] = mfma16(f.k[m], vb, S[m]);
}
template <int MT>
__device__ inline void update(floatx4 (&S)[MT], const GgFrag<float, MT>& f, const floatx4& vt) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int s = 0; s < 4; ++s) S[m] = mfma4(f.k[m][s], vt[s], S[m]);
}

// Everything one lane reads for one chunk; the recurrence loads chunk n + 1
// into a second set while it computes chunk n.  From 128 state rows on the
// second set would not fit in registers: with 128 rows of bf16 operands only
// the operands needed first (Q~, P, v, log beta) are loaded ahead, and K~ and
// e^{a}, needed last, at the start of their own chunk; past that nothing is
// loaded ahead (values parked in accumulator registers would cost a wait on
// every load in flight), and each chunk's loads are issued together.
template <typename T, int MT> struct GgIn {
  GgFrag<T, MT> f;
  f4 p, pd;     // P below the diagonal (A fragment), P[4g + e][4g + e]
  f4 ga[MT];    // e^{a} at the lane's state rows
  float v[4], lb[4];
};

// 2: all of chunk n + 1 loaded ahead; 1: the early operands; 0: nothing
template <typename T, int MT> constexpr int gg_ahead() {
  return MT <= 4 ? 2 : (MT == 8 ? 1 : 0);
}
// Chunks loaded ahead when everything is (gg_ahead == 2): two for bf16 state
// slices of up to 64 rows (a chunk step is shorter than the memory latency),
// else one.
template <typename T, int MT> constexpr int gg_depth() {
  return (sizeof(T) == 2 && MT <= 4) ? 2 : 1;
}

// MT: the wave's tiles; DKP: the record's channels; m0: the wave's first tile
template <typename T, int MT>
__device__ inline void gg_load_late(GgIn<T, MT>& in, const uint8_t* __restrict__ rec,
                                    size_t rec_bytes, int DKP, int m0, int bh, int n, int NC,
                                    int l, int g) {
  const T* kf = reinterpret_cast<const T*>(rec + ((size_t)bh * NC + n) * rec_bytes) + kGC * DKP;
  const float* pf = reinterpret_cast<const float*>(kf + kGC * DKP);
  load_k(in.f, kf + 256 * m0, l);
#pragma unroll
  for (int m = 0; m < MT; ++m)
    in.ga[m] = *reinterpret_cast<const f4*>(pf + kPfFloats + 16 * (m0 + m) + 4 * g);
}

template <typename T, int MT, typename TI>
__device__ inline void gg_load(GgIn<T, MT>& in, const uint8_t* __restrict__ rec, size_t rec_bytes,
                               int DKP, int m0, const TI* __restrict__ vb,
                               const float* __restrict__ lbb, int bh, int n, int NC, int L,
                               int dv, int rev, int l, int g) {
  const uint8_t* r = rec + ((size_t)bh * NC + n) * rec_bytes;
  const T* qf = reinterpret_cast<const T*>(r);
  const float* pf = reinterpret_cast<const float*>(qf + 2 * kGC * DKP);
  load_q(in.f, qf + 256 * m0, l);  // 256 elements per 16-channel tile in both layouts
  in.p = *reinterpret_cast<const f4*>(pf + 4 * l);
  in.pd = *reinterpret_cast<const f4*>(pf + 256 + 4 * g);
  if constexpr (gg_ahead<T, MT>() == 2) gg_load_late(in, rec, rec_bytes, DKP, m0, bh, n, NC, l, g);
  // unconditional loads of a clamped row, kept raw: a load under a branch, or
  // a select on its value here, would wait for it at once; the rows past the
  // sequence are zeroed where the values are used (gg_valid)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int u = n * kGC + 4 * g + e;
    const int dr = data_row(u, L, rev), gr = gate_row(u, L, rev);
    in.v[e] = to_f32(vb[(size_t)(dr > 0 ? dr : 0) * dv]);
    in.lb[e] = lbb[(size_t)(gr > 0 ? gr : 0) * dv];
  }
}

// v and log beta of chunk n as loaded by gg_load, with the rows that have no
// value (past the sequence) or no gate (the first row of a reversed pass)
// set to zero.
template <typename T, int MT>
__device__ inline void gg_valid(const GgIn<T, MT>& in, int n, int L, int rev, int g, float* v,
                                float* lb) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int u = n * kGC + 4 * g + e;
    v[e] = data_row(u, L, rev) >= 0 ? in.v[e] : 0.f;
    lb[e] = gate_row(u, L, rev) >= 0 ? in.lb[e] : 0.f;
  }
}

// grid (dv / 16 * BH), NWR waves per workgroup; the dv / 16 column tiles of a
// (batch, head), which read the same chunk records, take consecutive logical
// ids placed on one XCD so that its L2 serves their repeated reads.  The NWR
// waves split the state tile's MT 16-row blocks between them (twice the waves
// of one per tile, half the per-chunk work each): each forms its share of the
// inter term Q~ S, the others hand theirs to wave 0 through LDS, and wave 0
// adds the intra term and writes the output; each wave decays and updates its
// own rows.  Lane (j, g) = (l % 16, l / 16) owns state column j of the tile
// and, in every 16 x 16 accumulator tile, rows 4 g + e.
// init: [BH][dk][dv] ([BH][dv][dk] when init_t), or null for zeros.  o (if
// not null) receives the output, ooff (if not null) the output without the
// same-token term, in fp32.  fin (if not null) receives the final state
// [BH][dk][dv], first multiplied by the gate of sequence token 0 when
// fin_la / fin_lb are given.
template <typename T, typename TO, int MT, int NWR, typename TI>
__global__ __launch_bounds__(kWave * NWR) void k_gg_recur(
    const uint8_t* __restrict__ rec, size_t rec_bytes, const TI* __restrict__ v,
    const float* __restrict__ lb, const float* __restrict__ init, int init_t,
    TO* __restrict__ o, float* __restrict__ ooff, float* __restrict__ fin,
    const float* __restrict__ fin_la,
    const float* __restrict__ fin_lb, int L, int dk, int dv, int NC, int rev) {
  constexpr int DKP = MT * 16, MTW = MT / NWR;
  static_assert(MT % NWR == 0 && (sizeof(T) == 4 || MTW % 2 == 0), "row split");
  __shared__ f4 red[2][NWR > 1 ? NWR - 1 : 1][kWave];  // partial inter terms
  const int w = threadIdx.x / kWave, l = threadIdx.x & (kWave - 1), j = l & 15, g = l >> 4;
  const int m0 = w * MTW;
  const int nt = dv / 16, lid = xcd_logical(blockIdx.x, gridDim.x);
  const int bh = lid / nt, jc = (lid - bh * nt) * 16 + j;
  floatx4 S[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * (m0 + m) + 4 * g + e;
      float x = 0.f;
      if (init && row < dk)
        x = init_t ? init[((size_t)bh * dv + jc) * dk + row] : init[((size_t)bh * dk + row) * dv + jc];
      S[m][e] = x;
    }
  const TI* vb = v + (size_t)bh * L * dv + jc;
  const float* lbb = lb + (size_t)bh * L * dv + jc;

  constexpr int AHEAD = gg_ahead<T, MTW>(), DEPTH = AHEAD == 2 ? gg_depth<T, MTW>() : 1;
  // One chunk step: chunk n from `cur`; first the loads of chunk `nl` (if in
  // range) go into `ld`.  The loop below is unrolled by the number of register
  // sets so that the sets change roles without copies: a copy of a register
  // whose load is in flight would wait for that load.
  auto step = [&](int n, GgIn<T, MTW>& cur, GgIn<T, MTW>& ld, int nl) {
    if constexpr (AHEAD == 0)
      gg_load(cur, rec, rec_bytes, DKP, m0, vb, lbb, bh, n, NC, L, dv, rev, l, g);
    if constexpr (AHEAD < 2) gg_load_late(cur, rec, rec_bytes, DKP, m0, bh, n, NC, l, g);
    // the prefetch is unconditional (past the end it reloads the last chunk,
    // unused): under a branch, the wait counts at its join would force waits
    // on the current set's loads as well
    if constexpr (AHEAD > 0)
      gg_load(ld, rec, rec_bytes, DKP, m0, vb, lbb, bh, nl < NC ? nl : NC - 1, NC, L, dv, rev, l, g);
    const GgFrag<T, MTW>& f = cur.f;
    const f4 p = cur.p, pd = cur.pd;
    const float* pf = reinterpret_cast<const float*>(
        rec + ((size_t)bh * NC + n) * rec_bytes + (size_t)32 * DKP * sizeof(T));
    float vv[4], c[4];
    gg_valid(cur, n, L, rev, g, vv, c);
    // chunk-local inclusive cumsum of log beta down the 16 rows of column j,
    // as hi (c) + lo (cl) pairs: within the lane's 4 rows, then the totals of
    // the lanes above it (row groups g' < g) added in front
    float cl[4], err;
    cl[0] = 0.f;
#pragma unroll
    for (int e = 1; e < 4; ++e) {
      c[e] = csum<T>(c[e - 1], c[e], err);
      cl[e] = cl[e - 1] + err;
    }
    float th[4], tl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      th[r] = __shfl(c[3], j + 16 * r);
      tl[r] = sizeof(T) == 4 ? __shfl(cl[3], j + 16 * r) : 0.f;
    }
    float eh = 0.f, el = 0.f;  // sum of the totals of row groups before g
    float bh_ = 0.f, bl_ = 0.f;  // chunk total
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < g) {
        eh = csum<T>(eh, th[r], err);
        el += tl[r] + err;
      }
      bh_ = csum<T>(bh_, th[r], err);
      bl_ += tl[r] + err;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = csum<T>(eh, c[e], err);
      cl[e] += el + err;
    }
    const float bt = bh_ + bl_;  // chunk total (rounded)
    floatx4 vt;
#pragma unroll
    for (int e = 0; e < 4; ++e) vt[e] = vv[e] * gexp<T>((bh_ - c[e]) + (bl_ - cl[e]));
    floatx4 a1 = inter(f, S);
    if constexpr (NWR > 1) {
      if (w > 0) red[n & 1][w - 1][l] = a1;
      __syncthreads();  // one per chunk: the buffers alternate, and the next
                        // write to this one comes after the next barrier
      if (w == 0)
#pragma unroll
        for (int r = 0; r < NWR - 1; ++r) {
          const f4 x = red[n & 1][r][l];
#pragma unroll
          for (int e = 0; e < 4; ++e) a1[e] += x[e];
        }
    }
    if (w == 0) {  // wave 0: intra term and output
      const floatx4 a2 = intra(p, vt, T());
      float res[4];
      const bool safe = bt >= -kSafeDecay;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        res[e] = gexp<T>(c[e] + cl[e]) * a1[e] + gexp<T>((c[e] - bh_) + (cl[e] - bl_)) * a2[e];
      if (__any(!safe)) {
        // log-space intra term: sum_{s < t} P[t][s] v_s e^{Bt_t - Bt_s}
        float sl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kGC; ++s) {
          const int src = j + 16 * (s >> 2);
          const float cs = __shfl(c[s & 3], src);
          const float ls = sizeof(T) == 4 ? __shfl(cl[s & 3], src) : 0.f;
          const float vs = __shfl(vv[s & 3], src);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * g + e;
            if (s < t) sl[e] += pf[pf_index(t, s)] * vs * gexp<T>((c[e] - cs) + (cl[e] - ls));
          }
        }
        if (!safe)
#pragma unroll
          for (int e = 0; e < 4; ++e) res[e] = gexp<T>(c[e] + cl[e]) * a1[e] + sl[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dr = data_row(n * kGC + 4 * g + e, L, rev);
        if (dr < 0) continue;
        const size_t x = ((size_t)bh * L + dr) * dv + jc;
        if (ooff) ooff[x] = res[e];
        if (o) o[x] = from_f32<TO>(res[e] + pd[e] * vv[e]);
      }
    }
    // decay and update
    const float gb = gexp<T>(bt);
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] *= cur.ga[m][e] * gb;
    update(S, f, vt);
  };
  GgIn<T, MTW> ra, rb, rc;
  if constexpr (AHEAD == 0) {
    for (int n = 0; n < NC; ++n) step(n, ra, ra, NC);
  } else if constexpr (DEPTH == 1) {
    gg_load(ra, rec, rec_bytes, DKP, m0, vb, lbb, bh, 0, NC, L, dv, rev, l, g);
    for (int n = 0; n < NC; n += 2) {
      step(n, ra, rb, n + 1);
      if (n + 1 < NC) step(n + 1, rb, ra, n + 2);
    }
  } else {
    gg_load(ra, rec, rec_bytes, DKP, m0, vb, lbb, bh, 0, NC, L, dv, rev, l, g);
    gg_load(rb, rec, rec_bytes, DKP, m0, vb, lbb, bh, NC > 1 ? 1 : 0, NC, L, dv, rev, l, g);
    for (int n = 0; n < NC; n += 3) {
      step(n, ra, rc, n + 2);
      if (n + 1 < NC) step(n + 1, rb, ra, n + 3);
      if (n + 2 < NC) step(n + 2, rc, rb, n + 4);
    }
  }
  if (fin) {
    const float gb = fin_lb ? gexp<T>(fin_lb[(size_t)bh * L * dv + jc]) : 1.f;
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (m0 + m) + 4 * g + e;
        if (row < dk) {
          const float gr = fin_la ? gexp<T>(fin_la[(size_t)bh * L * dk + row]) * gb : 1.f;
          fin[((size_t)bh * dk + row) * dv + jc] = S[m][e] * gr;
        }
      }
  }
}

// Closed-form gate gradients (App. C): per token,
//   dlog b_t = q_t ⊙ dq_t - k_t ⊙ dk_t       (d_k channels, alpha)
//   dlog d_t = o_t ⊙ do_t - v_t ⊙ dv_t       (d_v channels, beta)
// and each dlog gate is the sum over later tokens, plus the row / column sums
// of hT ⊙ dhT.  dq, dk, dv and o enter without their same-token terms, whose
// contributions to the two differences are equal and cancel exactly; what is
// left is the part that the gates decay.  Chunks of kGT tokens: totals first,
// then the carry-in.
constexpr int kGT = 64;

template <typename T>
__device__ inline float gg_term(int c, size_t row, int dk, int dv, const T* q, const T* k,
                                const float* dq, const float* dkk, const float* o32,
                                const T* dout, const T* v, const float* dvv) {
  if (c < dk) {
    const size_t x = row * dk + c;
    return to_f32(q[x]) * dq[x] - to_f32(k[x]) * dkk[x];
  }
  const size_t x = row * dv + (c - dk);
  return o32[x] * to_f32(dout[x]) - to_f32(v[x]) * dvv[x];
}

// grid (ceil(L / kGT), BH); tot [BH][NG][dk + dv]
template <typename T>
__global__ __launch_bounds__(kThreads) void k_gg_gate_tot(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ dq,
    const float* __restrict__ dkk, const float* __restrict__ o32, const T* __restrict__ dout,
    const T* __restrict__ v, const float* __restrict__ dvv, float* __restrict__ tot, int L,
    int dk, int dv) {
  const int cg = blockIdx.x, bh = blockIdx.y, NG = gridDim.x, D = dk + dv;
  const int t0 = cg * kGT, t1 = min(L, t0 + kGT);
  for (int c = threadIdx.x; c < D; c += kThreads) {
    float s = 0.f;
    for (int t = t0; t < t1; ++t)
      s += gg_term(c, (size_t)bh * L + t, dk, dv, q, k, dq, dkk, o32, dout, v, dvv);
    tot[((size_t)bh * NG + cg) * D + c] = s;
  }
}

// grid (BH); hs [BH][dk + dv] = row sums, then column sums, of hT ⊙ dhT
__global__ __launch_bounds__(kThreads) void k_gg_hsum(const float* __restrict__ hT,
                                                      const float* __restrict__ dhT,
                                                      float* __restrict__ hs, int dk, int dv) {
  const int bh = blockIdx.x;
  const float* h = hT + (size_t)bh * dk * dv;
  const float* d = dhT + (size_t)bh * dk * dv;
  for (int c = threadIdx.x; c < dk + dv; c += kThreads) {
    float s = 0.f;
    if (c < dk)
      for (int j = 0; j < dv; ++j) s += h[(size_t)c * dv + j] * d[(size_t)c * dv + j];
    else
      for (int i = 0; i < dk; ++i) s += h[(size_t)i * dv + c - dk] * d[(size_t)i * dv + c - dk];
    hs[(size_t)bh * (dk + dv) + c] = s;
  }
}

// grid (ceil(L / kGT), BH): dlog alpha and dlog beta
template <typename T>
__global__ __launch_bounds__(kThreads) void k_gg_gate_fin(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ dq,
    const float* __restrict__ dkk, const float* __restrict__ o32, const T* __restrict__ dout,
    const T* __restrict__ v, const float* __restrict__ dvv, const float* __restrict__ tot,
    const float* __restrict__ hs, float* __restrict__ dla, float* __restrict__ dlb, int L,
    int dk, int dv) {
  const int cg = blockIdx.x, bh = blockIdx.y, NG = gridDim.x, D = dk + dv;
  const int t0 = cg * kGT, t1 = min(L, t0 + kGT);
  for (int c = threadIdx.x; c < D; c += kThreads) {
    float run = hs ? hs[(size_t)bh * D + c] : 0.f;
    for (int g2 = cg + 1; g2 < NG; ++g2) run += tot[((size_t)bh * NG + g2) * D + c];
    for (int t = t1 - 1; t >= t0; --t) {
      const size_t row = (size_t)bh * L + t;
      run += gg_term(c, row, dk, dv, q, k, dq, dkk, o32, dout, v, dvv);
      if (c < dk) dla[row * dk + c] = run;
      else dlb[row * dv + c - dk] = run;
    }
  }
}

// ---- launchers ----

// Waves per state tile: two from 64 state rows on (32 for fp32), one below.
template <typename T> constexpr int gg_row_split(int MT) { return MT >= (sizeof(T) == 2 ? 4 : 2) ? 2 : 1; }

template <typename T, typename TO, typename TI>
static void launch_gg_recur(const GgPass& ps, int dkp, dim3 grid, const uint8_t* r, size_t rb,
                            int L, int NC, hipStream_t s) {
#define GG_RECUR(MT)                                                                          \
  hipLaunchKernelGGL((k_gg_recur<T, TO, MT, gg_row_split<T>(MT), TI>), grid,                    \
                     dim3(kWave * gg_row_split<T>(MT)), 0, s, r, rb, (const TI*)ps.v,          \
                     ps.lb, ps.init, ps.init_t, (TO*)ps.o, ps.o_off, ps.fin, ps.fin_la,       \
                     ps.fin_lb, L,                                                            \
                     ps.dk, ps.dv, NC, ps.rev)
  if constexpr (sizeof(T) == 4) {
    if (dkp == 16) { GG_RECUR(1); return; }
  }
  if (dkp == 32) GG_RECUR(2);
  else if (dkp == 64) GG_RECUR(4);
  else if (dkp == 128) GG_RECUR(8);
  else GG_RECUR(16);
#undef GG_RECUR
}

// part 0: k_gg_prep, part 1: k_gg_recur (separate so that each launch can be
// timed on its own).  is_bf16: the pass's records and arithmetic; in_bf16: the
// element type of its q, k and v (bf16 inputs may feed an fp32 pass).
template <typename T, typename TI>
static void launch_gg_prep(const GgPass& ps, dim3 pg, size_t lds, uint8_t* r, size_t rb, int L,
                           int dkp, int NC, hipStream_t s) {
  hipLaunchKernelGGL((k_gg_prep<T, TI>), pg, dim3(kThreads), lds, s, (const TI*)ps.q,
                     (const TI*)ps.k, ps.la, r, rb, L, ps.dk, dkp, NC, ps.rev);
}

template <typename T, typename TI>
static hipError_t gg_prep_lds(size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)k_gg_prep<T, TI>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_gg_pass(const GgPass& ps, int part, int is_bf16, int in_bf16, int BH, int L,
                          void* rec, hipStream_t s) {
  const int NC = (L + kGC - 1) / kGC;
  const int dkp = gg_padded_dim(is_bf16, ps.dk);
  if (dkp < 0 || ps.dv % 16 || BH <= 0 || NC <= 0 || (is_bf16 && !in_bf16))
    return hipErrorInvalidValue;
  const size_t rb = gg_rec_bytes(is_bf16, dkp);
  uint8_t* r = static_cast<uint8_t*>(rec);
  if (part == 0) {
    // 4 arrays of 16 padded rows, 4 partial P tiles, 8 mask words: 69.9 KB at 256 channels
    const size_t lds = sizeof(float) * (4 * kGC * (dkp + 1) + 1024 + 8);
    const dim3 pg(NC, BH);
    hipError_t e;
    if (is_bf16) {
      if ((e = gg_prep_lds<bf16, bf16>(lds)) != hipSuccess) return e;
      launch_gg_prep<bf16, bf16>(ps, pg, lds, r, rb, L, dkp, NC, s);
    } else if (in_bf16) {
      if ((e = gg_prep_lds<float, bf16>(lds)) != hipSuccess) return e;
      launch_gg_prep<float, bf16>(ps, pg, lds, r, rb, L, dkp, NC, s);
    } else {
      if ((e = gg_prep_lds<float, float>(lds)) != hipSuccess) return e;
      launch_gg_prep<float, float>(ps, pg, lds, r, rb, L, dkp, NC, s);
    }
  } else {
    const dim3 rg((ps.dv / 16) * BH);
    // o is written in the element type of the inputs (o_off, when asked
    // for, in fp32)
    if (is_bf16) launch_gg_recur<bf16, bf16, bf16>(ps, dkp, rg, r, rb, L, NC, s);
    else if (in_bf16) launch_gg_recur<float, bf16, bf16>(ps, dkp, rg, r, rb, L, NC, s);
    else launch_gg_recur<float, float, float>(ps, dkp, rg, r, rb, L, NC, s);
  }
  return hipGetLastError();
}

size_t gg_pass_rec_bytes(int is_bf16, int BH, int L, int d) {
  const int dkp = gg_padded_dim(is_bf16, d);
  if (dkp < 0) return 0;
  return gg_rec_bytes(is_bf16, dkp) * (size_t)BH * ((L + kGC - 1) / kGC);
}

int gg_gate_groups(int L) { return (L + kGT - 1) / kGT; }

hipError_t launch_gg_gates(int is_bf16, int BH, int L, int dk, int dv, const void* q,
                           const void* k, const float* dq32, const float* dk32, const float* o32,
                           const void* dout, const void* v, const float* dv32, const float* hT,
                           const float* dhT, float* tot, float* hs, float* dla, float* dlb,
                           hipStream_t s) {
  const dim3 grid(gg_gate_groups(L), BH);
  if (dhT) hipLaunchKernelGGL(k_gg_hsum, dim3(BH), dim3(kThreads), 0, s, hT, dhT, hs, dk, dv);
  const float* hsp = dhT ? hs : nullptr;
  if (is_bf16) {
    hipLaunchKernelGGL((k_gg_gate_tot<bf16>), grid, dim3(kThreads), 0, s, (const bf16*)q,
                       (const bf16*)k, dq32, dk32, o32, (const bf16*)dout, (const bf16*)v, dv32,
                       tot, L, dk, dv);
    hipLaunchKernelGGL((k_gg_gate_fin<bf16>), grid, dim3(kThreads), 0, s, (const bf16*)q,
                       (const bf16*)k, dq32, dk32, o32, (const bf16*)dout, (const bf16*)v, dv32,
                       tot, hsp, dla, dlb, L, dk, dv);
  } else {
    hipLaunchKernelGGL((k_gg_gate_tot<float>), grid, dim3(kThreads), 0, s, (const float*)q,
                       (const float*)k, dq32, dk32, o32, (const float*)dout, (const float*)v,
                       dv32, tot, L, dk, dv);
    hipLaunchKernelGGL((k_gg_gate_fin<float>), grid, dim3(kThreads), 0, s, (const float*)q,
                       (const float*)k, dq32, dk32, o32, (const float*)dout, (const float*)v,
                       dv32, tot, hsp, dla, dlb, L, dk, dv);
  }
  return hipGetLastError();
}

}  // namespace gla
