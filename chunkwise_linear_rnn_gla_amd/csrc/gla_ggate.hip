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
// (k_gg_gate_scan, k_gg_gate_carry, k_gg_gate_add).
#include "gla_common.h"
#include "gla_internal.h"
#include "gla_pblock.h"  // xcd_logical, load8

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

// One channel's 16 staged tokens as fp32, in 16-byte LDS units.
__device__ inline void lds16(const float* p, float* o) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * j);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[4 * j + e] = v[e];
  }
}
__device__ inline void lds16(const bf16* p, float* o) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 8 * j);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[8 * j + e] = static_cast<float>(v[e]);
  }
}
__device__ inline void sts16(float* p, const float* x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[4 * j + e];
    *reinterpret_cast<f32x4*>(p + 4 * j) = v;
  }
}
// State rows of a pass: up to 256 with bf16 records; the fp32 passes of the
// backward whose rows are the d_v channels take up to 512.
constexpr int kMaxRowsF32 = 512, kMaskWords = kMaxRowsF32 / 32;

size_t gg_rec_bytes(int is_bf16, int dkp) {
  return (size_t)32 * dkp * (is_bf16 ? 2 : 4) + 4 * kPfFloats + (size_t)4 * dkp;
}

int gg_padded_dim(int is_bf16, int d) {
  for (int p = is_bf16 ? 32 : 16; p <= (is_bf16 ? 256 : kMaxRowsF32); p *= 2)
    if (d <= p) return p;
  return -1;
}

// grid (NC, BH), 256 threads.  dk: channels of the pass's q and k; dkp: the
// record's (padded) channel count.
// T: the record and arithmetic type; TI: the element type of q and k (bf16
// inputs of an fp32 pass are converted as they are read); QS: the type q and
// k are staged in (TI, or fp32)
template <typename T, typename TI, typename QS>
__global__ __launch_bounds__(kThreads) void k_gg_prep(const TI* __restrict__ q,
                                                      const TI* __restrict__ k,
                                                      const float* __restrict__ la,
                                                      uint8_t* __restrict__ rec, size_t rec_bytes,
                                                      int L, int dk, int dkp, int NC, int rev) {
  extern __shared__ float sm[];
  // The chunk's q, k and cumsum are staged channel-major, [dkp][16]: a
  // channel's 16 tokens are contiguous (the per-channel cumsum reads and
  // writes them in 16-byte units), and the P loop's 64 lanes (16 tokens of 4
  // channels) read 64 consecutive words.
  // q and k staged in QS: bf16 inputs are exact in bf16, half the LDS of an
  // fp32 copy, which lets the 256-channel passes fit one more workgroup per
  // CU (below 256 channels fp32 staging measured faster)
  QS* qs = reinterpret_cast<QS*>(sm);
  QS* ks = qs + kGC * dkp;
  float* cs = reinterpret_cast<float*>(ks + kGC * dkp);  // cumsum, hi part
  // lo part of the cumsum: fp32 passes only (for bf16 records the cumsum is
  // not compensated, its lo part is 0, and the array is left out)
  constexpr bool LO = sizeof(T) == 4;
  float* cl = cs + kGC * dkp;
  float* part = (LO ? cl + kGC * dkp : cl);  // the four waves' partial P tiles
  uint32_t* umask = reinterpret_cast<uint32_t*>(part + 1024);  // channels left to the log-space sum
  // bf16: Q~ and K~ in record order, written out in 16-byte units (16-byte
  // aligned: the arrays above are 2 (16 dkp) QS, 16 dkp + 1024 + kMaskWords
  // floats).  fp32
  // stores its elements directly: staging would take the 256-channel
  // passes' LDS past what lets two workgroups share a CU.
  constexpr bool STAGE = sizeof(T) == 2;
  uint8_t* r = rec + ((size_t)blockIdx.y * NC + blockIdx.x) * rec_bytes;
  T* stg = STAGE ? reinterpret_cast<T*>(umask + kMaskWords) : reinterpret_cast<T*>(r);
  const int n = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  if (tid < kMaskWords) umask[tid] = 0u;
  // q, k and log alpha of the chunk, 8 channels per load (dk is a multiple of
  // 16 and the padded channels are zero); consecutive lanes take consecutive
  // rows, so that a 16-lane group's channel-major stores are consecutive
  for (int x = tid; x < kGC * (dkp / 8); x += kThreads) {
    const int t = x % kGC, i = (x / kGC) * 8, u = n * kGC + t;
    const int dr = data_row(u, L, rev), gr = gate_row(u, L, rev);
    float qv[8], kv[8], av[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = kv[e] = av[e] = 0.f;
    if (i < dk && dr >= 0) {
      const size_t o = ((size_t)bh * L + dr) * dk + i;
      load8(q + o, qv);
      load8(k + o, kv);
    }
    if (i < dk && gr >= 0) {
      const f32x4* a4 = reinterpret_cast<const f32x4*>(la + ((size_t)bh * L + gr) * dk + i);
      const f32x4 a0 = a4[0], a1 = a4[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        av[e] = a0[e];
        av[e + 4] = a1[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs[(i + e) * kGC + t] = from_f32<QS>(qv[e]);
      ks[(i + e) * kGC + t] = from_f32<QS>(kv[e]);
      cs[(i + e) * kGC + t] = av[e];
    }
  }
  __syncthreads();
  float* pf = reinterpret_cast<float*>(r + (size_t)2 * kGC * dkp * sizeof(T));
  float* ga = pf + kPfFloats;
  // a thread per channel: its column of log alpha, q and k read into
  // registers first (the arrays are written in the same loop, and a load
  // after a store that may alias it would wait for that store)
  for (int i = tid; i < dkp; i += kThreads) {
    float at[kGC], al[kGC], qv[kGC], kv[kGC];
    lds16(cs + i * kGC, at);
    lds16(qs + i * kGC, qv);
    lds16(ks + i * kGC, kv);
    float c = 0.f, e = 0.f;
#pragma unroll
    for (int t = 0; t < kGC; ++t) {
      float err;
      c = csum<T>(c, at[t], err);
      e += err;
      at[t] = c;
      al[t] = e;
    }
    sts16(cs + i * kGC, at);
    if constexpr (LO) sts16(cl + i * kGC, al);
    ga[i] = gexp<T>(c + e);
    if (at[0] - c > kSafeP) atomicOr(&umask[i >> 5], 1u << (i & 31));
#pragma unroll
    for (int t = 0; t < kGC; ++t) {
      stg[qf_index<T>(t, i)] = from_f32<T>(qv[t] * gexp<T>(at[t] + al[t]));
      stg[kGC * dkp + kf_index(t, i)] = from_f32<T>(kv[t] * gexp<T>((c - at[t]) + (e - al[t])));
    }
  }
  __syncthreads();
  // the Q~ and K~ records (contiguous at the record's start)
  if constexpr (STAGE) {
    const int units = 2 * kGC * dkp * (int)sizeof(T) / 16;
    const f32x4* src = reinterpret_cast<const f32x4*>(stg);
    f32x4* dst = reinterpret_cast<f32x4*>(r);
    for (int x = tid; x < units; x += kThreads) dst[x] = src[x];
  }
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
      const int it = i * kGC;
      const float c0 = cs[it], l0 = LO ? cl[it] : 0.f;
      const float a = sf ? to_f32(qs[it + r16]) *
                               gexp<T>((cs[it + r16] - c0) + (LO ? cl[it + r16] - l0 : 0.f))
                         : 0.f;
      const float b = sf ? to_f32(ks[it + r16]) *
                               gexp<T>((c0 - cs[it + r16]) + (LO ? l0 - cl[it + r16] : 0.f))
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
    for (int wd = 0; wd < ((dkp + 31) >> 5); ++wd)
      for (uint32_t m = umask[wd]; m; m &= m - 1) {
        const int i = (wd * 32 + __builtin_ctz(m)) * kGC;
        acc += to_f32(qs[i + t]) * to_f32(ks[i + s]) *
               gexp<T>((cs[i + t] - cs[i + s]) + (LO ? cl[i + t] - cl[i + s] : 0.f));
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

// Buffer resource over bytes [p, p + bytes): loads outside read 0 and stores
// outside are dropped.
__device__ inline __amdgpu_buffer_rsrc_t gg_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Fragment loads from a chunk record's resource; off: byte offset of the
// wave's first tile.
template <int MT>
__device__ inline void load_q(GgFrag<bf16, MT>& f, __amdgpu_buffer_rsrc_t r, int off, int l) {
#pragma unroll
  for (int p = 0; p < MT / 2; ++p)
    f.q[p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            r, off + (((p * 64 + l) << 3) << 1), 0, 0));
}
template <int MT>
__device__ inline void load_q(GgFrag<float, MT>& f, __amdgpu_buffer_rsrc_t r, int off, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
    f.q[m] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                        r, off + (((m * 64 + l) << 2) << 2), 0, 0));
}
template <int MT>
__device__ inline void load_k(GgFrag<bf16, MT>& f, __amdgpu_buffer_rsrc_t r, int off, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
    f.k[m] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(
                                            r, off + (((m * 64 + l) << 2) << 1), 0, 0));
}
template <int MT>
__device__ inline void load_k(GgFrag<float, MT>& f, __amdgpu_buffer_rsrc_t r, int off, int l) {
#pragma unroll
  for (int m = 0; m < MT; ++m)
    f.k[m] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                        r, off + (((m * 64 + l) << 2) << 2), 0, 0));
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
// Chunks loaded ahead when everything is (gg_ahead == 2): two for state
// slices of up to 64 rows (a chunk step is shorter than the memory latency),
// except for fp32 slices in workgroups of more than four waves, whose
// 256-register budget does not hold the third register set; else one.
template <typename T, int MT, int NWR> constexpr int gg_depth() {
  return MT <= 4 && (sizeof(T) == 2 || NWR <= 4) ? 2 : 1;
}

// The sequence rows of pass chunk n.  Forward: data row d = u = 16 n + t for
// the chunk's token t, in the window [16 n, min(16 n + 16, L)).  Reversed: d =
// L - 1 - u, in the window [max(L - 16 (n + 1), 0), L - 16 n).  A lane's row
// relative to the window's first row is t (forward) or 15 - t + adj with adj =
// min(L - 16 (n + 1), 0) (reversed); rows off the window (past the sequence)
// fall outside the buffer resources built on it, so they read 0 and take no
// stores.  The log beta rows of a reversed pass are the data rows + 1 (the
// gate of original token L - u), valid up to row L - 1: their window starts a
// row later and, in chunk 0, holds a row fewer (token 0 has no gate).
struct GgWin {
  int base, rows, adj;
};
__device__ inline GgWin gg_window(int n, int L, int rev) {
  if (!rev) {
    const int b = kGC * n;
    return {b, min(kGC, L - b), 0};
  }
  const int lo = L - kGC * (n + 1), b = max(lo, 0);
  return {b, L - kGC * n - b, min(lo, 0)};
}
// Lane-constant parts of the v / log beta / output offsets (elements, window
// row 0 at adj = 0): (t or 15 - t) dv + jc for the lane's rows t = 4 g + e.
struct GgLane {
  int off[4];
};

// MT: the wave's tiles; DKP: the record's channels; m0: the wave's first tile
template <typename T, int MT>
__device__ inline void gg_load_late(GgIn<T, MT>& in, __amdgpu_buffer_rsrc_t rr, int DKP, int m0,
                                    int l, int g) {
  const int kf = kGC * DKP * (int)sizeof(T), pf = 2 * kf;
  load_k(in.f, rr, kf + 256 * m0 * (int)sizeof(T), l);
#pragma unroll
  for (int m = 0; m < MT; ++m)
    in.ga[m] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rr, pf + 4 * (kPfFloats + 16 * (m0 + m) + 4 * g), 0, 0));
}
template <typename T>
__device__ inline __amdgpu_buffer_rsrc_t gg_rec_rsrc(const uint8_t* rec, size_t rec_bytes, int bh,
                                                     int n, int NC) {
  return gg_rsrc(rec + ((size_t)bh * NC + n) * rec_bytes, (int)rec_bytes);
}

// vbh, lbh: v and log beta of the (batch, head).  The loads are unconditional
// and kept raw: a load under a branch, or a select on its value, would wait
// for it at once.
template <typename T, int MT, typename TI>
__device__ inline void gg_load(GgIn<T, MT>& in, const uint8_t* __restrict__ rec, size_t rec_bytes,
                               int DKP, int m0, const TI* __restrict__ vbh,
                               const float* __restrict__ lbh, const GgLane& ln, int bh, int n,
                               int NC, int L, int dv, int rev, int l, int g) {
  const __amdgpu_buffer_rsrc_t rr = gg_rec_rsrc<T>(rec, rec_bytes, bh, n, NC);
  const int pf = 2 * kGC * DKP * (int)sizeof(T);
  load_q(in.f, rr, 256 * m0 * (int)sizeof(T), l);  // 256 elements per 16-channel tile
  in.p = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rr, pf + 16 * l, 0, 0));
  in.pd = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rr, pf + 4 * (256 + 4 * g), 0, 0));
  if constexpr (gg_ahead<T, MT>() == 2) gg_load_late(in, rr, DKP, m0, l, g);
  const GgWin w = gg_window(n, L, rev);
  const __amdgpu_buffer_rsrc_t rv = gg_rsrc(vbh + (size_t)w.base * dv, w.rows * dv * (int)sizeof(TI));
  const __amdgpu_buffer_rsrc_t rl =
      gg_rsrc(lbh + (size_t)(w.base + rev) * dv, (w.rows - (rev && n == 0)) * dv * 4);
  const int adj = w.adj * dv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int x = ln.off[e] + adj;
    if constexpr (sizeof(TI) == 2)
      in.v[e] = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(rv, 2 * x, 0, 0) << 16);
    else
      in.v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, 4 * x, 0, 0));
    in.lb[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, 4 * x, 0, 0));
  }
}

// grid (dv / 16 * BH), NWR waves per workgroup; the dv / 16 column tiles of a
// (batch, head), which read the same chunk records, take consecutive logical
// ids placed on one XCD so that its L2 serves their repeated reads.  The NWR
// waves (1 to 8, chosen by the launcher) split the state tile's MT 16-row
// blocks between them: each forms its share of the inter term Q~ S, the
// others hand theirs to wave 0 through LDS, and wave 0 adds the intra term
// and writes the output; each wave decays and updates its own rows.  Lane (j, g) = (l % 16, l / 16) owns state column j of the tile
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
  const TI* vbh = v + (size_t)bh * L * dv;
  const float* lbh = lb + (size_t)bh * L * dv;
  GgLane ln;
#pragma unroll
  for (int e = 0; e < 4; ++e) ln.off[e] = (rev ? 15 - (4 * g + e) : 4 * g + e) * dv + jc;

  constexpr int AHEAD = gg_ahead<T, MTW>(), DEPTH = AHEAD == 2 ? gg_depth<T, MTW, NWR>() : 1;
  // fp32 passes that load v and log beta ahead (PIPE) do chunk n + 1's column
  // work at the end of chunk n's step (`step`), off the chain that runs from
  // the state through the inter term, the barrier and the update; their
  // compensated cumsums make that work long.  The others keep it inside the
  // step (`step_plain`), which measured faster for them.
  constexpr bool PIPE = AHEAD >= 1 && sizeof(T) == 4;
  // The per-column work of a chunk, which does not involve the state: the
  // chunk-local inclusive cumsum of log beta down the 16 rows of column j as
  // hi (c) + lo (cl) pairs (within the lane's 4 rows, then the totals of the
  // lanes above it, row groups g' < g, added in front), the chunk total, V~ =
  // v e^{b - B} and e^{b}; colscales adds wave 0's output scales e^{B} and
  // e^{B - b}.
  struct GgCol {
    float vv[4], c[4], cl[4], bh, bl, gb;
    floatx4 vt;
    float sq[4], sk[4];
  };
  auto colwork = [&](const GgIn<T, MTW>& in, GgCol& k) __attribute__((always_inline)) {
    float err;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k.vv[e] = in.v[e];
      k.c[e] = in.lb[e];
    }
    k.cl[0] = 0.f;
#pragma unroll
    for (int e = 1; e < 4; ++e) {
      k.c[e] = csum<T>(k.c[e - 1], k.c[e], err);
      k.cl[e] = k.cl[e - 1] + err;
    }
    float th[4], tl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      th[r] = __shfl(k.c[3], j + 16 * r);
      tl[r] = sizeof(T) == 4 ? __shfl(k.cl[3], j + 16 * r) : 0.f;
    }
    float eh = 0.f, el = 0.f;  // sum of the totals of row groups before g
    k.bh = 0.f;
    k.bl = 0.f;  // chunk total
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < g) {
        eh = csum<T>(eh, th[r], err);
        el += tl[r] + err;
      }
      k.bh = csum<T>(k.bh, th[r], err);
      k.bl += tl[r] + err;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k.c[e] = csum<T>(eh, k.c[e], err);
      k.cl[e] += el + err;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) k.vt[e] = k.vv[e] * gexp<T>((k.bh - k.c[e]) + (k.bl - k.cl[e]));
    k.gb = gexp<T>(k.bh + k.bl);
  };
  // wave 0's output scales
  auto colscales = [&](GgCol& k) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k.sq[e] = gexp<T>(k.c[e] + k.cl[e]);
      k.sk[e] = gexp<T>((k.c[e] - k.bh) + (k.cl[e] - k.bl));
    }
  };

  // One chunk step: chunk n from `cur`; first the loads of chunk `nl` (if in
  // range) go into `ld`.  The loop below is unrolled by the number of register
  // sets so that the sets change roles without copies: a copy of a register
  // whose load is in flight would wait for that load.
  auto step_plain = [&](int n, GgIn<T, MTW>& cur, GgIn<T, MTW>& ld, int nl) {
    if constexpr (AHEAD == 0)
      gg_load(cur, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, n, NC, L, dv, rev, l, g);
    if constexpr (AHEAD < 2) gg_load_late(cur, gg_rec_rsrc<T>(rec, rec_bytes, bh, n, NC), DKP, m0, l, g);
    // the prefetch is unconditional (past the end it reloads the last chunk,
    // unused): under a branch, the wait counts at its join would force waits
    // on the current set's loads as well
    if constexpr (AHEAD > 0)
      gg_load(ld, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, nl < NC ? nl : NC - 1, NC, L, dv, rev,
              l, g);
    const GgFrag<T, MTW>& f = cur.f;
    const f4 p = cur.p, pd = cur.pd;
    const float* pf = reinterpret_cast<const float*>(
        rec + ((size_t)bh * NC + n) * rec_bytes + (size_t)32 * DKP * sizeof(T));
    float vv[4], c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vv[e] = cur.v[e];
      c[e] = cur.lb[e];
    }
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
      // stores through resources on the chunk's window: rows past the
      // sequence fall outside and are dropped
      const GgWin wn = gg_window(n, L, rev);
      const size_t wo = ((size_t)bh * L + wn.base) * dv;
      const int adj = wn.adj * dv;
      if (ooff) {
        const __amdgpu_buffer_rsrc_t ro = gg_rsrc(ooff + wo, wn.rows * dv * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[e]), ro, 4 * (ln.off[e] + adj), 0, 0);
      }
      if (o) {
        const __amdgpu_buffer_rsrc_t ro = gg_rsrc(o + wo, wn.rows * dv * (int)sizeof(TO));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const TO y = from_f32<TO>(res[e] + pd[e] * vv[e]);
          if constexpr (sizeof(TO) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, y), ro,
                                                  2 * (ln.off[e] + adj), 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ro, 4 * (ln.off[e] + adj), 0, 0);
        }
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
  // The PIPE step: as step_plain, with chunk n's column work in `col`; at its
  // end chunk n + 1's goes into coln from nxt, the set holding that chunk.
  auto step = [&](int n, GgIn<T, MTW>& cur, GgIn<T, MTW>& ld, int nl, GgCol& col,
                  const GgIn<T, MTW>& nxt, GgCol& coln) {
    if constexpr (AHEAD < 2) gg_load_late(cur, gg_rec_rsrc<T>(rec, rec_bytes, bh, n, NC), DKP, m0, l, g);
    gg_load(ld, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, nl < NC ? nl : NC - 1, NC, L, dv, rev, l,
            g);
    const GgFrag<T, MTW>& f = cur.f;
    const f4 p = cur.p, pd = cur.pd;
    const float* pf = reinterpret_cast<const float*>(
        rec + ((size_t)bh * NC + n) * rec_bytes + (size_t)32 * DKP * sizeof(T));
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
      const floatx4 a2 = intra(p, col.vt, T());
      float res[4];
      const bool safe = col.bh + col.bl >= -kSafeDecay;
#pragma unroll
      for (int e = 0; e < 4; ++e) res[e] = col.sq[e] * a1[e] + col.sk[e] * a2[e];
      if (__any(!safe)) {
        // log-space intra term: sum_{s < t} P[t][s] v_s e^{Bt_t - Bt_s}
        float sl[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kGC; ++s) {
          const int src = j + 16 * (s >> 2);
          const float cs = __shfl(col.c[s & 3], src);
          const float ls = sizeof(T) == 4 ? __shfl(col.cl[s & 3], src) : 0.f;
          const float vs = __shfl(col.vv[s & 3], src);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * g + e;
            if (s < t)
              sl[e] += pf[pf_index(t, s)] * vs * gexp<T>((col.c[e] - cs) + (col.cl[e] - ls));
          }
        }
        if (!safe)
#pragma unroll
          for (int e = 0; e < 4; ++e) res[e] = col.sq[e] * a1[e] + sl[e];
      }
      // stores through resources on the chunk's window: rows past the
      // sequence fall outside and are dropped
      const GgWin wn = gg_window(n, L, rev);
      const size_t wo = ((size_t)bh * L + wn.base) * dv;
      const int adj = wn.adj * dv;
      if (ooff) {
        const __amdgpu_buffer_rsrc_t ro = gg_rsrc(ooff + wo, wn.rows * dv * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(res[e]), ro, 4 * (ln.off[e] + adj), 0, 0);
      }
      if (o) {
        const __amdgpu_buffer_rsrc_t ro = gg_rsrc(o + wo, wn.rows * dv * (int)sizeof(TO));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const TO y = from_f32<TO>(res[e] + pd[e] * col.vv[e]);
          if constexpr (sizeof(TO) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, y), ro,
                                                  2 * (ln.off[e] + adj), 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ro, 4 * (ln.off[e] + adj), 0, 0);
        }
      }
    }
    // decay and update
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][e] *= cur.ga[m][e] * col.gb;
    update(S, f, col.vt);
    colwork(nxt, coln);
    if (w == 0) colscales(coln);
  };
  GgIn<T, MTW> ra, rb, rc;
  if constexpr (AHEAD == 0) {
    for (int n = 0; n < NC; ++n) step_plain(n, ra, ra, NC);
  } else if constexpr (DEPTH == 1) {
    gg_load(ra, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, 0, NC, L, dv, rev, l, g);
    if constexpr (PIPE) {
      GgCol ca, cb;
      colwork(ra, ca);
      if (w == 0) colscales(ca);
      for (int n = 0; n < NC; n += 2) {
        step(n, ra, rb, n + 1, ca, rb, cb);
        if (n + 1 < NC) step(n + 1, rb, ra, n + 2, cb, ra, ca);
      }
    } else {
      for (int n = 0; n < NC; n += 2) {
        step_plain(n, ra, rb, n + 1);
        if (n + 1 < NC) step_plain(n + 1, rb, ra, n + 2);
      }
    }
  } else {
    gg_load(ra, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, 0, NC, L, dv, rev, l, g);
    gg_load(rb, rec, rec_bytes, DKP, m0, vbh, lbh, ln, bh, NC > 1 ? 1 : 0, NC, L, dv, rev, l, g);
    if constexpr (PIPE) {
      GgCol ca, cb;
      colwork(ra, ca);
      if (w == 0) colscales(ca);
      // the column sets alternate; the loop covers six chunks per iteration
      // so that both rotations line up without copies
      for (int n = 0; n < NC; n += 6) {
        step(n, ra, rc, n + 2, ca, rb, cb);
        if (n + 1 < NC) step(n + 1, rb, ra, n + 3, cb, rc, ca);
        if (n + 2 < NC) step(n + 2, rc, rb, n + 4, ca, ra, cb);
        if (n + 3 < NC) step(n + 3, ra, rc, n + 5, cb, rb, ca);
        if (n + 4 < NC) step(n + 4, rb, ra, n + 6, ca, rc, cb);
        if (n + 5 < NC) step(n + 5, rc, rb, n + 7, cb, ra, ca);
      }
    } else {
      for (int n = 0; n < NC; n += 3) {
        step_plain(n, ra, rc, n + 2);
        if (n + 1 < NC) step_plain(n + 1, rb, ra, n + 3);
        if (n + 2 < NC) step_plain(n + 2, rc, rb, n + 4);
      }
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
// left is the part that the gates decay.  The suffix sums run in groups of kGT
// tokens: each group's own suffix sums and its total (k_gg_gate_scan), the
// carry into each group from the totals after it (k_gg_gate_carry), then the
// carry added to the group's rows (k_gg_gate_add).  Every operand is read
// once, four channels per lane.
constexpr int kGT = 64;

// Four consecutive elements as fp32 (8- or 16-byte loads).
template <typename T> __device__ inline f4 ld4(const T* p);
template <> __device__ inline f4 ld4<float>(const float* p) {
  return *reinterpret_cast<const f4*>(p);
}
template <> __device__ inline f4 ld4<bf16>(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

// The channel blocks of the gate kernels: 256 channels (four per lane) each,
// the d_k blocks first, then the d_v blocks (grid z).
constexpr int kGQ = 4 * kWave;
__device__ inline void gg_gate_block(int z, int dk, int dv, int& half, int& c) {
  const int nzk = (dk + kGQ - 1) / kGQ;
  half = z >= nzk;
  c = 4 * (int)threadIdx.x + kGQ * (half ? z - nzk : z);
}
int gg_gate_zblocks(int dk, int dv) { return (dk + kGQ - 1) / kGQ + (dv + kGQ - 1) / kGQ; }

// grid (ceil(L / kGT), BH, gg_gate_zblocks), one wave; the d_k channels take
// q ⊙ dq - k ⊙ dk into dla, the d_v channels do ⊙ o - v ⊙ dv into dlb.  Writes the group's suffix sums to dla /
// dlb and its totals to tot [BH][NG][dk + dv].
template <typename T>
__global__ __launch_bounds__(kWave) void k_gg_gate_scan(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ dq,
    const float* __restrict__ dkk, const float* __restrict__ o32, const T* __restrict__ dout,
    const T* __restrict__ v, const float* __restrict__ dvv, float* __restrict__ tot,
    float* __restrict__ dla, float* __restrict__ dlb, int L, int dk, int dv) {
  const int cg = blockIdx.x, bh = blockIdx.y, NG = gridDim.x;
  int half, c;
  gg_gate_block(blockIdx.z, dk, dv, half, c);
  const int d = half ? dv : dk;
  if (c >= d) return;
  const T* a = half ? dout : q;
  const float* b = half ? o32 : dq;
  const T* x2 = half ? v : k;
  const float* y2 = half ? dvv : dkk;
  float* out = half ? dlb : dla;
  const int t0 = cg * kGT, t1 = min(L, t0 + kGT);
  f4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int t = t1 - 1; t >= t0; --t) {
    const size_t x = ((size_t)bh * L + t) * d + c;
    const f4 av = ld4(a + x), bv = ld4(b + x), cv = ld4(x2 + x), ev = ld4(y2 + x);
#pragma unroll
    for (int e = 0; e < 4; ++e) run[e] += av[e] * bv[e] - cv[e] * ev[e];
    *reinterpret_cast<f4*>(out + x) = run;
  }
  *reinterpret_cast<f4*>(tot + ((size_t)bh * NG + cg) * (dk + dv) + (half ? dk : 0) + c) = run;
}

// grid (BH, ceil((dk + dv) / kWave)), one wave: tot[bh][g][c] <- hs[bh][c] +
// the totals of the groups after g (hs: null for zeros).  The totals are read
// in batches ahead of the stores that overwrite them.
__global__ __launch_bounds__(kWave) void k_gg_gate_carry(float* __restrict__ tot,
                                                         const float* __restrict__ hs, int NG,
                                                         int D) {
  const int bh = blockIdx.x, c = blockIdx.y * kWave + threadIdx.x;
  if (c >= D) return;
  float run = hs ? hs[(size_t)bh * D + c] : 0.f;
  float* p = tot + (size_t)bh * NG * D + c;
  constexpr int kB = 16;
  for (int g1 = NG; g1 > 0; g1 -= kB) {
    float x[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) x[i] = g1 - 1 - i >= 0 ? p[(size_t)(g1 - 1 - i) * D] : 0.f;
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (g1 - 1 - i >= 0) {
        p[(size_t)(g1 - 1 - i) * D] = run;
        run += x[i];
      }
  }
}

// grid as k_gg_gate_scan: the carry of k_gg_gate_carry added to the group's
// rows of dla / dlb.
__global__ __launch_bounds__(kWave) void k_gg_gate_add(const float* __restrict__ tot,
                                                       float* __restrict__ dla,
                                                       float* __restrict__ dlb, int L, int dk,
                                                       int dv) {
  const int cg = blockIdx.x, bh = blockIdx.y, NG = gridDim.x;
  int half, c;
  gg_gate_block(blockIdx.z, dk, dv, half, c);
  const int d = half ? dv : dk;
  if (c >= d) return;
  float* out = half ? dlb : dla;
  const f4 cy =
      *reinterpret_cast<const f4*>(tot + ((size_t)bh * NG + cg) * (dk + dv) + (half ? dk : 0) + c);
  const int t0 = cg * kGT, t1 = min(L, t0 + kGT);
  // eight rows read before any is written back: the stores go to the array
  // the loads come from, so the compiler keeps each load after the previous
  // row's store unless they are batched by hand
  constexpr int kB = 8;
  for (int t = t0; t < t1; t += kB) {
    f4 x[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (t + u < t1) x[u] = *reinterpret_cast<const f4*>(out + ((size_t)bh * L + t + u) * d + c);
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (t + u < t1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] += cy[e];
        *reinterpret_cast<f4*>(out + ((size_t)bh * L + t + u) * d + c) = x[u];
      }
  }
}

// grid (BH), kThreads; hs [BH][dk + dv] = row sums, then column sums, of
// hT ⊙ dhT: a wave per row for the row sums, a lane per column for the
// column sums (both read along the rows).
__global__ __launch_bounds__(kThreads) void k_gg_hsum(const float* __restrict__ hT,
                                                      const float* __restrict__ dhT,
                                                      float* __restrict__ hs, int dk, int dv) {
  const int bh = blockIdx.x, w = threadIdx.x / kWave, l = threadIdx.x & (kWave - 1);
  const float* h = hT + (size_t)bh * dk * dv;
  const float* d = dhT + (size_t)bh * dk * dv;
  for (int i = w; i < dk; i += kThreads / kWave) {
    float s = 0.f;
    for (int j = l; j < dv; j += kWave) s += h[(size_t)i * dv + j] * d[(size_t)i * dv + j];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (l == 0) hs[(size_t)bh * (dk + dv) + i] = s;
  }
  for (int j = threadIdx.x; j < dv; j += kThreads) {
    float s = 0.f;
    for (int i = 0; i < dk; ++i) s += h[(size_t)i * dv + j] * d[(size_t)i * dv + j];
    hs[(size_t)bh * (dk + dv) + dk + j] = s;
  }
}

// ---- launchers ----

// Waves per state tile: two from 64 state rows on (32 for fp32), one below;
// four for the 512 rows of an fp32 pass.
template <typename T> constexpr int gg_row_split(int MT) {
  return MT >= 32 ? 4 : (MT >= (sizeof(T) == 2 ? 4 : 2) ? 2 : 1);
}
// SIMDs of the chip (256 CUs x 4).  A launch whose workgroups hold fewer
// waves than this leaves SIMDs idle; at 128 and 256 state rows it then splits
// the rows over 4 or 8 waves (32 rows each: ~200-230 VGPRs, two waves per
// SIMD), trading the per-column work that every wave repeats for the idle
// SIMDs.  With the chip already full the extra waves only queue.
constexpr long kChipSimds = 1024;

template <typename T, typename TO, typename TI>
static void launch_gg_recur(const GgPass& ps, int dkp, dim3 grid, const uint8_t* r, size_t rb,
                            int L, int NC, hipStream_t s) {
#define GG_RECUR_W(MT, NWR)                                                                   \
  hipLaunchKernelGGL((k_gg_recur<T, TO, MT, NWR, TI>), grid, dim3(kWave * (NWR)), 0, s, r, rb,  \
                     (const TI*)ps.v, ps.lb, ps.init, ps.init_t, (TO*)ps.o, ps.o_off, ps.fin,  \
                     ps.fin_la, ps.fin_lb, L, ps.dk, ps.dv, NC, ps.rev)
#define GG_RECUR(MT) GG_RECUR_W(MT, gg_row_split<T>(MT))
  const bool sparse = (long)grid.x * 2 < kChipSimds;  // two waves per workgroup leave SIMDs idle
  if constexpr (sizeof(T) == 4) {
    if (dkp == 16) { GG_RECUR(1); return; }
    if (dkp == 512) { GG_RECUR(32); return; }
  }
  if (dkp == 32) GG_RECUR(2);
  else if (dkp == 64) GG_RECUR(4);
  else if (dkp == 128) {
    if (sparse) GG_RECUR_W(8, 4);
    else GG_RECUR(8);
  } else {
    if (sparse) GG_RECUR_W(16, 8);
    else GG_RECUR(16);
  }
#undef GG_RECUR
#undef GG_RECUR_W
}

// part 0: k_gg_prep, part 1: k_gg_recur (separate so that each launch can be
// timed on its own).  is_bf16: the pass's records and arithmetic; in_bf16: the
// element type of its q, k and v (bf16 inputs may feed an fp32 pass).
template <typename T, typename TI, typename QS>
static hipError_t launch_gg_prep(const GgPass& ps, dim3 pg, size_t lds, uint8_t* r, size_t rb,
                                 int L, int dkp, int NC, hipStream_t s) {
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)k_gg_prep<T, TI, QS>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gg_prep<T, TI, QS>), pg, dim3(kThreads), lds, s, (const TI*)ps.q,
                     (const TI*)ps.k, ps.la, r, rb, L, ps.dk, dkp, NC, ps.rev);
  return hipSuccess;
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
    // q and k (16 padded rows each; bf16 from 256 bf16 input channels on,
    // else fp32), the cumsum (and for fp32 its lo part), 4 partial P tiles,
    // the mask words (53.5 KB at 256 fp32 channels with bf16 inputs, 69.9 KB
    // with fp32 ones, 135.5 KB at 512 fp32), and for bf16 the staged Q~, K~
    const bool qsb = in_bf16 && dkp >= 256;
    const size_t lds = (size_t)2 * kGC * dkp * (qsb ? 2 : 4) +
                       sizeof(float) * ((is_bf16 ? 1 : 2) * kGC * dkp + 1024 + kMaskWords) +
                       (is_bf16 ? (size_t)2 * kGC * dkp * 2 : 0);
    const dim3 pg(NC, BH);
    hipError_t e;
    if (is_bf16)
      e = qsb ? launch_gg_prep<bf16, bf16, bf16>(ps, pg, lds, r, rb, L, dkp, NC, s)
              : launch_gg_prep<bf16, bf16, float>(ps, pg, lds, r, rb, L, dkp, NC, s);
    else if (in_bf16)
      e = qsb ? launch_gg_prep<float, bf16, bf16>(ps, pg, lds, r, rb, L, dkp, NC, s)
              : launch_gg_prep<float, bf16, float>(ps, pg, lds, r, rb, L, dkp, NC, s);
    else
      e = launch_gg_prep<float, float, float>(ps, pg, lds, r, rb, L, dkp, NC, s);
    if (e != hipSuccess) return e;
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
  const int NG = gg_gate_groups(L), D = dk + dv;
  const dim3 grid(NG, BH, gg_gate_zblocks(dk, dv));
  if (dhT) hipLaunchKernelGGL(k_gg_hsum, dim3(BH), dim3(kThreads), 0, s, hT, dhT, hs, dk, dv);
  if (is_bf16)
    hipLaunchKernelGGL((k_gg_gate_scan<bf16>), grid, dim3(kWave), 0, s, (const bf16*)q,
                       (const bf16*)k, dq32, dk32, o32, (const bf16*)dout, (const bf16*)v, dv32,
                       tot, dla, dlb, L, dk, dv);
  else
    hipLaunchKernelGGL((k_gg_gate_scan<float>), grid, dim3(kWave), 0, s, (const float*)q,
                       (const float*)k, dq32, dk32, o32, (const float*)dout, (const float*)v,
                       dv32, tot, dla, dlb, L, dk, dv);
  hipLaunchKernelGGL(k_gg_gate_carry, dim3(BH, (D + kWave - 1) / kWave), dim3(kWave), 0, s, tot,
                     dhT ? hs : nullptr, NG, D);
  hipLaunchKernelGGL(k_gg_gate_add, grid, dim3(kWave), 0, s, tot, dla, dlb, L, dk, dv);
  return hipGetLastError();
}

}  // namespace gla
