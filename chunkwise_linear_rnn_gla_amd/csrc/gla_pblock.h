// gla_pblock.h -- building the chunk's causal gated score matrix
//   P[m][r] = sum_k q_mk k_rk exp(B_mk - B_rk),  r <= m  (0 above the diagonal)
// for one chunk of C rows, walking d_k in slices of KS channels (papercache.org
// notes §4.1 log-space parallel form restricted to a chunk; §4.3 / Figure 3
// secondary chunking).
//
//  * Off-diagonal sub-chunk blocks (query sub-chunk j, key sub-chunk u < j):
//    MFMA on (Q_j ⊙ e^{B_j - z}) (K_u ⊙ e^{z - B_u})^T with z = B at the
//    first row of sub-chunk j (the App. B listing's reference row), so both
//    factors are <= 1.
//  * Diagonal 16 x 16 blocks: fp32 on the vector ALUs.  The decay between rows
//    r <= m is the running product alpha_{r+1} ... alpha_m of the per-row gates
//    alpha_s = e^{B_s - B_{s-1}}: equal to e^{B_m - B_r} up to rounding, no
//    division, no overflow.  Lane (p, g) of a block team owns rows p and
//    15 - p (17 (row, key) pairs in all) over a channel group g.
#pragma once

#include "gla_common.h"

namespace gla {

// Off-diagonal sub-chunk pair number pi -> (query sub-chunk j, key sub-chunk u < j).
__device__ inline void pair_of(int pi, int& j, int& u) {
  j = 1;
  while (pi >= j) { pi -= j; ++j; }
  u = pi;
}

// Load / store 8 consecutive elements as fp32.
__device__ inline void load8(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[e + 4] = b[e]; }
}
__device__ inline void load8(const bf16* p, float* o) {
  bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = static_cast<float>(a[e]);
}
__device__ inline void store8(float* p, const float* x) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = x[e]; b[e] = x[e + 4]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}
__device__ inline void store8(bf16* p, const float* x) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<bf16x8*>(p) = a;
}
// Store 8 consecutive elements to a destination that is only 8-byte aligned.
__device__ inline void store8_aligned8(float* p, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    float2 v2 = {x[e], x[e + 1]};
    *reinterpret_cast<float2*>(p + e) = v2;
  }
}
__device__ inline void store8_aligned8(bf16* p, const float* x) {
#pragma unroll
  for (int e = 0; e < 8; e += 4) {
    bf16x4 a;
#pragma unroll
    for (int f = 0; f < 4; ++f) a[f] = static_cast<bf16>(x[e + f]);
    *reinterpret_cast<bf16x4*>(p + e) = a;
  }
}
__device__ inline void store4(float* p, floatx4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ inline floatx4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ inline floatx4 load4(const bf16* p) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  floatx4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(a[e]);
  return r;
}
__device__ inline void store4(bf16* p, floatx4 x) {
  bf16x4 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<bf16x4*>(p) = a;
}

// Register staging of 8 consecutive elements of T (one 16- or 32-byte load).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { bf16x8 v; };
template <> struct Raw8<float> { f32x4 v[2]; };
__device__ inline void raw_load(Raw8<bf16>& r, const bf16* p) { r.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ inline void raw_load(Raw8<float>& r, const float* p) {
  r.v[0] = *reinterpret_cast<const f32x4*>(p);
  r.v[1] = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ inline float raw_get(const Raw8<bf16>& r, int e) { return static_cast<float>(r.v[e]); }
__device__ inline float raw_get(const Raw8<float>& r, int e) { return r.v[e >> 2][e & 3]; }
__device__ inline void raw_zero(Raw8<bf16>& r) { r.v = bf16x8{}; }
__device__ inline void raw_zero(Raw8<float>& r) { r.v[0] = f32x4{}; r.v[1] = f32x4{}; }

// XCD-aware renumbering of a 1-D grid of n workgroups: consecutive logical
// ids land on the same XCD.
__device__ inline int xcd_logical(int w, int n) {
  const int per = n / 8, rem = n % 8, x = w % 8, i = w / 8;
  // XCDs 0..rem-1 own per+1 logical ids, the others per
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// Gather a fragment of KPL elements spaced `stride` apart (a column read of a
// row-major LDS array: the MFMA operand wants consecutive K per lane, and K
// runs down the rows).
template <typename T>
__device__ inline typename Mma<T>::frag gather_frag(const T* p, int stride);
template <> __device__ inline bf16x8 gather_frag<bf16>(const bf16* p, int stride) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = p[e * stride];
  return r;
}
template <> __device__ inline float gather_frag<float>(const float* p, int stride) { return p[0]; }

// Row padding (elements) of a row-major LDS array of width W read by
// gather_frag: the four 16-lane groups of a wave read rows KPL apart, and the
// padding puts their 64-byte (fp32) / 32-byte (bf16) column windows in
// disjoint LDS banks.
template <typename T> constexpr int gather_pad(int W) {
  if (sizeof(T) == 2) {
    // stride s dwords with 8 s = 16 (mod 64)
    for (int p = 0; p < 64; p += 2)
      if ((((W + p) / 2) * 8) % 64 == 16) return p;
    return 0;
  }
  for (int p = 0; p < 64; p += 4)
    if ((W + p) % 64 == 16 || (W + p) % 64 == 48) return p;
  return 0;
}

// S: element type of the q / k slice arrays in LDS (T, or fp32 so that the
// vector-ALU reads need no conversion).
template <typename T, int C, int NWV = 4, typename S = T>
struct PBuilder {
  static constexpr int NTH = NWV * kWave;          // threads of the workgroup
  using M = Mma<T>;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int KS = BF ? 32 : 16;          // d_k slice
  static constexpr int PT = 16 / (int)sizeof(S);
  static constexpr int LDT = KS + PT;              // row length of the S slice arrays
  static constexpr int LDF = KS + 4;               // row length of fp32 slice arrays
  static constexpr int NRT = C / 16;               // sub-chunks per chunk
  static constexpr int NP = NRT * (NRT - 1) / 2;   // off-diagonal pairs
  static constexpr int NPW = (NP + NWV - 1) / NWV;
  static constexpr int NPA = NPW > 0 ? NPW : 1;
  static constexpr int WPB = NWV / NRT;            // waves per diagonal block
  static constexpr int NG = 8 * WPB;               // channel groups per block
  static constexpr int CPL = KS / NG > 0 ? KS / NG : 1;
  // LDS: q, k (T), cumsum and gates (fp32), one slice
  static constexpr int SLICE_BYTES = 2 * C * LDT * (int)sizeof(S) + 2 * C * LDF * 4;

  float dsum[17];
  floatx4 pacc[NPA];
  int db, dp, dg, w, l;

  __device__ void init() {
    w = wave_id();
    l = lane_id();
    const int tb = (w % WPB) * kWave + l;
    db = w / WPB;
    dp = tb & 7;
    dg = tb >> 3;
#pragma unroll
    for (int i = 0; i < 17; ++i) dsum[i] = 0.f;
#pragma unroll
    for (int t = 0; t < NPA; ++t) pacc[t] = zero4();
  }

  // Stage rows [r0, r0 + C) x channels [s0, s0 + KS) of q, k and the chunk-local
  // cumsum into LDS.  Rows >= rv are padding: q = k = 0 and the cumsum of the
  // last valid row (log alpha = 0 there).  Optionally also writes
  // qt = T(q ⊙ e^B) (row-major, LDT) for the inter-chunk MFMA.
  __device__ static void stage(const T* q, const T* k, const float* cum, size_t qo, int r0,
                               int rv, int dk, int s0, S* qs, S* ks, float* bs, T* qt) {
    for (int it = threadIdx.x; it < C * (KS / 8); it += NTH) {
      const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
      const bool valid = row < rv;
      const int crow = valid ? r0 + row : r0 + rv - 1;
      float qv[8], kv[8], bv[8];
      load8(cum + qo + (size_t)crow * dk + s0 + c8, bv);
      if (valid) {
        load8(q + qo + (size_t)crow * dk + s0 + c8, qv);
        load8(k + qo + (size_t)crow * dk + s0 + c8, kv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = kv[e] = 0.f;
      }
      store8(qs + row * LDT + c8, qv);
      store8(ks + row * LDT + c8, kv);
      store8(bs + row * LDF + c8, bv);
      if (qt) {
        float t8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t8[e] = qv[e] * gexp<T>(bv[e]);
        store8(qt + row * LDT + c8, t8);
      }
    }
  }

  // The low part of a compensated cumsum (cum_lo) for the staged slice, in
  // the layout of bs (rows past rv repeat the last valid row).
  __device__ static void stage_lo(const float* cum_lo, size_t qo, int r0, int rv, int dk, int s0,
                                  float* bsl) {
    for (int it = threadIdx.x; it < C * (KS / 8); it += NTH) {
      const int row = it / (KS / 8), c8 = (it % (KS / 8)) * 8;
      const int crow = row < rv ? r0 + row : r0 + rv - 1;
      float bv[8];
      load8(cum_lo + qo + (size_t)crow * dk + s0 + c8, bv);
      store8(bsl + row * LDF + c8, bv);
    }
  }

  // Per-row gates within each sub-chunk: als[row] = e^{B_row - B_{row-1}}
  // (1 at a sub-chunk's first row, where it is never used); with bsl, the
  // difference of the cumsum's hi + lo pairs.
  template <bool LO = false>
  __device__ static void gates(const float* bs, float* als, const float* bsl = nullptr) {
    for (int it = threadIdx.x; it < C * KS; it += NTH) {
      const int row = it / KS, c = it % KS;
      float d = 0.f;
      if (row & 15) {
        d = bs[row * LDF + c] - bs[(row - 1) * LDF + c];
        if constexpr (LO) d += bsl[row * LDF + c] - bsl[(row - 1) * LDF + c];
      }
      als[row * LDF + c] = (row & 15) ? gexp<T>(d) : 1.f;
    }
  }

  // Off-diagonal blocks, MFMA, accumulated over slices.  Needs qs, ks, bs
  // (and, LO, the cumsum's low part bsl).
  template <bool LO = false>
  __device__ void offdiag(const S* qs, const S* ks, const float* bs, const float* bsl = nullptr) {
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      const int pi = w + NWV * t;
      if (pi >= NP) continue;
      int jq, ju;
      pair_of(pi, jq, ju);
      const int m = l & 15;
      for (int kk = 0; kk < KS; kk += M::K) {
        const int cq = kk + (l >> 4) * M::KPL;
        float sa[M::KPL], sb[M::KPL];
#pragma unroll
        for (int e = 0; e < M::KPL; ++e) {
          const float z = bs[(jq * 16) * LDF + cq + e];
          float da = bs[(jq * 16 + m) * LDF + cq + e] - z, db = z - bs[(ju * 16 + m) * LDF + cq + e];
          if constexpr (LO) {
            const float zl = bsl[(jq * 16) * LDF + cq + e];
            da += bsl[(jq * 16 + m) * LDF + cq + e] - zl;
            db += zl - bsl[(ju * 16 + m) * LDF + cq + e];
          }
          sa[e] = gexp<T>(da);
          sb[e] = gexp<T>(db);
        }
        typename M::frag a, b;
        if constexpr (BF && sizeof(S) == 4) {
          a = scaled_frag_from_f32(qs + (jq * 16 + m) * LDT + cq, sa);
          b = scaled_frag_from_f32(ks + (ju * 16 + m) * LDT + cq, sb);
        } else {
          a = scaled_frag<T>(qs + (jq * 16 + m) * LDT + cq, sa);
          b = scaled_frag<T>(ks + (ju * 16 + m) * LDT + cq, sb);
        }
        pacc[t] = M::run(a, b, pacc[t]);
      }
    }
  }

  // CPL consecutive channels as fp32 (vector LDS loads).
  __device__ static inline void ldc(const float* p, float* o) {
    if constexpr (CPL == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = v[c];
    } else if constexpr (CPL == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      o[0] = v.x;
      o[1] = v.y;
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] = p[c];
    }
  }
  __device__ static inline void ldc(const bf16* p, float* o) {
    if constexpr (CPL == 4) {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = static_cast<float>(v[c]);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] = static_cast<float>(p[c]);
    }
  }

  // Diagonal blocks, fp32 VALU, accumulated over slices.  Needs qs, ks, als.
  // The lane's two query rows are loaded once; each step then reads one key
  // row and one gate row (vector loads) and extends the running gate product.
  __device__ void diag(const S* qs, const S* ks, const float* als) {
    if (dg * CPL >= KS) return;
    const int cb = dg * CPL;
    const int m2 = 15 - dp;
    float q1[CPL], q2[CPL], wv[CPL];
    ldc(qs + (db * 16 + dp) * LDT + cb, q1);
    ldc(qs + (db * 16 + m2) * LDT + cb, q2);
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      const bool first = i <= dp;
      const int r = first ? (dp - i) : (m2 - (i - dp - 1));
      const int Rk = db * 16 + r;
      const int Ra = (Rk + 1 < C) ? Rk + 1 : Rk;
      float kv[CPL], av[CPL];
      ldc(ks + Rk * LDT + cb, kv);
      ldc(als + Ra * LDF + cb, av);
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (i == 0) wv[c] = q1[c];
        else wv[c] = (i == dp + 1) ? q2[c] : wv[c] * av[c];
        part += wv[c] * kv[c];
      }
      dsum[i] += part;
    }
  }

  // After the last slice (and a barrier): reduce the diagonal partials and
  // hand every entry of P to emit(m, r, value), r <= m.  Off-diagonal entries
  // are emitted by the wave that owns the block, diagonal ones after a
  // cross-wave sum through pd (NWV x 16 x 17 floats of LDS).
  template <typename Emit>
  __device__ void finish(float (*pd)[16][17], Emit emit) {
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      dsum[i] += __shfl_xor(dsum[i], 8);
      dsum[i] += __shfl_xor(dsum[i], 16);
      dsum[i] += __shfl_xor(dsum[i], 32);
    }
    if ((l >> 3) == 0) {
#pragma unroll
      for (int i = 0; i < 17; ++i) {
        const bool first = i <= dp;
        const int m = first ? dp : 15 - dp;
        const int r = first ? (dp - i) : (15 - dp - (i - dp - 1));
        pd[w][m][r] = dsum[i];
      }
    }
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      const int pi = w + NWV * t;
      if (pi >= NP) continue;
      int jq, ju;
      pair_of(pi, jq, ju);
#pragma unroll
      for (int r = 0; r < 4; ++r) emit(jq * 16 + (l >> 4) * 4 + r, ju * 16 + (l & 15), pacc[t][r]);
    }
    lds_barrier();
    for (int it = threadIdx.x; it < NRT * 256; it += NTH) {
      const int b = it >> 8, m = (it >> 4) & 15, r = it & 15;
      if (r > m) continue;
      float val = 0.f;
#pragma unroll
      for (int ww = 0; ww < WPB; ++ww) val += pd[b * WPB + ww][m][r];
      emit(b * 16 + m, b * 16 + r, val);
    }
  }
};

}  // namespace gla
