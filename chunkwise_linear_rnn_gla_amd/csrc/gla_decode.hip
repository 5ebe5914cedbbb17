// gla_decode.hip -- one token of the recurrent form, in place on the state
// (gfx950).
//
// Per (batch, head), with a = log alpha of the token:
//   S <- diag(e^{a}) S + k^T v,      o = q S   (the updated state)
// (papercache.org notes §2.1 and §4.1, recurrent form: constant memory per
// token, the inference form of the layer).  The work is one read and one
// write of the d_k x d_v fp32 state, so the kernel is bound by HBM: each
// lane streams one state column with coalesced row loads (a wave covers CW
// consecutive columns of 64 / CW rows), several rows in flight, and the
// 256 / CW row groups of a workgroup split the d_k rows; their partial
// outputs meet in LDS.  CW = 32 columns per workgroup doubles the grid, which
// keeps more rows in flight while B x H is small; CW = 64 is faster once the
// grid fills the chip.
#include "gla_common.h"
#include "gla_internal.h"

namespace gla {

namespace {

constexpr int kDecUnroll = 8;  // rows in flight per lane

}  // namespace

// grid (ceil(dv / CW), B * H), 256 threads.  Thread t takes column t % CW
// and row group g = t / CW, rows [g R, (g + 1) R), R = dk CW / 256 (dk is a
// multiple of 16); lanes past dv only take part in the barriers.
template <typename T, int CW>
__global__ __launch_bounds__(kThreads) void k_decode(const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const float* __restrict__ la,
                                                     float* __restrict__ state,
                                                     T* __restrict__ o, int dk, int dv) {
  __shared__ float qs[256], ks[256], gs[256];
  constexpr int kDecCols = CW, kDecGroups = kThreads / CW;
  __shared__ float part[kDecGroups][kDecCols];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int c = tid % kDecCols, g = tid / kDecCols;
  const int j = blockIdx.x * kDecCols + c;  // this lane's state column
  const bool live = j < dv;
  for (int i = tid; i < dk; i += kThreads) {
    qs[i] = to_f32(q[(size_t)bh * dk + i]);
    ks[i] = to_f32(k[(size_t)bh * dk + i]);
    gs[i] = gexp<T>(la[(size_t)bh * dk + i]);
  }
  const float vj = live ? to_f32(v[(size_t)bh * dv + j]) : 0.f;
  __syncthreads();

  const int R = dk / kDecGroups, i0 = g * R;
  float* s = state + ((size_t)bh * dk + i0) * dv + j;
  float acc = 0.f;
  int i = live ? 0 : R;
  for (; i + kDecUnroll <= R; i += kDecUnroll) {
    float x[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) x[u] = s[(size_t)(i + u) * dv];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int r = i0 + i + u;
      x[u] = gs[r] * x[u] + ks[r] * vj;
      acc += qs[r] * x[u];
      s[(size_t)(i + u) * dv] = x[u];
    }
  }
  for (; i < R; ++i) {
    const int r = i0 + i;
    const float x = gs[r] * s[(size_t)i * dv] + ks[r] * vj;
    acc += qs[r] * x;
    s[(size_t)i * dv] = x;
  }
  part[g][c] = acc;
  __syncthreads();
  if (g == 0 && live) {
    float sum = 0.f;
#pragma unroll
    for (int gg = 0; gg < kDecGroups; ++gg) sum += part[gg][c];
    o[(size_t)bh * dv + j] = from_f32<T>(sum);
  }
}

template <int CW>
static hipError_t launch_decode_w(const Plan& p, const void* q, const void* k, const void* v,
                                  const float* la, float* state, void* o, hipStream_t s) {
  const dim3 grid((p.dv + CW - 1) / CW, p.BH);
  if (p.bf16)
    hipLaunchKernelGGL((k_decode<bf16, CW>), grid, dim3(kThreads), 0, s, (const bf16*)q,
                       (const bf16*)k, (const bf16*)v, la, state, (bf16*)o, p.dk, p.dv);
  else
    hipLaunchKernelGGL((k_decode<float, CW>), grid, dim3(kThreads), 0, s, (const float*)q,
                       (const float*)k, (const float*)v, la, state, (float*)o, p.dk, p.dv);
  return hipGetLastError();
}

hipError_t launch_decode(const Plan& p, const void* q, const void* k, const void* v,
                         const float* la, float* state, void* o, hipStream_t s) {
  // 64-column workgroups once they alone give two per compute unit
  if ((long)p.BH * ((p.dv + 63) / 64) >= 512)
    return launch_decode_w<64>(p, q, k, v, la, state, o, s);
  return launch_decode_w<32>(p, q, k, v, la, state, o, s);
}

}  // namespace gla
