// gla_api.hip -- the C ABI declared in include/gla.h: validation, workspace
// layout and the stream-ordered launch sequences.
#include <stdint.h>
#include <stdlib.h>

#include "../../include/gla.h"
#include "gla_internal.h"

namespace gla {

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_plan(int B, int H, int L, int dk, int dv, int C, int c, int bf16, Plan* p) {
  if (B < 0 || H < 0 || L < 0) return false;
  if (c != 16) return false;
  if (bf16) {
    if (C != 32 && C != 64) return false;
    if (dk % 32 || dv % 32) return false;
  } else {
    if (C != 16 && C != 32 && C != 64) return false;
    if (dk % 16 || dv % 16) return false;
  }
  if (dk < 16 || dk > 256 || dv < 16 || dv > 512) return false;
  if ((int64_t)B * H > (1 << 20) || L > (1 << 24)) return false;
  Plan& P = *p;
  P.B = B; P.H = H; P.L = L; P.dk = dk; P.dv = dv; P.C = C; P.c = c; P.bf16 = bf16;
  P.BH = B * H;
  P.NC = (L + C - 1) / C;
  P.esize = bf16 ? 2 : 4;
  P.TS = (dk % 64 == 0 && dv % 64 == 0) ? 64 : (dk % 32 == 0 && dv % 32 == 0) ? 32 : 16;
  const int tv_max = bf16 ? 256 : 128;
  P.TVO = 16;
  for (int t = tv_max; t >= 16; t /= 2)
    if (dv % t == 0) { P.TVO = t; break; }
  // Sequence segments for the state recurrence: enough workgroups to cover
  // the chip when batch * heads * state tiles alone is too few.
  const int64_t tiles = (int64_t)P.BH * (dk / P.TS) * (dv / P.TS);
  P.NSEG = 1;
  P.seg_chunks = P.NC > 0 ? P.NC : 1;
  if (tiles > 0 && tiles < 256 && P.NC > 1) {
    int64_t want = (512 + tiles - 1) / tiles;
    if (want > P.NC) want = P.NC;
    P.seg_chunks = (int)((P.NC + want - 1) / want);
    P.NSEG = (P.NC + P.seg_chunks - 1) / P.seg_chunks;
  }
  const size_t BH = (size_t)P.BH, S = (size_t)dk * dv;
  size_t off = 0;
  P.off_cum = off; off = align_up(off + BH * L * dk * 4);
  P.off_st = off; off = align_up(off + BH * P.NC * S * P.esize);
  P.off_seg_u = off; off = align_up(off + (P.NSEG > 1 ? BH * P.NSEG * S * 4 : 0));
  P.off_seg_in = off; off = align_up(off + (P.NSEG > 1 ? BH * P.NSEG * S * 4 : 0));
  P.ws_fwd = off;
  // backward extras: dS per chunk in two layouts, hT, chunk totals of
  // dlog b, rowsum(hT * dhT)
  P.off_st2 = off; off = align_up(off + 2 * BH * P.NC * S * P.esize);
  P.off_end = off; off = align_up(off + BH * S * 4);
  P.off_dlt = off; off = align_up(off + BH * P.NC * dk * 4);
  P.off_rs = off; off = align_up(off + BH * dk * 4);
  P.ws_bwd = off;
  return true;
}

}  // namespace gla

using namespace gla;

static bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15) != 0; }

static gla_status validate(const gla_dims* d, int dtype, Plan* p) {
  if (!d) return GLA_ERR_NULL;
  if (dtype != GLA_FP32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (!make_plan(d->B, d->H, d->L, d->dk, d->dv, d->chunk, d->subchunk, dtype == GLA_BF16, p))
    return GLA_ERR_SHAPE;
  return GLA_OK;
}

static gla_status check_ptrs(std::initializer_list<const void*> required,
                             std::initializer_list<const void*> optional) {
  for (const void* x : required)
    if (!x) return GLA_ERR_NULL;
  for (const void* x : required)
    if (misaligned(x)) return GLA_ERR_ALIGN;
  for (const void* x : optional)
    if (x && misaligned(x)) return GLA_ERR_ALIGN;
  return GLA_OK;
}

#define GLA_TRY(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return GLA_ERR_HIP;  \
  } while (0)

extern "C" {

int gla_abi_version(void) { return GLA_ABI_VERSION; }

const char* gla_status_string(int status) {
  switch (status) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL: return "required pointer is NULL";
    case GLA_ERR_SHAPE: return "unsupported or inconsistent sizes";
    case GLA_ERR_DTYPE: return "unknown dtype";
    case GLA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

gla_status gla_fwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  Plan p;
  gla_status st = validate(dims, dtype, &p);
  if (st != GLA_OK) return st;
  *bytes = p.ws_fwd;
  return GLA_OK;
}

gla_status gla_bwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  Plan p;
  gla_status st = validate(dims, dtype, &p);
  if (st != GLA_OK) return st;
  *bytes = p.ws_bwd;
  return GLA_OK;
}

gla_status gla_fwd(const gla_dims* dims, int dtype, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* h0, void* o, float* hT,
                   void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  gla_status st = validate(dims, dtype, &p);
  if (st != GLA_OK) return st;
  if (p.BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p.L == 0) {
    if ((st = check_ptrs({}, {h0, hT})) != GLA_OK) return st;
    if (hT) GLA_TRY(launch_copy_state(p, h0, hT, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, o}, {h0, hT})) != GLA_OK) return st;
  if (!workspace || workspace_bytes < p.ws_fwd) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;

  char* ws = (char*)workspace;
  float* cum = (float*)(ws + p.off_cum);
  void* states = ws + p.off_st;
  float* seg_u = (float*)(ws + p.off_seg_u);
  float* seg_in = (float*)(ws + p.off_seg_in);

  GLA_TRY(launch_cumsum(p, log_alpha, cum, s));
  if (p.NSEG > 1) {
    GLA_TRY(launch_chunk_state(p, 0, SEG_LOCAL, k, v, cum, nullptr, nullptr, nullptr, nullptr,
                               nullptr, seg_u, s));
    GLA_TRY(launch_segment_scan(p, 0, cum, h0, seg_u, seg_in, hT, s));
    GLA_TRY(launch_chunk_state(p, 0, SEG_FILL, k, v, cum, h0, seg_in, states, nullptr, nullptr,
                               nullptr, s));
  } else {
    GLA_TRY(launch_chunk_state(p, 0, SEG_FILL, k, v, cum, h0, nullptr, states, nullptr, hT,
                               nullptr, s));
  }
  GLA_TRY(launch_chunk_output(p, q, k, v, cum, states, o, s));
  return GLA_OK;
}

gla_status gla_bwd(const gla_dims* dims, int dtype, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* h0, const void* dout, const float* dhT,
                   void* dq, void* dk, void* dv, float* dlog_alpha, float* dh0,
                   void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  gla_status st = validate(dims, dtype, &p);
  if (st != GLA_OK) return st;
  if (p.BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p.L == 0) {
    if ((st = check_ptrs({}, {dhT, dh0})) != GLA_OK) return st;
    if (dh0) GLA_TRY(launch_copy_state(p, dhT, dh0, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, dout, dq, dk, dv, dlog_alpha}, {h0, dhT, dh0})) !=
      GLA_OK)
    return st;
  if (!workspace || workspace_bytes < p.ws_bwd) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;

  char* ws = (char*)workspace;
  float* cum = (float*)(ws + p.off_cum);
  void* st_n = ws + p.off_st;                       // S_{n-1}, [dk][dv]
  void* dst_n = ws + p.off_st2;                     // dS_n, [dk][dv]
  void* dst_t = ws + p.off_st2 + (size_t)p.BH * p.NC * p.dk * p.dv * p.esize;  // dS_n, [dv][dk]
  float* seg_u = (float*)(ws + p.off_seg_u);
  float* seg_in = (float*)(ws + p.off_seg_in);
  float* hT = (float*)(ws + p.off_end);
  float* dlt = (float*)(ws + p.off_dlt);
  float* rs = (float*)(ws + p.off_rs);

  // recompute the chunk states (not stored by the forward)
  GLA_TRY(launch_cumsum(p, log_alpha, cum, s));
  if (p.NSEG > 1) {
    GLA_TRY(launch_chunk_state(p, 0, SEG_LOCAL, k, v, cum, nullptr, nullptr, nullptr, nullptr,
                               nullptr, seg_u, s));
    GLA_TRY(launch_segment_scan(p, 0, cum, h0, seg_u, seg_in, hT, s));
    GLA_TRY(launch_chunk_state(p, 0, SEG_FILL, k, v, cum, h0, seg_in, nullptr, st_n, nullptr,
                               nullptr, s));
  } else {
    GLA_TRY(launch_chunk_state(p, 0, SEG_FILL, k, v, cum, h0, nullptr, nullptr, st_n, hT,
                               nullptr, s));
  }
  // reverse recurrence of the state gradient
  if (p.NSEG > 1) {
    GLA_TRY(launch_chunk_state(p, 1, SEG_LOCAL, q, dout, cum, nullptr, nullptr, nullptr, nullptr,
                               nullptr, seg_u, s));
    GLA_TRY(launch_segment_scan(p, 1, cum, dhT, seg_u, seg_in, dh0, s));
    GLA_TRY(launch_chunk_state(p, 1, SEG_FILL, q, dout, cum, dhT, seg_in, dst_t, dst_n, nullptr,
                               nullptr, s));
  } else {
    GLA_TRY(launch_chunk_state(p, 1, SEG_FILL, q, dout, cum, dhT, nullptr, dst_t, dst_n, dh0,
                               nullptr, s));
  }
  GLA_TRY(launch_chunk_grad(p, q, k, v, dout, cum, st_n, dst_n, dst_t, dq, dk, dv, dlog_alpha,
                            dlt, s));
  GLA_TRY(launch_rowsum_state(p, dhT ? hT : nullptr, dhT, rs, s));
  GLA_TRY(launch_dla_carry(p, dlt, rs, dlog_alpha, s));
  return GLA_OK;
}

}  // extern "C"
