// gla_api.hip -- the C ABI declared in include/gla.h: validation, workspace
// layout and the stream-ordered launch sequences.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/gla.h"
#include "gla_internal.h"

namespace gla {

static size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_plan(int B, int H, int L, int dk, int dv, int C, int c, int bf16, Plan* p,
               const FwdOptions& opt) {
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
  // B * H is a grid dimension (y or z) of most launches, which HIP caps at 65535
  if ((int64_t)B * H > 65535 || L > (1 << 24)) return false;
  if (opt.algo < FWD_AUTO || opt.algo > FWD_MATERIALIZED) return false;
  if (opt.bwd_algo < BWD_AUTO || opt.bwd_algo > BWD_RECURRENT) return false;
  if (opt.recur_waves < 0 || opt.recur_segments < 0) return false;
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
  // Forward path: the two-pass forward (chunk prep + recurrence) wherever its
  // kernels are instantiated, unless the caller asks for another one; an
  // explicitly requested path that the shape does not support is an error,
  // not a silent substitution.
  const bool can_recur = recur_supported(bf16, C, dk, dv, L);
  const bool can_fused = fused_supported(bf16, C, dk, dv);
  switch (opt.algo) {
    case FWD_TWO_PASS:
      if (!can_recur) return false;
      P.recur = 1; P.fused = 0;
      break;
    case FWD_FUSED:
      if (!can_fused) return false;
      P.recur = 0; P.fused = 1;
      break;
    case FWD_MATERIALIZED:
      P.recur = 0; P.fused = 0;
      break;
    default:
      P.recur = can_recur;
      P.fused = !can_recur && can_fused;
      break;
  }
  // Fused forward: one workgroup per (batch-head, segment, d_v tile); enough
  // segments to give every compute unit a workgroup.
  P.DVTF = fused_dv_tile(bf16, dk, dv);
  P.NSEGF = 1;
  P.segf_chunks = P.NC > 0 ? P.NC : 1;
  if (P.fused && P.NC > 1 && P.BH > 0) {
    const int64_t units = (int64_t)P.BH * (dv / P.DVTF);
    int64_t want = units >= 256 ? 1 : (256 + units - 1) / units;
    if (want > P.NC) want = P.NC;
    P.segf_chunks = (int)((P.NC + want - 1) / want);
    P.NSEGF = (P.NC + P.segf_chunks - 1) / P.segf_chunks;
  }
  // Recurrence: 16 state columns per wave; the largest workgroup that still
  // gives 256 workgroups, and sequence segments when even one wave per
  // workgroup leaves the chip mostly idle.  Explicit wave and segment counts
  // apply to the two-pass forward only.
  if (!P.recur && (opt.recur_waves || opt.recur_segments)) return false;
  // When even the narrowest workgroups leave the chip under-filled, the
  // sequence is split into segments anyway: then the widest workgroup is
  // best, since every workgroup of a (batch, head) streams all of its chunk
  // records (16 segments of four-wave workgroups run the long-sequence
  // workload, B1 H4 L16384, in 85 us against 119 us for 4 segments of
  // one-wave workgroups).
  const int wmin = recur_min_waves(bf16, dk), wmax = recur_max_waves(bf16, dk);
  const bool starved = (int64_t)P.BH * (dv / (16 * wmin)) < 128;
  P.NWVR = wmin;
  for (int w = wmax; w >= wmin; w /= 2) {
    if (dv % (16 * w)) continue;
    P.NWVR = w;
    if (starved || (int64_t)P.BH * (dv / (16 * w)) >= 256) break;
  }
  if (opt.recur_waves) {
    const int w = opt.recur_waves;
    if ((w != 1 && w != 2 && w != 4) || w < wmin || w > wmax || dv % (16 * w)) return false;
    P.NWVR = w;
  }
  P.NSEGR = 1;
  P.segr_chunks = P.NC > 0 ? P.NC : 1;
  if (P.recur && P.NC > 1 && P.BH > 0) {
    const int64_t units = (int64_t)P.BH * (dv / (16 * P.NWVR));
    int64_t want = 1;
    if (units < 128) want = (256 + units - 1) / units;
    if (opt.recur_segments) want = opt.recur_segments;
    if (want > P.NC) want = P.NC;
    if (want > 1) {
      P.segr_chunks = (int)((P.NC + want - 1) / want);
      P.NSEGR = (P.NC + P.segr_chunks - 1) / P.segr_chunks;
    }
  }
  const size_t BH = (size_t)P.BH, S = (size_t)dk * dv;
  size_t off = 0;
  // the chunk cumsum; fp32: followed by its low part (cum_lo_of)
  P.off_cum = off; off = align_up(off + BH * L * dk * 4 * (bf16 ? 1 : 2));
  P.off_sg = off; off = align_up(off + BH * (size_t)(P.NSEG > P.NSEGF ? P.NSEG : P.NSEGF) * dk * 4);
  P.off_st = off; off = align_up(off + BH * P.NC * S * P.esize);
  P.off_seg_u = off; off = align_up(off + (P.NSEG > 1 ? BH * P.NSEG * S * 4 : 0));
  P.off_seg_in = off; off = align_up(off + (P.NSEG > 1 ? BH * P.NSEG * S * 4 : 0));
  // the materialised forward's layout (also the start of the backward's)
  const size_t ws_mat = off;
  {
    // the fused forward reuses the cumsum region and needs its own segment states
    size_t f = P.off_st;
    P.off_fu = f; f = align_up(f + (P.NSEGF > 1 ? BH * P.NSEGF * S * 4 : 0));
    P.off_fi = f; f = align_up(f + (P.NSEGF > 1 ? BH * P.NSEGF * S * 4 : 0));
    P.ws_fused = f;
  }
  {
    // the two-pass forward's buffers (its own region from the start)
    const size_t NCC = (size_t)P.NC * C;
    size_t f = 0;
    P.off_qg = f; f = align_up(f + BH * NCC * dk * P.esize);
    P.off_kg = f; f = align_up(f + BH * NCC * dk * P.esize);
    P.off_ph = f; f = align_up(f + BH * P.NC * recur_prec_bytes(bf16, C));
    P.off_pl = f; f = align_up(f + (bf16 ? BH * NCC * 16 * P.esize : 0));
    P.off_gl = f; f = align_up(f + BH * P.NC * recur_grec_bytes(dk));
    P.off_ru = f; f = align_up(f + (P.NSEGR > 1 ? BH * P.NSEGR * S * 4 : 0));
    P.off_ri = f; f = align_up(f + (P.NSEGR > 1 ? BH * P.NSEGR * S * 4 : 0));
    P.off_rg = f; f = align_up(f + (P.NSEGR > 1 ? BH * P.NSEGR * dk * 4 : 0));
    P.ws_recur = f;
  }
  P.ws_fwd = P.recur ? P.ws_recur : (P.fused ? P.ws_fused : ws_mat);
  off = ws_mat > P.ws_fused ? ws_mat : P.ws_fused;
  // backward extras: dS per chunk in two layouts, hT, chunk totals of
  // dlog b, rowsum(hT * dhT)
  P.off_st2 = off; off = align_up(off + 2 * BH * P.NC * S * P.esize);
  P.off_end = off; off = align_up(off + BH * S * 4);
  P.off_dlt = off; off = align_up(off + BH * P.NC * dk * 4);
  P.off_rs = off; off = align_up(off + BH * dk * 4);
  P.off_A = off; off = align_up(off + BH * P.NC * C * C * 4);
  P.off_dA = off; off = align_up(off + BH * P.NC * C * C * 4);
  // low halves of the recomputed states and state gradients (bf16 split)
  P.off_stlo = off; off = align_up(off + (bf16 ? BH * P.NC * S * 2 : 0));
  P.off_dstlo = off; off = align_up(off + (bf16 ? BH * P.NC * S * 2 : 0));
  const size_t ws_bwd_mat = off;
  // the backward with the states on chip, where its kernels exist for the
  // shape (the dv pass reuses the two-pass forward's kernels and plan)
  const bool can_rec = bwd_inter_supported(bf16, C, dk, dv, L) && recur_supported(bf16, C, dk, dv, L);
  if (opt.bwd_algo == BWD_RECURRENT && !can_rec) return false;
  P.bwd_rec = opt.bwd_algo == BWD_RECURRENT || (opt.bwd_algo == BWD_AUTO && can_rec);
  {
    const size_t LD = BH * (size_t)L * dk * 4;
    size_t f = 0;
    P.off_bcum = f; f = align_up(f + LD);
    P.off_bdA = f; f = align_up(f + BH * P.NC * C * C * 4);
    P.off_bdqi = f; f = align_up(f + LD);
    P.off_bdki = f; f = align_up(f + LD);
    // running sums of the gate gradient's inter terms (two halves per chunk)
    P.off_bqpre = f; f = align_up(f + BH * P.NC * 2 * dk * 4);
    P.off_bksuf = f; f = align_up(f + BH * P.NC * 2 * dk * 4);
    P.off_brs = f; f = align_up(f + BH * dk * 4);
    P.off_bvrec = f; f = align_up(f + P.ws_recur);
    P.ws_bwd = P.bwd_rec ? f : ws_bwd_mat;
  }
  return true;
}

}  // namespace gla

using namespace gla;

static bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15) != 0; }

static FwdOptions options(const gla_fwd_config* cfg, const gla_bwd_config* bcfg) {
  FwdOptions o;
  if (cfg) {
    o.algo = cfg->algo;
    o.recur_waves = cfg->recur_waves;
    o.recur_segments = cfg->recur_segments;
  }
  if (bcfg) o.bwd_algo = bcfg->algo;
  return o;
}

static gla_status validate(const gla_dims* d, int dtype, Plan* p,
                           const gla_fwd_config* cfg = nullptr,
                           const gla_bwd_config* bcfg = nullptr) {
  if (!d) return GLA_ERR_NULL;
  if (dtype != GLA_FP32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  if (!make_plan(d->B, d->H, d->L, d->dk, d->dv, d->chunk, d->subchunk, dtype == GLA_BF16, p,
                 options(cfg, bcfg)))
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

// ---- launch profiling: HIP events around each launch on its stream.  A
// mutex guards the record table; the slot a launch reserved before it was
// enqueued is remembered per thread until its closing event is recorded.
namespace {
struct ProfRec {
  const char* name;  // null: the opening event could not be recorded
  hipEvent_t a, b;
  int done;          // closing event recorded
};
std::mutex g_prof_mu;
ProfRec* g_recs = nullptr;
int g_cap = 0, g_n = 0;
std::atomic<int> g_on{0};
thread_local int t_pending = -1;

void prof_before(const char* name, hipStream_t s) {
  t_pending = -1;
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_on.load(std::memory_order_relaxed) || g_n >= g_cap) return;
  const int i = g_n++;
  g_recs[i].done = 0;
  g_recs[i].name = hipEventRecord(g_recs[i].a, s) == hipSuccess ? name : nullptr;
  if (g_recs[i].name) t_pending = i;
}
void prof_after(hipStream_t s) {
  if (t_pending < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (t_pending < g_cap && hipEventRecord(g_recs[t_pending].b, s) == hipSuccess)
    g_recs[t_pending].done = 1;
  t_pending = -1;
}
}  // namespace

// Launch `expr` (a hipError_t-returning launcher) under the name `nm`.
#define GLA_LAUNCH(nm, expr)                         \
  do {                                               \
    prof_before(nm, s);                              \
    if ((expr) != hipSuccess) return GLA_ERR_HIP;    \
    prof_after(s);                                   \
  } while (0)

// The two-pass forward on workspace ws (the chunk records of pass 1, and the
// segment states when the recurrence is split into sequence segments).
static gla_status run_two_pass(const Plan& p, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* h0, void* o, float* hT,
                               char* ws, hipStream_t s) {
  // pass 1: per-chunk operands and score matrices; pass 2: the recurrence
  // (segment local states and a scan over segments first when segmented)
  void* qg = ws + p.off_qg;
  void* kg = ws + p.off_kg;
  void* ph = ws + p.off_ph;
  void* pl = ws + p.off_pl;
  float* gl = (float*)(ws + p.off_gl);
  float* ru = (float*)(ws + p.off_ru);
  float* ri = (float*)(ws + p.off_ri);
  float* rg = (float*)(ws + p.off_rg);
  GLA_LAUNCH("chunk_prep", launch_chunk_prep(p, q, k, log_alpha, v, qg, kg, gl, ph, pl, s));
  if (p.NSEGR > 1) {
    GLA_LAUNCH("recur_local", launch_chunk_recur(p, 0, qg, kg, ph, pl, gl, v, nullptr, nullptr, ru, rg, s));
    Plan ps = p;
    ps.NSEG = p.NSEGR;
    GLA_LAUNCH("segment_scan", launch_segment_scan(ps, 0, rg, h0, ru, ri, hT, s));
    GLA_LAUNCH("chunk_recur", launch_chunk_recur(p, 1, qg, kg, ph, pl, gl, v, ri, o, nullptr, nullptr, s));
  } else {
    GLA_LAUNCH("chunk_recur", launch_chunk_recur(p, 1, qg, kg, ph, pl, gl, v, h0, o, hT, nullptr, s));
  }
  return GLA_OK;
}

// The backward with the states kept on chip (bf16, C = 64):
//  * the chunk-local cumsum B of log alpha and dA = (dO V^T) masked, per chunk
//    in one launch;
//  * one launch of two recurrences over the chunks with the transposed state
//    (k_bwd_inter): the inter-chunk terms of dq (S, chunks in order) and of dk
//    (dS, chunks backwards), rowsum(hT ⊙ dhT) and dh0;
//  * the intra-chunk terms of dq and dk added per chunk, with the closed-form
//    dlog b = q ⊙ dq - k ⊙ dk and its reverse cumsum inside the chunk plus
//    the carry over later chunks (zako-mio report ch. 3.4), whose chunk
//    totals k_bwd_inter has summed from the inter terms;
//  * dv: the gradient of v is the forward of the time-reversed sequence with
//    queries k, keys q, values dout, the gates shifted by one token and dhT
//    as the initial state, so the two-pass forward's kernels compute it in
//    their reversed mode.
static gla_status run_bwd_recurrent(const Plan& p, const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* h0, const void* dout,
                                    const float* dhT, void* dq, void* dk, void* dv,
                                    float* dlog_alpha, float* dh0, char* ws, hipStream_t s) {
  float* cum = (float*)(ws + p.off_bcum);
  float* dA = (float*)(ws + p.off_bdA);
  float* dqi = (float*)(ws + p.off_bdqi);
  float* dki = (float*)(ws + p.off_bdki);
  float* qpre = (float*)(ws + p.off_bqpre);
  float* ksuf = (float*)(ws + p.off_bksuf);
  float* rs = (float*)(ws + p.off_brs);
  char* vr = ws + p.off_bvrec;
  GLA_LAUNCH("chunk_da_cum", launch_chunk_da_cum(p, v, dout, log_alpha, cum, dA, s));
  const BwdInterJob jq{dout, v, k, h0, dqi, rs, dhT, nullptr, 0, q, qpre};
  const BwdInterJob jk{v, dout, q, dhT, dki, nullptr, nullptr, dh0, 1, k, ksuf};
  GLA_LAUNCH("bwd_inter", launch_bwd_inter(p, jq, jk, cum, s));
  GLA_LAUNCH("chunk_dqdk", launch_chunk_dqdk_inter(p, q, k, cum, dA, dqi, dki, dq, dk,
                                                   dlog_alpha, qpre, ksuf, rs, s));
  // dv: the forward's passes over the reversed sequence (q <- k, k <- q,
  // v <- dout, h0 <- dhT); its final state is not needed (dh0 came above)
  void* qg = vr + p.off_qg;
  void* kg = vr + p.off_kg;
  void* ph = vr + p.off_ph;
  void* pl = vr + p.off_pl;
  float* gl = (float*)(vr + p.off_gl);
  GLA_LAUNCH("chunk_prep_rev", launch_chunk_prep_rev(p, k, q, log_alpha, dout, qg, kg, gl, ph, pl, s));
  if (p.NSEGR > 1) {
    float* ru = (float*)(vr + p.off_ru);
    float* ri = (float*)(vr + p.off_ri);
    float* rg = (float*)(vr + p.off_rg);
    GLA_LAUNCH("recur_local_rev", launch_chunk_recur_rev(p, 0, qg, kg, ph, pl, gl, dout, nullptr, nullptr, ru, rg, s));
    Plan ps = p;
    ps.NSEG = p.NSEGR;
    GLA_LAUNCH("segment_scan_rev", launch_segment_scan(ps, 0, rg, dhT, ru, ri, nullptr, s));
    GLA_LAUNCH("chunk_recur_rev", launch_chunk_recur_rev(p, 1, qg, kg, ph, pl, gl, dout, ri, dv, nullptr, nullptr, s));
  } else {
    GLA_LAUNCH("chunk_recur_rev", launch_chunk_recur_rev(p, 1, qg, kg, ph, pl, gl, dout, dhT, dv, nullptr, nullptr, s));
  }
  return GLA_OK;
}

// ---- scratch of the allocation-free forward (gla_fwd_noalloc)
// The two-pass forward's records live in this array of the library instead
// of a caller's workspace.  Each GPU the library runs on holds its own copy
// (GLA_NOALLOC_SCRATCH_BYTES, as .bss of the code object) until the process
// ends.  On the host, `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with that device
// current (hipGetSymbolAddress), and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[GLA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch copy (looked up on the
// first call on that device).
gla_status scratch_address(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GLA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GLA_ERR_HIP;
    g_scratch_addr[dev] = (char*)ptr;
  }
  *out = g_scratch_addr[dev];
  return GLA_OK;
}
}  // namespace

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

gla_status gla_fwd_ex_workspace_size(const gla_dims* dims, int dtype, const gla_fwd_config* cfg,
                                     size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  Plan p;
  gla_status st = validate(dims, dtype, &p, cfg);
  if (st != GLA_OK) return st;
  *bytes = p.ws_fwd;
  return GLA_OK;
}

gla_status gla_fwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  return gla_fwd_ex_workspace_size(dims, dtype, nullptr, bytes);
}

gla_status gla_bwd_ex_workspace_size(const gla_dims* dims, int dtype, const gla_bwd_config* cfg,
                                     size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  Plan p;
  gla_status st = validate(dims, dtype, &p, nullptr, cfg);
  if (st != GLA_OK) return st;
  *bytes = p.ws_bwd;
  return GLA_OK;
}

gla_status gla_bwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  return gla_bwd_ex_workspace_size(dims, dtype, nullptr, bytes);
}

gla_status gla_fwd(const gla_dims* dims, int dtype, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* h0, void* o, float* hT,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return gla_fwd_ex(dims, dtype, nullptr, q, k, v, log_alpha, h0, o, hT, workspace,
                    workspace_bytes, stream);
}

gla_status gla_fwd_ex(const gla_dims* dims, int dtype, const gla_fwd_config* cfg, const void* q,
                      const void* k, const void* v, const float* log_alpha, const float* h0,
                      void* o, float* hT, void* workspace, size_t workspace_bytes,
                      void* stream) {
  Plan p;
  gla_status st = validate(dims, dtype, &p, cfg);
  if (st != GLA_OK) return st;
  if (p.BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p.L == 0) {
    if ((st = check_ptrs({}, {h0, hT})) != GLA_OK) return st;
    if (hT) GLA_LAUNCH("copy_state", launch_copy_state(p, h0, hT, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, o}, {h0, hT})) != GLA_OK) return st;
  if (!workspace || workspace_bytes < p.ws_fwd) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;

  char* ws = (char*)workspace;
  float* cum = (float*)(ws + p.off_cum);
  float* sg = (float*)(ws + p.off_sg);
  void* states = ws + p.off_st;
  float* seg_u = (float*)(ws + p.off_seg_u);
  float* seg_in = (float*)(ws + p.off_seg_in);

  if (p.recur) return run_two_pass(p, q, k, v, log_alpha, h0, o, hT, ws, s);
  GLA_LAUNCH("chunk_cumsum", launch_cumsum(p, log_alpha, cum, cum_lo_of(p, cum), s));
  if (p.fused) {
    // segment entry states from the segments' local states, then one fused
    // pass per segment that keeps the state on chip
    float* fu = (float*)(ws + p.off_fu);
    float* fi = (float*)(ws + p.off_fi);
    if (p.NSEGF > 1) {
      Plan ps = p;
      ps.NSEG = p.NSEGF;
      ps.seg_chunks = p.segf_chunks;
      GLA_LAUNCH("chunk_state_local", launch_chunk_state(ps, 0, SEG_LOCAL, 0, k, v, cum, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, fu, sg, s));
      GLA_LAUNCH("segment_scan", launch_segment_scan(ps, 0, sg, h0, fu, fi, hT, s));
    }
    GLA_LAUNCH("seg_output", launch_seg_output(p, q, k, v, cum, h0, fi, o, hT, s));
    return GLA_OK;
  }
  if (p.NSEG > 1) {
    GLA_LAUNCH("chunk_state_local", launch_chunk_state(p, 0, SEG_LOCAL, 0, k, v, cum, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seg_u, sg, s));
    GLA_LAUNCH("segment_scan", launch_segment_scan(p, 0, sg, h0, seg_u, seg_in, hT, s));
    GLA_LAUNCH("chunk_state", launch_chunk_state(p, 0, SEG_FILL, 0, k, v, cum, h0, seg_in, states, nullptr, nullptr, nullptr, nullptr, nullptr, s));
  } else {
    GLA_LAUNCH("chunk_state", launch_chunk_state(p, 0, SEG_FILL, 0, k, v, cum, h0, nullptr, states, nullptr, nullptr, hT, nullptr, nullptr, s));
  }
  GLA_LAUNCH("chunk_output", launch_chunk_output(p, q, k, v, cum, states, o, s));
  return GLA_OK;
}

gla_status gla_fwd_noalloc(const gla_dims* dims, int dtype, const void* q, const void* k,
                           const void* v, const float* log_alpha, const float* h0, void* o,
                           float* hT, void* stream) {
  const gla_fwd_config cfg{GLA_FWD_TWO_PASS, 0, 0};
  Plan p;
  gla_status st = validate(dims, dtype, &p, &cfg);
  if (st != GLA_OK) return st;
  if (p.ws_fwd > (size_t)GLA_NOALLOC_SCRATCH_BYTES) return GLA_ERR_WORKSPACE;
  if (p.BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p.L == 0) {
    if ((st = check_ptrs({}, {h0, hT})) != GLA_OK) return st;
    if (hT) GLA_LAUNCH("copy_state", launch_copy_state(p, h0, hT, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, o}, {h0, hT})) != GLA_OK) return st;
  char* ws = nullptr;
  if ((st = scratch_address(&ws)) != GLA_OK) return st;
  return run_two_pass(p, q, k, v, log_alpha, h0, o, hT, ws, s);
}

gla_status gla_bwd(const gla_dims* dims, int dtype, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* h0, const void* dout, const float* dhT,
                   void* dq, void* dk, void* dv, float* dlog_alpha, float* dh0,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return gla_bwd_ex(dims, dtype, nullptr, q, k, v, log_alpha, h0, dout, dhT, dq, dk, dv,
                    dlog_alpha, dh0, workspace, workspace_bytes, stream);
}

gla_status gla_bwd_ex(const gla_dims* dims, int dtype, const gla_bwd_config* cfg, const void* q,
                      const void* k, const void* v, const float* log_alpha, const float* h0,
                      const void* dout, const float* dhT, void* dq, void* dk, void* dv,
                      float* dlog_alpha, float* dh0, void* workspace, size_t workspace_bytes,
                      void* stream) {
  Plan p;
  gla_status st = validate(dims, dtype, &p, nullptr, cfg);
  if (st != GLA_OK) return st;
  if (p.BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (p.L == 0) {
    if ((st = check_ptrs({}, {dhT, dh0})) != GLA_OK) return st;
    if (dh0) GLA_LAUNCH("copy_state", launch_copy_state(p, dhT, dh0, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, dout, dq, dk, dv, dlog_alpha}, {h0, dhT, dh0})) !=
      GLA_OK)
    return st;
  if (!workspace || workspace_bytes < p.ws_bwd) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;

  char* ws = (char*)workspace;
  if (p.bwd_rec) return run_bwd_recurrent(p, q, k, v, log_alpha, h0, dout, dhT, dq, dk, dv,
                                          dlog_alpha, dh0, ws, s);
  float* cum = (float*)(ws + p.off_cum);
  float* sg = (float*)(ws + p.off_sg);
  void* st_n = ws + p.off_st;                       // S_{n-1}, [dk][dv]
  void* dst_n = ws + p.off_st2;                     // dS_n, [dk][dv]
  void* dst_t = ws + p.off_st2 + (size_t)p.BH * p.NC * p.dk * p.dv * p.esize;  // dS_n, [dv][dk]
  float* seg_u = (float*)(ws + p.off_seg_u);
  float* seg_in = (float*)(ws + p.off_seg_in);
  float* hT = (float*)(ws + p.off_end);
  float* dlt = (float*)(ws + p.off_dlt);
  float* rs = (float*)(ws + p.off_rs);
  float* Aw = (float*)(ws + p.off_A);
  float* dAw = (float*)(ws + p.off_dA);
  void* st_lo = p.bf16 ? (void*)(ws + p.off_stlo) : nullptr;
  void* dst_lo = p.bf16 ? (void*)(ws + p.off_dstlo) : nullptr;

  // recompute the chunk states (not stored by the forward), and the reverse
  // recurrence of the state gradient: independent, so one launch runs both
  GLA_LAUNCH("chunk_cumsum", launch_cumsum(p, log_alpha, cum, cum_lo_of(p, cum), s));
  if (p.NSEG > 1) {
    GLA_LAUNCH("chunk_state_local", launch_chunk_state(p, 0, SEG_LOCAL, p.bf16, k, v, cum, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seg_u, sg, s));
    GLA_LAUNCH("segment_scan", launch_segment_scan(p, 0, sg, h0, seg_u, seg_in, hT, s));
    GLA_LAUNCH("chunk_state", launch_chunk_state(p, 0, SEG_FILL, p.bf16, k, v, cum, h0, seg_in, nullptr, st_n, st_lo, nullptr, nullptr, nullptr, s));
    GLA_LAUNCH("chunk_state_rev_local", launch_chunk_state(p, 1, SEG_LOCAL, p.bf16, q, dout, cum, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seg_u, sg, s));
    GLA_LAUNCH("segment_scan_rev", launch_segment_scan(p, 1, sg, dhT, seg_u, seg_in, dh0, s));
    GLA_LAUNCH("chunk_state_rev", launch_chunk_state(p, 1, SEG_FILL, p.bf16, q, dout, cum, dhT, seg_in, dst_t, dst_n, dst_lo, nullptr, nullptr, nullptr, s));
  } else {
    const StateJob fwd{0, SEG_FILL, k, v, cum, h0, nullptr, nullptr, st_n, st_lo, hT, nullptr, nullptr};
    const StateJob rev{1, SEG_FILL, q, dout, cum, dhT, nullptr, dst_t, dst_n, dst_lo, dh0, nullptr, nullptr};
    GLA_LAUNCH("chunk_state_pair", launch_chunk_state_pair(p, p.bf16, fwd, rev, s));
  }
  GLA_LAUNCH("chunk_attn", launch_chunk_attn(p, q, k, v, dout, cum, Aw, dAw, s));
  GLA_LAUNCH("chunk_dqdk", launch_chunk_dqdk(p, q, k, v, dout, cum, st_n, st_lo, dst_n,
                                             dst_lo, dAw, dq, dk, dlog_alpha, dlt, s));
  GLA_LAUNCH("chunk_dv", launch_chunk_dv(p, k, dout, cum, dst_t, Aw, dv, s));
  GLA_LAUNCH("rowsum_state", launch_rowsum_state(p, dhT ? hT : nullptr, dhT, rs, s));
  GLA_LAUNCH("dla_carry", launch_dla_carry(p, dlt, rs, dlog_alpha, s));
  return GLA_OK;
}

gla_status gla_decode(const gla_dims* dims, int dtype, const void* q, const void* k,
                      const void* v, const float* log_alpha, float* state, void* o,
                      void* stream) {
  if (!dims) return GLA_ERR_NULL;
  if (dtype != GLA_FP32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  // one token: B, H, dk and dv are checked as for gla_fwd (the sequence and
  // chunk fields of dims do not apply)
  Plan p;
  if (!make_plan(dims->B, dims->H, 1, dims->dk, dims->dv, 64, 16, dtype == GLA_BF16, &p))
    return GLA_ERR_SHAPE;
  if (p.BH == 0) return GLA_OK;
  gla_status st = check_ptrs({q, k, v, log_alpha, state, o}, {});
  if (st != GLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  GLA_LAUNCH("decode", launch_decode(p, q, k, v, log_alpha, state, o, s));
  return GLA_OK;
}

// ---- general gate G = alpha^T beta
static gla_status gg_validate(const gla_dims* d, int dtype) {
  if (!d) return GLA_ERR_NULL;
  if (dtype != GLA_FP32 && dtype != GLA_BF16) return GLA_ERR_DTYPE;
  const int q = dtype == GLA_BF16 ? 32 : 16;
  if (d->B < 0 || d->H < 0 || d->L < 0 || d->L > (1 << 24)) return GLA_ERR_SHAPE;
  if ((int64_t)d->B * d->H > 65535) return GLA_ERR_SHAPE;
  if (d->dk < 16 || d->dk > 256 || d->dv < 16 || d->dv > 512) return GLA_ERR_SHAPE;
  if (d->dk % q || d->dv % q) return GLA_ERR_SHAPE;
  return GLA_OK;
}

namespace {
// Workspace of the general gate.  Forward: the pass records.  Backward: the
// records of fp32 passes, the recomputed output without its same-token term
// (o_off) and hT, and dq, dk, dv without their same-token terms, all fp32;
// gate-gradient partial sums.  The passes write dq, dk, dv in the I/O dtype
// to the caller's buffers.
struct GgWs {
  size_t ooff, hT32, oq, ok, ov, tot, hs, end;
};
GgWs gg_layout(const gla_dims* d, int bf16, int bwd) {
  const size_t BH = (size_t)d->B * d->H, L = (size_t)d->L;
  GgWs w{};
  size_t off;
  if (!bwd) {
    off = align_up(gg_pass_rec_bytes(bf16, (int)BH, d->L, d->dk));
  } else {
    size_t r = gg_pass_rec_bytes(0, (int)BH, d->L, d->dk);
    const size_t r2 = gg_pass_rec_bytes(0, (int)BH, d->L, d->dv);
    off = align_up(r > r2 ? r : r2);
    const size_t nk = align_up(BH * L * d->dk * 4), nv = align_up(BH * L * d->dv * 4);
    w.ooff = off; off += nv;
    w.hT32 = off; off += align_up(BH * d->dk * d->dv * 4);
    w.oq = off; off += nk;
    w.ok = off; off += nk;
    w.ov = off; off += nv;
    w.tot = off; off += align_up(BH * gg_gate_groups(d->L) * (d->dk + d->dv) * 4);
    w.hs = off; off += align_up(BH * (d->dk + d->dv) * 4);
  }
  w.end = off;
  return w;
}
Plan gg_state_plan(const gla_dims* d) {
  Plan p{};
  p.B = d->B; p.H = d->H; p.BH = d->B * d->H; p.dk = d->dk; p.dv = d->dv;
  return p;
}
}  // namespace

gla_status ggla_fwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  gla_status st = gg_validate(dims, dtype);
  if (st != GLA_OK) return st;
  *bytes = gg_layout(dims, dtype == GLA_BF16, 0).end;
  return GLA_OK;
}

gla_status ggla_bwd_workspace_size(const gla_dims* dims, int dtype, size_t* bytes) {
  if (!bytes) return GLA_ERR_NULL;
  gla_status st = gg_validate(dims, dtype);
  if (st != GLA_OK) return st;
  *bytes = gg_layout(dims, dtype == GLA_BF16, 1).end;
  return GLA_OK;
}

gla_status ggla_fwd(const gla_dims* dims, int dtype, const void* q, const void* k,
                    const void* v, const float* log_alpha, const float* log_beta,
                    const float* h0, void* o, float* hT, void* workspace,
                    size_t workspace_bytes, void* stream) {
  gla_status st = gg_validate(dims, dtype);
  if (st != GLA_OK) return st;
  const int bf16 = dtype == GLA_BF16, BH = dims->B * dims->H, L = dims->L;
  if (BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (L == 0) {
    if ((st = check_ptrs({}, {h0, hT})) != GLA_OK) return st;
    if (hT) GLA_LAUNCH("copy_state", launch_copy_state(gg_state_plan(dims), h0, hT, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, log_beta, o}, {h0, hT})) != GLA_OK) return st;
  const GgWs w = gg_layout(dims, bf16, 0);
  if (!workspace || workspace_bytes < w.end) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;
  const GgPass ps{q, k, v, log_alpha, log_beta, dims->dk, dims->dv, 0, h0, 0, o, nullptr, hT,
                  nullptr, nullptr};
  GLA_LAUNCH("gg_prep", launch_gg_pass(ps, 0, bf16, bf16, BH, L, workspace, s));
  GLA_LAUNCH("gg_recur", launch_gg_pass(ps, 1, bf16, bf16, BH, L, workspace, s));
  return GLA_OK;
}

gla_status ggla_bwd(const gla_dims* dims, int dtype, const void* q, const void* k,
                    const void* v, const float* log_alpha, const float* log_beta,
                    const float* h0, const void* dout, const float* dhT, void* dq, void* dk,
                    void* dv, float* dlog_alpha, float* dlog_beta, float* dh0, void* workspace,
                    size_t workspace_bytes, void* stream) {
  gla_status st = gg_validate(dims, dtype);
  if (st != GLA_OK) return st;
  const int bf16 = dtype == GLA_BF16, BH = dims->B * dims->H, L = dims->L;
  const int DK = dims->dk, DV = dims->dv;
  if (BH == 0) return GLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (L == 0) {
    if ((st = check_ptrs({}, {dhT, dh0})) != GLA_OK) return st;
    if (dh0) GLA_LAUNCH("copy_state", launch_copy_state(gg_state_plan(dims), dhT, dh0, s));
    return GLA_OK;
  }
  if ((st = check_ptrs({q, k, v, log_alpha, log_beta, dout, dq, dk, dv, dlog_alpha, dlog_beta},
                       {h0, dhT, dh0})) != GLA_OK)
    return st;
  const GgWs w = gg_layout(dims, bf16, 1);
  if (!workspace || workspace_bytes < w.end) return GLA_ERR_WORKSPACE;
  if (misaligned(workspace)) return GLA_ERR_ALIGN;
  char* ws = (char*)workspace;
  // The passes run in fp32 arithmetic (bf16 inputs are converted as they are
  // read): the closed-form gate gradients subtract terms tens of times larger
  // than their result, which bf16 operands in the passes would not resolve.
  float* ooff = (float*)(ws + w.ooff);
  float* hT32 = (float*)(ws + w.hT32);
  float *oq = (float*)(ws + w.oq), *ok = (float*)(ws + w.ok), *ov = (float*)(ws + w.ov);
  // the forward again, for o and hT (closed-form gate gradients)
  const GgPass p0{q, k, v, log_alpha, log_beta, DK, DV, 0, h0, 0, nullptr, ooff,
                  dhT ? hT32 : nullptr, nullptr, nullptr};
  // dq_t = S_t do_t: the transposed state, q <- do, k <- v, v <- k, gates swapped
  const GgPass p1{dout, v, k, log_beta, log_alpha, DV, DK, 0, h0, 1, dq, oq, nullptr, nullptr,
                  nullptr};
  // dv_s = k_s dS_s, dS_s = G_{s+1} ⊙ dS_{s+1} + q_s^T do_s from dS = dhT: the
  // reversed sequence with q <- k, k <- q, v <- do; its final state dS_0 times
  // token 0's gate is dh0
  const GgPass p2{k, q, dout, log_alpha, log_beta, DK, DV, 1, dhT, 0, dv, ov, dh0, log_alpha,
                  log_beta};
  // dk_s = dS_s v_s: the same, transposed: q <- v, k <- do, v <- q, gates swapped
  const GgPass p3{v, dout, q, log_beta, log_alpha, DV, DK, 1, dhT, 1, dk, ok, nullptr, nullptr,
                  nullptr};
  const GgPass* passes[4] = {&p0, &p1, &p2, &p3};
  static const char* names[4][2] = {{"gg_prep", "gg_recur"}, {"gg_prep_dq", "gg_recur_dq"},
                                    {"gg_prep_dv", "gg_recur_dv"}, {"gg_prep_dk", "gg_recur_dk"}};
  for (int i = 0; i < 4; ++i) {
    GLA_LAUNCH(names[i][0], launch_gg_pass(*passes[i], 0, 0, bf16, BH, L, ws, s));
    GLA_LAUNCH(names[i][1], launch_gg_pass(*passes[i], 1, 0, bf16, BH, L, ws, s));
  }
  GLA_LAUNCH("gg_gates", launch_gg_gates(bf16, BH, L, DK, DV, q, k, oq, ok, ooff, dout, v, ov,
                                         hT32, dhT, (float*)(ws + w.tot), (float*)(ws + w.hs),
                                         dlog_alpha, dlog_beta, s));
  return GLA_OK;
}

gla_status gla_profile_begin(int capacity) {
  if (capacity < 1) return GLA_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_on.store(0);
  if (capacity != g_cap) {
    for (int i = 0; i < g_cap; ++i) {
      (void)hipEventDestroy(g_recs[i].a);
      (void)hipEventDestroy(g_recs[i].b);
    }
    free(g_recs);
    g_cap = 0;
    g_n = 0;
    g_recs = (ProfRec*)calloc((size_t)capacity, sizeof(ProfRec));
    if (!g_recs) return GLA_ERR_HIP;
    for (int i = 0; i < capacity; ++i) {
      if (hipEventCreate(&g_recs[i].a) != hipSuccess) {
        g_cap = i;
        return GLA_ERR_HIP;
      }
      if (hipEventCreate(&g_recs[i].b) != hipSuccess) {
        (void)hipEventDestroy(g_recs[i].a);
        g_cap = i;
        return GLA_ERR_HIP;
      }
      g_cap = i + 1;
    }
  }
  g_n = 0;
  g_on.store(1);
  return GLA_OK;
}

void gla_profile_end(void) { g_on.store(0); }

int gla_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return g_n;
}

gla_status gla_profile_get(int index, const char** kernel, float* ms) {
  if (!kernel || !ms) return GLA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (index < 0 || index >= g_n) return GLA_ERR_SHAPE;
  const ProfRec& r = g_recs[index];
  if (!r.name || !r.done) return GLA_ERR_HIP;
  if (hipEventElapsedTime(ms, r.a, r.b) != hipSuccess) return GLA_ERR_HIP;
  *kernel = r.name;
  return GLA_OK;
}

}  // extern "C"
