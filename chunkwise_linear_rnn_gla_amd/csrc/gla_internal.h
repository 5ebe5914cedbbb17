// gla_internal.h -- launch plan and kernel launchers shared by the GLA
// translation units.  Not part of the public ABI (include/gla.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gla {

// Everything a launch sequence needs, derived once from the problem sizes.
struct Plan {
  int B, H, L, dk, dv, C, c;
  int bf16;          // 1: q, k, v, ... are bf16; 0: fp32
  int BH;            // B * H
  int NC;            // number of chunks, ceil(L / C)
  int TS;            // square state-tile edge for the chunk-state kernel
  int NSEG;          // sequence segments for the chunk-state recurrence
  int seg_chunks;    // chunks per segment
  int TVO;           // output column tile of the output kernels
  int fused;         // forward runs the fused segment kernel (else materialised states)
  int NSEGF;         // sequence segments of the fused forward
  int segf_chunks;   // chunks per fused segment
  int DVTF;          // d_v tile of the fused segment kernel
  int recur;         // forward runs chunk prep + chunk recurrence (two passes)
  int NWVR;          // waves (16 state columns each) per recurrence workgroup
  int NSEGR;         // sequence segments of the recurrence
  int segr_chunks;   // chunks per recurrence segment
  size_t esize;      // bytes per I/O element
  // workspace layout (byte offsets); 0-sized regions have offset 0
  size_t off_cum, off_st, off_st2, off_seg_u, off_seg_in, off_end, off_dlt, off_rs;
  size_t off_A, off_dA, off_stlo, off_dstlo;
  size_t off_fu, off_fi;   // fused forward: segment local states, segment entry states
  size_t off_sg;           // segment total log decays [BH][max(NSEG, NSEGF)][dk]
  // two-pass forward: Q~, K~ [BH][NC*C][dk], P [BH][NC][C][C], low part of P's
  // diagonal blocks [BH][NC][C][16], chunk log decays [BH][NC][dk], segment
  // local states / entry states [BH][NSEGR][dk][dv], segment log decays
  size_t off_qg, off_kg, off_ph, off_pl, off_gl, off_ru, off_ri, off_rg;
  size_t ws_fwd, ws_bwd;    // workspace of the chosen forward path; of the backward
  size_t ws_recur, ws_fused;  // workspace of the two-pass and of the fused forward
  // backward with the states on chip (bwd_rec): cumsum, dA, the inter terms of
  // dq and dk (fp32), chunk totals of dlog b, rowsum(hT * dhT), and the
  // two-pass records of the reversed-sequence dv pass (at off_bvrec)
  int bwd_rec;
  size_t off_bcum, off_bdA, off_bdqi, off_bdki, off_bqpre, off_bksuf, off_brs, off_bvrec;
};

// Forward path and its tuning, as the caller chose them (gla_fwd_config in
// include/gla.h); zeros mean "automatic".
enum FwdAlgo { FWD_AUTO = 0, FWD_TWO_PASS = 1, FWD_FUSED = 2, FWD_MATERIALIZED = 3 };
enum BwdAlgo { BWD_AUTO = 0, BWD_MATERIALIZED = 1, BWD_RECURRENT = 2 };
struct FwdOptions {
  int algo = FWD_AUTO;
  int recur_waves = 0;
  int recur_segments = 0;
  int bwd_algo = BWD_AUTO;  // the backward's path (gla_bwd_config)
};

// Fills everything but the status; returns false if the sizes (or the
// requested forward path) are unsupported.
bool make_plan(int B, int H, int L, int dk, int dv, int C, int c, int bf16, Plan* p,
               const FwdOptions& opt = FwdOptions());

// ---- forward kernels (gla_fwd.hip) ----
// cum_lo (nullable): the low part of a compensated cumsum.
hipError_t launch_cumsum(const Plan& p, const float* a, float* cum, float* cum_lo, hipStream_t s);
// The materialised and fused paths' fp32 chunk cumsum is followed in the
// workspace by its low part (the two-sum compensation written by
// k_cumsum); bf16 keeps no low part.
inline float* cum_lo_of(const Plan& p, float* cum) {
  return p.bf16 ? nullptr : cum + (size_t)p.BH * p.L * p.dk;
}
inline const float* cum_lo_of(const Plan& p, const float* cum) {
  return p.bf16 ? nullptr : cum + (size_t)p.BH * p.L * p.dk;
}

// Chunk-state recurrence.  Forward (rev = 0): S_n = diag(g_n) S_{n-1} +
// (X ⊙ e^{b_n - B})^T Y with X = k, Y = v; writes S_{n-1} per chunk.
// Reverse (rev = 1): dS_{n-1} = diag(g_n) dS_n + (X ⊙ e^{B})^T Y with X = q,
// Y = dO; writes dS_n per chunk.  st_t: per-chunk states laid out [dv][dk];
// st_n: laid out [dk][dv]; either may be null.
//   mode SEG_LOCAL : zero start per segment, end state -> seg_u[seg]
//   mode SEG_FILL  : start from seg_in[seg] (or init / zeros if NSEG == 1),
//                    writes per-chunk states, end state -> end_out (last seg)
enum StateMode { SEG_LOCAL = 0, SEG_FILL = 1 };
// The arguments of one recurrence (as for launch_chunk_state).
struct StateJob {
  int rev, mode;
  const void* X;
  const void* Y;
  const float* cum;
  const float* init;
  const float* seg_in;
  void* st_t;
  void* st_n;
  void* st_n_lo;
  float* end_out;
  float* seg_out;
  float* seg_g;
};
inline const float* cum_of(const StateJob& j) { return j.cum; }
// split (bf16 only): hi/lo operand split, and st_n_lo receives the low part of
// the states written to st_n.
// In SEG_LOCAL mode seg_g (if not null) receives each segment's total log decay
// per key channel, [BH][NSEG][dk].
hipError_t launch_chunk_state(const Plan& p, int rev, int mode, int split, const void* X,
                              const void* Y, const float* cum, const float* init,
                              const float* seg_u_in, void* st_t, void* st_n, void* st_n_lo,
                              float* end_out, float* seg_u_out, float* seg_g, hipStream_t s);
// Two recurrences over the same segments and cumsum in one launch (the
// workgroups of a first, then those of b), e.g. the forward recurrence of S
// and the reverse one of dS, which are independent.
hipError_t launch_chunk_state_pair(const Plan& p, int split, const StateJob& a, const StateJob& b,
                                   hipStream_t s);
// Combine per-segment local states: seg_in[seg] = state entering segment seg
// (forward order, or reverse order when rev), end_out = final state.
hipError_t launch_segment_scan(const Plan& p, int rev, const float* seg_g, const float* init,
                               const float* seg_u, float* seg_in, float* end_out,
                               hipStream_t s);
hipError_t launch_chunk_output(const Plan& p, const void* q, const void* k, const void* v,
                               const float* cum, const void* st_t, void* o, hipStream_t s);
hipError_t launch_copy_state(const Plan& p, const float* src, float* dst, hipStream_t s);

// ---- fused segment forward (gla_fused.hip) ----
bool fused_supported(int bf16, int C, int dk, int dv);
int fused_dv_tile(int bf16, int dk, int dv);
// Per (batch-head, segment p.NSEGF, d_v tile p.DVTF): o for the segment's
// chunks from the segment entry state (seg_in, or h0 when NSEGF == 1, when
// hT also receives the final state).
hipError_t launch_seg_output(const Plan& p, const void* q, const void* k, const void* v,
                             const float* cum, const float* h0, const float* seg_in, void* o,
                             float* hT, hipStream_t s);

// ---- two-pass forward (gla_prep.hip, gla_recur.hip) ----
// Waves per recurrence workgroup needed to hold the state slice: one wave's
// 16 columns of a 256-channel bf16 or 128-channel fp32 state leave too few
// registers for the operands.
constexpr int recur_min_waves(bool bf16, int dk) { return (bf16 ? dk >= 256 : dk >= 128) ? 2 : 1; }
// ... and at most: with four computing waves and the loading wave, a
// 256-channel bf16 state slice leaves too few registers.
constexpr int recur_max_waves(bool bf16, int dk) { return (bf16 && dk >= 256) ? 2 : 4; }
bool recur_supported(int bf16, int C, int dk, int dv, int L);
// Per (batch-head, chunk) records, in the fragment-blocked layouts of
// gla_records.h: Q~ = Q ⊙ e^B and K~ = K ⊙ e^{b - B} (C x dk each, rows past
// the sequence zero), the chunk's gated score matrix P (C x C) and, for bf16,
// the low part of its diagonal blocks (C x 16); grec holds e^b then b per key
// channel, recur_grec_bytes(dk) bytes per chunk.
size_t recur_grec_bytes(int dk);
// Bytes of one chunk's packed P record (row blocks above the diagonal left out).
size_t recur_prec_bytes(int is_bf16, int C);
hipError_t launch_chunk_prep(const Plan& p, const void* q, const void* k, const float* la,
                             const void* v, void* qg, void* kg, float* grec, void* ph, void* pl,
                             hipStream_t s);
// Per (batch-head, segment p.NSEGR, d_v tile of 16 p.NWVR columns).
//   out = 1: o from the segment entry state (init = seg_in when NSEGR > 1,
//            else h0 or null); fin receives the final state when NSEGR == 1.
//   out = 0: the segment's local state from zero -> fin [BH][NSEGR][dk][dv],
//            its total log decay -> seg_g [BH][NSEGR][dk].
hipError_t launch_chunk_recur(const Plan& p, int out, const void* qg, const void* kg,
                              const void* ph, const void* pl, const float* grec, const void* v,
                              const float* init, void* o, float* fin, float* seg_g,
                              hipStream_t s);

// The two passes over the time-reversed sequence (bf16, C = 64): row p is
// row L - 1 - p of q, k, v and o in memory and takes the log gate of row
// L - p (0 at p = 0).  Given (q, k, v) = (k, q, dout) and init = dhT, the
// output is dv (papercache.org notes §4.2 chunkwise form, run backwards).
hipError_t launch_chunk_prep_rev(const Plan& p, const void* q, const void* k, const float* la,
                                 const void* v, void* qg, void* kg, float* grec, void* ph,
                                 void* pl, hipStream_t s);
hipError_t launch_chunk_recur_rev(const Plan& p, int out, const void* qg, const void* kg,
                                  const void* ph, const void* pl, const float* grec,
                                  const void* v, const float* init, void* o, float* fin,
                                  float* seg_g, hipStream_t s);

// ---- backward kernels (gla_bwd.hip) ----
// A (chunk score matrix) and dA = (dO V^T) ⊙ M per chunk, fp32 C x C blocks
// (Aw null: dA only).
// The recurrent backward's chunk-local cumsum of log alpha and masked dA =
// dO V^T in one launch (bf16, C = 64).
hipError_t launch_chunk_da_cum(const Plan& p, const void* v, const void* dout, const float* a,
                               float* cum, float* dA, hipStream_t s);
hipError_t launch_chunk_attn(const Plan& p, const void* q, const void* k, const void* v,
                             const void* dout, const float* cum, float* Aw, float* dAw,
                             hipStream_t s);
// dq, dk, chunk-local reverse cumsum of dlog b (into dla) and chunk totals.
// st_lo / dst_lo: low parts of the states (bf16 split), or null.
hipError_t launch_chunk_dqdk(const Plan& p, const void* q, const void* k, const void* v,
                             const void* dout, const float* cum, const void* st_n,
                             const void* st_lo, const void* dst_n, const void* dst_lo,
                             const float* dAw, void* dq, void* dk, float* dla, float* dlt,
                             hipStream_t s);
// The same with the inter-chunk terms (scaled) from dqi / dki [BH][L][dk]
// fp32 (bf16 I/O, C = 64, dk % 32 == 0), writing the whole dlog alpha: the
// later chunks' totals come from k_bwd_inter's running sums (qpre, ksuf, as
// BwdInterJob::tsum) and rs = rowsum(hT ⊙ dhT) [BH][dk].
hipError_t launch_chunk_dqdk_inter(const Plan& p, const void* q, const void* k, const float* cum,
                                   const float* dAw, const float* dqi, const float* dki, void* dq,
                                   void* dk, float* dla, const float* qpre, const float* ksuf,
                                   const float* rs, hipStream_t s);
hipError_t launch_chunk_dv(const Plan& p, const void* k, const void* dout, const float* cum,
                           const void* dst_t, const float* Aw, void* dv, hipStream_t s);
hipError_t launch_rowsum_state(const Plan& p, const float* hT, const float* dhT, float* rs,
                               hipStream_t s);
// One token of the recurrent form in place on the state (gla_decode.hip):
// state <- diag(e^{la}) state + k^T v, o = q state; q, k, la [BH][dk],
// v, o [BH][dv], state [BH][dk][dv] fp32.
hipError_t launch_decode(const Plan& p, const void* q, const void* k, const void* v,
                         const float* la, float* state, void* o, hipStream_t s);

// ---- general gate G = alpha^T beta (gla_ggate.hip) ----
// One pass of the general-gate recurrence over [BH][L] rows: state rows = the
// channels of q and k (dk), columns = those of v (dv); la [BH][L][dk] and
// lb [BH][L][dv] are the log row and column gates.  rev: the pass runs the
// sequence backwards, applying at its token u the gates of token L - u (none
// at u = 0).  init: [BH][dk][dv] (transposed, [BH][dv][dk], when init_t) or
// null; o [BH][L][dv] (or null) in the pass's dtype; o_off (or null) fp32, the
// output without its same-token term; fin
// (or null) receives the final state, multiplied by the gate of sequence
// token 0 (fin_la, fin_lb) when those are given.
struct GgPass {
  const void* q;
  const void* k;
  const void* v;
  const float* la;
  const float* lb;
  int dk, dv, rev;
  const float* init;
  int init_t;
  void* o;
  float* o_off;
  float* fin;
  const float* fin_la;
  const float* fin_lb;
};
// State rows are padded to the next of 16 (fp32 only), 32, 64, 128, 256;
// -1 past 256.
int gg_padded_dim(int is_bf16, int d);
// Record bytes of one pass over [BH][L] with d state rows.
size_t gg_pass_rec_bytes(int is_bf16, int BH, int L, int d);
// part 0 launches the per-chunk prep (records into rec), part 1 the recurrence.
// is_bf16: the records and arithmetic; in_bf16: the element type of q, k, v
// (bf16 inputs may feed an fp32 pass, not the reverse).
hipError_t launch_gg_pass(const GgPass& ps, int part, int is_bf16, int in_bf16, int BH, int L,
                          void* rec, hipStream_t s);
// Token groups of the gate-gradient kernels (their totals are [BH][groups][dk + dv]).
int gg_gate_groups(int L);
// dlog alpha, dlog beta by the closed form from dq32, dk32, dv32, o32 (fp32,
// without their same-token terms).  hs: [BH][dk + dv] scratch (used when dhT
// is given).
hipError_t launch_gg_gates(int is_bf16, int BH, int L, int dk, int dv, const void* q,
                           const void* k, const float* dq32, const float* dk32, const float* o32,
                           const void* dout, const void* v, const float* dv32, const float* hT,
                           const float* dhT, float* tot, float* hs, float* dla, float* dlb,
                           hipStream_t s);

// ---- the backward's inter-chunk terms with the states on chip (gla_bwd_recur.hip) ----
// One job of k_bwd_inter (bf16 rows): the output product X_y U scaled by
// Lambda (dq job, rev = 0, U = S^T, chunks in order) or Gamma (dk job,
// rev = 1, U = dS^T, chunks backwards), in fp32 to `out` [BH][L][dk]; U is
// updated with X_u^T (z ⊙ Gamma) (dq) or X_u^T (z ⊙ Lambda) (dk).  init:
// entering state [BH][dk][dv] (h0 or dhT) or null.  fin_rs (dq job):
// rowsum(hT ⊙ fin_with) [BH][dk] (zeros when fin_with is null).  fin_state
// (dk job): dh0 [BH][dk][dv].
struct BwdInterJob {
  const void* xy;
  const void* xu;
  const void* z;
  const float* init;
  float* out;
  float* fin_rs;
  const float* fin_with;
  float* fin_state;
  int rev;
  // the closed-form gate gradient's chunk sums of the inter term: tin is the
  // input multiplying it (q for the dq job, k for the dk job), tsum receives,
  // per chunk and half of the chunk's rows, sum_rows tin ⊙ term as a running
  // sum: inclusive prefix over chunks (dq job) or exclusive suffix (dk job),
  // [BH][NC][2][dk] fp32.  Both may be null (no sums).
  const void* tin;
  float* tsum;
};
bool bwd_inter_supported(int bf16, int C, int dk, int dv, int L);
hipError_t launch_bwd_inter(const Plan& p, const BwdInterJob& jq, const BwdInterJob& jk,
                            const float* cum, hipStream_t s);

// dla += rs + the dlog b totals of all later chunks (dlt [BH][NC][dk]).
hipError_t launch_dla_carry(const Plan& p, const float* dlt, const float* rs, float* dla,
                            hipStream_t s);

}  // namespace gla
