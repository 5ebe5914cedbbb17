/*
 * gla.h -- C ABI of the MI355X (gfx950) Gated Linear Attention library.
 *
 * The library computes the chunkwise-parallel forward and backward of the
 * GLA layer, per (batch, head):
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,      o_t = q_t S_t,
 *
 * with the row gate G_t = alpha_t^T 1 given as a = log alpha_t in R^{d_k}
 * ("Gated Linear Attention Transformers with Hardware-Efficient Training",
 * papercache.org notes §4.1 recurrent form; chunkwise form §4.2; secondary
 * chunking §4.3 / Figure 3; zako-mio deep-reading report ch. 2.3 and 3.4).
 * The output includes the current token, S_0 = h0 may come from a previous
 * segment (notes §2.2) and hT = S_L.  There is no normaliser and no scaling
 * of q inside the library (notes §2.1, unnormalised linear attention).
 *
 * Conventions for every entry point
 * ---------------------------------
 * Pointers    : device pointers (HIP) to contiguous row-major arrays, each
 *               16-byte aligned.  Outputs must not alias inputs or each other.
 * Layouts     : q, k, dq, dk, log_alpha, dlog_alpha : [B][H][L][dk]
 *               v, o, dout, dv                      : [B][H][L][dv]
 *               h0, hT, dhT, dh0                    : [B][H][dk][dv]
 * Dtypes      : q, k, v, o, dout, dq, dk, dv use the I/O dtype (GLA_FP32 or
 *               GLA_BF16, bf16 = IEEE binary32 upper half, rounded to nearest
 *               even).  log_alpha, dlog_alpha, h0, hT, dhT, dh0 are always
 *               fp32.  Accumulation is fp32 throughout.
 * Ownership   : the caller owns every buffer, including the workspace; the
 *               library never allocates, frees or synchronises.
 * Streams     : `stream` is a hipStream_t (NULL = the null stream).  All work
 *               is enqueued on it in order; calls return without waiting.
 * Errors      : validation happens before anything is enqueued, so any status
 *               other than GLA_OK or GLA_ERR_HIP means nothing was launched.
 *               GLA_ERR_HIP means a launch was rejected (hipGetLastError);
 *               faults during execution surface at the caller's next sync.
 *               NaN/Inf inputs are not checked; they propagate.
 * Determinism : no atomics; repeated calls give bitwise-identical results.
 * Shapes      : B, H, L >= 0 (L need not be a multiple of the chunk: the last
 *               chunk is padded with log alpha = 0, k = v = 0 rows that never
 *               reach memory).  chunk in {16, 32, 64} for GLA_FP32 and
 *               {32, 64} for GLA_BF16; subchunk == 16.  dk and dv multiples
 *               of 16 (GLA_FP32) or 32 (GLA_BF16), 16 <= dk <= 256,
 *               16 <= dv <= 512; B * H <= 65535 and L <= 2^24.  Otherwise
 *               GLA_ERR_SHAPE.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GLA_ABI_VERSION 2

typedef enum { GLA_FP32 = 0, GLA_BF16 = 1 } gla_dtype;

typedef enum {
  GLA_OK = 0,
  GLA_ERR_NULL = 1,      /* a required pointer (or dims) is NULL            */
  GLA_ERR_SHAPE = 2,     /* sizes outside the supported set                 */
  GLA_ERR_DTYPE = 3,     /* dtype is not a gla_dtype value                  */
  GLA_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                */
  GLA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required         */
  GLA_ERR_HIP = 6        /* the HIP runtime rejected a launch               */
} gla_status;

/* Problem sizes.  chunk = C (tokens per chunk), subchunk = c (tokens per
 * secondary chunk; papercache.org notes §4.3). */
typedef struct {
  int32_t B, H, L, dk, dv, chunk, subchunk;
} gla_dims;

/* ABI version of the loaded library (GLA_ABI_VERSION at build time). */
int gla_abi_version(void);

/* Static text for a status code ("unknown status" for other values). */
const char *gla_status_string(int status);

/* Bytes of device workspace gla_fwd / gla_bwd need for `dims` and `dtype`.
 * Writes *bytes and returns GLA_OK, or returns the validation error that the
 * matching call would return (then *bytes is left unchanged).  bytes != NULL. */
gla_status gla_fwd_workspace_size(const gla_dims *dims, int dtype, size_t *bytes);
gla_status gla_bwd_workspace_size(const gla_dims *dims, int dtype, size_t *bytes);

/* Forward (papercache.org notes §4.2-4.3; App. B forward listing).
 *   in : q, k [B,H,L,dk] and v [B,H,L,dv] in `dtype`; log_alpha [B,H,L,dk]
 *        fp32 (entries <= 0 expected; not checked); h0 [B,H,dk,dv] fp32 or
 *        NULL for zeros.
 *   out: o [B,H,L,dv] in `dtype`; hT [B,H,dk,dv] fp32, or NULL to skip.
 *   Steps on `stream` (default path): one pass over all chunks in parallel
 *   forms the chunk-local cumsum of log_alpha, Q ⊙ e^B, K ⊙ e^{b-B}, the
 *   chunk decay and the chunk's gated score matrix (MFMA between
 *   sub-chunks, fp32 on diagonal sub-blocks); a second pass walks the chunks
 *   in order with the state on chip and writes o (and hT).  Long sequences
 *   with few (batch, head) pairs are split into segments whose entry states
 *   come from a scan of the segments' local states.
 *   workspace: device memory of at least gla_fwd_workspace_size bytes,
 *   16-byte aligned, contents on entry irrelevant, clobbered on exit. */
gla_status gla_fwd(const gla_dims *dims, int dtype,
                   const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *h0,
                   void *o, float *hT,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Forward path selection and tuning for gla_fwd_ex (zeros: automatic).  The
 * paths compute the same function (papercache.org notes §4.2-4.3) and differ
 * in where the chunk states live (notes §3.3 / Figure 1: materialised in
 * memory, or kept on chip):
 *   GLA_FWD_AUTO          the two-pass forward wherever it supports the shape
 *                         (gla_fwd's choice), else the fused one, else the
 *                         materialised one;
 *   GLA_FWD_TWO_PASS      per-chunk prep pass over all chunks in parallel, then
 *                         a recurrence pass with the state on chip;
 *   GLA_FWD_FUSED         one pass per sequence segment with the state on chip
 *                         (C = 64, dk in {64, 128, 256} (fp32: 64, 128),
 *                         dv % 128 == 0);
 *   GLA_FWD_MATERIALIZED  chunk states S_{n-1} written to the workspace, then
 *                         one output pass over all chunks in parallel.
 * recur_waves (1, 2 or 4 computing waves of 16 state columns per recurrence
 * workgroup) and recur_segments (>= 1 sequence segments of the recurrence)
 * apply to the two-pass forward only.  A path or setting the shape does not
 * support gives GLA_ERR_SHAPE (no silent substitution). */
typedef enum {
  GLA_FWD_AUTO = 0,
  GLA_FWD_TWO_PASS = 1,
  GLA_FWD_FUSED = 2,
  GLA_FWD_MATERIALIZED = 3
} gla_fwd_algo;

typedef struct {
  int32_t algo;            /* gla_fwd_algo */
  int32_t recur_waves;     /* 0 = automatic */
  int32_t recur_segments;  /* 0 = automatic */
} gla_fwd_config;

/* gla_fwd with an explicit path and tuning; cfg == NULL is gla_fwd itself.
 * The workspace depends on the configuration: size it with
 * gla_fwd_ex_workspace_size for the same cfg. */
gla_status gla_fwd_ex_workspace_size(const gla_dims *dims, int dtype, const gla_fwd_config *cfg,
                                     size_t *bytes);
gla_status gla_fwd_ex(const gla_dims *dims, int dtype, const gla_fwd_config *cfg,
                      const void *q, const void *k, const void *v,
                      const float *log_alpha, const float *h0,
                      void *o, float *hT,
                      void *workspace, size_t workspace_bytes, void *stream);

/* ---- allocation-free forward ----
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gla_fwd's
 * two-pass path (GLA_FWD_TWO_PASS) with its scratch, the per-chunk records of
 * the prep pass (and the recurrence's segment states), in a static device
 * array of the library instead of a workspace argument.  The array holds
 * GLA_NOALLOC_SCRATCH_BYTES; each GPU the library runs on keeps its own copy
 * until the process ends.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine); on its first call on a device it looks up
 * that device's copy (hipGetSymbolAddress).
 *   Arguments, layouts, results and errors as gla_fwd, on the current device
 *   (the stream must belong to it).  Shapes outside the two-pass forward's
 *   (gla_fwd_ex_workspace_size with GLA_FWD_TWO_PASS refuses them) give
 *   GLA_ERR_SHAPE; shapes whose records exceed the array
 *   (gla_fwd_ex_workspace_size with GLA_FWD_TWO_PASS > GLA_NOALLOC_SCRATCH_BYTES;
 *   the GLA-340M layer shape B8 H4 L2048 dk128 dv256 bf16 needs 41 MiB, twice
 *   that batch 82 MiB) give GLA_ERR_WORKSPACE, both before anything is
 *   enqueued.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (different streams or threads, without ordering between them) race
 *   and give wrong results.  The kernels need no particular initial contents,
 *   so nothing is cleared between calls. */
#define GLA_NOALLOC_SCRATCH_BYTES (64u << 20)
gla_status gla_fwd_noalloc(const gla_dims *dims, int dtype,
                           const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *h0,
                           void *o, float *hT, void *stream);

/* Backward of gla_fwd for the loss gradients dout = dL/do and dhT = dL/dhT
 * (NULL for zeros).  States are recomputed, not read from a forward call
 * (zako-mio report ch. 2.2: materialise in the forward, recompute in the
 * backward).  The gate gradient uses the closed form
 *     dlog_alpha_t = sum_{i >= t} (q_i ⊙ dq_i - k_i ⊙ dk_i) + rowsum(hT ⊙ dhT)
 * (zako-mio report ch. 3.4; papercache.org notes §4.3, App. B; the last term
 * is the final-state path, zero when dhT is NULL).
 *   out: dq, dk [B,H,L,dk], dv [B,H,L,dv] in `dtype`; dlog_alpha [B,H,L,dk]
 *        fp32; dh0 [B,H,dk,dv] fp32, or NULL to skip.
 *   workspace: at least gla_bwd_workspace_size bytes, as for gla_fwd. */
gla_status gla_bwd(const gla_dims *dims, int dtype,
                   const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *h0,
                   const void *dout, const float *dhT,
                   void *dq, void *dk, void *dv, float *dlog_alpha, float *dh0,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Backward path selection for gla_bwd_ex (zeros: automatic).  Both paths
 * recompute the states rather than reading them from a forward call:
 *   GLA_BWD_AUTO          the recurrent path wherever it supports the shape
 *                         (gla_bwd's choice), else the materialised one;
 *   GLA_BWD_MATERIALIZED  the chunk states S_{n-1} and state gradients dS_n
 *                         are written to the workspace (bf16 high and low
 *                         parts) and read back per chunk;
 *   GLA_BWD_RECURRENT     no state leaves the chip: one launch walks the
 *                         chunks with the transposed state S^T (in order) and
 *                         dS^T (backwards) and emits the inter-chunk parts of
 *                         dq and dk; dv is the forward of the time-reversed
 *                         sequence (queries k, keys q, values dout, gates
 *                         shifted by one token, initial state dhT).  bf16 I/O,
 *                         chunk 64, dk % 32 == 0, dv in {128, 256}.
 * A path the shape does not support gives GLA_ERR_SHAPE. */
typedef enum {
  GLA_BWD_AUTO = 0,
  GLA_BWD_MATERIALIZED = 1,
  GLA_BWD_RECURRENT = 2
} gla_bwd_algo;

typedef struct {
  int32_t algo;  /* gla_bwd_algo */
} gla_bwd_config;

/* gla_bwd with an explicit path; cfg == NULL is gla_bwd itself.  Size the
 * workspace with gla_bwd_ex_workspace_size for the same cfg. */
gla_status gla_bwd_ex_workspace_size(const gla_dims *dims, int dtype, const gla_bwd_config *cfg,
                                     size_t *bytes);
gla_status gla_bwd_ex(const gla_dims *dims, int dtype, const gla_bwd_config *cfg,
                      const void *q, const void *k, const void *v,
                      const float *log_alpha, const float *h0,
                      const void *dout, const float *dhT,
                      void *dq, void *dk, void *dv, float *dlog_alpha, float *dh0,
                      void *workspace, size_t workspace_bytes, void *stream);

/* One token of the recurrent form, in place on the state (papercache.org
 * notes §2.1 and §4.1, recurrent form: the constant-memory inference step).
 * Per (batch, head), with a = log_alpha of the token:
 *     state <- diag(e^{a}) state + k^T v,      o = q state
 * (the output includes the token, as in gla_fwd).  Repeated calls over the
 * tokens of a sequence give gla_fwd's o and hT up to rounding.
 *   dims: B, H, dk, dv with gla_fwd's limits; L, chunk and subchunk are not
 *         used.
 *   in : q, k [B,H,dk] and v [B,H,dv] in `dtype`; log_alpha [B,H,dk] fp32.
 *   in/out: state [B,H,dk,dv] fp32, read and overwritten.
 *   out: o [B,H,dv] in `dtype` (must not alias the inputs or state).
 *   No workspace.  Errors as for gla_fwd; B * H == 0 is a no-op. */
gla_status gla_decode(const gla_dims *dims, int dtype,
                      const void *q, const void *k, const void *v,
                      const float *log_alpha, float *state, void *o, void *stream);

/* ---- general gate G_t = alpha_t^T beta_t (papercache.org notes, App. C) ----
 * The recurrence with an outer-product gate: log_alpha gates the d_k rows of
 * the state and log_beta its d_v columns,
 *     S_t = (alpha_t^T beta_t) ⊙ S_{t-1} + k_t^T v_t,     o_t = q_t S_t
 * (App. C.1 parallel form O = (((Q ⊙ B)(K / B)^T ⊙ M)(V / D)) ⊙ D with B, D
 * the cumulative products of alpha, beta; log_beta = 0 gives gla_fwd).  It is
 * computed chunkwise (App. C.2) in 16-token chunks; the chunk and subchunk
 * fields of dims are not used.
 *   dims: dk and dv multiples of 16 (GLA_FP32) or 32 (GLA_BF16), dk in
 *         [16, 256] and dv in [16, 512] (the GLA-1.3B head shape, dk 256 and
 *         dv 512, included); B * H <= 65535; otherwise GLA_ERR_SHAPE.
 *   in : q, k [B,H,L,dk], v [B,H,L,dv] in `dtype`; log_alpha [B,H,L,dk] and
 *        log_beta [B,H,L,dv] fp32 (entries <= 0 expected; not checked);
 *        h0 [B,H,dk,dv] fp32 or NULL for zeros.
 *   out: o [B,H,L,dv] in `dtype`; hT [B,H,dk,dv] fp32 or NULL to skip.
 *   workspace: at least ggla_fwd_workspace_size bytes, 16-byte aligned,
 *   clobbered.  Errors as for gla_fwd. */
gla_status ggla_fwd_workspace_size(const gla_dims *dims, int dtype, size_t *bytes);
gla_status ggla_bwd_workspace_size(const gla_dims *dims, int dtype, size_t *bytes);
gla_status ggla_fwd(const gla_dims *dims, int dtype,
                    const void *q, const void *k, const void *v,
                    const float *log_alpha, const float *log_beta, const float *h0,
                    void *o, float *hT,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Backward of ggla_fwd for dout = dL/do and dhT = dL/dhT (NULL for zeros).
 * dq, dk and dv are each a pass of the same recurrence with the roles of the
 * operands exchanged (dk and dv on the reversed sequence, gates shifted by
 * one token).  The gate gradients use App. C's closed form:
 *     dlog_alpha_t = sum_{i >= t} (q_i ⊙ dq_i - k_i ⊙ dk_i) + rowsum(hT ⊙ dhT)
 *     dlog_beta_t  = sum_{i >= t} (o_i ⊙ do_i - v_i ⊙ dv_i) + colsum(hT ⊙ dhT)
 *   out: dq, dk [B,H,L,dk], dv [B,H,L,dv] in `dtype`; dlog_alpha [B,H,L,dk],
 *        dlog_beta [B,H,L,dv] fp32; dh0 [B,H,dk,dv] fp32 or NULL to skip.
 *   workspace: at least ggla_bwd_workspace_size bytes, as for ggla_fwd. */
gla_status ggla_bwd(const gla_dims *dims, int dtype,
                    const void *q, const void *k, const void *v,
                    const float *log_alpha, const float *log_beta, const float *h0,
                    const void *dout, const float *dhT,
                    void *dq, void *dk, void *dv, float *dlog_alpha, float *dlog_beta,
                    float *dh0, void *workspace, size_t workspace_bytes, void *stream);

/* ---- launch profiling (measurement support; not part of the computation) ----
 * While enabled, every kernel launch made by the entry points above is
 * bracketed by two HIP events recorded on the launch stream, so per-kernel GPU
 * durations can be read back after the caller synchronises.  Records beyond
 * `capacity` are dropped.  Enabling creates the events (host-side HIP calls);
 * it must not be done inside a captured stream.  The record table is guarded
 * by a mutex, so launches from several threads may be profiled together (one
 * table per process; a begin while others launch restarts it).
 *   gla_profile_begin : enable and clear; capacity >= 1 records.
 *                       GLA_ERR_SHAPE if capacity < 1, GLA_ERR_HIP if the
 *                       events cannot be created.
 *   gla_profile_end   : disable (records stay readable until the next begin).
 *   gla_profile_count : number of records kept so far (dropped ones excluded).
 *   gla_profile_get   : name of the i-th record's kernel (static string) and its
 *                       duration in ms; GLA_ERR_SHAPE for a bad index,
 *                       GLA_ERR_NULL for NULL outputs, GLA_ERR_HIP if one of
 *                       its events could not be recorded or has not completed
 *                       (caller did not sync). */
gla_status gla_profile_begin(int capacity);
void gla_profile_end(void);
int gla_profile_count(void);
gla_status gla_profile_get(int index, const char **kernel, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
