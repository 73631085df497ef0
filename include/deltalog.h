/*
 * deltalog.h -- C ABI of the DeltaLog decode library for AMD MI355X (gfx950).
 *
 * What it computes.  "DeltaLog: Deferred Materialization of Recurrent States
 * for Linear Attention Decoding" (newx.sg page, Abstract) keeps a linear
 * attention layer's recurrent state as two parts, a dense base and a log of
 * bounded length that holds the latest low-rank updates.  A typical decode step
 * only adds one update's factors to the log; now and then a merge folds the
 * logged updates into the base; and every output is the one eager decoding
 * (read the whole state, update it, write it back after each token) would
 * give.  The page's AI Summary says the same: small appends take the place of
 * whole-state write-backs.  This library implements that
 * scheme, and the eager comparator, for three recurrences the page names
 * (GDN, KDA, RWKV6).  With S the dk x dv state of one head, rows indexed by key
 * channel, and one decode step t:
 *
 *   GDN   D = alpha_t S,        u = beta_t (v - D^T k),  S' = D + k u^T,  o = S'^T q
 *   KDA   D = diag(a_t) S,      u and S' as GDN,                          o = S'^T q
 *   RWKV6 o = S^T r + (sum_i r_i bonus_i k_i) v,          S' = diag(w_t) S + k v^T
 *
 * (Gated decay plus a delta-rule write that subtracts the current read: the
 * Kaczmarz Linear Attention and Gated DeltaNet-2 abstracts on the card pages;
 * KDA's channel-wise decay: Gated DeltaNet-2 abstract.  RWKV6 is only named by
 * the pages; the form above is the standard one.)
 *
 * Deferred form kept by the pool.  c is the cumulative log2-decay since the
 * last merge (a scalar per entry for GDN, a dk-vector for KDA and RWKV6):
 *   S_t = diag(2^c_t) B + sum_j diag(2^(c_t - c_j)) k_j u_j^T
 * where B is the base and entry j = (k_j, u_j, c_j) is the rank-1 write of step
 * j (u_j = v_j for RWKV6).  Each step's log2 decay is clamped below at -126.
 *
 * Schedule.  Between calls every tile's fill n is in [0, L).  A decode step
 * appends to slot n; when that makes n + 1 == L the same step folds all L
 * updates into the base instead (the base is rewritten, the slot is not) and
 * the fill returns to 0.  All heads of one sequence share one fill value;
 * it is stored per (sequence, head) so each tile has a single reader/writer.
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device pointers the caller owns
 *    (allocate them with PyTorch or hipMalloc); the library allocates no
 *    device memory, keeps no state between calls and is reentrant for
 *    distinct pools.  Every array is C-contiguous in the layout given.  Arrays
 *    with one scalar per tile (fill, out, beta, GDN's decay and log_c) must be
 *    4-byte aligned, every other device pointer 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; calls on one pool must be serialized on one stream.
 *  - Return value: DL_OK or a negative status.  All argument checks happen on
 *    the host before anything is enqueued, so a failed check leaves device
 *    memory untouched.  A launch failure reported by the runtime returns
 *    DL_EHIP.  Device-side faults surface at the caller's next stream sync.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).
 */
#ifndef DELTALOG_H
#define DELTALOG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DL_GDN = 0, DL_KDA = 1, DL_RWKV6 = 2 } dl_variant;

enum {
  DL_OK = 0,
  DL_EINVAL = -1,       /* null required pointer, bad dims, L outside [1,128], fill outside [0,L),
                           unknown base_dtype */
  DL_EUNSUPPORTED = -2, /* dk or dv not 64/128, or a pointer given/missing for this variant */
  DL_EALIGN = -3,       /* a device pointer is not aligned as required (16 or 4 bytes) */
  DL_EHIP = -4          /* the HIP runtime reported an error when enqueuing */
};

#define DL_MAX_LOG_LEN 128

/* Storage type of the base state. */
enum { DL_BASE_F32 = 0, DL_BASE_BF16 = 1 };

/* Shape of one pool.  batch >= 0 (0: every call returns DL_OK at once, after
 * checking only the other dims, and no pointer is looked at), heads >= 1,
 * dk, dv in {64, 128}, 1 <= log_len (L) <= DL_MAX_LOG_LEN, batch*heads < 2^31. */
typedef struct {
  int32_t variant; /* dl_variant */
  int32_t batch;
  int32_t heads;
  int32_t dk;
  int32_t dv;
  int32_t log_len;
  int32_t base_dtype; /* DL_BASE_F32, or DL_BASE_BF16: a low-bit base.  The log and all
                         arithmetic stay fp32; the base is rounded to bf16 (to nearest,
                         ties to even) only where it is written: at init and at folds.
                         Every output then reads the bf16 base together with the
                         pending updates kept in fp32 (the scheme of the LeapQuant
                         abstract, on the FPGA-titled card page). */
} dl_dims;

/* The per-layer state pool (all device, caller-owned).  G = 1 for GDN, dk otherwise. */
typedef struct {
  void *base;      /* fp32 (or bf16) [batch][heads][dk][dv]  base state B (rows = key channels) */
  uint16_t *log_k; /* bf16 [batch][heads][L][dk]   keys of the logged updates                  */
  void *log_u;     /* GDN/KDA: fp32 [batch][heads][L][dv] factors u_j;
                      RWKV6:   bf16 [batch][heads][L][dv] values v_j                          */
  float *log_c;    /* fp32 [batch][heads][L][G]    cumulative log2-decay since the last merge  */
  int32_t *fill;   /* int32 [batch][heads]         entries in the log, in [0, L)              */
} dl_pool;

/* One decode step's inputs and output (all device). */
typedef struct {
  const uint16_t *q;   /* bf16 [batch][heads][dk]  query (RWKV6: receptance r)                  */
  const uint16_t *k;   /* bf16 [batch][heads][dk]  key                                          */
  const uint16_t *v;   /* bf16 [batch][heads][dv]  value                                        */
  const float *decay;  /* GDN: fp32 [batch][heads] alpha; KDA/RWKV6: fp32 [batch][heads][dk];
                          values in (0, 1]                                                      */
  const float *beta;   /* GDN/KDA: fp32 [batch][heads] step size; RWKV6: must be NULL           */
  const float *bonus;  /* RWKV6: fp32 [heads][dk]; GDN/KDA: must be NULL                        */
  float *out;          /* fp32 [batch][heads][dv]  this step's output (written)                 */
  const float *eta;    /* GDN/KDA, instead of beta: fp32 [batch][heads]; the step size is then
                          the Kaczmarz one, beta = eta / (||k||^2 + eps) with k as passed
                          (Kaczmarz Linear Attention abstract).  RWKV6: must be NULL.           */
  float eps;           /* the eps above, >= 0 (ignored when eta is NULL)                        */
} dl_step_io;

/* Start a pool (DeltaLog Abstract: the dense base plus an initially empty or
 * partly filled log).  Copies `init_base` (device, fp32 [batch][heads][dk][dv];
 * NULL = all-zero state; equal to pool->base = keep the base as it is; must not
 * otherwise overlap it) into the base, sets every
 * head of sequence b to fill init_fill[b] (host, int32 [batch]; NULL = all 0)
 * and zeroes the whole log, so a non-zero start fill is that many phantom
 * entries (k = 0, u = 0, c = 0) that change nothing but the merge phase.
 * Synchronizes `stream` before returning (init_fill is read on the host).
 * Errors: DL_EINVAL if init_fill[b] is outside [0, L). */
int dl_init_state(const dl_dims *dims, const dl_pool *pool, const float *init_base,
                  const int32_t *init_fill, void *stream);

/* One decode step for every (sequence, head) of the pool (DeltaLog Abstract:
 * the read and output come from base plus log; the step appends one compact
 * update; a step that fills the log merges it into the base).  Reads the base
 * but never writes it except on merging steps; writes io->out, one log entry
 * per tile, and the fills.  A tile whose fill lies outside [0, L) (a pool that was
 * never started) is left untouched.  Errors: DL_EINVAL for null q/k/v/decay/out or
 * pool arrays, or eps < 0 with eta set; DL_EUNSUPPORTED if beta/eta/bonus presence
 * does not match the variant (GDN/KDA: exactly one of beta and eta; RWKV6: bonus only). */
int dl_decode_step(const dl_dims *dims, const dl_pool *pool, const dl_step_io *io, void *stream);

/* Merge modes: the two named values of dl_merge's min_fill. */
enum {
  DL_MERGE_DUE = 0, /* fold only logs that are due, i.e. full: a decode step folds a log in
                       the same call that fills it, so between calls none is due and this
                       mode leaves the pool unchanged (after the argument checks)          */
  DL_MERGE_ALL = 1  /* fold every non-empty log: min_fill = 1                               */
};

/* Fold the log of every tile whose fill is >= min_fill (0 <= min_fill <= L; a
 * tile whose fill lies outside [0, L) is left untouched) into its base and set
 * its fill to 0 (DeltaLog Abstract: the merge that
 * moves logged updates into the base).  min_fill = DL_MERGE_ALL (1) folds
 * every non-empty log, after which `base` holds the dense state S_t of every
 * tile (for a checkpoint, or to read the state); min_fill = DL_MERGE_DUE (0)
 * folds only full logs, of which there are none between calls.  Errors:
 * DL_EINVAL for min_fill outside [0, L]. */
int dl_merge(const dl_dims *dims, const dl_pool *pool, int32_t min_fill, void *stream);

/* Arithmetic unit of a fold, for dl_merge_on. */
enum {
  DL_UNIT_AUTO = 0, /* what dl_merge uses: the unit measured faster for the pool's shape and L */
  DL_UNIT_VALU = 1, /* vector FMAs; the tile is streamed once per 16 or 32 staged entries     */
  DL_UNIT_MFMA = 2  /* v_mfma_f32_4x4x1_16b_f32 (fp32 products and sums); the tile stays in
                       registers, one read and one write at any log length                  */
};

/* dl_merge with the fold's arithmetic unit named by the caller (the merge of
 * the DeltaLog Abstract, a rank-n update of each base, n = the tile's fill).
 * On an fp32 base both units give the same bits: each scales the base, then
 * adds the entries one at a time in log order with one fused multiply-add per
 * element.  A bf16 base is rounded once by the MFMA fold and once per stage of
 * 16 entries (32 at 64 x 64) by the vector fold.  min_fill as for dl_merge
 * (DL_MERGE_DUE, DL_MERGE_ALL or a threshold up to L).  Errors: those of
 * dl_merge, and DL_EINVAL for a unit outside the enum above. */
int dl_merge_on(const dl_dims *dims, const dl_pool *pool, int32_t min_fill, int32_t unit, void *stream);

/* The arithmetic unit dl_merge uses for pools of this shape, base type and log length:
 * DL_UNIT_VALU or DL_UNIT_MFMA (the table measured on MI355X, in api.cpp), or a
 * negative status for invalid dims.  Host only: touches no device memory. */
int dl_merge_unit(const dl_dims *dims);

/* The eager comparator (DeltaLog Abstract: the usual decoder, which rewrites
 * the whole recurrent state after each generated token): reads `state` (device,
 * fp32 [batch][heads][dk][dv]), writes the updated state in place and io->out.
 * dims->log_len is ignored (may be any value in [1, 128]); base_dtype must be
 * DL_BASE_F32 (else DL_EUNSUPPORTED). */
int dl_eager_step(const dl_dims *dims, float *state, const dl_step_io *io, void *stream);

/* A prompt's inputs and outputs for dl_prefill (all device).  T = tokens >= 0;
 * row t of a sequence is its t-th prompt token. */
typedef struct {
  const uint16_t *q;   /* bf16 [batch][T][heads][dk]  (RWKV6: receptance r)                    */
  const uint16_t *k;   /* bf16 [batch][T][heads][dk]                                           */
  const uint16_t *v;   /* bf16 [batch][T][heads][dv]                                           */
  const float *decay;  /* GDN: fp32 [batch][T][heads] alpha; KDA/RWKV6: fp32 [batch][T][heads][dk];
                          values in (0, 1]                                                      */
  const float *beta;   /* GDN/KDA: fp32 [batch][T][heads], or NULL with eta; RWKV6: NULL        */
  const float *bonus;  /* RWKV6: fp32 [heads][dk]; GDN/KDA: NULL                                */
  float *out;          /* fp32 [batch][T][heads][dv]  every token's output (written)            */
  const float *eta;    /* GDN/KDA instead of beta: fp32 [batch][T][heads], the Kaczmarz step
                          size beta = eta / (||k||^2 + eps) (Kaczmarz Linear Attention abstract) */
  float eps;           /* >= 0 (ignored when eta is NULL)                                       */
  int32_t tokens;      /* T                                                                     */
} dl_prefill_io;

/* Prefill: run the recurrence over T prompt tokens for every (sequence, head),
 * starting from the dense state the pool stands for, and leave the state after
 * the last token in the base with an empty log, ready for dl_decode_step.  Every
 * token's output is written.  The result equals T eager steps; it is computed
 * chunk by chunk in the chunkwise-parallel form that the Q-Delta, Kaczmarz
 * Linear Attention and Gated DeltaNet-2 abstracts (card pages) name for
 * delta-rule models: within a chunk, the delta-rule writes come from a
 * triangular solve (the WY form) and every product with the state is a matrix
 * product.  Any non-empty log is folded into the base first, as dl_merge with
 * min_fill = 1 would.  With a bf16 base the final state is rounded once.
 * All three variants; for KDA and RWKV6 (a decay per key channel) the
 * decay-weighted products inside a chunk are split around a reference token
 * per half chunk and run on matrix units when no channel decays by more than
 * 2^-60 over half a chunk, else they are formed pair by pair.  Errors:
 * DL_EINVAL for tokens < 0, heads > 131071 (a chunk's rows of one sequence are
 * addressed with 32-bit offsets), null q/k/v/decay/out, or eps < 0 with eta set;
 * DL_EUNSUPPORTED if beta/eta/bonus do not match the variant (GDN/KDA: exactly
 * one of beta and eta, no bonus; RWKV6: bonus only).  tokens == 0 only folds
 * the logs and looks at no prompt pointer. */
int dl_prefill(const dl_dims *dims, const dl_pool *pool, const dl_prefill_io *io, void *stream);

/* A static, human-readable name for a status code (never NULL). */
const char *dl_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_H */
