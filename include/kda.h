/*
 * kda.h -- C ABI of libkda: the Kimi Delta Attention (KDA) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * KDA is the gated delta rule with one decay per key channel ("per-channel-decay
 * KDA"; page "spike(kimi-linear): chunk_kda prefill AOT port -- kernel set +
 * pinned-config recipe", section Delivered).  Per (sequence, head) it keeps an
 * fp32 state S with dk rows (key channels) and dv columns (value channels).
 * One token with query q, key k, value v, log-decay g (natural log, one value
 * per key channel) and write strength beta does
 *
 *     S <- (I - beta k k^T) Diag(exp(g)) S + beta k v^T
 *     o  = scale * S^T q                 (the state after the update)
 *
 * The pages run this in two forms (page "Kimi-Linear: paged-incremental decode
 * (prefill-once + carried-state decode)", squash commit): a chunked prefill
 * over the prompt that returns the final state, and a recurrent decode that
 * advances one token per call from the carried state and must read the state
 * it is given.  Those are the two entry points below.
 *
 * Conventions (borrowed from the versioned C ABI on page "model(kimi_linear):
 * ONE-SURFACE ROW 7 -- fold Kimi-Linear onto the shared paged runner",
 * section Landed: a version constant, explicit descriptors, loud failure):
 *   - Every descriptor starts with struct_size = sizeof(the struct); a
 *     mismatch returns KDA_ERR_VERSION.  Fields documented "0 = default" may be
 *     left zero.
 *   - All pointers except those marked "host" are DEVICE pointers on the
 *     current HIP device, owned by the caller.  The library allocates no device
 *     memory and keeps no state between calls; calls are re-entrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; no call synchronises.
 *   - Every argument check runs on the host before anything is enqueued; a
 *     failed check returns a negative kda_status and enqueues nothing.  A
 *     failed kernel launch returns KDA_ERR_HIP (kda_last_hip_error() has the
 *     hipError_t).  NaN/Inf in the data propagate; data is not inspected.
 *   - Tensors are dense row-major with the last index contiguous.  Alignment:
 *     16 bytes for everything read as vectors: q, k, v, g, the raw gate x,
 *     dt_bias, h0 and ht of a prefill; the state, q, k, g, x and dt_bias of
 *     a decode step.  Every other pointer (beta, o, a_log, the decode v, the
 *     index tables), its element size.
 *   - Supported: dk = dv = d in {32, 64, 128}; chunk in {16, 32, 64};
 *     dtype KDA_DTYPE_F32 or KDA_DTYPE_BF16 for q, k, v, beta and o.
 *     g is fp32.  h0, ht and the decode state are fp32, or bf16 when
 *     state_dtype asks for it (bf16 inputs only): the state dtype is a
 *     property of the state pool (page "model(kimi_linear): ONE-SURFACE ROW
 *     7", B3: the conv cache dtype mirrors kda_state_dtype).  The
 *     arithmetic stays fp32; a bf16 state is rounded (to nearest even) once
 *     per call when it is written.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 5

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL                      */
  KDA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be,
                               or too large: t_total <= 2^31 - 65, and for a
                               prefill n_seqs * n_heads * (dk / 16) and
                               (t_total / chunk + n_seqs) * n_heads below 2^31 */
  KDA_ERR_DTYPE = -3,       /* dtype is not one of kda_dtype                   */
  KDA_ERR_UNSUPPORTED = -4, /* head dim, chunk size or plan not supported     */
  KDA_ERR_ALIGN = -5,       /* a pointer breaks its alignment rule (below)     */
  KDA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
  KDA_ERR_HIP = -7,         /* a HIP launch failed; see kda_last_hip_error()   */
  KDA_ERR_VERSION = -8,     /* struct_size does not match this library        */
  KDA_ERR_ALIAS = -9,       /* an output overlaps an input it may not overlap  */
  KDA_ERR_SEQLENS = -10,    /* cu_seqlens content invalid (reported through
                               kda_workspace_status, never by a call's return) */
  KDA_ERR_SYNC = -11        /* reserved: no kernel of this version reports it */
} kda_status;

typedef enum { KDA_DTYPE_F32 = 1, KDA_DTYPE_BF16 = 2 } kda_dtype;

/* Decay input.  GIVEN: the caller passes g, the natural-log decay, fp32.
 * KIMI: the gate activation is computed inside the kernels from the raw gate
 * x (dtype of q), a per-head a_log [H] and a per-(head, channel) dt_bias
 * [H, dk], both fp32:  g = -exp(a_log[h]) * softplus(x + dt_bias[h, c]),
 * softplus(z) = log(1 + e^z).  The pages run this activation fused into the
 * chunked forward (page "spike(kimi-linear): chunk_kda prefill AOT port",
 * commit message: the gate/cumsum kernel of chunk_kda_with_fused_gate); the
 * formula is the Kimi-Linear gate of the workload definition.  Fusing it
 * means the kernels read x in the input dtype instead of an fp32 g. */
typedef enum { KDA_GATE_GIVEN = 0, KDA_GATE_KIMI = 1 } kda_gate;

typedef struct {
  int32_t mode;               /* kda_gate; 0 = g given                          */
  const void* x;              /* KIMI: raw gate [.., H, dk], dtype of q         */
  const float* a_log;         /* KIMI: [H] fp32                                 */
  const float* dt_bias;       /* KIMI: [H, dk] fp32                             */
} kda_gate_desc;

/* Launch plan of the chunked prefill.  TWO_PASS (what AUTO selects) writes
 * the chunk-local results to the workspace and reads them back in the state
 * scan.  FUSED is a reserved value: this library does not build such a plan,
 * and a request for it returns KDA_ERR_UNSUPPORTED before anything is
 * launched. */
typedef enum { KDA_PLAN_AUTO = 0, KDA_PLAN_FUSED = 1, KDA_PLAN_TWO_PASS = 2 } kda_plan;

/* Chunked prefill over a packed batch of N sequences (T_total tokens).
 *
 * Computes, for every sequence n and head h, the recurrence above over the
 * tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 starting from h0[n,h] (zero when
 * h0 is NULL), writes o for every token and the final state to ht[n,h].  The
 * chunked form (cumulative decay, decayed K K^T, triangular solve, W/U, state
 * recurrence, output; page "spike(kimi-linear): chunk_kda prefill AOT port",
 * commit message) gives the same result as the token loop up to rounding, for
 * any chunk size.
 *
 * Layouts: q, k [T_total, Hg, dk]; g [T_total, H, dk]; v, o [T_total, H, dv];
 * beta [T_total, H]; h0, ht [N, H, dk, dv].  Hg = n_k_heads key/query heads
 * are shared by groups of H / Hg consecutive value heads: value head h reads
 * key head h / (H / Hg) (Hg = H, the default, is one key head per head).  An
 * empty sequence (length 0) writes no o and sets ht = h0 (zeros when h0 is
 * NULL).
 *
 * qk_l2norm = 1 normalises every q and k row (one token, one key head) inside
 * the kernels before use: q / sqrt(sum q^2 + 1e-6), in fp32.
 *
 * cu_seqlens: device int32 [N + 1], cu[0] = 0, non-decreasing,
 * cu[N] = t_total.  May be NULL only when n_seqs == 1.  Its contents are read
 * on the device only: when they break these rules no o and no ht is written
 * and kda_workspace_status() returns KDA_ERR_SEQLENS.
 *
 * Aliasing: ht may equal h0 (in-place carry).  o must not overlap any input.
 * g is expected to be <= 0 (a decay); positive values are computed exactly as
 * written but lose the bounds that keep the chunked factors in range. */
typedef struct {
  uint32_t struct_size;       /* sizeof(kda_prefill_desc)                       */
  int32_t dtype;              /* kda_dtype of q, k, v, beta, o                  */
  int32_t n_seqs;             /* N >= 1                                         */
  int32_t n_heads;            /* H >= 1                                         */
  int32_t dk, dv;             /* head dims; dk == dv in {32, 64, 128}           */
  int32_t chunk;              /* 0 = 64; else 16, 32 or 64                      */
  int32_t plan;               /* kda_plan; 0 = auto                             */
  int64_t t_total;            /* packed tokens, >= 0                            */
  float scale;                /* 0 = dk^-1/2                                    */
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const void* h0;             /* NULL = zero initial state; state_dtype         */
  const int32_t* cu_seqlens;  /* NULL allowed when n_seqs == 1                  */
  void* o;
  void* ht;                   /* NULL = final state not returned; state_dtype  */
  kda_gate_desc gate;         /* g, or the raw gate and its parameters; g may  */
                              /* be NULL when gate.mode = KIMI                 */
  const int32_t* state_indices; /* NULL, or device [N]: h0 and ht are state    */
                              /* pools [n_slots, H, dk, dv] and sequence n     */
                              /* reads h0[state_indices[n]], writes ht[..] ;   */
                              /* a negative index (or one >= n_slots) skips    */
                              /* the sequence: no o, no state.  Indices must   */
                              /* be distinct.                                  */
  int32_t n_slots;            /* pool size when state_indices is set           */
  int32_t n_k_heads;          /* Hg, dividing H; 0 = H                         */
  int32_t qk_l2norm;          /* 1 = L2-normalise q and k rows in the kernels  */
  int32_t state_dtype;        /* kda_dtype of h0 and ht; 0 = fp32              */
} kda_prefill_desc;

/* One recurrent decode step for a batch of N sequences, one token each.
 * state [N, H, dk, dv] fp32 is read and updated IN PLACE; q, k [N, Hg, dk];
 * g [N, H, dk]; v, o [N, H, dv]; beta [N, H].  n_k_heads and qk_l2norm as in
 * kda_prefill_desc.  o must not overlap state or any input. */
typedef struct {
  uint32_t struct_size;       /* sizeof(kda_decode_desc)                        */
  int32_t dtype;              /* kda_dtype of q, k, v, beta, o                  */
  int32_t n_seqs;             /* N >= 0 (0 = nothing to do)                     */
  int32_t n_heads;            /* H >= 1                                         */
  int32_t dk, dv;             /* dk == dv in {32, 64, 128}                      */
  float scale;                /* 0 = dk^-1/2                                    */
  void* state;                /* state_dtype (fp32 unless asked for bf16)       */
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  void* o;
  kda_gate_desc gate;         /* as in kda_prefill_desc; x is [N, H, dk]        */
  const int32_t* state_indices; /* NULL, or device [N]: state is a pool        */
                              /* [n_slots, H, dk, dv], sequence n updates slot */
                              /* state_indices[n]; negative (or >= n_slots)    */
                              /* skips it (no o).  Indices must be distinct.   */
  int32_t n_slots;            /* pool size when state_indices is set           */
  int32_t n_k_heads;          /* Hg, dividing H; 0 = H                         */
  int32_t qk_l2norm;          /* 1 = L2-normalise q and k in the kernel        */
  int32_t state_dtype;        /* kda_dtype of the state; 0 = fp32              */
} kda_decode_desc;

/* Recurrent prefill: the same computation as kda_chunk_prefill (same
 * descriptor; chunk and plan are ignored, no workspace), run token by token
 * with each (sequence, head) state held on chip from the first token to the
 * last.  For continuing prefills of a few tokens on a carried state, where
 * the chunked form has nothing to amortise (page "model(kimi_linear):
 * ONE-SURFACE ROW 7 -- fold Kimi-Linear onto the shared paged runner", B2:
 * the recurrent op serves decode and continuing prefills).  cu_seqlens is
 * read clamped to [0, t_total]: contents that break the rules give
 * unspecified o and ht but no access out of bounds.  fp32 and bf16 at every
 * supported head dim. */
int kda_recurrent_prefill(const kda_prefill_desc* d, void* stream);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Static text for a kda_status value ("unknown status" otherwise). */
const char* kda_status_string(int status);

/* hipError_t behind the last KDA_ERR_HIP returned on this thread (0 if none). */
int kda_last_hip_error(void);

/* Bytes of device workspace kda_chunk_prefill needs for this descriptor
 * (depends on n_seqs, n_heads, dk, dv, chunk, dtype and t_total only).
 * Returns 0 when the descriptor is invalid; *status (host, may be NULL)
 * receives the kda_status of the check. */
size_t kda_chunk_prefill_workspace_bytes(const kda_prefill_desc* d, int* status);

/* Enqueue the chunked prefill on `stream`.  workspace: device buffer of at
 * least kda_chunk_prefill_workspace_bytes(d) bytes, 256-byte aligned, owned by
 * the caller, not shared with a concurrent call.  Returns a kda_status. */
int kda_chunk_prefill(const kda_prefill_desc* d, void* workspace, size_t workspace_bytes,
                      void* stream);

/* kda_chunk_prefill that also records four caller-created hipEvent_t handles
 * (passed as void*) on `stream`: events[0] before the first launch, then one
 * after each of the three launches (chunk map, chunk-local stage, state scan),
 * so the caller can time each stage.  events may be NULL (no recording). */
int kda_chunk_prefill_timed(const kda_prefill_desc* d, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events);

/* Device-side status of the last prefill that used `workspace`: KDA_OK or
 * KDA_ERR_SEQLENS.  Copies one int to the host and synchronises `stream`.
 * Returns KDA_ERR_HIP if the copy fails. */
int kda_workspace_status(const void* workspace, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kda_chunk_prefill with its workspace taken from a buffer of
 * KDA_NOALLOC_WORKSPACE_BYTES that the library holds in static device memory,
 * one per device, until the process ends (its address is looked up on the
 * first call on each device).  The call allocates nothing; the caller passes
 * every input and output as for kda_chunk_prefill.  Returns
 * KDA_ERR_WORKSPACE, before anything is enqueued, when
 * kda_chunk_prefill_workspace_bytes(d) exceeds the buffer (64 MiB: at H = 32,
 * dk = dv = 128, chunk 64 that is t_total / 64 + n_seqs <= 25 chunks, one
 * sequence of up to 1,536 tokens).  Every call on a device shares that device's buffer and
 * leaves its contents behind: calls on one stream are ordered, but calls that
 * overlap on one device (other streams, other threads) race and must not be
 * issued.  The device status word that kda_workspace_status reads for the
 * other entry point lives in this buffer and is not exposed: invalid
 * cu_seqlens contents write no o and no ht, unreported. */
#define KDA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
int kda_chunk_prefill_noalloc(const kda_prefill_desc* d, void* stream);

/* Enqueue one recurrent decode step on `stream`.  Returns a kda_status. */
int kda_recurrent_decode(const kda_decode_desc* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
