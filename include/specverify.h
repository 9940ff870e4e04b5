/*
 * specverify.h -- C ABI of the speculative-decoding verification sampler
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (velog "6-1편. Speculative Decoding", section 2 "알고리즘
 * 4단계", steps 2-4, and sections 2-1 and 2-2): for every sequence b of a
 * batch, given the target logits of gamma_b + 1 positions, the draft logits
 * of gamma_b positions, the gamma_b drafted tokens x_i and gamma_b + 1
 * uniforms u_i, compute p_i = softmax(target_i / T_b) and
 * q_i = softmax(draft_i / T_b), accept x_i while u_i < min(1, p_i(x_i) /
 * q_i(x_i)), and at the first rejection n emit one token sampled (inverse
 * CDF, token order, uniform u_gamma) from norm(max(0, p_n - q_n)); if all
 * gamma_b drafts are accepted emit a bonus token sampled from p_gamma.
 * With T_b = 0 the rule is greedy: accept while x_i equals argmax of the
 * target logits, emit that argmax at the first mismatch, or the argmax of
 * the last position as the bonus ("How to Scale Your Model -- All About
 * Transformer Inference", Appendix D "Speculative Sampling").  The
 * accepted length stays on the device, so the caller needs no
 * device-to-host synchronisation to consume it (Perplexity "Accelerating
 * Sonar through speculation", section "단일 토큰에 대한 MTP 스케줄링": the
 * sync on the accepted length is what extra GPU work avoids).
 *
 * Token-only drafts.  A drafter that proposes tokens without a distribution
 * (an n-gram or token-matching drafter: velog "6-1편. Speculative Decoding",
 * section 4, N-gram; "How to Scale Your Model", Appendix D) passes
 * draft_logits = NULL with its tokens.  Its distribution is then the point
 * mass q_i = delta_{x_i}, and the same rule gives: accept while u_i < p_i(x_i);
 * the residual is p_n without x_n, renormalised; q(x) = 1, beta = p(x),
 * Z = 1 - p(x); greedy (T = 0) accepts while x_i is the target argmax.  Only
 * the target logits are read.
 *
 * Packed ragged layout.  Sequence b owns draft rows cu_draft[b] ..
 * cu_draft[b+1] - 1 and target rows cu_t[b] .. cu_t[b] + gamma_b with
 * cu_t[b] = cu_draft[b] + b (so R_t = R_d + B target rows in total).
 * A uniform draft length is the special case cu_draft[b] = b * gamma.
 * cu_draft must be non-decreasing with cu_draft[0] = 0, cu_draft[B] = R_d
 * and every gamma_b <= max_gamma; if it is not, every sequence reports
 * accepted_len -1 and every out_tokens entry is -1, and no memory outside
 * the declared buffers is touched for any cu_draft.
 *
 * Ownership.  The caller owns every input and output buffer (device
 * memory).  A handle owns only its device workspace, allocated in
 * specverify_create and freed in specverify_destroy.  specverify_run
 * allocates nothing, never synchronises and is asynchronous on the given
 * stream; consumers of the outputs must be ordered after it on that
 * stream.  One handle must not have two runs in flight on different
 * streams at once (they share the workspace); destroy only after the
 * caller has synchronised with its last run.
 *
 * Errors.  Problems visible on the host (NULL pointers, sizes beyond the
 * handle's limits, logits not aligned to their element size) return a
 * status before any launch.
 * Problems in the data are detected on the device per sequence and
 * reported in accepted_len: -1 = invalid data (a NaN or +inf logit in any
 * of the sequence's rows, a row of only -inf, a drafted token outside
 * [0, V), a temperature that is negative, not finite or in (0, FLT_MIN), a
 * uniform of the sequence outside [0, 1) or NaN -- uniforms are draws from
 * the unit interval, velog page, section 2 step 3), -2 = internal error:
 * statistics of one of the sequence's rows were still missing after the
 * bounded wait and its recomputation (not expected to happen; the kernels
 * always terminate).  The tokens of such a sequence are -1 and its
 * diagnostics unspecified.
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct specverify_ctx* specverify_handle;

typedef enum {
  SPECVERIFY_OK = 0,
  SPECVERIFY_ERR_INVALID_ARGUMENT = 1, /* bad pointer / size / config     */
  SPECVERIFY_ERR_UNSUPPORTED = 2,      /* unaligned logits, V too big     */
  SPECVERIFY_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed     */
  SPECVERIFY_ERR_DEVICE = 4,           /* HIP runtime / launch failure    */
  SPECVERIFY_ERR_TOO_LARGE = 5         /* run_static: beyond its scratch  */
} specverify_status;

typedef enum { SPECVERIFY_F32 = 0, SPECVERIFY_BF16 = 1 } specverify_dtype;

/* Fixed per handle.  Limits: 1 <= vocab <= 262144 (at most 128 chunks of
 * 4 KB per bf16 row, 256 per f32 row), max_batch >= 1,
 * 0 <= max_gamma <= 255, max_batch * (max_gamma + 1) <= 2^24.  create also
 * returns UNSUPPORTED on a device too small to keep one row's chunks in
 * flight together (fewer than 8 * chunks resident waves). */
typedef struct {
  int32_t max_batch;   /* largest B a run may use                                 */
  int32_t max_gamma;   /* largest draft length; bounds R_t <= max_batch*(max_gamma+1) */
  int32_t vocab;       /* V of every logits row                                   */
  int32_t dtype;       /* specverify_dtype of both logits tensors                 */
  int32_t device;      /* HIP device ordinal the workspace lives on               */
  int32_t spin_limit;  /* polls for other waves' chunk statistics before a wave
                          computes the missing ones itself (0 = default, 64; at
                          most 2^20); any value gives the same results             */
} specverify_config;

/* Inputs of one run; every pointer is device memory. */
typedef struct {
  int32_t batch;              /* B >= 0 (0 = nothing to do)                        */
  int32_t gamma;              /* uniform draft length, used iff cu_draft == NULL   */
  const int32_t* cu_draft;    /* [B+1] prefix offsets of draft rows, or NULL       */
  int32_t num_draft_rows;     /* R_d = cu_draft[B] (host copy), used iff cu_draft  */
  const void* target_logits;  /* [R_t, target_stride] f32 or bf16; when both tensors'
                                 rows start on 16-byte boundaries and V * esize is a
                                 multiple of 16 the kernels use 16-byte loads, else
                                 element loads                                      */
  int64_t target_stride;      /* elements between rows, >= V                       */
  const void* draft_logits;   /* [R_d, draft_stride]; NULL = token-only drafts      */
  int64_t draft_stride;
  const int32_t* draft_tokens;/* [R_d] drafted ids x_i; may be NULL iff R_d == 0   */
  const float* uniforms;      /* [R_t] u in [0,1) (else invalid data): uniforms[cu_t[b]+i], i < gamma_b,
                                 test draft i; uniforms[cu_t[b]+gamma_b] is the one
                                 uniform of the final (residual or bonus) sample   */
  const float* temperatures;  /* [B] T_b; 0 = greedy                               */
} specverify_inputs;

/* Outputs of one run; device memory owned by the caller. */
typedef struct {
  int32_t* accepted_len;      /* [B] n_b in [0, gamma_b]; -1 invalid data; -2 wait expired */
  int32_t* out_tokens;        /* [R_t] at cu_t[b]+j: x_j for j < n_b, the sampled token at
                                 j = n_b, -1 for j > n_b (all -1 if n_b < 0)          */
  float* p_draft;             /* [R_d] p_i(x_i), or NULL                            */
  float* q_draft;             /* [R_d] q_i(x_i), or NULL                            */
  float* beta;                /* [R_d] sum_k min(p_i, q_i), or NULL                 */
  float* resid_mass;          /* [R_d] sum_k max(0, p_i - q_i), or NULL             */
} specverify_outputs;

/* Allocate a handle and its workspace on cfg->device.  On failure *out is
 * NULL.  Errors: INVALID_ARGUMENT (NULL or out-of-range config),
 * UNSUPPORTED (vocab too large; or a library build whose kernels would
 * spill registers to scratch memory, which is refused rather than run),
 * DEVICE (no such device / runtime error), OUT_OF_MEMORY. */
specverify_status specverify_create(const specverify_config* cfg, specverify_handle* out);

/* Verify one batch, asynchronously on hip_stream (a hipStream_t; NULL = the
 * default stream): one kernel launch (two for a ragged batch, whose layout
 * is checked first).  Writes accepted_len, out_tokens and the non-NULL
 * diagnostics; nothing else.  Errors (no launch happens): INVALID_ARGUMENT
 * for a NULL handle / inputs / outputs or required pointer, B > max_batch,
 * gamma outside [0, max_gamma], R_t > max_batch * (max_gamma + 1), a
 * stride < V; UNSUPPORTED for logits pointers not aligned to the element
 * size; DEVICE if the launch fails. */
specverify_status specverify_run(specverify_handle h, const specverify_inputs* in,
                                 const specverify_outputs* out, void* hip_stream);

/* Verification over a draft tree (Perplexity "Accelerating Sonar through
 * speculation", sections "추측적 디코딩", stage 2, and "EAGLE": the drafter
 * explores a tree and keeps its Top-K candidates at every node).  The pages
 * give no rule for several candidates of one node; this library reads each
 * candidate as a token-only draft (q = delta_c) and applies the chain's rule
 * per candidate: the children of the current node are tested in node order,
 * candidate c accepted when u_c < r(c), r the node's target distribution
 * with the candidates rejected so far removed and renormalised (velog
 * "6-1편. Speculative Decoding", section 2-1 with q = delta_c, and the
 * residual of section 2-2); an accepted candidate is emitted and the walk
 * continues at it; when every child is rejected, or at a leaf, the final
 * token is sampled from that residual (inverse CDF in token order).  T = 0:
 * the first child equal to its node's target argmax; else the argmax.
 *
 * Layout, per sequence b with N_b drafted nodes (numbered 1 .. N_b; node 0
 * is the root, the last committed token): nodes cu_nodes[b] ..
 * cu_nodes[b+1] - 1 of parents[] and tokens[]; parents[cu_nodes[b] + k - 1]
 * is node k's parent, in [0, k - 1]; target rows and uniforms at
 * cu_t[b] = cu_nodes[b] + b: row cu_t[b] + k is the target distribution
 * after node k (k = 0: after the root); uniforms[cu_t[b] + k - 1] tests
 * node k and uniforms[cu_t[b] + N_b] drives the final sample.  A chain
 * (node k's parent k - 1) is exactly specverify_run with token-only drafts.
 * Invalid data (the chain case's rules, a parent outside [0, k - 1]) gives
 * accepted_len -1 and -1 outputs.  Limits: N_b <= max_gamma, R_t = N + B <=
 * max_batch * (max_gamma + 1).  One kernel launch after the layout check. */
typedef struct {
  int32_t batch;              /* B >= 0                                            */
  const int32_t* cu_nodes;    /* [B+1] node offsets (device), cu_nodes[0] = 0      */
  int32_t num_nodes;          /* N = cu_nodes[B] (host copy)                       */
  const int32_t* parents;     /* [N] parent of each node, local index (device)     */
  const int32_t* tokens;      /* [N] each node's candidate token (device)          */
  const void* target_logits;  /* [R_t, target_stride] f32 or bf16, R_t = N + B     */
  int64_t target_stride;      /* elements between rows, >= V                       */
  const float* uniforms;      /* [R_t] u in [0, 1)                                 */
  const float* temperatures;  /* [B] T_b; 0 = greedy                               */
} specverify_tree_inputs;

typedef struct {
  int32_t* accepted_len;      /* [B] n_b, the accepted depth; -1 invalid; -2 wait expired */
  int32_t* out_tokens;        /* [R_t] at cu_t[b] + j: the j-th accepted node's token for
                                 j < n_b, the final token at j = n_b, -1 after            */
  int32_t* out_nodes;         /* [R_t] at cu_t[b] + j: the j-th accepted node (1-based) for
                                 j < n_b, -1 after; or NULL                               */
  float* p_cand;              /* [N] each candidate's p under its parent's target row (T = 0:
                                 1 if it is the argmax, else 0); NaN if invalid; or NULL */
} specverify_tree_outputs;

/* Errors as specverify_run (no launch happens): INVALID_ARGUMENT also for
 * NULL cu_nodes (B > 0) or NULL parents / tokens (N > 0). */
specverify_status specverify_run_tree(specverify_handle h, const specverify_tree_inputs* in,
                                      const specverify_tree_outputs* out, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * run as specverify_run, with the same kernels, results, arguments and
 * errors, but without a handle.  cfg is read as by specverify_create (its
 * limits bound this call's batch); the workspace is a 16 MiB array of the
 * library in device memory, one per device, that the device holds until the
 * process ends.  The call allocates nothing: the first call on a device
 * looks up that device's array (hipGetSymbolAddress) and clears it with a
 * kernel on hip_stream; later calls launch only the run.  A run needs
 * 48 * R_t * C bytes (C = ceil(V / 2048) for bf16, ceil(V / 1024) for f32)
 * plus 64 bytes per wave of its grid (at most the device's resident waves,
 * 0.5 MiB on an MI355X) and a few KB, each region rounded up to 256 bytes;
 * a run that needs more than 16 MiB returns TOO_LARGE before any launch
 * (B = 64, gamma = 4, V = 128256 bf16 needs 1.1 MiB; B = 512 with 2601
 * target rows at V = 152064, 9.1 MiB).  UNSUPPORTED also for a device
 * ordinal of 64 or more.
 * Every call on a device shares its array and leaves its contents there;
 * what a run reads from it carries the run's epoch, a per-device counter
 * kept on the host, so stale contents are never taken for new ones.  Calls
 * on one device must not overlap: put them on one stream or order them
 * (overlapping calls race on the array).  A captured graph keeps the epoch
 * it was captured with, so replaying it more than once is not supported.
 * Thread-safe on the host. */
specverify_status specverify_run_static(const specverify_config* cfg, const specverify_inputs* in,
                                        const specverify_outputs* out, void* hip_stream);

/* On-device commit of a verification step (Perplexity "Accelerating Sonar
 * through speculation", section "단일 토큰에 대한 MTP 스케줄링": after the drafts
 * are verified, a kernel places the next target token after the target's
 * shifted input tokens, so the accepted length never has to reach the host).
 * For every sequence b with 0 <= n_b = accepted_len[b] <= gamma_b, the
 * n_b + 1 emitted tokens out_tokens[cu_t[b] .. cu_t[b] + n_b] are appended to
 * row b of seq_tokens at seq_lens[b]; seq_lens[b] grows by n_b + 1,
 * appended[b] = n_b + 1 and next_token[b] = out_tokens[cu_t[b] + n_b] (the
 * token that starts b's next step).  A sequence with n_b < 0 (invalid) or
 * n_b > gamma_b, or whose layout lies outside the R_d draft rows, is left
 * unchanged with appended[b] = 0; one whose tokens do not fit (seq_lens[b]
 * < 0 or seq_lens[b] + n_b + 1 > capacity) is left unchanged with
 * appended[b] = -1; both get next_token[b] = -1.  The layout is the run's:
 * cu_t[b] = cu_draft[b] + b, or b * (gamma + 1) when cu_draft is NULL.
 * Every pointer is device memory; the call is asynchronous on hip_stream and
 * must be ordered after the run whose outputs it reads. */
typedef struct {
  int32_t batch;                /* B <= max_batch (0 = nothing to do)                 */
  int32_t gamma;                /* uniform draft length, used iff cu_draft == NULL    */
  const int32_t* cu_draft;      /* [B+1] draft-row offsets of the run, or NULL        */
  int32_t num_draft_rows;       /* R_d = cu_draft[B] (host copy), used iff cu_draft   */
  const int32_t* accepted_len;  /* [B] from specverify_run                            */
  const int32_t* out_tokens;    /* [R_t] from specverify_run                          */
  int32_t* seq_tokens;          /* [B, seq_stride] committed tokens, in/out           */
  int64_t seq_stride;           /* elements between rows, >= capacity                 */
  int32_t capacity;             /* tokens a row may hold                              */
  int32_t* seq_lens;            /* [B] committed lengths, in/out                      */
  int32_t* appended;            /* [B] out: n_b + 1, 0 or -1 as above; or NULL        */
  int32_t* next_token;          /* [B] out, or NULL                                   */
} specverify_commit_args;

/* Errors (no launch happens): INVALID_ARGUMENT for a NULL handle, args or
 * required pointer, B > max_batch, gamma outside [0, max_gamma], R_t above
 * the handle's rows, capacity < 0 or seq_stride < capacity; DEVICE if the
 * launch fails. */
specverify_status specverify_commit(specverify_handle h, const specverify_commit_args* a,
                                    void* hip_stream);

/* Free the workspace and the handle (NULL is accepted). */
specverify_status specverify_destroy(specverify_handle h);

/* Timing of a run's kernels, measured with HIP events recorded on the run's
 * stream: stream_ms covers every launch of the run (the layout check of a
 * ragged batch, then the verification kernel, which streams the logits and
 * resolves the sequences); finish_ms is the time between the end of those
 * launches and the run's last event, about 0 (kept so that a caller can
 * time work placed there).  set_timing(h, 1) starts a new
 * measurement: the next SPECVERIFY_TIMING_RUNS runs record their events (later
 * runs record none); set_timing(h, 0) stops recording.  timing_totals waits
 * for the last recorded run and returns the number of recorded runs and the
 * summed durations of both kernels in milliseconds, then starts counting
 * afresh.  Errors: INVALID_ARGUMENT for a NULL pointer, DEVICE if an event
 * call fails (also from set_timing, which creates the events). */
#define SPECVERIFY_TIMING_RUNS 1024
specverify_status specverify_set_timing(specverify_handle h, int32_t enable);
specverify_status specverify_timing_totals(specverify_handle h, int32_t* runs, float* stream_ms,
                                           float* finish_ms);

/* Measurement probe (for benchmarks, not part of the method): one launch on
 * hip_stream that reads every byte of the ranges [a, a + a_bytes) and
 * [b, b + b_bytes) of device memory once, in 4 KB chunks with 16-byte
 * nontemporal loads spread over the whole device (the verification kernel's
 * access pattern), and does nothing else; it XOR-folds the words per wave
 * and writes a fold to *sink (one device uint32) only when it equals the
 * constant 0x9E3779B9, so *sink is normally left as it was; the condition
 * keeps every load.  Its bandwidth is the device's
 * practical streaming-read ceiling for the bytes a run reads (pass the
 * target and draft logits).  Pointers 16-byte aligned, sizes multiples of
 * 16, else INVALID_ARGUMENT; DEVICE if the launch fails.  Uses the current
 * HIP device. */
specverify_status specverify_probe_read(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                                        uint32_t* sink, void* hip_stream);

/* Number of V-chunks (4 KB of a row: 2048 bf16 or 1024 f32 logits) a row
 * is split into for this handle, and the workspace size in bytes; for tools
 * and tests. */
int32_t specverify_chunks_per_row(specverify_handle h);
int64_t specverify_workspace_bytes(specverify_handle h);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
