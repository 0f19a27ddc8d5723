/*
 * onela.h - C ABI of the OneLA large-beam Gated DeltaNet decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes (OneLA abstract, readsearch.ai page; OneLA review,
 * evolve.pub, "Summary", "Key claims", "Scope & Claims", paper Eq. 2-4):
 * every request holds ONE prompt-derived state S0 per head (d_v x d_k) that
 * all W beams share. At decode step t each beam b of a request, whose history
 * is the list of transition records (alpha_j, delta_j, k_j) of its ancestors,
 * advances the GDN recurrence
 *
 *     delta_t = beta_t * (v_t - alpha_t * S_{t-1} k_t)
 *     S_t     = alpha_t * S_{t-1} + delta_t k_t^T
 *     o_t     = S_t q_t
 *
 * without ever forming its own S: S_{t-1} x (x = k_t, q_t) is S0 x plus a
 * replay of the ancestral records, y <- alpha_j y + (k_j . x) delta_j. The step
 * then appends the record (alpha_t, delta_t, k_t) for the beam and returns o_t.
 * Records are append-only; an ancestry index (one per request, shared by all
 * heads) lists the record ids of each beam's history. When beams fork only
 * record ids are copied, never records.
 *
 * Conventions used by this library (the pages do not fix them):
 *   - steps are t = 1..max_steps per episode; at t = 1 all beams start from
 *     S0 and parent_idx is ignored;
 *   - the record of beam b written at step t has id rid = (t-1)*W + b (the
 *     ids the inspection calls report; internally records are stored in the
 *     order the kernels process the beams, and the index holds those ids);
 *   - ancestry row of beam b at step t = record ids of its t-1 ancestors,
 *     oldest first;
 *   - no query scaling and no normalisation inside: the caller folds those
 *     into q and k;
 *   - alpha, beta are one float per (beam, head); S0, delta, o are float32;
 *     q, k, v are bf16 (passed as uint16_t bit patterns).
 *
 * Memory and execution:
 *   - every pointer marked "device" is HIP device memory owned by the caller,
 *     which must keep it alive until the work enqueued on the context's
 *     stream has finished;
 *   - the library owns its state (S0 planes, record store, ancestry index,
 *     error words) and allocates all of it in onela_create; onela_step
 *     allocates nothing;
 *   - every call that launches work is asynchronous on the stream given to
 *     onela_create; getters synchronise that stream;
 *   - one host thread at a time per context.
 *
 * Errors: every function returns ONELA_OK (0) or a negative status. Misuse
 * that the host can see (NULL pointers, bad ids, wrong state, capacity) is
 * rejected before anything is enqueued and leaves the context unchanged. A
 * parent index outside [0, W) is found on the device: the affected request's
 * outputs for that step are undefined, the request is poisoned, and the next
 * onela_sync or getter for it returns ONELA_E_PARENT_RANGE; onela_reset or
 * onela_init_request clears the poison.
 */
#ifndef ONELA_H
#define ONELA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t onela_status;

#define ONELA_OK               0
#define ONELA_E_INVALID_ARG   (-1)  /* NULL pointer, id out of range, duplicate id */
#define ONELA_E_BAD_STATE     (-2)  /* request not initialised, or poisoned */
#define ONELA_E_CAPACITY      (-3)  /* request already did max_steps steps */
#define ONELA_E_PARENT_RANGE  (-4)  /* a parent index was outside [0, W) */
#define ONELA_E_HIP           (-5)  /* a HIP call failed; see onela_last_error */
#define ONELA_E_OOM           (-6)  /* device allocation failed in onela_create */
#define ONELA_E_UNSUPPORTED   (-7)  /* head dims or step count the library has no kernel for */

/* Fixed shape of one context (one GDN layer). Supported: d_k == d_v in
 * {32, 64, 128}; 1 <= beam_width; 1 <= max_steps <= ONELA_MAX_STEPS;
 * beam_width * num_heads * d and max_steps * beam_width * d below 2^31
 * (otherwise ONELA_E_UNSUPPORTED). */
#define ONELA_MAX_STEPS 64

typedef struct onela_config {
    int32_t max_requests;  /* request slots, ids 0..max_requests-1 */
    int32_t num_heads;     /* H; heads are independent (equal q/k/v head counts) */
    int32_t d_k;
    int32_t d_v;
    int32_t beam_width;    /* W */
    int32_t max_steps;     /* decode steps per episode (record store depth) */
} onela_config;

typedef struct onela_ctx onela_ctx;

/* Create a context (one GDN layer) on the current HIP device. It holds what
 * the method keeps per request (OneLA abstract, readsearch.ai page: one
 * shared prompt-derived state per request, append-only transition records,
 * a lightweight ancestry index; OneLA review, evolve.pub, "Summary": the
 * persistent state is the shared state plus the records), allocated here
 * once for the largest episode. hip_stream is a hipStream_t
 * (NULL = the null stream). Allocates S0 planes (4*H*d_v*d_k bytes per
 * request), the record store ((4 + 4*d_v + 2*d_k) bytes per record,
 * max_requests*H*max_steps*W records), the ancestry index
 * (2*max_requests*W*max_steps int32), the per-request beam processing
 * order (2*max_requests*W int32) and, for W <= 1024, the processing order of
 * every step (max_requests*max_steps*W int32). On failure *out is NULL. */
onela_status onela_create(const onela_config* cfg, void* hip_stream, onela_ctx** out);

/* A context for another GDN layer of the same requests that reads the
 * ancestry index of `index_owner` instead of keeping its own: the beam tree
 * is one per request, whatever the number of layers (OneLA abstract: a
 * lightweight ancestry index tracks each beam's records), so one index
 * update per decode step serves every layer. cfg may differ from the owner's
 * in num_heads, d_k, d_v; max_requests, beam_width and max_steps must match
 * (else ONELA_E_INVALID_ARG; an owner cannot itself share another's index).
 * The owner's onela_step writes the index and the order in which step t
 * processes the beams (records are stored in that order, the same in every
 * layer); a sharing context's step t of a request reads the rows the owner's
 * step t-1 wrote and the order of the owner's step t, so for every request:
 *   - the sharing context's step t (t >= 2) runs after the owner's step t
 *     and before the owner's step t+1 (else ONELA_E_BAD_STATE, nothing
 *     enqueued); when they use different streams the caller orders them;
 *   - after onela_init_request / onela_reset of a request on the owner, every
 *     sharing context that had stepped it must restart it too before its next
 *     step there (else ONELA_E_BAD_STATE).
 * Allocates what onela_create does minus the ancestry index and orders.
 * Destroy sharing contexts before their owner (onela_destroy of an owner that
 * still has sharers returns ONELA_E_BAD_STATE and frees nothing). */
onela_status onela_create_sharing_index(const onela_config* cfg, void* hip_stream, onela_ctx* index_owner,
                                        onela_ctx** out);

/* Synchronise the stream and free everything the context owns (the shared
 * states, record store and ancestry index of its requests; OneLA abstract:
 * the state the method keeps per request). NULL is OK. An index owner with
 * live sharing contexts: ONELA_E_BAD_STATE. */
onela_status onela_destroy(onela_ctx* ctx);

/* Load the shared prompt-derived state of request `req` and rewind it to
 * step 0 (OneLA abstract: one shared prompt-derived state per request).
 * S0: device float32 [H][d_v][d_k], row-major (rows index d_v). The library
 * keeps its own copy (split into two bf16 planes whose sum carries S0 to
 * about 2^-17 relative), so S0 may be freed once the stream has passed this
 * call. */
onela_status onela_init_request(onela_ctx* ctx, int32_t req, const float* S0);

/* Like onela_init_request for n_req requests at once, with each S0 computed
 * on the GPU from the request's prompt: the GDN recurrence (OneLA review,
 * evolve.pub, paper Eq. 2) run over seq_len tokens from a zero state and
 * written straight into the library's two bf16 planes (OneLA abstract: the
 * shared state is prompt-derived). reqs: host [n_req], distinct ids.
 * k: device bf16 [n_req][seq_len][H][d_k]; v: device bf16
 * [n_req][seq_len][H][d_v]; alpha, beta: device float32 [n_req][seq_len][H];
 * k and v 16-byte aligned. seq_len = 0 gives the zero state. Same state
 * change as onela_init_request for every listed request (step 0, poison
 * cleared); one workgroup per (request, head). */
onela_status onela_init_requests_from_prompts(onela_ctx* ctx, int32_t n_req, const int32_t* reqs,
                                              int32_t seq_len, const uint16_t* k, const uint16_t* v,
                                              const float* alpha, const float* beta);

/* Prefill without a context: fold n_seq prompts of seq_len tokens each into
 * float32 states with the GDN recurrence (OneLA review, evolve.pub, paper
 * Eq. 2), per sequence and head, starting from S_init (device float32
 * [n_seq][H][d_v][d_k], or NULL for the zero state). Layouts: k device bf16
 * [n_seq][seq_len][H][d_k]; v [n_seq][seq_len][H][d_v]; alpha, beta float32
 * [n_seq][seq_len][H]; S_out device float32 [n_seq][H][d_v][d_k]. S_out may
 * equal S_init (in place). Folding a prompt in two calls (the second starting
 * from the first's S_out) gives bit-identical states to one call when the
 * first call's length is a multiple of 32 tokens (else agreeing to about
 * 1e-5: the prompt is folded in pairs of 16-token chunks). Pointers of
 * k, v, S_init, S_out are 16-byte aligned; d_k = d_v in {32, 64, 128}
 * (else ONELA_E_UNSUPPORTED). Asynchronous on hip_stream (NULL = the null
 * stream); errors of the launch itself return ONELA_E_HIP. Allocates nothing. */
onela_status onela_prefill(int32_t n_seq, int32_t num_heads, int32_t d_k, int32_t d_v, int32_t seq_len,
                           const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                           const float* S_init, float* S_out, void* hip_stream);

/* One decode step of one GDN layer for n_req requests (OneLA review,
 * "Key claims" and "Scope & Claims", paper Eq. 2-4: records (alpha, delta, k)
 * appended per step, projection replay over the ancestry).
 *   n_req      1 <= n_req <= max_requests (else ONELA_E_INVALID_ARG).
 *   reqs       host int32 [n_req], distinct initialised request ids; each
 *              request advances its own step counter t (requests may be at
 *              different depths).
 *   q, k       device bf16 [n_req*W][H][d_k]   (request i owns rows i*W..)
 *   v          device bf16 [n_req*W][H][d_v]
 *   alpha,beta device float32 [n_req*W][H]
 *   parent_idx device int32 [n_req][W]: beam b of request i continues beam
 *              parent_idx[i][b] of the previous step. Read only for requests
 *              at t >= 2; may be NULL if every request is at t == 1.
 *   o          device float32 [n_req*W][H][d_v], written (o_t = S_t q_t)
 *   delta_out  optional device float32 [n_req*W][H][d_v]; receives delta_t
 *              (the same values appended to the record store), or NULL.
 * Nothing is allocated. Returns after enqueueing. */
onela_status onela_step(onela_ctx* ctx, int32_t n_req, const int32_t* reqs,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* alpha, const float* beta,
                        const int32_t* parent_idx, float* o, float* delta_out);

/* Rewind request `req` to step 0, keeping its S0 (OneLA abstract: the
 * shared state is fixed by the prompt, and records are only ever appended, so
 * a new episode needs no copy of anything: the records of the old episode
 * become dead and are overwritten by the next one). Host-only and
 * O(1): nothing is enqueued; a device error left by the old episode no
 * longer counts. */
onela_status onela_reset(onela_ctx* ctx, int32_t req);

/* Wait for the stream. Returns ONELA_E_PARENT_RANGE if any request is
 * poisoned by a bad parent index (each beam continues a beam of the previous
 * step; OneLA abstract: the ancestry index follows the beam tree), ONELA_E_HIP
 * on a HIP failure. */
onela_status onela_sync(onela_ctx* ctx);

/* ---- input-side fusion ----------------------------------------------------
 * A GDN layer forms q, k, alpha and beta from its projections before the
 * step. The pages do not describe that part; this entry point takes the usual
 * gated DeltaNet parametrisation and fuses it into the step launch:
 *   q = q_raw / sqrt(|q_raw|^2 + norm_eps), k likewise (per head, float32,
 *     rounded to bf16 before use; the records hold these keys),
 *   alpha = exp(-exp(A_log[h]) * softplus(a_raw + dt_bias[h])),
 *   beta  = sigmoid(b_raw),
 * and writes o as bf16 (nearest, ties to even) for the layer's next matmul.
 * The records' alpha are the computed alpha. */
typedef struct {
    const float* A_log;     /* device float32 [H] */
    const float* dt_bias;   /* device float32 [H] */
    float norm_eps;         /* >= 0, added to the sum of squares (e.g. 1e-6) */
} onela_gate_params;

/* onela_step (the step of OneLA review, evolve.pub, "Summary", paper Eq. 2-4)
 * with raw inputs, the fused input side above not being on the pages:
 * q_raw, k_raw device bf16 [n_req*W][H][d_k]
 * (16-byte aligned), v as in onela_step, a_raw, b_raw device float32
 * [n_req*W][H], gates (host struct, device arrays), o_bf16 device bf16
 * [n_req*W][H][d_v] (8-byte aligned). delta_out (float32), parents, request
 * list, errors and state changes as in onela_step; graph mode applies. */
onela_status onela_step_raw(onela_ctx* ctx, int32_t n_req, const int32_t* reqs,
                            const uint16_t* q_raw, const uint16_t* k_raw, const uint16_t* v,
                            const float* a_raw, const float* b_raw, const onela_gate_params* gates,
                            const int32_t* parent_idx, uint16_t* o_bf16, float* delta_out);

/* Graph mode on (1) or off (0). In graph mode each request's step index and
 * episode number live in device memory and each step launch advances them
 * itself (the last workgroup of a request to finish), so the launches of a
 * decode step (of every layer) can be captured once in
 * a HIP graph and replayed for the following decode steps, the caller
 * refilling the same input buffers before each replay (the pages' serving
 * loop is decode-forward, OneLA review, evolve.pub, "Summary"). In this mode:
 *   - onela_step requires parent_idx (ignored for requests at t = 1) and
 *     does no step-count checks on the host; a step past max_steps is found
 *     on the device, writes nothing, and makes the next onela_sync return
 *     ONELA_E_CAPACITY (cleared by onela_reset / onela_init_request);
 *   - the host ordering checks of a shared index are off: step every layer
 *     of a decode step, owner first, as the eager calls would;
 *   - onela_reset and onela_init_request enqueue a small counter write, so
 *     they belong outside captured graphs;
 *   - getters and onela_sync refresh the host's step counters from the
 *     device.
 * Switching synchronises the stream. Default: off (step counters on the
 * host, onela_reset enqueues nothing). */
onela_status onela_set_graph_mode(onela_ctx* ctx, int32_t on);

/* Beams handled by one workgroup (0 = automatic). Must be 0 or a multiple of
 * 64, else ONELA_E_INVALID_ARG. Results do not depend on it; only the launch
 * shape does: one workgroup projects the shared state once for all the beams
 * it holds (OneLA abstract: the fused kernel reuses the shared state across
 * beams), so fewer splits mean fewer reads of it. */
onela_status onela_set_beams_per_block(onela_ctx* ctx, int32_t beams);

/* Beam processing order of the step kernel: -1 = automatic (default), 0 =
 * beam-index order, 1 = ancestry order (siblings adjacent, so that one chunk
 * of beams gathers mostly the same ancestral records; beam widths up to 1024).
 * Beams that share history share records (OneLA abstract: the ancestry index
 * lists the transition records that make up each beam's history).
 * Automatic orders a launch when its (request, head) pairs hold at least 32768
 * beams in all (below that a launch is bound by each workgroup's dependent
 * loads, which the ordering lengthens) and each beam set is split over at most
 * two workgroups (each workgroup orders the whole set to process its share).
 * Results do not depend on it (every beam's arithmetic is its own); only the
 * records each chunk shares do. Returns ONELA_E_INVALID_ARG for any other
 * value. */
onela_status onela_set_beam_order(onela_ctx* ctx, int32_t mode);

/* ---- inspection (synchronous; for tests and accounting) ---------------- */

/* Steps done by `req` in the current episode (0 after init or reset): the
 * number of records each of its beams has appended (OneLA abstract:
 * append-only transition records). */
onela_status onela_get_step(onela_ctx* ctx, int32_t req, int32_t* t_done);

/* Ancestry rows the last step of `req` used (OneLA abstract: the ancestry
 * index lists the records that make up each beam's history): host int32
 * [W][max_steps]; row b holds t_done-1 record ids (oldest first) and -1
 * after them. Record id (j-1)*W + c names the record beam c appended at step
 * j, whatever order the kernels stored the records in. */
onela_status onela_get_ancestry(onela_ctx* ctx, int32_t req, int32_t* host_out);

/* Records 0..n_rec-1 of (req, head), n_rec <= t_done*W (OneLA review,
 * evolve.pub, "Summary": a record holds (alpha_t, delta_t, k_t)), record
 * (j-1)*W + c being the one beam c appended at step j. Host outputs, each may
 * be NULL: alpha float32 [n_rec], delta float32 [n_rec][d_v], key bf16 bits
 * [n_rec][d_k]. */
onela_status onela_get_records(onela_ctx* ctx, int32_t req, int32_t head, int32_t n_rec,
                               float* alpha, float* delta, uint16_t* key);

/* Device bytes the context owns, the state whose size the method reduces
 * (OneLA review, evolve.pub, "Summary"): S0 planes, record store, and in index_bytes
 * the ancestry index and beam order (none on a context sharing another's
 * index) plus five int32 words per request (error words, graph-mode
 * counters). */
onela_status onela_get_memory(const onela_ctx* ctx, uint64_t* s0_bytes,
                              uint64_t* record_bytes, uint64_t* index_bytes);

/* ---- comparator: a full state per beam ---------------------------------
 * The decode step OneLA replaces (OneLA review, evolve.pub, "Summary" and
 * "Scope & Claims": the FullState serving path keeps a full d_v x d_k state
 * for every beam, Theta(W d_v d_k) memory and traffic per step). Same
 * recurrence, conventions, argument layouts and error behaviour as the
 * onela_* calls above; the library owns S0 copies and two float32 states per
 * (request, head, beam) (the parents' and the new ones), allocated in
 * onela_fs_create. Used to measure what the shared-state representation saves.
 */
typedef struct onela_fs_ctx onela_fs_ctx;

/* Allocates 4*d_v*d_k*max_requests*num_heads*(2*beam_width + 1) bytes. */
onela_status onela_fs_create(const onela_config* cfg, void* hip_stream, onela_fs_ctx** out);
onela_status onela_fs_destroy(onela_fs_ctx* ctx);
/* Copies S0 (device float32 [H][d_v][d_k]) and rewinds the request to step 0. */
onela_status onela_fs_init_request(onela_fs_ctx* ctx, int32_t req, const float* S0);
/* One decode step; arguments as for onela_step. Reads each beam's parent
 * state, writes the beam's new state, o and optionally delta. */
onela_status onela_fs_step(onela_fs_ctx* ctx, int32_t n_req, const int32_t* reqs,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* alpha, const float* beta,
                           const int32_t* parent_idx, float* o, float* delta_out);
onela_status onela_fs_reset(onela_fs_ctx* ctx, int32_t req);
onela_status onela_fs_sync(onela_fs_ctx* ctx);
/* Device bytes of persistent state the comparator owns. */
onela_status onela_fs_get_memory(const onela_fs_ctx* ctx, uint64_t* state_bytes);

/* ---- comparator: every beam replays its own history ---------------------
 * The replay-based serving path (OneLA review, evolve.pub, "Summary" and
 * "Scope & Claims": the ReplaySSM baseline checkpoints the state only at the
 * prompt boundary and treats every beam as an independent request that
 * replays its shared history). At every step each beam starts from S0,
 * applies its ancestral records (alpha_j, delta_j, k_j) oldest first as full
 * rank-one updates S <- alpha_j S + delta_j k_j^T, takes the GDN step on the
 * rebuilt d_v x d_k state and appends its record; nothing is shared between
 * beams (not even S0 k) and no per-beam state persists: Theta(W t d_v d_k)
 * work per step at depth t. Same recurrence, conventions, argument layouts
 * and error behaviour as the onela_* calls above; the library owns S0 copies
 * (float32), the record store (the same records onela_step appends) and the
 * parents given at every step, allocated in onela_rs_create. Used to measure
 * what sharing the projection saves.
 */
typedef struct onela_rs_ctx onela_rs_ctx;

/* Allocates max_requests * (num_heads * (4 d_v d_k + max_steps * beam_width *
 * (4 + 4 d_v + 2 d_k)) + 4 max_steps * beam_width) + 4 max_requests bytes. */
onela_status onela_rs_create(const onela_config* cfg, void* hip_stream, onela_rs_ctx** out);
onela_status onela_rs_destroy(onela_rs_ctx* ctx);
/* Copies S0 (device float32 [H][d_v][d_k]) and rewinds the request to step 0. */
onela_status onela_rs_init_request(onela_rs_ctx* ctx, int32_t req, const float* S0);
/* One decode step; arguments as for onela_step. A parent index outside
 * [0, W) poisons the request (reported by onela_rs_sync as
 * ONELA_E_PARENT_RANGE), as in onela_step. */
onela_status onela_rs_step(onela_rs_ctx* ctx, int32_t n_req, const int32_t* reqs,
                           const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* alpha, const float* beta,
                           const int32_t* parent_idx, float* o, float* delta_out);
onela_status onela_rs_reset(onela_rs_ctx* ctx, int32_t req);
onela_status onela_rs_sync(onela_rs_ctx* ctx);
/* Device bytes of persistent state the comparator owns (S0, records, parents). */
onela_status onela_rs_get_memory(const onela_rs_ctx* ctx, uint64_t* state_bytes);

/* Static text for a status code (a library utility: no passage defines it). */
const char* onela_status_string(onela_status s);

/* Text of the last HIP error seen by this context ("" if none; a library
 * utility: no passage defines it). */
const char* onela_last_error(const onela_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* ONELA_H */
