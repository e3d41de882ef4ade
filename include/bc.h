/*
 * bc.h -- C ABI of the block-causal masked-diffusion denoising step for
 * AMD Instinct MI355X (gfx950).
 *
 * One denoising step of a block-diffusion decoder (the mechanism shared by
 * Fast-dDrive, WAM-Diff2 and Fast-dVLA) is:
 *
 *   bc_attn_step      block-causal GQA attention of the active block(s) over
 *                     the committed KV prefix plus the blocks' own K/V
 *   (model layers and LM head: outside this library)
 *   bc_unmask_select  per-row max / argmax / softmax confidence over the
 *                     vocabulary, then threshold + ceil(remaining / n) reveal
 *   bc_kv_commit      append a completed block's K/V to the cache
 *   bc_spec_verify    scaffold speculative verification (accept length and
 *                     bonus token) for the AR verify pass
 *
 * Conventions common to every entry point
 *   - Every tensor argument is a caller-owned DEVICE pointer unless the
 *     comment says HOST.  All device tensors are dense, row-major (C order)
 *     with the layout given in brackets, and at least 16-byte aligned.
 *   - The library allocates no memory and keeps no state between calls.
 *     Scratch space is a caller-provided workspace whose minimum size is
 *     returned by the matching *_workspace_bytes query.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is only enqueued; results are valid once the stream has been
 *     synchronised.  HOST arrays are read before the call returns and are
 *     not retained.
 *   - Arguments are validated on the host first.  On any failure a negative
 *     bc_status is returned and nothing has been enqueued; BC_ERR_HIP means a
 *     kernel launch was rejected by the runtime.
 *   - Floating-point inputs must be finite.
 *   - Calls on one stream that share a workspace run in stream order and may
 *     reuse it; concurrent calls on different streams need their own.
 */
#ifndef BC_H
#define BC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BC_MAX_SEQ 64      /* sequences (or rollouts) per bc_attn_step call */
#define BC_MAX_BLOCKS 64   /* active blocks per call */
#define BC_MAX_BLOCK_ROWS 1024 /* rows of one block in bc_unmask_select */
#define BC_MAX_SCAN_ROWS 4096  /* logit rows per bc_unmask_select / bc_spec_verify call */

typedef enum {
  BC_OK = 0,
  BC_ERR_ARG = -1,          /* malformed argument (null pointer, bad shape, ...) */
  BC_ERR_UNSUPPORTED = -2,  /* well-formed but outside what the kernels handle */
  BC_ERR_CAPACITY = -3,     /* a commit would grow a sequence past its capacity */
  BC_ERR_ORDER = -4,        /* a commit that does not start at the current length */
  BC_ERR_WORKSPACE = -5,    /* workspace missing or smaller than the query says */
  BC_ERR_HIP = -6,          /* the HIP runtime rejected a launch */
  BC_ERR_SCRATCH = -7,      /* the call needs more than the static scratch holds */
  BC_ERR_CALLBACK = -8      /* a caller callback returned nonzero */
} bc_status;

typedef enum { BC_F32 = 0, BC_BF16 = 1 } bc_dtype;

/* Visibility among the active rows.  Across blocks both modes are causal
 * (a block sees earlier blocks and never later ones); inside a block BIDIR is
 * bidirectional (the MDM draft / denoise pass) and CAUSAL is causal (the AR
 * verify pass).  Every committed (prefix / private) key is visible to every
 * active row of its sequence. */
typedef enum { BC_MASK_BLOCK_BIDIR = 0, BC_MASK_BLOCK_CAUSAL = 1 } bc_mask;

/* Reveal rule of one block (Fast-dVLA notes, key design 4, pipelined
 * parallel decoding): SEMI reveals only rows whose confidence exceeds the
 * threshold; FULL also reveals at least ceil(|masked| / n) rows. */
typedef enum { BC_UNMASK_SEMI = 0, BC_UNMASK_FULL = 1 } bc_unmask_mode;

/* A KV cache: k and v are each [n_seq][n_kv_heads][capacity][head_dim] of
 * `dtype`.  The number of valid rows per sequence is kept by the caller (a
 * HOST int32 array) and advanced only by bc_kv_commit. */
typedef struct {
  void *k, *v;
  int32_t dtype;        /* bc_dtype */
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t head_dim;     /* 64 or 128 */
  int32_t capacity;     /* rows allocated per (sequence, kv head) */
} bc_kv_cache;

/* The active rows of one step: every sequence has the same n_rows rows cut
 * into the same n_blk blocks.
 *   q    [n_seq][n_rows][n_q_heads][head_dim]
 *   k, v [n_seq][n_kv_heads][n_rows][head_dim]  (recomputed every step)
 *   blk_off  HOST [n_blk + 1], blk_off[0] = 0 < blk_off[1] < ... <
 *            blk_off[n_blk] = n_rows; row j is in block b when
 *            blk_off[b] <= j < blk_off[b + 1].
 * q, k and v have the dtype of the cache they are attended with. */
typedef struct {
  const void *q, *k, *v;
  const int32_t *blk_off;
  int32_t n_blk;
  int32_t n_seq;
  int32_t n_rows;
  int32_t n_q_heads;    /* a multiple of the caches' n_kv_heads */
} bc_active;

/* ------------------------------------------------------------------------ */
/* KV commit.
 * Fast-dVLA notes, key design 1, and Fast-dDrive method summary sec. 3.1:
 * a completed block's K/V never change again and are cached; only a prefix
 * whose predecessors are all complete may be cached, so commits are
 * append-only and in order.
 *
 * Copies blk_k / blk_v [n_kv_heads][n_rows][head_dim] (device, cache dtype)
 * into rows [start, start + n_rows) of sequence `seq` and sets
 * len[seq] = start + n_rows.  `len` is HOST [cache->n_seq], in/out.
 * With seq == BC_ALL_SEQ every sequence commits a block of n_rows at once
 * (one launch): blk_k / blk_v are [n_seq][n_kv_heads][n_rows][head_dim] and
 * every len[s] must equal start.
 * Errors: BC_ERR_ORDER if start != len[seq] (any len[s] with BC_ALL_SEQ);
 * BC_ERR_CAPACITY if start + n_rows > capacity; BC_ERR_ARG for a bad seq,
 * n_rows < 1 or null pointers.  The copy is bit-exact. */
#define BC_ALL_SEQ (-1)
int bc_kv_commit(const bc_kv_cache *cache, int32_t *len, int32_t seq, int32_t start,
                 int32_t n_rows, const void *blk_k, const void *blk_v, void *stream);

/* ------------------------------------------------------------------------ */
/* Block-causal GQA attention of the active rows.
 * WAM-Diff2 article sec. 2.1 and Fast-dVLA notes, key design 1: blocks are
 * bidirectional inside and causal across, so a block sees the prefix,
 * earlier blocks and itself; Fast-dDrive method summary sec. 3.2 step 3: the
 * AR verify pass is causal over the block; sec. 3.3 and the Fast-dDrive
 * abstract: N rollouts fork from one shared prefix KV cache.
 *
 * For query head h of row i (kv head h / (n_q_heads / n_kv_heads)):
 *   out[s][i][h] = sum_j softmax_j(scale * q.k_j) v_j
 * over the visible keys j of sequence s: every prefix row < prefix_len,
 * every private row < priv_len[s] (fork), and active rows by `mask`.
 *
 *   prefix      committed cache.  Without a fork, prefix->n_seq == a->n_seq.
 *               With a fork (priv != NULL), prefix->n_seq == 1 and all
 *               a->n_seq rollouts read it.
 *   prefix_len  HOST [prefix->n_seq], 0 <= len <= capacity.
 *   priv        NULL, or each rollout's private cache (n_seq == a->n_seq).
 *   priv_len    HOST [a->n_seq] when priv != NULL.
 *   mask        bc_mask.
 *   scale       softmax scale (finite, > 0), normally 1 / sqrt(head_dim).
 *   n_prefix_splits  0 = automatic (a cost model over the shapes and the
 *               prefix lengths, limited to what `ws` holds); otherwise the
 *               number of key chunks the prefix is cut into (1 .. 256), for
 *               tuning and tests.
 *   out         [n_seq][n_rows][n_q_heads][head_dim] in the q dtype.
 *   ws          workspace of at least bc_attn_workspace_bytes(...) bytes
 *               for the same shapes, capacities and n_prefix_splits.  With
 *               automatic splits a smaller workspace is accepted as long as
 *               it holds one split; fewer splits are then used.
 * Errors: BC_ERR_ARG (shapes / pointers / blk_off / lengths);
 * BC_ERR_UNSUPPORTED (head_dim not 64 or 128, n_seq > BC_MAX_SEQ,
 * n_blk > BC_MAX_BLOCKS, mixed dtypes); BC_ERR_WORKSPACE (ws NULL, or too
 * small for the explicit split count, or for one split). */
size_t bc_attn_workspace_bytes(const bc_kv_cache *prefix, const bc_kv_cache *priv,
                               const bc_active *a, int32_t n_prefix_splits);
int bc_attn_step(const bc_kv_cache *prefix, const int32_t *prefix_len,
                 const bc_kv_cache *priv, const int32_t *priv_len,
                 const bc_active *a, int32_t mask, float scale, int32_t n_prefix_splits,
                 void *out, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Confidence unmask.
 * Fast-dVLA notes, key design 4: a semi-active block reveals only positions
 * whose prediction confidence exceeds the threshold; a fully-active block
 * also ranks the remaining positions by confidence and reveals at least a
 * 1/n fraction of them.  Revealed tokens never change (key design 2).
 *
 * For every row r with masked[r] != 0:
 *   conf_r = 1 / sum_v exp(l_rv - max_v l_rv)   (max softmax probability)
 *   tok_r  = argmax_v l_rv (lowest index on ties)
 * Then per block b with masked set E and A = {r in E : conf_r > threshold}:
 *   k = |A|                                     (mode[b] == SEMI)
 *   k = min(|E|, max(|A|, ceil(|E| / n_div[b]))) (mode[b] == FULL)
 * and the first k rows of E in (conf descending, row ascending) order get
 * tokens[r] = tok_r, masked[r] = 0.  n_commit[b] = k.
 * Decisions are exact with respect to float64 confidences: rows whose float32
 * confidence lies too close to the threshold or to the ranking cut for the
 * float32 error bound are recomputed in float64 before deciding.
 *
 *   logits  [n_rows][vocab] float32
 *   blk_off HOST [n_blk + 1] as in bc_active; each block <= BC_MAX_BLOCK_ROWS
 *   mode    HOST [n_blk] bc_unmask_mode;  n_div HOST [n_blk], >= 1
 *   masked  [n_rows] uint8, in/out (1 = still masked)
 *   tokens  [n_rows] int32, in/out (rows revealed now are written)
 *   conf    [n_rows] float32 or NULL: confidence of every row masked on
 *           entry (other rows are left untouched)
 *   n_commit [n_blk] int32
 *   ws      at least bc_unmask_workspace_bytes(n_rows, vocab) bytes (any
 *           contents; it holds the per-chunk scan results between the two
 *           kernels of the call)
 * Errors: BC_ERR_ARG; BC_ERR_UNSUPPORTED (a block over BC_MAX_BLOCK_ROWS rows,
 * n_rows over BC_MAX_SCAN_ROWS); BC_ERR_WORKSPACE. */
size_t bc_unmask_workspace_bytes(int32_t n_rows, int32_t vocab);
int bc_unmask_select(const float *logits, int32_t n_rows, int32_t vocab,
                     const int32_t *blk_off, int32_t n_blk,
                     const int32_t *mode, const int32_t *n_div, float threshold,
                     uint8_t *masked, int32_t *tokens, float *conf, int32_t *n_commit,
                     void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Scaffold speculative verify.
 * Fast-dDrive method summary sec. 3.2, Scaffold Speculative decoding:
 * scaffold positions are accepted without a check; the AR pass gives
 * p_AR(. | x_<i) for every position; walking left to right a draft equal to
 * the AR argmax is accepted, and at the first mismatch the AR prediction is
 * taken as a bonus token and later drafts are dropped.
 *
 * Per sequence s, with t_i = argmax logits[s][i] (lowest index on ties):
 *   k = the first i in [first[s], m) with fixed[s][i] == 0 and
 *       t_i != draft[s][i], or m if there is none;
 *   accept_len[s] = k - first[s];  bonus[s] = t_k if k < n_lrows else -1.
 *
 *   logits   [n_seq][n_lrows][vocab] float32, row i already aligned with
 *            draft position i (row i = p_AR(. | x_<i))
 *   draft    [n_seq][m] int32, 1 <= m <= n_lrows
 *   fixed    [n_seq][m] uint8 or NULL (scaffold rows, auto-accepted)
 *   first    [n_seq] int32 device, each in [0, m] (clamped to it)
 *   accept_len, bonus  [n_seq] int32
 *   ws       at least bc_verify_workspace_bytes(n_seq, n_lrows, vocab) bytes
 *            (any contents).
 * Errors: BC_ERR_ARG; BC_ERR_UNSUPPORTED (n_seq * n_lrows over
 * BC_MAX_SCAN_ROWS); BC_ERR_WORKSPACE. */
size_t bc_verify_workspace_bytes(int32_t n_seq, int32_t n_lrows, int32_t vocab);
int bc_spec_verify(const float *logits, int32_t n_seq, int32_t n_lrows, int32_t vocab,
                   const int32_t *draft, int32_t m, const uint8_t *fixed,
                   const int32_t *first, int32_t *accept_len, int32_t *bonus,
                   void *ws, size_t ws_bytes, void *stream);

/* Scaffold speculative verify with a sampled AR pass.
 * Fast-dDrive method summary sec. 3.3, design principle one (and the
 * Fast-dDrive paper's introduction): the trajectory section samples the AR
 * verifier instead of taking its argmax, to fork diverse rollouts.  The
 * sample is Gumbel-max over caller-supplied noise, so it is reproducible:
 *   t_i = argmax_v (logits[s][i][v] * inv_temperature + noise[s][i][v])
 * (lowest index on ties), one float32 multiply and one float32 add, each
 * rounded, no fused multiply-add; with noise drawn as -log(-log U), U
 * uniform in (0, 1), t_i is a draw from softmax(logits / temperature).
 * Everything else is bc_spec_verify.
 *
 *   noise            [n_seq][n_lrows][vocab] float32, finite
 *   inv_temperature  1 / temperature, finite and > 0
 * Errors: as bc_spec_verify; BC_ERR_ARG for a NULL noise or a bad
 * inv_temperature. */
int bc_spec_verify_sampled(const float *logits, const float *noise, float inv_temperature,
                           int32_t n_seq, int32_t n_lrows, int32_t vocab,
                           const int32_t *draft, int32_t m, const uint8_t *fixed,
                           const int32_t *first, int32_t *accept_len, int32_t *bonus,
                           void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Sub-steps, exported so that each kernel can be timed or scheduled on its
 * own.  They take exactly the arguments of the call they make up and must
 * run on the same stream and workspace, in this order.
 *
 * bc_attn_step(args) == bc_attn_partial(args); bc_attn_combine(args).
 *   The partial pass leaves, per key split, the running max, the softmax
 *   denominator and the unnormalised output of every row in the workspace
 *   (float32; for bf16 inputs with n_seq * n_rows * n_q_heads >= 1024, int16
 *   against a power of two per row and split, within 2^-14 of the row's
 *   largest element); the combine pass merges them with log-sum-exp weights
 *   into `out`.  Shared-prefix fork calls with a single key split in the
 *   row-tile form have no split partials: their partial pass writes `out`
 *   itself and their combine pass does nothing.  Those are the bf16,
 *   head_dim 128 fork calls with n_prefix_splits = 0,
 *   2 * n_seq * n_kv_heads >= 256 and 97 to 192 rows per rollout and KV
 *   head (n_rows * n_q_heads / n_kv_heads).
 *
 * bc_unmask_select(args) == bc_vocab_scan(logits, n_rows, vocab, masked, 1,
 *   ws, ws_bytes, stream); bc_unmask_decide(args).
 *   bc_vocab_scan leaves, for every row r with row_mask == NULL or
 *   row_mask[r] != 0, the max, the lowest argmax and (with_sum != 0) the sum
 *   of exp(l - max) of each 4096-logit chunk of the row in the workspace
 *   (sized by bc_unmask_workspace_bytes); bc_unmask_decide merges them and
 *   takes the decisions.  `masked` must not change between the two. */
int bc_attn_partial(const bc_kv_cache *prefix, const int32_t *prefix_len,
                    const bc_kv_cache *priv, const int32_t *priv_len,
                    const bc_active *a, int32_t mask, float scale, int32_t n_prefix_splits,
                    void *out, void *ws, size_t ws_bytes, void *stream);
int bc_attn_combine(const bc_kv_cache *prefix, const int32_t *prefix_len,
                    const bc_kv_cache *priv, const int32_t *priv_len,
                    const bc_active *a, int32_t mask, float scale, int32_t n_prefix_splits,
                    void *out, void *ws, size_t ws_bytes, void *stream);
int bc_vocab_scan(const float *logits, int32_t n_rows, int32_t vocab, const uint8_t *row_mask,
                  int32_t with_sum, void *ws, size_t ws_bytes, void *stream);
int bc_unmask_decide(const float *logits, int32_t n_rows, int32_t vocab,
                     const int32_t *blk_off, int32_t n_blk,
                     const int32_t *mode, const int32_t *n_div, float threshold,
                     uint8_t *masked, int32_t *tokens, float *conf, int32_t *n_commit,
                     void *ws, size_t ws_bytes, void *stream);

/* ---- Pipelined parallel decoding schedule (host only) --------------------
 * Fast-dVLA reading notes, key design 4 ("pipelined parallel decoding"):
 * several consecutive blocks of one sequence are denoised together; the
 * first uncommitted block is fully active (threshold, plus at least
 * ceil(remaining / n_div) per step), the block after an active one joins as
 * semi-active (threshold only) once its predecessor's completion ratio --
 * revealed rows / block size in double precision -- exceeds `add` (strictly,
 * like the confidence threshold) and fewer than `window` blocks are active,
 * and turns fully active once that ratio exceeds `act`.  With add = act = 1
 * no block starts before its predecessor is committed.  Blocks are committed strictly in order,
 * right after the step that reveals their last row.
 *
 * This is the schedule's state machine only; it runs on the host and touches
 * no GPU.  Per step the caller asks for the plan (bc_pipeline_next), runs the
 * step -- bc_attn_step over the active blocks' rows (BC_MASK_BLOCK_BIDIR,
 * blk_off as planned), the model, bc_unmask_select with the planned modes
 * and n_div over the same rows -- and reports the step's n_commit
 * (bc_pipeline_report), which returns the blocks to bc_kv_commit, in order.
 *
 * bc_pipeline_create: block_sizes[n_blocks] (each >= 1, n_blocks <= 4096),
 *   1 <= window <= BC_MAX_BLOCKS, n_div >= 1, add and act finite.  The
 *   library allocates the state (host memory) and owns it until
 *   bc_pipeline_destroy.  Errors: BC_ERR_ARG.
 * bc_pipeline_next: writes, for the n active blocks (n <= window, returned;
 *   0 once every block is committed), their ids (consecutive, oldest first),
 *   local_step (how many steps each has been active before this one),
 *   mode (BC_UNMASK_FULL / BC_UNMASK_SEMI), n_div (n_div for FULL, 1 for
 *   SEMI) and blk_off[n + 1] (row offsets inside the step; rows are the
 *   blocks' rows concatenated), and *row0, the first output row of the
 *   first active block (output rows = all blocks' rows concatenated).
 *   Calling it twice without a report returns the same plan.  Arrays hold
 *   at least `window` (+1 for blk_off) entries.  Errors: BC_ERR_ARG.
 * bc_pipeline_report: n_commit[n] of the planned step (0 <= n_commit[j] <=
 *   the block's still-masked rows); writes the ids of the blocks that are
 *   now complete and next in commit order to done[] (room for `window`)
 *   and returns their count.  Errors: BC_ERR_ORDER without a plan,
 *   BC_ERR_ARG for counts out of range (the state is left unchanged). */
typedef struct bc_pipeline bc_pipeline;
int bc_pipeline_create(const int32_t *block_sizes, int32_t n_blocks, int32_t window, double add,
                       double act, int32_t n_div, bc_pipeline **out);
void bc_pipeline_destroy(bc_pipeline *p);
int bc_pipeline_next(bc_pipeline *p, int32_t *active, int32_t *local_step, int32_t *mode,
                     int32_t *n_div, int32_t *blk_off, int32_t *row0);
int bc_pipeline_report(bc_pipeline *p, const int32_t *n_commit, int32_t *done);

/* ---- Pipelined parallel decoding, the whole step loop natively ----------
 * The same schedule (Fast-dVLA reading notes, key design 4 and its complete
 * example) with the per-step loop inside the library: plan, the model's
 * outputs for the step (from the caller's callback), bc_attn_step over the
 * active blocks' rows (BC_MASK_BLOCK_BIDIR), bc_unmask_select with the
 * planned modes and n_div, the report, and bc_kv_commit of the blocks it
 * returns, in order, each with the K/V of the step that completed it.  The
 * unmask writes each step's commit counts into host memory that the library
 * maps for the device (hipHostMalloc, mapped and coherent: one small buffer
 * per device, allocated on first use and held until the process ends), and
 * the host polls it instead of copying and synchronising the stream.
 * Decodes on one device take turns on that buffer (a lock), so overlapping
 * calls serialise.
 *
 * bc_step_inputs, filled by `inputs` for the planned step (device pointers,
 * rows = the active blocks' rows concatenated, oldest block first):
 *   q [1][rows][n_q_heads][head_dim]; k, v [1][n_kv_heads][rows][head_dim]
 *   (the cache's dtype); logits [rows][vocab] float32; blk_k[j], blk_v[j]
 *   [n_kv_heads][block rows][head_dim]: active block j's own K/V, appended to
 *   the cache if the block completes at this step.  They must stay valid
 *   until the step's work has run (the next callback, or the return).
 * inputs(user, step, n, active[n], local_step[n], in): returns 0, or nonzero
 *   to stop the decode (then BC_ERR_CALLBACK).
 * after_attn(user, step, n, active[n], local_step[n], cache_len, out): NULL,
 *   or called once the step's attention call is enqueued on `stream` (it may
 *   synchronise it to read `out`); nonzero stops the decode as above.
 *
 *   p        a schedule from bc_pipeline_create; the loop runs from its
 *            current state until every block is committed.
 *   cache    n_seq == 1; cache_len HOST [1], in/out, advanced by the commits.
 *   masked, tokens  device [sum of block sizes] uint8 / int32, in/out (all
 *            blocks' rows concatenated, as bc_pipeline_next's row0 counts).
 *   out      device [widest step's rows][n_q_heads][head_dim], cache dtype.
 *   ws_attn / ws_unmask  workspaces for the widest step (bc_attn_workspace_bytes
 *            and bc_unmask_workspace_bytes of that step's shapes).
 *   trace    HOST [max_steps][BC_PIPE_TRACE_INTS(window)] or NULL: per step
 *            n, n_done, active[window], mode[window], n_commit[window],
 *            done[window] (entries past n or n_done are -1).
 *   *n_steps the number of steps run.
 * Errors: BC_ERR_ARG (pointers, cache->n_seq != 1, max_steps < 0);
 * BC_ERR_CAPACITY when the decode needs more than max_steps steps (trace
 * given); BC_ERR_CALLBACK; any error of the calls above, returned as is
 * (the schedule and the buffers are then left where the failing step
 * stopped). */
#define BC_PIPE_TRACE_INTS(window) (2 + 4 * (window))
typedef struct {
  const void *q, *k, *v;
  const float *logits;
  const void *blk_k[BC_MAX_BLOCKS], *blk_v[BC_MAX_BLOCKS];
} bc_step_inputs;
typedef int (*bc_step_inputs_fn)(void *user, int32_t step, int32_t n_active, const int32_t *active,
                                 const int32_t *local_step, bc_step_inputs *in);
typedef int (*bc_after_attn_fn)(void *user, int32_t step, int32_t n_active, const int32_t *active,
                                const int32_t *local_step, int32_t cache_len, void *out);
int bc_pipeline_decode(bc_pipeline *p, const bc_kv_cache *cache, int32_t *cache_len, int32_t n_q_heads,
                       int32_t vocab, float scale, float threshold, uint8_t *masked, int32_t *tokens,
                       void *out, void *ws_attn, size_t ws_attn_bytes, void *ws_unmask, size_t ws_unmask_bytes,
                       bc_step_inputs_fn inputs, bc_after_attn_fn after_attn, void *user,
                       int32_t *trace, int32_t max_steps, int32_t *n_steps, void *stream);

/* ---- Pipelined parallel decoding with the schedule on the device --------
 * The same schedule and step as bc_pipeline_decode (Fast-dVLA reading notes,
 * key design 4), with the state machine run by a one-workgroup kernel after
 * each step's unmask: it takes the step's commit counts, appends the blocks
 * the step completed to the cache (in order, with the step's K/V rows), and
 * writes the next step's plan into device memory, where the next step's
 * kernels -- and the caller's model -- read it.  No step needs the host, so
 * runs of steps can be captured in one HIP graph and replayed; once every
 * block is committed, further steps do nothing.  Results (tokens, masks,
 * cache, per-step trace) are those of bc_pipeline_decode on the same model
 * outputs; attention is within the tolerance of a different split plan.
 *
 * Step buffers, the caller's device memory, hold R rows (R =
 * bc_pipeline_dev_rows: the widest step, the largest sum of `window`
 * consecutive block sizes); the step's rows come first, in plan order:
 *   q [R][n_q_heads][head_dim], k / v [n_kv_heads][R][head_dim] (cache dtype),
 *   logits [R][vocab] float32, out [R][n_q_heads][head_dim] (cache dtype).
 * Before each bc_pipeline_dev_step the caller's model writes the step's rows
 * of q, k, v and logits, as the plan (bc_pipeline_dev_plan) lays them out;
 * rows past plan->rows are never read for a result.
 *
 * bc_pipeline_dev_create: the schedule's parameters as bc_pipeline_create;
 *   cache with n_seq == 1 and prefix_len committed rows; masked / tokens
 *   device [sum of block sizes] (all blocks' rows); max_steps >= 1 bounds
 *   the trace.  The library allocates its device state, workspaces and trace
 *   (hipMalloc) and a small mapped host status, and owns them until
 *   bc_pipeline_dev_destroy.  Errors: BC_ERR_ARG, BC_ERR_UNSUPPORTED (as
 *   bc_attn_step / bc_unmask_select for the widest step, or a vocabulary
 *   that is not a multiple of 4), BC_ERR_HIP.
 * bc_pipeline_dev_reset: enqueues the start of a decode (initial state, the
 *   first plan); masked and tokens are the caller's to initialise.
 * bc_pipeline_dev_step: enqueues one step: attention over the planned rows,
 *   the unmask, the schedule kernel.  Nothing is read on the host.
 * bc_pipeline_dev_replay: a stand-in for the model, for tests and replays of
 *   recorded outputs: enqueues a copy of the planned blocks' rows from
 *   table[block * max_local + local_step] (device array of bc_step_block:
 *   q [size][n_q_heads][head_dim], k / v [n_kv_heads][size][head_dim],
 *   logits [size][vocab]) into the step buffers.  A missing entry (local
 *   step >= max_local or a null pointer) stops the decode with error 3.
 * bc_pipeline_dev_status: the state after the enqueued work has run (the
 *   caller synchronises first): finished (1 once every block is committed,
 *   or on an error), the steps run, the cache length, and error (0; 1 a
 *   commit count out of range; 2 more steps than max_steps; 3 a missing
 *   replay input).
 * bc_pipeline_dev_trace: waits for the device, then copies the per-step
 *   trace (the layout of bc_pipeline_decode's) of the steps run to the host
 *   and returns their count.
 * bc_pipeline_dev_read_plan: copies the next step's plan to the host once
 *   the device is idle (synchronous). */
typedef struct {
  int32_t n;        /* active blocks; 0 once every block is committed */
  int32_t rows;     /* their rows: the step's rows */
  int32_t row0;     /* first row of the first active block in masked / tokens */
  int32_t len;      /* committed cache length the step's attention sees */
  int32_t n_blk;    /* blocks of the attention: the active ones, then rows [rows, R) if any */
  int32_t blk_off[BC_MAX_BLOCKS + 2];
  int32_t active[BC_MAX_BLOCKS], local_step[BC_MAX_BLOCKS], mode[BC_MAX_BLOCKS], n_div[BC_MAX_BLOCKS];
} bc_dev_plan;
typedef struct {
  const void *q, *k, *v;
  const float *logits;
} bc_step_block;
typedef struct bc_pipeline_dev bc_pipeline_dev;
int bc_pipeline_dev_create(const int32_t *block_sizes, int32_t n_blocks, int32_t window, double add, double act,
                           int32_t n_div, const bc_kv_cache *cache, int32_t prefix_len, int32_t n_q_heads,
                           int32_t vocab, float scale, float threshold, uint8_t *masked, int32_t *tokens, void *q,
                           void *k, void *v, float *logits, void *out, int32_t max_steps, bc_pipeline_dev **dev);
void bc_pipeline_dev_destroy(bc_pipeline_dev *dev);
int bc_pipeline_dev_rows(const bc_pipeline_dev *dev);
const bc_dev_plan *bc_pipeline_dev_plan(const bc_pipeline_dev *dev);
int bc_pipeline_dev_reset(bc_pipeline_dev *dev, void *stream);
int bc_pipeline_dev_step(bc_pipeline_dev *dev, void *stream);
int bc_pipeline_dev_replay(bc_pipeline_dev *dev, const bc_step_block *table, int32_t max_local, void *stream);
int bc_pipeline_dev_status(const bc_pipeline_dev *dev, int32_t *finished, int32_t *n_steps, int32_t *cache_len,
                           int32_t *error);
int bc_pipeline_dev_trace(const bc_pipeline_dev *dev, int32_t *trace, int32_t max_steps);
int bc_pipeline_dev_read_plan(const bc_pipeline_dev *dev, bc_dev_plan *plan);

/* ------------------------------------------------------------------------ */
/* Attention without allocation or workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.
 *
 * Exactly bc_attn_step (same arguments, same kernels, same results), except
 * that the split partials live in the library's own scratch: one static
 * device array of BC_STATIC_SCRATCH_BYTES per GPU, which that GPU holds until
 * the process ends.  The call allocates nothing.  The first call on a device
 * looks the array's address up (with that device current); later calls reuse
 * it.  With n_prefix_splits == 0 the automatic split count is reduced to what
 * the scratch holds; a call that needs more than BC_STATIC_SCRATCH_BYTES even
 * with one split, or whose explicit split count does not fit, returns
 * BC_ERR_SCRATCH with nothing enqueued.  At most 64 devices.
 *
 * Every call on one GPU shares that GPU's array, and it keeps the last
 * call's contents (nothing in it needs to start at zero).  Calls that may
 * overlap on one GPU -- on different streams, or from different host threads
 * without ordering -- race on the array and give wrong results: issue them
 * on one stream, or use bc_attn_step with separate workspaces. */
#define BC_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int bc_attn_step_static(const bc_kv_cache *prefix, const int32_t *prefix_len,
                        const bc_kv_cache *priv, const int32_t *priv_len,
                        const bc_active *a, int32_t mask, float scale, int32_t n_prefix_splits,
                        void *out, void *stream);

/* Human-readable name of a bc_status value (never NULL). */
const char *bc_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* BC_H */
