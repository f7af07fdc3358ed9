/*
 * dflash.h -- C ABI of the DFlash draft-block hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (block-diffusion speculative decoding, "DFlash"):
 *   - kongchang.com, "D-Flash: diffusion drafting speeds LLM inference 3.5x",
 *     sections "System architecture", "Innovation 1: block-diffusion parallel
 *     drafting" and "Innovation 2: target-feature KV injection";
 *   - Google Developers Blog (zh translation on aihot.virxact.com), sections
 *     "Dual cache for attention", "Smart context management" and "Bridging the
 *     metadata gap in TPU inference".
 *
 * A proposer keeps, per sequence, a context buffer of projected target
 * features, one static (non-paged) K/V cache per draft layer, and the count
 * of committed positions that fixes the RoPE offset.  Each step:
 *   dflash_draft_block  -- one non-causal forward of [anchor, masks...] gives
 *                          K draft tokens;
 *   dflash_accept       -- greedy longest-prefix acceptance against the
 *                          target's tokens gives tau in [1, K+1];
 *   dflash_project_ctx  -- the tau newly committed positions are projected
 *                          and appended (never the drafts still being
 *                          verified), advancing the state by tau.
 *
 * Conventions for every entry point:
 *   - All functions have C linkage, never throw, and return dflash_status.
 *     On a non-OK status dflash_last_error() gives a message (per thread).
 *   - "dev" pointers are device memory on the current HIP device; "host"
 *     pointers are host memory.  The caller owns every input and output
 *     buffer.  Streams are hipStream_t handles passed as void* (NULL = the
 *     null stream).  Work is stream-ordered; outputs are valid once the
 *     stream has reached the call.  Host-side state (ctx_len, cap) is updated
 *     when the call is enqueued.
 *   - Arguments are checked before anything is enqueued; a rejected call
 *     (DFLASH_E_ARG / DFLASH_E_SHAPE / DFLASH_E_STATE) leaves all state
 *     untouched.  DFLASH_E_HIP reports a failed HIP call; after a device
 *     fault the context is undefined and must be destroyed.
 *   - A model is immutable after creation and may be shared by contexts; a
 *     context must be used from one thread at a time.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 1
#define DFLASH_MAX_BATCH 256
#define DFLASH_MAX_K 1024

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_ARG = -1,            /* NULL pointer, out-of-range value            */
  DFLASH_E_SHAPE = -2,          /* shapes that do not fit the model/context    */
  DFLASH_E_ALLOC = -3,          /* allocator returned NULL                     */
  DFLASH_E_HIP = -4,            /* a HIP runtime call failed                   */
  DFLASH_E_STATE = -5,          /* call not valid in the current state         */
  DFLASH_E_UNIMPLEMENTED = -6
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  head_dim must be a multiple of 16, n_q_heads a multiple of
 * n_kv_heads, intermediate a multiple of 8.  rope_theta is the RoPE base
 * (rotate-half pairs m, m + head_dim/2, angle p * theta^(-2m/head_dim)),
 * rms_eps the RMSNorm epsilon. */
typedef struct {
  int32_t hidden;
  int32_t n_layers;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  int32_t n_feat;
  double rope_theta;
  double rms_eps;
  dflash_dtype dtype;           /* storage and MFMA input type of weights and
                                   features (the KV caches: see
                                   dflash_ctx_buffers) */
} dflash_config;

/* One draft layer; dev pointers, dtype of the config, row-major [out, in]:
 *   attn_norm, mlp_norm [hidden]; wq [nq*d, hidden]; wk, wv [nkv*d, hidden];
 *   wo [hidden, nq*d]; w_gate, w_up [intermediate, hidden];
 *   w_down [hidden, intermediate]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *mlp_norm, *w_gate, *w_up, *w_down;
} dflash_layer_weights;

/* embed [vocab, hidden]; lm_head [vocab, hidden] (may equal embed: tied);
 * fc [hidden, n_feat*hidden]; final_norm [hidden]; layers: HOST array of
 * n_layers entries.  Only `embed` is borrowed after dflash_model_create
 * returns (it must outlive the model); everything else is repacked into
 * model-owned memory. */
typedef struct {
  const void *embed, *lm_head, *fc, *final_norm;
  const dflash_layer_weights *layers;
} dflash_weights;

/* Device-memory allocator used for every buffer the library owns.  NULL
 * allocator = hipMalloc / hipFree.  `free` may be called while work that
 * used the block is still queued on the stream given to the call that frees
 * it; the allocator must keep stream-ordered reuse safe (a caching allocator
 * tied to that stream is). */
typedef struct {
  void *(*alloc)(size_t bytes, void *user);
  void (*free)(void *ptr, void *user);
  void *user;
} dflash_allocator;

typedef struct dflash_model dflash_model;
typedef struct dflash_ctx dflash_ctx;

/* Library version string and ABI version. */
const char *dflash_version(void);
int32_t dflash_abi_version(void);

/* Message for the last non-OK status returned on this thread. */
const char *dflash_last_error(void);

/* The drafter (kongchang.com, "D-Flash: diffusion drafting speeds LLM
 * inference 3.5x", "System architecture": draft layers of bidirectional
 * attention and an MLP, conditioned on a light projection of hidden states
 * taken from several target layers, logits from the target's LM head;
 * "Innovation 2: target-feature KV injection": that projection enters every
 * layer through the layer's own K/V projections).
 *   cfg    host, the shape; checked (DFLASH_E_ARG / DFLASH_E_SHAPE).
 *   w      host struct of dev pointers in cfg->dtype (see dflash_weights).
 *   alloc  host, the allocator for every model-owned buffer, or NULL.
 *   out    host, receives the model handle (NULL on failure).
 * Validates the config, allocates model memory through `alloc` and repacks
 * the weights into tiles laid out for gfx950 MFMA (a private copy; rows of
 * W_q/W_k are reordered to pair RoPE channels, W_gate/W_up are interleaved,
 * the per-layer W_k/W_v are stacked for context injection).  The repack runs
 * on `stream` and is complete when the call returns; on failure everything
 * allocated is released.  dflash_model_destroy releases the model's memory
 * (no context of it may be used afterwards; NULL is accepted). */
dflash_status dflash_model_create(const dflash_config *cfg, const dflash_weights *w,
                                  const dflash_allocator *alloc, void *stream,
                                  dflash_model **out);
dflash_status dflash_model_destroy(dflash_model *m);

/* Target model for block verification (Google Developers Blog, "Overcoming
 * the autoregressive bottleneck" and "K-Flat"; kongchang.com "D-Flash",
 * "System architecture"): a decoder of the same layer form as the drafter
 * (RMSNorm, GQA attention with rotate-half RoPE, SwiGLU MLP, final RMSNorm,
 * LM head) but causal, with no context projection.  cfg->n_feat is the
 * number of tapped layers (0 allowed) and taps (host [n_feat], increasing
 * layer indices) the layers whose output residual rows dflash_verify_block
 * returns as the drafter's features, concatenated in tap order.  w->fc is
 * ignored (may be NULL).  Packing, ownership and errors as in
 * dflash_model_create.  Contexts of a target come from dflash_ctx_create;
 * they hold the target's K/V cache of committed positions and accept only
 * dflash_verify_block and dflash_commit (the drafter calls return
 * DFLASH_E_STATE on them, and the verification calls on a drafter's). */
dflash_status dflash_target_create(const dflash_config *cfg, const dflash_weights *w,
                                   const int32_t *taps, const dflash_allocator *alloc, void *stream,
                                   dflash_model **out);

/* Weight bytes the hot path streams per draft block (packed matrices plus
 * gains), for roofline accounting. */
dflash_status dflash_model_bytes(const dflash_model *m, int64_t *layer_bytes,
                                 int64_t *lm_head_bytes, int64_t *proj_bytes);

/* Proposer state (Google Developers Blog, "Dual cache for attention": the
 * drafter keeps a static, non-paged cache of its own beside the target's
 * paged one; "Smart context management": a context buffer of power-of-two
 * capacity that only newly accepted positions are appended to;
 * "Bridging the metadata gap in TPU inference": the committed length and
 * RoPE offset persist across steps).
 * Creates proposer state for `batch` sequences (1..DFLASH_MAX_BATCH) of
 * model m (which must outlive it).
 *   init_cap  host [batch] powers of two, the initial context capacity of
 *             each sequence, or NULL for capacity 0 (buffers are then
 *             created by the first dflash_project_ctx); checked (E_ARG).
 *   alloc     host, the allocator for every buffer the context owns, or NULL.
 *   stream    the stream the initial buffer set-up is enqueued on.
 *   out       host, receives the handle (NULL on failure).
 * All sequences start with ctx_len = 0.  dflash_ctx_destroy releases every
 * buffer through the allocator (work still queued on them must be on the
 * stream the allocator orders reuse by; NULL is accepted). */
dflash_status dflash_ctx_create(const dflash_model *m, int32_t batch, const int32_t *init_cap,
                                const dflash_allocator *alloc, void *stream,
                                dflash_ctx **out);
dflash_status dflash_ctx_destroy(dflash_ctx *c);

/* (a1)-(a3): context projection, append and KV injection.
 * Appends n_new[b] positions to sequence b: c_j = W_fc feats_j is written to
 * the context buffer at row ctx_len[b] + j, and for every layer l,
 * K_l = RoPE(W_k^l c_j, pos_j) and V_l = W_v^l c_j to that layer's cache at
 * the same row (kongchang.com, "System architecture" and "Innovation 2";
 * Google Developers Blog, "Smart context management").
 *   feats     dev [sum(n_new), n_feat*hidden], config dtype, row-major,
 *             sequences concatenated in batch order.
 *   n_new     host [batch], each >= 0.  The committed count of the last step
 *             (tau), never the drafted length.
 *   positions dev [sum(n_new)] int32 RoPE positions, or NULL for
 *             ctx_len[b] + j.
 * If ctx_len[b] + n_new[b] exceeds cap[b], the sequence's buffers are
 * reallocated with cap = the next power of two of the new length, and the
 * held rows copied, on `stream`.  Afterwards ctx_len[b] += n_new[b].
 * Rejects ctx_len + n_new > 2^30 (DFLASH_E_SHAPE). */
dflash_status dflash_project_ctx(dflash_ctx *c, const void *feats, const int32_t *n_new,
                                 const int32_t *positions, void *stream);

/* (a4)-(a9): one draft block for every sequence.
 *   block_ids dev [batch, K] int32: row 0 the anchor (last verified token),
 *             rows 1..K-1 mask tokens.  Ids outside [0, vocab) are clamped.
 *   K         1..DFLASH_MAX_K.
 *   draft_ids dev [batch, K] int32 out: argmax of row i's logits (the draft
 *             for position ctx_len + 1 + i); ties go to the lowest index.
 *   logits    dev [batch, K, vocab] float32 out, or NULL.
 *   hidden    dev [batch, K, hidden] out, config dtype, the final-normed
 *             hidden state fed to the LM head, or NULL.
 * Row i sits at position ctx_len[b] + i.  Every layer: RMSNorm, Q/K/V with
 * RoPE, attention of every block row over the sequence's whole context
 * and the whole block (no causal mask), output projection + residual,
 * RMSNorm, SwiGLU MLP + residual; then final RMSNorm, LM head, argmax
 * (kongchang.com, "System architecture", "Innovation 1"; Google Developers
 * Blog, "Dual cache for attention").  Does not change the state.
 * Arithmetic of DFLASH_BF16 models: bf16 weights, the residual stream in
 * fp32, every product's activations fed as a bf16 hi/lo pair (about fp32)
 * but the LM head's above 32 rows (bf16), fp32 sums; attention operands
 * fp16, softmax in fp32. */
dflash_status dflash_draft_block(dflash_ctx *c, const int32_t *block_ids, int32_t K,
                                 int32_t *draft_ids, float *logits, void *hidden,
                                 void *stream);

/* (a1)-(a9) in one call: dflash_project_ctx(feats, n_new, positions = NULL)
 * followed by dflash_draft_block(block_ids, K, ...), with the same results
 * up to rounding.  The projected features of the appended positions join
 * the block rows in each layer's Q/K/V product, which writes their K and V
 * into that layer's cache (the W_k / W_v of the layer stream once for both;
 * kongchang.com, "Innovation 2: target-feature KV injection"; Google
 * Developers Blog, "Smart context management": only newly accepted
 * positions are projected).  Appends of more than 64 rows in all, or whose
 * rows and the block's need more than four 16-row tiles, run as the two
 * separate calls.  Arguments, ownership and errors as in those calls;
 * state advances by n_new exactly as dflash_project_ctx does. */
dflash_status dflash_step(dflash_ctx *c, const void *feats, const int32_t *n_new,
                          const int32_t *block_ids, int32_t K, int32_t *draft_ids,
                          float *logits, void *hidden, void *stream);

/* (a10): greedy acceptance (Google Developers Blog, "Overcoming the
 * autoregressive bottleneck"; table 2 caption: greedy decoding).
 *   draft_ids, target_ids dev [batch, K] int32; accept_len dev [batch] int32
 *   out: 1 + the number of leading positions where the two agree. */
dflash_status dflash_accept(const int32_t *draft_ids, const int32_t *target_ids, int32_t batch,
                            int32_t K, int32_t *accept_len, void *stream);

/* Loss-decay weighted cross-entropy for training the drafter (kongchang.com,
 * "D-Flash", "Innovation 4: loss-decay weighted training": the CE of the
 * token at in-block position k is weighted by gamma^k; "Innovation 3: random
 * anchor sampling": block row k predicts the token k + 1 places after the
 * block's clean anchor).  Rows are laid out as consecutive blocks of `block`
 * rows, row r at in-block position r % block:
 *   w_r  = gamma^(r % block) if 0 <= targets[r] < vocab, else 0
 *   ce_r = logsumexp(logits_r) - logits_r[targets_r]      (0 if w_r = 0)
 *   loss = sum_r w_r ce_r / sum_r w_r                      (0 if sum w = 0)
 *   grad = d loss / d logits = w_r / sum w * (softmax(logits_r) - onehot)
 * Arguments:
 *   logits    dev [rows, vocab] of dtype, row-major, finite values
 *   targets   dev [rows] int32; values outside [0, vocab) mark rows without
 *             a token
 *   rows      >= 0 (0 gives loss 0); vocab >= 1; block >= 1; gamma > 0
 *   loss      dev [1] float out
 *   ce        dev [rows] float out (may be NULL when rows = 0)
 *   grad      dev [rows, vocab] of dtype out, or NULL for no gradient
 *   workspace dev, DFLASH_DECAY_CE_WORKSPACE bytes, 8-byte aligned, owned by
 *             the caller; calls that share it must be ordered on one stream
 * Arithmetic in fp32 with fp64 sums over rows, in an order fixed by rows
 * alone (the loss is reproducible bit for bit).  Logits are read once from
 * HBM when rows are 16-byte aligned and vocab * element size is a multiple
 * of 16 with at most 20480 16-byte vectors per row (bf16 vocab <= 163840,
 * fp32 <= 81920), else twice.  Asynchronous on `stream`. */
#define DFLASH_DECAY_CE_WORKSPACE 256
dflash_status dflash_decay_ce(const void *logits, dflash_dtype dtype, const int32_t *targets,
                              int32_t rows, int32_t vocab, int32_t block, double gamma, float *loss,
                              float *ce, void *grad, void *workspace, void *stream);

/* dflash_decay_ce without the workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, serving loops and
 * harnesses that forbid allocation): the library allocates nothing in this
 * call.  The workspace is a file-scope device array of
 * DFLASH_DECAY_CE_WORKSPACE bytes, one per GPU, held until the process
 * ends; its device address is looked up on the first call on each GPU.
 * The kernels use one double of it whatever rows and vocab are, so no input
 * size exceeds it; other arguments, limits, results and errors as in
 * dflash_decay_ce (the same kernels).  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams) race;
 * calls ordered on one stream do not (each writes the slot before reading
 * it).  Asynchronous on `stream`. */
dflash_status dflash_decay_ce_noalloc(const void *logits, dflash_dtype dtype, const int32_t *targets,
                                      int32_t rows, int32_t vocab, int32_t block, double gamma, float *loss,
                                      float *ce, void *grad, void *stream);

/* Target-side verification of a block of K1 rows per sequence: the anchor
 * (at position ctx_len) and the K1 - 1 drafts after it (Google Developers
 * Blog, "Overcoming the autoregressive bottleneck": one parallel forward of
 * the target checks the whole block).  Row i attends to the committed
 * positions and to block rows 0..i; its K/V are written to the cache at
 * slot ctx_len + i (growing the capacity to the next power of two of
 * ctx_len + K1 first if needed) but not committed.
 *   block_ids  dev [batch, K1] int32 (ids outside [0, V) are clamped)
 *   target_ids dev [batch, K1] int32 out: argmax of row i (lowest index on
 *              ties), the target's token for position ctx_len + 1 + i
 *   logits     dev [batch, K1, V] float32 out, or NULL
 *   taps       dev [batch, K1, n_feat * hidden] model dtype out, or NULL:
 *              the residual rows after each tapped layer, in tap order
 * 1 <= K1 <= DFLASH_MAX_K.  Asynchronous on `stream`.
 * dflash_commit then keeps the first n_acc[b] rows of sequence b's last
 * verified block (n_acc host [batch], 0 <= n_acc[b] <= K1; normally the
 * acceptance length tau of dflash_accept): ctx_len advances by n_acc[b]
 * (Google Developers Blog, "Bridging the metadata gap": only accepted
 * positions count).  A commit consumes the verification; committing again,
 * or more rows than were verified, returns DFLASH_E_STATE. */
dflash_status dflash_verify_block(dflash_ctx *c, const int32_t *block_ids, int32_t K1,
                                  int32_t *target_ids, float *logits, void *taps, void *stream);
dflash_status dflash_commit(dflash_ctx *c, const int32_t *n_acc, void *stream);

/* Adaptive block size (host computation; kongchang.com "D-Flash",
 * "Ablations": a drafter trained on a large block serves smaller blocks, so
 * the block size can follow the load; Google Developers Blog, "Scaling
 * theory" and "Predictability": acceptance at block position i has
 * probability a * gamma^i, the decay depending on the task).
 *   dflash_adapt_create   kmax: largest block size observed (1..DFLASH_MAX_K);
 *                         decay in (0, 1]: forgetting factor applied to the
 *                         statistics at every observed step; min_count: the
 *                         weight a position needs to enter the fit; (a0,
 *                         gamma0) in (0, 1]: the estimate until two
 *                         positions qualify.
 *   dflash_adapt_observe  one step drafted at block size K (<= kmax) with
 *                         acceptance length tau in [1, K + 1].
 *   dflash_adapt_choose   the current (a, gamma) (weighted least squares of
 *                         log((agreed + 1/2) / (reached + 1)) on the
 *                         position, weights = reached, clamped to [1e-6, 1])
 *                         and, among the n candidates Ks (host, strictly
 *                         increasing) with per-step costs cost (host, > 0,
 *                         e.g. draft + verify latency at that K), the K
 *                         maximising E[tau | K] / cost(K) with
 *                         E[tau | K] = 1 + sum_{m<=K} prod_{i<m} a gamma^i,
 *                         the smaller K on ties; *tokens_per_cost is that
 *                         maximum.  Outputs may be NULL.
 * The policy is plain host memory: no device, no stream; one thread at a
 * time per policy. */
typedef struct dflash_adapt dflash_adapt;
dflash_status dflash_adapt_create(int32_t kmax, double decay, double min_count, double a0, double gamma0,
                                  dflash_adapt **out);
dflash_status dflash_adapt_destroy(dflash_adapt *p);
dflash_status dflash_adapt_observe(dflash_adapt *p, int32_t K, int32_t tau);
dflash_status dflash_adapt_choose(const dflash_adapt *p, const int32_t *Ks, const double *cost, int32_t n,
                                  int32_t *K, double *a, double *gamma, double *tokens_per_cost);

/* Host copies of the state (Google Developers Blog, "Bridging the metadata
 * gap in TPU inference": the host keeps the committed length that fixes
 * the RoPE offset; "Smart context management": the power-of-two capacity):
 * ctx_len and cap, host [batch] each, written by the call (either may be
 * NULL).  No device work: the host values are authoritative and were
 * updated when the last call was enqueued. */
dflash_status dflash_ctx_query(const dflash_ctx *c, int32_t *ctx_len, int32_t *cap);

/* Device buffers of sequence b (Google Developers Blog, "Dual cache for
 * attention" and "Smart context management": the static cache and the
 * context buffer; for tests and snapshots).  b in [0, batch), else E_ARG.
 * Outputs are host pointers to write (any may be NULL); the buffers stay
 * owned by the context:
 *   ctxbuf  [phys_rows, hidden] float32           projected features
 *   k_cache [n_layers, n_kv_heads, phys_rows, head_dim]   RoPE applied
 *   v_cache [n_layers, n_kv_heads, head_dim, phys_rows]   (transposed)
 * The caches hold fp16 for DFLASH_BF16 models (same bytes as bf16, finer
 * rounding; stores saturate at +-65504) and float32 for DFLASH_F32 models.
 * Rows [0, ctx_len) are valid; phys_rows >= cap.  Pointers change when the
 * buffers grow. */
dflash_status dflash_ctx_buffers(const dflash_ctx *c, int32_t b, const void **ctxbuf,
                                 const void **k_cache, const void **v_cache,
                                 int32_t *phys_rows);

/* Single-launch draft block.  For bf16 drafters of at most 16 layers whose
 * block has at most 16 rows in all (batch * K <= 16) and at most 64 query
 * rows per KV head ((n_q_heads / n_kv_heads) * K <= 64), and whose products
 * split into at most 40 passes per workgroup, dflash_draft_block runs a4-a9
 * as one cooperative launch of one workgroup per compute unit, with the same
 * arithmetic as the per-product kernels up to summation order (kongchang.com,
 * "System architecture": one forward per block).  In each workgroup four
 * loader waves stream the weights of every product of the block, in order,
 * into LDS rings that four compute waves consume, so the weight stream runs
 * on across the dependencies between products.  Its grid barriers and ring
 * waits end after about 2 s; an expired wait abandons the launch and is
 * reported by dflash_ctx_check.  In dflash_step the appended positions then
 * go through dflash_project_ctx before the block.  The path is slower than
 * the per-product kernels on the shapes measured so far (off by default).
 *   dflash_ctx_set_persistent   enable or disable (default) the path for c;
 *                               the environment variable DFLASH_PERSISTENT=1
 *                               enables it for contexts created afterwards.
 *   dflash_ctx_persistent_path  *yes = 1 if a block of K rows per sequence
 *                               takes the path on this device, else 0.
 *   dflash_ctx_check            waits for `stream`, then returns DFLASH_E_HIP
 *                               if a launch on c was abandoned since the last
 *                               check (its outputs are invalid; the barrier
 *                               state is reset), else DFLASH_OK. */
dflash_status dflash_ctx_set_persistent(dflash_ctx *c, int32_t enable);
dflash_status dflash_ctx_persistent_path(dflash_ctx *c, int32_t K, int32_t *yes);
dflash_status dflash_ctx_check(dflash_ctx *c, void *stream);

/* Per-kernel timing with HIP events recorded on the call's stream around
 * every launch of dflash_project_ctx / dflash_draft_block that belongs to a
 * phase selected by dflash_profile_enable (bit p of phase_mask selects phase
 * p; 0 turns timing off; bits past the last phase are ignored).
 * Phases (index: name): 0 embed, 1 qkv, 2 attention, 3 o_proj, 4 gate_up,
 * 5 down, 6 lm_head, 7 finalize, 8 fc, 9 kv_inject, 10 grow, 11 rowmap,
 * 12 attn_combine, 13 resid_norm (blocks of more than 64 rows; smaller
 * ones add into the residual in the products' epilogue), 14 fc_finalize,
 * 15 persistent_draft (the whole draft block as one launch, see
 * dflash_ctx_set_persistent).
 * dflash_profile_read waits for the recorded events, adds their durations
 * (milliseconds) and launch counts per phase into ms[] / count[] (host
 * arrays of DFLASH_NUM_PHASES entries, overwritten) and clears the record. */
#define DFLASH_NUM_PHASES 16
dflash_status dflash_profile_enable(dflash_ctx *c, uint32_t phase_mask);
/* Timeline of the last single-launch draft block run while phase 15 was
 * selected: *nwg workgroups x *stride slots (host out [nwg * stride] uint64,
 * capacity entries), ticks of the GPU's constant 100 MHz clock per
 * workgroup, 8 slots per phase (embed, then qkv, attention, attention merge,
 * o_proj, gate_up, down per layer, then lm_head): 0 start, 1-5 marks inside
 * the phase (2 first pass's product done, 3 its sums and epilogue done, 4
 * all passes done), 6
 * arrival at the barrier that ends it (lm_head: end of work), 7 release;
 * unwritten slots are 0.  *nwg = 0 if none was recorded; out = NULL only returns the sizes.
 * Waits for the device. */
dflash_status dflash_persist_trace(dflash_ctx *c, uint64_t *out, int64_t capacity, int32_t *nwg,
                                   int32_t *stride);
dflash_status dflash_profile_read(dflash_ctx *c, double *ms, int64_t *count);
const char *dflash_phase_name(int32_t phase);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
