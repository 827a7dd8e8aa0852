/* dflash.h - C ABI of the DFlash drafting + verification cycle for AMD gfx950.
 *
 * Source of the method: "DFlash: Block Diffusion for Flash Speculative
 * Decoding" (technical summary on gist.science, Japanese and Dutch pages;
 * abstract on the fugumt.com paper page).  The three calls follow the
 * summary's statement of the inference path (section 2.2):
 *   - dflash_inject_kv:   context-feature fusion (first bullet) and KV injection
 *                         into every draft layer's cache (second bullet);
 *   - dflash_draft_block: one forward pass of the drafter over a block made of
 *                         a clean anchor token plus gamma-1 mask tokens (third
 *                         bullet; anchor from section 2.3), ending in the
 *                         target's shared LM head (section 2.3, architecture);
 *   - dflash_verify:      greedy verification - the longest prefix of drafts
 *                         equal to the target's greedy tokens plus one bonus
 *                         token (sections 1, 4 and 5: lossless vs. greedy).
 * Around the cycle, for a target model of the drafter's layer recipe:
 *   - dflash_target_forward: the target's parallel check of a block (the
 *                         verification forward of sections 1 and 2.2) with its
 *                         greedy tokens and the tapped hidden states that the
 *                         next dflash_inject_kv consumes (section 2.2, first
 *                         bullet: evenly spread target layers);
 *   - dflash_advance_len: len += accepted rows after verification.
 *
 * General rules
 *   - Pointers are device pointers unless marked [host].  The library never
 *     allocates, frees or synchronises; every call is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and returns immediately.
 *   - The caller owns every buffer; buffers must stay alive until the queued
 *     work has finished.  The library keeps no global mutable state: calls on
 *     different streams are safe when they use disjoint buffers (including
 *     disjoint workspaces).
 *   - Errors the host can see (NULL pointers, sizes out of range, unsupported
 *     shapes, a workspace that is too small) return a negative dflash_status
 *     and enqueue nothing.  Errors only the device can see (a cache that would
 *     overflow, a token id outside the vocabulary, a negative row count) set a
 *     sticky bit in *kv->status and skip the offending write; nothing is ever
 *     written out of bounds.  The library never prints or aborts.
 *
 * Storage types: every weight, the K/V cache and the input features use the
 * configuration's dtype (DFLASH_F32 or DFLASH_BF16, bf16 = raw bit patterns).
 * Activations between layers are fp32; every GEMM input is rounded to the
 * storage type (round-to-nearest-even), as are q, k and v.
 *
 * Layouts (row-major, innermost last):
 *   weight matrices           [out][in]   (as torch.nn.Linear.weight)
 *   w_fuse                    [H][F*H]    (input = the F feature rows concatenated,
 *                                          shallowest tapped layer first)
 *   K cache  kv->k            [L][max_batch][n_kv][kv_capacity][D]
 *   V cache  kv->v            [L][max_batch][n_kv][kv_capacity/32][D][32]: blocks of 32
 *                             positions, each stored transposed (the value of position
 *                             32*i + j, dimension d at [i][d][j]), so the values of 32
 *                             consecutive positions are one contiguous span
 *   kv->len                   int32 [max_batch]: rows of context held per sequence
 *   rope_cos / rope_sin       fp32 [rope_rows][D/2]: cos/sin of p * theta^(-2i/D)
 *                             for position p (rotate-half pairs (i, i+D/2))
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFLASH_OK = 0,
    DFLASH_EINVAL = -1,        /* NULL pointer or size out of range */
    DFLASH_EUNSUPPORTED = -2,  /* shape or dtype this build does not handle */
    DFLASH_EWORKSPACE = -3,    /* workspace NULL or smaller than dflash_workspace_bytes() */
    DFLASH_ELAUNCH = -4,       /* the HIP runtime rejected a launch */
    DFLASH_ESCRATCH = -5       /* dflash_draft_block_noalloc: the call needs more than the fixed scratch */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Device-side sticky status bits (OR-ed into *kv->status). */
#define DFLASH_STATUS_KV_OVERFLOW 1u  /* len + new rows (or block) exceeds kv_capacity / rope_rows */
#define DFLASH_STATUS_BAD_TOKEN   2u  /* anchor id outside [0, vocab) (id 0 used instead) */
#define DFLASH_STATUS_BAD_COUNT   4u  /* n_new outside [0, rows_stride] or len < 0 */

/* Model shape [host].  Supported: head_dim*sizeof(dtype) == 256 (bf16 D=128,
 * f32 D=64); n_q_heads % n_kv_heads == 0; hidden, inter, n_feat*hidden and
 * n_q_heads*head_dim multiples of 256 (bf16) / 128 (f32); n_kv_heads*head_dim
 * a multiple of 128; inter a multiple of 64; 2 <= gamma_max <= 16;
 * kv_capacity a multiple of 64. */
typedef struct {
    int32_t hidden;         /* H */
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;       /* D */
    int32_t inter;          /* SwiGLU intermediate size I */
    int32_t n_layers;       /* L draft layers */
    int32_t n_feat;         /* F target layers fused */
    int32_t vocab;          /* V */
    int32_t gamma_max;      /* largest block size used with this cache/workspace */
    int32_t mask_token_id;  /* embedding row used for the gamma-1 mask positions */
    int32_t max_batch;      /* sequences held by the cache */
    int32_t kv_capacity;    /* cache rows per (layer, sequence, kv head) */
    float rms_eps;
    int32_t dtype;          /* dflash_dtype */
} dflash_config;

/* One draft layer (all [host] struct, device pointers inside). */
typedef struct {
    const void *in_norm;    /* [H]        input RMSNorm scale (also applied to context rows) */
    const void *wq;         /* [n_q*D][H] */
    const void *wk;         /* [n_kv*D][H] */
    const void *wv;         /* [n_kv*D][H] */
    const void *q_norm;     /* [D]        per-head RMSNorm scale of q */
    const void *k_norm;     /* [D]        per-head RMSNorm scale of k */
    const void *wo;         /* [H][n_q*D] */
    const void *post_norm;  /* [H]        RMSNorm before the MLP */
    const void *w_gate;     /* [I][H] */
    const void *w_up;       /* [I][H] */
    const void *w_down;     /* [H][I] */
} dflash_layer_weights;

typedef struct {
    const void *w_fuse;      /* [H][F*H] */
    const void *embed;       /* [V][H]   the target's frozen token embedding */
    const void *final_norm;  /* [H] */
    const void *lm_head;     /* [V][H]   the target's frozen LM head (may alias embed) */
    const float *rope_cos;   /* [rope_rows][D/2] */
    const float *rope_sin;   /* [rope_rows][D/2] */
    int32_t rope_rows;       /* must be >= kv_capacity + gamma_max */
    const dflash_layer_weights *layers;  /* [host] array of n_layers */
} dflash_weights;

typedef struct {
    void *k;           /* K cache, layout above */
    void *v;           /* V cache (32-position blocks, each transposed), layout above */
    int32_t *len;      /* [max_batch] */
    uint32_t *status;  /* [1] sticky device status bits */
} dflash_kv;

/* Bytes of workspace needed by dflash_inject_kv / dflash_draft_block for up to
 * `batch` sequences and up to `max_rows_per_seq` injected rows per sequence per
 * call.  The workspace is scratch: every call writes whatever it later reads
 * from it, so it needs no initialisation and keeps nothing between calls.
 * Calls that share a workspace must be ordered (e.g. on one stream).
 * Returns 0 for an invalid or unsupported configuration. */
size_t dflash_workspace_bytes(const dflash_config *cfg, int32_t batch, int32_t max_rows_per_seq);

/* Stages 1-2 (summary section 2.2): for every sequence b < batch and row
 * i < n_new[b], fuse feat[b][i][0..F-1][0..H-1] with W_fuse, pass the fused
 * feature through every layer's input RMSNorm, W_k / W_v, per-head k RMSNorm
 * and RoPE at position len[b] + i, and store the rounded k and v rows at that
 * position of each layer's cache; then len[b] += n_new[b].
 *   feat     [batch][rows_stride][F][H] in the storage dtype
 *   n_new    device int32 [batch], each in [0, rows_stride] (the accept_len of
 *            dflash_verify can be passed straight in)
 * If len[b] + n_new[b] > kv_capacity nothing is written for b, len[b] is
 * unchanged and DFLASH_STATUS_KV_OVERFLOW is set.
 * 1 <= rows_stride <= max_rows_per_seq given to dflash_workspace_bytes. */
int dflash_inject_kv(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                     int32_t batch, const void *feat, int32_t rows_stride, const int32_t *n_new,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Stage 3 (summary section 2.2, third bullet): for each sequence b, one
 * forward pass over ids [anchor[b], MASK x (gamma-1)] at positions
 * len[b] .. len[b]+gamma-1 with attention over [cached context (len[b] rows)
 * ; the block's own keys/values], no mask inside the block; then the final
 * RMSNorm, the LM head and a row-wise argmax (ties -> lowest id) on the gamma-1
 * mask rows.  The block's own K/V are not written to the cache and len is not
 * changed.  Requires len[b] + gamma <= rope_rows.  The argmax is taken before the final
 * RMSNorm's row factor (positive, the same for every id of a row, so it moves no row's
 * maximum): ties go to the lowest id among equal pre-factor logits.
 *   anchor      int32 [batch]
 *   draft       int32 [batch][gamma-1]   d_1 .. d_{gamma-1}
 *   dbg_hidden  nullable fp32 [batch][gamma][H]: final residual stream (before the final norm)
 *   dbg_logits  nullable fp32 [batch][gamma-1][V]: logits of the mask rows, with the row factor
 *               (each draft id's logit is its row's maximum)
 * 2 <= gamma <= gamma_max, 1 <= batch <= max_batch. */
int dflash_draft_block(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                       int32_t batch, int32_t gamma, const int32_t *anchor, int32_t *draft,
                       float *dbg_hidden, float *dbg_logits,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Stage 4 (summary sections 1, 4, 5): per sequence, k = the number of leading
 * j in 1..gamma-1 with draft[b][j-1] == target[b][j-1]; accept_len[b] = k + 1;
 * committed[b][0..k] = target[b][0..k], the rest -1; next_anchor[b] =
 * target[b][k].  target[b][j] is the target's greedy token at block position j
 * (its choice for the position that draft d_{j+1} filled).
 *   draft  int32 [batch][gamma-1];  target int32 [batch][gamma]
 * 2 <= gamma <= 1024, batch >= 1.  Exact integer work. */
int dflash_verify(int32_t batch, int32_t gamma, const int32_t *draft, const int32_t *target,
                  int32_t *accept_len, int32_t *committed, int32_t *next_anchor, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as dflash_draft_block, with the same arguments except the workspace,
 * which is a fixed array inside the library instead - one per GPU, of
 * dflash_noalloc_scratch_bytes() bytes (64 MiB), placed in each device's
 * memory when the library is loaded and held until the process ends.  Neither
 * call allocates or frees anything (the array's device address is looked up
 * once per device, on the first call made with that device current, which
 * must be the device of `stream`).  Every call on a GPU uses that GPU's one
 * array: calls that may overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  Nothing in the array needs to start
 * at zero (each call writes what it later reads).  Results are the same as
 * dflash_draft_block's, bit for bit.  A call whose workspace
 * (dflash_workspace_bytes(cfg, batch, 0)) exceeds the array returns
 * DFLASH_ESCRATCH and enqueues nothing; other errors as for dflash_draft_block. */
size_t dflash_noalloc_scratch_bytes(void);
int dflash_draft_block_noalloc(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                               int32_t batch, int32_t gamma, const int32_t *anchor, int32_t *draft,
                               float *dbg_hidden, float *dbg_logits, void *stream);

/* Tracing (optional per-launch timing).  The caller creates hipEvents and
 * passes their handles; the *_traced variants record events[2*i] before and
 * events[2*i+1] after the i-th kernel launch of the call, on `stream`, for
 * every i < capacity whose handles are non-NULL.  On return `count` holds the
 * number of launches the call made and, when `names` is non-NULL, names[i]
 * points to a static string naming launch i (e.g. "lm_head_argmax").  A call
 * with events == NULL records nothing; launch order is the same as for the
 * untraced call, so a first call can be used to learn count and names. */
typedef struct {
    void **events;         /* [host] 2*capacity hipEvent_t handles, entries may be NULL */
    int32_t capacity;      /* launch slots described by events / names */
    int32_t count;         /* [out] launches made */
    const char **names;    /* [host, optional] [capacity] out: launch names */
} dflash_trace;

int dflash_inject_kv_traced(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                            int32_t batch, const void *feat, int32_t rows_stride, const int32_t *n_new,
                            void *workspace, size_t workspace_bytes, void *stream, dflash_trace *trace);

int dflash_draft_block_traced(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                              int32_t batch, int32_t gamma, const int32_t *anchor, int32_t *draft,
                              float *dbg_hidden, float *dbg_logits,
                              void *workspace, size_t workspace_bytes, void *stream, dflash_trace *trace);

/* Target-side verification forward (summary sections 1 and 2.2): a causal
 * model with the drafter's layer recipe (n_layers decoder layers, its own K/V
 * cache in `kv`, same layouts; the embedding and LM head may be the pointers
 * the drafter uses, which shares them with the target - section 2.3).  For each
 * sequence b, the `rows` tokens tokens[b][*] at positions len[b] .. len[b] +
 * rows - 1: writes their k (RMSNorm + RoPE) and v rows into every layer's cache
 * at those positions, attends to [cached context (len[b] rows) ; the block's
 * rows up to and including its own position], and returns
 *   y     int32 [batch][rows]: argmax of the logits of every row - the target's
 *         greedy token after each position (taken as in dflash_draft_block: before the
 *         final norm's positive row factor, ties to the lowest id);
 *   feat  nullable, storage dtype [batch][rows][n_taps][H]: the residual stream
 *         after decoder layer taps[f] (1-based), the layout dflash_inject_kv reads;
 *   dbg_logits nullable fp32 [batch][rows][V].
 * len is not changed: after dflash_verify, dflash_advance_len(cfg, kv, batch,
 * accept_len) keeps the accepted rows (later rows are overwritten next time);
 * a prompt is processed in chunks of at most gamma_max rows, each followed by
 * dflash_advance_len with n = rows.  w->w_fuse is not used (may be NULL).
 * 1 <= rows <= gamma_max, 1 <= batch <= max_batch, 0 <= n_taps <= 16, taps
 * [host] in 1 .. n_layers, n_layers <= 128.  Workspace: dflash_workspace_bytes
 * (cfg, batch, 0).  Device errors (token id, len + rows > kv_capacity) set
 * status bits as for the other calls. */
int dflash_target_forward(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                          int32_t batch, int32_t rows, const int32_t *tokens, int32_t *y, void *feat,
                          const int32_t *taps, int32_t n_taps, float *dbg_logits,
                          void *workspace, size_t workspace_bytes, void *stream);

/* len[b] += n[b] for b < batch (n device int32 [batch], e.g. dflash_verify's
 * accept_len); the capacity is cfg->kv_capacity, the one the cache was sized
 * with.  A count that is negative or would pass kv_capacity sets
 * DFLASH_STATUS_BAD_COUNT / DFLASH_STATUS_KV_OVERFLOW and leaves len[b].
 * 1 <= batch <= max_batch. */
int dflash_advance_len(const dflash_config *cfg, const dflash_kv *kv, int32_t batch, const int32_t *n,
                       void *stream);

/* Block size for the next cycle (summary section 4, ablations: a drafter trained
 * on 16-token blocks also drafts smaller ones at inference; picking the size per
 * cycle is this library's policy, not the summary's).  Host-only: [host] arrays,
 * no GPU work, usable while the previous cycle still runs.
 * Model: every draft position is accepted with the same probability p once the
 * ones before it were, so a cycle of block size g commits on average
 * E(g) = 1 + p + ... + p^(g-1) tokens.  p is estimated from recent cycles by
 * maximum likelihood with pseudo-counts: a cycle with accept length t and block
 * size g contributes t-1 accepted positions and, if t < g, one rejected one;
 *   p = (accepted + prior_weight * prior_p) / (accepted + rejected + prior_weight)
 * (prior_p when the denominator is 0).  The choice maximises E(g) / cost_us[g]
 * over gamma_min <= g <= gamma_max with cost_us[g] > 0 (ties: the smaller g).
 *   tau, gamma_used  [host] int32 [n]: 1 <= tau[i] <= gamma_used[i] <= 16, n >= 0
 *   cost_us          [host] float [gamma_max + 1]: time of one cycle at block size g
 *   2 <= gamma_min <= gamma_max <= 16; 0 <= prior_p <= 1; prior_weight >= 0
 *   gamma_out        [host] the choice; p_out [host, nullable] the estimate of p
 * Returns DFLASH_EINVAL for arguments out of range or no candidate with a cost. */
int dflash_choose_gamma(const int32_t *tau, const int32_t *gamma_used, int32_t n, const float *cost_us,
                        int32_t gamma_min, int32_t gamma_max, double prior_p, double prior_weight,
                        int32_t *gamma_out, double *p_out);

/* Input-fusion conditioning: the alternative that the summary's KV injection
 * is measured against (section 2.2, KV-injection bullet: features fused only at
 * the input layer are diluted with depth; section 4 ablations).  Cost
 * comparison only.  For every sequence b: c_i = W_fuse . concat(feat[b][i])
 * (as in dflash_inject_kv) is the drafter's input hidden state at position
 * len[b] + i, for i < rows_stride; every draft layer runs over these rows with
 * the drafter's recipe (input RMSNorm, q/k head RMSNorm + RoPE, attention to
 * the cached context and causally to the rows before it, W_o, SwiGLU MLP) and
 * keeps each row's k and v at its position in that layer's cache.  Then
 * len[b] += n_new[b]: rows at or past n_new[b] are computed but overwritten
 * later.  The cache must hold len[b] + rows_stride rows (else
 * DFLASH_STATUS_KV_OVERFLOW and nothing is written for b); n_new[b] outside
 * [0, rows_stride] sets DFLASH_STATUS_BAD_COUNT and leaves len[b].
 * dflash_draft_block then drafts from the cache as usual.
 *   feat     [batch][rows_stride][F][H] in the storage dtype
 *   n_new    device int32 [batch]
 * 1 <= rows_stride <= gamma_max; workspace: dflash_workspace_bytes(cfg, batch,
 * rows_stride). */
int dflash_inject_kv_input_fusion(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                                  int32_t batch, const void *feat, int32_t rows_stride, const int32_t *n_new,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Training objective of the drafter (summary section 2.3, loss weighting):
 * the drafter's forward pass exactly as dflash_draft_block (same anchor, mask
 * rows and context), then, for each mask row j = 1 .. gamma-1 of sequence b,
 * the cross-entropy CE[b][j] = logsumexp(logits) - logit[label] against
 * labels[b][j-1] (the target's token at block position j), weighted by block
 * position: w_j = exp(-(j - 1) / gamma), so early positions count most;
 *   loss[0] = sum_b sum_j w_j CE[b][j] / (batch * sum_j w_j).
 *   labels      int32 [batch][gamma-1], each in [0, vocab)
 *   loss        fp32 [1]
 *   row_loss    nullable fp32 [batch][gamma-1]: CE[b][j]
 *   dlogits     nullable fp32 [batch][gamma-1][V]: d loss / d logits =
 *               w_j / (batch * sum_j w_j) * (softmax(logits)[v] - [v == label]);
 *               when dbg_logits is NULL the logits are first written here and
 *               then replaced by the gradient
 *   dbg_logits  nullable fp32 [batch][gamma-1][V]: logits of the mask rows
 * The block's K/V are not written, len is not changed.  A label outside
 * [0, vocab) sets DFLASH_STATUS_BAD_TOKEN and makes its row's CE and loss NaN.
 * Sums run in fixed orders: the result is deterministic.  The gradient stops
 * at the logits (no backward pass through the drafter).  Workspace: dflash_workspace_bytes(cfg, batch, 0); argument
 * errors as for dflash_draft_block. */
int dflash_block_loss(const dflash_config *cfg, const dflash_weights *w, const dflash_kv *kv,
                      int32_t batch, int32_t gamma, const int32_t *anchor, const int32_t *labels,
                      float *loss, float *row_loss, float *dlogits, float *dbg_logits,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Host-only self-check of the launch plans (no GPU work, no device memory
 * touched, usable on a machine without a GPU).  Runs the launch sequences of
 * dflash_inject_kv (rows_stride rows per sequence), dflash_inject_kv_input_fusion
 * (min(rows_stride, gamma_max) rows), dflash_draft_block, dflash_block_loss
 * (with its gradient) and dflash_target_forward (one tap), each for `batch`
 * sequences and block size `gamma`, with stand-in pointers and without launching
 * anything.  For every launch it takes the byte range of each workspace buffer
 * that the kernel writes, computed from that launch's arguments and grid the way
 * the kernel indexes, and checks that the range lies inside the region of the
 * workspace layout (the one dflash_workspace_bytes() sizes) where it starts.
 *   launches, writes, violations  [host] out: launches audited, write ranges
 *                                 checked, ranges leaving their region (0 = all
 *                                 inside)
 * Returns DFLASH_OK, or the status the audited calls return for this shape. */
int dflash_audit_workspace(const dflash_config *cfg, int32_t batch, int32_t gamma, int32_t rows_stride,
                           int32_t *launches, int32_t *writes, int32_t *violations);

/* Human-readable name of a dflash_status value (static string). */
const char *dflash_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H_ */
