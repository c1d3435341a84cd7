/*
 * dflash.h -- C-ABI of the DFlash block-diffusion draft round on MI355X (gfx950).
 *
 * One draft round has four calls, in this order:
 *   dflash_fuse_taps      target tap planes -> fused context rows (fc, hidden_norm)
 *   dflash_inject_kv      fused rows -> k and v of every draft layer, written into a paged cache
 *   dflash_draft_block    one non-causal forward over anchor + (B-1) mask rows, LM-head argmax
 *   dflash_verify_greedy  longest prefix equal to the target's argmax, plus the bonus token
 *   dflash_sample_rows    inverse-CDF draws from tempered softmax rows
 *   dflash_verify_sampling speculative-sampling acceptance with the residual draw
 *
 * The round is the one described by TensorFold pull request #1851 ("What this
 * changes", items 1-4), the DFlash explainer (sections 3 and 4) and "Port the
 * DFlash2 protocol, not its checkpoint" ("What is portable").
 *
 * Conventions shared by every call:
 *   - Every call returns a dflash_status; on failure dflash_last_error() names the cause.
 *   - Arguments, shapes and capacities are checked on the host BEFORE anything is
 *     enqueued, so a refused call has no side effect on device memory.
 *   - All device memory (weights, caches, inputs, outputs, workspace) is owned by the
 *     caller; the library never allocates or frees device memory and never copies weights.
 *   - Calls are asynchronous on the given stream (a hipStream_t passed as void *;
 *     NULL is the null stream). A device fault surfaces on the caller's next sync.
 *   - A handle is used by one host thread at a time. Calls that share a workspace
 *     must be ordered on one stream.
 *   - Device pointers must be 16-byte aligned. Tensors are dense row-major.
 *   - Element type of every weight, activation and cache is the config's dtype
 *     (DFLASH_BF16: bfloat16 bit patterns; DFLASH_F32: IEEE float).
 *   - Token ids, positions, lengths and page ids are int32.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_LAYERS 64
#define DFLASH_MAX_TAPS 8

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_ARG = -1,        /* null / misaligned pointer, bad count */
  DFLASH_ERR_CONFIG = -2,     /* the config is refused (see dflash_create) */
  DFLASH_ERR_SHAPE = -3,      /* a weight's shape does not match the config */
  DFLASH_ERR_CAPACITY = -4,   /* a request past the cache span, the stream count or the workspace */
  DFLASH_ERR_STATE = -5,      /* weights not bound, or workspace not initialised */
  DFLASH_ERR_DEVICE = -6,     /* a HIP launch failed */
  DFLASH_ERR_UNIMPLEMENTED = -7
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/*
 * Drafter config (a DFlash v1 drafter: a plain qwen3 body, no conv, no selector).
 * TensorFold #1851 item 1: taps (up to eight), block, mask token and layer kinds
 * come from the config; a causal draft and taps past the target or repeated are
 * refused. Item 4: sliding layers attend their own window, the full layer all.
 *
 * dflash_create refuses (DFLASH_ERR_CONFIG) when any of these fails:
 *   dtype is DFLASH_F32 or DFLASH_BF16;
 *   1 <= n_layers <= 64; head_dim is 64 or 128; n_q_heads % n_kv_heads == 0;
 *   hidden, intermediate, n_q_heads*head_dim, n_kv_heads*head_dim are multiples of 128;
 *   hidden <= 16384 (bf16) or 8192 (f32);
 *   vocab >= 2; 1 <= n_taps <= 8; tap ids strictly ascending (so never repeated),
 *   each in [0, target_n_layers); 2 <= block_size <= 32; 0 <= mask_token_id < vocab;
 *   causal == 0; layer_window[l] >= 0 (0 = full attention) for l < n_layers;
 *   rope_theta > 0; rms_eps >= 0; max_streams >= 1; page_size == 16; pool_pages >= 1;
 *   pool_pages * n_kv_heads <= 2^31 - 1 (a (page, kv head) pair is indexed in 32 bits).
 */
typedef struct {
  int32_t dtype;
  int32_t hidden, n_layers, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  int32_t n_taps, tap_layer_ids[DFLASH_MAX_TAPS], target_n_layers;
  int32_t block_size, mask_token_id, causal;
  int32_t layer_window[DFLASH_MAX_LAYERS];
  float rope_theta, rms_eps;
  int32_t max_streams, page_size, pool_pages;
} dflash_config;

/*
 * Weight pointers (device). Shapes, [rows, cols] row-major:
 *   embed, lm_head [vocab, hidden]  (shared with the target, frozen)
 *   fc [hidden, n_taps*hidden]; hidden_norm, norm [hidden]
 *   per layer l: in_norm, post_norm [hidden]; wq [n_q*d, hidden]; wk, wv [n_kv*d, hidden];
 *   wo [hidden, n_q*d]; q_norm, k_norm [d]; w_gate, w_up [intermediate, hidden];
 *   w_down [hidden, intermediate].
 * That is 11 tensors a layer plus fc, hidden_norm and norm (TensorFold #1851, item 1).
 */
typedef struct {
  const void *embed, *lm_head, *fc, *hidden_norm, *norm;
  const void *in_norm[DFLASH_MAX_LAYERS], *wq[DFLASH_MAX_LAYERS], *wk[DFLASH_MAX_LAYERS],
      *wv[DFLASH_MAX_LAYERS], *wo[DFLASH_MAX_LAYERS], *q_norm[DFLASH_MAX_LAYERS],
      *k_norm[DFLASH_MAX_LAYERS], *post_norm[DFLASH_MAX_LAYERS], *w_gate[DFLASH_MAX_LAYERS],
      *w_up[DFLASH_MAX_LAYERS], *w_down[DFLASH_MAX_LAYERS];
} dflash_weights;

/*
 * Paged draft K/V cache (device), one K pool and one V pool per layer, each
 * [pool_pages, n_kv_heads, page_size, head_dim]. Stream s's position p lives in
 * page page_table[s * pages_per_stream + p / page_size], slot p % page_size.
 * Every layer's cache holds the whole served span; a sliding layer only reads
 * its window of it (TensorFold #1851, item 4). page_table is device int32
 * [max_streams, pages_per_stream]; entries outside [0, pool_pages) are never
 * dereferenced (such keys are skipped on read and on write).
 */
typedef struct {
  void *k_pool[DFLASH_MAX_LAYERS], *v_pool[DFLASH_MAX_LAYERS];
  const int32_t *page_table;
  int32_t pages_per_stream;
} dflash_kv;

typedef struct dflash dflash;

/* Fill a config with the defaults: rope_theta 1e6, rms_eps 1e-6, page_size 16, causal 0,
 * all layers full attention; shape fields zero. */
void dflash_config_init(dflash_config *cfg);

/* Validate a config and create a handle. No device work. On DFLASH_ERR_CONFIG *out is
 * NULL and dflash_last_error(NULL) names the failed check. */
int dflash_create(const dflash_config *cfg, dflash **out);

/* Number of drafter tensors, 11 * n_layers + 3 (TensorFold #1851, item 1: 69 names at 6 layers). */
int32_t dflash_tensor_count(const dflash_config *cfg);

/*
 * Bind weights by pointer. `shapes` holds 2 int64 per tensor in this order:
 * embed, lm_head, fc, hidden_norm, norm, then for each layer in_norm, wq, wk, wv, wo,
 * q_norm, k_norm, post_norm, w_gate, w_up, w_down; a vector's shape is (n, 1).
 * Every pointer must be non-null and 16-byte aligned and every shape must match the
 * config, or the whole bind is refused (DFLASH_ERR_SHAPE / DFLASH_ERR_ARG) and any
 * previous binding is left as it was: there is no partial bind ("Port the DFlash2
 * protocol, not its checkpoint", "The public configs prove target binding").
 */
int dflash_bind_weights(dflash *h, const dflash_weights *w, const int64_t *shapes);

/* Bytes of one fused context row: hidden * element size (8 KiB at hidden 4096 bf16;
 * TensorFold #1851, item 4). */
int64_t dflash_fused_row_bytes(const dflash_config *cfg);

/* Planner price of a prompt row's taps (TensorFold #1851, item 3): with fusing != 0,
 * (2 * n_taps + 2) * hidden * element size (planes, their row-major copy, fc's output
 * row, the fused row: 18 x hidden x 2 bytes for eight bf16 taps); with fusing == 0 the
 * raw planes only, n_taps * hidden * element size. Returns -1 for a null config. */
int64_t dflash_tap_row_bytes(const dflash_config *cfg, int32_t fusing);

/*
 * The skinny GEMMs' weights in their packed layout. dflash_pack_weights copies the
 * bound fc, LM head and every layer's [wq | wk | wv], wo, [w_gate | w_up] and w_down
 * into `buf` (caller-owned device memory of at least dflash_packed_weight_bytes bytes,
 * 256-byte aligned; else DFLASH_ERR_ARG / DFLASH_ERR_CAPACITY), on `stream`. In the
 * packed layout the 32 output columns a workgroup computes are K / KI consecutive
 * chunks of 32 rows x 128 bytes, so each workgroup streams one contiguous region of
 * HBM instead of 32 rows 2 K bytes apart; inside a chunk the 16-byte pieces stand in
 * the order the MFMAs take them (four 1 KB fragments; fragment 2 nt + u holds, at
 * 16 l, piece 2 (l / 16) + u of row 16 nt + l % 16), so each wave load is 1 KB
 * contiguous. The values are the bound weights' own. Every
 * GEMM then reads the packed copy; the bound embedding and norm gains stay in use (and
 * the bound pointers stay the source of any later packing). Required once after
 * dflash_bind_weights, before the first fuse,
 * inject or draft (else DFLASH_ERR_STATE); binding again drops the packing. The buffer
 * must outlive its use; the library never frees it.
 */
size_t dflash_packed_weight_bytes(const dflash *h);
int dflash_pack_weights(dflash *h, void *buf, size_t bytes, void *stream);

/*
 * 4-bit drafter weights (DFlash explainer, section 8: the drafter quantized at load with
 * 4 bits in groups of 64; TensorFold #1851, "Exactness", Precision: the drafter's 4-bit
 * copies beside bf16 activations and fp32 sums). dflash_pack_weights_q4 quantizes the
 * same GEMM weights as dflash_pack_weights into `buf` (dflash_q4_weight_bytes bytes,
 * 0 for an fp32 config): each run of 64 weights along a row becomes 64 4-bit codes
 * and a bf16 (scale, bias), bias = the run's minimum, scale = (max - min) / 15 rounded
 * once to bf16, code = (w - bias) / scale rounded to nearest even and clamped to
 * [0, 15], all decided in float64. The GEMMs then compute with bias + scale * code
 * exactly: sum_k x_k (bias + scale q_k) = scale * sum x q + bias * sum x per group.
 * The embedding and the norm gains stay bf16. The 4-bit path runs the skinny GEMMs only:
 * fuse and inject calls of more than 32 rows and drafts of more than 32 block rows are
 * refused (DFLASH_ERR_UNIMPLEMENTED). Packing again (either kind) replaces it; binding
 * again drops it. Errors otherwise as dflash_pack_weights.
 */
size_t dflash_q4_weight_bytes(const dflash *h);
int dflash_pack_weights_q4(dflash *h, void *buf, size_t bytes, void *stream);

/*
 * Workspace bytes for calls with at most `max_rows` fused/injected rows, `n_streams`
 * streams in a draft, and context length at most `max_ctx`. The workspace holds split-K
 * partials, block activations and attention partials, each written before it is read
 * within a call, so no part of it must start at zero.
 * Returns 0 if the arguments are out of range.
 */
size_t dflash_workspace_bytes(const dflash *h, int32_t max_rows, int32_t n_streams, int32_t max_ctx);

/* Register a workspace buffer (`ws_bytes` > 0, 16-byte aligned) with the handle;
 * nothing is enqueued on `stream`. Required once for every workspace buffer before its
 * first use on a handle, and again if it grows: calls given a workspace that was not
 * registered, or more bytes than were, are refused (DFLASH_ERR_STATE), which catches a
 * buffer passed in by mistake. */
int dflash_workspace_init(dflash *h, void *ws, size_t ws_bytes, void *stream);

/*
 * Fuse: for each of n_rows rows r, x = [T_0[r] | T_1[r] | ... | T_{n-1}[r]] (planes in
 * ascending tap-id order), y = fc . x (fp32 sums), fused[r] = y / sqrt(mean(y^2) + eps)
 * * hidden_norm, stored in the dtype (TensorFold #1851, items 3 and 4: the taps pass runs
 * fc and hidden_norm once a row's planes are complete).
 *   tap_planes: host array of n_taps device pointers; plane t is [n_rows, hidden] with
 *               a row stride of plane_row_stride elements (>= hidden, <= 2^27, multiple
 *               of 8; else DFLASH_ERR_ARG).
 *   fused_out:  device [n_rows, hidden].
 * n_rows == 0 is a no-op. A workspace sized for fewer rows -> DFLASH_ERR_CAPACITY. Calls
 * of more than 8192 rows (prompt scale) run as equal passes of at most 8192 rows, so the
 * workspace needed stops growing there; a row's result is the same bits in any call of
 * 33 rows or more.
 */
int dflash_fuse_taps(dflash *h, const void *const *tap_planes, int64_t plane_row_stride,
                     int32_t n_rows, void *fused_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Inject: for each fused row r (device [n_rows, hidden]) of stream row_stream[r] at
 * position row_pos[r], and for each layer l:
 *   K_l = RoPE_pos(k_norm_l(wk_l . f)) per kv head,  V_l = wv_l . f,
 * written into the layer's paged pools (k and v only; no q, no MLP, no input norm:
 * TensorFold #1851 item 4; DFlash explainer section 3, KV injection into every layer).
 * row_stream / row_pos are device int32 [n_rows]; rows with a stream outside
 * [0, max_streams), a position outside [0, pages_per_stream * page_size) or an invalid
 * page are skipped. n_rows == 0 is a no-op. Like dflash_fuse_taps, calls of more than
 * 8192 rows run in equal passes of at most 8192 rows.
 */
int dflash_inject_kv(dflash *h, const void *fused, int32_t n_rows, const int32_t *row_stream,
                     const int32_t *row_pos, const dflash_kv *kv, void *ws, size_t ws_bytes,
                     void *stream);

/*
 * Inject for the layers in layer_mask only (bit l = layer l; a bit at or past n_layers
 * -> DFLASH_ERR_ARG; an empty mask is a no-op): the prompt-side inject limited to the
 * layers that will read a row (TensorFold #1851, cold prefill with the drafter attached:
 * doing that work only for rows the drafter reads is the follow-up it names). A
 * selected layer's K/V are bitwise those dflash_inject_kv writes; the other layers'
 * pool slots are not touched. Arguments and errors otherwise as dflash_inject_kv.
 */
int dflash_inject_kv_layers(dflash *h, const void *fused, int32_t n_rows, const int32_t *row_stream,
                            const int32_t *row_pos, const dflash_kv *kv, uint64_t layer_mask, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * The layers that read context position pos in a round at context length ctx_len:
 * layer l when max(0, ctx_len - W_l) <= pos < ctx_len (W_l = layer_window[l]; every
 * position below ctx_len when W_l == 0), as in dflash_draft_block. A stream's committed
 * context never shrinks below its prompt, so with ctx_len = the prompt length this is
 * every layer that will ever read a prompt row at pos: the mask for
 * dflash_inject_kv_layers. 0 when pos is outside [0, ctx_len) or h is NULL. Host only.
 */
uint64_t dflash_layers_reading(const dflash *h, int32_t pos, int32_t ctx_len);

/*
 * Draft one block per stream. Stream s's block is [anchor[s], mask x (B-1)] at
 * positions C_s .. C_s+B-1 with C_s = ctx_len[s]; one non-causal forward of the qwen3
 * body (two residual adds a layer); layer l attends the context positions
 * [max(0, C_s - W_l), C_s) (all of [0, C_s) when W_l == 0) plus all B block rows.
 * After the final norm the shared LM head scores each mask row, and
 * draft_out[s, j-1] = argmax (lowest index on a tie) of mask row j, j = 1..B-1
 * (TensorFold #1851 items 1 and 4; DFlash explainer section 3 and section 5: top-1
 * at each position independently).
 *   anchor, ctx_len: device int32 [n_streams]; ctx_len[s] must be <= max_ctx_len
 *                    (larger values are clamped to it); anchor ids are clamped to
 *                    [0, vocab).
 *   max_ctx_len:     host bound used to size the launch; must satisfy
 *                    max_ctx_len <= kv->pages_per_stream * page_size (else
 *                    DFLASH_ERR_CAPACITY).
 *   draft_out:       device int32 [n_streams, B-1].
 *   logits_out:      NULL, or device float [n_streams, B-1, vocab] (fp32 logits).
 *   top2_out:        NULL, or device float [n_streams, B-1, 2] (largest and second
 *                    largest logit, fp32).
 * The block's own K/V are never written to the cache: only committed rows are, by
 * the next round's dflash_inject_kv, so rollback is rewinding ctx_len.
 */
int dflash_draft_block(dflash *h, int32_t n_streams, const int32_t *anchor,
                       const int32_t *ctx_len, int32_t max_ctx_len, const dflash_kv *kv,
                       int32_t *draft_out, void *logits_out, float *top2_out, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * dflash_draft_block for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The same
 * computation and kernels, bit for bit, with the workspace taken from a file-scope
 * device array of 32 MiB that each device holds from the library's load until the
 * process ends; the call itself calls no hipMalloc, hipFree or allocating routine,
 * creates no events (profiling is suspended inside it) and needs no
 * dflash_workspace_init. Its device address is looked up once per device, on the first
 * call with that device current. A draft whose workspace would exceed the array (more
 * than 32 MiB: dflash_workspace_bytes(h, 0, n_streams, max_ctx_len) tells; one stream
 * at the 9B shapes needs about 16 MiB) is refused with DFLASH_ERR_CAPACITY before
 * anything is enqueued. Nothing in the array must start at zero. Every call on one
 * device shares that device's array: calls that overlap on one device (other streams,
 * other threads, other handles) race and must be serialised by the caller. Arguments,
 * outputs and other errors as dflash_draft_block.
 */
int dflash_draft_block_noalloc(dflash *h, int32_t n_streams, const int32_t *anchor,
                               const int32_t *ctx_len, int32_t max_ctx_len, const dflash_kv *kv,
                               int32_t *draft_out, void *logits_out, float *top2_out, void *stream);

/*
 * Greedy verify (DFlash explainer section 4, greedy decoding; "Port the DFlash2
 * protocol", golden replay items 4-5). For each stream, with draft d_1..d_{B-1}
 * (device int32 [n_streams, B-1]) and target argmax t_0..t_{B-1} (device int32
 * [n_streams, B]):
 *   accept_len[s] = largest a <= B-1 with d_j == t_{j-1} for all j <= a;
 *   bonus[s]      = t_a;
 *   committed[s]  = d_1..d_a, t_a, then -1 up to B entries  (device int32 [n_streams, B]);
 *   ctx_len_inout[s] += a + 1 when ctx_len_inout is not NULL.
 * Works without bound weights (it touches no weight).
 */
int dflash_verify_greedy(dflash *h, int32_t n_streams, const int32_t *draft,
                         const int32_t *target_argmax, int32_t *accept_len, int32_t *bonus,
                         int32_t *committed, int32_t *ctx_len_inout, void *stream);

/*
 * Sampling (DFlash explainer section 4, "Sampling decoding"). Draws from tempered
 * softmax rows: token_out[r] is drawn from softmax(logits[r, :vocab] / temperature)
 * by inverse CDF over token ids in ascending order with the caller's uniform u[r] in
 * [0, 1): the smallest id whose running probability exceeds u[r]; an id of zero
 * probability is never drawn.
 *   logits:    device float [n_rows, row_stride] (row_stride >= vocab), e.g. the
 *              logits_out of dflash_draft_block;
 *   u:         device float [n_rows];
 *   token_out: device int32 [n_rows];
 *   prob_out:  NULL, or device float [n_rows]: the drawn token's probability.
 *   ws:        a workspace initialised with dflash_workspace_init whose
 *              dflash_workspace_bytes covered n_rows (max_rows, or n_streams * block_size,
 *              at least n_rows); it holds each row's per-slice max and weight sum.
 * temperature must be positive and finite; vocab at most 262144 (DFLASH_ERR_CONFIG
 * otherwise). n_rows == 0 is a no-op. Probabilities are fp32 exponentials summed in
 * float64. Works without bound weights.
 */
int dflash_sample_rows(dflash *h, int32_t n_rows, const float *logits, int64_t row_stride,
                       float temperature, const float *u, int32_t *token_out, float *prob_out,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Speculative-sampling verify (DFlash explainer section 4, "Sampling decoding": the
 * standard acceptance rule and the residual max(p_target - p_draft, 0)). Per stream,
 * with draft d_1..d_{B-1} (device int32 [n_streams, B-1]) drawn from the draft's
 * tempered distributions p_j = softmax(draft_logits[s, j-1] / T) (device float
 * [n_streams, B-1, row_stride]) and the target's q_i = softmax(target_logits[s, i] / T)
 * (device float [n_streams, B, row_stride]; row i: the token after the anchor and
 * d_1..d_i):
 *   d_j is accepted, for j = 1, 2, ..., while u_accept[s, j-1] * p_j(d_j) < q_{j-1}(d_j)
 *   (an id outside [0, vocab) is rejected);
 *   accept_len[s] = a, the number accepted;
 *   token[s] = a draw with u_sample[s] (inverse CDF, as dflash_sample_rows) from the
 *   residual max(q_a - p_{a+1}, 0) renormalised (q_a when the residual has no mass)
 *   if a < B-1, else from q_{B-1};
 *   committed[s] = d_1..d_a, token[s], then -1 up to B entries (device int32 [n_streams, B]);
 *   ctx_len_inout[s] += a + 1 when ctx_len_inout is not NULL.
 * u_accept: device float [n_streams, B-1]; u_sample: device float [n_streams]; all
 * uniforms in [0, 1). ws: a workspace initialised with dflash_workspace_init for at
 * least n_streams streams (it holds every row's per-slice max and weight sum and the
 * draw's per-slice sums). temperature must
 * be positive and finite; vocab at most 262144. Works without bound weights.
 */
int dflash_verify_sampling(dflash *h, int32_t n_streams, const int32_t *draft,
                           const float *draft_logits, const float *target_logits,
                           int64_t row_stride, float temperature, const float *u_accept,
                           const float *u_sample, int32_t *accept_len, int32_t *token,
                           int32_t *committed, int32_t *ctx_len_inout, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * DFlash2 candidate path selector (DFlash explainer, section 5: keep the top-k
 * candidates of every drafted position, score adjacent candidate pairs with a light
 * selector, pick one consistent path; DFlash2's config: top-k 16, rank 256; TensorFold
 * #1851 item 1: with no codebooks, rank 0, the pair term is zero and the path comes from
 * each position's marginals; Strata #3457, "Problem and result": a draft stops where
 * the selector's confidence falls below min-p).
 *   logits:   device fp32 [n_streams, B-1] rows of `row_stride` floats (>= vocab), e.g.
 *             dflash_draft_block's logits_out.
 *   code_u, code_w: device bf16 [vocab, rank] token codebooks; the pair score of token a
 *             at position j and token b at j+1 is <code_u[a], code_w[b]>, summed in
 *             float64. rank 0: no pair term (both may be NULL).
 *   top_k:    1..16 candidates a position: the largest logits, ties to the lowest id;
 *             node score log softmax(logits_j)(token), the partition sum in float64.
 *   The path maximises the sum of node and pair scores over the candidates (a tie goes
 *   to the earlier candidate, choosing the last position first and walking back).
 *   min_p:    the draft stops before the first position whose chosen token's
 *             probability is below min_p (0 keeps every position).
 *   draft_out: device int32 [n_streams, B-1]: the path's tokens, -1 past the stop (so
 *             dflash_verify_greedy accepts at most the draft length).
 *   draft_len: device int32 [n_streams].
 * ws as for a draft of n_streams streams (dflash_workspace_bytes). Errors: bad counts
 * or pointers -> DFLASH_ERR_ARG; workspace -> DFLASH_ERR_STATE / DFLASH_ERR_CAPACITY.
 * Works without bound weights.
 */
int dflash_select_path(dflash *h, int32_t n_streams, const float *logits, int64_t row_stride,
                       const void *code_u, const void *code_w, int32_t rank, int32_t top_k,
                       float min_p, int32_t *draft_out, int32_t *draft_len, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * Instrumentation (not part of the round). With profiling enabled, every kernel the
 * handle launches is bracketed by two hipEvents on its stream; dflash_profile_read
 * waits for the recorded events and writes one line per kernel name,
 * "<name> <launches> <total_ms>\n", into buf (NUL-terminated, truncated to len), then
 * clears the record. Returns the number of bytes written, or a negative status.
 */
int dflash_set_profiling(dflash *h, int32_t enable);
int dflash_profile_read(dflash *h, char *buf, size_t len);

/*
 * Stage trace (instrumentation for parity tests; not part of the round). With a trace
 * buffer set, dflash_draft_block also copies every tensor it stores into the buffer,
 * on its stream, so each step can be checked on exactly the inputs it read. Layout, in
 * elements of the activation dtype, with M = n_streams * B, Mm = n_streams * (B - 1):
 * for each layer l, one record of
 *   x_in [M, hidden]          the layer's input residual stream (the embedding rows
 *                             for layer 0; after residual add 2 of layer l - 1)
 *   a [M, hidden]             round(RMSNorm(x_in) * in_norm)
 *   q [M, n_q * d]            normalised, rotated queries
 *   k [n_streams, n_kv, 32, d]    block keys (rows >= B unused)
 *   v [n_streams, n_kv, d, 32]    block values, transposed (columns >= B unused)
 *   o [M, n_q * d]            attention output
 *   x_attn [M, hidden]        after residual add 1
 *   b [M, hidden]             round(RMSNorm(x_attn) * post_norm)
 *   m [M, intermediate]       SwiGLU product
 * then x_last [M, hidden] (after the last layer's add 2; only the mask rows are
 * updated) and z [Mm, hidden] (the final-normed mask rows, stream-major).
 * dflash_trace_bytes gives the size for n_streams (0 when out of range). A draft whose
 * trace would not fit the buffer is refused (DFLASH_ERR_CAPACITY). buf == NULL or
 * bytes == 0 turns the trace off. The buffer is caller-owned device memory.
 */
size_t dflash_trace_bytes(const dflash *h, int32_t n_streams);
int dflash_set_trace(dflash *h, void *buf, size_t bytes);

/* The last error message of a handle (or of dflash_create when h is NULL). Never NULL. */
const char *dflash_last_error(const dflash *h);

/* Destroy a handle (host memory only). NULL is allowed. */
void dflash_destroy(dflash *h);

/* Library version string. */
const char *dflash_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
