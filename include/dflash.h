/*
 * dflash.h — C ABI of the DFlash drafting hot path on AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages about DFlash, cited by page and section):
 *
 *   [guide]  "DFlash：块扩散加速的 LLM 推测解码技术" (txtmix.com DFlash guide)
 *   [news]   "DFlash 2 发布：并行草稿继续压低大模型推理延迟" (openai-hub.com)
 *   [repo]   llmapis.com post on the DFlash repository
 *
 * One speculative cycle maps onto three calls ([guide] section 4):
 *
 *   dflash_inject_context  target features of new positions -> draft KV cache
 *                          ([guide] section 3.2)
 *   dflash_draft_block     one forward of the block-diffusion draft over B mask
 *                          positions -> B greedy draft tokens ([guide] 3.1, 3.2)
 *   dflash_verify_accept   longest draft prefix matching the target's greedy
 *                          tokens ([news] "DFlash 2 的核心：一次写一块")
 *
 * plus the host-side feature-layer rule dflash_feature_layers ([guide] 3.2).
 *
 * Memory: the caller allocates every device buffer (weights, KV pool,
 * workspace, inputs, outputs); the library borrows weights, the KV pool and
 * the workspace for the handle's lifetime and everything else for the call.
 * Library calls never allocate device memory.  The handle itself is host
 * memory holding the configuration, the borrowed pointers and a host mirror
 * of each request slot's lengths and pages.
 *
 * Execution: every compute call validates its arguments on the host, then
 * enqueues kernels on the given stream (a hipStream_t; NULL = the default
 * stream) and returns without synchronising.  Outputs are valid once the
 * stream has reached the enqueued work.  Calls on one handle must not run
 * concurrently; distinct handles are independent.
 *
 * Errors: a nonzero status means nothing was enqueued and no state changed,
 * except DFLASH_E_HIP, which reports a failure of the HIP runtime itself
 * (after which the handle's device state is undefined).  dflash_last_error()
 * returns a thread-local message for the last failing call.  Token ids read
 * from device memory that fall outside [0, vocab) are clamped and recorded
 * in a sticky device error word that dflash_check reports.
 *
 * Data types: DFLASH_BF16 stores weights, hidden states, the KV cache and
 * activations in bfloat16 and accumulates in fp32; DFLASH_F32 stores them in
 * fp32.  Norms, softmax, the residual stream and logits are fp32 in both.
 *
 * Weight layout: every matrix is row-major [out_features, in_features]
 * (torch.nn.Linear layout).  Vectors are [hidden].
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 4
#define DFLASH_MAX_LAYERS 64
#define DFLASH_MAX_FEAT 8
#define DFLASH_MAX_BATCH 256
#define DFLASH_PAGE_SIZE 16
#define DFLASH_MAX_TOPK 16

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = 1,     /* bad argument or configuration */
  DFLASH_E_CAPACITY = 2,    /* an inject would exceed the slot's bound pages */
  DFLASH_E_UNSUPPORTED = 3, /* valid but not implemented for this shape */
  DFLASH_E_HIP = 4,         /* the HIP runtime reported an error */
  DFLASH_E_DEVICE = 5       /* sticky device error word was set */
} dflash_status;

typedef enum { DFLASH_BF16 = 0, DFLASH_F32 = 1 } dflash_dtype;

/* Shapes of one draft model and the capacity of one handle.
 * Requirements (checked by dflash_validate_config):
 *   hidden, ffn, n_q_heads*head_dim and n_feat*hidden multiples of 256;
 *   head_dim 64 or 128; n_q_heads a multiple of n_kv_heads with
 *   n_q_heads/n_kv_heads <= 8; 1 <= block_size <= 16; page_size == 16;
 *   1 <= n_layers <= DFLASH_MAX_LAYERS; 1 <= n_feat <= DFLASH_MAX_FEAT;
 *   0 <= mask_token_id < vocab; window 0 (unbounded) or a positive multiple
 *   of 16; topk 0 or 16; max_batch <= DFLASH_MAX_BATCH; selector_rank 0,
 *   or a multiple of 64 up to 512 with topk 16.  A target handle (target 1)
 *   takes 1 <= block_size <= 64 rows per request and no window, conv, top-16
 *   or selector; its fc and fc_norm may be NULL. */
typedef struct dflash_config {
  int32_t hidden;            /* d */
  int32_t n_q_heads;         /* Hq */
  int32_t n_kv_heads;        /* Hkv (grouped-query attention) */
  int32_t head_dim;          /* dh */
  int32_t ffn;               /* F, SwiGLU width */
  int32_t vocab;             /* V, shared LM head rows */
  int32_t n_layers;          /* L draft layers ([guide] 3.1: 5, or 8) */
  int32_t block_size;        /* B mask positions per draft ([guide] 3.1: 16, or 10) */
  int32_t n_feat;            /* K target layers concatenated ([guide] 3.2: 5) */
  int32_t dtype;             /* dflash_dtype */
  int32_t mask_token_id;     /* embedding row used for every block position */
  int32_t page_size;         /* KV page, must be 16 tokens */
  int32_t window;            /* draft sliding window in tokens ([repo]); 0 = none */
  int32_t conv2;             /* 1 = DFlash-2 two-tap conv ([guide] 7) */
  int32_t topk;              /* 0, or 16 = keep top-16 per position ([guide] 7) */
  int32_t max_batch;         /* request slots */
  int32_t max_pages;         /* pages in the KV pool (per layer) */
  int32_t max_pages_per_req; /* page-table width per slot, <= 4095 */
  int32_t max_position;      /* positions < max_position (RoPE table rows) */
  int32_t max_inject_rows;   /* rows per internal inject chunk (workspace size) */
  float rms_eps;             /* RMSNorm epsilon */
  float rope_theta;          /* RoPE base */
  int32_t selector_rank;     /* DFlash-2 path selector rank r ([guide] 7); 0 = none */
  int32_t target;            /* 1 = the handle is a target model (dflash_target_forward):
                                causal attention over its own KV cache, token inputs;
                                block_size is then the rows per request of one call */
  int32_t weight_bits;       /* 16 = the draft's matrices in the storage dtype; 4 = a 4-bit
                                draft ([guide] 8: --draft-bits 4): W_fc and every layer's
                                W_qkv, W_o, W_gate/up, W_down quantised by dflash_create,
                                per output row and group of 64 inputs, to codes q in 0..15
                                with scale s = bf16((max - min) / 15) and bias b = min
                                (q = round_half_even((w - b) / s) in fp32, 0 when s = 0);
                                the draft computes with s * q + b.  bf16 drafts only; the
                                shared embedding and LM head stay bf16 */
  int32_t conv_rank;         /* conv2 only: 0 = static conv taps; r in {32, 64} = dynamic
                                taps ([guide] 7): per row, the static taps plus U D x, x that row
                                of the conv's input, D [r, d], U [2d, r] per conv point
                                (storage-dtype weights only) */
} dflash_config;

/* Per-layer weights (device pointers, dtype of the config).
 *   wqkv      [(Hq + 2*Hkv)*dh, d]  rows: q heads, then k heads, then v heads
 *   wo        [d, Hq*dh]
 *   wgateup   [2*F, d]              rows: gate, then up
 *   wdown     [d, F]
 *   attn_norm [d], mlp_norm [d]     RMSNorm gains
 *   conv      [4][2][d] two-tap conv taps (w0, w1) at the four conv points, or
 *             NULL when conv2 == 0
 *   dconv_d   [4][r][d] dynamic taps: the rank-r projection of the conv input
 *             at each point (before attention, after it, before the MLP, after
 *             it), or NULL when conv_rank == 0
 *   dconv_u   [4][2d][r] dynamic taps: rows 0..d-1 add to w0, rows d..2d-1 to w1 */
typedef struct dflash_layer_weights {
  const void *wqkv, *wo, *wgateup, *wdown, *attn_norm, *mlp_norm, *conv;
  const void *dconv_d, *dconv_u;
} dflash_layer_weights;

/* Model weights (device pointers).
 *   embed [V, d] and lm_head [V, d] are the target's, shared by the draft
 *   ([guide] 3.1); fc [d, n_feat*d] and fc_norm [d] form the context
 *   projection ([guide] 3.2); final_norm [d] is the draft's last RMSNorm.
 *   sel_u, sel_v [r, d]: the path selector's low-rank bilinear form
 *   s(a, b) = (sel_u E[a]) . (sel_v E[b]) over shared-embedding rows
 *   ([guide] 7), NULL when selector_rank == 0. */
typedef struct dflash_weights {
  const void *embed, *lm_head, *fc, *fc_norm, *final_norm;
  dflash_layer_weights layers[DFLASH_MAX_LAYERS];
  const void *sel_u, *sel_v;
} dflash_weights;

typedef struct dflash_handle dflash_handle;

/* ABI version of the loaded library (DFLASH_ABI_VERSION). */
int32_t dflash_abi_version(void);

/* Thread-local message of the last failing call ("" if none). */
const char *dflash_last_error(void);

/* Checks a configuration; DFLASH_OK or DFLASH_E_INVALID. Host only. */
dflash_status dflash_validate_config(const dflash_config *cfg);

/* Feature-layer rule ([guide] 3.2): the k 0-based target layers, spaced
 * evenly with integer floor over [1, n_target_layers-3] (layer 2 to the
 * third-from-last in 1-based numbering), written to out[0..k).  Needs
 * k >= 2 and n_target_layers >= 4.  Host only. */
dflash_status dflash_feature_layers(int32_t n_target_layers, int32_t k, int32_t *out);

/* Bytes of device workspace / KV pool / packed weights a handle with this
 * config needs (0 for an invalid config).  The KV pool is n_layers *
 * max_pages pages of 2 * n_kv_heads * 16 * head_dim elements; the caller may
 * hand out pages to slots in any order.  The packed-weights buffer receives a
 * copy of every weight matrix in the library's streaming layout (MFMA
 * fragment order: 16-row tiles, 32-column steps, 64 lanes x 8 elements). */
size_t dflash_workspace_bytes(const dflash_config *cfg);
size_t dflash_kv_pool_bytes(const dflash_config *cfg);
size_t dflash_packed_weights_bytes(const dflash_config *cfg);

/* Creates a handle borrowing weights, kv_pool, workspace and packed (device
 * buffers of at least the sizes above, 256-byte aligned).  Device
 * initialisation happens on the first call that needs the device (normally
 * dflash_bind_request), on the current HIP device: the RoPE table, the slot
 * state, and the packing of every weight matrix of `w` into `packed`.  The
 * matrices of `w` are read only then; embed, the norm gains and the conv taps
 * are read by every draft.  Returns DFLASH_E_INVALID on a bad config or a
 * NULL pointer, DFLASH_E_UNSUPPORTED for a hidden size above 4096 (bf16) /
 * 2048 (fp32). */
dflash_status dflash_create(const dflash_config *cfg, const dflash_weights *w,
                            void *kv_pool, void *workspace, void *packed,
                            dflash_handle **out);

/* Releases the host handle (borrowed device memory is untouched). */
void dflash_destroy(dflash_handle *h);

/* Binds request slot `slot` to KV pages page_ids[0..n_pages) (host array of
 * pool page indices, each < max_pages, n_pages <= max_pages_per_req) and
 * resets its lengths: the next inject writes position `start_pos`, positions
 * below it are never visible.  With a window W the pages form a ring that
 * needs n_pages >= W/16 + 1; without one, positions below
 * 16*n_pages fit.  Synchronous (uploads the page table). */
dflash_status dflash_bind_request(dflash_handle *h, int32_t slot, const int32_t *page_ids,
                                  int32_t n_pages, int32_t start_pos);

/* Host mirror of a slot's committed context length (positions injected). */
int32_t dflash_context_length(const dflash_handle *h, int32_t slot);

/* Steps 1 and 2 ([guide] 3.2): for each of the n_req requests, the target
 * hidden states of n_new[i] new positions ctx_len .. ctx_len+n_new[i]-1 are
 * concatenated over the n_feat layers, projected by fc, RMSNormed by fc_norm
 * and written through every draft layer's K/V projection (K with RoPE at the
 * absolute position) into the slot's KV pages.
 *   slots   host [n_req] distinct bound slots
 *   n_new   host [n_req] >= 0 rows per request
 *   hidden  host array of n_feat device pointers, each [sum(n_new), d] in the
 *           config dtype, rows grouped by request in call order, feature
 *           layers in ascending target-layer order
 *   debug_f optional device [sum(n_new), d] (config dtype): the projected,
 *           normalised context feature; NULL in timed runs
 * DFLASH_E_CAPACITY if a slot without window would run past its pages or
 * past max_position. */
dflash_status dflash_inject_context(dflash_handle *h, void *stream, int32_t n_req,
                                    const int32_t *slots, const int32_t *n_new,
                                    const void *const *hidden, void *debug_f);

/* Optional validation outputs and inputs of dflash_draft_block (device
 * buffers; any field may be NULL):
 *   logits     [n_req, B, V] fp32 logits of every block position
 *   hidden     [L+1, n_req*B, d] fp32 residual stream entering layer 0..L-1
 *              and leaving the last layer
 *   hidden_in  [L+1, n_req*B, d] fp32 teacher forcing: the residual stream
 *              entering layer l (and the final norm, l = L) is replaced by
 *              hidden_in[l], so every layer and the head can be checked on
 *              given inputs.  The same kernels run; only their input changes. */
typedef struct dflash_draft_debug {
  float *logits;
  float *hidden;
  const float *hidden_in;
} dflash_draft_debug;

/* Steps 3 and 4 ([guide] 3.1, 3.2, 7): one forward of the draft over B mask
 * positions n .. n+B-1 (n = ctx_len + 1) of each request: pre-norm layers with
 * bidirectional attention over the visible context KV and the block, GQA,
 * SwiGLU; the draft's final RMSNorm; the shared LM head; greedy argmax with
 * ties to the lowest id.
 *   slots        host [n_req] distinct bound slots
 *   last_token   device [n_req] int32 last verified token (conv2 only, else
 *                may be NULL): the block start of the two-tap conv reads its
 *                embedding
 *   draft        device [n_req, B] int32 output
 *   topk_ids     device [n_req, B, 16] int32, topk_logits [n_req, B, 16] fp32:
 *                top-16 by logit descending then id ascending (topk == 16),
 *                else NULL
 *   debug        optional validation buffers (NULL in timed runs) */
dflash_status dflash_draft_block(dflash_handle *h, void *stream, int32_t n_req,
                                 const int32_t *slots, const int32_t *last_token,
                                 int32_t *draft, int32_t *topk_ids, float *topk_logits,
                                 const dflash_draft_debug *debug);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * draft as dflash_draft_block, same arguments, outputs and kernels, with its
 * scratch (residual stream, GEMM inputs, split-K partial planes, attention
 * split partials, selection keys and lists) taken from a static device array
 * of DFLASH_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU
 * it runs on until the process ends, instead of the handle's workspace.  The
 * handle's workspace still holds the request state.  Allocates nothing.
 * Every call on a GPU, from any handle, uses that GPU's one array and leaves
 * its contents behind; calls that overlap on one GPU (two streams, two
 * threads) race and must be serialised by the caller.  Returns
 * DFLASH_E_CAPACITY when n_req requests need more scratch than the array
 * holds (dflash_draft_static_bytes tells), else as dflash_draft_block. */
#define DFLASH_STATIC_SCRATCH_BYTES (64u << 20)
dflash_status dflash_draft_block_static(dflash_handle *h, void *stream, int32_t n_req,
                                        const int32_t *slots, const int32_t *last_token,
                                        int32_t *draft, int32_t *topk_ids, float *topk_logits,
                                        const dflash_draft_debug *debug);

/* Scratch bytes dflash_draft_block_static needs for a call of n_req requests
 * with this config (0 for an invalid config or n_req outside [1, max_batch]).
 * Host only. */
size_t dflash_draft_static_bytes(const dflash_config *cfg, int32_t n_req);

/* Target-side verify forward ([guide] section 4: the target runs once over
 * the context plus the drafted block and checks every drafted token; section
 * 3.2: its feature layers feed the draft).  On a target handle: for each of
 * the n_req requests, n_rows (<= block_size) new tokens at positions
 * ctx_len .. ctx_len+n_rows-1 go through the causal decoder (row i attends
 * to every cached position and to new rows 0..i); their K/V are appended to
 * the slot's pages and ctx_len advances by n_rows.  Per row: the greedy token
 * (argmax of the logits, ties to the lowest id) and, optionally, the logits
 * and the residual stream after each listed feature layer (storage dtype),
 * ready for dflash_inject_context of the draft.
 *   slots        host [n_req] distinct bound slots
 *   tokens       device [n_req * n_rows] int32, rows grouped by request
 *   greedy       device [n_req * n_rows] int32 output
 *   logits       device [n_req * n_rows, V] fp32 output, or NULL
 *   feat_layers  host [n_feat_out] 0-based layer ids (< n_layers), ascending
 *   feat_out     host array of n_feat_out device pointers, each
 *                [n_req * n_rows, d] storage dtype output
 * The verify of a B-token draft takes the pending token and the B drafts
 * (n_rows = B + 1); after acceptance, dflash_set_context_length rolls the
 * slot back to the committed length.  DFLASH_E_CAPACITY if a slot's pages or
 * max_position cannot hold the new rows; DFLASH_E_INVALID on a draft handle. */
dflash_status dflash_target_forward(dflash_handle *h, void *stream, int32_t n_req, const int32_t *slots,
                                    int32_t n_rows, const int32_t *tokens, int32_t *greedy,
                                    float *logits, int32_t n_feat_out, const int32_t *feat_layers,
                                    void *const *feat_out);

/* Sets a bound slot's context length to ctx_len.  Lowering it is the
 * target's rollback after verification: positions from ctx_len on become
 * invisible and are overwritten by later writes.  Raising it (handles
 * without a window only, up to what the bound pages hold and below
 * max_position) declares positions that the caller has already written into
 * the slot's pages visible, e.g. a cached prefix copied in.  The device copy
 * of the slot state is updated by a kernel on `stream`: the call does not
 * wait for the device, and later work on that stream sees the new length.
 * DFLASH_E_INVALID for an unbound slot or a length outside [kv_begin, that
 * limit] (with a window: [kv_begin, current length]). */
dflash_status dflash_set_context_length(dflash_handle *h, void *stream, int32_t slot, int32_t ctx_len);

/* DFlash-2 path selector ([guide] section 7, path selector bullet): from
 * the top-16 candidates of every block position (dflash_draft_block's
 * topk_ids / topk_logits), one path per request: position 0 takes its top-1
 * candidate; position i+1 takes the candidate b maximising
 *   topk_logits[i+1][b] + (sel_u E[c_i]) . (sel_v E[b])
 * with c_i the candidate chosen at position i (ties to the lower candidate
 * index).  The path replaces the argmax drafts in dflash_verify_accept.
 *   topk_ids     device [n_req, B, 16] int32 (ids outside [0, vocab) are
 *                clamped and set the sticky error word)
 *   topk_logits  device [n_req, B, 16] fp32
 *   path         device [n_req, B] int32 output
 *   step_scores  device [n_req, B] fp32 output (the chosen step's score; for
 *                position 0 its logit), or NULL
 * DFLASH_E_UNSUPPORTED when the handle has no selector (selector_rank 0).
 * The projected embedding rows sel_u E and sel_v E (fp32 [V, r] each) are
 * computed once at device initialisation into the packed-weights buffer. */
dflash_status dflash_select_path(dflash_handle *h, void *stream, int32_t n_req,
                                 const int32_t *topk_ids, const float *topk_logits,
                                 int32_t *path, float *step_scores);

/* Sampling settings of sampled drafting and verification, applied to a row
 * of logits in this order: divide by temperature (0.01 .. 1000), keep the
 * top_k largest (0 = all; 1 .. 64; ties to the lower id), softmax, keep the
 * smallest prefix (probability descending, then id) whose cumulative
 * probability reaches top_p (0 < top_p <= 1; below 1 only with top_k >= 1),
 * renormalise.  The draft side has only its top-16 candidates per position,
 * so its top-k is capped at 16. */
typedef struct dflash_sampling {
  float temperature;
  int32_t top_k;
  float top_p;
} dflash_sampling;

/* Sampled drafting ([guide] section 7: the path is walked greedily or by
 * sampling): one token per block position drawn from the draft's warped
 * distribution over its top-16 list, with uniform number v: the first list
 * entry whose running probability sum exceeds v times the total.
 *   topk_ids, topk_logits  device [n_req, B, 16] (dflash_draft_block's lists)
 *   uniforms               device [n_req, B] fp32 in [0, 1), one per position
 *   draft                  device [n_req, B] int32 output
 * DFLASH_E_UNSUPPORTED for a handle without top-16 lists or for top_p below 1
 * with top_k 0; DFLASH_E_INVALID for settings out of range. */
dflash_status dflash_draft_sample(dflash_handle *h, void *stream, int32_t n_req,
                                  const dflash_sampling *sampling, const int32_t *topk_ids,
                                  const float *topk_logits, const float *uniforms, int32_t *draft);

/* Lossless sampled verification ([guide] section 7: rejection sampling keeps
 * the output distribution exactly the target's; section 3.3: rejected
 * positions are resampled): position i's draft x is accepted while
 * u[i][0] < p_i(x) / q_i(x) (p the target's warped distribution, q the
 * draft's over its top-16 list); at the first rejection the committed token
 * is drawn with u[i][1] from max(0, p_i - q_i) renormalised, after B
 * acceptances from p_B with u[B][1].  Draws walk the target's kept top-k list
 * (probability descending, then id), or token ids ascending when top_k is 0.
 *   draft          device [n_req, B] int32 drafted tokens (e.g. from
 *                  dflash_draft_sample with the same settings)
 *   topk_ids, topk_logits  device [n_req, B, 16] the draft's lists
 *   target_logits  device [n_req, B+1, V] fp32 the target's logits at
 *                  positions n .. n+B
 *   uniforms       device [n_req, B+1, 2] fp32 in [0, 1)
 *   accept_len, committed, last_token  as dflash_verify_accept
 * Errors as dflash_draft_sample. */
dflash_status dflash_verify_sample(dflash_handle *h, void *stream, int32_t n_req,
                                   const dflash_sampling *sampling, const int32_t *draft,
                                   const int32_t *topk_ids, const float *topk_logits,
                                   const float *target_logits, const float *uniforms,
                                   int32_t *accept_len, int32_t *committed, int32_t *last_token);

/* Step 5 ([news] "DFlash 2 的核心：一次写一块"; [guide] 3.3): a = number of
 * leading positions where draft equals the target's greedy token; commits
 * draft[0..a) followed by target_greedy[a], which becomes the next pending
 * token.  A pure function of its inputs: it does not touch the KV cache.
 *   draft         device [n_req, B] int32
 *   target_greedy device [n_req, B+1] int32 target argmax at positions n..n+B
 *   accept_len    device [n_req] int32 output, in [0, B]
 *   committed     device [n_req, B+1] int32 output, -1 padded after a+1 tokens
 *   last_token    device [n_req] int32 output, = target_greedy[a] */
dflash_status dflash_verify_accept(dflash_handle *h, void *stream, int32_t n_req,
                                   const int32_t *draft, const int32_t *target_greedy,
                                   int32_t *accept_len, int32_t *committed,
                                   int32_t *last_token);

/* Kernel classes for optional launch timing. */
typedef enum {
  DFLASH_KERNEL_FC_GEMM = 0,     /* inject: concat + projection */
  DFLASH_KERNEL_NORM = 1,        /* RMSNorms without DFlash-2 conv taps */
  DFLASH_KERNEL_KV_GEMM = 2,     /* inject: all-layer K/V projection */
  DFLASH_KERNEL_SCATTER = 3,     /* inject: RoPE + page scatter */
  DFLASH_KERNEL_QKV_GEMM = 4,
  DFLASH_KERNEL_QKV_POST = 5,    /* block q/k RoPE, block KV page */
  DFLASH_KERNEL_ATTN = 6,
  DFLASH_KERNEL_COMBINE = 7,     /* merge of attention splits */
  DFLASH_KERNEL_O_GEMM = 8,
  DFLASH_KERNEL_GATEUP_GEMM = 9,
  DFLASH_KERNEL_DOWN_GEMM = 10,
  DFLASH_KERNEL_LM_HEAD = 11,    /* vocabulary GEMM + argmax */
  DFLASH_KERNEL_FINALIZE = 12,   /* argmax decode */
  DFLASH_KERNEL_VERIFY = 13,     /* greedy or sampled verification */
  DFLASH_KERNEL_SELECT = 14,     /* selection pass over split-K partial logits */
  DFLASH_KERNEL_CONV = 15,       /* RMSNorms that also apply DFlash-2 conv taps */
  DFLASH_KERNEL_TOPK = 16,       /* merge of the top-16 lists */
  DFLASH_KERNEL_PATH = 17,       /* DFlash-2 path selector */
  DFLASH_KERNEL_SAMPLE = 18,     /* sampled drafting */
  DFLASH_KERNEL_TARGET_ATTN = 19, /* target: q RoPE, K/V append, causal attention */
  DFLASH_KERNEL_COUNT = 20
} dflash_kernel;

/* Launch timing for measurement runs.  After dflash_profile_begin(h, mask),
 * every launch of a kernel class whose bit (1 << dflash_kernel) is set in
 * `mask` is bracketed by two HIP events recorded on the call's stream (the
 * stream the kernel runs on).  dflash_profile_end synchronises on the last
 * event, writes per class the summed duration in milliseconds and the
 * launch count to total_ms[0..DFLASH_KERNEL_COUNT) and
 * launches[0..DFLASH_KERNEL_COUNT) (host arrays), and turns timing off.
 * Events are created on first use and kept by the handle; no device memory
 * is allocated.  Timing off (the default) adds nothing to a call. */
dflash_status dflash_profile_begin(dflash_handle *h, uint32_t mask);
dflash_status dflash_profile_end(dflash_handle *h, float *total_ms, int32_t *launches);

/* Replaces the set of timed classes of a running measurement without
 * discarding the events recorded since dflash_profile_begin, so a run can
 * time one call in n (mask 0 in between) and keep the events' own cost
 * (each record briefly idles the stream) off the other calls.  Returns
 * DFLASH_E_INVALID for a NULL handle; bits of unknown classes are ignored. */
dflash_status dflash_profile_mask(dflash_handle *h, uint32_t mask);

/* Synchronises `stream` and reads the sticky device error word; returns
 * DFLASH_E_DEVICE (and clears the word) if a kernel recorded an
 * out-of-range token id, else DFLASH_OK. */
dflash_status dflash_check(dflash_handle *h, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
