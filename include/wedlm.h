/*
 * wedlm.h - C ABI of one window step of WeDLM's Streaming Parallel Decoding,
 * implemented as hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The step (hyper.ai summary of WeDLM, "Method"; sai.science review, "Summary"):
 *   1. wedlm_window_reorder  - filled slots of the sliding window are placed
 *      physically before the mask slots; every slot keeps its logical position.
 *   2. wedlm_rope_logical    - rotary embedding (RoFormer, listed under
 *      "Builds on" on the mlsanity.com page) applied at the logical positions,
 *      gathering the window into physical order.
 *   3. wedlm_window_attn     - causal GQA attention of the reordered window over
 *      the persistent paged KV-cache prefix plus the window itself.
 *   4. wedlm_entropy_select  - softmax entropy over the full vocabulary per slot,
 *      distance-penalised score, fill of the mask slots that clear a threshold.
 *   5. wedlm_commit_prefix   - the leftmost contiguous filled run is appended to
 *      the paged cache and the window is refilled with masks.
 * Fused forms of steps 2-3 and 2-5: wedlm_window_attn_rope and
 * wedlm_commit_prefix_rope apply the RoPE of step 2 as they load the window,
 * so a step can run reorder -> attn_rope -> entropy_select -> commit_rope
 * without the separate RoPE pass and its physical-order copies.
 * wedlm_lm_head_select fuses the vocabulary projection that produces the
 * logits with step 4, so the logits are never written (wedlm_lm_head_pack lays
 * the projection out for it once). wedlm_select_commit_reorder runs step 4,
 * the window-state half of step 5 and the next step's step 1 as one tail, so
 * steps chain as reorder -> (attn_rope -> select_commit_reorder) repeated.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller, unless a
 *    comment says "host". The library never allocates, frees or synchronises:
 *    every call only enqueues kernels on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) and returns.
 *  - Host-side arguments are validated before any launch. On error nothing is
 *    enqueued and a negative status is returned (see wedlm_status).
 *  - Device-resident values that steer the kernels (prefix lengths, block-table
 *    entries, run lengths) are clamped to the documented ranges inside the
 *    kernels, so out-of-contract values give wrong results but never an
 *    out-of-bounds access.
 *  - The library keeps no mutable global state: calls are re-entrant; calls on
 *    different streams that write the same buffers race, as usual.
 *  - Element type: WEDLM_F32 or WEDLM_BF16 for every floating-point tensor of a
 *    call (window projections, caches, outputs, logits). Accumulation is fp32.
 *
 * Tensor layouts (row-major, innermost last; B sequences, W window slots,
 * Hq query heads, Hkv kv heads, g = Hq / Hkv, D head dim, P page size, V vocab)
 *  - window q   [n_layers][B][W][Hq][D],  k, v [n_layers][B][W][Hkv][D]
 *    (slot order before wedlm_rope_logical, physical order after it).
 *  - k_cache    [n_layers][num_pages][Hkv][D / X][P][X] with X = 16 / sizeof(elt)
 *    (8 for bf16, 4 for f32): in a page, the X-wide slices of each position's
 *    key are stored position-major, so the keys of a page are read as contiguous
 *    16-byte vectors. Keys are stored AFTER RoPE.
 *  - v_cache    [n_layers][num_pages][Hkv][D][P]: a page stores each value
 *    dimension's P positions contiguously (a transposed page).
 *  - block_table [B][max_pages] int32: logical position t of sequence b lives in
 *    page block_table[b][t / P] at offset t % P. All layers share the table.
 *  - logits     [B][W][V] in slot order.
 */
#ifndef WEDLM_H
#define WEDLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum wedlm_status {
  WEDLM_OK = 0,
  WEDLM_ERR_INVALID = -1,     /* null pointer, size <= 0, Hq % Hkv != 0, W > 64, ... */
  WEDLM_ERR_UNSUPPORTED = -2, /* a shape or dtype the library has no kernel for   */
  WEDLM_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required    */
  WEDLM_ERR_HIP = -4,         /* the HIP runtime reported an error at launch        */
  WEDLM_ERR_SCRATCH_LIMIT = -5 /* sizes exceed the fixed scratch of a *_noalloc call */
};

/* Element types. */
enum wedlm_dtype { WEDLM_F32 = 0, WEDLM_BF16 = 1 };

/* flags of wedlm_window_attn / wedlm_window_attn_rope / wedlm_window_attn_rope_entropy */
enum wedlm_attn_flags {
  WEDLM_ATTN_SHARED_PAGES = 1, /* rows of block_table reference the same pages */
  WEDLM_ATTN_DEFER_COMBINE = 2 /* leave the split merge to wedlm_select_commit_reorder_combine */
};

/* Largest window the kernels accept (one 64-lane wavefront per sequence). */
#define WEDLM_MAX_WINDOW 64

/* Commit rules of wedlm_window_reorder_rule. */
enum wedlm_commit_rule {
  WEDLM_COMMIT_STREAM = 0, /* the leftmost contiguous filled run (streaming decoding) */
  WEDLM_COMMIT_BLOCK = 1   /* the whole window once every slot is filled, else nothing */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* wedlm_status_string(int status);

/* Version of this ABI: (major << 16) | minor. */
int wedlm_abi_version(void);

/*
 * wedlm_window_reorder - topological reorder of the window.
 * hyper.ai summary of WeDLM, "Method": observed tokens move to the physical
 * front, masks to the end, logical position IDs are kept; the streaming decoder
 * reorders its window at every step.
 *
 * in : filled[B][W] uint8 (nonzero = filled), prefix_len[B] int32 (L_b >= 0).
 * out: perm[B][W]      slot held at physical index p (filled slots in ascending
 *                      order, then mask slots in ascending order);
 *      inv_perm[B][W]  physical index of slot i;
 *      pos[B][W]       logical position of physical row p = L_b + perm[p];
 *      n_obs[B]        number of filled slots;
 *      run_len[B]      length of the leading all-filled run of the window.
 * Requires 1 <= W <= WEDLM_MAX_WINDOW, B >= 1. Any output pointer may not be NULL.
 */
int wedlm_window_reorder(int B, int W, const uint8_t* filled, const int32_t* prefix_len,
                         int32_t* perm, int32_t* inv_perm, int32_t* pos, int32_t* n_obs,
                         int32_t* run_len, void* stream);

/*
 * wedlm_window_reorder_rule - wedlm_window_reorder with a choice of commit rule
 * for run_len (everything else identical). hyper.ai summary of WeDLM,
 * "Method", contrasts streaming with block decoding, where a block is cached
 * only once it is entirely finalised; sai.science review, "Reproducibility &
 * code": the released engine has no block-wise decoder.
 *   WEDLM_COMMIT_STREAM: run_len = the leading filled run (as wedlm_window_reorder);
 *   WEDLM_COMMIT_BLOCK:  run_len = W when every slot is filled, else 0, so the
 *     commit caches the whole window at once and refills it with W masks
 *     (stop-and-wait decoding on the same kernels).
 * Another commit_rule value returns WEDLM_ERR_INVALID.
 */
int wedlm_window_reorder_rule(int B, int W, int commit_rule, const uint8_t* filled,
                              const int32_t* prefix_len, int32_t* perm, int32_t* inv_perm,
                              int32_t* pos, int32_t* n_obs, int32_t* run_len, void* stream);

/*
 * wedlm_rope_logical - rotary embedding at logical positions, gathered into
 * physical order. RoFormer rotation (mlsanity.com page, "Builds on"), kept at
 * logical positions through the reordering (hyper.ai summary, "Method").
 *
 * Pairing: dimension j rotates with j + D/2 (j < D/2) by angle pos * theta^(-2j/D):
 *   y_j = x_j cos - x_{j+D/2} sin,  y_{j+D/2} = x_{j+D/2} cos + x_j sin.
 * Angles are formed and their sine/cosine evaluated in double precision; the
 * rotation is done in fp32 and rounded once to the element type.
 *
 * in : q (slot order, [n_layers][B][W][Hq][D]), k, v ([n_layers][B][W][Hkv][D]),
 *      perm, pos from wedlm_window_reorder.
 * out: q_phys[l][b][p] = R(pos[b][p]) q[l][b][perm[b][p]], k_phys likewise,
 *      v_phys[l][b][p] = v[l][b][perm[b][p]] (no rotation), same layouts.
 * Outputs must not alias inputs. D must be even; D <= 256.
 */
int wedlm_rope_logical(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D, double theta,
                       const void* q, const void* k, const void* v, const int32_t* perm,
                       const int32_t* pos, void* q_phys, void* k_phys, void* v_phys, void* stream);

/*
 * Bytes of workspace wedlm_window_attn needs for these sizes. max_prefix_len is
 * a host-side upper bound of every prefix_len[b]. Returns 0 when no workspace is
 * needed (no key-range split) and also for invalid sizes. When the key ranges
 * are split (too few (layer, sequence, kv head) groups to fill the GPU), how
 * the workgroups are shared out between the sequences follows the prefix_len
 * values on the device at launch time, so the size depends only on the host
 * sizes and no host synchronisation is needed.
 */
size_t wedlm_window_attn_workspace_size(int dtype, int n_layers, int B, int W, int Hq, int Hkv,
                                        int D, int page_size, int max_prefix_len);

/*
 * wedlm_window_attn - causal GQA attention of the reordered window over
 * [paged KV prefix ; window]. hyper.ai summary, "Method": a causal forward pass
 * over the window conditioned on the persistent KV cache; sai.science review,
 * "Strengths": the plain causal mask is kept (prior art for the kernels:
 * FlashAttention and PagedAttention, mlsanity.com page, "Builds on").
 *
 * For physical row p of sequence b and query head h (kv head h / g):
 *   keys   = the L_b cached keys (positions 0..L_b-1) then window rows 0..p,
 *   out[l][b][p][h] = softmax(scale * q_phys . keys) @ values.
 * Online softmax with fp32 accumulation; output rounded once to the element type.
 * bf16: scores from bf16 q and k in fp32; in the PV product the probabilities
 * carry ~16 bits (a bf16 hi + lo pair) for groups of up to 128 query rows
 * (W * Hq / Hkv), and are rounded once to fp16 against fp16 values (converted
 * from bf16 exactly; |v| <= 65504) for groups of 129..256 rows, each output
 * then within 2^-11 * max|v| of the exact softmax average over its keys.
 *
 * in : q_phys, k_phys, v_phys (physical order, rotated q/k) as written by
 *      wedlm_rope_logical; k_cache, v_cache (layouts above, num_pages pages per
 *      layer); block_table[B][max_pages]; prefix_len[B] (device; clamped to
 *      [0, max_prefix_len]).
 * out: out_phys [n_layers][B][W][Hq][D], physical order.
 * Host sizes: page_size P in {16}; max_prefix_len <= max_pages * P; bf16 needs
 * D == 128; f32 needs D a multiple of 4 and <= 256; n_layers, B and Hq at most
 * 65535 (WEDLM_ERR_UNSUPPORTED otherwise). Cache positions at or past prefix_len[b] in a sequence's last
 * page may hold any bits, NaN and Inf included: they never reach the output.
 * workspace: at least
 * wedlm_window_attn_workspace_size(...) bytes (may be NULL if that is 0).
 * Block-table entries are clamped to [0, num_pages).
 * flags: 0 when every page is referenced by one row of block_table (each
 * sequence owns its pages, as in decoding): each page is then read once per
 * launch and the bf16 path loads it with the non-temporal cache hint.
 * WEDLM_ATTN_SHARED_PAGES when rows share pages (a shared prefix; the
 * dual-stream forward, where every block of a sample reads the sample's
 * memory rows): the loads keep the default cache policy so that the re-reads
 * hit in the caches. Results are identical either way.
 * WEDLM_ATTN_DEFER_COMBINE (bf16): when the call splits key ranges across
 * workgroups (few groups for the GPU), it launches no merge of the split
 * partials: out_phys is then written by wedlm_select_commit_reorder_combine,
 * which must follow on the same stream with the same shapes, workspace and
 * out_phys, before the workspace is reused. Without a split the flag changes
 * nothing. Any other bit is WEDLM_ERR_INVALID.
 */
int wedlm_window_attn(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D, int page_size,
                      int num_pages, int max_pages, int max_prefix_len, float scale,
                      const void* q_phys, const void* k_phys, const void* v_phys, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* prefix_len,
                      void* out_phys, void* workspace, size_t workspace_bytes, int flags,
                      void* stream);

/*
 * wedlm_window_attn_rope - wedlm_window_attn with the RoPE step fused into its
 * loads (the same operation as wedlm_rope_logical followed by
 * wedlm_window_attn; hyper.ai summary, "Method": tokens keep their logical
 * positions through the reordering).
 *
 * q, k, v are the window rows in slot order before RoPE, as wedlm_rope_logical
 * takes them. Physical row p reads slot perm[b][p] and is rotated at pos[b][p]
 * (query rows and window keys; values are only gathered). The angle is formed
 * and reduced to [-pi/4, pi/4] in double precision, its sine and cosine
 * evaluated in fp32 (error ~1e-7), the rotation done in fp32 and rounded once
 * to the element type before the products, as with wedlm_rope_logical.
 * No q_phys / k_phys / v_phys is written. All other arguments, layouts, sizes,
 * workspace, flags and errors are those of wedlm_window_attn; theta > 0; the
 * f32 path needs D a multiple of 8 (WEDLM_ERR_UNSUPPORTED otherwise).
 *
 * commit_run (device [B], may be NULL): when given, the call also performs the
 * cache half of the commit (hyper.ai summary, "Method": the leftmost filled
 * run is committed at once): rows 0..c-1 of the window, rotated at pos[b][0..c-1]
 * as for the attention, are written to positions L..L+c-1 of k_cache / v_cache
 * through block_table, with c = commit_run[b] clamped to [0, W] and to
 * max_pages * P - L, and L = max(prefix_len[b], 0). With pos from
 * wedlm_window_reorder, pos[b][j] = L + j for these rows: they are the rows
 * wedlm_commit_prefix_rope would write.
 * Pass run_len from wedlm_window_reorder, then call wedlm_commit_prefix_rope
 * with k = v = NULL for the window-state half. The appended positions are
 * never among those the call reads (they are >= L). k_cache / v_cache are
 * written only when commit_run is non-NULL.
 */
int wedlm_window_attn_rope(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                           int page_size, int num_pages, int max_pages, int max_prefix_len,
                           float scale, double theta, const void* q, const void* k, const void* v,
                           const int32_t* perm, const int32_t* pos, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* prefix_len,
                           const int32_t* commit_run, void* out_phys, void* workspace,
                           size_t workspace_bytes, int flags, void* stream);

/*
 * wedlm_window_attn_rope_entropy - wedlm_window_attn_rope and the entropy
 * chunk pass of the same step (wedlm_entropy_partials) in one launch: the
 * workgroups past the attention's each reduce one chunk of one logit row, so
 * the chunk pass fills the GPU wherever the attention leaves it idle (a
 * batch too small to occupy every CU, the workgroups of a ragged batch that
 * end early, a last partial round) without a second stream. hyper.ai summary
 * of WeDLM, "Method": one forward pass yields the attention outputs and the
 * predictions whose entropies the selection ranks; with synthetic inputs the
 * logits are given, and the two reductions are independent.
 *
 * Arguments up to flags are those of wedlm_window_attn_rope (bf16 only, else
 * WEDLM_ERR_UNSUPPORTED); V, logits [B][W][V] bf16 and ent_workspace (at
 * least wedlm_entropy_select_workspace_size(dtype, B, W, V) bytes, else
 * WEDLM_ERR_WORKSPACE) are those of wedlm_entropy_partials. Results are
 * bitwise those of the two calls; follow with
 * wedlm_select_commit_reorder_partials on the same stream.
 */
int wedlm_window_attn_rope_entropy(int dtype, int n_layers, int B, int W, int Hq, int Hkv, int D,
                                   int page_size, int num_pages, int max_pages,
                                   int max_prefix_len, float scale, double theta, const void* q,
                                   const void* k, const void* v, const int32_t* perm,
                                   const int32_t* pos, void* k_cache, void* v_cache,
                                   const int32_t* block_table, const int32_t* prefix_len,
                                   const int32_t* commit_run, void* out_phys, void* workspace,
                                   size_t workspace_bytes, int flags, int V, const void* logits,
                                   void* ent_workspace, size_t ent_workspace_bytes,
                                   void* stream);

/* Bytes of workspace wedlm_entropy_select needs (per-chunk partial reductions). */
size_t wedlm_entropy_select_workspace_size(int dtype, int B, int W, int V);

/*
 * wedlm_entropy_select - per-slot softmax entropy and distance-penalised fill.
 * hyper.ai summary, "Method": positions are chosen by a distance-penalised
 * entropy rule favouring earlier positions; sai.science review, "Weaknesses":
 * the adjusted-entropy equation is missing from the text; "Reproducibility &
 * code": an entropy threshold controls filling and a None threshold decodes one
 * token per step.
 *
 * For every slot i of sequence b (all W slots are reduced; only masks are used):
 *   entropy  = Shannon entropy in nats of softmax(logits[b][i][:]) over all V,
 *   argmax   = lowest vocabulary id holding the maximum logit,
 *   score    = entropy + lambda * i   (fp32: product rounded, then the sum).
 * Selection among mask slots (filled[b][i] == 0): selected = score < tau.
 * If no mask slot is selected, min_fill == 1 and a mask slot exists, the mask
 * slot with the lowest score (lowest i on equal scores) is selected.
 * tau = -INFINITY with min_fill = 1 is one-token-per-step decoding.
 *
 * in : logits [B][W][V], filled [B][W]. Logits are finite (no NaN; the
 *      result of a row holding one is unspecified).
 * out: entropy, score [B][W] float32; argmax_tok [B][W] int32; selected [B][W]
 *      uint8 (0/1). workspace >= wedlm_entropy_select_workspace_size(...).
 */
int wedlm_entropy_select(int dtype, int B, int W, int V, const void* logits, const uint8_t* filled,
                         float lambda, float tau, int min_fill, float* entropy, float* score,
                         int32_t* argmax_tok, uint8_t* selected, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch of wedlm_entropy_select_noalloc (per GPU). */
#define WEDLM_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * wedlm_entropy_select_noalloc - wedlm_entropy_select without a workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same operation, arguments (minus workspace / workspace_bytes), layouts,
 * results (bitwise those of wedlm_entropy_select on the same inputs) and
 * errors as wedlm_entropy_select. The per-chunk partial reductions go to a
 * fixed array in device memory that the library owns: WEDLM_NOALLOC_SCRATCH_BYTES
 * (4 MiB) on every GPU the library runs on, held until the process ends. Sizes
 * whose partials need more - wedlm_entropy_select_workspace_size(dtype, B, W, V)
 * above 4 MiB, e.g. B * W rows of a 152k vocabulary beyond about 26k rows -
 * return WEDLM_ERR_SCRATCH_LIMIT before anything is enqueued. The call
 * allocates and frees nothing (the array's device address is looked up once
 * per device, on the first call with that device current; a failure there
 * returns WEDLM_ERR_HIP).
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or other host threads) race and may return
 * wrong results; calls ordered on one stream are safe. Nothing in the array
 * has to start cleared: each call writes every partial before reading it.
 */
int wedlm_entropy_select_noalloc(int dtype, int B, int W, int V, const void* logits,
                                 const uint8_t* filled, float lambda, float tau, int min_fill,
                                 float* entropy, float* score, int32_t* argmax_tok,
                                 uint8_t* selected, void* stream);

/* Bytes of the packed projection wedlm_lm_head_pack writes (0 for an unsupported shape). */
size_t wedlm_lm_head_packed_size(int dtype, int hidden, int V);

/*
 * wedlm_lm_head_pack - lays the vocabulary projection out for
 * wedlm_lm_head_select (once per model: the weights do not change between
 * steps). w_vocab [V][hidden] bf16 (row v = vocabulary entry v) is copied into
 * 4 KB tiles: tile (b, c), at element offset (b * hidden / 64 + c) * 2048,
 * holds rows 32b .. 32b+31 and hidden elements 64c .. 64c+63, ordered
 * [ks][kg][row][8] with ks in 0..3, kg in 0..1, where the 8 elements are hidden
 * 64c + 32kg + 8ks .. +7 of that row (the operand order of one MFMA K-step).
 * Rows 32 * ceil(V / 32) > v >= V are zeros. w_packed holds
 * wedlm_lm_head_packed_size bytes; both pointers 16-byte aligned.
 * dtype WEDLM_BF16 and hidden a multiple of 256, else WEDLM_ERR_UNSUPPORTED.
 */
int wedlm_lm_head_pack(int dtype, int hidden, int V, const void* w_vocab, void* w_packed,
                       void* stream);

/* Bytes of workspace wedlm_lm_head_select needs (per-tile partial reductions). */
size_t wedlm_lm_head_select_workspace_size(int dtype, int B, int W, int hidden, int V);

/*
 * wedlm_lm_head_select - vocabulary projection fused with wedlm_entropy_select.
 * hyper.ai summary of WeDLM, "Method": the causal forward pass over the window
 * produces the predictions that the distance-penalised entropy rule ranks; its
 * last operation maps each slot's final hidden state to vocabulary logits.
 *
 * For every slot i of sequence b the logits are z = hidden[b][i][:] . w^T
 * (z_v = sum_k hidden[b][i][k] * w[v][k], products of the bf16 inputs
 * accumulated in fp32; no bias), and entropy, argmax, score and selected are
 * then exactly those wedlm_entropy_select computes from z (same readings,
 * same fp32 score arithmetic and threshold / floor rule). z itself is never
 * stored.
 *
 *   hidden_states  [B][W][hidden] bf16, slot order, 16-byte aligned.
 *   w_packed       the projection w [V][hidden] as wedlm_lm_head_pack wrote it.
 *   filled, lambda, tau, min_fill, entropy, score, argmax_tok, selected:
 *                  as wedlm_entropy_select.
 *   workspace >= wedlm_lm_head_select_workspace_size(...).
 * dtype must be WEDLM_BF16 and hidden a multiple of 256 (else
 * WEDLM_ERR_UNSUPPORTED); W <= WEDLM_MAX_WINDOW, B * W <= 65535.
 */
int wedlm_lm_head_select(int dtype, int B, int W, int hidden, int V, const void* hidden_states,
                         const void* w_packed, const uint8_t* filled, float lambda, float tau,
                         int min_fill, float* entropy, float* score, int32_t* argmax_tok,
                         uint8_t* selected, void* workspace, size_t workspace_bytes, void* stream);

/*
 * wedlm_commit_prefix - commit of the leading filled run, paged append, refill.
 * hyper.ai summary, "Method": the leftmost contiguous filled prefix is committed
 * to the cache at once (under the causal mask its KV depends only on earlier
 * tokens) and new masks are appended to keep the window W wide.
 *
 * With c = run_len[b] (the run at forward time; physical rows 0..c-1 are slots
 * 0..c-1) and L = prefix_len[b]:
 *   - for every layer, k_phys/v_phys rows 0..c-1 are written to cache positions
 *     L..L+c-1 through block_table; cache_slot[b][j] = page * P + offset for
 *     j < c, -1 otherwise;
 *   - the window is updated in place: slots chosen by `selected` become filled
 *     with argmax_tok; the window shifts left by c; c masks (token mask_id,
 *     filled 0) are appended; prefix_len[b] += c; commit_len[b] = c.
 * c is clamped to [0, W] and to the pages the table holds (max_pages * P - L).
 * Page size P = page_size must be 16 (WEDLM_ERR_UNSUPPORTED otherwise). The
 * cache lines holding the committed rows are rewritten whole: positions of
 * those pages beyond L+c-1 keep their previous contents.
 *
 * in : run_len, selected, argmax_tok (from the reorder / select calls of the
 *      same step), k_phys, v_phys (physical order), block_table.
 * in/out: k_cache, v_cache (rows written), tokens [B][W] int32, filled [B][W]
 *      uint8, prefix_len [B] int32.
 * out: commit_len [B] int32, cache_slot [B][W] int32.
 */
int wedlm_commit_prefix(int dtype, int n_layers, int B, int W, int Hkv, int D, int page_size,
                        int num_pages, int max_pages, const int32_t* run_len,
                        const uint8_t* selected, const int32_t* argmax_tok, const void* k_phys,
                        const void* v_phys, const int32_t* block_table, void* k_cache,
                        void* v_cache, int32_t* tokens, uint8_t* filled, int32_t* prefix_len,
                        int32_t* commit_len, int32_t* cache_slot, int32_t mask_id, void* stream);

/*
 * wedlm_commit_prefix_rope - wedlm_commit_prefix taking the window rows in slot
 * order before RoPE (k, v as given to wedlm_rope_logical) instead of k_phys /
 * v_phys. The committed rows 0..c-1 are slots 0..c-1 (the leading filled run
 * comes first in physical order), so values are copied as they are and each
 * committed key row j is rotated at its logical position L + j (angle and
 * rounding as in wedlm_window_attn_rope) before it is written. With
 * wedlm_window_attn_rope this makes the step's RoPE pass unnecessary. Other
 * arguments, layouts and errors are those of wedlm_commit_prefix; theta > 0;
 * D <= 256. k = v = NULL: the rows were appended by wedlm_window_attn_rope
 * (commit_run = run_len) and only the window state is updated (cache_slot,
 * tokens, filled, prefix_len, commit_len, exactly as otherwise).
 */
int wedlm_commit_prefix_rope(int dtype, int n_layers, int B, int W, int Hkv, int D, int page_size,
                             int num_pages, int max_pages, double theta, const int32_t* run_len,
                             const uint8_t* selected, const int32_t* argmax_tok, const void* k,
                             const void* v, const int32_t* block_table, void* k_cache,
                             void* v_cache, int32_t* tokens, uint8_t* filled,
                             int32_t* prefix_len, int32_t* commit_len, int32_t* cache_slot,
                             int32_t mask_id, void* stream);

/*
 * wedlm_select_commit_reorder - the step's tail in one call: entropy and
 * selection (wedlm_entropy_select), the window-state half of the commit
 * (wedlm_commit_prefix_rope with k = v = NULL) and the next step's reorder
 * (wedlm_window_reorder_rule) of the refreshed window. hyper.ai summary of
 * WeDLM, "Method": after the forward the decoder fills positions by the
 * distance-penalised entropy rule, commits the leftmost filled run, appends
 * masks, and the next forward starts from the window reordered again.
 *
 * Results are bitwise those of the three calls in that order on the same
 * inputs: entropy, score, argmax_tok, selected as wedlm_entropy_select;
 * tokens, filled, prefix_len, commit_len, cache_slot as the commit (with c
 * from this step's run_len, clamped as there); then perm, inv_perm, pos,
 * n_obs and run_len of the new window as wedlm_window_reorder_rule under
 * commit_rule.
 *
 * The committed rows must already be in the cache: the step's
 * wedlm_window_attn_rope ran with commit_run = run_len. run_len is in/out:
 * read as this step's run (from the reorder that ordered this step's
 * window), overwritten with the next step's. The perm / pos the step's
 * attention read are overwritten too, so the call must follow that attention
 * on the same stream (it always does when both are on one stream).
 *   logits [B][W][V] (dtype), 16-byte aligned for the vector path.
 *   block_table [B][max_pages]; page_size must be 16 (else
 *   WEDLM_ERR_UNSUPPORTED). Other arguments and layouts as in the three calls.
 *   workspace >= wedlm_entropy_select_workspace_size(dtype, B, W, V).
 * B * W <= 65535; W <= WEDLM_MAX_WINDOW.
 */
int wedlm_select_commit_reorder(int dtype, int B, int W, int V, const void* logits, float lambda,
                                float tau, int min_fill, int page_size, int num_pages,
                                int max_pages, int commit_rule, const int32_t* block_table,
                                int32_t* run_len, int32_t* tokens, uint8_t* filled,
                                int32_t* prefix_len, int32_t* commit_len, int32_t* cache_slot,
                                int32_t mask_id, float* entropy, float* score,
                                int32_t* argmax_tok, uint8_t* selected, int32_t* perm,
                                int32_t* inv_perm, int32_t* pos, int32_t* n_obs, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * wedlm_entropy_partials / wedlm_select_commit_reorder_partials - the two
 * halves of wedlm_select_commit_reorder as separate calls. The first reads
 * only the logits: it reduces every row's chunks of the vocabulary to
 * partial (max, sum, weighted sum, argmax) records in `workspace`; the second
 * merges them and runs the selection, window-state commit and next reorder
 * exactly as wedlm_select_commit_reorder does. Since the chunk pass needs
 * nothing the step's attention writes, it can run on a second stream
 * concurrently with wedlm_window_attn_rope (hyper.ai summary of WeDLM,
 * "Method": the entropy rule reads the forward pass's predictions; with
 * synthetic inputs those are given before the attention runs); the caller
 * orders the tail after both (and the next chunk pass after this tail, which
 * reads the same workspace).
 *
 * Results are bitwise those of wedlm_select_commit_reorder on the same
 * inputs. Both calls take the same dtype, B, W, V and a workspace of at least
 * wedlm_entropy_select_workspace_size(dtype, B, W, V) bytes; other arguments
 * and layouts as there (logits 16-byte aligned for the vector path).
 */
int wedlm_entropy_partials(int dtype, int B, int W, int V, const void* logits, void* workspace,
                           size_t workspace_bytes, void* stream);
int wedlm_select_commit_reorder_partials(int dtype, int B, int W, int V, float lambda, float tau,
                                         int min_fill, int page_size, int num_pages,
                                         int max_pages, int commit_rule,
                                         const int32_t* block_table, int32_t* run_len,
                                         int32_t* tokens, uint8_t* filled, int32_t* prefix_len,
                                         int32_t* commit_len, int32_t* cache_slot,
                                         int32_t mask_id, float* entropy, float* score,
                                         int32_t* argmax_tok, uint8_t* selected, int32_t* perm,
                                         int32_t* inv_perm, int32_t* pos, int32_t* n_obs,
                                         const void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * wedlm_select_commit_reorder_combine - wedlm_select_commit_reorder_partials
 * and the merge of the step's split attention partials in one launch: the
 * merge a wedlm_window_attn* call with WEDLM_ATTN_DEFER_COMBINE left out
 * runs as workgroups beside the per-sequence tail. The merge
 * (out = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m) over the splits, the
 * online-softmax merge of FlashAttention, mlsanity.com page on WeDLM,
 * "Builds on") and the tail (hyper.ai summary of WeDLM, "Method": selection,
 * commit and refill of the window) read disjoint data, so one launch replaces
 * two at the end of a step.
 *
 * Arguments up to workspace_bytes are those of
 * wedlm_select_commit_reorder_partials (B and W are shared with the
 * attention). attn_n_layers, attn_Hq, attn_Hkv, attn_D, attn_max_prefix_len,
 * attn_workspace / attn_workspace_bytes and attn_out are the shapes,
 * workspace and out_phys of the preceding attention call (same dtype), which
 * must have run on the same stream with WEDLM_ATTN_DEFER_COMBINE. When those
 * shapes make no split, only the tail runs. Results are bitwise those of the
 * attention call without the flag followed by
 * wedlm_select_commit_reorder_partials. Errors: as the tail's, plus the
 * attention's shape checks; WEDLM_ERR_WORKSPACE when attn_workspace is
 * smaller than the attention's; WEDLM_ERR_INVALID for a NULL attn_out with a
 * split.
 */
int wedlm_select_commit_reorder_combine(
    int dtype, int B, int W, int V, float lambda, float tau, int min_fill, int page_size,
    int num_pages, int max_pages, int commit_rule, const int32_t* block_table, int32_t* run_len,
    int32_t* tokens, uint8_t* filled, int32_t* prefix_len, int32_t* commit_len,
    int32_t* cache_slot, int32_t mask_id, float* entropy, float* score, int32_t* argmax_tok,
    uint8_t* selected, int32_t* perm, int32_t* inv_perm, int32_t* pos, int32_t* n_obs,
    const void* workspace, size_t workspace_bytes, int attn_n_layers, int attn_Hq, int attn_Hkv,
    int attn_D, int attn_max_prefix_len, const void* attn_workspace,
    size_t attn_workspace_bytes, void* attn_out, void* stream);

/*
 * wedlm_block_attn_rope - the attention of the windows of S sequences laid
 * end to end (hyper.ai summary of WeDLM, "Method": in training, a masked
 * prediction stream is cut into blocks that are reordered inside; a block's
 * tokens attend to the memory stream's context before the block and,
 * causally, to their own block; the memory stream itself is causal).
 *
 * Sequence s holds N positions as nb = N / W consecutive windows; window j
 * of sequence s is batch row b = s * nb + j of q, k, v, perm, pos and out.
 * The result is that of wedlm_window_attn_rope (n_layers = 1, B = S * nb,
 * flags = WEDLM_ATTN_SHARED_PAGES, no commit_run) with prefix_len[b] = j * W
 * and block-table row b = row s of block_table: window j attends to cache
 * positions 0 .. jW-1 of its sequence and to its own W keys causally in
 * physical order (physical row p reads slot perm[b][p], rotated at pos[b][p]).
 * Up to rounding: the key tiles are visited in another order, each workgroup
 * takes 256 query rows of consecutive windows against every key tile it reads
 * (bf16, D = 128, P = 16 only), and the probabilities enter the PV product in
 * fp16 (the values converted from bf16 exactly), so each output row is within
 * 2^-11 * max|v| of the exact softmax average over its keys, max|v| being the
 * largest value magnitude the row attends to. Values must lie within fp16's
 * range (|v| <= 65504).
 *
 * q [S*nb][W][Hq][D], k, v [S*nb][W][Hkv][D] (slot order, before RoPE);
 * perm, pos [S*nb][W]; k_cache / v_cache the cache layout of
 * wedlm_window_attn (one layer), read only; block_table [S][max_pages]
 * (entries clamped to the pool); out [S*nb][W][Hq][D] in physical order.
 * Every position below N - W of each sequence that some window attends to
 * must hold its key and value (e.g. written by wedlm_commit_prefix_rope).
 * All device pointers; caller-owned; one kernel on stream.
 *
 * Errors: WEDLM_ERR_INVALID for NULL pointers, sizes <= 0, W > 64, N % W != 0,
 * Hq % Hkv != 0, scale <= 0, theta <= 0, max_pages * P < N - W;
 * WEDLM_ERR_UNSUPPORTED unless dtype is bf16, D = 128, page_size = 16 and
 * 256 % (Hq / Hkv) == 0.
 */
int wedlm_block_attn_rope(int dtype, int S, int N, int W, int Hq, int Hkv, int D, int page_size,
                          int num_pages, int max_pages, float scale, double theta, const void* q,
                          const void* k, const void* v, const int32_t* perm, const int32_t* pos,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          void* out, void* stream);

/*
 * wedlm_read_probe - HBM read-rate probe, a measurement aid beside the step
 * (not a step of the method): the rate this GPU reaches on a plain streaming
 * read and on the paged cache's pattern gives the step kernels' roofline
 * fractions their context.
 *
 * block_order == NULL: reads all of src[0 .. bytes) once as 16-byte vectors
 *   (grid-stride, non-temporal).
 * block_order != NULL: reads n_blocks 4 KB blocks of src, block
 *   block_order[j] for j = 0 .. n_blocks-1 (entries clamped to the
 *   bytes / 4096 blocks src holds), one wavefront per block at a time.
 * src 16-byte aligned, bytes >= 16; sink holds grid * 256 uint32 (one
 * xor-fold per thread, written so that no read is dead code);
 * 0 < grid <= 2^20. Enqueues one kernel on stream.
 */
int wedlm_read_probe(const void* src, size_t bytes, const int32_t* block_order, int n_blocks,
                     uint32_t* sink, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WEDLM_H */
