/*
 * nsa.h -- C ABI of libnsa: Native Sparse Attention (NSA) forward pass, decode
 * step and backward pass on AMD MI355X (gfx950).
 *
 * NSA passes the same queries through three attention branches and sums
 * them with per-head gates (deepdaiv newsletter on DeepSeek's NSA,
 * deepdaiv.stibee.com/p/82, paragraphs on token compression, token selection
 * and the sliding window; valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파,
 * 딥시크의 새 어텐션 기술 화제", section II for the sizes l=32, d=16, l'=64,
 * n=16 including 1 initial and 2 local blocks, w=512):
 *   1. compressed branch: attention over one summary vector per block of l
 *      tokens taken every d tokens;
 *   2. selected branch: attention over the n selection blocks of l' tokens
 *      that rank highest by importance derived from the compressed branch's
 *      attention probabilities (the first block and the 2 most recent blocks
 *      are always kept);
 *   3. sliding window: attention over the w most recent tokens.
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers, row-major, densely packed, in
 *    the element type given by nsa_config.dtype (fp32 or bf16), except the
 *    int32 index tensors, the fp32 score tensor and the int32 seq_lens.
 *    Every tensor pointer must be 16-byte aligned; the workspace 256-byte
 *    aligned.
 *  - The caller owns all memory, including the workspace; the library never
 *    allocates device memory and never synchronizes.  Work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) in argument order,
 *    and the call returns once it is enqueued.
 *  - Arguments are checked on the host before anything is enqueued; on a
 *    failed check the call returns an error status and enqueues nothing.
 *    A failed launch returns NSA_ERR_HIP.  Faults inside kernels surface at
 *    the caller's next synchronization.  No C++ exception crosses the ABI.
 *  - The library holds no state between calls; calls on different streams
 *    may run concurrently if their outputs and workspaces do not overlap.
 *
 * Layouts (B batch, T tokens, Hkv KV heads, G query heads per KV head,
 * Hq = Hkv*G, dk/dv head dims, N_cmp = floor((T-32)/16)+1 compressed blocks
 * (0 if T < 32), N_pad = max(64, N_cmp rounded up to a multiple of 64),
 * NB = ceil(T/64) selection blocks):
 *   q      [B][T][Hq][dk]       query head h belongs to KV head h / G
 *   k      [B][Hkv][T][dk]      v [B][Hkv][T][dv]
 *   cmp_k  [B][Hkv][N_pad][dk]  cmp_v [B][Hkv][N_pad][dv]  (rows >= N_cmp are 0)
 *   w_ck   [dk][32*dk]  pe_k [32][dk]   w_cv [dv][32*dv]  pe_v [32][dv]
 *   w_g    [Hq][3][dk]  b_g  [Hq][3]    gate order: compressed, selected, window
 *   o      [B][T][Hq][dv]
 *   idx    [B][Hkv][T][n] int32, ascending, padded with -1
 *   scores [B][Hkv][T][NB] fp32; entries j > floor(t/64) are unspecified
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NSA_OK = 0,
    NSA_ERR_NULL = -1,      /* a required pointer is NULL */
    NSA_ERR_SHAPE = -2,     /* a size is out of the supported range */
    NSA_ERR_DTYPE = -3,     /* dtype is not NSA_FP32 or NSA_BF16 */
    NSA_ERR_PARAM = -4,     /* l, d, l_sel, n, w, scale or a scalar argument unsupported */
    NSA_ERR_WORKSPACE = -5, /* workspace NULL or smaller than nsa_workspace_bytes */
    NSA_ERR_HIP = -6,       /* a HIP launch failed */
    NSA_ERR_ALIGN = -7      /* a pointer is not aligned as required */
} nsa_status;

typedef enum { NSA_FP32 = 0, NSA_BF16 = 1 } nsa_dtype;

typedef enum {
    NSA_OP_FORWARD = 0, /* nsa_forward */
    NSA_OP_SELECT = 1,  /* nsa_select_blocks */
    NSA_OP_DECODE = 2,  /* nsa_decode_step */
    NSA_OP_SPARSE = 3,  /* nsa_sparse_attention */
    NSA_OP_BACKWARD = 4, /* nsa_backward */
    NSA_OP_DSA_DECODE = 5, /* nsa_dsa_decode: B*T fp32 indexer scores, then the split attention's partials */
    NSA_OP_DSA_PREFILL = 6, /* nsa_dsa_prefill: the indexer scores of one chunk of rows (<= 256 MiB) */
    NSA_OP_BACKWARD_MLP = 7, /* nsa_backward_mlp */
    NSA_OP_CMP_WINDOW = 8 /* nsa_compressed_window_attention: o_cmp when not run as one kernel */
} nsa_op;

/* Problem description.  Supported ranges (checked on every call):
 *   B >= 1; 1 <= T <= 524288; Hkv >= 1; 1 <= group <= 16;
 *   d_k, d_v multiples of 8 in [8, 256];
 *   l = 32, d = 16, l_sel = 64 (the sizes the kernels are built around);
 *   3 <= n <= 16 (n counts the 3 always-kept blocks); 1 <= w <= 8192;
 *   scale > 0, or 0 for 1/sqrt(d_k). */
typedef struct {
    int32_t B, T, H_kv, group, d_k, d_v;
    int32_t l, d, l_sel, n, w;
    float scale;
    int32_t dtype; /* nsa_dtype */
} nsa_config;

/* Bytes of workspace `op` needs for `cfg` (0 if cfg is invalid). */
size_t nsa_workspace_bytes(const nsa_config *cfg, int op);

/* Token compression (deepdaiv newsletter, token compression paragraph: each
 * block of consecutive tokens is summarised into one vector by a small
 * learned map with a position encoding of each token in the block).
 * For every (b, h) and block i < N_cmp:
 *   cmp_k[b][h][i][c] = sum_{tau<32, e<dk} w_ck[c][tau*dk+e] * (k[b][h][16i+tau][e] + pe_k[tau][e])
 * and likewise cmp_v from v, w_cv, pe_v.  Rows N_cmp..N_pad-1 are written as 0.
 * fp32 accumulation; bf16 outputs are rounded to nearest even. */
nsa_status nsa_compress_kv(const nsa_config *cfg, const void *k, const void *v, const void *w_ck,
                           const void *pe_k, const void *w_cv, const void *pe_v, void *cmp_k, void *cmp_v,
                           void *stream);

/* Token compression by a small two-layer network (deepdaiv newsletter, token
 * compression paragraph: a small neural network with a position encoding
 * summarises each block; the page gives no layer count, width or
 * activation, and this variant takes two layers of width d, ReLU, no
 * biases).  For every (b, h) and block i < N_cmp:
 *   a[j]   = sum_{tau<32, e<dk} w1_k[j][tau*dk+e] * (k[b][h][16i+tau][e] + pe_k[tau][e])
 *   cmp_k[b][h][i][c] = sum_{j<dk} w2_k[c][j] * max(a[j], 0)
 * and likewise cmp_v from v, w1_v, pe_v, w2_v (w2_v [dv][dv]).  a is rounded
 * to the storage type (a bf16 hidden layer for bf16 storage), the output to
 * nearest even; fp32 accumulation.  Rows N_cmp..N_pad-1 are written as 0.
 * w1_k, pe_k, w1_v, pe_v have the shapes of w_ck, pe_k, w_cv, pe_v above;
 * w2_k [dk][dk], w2_v [dv][dv] row-major, storage dtype, 16-byte aligned.
 * The compressed outputs feed nsa_compressed_attention, nsa_forward and
 * nsa_decode_step unchanged; nsa_backward_mlp is the backward pass with this
 * map, and nsa_compress_append_mlp its incremental form for decoding. */
nsa_status nsa_compress_kv_mlp(const nsa_config *cfg, const void *k, const void *v, const void *w1_k,
                               const void *pe_k, const void *w2_k, const void *w1_v, const void *pe_v,
                               const void *w2_v, void *cmp_k, void *cmp_v, void *stream);

/* Incremental compression of caches that grow token by token (the decode
 * step of valuable12.com section III.3 reads compressed entries for every
 * complete block; with the token compression of the deepdaiv newsletter a
 * new block completes every 16 tokens).  cfg->T is the cache capacity; the
 * caches are laid out as k/v and cmp_k/cmp_v above with T = capacity.
 * For each sequence b, the blocks i with 16i+31 < len_new[b] that were not
 * complete at len_old[b] tokens (16i+31 >= len_old[b]) are computed from
 * k_cache/v_cache as nsa_compress_kv defines them and written to cmp_k /
 * cmp_v; no other entry is touched.  len_old, len_new: device int32 [B],
 * clamped to 0 <= len_old <= len_new <= T; len_old may be NULL (all zero:
 * the hand-off of a prompt's caches to decoding).  max_append (host, 1..T):
 * an upper bound on len_new[b] - len_old[b] that only sizes the launch; the
 * result does not depend on it.  Each block comes out bit for bit as
 * nsa_compress_kv writes it for the same tokens. */
nsa_status nsa_compress_append(const nsa_config *cfg, const int32_t *len_old, const int32_t *len_new,
                               int32_t max_append, const void *k_cache, const void *v_cache, const void *w_ck,
                               const void *pe_k, const void *w_cv, const void *pe_v, void *cmp_k, void *cmp_v,
                               void *stream);

/* nsa_compress_append with the two-layer map of nsa_compress_kv_mlp (the
 * deepdaiv newsletter's small network; shapes of w1_k, pe_k, w2_k, w1_v,
 * pe_v, w2_v as there): the blocks that growing the caches from len_old[b] to
 * len_new[b] tokens completes are computed as nsa_compress_kv_mlp defines
 * them, each bit for bit as nsa_compress_kv_mlp makes it; no other entry is
 * touched.  Arguments and errors as nsa_compress_append. */
nsa_status nsa_compress_append_mlp(const nsa_config *cfg, const int32_t *len_old, const int32_t *len_new,
                                   int32_t max_append, const void *k_cache, const void *v_cache, const void *w1_k,
                                   const void *pe_k, const void *w2_k, const void *w1_v, const void *pe_v,
                                   const void *w2_v, void *cmp_k, void *cmp_v, void *stream);

/* Stage S2 -- compressed attention and block importance (deepdaiv
 * newsletter, token compression and token selection paragraphs: the block
 * scores are computed from the compressed tokens).  For each (b, g, t) and
 * each of the G query heads h of KV head g:
 *   p_h[i] = softmax over visible blocks i (16i+31 <= t) of scale*q_h.cmp_k[i]
 *   o_cmp[b][t][h] = sum_i p_h[i] cmp_v[i]          (0 if no block is visible)
 *   scores[b][g][t][j] = sum_h sum_i overlap(i, j)/16 * p_h[i]
 * where overlap(i, j) counts the tokens compression block i shares with
 * selection block j (weights 1,2,2,2,1 over i = 4j-1 .. 4j+3).  Only the
 * entries j <= floor(t/64) are written (rows with no visible block score 0);
 * the others are left as they were.
 *   cmp_v / o_cmp: may both be NULL (scores only); o_cmp [B][T][Hq][dv] in
 *   the config dtype.  scores: required, fp32. */
nsa_status nsa_compressed_attention(const nsa_config *cfg, const void *q, const void *cmp_k, const void *cmp_v,
                                    void *o_cmp, float *scores, void *stream);

/* Stage S3 -- top-n block selection (valuable12.com section II: n blocks
 * including the initial block and 2 local blocks).  For each (b, g, t) with
 * jc = floor(t/64): blocks {0, jc-1, jc} are always kept; the other
 * n - #kept are the highest-scoring remaining blocks (ties: lower j), or all
 * of them when there are no more than that.  idx [B][Hkv][T][n], ascending,
 * -1 padded.  scores as written by nsa_compressed_attention. */
nsa_status nsa_select_topn(const nsa_config *cfg, const float *scores, int32_t *idx, void *stream);

/* Stage S4 -- selected-block attention, window attention and the gated sum.
 * For each (b, t) and head h:
 *   o_slc = one softmax attention over the tokens tau <= t of the blocks in
 *           idx[b][h/G][t] (as a set; entries outside 0..floor(t/64) add
 *           nothing; allinfo.ai.kr DSA explainer, "쉽게 이해하기": the softmax
 *           normalises over the selected set only);
 *   o_win = softmax attention over tokens [max(0, t-w+1), t] (deepdaiv
 *           newsletter, sliding window paragraph);
 *   o = sigmoid(w_g[h][0].q_h + b_g[h][0]) * o_cmp + sigmoid(w_g[h][1].q_h
 *       + b_g[h][1]) * o_slc + sigmoid(w_g[h][2].q_h + b_g[h][2]) * o_win.
 * o_cmp as written by nsa_compressed_attention.  ws: nsa_workspace_bytes(cfg,
 * NSA_OP_SPARSE) bytes (it holds K and V repacked per 64-token block); may
 * be NULL when that size is 0. */
nsa_status nsa_sparse_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                const void *o_cmp, const int32_t *idx, const void *w_g, const void *b_g, void *o,
                                void *ws, size_t ws_bytes, void *stream);

/* Stage S4 in parts, for callers that schedule them separately (for
 * example to overlap the window half with other work or to time each
 * kernel).  nsa_sparse_attention equals nsa_pack_kv_blocks, then
 * nsa_window_attention, then nsa_selected_attention on the same o: bit for
 * bit where the packed-block workspace is used (NSA_OP_SPARSE size > 0);
 * elsewhere to the rounding of o (the one-call form rounds the gated sum of
 * the three branches once, the parts round after the window and compressed
 * terms and again after the selected one).
 *   nsa_pack_kv_blocks:     writes K and V, repacked per 64-token block,
 *                           into ws (nsa_workspace_bytes(cfg,
 *                           NSA_OP_SPARSE) bytes; nothing is written when
 *                           that size is 0 and ws may then be NULL);
 *   nsa_window_attention:   o = g_cmp * o_cmp + g_win * o_win (o written);
 *   nsa_selected_attention: o += g_slc * o_slc (o read and written).  ws
 *                           must hold what nsa_pack_kv_blocks wrote for the
 *                           same k and v (it is read, not rewritten); k and
 *                           v are read directly when the workspace size is 0.
 * Definitions and layouts as for nsa_sparse_attention. */
nsa_status nsa_pack_kv_blocks(const nsa_config *cfg, const void *k, const void *v, void *ws, size_t ws_bytes,
                              void *stream);
nsa_status nsa_window_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                const void *o_cmp, const void *w_g, const void *b_g, void *o, void *stream);
nsa_status nsa_selected_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                  const int32_t *idx, const void *w_g, const void *b_g, void *o, void *ws,
                                  size_t ws_bytes, void *stream);

/* Stage S2 and the window half of S4 in one call: scores as written by
 * nsa_compressed_attention, and o = g_cmp * o_cmp + g_win * o_win as written
 * by nsa_window_attention (definitions as for those two; the 16-head bf16
 * configurations at d_k/d_v = 192/128, 128/128, 64/64 run it as one kernel,
 * which reuses each workgroup's query fragments and o_cmp for its window
 * rows).  o_cmp: written if non-NULL, else only used internally.  Followed
 * by nsa_select_topn, nsa_pack_kv_blocks and nsa_selected_attention on the
 * same o, it is nsa_forward in parts (for callers that schedule or time
 * them): bit for bit where NSA_OP_SPARSE's workspace size is non-zero,
 * elsewhere to the rounding of o as for nsa_sparse_attention's parts.  ws: nsa_workspace_bytes(cfg, NSA_OP_CMP_WINDOW)
 * bytes, 256-byte aligned, needed only when that size is non-zero and o_cmp
 * is NULL (it then holds o_cmp). */
nsa_status nsa_compressed_window_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                           const void *cmp_k, const void *cmp_v, const void *w_g, const void *b_g,
                                           float *scores, void *o, void *o_cmp, void *ws, size_t ws_bytes,
                                           void *stream);

/* Block selection alone: S2 (scores only) followed by S3, i.e. the
 * importance of each selection block derived from the compressed branch's
 * attention (deepdaiv newsletter, token selection paragraph) and the top-n
 * blocks with the initial and the 2 local blocks always kept (valuable12.com
 * section II).  Definitions, layouts and the scores written as for
 * nsa_compressed_attention and nsa_select_topn.  scores_out may be NULL (the
 * workspace holds them then); idx_out is required.  ws:
 * nsa_workspace_bytes(cfg, NSA_OP_SELECT) bytes, 256-byte aligned. */
nsa_status nsa_select_blocks(const nsa_config *cfg, const void *q, const void *cmp_k, float *scores_out,
                             int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* Full NSA forward for every position of every sequence: the three branches
 * over the same queries combined by per-head gates (deepdaiv newsletter,
 * paragraphs on token compression, token selection and the sliding window;
 * valuable12.com section II for l=32, d=16, l'=64, n=16, w=512), i.e. S2, S3
 * (unless idx_in is given), S4 as defined above.  idx_in: if non-NULL, these block lists
 * ([B][Hkv][T][n]) replace the selection.  idx_out / scores_out: optional
 * copies of the indices used / the scores (scores exist only when
 * selecting).  cmp_k/cmp_v as written by nsa_compress_kv.  The workspace
 * (nsa_workspace_bytes(cfg, NSA_OP_FORWARD) bytes, 256-byte aligned) holds
 * o_cmp, the repacked K/V blocks and, when not supplied by the caller, scores
 * and indices. */
nsa_status nsa_forward(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                       const void *cmp_v, const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                       int32_t *idx_out, float *scores_out, void *ws, size_t ws_bytes, void *stream);

/* nsa_forward for training: the same results, and each branch's softmax
 * statistics saved for the backward calls below.  The branches and their
 * softmaxes are nsa_forward's; keeping a softmax's row statistics so that its
 * backward need not recompute them is the FlashAttention practice.  For
 * branch c (0 compressed, 1 selected, 2 window), row t of
 * sequence b and query head h:
 *   lse      [3][B][T][Hq] fp32: the natural log of sum_i exp(scale q.K_i)
 *            over the branch's keys, -inf when the branch has none (the
 *            compressed branch for t < 31, or an index list with no valid
 *            block)
 *   o_branch [3][B][T][Hq][dv] config dtype: the branch's normalised output
 *            before gating (0 where lse is -inf)
 * so o = sum_c g_c o_branch[c] up to rounding.  Both are required (NULL:
 * NSA_ERR_NULL) and 16-byte aligned; every element is written.  Workspace
 * as nsa_forward (NSA_OP_FORWARD). */
nsa_status nsa_forward_train(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                             const void *cmp_v, const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                             int32_t *idx_out, float *scores_out, float *lse, void *o_branch, void *ws,
                             size_t ws_bytes, void *stream);

/* One decode step for B sequences (valuable12.com section III.3: at 64k
 * context a step reads 5,632 tokens' keys and values instead of 65,536).
 * cfg->T is the cache capacity.  Sequence b holds seq_lens[b] tokens
 * (device int32 [B], each in 1..T; values outside are clamped into that
 * range); its new query q[b] ([B][Hq][dk]) is the last cached token, so the
 * row computed is the forward row t = seq_lens[b]-1 over the caches
 * k_cache/v_cache ([B][Hkv][T][dk|dv]) and the compressed caches
 * cmp_k/cmp_v ([B][Hkv][N_pad][dk|dv], complete for every block with
 * 16i+31 < seq_lens[b]).  o: [B][Hq][dv]; idx_in/idx_out: [B][Hkv][n]. */
nsa_status nsa_decode_step(const nsa_config *cfg, const int32_t *seq_lens, const void *q, const void *k_cache,
                           const void *v_cache, const void *cmp_k, const void *cmp_v, const void *w_g,
                           const void *b_g, const int32_t *idx_in, void *o, int32_t *idx_out, void *ws,
                           size_t ws_bytes, void *stream);

/* nsa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation).  It allocates nothing: the workspace is
 * a 32 MiB array in the library's device memory, one per device the library
 * runs on, held until the process ends.  Arguments, results and errors as
 * nsa_decode_step; NSA_ERR_WORKSPACE when nsa_workspace_bytes(cfg,
 * NSA_OP_DECODE) exceeds 32 MiB (at 65,536-token caches, 16 heads per KV
 * head and d_v = 128, more than 192 (sequence, KV head) pairs); NSA_ERR_HIP
 * if the array's address cannot be looked up.  Every call on a device uses
 * the same array, so calls that overlap on one device (two streams, two host
 * threads) race; calls ordered on one stream do not. */
nsa_status nsa_decode_step_noalloc(const nsa_config *cfg, const int32_t *seq_lens, const void *q,
                                   const void *k_cache, const void *v_cache, const void *cmp_k, const void *cmp_v,
                                   const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                                   int32_t *idx_out, void *stream);

/* Backward pass of the prefill forward (deepdaiv newsletter, on native
 * trainability: the sparse pattern is learned in training, so gradients flow
 * through the three branches, the compression maps and the gates).  With
 * L = sum(d_o * o) for the forward output o computed from these inputs and
 * the block lists idx (held fixed: the selection is piecewise constant and
 * passes no gradient to the importance scores), the call writes
 *   d_q [B][T][Hq][dk], d_k [B][Hkv][T][dk], d_v [B][Hkv][T][dv]   config dtype
 *   d_wck [dk][32*dk], d_pek [32][dk], d_wcv [dv][32*dv], d_pev [32][dv],
 *   d_wg [Hq][3][dk], d_bg [Hq][3]                                  fp32
 * (every element is written; nothing is accumulated into).  cmp_k / cmp_v
 * must be what nsa_compress_kv makes of k / v with these maps: the gradient
 * treats their bf16 rounding as the identity.  idx is what nsa_forward used
 * (its idx_out, or the idx_in given to it); d_o [B][T][Hq][dv] config dtype.
 * The result is deterministic (no floating-point atomics).
 * lse_saved, o_saved: both NULL, or both the lse and o_branch that
 * nsa_forward_train wrote for these inputs and this idx (one without the
 * other: NSA_ERR_NULL).  With them the backward reads each branch's
 * log-sum-exp and d_o . o_branch instead of recomputing them (the 16-head,
 * bf16 configurations at d_k/d_v = 192/128, 128/128, 64/64; others ignore
 * them); the gradients agree with the recomputing call to rounding.
 * ws: nsa_workspace_bytes(cfg, NSA_OP_BACKWARD) bytes.  B*H_kv <= 65535. */
nsa_status nsa_backward(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                        const void *cmp_v, const void *w_ck, const void *pe_k, const void *w_cv, const void *pe_v,
                        const void *w_g, const void *b_g, const int32_t *idx, const void *d_o, void *d_q,
                        void *d_k, void *d_v, float *d_wck, float *d_pek, float *d_wcv, float *d_pev,
                        float *d_wg, float *d_bg, const float *lse_saved, const void *o_saved, void *ws,
                        size_t ws_bytes, void *stream);

/* Backward pass with the two-layer compression map of nsa_compress_kv_mlp
 * (deepdaiv newsletter: a small network summarises each block, and the
 * method is trained natively, so gradients reach that network's weights).
 * As nsa_backward, with cmp_k / cmp_v what nsa_compress_kv_mlp makes of k / v
 * with w1_k, pe_k, w2_k, w1_v, pe_v, w2_v (shapes as there), and
 *   d_w1k [dk][32*dk], d_pek [32][dk], d_w2k [dk][dk],
 *   d_w1v [dv][32*dv], d_pev [32][dv], d_w2v [dv][dv]              fp32
 * in place of the linear map's gradients.  The hidden layer is recomputed;
 * its bf16 rounding and the output's are treated as the identity, and the
 * ReLU's derivative is taken as 0 at 0.  Deterministic.  lse_saved,
 * o_saved as in nsa_backward.  ws: nsa_workspace_bytes(cfg,
 * NSA_OP_BACKWARD_MLP) bytes (nsa_backward's plus the hidden layers and their
 * gradient), 256-byte aligned.  B*H_kv <= 65535. */
nsa_status nsa_backward_mlp(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                            const void *cmp_v, const void *w1_k, const void *pe_k, const void *w2_k,
                            const void *w1_v, const void *pe_v, const void *w2_v, const void *w_g, const void *b_g,
                            const int32_t *idx, const void *d_o, void *d_q, void *d_k, void *d_v, float *d_w1k,
                            float *d_pek, float *d_w2k, float *d_w1v, float *d_pev, float *d_w2v, float *d_wg,
                            float *d_bg, const float *lse_saved, const void *o_saved, void *ws, size_t ws_bytes,
                            void *stream);

/* DSA-style decode step (DSA explainer, allinfo.ai.kr, section "쉽게
 * 이해하기": a lightning indexer with several small heads and one key per
 * token shared by the heads scores every cached token by a weighted sum of
 * ReLU dot products; a selector keeps the top-k tokens (2,048 on the page)
 * for each query; attention runs over the selected tokens only, the softmax
 * denominator summed over that set).  One query per sequence, the token at
 * t = clamp(seq_lens[b], 1, T) - 1; the cached tokens s <= t are candidates.
 *   I[b][s] = sum_{j<idx_heads} w_idx[b][j] * max(q_idx[b][j] . k_idx[b][s], 0)
 *   sel[b]  = the topk positions with the highest I (equal scores: the lower
 *             position first; all of them when t + 1 <= topk), ascending,
 *             -1 padded; one selection per sequence, shared by every head
 *   o[b][h] = sum_{s in sel[b]} softmax_s(scale q[b][h] . k[b][g][s]) v[b][g][s],
 *             g = h / group
 * cfg: B, T (cache capacity), H_kv, group, d_k, d_v, scale and dtype are
 * used (the NSA fields must still be valid); supported: bf16, group = 16,
 * (d_k, d_v) = (192, 128), (128, 128) or (64, 64), else NSA_ERR_SHAPE.
 * idx_heads 1..16, idx_dim 8..256 (a multiple of 8), topk 1..8192, else
 * NSA_ERR_PARAM.  Layouts (bf16): q_idx [B][idx_heads][idx_dim], w_idx
 * [B][idx_heads], k_idx [B][T][idx_dim], q [B][Hq][d_k], k [B][H_kv][T][d_k],
 * v [B][H_kv][T][d_v], o [B][Hq][d_v]; seq_lens device int32 [B]; sel
 * device int32 [B][topk].  fp32 arithmetic.  With sel_in (a selection as
 * above: entries -1 or positions below seq_lens[b]; entries outside 0..T-1
 * count as -1) the indexer and selector are skipped and q_idx, w_idx, k_idx,
 * sel_out and ws may be NULL; otherwise sel_out receives the selection and
 * ws holds nsa_workspace_bytes(cfg, NSA_OP_DSA_DECODE) bytes.  A non-NULL ws
 * must be 256-byte aligned (else NSA_ERR_ALIGN).  A ws of at least
 * 4*B*H_kv*S*(32 + 16*d_v) bytes also serves the attention: each KV group's
 * slots are then split over S workgroups and merged, which changes only the
 * fp32 summation order; S = 4 when ws holds that much (always the case with
 * the size nsa_workspace_bytes reports), else S = 2 when it holds that much;
 * with sel_in and a NULL or smaller ws one workgroup takes each KV group.
 * q_idx, k_idx, q, k, v, o 16-byte aligned. */
nsa_status nsa_dsa_decode(const nsa_config *cfg, int32_t idx_heads, int32_t idx_dim, int32_t topk,
                          const int32_t *seq_lens, const void *q_idx, const void *w_idx, const void *k_idx,
                          const void *q, const void *k, const void *v, const int32_t *sel_in, int32_t *sel_out,
                          void *o, void *ws, size_t ws_bytes, void *stream);

/* DSA-style attention for every position of B sequences of T tokens (the
 * prefill form of nsa_dsa_decode: the same indexer, selector and attention,
 * each position t a query whose candidates are the tokens s <= t of its own
 * sequence; the DSA explainer (allinfo.ai.kr) has the selection made for each
 * query position independently).  Layouts (bf16): q_idx [B][T][idx_heads]
 * [idx_dim], w_idx [B][T][idx_heads], k_idx [B][T][idx_dim], q [B][T][Hq][d_k],
 * k [B][H_kv][T][d_k], v [B][H_kv][T][d_v], o [B][T][Hq][d_v]; sel device
 * int32 [B][T][topk] (ascending, -1 padded: position t has min(t + 1, topk)
 * entries).  Shapes, sizes, sel_in and alignment as nsa_dsa_decode; ws holds
 * nsa_workspace_bytes(cfg, NSA_OP_DSA_PREFILL) bytes unless sel_in is given:
 * the indexer and selector run over the B*T rows in chunks of
 * min(B*T, floor(2^28 / (4*T))) rows, one chunk's fp32 scores at a time, so
 * the workspace stays within 256 MiB whatever B and T are; the result does
 * not depend on the chunking.  B*T*H_kv < 2^31. */
nsa_status nsa_dsa_prefill(const nsa_config *cfg, int32_t idx_heads, int32_t idx_dim, int32_t topk, const void *q_idx,
                           const void *w_idx, const void *k_idx, const void *q, const void *k, const void *v,
                           const int32_t *sel_in, int32_t *sel_out, void *o, void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *nsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
