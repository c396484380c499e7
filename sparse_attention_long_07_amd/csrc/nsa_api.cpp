// C ABI of libnsa: argument checks, workspace layout and launch order.
// Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <math.h>
#include <string.h>

#include <initializer_list>

#include "nsa_internal.h"

using namespace nsa;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

nsa_status check_config(const nsa_config *c, Dims *out)
{
    if (!c) return NSA_ERR_NULL;
    if (c->dtype != NSA_FP32 && c->dtype != NSA_BF16) return NSA_ERR_DTYPE;
    if (c->B < 1 || c->T < 1 || c->T > 524288 || c->H_kv < 1 || c->group < 1 || c->group > 16)
        return NSA_ERR_SHAPE;
    if (c->d_k < 8 || c->d_k > 256 || c->d_k % 8 || c->d_v < 8 || c->d_v > 256 || c->d_v % 8)
        return NSA_ERR_SHAPE;
    if ((long)c->B * c->H_kv * c->group > (1L << 20)) return NSA_ERR_SHAPE;
    if (c->l != 32 || c->d != 16 || c->l_sel != 64) return NSA_ERR_PARAM;
    if (c->n < 3 || c->n > 16 || c->w < 1 || c->w > 8192) return NSA_ERR_PARAM;
    if (!(c->scale >= 0.f) || isinf(c->scale)) return NSA_ERR_PARAM;
    if (out) {
        Dims &d = *out;
        d.B = c->B;
        d.T = c->T;
        d.Hkv = c->H_kv;
        d.G = c->group;
        d.Hq = c->H_kv * c->group;
        d.dk = c->d_k;
        d.dv = c->d_v;
        d.n = c->n;
        d.w = c->w;
        d.ncmp = c->T < 32 ? 0 : (c->T - 32) / 16 + 1;
        d.npad = d.ncmp <= 64 ? 64 : (d.ncmp + 63) / 64 * 64;
        d.nb = (c->T + 63) / 64;
        d.scale = c->scale > 0.f ? c->scale : 1.f / sqrtf((float)c->d_k);
        d.dtype = c->dtype;
    }
    return NSA_OK;
}

// Workspace regions (each 256-byte aligned), for R rows per sequence:
//   ocmp   [B][R][Hq][dv]  storage dtype  compressed-branch output
//   scores [B][Hkv][R][nb] fp32  importance scores (when the caller passes none)
//   idx    [B][Hkv][R][n]  int32 selected blocks (when the caller passes none)
//   vt     V^T per 64-token block, for the matrix-core sparse stage (prefill)
struct Layout {
    size_t ocmp, scores, idx, vt, total;
};

Layout layout(const Dims &d, long R)
{
    Layout L;
    size_t off = 0;
    L.ocmp = off;
    off = align_up(off + (d.dtype == NSA_FP32 ? 4 : 2) * (size_t)d.B * R * d.Hq * d.dv);
    L.scores = off;
    off = align_up(off + sizeof(float) * (size_t)d.B * d.Hkv * R * d.nb);
    L.idx = off;
    off = align_up(off + sizeof(int32_t) * (size_t)d.B * d.Hkv * R * d.n);
    L.vt = off;
    if (R == d.T && sparse_mfma_supported(d)) off = align_up(off + sparse_mfma_ws_bytes(d));
    L.total = off;
    return L;
}

nsa_status check_ws(const Dims &d, long R, void *ws, size_t ws_bytes, Layout *L)
{
    *L = layout(d, R);
    if (!ws || ws_bytes < L->total) return NSA_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    return NSA_OK;
}

nsa_status hip_status(hipError_t e) { return e == hipSuccess ? NSA_OK : NSA_ERR_HIP; }

#define NSA_TRY(expr)                              \
    do {                                           \
        nsa_status st_ = hip_status(expr);         \
        if (st_ != NSA_OK) return st_;             \
    } while (0)

RowArgs row_args(const Dims &d, long R)
{
    RowArgs a;
    memset(&a, 0, sizeof a);
    a.d = d;
    a.R = (int)R;
    return a;
}

// Row arguments of a prefill call: every position of every sequence.
RowArgs prefill_args(const Dims &d, const void *q)
{
    RowArgs a = row_args(d, d.T);
    a.q = q;
    a.q_sb = (long)d.T * d.Hq * d.dk;
    a.q_sr = (long)d.Hq * d.dk;
    a.o_sb = (long)d.T * d.Hq * d.dv;
    a.o_sr = (long)d.Hq * d.dv;
    return a;
}

// S2 and the window half of S4 as one kernel
bool cmp_window_fused(const Dims &d) { return cmp_attn_mfma_supported(d) && sparse_mfma_supported(d); }

bool all_aligned(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!aligned16(p)) return false;
    return true;
}

}  // namespace

extern "C" {

size_t nsa_workspace_bytes(const nsa_config *cfg, int op)
{
    Dims d;
    if (check_config(cfg, &d) != NSA_OK) return 0;
    switch (op) {
    case NSA_OP_FORWARD:
    case NSA_OP_SELECT:
        return layout(d, d.T).total;
    case NSA_OP_DECODE:
        return decode_mfma_supported(d) ? decode_mfma_layout(d, nullptr, nullptr) : layout(d, 1).total;
    case NSA_OP_SPARSE:
        return sparse_mfma_supported(d) ? align_up(sparse_mfma_ws_bytes(d)) : 0;
    case NSA_OP_BACKWARD:
        return backward_layout(d, nullptr, nullptr);
    case NSA_OP_BACKWARD_MLP:
        return backward_layout(d, nullptr, nullptr, true);
    case NSA_OP_CMP_WINDOW:
        return cmp_window_fused(d) ? 0 : align_up((d.dtype == NSA_FP32 ? 4 : 2) * (size_t)d.B * d.T * d.Hq * d.dv);
    case NSA_OP_DSA_DECODE:
        // the indexer scores, later reused for the split attention's partials
        return dsa_supported(d) ? align_up(std::max(sizeof(float) * (size_t)d.B * d.T, dsa_split_bytes(d, kDsaMaxSplit)))
                                : 0;
    case NSA_OP_DSA_PREFILL:
        // the indexer scores of one chunk of rows
        return dsa_supported(d) ? align_up(sizeof(float) * (size_t)dsa_prefill_chunk_rows(d) * d.T) : 0;
    default:
        return 0;
    }
}

nsa_status nsa_compress_kv(const nsa_config *cfg, const void *k, const void *v, const void *w_ck, const void *pe_k,
                           const void *w_cv, const void *pe_v, void *cmp_k, void *cmp_v, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!k || !v || !w_ck || !pe_k || !w_cv || !pe_v || !cmp_k || !cmp_v) return NSA_ERR_NULL;
    const void *ptrs[] = {k, v, w_ck, pe_k, w_cv, pe_v, cmp_k, cmp_v};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (compress_bf16_supported(d)) {
        NSA_TRY(launch_compress_bf16(d, k, v, w_ck, pe_k, w_cv, pe_v, cmp_k, cmp_v, s));
        return NSA_OK;
    }
    NSA_TRY(launch_compress_generic(d, k, w_ck, pe_k, cmp_k, d.dk, s));
    NSA_TRY(launch_compress_generic(d, v, w_cv, pe_v, cmp_v, d.dv, s));
    return NSA_OK;
}

nsa_status nsa_compress_kv_mlp(const nsa_config *cfg, const void *k, const void *v, const void *w1_k,
                               const void *pe_k, const void *w2_k, const void *w1_v, const void *pe_v,
                               const void *w2_v, void *cmp_k, void *cmp_v, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!k || !v || !w1_k || !pe_k || !w2_k || !w1_v || !pe_v || !w2_v || !cmp_k || !cmp_v) return NSA_ERR_NULL;
    const void *ptrs[] = {k, v, w1_k, pe_k, w2_k, w1_v, pe_v, w2_v, cmp_k, cmp_v};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    // first layer: the linear compression with W1, pre-activations in cmp_k / cmp_v
    if (compress_bf16_supported(d)) {
        NSA_TRY(launch_compress_bf16(d, k, v, w1_k, pe_k, w1_v, pe_v, cmp_k, cmp_v, s));
    } else {
        NSA_TRY(launch_compress_generic(d, k, w1_k, pe_k, cmp_k, d.dk, s));
        NSA_TRY(launch_compress_generic(d, v, w1_v, pe_v, cmp_v, d.dv, s));
    }
    // second layer in place
    NSA_TRY(launch_compress_mlp2(d, w2_k, w2_v, cmp_k, cmp_v, s));
    return NSA_OK;
}

nsa_status nsa_dsa_decode(const nsa_config *cfg, int32_t idx_heads, int32_t idx_dim, int32_t topk,
                          const int32_t *seq_lens, const void *q_idx, const void *w_idx, const void *k_idx,
                          const void *q, const void *k, const void *v, const int32_t *sel_in, int32_t *sel_out,
                          void *o, void *ws, size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!dsa_supported(d)) return NSA_ERR_SHAPE;
    if (idx_heads < 1 || idx_heads > 16 || idx_dim < 8 || idx_dim > 256 || idx_dim % 8 || topk < 1 || topk > 8192)
        return NSA_ERR_PARAM;
    if (!seq_lens || !q || !k || !v || !o) return NSA_ERR_NULL;
    if (!sel_in && (!q_idx || !w_idx || !k_idx || !sel_out)) return NSA_ERR_NULL;
    const void *ptrs[] = {q, k, v, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    if (!sel_in && (!aligned16(q_idx) || !aligned16(k_idx))) return NSA_ERR_ALIGN;
    if (!sel_in && (!ws || ws_bytes < nsa_workspace_bytes(cfg, NSA_OP_DSA_DECODE))) return NSA_ERR_WORKSPACE;
    if (ws && (uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (!sel_in) {
        NSA_TRY(launch_dsa_select(d, idx_heads, idx_dim, topk, seq_lens, q_idx, w_idx, k_idx, (float *)ws, sel_out, s));
    }
    // a workspace that holds the partial results (the scores are consumed by
    // then, on the same stream) lets four (or two) workgroups share each KV
    // group's slots
    const int ns = !ws ? 1 : ws_bytes >= dsa_split_bytes(d, 4) ? 4 : ws_bytes >= dsa_split_bytes(d, 2) ? 2 : 1;
    NSA_TRY(launch_dsa_attn(d, topk, q, k, v, sel_in ? sel_in : sel_out, o, s, false, ns > 1 ? ws : nullptr, ns));
    return NSA_OK;
}

nsa_status nsa_dsa_prefill(const nsa_config *cfg, int32_t idx_heads, int32_t idx_dim, int32_t topk, const void *q_idx,
                           const void *w_idx, const void *k_idx, const void *q, const void *k, const void *v,
                           const int32_t *sel_in, int32_t *sel_out, void *o, void *ws, size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!dsa_supported(d) || (long)d.B * d.T * d.Hkv >= (1L << 31)) return NSA_ERR_SHAPE;
    if (idx_heads < 1 || idx_heads > 16 || idx_dim < 8 || idx_dim > 256 || idx_dim % 8 || topk < 1 || topk > 8192)
        return NSA_ERR_PARAM;
    if (!q || !k || !v || !o) return NSA_ERR_NULL;
    if (!sel_in && (!q_idx || !w_idx || !k_idx || !sel_out)) return NSA_ERR_NULL;
    const void *ptrs[] = {q, k, v, o};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    if (!sel_in && (!aligned16(q_idx) || !aligned16(k_idx))) return NSA_ERR_ALIGN;
    if (!sel_in && (!ws || ws_bytes < nsa_workspace_bytes(cfg, NSA_OP_DSA_PREFILL))) return NSA_ERR_WORKSPACE;
    if (ws && (uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (!sel_in) {
        // the rows in chunks whose scores fit the workspace, in order on the stream
        const int total = d.B * d.T, chunk = dsa_prefill_chunk_rows(d);
        for (int r0 = 0; r0 < total; r0 += chunk)
            NSA_TRY(launch_dsa_select(d, idx_heads, idx_dim, topk, nullptr, q_idx, w_idx, k_idx, (float *)ws, sel_out,
                                      s, true, r0, std::min(chunk, total - r0)));
    }
    NSA_TRY(launch_dsa_attn(d, topk, q, k, v, sel_in ? sel_in : sel_out, o, s, true));
    return NSA_OK;
}

nsa_status nsa_compress_append(const nsa_config *cfg, const int32_t *len_old, const int32_t *len_new,
                               int32_t max_append, const void *k_cache, const void *v_cache, const void *w_ck,
                               const void *pe_k, const void *w_cv, const void *pe_v, void *cmp_k, void *cmp_v,
                               void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!len_new || !k_cache || !v_cache || !w_ck || !pe_k || !w_cv || !pe_v || !cmp_k || !cmp_v)
        return NSA_ERR_NULL;
    if (max_append < 1 || max_append > d.T) return NSA_ERR_PARAM;
    const void *ptrs[] = {k_cache, v_cache, w_ck, pe_k, w_cv, pe_v, cmp_k, cmp_v};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    // appending a tokens completes at most a/16 + 1 blocks (capped by the cache)
    const int max_blocks = std::min(max_append / 16 + 1, d.npad);
    if (compress_bf16_supported(d)) {
        NSA_TRY(launch_compress_bf16(d, k_cache, v_cache, w_ck, pe_k, w_cv, pe_v, cmp_k, cmp_v, s, len_old, len_new,
                                     max_blocks));
        return NSA_OK;
    }
    const int tiles = (max_blocks + 63) / 64;
    NSA_TRY(launch_compress_generic(d, k_cache, w_ck, pe_k, cmp_k, d.dk, s, len_old, len_new, tiles));
    NSA_TRY(launch_compress_generic(d, v_cache, w_cv, pe_v, cmp_v, d.dv, s, len_old, len_new, tiles));
    return NSA_OK;
}

nsa_status nsa_compress_append_mlp(const nsa_config *cfg, const int32_t *len_old, const int32_t *len_new,
                                   int32_t max_append, const void *k_cache, const void *v_cache, const void *w1_k,
                                   const void *pe_k, const void *w2_k, const void *w1_v, const void *pe_v,
                                   const void *w2_v, void *cmp_k, void *cmp_v, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!len_new || !k_cache || !v_cache || !w1_k || !pe_k || !w2_k || !w1_v || !pe_v || !w2_v || !cmp_k || !cmp_v)
        return NSA_ERR_NULL;
    if (max_append < 1 || max_append > d.T) return NSA_ERR_PARAM;
    const void *ptrs[] = {k_cache, v_cache, w1_k, pe_k, w2_k, w1_v, pe_v, w2_v, cmp_k, cmp_v};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const int max_blocks = std::min(max_append / 16 + 1, d.npad);
    // first layer: the linear append with W1 (pre-activations of the new blocks)
    if (compress_bf16_supported(d)) {
        NSA_TRY(launch_compress_bf16(d, k_cache, v_cache, w1_k, pe_k, w1_v, pe_v, cmp_k, cmp_v, s, len_old, len_new,
                                     max_blocks));
    } else {
        const int tiles = (max_blocks + 63) / 64;
        NSA_TRY(launch_compress_generic(d, k_cache, w1_k, pe_k, cmp_k, d.dk, s, len_old, len_new, tiles));
        NSA_TRY(launch_compress_generic(d, v_cache, w1_v, pe_v, cmp_v, d.dv, s, len_old, len_new, tiles));
    }
    // second layer on the same rows only
    NSA_TRY(launch_compress_mlp2(d, w2_k, w2_v, cmp_k, cmp_v, s, len_old, len_new, max_blocks));
    return NSA_OK;
}

nsa_status nsa_compressed_attention(const nsa_config *cfg, const void *q, const void *cmp_k, const void *cmp_v,
                                    void *o_cmp, float *scores, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !cmp_k || !scores || (!cmp_v) != (!o_cmp)) return NSA_ERR_NULL;
    if (!all_aligned({q, cmp_k, cmp_v, o_cmp, scores})) return NSA_ERR_ALIGN;
    RowArgs a = prefill_args(d, q);
    a.kc = cmp_k;
    a.vc = cmp_v;
    a.ocmp = o_cmp;
    a.scores = scores;
    if (cmp_attn_mfma_supported(d))
        return hip_status(launch_cmp_attn_mfma(a, o_cmp != nullptr, (hipStream_t)stream));
    return hip_status(launch_cmp_attn_generic(a, o_cmp != nullptr, (hipStream_t)stream));
}

nsa_status nsa_compressed_window_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                           const void *cmp_k, const void *cmp_v, const void *w_g, const void *b_g,
                                           float *scores, void *o, void *o_cmp, void *ws, size_t ws_bytes,
                                           void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !k || !v || !cmp_k || !cmp_v || !w_g || !b_g || !scores || !o) return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, cmp_k, cmp_v, w_g, b_g, scores, o, o_cmp})) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    RowArgs a = prefill_args(d, q);
    a.kc = cmp_k;
    a.vc = cmp_v;
    a.scores = scores;
    a.k = k;
    a.v = v;
    a.wg = w_g;
    a.bg = b_g;
    a.o = o;
    a.ocmp = o_cmp;
    if (cmp_window_fused(d)) return hip_status(launch_cmp_win_mfma(a, s));
    if (!o_cmp) {
        if (!ws || ws_bytes < nsa_workspace_bytes(cfg, NSA_OP_CMP_WINDOW)) return NSA_ERR_WORKSPACE;
        if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
        a.ocmp = ws;
    }
    if (cmp_attn_mfma_supported(d)) NSA_TRY(launch_cmp_attn_mfma(a, true, s));
    else NSA_TRY(launch_cmp_attn_generic(a, true, s));
    a.part = 1;
    if (sparse_mfma_supported(d)) return hip_status(launch_sparse_mfma(a, nullptr, s));
    return hip_status(launch_sparse_generic(a, s));
}

nsa_status nsa_select_topn(const nsa_config *cfg, const float *scores, int32_t *idx, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!scores || !idx) return NSA_ERR_NULL;
    if (!all_aligned({scores, idx})) return NSA_ERR_ALIGN;
    RowArgs a = prefill_args(d, nullptr);
    a.scores = (float *)scores;
    a.idx_sel = idx;
    return hip_status(launch_select_generic(a, (hipStream_t)stream));
}

nsa_status nsa_sparse_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                const void *o_cmp, const int32_t *idx, const void *w_g, const void *b_g, void *o,
                                void *ws, size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !k || !v || !o_cmp || !idx || !w_g || !b_g || !o) return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, o_cmp, idx, w_g, b_g, o})) return NSA_ERR_ALIGN;
    const bool mfma = sparse_mfma_supported(d);
    if (mfma) {
        if (!ws || ws_bytes < sparse_mfma_ws_bytes(d)) return NSA_ERR_WORKSPACE;
        if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    }
    RowArgs a = prefill_args(d, q);
    a.k = k;
    a.v = v;
    a.ocmp = (void *)o_cmp;
    a.idx = idx;
    a.wg = w_g;
    a.bg = b_g;
    a.o = o;
    if (mfma) return hip_status(launch_sparse_mfma(a, ws, (hipStream_t)stream));
    return hip_status(launch_sparse_generic(a, (hipStream_t)stream));
}

nsa_status nsa_pack_kv_blocks(const nsa_config *cfg, const void *k, const void *v, void *ws, size_t ws_bytes,
                              void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!k || !v) return NSA_ERR_NULL;
    if (!all_aligned({k, v})) return NSA_ERR_ALIGN;
    if (!sparse_mfma_supported(d)) return NSA_OK;     // the generic path reads K and V as they are
    if (!ws || ws_bytes < sparse_mfma_ws_bytes(d)) return NSA_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    RowArgs a = prefill_args(d, nullptr);
    a.k = k;
    a.v = v;
    a.part = 3;
    return hip_status(launch_sparse_mfma(a, ws, (hipStream_t)stream));
}

nsa_status nsa_window_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                const void *o_cmp, const void *w_g, const void *b_g, void *o, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !k || !v || !o_cmp || !w_g || !b_g || !o) return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, o_cmp, w_g, b_g, o})) return NSA_ERR_ALIGN;
    RowArgs a = prefill_args(d, q);
    a.k = k;
    a.v = v;
    a.ocmp = (void *)o_cmp;
    a.wg = w_g;
    a.bg = b_g;
    a.o = o;
    a.part = 1;
    if (sparse_mfma_supported(d)) return hip_status(launch_sparse_mfma(a, nullptr, (hipStream_t)stream));
    return hip_status(launch_sparse_generic(a, (hipStream_t)stream));
}

nsa_status nsa_selected_attention(const nsa_config *cfg, const void *q, const void *k, const void *v,
                                  const int32_t *idx, const void *w_g, const void *b_g, void *o, void *ws,
                                  size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !k || !v || !idx || !w_g || !b_g || !o) return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, idx, w_g, b_g, o})) return NSA_ERR_ALIGN;
    const bool mfma = sparse_mfma_supported(d);
    if (mfma) {
        if (!ws || ws_bytes < sparse_mfma_ws_bytes(d)) return NSA_ERR_WORKSPACE;
        if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    }
    RowArgs a = prefill_args(d, q);
    a.k = k;
    a.v = v;
    a.idx = idx;
    a.wg = w_g;
    a.bg = b_g;
    a.o = o;
    a.part = 2;
    if (mfma) return hip_status(launch_sparse_mfma(a, ws, (hipStream_t)stream));
    return hip_status(launch_sparse_generic(a, (hipStream_t)stream));
}

nsa_status nsa_select_blocks(const nsa_config *cfg, const void *q, const void *cmp_k, float *scores_out,
                             int32_t *idx_out, void *ws, size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !cmp_k || !idx_out) return NSA_ERR_NULL;
    if (!all_aligned({q, cmp_k, scores_out, idx_out})) return NSA_ERR_ALIGN;
    Layout L;
    if ((st = check_ws(d, d.T, ws, ws_bytes, &L)) != NSA_OK) return st;
    float *scores = scores_out ? scores_out : (float *)((char *)ws + L.scores);
    if ((st = nsa_compressed_attention(cfg, q, cmp_k, nullptr, nullptr, scores, stream)) != NSA_OK) return st;
    return nsa_select_topn(cfg, scores, idx_out, stream);
}

// The prefill forward; with lse and o_branch (both or neither) it also saves
// each branch's log-sum-exp and output for the backward.
static nsa_status forward_impl(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                               const void *cmp_v, const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                               int32_t *idx_out, float *scores_out, float *lse, void *o_branch, void *ws,
                               size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!q || !k || !v || !cmp_k || !cmp_v || !w_g || !b_g || !o) return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out, scores_out, lse, o_branch}))
        return NSA_ERR_ALIGN;
    Layout L;
    if ((st = check_ws(d, d.T, ws, ws_bytes, &L)) != NSA_OK) return st;
    char *w = (char *)ws;
    hipStream_t s = (hipStream_t)stream;
    // with saved statistics the compressed-branch output goes to its slot
    void *ocmp = o_branch ? o_branch : (void *)(w + L.ocmp);
    float *scores = scores_out ? scores_out : (float *)(w + L.scores);
    // matrix-core shapes: the window half of S4 runs inside the S2 launch,
    // which then writes o_cmp only into the saved statistics
    const bool fused = cmp_window_fused(d);
    {
        RowArgs a = prefill_args(d, q);
        a.kc = cmp_k;
        a.vc = cmp_v;
        a.ocmp = ocmp;
        a.scores = scores;
        a.lse = lse;
        if (fused) {
            a.ocmp = o_branch;
            a.k = k;
            a.v = v;
            a.wg = w_g;
            a.bg = b_g;
            a.o = o;
            a.osave = o_branch;
            NSA_TRY(launch_cmp_win_mfma(a, s));
        } else if (cmp_attn_mfma_supported(d)) {
            NSA_TRY(launch_cmp_attn_mfma(a, true, s));
        } else {
            NSA_TRY(launch_cmp_attn_generic(a, true, s));
        }
    }
    const int32_t *idx = idx_in;
    if (idx_in) {
        if (idx_out)
            NSA_TRY(hipMemcpyAsync(idx_out, idx_in, sizeof(int32_t) * (size_t)d.B * d.Hkv * d.T * d.n,
                                   hipMemcpyDeviceToDevice, s));
    } else {
        int32_t *sel = idx_out ? idx_out : (int32_t *)(w + L.idx);
        if ((st = nsa_select_topn(cfg, scores, sel, stream)) != NSA_OK) return st;
        idx = sel;
    }
    RowArgs a = prefill_args(d, q);
    a.k = k;
    a.v = v;
    a.ocmp = ocmp;
    a.idx = idx;
    a.wg = w_g;
    a.bg = b_g;
    a.o = o;
    a.lse = lse;
    a.osave = o_branch;
    if (fused) {   // the window half is done: pack the K/V blocks, then the selected half
        a.part = 3;
        NSA_TRY(launch_sparse_mfma(a, w + L.vt, s));
        a.part = 2;
        return hip_status(launch_sparse_mfma(a, w + L.vt, s));
    }
    if (sparse_mfma_supported(d)) return hip_status(launch_sparse_mfma(a, w + L.vt, s));
    return hip_status(launch_sparse_generic(a, s));
}

nsa_status nsa_forward(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                       const void *cmp_v, const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                       int32_t *idx_out, float *scores_out, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(cfg, q, k, v, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out, scores_out, nullptr, nullptr, ws,
                        ws_bytes, stream);
}

nsa_status nsa_forward_train(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                             const void *cmp_v, const void *w_g, const void *b_g, const int32_t *idx_in, void *o,
                             int32_t *idx_out, float *scores_out, float *lse, void *o_branch, void *ws,
                             size_t ws_bytes, void *stream)
{
    if (!lse || !o_branch) {
        Dims d;
        const nsa_status st = check_config(cfg, &d);
        return st != NSA_OK ? st : NSA_ERR_NULL;
    }
    return forward_impl(cfg, q, k, v, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out, scores_out, lse, o_branch, ws,
                        ws_bytes, stream);
}

nsa_status nsa_decode_step(const nsa_config *cfg, const int32_t *seq_lens, const void *q, const void *k_cache,
                           const void *v_cache, const void *cmp_k, const void *cmp_v, const void *w_g,
                           const void *b_g, const int32_t *idx_in, void *o, int32_t *idx_out, void *ws,
                           size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if (!seq_lens || !q || !k_cache || !v_cache || !cmp_k || !cmp_v || !w_g || !b_g || !o) return NSA_ERR_NULL;
    const void *ptrs[] = {seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in, o, idx_out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return NSA_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (decode_mfma_supported(d)) {
        if (!ws || ws_bytes < decode_mfma_layout(d, nullptr, nullptr)) return NSA_ERR_WORKSPACE;
        if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
        DecArgs A;
        memset(&A, 0, sizeof A);
        A.d = d;
        A.seq_lens = seq_lens;
        A.q = q;
        A.k = k_cache;
        A.v = v_cache;
        A.kc = cmp_k;
        A.vc = cmp_v;
        A.wg = w_g;
        A.bg = b_g;
        A.idx_in = idx_in;
        A.o = o;
        decode_mfma_layout(d, ws, &A);
        if (idx_out && !idx_in) A.idx = idx_out;
        NSA_TRY(launch_decode_mfma(A, s));
        if (idx_out && idx_in)
            NSA_TRY(hipMemcpyAsync(idx_out, idx_in, sizeof(int32_t) * (size_t)d.B * d.Hkv * d.n,
                                   hipMemcpyDeviceToDevice, s));
        return NSA_OK;
    }
    Layout L;
    if ((st = check_ws(d, 1, ws, ws_bytes, &L)) != NSA_OK) return st;
    char *w = (char *)ws;
    RowArgs a = row_args(d, 1);
    a.seq_lens = seq_lens;
    a.q = q;
    a.q_sb = (long)d.Hq * d.dk;
    a.q_sr = 0;
    a.k = k_cache;
    a.v = v_cache;
    a.kc = cmp_k;
    a.vc = cmp_v;
    a.wg = w_g;
    a.bg = b_g;
    a.ocmp = w + L.ocmp;
    a.scores = (float *)(w + L.scores);
    a.idx_sel = idx_out ? idx_out : (int32_t *)(w + L.idx);
    a.o = o;
    a.o_sb = (long)d.Hq * d.dv;
    a.o_sr = 0;
    NSA_TRY(launch_cmp_attn_generic(a, true, s));
    if (idx_in) {
        a.idx = idx_in;
        if (idx_out)
            NSA_TRY(hipMemcpyAsync(idx_out, idx_in, sizeof(int32_t) * (size_t)d.B * d.Hkv * d.n,
                                   hipMemcpyDeviceToDevice, s));
    } else {
        NSA_TRY(launch_select_generic(a, s));
        a.idx = a.idx_sel;
    }
    NSA_TRY(launch_sparse_generic(a, s));
    return NSA_OK;
}

nsa_status nsa_backward(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                        const void *cmp_v, const void *w_ck, const void *pe_k, const void *w_cv, const void *pe_v,
                        const void *w_g, const void *b_g, const int32_t *idx, const void *d_o, void *d_q,
                        void *d_k, void *d_v, float *d_wck, float *d_pek, float *d_wcv, float *d_pev,
                        float *d_wg, float *d_bg, const float *lse_saved, const void *o_saved, void *ws,
                        size_t ws_bytes, void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if ((long)d.B * d.Hkv > 65535) return NSA_ERR_SHAPE;
    if (!q || !k || !v || !cmp_k || !cmp_v || !w_ck || !pe_k || !w_cv || !pe_v || !w_g || !b_g || !idx || !d_o ||
        !d_q || !d_k || !d_v || !d_wck || !d_pek || !d_wcv || !d_pev || !d_wg || !d_bg || (!lse_saved) != (!o_saved))
        return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, cmp_k, cmp_v, w_ck, pe_k, w_cv, pe_v, w_g, b_g, idx, d_o, d_q, d_k, d_v, d_wck,
                      d_pek, d_wcv, d_pev, d_wg, d_bg, lse_saved, o_saved}))
        return NSA_ERR_ALIGN;
    const size_t need = backward_layout(d, nullptr, nullptr);
    if (!ws || ws_bytes < need) return NSA_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    BwdArgs A;
    memset(&A, 0, sizeof A);
    A.d = d;
    A.q = q;
    A.k = k;
    A.v = v;
    A.kc = cmp_k;
    A.vc = cmp_v;
    A.wck = w_ck;
    A.pek = pe_k;
    A.wcv = w_cv;
    A.pev = pe_v;
    A.wg = w_g;
    A.bg = b_g;
    A.idx = idx;
    A.dO = d_o;
    A.dq = d_q;
    A.dk = d_k;
    A.dv = d_v;
    A.dwck = d_wck;
    A.dpek = d_pek;
    A.dwcv = d_wcv;
    A.dpev = d_pev;
    A.dwg = d_wg;
    A.dbg = d_bg;
    A.lse_sv = lse_saved;
    A.o_sv = o_saved;
    backward_layout(d, ws, &A);
    return hip_status(launch_backward(A, (hipStream_t)stream));
}

nsa_status nsa_backward_mlp(const nsa_config *cfg, const void *q, const void *k, const void *v, const void *cmp_k,
                            const void *cmp_v, const void *w1_k, const void *pe_k, const void *w2_k,
                            const void *w1_v, const void *pe_v, const void *w2_v, const void *w_g, const void *b_g,
                            const int32_t *idx, const void *d_o, void *d_q, void *d_k, void *d_v, float *d_w1k,
                            float *d_pek, float *d_w2k, float *d_w1v, float *d_pev, float *d_w2v, float *d_wg,
                            float *d_bg, const float *lse_saved, const void *o_saved, void *ws, size_t ws_bytes,
                            void *stream)
{
    Dims d;
    nsa_status st = check_config(cfg, &d);
    if (st != NSA_OK) return st;
    if ((long)d.B * d.Hkv > 65535) return NSA_ERR_SHAPE;
    if (!q || !k || !v || !cmp_k || !cmp_v || !w1_k || !pe_k || !w2_k || !w1_v || !pe_v || !w2_v || !w_g || !b_g ||
        !idx || !d_o || !d_q || !d_k || !d_v || !d_w1k || !d_pek || !d_w2k || !d_w1v || !d_pev || !d_w2v || !d_wg ||
        !d_bg || (!lse_saved) != (!o_saved))
        return NSA_ERR_NULL;
    if (!all_aligned({q, k, v, cmp_k, cmp_v, w1_k, pe_k, w2_k, w1_v, pe_v, w2_v, w_g, b_g, idx, d_o, d_q, d_k, d_v,
                      d_w1k, d_pek, d_w2k, d_w1v, d_pev, d_w2v, d_wg, d_bg, lse_saved, o_saved}))
        return NSA_ERR_ALIGN;
    const size_t need = backward_layout(d, nullptr, nullptr, true);
    if (!ws || ws_bytes < need) return NSA_ERR_WORKSPACE;
    if ((uintptr_t)ws % kAlign) return NSA_ERR_ALIGN;
    BwdArgs A;
    memset(&A, 0, sizeof A);
    A.d = d;
    A.q = q;
    A.k = k;
    A.v = v;
    A.kc = cmp_k;
    A.vc = cmp_v;
    A.wck = w1_k;   // the first layers take the linear map's place
    A.pek = pe_k;
    A.wcv = w1_v;
    A.pev = pe_v;
    A.wg = w_g;
    A.bg = b_g;
    A.idx = idx;
    A.dO = d_o;
    A.dq = d_q;
    A.dk = d_k;
    A.dv = d_v;
    A.dwck = d_w1k;
    A.dpek = d_pek;
    A.dwcv = d_w1v;
    A.dpev = d_pev;
    A.dwg = d_wg;
    A.dbg = d_bg;
    A.mlp = true;
    A.w2k = w2_k;
    A.w2v = w2_v;
    A.dw2k = d_w2k;
    A.dw2v = d_w2v;
    A.lse_sv = lse_saved;
    A.o_sv = o_saved;
    backward_layout(d, ws, &A, true);
    return hip_status(launch_backward(A, (hipStream_t)stream));
}

const char *nsa_status_string(int status)
{
    switch (status) {
    case NSA_OK: return "ok";
    case NSA_ERR_NULL: return "a required pointer is NULL";
    case NSA_ERR_SHAPE: return "a size is out of the supported range";
    case NSA_ERR_DTYPE: return "unsupported dtype";
    case NSA_ERR_PARAM: return "unsupported method parameter (l, d, l_sel, n, w or scale)";
    case NSA_ERR_WORKSPACE: return "workspace missing or too small";
    case NSA_ERR_HIP: return "HIP launch failed";
    case NSA_ERR_ALIGN: return "pointer not aligned as required";
    default: return "unknown status";
    }
}

}  // extern "C"
