// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nsa.h"

namespace nsa {

typedef uint16_t bf16_t;

// bf16 <-> fp32.  bf16 is the upper half of an IEEE single; conversion to
// bf16 rounds to nearest, ties to even (NaN maps to a quiet NaN).
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ bf16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

// Compression blocks complete in a sequence of len tokens: block i covers
// tokens 16i .. 16i+31.
__device__ __forceinline__ int cmp_blocks(int len) { return len >= 32 ? (len - 32) / 16 + 1 : 0; }

// Blocks that an append from len_old[b] to len_new[b] tokens completes, as
// [lo, hi); lengths are clamped to 0 <= len_old <= len_new <= T.
__device__ __forceinline__ void append_range(const int32_t *len_old, const int32_t *len_new, int b, int T, int &lo,
                                             int &hi)
{
    int ln = len_new[b];
    ln = ln < 0 ? 0 : (ln > T ? T : ln);
    int lo_len = len_old ? len_old[b] : 0;
    lo_len = lo_len < 0 ? 0 : (lo_len > ln ? ln : lo_len);
    lo = cmp_blocks(lo_len);
    hi = cmp_blocks(ln);
}

// Resolved problem sizes (from nsa_config after validation).
struct Dims {
    int B, T, Hkv, G, Hq, dk, dv, n, w;
    int ncmp;   // complete compression blocks of a length-T sequence
    int npad;   // compressed slots per (b, h)
    int nb;     // selection blocks, ceil(T/64)
    float scale;
    int dtype;
};

// Arguments of the per-row kernels.  A "row" is one query position of one
// sequence: prefill rows are r = 0..T-1 with t = r; a decode step has one row
// per sequence with t = clamp(seq_lens[b], 1, T) - 1.
struct RowArgs {
    Dims d;
    int R;                      // rows per sequence
    const int32_t *seq_lens;    // decode: device [B]; prefill: nullptr
    const void *q;              // row (b, r) head h at q + b*q_sb + r*q_sr + h*dk
    long q_sb, q_sr;
    const void *k, *v;          // [B][Hkv][T][dk|dv]
    const void *kc, *vc;        // [B][Hkv][npad][dk|dv]
    const void *wg, *bg;        // [Hq][3][dk], [Hq][3]
    void *ocmp;                 // [B][R][Hq][dv] compressed-branch output, storage dtype
    float *scores;              // [B][Hkv][R][nb]
    const int32_t *idx;         // [B][Hkv][R][n] blocks used by the sparse kernel
    int32_t *idx_sel;           // [B][Hkv][R][n] written by the selector
    void *o;                    // row (b, r) head h at o + b*o_sb + r*o_sr + h*dv
    long o_sb, o_sr;
    int part;                   // sparse stage: 0 everything, 1 window (o written), 2 selected from packed blocks
                                // (added to o), 3 pack K/V blocks only
    // Saved statistics for the backward (prefill only), or nullptr: per branch
    // c (0 compressed, 1 selected, 2 window) the natural-log log-sum-exp of
    // its softmax, lse[c][B][R][Hq] (-inf for an empty branch), and its
    // normalised output, osave[c][B][R][Hq][dv] in the storage dtype.  The
    // compressed branch's output is ocmp, which then points at slot 0.
    float *lse;
    void *osave;
};

// Arguments of the matrix-core decode step (one row per sequence).  Each
// (sequence, KV head) pair has nslot = nq + nw + 1 + ns partial slots of
// [16 max][16 sum][16][dv] fp32 (unnormalised outputs): the compressed cache
// in nq ranges, the window in nw ranges, the always-kept selected blocks, the
// other selected blocks in ns groups.
struct DecArgs {
    Dims d;
    const int32_t *seq_lens;      // device [B]
    const void *q, *k, *v;        // q [B][Hq][dk]; caches [B][Hkv][T][dk|dv]
    const void *kc, *vc;          // compressed caches [B][Hkv][npad][dk|dv]
    const void *wg, *bg;
    const int32_t *idx_in;        // [B][Hkv][n] or nullptr
    void *o;                      // [B][Hq][dv]
    int nq, nw, ns, nslot;        // partial slots per pair (see above)
    int cmp_keys;                 // compressed slots per k_dec_cmp workgroup
    int ngrp, nbp;                // 32-slot groups and 4-slot blocks of the compressed cache
    float *part;                  // [pair][nq+nw+ns][32 + 16 dv]
    float *bt;                    // [pair][nbp][16] block-importance terms (see k_decode.hip)
    float *gmax;                  // [pair][ngrp][16] softmax reference of each group's terms
    float *gtail;                 // [pair][ngrp][16] the group's last-slot probability
    float *gates;                 // [pair][16][3]
    int32_t *idx;                 // selection output [B][Hkv][n]
};

// Arguments of the backward pass.
struct BwdArgs {
    Dims d;
    const void *q, *k, *v, *kc, *vc;        // forward inputs (storage dtype)
    const void *wck, *pek, *wcv, *pev, *wg, *bg;
    const int32_t *idx;                     // [B][Hkv][T][n] selection used by the forward
    const void *dO;                         // [B][T][Hq][dv]
    void *dq, *dk, *dv;                     // storage dtype, input layouts
    float *dwck, *dpek, *dwcv, *dpev, *dwg, *dbg;
    // workspace (fp32)
    float *rs;        // [B][T][Hq][3][4] per row, head and branch: lse, D, gate, dz
    float *dk_raw;    // [B][Hkv][T][dk] raw-key gradient from the window and selected branches
    float *dv_raw;    // [B][Hkv][T][dv]
    float *part;      // [nchunk][B*Hkv][npad][dk+dv] compressed K/V gradient per row chunk
    float *kcv;       // [B*Hkv][npad][dk+dv] compressed K/V gradient
    float *colsum;    // [dk+dv] sum of kcv over sequences, heads and blocks
    float *cspart;    // [32][dk+dv] colsum partials per row chunk
    float *gpart;     // [Hq][ngc][3][dk+1] gate gradient per row chunk
    uint32_t *selbm;  // [B*Hkv][NB][ceil(T/32)] bit t of row j: row t selected block j
    float *kpart;     // matrix-core key pass: per row chunk c, [B*Hkv][min(T, (c+1) krc)][dk+dv] partial raw dK, dV
    int nchunk, ngc;
    int krc, nkc;     // rows per chunk and chunks of the matrix-core key pass
    // two-layer compression map (wck/pek/wcv/pev then hold the first layers):
    // the second layers and their gradients, the recomputed hidden layers
    // (storage dtype, [B*Hkv][npad][dk|dv], before the ReLU) and the gradient
    // of the hidden layers (fp32, kcv's layout)
    bool mlp;
    const void *w2k, *w2v;
    float *dw2k, *dw2v;
    void *hk, *hv;
    float *da;
    // the forward's saved statistics (RowArgs::lse, RowArgs::osave layouts,
    // R = T) or nullptr: the row pass then takes lse and dO . o per branch
    // from them instead of sweeping each branch's keys twice
    const float *lse_sv;
    const void *o_sv;
};
// per (row, head) row statistics of the backward: {lse, D, gate, dz} for each
// of the 3 branches (compressed, selected, window)
constexpr int kBwdStat = 12;
// rows per partial of the compressed-key gradient
constexpr int kBwdRowChunk = 1024;
size_t backward_layout(const Dims &d, void *ws, BwdArgs *A, bool mlp = false);   // bytes; carves A's buffers if ws
hipError_t launch_backward(const BwdArgs &A, hipStream_t s);
// raw-key gradients on the matrix cores (bf16, 16 heads per KV head, the
// forward's (d_k, d_v) pairs); needs selbm built and rs filled
bool bwd_keys_mfma_ok(const Dims &d);
void bwd_key_chunks(const Dims &d, int *rc, int *nkc, size_t *part_floats);
hipError_t launch_bwd_keys_mfma(const BwdArgs &A, hipStream_t s);
// compressed-key gradient partials (part) on the matrix cores, same shapes
hipError_t launch_bwd_cmp_keys_mfma(const BwdArgs &A, hipStream_t s);
// weight gradient of the K (isk) or V compression map on the matrix cores,
// same shapes; needs kcv and colsum
hipError_t launch_bwd_dw_mfma(const BwdArgs &A, bool isk, hipStream_t s);
// token gradient of the K (isk) or V compression map on the matrix cores, added
// to the raw-key gradient and stored in the storage dtype (same shapes)
hipError_t launch_bwd_dx_mfma(const BwdArgs &A, bool isk, hipStream_t s);
// the row pass (rs and dq) on the matrix cores, same shapes
hipError_t launch_bwd_rows_mfma(const BwdArgs &A, hipStream_t s);

// Generic kernels: plain VALU code, any supported shape, fp32 or bf16 storage.
// Compression launchers: every block of the T-token sequences when len_new is
// null; otherwise (caches of capacity T) the blocks an append from len_old[b]
// to len_new[b] tokens completes, with `tiles` workgroups per (b, head)
// striding over them.
hipError_t launch_compress_generic(const Dims &d, const void *x, const void *W, const void *PE, void *out,
                                   int dim, hipStream_t s, const int32_t *len_old = nullptr,
                                   const int32_t *len_new = nullptr, int tiles = 0);
hipError_t launch_cmp_attn_generic(const RowArgs &a, bool with_v, hipStream_t s);
// DSA-style decode step: indexer scores + top-k selection, and attention over
// the selected tokens (bf16, 16 heads per KV head, the MFMA (d_k, d_v) pairs)
bool dsa_supported(const Dims &d);
// (prefill: every position of the B sequences is a query row)
// Indexer scores and top-k selection of rows row0 .. row0+rows-1 (rows < 0:
// every row); scores holds the rows' T fp32 scores each, in launch order.
hipError_t launch_dsa_select(const Dims &d, int HI, int DI, int topk, const int32_t *seq_lens, const void *q_idx,
                             const void *w_idx, const void *k_idx, float *scores, int32_t *sel, hipStream_t s,
                             bool prefill = false, int row0 = 0, int rows = -1);
// The prefill's indexer scores are held for this many bytes' worth of rows
// at a time (the last chunk may be shorter).
constexpr size_t kDsaScoreBudget = 256u << 20;
int dsa_prefill_chunk_rows(const Dims &d);
hipError_t launch_dsa_attn(const Dims &d, int topk, const void *q, const void *k, const void *v, const int32_t *sel,
                           void *o, hipStream_t s, bool prefill = false, void *part = nullptr, int nsplit = 1);
// bytes of the partial results an nsplit-way slot split of the decode attention needs
size_t dsa_split_bytes(const Dims &d, int nsplit);
constexpr int kDsaMaxSplit = 4;
// second layer of the two-layer compression, in place: rows <- W2 relu(rows)
hipError_t launch_compress_mlp2(const Dims &d, const void *W2k, const void *W2v, void *cmp_k, void *cmp_v,
                                hipStream_t s, const int32_t *len_old = nullptr, const int32_t *len_new = nullptr,
                                int max_blocks = 0);
hipError_t launch_select_generic(const RowArgs &a, hipStream_t s);
hipError_t launch_sparse_generic(const RowArgs &a, hipStream_t s);

// Token compression for bf16 storage on the vector ALUs (bf16 dot products).
bool compress_bf16_supported(const Dims &d);
hipError_t launch_compress_bf16(const Dims &d, const void *k, const void *v, const void *Wk, const void *PEk,
                                const void *Wv, const void *PEv, void *ok, void *ov, hipStream_t s,
                                const int32_t *len_old = nullptr, const int32_t *len_new = nullptr,
                                int max_new_blocks = 0);

// Matrix-core kernels (bf16 storage, G = 16; prefill rows only).
bool cmp_attn_mfma_supported(const Dims &d);
hipError_t launch_cmp_attn_mfma(const RowArgs &a, bool with_v, hipStream_t s);
// S2 and the window half of S4 in one launch (cmp_attn_mfma_supported shapes):
// needs q, kc, vc, scores, k, v, wg, bg, o; writes scores and o = g_cmp o_cmp
// + g_win o_win, and o_cmp only where a.ocmp is set (with lse / osave: the
// saved statistics of the compressed and window branches)
hipError_t launch_cmp_win_mfma(const RowArgs &a, hipStream_t s);
bool sparse_mfma_supported(const Dims &d);
size_t sparse_mfma_ws_bytes(const Dims &d);   // K and V packed per 64-token block
hipError_t launch_sparse_mfma(const RowArgs &a, void *vt_ws, hipStream_t s);   // honours a.part
bool decode_mfma_supported(const Dims &d);
size_t decode_mfma_layout(const Dims &d, void *ws, DecArgs *A);   // bytes; fills A's buffers if ws
hipError_t launch_decode_mfma(const DecArgs &A, hipStream_t s);

}  // namespace nsa
