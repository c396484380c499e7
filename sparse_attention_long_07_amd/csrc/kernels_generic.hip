// Generic NSA kernels: plain VALU arithmetic in fp32, fp32 or bf16 storage,
// any shape the C ABI accepts.  They carry the fp32 configuration and every
// shape the matrix-core kernels do not specialise.
//
// Method: deepdaiv newsletter on DeepSeek's NSA (deepdaiv.stibee.com/p/82),
// paragraphs on token compression, token selection and the sliding window;
// sizes from valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새
// 어텐션 기술 화제", section II.
#include "nsa_internal.h"
#include "select_util.h"

#include <math.h>

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kChunk = 64;   // keys per inner-loop chunk (one per lane of a wave)

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ int row_t(const RowArgs &a, int b, int r)
{
    if (!a.seq_lens) return r;
    int L = a.seq_lens[b];
    L = L < 1 ? 1 : (L > a.d.T ? a.d.T : L);
    return L - 1;
}

// ---------------------------------------------------------------------------
// Token compression as a tiled matrix product.  Flattening block i of a
// [T][dim] sequence token-major gives 32*dim consecutive elements starting at
// row 16*i, so out[i][c] = sum_m (x[16*i*dim + m] + PE[m]) * W[c][m] with
// m = tau*dim + e.  Tile: 64 blocks x 64 channels, 32 inputs per step; each
// thread owns a 4x4 patch of the tile.
template <typename T>
__device__ __forceinline__ void compress_generic_tile(const T *__restrict__ x, const T *__restrict__ W,
                                                      const T *__restrict__ PE, T *__restrict__ out, int seqlen,
                                                      int dim, int ncmp, int npad, int bh, int i0, int c0, int wlo,
                                                      int whi, float (&Xs)[32][65], float (&Ws)[32][65])
{
    const T *xs = x + (long)bh * seqlen * dim;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const long K = 32L * dim;
    float acc[4][4] = {};
    for (long m0 = 0; m0 < K; m0 += 32) {
        for (int e = threadIdx.x; e < 64 * 32; e += kThreads) {
            int ii = e / 32, mm = e % 32;
            int i = i0 + ii, c = c0 + ii;
            long m = m0 + mm;
            Xs[mm][ii] = i < ncmp ? to_f(xs[16L * i * dim + m]) + to_f(PE[m]) : 0.f;
            Ws[mm][ii] = c < dim ? to_f(W[(long)c * K + m]) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int mm = 0; mm < 32; mm++) {
            float a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                a[u] = Xs[mm][ty * 4 + u];
                b[u] = Ws[mm][tx * 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int w = 0; w < 4; w++) acc[u][w] += a[u] * b[w];
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int w = 0; w < 4; w++) {
            int i = i0 + ty * 4 + u, c = c0 + tx * 4 + w;
            if (i >= wlo && i < whi && i < npad && c < dim)
                out[((long)bh * npad + i) * dim + c] = from_f<T>(i < ncmp ? acc[u][w] : 0.f);
        }
}

// Without lengths every block of the seqlen-token sequences is written (pads as
// 0); with lengths (a cache of capacity seqlen) only the blocks that an append
// from len_old[b] to len_new[b] tokens completes, workgroups striding over
// them.  A block's value does not depend on the tile that computes it.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_compress_generic(const T *__restrict__ x, const T *__restrict__ W,
                                                              const T *__restrict__ PE, T *__restrict__ out,
                                                              int seqlen, int dim, int ncmp, int npad, int Hkv,
                                                              const int32_t *len_old, const int32_t *len_new)
{
    __shared__ float Xs[32][65];
    __shared__ float Ws[32][65];
    const int bh = blockIdx.z, c0 = blockIdx.y * 64;
    int lo = 0, hi = ncmp;
    if (len_new) append_range(len_old, len_new, bh / Hkv, seqlen, lo, hi);
    const int wend = len_new ? hi : npad;
    for (int i0 = lo + (int)blockIdx.x * 64; i0 < wend; i0 += (int)gridDim.x * 64) {
        compress_generic_tile<T>(x, W, PE, out, seqlen, dim, hi, npad, bh, i0, c0, len_new ? lo : i0, wend, Xs, Ws);
        if (!len_new) break;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Compressed attention and block importance for one (row, KV head).
// Pass 1 finds each head's log-sum-exp over the visible compressed blocks
// (16*i + 31 <= t).  Pass 2 recomputes the logits, forms the exact
// probabilities p_h[i], sums them over the group's heads (P[i]) and maps them
// onto selection blocks: block j collects keys 4j-1 .. 4j+3 with weights
// 1,2,2,2,1 (tokens shared with [64j, 64j+64) divided by the stride 16).  A
// chunk of 64 keys covers exactly the 16 blocks 16c .. 16c+15 given the
// previous chunk's last key, so every score is formed once, in a fixed order.
template <typename T, bool WITH_V>
__global__ __launch_bounds__(kThreads) void k_cmp_attn_generic(RowArgs a)
{
    extern __shared__ float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv;
    float *qs = smem;                 // [G][dk]
    float *sb = qs + G * dk;          // [G][64]
    float *Pb = sb + G * kChunk;      // [65]: Pb[0] = previous chunk's last key
    float *S = Pb + 68;               // [nb]
    __shared__ float m_s[16], l_s[16], lse_s[16];

    const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t = row_t(a, b, r);
    const int nvis = t >= 31 ? (t - 31) / 16 + 1 : 0;
    const int jcur = t / 64;
    const T *qrow = (const T *)a.q + b * a.q_sb + r * a.q_sr + (long)g * G * dk;
    for (int e = tid; e < G * dk; e += kThreads) qs[e] = to_f(qrow[e]);
    for (int j = tid; j < d.nb; j += kThreads) S[j] = 0.f;
    if (tid < 16) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.f;
    }
    if (tid == 0) Pb[0] = 0.f;
    __syncthreads();
    const T *kc = (const T *)a.kc + ((long)b * d.Hkv + g) * d.npad * dk;
    const T *vc = (const T *)a.vc + ((long)b * d.Hkv + g) * d.npad * dv;

    // pass 1: per-head max and sum
    for (int c0 = 0; c0 < nvis; c0 += kChunk) {
        for (int e = tid; e < G * kChunk; e += kThreads) {
            int h = e / kChunk, ii = e % kChunk, i = c0 + ii;
            float s = -INFINITY;
            if (i < nvis) {
                float acc = 0.f;
                const T *kr = kc + (long)i * dk;
                for (int x = 0; x < dk; x++) acc += qs[h * dk + x] * to_f(kr[x]);
                s = acc * d.scale;
            }
            sb[h * kChunk + ii] = s;
        }
        __syncthreads();
        for (int h = wave; h < G; h += kThreads / kWave) {
            float v = sb[h * kChunk + lane];
            float mo = m_s[h];
            float mn = fmaxf(mo, wave_max(v));
            float sum = wave_sum(__expf(v - mn));
            if (lane == 0) {
                l_s[h] = l_s[h] * __expf(mo - mn) + sum;
                m_s[h] = mn;
            }
        }
        __syncthreads();
    }
    if (tid < G) lse_s[tid] = nvis > 0 ? m_s[tid] + __logf(l_s[tid]) : -INFINITY;
    __syncthreads();

    // pass 2: probabilities, importance, output
    const int nout = WITH_V ? (G * dv + kThreads - 1) / kThreads : 0;
    float oacc[16];
#pragma unroll
    for (int u = 0; u < 16; u++) oacc[u] = 0.f;
    for (int c0 = 0; c0 < nvis; c0 += kChunk) {
        for (int e = tid; e < G * kChunk; e += kThreads) {
            int h = e / kChunk, ii = e % kChunk, i = c0 + ii;
            float p = 0.f;
            if (i < nvis) {
                float acc = 0.f;
                const T *kr = kc + (long)i * dk;
                for (int x = 0; x < dk; x++) acc += qs[h * dk + x] * to_f(kr[x]);
                p = __expf(acc * d.scale - lse_s[h]);
            }
            sb[h * kChunk + ii] = p;
        }
        __syncthreads();
        if (tid < kChunk) {
            float P = 0.f;
            for (int h = 0; h < G; h++) P += sb[h * kChunk + tid];
            Pb[1 + tid] = P;
        }
        __syncthreads();
        if (tid < 16) {
            int j = c0 / 4 + tid;
            if (j < d.nb)
                S[j] = Pb[4 * tid] + 2.f * (Pb[4 * tid + 1] + Pb[4 * tid + 2] + Pb[4 * tid + 3]) + Pb[4 * tid + 4];
        }
        if (WITH_V) {
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u >= nout) break;
                int e = tid + u * kThreads;
                if (e < G * dv) {
                    int h = e / dv, c = e % dv;
                    float acc = oacc[u];
                    int lim = nvis - c0 < kChunk ? nvis - c0 : kChunk;
                    for (int ii = 0; ii < lim; ii++) acc += sb[h * kChunk + ii] * to_f(vc[(long)(c0 + ii) * dv + c]);
                    oacc[u] = acc;
                }
            }
        }
        __syncthreads();
        if (tid == 0) Pb[0] = Pb[kChunk];
        __syncthreads();
    }
    // the last visible key, when it closes a chunk, also reaches the first
    // block of the chunk that was not run
    if (tid == 0 && nvis > 0 && nvis % kChunk == 0 && nvis / 4 < d.nb) S[nvis / 4] = Pb[0];
    __syncthreads();

    float *srow = a.scores + (((long)b * d.Hkv + g) * a.R + r) * d.nb;
    for (int j = tid; j < d.nb; j += kThreads) srow[j] = j <= jcur ? S[j] : -INFINITY;
    // the branch's log-sum-exp for the backward, when asked for
    if (WITH_V && a.lse && tid < G) a.lse[((long)b * a.R + r) * d.Hq + (long)g * G + tid] = lse_s[tid];
    if (WITH_V) {
        T *orow = (T *)a.ocmp + (((long)b * a.R + r) * d.Hq + (long)g * G) * dv;
#pragma unroll
        for (int u = 0; u < 16; u++) {
            if (u >= nout) break;
            int e = tid + u * kThreads;
            if (e < G * dv) orow[e] = from_f<T>(oacc[u]);
        }
    }
}

// ---------------------------------------------------------------------------
// Top-n block selection, one wavefront per (row, KV head): see select_util.h.
__global__ __launch_bounds__(kThreads) void k_select_generic(RowArgs a)
{
    __shared__ uint2 cand[kThreads / kWave][64];
    const Dims &d = a.d;
    const int lane = threadIdx.x % kWave;
    const long row = (long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const long nrows = (long)d.B * d.Hkv * a.R;
    if (row >= nrows) return;
    const int r = (int)(row % a.R);
    const int b = (int)(row / ((long)d.Hkv * a.R));
    const int t = row_t(a, b, r);
    wave_select_topn_fast(a.scores + row * d.nb, t / 64, d.n, a.idx_sel + row * d.n, lane,
                          cand[threadIdx.x / kWave]);
}

// ---------------------------------------------------------------------------
// Selected-block attention, window attention and the gated combination for
// one (row, KV head).  Both branches stream 64-key chunks with an online
// softmax; the selected branch walks the distinct valid blocks of the row's
// list (one softmax over their union), the window walks [max(0,t-w+1), t].
template <typename T>
__global__ __launch_bounds__(kThreads) void k_sparse_generic(RowArgs a)
{
    extern __shared__ float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv;
    float *qs = smem;                 // [G][dk]
    float *sb = qs + G * dk;          // [G][64]
    __shared__ float m_s[16], l_s[16], al_s[16], gate_s[48];
    __shared__ int blk[64];
    __shared__ int nblk_s;

    const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int t = row_t(a, b, r);
    const int jcur = t / 64;
    const T *qrow = (const T *)a.q + b * a.q_sb + r * a.q_sr + (long)g * G * dk;
    for (int e = tid; e < G * dk; e += kThreads) qs[e] = to_f(qrow[e]);
    if (tid == 0) {
        // the window-only part has no index list (a.idx is null there)
        const int32_t *ir = a.part == 1 ? nullptr : a.idx + (((long)b * d.Hkv + g) * a.R + r) * d.n;
        int m = 0;
        for (int q2 = 0; ir && q2 < d.n; q2++) {
            int j = ir[q2];
            if (j < 0 || j > jcur) continue;
            int pos = m;                       // insertion sort, skipping repeats
            bool dup = false;
            for (int u = 0; u < m; u++) {
                if (blk[u] == j) dup = true;
            }
            if (dup) continue;
            while (pos > 0 && blk[pos - 1] > j) {
                blk[pos] = blk[pos - 1];
                pos--;
            }
            blk[pos] = j;
            m++;
        }
        nblk_s = m;
    }
    __syncthreads();
    // gates: sigmoid(w_g[h][c] . q_h + b_g[h][c])
    if (tid < 3 * G) {
        int h = tid / 3, c = tid % 3;
        const T *wr = (const T *)a.wg + (((long)g * G + h) * 3 + c) * dk;
        float z = to_f(((const T *)a.bg)[((long)g * G + h) * 3 + c]);
        for (int x = 0; x < dk; x++) z += to_f(wr[x]) * qs[h * dk + x];
        gate_s[tid] = 1.f / (1.f + __expf(-z));
    }
    const T *K = (const T *)a.k + ((long)b * d.Hkv + g) * d.T * dk;
    const T *V = (const T *)a.v + ((long)b * d.Hkv + g) * d.T * dv;
    const int nout = (G * dv + kThreads - 1) / kThreads;
    float res[2][16];
    const int lo = t - d.w + 1 > 0 ? t - d.w + 1 : 0;

    for (int br = 0; br < 2; br++) {
        // part 1 computes only the window (br 1), part 2 only the selected branch (br 0)
        if ((a.part == 1 && br == 0) || (a.part == 2 && br == 1)) {
#pragma unroll
            for (int u = 0; u < 16; u++) res[br][u] = 0.f;
            continue;
        }
        float acc[16];
#pragma unroll
        for (int u = 0; u < 16; u++) acc[u] = 0.f;
        if (tid < 16) {
            m_s[tid] = -INFINITY;
            l_s[tid] = 0.f;
        }
        __syncthreads();
        const int nch = br == 0 ? nblk_s : (t - lo + kChunk) / kChunk;
        for (int ch = 0; ch < nch; ch++) {
            const int key0 = br == 0 ? blk[ch] * 64 : lo + ch * kChunk;
            for (int e = tid; e < G * kChunk; e += kThreads) {
                int h = e / kChunk, ii = e % kChunk, key = key0 + ii;
                float s = -INFINITY;
                if (key <= t) {
                    float z = 0.f;
                    const T *kr = K + (long)key * dk;
                    for (int x = 0; x < dk; x++) z += qs[h * dk + x] * to_f(kr[x]);
                    s = z * d.scale;
                }
                sb[h * kChunk + ii] = s;
            }
            __syncthreads();
            for (int h = wave; h < G; h += kThreads / kWave) {
                float v = sb[h * kChunk + lane];
                float mo = m_s[h];
                float mn = fmaxf(mo, wave_max(v));
                float p = __expf(v - mn);
                sb[h * kChunk + lane] = p;
                float sum = wave_sum(p);
                if (lane == 0) {
                    float al = __expf(mo - mn);
                    l_s[h] = l_s[h] * al + sum;
                    m_s[h] = mn;
                    al_s[h] = al;
                }
            }
            __syncthreads();
            const int lim = t - key0 + 1 < kChunk ? t - key0 + 1 : kChunk;
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u >= nout) break;
                int e = tid + u * kThreads;
                if (e < G * dv) {
                    int h = e / dv, c = e % dv;
                    float z = acc[u] * al_s[h];
                    for (int ii = 0; ii < lim; ii++) z += sb[h * kChunk + ii] * to_f(V[(long)(key0 + ii) * dv + c]);
                    acc[u] = z;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < 16; u++) {
            int e = tid + u * kThreads;
            int h = e / dv;
            res[br][u] = (u < nout && e < G * dv && l_s[h < 16 ? h : 0] > 0.f) ? acc[u] / l_s[h] : 0.f;
        }
        // saved statistics for the backward: slot 1 selected, slot 2 window
        if (a.lse) {
            const long slot = (long)d.B * a.R * d.Hq, rh = ((long)b * a.R + r) * d.Hq + (long)g * G;
            if (tid < G) a.lse[(1 + br) * slot + rh + tid] = l_s[tid] > 0.f ? m_s[tid] + __logf(l_s[tid]) : -INFINITY;
            T *osv = (T *)a.osave + ((1 + br) * slot + rh) * dv;
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u >= nout) break;
                const int e = tid + u * kThreads;
                if (e < G * dv) osv[e] = from_f<T>(res[br][u]);
            }
        }
        __syncthreads();
    }
    const T *oc = (const T *)a.ocmp + (((long)b * a.R + r) * d.Hq + (long)g * G) * dv;
    T *orow = (T *)a.o + b * a.o_sb + r * a.o_sr + (long)g * G * dv;
#pragma unroll
    for (int u = 0; u < 16; u++) {
        if (u >= nout) break;
        int e = tid + u * kThreads;
        if (e < G * dv) {
            int h = e / dv;
            float y;
            if (a.part == 2) y = to_f(orow[e]) + gate_s[h * 3 + 1] * res[0][u];
            else y = gate_s[h * 3] * to_f(oc[e]) + gate_s[h * 3 + 1] * res[0][u] + gate_s[h * 3 + 2] * res[1][u];
            orow[e] = from_f<T>(y);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_compress_generic(const Dims &d, const void *x, const void *W, const void *PE, void *out,
                                   int dim, hipStream_t s, const int32_t *len_old, const int32_t *len_new,
                                   int tiles)
{
    dim3 grid(len_new ? tiles : d.npad / 64, (dim + 63) / 64, d.B * d.Hkv);
    if (d.dtype == NSA_FP32)
        hipLaunchKernelGGL(k_compress_generic<float>, grid, dim3(kThreads), 0, s, (const float *)x,
                           (const float *)W, (const float *)PE, (float *)out, d.T, dim, d.ncmp, d.npad, d.Hkv,
                           len_old, len_new);
    else
        hipLaunchKernelGGL(k_compress_generic<bf16_t>, grid, dim3(kThreads), 0, s, (const bf16_t *)x,
                           (const bf16_t *)W, (const bf16_t *)PE, (bf16_t *)out, d.T, dim, d.ncmp, d.npad, d.Hkv,
                           len_old, len_new);
    return hipGetLastError();
}

hipError_t launch_cmp_attn_generic(const RowArgs &a, bool with_v, hipStream_t s)
{
    const Dims &d = a.d;
    size_t lds = sizeof(float) * ((size_t)d.G * d.dk + (size_t)d.G * kChunk + 68 + d.nb);
    dim3 grid(a.R, d.Hkv, d.B);
    if (d.dtype == NSA_FP32) {
        if (with_v) hipLaunchKernelGGL((k_cmp_attn_generic<float, true>), grid, dim3(kThreads), lds, s, a);
        else hipLaunchKernelGGL((k_cmp_attn_generic<float, false>), grid, dim3(kThreads), lds, s, a);
    } else {
        if (with_v) hipLaunchKernelGGL((k_cmp_attn_generic<bf16_t, true>), grid, dim3(kThreads), lds, s, a);
        else hipLaunchKernelGGL((k_cmp_attn_generic<bf16_t, false>), grid, dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_select_generic(const RowArgs &a, hipStream_t s)
{
    const Dims &d = a.d;
    long rows = (long)d.B * d.Hkv * a.R;
    dim3 grid((unsigned)((rows + 3) / 4));
    hipLaunchKernelGGL(k_select_generic, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sparse_generic(const RowArgs &a, hipStream_t s)
{
    const Dims &d = a.d;
    size_t lds = sizeof(float) * ((size_t)d.G * d.dk + (size_t)d.G * kChunk);
    dim3 grid(a.R, d.Hkv, d.B);
    if (d.dtype == NSA_FP32) hipLaunchKernelGGL(k_sparse_generic<float>, grid, dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL(k_sparse_generic<bf16_t>, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace nsa
