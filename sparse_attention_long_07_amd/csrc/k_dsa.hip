// DSA-style decode step (DSA explainer, allinfo.ai.kr, section "쉽게 이해하기"):
// a lightning indexer scores every cached token with a weighted sum of ReLU
// dot products over several small heads that share one key per token; a
// selector keeps the top-k positions (2,048 on the page) for the query; the
// attention runs over the selected tokens only, its softmax denominator
// summed over that set.  One selection per sequence serves every query head
// and KV group.  bf16 storage, fp32 arithmetic.
//
// k_dsa_index  one thread per cached token: I[s] = sum_j w_j relu(q_j . k_s)
//              (HBM: the indexer keys are read once).
// k_dsa_topk   one 1024-thread workgroup per sequence: radix select of the
//              k-th largest score over order-preserving 32-bit keys (four
//              8-bit digits, histograms with integer LDS atomics), then an
//              ordered compaction: every key above the threshold and the
//              lowest-position keys equal to it, ascending, -1 padded.
// k_dsa_attn   one 8-wave workgroup per (sequence, KV head); wave w takes
//              selected slots [w k/8, (w+1) k/8) in sub-chunks of 32 tokens:
//              S^T = K Q^T on gathered K rows (16x16x32 MFMA, the 16 heads
//              as N), online softmax, O^T += V^T P^T with V staged in a
//              wave-private LDS buffer and read by transposing reads; the
//              waves' (max, sum, O) are merged in LDS.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kAttnWaves = 8;

__device__ __forceinline__ int seq_len_of(const int32_t *seq_lens, int b, int T)
{
    const int L = seq_lens[b];
    return L < 1 ? 1 : (L > T ? T : L);
}

// q_idx [B][HI][DI], w_idx [B][HI], k_idx [B][T][DI] (bf16); scores [B][T] fp32
__global__ __launch_bounds__(kThreads) void k_dsa_index(const uint16_t *__restrict__ q_idx,
                                                        const uint16_t *__restrict__ w_idx,
                                                        const uint16_t *__restrict__ k_idx,
                                                        const int32_t *__restrict__ seq_lens, float *__restrict__ scores,
                                                        int T, int HI, int DI)
{
    __shared__ float qs[16 * 256];
    __shared__ float ws[16];
    const int b = blockIdx.y, tid = threadIdx.x;
    for (int e = tid; e < HI * DI; e += kThreads) qs[e] = bf2f(q_idx[(long)b * HI * DI + e]);
    if (tid < HI) ws[tid] = bf2f(w_idx[(long)b * HI + tid]);
    __syncthreads();
    const int L = seq_len_of(seq_lens, b, T);
    const int s = blockIdx.x * kThreads + tid;
    if (s >= L) return;
    const uint16_t *kr = k_idx + ((long)b * T + s) * DI;
    float dot[16];
#pragma unroll
    for (int j = 0; j < 16; j++) dot[j] = 0.f;
    for (int e0 = 0; e0 < DI; e0 += 8) {
        const u32x4 v = ld16(kr + e0);
        float x[8];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t w = v[e];
            x[2 * e] = __uint_as_float(w << 16);
            x[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 16; j++)
            if (j < HI)
#pragma unroll
                for (int e = 0; e < 8; e++) dot[j] = __builtin_fmaf(qs[j * DI + e0 + e], x[e], dot[j]);
    }
    float I = 0.f;
#pragma unroll
    for (int j = 0; j < 16; j++)
        if (j < HI) I = __builtin_fmaf(ws[j], fmaxf(dot[j], 0.f), I);
    scores[(long)b * T + s] = I;
}

// larger float -> larger key (no NaN among the scores)
__device__ __forceinline__ uint32_t order_key(float x)
{
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix over the block's threads of v (kTopkThreads = 16 waves);
// total returned through *tot
__device__ __forceinline__ int block_exscan(int v, int *wsum, int *tot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
    for (int w = 0; w < kTopkThreads / 64; w++) {
        const int c = wsum[w];
        base += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *tot = all;
    return base + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void k_dsa_topk(const float *__restrict__ scores,
                                                           const int32_t *__restrict__ seq_lens,
                                                           int32_t *__restrict__ sel, int T, int topk)
{
    __shared__ int hist[256];
    __shared__ int wsum[kTopkThreads / 64];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remain;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int L = seq_len_of(seq_lens, b, T);
    const float *sc = scores + (long)b * T;
    int32_t *out = sel + (long)b * topk;
    if (L <= topk) {
        for (int i = tid; i < topk; i += kTopkThreads) out[i] = i < L ? i : -1;
        return;
    }
    // radix select: prefix/mask of the k-th largest key, digit by digit
    uint32_t prefix = 0, mask = 0;
    int remain = topk;   // how many of the keys matching the prefix are still to be taken
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int s = tid; s < L; s += kTopkThreads) {
            const uint32_t u = order_key(sc[s]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 255-4l .. 252-4l (high to low); inclusive
            // suffix sums from digit 255 down
            int c[4], own = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                c[i] = hist[255 - 4 * lane - i];
                own += c[i];
            }
            int x = own;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            int above = x - own;   // keys with a higher digit than this lane's first
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (above < remain && above + c[i] >= remain) {
                    s_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
                    s_remain = remain - above;
                }
                above += c[i];
            }
        }
        __syncthreads();
        prefix = s_prefix;
        remain = s_remain;
        mask |= 255u << shift;
        __syncthreads();
    }
    // ordered compaction over contiguous ranges: keys above the threshold,
    // then the first `remain` keys equal to it in position order
    const int per = (L + kTopkThreads - 1) / kTopkThreads;
    const int lo = min(L, tid * per), hi = min(L, lo + per);
    int gt = 0, eq = 0;
    for (int s = lo; s < hi; s++) {
        const uint32_t u = order_key(sc[s]);
        gt += u > prefix;
        eq += u == prefix;
    }
    int tot;
    const int eq_before = block_exscan(eq, wsum, &tot);
    const int take_eq = max(0, min(eq, remain - eq_before));
    const int pos0 = block_exscan(gt + take_eq, wsum, &tot);
    int pos = pos0, eq_taken = 0;
    for (int s = lo; s < hi; s++) {
        const uint32_t u = order_key(sc[s]);
        bool keep = u > prefix;
        if (u == prefix) {
            keep = eq_taken < take_eq;
            eq_taken++;
        }
        if (keep) out[pos++] = s;
    }
    for (int i = tot + tid; i < topk; i += kTopkThreads) out[i] = -1;
    (void)lane;
}

template <int DK, int DV>
__global__ __launch_bounds__(kAttnWaves * 64) void k_dsa_attn(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v,
                                                             const int32_t *__restrict__ sel, uint16_t *__restrict__ o,
                                                             int T, int Hkv, int topk, float scale)
{
    constexpr int NQ = DK / 32, NO = DV / 16, VS = DV + 16;
    constexpr int kStage = 32 * VS;                       // bf16 per wave
    constexpr int kMerge = 16 * DV * (int)sizeof(float) / 2;   // the same bytes, counted in bf16
    __shared__ __align__(16) uint16_t vst[kAttnWaves][kStage > kMerge ? kStage : kMerge];
    __shared__ int ss[8192];
    __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
    for (int i = tid; i < topk; i += kAttnWaves * 64) ss[i] = sel[(long)b * topk + i];
    // B operand Q^T: head li of the group, columns 32 c + 8 lg .. +7
    u32x4 qf[NQ];
    const long qrow = ((long)b * Hkv * 16 + g * 16 + li) * DK;
#pragma unroll
    for (int c = 0; c < NQ; c++) qf[c] = ld16(q + qrow + 32 * c + 8 * lg);
    __syncthreads();
    const uint16_t *K = k + (long)bg * T * DK;
    const uint16_t *V = v + (long)bg * T * DV;
    uint16_t *vw = vst[wave];
    const float sl2 = scale * kLog2e;
    f32x4 acc[NO];
#pragma unroll
    for (int i = 0; i < NO; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    const int per = (topk + kAttnWaves - 1) / kAttnWaves;
    const int beg = wave * per, end = min(topk, beg + per);
    const int trow = li >> 2, tcol = 4 * (li & 3);
    for (int c0 = beg; c0 < end; c0 += 32) {
        float sc[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            // A operand K: slot c0 + 16 kt + li (an empty slot, or an entry
            // outside the cache, reads token 0 and is masked below)
            const int slot = c0 + 16 * kt + li;
            const int tok = slot < end ? ss[slot] : -1;
            const int tl = tok >= 0 && tok < T ? tok : 0;
            f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NQ; c++) S = mfma16(as_bf16x8(ld16(K + (long)tl * DK + 32 * c + 8 * lg)), as_bf16x8(qf[c]), S);
#pragma unroll
            for (int c = 0; c < DV / 32; c++) st16(vw + (16 * kt + li) * VS + 32 * c + 8 * lg, ld16(V + (long)tl * DV + 32 * c + 8 * lg));
            // C[i = slot][j = head]: lane j + 16 (i / 4), element i % 4
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int sl = c0 + 16 * kt + 4 * lg + e;
                const bool ok = sl < end && ss[sl] >= 0 && ss[sl] < T;
                sc[kt][e] = ok ? S[e] * sl2 : -INFINITY;
            }
        }
        float mc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int e = 0; e < 4; e++) mc = fmaxf(mc, sc[kt][e]);
        mc = fmaxf(mc, __shfl_xor(mc, 16));
        mc = fmaxf(mc, __shfl_xor(mc, 32));
        const float mn = fmaxf(m, mc);
        if (mn == -INFINITY) continue;   // no valid slot in this sub-chunk (the whole wave agrees)
        const float al = fast_exp2(m - mn);
        float p[2][4], ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                p[kt][e] = fast_exp2(sc[kt][e] - mn);
                ls += p[kt][e];
            }
        l = __builtin_fmaf(l, al, ls);
        m = mn;
        // contraction slot 8 lg + e <-> token 4 lg + e (e < 4) or 16 + 4 lg + e - 4
        u32x4 y;
        y[0] = pack_bf16x2(p[0][0], p[0][1]);
        y[1] = pack_bf16x2(p[0][2], p[0][3]);
        y[2] = pack_bf16x2(p[1][0], p[1][1]);
        y[3] = pack_bf16x2(p[1][2], p[1][3]);
        const bf16x8 bp = as_bf16x8(y);
        const int r0 = 4 * lg + trow;
#pragma unroll
        for (int dt = 0; dt < NO; dt++) {
            acc[dt] *= al;
            const uint2 lo = ld_tr16(vw + r0 * VS + 16 * dt + tcol);
            const uint2 hi = ld_tr16(vw + (r0 + 16) * VS + 16 * dt + tcol);
            acc[dt] = mfma16(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), bp, acc[dt]);
        }
    }
    // merge the waves: per head (max, sum) and O^T (C[i = column][j = head])
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (lg == 0) {
        s_m[wave][li] = m;
        s_l[wave][li] = l;
    }
    __syncthreads();   // every wave is done with its V staging buffer
    float *ow = (float *)vst[wave];   // [16 heads][DV]
#pragma unroll
    for (int dt = 0; dt < NO; dt++)
#pragma unroll
        for (int e = 0; e < 4; e++) ow[li * DV + 16 * dt + 4 * lg + e] = acc[dt][e];
    __syncthreads();
    for (int i = tid; i < 16 * DV; i += kAttnWaves * 64) {
        const int h = i / DV;
        float M = -INFINITY;
        for (int w = 0; w < kAttnWaves; w++) M = fmaxf(M, s_m[w][h]);
        float num = 0.f, den = 0.f;
        for (int w = 0; w < kAttnWaves; w++) {
            const float f = s_m[w][h] == -INFINITY ? 0.f : fast_exp2(s_m[w][h] - M);
            num = __builtin_fmaf(f, ((const float *)vst[w])[i], num);
            den = __builtin_fmaf(f, s_l[w][h], den);
        }
        o[((long)b * Hkv * 16 + g * 16) * DV + i] = f2bf(den > 0.f ? num / den : 0.f);
    }
}

}  // namespace

bool dsa_supported(const Dims &d)
{
    return d.dtype == NSA_BF16 && d.G == 16 &&
           ((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64));
}

hipError_t launch_dsa_select(const Dims &d, int HI, int DI, int topk, const int32_t *seq_lens, const void *q_idx,
                             const void *w_idx, const void *k_idx, float *scores, int32_t *sel, hipStream_t s)
{
    hipLaunchKernelGGL(k_dsa_index, dim3((d.T + kThreads - 1) / kThreads, d.B), dim3(kThreads), 0, s,
                       (const uint16_t *)q_idx, (const uint16_t *)w_idx, (const uint16_t *)k_idx, seq_lens, scores, d.T,
                       HI, DI);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_dsa_topk, dim3(d.B), dim3(kTopkThreads), 0, s, scores, seq_lens, sel, d.T, topk);
    return hipGetLastError();
}

hipError_t launch_dsa_attn(const Dims &d, int topk, const void *q, const void *k, const void *v, const int32_t *sel,
                           void *o, hipStream_t s)
{
    const dim3 grid(d.B * d.Hkv), block(kAttnWaves * 64);
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *oo = (uint16_t *)o;
    if (d.dk == 192) hipLaunchKernelGGL((k_dsa_attn<192, 128>), grid, block, 0, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale);
    else if (d.dk == 128) hipLaunchKernelGGL((k_dsa_attn<128, 128>), grid, block, 0, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale);
    else hipLaunchKernelGGL((k_dsa_attn<64, 64>), grid, block, 0, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale);
    return hipGetLastError();
}

}  // namespace nsa
