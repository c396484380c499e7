// DSA-style decode step and prefill (DSA explainer, allinfo.ai.kr, section "쉽게 이해하기"):
// a lightning indexer scores every cached token with a weighted sum of ReLU
// dot products over several small heads that share one key per token; a
// selector keeps the top-k positions (2,048 on the page) for the query; the
// attention runs over the selected tokens only, its softmax denominator
// summed over that set.  One selection per query serves every query head and
// KV group.  bf16 storage, fp32 arithmetic.  A "row" is one query: a
// sequence's last token (decode: cache b, length seq_lens[b]) or one position
// of a prefill (row r = b T + t: cache b, length t + 1).
//
// k_dsa_index  I[s] = sum_j w_j relu(q_j . k_s) on the matrix cores (keys as
//              M, indexer heads as N), the head sum by DPP row reductions
//              (HBM: the indexer keys are read once).
// k_dsa_topk   one 1024-thread workgroup per sequence: radix select of the
//              k-th largest score over order-preserving 32-bit keys (digits
//              of 12, 12 and 8 bits, histograms with integer LDS atomics),
//              then an ordered compaction by wave ballots: every key above
//              the threshold and the lowest-position keys equal to it,
//              ascending (exactly k of them, since more than k candidates).
//              Rows up to 65,536 positions are read once into registers (up
//              to 64 scores per lane) and every pass runs from them.
// k_dsa_attn   one 8-wave workgroup per (sequence, KV head); wave w takes
//              selected slots [w k/8, (w+1) k/8) in sub-chunks of 32 tokens:
//              S^T = K Q^T on gathered K rows (16x16x32 MFMA, the 16 heads
//              as N), online softmax, O^T += V^T P^T with V staged in a
//              wave-private LDS buffer and read by transposing reads; the
//              waves' (max, sum, O) are merged in LDS.  With nsplit = 2 or 4
//              that many workgroups take equal shares of the slots and leave
//              (max, sum, unnormalised O) per head in a workspace that
//              k_dsa_merge combines (decode: 128 workgroups would otherwise
//              leave half the chip idle; with 4 the selection share in LDS is
//              small enough for two workgroups per CU).
#include <algorithm>

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

// q_idx [B][HI][DI], w_idx [B][HI], k_idx [B][T][DI] (bf16); scores [B][T] fp32.
// Scores^T = K Q^T on the matrix cores: 16 keys as M, the indexer heads as N
// (zero past HI), DI as the contraction in NC steps of 32 (zero past DI).
// Lane (key li, group lg) loads its key's 8 columns per step; in the result
// lane (head li, group lg) holds keys 4 lg .. 4 lg + 3, so the weighted ReLU
// sum over heads is a 16-lane row sum.  Each wave takes 64 keys, all loads
// issued first.
template <int NC>
__global__ __launch_bounds__(kThreads) void k_dsa_index(const uint16_t *__restrict__ q_idx,
                                                        const uint16_t *__restrict__ w_idx,
                                                        const uint16_t *__restrict__ k_idx,
                                                        const int32_t *__restrict__ seq_lens, float *__restrict__ scores,
                                                        int T, int HI, int DI, int prefill, int row0)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int b = row0 + blockIdx.x;   // the row: a sequence (decode) or a position (prefill)
    float *srow = scores + (long)blockIdx.x * T;   // the scores of this launch's rows
    const int cb = prefill ? b / T : b;
    const int L = prefill ? b % T + 1 : seq_len_of(seq_lens, b, T);
    const int key0 = blockIdx.y * kThreads + wave * 64;
    if (key0 >= L) return;   // no barriers in this kernel
    const u32x4 z = {0u, 0u, 0u, 0u};
    u32x4 ka[4][NC], qb[NC];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
        const int sl = min(key0 + 16 * kt + li, L - 1);   // keys past the length read the last one
#pragma unroll
        for (int c = 0; c < NC; c++) {
            const int e0 = 32 * c + 8 * lg;
            // read once per step: a non-temporal load keeps the keys from
            // displacing other data in the caches
            ka[kt][c] = e0 < DI ? __builtin_nontemporal_load((const u32x4 *)(k_idx + ((long)cb * T + sl) * DI + e0)) : z;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int e0 = 32 * c + 8 * lg;
        qb[c] = li < HI && e0 < DI ? ld16(q_idx + ((long)b * HI + li) * DI + e0) : z;
    }
    const float wj = li < HI ? bf2f(w_idx[(long)b * HI + li]) : 0.f;
    // the row sums leave every lane of a row with all four sums, so lane
    // (li, lg) can store key 16 (li / 4) + 4 lg + li % 4: one store for the
    // wave's 64 keys
    float mine = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; c++) acc = mfma16(as_bf16x8(ka[kt][c]), as_bf16x8(qb[c]), acc);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float v = row_sum16(wj * fmaxf(acc[e], 0.f));
            if (li == 4 * kt + e) mine = v;
        }
    }
    const int s = key0 + 16 * (li >> 2) + 4 * lg + (li & 3);
    if (s < L) srow[s] = mine;
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

// hist[bin] += 1 for the active lanes, the lanes that share the first
// active lane's bin with one atomic: with many equal keys (ties) per-lane
// atomics on one address serialise across the wave
__device__ __forceinline__ void hist_add(int *hist, int bin, bool active)
{
    const unsigned long long am = __ballot(active);
    if (am == 0ull) return;
    const int lane = threadIdx.x & 63, first = (int)__builtin_ctzll(am);
    const int b0 = __shfl(bin, first, 64);
    const unsigned long long same = __ballot(active && bin == b0);
    if (lane == first) atomicAdd(&hist[b0], (int)__popcll(same));
    else if (active && bin != b0) atomicAdd(&hist[bin], 1);
}

// the lowest n set bits of x (none for n <= 0; __popc is unsigned, so the
// comparison is made in int)
__device__ __forceinline__ uint32_t lowest_bits(uint32_t x, int n)
{
    if (n <= 0) return 0u;
    if (n >= (int)__popc(x)) return x;
    uint32_t r = 0;
    for (int k = 0; k < n; k++) {
        r |= x & (0u - x);
        x &= x - 1;
    }
    return r;
}

// NR > 0: every score of the row is loaded once into registers (NR per lane,
// rows of at most 1024 NR positions).  A sample of one register step in
// eight bounds the k-th score from below by a first digit; the keys at or
// above it (a few more than k) are compacted into LDS, the radix select runs
// over them only, and the kept positions go out through a bitmap in
// ascending order.  When the candidates are fewer than k (an unlucky sample)
// or more than the LDS list holds, the five passes run over all registers.
// NR = 0: each pass reads the scores again (rows of any length).
template <int NR>
__global__ __launch_bounds__(kTopkThreads) void k_dsa_topk(const float *__restrict__ scores,
                                                           const int32_t *__restrict__ seq_lens,
                                                           int32_t *__restrict__ sel, int T, int topk, int prefill,
                                                           int row0)
{
    constexpr int kWaves = kTopkThreads / 64;
    constexpr int kCap = NR > 0 ? 12288 : 1;   // candidate list: keys, positions
    __shared__ int hist[4096];   // histograms; in the candidate path then two position bitmaps
    __shared__ uint32_t cand_k[kCap];
    __shared__ uint16_t cand_p[kCap];
    __shared__ int wsum[kWaves];
    __shared__ int wgt[kWaves], weq[kWaves];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remain, s_nbin, s_found, s_cnt;
    const int b = row0 + blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the range bounds stay scalar
    const int L = prefill ? b % T + 1 : seq_len_of(seq_lens, b, T);
    const float *sc = scores + (long)blockIdx.x * T;
    int32_t *out = sel + (long)b * topk;
    if (L <= topk) {
        for (int i = tid; i < topk; i += kTopkThreads) out[i] = i < L ? i : -1;
        return;
    }
    // wave w owns the contiguous 64-aligned range [lo, hi): the compaction
    // reads it in order, and with NR > 0 its lane l caches positions lo + 64 i + l
    const int per = ((L + kWaves - 1) / kWaves + 63) / 64 * 64;
    const int lo = min(L, wave * per), hi = min(L, lo + per);
    // Key 0 marks a slot past the range: every real score's key is at least
    // order_key(-inf) = 0x007fffff (top digit 7), so with more than k real
    // keys the k-th largest never falls to it; after the first digit it
    // matches no prefix, and it is never kept.
    // The loads go through a buffer resource bounded by the row's length (the
    // hardware returns 0 past it), one address register and a constant offset
    // each, so they are issued back to back without a branch each.
    uint32_t uc[NR > 0 ? NR : 1];
    int nch = (hi - lo + 63) >> 6;   // 64-slot steps of this wave's range
    if constexpr (NR > 0) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)sc, 0, L * 4, 0x00020000);
        const int voff = (lo + lane) * 4;
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++) uc[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 256 * i, 0);
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++) {
            asm volatile("" : "+v"(uc[i]));   // every load issued unconditionally, none sunk into a branch
            uc[i] = lane < hi - lo - 64 * i ? order_key(__uint_as_float(uc[i])) : 0u;
            asm volatile("" : "+v"(uc[i]));   // the key formed once, not again at every use
        }
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    // After a histogram of `bins` digits at `shift` under prefix `pre`: the
    // digit holding the rem-th largest counted key (s_found stays 0 when fewer
    // than rem keys were counted), and how many keys share it.
    auto find_digit = [&](int bins, int shift, uint32_t pre, int rem) {
        int c[4], own = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int dgt = bins - 1 - 4 * tid - i;
            c[i] = dgt >= 0 ? hist[dgt] : 0;
            own += c[i];
        }
        int tot;
        int above = block_exscan(own, wsum, &tot);   // keys with a higher digit than this thread's first
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (above < rem && above + c[i] >= rem) {
                s_prefix = pre | ((uint32_t)(bins - 1 - 4 * tid - i) << shift);
                s_remain = rem - above;
                s_nbin = c[i];
                s_found = 1;
            }
            above += c[i];
        }
        __syncthreads();
    };
    if constexpr (NR > 0) {
        // (a) the sample's first digits
        for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
        if (tid == 0) {
            s_found = 0;
            s_cnt = 0;
        }
        __syncthreads();
        asm volatile("" : "+s"(nch));
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i += 8)
            if (i < nch) hist_add(hist, (int)(uc[i] >> 20), uc[i] != 0u);
        __syncthreads();
        // about 4 standard deviations above the sample's expected share of k
        find_digit(4096, 20, 0u, topk / 8 + topk / 32 + 16);
        const uint32_t tau = s_found ? max(s_prefix, 1u) : 1u;   // key 0 (past the range) never qualifies
        // (b) candidates into LDS: each lane counts its own, a wave scan gives
        // each lane its offset after one reservation per wave, and each lane
        // writes its candidates in turn (the list's order does not matter).
        // Key 0, past the range, is below tau >= 1: no range test is needed.
        int cl = 0;
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++) cl += uc[i] >= tau ? 1 : 0;
        int x = cl;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        int base = 0;
        if (lane == 63) base = atomicAdd(&s_cnt, x);   // x is the wave's total in lane 63
        int off = __shfl(base, 63) + x - cl;
        int pos0 = lo + lane;
        uint32_t tau2 = tau;
        // positions formed at the writes, and the comparisons made again
        // rather than NR flags held from the counting loop
        asm volatile("" : "+v"(pos0), "+v"(tau2));
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++) {
            const bool c = uc[i] >= tau2;
            if (c && off < kCap) {
                cand_k[off] = uc[i];
                cand_p[off] = (uint16_t)(pos0 + 64 * i);
            }
            off += c ? 1 : 0;
        }
        __syncthreads();
        const int C = s_cnt;
        if (C >= topk && C <= kCap) {
            // (c) radix select among the candidates: the k-th largest of the
            // row is the k-th largest of them, every other key being smaller
            uint32_t prefix = 0, mask = 0;
            int remain = topk, nbin = 0;
            for (int pass = 0; pass < 3; pass++) {
                const int shift = pass == 0 ? 20 : pass == 1 ? 8 : 0;
                const int bins = pass == 2 ? 256 : 4096;
                for (int i = tid; i < bins; i += kTopkThreads) hist[i] = 0;
                __syncthreads();
                for (int j0 = 0; j0 < C; j0 += kTopkThreads) {   // whole waves, for the aggregation
                    const int j = j0 + tid;
                    const uint32_t u = j < C ? cand_k[j] : 0u;
                    hist_add(hist, (int)((u >> shift) & (bins - 1)), j < C && (u & mask) == prefix);
                }
                __syncthreads();
                find_digit(bins, shift, prefix, remain);
                prefix = s_prefix;
                remain = s_remain;
                nbin = s_nbin;
                mask |= (uint32_t)(bins - 1) << shift;
                __syncthreads();
            }
            // (d) kept positions as bits (A: above the k-th key, and the keys
            // equal to it when all of them are kept; B: the equal keys when
            // only the lowest `remain` positions among them are), then out in
            // ascending order, two bitmap words per thread
            uint32_t *A = (uint32_t *)hist, *Bq = (uint32_t *)hist + 2048;
            for (int i = tid; i < 4096; i += kTopkThreads) hist[i] = 0;
            __syncthreads();
            const bool all_eq = nbin == remain;
            for (int j = tid; j < C; j += kTopkThreads) {
                const uint32_t u = cand_k[j], p = cand_p[j];
                if (u > prefix || (u == prefix && all_eq)) atomicOr(&A[p >> 5], 1u << (p & 31));
                else if (u == prefix) atomicOr(&Bq[p >> 5], 1u << (p & 31));
            }
            __syncthreads();
            const int w0 = 2 * tid, w1 = w0 + 1;
            uint32_t a0 = A[w0], a1 = A[w1];
            int tot;
            if (!all_eq) {
                const uint32_t b0 = Bq[w0], b1 = Bq[w1];
                int ex = block_exscan(__popc(b0) + __popc(b1), wsum, &tot);
                a0 |= lowest_bits(b0, remain - ex);
                ex += __popc(b0);
                a1 |= lowest_bits(b1, remain - ex);
            }
            int at = block_exscan(__popc(a0) + __popc(a1), wsum, &tot);
            for (uint32_t bits = a0; bits; bits &= bits - 1) out[at++] = 32 * w0 + __builtin_ctz(bits);
            for (uint32_t bits = a1; bits; bits &= bits - 1) out[at++] = 32 * w1 + __builtin_ctz(bits);
            return;
        }
    }
    // radix select of the k-th largest key: digits of 12, 12 and 8 bits
    uint32_t prefix = 0, mask = 0;
    int remain = topk;   // how many of the keys matching the prefix are still to be taken
    for (int pass = 0; pass < 3; pass++) {
        const int shift = pass == 0 ? 20 : pass == 1 ? 8 : 0;
        const int bins = pass == 2 ? 256 : 4096;
        for (int i = tid; i < bins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        if constexpr (NR > 0) {
            // a fresh copy of the step count per pass keeps the compiler from
            // holding NR loop-invariant conditions in scalar registers
            asm volatile("" : "+s"(nch));
#pragma clang loop unroll(full)
            for (int i = 0; i < NR; i++)   // key 0 adds to digit 0, below every real key's digit
                if (i < nch) hist_add(hist, (int)((uc[i] >> shift) & (bins - 1)), (uc[i] & mask) == prefix);
        } else {
            // 8 loads in flight per thread before their atomics
            for (int s0 = tid; s0 < L; s0 += 8 * kTopkThreads) {
                uint32_t u[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const int s = s0 + i * kTopkThreads;
                    u[i] = s < L ? order_key(sc[s]) : 0u;
                }
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    if (s0 + i * kTopkThreads < L && (u[i] & mask) == prefix)
                        atomicAdd(&hist[(u[i] >> shift) & (bins - 1)], 1);
                }
            }
        }
        __syncthreads();
        // thread t owns digits bins-1-4t .. bins-4-4t (high to low)
        int c[4], own = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int dgt = bins - 1 - 4 * tid - i;
            c[i] = dgt >= 0 ? hist[dgt] : 0;
            own += c[i];
        }
        int tot;
        int above = block_exscan(own, wsum, &tot);   // keys with a higher digit than this thread's first
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (above < remain && above + c[i] >= remain) {
                s_prefix = prefix | ((uint32_t)(bins - 1 - 4 * tid - i) << shift);
                s_remain = remain - above;
            }
            above += c[i];
        }
        __syncthreads();
        prefix = s_prefix;
        remain = s_remain;
        mask |= (uint32_t)(bins - 1) << shift;
        __syncthreads();
    }
    // ordered compaction: each wave counts its range (ballots), then writes
    // its kept positions in order after those of the waves before it
    int ngt = 0, neq = 0;
    if constexpr (NR > 0) {
        asm volatile("" : "+s"(nch));
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++) {
            if (i < nch) {
                ngt += __popcll(__ballot(uc[i] > prefix));
                neq += __popcll(__ballot(uc[i] == prefix));
            }
        }
    } else {
        for (int i0 = lo; i0 < hi; i0 += 4 * 64) {
            uint32_t u[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int s = i0 + 64 * i + lane;
                u[i] = s < hi ? order_key(sc[s]) : 0u;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int s = i0 + 64 * i + lane;
                ngt += __popcll(__ballot(s < hi && u[i] > prefix));
                neq += __popcll(__ballot(s < hi && u[i] == prefix));
            }
        }
    }
    if (lane == 0) {
        wgt[wave] = ngt;
        weq[wave] = neq;
    }
    __syncthreads();
    int eq_before = 0, pos = 0;
    for (int w = 0; w < wave; w++) {
        const int take = max(0, min(weq[w], remain - eq_before));
        pos += wgt[w] + take;
        eq_before += weq[w];
    }
    const int take_eq = max(0, min(neq, remain - eq_before));
    int eq_seen = 0;
    auto emit = [&](int s, uint32_t u) {   // u = 0 past the range (never kept)
        const bool g = u > prefix, e = u == prefix;
        const unsigned long long em = __ballot(e);
        const bool keep = g || (e && eq_seen + (int)__popcll(em & below) < take_eq);
        const unsigned long long km = __ballot(keep);
        if (keep) out[pos + __popcll(km & below)] = s;
        pos += __popcll(km);
        eq_seen += __popcll(em);
    };
    if constexpr (NR > 0) {
        asm volatile("" : "+s"(nch));
#pragma clang loop unroll(full)
        for (int i = 0; i < NR; i++)
            if (i < nch) emit(lo + 64 * i + lane, uc[i]);
    } else {
        for (int i0 = lo; i0 < hi; i0 += 4 * 64) {
            uint32_t u[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int s = i0 + 64 * i + lane;
                u[i] = s < hi ? order_key(sc[s]) : 0u;
            }
#pragma unroll
            for (int i = 0; i < 4; i++) emit(i0 + 64 * i + lane, u[i]);
        }
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(kAttnWaves * 64) void k_dsa_attn(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ k,
                                                             const uint16_t *__restrict__ v,
                                                             const int32_t *__restrict__ sel, uint16_t *__restrict__ o,
                                                             int T, int Hkv, int topk, float scale, int prefill,
                                                             int nsplit, float *__restrict__ part)
{
    constexpr int NQ = DK / 32, NO = DV / 16, VS = DV + 16;
    constexpr int kStage = 32 * VS;                       // bf16 per wave
    constexpr int kMerge = 16 * DV * (int)sizeof(float) / 2;   // the same bytes, counted in bf16
    __shared__ __align__(16) uint16_t vst[kAttnWaves][kStage > kMerge ? kStage : kMerge];
    extern __shared__ int ss[];   // this workgroup's share of the selection (dynamic: ceil(topk / nsplit))
    __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bg = blockIdx.x / nsplit, half = blockIdx.x % nsplit, b = bg / Hkv, g = bg % Hkv;
    const int span = (topk + nsplit - 1) / nsplit;
    const int h0 = half * span, h1 = min(topk, h0 + span);
    for (int i = tid; i < h1 - h0; i += kAttnWaves * 64) ss[i] = sel[(long)b * topk + h0 + i];
    // B operand Q^T: head li of the group, columns 32 c + 8 lg .. +7
    u32x4 qf[NQ];
    const long qrow = ((long)b * Hkv * 16 + g * 16 + li) * DK;
#pragma unroll
    for (int c = 0; c < NQ; c++) qf[c] = ld16(q + qrow + 32 * c + 8 * lg);
    __syncthreads();
    const long cbg = (long)(prefill ? b / T : b) * Hkv + g;   // the cache of this row
    const uint16_t *K = k + cbg * T * DK;
    const uint16_t *V = v + cbg * T * DV;
    uint16_t *vw = vst[wave];
    const float sl2 = scale * kLog2e;
    f32x4 acc[NO];
#pragma unroll
    for (int i = 0; i < NO; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    const int per = (max(h1 - h0, 0) + kAttnWaves - 1) / kAttnWaves;
    const int beg = h0 + wave * per, end = min(h1, beg + per);
    const int trow = li >> 2, tcol = 4 * (li & 3);
    for (int c0 = beg; c0 < end; c0 += 32) {
        float sc[2][4];
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            // A operand K: slot c0 + 16 kt + li (an empty slot, or an entry
            // outside the cache, reads token 0 and is masked below)
            const int slot = c0 + 16 * kt + li;
            const int tok = slot < end ? ss[slot - h0] : -1;
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
                const bool ok = sl < end && ss[sl - h0] >= 0 && ss[sl - h0] < T;
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
        if (nsplit == 1) {
            o[((long)b * Hkv * 16 + g * 16) * DV + i] = f2bf(den > 0.f ? num / den : 0.f);
        } else {
            // [16 max][16 sum][16][DV] unnormalised O, per (group, split)
            float *pw = part + (long)blockIdx.x * (32 + 16 * DV);
            if (i % DV == 0) {
                pw[h] = M;
                pw[16 + h] = den;
            }
            pw[32 + i] = num;
        }
    }
}

// o = the splits' (max, sum, O) combined, per (sequence, KV group)
template <int DV>
__global__ __launch_bounds__(kThreads) void k_dsa_merge(const float *__restrict__ part, uint16_t *__restrict__ o,
                                                        int nsplit)
{
    const int bg = blockIdx.x;
    const float *p0 = part + (long)(nsplit * bg) * (32 + 16 * DV);
    const int i = blockIdx.y * kThreads + threadIdx.x, h = i / DV;   // grid.y = 16 DV / 256
    float M = -INFINITY;
    for (int r = 0; r < nsplit; r++) M = fmaxf(M, p0[r * (32 + 16 * DV) + h]);
    float num = 0.f, den = 0.f;
    for (int r = 0; r < nsplit; r++) {
        const float *pr = p0 + r * (32 + 16 * DV);
        const float f = pr[h] == -INFINITY ? 0.f : fast_exp2(pr[h] - M);
        num = __builtin_fmaf(f, pr[32 + i], num);
        den = __builtin_fmaf(f, pr[16 + h], den);
    }
    o[(long)bg * 16 * DV + i] = f2bf(den > 0.f ? num / den : 0.f);
}

}  // namespace

bool dsa_supported(const Dims &d)
{
    return d.dtype == NSA_BF16 && d.G == 16 &&
           ((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64));
}

hipError_t launch_dsa_select(const Dims &d, int HI, int DI, int topk, const int32_t *seq_lens, const void *q_idx,
                             const void *w_idx, const void *k_idx, float *scores, int32_t *sel, hipStream_t s,
                             bool prefill, int row0, int rows)
{
    const int pf = prefill ? 1 : 0;
    if (rows < 0) rows = prefill ? d.B * d.T : d.B;
    const dim3 grid(rows, (d.T + kThreads - 1) / kThreads);
    const uint16_t *qi = (const uint16_t *)q_idx, *wi = (const uint16_t *)w_idx, *ki = (const uint16_t *)k_idx;
    if (DI <= 32) hipLaunchKernelGGL(k_dsa_index<1>, grid, dim3(kThreads), 0, s, qi, wi, ki, seq_lens, scores, d.T, HI, DI, pf, row0);
    else if (DI <= 64) hipLaunchKernelGGL(k_dsa_index<2>, grid, dim3(kThreads), 0, s, qi, wi, ki, seq_lens, scores, d.T, HI, DI, pf, row0);
    else if (DI <= 128) hipLaunchKernelGGL(k_dsa_index<4>, grid, dim3(kThreads), 0, s, qi, wi, ki, seq_lens, scores, d.T, HI, DI, pf, row0);
    else hipLaunchKernelGGL(k_dsa_index<8>, grid, dim3(kThreads), 0, s, qi, wi, ki, seq_lens, scores, d.T, HI, DI, pf, row0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // register-cached selection while a row fits in 64 scores per lane
    const dim3 tg(rows), tb(kTopkThreads);
    if (d.T <= 16 * kTopkThreads) hipLaunchKernelGGL(k_dsa_topk<16>, tg, tb, 0, s, scores, seq_lens, sel, d.T, topk, pf, row0);
    else if (d.T <= 32 * kTopkThreads) hipLaunchKernelGGL(k_dsa_topk<32>, tg, tb, 0, s, scores, seq_lens, sel, d.T, topk, pf, row0);
    else if (d.T <= 64 * kTopkThreads) hipLaunchKernelGGL(k_dsa_topk<64>, tg, tb, 0, s, scores, seq_lens, sel, d.T, topk, pf, row0);
    else hipLaunchKernelGGL(k_dsa_topk<0>, tg, tb, 0, s, scores, seq_lens, sel, d.T, topk, pf, row0);
    return hipGetLastError();
}

int dsa_prefill_chunk_rows(const Dims &d)
{
    const long total = (long)d.B * d.T;
    const long fit = (long)(kDsaScoreBudget / (sizeof(float) * (size_t)d.T));
    return (int)std::max(1L, std::min(total, fit));
}

size_t dsa_split_bytes(const Dims &d, int nsplit)
{
    return sizeof(float) * (size_t)d.B * d.Hkv * nsplit * (32 + 16 * (size_t)d.dv);
}

hipError_t launch_dsa_attn(const Dims &d, int topk, const void *q, const void *k, const void *v, const int32_t *sel,
                           void *o, hipStream_t s, bool prefill, void *part, int nsplit)
{
    const int pf = prefill ? 1 : 0, ns = part ? nsplit : 1;
    const long groups = (prefill ? (long)d.B * d.T : (long)d.B) * d.Hkv;
    const dim3 grid((unsigned)(groups * ns)), block(kAttnWaves * 64);
    const size_t lds = sizeof(int) * (size_t)((topk + ns - 1) / ns);
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *oo = (uint16_t *)o;
    float *pp = (float *)part;
    if (d.dk == 192) hipLaunchKernelGGL((k_dsa_attn<192, 128>), grid, block, lds, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale, pf, ns, pp);
    else if (d.dk == 128) hipLaunchKernelGGL((k_dsa_attn<128, 128>), grid, block, lds, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale, pf, ns, pp);
    else hipLaunchKernelGGL((k_dsa_attn<64, 64>), grid, block, lds, s, qq, kk, vv, sel, oo, d.T, d.Hkv, topk, d.scale, pf, ns, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    if (d.dv == 128) hipLaunchKernelGGL(k_dsa_merge<128>, dim3((unsigned)groups, 16 * 128 / kThreads), dim3(kThreads), 0, s, pp, oo, ns);
    else hipLaunchKernelGGL(k_dsa_merge<64>, dim3((unsigned)groups, 16 * 64 / kThreads), dim3(kThreads), 0, s, pp, oo, ns);
    return hipGetLastError();
}

}  // namespace nsa
