// Top-n block selection for one (position, KV head) row by one wavefront
// (valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션 기술
// 화제", section II: n blocks including the initial block and 2 local blocks).
//
// Candidates are blocks 0..jc (jc = t/64).  Blocks 0, jc-1 and jc are always
// kept; the other k = n - #kept are the highest-scoring remaining blocks
// (lower block on ties).  Two routines give the same result:
//  * wave_select_topn: k rounds of a wavefront argmax.  Lane L owns blocks
//    L, L+64, ...; the first 16 of them are cached in registers.  The argmax
//    reduces within each row of 16 lanes with DPP moves and across the four
//    rows with readlane.  Any number of candidates.
//  * wave_select_topn_fast (up to 1024 candidates): a threshold search.  The
//    k-th largest of the 64 per-lane maxima bounds the k-th largest score from
//    below, so every block scoring at least that much is a candidate (usually
//    a few more than k).  Those are compacted into LDS in ascending block
//    order, and the k-th largest score among them is found by bisection on the
//    order-preserving integer image of the scores, counting with ballots; ties
//    at that score go to the lowest blocks.  Falls back to the argmax rounds
//    when more than 64 blocks pass the first threshold.
//  * wave_select_topn_sort (any number of candidates): the same threshold
//    idea with sorts instead of bisections.  Each candidate gets a distinct
//    64-bit key, its score's order-preserving image above the complement of
//    its block, so a larger key is a better block and equal scores rank the
//    lower block first.  A bitonic sort of the 64 lane maxima gives the
//    threshold; the candidates at or above it are compacted and sorted, and
//    the first k are taken.  Two 21-stage sorts replace two 32-step
//    bisections whose every step waited on a ballot.
// The chosen set is written in ascending order and padded with -1.
#pragma once

#include "mfma_util.h"

namespace nsa {


template <int CTRL>
__device__ __forceinline__ int dppi(int x)
{
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ void keep_better(float &s, int &j, float os, int oj)
{
    if (os > s || (os == s && oj < j)) {
        s = os;
        j = oj;
    }
}

// Wavefront-wide argmax of (s desc, j asc); every lane returns the winner.
__device__ __forceinline__ int wave_argmax(float s, int j)
{
    keep_better(s, j, dpp<kQuadXor1>(s), dppi<kQuadXor1>(j));
    keep_better(s, j, dpp<kQuadXor2>(s), dppi<kQuadXor2>(j));
    keep_better(s, j, dpp<kRowHalfMirror>(s), dppi<kRowHalfMirror>(j));
    keep_better(s, j, dpp<kRowMirror>(s), dppi<kRowMirror>(j));
    float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 0));
    int bj = __builtin_amdgcn_readlane(j, 0);
#pragma unroll
    for (int r = 1; r < 4; r++) {
        const float os = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 16 * r));
        const int oj = __builtin_amdgcn_readlane(j, 16 * r);
        keep_better(bs, bj, os, oj);
    }
    return bj;
}

// S: scores of the row (global or LDS), valid for j <= jcur.  ncand <= 8192.
__device__ __forceinline__ void wave_select_topn(const float *S, int jcur, int n, int32_t *out, int lane)
{
    const int ncand = jcur + 1;
    const int nforced = jcur == 0 ? 1 : (jcur == 1 ? 2 : 3);
    const int k = n - nforced;
    const int RR = (ncand + 63) / 64;
    uint64_t c0 = 0, c1 = 0;   // chosen flags of rr = 0..63 and 64..127
    auto setbit = [&](int rr) {
        if (rr < 64) c0 |= 1ull << rr;
        else c1 |= 1ull << (rr - 64);
    };
    auto getbit = [&](int rr) { return rr < 64 ? (c0 >> rr) & 1ull : (c1 >> (rr - 64)) & 1ull; };
    if (lane == 0) setbit(0);
    if (jcur >= 1 && (jcur - 1) % 64 == lane) setbit((jcur - 1) / 64);
    if (jcur % 64 == lane) setbit(jcur / 64);
    if (ncand - nforced <= k) {
        for (int rr = 0; rr < RR; rr++)
            if (lane + rr * 64 < ncand) setbit(rr);
    } else {
        // unconditional loads at clamped (valid) indices, so all 16 are in
        // flight at once; entries past jc are masked afterwards
        float cache[16];
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            const int j = lane + 64 * rr;
            const float sv = S[j < ncand ? j : ncand - 1];
            const float v = j < ncand ? sv : -INFINITY;
            cache[rr] = v == v ? v : -INFINITY;
        }
        for (int round = 0; round < k; round++) {
            float bs = -INFINITY;
            int bj = 0x7fffffff;
#pragma unroll
            for (int rr = 0; rr < 16; rr++) {
                const int j = lane + 64 * rr;
                if (j < ncand && !getbit(rr)) keep_better(bs, bj, cache[rr], j);
            }
            for (int rr = 16; rr < RR; rr++) {
                const int j = lane + 64 * rr;
                if (j < ncand && !getbit(rr)) {
                    float v = S[j];
                    keep_better(bs, bj, v == v ? v : -INFINITY, j);
                }
            }
            const int w = wave_argmax(bs, bj);
            if (w % 64 == lane) setbit(w / 64);
        }
    }
    int base = 0;
    const uint64_t lt = __lanemask_lt();
    for (int rr = 0; rr < RR; rr++) {
        const bool bit = getbit(rr) && (lane + rr * 64 < ncand);
        const uint64_t bal = __ballot(bit);
        if (bit) out[base + __popcll(bal & lt)] = lane + rr * 64;
        base += __popcll(bal);
    }
    for (int qq = base + lane; qq < n; qq += 64) out[qq] = -1;
}

// Integer image of a float that orders like the float (NaN maps below -inf).
__device__ __forceinline__ uint32_t ordered_key(float v)
{
    if (v != v) return 0u;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest x with at least k lanes (of those with `valid`) holding key >= x.
// Requires at least k valid lanes.  32 bisection steps on wave-uniform bounds.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t key, bool valid, int k)
{
    // k is the same on every lane; saying so keeps the bounds and the loop in
    // scalar registers (otherwise every step runs as a divergent vector loop)
    k = __builtin_amdgcn_readfirstlane(k);
    uint32_t lo = 0u, hi = 0xffffffffu;
    while (lo < hi) {
        const uint32_t mid = lo + (uint32_t)(((uint64_t)hi - lo + 1u) >> 1);
        const int cnt = __popcll(__ballot(valid && key >= mid));
        if (cnt >= k) lo = mid;
        else hi = mid - 1u;
    }
    return lo;
}

// cand: 64 entries of LDS scratch owned by this wavefront.
__device__ __forceinline__ void wave_select_topn_fast(const float *S, int jcur, int n, int32_t *out, int lane,
                                                      uint2 *cand)
{
    jcur = __builtin_amdgcn_readfirstlane(jcur);   // one row per wavefront: uniform
    n = __builtin_amdgcn_readfirstlane(n);
    const int ncand = jcur + 1;
    const int nforced = jcur == 0 ? 1 : (jcur == 1 ? 2 : 3);
    const int k = n - nforced;
    if (ncand > 1024 || ncand - nforced <= k || k <= 0) {
        wave_select_topn(S, jcur, n, out, lane);
        return;
    }
    // keys of this lane's blocks j = lane + 64 rr; forced blocks and blocks past jc excluded
    uint32_t key[16];
    bool ok[16];
    uint32_t lmax = 0u;
    bool lvalid = false;
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        const int j = lane + 64 * rr;
        const float sv = S[j < ncand ? j : ncand - 1];   // unconditional: all loads in flight at once
        ok[rr] = j < ncand && j != 0 && j != jcur && j != jcur - 1;
        key[rr] = ok[rr] ? ordered_key(sv) : 0u;
        if (ok[rr] && (!lvalid || key[rr] > lmax)) lmax = key[rr];
        lvalid |= ok[rr];
    }
    // at least k lanes hold a free candidate (k <= 13 and every lane but the
    // last few holds one once more than k + 3 blocks exist)
    if (__popcll(__ballot(lvalid)) < k) {
        wave_select_topn(S, jcur, n, out, lane);
        return;
    }
    const uint32_t x = wave_kth_largest(lmax, lvalid, k);
    // compact blocks with key >= x, ascending j
    const uint64_t lt = __lanemask_lt();
    int C = 0;
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        const bool p = ok[rr] && key[rr] >= x;
        const uint64_t bal = __ballot(p);
        const int pos = C + __popcll(bal & lt);
        if (p && pos < 64) cand[pos] = make_uint2(key[rr], (uint32_t)(lane + 64 * rr));
        C += __popcll(bal);
    }
    if (C > 64) {
        wave_select_topn(S, jcur, n, out, lane);
        return;
    }
    __builtin_amdgcn_wave_barrier();
    const bool have = lane < C;
    const uint2 cv = have ? cand[lane] : make_uint2(0u, 0u);
    // k-th largest score among the candidates; all above it are taken, and
    // the lowest blocks among those equal to it fill up to k
    const uint32_t sk = wave_kth_largest(cv.x, have, k);
    const bool above = have && cv.x > sk;
    const int nabove = __popcll(__ballot(above));
    const bool tie = have && cv.x == sk;
    const uint64_t tb = __ballot(tie);
    const bool take = above || (tie && (int)__popcll(tb & lt) < k - nabove);
    // Here jc >= 2, so the forced blocks are 0 < (chosen blocks) < jc-1 < jc:
    // out = 0, the k chosen blocks ascending, jc-1, jc.
    const uint64_t tk = __ballot(take);
    if (take) out[1 + __popcll(tk & lt)] = (int)cv.y;
    if (lane == 0) {
        out[0] = 0;
        out[k + 1] = jcur - 1;
        out[k + 2] = jcur;
    }
    for (int q = nforced + k + lane; q < n; q += 64) out[q] = -1;
}

// Candidate key: the score's order-preserving image above the complement of
// the block, so distinct blocks have distinct keys, larger is better and
// equal scores rank the lower block first.  0 is no candidate.
__device__ __forceinline__ uint64_t cand_key(float s, int j)
{
    return ((uint64_t)ordered_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m)
{
    const int lo = __shfl_xor((int)(uint32_t)v, m, 64), hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
    return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

// Bitonic sort of one 64-bit key per lane over the wavefront, descending
// (lane 0 ends with the largest).  At stage (k, j) lane i and lane i ^ j
// compare; within a run of k lanes that ends descending the lower lane keeps
// the larger key.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane)
{
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint64_t o = shfl_xor64(v, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
        }
    return v;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// cand: 64 entries of LDS scratch owned by this wavefront.  Same result as
// wave_select_topn.
__device__ __forceinline__ void wave_select_topn_sort(const float *S, int jcur, int n, int32_t *out, int lane,
                                                      uint64_t *cand)
{
    jcur = __builtin_amdgcn_readfirstlane(jcur);   // one row per wavefront: uniform
    n = __builtin_amdgcn_readfirstlane(n);
    const int ncand = jcur + 1;
    const int nforced = jcur == 0 ? 1 : (jcur == 1 ? 2 : 3);
    const int k = n - nforced;
    if (ncand - nforced <= k || k <= 0) {
        wave_select_topn(S, jcur, n, out, lane);   // every block is taken
        return;
    }
    const int RR = (ncand + 63) / 64;
    auto key_of = [&](int j) -> uint64_t {
        const float v = S[j < ncand ? j : ncand - 1];   // unconditional: the loads go out together
        const bool ok = j < ncand && j != 0 && j != jcur && j != jcur - 1;
        return ok ? cand_key(v, j) : 0ull;
    };
    // this lane's blocks j = lane + 64 rr: the first 16 kept in registers
    uint64_t kc[16];
    uint64_t lmax = 0ull;
#pragma unroll
    for (int rr = 0; rr < 16; rr++) {
        kc[rr] = key_of(lane + 64 * rr);
        lmax = kc[rr] > lmax ? kc[rr] : lmax;
    }
    for (int rr = 16; rr < RR; rr++) {
        const uint64_t kv = key_of(lane + 64 * rr);
        lmax = kv > lmax ? kv : lmax;
    }
    // the k-th largest lane maximum: at least k candidates reach it
    const uint64_t x = readlane64(wave_sort_desc(lmax, lane), k - 1);
    // the candidates at or above it, compacted in block order
    const uint64_t lt = __lanemask_lt();
    int C = 0;
    auto take = [&](uint64_t kv) {
        const bool p = kv != 0ull && kv >= x;
        const uint64_t bal = __ballot(p);
        const int pos = C + __popcll(bal & lt);
        if (p && pos < 64) cand[pos] = kv;
        C += __popcll(bal);
    };
#pragma unroll
    for (int rr = 0; rr < 16; rr++) take(kc[rr]);
    for (int rr = 16; rr < RR; rr++) take(key_of(lane + 64 * rr));
    if (x == 0ull || C > 64) {
        wave_select_topn(S, jcur, n, out, lane);
        return;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the compacted keys are in LDS
    __builtin_amdgcn_wave_barrier();
    const uint64_t top = wave_sort_desc(lane < C ? cand[lane] : 0ull, lane);
    // lanes 0 .. k-1 hold the picks; write them in ascending block order
    const int jl = (int)(0xFFFFFFFFu - (uint32_t)top);
    int rank = 0;
    for (int m = 0; m < k; m++) {
        const int jm = __builtin_amdgcn_readlane(jl, m);
        rank += jm < jl ? 1 : 0;
    }
    // Here jc >= 2, so the forced blocks are 0 < (chosen blocks) < jc-1 < jc
    if (lane < k) out[1 + rank] = jl;
    if (lane == 0) {
        out[0] = 0;
        out[k + 1] = jcur - 1;
        out[k + 2] = jcur;
    }
    for (int q = nforced + k + lane; q < n; q += 64) out[q] = -1;
}

}  // namespace nsa
