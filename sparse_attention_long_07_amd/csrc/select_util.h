// Top-n block selection for one (position, KV head) row by one wavefront
// (valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션 기술
// 화제", section II: n blocks including the initial block and 2 local blocks).
//
// Candidates are blocks 0..jc (jc = t/64).  Blocks 0, jc-1 and jc are always
// kept; the other n - #kept are chosen one at a time by a wavefront argmax
// (higher score first, lower block on ties).  Lane L owns blocks L, L+64, ...;
// the first 16 of them are cached in registers.  The argmax reduces within
// each row of 16 lanes with DPP moves and across the four rows with
// readlane.  The chosen set is written in ascending order with a ballot
// prefix count and padded with -1.
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
        float cache[16];
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            const int j = lane + 64 * rr;
            float v = j < ncand ? S[j] : -INFINITY;
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

}  // namespace nsa
