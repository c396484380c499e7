// NSA decode step on the matrix cores (bf16 storage, 16 query heads per KV
// head).  valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션
// 기술 화제", section III.3: a 64k-context decode step reads the keys and
// values of 5,632 tokens instead of 65,536 -- the compressed cache, the
// selected blocks and the window.  The step is bound by HBM bandwidth, so
// the work is split along the keys across many workgroups (split-K) and
// merged afterwards:
//   phase A  compressed slots (256 per workgroup) and the window (256 keys
//            per workgroup): per-workgroup (max, sum, unnormalised output),
//            plus, for the compressed slots, each block's importance terms;
//   phase B  per (sequence, KV head): exact log-sum-exp over the compressed
//            splits, o_cmp, block scores (heads summed, weights 1,2,2,2,1)
//            and the top-n selection;
//   phase C  the selected blocks (4 per workgroup, one per wavefront);
//   phase D  merge of the compressed, window and selected partials and the
//            gated sum.
// Every wavefront issues all loads of its 64 keys (K into MFMA operand
// registers, V into registers for the LDS transpose) before it computes, so
// each one keeps 40 KB in flight.
//
// Lane view (one position, 16 heads, wave64): head hd = lane%16, key group
// q = lane/16.  A 32-key step is two 16x16x32 S^T tiles whose rows hold keys
// 8*(i/4) + i%4 and 8*(i/4) + 4 + i%4, so lane (q, hd) ends with the logits
// of keys 8q .. 8q+7 of the step for head hd: exactly the B operand of
// O^T = V^T P^T.  V is transposed through a per-wave LDS tile.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaveKeys = 64;                // keys per wavefront (two 32-key steps)
constexpr int kSplitKeys = 4 * kWaveKeys;    // keys per phase-A workgroup
constexpr int kSelPerWg = 4;                 // selected blocks per phase-C workgroup
constexpr int kVtS = 40;                     // bf16 per V^T row in LDS (32 keys + pad)

__device__ __forceinline__ float sigmoidf_(float z) { return 1.f / (1.f + __expf(-z)); }

__device__ __forceinline__ int dec_t(const int32_t *seq_lens, int b, int T)
{
    int L = seq_lens[b];
    L = L < 1 ? 1 : (L > T ? T : L);
    return L - 1;
}

template <int DK>
__device__ __forceinline__ void load_qf(const uint16_t *qrow, int q, bf16x8 (&qf)[DK / 32])
{
#pragma unroll
    for (int kk = 0; kk < DK / 32; kk++) qf[kk] = as_bf16x8(ld16(qrow + 32 * kk + 8 * q));
}

// Raw logits of keys base + 8q .. base + 8q + 7 for head hd (rows clamped
// to kclamp so every load stays inside the cache; callers mask).
template <int DK>
__device__ __forceinline__ void logits_step(const uint16_t *K, int base, int kclamp, const bf16x8 (&qf)[DK / 32],
                                            int hd, int q, float (&s)[8])
{
    const int kr = 8 * (hd >> 2) + (hd & 3);
    const int kA = min(base + kr, kclamp), kB = min(base + kr + 4, kclamp);
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; kk++) {
        accA = mfma16(as_bf16x8(ld16(K + (long)kA * DK + 32 * kk + 8 * q)), qf[kk], accA);
        accB = mfma16(as_bf16x8(ld16(K + (long)kB * DK + 32 * kk + 8 * q)), qf[kk], accB);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
        s[u] = accA[u];
        s[4 + u] = accB[u];
    }
}

// V rows base .. base+31: four (key pair, 8-dv chunk) tasks per lane,
// loaded into registers, later written transposed to vt[dv][key].
template <int DV>
struct VRegs {
    static constexpr int N = 16 * (DV / 8) / 64;   // tasks per lane
    u32x4 v0[N], v1[N];
};

template <int DV>
__device__ __forceinline__ void load_v(const uint16_t *V, int base, int kclamp, int lane, VRegs<DV> &r)
{
#pragma unroll
    for (int i = 0; i < VRegs<DV>::N; i++) {
        const int task = lane + 64 * i, kp = task & 15, dc = task >> 4;
        const int k0 = min(base + 2 * kp, kclamp), k1 = min(base + 2 * kp + 1, kclamp);
        r.v0[i] = ld16(V + (long)k0 * DV + dc * 8);
        r.v1[i] = ld16(V + (long)k1 * DV + dc * 8);
    }
}

template <int DV>
__device__ __forceinline__ void store_vt(const VRegs<DV> &r, uint16_t *vt, int lane)
{
#pragma unroll
    for (int i = 0; i < VRegs<DV>::N; i++) {
        const int task = lane + 64 * i, kp = task & 15, dc = task >> 4;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t x0 = (r.v0[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            const uint32_t x1 = (r.v1[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            *(uint32_t *)&vt[(dc * 8 + e) * kVtS + 2 * kp] = x0 | (x1 << 16);
        }
    }
}

template <int DV>
__device__ __forceinline__ void pv_step(const uint16_t *vt, const float (&p)[8], int hd, int q,
                                        f32x4 (&oacc)[DV / 16])
{
    const bf16x8 pb = pack8(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++)
        oacc[dt] = mfma16(as_bf16x8(ld16(vt + (16 * dt + hd) * kVtS + 8 * q)), pb, oacc[dt]);
}

__device__ __forceinline__ float head_max(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float head_sum(float x)
{
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

template <int DV>
struct DecLds {
    union {
        uint16_t vt[4][2 * DV * kVtS];   // two 32-key steps per wavefront
        float ol[4][16][DV];
    } u;
    float mx[4][16];
    float ls[4][16];
};

// Workgroup-level merge of four wavefronts that used the same max M:
// sums l and O in wave order and writes (M, l, O) for the 16 heads.
template <int DV>
__device__ __forceinline__ void wg_store_partial(DecLds<DV> &sm, int wave, int lane, float M, float l,
                                                 const f32x4 (&oacc)[DV / 16], float *pm, float *pl, float *po)
{
    const int hd = lane & 15, q = lane >> 4;
    __syncthreads();   // the V^T tiles alias the merge buffer
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++)
#pragma unroll
        for (int u = 0; u < 4; u++) sm.u.ol[wave][hd][16 * dt + 4 * q + u] = oacc[dt][u];
    if (q == 0) sm.ls[wave][hd] = l;
    __syncthreads();
    const int tid = wave * 64 + lane;
    for (int e = tid; e < 16 * DV; e += kThreads) {
        const int h = e / DV, c = e % DV;
        po[e] = sm.u.ol[0][h][c] + sm.u.ol[1][h][c] + sm.u.ol[2][h][c] + sm.u.ol[3][h][c];
    }
    if (tid < 16) {
        pl[tid] = sm.ls[0][tid] + sm.ls[1][tid] + sm.ls[2][tid] + sm.ls[3][tid];
        pm[tid] = M;   // every lane of every wave holds the same M for head tid; see callers
    }
}

// ---------------------------------------------------------------------------
// Phase A.  Workgroup (pair, split): splits 0..CS-1 cover compressed slots
// [512 s, 512 s + 512), splits CS.. cover window keys from max(0, t-w+1).
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_phase_a(DecArgs A)
{
    __shared__ DecLds<DV> sm;
    const Dims &d = A.d;
    const int nsplit = A.cs + A.ws;
    const int pair = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = lane & 15, q = lane >> 4;
    const int t = dec_t(A.seq_lens, b, d.T);
    const bool cmp = split < A.cs;
    int kbeg, kend, kclamp;
    const uint16_t *K, *V;
    if (cmp) {
        const int nvis = t >= 31 ? (t - 31) / 16 + 1 : 0;
        kbeg = split * kSplitKeys + wave * kWaveKeys;
        kend = min(kbeg + kWaveKeys, nvis);
        kclamp = d.npad - 1;
        K = (const uint16_t *)A.kc + (long)pair * d.npad * DK;
        V = (const uint16_t *)A.vc + (long)pair * d.npad * DV;
    } else {
        const int lo = max(0, t - d.w + 1);
        kbeg = lo + (split - A.cs) * kSplitKeys + wave * kWaveKeys;
        kend = min(kbeg + kWaveKeys, t + 1);
        kclamp = d.T - 1;
        K = (const uint16_t *)A.k + (long)pair * d.T * DK;
        V = (const uint16_t *)A.v + (long)pair * d.T * DV;
    }
    const float sl2 = d.scale * kLog2e;
    bf16x8 qf[DK / 32];
    load_qf<DK>((const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK, q, qf);

    float s[2][8];
    VRegs<DV> vr[2];
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; st++) {
        const int base = kbeg + 32 * st;
        if (base < kend) {   // uniform over the wavefront
            load_v<DV>(V, base, kclamp, lane, vr[st]);
            logits_step<DK>(K, base, kclamp, qf, hd, q, s[st]);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                s[st][e] = base + 8 * q + e < kend ? s[st][e] * sl2 : -INFINITY;
                mx = fmaxf(mx, s[st][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) s[st][e] = -INFINITY;
        }
    }
    mx = head_max(mx);
    if (q == 0) sm.mx[wave][hd] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm.mx[0][hd], sm.mx[1][hd]), fmaxf(sm.mx[2][hd], sm.mx[3][hd]));
    float l = 0.f;
    f32x4 oacc[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t *vt = sm.u.vt[wave];
    float *bx = A.bx + (long)pair * 16 * A.nbp + (long)hd * A.nbp;
    float *by = A.by + (long)pair * 16 * A.nbp + (long)hd * A.nbp;
#pragma unroll
    for (int st = 0; st < 2; st++) {
        const int base = kbeg + 32 * st;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; e++) p[e] = M == -INFINITY ? 0.f : fast_exp2(s[st][e] - M);
        if (cmp) {
            // block a = (base + 8q)/4 gets keys 4a..4a+3 here (weights 2,2,2,1);
            // its remaining weight-1 key 4a-1 is the previous block's Y term
            const int a = (base + 8 * q) >> 2;
            if (a + 1 < A.nbp) {
                *(float2 *)&bx[a] = make_float2(2.f * (p[0] + p[1] + p[2]) + p[3], 2.f * (p[4] + p[5] + p[6]) + p[7]);
                *(float2 *)&by[a] = make_float2(p[3], p[7]);
            }
        }
        if (base < kend) {   // uniform over the wavefront
#pragma unroll
            for (int e = 0; e < 8; e++) l += p[e];
            store_vt<DV>(vr[st], vt + st * DV * kVtS, lane);
            pv_step<DV>(vt + st * DV * kVtS, p, hd, q, oacc);
        }
    }
    l = head_sum(l);
    const long pidx = (long)pair * nsplit + split;
    wg_store_partial<DV>(sm, wave, lane, M, l, oacc, A.pm + pidx * 16, A.pl + pidx * 16, A.po + pidx * 16 * DV);
}

// ---------------------------------------------------------------------------
// Phase B.  One workgroup per (sequence, KV head): the exact log-sum-exp of
// each head over the compressed splits, the block scores and the selection.
template <int DV>
__global__ __launch_bounds__(kThreads) void k_dec_phase_b(DecArgs A)
{
    extern __shared__ float S[];   // [nb] block scores
    __shared__ float wsp[64][16];  // weight exp2(m_split - lse) of split s for head h
    __shared__ float lse[16];
    const Dims &d = A.d;
    const int pair = blockIdx.x;
    const int b = pair / d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int jcur = t / 64;
    const int nsplit = A.cs + A.ws;
    const float *pm = A.pm + (long)pair * nsplit * 16, *pl = A.pl + (long)pair * nsplit * 16;
    if (tid < 16) {
        float M = -INFINITY;
        for (int s = 0; s < A.cs; s++) M = fmaxf(M, pm[s * 16 + tid]);
        float L = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < A.cs; s++) L += pl[s * 16 + tid] * fast_exp2(pm[s * 16 + tid] - M);
        lse[tid] = M == -INFINITY ? -INFINITY : M + fast_log2(L);
    }
    __syncthreads();
    for (int e = tid; e < A.cs * 16; e += kThreads) {
        const int s = e >> 4, h = e & 15;
        wsp[s][h] = lse[h] == -INFINITY ? 0.f : fast_exp2(pm[s * 16 + h] - lse[h]);
    }
    __syncthreads();
    // block j: its own keys 4j..4j+3 (X) plus key 4j-1 (Y of block j-1);
    // phase A wrote blocks 0..nbp-1, a block past them has no key of its own
    const float *bx = A.bx + (long)pair * 16 * A.nbp, *by = A.by + (long)pair * 16 * A.nbp;
    constexpr int kBlkPerSplit = kSplitKeys / 4;
    for (int j = tid; j <= jcur; j += kThreads) {
        const int sj = j / kBlkPerSplit, sp = (j - 1) / kBlkPerSplit;
        const bool hx = j < A.nbp, hy = j > 0 && j - 1 < A.nbp;
        float xv[16], yv[16];
#pragma unroll
        for (int h = 0; h < 16; h++) {
            xv[h] = hx ? bx[(long)h * A.nbp + j] : 0.f;
            yv[h] = hy ? by[(long)h * A.nbp + j - 1] : 0.f;
        }
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 16; h++) {
            acc += xv[h] * wsp[sj][h];
            if (hy) acc += yv[h] * wsp[sp][h];
        }
        S[j] = acc;
    }
    __syncthreads();
    if (A.idx_in) return;
    // top-n selection (wave 0): forced {0, jcur-1, jcur}, then argmax rounds
    if (wave != 0) return;
    int32_t *out = A.idx + (long)pair * d.n;
    const int ncand = jcur + 1;
    const int nforced = jcur == 0 ? 1 : (jcur == 1 ? 2 : 3);
    const int k = d.n - nforced;
    const int RR = (ncand + 63) / 64;
    uint64_t chosen[2] = {0, 0};
    auto setbit = [&](int rr) { chosen[rr >> 6] |= 1ull << (rr & 63); };
    auto getbit = [&](int rr) { return (chosen[rr >> 6] >> (rr & 63)) & 1ull; };
    if (lane == 0) setbit(0);
    if (jcur >= 1 && (jcur - 1) % 64 == lane) setbit((jcur - 1) / 64);
    if (jcur % 64 == lane) setbit(jcur / 64);
    if (ncand - nforced <= k) {
        for (int rr = 0; rr < RR; rr++)
            if (lane + rr * 64 < ncand) setbit(rr);
    } else {
        for (int round = 0; round < k; round++) {
            float bs = -INFINITY;
            int bj = 0x7fffffff;
            for (int rr = 0; rr < RR; rr++) {
                const int j = lane + rr * 64;
                if (j < ncand && !getbit(rr)) {
                    float sc = S[j];
                    sc = sc == sc ? sc : -INFINITY;
                    if (sc > bs || (sc == bs && j < bj)) {
                        bs = sc;
                        bj = j;
                    }
                }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const float os = __shfl_xor(bs, off, 64);
                const int oj = __shfl_xor(bj, off, 64);
                if (os > bs || (os == bs && oj < bj)) {
                    bs = os;
                    bj = oj;
                }
            }
            if (bj % 64 == lane) setbit(bj / 64);
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
    for (int qq = base + lane; qq < d.n; qq += 64) out[qq] = -1;
}

// ---------------------------------------------------------------------------
// Phase C.  Workgroup (pair, split): wavefront w takes the (4*split + w)-th
// distinct valid block of the pair's list.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_phase_c(DecArgs A)
{
    __shared__ DecLds<DV> sm;
    const Dims &d = A.d;
    const int pair = blockIdx.x / A.ss, split = blockIdx.x % A.ss;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = lane & 15, q = lane >> 4;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int jcur = t / 64;
    const int32_t *ir = (A.idx_in ? A.idx_in : A.idx) + (long)pair * d.n;
    int jb = lane < d.n ? ir[lane] : -1;
    bool ok = jb >= 0 && jb <= jcur;
    for (int u = 0; u < 16; u++) {
        const int other = __shfl(jb, u, 64);
        if (u < lane && other == jb) ok = false;
    }
    const uint64_t valid = __ballot(ok);
    const int want = kSelPerWg * split + wave;
    int j = -1;
    {
        uint64_t v = valid;
        for (int r = 0; r < want && v; r++) v &= v - 1;
        if (v) j = __shfl(jb, __builtin_ctzll(v), 64);
    }
    const uint16_t *K = (const uint16_t *)A.k + (long)pair * d.T * DK;
    const uint16_t *V = (const uint16_t *)A.v + (long)pair * d.T * DV;
    const float sl2 = d.scale * kLog2e;
    bf16x8 qf[DK / 32];
    load_qf<DK>((const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK, q, qf);
    float s[2][8];
    VRegs<DV> vr[2];
    float mx = -INFINITY;
    const int kend = j < 0 ? 0 : min(64 * j + 64, t + 1);
#pragma unroll
    for (int st = 0; st < 2; st++) {
        const int base = 64 * j + 32 * st;
        if (j >= 0 && base < kend) {
            load_v<DV>(V, base, d.T - 1, lane, vr[st]);
            logits_step<DK>(K, base, d.T - 1, qf, hd, q, s[st]);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                s[st][e] = base + 8 * q + e < kend ? s[st][e] * sl2 : -INFINITY;
                mx = fmaxf(mx, s[st][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) s[st][e] = -INFINITY;
        }
    }
    mx = head_max(mx);
    if (q == 0) sm.mx[wave][hd] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm.mx[0][hd], sm.mx[1][hd]), fmaxf(sm.mx[2][hd], sm.mx[3][hd]));
    float l = 0.f;
    f32x4 oacc[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t *vt = sm.u.vt[wave];
#pragma unroll
    for (int st = 0; st < 2; st++) {
        const int base = 64 * j + 32 * st;
        if (j >= 0 && base < kend) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                p[e] = fast_exp2(s[st][e] - M);
                l += p[e];
            }
            store_vt<DV>(vr[st], vt + st * DV * kVtS, lane);
            pv_step<DV>(vt + st * DV * kVtS, p, hd, q, oacc);
        }
    }
    l = head_sum(l);
    const long pidx = (long)pair * A.ss + split;
    wg_store_partial<DV>(sm, wave, lane, M, l, oacc, A.sm + pidx * 16, A.sl + pidx * 16, A.so + pidx * 16 * DV);
}

// ---------------------------------------------------------------------------
// Phase D.  Four workgroups per (sequence, KV head), four heads each: merge
// the compressed, window and selected partials, the gates, and
// o = g_cmp o_cmp + g_slc o_slc + g_win o_win.
constexpr int kDHeads = 4;

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_phase_d(DecArgs A)
{
    __shared__ float wts[3][64][kDHeads];   // [branch][split][head] merge weights
    __shared__ float gate[kDHeads][3];
    const Dims &d = A.d;
    const int pair = blockIdx.x / (16 / kDHeads), h0 = (blockIdx.x % (16 / kDHeads)) * kDHeads;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int tid = threadIdx.x;
    const int nsplit = A.cs + A.ws;
    const float *pmA = A.pm + (long)pair * nsplit * 16, *plA = A.pl + (long)pair * nsplit * 16;
    const float *pmC = A.sm + (long)pair * A.ss * 16, *plC = A.sl + (long)pair * A.ss * 16;
    if (tid < 3 * kDHeads) {
        // branch 0: compressed (splits 0..cs-1), 1: window (cs..cs+ws-1), 2: selected
        const int br = tid / kDHeads, h = h0 + tid % kDHeads;
        const int ns = br == 0 ? A.cs : (br == 1 ? A.ws : A.ss);
        const float *pm = br == 2 ? pmC : pmA + (br == 1 ? A.cs * 16 : 0);
        const float *pl = br == 2 ? plC : plA + (br == 1 ? A.cs * 16 : 0);
        float M = -INFINITY;
        for (int s = 0; s < ns; s++) M = fmaxf(M, pm[s * 16 + h]);
        float L = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < ns; s++) L += pl[s * 16 + h] * fast_exp2(pm[s * 16 + h] - M);
        for (int s = 0; s < ns; s++)
            wts[br][s][tid % kDHeads] = (M == -INFINITY || L <= 0.f) ? 0.f : fast_exp2(pm[s * 16 + h] - M) / L;
    }
    // gates: 16 threads per (head, gate) dot product of length DK
    if (tid < 16 * 3 * kDHeads) {
        const int dot = tid >> 4, part = tid & 15;
        const int h = h0 + dot / 3, c = dot % 3;
        const uint16_t *qr = (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + h) * DK;
        const uint16_t *wr = (const uint16_t *)A.wg + ((long)(g * 16 + h) * 3 + c) * DK;
        float z = 0.f;
        for (int ch = part; ch < DK / 8; ch += 16) {
            const u32x4 wv = ld16(wr + 8 * ch), qv = ld16(qr + 8 * ch);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                z += __uint_as_float(wv[e] << 16) * __uint_as_float(qv[e] << 16);
                z += __uint_as_float(wv[e] & 0xffff0000u) * __uint_as_float(qv[e] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) z += __shfl_xor(z, off, 16);
        if (part == 0) {
            z += __uint_as_float((uint32_t)((const uint16_t *)A.bg)[(g * 16 + h) * 3 + c] << 16);
            gate[dot / 3][c] = sigmoidf_(z);
        }
    }
    __syncthreads();
    const float *poA = A.po + (long)pair * nsplit * 16 * DV, *poC = A.so + (long)pair * A.ss * 16 * DV;
    uint16_t *o = (uint16_t *)A.o + ((long)b * d.Hq + g * 16) * DV;
    for (int e = tid; e < kDHeads * DV; e += kThreads) {
        const int hl = e / DV, h = h0 + hl, c = e % DV;
        const long off = (long)h * DV + c;
        float oc = 0.f, ow = 0.f, os = 0.f;
#pragma unroll 4
        for (int s = 0; s < A.cs; s++) oc += poA[(long)s * 16 * DV + off] * wts[0][s][hl];
#pragma unroll 2
        for (int s = 0; s < A.ws; s++) ow += poA[(long)(A.cs + s) * 16 * DV + off] * wts[1][s][hl];
#pragma unroll 4
        for (int s = 0; s < A.ss; s++) os += poC[(long)s * 16 * DV + off] * wts[2][s][hl];
        const float y = gate[hl][0] * oc + gate[hl][1] * os + gate[hl][2] * ow;
        __bf16 yb = (__bf16)y;
        o[off] = __builtin_bit_cast(uint16_t, yb);
    }
}

template <int DK, int DV>
hipError_t launch_decode_dims(const DecArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int pairs = d.B * d.Hkv;
    hipLaunchKernelGGL((k_dec_phase_a<DK, DV>), dim3(pairs * (A.cs + A.ws)), dim3(kThreads), 0, s, A);
    hipLaunchKernelGGL((k_dec_phase_b<DV>), dim3(pairs), dim3(kThreads), sizeof(float) * d.nb, s, A);
    hipLaunchKernelGGL((k_dec_phase_c<DK, DV>), dim3(pairs * A.ss), dim3(kThreads), 0, s, A);
    hipLaunchKernelGGL((k_dec_phase_d<DK, DV>), dim3(pairs * (16 / kDHeads)), dim3(kThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const Dims &d)
{
    if (d.dtype != NSA_BF16 || d.G != 16) return false;
    if (!((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64))) return false;
    const int cs = (d.npad + kSplitKeys - 1) / kSplitKeys, ws = (d.w + kSplitKeys - 1) / kSplitKeys;
    return cs + ws <= 64 && d.npad / 4 <= 16384;
}

// Workspace of the matrix-core decode step, carved from `ws` when non-null.
size_t decode_mfma_layout(const Dims &d, void *ws, DecArgs *A)
{
    const long pairs = (long)d.B * d.Hkv;
    const int cs = (d.npad + kSplitKeys - 1) / kSplitKeys, wsplit = (d.w + kSplitKeys - 1) / kSplitKeys;
    const int ss = (d.n + kSelPerWg - 1) / kSelPerWg;
    const int nbp = d.npad / 4;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = (off + bytes + 255) / 256 * 256;
        return o;
    };
    const size_t o_pm = take(4 * pairs * (cs + wsplit) * 16), o_pl = take(4 * pairs * (cs + wsplit) * 16);
    const size_t o_po = take(4 * pairs * (cs + wsplit) * 16 * d.dv);
    const size_t o_bx = take(4 * pairs * 16 * nbp), o_by = take(4 * pairs * 16 * nbp);
    const size_t o_sm = take(4 * pairs * ss * 16), o_sl = take(4 * pairs * ss * 16), o_so = take(4 * pairs * ss * 16 * d.dv);
    const size_t o_oc = take(4 * pairs * 16 * d.dv), o_idx = take(4 * pairs * d.n);
    if (A && ws) {
        char *w = (char *)ws;
        A->cs = cs;
        A->ws = wsplit;
        A->ss = ss;
        A->nbp = nbp;
        A->pm = (float *)(w + o_pm);
        A->pl = (float *)(w + o_pl);
        A->po = (float *)(w + o_po);
        A->bx = (float *)(w + o_bx);
        A->by = (float *)(w + o_by);
        A->sm = (float *)(w + o_sm);
        A->sl = (float *)(w + o_sl);
        A->so = (float *)(w + o_so);
        A->ocmp = (float *)(w + o_oc);
        A->idx = (int32_t *)(w + o_idx);
    }
    return off;
}

hipError_t launch_decode_mfma(const DecArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    if (d.dk == 192 && d.dv == 128) return launch_decode_dims<192, 128>(A, s);
    if (d.dk == 128 && d.dv == 128) return launch_decode_dims<128, 128>(A, s);
    if (d.dk == 64 && d.dv == 64) return launch_decode_dims<64, 64>(A, s);
    return hipErrorInvalidValue;
}

}  // namespace nsa
