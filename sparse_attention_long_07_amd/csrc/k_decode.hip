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
// Every wavefront issues all (coalesced) loads of its 64 keys before it
// computes, so each one keeps 40 KB in flight.
//
// Lane view (one position, 16 heads, wave64): head hd = lane%16, key group
// q = lane/16.  A 32-key step is two 16x16x32 S^T tiles whose rows hold keys
// 8*(i/4) + i%4 and 8*(i/4) + 4 + i%4, so lane (q, hd) ends with the logits
// of keys 8q .. 8q+7 of the step for head hd: exactly the B operand of
// O^T = V^T P^T.  K and V reach the operands through a per-wave LDS stage.
#include "mfma_util.h"
#include "nsa_internal.h"
#include "select_util.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaveKeys = 64;                // keys per wavefront (two 32-key steps)
constexpr int kSplitKeys = 4 * kWaveKeys;    // keys per phase-A workgroup
constexpr int kSelPerWg = 4;                 // selected blocks per phase-C workgroup
constexpr int kPersistentWgs = 256;         // split-K workgroups: one per CU (87 KB of LDS each)
constexpr int kMaxItemsPerWg = 256;         // work items one split-K workgroup can take

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

// One 32-key step is fetched with coalesced 16-byte loads (adjacent lanes,
// adjacent bytes) into registers, then written to the wavefront's LDS stage,
// from where the MFMA operand fragments are read:
//  * K row of key k goes to LDS row 16*((k%8)/4) + 4*(k/8) + k%4, so the two
//    16-key S^T tiles (rows 8*(i/4) + i%4 and 8*(i/4) + 4 + i%4) are LDS rows
//    0..15 and 16..31 and the 16 lanes of a fragment read 16 consecutive rows;
//  * V stays key-major; eight 2-byte reads build each V^T fragment, and every
//    group of 8 keys is shifted by 16 bytes so the four key groups of a read
//    fall in different banks.
template <int DK, int DV>
struct StageRegs {
    static constexpr int NK = DK / 16, NV = DV / 16;   // 16-byte chunks per lane per step
    u32x4 k[NK], v[NV];
};

template <int DK, int DV>
struct StageLds {
    static constexpr int KS = DK + 8;                   // bf16 per K row
    static constexpr int VS = DV + 8;                   // bf16 per V row
    uint16_t k[32 * KS];
    uint16_t v[32 * VS + 4 * 8];
    __device__ static int vrow(int key) { return key * VS + (key >> 3) * 8; }
};

__device__ __forceinline__ int kperm(int k) { return 16 * ((k & 7) >> 2) + 4 * (k >> 3) + (k & 3); }

template <int DK, int DV>
__device__ __forceinline__ void stage_load_k(const uint16_t *K, int base, int kclamp, int lane, StageRegs<DK, DV> &r)
{
    constexpr int CK = DK / 8;
#pragma unroll
    for (int i = 0; i < StageRegs<DK, DV>::NK; i++) {
        const int c = 64 * i + lane, key = c / CK, col = c % CK;
        r.k[i] = ld16(K + (long)min(base + key, kclamp) * DK + col * 8);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void stage_load_v(const uint16_t *V, int base, int kclamp, int lane, StageRegs<DK, DV> &r)
{
    constexpr int CV = DV / 8;
#pragma unroll
    for (int i = 0; i < StageRegs<DK, DV>::NV; i++) {
        const int c = 64 * i + lane, key = c / CV, col = c % CV;
        r.v[i] = ld16(V + (long)min(base + key, kclamp) * DV + col * 8);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void stage_store_k(const StageRegs<DK, DV> &r, StageLds<DK, DV> &st, int lane)
{
    constexpr int CK = DK / 8;
#pragma unroll
    for (int i = 0; i < StageRegs<DK, DV>::NK; i++) {
        const int c = 64 * i + lane, key = c / CK, col = c % CK;
        st16(&st.k[kperm(key) * StageLds<DK, DV>::KS + col * 8], r.k[i]);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void stage_store_v(const StageRegs<DK, DV> &r, StageLds<DK, DV> &st, int lane)
{
    constexpr int CV = DV / 8;
#pragma unroll
    for (int i = 0; i < StageRegs<DK, DV>::NV; i++) {
        const int c = 64 * i + lane, key = c / CV, col = c % CV;
        st16(&st.v[StageLds<DK, DV>::vrow(key) + col * 8], r.v[i]);
    }
}

// Raw logits of keys 8q .. 8q+7 of the staged step for head hd.
template <int DK, int DV>
__device__ __forceinline__ void logits_lds(const StageLds<DK, DV> &st, const bf16x8 (&qf)[DK / 32], int hd, int q,
                                           float (&s)[8])
{
    constexpr int KS = StageLds<DK, DV>::KS;
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; kk++) {
        accA = mfma16(as_bf16x8(ld16(&st.k[hd * KS + 32 * kk + 8 * q])), qf[kk], accA);
        accB = mfma16(as_bf16x8(ld16(&st.k[(16 + hd) * KS + 32 * kk + 8 * q])), qf[kk], accB);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
        s[u] = accA[u];
        s[4 + u] = accB[u];
    }
}

// O^T += V^T P^T for the staged step (P^T = this lane's keys 8q .. 8q+7).
template <int DK, int DV>
__device__ __forceinline__ void pv_lds(const StageLds<DK, DV> &st, const float (&p)[8], int hd, int q,
                                       f32x4 (&oacc)[DV / 16])
{
    const bf16x8 pb = pack8(p);
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++) {
        u32x4 a;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t lo = st.v[StageLds<DK, DV>::vrow(8 * q + 2 * e) + 16 * dt + hd];
            const uint32_t hi = st.v[StageLds<DK, DV>::vrow(8 * q + 2 * e + 1) + 16 * dt + hd];
            a[e] = lo | (hi << 16);
        }
        oacc[dt] = mfma16(as_bf16x8(a), pb, oacc[dt]);
    }
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

template <int DK, int DV>
struct DecLds {
    union {
        StageLds<DK, DV> st[4];     // one stage per wavefront
        float ol[4][16][DV + 4];    // merge buffer; padded rows spread the 16 heads over banks
    } u;
    float mx[4][16];
    float ls[4][16];
};

// Workgroup-level merge of four wavefronts that used the same max M:
// sums l and O in wave order and writes (M, l, O) for the 16 heads.
template <int DK, int DV>
__device__ __forceinline__ void wg_store_partial(DecLds<DK, DV> &sm, int wave, int lane, float M, float l,
                                                 const f32x4 (&oacc)[DV / 16], float *pm, float *pl, float *po)
{
    const int hd = lane & 15, q = lane >> 4;
    lds_barrier();   // the stages alias the merge buffer
#pragma unroll
    for (int dt = 0; dt < DV / 16; dt++)
#pragma unroll
        for (int u = 0; u < 4; u++) sm.u.ol[wave][hd][16 * dt + 4 * q + u] = oacc[dt][u];
    if (q == 0) sm.ls[wave][hd] = l;
    lds_barrier();
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
// Phases A and C: persistent split-K workgroups.  Work item = (pair, slot);
// workgroup w takes items w, w + gridDim.x, ...  Phase-A slots 0..cs-1 cover
// compressed slots [256 s, 256 s + 256), slots cs.. cover window keys from
// max(0, t-w+1); phase-C slot s covers the selected blocks 4s .. 4s+3 of the
// pair's (deduplicated) list, one block per wavefront.  As soon as one item's
// K (then V) registers are in the LDS stage, the next item's loads are issued
// into them, so the memory system stays busy while the item computes.
constexpr int kPhaseA = 0, kPhaseC = 1;

struct WaveItem {
    int pair, slot, t;
    int kbeg, kend, kclamp;
    bool cmp;
    const uint16_t *K, *V;
};

// t and (phase C) the block list of the workgroup's k-th item come from LDS,
// filled once at kernel start, so no item waits on a dependent global load.
template <int DK, int DV, int KIND>
__device__ __forceinline__ WaveItem wave_item(const DecArgs &A, int item, int k, const int *it_t, const int *it_idx,
                                              int wave, int lane)
{
    const Dims &d = A.d;
    WaveItem r;
    if (KIND == kPhaseA) {
        const int nsplit = A.cs + A.ws;
        r.pair = item / nsplit;
        r.slot = item % nsplit;
        r.t = it_t[k];
        r.cmp = r.slot < A.cs;
        if (r.cmp) {
            const int nvis = r.t >= 31 ? (r.t - 31) / 16 + 1 : 0;
            r.kbeg = r.slot * kSplitKeys + wave * kWaveKeys;
            r.kend = min(r.kbeg + kWaveKeys, nvis);
            r.kclamp = d.npad - 1;
            r.K = (const uint16_t *)A.kc + (long)r.pair * d.npad * DK;
            r.V = (const uint16_t *)A.vc + (long)r.pair * d.npad * DV;
        } else {
            const int lo = max(0, r.t - d.w + 1);
            r.kbeg = lo + (r.slot - A.cs) * kSplitKeys + wave * kWaveKeys;
            r.kend = min(r.kbeg + kWaveKeys, r.t + 1);
            r.kclamp = d.T - 1;
            r.K = (const uint16_t *)A.k + (long)r.pair * d.T * DK;
            r.V = (const uint16_t *)A.v + (long)r.pair * d.T * DV;
        }
    } else {
        r.pair = item / A.ss;
        r.slot = item % A.ss;
        r.t = it_t[k];
        r.cmp = false;
        const int jcur = r.t / 64;
        const int jb = lane < d.n ? it_idx[k * 16 + lane] : -1;
        bool ok = jb >= 0 && jb <= jcur;
        for (int u = 0; u < 16; u++) {
            const int other = __shfl(jb, u, 64);
            if (u < lane && other == jb) ok = false;
        }
        uint64_t v = __ballot(ok);
        for (int c = 0; c < kSelPerWg * r.slot + wave && v; c++) v &= v - 1;
        const int j = v ? __shfl(jb, __builtin_ctzll(v), 64) : -1;
        r.kbeg = j < 0 ? 0 : 64 * j;
        r.kend = j < 0 ? 0 : min(64 * j + 64, r.t + 1);
        r.kclamp = d.T - 1;
        r.K = (const uint16_t *)A.k + (long)r.pair * d.T * DK;
        r.V = (const uint16_t *)A.v + (long)r.pair * d.T * DV;
    }
    return r;
}

template <int DK, int DV, int KIND>
__global__ __launch_bounds__(kThreads) void k_dec_splitk(DecArgs A, int total)
{
    __shared__ DecLds<DK, DV> sm;
    const Dims &d = A.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = lane & 15, q = lane >> 4;
    const float sl2 = d.scale * kLog2e;
    const int nslots = KIND == kPhaseA ? A.cs + A.ws : A.ss;
    int item = blockIdx.x;
    if (item >= total) return;
    // per-item t (and block lists) of this workgroup's items, loaded at once
    __shared__ int it_t[kMaxItemsPerWg];
    __shared__ int it_idx[KIND == kPhaseC ? kMaxItemsPerWg * 16 : 1];
    const int nitems = (total - 1 - blockIdx.x) / gridDim.x + 1;
    for (int k = tid; k < nitems; k += kThreads) {
        const int pair = (blockIdx.x + k * gridDim.x) / nslots;
        it_t[k] = dec_t(A.seq_lens, pair / d.Hkv, d.T);
    }
    if (KIND == kPhaseC) {
        const int32_t *isrc = A.idx_in ? A.idx_in : A.idx;
        for (int e = tid; e < nitems * 16; e += kThreads) {
            const int pair = (blockIdx.x + (e >> 4) * gridDim.x) / nslots;
            it_idx[e] = (e & 15) < d.n ? isrc[(long)pair * d.n + (e & 15)] : -1;
        }
    }
    lds_barrier();
    int k_it = 0;
    WaveItem r = wave_item<DK, DV, KIND>(A, item, k_it, it_t, it_idx, wave, lane);
    StageRegs<DK, DV> rg[2];
    bf16x8 qf[DK / 32];
    auto qrow = [&](const WaveItem &x) {
        return (const uint16_t *)A.q + ((long)(x.pair / d.Hkv) * d.Hq + (x.pair % d.Hkv) * 16 + hd) * DK;
    };
#pragma unroll
    for (int st = 0; st < 2; st++)
        if (r.kbeg + 32 * st < r.kend) {
            stage_load_k<DK, DV>(r.K, r.kbeg + 32 * st, r.kclamp, lane, rg[st]);
            stage_load_v<DK, DV>(r.V, r.kbeg + 32 * st, r.kclamp, lane, rg[st]);
        }
    load_qf<DK>(qrow(r), q, qf);
    StageLds<DK, DV> &stg = sm.u.st[wave];
    while (true) {
        const int nxt = item + gridDim.x;
        const bool more = nxt < total;
        WaveItem rn = r;
        if (more) rn = wave_item<DK, DV, KIND>(A, nxt, k_it + 1, it_t, it_idx, wave, lane);
        lds_barrier();   // the previous item's merge is done with the stage memory
        float s[2][8];
        float mx = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; st++) {
            const int base = r.kbeg + 32 * st;
            if (base < r.kend) {   // uniform over the wavefront
                stage_store_k<DK, DV>(rg[st], stg, lane);
                logits_lds<DK, DV>(stg, qf, hd, q, s[st]);
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    s[st][e] = base + 8 * q + e < r.kend ? s[st][e] * sl2 : -INFINITY;
                    mx = fmaxf(mx, s[st][e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) s[st][e] = -INFINITY;
            }
        }
        if (more) {   // K registers and q fragments are free: prefetch the next item's
#pragma unroll
            for (int st = 0; st < 2; st++)
                if (rn.kbeg + 32 * st < rn.kend) stage_load_k<DK, DV>(rn.K, rn.kbeg + 32 * st, rn.kclamp, lane, rg[st]);
            load_qf<DK>(qrow(rn), q, qf);
        }
        mx = head_max(mx);
        if (q == 0) sm.mx[wave][hd] = mx;
        lds_barrier();
        const float M = fmaxf(fmaxf(sm.mx[0][hd], sm.mx[1][hd]), fmaxf(sm.mx[2][hd], sm.mx[3][hd]));
        float l = 0.f;
        f32x4 oacc[DV / 16];
#pragma unroll
        for (int dt = 0; dt < DV / 16; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float *bx = A.bx + (long)r.pair * 16 * A.nbp + (long)hd * A.nbp;
        float *by = A.by + (long)r.pair * 16 * A.nbp + (long)hd * A.nbp;
#pragma unroll
        for (int st = 0; st < 2; st++) {
            const int base = r.kbeg + 32 * st;
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; e++) p[e] = M == -INFINITY ? 0.f : fast_exp2(s[st][e] - M);
            if (KIND == kPhaseA && r.cmp) {
                // block a = (base + 8q)/4 gets keys 4a..4a+3 here (weights 2,2,2,1);
                // its remaining weight-1 key 4a-1 is the previous block's Y term
                const int a = (base + 8 * q) >> 2;
                if (a + 1 < A.nbp) {
                    *(float2 *)&bx[a] =
                        make_float2(2.f * (p[0] + p[1] + p[2]) + p[3], 2.f * (p[4] + p[5] + p[6]) + p[7]);
                    *(float2 *)&by[a] = make_float2(p[3], p[7]);
                }
            }
            if (base < r.kend) {   // uniform over the wavefront
#pragma unroll
                for (int e = 0; e < 8; e++) l += p[e];
                stage_store_v<DK, DV>(rg[st], stg, lane);
                pv_lds<DK, DV>(stg, p, hd, q, oacc);
            }
        }
        if (more) {
#pragma unroll
            for (int st = 0; st < 2; st++)
                if (rn.kbeg + 32 * st < rn.kend) stage_load_v<DK, DV>(rn.V, rn.kbeg + 32 * st, rn.kclamp, lane, rg[st]);
        }
        l = head_sum(l);
        const long pidx = (long)r.pair * nslots + r.slot;
        if (KIND == kPhaseA)
            wg_store_partial<DK, DV>(sm, wave, lane, M, l, oacc, A.pm + pidx * 16, A.pl + pidx * 16,
                                     A.po + pidx * 16 * DV);
        else
            wg_store_partial<DK, DV>(sm, wave, lane, M, l, oacc, A.sm + pidx * 16, A.sl + pidx * 16,
                                     A.so + pidx * 16 * DV);
        if (!more) break;
        item = nxt;
        k_it++;
        r = rn;
    }
}

// ---------------------------------------------------------------------------
// Phase B.  One workgroup per (sequence, KV head): the exact log-sum-exp of
// each head over the compressed splits, the block scores and the selection.
template <int DV>
__global__ __launch_bounds__(kThreads) void k_dec_phase_b(DecArgs A)
{
    extern __shared__ float S[];   // [nb] block scores
    __shared__ uint2 cand[64];      // selector scratch
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
    __shared__ float lm[64][16], ll[64][16];
    for (int e = tid; e < A.cs * 16; e += kThreads) {   // all loads in flight at once
        lm[e >> 4][e & 15] = pm[e];
        ll[e >> 4][e & 15] = pl[e];
    }
    lds_barrier();
    if (tid < 16) {
        float M = -INFINITY;
        for (int s = 0; s < A.cs; s++) M = fmaxf(M, lm[s][tid]);
        float L = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < A.cs; s++) L += ll[s][tid] * fast_exp2(lm[s][tid] - M);
        lse[tid] = M == -INFINITY ? -INFINITY : M + fast_log2(L);
    }
    lds_barrier();
    for (int e = tid; e < A.cs * 16; e += kThreads) {
        const int s = e >> 4, h = e & 15;
        wsp[s][h] = lse[h] == -INFINITY ? 0.f : fast_exp2(lm[s][h] - lse[h]);
    }
    lds_barrier();
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
    lds_barrier();
    if (A.idx_in || wave != 0) return;
    wave_select_topn_fast(S, jcur, d.n, A.idx + (long)pair * d.n, lane, cand);
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
    // (max, sum) of every split of the three branches into LDS, loads in parallel:
    // branch 0 compressed (phase-A splits 0..cs-1), 1 window (cs..), 2 selected
    __shared__ float lm[3][64][kDHeads], ll[3][64][kDHeads];
    for (int e = tid; e < 3 * 64 * kDHeads; e += kThreads) {
        const int br = e / (64 * kDHeads), s = (e / kDHeads) % 64, hl = e % kDHeads;
        const int ns = br == 0 ? A.cs : (br == 1 ? A.ws : A.ss);
        if (s < ns) {
            const long src = (long)(br == 1 ? A.cs + s : s) * 16 + h0 + hl;
            lm[br][s][hl] = br == 2 ? pmC[src] : pmA[src];
            ll[br][s][hl] = br == 2 ? plC[src] : plA[src];
        }
    }
    lds_barrier();
    if (tid < 3 * kDHeads) {
        const int br = tid / kDHeads, hl = tid % kDHeads;
        const int ns = br == 0 ? A.cs : (br == 1 ? A.ws : A.ss);
        float M = -INFINITY;
        for (int s = 0; s < ns; s++) M = fmaxf(M, lm[br][s][hl]);
        float L = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < ns; s++) L += ll[br][s][hl] * fast_exp2(lm[br][s][hl] - M);
        for (int s = 0; s < ns; s++)
            wts[br][s][hl] = (M == -INFINITY || L <= 0.f) ? 0.f : fast_exp2(lm[br][s][hl] - M) / L;
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
    lds_barrier();
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
    const int na = pairs * (A.cs + A.ws), nc = pairs * A.ss;
    hipLaunchKernelGGL((k_dec_splitk<DK, DV, kPhaseA>), dim3(min(na, kPersistentWgs)), dim3(kThreads), 0, s, A, na);
    hipLaunchKernelGGL((k_dec_phase_b<DV>), dim3(pairs), dim3(kThreads), sizeof(float) * d.nb, s, A);
    hipLaunchKernelGGL((k_dec_splitk<DK, DV, kPhaseC>), dim3(min(nc, kPersistentWgs)), dim3(kThreads), 0, s, A, nc);
    hipLaunchKernelGGL((k_dec_phase_d<DK, DV>), dim3(pairs * (16 / kDHeads)), dim3(kThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const Dims &d)
{
    if (d.dtype != NSA_BF16 || d.G != 16) return false;
    if (!((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64))) return false;
    const int cs = (d.npad + kSplitKeys - 1) / kSplitKeys, ws = (d.w + kSplitKeys - 1) / kSplitKeys;
    const long pairs = (long)d.B * d.Hkv;
    const int ss = (d.n + kSelPerWg - 1) / kSelPerWg;
    return cs + ws <= 64 && d.npad / 4 <= 16384 && pairs * (cs + ws) <= (long)kPersistentWgs * kMaxItemsPerWg &&
           pairs * ss <= (long)kPersistentWgs * kMaxItemsPerWg;
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
