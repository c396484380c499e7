// NSA decode step on the matrix cores (bf16 storage, 16 query heads per KV
// head).  valuable12.com, "AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션
// 기술 화제", section III.3: a 64k-context decode step reads the keys and
// values of 5,632 tokens instead of 65,536 -- the compressed cache, the
// selected blocks and the window.  The step is bound by HBM bandwidth.  Its
// one dependency is the selection, which needs the compressed branch's
// exact probabilities, so it runs as four launches:
//   k_dec_stream  the compressed cache: nq workgroups per (sequence, KV head)
//                 pair, up to 1,024 slots each (two workgroups per CU, one
//                 round at 32 x 64k caches).  Each of the 4 wavefronts streams
//                 32-slot steps with the next step's loads in flight and its
//                 own running maximum, and leaves its blocks' importance
//                 terms relative to that maximum (staged in LDS, written once).
//   k_dec_select  one workgroup per pair: the compressed branch's exact
//                 log-sum-exp, the block scores and the top-n selection (one
//                 round of loads, a sort-based selection), and the gates;
//                 beside them, work that needs no selection and streams
//                 meanwhile: the window in workgroups of 256 keys and the
//                 always-kept blocks 0, j-1 and j (one workgroup per pair).
//   k_dec_gather  the other selected blocks, one 64-token block per
//                 wavefront, all of a block's loads issued at once.
//   k_dec_merge   per pair: the branches' partials merged, gated, o.
// Every partial is (max, sum, unnormalised output) per head in fp32.  Slots
// of a pair: nq compressed ranges, nw window ranges, the always-kept blocks,
// then ns gather groups (the selected branch is the last 1 + ns).
//
// Lane view (one query position, 16 heads, wave64): head hd = lane%16, key
// group q = lane/16.  A 32-key step is two 16x16x32 S^T tiles whose rows hold
// keys 8*(i/4) + i%4 and 8*(i/4) + 4 + i%4, so lane (q, hd) ends with the
// logits of keys 8q .. 8q+7 of the step for head hd: exactly the B operand of
// O^T = V^T P^T.  K is loaded straight into the A-operand registers of the
// S^T tiles; V goes through a per-wavefront LDS region and comes back as V^T
// operand fragments by transpose reads.
//
// Block importance (deepdaiv newsletter, token selection paragraph: the block
// scores come from the compressed branch's attention): selection block j
// takes compressed slots 4j-1 .. 4j+3 with weights 1,2,2,2,1 (the tokens each
// shares with the block, in units of the stride).  A step's lane holds slots
// 8q .. 8q+7 = the own slots of blocks a = (kbeg+8q)/4 and a+1; the weight-1
// slot 4a-1 of block a is the previous lane group's last slot, except for the
// first block of the step, whose slot 4a-1 is the previous step's last slot
// (kept per 32-slot group as `gtail`).
#include <algorithm>

#include "mfma_util.h"
#include "nsa_internal.h"
#include "select_util.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;               // 4 wavefronts in every decode kernel
constexpr int kWaves = kThreads / 64;
constexpr int kStepKeys = 32;               // keys per wavefront step
constexpr int kCmpRound = kWaves * kStepKeys * 2;        // k_dec_cmp ranges are multiples of 256 slots
constexpr int kWinKeys = kWaves * kStepKeys * 2;          // 256 window keys per workgroup
constexpr int kBlocksPerGather = kWaves;                  // selected blocks per k_dec_gather workgroup
constexpr int kMaxCmpKeys = 1024;                         // slots per k_dec_cmp workgroup at most
constexpr int kMaxCmpSlots = 128;                         // k_dec_cmp workgroups per pair at most
constexpr int kMaxSlots = 192;                            // partial slots per pair at most
constexpr int kMaxGroups = 512;                           // 32-slot groups of the compressed cache at most

__device__ __forceinline__ float sigmoidf_(float z) { return 1.f / (1.f + __expf(-z)); }

__device__ __forceinline__ int dec_t(const int32_t *seq_lens, int b, int T)
{
    int L = seq_lens[b];
    L = L < 1 ? 1 : (L > T ? T : L);
    return L - 1;
}

__device__ __forceinline__ int n_visible(int t) { return t >= 31 ? (t - 31) / 16 + 1 : 0; }

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

// Per-wavefront LDS region: the step's V rows (key-major, DV bf16 = U units
// of 32 bytes each), unit u of row r stored at unit u ^ sigma(r) with
// sigma(r) = (r%4) | 4*((r/8)%2) (mod U).  The transpose reads of a V^T
// fragment touch one unit of rows {8g + 0..3} (then + 4) for the four lane
// groups g, and sigma spreads the rows of each half-wave over distinct units;
// the 16-byte row stores fill whole rows.  At the end the same bytes hold the
// wavefront's output for the workgroup merge.
template <int DV>
struct WaveLds {
    static constexpr int U = DV / 16;
    static constexpr int VBYTES = kStepKeys * 2 * DV;
    static constexpr int OBYTES = 16 * (DV + 4) * 4;   // [16][DV+4] fp32
    static constexpr int BYTES = VBYTES > OBYTES ? VBYTES : OBYTES;
    __device__ static int vaddr(int r, int unit, int byte)
    {
        const int sig = ((r & 3) | ((r >> 1) & 4)) & (U - 1);
        return r * 2 * DV + ((unit ^ sig) << 5) + byte;
    }
};

template <int DV>
struct StreamLds {
    unsigned char wave[kWaves][WaveLds<DV>::BYTES];
    float wm[kWaves][16], wl[kWaves][16];
};

// One wavefront's 32-key step: K rows straight into the S^T operand
// registers (tile A row i holds key 8(i/4) + i%4, tile B key 8(i/4) + 4 + i%4),
// V rows into registers bound for the LDS region.
template <int DK, int DV>
struct Step {
    static constexpr int KS = DK / 32, VC = DV / 8, VL = kStepKeys * VC / 64;
    u32x4 ka[KS], kb[KS], vr[VL];
};

// Keys kbeg .. kbeg+31 of K/V (rows of DK/DV bf16).  K rows past kmax read
// row kmax; V rows of keys at or past kend read row kend-1, a row the caller
// has written (a key past kend enters with probability 0, and 0 * NaN would
// reach the output).  kend > kbeg is not required: an inactive step loads
// valid rows and is not computed.
template <int DK, int DV>
__device__ __forceinline__ void load_step(Step<DK, DV> &st, const uint16_t *K, const uint16_t *V, int kbeg, int kend,
                                          int kmax, int lane)
{
    using S = Step<DK, DV>;
    const int hd = lane & 15, q = lane >> 4;
    const int kA = kbeg + 8 * (hd >> 2) + (hd & 3);
    const uint16_t *ra = K + (long)max(0, min(kA, kmax)) * DK + 8 * q;
    const uint16_t *rb = K + (long)max(0, min(kA + 4, kmax)) * DK + 8 * q;
#pragma unroll
    for (int kk = 0; kk < S::KS; kk++) {
        st.ka[kk] = ld16(ra + 32 * kk);
        st.kb[kk] = ld16(rb + 32 * kk);
    }
    const int vlast = max(0, kend - 1);
#pragma unroll
    for (int u = 0; u < S::VL; u++) {
        const int c = 64 * u + lane, key = c / S::VC, ch = c % S::VC;
        st.vr[u] = ld16(V + (long)min(kbeg + key, vlast) * DV + ch * 8);
    }
}

// Online-softmax state of one wavefront: running max m (log2 units, the same
// on the 4 lanes of a head), this lane's share of the sum, and O^T.
template <int DV>
struct Acc {
    static constexpr int DT = DV / 16;
    float m, l;
    f32x4 o[DT];
    __device__ void init()
    {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
};

// First half of a step: the logits of keys kbeg .. kbeg+31 (those at or past
// kend are -inf) and the V rows written to the wavefront's LDS region.  It
// consumes the step's registers, so the next step's loads may follow it.
template <int DK, int DV>
__device__ __forceinline__ void step_logits(const Step<DK, DV> &st, const bf16x8 (&qf)[DK / 32], int kbeg, int kend,
                                            float sl2, unsigned char *reg, int lane, float (&s)[8])
{
    using S = Step<DK, DV>;
    using WL = WaveLds<DV>;
    const int q = lane >> 4;
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < S::KS; kk++) {
        accA = mfma16(as_bf16x8(st.ka[kk]), qf[kk], accA);
        accB = mfma16(as_bf16x8(st.kb[kk]), qf[kk], accB);
    }
#pragma unroll
    for (int u = 0; u < S::VL; u++) {
        const int c = 64 * u + lane, key = c / S::VC, ch = c % S::VC;
        st16(reg + WL::vaddr(key, ch >> 1, 16 * (ch & 1)), st.vr[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
        s[u] = kbeg + 8 * q + u < kend ? accA[u] * sl2 : -INFINITY;
        s[4 + u] = kbeg + 8 * q + 4 + u < kend ? accB[u] * sl2 : -INFINITY;
    }
}

// Second half: the running max raised, probabilities p (returned, relative to
// the new max), O^T += V^T P^T from the LDS region.  Requires the step's first
// key to be visible (so the max is finite).
template <int DV>
__device__ __forceinline__ void step_update(const float (&s)[8], Acc<DV> &acc, unsigned char *reg, int lane,
                                            float (&p)[8])
{
    using WL = WaveLds<DV>;
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; e++) mx = fmaxf(mx, s[e]);
    mx = head_max(mx);
    const float mn = fmaxf(acc.m, mx);
    const float al = fast_exp2(acc.m - mn);   // 0 on the first step (m = -inf)
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        p[e] = fast_exp2(s[e] - mn);
        sum += p[e];
    }
    acc.l = __builtin_fmaf(acc.l, al, sum);
    acc.m = mn;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's V stores are in LDS
    __builtin_amdgcn_wave_barrier();
    const bf16x8 pb = pack8(p);
    // lane (g, s) of a 16-lane group points at columns 16dt + 4(s%4) of rows
    // 8g + s/4 (then + 4): lane i then holds dv 16dt + i for keys 8g .. 8g+7,
    // the A operand of O^T = V^T P^T
    const int g = lane >> 4, sl = lane & 15;
    const int r0 = 8 * g + (sl >> 2);
#pragma unroll
    for (int dt = 0; dt < Acc<DV>::DT; dt++) {
        const uint2 lo = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0, dt, 8 * (sl & 3))));
        const uint2 hi = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0 + 4, dt, 8 * (sl & 3))));
        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
        acc.o[dt] *= al;
        acc.o[dt] = mfma16(as_bf16x8(w), pb, acc.o[dt]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the transpose reads are done before the region is rewritten
    __builtin_amdgcn_wave_barrier();
}

// A whole step (both halves).
template <int DK, int DV>
__device__ __forceinline__ void compute_step(const Step<DK, DV> &st, const bf16x8 (&qf)[DK / 32], int kbeg, int kend,
                                             float sl2, Acc<DV> &acc, unsigned char *reg, int lane, float (&p)[8])
{
    float s[8];
    step_logits(st, qf, kbeg, kend, sl2, reg, lane, s);
    step_update(s, acc, reg, lane, p);
}

__device__ __forceinline__ void load_q(const uint16_t *qrow, int lane, bf16x8 *qf, int ks)
{
    const int q = lane >> 4;
    for (int kk = 0; kk < ks; kk++) qf[kk] = as_bf16x8(ld16(qrow + 32 * kk + 8 * q));
}

// The workgroup's 4 wavefront states merged into partial slot `dst`
// ([16 max][16 sum][16][DV], unnormalised output relative to the max).
template <int DV>
__device__ __forceinline__ void merge_waves(const Acc<DV> &acc, StreamLds<DV> &sm, float *dst, int tid)
{
    const int lane = tid & 63, wave = tid >> 6, hd = lane & 15, q = lane >> 4;
    float *ol = (float *)sm.wave[wave];   // [16][DV+4]; the region's last transpose reads are done
#pragma unroll
    for (int dt = 0; dt < Acc<DV>::DT; dt++)
#pragma unroll
        for (int u = 0; u < 4; u++) ol[hd * (DV + 4) + 16 * dt + 4 * q + u] = acc.o[dt][u];
    const float lsum = head_sum(acc.l);
    if (q == 0) {
        sm.wm[wave][hd] = acc.m;
        sm.wl[wave][hd] = lsum;
    }
    lds_barrier();
    for (int e = tid; e < 16 * DV; e += kThreads) {
        const int h = e / DV, c = e % DV;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, sm.wm[w][h]);
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = sm.wm[w][h];
            if (mw != -INFINITY) o = __builtin_fmaf(((const float *)sm.wave[w])[h * (DV + 4) + c], fast_exp2(mw - M), o);
        }
        dst[32 + e] = o;
    }
    if (tid < 16) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, sm.wm[w][tid]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float mw = sm.wm[w][tid];
            if (mw != -INFINITY) L = __builtin_fmaf(sm.wl[w][tid], fast_exp2(mw - M), L);
        }
        dst[tid] = M;
        dst[16 + tid] = L;
    }
}

template <int DV>
__device__ __forceinline__ long part_stride() { return 32 + 16 * DV; }

// ---------------------------------------------------------------------------
// k_dec_stream.  Compressed range: workgroup (pair, r) takes slots [C r, C r + C) with
// C = A.cmp_keys (a multiple of 256, at most 1,024); wavefront w takes the
// 32-slot steps at C r + 128 i + 32 w.  The block terms and group values of
// the range are kept in LDS and written out once, at the end.
template <int DV>
struct StreamKLds {
    struct {
        StreamLds<DV> st;
        float bt[kMaxCmpKeys / 4][16];
        float gmax[kMaxCmpKeys / kStepKeys][16], gtail[kMaxCmpKeys / kStepKeys][16];
    } c;
};

// Blocks {0, jcur-1, jcur} (fewer when jcur < 2), the selection's always-kept
// part; the k-th of them or -1.
__device__ __forceinline__ int forced_block(int k, int jcur)
{
    const int nf = jcur == 0 ? 1 : (jcur == 1 ? 2 : 3);
    return k >= nf ? -1 : (k == 0 ? 0 : (k == 1 ? (nf == 2 ? 1 : jcur - 1) : jcur));
}

// One wavefront attends to 64-token block j (two 32-key steps, loaded at
// once), tokens up to t.
template <int DK, int DV>
__device__ __forceinline__ void attend_block(const uint16_t *K, const uint16_t *V, const uint16_t *qrow, int j, int t,
                                             int T, float sl2, Acc<DV> &acc, unsigned char *reg, int lane)
{
    constexpr int KS = DK / 32;
    const int kend = t + 1, k0 = 64 * j, k1 = k0 + kStepKeys;
    Step<DK, DV> sa, sb;
    load_step(sa, K, V, k0, kend, T - 1, lane);
    load_step(sb, K, V, k1, kend, T - 1, lane);
    bf16x8 qf[KS];
    load_q(qrow, lane, qf, KS);
    float p[8];
    compute_step(sa, qf, k0, kend, sl2, acc, reg, lane, p);   // k0 <= t: the block is causal
    if (k1 < kend) compute_step(sb, qf, k1, kend, sl2, acc, reg, lane, p);
}

template <int DK, int DV>
__device__ __forceinline__ void stream_cmp(const DecArgs &A, StreamKLds<DV> &sm, int pair, int r)
{
    constexpr int KS = DK / 32;
    const Dims &d = A.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hd = lane & 15, q = lane >> 4;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int nvis = n_visible(t);
    const float sl2 = d.scale * kLog2e;
    const uint16_t *K = (const uint16_t *)A.kc + (long)pair * d.npad * DK;
    const uint16_t *V = (const uint16_t *)A.vc + (long)pair * d.npad * DV;
    const int kbase = r * A.cmp_keys;
    const int key0 = kbase + wave * kStepKeys;
    const int kstop = min(nvis, kbase + A.cmp_keys);   // this workgroup's visible slots end here
    constexpr int kStride = kWaves * kStepKeys;

    Acc<DV> acc;
    acc.init();
    unsigned char *reg = sm.c.st.wave[wave];
    Step<DK, DV> st;
    load_step(st, K, V, key0, nvis, d.npad - 1, lane);
    bf16x8 qf[KS];
    load_q((const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK, lane, qf, KS);

    // the step's block terms (see the file comment) and the group's maximum
    auto terms = [&](int kbeg, const float (&p)[8]) {
        const int a = (kbeg - kbase + 8 * q) >> 2, grp = (kbeg - kbase) / kStepKeys;
        const float prev = __shfl(p[7], (lane - 16) & 63, 64);   // slot 4a-1 of lane group q-1
        sm.c.bt[a][hd] = __builtin_fmaf(2.f, p[0] + p[1] + p[2], p[3]) + (q ? prev : 0.f);
        sm.c.bt[a + 1][hd] = __builtin_fmaf(2.f, p[4] + p[5] + p[6], p[7]) + p[3];
        if (q == 0) sm.c.gmax[grp][hd] = acc.m;
        if (q == 3) sm.c.gtail[grp][hd] = p[7];
    };
    // one register set: once a step's K has gone into its products and its V
    // into LDS, the next step's loads go out, under the rest of the step
    for (int k0 = key0; k0 < kstop; k0 += kStride) {
        float s[8], p[8];
        step_logits(st, qf, k0, nvis, sl2, reg, lane, s);
        if (k0 + kStride < kstop) load_step(st, K, V, k0 + kStride, nvis, d.npad - 1, lane);
        __builtin_amdgcn_sched_barrier(0);
        step_update(s, acc, reg, lane, p);
        terms(k0, p);
    }
    merge_waves(acc, sm.c.st, A.part + ((long)pair * A.nslot + r) * part_stride<DV>(), tid);
    // the visible groups' terms, 16-byte stores (the barrier in merge_waves
    // has ordered the LDS writes above)
    const int ngv = (max(0, kstop - kbase) + kStepKeys - 1) / kStepKeys;   // groups with a visible slot
    float *bt = A.bt + ((long)pair * A.nbp + kbase / 4) * 16;
    float *gmax = A.gmax + ((long)pair * A.ngrp + kbase / kStepKeys) * 16;
    float *gtail = A.gtail + ((long)pair * A.ngrp + kbase / kStepKeys) * 16;
    for (int i = tid; i < ngv * 8 * 4; i += kThreads)   // 8 blocks x 4 chunks of 4 heads per group
        st16(bt + 4 * i, ld16(&sm.c.bt[i >> 2][4 * (i & 3)]));
    for (int i = tid; i < ngv * 4; i += kThreads) {
        st16(gmax + 4 * i, ld16(&sm.c.gmax[i >> 2][4 * (i & 3)]));
        st16(gtail + 4 * i, ld16(&sm.c.gtail[i >> 2][4 * (i & 3)]));
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_stream(DecArgs A)
{
    __shared__ StreamKLds<DV> sm;
    stream_cmp<DK, DV>(A, sm, blockIdx.x / A.nq, blockIdx.x % A.nq);
}

// ---------------------------------------------------------------------------
// k_dec_select: workgroups [0, P) select (P pairs), [P, P + P nw) take the
// window, [P + P nw, 2P + P nw) the always-kept blocks.
//
// Selection: every load the block scores need goes out in one round: the
// compressed partials' (max, sum), each visible group's maximum and last-slot
// probability, and the blocks' terms (in batches of 16 per thread for very
// long caches).  The exact log-sum-exp lse_h follows; then group weights
// W[g][h] = 2^(gmax - lse_h), and
//   S[j] = sum_h W[g(4j)][h] bt[j][h] + (j % 8 == 0 ? sum_h W[g-1][h] gtail[g-1][h] : 0).
// Its LDS is sized per launch (dynamic shared memory): lse, W of the groups,
// the groups' weighted tails, then the compressed partials' (max, sum) or,
// once they are reduced, the block scores, then the selection scratch.
constexpr int kSelItems = 16;   // block-term chunks per thread per batch

struct SelLayout {
    int w, ysum, u, cand, bytes;   // byte offsets
};

__host__ __device__ inline SelLayout sel_layout(int ngrp, int nq, int nb, int stream_bytes)
{
    SelLayout L;
    L.w = 64;
    L.ysum = L.w + ngrp * 64;
    L.u = L.ysum + ngrp * 4;
    const int u = nq * 128 > nb * 4 ? nq * 128 : nb * 4;
    L.cand = (L.u + u + 15) / 16 * 16;
    L.bytes = L.cand + 64 * 8;
    if (L.bytes < stream_bytes) L.bytes = stream_bytes;
    return L;
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_select(DecArgs A)
{
    constexpr int KS = DK / 32;
    extern __shared__ __align__(16) unsigned char dsm[];
    const Dims &d = A.d;
    const int pairs = d.B * d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hd = lane & 15;
    const float sl2 = d.scale * kLog2e;

    if ((int)blockIdx.x >= pairs) {
        StreamLds<DV> &sw = *(StreamLds<DV> *)dsm;
        const int id = blockIdx.x - pairs;
        const bool win = id < pairs * A.nw;
        const int pair = win ? id / A.nw : id - pairs * A.nw, r = win ? id % A.nw : 0;
        const int b = pair / d.Hkv, g = pair % d.Hkv;
        const int t = dec_t(A.seq_lens, b, d.T);
        const uint16_t *K = (const uint16_t *)A.k + (long)pair * d.T * DK;
        const uint16_t *V = (const uint16_t *)A.v + (long)pair * d.T * DV;
        const uint16_t *qrow = (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK;
        Acc<DV> acc;
        acc.init();
        unsigned char *reg = sw.wave[wave];
        if (win) {
            // ---- window: keys [lo + 256 r, lo + 256 r + 256) of [lo, t]; wavefront w
            // takes the two 32-key steps at lo + 256 r + 128 s + 32 w, loaded at once
            const int lo = max(0, t - d.w + 1), kend = t + 1;
            const int k0 = lo + r * kWinKeys + wave * kStepKeys, k1 = k0 + kWaves * kStepKeys;
            if (k0 < kend) {   // uniform over the wavefront
                Step<DK, DV> sa, sb;
                load_step(sa, K, V, k0, kend, d.T - 1, lane);
                load_step(sb, K, V, k1, kend, d.T - 1, lane);
                bf16x8 qf[KS];
                load_q(qrow, lane, qf, KS);
                float p[8];
                compute_step(sa, qf, k0, kend, sl2, acc, reg, lane, p);
                if (k1 < kend) compute_step(sb, qf, k1, kend, sl2, acc, reg, lane, p);
            }
            merge_waves(acc, sw, A.part + ((long)pair * A.nslot + A.nq + r) * part_stride<DV>(), tid);
        } else {
            // ---- the always-kept blocks, one per wavefront (none when the block
            // lists are given: they need not contain them)
            const int j = A.idx_in ? -1 : forced_block(wave, t / 64);
            if (j >= 0) attend_block<DK, DV>(K, V, qrow, j, t, d.T, sl2, acc, reg, lane);
            merge_waves(acc, sw, A.part + ((long)pair * A.nslot + A.nq + A.nw) * part_stride<DV>(), tid);
        }
        return;
    }

    // ---- selection of pair blockIdx.x
    const SelLayout Ly = sel_layout(A.ngrp, A.nq, d.nb, 0);
    float *s_lse = (float *)dsm;
    float(*s_W)[16] = (float(*)[16])(dsm + Ly.w);
    float *s_ysum = (float *)(dsm + Ly.ysum);
    float(*s_pm)[16] = (float(*)[16])(dsm + Ly.u);
    float(*s_pl)[16] = s_pm + A.nq;
    float *s_S = (float *)(dsm + Ly.u);        // after the partials are reduced
    uint64_t *s_cand = (uint64_t *)(dsm + Ly.cand);
    const int pair = blockIdx.x, b = pair / d.Hkv, g = pair % d.Hkv;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int jcur = t / 64, nvis = n_visible(t);
    const float *pp = A.part + (long)pair * A.nslot * part_stride<DV>();
    if (!A.idx_in) {
        const int ngv = (nvis + kStepKeys - 1) / kStepKeys;   // groups with a visible slot
        const float *bt = A.bt + (long)pair * A.nbp * 16;
        const float *gmax = A.gmax + (long)pair * A.ngrp * 16;
        const float *gtail = A.gtail + (long)pair * A.ngrp * 16;
        const int nitem = 4 * (jcur + 1);   // chunk c = 4 j + hq: heads 4 hq .. 4 hq + 3 of block j
        const u32x4 z = {0u, 0u, 0u, 0u};
        // ---- one round of loads
        float pmv[2], plv[2];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int i = tid + u * kThreads, r = i >> 4, h = i & 15;
            pmv[u] = r < A.nq ? pp[r * part_stride<DV>() + h] : -INFINITY;
            plv[u] = r < A.nq ? pp[r * part_stride<DV>() + 16 + h] : 0.f;
        }
        constexpr int kG = kMaxGroups * 4 / kThreads;   // group chunks per thread at most
        u32x4 gm[kG], gt[kG];
#pragma unroll
        for (int u = 0; u < kG; u++) {
            const int c = tid + u * kThreads;
            gm[u] = c < ngv * 4 ? ld16(gmax + 4 * c) : z;
            gt[u] = c < ngv * 4 ? ld16(gtail + 4 * c) : z;
        }
        u32x4 bv[kSelItems];
#pragma unroll
        for (int u = 0; u < kSelItems; u++) {
            const int c = tid + u * kThreads;
            bv[u] = c < nitem && (c >> 5) < ngv ? ld16(bt + 4 * c) : z;   // block c/4 lies in group c/32
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int i = tid + u * kThreads;
            if (i < A.nq * 16) {
                s_pm[i >> 4][i & 15] = pmv[u];
                s_pl[i >> 4][i & 15] = plv[u];
            }
        }
        for (int i = tid + 2 * kThreads; i < A.nq * 16; i += kThreads) {   // more than 32 compressed ranges
            s_pm[i >> 4][i & 15] = pp[(i >> 4) * part_stride<DV>() + (i & 15)];
            s_pl[i >> 4][i & 15] = pp[(i >> 4) * part_stride<DV>() + 16 + (i & 15)];
        }
        lds_barrier();
        // ---- exact log-sum-exp of the compressed branch per head (log2 units)
        if (tid < 16) {
            float M = -INFINITY;
#pragma unroll 4
            for (int r = 0; r < A.nq; r++) M = fmaxf(M, s_pm[r][tid]);
            float L = 0.f;
#pragma unroll 4
            for (int r = 0; r < A.nq; r++)
                if (s_pm[r][tid] != -INFINITY) L = __builtin_fmaf(s_pl[r][tid], fast_exp2(s_pm[r][tid] - M), L);
            s_lse[tid] = L > 0.f ? M + fast_log2(L) : -INFINITY;
        }
        lds_barrier();
        // ---- group weights and the weighted last-slot terms
        {
            const int hq = tid & 3;
            float ls[4];
#pragma unroll
            for (int e = 0; e < 4; e++) ls[e] = s_lse[4 * hq + e];
#pragma unroll
            for (int u = 0; u < kG; u++) {
                // chunk c of the group arrays: heads 4 hq .. 4 hq + 3 of group c / 4
                const int c = tid + u * kThreads, grp = c >> 2;
                const bool valid = c < ngv * 4;
                float yq = 0.f;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float w = valid ? fast_exp2(__uint_as_float(gm[u][e]) - ls[e]) : 0.f;
                    if (valid) s_W[grp][4 * hq + e] = w;
                    yq = __builtin_fmaf(w, __uint_as_float(gt[u][e]), yq);
                }
                yq += __shfl_xor(yq, 1, 64);
                yq += __shfl_xor(yq, 2, 64);
                if (valid && hq == 0) s_ysum[grp] = yq;
            }
        }
        lds_barrier();
        // ---- block scores; the four chunks of a block are a quad of lanes
        for (int c0 = 0; c0 < nitem; c0 += kSelItems * kThreads) {   // uniform trip count
            if (c0 > 0) {
#pragma unroll
                for (int u = 0; u < kSelItems; u++) {
                    const int c = c0 + tid + u * kThreads;
                    bv[u] = c < nitem && (c >> 5) < ngv ? ld16(bt + 4 * c) : z;
                }
            }
#pragma unroll
            for (int u = 0; u < kSelItems; u++) {
                const int c = c0 + tid + u * kThreads, j = c >> 2, grp = j >> 3, hq = c & 3;
                float acc = 0.f;
                if (c < nitem && grp < ngv) {
#pragma unroll
                    for (int e = 0; e < 4; e++) acc = __builtin_fmaf(__uint_as_float(bv[u][e]), s_W[grp][4 * hq + e], acc);
                }
                acc += __shfl_xor(acc, 1, 64);
                acc += __shfl_xor(acc, 2, 64);
                if (c < nitem && hq == 0) s_S[j] = acc + ((j & 7) == 0 && j > 0 && grp - 1 < ngv ? s_ysum[grp - 1] : 0.f);
            }
        }
        lds_barrier();
    }
    if (wave == 0) {
        if (!A.idx_in) wave_select_topn_sort(s_S, jcur, d.n, A.idx + (long)pair * d.n, lane, s_cand);
    } else {
        // gates: 4 lanes per (head, gate) dot product of length DK
        const int t1 = tid - 64;   // 0 .. 191 = 48 dot products x 4 lanes
        const int dot = t1 >> 2, part = t1 & 3;
        const int h = dot / 3, c = dot % 3;
        const uint16_t *qr = (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + h) * DK;
        const uint16_t *wr = (const uint16_t *)A.wg + ((long)(g * 16 + h) * 3 + c) * DK;
        float z = 0.f;
        for (int ch = part; ch < DK / 8; ch += 4) z = dot8_bf16(ld16(wr + 8 * ch), ld16(qr + 8 * ch), z);
        z += __shfl_xor(z, 1, 64);
        z += __shfl_xor(z, 2, 64);
        if (part == 0) {
            z += __uint_as_float((uint32_t)((const uint16_t *)A.bg)[(g * 16 + h) * 3 + c] << 16);
            A.gates[(long)pair * 48 + h * 3 + c] = sigmoidf_(z);
        }
    }
}

// ---------------------------------------------------------------------------
// Merge of one pair's partial slots: each branch's slots combined (max,
// rescaled sums and outputs), normalised, gated and summed into o.  Thread
// (slot, head) computes its slot's weight gate * 2^(m_slot - M) / L from the
// branch's (max, sum) pairs in LDS (independent reads); then each thread
// issues the loads of every slot for its 4-column chunk at once.
constexpr int kMergeThreads = 512;
constexpr int kMergeBatch = 12;   // slots whose chunks one thread loads together

struct MergeLds {
    float m[kMaxSlots][16], l[kMaxSlots][16], w[kMaxSlots][16];
};

template <int DV>
__device__ __forceinline__ void merge_pair(const DecArgs &A, MergeLds &sm, int pair)
{
    const Dims &d = A.d;
    const int tid = threadIdx.x;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int nslot = A.nslot;
    const float *pp = A.part + (long)pair * nslot * part_stride<DV>();
    for (int i = tid; i < nslot * 16; i += kMergeThreads) {
        const int r = i >> 4, h = i & 15;
        sm.m[r][h] = pp[r * part_stride<DV>() + h];
        sm.l[r][h] = pp[r * part_stride<DV>() + 16 + h];
    }
    __syncthreads();
    for (int i = tid; i < nslot * 16; i += kMergeThreads) {
        const int r = i >> 4, h = i & 15;
        // the slot's branch (0 compressed, 1 selected, 2 window: the gate order)
        const int br = r < A.nq ? 0 : (r < A.nq + A.nw ? 2 : 1);
        const int s0 = br == 0 ? 0 : (br == 1 ? A.nq + A.nw : A.nq);
        const int n = br == 0 ? A.nq : (br == 1 ? 1 + A.ns : A.nw);
        float M = -INFINITY;
#pragma unroll 4
        for (int u = s0; u < s0 + n; u++) M = fmaxf(M, sm.m[u][h]);
        float L = 0.f;
#pragma unroll 4
        for (int u = s0; u < s0 + n; u++)
            if (sm.m[u][h] != -INFINITY) L = __builtin_fmaf(sm.l[u][h], fast_exp2(sm.m[u][h] - M), L);
        const float gate = A.gates[(long)pair * 48 + h * 3 + br];
        sm.w[r][h] = sm.m[r][h] != -INFINITY && L > 0.f ? gate * fast_exp2(sm.m[r][h] - M) / L : 0.f;
    }
    __syncthreads();
    uint16_t *o = (uint16_t *)A.o + ((long)b * d.Hq + g * 16) * DV;
    for (int c4 = tid; c4 < 16 * DV / 4; c4 += kMergeThreads) {
        const int e = 4 * c4, h = e / DV;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nslot; s0 += kMergeBatch) {
            u32x4 v[kMergeBatch];
#pragma unroll
            for (int u = 0; u < kMergeBatch; u++) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                v[u] = s0 + u < nslot ? ld16(pp + (s0 + u) * part_stride<DV>() + 32 + e) : z;
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; u++) {
                const float w = s0 + u < nslot ? sm.w[s0 + u][h] : 0.f;
#pragma unroll
                for (int c = 0; c < 4; c++) y[c] = __builtin_fmaf(w, __uint_as_float(v[u][c]), y[c]);
            }
        }
        uint2 out;
        out.x = pack_bf16x2(y[0], y[1]);
        out.y = pack_bf16x2(y[2], y[3]);
        *(uint2 *)(o + e) = out;
    }
}

// ---------------------------------------------------------------------------
// Selected blocks: workgroup (pair, r) takes the distinct valid entries
// 4r .. 4r+3 of the pair's list in ascending order, one per wavefront --
// without the always-kept blocks, which k_dec_select's block workgroups
// took, unless the lists were given.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_dec_gather(DecArgs A)
{
    __shared__ StreamLds<DV> sm;
    const Dims &d = A.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hd = lane & 15;
    const int pair = blockIdx.x / A.ns, r = blockIdx.x % A.ns;
    const int b = pair / d.Hkv, g = pair % d.Hkv;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int jcur = t / 64;
    const float sl2 = d.scale * kLog2e;
    const int32_t *ilist = (A.idx_in ? A.idx_in : A.idx) + (long)pair * d.n;
    const int jb = lane < d.n ? ilist[lane] : -1;
    bool ok = jb >= 0 && jb <= jcur;
    if (!A.idx_in) ok = ok && jb != forced_block(0, jcur) && jb != forced_block(1, jcur) && jb != forced_block(2, jcur);
    for (int u = 0; u < 16; u++) {
        const int other = __shfl(jb, u, 64);
        if (u < lane && other == jb) ok = false;
    }
    // rank of each kept entry by value (a given list need not be ascending)
    const uint64_t v = __ballot(ok);
    int rank = 0;
    for (int u = 0; u < 16; u++) {
        const int other = __shfl(jb, u, 64);
        if (((v >> u) & 1ull) && other < jb) rank++;
    }
    const uint64_t hit = __ballot(ok && rank == kBlocksPerGather * r + wave);
    const int j = hit ? __shfl(jb, __builtin_ctzll(hit), 64) : -1;   // uniform
    Acc<DV> acc;
    acc.init();
    if (j >= 0)
        attend_block<DK, DV>((const uint16_t *)A.k + (long)pair * d.T * DK, (const uint16_t *)A.v + (long)pair * d.T * DV,
                             (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK, j, t, d.T, sl2, acc,
                             sm.wave[wave], lane);
    merge_waves(acc, sm, A.part + ((long)pair * A.nslot + A.nq + A.nw + 1 + r) * part_stride<DV>(), tid);
}

template <int DV>
__global__ __launch_bounds__(kMergeThreads) void k_dec_merge(DecArgs A)
{
    __shared__ MergeLds sm;
    merge_pair<DV>(A, sm, blockIdx.x);
}

template <int DK, int DV>
hipError_t launch_decode_dims(const DecArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int pairs = d.B * d.Hkv;
    const SelLayout L = sel_layout(A.ngrp, A.nq, d.nb, (int)sizeof(StreamLds<DV>));
    hipLaunchKernelGGL((k_dec_stream<DK, DV>), dim3(pairs * A.nq), dim3(kThreads), 0, s, A);
    hipLaunchKernelGGL((k_dec_select<DK, DV>), dim3(pairs * (2 + A.nw)), dim3(kThreads), L.bytes, s, A);
    hipLaunchKernelGGL((k_dec_gather<DK, DV>), dim3(pairs * A.ns), dim3(kThreads), 0, s, A);
    hipLaunchKernelGGL((k_dec_merge<DV>), dim3(pairs), dim3(kMergeThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace

// Workgroups per pair over the compressed cache and slots per workgroup: at
// least 512 workgroups in all when the cache allows (the compressed ranges
// run two workgroups per CU), each range a multiple of 256 slots and at most
// 1,024.
static int cmp_split(const Dims &d, int *keys)
{
    const long pairs = (long)d.B * d.Hkv;
    const int rounds = (d.npad + kCmpRound - 1) / kCmpRound;          // 256-slot rounds in the cache
    const int want = (int)std::min<long>(rounds, std::max<long>(1, (512 + pairs - 1) / pairs));
    const int per = std::min((rounds + want - 1) / want, kMaxCmpKeys / kCmpRound);   // rounds per workgroup
    *keys = per * kCmpRound;
    return (rounds + per - 1) / per;
}

// Gather workgroups per pair: four blocks each, enough for all n entries of
// a given list (without one, the n - 3 free picks need fewer).
static int gather_groups(const Dims &d) { return (d.n + kBlocksPerGather - 1) / kBlocksPerGather; }

bool decode_mfma_supported(const Dims &d)
{
    if (d.dtype != NSA_BF16 || d.G != 16) return false;
    if (!((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64))) return false;
    const long pairs = (long)d.B * d.Hkv;
    int cmp_keys;
    const long nq = cmp_split(d, &cmp_keys), nw = (d.w + kWinKeys - 1) / kWinKeys, ns = gather_groups(d);
    return d.nb <= 8192 && d.npad / kStepKeys <= kMaxGroups && nq <= kMaxCmpSlots && nq + nw + 1 + ns <= kMaxSlots &&
           sel_layout(d.npad / kStepKeys, (int)nq, d.nb, 0).bytes <= 64 * 1024 && pairs * (2 + nw) <= 0x7fffffffL &&
           pairs * nq <= 0x7fffffffL && pairs * ns <= 0x7fffffffL;
}

// Workspace of the matrix-core decode step, carved from `ws` when non-null.
size_t decode_mfma_layout(const Dims &d, void *ws, DecArgs *A)
{
    const long pairs = (long)d.B * d.Hkv;
    int cmp_keys;
    const int nq = cmp_split(d, &cmp_keys), nw = (d.w + kWinKeys - 1) / kWinKeys, ns = gather_groups(d);
    const int nslot = nq + nw + 1 + ns;
    const int nbp = d.npad / 4, ngrp = d.npad / kStepKeys;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = (off + bytes + 255) / 256 * 256;
        return o;
    };
    const size_t o_part = take(4 * pairs * nslot * (32 + 16 * (size_t)d.dv));
    const size_t o_bt = take(4 * pairs * nbp * 16);
    const size_t o_gm = take(4 * pairs * ngrp * 16), o_gt = take(4 * pairs * ngrp * 16);
    const size_t o_gates = take(4 * pairs * 48);
    const size_t o_idx = take(4 * pairs * d.n);
    if (A && ws) {
        char *w = (char *)ws;
        A->nq = nq;
        A->cmp_keys = cmp_keys;
        A->nw = nw;
        A->ns = ns;
        A->nslot = nslot;
        A->nbp = nbp;
        A->ngrp = ngrp;
        A->part = (float *)(w + o_part);
        A->bt = (float *)(w + o_bt);
        A->gmax = (float *)(w + o_gm);
        A->gtail = (float *)(w + o_gt);
        A->gates = (float *)(w + o_gates);
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
