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
//            splits, block scores (heads summed, weights 1,2,2,2,1) and the
//            top-n selection;
//   phase C  the selected blocks (one wavefront per block, online softmax);
//   phase D  merge of the compressed, window and selected partials and the
//            gated sum.
// Phase A is one kernel, one workgroup of 8 wavefronts per (pair, split) of
// 256 keys; each wavefront issues every load of its 32 keys on entry, so a CU
// keeps several hundred KB in flight.  B, C and D run in a second kernel, one
// workgroup of 16 wavefronts per (sequence, KV head), so the step costs two
// launches.
//
// Lane view (one position, 16 heads, wave64): head hd = lane%16, key group
// q = lane/16.  A 32-key step is two 16x16x32 S^T tiles whose rows hold keys
// 8*(i/4) + i%4 and 8*(i/4) + 4 + i%4, so lane (q, hd) ends with the logits
// of keys 8q .. 8q+7 of the step for head hd: exactly the B operand of
// O^T = V^T P^T.  K is loaded straight into the A-operand registers of the
// S^T tiles; V goes through a per-wavefront LDS region and comes back as V^T
// operand fragments by transpose reads.
#include "mfma_util.h"
#include "nsa_internal.h"
#include "select_util.h"

namespace nsa {

namespace {

constexpr int kSThreads = 512;              // phase A: 8 wavefronts
constexpr int kWaveKeys = 32;               // keys per wavefront (one 32-key step)
constexpr int kSplitKeys = 8 * kWaveKeys;   // keys per phase-A workgroup

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
// the 16-byte row stores fill whole rows.  Afterwards the same bytes hold the
// wavefront's output for the workgroup merge.
template <int DV>
struct DecWaveLds {
    static constexpr int U = DV / 16;                            // 32-byte units per V row
    static constexpr int VBYTES = kWaveKeys * 2 * DV;
    static constexpr int OBYTES = 16 * (DV + 4) * 4;             // [16][DV+4] fp32
    static constexpr int BYTES = VBYTES > OBYTES ? VBYTES : OBYTES;
    __device__ static int vaddr(int r, int unit, int byte)
    {
        const int sig = ((r & 3) | ((r >> 1) & 4)) & (U - 1);
        return r * 2 * DV + ((unit ^ sig) << 5) + byte;
    }
};

template <int DV>
struct DecLds {
    unsigned char wave[8][DecWaveLds<DV>::BYTES];
    float mx[8][16];
    float ls[8][16];
};

// Phase A.  Workgroup = (pair, slot): slots 0..cs-1 are the compressed slots
// [256 s, 256 s + 256), slots cs.. the window keys from max(0, t-w+1) in
// steps of 256.  Wavefront w takes keys kbeg .. kbeg+31; all 8 use the
// workgroup's maximum per head, so the partial (max, sum, unnormalised
// output) is one sum.
template <int DK, int DV>
__global__ __launch_bounds__(kSThreads) void k_dec_stream(DecArgs A)
{
    constexpr int KS = DK / 32;      // 16x16x32 steps over the head dim
    constexpr int DT = DV / 16;      // 16-wide dv tiles
    constexpr int VC = DV / 8;       // 16-byte chunks per V row
    constexpr int VL = kWaveKeys * VC / 64;   // V chunks per lane
    using WL = DecWaveLds<DV>;
    __shared__ DecLds<DV> sm;
    const Dims &d = A.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = lane & 15, q = lane >> 4;
    const float sl2 = d.scale * kLog2e;
    const int nslots = A.cs + A.ws;
    const int pair = blockIdx.x / nslots, slot = blockIdx.x % nslots;
    const int b = pair / d.Hkv;
    const int t = dec_t(A.seq_lens, b, d.T);

    // this wavefront's keys
    int kbeg, kend, kclamp;
    const bool cmp = slot < A.cs;
    const uint16_t *K, *V;
    if (cmp) {
        const int nvis = t >= 31 ? (t - 31) / 16 + 1 : 0;
        kbeg = slot * kSplitKeys + wave * kWaveKeys;
        kend = min(kbeg + kWaveKeys, nvis);
        kclamp = d.npad - 1;
        K = (const uint16_t *)A.kc + (long)pair * d.npad * DK;
        V = (const uint16_t *)A.vc + (long)pair * d.npad * DV;
    } else {
        const int lo = max(0, t - d.w + 1);
        kbeg = lo + (slot - A.cs) * kSplitKeys + wave * kWaveKeys;
        kend = min(kbeg + kWaveKeys, t + 1);
        kclamp = d.T - 1;
        K = (const uint16_t *)A.k + (long)pair * d.T * DK;
        V = (const uint16_t *)A.v + (long)pair * d.T * DV;
    }
    const bool active = kbeg < kend;   // uniform over the wavefront

    // issue every load of the step: K into the S^T operand registers (tile A
    // row i holds key 8(i/4) + i%4, tile B key 8(i/4) + 4 + i%4), V rows into
    // registers for the LDS region, the query fragments
    const int kA = kbeg + 8 * (hd >> 2) + (hd & 3);
    u32x4 ka[KS], kb2[KS], vr[VL];
    bf16x8 qf[KS];
    if (active) {
        const uint16_t *ra = K + (long)min(kA, kclamp) * DK + 8 * q;
        const uint16_t *rb = K + (long)min(kA + 4, kclamp) * DK + 8 * q;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            ka[kk] = ld16(ra + 32 * kk);
            kb2[kk] = ld16(rb + 32 * kk);
        }
        // Keys past kend enter the PV product with probability 0; their V
        // rows are read from key kend-1 instead, a slot or token the caller
        // has written, because the rows past it need not be finite and
        // 0 * NaN would reach the output.
#pragma unroll
        for (int u = 0; u < VL; u++) {
            const int c = 64 * u + lane, key = c / VC, ch = c % VC;
            vr[u] = ld16(V + (long)min(kbeg + key, kend - 1) * DV + ch * 8);
        }
        const uint16_t *qrow = (const uint16_t *)A.q + ((long)b * d.Hq + (pair % d.Hkv) * 16 + hd) * DK;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) qf[kk] = as_bf16x8(ld16(qrow + 32 * kk + 8 * q));
    }

    // logits of keys kbeg + 8q .. +7 for head hd
    float s[8];
    float mx = -INFINITY;
    if (active) {
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            accA = mfma16(as_bf16x8(ka[kk]), qf[kk], accA);
            accB = mfma16(as_bf16x8(kb2[kk]), qf[kk], accB);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            s[u] = kbeg + 8 * q + u < kend ? accA[u] * sl2 : -INFINITY;
            s[4 + u] = kbeg + 8 * q + 4 + u < kend ? accB[u] * sl2 : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 8; e++) mx = fmaxf(mx, s[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) s[e] = -INFINITY;
    }
    mx = head_max(mx);
    if (q == 0) sm.mx[wave][hd] = mx;
    lds_barrier();
    float M = sm.mx[0][hd];
#pragma unroll
    for (int w = 1; w < 8; w++) M = fmaxf(M, sm.mx[w][hd]);

    float p[8], l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        p[e] = M == -INFINITY ? 0.f : fast_exp2(s[e] - M);
        l += p[e];
    }
    if (cmp) {
        // block a = (kbeg + 8q)/4 gets keys 4a..4a+3 here (weights 2,2,2,1);
        // its remaining weight-1 key 4a-1 is the previous block's Y term
        float *bx = A.bx + (long)pair * 16 * A.nbp + (long)hd * A.nbp;
        float *by = A.by + (long)pair * 16 * A.nbp + (long)hd * A.nbp;
        const int a = (kbeg + 8 * q) >> 2;
        if (a + 1 < A.nbp) {
            *(float2 *)&bx[a] = make_float2(2.f * (p[0] + p[1] + p[2]) + p[3], 2.f * (p[4] + p[5] + p[6]) + p[7]);
            *(float2 *)&by[a] = make_float2(p[3], p[7]);
        }
    }
    l = head_sum(l);

    // O^T += V^T P^T through this wavefront's LDS region
    unsigned char *reg = sm.wave[wave];
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
        for (int u = 0; u < VL; u++) {
            const int c = 64 * u + lane, key = c / VC, ch = c % VC;
            st16(reg + WL::vaddr(key, ch >> 1, 16 * (ch & 1)), vr[u]);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's stores are in LDS
        __builtin_amdgcn_wave_barrier();
        const bf16x8 pb = pack8(p);
        // lane (g, s) of a 16-lane group points at columns 16dt + 4(s%4) of
        // rows 8g + s/4 (then + 4): lane i then holds dv 16dt + i for keys
        // 8g .. 8g+7, the A operand of O^T = V^T P^T
        const int g = lane >> 4, sl = lane & 15;
        const int r0 = 8 * g + (sl >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const uint2 lo = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0, dt, 8 * (sl & 3))));
            const uint2 hi = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0 + 4, dt, 8 * (sl & 3))));
            const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
            oacc[dt] = mfma16(as_bf16x8(w), pb, oacc[dt]);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // the transpose reads are done before the region is reused
        __builtin_amdgcn_wave_barrier();
    }
    // merge of the 8 wavefronts (same M): O and l summed in wave order
    float *ol = (float *)reg;   // [16][DV+4]
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int u = 0; u < 4; u++) ol[hd * (DV + 4) + 16 * dt + 4 * q + u] = oacc[dt][u];
    if (q == 0) sm.ls[wave][hd] = l;
    lds_barrier();
    const long pidx = (long)pair * nslots + slot;
    float *pm = A.pm + pidx * 16;
    float *pl = A.pl + pidx * 16;
    float *po = A.po + pidx * 16 * DV;
    for (int e = tid; e < 16 * DV; e += kSThreads) {
        const int h = e / DV, c = e % DV;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 8; w++) acc += ((const float *)sm.wave[w])[h * (DV + 4) + c];
        po[e] = acc;
    }
    if (tid < 16) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < 8; w++) L += sm.ls[w][tid];
        pl[tid] = L;
        pm[tid] = M;   // the workgroup maximum of head tid (lane tid holds head tid)
    }
}

// ---------------------------------------------------------------------------
// Phases B, C and D for one (sequence, KV head): one workgroup of 16
// wavefronts.
constexpr int kTailThreads = 1024;
constexpr int kTailWaves = 16;

template <int DV>
struct TailLds {
    union {
        struct {                       // phase B
            float wsp[64][16];         // merge weight of each compressed split (per head)
            float wwp[64][16];         // ... and window split
            float lse[16];
            uint2 cand[64];
            float S[8192];             // block scores (nb <= 8192)
        } b;
        unsigned char wave[kTailWaves][DecWaveLds<DV>::BYTES];   // phase C
    } u;
    float2 ocw[16][DV];                // merged compressed and window outputs (normalised)
    float gate[16][3];
    float ms[16], lsum[16];            // selected branch: max / sum per head
    float wm[kTailWaves][16], wl[kTailWaves][16];
    int blist[16];
    int nblk;
};

template <int DK, int DV>
__global__ __launch_bounds__(kTailThreads) void k_dec_tail(DecArgs A)
{
    constexpr int KS = DK / 32, DT = DV / 16, VC = DV / 8, VL = kWaveKeys * VC / 64;
    constexpr int NT = kTailThreads;
    using WL = DecWaveLds<DV>;
    __shared__ TailLds<DV> sm;
    const Dims &d = A.d;
    const int pair = blockIdx.x, b = pair / d.Hkv, g = pair % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hd = lane & 15, q = lane >> 4;
    const int t = dec_t(A.seq_lens, b, d.T);
    const int jcur = t / 64;
    const float sl2 = d.scale * kLog2e;
    const int nsplit = A.cs + A.ws;
    const float *pm = A.pm + (long)pair * nsplit * 16, *pl = A.pl + (long)pair * nsplit * 16;

    // ---- phase B: exact log-sum-exp per head and branch, merge weights of
    // the splits, block scores; then wavefront 0 selects the blocks while the
    // others merge the compressed and window partials and form the gates
    const int32_t *ilist = A.idx_in ? A.idx_in + (long)pair * d.n : A.idx + (long)pair * d.n;
    auto &B = sm.u.b;
    // block j: its own keys 4j..4j+3 (X) plus key 4j-1 (Y of block j-1);
    // phase A wrote blocks 0..nbp-1, a block past them has no key of its own.
    // Thread tid's first block is loaded now, so that these loads overlap the
    // log-sum-exp below.
    const float *bx = A.bx + (long)pair * 16 * A.nbp, *by = A.by + (long)pair * 16 * A.nbp;
    float xv[16], yv[16];
    auto load_terms = [&](int j) {
        const bool hx = j < A.nbp, hy = j > 0 && j - 1 < A.nbp;
#pragma unroll
        for (int h = 0; h < 16; h++) {
            xv[h] = hx ? bx[(long)h * A.nbp + j] : 0.f;
            yv[h] = hy ? by[(long)h * A.nbp + j - 1] : 0.f;
        }
    };
    if (!A.idx_in && tid <= jcur) load_terms(tid);
    {
        // wavefront h: head h; lane s holds split s of each branch (cs, ws <= 64)
        const int h = wave;
        auto branch = [&](int s0, int ns, float(*wp)[16]) {
            const float mv = lane < ns ? pm[(long)(s0 + lane) * 16 + h] : -INFINITY;
            const float lv = lane < ns ? pl[(long)(s0 + lane) * 16 + h] : 0.f;
            float M = mv;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
            float L = M == -INFINITY ? 0.f : lv * fast_exp2(mv - M);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
            const float lse = M == -INFINITY || L <= 0.f ? -INFINITY : M + fast_log2(L);
            if (lane < ns) wp[lane][h] = lse == -INFINITY ? 0.f : fast_exp2(mv - lse);
            return lse;
        };
        const float lse = branch(0, A.cs, B.wsp);
        branch(A.cs, A.ws, B.wwp);
        if (lane == 0) B.lse[h] = lse;
    }
    lds_barrier();
    if (!A.idx_in) {
        constexpr int kBlkPerSplit = kSplitKeys / 4;
        for (int j = tid; j <= jcur; j += NT) {
            if (j != tid) load_terms(j);
            const int sj = j / kBlkPerSplit, sp = (j - 1) / kBlkPerSplit;
            const bool hy = j > 0 && j - 1 < A.nbp;
            float acc = 0.f;
#pragma unroll
            for (int h = 0; h < 16; h++) {
                acc += xv[h] * B.wsp[sj][h];
                if (hy) acc += yv[h] * B.wsp[sp][h];
            }
            B.S[j] = acc;
        }
        lds_barrier();
    }
    const float *po = A.po + (long)pair * nsplit * 16 * DV;
    if (wave == 0) {
        if (!A.idx_in) {
            wave_select_topn_fast(B.S, jcur, d.n, A.idx + (long)pair * d.n, lane, B.cand);
            // the list is read back below by this wavefront's lanes
            __builtin_amdgcn_s_waitcnt(0);
            __threadfence_block();
        }
        // the distinct valid blocks, ascending (the list is ascending unless supplied)
        const int jb = lane < d.n ? ilist[lane] : -1;
        bool ok = jb >= 0 && jb <= jcur;
        for (int u2 = 0; u2 < 16; u2++) {
            const int other = __shfl(jb, u2, 64);
            if (u2 < lane && other == jb) ok = false;
        }
        const uint64_t v = __ballot(ok);
        if (ok) sm.blist[__popcll(v & __lanemask_lt())] = jb;
        if (lane == 0) sm.nblk = __popcll(v);
    } else {
        const int t1 = tid - 64;   // 0 .. NT-65
        // gates: 16 threads per (head, gate) dot product of length DK
        for (int task = t1; task < 16 * 3 * 16; task += NT - 64) {
            const int dot = task >> 4, part = task & 15;
            const int h = dot / 3, c = dot % 3;
            const uint16_t *qr = (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + h) * DK;
            const uint16_t *wr = (const uint16_t *)A.wg + ((long)(g * 16 + h) * 3 + c) * DK;
            float z = 0.f;
            for (int ch = part; ch < DK / 8; ch += 16) {
                const u32x4 wv = ld16(wr + 8 * ch), qv = ld16(qr + 8 * ch);
                z = dot8_bf16(wv, qv, z);
            }
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) z += __shfl_xor(z, off, 16);
            if (part == 0) {
                z += __uint_as_float((uint32_t)((const uint16_t *)A.bg)[(g * 16 + h) * 3 + c] << 16);
                sm.gate[h][c] = sigmoidf_(z);
            }
        }
        // compressed and window outputs: the splits' partials, weighted
        for (int e = t1; e < 16 * DV; e += NT - 64) {
            const int h = e / DV, c = e % DV;
            float oc = 0.f, ow = 0.f;
#pragma unroll 4
            for (int s2 = 0; s2 < A.cs; s2++) oc += po[(long)s2 * 16 * DV + e] * B.wsp[s2][h];
#pragma unroll 2
            for (int s2 = 0; s2 < A.ws; s2++) ow += po[(long)(A.cs + s2) * 16 * DV + e] * B.wwp[s2][h];
            sm.ocw[h][c] = make_float2(oc, ow);
        }
    }
    lds_barrier();

    // ---- phase C: wavefront w attends to block blist[w] (two 32-key steps)
    float m = -INFINITY, l = 0.f;
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    unsigned char *reg = sm.u.wave[wave];
    if (wave < sm.nblk) {
        const int j = sm.blist[wave];
        const uint16_t *K = (const uint16_t *)A.k + (long)pair * d.T * DK;
        const uint16_t *V = (const uint16_t *)A.v + (long)pair * d.T * DV;
        const uint16_t *qrow = (const uint16_t *)A.q + ((long)b * d.Hq + g * 16 + hd) * DK;
        bf16x8 qf[KS];
#pragma unroll
        for (int kk = 0; kk < KS; kk++) qf[kk] = as_bf16x8(ld16(qrow + 32 * kk + 8 * q));
        for (int st = 0; st < 2; st++) {
            const int kbeg = 64 * j + kWaveKeys * st, kend = min(kbeg + kWaveKeys, t + 1);
            if (kbeg >= kend) break;   // uniform over the wavefront
            const int kA = min(kbeg + 8 * (hd >> 2) + (hd & 3), d.T - 1);
            const int kB = min(kbeg + 8 * (hd >> 2) + (hd & 3) + 4, d.T - 1);
            u32x4 ka[KS], kb2[KS], vr[VL];
#pragma unroll
            for (int kk = 0; kk < KS; kk++) {
                ka[kk] = ld16(K + (long)kA * DK + 8 * q + 32 * kk);
                kb2[kk] = ld16(K + (long)kB * DK + 8 * q + 32 * kk);
            }
#pragma unroll
            for (int u = 0; u < VL; u++) {
                const int c = 64 * u + lane, key = c / VC, ch = c % VC;
                // tokens past t read from token t's row (see phase A)
                vr[u] = ld16(V + (long)min(kbeg + key, kend - 1) * DV + ch * 8);
            }
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; kk++) {
                accA = mfma16(as_bf16x8(ka[kk]), qf[kk], accA);
                accB = mfma16(as_bf16x8(kb2[kk]), qf[kk], accB);
            }
            float sv[8], mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; u++) {
                sv[u] = kbeg + 8 * q + u < kend ? accA[u] * sl2 : -INFINITY;
                sv[4 + u] = kbeg + 8 * q + 4 + u < kend ? accB[u] * sl2 : -INFINITY;
                mx = fmaxf(mx, fmaxf(sv[u], sv[4 + u]));
            }
            mx = head_max(mx);
            const float mn = fmaxf(m, mx);   // finite: the step has a visible key
            const float al = fast_exp2(m - mn);
            float p[8], sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                p[e] = fast_exp2(sv[e] - mn);
                sum += p[e];
            }
            l = l * al + head_sum(sum);
            m = mn;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) oacc[dt] *= al;
#pragma unroll
            for (int u = 0; u < VL; u++) {
                const int c = 64 * u + lane, key = c / VC, ch = c % VC;
                st16(reg + WL::vaddr(key, ch >> 1, 16 * (ch & 1)), vr[u]);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's stores are in LDS
            __builtin_amdgcn_wave_barrier();
            const bf16x8 pb = pack8(p);
            const int gq = lane >> 4, sl = lane & 15, r0 = 8 * gq + (sl >> 2);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const uint2 lo = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0, dt, 8 * (sl & 3))));
                const uint2 hi = ld_tr16((const uint16_t *)(reg + WL::vaddr(r0 + 4, dt, 8 * (sl & 3))));
                const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
                oacc[dt] = mfma16(as_bf16x8(w), pb, oacc[dt]);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);   // the region is rewritten by the next step
            __builtin_amdgcn_wave_barrier();
        }
    }
    // merge of the wavefronts: max, rescaled sums and outputs per head
    float *ol = (float *)reg;   // [16][DV+4]
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int u = 0; u < 4; u++) ol[hd * (DV + 4) + 16 * dt + 4 * q + u] = oacc[dt][u];
    if (q == 0) {
        sm.wm[wave][hd] = m;
        sm.wl[wave][hd] = l;
    }
    lds_barrier();
    if (tid < 16) {
        float M = -INFINITY;
        for (int w = 0; w < kTailWaves; w++) M = fmaxf(M, sm.wm[w][tid]);
        float L = 0.f;
        for (int w = 0; w < kTailWaves; w++)
            if (sm.wm[w][tid] != -INFINITY) L += sm.wl[w][tid] * fast_exp2(sm.wm[w][tid] - M);
        sm.ms[tid] = M;
        sm.lsum[tid] = L;
    }
    lds_barrier();
    // ---- phase D: selected branch merged over the wavefronts, gated sum
    uint16_t *o = (uint16_t *)A.o + ((long)b * d.Hq + g * 16) * DV;
    for (int e = tid; e < 16 * DV; e += NT) {
        const int h = e / DV, c = e % DV;
        const float M = sm.ms[h], L = sm.lsum[h];
        float acc = 0.f;
        for (int w = 0; w < kTailWaves; w++) {
            const float mw = sm.wm[w][h];
            if (mw != -INFINITY) acc += ((const float *)sm.u.wave[w])[h * (DV + 4) + c] * fast_exp2(mw - M);
        }
        const float os = L > 0.f ? acc / L : 0.f;
        const float2 cw = sm.ocw[h][c];
        const float y = sm.gate[h][0] * cw.x + sm.gate[h][1] * os + sm.gate[h][2] * cw.y;
        __bf16 yb = (__bf16)y;
        o[e] = __builtin_bit_cast(uint16_t, yb);
    }
}

template <int DK, int DV>
hipError_t launch_decode_dims(const DecArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int pairs = d.B * d.Hkv;
    const int na = pairs * (A.cs + A.ws);
    hipLaunchKernelGGL((k_dec_stream<DK, DV>), dim3(na), dim3(kSThreads), 0, s, A);
    hipLaunchKernelGGL((k_dec_tail<DK, DV>), dim3(pairs), dim3(kTailThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace

bool decode_mfma_supported(const Dims &d)
{
    if (d.dtype != NSA_BF16 || d.G != 16) return false;
    if (!((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64))) return false;
    const int cs = (d.npad + kSplitKeys - 1) / kSplitKeys, ws = (d.w + kSplitKeys - 1) / kSplitKeys;
    const long pairs = (long)d.B * d.Hkv;
    return cs + ws <= 64 && d.npad / 4 <= 16384 && pairs * (cs + ws) <= 0x7fffffffL;
}

// Workspace of the matrix-core decode step, carved from `ws` when non-null.
size_t decode_mfma_layout(const Dims &d, void *ws, DecArgs *A)
{
    const long pairs = (long)d.B * d.Hkv;
    const int cs = (d.npad + kSplitKeys - 1) / kSplitKeys, wsplit = (d.w + kSplitKeys - 1) / kSplitKeys;
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
    const size_t o_idx = take(4 * pairs * d.n);
    if (A && ws) {
        char *w = (char *)ws;
        A->cs = cs;
        A->ws = wsplit;
        A->nbp = nbp;
        A->pm = (float *)(w + o_pm);
        A->pl = (float *)(w + o_pl);
        A->po = (float *)(w + o_po);
        A->bx = (float *)(w + o_bx);
        A->by = (float *)(w + o_by);
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
