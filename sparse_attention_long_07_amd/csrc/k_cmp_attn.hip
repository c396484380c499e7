// Stage S2 on the matrix cores: compressed attention and block importance.
//
// deepdaiv newsletter on DeepSeek's NSA (deepdaiv.stibee.com/p/82), token
// compression and token selection paragraphs: queries attend to one summary
// vector per compression block, and the block-importance scores that drive
// selection come from that attention.  The 16 query heads of a KV group share
// the group's compressed keys (ctol-kr.com article, "하드웨어 인식 설계":
// group-centric loading with a shared KV fetch), so a workgroup takes 16
// consecutive positions x 16 heads = 256 query rows of one KV group and
// streams the group's compressed keys through LDS once per pass for all of
// them.
//
// Orientation: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 -- 32 keys (M) by
// 32 query rows (N, two positions x 16 heads) -- so every lane owns the
// softmax state of one query row; eight waves cover the 16 positions, two
// waves per SIMD, so one wave's softmax arithmetic overlaps the other's
// matrix work.  K rows are stored in LDS permuted so that the 16 accumulators a lane holds are
// 16 consecutive keys; P^T then feeds O^T = V^T P^T directly as the B operand,
// with V^T transposed into LDS.
//
// Pass 1 computes each row's exact log-sum-exp.  Pass 2 recomputes the logits
// and forms exact probabilities, which give o_cmp and the group's block
// importance: block j takes keys 4j-1 .. 4j+3 with weights 1,2,2,2,1, so a
// lane first folds its 16 keys into four block partials plus the weight-1
// share of its last key in the next block, and the 16 heads are then summed
// through LDS.
//
// Pipeline: the next tile's K (and V) is loaded into registers while the
// current tile is computed, then written to the other LDS buffer; one
// barrier per tile.  Causal masking is applied only on a wave's last tiles.
#include "mfma_util.h"
#include "nsa_internal.h"
#include "window_phase.h"

namespace nsa {

namespace {

constexpr int kPos = 16;     // query positions per workgroup (2 per wave)
constexpr int kTile = 64;    // compressed keys per LDS tile
constexpr int kThreads = 512;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSgValu = 0x402;      // VALU, transcendental included
constexpr int kSgMfma = 0x008;
constexpr int kSgVmemRead = 0x020;
constexpr int kSgDsRead = 0x100;

template <int DK, int DV>
struct CmpLds {
    static constexpr int KS = DK + 8;      // bf16 per K row (padded against bank conflicts)
    static constexpr int VS = DV + 32;     // bf16 per V row: rows 64 B apart in the banks
    uint16_t k[2][kTile * KS];
    uint16_t v[2][kTile * VS];             // V key-major; V^T fragments come from transpose reads
};


// LDS row of key k (0..31) inside a 32-key M-tile.  MFMA output row i sits in
// lane half (i/4)%2, register 4*(i/8) + i%4; putting key 16*h + r in row
// 8*(r/4) + 4*h + r%4 makes register r of lane half h hold key 16*h + r.
__device__ __forceinline__ int krow(int k)
{
    int h = k >> 4, m = (k >> 2) & 3, u = k & 3;
    return 8 * m + 4 * h + u;
}

__device__ __forceinline__ int n_visible(int t) { return t >= 31 ? (t - 31) / 16 + 1 : 0; }

}  // namespace

// Workgroup -> ((b, g) pair, tile of positions).  When the (b, g) pairs
// divide the 8 XCDs, each XCD works on one pair only (its compressed K/V
// stays in that XCD's L2); tiles run heaviest (latest positions) first.
__device__ __forceinline__ bool cmp_map_wg(int id, int BG, int ntp, int &bg, int &ptile)
{
    int p;
    if (BG <= 8 && 8 % BG == 0) {
        const int per = 8 / BG, xcd = id & 7, s = id >> 3;
        bg = xcd / per;
        p = s * per + xcd % per;
    } else {
        bg = id % BG;
        p = id / BG;
    }
    if (p >= ntp) return false;
    ptile = ntp - 1 - p;
    return true;
}

// LDS of the kernel: with WIN the window phase reuses it once the
// compressed phase is done.
template <int DK, int DV, bool WIN>
struct CmpShared {
    CmpLds<DK, DV> c;
};
template <int DK, int DV>
struct CmpShared<DK, DV, true> {
    union {
        CmpLds<DK, DV> c;
        win::WinLds<DK, DV> w;
    };
};

// WIN (with WITH_V): the workgroup goes on to the window branch of its 16
// positions and writes o = g_cmp o_cmp + g_win o_win (window_phase.h) from
// the query fragments and o_cmp it holds; o_cmp is stored only where a.ocmp
// asks for it (the saved statistics' slot).
template <int DK, int DV, bool WITH_V, bool WIN = false>
__global__ __launch_bounds__(kThreads) void k_cmp_attn_mfma(RowArgs a, int ntp, int BG)
{
    static_assert(!WIN || WITH_V, "the window phase needs o_cmp");
    constexpr int KSTEPS = DK / 16;
    constexpr int DT = DV / 32;
    constexpr int CH = DK / 8;                                  // 16-byte chunks per K row
    constexpr int KTASKS = kTile * CH;
    constexpr int KLD = (KTASKS + kThreads - 1) / kThreads;    // K chunks per thread per tile
    constexpr int VTASKS = kTile * (DV / 8);                    // 16-byte V chunks per tile
    constexpr int VTK = (VTASKS + kThreads - 1) / kThreads;
    using L = CmpLds<DK, DV>;
    __shared__ CmpShared<DK, DV, WIN> sh;
    L &sm = sh.c;

    const Dims &d = a.d;
    int bg, ptile;
    if (!cmp_map_wg(blockIdx.x, BG, ntp, bg, ptile)) return;
    const int b = bg / d.Hkv, g = bg % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5;             // which 16 keys of each 32-key M-tile this lane holds
    const int row = lane & 31;           // query row inside the wave's N-tile
    const int head = row & 15;
    const int pos0 = ptile * kPos;
    const int pw = 2 * wave + (row >> 4);   // position inside the workgroup
    const int t = pos0 + pw;
    const bool live = t < d.T;
    const int nv = live ? n_visible(t) : 0;
    // wave-uniform tile counts: tiles below nfull need no causal mask (a wave
    // with a row past the sequence end masks every tile)
    const int tw0 = pos0 + 2 * wave;
    const int nfull = tw0 + 1 < d.T ? n_visible(tw0) / kTile : 0;
    const int ntw = tw0 < d.T ? (n_visible(min(tw0 + 1, d.T - 1)) + kTile - 1) / kTile : 0;
    const int ntiles = (n_visible(min(pos0 + kPos - 1, d.T - 1)) + kTile - 1) / kTile;
    // Tiles below nmain are unmasked for every wave and have a successor to
    // prefetch: their loop bodies are straight-line code, so the exponentials
    // of one 32-key M-tile can be scheduled under the matrix work of the next.
    const int nmain = pos0 + kPos - 1 < d.T ? min(n_visible(pos0) / kTile, ntiles - 1) : 0;
    const float sl2 = d.scale * kLog2e;

    const uint16_t *kc = (const uint16_t *)a.kc + (long)bg * d.npad * DK;
    const uint16_t *vc = (const uint16_t *)a.vc + (long)bg * d.npad * DV;

    u32x4 kreg[KLD], vreg[VTK];
    auto load_k = [&](int c) {
        const uint16_t *src = kc + (long)c * kTile * DK;
#pragma unroll
        for (int u = 0; u < KLD; u++) {
            const int task = tid + u * kThreads, key = task / CH, ch = task % CH;
            if (KTASKS % kThreads == 0 || task < KTASKS) kreg[u] = ld16(src + key * DK + ch * 8);
        }
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int u = 0; u < KLD; u++) {
            const int task = tid + u * kThreads, key = task / CH, ch = task % CH;
            const int r = (key & ~31) | krow(key & 31);
            if (KTASKS % kThreads == 0 || task < KTASKS) st16(&sm.k[buf][r * L::KS + ch * 8], kreg[u]);
        }
    };
    auto load_v = [&](int c) {
        const uint16_t *src = vc + (long)c * kTile * DV;
#pragma unroll
        for (int u = 0; u < VTK; u++) {
            const int task = tid + u * kThreads;
            if (VTASKS % kThreads == 0 || task < VTASKS) vreg[u] = ld16(src + (long)task * 8);
        }
    };
    auto store_vt = [&](int buf) {
        constexpr int CV = DV / 8;
#pragma unroll
        for (int u = 0; u < VTK; u++) {
            const int task = tid + u * kThreads, key = task / CV, ch = task % CV;
            if (VTASKS % kThreads == 0 || task < VTASKS) st16(&sm.v[buf][key * L::VS + ch * 8], vreg[u]);
        }
    };
    // the first K tile is in flight while the query loads land
    if (ntiles > 0) load_k(0);
    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qr = (const uint16_t *)a.q + (long)b * a.q_sb + (long)t * a.q_sr +
                             (long)(g * 16 + head) * DK + 8 * h;
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) qf[kk] = as_bf16x8(live ? ld16(qr + 16 * kk) : z);
    }
    // Let the query loads land before the tile loop: the compiler cannot tell
    // them from the next tile's prefetch, and would otherwise wait for every
    // outstanding load (the prefetch included) at the first matrix op of
    // each tile.
    wait_vmem_all();
    // V^T fragment of the PV product: dv rows 32*dt + (lane % 32), keys
    // kb .. kb+7 with kb = 32*mt + 16*(lane/32) + 8*s2 (the 8 keys this lane's
    // half of the 16-key step holds), read as two transposed 4-key pieces.
    const int vg = lane >> 4, vs = lane & 15;
    auto vt_frag = [&](int buf, int dt, int mt, int s2) {
        const uint16_t *p = &sm.v[buf][(32 * mt + 16 * (vg >> 1) + 8 * s2 + (vs >> 2)) * L::VS + 32 * dt +
                                       16 * (vg & 1) + 4 * (vs & 3)];
        const uint2 lo = ld_tr16(p), hi = ld_tr16(p + 4 * L::VS);
        const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
        return as_bf16x8(w);
    };
    auto logits = [&](int buf, int mt) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; r++) acc[r] = 0.f;
        const uint16_t *kr = &sm.k[buf][(32 * mt + row) * L::KS + 8 * h];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) acc = mfma32(as_bf16x8(ld16(kr + 16 * kk)), qf[kk], acc);
        return acc;
    };

    // ---- pass 1: log-sum-exp of every row (log2 domain)
    float m = -INFINITY, l = 0.f;
    // online update with the 16 logits one lane holds of a 32-key M-tile
    // (masked keys already -inf); a tile of -inf leaves m = -inf, l = 0 as is
    auto lse_update = [&](const f32x16 &acc) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, acc[r]);
        const float mn = fmaxf(m, mx * sl2);
        const float ms = mn == -INFINITY ? 0.f : mn;   // rows with nothing visible yet
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r++) sum += fast_exp2(__builtin_fmaf(acc[r], sl2, -ms));
        l = __builtin_fmaf(l, fast_exp2(m - ms), sum);
        m = mn;
    };
    // one tile; `masked` (wave-uniform) applies the causal limit
    auto pass1_tile = [&](int c, bool masked) {
        const int buf = c & 1;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            f32x16 acc = logits(buf, mt);
            const int kb = c * kTile + 32 * mt + 16 * h;
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; r++) acc[r] = kb + r < nv ? acc[r] : -INFINITY;
            }
            lse_update(acc);
        }
    };
    if (ntiles > 0) {
        store_k(0);
        lds_barrier();
    }
    // Main tiles run software-pipelined: the softmax of the previous tile's
    // second M-tile is issued under this tile's first 32x32 product chain and
    // the first M-tile's under the second chain.  The updates keep key order.
    int c1 = 0;
    {
        f32x16 pend;
#pragma unroll
        for (int r = 0; r < 16; r++) pend[r] = -INFINITY;
        for (; c1 < nmain; c1++) {
            load_k(c1 + 1);
            const f32x16 a0 = logits(c1 & 1, 0);
            lse_update(pend);
            const f32x16 a1 = logits(c1 & 1, 1);
            lse_update(a0);
            store_k((c1 + 1) & 1);
            lds_barrier();
            pend = a1;
            // issue order: the prefetch loads, three LDS fragment reads
            // ahead, then per product the product, the next read and a
            // share of the softmax
            __builtin_amdgcn_sched_group_barrier(kSgVmemRead, KLD, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 3, 0);
#pragma unroll
            for (int i = 0; i < 2 * KSTEPS; i++) {
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgValu, 6, 0);
            }
        }
        lse_update(pend);
    }
    for (int c = c1; c < ntiles; c++) {
        if (c + 1 < ntiles) load_k(c + 1);
        if (c < ntw) pass1_tile(c, c >= nfull);
        if (c + 1 < ntiles) store_k((c + 1) & 1);
        lds_barrier();
    }
    float lse2;
    {
        // the two lane halves combine their partial sums in the same order
        // (half 0 first), so both hold the same bits of the row's value
        const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
        const float m0 = h ? mo : m, l0 = h ? lo : l, m1 = h ? m : mo, l1 = h ? l : lo;
        const float M = fmaxf(m0, m1);
        lse2 = M == -INFINITY ? -INFINITY
                              : M + fast_log2(__builtin_fmaf(l0, fast_exp2(m0 - M), l1 * fast_exp2(m1 - M)));
    }

    // ---- pass 2: probabilities -> o_cmp and block importance
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] = 0.f;
    // probabilities of one lane's 16 keys of M-tile `mt`
    auto probs = [&](const f32x16 &acc, int kb, bool masked, float *p) {
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = fast_exp2(__builtin_fmaf(acc[r], sl2, -lse2));
        if (masked) {
#pragma unroll
            for (int r = 0; r < 16; r++) p[r] = kb + r < nv ? p[r] : 0.f;
        }
    };
    auto pv = [&](int buf, int mt, const float *p) {
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
            const bf16x8 pb = pack8(&p[8 * s2]);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) oacc[dt] = mfma32(vt_frag(buf, dt, mt, s2), pb, oacc[dt]);
        }
    };
    auto pv_packed = [&](int buf, int mt, const bf16x8 *pb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++) oacc[dt] = mfma32(vt_frag(buf, dt, mt, s2), pb[s2], oacc[dt]);
    };
    // Block importance of M-tile `mt` of tile c.  The 16 lanes of a DPP row
    // hold the 16 heads of one position for the same 16 keys (group
    // grp = 2*mt + h of the tile), so the head sum is a row reduction.  Block
    // 16c + 4*grp + u takes keys 4u-1 .. 4u+3 of the group with weights
    // 1,2,2,2,1; key -1 is the previous group's last key, which lives in the
    // other lane half (h = 1) or, for h = 0, in `carry` from the previous
    // M-tile.  Lanes (l % 16) < 4 store the group's four blocks.
    float carry = 0.f;
    float *srow = a.scores + ((long)bg * a.R + t) * d.nb;
    const int tb = t / 64;   // last causal block of this row
    // The stores go through a buffer resource over the workgroup's 16 score
    // rows: a lane with nothing to store gets an offset past the range, which
    // the hardware drops, so no branch splits the scheduled regions.
    const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
        a.scores + ((long)bg * a.R + pos0) * d.nb, 0, kPos * d.nb * 4, 0x00020000);
    constexpr int kDropOffset = 0x7fffffff;
    auto importance = [&](int c, int mt, const float *p) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const float *q4 = &p[4 * u];
            v[u] = __builtin_fmaf(2.f, q4[0] + q4[1] + q4[2], q4[3]);
            if (u) v[u] += q4[-1];
            v[u] = row_sum16(v[u]);
        }
        const float last = row_sum16(p[15]);
        const float other = __shfl_xor(last, 32, 64);
        v[0] += h ? other : carry;
        carry = other;   // kept by the h = 0 lanes: the h = 1 group's last key
        const int u = lane & 15;
        const int j = 16 * c + 4 * (2 * mt + h) + u;
        // the empty asm keeps the sums materialised, so the selects below
        // stay v_cndmask instead of becoming branches
#pragma unroll
        for (int q = 0; q < 4; q++) asm volatile("" : "+v"(v[q]));
        const float lo = (u & 1) ? v[1] : v[0], hi = (u & 1) ? v[3] : v[2];
        const float val = (u & 2) ? hi : lo;
        const int off = u < 4 && live && j <= tb ? (pw * d.nb + j) * 4 : kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), srsrc, off, 0, 0);
    };
    auto pass2_tile = [&](int c, bool masked) {
        const int buf = c & 1;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            const f32x16 acc = logits(buf, mt);
            float p[16];
            probs(acc, c * kTile + 32 * mt + 16 * h, masked, p);
            if (WITH_V) pv(buf, mt, p);
            importance(c, mt, p);
        }
    };
    if (ntiles > 0) {
        load_k(0);
        if (WITH_V) load_v(0);
        store_k(0);
        if (WITH_V) store_vt(0);
        lds_barrier();
    }
    int c2 = 0;
    for (; c2 < nmain; c2++) {
        load_k(c2 + 1);
        if (WITH_V) load_v(c2 + 1);
        // Four scheduling regions per tile: the first logit chain; the second
        // chain under the first M-tile's exponentials and importance sums;
        // the first PV chain under the second M-tile's; the second PV chain.
        // Only the packed bf16 probabilities stay live into the PV chains.
        const int buf = c2 & 1;
        const f32x16 s0 = logits(buf, 0);
        __builtin_amdgcn_sched_barrier(0);
        const f32x16 s1 = logits(buf, 1);
        bf16x8 pb0[2], pb1[2];
        {
            float p0[16];
            probs(s0, 0, false, p0);
            pb0[0] = pack8(&p0[0]);
            pb0[1] = pack8(&p0[8]);
            importance(c2, 0, p0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 3, 0);
#pragma unroll
        for (int i = 0; i < KSTEPS; i++) {
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the next tile's buffer is free all iteration: storing the prefetch
        // here ends the staging registers' live range before the PV chains
        store_k((c2 + 1) & 1);
        if (WITH_V) store_vt((c2 + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        if (WITH_V) pv_packed(buf, 0, pb0);
        {
            float p1[16];
            probs(s1, 0, false, p1);
            pb1[0] = pack8(&p1[0]);
            pb1[1] = pack8(&p1[8]);
            importance(c2, 1, p1);
        }
        if constexpr (WITH_V) {
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * DT; i++) {
                __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
                __builtin_amdgcn_sched_group_barrier(kSgValu, 7, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            pv_packed(buf, 1, pb1);
            __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();
    }
    for (int c = c2; c < ntiles; c++) {
        if (c + 1 < ntiles) {
            load_k(c + 1);
            if (WITH_V) load_v(c + 1);
        }
        if (c < ntw) pass2_tile(c, c >= nfull);
        if (c + 1 < ntiles) {
            store_k((c + 1) & 1);
            if (WITH_V) store_vt((c + 1) & 1);
        }
        lds_barrier();
    }
    // The last key of the wave's final tile also reaches block 16*ntw, the
    // only later block a row of this wave can see (its first key is not
    // visible to it).
    if (h == 0 && (lane & 15) == 0 && live && 16 * ntw <= tb) srow[16 * ntw] = carry;

    if constexpr (WIN) {
        uint2 ocw[DT][4];
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                ocw[dt][q4].x = pack_bf16x2(oacc[dt][4 * q4], oacc[dt][4 * q4 + 1]);
                ocw[dt][q4].y = pack_bf16x2(oacc[dt][4 * q4 + 2], oacc[dt][4 * q4 + 3]);
            }
        if (live) {
            if (a.lse && h == 0) a.lse[((long)b * a.R + t) * d.Hq + g * 16 + head] = lse2 * kLn2;
            if (a.ocmp) {
                uint16_t *orow = (uint16_t *)a.ocmp + (((long)b * a.R + t) * d.Hq + g * 16 + head) * DV;
#pragma unroll
                for (int dt = 0; dt < DT; dt++)
#pragma unroll
                    for (int q4 = 0; q4 < 4; q4++) *(uint2 *)(orow + 32 * dt + 8 * q4 + 4 * h) = ocw[dt][q4];
            }
        }
        // every wave's last reads of the compressed tiles passed the loop's
        // final barrier, so the window phase may overwrite the LDS
        win::window_phase<DK, DV, true>(a, sh.w, bg, ptile, qf, ocw);
    } else if (WITH_V && live) {
        // the branch's log-sum-exp for the backward, when asked for
        if (a.lse && h == 0) a.lse[((long)b * a.R + t) * d.Hq + g * 16 + head] = lse2 * kLn2;
        uint16_t *orow = (uint16_t *)a.ocmp + (((long)b * a.R + t) * d.Hq + g * 16 + head) * DV;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const int dv = 32 * dt + 8 * q4 + 4 * h;
                uint2 w;
                w.x = pack_bf16x2(oacc[dt][4 * q4], oacc[dt][4 * q4 + 1]);
                w.y = pack_bf16x2(oacc[dt][4 * q4 + 2], oacc[dt][4 * q4 + 3]);
                *(uint2 *)(orow + dv) = w;
            }
    }
}

bool cmp_attn_mfma_supported(const Dims &d)
{
    return d.dtype == NSA_BF16 && d.G == 16 &&
           ((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64));
}

template <int DK, int DV>
static hipError_t launch_dims(const RowArgs &a, bool with_v, hipStream_t s)
{
    const Dims &d = a.d;
    const int ntp = (a.R + kPos - 1) / kPos;
    const int BG = d.B * d.Hkv;
    long nwg;
    if (BG <= 8 && 8 % BG == 0) nwg = 8L * ((ntp + 8 / BG - 1) / (8 / BG));
    else nwg = (long)BG * ntp;
    if (with_v) hipLaunchKernelGGL((k_cmp_attn_mfma<DK, DV, true>), dim3((unsigned)nwg), dim3(kThreads), 0, s, a, ntp, BG);
    else hipLaunchKernelGGL((k_cmp_attn_mfma<DK, DV, false>), dim3((unsigned)nwg), dim3(kThreads), 0, s, a, ntp, BG);
    return hipGetLastError();
}

// S2 with the window branch fused (the k_window_mfma work of the same 16
// positions, on the same workgroup)
template <int DK, int DV>
static hipError_t launch_win_dims(const RowArgs &a, hipStream_t s)
{
    static_assert(kPos == win::kPos && kThreads == win::kThreads, "one workgroup shape for both phases");
    const Dims &d = a.d;
    const int ntp = (a.R + kPos - 1) / kPos;
    const int BG = d.B * d.Hkv;
    long nwg;
    if (BG <= 8 && 8 % BG == 0) nwg = 8L * ((ntp + 8 / BG - 1) / (8 / BG));
    else nwg = (long)BG * ntp;
    hipLaunchKernelGGL((k_cmp_attn_mfma<DK, DV, true, true>), dim3((unsigned)nwg), dim3(kThreads), 0, s, a, ntp, BG);
    return hipGetLastError();
}

hipError_t launch_cmp_win_mfma(const RowArgs &a, hipStream_t s)
{
    const Dims &d = a.d;
    if (d.dk == 192 && d.dv == 128) return launch_win_dims<192, 128>(a, s);
    if (d.dk == 128 && d.dv == 128) return launch_win_dims<128, 128>(a, s);
    if (d.dk == 64 && d.dv == 64) return launch_win_dims<64, 64>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_cmp_attn_mfma(const RowArgs &a, bool with_v, hipStream_t s)
{
    const Dims &d = a.d;
    if (d.dk == 192 && d.dv == 128) return launch_dims<192, 128>(a, with_v, s);
    if (d.dk == 128 && d.dv == 128) return launch_dims<128, 128>(a, with_v, s);
    if (d.dk == 64 && d.dv == 64) return launch_dims<64, 64>(a, with_v, s);
    return hipErrorInvalidValue;
}

}  // namespace nsa
