// The window branch and the gated sum of the compressed and window branches,
// one workgroup's share: 16 positions x 16 heads of one KV head.  Shared by
// the window kernel of stage S4 and by the compressed-attention kernel, which
// can run it right after its own phase on the same workgroup (the query
// fragments and o_cmp are then already in registers).
//
// deepdaiv newsletter on DeepSeek's NSA (deepdaiv.stibee.com/p/82), sliding
// window paragraph: a fixed window of the most recent tokens is attended
// densely; its output enters the gated sum with the compressed and selected
// branches.
#pragma once

#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {
namespace win {

constexpr int kTile = 64;
constexpr int kPos = 16;        // query positions per workgroup
constexpr int kThreads = 512;   // 8 waves, two positions each

// LDS row of key k (0..31) inside a 32-key M-tile: register r of lane half h
// of the 32x32 product then holds key 16 h + r.
__device__ __forceinline__ int krow(int k)
{
    int h = k >> 4, m = (k >> 2) & 3, u = k & 3;
    return 8 * m + 4 * h + u;
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

template <int DK, int DV>
struct WinLds {
    static constexpr int KS = DK + 8;
    static constexpr int VS = kTile + 8;
    static constexpr int GS = 3 * DK + 8;   // bf16 per head's three gate rows (padded)
    uint16_t k[2][kTile * KS];
    uint16_t vt[2][DV * VS];
    uint16_t wg[16 * GS];                   // gate weights of the group's 16 heads
};

// Window branch + compressed term.  16 positions x 16 heads per workgroup,
// 8 waves of 32 rows (two waves per SIMD); the window's 64-key tiles are
// loaded into registers one tile ahead and written to the other LDS buffer,
// one barrier per tile.  Only a wave's edge tiles are masked.  The running
// maximum is raised only when a tile's maximum exceeds it by more than 2^8
// (one wave-wide decision), so most tiles skip rescaling the accumulators;
// p then stays below 2^8, which fp32 sums and bf16 operands hold exactly as
// well as values below 1.
//
// QIN: qf holds the query fragments of this lane's row and ocw its o_cmp
// (bf16 pairs at columns 32 dt + 8 q4 + 4 h .. +3, as the compressed phase
// stores them), so neither is read from memory; otherwise qf is loaded here
// and o_cmp read from a.ocmp.
template <int DK, int DV, bool QIN>
__device__ __forceinline__ void window_phase(const RowArgs &a, WinLds<DK, DV> &sm, int bg, int ptile,
                                             bf16x8 (&qf)[DK / 16], const uint2 (&ocw)[DV / 32][4])
{
    constexpr int KSTEPS = DK / 16;
    constexpr int DT = DV / 32;
    constexpr int CH = DK / 8;
    constexpr int KTASKS = kTile * CH;
    constexpr int KLD = (KTASKS + kThreads - 1) / kThreads;
    constexpr int VTASKS = 32 * (DV / 8);
    constexpr int VTK = (VTASKS + kThreads - 1) / kThreads;
    constexpr float kLazy = 8.f;   // log2 headroom before the running max is raised
    using L = WinLds<DK, DV>;

    const Dims &d = a.d;
    const int b = bg / d.Hkv, g = bg % d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, row = lane & 31, head = row & 15;
    const int pos0 = ptile * kPos;
    const int t = pos0 + 2 * wave + (row >> 4);
    const bool live = t < d.T;
    const int lo = max(0, t - d.w + 1);
    const int tlast = min(pos0 + kPos - 1, d.T - 1);
    const int c_first = max(0, pos0 - d.w + 1) / kTile, c_last = tlast / kTile;
    // this wave's two positions: keys it needs and tiles it sees unmasked
    const int tw0 = pos0 + 2 * wave, tw1 = tw0 + 1;
    const bool wlive = tw0 < d.T;
    const int wk_lo = max(0, tw0 - d.w + 1), wk_hi = min(tw1, d.T - 1);
    const int full_lo = max(0, tw1 - d.w + 1);      // unmasked: full_lo <= 64c and 64c+63 <= tw0
    const bool both = tw1 < d.T;
    const float sl2 = d.scale * kLog2e;

    const uint16_t *kg = (const uint16_t *)a.k + (long)bg * d.T * DK;
    const uint16_t *vg = (const uint16_t *)a.v + (long)bg * d.T * DV;
    u32x4 kreg[KLD], vreg[VTK][2];
    auto load_tile = [&](int c) {
#pragma unroll
        for (int u = 0; u < KLD; u++) {
            const int task = tid + u * kThreads, key = task / CH, ch = task % CH;
            const u32x4 z = {0, 0, 0, 0};
            kreg[u] = z;
            if ((KTASKS % kThreads == 0 || task < KTASKS) && c * kTile + key < d.T)
                kreg[u] = ld16(kg + (long)(c * kTile + key) * DK + ch * 8);
        }
#pragma unroll
        for (int u = 0; u < VTK; u++) {
            const int task = tid + u * kThreads, kp = task & 31, dc = task >> 5;
            const int k0 = c * kTile + 2 * kp;
            const u32x4 z = {0, 0, 0, 0};
            vreg[u][0] = z;
            vreg[u][1] = z;
            if (VTASKS % kThreads == 0 || task < VTASKS) {
                if (k0 < d.T) vreg[u][0] = ld16(vg + (long)k0 * DV + dc * 8);
                if (k0 + 1 < d.T) vreg[u][1] = ld16(vg + (long)(k0 + 1) * DV + dc * 8);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < KLD; u++) {
            const int task = tid + u * kThreads, key = task / CH, ch = task % CH;
            const int r = (key & ~31) | krow(key & 31);
            if (KTASKS % kThreads == 0 || task < KTASKS) st16(&sm.k[buf][r * L::KS + ch * 8], kreg[u]);
        }
#pragma unroll
        for (int u = 0; u < VTK; u++) {
            const int task = tid + u * kThreads, kp = task & 31, dc = task >> 5;
            if (VTASKS % kThreads == 0 || task < VTASKS) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const uint32_t w = __builtin_amdgcn_perm(vreg[u][1][e >> 1], vreg[u][0][e >> 1],
                                                             (e & 1) ? 0x07060302u : 0x05040100u);
                    *(uint32_t *)&sm.vt[buf][(dc * 8 + e) * L::VS + 2 * kp] = w;
                }
            }
        }
    };

    // the first K/V tile is in flight while the query and gate loads land
    load_tile(c_first);

    if constexpr (!QIN) {
        const uint16_t *qr = (const uint16_t *)a.q + (long)b * a.q_sb + (long)t * a.q_sr +
                             (long)(g * 16 + head) * DK + 8 * h;
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) qf[kk] = as_bf16x8(live ? ld16(qr + 16 * kk) : z);
    }
    // The gate rows of the group's 16 heads (16 x 3 x DK bf16) are staged in
    // LDS once per workgroup: every lane needs its head's three rows and 16
    // lanes share each head, so per-lane loads would fetch each row 16 times.
    constexpr int GCH = 16 * 3 * DK / 8;          // 16-byte chunks
    constexpr int GLD = (GCH + kThreads - 1) / kThreads;
    u32x4 greg[GLD];
    {
        const uint16_t *src = (const uint16_t *)a.wg + (long)g * 16 * 3 * DK;
#pragma unroll
        for (int u = 0; u < GLD; u++) {
            const int task = tid + u * kThreads;
            if (GCH % kThreads == 0 || task < GCH) greg[u] = ld16(src + (long)task * 8);
        }
    }
    float gbias[3];
#pragma unroll
    for (int c = 0; c < 3; c++)
        gbias[c] = __uint_as_float((uint32_t)((const uint16_t *)a.bg)[(g * 16 + head) * 3 + c] << 16);

    // let the query and gate loads land before the tile loop (see the
    // compressed-attention kernel: otherwise every tile waits for its prefetch)
    wait_vmem_all();
#pragma unroll
    for (int u = 0; u < GLD; u++) {
        const int task = tid + u * kThreads;
        const int hh = task / (3 * DK / 8), off = task % (3 * DK / 8);
        if (GCH % kThreads == 0 || task < GCH) st16(&sm.wg[hh * L::GS + off * 8], greg[u]);
    }
    float m = -INFINITY, l = 0.f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] = 0.f;

    auto tile = [&](int c, bool masked) {
        const int buf = c & 1;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; r++) acc[r] = 0.f;
            const uint16_t *kr = &sm.k[buf][(32 * mt + row) * L::KS + 8 * h];
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++) acc = mfma32(as_bf16x8(ld16(kr + 16 * kk)), qf[kk], acc);
            const int kb = c * kTile + 32 * mt + 16 * h;
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = kb + r;
                    acc[r] = (live && key >= lo && key <= t) ? acc[r] : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; r++) mx = fmaxf(mx, acc[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
            if (__any(mx > m + kLazy)) {
                const float mn = fmaxf(m, mx);
                const float al = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
                l *= al;
#pragma unroll
                for (int dt = 0; dt < DT; dt++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[dt][r] *= al;
                m = mn;
            }
            const float ms = m == -INFINITY ? 0.f : m;   // rows that have seen no key yet
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                p[r] = fast_exp2(__builtin_fmaf(acc[r], sl2, -ms));
                l += p[r];
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; s2++) {
                const bf16x8 pb = pack8(&p[8 * s2]);
#pragma unroll
                for (int dt = 0; dt < DT; dt++) {
                    const uint16_t *vr = &sm.vt[buf][(32 * dt + row) * L::VS + 32 * mt + 16 * h + 8 * s2];
                    oacc[dt] = mfma32(as_bf16x8(ld16(vr)), pb, oacc[dt]);
                }
            }
        }
    };

    store_tile(c_first & 1);
    lds_barrier();
    // gates of this row from the staged rows: each lane half holds half of
    // the dimensions
    float gate[3];
    {
        const uint16_t *wr = &sm.wg[head * L::GS + 8 * h];
#pragma unroll
        for (int c = 0; c < 3; c++) {
            float z = 0.f;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++)
                z = dot8_bf16(ld16(wr + c * DK + 16 * kk), __builtin_bit_cast(u32x4, qf[kk]), z);
            z += __shfl_xor(z, 32, 64);
            gate[c] = live ? sigmoid(z + gbias[c]) : 0.f;
        }
    }
    for (int c = c_first; c <= c_last; c++) {
        if (c < c_last) load_tile(c + 1);
        const int k0 = c * kTile;
        if (wlive && k0 + kTile - 1 >= wk_lo && k0 <= wk_hi)
            tile(c, !(both && k0 >= full_lo && k0 + kTile - 1 <= tw0));
        if (c < c_last) store_tile((c + 1) & 1);
        lds_barrier();
    }
    const float ltot = l + __shfl_xor(l, 32, 64);
    if (!live) return;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    const long rh = ((long)b * a.R + t) * d.Hq + g * 16 + head;
    const long ooff = rh * DV;
    const uint16_t *oc = QIN ? nullptr : (const uint16_t *)a.ocmp + ooff;
    uint16_t *orow = (uint16_t *)a.o + ooff;
    // saved statistics for the backward (slot 2: the window branch)
    const long slot = (long)d.B * a.R * d.Hq;
    uint16_t *osv = a.osave ? (uint16_t *)a.osave + 2 * slot * DV + ooff : nullptr;
    if (a.lse && h == 0) a.lse[2 * slot + rh] = ltot > 0.f ? (m + fast_log2(ltot)) * kLn2 : -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const int dv = 32 * dt + 8 * q4 + 4 * h;
            const uint2 cv = QIN ? ocw[dt][q4] : *(const uint2 *)(oc + dv);
            float y[4], ow[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t word = e < 2 ? cv.x : cv.y;
                const float ocv = __uint_as_float(e & 1 ? word & 0xffff0000u : word << 16);
                ow[e] = oacc[dt][4 * q4 + e] * inv;
                y[e] = gate[0] * ocv + gate[2] * ow[e];
            }
            uint2 w;
            w.x = pack_bf16x2(y[0], y[1]);
            w.y = pack_bf16x2(y[2], y[3]);
            *(uint2 *)(orow + dv) = w;
            if (osv) *(uint2 *)(osv + dv) = uint2{pack_bf16x2(ow[0], ow[1]), pack_bf16x2(ow[2], ow[3])};
        }
}

}  // namespace win
}  // namespace nsa
