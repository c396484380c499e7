// Stage S4 on the matrix cores: sliding-window attention, selected-block
// attention and the gated sum, for bf16 storage with 16 query heads per KV
// head.
//
// deepdaiv newsletter on DeepSeek's NSA (deepdaiv.stibee.com/p/82): the
// selected blocks are attended at full resolution and a fixed window of the
// most recent tokens is attended densely; allinfo.ai.kr's DSA explainer
// ("쉽게 이해하기"): the selected branch normalises over the selected set only.
//
// Two kernels, each shaped by its own bound:
//  * k_window_mfma -- the window keys of neighbouring positions coincide, so a
//    workgroup takes 16 positions x 16 heads (256 query rows) of one KV head
//    and streams the window's 64-key tiles through LDS once for all of them
//    (v_mfma_f32_32x32x16_bf16, S^T = K Q^T as in the compressed stage).  It
//    writes o = g_cmp * o_cmp + g_win * o_win.
//  * k_selected_mfma -- selected blocks differ from position to position, so
//    one wavefront takes one position: its 16 heads are the N dimension of
//    v_mfma_f32_16x16x32_bf16 (the GQA group shares every key fetch), and each
//    selected 64-token block is read once, straight into registers.  This
//    part is bound by how fast blocks can be gathered, not by the MFMA.  It
//    adds g_slc * o_slc to o.
// K and V enter the selected kernel packed per 64-token block in the order the
// MFMA operands are held by the lanes (k_pack_blocks): adjacent lanes read
// adjacent 16 bytes, so each operand fetch is one coalesced 1 KB load instead
// of sixteen scattered row pieces.
#include "mfma_util.h"
#include "nsa_internal.h"
#include "window_phase.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

// Fragment-major packing of K and V per 64-token block, so that every operand
// fetch of the selected-block kernel is one coalesced 1 KB wavefront load.
// Half block s (keys 32s .. 32s+31 of block j), lane l = 16q + hd:
//   Kp[bg][j][s][X][kk][l] = K[64j + 32s + r(hd) + 4X][32kk + 8q .. +8]
//      with r(i) = 8*(i/4) + i%4, X = 0/1 the two 16-key MFMA row tiles
//   Vp[bg][j][s][dt][l]    = V[64j + 32s + 8q .. +8][16dt + hd]   (V^T)
// Tokens past T are 0.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_pack_blocks(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                          uint16_t *__restrict__ kp, uint16_t *__restrict__ vp, int T,
                                                          int NB)
{
    constexpr int KS = DK / 32, DT = DV / 16;
    __shared__ uint16_t kt[kTile][DK + 8];
    __shared__ uint16_t vtile[kTile][DV + 2];
    const int j = blockIdx.x, bg = blockIdx.y, tid = threadIdx.x;
    const uint16_t *ks = k + ((long)bg * T + (long)kTile * j) * DK;
    const uint16_t *vs = v + ((long)bg * T + (long)kTile * j) * DV;
    for (int e = tid; e < kTile * DK / 8; e += kThreads) {
        const int key = e / (DK / 8), ch = e % (DK / 8);
        u32x4 x = {0, 0, 0, 0};
        if (kTile * j + key < T) x = ld16(ks + (long)key * DK + ch * 8);
        st16(&kt[key][ch * 8], x);
    }
    for (int e = tid; e < kTile * DV / 8; e += kThreads) {
        const int key = e / (DV / 8), ch = e % (DV / 8);
        u32x4 x = {0, 0, 0, 0};
        if (kTile * j + key < T) x = ld16(vs + (long)key * DV + ch * 8);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            vtile[key][ch * 8 + 2 * q] = (uint16_t)(x[q] & 0xffffu);
            vtile[key][ch * 8 + 2 * q + 1] = (uint16_t)(x[q] >> 16);
        }
    }
    __syncthreads();
    uint16_t *kd = kp + ((long)bg * NB + j) * kTile * DK;
    for (int e = tid; e < 2 * 2 * KS * 64; e += kThreads) {
        const int l = e & 63, kk = (e >> 6) % KS, X = (e / (64 * KS)) & 1, s = e / (128 * KS);
        const int q = l >> 4, hd = l & 15;
        const int key = 32 * s + 8 * (hd >> 2) + (hd & 3) + 4 * X;
        st16(kd + (long)e * 8, ld16(&kt[key][32 * kk + 8 * q]));
    }
    uint16_t *vd = vp + ((long)bg * NB + j) * kTile * DV;
    for (int e = tid; e < 2 * DT * 64; e += kThreads) {
        const int l = e & 63, dt = (e >> 6) % DT, s = e / (64 * DT);
        const int q = l >> 4, hd = l & 15;
        const int key0 = 32 * s + 8 * q, dv = 16 * dt + hd;
        u32x4 x;
#pragma unroll
        for (int u = 0; u < 4; u++)
            x[u] = (uint32_t)vtile[key0 + 2 * u][dv] | ((uint32_t)vtile[key0 + 2 * u + 1][dv] << 16);
        st16(vd + (long)e * 8, x);
    }
}

// ---------------------------------------------------------------------------
// Window branch + compressed term (window_phase.h).  Workgroups of one (b, g)
// pair take consecutive position tiles on the same XCD, so the overlapping
// window tiles are served from that XCD's L2.
template <int DK, int DV>
__global__ __launch_bounds__(win::kThreads) void k_window_mfma(RowArgs a, int ntp)
{
    __shared__ win::WinLds<DK, DV> sm;
    const Dims &d = a.d;
    const int BG = d.B * d.Hkv;
    const long total = (long)BG * ntp;
    const long per_xcd = (total + 7) / 8;
    const long vid = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (vid >= total) return;
    bf16x8 qf[DK / 16];
    uint2 ocw[DV / 32][4];
    win::window_phase<DK, DV, false>(a, sm, (int)(vid / ntp), (int)(vid % ntp), qf, ocw);
}

// ---------------------------------------------------------------------------
// Selected branch.  One wavefront per (b, g, position); lane l holds head
// l%16 and, of every 32-key half block, keys 8*(l/16) .. 8*(l/16)+7: the two
// 16-key MFMA row tiles of a half block take keys 8*(i/4) + i%4 (tile A) and
// 8*(i/4) + 4 + i%4 (tile B) in row i, so their outputs are exactly the
// B operand of O^T = V^T P^T.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_selected_mfma(RowArgs a, const uint16_t *__restrict__ kpk,
                                                            const uint16_t *__restrict__ vpk, int ntp)
{
    constexpr int KS = DK / 32;     // 16x16x32 steps over the head dim
    constexpr int DT = DV / 16;     // 16-wide dv tiles
    const Dims &d = a.d;
    const int BG = d.B * d.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // workgroup -> (b, g, 4 positions), heaviest (latest) positions first
    const long total = (long)BG * ntp;
    const long per_xcd = (total + 7) / 8;
    const long vid = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (vid >= total) return;
    const int bg = (int)(vid / ntp), ptile = ntp - 1 - (int)(vid % ntp);
    const int t = ptile * 4 + wave;
    if (t >= d.T) return;
    const int b = bg / d.Hkv, g = bg % d.Hkv;
    const int q = lane >> 4, hd = lane & 15;
    const int jcur = t / kTile;
    const float sl2 = d.scale * kLog2e;

    // the row's block list first: the first gathers wait on it, and its load
    // then overlaps the query and gate loads
    int jb = -1;
    if (lane < d.n) jb = a.idx[((long)bg * a.R + t) * d.n + lane];
    const uint16_t *qr = (const uint16_t *)a.q + (long)b * a.q_sb + (long)t * a.q_sr + (long)(g * 16 + hd) * DK + 8 * q;
    bf16x8 qf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; kk++) qf[kk] = as_bf16x8(ld16(qr + 32 * kk));
    float gsl;
    {
        const uint16_t *wr = (const uint16_t *)a.wg + ((long)(g * 16 + hd) * 3 + 1) * DK + 8 * q;
        float z = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            const u32x4 wv = ld16(wr + 32 * kk);
            const u32x4 qv = ld16(qr + 32 * kk);
            z = dot8_bf16(wv, qv, z);
        }
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        const uint16_t *bp = (const uint16_t *)a.bg + (long)(g * 16 + hd) * 3 + 1;
        gsl = sigmoid(z + __uint_as_float((uint32_t)*bp << 16));
    }

    // the row's blocks: valid (0..jcur) and first occurrence only, compacted
    // into this wavefront's slot list
    __shared__ int blist[4][16];
    bool ok = jb >= 0 && jb <= jcur;
    for (int u = 0; u < 16; u++) {
        const int other = __shfl(jb, u, 64);
        if (u < lane && other == jb) ok = false;
    }
    const uint64_t valid = __ballot(ok);
    if (ok) blist[wave][__popcll(valid & __lanemask_lt())] = jb;
    // other lanes of this wavefront read the list: the stores are in LDS first
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    const int nitems = 2 * __popcll(valid);   // half blocks of 32 keys

    const uint16_t *kpg = kpk + (long)bg * d.nb * kTile * DK;
    const uint16_t *vpg = vpk + (long)bg * d.nb * kTile * DV;
    float m = -INFINITY, l = 0.f;
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Half block `it` = keys 32*(it%2) .. +31 of block blist[it/2].  Loads of
    // the next half block are issued before the current one is computed.
    struct Stage {
        bf16x8 fa[KS], fb[KS], fv[DT];
    };
    auto load_item = [&](int it, Stage &st) {
        const int j = blist[wave][it >> 1], s = it & 1;
        const uint16_t *kb = kpg + ((long)j * 2 + s) * 32 * DK + lane * 8;
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            st.fa[kk] = as_bf16x8(ld16(kb + kk * 512));
            st.fb[kk] = as_bf16x8(ld16(kb + (KS + kk) * 512));
        }
        const uint16_t *vb = vpg + ((long)j * 2 + s) * 32 * DV + lane * 8;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) st.fv[dt] = as_bf16x8(ld16(vb + dt * 512));
    };
    auto compute_item = [&](int it, const Stage &st) {
        const int key0 = blist[wave][it >> 1] * kTile + 32 * (it & 1);
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; kk++) {
            accA = mfma16(st.fa[kk], qf[kk], accA);
            accB = mfma16(st.fb[kk], qf[kk], accB);
        }
        float sv[8], mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int ka = key0 + 8 * q + u;
            sv[u] = ka <= t ? accA[u] * sl2 : -INFINITY;
            sv[4 + u] = ka + 4 <= t ? accB[u] * sl2 : -INFINITY;
            mx = fmaxf(mx, fmaxf(sv[u], sv[4 + u]));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx);
        if (mn == -INFINITY) return;   // every key of this half block is past t: uniform over the wave
        const float al = fast_exp2(m - mn);
        float p[8], sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            p[e] = fast_exp2(sv[e] - mn);
            sum += p[e];
        }
        l = l * al + sum;
        m = mn;
        const bf16x8 pb = pack8(p);
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            oacc[dt] *= al;
            oacc[dt] = mfma16(st.fv[dt], pb, oacc[dt]);
        }
    };
    Stage sa, sb;
    if (nitems > 0) load_item(0, sa);
    for (int it = 0; it < nitems; it += 2) {
        if (it + 1 < nitems) load_item(it + 1, sb);
        compute_item(it, sa);
        if (it + 1 >= nitems) break;
        if (it + 2 < nitems) load_item(it + 2, sa);
        compute_item(it + 1, sb);
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float w = l > 0.f ? gsl / l : 0.f;
    const long rh = ((long)b * a.R + t) * d.Hq + g * 16 + hd;
    uint16_t *orow = (uint16_t *)a.o + rh * DV + 4 * q;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
        uint2 cur = *(uint2 *)(orow + 16 * dt);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t word = e < 2 ? cur.x : cur.y;
            y[e] = __uint_as_float(e & 1 ? word & 0xffff0000u : word << 16) + w * oacc[dt][e];
        }
        cur.x = pack_bf16x2(y[0], y[1]);
        cur.y = pack_bf16x2(y[2], y[3]);
        *(uint2 *)(orow + 16 * dt) = cur;
    }
    // saved statistics for the backward (slot 1: the selected branch)
    if (a.lse) {
        const long slot = (long)d.B * a.R * d.Hq;
        if (q == 0) a.lse[slot + rh] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *osv = (uint16_t *)a.osave + (slot + rh) * DV + 4 * q;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
            *(uint2 *)(osv + 16 * dt) = uint2{pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                                              pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv)};
    }
}

template <int DK, int DV>
hipError_t launch_sparse_dims(const RowArgs &a, void *vt_ws, hipStream_t s)
{
    const Dims &d = a.d;
    const int BG = d.B * d.Hkv;
    uint16_t *kpk = (uint16_t *)vt_ws;
    uint16_t *vpk = kpk + (size_t)BG * d.nb * kTile * DK;
    if (a.part == 0 || a.part == 1) {
        const int ntp = (a.R + win::kPos - 1) / win::kPos;
        long nwg = (long)BG * ntp;
        nwg = (nwg + 7) / 8 * 8;
        hipLaunchKernelGGL((k_window_mfma<DK, DV>), dim3((unsigned)nwg), dim3(win::kThreads), 0, s, a, ntp);
    }
    if (a.part == 0 || a.part == 3)
        hipLaunchKernelGGL((k_pack_blocks<DK, DV>), dim3(d.nb, BG), dim3(kThreads), 0, s, (const uint16_t *)a.k,
                           (const uint16_t *)a.v, kpk, vpk, d.T, d.nb);
    if (a.part == 0 || a.part == 2) {
        const int ntp4 = (a.R + 3) / 4;
        long nwg4 = ((long)BG * ntp4 + 7) / 8 * 8;
        hipLaunchKernelGGL((k_selected_mfma<DK, DV>), dim3((unsigned)nwg4), dim3(kThreads), 0, s, a, kpk, vpk,
                           ntp4);
    }
    return hipGetLastError();
}

}  // namespace

bool sparse_mfma_supported(const Dims &d)
{
    return d.dtype == NSA_BF16 && d.G == 16 &&
           ((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64));
}

size_t sparse_mfma_ws_bytes(const Dims &d) { return (size_t)d.B * d.Hkv * d.nb * 64 * (d.dk + d.dv) * 2; }

hipError_t launch_sparse_mfma(const RowArgs &a, void *vt_ws, hipStream_t s)
{
    const Dims &d = a.d;
    if (d.dk == 192 && d.dv == 128) return launch_sparse_dims<192, 128>(a, vt_ws, s);
    if (d.dk == 128 && d.dv == 128) return launch_sparse_dims<128, 128>(a, vt_ws, s);
    if (d.dk == 64 && d.dv == 64) return launch_sparse_dims<64, 64>(a, vt_ws, s);
    return hipErrorInvalidValue;
}

}  // namespace nsa
