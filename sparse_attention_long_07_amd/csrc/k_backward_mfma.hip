// Key-side gradients on the matrix cores (bf16 storage, 16 query heads per KV
// head, (d_k, d_v) = (192, 128), (128, 128) or (64, 64)): raw keys from the
// window and selected branches, and compressed keys from the compressed
// branch (row t sees compressed key i when 16 i + 31 <= t).
//
// Per KV head, a query row t attends to raw key s in the selected branch when
// s's 64-token block is in t's selection and s <= t, and in the window branch
// when t - w < s <= t.  With branch probabilities p = exp(scale q.k - lse),
// gate gamma and D = gamma dO . o_branch (from the row pass):
//   dV_s += gamma p dO,   dK_s += scale p (gamma dO . V_s - D) q,
// summed over the rows and heads that attend to s.
//
// One workgroup owns one 64-key block j and one chunk of RC consecutive rows.
// Raw keys: it visits the chunk's window rows of the block, then the chunk's
// rows whose selection holds j (read from the (block, row) bitmap in ascending
// order); compressed keys: the chunk's rows from 16 (64 j) + 31 on.  Rows come
// in tiles of 4 rows x 16 heads = 64 query vectors.  Wave w keeps the fragments
// of keys 16w .. 16w+15 in registers and per tile forms
//   S = Q K^T, dP = dO V^T              (16x16x32 MFMA, A from LDS)
//   P, dS                               (fp32, packed to bf16 in place)
//   dV^T += dO^T P,  dK^T += Q^T dS     (A: transposing LDS reads)
// The C layout of S holds, per lane, 4 heads of one key; two row tiles give
// the 8 contraction slots of a B operand, with the slot order mirrored in the
// A operand's transposing reads.  Each workgroup writes its block's partial
// dK, dV; the chunks are then summed in order, so the result does not depend
// on scheduling.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;        // rows per tile
constexpr int kM = 16 * kRows;  // query vectors per tile
constexpr int kBatchWords = kThreads;   // bitmap words per batch of selected rows (one per thread)

struct Chunking {
    int rc, nkc;
};

// Row chunks: at most 16, at least 1024 rows each, a multiple of 64 rows.
Chunking chunking(const Dims &d)
{
    int rc = (d.T + 15) / 16;
    rc = (rc + 63) / 64 * 64;
    if (rc < 1024) rc = 1024;
    return {rc, (d.T + rc - 1) / rc};
}

// first float of chunk c's partial ([B*Hkv][kend_c][dk+dv], kend_c = keys
// below the chunk's end)
__host__ __device__ __forceinline__ long part_base(int c, int rc, long BH, int DD)
{
    return (long)rc * c * (c + 1) / 2 * BH * DD;
}

template <int DK, int DV, bool CMP>
__global__ __launch_bounds__(kThreads) void k_bwd_keys_mfma(BwdArgs a)
{
    constexpr int QS = DK + 16, OS = DV + 16;   // LDS row strides (bf16): 16-byte rows, transposing reads conflict-free
    constexpr int NQ = DK / 32, NO = DV / 32;   // 16-byte pieces per thread of a tile's Q and dO; K, V fragments
    constexpr int DD = DK + DV;
    __shared__ __align__(16) uint16_t qt[kM * QS];
    __shared__ __align__(16) uint16_t ot[kM * OS];
    __shared__ __align__(16) float s_lse[kM], s_D[kM], s_g[kM];
    __shared__ uint16_t rows[kBatchWords * 32];   // selected rows of a batch, less its first row
    __shared__ int wcnt[kThreads];
    __shared__ int nsel_s;

    const Dims &d = a.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int jb = blockIdx.x, c = blockIdx.y, bgi = blockIdx.z;
    const int b = bgi / d.Hkv, g = bgi % d.Hkv;
    const int key0 = jb * 64;
    const int rc = CMP ? kBwdRowChunk : a.krc;
    const int rbeg = c * rc, rend = min(d.T, rbeg + rc);
    // raw keys: rows before the block do not attend, and no partial is read
    // for such a chunk; compressed keys: every chunk's partial is summed
    if (!CMP && rend <= key0) return;
    const long BH = (long)d.B * d.Hkv;
    float *outp = CMP ? a.part + ((long)c * BH + bgi) * d.npad * DD
                      : a.kpart + part_base(c, rc, BH, DD) + ((long)bgi * rend) * DD;   // rend keys per head

    // this lane's key and its K, V fragments (B operands of S and dP)
    const int kk = key0 + 16 * wave + li;
    const int nkeys = CMP ? d.ncmp : d.T, kstride = CMP ? d.npad : d.T;
    u32x4 kf[NQ], vf[NO];
    {
        const uint16_t *K = (const uint16_t *)(CMP ? a.kc : a.k) + ((long)bgi * kstride + kk) * DK + 8 * lg;
        const uint16_t *V = (const uint16_t *)(CMP ? a.vc : a.v) + ((long)bgi * kstride + kk) * DV + 8 * lg;
#pragma unroll
        for (int i = 0; i < NQ; i++) kf[i] = kk < nkeys ? ld16(K + 32 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NO; i++) vf[i] = kk < nkeys ? ld16(V + 32 * i) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 acck[DK / 16], accv[DV / 16];
#pragma unroll
    for (int i = 0; i < DK / 16; i++) acck[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DV / 16; i++) accv[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const float sl2 = d.scale * kLog2e;
    // a tile's rows in registers: Q and dO pieces, and (threads 0..63, one
    // query vector each) log2-scaled lse, D and gate
    u32x4 qr[NQ], orr[NO];
    float st0 = 0.f, st1 = 0.f, st2 = 0.f;
    auto fetch = [&](const int *tr, int br) {
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const int p = tid + kThreads * i;          // piece: row slot p / (2 DK), offset 8 (p % (2 DK))
            const int r = p / (2 * DK), e = 8 * (p % (2 * DK));
            qr[i] = tr[r] >= 0 ? ld16((const uint16_t *)a.q + ((long)b * d.T + tr[r]) * d.Hq * DK + (long)g * 16 * DK + e)
                               : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NO; i++) {
            const int p = tid + kThreads * i;
            const int r = p / (2 * DV), e = 8 * (p % (2 * DV));
            orr[i] = tr[r] >= 0 ? ld16((const uint16_t *)a.dO + ((long)b * d.T + tr[r]) * d.Hq * DV + (long)g * 16 * DV + e)
                                : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < kM) {
            const int r = tid >> 4, h = tid & 15;
            if (tr[r] >= 0) {
                const float *st = a.rs + (((long)b * d.T + tr[r]) * d.Hq + g * 16 + h) * kBwdStat + br * 4;
                st0 = st[0] * kLog2e;
                st1 = st[1];
                st2 = st[2];
            } else {
                st0 = st1 = st2 = 0.f;
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const int p = tid + kThreads * i;
            const int r = p / (2 * DK), e = 8 * (p % (2 * DK));
            st16(qt + (16 * r + e / DK) * QS + e % DK, qr[i]);
        }
#pragma unroll
        for (int i = 0; i < NO; i++) {
            const int p = tid + kThreads * i;
            const int r = p / (2 * DV), e = 8 * (p % (2 * DV));
            st16(ot + (16 * r + e / DV) * OS + e % DV, orr[i]);
        }
        if (tid < kM) {
            s_lse[tid] = st0;
            s_D[tid] = st1;
            s_g[tid] = st2;
        }
    };
    // one tile from LDS; tr = its rows (-1: empty slot), br = branch (0 compressed, 1 selected, 2 window)
    auto tile = [&](const int *tr, int br) {
        f32x4 S[kRows], P[kRows];
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            S[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            P[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < NQ; i++)
#pragma unroll
            for (int r = 0; r < kRows; r++)
                S[r] = mfma16(as_bf16x8(ld16(qt + (16 * r + li) * QS + 32 * i + 8 * lg)), as_bf16x8(kf[i]), S[r]);
#pragma unroll
        for (int i = 0; i < NO; i++)
#pragma unroll
            for (int r = 0; r < kRows; r++)
                P[r] = mfma16(as_bf16x8(ld16(ot + (16 * r + li) * OS + 32 * i + 8 * lg)), as_bf16x8(vf[i]), P[r]);
        // p and ds of (head 4 lg + e of row r, key kk)
        float pg[kRows][4], ds[kRows][4];
#pragma unroll
        for (int r = 0; r < kRows; r++) {
            const int t = tr[r];
            bool vis;
            if constexpr (CMP) vis = kk < d.ncmp && 16 * kk + 31 <= t;
            else vis = kk <= t && (br == 1 || kk > t - d.w);
            const f32x4 l4 = *(const f32x4 *)(s_lse + 16 * r + 4 * lg);
            const f32x4 D4 = *(const f32x4 *)(s_D + 16 * r + 4 * lg);
            const f32x4 g4 = *(const f32x4 *)(s_g + 16 * r + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float p = vis ? fast_exp2(__builtin_fmaf(S[r][e], sl2, -l4[e])) : 0.f;
                pg[r][e] = p * g4[e];
                ds[r][e] = p * __builtin_fmaf(g4[e], P[r][e], -D4[e]) * d.scale;
            }
        }
        // B operands: contraction slot 8 lg + e <-> query vector 32 s + 4 lg + e
        // (e < 4, row tile 2s) or 32 s + 16 + 4 lg + e - 4 (row tile 2s + 1)
        bf16x8 bp[2], bs[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
            u32x4 x, y;
            x[0] = pack_bf16x2(pg[2 * s2][0], pg[2 * s2][1]);
            x[1] = pack_bf16x2(pg[2 * s2][2], pg[2 * s2][3]);
            x[2] = pack_bf16x2(pg[2 * s2 + 1][0], pg[2 * s2 + 1][1]);
            x[3] = pack_bf16x2(pg[2 * s2 + 1][2], pg[2 * s2 + 1][3]);
            y[0] = pack_bf16x2(ds[2 * s2][0], ds[2 * s2][1]);
            y[1] = pack_bf16x2(ds[2 * s2][2], ds[2 * s2][3]);
            y[2] = pack_bf16x2(ds[2 * s2 + 1][0], ds[2 * s2 + 1][1]);
            y[3] = pack_bf16x2(ds[2 * s2 + 1][2], ds[2 * s2 + 1][3]);
            bp[s2] = as_bf16x8(x);
            bs[s2] = as_bf16x8(y);
        }
        // transposing reads: lane li of group lg points at row r0 + li / 4,
        // columns 4 (li % 4) .. +3 of the column tile, and receives column li
        // of rows r0 .. r0 + 3
        const int trow = li >> 2, tcol = 4 * (li & 3);
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++) {
            const int r0 = 32 * s2 + 4 * lg + trow, r1 = r0 + 16;
#pragma unroll
            for (int dt = 0; dt < DV / 16; dt++) {
                const uint2 lo = ld_tr16(ot + r0 * OS + 16 * dt + tcol);
                const uint2 hi = ld_tr16(ot + r1 * OS + 16 * dt + tcol);
                accv[dt] = mfma16(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), bp[s2], accv[dt]);
            }
#pragma unroll
            for (int dt = 0; dt < DK / 16; dt++) {
                const uint2 lo = ld_tr16(qt + r0 * QS + 16 * dt + tcol);
                const uint2 hi = ld_tr16(qt + r1 * QS + 16 * dt + tcol);
                acck[dt] = mfma16(as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}), bs[s2], acck[dt]);
            }
        }
    };
    // tiles over a list of n rows (row(i) gives the i-th), one branch
    auto run = [&](int n, int br, auto row) {
        if (n <= 0) return;
        int tr[kRows], tn[kRows];
#pragma unroll
        for (int r = 0; r < kRows; r++) tn[r] = r < n ? row(r) : -1;
        fetch(tn, br);
        for (int i0 = 0; i0 < n; i0 += kRows) {
#pragma unroll
            for (int r = 0; r < kRows; r++) tr[r] = tn[r];
            lds_barrier();   // the previous tile's LDS reads are done
            stash();
            lds_barrier();
            if (i0 + kRows < n) {
#pragma unroll
                for (int r = 0; r < kRows; r++) tn[r] = i0 + kRows + r < n ? row(i0 + kRows + r) : -1;
                fetch(tn, br);
            }
            tile(tr, br);
        }
    };

    if constexpr (CMP) {
        const int lo = max(rbeg, 16 * key0 + 31);
        run(rend - lo, 0, [&](int i) { return lo + i; });
    } else {
    // window rows of the block in this chunk
    {
        const int lo = max(key0, rbeg), hi = min(min(d.T - 1, key0 + 63 + d.w - 1), rend - 1);
        run(hi - lo + 1, 2, [&](int i) { return lo + i; });
    }
    // selected rows in this chunk, one batch of bitmap words at a time
    {
        const int nw = (d.T + 31) / 32;
        const uint32_t *bm = a.selbm + ((long)bgi * d.nb + jb) * nw;
        const int wlo = max(rbeg, key0) / 32, whi = (rend + 31) / 32;   // rbeg, key0, rc: multiples of 64
        for (int w0 = wlo; w0 < whi; w0 += kBatchWords) {
            const int w = w0 + tid;
            uint32_t word = w < whi ? bm[w] : 0u;
            if (32 * w + 32 > rend) word &= (1u << (rend - 32 * w)) - 1u;   // a partial last word (rend = T)
            lds_barrier();   // rows of the previous batch are no longer read
            wcnt[tid] = __popc(word);
            lds_barrier();
            if (tid == 0) {
                int acc = 0;
                for (int i = 0; i < kThreads; i++) {
                    const int x = wcnt[i];
                    wcnt[i] = acc;
                    acc += x;
                }
                nsel_s = acc;
            }
            lds_barrier();
            {
                int o = wcnt[tid];
                for (uint32_t x = word; x; x &= x - 1) rows[o++] = (uint16_t)(32 * tid + __ffs(x) - 1);
            }
            lds_barrier();
            const int base = 32 * w0;
            run(nsel_s, 1, [&](int i) { return base + (int)rows[i]; });
        }
    }
    }
    // partial dK, dV of the block: C[i = column][j = key] sits in lane j + 16 (i / 4), element i % 4
    if (kk < kstride) {
        float *o = outp + (long)kk * DD;
#pragma unroll
        for (int dt = 0; dt < DK / 16; dt++) *(f32x4 *)(o + 16 * dt + 4 * lg) = acck[dt];
#pragma unroll
        for (int dt = 0; dt < DV / 16; dt++) *(f32x4 *)(o + DK + 16 * dt + 4 * lg) = accv[dt];
    }
}

// dk_raw, dv_raw = sum over the row chunks that hold the key, in chunk order.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_bwd_keys_sum(BwdArgs a)
{
    constexpr int DD = DK + DV, N4 = DD / 4;
    const Dims &d = a.d;
    const long BH = (long)d.B * d.Hkv;
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;   // (bg, key, column quad)
    if (i >= BH * d.T * N4) return;
    const int q4 = (int)(i % N4);
    const long bk = i / N4;
    const int kk = (int)(bk % d.T);
    const long bgi = bk / d.T;
    const int rc = a.krc;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int c = kk / rc; c < a.nkc; c++) {
        const int kend = min(d.T, (c + 1) * rc);
        s += *(const f32x4 *)(a.kpart + part_base(c, rc, BH, DD) + (bgi * kend + kk) * DD + 4 * q4);
    }
    if (4 * q4 < DK) *(f32x4 *)(a.dk_raw + (bgi * d.T + kk) * DK + 4 * q4) = s;
    else *(f32x4 *)(a.dv_raw + (bgi * d.T + kk) * DV + 4 * q4 - DK) = s;
}

template <int DK, int DV>
hipError_t launch_cmp_dims(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    hipLaunchKernelGGL((k_bwd_keys_mfma<DK, DV, true>), dim3(d.npad / 64, A.nchunk, d.B * d.Hkv), dim3(kThreads), 0, s,
                       A);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int BH = d.B * d.Hkv;
    hipLaunchKernelGGL((k_bwd_keys_mfma<DK, DV, false>), dim3(d.nb, A.nkc, BH), dim3(kThreads), 0, s, A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long n4 = (long)BH * d.T * ((DK + DV) / 4);
    hipLaunchKernelGGL((k_bwd_keys_sum<DK, DV>), dim3((unsigned)((n4 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, A);
    return hipGetLastError();
}

}  // namespace

bool bwd_keys_mfma_ok(const Dims &d)
{
    return d.dtype == NSA_BF16 && d.G == 16 &&
           ((d.dk == 192 && d.dv == 128) || (d.dk == 128 && d.dv == 128) || (d.dk == 64 && d.dv == 64));
}

void bwd_key_chunks(const Dims &d, int *rc, int *nkc, size_t *part_floats)
{
    const Chunking c = chunking(d);
    *rc = c.rc;
    *nkc = c.nkc;
    // chunks 0 .. nkc-2 hold (c+1) rc keys, the last one T
    *part_floats = (size_t)((long)c.rc * (c.nkc - 1) * c.nkc / 2 + d.T) * d.B * d.Hkv * (d.dk + d.dv);
}

hipError_t launch_bwd_keys_mfma(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    if (d.dk == 192) return launch_dims<192, 128>(A, s);
    if (d.dk == 128) return launch_dims<128, 128>(A, s);
    return launch_dims<64, 64>(A, s);
}

hipError_t launch_bwd_cmp_keys_mfma(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    if (d.dk == 192) return launch_cmp_dims<192, 128>(A, s);
    if (d.dk == 128) return launch_cmp_dims<128, 128>(A, s);
    return launch_cmp_dims<64, 64>(A, s);
}

}  // namespace nsa
