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
// in tiles of 4 rows x 16 heads = 64 query vectors.  Eight waves: wave w keeps
// the fragments of keys 16 (w % 4) .. +15 in registers and takes the tile's
// rows 2 (w / 4) and 2 (w / 4) + 1, forming per tile
//   S = Q K^T, dP = dO V^T              (16x16x32 MFMA, A from LDS)
//   P, dS                               (fp32, packed to bf16 in place)
//   dV^T += dO^T P,  dK^T += Q^T dS     (A: transposing LDS reads)
// The C layout of S holds, per lane, 4 heads of one key; the wave's two row
// tiles give the 8 contraction slots of a B operand, with the slot order
// mirrored in the A operand's transposing reads.  Halving each wave's rows
// keeps it under 256 registers, so two waves share each SIMD and hide each
// other's waits.  The two row halves' partial sums of a key are added through
// LDS (half 0 + half 1), each workgroup writes its block's partial dK, dV, and
// the chunks are then summed in order, so the result does not depend on
// scheduling.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kKThreads = 512;  // key pass: 8 waves, 4 key groups x 2 row halves
constexpr int kRows = 4;        // rows per tile
constexpr int kM = 16 * kRows;  // query vectors per tile
constexpr int kBatchWords = 256;   // bitmap words per batch of selected rows (one per thread of the first 256)

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
__global__ __launch_bounds__(kKThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_keys_mfma(BwdArgs a)
{
    constexpr int QS = DK + 16, OS = DV + 16;   // LDS row strides (bf16): 16-byte rows, transposing reads conflict-free
    constexpr int NQ = DK / 32, NO = DV / 32;   // K, V fragments (16-byte pieces) per lane
    constexpr int QP = kM * DK / 8 / kKThreads, OP = kM * DV / 8 / kKThreads;   // a tile's pieces per thread
    static_assert(QP * kKThreads == kM * DK / 8 && OP * kKThreads == kM * DV / 8, "tile pieces split evenly");
    constexpr int DD = DK + DV;
    constexpr int NA = DK / 16 + DV / 16;       // 16x16 accumulator tiles per lane
    // one LDS region: two tile buffers (a tile's Q and dO rows each), and at
    // the end the second row half's partial sums
    constexpr int kBuf = kM * QS + kM * OS;
    __shared__ __align__(16) uint16_t qo[2 * kBuf];
    __shared__ __align__(16) float s_lse[2][kM], s_D[2][kM], s_g[2][kM];
    // window tiles of raw keys: the selected branch's statistics of rows that
    // also selected the block (+inf log-sum-exp, so p = 0, for the others)
    __shared__ __align__(16) float s_lse2[2][kM], s_D2[2][kM], s_g2[2][kM];
    __shared__ uint16_t rows[kBatchWords * 32];   // selected rows of a batch, less its first row
    __shared__ int wcnt[kKThreads / 64];
    __shared__ int nsel_s;

    const Dims &d = a.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = wave & 3, hf = wave >> 2;    // key group, row half
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
    const int kk = key0 + 16 * kg + li;
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
    u32x4 qr[QP], orr[OP];
    float st0 = 0.f, st1 = 0.f, st2 = 0.f, st3 = 0.f, st4 = 0.f, st5 = 0.f;
    bool stv = false;   // the statistics belong to a row (not an empty slot)
    uint32_t sw = 0u;   // window tiles: the bitmap word of the row's (block, row) bit,
    int sb = 0;         // and the bit's position in it
    // row of slot r (r depends on the thread: a select chain, not an indexed array)
    auto slot = [](const int *tr, int r) { return r == 0 ? tr[0] : r == 1 ? tr[1] : r == 2 ? tr[2] : tr[3]; };
    auto fetch = [&](const int *tr, int br) {
#pragma unroll
        for (int i = 0; i < QP; i++) {
            const int p = tid + kKThreads * i;          // piece: row slot p / (2 DK), offset 8 (p % (2 DK))
            const int r = p / (2 * DK), e = 8 * (p % (2 * DK)), t = slot(tr, r);
            qr[i] = t >= 0 ? ld16((const uint16_t *)a.q + ((long)b * d.T + t) * d.Hq * DK + (long)g * 16 * DK + e)
                           : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < OP; i++) {
            const int p = tid + kKThreads * i;
            const int r = p / (2 * DV), e = 8 * (p % (2 * DV)), t = slot(tr, r);
            orr[i] = t >= 0 ? ld16((const uint16_t *)a.dO + ((long)b * d.T + t) * d.Hq * DV + (long)g * 16 * DV + e)
                            : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < kM) {
            const int r = tid >> 4, h = tid & 15, t = slot(tr, r);
            // an empty slot reads row 0 and stores zeros; the loaded values
            // are used only at the stash, so that nothing here waits for them
            // (or for the Q and dO loads just issued)
            const float *st = a.rs + (((long)b * d.T + max(t, 0)) * d.Hq + g * 16 + h) * kBwdStat;
            st0 = st[br * 4];
            st1 = st[br * 4 + 1];
            st2 = st[br * 4 + 2];
            stv = t >= 0;
            if (!CMP && br == 2) {
                st3 = st[4];
                st4 = st[5];
                st5 = st[6];
                sw = a.selbm[((long)bgi * d.nb + jb) * ((d.T + 31) / 32) + max(t, 0) / 32];
                sb = max(t, 0) & 31;
            }
        }
    };
    // the fetched tile into LDS buffer bf
    auto stash = [&](int bf) {
        uint16_t *qt = qo + bf * kBuf, *ot = qt + kM * QS;
#pragma unroll
        for (int i = 0; i < QP; i++) {
            const int p = tid + kKThreads * i;
            const int r = p / (2 * DK), e = 8 * (p % (2 * DK));
            st16(qt + (16 * r + e / DK) * QS + e % DK, qr[i]);
        }
#pragma unroll
        for (int i = 0; i < OP; i++) {
            const int p = tid + kKThreads * i;
            const int r = p / (2 * DV), e = 8 * (p % (2 * DV));
            st16(ot + (16 * r + e / DV) * OS + e % DV, orr[i]);
        }
        if (tid < kM) {
            s_lse[bf][tid] = stv ? st0 * kLog2e : 0.f;
            s_D[bf][tid] = stv ? st1 : 0.f;
            s_g[bf][tid] = stv ? st2 : 0.f;
            if (!CMP) {
                // (sw, sb are set in window tiles only; elsewhere sel is unused)
                const bool sel = stv && ((sw >> sb) & 1u);
                s_lse2[bf][tid] = sel ? st3 * kLog2e : INFINITY;
                s_D2[bf][tid] = sel ? st4 : 0.f;
                s_g2[bf][tid] = sel ? st5 : 0.f;
            }
        }
    };
    // this wave's half of the tile in LDS buffer bf: row slots 2 hf and
    // 2 hf + 1 (rows t0, t1, -1: empty), br = branch (0 compressed, 1 selected,
    // 2 window)
    auto tile = [&](int bf, int t0, int t1, int br) {
        const uint16_t *qt = qo + bf * kBuf, *ot = qt + kM * QS;
        f32x4 S[2], P[2];
#pragma unroll
        for (int r = 0; r < 2; r++) {
            S[r] = f32x4{0.f, 0.f, 0.f, 0.f};
            P[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int v0 = 32 * hf + li;   // query vector of this lane's A rows (row slot 2 hf, head li)
        // A fragments of step i + 1 are read while step i's products run
        {
            u32x4 an[2], cur[2];
#pragma unroll
            for (int r = 0; r < 2; r++) an[r] = ld16(qt + (v0 + 16 * r) * QS + 8 * lg);
#pragma unroll
            for (int i = 0; i < NQ + NO; i++) {
#pragma unroll
                for (int r = 0; r < 2; r++) cur[r] = an[r];
                if (i + 1 < NQ + NO) {
                    const int j = i + 1;
#pragma unroll
                    for (int r = 0; r < 2; r++)
                        an[r] = j < NQ ? ld16(qt + (v0 + 16 * r) * QS + 32 * j + 8 * lg)
                                       : ld16(ot + (v0 + 16 * r) * OS + 32 * (j - NQ) + 8 * lg);
                }
#pragma unroll
                for (int r = 0; r < 2; r++) {
                    if (i < NQ) S[r] = mfma16(as_bf16x8(cur[r]), as_bf16x8(kf[i]), S[r]);
                    else P[r] = mfma16(as_bf16x8(cur[r]), as_bf16x8(vf[i - NQ]), P[r]);
                }
            }
        }
        // p and ds of (head 4 lg + e of row slot 2 hf + r, key kk); a window
        // tile also carries the selected branch of rows that selected the
        // block (its keys <= t), so S and dP serve both branches
        float pg[2][4], ds[2][4];
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const int t = r ? t1 : t0;
            bool vis;
            if constexpr (CMP) vis = kk < d.ncmp && 16 * kk + 31 <= t;
            else vis = kk <= t && (br == 1 || kk > t - d.w);
            const int q0 = 32 * hf + 16 * r + 4 * lg;
            const f32x4 l4 = *(const f32x4 *)(&s_lse[bf][q0]);
            const f32x4 D4 = *(const f32x4 *)(&s_D[bf][q0]);
            const f32x4 g4 = *(const f32x4 *)(&s_g[bf][q0]);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float p = vis ? fast_exp2(__builtin_fmaf(S[r][e], sl2, -l4[e])) : 0.f;
                pg[r][e] = p * g4[e];
                ds[r][e] = p * __builtin_fmaf(g4[e], P[r][e], -D4[e]);
            }
            if (!CMP && br == 2) {
                const bool vis2 = kk <= t;
                const f32x4 l4s = *(const f32x4 *)(&s_lse2[bf][q0]);
                const f32x4 D4s = *(const f32x4 *)(&s_D2[bf][q0]);
                const f32x4 g4s = *(const f32x4 *)(&s_g2[bf][q0]);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float p = vis2 ? fast_exp2(__builtin_fmaf(S[r][e], sl2, -l4s[e])) : 0.f;
                    pg[r][e] = __builtin_fmaf(p, g4s[e], pg[r][e]);
                    ds[r][e] = __builtin_fmaf(p, __builtin_fmaf(g4s[e], P[r][e], -D4s[e]), ds[r][e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; e++) ds[r][e] *= d.scale;
        }
        // B operands: contraction slot 8 lg + e <-> query vector 32 hf + 4 lg + e
        // (e < 4, row slot 2 hf) or 32 hf + 16 + 4 lg + e - 4 (row slot 2 hf + 1)
        bf16x8 bp, bs;
        {
            u32x4 x, y;
            x[0] = pack_bf16x2(pg[0][0], pg[0][1]);
            x[1] = pack_bf16x2(pg[0][2], pg[0][3]);
            x[2] = pack_bf16x2(pg[1][0], pg[1][1]);
            x[3] = pack_bf16x2(pg[1][2], pg[1][3]);
            y[0] = pack_bf16x2(ds[0][0], ds[0][1]);
            y[1] = pack_bf16x2(ds[0][2], ds[0][3]);
            y[2] = pack_bf16x2(ds[1][0], ds[1][1]);
            y[3] = pack_bf16x2(ds[1][2], ds[1][3]);
            bp = as_bf16x8(x);
            bs = as_bf16x8(y);
        }
        // transposing reads: lane li of group lg points at row r0 + li / 4,
        // columns 4 (li % 4) .. +3 of the column tile, and receives column li
        // of rows r0 .. r0 + 3
        const int trow = li >> 2, tcol = 4 * (li & 3);
        const int r0 = 32 * hf + 4 * lg + trow, r1 = r0 + 16;
        // transposing reads in groups of 4 column tiles, issued before their products
#pragma unroll
        for (int d0 = 0; d0 < DV / 16; d0 += 4) {
            uint2 lo[4], hi[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                lo[u] = ld_tr16(ot + r0 * OS + 16 * (d0 + u) + tcol);
                hi[u] = ld_tr16(ot + r1 * OS + 16 * (d0 + u) + tcol);
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
                accv[d0 + u] = mfma16(as_bf16x8(u32x4{lo[u].x, lo[u].y, hi[u].x, hi[u].y}), bp, accv[d0 + u]);
        }
#pragma unroll
        for (int d0 = 0; d0 < DK / 16; d0 += 4) {
            uint2 lo[4], hi[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                lo[u] = ld_tr16(qt + r0 * QS + 16 * (d0 + u) + tcol);
                hi[u] = ld_tr16(qt + r1 * QS + 16 * (d0 + u) + tcol);
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
                acck[d0 + u] = mfma16(as_bf16x8(u32x4{lo[u].x, lo[u].y, hi[u].x, hi[u].y}), bs, acck[d0 + u]);
        }
    };
    // tiles over a list of n rows (row(i) gives the i-th), one branch.  Tile
    // k is computed from LDS buffer k % 2 while tile k + 1, fetched into
    // registers during tile k - 1, is stored into the other buffer and tile
    // k + 2 is fetched: one barrier per tile, and each fetch has a tile's
    // work to land.
    auto run = [&](int n, int br, auto row) {
        if (n <= 0) return;
        int tn[kRows];
#pragma unroll
        for (int r = 0; r < kRows; r++) tn[r] = r < n ? row(r) : -1;
        fetch(tn, br);
        // this wave's two rows of the tile in the registers
        int t0 = hf ? tn[2] : tn[0], t1 = hf ? tn[3] : tn[1];
        lds_barrier();   // the buffers' previous readers are done
        stash(0);
        if (kRows < n) {
#pragma unroll
            for (int r = 0; r < kRows; r++) tn[r] = kRows + r < n ? row(kRows + r) : -1;
            fetch(tn, br);
        }
        lds_barrier();
        int bf = 0;
        for (int i0 = 0; i0 < n; i0 += kRows) {
            tile(bf, t0, t1, br);
            if (i0 + kRows < n) {
                t0 = hf ? tn[2] : tn[0];
                t1 = hf ? tn[3] : tn[1];
                stash(bf ^ 1);   // its last readers finished before the previous barrier
                if (i0 + 2 * kRows < n) {
#pragma unroll
                    for (int r = 0; r < kRows; r++)
                        tn[r] = i0 + 2 * kRows + r < n ? row(i0 + 2 * kRows + r) : -1;
                    fetch(tn, br);
                }
            }
            lds_barrier();   // buffer bf ^ 1 is written, buffer bf is read
            bf ^= 1;
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
    // selected rows in this chunk, one batch of bitmap words at a time (one
    // word per thread of the first kBatchWords)
    {
        const int nw = (d.T + 31) / 32;
        const uint32_t *bm = a.selbm + ((long)bgi * d.nb + jb) * nw;
        const int wlo = max(rbeg, key0) / 32, whi = (rend + 31) / 32;   // rbeg, key0, rc: multiples of 64
        const int wend = key0 + 63 + d.w - 1;   // the last row whose window reaches the block
        for (int w0 = wlo; w0 < whi; w0 += kBatchWords) {
            const int w = w0 + tid;
            uint32_t word = tid < kBatchWords && w < whi ? bm[w] : 0u;
            if (word && 32 * w + 32 > rend) word &= (1u << (rend - 32 * w)) - 1u;   // a partial last word (rend = T)
            // rows up to the window range's end were taken with the window tiles
            if (32 * w + 31 <= wend) word = 0u;
            else if (32 * w <= wend) word &= ~((1u << (wend - 32 * w + 1)) - 1u);
            // exclusive prefix of the words' bit counts: within each wave by
            // shuffles, then over the waves' totals
            const int cnt = __popc(word);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            lds_barrier();   // rows and wave totals of the previous batch are no longer read
            if (lane == 63) wcnt[wave] = incl;
            lds_barrier();
            int before = 0;
            for (int w2 = 0; w2 < wave; w2++) before += wcnt[w2];
            {
                int o = before + incl - cnt;
                for (uint32_t x = word; x; x &= x - 1) rows[o++] = (uint16_t)(32 * tid + __ffs(x) - 1);
            }
            if (tid == 0) {
                int tot = 0;
                for (int w2 = 0; w2 < kKThreads / 64; w2++) tot += wcnt[w2];
                nsel_s = tot;
            }
            lds_barrier();
            const int base = 32 * w0;
            run(nsel_s, 1, [&](int i) { return base + (int)rows[i]; });
        }
    }
    }
    // the two row halves' partial dK, dV of each key, added in a fixed order
    // (half 0 + half 1) through LDS, in rounds of kRed accumulator tiles
    auto acc = [&](int i) -> f32x4 & { return i < DK / 16 ? acck[i] : accv[i - DK / 16]; };
    constexpr int kRed = 2 * kBuf * 2 / (4 * 64 * 4 * 4);   // f32x4 tiles per lane per round
    float *red = (float *)qo;
#pragma unroll
    for (int i0 = 0; i0 < NA; i0 += kRed) {
        lds_barrier();   // the tile buffers (or the previous round) are no longer read
        if (hf == 1) {
#pragma unroll
            for (int i = i0; i < NA && i < i0 + kRed; i++)
                *(f32x4 *)(red + (((i - i0) * 4 + kg) * 64 + lane) * 4) = acc(i);
        }
        lds_barrier();
        if (hf == 0) {
#pragma unroll
            for (int i = i0; i < NA && i < i0 + kRed; i++)
                acc(i) += *(const f32x4 *)(red + (((i - i0) * 4 + kg) * 64 + lane) * 4);
        }
    }
    // partial dK, dV of the block: C[i = column][j = key] sits in lane j + 16 (i / 4), element i % 4
    if (hf == 0 && kk < kstride) {
        float *o = outp + (long)kk * DD;
#pragma unroll
        for (int dt = 0; dt < DK / 16; dt++) *(f32x4 *)(o + 16 * dt + 4 * lg) = acck[dt];
#pragma unroll
        for (int dt = 0; dt < DV / 16; dt++) *(f32x4 *)(o + DK + 16 * dt + 4 * lg) = accv[dt];
    }
}

// Row pass: one wave per (b, t, KV head) with its 16 heads, 4 consecutive
// positions per workgroup; per branch (0 compressed, 1 selected, 2 window)
// two sweeps over 64-key chunks:
//   1. S^T = K Q^T and dP^T = V dO^T; online max m, sum l of exp(S) and sum of
//      exp(S) dP, which give lse and dO . o_branch = (sum p dP) / l without
//      forming o_branch; then D = gate dO . o and the gate's logit gradient.
//   2. S^T, dP^T again; dS^T = scale p (gate dP - D) feeds dQ^T += K^T dS^T
//      directly from the score layout; K reaches the A operand through LDS,
//      read with transposing reads.
// SAVED: the forward kept each branch's log-sum-exp and output, so sweep 1
// becomes one read of them (dO . o_branch as a dot product), as FlashAttention
// does with its saved softmax statistics, and every key is visited once.
// Chunks (as in the forward): compressed blocks [0, nvis), 16 i + 31 <= t;
// the distinct valid selected blocks in ascending order, tokens <= t; the
// window [t - w + 1, t].  The compressed and window chunks of the 4 positions
// nearly coincide, so the workgroup walks one chunk sequence for all of them
// (up to the last position's range) and stages each chunk's K and V in LDS
// once; each wave masks the keys its position does not see and skips chunks
// with none.  Selected blocks differ per position: each wave loads its own
// and passes K through a private 32-key LDS buffer.  Loads of keys outside a
// range read the nearest valid key instead, so no unwritten or stale value
// enters a product.
template <int DK, int DV, bool SAVED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_rows_mfma(BwdArgs a)
{
    constexpr int KS = DK + 16, VS = DV + 16;
    constexpr int NQ = DK / 32, NO = DV / 32;
    constexpr int kShared = 64 * KS + 64 * VS, kPrivate = (kThreads / 64) * 32 * KS;
    // one buffer, two uses: the shared K and V chunk (compressed, window) or
    // the waves' private K buffers (selected)
    __shared__ __align__(16) uint16_t lds[kShared > kPrivate ? kShared : kPrivate];
    __shared__ int blks[kThreads / 64][16];
    uint16_t *ksh = lds, *vsh = lds + 64 * KS;
    const Dims &d = a.d;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int g = blockIdx.y, b = blockIdx.z;
    const int t_lo = blockIdx.x * (kThreads / 64), t_hi = min(d.T - 1, t_lo + kThreads / 64 - 1);
    // a wave past the sequence computes position T-1 and stores nothing
    const bool act = t_lo + wave < d.T;
    const int t = act ? t_lo + wave : d.T - 1;
    uint16_t *kw = lds + wave * 32 * KS;
    int *blk = blks[wave];
    const long bgi = (long)b * d.Hkv + g;
    const long row0 = ((long)b * d.T + t) * d.Hq + (long)g * 16;
    const int h = li;   // the head of this lane in the B operands and the score layout

    // B operands Q^T, dO^T: head li, columns 32 c + 8 lg .. +7
    u32x4 qf[NQ], of[NO];
#pragma unroll
    for (int c = 0; c < NQ; c++) qf[c] = ld16((const uint16_t *)a.q + (row0 + h) * DK + 32 * c + 8 * lg);
#pragma unroll
    for (int c = 0; c < NO; c++) of[c] = ld16((const uint16_t *)a.dO + (row0 + h) * DV + 32 * c + 8 * lg);
    float gate[3];
#pragma unroll
    for (int br = 0; br < 3; br++) {
        const uint16_t *wr = (const uint16_t *)a.wg + (((long)g * 16 + h) * 3 + br) * DK + 8 * lg;
        float z = 0.f;
#pragma unroll
        for (int c = 0; c < NQ; c++) z = dot8_bf16(qf[c], ld16(wr + 32 * c), z);
        z += __shfl_xor(z, 16);
        z += __shfl_xor(z, 32);
        z += bf2f(((const uint16_t *)a.bg)[((long)g * 16 + h) * 3 + br]);
        gate[br] = 1.f / (1.f + __expf(-z));
    }
    // The distinct valid selected blocks, ascending.  Blocks from jlo on start
    // inside the window's staged key range [max(0, t_lo - w + 1), t_hi] (at
    // most 64 of them): their dS terms are added in the window sweep, where
    // S and dP of those keys are formed anyway; the selected sweep takes the
    // nlow blocks below jlo.  sm_lo, sm_hi: bit j - jlo of those blocks.
    const int jcur = t / 64;
    const int jlo = max((max(0, t_lo - d.w + 1) + 63) / 64, jcur - 63);
    int nsel, nlow;
    uint32_t sm_lo, sm_hi;
    {
        const int j = lane < d.n ? a.idx[(bgi * d.T + t) * d.n + lane] : -1;
        bool keep = j >= 0 && j <= jcur;
        for (int u = 0; u < d.n; u++) {
            const int x = __shfl(j, u);
            if (u < lane && x == j) keep = false;
        }
        const int kx = keep ? j : 0x7fffffff;
        int rank = 0;
        nsel = 0;
        nlow = 0;
        for (int u = 0; u < d.n; u++) {
            const int x = __shfl(kx, u);
            rank += x < kx;
            nsel += x != 0x7fffffff;
            nlow += x < jlo;
        }
        if (keep) blk[rank] = j;
        const int bit = keep && j >= jlo ? j - jlo : -1;
        uint32_t lo = bit >= 0 && bit < 32 ? 1u << bit : 0u, hi = bit >= 32 ? 1u << (bit - 32) : 0u;
        for (int off = 1; off < 64; off <<= 1) {
            lo |= __shfl_xor(lo, off);
            hi |= __shfl_xor(hi, off);
        }
        sm_lo = lo;
        sm_hi = hi;
    }
    // the first key of those blocks (the window sweep's lower limit for this row)
    const int sel_k0 = sm_lo ? 64 * (jlo + __builtin_ctz(sm_lo)) : sm_hi ? 64 * (jlo + 32 + __builtin_ctz(sm_hi)) : d.T;

    const float sl2 = d.scale * kLog2e;
    const int nvis = t >= 31 ? (t - 31) / 16 + 1 : 0;
    const int nvis_hi = t_hi >= 31 ? (t_hi - 31) / 16 + 1 : 0;
    const int wlo = max(0, t - d.w + 1), wlo0 = max(0, t_lo - d.w + 1);
    f32x4 dqa[DK / 16];
#pragma unroll
    for (int i = 0; i < DK / 16; i++) dqa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dzs[3];
    const int trow = li >> 2, tcol = 4 * (li & 3);

    // S^T and dP^T of one 16-key tile from K rows kr (A operand layout: key
    // li, columns 32 c + 8 lg .. +7) and V rows vr; kfr keeps the K pieces
    auto tile_scores = [&](const uint16_t *kr, long ks, const uint16_t *vr, long vs, f32x4 &S, f32x4 &P, u32x4 *kfr) {
        S = f32x4{0.f, 0.f, 0.f, 0.f};
        P = f32x4{0.f, 0.f, 0.f, 0.f};
        // every read issued before the products that use them
        u32x4 vfr[NO];
#pragma unroll
        for (int c = 0; c < NQ; c++) kfr[c] = ld16(kr + li * ks + 32 * c + 8 * lg);
#pragma unroll
        for (int c = 0; c < NO; c++) vfr[c] = ld16(vr + li * vs + 32 * c + 8 * lg);
#pragma unroll
        for (int c = 0; c < NQ; c++) S = mfma16(as_bf16x8(kfr[c]), as_bf16x8(qf[c]), S);
#pragma unroll
        for (int c = 0; c < NO; c++) P = mfma16(as_bf16x8(vfr[c]), as_bf16x8(of[c]), P);
    };
    // sweep-1 update over a 64-key chunk: sc, dp hold its scores (log2 units,
    // -inf where masked) and dP
    auto online = [&](float (&sc)[4][4], float (&dp)[4][4], float &m, float &l, float &acc) {
        float mc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int e = 0; e < 4; e++) mc = fmaxf(mc, sc[kt][e]);
        mc = fmaxf(mc, __shfl_xor(mc, 16));
        mc = fmaxf(mc, __shfl_xor(mc, 32));
        const float mn = fmaxf(m, mc);
        const float al = fast_exp2(m - mn);
        float ls = 0.f, as = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float p = fast_exp2(sc[kt][e] - mn);
                ls += p;
                as = __builtin_fmaf(p, sc[kt][e] == -INFINITY ? 0.f : dp[kt][e], as);
            }
        l = __builtin_fmaf(l, al, ls);
        acc = __builtin_fmaf(acc, al, as);
        m = mn;
    };
    // the branch's statistics from lse (log2 units) and dO . o_branch
    auto put_stats = [&](int br, float lse2, float dOo, float &D) {
        const float gv = gate[br];
        D = gv * dOo;
        dzs[br] = dOo * gv * (1.f - gv);
        if (act && lg == 0) {
            float *st = a.rs + (row0 + h) * kBwdStat + br * 4;
            st[0] = lse2 * kLn2;
            st[1] = D;
            st[2] = gv;
            st[3] = dzs[br];
        }
    };
    // ... from the sweep-1 sums
    auto finish = [&](int br, float m, float l, float acc, float &lse2, float &D) {
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        lse2 = l > 0.f ? m + fast_log2(l) : -INFINITY;
        put_stats(br, lse2, l > 0.f ? acc / l : 0.f, D);
    };
    // ... from the forward's saved log-sum-exp and branch output (o_branch
    // row of head h, columns 32 c + 8 lg .. +7 as in of[c])
    auto from_saved = [&](int br, float &lse2, float &D) {
        const long slot = (long)d.B * d.T * d.Hq;
        lse2 = a.lse_sv[br * slot + row0 + h] * kLog2e;
        const uint16_t *orow = (const uint16_t *)a.o_sv + (br * slot + row0 + h) * DV + 8 * lg;
        float dOo = 0.f;
#pragma unroll
        for (int c = 0; c < NO; c++) dOo = dot8_bf16(of[c], ld16(orow + 32 * c), dOo);
        dOo += __shfl_xor(dOo, 16);
        dOo += __shfl_xor(dOo, 32);
        put_stats(br, lse2, dOo, D);
    };
    // ds of a tile's 4 keys per lane, scaled
    auto tile_ds = [&](const f32x4 &S, const f32x4 &P, int k16, int klo, int khi, float lse2, float gv, float D,
                       float *ds) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int key = k16 + 4 * lg + e;
            const float p = key >= klo && key <= khi ? fast_exp2(__builtin_fmaf(S[e], sl2, -lse2)) : 0.f;
            ds[e] = p * __builtin_fmaf(gv, P[e], -D) * d.scale;
        }
    };
    // ... and in the window sweep, with the selected branch's terms of keys
    // in its blocks from jlo on (statistics lse2s, Ds, gate gs)
    auto tile_ds_win = [&](const f32x4 &S, const f32x4 &P, int k16, int klo, int khi, float lse2, float gv, float D,
                           float lse2s, float gs, float Ds, float *ds) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int key = k16 + 4 * lg + e;
            const float pw = key >= klo && key <= khi ? fast_exp2(__builtin_fmaf(S[e], sl2, -lse2)) : 0.f;
            const int rel = (key >> 6) - jlo;
            const uint32_t word = rel < 32 ? sm_lo : sm_hi;
            const bool sel = key <= t && rel >= 0 && ((word >> (rel & 31)) & 1u);
            const float ps = sel ? fast_exp2(__builtin_fmaf(S[e], sl2, -lse2s)) : 0.f;
            ds[e] = __builtin_fmaf(pw, __builtin_fmaf(gv, P[e], -D), ps * __builtin_fmaf(gs, P[e], -Ds)) * d.scale;
        }
    };
    // dQ^T += K^T dS^T over 32 keys whose K rows sit at kb (stride KS):
    // contraction slot 8 lg + e <-> key 4 lg + e (e < 4) or 16 + 4 lg + e - 4
    auto dq_step = [&](const uint16_t *kb, const float *ds0, const float *ds1) {
        u32x4 y;
        y[0] = pack_bf16x2(ds0[0], ds0[1]);
        y[1] = pack_bf16x2(ds0[2], ds0[3]);
        y[2] = pack_bf16x2(ds1[0], ds1[1]);
        y[3] = pack_bf16x2(ds1[2], ds1[3]);
        const bf16x8 bs = as_bf16x8(y);
        const int r0 = 4 * lg + trow;
#pragma unroll
        for (int d0 = 0; d0 < DK / 16; d0 += 4) {
            uint2 lo[4], hi[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                lo[u] = ld_tr16(kb + r0 * KS + 16 * (d0 + u) + tcol);
                hi[u] = ld_tr16(kb + (r0 + 16) * KS + 16 * (d0 + u) + tcol);
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
                dqa[d0 + u] = mfma16(as_bf16x8(u32x4{lo[u].x, lo[u].y, hi[u].x, hi[u].y}), bs, dqa[d0 + u]);
        }
    };

    float lse2s = -INFINITY, Ds = 0.f;   // the selected branch's statistics, for the window sweep
    for (int br = 0; br < 3; br++) {
        const float gv = gate[br];
        if (br == 1) {
            // selected: every wave on its own blocks, K via its private buffer
            lds_barrier();   // the shared chunk of the compressed branch is no longer read
            const uint16_t *K = (const uint16_t *)a.k + bgi * d.T * DK;
            const uint16_t *V = (const uint16_t *)a.v + bgi * d.T * DV;
            float lse2, D;
            if constexpr (SAVED) from_saved(1, lse2, D);
            else {
                float m = -INFINITY, l = 0.f, acc = 0.f;
                for (int ch = 0; ch < nsel; ch++) {
                    const int key0 = 64 * blk[ch], khi = min(t, key0 + 63);
                    float sc[4][4], dp[4][4];
#pragma unroll
                    for (int kt = 0; kt < 4; kt++) {
                        f32x4 S, P;
                        u32x4 kfr[NQ];
                        const int row = min(key0 + 16 * kt + li, khi);   // rows past the range read its last key
                        tile_scores(K + (long)(row - li) * DK, DK, V + (long)(row - li) * DV, DV, S, P, kfr);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int key = key0 + 16 * kt + 4 * lg + e;
                            sc[kt][e] = key <= khi ? S[e] * sl2 : -INFINITY;
                            dp[kt][e] = P[e];
                        }
                    }
                    online(sc, dp, m, l, acc);
                }
                finish(1, m, l, acc, lse2, D);
            }
            lse2s = lse2;
            Ds = D;
            for (int ch = 0; ch < nlow; ch++) {
                const int key0 = 64 * blk[ch], khi = min(t, key0 + 63);
#pragma unroll
                for (int half = 0; half < 2; half++) {
                    float ds[2][4];
#pragma unroll
                    for (int kh = 0; kh < 2; kh++) {
                        f32x4 S, P;
                        u32x4 kfr[NQ];
                        const int k16 = key0 + 32 * half + 16 * kh;
                        const int row = min(k16 + li, khi);
                        tile_scores(K + (long)(row - li) * DK, DK, V + (long)(row - li) * DV, DV, S, P, kfr);
#pragma unroll
                        for (int c = 0; c < NQ; c++) st16(kw + (16 * kh + li) * KS + 32 * c + 8 * lg, kfr[c]);
                        tile_ds(S, P, k16, key0, khi, lse2, gv, D, ds[kh]);
                    }
                    dq_step(kw, ds[0], ds[1]);
                }
            }
            continue;
        }
        // compressed or window: one chunk sequence for the workgroup
        const uint16_t *K = br == 0 ? (const uint16_t *)a.kc + bgi * d.npad * DK : (const uint16_t *)a.k + bgi * d.T * DK;
        const uint16_t *V = br == 0 ? (const uint16_t *)a.vc + bgi * d.npad * DV : (const uint16_t *)a.v + bgi * d.T * DV;
        const int glo = br == 0 ? 0 : wlo0, ghi = br == 0 ? nvis_hi - 1 : t_hi;   // keys loaded
        const int klo = br == 0 ? 0 : wlo, khi = br == 0 ? nvis - 1 : t;          // keys this row sees
        const int klo2 = br == 0 ? 0 : min(wlo, sel_k0);   // ... with the selected blocks from jlo on
        const int nch = ghi >= glo ? (ghi - glo + 64) / 64 : 0;
        auto stage = [&](int key0) {
            // 64 K rows and 64 V rows, rows past the range read its last key;
            // all of K's loads are issued before its first store, then V's, so
            // the chunk costs two load latencies (not one per piece)
            constexpr int NKP = 64 * DK / 8 / kThreads, NVP = 64 * DV / 8 / kThreads;
            static_assert(NKP * kThreads == 64 * DK / 8 && NVP * kThreads == 64 * DV / 8, "chunk pieces split evenly");
            {
                u32x4 kp[NKP];
#pragma unroll
                for (int i = 0; i < NKP; i++) {
                    const int pc = tid + kThreads * i, r = pc / (DK / 8), cc = 8 * (pc % (DK / 8));
                    kp[i] = ld16(K + (long)min(key0 + r, ghi) * DK + cc);
                }
#pragma unroll
                for (int i = 0; i < NKP; i++) {
                    const int pc = tid + kThreads * i, r = pc / (DK / 8), cc = 8 * (pc % (DK / 8));
                    st16(ksh + r * KS + cc, kp[i]);
                }
            }
            {
                u32x4 vp[NVP];
#pragma unroll
                for (int i = 0; i < NVP; i++) {
                    const int pc = tid + kThreads * i, r = pc / (DV / 8), cc = 8 * (pc % (DV / 8));
                    vp[i] = ld16(V + (long)min(key0 + r, ghi) * DV + cc);
                }
#pragma unroll
                for (int i = 0; i < NVP; i++) {
                    const int pc = tid + kThreads * i, r = pc / (DV / 8), cc = 8 * (pc % (DV / 8));
                    st16(vsh + r * VS + cc, vp[i]);
                }
            }
        };
        float lse2, D;
        if constexpr (SAVED) from_saved(br, lse2, D);
        else {
            float m = -INFINITY, l = 0.f, acc = 0.f;
            for (int ch = 0; ch < nch; ch++) {
                const int key0 = glo + 64 * ch;
                lds_barrier();
                stage(key0);
                lds_barrier();
                if (max(key0, klo) > min(key0 + 63, khi)) continue;   // nothing this row sees
                float sc[4][4], dp[4][4];
#pragma unroll
                for (int kt = 0; kt < 4; kt++) {
                    f32x4 S, P;
                    u32x4 kfr[NQ];
                    tile_scores(ksh + 16 * kt * KS, KS, vsh + 16 * kt * VS, VS, S, P, kfr);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int key = key0 + 16 * kt + 4 * lg + e;
                        sc[kt][e] = key >= klo && key <= khi ? S[e] * sl2 : -INFINITY;
                        dp[kt][e] = P[e];
                    }
                }
                online(sc, dp, m, l, acc);
            }
            finish(br, m, l, acc, lse2, D);
        }
        for (int ch = 0; ch < nch; ch++) {
            const int key0 = glo + 64 * ch;
            lds_barrier();
            stage(key0);
            lds_barrier();
            if (max(key0, klo2) > min(key0 + 63, khi)) continue;
#pragma unroll
            for (int half = 0; half < 2; half++) {
                float ds[2][4];
#pragma unroll
                for (int kh = 0; kh < 2; kh++) {
                    f32x4 S, P;
                    u32x4 kfr[NQ];
                    const int r16 = 32 * half + 16 * kh;
                    tile_scores(ksh + r16 * KS, KS, vsh + r16 * VS, VS, S, P, kfr);
                    if (br == 2) tile_ds_win(S, P, key0 + r16, klo, khi, lse2, gv, D, lse2s, gate[1], Ds, ds[kh]);
                    else tile_ds(S, P, key0 + r16, klo, khi, lse2, gv, D, ds[kh]);
                }
                dq_step(ksh + 32 * half * KS, ds[0], ds[1]);
            }
        }
    }
    if (!act) return;
    // dq = dQ^T (C[i = column][j = head]: lane j + 16 (i / 4), element i % 4)
    // plus the gate terms sum_c dz_c W_g[h][c]
    uint16_t *dq = (uint16_t *)a.dq + (row0 + h) * DK;
    const uint16_t *wg = (const uint16_t *)a.wg + ((long)g * 16 + h) * 3 * DK;
    // all gate-weight loads are issued before the first store (the two
    // pointers may alias as far as the compiler knows)
    uint2 wv[DK / 16][3];
#pragma unroll
    for (int dt = 0; dt < DK / 16; dt++)
#pragma unroll
        for (int br = 0; br < 3; br++) wv[dt][br] = *(const uint2 *)(wg + br * DK + 16 * dt + 4 * lg);
#pragma unroll
    for (int dt = 0; dt < DK / 16; dt++) {
        const int col = 16 * dt + 4 * lg;
        float z[4] = {dqa[dt][0], dqa[dt][1], dqa[dt][2], dqa[dt][3]};
#pragma unroll
        for (int br = 0; br < 3; br++) {
            const uint2 w = wv[dt][br];
            z[0] = __builtin_fmaf(dzs[br], bf2f((uint16_t)(w.x & 0xffffu)), z[0]);
            z[1] = __builtin_fmaf(dzs[br], bf2f((uint16_t)(w.x >> 16)), z[1]);
            z[2] = __builtin_fmaf(dzs[br], bf2f((uint16_t)(w.y & 0xffffu)), z[2]);
            z[3] = __builtin_fmaf(dzs[br], bf2f((uint16_t)(w.y >> 16)), z[3]);
        }
        *(uint2 *)(dq + col) = uint2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
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

// Weight gradient of one compression map on the matrix cores:
//   dW[c][m] = sum_r G[r][c] x_r[m] + colsum[c] PE[m],  r = (b, head, block i < ncmp),
// x_r = the 32 dim tokens of block i flattened, G = the compressed-key (or
// -value) gradient, colsum[c] = sum_r G[r][c].  A workgroup owns a 64 x 64
// tile of dW (wave w: channels 16 w .. 16 w + 15); per 64-row step G (as
// bf16) and x are staged in LDS and both operands are read with transposing
// reads (the contraction index r is the row index of both).
template <int DIM>
__global__ __launch_bounds__(kThreads) void k_bwd_dw_mfma(const float *__restrict__ G, int gs,
                                                          const uint16_t *__restrict__ x, const uint16_t *__restrict__ pe,
                                                          const float *__restrict__ colsum, float *__restrict__ out,
                                                          int T, int ncmp, int npad, int rows)
{
    constexpr int RS = 72;   // LDS row stride (bf16) of the staged tiles
    constexpr int N = 32 * DIM;
    __shared__ __align__(16) uint16_t gt[64 * RS], xt[64 * RS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int c0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
    f32x4 acc[4];
#pragma unroll
    for (int n = 0; n < 4; n++) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // staging: thread -> (row tid / 4, 16 columns from 16 (tid % 4))
    const int sr = tid >> 2, sc = 16 * (tid & 3);
    const int trow = li >> 2, tcol = 4 * (li & 3);
    for (int r0 = 0; r0 < rows; r0 += 64) {
        const int r = r0 + sr;
        u32x4 gv0 = {0u, 0u, 0u, 0u}, gv1 = {0u, 0u, 0u, 0u}, xv0 = {0u, 0u, 0u, 0u}, xv1 = {0u, 0u, 0u, 0u};
        if (r < rows) {
            const int bh = r / ncmp, i = r % ncmp;
            const float *gr = G + ((long)bh * npad + i) * gs + c0 + sc;
            const float4 f0 = *(const float4 *)gr, f1 = *(const float4 *)(gr + 4);
            const float4 f2 = *(const float4 *)(gr + 8), f3 = *(const float4 *)(gr + 12);
            gv0 = u32x4{pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y), pack_bf16x2(f1.z, f1.w)};
            gv1 = u32x4{pack_bf16x2(f2.x, f2.y), pack_bf16x2(f2.z, f2.w), pack_bf16x2(f3.x, f3.y), pack_bf16x2(f3.z, f3.w)};
            const uint16_t *xr = x + ((long)bh * T + 16L * i) * DIM + m0 + sc;
            xv0 = ld16(xr);
            xv1 = ld16(xr + 8);
        }
        lds_barrier();   // the previous step's reads are done
        st16(gt + sr * RS + sc, gv0);
        st16(gt + sr * RS + sc + 8, gv1);
        st16(xt + sr * RS + sc, xv0);
        st16(xt + sr * RS + sc + 8, xv1);
        lds_barrier();
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            // A[i = channel][k = row]: rows 32 ks + 8 lg .. +7 of channel 16 wave + li
            const int ra = 32 * ks + 8 * lg + trow;
            const uint2 a0 = ld_tr16(gt + ra * RS + 16 * wave + tcol);
            const uint2 a1 = ld_tr16(gt + (ra + 4) * RS + 16 * wave + tcol);
            const bf16x8 av = as_bf16x8(u32x4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
            for (int n = 0; n < 4; n++) {
                const uint2 b0 = ld_tr16(xt + ra * RS + 16 * n + tcol);
                const uint2 b1 = ld_tr16(xt + (ra + 4) * RS + 16 * n + tcol);
                acc[n] = mfma16(av, as_bf16x8(u32x4{b0.x, b0.y, b1.x, b1.y}), acc[n]);
            }
        }
    }
    // C[i = channel][j = column]: lane j + 16 (i / 4), element i % 4
#pragma unroll
    for (int n = 0; n < 4; n++) {
        const int m = m0 + 16 * n + li;
        const float pm = bf2f(pe[m]);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int c = c0 + 16 * wave + 4 * lg + e;
            out[(long)c * N + m] = __builtin_fmaf(colsum[c], pm, acc[n][e]);
        }
    }
}

// Token gradient of one compression map on the matrix cores, added to the
// raw-key gradient.  Block i covers tokens 16 i .. 16 i + 31, so token 16 m + u
// (u < 16) is position u of block m and position 16 + u of block m - 1:
//   dx[bh][16 m + u][e] = raw + sum_c G[bh][m][c] W[c][u DIM + e]
//                             + sum_c G[bh][m-1][c] W[c][(16 + u) DIM + e]
// (blocks outside 0 .. ncmp-1 contribute nothing).  A workgroup owns 64 token
// groups m x 64 columns n = u DIM + e of one (b, KV head), wave w the groups
// 16 w .. 16 w + 15.  Per 32-deep step over (block m or m - 1, channel) the W
// tile (32 channels x 64 columns) is staged in LDS, double-buffered, and read
// as the B operand by transposing reads; the A operand (G rows, fp32 to bf16)
// comes straight from memory, one step ahead.
template <int DIM>
__global__ __launch_bounds__(kThreads) void k_bwd_dx_mfma(const float *__restrict__ G, int gs,
                                                          const uint16_t *__restrict__ W, const float *__restrict__ raw,
                                                          uint16_t *__restrict__ dx, int T, int ncmp, int npad)
{
    constexpr int RS = 72;                 // LDS row stride (bf16) of the staged W tile
    constexpr int CS = DIM / 32;           // 32-channel steps per block
    constexpr int NSTEP = 2 * CS;
    __shared__ __align__(16) uint16_t wt[2][32 * RS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64, bh = blockIdx.z;
    const int trow = li >> 2, tcol = 4 * (li & 3);
    const int sr = tid >> 3, sc = 8 * (tid & 7);   // staging: channel row, 8 columns
    const int m = m0 + 16 * wave + li;            // this lane's A row (token group)
    f32x4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto wload = [&](int st) {
        const int c = 32 * (st % CS) + sr;
        return ld16(W + (long)c * 32 * DIM + 16 * DIM * (st / CS) + n0 + sc);
    };
    auto aload = [&](int st) {
        const int i = m - st / CS, c = 32 * (st % CS) + 8 * lg;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (i >= 0 && i < ncmp) {
            const float *gr = G + ((long)bh * npad + i) * gs + c;
            const float4 f0 = *(const float4 *)gr, f1 = *(const float4 *)(gr + 4);
            v = u32x4{pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y),
                      pack_bf16x2(f1.z, f1.w)};
        }
        return v;
    };
    u32x4 wv = wload(0), av = aload(0);
    for (int st = 0; st < NSTEP; st++) {
        const int buf = st & 1;
        // buffer buf's last readers (step st - 2) passed the previous barrier
        st16(wt[buf] + sr * RS + sc, wv);
        const bf16x8 a = as_bf16x8(av);
        if (st + 1 < NSTEP) {
            wv = wload(st + 1);
            av = aload(st + 1);
        }
        lds_barrier();
        uint2 lo[4], hi[4];
#pragma unroll
        for (int nt = 0; nt < 4; nt++) {
            lo[nt] = ld_tr16(wt[buf] + (8 * lg + trow) * RS + 16 * nt + tcol);
            hi[nt] = ld_tr16(wt[buf] + (8 * lg + 4 + trow) * RS + 16 * nt + tcol);
        }
#pragma unroll
        for (int nt = 0; nt < 4; nt++)
            acc[nt] = mfma16(a, as_bf16x8(u32x4{lo[nt].x, lo[nt].y, hi[nt].x, hi[nt].y}), acc[nt]);
    }
    // C[i = group][j = column]: lane j + 16 (i / 4), element i % 4
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
        const int n = n0 + 16 * nt + li, u = n / DIM, e = n % DIM;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int tok = 16 * (m0 + 16 * wave + 4 * lg + r) + u;
            if (tok < T) {
                const long o = ((long)bh * T + tok) * DIM + e;
                dx[o] = f2bf(raw[o] + acc[nt][r]);
            }
        }
    }
}

template <int DK, int DV>
hipError_t launch_cmp_dims(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    hipLaunchKernelGGL((k_bwd_keys_mfma<DK, DV, true>), dim3(d.npad / 64, A.nchunk, d.B * d.Hkv), dim3(kKThreads), 0,
                       s, A);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int BH = d.B * d.Hkv;
    hipLaunchKernelGGL((k_bwd_keys_mfma<DK, DV, false>), dim3(d.nb, A.nkc, BH), dim3(kKThreads), 0, s, A);
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

hipError_t launch_bwd_rows_mfma(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const dim3 grid((d.T + kThreads / 64 - 1) / (kThreads / 64), d.Hkv, d.B);
    if (A.lse_sv) {
        if (d.dk == 192) hipLaunchKernelGGL((k_bwd_rows_mfma<192, 128, true>), grid, dim3(kThreads), 0, s, A);
        else if (d.dk == 128) hipLaunchKernelGGL((k_bwd_rows_mfma<128, 128, true>), grid, dim3(kThreads), 0, s, A);
        else hipLaunchKernelGGL((k_bwd_rows_mfma<64, 64, true>), grid, dim3(kThreads), 0, s, A);
    } else {
        if (d.dk == 192) hipLaunchKernelGGL((k_bwd_rows_mfma<192, 128, false>), grid, dim3(kThreads), 0, s, A);
        else if (d.dk == 128) hipLaunchKernelGGL((k_bwd_rows_mfma<128, 128, false>), grid, dim3(kThreads), 0, s, A);
        else hipLaunchKernelGGL((k_bwd_rows_mfma<64, 64, false>), grid, dim3(kThreads), 0, s, A);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dx_mfma(const BwdArgs &A, bool isk, hipStream_t s)
{
    const Dims &d = A.d;
    const int dim = isk ? d.dk : d.dv;
    const float *G = A.kcv + (isk ? 0 : d.dk);
    const uint16_t *W = (const uint16_t *)(isk ? A.wck : A.wcv);
    const float *raw = isk ? A.dk_raw : A.dv_raw;
    uint16_t *dx = (uint16_t *)(isk ? A.dk : A.dv);
    const int gs = d.dk + d.dv;
    const dim3 grid(16 * dim / 64, ((d.T + 15) / 16 + 63) / 64, d.B * d.Hkv);
    if (dim == 192) hipLaunchKernelGGL(k_bwd_dx_mfma<192>, grid, dim3(kThreads), 0, s, G, gs, W, raw, dx, d.T, d.ncmp, d.npad);
    else if (dim == 128) hipLaunchKernelGGL(k_bwd_dx_mfma<128>, grid, dim3(kThreads), 0, s, G, gs, W, raw, dx, d.T, d.ncmp, d.npad);
    else hipLaunchKernelGGL(k_bwd_dx_mfma<64>, grid, dim3(kThreads), 0, s, G, gs, W, raw, dx, d.T, d.ncmp, d.npad);
    return hipGetLastError();
}

hipError_t launch_bwd_dw_mfma(const BwdArgs &A, bool isk, hipStream_t s)
{
    const Dims &d = A.d;
    const int dim = isk ? d.dk : d.dv;
    const float *G = A.kcv + (isk ? 0 : d.dk);
    const uint16_t *x = (const uint16_t *)(isk ? A.k : A.v), *pe = (const uint16_t *)(isk ? A.pek : A.pev);
    const float *cs = A.colsum + (isk ? 0 : d.dk);
    float *out = isk ? A.dwck : A.dwcv;
    const int rows = d.B * d.Hkv * d.ncmp;
    const dim3 grid(dim / 64, 32 * dim / 64);
    const int gs = d.dk + d.dv;
    if (dim == 192) hipLaunchKernelGGL(k_bwd_dw_mfma<192>, grid, dim3(kThreads), 0, s, G, gs, x, pe, cs, out, d.T, d.ncmp, d.npad, rows);
    else if (dim == 128) hipLaunchKernelGGL(k_bwd_dw_mfma<128>, grid, dim3(kThreads), 0, s, G, gs, x, pe, cs, out, d.T, d.ncmp, d.npad, rows);
    else hipLaunchKernelGGL(k_bwd_dw_mfma<64>, grid, dim3(kThreads), 0, s, G, gs, x, pe, cs, out, d.T, d.ncmp, d.npad, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_cmp_keys_mfma(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    if (d.dk == 192) return launch_cmp_dims<192, 128>(A, s);
    if (d.dk == 128) return launch_cmp_dims<128, 128>(A, s);
    return launch_cmp_dims<64, 64>(A, s);
}

}  // namespace nsa
