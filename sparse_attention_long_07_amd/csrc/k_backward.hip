// NSA backward pass: gradients of L = sum(dO * o) for every input of the
// forward pass, with the block selection held fixed (top-n is piecewise
// constant, so no gradient flows through the importance scores).  The
// sparsity is trained with the model (deepdaiv newsletter on DeepSeek's NSA,
// deepdaiv.stibee.com/p/82, on native trainability), which needs gradients
// through the three branches, the compression map and the gates.
//
// For one softmax branch with probabilities p over its keys, gated output
// gradient dO_c = gate_c * dO and D_c = dO_c . o_c:
//   dV_key += p dO_c,  ds = p (dO_c . V_key - D_c),
//   dq += scale ds K_key,  dK_key += scale ds q.
// Gate c of a head: dz_c = (dO . o_c) gate_c (1 - gate_c); dW_g += dz_c q,
// db_g += dz_c, dq += dz_c W_g.  Compression (K_cmp[i] = W vec(x[16i..16i+31]
// + PE)): dW = sum_i dK_cmp[i] (x_i + PE)^T, dPE = W^T sum_i dK_cmp[i] and
// token 16i + tau collects (W^T dK_cmp[i]) at slot tau.
//
// Passes, all plain VALU arithmetic in fp32 and free of float atomics, so the
// result is the same bit for bit on every run:
//  1. k_bwd_rows      one (position, KV head) per workgroup: recomputes the
//                     three branches (log-sum-exp, output), forms D, the gate
//                     terms and the complete dq; stores the per-row
//                     statistics for the key-side passes.
//  2. k_bwd_keys<raw> one 16-key tile per workgroup: dK, dV from the window
//                     rows and from every row whose selection holds the tile's
//                     block (found by scanning idx, in ascending row order).
//  3. k_bwd_keys<cmp> one 16-block tile of compressed keys per workgroup and
//                     row chunk; the chunk partials are summed in order.
//  4. tiled GEMMs     dW and the token gradient of the compression map; the
//                     token gradient is added to the raw-key gradient and
//                     written in the storage dtype.
//  5. gate reduction  dW_g and db_g, per row chunk, then summed in order.
#include "nsa_internal.h"

#include <math.h>

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kChunk = 64;       // keys per chunk of the row pass
constexpr int kKeyTile = 16;     // keys per workgroup of the key passes
constexpr int kRowChunk = 1024;  // rows per partial of the compressed-key gradient
constexpr int kGateRows = 256;   // rows per partial of the gate gradient
constexpr int kStat = 12;        // per (row, head): {lse, D, gate, dz} for each of the 3 branches

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------------------------
// Pass 1.  Per (b, t, g): for each branch (0 compressed, 1 selected, 2
// window) an online-softmax sweep gives the log-sum-exp and o_c, then a
// second sweep recomputes p and accumulates dq.  Key chunks as in the
// forward: compressed blocks [0, nvis) with 16i+31 <= t; the distinct valid
// selected blocks in ascending order, tokens <= t; the window [t-w+1, t].
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_rows(BwdArgs a)
{
    extern __shared__ float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv;
    float *qs = smem;              // [G][dk]
    float *dos = qs + G * dk;      // [G][dv]  output gradient (not gated)
    float *sb = dos + G * dv;      // [G][64]  logits, then probabilities, then ds
    float *ob = sb + G * kChunk;   // [G][dv]  branch output
    __shared__ float m_s[16], l_s[16], al_s[16], lse_s[16], D_s[16], gate_s[48], dz_s[48];
    __shared__ int blk[64];
    __shared__ int nblk_s;

    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int jcur = t / 64;
    const long row0 = ((long)b * d.T + t) * d.Hq + (long)g * G;   // first head of the group
    const T *qrow = (const T *)a.q + row0 * dk;
    const T *dorow = (const T *)a.dO + row0 * dv;
    for (int e = tid; e < G * dk; e += kThreads) qs[e] = to_f(qrow[e]);
    for (int e = tid; e < G * dv; e += kThreads) dos[e] = to_f(dorow[e]);
    if (tid == 0) {
        const int32_t *ir = a.idx + (((long)b * d.Hkv + g) * d.T + t) * d.n;
        int m = 0;
        for (int q2 = 0; q2 < d.n; q2++) {
            int j = ir[q2];
            if (j < 0 || j > jcur) continue;
            bool dup = false;
            for (int u = 0; u < m; u++) dup |= blk[u] == j;
            if (dup) continue;
            int pos = m;
            while (pos > 0 && blk[pos - 1] > j) {
                blk[pos] = blk[pos - 1];
                pos--;
            }
            blk[pos] = j;
            m++;
        }
        nblk_s = m;
    }
    __syncthreads();
    if (tid < 3 * G) {
        const int h = tid / 3, c = tid % 3;
        const T *wr = (const T *)a.wg + (((long)g * G + h) * 3 + c) * dk;
        float z = to_f(((const T *)a.bg)[((long)g * G + h) * 3 + c]);
        for (int x = 0; x < dk; x++) z += to_f(wr[x]) * qs[h * dk + x];
        gate_s[tid] = 1.f / (1.f + __expf(-z));
    }
    __syncthreads();

    const long bgi = (long)b * d.Hkv + g;
    const T *Kr = (const T *)a.k + bgi * d.T * dk;
    const T *Vr = (const T *)a.v + bgi * d.T * dv;
    const T *Kc = (const T *)a.kc + bgi * d.npad * dk;
    const T *Vc = (const T *)a.vc + bgi * d.npad * dv;
    const int nvis = t >= 31 ? (t - 31) / 16 + 1 : 0;
    const int lo = t - d.w + 1 > 0 ? t - d.w + 1 : 0;
    const int nq = (G * dk + kThreads - 1) / kThreads;
    const int no = (G * dv + kThreads - 1) / kThreads;
    float dq[16];
#pragma unroll
    for (int u = 0; u < 16; u++) dq[u] = 0.f;

    for (int br = 0; br < 3; br++) {
        const T *K = br == 0 ? Kc : Kr;
        const T *V = br == 0 ? Vc : Vr;
        const int nch = br == 0 ? (nvis + kChunk - 1) / kChunk : br == 1 ? nblk_s : (t - lo + kChunk) / kChunk;
        auto chunk = [&](int ch, int &key0, int &lim) {
            if (br == 0) {
                key0 = ch * kChunk;
                lim = min(kChunk, nvis - key0);
            } else {
                key0 = br == 1 ? blk[ch] * 64 : lo + ch * kChunk;
                lim = min(kChunk, t - key0 + 1);
            }
        };
        // sweep 1: log-sum-exp and output of the branch
        float acc[16];
#pragma unroll
        for (int u = 0; u < 16; u++) acc[u] = 0.f;
        if (tid < 16) {
            m_s[tid] = -INFINITY;
            l_s[tid] = 0.f;
        }
        __syncthreads();
        for (int ch = 0; ch < nch; ch++) {
            int key0, lim;
            chunk(ch, key0, lim);
            for (int e = tid; e < G * kChunk; e += kThreads) {
                const int h = e / kChunk, ii = e % kChunk;
                float s = -INFINITY;
                if (ii < lim) {
                    const T *kr = K + (long)(key0 + ii) * dk;
                    float z = 0.f;
                    for (int x = 0; x < dk; x++) z += qs[h * dk + x] * to_f(kr[x]);
                    s = z * d.scale;
                }
                sb[e] = s;
            }
            __syncthreads();
            for (int h = wave; h < G; h += kThreads / kWave) {
                const float v = sb[h * kChunk + lane];
                const float mo = m_s[h];
                const float mn = fmaxf(mo, wave_max(v));
                const float p = __expf(v - mn);
                sb[h * kChunk + lane] = p;
                const float sum = wave_sum(p);
                if (lane == 0) {
                    const float al = __expf(mo - mn);
                    l_s[h] = l_s[h] * al + sum;
                    m_s[h] = mn;
                    al_s[h] = al;
                }
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int e = tid + u * kThreads;
                if (u < no && e < G * dv) {
                    const int h = e / dv, c = e % dv;
                    float z = acc[u] * al_s[h];
                    for (int ii = 0; ii < lim; ii++) z += sb[h * kChunk + ii] * to_f(V[(long)(key0 + ii) * dv + c]);
                    acc[u] = z;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < 16; u++) {
            const int e = tid + u * kThreads;
            if (u < no && e < G * dv) {
                const int h = e / dv;
                ob[e] = l_s[h] > 0.f ? acc[u] / l_s[h] : 0.f;
            }
        }
        if (tid < G) lse_s[tid] = l_s[tid] > 0.f ? m_s[tid] + __logf(l_s[tid]) : -INFINITY;
        __syncthreads();
        // D_c = gate_c dO . o_c and the gate's logit gradient
        for (int h = wave; h < G; h += kThreads / kWave) {
            float x = 0.f;
            for (int c = lane; c < dv; c += kWave) x += dos[h * dv + c] * ob[h * dv + c];
            const float dg = wave_sum(x);
            if (lane == 0) {
                const float gv = gate_s[h * 3 + br];
                dz_s[h * 3 + br] = dg * gv * (1.f - gv);
                D_s[h] = gv * dg;
            }
        }
        __syncthreads();
        // sweep 2: ds and dq
        for (int ch = 0; ch < nch; ch++) {
            int key0, lim;
            chunk(ch, key0, lim);
            for (int e = tid; e < G * kChunk; e += kThreads) {
                const int h = e / kChunk, ii = e % kChunk;
                float ds = 0.f;
                if (ii < lim) {
                    const T *kr = K + (long)(key0 + ii) * dk;
                    const T *vr = V + (long)(key0 + ii) * dv;
                    float z = 0.f, y = 0.f;
                    for (int x = 0; x < dk; x++) z += qs[h * dk + x] * to_f(kr[x]);
                    for (int c = 0; c < dv; c++) y += dos[h * dv + c] * to_f(vr[c]);
                    const float p = __expf(z * d.scale - lse_s[h]);
                    ds = p * (gate_s[h * 3 + br] * y - D_s[h]);
                }
                sb[e] = ds;
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int e = tid + u * kThreads;
                if (u < nq && e < G * dk) {
                    const int h = e / dk, x = e % dk;
                    float z = 0.f;
                    for (int ii = 0; ii < lim; ii++) z += sb[h * kChunk + ii] * to_f(K[(long)(key0 + ii) * dk + x]);
                    dq[u] += d.scale * z;
                }
            }
            __syncthreads();
        }
        if (tid < G) {
            float *st = a.rs + (row0 + tid) * kStat + br * 4;
            st[0] = lse_s[tid];
            st[1] = D_s[tid];
            st[2] = gate_s[tid * 3 + br];
            st[3] = dz_s[tid * 3 + br];
        }
        __syncthreads();
    }
    T *dqrow = (T *)a.dq + row0 * dk;
#pragma unroll
    for (int u = 0; u < 16; u++) {
        const int e = tid + u * kThreads;
        if (u < nq && e < G * dk) {
            const int h = e / dk, x = e % dk;
            float z = dq[u];
            for (int c = 0; c < 3; c++)
                z += dz_s[h * 3 + c] * to_f(((const T *)a.wg)[(((long)g * G + h) * 3 + c) * dk + x]);
            dqrow[e] = from_f<T>(z);
        }
    }
}

// ---------------------------------------------------------------------------
// Passes 2 and 3.  A workgroup owns kKeyTile consecutive keys of one (b, g):
// raw tokens (CMP = false) or compressed blocks (CMP = true).  Keys and values
// sit in LDS; the rows that attend to them are visited one at a time, all G
// heads of a row together.  Thread (key = tid % 16, h = tid / 16) forms p and
// ds of head h; then thread (key, part = tid / 16) adds every head's
// contribution to the columns part, part + 16, ... of dK and dV.
template <typename T, bool CMP>
__global__ __launch_bounds__(kThreads) void k_bwd_keys(BwdArgs a)
{
    extern __shared__ float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv, KS = dk + 1, VS = dv + 1;
    float *Ks = smem;                  // [16][dk+1]
    float *Vs = Ks + kKeyTile * KS;    // [16][dv+1]
    float *qs = Vs + kKeyTile * VS;    // [G][dk]
    float *dos = qs + G * dk;          // [G][dv]
    float *ps = dos + G * dv;          // [G][16]  gate * p
    float *dss = ps + G * kKeyTile;    // [G][16]  scale * ds
    __shared__ float st_lse[16], st_D[16], st_g[16];
    __shared__ int rowlist[kThreads];
    __shared__ int wcount[kThreads / kWave];

    const int tid = threadIdx.x;
    const int bgi = blockIdx.z;                       // b * Hkv + g
    const int b = bgi / d.Hkv, g = bgi % d.Hkv;
    const int key0 = blockIdx.x * kKeyTile;
    const int nkeys = CMP ? d.ncmp : d.T;
    const T *K = CMP ? (const T *)a.kc + (long)bgi * d.npad * dk : (const T *)a.k + (long)bgi * d.T * dk;
    const T *V = CMP ? (const T *)a.vc + (long)bgi * d.npad * dv : (const T *)a.v + (long)bgi * d.T * dv;
    for (int e = tid; e < kKeyTile * dk; e += kThreads) {
        const int r = e / dk, x = e % dk;
        Ks[r * KS + x] = key0 + r < nkeys ? to_f(K[(long)(key0 + r) * dk + x]) : 0.f;
    }
    for (int e = tid; e < kKeyTile * dv; e += kThreads) {
        const int r = e / dv, c = e % dv;
        Vs[r * VS + c] = key0 + r < nkeys ? to_f(V[(long)(key0 + r) * dv + c]) : 0.f;
    }
    const int key = tid % kKeyTile, part = tid / kKeyTile;   // part in 0..15, also the head of the p/ds step
    const int kk = key0 + key;
    const int ndk = dk / 16 + (part < dk % 16), ndv = dv / 16 + (part < dv % 16);
    float adk[16], adv[16];
#pragma unroll
    for (int u = 0; u < 16; u++) adk[u] = adv[u] = 0.f;

    // One attending row t of branch br: every thread calls this together.
    auto row = [&](int t, int br) {
        const long row0 = ((long)b * d.T + t) * d.Hq + (long)g * G;
        const T *qrow = (const T *)a.q + row0 * dk;
        const T *dorow = (const T *)a.dO + row0 * dv;
        for (int e = tid; e < G * dk; e += kThreads) qs[e] = to_f(qrow[e]);
        for (int e = tid; e < G * dv; e += kThreads) dos[e] = to_f(dorow[e]);
        if (tid < G) {
            const float *st = a.rs + (row0 + tid) * kStat + br * 4;
            st_lse[tid] = st[0];
            st_D[tid] = st[1];
            st_g[tid] = st[2];
        }
        __syncthreads();
        bool vis;
        if (CMP) vis = kk < d.ncmp && 16 * kk + 31 <= t;
        else vis = kk <= t && (br == 1 || kk >= t - d.w + 1);
        const int h = part;
        if (h < G) {
            float p = 0.f, ds = 0.f;
            if (vis) {
                float z = 0.f, y = 0.f;
                for (int x = 0; x < dk; x++) z += qs[h * dk + x] * Ks[key * KS + x];
                for (int c = 0; c < dv; c++) y += dos[h * dv + c] * Vs[key * VS + c];
                const float gv = st_g[h];
                p = __expf(z * d.scale - st_lse[h]);
                ds = p * (gv * y - st_D[h]);
                p *= gv;
            }
            ps[h * kKeyTile + key] = p;
            dss[h * kKeyTile + key] = ds * d.scale;
        }
        __syncthreads();
        for (int hh = 0; hh < G; hh++) {
            const float pk = ps[hh * kKeyTile + key], sk = dss[hh * kKeyTile + key];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u < ndv) adv[u] += pk * dos[hh * dv + part + 16 * u];
                if (u < ndk) adk[u] += sk * qs[hh * dk + part + 16 * u];
            }
        }
        __syncthreads();
    };

    if (CMP) {
        const int chunk = blockIdx.y;
        const int t_lo = max(chunk * kRowChunk, 16 * key0 + 31), t_hi = min(d.T, (chunk + 1) * kRowChunk);
        for (int t = t_lo; t < t_hi; t++) row(t, 0);
        if (kk < d.npad) {
            float *out = a.part + (((long)chunk * d.B * d.Hkv + bgi) * d.npad + kk) * (dk + dv);
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u < ndk) out[part + 16 * u] = adk[u];
                if (u < ndv) out[dk + part + 16 * u] = adv[u];
            }
        }
    } else {
        // window rows: the tile's keys are in the window of t for t in [key0, key0+15+w-1]
        const int whi = min(d.T - 1, key0 + kKeyTile - 1 + d.w - 1);
        for (int t = key0; t <= whi; t++) row(t, 2);
        // selected rows: t >= key0 whose list holds the tile's block
        const int jb = key0 / 64;
        const int32_t *ib = a.idx + (long)bgi * d.T * d.n;
        const int wv = tid / kWave, ln = tid % kWave;
        for (int base = key0; base < d.T; base += kThreads) {
            const int t = base + tid;
            bool mem = false;
            if (t < d.T)
                for (int u = 0; u < d.n; u++) mem |= ib[(long)t * d.n + u] == jb;
            const unsigned long long bal = __ballot(mem);
            if (ln == 0) wcount[wv] = __popcll(bal);
            __syncthreads();
            int off = 0, cnt = 0;
            for (int w2 = 0; w2 < kThreads / kWave; w2++) {
                off += w2 < wv ? wcount[w2] : 0;
                cnt += wcount[w2];
            }
            if (mem) rowlist[off + __popcll(bal & ((1ull << ln) - 1ull))] = t;
            __syncthreads();
            for (int r = 0; r < cnt; r++) row(rowlist[r], 1);
            __syncthreads();
        }
        if (kk < d.T) {
            float *ok = a.dk_raw + ((long)bgi * d.T + kk) * dk;
            float *ov = a.dv_raw + ((long)bgi * d.T + kk) * dv;
#pragma unroll
            for (int u = 0; u < 16; u++) {
                if (u < ndk) ok[part + 16 * u] = adk[u];
                if (u < ndv) ov[part + 16 * u] = adv[u];
            }
        }
    }
}

// Sum of the compressed K/V gradient partials over row chunks, in order.
__global__ __launch_bounds__(kThreads) void k_bwd_sum_parts(BwdArgs a)
{
    const Dims &d = a.d;
    const long n = (long)d.B * d.Hkv * d.npad * (d.dk + d.dv);
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;
    if (e >= n) return;
    float s = 0.f;
    for (int c = 0; c < a.nchunk; c++) s += a.part[(long)c * n + e];
    a.kcv[e] = s;
}

// colsum[c] = sum over sequences, KV heads and complete blocks of kcv[..][c].
__global__ __launch_bounds__(kThreads) void k_bwd_colsum(BwdArgs a)
{
    const Dims &d = a.d;
    const int W = d.dk + d.dv;
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= W) return;
    float s = 0.f;
    for (int bh = 0; bh < d.B * d.Hkv; bh++)
        for (int i = 0; i < d.ncmp; i++) s += a.kcv[((long)bh * d.npad + i) * W + c];
    a.colsum[c] = s;
}

// dPE[m] = sum_c W[c][m] colsum[c] for the K map (m < 32 dk) and the V map.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_dpe(BwdArgs a)
{
    const Dims &d = a.d;
    const int m = blockIdx.x * kThreads + threadIdx.x;
    const bool isk = blockIdx.y == 0;
    const int dim = isk ? d.dk : d.dv;
    if (m >= 32 * dim) return;
    const T *W = (const T *)(isk ? a.wck : a.wcv);
    const float *cs = a.colsum + (isk ? 0 : d.dk);
    float s = 0.f;
    for (int c = 0; c < dim; c++) s += to_f(W[(long)c * 32 * dim + m]) * cs[c];
    (isk ? a.dpek : a.dpev)[m] = s;
}

// ---------------------------------------------------------------------------
// Tiled fp32 product C[m][n] = sum_k A(m, k) B(k, n) over a 64 x 64 tile,
// 16-deep steps through LDS, a 4 x 4 patch per thread.  The problem type
// supplies the operand reads and the store; blockIdx.z selects a batch item.
template <class P>
__global__ __launch_bounds__(kThreads) void k_gemm(P p)
{
    __shared__ float As[16][68];
    __shared__ float Bs[16][68];
    const int z = blockIdx.z, m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += 16) {
        for (int e = tid; e < 16 * 64; e += kThreads) {
            const int kq = e / 64, r = e % 64;
            const bool kin = k0 + kq < p.K;
            As[kq][r] = kin && m0 + r < p.M ? p.a(z, m0 + r, k0 + kq) : 0.f;
            Bs[kq][r] = kin && n0 + r < p.N ? p.b(z, k0 + kq, n0 + r) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 16; kq++) {
            float x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                x[u] = As[kq][ty * 4 + u];
                y[u] = Bs[kq][tx * 4 + u];
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int w = 0; w < 4; w++) acc[u][w] += x[u] * y[w];
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const int m = m0 + ty * 4 + u, n = n0 + tx * 4 + w;
            if (m < p.M && n < p.N) p.store(z, m, n, acc[u][w]);
        }
}

// dW[c][mm] = sum over (bh, i < ncmp) of G[bh][i][c] (x[bh][16 i + mm/dim][mm%dim] + PE[mm]):
// M = dim, N = 32 dim, K = B*Hkv*ncmp.
template <typename T>
struct DwProblem {
    int M, N, K;
    const float *G;   // kcv with column offset applied
    int gs;           // row stride of kcv (dk + dv)
    const T *x, *pe;
    int T_, dim, ncmp, npad;
    float *out;
    __device__ float a(int, int m, int k) const
    {
        const int bh = k / ncmp, i = k % ncmp;
        return G[((long)bh * npad + i) * gs + m];
    }
    __device__ float b(int, int k, int n) const
    {
        const int bh = k / ncmp, i = k % ncmp;
        return to_f(x[((long)bh * T_ + 16L * i) * dim + n]) + to_f(pe[n]);
    }
    __device__ void store(int, int m, int n, float v) const { out[(long)m * N + n] = v; }
};

// Token gradient of the compression map for sequence/head z, 16 tokens per
// row: token 16m + r lies in block m at slot r and in block m-1 at slot 16+r,
// so out[m][r dim + e] = sum_c G[m][c] W[c][r dim + e] + G[m-1][c] W[c][(16+r) dim + e]:
// M = ceil(T/16), N = 16 dim, K = 2 dim.  The store adds the raw-key gradient
// and writes the storage dtype.
template <typename T>
struct DxProblem {
    int M, N, K;
    const float *G;
    int gs;
    const T *W;
    const float *raw;
    T *dx;
    int T_, dim, ncmp, npad;
    __device__ float a(int z, int m, int k) const
    {
        const int i = k < dim ? m : m - 1, c = k < dim ? k : k - dim;
        return i >= 0 && i < ncmp ? G[((long)z * npad + i) * gs + c] : 0.f;
    }
    __device__ float b(int, int k, int n) const
    {
        return k < dim ? to_f(W[(long)k * 32 * dim + n]) : to_f(W[(long)(k - dim) * 32 * dim + 16 * dim + n]);
    }
    __device__ void store(int z, int m, int n, float v) const
    {
        const int tok = 16 * m + n / dim, e = n % dim;
        if (tok < T_) {
            const long o = ((long)z * T_ + tok) * dim + e;
            dx[o] = from_f<T>(raw[o] + v);
        }
    }
};

// Gate gradients per chunk of kGateRows rows of one head: element e of
// [3][dk+1] (column dk is the bias) sums dz_c * q (or dz_c).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_gate_part(BwdArgs a)
{
    const Dims &d = a.d;
    const int h = blockIdx.x, chunk = blockIdx.y;
    const int W1 = d.dk + 1;
    const long r0 = (long)chunk * kGateRows, r1 = min((long)d.B * d.T, r0 + kGateRows);
    for (int e = threadIdx.x; e < 3 * W1; e += kThreads) {
        const int c = e / W1, x = e % W1;
        float s = 0.f;
        for (long r = r0; r < r1; r++) {
            const float dz = a.rs[(r * d.Hq + h) * kStat + c * 4 + 3];
            s += dz * (x < d.dk ? to_f(((const T *)a.q)[(r * d.Hq + h) * d.dk + x]) : 1.f);
        }
        a.gpart[((long)h * a.ngc + chunk) * 3 * W1 + e] = s;
    }
}

__global__ __launch_bounds__(kThreads) void k_bwd_gate_sum(BwdArgs a)
{
    const Dims &d = a.d;
    const int W1 = d.dk + 1;
    const long e = (long)blockIdx.x * kThreads + threadIdx.x;
    if (e >= (long)d.Hq * 3 * W1) return;
    const int h = (int)(e / (3 * W1)), j = (int)(e % (3 * W1)), c = j / W1, x = j % W1;
    float s = 0.f;
    for (int ch = 0; ch < a.ngc; ch++) s += a.gpart[((long)h * a.ngc + ch) * 3 * W1 + j];
    if (x < d.dk) a.dwg[((long)h * 3 + c) * d.dk + x] = s;
    else a.dbg[h * 3 + c] = s;
}

template <class K>
hipError_t set_lds(K kernel, size_t bytes)
{
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T>
hipError_t launch_all(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int BH = d.B * d.Hkv;
    hipError_t e;
    // 1. rows
    {
        const size_t lds = sizeof(float) * ((size_t)d.G * (d.dk + 2 * d.dv + kChunk));
        if ((e = set_lds(k_bwd_rows<T>, lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_bwd_rows<T>, dim3(d.T, d.Hkv, d.B), dim3(kThreads), lds, s, A);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t klds = sizeof(float) * ((size_t)kKeyTile * (d.dk + d.dv + 2) + (size_t)d.G * (d.dk + d.dv) +
                                         2 * (size_t)d.G * kKeyTile);
    // 2. raw keys
    if ((e = set_lds(k_bwd_keys<T, false>, klds)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_keys<T, false>), dim3((d.T + kKeyTile - 1) / kKeyTile, 1, BH), dim3(kThreads), klds,
                       s, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 3. compressed keys, then the sum over row chunks
    if ((e = set_lds(k_bwd_keys<T, true>, klds)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bwd_keys<T, true>), dim3(d.npad / kKeyTile, A.nchunk, BH), dim3(kThreads), klds, s, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        const long n = (long)BH * d.npad * (d.dk + d.dv);
        hipLaunchKernelGGL(k_bwd_sum_parts, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                           A);
        hipLaunchKernelGGL(k_bwd_colsum, dim3((d.dk + d.dv + kThreads - 1) / kThreads), dim3(kThreads), 0, s, A);
        hipLaunchKernelGGL(k_bwd_dpe<T>, dim3((32 * (d.dk > d.dv ? d.dk : d.dv) + kThreads - 1) / kThreads, 2),
                           dim3(kThreads), 0, s, A);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 4. compression map: weight gradients and token gradients
    for (int isk = 1; isk >= 0; isk--) {
        const int dim = isk ? d.dk : d.dv;
        DwProblem<T> pw;
        pw.M = dim;
        pw.N = 32 * dim;
        pw.K = BH * d.ncmp;
        pw.G = A.kcv + (isk ? 0 : d.dk);
        pw.gs = d.dk + d.dv;
        pw.x = (const T *)(isk ? A.k : A.v);
        pw.pe = (const T *)(isk ? A.pek : A.pev);
        pw.T_ = d.T;
        pw.dim = dim;
        pw.ncmp = d.ncmp;
        pw.npad = d.npad;
        pw.out = isk ? A.dwck : A.dwcv;
        hipLaunchKernelGGL(k_gemm<DwProblem<T>>, dim3((pw.M + 63) / 64, (pw.N + 63) / 64, 1), dim3(kThreads), 0, s,
                           pw);
        DxProblem<T> px;
        px.M = (d.T + 15) / 16;
        px.N = 16 * dim;
        px.K = 2 * dim;
        px.G = pw.G;
        px.gs = pw.gs;
        px.W = (const T *)(isk ? A.wck : A.wcv);
        px.raw = isk ? A.dk_raw : A.dv_raw;
        px.dx = (T *)(isk ? A.dk : A.dv);
        px.T_ = d.T;
        px.dim = dim;
        px.ncmp = d.ncmp;
        px.npad = d.npad;
        hipLaunchKernelGGL(k_gemm<DxProblem<T>>, dim3((px.M + 63) / 64, (px.N + 63) / 64, BH), dim3(kThreads), 0, s,
                           px);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 5. gates
    hipLaunchKernelGGL(k_bwd_gate_part<T>, dim3(d.Hq, A.ngc), dim3(kThreads), 0, s, A);
    {
        const long n = (long)d.Hq * 3 * (d.dk + 1);
        hipLaunchKernelGGL(k_bwd_gate_sum, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, A);
    }
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t backward_layout(const Dims &d, void *ws, BwdArgs *A)
{
    const int nchunk = (d.T + kRowChunk - 1) / kRowChunk;
    const int ngc = (int)(((long)d.B * d.T + kGateRows - 1) / kGateRows);
    const long BH = (long)d.B * d.Hkv;
    size_t off = 0;
    auto carve = [&](size_t floats) {
        size_t o = off;
        off = align256(off + sizeof(float) * floats);
        return o;
    };
    const size_t o_rs = carve((size_t)d.B * d.T * d.Hq * kStat);
    const size_t o_dkr = carve((size_t)BH * d.T * d.dk);
    const size_t o_dvr = carve((size_t)BH * d.T * d.dv);
    const size_t o_part = carve((size_t)nchunk * BH * d.npad * (d.dk + d.dv));
    const size_t o_kcv = carve((size_t)BH * d.npad * (d.dk + d.dv));
    const size_t o_cs = carve((size_t)(d.dk + d.dv));
    const size_t o_gp = carve((size_t)d.Hq * ngc * 3 * (d.dk + 1));
    if (ws && A) {
        char *w = (char *)ws;
        A->rs = (float *)(w + o_rs);
        A->dk_raw = (float *)(w + o_dkr);
        A->dv_raw = (float *)(w + o_dvr);
        A->part = (float *)(w + o_part);
        A->kcv = (float *)(w + o_kcv);
        A->colsum = (float *)(w + o_cs);
        A->gpart = (float *)(w + o_gp);
        A->nchunk = nchunk;
        A->ngc = ngc;
    }
    return off;
}

hipError_t launch_backward(const BwdArgs &A, hipStream_t s)
{
    if (A.d.dtype == NSA_FP32) return launch_all<float>(A, s);
    return launch_all<bf16_t>(A, s);
}

}  // namespace nsa
