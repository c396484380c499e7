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
// Passes, free of float atomics, so the result is the same bit for bit on
// every run.  For bf16 storage with 16 query heads per KV head and the
// forward's (d_k, d_v) pairs, passes 1-3 run on the matrix cores
// (k_backward_mfma.hip); every other shape takes the fp32 VALU kernels here:
//  1. k_bwd_rows      one (position, KV head) per workgroup: recomputes the
//                     three branches (log-sum-exp, output), forms D, the gate
//                     terms and the complete dq; stores the per-row
//                     statistics for the key-side passes.
//  2. k_bwd_keys_blk  one 64-key block per workgroup: dK, dV from the window
//                     rows and then from every row whose selection holds the
//                     block, in ascending row order, read from a bitmap of
//                     (block, row) pairs built by k_bwd_selmap (integer OR, so
//                     the bitmap does not depend on the order of the writes).
//  3. k_bwd_keys_cmp  one 16-block tile of compressed keys per workgroup and
//                     row chunk; the chunk partials are summed in order.
//  4. tiled GEMMs     dW and the token gradient of the compression map; the
//                     token gradient is added to the raw-key gradient and
//                     written in the storage dtype.
//  5. gate reduction  dW_g and db_g, per row chunk, then summed in order.
#include "nsa_internal.h"

#include <math.h>

#include <algorithm>

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kChunk = 64;       // keys per chunk of the row pass
constexpr int kKeyTile = 16;     // compressed blocks per workgroup of pass 3
constexpr int kRowChunk = kBwdRowChunk;  // rows per partial of the compressed-key gradient
constexpr int kGateRows = 256;   // rows per partial of the gate gradient
constexpr size_t kLdsBytes = 160 * 1024;   // LDS of one workgroup on gfx950
constexpr int kStat = kBwdStat;  // per (row, head): {lse, D, gate, dz} for each of the 3 branches

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

// LDS row stride (elements) of a staged key or value row: rows start on
// 16-byte boundaries, and for widths that are multiples of 64 the stride is
// 4 words past a multiple of 32, so 8 lanes reading 16 bytes of 8 different
// rows at the same column cover all 32 banks once.
template <typename T> constexpr int stage_stride(int dim) { return sizeof(T) == 2 ? dim + 8 : dim + 4; }

// sum_x a[x] * r[x] over n elements (n a multiple of 8; a and r 16-byte
// aligned): 16-byte reads, two accumulators
__device__ __forceinline__ float dot_staged(const float *a, const bf16_t *r, int n)
{
    float z0 = 0.f, z1 = 0.f;
#pragma unroll 4
    for (int x = 0; x < n; x += 8) {
        const uint4 w = *(const uint4 *)(r + x);
        const float4 a0 = *(const float4 *)(a + x), a1 = *(const float4 *)(a + x + 4);
        z0 = __builtin_fmaf(a0.x, __uint_as_float(w.x << 16), z0);
        z1 = __builtin_fmaf(a0.y, __uint_as_float(w.x & 0xffff0000u), z1);
        z0 = __builtin_fmaf(a0.z, __uint_as_float(w.y << 16), z0);
        z1 = __builtin_fmaf(a0.w, __uint_as_float(w.y & 0xffff0000u), z1);
        z0 = __builtin_fmaf(a1.x, __uint_as_float(w.z << 16), z0);
        z1 = __builtin_fmaf(a1.y, __uint_as_float(w.z & 0xffff0000u), z1);
        z0 = __builtin_fmaf(a1.z, __uint_as_float(w.w << 16), z0);
        z1 = __builtin_fmaf(a1.w, __uint_as_float(w.w & 0xffff0000u), z1);
    }
    return z0 + z1;
}
__device__ __forceinline__ float dot_staged(const float *a, const float *r, int n)
{
    float z0 = 0.f, z1 = 0.f;
#pragma unroll 4
    for (int x = 0; x < n; x += 8) {
        const float4 r0 = *(const float4 *)(r + x), r1 = *(const float4 *)(r + x + 4);
        const float4 a0 = *(const float4 *)(a + x), a1 = *(const float4 *)(a + x + 4);
        z0 = __builtin_fmaf(a0.x, r0.x, z0);
        z1 = __builtin_fmaf(a0.y, r0.y, z1);
        z0 = __builtin_fmaf(a0.z, r0.z, z0);
        z1 = __builtin_fmaf(a0.w, r0.w, z1);
        z0 = __builtin_fmaf(a1.x, r1.x, z0);
        z1 = __builtin_fmaf(a1.y, r1.y, z1);
        z0 = __builtin_fmaf(a1.z, r1.z, z0);
        z1 = __builtin_fmaf(a1.w, r1.w, z1);
    }
    return z0 + z1;
}

// rows key0 .. key0+lim-1 of src ([key][dim]) into dst with stride ds; 16-byte
// global loads (dim is a multiple of 8 and rows are 16-byte aligned)
template <typename T>
__device__ __forceinline__ void stage_rows(T *dst, int ds, const T *src, int key0, int lim, int dim)
{
    constexpr int PER = 16 / sizeof(T);
    const int cpr = dim / PER;   // 16-byte pieces per row
    for (int e = threadIdx.x; e < lim * cpr; e += kThreads) {
        const int r = e / cpr, c = e % cpr;
        *(uint4 *)(dst + r * ds + c * PER) = *(const uint4 *)(src + (long)(key0 + r) * dim + c * PER);
    }
}

// ---------------------------------------------------------------------------
// Pass 1.  Per (b, t, g): for each branch (0 compressed, 1 selected, 2
// window) an online-softmax sweep gives the log-sum-exp and o_c, then a
// second sweep recomputes p and accumulates dq.  Key chunks as in the
// forward: compressed blocks [0, nvis) with 16i+31 <= t; the distinct valid
// selected blocks in ascending order, tokens <= t; the window [t-w+1, t].
template <typename T, bool STAGED>
__global__ __launch_bounds__(kThreads) void k_bwd_rows(BwdArgs a)
{
    extern __shared__ __align__(16) float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv;
    const int KSt = stage_stride<T>(dk), VSt = stage_stride<T>(dv);
    float *qs = smem;              // [G][dk]
    float *dos = qs + G * dk;      // [G][dv]  output gradient (not gated)
    float *sb = dos + G * dv;      // [G][64]  logits, then probabilities, then ds
    float *ob = sb + G * kChunk;   // [G][dv]  branch output
    T *Ks = (T *)(ob + G * dv);    // [64][KSt] the chunk's keys, staged once for all heads (STAGED)
    T *Vs = Ks + kChunk * KSt;     // [64][VSt] and values
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
    // the chunk's K and V rows: staged in LDS, or read in place when the
    // staging buffers would not fit (fp32 with wide heads)
    auto chunk_rows = [&](const T *K, const T *V, int key0, int lim, const T *&Kx, const T *&Vx, int &kst, int &vst) {
        if constexpr (STAGED) {
            stage_rows<T>(Ks, KSt, K, key0, lim, dk);
            stage_rows<T>(Vs, VSt, V, key0, lim, dv);
            Kx = Ks;
            Vx = Vs;
            kst = KSt;
            vst = VSt;
        } else {
            Kx = K + (long)key0 * dk;
            Vx = V + (long)key0 * dv;
            kst = dk;
            vst = dv;
        }
    };
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
            const T *Kx, *Vx;
            int kst, vst;
            chunk_rows(K, V, key0, lim, Kx, Vx, kst, vst);
            __syncthreads();
            for (int e = tid; e < G * kChunk; e += kThreads) {
                const int h = e / kChunk, ii = e % kChunk;
                sb[e] = ii < lim ? dot_staged(qs + h * dk, Kx + ii * kst, dk) * d.scale : -INFINITY;
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
                    for (int ii = 0; ii < lim; ii++) z += sb[h * kChunk + ii] * to_f(Vx[ii * vst + c]);
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
            const T *Kx, *Vx;
            int kst, vst;
            chunk_rows(K, V, key0, lim, Kx, Vx, kst, vst);
            __syncthreads();
            for (int e = tid; e < G * kChunk; e += kThreads) {
                const int h = e / kChunk, ii = e % kChunk;
                float ds = 0.f;
                if (ii < lim) {
                    const float z = dot_staged(qs + h * dk, Kx + ii * kst, dk);
                    const float y = dot_staged(dos + h * dv, Vx + ii * vst, dv);
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
                    for (int ii = 0; ii < lim; ii++) z += sb[h * kChunk + ii] * to_f(Kx[ii * kst + x]);
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
// Pass 3.  A workgroup owns kKeyTile consecutive compressed blocks of one
// (b, g) and one chunk of kRowChunk rows.  Keys and values sit in LDS; the
// rows that attend to them are visited one at a time, all G heads of a row
// together.  Thread (key = tid % 16, h = tid / 16) forms p and
// ds of head h; then thread (key, part = tid / 16) adds every head's
// contribution to the columns part, part + 16, ... of dK and dV.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_keys_cmp(BwdArgs a)
{
    extern __shared__ __align__(16) float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv, KS = dk + 1, VS = dv + 1;
    float *Ks = smem;                  // [16][dk+1]
    float *Vs = Ks + kKeyTile * KS;    // [16][dv+1]
    float *qs = Vs + kKeyTile * VS;    // [G][dk]
    float *dos = qs + G * dk;          // [G][dv]
    float *ps = dos + G * dv;          // [G][16]  gate * p
    float *dss = ps + G * kKeyTile;    // [G][16]  scale * ds
    __shared__ float st_lse[16], st_D[16], st_g[16];

    const int tid = threadIdx.x;
    const int bgi = blockIdx.z;                       // b * Hkv + g
    const int b = bgi / d.Hkv, g = bgi % d.Hkv;
    const int key0 = blockIdx.x * kKeyTile;
    const int nkeys = d.ncmp;
    const T *K = (const T *)a.kc + (long)bgi * d.npad * dk;
    const T *V = (const T *)a.vc + (long)bgi * d.npad * dv;
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

    // One attending row t: every thread calls this together.
    auto row = [&](int t) {
        const long row0 = ((long)b * d.T + t) * d.Hq + (long)g * G;
        const T *qrow = (const T *)a.q + row0 * dk;
        const T *dorow = (const T *)a.dO + row0 * dv;
        for (int e = tid; e < G * dk; e += kThreads) qs[e] = to_f(qrow[e]);
        for (int e = tid; e < G * dv; e += kThreads) dos[e] = to_f(dorow[e]);
        if (tid < G) {
            const float *st = a.rs + (row0 + tid) * kStat;   // branch 0
            st_lse[tid] = st[0];
            st_D[tid] = st[1];
            st_g[tid] = st[2];
        }
        __syncthreads();
        const bool vis = kk < d.ncmp && 16 * kk + 31 <= t;
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

    const int chunk = blockIdx.y;
    const int t_lo = max(chunk * kRowChunk, 16 * key0 + 31), t_hi = min(d.T, (chunk + 1) * kRowChunk);
    for (int t = t_lo; t < t_hi; t++) row(t);
    if (kk < d.npad) {
        float *out = a.part + (((long)chunk * d.B * d.Hkv + bgi) * d.npad + kk) * (dk + dv);
#pragma unroll
        for (int u = 0; u < 16; u++) {
            if (u < ndk) out[part + 16 * u] = adk[u];
            if (u < ndv) out[dk + part + 16 * u] = adv[u];
        }
    }
}

// Selection bitmap: bit t % 32 of word [bg][j][t / 32] is set when row t of
// (b, KV head) bg selected block j (only blocks j <= t / 64 count).
__global__ __launch_bounds__(kThreads) void k_bwd_fill_u32(uint32_t *p, long n)
{
    for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads) p[i] = 0u;
}

// The same bitmap for kThreads consecutive rows of one (b, KV head) per
// workgroup: the bits are gathered with LDS atomics, then every word of those
// rows is stored (zeros included), so no fill is needed.  nb * 8 words of LDS.
__global__ __launch_bounds__(kThreads) void k_bwd_selmap_lds(BwdArgs a)
{
    extern __shared__ uint32_t wbits[];   // [nb][kThreads / 32]
    constexpr int WPB = kThreads / 32;    // words of one block's bits in this workgroup
    const Dims &d = a.d;
    const int tid = threadIdx.x, t0 = blockIdx.x * kThreads, bgi = blockIdx.y;
    for (int i = tid; i < d.nb * WPB; i += kThreads) wbits[i] = 0u;
    __syncthreads();
    const int t = t0 + tid;
    if (t < d.T) {
        const int32_t *ir = a.idx + ((long)bgi * d.T + t) * d.n;
        for (int u = 0; u < d.n; u++) {
            const int j = ir[u];
            if (j >= 0 && j <= t / 64) atomicOr(&wbits[j * WPB + tid / 32], 1u << (tid & 31));
        }
    }
    __syncthreads();
    const int nw = (d.T + 31) / 32, w0 = t0 / 32, nwl = min(WPB, nw - w0);
    for (int i = tid; i < d.nb * WPB; i += kThreads) {
        const int j = i / WPB, wl = i % WPB;
        if (wl < nwl) a.selbm[((long)bgi * d.nb + j) * nw + w0 + wl] = wbits[i];
    }
}

__global__ __launch_bounds__(kThreads) void k_bwd_selmap(BwdArgs a)
{
    const Dims &d = a.d;
    const int t = blockIdx.x * kThreads + threadIdx.x, bgi = blockIdx.y;
    if (t >= d.T) return;
    const int nw = (d.T + 31) / 32;
    const int32_t *ir = a.idx + ((long)bgi * d.T + t) * d.n;
    for (int u = 0; u < d.n; u++) {
        const int j = ir[u];
        if (j >= 0 && j <= t / 64)
            atomicOr(a.selbm + ((long)bgi * d.nb + j) * nw + t / 32, 1u << (t & 31));
    }
}

// Raw-key gradients of one 64-key block (b, KV head, block jb).  K and V of
// the block are staged once; the rows that attend to it come in a fixed
// order: the window rows t = key0 .. key0+63+w-1, then the rows that selected
// the block, ascending.  Each row's q and dO are loaded one row ahead.  Thread
// (key = tid % 64, part = tid / 64) keeps dK, dV columns part, part+4, ...
template <typename T, bool STAGED>
__global__ __launch_bounds__(kThreads) void k_bwd_keys_blk(BwdArgs a)
{
    constexpr int kBK = 64;                       // keys per block
    constexpr int kMaxCols = 64;                  // dk / 4 and dv / 4 for d <= 256
    constexpr int PER = 16 / sizeof(T);           // elements per 16-byte load
    extern __shared__ __align__(16) float smem[];
    const Dims &d = a.d;
    const int G = d.G, dk = d.dk, dv = d.dv;
    const int KSt = stage_stride<T>(dk), VSt = stage_stride<T>(dv);
    float *qs = smem;                   // [G][dk]
    float *dos = qs + G * dk;           // [G][dv]
    float *ps = dos + G * dv;           // [G][64] gate * p
    float *dss = ps + G * kBK;          // [G][64] scale * ds
    T *Ks = (T *)(dss + G * kBK);       // [64][KSt] (STAGED)
    T *Vs = Ks + kBK * KSt;             // [64][VSt]
    __shared__ float st_lse[16], st_D[16], st_g[16];
    __shared__ uint16_t rows[kThreads * 32];  // selected rows of one bitmap chunk, less 32 * its first word
    __shared__ int wcnt[kThreads];
    __shared__ int nrows_s;

    const int tid = threadIdx.x, jb = blockIdx.x, bgi = blockIdx.y;
    const int b = bgi / d.Hkv, g = bgi % d.Hkv;
    const int key0 = jb * kBK, nk = min(kBK, d.T - key0);
    const T *K = (const T *)a.k + (long)bgi * d.T * dk;
    const T *V = (const T *)a.v + (long)bgi * d.T * dv;
    // the block's K and V rows: staged, or read in place when the staging
    // buffers would not fit (fp32 with wide heads)
    const T *Kx = K + (long)key0 * dk, *Vx = V + (long)key0 * dv;
    int kst = dk, vst = dv;
    if constexpr (STAGED) {
        stage_rows<T>(Ks, KSt, K, key0, nk, dk);
        stage_rows<T>(Vs, VSt, V, key0, nk, dv);
        Kx = Ks;
        Vx = Vs;
        kst = KSt;
        vst = VSt;
    }
    const int key = tid % kBK, part = tid / kBK, kk = key0 + key;
    // this thread's dK and dV columns: whole groups of 4 columns, the groups
    // split into 4 ranges (reads of q and dO are wave-uniform, 16 bytes)
    const int gk = (dk / 4 + 3) / 4, gv = (dv / 4 + 3) / 4;        // groups per part, at most 16
    const int ck0 = 4 * gk * part, cv0 = 4 * gv * part;              // first column
    const int nk4 = max(0, min(4 * gk, dk - ck0)), nv4 = max(0, min(4 * gv, dv - cv0));   // columns owned
    float adk[kMaxCols], adv[kMaxCols];
#pragma unroll
    for (int u = 0; u < kMaxCols; u++) adk[u] = adv[u] = 0.f;

    // q / dO of a row into registers (16-byte pieces; at most 4 per thread)
    const int qch = G * dk / PER, dch = G * dv / PER;
    uint4 qreg[4], dreg[4];
    float sreg[3];
    auto fetch = [&](int t, int br) {
        const long row0 = ((long)b * d.T + t) * d.Hq + (long)g * G;
        const T *qrow = (const T *)a.q + row0 * dk;
        const T *dorow = (const T *)a.dO + row0 * dv;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = tid + i * kThreads;
            if (c < qch) qreg[i] = *(const uint4 *)(qrow + (long)c * PER);
            if (c < dch) dreg[i] = *(const uint4 *)(dorow + (long)c * PER);
        }
        if (tid < G) {
            const float *st = a.rs + (row0 + tid) * kStat + br * 4;
            sreg[0] = st[0];
            sreg[1] = st[1];
            sreg[2] = st[2];
        }
    };
    auto unpack = [&](float *dst, const uint4 &v) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                dst[2 * e] = __uint_as_float(w[e] << 16);
                dst[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        } else {
            dst[0] = __uint_as_float(v.x);
            dst[1] = __uint_as_float(v.y);
            dst[2] = __uint_as_float(v.z);
            dst[3] = __uint_as_float(v.w);
        }
    };
    // one attending row, its q/dO already in registers; next = the row to
    // fetch meanwhile (t < 0: none)
    auto row = [&](int t, int br, int tn, int brn) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = tid + i * kThreads;
            if (c < qch) unpack(qs + c * PER, qreg[i]);
            if (c < dch) unpack(dos + c * PER, dreg[i]);
        }
        if (tid < G) {
            st_lse[tid] = sreg[0];
            st_D[tid] = sreg[1];
            st_g[tid] = sreg[2];
        }
        __syncthreads();
        if (tn >= 0) fetch(tn, brn);
        const bool vis = kk < d.T && kk <= t && (br == 1 || kk >= t - d.w + 1);
        for (int h = part; h < G; h += kThreads / kBK) {
            float p = 0.f, ds = 0.f;
            if (vis) {
                const float z = dot_staged(qs + h * dk, Kx + key * kst, dk);
                const float y = dot_staged(dos + h * dv, Vx + key * vst, dv);
                const float gv = st_g[h];
                p = __expf(z * d.scale - st_lse[h]);
                ds = p * (gv * y - st_D[h]);
                p *= gv;
            }
            ps[h * kBK + key] = p;
            dss[h * kBK + key] = ds * d.scale;
        }
        __syncthreads();
        for (int hh = 0; hh < G; hh++) {
            const float pk = ps[hh * kBK + key], sk = dss[hh * kBK + key];
            const float4 *dr = (const float4 *)(dos + hh * dv + cv0);
            const float4 *qr = (const float4 *)(qs + hh * dk + ck0);
#pragma unroll
            for (int u4 = 0; u4 < kMaxCols / 4; u4++) {
                if (4 * u4 < nv4) {
                    const float4 x = dr[u4];
                    adv[4 * u4] += pk * x.x;
                    adv[4 * u4 + 1] += pk * x.y;
                    adv[4 * u4 + 2] += pk * x.z;
                    adv[4 * u4 + 3] += pk * x.w;
                }
                if (4 * u4 < nk4) {
                    const float4 x = qr[u4];
                    adk[4 * u4] += sk * x.x;
                    adk[4 * u4 + 1] += sk * x.y;
                    adk[4 * u4 + 2] += sk * x.z;
                    adk[4 * u4 + 3] += sk * x.w;
                }
            }
        }
        __syncthreads();
    };

    // window rows
    const int whi = min(d.T - 1, key0 + kBK - 1 + d.w - 1);
    fetch(key0, 2);
    for (int t = key0; t <= whi; t++) row(t, 2, t < whi ? t + 1 : -1, 2);
    // selected rows, one bitmap chunk (kThreads words = 8192 rows) at a time
    const int nw = (d.T + 31) / 32;
    const uint32_t *bm = a.selbm + ((long)bgi * d.nb + jb) * nw;
    for (int w0 = key0 / 32; w0 < nw; w0 += kThreads) {
        const int w = w0 + tid;
        const uint32_t word = w < nw ? bm[w] : 0u;
        wcnt[tid] = __popc(word);
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int i = 0; i < kThreads; i++) {
                const int c = wcnt[i];
                wcnt[i] = acc;
                acc += c;
            }
            nrows_s = acc;
        }
        __syncthreads();
        {
            int o = wcnt[tid];
            for (uint32_t x = word; x; x &= x - 1) rows[o++] = (uint16_t)(32 * tid + __ffs(x) - 1);
        }
        __syncthreads();
        const int nr = nrows_s;
        const int tb = 32 * w0;
        if (nr > 0) fetch(tb + rows[0], 1);
        for (int r = 0; r < nr; r++) row(tb + rows[r], 1, r + 1 < nr ? tb + rows[r + 1] : -1, 1);
        __syncthreads();
    }
    if (kk < d.T) {
        float *ok = a.dk_raw + ((long)bgi * d.T + kk) * dk;
        float *ov = a.dv_raw + ((long)bgi * d.T + kk) * dv;
#pragma unroll
        for (int u4 = 0; u4 < kMaxCols / 4; u4++) {
            if (4 * u4 < nk4)
                *(float4 *)(ok + ck0 + 4 * u4) = make_float4(adk[4 * u4], adk[4 * u4 + 1], adk[4 * u4 + 2], adk[4 * u4 + 3]);
            if (4 * u4 < nv4)
                *(float4 *)(ov + cv0 + 4 * u4) = make_float4(adv[4 * u4], adv[4 * u4 + 1], adv[4 * u4 + 2], adv[4 * u4 + 3]);
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

// colsum[c] = sum over sequences, KV heads and complete blocks of kcv[..][c],
// in two fixed-order levels: workgroup (column group of 64, row chunk y of
// kColChunks) sums its chunk of the (b, head, block) rows, each wave a
// quarter of it in row order, the quarters in order; then the chunk
// partials are added in chunk order.
constexpr int kColChunks = 32;
__global__ __launch_bounds__(kThreads) void k_bwd_colsum_part(BwdArgs a)
{
    const Dims &d = a.d;
    const int W = d.dk + d.dv;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int c = blockIdx.x * kWave + lane;
    const long R = (long)d.B * d.Hkv * d.ncmp;   // rows r = bh * ncmp + i
    const long per = (R + kColChunks - 1) / kColChunks;
    const long r0 = blockIdx.y * per, r1 = r0 + per < R ? r0 + per : R;
    const long q = (r1 - r0 + 3) / 4;
    const long lo = r0 + wave * q, hi = lo + q < r1 ? lo + q : r1;
    float s = 0.f;
    if (c < W)
        for (long r = lo; r < hi; r++) s += a.kcv[((r / d.ncmp) * d.npad + r % d.ncmp) * W + c];
    __shared__ float ws[kThreads / kWave][kWave];
    ws[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && c < W) a.cspart[(long)blockIdx.y * W + c] = ((ws[0][lane] + ws[1][lane]) + ws[2][lane]) + ws[3][lane];
}
__global__ __launch_bounds__(kThreads) void k_bwd_colsum(BwdArgs a)
{
    const Dims &d = a.d;
    const int W = d.dk + d.dv;
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= W) return;
    float s = 0.f;
    for (int y = 0; y < kColChunks; y++) s += a.cspart[(long)y * W + c];
    a.colsum[c] = s;
}

// dPE[m] = sum_c W[c][m] colsum[c] for the K map (m < 32 dk) and the V map.
// A workgroup takes 64 columns m; wave w sums the channels c = w mod 4, and
// the four partial sums are added in wave order.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_dpe(BwdArgs a)
{
    __shared__ float part[kThreads / kWave][kWave];
    const Dims &d = a.d;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int m = blockIdx.x * kWave + lane;
    const bool isk = blockIdx.y == 0;
    const int dim = isk ? d.dk : d.dv;
    const T *W = (const T *)(isk ? a.wck : a.wcv);
    const float *cs = a.colsum + (isk ? 0 : d.dk);
    float s = 0.f;
    if (m < 32 * dim) {
#pragma unroll 8
        for (int c = wave; c < dim; c += kThreads / kWave) s += to_f(W[(long)c * 32 * dim + m]) * cs[c];
    }
    part[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && m < 32 * dim) {
        float t = part[0][lane];
        for (int w = 1; w < kThreads / kWave; w++) t += part[w][lane];
        (isk ? a.dpek : a.dpev)[m] = t;
    }
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

// Two-layer compression map, second layer (c = W2 max(h, 0)), backward.
// dW2[c][j] = sum over (bh, i < ncmp) of G[bh][i][c] max(h[bh][i][j], 0):
// M = N = dim, K = B*Hkv*ncmp.
template <typename T>
struct Dw2Problem {
    int M, N, K;
    const float *G;   // kcv with column offset applied
    int gs;
    const T *h;       // hidden layer [B*Hkv][npad][dim]
    int dim, ncmp, npad;
    float *out;
    __device__ float a(int, int m, int k) const
    {
        const int bh = k / ncmp, i = k % ncmp;
        return G[((long)bh * npad + i) * gs + m];
    }
    __device__ float b(int, int k, int n) const
    {
        const int bh = k / ncmp, i = k % ncmp;
        return fmaxf(to_f(h[((long)bh * npad + i) * dim + n]), 0.f);
    }
    __device__ void store(int, int m, int n, float v) const { out[(long)m * N + n] = v; }
};

// Dw2Problem with its contraction split into ranges of K rows: split z (the
// batch index of k_gemm) covers rows z K .. z K + K - 1 of the Ktot and writes
// its partial product to part[z]; k_sum_splits then adds the splits in order.
// (9 or 4 workgroups over 4,092 rows took 0.87 ms each at T=16384.)
template <typename T>
struct Dw2SplitProblem {
    int M, N, K, Ktot;
    Dw2Problem<T> base;
    float *part;   // [nsplit][M][N]
    __device__ float a(int z, int m, int k) const
    {
        const int kg = z * K + k;
        return kg < Ktot ? base.a(0, m, kg) : 0.f;
    }
    __device__ float b(int z, int k, int n) const
    {
        const int kg = z * K + k;
        return kg < Ktot ? base.b(0, kg, n) : 0.f;
    }
    __device__ void store(int z, int m, int n, float v) const { part[((long)z * M + m) * N + n] = v; }
};

__global__ __launch_bounds__(kThreads) void k_sum_splits(const float *__restrict__ part, int nsplit, long n,
                                                         float *__restrict__ out)
{
    const long i = (long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int z = 0; z < nsplit; z++) s += part[(long)z * n + i];
    out[i] = s;
}

// dA[z][i][j] = (sum_c G[z][i][c] W2[c][j]) [h[z][i][j] > 0] for sequence and
// head z (the ReLU's derivative taken as 0 at 0), rows i >= ncmp zero:
// M = npad, N = K = dim.  Written in kcv's layout (column offset applied).
template <typename T>
struct DaProblem {
    int M, N, K;
    const float *G;
    int gs;
    const T *W2, *h;
    float *da;
    int dim, ncmp, npad;
    __device__ float a(int z, int m, int k) const { return m < ncmp ? G[((long)z * npad + m) * gs + k] : 0.f; }
    __device__ float b(int, int k, int n) const { return to_f(W2[(long)k * dim + n]); }
    __device__ void store(int z, int m, int n, float v) const
    {
        const bool open = m < ncmp && to_f(h[((long)z * npad + m) * dim + n]) > 0.f;
        da[((long)z * npad + m) * gs + n] = open ? v : 0.f;
    }
};

// Gate gradients per chunk of kGateRows rows of one head: element e of
// [3][dk+1] (column dk is the bias) sums dz_c * q (or dz_c).  A thread owns 8
// consecutive columns (one 16-byte load of a bf16 row, two of an fp32 row) of
// every nrl-th row of the chunk, for all three branches; the row lanes' sums
// are then added in lane order through LDS, so the result does not depend on
// scheduling.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_gate_part(BwdArgs a)
{
    __shared__ float red[kThreads * 24];   // per thread: 3 branches x 8 columns
    __shared__ float bred[kThreads * 3];   // per row lane: 3 bias sums (threads of column group 0)
    const Dims &d = a.d;
    const int h = blockIdx.x, chunk = blockIdx.y;
    const int W1 = d.dk + 1;
    const int ncg = d.dk / 8;             // column groups (d_k is a multiple of 8, at most 256)
    const int nrl = kThreads / ncg;       // row lanes
    const int tid = threadIdx.x, rl = tid / ncg, cg = tid % ncg;
    const long r0 = (long)chunk * kGateRows, r1 = min((long)d.B * d.T, r0 + kGateRows);
    float acc[3][8], bacc[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 3; c++)
#pragma unroll
        for (int i = 0; i < 8; i++) acc[c][i] = 0.f;
    if (rl < nrl) {
        for (long r = r0 + rl; r < r1; r += nrl) {
            const float *st = a.rs + (r * d.Hq + h) * kStat;
            const float z0 = st[3], z1 = st[7], z2 = st[11];
            const T *qr = (const T *)a.q + (r * d.Hq + h) * d.dk + 8 * cg;
            float q[8];
            if constexpr (sizeof(T) == 2) {
                const uint4 w = *(const uint4 *)qr;
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    q[2 * i] = __uint_as_float(ws[i] << 16);
                    q[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
                }
            } else {
                const float4 w0 = *(const float4 *)qr, w1 = *(const float4 *)(qr + 4);
                q[0] = w0.x; q[1] = w0.y; q[2] = w0.z; q[3] = w0.w;
                q[4] = w1.x; q[5] = w1.y; q[6] = w1.z; q[7] = w1.w;
            }
#pragma unroll
            for (int i = 0; i < 8; i++) {
                acc[0][i] = __builtin_fmaf(z0, q[i], acc[0][i]);
                acc[1][i] = __builtin_fmaf(z1, q[i], acc[1][i]);
                acc[2][i] = __builtin_fmaf(z2, q[i], acc[2][i]);
            }
            bacc[0] += z0;
            bacc[1] += z1;
            bacc[2] += z2;
        }
    }
#pragma unroll
    for (int c = 0; c < 3; c++)
#pragma unroll
        for (int i = 0; i < 8; i++) red[tid * 24 + c * 8 + i] = acc[c][i];
    if (cg == 0 && rl < nrl) {
        bred[rl * 3] = bacc[0];
        bred[rl * 3 + 1] = bacc[1];
        bred[rl * 3 + 2] = bacc[2];
    }
    __syncthreads();
    float *gp = a.gpart + ((long)h * a.ngc + chunk) * 3 * W1;
    for (int e = tid; e < 3 * W1; e += kThreads) {
        const int c = e / W1, x = e % W1;
        float sum = 0.f;
        if (x < d.dk) {
            for (int l = 0; l < nrl; l++) sum += red[(l * ncg + x / 8) * 24 + c * 8 + x % 8];
        } else {
            for (int l = 0; l < nrl; l++) sum += bred[l * 3 + c];
        }
        gp[e] = sum;
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

// whether a launch with `bytes` of dynamic LDS fits a workgroup's 160 KB
// next to the kernel's static LDS
template <typename K>
bool fits_lds(K kernel, size_t bytes)
{
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, (const void *)kernel) != hipSuccess) return false;
    return fa.sharedSizeBytes + bytes <= kLdsBytes;
}

template <typename T>
hipError_t launch_all(const BwdArgs &A, hipStream_t s)
{
    const Dims &d = A.d;
    const int BH = d.B * d.Hkv;
    hipError_t e;
    // 1. rows
    {
        const size_t lds = sizeof(float) * ((size_t)d.G * (d.dk + 2 * d.dv + kChunk)) +
                           sizeof(T) * (size_t)kChunk * (stage_stride<T>(d.dk) + stage_stride<T>(d.dv));
        const size_t lds0 = sizeof(float) * ((size_t)d.G * (d.dk + 2 * d.dv + kChunk));
        if (bwd_keys_mfma_ok(d)) {
            if ((e = launch_bwd_rows_mfma(A, s)) != hipSuccess) return e;
        } else if (fits_lds(k_bwd_rows<T, true>, lds)) {
            if ((e = set_lds(k_bwd_rows<T, true>, lds)) != hipSuccess) return e;
            hipLaunchKernelGGL((k_bwd_rows<T, true>), dim3(d.T, d.Hkv, d.B), dim3(kThreads), lds, s, A);
        } else {
            if ((e = set_lds(k_bwd_rows<T, false>, lds0)) != hipSuccess) return e;
            hipLaunchKernelGGL((k_bwd_rows<T, false>), dim3(d.T, d.Hkv, d.B), dim3(kThreads), lds0, s, A);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t klds = sizeof(float) * ((size_t)kKeyTile * (d.dk + d.dv + 2) + (size_t)d.G * (d.dk + d.dv) +
                                         2 * (size_t)d.G * kKeyTile);
    // 2. raw keys: the selection bitmap, then one workgroup per 64-key block
    {
        const size_t lds = sizeof(uint32_t) * (size_t)d.nb * (kThreads / 32);
        if (lds <= 64 * 1024) {
            hipLaunchKernelGGL(k_bwd_selmap_lds, dim3((d.T + kThreads - 1) / kThreads, BH), dim3(kThreads), lds, s, A);
        } else {
            const long nwords = (long)BH * d.nb * ((d.T + 31) / 32);
            hipLaunchKernelGGL(k_bwd_fill_u32, dim3((unsigned)std::min<long>((nwords + kThreads - 1) / kThreads, 4096)),
                               dim3(kThreads), 0, s, A.selbm, nwords);
            hipLaunchKernelGGL(k_bwd_selmap, dim3((d.T + kThreads - 1) / kThreads, BH), dim3(kThreads), 0, s, A);
        }
        if (bwd_keys_mfma_ok(d)) {
            if ((e = launch_bwd_keys_mfma(A, s)) != hipSuccess) return e;
        } else {
            const size_t blds = sizeof(float) * ((size_t)d.G * (d.dk + d.dv) + 2 * (size_t)d.G * 64) +
                                sizeof(T) * (size_t)64 * (stage_stride<T>(d.dk) + stage_stride<T>(d.dv));
            const size_t blds0 = sizeof(float) * ((size_t)d.G * (d.dk + d.dv) + 2 * (size_t)d.G * 64);
            if (fits_lds(k_bwd_keys_blk<T, true>, blds)) {
                if ((e = set_lds(k_bwd_keys_blk<T, true>, blds)) != hipSuccess) return e;
                hipLaunchKernelGGL((k_bwd_keys_blk<T, true>), dim3(d.nb, BH), dim3(kThreads), blds, s, A);
            } else {
                if ((e = set_lds(k_bwd_keys_blk<T, false>, blds0)) != hipSuccess) return e;
                hipLaunchKernelGGL((k_bwd_keys_blk<T, false>), dim3(d.nb, BH), dim3(kThreads), blds0, s, A);
            }
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    // 3. compressed keys, then the sum over row chunks
    if (bwd_keys_mfma_ok(d)) {
        if ((e = launch_bwd_cmp_keys_mfma(A, s)) != hipSuccess) return e;
    } else {
        if ((e = set_lds(k_bwd_keys_cmp<T>, klds)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_bwd_keys_cmp<T>, dim3(d.npad / kKeyTile, A.nchunk, BH), dim3(kThreads), klds, s, A);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        const long n = (long)BH * d.npad * (d.dk + d.dv);
        hipLaunchKernelGGL(k_bwd_sum_parts, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                           A);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // Two-layer map: kcv holds the gradient G of the compressed K/V.  The
    // hidden layers are recomputed (the first layers' compression), the
    // second layers' gradients formed, and G is carried through the second
    // layer and the ReLU into da, which then takes kcv's place for the first
    // layers' (the linear map's) gradients below.
    BwdArgs Am = A;
    if (A.mlp) {
        if (compress_bf16_supported(d)) {
            if ((e = launch_compress_bf16(d, A.k, A.v, A.wck, A.pek, A.wcv, A.pev, A.hk, A.hv, s)) != hipSuccess)
                return e;
        } else {
            if ((e = launch_compress_generic(d, A.k, A.wck, A.pek, A.hk, d.dk, s)) != hipSuccess) return e;
            if ((e = launch_compress_generic(d, A.v, A.wcv, A.pev, A.hv, d.dv, s)) != hipSuccess) return e;
        }
        for (int isk = 1; isk >= 0; isk--) {
            const int dim = isk ? d.dk : d.dv;
            Dw2Problem<T> p2;
            p2.M = p2.N = dim;
            p2.K = BH * d.ncmp;
            p2.G = A.kcv + (isk ? 0 : d.dk);
            p2.gs = d.dk + d.dv;
            p2.h = (const T *)(isk ? A.hk : A.hv);
            p2.dim = dim;
            p2.ncmp = d.ncmp;
            p2.npad = d.npad;
            p2.out = isk ? A.dw2k : A.dw2v;
            {
                // split over the compressed-key partials' buffer, which the
                // chunk sum above has consumed: at most 32 splits of at least
                // 64 rows, as many as the buffer holds
                const long cap = (long)A.nchunk * BH * d.npad * (d.dk + d.dv);
                int ns = (int)std::min<long>(32, std::max<long>(1, cap / ((long)dim * dim)));
                ns = std::min(ns, std::max(1, (p2.K + 63) / 64));
                Dw2SplitProblem<T> ps;
                ps.M = ps.N = dim;
                ps.K = (p2.K + ns - 1) / ns;
                ps.Ktot = p2.K;
                ps.base = p2;
                ps.part = A.part;
                hipLaunchKernelGGL(k_gemm<Dw2SplitProblem<T>>, dim3((dim + 63) / 64, (dim + 63) / 64, ns),
                                   dim3(kThreads), 0, s, ps);
                const long n = (long)dim * dim;
                hipLaunchKernelGGL(k_sum_splits, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                                   (const float *)A.part, ns, n, p2.out);
            }
            DaProblem<T> pa;
            pa.M = d.npad;
            pa.N = pa.K = dim;
            pa.G = p2.G;
            pa.gs = p2.gs;
            pa.W2 = (const T *)(isk ? A.w2k : A.w2v);
            pa.h = p2.h;
            pa.da = A.da + (isk ? 0 : d.dk);
            pa.dim = dim;
            pa.ncmp = d.ncmp;
            pa.npad = d.npad;
            hipLaunchKernelGGL(k_gemm<DaProblem<T>>, dim3((d.npad + 63) / 64, (dim + 63) / 64, BH), dim3(kThreads), 0,
                               s, pa);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        Am.kcv = A.da;
    }
    {
        hipLaunchKernelGGL(k_bwd_colsum_part, dim3((d.dk + d.dv + kWave - 1) / kWave, kColChunks), dim3(kThreads), 0, s,
                           Am);
        hipLaunchKernelGGL(k_bwd_colsum, dim3((d.dk + d.dv + kThreads - 1) / kThreads), dim3(kThreads), 0, s, Am);
        hipLaunchKernelGGL(k_bwd_dpe<T>, dim3((32 * (d.dk > d.dv ? d.dk : d.dv) + kWave - 1) / kWave, 2),
                           dim3(kThreads), 0, s, Am);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 4. compression map: weight gradients and token gradients
    for (int isk = 1; isk >= 0; isk--) {
        const int dim = isk ? d.dk : d.dv;
        DwProblem<T> pw;
        pw.M = dim;
        pw.N = 32 * dim;
        pw.K = BH * d.ncmp;
        pw.G = Am.kcv + (isk ? 0 : d.dk);
        pw.gs = d.dk + d.dv;
        pw.x = (const T *)(isk ? A.k : A.v);
        pw.pe = (const T *)(isk ? A.pek : A.pev);
        pw.T_ = d.T;
        pw.dim = dim;
        pw.ncmp = d.ncmp;
        pw.npad = d.npad;
        pw.out = isk ? A.dwck : A.dwcv;
        if (bwd_keys_mfma_ok(d)) {
            if ((e = launch_bwd_dw_mfma(Am, isk == 1, s)) != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(k_gemm<DwProblem<T>>, dim3((pw.M + 63) / 64, (pw.N + 63) / 64, 1), dim3(kThreads), 0,
                               s, pw);
        }
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
        if (bwd_keys_mfma_ok(d)) {
            if ((e = launch_bwd_dx_mfma(Am, isk == 1, s)) != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL(k_gemm<DxProblem<T>>, dim3((px.M + 63) / 64, (px.N + 63) / 64, BH), dim3(kThreads), 0,
                               s, px);
        }
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

size_t backward_layout(const Dims &d, void *ws, BwdArgs *A, bool mlp)
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
    const size_t o_csp = carve((size_t)kColChunks * (d.dk + d.dv));
    const size_t o_gp = carve((size_t)d.Hq * ngc * 3 * (d.dk + 1));
    const size_t o_bm = carve((size_t)BH * d.nb * ((d.T + 31) / 32));   // 32-bit words
    int krc = 0, nkc = 0;
    size_t kp_floats = 0;
    if (bwd_keys_mfma_ok(d)) bwd_key_chunks(d, &krc, &nkc, &kp_floats);
    const size_t o_kp = carve(kp_floats);
    size_t o_hk = 0, o_hv = 0, o_da = 0;
    if (mlp) {
        const size_t es = d.dtype == NSA_FP32 ? 4 : 2;   // storage bytes per element
        o_hk = carve((BH * d.npad * d.dk * es + 3) / 4);
        o_hv = carve((BH * d.npad * d.dv * es + 3) / 4);
        o_da = carve((size_t)BH * d.npad * (d.dk + d.dv));
    }
    if (ws && A) {
        char *w = (char *)ws;
        A->rs = (float *)(w + o_rs);
        A->dk_raw = (float *)(w + o_dkr);
        A->dv_raw = (float *)(w + o_dvr);
        A->part = (float *)(w + o_part);
        A->kcv = (float *)(w + o_kcv);
        A->colsum = (float *)(w + o_cs);
        A->cspart = (float *)(w + o_csp);
        A->gpart = (float *)(w + o_gp);
        A->selbm = (uint32_t *)(w + o_bm);
        A->kpart = (float *)(w + o_kp);
        A->krc = krc;
        A->nkc = nkc;
        A->nchunk = nchunk;
        A->ngc = ngc;
        if (mlp) {
            A->hk = w + o_hk;
            A->hv = w + o_hv;
            A->da = (float *)(w + o_da);
        }
    }
    return off;
}

hipError_t launch_backward(const BwdArgs &A, hipStream_t s)
{
    if (A.d.dtype == NSA_FP32) return launch_all<float>(A, s);
    return launch_all<bf16_t>(A, s);
}

}  // namespace nsa
