// Stage S2 on the matrix cores: compressed attention and block importance.
//
// deepdaiv newsletter on DeepSeek's NSA (deepdaiv.stibee.com/p/82), token
// compression and token selection paragraphs: queries attend to one summary
// vector per compression block, and the block-importance scores that drive
// selection come from that attention.  The 16 query heads of a KV group share
// the group's compressed keys (ctol-kr.com article, "하드웨어 인식 설계":
// group-centric loading with a shared KV fetch), so a workgroup takes 8
// consecutive positions x 16 heads = 128 query rows of one KV group and
// streams the group's compressed keys through LDS once per pass for all of
// them.
//
// Orientation: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 -- 32 keys (M) by
// 32 query rows (N, two positions x 16 heads per wave) -- so every lane owns
// the softmax state of one query row.  K rows are stored in LDS permuted so
// that the 16 accumulators a lane holds are 16 consecutive keys; P^T then
// feeds O^T = V^T P^T directly as the B operand, with V^T transposed into LDS.
//
// Pass 1 computes each row's exact log-sum-exp.  Pass 2 recomputes the logits
// and forms exact probabilities, which give o_cmp and, summed over the 16
// heads in fp32 (a DPP transpose-reduce over each 16-lane row), the group's
// per-key importance; block j takes keys 4j-1 .. 4j+3 with weights 1,2,2,2,1.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kPos = 8;      // query positions per workgroup
constexpr int kTile = 64;    // compressed keys per LDS tile
constexpr int kThreads = 256;

template <int DK, int DV>
struct CmpLds {
    static constexpr int KS = DK + 8;      // bf16 per K row (padded against bank conflicts)
    static constexpr int VS = kTile + 8;   // bf16 per V^T row
    uint16_t k[kTile * KS];
    uint16_t vt[DV * VS];
    float pl[kPos][kTile];                 // head-summed probabilities of the current tile
};

// LDS row of key k (0..31) inside a 32-key M-tile.  MFMA output row i sits in
// lane half (i/4)%2, register 4*(i/8) + i%4; putting key 16*h + r in row
// 8*(r/4) + 4*h + r%4 makes register r of lane half h hold key 16*h + r.
__device__ __forceinline__ int krow(int k)
{
    int h = k >> 4, m = (k >> 2) & 3, u = k & 3;
    return 8 * m + 4 * h + u;
}

}  // namespace

// Workgroup -> ((b, g) pair, tile of 8 positions).  When the (b, g) pairs
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

template <int DK, int DV, bool WITH_V>
__global__ __launch_bounds__(kThreads) void k_cmp_attn_mfma(RowArgs a, int ntp, int BG)
{
    constexpr int KSTEPS = DK / 16;
    constexpr int DT = DV / 32;
    using L = CmpLds<DK, DV>;
    __shared__ L sm;

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
    const int nvis = (live && t >= 31) ? (t - 31) / 16 + 1 : 0;
    const int tlast = min(pos0 + kPos - 1, d.T - 1);
    const int nvis_max = tlast >= 31 ? (tlast - 31) / 16 + 1 : 0;
    const int ntiles = (nvis_max + kTile - 1) / kTile;
    const float sl2 = d.scale * kLog2e;

    bf16x8 qf[KSTEPS];
    {
        const uint16_t *qr = (const uint16_t *)a.q + (long)b * a.q_sb + (long)t * a.q_sr +
                             (long)(g * 16 + head) * DK + 8 * h;
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) qf[kk] = as_bf16x8(live ? ld16(qr + 16 * kk) : z);
    }
    const uint16_t *kc = (const uint16_t *)a.kc + (long)bg * d.npad * DK;
    const uint16_t *vc = (const uint16_t *)a.vc + (long)bg * d.npad * DV;

    auto load_k = [&](int c) {
        constexpr int CH = DK / 8;
        const uint16_t *src = kc + (long)c * kTile * DK;
        for (int task = tid; task < kTile * CH; task += kThreads) {
            const int key = task / CH, ch = task % CH;
            const int r = (key & ~31) | krow(key & 31);
            st16(&sm.k[r * L::KS + ch * 8], ld16(src + key * DK + ch * 8));
        }
    };
    auto load_vt = [&](int c) {
        constexpr int NDC = DV / 8;
        const uint16_t *src = vc + (long)c * kTile * DV;
        for (int task = tid; task < 32 * NDC; task += kThreads) {
            const int kp = task & 31, dc = task >> 5;
            const u32x4 v0 = ld16(src + (2 * kp) * DV + dc * 8);
            const u32x4 v1 = ld16(src + (2 * kp + 1) * DV + dc * 8);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t lo = (v0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                const uint32_t hi = (v1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                *(uint32_t *)&sm.vt[(dc * 8 + e) * L::VS + 2 * kp] = lo | (hi << 16);
            }
        }
    };
    auto logits = [&](int mt) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; r++) acc[r] = 0.f;
        const uint16_t *kr = &sm.k[(32 * mt + row) * L::KS + 8 * h];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) acc = mfma32(as_bf16x8(ld16(kr + 16 * kk)), qf[kk], acc);
        return acc;
    };

    // ---- pass 1: log-sum-exp of every row (log2 domain)
    float m = -INFINITY, l = 0.f;
    for (int c = 0; c < ntiles; c++) {
        __syncthreads();
        load_k(c);
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            const f32x16 acc = logits(mt);
            const int kb = c * kTile + 32 * mt + 16 * h;
            float s[16], mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                s[r] = kb + r < nvis ? acc[r] * sl2 : -INFINITY;
                mx = fmaxf(mx, s[r]);
            }
            const float mn = fmaxf(m, mx);
            if (mn != -INFINITY) {
                float sum = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r++) sum += fast_exp2(s[r] - mn);
                l = l * fast_exp2(m - mn) + sum;
                m = mn;
            }
        }
    }
    float lse2 = -INFINITY;
    {
        const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
        const float M = fmaxf(m, mo);
        if (M != -INFINITY) lse2 = M + fast_log2(l * fast_exp2(m - M) + lo * fast_exp2(mo - M));
    }

    // ---- pass 2: probabilities -> o_cmp and block importance
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] = 0.f;
    float carry = 0.f;   // P of the previous tile's last key (threads forming block 16c)
    float *scores = a.scores + (long)bg * a.R * d.nb;
    for (int c = 0; c < ntiles; c++) {
        __syncthreads();
        load_k(c);
        if (WITH_V) load_vt(c);
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            const f32x16 acc = logits(mt);
            const int kb = c * kTile + 32 * mt + 16 * h;
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; r++) p[r] = kb + r < nvis ? fast_exp2(acc[r] * sl2 - lse2) : 0.f;
            if (WITH_V) {
#pragma unroll
                for (int s2 = 0; s2 < 2; s2++) {
                    const bf16x8 pb = pack8(&p[8 * s2]);
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const uint16_t *vr = &sm.vt[(32 * dt + row) * L::VS + 32 * mt + 16 * h + 8 * s2];
                        oacc[dt] = mfma32(as_bf16x8(ld16(vr)), pb, oacc[dt]);
                    }
                }
            }
            sm.pl[pw][32 * mt + 16 * h + (lane & 15)] = row_transpose_sum16(p, lane);
        }
        __syncthreads();
        if (tid < kPos * 16) {
            const int pp = tid >> 4, jj = tid & 15;
            const float *P = sm.pl[pp];
            const float prev = jj ? P[4 * jj - 1] : carry;
            const float S = prev + 2.f * (P[4 * jj] + P[4 * jj + 1] + P[4 * jj + 2]) + P[4 * jj + 3];
            if (jj == 0) carry = P[kTile - 1];
            const int tt = pos0 + pp, j = 16 * c + jj;
            if (tt < d.T && j <= tt / 64) scores[(long)tt * d.nb + j] = S;
        }
    }
    // the last key of the final tile also reaches block 16*ntiles
    if (tid < kPos * 16 && (tid & 15) == 0) {
        const int tt = pos0 + (tid >> 4), j = 16 * ntiles;
        if (tt < d.T && j <= tt / 64) scores[(long)tt * d.nb + j] = carry;
    }

    if (WITH_V && live) {
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

hipError_t launch_cmp_attn_mfma(const RowArgs &a, bool with_v, hipStream_t s)
{
    const Dims &d = a.d;
    if (d.dk == 192 && d.dv == 128) return launch_dims<192, 128>(a, with_v, s);
    if (d.dk == 128 && d.dv == 128) return launch_dims<128, 128>(a, with_v, s);
    if (d.dk == 64 && d.dv == 64) return launch_dims<64, 64>(a, with_v, s);
    return hipErrorInvalidValue;
}

}  // namespace nsa
