// Token compression for bf16 storage (deepdaiv newsletter on DeepSeek's NSA,
// deepdaiv.stibee.com/p/82, token compression paragraph: each block of l = 32
// consecutive tokens, taken every d = 16 tokens, is summarised by one learned
// map with an intra-block position encoding).
//
//   out[bh][i][c] = sum_{m < 32*dim} W[c][m] * (x[bh][16 i * dim + m] + PE[m])
//                 = sum_m W[c][m] x[...] + sum_m W[c][m] PE[m]
//
// Block i flattened token-major is the 32*dim consecutive elements starting
// at token 16 i, so the product is a plain matrix product whose rows overlap.
// The bf16 operands are used as stored and the position term is accumulated
// beside the main product, so x + PE never has to be rounded.
//
// k_compress_mfma_kv (d = 64, 128, 192; K and V in one launch):
// v_mfma_f32_32x32x16_bf16.  A workgroup
// takes 63 blocks plus one extra operand row that holds PE, so the same
// matrix product yields sum_m W[c][m] PE[m] in that row; 64 rows x all d
// channels, 64-element K steps staged through LDS one step ahead.
// k_compress_bf16 (other d): the same sums on the vector ALUs with
// v_dot2c_f32_bf16, 128 blocks x 64 channels per workgroup.
#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;
constexpr int kTI = 128;     // blocks per tile
constexpr int kTC = 64;      // channels per tile
constexpr int kKS = 64;      // input elements per step
constexpr int kRS = kKS + 8; // LDS row stride (bf16): 144 bytes, 9 x 16 B, so 16 rows hit 16 bank groups

struct CompressLds {
    uint16_t a[2][kTI * kRS];
    uint16_t b[2][kTC * kRS];
    uint16_t pe[2][kKS];
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

__device__ __forceinline__ void compress_bf16_tile(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                                                   const uint16_t *__restrict__ PE, uint16_t *__restrict__ out,
                                                   int T, int dim, int ncmp, int npad, int bh, int i0, int c0,
                                                   int wlo, int whi, CompressLds &sm)
{
    const int tid = threadIdx.x, ti = tid & 15, tc = tid >> 4;
    const long L = 32L * dim;
    const uint16_t *xs = x + (long)bh * T * dim;
    const int nsteps = (int)(L / kKS);

    // prefetch registers: 4 A chunks, 2 B chunks, 1 PE chunk (threads 0..7)
    u32x4 ra[4], rb[2], rp;
    auto load = [&](int s) {
        const long k0 = (long)s * kKS;
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            const int i = i0 + row;
            ra[q] = i < ncmp ? ld16(xs + 16L * i * dim + k0 + ch * 8) : z;
        }
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            const int c = c0 + row;
            rb[q] = c < dim ? ld16(W + (long)c * L + k0 + ch * 8) : z;
        }
        if (tid < 8) rp = ld16(PE + k0 + tid * 8);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            st16(&sm.a[buf][row * kRS + ch * 8], ra[q]);
        }
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            st16(&sm.b[buf][row * kRS + ch * 8], rb[q]);
        }
        if (tid < 8) st16(&sm.pe[buf][tid * 8], rp);
    };

    float acc[8][4], cacc[4];
#pragma unroll
    for (int u = 0; u < 8; u++)
#pragma unroll
        for (int v = 0; v < 4; v++) acc[u][v] = 0.f;
#pragma unroll
    for (int v = 0; v < 4; v++) cacc[v] = 0.f;

    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nsteps; s++) {
        const int buf = s & 1;
        if (s + 1 < nsteps) load(s + 1);
#pragma unroll 2
        for (int kc = 0; kc < kKS / 8; kc++) {
            u32x4 av[8], bv[4];
#pragma unroll
            for (int u = 0; u < 8; u++) av[u] = ld16(&sm.a[buf][(ti + 16 * u) * kRS + kc * 8]);
#pragma unroll
            for (int v = 0; v < 4; v++) bv[v] = ld16(&sm.b[buf][(4 * tc + v) * kRS + kc * 8]);
            const u32x4 pv = ld16(&sm.pe[buf][kc * 8]);
#pragma unroll
            for (int p = 0; p < 4; p++) {
#pragma unroll
                for (int u = 0; u < 8; u++)
#pragma unroll
                    for (int v = 0; v < 4; v++) acc[u][v] = dot2(av[u][p], bv[v][p], acc[u][v]);
#pragma unroll
                for (int v = 0; v < 4; v++) cacc[v] = dot2(pv[p], bv[v][p], cacc[v]);
            }
        }
        if (s + 1 < nsteps) store(buf ^ 1);
        lds_barrier();
    }
    // rows wlo <= i < whi are written, as zero from ncmp on
    const int c = c0 + 4 * tc;
    if (c >= dim) return;
#pragma unroll
    for (int u = 0; u < 8; u++) {
        const int i = i0 + ti + 16 * u;
        if (i < wlo || i >= whi || i >= npad) continue;
        uint2 w = {0u, 0u};
        if (i < ncmp) {
            w.x = pack_bf16x2(acc[u][0] + cacc[0], acc[u][1] + cacc[1]);
            w.y = pack_bf16x2(acc[u][2] + cacc[2], acc[u][3] + cacc[3]);
        }
        *(uint2 *)(out + ((long)bh * npad + i) * dim + c) = w;
    }
}

// Block ranges as in k_compress_mfma_kv: all blocks (pads written as 0), or
// with lengths only the blocks an append completes.
__global__ __launch_bounds__(kThreads) void k_compress_bf16(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ W,
                                                            const uint16_t *__restrict__ PE,
                                                            uint16_t *__restrict__ out, int T, int dim, int ncmp,
                                                            int npad, int Hkv, const int32_t *len_old,
                                                            const int32_t *len_new)
{
    __shared__ CompressLds sm;
    const int bh = blockIdx.z, c0 = blockIdx.y * kTC;
    int lo = 0, hi = ncmp;
    if (len_new) append_range(len_old, len_new, bh / Hkv, T, lo, hi);
    const int wend = len_new ? hi : npad;
    for (int i0 = lo + (int)blockIdx.x * kTI; i0 < wend; i0 += (int)gridDim.x * kTI) {
        compress_bf16_tile(x, W, PE, out, T, dim, hi, npad, bh, i0, c0, len_new ? lo : i0, wend, sm);
        if (!len_new) break;
        __syncthreads();
    }
}

constexpr int kMRows = 64;        // operand rows per workgroup: 63 blocks + the PE row
constexpr int kMBlocks = kMRows - 1;
constexpr int kMK = 64;           // K elements per step
constexpr int kMS = kMK + 8;      // LDS row stride (bf16)

template <int DIM>
struct CompressMfmaLds {
    uint16_t a[2][kMRows * kMS];
    uint16_t b[2][DIM * kMS];
    float pe[DIM];                // sum_m W[c][m] PE[m]
};

// One workgroup tile: blocks i0 .. i0+62 of one (b, KV head).  Blocks below
// ncmp are loaded; rows wlo <= i < whi are written, as 0 when i >= ncmp.  Each
// output row depends only on its own operand row and W, so a block comes out
// bit for bit the same whichever tile computes it.  4 waves: wave w takes
// operand rows 32 (w % 2) .. +31 and channels (w / 2) * DIM/2 .. +DIM/2
// (DIM/64 tiles of 32 x 32).
template <int DIM>
__device__ __forceinline__ void compress_mfma_tile(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                                                   const uint16_t *__restrict__ PE, uint16_t *__restrict__ out,
                                                   int T, int ncmp, int npad, int bh, int i0, int wlo, int whi,
                                                   CompressMfmaLds<DIM> &sm)
{
    constexpr int NT = DIM / 64;                 // 32-channel tiles per wave
    constexpr int L = 32 * DIM;
    constexpr int BTASK = DIM * (kMK / 8) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rw = 32 * (wave & 1), cw = (wave >> 1) * (DIM / 2);
    const uint16_t *xs = x + (long)bh * T * DIM;

    u32x4 ra[2], rb[BTASK];
    auto load = [&](int st) {
        const int k0 = st * kMK;
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            const int i = i0 + row;
            if (row == kMBlocks) ra[q] = ld16(PE + k0 + ch * 8);
            else ra[q] = i < ncmp ? ld16(xs + 16L * i * DIM + k0 + ch * 8) : z;
        }
#pragma unroll
        for (int q = 0; q < BTASK; q++) {
            const int task = tid + q * kThreads, c = task >> 3, ch = task & 7;
            rb[q] = ld16(W + (long)c * L + k0 + ch * 8);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int task = tid + q * kThreads, row = task >> 3, ch = task & 7;
            st16(&sm.a[buf][row * kMS + ch * 8], ra[q]);
        }
#pragma unroll
        for (int q = 0; q < BTASK; q++) {
            const int task = tid + q * kThreads, c = task >> 3, ch = task & 7;
            st16(&sm.b[buf][c * kMS + ch * 8], rb[q]);
        }
    };

    f32x16 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; n++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[n][r] = 0.f;

    constexpr int nsteps = L / kMK;
    load(0);
    store(0);
    lds_barrier();
    const int fr = lane & 31, fk = 8 * (lane >> 5);   // operand row / K offset of this lane
    for (int st = 0; st < nsteps; st++) {
        const int buf = st & 1;
        if (st + 1 < nsteps) load(st + 1);
#pragma unroll
        for (int ks = 0; ks < kMK / 16; ks++) {
            const bf16x8 af = as_bf16x8(ld16(&sm.a[buf][(rw + fr) * kMS + 16 * ks + fk]));
#pragma unroll
            for (int n = 0; n < NT; n++) {
                const bf16x8 bf = as_bf16x8(ld16(&sm.b[buf][(cw + 32 * n + fr) * kMS + 16 * ks + fk]));
                acc[n] = mfma32(af, bf, acc[n]);
            }
        }
        if (st + 1 < nsteps) store(buf ^ 1);
        lds_barrier();
    }
    // lane l holds channel cw + 32n + l%32 of rows rw + 8(e/4) + 4(l/32) + e%4;
    // operand row 63 (the PE row) is e = 15 of the upper lane half of wave 1/3
    if ((wave & 1) && lane >= 32) {
#pragma unroll
        for (int n = 0; n < NT; n++) sm.pe[cw + 32 * n + (lane & 31)] = acc[n][15];
    }
    lds_barrier();
#pragma unroll
    for (int n = 0; n < NT; n++) {
        const int c = cw + 32 * n + (lane & 31);
        const float pc = sm.pe[c];
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int row = rw + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int i = i0 + row;
            if (row == kMBlocks || i < wlo || i >= whi || i >= npad) continue;
            const __bf16 y = i < ncmp ? (__bf16)(acc[n][e] + pc) : (__bf16)0.f;
            out[((long)bh * npad + i) * DIM + c] = __builtin_bit_cast(uint16_t, y);
        }
    }
}

// K and V of every (b, KV head) in one launch: grid.y 0 .. BH-1 take K
// (d = DK), BH .. 2BH-1 take V (d = DV), so the two products share the chip.
// Without lengths: every block of the T-token sequences, pads written as 0.
// With lengths (a cache of capacity T): only the blocks that are complete at
// len_new[b] tokens but not at len_old[b]; workgroups stride over those tiles.
template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void k_compress_mfma_kv(const uint16_t *__restrict__ k,
                                                               const uint16_t *__restrict__ v,
                                                               const uint16_t *__restrict__ Wk,
                                                               const uint16_t *__restrict__ PEk,
                                                               const uint16_t *__restrict__ Wv,
                                                               const uint16_t *__restrict__ PEv,
                                                               uint16_t *__restrict__ ok, uint16_t *__restrict__ ov,
                                                               int T, int ncmp, int npad, int BH, int Hkv,
                                                               const int32_t *len_old, const int32_t *len_new)
{
    constexpr size_t SK = sizeof(CompressMfmaLds<DK>), SV = sizeof(CompressMfmaLds<DV>);
    __shared__ __attribute__((aligned(16))) unsigned char smem[SK > SV ? SK : SV];
    const int y = blockIdx.y;
    const int bh = y < BH ? y : y - BH;
    int lo = 0, hi = ncmp;
    if (len_new) append_range(len_old, len_new, bh / Hkv, T, lo, hi);
    for (int i0 = lo + (int)blockIdx.x * kMBlocks; i0 < (len_new ? hi : npad); i0 += (int)gridDim.x * kMBlocks) {
        const int wlo = len_new ? lo : i0, whi = len_new ? hi : npad;
        if (y < BH)
            compress_mfma_tile<DK>(k, Wk, PEk, ok, T, hi, npad, bh, i0, wlo, whi,
                                   *reinterpret_cast<CompressMfmaLds<DK> *>(smem));
        else
            compress_mfma_tile<DV>(v, Wv, PEv, ov, T, hi, npad, bh, i0, wlo, whi,
                                   *reinterpret_cast<CompressMfmaLds<DV> *>(smem));
        if (!len_new) break;   // one tile per workgroup: the grid covers every block
        lds_barrier();         // the next tile reuses the LDS buffers
    }
}

}  // namespace

bool compress_bf16_supported(const Dims &d) { return d.dtype == NSA_BF16; }

hipError_t launch_compress_bf16(const Dims &d, const void *k, const void *v, const void *Wk, const void *PEk,
                                const void *Wv, const void *PEv, void *ok, void *ov, hipStream_t s,
                                const int32_t *len_old, const int32_t *len_new, int max_new_blocks)
{
    const int BH = d.B * d.Hkv;
    // append: enough workgroups for max_new_blocks; each strides over its tiles
    auto tiles = [&](int per) {
        return len_new ? (max_new_blocks + per - 1) / per : (d.npad + per - 1) / per;
    };
    const dim3 mgrid(tiles(kMBlocks), 2 * BH);
    const uint16_t *ks = (const uint16_t *)k, *vs = (const uint16_t *)v;
    const uint16_t *wk = (const uint16_t *)Wk, *pk = (const uint16_t *)PEk, *wv = (const uint16_t *)Wv,
                   *pv = (const uint16_t *)PEv;
    uint16_t *oks = (uint16_t *)ok, *ovs = (uint16_t *)ov;
    if (d.dk == 192 && d.dv == 128) {
        hipLaunchKernelGGL((k_compress_mfma_kv<192, 128>), mgrid, dim3(kThreads), 0, s, ks, vs, wk, pk, wv, pv, oks,
                           ovs, d.T, d.ncmp, d.npad, BH, d.Hkv, len_old, len_new);
    } else if (d.dk == 128 && d.dv == 128) {
        hipLaunchKernelGGL((k_compress_mfma_kv<128, 128>), mgrid, dim3(kThreads), 0, s, ks, vs, wk, pk, wv, pv, oks,
                           ovs, d.T, d.ncmp, d.npad, BH, d.Hkv, len_old, len_new);
    } else if (d.dk == 64 && d.dv == 64) {
        hipLaunchKernelGGL((k_compress_mfma_kv<64, 64>), mgrid, dim3(kThreads), 0, s, ks, vs, wk, pk, wv, pv, oks,
                           ovs, d.T, d.ncmp, d.npad, BH, d.Hkv, len_old, len_new);
    } else {
        // other widths: the vector-ALU kernel, one launch per tensor
        for (int u = 0; u < 2; u++) {
            const int dim = u == 0 ? d.dk : d.dv;
            dim3 grid(tiles(kTI), (dim + kTC - 1) / kTC, BH);
            hipLaunchKernelGGL(k_compress_bf16, grid, dim3(kThreads), 0, s, u == 0 ? ks : vs, u == 0 ? wk : wv,
                               u == 0 ? pk : pv, u == 0 ? oks : ovs, d.T, dim, d.ncmp, d.npad, d.Hkv, len_old,
                               len_new);
        }
    }
    return hipGetLastError();
}

}  // namespace nsa
