// Second layer of the two-layer compression map (deepdaiv newsletter on
// DeepSeek's NSA, deepdaiv.stibee.com/p/82, token compression paragraph: a
// small neural network with an intra-block position encoding summarises each
// block).  The first layer is the linear compression with W1 in place of the
// linear map, which leaves a = W1 vec(block + PE) in the storage type in the
// output buffers; this pass replaces each row in place by
//   out = W2 relu(a),   W2 [dim][dim], out[c] = sum_j W2[c][j] relu(a[j]).
// relu commutes with rounding to the storage type (rounding keeps the sign),
// so relu(round(a)) is the rounded hidden layer.  Pad rows (a = 0) stay 0.
//
// k_mlp2_mfma (bf16, dim = 64, 128, 192): out^T = W2 relu(A)^T with
// v_mfma_f32_16x16x32_bf16; wave w of a workgroup owns rows 16 w .. 16 w + 15
// of a 64-row tile, loads all of them before it writes any, and stores four
// consecutive channels of one row per lane.
// k_mlp2_generic (fp32, other widths): 16 rows staged in LDS, then written.
// With an append's lengths only the newly completed blocks are rewritten
// (the same arithmetic, so those rows equal a full pass's bit for bit).
#include <algorithm>

#include "mfma_util.h"
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kThreads = 256;

// relu on two packed bf16: a half with its sign bit set becomes +0
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w)
{
    const uint32_t m = ((w & 0x80008000u) >> 15) * 0xffffu;
    return w & ~m;
}

// The rows [lo, hi] of sequence-head bh that a launch rewrites: every row, or
// with an append (len_new non-null) the blocks that growing the cache from
// len_old[b] to len_new[b] tokens completes (block i is complete at length L
// when 16 i + 31 < L; lengths clamped to 0 <= len_old <= len_new <= T).
struct RowRange {
    int lo, hi;
};
__device__ __forceinline__ RowRange row_range(const int32_t *len_old, const int32_t *len_new, int bh, int Hkv,
                                              int T, int npad)
{
    if (!len_new) return {0, npad - 1};
    const int b = bh / Hkv;
    const int ln = min(max(len_new[b], 0), T), lo = len_old ? min(max(len_old[b], 0), ln) : 0;
    return {lo > 31 ? (lo - 31 + 15) / 16 : 0, ln >= 32 ? (ln - 32) / 16 : -1};
}

template <int DIM>
__global__ __launch_bounds__(kThreads) void k_mlp2_mfma(uint16_t *__restrict__ buf, const uint16_t *__restrict__ W2,
                                                        int npad, const int32_t *__restrict__ len_old,
                                                        const int32_t *__restrict__ len_new, int Hkv, int T)
{
    constexpr int NK = DIM / 32, NT = DIM / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const RowRange rr = row_range(len_old, len_new, blockIdx.y, Hkv, T, npad);
    const int tile = rr.lo / 64 + blockIdx.x;
    if (tile * 64 > rr.hi || tile * 64 >= npad) return;   // no barriers in this kernel
    const int i = tile * 64 + 16 * wave + li;              // this lane's row
    const bool mine = i >= rr.lo && i <= rr.hi;
    const long row = (long)blockIdx.y * npad + i;
    uint16_t *r = buf + row * DIM;
    // B operand relu(A)^T: row li, channels 32 c + 8 lg .. +7
    u32x4 hb[NK];
#pragma unroll
    for (int c = 0; c < NK; c++) {
        u32x4 v = ld16(r + 32 * c + 8 * lg);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t x = v[e];
            v[e] = relu_bf16x2(x);
        }
        hb[c] = v;
    }
    // every load of the row slice is done before any store below
    wait_vmem_all();
#pragma unroll
    for (int n = 0; n < NT; n++) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NK; c++)
            acc = mfma16(as_bf16x8(ld16(W2 + (16 * n + li) * DIM + 32 * c + 8 * lg)), as_bf16x8(hb[c]), acc);
        // C[i = channel][j = row]: lane j + 16 (i / 4), element i % 4
        if (mine) *(uint2 *)(r + 16 * n + 4 * lg) = uint2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_mlp2_generic(T *__restrict__ buf, const T *__restrict__ W2, int dim,
                                                           int npad, const int32_t *__restrict__ len_old,
                                                           const int32_t *__restrict__ len_new, int Hkv, int T_)
{
    extern __shared__ float hs[];   // [16][dim] relu of the rows
    const int tid = threadIdx.x;
    const RowRange rr = row_range(len_old, len_new, blockIdx.y, Hkv, T_, npad);
    const int r0 = (rr.lo / 16 + (int)blockIdx.x) * 16;
    if (r0 > rr.hi || r0 >= npad) return;   // uniform: before the barrier
    T *rows = buf + ((long)blockIdx.y * npad + r0) * dim;
    for (int e = tid; e < 16 * dim; e += kThreads) hs[e] = fmaxf(to_f(rows[e]), 0.f);
    __syncthreads();
    for (int e = tid; e < 16 * dim; e += kThreads) {
        const int r = e / dim, c = e % dim;
        if (r0 + r < rr.lo || r0 + r > rr.hi) continue;
        float acc = 0.f;
        for (int j = 0; j < dim; j++) acc += to_f(W2[(long)c * dim + j]) * hs[r * dim + j];
        rows[e] = from_f<T>(acc);
    }
}

// groups: 64-row tiles (MFMA) or 16-row groups (generic) per sequence-head,
// counted from the first rewritten row's tile or group
template <typename T>
hipError_t launch_generic(const Dims &d, void *buf, const void *W2, int dim, hipStream_t s, const int32_t *len_old,
                          const int32_t *len_new, int rows)
{
    const size_t lds = sizeof(float) * 16 * (size_t)dim;
    const int groups = len_new ? std::min(rows / 16 + 2, d.npad / 16) : d.npad / 16;
    hipLaunchKernelGGL(k_mlp2_generic<T>, dim3(groups, d.B * d.Hkv), dim3(kThreads), lds, s, (T *)buf,
                       (const T *)W2, dim, d.npad, len_old, len_new, d.Hkv, d.T);
    return hipGetLastError();
}

hipError_t launch_one(const Dims &d, void *buf, const void *W2, int dim, hipStream_t s, const int32_t *len_old,
                      const int32_t *len_new, int rows)
{
    const int tiles = len_new ? std::min(rows / 64 + 2, d.npad / 64) : d.npad / 64;
    const dim3 grid(tiles, d.B * d.Hkv);
    if (d.dtype == NSA_BF16) {
        uint16_t *b = (uint16_t *)buf;
        const uint16_t *w = (const uint16_t *)W2;
        if (dim == 192)
            hipLaunchKernelGGL(k_mlp2_mfma<192>, grid, dim3(kThreads), 0, s, b, w, d.npad, len_old, len_new, d.Hkv, d.T);
        else if (dim == 128)
            hipLaunchKernelGGL(k_mlp2_mfma<128>, grid, dim3(kThreads), 0, s, b, w, d.npad, len_old, len_new, d.Hkv, d.T);
        else if (dim == 64)
            hipLaunchKernelGGL(k_mlp2_mfma<64>, grid, dim3(kThreads), 0, s, b, w, d.npad, len_old, len_new, d.Hkv, d.T);
        else return launch_generic<bf16_t>(d, buf, W2, dim, s, len_old, len_new, rows);
        return hipGetLastError();
    }
    return launch_generic<float>(d, buf, W2, dim, s, len_old, len_new, rows);
}

}  // namespace

hipError_t launch_compress_mlp2(const Dims &d, const void *W2k, const void *W2v, void *cmp_k, void *cmp_v,
                                hipStream_t s, const int32_t *len_old, const int32_t *len_new, int max_blocks)
{
    hipError_t e = launch_one(d, cmp_k, W2k, d.dk, s, len_old, len_new, max_blocks);
    if (e != hipSuccess) return e;
    return launch_one(d, cmp_v, W2v, d.dv, s, len_old, len_new, max_blocks);
}

}  // namespace nsa
