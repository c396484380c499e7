// Small helpers for the gfx950 matrix-core kernels.
//
// bf16 MFMA operand layouts on gfx950 (verified on the device):
//  v_mfma_f32_32x32x16_bf16: A[i][k] in lane i + 32*(k/8), element k%8;
//    B[k][j] in lane j + 32*(k/8), element k%8; C[i][j] in lane j + 32*((i/4)%2),
//    element 4*(i/8) + i%4.
//  v_mfma_f32_16x16x32_bf16: A[i][k] in lane i + 16*(k/8), element k%8;
//    B[k][j] in lane j + 16*(k/8), element k%8; C[i][j] in lane j + 16*(i/4),
//    element i%4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte loads/stores of eight bf16 values.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *(u32x4 *)p = v; }

// Pack two floats into a bf16 pair (round to nearest even).  The vector
// conversion becomes one v_cvt_pk_bf16_f32; converting the halves one at a
// time costs two conversions plus a shift and an or.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ bf16x8 pack8(const float *p)
{
    u32x4 v;
    v[0] = pack_bf16x2(p[0], p[1]);
    v[1] = pack_bf16x2(p[2], p[3]);
    v[2] = pack_bf16x2(p[4], p[5]);
    v[3] = pack_bf16x2(p[6], p[7]);
    return as_bf16x8(v);
}

// c + sum of the 8 products of two rows of 8 bf16 (4 packed words each), in
// fp32: four v_dot2_f32_bf16, no unpacking of the halves.  Each word is copied
// to a scalar before the bit cast: a bit cast applied to the vector element
// expression itself reads the vector's first word for every element.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float c)
{
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t x = a[e], y = b[e];
        c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), c, false);
    }
    return c;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane moves within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kRowMirror = 0x140;      // lane j <- lane 15-j
constexpr int kRowHalfMirror = 0x141;  // lane j <- lane (j&8) | (7-(j&7))
constexpr int kQuadXor2 = 0x4E;        // lane j <- lane j^2
constexpr int kQuadXor1 = 0xB1;        // lane j <- lane j^1

// Transposing sum over the 16 lanes of a DPP row: lane j of the row returns
// sum over the row's lanes of v[j].  Four exchange steps; in each, partner
// lanes differ in one bit of j (3, 2, 1, 0), keep the half of the registers
// that bit selects and add the partner's copy of it.
__device__ __forceinline__ float row_transpose_sum16(const float v[16], int lane)
{
    const int j = lane & 15;
    const bool b3 = j & 8, b2 = j & 4, b1 = j & 2, b0 = j & 1;
    float w[8], x[4], y[2];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        float keep = b3 ? v[r + 8] : v[r];
        float send = b3 ? v[r] : v[r + 8];
        w[r] = keep + dpp<kRowMirror>(send);
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        float keep = b2 ? w[r + 4] : w[r];
        float send = b2 ? w[r] : w[r + 4];
        x[r] = keep + dpp<kRowHalfMirror>(send);
    }
#pragma unroll
    for (int r = 0; r < 2; r++) {
        float keep = b1 ? x[r + 2] : x[r];
        float send = b1 ? x[r] : x[r + 2];
        y[r] = keep + dpp<kQuadXor2>(send);
    }
    float keep = b0 ? y[1] : y[0];
    float send = b0 ? y[0] : y[1];
    return keep + dpp<kQuadXor1>(send);
}

// Sum over the 16 lanes of each DPP row (row rotations by 8, 4, 2, 1).  Every
// step adds two values in either order, so all 16 lanes end with the same bits.
__device__ __forceinline__ float row_sum16(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
    return x;
}

// Wait until every outstanding vector-memory load of this wave has returned
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS transpose read of 16-bit elements (ds_read_b64_tr_b16; lane mapping
// checked on the device): within each group of 16 lanes, lane i receives
// element (i % 4) of the 8-byte pieces addressed by lanes 4e + i/4, e = 0..3.
// So if lane s of a group points at 4 consecutive columns 4*(s%4) .. +3 of
// row r0 + s/4 of a row-major matrix, lane i gets column i of rows r0 .. r0+3
// -- four consecutive rows of one column, the layout of half an MFMA operand
// whose reduction index runs along those rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ uint2 ld_tr16(const uint16_t *p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uint16_t *)p);
    return __builtin_bit_cast(uint2, v);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which makes every wave wait for its outstanding global loads
// first and so cancels any prefetch in flight; the barriers in these kernels
// only ever protect LDS data.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace nsa
