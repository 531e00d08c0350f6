// Shared device helpers of the gfx950 preshuffled-B GEMM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgp {

// The LDS-poison debug build compiles every source with DGP_LDS_POISON=1
// (gemm_common.h: lds_poison_fill, lds_dma).
#ifndef DGP_LDS_POISON
#define DGP_LDS_POISON 0
#endif
constexpr bool kLdsPoison = DGP_LDS_POISON != 0;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kNumXcd = 8;          // gfx950: 8 XCDs, workgroups dealt round-robin
constexpr int kDtypeBf16 = 0;
constexpr int kDtypeFp8 = 1;
constexpr int kDtypeFp4 = 2;         // OCP E2M1, two per byte
constexpr int kScaleNone = 0;
constexpr int kScaleTensor = 1;
constexpr int kScaleBlock = 2;
constexpr int kScaleMx = 3;         // mxfp8: E8M0 byte per 128-K block per row of A / of B
constexpr int kScaleMx32 = 4;       // mxfp4: E8M0 byte per 32-K block per row of A / of B
constexpr int kOutBf16 = 0;         // direct epilogue: bf16 C
constexpr int kOutPartial = 1;      // split-K pass 1: fp32 partials

// Buffer-load cache-policy bits (aux operand) on gfx950.
constexpr int kAuxNone = 0;
constexpr int kAuxNonTemporal = 2;

// ---------------------------------------------------------------- tile map
//
// Workgroup id -> (tile_m, tile_n, split).  With remap, ids are regrouped so
// the workgroups placed on one XCD (ids congruent mod 8) get consecutive
// logical ids; ids past the last full round of 8 keep their own value, so the
// map stays a bijection for any grid size.  Logical ids then run split-major,
// and inside a split raster over groups of group_m tile rows.  Shared by the
// kernels and the host mirror, so both compute the identical map.
template <typename I>
struct TileCoordT {
    I tm, tn, s;
};
using TileCoord = TileCoordT<int64_t>;

// I = int in the kernels (grids are validated to fit), int64_t on the host.
template <typename I>
__host__ __device__ inline TileCoordT<I> tile_of_workgroup(I wg, I tiles_m, I tiles_n, I splits, int remap,
                                                           int group_m)
{
    const I total = tiles_m * tiles_n * splits;
    I logical = wg;
    if (remap) {
        const I per = total / kNumXcd;
        if (wg < per * kNumXcd)
            logical = (wg % kNumXcd) * per + wg / kNumXcd;
    }
    const I per_split = tiles_m * tiles_n;
    TileCoordT<I> c;
    c.s = logical / per_split;
    const I t = logical % per_split;
    if (!remap || group_m <= 1) {  // plain raster, n fastest
        c.tm = t / tiles_n;
        c.tn = t % tiles_n;
        return c;
    }
    const I in_group = (I)group_m * tiles_n;
    const I first_m = (t / in_group) * group_m;
    I rows = tiles_m - first_m;
    if (rows > group_m)
        rows = group_m;
    const I r = t % in_group;
    c.tm = first_m + r % rows;
    c.tn = r / rows;
    return c;
}

// --------------------------------------------------------- buffer resources
//
// A raw buffer resource: loads at byte offsets >= num_bytes return zero and
// touch no memory.  The GEMM relies on that for rows past M, strips past N and
// the out-of-range lanes of its software pipeline.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                             0x00020000);
}

__device__ inline uint32_t clamp_bytes(int64_t n)
{
    return n <= 0 ? 0u : (n >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)n);
}

template <int AUX>
__device__ inline i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX);
}

// ------------------------------------------------------------- conversions

__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = (__bf16)lo;   // v_cvt_pk_bf16_f32: round to nearest even
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace dgp
