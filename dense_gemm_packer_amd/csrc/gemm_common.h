// Device helpers shared by the GEMM kernel families (gemm_tiled.hip,
// gemm_stream.hip): matrix-core operations, LDS fragment reads, the async
// global->LDS copy, and the epilogue store.
//
// Matrix-core operands.  bf16 uses v_mfma_f32_16x16x32_bf16 (the K32 MFMA
// selected for bf16 on gfx950, FlyDSL PR #1008 review excerpt) and fp8 the
// 128-deep v_mfma_f32_16x16x128_f8f6f4 (same excerpt; scale operands left at
// 0, which selects the unscaled form).  The preshuffled B fragment is passed
// as the instruction's FIRST operand and the A fragment as its second, so the
// instruction produces the 16x16 tile of C^T: lane l holds
// C[m = l%16][n = 4*(l/16) + r], r = 0..3 -- four consecutive columns of one
// row, written with a single 8-byte (bf16) or 16-byte (fp32) store.  Both
// operands use the same in-register K order, so any K permutation the
// hardware applies inside one instruction is applied to both alike.
//
// A in LDS.  The A tile is stored in the same 1 KiB operand blocks as the
// preshuffled B: block (row group rg, 64-byte K chunk c) holds, at byte
// 16*l, the 16 bytes of row 16*rg + l%16 at K-bytes 64*c + 16*(l/16).  The
// writer (the async copy, whose LDS side is linear per wave) realises this
// permutation through the global addresses of its lanes; the reader reads
// 16 consecutive bytes per lane.  Writer and reader share the one mapping,
// and both sides touch 64 distinct 16-byte bank groups per wave: no bank
// conflicts by construction.  (The pages keep a row-major tile with an XOR
// swizzle whose writer and reader had to be made to agree, FlyDSL PR #1008
// "Changes" item 2; this mapping is the same idea -- a 16-byte-granular LDS
// permutation known to both sides -- chosen for the operand order.)
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"

namespace dgp {

// ---------------------------------------------------------------- MFMA

__device__ inline f32x4 mfma_op(const i32x4 &b, const i32x4 &a, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                   __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

__device__ inline f32x4 mfma_op(const i32x8 &b, const i32x8 &a, const f32x4 &c)
{
    // cbsz = blgp = 0: both operands OCP e4m3; zero scale operands: unscaled.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
}

// Hardware-scaled e4m3 MFMA (mxfp8): eb, ea are E8M0 bytes (2^(e-127)) for the
// B fragment (first operand: lane l's byte scales row l%16 of it) and the A
// fragment (second operand: column l%16) over the K block lane l / 16 selects;
// in the operand order of this library that block is K [32q, 32q+32) of the
// 128-deep step, so an MX scale that is constant over the step (128-element
// blocks) applies to the whole step.
__device__ inline f32x4 mfma_mx(const i32x8 &b, const i32x8 &a, const f32x4 &c, int eb, int ea)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, eb, 0, ea);
}

// Hardware-scaled E2M1 MFMA (mxfp4): 16 bytes = 32 values per lane, lane l
// holding K [32g, 32g+32) (g = l/16) of its row -- exactly one 32-element
// microscaling block -- whose E8M0 scales are eb (B fragment, first operand)
// and ea (A fragment, second operand).
__device__ inline f32x4 mfma_mx4(const i32x4 &b, const i32x4 &a, const f32x4 &c, int eb, int ea)
{
    const i32x8 b8 = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
    const i32x8 a8 = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, c, 4, 4, 0, eb, 0, ea);
}

__device__ inline i32x8 cat(const i32x4 &lo, const i32x4 &hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int DT>
struct Op;
template <>
struct Op<kDtypeBf16> {
    using Frag = i32x4;
    static constexpr int kBlocks = 1;   // 1 KiB operand blocks per MFMA step (64 K-bytes)
};
template <>
struct Op<kDtypeFp8> {
    using Frag = i32x8;
    static constexpr int kBlocks = 2;   // 128 K-bytes
};
template <>
struct Op<kDtypeFp4> {
    using Frag = i32x4;
    static constexpr int kBlocks = 1;   // 64 K-bytes = 128 elements
};

template <int DT>
__device__ inline typename Op<DT>::Frag lds_frag(const uint8_t *p)
{
    if constexpr (Op<DT>::kBlocks == 1) {
        return *reinterpret_cast<const i32x4 *>(p);
    } else {
        return cat(*reinterpret_cast<const i32x4 *>(p), *reinterpret_cast<const i32x4 *>(p + 1024));
    }
}

// ------------------------------------------------------------ LDS poison
//
// The LDS-poison debug build (the library compiled a second time with
// DGP_LDS_POISON=1, libdgp_lds_poison.so) turns a kernel that reads LDS its
// copies have not filled -- a tile only partly loaded, or a read that runs
// ahead of the wait for its copy -- into a parity failure instead of a quiet
// wrong answer at full speed.  Every kernel fills its LDS with 0xFF bytes
// before its first copy (a NaN in bf16, e4m3, E8M0 and fp32; -6 in E2M1),
// and every global -> LDS copy first overwrites its own destination with
// 0xFF and waits for that write, so LDS holds poison from the moment a
// stage is handed to a copy until the copy lands.  The library built
// without the flag (kLdsPoison false, common.h) compiles none of it.
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) int lds_i32;

// Poison build: fill bytes [0, bytes) of an LDS array (bytes a multiple of
// 16) with 0xFF, spread over the workgroup's threads.  The caller
// synchronises the workgroup before the first copy.
__device__ inline void lds_poison_fill(void *lds_base, int bytes)
{
    if constexpr (kLdsPoison) {
        lds_i32x4 *d = (lds_i32x4 *)lds_base;
        for (int i = (int)threadIdx.x; i < bytes / 16; i += (int)(blockDim.x * blockDim.y * blockDim.z))
            d[i] = i32x4{-1, -1, -1, -1};
    }
}

// Async global -> LDS copy of BYTES (16, 4, 2 or 1) per lane: lane l's
// 16 bytes land at lds_dst + 16 l, a narrow copy's value zero-extended in
// dword l.  Poison build: that destination is overwritten with 0xFF first.
template <int BYTES>
__device__ inline void lds_dma(__amdgpu_buffer_rsrc_t r, void *lds_dst, uint32_t voff, uint32_t soff)
{
    static_assert(BYTES == 16 || BYTES == 4 || BYTES == 2 || BYTES == 1, "copy width");
    if constexpr (kLdsPoison) {
        const int lane = (int)(threadIdx.x & 63);
        if constexpr (BYTES == 16)
            ((lds_i32x4 *)lds_dst)[lane] = i32x4{-1, -1, -1, -1};
        else
            ((lds_i32 *)lds_dst)[lane] = -1;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    auto *d = (__attribute__((address_space(3))) void *)lds_dst;
    if constexpr (BYTES == 16)   // (the size operand must be a literal)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, voff, soff, 0, 0);
    else if constexpr (BYTES == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 4, voff, soff, 0, 0);
    else if constexpr (BYTES == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 2, voff, soff, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 1, voff, soff, 0, 0);
}

__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds_dst, uint32_t voff, uint32_t soff)
{
    lds_dma<16>(r, lds_dst, voff, soff);
}

// ------------------------------------------------------------ load ring
//
// ring_run<DEPTH>(n, load, consume) -- one wave's slice of n steps through a
// ring of DEPTH slots: load(d, i) issues step i's loads into slot d and
// consume(d, i) uses them, slot d = i % DEPTH (a compile-time index).  Loads
// run DEPTH steps ahead and are issued for steps < n only.  Every stretch of
// code is branch-free with loads and consumes in slot order (scheduling
// fences), so the compiler waits for exactly the slot a step needs: a loop
// whose iterations consume and refill DEPTH slots while at least 2*DEPTH
// steps remain, then one of 2*DEPTH straight-line tails chosen by the count
// left (a wave-uniform branch).

// The last t < 2*DEPTH steps from step i0; with PRE their first min(t, DEPTH)
// loads are issued here, else they are already in flight in slot order.
template <int DEPTH, int T, bool PRE, class Load, class Consume>
__device__ __attribute__((always_inline)) inline void ring_tail(int i0, Load &load, Consume &consume)
{
    constexpr int L = T < DEPTH ? T : DEPTH;
    if constexpr (PRE) {
#pragma unroll
        for (int d = 0; d < L; ++d) {
            load(d, i0 + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < L; ++d) {
        consume(d, i0 + d);
        if constexpr (DEPTH < T) {
            if (d + DEPTH < T)   // compile-time after unrolling
                load(d, i0 + DEPTH + d);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d + DEPTH < T; ++d) {
        consume(d, i0 + DEPTH + d);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int DEPTH, bool PRE, class Load, class Consume, int... Ts>
__device__ __attribute__((always_inline)) inline void ring_tail_of(int t, int i0, Load &load, Consume &consume, std::integer_sequence<int, Ts...>)
{
    ((t == Ts ? ring_tail<DEPTH, Ts, PRE>(i0, load, consume) : void()), ...);
}

template <int DEPTH, class Load, class Consume>
__device__ __attribute__((always_inline)) inline void ring_run(int n, Load &&load, Consume &&consume)
{
    using Counts = std::make_integer_sequence<int, 2 * DEPTH>;
    if (n < 2 * DEPTH) {
        ring_tail_of<DEPTH, true>(n, 0, load, consume, Counts{});
        return;
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    int i0 = 0;
    for (; i0 + 2 * DEPTH <= n; i0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            consume(d, i0 + d);
            load(d, i0 + DEPTH + d);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    ring_tail_of<DEPTH, false>(n - i0, i0, load, consume, Counts{});
}

// ------------------------------------------------------------- epilogue

template <int OUT>
__device__ inline void store_tile(const GemmArgs &p, int split, int m, int n, f32x4 v)
{
    if (m >= p.M || n >= p.N)
        return;
    if constexpr (OUT == kOutBf16) {
        u32x2 packed;
        packed.x = pack_bf16x2(v.x, v.y);
        packed.y = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<u32x2 *>(static_cast<uint8_t *>(p.C) + ((int64_t)m * p.N + n) * 2) = packed;
    } else {
        *reinterpret_cast<f32x4 *>(p.ws + ((int64_t)split * p.M + m) * p.N + n) = v;
    }
}

// Per-wave counts of a TM x TN workgroup tile split over WM x WN waves, with
// KT-byte k-tiles (the tiled kernel families).
template <int DT, int TM, int TN, int WM, int WN, int KT>
struct TiledShape {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kMT = TM / WM / 16;             // 16-row tiles per wave
    static constexpr int kNT = TN / WN / 16;             // 16-column strips per wave
    static constexpr int kCH = KT / 64;                  // 64-byte K chunks per k-tile
    static constexpr int kStepCh = Op<DT>::kBlocks;
    static constexpr int kSteps = kCH / kStepCh;         // MFMA k-steps per k-tile
    static constexpr int kABlocks = (TM / 16) * kCH;     // 1 KiB A blocks per k-tile
    static constexpr int kDmaPerWave = kABlocks / kWaves;
    static constexpr int kBufBytes = TM * KT;
    static constexpr int kBLoads = kNT * kCH;            // B loads per wave per k-tile
    static_assert(TM % (16 * WM) == 0 && TN % (16 * WN) == 0, "tile must split into 16x16 wave tiles");
    // The A-tile granularity rule of FlyDSL PR #974's follow-up commit (item 1):
    // the tile must split into whole 16-byte loads per thread, i.e.
    // TM*KT % (threads*16) == 0 -- with fewer loads the tail of the tile is
    // never fetched and the kernel computes on stale LDS.
    static_assert((TM * KT) % (kThreads * 16) == 0, "A tile must split into whole 16-byte loads");
    static_assert(kCH % kStepCh == 0, "k-tile must hold whole MFMA steps");
    static_assert(kCH <= 4, "B block offsets must fit the 12-bit immediate");
};

}  // namespace dgp
