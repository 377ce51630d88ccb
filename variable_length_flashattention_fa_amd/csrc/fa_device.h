// Device helpers shared by the gfx950 attention kernels (backward and forward): MFMA
// wrappers, the swizzled LDS tile layout, transposing LDS reads and the LDS DMA copies.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fa_kernels.h"

namespace fa {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((vector_size(8)));
typedef short s16x8 __attribute__((vector_size(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

template <typename T>
struct Op16;
template <>
struct Op16<__bf16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Op16<_Float16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Row (within a 32-row tile) of accumulator slot a for lane half h: 8*(a/4) + 4*h + a%4.
__device__ __forceinline__ int acc_row(int a, int h) { return 8 * (a >> 2) + 4 * h + (a & 3); }

// ---- swizzled [rows][D] tiles -----------------------------------------------------------------
// Chunk c (16 bytes) of row r is stored at chunk c ^ swz(r).  For D = 128 a row fills all 64
// banks; for D = 64 two rows share them.  The swizzle is a bijection on the chunk positions of
// 16 consecutive rows (so 16 lanes reading one logical chunk of 16 rows hit 16 distinct bank
// groups), and gives the four rows r0 .. r0+3 (r0 a multiple of 4) that a transposing read
// touches chunk blocks that do not overlap for logical chunks 0..3 (32 lanes, 16 distinct
// bank groups).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) {
        return ((row & 3) << 2) | ((row >> 2) & 3);
    } else {
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    }
}

template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
    return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// Raw buffer resource over `bytes` bytes at base: 32-bit data format, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 32 float2 row statistics {delta, beta} of a tile -> LDS (one 4-byte lane each).
__device__ __forceinline__ void dma_stats32(float2* dst, const float2* g, int valid, int lane) {
    const uint32_t bytes = valid > 0 ? static_cast<uint32_t>(min(valid, 32) * 8) : 0u;
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(g, bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 4, lane * 4, 0, 0, 0);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// vmcnt(N): all but the N most recently issued vector-memory loads have completed (loads
// complete in issue order for this count)
template <int N>
__device__ __forceinline__ void wait_dma_but() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// The same 16-byte-per-lane HBM -> LDS copy issued from inline assembly: the compiler then
// does not track the LDS write, so it adds no wait between the copy of the next tile and the
// reads of the current one.  The caller synchronises with wait_dma() and a barrier.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 d;
    d[0] = static_cast<int>(a & 0xffffffffu);
    d[1] = static_cast<int>((a >> 32) & 0xffffu);  // stride 0: raw buffer
    d[2] = static_cast<int>(bytes);
    d[3] = 0x00020000;                             // 32-bit data format
    return d;
}

template <typename T>
__device__ __forceinline__ void dma16_async(T* lds, const i32x4& desc, int voff) {
    // uniform; the read keeps it in a scalar register
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds)));
    uint32_t saved;
    // M0 is restored afterwards; the LDS DMA needs one wait state after M0 is written
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0), "v"(voff), "s"(desc)
        : "memory");
}

// One 16-byte-per-lane run of TW KiB: LDS destination m0 + 1 KiB * u + 16 * lane for
// instruction u, global source desc + v[u] + 1 KiB * u.  M0 is restored afterwards.
template <int TW>
__device__ __forceinline__ void dma_run(uint32_t m0, const i32x4& d, const int* v) {
    uint32_t saved;
    if constexpr (TW == 4) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
            "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
            "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(d)
            : "memory");
    } else if constexpr (TW == 2) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "v"(v[1]), "s"(d)
            : "memory");
    } else {
        static_assert(TW == 1, "runs of 1, 2 or 4 KiB");
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "s"(d)
            : "memory");
    }
}

// Copy of two 16-byte-per-lane runs, TW KiB of tensor a (e.g. Q of a tile) and TB KiB of tensor
// b (dY): LDS destination m0x + 1 KiB * u + 16 * lane for instruction u, global source
// desc + voff[u] + 1 KiB * u (the instruction offset moves both addresses).  With equal runs one
// M0 save / restore covers both.
template <int TW, int TB = TW>
__device__ __forceinline__ void dma_pair(uint32_t m0a, const i32x4& da, const int* va, uint32_t m0b,
                                         const i32x4& db, const int* vb) {
    uint32_t saved;
    if constexpr (TW != TB) {
        dma_run<TW>(m0a, da, va);
        dma_run<TB>(m0b, db, vb);
    } else if constexpr (TW == 4) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
            "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
            "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
            "s_mov_b32 m0, %7\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %8, %12, 0 offen lds\n\t"
            "buffer_load_dwordx4 %9, %12, 0 offen offset:1024 lds\n\t"
            "buffer_load_dwordx4 %10, %12, 0 offen offset:2048 lds\n\t"
            "buffer_load_dwordx4 %11, %12, 0 offen offset:3072 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0a), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "s"(da), "s"(m0b), "v"(vb[0]), "v"(vb[1]),
              "v"(vb[2]), "v"(vb[3]), "s"(db)
            : "memory");
    } else if constexpr (TW == 1) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
            "s_mov_b32 m0, %4\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %5, %6, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0a), "v"(va[0]), "s"(da), "s"(m0b), "v"(vb[0]), "s"(db)
            : "memory");
    } else {
        static_assert(TW == 2, "runs of 1, 2 or 4 KiB");
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds\n\t"
            "s_mov_b32 m0, %5\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %6, %8, 0 offen lds\n\t"
            "buffer_load_dwordx4 %7, %8, 0 offen offset:1024 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0a), "v"(va[0]), "v"(va[1]), "s"(da), "s"(m0b), "v"(vb[0]), "v"(vb[1]), "s"(db)
            : "memory");
    }
}

// ---- transposing LDS reads --------------------------------------------------------------------
// gfx950's ds_read_b64_tr_b16 works on groups of 16 lanes: lane j supplies the address of
// 4 consecutive 16-bit values; lane i receives element (i % 4) of the quartets of lanes
// 4e + i/4, e = 0..3.  With lane j pointing at row r0 + j/4, columns c0 + 4*(j%4), lane i
// receives X[r0 + e][c0 + i]: four consecutive rows of one column -- the MFMA operand
// layout for a contraction over the row index.
template <typename T>
__device__ __forceinline__ s16x4 ds_read_tr(const T* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 8-value operand X[r0 + e][c], X[r1 + e][c] (e = 0..3) of a swizzled tile, c = c0 + lane%16.
template <typename vec, int D, typename T>
__device__ __forceinline__ vec tr_operand(const T* tile, int r0, int r1, int c0, int i) {
    const int ra = r0 + (i >> 2);
    const int rb = r1 + (i >> 2);
    const int c = c0 + 4 * (i & 3);
    const s16x4 lo = ds_read_tr(tile + swz_off<D>(ra, c));
    const s16x4 hi = ds_read_tr(tile + swz_off<D>(rb, c));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(vec, v);
}

// Row operand: 8 consecutive columns c..c+7 (c a multiple of 8) of row r of a swizzled tile.
template <typename vec, int D, typename T>
__device__ __forceinline__ vec row_operand(const T* tile, int r, int c) {
    return *reinterpret_cast<const vec*>(tile + swz_off<D>(r, c));
}

template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, t2));  // one packed conversion
}

template <bool V>
struct Tag {
    static constexpr bool value = V;
};

template <typename T>
struct TypeTag {
    using type = T;
};



// Per-lane LDS offsets (elements) of the swizzled reads.  Kernels whose two tile kinds have
// the same row length share one set (see offsets_for).  Rows of the reads below are
// R + lane%32 (row reads) or R + 4h + (lane%16)/4 (+8) (transposing reads) with R a
// multiple of 16, so the swizzle term depends on the lane only and R*D can be added as a
// compile-time constant.
template <int D>
struct LdsOffsets {
    int row[D / 16];      // row read of columns 16s + 8h .. +7 in row lane%32
    int tr[D / 32][2];    // transposing read, columns 32t + lane%32 of rows 4h + (lane%16)/4 + 8x

    __device__ __forceinline__ void init(int lane) {
        const int col = lane & 31;
        const int h = lane >> 5;
        const int gi = lane & 15;
        const int gc = 16 * ((lane >> 4) & 1);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) row[s] = col * D + (((2 * s + h) ^ swz<D>(col)) << 3);
        const int rr = 4 * h + (gi >> 2);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = rr + 8 * x;
                const int c = 32 * t + gc + 4 * (gi & 3);
                tr[t][x] = r * D + (((c >> 3) ^ swz<D>(r)) << 3) + (c & 7);
            }
        }
    }
};

// The offsets of tiles with rows of DB elements: `a` itself when DA == DB (one register set),
// else `b`, which the caller has initialised.
template <int DA, int DB>
__device__ __forceinline__ const LdsOffsets<DB>& offsets_for(const LdsOffsets<DA>& a, const LdsOffsets<DB>& b) {
    if constexpr (DA == DB) {
        return a;
    } else {
        return b;
    }
}

template <typename vec, typename T>
__device__ __forceinline__ vec lds_row(const T* base, int off) {
    return *reinterpret_cast<const vec*>(base + off);
}

template <typename vec, typename T>
__device__ __forceinline__ vec lds_tr(const T* base, int off0, int off1) {
    const s16x4 lo = ds_read_tr(base + off0);
    const s16x4 hi = ds_read_tr(base + off1);
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(vec, v);
}

// Byte offset, within a tile whose row 0 is at the buffer base, of the 16-byte chunk that
// lane `lane` copies in DMA instruction i of a swizzled [rows][D] tile (row stride st).
template <int D>
__device__ __forceinline__ int dma_offset(int i, int lane, int64_t st) {
    constexpr int CPR = D / 8;
    const int pc = i * 64 + lane;
    const int row = pc / CPR;
    const int lc = (pc % CPR) ^ swz<D>(row);
    return static_cast<int>(row * st * 2) + lc * 16;
}

// One DMA instruction of a tile copy: 64 lanes x 16 bytes into LDS at dst + 1 KiB * i.
template <typename T>
__device__ __forceinline__ void dma_issue(T* dst, int i, __amdgpu_buffer_rsrc_t rs, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + i * 512), 16, voff, 0, 0, 0);
}

__device__ __forceinline__ uint32_t tile_bytes(int valid, int rows, int64_t st) {
    const int r = min(valid, rows);
    return r > 0 ? static_cast<uint32_t>(r * st * 2) : 0u;
}


// The (item, head) unit of this workgroup.  The hardware deals workgroups to the eight XCDs in
// turn (linear id x + y * gridDim.x; XCD = id % 8), and each XCD has its own L2.  With `grouped`
// (the host sets it when gridDim.y is a multiple of 8), XCD k runs the contiguous range k of the
// head-major order -- whole heads, each with its items in the work list's longest-first order --
// so the workgroups that read the same tiles of one (sequence, head) share an L2.  Without it the
// unit is (blockIdx.x, blockIdx.y).
struct Unit {
    int item;
    int head;
};
__device__ __forceinline__ Unit wg_unit(bool grouped) {
    if (!grouped) return {static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y)};
    const unsigned nx = gridDim.x;
    const unsigned g = blockIdx.x + blockIdx.y * nx;
    const unsigned per = (nx * gridDim.y) >> 3;
    const unsigned u = (g & 7u) * per + (g >> 3);
    return {static_cast<int>(u % nx), static_cast<int>(u / nx)};
}

template <int V>
using IC = std::integral_constant<int, V>;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(IC<I>{});
        static_for<I + 1, N>(f);
    }
}

// Empty instruction that claims to read and write x.  Volatile asm statements and LDS accesses
// keep their program order through instruction selection, so fencing the inputs and outputs
// of a piece of arithmetic pins it between its neighbours in the slot schedule below.
template <typename X>
__device__ __forceinline__ void pin(X& x) {
    asm volatile("" : "+v"(x));
}

// acc += A B with acc in accumulation registers (volatile: keeps its slot).
template <typename T>
struct MfmaAccV;
template <>
struct MfmaAccV<__bf16> {
    static __device__ __forceinline__ void run(f32x16& acc, bf16x8 a, bf16x8 b) {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
};
template <>
struct MfmaAccV<_Float16> {
    static __device__ __forceinline__ void run(f32x16& acc, f16x8 a, f16x8 b) {
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
};

}  // namespace
}  // namespace fa
