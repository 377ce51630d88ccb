// Device helpers shared by the gfx950 attention kernels (backward and forward): MFMA
// wrappers, the LDS tile layouts, transposing LDS reads and the LDS DMA copies.
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

// Raw buffer resource over `bytes` bytes at base: 32-bit data format, no swizzle.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// vmcnt(N): all but the N most recently issued vector-memory loads have completed (loads
// complete in issue order for this count)
template <int N>
__device__ __forceinline__ void wait_dma_but() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    // vmcnt is six bits: the low four at [3:0], the high two at [15:14]
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// vmcnt(PER * tiles) for a wave that issued PER loads per tile, tiles in [T, MAXT] (uniform)
template <int PER, int MAXT, int T = 0>
__device__ __forceinline__ void wait_dma_but_tiles(int tiles) {
    if constexpr (T <= MAXT) {
        if (tiles == T) {
            wait_dma_but<PER * T>();
        } else {
            wait_dma_but_tiles<PER, MAXT, T + 1>(tiles);
        }
    }
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

// TW DMA instructions of 16 bytes per lane: instruction u writes LDS at m0 + RS * u + 16 * lane
// from global desc + v[u] + RS * u (the instruction offset moves both addresses; v[u] makes up
// for it on the global side).  M0 is restored afterwards; the DMA needs one wait state after M0
// is written.
template <int TW, int RS>
__device__ __forceinline__ void dma_run(uint32_t m0, const i32x4& d, const int* v) {
    static_assert(RS * (TW - 1) < 4096, "instruction offset field");
    uint32_t saved;
    if constexpr (TW == 4) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %6, 0 offen offset:%7 lds\n\t"
            "buffer_load_dwordx4 %4, %6, 0 offen offset:%8 lds\n\t"
            "buffer_load_dwordx4 %5, %6, 0 offen offset:%9 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(d), "n"(RS), "n"(2 * RS), "n"(3 * RS)
            : "memory");
    } else if constexpr (TW == 2) {
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
            "buffer_load_dwordx4 %3, %4, 0 offen offset:%5 lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "v"(v[1]), "s"(d), "n"(RS)
            : "memory");
    } else {
        static_assert(TW == 1, "1, 2 or 4 instructions");
        asm volatile(
            "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
            "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(m0), "v"(v[0]), "s"(d)
            : "memory");
    }
}

// The copies of two tiles (e.g. Q and dY of one query tile): dma_run<TA, RA> of tensor a, then
// dma_run<TB, RB> of tensor b.
template <int TA, int RA, int TB, int RB>
__device__ __forceinline__ void dma_pair(uint32_t m0a, const i32x4& da, const int* va, uint32_t m0b,
                                         const i32x4& db, const int* vb) {
    dma_run<TA, RA>(m0a, da, va);
    dma_run<TB, RB>(m0b, db, vb);
}

// ---- [64][D] tiles of 16-bit values in LDS -----------------------------------------------------
// Every tile is copied in by DMA instructions that each fill one run: 1 KiB of contiguous LDS,
// 16 bytes per lane.  The kernels read a tile in two ways:
//   row read:  lane (col = lane % 32, h = lane / 32) reads values 16 s + 8 h .. + 7 of row R + col
//              (ds_read_b128; R a multiple of 16);
//   transposing read (ds_read_b64_tr_b16, see below): lane reads 4 values at row
//              R + 4 h + (lane % 16) / 4 + 8 x, columns 32 t + 16 ((lane / 16) % 2) + 4 (lane % 4)
//              (R a multiple of 16, x = 0 or 1).
// Tile<D> gives the layout, the DMA source offsets and each lane's read offsets (in values), so
// that a read is lds_row / lds_tr at tile + imm(...) with the lane's offset.
//
// D = 128 (rows of 256 bytes): run c (c = 0..15) starts at byte 1040 c -- 16 bytes of gap after
// each -- and holds rows j, j + 16, j + 32, j + 48 of j = jrow(c) = 8 (c % 2) + 4 ((c / 2) % 2)
// + c / 4, each row's 16-byte chunks in order.  Row r starts at byte 1040 cls(r % 16) + 256 (r / 16)
// with cls the inverse of jrow, so a row starts at bank group cls(r % 16) (1040 = 16 mod 256):
// - a row read's 16 lanes of one 256-byte transfer cover rows R .. R + 15, whose cls are all
//   distinct: 16 distinct bank groups;
// - a transposing read's 32 lanes of one transfer cover rows r0 .. r0 + 3 (r0 = 4 h + 8 x + R)
//   over 64 bytes each; their cls are 4 apart, so the four 64-byte pieces do not share a bank;
// - and every offset that varies between the reads of a lane is a constant: one lane offset per
//   read kind serves the whole tile (and any tile at a fixed distance from it), the rest goes
//   into the instruction's offset field.
// D = 64 (rows of 128 bytes): rows are contiguous and chunk c of row r sits at c ^ swz(r), with
// swz(r) = 4 ((r / 2) % 2) + (r / 4) % 4: 16 lanes reading one logical chunk of rows R .. R + 15
// hit 16 distinct bank groups, and the four rows of a transposing read occupy disjoint 64-byte
// pieces; the per-lane offsets then differ per chunk (one register per s and per (t, x)).
template <int D>
struct Tile;

template <>
struct Tile<128> {
    static constexpr int kRunBytes = 1040;
    static constexpr int kElems = 16 * kRunBytes / 2;  // values of LDS one tile spans
    static __host__ __device__ __forceinline__ int cls(int j) { return 4 * (j & 3) + 2 * ((j >> 2) & 1) + ((j >> 3) & 1); }
    static __host__ __device__ __forceinline__ int jrow(int c) { return 8 * (c & 1) + 4 * ((c >> 1) & 1) + (c >> 2); }

    int rowb;  // lane offset of the row reads
    int trb;   // ... and of the transposing reads
    __host__ __device__ __forceinline__ void init(int lane) {
        const int col = lane & 31;
        const int h = lane >> 5;
        const int gi = lane & 15;
        rowb = (kRunBytes * cls(col & 15) + 256 * (col >> 4)) / 2 + 8 * h;
        trb = kRunBytes * cls(4 * h + (gi >> 2)) / 2 + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
    }
    __host__ __device__ __forceinline__ int row_off(int) const { return rowb; }
    static constexpr int row_imm(int R, int s) { return 8 * R + 16 * s; }
    __host__ __device__ __forceinline__ int tr_off(int, int) const { return trb; }
    static constexpr int tr_imm(int R, int t, int x) { return 8 * R + 32 * t + x * kRunBytes / 2; }

    // Byte offset, from the tile's row 0 in global memory (row stride st values), of the 16 bytes
    // lane `lane` copies in DMA instruction i (= run i).
    static __host__ __device__ __forceinline__ int dma_offset(int i, int lane, int64_t st) {
        const int row = jrow(i) + 16 * (lane >> 4);
        return static_cast<int>(row * st * 2) + 16 * (lane & 15);
    }
};

template <>
struct Tile<64> {
    static constexpr int kRunBytes = 1024;
    static constexpr int kElems = 64 * 64;
    static __host__ __device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

    int row[4];
    int tr[2][2];
    __host__ __device__ __forceinline__ void init(int lane) {
        const int col = lane & 31;
        const int h = lane >> 5;
        const int gi = lane & 15;
        const int gc = 16 * ((lane >> 4) & 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) row[s] = col * 64 + (((2 * s + h) ^ swz(col)) << 3);
        const int rr = 4 * h + (gi >> 2);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = rr + 8 * x;
                const int c = 32 * t + gc + 4 * (gi & 3);
                tr[t][x] = r * 64 + (((c >> 3) ^ swz(r)) << 3) + (c & 7);
            }
        }
    }
    __host__ __device__ __forceinline__ int row_off(int s) const { return row[s]; }
    static constexpr int row_imm(int R, int) { return 64 * R; }
    __host__ __device__ __forceinline__ int tr_off(int t, int x) const { return tr[t][x]; }
    static constexpr int tr_imm(int R, int, int) { return 64 * R; }

    static __host__ __device__ __forceinline__ int dma_offset(int i, int lane, int64_t st) {
        const int pc = i * 64 + lane;
        const int row = pc >> 3;
        const int lc = (pc & 7) ^ swz(row);
        return static_cast<int>(row * st * 2) + lc * 16;
    }
};

// The lane offsets of a tile of DB values per row: `a` itself when DA == DB (one register set),
// else `b`, which the caller has initialised.
template <int DA, int DB>
__device__ __forceinline__ const Tile<DB>& tile_for(const Tile<DA>& a, const Tile<DB>& b) {
    if constexpr (DA == DB) {
        return a;
    } else {
        return b;
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

template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, t2));  // one packed conversion
}

// Keep-bit records of 64 query rows for one 64-key tile, one row per lane: row `lane`'s record is
// the 16 bytes of the dropout mask that start at the word holding bit b0 + lane * K (the row's bit
// of the tile's first key), stored at dst + 4 * lane.  Its bits s .. s + 63, s = that bit mod 32,
// are the row's bits of the tile's keys (keep_windows).  A 16-byte copy that runs past the end of
// the mask may read as zero as a whole, its bytes inside the mask included, so records ending inside
// the mask are copied by LDS DMA (complete at the next wait for all loads); otherwise (the mask's
// last rows) every byte is loaded on its own, bytes past the mask reading as zero, and the lane
// stores the words itself, a word at a time in a loop kept rolled (few registers are free at the
// callers).  Uniform arguments except lane.
__device__ __forceinline__ void copy_keep_records(uint32_t* dst, const uint8_t* mask, int64_t mask_bytes,
                                                  int64_t b0, int K, int lane) {
    const int64_t byte0 = (b0 >> 5) << 2;
    const int64_t left = mask_bytes - byte0;
    const uint32_t nrec = left <= 0 ? 0u : (left >= 0xffffffffll ? 0xffffffffu : static_cast<uint32_t>(left));
    const int s0 = static_cast<int>(b0 & 31);
    const int o = 4 * ((s0 + lane * K) >> 5);
    if (4 * static_cast<int64_t>((s0 + 63 * K) >> 5) + 16 <= left) {
        dma16_async(dst, buffer_desc(mask + byte0, nrec), o);
    } else {
        const __amdgpu_buffer_rsrc_t rb = raw_rsrc(mask + byte0, nrec);
#pragma unroll 1
        for (int j = 0; j < 4; ++j) {
            uint32_t wv = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wv |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(rb, o + 4 * j + e, 0, 0)) << (8 * e);
            dst[4 * lane + j] = wv;
        }
    }
}

// The two 32-bit keep windows of a record (see copy_keep_records): bit t of win[i] is the bit of key
// 32 i + t of the tile; `bit` is the row's bit of the tile's first key (only its low 5 bits count).
__device__ __forceinline__ void keep_windows(const uint32_t* rec, uint32_t bit, uint32_t* win) {
    const uint4 r = *reinterpret_cast<const uint4*>(rec);
    win[0] = __builtin_amdgcn_alignbit(r.y, r.x, bit & 31u);
    win[1] = __builtin_amdgcn_alignbit(r.z, r.y, bit & 31u);
}

// 1 / keep_prob where bit `pos` (taken modulo 32) of `bits` is set, else 0: the sign-extended bit
// masks the bit pattern of 1 / keep_prob (`inv_keep_bits`), two instructions and no compare.
__device__ __forceinline__ float keep_scale(uint32_t bits, int pos, uint32_t inv_keep_bits) {
    const int bit = __builtin_amdgcn_sbfe(static_cast<int>(bits), static_cast<unsigned>(pos), 1u);
    return __builtin_bit_cast(float, static_cast<uint32_t>(bit) & inv_keep_bits);
}

template <bool V>
struct Tag {
    static constexpr bool value = V;
};

template <typename T>
struct TypeTag {
    using type = T;
};



template <typename vec, typename T>
__device__ __forceinline__ vec lds_row(const T* base, int off) {
    return *reinterpret_cast<const vec*>(base + off);
}

// Two transposing reads (rows r0 + e and r0 + 8 + e) forming one 8-value MFMA operand.
template <typename vec, typename T>
__device__ __forceinline__ vec lds_tr(const T* base0, int off0, const T* base1, int off1) {
    const s16x4 lo = ds_read_tr(base0 + off0);
    const s16x4 hi = ds_read_tr(base1 + off1);
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(vec, v);
}

// Row read s of rows R .. of `tile` (see Tile).
template <typename vec, int D, typename T>
__device__ __forceinline__ vec tile_row(const T* tile, const Tile<D>& lo, int R, int s) {
    return lds_row<vec>(tile + Tile<D>::row_imm(R, s), lo.row_off(s));
}

// Transposing operand of columns 32 t .. of rows R .. R + 15 of `tile` (see Tile).
template <typename vec, int D, typename T>
__device__ __forceinline__ vec tile_tr(const T* tile, const Tile<D>& lo, int R, int t) {
    return lds_tr<vec>(tile + Tile<D>::tr_imm(R, t, 0), lo.tr_off(t, 0), tile + Tile<D>::tr_imm(R, t, 1), lo.tr_off(t, 1));
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

// Empty instruction that reads x.  Volatile asm statements and LDS accesses keep their program
// order through instruction selection, so fencing the inputs and results of a piece of
// arithmetic pins it between its neighbours in the slot schedule below.  It only reads: the
// compiler puts a wait state between an asm statement that writes a register and the next
// instruction that reads it, which a fence that also claimed to write x would add at every use.
// (Device pass only: the host pass, which also instantiates the kernels, has no such registers.)
template <typename X>
__device__ __forceinline__ void pin(const X& x) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" ::"v"(x));
#else
    (void)x;
#endif
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
