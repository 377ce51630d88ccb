// gfx950 backward kernels for 16-bit inputs (bf16 / fp16), without atomics.
//
// Formulas section of the "FlashAttention梯度V2" page: dV = P^T dY,
// dQ = scale dS K, dK = scale dS^T Q, with dP = dY V^T and
// dS = Ps o (dP o Z/kp - D), D_i = sum_d dY_i,d Y_i,d; Ps is rebuilt from the
// forward row statistics as exp2(S * scale * log2 e - beta_i) with
// beta_i = max_i * log2 e + log2(sum_i) (computed by the row preprocess).
//
// Two kernels; each wave owns 32 rows of the resident block:
//   dkdv: 4 waves (one per SIMD), one workgroup per (block of 128 keys, head).  Each
//         wave keeps its keys' K and V rows and dK / dV accumulators in registers,
//         and walks the 64-row query tiles that can see the block:
//           S = Q K^T, dP = dY V^T        (A from the Q / dY tile, B from K / V regs)
//           dV += Pd^T dY, dK += dS^T Q   (A straight from the S / dP accumulators)
//   dq:   8 waves (two per SIMD), one workgroup per (block of 256 queries, head).  Each wave keeps its
//         queries' Q and dY rows, row statistics and dQ^T accumulator in
//         registers, and walks the 32-row key tiles they can see:
//           S^T = K Q^T, dP^T = V dY^T    (A from the K / V tile, B from Q / dY regs)
//           dQ^T += K^T dS^T              (B straight from the dP^T accumulator)
// The dq kernel repeats S and dP (three contractions per pair instead of one)
// so that each query row's dQ has a single owner: no cross-workgroup reduction.
//
// Tiles move HBM -> LDS with buffer loads that write LDS directly (16 bytes per
// lane, lane l at byte 16*l of a 1 KiB run).  Rows are unpadded; the 16-byte
// chunks of a row are XOR-swizzled so that the row reads (one row per lane) and
// the transposing reads (four rows per 16 lanes) hit distinct banks.
#include <hip/hip_runtime.h>

#include <cstdint>

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
// Chunk c (16 bytes) of row r is stored at chunk c ^ swz(r).  For D = 128 a row fills
// all 64 banks; for D = 64 two rows share them.  Both functions make 16 consecutive
// rows read at one logical chunk land on 16 distinct chunk positions, and make
// 4 consecutive rows (first one a multiple of 4) read at two adjacent logical chunks
// land on 8 distinct positions.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) {
        return ((row & 7) << 1) | ((row >> 3) & 1);
    } else {
        return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);
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
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(desc)
                 : "memory", "m0");
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
    T t[2] = {static_cast<T>(a), static_cast<T>(b)};
    return __builtin_bit_cast(uint32_t, t);
}

template <bool V>
struct Tag {
    static constexpr bool value = V;
};

}  // namespace

// Per-lane LDS offsets (elements) of the swizzled reads.  Rows of the reads below are
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

// ------------------------------------------------------------------------------------------------
// dK / dV
// ------------------------------------------------------------------------------------------------
// Workgroup: 4 waves (one per SIMD), FA16_DKDV_BLOCK = 128 keys; wave w owns keys 32w .. 32w+31
// and walks 64-row query tiles as two 32-row halves (independent MFMA chains).

template <typename T, int D, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_dkdv16_kernel(const Bwd16Args p) {
    using vec = typename Op16<T>::vec;
    constexpr int NW = 4;
    constexpr int BQ = FA16_DKDV_TILE_Q;  // query tile rows (64)
    constexpr int MT = BQ / 32;           // 32-row halves
    constexpr int BKV = FA16_DKDV_BLOCK;  // keys per workgroup
    constexpr int NT = D / 32;
    constexpr int TI = BQ * D / 8 / 64;   // DMA instructions per query tile and tensor
    constexpr int TW = TI / NW;           // ... per wave
    static_assert(BQ == 64 && BKV == 32 * NW && TI % NW == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) T sQ[2][BQ * D];
    __shared__ __attribute__((aligned(16))) T sdY[2][BQ * D];
    __shared__ __attribute__((aligned(16))) float2 sSt[2][BQ];

    const fa_work_item_t it = p.items_kv[blockIdx.x];
    const int n = blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int j0 = it.block * BKV;
    const int jw = j0 + 32 * w + col;  // this lane's key

    LdsOffsets<D> lo_;
    lo_.init(lane);

    const T* gq = static_cast<const T*>(p.q) + static_cast<int64_t>(it.q_start) * p.q_st + n * p.q_sh;
    const T* gdy = static_cast<const T*>(p.dy) + static_cast<int64_t>(it.q_start) * p.dy_st + n * p.dy_sh;
    const float2* gstat = p.rowstat + static_cast<int64_t>(n) * p.tq + it.q_start;
    int qoff[TW];
    int dyoff[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
        qoff[u] = dma_offset<D>(w + NW * u, lane, p.q_st);
        dyoff[u] = dma_offset<D>(w + NW * u, lane, p.dy_st);
    }

    // this lane's K and V rows: B operands of S = Q K^T and dP = dY V^T
    vec kreg[D / 16];
    vec vreg[D / 16];
    {
        const bool ok = jw < K;
        const int64_t row = it.kv_start + (ok ? jw : 0);
        const vec* kr = reinterpret_cast<const vec*>(static_cast<const T*>(p.k) + row * p.k_st + n * p.k_sh);
        const vec* vr = reinterpret_cast<const vec*>(static_cast<const T*>(p.v) + row * p.v_st + n * p.v_sh);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            kreg[s] = ok ? kr[2 * s + h] : vec{};
            vreg[s] = ok ? vr[2 * s + h] : vec{};
        }
    }

    f32x16 accK[NT];
    f32x16 accV[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        accK[i] = zero16();
        accV[i] = zero16();
    }

    // HBM -> LDS copy of query tile t (Q, dY, row statistics) into buffer b
    auto issue = [&](int t, int b) {
        const int q0 = t * BQ;
        const i32x4 rq = buffer_desc(gq + static_cast<int64_t>(q0) * p.q_st, tile_bytes(L - q0, BQ, p.q_st));
        const i32x4 rd = buffer_desc(gdy + static_cast<int64_t>(q0) * p.dy_st, tile_bytes(L - q0, BQ, p.dy_st));
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            dma16_async(sQ[b] + (w + NW * u) * 512, rq, qoff[u]);
            dma16_async(sdY[b] + (w + NW * u) * 512, rd, dyoff[u]);
        }
        if (w == NW - 1 && lane < BQ / 2) {
            const i32x4 rs = buffer_desc(gstat + q0, q0 < L ? static_cast<uint32_t>(min(L - q0, BQ) * 8) : 0u);
            dma16_async(sSt[b], rs, lane * 16);
        }
    };

    if (it.tile_begin < it.tile_end) issue(it.tile_begin, 0);
    for (int t = it.tile_begin; t < it.tile_end; ++t) {
        const int b = (t - it.tile_begin) & 1;
        const T* cQ = sQ[b];
        const T* cdY = sdY[b];
        const float2* cSt = sSt[b];
        wait_dma();
        __syncthreads();  // tile t is in buffer b; every wave is done with buffer b ^ 1
        if (t + 1 < it.tile_end) issue(t + 1, b ^ 1);
        const int q0 = t * BQ;

        // S = Q K^T and dP = dY V^T (the tile's query rows x this wave's 32 keys)
        f32x16 accS[MT];
        f32x16 accP[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            accS[mt] = zero16();
            accP[mt] = zero16();
        }
        // operands of step s + 1 are read while step s runs (two steps live at most)
        vec aq[2][MT];
        vec ad[2][MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            aq[0][mt] = lds_row<vec>(cQ + 32 * mt * D, lo_.row[0]);
            ad[0][mt] = lds_row<vec>(cdY + 32 * mt * D, lo_.row[0]);
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int c = s & 1;
            if (s + 1 < D / 16) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    aq[c ^ 1][mt] = lds_row<vec>(cQ + 32 * mt * D, lo_.row[s + 1]);
                    ad[c ^ 1][mt] = lds_row<vec>(cdY + 32 * mt * D, lo_.row[s + 1]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                accS[mt] = Op16<T>::mfma(aq[c][mt], kreg[s], accS[mt]);
                accP[mt] = Op16<T>::mfma(ad[c][mt], vreg[s], accP[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Ps / Pd into accS, dS into accP; element (query row 32mt + acc_row(a, h), key jw)
        bool full = (q0 + BQ <= L) && (j0 + BKV <= K);
        if (p.mode == FA_MASK_CAUSAL) {
            full = full && (j0 + BKV - 1 <= q0 + off);
        } else if (p.mode == FA_MASK_BAND) {
            full = full && (j0 >= q0 + BQ - 1 + off - p.pre) && (j0 + BKV - 1 <= q0 + off + p.nxt);
        }
        auto softmax_grad = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            int lo = 0;
            int hi = BQ - 1;
            if constexpr (MASKED) {
                hi = min(L - q0, BQ) - 1;
                if (jw >= K) hi = -1;
                if (p.mode == FA_MASK_CAUSAL) {
                    lo = max(lo, jw - off - q0);
                } else if (p.mode == FA_MASK_BAND) {
                    lo = max(lo, jw - off - p.nxt - q0);
                    hi = min(hi, jw - off + p.pre - q0);
                }
                lo -= 4 * h;
                hi -= 4 * h;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int rb = 32 * mt + 8 * g + 4 * h;
                    const f32x4 s01 = *reinterpret_cast<const f32x4*>(&cSt[rb]);
                    const f32x4 s23 = *reinterpret_cast<const f32x4*>(&cSt[rb + 2]);
                    const float dl[4] = {s01[0], s01[2], s23[0], s23[2]};
                    const float bt[4] = {s01[1], s01[3], s23[1], s23[3]};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int a = 4 * g + r;
                        const int c = 32 * mt + 8 * g + r;
                        float pv = __builtin_amdgcn_exp2f(accS[mt][a] * p.exp_scale - bt[r]);
                        bool adm = true;
                        if constexpr (MASKED) {
                            adm = (c >= lo) && (c <= hi);
                            pv = adm ? pv : 0.f;
                        }
                        if constexpr (DROP) {
                            float zk = 0.f;
                            if (adm) {
                                const int64_t bit =
                                    it.drop_base + (static_cast<int64_t>(n) * L + q0 + c + 4 * h) * K + jw;
                                zk = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
                            }
                            accP[mt][a] = pv * (accP[mt][a] * zk - dl[r]);
                            accS[mt][a] = pv * zk;
                        } else {
                            accP[mt][a] = pv * (accP[mt][a] - dl[r]);
                            accS[mt][a] = pv;
                        }
                    }
                }
            }
        };
        if (full) {
            softmax_grad(Tag<false>{});
        } else {
            softmax_grad(Tag<true>{});
        }

        // dV += Pd^T dY, dK += dS^T Q: slots 8kk..8kk+3 are rows 32mt + 16kk + 4h + 0..3,
        // slots 8kk+4..8kk+7 rows 32mt + 16kk + 8 + 4h + 0..3
        // the transposing reads of step i + 1 are issued while step i runs
        constexpr int NSTEP = MT * 2 * NT;  // (mt, kk, nt)
        vec bd[2];
        vec bq[2];
        auto tr_load = [&](int i, int slot) {
            const int nt = i % NT;
            const int rowoff = 16 * (i / NT) * D;  // 32mt + 16kk = 16 * (i / NT)
            bd[slot] = lds_tr<vec>(cdY + rowoff, lo_.tr[nt][0], lo_.tr[nt][1]);
            bq[slot] = lds_tr<vec>(cQ + rowoff, lo_.tr[nt][0], lo_.tr[nt][1]);
        };
        tr_load(0, 0);
        vec ap, as;
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            const int nt = i % NT;
            const int q16 = i / NT;  // 2 * mt + kk
            if (nt == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ap[e] = static_cast<T>(accS[q16 >> 1][8 * (q16 & 1) + e]);
                    as[e] = static_cast<T>(accP[q16 >> 1][8 * (q16 & 1) + e]);
                }
            }
            if (i + 1 < NSTEP) tr_load(i + 1, (i + 1) & 1);
            accV[nt] = Op16<T>::mfma(ap, bd[i & 1], accV[nt]);
            accK[nt] = Op16<T>::mfma(as, bq[i & 1], accK[nt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // epilogue: dK = scale * sum dS^T Q, dV = sum Pd^T dY; the lane holds column nt*32 + col
    // of key rows 8g + 4h + r
    T* gdk = static_cast<T*>(p.dk) + static_cast<int64_t>(it.kv_start) * p.dk_st + n * p.dk_sh;
    T* gdv = static_cast<T*>(p.dv) + static_cast<int64_t>(it.kv_start) * p.dv_st + n * p.dv_sh;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int j = j0 + 32 * w + acc_row(a, h);
            if (j < K) {
                gdk[static_cast<int64_t>(j) * p.dk_st + nt * 32 + col] = static_cast<T>(accK[nt][a] * p.scale);
                gdv[static_cast<int64_t>(j) * p.dv_st + nt * 32 + col] = static_cast<T>(accV[nt][a]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------------------
// Workgroup: 8 waves, FA16_DQ_BLOCK = 256 queries; wave w owns queries 32w .. 32w+31.

template <typename T, int D, bool DROP>
__global__ __launch_bounds__(512, 1) void bwd_dq16_kernel(const Bwd16Args p) {
    using vec = typename Op16<T>::vec;
    constexpr int NW = 8;
    constexpr int BQ = FA16_DQ_BLOCK;    // queries per workgroup
    constexpr int BK = FA16_DQ_TILE_K;   // key tile rows (32)
    constexpr int ND = D / 32;           // 32-row head-dim tiles of dQ^T
    constexpr int TI = BK * D / 8 / 64;  // DMA instructions per key tile and tensor
    static_assert(BQ == 32 * NW && BK == 32 && TI <= NW, "tile shape");

    __shared__ __attribute__((aligned(16))) T sK0[BK * D];
    __shared__ __attribute__((aligned(16))) T sK1[BK * D];
    __shared__ __attribute__((aligned(16))) T sV0[BK * D];
    __shared__ __attribute__((aligned(16))) T sV1[BK * D];

    const fa_work_item_t it = p.items_q[blockIdx.x];
    const int n = blockIdx.y;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int i0 = it.block * BQ + 32 * w;  // first query of this wave
    const int qi = i0 + col;                // this lane's query

    LdsOffsets<D> lo_;
    lo_.init(lane);

    const T* gk = static_cast<const T*>(p.k) + static_cast<int64_t>(it.kv_start) * p.k_st + n * p.k_sh;
    const T* gv = static_cast<const T*>(p.v) + static_cast<int64_t>(it.kv_start) * p.v_st + n * p.v_sh;
    const int koff = w < TI ? dma_offset<D>(w, lane, p.k_st) : 0;
    const int voff = w < TI ? dma_offset<D>(w, lane, p.v_st) : 0;

    // this lane's Q and dY rows (B operands of S^T = K Q^T and dP^T = V dY^T) and statistics
    vec qreg[D / 16];
    vec dyreg[D / 16];
    float delta = 0.f;
    float beta = 0.f;
    {
        const bool ok = qi < L;
        const int64_t row = it.q_start + (ok ? qi : 0);
        const vec* qr = reinterpret_cast<const vec*>(static_cast<const T*>(p.q) + row * p.q_st + n * p.q_sh);
        const vec* dr = reinterpret_cast<const vec*>(static_cast<const T*>(p.dy) + row * p.dy_st + n * p.dy_sh);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            qreg[s] = ok ? qr[2 * s + h] : vec{};
            dyreg[s] = ok ? dr[2 * s + h] : vec{};
        }
        if (ok) {
            const float2 st = p.rowstat[static_cast<int64_t>(n) * p.tq + it.q_start + qi];
            delta = st.x;
            beta = st.y;
        }
    }
    // keys this lane's query admits: [klo, khi]
    int klo = 0;
    int khi = qi < L ? K - 1 : -1;
    if (p.mode == FA_MASK_CAUSAL) {
        khi = min(khi, qi + off);
    } else if (p.mode == FA_MASK_BAND) {
        klo = max(klo, qi + off - p.pre);
        khi = min(khi, qi + off + p.nxt);
    }
    // keys admitted by every query of the wave (uniform): tiles inside need no mask
    const bool wave_rows_full = i0 + 31 < L;
    int wlo = 0;
    int whi = K - 1;
    if (p.mode == FA_MASK_CAUSAL) {
        whi = min(whi, i0 + off);
    } else if (p.mode == FA_MASK_BAND) {
        wlo = max(wlo, i0 + 31 + off - p.pre);
        whi = min(whi, i0 + off + p.nxt);
    }

    f32x16 accQ[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) accQ[i] = zero16();

    auto issue = [&](int kt, T* dK, T* dV) {
        const int k0 = kt * BK;
        if (w < TI) {
            dma_issue(dK, w, raw_rsrc(gk + static_cast<int64_t>(k0) * p.k_st, tile_bytes(K - k0, BK, p.k_st)), koff);
            dma_issue(dV, w, raw_rsrc(gv + static_cast<int64_t>(k0) * p.v_st, tile_bytes(K - k0, BK, p.v_st)), voff);
        }
    };

    auto body = [&](int kt, const T* cK, const T* cV, T* nK, T* nV) {
        wait_dma();
        __syncthreads();
        if (kt + 1 < it.tile_end) issue(kt + 1, nK, nV);
        const int k0 = kt * BK;

        // S^T = K Q^T, dP^T = V dY^T (32 keys x this wave's 32 queries)
        f32x16 accS = zero16();
        f32x16 accP = zero16();
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const vec ak = lds_row<vec>(cK, lo_.row[s]);
            const vec av = lds_row<vec>(cV, lo_.row[s]);
            accS = Op16<T>::mfma(ak, qreg[s], accS);
            accP = Op16<T>::mfma(av, dyreg[s], accP);
        }

        // dS^T = Ps (dP Z/kp - D) into accP; element (key k0 + acc_row(a, h), query qi)
        const bool full = wave_rows_full && (k0 >= wlo) && (k0 + BK - 1 <= whi);
        auto softmax_grad = [&](auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            int lo = 0;
            int hi = 0;
            if constexpr (MASKED) {
                lo = klo - k0 - 4 * h;
                hi = khi - k0 - 4 * h;
            }
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int c = 8 * (a >> 2) + (a & 3);
                float pv = __builtin_amdgcn_exp2f(accS[a] * p.exp_scale - beta);
                bool adm = true;
                if constexpr (MASKED) {
                    adm = (c >= lo) && (c <= hi);
                    pv = adm ? pv : 0.f;
                }
                if constexpr (DROP) {
                    float zk = 0.f;
                    if (adm) {
                        const int64_t bit =
                            it.drop_base + (static_cast<int64_t>(n) * L + qi) * K + k0 + c + 4 * h;
                        zk = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
                    }
                    accP[a] = pv * (accP[a] * zk - delta);
                } else {
                    accP[a] = pv * (accP[a] - delta);
                }
            }
        };
        if (full) {
            softmax_grad(Tag<false>{});
        } else {
            softmax_grad(Tag<true>{});
        }

        // dQ^T[d][q] += sum_key K[key][d] dS^T[key][q]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            vec bs;
#pragma unroll
            for (int e = 0; e < 8; ++e) bs[e] = static_cast<T>(accP[8 * kk + e]);
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
                const vec ak = lds_tr<vec>(cK + 16 * kk * D, lo_.tr[nd][0], lo_.tr[nd][1]);
                accQ[nd] = Op16<T>::mfma(ak, bs, accQ[nd]);
            }
        }
    };

    if (it.tile_begin < it.tile_end) issue(it.tile_begin, sK0, sV0);
    for (int kt = it.tile_begin; kt < it.tile_end; kt += 2) {
        body(kt, sK0, sV0, sK1, sV1);
        if (kt + 1 < it.tile_end) body(kt + 1, sK1, sV1, sK0, sV0);
    }

    // epilogue: dQ = scale * (dQ^T)^T; the lane holds query qi, head-dim rows
    // nd*32 + 8g + 4h + 0..3 (four consecutive values)
    if (qi < L) {
        T* dst = static_cast<T*>(p.dq) + static_cast<int64_t>(it.q_start + qi) * p.dq_st + n * p.dq_sh;
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t w0 = pack2<T>(accQ[nd][4 * g] * p.scale, accQ[nd][4 * g + 1] * p.scale);
                const uint32_t w1 = pack2<T>(accQ[nd][4 * g + 2] * p.scale, accQ[nd][4 * g + 3] * p.scale);
                *reinterpret_cast<uint2*>(dst + nd * 32 + 8 * g + 4 * h) = make_uint2(w0, w1);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------

template <typename T, int D, bool DROP>
static hipError_t launch_dkdv_t(const Bwd16Args& a, int64_t n, hipStream_t stream) {
    bwd_dkdv16_kernel<T, D, DROP><<<dim3(static_cast<unsigned>(n), static_cast<unsigned>(a.heads)), dim3(256), 0,
                                    stream>>>(a);
    return hipGetLastError();
}

template <typename T, int D, bool DROP>
static hipError_t launch_dq_t(const Bwd16Args& a, int64_t n, hipStream_t stream) {
    bwd_dq16_kernel<T, D, DROP><<<dim3(static_cast<unsigned>(n), static_cast<unsigned>(a.heads)), dim3(512), 0,
                                  stream>>>(a);
    return hipGetLastError();
}

#define FA_DISPATCH16(FN)                                                                        \
    if (n_items <= 0) return hipSuccess;                                                         \
    if (dtype == FA_BF16) {                                                                      \
        if (head_dim == 128)                                                                     \
            return dropout ? FN<__bf16, 128, true>(a, n_items, stream) : FN<__bf16, 128, false>(a, n_items, stream); \
        return dropout ? FN<__bf16, 64, true>(a, n_items, stream) : FN<__bf16, 64, false>(a, n_items, stream);       \
    }                                                                                            \
    if (head_dim == 128)                                                                         \
        return dropout ? FN<_Float16, 128, true>(a, n_items, stream) : FN<_Float16, 128, false>(a, n_items, stream); \
    return dropout ? FN<_Float16, 64, true>(a, n_items, stream) : FN<_Float16, 64, false>(a, n_items, stream)

hipError_t launch_dkdv16(int32_t dtype, int head_dim, bool dropout, const Bwd16Args& a, int64_t n_items,
                         hipStream_t stream) {
    FA_DISPATCH16(launch_dkdv_t);
}

hipError_t launch_dq16(int32_t dtype, int head_dim, bool dropout, const Bwd16Args& a, int64_t n_items,
                       hipStream_t stream) {
    FA_DISPATCH16(launch_dq_t);
}

#undef FA_DISPATCH16

}  // namespace fa
