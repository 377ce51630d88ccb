// Varlen attention forward for gfx950: the operator the backward's inputs come from.
//
// Formulas section of the "FlashAttention梯度V2" page (forward part): S = scale Q K^T with the
// mask applied, P = Softmax(S), Y = Dropout(P, keepProb) V.  The row statistics softmaxMax
// (max of the admitted scaled scores) and softmaxSum (sum of exp(S - max) over admitted keys)
// are written as [N, T, 8] fp32 with the value repeated over the last axis; a row with no
// admitted key gets max -inf, sum 0 and Y = 0.  Dropout keeps a pair when its mask bit is 1 and
// scales it by 1 / keepProb; the statistics are those of the softmax before dropout.
#include <cmath>

#include "fa_device.h"

namespace fa {

// ------------------------------------------------------------------------------------------------
// bf16 / fp16.  Workgroup: 8 waves (two per SIMD), FA16_DQ_BLOCK = 256 queries; wave w owns
// queries 32w .. 32w+31 and keeps their Q rows (B operands), the
// online-softmax state and an O^T accumulator.  Key tiles of FA16_DQ_TILE_K = 64 rows are
// walked as two 32-key steps:
//   S^T = K Q^T                            (A = K rows from LDS)
//   P^T = exp2(S^T scale log2e - mref)     (each lane holds one query, so its running max and
//                                           sum are scalars; the two lane halves hold 16 keys
//                                           each and combine their max every step)
//   O^T += V^T (P^T o Z / kp)              (A = transposing reads of V, B = P^T from registers)
// O^T is rescaled only when a query's max grows past its reference mref by more than 8 (in
// log2 units: P stays below 256), decided per wave, so most steps skip the rescale.

template <typename T, int DK, int DV, bool DROP, bool XM>
__global__ __launch_bounds__(512, 1) void fwd16_kernel(const FwdArgs p) {
    using vec = typename Op16<T>::vec;
    constexpr int NW = 8;
    constexpr int BQ = FA16_DQ_BLOCK;
    constexpr int BK = FA16_DQ_TILE_K;
    constexpr int ND = DV / 32;              // 32-row head-dim tiles of O^T
    constexpr int NS = DK / 16;              // MFMAs per step for S^T
    constexpr int TWK = BK * DK / 8 / 64 / NW;  // DMA instructions per wave and key tile
    constexpr int TWV = BK * DV / 8 / 64 / NW;  // ... and value tile
    static_assert(BQ == 32 * NW && BK == 64 && (BK * DV / 8 / 64) % NW == 0 && DV <= DK, "tile shape");

    __shared__ __attribute__((aligned(16))) T sK[2][Tile<DK>::kElems];
    __shared__ __attribute__((aligned(16))) T sV[2][Tile<DV>::kElems];
    // dropout keep bits of buffer b: the record of query row r of the workgroup (r = 0 .. BQ - 1) at
    // sKeep[b][4r .. 4r + 3] (copy_keep_records)
    __shared__ __attribute__((aligned(16))) uint32_t sKeep[2][DROP ? BQ * 4 : 1];

    const Unit unit = wg_unit(p.xcd_group != 0);
    const fa_work_item_t it = p.items[unit.item];
    const int n = unit.head;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int i0 = it.block * BQ + 32 * w;
    const int qi = i0 + col;

    Tile<DK> loK;
    loK.init(lane);
    Tile<DV> loV_;
    if constexpr (DK != DV) loV_.init(lane);
    const Tile<DV>& loV = tile_for(loK, loV_);

    const int hk = n / p.group;  // the key/value head this query head reads
    const T* gk = static_cast<const T*>(p.k) + static_cast<int64_t>(it.kv_start) * p.k_st + hk * p.k_sh;
    const T* gv = static_cast<const T*>(p.v) + static_cast<int64_t>(it.kv_start) * p.v_st + hk * p.v_sh;
    int koff[TWK];
    int voff[TWV];
#pragma unroll
    for (int u = 0; u < TWK; ++u) koff[u] = Tile<DK>::dma_offset(w * TWK + u, lane, p.k_st) - Tile<DK>::kRunBytes * u;
#pragma unroll
    for (int u = 0; u < TWV; ++u) voff[u] = Tile<DV>::dma_offset(w * TWV + u, lane, p.v_st) - Tile<DV>::kRunBytes * u;
    auto issue = [&](int kt, int b) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        const i32x4 rk = buffer_desc(gk + static_cast<int64_t>(k0) * p.k_st, tile_bytes(K - k0, BK, p.k_st));
        const i32x4 rv = buffer_desc(gv + static_cast<int64_t>(k0) * p.v_st, tile_bytes(K - k0, BK, p.v_st));
        const uint32_t mk = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((lds_void*)(sK[b] + w * TWK * Tile<DK>::kRunBytes / 2)));
        const uint32_t mv = static_cast<uint32_t>(
            reinterpret_cast<uintptr_t>((lds_void*)(sV[b] + w * TWV * Tile<DV>::kRunBytes / 2)));
        // keep-bit records of rows 64w .. 64w + 63 of the workgroup (waves 0 .. 3)
        if constexpr (DROP) {
            if (w < BQ / 64)
                copy_keep_records(sKeep[b] + 256 * w, p.drop_mask, p.drop_bytes,
                                  it.drop_base + (static_cast<int64_t>(n) * L + it.block * BQ + 64 * w) * K + k0, K, lane);
        }
        dma_pair<TWK, Tile<DK>::kRunBytes, TWV, Tile<DV>::kRunBytes>(__builtin_amdgcn_readfirstlane(mk), rk, koff,
                                                                     __builtin_amdgcn_readfirstlane(mv), rv, voff);
    };

    // this lane's Q row
    vec qreg[NS];
    {
        const bool ok = qi < L;
        const int64_t row = it.q_start + (ok ? qi : 0);
        const vec* qr = reinterpret_cast<const vec*>(static_cast<const T*>(p.q) + row * p.q_st + n * p.q_sh);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qreg[s] = ok ? qr[2 * s + h] : vec{};
        }
    }
    // keys this lane's query admits, [klo, khi]: element a of a step at key k0s (key
    // k0s + 4h + cc(a), cc(a) = 8*(a/4) + a%4) is admitted iff
    // (unsigned)(cc(a) - (kbase - k0s)) <= krng
    int kbase;
    int krng;
    {
        int klo = 0;
        int khi = K - 1;
        if (p.mode == FA_MASK_CAUSAL) {
            khi = min(khi, qi + off);
        } else if (p.mode == FA_MASK_BAND) {
            klo = max(klo, qi + off - p.pre);
            khi = min(khi, qi + off + p.nxt);
        }
        if (qi < L && klo <= khi) {
            kbase = klo - 4 * h;
            krng = khi - klo;
        } else {
            kbase = -(1 << 30);
            krng = 0;
        }
    }
    const bool wave_rows_full = i0 + 31 < L;
    int wlo = 0;
    int whi = K - 1;
    if (p.mode == FA_MASK_CAUSAL) {
        whi = min(whi, i0 + off);
    } else if (p.mode == FA_MASK_BAND) {
        wlo = max(wlo, i0 + 31 + off - p.pre);
        whi = min(whi, i0 + off + p.nxt);
    }
    // keys admitted by some query of the wave (uniform): a step outside them contributes nothing
    // to the wave's rows, and the wave skips its work (it still copies its part of each tile and
    // meets every barrier)
    int alo = 0;
    int ahi = i0 < L ? K - 1 : -1;
    if (p.mode == FA_MASK_CAUSAL) {
        ahi = min(ahi, i0 + 31 + off);
    } else if (p.mode == FA_MASK_BAND) {
        alo = max(alo, i0 + off - p.pre);
        ahi = min(ahi, i0 + 31 + off + p.nxt);
    }

    // explicit mask block of this (sequence, head); this lane reads row qi
    __amdgpu_buffer_rsrc_t mrs;
    if constexpr (XM) {
        const uint8_t* mb = p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn;
        mrs = raw_rsrc(mb, static_cast<uint32_t>((L - 1) * p.mask.am_sq + K));
    }

    f32x16 accO[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) accO[i] = zero16();
    float mtrue = -INFINITY;  // running max of the admitted scaled scores of this query (log2 units)
    float mref = -INFINITY;   // the max the P values and O^T are relative to
    float lsum = 0.f;         // sum of P over this lane's keys (relative to mref)

    // one 32-key step (keys k0s .. k0s + 31, rows R .. R + 31 of the tiles cK / cV); win: the
    // dropout keep bits of this lane's query for those keys (bit t = key k0s + t)
    auto kstep = [&](const T* cK, const T* cV, auto rc, int k0s, uint32_t win) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
        if (k0s > ahi || k0s + 31 < alo) return;
        // explicit mask bytes of keys k0s + 4h + cc(a), issued before the product that hides them
        uint32_t mk[16];
        if constexpr (XM) {
            const uint32_t mrow = static_cast<uint32_t>(qi) * static_cast<uint32_t>(p.mask.am_sq) +
                                  static_cast<uint32_t>(k0s + 4 * h);
#pragma unroll
            for (int a = 0; a < 16; ++a)
                mk[a] = __builtin_amdgcn_raw_buffer_load_b8(mrs, mrow + 8 * (a >> 2) + (a & 3), 0, 0);
        }
        f32x16 accS = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const vec ak = tile_row<vec>(cK, loK, R, s);
            accS = Op16<T>::mfma(ak, qreg[s], accS);
        }
        const bool full = !XM && wave_rows_full && (k0s >= wlo) && (k0s + 31 <= whi);
        float x[16];
        auto scores = [&](auto masked_tag) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int lo_h = kbase - k0s;
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                x[a] = accS[a] * p.exp_scale;
                if constexpr (MASKED) {
                    const int cc = 8 * (a >> 2) + (a & 3);
                    bool adm = static_cast<unsigned>(cc - lo_h) <= static_cast<unsigned>(krng);
                    if constexpr (XM) adm = adm && mk[a] == 0;
                    x[a] = adm ? x[a] : -INFINITY;
                }
            }
        };
        if (full) {
            scores(Tag<false>{});
        } else {
            scores(Tag<true>{});
        }
        float mloc = x[0];
#pragma unroll
        for (int a = 1; a < 16; ++a) mloc = fmaxf(mloc, x[a]);
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        mtrue = fmaxf(mtrue, mloc);
        // rescale when the max outgrew the reference (never when it is still -inf)
        const bool need = mtrue > mref + 8.f;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float alpha = need ? (mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - mtrue)) : 1.f;
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
                for (int a = 0; a < 16; ++a) accO[nd][a] *= alpha;
            }
            lsum *= alpha;
            mref = need ? mtrue : mref;
        }
        // mref is -inf only while every score so far was masked; those give P = 0
        const float mb = mref == -INFINITY ? 0.f : mref;
        uint32_t pw[2][4];
#pragma unroll
        for (int a = 0; a < 16; a += 2) {
            float pd[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float pv = __builtin_amdgcn_exp2f(x[a + e] - mb);
                lsum += pv;
                if constexpr (DROP) {
                    const int cc = 8 * ((a + e) >> 2) + ((a + e) & 3);
                    pd[e] = pv * keep_scale(win, cc + 4 * h, __builtin_bit_cast(uint32_t, p.inv_keep));
                } else {
                    pd[e] = pv;
                }
            }
            pw[a >> 3][(a & 7) >> 1] = pack2<T>(pd[0], pd[1]);
        }
        // O^T[d][q] += sum_key V[key][d] Pd^T[key][q]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const vec bp = __builtin_bit_cast(vec, make_uint4(pw[kk][0], pw[kk][1], pw[kk][2], pw[kk][3]));
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
                const vec av = tile_tr<vec>(cV, loV, R + 16 * kk, nd);
                accO[nd] = Op16<T>::mfma(av, bp, accO[nd]);
            }
        }
    };

    // one key tile in buffer B (a constant, so that every LDS address of the tile is a fixed
    // offset from the lane's own)
    auto tile = [&](int kt, auto bc) __attribute__((always_inline)) {
        constexpr int B = decltype(bc)::value;
        wait_dma();
        __syncthreads();  // tile kt is in buffer B; every wave is done with buffer B ^ 1
        if (kt + 1 < it.tile_end) issue(kt + 1, B ^ 1);
        uint32_t win[2] = {0u, 0u};
        if constexpr (DROP) {
            // this lane's keep bits for the tile's 64 keys (low five bits of the bit index only)
            keep_windows(&sKeep[B][4 * (32 * w + col)],
                         static_cast<uint32_t>(it.drop_base) +
                             (static_cast<uint32_t>(n) * static_cast<uint32_t>(L) + static_cast<uint32_t>(qi)) *
                                 static_cast<uint32_t>(K) +
                             static_cast<uint32_t>(kt * BK),
                         win);
        }
        kstep(sK[B], sV[B], IC<0>{}, kt * BK, win[0]);
        kstep(sK[B], sV[B], IC<32>{}, kt * BK + 32, win[1]);
    };
    if (it.tile_begin < it.tile_end) issue(it.tile_begin, 0);
    int kt = it.tile_begin;
    for (; kt + 1 < it.tile_end; kt += 2) {
        tile(kt, IC<0>{});
        tile(kt + 1, IC<1>{});
    }
    if (kt < it.tile_end) tile(kt, IC<0>{});

    // epilogue: the two lane halves' sums; Y = O / l; statistics in natural units
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    // Y rows: the lane holds head-dim values nd*32 + 8g + 4h + 0..3 of its query, 8 bytes of its
    // row per store, each store touching 32 rows.  Instead each wave stages its 32 rows in the
    // key-tile buffers (free after a barrier; waves 0..3, then waves 4..7) and writes whole rows
    // back, 16 bytes per lane.  Chunk c (8 values) of staged row r sits at chunk c ^ (r % CH), so
    // that the rows of a write do not all start on one bank.
    constexpr int CH = DV / 8;
    static_assert(4 * 32 * DV <= 2 * Tile<DK>::kElems, "staging area");
    T* stage = reinterpret_cast<T*>(sK) + (w & 3) * 32 * DV;
    for (int round = 0; round < 2; ++round) {
        __syncthreads();  // every wave is done with the LDS about to be overwritten
        if ((w >> 2) == round) {
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t w0 = pack2<T>(accO[nd][4 * g] * inv, accO[nd][4 * g + 1] * inv);
                    const uint32_t w1 = pack2<T>(accO[nd][4 * g + 2] * inv, accO[nd][4 * g + 3] * inv);
                    *reinterpret_cast<uint2*>(stage + col * DV + (((4 * nd + g) ^ (col % CH)) * 8) + 4 * h) =
                        make_uint2(w0, w1);
                }
            }
        }
        __syncthreads();  // the rows are staged (lanes read what other lanes wrote)
        if ((w >> 2) == round) {
#pragma unroll
            for (int i = 0; i < 32 * CH / 64; ++i) {
                const int c = lane + 64 * i;
                const int row = c / CH;
                const int q = i0 + row;
                if (q < L)
                    *reinterpret_cast<uint4*>(static_cast<T*>(p.y) + static_cast<int64_t>(it.q_start + q) * p.y_st +
                                              n * p.y_sh + (c % CH) * 8) =
                        *reinterpret_cast<const uint4*>(stage + row * DV + (((c % CH) ^ (row % CH)) * 8));
            }
        }
    }
    if (qi < L) {
        const bool empty = mtrue == -INFINITY;
        const float mnat = empty ? -INFINITY : mtrue * 0.69314718055994531f;
        const float lnat = empty ? 0.f : ltot * __builtin_amdgcn_exp2f(mref - mtrue);
        const float val = h == 0 ? mnat : lnat;
        float* srow = (h == 0 ? p.smax : p.ssum) + (static_cast<int64_t>(n) * p.tq + it.q_start + qi) * 8;
        const float4 v4 = make_float4(val, val, val, val);
        reinterpret_cast<float4*>(srow)[0] = v4;
        reinterpret_cast<float4*>(srow)[1] = v4;
    }
}

// ------------------------------------------------------------------------------------------------
// fp32: one thread per (query, head) with an online softmax over its admitted keys, the O row in
// registers.  Made for small problems.

template <int DK, int DV, bool DROP>
__global__ __launch_bounds__(FA32_FWD_BLOCK) void fwd32_kernel(const FwdArgs p) {
    const fa_work_item_t it = p.items[blockIdx.x];
    const int n = blockIdx.y;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int qi = it.block * FA32_FWD_BLOCK + static_cast<int>(threadIdx.x);
    if (qi >= L) return;
    const int off = K - L;
    int klo = 0;
    int khi = K - 1;
    if (p.mode == FA_MASK_CAUSAL) {
        khi = min(khi, qi + off);
    } else if (p.mode == FA_MASK_BAND) {
        klo = max(klo, qi + off - p.pre);
        khi = min(khi, qi + off + p.nxt);
    }
    const float* q = static_cast<const float*>(p.q) + static_cast<int64_t>(it.q_start + qi) * p.q_st + n * p.q_sh;
    const int hk = n / p.group;  // the key/value head this query head reads
    const float* kb = static_cast<const float*>(p.k) + static_cast<int64_t>(it.kv_start) * p.k_st + hk * p.k_sh;
    const float* vb = static_cast<const float*>(p.v) + static_cast<int64_t>(it.kv_start) * p.v_st + hk * p.v_sh;
    float qr[DK];
    float o[DV];
#pragma unroll
    for (int d = 0; d < DK; ++d) qr[d] = q[d];
#pragma unroll
    for (int d = 0; d < DV; ++d) o[d] = 0.f;
    const int64_t bit0 = it.drop_base + (static_cast<int64_t>(n) * L + qi) * K;
    // this query's row of the explicit mask, if any
    const uint8_t* mrow = p.mask.amask == nullptr
                              ? nullptr
                              : p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn +
                                    static_cast<int64_t>(qi) * p.mask.am_sq;
    float m = -INFINITY;
    float l = 0.f;
    for (int j = klo; j <= khi; ++j) {
        if (mrow != nullptr && mrow[j] != 0) continue;
        const float* kr = kb + static_cast<int64_t>(j) * p.k_st;
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DK; ++d) s = fmaf(qr[d], kr[d], s);
        s *= p.scale;
        if (s > m) {
            const float alpha = m == -INFINITY ? 0.f : expf(m - s);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < DV; ++d) o[d] *= alpha;
            m = s;
        }
        const float pj = expf(s - m);
        l += pj;
        float z = 1.f;
        if constexpr (DROP) {
            const int64_t bit = bit0 + j;
            z = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
        }
        const float c = pj * z;
        const float* vr = vb + static_cast<int64_t>(j) * p.v_st;
#pragma unroll
        for (int d = 0; d < DV; ++d) o[d] = fmaf(c, vr[d], o[d]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* y = static_cast<float*>(p.y) + static_cast<int64_t>(it.q_start + qi) * p.y_st + n * p.y_sh;
#pragma unroll
    for (int d = 0; d < DV; ++d) y[d] = o[d] * inv;
    const int64_t srow = (static_cast<int64_t>(n) * p.tq + it.q_start + qi) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        p.smax[srow + e] = m;
        p.ssum[srow + e] = l;
    }
}

// ------------------------------------------------------------------------------------------------

template <typename T, int DK, int DV, bool DROP, bool XM>
static hipError_t launch_fwd16_t(const FwdArgs& a, int64_t n, hipStream_t stream) {
    FwdArgs g = a;
    g.xcd_group = a.heads % 8 == 0;  // whole heads per XCD (wg_unit)
    fwd16_kernel<T, DK, DV, DROP, XM>
        <<<dim3(static_cast<unsigned>(n), static_cast<unsigned>(a.heads)), dim3(512), 0, stream>>>(g);
    return hipGetLastError();
}

// dtype parts: each instantiated in a compile part of its own (FA_FWD_PART 1 = bf16, 2 = fp16 and
// the fp32 kernels; without it, all), so that the build compiles them in parallel
template <typename T>
static hipError_t fwd16_dims(int dk, int dv, bool dropout, bool xmask, const FwdArgs& a, int64_t n,
                             hipStream_t stream) {
    auto flags = [&](auto dk_c, auto dv_c) -> hipError_t {
        constexpr int DK = decltype(dk_c)::value;
        constexpr int DV = decltype(dv_c)::value;
        if (dropout)
            return xmask ? launch_fwd16_t<T, DK, DV, true, true>(a, n, stream)
                         : launch_fwd16_t<T, DK, DV, true, false>(a, n, stream);
        return xmask ? launch_fwd16_t<T, DK, DV, false, true>(a, n, stream)
                     : launch_fwd16_t<T, DK, DV, false, false>(a, n, stream);
    };
    if (dk == 128 && dv == 128) return flags(IC<128>{}, IC<128>{});
    if (dk == 128 && dv == 64) return flags(IC<128>{}, IC<64>{});
    if (dk == 64 && dv == 64) return flags(IC<64>{}, IC<64>{});
    return hipErrorInvalidValue;
}

hipError_t fwd16_bf16(int dk, int dv, bool dropout, bool xmask, const FwdArgs& a, int64_t n, hipStream_t s);
hipError_t fwd16_f16(int dk, int dv, bool dropout, bool xmask, const FwdArgs& a, int64_t n, hipStream_t s);

#if !defined(FA_FWD_PART) || FA_FWD_PART == 1
hipError_t fwd16_bf16(int dk, int dv, bool dropout, bool xmask, const FwdArgs& a, int64_t n, hipStream_t s) {
    return fwd16_dims<__bf16>(dk, dv, dropout, xmask, a, n, s);
}

hipError_t launch_fwd16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask, const FwdArgs& a,
                        int64_t n_items, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    return dtype == FA_BF16 ? fwd16_bf16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream)
                            : fwd16_f16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream);
}
#endif

#if !defined(FA_FWD_PART) || FA_FWD_PART == 2
hipError_t fwd16_f16(int dk, int dv, bool dropout, bool xmask, const FwdArgs& a, int64_t n, hipStream_t s) {
    return fwd16_dims<_Float16>(dk, dv, dropout, xmask, a, n, s);
}

template <int DK, int DV>
static void fwd32_launch(bool dropout, const FwdArgs& a, dim3 grid, hipStream_t stream) {
    if (dropout) fwd32_kernel<DK, DV, true><<<grid, dim3(FA32_FWD_BLOCK), 0, stream>>>(a);
    else fwd32_kernel<DK, DV, false><<<grid, dim3(FA32_FWD_BLOCK), 0, stream>>>(a);
}

hipError_t launch_fwd32(int head_dim_k, int head_dim_v, bool dropout, const FwdArgs& a, int64_t n_items,
                        hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(n_items), static_cast<unsigned>(a.heads));
    if (head_dim_k == 128 && head_dim_v == 128) fwd32_launch<128, 128>(dropout, a, grid, stream);
    else if (head_dim_k == 128 && head_dim_v == 64) fwd32_launch<128, 64>(dropout, a, grid, stream);
    else if (head_dim_k == 64 && head_dim_v == 64) fwd32_launch<64, 64>(dropout, a, grid, stream);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

#endif

}  // namespace fa
