// gfx950 (CDNA4) kernels of the varlen attention backward.
//
// The backward follows the formulas section of the "FlashAttention梯度V2" page
// (dV = P^T dY, dQ = scale dS K, dK = scale dS^T Q) with the softmax Jacobian
// step dP = dY V^T, dS = Ps o (dP o Z/kp - D), D_i = sum_d dY_i,d Y_i,d, and
// Ps rebuilt from the forward's row max / row sum (the page's softmaxMax and
// softmaxSum inputs).
//
// Work split: one workgroup (4 wave64s) per (key block of 128 rows, head).  The
// workgroup keeps its K and V rows and its dK / dV accumulators in registers
// and walks the query tiles that can see the block.  All five contractions run
// on 32x32 MFMA (bf16 / fp16 with fp32 accumulation; fp32 MFMA for fp32), with
// dQ accumulated in fp32 with atomics and converted by a separate pass.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_kernels.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------------------
// element traits: operand width of the 32x32 MFMA for each input type
// ----------------------------------------------------------------------------

template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
    static constexpr int KL = 8;  // operand elements per lane per MFMA (K = 2 * KL)
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Elem<_Float16> {
    static constexpr int KL = 8;
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Elem<float> {
    static constexpr int KL = 1;
    typedef float vec;
    static __device__ __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// lane element access that works for both vector and scalar operand types
template <typename V, typename T>
__device__ __forceinline__ void vset(V& v, int e, T x) { v[e] = x; }
template <>
__device__ __forceinline__ void vset<float, float>(float& v, int, float x) { v = x; }

template <typename T>
__device__ __forceinline__ T cvt(float x) { return static_cast<T>(x); }

// 16-byte chunk of a row
template <typename T>
struct alignas(16) Chunk {
    static constexpr int N = 16 / sizeof(T);
    T e[N];
};

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Row (within a 32-row MFMA tile) held by accumulator slot a of a lane in half h:
// the 32x32 output layout gives each lane one column and rows 8*(a/4) + 4*h + a%4.
__device__ __forceinline__ int acc_row(int a, int h) { return 8 * (a >> 2) + 4 * h + (a & 3); }

// ----------------------------------------------------------------------------
// preprocess: row delta, folded stats, dQ accumulator zeroing
// ----------------------------------------------------------------------------

template <typename T, int D, int DQ>
__global__ __launch_bounds__(256) void preprocess_kernel(const T* __restrict__ dy, int64_t dy_st, int64_t dy_sh,
                                                         const T* __restrict__ y, int64_t y_st, int64_t y_sh,
                                                         const float* __restrict__ smax,
                                                         const float* __restrict__ ssum,
                                                         float2* __restrict__ rowstat, float* __restrict__ dq_acc,
                                                         int64_t tq, int heads) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int TPR = D / VEC;    // threads per (token, head) row of dY and Y (D = V's head dim)
    constexpr int RPB = 256 / TPR;
    constexpr int ZPT = DQ / TPR;   // dQ accumulator floats zeroed per thread (DQ = Q's head dim)
    static_assert(ZPT % 4 == 0, "accumulator row split");
    const int sub = threadIdx.x % TPR;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
    const bool valid = r < tq * heads;
    float part = 0.f;
    int64_t t = 0;
    int n = 0;
    if (valid) {
        t = r / heads;
        n = static_cast<int>(r - t * heads);
        const Chunk<T> a = *reinterpret_cast<const Chunk<T>*>(dy + t * dy_st + n * dy_sh + sub * VEC);
        const Chunk<T> b = *reinterpret_cast<const Chunk<T>*>(y + t * y_st + n * y_sh + sub * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) part += static_cast<float>(a.e[e]) * static_cast<float>(b.e[e]);
        if (dq_acc != nullptr) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4* acc = reinterpret_cast<f32x4*>(dq_acc + (static_cast<int64_t>(n) * tq + t) * DQ + sub * ZPT);
#pragma unroll
            for (int e = 0; e < ZPT / 4; ++e) acc[e] = z;
        }
    }
#pragma unroll
    for (int m = TPR / 2; m > 0; m >>= 1) part += __shfl_xor(part, m, TPR);
    if (valid && sub == 0) {
        const int64_t s = (static_cast<int64_t>(n) * tq + t) * 8;
        const float mx = smax[s];
        const float sm = ssum[s];
        rowstat[static_cast<int64_t>(n) * tq + t] = make_float2(part, mx * kLog2e + __builtin_amdgcn_logf(sm));
    }
}

// ----------------------------------------------------------------------------
// convert: dq = scale * dq_acc
// ----------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ acc, T* __restrict__ dq, int64_t st,
                                                      int64_t sh, int64_t tq, int heads, float scale) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int TPR = D / VEC;
    constexpr int RPB = 256 / TPR;
    const int sub = threadIdx.x % TPR;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
    if (r >= tq * heads) return;
    const int64_t t = r / heads;
    const int n = static_cast<int>(r - t * heads);
    const f32x4* src = reinterpret_cast<const f32x4*>(acc + (static_cast<int64_t>(n) * tq + t) * D + sub * VEC);
    Chunk<T> out;
#pragma unroll
    for (int e = 0; e < VEC / 4; ++e) {
        const f32x4 x = src[e];
#pragma unroll
        for (int i = 0; i < 4; ++i) out.e[4 * e + i] = cvt<T>(x[i] * scale);
    }
    *reinterpret_cast<Chunk<T>*>(dq + t * st + n * sh + sub * VEC) = out;
}

// ----------------------------------------------------------------------------
// main kernel
// ----------------------------------------------------------------------------

struct DevArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dy;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, dy_st, dy_sh;
    void* dk;
    void* dv;
    int64_t dk_st, dk_sh, dv_st, dv_sh;
    const float2* rowstat;
    float* dq_acc;
    const fa_work_item_t* items;
    const uint8_t* drop_mask;
    int32_t tq, heads, group, mode, pre, nxt;  // heads: query heads; group: query heads per key/value head
    float exp_scale, inv_keep, scale;
};

template <typename T, int DK, int DV, bool DROP>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(const DevArgs p) {
    using E = Elem<T>;
    using vec = typename E::vec;
    constexpr int KL = E::KL;
    constexpr int KS = 2 * KL;                      // MFMA K
    constexpr int BQ = sizeof(T) == 4 ? 32 : 64;    // query tile rows (fp32 lists use 32)
    constexpr int BKV = 128;                        // key block rows (4 waves x 32)
    constexpr int MT = BQ / 32;                     // 32-row query sub-tiles
    constexpr int NTK = DK / 32;                    // 32-column sub-tiles of dK and dQ
    constexpr int NTV = DV / 32;                    // ... of dV
    constexpr int PADE = 16 / sizeof(T);            // 16-byte row padding
    constexpr int PQ = DK + PADE;                   // pitch of row-major Q tiles
    constexpr int PD = DV + PADE;                   // pitch of row-major dY tiles
    constexpr int PT = BQ + PADE;                   // pitch of transposed Q / dY tiles
    constexpr int PS = BKV + PADE;                  // pitch of dS and K^T
    constexpr int VEC = 16 / sizeof(T);
    constexpr int VPRQ = DK / VEC;
    constexpr int VPRD = DV / VEC;

    __shared__ __attribute__((aligned(16))) T sQ[BQ * PQ];
    __shared__ __attribute__((aligned(16))) T sdY[BQ * PD];
    __shared__ __attribute__((aligned(16))) T sQt[DK * PT];
    __shared__ __attribute__((aligned(16))) T sdYt[DV * PT];
    __shared__ __attribute__((aligned(16))) T sdS[BQ * PS];
    __shared__ __attribute__((aligned(16))) T sKt[DK * PS];
    __shared__ float2 sStat[BQ];

    const fa_work_item_t it = p.items[blockIdx.x];
    const int hk = blockIdx.y;  // key/value head; its group of query heads is walked in turn
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int j0 = it.block * BKV;
    const int jw = j0 + 32 * w + col;  // this lane's key (sequence coordinates) in S / P

    // K and V rows of this lane as B operands of S = Q K^T and dP = dY V^T
    vec kreg[DK / KS];
    vec vreg[DV / KS];
    {
        const bool ok = jw < K;
        const T* kr = static_cast<const T*>(p.k) + static_cast<int64_t>(it.kv_start + (ok ? jw : 0)) * p.k_st + hk * p.k_sh;
        const T* vr = static_cast<const T*>(p.v) + static_cast<int64_t>(it.kv_start + (ok ? jw : 0)) * p.v_st + hk * p.v_sh;
#pragma unroll
        for (int s = 0; s < DK / KS; ++s) {
#pragma unroll
            for (int e = 0; e < KL; ++e) vset(kreg[s], e, ok ? kr[s * KS + h * KL + e] : static_cast<T>(0.f));
        }
#pragma unroll
        for (int s = 0; s < DV / KS; ++s) {
#pragma unroll
            for (int e = 0; e < KL; ++e) vset(vreg[s], e, ok ? vr[s * KS + h * KL + e] : static_cast<T>(0.f));
        }
        // K^T in LDS for the dQ = dS K contraction (over keys)
#pragma unroll
        for (int s = 0; s < DK / KS; ++s) {
#pragma unroll
            for (int e = 0; e < KL; ++e) {
                T x;
                if constexpr (KL == 1) x = kreg[s]; else x = kreg[s][e];
                sKt[(s * KS + h * KL + e) * PS + 32 * w + col] = x;
            }
        }
    }

    f32x16 accK[NTK];
    f32x16 accV[NTV];
#pragma unroll
    for (int i = 0; i < NTK; ++i) accK[i] = zero16();
#pragma unroll
    for (int i = 0; i < NTV; ++i) accV[i] = zero16();

    for (int r = 0; r < p.group; ++r) {
        const int n = hk * p.group + r;  // query head
        const T* __restrict__ gq = static_cast<const T*>(p.q) + static_cast<int64_t>(it.q_start) * p.q_st + n * p.q_sh;
        const T* __restrict__ gdy = static_cast<const T*>(p.dy) + static_cast<int64_t>(it.q_start) * p.dy_st + n * p.dy_sh;
        const int64_t drop_row0 = DROP ? it.drop_base + static_cast<int64_t>(n) * L * K : 0;

        for (int t = it.tile_begin; t < it.tile_end; ++t) {
            const int q0 = t * BQ;
            __syncthreads();  // previous tile's LDS reads are done
            for (int idx = tid; idx < BQ * VPRQ; idx += 256) {
                const int r = idx / VPRQ;
                const int cv = idx - r * VPRQ;
                const int qi = q0 + r;
                Chunk<T> xq;
                if (qi < L) {
                    xq = *reinterpret_cast<const Chunk<T>*>(gq + static_cast<int64_t>(qi) * p.q_st + cv * VEC);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) xq.e[e] = static_cast<T>(0.f);
                }
                *reinterpret_cast<Chunk<T>*>(&sQ[r * PQ + cv * VEC]) = xq;
#pragma unroll
                for (int e = 0; e < VEC; ++e) sQt[(cv * VEC + e) * PT + r] = xq.e[e];
            }
            for (int idx = tid; idx < BQ * VPRD; idx += 256) {
                const int r = idx / VPRD;
                const int cv = idx - r * VPRD;
                const int qi = q0 + r;
                Chunk<T> xd;
                if (qi < L) {
                    xd = *reinterpret_cast<const Chunk<T>*>(gdy + static_cast<int64_t>(qi) * p.dy_st + cv * VEC);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) xd.e[e] = static_cast<T>(0.f);
                }
                *reinterpret_cast<Chunk<T>*>(&sdY[r * PD + cv * VEC]) = xd;
#pragma unroll
                for (int e = 0; e < VEC; ++e) sdYt[(cv * VEC + e) * PT + r] = xd.e[e];
            }
            if (tid < BQ) {
                const int qi = q0 + tid;
                sStat[tid] = qi < L ? p.rowstat[static_cast<int64_t>(n) * p.tq + it.q_start + qi] : make_float2(0.f, 0.f);
            }
            __syncthreads();

            // S = Q K^T and dP = dY V^T for this wave's 32 keys
            f32x16 accS[MT];
            f32x16 accP[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                accS[mt] = zero16();
                accP[mt] = zero16();
#pragma unroll
                for (int s = 0; s < DK / KS; ++s) {
                    const vec aq = *reinterpret_cast<const vec*>(&sQ[(mt * 32 + col) * PQ + s * KS + h * KL]);
                    accS[mt] = E::mfma(aq, kreg[s], accS[mt]);
                }
#pragma unroll
                for (int s = 0; s < DV / KS; ++s) {
                    const vec ad = *reinterpret_cast<const vec*>(&sdY[(mt * 32 + col) * PD + s * KS + h * KL]);
                    accP[mt] = E::mfma(ad, vreg[s], accP[mt]);
                }
            }

            // Is every pair of the (tile, block) admitted and in range?
            bool full = (q0 + BQ <= L) && (j0 + BKV <= K);
            if (p.mode == FA_MASK_CAUSAL) {
                full = full && (j0 + BKV - 1 <= q0 + off);
            } else if (p.mode == FA_MASK_BAND) {
                full = full && (j0 >= q0 + BQ - 1 + off - p.pre) && (j0 + BKV - 1 <= q0 + off + p.nxt);
            }

            // Ps, Pd = Ps Z / kp and dS = Ps (dP Z / kp - D), in place of S and dP
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int il = mt * 32 + acc_row(a, h);
                    const float2 st = sStat[il];
                    float pv = __builtin_amdgcn_exp2f(accS[mt][a] * p.exp_scale - st.y);
                    float zk = 1.f;
                    if (!full) {
                        const int i = q0 + il;
                        bool adm = (i < L) && (jw < K);
                        if (p.mode == FA_MASK_CAUSAL) {
                            adm = adm && (jw <= i + off);
                        } else if (p.mode == FA_MASK_BAND) {
                            adm = adm && (jw >= i + off - p.pre) && (jw <= i + off + p.nxt);
                        }
                        pv = adm ? pv : 0.f;
                        if constexpr (DROP) {
                            if (adm) {
                                const int64_t bit = drop_row0 + static_cast<int64_t>(i) * K + jw;
                                zk = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
                            }
                        }
                    } else if constexpr (DROP) {
                        const int i = q0 + il;
                        const int64_t bit = drop_row0 + static_cast<int64_t>(i) * K + jw;
                        zk = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
                    }
                    const float ds = pv * (accP[mt][a] * zk - st.x);
                    accS[mt][a] = pv * zk;
                    accP[mt][a] = ds;
                }
            }

            // dV += Pd^T dY and dK += dS^T Q: contraction over the tile's query rows,
            // taken straight from the accumulator layout (lane = key, slots = rows)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int kk = 0; kk < 32 / KS; ++kk) {
                    vec ap, as;
#pragma unroll
                    for (int e = 0; e < KL; ++e) {
                        vset(ap, e, cvt<T>(accS[mt][kk * KL + e]));
                        vset(as, e, cvt<T>(accP[mt][kk * KL + e]));
                    }
#pragma unroll
                    for (int nt = 0; nt < NTV; ++nt) {
                        vec bd;
#pragma unroll
                        for (int e = 0; e < KL; ++e)
                            vset(bd, e, sdYt[(nt * 32 + col) * PT + mt * 32 + acc_row(kk * KL + e, h)]);
                        accV[nt] = E::mfma(ap, bd, accV[nt]);
                    }
#pragma unroll
                    for (int nt = 0; nt < NTK; ++nt) {
                        vec bq;
#pragma unroll
                        for (int e = 0; e < KL; ++e)
                            vset(bq, e, sQt[(nt * 32 + col) * PT + mt * 32 + acc_row(kk * KL + e, h)]);
                        accK[nt] = E::mfma(as, bq, accK[nt]);
                    }
                }
            }

            // dS to LDS as [query][key] so dQ can contract over all 128 keys
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    sdS[(mt * 32 + acc_row(a, h)) * PS + 32 * w + col] = cvt<T>(accP[mt][a]);
                }
            }
            __syncthreads();

            // dQ_acc[tile] += dS K  (unscaled; the convert pass applies scale)
            for (int tt = w; tt < MT * NTK; tt += 4) {
                const int mq = tt / NTK;
                const int nd = tt - mq * NTK;
                f32x16 acc = zero16();
#pragma unroll
                for (int s = 0; s < BKV / KS; ++s) {
                    const vec a = *reinterpret_cast<const vec*>(&sdS[(mq * 32 + col) * PS + s * KS + h * KL]);
                    const vec b = *reinterpret_cast<const vec*>(&sKt[(nd * 32 + col) * PS + s * KS + h * KL]);
                    acc = E::mfma(a, b, acc);
                }
#pragma unroll
                for (int a = 0; a < 16; ++a) {
                    const int i = q0 + mq * 32 + acc_row(a, h);
                    if (i < L) {
                        float* dst = p.dq_acc + (static_cast<int64_t>(n) * p.tq + it.q_start + i) * DK + nd * 32 + col;
                        unsafeAtomicAdd(dst, acc[a]);
                    }
                }
            }
        }
    }  // query heads of the group

    // epilogue: dK = scale * sum dS^T Q, dV = sum Pd^T dY for this wave's 32 keys
    T* gdk = static_cast<T*>(p.dk) + static_cast<int64_t>(it.kv_start) * p.dk_st + hk * p.dk_sh;
    T* gdv = static_cast<T*>(p.dv) + static_cast<int64_t>(it.kv_start) * p.dv_st + hk * p.dv_sh;
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int j = j0 + 32 * w + acc_row(a, h);
            if (j < K) {
                gdk[static_cast<int64_t>(j) * p.dk_st + nt * 32 + col] = cvt<T>(accK[nt][a] * p.scale);
                if (nt < NTV) gdv[static_cast<int64_t>(j) * p.dv_st + nt * 32 + col] = cvt<T>(accV[nt][a]);
            }
        }
    }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

template <typename T, int D, int DQ>
static hipError_t preprocess_t(TensorArg dy, TensorArg y, const float* smax, const float* ssum, float2* rowstat,
                               float* dq_acc, int64_t tq, int64_t heads, hipStream_t stream) {
    constexpr int TPR = D / (16 / sizeof(T));
    constexpr int RPB = 256 / TPR;
    const int64_t rows = tq * heads;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    preprocess_kernel<T, D, DQ><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        static_cast<const T*>(dy.data), dy.stride_t, dy.stride_h, static_cast<const T*>(y.data), y.stride_t,
        y.stride_h, smax, ssum, rowstat, dq_acc, tq, static_cast<int>(heads));
    return hipGetLastError();
}

template <typename T>
static hipError_t preprocess_dims(int dv, int dk, TensorArg dy, TensorArg y, const float* smax, const float* ssum,
                                  float2* rowstat, float* dq_acc, int64_t tq, int64_t heads, hipStream_t stream) {
    if (dv == 128 && dk == 128) return preprocess_t<T, 128, 128>(dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
    if (dv == 64 && dk == 128) return preprocess_t<T, 64, 128>(dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
    if (dv == 64 && dk == 64) return preprocess_t<T, 64, 64>(dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_preprocess(int32_t dtype, int head_dim_v, int head_dim_k, TensorArg dy, TensorArg y,
                             const float* smax, const float* ssum, float2* rowstat, float* dq_acc, int64_t tq,
                             int64_t heads, hipStream_t stream) {
    if (dtype == FA_BF16)
        return preprocess_dims<__bf16>(head_dim_v, head_dim_k, dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
    if (dtype == FA_F16)
        return preprocess_dims<_Float16>(head_dim_v, head_dim_k, dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
    return preprocess_dims<float>(head_dim_v, head_dim_k, dy, y, smax, ssum, rowstat, dq_acc, tq, heads, stream);
}

template <typename T, int D>
static hipError_t convert_t(const float* acc, void* dq, int64_t st, int64_t sh, int64_t tq, int64_t heads,
                            float scale, hipStream_t stream) {
    constexpr int TPR = D / (16 / sizeof(T));
    constexpr int RPB = 256 / TPR;
    const int64_t rows = tq * heads;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    convert_kernel<T, D><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(
        acc, static_cast<T*>(dq), st, sh, tq, static_cast<int>(heads), scale);
    return hipGetLastError();
}

hipError_t launch_convert(int32_t dtype, int head_dim, const float* dq_acc, void* dq, int64_t dq_st, int64_t dq_sh,
                          int64_t tq, int64_t heads, float scale, hipStream_t stream) {
#define FA_CVT(T, D) return convert_t<T, D>(dq_acc, dq, dq_st, dq_sh, tq, heads, scale, stream)
    if (dtype == FA_BF16) { if (head_dim == 128) FA_CVT(__bf16, 128); FA_CVT(__bf16, 64); }
    if (dtype == FA_F16) { if (head_dim == 128) FA_CVT(_Float16, 128); FA_CVT(_Float16, 64); }
    if (head_dim == 128) FA_CVT(float, 128);
    FA_CVT(float, 64);
#undef FA_CVT
}

template <typename T, int DK, int DV, bool DROP>
static hipError_t main_t(const DevArgs& d, int64_t n_items, int heads, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(n_items), static_cast<unsigned>(heads));
    bwd_main_kernel<T, DK, DV, DROP><<<grid, dim3(256), 0, stream>>>(d);
    return hipGetLastError();
}

hipError_t launch_main(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, const MainArgs& a,
                       int64_t n_items, hipStream_t stream) {
    DevArgs d;
    d.q = a.q.data;
    d.k = a.k.data;
    d.v = a.v.data;
    d.dy = a.dy.data;
    d.q_st = a.q.stride_t;
    d.q_sh = a.q.stride_h;
    d.k_st = a.k.stride_t;
    d.k_sh = a.k.stride_h;
    d.v_st = a.v.stride_t;
    d.v_sh = a.v.stride_h;
    d.dy_st = a.dy.stride_t;
    d.dy_sh = a.dy.stride_h;
    d.dk = a.dk;
    d.dv = a.dv;
    d.dk_st = a.dk_st;
    d.dk_sh = a.dk_sh;
    d.dv_st = a.dv_st;
    d.dv_sh = a.dv_sh;
    d.rowstat = a.rowstat;
    d.dq_acc = a.dq_acc;
    d.items = a.items;
    d.drop_mask = a.drop_mask;
    d.tq = a.tq;
    d.heads = a.heads;
    d.group = a.group;
    d.mode = a.mode;
    d.pre = a.pre;
    d.nxt = a.nxt;
    d.exp_scale = a.exp_scale;
    d.inv_keep = a.inv_keep;
    d.scale = a.scale;
#define FA_MAIN(DK, DV)                                                                   \
    return dropout ? main_t<float, DK, DV, true>(d, n_items, a.heads / a.group, stream)     \
                   : main_t<float, DK, DV, false>(d, n_items, a.heads / a.group, stream)
    if (dtype != FA_F32) return hipErrorInvalidValue;  // 16-bit inputs run launch_dkdv16 / launch_dq16
    if (head_dim_k == 128 && head_dim_v == 128) FA_MAIN(128, 128);
    if (head_dim_k == 128 && head_dim_v == 64) FA_MAIN(128, 64);
    if (head_dim_k == 64 && head_dim_v == 64) FA_MAIN(64, 64);
    return hipErrorInvalidValue;
#undef FA_MAIN
}

}  // namespace fa
