// gfx950 (CDNA4) kernels of the varlen attention backward for fp32 inputs: the row pass
// (preprocess) and the dK/dV and dQ kernels.  (For bf16 / fp16 the dQ kernel does the row pass.)
//
// The backward follows the formulas section of the "FlashAttention梯度V2" page
// (dV = P^T dY, dQ = scale dS K, dK = scale dS^T Q) with the softmax Jacobian
// step dP = dY V^T, dS = Ps o (dP o Z/kp - D), D_i = sum_d dY_i,d Y_i,d, and
// Ps rebuilt from the forward's row max / row sum (the page's softmaxMax and
// softmaxSum inputs).
//
// fp32 work split, deterministic (no atomics):
//   dK/dV: one workgroup (4 wave64s) per (key block of 128 rows, key/value head).  It keeps
//          its K and V rows and dK / dV accumulators in registers and walks the query tiles
//          that can see the block, for every query head of the group; S, dP, dV and dK run
//          on the fp32 32x32x2 MFMA.
//   dQ:    two lanes per (query, head) walk the keys the query admits and recompute S and dP
//          for them (the fp32 path serves small problems; each dQ row has one owner).
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
// preprocess: row delta and folded stats
// ----------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const T* __restrict__ dy, int64_t dy_st, int64_t dy_sh,
                                                         const T* __restrict__ y, int64_t y_st, int64_t y_sh,
                                                         const float* __restrict__ smax,
                                                         const float* __restrict__ ssum,
                                                         float* __restrict__ rowstat, int64_t tq, int heads) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int TPR = D / VEC;    // threads per (token, head) row of dY and Y (D = V's head dim)
    constexpr int RPB = 256 / TPR;
    // one head per grid row, consecutive tokens per block: the statistics reads and the plane
    // writes of a block are contiguous
    const int sub = threadIdx.x % TPR;
    const int n = blockIdx.y;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / TPR;
    const bool valid = t < tq;
    float part = 0.f;
    if (valid) {
        const Chunk<T> a = *reinterpret_cast<const Chunk<T>*>(dy + t * dy_st + n * dy_sh + sub * VEC);
        const Chunk<T> b = *reinterpret_cast<const Chunk<T>*>(y + t * y_st + n * y_sh + sub * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) part += static_cast<float>(a.e[e]) * static_cast<float>(b.e[e]);
    }
#pragma unroll
    for (int m = TPR / 2; m > 0; m >>= 1) part += __shfl_xor(part, m, TPR);
    if (valid && sub == 0) {
        const int64_t s = (static_cast<int64_t>(n) * tq + t) * 8;
        const float mx = smax[s];
        const float sm = ssum[s];
        const int64_t o = static_cast<int64_t>(n) * tq + t;
        rowstat[o] = -part;
        rowstat[static_cast<int64_t>(heads) * tq + o] = -(mx * kLog2e + __builtin_amdgcn_logf(sm));
    }
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
    void* dq;
    void* dk;
    void* dv;
    int64_t dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh;
    const float* rowstat;
    const fa_work_item_t* items;    // key-block items (dK / dV)
    const fa_work_item_t* items_q;  // query-block items (dQ)
    const uint8_t* drop_mask;
    MaskArg mask;
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
    constexpr int VEC = 16 / sizeof(T);
    constexpr int VPRQ = DK / VEC;
    constexpr int VPRD = DV / VEC;

    __shared__ __attribute__((aligned(16))) T sQ[BQ * PQ];
    __shared__ __attribute__((aligned(16))) T sdY[BQ * PD];
    __shared__ __attribute__((aligned(16))) T sQt[DK * PT];
    __shared__ __attribute__((aligned(16))) T sdYt[DV * PT];
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
        // this (sequence, head) block of the explicit mask, if any
        const uint8_t* mblk =
            p.mask.amask == nullptr ? nullptr : p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn;

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
                const int64_t o = static_cast<int64_t>(n) * p.tq + it.q_start + qi;
                const int64_t plane = static_cast<int64_t>(p.heads) * p.tq;
                sStat[tid] = qi < L ? make_float2(-p.rowstat[o], -p.rowstat[plane + o]) : make_float2(0.f, 0.f);
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
            bool full = mblk == nullptr && (q0 + BQ <= L) && (j0 + BKV <= K);
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
                        if (adm && mblk != nullptr) adm = mblk[static_cast<int64_t>(i) * p.mask.am_sq + jw] == 0;
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

// dQ for fp32: two lanes per (query qi, query head n), each holding half of the head dims.
// dQ_i = scale * sum_j dS_ij K_j over the keys j that query i admits, with
// dS_ij = Ps_ij (dP_ij Z_ij / kp - D_i), Ps_ij = exp2(S_ij * scale * log2 e - beta_i) and
// dP_ij = dY_i . V_j, summed in key order.
template <int DK, int DV, bool DROP>
__global__ __launch_bounds__(2 * FA32_FWD_BLOCK) void bwd_dq32_kernel(const DevArgs p) {
    constexpr int HK = DK / 2;  // this lane's share of Q / K / dQ columns
    constexpr int HV = DV / 2;  // ... of dY / V columns
    const fa_work_item_t it = p.items_q[blockIdx.x];
    const int n = blockIdx.y;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int half = static_cast<int>(threadIdx.x & 1);
    const int qi = it.block * FA32_FWD_BLOCK + static_cast<int>(threadIdx.x >> 1);
    if (qi >= L) return;  // both lanes of a query leave together
    const int off = K - L;
    int klo = 0;
    int khi = K - 1;
    if (p.mode == FA_MASK_CAUSAL) {
        khi = min(khi, qi + off);
    } else if (p.mode == FA_MASK_BAND) {
        klo = max(klo, qi + off - p.pre);
        khi = min(khi, qi + off + p.nxt);
    }
    const int64_t row = it.q_start + qi;
    const float* q = static_cast<const float*>(p.q) + row * p.q_st + n * p.q_sh + half * HK;
    const float* dy = static_cast<const float*>(p.dy) + row * p.dy_st + n * p.dy_sh + half * HV;
    const int hk = n / p.group;  // the key/value head this query head reads
    const float* kb = static_cast<const float*>(p.k) + static_cast<int64_t>(it.kv_start) * p.k_st + hk * p.k_sh + half * HK;
    const float* vb = static_cast<const float*>(p.v) + static_cast<int64_t>(it.kv_start) * p.v_st + hk * p.v_sh + half * HV;
    float qr[HK];
    float dyr[HV];
    float acc[HK];
#pragma unroll
    for (int d = 0; d < HK; ++d) {
        qr[d] = q[d];
        acc[d] = 0.f;
    }
#pragma unroll
    for (int d = 0; d < HV; ++d) dyr[d] = dy[d];
    const int64_t so = static_cast<int64_t>(n) * p.tq + row;
    const float2 st = make_float2(-p.rowstat[so], -p.rowstat[static_cast<int64_t>(p.heads) * p.tq + so]);  // {D_i, beta_i}
    const int64_t bit0 = it.drop_base + (static_cast<int64_t>(n) * L + qi) * K;
    // this query's row of the explicit mask, if any (both lanes of the query skip the same keys)
    const uint8_t* mrow = p.mask.amask == nullptr
                              ? nullptr
                              : p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn +
                                    static_cast<int64_t>(qi) * p.mask.am_sq;
    for (int j = klo; j <= khi; ++j) {
        if (mrow != nullptr && mrow[j] != 0) continue;
        const float* kr = kb + static_cast<int64_t>(j) * p.k_st;
        const float* vr = vb + static_cast<int64_t>(j) * p.v_st;
        float sc = 0.f;
#pragma unroll
        for (int d = 0; d < HK; ++d) sc = fmaf(qr[d], kr[d], sc);
        float dp = 0.f;
#pragma unroll
        for (int d = 0; d < HV; ++d) dp = fmaf(dyr[d], vr[d], dp);
        sc += __shfl_xor(sc, 1);  // the two halves of each dot product
        dp += __shfl_xor(dp, 1);
        const float pv = __builtin_amdgcn_exp2f(sc * p.exp_scale - st.y);
        float zk = 1.f;
        if constexpr (DROP) {
            const int64_t bit = bit0 + j;
            zk = ((p.drop_mask[bit >> 3] >> (bit & 7)) & 1) ? p.inv_keep : 0.f;
        }
        const float ds = pv * (dp * zk - st.x);
#pragma unroll
        for (int d = 0; d < HK; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
    }
    float* dq = static_cast<float*>(p.dq) + row * p.dq_st + n * p.dq_sh + half * HK;
#pragma unroll
    for (int d = 0; d < HK; ++d) dq[d] = acc[d] * p.scale;
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------

template <typename T, int D>
static hipError_t preprocess_t(TensorArg dy, TensorArg y, const float* smax, const float* ssum, float* rowstat,
                               int64_t tq, int64_t heads, hipStream_t stream) {
    constexpr int TPR = D / (16 / sizeof(T));
    constexpr int RPB = 256 / TPR;
    const int64_t blocks = (tq + RPB - 1) / RPB;
    preprocess_kernel<T, D><<<dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(heads)), dim3(256), 0, stream>>>(
        static_cast<const T*>(dy.data), dy.stride_t, dy.stride_h, static_cast<const T*>(y.data), y.stride_t,
        y.stride_h, smax, ssum, rowstat, tq, static_cast<int>(heads));
    return hipGetLastError();
}

hipError_t launch_preprocess(int32_t dtype, int head_dim_v, TensorArg dy, TensorArg y, const float* smax,
                             const float* ssum, float* rowstat, int64_t tq, int64_t heads, hipStream_t stream) {
#define FA_PRE(T, D) return preprocess_t<T, D>(dy, y, smax, ssum, rowstat, tq, heads, stream)
    if (dtype == FA_BF16) { if (head_dim_v == 128) FA_PRE(__bf16, 128); FA_PRE(__bf16, 64); }
    if (dtype == FA_F16) { if (head_dim_v == 128) FA_PRE(_Float16, 128); FA_PRE(_Float16, 64); }
    if (head_dim_v == 128) FA_PRE(float, 128);
    FA_PRE(float, 64);
#undef FA_PRE
}

template <typename T, int DK, int DV, bool DROP>
static hipError_t main_t(const DevArgs& d, int64_t n_items, int heads, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(n_items), static_cast<unsigned>(heads));
    bwd_main_kernel<T, DK, DV, DROP><<<grid, dim3(256), 0, stream>>>(d);
    return hipGetLastError();
}

template <int DK, int DV, bool DROP>
static hipError_t dq32_t(const DevArgs& d, int64_t n_items, int heads, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(n_items), static_cast<unsigned>(heads));
    bwd_dq32_kernel<DK, DV, DROP><<<grid, dim3(2 * FA32_FWD_BLOCK), 0, stream>>>(d);
    return hipGetLastError();
}

static DevArgs dev_args(const MainArgs& a) {
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
    d.dq = a.dq;
    d.dk = a.dk;
    d.dv = a.dv;
    d.dq_st = a.dq_st;
    d.dq_sh = a.dq_sh;
    d.dk_st = a.dk_st;
    d.dk_sh = a.dk_sh;
    d.dv_st = a.dv_st;
    d.dv_sh = a.dv_sh;
    d.rowstat = a.rowstat;
    d.items = a.items;
    d.items_q = a.items_q;
    d.drop_mask = a.drop_mask;
    d.mask = a.mask;
    d.tq = a.tq;
    d.heads = a.heads;
    d.group = a.group;
    d.mode = a.mode;
    d.pre = a.pre;
    d.nxt = a.nxt;
    d.exp_scale = a.exp_scale;
    d.inv_keep = a.inv_keep;
    d.scale = a.scale;
    return d;
}

hipError_t launch_dq32(int head_dim_k, int head_dim_v, bool dropout, const MainArgs& a, int64_t n_items,
                       hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    const DevArgs d = dev_args(a);
#define FA_DQ32(DK, DV) \
    return dropout ? dq32_t<DK, DV, true>(d, n_items, a.heads, stream) : dq32_t<DK, DV, false>(d, n_items, a.heads, stream)
    if (head_dim_k == 128 && head_dim_v == 128) FA_DQ32(128, 128);
    if (head_dim_k == 128 && head_dim_v == 64) FA_DQ32(128, 64);
    if (head_dim_k == 64 && head_dim_v == 64) FA_DQ32(64, 64);
    return hipErrorInvalidValue;
#undef FA_DQ32
}

hipError_t launch_main(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, const MainArgs& a,
                       int64_t n_items, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    const DevArgs d = dev_args(a);
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
