// gfx950 backward kernels for 16-bit inputs (bf16 / fp16), without atomics.
//
// Formulas section of the "FlashAttention梯度V2" page: dV = P^T dY,
// dQ = scale dS K, dK = scale dS^T Q, with dP = dY V^T and
// dS = Ps o (dP o Z/kp - D), D_i = sum_d dY_i,d Y_i,d; Ps is rebuilt from the
// forward row statistics as exp2(S * scale * log2 e - beta_i) with
// beta_i = max_i * log2 e + log2(sum_i).
//
// Two kernels, launched dq first; each wave owns 32 rows of the resident block:
//   dkdv: 4 waves (one per SIMD), one workgroup per (block of 128 keys, key/value head).
//         Each wave keeps its keys' K and V rows and dK / dV accumulators in registers,
//         and walks, for every query head that reads the key/value head, the 64-row
//         query tiles that can see the block:
//           S = Q K^T, dP = dY V^T        (A from the Q / dY tile, B from K / V regs)
//           dV += Pd^T dY, dK += dS^T Q   (A straight from the S / dP accumulators)
//   dq:   8 waves (two per SIMD), one workgroup per (block of 256 queries, head).  Its prologue
//         computes D and beta of its queries (the row pass) and writes them for the dkdv kernel.
//         Each wave keeps its queries' Q and dY rows, row statistics and dQ^T accumulator in
//         registers, and walks the 32-row key tiles they can see:
//           S^T = K Q^T, dP^T = V dY^T    (A from the K / V tile, B from Q / dY regs)
//           dQ^T += K^T dS^T              (B straight from the dP^T accumulator)
// The dq kernel repeats S and dP (three contractions per pair instead of one)
// so that each query row's dQ has a single owner: no cross-workgroup reduction.
//
// Tiles move HBM -> LDS with buffer loads that write LDS directly (16 bytes per
// lane, lane l at byte 16*l of a 1 KiB run).  The runs are laid out (Tile) so that
// the row reads (one row per lane) and the transposing reads (four rows per 16
// lanes) hit distinct banks, and so that each lane reads a whole tile from one
// address register plus instruction offsets.
#include "fa_device.h"

namespace fa {

// ------------------------------------------------------------------------------------------------
// dK / dV
// ------------------------------------------------------------------------------------------------
// Workgroup: 4 waves (one per SIMD), FA16_DKDV_BLOCK = 128 keys; wave w owns keys 32w .. 32w+31.
// The query rows are walked in steps of 32 rows (two per 64-row tile) through a three-stage
// software pipeline.  Step i of a wave interleaves, slot by slot,
//   X: S and dP of step i + 1           MFMA; A = Q / dY rows (LDS), B = K / V rows (registers)
//   the softmax gradient of step i      VALU; P and dS from the S and dP made during step i - 1
//   Y: dV and dK updates of step i - 1  MFMA; A = packed P / dS, B = transposing LDS reads
// so that the exponentials and the dS arithmetic of one step run under the matrix products of
// its neighbours (one wave per SIMD: nothing else would fill the gaps).  dK and dV accumulate
// in the accumulation registers through MFMAs written in assembly; S and dP use ordinary
// VGPRs, where the VALU reads them.  Query tiles rotate through four LDS buffers (three with
// dropout or an explicit mask): while tiles t and t + 1 are read, tiles t + 2 (and t + 3) are
// copied in; one barrier per tile, between its two steps, hands the buffer of tile t - 1 back.

// Kinds of pipeline step.  For the tile in buffer b (tile t):
//   A: X = rows 32.. of tile t (buffer b), softmax = rows 0.. of tile t, Y = rows 32.. of tile
//      t - 1 (buffer b + 2); ends with the tile barrier, after which tile t + 2 is fetched into
//      buffer b + 2
//   B: X = rows 0.. of tile t + 1 (buffer b + 1), softmax = rows 32.. of tile t, Y = rows 0..
//      of tile t (buffer b)
//   FIRST: X = rows 0.. of the first tile (buffer 0) only;  LAST: Y = rows 32.. of the last
//   tile (buffer b) only.  (buffer indices mod 3)
enum StepKind { kStepA = 0, kStepB = 1, kStepFirst = 2, kStepLast = 3 };

// Order of two MFMA chains of NA and NB instructions over the slots of a step: slot j runs
// chain A (j even) or chain B (j odd) while both last, then the rest of the longer one.
// index(j) is the position of slot j's instruction within its chain.
template <int NA, int NB>
struct Interleave {
    static constexpr int M = NA < NB ? NA : NB;
    static constexpr bool is_a(int j) { return j < 2 * M ? j % 2 == 0 : NA > NB; }
    static constexpr int index(int j) { return j < 2 * M ? j / 2 : M + (j - 2 * M); }
};

// Order of two MFMA chains of NA and NB instructions in which chain A leads with LEAD
// instructions, then B and A alternate while both last, then the rest of the longer one.
template <int NA, int NB, int LEAD>
struct LeadInterleave {
    static constexpr bool pick_a(int x, int a, int b) {
        return a < NA && (b >= NB || a < LEAD || (x - LEAD) % 2 == 1);
    }
    static constexpr bool is_a(int j) {
        int a = 0, b = 0;
        for (int x = 0; x < j; ++x) (pick_a(x, a, b) ? a : b) += 1;
        return pick_a(j, a, b);
    }
    static constexpr int index(int j) {
        int a = 0, b = 0;
        for (int x = 0; x < j; ++x) (pick_a(x, a, b) ? a : b) += 1;
        return pick_a(j, a, b) ? a : b;
    }
    static constexpr int first_b() {  // slot of chain B's first instruction
        int x = 0;
        while (is_a(x)) ++x;
        return x;
    }
};

// Slots of the softmax-gradient work of element a (16 per step) among the NOPS slots: P at
// p_slot(a), dS at d_slot(a) (the same slot when NOPS == 16, P first).
constexpr int p_slot(int a, int nops) { return a * nops / 16; }
constexpr int d_slot(int a, int nops) { return (a * nops + nops / 2) / 16; }

template <typename T, int DK, int DV, bool DROP, bool XM>
__global__ __launch_bounds__(256, 1) void bwd_dkdv16_kernel(const Bwd16Args p) {
    using vec = typename Op16<T>::vec;
    constexpr int NW = 4;
    constexpr int BQ = FA16_DKDV_TILE_Q;  // query tile rows (64)
    constexpr int BKV = FA16_DKDV_BLOCK;  // keys per workgroup
    constexpr int NTK = DK / 32;          // 32-column tiles of dK
    constexpr int NTV = DV / 32;          // ... of dV
    constexpr int SK = DK / 16;           // MFMAs per step for S (as many for dK)
    constexpr int SV = DV / 16;           // ... for dP (as many for dV)
    constexpr int NX = SK + SV;           // X MFMAs per step (as many Y MFMAs)
    constexpr int NOPS = 2 * NX;          // slots per step: X and Y MFMAs alternate
    constexpr int LA = 4;                 // LDS reads run LA slots ahead of their MFMA
    // Query tile buffers.  With four, the copy of a tile has two tile periods to land before the
    // barrier that waits for it.  With an explicit mask, byte loads interleave with the tile copies
    // in the load counter, so that kernel keeps three buffers and waits for all loads.  (Dropout
    // keep bits come with the tile copies: see sKeep.)
    constexpr int NB = XM ? 3 : 4;
    constexpr int TILEQ = BQ * DK;
    constexpr int TILED = BQ * DV;
    constexpr int TWQ = TILEQ / 8 / 64 / NW;  // DMA instructions per wave and Q tile
    constexpr int TWD = TILED / 8 / 64 / NW;  // ... and dY tile
    static_assert(TWQ + TWD < 16, "load counter");
    // Without dropout the dP chain of a step starts from -D of its rows, so that it ends with
    // dP - D; with dropout the keep bit scales dP but not D, and the chain starts from zero.
    constexpr bool FOLD_D = !DROP;
    // Likewise the S chain starts from -beta of its rows, with this lane's K row scaled by
    // scale * log2(e) (once, before rounding to the operand type), so that it ends with
    // S * scale * log2(e) - beta and P = exp2(acc).  Its start block is read at the end of the step
    // before.  With an explicit mask those registers are taken: the plain form stays.
    constexpr bool FOLD_B = !XM;
    // X slots: S (chain A) and dP (chain B); S leads by LA / 2 so that the start of the dP chain
    // (-D of the step's rows) can be read from LDS LA slots ahead, within the step
    // (with dropout the chain starts at zero and the plain alternation is kept)
    using XL = LeadInterleave<SK, SV, LA / 2>;
    using XS = std::conditional_t<FOLD_D, XL, Interleave<SK, SV>>;
    constexpr int KD = FOLD_D ? 2 * XL::first_b() : LA;  // slot of the first dP MFMA
    using YS = Interleave<SV, SK>;        // Y slots: dV (chain A) and dK (chain B)
    static_assert(BQ == 64 && BKV == 32 * NW && (TILED / 8 / 64) % NW == 0 && NOPS >= 16 && LA % 2 == 0 &&
                  LA < NOPS && DV <= DK && KD >= LA, "tile shape");

    // buffer b: Q tile at sBuf[b], dY tile at sBuf[b] + TEQ (one array, so that the reads of
    // both tiles share one base address and differ by an immediate offset)
    constexpr int TEQ = Tile<DK>::kElems;  // LDS values a Q tile spans (see Tile)
    constexpr int TED = Tile<DV>::kElems;
    __shared__ __attribute__((aligned(16))) T sBuf[NB][TEQ + TED];
    // row statistics of buffer b: sSt[b][0] = -D, sSt[b][1] = -beta of the tile's rows
    __shared__ __attribute__((aligned(16))) float sSt[NB][2][BQ];
    // dropout keep bits of buffer b: row r of the tile at sKeep[b][8r .. 8r + 7], the 8 words of the
    // mask that start with the word holding the bit of (row r, the block's first key)
    __shared__ __attribute__((aligned(16))) uint32_t sKeep[NB][DROP ? BQ * 8 : 1];
    auto qtile = [&](int b) -> T* { return sBuf[b]; };
    auto dtile = [&](int b) -> T* { return sBuf[b] + TEQ; };

    const Unit unit = wg_unit(p.xcd_group != 0);
    const fa_work_item_t it = p.items_kv[unit.item];
    const int hk = unit.head;  // key/value head; query heads hk * group .. hk * group + group - 1 read it
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int j0 = it.block * BKV;
    const int jw = j0 + 32 * w + col;  // this lane's key
    // the bit of (query row q of this sequence and head n, key j0) in the dropout mask
    auto keep_bit0 = [&](int nq, int q) -> int64_t {
        return it.drop_base + (static_cast<int64_t>(nq) * L + q) * K + j0;
    };
    const uint32_t inv_keep_bits = __builtin_bit_cast(uint32_t, p.inv_keep);
    const int tb = it.tile_begin;
    const int te = it.tile_end;

    f32x16 accK[NTK];
    f32x16 accV[NTV];
#pragma unroll
    for (int i = 0; i < NTK; ++i) accK[i] = zero16();
#pragma unroll
    for (int i = 0; i < NTV; ++i) accV[i] = zero16();

    if (tb < te) {
        Tile<DK> loQ;
        loQ.init(lane);
        Tile<DV> loD_;
        if constexpr (DK != DV) loD_.init(lane);
        const Tile<DV>& loD = tile_for(loQ, loD_);

        // the query head being walked (set per head below), its tensors and (XM) its block of the
        // explicit mask
        int n = hk * p.group;
        const T* gq = nullptr;
        const T* gdy = nullptr;
        const float* gstat = nullptr;  // -D of the head's rows; beta follows one plane later
        const int64_t plane = static_cast<int64_t>(p.heads) * p.tq;
        __amdgpu_buffer_rsrc_t mrs;
        int qoff[TWQ];
        int dyoff[TWD];
        // wave w copies runs w*TWQ .. w*TWQ + TWQ - 1 of each Q tile, and likewise TWD runs of
        // each dY tile
#pragma unroll
        for (int u = 0; u < TWQ; ++u)
            qoff[u] = Tile<DK>::dma_offset(w * TWQ + u, lane, p.q_st) - Tile<DK>::kRunBytes * u;
#pragma unroll
        for (int u = 0; u < TWD; ++u)
            dyoff[u] = Tile<DV>::dma_offset(w * TWD + u, lane, p.dy_st) - Tile<DV>::kRunBytes * u;

        // this lane's K and V rows: B operands of S = Q K^T and dP = dY V^T
        vec kreg[SK];
        vec vreg[SV];
        {
            const bool ok = jw < K;
            const int64_t row = it.kv_start + (ok ? jw : 0);
            const vec* kr = reinterpret_cast<const vec*>(static_cast<const T*>(p.k) + row * p.k_st + hk * p.k_sh);
            const vec* vr = reinterpret_cast<const vec*>(static_cast<const T*>(p.v) + row * p.v_st + hk * p.v_sh);
#pragma unroll
            for (int s = 0; s < SV; ++s) {
                kreg[s] = ok ? kr[2 * s + h] : vec{};
                vreg[s] = ok ? vr[2 * s + h] : vec{};
            }
#pragma unroll
            for (int s = SV; s < SK; ++s) kreg[s] = ok ? kr[2 * s + h] : vec{};
            if constexpr (FOLD_B) {
#pragma unroll
                for (int s = 0; s < SK; ++s) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        kreg[s][e] = static_cast<T>(static_cast<float>(kreg[s][e]) * p.exp_scale);
                }
            }
            // wait for these rows here, before the tile copies are issued: a wait at their first use
            // would also wait for every copy issued before it (loads complete in issue order)
#pragma unroll
            for (int s = 0; s < SK; ++s) pin(kreg[s]);
#pragma unroll
            for (int s = 0; s < SV; ++s) pin(vreg[s]);
        }

        // Query rows this lane's key admits, [lo_row, hi_row]; the element of step rows q0s..
        // in accumulator slot a (query row q0s + 4h + cc(a), cc(a) = 8*(a/4) + a%4) is admitted
        // iff (unsigned)(cc(a) - (lo_base - q0s)) <= rng.
        int lo_base;
        int rng;
        {
            int lo_row = 0;
            int hi_row = L - 1;
            if (p.mode == FA_MASK_CAUSAL) {
                lo_row = max(0, jw - off);
            } else if (p.mode == FA_MASK_BAND) {
                lo_row = max(0, jw - off - p.nxt);
                hi_row = min(hi_row, jw - off + p.pre);
            }
            if (jw < K && lo_row <= hi_row) {
                lo_base = lo_row - 4 * h;
                rng = hi_row - lo_row;
            } else {
                lo_base = -(1 << 30);
                rng = 0;
            }
        }

        // HBM -> LDS copy of query tile t (Q, dY, row statistics) into buffer b
        auto issue = [&](int t, int b) {
            const int q0 = t * BQ;
            const i32x4 rq = buffer_desc(gq + static_cast<int64_t>(q0) * p.q_st, tile_bytes(L - q0, BQ, p.q_st));
            const i32x4 rd = buffer_desc(gdy + static_cast<int64_t>(q0) * p.dy_st, tile_bytes(L - q0, BQ, p.dy_st));
            const uint32_t mq = static_cast<uint32_t>(
                reinterpret_cast<uintptr_t>((lds_void*)(qtile(b) + w * TWQ * Tile<DK>::kRunBytes / 2)));
            const uint32_t md = static_cast<uint32_t>(
                reinterpret_cast<uintptr_t>((lds_void*)(dtile(b) + w * TWD * Tile<DV>::kRunBytes / 2)));
            // statistics and keep bits first: the last TWQ + TWD loads a wave issues for a tile are
            // its Q / dY copies
            if (w == NW - 1 && lane < BQ / 4) {
                // rows past the sequence read as zero
                const uint32_t nbytes = q0 < L ? static_cast<uint32_t>(min(L - q0, BQ) * 4) : 0u;
                dma16_async(sSt[b][0], buffer_desc(gstat + q0, nbytes), lane * 16);
                dma16_async(sSt[b][1], buffer_desc(gstat + plane + q0, nbytes), lane * 16);
            }
            if constexpr (DROP) {
                if (w == NW - 2) {
                    // 32 rows per copy, 16 bytes per lane: row r's 32 bytes start at the word holding
                    // bit B_r = B_0 + r K (its first key's bit)
                    const int64_t b0 = keep_bit0(n, q0);
                    const int64_t byte0 = (b0 >> 5) << 2;
                    const int64_t left = p.drop_bytes - byte0;
                    const uint32_t nrec =
                        left <= 0 ? 0u : (left >= 0xffffffffll ? 0xffffffffu : static_cast<uint32_t>(left));
                    const int s0 = static_cast<int>(b0 & 31);
                    // A 16-byte copy that runs past the end of the mask may read as zero as a whole,
                    // its bytes inside the mask included.  Records ending inside the mask (all but
                    // those of the mask's last rows) are copied; otherwise every byte is loaded on
                    // its own (bytes past the mask read as zero) and stored by the lane.  The byte
                    // loads are waited for here, and with them every earlier copy of this wave.
                    if (4 * static_cast<int64_t>((s0 + (BQ - 1) * K) >> 5) + 32 <= left) {
                        const i32x4 rk = buffer_desc(p.drop_mask + byte0, nrec);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const int r = 32 * i + (lane >> 1);
                            dma16_async(sKeep[b] + 256 * i, rk, 4 * ((s0 + r * K) >> 5) + 16 * (lane & 1));
                        }
                    } else {
                        const __amdgpu_buffer_rsrc_t rk = raw_rsrc(p.drop_mask + byte0, nrec);
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const int r = 32 * i + (lane >> 1);
                            const int o = 4 * ((s0 + r * K) >> 5) + 16 * (lane & 1);
                            uint32_t wv[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                wv[j] = 0;
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    wv[j] |= static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b8(rk, o + 4 * j + e, 0, 0))
                                             << (8 * e);
                            }
                            *reinterpret_cast<uint4*>(&sKeep[b][256 * i + 4 * lane]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                        }
                    }
                }
            }
            dma_pair<TWQ, Tile<DK>::kRunBytes, TWD, Tile<DV>::kRunBytes>(__builtin_amdgcn_readfirstlane(mq), rq, qoff,
                                                                         __builtin_amdgcn_readfirstlane(md), rd, dyoff);
        };

        // where a step reads: X rows 32*xm.. of buffer xb, softmax statistics of rows 32*sm..
        // of buffer sb, Y rows 32*ym.. of buffer yb
        struct Where {
            int xb, xm, sb, sm, yb, ym;
        };
        auto where = [](int kind, int b) -> Where {
            const int b1 = b == NB - 1 ? 0 : b + 1;
            const int b2 = b == 0 ? NB - 1 : b - 1;
            if (kind == kStepA) return {b, 1, b, 0, b2, 1};
            if (kind == kStepB) return {b1, 0, b, 1, b, 0};
            if (kind == kStepFirst) return {0, 0, 0, 0, 0, 0};
            return {b, 0, b, 0, b, 1};  // last
        };
        // operand of slot k of a step: k even -> X (row read of Q for S, of dY for dP), k odd ->
        // Y (transposing read of dY for dV, of Q for dK)
        auto read_op = [&](const Where& wh, auto kc) -> vec {
            constexpr int k = decltype(kc)::value;
            constexpr int j = k / 2;
            if constexpr (k % 2 == 0) {
                constexpr int s = XS::index(j);
                if constexpr (XS::is_a(j)) {
                    return tile_row<vec>(qtile(wh.xb), loQ, 32 * wh.xm, s);
                } else {
                    return tile_row<vec>(dtile(wh.xb), loD, 32 * wh.xm, s);
                }
            } else {
                constexpr int i = YS::index(j);
                if constexpr (YS::is_a(j)) {
                    constexpr int kk = i / NTV;
                    constexpr int nt = i % NTV;
                    return tile_tr<vec>(dtile(wh.yb), loD, 32 * wh.ym + 16 * kk, nt);
                } else {
                    constexpr int kk = i / NTK;
                    constexpr int nt = i % NTK;
                    return tile_tr<vec>(qtile(wh.yb), loQ, 32 * wh.ym + 16 * kk, nt);
                }
            }
        };
        // statistics of rows 32*sm + 8g + 4h + 0..3: dst[0] = -D (needed only with dropout),
        // dst[1] = -beta
        auto read_stats = [&](const Where& wh, int g, f32x4* dst) {
            const int r = 32 * wh.sm + 8 * g + 4 * h;
            if constexpr (!FOLD_D) dst[0] = *reinterpret_cast<const f32x4*>(&sSt[wh.sb][0][r]);
            if constexpr (!FOLD_B) dst[1] = *reinterpret_cast<const f32x4*>(&sSt[wh.sb][1][r]);
        };
        // -beta of the X rows, in accumulator order: the start of the S chain
        auto read_binit = [&](const Where& wh, f32x16& dst) {
            if constexpr (FOLD_B) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(&sSt[wh.xb][1][32 * wh.xm + 8 * g + 4 * h]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[4 * g + r] = v[r];
                }
            }
        };
        // -D of the X rows 32*xm + 4h + 8*(a/4) + a%4, in accumulator order: the start of the dP chain
        auto read_dinit = [&](const Where& wh, f32x16& dst) {
            if constexpr (FOLD_D) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(&sSt[wh.xb][0][32 * wh.xm + 8 * g + 4 * h]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[4 * g + r] = v[r];
                }
            }
        };

        // pipeline state carried from step to step
        vec opr[NOPS];         // operand of each slot, read LA slots ahead
        f32x4 stC[4][2];       // statistics of the softmax rows of the step
        f32x16 bC = zero16();  // start of this step's S chain (-beta of its X rows, or zero)
        f32x16 sC = zero16();  // S and dP consumed by this step's softmax gradient
        f32x16 pC = zero16();
        vec pkY[2];            // packed P and dS consumed by this step's Y (two 16-row halves)
        vec dsY[2];
        uint32_t dwC = 0;      // keep bits of this lane's key for the softmax rows (bit = row in step)
        uint32_t mkC[16];      // explicit mask bytes of the softmax rows (XM)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            pkY[i] = vec{};
            dsY[i] = vec{};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mkC[i] = 0;

        // One step (see the kinds above) of the tile in buffer b, tile index t; nkind / nb:
        // the step that follows (its first operands and statistics are read at the end).
        auto step = [&](auto kc, auto nkc, auto mc, int t, int b, int nb) {
            constexpr int KIND = decltype(kc)::value;
            constexpr int NKIND = decltype(nkc)::value;
            constexpr bool MASKED = decltype(mc)::value != 0;  // tile t has pairs outside the mask
            constexpr bool HX = KIND != kStepLast;
            constexpr bool HS = KIND == kStepA || KIND == kStepB;
            constexpr bool HY = KIND != kStepFirst;
            const Where wh = where(KIND, b);
            const Where nw = where(NKIND, nb);
            const int lo_h = lo_base - (t * BQ + 32 * wh.sm);
            f32x16 sN = zero16();
            f32x16 pN = zero16();
            f32x16 dX = zero16();  // start of this step's dP chain (-D of its X rows, or zero)
            f32x16 bN = zero16();  // start of the next step's S chain
            uint32_t pkw[2][4];
            uint32_t dsw[2][4];
            vec nopr[LA];
            f32x4 stN[2];
            float pv[16];
            float pdv[16];
            float dsv[16];
            uint32_t dwN = 0;  // keep bits of the X rows, transposed to this lane's key
            uint32_t kw[2];    // the words of this lane's row (row lane % 32 of the X rows) ...
            int ks = 0;        // ... and the bit offset of the wave's first key in them
            uint32_t mkN[16];
            // explicit mask bytes of the X rows: element a sits at mbN + cc(a) * am_sq of the block
            uint32_t mbN = 0;
            if constexpr (XM && HX) {
                const int xt = t + (KIND == kStepB ? 1 : 0);
                mbN = static_cast<uint32_t>(xt * BQ + 32 * wh.xm + 4 * h) * static_cast<uint32_t>(p.mask.am_sq) +
                      static_cast<uint32_t>(jw);
            }
            // dropout keep bits of the X rows: lane l takes the 32 bits of row l % 32 for the wave's
            // keys from its record (bit B_r + 32 w on, B_r the row's first key's bit), and a 32 x 32
            // bit transpose across each half wave leaves in lane (col, h) the bits of key j0 + 32 w +
            // col for rows 0..31 of the step: bit 4h + cc(a) is element a's
            int xrow = 0;
            if constexpr (DROP && HX) {
                const int xt = t + (KIND == kStepB ? 1 : 0);
                xrow = 32 * wh.xm + col;
                // low five bits only: 32-bit arithmetic suffices
                ks = static_cast<int>((static_cast<uint32_t>(keep_bit0(n, xt * BQ)) +
                                       static_cast<uint32_t>(xrow * K)) & 31u);
            }
            static_for<0, NOPS>([&](auto slot) {
                constexpr int k = decltype(slot)::value;
                constexpr int j = k / 2;
                // ---- the MFMA of slot k
                if constexpr (k % 2 == 0) {
                    if constexpr (HX) {
                        constexpr int s = XS::index(j);
                        vec a = opr[k];
                        pin(a);
                        if constexpr (XS::is_a(j)) {
                            sN = Op16<T>::mfma(a, kreg[s], s == 0 ? (FOLD_B ? bC : zero16()) : sN);
                            pin(sN);
                        } else {
                            pN = Op16<T>::mfma(a, vreg[s], s == 0 ? dX : pN);
                            pin(pN);
                        }
                    }
                } else {
                    if constexpr (HY) {
                        constexpr int i = YS::index(j);
                        if constexpr (YS::is_a(j)) {
                            MfmaAccV<T>::run(accV[i % NTV], pkY[i / NTV], opr[k]);
                        } else {
                            MfmaAccV<T>::run(accK[i % NTK], dsY[i / NTK], opr[k]);
                        }
                    }
                }
                // ---- softmax gradient of the elements whose parts fall in slot k: P in part
                // one, dS in part two
                if constexpr (HS) static_for<0, 16>([&](auto ac) {
                    constexpr int a = decltype(ac)::value;
                    constexpr int cc = 8 * (a / 4) + (a % 4);
                    if constexpr (p_slot(a, NOPS) == k) {
                        float x = sC[a];
                        pin(x);
                        float e;
                        if constexpr (FOLD_B) {
                            e = __builtin_amdgcn_exp2f(x);  // x = S * scale * log2(e) - beta
                        } else {
                            e = __builtin_amdgcn_exp2f(x * p.exp_scale + stC[a / 4][1][a % 4]);
                        }
                        if constexpr (MASKED) {
                            bool adm = static_cast<unsigned>(cc - lo_h) <= static_cast<unsigned>(rng);
                            if constexpr (XM) adm = adm && mkC[a] == 0;
                            pv[a] = adm ? e : 0.f;
                        } else {
                            pv[a] = e;
                        }
                        pin(pv[a]);
                    }
                    if constexpr (d_slot(a, NOPS) == k) {
                        float y = pC[a];
                        pin(y);
                        if constexpr (DROP) {
                            // z = Z / keepProb of the element; dS = P (dP z - D), Pd = P z
                            const float ndl = stC[a / 4][0][a % 4];
                            const float z = keep_scale(dwC, 4 * h + cc, inv_keep_bits);
                            pdv[a] = pv[a] * z;
                            dsv[a] = pv[a] * fmaf(y, z, ndl);
                        } else {
                            pdv[a] = pv[a];
                            dsv[a] = pv[a] * y;  // y = dP - D
                        }
                        if constexpr (a % 2 == 1) {
                            pkw[a / 8][(a % 8) / 2] = pack2<T>(pdv[a - 1], pdv[a]);
                            dsw[a / 8][(a % 8) / 2] = pack2<T>(dsv[a - 1], dsv[a]);
                            pin(pkw[a / 8][(a % 8) / 2]);
                            pin(dsw[a / 8][(a % 8) / 2]);
                        }
                    }
                });
                // ---- tile barrier: tile t + 1 has landed and every wave is done with the buffer
                // of tile t - 1, which then receives tile t + NB - 1 (with four buffers, tile t + 2
                // may still be in flight)
                if constexpr (KIND == kStepA && k == NOPS - LA) {
                    if constexpr (NB == 4) {
                        if (t + 2 < te) {
                            wait_dma_but<TWQ + TWD>();
                        } else {
                            wait_dma();
                        }
                    } else {
                        wait_dma();
                    }
                    __syncthreads();
                    if (t + NB - 1 < te) issue(t + NB - 1, wh.yb);
                }
                // ---- LDS reads for slot k + LA (of the next step near the end)
                constexpr int kr = k + LA;
                if constexpr (HX && kr == KD) read_dinit(wh, dX);
                if constexpr (kr < NOPS) {
                    if constexpr ((kr % 2 == 0 && HX) || (kr % 2 == 1 && HY)) opr[kr] = read_op(wh, IC<kr>{});
                    // statistics of elements 4g .. 4g + 3, LA slots before the first of them (group 0
                    // is read during the step before)
                    static_for<1, 4>([&](auto gc) {
                        constexpr int g = decltype(gc)::value;
                        if constexpr (HS && kr == p_slot(4 * g, NOPS)) read_stats(wh, g, stC[g]);
                    });
                } else if constexpr (KIND != kStepLast) {
                    nopr[kr - NOPS] = read_op(nw, IC<kr - NOPS>{});
                    if constexpr (kr == NOPS && (NKIND == kStepA || NKIND == kStepB)) read_stats(nw, 0, stN);
                    if constexpr (kr == NOPS && NKIND != kStepLast) read_binit(nw, bN);
                }
                // ---- dropout keep bits of the X rows: record words at slot 0, the window and the five
                // transpose stages (swap the off-diagonal j-blocks with lane ^ j) every two slots
                if constexpr (DROP && HX) {
                    if constexpr (k == 0) {
                        const uint32_t* rec = &sKeep[wh.xb][8 * xrow + w];
                        kw[0] = rec[0];
                        kw[1] = rec[1];
                    }
                    if constexpr (k == 2) dwN = __builtin_amdgcn_alignbit(kw[1], kw[0], static_cast<uint32_t>(ks));
                    if constexpr (k >= 2 && k <= 10 && k % 2 == 0) {
                        constexpr int st = k / 2 - 1;  // stage of slots 2, 4, .., 10: j = 16, 8, .., 1
                        constexpr int jj = 16 >> st;
                        constexpr uint32_t msk = jj == 16 ? 0x0000FFFFu
                                                          : jj == 8 ? 0x00FF00FFu
                                                                    : jj == 4 ? 0x0F0F0F0Fu : jj == 2 ? 0x33333333u : 0x55555555u;
                        // the partner lane's word, lane ^ j: across the two 16-lane rows of each 32
                        // lanes (j = 16) by ds_swizzle in xor mode; within a row by DPP, where a row
                        // rotate by r gives lane i the word of lane i - r (mod 16): j = 8, rotate by 8;
                        // j = 4, rotate by 12 (lane i + 4) for the lanes with bit 2 clear and by 4
                        // (lane i - 4) for the others; j = 2, 1: quad permutations
                        uint32_t yu;  // partner of the lanes with bit j clear
                        uint32_t yd;  // ... with bit j set
                        if constexpr (jj == 16) {
                            yu = static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(dwN), 0x1F | (16 << 10)));
                            yd = yu;
                        } else if constexpr (jj == 8) {
                            yu = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(dwN), 0x128, 0xF, 0xF, false));
                            yd = yu;
                        } else if constexpr (jj == 4) {
                            yu = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(dwN), 0x12C, 0xF, 0xF, false));
                            yd = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(dwN), 0x124, 0xF, 0xF, false));
                        } else {
                            constexpr int qp = jj == 2 ? 0x4E : 0xB1;  // [2,3,0,1] / [1,0,3,2]
                            yu = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(dwN), qp, 0xF, 0xF, false));
                            yd = yu;
                        }
                        // lanes with bit j clear keep their msk bits and take the partner's shifted up;
                        // the others keep their ~msk bits and take the partner's shifted down
                        const uint32_t up = (dwN & msk) | ((yu << jj) & ~msk);
                        const uint32_t dn = ((yd >> jj) & msk) | (dwN & ~msk);
                        const uint32_t sel = static_cast<uint32_t>(__builtin_amdgcn_sbfe(col, 4 - st, 1));
                        dwN = (dn & sel) | (up & ~sel);
                    }
                }
                // ---- explicit mask byte of X element k (rows past the sequence read zero or are
                // excluded by the row range anyway)
                if constexpr (XM && HX && k < 16) {
                    constexpr int cc = 8 * (k / 4) + (k % 4);
                    mkN[k] = __builtin_amdgcn_raw_buffer_load_b8(
                        mrs, mbN + static_cast<uint32_t>(cc) * static_cast<uint32_t>(p.mask.am_sq), 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            // hand the pipeline over to the next step
            if constexpr (HX) {
                sC = sN;
                pC = pN;
                if constexpr (DROP) dwC = dwN;
                if constexpr (XM) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) mkC[i] = mkN[i];
                }
            }
            if constexpr (HS) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint4 pw = make_uint4(pkw[i][0], pkw[i][1], pkw[i][2], pkw[i][3]);
                    const uint4 dw = make_uint4(dsw[i][0], dsw[i][1], dsw[i][2], dsw[i][3]);
                    pkY[i] = __builtin_bit_cast(vec, pw);
                    dsY[i] = __builtin_bit_cast(vec, dw);
                    // formed here, well before the Y MFMAs of the next step read them
                    pin(pkY[i]);
                    pin(dsY[i]);
                }
            }
            if constexpr (KIND != kStepLast) {
#pragma unroll
                for (int i = 0; i < LA; ++i) opr[i] = nopr[i];
                if constexpr (FOLD_B && NKIND != kStepLast) bC = bN;
                if constexpr (NKIND == kStepA || NKIND == kStepB) {
                    stC[0][0] = stN[0];
                    stC[0][1] = stN[1];
                }
            }
        };

        // Tiles whose 64 rows all see all 128 keys of the block need no mask.  For the causal and
        // band windows they form one run [f0, f1): rows in range (t < L / 64), keys in range, and
        // the window admits the block's corner pairs.
        int f0 = tb;
        int f1 = tb;
        {
            auto floor_div = [](int a) { return a >= 0 ? a / BQ : -((-a + BQ - 1) / BQ); };
            auto ceil_div = [&](int a) { return -floor_div(-a); };
            int lo = tb;
            int hi = min(te, L / BQ);
            if (j0 + BKV > K) hi = lo;
            if (p.mode == FA_MASK_CAUSAL) {
                lo = max(lo, ceil_div(j0 + BKV - 1 - off));
            } else if (p.mode == FA_MASK_BAND) {
                lo = max(lo, ceil_div(j0 + BKV - 1 - off - p.nxt));
                hi = min(hi, floor_div(j0 - (BQ - 1) - off + p.pre) + 1);
            }
            f0 = min(max(lo, tb), te);
            f1 = min(max(hi, f0), te);
            if (XM) {
                f0 = te;  // an explicit mask can exclude pairs anywhere: every tile is masked
                f1 = te;
            }
        }
        for (int r = 0; r < p.group; ++r) {
            n = hk * p.group + r;
            gq = static_cast<const T*>(p.q) + static_cast<int64_t>(it.q_start) * p.q_st + n * p.q_sh;
            gdy = static_cast<const T*>(p.dy) + static_cast<int64_t>(it.q_start) * p.dy_st + n * p.dy_sh;
            gstat = p.rowstat + static_cast<int64_t>(n) * p.tq + it.q_start;  // plane of -D
            if constexpr (XM) {
                const uint8_t* mb = p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn;
                mrs = raw_rsrc(mb, static_cast<uint32_t>((L - 1) * p.mask.am_sq + K));
            }
            if (r > 0) {
                // every wave is done with the previous head's tiles before they are overwritten
                __syncthreads();
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    pkY[i] = vec{};
                    dsY[i] = vec{};
                }
            }
            // prologue: tiles tb .. tb + NB - 2 in flight, zeros in the last buffer (read by the Y
            // of the step before the first, whose packed P / dS are zero)
#pragma unroll
            for (int i = 0; i < NB - 1; ++i)
                if (tb + i < te) issue(tb + i, i);
            for (int i = threadIdx.x; i < (TEQ + TED) / 8; i += 64 * NW)
                reinterpret_cast<vec*>(sBuf[NB - 1])[i] = vec{};
            // the first step needs tile tb only: the copies of the tiles after it may still be in
            // flight (a wave's copies complete in issue order; wave NW - 1 also copies each
            // tile's statistics, two more loads per tile)
            {
                const int after = min(NB - 2, te - tb - 1);
                if (w == NW - 1 || (DROP && w == NW - 2)) {
                    wait_dma_but_tiles<TWQ + TWD + 2, NB - 2>(after);
                } else {
                    wait_dma_but_tiles<TWQ + TWD, NB - 2>(after);
                }
            }
            __syncthreads();
            {
                const Where w0 = where(kStepFirst, 0);
                read_binit(w0, bC);
                static_for<0, LA>([&](auto kc) {
                    if constexpr (decltype(kc)::value % 2 == 0) opr[decltype(kc)::value] = read_op(w0, kc);
                });
            }
            step(IC<kStepFirst>{}, IC<kStepA>{}, IC<0>{}, tb, 0, 0);
            int b = 0;
            auto next_buf = [](int x) { return x == NB - 1 ? 0 : x + 1; };
            for (int t = tb; t < f0; ++t) {
                step(IC<kStepA>{}, IC<kStepB>{}, IC<1>{}, t, b, b);
                step(IC<kStepB>{}, IC<kStepA>{}, IC<1>{}, t, b, next_buf(b));
                b = next_buf(b);
            }
            for (int t = f0; t < f1; ++t) {
                step(IC<kStepA>{}, IC<kStepB>{}, IC<0>{}, t, b, b);
                step(IC<kStepB>{}, IC<kStepA>{}, IC<0>{}, t, b, next_buf(b));
                b = next_buf(b);
            }
            for (int t = f1; t < te; ++t) {
                step(IC<kStepA>{}, IC<kStepB>{}, IC<1>{}, t, b, b);
                step(IC<kStepB>{}, IC<kStepA>{}, IC<1>{}, t, b, next_buf(b));
                b = next_buf(b);
            }
            // Y of the last tile's second half (buffer of tile te - 1)
            step(IC<kStepLast>{}, IC<kStepLast>{}, IC<0>{}, te - 1, b == 0 ? NB - 1 : b - 1, 0);
        }
    }

    // the accumulators were last written by MFMAs the compiler does not see: wait them out
    // before any other instruction reads them
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(accK[nt]));
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(accV[nt]));

    // epilogue: dK = scale * sum dS^T Q, dV = sum Pd^T dY.  The lane holds column nt*32 + col of
    // key rows 8g + 4h + r (acc_row), one value per key row: written as they are, that is one
    // 2-byte store per value.  Instead each wave stages its 32 key rows in LDS (the tile buffers,
    // free once every wave has left the tile loop) and writes whole rows back, 16 bytes per lane.
    T* gdk = static_cast<T*>(p.dk) + static_cast<int64_t>(it.kv_start) * p.dk_st + hk * p.dk_sh;
    T* gdv = static_cast<T*>(p.dv) + static_cast<int64_t>(it.kv_start) * p.dv_st + hk * p.dv_sh;
    constexpr int SROW = DK + 8;  // staged row (values), padded so that a row starts 4 banks on
    static_assert(NW * 32 * SROW <= NB * (TEQ + TED), "staging area");
    T* stage = reinterpret_cast<T*>(sBuf) + w * 32 * SROW;
    auto write_rows = [&](const f32x16* acc, auto ntc, float mul, T* dst, int64_t st) __attribute__((always_inline)) {
        constexpr int NT = decltype(ntc)::value;
        constexpr int CH = NT * 32 / 8;  // 16-byte chunks per row
        __syncthreads();  // every wave is done with the LDS it is about to overwrite
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int a = 0; a < 16; ++a) stage[acc_row(a, h) * SROW + nt * 32 + col] = static_cast<T>(acc[nt][a] * mul);
        }
        __syncthreads();  // the rows are staged (lanes read what other lanes wrote)
#pragma unroll
        for (int i = 0; i < 32 * CH / 64; ++i) {
            const int c = lane + 64 * i;
            const int row = c / CH;
            const int j = j0 + 32 * w + row;
            if (j < K)
                *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(j) * st + (c % CH) * 8) =
                    *reinterpret_cast<const uint4*>(stage + row * SROW + (c % CH) * 8);
        }
    };
    write_rows(accK, IC<NTK>{}, p.scale, gdk, p.dk_st);
    write_rows(accV, IC<NTV>{}, 1.0f, gdv, p.dv_st);
}

// ------------------------------------------------------------------------------------------------
// dQ
// ------------------------------------------------------------------------------------------------
// Workgroup: 8 waves (two per SIMD), FA16_DQ_BLOCK = 256 queries; wave w owns queries 32w ..
// 32w+31 and keeps their Q and dY rows, statistics and dQ^T
// accumulator.  Key tiles of FA16_DQ_TILE_K = 64 rows are walked as two 32-key steps:
//   S^T = K Q^T, dP^T = V dY^T   (A = K / V rows from LDS, B = Q / dY)
//   dS^T = Ps (dP Z/kp - D)      (each lane holds one query: its D and beta are scalars)
//   dQ^T += K^T dS^T             (A = transposing reads of K, B = dS^T straight from registers)

template <typename T, int DK, int DV, bool DROP, bool XM>
__global__ __launch_bounds__(512, 1) void bwd_dq16_kernel(const Bwd16Args p) {
    using vec = typename Op16<T>::vec;
    constexpr int NW = 8;
    constexpr int BQ = FA16_DQ_BLOCK;    // queries per workgroup
    constexpr int BK = FA16_DQ_TILE_K;   // key tile rows (64): two steps of 32
    constexpr int ND = DK / 32;                 // 32-row head-dim tiles of dQ^T
    constexpr int SK = DK / 16;                 // MFMAs per step for S^T
    constexpr int SV = DV / 16;                 // ... for dP^T
    constexpr int TWK = BK * DK / 8 / 64 / NW;  // DMA instructions per wave and key tile
    constexpr int TWV = BK * DV / 8 / 64 / NW;  // ... and value tile
    static_assert(BQ == 32 * NW && BK == 64 && (BK * DV / 8 / 64) % NW == 0 && DV <= DK, "tile shape");

    __shared__ __attribute__((aligned(16))) T sK[2][Tile<DK>::kElems];
    __shared__ __attribute__((aligned(16))) T sV[2][Tile<DV>::kElems];
    // dropout keep bits of buffer b: query row r of the workgroup (r = 0 .. BQ - 1) at
    // sKeep[b][4r .. 4r + 3], the 4 words of the mask that start with the word holding the bit of
    // (row r, the tile's first key)
    __shared__ __attribute__((aligned(16))) uint32_t sKeep[2][DROP ? BQ * 4 : 1];

    const Unit unit = wg_unit(p.xcd_group != 0);
    const fa_work_item_t it = p.items_q[unit.item];
    const int n = unit.head;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int h = lane >> 5;
    const int L = it.len_q;
    const int K = it.len_kv;
    const int off = K - L;
    const int i0 = it.block * BQ + 32 * w;  // first query of this wave
    const int qi = i0 + col;                // this lane's query
    const uint32_t inv_keep_bits = __builtin_bit_cast(uint32_t, p.inv_keep);

    Tile<DK> loK;
    loK.init(lane);
    Tile<DV> loV_;
    if constexpr (DK != DV) loV_.init(lane);
    const Tile<DV>& loV = tile_for(loK, loV_);

    const int hk = n / p.group;  // the key/value head this query head reads
    const T* gk = static_cast<const T*>(p.k) + static_cast<int64_t>(it.kv_start) * p.k_st + hk * p.k_sh;
    const T* gv = static_cast<const T*>(p.v) + static_cast<int64_t>(it.kv_start) * p.v_st + hk * p.v_sh;
    // wave w copies runs w*TWK .. w*TWK + TWK - 1 of each key tile, and likewise TWV runs of
    // each value tile
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

    // this lane's Q and dY rows (B operands of S^T = K Q^T and dP^T = V dY^T) and statistics
    vec qreg[SK];
    vec dyreg[SV];
    float ndelta = 0.f;  // -D of this lane's query
    float beta = 0.f;
    {
        const bool ok = qi < L;
        const int64_t row = it.q_start + (ok ? qi : 0);
        const vec* qr = reinterpret_cast<const vec*>(static_cast<const T*>(p.q) + row * p.q_st + n * p.q_sh);
        const vec* dr = reinterpret_cast<const vec*>(static_cast<const T*>(p.dy) + row * p.dy_st + n * p.dy_sh);
        const vec* yr = reinterpret_cast<const vec*>(static_cast<const T*>(p.y) + row * p.y_st + n * p.y_sh);
        vec yreg[SV];
#pragma unroll
        for (int s = 0; s < SK; ++s) qreg[s] = ok ? qr[2 * s + h] : vec{};
#pragma unroll
        for (int s = 0; s < SV; ++s) {
            dyreg[s] = ok ? dr[2 * s + h] : vec{};
            yreg[s] = ok ? yr[2 * s + h] : vec{};
        }
        // The row pass of the backward, done here for the workgroup's queries: D = sum over V's
        // head dim of dY * Y in fp32 (each lane half holds every other 8-element chunk of the
        // row) and beta = max * log2(e) + log2(sum) from element 0 of the forward statistics.
        // Written to the row statistics planes, which the dK/dV kernel reads afterwards.
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < SV; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) part += static_cast<float>(dyreg[s][e]) * static_cast<float>(yreg[s][e]);
        }
        part += __shfl_xor(part, 32);
        ndelta = -part;
        if (ok) {
            const int64_t o = static_cast<int64_t>(n) * p.tq + row;
            beta = p.softmax_max[8 * o] * 1.4426950408889634f + __builtin_amdgcn_logf(p.softmax_sum[8 * o]);
            if (h == 0) {
                p.rowstat[o] = ndelta;
                p.rowstat[static_cast<int64_t>(p.heads) * p.tq + o] = -beta;
            }
        }
    }
    // keys this lane's query admits, [klo, khi]; element a of a step starting at key k0s
    // (key k0s + 4h + cc(a)) is admitted iff (unsigned)(cc(a) - (kbase - k0s)) <= krng
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
    // keys admitted by every query of the wave (uniform): steps inside need no mask
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

    f32x16 accQ[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) accQ[i] = zero16();
    // Without dropout, dP^T - D is formed by the MFMA chain itself: it starts from -D (the lane's
    // query) instead of zero.  With dropout the keep bit scales dP but not D, so it starts at zero.
    constexpr bool FOLD_D = !DROP;
    f32x16 pinit;
#pragma unroll
    for (int i = 0; i < 16; ++i) pinit[i] = FOLD_D ? ndelta : 0.f;
    // The S^T chain, too, does the softmax's affine step: the lane's Q row is scaled by
    // scale * log2(e) (once, before rounding to the operand type) and the chain starts from
    // -beta, so it ends with S * scale * log2(e) - beta and P = exp2(acc) needs no multiply.
    // (With an explicit mask the registers are not there; the plain form stays.)
    constexpr bool FOLD_B = !XM;
    f32x16 sinit;
#pragma unroll
    for (int i = 0; i < 16; ++i) sinit[i] = FOLD_B ? -beta : 0.f;
    if constexpr (FOLD_B) {
#pragma unroll
        for (int s = 0; s < SK; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qreg[s][e] = static_cast<T>(static_cast<float>(qreg[s][e]) * p.exp_scale);
        }
    }

    // explicit mask block of this (sequence, head); this lane reads row qi
    __amdgpu_buffer_rsrc_t mrs;
    if constexpr (XM) {
        const uint8_t* mb = p.mask.amask + it.seq * p.mask.am_sb + n * p.mask.am_sn;
        mrs = raw_rsrc(mb, static_cast<uint32_t>((L - 1) * p.mask.am_sq + K));
    }

    // one 32-key step (keys k0s .. k0s + 31, rows R .. R + 31 of the tiles cK / cV); win: the
    // dropout keep bits of this lane's query for those keys (bit t = key k0s + t)
    auto kstep = [&](const T* cK, const T* cV, auto rc, int k0s, uint32_t win) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
        if (k0s > ahi || k0s + 31 < alo) return;
        // explicit mask bytes of keys k0s + 4h + cc(a), issued before the products that hide them
        // (with dropout as well: after them, to stay within the registers)
        uint32_t mk[16];
        auto load_mask_bytes = [&]() __attribute__((always_inline)) {
            const uint32_t mrow = static_cast<uint32_t>(qi) * static_cast<uint32_t>(p.mask.am_sq) +
                                  static_cast<uint32_t>(k0s + 4 * h);
#pragma unroll
            for (int a = 0; a < 16; ++a)
                mk[a] = __builtin_amdgcn_raw_buffer_load_b8(mrs, mrow + 8 * (a >> 2) + (a & 3), 0, 0);
        };
        if constexpr (XM && !DROP) load_mask_bytes();
        // The two waves of a SIMD run the same sequence and meet at every tile barrier, so they
        // tend to reach their products and their softmax gradients together, when the matrix
        // pipe idles.  A wave issuing its S / dP products takes issue priority over one in any
        // other phase, which pulls the two apart.
        __builtin_amdgcn_s_setprio(1);
        f32x16 accS = sinit;
        f32x16 accP = pinit;
#pragma unroll
        for (int s = 0; s < SV; ++s) {
            const vec ak = tile_row<vec>(cK, loK, R, s);
            const vec av = tile_row<vec>(cV, loV, R, s);
            accS = Op16<T>::mfma(ak, qreg[s], accS);
            accP = Op16<T>::mfma(av, dyreg[s], accP);
        }
#pragma unroll
        for (int s = SV; s < SK; ++s) accS = Op16<T>::mfma(tile_row<vec>(cK, loK, R, s), qreg[s], accS);
        __builtin_amdgcn_s_setprio(0);
        if constexpr (DROP && XM) load_mask_bytes();
        // dS^T = Ps (dP Z/kp - D); element (key k0s + 4h + cc(a), query qi)
        const bool full = !XM && wave_rows_full && (k0s >= wlo) && (k0s + 31 <= whi);
        uint32_t dsw[2][4];
        auto softmax_grad = [&](auto masked_tag) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int lo_h = kbase - k0s;
#pragma unroll
            for (int a = 0; a < 16; a += 2) {
                float ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int cc = 8 * ((a + e) >> 2) + ((a + e) & 3);
                    float pv = FOLD_B ? __builtin_amdgcn_exp2f(accS[a + e])
                                      : __builtin_amdgcn_exp2f(accS[a + e] * p.exp_scale - beta);
                    if constexpr (MASKED) {
                        bool adm = static_cast<unsigned>(cc - lo_h) <= static_cast<unsigned>(krng);
                        if constexpr (XM) adm = adm && mk[a + e] == 0;
                        pv = adm ? pv : 0.f;
                    }
                    if constexpr (DROP) {
                        const float zk = keep_scale(win, cc + 4 * h, inv_keep_bits);
                        ds[e] = pv * fmaf(accP[a + e], zk, ndelta);
                    } else {
                        ds[e] = pv * accP[a + e];  // accP already holds dP - D
                    }
                }
                dsw[a >> 3][(a & 7) >> 1] = pack2<T>(ds[0], ds[1]);
            }
        };
        if (full) {
            softmax_grad(Tag<false>{});
        } else {
            softmax_grad(Tag<true>{});
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const vec bs = __builtin_bit_cast(vec, make_uint4(dsw[kk][0], dsw[kk][1], dsw[kk][2], dsw[kk][3]));
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
                const vec ak = tile_tr<vec>(cK, loK, R + 16 * kk, nd);
                accQ[nd] = Op16<T>::mfma(ak, bs, accQ[nd]);
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
        // dropout keep bits of this lane's query for the tile's 64 keys, from its record
        uint32_t win[2] = {0u, 0u};
        if constexpr (DROP) {
            // (low five bits only: 32-bit arithmetic suffices)
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

    // epilogue: dQ = scale * (dQ^T)^T; the lane holds query qi, head-dim values nd*32 + 8g + 4h
    // + 0..3: 8 bytes of its row per store, each store touching 32 rows.  Instead each wave stages
    // its 32 rows in the key-tile buffers (free after a barrier; waves 0..3, then waves 4..7, whose
    // rows would not fit at once in every head-dim variant) and writes whole rows back, 16 bytes per
    // lane.  Chunk c (8 values) of staged row r sits at chunk c ^ (r % CH): the rows are not padded,
    // and without the swizzle every row of a write would start on the same bank.
    constexpr int CH = DK / 8;
    static_assert(4 * 32 * DK <= 2 * Tile<DK>::kElems, "staging area");
    T* stage = reinterpret_cast<T*>(sK) + (w & 3) * 32 * DK;
    for (int round = 0; round < 2; ++round) {
        __syncthreads();  // every wave is done with the LDS about to be overwritten
        if ((w >> 2) == round) {
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t w0 = pack2<T>(accQ[nd][4 * g] * p.scale, accQ[nd][4 * g + 1] * p.scale);
                    const uint32_t w1 = pack2<T>(accQ[nd][4 * g + 2] * p.scale, accQ[nd][4 * g + 3] * p.scale);
                    *reinterpret_cast<uint2*>(stage + col * DK + (((4 * nd + g) ^ (col % CH)) * 8) + 4 * h) =
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
                    *reinterpret_cast<uint4*>(static_cast<T*>(p.dq) + static_cast<int64_t>(it.q_start + q) * p.dq_st +
                                              n * p.dq_sh + (c % CH) * 8) =
                        *reinterpret_cast<const uint4*>(stage + row * DK + (((c % CH) ^ (row % CH)) * 8));
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------

constexpr bool kXcdGrouping = true;  // whole heads per XCD when the head count allows (wg_unit)

template <typename T, int DK, int DV, bool DROP, bool XM>
static hipError_t launch_dkdv_t(const Bwd16Args& a, int64_t n, hipStream_t stream) {
    Bwd16Args g = a;
    g.xcd_group = kXcdGrouping && (a.heads / a.group) % 8 == 0;
    bwd_dkdv16_kernel<T, DK, DV, DROP, XM>
        <<<dim3(static_cast<unsigned>(n), static_cast<unsigned>(a.heads / a.group)), dim3(256), 0, stream>>>(g);
    return hipGetLastError();
}

template <typename T, int DK, int DV, bool DROP, bool XM>
static hipError_t launch_dq_t(const Bwd16Args& a, int64_t n, hipStream_t stream) {
    Bwd16Args g = a;
    g.xcd_group = kXcdGrouping && a.heads % 8 == 0;
    bwd_dq16_kernel<T, DK, DV, DROP, XM>
        <<<dim3(static_cast<unsigned>(n), static_cast<unsigned>(a.heads)), dim3(512), 0, stream>>>(g);
    return hipGetLastError();
}

// head dims (Q/K, V) in {(128, 128), (128, 64), (64, 64)} x dropout x explicit mask, for one dtype
#define FA_DISPATCH16(FN, T)                                                                          \
    auto flags = [&](auto dk_c, auto dv_c) -> hipError_t {                                            \
        constexpr int DK = decltype(dk_c)::value;                                                     \
        constexpr int DV = decltype(dv_c)::value;                                                     \
        if (dropout) return xmask ? FN<T, DK, DV, true, true>(a, n, s) : FN<T, DK, DV, true, false>(a, n, s); \
        return xmask ? FN<T, DK, DV, false, true>(a, n, s) : FN<T, DK, DV, false, false>(a, n, s);    \
    };                                                                                                \
    if (dk == 128 && dv == 128) return flags(IC<128>{}, IC<128>{});                                    \
    if (dk == 128 && dv == 64) return flags(IC<128>{}, IC<64>{});                                      \
    if (dk == 64 && dv == 64) return flags(IC<64>{}, IC<64>{});                                        \
    return hipErrorInvalidValue

// The kernels of each (kernel, dtype) pair are instantiated in a compile part of their own
// (FA_BWD16_PART 1..4; without it, all of them), so that the build compiles them in parallel.
hipError_t dkdv16_bf16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s);
hipError_t dkdv16_f16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s);
hipError_t dq16_bf16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s);
hipError_t dq16_f16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s);

#if !defined(FA_BWD16_PART) || FA_BWD16_PART == 1
hipError_t dkdv16_bf16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s) {
    FA_DISPATCH16(launch_dkdv_t, __bf16);
}

hipError_t launch_dkdv16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask,
                         const Bwd16Args& a, int64_t n_items, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    return dtype == FA_BF16 ? dkdv16_bf16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream)
                            : dkdv16_f16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream);
}

hipError_t launch_dq16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask,
                       const Bwd16Args& a, int64_t n_items, hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    return dtype == FA_BF16 ? dq16_bf16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream)
                            : dq16_f16(head_dim_k, head_dim_v, dropout, xmask, a, n_items, stream);
}
#endif
#if !defined(FA_BWD16_PART) || FA_BWD16_PART == 2
hipError_t dkdv16_f16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s) {
    FA_DISPATCH16(launch_dkdv_t, _Float16);
}
#endif
#if !defined(FA_BWD16_PART) || FA_BWD16_PART == 3
hipError_t dq16_bf16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s) {
    FA_DISPATCH16(launch_dq_t, __bf16);
}
#endif
#if !defined(FA_BWD16_PART) || FA_BWD16_PART == 4
hipError_t dq16_f16(int dk, int dv, bool dropout, bool xmask, const Bwd16Args& a, int64_t n, hipStream_t s) {
    FA_DISPATCH16(launch_dq_t, _Float16);
}
#endif

#undef FA_DISPATCH16

}  // namespace fa
