// fa_bwd_kernels.hip -- exact attention backward for gfx950 (CDNA4).
//
// Gradients of L = sum(O * dO) for O = softmax(scale Q K^T) V (page
// "flash-attn 实现 prefill 阶段", section 问题分析), recomputing the
// probabilities from the row log-sum-exp the forward saved, so the sq x sk
// matrices never reach HBM (the reason the forward returns LSE; page "05 ·
// kernel 工程与四代演化", section 2.1, lists the backward as its own kernel
// class).  With P_ij = exp(scale q_i.k_j - LSE_i):
//   D_i   = dO_i . O_i                      (fa_bwd_dot)
//   dV_j  = sum_i P_ij dO_i                 (fa_bwd_dkdv)
//   dK_j  = scale sum_i dS_ij q_i           (fa_bwd_dkdv)
//   dQ_i  = scale sum_j dS_ij k_j           (fa_bwd_dq)
//   with dP_ij = dO_i . v_j and dS_ij = P_ij (dP_ij - D_i).
//
// fa_bwd_dkdv: one workgroup = 128 keys of one head, wave w owns keys
// [32w, 32w+32) and holds their K and V rows in registers for the whole
// query loop.  Per 64-query step the Q and dO tiles (and their LSE and D) are
// staged in LDS, double buffered.  Scores are computed untransposed,
// S = Q K^T, so in the 32x32 accumulator layout lane l holds one key (column
// l%32) and 16 queries -- exactly the B operand that dV^T += dO^T P and
// dK^T += Q^T dS need (lane = key, 8 queries per half-wave), so P and dS go
// from the accumulators to the matrix cores without a trip through LDS.  The
// A operands dO^T and Q^T come from 8-byte transpose reads of the same LDS
// tiles, in the query order the accumulator layout implies.
//
// fa_bwd_dq: one workgroup = 128 queries of one head, wave w owns 32 queries
// and holds their Q and dO rows in registers; K and V tiles of 64 keys are
// staged in LDS, double buffered.  Here the scores are transposed, S^T = K Q^T
// (lane = query, so LSE_i and D_i are one register each), and
// dQ^T += K^T dS^T takes dS^T as the B operand and K^T from transpose reads.
//
// Recomputing S and dP in both kernels (7 products where 5 would do with
// atomic dQ updates) keeps the result deterministic and needs no fp32 dQ
// accumulator in HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk swizzle for rows of CPR chunks that are read both as 16-byte
// row fragments (16 consecutive rows at one logical chunk) and with 8-byte
// transpose reads (4 consecutive rows x 4 consecutive chunks).  256-byte rows
// (CPR = 16): a bijection on the low four row bits, so 16 rows cover the 16
// chunk positions of a 256-byte bank line, and row bits 0-1 move chunk bits
// 2-3, so the 4 rows of a transpose read fall in different 4-chunk groups.
// 128-byte rows (CPR = 8): the row's parity already picks the half of a bank
// line, and row bits 1-3 pick the chunk, so 16 rows cover all 16 positions.
// 512-byte rows (CPR = 32) start on a bank line like 256-byte ones and take
// the same map (it only moves a chunk within its 16-chunk half of the row).
template <int CPR>
__device__ __forceinline__ int swz_b(int row)
{
    if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    return (row >> 1) & 7;
}

__device__ __forceinline__ float widen16(uint32_t bits, bool bf16)
{
    if (bf16) return __uint_as_float(bits << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// A operand of a 32x32x16 product from two 8-byte transpose reads at LDS
// byte addresses a0 and a1
__device__ __forceinline__ u32x4_t tr_pair(const char* a0, const char* a1)
{
    const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a0));
    const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a1));
    return u32x4_t{__builtin_bit_cast(u32x2_t, x0)[0], __builtin_bit_cast(u32x2_t, x0)[1],
                   __builtin_bit_cast(u32x2_t, x1)[0], __builtin_bit_cast(u32x2_t, x1)[1]};
}

// The rows one work item's (head, sequence) slice covers: its query and key
// counts and the offsets of its first query and key row in the [.][D] arrays
// (and of its first LSE / D entry).  Dense problems: slice bh of [bh][sq] and
// [bh][sk].  Variable-length batches: bh = head * batch + sequence, the
// sequence's rows taken from the offset arrays, clamped into [0, total] as the
// forward does, so malformed offsets cannot address outside the buffers.
struct Slice {
    int sq, sk;
    size_t q0, k0;
};
__device__ __forceinline__ Slice bwd_slice(const BwdParams& p, int bh)
{
    if (!p.cu_q) return Slice{p.sq, p.sk, (size_t)bh * p.sq, (size_t)bh * p.sk};
    const int hd = bh / p.batch, s = bh - hd * p.batch;
    const int qa = min(max(p.cu_q[s], 0), p.total_q), qb = min(max(p.cu_q[s + 1], qa), p.total_q);
    const int ka = min(max(p.cu_k[s], 0), p.total_k), kb = min(max(p.cu_k[s + 1], ka), p.total_k);
    return Slice{qb - qa, kb - ka, (size_t)hd * p.total_q + qa, (size_t)hd * p.total_k + ka};
}

}  // namespace

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i in fp32, one row per D/8 lanes (16 bytes of each tensor
// per lane)
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ void __launch_bounds__(256)
fa_bwd_dot(BwdParams p)
{
    constexpr int LPR = D / 8;        // lanes per row
    constexpr int RPB = 256 / LPR;    // rows per workgroup
    static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must fit one wave");
    const size_t rows = (size_t)p.bh * p.sq;
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int ch = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4_t a = *(const u32x4_t*)((const uint16_t*)p.dout + row * D + ch * 8);
        const u32x4_t b = *(const u32x4_t*)((const uint16_t*)p.o + row * D + ch * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(widen16(a[e] & 0xffffu, BF16), widen16(b[e] & 0xffffu, BF16), acc);
            acc = __builtin_fmaf(widen16(a[e] >> 16, BF16), widen16(b[e] >> 16, BF16), acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && ch == 0) p.dvec[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys of one head
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
fa_bwd_dkdv(BwdParams p)
{
    static_assert(D == 64 || D == 128 || D == 256, "128-, 256- or 512-byte rows");
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int NW = 4;                 // waves; wave w owns keys [32w, 32w+32)
    constexpr int BN = 32 * NW;           // keys per workgroup
    constexpr int BMQ = 64;               // queries per step (two 32-row blocks)
    constexpr int RB = D * 2;             // bytes per row
    constexpr int NKK = D / 16;           // k-steps of S and dP
    // d = 256: a work item accumulates dK^T and dV^T for one half of d (the
    // whole would take 256 registers per lane for the accumulators alone, and
    // the K and V fragments another 128), recomputing S and dP in each half
    constexpr int NSPLIT = D > 128 ? 2 : 1;
    constexpr int DH = D / NSPLIT;        // d range of this item's dK, dV
    constexpr int NDT = DH / 32;          // 32-wide d tiles of dK^T, dV^T
    constexpr int TQ = BMQ * RB;          // bytes of one Q or dO tile
    constexpr int OFF_LSE = 2 * TQ;       // stage layout: Q | dO | LSE (log2) | D
    constexpr int OFF_D = OFF_LSE + BMQ * 4;
    constexpr int STAGE = OFF_D + BMQ * 4;
    constexpr int DMA = TQ / 1024 / NW;   // 1 KiB copies per wave per tensor per step
    static_assert(DMA * 1024 * NW == TQ, "tile must split evenly over waves");
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    int bh, kt;
    if (!map_xcd_item(p.n_items, p.items_per_head, bh, kt)) return;
    const int hd = kt % NSPLIT;           // which half of d (d = 256)
    kt /= NSPLIT;
    const Slice sl = bwd_slice(p, bh);
    const int sq = sl.sq, sk = sl.sk;
    const int n0 = kt * BN;
    if (n0 >= sk) return;  // variable-length batch: past this sequence's keys
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const float c = p.c;
    const uint32_t dead_bits = c > 0.f ? 0xff800000u : 0x7f800000u;  // -inf * sign(c)

    const uint16_t* __restrict__ Q = (const uint16_t*)p.q + sl.q0 * D;
    const uint16_t* __restrict__ dO = (const uint16_t*)p.dout + sl.q0 * D;
    const float* __restrict__ LSE = p.lse + sl.q0;
    const float* __restrict__ DV = p.dvec + sl.q0;
    const uint16_t* __restrict__ K = (const uint16_t*)p.k + sl.k0 * D;
    const uint16_t* __restrict__ V = (const uint16_t*)p.v + sl.k0 * D;

    // this wave's keys: B operands of S = Q K^T and dP = dO V^T (lane = key,
    // 8 d values per half-wave); keys past the end re-read the last key
    const int key = n0 + 32 * w + l32;
    u32x4_t kf[NKK], vf[NKK];
    {
        const size_t kr = (size_t)min(key, sk - 1) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            kf[kk] = *(const u32x4_t*)(K + kr + 16 * kk);
            vf[kk] = *(const u32x4_t*)(V + kr + 16 * kk);
        }
    }

    // query steps: causal keys n0.. are seen by queries n0.. only
    const int qs_begin = CAUSAL ? n0 / BMQ : 0;
    const int qs_end = (sq + BMQ - 1) / BMQ;

    // ---- global -> LDS copies of the Q and dO tiles.  Copy j of wave w fills
    //      LDS chunks cc = (w*DMA + j)*64 + lane: row cc/16, physical chunk
    //      cc%16, fetched from the swizzled logical chunk ----
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds) + w * DMA * 1024);
    uint32_t cof[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int cc = (w * DMA + j) * 64 + lane;
        const int row = cc / CPR, pch = cc % CPR;
        cof[j] = row * RB + ((pch ^ swz_b<CPR>(row)) << 4);
    }
    // copy C (0..2*DMA-1: Q copies, then dO copies) of the tile at query q0
    // into stage ST; rows past the last query re-read it (masked later), by
    // arithmetic, so a copy is one branch-free instruction
    auto copy_one = [&](auto st_tag, auto c_tag, int q0) {
        constexpr int ST = decltype(st_tag)::value, C = decltype(c_tag)::value, J = C % DMA;
        const int row = ((w * DMA + J) * 64 + lane) / CPR;
        const uint32_t off = cof[J] - (uint32_t)(max(row - (sq - 1 - q0), 0) * RB);
        const void* src = uniform_ptr((C < DMA ? Q : dO) + (size_t)q0 * D);
        copy_1k<ST * STAGE + (C < DMA ? 0 : TQ) + J * 1024>(src, off, lbase);
    };
    auto issue = [&](auto st_tag, int q0) {
        constexpr int ST = decltype(st_tag)::value;
        const bool full = q0 + BMQ <= sq;
        const void* qsrc = uniform_ptr(Q + (size_t)q0 * D);
        const void* gsrc = uniform_ptr(dO + (size_t)q0 * D);
        static_for<DMA>([&](auto j_tag) {
            constexpr int J = decltype(j_tag)::value;
            uint32_t off = cof[J];
            if (!full) {  // rows past the last query re-read it (masked later)
                const int cc = (w * DMA + J) * 64 + lane;
                const int row = cc / CPR, pch = cc % CPR;
                off = min(row, sq - 1 - q0) * RB + ((pch ^ swz_b<CPR>(row)) << 4);
            }
            copy_1k<ST * STAGE + J * 1024>(qsrc, off, lbase);
            copy_1k<ST * STAGE + TQ + J * 1024>(gsrc, off, lbase);
        });
    };
    // LSE (converted to log2 units) and D of a step's 64 rows: wave 0 fetches
    // LSE, wave 1 fetches D, one row per lane, and writes them into the stage
    // just before the barrier that publishes it.  The conversion happens at
    // the store, so no wave waits for the load before its matrix-core work
    // (the copy wait before that barrier covers it).
    float pend = 0.f;
    auto fetch_rows = [&](int q0) {
        if (w < 2) {
            const int r = min(q0 + lane, sq - 1);
            pend = (w == 0) ? LSE[r] : DV[r];
        }
    };
    auto store_rows = [&](int st) {
        if (w < 2) *(float*)(lds + st * STAGE + OFF_LSE + w * BMQ * 4 + lane * 4) = (w == 0) ? pend * kLog2e : pend;
    };

    // ---- per-lane LDS read offsets (bytes within a stage) ----
    //  row fragments (A operand of S and dP): row l32, logical chunk 2kk + g
    uint32_t rq[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) rq[kk] = l32 * RB + (((2 * kk + g) ^ swz_b<CPR>(l32)) << 4);
    //  transpose reads (A operand of dV^T and dK^T): lane 4r + c of its 16-lane
    //  group reads query row 8j + 4g + r, d = 32dt + 16*half + 4c
    const int sub = lane & 15, tr_r = sub >> 2, tr_c = sub & 3, half = (lane >> 4) & 1;
    uint32_t rt[2][NDT];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + 4 * g + tr_r;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            rt[j][dt] = row * RB + (((hd * (DH / 8) + 4 * dt + 2 * half + (tr_c >> 1)) ^ swz_b<CPR>(row)) << 4) +
                        (tr_c & 1) * 8;
    }

    f32x16_t dva[NDT], dka[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dva[dt][r] = 0.f;
            dka[dt][r] = 0.f;
        }

    // One 32-query block (qb = 0, 1 of the stage) in three pieces, so that
    // two blocks can be interleaved: the score products, the softmax, and
    // the dV and dK products.
    // block_mask: the causal and ragged masks of a block's scores as one pass
    // (diagonal and ragged blocks only): score rr belongs to query qbase + 4g
    // + off(rr) and lives iff key <= query < sq; a dead score becomes
    // -inf * sign(c) (c is never zero), so its probability and dS are exactly
    // 0.  The select is a sign mask and a bit-field insert.
    auto block_mask = [&](f32x16_t& s, int qbase) {
        const bool need_mask = (qbase + 32 > sq) || (CAUSAL && qbase < n0 + 32 * w + 31);
        if (need_mask) {
            const int lo = CAUSAL ? key - qbase - 4 * g : -(1 << 20);
            const int hi1 = sq - qbase - 4 * g - 1;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int off = (rr >> 2) * 8 + (rr & 3);
                const uint32_t dead = (uint32_t)(((off - lo) | (hi1 - off)) >> 31);
                const float x = s[rr];  // through a scalar: a bit cast of a vector element reads element 0
                const uint32_t bits = __builtin_bit_cast(uint32_t, x);
                s[rr] = __builtin_bit_cast(float, (bits & ~dead) | (dead_bits & dead));
            }
        }
    };
    // the block's LSE (log2 units) and D: accumulator row r holds query
    // 8(r/4) + 4g + r%4 of the block
    auto block_rows = [&](const char* sb, int qb, f32x4_t (&l4)[4], f32x4_t (&d4)[4]) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            l4[rb] = *(const f32x4_t*)(sb + OFF_LSE + (32 * qb + 8 * rb + 4 * g) * 4);
            d4[rb] = *(const f32x4_t*)(sb + OFF_D + (32 * qb + 8 * rb + 4 * g) * 4);
        }
    };
    // softmax element rr: P = exp2(c s - LSE log2 e), dS = P (dP - D); the
    // pair (rr - 1, rr) is packed at odd rr
    auto soft_el = [&](int rr, const f32x16_t& s, const f32x16_t& dp, const f32x4_t (&l4)[4],
                       const f32x4_t (&d4)[4], float (&pr)[16], float (&dr)[16], u32x4_t (&pp)[2],
                       u32x4_t (&dsp)[2]) {
        pr[rr] = fast_exp2(__builtin_fmaf(s[rr], c, -l4[rr >> 2][rr & 3]));
        dr[rr] = pr[rr] * (dp[rr] - d4[rr >> 2][rr & 3]);
        if (rr & 1) {
            pp[rr >> 3][(rr >> 1) & 3] = pack2(pr[rr - 1], pr[rr], BF16);
            dsp[rr >> 3][(rr >> 1) & 3] = pack2(dr[rr - 1], dr[rr], BF16);
        }
    };

    // the simple form: the three pieces of one block one after another
    auto compute_block = [&](const char* sb, int qb, int qbase) {
        const char* qblk = sb + qb * 32 * RB;
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.f;
            dp[r] = 0.f;
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const u32x4_t aq = *(const u32x4_t*)(qblk + rq[kk]);
            const u32x4_t ag = *(const u32x4_t*)(qblk + TQ + rq[kk]);
            s = mfma16(aq, kf[kk], s, BF16);
            dp = mfma16(ag, vf[kk], dp, BF16);
        }
        // the transposed dO and Q operands of the dV and dK products go out
        // now, so their LDS latency hides behind the softmax
        u32x4_t opg[2][NDT], opq[2][NDT];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const char* base = qblk + kc * 16 * RB;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                opg[kc][dt] = tr_pair(base + TQ + rt[0][dt], base + TQ + rt[1][dt]);
                opq[kc][dt] = tr_pair(base + rt[0][dt], base + rt[1][dt]);
            }
        }
        f32x4_t l4[4], d4[4];
        block_rows(sb, qb, l4, d4);
        block_mask(s, qbase);
        float pr[16], dr[16];
        u32x4_t pp[2], dsp[2];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) soft_el(rr, s, dp, l4, d4, pr, dr, pp, dsp);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                dva[dt] = mfma16(opg[kc][dt], pp[kc], dva[dt], BF16);
                dka[dt] = mfma16(opq[kc][dt], dsp[kc], dka[dt], BF16);
            }
    };

    // A stage's two blocks.  When both are live they are interleaved:
    // S/dP(0); S/dP(1) with the softmax of block 0; dV/dK(0) with the softmax
    // of block 1; dV/dK(1).  One wave per SIMD, so the wave itself keeps its
    // matrix cores busy while its softmax runs (one softmax element per
    // matrix-core instruction).  Each stream's LDS operands come from a small
    // register ring; the empty volatile asm statements pin the softmax results
    // in place (otherwise the compiler sinks them to their first use and the
    // overlap is lost).
    // compute(S, q0, qn): the stage-S tile at q0; the copies of the tile at
    // qn into stage S^1 go out during the matrix-core streams (qn = q0 on the
    // last step: a harmless refill of a stage nobody reads again)
    auto compute = [&](auto st_tag, int q0, int qn) {
        constexpr int S = decltype(st_tag)::value;
        const char* sb = lds + S * STAGE;
        const bool ok0 = q0 < sq && !(CAUSAL && q0 + 31 < n0 + 32 * w);
        const bool ok1 = q0 + 32 < sq && !(CAUSAL && q0 + 63 < n0 + 32 * w);
        // copy C goes out with matrix-core instruction I of stream X
        auto copy_at = [&](auto x_tag, auto i_tag) {
            constexpr int X = decltype(x_tag)::value, I = decltype(i_tag)::value;
            constexpr int C = X == 0 ? (I == 2 ? 0 : I == 7 ? 1 : -1)
                            : X == 1 ? (I == 2 ? 2 : I == 7 ? 3 : I == 12 ? 4 : -1)
                                     : (I == 2 ? 5 : I == 7 ? 6 : I == 12 ? 7 : -1);
            if constexpr (C >= 0 && C < 2 * DMA) copy_one(Stage<S ^ 1>{}, Stage<C>{}, qn);
        };
        if constexpr (D <= 128) {
        static_assert(2 * DMA <= 8, "copy slots for at most eight copies per wave per step");
        if (ok0 && ok1) {
            constexpr int KA = 4;
            // ---- S/dP of block 0 ----
            f32x16_t s0, dp0, s1, dp1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s0[r] = 0.f;
                dp0[r] = 0.f;
            }
            {
                const char* qblk = sb;
                u32x4_t ring[KA];
                // instruction i: even -> S (Q fragment), odd -> dP (dO fragment), k-step i/2
                auto fetch = [&](auto f_tag) {
                    constexpr int F = decltype(f_tag)::value;
                    ring[F % KA] = *(const u32x4_t*)(qblk + (F % 2 ? TQ : 0) + rq[F / 2]);
                };
                static_for<KA>([&](auto f) { fetch(f); });
                static_for<2 * NKK>([&](auto i_tag) {
                    constexpr int I = decltype(i_tag)::value;
                    const u32x4_t a = ring[I % KA];
                    if constexpr (I + KA < 2 * NKK) fetch(Stage<I + KA>{});
                    if constexpr (I % 2 == 0) s0 = mfma16(a, kf[I / 2], s0, BF16);
                    else dp0 = mfma16(a, vf[I / 2], dp0, BF16);
                    copy_at(Stage<0>{}, Stage<I>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            // ---- S/dP of block 1 with the softmax of block 0 ----
            f32x4_t l40[4], d40[4];
            block_rows(sb, 0, l40, d40);
            block_mask(s0, q0);
            float pr0[16], dr0[16];
            u32x4_t pp0[2], dsp0[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s1[r] = 0.f;
                dp1[r] = 0.f;
            }
            {
                const char* qblk = sb + 32 * RB;
                u32x4_t ring[KA];
                auto fetch = [&](auto f_tag) {
                    constexpr int F = decltype(f_tag)::value;
                    ring[F % KA] = *(const u32x4_t*)(qblk + (F % 2 ? TQ : 0) + rq[F / 2]);
                };
                static_for<KA>([&](auto f) { fetch(f); });
                static_for<2 * NKK>([&](auto i_tag) {
                    constexpr int I = decltype(i_tag)::value;
                    const u32x4_t a = ring[I % KA];
                    if constexpr (I + KA < 2 * NKK) fetch(Stage<I + KA>{});
                    if constexpr (I % 2 == 0) s1 = mfma16(a, kf[I / 2], s1, BF16);
                    else dp1 = mfma16(a, vf[I / 2], dp1, BF16);
                    // the block's 16 softmax elements spread evenly over the stream
                    constexpr int EPS = 16 / (2 * NKK);
                    static_for<EPS>([&](auto j_tag) {
                        constexpr int E = I * EPS + decltype(j_tag)::value;
                        soft_el(E, s0, dp0, l40, d40, pr0, dr0, pp0, dsp0);
                        asm volatile("" : "+v"(pr0[E]), "+v"(dr0[E]));
                    });
                    copy_at(Stage<1>{}, Stage<I>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            // ---- dV/dK of block 0 with the softmax of block 1 ----
            f32x4_t l41[4], d41[4];
            block_rows(sb, 1, l41, d41);
            block_mask(s1, q0 + 32);
            float pr1[16], dr1[16];
            u32x4_t pp1[2], dsp1[2];
            auto pv_stream = [&](const char* qblk, u32x4_t (&pp)[2], u32x4_t (&dsp)[2], auto with_soft) {
                u32x4_t ring[KA];
                // instruction i: chunk kc = i / (2 NDT), d tile dt = (i / 2) % NDT,
                // even -> dV (dO^T operand), odd -> dK (Q^T operand)
                auto fetch = [&](auto f_tag) {
                    constexpr int F = decltype(f_tag)::value, kc = F / (2 * NDT), dt = (F / 2) % NDT;
                    const char* base = qblk + kc * 16 * RB + (F % 2 ? 0 : TQ);
                    ring[F % KA] = tr_pair(base + rt[0][dt], base + rt[1][dt]);
                };
                static_for<KA>([&](auto f) { fetch(f); });
                static_for<4 * NDT>([&](auto i_tag) {
                    constexpr int I = decltype(i_tag)::value, kc = I / (2 * NDT), dt = (I / 2) % NDT;
                    const u32x4_t a = ring[I % KA];
                    if constexpr (I + KA < 4 * NDT) fetch(Stage<I + KA>{});
                    if constexpr (I % 2 == 0) dva[dt] = mfma16(a, pp[kc], dva[dt], BF16);
                    else dka[dt] = mfma16(a, dsp[kc], dka[dt], BF16);
                    with_soft(Stage<I>{});
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            pv_stream(sb, pp0, dsp0, [&](auto i_tag) {
                constexpr int I = decltype(i_tag)::value;
                constexpr int EPS = 16 / (4 * NDT);
                static_for<EPS>([&](auto j_tag) {
                    constexpr int E = I * EPS + decltype(j_tag)::value;
                    soft_el(E, s1, dp1, l41, d41, pr1, dr1, pp1, dsp1);
                    asm volatile("" : "+v"(pr1[E]), "+v"(dr1[E]));
                });
                copy_at(Stage<2>{}, i_tag);
            });
            // ---- dV/dK of block 1 ----
            pv_stream(sb + 32 * RB, pp1, dsp1, [&](auto) {});
            return;
        }
        }
        // the simple form: one live block, or d = 256 (two blocks' scores and
        // a stream's operand ring do not fit beside the K and V fragments)
        static_for<2 * DMA>([&](auto c) { copy_one(Stage<S ^ 1>{}, c, qn); });
        if (ok0) compute_block(sb, 0, q0);
        if (ok1) compute_block(sb, 1, q0 + 32);
    };

    auto step = [&](auto st_tag, int t) {
        constexpr int S = decltype(st_tag)::value;
        store_rows(S);
        wait_copies();
        __syncthreads();  // stage S is complete; every wave is done with stage S^1
        const int qn = (t + 1 < qs_end ? t + 1 : t) * BMQ;
        fetch_rows(qn);
        compute(st_tag, t * BMQ, qn);
    };

    if (qs_begin < qs_end) {
        issue(Stage<0>{}, qs_begin * BMQ);
        fetch_rows(qs_begin * BMQ);
    }
    int t = qs_begin;
    for (; t + 1 < qs_end; t += 2) {
        step(Stage<0>{}, t);
        step(Stage<1>{}, t + 1);
    }
    if (t < qs_end) step(Stage<0>{}, t);

    // ---- epilogue: dV = (dV^T)^T, dK = scale (dK^T)^T; accumulator row r of
    //      d tile dt is d = 32dt + 8(r/4) + 4g + r%4 ----
    if (key < sk) {
        uint16_t* dvrow = (uint16_t*)p.dv + (sl.k0 + key) * D;
        uint16_t* dkrow = (uint16_t*)p.dk + (sl.k0 + key) * D;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = hd * DH + 32 * dt + 8 * rb + 4 * g;
                *(u32x2_t*)(dvrow + d0) = u32x2_t{pack2(dva[dt][4 * rb], dva[dt][4 * rb + 1], BF16),
                                                  pack2(dva[dt][4 * rb + 2], dva[dt][4 * rb + 3], BF16)};
                *(u32x2_t*)(dkrow + d0) = u32x2_t{pack2(dka[dt][4 * rb] * sc, dka[dt][4 * rb + 1] * sc, BF16),
                                                  pack2(dka[dt][4 * rb + 2] * sc, dka[dt][4 * rb + 3] * sc, BF16)};
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128 queries of one head
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(256, D > 128 ? 1 : 2)
fa_bwd_dq(BwdParams p)
{
    // d = 256: the Q and dO fragments (128 registers per lane) and the dQ^T
    // accumulators (128) need one wave per SIMD
    static_assert(D == 64 || D == 128 || D == 256, "128-, 256- or 512-byte rows");
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int NW = 4;                 // waves; wave w owns queries [32w, 32w+32)
    constexpr int BM = 32 * NW;           // queries per workgroup
    constexpr int BN = 64;                // keys per step (two 32-key blocks)
    constexpr int RB = D * 2;
    constexpr int NKK = D / 16;
    constexpr int NDT = D / 32;
    constexpr int TK = BN * RB;           // bytes of one K or V tile
    constexpr int STAGE = 2 * TK;         // stage layout: K | V
    constexpr int DMA = TK / 1024 / NW;
    static_assert(DMA * 1024 * NW == TK, "tile must split evenly over waves");
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    int bh, item;
    if (!map_xcd_item(p.n_items, p.items_per_head, bh, item)) return;
    const Slice sl = bwd_slice(p, bh);
    const int sq = sl.sq, sk = sl.sk;
    const int mt = CAUSAL ? p.items_per_head - 1 - item : item;  // causal: heaviest tiles first
    const int q0 = mt * BM;
    if (q0 >= sq) return;  // variable-length batch: past this sequence's queries
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const float c = p.c;
    const uint32_t dead_bits = c > 0.f ? 0xff800000u : 0x7f800000u;  // -inf * sign(c)

    const uint16_t* __restrict__ Q = (const uint16_t*)p.q + sl.q0 * D;
    const uint16_t* __restrict__ dO = (const uint16_t*)p.dout + sl.q0 * D;
    const uint16_t* __restrict__ K = (const uint16_t*)p.k + sl.k0 * D;
    const uint16_t* __restrict__ V = (const uint16_t*)p.v + sl.k0 * D;

    // this wave's queries: B operands of S^T = K Q^T and dP^T = V dO^T (lane =
    // query); rows past the end re-read the last row and are never stored
    const int wq = q0 + 32 * w;
    const int qrow = wq + l32;
    const int qr = min(qrow, sq - 1);
    u32x4_t qf[NKK], gf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        qf[kk] = *(const u32x4_t*)(Q + (size_t)qr * D + 16 * kk + 8 * g);
        gf[kk] = *(const u32x4_t*)(dO + (size_t)qr * D + 16 * kk + 8 * g);
    }
    const float lse2 = p.lse[sl.q0 + qr] * kLog2e;
    const float drow = p.dvec[sl.q0 + qr];

    const int q_end = min(q0 + BM, sq);
    const int kv_end = CAUSAL ? min(q_end, sk) : sk;
    const int nkv = (kv_end + BN - 1) / BN;
    const int w_kv_end = (wq >= sq) ? 0 : (CAUSAL ? min(min(wq + 32, sq), sk) : sk);

    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds) + w * DMA * 1024);
    uint32_t cof[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int cc = (w * DMA + j) * 64 + lane;
        const int row = cc / CPR, pch = cc % CPR;
        cof[j] = row * RB + ((pch ^ swz_b<CPR>(row)) << 4);
    }
    auto issue = [&](auto st_tag, int n0) {
        constexpr int ST = decltype(st_tag)::value;
        const bool full = n0 + BN <= sk;
        const void* ksrc = uniform_ptr(K + (size_t)n0 * D);
        const void* vsrc = uniform_ptr(V + (size_t)n0 * D);
        static_for<DMA>([&](auto j_tag) {
            constexpr int J = decltype(j_tag)::value;
            uint32_t off = cof[J];
            if (!full) {  // rows past the last key re-read it (masked)
                const int cc = (w * DMA + J) * 64 + lane;
                const int row = cc / CPR, pch = cc % CPR;
                off = min(row, sk - 1 - n0) * RB + ((pch ^ swz_b<CPR>(row)) << 4);
            }
            copy_1k<ST * STAGE + J * 1024>(ksrc, off, lbase);
            copy_1k<ST * STAGE + TK + J * 1024>(vsrc, off, lbase);
        });
    };

    uint32_t rk[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) rk[kk] = l32 * RB + (((2 * kk + g) ^ swz_b<CPR>(l32)) << 4);
    const int sub = lane & 15, tr_r = sub >> 2, tr_c = sub & 3, half = (lane >> 4) & 1;
    uint32_t rt[2][NDT];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + 4 * g + tr_r;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            rt[j][dt] = row * RB + (((4 * dt + 2 * half + (tr_c >> 1)) ^ swz_b<CPR>(row)) << 4) + (tr_c & 1) * 8;
    }

    f32x16_t dqa[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[dt][r] = 0.f;

    auto compute = [&](auto st_tag, int n0) {
        constexpr int S = decltype(st_tag)::value;
        const char* sb = lds + S * STAGE;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int kbase = n0 + 32 * kb;
            if (kbase >= w_kv_end) break;
            const char* kblk = sb + kb * 32 * RB;

            // ---- S^T = K Q^T and dP^T = V dO^T: lane = query, rows = keys ----
            f32x16_t s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4_t ak = *(const u32x4_t*)(kblk + rk[kk]);
                const u32x4_t av = *(const u32x4_t*)(kblk + TK + rk[kk]);
                s = mfma16(ak, qf[kk], s, BF16);
                dp = mfma16(av, gf[kk], dp, BF16);
            }

            // ---- dS^T = P^T (dP^T - D); row r holds key 8(r/4) + 4g + r%4.
            //      Masks (diagonal and ragged blocks only, one pass before the
            //      exponentials): key kbase + 4g + off(r) lives iff it is below
            //      min(sk, qrow + 1) when causal, else below sk; a dead score
            //      becomes -inf * sign(c), so its probability is exactly 0 ----
            const bool need_mask = (kbase + 32 > sk) || (CAUSAL && kbase + 31 > wq);
            if (need_mask) {
                const int lim = (CAUSAL ? min(sk, qrow + 1) : sk) - kbase - 4 * g - 1;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int off = (rr >> 2) * 8 + (rr & 3);
                    const uint32_t dead = (uint32_t)((lim - off) >> 31);
                    const float x = s[rr];  // through a scalar: a bit cast of a vector element reads element 0
                    const uint32_t bits = __builtin_bit_cast(uint32_t, x);
                    s[rr] = __builtin_bit_cast(float, (bits & ~dead) | (dead_bits & dead));
                }
            }
            u32x4_t dsp[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float dr[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int rr = r + e;
                    const float pv = fast_exp2(__builtin_fmaf(s[rr], c, -lse2));
                    dr[e] = pv * (dp[rr] - drow);
                }
                dsp[r >> 3][(r >> 1) & 3] = pack2(dr[0], dr[1], BF16);
            }

            // ---- dQ^T += K^T dS^T ----
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                const char* base = kblk + kc * 16 * RB;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const u32x4_t ak = tr_pair(base + rt[0][dt], base + rt[1][dt]);
                    dqa[dt] = mfma16(ak, dsp[kc], dqa[dt], BF16);
                }
            }
        }
    };

    auto step = [&](auto st_tag, int t) {
        constexpr int S = decltype(st_tag)::value;
        wait_copies();
        __syncthreads();
        if (t + 1 < nkv) issue(Stage<S ^ 1>{}, (t + 1) * BN);
        compute(st_tag, t * BN);
    };

    if (nkv > 0) issue(Stage<0>{}, 0);
    int t = 0;
    for (; t + 1 < nkv; t += 2) {
        step(Stage<0>{}, t);
        step(Stage<1>{}, t + 1);
    }
    if (t < nkv) step(Stage<0>{}, t);

    if (qrow < sq) {
        uint16_t* dqrow = (uint16_t*)p.dq + (sl.q0 + qrow) * D;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int d0 = 32 * dt + 8 * rb + 4 * g;
                *(u32x2_t*)(dqrow + d0) = u32x2_t{pack2(dqa[dt][4 * rb] * sc, dqa[dt][4 * rb + 1] * sc, BF16),
                                                  pack2(dqa[dt][4 * rb + 2] * sc, dqa[dt][4 * rb + 3] * sc, BF16)};
            }
    }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------
namespace {

int round8(int64_t n) { return (int)(((n + 7) / 8) * 8); }

template <int D, bool BF16>
hipError_t launch_bwd_t(BwdParams p, hipStream_t s)
{
    constexpr int RPB = 256 / (D / 8);
    // D over every row of dout and o: a variable-length batch's packed rows
    // are h * total_q rows of the same [.][D] layout
    BwdParams pd = p;
    if (p.cu_q) {
        pd.bh = p.bh / p.batch;
        pd.sq = p.total_q;
    }
    const int64_t rows = (int64_t)pd.bh * pd.sq;
    hipLaunchKernelGGL((fa_bwd_dot<D, BF16>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, pd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    p.items_per_head = (p.sk + 127) / 128 * (D > 128 ? 2 : 1);  // d = 256: two halves of d per key tile
    p.n_items = p.bh * p.items_per_head;
    auto dkdv = p.causal ? fa_bwd_dkdv<D, BF16, true> : fa_bwd_dkdv<D, BF16, false>;
    hipLaunchKernelGGL(dkdv, dim3(round8(p.n_items)), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    p.items_per_head = (p.sq + 127) / 128;
    p.n_items = p.bh * p.items_per_head;
    auto dq = p.causal ? fa_bwd_dq<D, BF16, true> : fa_bwd_dq<D, BF16, false>;
    hipLaunchKernelGGL(dq, dim3(round8(p.n_items)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool bwd_supported(int dtype, int d) { return (dtype == 1 || dtype == 2) && (d == 64 || d == 128 || d == 256); }

hipError_t launch_bwd(int dtype, int d, const BwdParams& p, hipStream_t stream)
{
    if (d == 128) {
        if (dtype == 2) return launch_bwd_t<128, true>(p, stream);
        if (dtype == 1) return launch_bwd_t<128, false>(p, stream);
    } else if (d == 64) {
        if (dtype == 2) return launch_bwd_t<64, true>(p, stream);
        if (dtype == 1) return launch_bwd_t<64, false>(p, stream);
    } else if (d == 256) {
        if (dtype == 2) return launch_bwd_t<256, true>(p, stream);
        if (dtype == 1) return launch_bwd_t<256, false>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
