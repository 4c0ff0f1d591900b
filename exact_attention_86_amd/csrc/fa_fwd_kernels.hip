// fa_fwd_kernels.hip -- exact attention prefill forward for gfx950 (CDNA4).
//
// Computes, per (batch, head) slice of contiguous [b, h, s, d] tensors,
//   O = softmax(scale * Q K^T) V   and   LSE_i = ln sum_j exp(scale q_i.k_j)
// (page "flash-attn 实现 prefill 阶段", section 问题分析), tile by tile with
// the online softmax of page "flash.cu" (forward_kernel: a running row max m
// and row sum l, rescaled per key tile), so the sq x sk score matrix never
// reaches HBM.
//
// Design (one workgroup = one tile of BM query rows of one head):
//  * NW waves of 64 lanes; wave w owns query rows [32w, 32w+32) of the tile,
//    so a row's softmax never leaves its wave (page "05 · kernel 工程与四代演化",
//    section 3, puts the warps of the FA2 traits along the query dimension).
//  * Scores are computed transposed, S^T = K Q^T, on the 32x32 matrix cores:
//    in the 32x32 accumulator layout lane l holds column l%32 -- one query --
//    and 16 key rows, so the row max and row sum are in-lane reductions plus
//    one exchange between the two 32-lane halves that share a query.
//  * The output is accumulated transposed too, O^T += V^T P^T: P^T is the B
//    operand straight from the score registers (no trip through LDS) and the
//    per-query rescale factor is in-lane.  The key order the score layout
//    imposes on P^T is matched by storing V^T in LDS with bits 2 and 3 of the
//    key index swapped inside each 16-key group (a contraction does not care
//    about the order of its summation index as long as both operands agree).
//  * Q stays in registers for the whole key loop; K and V^T tiles are double
//    buffered in LDS (padded rows against bank conflicts) and the next tile's
//    global loads are issued before the current tile's math.
//  * exp2 with the scale and log2(e) folded into one FMA; m is kept in log2
//    units and converted back for LSE.
//  * Causal: key tiles past a tile's last row are never loaded; a wave skips
//    the math of key tiles that lie wholly above its own diagonal; masks are
//    applied only on diagonal and ragged tiles.
//  * Schedule: workgroup ids are mapped XCD-aware (consecutive ids land on
//    different XCDs, so heads are grouped per XCD for L2 reuse of K/V) and,
//    for causal, heaviest query tiles first within a head.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// workgroup id -> (head slice, work item).  Consecutive workgroup ids are
// dispatched round-robin over the XCDs; slot s of XCD x takes item x*per + s of
// the head-major item order, so each XCD works through a contiguous run of
// heads and its L2 sees the same K/V from many query tiles.  Causal items pair
// query tile nQ-1-i (heaviest) with tile i (lightest), so every item costs
// about nQ+1 key tiles and the grid drains without a long tail.
__device__ __forceinline__ bool map_item(const Params& p, int& bh, int& item)
{
    const int id = blockIdx.x;
    const int per = (p.n_items + kXcds - 1) / kXcds;
    const int t = (id % kXcds) * per + id / kXcds;
    if (t >= p.n_items) return false;
    bh = t / p.items_per_head;
    item = t - bh * p.items_per_head;
    return true;
}

// query tiles of a work item, heaviest first; returns how many (1 or 2)
__device__ __forceinline__ int item_tiles(const Params& p, int item, int (&mt)[2])
{
    if (!p.causal) {
        mt[0] = item;
        return 1;
    }
    mt[0] = p.n_mtiles - 1 - item;
    mt[1] = item;
    return mt[0] == mt[1] ? 1 : 2;
}

// Persistent schedule: the grid is G workgroups (about one per CU, G a
// multiple of the XCD count) and each loops over work units, one unit = one
// query tile (bh, mt).  Units are numbered level-major in cost order: unit t
// is head t mod (b*h) at level t / (b*h), the heaviest causal tiles (the most
// key tiles) first; without the causal mask every level costs the same.  Slot
// s of XCD x (workgroup 8s + x) takes, in round r, unit r*G + 8*s' + x with
// s' = s in even rounds and S-1-s in odd ones (S = G/8 slots per XCD): this
// snake order gives the slot that drew one of the heaviest units of a round
// one of the lightest of the next, so every slot ends up with about the same
// number of key tiles without atomics or a workspace.  Unit t runs on XCD
// t mod 8, so when b*h is a multiple of 8 every tile of a head runs on one
// XCD and its L2 serves that head's K/V to all of them.
__device__ __forceinline__ bool persist_unit(const Params& p, int r, int& bh, int& mt)
{
    const int G = gridDim.x, S = G / kXcds;
    const int x = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
    const int s2 = (r & 1) ? S - 1 - s : s;
    const long long t = (long long)r * G + (long long)s2 * kXcds + x;
    if (t >= p.n_items) return false;
    const int level = (int)(t / p.bh);
    bh = (int)(t - (long long)level * p.bh);
    mt = p.causal ? p.n_mtiles - 1 - level : level;
    return true;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (fp16 / bf16 on the 32x32x16 matrix cores)
// ---------------------------------------------------------------------------

// XOR swizzles of the 16-byte chunks of K and V rows in LDS (physical chunk =
// logical chunk ^ swizzle(row)).  gfx950's LDS has 64 four-byte banks and
// serves 16 lanes per clock, so a 16-byte K-operand read (16 lanes = 16
// consecutive rows at one logical chunk) is conflict-free when the 16 rows map
// to 16 distinct 16-byte bank groups: a bijection on the low four row bits
// (three bits for 128-byte rows, whose row parity already picks the half of a
// 256-byte bank line).
// The V tile is read with 8-byte transpose reads: 32 lanes (256 bytes) are
// served per clock, and lanes 0-31 read 4 consecutive rows at the 4 logical
// chunks of one 64-byte column group.  Rows of 256 bytes or more therefore
// put row bits 0-1 on chunk bits 2-3 (the 4 rows land in 4 different 64-byte
// quarters of the bank line) and row bit 2 on chunk bit 1: conflict-free, where
// a 3-bit swizzle leaves a 2-way conflict (measured with the LDS bank-conflict
// counter: 12 % of the kernel's time stalled before, none after).  That
// swizzle is used for 256-byte rows (d = 128); other row lengths keep the
// 3-bit form, whose read offsets need half the registers (the d = 256 kernel
// has none to spare: the 4-bit form spilled more and ran slower there).
template <int CPR>
__device__ __forceinline__ int swz_k(int row)
{
    if (CPR >= 16)
        return ((row & 1) ? 8 : 0) ^ ((row & 2) ? 2 : 0) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 4 : 0);
    return ((row & 2) ? 4 : 0) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 2 : 0);
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row)
{
    if (CPR == 16) return ((row & 3) << 2) | (((row >> 2) & 1) << 1);
    return ((row & 3) << 1) | ((row >> 2) & 1);
}
// V transpose reads: NRV per-lane byte offsets (within the V tile, before the
// 16-key step); d tile dt reads at offset rv[dt % NRV] + (dt / NRV) * VSTEP.
// With the 4-bit swizzle every d tile of a 256-byte row has its own offset;
// with the 3-bit one, d tiles two apart differ by 128 bytes (chunk bit 3,
// which that swizzle does not touch).
template <int CPR>
struct VRead {
    static constexpr int NRV = CPR == 16 ? 4 : 2;
    static constexpr int VSTEP = CPR == 16 ? 256 : 128;
    static __device__ __forceinline__ uint32_t offset(int e, int v_row, int vhalf, int vc)
    {
        const int logical = (e & 1) * 4 + 2 * vhalf + (vc >> 1) + 8 * ((e >> 1) & 1);
        return v_row * CPR * 16 + ((logical ^ swz_v<CPR>(v_row)) << 4) + (vc & 1) * 8;
    }
};


// QB 32-row query blocks per wave: every K or V operand read from LDS feeds
// QB matrix-core instructions.  QB = 1 keeps two waves per SIMD; QB = 2 halves
// the LDS traffic per MFMA at one wave per SIMD (more registers per wave).
// SPLIT: a work item is one part of a query tile's key range (split-KV); the
// tile writes its partial O (normalised by its own row sum) and partial LSE in
// fp32 to the workspace, and fa_combine merges the parts.
// VARLEN: packed variable-length sequences; a work item is one query tile of
// one sequence of one head, and every address is offset to that sequence.
// KG = 2: two key groups of NW waves share the tile's query rows; group g
// takes key tiles g, g + 2, ... through its own LDS stages (both groups step
// through the same barriers), and at the end group 1 hands its unnormalised
// O, running max and row sum to group 0 through LDS, which merges them.  For
// problems with fewer work items than CUs: each wave walks half the key tiles
// and every SIMD holds two waves.
template <int D, int BN, int NW, int QB, bool BF16, bool CAUSAL, bool SPLIT, bool VARLEN = false, int KG = 1>
__global__ void __launch_bounds__(NW * KG * 64, QB == 1 && KG == 1 ? 2 : 1)
fa_fwd_16(Params p)
{
    constexpr int BM = NW * 32 * QB;     // query rows per workgroup tile
    constexpr int WR = 32 * QB;          // query rows per wave
    constexpr int NKB = BN / 32;         // 32-key blocks per key tile
    constexpr int NDT = D / 32;          // 32-wide d tiles of the output
    constexpr int NKK = D / 16;          // k-steps of the score product
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int RB = D * 2;            // bytes per K/V row
    constexpr int TILE = BN * D;         // elements of one K or V tile
    constexpr int TB = TILE * 2;         // bytes of one K or V tile
    constexpr int NCH = BN * CPR;        // 16-byte chunks per tile
    constexpr int DMA = NCH / 64 / NW;   // 1 KiB copies per wave per tensor per tile
    constexpr int NKR = NKK < 8 ? NKK : 8;  // distinct K-read lane offsets
    static_assert(CPR >= 8, "swizzles need at least 8 chunks per row");
    static_assert(DMA >= 1 && NCH % (64 * NW) == 0, "tile must split evenly over waves");
    static_assert(KG * 2 * 2 * TB <= 160 * 1024, "LDS budget");
    static_assert(KG == 1 || (KG == 2 && QB == 1 && !SPLIT), "key groups: one-block tiles, not split-KV");
    constexpr int GROUP_BYTES = 2 * 2 * TB;  // one key group's two stages

    // [key group][stage][0 = K, 1 = V][BN rows x D], rows row-major with
    // swizzled chunks
    __shared__ __attribute__((aligned(16))) uint16_t lds[KG][2][2][TILE];

    int bh, item;
    if (!map_item(p, bh, item)) return;

    const int tid = threadIdx.x;
    // (both wave-uniform; readfirstlane tells the compiler so, which keeps the
    // branches on them uniform and the copy bases in scalar registers)
    const int kg = KG > 1 ? __builtin_amdgcn_readfirstlane((tid >> 6) / NW) : 0;  // key group
    const int w = KG > 1 ? __builtin_amdgcn_readfirstlane((tid >> 6) % NW) : tid >> 6;  // wave within it
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    int sq = p.sq, sk = p.sk;
    size_t qoff = (size_t)bh * sq, koff = (size_t)bh * sk;  // first row of this slice
    int vtile = 0;
    if constexpr (VARLEN) {
        // bh = head; item = sequence * (query tiles of the longest sequence) + tile.
        // Offsets are clamped into [0, total] so malformed offsets cannot
        // address outside the buffers.
        const int seq = __builtin_amdgcn_readfirstlane(item / p.n_mtiles);
        vtile = item - seq * p.n_mtiles;
        const int q0s = min(max(p.cu_q[seq], 0), p.total_q), q1s = min(max(p.cu_q[seq + 1], q0s), p.total_q);
        const int k0s = min(max(p.cu_k[seq], 0), p.total_k), k1s = min(max(p.cu_k[seq + 1], k0s), p.total_k);
        sq = q1s - q0s;
        sk = k1s - k0s;
        if (vtile * BM >= sq || sk <= 0) return;  // the whole workgroup leaves together
        qoff = (size_t)bh * p.total_q + q0s;
        koff = (size_t)bh * p.total_k + k0s;
    }
    const float c = p.c;  // |scale| * log2(e)
    constexpr float kRescaleThreshold = 8.f;  // lazy rescale: p <= 2^8
    constexpr float kRescaleLimit = 256.f;    // partial row sum that forces the exact max

    const uint16_t* __restrict__ Q = (const uint16_t*)p.q + qoff * D;
    const uint16_t* __restrict__ K = (const uint16_t*)p.k + koff * D;
    const uint16_t* __restrict__ V = (const uint16_t*)p.v + koff * D;
    uint16_t* __restrict__ O = (uint16_t*)p.o + qoff * D;

    // ---- global -> LDS copies.  Copy j of wave w fills LDS chunks
    //      c = (w*DMA + j)*64 + lane: row c / CPR, physical chunk c % CPR,
    //      fetched from the swizzled logical chunk.  Per-lane byte offsets
    //      within a tile are fixed; the tile base is a scalar. ----
    uint32_t dk[DMA], dv[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int cc = (w * DMA + j) * 64 + lane;
        const int row = cc / CPR, pch = cc % CPR;
        dk[j] = row * RB + ((pch ^ swz_k<CPR>(row)) << 4);
        dv[j] = row * RB + ((pch ^ swz_v<CPR>(row)) << 4);
    }
    const uint32_t lds0 = lds_addr(&lds[0][0][0][0]) + kg * GROUP_BYTES;
    // copy j of K or V for the tile at n0 into stage `stage`.  full: the tile
    // lies inside [0, sk) and the precomputed offsets apply; otherwise rows
    // past the last key re-read the last key (finite data; those keys' scores
    // are masked).
    // LDS byte address of this wave's first copy slot (stage 0, K)
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds0 + w * DMA * 1024);
    auto copy_k = [&](auto j_tag, auto st_tag, int n0, bool full) {
        constexpr int J = decltype(j_tag)::value, ST = decltype(st_tag)::value;
        const void* src = K + (size_t)n0 * D;
        if constexpr (SPLIT || VARLEN) src = uniform_ptr(src);
        if (full) {
            copy_1k<ST * 2 * TB + J * 1024>(src, dk[J], lbase);
        } else {
            const int cc = (w * DMA + J) * 64 + lane;
            const int row = cc / CPR, pch = cc % CPR;
            copy_1k<ST * 2 * TB + J * 1024>(src, min(row, sk - 1 - n0) * RB + ((pch ^ swz_k<CPR>(row)) << 4), lbase);
        }
    };
    auto copy_v = [&](auto j_tag, auto st_tag, int n0, bool full) {
        constexpr int J = decltype(j_tag)::value, ST = decltype(st_tag)::value;
        const void* src = V + (size_t)n0 * D;
        if constexpr (SPLIT || VARLEN) src = uniform_ptr(src);
        if (full) {
            copy_1k<ST * 2 * TB + TB + J * 1024>(src, dv[J], lbase);
        } else {
            const int cc = (w * DMA + J) * 64 + lane;
            const int row = cc / CPR, pch = cc % CPR;
            copy_1k<ST * 2 * TB + TB + J * 1024>(src, min(row, sk - 1 - n0) * RB + ((pch ^ swz_v<CPR>(row)) << 4), lbase);
        }
    };
    auto issue_tile = [&](auto st_tag, int n0) {
        const bool full = n0 + BN <= sk;
        static_for<DMA>([&](auto j) {
            copy_k(j, st_tag, n0, full);
            copy_v(j, st_tag, n0, full);
        });
    };
    // copies of the next tile are spread over the current tile's matrix-core
    // work (K copies after each 32-key score block, V copies after each
    // 16-key PV chunk) instead of one burst that stalls the wave at issue.
    // Non-causal d = 256 (32-key tiles, one score block) takes them in one
    // burst between the score products and the softmax instead: measured 4.6 %
    // faster there; the same change made the causal d = 256 variant 68 %
    // slower (the compiler moved its register spills into the loop) and d = 128
    // with two key groups 3 % slower, so those keep the spread copies.
    constexpr bool COPY_BURST = D > 128 && !CAUSAL;
    constexpr int KC_PER = (DMA + NKB - 1) / NKB;
    constexpr int VC_PER = (DMA + 2 * NKB - 1) / (2 * NKB);

    // ---- per-lane LDS read offsets (bytes within a stage) ----
    //  K (S^T A operand): row kb*32 + l32, logical chunk 2kk + g
    uint32_t rk[NKR];
#pragma unroll
    for (int kk = 0; kk < NKR; ++kk) rk[kk] = kg * GROUP_BYTES + l32 * RB + (((2 * kk + g) ^ swz_k<CPR>(l32)) << 4);
    //  V (O^T A operand, transpose reads): lane 4r + c of its 16-lane group
    //  reads key row 16kc + 8j + 4g + r, d = 32dt + 16*half + 4c
    const int sub = lane & 15, vr = sub >> 2, vc = sub & 3, vhalf = (lane >> 4) & 1;
    const int v_row = 4 * g + vr;
    constexpr int NRV = VRead<CPR>::NRV < NDT ? VRead<CPR>::NRV : NDT;
    uint32_t rv[NRV];
#pragma unroll
    for (int e = 0; e < NRV; ++e) rv[e] = kg * GROUP_BYTES + TB + VRead<CPR>::offset(e, v_row, vhalf, vc);

    auto process = [&](const int mt, const int split) {
        const int q0 = mt * BM;

        // ---- key range of this tile and of this wave ----
        const int q_end = min(q0 + BM, sq);
        const int kv_end = CAUSAL ? min(q_end, sk) : sk;
        const int nkv = (kv_end + BN - 1) / BN;
        // key tiles [t_lo, t_hi) of this work item: all of them, or part
        // `split` of nsplit near-equal parts (possibly empty)
        int t_lo = 0, t_hi = nkv;
        if (SPLIT) {
            // (the division runs on the vector unit; the values are uniform)
            const int chunk = __builtin_amdgcn_readfirstlane((nkv + p.nsplit - 1) / p.nsplit);
            t_lo = __builtin_amdgcn_readfirstlane(min(nkv, split * chunk));
            t_hi = __builtin_amdgcn_readfirstlane(min(nkv, t_lo + chunk));
        }
        const int wq_first = q0 + w * WR;
        const int wq_end = min(wq_first + WR, sq);
        const int w_kv_end = (wq_end <= wq_first) ? 0 : (CAUSAL ? min(wq_end, sk) : sk);
        const int w_nkv = (w_kv_end + BN - 1) / BN;

        // ---- Q fragments: B operand of S^T = K Q^T, lane = query, 8 d values;
        //      rows past the end read the last row (finite, never stored) ----
        int qrow[QB];
        u32x4_t qf[QB][NKK];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            qrow[qb] = wq_first + qb * 32 + l32;
            const uint16_t* qptr = Q + (size_t)min(qrow[qb], sq - 1) * D + g * 8;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qf[qb][kk] = *(const u32x4_t*)(qptr + kk * 16) ^ p.qsign;
        }

        // ---- running softmax state (log2 units), output accumulators ----
        float m_run[QB], l_run[QB];
        f32x16_t oacc[QB][NDT];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][dt][r] = 0.f;
        }

        // PF_FULL: the next tile lies inside [0, sk) and its copies are issued
        // from inside this tile's math; otherwise the caller has issued them
        auto compute = [&](auto stage_tag, auto full_tag, int n0) {
            constexpr int S = decltype(stage_tag)::value;
            constexpr bool PF_FULL = decltype(full_tag)::value;
            const char* sb = (const char*)&lds[0][S][0][0];  // the key group's offset is in rk, rv
            const int nn = n0 + KG * BN;  // prefetched tile (this key group's next)

            // ---- S^T = K Q^T on the matrix cores (each K read feeds QB) ----
            f32x16_t s[QB][NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const u32x4_t a = *(const u32x4_t*)(sb + rk[kk & 7] + kb * 32 * RB + (kk >> 3) * 256);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma16(a, qf[qb][kk], s[qb][kb], BF16);
                }
                if (PF_FULL && !COPY_BURST)
                    static_for<DMA>([&](auto j) {
                        if (j.value >= kb * KC_PER && j.value < (kb + 1) * KC_PER)
                            copy_k(j, Stage<S ^ 1>{}, nn, true);
                    });
            }
            if (PF_FULL && COPY_BURST)
                static_for<DMA>([&](auto j) {
                    copy_k(j, Stage<S ^ 1>{}, nn, true);
                    copy_v(j, Stage<S ^ 1>{}, nn, true);
                });

            // ---- masks: ragged key tail, causal diagonal.  Score r of block kb
            //      is key n0 + 32kb + 4g + off(r); it lives iff key <= lim =
            //      min(sk - 1, qrow) (causal) or sk - 1, so the sign of
            //      lim - key selects -inf with a mask and a bit-field insert (no
            //      per-element compare: their lane masks would take scalar
            //      registers) ----
            const bool need_mask = (n0 + BN > sk) || (CAUSAL && n0 + BN - 1 > wq_first);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int lim0 = (CAUSAL ? min(sk - 1, qrow[qb]) : sk - 1) - n0 - 4 * g;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                            const uint32_t dead = (uint32_t)((lim0 - off) >> 31);
                            const float x = s[qb][kb][r];  // through a scalar: a bit cast of a vector element reads element 0
                            const uint32_t bits = __builtin_bit_cast(uint32_t, x);
                            s[qb][kb][r] = __builtin_bit_cast(float, (bits & ~dead) | (0xff800000u & dead));
                        }
                }
            }

            // ---- online softmax (log2 units) ----
            // The running max m is only a reference point: any m gives the same
            // result as long as no probability overflows.  So the tile is first
            // exponentiated against the running max; only when that max is
            // unset (a row's first tile) or some lane's partial row sum passes
            // 2^8 (a probability may exceed 2^8) is the exact tile max taken,
            // m raised (with O and l rescaled) if it grew by more than 2^8,
            // and the tile exponentiated again.  Probabilities therefore stay
            // <= 2^8 (fp16 P cannot overflow); the row sum adds the fp32 values.
            u32x4_t pk[QB][2 * NKB];
            float lsum[QB];
            auto exponentiate = [&]() {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const float m_use = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
                    float acc = 0.f;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) {
                            const float p0 = fast_exp2(__builtin_fmaf(s[qb][kb][r], c, -m_use));
                            const float p1 = fast_exp2(__builtin_fmaf(s[qb][kb][r + 1], c, -m_use));
                            acc += p0 + p1;
                            pk[qb][2 * kb + (r >> 3)][(r >> 1) & 3] = pack2(p0, p1, BF16);
                        }
                    lsum[qb] = acc;
                }
            };
            bool unset = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) unset = unset || (m_run[qb] == -INFINITY);
            bool exact = __builtin_amdgcn_ballot_w64(unset) != 0;
            if (!exact) {
                exponentiate();
                bool big = false;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) big = big || (lsum[qb] > kRescaleLimit);
                exact = __builtin_amdgcn_ballot_w64(big) != 0;
            }
            if (exact) {
                float mt_[QB];
                bool grow = false;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float mx = s[qb][0][0];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
                    mx = fmaxf(mx, __shfl_xor(mx, 32));  // lanes l and l+32 share a query
                    mt_[qb] = mx * c;
                    grow = grow || (mt_[qb] > m_run[qb] + kRescaleThreshold);
                }
                if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const float m_new = fmaxf(m_run[qb], mt_[qb]);
                        const float alpha = fast_exp2(m_run[qb] - m_new);  // 0 when m_run = -inf
                        l_run[qb] *= alpha;
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[qb][dt][r] *= alpha;
                        m_run[qb] = m_new;
                    }
                }
                exponentiate();
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_run[qb] += lsum[qb];

            // ---- O^T += V^T P^T: A operand = two 4-key transpose reads, each
            //      feeding QB matrix-core instructions ----
#pragma unroll
            for (int kc = 0; kc < 2 * NKB; ++kc) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const char* va = sb + rv[dt % NRV] + (dt / NRV) * VRead<CPR>::VSTEP + kc * 16 * RB;
                    const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va));
                    const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va + 8 * RB));
                    const u32x4_t a = u32x4_t{__builtin_bit_cast(u32x2_t, x0)[0], __builtin_bit_cast(u32x2_t, x0)[1],
                                              __builtin_bit_cast(u32x2_t, x1)[0], __builtin_bit_cast(u32x2_t, x1)[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma16(a, pk[qb][kc], oacc[qb][dt], BF16);
                }
                if (PF_FULL && !COPY_BURST)
                    static_for<DMA>([&](auto j) {
                        if (j.value >= kc * VC_PER && j.value < (kc + 1) * VC_PER)
                            copy_v(j, Stage<S ^ 1>{}, nn, true);
                    });
            }
        };

        // one key tile: publish its stage, then compute (the stage index is a
        // template constant so every LDS offset is an immediate).  Key group
        // kg takes tiles t_lo + kg, t_lo + kg + KG, ...; every group runs the
        // same number of steps (a group past its last tile only joins the
        // barrier)
        auto step = [&](auto stage_tag, int t) {
            constexpr int S = decltype(stage_tag)::value;
            wait_copies();
            __syncthreads();
            const bool pf = t + KG < t_hi;
            const bool pf_full = pf && (t + KG + 1) * BN <= sk;
            if (t < w_nkv && pf_full) {
                compute(stage_tag, Stage<1>{}, t * BN);
            } else {
                if (pf) issue_tile(Stage<S ^ 1>{}, (t + KG) * BN);
                if (t < w_nkv && t < t_hi) compute(stage_tag, Stage<0>{}, t * BN);
            }
        };

        const int g_lo = t_lo + kg;
        const int nsteps = (t_hi - t_lo + KG - 1) / KG;
        if (g_lo < t_hi) issue_tile(Stage<0>{}, g_lo * BN);
        int i = 0;
        for (; i + 1 < nsteps; i += 2) {
            step(Stage<0>{}, g_lo + i * KG);
            step(Stage<1>{}, g_lo + (i + 1) * KG);
        }
        if (i < nsteps) step(Stage<0>{}, g_lo + i * KG);

        if constexpr (KG > 1) {
            // ---- merge the key groups: group 1 parks its unnormalised O^T,
            //      running max and partial row sum in LDS (lane-major, so group
            //      0's wave w reads them back in its own register layout), and
            //      group 0 rescales both to the larger max and adds.  A group
            //      that saw no key of a row has m = -inf, l = 0, O = 0 and
            //      weight 0. ----
            constexpr int NR = NDT * 16;  // accumulator registers per lane
            static_assert(NW * (NR + 2) * 64 * 4 <= KG * GROUP_BYTES, "merge buffer inside the stages");
            float* mb = (float*)&lds[0][0][0][0] + (size_t)w * (NR + 2) * 64;
            __syncthreads();  // every wave is done with the stages
            if (kg == 1) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mb[(dt * 16 + r) * 64 + lane] = oacc[0][dt][r];
                mb[NR * 64 + lane] = m_run[0];
                mb[(NR + 1) * 64 + lane] = l_run[0];
            }
            __syncthreads();
            if (kg == 1) return;  // group 0 writes the tile
            const float m1 = mb[NR * 64 + lane], l1 = mb[(NR + 1) * 64 + lane];
            const float m = fmaxf(m_run[0], m1);
            const float a0 = m_run[0] == -INFINITY ? 0.f : fast_exp2(m_run[0] - m);
            const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[0][dt][r] = __builtin_fmaf(oacc[0][dt][r], a0, mb[(dt * 16 + r) * 64 + lane] * a1);
                __builtin_amdgcn_sched_barrier(0);  // one d tile's loads at a time
            }
            l_run[0] = __builtin_fmaf(l_run[0], a0, l1 * a1);
            m_run[0] = m;
        }

        // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ----
        if constexpr (SPLIT) {
            // partial results of key tiles [t_lo, t_hi) in fp32; a row that saw
            // no key here gets O = 0 and LSE = -inf (weight 0 in the merge)
            const size_t rows = (size_t)p.bh * sq;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
                if (qrow[qb] < sq) {
                    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
                    const size_t r = (size_t)split * rows + (size_t)bh * sq + qrow[qb];
                    float* orow = p.ws + r * D;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int rb = 0; rb < 4; ++rb) {
                            f32x4_t v4;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v4[e] = oacc[qb][dt][rb * 4 + e] * inv;
                            *(f32x4_t*)(orow + dt * 32 + rb * 8 + g * 4) = v4;
                        }
                    if (g == 0)
                        p.ws[(size_t)p.nsplit * rows * D + r] =
                            l_tot > 0.f ? (m_run[qb] + __log2f(l_tot)) * kLn2 : -INFINITY;
                }
            }
            return;
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
            if (qrow[qb] < sq) {
                const float inv = 1.f / l_tot;
                uint16_t* orow = O + (size_t)qrow[qb] * D;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        const uint32_t w0 = pack2(oacc[qb][dt][rb * 4 + 0] * inv, oacc[qb][dt][rb * 4 + 1] * inv, BF16);
                        const uint32_t w1 = pack2(oacc[qb][dt][rb * 4 + 2] * inv, oacc[qb][dt][rb * 4 + 3] * inv, BF16);
                        *(u32x2_t*)(orow + dt * 32 + rb * 8 + g * 4) = u32x2_t{w0, w1};
                    }
                if (g == 0) p.lse[qoff + qrow[qb]] = (m_run[qb] + __log2f(l_tot)) * kLn2;
            }
        }
    };

    if constexpr (VARLEN) {
        // one query tile of one sequence; heaviest first when causal
        const int ntiles = (sq + BM - 1) / BM;
        process(CAUSAL ? ntiles - 1 - vtile : vtile, 0);
        return;
    }
    if constexpr (SPLIT) {
        // item = query tile (heaviest first when causal) x key-range part
        const int mq = __builtin_amdgcn_readfirstlane(item / p.nsplit);
        process(CAUSAL ? p.n_mtiles - 1 - mq : mq, item - mq * p.nsplit);
        return;
    }
    int mts[2];
    const int nt = item_tiles(p, item, mts);
    process(mts[0], 0);
    if (nt > 1) {
        __syncthreads();  // every wave is done with the LDS stages
        process(mts[1], 0);
    }
}

// ---------------------------------------------------------------------------
// 16-bit ping-pong kernel: two wave groups alternate matrix-core and softmax
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per CU; waves 0-3 (group A) and 4-7 (group B) share
// the SIMDs pairwise.  Each key tile t is a window of two slots that starts at a
// workgroup barrier; group A runs its matrix-core phase M(t) = { S(t) = K(t) Q^T,
// O^T += V(t-1)^T P(t-1)^T } and then its softmax phase X(t) = softmax(S(t)) ->
// P(t), group B runs X(t-1) and then M(t):
//   slot 2t:   A: M(t)   B: X(t-1)
//   slot 2t+1: A: X(t)   B: M(t)
// so each SIMD has one wave issuing matrix-core work while the other issues
// VALU work.  The slots need no barrier between them (no LDS stage changes
// hands inside a window), so a wave moves on as soon as its own phase ends.
// K(t) and V(t-1) are read inside window t; the copies of K(t+1) and V(t) go
// out during it (each wave's at the start of its own softmax phase) into the
// stages freed by window t-1 and are awaited before the barrier that ends it.
// Group A's wave i owns query rows [64i, 64i+32) of the 256-row tile and
// group B's wave i rows [64i+32, 64i+64), so both groups reach the causal
// diagonal together.
// VARLEN: packed variable-length sequences (at most 64, h a multiple of 8);
// a work item is one causal pair (or, without the mask, one query tile) of
// one sequence of one head, and every address is offset to that sequence.
// Workgroup t is dispatched to XCD x = t mod 8, which owns heads x, x + 8, ...;
// its slot t / 8 walks the XCD's list: the sequences in descending order of
// cost (causal: query tiles; else keys; ties by index), for each the XCD's
// heads, for each head that sequence's items.  The heaviest items start
// first, and the items of one (head, sequence) start together on one XCD, so
// its L2 serves their K/V reads (the light tiles walk down as in the dense
// grid); with the heads innermost instead, a model of the L2 puts the K/V
// fetched at 2.3x the unique bytes on mixed lengths, this order at 1.6x.
template <int D, int BN, bool BF16, bool CAUSAL, bool PERSIST, bool VARLEN = false>
__global__ void __launch_bounds__(512, 1)
fa_fwd_16pp(Params p)
{
    static_assert(!(PERSIST && VARLEN), "the persistent schedule walks dense heads only");
    constexpr int NW = 8;                // waves per workgroup
    constexpr int BM = 256;              // query rows per workgroup tile
    constexpr int NKB = BN / 32;         // 32-key blocks per key tile
    constexpr int NDT = D / 32;          // 32-wide d tiles of the output
    constexpr int NKK = D / 16;          // k-steps of the score product
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int RB = D * 2;            // bytes per K/V row
    constexpr int TILE = BN * D;         // elements of one K or V tile
    constexpr int TB = TILE * 2;         // bytes of one K or V tile
    constexpr int NCH = BN * CPR;        // 16-byte chunks per tile
    constexpr int DMA = NCH / 64 / NW;   // 1 KiB copies per wave per tensor per tile
    constexpr int NKR = NKK < 8 ? NKK : 8;
    static_assert(CPR >= 8, "swizzles need at least 8 chunks per row");
    static_assert(DMA >= 1 && NCH % (64 * NW) == 0, "tile must split evenly over waves");
    static_assert(4 * TB <= 160 * 1024, "LDS budget");

    // [0..1] K stages, [2..3] V stages; BN rows x D, swizzled 16-byte chunks
    __shared__ __attribute__((aligned(16))) uint16_t lds[4][TILE];

    int bh = 0, item = 0;
    if constexpr (!PERSIST && !VARLEN) {
        if (!map_item(p, bh, item)) return;
    }

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int grp = w >> 2;              // 0: group A, 1: group B
    const int wi = w & 3;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    int sq = p.sq, sk = p.sk;  // per sequence when VARLEN
    const float c = p.c;  // |scale| * log2(e)
    constexpr float kRescaleThreshold = 8.f;
    constexpr float kRescaleLimit = 256.f;

    // this head's slices (set per work unit)
    const uint16_t* __restrict__ Q = nullptr;
    const uint16_t* __restrict__ K = nullptr;
    const uint16_t* __restrict__ V = nullptr;
    uint16_t* __restrict__ O = nullptr;
    size_t lse0 = 0;  // LSE index of the slice's first row
    auto set_head = [&](int h) {
        Q = (const uint16_t*)p.q + (size_t)h * sq * D;
        K = (const uint16_t*)p.k + (size_t)h * sk * D;
        V = (const uint16_t*)p.v + (size_t)h * sk * D;
        O = (uint16_t*)p.o + (size_t)h * sq * D;
        lse0 = (size_t)h * sq;
    };

    // ---- copies: wave w fills LDS chunks (w*DMA + j)*64 + lane of a tile ----
    uint32_t dk[DMA], dv[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int cc = (w * DMA + j) * 64 + lane;
        const int row = cc / CPR, pch = cc % CPR;
        dk[j] = row * RB + ((pch ^ swz_k<CPR>(row)) << 4);
        dv[j] = row * RB + ((pch ^ swz_v<CPR>(row)) << 4);
    }
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(&lds[0][0]) + w * DMA * 1024);
    auto copy_k = [&](auto j_tag, auto st_tag, int n0, bool full) {
        constexpr int J = decltype(j_tag)::value, ST = decltype(st_tag)::value;
        const void* src = K + (size_t)n0 * D;
        if constexpr (VARLEN) src = uniform_ptr(src);
        if (full) {
            copy_1k<ST * TB + J * 1024>(src, dk[J], lbase);
        } else {
            const int cc = (w * DMA + J) * 64 + lane;
            const int row = cc / CPR, pch = cc % CPR;
            copy_1k<ST * TB + J * 1024>(src, min(row, sk - 1 - n0) * RB + ((pch ^ swz_k<CPR>(row)) << 4), lbase);
        }
    };
    auto copy_v = [&](auto j_tag, auto st_tag, int n0, bool full) {
        constexpr int J = decltype(j_tag)::value, ST = decltype(st_tag)::value;
        const void* src = V + (size_t)n0 * D;
        if constexpr (VARLEN) src = uniform_ptr(src);
        if (full) {
            copy_1k<(2 + ST) * TB + J * 1024>(src, dv[J], lbase);
        } else {
            const int cc = (w * DMA + J) * 64 + lane;
            const int row = cc / CPR, pch = cc % CPR;
            copy_1k<(2 + ST) * TB + J * 1024>(src, min(row, sk - 1 - n0) * RB + ((pch ^ swz_v<CPR>(row)) << 4), lbase);
        }
    };

    // ---- per-lane LDS read offsets (bytes within a stage) ----
    uint32_t rk[NKR];
#pragma unroll
    for (int kk = 0; kk < NKR; ++kk) rk[kk] = l32 * RB + (((2 * kk + g) ^ swz_k<CPR>(l32)) << 4);
    const int sub = lane & 15, vr = sub >> 2, vc = sub & 3, vhalf = (lane >> 4) & 1;
    const int v_row = 4 * g + vr;
    static_assert(VRead<CPR>::NRV == NDT, "one read offset per d tile");
    uint32_t rv[NDT];
#pragma unroll
    for (int e = 0; e < NDT; ++e) rv[e] = VRead<CPR>::offset(e, v_row, vhalf, vc);

    // process(DESC, mt): query tile mt, key tiles in ascending (DESC false) or
    // descending order; window t works on key tile kt(t) = t or nkv-1-t.  A
    // wave whose rows end early skips the key tiles past its own last one:
    // the last windows (ascending) or the first ones (descending).  In either
    // order the first tile a wave computes holds a live key for every one of
    // its rows (the key at the tile's start is at most its first row), so no
    // row starts from a fully masked tile.
    auto process = [&](auto desc_tag, const int mt) {
        constexpr bool DESC = decltype(desc_tag)::value;
        const int q0 = mt * BM;
        const int q_end = min(q0 + BM, sq);
        const int kv_end = CAUSAL ? min(q_end, sk) : sk;
        const int nkv = (kv_end + BN - 1) / BN;
        const int wq_first = q0 + 64 * wi + 32 * grp;
        const int wq_end = min(wq_first + 32, sq);
        const int w_kv_end = (wq_end <= wq_first) ? 0 : (CAUSAL ? min(wq_end, sk) : sk);
        const int w_nkv = (w_kv_end + BN - 1) / BN;
        const int qrow = wq_first + l32;
        const int t_first = DESC ? nkv - w_nkv : 0;  // this wave's windows [t_first, t_end)
        const int t_end = DESC ? nkv : w_nkv;
        auto key0 = [&](int t) { return (DESC ? nkv - 1 - t : t) * BN; };

        // K(kt(0)) goes out before the Q loads
        {
            const int n0 = key0(0);
            const bool f = n0 + BN <= sk;
            static_for<DMA>([&](auto j) { copy_k(j, Stage<0>{}, n0, f); });
        }
        const uint16_t* qptr = Q + (size_t)min(qrow, sq - 1) * D + g * 8;
        u32x4_t qf[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qf[kk] = *(const u32x4_t*)(qptr + kk * 16) ^ p.qsign;

        float m_run = -INFINITY, l_run = 0.f;
        f32x16_t oacc[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
        f32x16_t s[NKB];
        u32x4_t pk[2 * NKB];

        // ---- M(t): S(t) from K stage KS and PV(t-1) from V stage VS ----
        auto mphase = [&](auto ks_tag, auto vs_tag, bool do_s, bool do_pv) {
            constexpr int KS = decltype(ks_tag)::value, VS = decltype(vs_tag)::value;
            const char* kb_ = (const char*)&lds[KS][0];
            const char* vb_ = (const char*)&lds[2 + VS][0];
            auto score = [&]() {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const u32x4_t a = *(const u32x4_t*)(kb_ + rk[kk & 7] + kb * 32 * RB + (kk >> 3) * 256);
                        s[kb] = mfma16(a, qf[kk], s[kb], BF16);
                    }
                }
            };
            auto pvm = [&]() {
#pragma unroll
                for (int kc = 0; kc < 2 * NKB; ++kc)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const char* va = vb_ + rv[dt] + kc * 16 * RB;
                        const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va));
                        const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va + 8 * RB));
                        const u32x4_t a = u32x4_t{__builtin_bit_cast(u32x2_t, x0)[0], __builtin_bit_cast(u32x2_t, x0)[1],
                                                  __builtin_bit_cast(u32x2_t, x1)[0], __builtin_bit_cast(u32x2_t, x1)[1]};
                        oacc[dt] = mfma16(a, pk[kc], oacc[dt], BF16);
                    }
            };
            if (do_s && do_pv) {
                // 32 steps alternating a PV and an S matrix-core instruction;
                // each step's LDS operand is fetched kAhead steps earlier into
                // a small register ring so LDS latency hides behind the MFMAs
                constexpr int NPV = 2 * NKB * NDT, NSC = NKB * NKK, NST = NPV + NSC;
                static_assert(NPV == NSC, "alternating schedule needs equal halves");
                constexpr int kAhead = 6;
                u32x4_t ring[kAhead];
                auto fetch = [&](auto i_tag) {
                    constexpr int I = decltype(i_tag)::value;
                    if constexpr (I % 2 == 0) {
                        constexpr int op = I / 2, kc = op / NDT, dt = op % NDT;
                        const char* va = vb_ + rv[dt] + kc * 16 * RB;
                        const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va));
                        const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(va + 8 * RB));
                        ring[I % kAhead] = u32x4_t{__builtin_bit_cast(u32x2_t, x0)[0], __builtin_bit_cast(u32x2_t, x0)[1],
                                                   __builtin_bit_cast(u32x2_t, x1)[0], __builtin_bit_cast(u32x2_t, x1)[1]};
                    } else {
                        constexpr int op = I / 2, kb = op / NKK, kk = op % NKK;
                        ring[I % kAhead] = *(const u32x4_t*)(kb_ + rk[kk & 7] + kb * 32 * RB + (kk >> 3) * 256);
                    }
                };
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
                static_for<kAhead>([&](auto i) { fetch(i); });
                static_for<NST>([&](auto i_tag) {
                    constexpr int I = decltype(i_tag)::value;
                    const u32x4_t a = ring[I % kAhead];
                    if constexpr (I + kAhead < NST) fetch(Stage<I + kAhead>{});
                    if constexpr (I % 2 == 0) {
                        constexpr int op = I / 2, kc = op / NDT, dt = op % NDT;
                        oacc[dt] = mfma16(a, pk[kc], oacc[dt], BF16);
                    } else {
                        constexpr int op = I / 2, kb = op / NKK, kk = op % NKK;
                        s[kb] = mfma16(a, qf[kk], s[kb], BF16);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else {
                if (do_pv) pvm();
                if (do_s) score();
            }
        };

        // ---- X(t): online softmax of S(t) -> P(t) (log2 units); see fa_fwd_16
        //      for the exponentiate-then-check scheme ----
        auto xphase = [&](int n0) {
            const bool need_mask = (n0 + BN > sk) || (CAUSAL && n0 + BN - 1 > wq_first);
            if (need_mask) {
                // score r of block kb is key n0 + 32kb + 4g + off(r), alive iff
                // key <= min(sk - 1, qrow) (causal) or sk - 1: the sign of the
                // difference selects -inf (no per-element compare, whose lane
                // masks would take scalar registers)
                const int lim0 = (CAUSAL ? min(sk - 1, qrow) : sk - 1) - n0 - 4 * g;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                        const uint32_t dead = (uint32_t)((lim0 - off) >> 31);
                        const float x = s[kb][r];  // through a scalar: a bit cast of a vector element reads element 0
                        const uint32_t bits = __builtin_bit_cast(uint32_t, x);
                        s[kb][r] = __builtin_bit_cast(float, (bits & ~dead) | (0xff800000u & dead));
                    }
            }
            float lsum = 0.f;
            auto exponentiate = [&]() {
                const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
                float acc = 0.f;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
                        const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, -m_use));
                        acc += p0 + p1;
                        pk[2 * kb + (r >> 3)][(r >> 1) & 3] = pack2(p0, p1, BF16);
                    }
                lsum = acc;
            };
            bool exact = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
            if (!exact) {
                exponentiate();
                exact = __builtin_amdgcn_ballot_w64(lsum > kRescaleLimit) != 0;
            }
            if (exact) {
                float mx = s[0][0];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));  // lanes l and l+32 share a query
                const float mt_ = mx * c;
                if (__builtin_amdgcn_ballot_w64(mt_ > m_run + kRescaleThreshold)) {
                    const float m_new = fmaxf(m_run, mt_);
                    const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
                    m_run = m_new;
                }
                exponentiate();
            }
            l_run += lsum;
        };

        // copies of K(kt(t+1)) -> K stage (t+1)&1 and V(kt(t)) -> V stage t&1
        auto issue = [&](auto kst_tag, auto vst_tag, int t) {
            if (t + 1 < nkv) {
                const int n0 = key0(t + 1);
                const bool f = n0 + BN <= sk;
                static_for<DMA>([&](auto j) { copy_k(j, kst_tag, n0, f); });
            }
            if (t < nkv) {
                const int n0 = key0(t);
                const bool f = n0 + BN <= sk;
                static_for<DMA>([&](auto j) { copy_v(j, vst_tag, n0, f); });
            }
        };

        // M(t) for this wave, t = window index; TP = t & 1
        auto do_m = [&](auto tp_tag, int t) {
            constexpr int TP = decltype(tp_tag)::value;
            const bool ds = t >= t_first && t < t_end;
            const bool dp = t - 1 >= t_first && t - 1 < t_end;
            mphase(Stage<TP>{}, Stage<TP ^ 1>{}, ds, dp);
        };
        // the softmax phase is the longer of the two, so its wave takes issue
        // priority over its SIMD partner's matrix-core phase (+0.4-1 % on the
        // causal b4 h32 s4096 workload, measured on two boxes)
        auto do_x = [&](int t) {
            __builtin_amdgcn_s_setprio(1);
            if (t >= t_first && t < t_end) xphase(key0(t));
            __builtin_amdgcn_s_setprio(0);
        };

        // prologue: K(0) resident for everyone
        wait_copies();
        __syncthreads();

        // slots, unrolled by four (two tiles) so every stage index is a constant
        const int nslots = 2 * nkv + 2;
        for (int k = 0; k < nslots; k += 4) {
            const int t = k >> 1;
            // slot k = 2t (t even): A: M(t), B: X(t-1); copies K(t+1), V(t).
            // Each wave issues its copies at the start of its own softmax
            // phase, so their issue overlaps the partner wave's matrix-core
            // phase instead of delaying it (the stages they fill were last
            // read before the barrier that opened this window)
            if (grp == 0) do_m(Stage<0>{}, t); else { issue(Stage<1>{}, Stage<0>{}, t); do_x(t - 1); }
            // slot 2t+1: A: X(t), B: M(t)
            if (grp == 0) { issue(Stage<1>{}, Stage<0>{}, t); do_x(t); } else do_m(Stage<0>{}, t);
            wait_copies();
            lds_barrier();
            if (k + 2 >= nslots) break;
            // slot 2t+2 = 2(t+1) (t+1 odd): A: M(t+1), B: X(t); copies K(t+2), V(t+1)
            if (grp == 0) do_m(Stage<1>{}, t + 1); else { issue(Stage<0>{}, Stage<1>{}, t + 1); do_x(t); }
            // slot 2t+3: A: X(t+1), B: M(t+1)
            if (grp == 0) { issue(Stage<0>{}, Stage<1>{}, t + 1); do_x(t + 1); } else do_m(Stage<1>{}, t + 1);
            wait_copies();
            lds_barrier();
        }

        // epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (qrow < sq) {
            const float inv = 1.f / l_tot;
            uint16_t* orow = O + (size_t)qrow * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const uint32_t w0 = pack2(oacc[dt][rb * 4 + 0] * inv, oacc[dt][rb * 4 + 1] * inv, BF16);
                    const uint32_t w1 = pack2(oacc[dt][rb * 4 + 2] * inv, oacc[dt][rb * 4 + 3] * inv, BF16);
                    *(u32x2_t*)(orow + dt * 32 + rb * 8 + g * 4) = u32x2_t{w0, w1};
                }
            if (g == 0) p.lse[lse0 + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
    };

    if constexpr (PERSIST) {
        // every wave computes the same unit, so the whole workgroup leaves together
        for (int r = 0;; ++r) {
            int mt;
            if (!persist_unit(p, r, bh, mt)) break;
            set_head(bh);
            if (r > 0) __syncthreads();  // every wave is done with the LDS stages
            process(Stage<0>{}, mt);
        }
    } else {
        // the second tile of a causal pair walks its keys downwards.  The
        // pairs of one head start together and cost the same, so pair i
        // starts its second tile (i) after nQ - i query-tile times and ends
        // with the others: walking down, every second tile of the head reads
        // key block nQ - T at time T and they share it in L2, where walking
        // up they would read block 0 again one after another, long after the
        // first tiles read it
        int mts[2];
        int nt;
        if constexpr (VARLEN) {
            // lane i holds sequence i: its lengths (offsets clamped into
            // [0, total], so malformed offsets cannot address outside the
            // buffers), its item count and cost, and the number of items of
            // the sequences ranked before it
            int q0i = 0, k0i = 0, sqi = 0, ski = 0;
            if (lane < p.batch) {
                q0i = min(max(p.cu_q[lane], 0), p.total_q);
                k0i = min(max(p.cu_k[lane], 0), p.total_k);
                sqi = min(max(p.cu_q[lane + 1], q0i), p.total_q) - q0i;
                ski = min(max(p.cu_k[lane + 1], k0i), p.total_k) - k0i;
            }
            const int nti = (sqi + BM - 1) / BM;
            const int cnt = ski > 0 ? (CAUSAL ? (nti + 1) / 2 : nti) : 0;
            const int cost = CAUSAL ? nti : ski;
            int first = 0;
            for (int jj = 0; jj < p.batch; ++jj) {
                const int cj = __builtin_amdgcn_readlane(cost, jj);
                const int nj = __builtin_amdgcn_readlane(cnt, jj);
                first += (cj > cost || (cj == cost && jj < lane)) ? nj : 0;
            }
            const int x = blockIdx.x % kXcds, sl = blockIdx.x / kXcds;
            const int hx = p.bh / kXcds;  // heads per XCD
            const uint64_t mine = __builtin_amdgcn_ballot_w64(cnt > 0 && sl >= hx * first && sl < hx * (first + cnt));
            if (mine == 0) return;  // past the last item: the whole workgroup leaves
            const int seq = __builtin_ffsll((long long)mine) - 1;
            const int c_seq = __builtin_amdgcn_readlane(cnt, seq);
            const int local = sl - hx * __builtin_amdgcn_readlane(first, seq);
            const int kh = local / c_seq;
            const int j = local - kh * c_seq;
            bh = x + kXcds * kh;
            const int q0s = __builtin_amdgcn_readlane(q0i, seq), k0s = __builtin_amdgcn_readlane(k0i, seq);
            sq = __builtin_amdgcn_readlane(sqi, seq);
            sk = __builtin_amdgcn_readlane(ski, seq);
            const int ntiles = (sq + BM - 1) / BM;
            Q = (const uint16_t*)p.q + ((size_t)bh * p.total_q + q0s) * D;
            K = (const uint16_t*)p.k + ((size_t)bh * p.total_k + k0s) * D;
            V = (const uint16_t*)p.v + ((size_t)bh * p.total_k + k0s) * D;
            O = (uint16_t*)p.o + ((size_t)bh * p.total_q + q0s) * D;
            lse0 = (size_t)bh * p.total_q + q0s;
            mts[0] = CAUSAL ? ntiles - 1 - j : j;
            mts[1] = j;
            nt = (CAUSAL && mts[0] != mts[1]) ? 2 : 1;
        } else {
            set_head(bh);
            nt = item_tiles(p, item, mts);
        }
        process(Stage<0>{}, mts[0]);
        if (nt > 1) {
            __syncthreads();  // every wave is done with the LDS stages
            process(Stage<1>{}, mts[1]);
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel (32x32x2 fp32 matrix cores; probabilities stay fp32)
// ---------------------------------------------------------------------------
template <int D, int BN, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64)
fa_fwd_32(Params p)
{
    constexpr int BM = NW * 32;
    constexpr int NT = NW * 64;
    constexpr int NKB = BN / 32;
    constexpr int NDT = D / 32;
    constexpr int NKK = D / 2;
    constexpr int KS = D + 1;            // odd stride: rows land in distinct banks
    constexpr int VS = D + 4;
    constexpr int KT = BN * KS;
    constexpr int VT = BN * VS;
    constexpr int CPR = D / 4;           // 16-byte chunks per row
    constexpr int CH = BN * CPR / NT;    // chunks per thread per tensor
    static_assert(CH >= 1 && BN * CPR % NT == 0, "tile must split evenly");
    static_assert(2 * (KT + VT) * 4 <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) float lds[2 * (KT + VT)];

    int bh, item;
    if (!map_item(p, bh, item)) return;

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const int sq = p.sq, sk = p.sk;
    auto process = [&](const int mt) {
        const int q0 = mt * BM;
        const float* __restrict__ Q = (const float*)p.q + (size_t)bh * sq * D;
        const float* __restrict__ K = (const float*)p.k + (size_t)bh * sk * D;
        const float* __restrict__ V = (const float*)p.v + (size_t)bh * sk * D;
        float* __restrict__ O = (float*)p.o + (size_t)bh * sq * D;

        const int qrow = q0 + w * 32 + l32;
        const float qs = p.qsign ? -1.f : 1.f;
        float qf[NKK];
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qf[kk] = (qrow < sq) ? qs * Q[(size_t)qrow * D + kk * 2 + g] : 0.f;

        const int q_end = min(q0 + BM, sq);
        const int kv_end = CAUSAL ? min(q_end, sk) : sk;
        const int nkv = (kv_end + BN - 1) / BN;
        const int wq_first = q0 + w * 32;
        const int wq_end = min(wq_first + 32, sq);
        const int w_kv_end = (wq_end <= wq_first) ? 0 : (CAUSAL ? min(wq_end, sk) : sk);
        const int w_nkv = (w_kv_end + BN - 1) / BN;

        float m_run = -INFINITY, l_run = 0.f;
        f32x16_t oacc[NDT];
    #pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
    #pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

        f32x4_t kreg[CH], vreg[CH];
        auto load_tile = [&](int n0) {
    #pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = tid + i * NT;
                const int row = c / CPR, col = c % CPR;
                const int key = n0 + row;
                const bool ok = key < sk;
                kreg[i] = ok ? *(const f32x4_t*)(K + (size_t)key * D + col * 4) : f32x4_t{0, 0, 0, 0};
                vreg[i] = ok ? *(const f32x4_t*)(V + (size_t)key * D + col * 4) : f32x4_t{0, 0, 0, 0};
            }
        };
        auto store_tile = [&](int buf) {
            float* Ks = lds + buf * (KT + VT);
            float* Vs = Ks + KT;
    #pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = tid + i * NT;
                const int row = c / CPR, col = c % CPR;
    #pragma unroll
                for (int e = 0; e < 4; ++e) Ks[row * KS + col * 4 + e] = kreg[i][e];
                *(f32x4_t*)(Vs + row * VS + col * 4) = vreg[i];
            }
        };

        const float c = p.c;

        load_tile(0);
        store_tile(0);
        __syncthreads();

        for (int t = 0; t < nkv; ++t) {
            const int n0 = t * BN;
            const bool more = (t + 1 < nkv);
            if (more) load_tile(n0 + BN);

            if (t < w_nkv) {
                const float* Ks = lds + (t & 1) * (KT + VT);
                const float* Vs = Ks + KT;

                f32x16_t s[NKB];
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
    #pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    #pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const float a = Ks[(kb * 32 + l32) * KS + kk * 2 + g];
                        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[kk], s[kb], 0, 0, 0);
                    }
                }

                const bool need_mask = (n0 + BN > sk) || (CAUSAL && n0 + BN - 1 > wq_first);
                if (need_mask) {
    #pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = n0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                            const bool dead = (key >= sk) || (CAUSAL && key > qrow);
                            if (dead) s[kb][r] = -INFINITY;
                        }
                }

                float mx = s[0][0];
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run, mx * c);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run - m_use);
                m_run = m_new;

                float lsum = 0.f;
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float pr = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
                        s[kb][r] = pr;
                        lsum += pr;
                    }
                l_run = l_run * alpha + lsum;
    #pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;

                // O^T += V^T P^T, one key per lane half per step: register r of
                // block kb holds key kb*32 + 8(r/4) + 4g + r%4
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
    #pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            const float a = Vs[key * VS + dt * 32 + l32];
                            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][r], oacc[dt], 0, 0, 0);
                        }
                    }
            }

            if (more) store_tile((t + 1) & 1);
            __syncthreads();
        }

        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (qrow < sq) {
            const float inv = 1.f / l_tot;
            float* orow = O + (size_t)qrow * D;
    #pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
    #pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4_t v4;
    #pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = oacc[dt][rb * 4 + e] * inv;
                    *(f32x4_t*)(orow + dt * 32 + rb * 8 + g * 4) = v4;
                }
            if (g == 0) p.lse[(size_t)bh * sq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
    };

    int mts[2];
    const int nt = item_tiles(p, item, mts);
    process(mts[0]);
    if (nt > 1) {
        __syncthreads();  // every wave is done with the LDS stages
        process(mts[1]);
    }
}

// ---------------------------------------------------------------------------
// split-KV merge of the partial results: LSE = ln sum_p e^{LSE_p},
// O = sum_p e^{LSE_p - LSE} O_p (page "05 · kernel 工程与四代演化", section 2.1,
// lists the split-KV forward class; the weights are the parts' shares of the
// row's softmax denominator)
// ---------------------------------------------------------------------------
// One thread per (row, 8 consecutive d values); the D/8 threads of a row read
// its partial LSEs (cached).  Memory-bound: nsplit * (D + 1) fp32 in per row.
template <int D, bool BF16>
__global__ void __launch_bounds__(256)
fa_combine(Params p)
{
    constexpr int TPR = D / 8;
    const size_t rows = (size_t)p.bh * p.sq;
    const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t row = gid / TPR;
    if (row >= rows) return;
    const int c8 = (int)(gid % TPR) * 8;
    const int ns = p.nsplit;
    const float* wl = p.ws + (size_t)ns * rows * D;
    float m = -INFINITY;
    for (int s = 0; s < ns; ++s) m = fmaxf(m, wl[(size_t)s * rows + row]);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float sum = 0.f;
    if (m != -INFINITY) {
        for (int s = 0; s < ns; ++s) {
            const float wgt = expf(wl[(size_t)s * rows + row] - m);  // 0 for an empty part
            sum += wgt;
            const float* op = p.ws + ((size_t)s * rows + row) * D + c8;
            const f32x4_t a = *(const f32x4_t*)op, b = *(const f32x4_t*)(op + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += wgt * a[e];
                acc[4 + e] += wgt * b[e];
            }
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    u32x4_t out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack2(acc[2 * e] * inv, acc[2 * e + 1] * inv, BF16);
    *(u32x4_t*)((uint16_t*)p.o + row * D + c8) = out;
    if (c8 == 0) p.lse[row] = sum > 0.f ? m + logf(sum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// library-owned scratch for fa_fwd_split_noalloc (callers that cannot
// allocate).  One copy of the array per GPU, held from the library's load
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: host code only ever passes the device address that
// hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) float scratch[kNoallocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* dev_ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// launch table
// ---------------------------------------------------------------------------
template <typename KernelT>
static hipError_t launch(KernelT kernel, int nw, const Params& p, hipStream_t stream)
{
    hipLaunchKernelGGL(kernel, dim3((unsigned)p.grid), dim3((unsigned)(nw * 64)), 0, stream, p);
    return hipGetLastError();
}

template <int D, int BN, int NW, int QB, bool BF16>
static hipError_t launch16(const Params& p, hipStream_t s)
{
    if (p.causal) return launch(fa_fwd_16<D, BN, NW, QB, BF16, true, false>, NW, p, s);
    return launch(fa_fwd_16<D, BN, NW, QB, BF16, false, false>, NW, p, s);
}

// the 4-wave kernel with two key groups (8 waves per workgroup)
template <int D, int BN, bool BF16>
static hipError_t launch16kg(const Params& p, hipStream_t s)
{
    if (p.causal) return launch(fa_fwd_16<D, BN, 4, 1, BF16, true, false, false, 2>, 8, p, s);
    return launch(fa_fwd_16<D, BN, 4, 1, BF16, false, false, false, 2>, 8, p, s);
}

// variable-length sequences (4-wave kernel; with two key groups: 8 waves)
template <int D, int BN, bool BF16>
static hipError_t launch16varlen(const Params& p, bool kg, hipStream_t s)
{
    if constexpr (D <= 128) {
        if (kg) {
            if (p.causal) return launch(fa_fwd_16<D, BN, 4, 1, BF16, true, false, true, 2>, 8, p, s);
            return launch(fa_fwd_16<D, BN, 4, 1, BF16, false, false, true, 2>, 8, p, s);
        }
    }
    if (p.causal) return launch(fa_fwd_16<D, BN, 4, 1, BF16, true, false, true>, 4, p, s);
    return launch(fa_fwd_16<D, BN, 4, 1, BF16, false, false, true>, 4, p, s);
}

// split-KV: the partial-result kernel, then the merge on the same stream
template <int D, int BN, int NW, bool BF16>
static hipError_t launch16split(const Params& p, hipStream_t s)
{
    const hipError_t e = p.causal ? launch(fa_fwd_16<D, BN, NW, 1, BF16, true, true>, NW, p, s)
                                  : launch(fa_fwd_16<D, BN, NW, 1, BF16, false, true>, NW, p, s);
    if (e != hipSuccess) return e;
    const size_t threads = (size_t)p.bh * p.sq * (D / 8);
    auto merge = fa_combine<D, BF16>;
    hipLaunchKernelGGL(merge, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D, int BN, bool BF16>
static hipError_t launch16pp(const Params& p, bool persist, hipStream_t s)
{
    if (persist) {
        if (p.causal) return launch(fa_fwd_16pp<D, BN, BF16, true, true>, 8, p, s);
        return launch(fa_fwd_16pp<D, BN, BF16, false, true>, 8, p, s);
    }
    if (p.causal) return launch(fa_fwd_16pp<D, BN, BF16, true, false>, 8, p, s);
    return launch(fa_fwd_16pp<D, BN, BF16, false, false>, 8, p, s);
}

// variable-length sequences on the ping-pong kernel
template <int D, int BN, bool BF16>
static hipError_t launch16ppvarlen(const Params& p, hipStream_t s)
{
    if (p.causal) return launch(fa_fwd_16pp<D, BN, BF16, true, false, true>, 8, p, s);
    return launch(fa_fwd_16pp<D, BN, BF16, false, false, true>, 8, p, s);
}

template <int D, int BN, int NW>
static hipError_t launch32(const Params& p, hipStream_t s)
{
    if (p.causal) return launch(fa_fwd_32<D, BN, NW, true>, NW, p, s);
    return launch(fa_fwd_32<D, BN, NW, false>, NW, p, s);
}

// tile configuration for a problem; the launch table below dispatches on
// exactly these values.  fp16/bf16 with d = 128 uses the ping-pong kernel
// (256-row tiles, one 8-wave workgroup per CU) when the problem has at least
// one work item per CU, else the 4-wave kernel (128-row tiles, two per CU).
// When even the 4-wave kernel's work items (128-row tiles, causal pairs)
// number fewer than the CUs and each tile sees at least 4 key tiles, d = 64
// and d = 128 take the 4-wave kernel with two key groups: 8 waves per
// workgroup, each walking half of the tile's keys.
bool tile_config(int dtype, int d, int64_t bh, int64_t sq, int64_t sk, int causal, TileConfig* tc)
{
    constexpr int64_t kCUs = 256;
    int bn = 0, nw = 0, qb = 1, lds = 0, kind = 0;
    if (dtype == 1 || dtype == 2) {
        if (d == 64) {
            bn = 128; nw = 4;
        } else if (d == 128) {
            const int64_t nq = (sq + 255) / 256;
            const int64_t items = bh * (causal ? (nq + 1) / 2 : nq);
            if (items >= kCUs) { bn = 64; nw = 8; kind = 1; }
            else { bn = 64; nw = 4; }
        } else if (d == 256) {
            bn = 32; nw = 4;
        } else {
            return false;
        }
        lds = 4 * bn * d * 2;
        if (kind == 0 && d <= 128) {
            const int64_t nq = (sq + 127) / 128;
            const int64_t items = bh * (causal ? (nq + 1) / 2 : nq);
            if (items < kCUs && (sk + bn - 1) / bn >= 4) {
                nw = 8;  // two key groups of 4 waves over 128-row tiles
                kind = 3;
                lds *= 2;
            }
        }
    } else if (dtype == 0) {
        if (d == 64)       { bn = 32; nw = 2; }
        else if (d == 128) { bn = 32; nw = 2; }
        else return false;
        lds = 2 * (bn * (d + 1) + bn * (d + 4)) * 4;
    } else {
        return false;
    }
    tc->block_m = (kind == 3 ? 4 : nw) * 32 * qb;
    tc->block_n = bn;
    tc->waves = nw;
    tc->lds = lds;
    tc->qb = qb;
    tc->kind = kind;
    return true;
}

// split-KV uses the 4-wave kernel's tiles for every head size
bool tile_config_split(int dtype, int d, TileConfig* tc)
{
    if (dtype != 1 && dtype != 2) return false;
    int bn;
    if (d == 64) bn = 128;
    else if (d == 128) bn = 64;
    else if (d == 256) bn = 32;
    else return false;
    tc->block_m = 128;
    tc->block_n = bn;
    tc->waves = 4;
    tc->lds = 4 * bn * d * 2;
    tc->qb = 1;
    tc->kind = 0;
    return true;
}

hipError_t launch_fwd_split(int dtype, int d, const TileConfig& tc, const Params& p, hipStream_t s)
{
    (void)tc;
    switch (dtype) {
    case 2:
        if (d == 64) return launch16split<64, 128, 4, true>(p, s);
        if (d == 128) return launch16split<128, 64, 4, true>(p, s);
        if (d == 256) return launch16split<256, 32, 4, true>(p, s);
        break;
    case 1:
        if (d == 64) return launch16split<64, 128, 4, false>(p, s);
        if (d == 128) return launch16split<128, 64, 4, false>(p, s);
        if (d == 256) return launch16split<256, 32, 4, false>(p, s);
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_varlen(int dtype, int d, const Params& p, int mode, hipStream_t s)
{
    const bool kg = mode == 1;
    switch (dtype) {
    case 2:
        if (d == 64) return launch16varlen<64, 128, true>(p, kg, s);
        if (d == 128) {
            if (mode == 2) return launch16ppvarlen<128, 64, true>(p, s);
            return launch16varlen<128, 64, true>(p, kg, s);
        }
        if (d == 256) return launch16varlen<256, 32, true>(p, false, s);
        break;
    case 1:
        if (d == 64) return launch16varlen<64, 128, false>(p, kg, s);
        if (d == 128) {
            if (mode == 2) return launch16ppvarlen<128, 64, false>(p, s);
            return launch16varlen<128, 64, false>(p, kg, s);
        }
        if (d == 256) return launch16varlen<256, 32, false>(p, false, s);
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(int dtype, int d, const TileConfig& tc, const Params& p, hipStream_t s)
{
    switch (dtype) {
    case 2:
        if (d == 64) return tc.kind == 3 ? launch16kg<64, 128, true>(p, s) : launch16<64, 128, 4, 1, true>(p, s);
        if (d == 128) {
            if (tc.kind == 1 || tc.kind == 2) return launch16pp<128, 64, true>(p, tc.kind == 2, s);
            return tc.kind == 3 ? launch16kg<128, 64, true>(p, s) : launch16<128, 64, 4, 1, true>(p, s);
        }
        if (d == 256) return launch16<256, 32, 4, 1, true>(p, s);
        break;
    case 1:
        if (d == 64) return tc.kind == 3 ? launch16kg<64, 128, false>(p, s) : launch16<64, 128, 4, 1, false>(p, s);
        if (d == 128) {
            if (tc.kind == 1 || tc.kind == 2) return launch16pp<128, 64, false>(p, tc.kind == 2, s);
            return tc.kind == 3 ? launch16kg<128, 64, false>(p, s) : launch16<128, 64, 4, 1, false>(p, s);
        }
        if (d == 256) return launch16<256, 32, 4, 1, false>(p, s);
        break;
    case 0:
        if (d == 64) return launch32<64, 32, 2>(p, s);
        if (d == 128) return launch32<128, 32, 2>(p, s);
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
