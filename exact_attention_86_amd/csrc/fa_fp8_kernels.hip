// fa_fp8_kernels.hip -- exact attention prefill forward with FP8 inputs on
// gfx950 (CDNA4).
//
// Q, K and V arrive as OCP FP8 E4M3 values with one descale factor per
// tensor; the result is the same attention (page "flash-attn 实现 prefill
// 阶段", section 问题分析) of the dequantized tensors:
//   O = softmax(scale (dq Q)(dk K)^T) (dv V)   (O in bf16, LSE in fp32).
// Both products run on the 32x32x64 FP8 matrix-core instruction.  The
// probabilities enter the second product as FP8 too, and follow the range
// trick of page "05 · kernel 工程与四代演化" (section 4.4): the row max used
// for the exponent is lowered by 8 (log2 units), so the largest probability
// of a row is 2^8 instead of 1 and small probabilities keep more of E4M3's
// narrow exponent range before they underflow.  The row sum adds the fp32
// probabilities; the result divides by it.
//
// Layout per workgroup (4 waves, 128 query rows, 64-key tiles), following the
// 16-bit kernels: scores transposed, S^T = K Q^T, so lane l holds one query
// (column l%32) and 16 keys of each 32-key block, and O^T += V^T P^T takes
// P^T straight from the score registers as the B operand.  Each lane's B
// operand holds 32 FP8 probabilities (16 keys of each of the two 32-key
// blocks); the A operand V^T must list the same keys in the same byte slots,
// which 8-byte transpose reads (ds_read_b64_tr_b8: lane s of a 16-lane group
// receives byte s%8 of the 8 bytes each of lanes 2b + s/8 addressed, for
// b = 0..7) deliver from V rows in LDS.  The exact tile max is taken every
// tile, but the exponent reference (the running max) is raised -- with the
// rescale of O and the row sum -- only when a row's tile max exceeds it by
// more than 0.75 in log2 units: any reference gives the same result up to
// rounding, no probability exceeds 2^8.75 < 448 (E4M3's largest value), the
// row max still contributes at least 2^8 to the row sum, and the O rescale
// becomes rare once the running maxima settle.  A negative exponent factor
// enters as Q with its sign bits flipped, so the tile max of the raw scores
// is the tile max of the exponents.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

// 32x32x64 product of E4M3 operands (format 0 for A and B), unit block scales
// (E8M0 value 127 = 2^0)
__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// four fp32 values -> four E4M3 bytes (round to nearest even), first value in
// the lowest byte
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d)
{
    int v = 0;
    v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, v, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    return v;
}

// 16-byte chunk swizzles for 128-byte rows (two rows per 256-byte bank line).
// K is read as 16-byte row fragments, 16 consecutive rows at one logical
// chunk: a bijection on row bits 1-3 (row bit 0 already picks the half line)
// spreads them over the 16 chunk slots.  V is read with 8-byte transpose
// reads that touch rows {0..3, 8..11} + 4g at one 16-byte chunk per 16-lane
// group and two adjacent chunks per 32 lanes: row bits 1 and 3 move chunk bits
// 1 and 2, so the four rows of each parity land in distinct chunk pairs.
__device__ __forceinline__ int swz_k8(int row) { return ((row & 2) ? 4 : 0) ^ ((row & 4) ? 1 : 0) ^ ((row & 8) ? 2 : 0); }
__device__ __forceinline__ int swz_v8(int row) { return (row & 2) | ((row >> 1) & 4); }

}  // namespace

template <bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fa_fwd_fp8(Fp8Params p)
{
    constexpr int D = 128;               // head size (bytes per FP8 row)
    constexpr int NW = 4;                // waves; wave w owns query rows [32w, 32w+32)
    constexpr int BM = 32 * NW;          // query rows per workgroup
    constexpr int BN = 64;               // keys per tile (two 32-key blocks)
    constexpr int RB = D;                // bytes per row
    constexpr int TB = BN * RB;          // bytes of one K or V tile
    constexpr int STAGE = 2 * TB;        // stage layout: K | V
    constexpr int DMA = TB / 1024 / NW;  // 1 KiB copies per wave per tensor per tile
    constexpr int NDT = D / 32;          // 32-wide d tiles of O^T
    static_assert(DMA * 1024 * NW == TB, "tile must split evenly over waves");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    int bh, item;
    if (!map_xcd_item(p.n_items, p.items_per_head, bh, item)) return;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int sq = p.sq, sk = p.sk;
    // |scale * dq * dk| * log2(e); a zero factor becomes 1e-30, which leaves
    // exp2 of every score at exactly 2^8 and keeps masked scores at -inf
    const float c = fmaxf(fabsf(p.c), 1e-30f);
    const int qsign = p.c < 0.f ? (int)0x80808080u : 0;  // negative factor: Q enters negated
    constexpr float kSlack = 0.75f;                      // log2 units: 2^(8 + 0.75) < 448
    const int mt = CAUSAL ? p.items_per_head - 1 - item : item;  // causal: heaviest tiles first
    const int q0 = mt * BM;

    const uint8_t* __restrict__ Q = (const uint8_t*)p.q + (size_t)bh * sq * D;
    const uint8_t* __restrict__ K = (const uint8_t*)p.k + (size_t)bh * sk * D;
    const uint8_t* __restrict__ V = (const uint8_t*)p.v + (size_t)bh * sk * D;
    uint16_t* __restrict__ O = (uint16_t*)p.o + (size_t)bh * sq * D;

    // ---- Q fragments: B operand of S^T = K Q^T (lane = query; k-step kk covers
    //      d = 64kk.., half-wave g holds its 32 bytes at 64kk + 32g); rows past
    //      the end read the last row and are never stored ----
    const int wq = q0 + 32 * w;
    const int qrow = wq + l32;
    i32x8_t qf[2];
    {
        const uint8_t* qp = Q + (size_t)min(qrow, sq - 1) * D + 32 * g;
        qf[0] = *(const i32x8_t*)(qp) ^ qsign;
        qf[1] = *(const i32x8_t*)(qp + 64) ^ qsign;
    }

    const int q_end = min(q0 + BM, sq);
    const int kv_end = CAUSAL ? min(q_end, sk) : sk;
    const int nkv = (kv_end + BN - 1) / BN;
    const int w_kv_end = (wq >= sq) ? 0 : (CAUSAL ? min(min(wq + 32, sq), sk) : sk);
    const int w_nkv = (w_kv_end + BN - 1) / BN;

    // ---- global -> LDS copies: copy j of wave w fills LDS chunks
    //      cc = (w*DMA + j)*64 + lane (row cc/8, physical chunk cc%8) from the
    //      swizzled logical chunk ----
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds) + w * DMA * 1024);
    uint32_t ck[DMA], cv[DMA];
#pragma unroll
    for (int j = 0; j < DMA; ++j) {
        const int cc = (w * DMA + j) * 64 + lane;
        const int row = cc >> 3, pch = cc & 7;
        ck[j] = row * RB + ((pch ^ swz_k8(row)) << 4);
        cv[j] = row * RB + ((pch ^ swz_v8(row)) << 4);
    }
    auto issue = [&](auto st_tag, int n0) {
        constexpr int ST = decltype(st_tag)::value;
        const bool full = n0 + BN <= sk;
        const void* ksrc = uniform_ptr(K + (size_t)n0 * D);
        const void* vsrc = uniform_ptr(V + (size_t)n0 * D);
        static_for<DMA>([&](auto j_tag) {
            constexpr int J = decltype(j_tag)::value;
            uint32_t ok = ck[J], ov = cv[J];
            if (!full) {  // rows past the last key re-read it (masked)
                const int cc = (w * DMA + J) * 64 + lane;
                const int row = cc >> 3, pch = cc & 7;
                const int src = min(row, sk - 1 - n0) * RB;
                ok = src + ((pch ^ swz_k8(row)) << 4);
                ov = src + ((pch ^ swz_v8(row)) << 4);
            }
            copy_1k<ST * STAGE + J * 1024>(ksrc, ok, lbase);
            copy_1k<ST * STAGE + TB + J * 1024>(vsrc, ov, lbase);
        });
    };

    // ---- per-lane LDS read offsets (bytes within a stage) ----
    //  K (A operand of S^T): row kb*32 + l32, logical chunks 4kk + 2g + e
    uint32_t rk[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 2; ++e) rk[kk][e] = l32 * RB + (((4 * kk + 2 * g + e) ^ swz_k8(l32)) << 4);
    //  V^T (A operand of O^T, transpose reads): for byte slots 8j..8j+7, lane t
    //  of its 16-lane group addresses key row 16j + 8(t/8) + 4g + (t/2)%4 at
    //  d = 32dt + 16*half + 8(t%2); lane t then receives d = 32dt + 16*half + t
    //  for those 8 keys -- the key order of the score registers
    const int t16 = lane & 15, half = (lane >> 4) & 1;
    const int vrow = 8 * (t16 >> 3) + 4 * g + ((t16 >> 1) & 3);
    uint32_t rv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        rv[dt] = TB + vrow * RB + (((2 * dt + half) ^ swz_v8(vrow)) << 4) + 8 * (t16 & 1);

    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

    auto compute = [&](auto st_tag, int n0) {
        constexpr int S = decltype(st_tag)::value;
        const uint8_t* sb = lds + S * STAGE;

        // ---- S^T = K Q^T: two 32-key blocks, two k-steps each ----
        f32x16_t s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4_t lo = *(const u32x4_t*)(sb + kb * 32 * RB + rk[kk][0]);
                const u32x4_t hi = *(const u32x4_t*)(sb + kb * 32 * RB + rk[kk][1]);
                const i32x8_t a = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kb] = mfma_fp8(a, qf[kk], s[kb]);
            }
        }

        // ---- masks (ragged keys, causal diagonal) on the raw scores, tile max ----
        const bool need_mask = (n0 + BN > sk) || (CAUSAL && n0 + BN - 1 > wq);
        if (need_mask) {
            // score r of block kb is key n0 + 32kb + 4g + off(r); it lives iff
            // key <= min(sk - 1, qrow) (causal) or sk - 1: one compare and one
            // select per score against a bound folded once per tile
            const int lim0 = (CAUSAL ? min(sk - 1, qrow) : sk - 1) - n0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + (r >> 2) * 8 + (r & 3);
                    s[kb][r] = off <= lim0 ? s[kb][r] : -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // lanes l and l+32 share a query
        const float mt = mx * c;

        // ---- online softmax: the reference m_run is raised to the exact
        //      running max only when a tile max exceeds it by more than kSlack;
        //      the exponent reference is m_run - 8, so probabilities lie in
        //      [0, 2^(8 + kSlack)] ----
        if (__builtin_amdgcn_ballot_w64(mt > m_run + kSlack)) {
            const float m_new = fmaxf(m_run, mt);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            m_run = m_new;
        }
        const float ref = m_run - 8.f;
        // B operand: byte slot i holds the probability of key block i/16, score
        // register i%16
        i32x8_t pb;
        float acc = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) {
            const int kb = q4 >> 2, r0 = (q4 & 3) * 4;
            const float p0 = fast_exp2(__builtin_fmaf(s[kb][r0], c, -ref));
            const float p1 = fast_exp2(__builtin_fmaf(s[kb][r0 + 1], c, -ref));
            const float p2 = fast_exp2(__builtin_fmaf(s[kb][r0 + 2], c, -ref));
            const float p3 = fast_exp2(__builtin_fmaf(s[kb][r0 + 3], c, -ref));
            acc += (p0 + p1) + (p2 + p3);
            pb[q4] = pack4_fp8(p0, p1, p2, p3);
        }
        l_run += acc;

        // ---- O^T += V^T P^T, one 64-key product per 32-wide d tile ----
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            i32x8_t a;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_i32x2_t*)(sb + rv[dt] + j * 16 * RB));
                a[2 * j] = x[0];
                a[2 * j + 1] = x[1];
            }
            oacc[dt] = mfma_fp8(a, pb, oacc[dt]);
        }
    };

    auto step = [&](auto st_tag, int t) {
        constexpr int S = decltype(st_tag)::value;
        wait_copies();
        __syncthreads();  // stage S is complete; every wave is done with stage S^1
        if (t + 1 < nkv) issue(Stage<S ^ 1>{}, (t + 1) * BN);
        if (t < w_nkv) compute(st_tag, t * BN);
    };

    if (nkv > 0) issue(Stage<0>{}, 0);
    int t = 0;
    for (; t + 1 < nkv; t += 2) {
        step(Stage<0>{}, t);
        step(Stage<1>{}, t + 1);
    }
    if (t < nkv) step(Stage<0>{}, t);

    // ---- epilogue: O = dv O^T / l (bf16), LSE = (m - 8 + log2 l) ln 2 ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow < sq) {
        const float inv = p.vscale / l_tot;
        uint16_t* orow = O + (size_t)qrow * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const uint32_t w0 = pack2(oacc[dt][rb * 4 + 0] * inv, oacc[dt][rb * 4 + 1] * inv, true);
                const uint32_t w1 = pack2(oacc[dt][rb * 4 + 2] * inv, oacc[dt][rb * 4 + 3] * inv, true);
                *(u32x2_t*)(orow + dt * 32 + rb * 8 + g * 4) = u32x2_t{w0, w1};
            }
        if (g == 0) p.lse[(size_t)bh * sq + qrow] = (m_run - 8.f + __log2f(l_tot)) * kLn2;
    }
}

hipError_t launch_fwd_fp8(const Fp8Params& p_in, hipStream_t s)
{
    Fp8Params p = p_in;
    p.items_per_head = (p.sq + 127) / 128;
    p.n_items = p.bh * p.items_per_head;
    const int grid = ((p.n_items + 7) / 8) * 8;
    auto kernel = p.causal ? fa_fwd_fp8<true> : fa_fwd_fp8<false>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace fa
