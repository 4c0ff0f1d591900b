/*
 * fa.h -- C ABI of the exact-attention prefill forward library for AMD
 * Instinct MI355X (gfx950).
 *
 * The one operation: for every batch b and head h independently,
 *
 *     O   = softmax(scale * Q K^T) V                (rows of the softmax over keys)
 *     LSE = log of the softmax denominator, per query row, natural-log units
 *
 * Page "flash-attn 实现 prefill 阶段", section 问题分析, states the formula
 * and the [batch, heads, seq_len, head_dim] layout; page "flash.cu"
 * (forward_kernel and forward) places the scale on the dot product before
 * the exponential and keeps the running row max m and row sum l that make
 * LSE = m + ln l.  Page "05 · kernel 工程与四代演化" (sections 2.1 and 6.1)
 * names the causal variant and the forward entry point this library mirrors.
 *
 * Everything is asynchronous on the caller's HIP stream; the library keeps no
 * state between calls and allocates no device memory (the one exception is
 * the fixed per-GPU scratch array behind fa_fwd_split_noalloc, which exists
 * from the library's load on).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

/* element types of q, k, v and o (lse is always fp32) */
enum fa_dtype { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 };

/* return codes */
enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* NULL pointer, size <= 0, non-finite scale,
                               causal not 0/1, outputs overlapping inputs  */
    FA_ERR_UNSUPPORTED = 2, /* unknown dtype, head size not served         */
    FA_ERR_MISALIGNED = 3,  /* q, k, v, o not 16-byte aligned; lse not 4   */
    FA_ERR_TOO_LARGE = 4,   /* a per-head slice or the grid exceeds 2^31-1 */
    FA_ERR_HIP = 5          /* the HIP runtime refused the launch          */
};

/*
 * fa_fwd -- exact attention prefill forward.
 *
 *   q      device pointer, [b, h, sq, d] contiguous row-major, dtype
 *   k, v   device pointers, [b, h, sk, d] contiguous row-major, dtype
 *   o      device pointer, [b, h, sq, d] contiguous row-major, dtype (output)
 *   lse    device pointer, [b, h, sq] fp32 (output)
 *   b, h   batch size and number of heads (>= 1)
 *   sq, sk query and key sequence lengths (>= 1; need not be multiples of
 *          any tile size)
 *   d      head size: 64, 128 or 256 for FA_F16/FA_BF16; 64 or 128 for FA_F32
 *   scale  multiplies q.k before the softmax (callers usually pass 1/sqrt(d));
 *          any finite value
 *   causal 0: every key attends; 1: query i attends to keys j <= i
 *          (top-left alignment; the same as bottom-right when sq == sk)
 *   dtype  FA_F32, FA_F16 or FA_BF16, shared by q, k, v and o
 *   stream hipStream_t to enqueue on (NULL = the default stream)
 *
 * Numerics: dot products and the softmax run in fp32 with fp32 accumulation;
 * for FA_F16/FA_BF16 the probabilities are rounded to the input type before
 * they multiply V (the matrix units take 16-bit operands), while the row sum
 * uses the unrounded fp32 values; for FA_F32 they stay fp32.  O is rounded to
 * the output type with round-to-nearest-even.
 *
 * Ownership: the caller allocates and owns every buffer; o and lse must not
 * overlap q, k, v or each other.  All argument checks happen on the host
 * before any HIP call, so a failing call enqueues nothing.  The call returns
 * after the launch is enqueued; faults during execution surface at the
 * caller's next synchronisation.  Results are bitwise reproducible for a
 * fixed device, shape and dtype (no atomics).
 *
 * Returns FA_OK or one of the fa_status codes; fa_last_error() then holds a
 * message.
 */
FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o,
                  float* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                  int64_t d, float scale, int causal, int dtype, void* stream);

/*
 * fa_query_config -- the tiling fa_fwd uses for a problem (dtype, d, causal,
 * b, h, sq, sk); the choice of kernel may depend on the sizes.
 *   block_m  query rows per workgroup tile
 *   block_n  keys per inner step (one K/V tile through LDS)
 *   waves    wavefronts per workgroup (64 lanes each; 8 with block_m 128
 *            means two groups of 4 waves that split the key tiles)
 *   lds      LDS bytes per workgroup
 * Any output pointer may be NULL.  Returns FA_OK, FA_ERR_INVALID_ARG (a size
 * below 1, causal not 0/1) or FA_ERR_UNSUPPORTED.  Host only; no HIP call.
 * One function answers for both the launcher and its callers (tests, the
 * benchmark), so the two cannot drift apart -- page "05 · kernel
 * 工程与四代演化", section 7, warns of block-size tables kept in sync by hand
 * in two places.
 */
FA_API int fa_query_config(int dtype, int64_t d, int causal, int64_t b, int64_t h,
                           int64_t sq, int64_t sk, int* block_m, int* block_n,
                           int* waves, int* lds);

/*
 * fa_query_launch -- the grid fa_fwd launches for a problem on the current
 * device (page "05 · kernel 工程与四代演化", section 4.3, describes the
 * persistent tile scheduler: about one workgroup per compute unit claiming
 * work items).
 *   grid        workgroups launched
 *   persistent  1: the 8-wave kernel runs on a persistent grid of about one
 *               workgroup per CU that loops over single query tiles in cost
 *               order (chosen for causal problems whose equal-cost pairs of
 *               query tiles would leave the last round of workgroups mostly
 *               empty); 0: one workgroup per work item (a causal pair of
 *               query tiles, or one tile)
 * Any output pointer may be NULL.  Asks the HIP runtime for the current
 * device's compute-unit count (no launch, no allocation); without a device it
 * reports the per-item grid.  Returns FA_OK, FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED or FA_ERR_TOO_LARGE as fa_fwd would.
 */
FA_API int fa_query_launch(int dtype, int64_t d, int causal, int64_t b, int64_t h,
                           int64_t sq, int64_t sk, int* grid, int* persistent);

/*
 * fa_fwd_split -- the same forward with each query tile's key range cut into
 * nsplit near-equal parts that run as separate work items (split-KV), for
 * problems with too few query tiles to fill the GPU (short prefills, few
 * heads, decode-shaped sq << sk).  Page "05 · kernel 工程与四代演化", section
 * 2.1, lists the split-KV forward as its own kernel class.  Each part writes
 * its partial result (O_p normalised by its own row sum, LSE_p) in fp32 to the
 * workspace; a second kernel on the same stream merges them:
 *
 *     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
 *
 * (a part that sees no key of a row contributes LSE_p = -inf, weight 0).  O
 * and LSE equal fa_fwd's up to rounding.
 *
 *   q ... dtype  as fa_fwd; dtype FA_F16 or FA_BF16, d = 64, 128 or 256
 *   nsplit       parts per query tile, 1..FA_MAX_SPLIT; nsplit = 1 is exactly
 *                fa_fwd (the workspace is not used and may be NULL)
 *   workspace    device buffer of at least fa_split_workspace_bytes() bytes,
 *                16-byte aligned, owned by the caller, not overlapping q, k,
 *                v, o or lse; its contents on entry do not matter and are
 *                scratch afterwards.  Calls that share a workspace must be
 *                ordered (same stream, or synchronised).
 *   workspace_bytes  its size in bytes
 *
 * Returns FA_OK or an fa_status code (FA_ERR_UNSUPPORTED for fp32 or another
 * head size; FA_ERR_INVALID_ARG for nsplit out of range or a missing, small
 * or overlapping workspace; FA_ERR_MISALIGNED for a misaligned workspace).
 */
#define FA_MAX_SPLIT 64
FA_API int fa_fwd_split(const void* q, const void* k, const void* v, void* o,
                        float* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                        int64_t d, float scale, int causal, int dtype, int nsplit,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_split_noalloc -- fa_fwd_split for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the partial results go to a scratch array the
 * library owns instead of a caller workspace.  Same arguments as
 * fa_fwd_split without workspace and workspace_bytes; same results, bit for
 * bit (the same kernels run).
 *
 * The scratch is a FA_NOALLOC_SCRATCH_BYTES device array, one copy per GPU,
 * held from the library's load until the process ends; its device address is
 * looked up once per device, on the first call with that device current.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine) and needs no clearing of the scratch: every partial result is
 * written before it is read.  Every call on one GPU shares that GPU's scratch,
 * so calls that overlap in time on one GPU (different streams, or different
 * threads without ordering) race and give wrong results: order them.
 *
 * Returns FA_ERR_TOO_LARGE when nsplit * b * h * sq * (d + 1) * 4 exceeds
 * FA_NOALLOC_SCRATCH_BYTES (checked before any HIP call), FA_ERR_HIP when the
 * scratch address cannot be obtained, otherwise as fa_fwd_split.  nsplit = 1
 * is exactly fa_fwd.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
FA_API int fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o,
                                float* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                                int64_t d, float scale, int causal, int dtype, int nsplit,
                                void* stream);

/* fa_split_workspace_bytes -- workspace size fa_fwd_split needs:
 * nsplit * b * h * sq * (d + 1) * 4 bytes (partial O and LSE in fp32); 0 for
 * nsplit = 1 and for invalid arguments.  Host only. */
FA_API size_t fa_split_workspace_bytes(int64_t b, int64_t h, int64_t sq, int64_t d, int nsplit);

/*
 * fa_fwd_varlen -- the same forward over a batch of packed sequences of
 * different lengths (page "05 · kernel 工程与四代演化", section 6.1, lists
 * the variable-length forward among the exported entry points).  Each head
 * stores its sequences back to back along the row axis:
 *
 *   q, o   [h, total_q, d] contiguous, dtype; sequence i owns query rows
 *          cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 of every head
 *   k, v   [h, total_k, d] contiguous, dtype; sequence i owns key rows
 *          cu_seqlens_k[i] .. cu_seqlens_k[i+1]-1
 *   lse    [h, total_q] fp32
 *
 * and every sequence is an independent attention problem (queries of
 * sequence i attend only to keys of sequence i; causal: local key j attends
 * to local query r iff j <= r, top-left as in fa_fwd).
 *
 *   cu_seqlens_q, cu_seqlens_k  device int32 arrays of batch + 1 offsets,
 *          starting at 0, non-decreasing, ending at total_q / total_k
 *   batch  number of sequences (>= 1)
 *   max_sq an upper bound of the query lengths (sets the grid; rows of a
 *          sequence past max_sq are not computed)
 *   d      64, 128 or 256; dtype FA_F16 or FA_BF16
 *
 * A sequence with no query rows is skipped; every sequence with query rows
 * needs at least one key (otherwise its rows are left unwritten).  The offset
 * arrays live on the device, so their contents are not checked on the host;
 * the kernel clamps them into [0, total] so malformed offsets cannot address
 * outside the buffers (the results are then unspecified).  Returns FA_OK or an
 * fa_status code as fa_fwd.
 */
FA_API int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                         float* lse, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int64_t batch, int64_t h,
                         int64_t total_q, int64_t total_k, int64_t max_sq,
                         int64_t d, float scale, int causal, int dtype,
                         void* stream);

/*
 * fa_bwd -- gradients of fa_fwd: given dout = dL/dO, writes dq = dL/dQ,
 * dk = dL/dK and dv = dL/dV for O = softmax(scale Q K^T) V (page "flash-attn
 * 实现 prefill 阶段", section 问题分析, differentiated; page "05 · kernel
 * 工程与四代演化", section 2.1, lists the backward as its own kernel class and
 * section 6.1 its export).  The probabilities are recomputed from the row LSE
 * the forward returned, so no sq x sk matrix is stored:
 *
 *     P_ij  = exp(scale q_i.k_j - LSE_i)      (0 where causal masks j > i)
 *     D_i   = dout_i . o_i
 *     dS_ij = P_ij (dout_i . v_j - D_i)
 *     dv_j  = sum_i P_ij dout_i
 *     dk_j  = scale sum_i dS_ij q_i
 *     dq_i  = scale sum_j dS_ij k_j
 *
 *   q, o, dout, dq   [b, h, sq, d] contiguous, dtype
 *   k, v, dk, dv     [b, h, sk, d] contiguous, dtype
 *   lse              [b, h, sq] fp32, as fa_fwd wrote it for these q, k, v,
 *                    scale and causal (o likewise)
 *   workspace        device buffer of at least fa_bwd_workspace_bytes()
 *                    bytes (holds D in fp32), 16-byte aligned, owned by the
 *                    caller; contents on entry do not matter.  Calls that
 *                    share a workspace must be ordered (same stream).
 *   workspace_bytes  its size in bytes
 *   d                64, 128 or 256;  dtype FA_F16 or FA_BF16
 *   scale, causal    as passed to fa_fwd
 *   stream           hipStream_t; three kernels are enqueued on it
 *
 * dq, dk, dv and the workspace must not overlap the inputs or each other.
 * P and dS are rounded to dtype before they enter the matrix cores (fp32
 * accumulation).  Deterministic: no atomics, the same inputs give the same
 * bits.  Returns FA_OK or an fa_status code as fa_fwd (FA_ERR_UNSUPPORTED for
 * fp32 or d other than 64, 128 and 256; FA_ERR_INVALID_ARG for a missing,
 * small or overlapping workspace).
 */
FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes, int64_t b, int64_t h,
                  int64_t sq, int64_t sk, int64_t d, float scale, int causal,
                  int dtype, void* stream);

/* fa_bwd_workspace_bytes -- workspace size fa_bwd needs: b * h * sq * 4
 * bytes; 0 for invalid arguments.  Host only. */
FA_API size_t fa_bwd_workspace_bytes(int64_t b, int64_t h, int64_t sq);

/*
 * fa_bwd_varlen -- fa_bwd over a batch of packed sequences of different
 * lengths, the gradients of fa_fwd_varlen (page "05 · kernel 工程与四代演化",
 * section 6.1, lists the variable-length backward among the exported entry
 * points).  Layout as fa_fwd_varlen, per head the sequences back to back:
 *
 *   q, o, dout, dq   [h, total_q, d] contiguous, dtype; sequence i owns rows
 *                    cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 of every head
 *   k, v, dk, dv     [h, total_k, d] contiguous, dtype; sequence i owns rows
 *                    cu_seqlens_k[i] .. cu_seqlens_k[i+1]-1
 *   lse              [h, total_q] fp32, as fa_fwd_varlen wrote it (o too)
 *   workspace        at least fa_bwd_workspace_bytes(1, h, total_q) bytes,
 *                    16-byte aligned, owned by the caller (holds D)
 *   cu_seqlens_q, cu_seqlens_k  device int32 arrays of batch + 1 offsets,
 *                    starting at 0, non-decreasing, ending at total_q /
 *                    total_k
 *   max_sq, max_sk   upper bounds of the query and key lengths (set the
 *                    grids; rows and keys of a sequence past them are not
 *                    computed)
 *   d                64, 128 or 256;  dtype FA_F16 or FA_BF16
 *
 * Each sequence's gradients are those of fa_bwd for that sequence alone
 * (causal: local key j attends to local query r iff j <= r).  The keys of a
 * sequence with no query rows get dk = dv = 0; the rows of a sequence with no
 * keys get dq = 0 (fa_fwd_varlen leaves their o and lse unwritten, so pass
 * any finite values there).  The offset arrays live on the device and are
 * not checked on the host; the kernels clamp them into [0, total] so
 * malformed offsets cannot address outside the buffers (the results are then
 * unspecified).  Same rounding, determinism, overlap rules and status codes
 * as fa_bwd.
 */
FA_API int fa_bwd_varlen(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int64_t batch, int64_t h,
                         int64_t total_q, int64_t total_k, int64_t max_sq,
                         int64_t max_sk, int64_t d, float scale, int causal,
                         int dtype, void* stream);

/*
 * fa_fwd_fp8 -- the forward with FP8 inputs (page "05 · kernel 工程与四代演化",
 * section 4.4, describes the FP8 forward and its exponent-range trick).
 * Computes the attention of the dequantized tensors
 *
 *     O   = softmax(scale (descale_q Q)(descale_k K)^T) (descale_v V)
 *     LSE = ln sum_j exp(scale descale_q descale_k q_i.k_j)
 *
 *   q          [b, h, sq, d] contiguous, OCP FP8 E4M3 (1 byte per element)
 *   k, v       [b, h, sk, d] contiguous, E4M3
 *   o          [b, h, sq, d] contiguous, bf16 (output)
 *   lse        [b, h, sq] fp32 (output)
 *   d          128
 *   scale      finite; descale_q, descale_k, descale_v: finite per-tensor
 *              factors that map the stored E4M3 values to the real ones;
 *              scale * descale_q * descale_k * log2(e) must be finite in fp32
 *   causal     0 or 1, as fa_fwd
 *
 * Both products run on FP8 matrix cores; the probabilities are rounded to
 * E4M3 before the second product, the row sum uses their fp32 values.  The
 * exponent reference is a running reference max minus 8, where the reference
 * never exceeds the row max seen so far and trails it by at most 0.75 (log2
 * units): the row max contributes at least 2^8 to the row sum and no
 * probability exceeds 2^8.75 (E4M3's largest value is 448).
 * Returns FA_OK or an fa_status code as fa_fwd (FA_ERR_UNSUPPORTED for
 * d != 128).
 */
FA_API int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o,
                      float* lse, int64_t b, int64_t h, int64_t sq, int64_t sk,
                      int64_t d, float scale, float descale_q, float descale_k,
                      float descale_v, int causal, void* stream);

/*
 * fa_clock_probe -- measurement aid, not part of the attention path: reads
 * the shader clock the GPU runs at.  One wave reads the shader-clock counter
 * and the constant 100 MHz real-time counter, spins for `ticks` real-time
 * ticks (10 ns each), and writes two values to `out` (device pointer, 2
 * uint64, 8-byte aligned, caller-owned): out[0] = shader-clock cycles and
 * out[1] = real-time ticks elapsed, so the clock is out[0] / out[1] * 100 MHz.
 * Enqueued on `stream` right behind attention launches, it sees the clock the
 * power manager chose for them.  The matrix-core peak is 4096 FLOP per clock
 * per compute unit at 16 bits, so this clock turns a throughput into a
 * fraction of the peak at the clock actually seen.
 * Returns FA_OK, FA_ERR_INVALID_ARG (NULL, ticks outside [1, 10^7]),
 * FA_ERR_MISALIGNED or FA_ERR_HIP.
 */
FA_API int fa_clock_probe(unsigned long long* out, int64_t ticks, void* stream);

/* fa_last_error -- message of the last failing call on this host thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
FA_API const char* fa_last_error(void);

/* fa_version -- library version, major*10000 + minor*100 + patch. */
FA_API int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
