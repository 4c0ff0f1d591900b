// fa_kernels.h -- internal interface between the C ABI layer (fa_api.cpp) and
// the gfx950 kernels (fa_fwd_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

// Launch parameters, passed by value as the kernel argument.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int bh;          // b * h head slices
    int sq, sk;      // sequence lengths
    float c;         // |scale| * log2(e): exponent factor in log2 units
    uint32_t qsign;  // 0x80008000 (16-bit) or 1 (fp32) when scale < 0: Q enters negated
    int causal;      // 1: key j attends to query i iff j <= i
    int n_mtiles;        // query tiles per head: ceil(sq / block_m)
    int items_per_head;  // work items per head (causal: tile pairs)
    int n_items;         // bh * items_per_head
    int grid;            // workgroups launched
    int nsplit;          // split-KV parts per query tile (1: no split)
    float* ws;           // split-KV workspace: O parts [nsplit][bh][sq][d], then LSE parts [nsplit][bh][sq]
    const int* cu_q;     // varlen: sequence offsets into the packed query rows (batch + 1)
    const int* cu_k;     // varlen: sequence offsets into the packed key rows (batch + 1)
    int total_q, total_k;  // varlen: packed rows per head
    int batch;             // varlen: sequences
};

struct TileConfig {
    int block_m, block_n, waves, lds;
    int qb;    // 32-row query blocks per wave
    int kind;  // 0: one wave group; 1: two ping-pong wave groups, one workgroup per
               // work item; 2: the same kernel on a persistent grid (fa_fwd sets it);
               // 3: one wave group per half of the key tiles (two key groups)
};

// Backward launch parameters (fa_bwd).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;    // forward row log-sum-exp, natural log, [bh][sq]
    void* dq;
    void* dk;
    void* dv;
    float* dvec;         // workspace: D_i = dO_i . O_i, [bh][sq] fp32
    int bh;
    int sq, sk;
    float c;             // scale * log2(e), signed
    float scale;
    int causal;
    int items_per_head;  // set per kernel by the launcher
    int n_items;
    // variable-length batches (fa_bwd_varlen): [batch + 1] device offsets of
    // each sequence's rows within a head's packed rows, or null for the dense
    // layout.  With them bh counts (head, sequence) pairs, sq and sk are the
    // longest lengths (grid sizes only) and total_q / total_k the packed rows.
    const int32_t* cu_q;
    const int32_t* cu_k;
    int batch;
    int total_q, total_k;
};

// FP8 forward launch parameters (fa_fwd_fp8).
struct Fp8Params {
    const void* q;       // E4M3 [bh][sq][128]
    const void* k;       // E4M3 [bh][sk][128]
    const void* v;       // E4M3 [bh][sk][128]
    void* o;             // bf16 [bh][sq][128]
    float* lse;          // fp32 [bh][sq]
    int bh;
    int sq, sk;
    float c;             // scale * descale_q * descale_k * log2(e), signed
    float vscale;        // descale_v
    int causal;
    int items_per_head;  // set by the launcher
    int n_items;
};

bool tile_config(int dtype, int d, int64_t bh, int64_t sq, int64_t sk, int causal, TileConfig* tc);
hipError_t launch_fwd(int dtype, int d, const TileConfig& tc, const Params& p, hipStream_t stream);
bool tile_config_split(int dtype, int d, TileConfig* tc);
// mode 0: the 4-wave kernel; 1: with two key groups (d <= 128); 2: the
// ping-pong kernel (d = 128, h a multiple of 8, at most 64 sequences; the grid covers
// h * batch * (items of the longest sequence), cost-ordered, the rest exit)
hipError_t launch_fwd_varlen(int dtype, int d, const Params& p, int mode, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream);
bool bwd_supported(int dtype, int d);
hipError_t launch_bwd(int dtype, int d, const BwdParams& p, hipStream_t stream);
hipError_t launch_fwd_split(int dtype, int d, const TileConfig& tc, const Params& p, hipStream_t stream);

// Library-owned device scratch of kNoallocScratchBytes for callers that cannot
// allocate: the current device's address of it (looked up once per device).
constexpr size_t kNoallocScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa
