// fa_api.cpp -- the C ABI of include/fa.h: argument checks, tiling, launch.
//
// Every check runs on the host before any HIP call, so an invalid call
// enqueues nothing and the checks are testable on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

thread_local char g_err[256] = "";

int fail(int code, const char* msg)
{
    snprintf(g_err, sizeof g_err, "%s", msg);
    return code;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// compute units of the current device, looked up once per device (0 if the
// runtime cannot say)
int device_cus()
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static int cus[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!cus[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = v;
    }
    return cus[dev];
}

// whether the ping-pong kernel (one workgroup per CU) runs on a persistent
// grid that loops over single query tiles in cost order, instead of one
// workgroup per (causal: pair of) query tile(s).  Causal pairs all cost the
// same, so the per-item grid drains in ceil(pairs / CUs) rounds; when that
// leaves the last round less than ~75 % full (pairs < 95 % of rounds x CUs)
// the persistent grid's cost-ordered single tiles fill it.  Otherwise the
// per-item grid wins: its head-major order shares each head's K/V among 8
// concurrent workgroups of one XCD (measured on one MI355X: persistent +8.7 %
// at 2.5 rounds of pairs, +1.9 % at 4.5, -3 % at exactly 4).  Without the
// mask every unit costs the same and the hardware's dispatch already balances.
bool use_persistent(int64_t bh, int64_t n_mtiles, int causal, int ncu)
{
    if (!causal || ncu <= 0) return false;
    const int64_t pairs = bh * ((n_mtiles + 1) / 2);
    const int64_t rounds = (pairs + ncu - 1) / ncu;
    return 20 * pairs < 19 * rounds * ncu;
}

// the launch fa_fwd makes for a problem: grid size, persistent or not
struct Launch {
    fa::TileConfig tc;
    int64_t n_mtiles, items_per_head, n_items, grid;
};

// the per-item launch (host arithmetic only, no HIP call)
bool plan_launch(int dtype, int64_t d, int causal, int64_t b, int64_t h, int64_t sq, int64_t sk, Launch* L)
{
    if (!fa::tile_config(dtype, (int)d, b * h, sq, sk, causal, &L->tc)) return false;
    // causal work items pair query tile nQ-1-i with tile i (equal cost)
    L->n_mtiles = (sq + L->tc.block_m - 1) / L->tc.block_m;
    L->items_per_head = causal ? (L->n_mtiles + 1) / 2 : L->n_mtiles;
    L->n_items = b * h * L->items_per_head;
    L->grid = ((L->n_items + 7) / 8) * 8;
    return true;
}

bool launch_too_large(const Launch& L, int64_t bh)
{
    return L.n_items > INT32_MAX - 8 || bh * L.n_mtiles > INT32_MAX - 8;
}

// switch the ping-pong kernel to its persistent grid where use_persistent
// says so (asks the runtime for the device's CU count)
void maybe_persist(Launch* L, int64_t bh, int causal)
{
    if (L->tc.kind != 1) return;
    const int ncu = device_cus() / 8 * 8;  // whole XCDs
    if (ncu >= 8 && use_persistent(bh, L->n_mtiles, causal, ncu)) {
        // one unit per query tile; about one workgroup per CU
        L->tc.kind = 2;
        L->items_per_head = L->n_mtiles;
        L->n_items = bh * L->n_mtiles;
        L->grid = std::min<int64_t>(((L->n_items + 7) / 8) * 8, ncu);
    }
}

}  // namespace

extern "C" {

FA_API const char* fa_last_error(void) { return g_err; }

FA_API int fa_version(void) { return 500; /* 0.5.0: adds fa_fwd_fp8 */ }

FA_API int fa_query_config(int dtype, int64_t d, int causal, int64_t b, int64_t h, int64_t sq,
                           int64_t sk, int* block_m, int* block_n, int* waves, int* lds)
{
    (void)sk;
    if (b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || (causal != 0 && causal != 1))
        return fail(FA_ERR_INVALID_ARG, "fa_query_config: sizes must be >= 1, causal 0 or 1");
    fa::TileConfig tc;
    if (d <= 0 || d > 4096 || !fa::tile_config(dtype, (int)d, b * h, sq, sk, causal, &tc))
        return fail(FA_ERR_UNSUPPORTED, "fa_query_config: dtype/head size not served");
    if (block_m) *block_m = tc.block_m;
    if (block_n) *block_n = tc.block_n;
    if (waves) *waves = tc.waves;
    if (lds) *lds = tc.lds;
    g_err[0] = 0;
    return FA_OK;
}

FA_API int fa_query_launch(int dtype, int64_t d, int causal, int64_t b, int64_t h, int64_t sq,
                           int64_t sk, int* grid, int* persistent)
{
    if (b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || (causal != 0 && causal != 1))
        return fail(FA_ERR_INVALID_ARG, "fa_query_launch: sizes must be >= 1, causal 0 or 1");
    if (b > INT32_MAX || h > INT32_MAX || sq > INT32_MAX || b * h > INT32_MAX)
        return fail(FA_ERR_TOO_LARGE, "fa_query_launch: too many tiles for one launch");
    Launch L;
    if (d <= 0 || d > 4096 || !plan_launch(dtype, d, causal, b, h, sq, sk, &L))
        return fail(FA_ERR_UNSUPPORTED, "fa_query_launch: dtype/head size not served");
    if (launch_too_large(L, b * h))
        return fail(FA_ERR_TOO_LARGE, "fa_query_launch: too many tiles for one launch");
    maybe_persist(&L, b * h, causal);
    if (grid) *grid = (int)L.grid;
    if (persistent) *persistent = L.tc.kind == 2;
    g_err[0] = 0;
    return FA_OK;
}

// checks shared by fa_fwd and fa_fwd_split; fills the launch parameters
// except the schedule fields.  `who` prefixes the messages.
static int check_common(const char* who, const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale, int causal,
                        int dtype, fa::Params* p)
{
    char msg[160];
    auto bad = [&](int code, const char* what) {
        snprintf(msg, sizeof msg, "%s: %s", who, what);
        return fail(code, msg);
    };
    if (!q || !k || !v || !o || !lse) return bad(FA_ERR_INVALID_ARG, "NULL pointer");
    if (b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || d <= 0)
        return bad(FA_ERR_INVALID_ARG, "b, h, sq, sk and d must be >= 1");
    if (!isfinite(scale)) return bad(FA_ERR_INVALID_ARG, "scale must be finite");
    if (causal != 0 && causal != 1) return bad(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return bad(FA_ERR_UNSUPPORTED, "unknown dtype");
    if (d > 4096) return bad(FA_ERR_UNSUPPORTED, "head size not served for this dtype");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
        return bad(FA_ERR_MISALIGNED, "q, k, v, o must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return bad(FA_ERR_MISALIGNED, "lse must be 4-byte aligned");
    // per-head slices use 32-bit offsets; head counts and the grid are int32
    const int64_t lim = INT32_MAX;
    if (sq * d > lim || sk * d > lim || b * h > lim || b > lim || h > lim)
        return bad(FA_ERR_TOO_LARGE, "a per-head slice exceeds 2^31-1 elements");
    const size_t esz = dtype == FA_F32 ? 4 : 2;
    const size_t nq = (size_t)(b * h * sq * d) * esz, nk = (size_t)(b * h * sk * d) * esz;
    const size_t nl = (size_t)(b * h * sq) * 4;
    if (overlap(o, nq, q, nq) || overlap(o, nq, k, nk) || overlap(o, nq, v, nk) ||
        overlap(lse, nl, q, nq) || overlap(lse, nl, k, nk) || overlap(lse, nl, v, nk) ||
        overlap(lse, nl, o, nq))
        return bad(FA_ERR_INVALID_ARG, "o and lse must not overlap the inputs or each other");

    p->q = q;
    p->k = k;
    p->v = v;
    p->o = o;
    p->lse = lse;
    p->bh = (int)(b * h);
    p->sq = (int)sq;
    p->sk = (int)sk;
    // exponent factor in log2 units; a zero scale keeps a tiny positive factor
    // so masked (-inf) scores still map to exp2(-inf) = 0 and every live score
    // gives exp2(0 +- 1e-30 |s|) = 1 exactly in fp32
    const float a = fabsf(scale);
    p->c = a > 0.f ? (float)((double)a * 1.4426950408889634) : 1e-30f;
    p->qsign = scale < 0.f ? (dtype == FA_F32 ? 1u : 0x80008000u) : 0u;
    p->causal = causal;
    p->nsplit = 1;
    p->ws = nullptr;
    p->cu_q = p->cu_k = nullptr;
    p->total_q = p->total_k = 0;
    return FA_OK;
}

// nsplit * b * h * sq * (d + 1) * 4, saturated at SIZE_MAX (callers have
// bounded every factor to 31 bits, but their product can exceed 64 bits)
static size_t split_ws_bytes(int64_t b, int64_t h, int64_t sq, int64_t d, int64_t nsplit)
{
    unsigned __int128 n = (unsigned __int128)nsplit * (unsigned __int128)(b * h);
    n *= (unsigned __int128)sq;
    n *= (unsigned __int128)(d + 1) * 4u;
    return n > (unsigned __int128)SIZE_MAX ? SIZE_MAX : (size_t)n;
}

FA_API int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale,
                  int causal, int dtype, void* stream)
{
    fa::Params p;
    const int rc = check_common("fa_fwd", q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, &p);
    if (rc != FA_OK) return rc;
    Launch L;
    if (!plan_launch(dtype, d, causal, b, h, sq, sk, &L))
        return fail(FA_ERR_UNSUPPORTED, "fa_fwd: head size not served for this dtype");
    if (launch_too_large(L, b * h)) return fail(FA_ERR_TOO_LARGE, "fa_fwd: too many tiles for one launch");
    maybe_persist(&L, b * h, causal);  // every argument is valid: the runtime may be asked now
    const fa::TileConfig tc = L.tc;
    p.n_mtiles = (int)L.n_mtiles;
    p.items_per_head = (int)L.items_per_head;
    p.n_items = (int)L.n_items;
    p.grid = (int)L.grid;

    hipError_t e = fa::launch_fwd(dtype, (int)d, tc, p, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "fa_fwd: launch failed: %s", hipGetErrorString(e));
        return FA_ERR_HIP;
    }
    g_err[0] = 0;
    return FA_OK;
}

FA_API size_t fa_split_workspace_bytes(int64_t b, int64_t h, int64_t sq, int64_t d, int nsplit)
{
    if (b <= 0 || h <= 0 || sq <= 0 || d <= 0 || nsplit < 1 || nsplit > FA_MAX_SPLIT) return 0;
    if (nsplit == 1) return 0;
    return split_ws_bytes(b, h, sq, d, nsplit);
}

// the split-KV forward with its partial results in `workspace` (the caller's
// buffer, or the library's scratch when `noalloc`); `who` prefixes messages
static int fwd_split(const char* who, const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale, int causal,
                     int dtype, int nsplit, void* workspace, size_t workspace_bytes, bool noalloc,
                     void* stream)
{
    char msg[192];
    auto bad = [&](int code, const char* what) {
        snprintf(msg, sizeof msg, "%s: %s", who, what);
        return fail(code, msg);
    };
    if (nsplit < 1 || nsplit > FA_MAX_SPLIT) return bad(FA_ERR_INVALID_ARG, "nsplit must be in [1, 64]");
    if (nsplit == 1)  // one part: exactly fa_fwd; no workspace is touched
        return fa_fwd(q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, stream);
    fa::Params p;
    const int rc = check_common(who, q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, &p);
    if (rc != FA_OK) return rc;
    fa::TileConfig tc;
    if (!fa::tile_config_split(dtype, (int)d, &tc))
        return bad(FA_ERR_UNSUPPORTED, "fp16/bf16 with d = 64, 128 or 256 only");
    const size_t need = split_ws_bytes(b, h, sq, d, nsplit);
    if (noalloc) {
        if (need > FA_NOALLOC_SCRATCH_BYTES) {
            snprintf(msg, sizeof msg, "%s: nsplit*b*h*sq*(d+1)*4 = %zu bytes exceeds the %zu-byte library scratch",
                     who, need, (size_t)FA_NOALLOC_SCRATCH_BYTES);
            return fail(FA_ERR_TOO_LARGE, msg);
        }
    } else {
        if (!workspace) return bad(FA_ERR_INVALID_ARG, "NULL workspace");
        if ((uintptr_t)workspace & 15u) return bad(FA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
        if (workspace_bytes < need)
            return bad(FA_ERR_INVALID_ARG, "workspace smaller than fa_split_workspace_bytes()");
        const size_t nq = (size_t)(b * h * sq * d) * 2, nk = (size_t)(b * h * sk * d) * 2;
        const size_t nl = (size_t)(b * h * sq) * 4;
        if (overlap(workspace, need, q, nq) || overlap(workspace, need, k, nk) ||
            overlap(workspace, need, v, nk) || overlap(workspace, need, o, nq) ||
            overlap(workspace, need, lse, nl))
            return bad(FA_ERR_INVALID_ARG, "workspace must not overlap the inputs or outputs");
    }
    const int64_t n_mtiles = (sq + tc.block_m - 1) / tc.block_m;
    const int64_t items_per_head = n_mtiles * nsplit;
    const int64_t n_items = b * h * items_per_head;
    const int64_t merge_blocks = (b * h * sq * (d / 8) + 255) / 256;
    if (n_items > INT32_MAX - 8 || items_per_head > INT32_MAX || merge_blocks > INT32_MAX)
        return bad(FA_ERR_TOO_LARGE, "too many tiles for one launch");
    hipError_t e = hipSuccess;
    if (noalloc) {
        // every argument is valid: only now touch the runtime
        e = fa::noalloc_scratch(&workspace);
        if (e != hipSuccess) {
            snprintf(msg, sizeof msg, "%s: library scratch unavailable: %s", who, hipGetErrorString(e));
            return fail(FA_ERR_HIP, msg);
        }
    }
    p.n_mtiles = (int)n_mtiles;
    p.items_per_head = (int)items_per_head;
    p.n_items = (int)n_items;
    p.grid = (int)(((n_items + 7) / 8) * 8);
    p.nsplit = nsplit;
    p.ws = (float*)workspace;

    e = fa::launch_fwd_split(dtype, (int)d, tc, p, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(msg, sizeof msg, "%s: launch failed: %s", who, hipGetErrorString(e));
        return fail(FA_ERR_HIP, msg);
    }
    g_err[0] = 0;
    return FA_OK;
}

FA_API int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale,
                        int causal, int dtype, int nsplit, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    return fwd_split("fa_fwd_split", q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype, nsplit,
                     workspace, workspace_bytes, false, stream);
}

FA_API int fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale,
                                int causal, int dtype, int nsplit, void* stream)
{
    return fwd_split("fa_fwd_split_noalloc", q, k, v, o, lse, b, h, sq, sk, d, scale, causal, dtype,
                     nsplit, nullptr, 0, true, stream);
}

FA_API int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t batch,
                         int64_t h, int64_t total_q, int64_t total_k, int64_t max_sq, int64_t d,
                         float scale, int causal, int dtype, void* stream)
{
    if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: NULL pointer");
    if (batch <= 0 || h <= 0 || total_q <= 0 || total_k <= 0 || max_sq <= 0 || d <= 0)
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: batch, h, total_q, total_k, max_sq and d must be >= 1");
    if (max_sq > total_q) return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: max_sq exceeds total_q");
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: causal must be 0 or 1");
    fa::TileConfig tc;
    if (d > 4096 || !fa::tile_config_split(dtype, (int)d, &tc))
        return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: fp16/bf16 with d = 64, 128 or 256 only");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
        return fail(FA_ERR_MISALIGNED, "fa_fwd_varlen: q, k, v, o must be 16-byte aligned");
    if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u)
        return fail(FA_ERR_MISALIGNED, "fa_fwd_varlen: lse and the offset arrays must be 4-byte aligned");
    const int64_t lim = INT32_MAX;
    if (total_q * d > lim || total_k * d > lim || h > lim || batch > lim - 1)
        return fail(FA_ERR_TOO_LARGE, "fa_fwd_varlen: a per-head slice exceeds 2^31-1 elements");
    const size_t nq = (size_t)(h * total_q * d) * 2, nk = (size_t)(h * total_k * d) * 2;
    const size_t nl = (size_t)(h * total_q) * 4;
    if (overlap(o, nq, q, nq) || overlap(o, nq, k, nk) || overlap(o, nq, v, nk) ||
        overlap(lse, nl, q, nq) || overlap(lse, nl, k, nk) || overlap(lse, nl, v, nk) ||
        overlap(lse, nl, o, nq))
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_varlen: o and lse must not overlap the inputs or each other");
    const int64_t tiles = (max_sq + tc.block_m - 1) / tc.block_m;
    const int64_t items_per_head = batch * tiles;
    const int64_t n_items = h * items_per_head;
    if (items_per_head > lim || n_items > lim - 8)
        return fail(FA_ERR_TOO_LARGE, "fa_fwd_varlen: too many tiles for one launch");

    fa::Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.bh = (int)h;
    p.sq = (int)max_sq;
    p.sk = (int)total_k;
    const float a = fabsf(scale);
    p.c = a > 0.f ? (float)((double)a * 1.4426950408889634) : 1e-30f;
    p.qsign = scale < 0.f ? 0x80008000u : 0u;
    p.causal = causal;
    p.n_mtiles = (int)tiles;
    p.items_per_head = (int)items_per_head;
    p.n_items = (int)n_items;
    p.grid = (int)(((n_items + 7) / 8) * 8);
    p.nsplit = 1;
    p.ws = nullptr;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = (int)total_q;
    p.total_k = (int)total_k;

    // fewer tiles with rows than CUs (at most ceil(total_q / block_m) + batch
    // per head; the grid's other items return at once) and at least 4 key
    // tiles per sequence on average: two key groups per tile (8 waves), as
    // fa_fwd does
    const int64_t live_items = h * ((total_q + tc.block_m - 1) / tc.block_m + batch);
    int mode = (d <= 128 && live_items < 256 && total_k >= 4 * (int64_t)tc.block_n * batch) ? 1 : 0;
    // d = 128, h a multiple of 8 (equal work per XCD), at most 64 sequences
    // of 1024 query rows or more on average, and at least one ping-pong work
    // item per CU (counted on whole 256-row tiles, two per causal pair), as
    // fa_fwd: the 8-wave ping-pong kernel, one work item per (head, sequence,
    // causal pair or query tile), ordered in the kernel; the grid covers the
    // longest sequence's item count for every sequence and the rest exit.  Measured at h = 32 against the
    // 4-wave kernel: equal lengths of 1024-4096 4-12 % faster, mixed lengths
    // of mean 1200-6800 within +-4 %, 64 sequences of mean 650 8-9 % slower
    // (256-row tiles leave more rows idle on short sequences).
    p.batch = (int)batch;
    if (d == 128 && h % 8 == 0 && batch <= 64 && total_q >= 1024 * batch &&
        h * (total_q / 256) / (causal ? 2 : 1) >= 256) {
        const int64_t t256 = (max_sq + 255) / 256;
        const int64_t per_seq = causal ? (t256 + 1) / 2 : t256;
        const int64_t pp_items = h * batch * per_seq;
        if (pp_items > lim - 8)
            return fail(FA_ERR_TOO_LARGE, "fa_fwd_varlen: too many tiles for one launch");
        mode = 2;
        p.n_items = (int)pp_items;
        p.grid = (int)(((pp_items + 7) / 8) * 8);
    }
    hipError_t e = fa::launch_fwd_varlen(dtype, (int)d, p, mode, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "fa_fwd_varlen: launch failed: %s", hipGetErrorString(e));
        return FA_ERR_HIP;
    }
    g_err[0] = 0;
    return FA_OK;
}

FA_API size_t fa_bwd_workspace_bytes(int64_t b, int64_t h, int64_t sq)
{
    if (b <= 0 || h <= 0 || sq <= 0) return 0;
    return (size_t)(b * h * sq) * 4;
}

// the backward's outputs and workspace (dq, dk, dv, D: nq, nk, nk, nw bytes)
// must be disjoint from its inputs (q, k, v, o, dout: nq, nk, nk, nq, nq
// bytes; lse: nl bytes) and from each other; returns the failing rule or null
static const char* bwd_overlap(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t nq,
                               size_t nk, size_t nl, size_t nw)
{
    const void* in[6] = {q, k, v, o, dout, lse};
    const size_t in_n[6] = {nq, nk, nk, nq, nq, nl};
    const void* outs[4] = {dq, dk, dv, workspace};
    const size_t out_n[4] = {nq, nk, nk, nw};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], out_n[i], in[j], in_n[j])) return "dq, dk, dv and workspace must not overlap the inputs";
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], out_n[i], outs[j], out_n[j]))
                return "dq, dk, dv and workspace must not overlap each other";
    }
    return nullptr;
}

// scale * log2(e), signed; a zero scale uses 1e-30 as the forward does
// (exp2(1e-30 s) is exactly 1 in fp32), so c is never zero and a masked
// score of -inf * sign(c) always exponentiates to 0
static float bwd_exp_factor(float scale)
{
    return scale != 0.f ? (float)((double)scale * 1.4426950408889634) : 1e-30f;
}

FA_API int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale, int causal,
                  int dtype, void* stream)
{
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd: NULL pointer");
    if (b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || d <= 0)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd: b, h, sq, sk and d must be >= 1");
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "fa_bwd: scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_bwd: causal must be 0 or 1");
    if (d > 4096 || !fa::bwd_supported(dtype, (int)d))
        return fail(FA_ERR_UNSUPPORTED, "fa_bwd: fp16/bf16 with d = 64, 128 or 256 only");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
        return fail(FA_ERR_MISALIGNED, "fa_bwd: tensors and workspace must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return fail(FA_ERR_MISALIGNED, "fa_bwd: lse must be 4-byte aligned");
    const int64_t lim = INT32_MAX;
    if (sq * d > lim || sk * d > lim || b * h > lim || b > lim || h > lim || b * h * sq > lim)
        return fail(FA_ERR_TOO_LARGE, "fa_bwd: a per-head slice exceeds 2^31-1 elements");
    const size_t need = fa_bwd_workspace_bytes(b, h, sq);
    if (workspace_bytes < need)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd: workspace smaller than fa_bwd_workspace_bytes()");
    const size_t nq = (size_t)(b * h * sq * d) * 2, nk = (size_t)(b * h * sk * d) * 2;
    const size_t nl = (size_t)(b * h * sq) * 4;
    if (const char* why = bwd_overlap(q, k, v, o, dout, lse, dq, dk, dv, workspace, nq, nk, nl, need)) {
        snprintf(g_err, sizeof g_err, "fa_bwd: %s", why);
        return FA_ERR_INVALID_ARG;
    }
    const int64_t items = b * h * ((std::max(sq, sk) + 127) / 128) * (d > 128 ? 2 : 1);
    if (items > lim - 8) return fail(FA_ERR_TOO_LARGE, "fa_bwd: too many tiles for one launch");

    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dvec = (float*)workspace;
    p.bh = (int)(b * h);
    p.sq = (int)sq;
    p.sk = (int)sk;
    p.c = bwd_exp_factor(scale);
    p.scale = scale;
    p.causal = causal;
    p.items_per_head = 0;
    p.n_items = 0;
    p.cu_q = nullptr;
    p.cu_k = nullptr;
    p.batch = 1;
    p.total_q = 0;
    p.total_k = 0;
    hipError_t e = fa::launch_bwd(dtype, (int)d, p, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "fa_bwd: launch failed: %s", hipGetErrorString(e));
        return FA_ERR_HIP;
    }
    g_err[0] = 0;
    return FA_OK;
}

FA_API int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int64_t batch, int64_t h, int64_t total_q, int64_t total_k, int64_t max_sq,
                         int64_t max_sk, int64_t d, float scale, int causal, int dtype, void* stream)
{
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace || !cu_seqlens_q ||
        !cu_seqlens_k)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd_varlen: NULL pointer");
    if (batch <= 0 || h <= 0 || total_q <= 0 || total_k <= 0 || max_sq <= 0 || max_sk <= 0 || d <= 0)
        return fail(FA_ERR_INVALID_ARG,
                    "fa_bwd_varlen: batch, h, total_q, total_k, max_sq, max_sk and d must be >= 1");
    if (max_sq > total_q || max_sk > total_k)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd_varlen: max_sq / max_sk exceed total_q / total_k");
    if (!isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "fa_bwd_varlen: scale must be finite");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_bwd_varlen: causal must be 0 or 1");
    if (d > 4096 || !fa::bwd_supported(dtype, (int)d))
        return fail(FA_ERR_UNSUPPORTED, "fa_bwd_varlen: fp16/bf16 with d = 64, 128 or 256 only");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
        return fail(FA_ERR_MISALIGNED, "fa_bwd_varlen: tensors and workspace must be 16-byte aligned");
    if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u)
        return fail(FA_ERR_MISALIGNED, "fa_bwd_varlen: lse and the offset arrays must be 4-byte aligned");
    const int64_t lim = INT32_MAX;
    if (total_q * d > lim || total_k * d > lim || h > lim || batch > lim - 1 || h * total_q > lim ||
        h * batch > lim)
        return fail(FA_ERR_TOO_LARGE, "fa_bwd_varlen: a per-head slice exceeds 2^31-1 elements");
    const size_t need = fa_bwd_workspace_bytes(1, h, total_q);
    if (workspace_bytes < need)
        return fail(FA_ERR_INVALID_ARG, "fa_bwd_varlen: workspace smaller than fa_bwd_workspace_bytes(1, h, total_q)");
    const size_t nq = (size_t)(h * total_q * d) * 2, nk = (size_t)(h * total_k * d) * 2;
    const size_t nl = (size_t)(h * total_q) * 4;
    if (const char* why = bwd_overlap(q, k, v, o, dout, lse, dq, dk, dv, workspace, nq, nk, nl, need)) {
        snprintf(g_err, sizeof g_err, "fa_bwd_varlen: %s", why);
        return FA_ERR_INVALID_ARG;
    }
    const int64_t items = h * batch * ((std::max(max_sq, max_sk) + 127) / 128) * (d > 128 ? 2 : 1);
    if (items > lim - 8) return fail(FA_ERR_TOO_LARGE, "fa_bwd_varlen: too many tiles for one launch");

    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dvec = (float*)workspace;
    p.bh = (int)(h * batch);  // (head, sequence) pairs
    p.sq = (int)max_sq;       // grid sizes; each work item reads its own lengths
    p.sk = (int)max_sk;
    p.c = bwd_exp_factor(scale);
    p.scale = scale;
    p.causal = causal;
    p.items_per_head = 0;
    p.n_items = 0;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.batch = (int)batch;
    p.total_q = (int)total_q;
    p.total_k = (int)total_k;
    hipError_t e = fa::launch_bwd(dtype, (int)d, p, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "fa_bwd_varlen: launch failed: %s", hipGetErrorString(e));
        return FA_ERR_HIP;
    }
    g_err[0] = 0;
    return FA_OK;
}

FA_API int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t b, int64_t h, int64_t sq, int64_t sk, int64_t d, float scale,
                      float descale_q, float descale_k, float descale_v, int causal, void* stream)
{
    if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: NULL pointer");
    if (b <= 0 || h <= 0 || sq <= 0 || sk <= 0 || d <= 0)
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: b, h, sq, sk and d must be >= 1");
    if (!isfinite(scale) || !isfinite(descale_q) || !isfinite(descale_k) || !isfinite(descale_v))
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: scale and descale factors must be finite");
    if (!isfinite((float)((double)scale * (double)descale_q * (double)descale_k * 1.4426950408889634)))
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: scale * descale_q * descale_k overflows fp32");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: causal must be 0 or 1");
    if (d != 128) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: d = 128 only");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
        return fail(FA_ERR_MISALIGNED, "fa_fwd_fp8: q, k, v, o must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return fail(FA_ERR_MISALIGNED, "fa_fwd_fp8: lse must be 4-byte aligned");
    const int64_t lim = INT32_MAX;
    if (sq * d > lim || sk * d > lim || b * h > lim || b > lim || h > lim)
        return fail(FA_ERR_TOO_LARGE, "fa_fwd_fp8: a per-head slice exceeds 2^31-1 elements");
    const int64_t items = b * h * ((sq + 127) / 128);
    if (items > lim - 8) return fail(FA_ERR_TOO_LARGE, "fa_fwd_fp8: too many tiles for one launch");
    const size_t nq = (size_t)(b * h * sq * d), nk = (size_t)(b * h * sk * d);
    const size_t no = nq * 2, nl = (size_t)(b * h * sq) * 4;
    if (overlap(o, no, q, nq) || overlap(o, no, k, nk) || overlap(o, no, v, nk) ||
        overlap(lse, nl, q, nq) || overlap(lse, nl, k, nk) || overlap(lse, nl, v, nk) ||
        overlap(lse, nl, o, no))
        return fail(FA_ERR_INVALID_ARG, "fa_fwd_fp8: o and lse must not overlap the inputs or each other");

    fa::Fp8Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.bh = (int)(b * h);
    p.sq = (int)sq;
    p.sk = (int)sk;
    p.c = (float)((double)scale * (double)descale_q * (double)descale_k * 1.4426950408889634);
    p.vscale = descale_v;
    p.causal = causal;
    p.items_per_head = 0;
    p.n_items = 0;
    hipError_t e = fa::launch_fwd_fp8(p, (hipStream_t)stream);
    if (e != hipSuccess) {
        snprintf(g_err, sizeof g_err, "fa_fwd_fp8: launch failed: %s", hipGetErrorString(e));
        return FA_ERR_HIP;
    }
    g_err[0] = 0;
    return FA_OK;
}

}  // extern "C"
