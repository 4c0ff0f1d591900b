// fa_device.h -- device helpers shared by the gfx950 kernels: vector types,
// the 32x32x16 matrix-core call, fp32 -> 16-bit packing, global -> LDS copies,
// waits and barriers, compile-time loops.  Internal; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16_t mfma16(u32x4_t a, u32x4_t b, f32x16_t c, bool bf16)
{
    if (bf16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// two fp32 -> two 16-bit values packed in one dword, round-to-nearest-even
__device__ __forceinline__ uint32_t pack2(float lo, float hi, bool bf16)
{
    if (bf16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        bf16x2_t p;
        p[0] = (__bf16)lo;
        p[1] = (__bf16)hi;
        return __builtin_bit_cast(uint32_t, p);
    }
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    f16x2_t p;
    p[0] = (_Float16)lo;
    p[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, p);
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* ptr)
{
    return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)ptr);
}

// a pointer the compiler cannot prove wave-uniform, moved to scalar registers
// (the caller knows it is uniform)
__device__ __forceinline__ const void* uniform_ptr(const void* ptr)
{
    const uint64_t v = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// One 1 KiB global -> LDS copy: lane i's 16 bytes at sbase + voff land at LDS
// byte address lds_base + 16 i.  Issued as inline assembly so the compiler does
// not serialise the other stage's LDS reads behind it; completion is awaited
// explicitly with wait_copies() before the barrier that publishes the stage.
template <int IMM>
__device__ __forceinline__ void copy_1k(const void* sbase, uint32_t voff, uint32_t lds_base)
{
#ifdef FA_LDS_POISON
    // Debug build (libfa_poison.so): this lane's 16 destination bytes are set
    // to all ones (NaN in fp16, bf16 and E4M3) just before the copy is issued.
    // A wave that reads a stage before its copies have landed, or a copy into
    // a stage another wave still reads, then shows up as NaN in the outputs
    // instead of as stale finite data.
    // (the base address and source pointer are wave-uniform: the callers say
    // so, and the copy below needs them in scalar registers)
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    sbase = uniform_ptr(sbase);
    typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
    *(lds_u32x4_t*)(uintptr_t)(lds_base + IMM + 16u * (threadIdx.x & 63u)) = u32x4_t{~0u, ~0u, ~0u, ~0u};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
    asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"(sbase), "n"(IMM)
                 : "memory", "m0", "scc");
}

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (n < 16)
template <int N>
__device__ __forceinline__ void wait_copies_le()
{
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// workgroup barrier after this wave's LDS operations have completed; unlike
// __syncthreads() it does not wait for outstanding global->LDS copies
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int S>
struct Stage {
    static constexpr int value = S;
};

// f(Stage<0>{}), ..., f(Stage<N-1>{}): compile-time indices for immediates
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (I < N) {
        f(Stage<I>{});
        static_for<N, I + 1>(f);
    }
}

// workgroup id -> (head slice, work item), spreading consecutive ids over the
// XCDs so each XCD takes a contiguous, head-major run of items (its L2 then
// sees the same head's tensors from many workgroups).  The grid is n_items
// rounded up to a multiple of kXcds; ids past the last item return false.
__device__ __forceinline__ bool map_xcd_item(int n_items, int items_per_head, int& bh, int& item)
{
    const int id = blockIdx.x;
    const int per = (n_items + kXcds - 1) / kXcds;
    const int t = (id % kXcds) * per + id / kXcds;
    if (t >= n_items) return false;
    bh = t / items_per_head;
    item = t - bh * items_per_head;
    return true;
}

}  // namespace fa
