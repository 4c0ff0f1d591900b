// fa_probe.hip -- shader-clock probe for measurement.
//
// The matrix-core peak of a GPU scales with its shader clock, which the power
// manager lowers under heavy matrix-core load.  This probe lets a caller read
// the clock the kernels actually ran at: one wave reads the shader-clock
// counter (s_memtime) and the constant 100 MHz real-time counter
// (s_memrealtime), spins on the real-time counter for a fixed number of its
// ticks, and reads both again.  Launched right behind a stream of attention
// launches on the same stream, it runs at the clock the power manager chose
// for them (the manager reacts on a millisecond scale; the probe lasts tens of
// microseconds).  The spin always ends: the real-time counter only grows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace {

__global__ void __launch_bounds__(64) clock_probe(unsigned long long* out, unsigned long long ticks)
{
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long r1 = r0;
    while (r1 - r0 < ticks) r1 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    // lanes 0 and 1 store the two differences (vector stores)
    const int lane = threadIdx.x;
    if (lane < 2) out[lane] = lane == 0 ? c1 - c0 : r1 - r0;
}

}  // namespace

extern "C" {

FA_API int fa_clock_probe(unsigned long long* out, int64_t ticks, void* stream)
{
    if (out == nullptr || ticks < 1 || ticks > 10000000) return FA_ERR_INVALID_ARG;
    if ((uintptr_t)out % 8 != 0) return FA_ERR_MISALIGNED;
    hipLaunchKernelGGL(clock_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, out,
                       (unsigned long long)ticks);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
