// clock_probe.hip -- a measurement aid of the benchmark (libfa_clock.so), not
// part of the attention library or its C ABI.
//
// The matrix-core peak a kernel is priced against assumes the 2.4 GHz peak
// shader clock; under a sustained matrix-core load the part runs slower.  The
// probe reports the clock the device is running at: launched right after a
// timed kernel on the same stream, each of its single-wave workgroups reads
// the shader-clock counter (s_memtime) and the constant 100 MHz real-time
// counter (s_memrealtime) at its start, spins until `ticks` real-time ticks
// have passed, and reads both again.  Shader cycles over real-time ticks,
// times 100 MHz, is the clock.  Workgroups are dispatched to the XCDs round
// robin, so `workgroups` = 8 samples each XCD once; each record also carries
// the XCC_ID hardware register.
//
// Record of workgroup g (4 x u64 at out + 4 g):
//   [0] shader cycles elapsed, [1] real-time ticks elapsed, [2] XCC id, [3] 0.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, int ticks)
{
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long r1 = r0;
    while (r1 - r0 < (unsigned long long)ticks) r1 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    // HW_REG_XCC_ID (hardware register 20), bits 3:0
    const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf;
    if (threadIdx.x == 0) {
        unsigned long long* rec = out + 4 * blockIdx.x;
        rec[0] = t1 - t0;
        rec[1] = r1 - r0;
        rec[2] = xcc;
        rec[3] = 0;
    }
}

}  // namespace

extern "C" {

// Enqueue the probe on `stream`: `workgroups` (1..1024) single-wave workgroups,
// each spinning `ticks` (1..100000) ticks of the 100 MHz counter and writing
// its record to out (device memory, 4 * workgroups u64).  Returns 0, 1 for a
// bad argument, 2 for a failed launch.
int fa_clock_probe(unsigned long long* out, int workgroups, int ticks, hipStream_t stream)
{
    if (!out || workgroups < 1 || workgroups > 1024 || ticks < 1 || ticks > 100000) return 1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(64), 0, stream, out, ticks);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
