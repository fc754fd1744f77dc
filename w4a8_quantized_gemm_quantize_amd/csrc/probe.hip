// probe.hip -- measurement aid: an int8 matrix-core loop with nothing else in
// it, the compute reference that the GEMMs' MFMA utilisation is quoted
// against, and a clock readout taken while it runs.
//
// Each wavefront keeps 16 independent v_mfma_i32_16x16x64_i8 accumulators
// (one dependent chain would leave the matrix core waiting on its own
// latency) and runs `iters` rounds of 16 products.  Two wavefronts per SIMD
// (8 per workgroup, one workgroup per compute unit).  Wavefront 0 of
// workgroup 0 reads the shader clock counter (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime) before and after its loop; their ratio is
// the shader clock during the run.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a8 {
namespace {

__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters, int *__restrict__ sink,
                                                         unsigned long long *__restrict__ clk) {
    const int tid = threadIdx.x;
    // operands that depend on the thread, so nothing can be folded
    const v4i a = {tid, tid ^ 0x55, (int)blockIdx.x, 0x01020304};
    const v4i b = {0x01010101 + tid, 7, (int)blockIdx.x * 3, tid * 5};
    v4i acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = v4i{j, 0, 0, 0};
    const bool timer = blockIdx.x == 0 && tid == 0;
    unsigned long long t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = mfma16x16x64(a, b, acc[j]);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    sink[(int64_t)blockIdx.x * blockDim.x + tid] = s;
    if (timer) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_mfma_probe(int64_t workgroups, int32_t iters, int32_t *sink, uint64_t *clocks,
                             hipStream_t stream) {
    mfma_probe_kernel<<<(unsigned)workgroups, 512, 0, stream>>>(
        iters, sink, (unsigned long long *)clocks);
    return hipGetLastError();
}

}  // namespace w4a8
