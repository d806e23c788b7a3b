// VALU issue-rate probe for gfx950: a measurement kernel, not part of the state step.  It gives the
// instruction-issue ceiling against which the step's own issue rate is read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace sq {

// ---- VALU issue-rate probe: every lane advances kProbeChains independent FMA chains for
// kProbeIters steps, so a wave issues kProbeChains * kProbeIters v_fma_f32 with nothing else to
// wait for.  The launch reserves dynamic LDS so that only a chosen number of workgroups (one wave
// per SIMD each) fit on a CU: the rate is then the FMA issue ceiling at that many waves per SIMD.
constexpr int kProbeIters = 1024, kProbeChains = 8, kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads) k_valu_probe(float* out, float m, float a) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    // vector-register operands, as in the step (an instruction that reads a scalar register
    // issues at a lower rate)
    float mv = m, av = a;
    __asm__ volatile("" : "+v"(mv), "+v"(av));
    float acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = (float)(tid + c);
    for (int i = 0; i < kProbeIters; ++i) {
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) acc[c] = fmaf(acc[c], mv, av);
    }
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) t += acc[c];
    out[(size_t)__builtin_amdgcn_workgroup_id_x() * kProbeThreads + tid] = t;
}

hipError_t launch_valu_probe(int waves_per_simd, int n_blocks, float* out, uint64_t* n_fma, int* blocks_per_cu,
                             hipStream_t s) {
    int dev = 0, lds_cu = 0, lds_block = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    // waves_per_simd workgroups fit in the CU's LDS, one more does not
    const size_t lds = (size_t(lds_cu) / size_t(waves_per_simd)) & ~size_t(1023);
    if (lds == 0 || lds > size_t(lds_block) || (waves_per_simd + 1) * lds <= size_t(lds_cu)) return hipErrorNotSupported;
    int fit = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, k_valu_probe, kProbeThreads, lds);
    if (e != hipSuccess) return e;
    *blocks_per_cu = fit;
    *n_fma = uint64_t(n_blocks) * (kProbeThreads / 64) * kProbeIters * kProbeChains;
    k_valu_probe<<<dim3(unsigned(n_blocks)), dim3(kProbeThreads), lds, s>>>(out, 0.999f, 0.001f);
    return hipGetLastError();
}

}  // namespace sq
