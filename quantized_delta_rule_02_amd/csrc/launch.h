// Kernel launchers (kernels.hip) called by the C ABI (api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "internal.h"

namespace sq {

bool shape_compiled(int dk, int dv);
int compiled_shapes(int32_t* out, int max_pairs);
// One launch over requests [p.b0, p.b0 + n_b) and layers [p.lz0, p.lz0 + n_z) of the call (relative to
// p.layer0), every head: a grid of (heads, n_b, n_z) workgroups.
hipError_t launch_state(int dk, int dv, int mode, const StepParams& p, int n_b, int n_z, hipStream_t s);
hipError_t launch_codec(int dk, int dv, bool do_export, const CodecParams& p, int n_states, hipStream_t s);
hipError_t launch_cmp(int dk, int dv, bool int8, int form, int n_heads, int n_slots, int layer0, int n_layers,
                      int batch, const int32_t* slots, int8_t* codes, float* scales, float* S, const float* q,
                      const float* k, const float* v, const float* gate, const float* beta, float* y,
                      hipStream_t s);
// Device address of the fixed split scratch (kStaticScratchFloats floats) on the current device, looked up
// once per device and kept; hipErrorInvalidDevice beyond the devices this process can hold.
hipError_t static_scratch(float** out);
hipError_t launch_copy(const void* src, void* dst, size_t n_bytes, hipStream_t s);
// hipErrorNotSupported: the device's LDS cannot cap residency at waves_per_simd workgroups per CU
hipError_t launch_valu_probe(int waves_per_simd, int n_blocks, float* out, uint64_t* n_fma, int* blocks_per_cu,
                             hipStream_t s);

}  // namespace sq
