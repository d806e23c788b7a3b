// gfx950 kernels of the quantized gated-delta state step.
//
// One workgroup of NW wave64s processes one (request, layer, head) state.
// Wave w owns RPW storage rows; lane l owns CPL adjacent value columns, so
//   * every key-row quantity (gate, k, q, row factor, impact) is uniform across
//     a wave and is read from LDS by broadcast,
//   * the column reductions k^T D S, q^T D S, the column base and the fit
//     objective accumulate in registers, then across the NW waves through LDS,
//   * the row maximum is the one cross-lane reduction (transpose-reduce).
// Per-row quantities (coefficients, row factors, rounding bounds) are computed
// by the wave that owns the row and live in LDS only for that wave, so the
// waves of a state meet at a workgroup barrier only for the three column
// reductions (k^T D S and q^T D S, the column base, the fit objective).
// The state never leaves registers between the unpack and the pack: HBM sees
// the packed codes and scales once in each direction plus q, k, v, gate, beta, y.
// See internal.h for the record layout.
//
// Method (STEPQuant pages): rcap.io post, decode-step pseudocode (unpack ->
// X = D S + beta k (v^T - k^T D S) -> y = X^T q before requantization -> row
// factors sqrt(row magnitude / row impact) -> impact-weighted column fit ->
// round at each unit's width); hyper.ai summary, section 方法 (Method), on the
// fused reconstruction + update + readout kernel and the dual-axis fit and
// packed write-back.  The column fit searches a fixed grid of candidates
// gamma * c0 with c0 = max_i |X_ij| / (r_i qmax_i).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "launch.h"

#ifndef STEP_WAVES_PER_EU
#define STEP_WAVES_PER_EU 4   // waves per SIMD the register allocation targets (128 VGPRs; the 128x128
                              // step spills two registers, on the path of 16-bit groups only)
#endif

namespace sq {

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}
__device__ __forceinline__ uint32_t f2h_bits(float x) {
    return (uint32_t)__half_as_ushort(__float2half_rn(x));
}
// binary16 value (as float) of a positive scale clamped to [2^-14, 65504]
__device__ __forceinline__ float scale_fp16(float x) {
    x = fminf(fmaxf(x, 0x1p-14f), 65504.0f);
    return __half2float(__float2half_rn(x));
}
__device__ __forceinline__ float med3(float x, float lo, float hi) {
    return __builtin_amdgcn_fmed3f(x, lo, hi);
}
__device__ __forceinline__ int bias_of(int bits) { return bits == 16 ? 0 : (1 << (bits - 1)); }
// Work-group and work-item indices straight from the hardware registers.  The library's own
// query functions are built with IEEE mode on, so with IEEE mode off here they are not inlined:
// each kernel would call them and receive the block index in a vector register.
__device__ __forceinline__ int block_idx() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int block_idy() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int block_idz() { return (int)__builtin_amdgcn_workgroup_id_z(); }
// A load whose address is the same for every lane, of memory no kernel of the launch writes (plan tables,
// slot lists, per-state inputs): read through the constant address space, so it becomes a scalar load.
template <class T>
__device__ __forceinline__ T ld_const(const T* p) {
    return *(const __attribute__((address_space(4))) T*)(uintptr_t)p;
}
__device__ __forceinline__ int thread_idx() { return (int)__builtin_amdgcn_workitem_id_x(); }
// a value every lane of the wave holds, moved to a scalar register
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
}

// Orders this wave's LDS writes before its later LDS reads (other lanes' values of the
// same wave); no other wave takes part.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16 entries of one lane in one group <-> container dwords (internal.h)
__device__ __forceinline__ void unpack4(const uint32_t* d, float* o) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = e & 7;
        o[e] = (float)((d[e >> 3] >> (8 * (i & 3) + 4 * (i >> 2))) & 0xFu);
    }
}
__device__ __forceinline__ void unpack6(const uint32_t* d, float* o) {
#pragma unroll
    for (int e = 0; e < 12; ++e) o[e] = (float)((d[e >> 2] >> (8 * (e & 3))) & 0x3Fu);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t s = 8 * k + 6;
        o[12 + k] = (float)(((d[0] >> s) & 3u) | (((d[1] >> s) & 3u) << 2) | (((d[2] >> s) & 3u) << 4));
    }
}
__device__ __forceinline__ void unpack8(const uint32_t* d, float* o) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (float)((d[e >> 2] >> (8 * (e & 3))) & 0xFFu);
}
// 2-bit: entry e = 4k + j at bits 8j + 2k of one dword.  3-bit: the low two bits likewise, the
// third bit of entry 4k + j at bit 4j + k of a 16-bit plane (internal.h).
__device__ __forceinline__ void unpack2(uint32_t lo, float* o) {
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (float)((lo >> (8 * (e & 3) + 2 * (e >> 2))) & 3u);
}
__device__ __forceinline__ void unpack3(uint32_t lo, uint32_t hi, float* o) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int j = e & 3, k = e >> 2;
        o[e] = (float)(((lo >> (8 * j + 2 * k)) & 3u) | (((hi >> (4 * j + k)) & 1u) << 2));
    }
}
__device__ __forceinline__ void pack2(const int* c, uint32_t* lo) {
    uint32_t x = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) x |= (uint32_t)(c[e] & 3) << (8 * (e & 3) + 2 * (e >> 2));
    *lo = x;
}
__device__ __forceinline__ void pack3(const int* c, uint32_t* lo, uint32_t* hi) {
    uint32_t x = 0, h = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int j = e & 3, k = e >> 2;
        x |= (uint32_t)(c[e] & 3) << (8 * j + 2 * k);
        h |= (uint32_t)((c[e] >> 2) & 1) << (4 * j + k);
    }
    *lo = x;
    *hi = h;
}
__device__ __forceinline__ void pack4(const int* c, uint32_t* d) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) x |= (uint32_t)(c[8 * w + i] & 0xF) << (8 * (i & 3) + 4 * (i >> 2));
        d[w] = x;
    }
}
__device__ __forceinline__ void pack6(const int* c, uint32_t* d) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = (uint32_t)(c[4 * w + k] & 0x3F) | ((((uint32_t)c[12 + k] >> (2 * w)) & 3u) << 6);
            x |= b << (8 * k);
        }
        d[w] = x;
    }
}
__device__ __forceinline__ void pack8(const int* c, uint32_t* d) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) x |= (uint32_t)(c[4 * w + k] & 0xFF) << (8 * k);
        d[w] = x;
    }
}

template <int NDW>
__device__ __forceinline__ void load_dw(const uint8_t* p, uint32_t* d) {
    if constexpr (NDW == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        d[0] = v.x; d[1] = v.y;
    } else if constexpr (NDW == 3) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        d[0] = q[0]; d[1] = q[1]; d[2] = q[2];
    } else if constexpr (NDW == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else {
        const uint4 v0 = reinterpret_cast<const uint4*>(p)[0];
        const uint4 v1 = reinterpret_cast<const uint4*>(p)[1];
        d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w;
        d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
    }
}
template <int NDW>
__device__ __forceinline__ void store_dw(uint8_t* p, const uint32_t* d) {
    if constexpr (NDW == 2) {
        *reinterpret_cast<uint2*>(p) = make_uint2(d[0], d[1]);
    } else if constexpr (NDW == 3) {
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        q[0] = d[0]; q[1] = d[1]; q[2] = d[2];
    } else if constexpr (NDW == 4) {
        *reinterpret_cast<uint4*>(p) = make_uint4(d[0], d[1], d[2], d[3]);
    } else {
        reinterpret_cast<uint4*>(p)[0] = make_uint4(d[0], d[1], d[2], d[3]);
        reinterpret_cast<uint4*>(p)[1] = make_uint4(d[4], d[5], d[6], d[7]);
    }
}

// Wave-level data movement for the row maximum.  v_permlane32_swap exchanges
// rows 2-3 of its first operand with rows 0-1 of its second (rows of 16
// lanes); v_permlane16_swap exchanges rows 1 and 3 of the first with rows 0
// and 2 of the second.  DPP: row_ror:8 pairs lane l with l^8 inside a 16-lane
// row, row_half_mirror pairs l with 7-(l&7) inside 8 lanes, quad_perm
// [2,3,0,1] / [1,0,3,2] pair l with l^2 / l^1.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRor8 = 0x128;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;

template <int D>
__device__ __forceinline__ float dpp_partner(float x) {
    if constexpr (D == 8) return dpp_f<kDppRor8>(x);
    else if constexpr (D == 4) return dpp_f<kDppHalfMirror>(x);
    else if constexpr (D == 2) return dpp_f<kDppXor2>(x);
    else return dpp_f<kDppXor1>(x);
}

// Sum over the 64 lanes of a wave (the result is valid in lane 0): xor-1, xor-2 and the
// two mirrors reduce each row of 16 lanes, lane reads add the four rows.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<0x140>(x);   // row_mirror
    const int xi = __float_as_int(x);
    return (__int_as_float(__builtin_amdgcn_readlane(xi, 0)) + __int_as_float(__builtin_amdgcn_readlane(xi, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(xi, 32)) + __int_as_float(__builtin_amdgcn_readlane(xi, 48)));
}

// Transpose-reduce of per-row maxima across the LPR lanes of a row band.
// Before: v[0..N) = this lane's partial max of local rows 0..N-1.  Each halving
// stage pairs every lane with a lane of the other half of a group of 2D lanes;
// the lane keeps the half of its rows selected by its bit D and takes the
// partner's values of those rows.  After: v[0] = the max of local row `row`
// over all LPR lanes (LPR/N lanes hold each row).
template <int D, int N>
struct RowMax {
    static __device__ __forceinline__ void run(float* v, int lane, int& row) {
        if constexpr (D >= 1) {
            if constexpr (N > 1) {
                const bool hi = (lane & D) != 0;
                if constexpr (D == 32 || D == 16) {
#pragma unroll
                    for (int i = 0; i < N / 2; ++i) {
                        uint32_t x = __float_as_uint(v[i]), y = __float_as_uint(v[i + N / 2]);
                        const auto r = (D == 32) ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                                                 : __builtin_amdgcn_permlane16_swap(x, y, false, false);
                        v[i] = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < N / 2; ++i) {
                        const float lo = fmaxf(v[i], dpp_partner<D>(v[i]));
                        const float up = fmaxf(v[i + N / 2], dpp_partner<D>(v[i + N / 2]));
                        v[i] = hi ? up : lo;
                    }
                }
                if (hi) row += N / 2;
                RowMax<D / 2, N / 2>::run(v, lane, row);
            } else {
                static_assert(D <= 8, "a butterfly across rows of 16 lanes is not needed by any shape");
                v[0] = fmaxf(v[0], dpp_partner<D>(v[0]));
                RowMax<D / 2, 1>::run(v, lane, row);
            }
        }
    }
};

// ---------------------------------------------------------------- the step kernel

template <int DK, int DV>
struct Shape {
    static constexpr int CPL = cpl_of(DV);
    static constexpr int LPR = lpr_of(DV);
    static constexpr int GR = gr_of(DV);
    static constexpr int RPW = rpw_of(DK, DV);
    static constexpr int NW = nw_of(DK, DV);
    static constexpr int GPW = RPW / GR;
    static constexpr int EPL = RPW * CPL;
    static constexpr int NG = ng_of(DK, DV);
    static_assert(RPW <= LPR, "row band taller than the lanes that reduce it");
    static_assert(GPW * GR == RPW && EPL == 16 * GPW, "group tiling");
};

template <int DK, int DV>
struct StepSmem {
    float2 acc[DK];    // column-sum coefficients: D_i r_i (k_i, q_i) on code rows, D_i (k_i, q_i) on pivot rows
    float2 upd[DK];    // update: D_i r_i (D_i on pivot rows), beta k_i
    float4 fit[DK];    // requantization: sqrt(w) r_new, -sqrt(w) r_new / 2, 1/2 - qmax, 1 / r_new
    float ir[DK];      // 1 / r_new, contiguous: four rows per wide read
    float iq[DK];      // 1 / qmax (0 on pivot rows)
    float2 fin[DK];    // final rounding bounds: magic + container bias -/+ qmax
    float rn[DK];      // new binary16 row factor
    float2 wf[DK];     // 1 / w and sqrt(w)
    int rb[DK];        // code width of the row (16 = pivot)
    float stage[Shape<DK, DV>::NW][3][DK];   // each wave's copy of k, q and the per-row gate, canonical order
    float part[Shape<DK, DV>::NW][4][DV];    // column sums of k^T D S, q^T D S; later the fit objective
    float cmax[Shape<DK, DV>::NW][DV];       // column base partial maxima
    float red[Shape<DK, DV>::NW];            // k^T q partials
};

constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23: x + kMagic rounds x to an integer in the low mantissa bits

// byte 0 of four registers -> one dword
__device__ __forceinline__ uint32_t gather4(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3) {
    const uint32_t a = __builtin_amdgcn_perm(r1, r0, 0x0C0C0400u);
    const uint32_t b = __builtin_amdgcn_perm(r3, r2, 0x0C0C0400u);
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// A v_and_b32 whose result the compiler cannot see through.  Given a masked dword, it would
// otherwise rewrite each byte's conversion as a bit-field extract plus a conversion (v_bfe_u32 issues
// at the slow VALU rate) instead of one v_cvt_f32_ubyteN (1% on the step).
template <uint32_t M>
__device__ __forceinline__ uint32_t and_opaque(uint32_t x) {
    uint32_t r;
    __asm__("v_and_b32 %0, %1, %2" : "=v"(r) : "i"(M), "v"(x));
    return r;
}

// fast unpack of one lane's 16 stored (offset) codes to float (layout in internal.h)
__device__ __forceinline__ void unpack4f(const uint32_t* d, float* o) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t lo = and_opaque<0x0F0F0F0Fu>(d[w]), hi = and_opaque<0x0F0F0F0Fu>(d[w] >> 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[8 * w + k] = (float)((lo >> (8 * k)) & 0xFFu);
            o[8 * w + 4 + k] = (float)((hi >> (8 * k)) & 0xFFu);
        }
    }
}
__device__ __forceinline__ void unpack6f(const uint32_t* d, float* o) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const uint32_t x = and_opaque<0x3F3F3F3Fu>(d[w]);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[4 * w + k] = (float)((x >> (8 * k)) & 0xFFu);
    }
    const uint32_t t0 = d[0] >> 6, t1 = d[1] >> 4, t2 = d[2] >> 2;
    uint32_t p = (t0 & 0x03030303u) | (t1 & ~0x03030303u);
    p = (p & 0x0F0F0F0Fu) | (t2 & ~0x0F0F0F0Fu);
    p &= 0x3F3F3F3Fu;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[12 + k] = (float)((p >> (8 * k)) & 0xFFu);
}

__device__ __forceinline__ void unpack2f(uint32_t lo, float* o) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = and_opaque<0x03030303u>(lo >> (2 * k));
#pragma unroll
        for (int j = 0; j < 4; ++j) o[4 * k + j] = (float)((x >> (8 * j)) & 0xFFu);
    }
}
__device__ __forceinline__ void unpack3f(uint32_t lo, uint32_t hi, float* o) {
    // nibble j of the plane -> low nibble of byte j
    const uint32_t H = (hi & 0xFu) | ((hi << 4) & 0xF00u) | ((hi << 8) & 0xF0000u) | ((hi << 12) & 0xF000000u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t x = and_opaque<0x03030303u>(lo >> (2 * k)) | (((H >> k) & 0x01010101u) << 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[4 * k + j] = (float)((x >> (8 * j)) & 0xFFu);
    }
}

// pack 16 magic-rounded codes (the code sits in the low bits of each float's pattern)
__device__ __forceinline__ void pack4m(const float* m, uint32_t* d) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t lo = gather4(__float_as_uint(m[8 * w]), __float_as_uint(m[8 * w + 1]),
                                    __float_as_uint(m[8 * w + 2]), __float_as_uint(m[8 * w + 3]));
        const uint32_t hi = gather4(__float_as_uint(m[8 * w + 4]), __float_as_uint(m[8 * w + 5]),
                                    __float_as_uint(m[8 * w + 6]), __float_as_uint(m[8 * w + 7]));
        d[w] = lo | (hi << 4);
    }
}
__device__ __forceinline__ void pack6m(const float* m, uint32_t* d) {
    const uint32_t p = gather4(__float_as_uint(m[12]), __float_as_uint(m[13]), __float_as_uint(m[14]),
                               __float_as_uint(m[15]));
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const uint32_t b = gather4(__float_as_uint(m[4 * w]), __float_as_uint(m[4 * w + 1]),
                                   __float_as_uint(m[4 * w + 2]), __float_as_uint(m[4 * w + 3]));
        d[w] = ((p << (6 - 2 * w)) & 0xC0C0C0C0u) | b;
    }
}
__device__ __forceinline__ void pack2m(const float* m, uint32_t* lo) {
    uint32_t x = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        x |= (gather4(__float_as_uint(m[4 * k]), __float_as_uint(m[4 * k + 1]), __float_as_uint(m[4 * k + 2]),
                      __float_as_uint(m[4 * k + 3])) & 0x03030303u) << (2 * k);
    *lo = x;
}
__device__ __forceinline__ void pack3m(const float* m, uint32_t* lo, uint32_t* hi) {
    uint32_t x = 0, H = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t g = gather4(__float_as_uint(m[4 * k]), __float_as_uint(m[4 * k + 1]),
                                   __float_as_uint(m[4 * k + 2]), __float_as_uint(m[4 * k + 3]));
        x |= (g & 0x03030303u) << (2 * k);
        H |= ((g >> 2) & 0x01010101u) << k;
    }
    *lo = x;
    *hi = (H & 0xFu) | ((H >> 4) & 0xF0u) | ((H >> 8) & 0xF00u) | ((H >> 12) & 0xF000u);
}
__device__ __forceinline__ void pack8m(const float* m, uint32_t* d) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
        d[w] = gather4(__float_as_uint(m[4 * w]), __float_as_uint(m[4 * w + 1]), __float_as_uint(m[4 * w + 2]),
                       __float_as_uint(m[4 * w + 3]));
}

template <int NDW>
__device__ __forceinline__ void load_group(const uint8_t* gp, int lane, bool act, uint32_t* d) {
    if (act) load_dw<NDW>(gp + lane * 4 * NDW, d);
    else {
#pragma unroll
        for (int i = 0; i < NDW; ++i) d[i] = 0;
    }
}

// Row of the split arrangement's scratch for (layer lz of the call, request b, head h), with a layer
// stride of n_slots * n_heads.
__device__ __forceinline__ size_t e_index(const StepParams& a, int lz, int b, int h) {
    return (size_t)lz * (size_t)a.e_layer_stride + (size_t)b * a.n_heads + h;
}

// Stored codes carry the container's offset 2^(W-1).  One FMA per entry turns a stored code into
// c_j Q_ij (exact: an 11-bit scale times a code of at most 8 bits), which the column sums and the
// update then use.  Summing offset codes and taking the offset's sum off afterwards would lose the
// cancellation to rounding: for a state whose stored scales are large next to its new values (a zero
// state keeps r = c = 1) the lost digits reach the rounding of the new codes.
template <int CPL>
__device__ __forceinline__ void scale_codes(float* xg, const float* c_old, float bias) {
#pragma unroll
    for (int e = 0; e < 16; ++e) xg[e] = fmaf(xg[e], c_old[e % CPL], -bias * c_old[e % CPL]);
}

// Unpack + accumulate of a wave whose groups all use one code container (2, 3, 4, 6 or 8 bits):
// straight-line code (no width branch between groups), so each group's coefficient reads and FMAs
// stay together and the register peak stays low.
template <int W, bool ACC, class Sh, class Smem>
__device__ __forceinline__ void unpack_acc_uniform(uint32_t (&raw)[Sh::GPW][4], float* X, const Smem& sm, int wave,
                                                   float* U1, float* P1, const uint8_t* rec, const uint32_t* goff,
                                                   int lane, bool act, const float* c_old) {
    constexpr int CPL = Sh::CPL, GR = Sh::GR, RPW = Sh::RPW, GPW = Sh::GPW, LPR = Sh::LPR;
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        float* xg = &X[16 * g];
        if constexpr (W == 4) unpack4f(raw[g], xg);
        else if constexpr (W == 6) unpack6f(raw[g], xg);
        else if constexpr (W == 8) unpack8(raw[g], xg);
        else if constexpr (W == 2) unpack2f(raw[g][0], xg);
        else {
            const uint32_t hi = act ? *reinterpret_cast<const uint16_t*>(rec + ld_const(goff + wave * GPW + g) +
                                                                       LPR * 4 + lane * 2) : 0u;
            unpack3f(raw[g][0], hi, xg);
        }
        scale_codes<CPL>(xg, c_old, (float)(1 << (W - 1)));
        if constexpr (ACC) {
#pragma unroll
            for (int r = 0; r < GR; ++r) {
                const float2 cf = sm.acc[wave * RPW + g * GR + r];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    U1[c] = fmaf(cf.x, xg[r * CPL + c], U1[c]);
                    P1[c] = fmaf(cf.y, xg[r * CPL + c], P1[c]);
                }
            }
        }
    }
}

// k^T D S and q^T D S partial sums of one group's rows (coefficients from LDS).
template <bool ACC, class Sh, class Smem>
__device__ __forceinline__ void acc_group(const Smem& sm, int wave, int g, const float* xg, float* U1, float* P1) {
    constexpr int CPL = Sh::CPL, GR = Sh::GR, RPW = Sh::RPW;
    if constexpr (ACC) {
        // called inside each width branch: the memory clobber keeps the group's coefficient reads inside the
        // branch (hoisted above the width dispatch, they are held across the unpack and spill)
        __asm__ volatile("" ::: "memory");
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const float2 cf = sm.acc[wave * RPW + g * GR + r];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                U1[c] = fmaf(cf.x, xg[r * CPL + c], U1[c]);
                P1[c] = fmaf(cf.y, xg[r * CPL + c], P1[c]);
            }
        }
    }
}

// Rounding, packing and stores of a wave whose groups all use one code container.
template <int W, class Sh, class Smem>
__device__ __forceinline__ void round_pack_uniform(const float* X, const float* ic, const Smem& sm, uint8_t* rec,
                                                   const uint32_t* goff, int wave, int lane, bool act) {
    constexpr int CPL = Sh::CPL, GR = Sh::GR, RPW = Sh::RPW, GPW = Sh::GPW, LPR = Sh::LPR;
    const float mb = kMagic + (float)bias_of(W);
    // the rounding bounds of a group's GR rows (two rows per wide broadcast read); the next group's are read
    // while this group is rounded and packed
    float4 fb[2][GR / 2];
#pragma unroll
    for (int i = 0; i < GR / 2; ++i) fb[0][i] = reinterpret_cast<const float4*>(sm.fin + wave * RPW)[i];
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        if (g + 1 < GPW) {
#pragma unroll
            for (int i = 0; i < GR / 2; ++i)
                fb[(g + 1) % 2][i] = reinterpret_cast<const float4*>(sm.fin + wave * RPW + (g + 1) * GR)[i];
        }
        uint8_t* gp = rec + ld_const(goff + wave * GPW + g);
        float m[16];
        uint32_t d[4];
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const float4 f4 = fb[g % 2][r / 2];
            const float lo = (r % 2) ? f4.z : f4.x, hi = (r % 2) ? f4.w : f4.y;
#pragma unroll
            for (int c = 0; c < CPL; ++c) m[r * CPL + c] = med3(fmaf(X[16 * g + r * CPL + c], ic[c], mb), lo, hi);
        }
        if constexpr (W == 4) { pack4m(m, d); if (act) store_dw<2>(gp + lane * 8, d); }
        else if constexpr (W == 6) { pack6m(m, d); if (act) store_dw<3>(gp + lane * 12, d); }
        else if constexpr (W == 8) { pack8m(m, d); if (act) store_dw<4>(gp + lane * 16, d); }
        else if constexpr (W == 2) { pack2m(m, d); if (act) *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0]; }
        else {
            pack3m(m, d, d + 1);
            if (act) {
                *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0];
                *reinterpret_cast<uint16_t*>(gp + LPR * 4 + lane * 2) = (uint16_t)d[1];
            }
        }
    }
}

// One LDS round of the column fit: KG candidates c = binary16(gamma * c0), the
// impact-weighted error F = c^2 sum_i (sqrt(w_i) r_i)^2 (t_ij / c - Q_ij)^2 of the
// wave's rows, combined over the waves; the best candidate so far is kept (strict <).
// part[] is read by every wave after the barrier: a later round must synchronize first.
//
// The residual y - Q of y = |t| / c >= 0 and Q = min(rint(y), qmax) comes without forming Q:
// with a = y + 1/2 - qmax (one FMA; qmax is an integer, so fract(a) = fract(y + 1/2)),
//   y <  qmax + 1/2:  a < 1 and fract(a) - 1/2 = y - round(y), and fract(a) >= a;
//   y >  qmax + 1/2:  a > 1, the code clips to qmax and the residual is y - qmax = a - 1/2 > fract(a) - 1/2;
//   y == qmax + 1/2:  a = 1, a half-way point: max(a, fract(a)) - 1/2 = 1/2, the residual of either rounding;
// so |y - Q| = |max(a, fract(a)) - 1/2| in every case (at any half-way point either rounding leaves the
// same squared residual).  Per candidate and entry: FMA, fract, max, the weight FMA and the
// accumulating FMA.  a carries the rounding of a sum of magnitude up to qmax, about 2^-24 qmax,
// the order of the float32 error that t itself already has.
template <class Sh, int KG, bool FREE0, class Smem>
__device__ __forceinline__ void grid_round(Smem& sm, const float* X, const float* c0, const float* grid, int g0,
                                           int n_grid, int wave, int lane, bool act, float* cbest, float* fbest) {
    constexpr int CPL = Sh::CPL, RPW = Sh::RPW, NW = Sh::NW;
    const int col0 = lane * CPL;
    float cg[KG][CPL], icg[KG][CPL], Fp[KG][CPL];
    // the rows' LDS addresses are formed inside each round: hoisted out of the caller's round loop
    // they would hold RPW registers across it
    int rbase = uniform(wave * RPW);
    if constexpr (!FREE0) __asm__ volatile("" : "+s"(rbase));
#pragma unroll
    for (int j = 0; j < KG; ++j) {
        const float gam = grid[min(g0 + j, n_grid - 1)];   // a short last round repeats a candidate
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            cg[j][c] = scale_fp16(gam * c0[c]);
            icg[j][c] = __builtin_amdgcn_rcpf(cg[j][c]);
            Fp[j][c] = 0.f;
        }
    }
    __builtin_amdgcn_s_setprio(0);   // the row loop at low priority (the kernel's note on wave priority)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        // two rows at a time: an empty asm "redefines" the inverse scales, so later rows' candidate
        // chains cannot be hoisted above it (interleaving all rows costs registers, not speed)
        if (r % 2 == 0) {
#pragma unroll
            for (int j = 0; j < KG; ++j)
#pragma unroll
                for (int c = 0; c < CPL; ++c) __asm__ volatile("" : "+v"(icg[j][c]));
        }
        const float4 f = sm.fit[rbase + r];
        const float sw = f.x, nsw = f.y, hq = f.z;
        // The error is odd in t and round-half-even is symmetric, so the fit works on |t| (a free
        // source modifier).  The first candidate of a round that starts at gamma = 1 cannot clip (the
        // caller checks that no column base exceeds the binary16 range) and skips the max.  The row's KG x CPL chains advance in stages separated by empty asm
        // statements: left alone, the scheduler runs each chain to its end before the next, and a
        // wave then stalls on every dependent step.
        float t[CPL], A[KG][CPL], E[KG][CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) t[c] = fabsf(X[r * CPL + c]);
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) A[j][c] = fmaf(t[c], icg[j][c], hq);
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) __asm__ volatile("" : "+v"(A[j][c]));
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float fr = __builtin_amdgcn_fractf(A[j][c]);
                // max(a, fract(a)) on the bit patterns: fract(a) >= +0, so a negative a (a negative
                // integer pattern) yields fract(a), and two non-negative floats order as their
                // patterns do.  The integer max issues beside the FMAs; the float max does not.
                E[j][c] = (FREE0 && j == 0) ? fr
                                            : __int_as_float(max(__float_as_int(A[j][c]), __float_as_int(fr)));
            }
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) __asm__ volatile("" : "+v"(E[j][c]));
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float ew = fmaf(E[j][c], sw, nsw);
                Fp[j][c] = fmaf(ew, ew, Fp[j][c]);
            }
    }
    __builtin_amdgcn_s_setprio(3);   // back to high before the round's barrier and reduction
    if (act) {
#pragma unroll
        for (int j = 0; j < KG; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c) sm.part[wave][j][col0 + c] = Fp[j][c];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KG; ++j) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float F = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) F += act ? sm.part[w][j][col0 + c] : 0.f;
            F *= cg[j][c] * cg[j][c];
            // the grid's first candidate is taken unconditionally, so an objective that overflows
            // (states beyond about 1e17 / sqrt(w)) still leaves a candidate of the grid, not the initial 1
            if ((g0 == 0 && j == 0) || F < fbest[c]) {
                fbest[c] = F;
                cbest[c] = cg[j][c];
            }
        }
    }
}

// NARROW: the plan has 2- or 3-bit containers (their unpack and pack paths are compiled in only
// then; the extra uniform branches cost the 4/6/8-bit step about 5%).
template <int DK, int DV, int MODE, int KG, bool NARROW>
__global__ void __launch_bounds__(nw_of(DK, DV) * 64, STEP_WAVES_PER_EU)
k_state(StepParams a) {
    using Sh = Shape<DK, DV>;
    constexpr int CPL = Sh::CPL, LPR = Sh::LPR, GR = Sh::GR, RPW = Sh::RPW, NW = Sh::NW;
    constexpr int GPW = Sh::GPW, EPL = Sh::EPL, NG = Sh::NG;
    constexpr bool kNeedOld = (MODE != kModePack);
    constexpr bool kUpdate = (MODE == kModeStep || MODE == kModeSplitA || MODE == kModeSplitB);
    constexpr bool kAccum = (MODE == kModeStep || MODE == kModeSplitA);
    __shared__ StepSmem<DK, DV> sm;

    // workgroup (x, y, z) = (head, request - b0, layer - layer0 - lz0): no index division
    const int h = block_idx();
    const int b = a.b0 + block_idy();
    const int lz = a.lz0 + block_idz();
    const int sid = (lz * a.batch + b) * a.n_heads + h;   // index of the state in the call's input arrays
    // Wave priority: high, except over the column fit's row loops (grid_round).  The other phases are chains
    // of dependent loads, LDS round trips and barriers, the row loops are long independent FMA chains; with
    // the SIMD's arbiter preferring the latency-bound waves, the fit's waves fill the gaps instead of
    // delaying them.
    __builtin_amdgcn_s_setprio(3);
    const int lh = (a.layer0 + lz) * a.n_heads + h;
    // per-state table values are the same for every lane: scalar loads, kept in scalar registers so
    // that the width dispatch below is a uniform branch
    const int slot = ld_const(a.slots + b);
    // a slot outside [0, n_slots) skips the state (uniform over the workgroup, before any barrier)
    if ((unsigned)slot >= (unsigned)a.n_slots) return;
    uint8_t* rec = a.pool + (uint64_t)slot * a.slot_bytes + ld_const(a.t.rec_off + lh);
    uint16_t* rs = reinterpret_cast<uint16_t*>(rec + ld_const(a.t.scale_off + lh));   // row factors, then column scales
    const int tid = thread_idx(), wave = uniform(tid >> 6), lane = tid & 63;
    const bool act = lane < LPR;
    const int col0 = lane * CPL;
    const uint8_t* gbits = a.t.grp_bits + (size_t)lh * NG;
    const uint32_t* goff = a.t.grp_off + (size_t)lh * NG;
    // the flags byte through a scalar dword load (the table is padded to whole dwords): a vector byte load
    // plus readfirstlane would make the wave wait for it before issuing the state's loads
    const int hflags = (int)((ld_const(reinterpret_cast<const uint32_t*>(a.t.head_flags) + (lh >> 2)) >>
                              (8 * (lh & 3))) & 0xFFu);

    // ---- every load of the state is issued here, at most one dependent level deep (the slot, then the
    // record): the packed groups and scales of the record; the plan's tables; the step's inputs, with
    // k, q and the per-row gate read in canonical order (not through the row permutation, which would
    // add a level) and staged through LDS.  Every lane loads 4 dwords of each group at its stride 2b
    // bytes: a 4- or 6-bit lane over-reads into its neighbour's data (or the record's scale vectors after
    // the last group), a 16-bit lane gets its first half.
    constexpr int EK = DK >= 64 ? DK / 64 : 1;   // canonical k / q / gate entries per lane
    float kc[EK], qc[EK], gc[EK], vv[CPL];
    if constexpr (kUpdate) {
        if (lane * EK < DK) {
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                kc[e] = a.k[(size_t)sid * DK + lane * EK + e];
                qc[e] = a.q[(size_t)sid * DK + lane * EK + e];
                gc[e] = (a.form == 1) ? a.gate[(size_t)sid * DK + lane * EK + e] : 1.f;
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if constexpr (MODE == kModeSplitB) vv[c] = act ? a.e_buf[e_index(a, lz, b, h) * DV + col0 + c] : 0.f;
            else vv[c] = act ? a.v[(size_t)sid * DV + col0 + c] : 0.f;
        }
    }
    uint32_t raw[GPW][4];
    int gb[GPW];
    if constexpr (GPW == 4 && NG % 4 == 0) {
        // the wave's four container widths are one aligned dword of the table: one scalar load
        const uint32_t w4 = ld_const(reinterpret_cast<const uint32_t*>(gbits + wave * GPW));
#pragma unroll
        for (int g = 0; g < GPW; ++g) gb[g] = (int)((w4 >> (8 * g)) & 0xFFu);
    } else {
#pragma unroll
        for (int g = 0; g < GPW; ++g) gb[g] = uniform((int)gbits[wave * GPW + g]);
    }
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        if constexpr (MODE != kModePack) {
            const uint8_t* gp = rec + ld_const(goff + wave * GPW + g);
            // one unconditional load per group (a branch here would make the compiler wait for it);
            // a 3-bit lane's dword sits at stride 4, its third-bit plane is loaded in phase 1
            if (act) load_dw<4>(gp + lane * ((NARROW && gb[g] == 3) ? 4 : 2 * gb[g]), raw[g]);
            else {
#pragma unroll
                for (int i = 0; i < 4; ++i) raw[g][i] = 0;
            }
        }
    }
    // the row tables and scales go out in the same batch as the groups, and one empty asm statement
    // takes every loaded word at once (the float conversions come after it): the wave waits for memory
    // once per state instead of once per dependent use
    uint32_t rbits_u = 16u, perm_u = 0u, rold_bits = 0x3C00u;   // binary16 1.0
    float2 wrow = make_float2(1.f, 1.f);
    if (lane < RPW) {
        const size_t t = (size_t)lh * DK + wave * RPW + lane;
        rbits_u = a.t.row_bits[t];
        wrow = a.t.row_wf[t];
        perm_u = a.t.perm[t];
        if constexpr (kNeedOld) rold_bits = rs[wave * RPW + lane];
    }
    // the lane's CPL column scales are adjacent binary16 values (4-byte aligned when CPL > 1): one load
    constexpr int CW = (CPL + 1) / 2;
    uint32_t cw[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) cw[i] = 0x3C003C00u;
    if constexpr (kNeedOld) {
        if (act) {
            if constexpr (CPL == 1) cw[0] = rs[DK + col0];
            else {
#pragma unroll
                for (int i = 0; i < CW; ++i) cw[i] = reinterpret_cast<const uint32_t*>(rs + DK + col0)[i];
            }
        }
    }
    __asm__ volatile("" : "+v"(rbits_u), "+v"(perm_u), "+v"(rold_bits), "+v"(wrow.x), "+v"(wrow.y));
#pragma unroll
    for (int i = 0; i < CW; ++i) __asm__ volatile("" : "+v"(cw[i]));
    const int rbits = (int)rbits_u, perm = (int)perm_u;
    float c_old[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        c_old[c] = kNeedOld ? h2f((cw[c / 2] >> (16 * (c % 2))) & 0xFFFFu) : 1.f;
        // converted once here: otherwise each use becomes a mixed-precision FMA, of the slow kind
        if constexpr (kNeedOld) __asm__ volatile("" : "+v"(c_old[c]));
    }
    const float rold = h2f(rold_bits);

    // ---- phase 0: per-row coefficients of this wave's rows (lane r < RPW takes row wave * RPW + r)
    if constexpr (kUpdate) {
        if (lane * EK < DK) {
#pragma unroll
            for (int e = 0; e < EK; ++e) {
                sm.stage[wave][0][lane * EK + e] = kc[e];
                sm.stage[wave][1][lane * EK + e] = qc[e];
                sm.stage[wave][2][lane * EK + e] = gc[e];
            }
        }
        wave_lds_sync();
    }
    float kq_part = 0.f;
    if (lane < RPW) {
        const int t = wave * RPW + lane;
        const bool piv = rbits == 16;
        sm.rb[t] = rbits;
        sm.wf[t] = wrow;
        if constexpr (kNeedOld) {
            float al = 1.f, kk = 0.f, qq = 0.f, bt = 0.f;
            if constexpr (kUpdate) {
                kk = sm.stage[wave][0][perm];
                qq = sm.stage[wave][1][perm];
                al = (a.form == 1) ? sm.stage[wave][2][perm] : ld_const(a.gate + sid);
                bt = ld_const(a.beta + sid);
            }
            // a pivot row stores its value as is: its coefficient is the gate alone
            const float A = piv ? al : al * rold;
            sm.acc[t] = make_float2(A * kk, A * qq);
            sm.upd[t] = make_float2(A, bt * kk);
            kq_part = kk * qq;
        }
    }
    if constexpr (kAccum) {
        kq_part = wave_sum(kq_part);
        if (lane == 0) sm.red[wave] = kq_part;
    }
    wave_lds_sync();

    float X[EPL];

    // ---- phase 1: unpack (c_j Q_ij on code rows, binary16 values on pivot rows), column sums k^T D S, q^T D S
    if constexpr (MODE == kModePack) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int t = wave * RPW + e / CPL;
            const int i = a.t.perm[(size_t)lh * DK + t];
            X[e] = act ? a.x_in[((size_t)sid * DK + i) * DV + col0 + (e % CPL)] : 0.f;
        }
    } else {
        float U1[CPL], P1[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) U1[c] = P1[c] = 0.f;
        bool same = true;
#pragma unroll
        for (int g = 1; g < GPW; ++g) same = same && gb[g] == gb[0];
        if (same && gb[0] == 6) unpack_acc_uniform<6, kAccum, Sh>(raw, X, sm, wave, U1, P1, rec, goff, lane, act, c_old);
        else if (same && gb[0] == 4) unpack_acc_uniform<4, kAccum, Sh>(raw, X, sm, wave, U1, P1, rec, goff, lane, act, c_old);
        else if (same && gb[0] == 8) unpack_acc_uniform<8, kAccum, Sh>(raw, X, sm, wave, U1, P1, rec, goff, lane, act, c_old);
        else if (NARROW && same && gb[0] == 2)
            unpack_acc_uniform<NARROW ? 2 : 4, kAccum, Sh>(raw, X, sm, wave, U1, P1, rec, goff, lane, act, c_old);
        else if (NARROW && same && gb[0] == 3)
            unpack_acc_uniform<NARROW ? 3 : 4, kAccum, Sh>(raw, X, sm, wave, U1, P1, rec, goff, lane, act, c_old);
        else if (same && gb[0] == 16) {
            // four 16-bit groups (a pivot head, or groups promoted by a pivot row): straight-line, with every
            // group's second half loaded first (through the per-group branches below these spill)
            uint32_t hi[GPW][4];
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                if (act) load_dw<4>(rec + ld_const(goff + wave * GPW + g) + lane * 32 + 16, hi[g]);
                else hi[g][0] = hi[g][1] = hi[g][2] = hi[g][3] = 0;
            }
            const bool all_pivot = !(hflags & kHasCodeRows);
#pragma unroll
            for (int g = 0; g < GPW; ++g) {
                float* xg = &X[16 * g];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t w = e < 8 ? raw[g][e >> 1] : hi[g][(e - 8) >> 1];
                    const uint32_t bits = (w >> (16 * (e & 1))) & 0xFFFFu;
                    if (all_pivot) xg[e] = h2f(bits);
                    else {
                        const int t = wave * RPW + (16 * g + e) / CPL;
                        xg[e] = (sm.rb[t] == 16) ? h2f(bits) : c_old[e % CPL] * (float)(int16_t)bits;
                    }
                }
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
        }
        else
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            // mixed widths: each branch accumulates its own group, so the compiler cannot gather the
            // coefficient reads of every group above the branches
            float* xg = &X[16 * g];
            if (gb[g] == 4) {
                unpack4f(raw[g], xg);
                scale_codes<CPL>(xg, c_old, 8.f);
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
            else if (NARROW && gb[g] == 2) {
                unpack2f(raw[g][0], xg);
                scale_codes<CPL>(xg, c_old, 2.f);
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
            else if (NARROW && gb[g] == 3) {
                const uint32_t hi = act ? *reinterpret_cast<const uint16_t*>(rec + ld_const(goff + wave * GPW + g) +
                                                                           LPR * 4 + lane * 2) : 0u;
                unpack3f(raw[g][0], hi, xg);
                scale_codes<CPL>(xg, c_old, 4.f);
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
            else if (gb[g] == 6) {
                unpack6f(raw[g], xg);
                scale_codes<CPL>(xg, c_old, 32.f);
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
            else if (gb[g] == 8) {
                unpack8(raw[g], xg);
                scale_codes<CPL>(xg, c_old, 128.f);
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
            else {
                uint32_t d16[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) d16[i] = raw[g][i];
                if (act) load_dw<4>(rec + ld_const(goff + wave * GPW + g) + lane * 32 + 16, d16 + 4);
                else d16[4] = d16[5] = d16[6] = d16[7] = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = wave * RPW + (16 * g + e) / CPL;
                    const uint32_t bits = (d16[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    xg[e] = (sm.rb[t] == 16) ? h2f(bits) : c_old[e % CPL] * (float)(int16_t)bits;
                }
                acc_group<kAccum, Sh>(sm, wave, g, xg, U1, P1);
            }
        }

        if constexpr (MODE == kModeUnpack) {
            // dequantized state r_i c_j Q_ij (binary16 value on pivot rows) -> canonical float layout
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int t = wave * RPW + e / CPL;
                const int c = e % CPL;
                const float s = sm.upd[t].x * X[e];   // r_i c_j Q_ij (1 times the value on pivot rows)
                const int i = a.t.perm[(size_t)lh * DK + t];
                if (act) a.x_out[((size_t)sid * DK + i) * DV + col0 + c] = s;
            }
            return;
        }

        float ecol[CPL];
        if constexpr (kAccum) {
            if (act) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    sm.part[wave][0][col0 + c] = U1[c];
                    sm.part[wave][1][col0 + c] = P1[c];
                }
            }
            __syncthreads();
            float kq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) kq += sm.red[w];
            const float bt = ld_const(a.beta + sid);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                float su = 0.f, sp = 0.f;
                if (act) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        su += sm.part[w][0][col0 + c];
                        sp += sm.part[w][1][col0 + c];
                    }
                }
                // su = k^T D S, sp = q^T D S
                const float e = act ? vv[c] - su : 0.f;
                ecol[c] = e;
                if (act && wave == 0) a.y[(size_t)sid * DV + col0 + c] = fmaf(bt * kq, e, sp);
                if constexpr (MODE == kModeSplitA) {
                    if (act && wave == 0) a.e_buf[e_index(a, lz, b, h) * DV + col0 + c] = e;
                }
            }
            if constexpr (MODE == kModeSplitA) return;
        } else {
            // split arrangement, second half: e = v - k^T D S comes from the first kernel
#pragma unroll
            for (int c = 0; c < CPL; ++c) ecol[c] = vv[c];
        }

        // ---- phase 2: the updated float state X = D S + beta k e^T in registers.  The rows' coefficients
        // come in blocks of RB rows, two rows per wide broadcast read, all of a block issued before its first
        // use (read one at a time, each would expose the LDS latency to a handful of FMAs).
        constexpr int RB = RPW < 16 ? RPW : 16;
#pragma unroll
        for (int r0 = 0; r0 < RPW; r0 += RB) {
            float4 uv[RB / 2];
#pragma unroll
            for (int i = 0; i < RB / 2; ++i) uv[i] = reinterpret_cast<const float4*>(sm.upd + wave * RPW + r0)[i];
            __asm__ volatile("" ::: "memory");
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float ux = (r % 2) ? uv[r / 2].z : uv[r / 2].x, uy = (r % 2) ? uv[r / 2].w : uv[r / 2].y;
#pragma unroll
                for (int c = 0; c < CPL; ++c) X[(r0 + r) * CPL + c] = fmaf(ux, X[(r0 + r) * CPL + c], uy * ecol[c]);
            }
        }
    }

    // ---- phase 3: row factors r_i = binary16(sqrt(max_j |X_ij| / w_i)) (rows are wave-uniform)
    {
        float rm[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            float m = fabsf(X[r * CPL]);
#pragma unroll
            for (int c = 1; c < CPL; ++c) m = fmaxf(m, fabsf(X[r * CPL + c]));
            rm[r] = act ? m : 0.f;
        }
        int row = 0;
        RowMax<LPR / 2, RPW>::run(rm, lane, row);
        if (act && (lane & (LPR / RPW - 1)) == 0) {
            const int t = wave * RPW + row;
            const int rbits = sm.rb[t];
            const bool piv = rbits == 16;
            const float m = rm[0];
            const float2 wf = sm.wf[t];
            const float qmax = piv ? 0.f : (float)((1 << (rbits - 1)) - 1);
            float rn = 1.f;
            // dual-axis sqrt(m / w); the ablation's per-row absmax m / qmax.  The hardware square root and
            // reciprocal are within a few float32 ulps, far inside the binary16 rounding they feed.
            if (!piv && m > 0.f)
                rn = scale_fp16(a.quant_mode == 0 ? __builtin_amdgcn_sqrtf(m * wf.x)
                                                  : m * __builtin_amdgcn_rcpf(qmax));
            sm.rn[t] = rn;
            const float sw = piv ? 0.f : wf.y * rn;
            const float irn = __builtin_amdgcn_rcpf(rn);
            sm.fit[t] = make_float4(sw, -0.5f * sw, 0.5f - qmax, irn);
            sm.ir[t] = irn;
            sm.iq[t] = piv ? 0.f : __builtin_amdgcn_rcpf(qmax);
            // the row's container width: its group's (wave-uniform values, selected per lane)
            int cb = gb[0];
#pragma unroll
            for (int g = 1; g < GPW; ++g) cb = row >= g * GR ? gb[g] : cb;
            const float mb = kMagic + (float)bias_of(cb);
            sm.fin[t] = make_float2(mb - qmax, mb + qmax);
        }
    }
    wave_lds_sync();

    // ---- phase 4: t = X / r_i (code rows; pivot rows have r = 1) and the column base
    float c0[CPL];
    {
        float c0p[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) c0p[c] = 0.f;
        // the rows' 1 / r_i in blocks of RB rows, four per wide broadcast read, and the groups' width
        // checks, all issued before the first use
        constexpr int RB = RPW < 16 ? RPW : 16;
        bool one_q[GPW];
        float iq0[GPW];
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            const int t0 = wave * RPW + g * GR;
            // rows are sorted by width, so a group whose first and last rows agree has one qmax
            one_q[g] = sm.rb[t0] == sm.rb[t0 + GR - 1];
            iq0[g] = sm.iq[t0];
        }
#pragma unroll
        for (int r0 = 0; r0 < RPW; r0 += RB) {
            float4 irv[RB / 4];
#pragma unroll
            for (int i = 0; i < RB / 4; ++i) irv[i] = reinterpret_cast<const float4*>(sm.ir + wave * RPW + r0)[i];
            __asm__ volatile("" ::: "memory");
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float4 v4 = irv[r / 4];
                const float ir = (r % 4 == 0) ? v4.x : (r % 4 == 1) ? v4.y : (r % 4 == 2) ? v4.z : v4.w;
#pragma unroll
                for (int c = 0; c < CPL; ++c) X[(r0 + r) * CPL + c] *= ir;
            }
        }
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            const int t0 = wave * RPW + g * GR;
            if (one_q[g]) {
                const float iq = iq0[g];
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    float mg = 0.f;
#pragma unroll
                    for (int r = 0; r < GR; ++r) mg = fmaxf(mg, fabsf(X[16 * g + r * CPL + c]));
                    c0p[c] = fmaxf(c0p[c], mg * iq);
                }
            } else {
#pragma unroll
                for (int r = 0; r < GR; ++r) {
                    const float iq = sm.iq[t0 + r];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) c0p[c] = fmaxf(c0p[c], fabsf(X[16 * g + r * CPL + c]) * iq);
                }
            }
        }
        if (act) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) sm.cmax[wave][col0 + c] = c0p[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float m = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) m = fmaxf(m, act ? sm.cmax[w][col0 + c] : 0.f);
            c0[c] = m;
        }
    }

    // ---- phase 5: column fit over the candidate grid, KG candidates per LDS round
    float cbest[CPL], fbest[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        cbest[c] = 1.f;
        fbest[c] = __builtin_inff();
    }
    if ((hflags & kHasCodeRows) && a.quant_mode == 0) {   // per-row absmax keeps every column scale at 1
        const int n_grid = a.n_grid;
        // with gamma = 1 no code can leave its range (|X / r| <= qmax c0 and the stored c is c0 rounded to
        // binary16, at most 2^-11 below it), so the first round skips the clamp of its first candidate when
        // grid[0] == 1 -- unless a column base exceeds the largest binary16 scale, which the stored c is
        // clamped to.  c0 is the workgroup's column maximum, so every wave takes the same branch.
        bool sat = false;
#pragma unroll
        for (int c = 0; c < CPL; ++c) sat = sat || c0[c] > 65504.f;
        if (a.unit_first && !__any(sat)) grid_round<Sh, KG, true>(sm, X, c0, a.grid, 0, n_grid, wave, lane, act, cbest, fbest);
        else grid_round<Sh, KG, false>(sm, X, c0, a.grid, 0, n_grid, wave, lane, act, cbest, fbest);
        for (int g0 = KG; g0 < n_grid; g0 += KG) {
            __syncthreads();   // every wave has read the previous round's partials
            grid_round<Sh, KG, false>(sm, X, c0, a.grid, g0, n_grid, wave, lane, act, cbest, fbest);
        }
    }
    float ic[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (!(c0[c] > 0.f)) cbest[c] = 1.f;      // all-zero column: scale 1, zero codes
        ic[c] = __builtin_amdgcn_rcpf(cbest[c]);
    }

    // ---- phase 6: round (magic-number RNE + clamp), pack and write back codes, row factors, column scales
    bool same6 = true;
#pragma unroll
    for (int g = 1; g < GPW; ++g) same6 = same6 && gb[g] == gb[0];
    if (same6 && gb[0] == 6) round_pack_uniform<6, Sh>(X, ic, sm, rec, goff, wave, lane, act);
    else if (same6 && gb[0] == 4) round_pack_uniform<4, Sh>(X, ic, sm, rec, goff, wave, lane, act);
    else if (same6 && gb[0] == 8) round_pack_uniform<8, Sh>(X, ic, sm, rec, goff, wave, lane, act);
    else if (NARROW && same6 && gb[0] == 2) round_pack_uniform<NARROW ? 2 : 4, Sh>(X, ic, sm, rec, goff, wave, lane, act);
    else if (NARROW && same6 && gb[0] == 3) round_pack_uniform<NARROW ? 3 : 4, Sh>(X, ic, sm, rec, goff, wave, lane, act);
    else if (same6 && gb[0] == 16 && !(hflags & kHasCodeRows)) {
        // a pivot head: every value stored as binary16, nothing to round to a code
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            uint32_t d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                d[i] = __builtin_amdgcn_perm(f2h_bits(fminf(fmaxf(X[16 * g + 2 * i + 1], -65504.f), 65504.f)),
                                             f2h_bits(fminf(fmaxf(X[16 * g + 2 * i], -65504.f), 65504.f)), 0x05040100u);
            if (act) store_dw<8>(rec + ld_const(goff + wave * GPW + g) + lane * 32, d);
        }
    }
    else
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
        const int gg = wave * GPW + g;
        const int sb = gb[g];
        uint8_t* gp = rec + ld_const(goff + gg);
        uint32_t d[8];
        float m[16];
        const float mb = kMagic + (float)bias_of(sb);
#pragma unroll
        for (int r = 0; r < GR; ++r) {
            const float2 bd = sm.fin[wave * RPW + g * GR + r];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int e = r * CPL + c;
                m[e] = med3(fmaf(X[16 * g + e], ic[c], mb), bd.x, bd.y);
            }
        }
        if (sb == 4) { pack4m(m, d); if (act) store_dw<2>(gp + lane * 8, d); }
        else if (NARROW && sb == 2) { pack2m(m, d); if (act) *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0]; }
        else if (NARROW && sb == 3) {
            pack3m(m, d, d + 1);
            if (act) {
                *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0];
                *reinterpret_cast<uint16_t*>(gp + LPR * 4 + lane * 2) = (uint16_t)d[1];
            }
        }
        else if (sb == 6) { pack6m(m, d); if (act) store_dw<3>(gp + lane * 12, d); }
        else if (sb == 8) { pack8m(m, d); if (act) store_dw<4>(gp + lane * 16, d); }
        else {
            uint32_t hv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int t = wave * RPW + (16 * g + e) / CPL;
                hv[e] = (sm.rb[t] == 16) ? f2h_bits(fminf(fmaxf(X[16 * g + e], -65504.f), 65504.f))
                                         : __float_as_uint(m[e]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) d[i] = __builtin_amdgcn_perm(hv[2 * i + 1], hv[2 * i], 0x05040100u);
            if (act) store_dw<8>(gp + lane * 32, d);
        }
    }
    if (lane < RPW) rs[wave * RPW + lane] = (uint16_t)f2h_bits(sm.rn[wave * RPW + lane]);
    if (wave == 0 && act) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) rs[DK + col0 + c] = (uint16_t)f2h_bits(cbest[c]);
    }
}

// ---------------------------------------------------------------- export / import

template <int DK, int DV, bool EXPORT>
__global__ void __launch_bounds__(nw_of(DK, DV) * 64)
k_codec(CodecParams a) {
    using Sh = Shape<DK, DV>;
    constexpr int CPL = Sh::CPL, LPR = Sh::LPR, RPW = Sh::RPW, GPW = Sh::GPW, NG = Sh::NG;
    const int sid = block_idx();
    const int h = sid % a.n_heads;
    const int b = (sid / a.n_heads) % a.batch;
    const int l = a.layer0 + sid / (a.n_heads * a.batch);
    const int lh = l * a.n_heads + h;
    const int slot = a.slots[b];
    if ((unsigned)slot >= (unsigned)a.n_slots) return;   // uniform over the workgroup: the state is skipped
    uint8_t* rec = a.pool + (uint64_t)slot * a.slot_bytes + a.t.rec_off[lh];
    uint16_t* rs = reinterpret_cast<uint16_t*>(rec + a.t.scale_off[lh]);
    const int tid = thread_idx(), wave = tid >> 6, lane = tid & 63;
    const int col0 = lane * CPL;
    const uint16_t* perm = a.t.perm + (size_t)lh * DK;
    const uint8_t* rbits = a.t.row_bits + (size_t)lh * DK;
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            const int gg = wave * GPW + g;
            const int sb = a.t.grp_bits[(size_t)lh * NG + gg];
            uint8_t* gp = rec + a.t.grp_off[(size_t)lh * NG + gg];
            const int bias = bias_of(sb);
            int code[16];
            uint32_t d[8];
            if constexpr (EXPORT) {
                if (sb == 16) {
                    load_dw<8>(gp + lane * 32, d);
#pragma unroll
                    for (int e = 0; e < 16; ++e) code[e] = (int)((d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                } else {
                    float f[16];
                    if (sb == 4) { load_dw<2>(gp + lane * 8, d); unpack4(d, f); }
                    else if (sb == 2) unpack2(*reinterpret_cast<const uint32_t*>(gp + lane * 4), f);
                    else if (sb == 3)
                        unpack3(*reinterpret_cast<const uint32_t*>(gp + lane * 4),
                                *reinterpret_cast<const uint16_t*>(gp + LPR * 4 + lane * 2), f);
                    else if (sb == 6) { load_dw<3>(gp + lane * 12, d); unpack6(d, f); }
                    else { load_dw<4>(gp + lane * 16, d); unpack8(d, f); }
#pragma unroll
                    for (int e = 0; e < 16; ++e) code[e] = (int)f[e] - bias;
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = wave * RPW + (16 * g + e) / CPL;
                    const int i = perm[t];
                    a.codes[((size_t)sid * DK + i) * DV + col0 + e % CPL] = (int16_t)code[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int t = wave * RPW + (16 * g + e) / CPL;
                    const int i = perm[t];
                    int v = a.codes[((size_t)sid * DK + i) * DV + col0 + e % CPL];
                    const int rb = rbits[t];
                    if (rb == 16) {
                        code[e] = v & 0xFFFF;
                    } else {
                        const int qm = (1 << (rb - 1)) - 1;
                        v = v < -qm ? -qm : (v > qm ? qm : v);
                        code[e] = (sb == 16) ? (v & 0xFFFF) : v + bias;
                    }
                }
                if (sb == 4) { pack4(code, d); store_dw<2>(gp + lane * 8, d); }
                else if (sb == 2) { pack2(code, d); *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0]; }
                else if (sb == 3) {
                    pack3(code, d, d + 1);
                    *reinterpret_cast<uint32_t*>(gp + lane * 4) = d[0];
                    *reinterpret_cast<uint16_t*>(gp + LPR * 4 + lane * 2) = (uint16_t)d[1];
                }
                else if (sb == 6) { pack6(code, d); store_dw<3>(gp + lane * 12, d); }
                else if (sb == 8) { pack8(code, d); store_dw<4>(gp + lane * 16, d); }
                else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) d[i] = (uint32_t)code[2 * i] | ((uint32_t)code[2 * i + 1] << 16);
                    store_dw<8>(gp + lane * 32, d);
                }
            }
        }
    }
    if (tid < DK) {
        const int i = perm[tid];
        if constexpr (EXPORT) a.r[(size_t)sid * DK + i] = rs[tid];
        else rs[tid] = a.r[(size_t)sid * DK + i];
    }
    for (int j = tid; j < DV; j += nw_of(DK, DV) * 64) {
        if constexpr (EXPORT) a.c[(size_t)sid * DV + j] = rs[DK + j];
        else rs[DK + j] = a.c[(size_t)sid * DV + j];
    }
}

// ---------------------------------------------------------------- comparators

struct CmpParams {
    int32_t n_heads, n_slots, layer0, batch, form;
    const int32_t* slots;
    int8_t* codes;
    float* scales;
    float* S;
    const float *q, *k, *v, *gate, *beta;
    float* y;
};

// Uniform INT8 per-row state and the unquantized FP32 state: same wave/lane
// mapping as the packed step.  The INT8 codes are stored group-interleaved like the
// pool's 8-bit containers (16 bytes per lane per group of 16 / CPL rows), the FP32
// state row-major.
// A lane's CPL adjacent entries of one row (CPL = 1, 2 or 4; the offset of the first is a
// multiple of CPL, so the access is naturally aligned).
// Byte offset of (state st, group g, lane) in the group-interleaved INT8 state.
template <class Sh>
__device__ __forceinline__ size_t cmp_group_offset(size_t st, int g, int lane) {
    return ((st * Sh::NG + (size_t)g) * Sh::LPR + (size_t)lane) * 16;
}
template <int CPL>
__device__ __forceinline__ void cmp_load_f32(const float* p, bool act, float* x) {
    if constexpr (CPL == 1) x[0] = act ? *p : 0.f;
    else if constexpr (CPL == 2) {
        const float2 v = act ? *reinterpret_cast<const float2*>(p) : make_float2(0.f, 0.f);
        x[0] = v.x; x[1] = v.y;
    } else {
        const float4 v = act ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
}
template <int CPL>
__device__ __forceinline__ void cmp_store_f32(float* p, const float* x) {
    if constexpr (CPL == 1) *p = x[0];
    else if constexpr (CPL == 2) *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    else *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

template <int DK, int DV, bool INT8>
__global__ void __launch_bounds__(nw_of(DK, DV) * 64)
k_cmp(CmpParams a) {
    using Sh = Shape<DK, DV>;
    constexpr int CPL = Sh::CPL, LPR = Sh::LPR, RPW = Sh::RPW, NW = Sh::NW, EPL = Sh::EPL;
    constexpr int GR = Sh::GR, GPW = Sh::GPW;
    __shared__ float s_ck[DK], s_cq[DK], s_al[DK], s_bk[DK], s_sc[DK], s_so[DK];
    __shared__ float s_part[NW][2][DV];
    __shared__ float s_red[NW];
    const int sid = block_idx();
    const int h = sid % a.n_heads;
    const int b = (sid / a.n_heads) % a.batch;
    const int ll = sid / (a.n_heads * a.batch);
    const int slot = a.slots[b];
    if ((unsigned)slot >= (unsigned)a.n_slots) return;   // uniform over the workgroup, before any barrier
    const size_t st = ((size_t)(a.layer0 + ll) * a.n_slots + slot) * a.n_heads + h;
    const int tid = thread_idx(), wave = tid >> 6, lane = tid & 63;
    const bool act = lane < LPR;
    const int col0 = lane * CPL;
    float kq = 0.f;
    if (tid < DK) {
        const float kk = a.k[(size_t)sid * DK + tid], qq = a.q[(size_t)sid * DK + tid];
        const float al = (a.form == 1) ? a.gate[(size_t)sid * DK + tid] : a.gate[sid];
        s_ck[tid] = al * kk;
        s_cq[tid] = al * qq;
        s_al[tid] = al;
        s_bk[tid] = a.beta[sid] * kk;
        if constexpr (INT8) s_so[tid] = a.scales[st * DK + tid];
        kq = kk * qq;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kq += __shfl_xor(kq, d);
    if (lane == 0) s_red[wave] = kq;
    __syncthreads();
    float X[EPL];
    float U[CPL], P[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) U[c] = P[c] = 0.f;
    if constexpr (INT8) {
        // one 16-byte access per lane and group; codes + 128 -> float, then s_i Q_ij with one exact-offset FMA
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
            if (act) load_dw<4>(reinterpret_cast<const uint8_t*>(a.codes) + cmp_group_offset<Sh>(st, wave * GPW + g, lane), d);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] ^= 0x80808080u;
            unpack8(d, &X[16 * g]);
#pragma unroll
            for (int r = 0; r < GR; ++r) {
                const float so = s_so[wave * RPW + g * GR + r];
#pragma unroll
                for (int c = 0; c < CPL; ++c) X[16 * g + r * CPL + c] = fmaf(X[16 * g + r * CPL + c], so, -128.f * so);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int t = wave * RPW + r;
        // FP32: the lane's CPL adjacent entries of the row in one access
        if constexpr (!INT8) cmp_load_f32<CPL>(a.S + (st * DK + t) * DV + col0, act, &X[r * CPL]);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            U[c] = fmaf(s_ck[t], X[r * CPL + c], U[c]);
            P[c] = fmaf(s_cq[t], X[r * CPL + c], P[c]);
        }
    }
    if (act) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            s_part[wave][0][col0 + c] = U[c];
            s_part[wave][1][col0 + c] = P[c];
        }
    }
    __syncthreads();
    float kqs = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) kqs += s_red[w];
    float ecol[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        float su = 0.f, sp = 0.f;
        if (act) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                su += s_part[w][0][col0 + c];
                sp += s_part[w][1][col0 + c];
            }
        }
        const float e = act ? a.v[(size_t)sid * DV + col0 + c] - su : 0.f;
        ecol[c] = e;
        if (act && wave == 0) a.y[(size_t)sid * DV + col0 + c] = fmaf(a.beta[sid] * kqs, e, sp);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int t = wave * RPW + r;
#pragma unroll
        for (int c = 0; c < CPL; ++c) X[r * CPL + c] = fmaf(s_al[t], X[r * CPL + c], s_bk[t] * ecol[c]);
    }
    if constexpr (!INT8) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int t = wave * RPW + r;
            if (act) cmp_store_f32<CPL>(a.S + (st * DK + t) * DV + col0, &X[r * CPL]);
        }
        return;
    } else {
        float rm[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            float m = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) m = fmaxf(m, fabsf(X[r * CPL + c]));
            rm[r] = act ? m : 0.f;
        }
        int row = 0;
        RowMax<LPR / 2, RPW>::run(rm, lane, row);
        if (act && (lane & (LPR / RPW - 1)) == 0) {
            const int t = wave * RPW + row;
            const float s = rm[0] > 0.f ? rm[0] / 127.f : 1.f;
            s_sc[t] = 1.f / s;   // one division per row, by the lane that holds the row maximum
            a.scales[st * DK + t] = s;
        }
        __syncthreads();
        // Q = clamp(rint(X / s), +-127): magic-number rounding with the +128 offset, packed by bytes
        constexpr float mb = kMagic + 128.f;
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
            float m[16];
#pragma unroll
            for (int r = 0; r < GR; ++r) {
                const float inv = s_sc[wave * RPW + g * GR + r];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    m[r * CPL + c] = med3(fmaf(X[16 * g + r * CPL + c], inv, mb), mb - 127.f, mb + 127.f);
            }
            uint32_t d[4];
            pack8m(m, d);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] ^= 0x80808080u;
            if (act) store_dw<4>(reinterpret_cast<uint8_t*>(a.codes) + cmp_group_offset<Sh>(st, wave * GPW + g, lane), d);
        }
    }
}

// Streaming copy for the achievable-bandwidth reference: each workgroup copies kCopyUnroll x 256
// consecutive 16-byte vectors once, all loads before the stores, non-temporal both ways (5.85 TB/s
// on 4 GiB against 4.75 for a grid-stride loop of single 16-byte copies).
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(kCopyThreads)
k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
    const size_t base = (size_t)block_idx() * (kCopyUnroll * kCopyThreads) + thread_idx();
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const size_t i = base + (size_t)u * kCopyThreads;
        if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const size_t i = base + (size_t)u * kCopyThreads;
        if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
}

// ---------------------------------------------------------------- launchers

template <int DK, int DV, int KG, bool NARROW>
static hipError_t launch_state_kgn(int mode, const StepParams& p, dim3 grid, hipStream_t s) {
    const dim3 blk(Shape<DK, DV>::NW * 64);
    switch (mode) {
        case kModeStep: k_state<DK, DV, kModeStep, KG, NARROW><<<grid, blk, 0, s>>>(p); break;
        case kModePack: k_state<DK, DV, kModePack, KG, NARROW><<<grid, blk, 0, s>>>(p); break;
        case kModeUnpack: k_state<DK, DV, kModeUnpack, 1, NARROW><<<grid, blk, 0, s>>>(p); break;
        case kModeSplitA: k_state<DK, DV, kModeSplitA, 1, NARROW><<<grid, blk, 0, s>>>(p); break;
        case kModeSplitB: k_state<DK, DV, kModeSplitB, KG, NARROW><<<grid, blk, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DK, int DV, int KG>
static hipError_t launch_state_kg(int mode, const StepParams& p, dim3 grid, hipStream_t s) {
    return p.narrow ? launch_state_kgn<DK, DV, KG, true>(mode, p, grid, s)
                    : launch_state_kgn<DK, DV, KG, false>(mode, p, grid, s);
}

// candidates per LDS round: one or two when the grid is that small, otherwise four; two for
// four columns per lane (d_v = 256), where four would spill (a last round with fewer candidates
// repeats the final one, which cannot change the choice)
template <int DK, int DV>
static hipError_t launch_state_t(int mode, const StepParams& p, dim3 grid, hipStream_t s) {
    if (p.n_grid == 1) return launch_state_kg<DK, DV, 1>(mode, p, grid, s);
    if (p.n_grid == 2 || Shape<DK, DV>::CPL > 2) return launch_state_kg<DK, DV, 2>(mode, p, grid, s);
    return launch_state_kg<DK, DV, 4>(mode, p, grid, s);
}

#define SQ_SHAPES(X) X(16, 16) X(64, 64) X(128, 128) X(128, 256)

bool shape_compiled(int dk, int dv) {
#define SQ_CASE(a, b) if (dk == a && dv == b) return true;
    SQ_SHAPES(SQ_CASE)
#undef SQ_CASE
    return false;
}

int compiled_shapes(int32_t* out, int max_pairs) {
    int n = 0;
#define SQ_CASE(a, b) if (n < max_pairs && out) { out[2 * n] = a; out[2 * n + 1] = b; } ++n;
    SQ_SHAPES(SQ_CASE)
#undef SQ_CASE
    return n;
}

hipError_t launch_state(int dk, int dv, int mode, const StepParams& p, int n_b, int n_z, hipStream_t s) {
    if (n_b <= 0 || n_z <= 0 || p.n_heads <= 0) return hipSuccess;
    if (n_b > 65535 || n_z > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.n_heads, (unsigned)n_b, (unsigned)n_z);
#define SQ_CASE(a, b) if (dk == a && dv == b) return launch_state_t<a, b>(mode, p, grid, s);
    SQ_SHAPES(SQ_CASE)
#undef SQ_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_codec(int dk, int dv, bool do_export, const CodecParams& p, int n_states, hipStream_t s) {
    if (n_states <= 0) return hipSuccess;
#define SQ_CASE(a, b)                                                                                  \
    if (dk == a && dv == b) {                                                                          \
        const dim3 blk(Shape<a, b>::NW * 64);                                                          \
        if (do_export) k_codec<a, b, true><<<n_states, blk, 0, s>>>(p);                               \
        else k_codec<a, b, false><<<n_states, blk, 0, s>>>(p);                                        \
        return hipGetLastError();                                                                      \
    }
    SQ_SHAPES(SQ_CASE)
#undef SQ_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_cmp(int dk, int dv, bool int8, int form, int n_heads, int n_slots, int layer0, int n_layers,
                      int batch, const int32_t* slots, int8_t* codes, float* scales, float* S, const float* q,
                      const float* k, const float* v, const float* gate, const float* beta, float* y,
                      hipStream_t s) {
    CmpParams p{n_heads, n_slots, layer0, batch, form, slots, codes, scales, S, q, k, v, gate, beta, y};
    const int n_states = n_layers * batch * n_heads;
    if (n_states <= 0) return hipSuccess;
#define SQ_CASE(a, b)                                                                                  \
    if (dk == a && dv == b) {                                                                          \
        const dim3 blk(Shape<a, b>::NW * 64);                                                          \
        if (int8) k_cmp<a, b, true><<<n_states, blk, 0, s>>>(p);                                      \
        else k_cmp<a, b, false><<<n_states, blk, 0, s>>>(p);                                          \
        return hipGetLastError();                                                                      \
    }
    SQ_SHAPES(SQ_CASE)
#undef SQ_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_copy(const void* src, void* dst, size_t n_bytes, hipStream_t s) {
    const size_t n = n_bytes / 16;
    if (n == 0) return hipSuccess;
    const size_t per = size_t(kCopyUnroll) * kCopyThreads;
    const size_t blocks = (n + per - 1) / per;
    if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
    k_copy<<<dim3((unsigned)blocks), dim3(kCopyThreads), 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fixed split scratch
// e = v - k^T D S of every state of one allocation-free split call, one copy per GPU for the life of
// the process.  Host code never passes the array's own name (on the host it is a stand-in, not a
// device address) but the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) float scratch[kStaticScratchFloats];

constexpr int kScratchDevices = 64;

hipError_t static_scratch(float** out) {
    static std::mutex mu;
    static float* ptr[kScratchDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* d = nullptr;
        e = hipGetSymbolAddress(&d, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptr[dev] = static_cast<float*>(d);
    }
    *out = ptr[dev];
    return hipSuccess;
}

}  // namespace sq
