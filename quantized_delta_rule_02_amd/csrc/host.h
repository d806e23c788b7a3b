// Host-side runtime objects behind the C ABI (plan, pool) and shared helpers.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/stepq.h"
#include "internal.h"

struct sq_plan {
    // configuration (scalars of sq_plan_cfg; host pointers are not kept)
    int32_t form, unit, L, H, dk, dv;
    std::vector<int32_t> widths;     // ascending
    int32_t budget_milli, pivot_ppm;
    int32_t quantizer = SQ_QUANT_DUAL_AXIS;
    std::vector<float> grid;
    // planner results, canonical order
    std::vector<double> lbar, lifetime, distortion;  // [U], [U], [U][n_widths]
    std::vector<int32_t> unit_bits;                  // [U] (16 = pivot)
    std::vector<int32_t> row_bits;                   // [L][H][dk]
    std::vector<float> impact;                       // [L][H][dk]
    // layout (see internal.h)
    std::vector<uint16_t> perm;                      // [LH][dk]
    std::vector<uint8_t> srow_bits;                  // [LH][dk]
    std::vector<float> srow_wf;                      // [LH][dk][2]: 1 / w and sqrt(w) of each storage row
    std::vector<uint8_t> grp_bits;                   // [LH][NG]
    std::vector<uint32_t> grp_off;                   // [LH][NG]
    std::vector<uint32_t> scale_off;                 // [LH]
    std::vector<uint64_t> rec_off;                   // [LH]
    std::vector<uint8_t> head_flags;                 // [LH]
    uint64_t slot_bytes = 0;
    uint64_t plan_id = 0;                            // identifies the plan a pool was bound to

    int n_units() const { return L * H * (unit == SQ_UNIT_HEAD ? 1 : dk); }
    int ng() const { return sq::ng_of(dk, dv); }
};

namespace sq {

void set_error(const char* fmt, ...);
bool shape_supported(int dk, int dv);

// Planner (planner.cpp).  Returns SQ_OK or an error (message via set_error).
sq_status run_planner(const sq_plan_cfg& cfg, sq_plan& plan);
sq_status build_layout(sq_plan& plan);
void generate_calib(uint64_t seed, int layer, int head, int n_seg, int seg_len, int dk, int dv,
                    float* q, float* k, float* v, float* beta);

// binary16 helpers on the host (round to nearest even, saturating)
double fp16_round_host(double x);
uint16_t fp16_bits_host(double x);   // x must already be a binary16 value

}  // namespace sq
