// Internal definitions shared by the host runtime and the gfx950 kernels.
//
// Pool layout (one record per (layer, head) inside each slot):
//
//   Every state S (d_k x d_v) is processed by NW waves.  Wave w owns the RPW
//   storage rows [w*RPW, (w+1)*RPW); lane l (< LPR) owns the CPL adjacent value
//   columns [l*CPL, (l+1)*CPL).  A "group" is GR = 16/CPL consecutive storage
//   rows, i.e. 16 entries per lane.  Inside a record the groups come first, in
//   storage-row order; group g of width b (2, 3, 4, 6, 8 or 16 bits) occupies
//   LPR * 2b bytes, lane l's 16 entries at byte l*2b (b/2 dwords; for b = 3 a
//   dword at l*4 and a 16-bit plane at LPR*4 + l*2), so one wave reads or
//   writes a group with contiguous vector accesses.  Entry e = r*CPL + c
//   (r = row inside the group, c = column inside the lane) is placed as:
//     2-bit : bits 8(e%4) + 2(e/4) of the dword         (Q + 2)
//     3-bit : low two bits as for 2-bit; the third bit at bit 4(e%4) + e/4 of
//             the 16-bit plane                          (Q + 4)
//     8-bit : byte e                                   (biased code Q + 128)
//     4-bit : dword e/8, byte e%4, high nibble if (e%8) >= 4  (Q + 8)
//     6-bit : e < 12: low 6 bits of byte (e%4) of dword e/4;
//             e >= 12: bits 0-1 / 2-3 / 4-5 in the top 2 bits of byte (e-12)
//             of dwords 0 / 1 / 2                      (Q + 32)
//     16-bit: half e%2 of dword e/2: the binary16 value on pivot rows,
//             the two's-complement code on code rows (no bias)
//   After the groups: binary16 row factors [d_k] (storage order), binary16
//   column scales [d_v]; the record is padded to 256 bytes.
//
//   Storage row order: pivot rows first, then rows by descending width, each
//   width in canonical order.  A group's storage width is the widest of its rows (a row
//   keeps its own code range; only the container is wider), so at most a few
//   groups per head use a wider container than their rows need.
#pragma once
#include <stdint.h>
#include <hip/hip_vector_types.h>

namespace sq {

constexpr int kWave = 64;

constexpr int cpl_of(int dv) { return dv >= 64 ? dv / 64 : 1; }           // columns per lane
constexpr int lpr_of(int dv) { return dv / cpl_of(dv); }                   // active lanes
constexpr int gr_of(int dv) { return 16 / cpl_of(dv); }                    // rows per group
constexpr int rpw_of(int dk, int dv) { return (64 / cpl_of(dv)) < dk ? 64 / cpl_of(dv) : dk; }
constexpr int nw_of(int dk, int dv) { return dk / rpw_of(dk, dv); }        // waves per state
constexpr int ng_of(int dk, int dv) { return dk / gr_of(dv); }             // groups per state

inline int group_bytes(int dv, int bits) { return lpr_of(dv) * 2 * bits; }

constexpr int kMaxGrid = 8;
// floats of the fixed split scratch (32 MiB per GPU) behind the allocation-free split step
constexpr int64_t kStaticScratchFloats = int64_t(8) << 20;

// Head flags
constexpr uint8_t kHasCodeRows = 1;
constexpr uint8_t kHasPivotRows = 2;

// Device-resident layout tables of a bound pool, indexed by lh = layer * H + head.
struct DevTables {
    const uint64_t* rec_off;    // [LH] byte offset of the record inside a slot
    const uint32_t* grp_off;    // [LH][NG] byte offset of each group inside the record
    const uint8_t* grp_bits;    // [LH][NG] container width 2/3/4/6/8/16
    const uint32_t* scale_off;  // [LH] byte offset of the binary16 row factors (column scales follow)
    const uint16_t* perm;       // [LH][d_k] storage row -> canonical row
    const uint8_t* row_bits;    // [LH][d_k] code width of the row, 16 = pivot (storage order)
    const float2* row_wf;       // [LH][d_k] 1 / w and sqrt(w) of the row-impact score w (storage order)
    const uint8_t* head_flags;  // [LH]
};

enum : int { kModeStep = 0, kModePack = 1, kModeUnpack = 2, kModeSplitA = 3, kModeSplitB = 4 };

struct StepParams {
    uint8_t* pool;
    uint64_t slot_bytes;
    DevTables t;
    int32_t n_heads, layer0, n_layers, batch, form;
    int32_t n_slots;     // slots of the pool: a request whose slot is outside [0, n_slots) is skipped
    const int32_t* slots;
    const float* q;
    const float* k;
    const float* v;
    const float* gate;
    const float* beta;
    float* y;
    const float* x_in;   // pack: float states [state][d_k][d_v] (canonical rows)
    float* x_out;        // unpack: float states
    float* e_buf;        // split arrangement: v - k^T D S, [layer][request index][head][d_v] from layer0
    int64_t e_layer_stride;  // split arrangement: states per layer of e_buf (n_slots * n_heads)
    int32_t lz0;         // first layer of the launch, relative to layer0 (split arrangement: of the chunk)
    int32_t b0;          // first request of the launch
    int32_t n_grid;
    int32_t unit_first;  // grid[0] == 1: the first candidate needs no clamp
    int32_t quant_mode;  // SQ_QUANT_DUAL_AXIS or SQ_QUANT_ROW_ABSMAX
    int32_t narrow;      // the plan has 2- or 3-bit containers
    float grid[kMaxGrid];
};

struct CodecParams {
    uint8_t* pool;
    uint64_t slot_bytes;
    DevTables t;
    int32_t n_heads, layer0, batch;
    int32_t n_slots;     // a request whose slot is outside [0, n_slots) is skipped
    const int32_t* slots;
    int16_t* codes;      // canonical [state][d_k][d_v]
    uint16_t* r;         // [state][d_k]
    uint16_t* c;         // [state][d_v]
};

}  // namespace sq
