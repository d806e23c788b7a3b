/*
 * stepq.h -- C ABI of the MI355X (gfx950) quantized gated-delta state step.
 *
 * The library implements the decode-time hot path of STEPQuant (Yao et al.,
 * 2026, "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State
 * Quantization"): every (request, layer, head) recurrent state S (d_k x d_v)
 * lives in a packed pool as mixed-width integer codes with a binary16 factor
 * per key row and a binary16 scale per value column, plus binary16 "pivot"
 * rows kept unquantized.  One step dequantizes the state, applies the gated
 * delta update, emits the readout y = X^T q from the float state, then refits
 * the row factors and column scales and packs the state back.
 *
 * Passages the calls follow (STEPQuant pages):
 *   - rcap.io post, decode-step pseudocode: unpack -> gated delta update ->
 *     readout before requantization -> row scales sqrt(row_mag)/sqrt(impact)
 *     -> weighted column fit -> quantize at each unit's width.
 *   - hyper.ai summary, section 方法 (Method): lifetime-aware bit allocation and
 *     FP16 pivot selection run offline; a fused kernel does chunked state
 *     reconstruction, the delta update and the readout; the dual-axis fit and
 *     packed write-back run on a separate stream, keeping the state compressed
 *     between tokens.
 *
 * Conventions
 *   - All sizes are element counts unless named *_bytes.
 *   - "d_" prefixed pointers are device pointers (HIP device memory on the
 *     current device); "h_" or unprefixed pointers in sq_plan_cfg are host.
 *   - Streams are passed as void* and hold a hipStream_t (NULL = the null stream).
 *   - Per-step arrays are laid out [n_layers][batch][H][d] (row-major, fp32).
 *     Device inputs must be finite (the kernels run with IEEE mode off and do
 *     not screen NaN or infinity); a non-finite input leaves the touched states
 *     unspecified, never memory outside them.
 *   - A call over an empty range (batch = 0 or n_layers = 0) validates its
 *     sizes and returns SQ_OK without touching any array (they may be NULL).
 *   - Host threads: a plan is read-only after creation and may be shared; calls
 *     on one pool may come from several threads (the split arrangement
 *     serializes its own set-up per pool).  Device work that touches the same
 *     slots must still be ordered by the caller (streams, events).
 *   - Every call validates its arguments on the host before enqueuing work and
 *     returns a negative sq_status on failure, with a message available from
 *     sq_last_error() on the calling thread.  Device work is asynchronous: a
 *     device fault surfaces at the caller's next synchronization.  No C++
 *     exception crosses this boundary.
 */
#ifndef STEPQ_H
#define STEPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sq_status;
#define SQ_OK                 0
#define SQ_ERR_ARG           -1   /* null pointer, bad enum, bad count */
#define SQ_ERR_SHAPE         -2   /* sizes inconsistent with the plan or the buffer */
#define SQ_ERR_UNSUPPORTED   -3   /* (d_k, d_v), width or grid size not compiled in */
#define SQ_ERR_SLOT          -4   /* slot out of range or repeated (validate mode) */
#define SQ_ERR_PLAN_MISMATCH -5   /* pool bound to another plan / layer range out of plan */
#define SQ_ERR_NOMEM         -6   /* host or device allocation failed */
#define SQ_ERR_HIP           -7   /* a HIP runtime call failed */

#define SQ_FORM_GDN 0             /* one retention gate per head: D = alpha I        */
#define SQ_FORM_KDA 1             /* one retention gate per key row: D = diag(alpha) */
#define SQ_UNIT_HEAD 0            /* allocation unit: a whole head state             */
#define SQ_UNIT_ROW  1            /* allocation unit: one key row of a head state    */
#define SQ_QUANT_DUAL_AXIS 0      /* row factors sqrt(m / w) + impact-weighted column fit (the method) */
#define SQ_QUANT_ROW_ABSMAX 1     /* per-row absmax r = m / qmax, column scales 1 (ablation: no fit) */

#define SQ_MAX_WIDTHS 8
#define SQ_MAX_GRID   8
#define SQ_PIVOT_BITS 16          /* width reported for a pivot (binary16) unit/row  */

/* Plan configuration (host memory; read during sq_plan_create only). */
typedef struct sq_plan_cfg {
    int32_t form;                 /* SQ_FORM_GDN or SQ_FORM_KDA */
    int32_t unit;                 /* SQ_UNIT_HEAD or SQ_UNIT_ROW */
    int32_t n_layers, n_heads, d_k, d_v;
    int32_t n_widths;             /* candidate code widths, each in {2, 3, 4, 6, 8} */
    int32_t widths[SQ_MAX_WIDTHS];
    int32_t budget_milli;         /* average bits x 1000 over non-pivot units */
    int32_t pivot_ppm;            /* pivot units: ceil(pivot_ppm * units / 1e6) */
    int32_t n_grid;               /* column-scale candidates gamma (1..8), relative to the column base */
    float   grid[SQ_MAX_GRID];
    const float* gate;            /* alpha per unit for calibration: [L][H] (GDN) or [L][H][d_k] (KDA) */
    const float* impact;          /* row-impact score w [L][H][d_k]; NULL = estimate from the traces */
    const int32_t* unit_bits;     /* optional fixed allocation per unit (a candidate width, 16 = pivot); NULL = plan */
    /* calibration traces; NULL q = draw them with the built-in Philox-4x32-10 generator */
    const float* calib_q;         /* [L][H][S][T][d_k] */
    const float* calib_k;         /* [L][H][S][T][d_k] */
    const float* calib_v;         /* [L][H][S][T][d_v] */
    const float* calib_beta;      /* [L][H][S][T] */
    uint64_t calib_seed;
    int32_t calib_segments;       /* S */
    int32_t calib_len;            /* T */
    int32_t n_threads;            /* planner threads; 0 = all hardware threads */
    int32_t quantizer;            /* SQ_QUANT_DUAL_AXIS (0) or SQ_QUANT_ROW_ABSMAX (1; rcap.io post, the
                                     ablation paragraph: the allocation without the dual-axis fit) */
} sq_plan_cfg;

typedef struct sq_plan sq_plan;   /* host-side plan (opaque) */
typedef struct sq_pool sq_pool;   /* a device pool bound to a plan (opaque) */

/* Summary of a plan's layout. */
typedef struct sq_plan_desc {
    int32_t n_layers, n_heads, d_k, d_v, form, unit, n_units, n_pivot_units;
    int32_t n_grid;
    int32_t n_widths;
    int32_t widths[SQ_MAX_WIDTHS];/* candidate widths, ascending */
    uint64_t slot_bytes;          /* bytes of one slot (all layers and heads of one request) */
    double code_bits_per_entry;   /* allocated bits per state entry, pivots at 16, scales excluded */
    double stored_bits_per_entry; /* slot_bytes * 8 / (L * H * d_k * d_v): codes + scales + padding */
    double compression_vs_fp32;   /* 32 / stored_bits_per_entry */
    int32_t quantizer;            /* SQ_QUANT_* */
} sq_plan_desc;

/* ---- plan (CPU) --------------------------------------------------------
 * Offline planner (hyper.ai summary, 方法, lifetime-aware bit allocation and
 * the row-impact score): lifetime weight per unit from its mean log retention,
 * reconstruction distortion at each candidate width on calibration snapshots,
 * FP16 pivots for the riskiest units, an exact budgeted allocation of widths,
 * and the packed layout.  Runs on the host only; the plan owns host memory.
 * Errors: SQ_ERR_ARG / SQ_ERR_UNSUPPORTED on bad configuration. */
sq_status sq_plan_create(const sq_plan_cfg* cfg, sq_plan** out);
void      sq_plan_destroy(sq_plan* plan);
sq_status sq_plan_describe(const sq_plan* plan, sq_plan_desc* out);
/* Per-unit planner quantities (host arrays of n_units; any pointer may be NULL):
 * mean log retention, lifetime weight, distortion [n_units][n_widths], width (16 = pivot). */
sq_status sq_plan_units(const sq_plan* plan, double* lbar, double* lifetime, double* distortion,
                        int32_t* unit_bits);
/* Per-row tables in canonical row order (host arrays [L][H][d_k]; any may be NULL):
 * quantization width (16 = pivot row) and the row-impact score used by the step. */
sq_status sq_plan_rows(const sq_plan* plan, int32_t* row_bits, float* impact);
/* Serialize to / restore from a byte buffer (host).  With buf == NULL, *bytes
 * receives the size needed.  sq_plan_load validates the buffer. */
sq_status sq_plan_save(const sq_plan* plan, void* buf, size_t* bytes);
sq_status sq_plan_load(const void* buf, size_t bytes, sq_plan** out);
/* The built-in calibration generator for one (layer, head): q, k [S][T][d_k]
 * (unit L2 norm), v [S][T][d_v], beta [S][T] (host arrays, fp32). */
sq_status sq_calib_generate(uint64_t seed, int32_t layer, int32_t head, int32_t n_seg,
                            int32_t seg_len, int32_t d_k, int32_t d_v,
                            float* q, float* k, float* v, float* beta);

/* ---- pool (device) -----------------------------------------------------
 * The caller owns the pool memory: n_slots slots of desc.slot_bytes each.  A
 * request's state for (layer l, head h) lives in its slot at the plan's
 * offset for (l, h).  Binding copies the plan's layout tables to the current
 * device (the pool object owns those small allocations until destroyed); calls
 * on the pool must run with that device current, otherwise SQ_ERR_ARG.  A slot
 * whose bytes are all zero holds the zero state (its scales are 0), so a new
 * request's slot may be cleared instead of imported.  Every call below that
 * takes d_slots skips a request whose slot lies outside [0, n_slots): no pool
 * byte is touched for it and its outputs keep their previous contents
 * (sq_state_step with SQ_STEP_VALIDATE returns SQ_ERR_SLOT instead). */
sq_status sq_pool_bytes(const sq_plan* plan, int32_t n_slots, size_t* bytes);
sq_status sq_pool_create(const sq_plan* plan, void* d_pool, size_t pool_bytes, int32_t n_slots,
                         sq_pool** out);
void      sq_pool_destroy(sq_pool* pool);
/* The same three calls under the names the method's decode-step interface is usually described
 * with: sq_plan_info = sq_plan_describe, sq_pool_bind = sq_pool_create (the caller's device buffer
 * is bound, not allocated), sq_pool_release = sq_pool_destroy. */
sq_status sq_plan_info(const sq_plan* plan, sq_plan_desc* out);
sq_status sq_pool_bind(const sq_plan* plan, void* d_pool, size_t pool_bytes, int32_t n_slots,
                       sq_pool** out);
void      sq_pool_release(sq_pool* pool);

#define SQ_STEP_SPLIT    1u       /* two kernels: readout on stream_main, fit + pack on stream_aux */
#define SQ_STEP_VALIDATE 2u       /* copy the slot list to the host and check range and uniqueness */
#define SQ_STEP_NO_JOIN  4u       /* with SQ_STEP_SPLIT: return without making stream_main wait for stream_aux */

/* ---- state_step --------------------------------------------------------
 * One decode step for batch requests over layers [layer0, layer0 + n_layers)
 * and every head (rcap.io post, decode-step pseudocode; hyper.ai 方法):
 *   S = unpack(codes, r, c, pivots);  X = D S + beta k (v^T - k^T D S);
 *   y = X^T q (written to d_y before requantization);
 *   r = binary16(sqrt(rowmax|X| / w));  c = argmin over the grid of the
 *   impact-weighted reconstruction error;  codes = clamp(rint(X / (r c))).
 * d_slots[b] is the pool slot of request b (int32, device).  d_q, d_k
 * [n_layers][batch][H][d_k]; d_v, d_y [..][d_v]; d_beta [..]; d_gate is alpha
 * in (0, 1]: [n_layers][batch][H] (GDN) or [n_layers][batch][H][d_k] (KDA).
 * Slots must be distinct within a call (otherwise the result is undefined;
 * SQ_STEP_VALIDATE checks it and returns SQ_ERR_SLOT).  Enqueued on
 * stream_main (and stream_aux with SQ_STEP_SPLIT; ordered by events, the call
 * returns with stream_main waiting for all of its work).
 * SQ_STEP_SPLIT | SQ_STEP_NO_JOIN leaves the fit + pack of the call running on
 * stream_aux so that later work on stream_main (another layer's readout, the
 * model's own kernels) overlaps it (hyper.ai summary, 方法, the second-stream
 * arrangement).  The caller then orders anything that touches the same layers
 * (the next step's call for them, sq_export, ...) after stream_aux; calls for
 * other layers may follow on stream_main at once.  The split scratch holds one
 * region per (layer, slot index < n_slots), so such calls do not share it. */
sq_status sq_state_step(sq_pool* pool, int32_t layer0, int32_t n_layers, int32_t batch,
                        const int32_t* d_slots, const float* d_q, const float* d_k,
                        const float* d_v, const float* d_gate, const float* d_beta, float* d_y,
                        void* stream_main, void* stream_aux, uint32_t flags);

/* ---- state_step, split, without allocation -----------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * two kernels as sq_state_step with SQ_STEP_SPLIT, both on one stream, with
 * the scratch e = v - k^T D S in a fixed array of SQ_SPLIT_STATIC_MAX_FLOATS
 * floats that the library holds on each GPU until the process ends (its
 * address is looked up when a pool is created on that GPU).  Same arguments
 * and layouts as sq_state_step; bitwise the same y and pool bytes.
 * n_layers * batch * H * d_v above the limit: SQ_ERR_ARG, nothing enqueued.
 * Every call on one GPU uses the same array: calls that overlap on that GPU
 * (other streams, other host threads, other pools) race and their results
 * are undefined; order them.  Makes no device allocation and no host copy. */
#define SQ_SPLIT_STATIC_MAX_FLOATS (8ll << 20)
sq_status sq_state_step_split_static(sq_pool* pool, int32_t layer0, int32_t n_layers,
                                     int32_t batch, const int32_t* d_slots, const float* d_q,
                                     const float* d_k, const float* d_v, const float* d_gate,
                                     const float* d_beta, float* d_y, void* stream);

/* ---- pack / unpack -----------------------------------------------------
 * sq_pack quantizes float states d_X [n_layers][batch][H][d_k][d_v] into the
 * slots (row factors, column fit, rounding; the requantization half of a
 * step).  sq_unpack writes the dequantized states r_i c_j Q_ij (binary16
 * value on pivot rows) to d_X in the same layout (rcap.io pseudocode, unpack). */
sq_status sq_pack(sq_pool* pool, int32_t layer0, int32_t n_layers, int32_t batch,
                  const int32_t* d_slots, const float* d_X, void* stream);
sq_status sq_unpack(sq_pool* pool, int32_t layer0, int32_t n_layers, int32_t batch,
                    const int32_t* d_slots, float* d_X, void* stream);

/* ---- export / import ---------------------------------------------------
 * Canonical (layout-independent) form of the packed states, in canonical
 * key-row order: d_codes int16 [n_layers][batch][H][d_k][d_v] holds the
 * signed code on code rows and the binary16 bit pattern on pivot rows;
 * d_r uint16 [..][d_k] binary16 row factors (1.0 on pivot rows); d_c uint16
 * [..][d_v] binary16 column scales.  Import clamps codes to each row's range. */
sq_status sq_export(sq_pool* pool, int32_t layer0, int32_t n_layers, int32_t batch,
                    const int32_t* d_slots, int16_t* d_codes, uint16_t* d_r, uint16_t* d_c,
                    void* stream);
sq_status sq_import(sq_pool* pool, int32_t layer0, int32_t n_layers, int32_t batch,
                    const int32_t* d_slots, const int16_t* d_codes, const uint16_t* d_r,
                    const uint16_t* d_c, void* stream);

/* ---- comparators (same inputs, other state formats) --------------------
 * Uniform INT8 per-row state (the baseline the pages compare against): state
 * i = (layer * n_slots + slot) * H + head holds d_k*d_v int8 codes at
 * d_codes + i*d_k*d_v and a binary32 row scale [d_k] at d_scales + i*d_k;
 * step: S = s_i Q, the same update and readout, s_i = max_j |X_ij| / 127,
 * Q = clamp(rint(X / s_i), +-127).  The codes of a state are group-interleaved
 * like the pool's 8-bit containers: with cpl = max(1, d_v / 64) columns per lane,
 * lpr = d_v / cpl lanes and gr = 16 / cpl rows per group, code (i, j) sits at
 * byte ((i / gr) * lpr + j / cpl) * 16 + (i % gr) * cpl + j % cpl of the state.
 * sq_fp32_step keeps float states d_S [(layer * n_slots + slot) * H + head]
 * [d_k][d_v] row-major (no quantization).  Alignment: d_codes to 16 bytes, d_S
 * to 4 * cpl bytes; otherwise SQ_ERR_ARG. */
sq_status sq_int8_step(int32_t form, int32_t n_heads, int32_t dim_k, int32_t dim_v, int32_t n_slots,
                       int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                       int8_t* d_codes, float* d_scales, const float* d_q, const float* d_k,
                       const float* d_v, const float* d_gate, const float* d_beta, float* d_y,
                       void* stream);
sq_status sq_fp32_step(int32_t form, int32_t n_heads, int32_t dim_k, int32_t dim_v, int32_t n_slots,
                       int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                       float* d_S, const float* d_q, const float* d_k, const float* d_v,
                       const float* d_gate, const float* d_beta, float* d_y, void* stream);
/* Streaming copy of n_bytes (multiple of 16, 16-byte aligned) for measuring achievable HBM bandwidth. */
sq_status sq_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream);
/* VALU issue-rate probe for measuring the instruction-issue ceiling of the step's occupancy:
 * n_blocks workgroups of 256 threads (4 wave64, one per SIMD), each lane running 8 independent
 * chains of 1024 fp32 FMAs, with dynamic LDS reserved so that at most waves_per_simd (1..8)
 * workgroups, i.e. waves per SIMD, are resident on a CU.  d_out (device, caller-owned) receives
 * n_blocks * 256 floats (the chains' sums).  On return *n_fma holds the wave-level FMA
 * instructions the launch issues (n_blocks * 4 * 8192) and *blocks_per_cu the residency the
 * runtime reports for that LDS reservation; time the launch on `stream` with events.
 * SQ_ERR_ARG for NULL pointers or out-of-range sizes; SQ_ERR_UNSUPPORTED when the device's LDS
 * cannot cap residency at waves_per_simd (the per-workgroup LDS limit); asynchronous otherwise. */
sq_status sq_valu_probe(int32_t waves_per_simd, int32_t n_blocks, float* d_out, uint64_t* n_fma,
                        int32_t* blocks_per_cu, void* stream);

/* ---- errors / info ------------------------------------------------------ */
const char* sq_status_str(sq_status s);
const char* sq_last_error(void);          /* thread-local; "" if none */
/* Shapes (d_k, d_v) the step kernels are compiled for, as pairs: out[2i], out[2i+1]. */
int32_t     sq_supported_shapes(int32_t* out, int32_t max_pairs);

#ifdef __cplusplus
}
#endif
#endif /* STEPQ_H */
