// C ABI of the quantized gated-delta state step: argument validation, plan and
// pool objects, and kernel launches.  See include/stepq.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "host.h"
#include "launch.h"

namespace sq {

static thread_local std::string g_err;
static std::atomic<uint64_t> g_plan_ids{1};

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

bool shape_supported(int dk, int dv) { return shape_compiled(dk, dv); }

static sq_status hip_fail(hipError_t e, const char* what) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SQ_ERR_HIP;
}

}  // namespace sq

using namespace sq;

struct sq_pool {
    uint64_t plan_id;
    int32_t L, H, dk, dv, form, n_slots, n_grid, quantizer;
    int32_t narrow;                  // some group uses a 2- or 3-bit container
    float grid[kMaxGrid];
    uint8_t* pool;
    size_t pool_bytes;
    uint64_t slot_bytes;
    int device;
    DevTables t;
    std::vector<void*> owned;        // device allocations of the tables
    float* e_buf = nullptr;          // split arrangement scratch (v - k^T D S per state)
    size_t e_cap = 0;                // floats
    std::vector<hipEvent_t> events;  // split arrangement: one per chunk
    std::mutex split_mu;             // serializes the split arrangement's lazy set-up and event use
};

// ------------------------------------------------------------------ errors / info

extern "C" const char* sq_status_str(sq_status s) {
    switch (s) {
        case SQ_OK: return "ok";
        case SQ_ERR_ARG: return "invalid argument";
        case SQ_ERR_SHAPE: return "shape mismatch";
        case SQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case SQ_ERR_SLOT: return "invalid slot list";
        case SQ_ERR_PLAN_MISMATCH: return "plan mismatch";
        case SQ_ERR_NOMEM: return "out of memory";
        case SQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* sq_last_error(void) { return g_err.c_str(); }

extern "C" int32_t sq_supported_shapes(int32_t* out, int32_t max_pairs) {
    return compiled_shapes(out, max_pairs < 0 ? 0 : max_pairs);
}

// ------------------------------------------------------------------ plan

static sq_status validate_cfg(const sq_plan_cfg* c) {
    if (!c) { set_error("cfg is NULL"); return SQ_ERR_ARG; }
    if (c->form != SQ_FORM_GDN && c->form != SQ_FORM_KDA) { set_error("form %d", c->form); return SQ_ERR_ARG; }
    if (c->unit != SQ_UNIT_HEAD && c->unit != SQ_UNIT_ROW) { set_error("unit %d", c->unit); return SQ_ERR_ARG; }
    if (c->n_layers < 1 || c->n_heads < 1 || c->n_layers > 4096 || c->n_heads > 4096) {
        set_error("n_layers %d / n_heads %d out of range", c->n_layers, c->n_heads);
        return SQ_ERR_ARG;
    }
    if (!shape_supported(c->d_k, c->d_v)) {
        set_error("state shape %dx%d is not compiled in", c->d_k, c->d_v);
        return SQ_ERR_UNSUPPORTED;
    }
    if (c->n_widths < 1 || c->n_widths > SQ_MAX_WIDTHS) { set_error("n_widths %d", c->n_widths); return SQ_ERR_ARG; }
    for (int i = 0; i < c->n_widths; ++i) {
        const int b = c->widths[i];
        if (b != 2 && b != 3 && b != 4 && b != 6 && b != 8) {
            set_error("width %d not in {2, 3, 4, 6, 8}", b);
            return SQ_ERR_UNSUPPORTED;
        }
        for (int j = 0; j < i; ++j)
            if (c->widths[j] == b) { set_error("width %d repeated", b); return SQ_ERR_ARG; }
    }
    if (c->pivot_ppm < 0 || c->pivot_ppm > 1000000) { set_error("pivot_ppm %d", c->pivot_ppm); return SQ_ERR_ARG; }
    if (c->quantizer != SQ_QUANT_DUAL_AXIS && c->quantizer != SQ_QUANT_ROW_ABSMAX) {
        set_error("quantizer %d", c->quantizer);
        return SQ_ERR_ARG;
    }
    if (c->n_grid < 1 || c->n_grid > SQ_MAX_GRID) { set_error("n_grid %d not in 1..%d", c->n_grid, SQ_MAX_GRID); return SQ_ERR_UNSUPPORTED; }
    for (int g = 0; g < c->n_grid; ++g)
        if (!(c->grid[g] > 0.f) || !std::isfinite(c->grid[g])) { set_error("grid[%d] not positive", g); return SQ_ERR_ARG; }
    if (!c->gate) { set_error("gate is NULL"); return SQ_ERR_ARG; }
    const size_t ng = size_t(c->n_layers) * c->n_heads * (c->form == SQ_FORM_GDN ? 1 : c->d_k);
    for (size_t i = 0; i < ng; ++i)
        if (!(c->gate[i] > 0.f && c->gate[i] <= 1.f)) { set_error("gate[%zu] = %g not in (0, 1]", i, c->gate[i]); return SQ_ERR_ARG; }
    if (c->impact) {
        const size_t ni = size_t(c->n_layers) * c->n_heads * c->d_k;
        for (size_t i = 0; i < ni; ++i)
            if (!(c->impact[i] > 0.f) || !std::isfinite(c->impact[i])) { set_error("impact[%zu] not positive", i); return SQ_ERR_ARG; }
    }
    return SQ_OK;
}

extern "C" sq_status sq_plan_create(const sq_plan_cfg* cfg, sq_plan** out) {
    if (!out) { set_error("out is NULL"); return SQ_ERR_ARG; }
    *out = nullptr;
    sq_status st = validate_cfg(cfg);
    if (st != SQ_OK) return st;
    sq_plan* p = new (std::nothrow) sq_plan();
    if (!p) { set_error("host allocation"); return SQ_ERR_NOMEM; }
    p->form = cfg->form; p->unit = cfg->unit;
    p->L = cfg->n_layers; p->H = cfg->n_heads; p->dk = cfg->d_k; p->dv = cfg->d_v;
    p->widths.assign(cfg->widths, cfg->widths + cfg->n_widths);
    std::sort(p->widths.begin(), p->widths.end());
    p->budget_milli = cfg->budget_milli; p->pivot_ppm = cfg->pivot_ppm;
    p->quantizer = cfg->quantizer;
    p->grid.assign(cfg->grid, cfg->grid + cfg->n_grid);
    try {
        st = run_planner(*cfg, *p);
        if (st == SQ_OK) st = build_layout(*p);
    } catch (const std::bad_alloc&) {
        set_error("host allocation in the planner");
        st = SQ_ERR_NOMEM;
    }
    if (st != SQ_OK) { delete p; return st; }
    p->plan_id = g_plan_ids.fetch_add(1);
    *out = p;
    return SQ_OK;
}

extern "C" void sq_plan_destroy(sq_plan* plan) { delete plan; }

extern "C" sq_status sq_plan_describe(const sq_plan* p, sq_plan_desc* out) {
    if (!p || !out) { set_error("NULL argument"); return SQ_ERR_ARG; }
    out->n_layers = p->L; out->n_heads = p->H; out->d_k = p->dk; out->d_v = p->dv;
    out->form = p->form; out->unit = p->unit; out->n_units = p->n_units();
    out->n_pivot_units = int32_t(std::count(p->unit_bits.begin(), p->unit_bits.end(), SQ_PIVOT_BITS));
    out->n_grid = int32_t(p->grid.size());
    out->n_widths = int32_t(p->widths.size());
    for (int i = 0; i < SQ_MAX_WIDTHS; ++i) out->widths[i] = i < out->n_widths ? p->widths[i] : 0;
    out->slot_bytes = p->slot_bytes;
    const double entries = double(p->L) * p->H * p->dk * p->dv;
    double bits = 0;
    for (int32_t b : p->row_bits) bits += double(b) * p->dv;
    out->code_bits_per_entry = bits / entries;
    out->stored_bits_per_entry = double(p->slot_bytes) * 8.0 / entries;
    out->compression_vs_fp32 = 32.0 / out->stored_bits_per_entry;
    out->quantizer = p->quantizer;
    return SQ_OK;
}

extern "C" sq_status sq_plan_units(const sq_plan* p, double* lbar, double* lifetime, double* distortion,
                                   int32_t* unit_bits) {
    if (!p) { set_error("plan is NULL"); return SQ_ERR_ARG; }
    if (lbar) std::copy(p->lbar.begin(), p->lbar.end(), lbar);
    if (lifetime) std::copy(p->lifetime.begin(), p->lifetime.end(), lifetime);
    if (distortion) std::copy(p->distortion.begin(), p->distortion.end(), distortion);
    if (unit_bits) std::copy(p->unit_bits.begin(), p->unit_bits.end(), unit_bits);
    return SQ_OK;
}

extern "C" sq_status sq_plan_rows(const sq_plan* p, int32_t* row_bits, float* impact) {
    if (!p) { set_error("plan is NULL"); return SQ_ERR_ARG; }
    if (row_bits) std::copy(p->row_bits.begin(), p->row_bits.end(), row_bits);
    if (impact) std::copy(p->impact.begin(), p->impact.end(), impact);
    return SQ_OK;
}

// serialization: "SQPLAN01", scalars, then length-prefixed vectors
namespace {
struct Writer {
    std::vector<uint8_t> b;
    template <class T> void put(const T& v) {
        const uint8_t* p = reinterpret_cast<const uint8_t*>(&v);
        b.insert(b.end(), p, p + sizeof(T));
    }
    template <class T> void vec(const std::vector<T>& v) {
        put<uint64_t>(v.size());
        const uint8_t* p = reinterpret_cast<const uint8_t*>(v.data());
        b.insert(b.end(), p, p + v.size() * sizeof(T));
    }
};
struct Reader {
    const uint8_t* p;
    size_t n, i = 0;
    bool ok = true;
    template <class T> T get() {
        T v{};
        if (i + sizeof(T) > n) { ok = false; return v; }
        std::memcpy(&v, p + i, sizeof(T));
        i += sizeof(T);
        return v;
    }
    template <class T> void vec(std::vector<T>& v, size_t expect) {
        const uint64_t m = get<uint64_t>();
        if (!ok || m != expect || i + m * sizeof(T) > n) { ok = false; return; }
        v.resize(m);
        std::memcpy(v.data(), p + i, m * sizeof(T));
        i += m * sizeof(T);
    }
};
const char kMagic[8] = {'S', 'Q', 'P', 'L', 'A', 'N', '0', '2'};
}  // namespace

static void serialize(const sq_plan& p, Writer& w) {
    for (char c : kMagic) w.put(c);
    w.put(p.form); w.put(p.unit); w.put(p.L); w.put(p.H); w.put(p.dk); w.put(p.dv);
    w.put(p.budget_milli); w.put(p.pivot_ppm); w.put(p.quantizer);
    w.vec(p.widths); w.vec(p.grid);
    w.vec(p.lbar); w.vec(p.lifetime); w.vec(p.distortion); w.vec(p.unit_bits); w.vec(p.row_bits); w.vec(p.impact);
}

extern "C" sq_status sq_plan_save(const sq_plan* p, void* buf, size_t* bytes) {
    if (!p || !bytes) { set_error("NULL argument"); return SQ_ERR_ARG; }
    Writer w;
    serialize(*p, w);
    if (!buf) { *bytes = w.b.size(); return SQ_OK; }
    if (*bytes < w.b.size()) { set_error("buffer of %zu bytes, need %zu", *bytes, w.b.size()); *bytes = w.b.size(); return SQ_ERR_SHAPE; }
    std::memcpy(buf, w.b.data(), w.b.size());
    *bytes = w.b.size();
    return SQ_OK;
}

extern "C" sq_status sq_plan_load(const void* buf, size_t bytes, sq_plan** out) {
    if (!buf || !out) { set_error("NULL argument"); return SQ_ERR_ARG; }
    *out = nullptr;
    Reader r{static_cast<const uint8_t*>(buf), bytes};
    for (char c : kMagic)
        if (r.get<char>() != c || !r.ok) { set_error("not a serialized plan"); return SQ_ERR_ARG; }
    sq_plan* p = new (std::nothrow) sq_plan();
    if (!p) { set_error("host allocation"); return SQ_ERR_NOMEM; }
    p->form = r.get<int32_t>(); p->unit = r.get<int32_t>(); p->L = r.get<int32_t>(); p->H = r.get<int32_t>();
    p->dk = r.get<int32_t>(); p->dv = r.get<int32_t>(); p->budget_milli = r.get<int32_t>(); p->pivot_ppm = r.get<int32_t>();
    p->quantizer = r.get<int32_t>();
    bool ok = r.ok && (p->form == 0 || p->form == 1) && (p->unit == 0 || p->unit == 1) && p->L >= 1 && p->H >= 1 &&
              (p->quantizer == SQ_QUANT_DUAL_AXIS || p->quantizer == SQ_QUANT_ROW_ABSMAX) &&
              p->L <= 4096 && p->H <= 4096 && shape_supported(p->dk, p->dv);
    if (ok) {
        const uint64_t nw = r.get<uint64_t>();
        r.i -= sizeof(uint64_t);
        ok = r.ok && nw >= 1 && nw <= SQ_MAX_WIDTHS;
        if (ok) r.vec(p->widths, nw);
        const uint64_t ng = r.get<uint64_t>();
        r.i -= sizeof(uint64_t);
        ok = ok && r.ok && ng >= 1 && ng <= SQ_MAX_GRID;
        if (ok) r.vec(p->grid, ng);
        const size_t U = size_t(p->n_units()), R = size_t(p->L) * p->H * p->dk;
        if (ok) {
            r.vec(p->lbar, U); r.vec(p->lifetime, U); r.vec(p->distortion, U * nw); r.vec(p->unit_bits, U);
            r.vec(p->row_bits, R); r.vec(p->impact, R);
            ok = r.ok && r.i == bytes;
        }
        if (ok)
            for (int32_t b : p->row_bits)
                if (b != 2 && b != 3 && b != 4 && b != 6 && b != 8 && b != SQ_PIVOT_BITS) ok = false;
        if (ok)
            for (float w : p->impact)
                if (!(w > 0.f) || !std::isfinite(w)) ok = false;
    }
    if (!ok) { delete p; set_error("corrupt or unsupported plan buffer"); return SQ_ERR_ARG; }
    build_layout(*p);
    p->plan_id = g_plan_ids.fetch_add(1);
    *out = p;
    return SQ_OK;
}

extern "C" sq_status sq_calib_generate(uint64_t seed, int32_t layer, int32_t head, int32_t n_seg, int32_t seg_len,
                                       int32_t d_k, int32_t d_v, float* q, float* k, float* v, float* beta) {
    if (!q || !k || !v || !beta) { set_error("NULL output"); return SQ_ERR_ARG; }
    if (layer < 0 || layer >= 65536 || head < 0 || head >= 65536 || n_seg < 0 || seg_len < 0 || d_k < 1 || d_v < 1) {
        set_error("bad generator arguments");
        return SQ_ERR_ARG;
    }
    generate_calib(seed, layer, head, n_seg, seg_len, d_k, d_v, q, k, v, beta);
    return SQ_OK;
}

// ------------------------------------------------------------------ pool

extern "C" sq_status sq_pool_bytes(const sq_plan* p, int32_t n_slots, size_t* bytes) {
    if (!p || !bytes) { set_error("NULL argument"); return SQ_ERR_ARG; }
    if (n_slots < 1) { set_error("n_slots %d", n_slots); return SQ_ERR_ARG; }
    *bytes = size_t(p->slot_bytes) * size_t(n_slots);
    return SQ_OK;
}

template <class T>
static sq_status upload(sq_pool* pl, const std::vector<T>& v, const T** dst) {
    void* d = nullptr;
    // whole 16-byte units: kernels read byte tables through dword loads
    const size_t n = (std::max<size_t>(v.size() * sizeof(T), 16) + 15) & ~size_t(15);
    hipError_t e = hipMalloc(&d, n);
    if (e != hipSuccess) { set_error("hipMalloc of %zu bytes: %s", n, hipGetErrorString(e)); return SQ_ERR_NOMEM; }
    pl->owned.push_back(d);
    if (!v.empty()) {
        e = hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy of the layout tables");
    }
    *dst = static_cast<const T*>(d);
    return SQ_OK;
}

extern "C" void sq_pool_destroy(sq_pool* pl) {
    if (!pl) return;
    for (hipEvent_t ev : pl->events) (void)hipEventDestroy(ev);
    for (void* d : pl->owned) (void)hipFree(d);
    if (pl->e_buf) (void)hipFree(pl->e_buf);
    delete pl;
}

extern "C" sq_status sq_pool_create(const sq_plan* p, void* d_pool, size_t pool_bytes, int32_t n_slots, sq_pool** out) {
    if (!out) { set_error("out is NULL"); return SQ_ERR_ARG; }
    *out = nullptr;
    if (!p || !d_pool) { set_error("NULL plan or pool memory"); return SQ_ERR_ARG; }
    if (n_slots < 1) { set_error("n_slots %d", n_slots); return SQ_ERR_ARG; }
    if (pool_bytes < size_t(p->slot_bytes) * size_t(n_slots)) {
        set_error("pool of %zu bytes, plan needs %zu for %d slots", pool_bytes, size_t(p->slot_bytes) * n_slots, n_slots);
        return SQ_ERR_SHAPE;
    }
    if (reinterpret_cast<uintptr_t>(d_pool) % 256 != 0) { set_error("pool memory must be 256-byte aligned"); return SQ_ERR_ARG; }
    sq_pool* pl = new (std::nothrow) sq_pool();
    if (!pl) { set_error("host allocation"); return SQ_ERR_NOMEM; }
    pl->plan_id = p->plan_id;
    pl->L = p->L; pl->H = p->H; pl->dk = p->dk; pl->dv = p->dv; pl->form = p->form; pl->n_slots = n_slots;
    pl->n_grid = int32_t(p->grid.size());
    pl->quantizer = p->quantizer;
    pl->narrow = std::any_of(p->grp_bits.begin(), p->grp_bits.end(), [](uint8_t b) { return b <= 3; }) ? 1 : 0;
    for (int g = 0; g < kMaxGrid; ++g) pl->grid[g] = g < pl->n_grid ? p->grid[g] : 1.f;
    pl->pool = static_cast<uint8_t*>(d_pool);
    pl->pool_bytes = pool_bytes;
    pl->slot_bytes = p->slot_bytes;
    hipError_t e = hipGetDevice(&pl->device);
    if (e != hipSuccess) { delete pl; return hip_fail(e, "hipGetDevice"); }
    float* scr = nullptr;
    e = static_scratch(&scr);   // set-up of the allocation-free split step's array on this device
    if (e != hipSuccess) { delete pl; return hip_fail(e, "looking up the fixed split scratch"); }
    sq_status st = SQ_OK;
    if (st == SQ_OK) st = upload(pl, p->rec_off, &pl->t.rec_off);
    if (st == SQ_OK) st = upload(pl, p->grp_off, &pl->t.grp_off);
    if (st == SQ_OK) st = upload(pl, p->grp_bits, &pl->t.grp_bits);
    if (st == SQ_OK) st = upload(pl, p->scale_off, &pl->t.scale_off);
    if (st == SQ_OK) st = upload(pl, p->perm, &pl->t.perm);
    if (st == SQ_OK) st = upload(pl, p->srow_bits, &pl->t.row_bits);
    if (st == SQ_OK) st = upload(pl, p->srow_wf, reinterpret_cast<const float**>(&pl->t.row_wf));
    if (st == SQ_OK) st = upload(pl, p->head_flags, &pl->t.head_flags);
    if (st != SQ_OK) { sq_pool_destroy(pl); return st; }
    *out = pl;
    return SQ_OK;
}

// ------------------------------------------------------------------ common validation

static sq_status check_range(const sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch) {
    if (!pl) { set_error("pool is NULL"); return SQ_ERR_ARG; }
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != pl->device) {
        set_error("pool bound on device %d, current device %d", pl->device, dev);
        return SQ_ERR_ARG;
    }
    if (layer0 < 0 || n_layers < 0 || layer0 + n_layers > pl->L) {
        set_error("layers [%d, %d) outside the plan's %d layers", layer0, layer0 + n_layers, pl->L);
        return SQ_ERR_PLAN_MISMATCH;
    }
    if (batch < 0 || batch > pl->n_slots) { set_error("batch %d with %d slots", batch, pl->n_slots); return SQ_ERR_ARG; }
    if (batch > 65535) { set_error("batch %d above 65535 requests per call", batch); return SQ_ERR_ARG; }
    const int64_t n_states = int64_t(n_layers) * batch * pl->H;
    if (n_states > int64_t(0x7FFFFFFF)) { set_error("too many states in one call"); return SQ_ERR_ARG; }
    return SQ_OK;
}

static sq_status check_slots_host(const int32_t* d_slots, int32_t batch, int32_t n_slots, hipStream_t s) {
    std::vector<int32_t> h(batch);
    hipError_t e = hipMemcpyAsync(h.data(), d_slots, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "copying the slot list");
    std::vector<char> seen(n_slots, 0);
    for (int i = 0; i < batch; ++i) {
        if (h[i] < 0 || h[i] >= n_slots) { set_error("slots[%d] = %d outside [0, %d)", i, h[i], n_slots); return SQ_ERR_SLOT; }
        if (seen[h[i]]) { set_error("slot %d repeated", h[i]); return SQ_ERR_SLOT; }
        seen[h[i]] = 1;
    }
    return SQ_OK;
}

static StepParams base_params(const sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* slots) {
    StepParams p{};
    p.pool = pl->pool;
    p.slot_bytes = pl->slot_bytes;
    p.t = pl->t;
    p.n_heads = pl->H;
    p.layer0 = layer0;
    p.n_layers = n_layers;
    p.batch = batch;
    p.form = pl->form;
    p.n_slots = pl->n_slots;
    p.slots = slots;
    p.n_grid = pl->n_grid;
    p.quant_mode = pl->quantizer;
    p.narrow = pl->narrow;
    p.unit_first = pl->grid[0] == 1.0f ? 1 : 0;
    for (int g = 0; g < kMaxGrid; ++g) p.grid[g] = pl->grid[g];
    return p;
}

// ------------------------------------------------------------------ state step

extern "C" sq_status sq_state_step(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                                   const float* d_q, const float* d_k, const float* d_v, const float* d_gate,
                                   const float* d_beta, float* d_y, void* stream_main, void* stream_aux, uint32_t flags) {
    sq_status st = check_range(pl, layer0, n_layers, batch);
    if (st != SQ_OK) return st;
    if (flags & ~(SQ_STEP_SPLIT | SQ_STEP_VALIDATE | SQ_STEP_NO_JOIN)) { set_error("unknown flags 0x%x", flags); return SQ_ERR_ARG; }
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!d_slots || !d_q || !d_k || !d_v || !d_gate || !d_beta || !d_y) { set_error("NULL device array"); return SQ_ERR_ARG; }
    hipStream_t sm = static_cast<hipStream_t>(stream_main);
    hipStream_t sa = stream_aux ? static_cast<hipStream_t>(stream_aux) : sm;
    if (flags & SQ_STEP_VALIDATE) {
        st = check_slots_host(d_slots, batch, pl->n_slots, sm);
        if (st != SQ_OK) return st;
    }
    StepParams p = base_params(pl, layer0, n_layers, batch, d_slots);
    p.q = d_q; p.k = d_k; p.v = d_v; p.gate = d_gate; p.beta = d_beta; p.y = d_y;
    hipError_t e;
    if (!(flags & SQ_STEP_SPLIT)) {
        e = launch_state(pl->dk, pl->dv, kModeStep, p, batch, n_layers, sm);
        return e == hipSuccess ? SQ_OK : hip_fail(e, "state step launch");
    }
    // split arrangement: per chunk, readout kernel on the main stream, fit + pack on the aux stream.
    // Scratch e = v - k^T D S: one region per (layer, request index, head), allocated once per pool.
    const int64_t layer_stride = int64_t(pl->n_slots) * pl->H;
    // host threads that enqueue split steps on one pool take turns (the scratch is allocated on first
    // use and the chunk events are shared); the device work itself is ordered by the streams and events
    std::lock_guard<std::mutex> lock(pl->split_mu);
    if (!pl->e_buf) {
        const size_t need = size_t(pl->L) * size_t(layer_stride) * pl->dv;
        e = hipMalloc(reinterpret_cast<void**>(&pl->e_buf), need * sizeof(float));
        if (e != hipSuccess) { set_error("hipMalloc of the split scratch: %s", hipGetErrorString(e)); return SQ_ERR_NOMEM; }
        pl->e_cap = need;
    }
    p.e_buf = pl->e_buf + size_t(layer0) * size_t(layer_stride) * pl->dv;
    p.e_layer_stride = layer_stride;
    // chunks: one layer each, or for a single layer up to four ranges of requests
    const int per_layer = batch * pl->H;
    const int n_chunks = n_layers > 1 ? n_layers : std::min(4, std::max(1, per_layer / 256));
    const int chunk_b = n_layers > 1 ? batch : (batch + n_chunks - 1) / n_chunks;
    while (int(pl->events.size()) < 2 * n_chunks + 1) {
        hipEvent_t ev;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        pl->events.push_back(ev);
    }
    if (sa != sm) {
        // the aux stream must not start before earlier work on the main stream
        e = hipEventRecord(pl->events[2 * n_chunks], sm);
        if (e == hipSuccess) e = hipStreamWaitEvent(sa, pl->events[2 * n_chunks], 0);
        if (e != hipSuccess) return hip_fail(e, "ordering the aux stream");
    }
    for (int c = 0; c < n_chunks; ++c) {
        p.lz0 = n_layers > 1 ? c : 0;
        p.b0 = n_layers > 1 ? 0 : c * chunk_b;
        const int nb = std::min(chunk_b, batch - p.b0);
        if (nb <= 0) break;
        e = launch_state(pl->dk, pl->dv, kModeSplitA, p, nb, 1, sm);
        if (e != hipSuccess) return hip_fail(e, "split readout launch");
        if (sa != sm) {
            e = hipEventRecord(pl->events[2 * c], sm);
            if (e == hipSuccess) e = hipStreamWaitEvent(sa, pl->events[2 * c], 0);
            if (e != hipSuccess) return hip_fail(e, "split event");
        }
        e = launch_state(pl->dk, pl->dv, kModeSplitB, p, nb, 1, sa);
        if (e != hipSuccess) return hip_fail(e, "split fit/pack launch");
    }
    if (sa != sm && !(flags & SQ_STEP_NO_JOIN)) {
        e = hipEventRecord(pl->events[1], sa);
        if (e == hipSuccess) e = hipStreamWaitEvent(sm, pl->events[1], 0);
        if (e != hipSuccess) return hip_fail(e, "joining the aux stream");
    }
    return SQ_OK;
}

static_assert(SQ_SPLIT_STATIC_MAX_FLOATS == kStaticScratchFloats, "fixed split scratch size");

extern "C" sq_status sq_state_step_split_static(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch,
                                                const int32_t* d_slots, const float* d_q, const float* d_k,
                                                const float* d_v, const float* d_gate, const float* d_beta,
                                                float* d_y, void* stream) {
    sq_status st = check_range(pl, layer0, n_layers, batch);
    if (st != SQ_OK) return st;
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!d_slots || !d_q || !d_k || !d_v || !d_gate || !d_beta || !d_y) { set_error("NULL device array"); return SQ_ERR_ARG; }
    const int64_t need = int64_t(n_layers) * batch * pl->H * pl->dv;
    if (need > kStaticScratchFloats) {
        set_error("split scratch of %lld floats (n_layers * batch * H * d_v) above the fixed %lld",
                  (long long)need, (long long)kStaticScratchFloats);
        return SQ_ERR_ARG;
    }
    float* scr = nullptr;
    hipError_t e = static_scratch(&scr);   // looked up when the pool was created on this device
    if (e != hipSuccess) return hip_fail(e, "fixed split scratch");
    StepParams p = base_params(pl, layer0, n_layers, batch, d_slots);
    p.q = d_q; p.k = d_k; p.v = d_v; p.gate = d_gate; p.beta = d_beta; p.y = d_y;
    p.e_buf = scr;                                  // [layer][request][head][d_v] of this call only
    p.e_layer_stride = int64_t(batch) * pl->H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = launch_state(pl->dk, pl->dv, kModeSplitA, p, batch, n_layers, s);
    if (e != hipSuccess) return hip_fail(e, "split readout launch");
    e = launch_state(pl->dk, pl->dv, kModeSplitB, p, batch, n_layers, s);
    return e == hipSuccess ? SQ_OK : hip_fail(e, "split fit/pack launch");
}

// ------------------------------------------------------------------ pack / unpack / export / import

extern "C" sq_status sq_pack(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                             const float* d_X, void* stream) {
    sq_status st = check_range(pl, layer0, n_layers, batch);
    if (st != SQ_OK) return st;
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!d_slots || !d_X) { set_error("NULL device array"); return SQ_ERR_ARG; }
    StepParams p = base_params(pl, layer0, n_layers, batch, d_slots);
    p.x_in = d_X;
    hipError_t e = launch_state(pl->dk, pl->dv, kModePack, p, batch, n_layers, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SQ_OK : hip_fail(e, "pack launch");
}

extern "C" sq_status sq_unpack(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                               float* d_X, void* stream) {
    sq_status st = check_range(pl, layer0, n_layers, batch);
    if (st != SQ_OK) return st;
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!d_slots || !d_X) { set_error("NULL device array"); return SQ_ERR_ARG; }
    StepParams p = base_params(pl, layer0, n_layers, batch, d_slots);
    p.x_out = d_X;
    hipError_t e = launch_state(pl->dk, pl->dv, kModeUnpack, p, batch, n_layers, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SQ_OK : hip_fail(e, "unpack launch");
}

static sq_status codec(sq_pool* pl, bool do_export, int32_t layer0, int32_t n_layers, int32_t batch,
                       const int32_t* d_slots, int16_t* codes, uint16_t* r, uint16_t* c, void* stream) {
    sq_status st = check_range(pl, layer0, n_layers, batch);
    if (st != SQ_OK) return st;
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!d_slots || !codes || !r || !c) { set_error("NULL device array"); return SQ_ERR_ARG; }
    CodecParams p{};
    p.pool = pl->pool; p.slot_bytes = pl->slot_bytes; p.t = pl->t; p.n_heads = pl->H; p.layer0 = layer0;
    p.batch = batch; p.n_slots = pl->n_slots; p.slots = d_slots; p.codes = codes; p.r = r; p.c = c;
    hipError_t e = launch_codec(pl->dk, pl->dv, do_export, p, n_layers * batch * pl->H, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SQ_OK : hip_fail(e, do_export ? "export launch" : "import launch");
}

extern "C" sq_status sq_export(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                               int16_t* d_codes, uint16_t* d_r, uint16_t* d_c, void* stream) {
    return codec(pl, true, layer0, n_layers, batch, d_slots, d_codes, d_r, d_c, stream);
}

extern "C" sq_status sq_import(sq_pool* pl, int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                               const int16_t* d_codes, const uint16_t* d_r, const uint16_t* d_c, void* stream) {
    return codec(pl, false, layer0, n_layers, batch, d_slots, const_cast<int16_t*>(d_codes),
                 const_cast<uint16_t*>(d_r), const_cast<uint16_t*>(d_c), stream);
}

// ------------------------------------------------------------------ comparators / copy

static sq_status cmp_step(bool int8, int32_t form, int32_t H, int32_t dk, int32_t dv, int32_t n_slots, int32_t layer0,
                          int32_t n_layers, int32_t batch, const int32_t* slots, int8_t* codes, float* scales, float* S,
                          const float* q, const float* k, const float* v, const float* gate, const float* beta,
                          float* y, void* stream) {
    if (form != SQ_FORM_GDN && form != SQ_FORM_KDA) { set_error("form %d", form); return SQ_ERR_ARG; }
    if (!shape_supported(dk, dv)) { set_error("state shape %dx%d is not compiled in", dk, dv); return SQ_ERR_UNSUPPORTED; }
    if (H < 1 || n_slots < 1 || layer0 < 0 || n_layers < 0 || batch < 0 || batch > n_slots) {
        set_error("bad sizes");
        return SQ_ERR_ARG;
    }
    if (int64_t(n_layers) * batch * H > int64_t(0x7FFFFFFF)) { set_error("too many states in one call"); return SQ_ERR_ARG; }
    if (batch == 0 || n_layers == 0) return SQ_OK;   // nothing to do
    if (!slots || !q || !k || !v || !gate || !beta || !y || (int8 ? (!codes || !scales) : !S)) {
        set_error("NULL device array");
        return SQ_ERR_ARG;
    }
    // INT8: one 16-byte access per lane and group; FP32: a lane's cpl adjacent entries of a row in one access
    const uintptr_t cpl = uintptr_t(cpl_of(dv));
    if (int8 ? (reinterpret_cast<uintptr_t>(codes) % 16 != 0) : (reinterpret_cast<uintptr_t>(S) % (4 * cpl) != 0)) {
        set_error("state array not aligned to %u bytes", unsigned(int8 ? 16 : 4 * cpl));
        return SQ_ERR_ARG;
    }
    hipError_t e = launch_cmp(dk, dv, int8, form, H, n_slots, layer0, n_layers, batch, slots, codes, scales, S, q, k, v,
                              gate, beta, y, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SQ_OK : hip_fail(e, int8 ? "int8 step launch" : "fp32 step launch");
}

extern "C" sq_status sq_int8_step(int32_t form, int32_t n_heads, int32_t dim_k, int32_t dim_v, int32_t n_slots,
                                  int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots,
                                  int8_t* d_codes, float* d_scales, const float* d_q, const float* d_k,
                                  const float* d_v, const float* d_gate, const float* d_beta, float* d_y,
                                  void* stream) {
    return cmp_step(true, form, n_heads, dim_k, dim_v, n_slots, layer0, n_layers, batch, d_slots, d_codes, d_scales,
                    nullptr, d_q, d_k, d_v, d_gate, d_beta, d_y, stream);
}

extern "C" sq_status sq_fp32_step(int32_t form, int32_t n_heads, int32_t dim_k, int32_t dim_v, int32_t n_slots,
                                  int32_t layer0, int32_t n_layers, int32_t batch, const int32_t* d_slots, float* d_S,
                                  const float* d_q, const float* d_k, const float* d_v, const float* d_gate,
                                  const float* d_beta, float* d_y, void* stream) {
    return cmp_step(false, form, n_heads, dim_k, dim_v, n_slots, layer0, n_layers, batch, d_slots, nullptr, nullptr, d_S,
                    d_q, d_k, d_v, d_gate, d_beta, d_y, stream);
}

extern "C" sq_status sq_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream) {
    if (!d_src || !d_dst) { set_error("NULL pointer"); return SQ_ERR_ARG; }
    if (n_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(d_src) % 16 || reinterpret_cast<uintptr_t>(d_dst) % 16) {
        set_error("copy needs 16-byte multiples and alignment");
        return SQ_ERR_ARG;
    }
    hipError_t e = launch_copy(d_src, d_dst, n_bytes, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SQ_OK : hip_fail(e, "copy launch");
}

extern "C" sq_status sq_valu_probe(int32_t waves_per_simd, int32_t n_blocks, float* d_out, uint64_t* n_fma,
                                   int32_t* blocks_per_cu, void* stream) {
    if (!d_out || !n_fma || !blocks_per_cu) { set_error("NULL pointer"); return SQ_ERR_ARG; }
    if (waves_per_simd < 1 || waves_per_simd > 8 || n_blocks < 1) {
        set_error("waves_per_simd must be in [1, 8] and n_blocks positive");
        return SQ_ERR_ARG;
    }
    int fit = 0;
    uint64_t n = 0;
    hipError_t e = launch_valu_probe(waves_per_simd, n_blocks, d_out, &n, &fit, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) {
        set_error("this device's LDS cannot cap residency at that many waves per SIMD");
        return SQ_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) return hip_fail(e, "VALU probe launch");
    *n_fma = n;
    *blocks_per_cu = fit;
    return SQ_OK;
}

// ------------------------------------------------------------------ alternative names

extern "C" sq_status sq_plan_info(const sq_plan* p, sq_plan_desc* out) { return sq_plan_describe(p, out); }

extern "C" sq_status sq_pool_bind(const sq_plan* p, void* d_pool, size_t pool_bytes, int32_t n_slots, sq_pool** out) {
    return sq_pool_create(p, d_pool, pool_bytes, n_slots, out);
}

extern "C" void sq_pool_release(sq_pool* pl) { sq_pool_destroy(pl); }
