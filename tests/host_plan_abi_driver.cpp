// Host-only exercise of the plan half of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer: valid plans, save/load round trips, truncated and corrupted buffers,
// invalid configurations.  The kernel launchers are stubbed (no GPU is touched).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include "stepq.h"
#include "launch.h"

namespace sq {
bool shape_compiled(int dk, int dv) {
    return (dk == 16 && dv == 16) || (dk == 64 && dv == 64) || (dk == 128 && dv == 128) || (dk == 128 && dv == 256);
}
int compiled_shapes(int32_t*, int) { return 4; }
hipError_t launch_state(int, int, int, const StepParams&, int, int, hipStream_t) { abort(); }
hipError_t launch_codec(int, int, bool, const CodecParams&, int, hipStream_t) { abort(); }
hipError_t launch_cmp(int, int, bool, int, int, int, int, int, int, const int32_t*, int8_t*, float*, float*,
                      const float*, const float*, const float*, const float*, const float*, float*, hipStream_t) { abort(); }
hipError_t launch_copy(const void*, void*, size_t, hipStream_t) { abort(); }
hipError_t launch_valu_probe(int, int, float*, uint64_t*, int*, hipStream_t) { abort(); }
hipError_t static_scratch(float**) { abort(); }
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, sq_last_error()); ++fails; } } while (0)

static sq_plan_cfg base(int form, int unit, int L, int H, int dk, int dv, std::vector<int> widths, int budget,
                        std::vector<float>& gate, std::vector<float>& imp, std::mt19937& g) {
    sq_plan_cfg c{};
    c.form = form; c.unit = unit; c.n_layers = L; c.n_heads = H; c.d_k = dk; c.d_v = dv;
    c.n_widths = (int)widths.size();
    for (size_t i = 0; i < widths.size(); ++i) c.widths[i] = widths[i];
    c.budget_milli = budget; c.pivot_ppm = 10000;
    c.n_grid = 4; c.grid[0] = 1.f; c.grid[1] = 0.875f; c.grid[2] = 0.75f; c.grid[3] = 0.625f;
    std::uniform_real_distribution<float> u(0.9f, 0.999f), w(0.5f, 2.f);
    gate.resize(size_t(L) * H * (form == SQ_FORM_GDN ? 1 : dk));
    for (auto& x : gate) x = u(g);
    imp.resize(size_t(L) * H * dk);
    for (auto& x : imp) x = w(g);
    c.gate = gate.data(); c.impact = imp.data();
    c.calib_seed = 7; c.calib_segments = 2; c.calib_len = 16; c.n_threads = 4;
    return c;
}

int main() {
    std::mt19937 g(1);
    struct Case { int form, unit, L, H, dk, dv; std::vector<int> w; int budget; int quant; };
    std::vector<Case> cases = {
        {0, 0, 1, 2, 16, 16, {4, 6, 8}, 6000, 0}, {0, 0, 2, 4, 128, 128, {4, 6, 8}, 6000, 0},
        {1, 1, 1, 3, 128, 128, {4, 6, 8}, 6000, 1}, {1, 1, 1, 2, 128, 256, {2, 3, 4, 6, 8}, 4000, 0},
        {0, 0, 1, 3, 64, 64, {2, 3, 4, 6, 8}, 4000, 0}, {1, 1, 1, 2, 64, 64, {8}, 8000, 0},
    };
    for (auto& cs : cases) {
        std::vector<float> gate, imp;
        sq_plan_cfg c = base(cs.form, cs.unit, cs.L, cs.H, cs.dk, cs.dv, cs.w, cs.budget, gate, imp, g);
        c.quantizer = cs.quant;
        sq_plan* p = nullptr;
        CHECK(sq_plan_create(&c, &p) == SQ_OK);
        if (!p) continue;
        sq_plan_desc d{};
        CHECK(sq_plan_describe(p, &d) == SQ_OK);
        std::vector<double> lbar(d.n_units), life(d.n_units), dist(size_t(d.n_units) * d.n_widths);
        std::vector<int32_t> ub(d.n_units), rb(size_t(cs.L) * cs.H * cs.dk);
        std::vector<float> rw(rb.size());
        CHECK(sq_plan_units(p, lbar.data(), life.data(), dist.data(), ub.data()) == SQ_OK);
        CHECK(sq_plan_rows(p, rb.data(), rw.data()) == SQ_OK);
        size_t n = 0;
        CHECK(sq_plan_save(p, nullptr, &n) == SQ_OK);
        std::vector<unsigned char> buf(n);
        CHECK(sq_plan_save(p, buf.data(), &n) == SQ_OK);
        sq_plan* q = nullptr;
        CHECK(sq_plan_load(buf.data(), n, &q) == SQ_OK);
        if (q) {
            sq_plan_desc d2{};
            CHECK(sq_plan_describe(q, &d2) == SQ_OK);
            CHECK(d2.slot_bytes == d.slot_bytes && d2.n_units == d.n_units);
            sq_plan_destroy(q);
        }
        // truncated buffers and random corruption: an error or a valid plan, never a crash
        for (size_t cut : {size_t(0), size_t(7), n / 3, n - 1}) {
            sq_plan* r = nullptr;
            CHECK(sq_plan_load(buf.data(), cut, &r) != SQ_OK);
            if (r) sq_plan_destroy(r);
        }
        std::uniform_int_distribution<size_t> pos(0, n - 1);
        std::uniform_int_distribution<int> byte(0, 255);
        for (int t = 0; t < 200; ++t) {
            std::vector<unsigned char> b2 = buf;
            for (int k = 0; k < 1 + t % 4; ++k) b2[pos(g)] = (unsigned char)byte(g);
            sq_plan* r = nullptr;
            const sq_status st = sq_plan_load(b2.data(), b2.size(), &r);
            if (st == SQ_OK) {
                sq_plan_desc d3{};
                CHECK(sq_plan_describe(r, &d3) == SQ_OK);
                sq_plan_destroy(r);
            } else {
                CHECK(r == nullptr);
            }
        }
        // fixed allocations, including pivots
        std::vector<int32_t> fixed(d.n_units);
        for (int u = 0; u < d.n_units; ++u) fixed[u] = (u % 5 == 4) ? 16 : cs.w[u % cs.w.size()];
        c.unit_bits = fixed.data();
        sq_plan* f = nullptr;
        CHECK(sq_plan_create(&c, &f) == SQ_OK);
        if (f) sq_plan_destroy(f);
        sq_plan_destroy(p);
    }
    // invalid configurations
    {
        std::vector<float> gate, imp;
        sq_plan_cfg c = base(0, 0, 1, 2, 128, 128, {4, 6, 8}, 6000, gate, imp, g);
        sq_plan* p = nullptr;
        sq_plan_cfg b = c; b.d_k = 96; CHECK(sq_plan_create(&b, &p) == SQ_ERR_UNSUPPORTED && !p);
        b = c; b.widths[0] = 5; CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        b = c; b.n_widths = 0; CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        b = c; b.n_grid = 9; CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        b = c; b.gate = nullptr; CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        b = c; b.quantizer = 2; CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        std::vector<float> g0 = gate; g0[1] = 1.5f; b = c; b.gate = g0.data(); CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
        CHECK(sq_plan_create(nullptr, &p) != SQ_OK);
        CHECK(sq_plan_create(&c, nullptr) != SQ_OK);
        std::vector<int32_t> bad(2, 5);
        b = c; b.unit_bits = bad.data(); CHECK(sq_plan_create(&b, &p) != SQ_OK && !p);
    }
    std::vector<float> q(2 * 3 * 16), k(2 * 3 * 16), v(2 * 3 * 16), be(2 * 3);
    CHECK(sq_calib_generate(5, 0, 1, 2, 3, 16, 16, q.data(), k.data(), v.data(), be.data()) == SQ_OK);
    CHECK(sq_calib_generate(5, -1, 1, 2, 3, 16, 16, q.data(), k.data(), v.data(), be.data()) != SQ_OK);
    // device entry points refuse a NULL pool before any HIP call
    CHECK(sq_state_step(nullptr, 0, 1, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, 0) == SQ_ERR_ARG);
    CHECK(sq_state_step_split_static(nullptr, 0, 1, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr) == SQ_ERR_ARG);
    std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
