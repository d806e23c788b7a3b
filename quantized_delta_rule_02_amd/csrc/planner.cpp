// Offline planner (host, C++): calibration recurrence, lifetime weights,
// distortion per candidate width, FP16 pivots, exact budgeted allocation, and
// the packed pool layout.
//
// Method (STEPQuant pages): hyper.ai summary, section 方法 (Method) -- the
// lifetime-aware bit allocation paragraph (mean log retention, exponential
// error-retention approximation, lifetime-weighted distortion under an
// average-bit budget, FP16 pivots for the riskiest units) and the spatial
// paragraph (row-impact score = expected squared readout weighting factor over
// calibration tokens); rcap.io post, "Temporal" paragraph (a unit is a head for
// GDN or a key row for KDA) and the note that allocation runs offline on 32
// calibration segments.
//
// Readings taken where the pages are open: the lifetime weight is the sum of
// exp(j * mean log retention) over j >= 0; distortion is the mean over
// segment-final calibration states of the squared error of the unit's entries
// when the whole state is quantized at one width with the step's own dual-axis
// quantizer (no pivots); pivots are ranked by lifetime, then distortion at the
// narrowest width; the allocation is an exact dynamic programme whose ties go to
// fewer bits and, within a unit, to the narrower width.
#include <algorithm>
#include <atomic>
#include <cfenv>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "host.h"
#include "philox.h"

namespace sq {

// ---------------------------------------------------------------- binary16

double fp16_round_host(double x) {
    const double a = std::fabs(x);
    int e;
    std::frexp(a, &e);                       // a = m * 2^e, m in [0.5, 1)
    int ex = (a > 0) ? e - 1 : -14;
    if (ex < -14) ex = -14;                  // subnormal binade spacing 2^-24
    const double ulp = std::ldexp(1.0, ex - 10);
    double r = std::nearbyint(a / ulp) * ulp;  // round-to-nearest-even (default mode)
    if (r > 65504.0) r = 65504.0;
    return std::copysign(r, x);
}

uint16_t fp16_bits_host(double x) {
    const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
    double a = std::fabs(x);
    if (a == 0) return sign;
    int e;
    double m = std::frexp(a, &e);            // a = m * 2^e
    int ex = e - 1;                          // a = (2m) * 2^ex, 2m in [1, 2)
    if (ex < -14) {                          // subnormal: a = frac * 2^-24
        return uint16_t(sign | uint16_t(std::lround(a * 0x1p24)));
    }
    const int frac = int(std::lround((2.0 * m - 1.0) * 1024.0));
    return uint16_t(sign | uint16_t((ex + 15) << 10) | uint16_t(frac));
}

// ---------------------------------------------------------------- calibration traces

void generate_calib(uint64_t seed, int layer, int head, int n_seg, int seg_len, int dk, int dv,
                    float* q, float* k, float* v, float* beta) {
    const int n = 2 * dk + dv + 1;
    const int n_blk = (n + 3) / 4;
    std::vector<double> z(size_t(n_blk) * 4);
    for (int s = 0; s < n_seg; ++s) {
        for (int t = 0; t < seg_len; ++t) {
            for (int b = 0; b < n_blk; ++b) {
                Philox4 c;
                c.v[0] = uint32_t(b);
                c.v[1] = uint32_t(t);
                c.v[2] = uint32_t(s);
                c.v[3] = (uint32_t(layer) << 16) | uint32_t(head);
                const Philox4 x = philox4x32_10(c, uint32_t(seed & 0xFFFFFFFFu), uint32_t(seed >> 32));
                for (int p = 0; p < 2; ++p) {
                    const double u0 = (double(x.v[2 * p]) + 0.5) * 0x1p-32;
                    const double u1 = (double(x.v[2 * p + 1]) + 0.5) * 0x1p-32;
                    const double rad = std::sqrt(-2.0 * std::log(u0));
                    const double th = 2.0 * M_PI * u1;
                    double sn, cs;
                    sincos(th, &sn, &cs);
                    z[size_t(b) * 4 + 2 * p] = rad * cs;
                    z[size_t(b) * 4 + 2 * p + 1] = rad * sn;
                }
            }
            const size_t tk = size_t(s) * seg_len + t;
            double qn = 0, kn = 0;
            for (int i = 0; i < dk; ++i) qn += z[i] * z[i];
            for (int i = 0; i < dk; ++i) kn += z[dk + i] * z[dk + i];
            qn = std::sqrt(qn);
            kn = std::sqrt(kn);
            for (int i = 0; i < dk; ++i) {
                q[tk * dk + i] = float(z[i] / qn);
                k[tk * dk + i] = float(z[dk + i] / kn);
            }
            for (int j = 0; j < dv; ++j) v[tk * dv + j] = float(z[2 * dk + j]);
            beta[tk] = float(1.0 / (1.0 + std::exp(-z[2 * dk + dv])));
        }
    }
}

// ---------------------------------------------------------------- dual-axis quantizer (double)

namespace {

double clamp_scale(double x) { return std::min(std::max(x, 0x1p-14), 65504.0); }

// Squared reconstruction error per key row of state X [dk][dv] quantized with
// every row at width `bits`, impact scores w, candidate grid.  row_err += ...
void quant_row_errors(const double* X, int dk, int dv, int bits, const double* w,
                      const std::vector<float>& grid, int quantizer, double* row_err) {
    const double qmax = std::ldexp(1.0, bits - 1) - 1.0;
    std::vector<double> r(dk), c0(dv, 0.0);
    for (int i = 0; i < dk; ++i) {
        double m = 0;
        for (int j = 0; j < dv; ++j) m = std::max(m, std::fabs(X[size_t(i) * dv + j]));
        const double pre = quantizer == SQ_QUANT_ROW_ABSMAX ? m / qmax : std::sqrt(m / w[i]);
        r[i] = (m > 0) ? fp16_round_host(clamp_scale(pre)) : 1.0;
    }
    if (quantizer == SQ_QUANT_ROW_ABSMAX) {          // per-row absmax: every column scale is 1
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                const double x = X[size_t(i) * dv + j];
                const double Q = std::min(std::max(std::nearbyint(x / r[i]), -qmax), qmax);
                const double err = x - r[i] * Q;
                row_err[i] += err * err;
            }
        return;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            c0[j] = std::max(c0[j], std::fabs(X[size_t(i) * dv + j]) / (r[i] * qmax));
    for (int j = 0; j < dv; ++j) {
        if (c0[j] == 0) continue;                    // zero column: exact, no error
        double bestF = INFINITY, bestc = 1.0;
        for (size_t g = 0; g < grid.size(); ++g) {
            const double c = fp16_round_host(clamp_scale(double(grid[g]) * c0[j]));
            double F = 0;
            for (int i = 0; i < dk; ++i) {
                const double x = X[size_t(i) * dv + j];
                const double rc = r[i] * c;
                const double Q = std::min(std::max(std::nearbyint(x / rc), -qmax), qmax);
                const double err = x - rc * Q;
                F += w[i] * err * err;
            }
            if (F < bestF) { bestF = F; bestc = c; }
        }
        for (int i = 0; i < dk; ++i) {
            const double x = X[size_t(i) * dv + j];
            const double rc = r[i] * bestc;
            const double Q = std::min(std::max(std::nearbyint(x / rc), -qmax), qmax);
            const double err = x - rc * Q;
            row_err[i] += err * err;
        }
    }
}

struct HeadJob {
    std::vector<double> w;          // [dk] impact used for this head
    std::vector<double> D;          // [units in head][n_widths]
};


// One calibration segment of the unquantized recurrence from S = 0, in one pass
// over the state per token: the pending rank-1 write of the previous token is
// applied together with this token's decay, while k^T D S accumulates.
//   S <- D (S + k_prev w_prev^T);  u = k^T (that);  w = beta (v - u)
template <bool>
__attribute__((always_inline)) static inline void segment_kernel(double* S, int dk, int dv, int T, const double* alpha, const float* k, const float* v,
                           const float* beta) {
    std::vector<double> u(dv), w(dv, 0.0), kp(dk, 0.0);
    std::fill(S, S + size_t(dk) * dv, 0.0);
    for (int t = 0; t < T; ++t) {
        const float* kk = k + size_t(t) * dk;
        std::fill(u.begin(), u.end(), 0.0);
        for (int i = 0; i < dk; ++i) {
            double* row = S + size_t(i) * dv;
            const double a = alpha[i], ki = kp[i], kn = double(kk[i]);
            for (int j = 0; j < dv; ++j) {
                const double x = a * (row[j] + ki * w[j]);
                row[j] = x;
                u[j] += kn * x;
            }
        }
        const double bt = double(beta[t]);
        const float* vv = v + size_t(t) * dv;
        for (int j = 0; j < dv; ++j) w[j] = bt * (double(vv[j]) - u[j]);
        for (int i = 0; i < dk; ++i) kp[i] = double(kk[i]);
    }
    for (int i = 0; i < dk; ++i) {
        double* row = S + size_t(i) * dv;
        for (int j = 0; j < dv; ++j) row[j] += kp[i] * w[j];
    }
}

__attribute__((target("avx2,fma"))) static void segment_avx2(double* S, int dk, int dv, int T, const double* alpha,
                                                             const float* k, const float* v, const float* beta) {
    segment_kernel<true>(S, dk, dv, T, alpha, k, v, beta);
}

static void segment_generic(double* S, int dk, int dv, int T, const double* alpha, const float* k, const float* v,
                            const float* beta) {
    segment_kernel<false>(S, dk, dv, T, alpha, k, v, beta);
}

static void run_segment(double* S, int dk, int dv, int T, const double* alpha, const float* k, const float* v,
                        const float* beta) {
    static const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
    if (avx2) segment_avx2(S, dk, dv, T, alpha, k, v, beta);
    else segment_generic(S, dk, dv, T, alpha, k, v, beta);
}

}  // namespace

sq_status run_planner(const sq_plan_cfg& cfg, sq_plan& p) {
    const int L = p.L, H = p.H, dk = p.dk, dv = p.dv;
    const int nwid = int(p.widths.size());
    const int per = (p.unit == SQ_UNIT_HEAD) ? 1 : dk;
    const int U = L * H * per;
    const int S = cfg.calib_segments, T = cfg.calib_len;
    const bool need_dist = (cfg.unit_bits == nullptr);
    const bool need_traces = need_dist || cfg.impact == nullptr;
    if (need_traces && (S <= 0 || T <= 0)) {
        set_error("calibration needs calib_segments > 0 and calib_len > 0");
        return SQ_ERR_ARG;
    }
    const bool user_traces = cfg.calib_q != nullptr;
    if (user_traces && (!cfg.calib_k || !cfg.calib_v || !cfg.calib_beta)) {
        set_error("calib_q given without calib_k / calib_v / calib_beta");
        return SQ_ERR_ARG;
    }

    // mean log retention and lifetime weight per unit (gate-only)
    p.lbar.assign(U, 0.0);
    p.lifetime.assign(U, 0.0);
    for (int l = 0; l < L; ++l)
        for (int h = 0; h < H; ++h) {
            const int lh = l * H + h;
            for (int r = 0; r < per; ++r) {
                double lb;
                if (cfg.form == SQ_FORM_GDN) {
                    lb = std::log(double(cfg.gate[lh]));
                } else if (p.unit == SQ_UNIT_ROW) {
                    lb = std::log(double(cfg.gate[size_t(lh) * dk + r]));
                } else {
                    double s = 0;
                    for (int i = 0; i < dk; ++i) s += std::log(double(cfg.gate[size_t(lh) * dk + i]));
                    lb = s / dk;
                }
                p.lbar[size_t(lh) * per + r] = lb;
                p.lifetime[size_t(lh) * per + r] = 1.0 / (1.0 - std::exp(std::min(lb, -0x1p-20)));
            }
        }

    // per-head calibration work, parallel over (layer, head)
    std::vector<HeadJob> jobs(size_t(L) * H);
    std::atomic<int> next{0};
    auto worker = [&]() {
        std::vector<float> q, k, v, b;
        std::vector<double> Sst, snap;
        for (;;) {
            const int lh = next.fetch_add(1);
            if (lh >= L * H) break;
            const int l = lh / H, h = lh % H;
            HeadJob& J = jobs[lh];
            J.w.assign(dk, 0.0);
            J.D.assign(size_t(per) * nwid, 0.0);
            const float *tq = nullptr, *tk = nullptr, *tv = nullptr, *tb = nullptr;
            if (need_traces) {
                const size_t nt = size_t(S) * T;
                if (user_traces) {
                    tq = cfg.calib_q + size_t(lh) * nt * dk;
                    tk = cfg.calib_k + size_t(lh) * nt * dk;
                    tv = cfg.calib_v + size_t(lh) * nt * dv;
                    tb = cfg.calib_beta + size_t(lh) * nt;
                } else {
                    q.resize(nt * dk); k.resize(nt * dk); v.resize(nt * dv); b.resize(nt);
                    generate_calib(cfg.calib_seed, l, h, S, T, dk, dv, q.data(), k.data(), v.data(), b.data());
                    tq = q.data(); tk = k.data(); tv = v.data(); tb = b.data();
                }
            }
            std::vector<double> alpha(dk);
            for (int i = 0; i < dk; ++i)
                alpha[i] = (cfg.form == SQ_FORM_GDN) ? double(cfg.gate[lh]) : double(cfg.gate[size_t(lh) * dk + i]);
            if (cfg.impact != nullptr) {
                for (int i = 0; i < dk; ++i) J.w[i] = double(cfg.impact[size_t(lh) * dk + i]);
            } else {
                // w_i = mean over tokens of (alpha_i (q_i - beta k_i k.q))^2
                const size_t nt = size_t(S) * T;
                std::vector<double> acc(dk, 0.0);
                for (size_t t = 0; t < nt; ++t) {
                    double kq = 0;
                    for (int i = 0; i < dk; ++i) kq += double(tk[t * dk + i]) * double(tq[t * dk + i]);
                    const double bt = double(tb[t]);
                    for (int i = 0; i < dk; ++i) {
                        const double a = alpha[i] * (double(tq[t * dk + i]) - bt * double(tk[t * dk + i]) * kq);
                        acc[i] += a * a;
                    }
                }
                for (int i = 0; i < dk; ++i) J.w[i] = acc[i] / double(nt);
            }
            if (!need_dist) continue;
            // unquantized recurrence from zero per segment; distortion of the segment-final state
            Sst.assign(size_t(dk) * dv, 0.0);
            std::vector<double> rowerr(dk);
            for (int s = 0; s < S; ++s) {
                const size_t t0 = size_t(s) * T;
                run_segment(Sst.data(), dk, dv, T, alpha.data(), tk + t0 * dk, tv + t0 * dv, tb + t0);
                for (int wi = 0; wi < nwid; ++wi) {
                    std::fill(rowerr.begin(), rowerr.end(), 0.0);
                    quant_row_errors(Sst.data(), dk, dv, p.widths[wi], J.w.data(), p.grid, p.quantizer, rowerr.data());
                    if (per == 1) {
                        double tot = 0;
                        for (int i = 0; i < dk; ++i) tot += rowerr[i];
                        J.D[wi] += tot;
                    } else {
                        for (int i = 0; i < dk; ++i) J.D[size_t(i) * nwid + wi] += rowerr[i];
                    }
                }
            }
            for (auto& d : J.D) d /= double(S);
        }
    };
    int nthr = cfg.n_threads > 0 ? cfg.n_threads : int(std::thread::hardware_concurrency());
    nthr = std::max(1, std::min(nthr, L * H));
    std::vector<std::thread> pool;
    for (int i = 1; i < nthr; ++i) pool.emplace_back(worker);
    worker();
    for (auto& t : pool) t.join();

    p.impact.assign(size_t(L) * H * dk, 0.0f);
    p.distortion.assign(size_t(U) * nwid, 0.0);
    for (int lh = 0; lh < L * H; ++lh) {
        for (int i = 0; i < dk; ++i) p.impact[size_t(lh) * dk + i] = float(jobs[lh].w[i]);
        for (int r = 0; r < per; ++r)
            for (int wi = 0; wi < nwid; ++wi)
                p.distortion[(size_t(lh) * per + r) * nwid + wi] = jobs[lh].D[size_t(r) * nwid + wi];
    }

    // allocation
    p.unit_bits.assign(U, 0);
    if (!need_dist) {
        for (int u = 0; u < U; ++u) {
            const int b = cfg.unit_bits[u];
            const bool ok = (b == SQ_PIVOT_BITS) || std::find(p.widths.begin(), p.widths.end(), b) != p.widths.end();
            if (!ok) {
                set_error("unit_bits[%d] = %d is neither a candidate width nor %d", u, b, SQ_PIVOT_BITS);
                return SQ_ERR_ARG;
            }
            p.unit_bits[u] = b;
        }
    } else {
        const int n_piv = int((int64_t(p.pivot_ppm) * U + 999999) / 1000000);
        std::vector<int> order(U);
        std::iota(order.begin(), order.end(), 0);
        std::sort(order.begin(), order.end(), [&](int a, int b) {
            if (p.lifetime[a] != p.lifetime[b]) return p.lifetime[a] > p.lifetime[b];
            const double da = p.distortion[size_t(a) * nwid], db = p.distortion[size_t(b) * nwid];
            if (da != db) return da > db;
            return a < b;
        });
        std::vector<char> is_piv(U, 0);
        for (int i = 0; i < n_piv && i < U; ++i) is_piv[order[i]] = 1;
        std::vector<int> rest;
        for (int u = 0; u < U; ++u)
            if (!is_piv[u]) rest.push_back(u);
        const int Up = int(rest.size());
        int step = 0;
        for (int wi = 1; wi < nwid; ++wi) step = std::gcd(step, p.widths[wi] - p.widths[0]);
        step = std::max(step, 1);
        std::vector<int> ex(nwid);
        for (int wi = 0; wi < nwid; ++wi) ex[wi] = (p.widths[wi] - p.widths[0]) / step;
        const int64_t num = int64_t(p.budget_milli) * Up - int64_t(1000) * p.widths[0] * Up;
        if (num < 0) {
            set_error("budget %d milli-bits is below the narrowest width %d", p.budget_milli, p.widths[0]);
            return SQ_ERR_ARG;
        }
        const int64_t E = std::min<int64_t>(num / (int64_t(1000) * step), int64_t(ex[nwid - 1]) * Up);
        std::vector<double> best(E + 1, INFINITY), nxt(E + 1);
        best[0] = 0.0;
        std::vector<int8_t> choice(size_t(Up) * (E + 1), 0);
        for (int ui = 0; ui < Up; ++ui) {
            const int u = rest[ui];
            std::fill(nxt.begin(), nxt.end(), INFINITY);
            int8_t* ch = &choice[size_t(ui) * (E + 1)];
            for (int wi = 0; wi < nwid; ++wi) {
                const double cst = p.lifetime[u] * p.distortion[size_t(u) * nwid + wi];
                const int e = ex[wi];
                for (int64_t x = e; x <= E; ++x) {
                    const double cand = best[x - e] + cst;
                    if (cand < nxt[x]) { nxt[x] = cand; ch[x] = int8_t(wi); }
                }
            }
            best.swap(nxt);
        }
        int64_t x = 0;
        for (int64_t i = 1; i <= E; ++i)
            if (best[i] < best[x]) x = i;
        for (int u = 0; u < U; ++u) p.unit_bits[u] = SQ_PIVOT_BITS;
        for (int ui = Up - 1; ui >= 0; --ui) {
            const int wi = choice[size_t(ui) * (E + 1) + x];
            p.unit_bits[rest[ui]] = p.widths[wi];
            x -= ex[wi];
        }
    }
    p.row_bits.assign(size_t(L) * H * dk, 0);
    for (int lh = 0; lh < L * H; ++lh)
        for (int i = 0; i < dk; ++i)
            p.row_bits[size_t(lh) * dk + i] = p.unit_bits[per == 1 ? lh : size_t(lh) * dk + i];
    return SQ_OK;
}

// ---------------------------------------------------------------- layout

sq_status build_layout(sq_plan& p) {
    const int L = p.L, H = p.H, dk = p.dk, dv = p.dv;
    const int LH = L * H;
    const int GR = gr_of(dv), NG = ng_of(dk, dv);
    p.perm.assign(size_t(LH) * dk, 0);
    p.srow_bits.assign(size_t(LH) * dk, 0);
    p.srow_wf.assign(size_t(LH) * dk * 2, 0.0f);
    p.grp_bits.assign(size_t(LH) * NG, 0);
    p.grp_off.assign(size_t(LH) * NG, 0);
    p.scale_off.assign(LH, 0);
    p.rec_off.assign(LH, 0);
    p.head_flags.assign(LH, 0);
    auto rank = [](int b) { return b == SQ_PIVOT_BITS ? 0 : 16 - b; };   // pivots, then descending width
    uint64_t off = 0;
    for (int lh = 0; lh < LH; ++lh) {
        std::vector<int> rows(dk);
        std::iota(rows.begin(), rows.end(), 0);
        const int32_t* rb = &p.row_bits[size_t(lh) * dk];
        std::stable_sort(rows.begin(), rows.end(), [&](int a, int b) { return rank(rb[a]) < rank(rb[b]); });
        uint8_t flags = 0;
        for (int t = 0; t < dk; ++t) {
            p.perm[size_t(lh) * dk + t] = uint16_t(rows[t]);
            p.srow_bits[size_t(lh) * dk + t] = uint8_t(rb[rows[t]]);
            const double w = p.impact[size_t(lh) * dk + rows[t]];
            p.srow_wf[(size_t(lh) * dk + t) * 2] = float(1.0 / w);
            p.srow_wf[(size_t(lh) * dk + t) * 2 + 1] = float(std::sqrt(w));
            flags |= (rb[rows[t]] == SQ_PIVOT_BITS) ? kHasPivotRows : kHasCodeRows;
        }
        p.head_flags[lh] = flags;
        uint32_t roff = 0;
        for (int g = 0; g < NG; ++g) {
            int wmax = 0;
            for (int r = 0; r < GR; ++r) wmax = std::max(wmax, int(p.srow_bits[size_t(lh) * dk + g * GR + r]));
            p.grp_bits[size_t(lh) * NG + g] = uint8_t(wmax);
            p.grp_off[size_t(lh) * NG + g] = roff;
            roff += uint32_t(group_bytes(dv, wmax));
        }
        p.scale_off[lh] = roff;
        roff += uint32_t(2 * (dk + dv));
        roff = (roff + 255u) & ~255u;
        p.rec_off[lh] = off;
        off += roff;
    }
    p.slot_bytes = off;
    return SQ_OK;
}

}  // namespace sq
