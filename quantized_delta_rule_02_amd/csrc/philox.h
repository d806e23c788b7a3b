// Philox-4x32-10 counter-based generator (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11) and the calibration
// trace recipe built on it.  Host only.
#pragma once
#include <cmath>
#include <cstdint>

namespace sq {

struct Philox4 {
    uint32_t v[4];
};

inline Philox4 philox4x32_10(Philox4 c, uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = uint64_t(0xD2511F53u) * c.v[0];
        const uint64_t p1 = uint64_t(0xCD9E8D57u) * c.v[2];
        const uint32_t hi0 = uint32_t(p0 >> 32), lo0 = uint32_t(p0);
        const uint32_t hi1 = uint32_t(p1 >> 32), lo1 = uint32_t(p1);
        Philox4 n;
        n.v[0] = hi1 ^ c.v[1] ^ k0;
        n.v[1] = lo1;
        n.v[2] = hi0 ^ c.v[3] ^ k1;
        n.v[3] = lo0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// Normal number `idx` of token (seg, tok) of head (layer, head): counter
// (block, tok, seg, layer << 16 | head), four uint32 -> two Box-Muller pairs.
inline double calib_normal(uint64_t seed, int layer, int head, int seg, int tok, int idx) {
    Philox4 c;
    c.v[0] = uint32_t(idx / 4);
    c.v[1] = uint32_t(tok);
    c.v[2] = uint32_t(seg);
    c.v[3] = (uint32_t(layer) << 16) | uint32_t(head);
    const Philox4 x = philox4x32_10(c, uint32_t(seed & 0xFFFFFFFFu), uint32_t(seed >> 32));
    const int lane = idx % 4;
    const int pair = lane / 2;
    const double u0 = (double(x.v[2 * pair]) + 0.5) * 0x1p-32;
    const double u1 = (double(x.v[2 * pair + 1]) + 0.5) * 0x1p-32;
    const double rad = std::sqrt(-2.0 * std::log(u0));
    const double th = 2.0 * M_PI * u1;
    return (lane % 2 == 0) ? rad * std::cos(th) : rad * std::sin(th);
}

}  // namespace sq
