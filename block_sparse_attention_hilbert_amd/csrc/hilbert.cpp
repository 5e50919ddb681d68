// 3D Hilbert token order (DFSAttn page, trick 1: tokens are reordered along a
// 3D Hilbert curve so that neighbours in the sequence are neighbours in space
// and time before the sequence is cut into blocks).
//
// The curve is J. Skilling's construction ("Programming the Hilbert curve",
// AIP Conf. Proc. 707, 2004).  This builder walks the curve forwards: for
// every index h = 0, 1, 2, ... of the cube of side 2^b it recovers the cell
// from the "transposed" index (Gray decoding followed by undoing the
// per-level rotations and reflections) and keeps the cells that fall inside
// the latent grid.  Axis 0 of the curve carries t, axis 1 carries y and
// axis 2 -- the axis of the curve's very first step, along which the first
// two octants are stacked -- carries x, the longest side of video latents.
#include <stdint.h>

#include <vector>

#include "sa_internal.h"

namespace sa {
namespace {

// Cell of the curve at index h in a cube of side 2^bits.
inline void curve_cell(uint64_t h, int bits, uint32_t X[3]) {
    // de-interleave: the most significant bit of every 3-bit group is axis 0
    X[0] = X[1] = X[2] = 0;
    for (int lvl = 0; lvl < bits; ++lvl)
        for (int a = 0; a < 3; ++a)
            X[a] |= (uint32_t)((h >> (3 * lvl + 2 - a)) & 1u) << lvl;
    // Gray decode (h ^ h/2 on the interleaved bits)
    uint32_t t = X[2] >> 1;
    X[2] ^= X[1];
    X[1] ^= X[0];
    X[0] ^= t;
    // undo the rotations/reflections, from the second-lowest level upwards
    const uint32_t top = 2u << (bits - 1);
    for (uint32_t q = 2; q != top; q <<= 1) {
        const uint32_t low = q - 1;
        for (int a = 2; a >= 0; --a) {
            if (X[a] & q) {
                X[0] ^= low;
            } else {
                uint32_t s = (X[0] ^ X[a]) & low;
                X[0] ^= s;
                X[a] ^= s;
            }
        }
    }
}

}  // namespace

sa_status build_hilbert_order(int32_t T, int32_t Hg, int32_t W, int32_t* perm,
                              int32_t* inv) {
    int32_t side = T > Hg ? T : Hg;
    side = side > W ? side : W;
    int bits = 1;
    while ((1 << bits) < side) ++bits;
    const int64_t N = (int64_t)T * Hg * W;
    const uint64_t cells = 1ull << (3 * bits);
    int64_t r = 0;
    for (uint64_t h = 0; h < cells && r < N; ++h) {
        uint32_t X[3];
        curve_cell(h, bits, X);
        const uint32_t t = X[0], y = X[1], x = X[2];
        if (t < (uint32_t)T && y < (uint32_t)Hg && x < (uint32_t)W) {
            const int32_t n = (int32_t)(((int64_t)t * Hg + y) * W + x);
            perm[r] = n;
            if (inv) inv[n] = (int32_t)r;
            ++r;
        }
    }
    if (r != N) return fail(SA_ERR_HIP, "hilbert_perm_build: internal error (%lld of %lld cells)",
                            (long long)r, (long long)N);
    return SA_OK;
}

}  // namespace sa
