// SICS scheme generation over shaped 3D tiles for gfx950 (SPADE page, part 1:
// a menu of ways to cut the latent video cube into blocks; part 2: the sum of
// intra-block cosine similarities decides the scheme per head and step).
//
// For a tile of unit vectors x^_a, the sum of cos(x_a, x_b) over ordered pairs
// a != b is |sum_a x^_a|^2 - (number of non-zero vectors).  Every menu shape's
// tiles are unions of "atoms" -- the tiles of the per-axis greatest common
// divisor of the menu's shapes -- so one pass over Q and K builds the atoms'
// unit-vector sums and each shape sums whole atoms:
//   k_sics_atoms   per (atom, b*h, side): fp64 sum of unit vectors, count of
//                  non-zero vectors (one wave per atom, 4 tokens at a time)
//   k_sics_tiles   per (tile, shape, b*h): the tile's SICS and pair count
//   k_sics_shapes  per (shape, b*h): mean intra-tile cosine over Q and K
//   k_sics_pick    per b*h: the best shape (the first of the menu on ties)
//   k_tile_assign  per token: its tile under the chosen shape (the partition
//                  the clustered path then lays out, one block per tile)
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kMaxShapes = 16;

struct Menu {
    int32_t n;
    int32_t t[kMaxShapes], y[kMaxShapes], x[kMaxShapes];
    int32_t nty[kMaxShapes], ntx[kMaxShapes], ntiles[kMaxShapes];
    int32_t at, ay, ax;          // atom shape
    int32_t nta, nya, nxa;       // atoms per axis
};

int gcd(int a, int b) {
    while (b) {
        const int r = a % b;
        a = b;
        b = r;
    }
    return a;
}

Menu make_menu(const Geometry& g, const sa_cluster_spec& cs) {
    Menu m{};
    m.n = cs.n_shapes;
    m.at = cs.shapes[0].t;
    m.ay = cs.shapes[0].y;
    m.ax = cs.shapes[0].x;
    for (int s = 0; s < m.n; ++s) {
        const sa_tile_shape sh = cs.shapes[s];
        m.t[s] = sh.t;
        m.y[s] = sh.y;
        m.x[s] = sh.x;
        m.nty[s] = (int32_t)ceil_div(g.Hg, sh.y);
        m.ntx[s] = (int32_t)ceil_div(g.W, sh.x);
        m.ntiles[s] = (int32_t)ceil_div(g.T, sh.t) * m.nty[s] * m.ntx[s];
        m.at = gcd(m.at, sh.t);
        m.ay = gcd(m.ay, sh.y);
        m.ax = gcd(m.ax, sh.x);
    }
    m.nta = (int32_t)ceil_div(g.T, m.at);
    m.nya = (int32_t)ceil_div(g.Hg, m.ay);
    m.nxa = (int32_t)ceil_div(g.W, m.ax);
    return m;
}

int64_t n_atoms(const Menu& m) { return (int64_t)m.nta * m.nya * m.nxa; }

struct SicsWs {
    size_t u, nz, scores, tsics, tpairs, total;
};

int menu_cmax(const Menu& m) {
    int c = 0;
    for (int s = 0; s < m.n; ++s) c = m.ntiles[s] > c ? m.ntiles[s] : c;
    return c;
}

SicsWs sics_ws(const Geometry& g, const Menu& m) {
    SicsWs w{};
    size_t o = 0;
    w.u = o; o = align_up(o + (size_t)g.BH() * 2 * n_atoms(m) * g.d * sizeof(double), 256);
    w.nz = o; o = align_up(o + (size_t)g.BH() * 2 * n_atoms(m) * sizeof(int32_t), 256);
    w.scores = o; o = align_up(o + (size_t)g.BH() * m.n * sizeof(double), 256);
    w.tsics = o; o = align_up(o + (size_t)g.BH() * m.n * menu_cmax(m) * sizeof(double), 256);
    w.tpairs = o; o = align_up(o + (size_t)g.BH() * m.n * menu_cmax(m) * sizeof(double), 256);
    w.total = o;
    return w;
}

// One wave per atom; the wave takes 4 tokens at a time, 16 lanes per token,
// lane L holding channels [(L % 16) * CPL, + CPL).  A token's squared norm is
// reduced over its 16 lanes; at the end the 4 token groups are added in a
// fixed order, so the sums are reproducible.
template <int D>
__global__ __launch_bounds__(256) void k_sics_atoms(const uint16_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ K,
                                                    double* __restrict__ U,
                                                    int32_t* __restrict__ NZ, Menu m, int T,
                                                    int Hg, int W, int64_t natoms) {
    constexpr int CPL = D / 16;                     // 8 (d = 128) or 4 (d = 64)
    const int64_t atom = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (atom >= natoms) return;
    const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
    const int64_t bh = blockIdx.y;
    const int side = blockIdx.z;
    const uint16_t* X = (side ? K : Q) + bh * (int64_t)T * Hg * W * D;
    const int ta = (int)(atom / ((int64_t)m.nya * m.nxa));
    const int ya = (int)((atom / m.nxa) % m.nya);
    const int xa = (int)(atom % m.nxa);
    const int t0 = ta * m.at, y0 = ya * m.ay, x0 = xa * m.ax;
    const int et = min(T, t0 + m.at) - t0, ey = min(Hg, y0 + m.ay) - y0, ex = min(W, x0 + m.ax) - x0;
    const int ntok = et * ey * ex;
    double u[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) u[k] = 0.0;
    int nz = 0;
    for (int i = grp; i - grp < ntok; i += 4) {
        double v[CPL];
        double sq = 0.0;
        if (i < ntok) {
            const int t = t0 + i / (ey * ex), y = y0 + (i / ex) % ey, x = x0 + i % ex;
            const uint16_t* row = X + (((int64_t)t * Hg + y) * W + x) * D + sub * CPL;
#pragma unroll
            for (int q = 0; q < CPL / 2; ++q) {
                const uint32_t w = reinterpret_cast<const uint32_t*>(row)[q];
                v[2 * q] = (double)__uint_as_float(w << 16);
                v[2 * q + 1] = (double)__uint_as_float(w & 0xffff0000u);
            }
#pragma unroll
            for (int k = 0; k < CPL; ++k) sq += v[k] * v[k];
        } else {
#pragma unroll
            for (int k = 0; k < CPL; ++k) v[k] = 0.0;
        }
        for (int off = 8; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 16);
        sq = __shfl(sq, 0, 16);                     // one value per token group
        if (sq > 0.0) {
            const double r = 1.0 / sqrt(sq);
#pragma unroll
            for (int k = 0; k < CPL; ++k) u[k] += v[k] * r;
            ++nz;
        }
    }
    // groups 1..3 into group 0, in order
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const double a1 = __shfl(u[k], sub + 16, 64), a2 = __shfl(u[k], sub + 32, 64),
                     a3 = __shfl(u[k], sub + 48, 64);
        u[k] = ((u[k] + a1) + a2) + a3;
    }
    const int nz1 = __shfl(nz, 16, 64), nz2 = __shfl(nz, 32, 64), nz3 = __shfl(nz, 48, 64);
    const int64_t base = (bh * 2 + side) * natoms + atom;
    if (grp == 0) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) U[base * D + sub * CPL + k] = u[k];
        if (sub == 0) NZ[base] = nz + nz1 + nz2 + nz3;
    }
}

// One workgroup of D threads per (tile, shape, b*h); thread c owns channel c.
// The tile's atoms are summed in raster order and the channels in a fixed
// tree; writes the tile's SICS (Q and K) and its ordered pair count, and with
// kcoh the mean cosine of its keys' ordered pairs, SICS_K / (n (n - 1)) (1 for
// a tile of fewer than two tokens: its mean is its token).
template <int D>
__global__ __launch_bounds__(D) void k_sics_tiles(const double* __restrict__ U,
                                                  const int32_t* __restrict__ NZ,
                                                  double* __restrict__ tile_sics,
                                                  double* __restrict__ tile_pairs,
                                                  double* __restrict__ kcoh, Menu m, int T,
                                                  int Hg, int W, int64_t natoms, int cmax) {
    __shared__ double wsum[D / 64], wsumk[D / 64];
    const int tile = blockIdx.x, s = blockIdx.y;
    const int64_t bh = blockIdx.z;
    if (tile >= m.ntiles[s]) return;
    const int c = threadIdx.x, lane = c & 63, wid = c >> 6;
    const double* Uq = U + (bh * 2) * natoms * D;
    const double* Uk = U + (bh * 2 + 1) * natoms * D;
    const int32_t* Nq = NZ + (bh * 2) * natoms;
    const int32_t* Nk = NZ + (bh * 2 + 1) * natoms;
    const int ts = m.t[s], ys = m.y[s], xs = m.x[s];
    const int tx = tile % m.ntx[s], ty = (tile / m.ntx[s]) % m.nty[s], tt = tile / (m.ntx[s] * m.nty[s]);
    const int t0 = tt * ts, y0 = ty * ys, x0 = tx * xs;
    const int t1 = min(T, t0 + ts), y1 = min(Hg, y0 + ys), x1 = min(W, x0 + xs);
    double uq = 0.0, uk = 0.0;
    int nz = 0, nzk = 0;
    for (int ta = t0 / m.at; ta < (t1 + m.at - 1) / m.at; ++ta)
        for (int ya = y0 / m.ay; ya < (y1 + m.ay - 1) / m.ay; ++ya)
            for (int xa = x0 / m.ax; xa < (x1 + m.ax - 1) / m.ax; ++xa) {
                const int64_t a = ((int64_t)ta * m.nya + ya) * m.nxa + xa;
                uq += Uq[a * D + c];
                uk += Uk[a * D + c];
                nz += Nq[a] + Nk[a];
                nzk += Nk[a];
            }
    double v = uq * uq + uk * uk, vk = uk * uk;
    for (int off = 32; off > 0; off >>= 1) {
        v += __shfl_down(v, off, 64);
        vk += __shfl_down(vk, off, 64);
    }
    if (lane == 0) {
        wsum[wid] = v;
        wsumk[wid] = vk;
    }
    __syncthreads();
    if (c == 0) {
        double tv = 0.0, tk = 0.0;
        for (int w = 0; w < D / 64; ++w) {
            tv += wsum[w];
            tk += wsumk[w];
        }
        const double n = (double)(t1 - t0) * (y1 - y0) * (x1 - x0);
        const int64_t o = (bh * m.n + s) * cmax + tile;
        tile_sics[o] = tv - (double)nz;
        tile_pairs[o] = n * (n - 1.0);
        if (kcoh) kcoh[o] = n < 2.0 ? 1.0 : (tk - (double)nzk) / (n * (n - 1.0));
    }
}

// Score of every (shape, b*h), one wave each: lane L sums tiles L, L+64, ...
// in order, then a fixed tree over the lanes.
__global__ __launch_bounds__(256) void k_sics_shapes(const double* __restrict__ tile_sics,
                                                     const double* __restrict__ tile_pairs,
                                                     double* __restrict__ scores, Menu m,
                                                     int64_t BH, int cmax) {
    const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);     // bh * n + s
    if (e >= BH * m.n) return;
    const int lane = threadIdx.x & 63;
    const int s = (int)(e % m.n);
    double total = 0.0, pairs = 0.0;
    for (int t = lane; t < m.ntiles[s]; t += 64) {
        total += tile_sics[e * cmax + t];
        pairs += tile_pairs[e * cmax + t];
    }
    for (int off = 32; off > 0; off >>= 1) {
        total += __shfl_down(total, off, 64);
        pairs += __shfl_down(pairs, off, 64);
    }
    if (lane == 0) scores[e] = pairs > 0.0 ? total / (2.0 * pairs) : 0.0;
}

__global__ void k_sics_pick(const double* __restrict__ scores, int32_t* __restrict__ shape_idx,
                            int n_shapes, int64_t BH) {
    const int64_t bh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bh >= BH) return;
    double best = scores[bh * n_shapes];
    int arg = 0;
    for (int s = 1; s < n_shapes; ++s) {
        const double v = scores[bh * n_shapes + s];
        if (v > best) {
            best = v;
            arg = s;
        }
    }
    shape_idx[bh] = arg;
}

__global__ void k_tile_assign(const int32_t* __restrict__ shape_idx, int32_t* __restrict__ assign,
                              Menu m, int T, int Hg, int W) {
    const int64_t bh = blockIdx.y;
    const int64_t N = (int64_t)T * Hg * W;
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    int s = shape_idx[bh];
    s = s < 0 ? 0 : (s >= m.n ? m.n - 1 : s);
    const int x = (int)(n % W), y = (int)((n / W) % Hg), t = (int)(n / ((int64_t)Hg * W));
    assign[bh * N + n] = ((t / m.t[s]) * m.nty[s] + y / m.y[s]) * m.ntx[s] + x / m.x[s];
}

}  // namespace

int menu_max_tiles(const Geometry& g, const sa_cluster_spec& cs) {
    int best = 0;
    for (int s = 0; s < cs.n_shapes; ++s) {
        const sa_tile_shape sh = cs.shapes[s];
        const int64_t nt = ceil_div(g.T, sh.t) * ceil_div(g.Hg, sh.y) * ceil_div(g.W, sh.x);
        if (nt > best) best = (int)(nt > INT32_MAX ? INT32_MAX : nt);
    }
    return best;
}

size_t sics_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs) {
    return sics_ws(g, make_menu(g, cs)).total;
}

sa_status launch_sics(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Q,
                      const uint16_t* K, double* scores, int32_t* shape_idx, char* ws,
                      hipStream_t st) {
    const Menu m = make_menu(g, cs);
    const SicsWs w = sics_ws(g, m);
    double* U = reinterpret_cast<double*>(ws + w.u);
    int32_t* NZ = reinterpret_cast<int32_t*>(ws + w.nz);
    double* sc = scores ? scores : reinterpret_cast<double*>(ws + w.scores);
    const int64_t na = n_atoms(m);
    const dim3 ga((unsigned)ceil_div(na, 4), (unsigned)g.BH(), 2);
    if (g.d == 128)
        hipLaunchKernelGGL((k_sics_atoms<128>), ga, dim3(256), 0, st, Q, K, U, NZ, m, g.T, g.Hg, g.W, na);
    else
        hipLaunchKernelGGL((k_sics_atoms<64>), ga, dim3(256), 0, st, Q, K, U, NZ, m, g.T, g.Hg, g.W, na);
    sa_status e = hip_check(hipGetLastError(), "k_sics_atoms launch");
    if (e != SA_OK) return e;
    const int cmax = menu_cmax(m);
    double* tsics = reinterpret_cast<double*>(ws + w.tsics);
    double* tpairs = reinterpret_cast<double*>(ws + w.tpairs);
    const dim3 gt((unsigned)cmax, (unsigned)m.n, (unsigned)g.BH());
    if (g.d == 128)
        hipLaunchKernelGGL((k_sics_tiles<128>), gt, dim3(128), 0, st, U, NZ, tsics, tpairs,
                           cs.tile_coherence, m, g.T, g.Hg, g.W, na, cmax);
    else
        hipLaunchKernelGGL((k_sics_tiles<64>), gt, dim3(64), 0, st, U, NZ, tsics, tpairs,
                           cs.tile_coherence, m, g.T, g.Hg, g.W, na, cmax);
    if ((e = hip_check(hipGetLastError(), "k_sics_tiles launch")) != SA_OK) return e;
    hipLaunchKernelGGL(k_sics_shapes, dim3((unsigned)ceil_div(g.BH() * m.n, 4)), dim3(256), 0, st,
                       tsics, tpairs, sc, m, g.BH(), cmax);
    if ((e = hip_check(hipGetLastError(), "k_sics_shapes launch")) != SA_OK) return e;
    hipLaunchKernelGGL(k_sics_pick, dim3((unsigned)ceil_div(g.BH(), 256)), dim3(256), 0, st, sc,
                       shape_idx, m.n, g.BH());
    return hip_check(hipGetLastError(), "k_sics_pick launch");
}

sa_status launch_tile_assign(const Geometry& g, const sa_cluster_spec& cs, int32_t* assign,
                             hipStream_t st) {
    const Menu m = make_menu(g, cs);
    hipLaunchKernelGGL(k_tile_assign, dim3((unsigned)ceil_div(g.N, 256), (unsigned)g.BH()),
                       dim3(256), 0, st, cs.shape_idx, assign, m, g.T, g.Hg, g.W);
    return hip_check(hipGetLastError(), "k_tile_assign launch");
}

}  // namespace sa
