// plan.cpp -- the host planner: F2 algebra from a BMMC (A, c) to kernel tables.
//
// Source: "Efficient GPU Implementation of Affine Index Permutations on
// Arrays" (FHPNC'23).  The page's method sections (tiling, bank conflicts,
// iterations, the tiled-BMMC class and its factorisation) are lost from the
// extracted text; their results survive in the introduction, evaluation and
// appendix.  What survives fixes the following, and this file builds on it:
//  * a BMMC is y = A.x XOR c over F2 with A invertible (introduction);
//  * tiled BMMCs include every BPC and one tile pass moves them coalesced
//    (introduction, contributions); any BMMC factors as A = T1.T2 into two
//    tiled BMMCs, applied T2 first (introduction);
//  * n_over counts the low input bits that land in the low output bits, and a
//    random BMMC's factors behave differently from a random BPC there
//    (evaluation, the naive-kernel column of Figure 9);
//  * the iterated variant amortises index work over several tiles
//    (evaluation; appendix, the iterated bit-reversal kernel).
// The reconstruction (tile test, factorisation, fused single pass) is
// written from the F2 algebra; each step says what it guarantees.
#include "plan.h"

#include "kernels/tiled_cfg.h"

#include <algorithm>
#include <cstring>
#include <vector>

namespace bmmc {

namespace {

// ---------------------------------------------------------------------------
// Unit normalisation.
//
// The byte-level map of an array of 2^n elements of 2^e bytes is
// diag(I_e, A) with complement c << e.  Every further low bit that the map
// leaves in place (identity row, column used by no other row, complement bit
// 0) just widens the run of bytes that moves as one block.  The kernels move
// "units" of 2^k bytes, k <= 4 (one 16-byte vector), over the remaining
// nb = n + e - k index bits.
// ---------------------------------------------------------------------------
struct UnitMap {
    int ulog2 = 0;  // log2 bytes of a unit
    int nb = 0;     // index bits at unit granularity
    Mat A;          // nb x nb
    u64 c = 0;
};

UnitMap normalize(int n, const Mat &A, u64 c, int e) {
    const int nb = n + e;
    Mat Ab = Mat::zeros(nb, nb);
    for (int r = 0; r < e; ++r) Ab.r[r] = u64(1) << r;
    for (int r = 0; r < n; ++r) Ab.r[e + r] = A.r[r] << e;
    const u64 cb = c << e;
    int k = e;
    while (k < 4 && k < nb) {
        if (Ab.r[k] != (u64(1) << k) || ((cb >> k) & 1u)) break;
        bool used = false;
        for (int r = k + 1; r < nb; ++r)
            if ((Ab.r[r] >> k) & 1u) { used = true; break; }
        if (used) break;
        ++k;
    }
    UnitMap m;
    m.ulog2 = k;
    m.nb = nb - k;
    m.A = Mat::zeros(m.nb, m.nb);
    for (int r = 0; r < m.nb; ++r) m.A.r[r] = Ab.r[r + k] >> k;
    m.c = cb >> k;
    return m;
}

// Number of low index bits s such that A = diag(I_s, Q): the map moves
// 2^s-unit segments as wholes.
int low_identity_bits(const Mat &A) {
    int s = 0;
    while (s < A.rows) {
        if (A.r[s] != (u64(1) << s)) break;
        bool used = false;
        for (int r = s + 1; r < A.rows; ++r)
            if ((A.r[r] >> s) & 1u) { used = true; break; }
        if (used) break;
        ++s;
    }
    return s;
}

int popcount(u64 v) { return __builtin_popcountll(v); }

// n_over = t - rank(A[t:, 0:t]): the dimension of the low input space that
// stays in the low output bits.
int n_over_of(const Mat &A, int t) {
    if (t <= 0 || t >= A.rows) return t > 0 ? t : 0;
    Mat sub = Mat::zeros(A.rows - t, t);
    for (int i = t; i < A.rows; ++i) sub.r[i - t] = A.r[i] & low_mask(t);
    return t - rank(sub);
}

// The tile test.  With B = A^{-1}, column j < b of B is the input index that
// lands on output index e_j.  A tile made of the input rows of 2^a units
// spanned by the low a bits and a set H of b higher bits covers whole output
// rows of 2^b units iff every such column lies in span(low a bits, H), i.e.
// iff the rows r >= a that column j < b uses lie in H.  Returns that row set
// S; A is tiled for (a, b) iff |S| <= b (then any H containing S works).
// Square tiles have a = b = t.
u64 tile_rows(const Mat &B, int a, int b) {
    u64 S = 0;
    for (int r = a; r < B.rows; ++r)
        if (B.r[r] & low_mask(b)) S |= u64(1) << r;
    return S;
}

// Pad the required row set S to b rows above the a in-row bits.  With
// `near_out`, prefer input bits whose image is a single output bit in
// [b, b + a), the output row bits next to the rows (keeps a BPC tile's
// output rows close together); then take the lowest free bits.
u64 pad_rows(const Mat &A, u64 S, int a, int b, bool near_out) {
    u64 H = S;
    for (int pass = near_out ? 0 : 1; pass < 2 && popcount(H) < b; ++pass) {
        for (int j = a; j < A.rows && popcount(H) < b; ++j) {
            if ((H >> j) & 1u) continue;
            if (pass == 0) {
                u64 col = A.col(j);
                bool single = col && !(col & (col - 1));
                if (!single) continue;
                int o = __builtin_ctzll(col);
                if (o < b || o >= a + b) continue;
            }
            H |= u64(1) << j;
        }
    }
    return H;
}

// The pages' factorisation route, rebuilt from the algebra: with B = A^{-1},
// take an independent subset of the high parts (above the a in-row bits) of
// B's first b columns and complete it by unit vectors to a basis Q_hh of the
// high coordinates.  With Q = diag(I_a, Q_hh): T2 = Q^{-1} only relabels
// 2^a-unit segments, and T1 = A.Q is tiled with input rows of 2^a units and
// output rows of 2^b, its tile rows inside {a, ..., a+b-1}: T1^{-1} = Q^{-1}.B
// keeps the low parts of B's first b columns and maps each high part into the
// span of the first chosen vectors, at most b of them.  A = T1.T2.  The
// pages' tiles are square (a = b = t).
bool factorize(const Mat &A, int a, int b, Mat &T1, Mat &T2) {
    const int n = A.rows;
    Mat B;
    if (!inverse(A, B)) return false;
    Basis chosen;
    std::vector<u64> qcols;
    for (int j = 0; j < b; ++j) {
        u64 v = B.col(j) & ~low_mask(a);
        if (chosen.add(v)) qcols.push_back(v);
    }
    Basis all = chosen;
    for (int m = a; m < n; ++m)
        if (all.add(u64(1) << m)) qcols.push_back(u64(1) << m);
    if ((int)qcols.size() != n - a) return false;
    Mat Q = Mat::identity(n);
    for (int k = 0; k < n - a; ++k) Q.set_col(a + k, qcols[k]);
    if (!inverse(Q, T2)) return false;
    T1 = mul(A, Q);
    return true;
}

// ---------------------------------------------------------------------------
// LDS bank model used to choose the tile swizzle.  A wave's LDS access is
// served in groups of lanes that together touch at most `banks` dwords; a
// group takes as many cycles as the largest number of distinct dwords that
// fall into one bank.  gfx950's exact bank count and grouping are measured
// with the LDS bank-conflict counter; the planner minimises the cost under
// both a 32-bank and a 64-bank model so that either is conflict-free when
// possible.
// ---------------------------------------------------------------------------
int bank_cycles(const uint32_t *addr, int lanes, int bytes, int banks) {
    int per = bytes >= 4 ? (4 * banks) / bytes : banks;
    if (per > 64) per = 64;
    if (per < 1) per = 1;
    const int words = bytes >= 4 ? bytes / 4 : 1;
    int total = 0;
    uint32_t seen[64][64];
    int count[64];
    for (int g0 = 0; g0 < lanes; g0 += per) {
        for (int b = 0; b < banks; ++b) count[b] = 0;
        int mx = 0;
        for (int l = g0; l < lanes && l < g0 + per; ++l) {
            for (int w = 0; w < words; ++w) {
                const uint32_t dw = addr[l] / 4 + (uint32_t)w;
                const int b = (int)(dw % (uint32_t)banks);
                bool dup = false;  // same dword: a broadcast, no extra cycle
                for (int i = 0; i < count[b]; ++i)
                    if (seen[b][i] == dw) { dup = true; break; }
                if (dup || count[b] >= 64) continue;
                seen[b][count[b]++] = dw;
                mx = std::max(mx, count[b]);
            }
        }
        total += std::max(mx, 1);
    }
    return total;
}

u64 splitmix(u64 &s) {
    u64 z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

struct TileGeom {
    int ulog2, t, wl;  // unit, tile side, log2 units per vector chunk
    int cpsl;          // log2 chunks per segment (tile row)
    int ntl;           // log2 threads per workgroup
    int rppl;          // log2 rows handled per pass by the workgroup
};

TileGeom tile_geom(int ulog2, int t, int tl) {
    TileGeom g;
    g.ulog2 = ulog2;
    g.t = t;
    g.wl = std::min(4 - ulog2, t);
    g.cpsl = t - g.wl;
    g.ntl = tile_threads_log2(ulog2, t, tl);
    g.rppl = g.ntl - g.cpsl;
    return g;
}

}  // namespace

int max_tile_log2(int ulog2) {
    static const int t[5] = {8, 7, 7, 6, 6};
    return (ulog2 >= 0 && ulog2 <= 4) ? t[ulog2] : 0;
}

namespace {

// Tile side per unit size: rows of at least 256 bytes, and tiles of at least
// 16 KiB so that the persistent launch keeps enough bytes in flight (8-byte
// units with 8 KiB tiles measured 0.72 of copy, with 32 KiB tiles 0.89).
int default_tile_log2(int ulog2) {
    static const int t[5] = {8, 7, 6, 6, 5};
    return t[ulog2];
}

// How the tile pass is launched (planner's defaults and caller's options).
struct LaunchChoice {
    int iters_log2;  // one-tile launch: tiles staged together
    int persistent;  // BMMC_LAUNCH_PERSISTENT or _STREAMED; 0: one-tile launch
    int grid_log2;   // persistent: log2 workgroups requested
    int walk;        // persistent: BMMC_WALK_RANGES or BMMC_WALK_INTERLEAVED
    int block_map;   // 1 identity, 2 reversed, 3-5 locality orders, >= 8 random (seed)
    int depth;       // streamed: tiles of loads in flight per loader wave
    bool auto_launch;  // launch style left to the planner
    int cache_hint;    // descriptor value: 3 non-temporal loads and stores, 0 plain
    int threads_log2;  // most threads per tile, log2 (8 or 9)
    bool split;        // one-tile launch staging each tile in LDS half at a time
    bool buffer_loads; // one-tile launch reading the input with buffer loads
};

// Highest set bit of a byte offset (-1 for 0).
int top_bit(u64 v) { return v ? 63 - __builtin_clzll(v) : -1; }

// Re-index the tiles: new block bit k selects the XOR of the old columns in
// column k of an invertible map L.  The three block tables are linear in the
// block index, so they are transformed alike and the set of tiles is unchanged.
// Modes 2 (reversed bit order) and >= 8 (a seeded random L); the locality
// orders 3-7 are built into the block basis itself (block_basis).
void remap_blocks(bmmc_pass_desc *d, int mode) {
    const int nbk = d->blk_bits;
    if ((mode != 2 && mode < 8) || nbk < 2) return;
    std::vector<u64> cols(nbk);
    if (mode == 2) {
        for (int k = 0; k < nbk; ++k) cols[k] = u64(1) << (nbk - 1 - k);
    } else {
        u64 seed = 0xB10C0000ull + (u64)mode;
        for (;;) {
            Mat L = Mat::zeros(nbk, nbk);
            for (int k = 0; k < nbk; ++k) L.set_col(k, splitmix(seed) & low_mask(nbk));
            if (rank(L) == nbk) {
                for (int k = 0; k < nbk; ++k) cols[k] = L.col(k);
                break;
            }
        }
    }
    uint64_t in2[BMMC_MAX_BITS] = {}, out2[BMMC_MAX_BITS] = {};
    uint32_t lds2[BMMC_MAX_BITS] = {};
    for (int k = 0; k < nbk; ++k)
        for (int j = 0; j < nbk; ++j)
            if ((cols[k] >> j) & 1u) {
                in2[k] ^= d->in_blk[j];
                out2[k] ^= d->out_blk[j];
                lds2[k] ^= d->lds_blk[j];
            }
    for (int k = 0; k < nbk; ++k) {
        d->in_blk[k] = in2[k];
        d->out_blk[k] = out2[k];
        d->lds_blk[k] = lds2[k];
    }
}

// Block basis of a tile pass: input vectors x_0 .. x_{m-1}, independent
// modulo the tile space V, such that block index b names the tile
// (XOR of x_k over the set bits k of b) + V.  Any such basis tiles the array;
// the choice only decides which tiles are in flight together.
//
// Mode 1 takes the input coordinates that are no pivot of V (the identity
// order).  Modes 3-7 draw from two candidate lists, each sorted nearest first
// by the top bit of the candidate's representative reduced modulo the tile's
// own span on that side: input-aligned vectors e_r (near on the input side)
// and output-aligned vectors B e_r (A x = e_r, near on the output side).  For
// a bit-permute-complement matrix the two lists hold the same vectors.  The
// tiles in flight together differ in the `conc` concurrent block bits (the
// top grid_log2 bits of a range walk, whose workgroups start far apart and
// move in step) or in the low bits (one-tile launches and the interleaved
// walk, conc = 0); picks go to the concurrent bits first, then to the other
// bits from bit 0 up:
//   3: alternately input- and output-nearest, 4: input-nearest,
//   5: output-nearest, 6: output-nearest for the concurrent bits and then
//   input-nearest, 7: the reverse of 6.
std::vector<u64> block_basis(const Mat &A, const Mat &B, int t, const Basis &vb,
                             const Basis &avb, const std::vector<int> &R, int mode, int conc) {
    const int nb = A.rows, m = (int)R.size();
    std::vector<u64> X(m);
    if (mode < 3 || mode > 7) {
        for (int k = 0; k < m; ++k) X[k] = u64(1) << R[k];
        return X;
    }
    struct Cand { int key; u64 x; };
    std::vector<Cand> near[2];
    for (int r = t; r < nb; ++r) {
        near[0].push_back({top_bit(vb.reduce(u64(1) << r)), u64(1) << r});
        near[1].push_back({top_bit(avb.reduce(u64(1) << r)), B.apply(u64(1) << r)});
    }
    for (auto &v : near)
        std::stable_sort(v.begin(), v.end(), [](const Cand &a, const Cand &b) { return a.key < b.key; });
    Basis acc = vb;
    size_t pos[2] = {0, 0};
    for (int i = 0; i < m; ++i) {
        int side;
        switch (mode) {
        case 3: side = i & 1; break;
        case 4: side = 0; break;
        case 5: side = 1; break;
        case 6: side = i < conc ? 1 : 0; break;
        default: side = i < conc ? 0 : 1; break;
        }
        // next independent candidate of that side; the other side if it has none
        u64 x = 0;
        for (int tries = 0; tries < 2 && !x; ++tries, side ^= 1)
            for (; pos[side] < near[side].size() && !x; ++pos[side])
                if (acc.add(near[side][pos[side]].x)) x = near[side][pos[side]].x;
        // stored reduced modulo V: only non-pivot coordinates >= t remain, so
        // the tile's input rows start on row boundaries
        const int k = i < conc ? m - conc + i : i - conc;
        X[k] = vb.reduce(x);
    }
    return X;
}

// Build the tile pass for unit map (A, c) with input rows of 2^a units (the
// low a bits) and b row vectors W (high coordinates, independent).  The tile
// of block x is the coset x XOR span(low a bits) XOR span(W); because W
// contains the high parts of B's first b columns, the tile's image is 2^a
// whole output rows of 2^b units.  Square tiles have a = b = t; rectangular
// ones keep 2^(a + b) = 2^(2t) units, the kernel's tile.
int build_tiled(const Mat &A, u64 c, int ulog2, int a, int b, const std::vector<u64> &W,
                const LaunchChoice &lc, bool swizzle, bmmc_pass_desc *d) {
    int iters_log2 = lc.iters_log2;
    const int nb = A.rows;
    const int K = a + b;  // log2 units per tile
    if (a < 1 || b < 1 || (K & 1) || (int)W.size() != b || K > nb) return BMMC_ERR_INVALID_ARG;
    const int t = K / 2;  // the kernel's tile side: 2^(2t) units per tile
    const u64 lo_a = low_mask(a), lo_b = low_mask(b);
    Basis wb;
    for (u64 w : W) {
        if (w & lo_a) return BMMC_ERR_INVALID_ARG;
        if (!wb.add(w)) return BMMC_ERR_INVALID_ARG;
    }
    // Block bits: high coordinates that are no pivot of W; together with W
    // they form a basis of the high coordinates.
    std::vector<int> R;
    const u64 piv = wb.pivot_mask();
    for (int r = a; r < nb; ++r)
        if (!((piv >> r) & 1u)) R.push_back(r);
    if ((int)R.size() != nb - K) return BMMC_ERR_INVALID_ARG;
    const int blk_bits = (int)R.size();
    if (iters_log2 > blk_bits) iters_log2 = blk_bits;

    // Output rows of the tile: a basis G of the high parts (above the b
    // in-row output bits) of A's image of the tile's local space.
    Basis gb;
    for (int j = 0; j < a; ++j) gb.add(A.apply(u64(1) << j) & ~lo_b);
    for (int k = 0; k < b; ++k) gb.add(A.apply(W[k]) & ~lo_b);
    if (gb.size() != a) return BMMC_ERR_INVALID_ARG;

    // M: local input coordinates (in-row bits 0..a-1, row bits a..K-1) ->
    // local output coordinates (position in the output row 0..b-1, output
    // row index b..K-1).
    Mat M = Mat::zeros(K, K);
    for (int j = 0; j < K; ++j) {
        u64 v = j < a ? A.apply(u64(1) << j) : A.apply(W[j - a]);
        u64 hi = v & ~lo_b;
        if (gb.reduce(hi) != 0) return BMMC_ERR_INVALID_ARG;
        M.set_col(j, (v & lo_b) | (gb.coords(hi) << b));
    }
    Mat Minv;
    if (!inverse(M, Minv)) return BMMC_ERR_INVALID_ARG;

    const TileGeom g = tile_geom(ulog2, t, lc.threads_log2);
    // both rows must hold whole vector chunks of the kernel's width
    if (a < g.wl || b < g.wl) return BMMC_ERR_INVALID_ARG;
    const int cpsl_in = a - g.wl, cpsl_out = b - g.wl;  // log2 chunks per row, each side
    const int cbits = K - g.wl;  // chunk-index bits of a tile: thread bits, then pass bits
    const int lane_bits = std::min(6, g.ntl);
    const int lanes = 1 << lane_bits;

    // Chunk coordinates.  Load phase: position p < cpsl is bit p of the
    // chunk's place in its input row, then the row bits; the threads of a
    // wave read whole rows.  Drain phase: coordinate k < cpsl is bit k of the
    // chunk's place in its output segment, then the segment bits; which
    // coordinate each thread bit takes (`rpos`) is chosen below.
    auto load_local = [&](int p) -> u64 {  // local input vector of load position p
        return p < cpsl_in ? (u64(1) << (g.wl + p)) : (u64(1) << (a + p - cpsl_in));
    };
    auto drain_local = [&](int k) -> u64 {  // local output vector of drain coordinate k
        return k < cpsl_out ? (u64(1) << (g.wl + k)) : (u64(1) << (b + k - cpsl_out));
    };

    // LDS layout: the slot of local (lo, h) is (h << a) | (P.lo XOR S.h),
    // with P an invertible map of the chunk index inside an input row and S
    // an XOR swizzle by row; both leave the units of a chunk together, so a
    // chunk is written with one vector access.  Sx = S's b columns, then P's
    // a columns.
    auto slot = [&](u64 u, const std::vector<u64> &Sx) -> u64 {
        u64 lo = u & lo_a, h = u >> a, s = 0;
        for (int k = 0; k < b; ++k)
            if ((h >> k) & 1u) s ^= Sx[k];
        for (int k = 0; k < a; ++k)
            if ((lo >> k) & 1u) s ^= Sx[b + k];
        return (h << a) | s;
    };

    // Bank model.  Measured on gfx950 with the LDS bank-conflict counter:
    // 4-byte reads behave as 32 banks serving a half-wave per cycle; 16-byte
    // accesses are conflict-free when each group of 8 lanes covers 8 distinct
    // 16-byte bank groups.  The cost weights that model first and a 64-bank
    // full-wave model second.
    const int rbytes = 1 << ulog2, wbytes = 1 << (ulog2 + g.wl);
    auto ideal_cycles = [&](int bytes, int banks) {
        const int per = std::min(64, bytes >= 4 ? (4 * banks) / bytes : banks);
        return (lanes + per - 1) / per;
    };
    const int ideal = 8 * ideal_cycles(rbytes, 32) + 2 * ideal_cycles(rbytes, 64) +
                      ideal_cycles(wbytes, 32) + ideal_cycles(wbytes, 64);
    std::vector<u64> lvec(cbits);  // local input vector of each load position
    for (int p = 0; p < cbits; ++p) lvec[p] = load_local(p);
    auto cost_lv = [&](const std::vector<u64> &lv, const std::vector<u64> &rv,
                       const std::vector<u64> &Sx) {
        uint32_t wa[64], ra[64];
        uint32_t wcol[6], rcol[6];
        for (int p = 0; p < lane_bits; ++p) {
            wcol[p] = (uint32_t)(slot(lv[p], Sx) << ulog2);
            rcol[p] = (uint32_t)(slot(rv[p], Sx) << ulog2);
        }
        for (int l = 0; l < lanes; ++l) {
            uint32_t a = 0, b = 0;
            for (int p = 0; p < lane_bits; ++p)
                if ((l >> p) & 1) { a ^= wcol[p]; b ^= rcol[p]; }
            wa[l] = a;
            ra[l] = b;
        }
        return 8 * bank_cycles(ra, lanes, rbytes, 32) + 2 * bank_cycles(ra, lanes, rbytes, 64) +
               bank_cycles(wa, lanes, wbytes, 32) + bank_cycles(wa, lanes, wbytes, 64);
    };
    auto cost = [&](const std::vector<u64> &rv, const std::vector<u64> &Sx) {
        return cost_lv(lvec, rv, Sx);
    };

    // Drain-phase lane layout: the first `pc` thread bits stay on the low
    // chunk bits of the output segment so that 8 lanes store one contiguous
    // 128-byte piece; the remaining lane bits of the wave are searched.
    int cb_log2 = ulog2 + g.wl;
    const int pc = std::min(cpsl_out, std::max(0, 7 - cb_log2));
    std::vector<int> rpos(cbits);
    for (int k = 0; k < cbits; ++k) rpos[k] = k;
    std::vector<u64> S(K, 0);
    for (int k = 0; k < a; ++k) S[b + k] = u64(1) << k;  // P = identity, S = 0
    auto read_vecs = [&](const std::vector<int> &rp) {
        std::vector<u64> rv(cbits);
        for (int p = 0; p < cbits; ++p) rv[p] = Minv.apply(drain_local(rp[p]));
        return rv;
    };
    if (swizzle && a > g.wl) {
        const u64 colmask = lo_a & ~low_mask(g.wl);
        // the square tiles keep the seed they were tuned and measured with
        u64 seed = 0x5EEDull ^ ((u64)t << 8) ^ (u64)ulog2 ^ ((u64)(b - a) << 16);
        for (int k = 0; k < K; ++k) seed = seed * 31 + Minv.r[k];
        int best_cost = 1 << 30;
        std::vector<int> best_rpos = rpos;
        std::vector<u64> best_S = S, cand(K);
        auto random_p = [&](std::vector<u64> &Sx) {
            for (;;) {
                Mat Pm = Mat::zeros(a, a);
                for (int k = 0; k < a; ++k)
                    Pm.set_col(k, k < g.wl ? (u64(1) << k) : (splitmix(seed) & colmask));
                if (rank(Pm) == a) {
                    for (int k = 0; k < a; ++k) Sx[b + k] = Pm.col(k);
                    return;
                }
            }
        };
        // Bits of a source position that no swizzle can move: the unit bits
        // inside a chunk that select different dwords.  The lanes of one
        // conflict group must span them.
        const u64 fixed = low_mask(g.wl) & ~low_mask(std::max(0, 2 - ulog2));
        const int grp_per = std::min(64, rbytes >= 4 ? 128 / rbytes : 32);
        const int grp_bits = std::min(lane_bits, __builtin_ctz((unsigned)grp_per));
        // ordered choices for the free lane positions pc .. lane_bits-1
        const int nfree = std::max(0, lane_bits - pc);
        std::vector<int> pool;
        for (int k = pc; k < cbits; ++k) pool.push_back(k);
        std::vector<int> sel(nfree, 0);
        int budget = 4000;
        bool more = true;
        while (more && best_cost > ideal && budget > 0) {
            // build rpos from sel (indices into pool, all distinct)
            bool distinct = true;
            for (int a = 0; a < nfree && distinct; ++a)
                for (int b = a + 1; b < nfree; ++b)
                    if (sel[a] == sel[b]) { distinct = false; break; }
            if (distinct && (int)pool.size() >= nfree) {
                std::vector<int> rp;
                for (int k = 0; k < pc; ++k) rp.push_back(k);
                for (int a = 0; a < nfree; ++a) rp.push_back(pool[sel[a]]);
                for (int k : pool)
                    if (std::find(rp.begin(), rp.end(), k) == rp.end()) rp.push_back(k);
                const std::vector<u64> rv = read_vecs(rp);
                // pre-filter: the conflict group's lanes must span the fixed bits
                Basis fb;
                for (int p = 0; p < grp_bits; ++p) fb.add(rv[p] & fixed);
                if (fb.size() == __builtin_popcountll(fixed)) {
                    auto consider = [&](const std::vector<u64> &Sx) {
                        --budget;
                        int cc = cost(rv, Sx);
                        if (cc < best_cost) { best_cost = cc; best_rpos = rp; best_S = Sx; }
                    };
                    for (int k = 0; k < b; ++k) cand[k] = 0;
                    for (int k = 0; k < a; ++k) cand[b + k] = u64(1) << k;
                    consider(cand);
                    for (int k = 0; k < b; ++k) cand[k] = (u64(1) << k) & colmask;
                    consider(cand);
                    for (int tries = 0; tries < 48 && best_cost > ideal && budget > 0; ++tries) {
                        for (int k = 0; k < b; ++k) cand[k] = splitmix(seed) & colmask;
                        if (tries & 1) random_p(cand);
                        else for (int k = 0; k < a; ++k) cand[b + k] = u64(1) << k;
                        consider(cand);
                    }
                }
            }
            // next tuple (odometer over pool indices)
            int a = nfree - 1;
            while (a >= 0 && ++sel[a] == (int)pool.size()) sel[a--] = 0;
            if (a < 0) more = false;
        }
        if (best_cost < (1 << 30)) {
            rpos = best_rpos;
            S = best_S;
        }
    }
    std::vector<u64> rvec = read_vecs(rpos), ovec(cbits);
    for (int p = 0; p < cbits; ++p) ovec[p] = drain_local(rpos[p]);

    // Split staging: the tile passes through LDS in two halves.  A linear
    // functional g of the local input coordinates names the half of every
    // unit; the tables are rebased so that g of a chunk is the top bit of its
    // chunk index on both sides (for the drain, after a per-tile flip folded
    // into the block tables), and the LDS slot drops one address bit on which
    // g is 1, so each half fits half the LDS.  g must be 0 on the units of a
    // chunk (on both sides), on the in-row load positions (each half still
    // reads whole input rows) and on the drain's 128-byte lane groups.
    const int top = cbits - 1;
    u64 gmask = 0;   // g(x) = parity(gmask & x)
    int qdrop = -1;  // LDS slot bit dropped
    auto par = [](u64 m, u64 x) { return (int)__builtin_parityll(m & x); };
    if (lc.split) {
        if (top < g.ntl) return BMMC_ERR_INVALID_ARG;  // one pass per tile: nothing to split
        Basis keep;
        for (int u = 0; u < g.wl; ++u) {
            keep.add(u64(1) << u);
            keep.add(Minv.apply(u64(1) << u));
        }
        for (int p = 0; p < cpsl_in; ++p) keep.add(lvec[p]);
        for (int p = 0; p < pc; ++p) keep.add(rvec[p]);
        // functionals vanishing on `keep`: one per free coordinate f, e_f plus
        // the pivots of the (fully reduced) kept vectors that have bit f
        std::vector<u64> ns;
        const u64 piv = keep.pivot_mask();
        for (int f = 0; f < K; ++f) {
            if ((piv >> f) & 1u) continue;
            u64 gv = u64(1) << f;
            for (int k = 0; k < keep.size(); ++k)
                if ((keep.vec[k] >> f) & 1u) gv |= u64(1) << keep.pivot[k];
            ns.push_back(gv);
        }
        // slot^-1 of each LDS address bit
        Mat SL = Mat::zeros(K, K);
        for (int i = 0; i < K; ++i) SL.set_col(i, slot(u64(1) << i, S));
        Mat SLinv;
        if (!inverse(SL, SLinv)) return BMMC_ERR_INVALID_ARG;
        // dropped bits stay above the 256 bytes of one row of LDS banks, so
        // the lanes of an access keep their banks
        const int qmin = std::max(0, 8 - ulog2);
        int best = 1 << 30, best_lt = -1, best_dt = -1;
        const int ncomb = ns.size() > 12 ? 1 << 12 : 1 << ns.size();
        for (int comb = 1; comb < ncomb; ++comb) {
            u64 gm = 0;
            for (size_t k = 0; k < ns.size(); ++k)
                if ((comb >> k) & 1) gm ^= ns[k];
            int q = -1;
            for (int bq = K - 1; bq >= qmin && q < 0; --bq)
                if (par(gm, SLinv.apply(u64(1) << bq))) q = bq;
            // the positions that become the top one: the highest on which g
            // is 1 (a pass bit where there is one, else a thread bit; g is 0
            // on the positions that must keep their place)
            int lt = -1, dt = -1;
            for (int p = top; p >= 0 && lt < 0; --p)
                if (par(gm, lvec[p])) lt = p;
            for (int p = top; p >= 0 && dt < 0; --p)
                if (par(gm, rvec[p])) dt = p;
            if (q < 0 || lt < 0 || dt < 0) continue;
            std::vector<u64> L = lvec, R = rvec;
            std::swap(L[lt], L[top]);
            std::swap(R[dt], R[top]);
            for (int p = 0; p < top; ++p) {
                if (par(gm, L[p])) L[p] ^= L[top];
                if (par(gm, R[p])) R[p] ^= R[top];
            }
            const int cc = cost_lv(L, R, S);
            if (cc < best) {
                best = cc;
                gmask = gm;
                qdrop = q;
                best_lt = lt;
                best_dt = dt;
            }
        }
        if (qdrop < 0) return BMMC_ERR_INVALID_ARG;
        std::swap(lvec[best_lt], lvec[top]);
        std::swap(rvec[best_dt], rvec[top]);
        std::swap(ovec[best_dt], ovec[top]);
        for (int p = 0; p < top; ++p) {
            if (par(gmask, lvec[p])) lvec[p] ^= lvec[top];
            if (par(gmask, rvec[p])) {
                rvec[p] ^= rvec[top];
                ovec[p] ^= ovec[top];
            }
        }
    }
    // byte offset in LDS of a slot (the dropped bit removed when split)
    auto lds_off = [&](u64 sl) -> uint32_t {
        if (qdrop >= 0) sl = (sl & low_mask(qdrop)) | ((sl >> (qdrop + 1)) << qdrop);
        return (uint32_t)(sl << ulog2);
    };
    // output offset (units) of a local output vector: in-row part plus rows
    auto out_local_of = [&](u64 ov) {
        u64 o = ov & lo_b;
        for (int k = 0; k < a; ++k)
            if (((ov >> b) >> k) & 1u) o ^= gb.vec[k];
        return o;
    };

    std::memset(d, 0, sizeof(*d));
    d->kernel = BMMC_KERNEL_TILED;
    d->unit_log2 = ulog2;
    d->nbits = nb;
    d->t = t;
    d->chunk_log2 = g.wl;
    d->blk_bits = blk_bits;
    d->in_row_log2 = a;
    d->out_row_log2 = b;
    d->threads_log2 = g.ntl;
    const u64 tile_bytes = u64(1) << (K + ulog2);
    int launch = lc.persistent;
    // Planner's choice, measured untuned with the default tile order: below
    // 2^14 tiles the streamed launch with loads two tiles ahead (the 64 MiB
    // transpose: 0.87 of copy against 0.84 persistent; random BPC and BMMC
    // at n = 24 alike); above, the persistent launch (the 16384 x 16384
    // transpose: 0.90 against 0.85 streamed; random BMMC n = 28 even).
    if (lc.auto_launch && launch) launch = blk_bits < 14 ? BMMC_LAUNCH_STREAMED
                                                         : BMMC_LAUNCH_PERSISTENT;
    // the streamed launch splits waves by role, so each role needs whole waves
    if (launch == BMMC_LAUNCH_STREAMED && g.ntl < 6) launch = BMMC_LAUNCH_PERSISTENT;
    if (launch && 2 * tile_bytes <= kMaxPersistentLdsBytes) {
        // persistent: two LDS tiles (double buffer), no staged iterations
        d->launch = launch;
        d->iters_log2 = 0;
        // One workgroup per compute unit (2^8 on a 256-CU MI355X) walking
        // long tile ranges measured best for large arrays; below 2^14 tiles
        // two per compute unit shorten each walk.
        const int want = lc.grid_log2 ? lc.grid_log2
                                      : (blk_bits >= 14 ? kDefaultGridLog2 : kDefaultGridLog2 + 1);
        d->grid_log2 = std::max(0, std::min(want, blk_bits));
        d->walk = lc.walk;
        d->depth = launch == BMMC_LAUNCH_STREAMED ? lc.depth : 1;
        d->lds_bytes = (uint32_t)(2 * tile_bytes);
    } else {
        d->launch = BMMC_LAUNCH_ONE_TILE;
        d->iters_log2 = iters_log2;
        d->lds_bytes = (uint32_t)(tile_bytes << iters_log2);
        if (lc.split) {
            if (iters_log2) return BMMC_ERR_INVALID_ARG;
            d->split_stage = 1;
            d->lds_bytes = (uint32_t)(tile_bytes / 2);
        }
    }
    if (lc.split && d->launch != BMMC_LAUNCH_ONE_TILE) return BMMC_ERR_INVALID_ARG;
    // Buffer loads address the input by 32-bit offsets from its base: whole
    // tiles of 4-byte units or larger, one per workgroup, in arrays of at
    // most 2^31 bytes (the offsets stay below the buffer's size limit).
    if (lc.buffer_loads) {
        if (d->launch != BMMC_LAUNCH_ONE_TILE || d->iters_log2 || d->split_stage ||
            ulog2 < 2 || nb + ulog2 > kBufferLoadMaxLog2)
            return BMMC_ERR_INVALID_ARG;
        d->buffer_loads = 1;
    }
    Basis vb, avb;  // the tile's span on the input side and on the output side
    for (int j = 0; j < a; ++j) vb.add(u64(1) << j);
    for (int j = 0; j < b; ++j) avb.add(u64(1) << j);
    for (int k = 0; k < b; ++k) vb.add(W[k]);
    for (int k = 0; k < a; ++k) avb.add(gb.vec[k]);
    Mat Binv;
    if (!inverse(A, Binv)) return BMMC_ERR_SINGULAR;
    const bool range_walk = d->launch != BMMC_LAUNCH_ONE_TILE && d->walk == BMMC_WALK_RANGES;
    const std::vector<u64> X =
        block_basis(A, Binv, std::min(a, b), vb, avb, R, lc.block_map,
                    range_walk ? d->grid_log2 : 0);
    // A tile's drain base is the local input vector of its in-row output
    // offset; where g is 1 on it, the split drain takes the halves in the
    // other order (the top drain position is XORed into the base), so that
    // drain half h again reads the units staged in half h.
    auto drain_base = [&](u64 zlo, u64 zhi, uint64_t &out_b, uint32_t &lds_b) {
        u64 x = Minv.apply(zlo), o = zhi;
        if (par(gmask, x)) {
            x ^= rvec[top];
            o ^= out_local_of(ovec[top]);
        }
        out_b = o << ulog2;
        lds_b = lds_off(slot(x, S));
    };
    for (int k = 0; k < blk_bits; ++k) {
        const u64 x = X[k];
        const u64 z = A.apply(x);
        d->in_blk[k] = x << ulog2;
        drain_base(z & lo_b, z & ~lo_b, d->out_blk[k], d->lds_blk[k]);
    }
    for (int p = 0; p < cbits; ++p) {
        const u64 lv = lvec[p];
        const u64 in_local = (lv & lo_a) | [&] {
            u64 h = lv >> a, off = 0;
            for (int k = 0; k < b; ++k)
                if ((h >> k) & 1u) off ^= W[k];
            return off;
        }();
        d->ld_in[p] = in_local << ulog2;
        d->ld_lds[p] = lds_off(slot(lv, S));
        d->st_out[p] = out_local_of(ovec[p]) << ulog2;
        d->st_lds[p] = lds_off(slot(rvec[p], S));
    }
    for (int u = 0; u < g.wl; ++u) d->st_unit[u] = lds_off(slot(Minv.apply(u64(1) << u), S));
    drain_base(c & lo_b, c & ~lo_b, d->out_c, d->lds_c);
    d->cache_hint = lc.cache_hint;
    d->block_map = lc.block_map;
    remap_blocks(d, lc.block_map);
    return BMMC_OK;
}

// Chunk pass: A = diag(I_s, Q) with s >= chunk bits; each chunk of 2^wl units
// moves as a whole, with the complement's low bits permuting units inside it.
// Also used, with one-unit chunks, for the naive pass (any A).
void build_chunk(const Mat &A, u64 c, int ulog2, int wl, int kernel, bmmc_pass_desc *d) {
    std::memset(d, 0, sizeof(*d));
    const int nb = A.rows;
    d->kernel = kernel;
    d->unit_log2 = ulog2;
    d->nbits = nb;
    d->chunk_log2 = wl;
    d->blk_bits = nb - wl;
    d->unit_xor = (int32_t)(c & low_mask(wl));
    if (kernel == BMMC_KERNEL_CHUNK) {
        // gather: output chunk y comes from input A^-1.(y XOR c); A keeps
        // the low wl bits, so A^-1 maps chunk bits to chunk bits and the
        // complement's low bits permute the units inside a chunk
        Mat Ainv;
        inverse(A, Ainv);
        for (int k = 0; k < nb - wl; ++k) d->in_blk[k] = Ainv.apply(u64(1) << (k + wl)) << ulog2;
        d->in_c = (Ainv.apply(c) & ~low_mask(wl)) << ulog2;
    } else {
        for (int k = 0; k < nb - wl; ++k) d->out_blk[k] = A.apply(u64(1) << (k + wl)) << ulog2;
        d->out_c = (c & ~low_mask(wl)) << ulog2;
    }
    // whole chunks stream through with non-temporal hints; the naive pass's
    // scattered one-unit stores measured far slower with them
    d->cache_hint = kernel == BMMC_KERNEL_NAIVE ? 0 : 3;
}

void build_copy(int nb, int ulog2, bmmc_pass_desc *d) {
    std::memset(d, 0, sizeof(*d));
    d->kernel = BMMC_KERNEL_COPY;
    d->unit_log2 = ulog2;
    d->nbits = nb;
}

// Element-level view of a unit-level factor: the d low element-index bits that
// the unit absorbed stay in place.
void to_element_level(const Mat &T, u64 c, int dlow, int n, uint64_t *rows, uint64_t *c_out) {
    for (int r = 0; r < n; ++r)
        rows[r] = r < dlow ? (u64(1) << r) : (T.r[r - dlow] << dlow);
    *c_out = c << dlow;
}

}  // namespace

int build_plan(int n, const uint64_t *Arows, uint64_t c, size_t elem_bytes,
               const bmmc_plan_options *opt, bmmc_plan *p) {
    bmmc_plan_options o = {};
    if (opt) o = *opt;
    if (n < 1 || n > BMMC_MAX_N || !Arows) return BMMC_ERR_INVALID_ARG;
    if (elem_bytes == 0 || elem_bytes > 16 || (elem_bytes & (elem_bytes - 1)))
        return BMMC_ERR_INVALID_ARG;
    if (o.route < BMMC_ROUTE_AUTO || o.route > BMMC_ROUTE_FUSED) return BMMC_ERR_INVALID_ARG;
    if (o.tile_log2 < 0 || o.tile_log2 > BMMC_MAX_TILE || o.iters_log2 < 0 || o.iters_log2 > 3)
        return BMMC_ERR_INVALID_ARG;
    if (o.launch < BMMC_LAUNCH_AUTO || o.launch > BMMC_LAUNCH_STREAMED || o.grid_log2 < 0 ||
        o.grid_log2 > 24)
        return BMMC_ERR_INVALID_ARG;
    if (o.launch >= BMMC_LAUNCH_PERSISTENT && o.iters_log2 > 0) return BMMC_ERR_INVALID_ARG;
    if (o.walk < BMMC_WALK_AUTO || o.walk > BMMC_WALK_INTERLEAVED) return BMMC_ERR_INVALID_ARG;
    if (o.tile_skew < -BMMC_MAX_TILE || o.tile_skew > BMMC_MAX_TILE) return BMMC_ERR_INVALID_ARG;
    LaunchChoice lc;
    lc.iters_log2 = o.iters_log2;
    lc.auto_launch = o.launch == BMMC_LAUNCH_AUTO;
    lc.persistent = o.launch >= BMMC_LAUNCH_PERSISTENT ? o.launch
                    : (o.launch == BMMC_LAUNCH_AUTO && o.iters_log2 == 0) ? BMMC_LAUNCH_PERSISTENT
                                                                          : 0;
    lc.grid_log2 = o.grid_log2;  // 0: chosen per pass from the tile count
    lc.walk = o.walk ? o.walk : BMMC_WALK_RANGES;
    if (o.block_map < 0) return BMMC_ERR_INVALID_ARG;
    if (o.depth < 0 || o.depth > 2) return BMMC_ERR_INVALID_ARG;
    if (o.cache_hint < 0 || o.cache_hint > 2) return BMMC_ERR_INVALID_ARG;
    // Planner's choice: non-temporal loads and stores (measured on the four
    // large workloads: +1% to +5% over no hint; loads alone lose).
    lc.cache_hint = o.cache_hint == 1 ? 0 : 3;
    // Planner's choice: one tile of loads in flight per loader wave.  Two
    // use every VGPR and spill 32 bytes per thread in the loop (4-byte units,
    // t = 7); tuning tries them, and keeps them only when they win by more
    // than its margin.
    lc.depth = o.depth ? o.depth : 1;
    lc.block_map = o.block_map ? o.block_map : kDefaultBlockMap;
    if (o.tile_threads_log2 < 0 || o.tile_threads_log2 > kTileWideNTL) return BMMC_ERR_INVALID_ARG;
    // Planner's choice: 256 threads per tile; 512 are a tuning candidate.
    // Below 256 chunks per tile the count is the chunk count either way.
    lc.threads_log2 = o.tile_threads_log2 ? std::max(o.tile_threads_log2, kTileMaxNTL)
                                          : kTileMaxNTL;
    // Split staging is a form of the one-tile launch.
    if (o.split_stage < 0 || o.split_stage > 1) return BMMC_ERR_INVALID_ARG;
    if (o.split_stage && (o.launch == BMMC_LAUNCH_PERSISTENT ||
                          o.launch == BMMC_LAUNCH_STREAMED || o.iters_log2 != 0))
        return BMMC_ERR_INVALID_ARG;
    lc.split = o.split_stage == 1;
    if (lc.split) lc.persistent = 0;
    // Buffer loads are a form of the one-tile launch of whole tiles.
    if (o.buffer_loads < 0 || o.buffer_loads > 1) return BMMC_ERR_INVALID_ARG;
    if (o.buffer_loads && (o.launch == BMMC_LAUNCH_PERSISTENT ||
                           o.launch == BMMC_LAUNCH_STREAMED || o.iters_log2 != 0 ||
                           o.split_stage))
        return BMMC_ERR_INVALID_ARG;
    lc.buffer_loads = o.buffer_loads == 1;
    if (lc.buffer_loads) lc.persistent = 0;
    const int e = __builtin_ctzll((u64)elem_bytes);
    if (n + e > BMMC_MAX_BITS) return BMMC_ERR_INVALID_ARG;
    const u64 hi = ~low_mask(n);
    Mat A = Mat::zeros(n, n);
    for (int r = 0; r < n; ++r) {
        if (Arows[r] & hi) return BMMC_ERR_INVALID_ARG;
        A.r[r] = Arows[r];
    }
    if (c & hi) return BMMC_ERR_INVALID_ARG;
    Mat Ainv;
    if (!inverse(A, Ainv)) return BMMC_ERR_SINGULAR;

    p->n = n;
    p->elem_bytes = (int)elem_bytes;
    std::memcpy(p->A, Arows, sizeof(uint64_t) * (size_t)n);
    p->c = c;

    const UnitMap m = normalize(n, A, c, e);
    const int dlow = m.ulog2 - e;
    bmmc_plan_info &info = p->info;
    info = bmmc_plan_info{};
    info.n = n;
    info.elem_bytes = (int)elem_bytes;
    info.unit_bytes = 1 << m.ulog2;
    info.unit_bits = m.nb;

    int t = o.tile_log2 ? o.tile_log2 : default_tile_log2(m.ulog2);
    t = std::min(t, max_tile_log2(m.ulog2));
    t = std::min(t, m.nb / 2);
    while (t > 0 && ((u64(1) << (2 * t + m.ulog2)) << o.iters_log2) > kMaxLdsBytes) --t;

    // classification
    const bool ident = m.nb == 0 || m.A.is_identity();
    Mat B;
    if (m.nb > 0) inverse(m.A, B);
    const u64 S = (m.nb > 0 && t > 0) ? tile_rows(B, t, t) : 0;
    if (ident) info.kind = BMMC_KIND_IDENTITY;
    else if (is_permutation_matrix(m.A)) info.kind = BMMC_KIND_BPC;
    else if (t > 0 && popcount(S) <= t) info.kind = BMMC_KIND_TILED;
    else info.kind = BMMC_KIND_GENERAL;
    info.n_over = (m.nb > 0 && t > 0) ? n_over_of(m.A, t) : 0;

    auto single = [&](int route) {
        p->npasses = 1;
        info.passes = 1;
        info.route = route;
        to_element_level(m.A, m.c, dlow, n, p->factor_A[0], &p->factor_c[0]);
    };

    // identity order: the copy kernel
    if (ident && m.c == 0) {
        build_copy(m.nb, m.ulog2, &p->pass[0]);
        single(BMMC_ROUTE_FUSED);
        return BMMC_OK;
    }
    // naive: forced, or too few bits for a tile
    if (o.route == BMMC_ROUTE_NAIVE || t < 1) {
        build_chunk(m.A, m.c, m.ulog2, 0, BMMC_KERNEL_NAIVE, &p->pass[0]);
        single(BMMC_ROUTE_NAIVE);
        return BMMC_OK;
    }
    // whole segments move: chunk kernel, no LDS
    const int sid = low_identity_bits(m.A);
    if (sid >= t) {
        const int wl = std::min(4 - m.ulog2, sid);
        // complement only (A = I after the unit merge): read in order, store
        // reversed; segment moves: write in order, gather
        build_chunk(m.A, m.c, m.ulog2, wl,
                    ident ? BMMC_KERNEL_CHUNK_SCATTER : BMMC_KERNEL_CHUNK, &p->pass[0]);
        single(BMMC_ROUTE_FUSED);
        return BMMC_OK;
    }
    const bool swz = !o.no_swizzle;
    // single-pass tile shape: input rows of 2^a units, output rows of 2^b
    const int a = t - o.tile_skew, b = t + o.tile_skew;
    if (a < 1 || b < 1) return BMMC_ERR_INVALID_ARG;
    const u64 Sab = o.tile_skew ? tile_rows(B, a, b) : S;
    if (info.kind != BMMC_KIND_GENERAL && popcount(Sab) <= b) {
        u64 H = pad_rows(m.A, Sab, a, b, true);
        std::vector<u64> W;
        for (int r = a; r < m.nb; ++r)
            if ((H >> r) & 1u) W.push_back(u64(1) << r);
        int st = build_tiled(m.A, m.c, m.ulog2, a, b, W, lc, swz, &p->pass[0]);
        if (st != BMMC_OK) return st;
        info.tile_log2 = t;
        single(BMMC_ROUTE_FUSED);
        return BMMC_OK;
    }
    if (o.route == BMMC_ROUTE_TWO_PASS) {
        Mat T1, T2;
        if (!factorize(m.A, a, b, T1, T2)) return BMMC_ERR_INVALID_ARG;
        // pass 0: T2 relabels 2^a-unit segments (complement 0)
        const int wl = std::min(4 - m.ulog2, a);
        build_chunk(T2, 0, m.ulog2, wl, BMMC_KERNEL_CHUNK, &p->pass[0]);
        // pass 1: T1 is tiled with rows inside {a, ..., a+b-1}
        Mat T1inv;
        inverse(T1, T1inv);
        u64 H = pad_rows(T1, tile_rows(T1inv, a, b), a, b, false);
        if (popcount(H) != b) return BMMC_ERR_INVALID_ARG;
        std::vector<u64> W;
        for (int r = a; r < m.nb; ++r)
            if ((H >> r) & 1u) W.push_back(u64(1) << r);
        int st = build_tiled(T1, m.c, m.ulog2, a, b, W, lc, swz, &p->pass[1]);
        if (st != BMMC_OK) return st;
        p->npasses = 2;
        info.passes = 2;
        info.route = BMMC_ROUTE_TWO_PASS;
        info.tile_log2 = t;
        info.scratch_bytes = (size_t)elem_bytes << n;
        to_element_level(T2, 0, dlow, n, p->factor_A[0], &p->factor_c[0]);
        to_element_level(T1, m.c, dlow, n, p->factor_A[1], &p->factor_c[1]);
        return BMMC_OK;
    }
    // fused single pass: tile rows span the high parts (above the a in-row
    // bits) of B's first b columns (reduced basis), padded with unit vectors.
    Basis vb;
    for (int j = 0; j < b; ++j) vb.add(B.col(j) & ~low_mask(a));
    std::vector<u64> W = vb.vec;
    Basis wb = vb;
    for (int r = a; r < m.nb && (int)W.size() < b; ++r)
        if (wb.add(u64(1) << r)) W.push_back(u64(1) << r);
    int st = build_tiled(m.A, m.c, m.ulog2, a, b, W, lc, swz, &p->pass[0]);
    if (st != BMMC_OK) return st;
    info.tile_log2 = t;
    single(BMMC_ROUTE_FUSED);
    return BMMC_OK;
}

}  // namespace bmmc
