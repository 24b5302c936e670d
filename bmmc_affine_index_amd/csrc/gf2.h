// gf2.h -- host-side linear algebra over F2 for the planner.
//
// A matrix is stored as row masks: row r is a uint64_t whose bit j is the
// entry (r, j).  Vectors are uint64_t with bit k = coordinate k.  Sizes are at
// most 64.  Everything is O(n^2) word operations on at most 64 words, so it
// runs in microseconds on the host ("Efficient GPU Implementation of Affine
// Index Permutations on Arrays", related work: BMMC implementations rest on
// Gaussian elimination and matrix decompositions over F2).
#pragma once

#include <cstdint>
#include <vector>

namespace bmmc {

using u64 = uint64_t;

inline u64 low_mask(int k) { return k >= 64 ? ~u64(0) : ((u64(1) << k) - 1); }

struct Mat {
    int rows = 0, cols = 0;
    u64 r[64] = {};

    static Mat zeros(int rows, int cols) {
        Mat m;
        m.rows = rows;
        m.cols = cols;
        return m;
    }
    static Mat identity(int n) {
        Mat m = zeros(n, n);
        for (int i = 0; i < n; ++i) m.r[i] = u64(1) << i;
        return m;
    }
    // Column j as a vector (bit i = entry (i, j)).
    u64 col(int j) const {
        u64 v = 0;
        for (int i = 0; i < rows; ++i) v |= ((r[i] >> j) & 1u) << i;
        return v;
    }
    void set_col(int j, u64 v) {
        for (int i = 0; i < rows; ++i) {
            r[i] &= ~(u64(1) << j);
            r[i] |= ((v >> i) & 1u) << j;
        }
    }
    // y = M x.
    u64 apply(u64 x) const {
        u64 y = 0;
        for (int i = 0; i < rows; ++i) y |= u64(__builtin_parityll(r[i] & x)) << i;
        return y;
    }
    bool operator==(const Mat &o) const {
        if (rows != o.rows || cols != o.cols) return false;
        for (int i = 0; i < rows; ++i)
            if (r[i] != o.r[i]) return false;
        return true;
    }
    bool is_identity() const { return rows == cols && *this == identity(rows); }
};

inline Mat from_cols(int rows, const std::vector<u64> &cols) {
    Mat m = Mat::zeros(rows, (int)cols.size());
    for (int j = 0; j < (int)cols.size(); ++j) m.set_col(j, cols[j]);
    return m;
}

// C = A B.
inline Mat mul(const Mat &A, const Mat &B) {
    Mat C = Mat::zeros(A.rows, B.cols);
    for (int i = 0; i < A.rows; ++i) {
        u64 acc = 0;
        for (int k = 0; k < A.cols; ++k)
            if ((A.r[i] >> k) & 1u) acc ^= B.r[k];
        C.r[i] = acc;
    }
    return C;
}

inline int rank(const Mat &M) {
    u64 a[64];
    for (int i = 0; i < M.rows; ++i) a[i] = M.r[i];
    int rk = 0;
    for (int col = 0; col < M.cols && rk < M.rows; ++col) {
        u64 bit = u64(1) << col;
        int piv = -1;
        for (int i = rk; i < M.rows; ++i)
            if (a[i] & bit) { piv = i; break; }
        if (piv < 0) continue;
        u64 t = a[piv]; a[piv] = a[rk]; a[rk] = t;
        for (int i = 0; i < M.rows; ++i)
            if (i != rk && (a[i] & bit)) a[i] ^= a[rk];
        ++rk;
    }
    return rk;
}

// Inverse of a square matrix; returns false if singular.
inline bool inverse(const Mat &M, Mat &inv) {
    const int n = M.rows;
    if (M.cols != n) return false;
    u64 a[64], b[64];
    for (int i = 0; i < n; ++i) { a[i] = M.r[i]; b[i] = u64(1) << i; }
    for (int col = 0; col < n; ++col) {
        u64 bit = u64(1) << col;
        int piv = -1;
        for (int i = col; i < n; ++i)
            if (a[i] & bit) { piv = i; break; }
        if (piv < 0) return false;
        u64 t = a[piv]; a[piv] = a[col]; a[col] = t;
        t = b[piv]; b[piv] = b[col]; b[col] = t;
        for (int i = 0; i < n; ++i)
            if (i != col && (a[i] & bit)) { a[i] ^= a[col]; b[i] ^= b[col]; }
    }
    inv = Mat::zeros(n, n);
    for (int i = 0; i < n; ++i) inv.r[i] = b[i];
    return true;
}

// Incremental basis in reduced echelon form: every stored vector has a pivot
// (its highest set bit) that no other stored vector has.
struct Basis {
    std::vector<u64> vec;   // reduced vectors
    std::vector<int> pivot; // pivot bit of each

    // Reduce v by the stored vectors.
    u64 reduce(u64 v) const {
        for (size_t k = 0; k < vec.size(); ++k)
            if ((v >> pivot[k]) & 1u) v ^= vec[k];
        return v;
    }
    bool contains(u64 v) const { return reduce(v) == 0; }
    // Add v if independent; keeps the basis fully reduced.  Returns whether
    // v was added.
    bool add(u64 v) {
        v = reduce(v);
        if (!v) return false;
        int p = 63 - __builtin_clzll(v);
        for (size_t k = 0; k < vec.size(); ++k)
            if ((vec[k] >> p) & 1u) vec[k] ^= v;
        vec.push_back(v);
        pivot.push_back(p);
        return true;
    }
    int size() const { return (int)vec.size(); }
    u64 pivot_mask() const {
        u64 m = 0;
        for (int p : pivot) m |= u64(1) << p;
        return m;
    }
    // Coordinates of v (which must lie in the span) in the stored basis:
    // since the basis is reduced, coordinate k is v's bit at pivot k.
    u64 coords(u64 v) const {
        u64 x = 0;
        for (size_t k = 0; k < vec.size(); ++k) x |= ((v >> pivot[k]) & 1u) << k;
        return x;
    }
};

inline bool is_permutation_matrix(const Mat &M) {
    if (M.rows != M.cols) return false;
    u64 seen = 0;
    for (int i = 0; i < M.rows; ++i) {
        u64 v = M.r[i];
        if (!v || (v & (v - 1))) return false;
        if (seen & v) return false;
        seen |= v;
    }
    return true;
}

}  // namespace bmmc
