/*
 * bmmc_oracle.c -- the plain CPU oracle for BMMC index permutations.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The GPU library
 * shares no code, header, table or helper with it, and never calls it.
 *
 * What it computes (Efficient GPU Implementation of Affine Index Permutations
 * on Arrays, FHPNC'23, introduction, the definition of a BMMC transformation):
 * an array index i in [0, 2^n) is read as a bit vector x in F2^n with x_0 the
 * least significant bit; a BMMC (A, c) maps it to y = A.x XOR c, where bit r of
 * y is the XOR over j of (A_rj AND x_j), XORed with bit r of c.  A must be
 * invertible over F2, which makes the map a permutation of [0, 2^n).
 *
 * Conventions shared with the pages' appendix kernels (they compute the output
 * address from the input address and store output[out_addr] = input[in_addr]):
 *   - A is given as n rows; row r is the mask of input bits feeding output bit r.
 *   - The permutation scatters: out[A.i XOR c] = in[i].
 *   - Elements are opaque runs of elem_bytes bytes; nothing is rounded.
 *
 * Everything here is the definition written out: a Gaussian elimination to
 * decide invertibility, a bit-by-bit matrix-vector product per index, and a
 * byte copy per element.  The per-index loop is split over POSIX threads by
 * index range only; the map is a bijection, so no two threads write the same
 * output element.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_SINGULAR 2
#define ORACLE_NOT_BIJECTIVE 3

/* Rank over F2 of the n x n matrix given as n row masks (Gaussian
 * elimination: pick a pivot row with the column's bit set, clear that bit in
 * every other row). */
int oracle_gf2_rank(int n, const uint64_t *rows)
{
    uint64_t m[64];
    int rank = 0;
    if (n < 0 || n > 64) return -1;
    for (int r = 0; r < n; ++r) m[r] = rows[r];
    for (int col = 0; col < 64 && rank < n; ++col) {
        uint64_t bit = (uint64_t)1 << col;
        int piv = -1;
        for (int r = rank; r < n; ++r)
            if (m[r] & bit) { piv = r; break; }
        if (piv < 0) continue;
        uint64_t tmp = m[piv]; m[piv] = m[rank]; m[rank] = tmp;
        for (int r = 0; r < n; ++r)
            if (r != rank && (m[r] & bit)) m[r] ^= m[rank];
        ++rank;
    }
    return rank;
}

/* Inverse over F2 by Gauss-Jordan on the augmented matrix [A | I].
 * Returns ORACLE_SINGULAR when A has rank < n. */
int oracle_gf2_inverse(int n, const uint64_t *A, uint64_t *Ainv)
{
    uint64_t a[64], b[64];
    if (n < 1 || n > 64 || !A || !Ainv) return ORACLE_BAD_ARG;
    for (int r = 0; r < n; ++r) { a[r] = A[r]; b[r] = (uint64_t)1 << r; }
    for (int col = 0; col < n; ++col) {
        uint64_t bit = (uint64_t)1 << col;
        int piv = -1;
        for (int r = col; r < n; ++r)
            if (a[r] & bit) { piv = r; break; }
        if (piv < 0) return ORACLE_SINGULAR;
        uint64_t t = a[piv]; a[piv] = a[col]; a[col] = t;
        t = b[piv]; b[piv] = b[col]; b[col] = t;
        for (int r = 0; r < n; ++r)
            if (r != col && (a[r] & bit)) { a[r] ^= a[col]; b[r] ^= b[col]; }
    }
    for (int r = 0; r < n; ++r) Ainv[r] = b[r];
    return ORACLE_OK;
}

/* y = A.x XOR c, one output bit at a time: bit r of y is the parity of the
 * input bits selected by row r, flipped by bit r of c. */
uint64_t oracle_map_index(int n, const uint64_t *A, uint64_t c, uint64_t x)
{
    uint64_t y = 0;
    for (int r = 0; r < n; ++r) {
        uint64_t bit = (uint64_t)__builtin_parityll(A[r] & x);
        y |= bit << r;
    }
    return y ^ c;
}

/* y[k] = A.x[k] XOR c for `count` indices: the same definition per index. */
void oracle_map_indices(int n, const uint64_t *A, uint64_t c, const uint64_t *x, uint64_t *y,
                        size_t count)
{
    for (size_t k = 0; k < count; ++k) y[k] = oracle_map_index(n, A, c, x[k]);
}

static int check_args(int n, const uint64_t *A, uint64_t c, size_t elem_bytes)
{
    if (n < 1 || n > 40 || !A || elem_bytes == 0) return ORACLE_BAD_ARG;
    uint64_t hi = ~(((uint64_t)1 << n) - 1);
    for (int r = 0; r < n; ++r)
        if (A[r] & hi) return ORACLE_BAD_ARG;
    if (c & hi) return ORACLE_BAD_ARG;
    if (oracle_gf2_rank(n, A) != n) return ORACLE_SINGULAR;
    return ORACLE_OK;
}

struct range_job {
    int n;
    const uint64_t *A;
    uint64_t c;
    size_t elem_bytes;
    const unsigned char *in;
    unsigned char *out;
    uint64_t lo, hi;
};

static void *range_worker(void *p)
{
    struct range_job *j = (struct range_job *)p;
    for (uint64_t i = j->lo; i < j->hi; ++i) {
        uint64_t y = oracle_map_index(j->n, j->A, j->c, i);
        memcpy(j->out + y * j->elem_bytes, j->in + i * j->elem_bytes, j->elem_bytes);
    }
    return NULL;
}

/* Scatter the elements with index in [i0, i1): out[A.i XOR c] = in[i].
 * `in` and `out` both hold 2^n elements of elem_bytes bytes.  The range is
 * split into `nthreads` contiguous pieces (1 when nthreads < 1). */
int oracle_bmmc_apply_range(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
                            const void *in, void *out, uint64_t i0, uint64_t i1,
                            int nthreads)
{
    int st = check_args(n, A, c, elem_bytes);
    if (st != ORACLE_OK) return st;
    if (!in || !out || i0 > i1 || i1 > ((uint64_t)1 << n)) return ORACLE_BAD_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    uint64_t total = i1 - i0;
    if ((uint64_t)nthreads > total) nthreads = total ? (int)total : 1;

    struct range_job jobs[256];
    pthread_t tid[256];
    uint64_t per = total / (uint64_t)nthreads, rem = total % (uint64_t)nthreads;
    uint64_t lo = i0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t len = per + ((uint64_t)t < rem ? 1 : 0);
        jobs[t] = (struct range_job){n, A, c, elem_bytes, (const unsigned char *)in,
                                     (unsigned char *)out, lo, lo + len};
        lo += len;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, range_worker, &jobs[t]) != 0) break;
        started = t;
    }
    range_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    /* threads that could not be started run here, serially */
    for (int t = started + 1; t < nthreads; ++t) range_worker(&jobs[t]);
    return ORACLE_OK;
}

/* The whole permutation: out[A.i XOR c] = in[i] for every i in [0, 2^n). */
int oracle_bmmc_apply(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
                      const void *in, void *out, int nthreads)
{
    if (n < 1 || n > 40) return ORACLE_BAD_ARG;
    return oracle_bmmc_apply_range(n, A, c, elem_bytes, in, out, 0, (uint64_t)1 << n,
                                   nthreads);
}

/* Bijectivity of the image: marks y = A.i XOR c for every i and reports
 * ORACLE_NOT_BIJECTIVE if some y is hit twice or never.  This does not rely on
 * the rank test, so it checks the invertibility criterion independently.
 * `seen` must hold 2^n bytes. */
int oracle_check_bijective(int n, const uint64_t *A, uint64_t c, unsigned char *seen)
{
    if (n < 1 || n > 34 || !A || !seen) return ORACLE_BAD_ARG;
    uint64_t N = (uint64_t)1 << n;
    memset(seen, 0, (size_t)N);
    for (uint64_t i = 0; i < N; ++i) {
        uint64_t y = oracle_map_index(n, A, c, i);
        if (y >= N || seen[y]) return ORACLE_NOT_BIJECTIVE;
        seen[y] = 1;
    }
    for (uint64_t y = 0; y < N; ++y)
        if (!seen[y]) return ORACLE_NOT_BIJECTIVE;
    return ORACLE_OK;
}

/* Sampled check for arrays too large to permute on the host: for each listed
 * input index i, compares the element at out[A.i XOR c] with in[i].  Returns
 * the number of mismatches (or -1 on bad arguments); the first mismatching
 * input index is written to *first_bad when that pointer is not NULL. */
int64_t oracle_check_sampled(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
                             const void *in, const void *out, const uint64_t *idx,
                             uint64_t count, uint64_t *first_bad)
{
    if (check_args(n, A, c, elem_bytes) != ORACLE_OK || !in || !out || (!idx && count))
        return -1;
    const unsigned char *pi = (const unsigned char *)in;
    const unsigned char *po = (const unsigned char *)out;
    uint64_t N = (uint64_t)1 << n;
    int64_t bad = 0;
    for (uint64_t k = 0; k < count; ++k) {
        uint64_t i = idx[k];
        if (i >= N) return -1;
        uint64_t y = oracle_map_index(n, A, c, i);
        if (memcmp(po + y * elem_bytes, pi + i * elem_bytes, elem_bytes) != 0) {
            if (bad == 0 && first_bad) *first_bad = i;
            ++bad;
        }
    }
    return bad;
}
