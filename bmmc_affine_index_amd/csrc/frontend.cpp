// frontend.cpp -- matrices of two users of the permutation: the parm
// combinator and permutations/flips of tensor dimensions.  Host-only.
#include <cstdint>
#include <cstring>

#include "../../include/bmmc.h"
#include "gf2.h"

extern "C" {

// parm ("Efficient GPU Implementation of Affine Index Permutations on
// Arrays", introduction: parm mask f xs splits xs by the F2 dot product
// i.mask, applies f to each part and stitches the results back; parm with
// mask m equals a BMMC, then parm on the two halves, then the inverse BMMC).
// Output bit n-1 is i.mask, so the first half holds the elements with
// i.mask = 0.  The other output bits are the input bits without the lowest
// set bit p of the mask, in order: two indices of the same part cannot first
// differ at bit p (that alone would change the dot product), so each half
// keeps increasing index order.
int bmmc_parm_matrix(int n, uint64_t mask, uint64_t *A_out) {
    if (n < 1 || n > BMMC_MAX_N || !A_out) return BMMC_ERR_INVALID_ARG;
    if (!mask || (n < 64 && (mask >> n))) return BMMC_ERR_INVALID_ARG;
    const int p = __builtin_ctzll(mask);
    int r = 0;
    for (int j = 0; j < n; ++j)
        if (j != p) A_out[r++] = uint64_t(1) << j;
    A_out[n - 1] = mask;
    return BMMC_OK;
}

// Tensor dimensions: an input of shape (2^b_0, ..., 2^b_{k-1}), row-major
// (the last dimension holds the lowest index bits), becomes the tensor whose
// dimension j is input dimension perm[j], after flipping the input
// dimensions whose bit is set in flip_mask.  Dimension d of the input holds
// index bits [off_d, off_d + b_d) with off_d the sum of b_e over e > d; output
// dimension j holds bits [ooff_j, ooff_j + b_perm[j]) likewise, so output bit
// ooff_j + q is input bit off_perm[j] + q, complemented when perm[j] is
// flipped (a flip of a power-of-two dimension is an XOR with all ones).
int bmmc_tensor_permute_matrix(int ndims, const int *dim_log2, const int *perm,
                               uint64_t flip_mask, uint64_t *A_out, uint64_t *c_out,
                               int *n_out) {
    if (ndims < 1 || ndims > 64 || !dim_log2 || !perm || !A_out || !c_out || !n_out)
        return BMMC_ERR_INVALID_ARG;
    int n = 0;
    uint64_t seen = 0;
    for (int d = 0; d < ndims; ++d) {
        if (dim_log2[d] < 0 || perm[d] < 0 || perm[d] >= ndims) return BMMC_ERR_INVALID_ARG;
        if ((seen >> perm[d]) & 1u) return BMMC_ERR_INVALID_ARG;
        seen |= uint64_t(1) << perm[d];
        n += dim_log2[d];
    }
    if (n > BMMC_MAX_N || (ndims < 64 && (flip_mask >> ndims))) return BMMC_ERR_INVALID_ARG;
    int off[64];
    int acc = 0;
    for (int d = ndims - 1; d >= 0; --d) {
        off[d] = acc;
        acc += dim_log2[d];
    }
    uint64_t c = 0;
    int ooff = 0;
    for (int j = ndims - 1; j >= 0; --j) {
        const int d = perm[j];
        for (int q = 0; q < dim_log2[d]; ++q) {
            A_out[ooff + q] = uint64_t(1) << (off[d] + q);
            if ((flip_mask >> d) & 1u) c |= uint64_t(1) << (ooff + q);
        }
        ooff += dim_log2[d];
    }
    *c_out = c;
    *n_out = n;
    return BMMC_OK;
}

// Inverse over F2 of n row masks (Gauss-Jordan).  The inverse BMMC of
// (A, c) is (A^{-1}, A^{-1}.c).
int bmmc_matrix_inverse(int n, const uint64_t *A, uint64_t *A_inv) {
    if (n < 1 || n > BMMC_MAX_N || !A || !A_inv) return BMMC_ERR_INVALID_ARG;
    bmmc::Mat M = bmmc::Mat::zeros(n, n), inv;
    for (int r = 0; r < n; ++r) {
        if (A[r] >> n) return BMMC_ERR_INVALID_ARG;
        M.r[r] = A[r];
    }
    if (!bmmc::inverse(M, inv)) return BMMC_ERR_SINGULAR;
    for (int r = 0; r < n; ++r) A_inv[r] = inv.r[r];
    return BMMC_OK;
}

}  // extern "C"
