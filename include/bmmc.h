/*
 * bmmc.h -- C ABI of the MI355X (gfx950) BMMC permutation library.
 *
 * A BMMC ("bit matrix multiply and complement") permutation of an array of
 * 2^n elements moves element i to index A.i XOR c, where the index is read as
 * a bit vector in F2^n (bit 0 = least significant bit), A is an invertible
 * n x n matrix over F2 and c is an n-bit vector ("Efficient GPU
 * Implementation of Affine Index Permutations on Arrays", FHPNC'23,
 * introduction: the BMMC definition; invertibility of A is what makes the map
 * a permutation).  Bit-reversal, power-of-two matrix transposes (rotations of
 * the index bits), bit permutations with complement (BPC) and arbitrary affine
 * maps over F2 are all such permutations.
 *
 *     out[A.i XOR c] = in[i]      for every i in [0, 2^n)
 *
 * The scatter direction matches that page's appendix kernels, which derive
 * the output address from the input address.
 *
 * Matrix layout: A is passed as n row masks, A[r] holding output bit r's
 * inputs; bit j of A[r] is the entry A_rj.  So y_r = parity(A[r] & i) ^ c_r.
 *
 * Every function is extern "C" and takes plain pointers and sizes.  Device
 * pointers are HIP device allocations on the current device; `stream` is a
 * hipStream_t passed as void* (NULL = the default stream).  No call aborts:
 * each returns a status (or NULL plus bmmc_last_error()).
 */
#ifndef BMMC_H
#define BMMC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define BMMC_OK 0
#define BMMC_ERR_INVALID_ARG 1   /* n, elem_bytes, stray bits, NULL, alignment */
#define BMMC_ERR_SINGULAR 2      /* A is not invertible over F2 */
#define BMMC_ERR_UNSUPPORTED 3   /* a valid request no compiled kernel serves */
#define BMMC_ERR_ALIAS 4         /* the in and out byte ranges overlap */
#define BMMC_ERR_OUT_OF_MEMORY 5 /* scratch allocation failed */
#define BMMC_ERR_HIP 6           /* a HIP runtime call or kernel launch failed */
#define BMMC_ERR_SCRATCH_LIMIT 7 /* bmmc_execute_noalloc: the plan needs more scratch than
                                    the fixed BMMC_NOALLOC_SCRATCH_BYTES */

/* ---- classification of A (at the granularity the kernels move) --------- */
#define BMMC_KIND_IDENTITY 0 /* A = I: a copy, or a complement-only XOR */
#define BMMC_KIND_BPC 1      /* A is a permutation matrix: BP (c = 0) or BPC */
#define BMMC_KIND_TILED 2    /* one tile pass with index-aligned tile rows */
#define BMMC_KIND_GENERAL 3  /* anything else */

/* ---- routes a plan may take -------------------------------------------- */
#define BMMC_ROUTE_AUTO 0     /* planner's choice (fused single pass) */
#define BMMC_ROUTE_NAIVE 1    /* one unit per lane, scattered stores */
#define BMMC_ROUTE_TWO_PASS 2 /* general A as two tiled factors: segment relabel T2, then T1 */
#define BMMC_ROUTE_FUSED 3    /* every A in one tile pass (tile rows need not be index-aligned) */

/* ---- kernels a pass may run -------------------------------------------- */
#define BMMC_KERNEL_COPY 0  /* identity order */
#define BMMC_KERNEL_CHUNK 1 /* chunks move as units (a gather): segment relabel, block moves */
#define BMMC_KERNEL_TILED 2 /* LDS-staged tile pass */
#define BMMC_KERNEL_NAIVE 3 /* one unit per lane */
#define BMMC_KERNEL_CHUNK_SCATTER 4 /* chunks read in order, stored at permuted places:
                                       complement-only maps (A = I, c != 0) */

#define BMMC_MAX_N 32      /* largest index width accepted */
#define BMMC_MAX_BITS 36   /* index bits at byte-merged unit granularity */
#define BMMC_MAX_TILE 8    /* largest tile side, log2 units */
#define BMMC_MAX_PASSES 2

/* Options for bmmc_plan_create_ex.  Zero-initialise, then set fields; a zero
 * field means "planner's choice". */
typedef struct bmmc_plan_options {
    int route;      /* BMMC_ROUTE_* */
    int tile_log2;  /* tile side in units (log2); 0 = planner's choice */
    int no_swizzle; /* 1 = plain row-major LDS tile (bank-conflict ablation) */
    int iters_log2; /* one-tile launch: log2 of tiles staged together per workgroup */
    int launch;     /* BMMC_LAUNCH_*: how the tile pass is launched */
    int grid_log2;  /* persistent launch: log2 of workgroups; 0 = planner's choice */
    int walk;       /* persistent launch: BMMC_WALK_* order of tiles; 0 = planner's choice */
    int depth;      /* streamed launch: tiles of loads in flight per loader wave (1 or 2);
                       0 = planner's choice (1) */
    int cache_hint; /* tile pass: 0 = planner's choice (non-temporal loads and stores),
                       1 = none, 2 = non-temporal loads and stores */
    int block_map;  /* re-indexing of the tiles: 0 = planner's choice (5), 1 = identity,
                       2 = reversed bit order, 3 = tiles in flight together form a
                       patch dense on both the input and the output side, 4 = dense on
                       the input side, 5 = dense on the output side, 6 = (range walk)
                       workgroups in step are dense on the output side and each
                       workgroup's successive tiles on the input side, 7 = the reverse
                       of 6, >= 8 = a random invertible F2 map seeded with the value
                       (the set of tiles is the same; only the order in which
                       workgroups meet them changes) */
    int tile_skew;  /* single-pass tile shape: 0 = square tiles of 2^t rows of 2^t units;
                       s != 0 = rectangular tiles of the same 2^(2t) units whose input
                       rows hold 2^(t-s) units and output rows 2^(t+s) (longer output
                       pieces for s > 0); |s| < t, and both rows must hold at least one
                       16-byte vector (or the whole row when t is small) */
    int tile_threads_log2; /* tile pass: log2 of the most threads that move one tile,
                              8 (256) or 9 (512); 0 = planner's choice (8).  Tiles of
                              fewer chunks use one thread per chunk. */
    int split_stage; /* tile pass, one-tile launch only: 1 = stage each tile in LDS half
                        at a time (half the LDS per workgroup, so more tiles can hold
                        LDS on a compute unit at once: up to five 32 KiB halves of
                        64 KiB tiles against two whole ones); 0 = planner's choice
                        (whole tiles).
                        Not every matrix admits it at every tile shape
                        (BMMC_ERR_INVALID_ARG then); launch must be AUTO or ONE_TILE
                        and iters_log2 0. */
    int buffer_loads; /* tile pass, one-tile launch of whole tiles only: 1 = read the
                         input with buffer loads, whose per-lane address is a 32-bit
                         offset from a base held in scalar registers, instead of
                         64-bit global addresses (same bytes, same cache policy; which
                         form is faster depends on the matrix); 0 = planner's choice
                         (global loads).  Needs units of 4 bytes or more and an array
                         of at most 2^31 bytes, launch AUTO or ONE_TILE, iters_log2 0
                         and split_stage 0 (BMMC_ERR_INVALID_ARG otherwise). */
} bmmc_plan_options;

/* Tile orders of the persistent launch. */
#define BMMC_WALK_AUTO 0
#define BMMC_WALK_RANGES 1      /* workgroup w walks the contiguous block range of w */
#define BMMC_WALK_INTERLEAVED 2 /* at each step the workgroups take adjacent blocks */

/* Launch styles of the tile pass. */
#define BMMC_LAUNCH_AUTO 0       /* planner's choice */
#define BMMC_LAUNCH_ONE_TILE 1   /* one workgroup per tile (or per 2^iters_log2 tiles) */
#define BMMC_LAUNCH_PERSISTENT 2 /* 2^grid_log2 workgroups, each walking a range of tiles
                                    with the next tile's loads overlapping this tile's stores */
#define BMMC_LAUNCH_STREAMED 3   /* as PERSISTENT, with loader waves and storer waves */

/* What a plan does, for tests and benchmarks. */
typedef struct bmmc_plan_info {
    int n;              /* index bits as given */
    int elem_bytes;     /* element size as given */
    int kind;           /* BMMC_KIND_* of the unit-level matrix */
    int route;          /* BMMC_ROUTE_* actually taken (never AUTO) */
    int passes;         /* kernel launches per bmmc_execute (1 or 2) */
    int unit_bytes;     /* bytes moved as one unit: elem_bytes times the
                           largest run of low index bits the map keeps */
    int unit_bits;      /* index bits at unit granularity */
    int tile_log2;      /* tile side (log2 units) of the tiled pass, 0 if none */
    int n_over;         /* t - rank of A[t:, 0:t]: low input bits that stay low */
    size_t scratch_bytes; /* device scratch a two-pass plan allocates */
} bmmc_plan_info;

/* Kernel tables of one pass.  All offsets are byte offsets; every table entry
 * is XORed in when the corresponding index bit is 1, which is how the kernels
 * evaluate A.x XOR c without a per-element matrix-vector product (the map is
 * affine, so the address of any element is the XOR of the contributions of
 * its block, chunk and unit bits).
 *
 * TILED: the array is cut into 2^blk_bits tiles of 2^(2t) units, each
 * 2^(2t - in_row_log2) input rows of 2^in_row_log2 contiguous units and
 * 2^(2t - out_row_log2) output rows of 2^out_row_log2 units; tile b
 * starts at input offset XOR_k in_blk[k] over the set bits k of b.  With the
 * one-tile launch a workgroup moves tiles b = (w << iters_log2) | s; with
 * the persistent and streamed launches workgroup w, as walker
 * v = w XOR ((w >> 3) & 7), walks, for k < 2^r with r = blk_bits - grid_log2
 * and gray(k) = k XOR (k >> 1), the tiles v * 2^r XOR gray(k) (ranges) or
 * gray(k) * 2^grid_log2 XOR v (interleaved).
 * A tile is moved in chunks of 2^chunk_log2 units: chunk c = (j << T) | tid
 * (T = threads_log2, j the pass) is loaded from input offset
 * tile base XOR_p ld_in[p] and written to LDS address XOR_p ld_lds[p] over
 * the set bits p of c; in the drain phase chunk c is stored at output offset
 * XOR_k out_blk[k] XOR out_c XOR_p st_out[p], its unit e read from LDS
 * address XOR_k lds_blk[k] XOR lds_c XOR_p st_lds[p] XOR_b st_unit[b] over
 * the set bits b of e.
 * CHUNK (a gather): output chunk y is written at y * chunk_bytes and read
 * from input offset XOR_k in_blk[k] over the set bits k of y, XOR in_c; unit
 * e of the output chunk is unit e XOR unit_xor of the input chunk.  Writing
 * in order and reading in permuted order is the faster way round on MI355X.
 * NAIVE and CHUNK_SCATTER (scatters): input chunk (one unit for NAIVE)
 * index bit k moves the output by out_blk[k]; out_c is the constant; the
 * input chunk is read at chunk_index * chunk_bytes; units inside a chunk as
 * for CHUNK.  For complement-only maps the scatter is the faster form (a
 * gather would read each wave's chunks in descending order).
 * COPY: nothing but nbits/unit_log2. */
#define BMMC_MAX_CHUNK_BITS 16
typedef struct bmmc_pass_desc {
    int32_t kernel;      /* BMMC_KERNEL_* */
    int32_t unit_log2;   /* log2 bytes of one unit */
    int32_t nbits;       /* index bits at unit granularity */
    int32_t t;           /* tile side / segment length, log2 units (TILED) */
    int32_t chunk_log2;  /* log2 units per vector chunk */
    int32_t blk_bits;    /* tile-index bits (TILED), chunk-index bits (CHUNK),
                            unit-index bits (NAIVE) */
    int32_t iters_log2;  /* one-tile launch: tiles staged together, log2 (TILED) */
    int32_t unit_xor;    /* in-chunk unit permutation (CHUNK) */
    int32_t launch;      /* BMMC_LAUNCH_ONE_TILE, _PERSISTENT or _STREAMED (TILED) */
    int32_t grid_log2;   /* persistent launch: 2^grid_log2 workgroups (TILED) */
    int32_t walk;        /* persistent launch: BMMC_WALK_RANGES or _INTERLEAVED (TILED) */
    int32_t depth;       /* streamed launch: tiles of loads in flight per loader wave, 1 or 2 */
    int32_t cache_hint;  /* 3 = non-temporal loads and stores, 0 = plain (others unsupported) */
    int32_t block_map;   /* tile order the tables were built with (TILED; 0 otherwise) */
    uint64_t out_c;
    uint32_t lds_c;
    uint32_t lds_bytes;  /* LDS bytes per workgroup (TILED) */
    uint64_t in_blk[BMMC_MAX_BITS];
    uint64_t out_blk[BMMC_MAX_BITS];
    uint32_t lds_blk[BMMC_MAX_BITS];
    uint64_t ld_in[BMMC_MAX_CHUNK_BITS];
    uint32_t ld_lds[BMMC_MAX_CHUNK_BITS];
    uint64_t st_out[BMMC_MAX_CHUNK_BITS];
    uint32_t st_lds[BMMC_MAX_CHUNK_BITS];
    uint32_t st_unit[4];
    uint64_t in_c;       /* CHUNK: input offset of output chunk 0 */
    int32_t in_row_log2;  /* TILED: log2 units per input row of a tile (t - skew) */
    int32_t out_row_log2; /* TILED: log2 units per output row of a tile (t + skew);
                             a tile holds 2^(in_row_log2 + out_row_log2) = 2^(2t) units */
    int32_t threads_log2; /* TILED: log2 threads that move one tile (the thread bits of
                             the chunk index c = (j << threads_log2) | tid) */
    int32_t split_stage;  /* TILED, one-tile launch: 1 = the tile passes through LDS in
                             two halves, the chunks whose top chunk-index bit is h in
                             half h, on both the load and the drain side; lds_bytes is
                             then half a tile */
    int32_t buffer_loads; /* TILED, one-tile launch: 1 = the input is read with buffer
                             loads (32-bit offsets from the array's base; the array
                             holds at most 2^31 bytes), 0 = global loads */
} bmmc_pass_desc;

typedef struct bmmc_plan bmmc_plan; /* opaque; changed after creation only by bmmc_plan_tune */

/* Plan the permutation out[A.i XOR c] = in[i] of 2^n elements of elem_bytes
 * bytes.  Host-only: validates (1 <= n <= 32, elem_bytes in {1,2,4,8,16},
 * no bits of A[r] or c at positions >= n, total bytes <= 2^36), inverts A over
 * F2 (singular -> BMMC_ERR_SINGULAR), classifies it (identity, BPC, tiled,
 * general), factorises a general A into at most two tiled factors when the
 * two-pass route is chosen ("Efficient GPU Implementation of Affine Index
 * Permutations on Arrays", introduction: any BMMC is a product T1.T2 of two
 * tiled BMMCs, applied T2 first), and builds each pass's kernel tables.
 * Makes no GPU call.  Copies A; the caller keeps ownership of its array.
 * Returns NULL on failure, with the reason in bmmc_last_error(). */
bmmc_plan *bmmc_plan_create(int n, const uint64_t *A, uint64_t c, size_t elem_bytes);

/* As bmmc_plan_create, with options (NULL = defaults). */
bmmc_plan *bmmc_plan_create_ex(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
                               const bmmc_plan_options *opt);

/* Run the plan on `stream`, asynchronously: out[A.i XOR c] = in[i].
 * `in` and `out` are device pointers to 2^n * elem_bytes bytes each, aligned
 * to 16 bytes (to the array size if smaller), and must not overlap
 * (BMMC_ERR_ALIAS).  A two-pass plan allocates its scratch buffer (the size
 * of one array) on its first call and keeps it until bmmc_plan_destroy;
 * calls of one two-pass plan on different streams must not overlap in time.
 * Launch failures return BMMC_ERR_HIP; faults inside a kernel surface at the
 * caller's next synchronisation, as HIP reports them. */
int bmmc_execute(const bmmc_plan *plan, const void *in, void *out, void *stream);

/* bmmc_execute for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, result and errors as bmmc_execute, and the same kernels;
 * it calls no hipMalloc, hipFree or other allocating routine.  One-pass plans
 * need nothing beyond in and out.  A two-pass plan stages the array between
 * its passes in a fixed device buffer of BMMC_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every GPU it runs on until the process ends;
 * plans whose array (2^n * elem_bytes) is larger return
 * BMMC_ERR_SCRATCH_LIMIT before any GPU call.  Every call on one GPU shares
 * that GPU's buffer: two-pass calls that overlap in time on one GPU (on
 * different streams, or from different threads) race on it and must be
 * serialised by the caller.  Nothing in the buffer needs clearing: the first
 * pass writes all of it that the second pass reads. */
#define BMMC_NOALLOC_SCRATCH_BYTES ((size_t)1 << 26)
int bmmc_execute_noalloc(const bmmc_plan *plan, const void *in, void *out, void *stream);

/* Measure and keep the fastest tile order for this plan on this device.
 * Which tiles run together decides how well the DRAM pages of HBM are reused,
 * and the best order depends on the matrix ("Efficient GPU Implementation of
 * Affine Index Permutations on Arrays", limitations: on the AMD card the
 * running time varied with the permutation).  Every candidate computes the
 * same permutation; they differ in the tile side (the planner's and the next
 * larger), the launch style (the planner's persistent or streamed walk, or
 * one workgroup per tile), the loads in flight of a streamed walk (one or two
 * tiles per loader wave) and the block order (bmmc_plan_options.block_map 5,
 * the planner's, 1, 3 and 6, and the random orders 8 and 9), plus
 * rectangular tiles (tile_skew 1, -1, 2 and -2 at the larger side, orders 5,
 * 6 and 3), 512 threads per tile (skew 0, 1, -1, 2 and -2 at the larger
 * side on every launch style, orders 5 and 6), one tile per workgroup at the
 * planner's side with skew 0, 1, -1, 2 and -2 and 256 or 512 threads (orders
 * 5 and 6), and tiles staged in LDS half at a time (split_stage; skew 0, 1,
 * -1 and 2, 256 and 512 threads, order 5, where the matrix admits them), and
 * for arrays of at most 2^31 bytes of 4-byte units or larger, each one-tile
 * candidate of whole tiles again with buffer loads (buffer_loads): up to
 * 130 candidates, and up to about 60 more with buffer loads, fewer where two
 * build the same tables or where a rectangular tile's shorter rows would
 * hold less than 128 bytes.  An option the caller fixed at plan creation is kept.
 * Each candidate runs `reps` times (0 = enough runs
 * for about 2 ms of work, 3 to 200) on `stream`, in five rounds that
 * interleave the candidates, timed with HIP events (for arrays below about
 * 250 MB each candidate's runs are captured once into a HIP graph on a
 * private stream and the graph is replayed on `stream`, so that launch costs
 * do not mask the kernels; eager launches if capture fails); the candidate
 * with the fastest median round replaces the plan's kernel tables if it beats the
 * planner's own choice by more than 2%, and the chosen tables are then run
 * once on ins[0] -> outs[0].
 *
 * Runs rotate over the npairs (1 .. BMMC_MAX_TUNE_PAIRS) device buffer pairs
 * ins[k] -> outs[k], each with bmmc_execute's requirements; pass the working
 * set the plan will meet (for arrays that fit the 256 MB Infinity Cache, one
 * pair times cache-resident runs).  On return outs[0] holds the permutation
 * of ins[0]; every other outs[k] holds the permutation of ins[k] or is
 * untouched.  Blocks the host until the stream has drained; the plan must not
 * be executed concurrently.  A plan with no tile pass has nothing to choose
 * and is run once.  Errors as bmmc_execute; on any error the plan is
 * unchanged.  Pointer arrays are the caller's and are not kept. */
#define BMMC_MAX_TUNE_PAIRS 4096
int bmmc_plan_tune_pairs(bmmc_plan *plan, const void *const *ins, void *const *outs, int npairs,
                         void *stream, int reps);

/* The candidates bmmc_plan_tune_pairs would time for this plan, as the
 * options that build each (bmmc_plan_create_ex with them gives that
 * candidate's tables), in the order it times them, the planner's own choice
 * first.  Writes min(count, capacity) entries to opts and the number of
 * candidates to *count (0 for a plan with no tile pass).  Host-only; for
 * profiling every plan a tuning may pick. */
int bmmc_plan_tune_candidates(const bmmc_plan *plan, bmmc_plan_options *opts, int capacity,
                              int *count);

/* bmmc_plan_tune_pairs with the one pair in -> out. */
int bmmc_plan_tune(bmmc_plan *plan, const void *in, void *out, void *stream, int reps);

/* The ceiling: copy nbytes from `in` to `out` (device pointers, no overlap)
 * with the same vector width and launch style as the permutation kernels,
 * asynchronously on `stream` ("A kernel that is correct": the copy moves the
 * same bytes in the easiest order and is the ceiling a card can reach). */
int bmmc_copy(const void *in, void *out, size_t nbytes, void *stream);

/* Free a plan and its scratch buffer.  NULL is accepted. */
void bmmc_plan_destroy(bmmc_plan *plan);

/* Status of the last bmmc_plan_create(_ex) on this thread. */
int bmmc_last_error(void);

/* A static English string for a status code. */
const char *bmmc_status_string(int status);

/* Describe a plan (host-only). */
int bmmc_plan_get_info(const bmmc_plan *plan, bmmc_plan_info *info);

/* The options that rebuild this plan's current kernel tables: the caller's
 * options with every choice the planner or bmmc_plan_tune made written out
 * (tile side, tile skew, threads per tile, split staging, launch style, grid,
 * walk, depth, tile order, cache hint), so
 * bmmc_plan_create_ex(n, A, c, elem_bytes, opt) gives the same tables without
 * timing anything again.  Host-only. */
int bmmc_plan_get_options(const bmmc_plan *plan, bmmc_plan_options *opt);

/* The matrix and complement that pass `pass` applies, at element granularity
 * (n rows); the passes compose to the planned (A, c).  Host-only. */
int bmmc_plan_get_factor(const bmmc_plan *plan, int pass, uint64_t *A_out, uint64_t *c_out);

/* The kernel tables of pass `pass` (layout above), so that a host replay can
 * check addressing, coalescing and LDS banks without a GPU.  Host-only. */
int bmmc_plan_get_pass(const bmmc_plan *plan, int pass, bmmc_pass_desc *desc);

/* ---- users of the permutation (host-only matrix builders) -------------- */

/* The BMMC of parm ("Efficient GPU Implementation of Affine Index
 * Permutations on Arrays", introduction: parm mask f xs splits xs by the F2
 * dot product i.mask, applies f to both parts and stitches them back; parm
 * with mask m is a BMMC, parm on the two halves, and the inverse BMMC).
 * Writes n row masks to A_out: output bit n-1 = i.mask, the other output
 * bits are the input bits except the mask's lowest set bit, in order, so the
 * first half holds the elements with i.mask = 0 and both halves keep
 * increasing index order.  mask must be nonzero with no bits at >= n. */
int bmmc_parm_matrix(int n, uint64_t mask, uint64_t *A_out);

/* Inverse over F2 of n row masks (for the inverse permutation: (A, c) is
 * undone by (A^{-1}, A^{-1}.c)).  BMMC_ERR_SINGULAR if A is singular. */
int bmmc_matrix_inverse(int n, const uint64_t *A, uint64_t *A_inv);

/* The BPC that permutes (and flips) the dimensions of a row-major tensor of
 * shape (2^dim_log2[0], ..., 2^dim_log2[ndims-1]): output dimension j is
 * input dimension perm[j]; input dimension d is reversed when bit d of
 * flip_mask is set.  Writes n = sum(dim_log2) row masks to A_out (room for
 * BMMC_MAX_N), the complement to *c_out and n to *n_out.  Host-only. */
int bmmc_tensor_permute_matrix(int ndims, const int *dim_log2, const int *perm,
                               uint64_t flip_mask, uint64_t *A_out, uint64_t *c_out,
                               int *n_out);

#ifdef __cplusplus
}
#endif

#endif /* BMMC_H */
