/*
 * bmmc_testing.h -- fault injection for tests of the BMMC library's error
 * paths.  Not for production use: a program that never calls it behaves as
 * if it did not exist.
 */
#ifndef BMMC_TESTING_H
#define BMMC_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Make the next `count` allocations of a two-pass plan's scratch array (by
 * bmmc_execute or bmmc_plan_tune_pairs, on a plan that holds none yet) fail
 * as if the device had no memory left: the call returns
 * BMMC_ERR_OUT_OF_MEMORY before any HIP call and the plan keeps no scratch,
 * so a later call allocates again.  count = 0 turns the injection off.
 * Process-wide; returns BMMC_OK, or BMMC_ERR_INVALID_ARG for count < 0.
 * bmmc_execute_noalloc allocates nothing and is not affected. */
int bmmc_testing_fail_scratch_allocs(int count);

#ifdef __cplusplus
}
#endif

#endif /* BMMC_TESTING_H */
