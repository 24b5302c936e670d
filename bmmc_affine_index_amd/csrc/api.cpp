// api.cpp -- the extern "C" entry points declared in include/bmmc.h.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "../../include/bmmc.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local int g_last_error = BMMC_OK;

int run_pass(const bmmc_pass_desc &d, const void *in, void *out, hipStream_t s) {
    switch (d.kernel) {
    case BMMC_KERNEL_COPY:
        return bmmc::launch_copy(in, out, (size_t)1 << (d.nbits + d.unit_log2), s);
    case BMMC_KERNEL_CHUNK:
    case BMMC_KERNEL_NAIVE:
        return bmmc::launch_chunk(d, in, out, s);
    case BMMC_KERNEL_TILED:
        return bmmc::launch_tiled(d, in, out, s);
    default:
        return BMMC_ERR_INVALID_ARG;
    }
}

bool overlaps(const void *a, const void *b, size_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bytes && y < x + bytes;
}

}  // namespace

extern "C" {

bmmc_plan *bmmc_plan_create_ex(int n, const uint64_t *A, uint64_t c, size_t elem_bytes,
                               const bmmc_plan_options *opt) {
    bmmc_plan *p = new (std::nothrow) bmmc_plan();
    if (!p) {
        g_last_error = BMMC_ERR_OUT_OF_MEMORY;
        return nullptr;
    }
    int st = bmmc::build_plan(n, A, c, elem_bytes, opt, p);
    if (st == BMMC_OK) {
        for (int k = 0; k < p->npasses; ++k) {
            const bmmc_pass_desc &d = p->pass[k];
            if (d.kernel == BMMC_KERNEL_TILED &&
                !bmmc::tiled_supported(d.unit_log2, d.t, d.iters_log2, d.launch))
                st = BMMC_ERR_UNSUPPORTED;
        }
    }
    if (st != BMMC_OK) {
        delete p;
        g_last_error = st;
        return nullptr;
    }
    g_last_error = BMMC_OK;
    return p;
}

bmmc_plan *bmmc_plan_create(int n, const uint64_t *A, uint64_t c, size_t elem_bytes) {
    return bmmc_plan_create_ex(n, A, c, elem_bytes, nullptr);
}

int bmmc_execute(const bmmc_plan *p, const void *in, void *out, void *stream) {
    if (!p || !in || !out) return BMMC_ERR_INVALID_ARG;
    const size_t bytes = (size_t)p->elem_bytes << p->n;
    const size_t align = bytes < 16 ? bytes : 16;
    if (((uintptr_t)in % align) || ((uintptr_t)out % align)) return BMMC_ERR_INVALID_ARG;
    if (overlaps(in, out, bytes)) return BMMC_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p->npasses == 1) return run_pass(p->pass[0], in, out, s);

    void *scratch = nullptr;
    {
        std::lock_guard<std::mutex> lock(p->scratch_mu);
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return BMMC_ERR_HIP;
        if (p->scratch && p->scratch_device != dev) {
            (void)hipFree(p->scratch);
            p->scratch = nullptr;
        }
        if (!p->scratch) {
            if (hipMalloc(&p->scratch, bytes) != hipSuccess) {
                (void)hipGetLastError();
                p->scratch = nullptr;
                return BMMC_ERR_OUT_OF_MEMORY;
            }
            p->scratch_device = dev;
        }
        scratch = p->scratch;
    }
    if (overlaps(in, scratch, bytes) || overlaps(out, scratch, bytes)) return BMMC_ERR_ALIAS;
    int st = run_pass(p->pass[0], in, scratch, s);
    if (st != BMMC_OK) return st;
    return run_pass(p->pass[1], scratch, out, s);
}

int bmmc_copy(const void *in, void *out, size_t nbytes, void *stream) {
    if (nbytes == 0) return BMMC_OK;
    if (!in || !out) return BMMC_ERR_INVALID_ARG;
    if (overlaps(in, out, nbytes)) return BMMC_ERR_ALIAS;
    return bmmc::launch_copy(in, out, nbytes, static_cast<hipStream_t>(stream));
}

void bmmc_plan_destroy(bmmc_plan *p) {
    if (!p) return;
    if (p->scratch) (void)hipFree(p->scratch);
    delete p;
}

int bmmc_last_error(void) { return g_last_error; }

const char *bmmc_status_string(int status) {
    switch (status) {
    case BMMC_OK: return "ok";
    case BMMC_ERR_INVALID_ARG: return "invalid argument";
    case BMMC_ERR_SINGULAR: return "matrix is singular over F2";
    case BMMC_ERR_UNSUPPORTED: return "unsupported configuration";
    case BMMC_ERR_ALIAS: return "input and output overlap";
    case BMMC_ERR_OUT_OF_MEMORY: return "out of memory";
    case BMMC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int bmmc_plan_get_info(const bmmc_plan *p, bmmc_plan_info *info) {
    if (!p || !info) return BMMC_ERR_INVALID_ARG;
    *info = p->info;
    return BMMC_OK;
}

int bmmc_plan_get_factor(const bmmc_plan *p, int pass, uint64_t *A_out, uint64_t *c_out) {
    if (!p || !A_out || !c_out || pass < 0 || pass >= p->npasses) return BMMC_ERR_INVALID_ARG;
    std::memcpy(A_out, p->factor_A[pass], sizeof(uint64_t) * (size_t)p->n);
    *c_out = p->factor_c[pass];
    return BMMC_OK;
}

int bmmc_plan_get_pass(const bmmc_plan *p, int pass, bmmc_pass_desc *desc) {
    if (!p || !desc || pass < 0 || pass >= p->npasses) return BMMC_ERR_INVALID_ARG;
    *desc = p->pass[pass];
    return BMMC_OK;
}

}  // extern "C"
