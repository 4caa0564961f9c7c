// Validation of the device arrays a launch trusts (bounds, page-table rows,
// page ids), reported through a status word instead of a separate debug
// build.  The launch itself stays safe on bad values (bounds are clamped, a
// bad page-table row or page id scores NaN); this tells the caller they were
// there.  Status bits (OR-ed by the rows that see them):
//   1  a row_bound outside [0, max_bound]
//   2  a row_pt outside [0, pt_rows)
//   4  a page id the row would read (pages below ceil(min(bound, max_bound) / 64))
//      outside [0, num_pages)
#include "common.h"

namespace fp8idx {

__global__ __launch_bounds__(256) void validate_kernel(const int32_t *page_table, const int32_t *row_pt,
                                                       const int32_t *row_bound, uint32_t *status, int num_pages,
                                                       int pt_rows, int pt_stride, int max_bound) {
    const int r = blockIdx.x, t = threadIdx.x;
    const int b = row_bound[r], pr = row_pt[r];
    uint32_t bad = 0;
    if (t == 0 && (b < 0 || b > max_bound)) bad |= 1u;
    if (t == 0 && (pr < 0 || pr >= pt_rows)) bad |= 2u;
    if (pr >= 0 && pr < pt_rows) {
        const int bc = b < 0 ? 0 : (b > max_bound ? max_bound : b);
        const int npg = (bc + kPage - 1) / kPage;   // <= pt_stride (max_bound <= pt_stride * 64)
        const int32_t *pt = page_table + (int64_t)pr * pt_stride;
        for (int i = t; i < npg; i += 256) {
            const int pg = pt[i];
            if (pg < 0 || pg >= num_pages) bad |= 4u;
        }
    }
    if (bad) atomicOr(status, bad);
}

hipError_t launch_validate(const int32_t *page_table, const int32_t *row_pt, const int32_t *row_bound,
                           uint32_t *status, int rows, int num_pages, int pt_rows, int pt_stride, int max_bound,
                           hipStream_t st) {
    hipError_t e = launch_fill_zero(status, 4, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(validate_kernel, dim3(rows), dim3(256), 0, st, page_table, row_pt, row_bound, status,
                       num_pages, pt_rows, pt_stride, max_bound);
    return hipGetLastError();
}

}  // namespace fp8idx
