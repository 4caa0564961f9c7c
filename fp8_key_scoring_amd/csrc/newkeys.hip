// New-key write on gfx950: each query row's own key, quantized to E4M3 codes
// plus one fp32 scale, written into the paged key cache ahead of scoring.
//
// The sglang pull request page "sgl-project/sglang#48224" (sgl-amd-mono #86
// commit body, Modifications row 2, and the Reviewer notes on new keys) has
// the launch write keys and every row of the request score them: the row at
// position p (bound p + 1) writes its key at logical position p, and every
// row of its request whose bound passes p scores it.  The pages give no
// quantization rule; the plain per-key one is used:
//   amax  = max |k[i]| over the key's 128 bf16 elements,
//   scale = amax / 448 (fp32, round to nearest even; 448 is the largest
//           finite E4M3 value), or 1 when amax is 0 (then every code is 0),
//   code  = E4M3 of the fp32 quotient k[i] / scale, round to nearest even
//           (the quotient of the largest element is 448 to within an ulp,
//           which rounds to 448, so no quotient overflows).
//
// One wave per row: lane l holds elements 2l and 2l+1 (one 4-byte load), the
// wave's max is a butterfly of lane exchanges, the hardware conversion
// v_cvt_pk_fp8_f32 (OCP E4M3FN on gfx950) turns the two quotients into two
// codes, and each lane stores its two bytes (one 128-byte store per wave)
// with lane 0 storing the scale.  The write runs as its own kernel ahead of
// the scoring kernel on the same stream, so every scoring workgroup that
// reads the slot sees the new codes.
#include "common.h"

namespace fp8idx {

__global__ __launch_bounds__(64) void write_keys_kernel(const uint16_t *k_new, uint8_t *k8, float *kscale,
                                                         const int32_t *page_table, const int32_t *row_pt,
                                                         const int32_t *row_bound, int num_pages, int pt_rows,
                                                         int pt_stride, int max_bound) {
    const int r = blockIdx.x, lane = threadIdx.x;
    int b = row_bound[r];
    b = b < 0 ? 0 : (b > max_bound ? max_bound : b);
    const int pr = row_pt[r];
    if (b == 0 || pr < 0 || pr >= pt_rows) return;   // nothing to write (wave-uniform)
    const int pos = b - 1;
    const int page = page_table[(int64_t)pr * pt_stride + pos / kPage];
    if (page < 0 || page >= num_pages) return;

    const uint32_t two = ((const uint32_t *)(k_new + (int64_t)r * kDim))[lane];   // elements 2l, 2l+1
    const float x0 = __uint_as_float(two << 16), x1 = __uint_as_float(two & 0xffff0000u);
    const float amax = wave_max_f32(fmaxf(fabsf(x0), fabsf(x1)));
    const bool zero = amax == 0.0f;
    const float scale = zero ? 1.0f : __fdiv_rn(amax, 448.0f);
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x0, scale), __fdiv_rn(x1, scale), 0, false);
    const uint16_t codes = zero ? (uint16_t)0 : (uint16_t)(packed & 0xffff);
    const int64_t slot = (int64_t)page * kPage + pos % kPage;
    ((uint16_t *)(k8 + slot * kDim))[lane] = codes;
    if (lane == 0) kscale[slot] = scale;
}

hipError_t launch_write_keys(const uint16_t *k_new, uint8_t *k8, float *kscale, const int32_t *page_table,
                             const int32_t *row_pt, const int32_t *row_bound, int rows, int num_pages,
                             int pt_rows, int pt_stride, int max_bound, hipStream_t st) {
    hipLaunchKernelGGL(write_keys_kernel, dim3(rows), dim3(64), 0, st, k_new, k8, kscale, page_table, row_pt,
                       row_bound, num_pages, pt_rows, pt_stride, max_bound);
    return hipGetLastError();
}

}  // namespace fp8idx
