// lse_merge.hip -- the log-sum-exp merge of two partial attention results
// over disjoint key sets (handbook page "上下文并行：Ring Attention 与
// Ulysses", section "Ring Attention：KV 沿环传一圈"; "Sequence Parallel vs
// Context Parallel" blog, section 3.2):
//   lse = log(e^lse1 + e^lse2),  o = o1 e^(lse1 - lse) + o2 e^(lse2 - lse).
//
// HBM-bound elementwise kernel.  o is [Sq][H][D] float32 and lse is [H][Sq].
// One (row, head) group of D floats is handled by L = D/4 consecutive lanes
// with 16-byte vectors; a wavefront holds G = 64/L whole groups, so every
// group's lse values are read by the same instruction stream before its lse
// is written.  That ordering makes exact aliasing (o == o1, lse == lse1)
// safe.
#include "cp_kernels.h"

#include <math.h>

namespace cpattn {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// No pointer is declared __restrict__: o may be o1 or o2 (and lse may be
// lse1 or lse2) exactly, and without the qualifier the compiler has to
// assume they alias, so it keeps every element's loads ahead of its store.
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(
    const f32x4 *o1, const float *lse1, const f32x4 *o2, const float *lse2, f32x4 *o,
    float *lse, int64_t Sq, int H, int L, int G, int64_t n_groups)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / L;
    const int e = lane - sub * L;
    const int64_t n_waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t g0 = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * G; g0 < n_groups;
         g0 += n_waves * G) {
        const int64_t g = g0 + sub;
        if (sub >= G || g >= n_groups)
            continue;
        const int64_t i = g / H;
        const int h = (int)(g - i * H);
        const int64_t li = (int64_t)h * Sq + i;
        const float a = lse1[li];
        const float b = lse2[li];
        const float mx = fmaxf(a, b);
        float l, wa, wb;
        if (mx == -INFINITY) {
            l = -INFINITY;
            wa = 0.f;
            wb = 0.f;
        } else {
            l = mx + log1pf(expf(-fabsf(a - b)));
            wa = expf(a - l);
            wb = expf(b - l);
        }
        const int64_t vi = g * L + e;
        const f32x4 x = o1[vi];
        const f32x4 y = o2[vi];
        o[vi] = x * wa + y * wb;
        if (e == 0)
            lse[li] = l;
    }
}

}  // namespace

hipError_t launch_lse_merge(const float *o1, const float *lse1, const float *o2,
                            const float *lse2, float *o, float *lse, int64_t Sq, int H,
                            int D, hipStream_t stream)
{
    const int L = D / 4;
    const int G = 64 / L;
    const int64_t n_groups = Sq * (int64_t)H;
    if (n_groups == 0)
        return hipSuccess;
    const int64_t groups_per_block = (int64_t)G * (kThreads / 64);
    int64_t blocks = (n_groups + groups_per_block - 1) / groups_per_block;
    // one loop trip per wavefront up to 2^20 workgroups (grid-stride
    // beyond): measured faster than 16 or 4 workgroups per CU looping
    if (blocks > (1 << 20))
        blocks = 1 << 20;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       (const f32x4 *)o1, lse1, (const f32x4 *)o2, lse2, (f32x4 *)o, lse, Sq,
                       H, L, G, n_groups);
    return hipGetLastError();
}

}  // namespace cpattn
