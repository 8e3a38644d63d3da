// repack.hip -- strided unit copy behind the Ulysses layout changes
// (handbook page "上下文并行：Ring Attention 与 Ulysses", section "Ulysses：
// 在序列和头之间转置").  On one GPU the all-to-all between P ranks is a copy of
// runs of Hp*D contiguous elements ("units") between the sequence-major
// [S][H][D] layout and the per-rank [S][Hp][D] layouts.  The host computes
// each unit's source and destination byte offsets as
//   off(u) = base + (u / per) * stride_a + (u % per) * stride_b.
//
// HBM-bound: every byte is read once and written once, with the widest
// vector (16, 4 or 2 bytes) that the unit size and offsets allow.
#include "cp_kernels.h"

namespace cpattn {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <typename V, typename I>
__global__ __launch_bounds__(kThreads) void unit_copy_kernel(
    const char *__restrict__ src, char *__restrict__ dst, I vecs_per_unit, I per, I total,
    int64_t src_base, int64_t src_a, int64_t src_b, int64_t dst_base, int64_t dst_a,
    int64_t dst_b)
{
    const I stride = (I)gridDim.x * kThreads;
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
        const I u = e / vecs_per_unit;
        const I w = e - u * vecs_per_unit;
        const I ua = u / per;
        const I ub = u - ua * per;
        const int64_t so = src_base + (int64_t)ua * src_a + (int64_t)ub * src_b +
                           (int64_t)w * (int64_t)sizeof(V);
        const int64_t d = dst_base + (int64_t)ua * dst_a + (int64_t)ub * dst_b +
                          (int64_t)w * (int64_t)sizeof(V);
        *(V *)(dst + d) = *(const V *)(src + so);
    }
}

template <typename V>
hipError_t launch_v(const UnitCopy &c, hipStream_t stream)
{
    const int64_t vpu = c.unit_bytes / (int64_t)sizeof(V);
    const int64_t total = vpu * c.n_units;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 8192)
        blocks = 8192;
    if (total < (int64_t(1) << 31)) {
        hipLaunchKernelGGL((unit_copy_kernel<V, uint32_t>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, (const char *)c.src, (char *)c.dst,
                           (uint32_t)vpu, (uint32_t)c.per, (uint32_t)total, c.src_base,
                           c.src_a, c.src_b, c.dst_base, c.dst_a, c.dst_b);
    } else {
        hipLaunchKernelGGL((unit_copy_kernel<V, uint64_t>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, stream, (const char *)c.src, (char *)c.dst,
                           (uint64_t)vpu, (uint64_t)c.per, (uint64_t)total, c.src_base,
                           c.src_a, c.src_b, c.dst_base, c.dst_a, c.dst_b);
    }
    return hipGetLastError();
}

bool aligned_to(const UnitCopy &c, int64_t n)
{
    return c.unit_bytes % n == 0 && c.src_base % n == 0 && c.src_a % n == 0 &&
           c.src_b % n == 0 && c.dst_base % n == 0 && c.dst_a % n == 0 &&
           c.dst_b % n == 0 && ((uintptr_t)c.src) % n == 0 && ((uintptr_t)c.dst) % n == 0;
}

}  // namespace

hipError_t launch_unit_copy(const UnitCopy &c, hipStream_t stream)
{
    if (c.n_units == 0 || c.unit_bytes == 0)
        return hipSuccess;
    if (aligned_to(c, 16))
        return launch_v<u32x4>(c, stream);
    if (aligned_to(c, 4))
        return launch_v<uint32_t>(c, stream);
    return launch_v<uint16_t>(c, stream);
}

}  // namespace cpattn
