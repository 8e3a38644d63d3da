// bwd_f32.hip -- float32 attention backward (the exactness path) and the
// row dot product dvec = rowsum(dout * out) used by both backward paths.
//
// Gradients of L = sum(dout * out) for the attention of the handbook page
// "上下文并行：Ring Attention 与 Ulysses", section "哪些运算可以直接切",
// function attention(), by the chain rule through its definition (the
// pages give no backward algorithm):
//   P_ij = exp(s_ij - lse_i),  ds_ij = P_ij (dout_i . v_j - dvec_i),
//   dq_i = sum_j ds_ij k_j / sqrt(D),  dk_j = sum_i ds_ij q_i / sqrt(D),
//   dv_j = sum_i P_ij dout_i,
// with lse and dvec the query rows' final values.
//
// Layout of the work: one wavefront per output row (a query row and head
// for dq, a key row and KV head for dk/dv); its lanes cover the D columns
// (two per lane at D = 128) and every dot product over D is a wavefront
// reduction.  Plain and obviously correct rather than fast: this path
// checks exactness at small sizes.
#include "cp_kernels.h"

#include <math.h>

namespace cpattn {

namespace {

constexpr int kThreads = 256;          // 4 wavefronts
constexpr int kMaxPerLane = 2;         // D <= 128

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ float ld_elem(const void *p, int bf16, int64_t idx)
{
    if (bf16)
        return (float)((const __bf16 *)p)[idx];
    return ((const float *)p)[idx];
}

__global__ __launch_bounds__(kThreads) void bwd_dvec_kernel(const float *out, const void *dout,
                                                            int dout_bf16, float *dvec,
                                                            int64_t ld, int64_t Sq, int Hq, int D)
{
    const int lane = threadIdx.x & 63;
    const int64_t n_rows = Sq * Hq;
    const int64_t wave0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * kThreads) >> 6;
    for (int64_t r = wave0; r < n_rows; r += n_waves) {     // r = i * Hq + h
        float acc = 0.f;
        for (int d = lane; d < D; d += 64)
            acc += out[r * D + d] * ld_elem(dout, dout_bf16, r * D + d);
        acc = wave_sum(acc);
        if (lane == 0) {
            const int64_t i = r / Hq;
            const int h = (int)(r % Hq);
            dvec[h * ld + i] = acc;
        }
    }
}

// dq rows: wavefront per (query row i, head h)
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(BwdLaunch b)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    if (w >= b.Sq * b.Hq)
        return;
    const int64_t i = w / b.Hq;
    const int h = (int)(w % b.Hq);
    const int g = h / (b.Hq / b.Hkv);
    const int D = b.D;
    const float *q = (const float *)b.q;
    const float *k = (const float *)b.k;
    const float *v = (const float *)b.v;
    const float *dout = (const float *)b.dout;
    const float scale = 1.f / sqrtf((float)D);
    float qi[kMaxPerLane], di[kMaxPerLane], acc[kMaxPerLane];
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
        const int d = lane + 64 * e;
        qi[e] = d < D ? q[(i * b.Hq + h) * D + d] : 0.f;
        di[e] = d < D ? dout[(i * b.Hq + h) * D + d] : 0.f;
        acc[e] = 0.f;
    }
    const float l = b.lse[h * b.stat_ld + i];
    const float dvi = b.dvec[h * b.stat_ld + i];
    if (l != -INFINITY) {
        int64_t j_end = b.Sk;                                 // visible: k_offset + j <= q_offset + i
        if (b.causal)
            j_end = min(b.Sk, max((int64_t)0, b.q_offset + i - b.k_offset + 1));
        for (int64_t j = 0; j < j_end; ++j) {
            float s = 0.f, dp = 0.f, kj[kMaxPerLane];
#pragma unroll
            for (int e = 0; e < kMaxPerLane; ++e) {
                const int d = lane + 64 * e;
                kj[e] = d < D ? k[(j * b.Hkv + g) * D + d] : 0.f;
                const float vj = d < D ? v[(j * b.Hkv + g) * D + d] : 0.f;
                s += qi[e] * kj[e];
                dp += di[e] * vj;
            }
            s = wave_sum(s);
            dp = wave_sum(dp);
            const float p = expf(s * scale - l);
            const float ds = p * (dp - dvi);
#pragma unroll
            for (int e = 0; e < kMaxPerLane; ++e)
                acc[e] += ds * kj[e];
        }
    }
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
        const int d = lane + 64 * e;
        if (d < D) {
            float *dst = &b.dq[(i * b.Hq + h) * D + d];
            *dst = (b.accumulate ? *dst : 0.f) + acc[e] * scale;
        }
    }
}

// dk, dv rows: wavefront per (key row j, KV head g)
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(BwdLaunch b)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    if (w >= b.Sk * b.Hkv)
        return;
    const int64_t j = w / b.Hkv;
    const int g = (int)(w % b.Hkv);
    const int group = b.Hq / b.Hkv;
    const int D = b.D;
    const float *q = (const float *)b.q;
    const float *k = (const float *)b.k;
    const float *v = (const float *)b.v;
    const float *dout = (const float *)b.dout;
    const float scale = 1.f / sqrtf((float)D);
    float kj[kMaxPerLane], vj[kMaxPerLane], ak[kMaxPerLane], av[kMaxPerLane];
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
        const int d = lane + 64 * e;
        kj[e] = d < D ? k[(j * b.Hkv + g) * D + d] : 0.f;
        vj[e] = d < D ? v[(j * b.Hkv + g) * D + d] : 0.f;
        ak[e] = 0.f;
        av[e] = 0.f;
    }
    int64_t i0 = 0;                                           // first row that sees key j
    if (b.causal)
        i0 = min(b.Sq, max((int64_t)0, b.k_offset + j - b.q_offset));
    for (int h = g * group; h < (g + 1) * group; ++h) {
        for (int64_t i = i0; i < b.Sq; ++i) {
            const float l = b.lse[h * b.stat_ld + i];
            if (l == -INFINITY)
                continue;
            float s = 0.f, dp = 0.f, qi[kMaxPerLane], di[kMaxPerLane];
#pragma unroll
            for (int e = 0; e < kMaxPerLane; ++e) {
                const int d = lane + 64 * e;
                qi[e] = d < D ? q[(i * b.Hq + h) * D + d] : 0.f;
                di[e] = d < D ? dout[(i * b.Hq + h) * D + d] : 0.f;
                s += qi[e] * kj[e];
                dp += di[e] * vj[e];
            }
            s = wave_sum(s);
            dp = wave_sum(dp);
            const float p = expf(s * scale - l);
            const float ds = p * (dp - b.dvec[h * b.stat_ld + i]);
#pragma unroll
            for (int e = 0; e < kMaxPerLane; ++e) {
                av[e] += p * di[e];
                ak[e] += ds * qi[e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < kMaxPerLane; ++e) {
        const int d = lane + 64 * e;
        if (d < D) {
            float *pk = &b.dk[(j * b.Hkv + g) * D + d];
            float *pv = &b.dv[(j * b.Hkv + g) * D + d];
            *pk = (b.accumulate ? *pk : 0.f) + ak[e] * scale;
            *pv = (b.accumulate ? *pv : 0.f) + av[e];
        }
    }
}

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float *p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        p[i] = 0.f;
}

// p[r * ld + c] = value for r < n_rows, c < n_cols (padding rows of an
// output: out rows are one run, lse entries one run per head).
__global__ __launch_bounds__(kThreads) void fill_2d_kernel(float *p, int64_t ld, int64_t n_rows,
                                                           int64_t n_cols, float value)
{
    const int64_t n = n_rows * n_cols;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        p[(i / n_cols) * ld + i % n_cols] = value;
}

int64_t blocks_for_waves(int64_t n_waves) { return (n_waves + kThreads / 64 - 1) / (kThreads / 64); }

}  // namespace

hipError_t launch_bwd_dvec(const float *out, const void *dout, int dout_bf16, float *dvec,
                           int64_t ld, int64_t Sq, int Hq, int D, hipStream_t stream)
{
    const int64_t rows = Sq * Hq;
    if (rows == 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>(blocks_for_waves(rows), 256 * 16);
    hipLaunchKernelGGL(bwd_dvec_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, out,
                       dout, dout_bf16, dvec, ld, Sq, Hq, D);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 256 * 32);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_fill_2d(float *p, int64_t ld, int64_t n_rows, int64_t n_cols, float value,
                          hipStream_t stream)
{
    const int64_t n = n_rows * n_cols;
    if (n == 0)
        return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 256 * 32);
    hipLaunchKernelGGL(fill_2d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, ld,
                       n_rows, n_cols, value);
    return hipGetLastError();
}

hipError_t launch_bwd_f32(const BwdLaunch &b, hipStream_t stream)
{
    if (b.Sq > 0) {
        hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)blocks_for_waves(b.Sq * b.Hq)),
                           dim3(kThreads), 0, stream, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (b.Sk > 0)
        hipLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3((unsigned)blocks_for_waves(b.Sk * b.Hkv)),
                           dim3(kThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace cpattn
