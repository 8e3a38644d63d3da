// attn_f32.hip -- float32 blockwise attention with per-row log-sum-exp, the
// exactness path (handbook page "上下文并行：Ring Attention 与 Ulysses",
// section "哪些运算可以直接切", function attention()).
//
// One wavefront per (64 query rows, head).  Each lane owns one query row: q
// and the running output live in registers, keys and values are staged in
// LDS 32 at a time and read as broadcasts.  The softmax is the running
// (m, l, o) form ("Sequence Parallel vs Context Parallel" blog, section 3.2)
// updated key by key in float32 with the natural exponential.  The causal
// mask compares absolute positions: key j of a segment is visible to row i
// iff kv.pos0 + j <= q.pos0 + i.
#include "cp_kernels.h"

#include <math.h>

namespace cpattn {

namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wavefront)
constexpr int kKeys = 32;   // keys staged per LDS tile

struct TileMap {
    int32_t start[kMaxQSegs + 1];  // prefix sum of row tiles over the segments
};

template <int DMAX>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(AttnLaunch a, TileMap tm)
{
    __shared__ float ks[kKeys][DMAX];
    __shared__ float vs[kKeys][DMAX];

    const int h = blockIdx.y;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.n_q && tile >= tm.start[s + 1])
        ++s;
    const QSeg &qs = a.qs[s];
    const int64_t row_in_seg = (int64_t)(tile - tm.start[s]) * kRows + threadIdx.x;
    const bool row_ok = row_in_seg < qs.len;
    const int D = a.D;
    const int g = h / (a.Hq / a.Hkv);
    const float scale = 1.0f / sqrtf((float)D);
    const float *q = (const float *)a.q;
    const float *k = (const float *)a.k;
    const float *v = (const float *)a.v;

    float qr[DMAX];
    float o[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) {
        qr[d] = (row_ok && d < D) ? q[((qs.row0 + row_in_seg) * a.Hq + h) * D + d] * scale : 0.f;
        o[d] = 0.f;
    }
    const int64_t qpos = qs.pos0 + row_in_seg;
    const int64_t tile_first = (int64_t)(tile - tm.start[s]) * kRows;
    const int64_t tile_last = min(tile_first + kRows, qs.len) - 1;
    float m = -INFINITY;
    float l = 0.f;

    for (int kv_i = 0; kv_i < qs.n_kv; ++kv_i) {
        const KvSeg kv = qs.kv[kv_i];
        int64_t n_keys = kv.len;
        if (a.causal) {
            const int64_t last_pos = qs.pos0 + tile_last;
            n_keys = min(max(last_pos - kv.pos0 + 1, (int64_t)0), kv.len);
        }
        for (int64_t j0 = 0; j0 < n_keys; j0 += kKeys) {
            __syncthreads();
            for (int e = threadIdx.x; e < kKeys * DMAX; e += kRows) {
                const int jj = e / DMAX;
                const int d = e - jj * DMAX;
                const bool ok = (j0 + jj < kv.len) && d < D;
                const int64_t src = ((kv.row0 + j0 + jj) * a.Hkv + g) * D + d;
                ks[jj][d] = ok ? k[src] : 0.f;
                vs[jj][d] = ok ? v[src] : 0.f;
            }
            __syncthreads();
            const int jn = (int)min((int64_t)kKeys, n_keys - j0);
            for (int jj = 0; jj < jn; ++jj) {
                if (a.causal && kv.pos0 + j0 + jj > qpos)
                    continue;
                float sc = 0.f;
#pragma unroll
                for (int d = 0; d < DMAX; ++d)
                    sc = fmaf(qr[d], ks[jj][d], sc);
                if (sc > m) {
                    const float alpha = expf(m - sc);   // 0 when m = -inf
                    l = l * alpha + 1.f;
#pragma unroll
                    for (int d = 0; d < DMAX; ++d)
                        o[d] = fmaf(o[d], alpha, vs[jj][d]);
                    m = sc;
                } else {
                    const float p = expf(sc - m);
                    l += p;
#pragma unroll
                    for (int d = 0; d < DMAX; ++d)
                        o[d] = fmaf(p, vs[jj][d], o[d]);
                }
            }
        }
    }
    if (!row_ok)
        return;
    const int64_t orow = qs.out_row0 + row_in_seg;
    float *out = a.out + (orow * a.Hq + h) * D;
    float *lse = a.lse + (int64_t)h * a.lse_ld + orow;
    const float lse_blk = l > 0.f ? m + logf(l) : -INFINITY;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    if (!qs.merge) {
#pragma unroll
        for (int d = 0; d < DMAX; ++d)
            if (d < D)
                out[d] = o[d] * inv_l;
        *lse = lse_blk;
        return;
    }
    const float lse_old = *lse;
    const float mx = fmaxf(lse_old, lse_blk);
    if (mx == -INFINITY)
        return;  // both empty: the stored (0, -inf) stays
    const float lse_new = mx + log1pf(expf(-fabsf(lse_old - lse_blk)));
    const float w_old = expf(lse_old - lse_new);
    const float w_blk = expf(lse_blk - lse_new) * inv_l;
#pragma unroll
    for (int d = 0; d < DMAX; ++d)
        if (d < D)
            out[d] = out[d] * w_old + o[d] * w_blk;
    *lse = lse_new;
}

template <int DMAX>
hipError_t launch_dmax(const AttnLaunch &a, const TileMap &tm, int total_tiles,
                       hipStream_t stream)
{
    hipLaunchKernelGGL((attn_f32_kernel<DMAX>), dim3(total_tiles, a.Hq), dim3(kRows), 0,
                       stream, a, tm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnLaunch &a, hipStream_t stream)
{
    TileMap tm{};
    int64_t total = 0;
    for (int s = 0; s < a.n_q; ++s) {
        tm.start[s] = (int32_t)total;
        total += (a.qs[s].len + kRows - 1) / kRows;
    }
    tm.start[a.n_q] = (int32_t)total;
    if (total == 0 || a.Hq == 0)
        return hipSuccess;
    if (a.D <= 32)
        return launch_dmax<32>(a, tm, (int)total, stream);
    if (a.D <= 64)
        return launch_dmax<64>(a, tm, (int)total, stream);
    return launch_dmax<128>(a, tm, (int)total, stream);
}

}  // namespace cpattn
