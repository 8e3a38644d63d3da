// attn_bf16.hip -- bf16 blockwise attention with per-row log-sum-exp on
// CDNA4 matrix cores (gfx950), D = 128.
//
// Operation (handbook page "上下文并行：Ring Attention 与 Ulysses", section
// "哪些运算可以直接切", function attention()): s = q.k / sqrt(D), keys after
// the query's absolute position masked, lse = logsumexp(s), out =
// softmax(s) v.  The softmax runs in the streaming (m, l, o) form ("Sequence
// Parallel vs Context Parallel" blog, section 3.2), in base 2 with
// log2(e)/sqrt(D) folded into one multiply; lse is converted back to nats.
//
// Work decomposition
//   * A workgroup of 4 wavefronts owns BM = 128 query rows of one head; each
//     wavefront owns 32 rows.  Keys stream through LDS BN = 64 at a time.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = 16 dims x
//     32 queries held in VGPRs for the whole kernel).  In the accumulator
//     layout lane l then holds 16 scores of query l%32, so row max and row sum
//     are in-lane reductions plus one exchange with lane l^32.
//   * The output is accumulated transposed, O^T += V^T P^T.  The B operand
//     P^T needs, per lane, 8 scores of its own query: exactly 8 consecutive
//     accumulator registers, converted to bf16 in place (no data movement).
//     The key order inside a 16-key MFMA step is permuted consistently for P
//     and V; the A operand V^T is read from a d-major copy of the V tile in
//     LDS.  O^T keeps each lane on one query, so the rescale by
//     exp2(m_old - m_new) is a per-lane scalar.
//   * Tiles strictly below the causal diagonal run without the mask; only
//     tiles crossing the diagonal (or a ragged end) compare positions.
//   * The epilogue either writes (out, lse) or folds the block result into
//     the (out, lse) already stored (log-sum-exp merge, handbook section
//     "Ring Attention：KV 沿环传一圈").
#include "cp_kernels.h"

#include <math.h>

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;            // head dimension
constexpr int BM = 128;            // query rows per workgroup
constexpr int BN = 64;             // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int VT_LD = 66;          // bf16 per row of the d-major V tile (padded)

struct TileMap {
    int32_t start[kMaxQSegs + 1];  // prefix sum of row tiles over the segments
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ float wave_xor32(float x)
{
    return __shfl_xor(x, 32, 64);
}

__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(AttnLaunch a, TileMap tm,
                                                             float scale_log2)
{
    __shared__ u32x4 k_lds[BN * 16];                 // [key][16-byte chunk], XOR-swizzled
    __shared__ unsigned short vt_lds[HD * VT_LD];    // [d][key], padded rows

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int h = blockIdx.y;

    int s = 0;
    while (s + 1 < a.n_q && (int)blockIdx.x >= tm.start[s + 1])
        ++s;
    const QSeg &qs = a.qs[s];
    const int n_tiles_seg = tm.start[s + 1] - tm.start[s];
    // heavy tiles (later rows see more keys under the causal mask) first
    const int tile = n_tiles_seg - 1 - ((int)blockIdx.x - tm.start[s]);
    const int64_t tile_row0 = (int64_t)tile * BM;
    const int64_t my_row = tile_row0 + wave * 32 + l32;
    const bool row_ok = my_row < qs.len;
    const int64_t my_pos = qs.pos0 + my_row;
    const int g = h / (a.Hq / a.Hkv);

    const __bf16 *qg = (const __bf16 *)a.q;
    const __bf16 *kg = (const __bf16 *)a.k;
    const __bf16 *vg = (const __bf16 *)a.v;

    // Q^T fragments: B operand of step sd holds dims 16*sd + 8*hi + [0, 8) of row l32.
    bf16x8 qf[8];
    {
        const int64_t r = row_ok ? my_row : 0;
        const u32x4 *src = (const u32x4 *)(qg + ((qs.row0 + r) * a.Hq + h) * HD + 8 * hi);
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            u32x4 x = src[2 * sd];
            if (!row_ok)
                x = u32x4{0, 0, 0, 0};
            qf[sd] = as_bf16x8(x);
        }
    }

    f32x16 o_acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o_acc[i] = f32x16{};
    float m_run = -INFINITY;   // running max, log2 units
    float l_run = 0.f;         // running sum of exp2(s - m_run)

    const int64_t first_pos = qs.pos0 + tile_row0;
    const int64_t last_pos = qs.pos0 + min(tile_row0 + BM, qs.len) - 1;

    for (int kv_i = 0; kv_i < qs.n_kv; ++kv_i) {
        const KvSeg kv = qs.kv[kv_i];
        int64_t n_keys = kv.len;
        if (a.causal)
            n_keys = min(max(last_pos - kv.pos0 + 1, (int64_t)0), kv.len);
        for (int64_t key0 = 0; key0 < n_keys; key0 += BN) {
            // ---- stage K (swizzled, row-major) and V (transposed) in LDS
            __syncthreads();
#pragma unroll
            for (int it = 0; it < (BN * 16) / kThreads; ++it) {
                const int cid = it * kThreads + threadIdx.x;
                const int row = cid >> 4;
                const int c = cid & 15;
                const int64_t key = key0 + row;
                u32x4 kx = u32x4{0, 0, 0, 0};
                u32x4 vx = u32x4{0, 0, 0, 0};
                if (key < kv.len) {
                    const int64_t off = ((kv.row0 + key) * a.Hkv + g) * HD + c * 8;
                    kx = *(const u32x4 *)(kg + off);
                    vx = *(const u32x4 *)(vg + off);
                }
                k_lds[row * 16 + (c ^ (row & 15))] = kx;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vt_lds[(c * 8 + 2 * e) * VT_LD + row] = (unsigned short)(vx[e] & 0xffffu);
                    vt_lds[(c * 8 + 2 * e + 1) * VT_LD + row] = (unsigned short)(vx[e] >> 16);
                }
            }
            __syncthreads();

            // ---- S^T = K Q^T for two 32-key blocks
            f32x16 sc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                sc[kb] = f32x16{};
                const int row = kb * 32 + l32;
#pragma unroll
                for (int sd = 0; sd < 8; ++sd) {
                    const int c = 2 * sd + hi;
                    const bf16x8 kf = as_bf16x8(k_lds[row * 16 + (c ^ (row & 15))]);
                    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[sd], sc[kb], 0, 0, 0);
                }
            }

            // ---- scale, mask, running max
            const bool need_mask =
                (key0 + BN > kv.len) || (a.causal && kv.pos0 + key0 + BN - 1 > first_pos);
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float x = sc[kb][i] * scale_log2;
                    if (need_mask) {
                        const int key = kb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
                        const bool dead = (key0 + key >= kv.len) ||
                                          (a.causal && kv.pos0 + key0 + key > my_pos);
                        x = dead ? -INFINITY : x;
                    }
                    sc[kb][i] = x;
                    mx = fmaxf(mx, x);
                }
            }
            mx = fmaxf(mx, wave_xor32(mx));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(sc[kb][i] - m_use);
                    sc[kb][i] = p;
                    rs += p;
                }
            }
            rs += wave_xor32(rs);
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o_acc[db] *= alpha;

            // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 pf;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pf[j] = (__bf16)sc[ks >> 1][8 * (ks & 1) + j];
                // keys of this lane for MFMA k-index 8*hi + j:
                //   16*ks + 8*(j/4) + 4*hi + (j%4)
                const int ka = 16 * ks + 4 * hi;
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int d = db * 32 + l32;
                    const unsigned int *vrow = (const unsigned int *)(vt_lds + d * VT_LD);
                    u32x4 vx;
                    vx[0] = vrow[ka / 2];
                    vx[1] = vrow[ka / 2 + 1];
                    vx[2] = vrow[(ka + 8) / 2];
                    vx[3] = vrow[(ka + 8) / 2 + 1];
                    o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vx), pf,
                                                                        o_acc[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: lane l holds O^T[d = 32*db + 8*(i/4) + 4*hi + i%4][row l32]
    if (!row_ok)
        return;
    const int64_t orow = qs.out_row0 + my_row;
    float *out = a.out + (orow * a.Hq + h) * HD;
    float *lse_p = a.lse + (int64_t)h * a.lse_ld + orow;
    const float kLn2 = 0.6931471805599453f;
    const float lse_blk = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
    if (!qs.merge) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = o_acc[db][4 * i4 + e] * inv_l;
                *(f32x4 *)(out + db * 32 + 8 * i4 + 4 * hi) = v4;
            }
        if (hi == 0)
            *lse_p = lse_blk;
        return;
    }
    const float lse_old = *lse_p;
    const float mxl = fmaxf(lse_old, lse_blk);
    if (mxl == -INFINITY)
        return;
    const float lse_new = mxl + log1pf(expf(-fabsf(lse_old - lse_blk)));
    const float w_old = expf(lse_old - lse_new);
    const float w_blk = expf(lse_blk - lse_new) * inv_l;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 *dst = (f32x4 *)(out + db * 32 + 8 * i4 + 4 * hi);
            f32x4 old = *dst;
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v4[e] = old[e] * w_old + o_acc[db][4 * i4 + e] * w_blk;
            *dst = v4;
        }
    // both halves of the wavefront read lse_old above before this store
    if (hi == 0)
        *lse_p = lse_new;
}

}  // namespace

hipError_t launch_attn_bf16(const AttnLaunch &a, hipStream_t stream)
{
    TileMap tm{};
    int64_t total = 0;
    for (int s = 0; s < a.n_q; ++s) {
        tm.start[s] = (int32_t)total;
        total += (a.qs[s].len + BM - 1) / BM;
    }
    tm.start[a.n_q] = (int32_t)total;
    if (total == 0 || a.Hq == 0)
        return hipSuccess;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)total, a.Hq), dim3(kThreads), 0, stream,
                       a, tm, scale_log2);
    return hipGetLastError();
}

}  // namespace cpattn
