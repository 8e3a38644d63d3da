// bwd_bf16.hip -- bf16 attention backward on CDNA4 matrix cores (gfx950),
// D = 128.
//
// Gradients of L = sum(dout * out) for the attention of the handbook page
// "上下文并行：Ring Attention 与 Ulysses", section "哪些运算可以直接切",
// function attention(), by the chain rule through its definition (the pages
// give no backward algorithm; they only ask, "Sequence Parallel vs Context
// Parallel" blog section 5.3, that gradients with context parallelism match
// those of one card):
//   P_ij  = exp(s_ij - lse_i)         (lse: the rows' final log-sum-exp)
//   ds_ij = P_ij (dout_i . v_j - dvec_i),  dvec_i = dout_i . out_i
//   dq_i  = sum_j ds_ij k_j / sqrt(D)
//   dk_j  = sum_i ds_ij q_i / sqrt(D),     dv_j = sum_i P_ij dout_i
// P and ds are rounded to bf16 before the products that take them; every
// product accumulates in float32.  No running max is needed: lse is known.
//
// Two kernels, each owning its outputs (no atomics):
//   * bwd_dq_kernel: a workgroup of 8 wavefronts owns 256 query rows of one
//     head (32 per wavefront) and streams the KV block through LDS 32 keys
//     at a time (3-stage ring of direct buffer->LDS loads).  Per 32-key
//     tile: S^T = K Q^T and dP^T = V dO^T (A = K or V fragments read from
//     LDS, B = Q^T or dO^T kept in VGPRs), ds in registers, then
//     dQ^T += K^T ds^T with K^T from transpose reads of the same K tile.  The
//     lane holds one query row, so lse and dvec are per-lane scalars.
//   * bwd_dkdv_kernel: a workgroup of 4 wavefronts (one per SIMD, so each
//     has 512 registers and dK, dV stay in accumulation registers) owns 128
//     keys of one KV head (32 per wavefront) and streams the query rows of
//     every head of its group through LDS 32 at a time (q, dout, lse and
//     dvec; 4-stage ring).  Per 32-query tile: S = Q K^T and dP = dO V^T
//     (A = Q or dO fragments from LDS, B = K^T or V^T in VGPRs), then
//     dV += P^T dO and dK += ds^T Q with P and ds from registers and dO, Q
//     from transpose reads.  The loop is software-pipelined: the MFMAs of
//     the next tile's S and dP are interleaved (scheduling groups) with this
//     tile's exponentials and ds, which a single wavefront per SIMD could
//     not otherwise overlap.
// Tiles use the forward kernel's layout: 256-byte rows with a 16-byte-chunk
// XOR swizzle that keeps ds_read_b128 row fragments and ds_read_b64_tr_b16
// column fragments free of bank conflicts.
#include "cp_kernels.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#include <utility>

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int HD = 128;
// Rows per streamed tile.  32 keeps a 3-stage ring of two tiles (plus the
// per-row statistics) below 64 KiB of LDS, so every fragment address is a
// per-lane offset plus an immediate; larger rings need extra address
// registers per stage, which the compiler keeps live across the loop.
constexpr int kTileRows = 32;
constexpr int kTileBytes = kTileRows * HD * 2;         // 8 KiB
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ tile helpers
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int c) { return r * 256 + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ bf16x8 lds_b128(const char LDS_AS *base, int off)
{
    return __builtin_bit_cast(bf16x8, *(const u32x4 LDS_AS *)(base + off));
}

__device__ __forceinline__ i16x4 lds_tr(const char LDS_AS *base, int off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(base + off));
}

// Per-lane LDS offsets of the fragments of a 32-row half tile:
//   row fragment (A or B operand with 8 consecutive columns of one row):
//     row l%32, columns 16*sd + 8*hi + [0, 8)  -> rowf[sd]
//   column fragment (8 rows of one column, the rows in the key order of the
//     accumulator registers 8*kh .. 8*kh+7): two transpose reads -> col[2][db]
struct FragOffsets {
    int rowf[8];
    int col[2][4];
};

__device__ __forceinline__ FragOffsets frag_offsets(int lane)
{
    FragOffsets f;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int sd = 0; sd < 8; ++sd)
        f.rowf[sd] = tile_off(l32, 2 * sd + hi);
    const int grp = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int dcol = db * 32 + 16 * (grp & 1) + 4 * (gi & 3);
        const int r0 = 4 * (grp >> 1) + (gi >> 2);
        f.col[0][db] = tile_off(r0, dcol >> 3) + (dcol & 7) * 2;
        f.col[1][db] = tile_off(r0 + 8, dcol >> 3) + (dcol & 7) * 2;
    }
    return f;
}

// Column fragment for 16-row step ks of a tile and 32-column block db.
__device__ __forceinline__ bf16x8 col_frag(const char LDS_AS *t, const FragOffsets &f, int ks,
                                           int db)
{
    const i16x4 lo = lds_tr(t, ks * 16 * 256 + f.col[0][db]);
    const i16x4 up = lds_tr(t, ks * 16 * 256 + f.col[1][db]);
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, up),
                                   0, 1, 2, 3, 4, 5, 6, 7);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (V#) over `bytes` bytes at `p`: no stride, the default
// data format of a gfx9 descriptor (word 3).  Loads through it whose offset
// lies past `bytes` return zeros.
__device__ __forceinline__ i32x4 rsrc(const void *p, int bytes)
{
    const uint64_t addr = (uint64_t)p;
    return i32x4{(int)(uint32_t)addr, (int)(uint32_t)(addr >> 32) & 0xffff, bytes, 0x00020000};
}

// The tile loads go to LDS directly (buffer_load ... lds, M0 = destination)
// and are written in assembly so that the compiler does not track them: its
// own tracking of such loads cannot tell the ring's stages apart in a rolled
// loop and would wait for every load in flight before each LDS read.  The
// kernels wait for them explicitly (s_waitcnt vmcnt before the barrier that
// publishes a tile).
__device__ __forceinline__ void dma16(uint32_t lds, int voff, const i32x4 &r)
{
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(lds), "v"(voff), "s"(r)
                     : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, int voff, const i32x4 &r)
{
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :
                     : "s"(lds), "v"(voff), "s"(r)
                     : "memory", "m0");
}

// Rows row0 .. row0+kTileRows-1 (of `len`) of two bf16 tensors with
// `row_stride` elements between rows (128 elements each) into the tiles at
// LDS addresses ta and tb: lane l of a load fills 16 bytes of a 1-KiB block
// (4 rows); rows past len read as zeros.  kWavesT wavefronts share the
// blocks; each issues 2 * kTileRows / 4 / kWavesT loads.
template <int kWavesT>
__device__ __forceinline__ void load_two_tiles(uint32_t ta, uint32_t tb, const __bf16 *a,
                                               const __bf16 *b, int64_t row_stride,
                                               int64_t row0, int64_t len, int wave, int lane)
{
    constexpr int kBlocks = kTileRows / 4;
    static_assert(kBlocks % kWavesT == 0, "blocks per wavefront");
    constexpr int kPer = kBlocks / kWavesT;
    __asm__ volatile("" : "+v"(lane));
    const int64_t rows = min(len - row0, (int64_t)kTileRows);   // >= 1
    const int row_bytes = (int)(row_stride * 2);
    const int bytes = (int)(rows - 1) * row_bytes + HD * 2;
    const i32x4 ra = rsrc(a + row0 * row_stride, bytes);
    const i32x4 rb = rsrc(b + row0 * row_stride, bytes);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int blk = wave * kPer + i;
        const int r = blk * 4 + (lane >> 4);
        const int off = r * row_bytes + (((lane & 15) ^ swz(r)) << 4);
        dma16(ta + blk * 1024, off, ra);
        dma16(tb + blk * 1024, off, rb);
    }
}

// s_waitcnt operand waiting for the vector-memory counter only (gfx9
// encoding: vmcnt bits 3:0 and 15:14; expcnt 6:4, lgkmcnt 11:8 at maximum)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// every wavefront's LDS reads done, then the workgroup barrier
__device__ __forceinline__ void lds_barrier()
{
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ============================================================== dq kernel
constexpr int kDqWaves = 8;
constexpr int kDqRows = kDqWaves * 32;                 // 256 query rows
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kDqStage = 2 * kTileBytes;               // K then V

// the ring's three stages, K then V in each
__shared__ __attribute__((aligned(1024))) char g_dq[3 * kDqStage];
constexpr int kDqLoads = 2 * (kTileRows / 4) / kDqWaves;   // tile loads per wavefront

__global__ __launch_bounds__(kDqThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdLaunch b, int n_row_tiles)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    // later row tiles (more visible keys under the causal mask) first
    const int h = blockIdx.x % b.Hq;
    const int tile = n_row_tiles - 1 - (int)(blockIdx.x / b.Hq);
    const int64_t tile_row0 = (int64_t)tile * kDqRows;
    const int g = h / (b.Hq / b.Hkv);
    const int64_t q_stride = (int64_t)b.Hq * HD, kv_stride = (int64_t)b.Hkv * HD;
    const int64_t my_row = tile_row0 + wave * 32 + l32;
    const bool row_ok = my_row < b.Sq;

    // Q^T and dO^T fragments: row my_row, dims 16*sd + 8*hi + [0, 8)
    bf16x8 qf[8], df[8];
    {
        const int64_t r = row_ok ? my_row : 0;
        const u32x4 *qs = (const u32x4 *)((const __bf16 *)b.q + r * q_stride + h * HD + 8 * hi);
        const u32x4 *ds = (const u32x4 *)((const __bf16 *)b.dout + r * q_stride + h * HD + 8 * hi);
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            u32x4 x = qs[2 * sd], y = ds[2 * sd];
            if (!row_ok) {
                x = u32x4{0, 0, 0, 0};
                y = u32x4{0, 0, 0, 0};
            }
            qf[sd] = __builtin_bit_cast(bf16x8, x);
            df[sd] = __builtin_bit_cast(bf16x8, y);
        }
    }
    const float scale = 1.f / sqrtf((float)HD);
    const float c = kLog2e * scale;
    float lse2 = INFINITY, dvi = 0.f;         // rows without keys (or past Sq): P = 0
    if (row_ok) {
        const float l = b.lse[h * b.stat_ld + my_row];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dvi = b.dvec[h * b.stat_ld + my_row];
    }

    // keys visible to the tile's last row
    const int64_t first_pos = b.q_offset + tile_row0;
    const int64_t last_pos = b.q_offset + min(tile_row0 + kDqRows, b.Sq) - 1;
    int64_t n_keys = b.Sk;
    if (b.causal)
        n_keys = min(max(last_pos - b.k_offset + 1, (int64_t)0), b.Sk);
    const int n_tiles = (int)((n_keys + kTileRows - 1) / kTileRows);

    const __bf16 *kg = (const __bf16 *)b.k + g * HD;
    const __bf16 *vg = (const __bf16 *)b.v + g * HD;
    const uint32_t ring = (uint32_t)(uintptr_t)(char LDS_AS *)g_dq;
    auto issue = [&](int t) {
        if (t < n_tiles) {
            const uint32_t st = ring + (uint32_t)(t % 3) * kDqStage;
            load_two_tiles<kDqWaves>(st, st + kTileBytes, kg, vg, kv_stride,
                                     (int64_t)t * kTileRows, b.Sk, wave, lane);
        }
    };
    const FragOffsets fo = frag_offsets(lane);
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = f32x16{};

    auto tile_step = [&](int t) {
        // tile t landed in every wavefront (tile t+1, issued after it, may
        // still be in flight); tile t-1's stage, which takes tile t+2, is no
        // longer read
        if (t + 1 < n_tiles)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDqLoads));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        issue(t + 2);
        const char LDS_AS *kt = (const char LDS_AS *)g_dq + (t % 3) * kDqStage;
        const char LDS_AS *vt = kt + kTileBytes;
#pragma unroll
        for (int half = 0; half < kTileRows / 32; ++half) {
            // S^T = K Q^T, then dP^T = V dO^T, for the 32 keys of this half;
            // one set of eight fragments is live at a time
            f32x16 s = f32x16{}, dp = f32x16{};
            {
                bf16x8 kf[8];
#pragma unroll
                for (int sd = 0; sd < 8; ++sd)
                    kf[sd] = lds_b128(kt + half * 32 * 256, fo.rowf[sd]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int sd = 0; sd < 8; ++sd)
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sd], qf[sd], s, 0, 0, 0);
            }
            {
                bf16x8 vf[8];
#pragma unroll
                for (int sd = 0; sd < 8; ++sd)
                    vf[sd] = lds_b128(vt + half * 32 * 256, fo.rowf[sd]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int sd = 0; sd < 8; ++sd)
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[sd], df[sd], dp, 0, 0, 0);
            }
            // K^T fragments for dQ^T, requested while the MFMAs run
            bf16x8 kc[2][4];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    kc[kh][db] = col_frag(kt, fo, 2 * half + kh, db);
            __builtin_amdgcn_sched_barrier(0);
            const int64_t key0 = (int64_t)t * kTileRows + half * 32;
            const bool need_mask = (key0 + 32 > b.Sk) ||
                                   (b.causal && b.k_offset + key0 + 31 > first_pos);
            if (need_mask) {
                // key k (0..31) of the half is visible to this lane's row iff k <= lim
                const int tail = (int)min(max(b.Sk - 1 - key0, (int64_t)-1), (int64_t)64);
                const int base_c = (int)min(max(first_pos - b.k_offset - key0, (int64_t)-512),
                                            (int64_t)512);
                const int lim = b.causal ? min(tail, base_c + wave * 32 + l32) : tail;
                const int lim_l = max(lim, -1) - 4 * hi;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kc_i = 8 * (i >> 2) + (i & 3);   // key of register i
                    s[i] = kc_i > lim_l ? -INFINITY : s[i];
                }
            }
            bf16x8 dsf[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -lse2));
                dsf[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dvi));
            }
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[kh][db], dsf[kh],
                                                                     acc[db], 0, 0, 0);
            // the next half's fragments are not read ahead of these MFMAs
            // (that would hold two halves' registers at once)
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    issue(0);
    issue(1);
    for (int t = 0; t < n_tiles; ++t)
        tile_step(t);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no tile load outlives the loop

    // epilogue: lane holds dQ^T[d = 32*db + 8*(i/4) + 4*hi + i%4][row l32]
    if (!row_ok)
        return;
    float *dst = b.dq + (my_row * b.Hq + h) * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 *p = (f32x4 *)(dst + db * 32 + 8 * i4 + 4 * hi);
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v4[e] = acc[db][4 * i4 + e] * scale;
            if (b.accumulate)
                v4 += *p;
            *p = v4;
        }
}

// ============================================================ dk/dv kernel
constexpr int kKvWaves = 4;
constexpr int kKvRows = kKvWaves * 32;                 // 128 keys
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kStatBytes = 64 * 4;                     // one float per lane of the loading wave
constexpr int kKvStage = 2 * kTileBytes + 2 * kStatBytes;   // q, dout, lse, dvec

// the ring's three stages: q tile, dout tile, lse, dvec in each
__shared__ __attribute__((aligned(1024))) char g_kv[4 * kKvStage];
constexpr int kKvLoads = 2 * (kTileRows / 4) / kKvWaves;   // tile loads per wavefront
constexpr int kKvLoads0 = kKvLoads + 2;                     // wavefront 0 also loads lse, dvec

__global__ __launch_bounds__(kKvThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdLaunch b)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    // earlier key tiles (seen by more query rows under the causal mask) first
    const int g = blockIdx.x % b.Hkv;
    const int tile = (int)(blockIdx.x / b.Hkv);
    const int64_t key_row0 = (int64_t)tile * kKvRows;
    const int group = b.Hq / b.Hkv;
    const int64_t q_stride = (int64_t)b.Hq * HD, kv_stride = (int64_t)b.Hkv * HD;
    const int64_t my_key = key_row0 + wave * 32 + l32;
    const bool key_ok = my_key < b.Sk;

    // K^T and V^T fragments (B operands): key my_key, dims 16*sd + 8*hi + [0, 8)
    bf16x8 kf[8], vf[8];
    {
        const int64_t r = key_ok ? my_key : 0;
        const u32x4 *ks = (const u32x4 *)((const __bf16 *)b.k + r * kv_stride + g * HD + 8 * hi);
        const u32x4 *vs = (const u32x4 *)((const __bf16 *)b.v + r * kv_stride + g * HD + 8 * hi);
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            u32x4 x = ks[2 * sd], y = vs[2 * sd];
            if (!key_ok) {
                x = u32x4{0, 0, 0, 0};
                y = u32x4{0, 0, 0, 0};
            }
            kf[sd] = __builtin_bit_cast(bf16x8, x);
            vf[sd] = __builtin_bit_cast(bf16x8, y);
        }
    }
    const float scale = 1.f / sqrtf((float)HD);
    const float c = kLog2e * scale;

    // query tiles that see any of the workgroup's keys
    const int64_t first_key_pos = b.k_offset + key_row0;
    int64_t q_begin = 0;
    if (b.causal)
        q_begin = min(max(first_key_pos - b.q_offset, (int64_t)0), b.Sq);
    const int qt_begin = (int)(q_begin / kTileRows);
    const int n_qt = (int)((b.Sq + kTileRows - 1) / kTileRows) - qt_begin;
    const int n_iter = n_qt > 0 ? n_qt * group : 0;        // (head, query tile) pairs

    const uint32_t ring = (uint32_t)(uintptr_t)(char LDS_AS *)g_kv;
    auto issue = [&](int it) {
        if (it < n_iter) {
            const int h = g * group + it / n_qt;
            const int64_t q0 = (int64_t)(qt_begin + it % n_qt) * kTileRows;
            const uint32_t st = ring + (uint32_t)(it % 4) * kKvStage;
            load_two_tiles<kKvWaves>(st, st + kTileBytes, (const __bf16 *)b.q + h * HD,
                                     (const __bf16 *)b.dout + h * HD, q_stride, q0, b.Sq, wave,
                                     lane);
            if (wave == 0) {
                // lse and dvec of the tile's rows (rows past Sq read as zeros)
                const int64_t rows = min(b.Sq - q0, (int64_t)kTileRows);
                const int bytes = (int)rows * 4;
                dma4(st + 2 * kTileBytes, lane * 4, rsrc(b.lse + h * b.stat_ld + q0, bytes));
                dma4(st + 2 * kTileBytes + kStatBytes, lane * 4,
                     rsrc(b.dvec + h * b.stat_ld + q0, bytes));
            }
        }
    };

    const FragOffsets fo = frag_offsets(lane);
    f32x16 dka[4], dva[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dka[i] = f32x16{};
        dva[i] = f32x16{};
    }

    // S = Q K^T and dP = dO V^T of query tile it (its stage in the ring)
    // K^T and V^T fragments stay in AGPRs and the MFMAs read them there
    // directly (about 1.6% faster than letting the compiler copy them to
    // VGPRs each tile).  The compiler does not see inline-assembly MFMAs as
    // MFMAs, so the hazards it would cover are covered by the code's shape:
    // the first result is early-clobber (it must not alias Q or dO), each
    // chain accumulates into exactly its own destination, and S and dP are
    // first read by the VALU in the next pipeline step, after the 16 dV/dK
    // MFMAs behind the scheduling barrier have passed through the same
    // in-order matrix pipe.
    auto scores = [&](int it, f32x16 &s, f32x16 &dp) {
        const char LDS_AS *qt = (const char LDS_AS *)g_kv + (it % 4) * kKvStage;
        const char LDS_AS *dt = qt + kTileBytes;
        bf16x8 qa[8];
#pragma unroll
        for (int sd = 0; sd < 8; ++sd)
            qa[sd] = lds_b128(qt, fo.rowf[sd]);
        __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=&v"(s) : "v"(qa[0]), "a"(kf[0]));
#pragma unroll
        for (int sd = 1; sd < 8; ++sd)
            __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+v"(s) : "v"(qa[sd]), "a"(kf[sd]));
        bf16x8 da[8];
#pragma unroll
        for (int sd = 0; sd < 8; ++sd)
            da[sd] = lds_b128(dt, fo.rowf[sd]);
        __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                         : "=&v"(dp) : "v"(da[0]), "a"(vf[0]));
#pragma unroll
        for (int sd = 1; sd < 8; ++sd)
            __asm__ volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                             : "+v"(dp) : "v"(da[sd]), "a"(vf[sd]));
    };
    // waits until tile `it` is complete in every wavefront, `ahead` later
    // tiles may still be in flight
    auto wait_tile = [&](int ahead) {
        if (ahead >= 2) {
            if (wave == 0)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kKvLoads0));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kKvLoads));
        } else if (ahead == 1) {
            if (wave == 0)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kKvLoads0));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(kKvLoads));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        lds_barrier();
    };

    // Software pipeline over query tiles: step it runs S and dP of tile it+1
    // on the matrix cores while the VALU turns tile it's S and dP into P and
    // dS, then dV += P^T dO and dK += dS^T Q for tile it.  Four ring stages:
    // tiles it and it+1 are read, it+2 is in flight, it+3 is issued into the
    // stage of it-1.
    f32x16 s_cur, dp_cur;
    issue(0);
    issue(1);
    issue(2);
    if (n_iter > 0) {
        wait_tile(min(n_iter - 1, 2));
        scores(0, s_cur, dp_cur);
    }
    // one pipeline step: consumes tile it's S and dP (s_c, dp_c), produces
    // tile it+1's (s_n, dp_n; recomputed from tile it on the last step, and
    // unused) -- unconditional, so the scheduler sees the MFMAs and the VALU
    // work in one block
    auto step = [&](int it, f32x16 &s_c, f32x16 &dp_c, f32x16 &s_n, f32x16 &dp_n) {
        if (it + 1 < n_iter) {
            // outstanding: tiles it+1 and (if any) it+2
            wait_tile(min(n_iter - 2 - it, 1));
            issue(it + 3);
        }
        const char LDS_AS *qt = (const char LDS_AS *)g_kv + (it % 4) * kKvStage;
        const char LDS_AS *dt = qt + kTileBytes;
        const float LDS_AS *lt = (const float LDS_AS *)(qt + 2 * kTileBytes);
        const float LDS_AS *vt = lt + kStatBytes / 4;
        f32x4 l4s[4], d4s[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            l4s[i4] = *(const f32x4 LDS_AS *)(lt + 8 * i4 + 4 * hi);
            d4s[i4] = *(const f32x4 LDS_AS *)(vt + 8 * i4 + 4 * hi);
        }
        scores(it + 1 < n_iter ? it + 1 : it, s_n, dp_n);
        const int64_t q0 = (int64_t)(qt_begin + it % n_qt) * kTileRows;
        const int64_t qpos0 = b.q_offset + q0;
        const bool need_mask = b.causal && first_key_pos + kKvRows - 1 > qpos0;
        int lim = -1;
        if (need_mask)
            lim = (int)min(max(b.k_offset + my_key - qpos0, (int64_t)-1), (int64_t)64);
        bf16x8 pf[2], sf[2];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 l4 = l4s[i4];
            const f32x4 d4 = d4s[i4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * i4 + e;
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_c[i], c, -l4[e] * kLog2e));
                const int qi = 8 * i4 + 4 * hi + e;
                p = qi >= lim ? p : 0.f;
                pf[i >> 3][i & 7] = (__bf16)p;
                sf[i >> 3][i & 7] = (__bf16)(p * (dp_c[i] - d4[e]));
            }
        }
        // interleave: the 16 MFMAs of the next tile's S and dP, each followed
        // by a share of this tile's VALU work
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
            bf16x8 dc[2][4];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dc[kh][db] = col_frag(dt, fo, kh, db);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[kh], dc[kh][db], dva[db],
                                                                     0, 0, 0);
        }
        {
            bf16x8 qc[2][4];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    qc[kh][db] = col_frag(qt, fo, kh, db);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf[kh], qc[kh][db], dka[db],
                                                                     0, 0, 0);
        }
    };
    f32x16 s_alt, dp_alt;
    for (int it = 0; it < n_iter; it += 2) {
        step(it, s_cur, dp_cur, s_alt, dp_alt);
        if (it + 1 >= n_iter)
            break;
        step(it + 1, s_alt, dp_alt, s_cur, dp_cur);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no tile load outlives the loop

    // epilogue: lane holds dK[key = 8*(i/4) + 4*hi + i%4][d = 32*db + l32]
    // (and dV likewise) for the wavefront's 32 keys
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t key = key_row0 + wave * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (key >= b.Sk)
            continue;
        float *pk = b.dk + (key * b.Hkv + g) * HD + l32;
        float *pv = b.dv + (key * b.Hkv + g) * HD + l32;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const float k_val = dka[db][i] * scale + (b.accumulate ? pk[db * 32] : 0.f);
            const float v_val = dva[db][i] + (b.accumulate ? pv[db * 32] : 0.f);
            pk[db * 32] = k_val;
            pv[db * 32] = v_val;
        }
    }
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdLaunch &b, hipStream_t stream)
{
    if (b.Sq > 0) {
        const int n_row_tiles = (int)((b.Sq + kDqRows - 1) / kDqRows);
        hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((int64_t)n_row_tiles * b.Hq)),
                           dim3(kDqThreads), 0, stream, b, n_row_tiles);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (b.Sk > 0) {
        const int64_t n_key_tiles = (b.Sk + kKvRows - 1) / kKvRows;
        hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(n_key_tiles * b.Hkv)),
                           dim3(kKvThreads), 0, stream, b);
    }
    return hipGetLastError();
}

}  // namespace cpattn
