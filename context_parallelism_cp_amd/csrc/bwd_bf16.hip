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
//     at a time (3-stage ring of direct buffer->LDS loads); the launch's
//     row tiles are spread over the XCDs so that the workgroups an XCD holds
//     at a time stream the same K/V tiles.  Per 32-key
//     tile: S^T = K Q^T and dP^T = V dO^T (A = K or V fragments read from
//     LDS, B = Q^T or dO^T kept in VGPRs; the dP product starts from -dvec
//     instead of zero, so it yields dP - dvec), ds in registers, then
//     dQ^T += K^T ds^T with K^T from transpose reads of the same K tile.  The
//     lane holds one query row, so lse and dvec are per-lane scalars.
//   * bwd_dkdv_kernel: a workgroup of 8 wavefronts (two per SIMD) owns 128
//     keys of one KV head, 32 per pair of wavefronts on one SIMD, and
//     streams the query rows of every head of its group through LDS 32 at a
//     time (q, dout, lse and dvec; 5-stage ring).  The pair splits the work
//     by role: one wavefront keeps K^T in registers and computes S = Q K^T,
//     P and dV += P^T dO; the other keeps V^T and computes dP = dO V^T,
//     dS = P (dP - dvec) and dK += dS^T Q one tile later, P passing between
//     them through LDS.  Halving each wavefront's registers this way puts two
//     of them on a SIMD.  Under the causal mask a workgroup takes key tiles
//     t and n-1-t (equal work), walking the first one's query tiles down and
//     the second one's up, and the workgroups an XCD holds at a time belong
//     to one KV head, so they read the same query tiles from L2 together.
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
static_assert(kTileRows == 32 && kDqLoads == 2, "one K and one V block per wavefront and tile");

// Order of the dq launch's (head, row tile) units over the XCDs (workgroup
// b runs on XCD b % 8, as its slot b / 8):
//   mode 0: the units head-major, later row tiles (more keys under the
//     causal mask) first within a head, cut into 8 contiguous runs of
//     per_xcd: the workgroups an XCD holds at a time stream one head's K/V;
//   mode 1 (causal, KV heads not a multiple of 8): per head, the row tiles
//     cut into 16 bands (sizes differing by one at most, `band` the
//     largest); XCD x takes band 15 - x, then band x, each from its last
//     tile down (equal work per XCD; an XCD's
//     workgroups are neighbouring row tiles that stream the same keys at
//     about the same time).
struct DqWork {
    int mode;
    int n_row_tiles;
    int per_xcd;      // mode 0
    int band;         // mode 1
};

__global__ __launch_bounds__(kDqThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdLaunch b, DqWork w)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int n_row_tiles = w.n_row_tiles;
    int h, tile;
    {
        const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
        if (w.mode == 0) {
            const int64_t lin = (int64_t)x * w.per_xcd + slot;
            if (slot >= w.per_xcd || lin >= (int64_t)n_row_tiles * b.Hq)
                return;
            h = (int)(lin / n_row_tiles);
            tile = n_row_tiles - 1 - (int)(lin % n_row_tiles);
        } else {
            // band k holds row tiles [k*M/16, (k+1)*M/16)
            const int M = n_row_tiles;
            h = slot / (2 * w.band);
            const int s = slot % (2 * w.band);
            const int h0 = (15 - x) * M / 16, sh = (16 - x) * M / 16 - h0;
            const int l0 = x * M / 16, sl = (x + 1) * M / 16 - l0;
            tile = s < sh ? h0 + (sh - 1 - s) : (s - sh < sl ? l0 + (sl - 1 - (s - sh)) : M);
            if (h >= b.Hq || tile >= n_row_tiles)
                return;
        }
    }
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
    // 32-bit key bounds for the loads and the mask (Sk < 2^30): key k is past
    // the block iff k >= sk32, and the wavefront's row at offset r sees k
    // iff k <= diag32 + r (first_pos - k_offset clamped to [-512, Sk + 64],
    // which changes no decision: rows are fewer than 512, keys end at Sk)
    const int sk32 = (int)b.Sk;
    const int diag32 = __builtin_amdgcn_readfirstlane(
        (int)min(max(first_pos - b.k_offset, (int64_t)-512), b.Sk + 64));
    // each lane's byte offsets into a tile for its share of the loads
    const int row_bytes = (int)(kv_stride * 2);
    int dma_off[kDqLoads / 2];
#pragma unroll
    for (int i = 0; i < kDqLoads / 2; ++i) {
        const int rr = (wave * (kDqLoads / 2) + i) * 4 + (lane >> 4);
        dma_off[i] = rr * row_bytes + (((lane & 15) ^ swz(rr)) << 4);
    }
    auto issue = [&](int t) {
        if (t < n_tiles) {
            const uint32_t st = ring + (uint32_t)(t % 3) * kDqStage;
            const int key0 = t * kTileRows;
            const int rows = min(sk32 - key0, kTileRows);
            const int bytes = (rows - 1) * row_bytes + HD * 2;
            const i32x4 ra = rsrc(kg + (int64_t)key0 * kv_stride, bytes);
            const i32x4 rb = rsrc(vg + (int64_t)key0 * kv_stride, bytes);
#pragma unroll
            for (int i = 0; i < kDqLoads / 2; ++i) {
                const int blk = wave * (kDqLoads / 2) + i;
                dma16(st + blk * 1024, dma_off[i], ra);
                dma16(st + kTileBytes + blk * 1024, dma_off[i], rb);
            }
        }
    };
    const FragOffsets fo = frag_offsets(lane);
    // dP - dvec comes out of the dP product directly: its accumulator input
    // is -dvec (the lane's row) instead of zero
    f32x16 neg_dv;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        neg_dv[i] = -dvi;
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
        // this step's per-lane LDS addresses: the stage offset added once to
        // each fragment's lane offset, the K / V / row parts as immediates
        int so = (t % 3) * kDqStage;
        // opaque, so that the compiler adds it once per fragment instead of
        // strength-reducing the modulo into extra per-read arithmetic
        __asm__ volatile("" : "+s"(so));
        int rowb[8], colb[2][4];
#pragma unroll
        for (int sd = 0; sd < 8; ++sd)
            rowb[sd] = fo.rowf[sd] + so;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                colb[x][db] = fo.col[x][db] + so;
        const char LDS_AS *lds = (const char LDS_AS *)g_dq;
        // S^T = K Q^T, then dP^T = V dO^T, for the tile's 32 keys; one set of
        // eight fragments is live at a time
        f32x16 s = f32x16{}, dp = neg_dv;
        {
            bf16x8 kf[8];
#pragma unroll
            for (int sd = 0; sd < 8; ++sd)
                kf[sd] = lds_b128(lds, rowb[sd]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int sd = 0; sd < 8; ++sd)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sd], qf[sd], s, 0, 0, 0);
        }
        {
            bf16x8 vf[8];
#pragma unroll
            for (int sd = 0; sd < 8; ++sd)
                vf[sd] = lds_b128(lds + kTileBytes, rowb[sd]);
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
            for (int db = 0; db < 4; ++db) {
                const i16x4 lo = lds_tr(lds + kh * 16 * 256, colb[0][db]);
                const i16x4 up = lds_tr(lds + kh * 16 * 256, colb[1][db]);
                kc[kh][db] = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                     __builtin_bit_cast(bf16x4, up), 0, 1, 2, 3,
                                                     4, 5, 6, 7);
            }
        __builtin_amdgcn_sched_barrier(0);
        const int key0 = t * kTileRows;
        const bool need_mask = (key0 + 32 > sk32) || (b.causal && key0 + 31 > diag32);
        if (need_mask) {
            // key k (0..31) of the tile is visible to this lane's row iff k <= lim
            const int tail = min(max(sk32 - 1 - key0, -1), 64);
            const int base_c = min(max(diag32 - key0, -512), 512);
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
            dsf[i >> 3][i & 7] = (__bf16)(p * dp[i]);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[kh][db], dsf[kh], acc[db], 0,
                                                                 0, 0);
        __builtin_amdgcn_sched_barrier(0);
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
    // every load before the first store (the loads in flight together, the
    // stores without waits between them)
    f32x4 v4[4][4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v4[db][i4][e] = acc[db][4 * i4 + e] * scale;
    if (b.accumulate) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                v4[db][i4] += *(const f32x4 *)(dst + db * 32 + 8 * i4 + 4 * hi);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *(f32x4 *)(dst + db * 32 + 8 * i4 + 4 * hi) = v4[db][i4];
}

// ============================================================ dk/dv kernel
// A workgroup of 8 wavefronts owns 128 keys of one KV head: 4 pairs of 32
// keys, the two wavefronts of a pair on one SIMD (wavefronts w and w + 4).
// The pair splits the work of its keys by role:
//   role 0 keeps K^T in registers: S = Q K^T, P = exp(S - lse) (masked),
//          dV += P^T dO; it passes P (float32) to role 1 through LDS;
//   role 1 keeps V^T in registers: dP - dvec = dO V^T - dvec (the product
//          starts from the rows' negated dvec), dS = P (dP - dvec),
//          dK += dS^T Q, one query tile behind role 0 (it reads the P that
//          role 0 wrote before the previous barrier).
// Each wavefront then holds one key-side operand and one accumulator pair
// (about half of what one wavefront doing all four products needs), so two
// fit on a SIMD and the SIMD interleaves one's matrix work with the other's
// exponentials and waits.  Every product is the one the single-wavefront
// form computes, in the same order.
//
// LDS: the ring's q tiles, then its dout tiles, then its lse/dvec rows, then
// P (double-buffered).  Each role keeps per-lane base registers into the
// regions it reads (row fragments, column fragments, its statistics, its
// pair's P) and the step adds one uniform stage offset: one address add per
// fragment read.  Every batch of LDS reads (row fragments, statistics, P,
// column fragments) is issued whole before the arithmetic that takes it (a
// scheduling barrier after the batch): left to itself the scheduler
// interleaved read, wait and product one fragment at a time, eight LDS round
// trips in a row.  The epilogue's addresses are computed from an opaque copy
// of the lane index so that they are not hoisted out of the step loop and
// kept live across it (34 registers).
constexpr int kKvWaves = 8;
constexpr int kKvPairs = 4;
constexpr int kKvRows = kKvPairs * 32;                 // 128 keys
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKvStages = 5;
constexpr int kKvAhead = 3;        // tile it + 3 is requested at step it (stages - 2)
constexpr int kStatBytes = 64 * 4;                     // one float per lane of the loading wave
constexpr int kPBytes = 64 * 16 * 4;                   // a pair's P: 16 floats per lane
constexpr int kQOff = 0;                               // q tile of stage s: kQOff + s * kTileBytes
constexpr int kDOff = kKvStages * kTileBytes;          // dout tile of stage s
constexpr int kSOff = 2 * kKvStages * kTileBytes;      // lse of stage s, then dvec (+kStatBytes)
constexpr int kPOff = kSOff + (kKvStages * 2 * kStatBytes + 1023) / 1024 * 1024;   // P: pair, buffer
constexpr int kKvLds = kPOff + 2 * kKvPairs * kPBytes;
static_assert(kDOff + kKvStages * kTileBytes <= kSOff && kPOff % 1024 == 0, "LDS layout");

__shared__ __attribute__((aligned(1024))) char g_kv[kKvLds];
constexpr int kKvLoads = 2 * (kTileRows / 4) / kKvWaves;   // tile loads per wavefront
constexpr int kKvLoads0 = kKvLoads + 2;                     // wavefront 0 also loads lse, dvec
static_assert(kKvLoads == 2, "one q and one dout block per wavefront and tile");

// Work of one block's dk/dv: `units` per KV head, each one key tile or
// (under the causal mask) the pair of key tiles t and n_key_tiles - 1 - t,
// whose visible query rows add up to about the same count for every t.
// A launch takes the units of all KV heads, head-major (with two blocks in
// one launch, the first block's units, then the second's), cut into 8
// contiguous runs of `per_xcd`, one per XCD (workgroup b runs on XCD b % 8),
// so the workgroups an XCD holds at a time belong to one KV head and read
// the same query tiles.
struct KvWork {
    int units;        // units per KV head
    int per_xcd;      // units per XCD (of the launch)
    int paired;       // 1: a unit is a pair of key tiles
    int n_key_tiles;
};

template <int N>
using IC = std::integral_constant<int, N>;

// kBlocks = 2: two blocks whose dk/dv rows are disjoint in one launch (a
// causal block of few KV heads has fewer key-tile pairs than the chip has
// CUs; two of them fill it); the second block's arguments are b1, w1.
template <int kBlocks>
__global__ __launch_bounds__(kKvThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdLaunch b, KvWork w, BwdLaunch b1, KvWork w1)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = wave % kKvPairs;
    const int role = wave / kKvPairs;
    const int l32 = lane & 31, hi = lane >> 5;
    int g, tiles[2], n_phase;
    {
        const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
        int64_t lin = (int64_t)x * w.per_xcd + slot;
        int64_t n_units = (int64_t)w.units * b.Hkv;
        if constexpr (kBlocks == 2) {
            if (lin >= n_units) {
                lin -= n_units;
                const int per_xcd = w.per_xcd;
                b = b1;
                w = w1;
                w.per_xcd = per_xcd;
                n_units = (int64_t)w.units * b.Hkv;
            }
        }
        if (slot >= w.per_xcd || lin >= n_units)
            return;
        g = (int)(lin / w.units);
        const int u = (int)(lin % w.units);
        tiles[0] = u;
        tiles[1] = w.n_key_tiles - 1 - u;
        n_phase = (w.paired && tiles[1] != u) ? 2 : 1;
    }
    const int group = b.Hq / b.Hkv;
    const int64_t q_stride = (int64_t)b.Hq * HD, kv_stride = (int64_t)b.Hkv * HD;
    const float scale = 1.f / sqrtf((float)HD);
    const float c = kLog2e * scale;
    const int n_qt_all = (int)((b.Sq + kTileRows - 1) / kTileRows);
    const uint32_t ring = (uint32_t)(uintptr_t)(char LDS_AS *)g_kv;
    const int row_bytes = (int)(q_stride * 2);
    // this wavefront's 16-byte chunk of the tile loads: block `wave` (rows
    // 4*wave .. 4*wave+3) of every q and dout tile
    const int dma_row = wave * 4 + (lane >> 4);
    const int dma_off = dma_row * row_bytes + (((lane & 15) ^ swz(dma_row)) << 4);

    for (int ph = 0; ph < n_phase; ++ph) {
        const int64_t key_row0 = (int64_t)tiles[ph] * kKvRows;
        const int lane_key = pair * 32 + l32;               // key row within the tile
        const int keys_here = (int)min(b.Sk - key_row0, (int64_t)kKvRows);
        const bool key_ok = lane_key < keys_here;
        const bool down = ph == 0;

        // the key-side operand of this wavefront's role: K^T (role 0) or V^T
        // (role 1), key row lane_key of the tile, dims 16*sd + 8*hi + [0, 8)
        bf16x8 kv[8];
        {
            const __bf16 *src = (const __bf16 *)(role == 0 ? b.k : b.v) +
                                (key_row0 * kv_stride + g * HD + 8 * hi);
            const u32x4 *p4 = (const u32x4 *)(src + (key_ok ? lane_key : 0) * kv_stride);
#pragma unroll
            for (int sd = 0; sd < 8; ++sd) {
                u32x4 x = p4[2 * sd];
                if (!key_ok)
                    x = u32x4{0, 0, 0, 0};
                kv[sd] = __builtin_bit_cast(bf16x8, x);
            }
        }

        // query tiles that see any of the workgroup's keys
        const int64_t first_key_pos = b.k_offset + key_row0;
        int64_t q_begin = 0;
        if (b.causal)
            q_begin = min(max(first_key_pos - b.q_offset, (int64_t)0), b.Sq);
        const int qt_begin = (int)(q_begin / kTileRows);
        const int n_qt = n_qt_all - qt_begin;
        const int n_iter = n_qt > 0 ? n_qt * group : 0;     // (query tile, head) pairs
        // Phase 0 walks its query tiles from the last one down, phase 1 from
        // its first visible one up: with paired units every workgroup is then
        // at query tile (last - s) or (s - const) after s tiles, so the
        // workgroups of an XCD stream the same tiles at the same time.  The
        // heads of the KV head's group are the inner loop.

        // Step it's q and dout rows and its lse, dvec go into stage
        // it % kKvStages.  The loads walk the (query tile, head) pairs in step
        // order; the next pair to request is a cursor advanced by one per
        // call, so a request costs no division by the group size.
        // The cursor also carries the pair's element offsets into q / dout
        // and into the statistics (scalar adds per call, no 64-bit products).
        int c_it = 0, c_h = 0, c_st = 0;
        int c_q0 = down ? (n_qt_all - 1) * kTileRows : qt_begin * kTileRows;   // first row
        const int q_step = down ? -kTileRows : kTileRows;
        int64_t c_e0 = (int64_t)c_q0 * q_stride + (int64_t)g * group * HD;   // q / dout element
        int64_t c_s0 = (int64_t)g * group * b.stat_ld + c_q0;                // lse / dvec element
        const int64_t e_next_k = (int64_t)q_step * q_stride - (int64_t)(group - 1) * HD;
        const int64_t s_next_k = (int64_t)q_step - (int64_t)(group - 1) * b.stat_ld;
        const int sq32 = (int)b.Sq;
        auto issue_next = [&]() {
            if (c_it < n_iter) {
                const int rows = min(sq32 - c_q0, kTileRows);   // >= 1
                const int bytes = (rows - 1) * row_bytes + HD * 2;
                dma16(ring + kQOff + c_st * kTileBytes + wave * 1024, dma_off,
                      rsrc((const __bf16 *)b.q + c_e0, bytes));
                dma16(ring + kDOff + c_st * kTileBytes + wave * 1024, dma_off,
                      rsrc((const __bf16 *)b.dout + c_e0, bytes));
                if (wave == 0) {
                    // lse and dvec of the tile's rows (rows past Sq read as zeros)
                    const int sb = rows * 4;
                    dma4(ring + kSOff + c_st * 2 * kStatBytes, lane * 4, rsrc(b.lse + c_s0, sb));
                    dma4(ring + kSOff + c_st * 2 * kStatBytes + kStatBytes, lane * 4,
                         rsrc(b.dvec + c_s0, sb));
                }
            }
            ++c_it;
            c_st = c_st == kKvStages - 1 ? 0 : c_st + 1;
            if (++c_h == group) {
                c_h = 0;
                c_q0 += q_step;
                c_e0 += e_next_k;
                c_s0 += s_next_k;
            } else {
                c_e0 += HD;
                c_s0 += b.stat_ld;
            }
        };

        // step it: every wavefront's loads of tiles it and it + 1 have landed
        // (tile it + 2 may still be in flight), every wavefront has finished
        // step it - 1, then tile it + kKvAhead is requested into the stage of
        // tile it + kKvAhead - kKvStages = it - 2, whose last reader (role 1)
        // was in step it - 1.
        if (ph > 0)
            lds_barrier();      // the previous phase's stages are no longer read
        for (int t = 0; t < kKvAhead; ++t)
            issue_next();
        // wait until at most `k` tiles' loads of this wavefront are in flight
        // (wavefront 0 also loads the statistics)
        auto wait_tiles = [&](int k) {
            if (k >= 2) {
                if (wave == 0)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kKvLoads0));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kKvLoads));
            } else if (k == 1) {
                if (wave == 0)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kKvLoads0));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kKvLoads));
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
        };
        // The rows' lse is used in log2 units (P = exp2(S c - lse log2 e)):
        // one wavefront converts a tile's lse in LDS once, the step before
        // the softmax role reads it (tile it + 1 during step it, tile 0
        // here), instead of every softmax wavefront multiplying its 16 values
        // every step.
        auto lse_to_log2 = [&](int stage) {
            float LDS_AS *lp =
                (float LDS_AS *)((char LDS_AS *)g_kv + kSOff + stage * 2 * kStatBytes);
            lp[lane] = lp[lane] * kLog2e;
            lp[64 + lane] = -lp[64 + lane];     // dvec negated: the dP product's input
        };
        if (n_iter > 0) {
            wait_tiles(min(kKvAhead - 1, n_iter - 1));
            lds_barrier();
            if (wave == kKvPairs)
                lse_to_log2(0);
        }

        // the step loop, compiled once per role (separate register lifetimes)
        auto steps = [&](auto role_c) {
            constexpr int kRole = decltype(role_c)::value;
            // per-lane LDS bases: row fragments from the role's first operand
            // tile (q for role 0, dout for role 1), column fragments from the
            // other, stage offsets as immediates
            constexpr int kRowOff = kRole == 0 ? kQOff : kDOff;
            constexpr int kColOff = kRole == 0 ? kDOff : kQOff;
            const FragOffsets fo = frag_offsets(lane);
            int rowb[8], colb[2][4];
#pragma unroll
            for (int sd = 0; sd < 8; ++sd)
                rowb[sd] = fo.rowf[sd] + kRowOff;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    colb[x][db] = fo.col[x][db] + kColOff;
            const int statb = kSOff + (kRole == 0 ? 0 : kStatBytes) + hi * 16;
            const int pl = kPOff + pair * kPBytes + lane * 16;
            const char LDS_AS *lds = (const char LDS_AS *)g_kv;
            auto colf = [&](int so, int kh, int db) {
                const char LDS_AS *t = lds + so + kh * 16 * 256;
                const i16x4 lo = lds_tr(t, colb[0][db]);
                const i16x4 up = lds_tr(t, colb[1][db]);
                return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                               __builtin_bit_cast(bf16x4, up), 0, 1, 2, 3, 4,
                                               5, 6, 7);
            };
            f32x16 acc[4];          // dV (role 0) or dK (role 1)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = f32x16{};

            // byte offsets (uniform) of the stages of tiles it, it - 1 and
            // it + kKvAhead, advanced around the ring each step
            int so_cur = 0, so_prev = (kKvStages - 1) * kTileBytes;
            int cur_h = 0;                  // head of step it within the group
            // first query row of step it, and the key tile's first position
            // minus the query block's, clamped to 32 bits: the mask decisions
            // compare it with row offsets in [0, 2^30), so [-2^30, 2^30 + 4096]
            // keeps every decision and the clamped window below
            int cur_q0 = down ? (n_qt_all - 1) * kTileRows : qt_begin * kTileRows;
            const int dk32 = (int)min(max(first_key_pos - b.q_offset, -((int64_t)1 << 30)),
                                      ((int64_t)1 << 30) + 4096);
            for (int it = 0; n_iter > 0 && it <= n_iter; ++it) {
                // tiles it and it + 1 landed in every wavefront (tile it + 2
                // may still be in flight)
                wait_tiles(max(0, min(1, n_iter - 2 - it)));
                lds_barrier();
                const int st_cur = so_cur / kTileBytes, st_prev = so_prev / kTileBytes;
                if (kRole == 1 && wave == kKvPairs && it + 1 < n_iter)
                    lse_to_log2(st_cur == kKvStages - 1 ? 0 : st_cur + 1);
                // The next tile's loads are requested after this step's first
                // LDS reads, so that their scalar address work runs while
                // those reads are in flight.
                if constexpr (kRole == 0) {
                    if (it < n_iter) {
                        // S = Q K^T: lane holds key l32 and query rows 8*(i/4) + 4*hi + i%4;
                        // the rows' lse read with the q fragments
                        const char LDS_AS *lt = lds + st_cur * 2 * kStatBytes;
                        bf16x8 qa[8];
                        f32x4 l4s[4];
#pragma unroll
                        for (int sd = 0; sd < 8; ++sd)
                            qa[sd] = lds_b128(lds + so_cur, rowb[sd]);
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4)
                            l4s[i4] = *(const f32x4 LDS_AS *)(lt + i4 * 32 + statb);
                        issue_next();
                        __builtin_amdgcn_sched_barrier(0);
                        f32x16 sc = f32x16{};
#pragma unroll
                        for (int sd = 0; sd < 8; ++sd)
                            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[sd], kv[sd], sc, 0, 0,
                                                                         0);
                        // dout column fragments for dV, in flight during the softmax
                        bf16x8 dc[2][4];
#pragma unroll
                        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                            for (int db = 0; db < 4; ++db)
                                dc[kh][db] = colf(so_cur, kh, db);
                        __builtin_amdgcn_sched_barrier(0);
                        const bool need_mask = b.causal && dk32 + kKvRows - 1 > cur_q0;
                        // P, then to the pair's role-1 wavefront (lane to lane)
                        const char LDS_AS *pw = lds + (it & 1) * (kKvPairs * kPBytes);
                        bf16x8 pf[2];
                        // the mask compares run only on tiles that cross the diagonal
                        auto softmax = [&](auto masked_c) {
                            constexpr bool kMasked = decltype(masked_c)::value;
                            int lim = -1;
                            if constexpr (kMasked) {
                                // lane's key position minus the tile's first query position
                                const int base = min(max(dk32 - cur_q0, -1024), 1024);
                                lim = min(max(base + lane_key, -1), 64);
                            }
#pragma unroll
                            for (int i4 = 0; i4 < 4; ++i4) {
                                const f32x4 l4 = l4s[i4];
                                f32x4 p4;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int i = 4 * i4 + e;
                                    float p = __builtin_amdgcn_exp2f(
                                        __builtin_fmaf(sc[i], c, -l4[e]));
                                    if constexpr (kMasked) {
                                        const int qi = 8 * i4 + 4 * hi + e;
                                        p = qi >= lim ? p : 0.f;
                                    }
                                    p4[e] = p;
                                    pf[i >> 3][i & 7] = (__bf16)p;
                                }
                                *(f32x4 LDS_AS *)(pw + i4 * 1024 + pl) = p4;
                            }
                        };
                        if (need_mask)
                            softmax(std::true_type{});
                        else
                            softmax(std::false_type{});
                        // dV += P^T dO
#pragma unroll
                        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                            for (int db = 0; db < 4; ++db)
                                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    pf[kh], dc[kh][db], acc[db], 0, 0, 0);
                    } else {
                        issue_next();
                    }
                } else {
                    if (it > 0) {
                        // dP = dO V^T (tile it - 1), same layout as S; role 0's P
                        // and the rows' dvec read with the dout fragments
                        const char LDS_AS *pr = lds + ((it - 1) & 1) * (kKvPairs * kPBytes);
                        const char LDS_AS *vt = lds + st_prev * 2 * kStatBytes;
                        bf16x8 da[8];
                        f32x4 p4s[4], d4s[4];
                        // in the order of use: the product's accumulator input,
                        // its operands, then P, so the first product waits on
                        // five reads rather than all sixteen
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4)
                            d4s[i4] = *(const f32x4 LDS_AS *)(vt + i4 * 32 + statb);
#pragma unroll
                        for (int sd = 0; sd < 8; ++sd)
                            da[sd] = lds_b128(lds + so_prev, rowb[sd]);
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4)
                            p4s[i4] = *(const f32x4 LDS_AS *)(pr + i4 * 1024 + pl);
                        issue_next();
                        __builtin_amdgcn_sched_barrier(0);
                        // dP - dvec directly: the product's accumulator input is
                        // the rows' negated dvec (negated in LDS with the lse)
                        f32x16 dp;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            dp[i] = d4s[i >> 2][i & 3];
#pragma unroll
                        for (int sd = 0; sd < 8; ++sd)
                            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[sd], kv[sd], dp, 0, 0,
                                                                         0);
                        // q column fragments for dK, in flight during dS
                        bf16x8 qc[2][4];
#pragma unroll
                        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                            for (int db = 0; db < 4; ++db)
                                qc[kh][db] = colf(so_prev, kh, db);
                        __builtin_amdgcn_sched_barrier(0);
                        bf16x8 sf[2];
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) {
                            const f32x4 p4 = p4s[i4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int i = 4 * i4 + e;
                                sf[i >> 3][i & 7] = (__bf16)(p4[e] * dp[i]);
                            }
                        }
                        // dK += dS^T Q
#pragma unroll
                        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                            for (int db = 0; db < 4; ++db)
                                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    sf[kh], qc[kh][db], acc[db], 0, 0, 0);
                    } else {
                        issue_next();
                    }
                }
                if (++cur_h == group) {
                    cur_h = 0;
                    cur_q0 += down ? -kTileRows : kTileRows;
                }
                so_prev = so_cur;
                so_cur = so_cur == (kKvStages - 1) * kTileBytes ? 0 : so_cur + kTileBytes;
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // no tile load outlives the phase

            // epilogue: lane holds dV (role 0) or dK (role 1) at
            // [key = 8*(i/4) + 4*hi + i%4][d = 32*db + l32] of the pair's 32 keys
            // (the lane index is made opaque so that the compiler does not
            // hoist these addresses out of the step loop and keep them live)
            int eln = lane;
            __asm__ volatile("" : "+v"(eln));
            const int el32 = eln & 31, ehi = eln >> 5;
            float *dst = (kRole == 0 ? b.dv : b.dk) + (key_row0 * b.Hkv + g) * HD + el32;
            const float mul = kRole == 0 ? 1.f : scale;
            // every load before the first store, so that the loads are in
            // flight together and the stores follow without waits
            if (b.accumulate) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = pair * 32 + 8 * (i >> 2) + 4 * ehi + (i & 3);
                    const float *pk = dst + (int64_t)min(kk, keys_here - 1) * b.Hkv * HD;
#pragma unroll
                    for (int db = 0; db < 4; ++db)
                        acc[db][i] = acc[db][i] * mul + pk[db * 32];
                }
            } else {
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    acc[db] *= mul;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kk = pair * 32 + 8 * (i >> 2) + 4 * ehi + (i & 3);
                if (kk >= keys_here)
                    continue;
                float *pk = dst + (int64_t)kk * b.Hkv * HD;
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    pk[db * 32] = acc[db][i];
            }
        };
        if (role == 0) {
            // the exponentials' wavefront is the longer chain of the pair:
            // it goes first when both can issue (+1% measured)
            __builtin_amdgcn_s_setprio(1);
            steps(IC<0>{});
        } else {
            steps(IC<1>{});
        }
    }
}

KvWork kv_work(const BwdLaunch &b)
{
    KvWork w{};
    w.n_key_tiles = (int)((b.Sk + kKvRows - 1) / kKvRows);
    w.paired = b.causal && w.n_key_tiles > 1 ? 1 : 0;
    w.units = w.paired ? (w.n_key_tiles + 1) / 2 : w.n_key_tiles;
    return w;
}

}  // namespace

hipError_t launch_bwd_bf16_dq(const BwdLaunch &b, hipStream_t stream)
{
    if (b.Sq > 0) {
        DqWork w{};
        w.n_row_tiles = (int)((b.Sq + kDqRows - 1) / kDqRows);
        w.mode = (b.causal && (b.Hkv % 8 != 0 || b.Hq % 8 != 0)) ? 1 : 0;
        int64_t grid;
        if (w.mode == 0) {
            w.per_xcd = (int)(((int64_t)w.n_row_tiles * b.Hq + 7) / 8);
            grid = 8 * (int64_t)w.per_xcd;
        } else {
            w.band = (w.n_row_tiles + 15) / 16;
            grid = 8 * (int64_t)b.Hq * 2 * w.band;
        }
        hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)grid), dim3(kDqThreads), 0, stream, b,
                           w);
    }
    return hipGetLastError();
}

int64_t bwd_bf16_dkdv_units(const BwdLaunch &b)
{
    if (b.Sk <= 0)
        return 0;
    return (int64_t)kv_work(b).units * b.Hkv;
}

hipError_t launch_bwd_bf16_dkdv(const BwdLaunch *bs, int n, hipStream_t stream)
{
    if (n < 1 || n > 2)
        return hipErrorInvalidValue;
    // blocks without key rows write nothing
    const BwdLaunch *live[2];
    int nl = 0;
    for (int m = 0; m < n; ++m)
        if (bs[m].Sk > 0)
            live[nl++] = &bs[m];
    if (nl == 0)
        return hipGetLastError();
    KvWork w0 = kv_work(*live[0]);
    KvWork w1 = nl == 2 ? kv_work(*live[1]) : KvWork{};
    const int64_t total = (int64_t)w0.units * live[0]->Hkv +
                          (nl == 2 ? (int64_t)w1.units * live[1]->Hkv : 0);
    w0.per_xcd = (int)((total + 7) / 8);
    const dim3 grid((unsigned)(8 * (int64_t)w0.per_xcd));
    if (nl == 1)
        hipLaunchKernelGGL(bwd_dkdv_kernel<1>, grid, dim3(kKvThreads), 0, stream, *live[0], w0,
                           BwdLaunch{}, KvWork{});
    else
        hipLaunchKernelGGL(bwd_dkdv_kernel<2>, grid, dim3(kKvThreads), 0, stream, *live[0], w0,
                           *live[1], w1);
    return hipGetLastError();
}

hipError_t launch_bwd_bf16(const BwdLaunch &b, hipStream_t stream)
{
    const hipError_t e = launch_bwd_bf16_dq(b, stream);
    if (e != hipSuccess)
        return e;
    return launch_bwd_bf16_dkdv(&b, 1, stream);
}

}  // namespace cpattn
