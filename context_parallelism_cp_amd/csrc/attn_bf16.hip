// attn_bf16.hip -- bf16 blockwise attention with per-row log-sum-exp on
// CDNA4 matrix cores (gfx950), D = 128.
//
// Operation (handbook page "上下文并行：Ring Attention 与 Ulysses", section
// "哪些运算可以直接切", function attention()): s = q.k / sqrt(D), keys after
// the query's absolute position masked, lse = logsumexp(s), out =
// softmax(s) v.  The softmax runs in the streaming (m, l, o) form ("Sequence
// Parallel vs Context Parallel" blog, section 3.2) in base 2, with
// log2(e)/sqrt(D) folded into one fused multiply-add; lse is returned in nats.
//
// Work decomposition
//   * A workgroup of 8 wavefronts (two per SIMD) owns BM = 256 query rows of
//     one head; each wavefront owns 32 rows.  With grouped-query attention,
//     when the query heads per KV head (pack) divide 8, the workgroup owns
//     256 / pack rows of all pack heads of one KV head instead (8 / pack
//     wavefronts per head), so one K/V stream through LDS serves them all.
//     The two wavefronts of a SIMD overlap one's matrix work with the
//     other's softmax.
//   * Keys stream through LDS BN = 64 at a time in a 3-stage ring filled by
//     direct buffer->LDS 16-byte loads (no staging registers); the buffer
//     resource of a tile ends at the segment's last row, so rows past it read
//     as zeros.  K and V tiles are both stored row-major with a 16-byte-chunk
//     XOR swizzle that keeps the K reads (ds_read_b128) and the V transpose
//     reads (ds_read_b64_tr_b16) free of bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = 16 dims x
//     32 queries kept in VGPRs for the whole kernel).  In the accumulator
//     layout lane l holds 16 scores of query l%32, so row max and row sum are
//     in-lane reductions plus one exchange with lane l^32.
//   * The output is accumulated transposed, O^T += V^T P^T.  P^T's fragment
//     for a 16-key step is 8 consecutive accumulator registers of the lane,
//     converted to bf16 in place; the key order inside the step is permuted
//     identically for P and V, and the V^T fragment is two transpose reads of
//     the row-major V tile.  Each lane keeps one query, so the rescale by
//     exp2(m_old - m_new) is a per-lane scalar.
//   * Per 32-key half tile, all V fragments are requested from LDS before
//     their first use, and the K fragments one half tile ahead, so the LDS
//     latency lands during the softmax rather than in front of the MFMAs.
//   * The running max is only raised when a half tile's max exceeds it by
//     more than 2^8 (in base 2), so the 64-register rescale of O is rare; the
//     exponentials stay <= 2^8 and the final O / l is unchanged.  The
//     exponentials are taken against the running max first; the half tile's
//     max is computed only when some lane's partial sum reaches 2^8 (or the
//     row has no finite max yet), so the common path has no max at all.
//   * Half tiles strictly below the causal diagonal run without the mask;
//     half tiles crossing it (or a ragged end) compare absolute positions.
//   * Workgroups are mapped XCD-aware: the heads of a launch are spread over
//     the 8 XCDs, a head's tiles stay on its XCD(s), and every XCD walks its
//     tiles heaviest-first (most visible keys first).  With a multiple of 8
//     heads an XCD takes its heads one after another, so its CUs stream the
//     same head's K/V tiles through its L2 at the same time.
//   * The epilogue either writes (out, lse) or folds the block result into
//     the (out, lse) already stored (log-sum-exp merge, handbook section
//     "Ring Attention：KV 沿环传一圈").
#include "cp_kernels.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

namespace cpattn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int HD = 128;                 // head dimension
constexpr int BN = 64;                  // keys per LDS tile
constexpr int QB = 1;                   // 32-row query blocks per wavefront
constexpr int kWaves = 8;
constexpr int BM = kWaves * QB * 32;    // 256 query rows per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;
constexpr int kTileBytes = BN * HD * 2;             // 16 KiB per K or V tile
constexpr int kStageBytes = 2 * kTileBytes;         // K then V
constexpr float kTau = 8.0f;            // lazy-rescale threshold, log2 units
constexpr float kSumBound = 256.0f;     // 2^kTau
constexpr int kMaxOrder = 768;          // tiles of the heaviest-first table
constexpr int kXcds = 8;

struct TileMap {
    int32_t start[kMaxQSegs + 1];       // prefix sum of row tiles over the segments
    int32_t total;                      // row tiles in the launch
    int32_t use_order;                  // order[] valid (total <= kMaxOrder)
    int32_t xcd_mode;                   // 0 linear, 1 Hq % 8 == 0, 2 8 % Hq == 0, 3 bands
    int32_t band;                       // row tiles per band (xcd_mode 3)
    int32_t slots;                      // tile positions walked per XCD lane
    int32_t pack;                       // query heads per workgroup (they share one KV head)
    uint16_t order[kMaxOrder];          // tile positions, heaviest first
};

// 16-byte-chunk XOR swizzle of a 256-byte tile row.  The LDS has 64 banks of
// 4 bytes, so a 256-byte row covers every bank once; 16 lanes of a
// ds_read_b128 (16 consecutive rows, one chunk) and 32 lanes of a transpose
// read (4 consecutive rows x 4 consecutive chunks) then land in 16 distinct
// chunk slots.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Byte offset inside a tile of the 16-byte chunk c of row r.
__device__ __forceinline__ int tile_off(int r, int c) { return r * 256 + ((c ^ swz(r)) << 4); }

__device__ __forceinline__ bf16x8 lds_b128(const char LDS_AS *base, int off)
{
    return __builtin_bit_cast(bf16x8, *(const u32x4 LDS_AS *)(base + off));
}

__device__ __forceinline__ i16x4 lds_tr(const char LDS_AS *base, int off)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(base + off));
}

// max / sum of x over lanes l and l^32 (v_permlane32_swap exchanges the halves)
__device__ __forceinline__ float max_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer resource over `bytes` bytes at `p` (no stride, the default
// data format of a gfx9 descriptor).  Loads through it whose offset lies past
// `bytes` are dropped by the address unit and return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes,
                                             0x00020000);
}

constexpr int kLoadsPerLane = 16 / kWaves;  // 1 KiB blocks of a tile filled per wave

// Issue the direct-to-LDS loads of one K tile and one V tile (the `rows`
// rows at kbase and vbase, rows <= 64, row_bytes apart) into `stage`.  The
// buffer resources end after the last row, so the chunks of rows past it
// read as zeros (their scores are masked).  The tile's address arithmetic
// is uniform (scalar unit); a lane adds only its fixed offset off[i]: the
// chunk it copies sits in row blk*4 + lane/16 of the tile and lands in the
// LDS slot the swizzle gives it.
__device__ __forceinline__ void load_tile(char LDS_AS *stage, const __bf16 *kbase,
                                          const __bf16 *vbase, int row_bytes, int rows,
                                          const int (&off)[kLoadsPerLane], int wave)
{
    const int bytes = (rows - 1) * row_bytes + HD * 2;
    const auto rk = buffer_rsrc(kbase, bytes);
    const auto rv = buffer_rsrc(vbase, bytes);
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
        const int blk = wave * kLoadsPerLane + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (void LDS_AS *)(stage + blk * 1024), 16,
                                                 off[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (void LDS_AS *)(stage + kTileBytes + blk * 1024), 16, off[i], 0, 0, 0);
    }
}

struct TileRef {
    int seg;          // KV segment index
    int64_t key0;     // first key of the tile within the segment
};

// The three pipeline stages are distinct LDS objects, and every access names
// its stage at compile time: the compiler then sees that the loads landing
// in one stage cannot alias reads of another and does not wait for them.
__shared__ __attribute__((aligned(1024))) char g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_stage2[kStageBytes];

template <int ST>
__device__ __forceinline__ char LDS_AS *stage_base()
{
    if constexpr (ST == 0)
        return (char LDS_AS *)g_stage0;
    else if constexpr (ST == 1)
        return (char LDS_AS *)g_stage1;
    else
        return (char LDS_AS *)g_stage2;
}

// One workgroup per CU (its LDS ring fills most of the CU's LDS), i.e. two
// wavefronts per SIMD: telling the compiler lets its scheduler spend up to
// 256 VGPRs on reading LDS fragments ahead of the MFMAs instead of
// minimising registers for an occupancy the LDS cannot give.
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(AttnLaunch a, TileMap tm, float scale_log2)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // ---- which (head group, row tile) this workgroup owns.  A head group is
    // `pack` consecutive query heads sharing one KV head; each head gets
    // kWaves / pack wavefronts, i.e. bm = 32 * kWaves / pack rows.
    const int pack = tm.pack;
    const int wph = kWaves / pack;                 // wavefronts per query head
    const int bm = 32 * wph;                       // rows per workgroup
    const int n_hg = a.Hq / pack;
    int hg, tp;
    {
        const int bid = blockIdx.x;
        if (tm.xcd_mode == 1) {
            const int x = bid % kXcds, s = bid / kXcds;
            hg = x + kXcds * (s / tm.total);
            tp = s % tm.total;
        } else if (tm.xcd_mode == 2) {
            const int x = bid % kXcds, s = bid / kXcds;
            const int xph = kXcds / n_hg;
            hg = x % n_hg;
            tp = s * xph + x / n_hg;
        } else if (tm.xcd_mode == 3) {
            // one causal segment: its row tiles cut into 2 * xph bands whose
            // sizes differ by one at most; XCD lane j of the head group takes
            // band 2*xph-1-j, then band j, each from its last row tile down
            // (equal work per XCD; the workgroups an XCD holds at a time are
            // neighbouring row tiles that stream the same keys at about the
            // same time)
            const int x = bid % kXcds, s = bid / kXcds;
            const int xph = kXcds / n_hg;
            const int nb = 2 * xph;                    // band k: [k*T/nb, (k+1)*T/nb)
            const int j = x / n_hg;
            hg = x % n_hg;
            const int kh = nb - 1 - j;
            const int h0 = (int)((int64_t)kh * tm.total / nb);
            const int sh = (int)((int64_t)(kh + 1) * tm.total / nb) - h0;
            const int l0 = (int)((int64_t)j * tm.total / nb);
            const int sl = (int)((int64_t)(j + 1) * tm.total / nb) - l0;
            tp = s < sh ? h0 + (sh - 1 - s) : (s - sh < sl ? l0 + (sl - 1 - (s - sh)) : tm.total);
        } else {
            hg = bid / tm.total;
            tp = bid % tm.total;
        }
        if (hg >= n_hg || tp >= tm.total)
            return;
    }
    const int h = hg * pack + wave / wph;          // this wavefront's query head
    int tile_lin;
    if (tm.use_order) {
        tile_lin = tm.order[tp];
    } else {
        tile_lin = tp;
    }
    int s = 0;
    while (s + 1 < a.n_q && tile_lin >= tm.start[s + 1])
        ++s;
    const QSeg &qs = a.qs[s];
    int tile = tile_lin - tm.start[s];
    if (!tm.use_order && a.causal && tm.xcd_mode != 3)   // without the table: later rows first
        tile = (tm.start[s + 1] - tm.start[s]) - 1 - tile;
    const int64_t tile_row0 = (int64_t)tile * bm;
    const int g = h / (a.Hq / a.Hkv);              // the same for every wavefront

    const __bf16 *qg = (const __bf16 *)a.q;
    const int64_t q_stride = (int64_t)a.Hq * HD;
    const int64_t kv_stride = (int64_t)a.Hkv * HD;
    const __bf16 *kg = (const __bf16 *)a.k + g * HD;
    const __bf16 *vg = (const __bf16 *)a.v + g * HD;

    // ---- rows of this wavefront: block qb holds tile rows row_off[qb] =
    // wave*32*QB + qb*32 + [0, 32)
    int row_off[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
        row_off[qb] = (wave % wph) * 32 * QB + qb * 32 + l32;

    // Q^T fragments: B operand of step sd holds dims 16*sd + 8*hi + [0, 8).
    bf16x8 qf[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const bool ok = tile_row0 + row_off[qb] < qs.len;
        const int64_t r = ok ? tile_row0 + row_off[qb] : 0;
        const u32x4 *src = (const u32x4 *)(qg + (qs.row0 + r) * q_stride + h * HD + 8 * hi);
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
            u32x4 x = src[2 * sd];
            if (!ok)
                x = u32x4{0, 0, 0, 0};
            qf[qb][sd] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- the tile stream: every KV segment's tiles up to the causal bound
    const int64_t first_pos = qs.pos0 + tile_row0;
    const int64_t last_pos = qs.pos0 + min(tile_row0 + bm, qs.len) - 1;
    int seg_tiles[2] = {0, 0};
    for (int kv_i = 0; kv_i < qs.n_kv; ++kv_i) {
        const KvSeg &kv = qs.kv[kv_i];
        int64_t n_keys = kv.len;
        if (a.causal)
            n_keys = min(max(last_pos - kv.pos0 + 1, (int64_t)0), kv.len);
        seg_tiles[kv_i] = (int)((n_keys + BN - 1) / BN);
    }
    const int n_tiles = seg_tiles[0] + seg_tiles[1];
    // Per segment, 32-bit bounds for the mask decisions (segments are
    // shorter than 2^30 keys): key k of the segment is past its end iff
    // k >= seg_len, and the workgroup's row at offset r sees k iff
    // k <= seg_diag + r.  seg_diag is first_pos - pos0 clamped to
    // [-512, len + 64], which changes no decision: rows are fewer than 512
    // and no tile reaches past len.
    int seg_len[2] = {0, 0}, seg_diag[2] = {0, 0};
#pragma unroll
    for (int kv_i = 0; kv_i < 2; ++kv_i) {
        if (kv_i < qs.n_kv) {
            const KvSeg &kv = qs.kv[kv_i];
            seg_len[kv_i] = __builtin_amdgcn_readfirstlane((int)kv.len);
            seg_diag[kv_i] = __builtin_amdgcn_readfirstlane(
                (int)min(max(first_pos - kv.pos0, (int64_t)-512), kv.len + 64));
        }
    }

    auto tile_ref = [&](int t) {
        TileRef r;
        r.seg = t < seg_tiles[0] ? 0 : 1;
        r.key0 = (int64_t)(r.seg == 0 ? t : t - seg_tiles[0]) * BN;
        return r;
    };
    // Each lane's byte offsets into a tile for its share of the loads (the
    // same for every tile, kept in registers across the loop).
    const int row_bytes = (int)(kv_stride * 2);
    int dma_off[kLoadsPerLane];
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
        const int rr = (wave * kLoadsPerLane + i) * 4 + (lane >> 4);
        dma_off[i] = rr * row_bytes + (((lane & 15) ^ swz(rr)) << 4);
    }
    // loads of tile t into stage ST (ST == t % 3)
    auto issue = [&](int t, auto st) {
        if (t < n_tiles) {
            const TileRef r = tile_ref(t);
            const KvSeg &kv = qs.kv[r.seg];
            const int rows = min((r.seg == 0 ? seg_len[0] : seg_len[1]) - (int)r.key0, BN);
            const int64_t e0 = (kv.row0 + r.key0) * kv_stride;
            load_tile(stage_base<decltype(st)::value>(), kg + e0, vg + e0, row_bytes, rows,
                      dma_off, wave);
        }
    };

    f32x16 o_acc[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o_acc[qb][i] = f32x16{};
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }

    // S^T = K Q^T for sub-tile u (32 keys: half u%2 of LDS tile u/2): sc[qb].
    // per-lane byte offsets of the K fragments inside a 32-row half tile
    // (rows l32 and 32 + l32 share a swizzle: it depends on row % 16)
    int k_off[8];
#pragma unroll
    for (int sd = 0; sd < 8; ++sd)
        k_off[sd] = tile_off(l32, 2 * sd + hi);
    // K fragments of the next half tile to be scored.  They are requested
    // one half tile ahead, right after the V fragments, so they land while
    // the softmax runs instead of stalling the score MFMAs: for the first
    // half of a tile from the same tile, for the second half from the next
    // tile, whose loads every wavefront waited for before this tile's
    // barrier (its stage is overwritten only after the next tile's one).
    bf16x8 kf[8];
    auto load_k = [&](const char LDS_AS *kt) {
#pragma unroll
        for (int sd = 0; sd < 8; ++sd)
            kf[sd] = lds_b128(kt, k_off[sd]);
    };
    // S^T of the half tile whose K fragments are in kf
    auto scores = [&](f32x16 (&sc)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            sc[qb] = f32x16{};
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sd], qf[qb][sd], sc[qb], 0,
                                                                 0, 0);
        }
    };

    // V^T fragment for 16-key step ks of a tile and 32-dim block db (two
    // transpose reads; see the key order in the header comment).
    const int grp = lane >> 4;          // 16-lane group
    const int gi = lane & 15;
    // rows 16*ks + r0 share swz(r0) because swz depends on row % 16; the
    // second read (rows r0 + 8) has its own offsets
    int v_off[2][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const int dcol = db * 32 + 16 * (grp & 1) + 4 * (gi & 3);   // first of 4 columns
        const int r0 = 4 * (grp >> 1) + (gi >> 2);
        v_off[0][db] = tile_off(r0, dcol >> 3) + (dcol & 7) * 2;
        v_off[1][db] = tile_off(r0 + 8, dcol >> 3) + (dcol & 7) * 2;
    }
    auto v_frag = [&](const char LDS_AS *vt, int ks, int db) {
        const i16x4 lo = lds_tr(vt, ks * 16 * 256 + v_off[0][db]);
        const i16x4 up = lds_tr(vt, ks * 16 * 256 + v_off[1][db]);
        const bf16x4 blo = __builtin_bit_cast(bf16x4, lo);
        const bf16x4 bup = __builtin_bit_cast(bf16x4, up);
        return __builtin_shufflevector(blo, bup, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // One 64-key tile in stage ST: for each 32-key half, scores, masking and
    // running max, exponentials, then O^T += V^T P^T.
    auto tile_step = [&](int t, auto st) {
        constexpr int ST = decltype(st)::value;
        // tile t complete in every wavefront; the stage the new loads overwrite
        // (tile t-1's) is no longer read
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue(t + 2, std::integral_constant<int, (ST + 2) % 3>{});
        const TileRef r = tile_ref(t);
        int len_c = r.seg == 0 ? seg_len[0] : seg_len[1];
        int diag_c = r.seg == 0 ? seg_diag[0] : seg_diag[1];
        __asm__ volatile("" : "+s"(len_c), "+s"(diag_c));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x16 cur[QB];
            scores(cur);
            // V fragments of this half tile and K fragments of the next one,
            // requested now: they land while the softmax runs
            const char LDS_AS *vt = stage_base<ST>() + kTileBytes;
            bf16x8 vfr[2][4];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    vfr[kh][db] = v_frag(vt, 2 * half + kh, db);
            if (half == 0)
                load_k(stage_base<ST>() + 32 * 256);
            else if (t + 1 < n_tiles)
                load_k(stage_base<(ST + 1) % 3>());
            __builtin_amdgcn_sched_barrier(0);
            const int key0 = (int)r.key0 + half * 32;     // first key of the half tile
            const bool need_mask = (key0 + 32 > len_c) || (a.causal && key0 + 31 > diag_c);
            if (need_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    // key k of the half tile (0..31) is visible iff k <= lim
                    const int tail = min(max(len_c - 1 - key0, -1), 64);
                    const int base_c = min(max(diag_c - key0, -512), 512);
                    const int lim = a.causal ? min(tail, base_c + row_off[qb]) : tail;
                    const int lim_l = max(lim, -1) - 4 * hi;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        // this register holds key 8*(i/4) + 4*hi + i%4
                        const int kc = 8 * (i >> 2) + (i & 3);
                        cur[qb][i] = kc > lim_l ? -INFINITY : cur[qb][i];
                    }
                }
            }
            // Exponentials against the running max as it stands.  They are
            // kept when every lane's partial sum stays below 2^kTau: then
            // every exponential does, i.e. no score exceeds the running max
            // by kTau and the max would not have been raised.  Otherwise
            // the wavefront takes the exact path: half-tile max, lazy raise,
            // rescale, exponentials again.
            bf16x8 pf[QB][2];
            float rs[QB], rs2[QB][2];
            auto exps = [&](bool first) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    // A row without a finite running max yet gives +inf or NaN
                    // exponentials on the first pass (-m_run = +inf), which
                    // fails the sum test below; the exact pass uses 0 instead.
                    const float m_use =
                        first ? m_run[qb] : (m_run[qb] == -INFINITY ? 0.f : m_run[qb]);
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float p = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(cur[qb][8 * kh + j], scale_log2, -m_use));
                            // two interleaved partial sums (keys of even / odd j)
                            if (kh == 0 && j < 2)
                                rs2[qb][j] = p;
                            else
                                rs2[qb][j & 1] += p;
                            pf[qb][kh][j] = (__bf16)p;
                        }
                    rs[qb] = rs2[qb][0] + rs2[qb][1];
                }
            };
            exps(true);
            bool exact = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                exact |= !(rs[qb] < kSumBound);   // also true for NaN
            if (__any(exact)) {
                float alpha[QB];
                bool any_rescale = false;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        mx = fmaxf(mx, cur[qb][i]);
                    mx = max_xor32(mx) * scale_log2;
                    const bool up = mx > m_run[qb] + kTau;
                    any_rescale |= up;
                    const float m_new = up ? mx : m_run[qb];
                    alpha[qb] = up ? __builtin_amdgcn_exp2f(m_run[qb] - m_new) : 1.f;
                    m_run[qb] = m_new;
                }
                if (__any(any_rescale)) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        l_run[qb] *= alpha[qb];
#pragma unroll
                        for (int db = 0; db < 4; ++db)
                            o_acc[qb][db] *= alpha[qb];
                    }
                }
                exps(false);
            }
            // each lane keeps its own partial row sum; the two halves of a
            // row are added in the epilogue
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                l_run[qb] += rs[qb];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o_acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            vfr[kh][db], pf[qb][kh], o_acc[qb][db], 0, 0, 0);
                }
        }
    };

    // ---- tiles 0 and 1 in flight before the loop; tile t uses stage t % 3
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    issue(0, I0{});
    issue(1, I1{});
    // the first half tile's K fragments (the loop's barriers then keep one
    // half tile ahead)
    if (n_tiles > 0) {
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_k(stage_base<0>());
    }
    for (int t = 0; t < n_tiles; t += 3) {
        tile_step(t, I0{});
        if (t + 1 >= n_tiles)
            break;
        tile_step(t + 1, I1{});
        if (t + 2 >= n_tiles)
            break;
        tile_step(t + 2, I2{});
    }

    // ---- epilogue: lane l holds O^T[d = 32*db + 8*(i/4) + 4*hi + i%4][row l32]
    const float kLn2 = 0.6931471805599453f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        // lanes l and l ^ 32 hold partial sums of the same row
        const float l = sum_xor32(l_run[qb]);
        const int64_t my_row = tile_row0 + row_off[qb];
        if (my_row >= qs.len)
            continue;
        const int64_t orow = qs.out_row0 + my_row;
        float *out = a.out + (orow * a.Hq + h) * HD;
        float *lse_p = a.lse + (int64_t)h * a.lse_ld + orow;
        const float lse_blk = l > 0.f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
        const float inv_l = l > 0.f ? 1.f / l : 0.f;
        if (!qs.merge) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    f32x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v4[e] = o_acc[qb][db][4 * i4 + e] * inv_l;
                    *(f32x4 *)(out + db * 32 + 8 * i4 + 4 * hi) = v4;
                }
            if (hi == 0)
                *lse_p = lse_blk;
            continue;
        }
        const float lse_old = *lse_p;
        const float mxl = fmaxf(lse_old, lse_blk);
        if (mxl == -INFINITY)
            continue;
        const float lse_new = mxl + log1pf(expf(-fabsf(lse_old - lse_blk)));
        const float w_old = expf(lse_old - lse_new);
        const float w_blk = expf(lse_blk - lse_new) * inv_l;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 *dst = (f32x4 *)(out + db * 32 + 8 * i4 + 4 * hi);
                const f32x4 old = *dst;
                f32x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v4[e] = old[e] * w_old + o_acc[qb][db][4 * i4 + e] * w_blk;
                *dst = v4;
            }
        // both halves of the wavefront read lse_old above before this store
        if (hi == 0)
            *lse_p = lse_new;
    }
}

// Visible keys of the last row of row tile `tile` (bm rows) of segment `s`.
int64_t tile_work(const AttnLaunch &a, int s, int tile, int bm)
{
    const QSeg &q = a.qs[s];
    const int64_t last = q.pos0 + std::min<int64_t>((int64_t)(tile + 1) * bm, q.len) - 1;
    int64_t w = 0;
    for (int k = 0; k < q.n_kv; ++k) {
        const KvSeg &kv = q.kv[k];
        w += a.causal ? std::min(std::max<int64_t>(last - kv.pos0 + 1, 0), kv.len) : kv.len;
    }
    return w;
}

}  // namespace

// The launch arguments travel in the kernel-argument segment (4 KiB).
static_assert(sizeof(AttnLaunch) + sizeof(TileMap) + sizeof(float) <= 4096,
              "attention kernel arguments exceed the kernel-argument segment");

hipError_t launch_attn_bf16(const AttnLaunch &a, hipStream_t stream)
{
    TileMap tm{};
    // Query heads that share a KV head go into one workgroup when their
    // number divides the wavefront count: the K/V tiles in LDS then serve
    // all of them (one L2 stream instead of one per query head).
    const int group = a.Hkv > 0 ? a.Hq / a.Hkv : 1;
    tm.pack = (group >= 1 && group <= kWaves && kWaves % group == 0) ? group : 1;
    const int bm = BM / tm.pack;
    const int n_hg = a.Hq / tm.pack;
    int64_t total = 0;
    for (int s = 0; s < a.n_q; ++s) {
        tm.start[s] = (int32_t)total;
        total += (a.qs[s].len + bm - 1) / bm;
    }
    tm.start[a.n_q] = (int32_t)total;
    if (total == 0 || n_hg == 0)
        return hipSuccess;
    tm.total = (int32_t)total;
    tm.use_order = total <= kMaxOrder ? 1 : 0;
    if (tm.use_order) {
        // heaviest first; ties keep later rows first
        std::vector<std::pair<int64_t, int>> w;
        w.reserve(total);
        for (int s = 0; s < a.n_q; ++s)
            for (int t = tm.start[s]; t < tm.start[s + 1]; ++t)
                w.push_back({-tile_work(a, s, t - tm.start[s], bm), -t});
        std::sort(w.begin(), w.end());
        for (int64_t i = 0; i < total; ++i)
            tm.order[i] = (uint16_t)(-w[i].second);
    }
    int64_t grid;
    if (n_hg % kXcds == 0) {
        tm.xcd_mode = 1;
        grid = total * n_hg;
    } else if (kXcds % n_hg == 0 && !tm.use_order && a.causal && a.n_q == 1) {
        tm.xcd_mode = 3;
        const int bands = 2 * (kXcds / n_hg);
        tm.band = (int32_t)((total + bands - 1) / bands);   // largest band
        grid = (int64_t)kXcds * 2 * tm.band;
    } else if (kXcds % n_hg == 0) {
        tm.xcd_mode = 2;
        const int xph = kXcds / n_hg;
        const int64_t slots = (total + xph - 1) / xph;
        grid = slots * kXcds;
    } else {
        tm.xcd_mode = 0;
        grid = total * n_hg;
    }
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
    hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, tm,
                       scale_log2);
    return hipGetLastError();
}

}  // namespace cpattn
