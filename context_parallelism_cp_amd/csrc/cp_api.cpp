// cp_api.cpp -- host side of libcpattn.so: argument validation, the ring
// planner, the Ulysses repack offsets, kernel launches and kernel timing.
// The public contract is include/cp_attn.h.
//
// Ring schedule (handbook page "上下文并行：Ring Attention 与 Ulysses",
// section "Ring Attention：KV 沿环传一圈"): at step t rank r holds the KV block
// of rank src = (r - t) mod P.  The zigzag split ("之字形切分") gives rank r
// chunks r and 2P-1-r of a 2P-way split; a (query chunk, key chunk) pair is
// skipped when the key chunk comes after the query chunk, masked when they
// are the same chunk and computed in full otherwise.  One kernel launch per
// ring step covers every query chunk of every rank that step touches (ranks
// are independent), each query chunk attending to the key chunks of its step
// in one pass; the log-sum-exp merge into the running result is fused into
// the kernel epilogue.
#include "../../include/cp_attn.h"
#include "cp_kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <limits>
#include <vector>

using namespace cpattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return CP_OK;
}

bool aligned(const void *p, size_t n) { return ((uintptr_t)p) % n == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0)
        return false;
    const char *x = (const char *)a;
    const char *y = (const char *)b;
    return x < y + nb && y < x + na;
}

// ------------------------------------------------------------------ timing
constexpr int kKernelKinds = 7;   // cp_kernel_kind values

struct Timing {
    std::mutex mu;
    bool enabled = false;
    struct Rec {
        int kind;
        hipEvent_t start, stop;
    };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> pool;
    double total_ms[kKernelKinds] = {};
    int64_t launches[kKernelKinds] = {};
};

Timing &timing()
{
    static Timing t;
    return t;
}

hipEvent_t take_event(Timing &t)
{
    if (!t.pool.empty()) {
        hipEvent_t e = t.pool.back();
        t.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

// Launch `fn` on `stream`, bracketed by events when timing is enabled.
template <typename F>
int timed_launch(int kind, hipStream_t stream, F &&fn)
{
    Timing &t = timing();
    std::unique_lock<std::mutex> lock(t.mu, std::defer_lock);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (t.enabled) {
        lock.lock();
        e0 = take_event(t);
        e1 = take_event(t);
        if (!e0 || !e1)
            return fail(CP_ERR_HIP, "hipEventCreate failed");
        if (hipEventRecord(e0, stream) != hipSuccess)
            return fail(CP_ERR_HIP, "hipEventRecord failed");
    }
    const hipError_t err = fn();
    if (err != hipSuccess)
        return fail(CP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    if (e0) {
        if (hipEventRecord(e1, stream) != hipSuccess)
            return fail(CP_ERR_HIP, "hipEventRecord failed");
        t.pending.push_back({kind, e0, e1});
    }
    return CP_OK;
}

// ------------------------------------------------------------- validation
int check_attn_common(const void *q, const void *k, const void *v, const float *out,
                      const float *lse, int64_t Sq, int64_t Sk, int Hq, int Hkv, int D,
                      cp_dtype dtype)
{
    // a pointer may be NULL only when its tensor is empty
    if ((Sq > 0 && (!q || !out || !lse)) || (Sk > 0 && (!k || !v)))
        return fail(CP_ERR_NULL, "q, k, v, out and lse must be non-NULL");
    if (Sq < 0 || Sk < 0)
        return fail(CP_ERR_SHAPE, "negative sequence length (Sq=%lld, Sk=%lld)",
                    (long long)Sq, (long long)Sk);
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(CP_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and Hkv dividing Hq (Hq=%d, Hkv=%d)",
                    Hq, Hkv);
    if (dtype == CP_BF16) {
        if (D != 128)
            return fail(CP_ERR_UNSUPPORTED, "bf16 attention supports D = 128 only (D=%d)", D);
        // a 64-row K or V tile is addressed with 32-bit byte offsets
        if ((int64_t)Hkv * D >= ((int64_t)1 << 24))
            return fail(CP_ERR_UNSUPPORTED, "bf16 attention needs Hkv * D < 2^24 (Hkv=%d)", Hkv);
        // the kernel takes its mask decisions on 32-bit in-segment key indices
        if (Sq >= ((int64_t)1 << 30) || Sk >= ((int64_t)1 << 30))
            return fail(CP_ERR_UNSUPPORTED, "bf16 attention needs Sq, Sk < 2^30 (Sq=%lld, Sk=%lld)",
                        (long long)Sq, (long long)Sk);
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
            return fail(CP_ERR_ALIGN, "bf16 attention needs 16-byte aligned q, k, v and out");
    } else if (dtype == CP_F32) {
        if (D < 1 || D > 128)
            return fail(CP_ERR_UNSUPPORTED, "float32 attention supports 1 <= D <= 128 (D=%d)", D);
        if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(out, 4))
            return fail(CP_ERR_ALIGN, "float32 attention needs 4-byte aligned pointers");
    } else {
        return fail(CP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    }
    if (!aligned(lse, 4))
        return fail(CP_ERR_ALIGN, "lse must be 4-byte aligned");
    const size_t eb = dtype == CP_BF16 ? 2 : 4;
    const size_t qb = (size_t)Sq * Hq * D * eb, kb = (size_t)Sk * Hkv * D * eb;
    const size_t ob = (size_t)Sq * Hq * D * 4, lb = (size_t)Sq * Hq * 4;
    if (overlaps(q, qb, out, ob) || overlaps(k, kb, out, ob) || overlaps(v, kb, out, ob) ||
        overlaps(q, qb, lse, lb) || overlaps(k, kb, lse, lb) || overlaps(v, kb, lse, lb) ||
        overlaps(out, ob, lse, lb))
        return fail(CP_ERR_ALIGN, "q, k, v, out and lse must not overlap");
    return CP_OK;
}

int launch_attn(const AttnLaunch &a, cp_dtype dtype, hipStream_t stream)
{
    if (dtype == CP_BF16)
        return timed_launch(CP_KERNEL_ATTN_BF16, stream, [&] { return launch_attn_bf16(a, stream); });
    return timed_launch(CP_KERNEL_ATTN_F32, stream, [&] { return launch_attn_f32(a, stream); });
}

// ---------------------------------------------------------------- backward
int check_bwd(const void *q, const void *k, const void *v, const void *dout, const float *lse,
              const float *dvec, const float *dq, const float *dk, const float *dv, int64_t Sq,
              int64_t Sk, int Hq, int Hkv, int D, cp_dtype dtype)
{
    if ((Sq > 0 && (!q || !dout || !lse || !dvec || !dq)) || (Sk > 0 && (!k || !v || !dk || !dv)))
        return fail(CP_ERR_NULL, "q, k, v, dout, lse, dvec, dq, dk and dv must be non-NULL");
    if (Sq < 0 || Sk < 0)
        return fail(CP_ERR_SHAPE, "negative sequence length (Sq=%lld, Sk=%lld)",
                    (long long)Sq, (long long)Sk);
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(CP_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and Hkv dividing Hq (Hq=%d, Hkv=%d)",
                    Hq, Hkv);
    if (dtype == CP_BF16) {
        if (D != 128)
            return fail(CP_ERR_UNSUPPORTED, "bf16 backward supports D = 128 only (D=%d)", D);
        if ((int64_t)Hkv * D >= ((int64_t)1 << 24))
            return fail(CP_ERR_UNSUPPORTED, "bf16 backward needs Hkv * D < 2^24 (Hkv=%d)", Hkv);
        // the kernels take their mask decisions on 32-bit key indices
        if (Sq >= ((int64_t)1 << 30) || Sk >= ((int64_t)1 << 30))
            return fail(CP_ERR_UNSUPPORTED, "bf16 backward needs Sq, Sk < 2^30 (Sq=%lld, Sk=%lld)",
                        (long long)Sq, (long long)Sk);
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
            !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
            return fail(CP_ERR_ALIGN, "bf16 backward needs 16-byte aligned tensors");
    } else if (dtype == CP_F32) {
        if (D < 1 || D > 128)
            return fail(CP_ERR_UNSUPPORTED, "float32 backward supports 1 <= D <= 128 (D=%d)", D);
        if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(dout, 4) ||
            !aligned(dq, 4) || !aligned(dk, 4) || !aligned(dv, 4))
            return fail(CP_ERR_ALIGN, "float32 backward needs 4-byte aligned pointers");
    } else {
        return fail(CP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    }
    if (!aligned(lse, 4) || !aligned(dvec, 4))
        return fail(CP_ERR_ALIGN, "lse and dvec must be 4-byte aligned");
    const size_t eb = dtype == CP_BF16 ? 2 : 4;
    const size_t qb = (size_t)Sq * Hq * D * eb, kb = (size_t)Sk * Hkv * D * eb;
    const size_t gqb = (size_t)Sq * Hq * D * 4, gkb = (size_t)Sk * Hkv * D * 4;
    const size_t sb = (size_t)Sq * Hq * 4;
    const void *ins[6] = {q, k, v, dout, lse, dvec};
    const size_t in_b[6] = {qb, kb, kb, qb, sb, sb};
    const void *outs[3] = {dq, dk, dv};
    const size_t out_b[3] = {gqb, gkb, gkb};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(outs[o], out_b[o], ins[i], in_b[i]))
                return fail(CP_ERR_ALIGN, "gradient buffers must not overlap the inputs");
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (overlaps(outs[o], out_b[o], outs[o2], out_b[o2]))
                return fail(CP_ERR_ALIGN, "dq, dk and dv must not overlap");
    }
    return CP_OK;
}

int launch_bwd(const BwdLaunch &b, cp_dtype dtype, hipStream_t stream)
{
    if (dtype == CP_BF16)
        return timed_launch(CP_KERNEL_BWD_BF16, stream, [&] { return launch_bwd_bf16(b, stream); });
    return timed_launch(CP_KERNEL_BWD_F32, stream, [&] { return launch_bwd_f32(b, stream); });
}

int fill_zero(float *p, int64_t n, hipStream_t stream)
{
    const hipError_t e = launch_fill_zero(p, n, stream);
    return e == hipSuccess ? CP_OK : fail(CP_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
}

// Output rows [row0, row0 + n) of out [rows][H][D] and lse [H][rows] (ld =
// rows) set to the padding value (0, -inf).
int fill_pad_rows(float *out, float *lse, int64_t rows, int H, int D, int64_t row0, int64_t n,
                  hipStream_t st)
{
    hipError_t e = launch_fill_2d(out + (size_t)row0 * H * D, 0, 1, n * H * D, 0.f, st);
    if (e == hipSuccess)
        e = launch_fill_2d(lse + row0, rows, H, n, -std::numeric_limits<float>::infinity(), st);
    return e == hipSuccess ? CP_OK : fail(CP_ERR_HIP, "fill launch failed: %s", hipGetErrorString(e));
}

// ------------------------------------------------------------ ring helpers
int check_ring_shape(int64_t S, int P, cp_layout layout, int rank)
{
    if (P < 1)
        return fail(CP_ERR_SHAPE, "P must be >= 1 (P=%d)", P);
    if (rank < -1 || rank >= P)
        return fail(CP_ERR_SHAPE, "rank must be -1 or in [0, P) (rank=%d, P=%d)", rank, P);
    if (S < 0)
        return fail(CP_ERR_SHAPE, "negative sequence length");
    if (layout != CP_LAYOUT_CONTIGUOUS && layout != CP_LAYOUT_ZIGZAG &&
        layout != CP_LAYOUT_STRIPED)
        return fail(CP_ERR_SHAPE, "unknown layout %d", (int)layout);
    if (S > ((int64_t)1 << 40))
        return fail(CP_ERR_SHAPE, "sequence too long");
    return CP_OK;
}

// Length of the padded sequence: S rounded up to a multiple of the split
// (P chunks; 2P for zigzag).  Positions >= S are padding: never read,
// never visible as keys, and their output rows are written as (0, -inf).
int64_t padded_len(int64_t S, int P, cp_layout layout)
{
    const int64_t m = layout == CP_LAYOUT_ZIGZAG ? 2 * (int64_t)P : P;
    return (S + m - 1) / m * m;
}

// Rows of the q / k / v tensors: the real length in natural order, the
// padded length in striped order (every shard has S_pad / P rows).
int64_t input_rows(int64_t S, int P, cp_layout layout)
{
    return layout == CP_LAYOUT_STRIPED ? padded_len(S, P, layout) : S;
}

int pair_kind(int causal, int qc, int kc)
{
    if (!causal || kc < qc)
        return CP_PAIR_FULL;
    return kc == qc ? CP_PAIR_DIAG : CP_PAIR_SKIP;
}

// Query chunks a rank holds (its local slots).
int n_slots(cp_layout layout) { return layout == CP_LAYOUT_ZIGZAG ? 2 : 1; }

// One (query chunk, key chunk) pair of a ring step: where its rows sit in the
// q / k tensors, how many of them are real, and the positions the causal
// mask compares.
struct RingPair {
    int slot;            // local query slot of the rank
    int qc, kc;          // chunk ids (striped: the rank ids)
    int64_t q_row, k_row;
    int64_t cap;         // rows of a chunk in the padded split
    int64_t len_q, len_k;  // real rows of the query and key chunk
    int64_t q_pos, k_pos;
    int kind;
};

int64_t clip_rows(int64_t S, int64_t row0, int64_t cap)
{
    return std::min(std::max<int64_t>(S - row0, 0), cap);
}

// Striped: rank r's real rows, positions r + jP < S for j < cap.
int64_t striped_rows(int64_t S, int P, int r, int64_t cap)
{
    return S > r ? std::min<int64_t>(cap, (S - r + P - 1) / P) : 0;
}

// The pairs of rank r at the step where it holds rank src's KV block, in
// order query slot, then key chunk, for the real length S (split as the
// padded length; a pair with no real query or key row is SKIP).
//  contiguous / zigzag: chunks of C rows at their natural positions, the
//    tensors in natural order;
//  striped: rank r's local row j is position r + jP, the tensors are the
//    ranks' shards back to back; key j of rank src is visible to query i
//    iff src + jP <= r + iP, i.e. j <= i when src <= r and j <= i - 1 when
//    src > r -- the plain causal mask with local positions q_pos = 0 and
//    k_pos = (src > r).
int ring_step_pairs(cp_layout layout, int64_t S, int P, int r, int src, int causal,
                    RingPair out[4])
{
    const int64_t Sp = padded_len(S, P, layout);
    int n = 0;
    if (layout == CP_LAYOUT_STRIPED) {
        const int64_t C = Sp / P;
        out[n++] = RingPair{0, r, src, (int64_t)r * C, (int64_t)src * C, C,
                            striped_rows(S, P, r, C), striped_rows(S, P, src, C), 0,
                            src > r ? 1 : 0, causal ? CP_PAIR_DIAG : CP_PAIR_FULL};
    } else if (layout == CP_LAYOUT_CONTIGUOUS) {
        const int64_t C = Sp / P;
        out[n++] = RingPair{0, r, src, r * C, src * C, C, clip_rows(S, r * C, C),
                            clip_rows(S, src * C, C), r * C, src * C, pair_kind(causal, r, src)};
    } else {
        const int64_t C = Sp / (2 * P);
        const int mine[2] = {r, 2 * P - 1 - r};
        const int theirs[2] = {src, 2 * P - 1 - src};
        for (int slot = 0; slot < 2; ++slot)
            for (int kc : theirs) {
                const int qc = mine[slot];
                out[n++] = RingPair{slot, qc, kc, qc * C, kc * C, C, clip_rows(S, qc * C, C),
                                    clip_rows(S, kc * C, C), qc * C, kc * C,
                                    pair_kind(causal, qc, kc)};
            }
    }
    for (int i = 0; i < n; ++i)
        if (out[i].len_q == 0 || out[i].len_k == 0)
            out[i].kind = CP_PAIR_SKIP;
    return n;
}

// First output row of query slot `slot` of a pair: the pair's own rows when
// every rank is computed (natural order, or the striped shards back to
// back), the rank's local order otherwise.
int64_t out_row_of(int rank_arg, const RingPair &p)
{
    return rank_arg < 0 ? p.q_row : (int64_t)p.slot * p.cap;
}

// Output rows of a ring call: every rank in the inputs' order, or one rank's
// padded share.
int64_t ring_rows_out(int64_t S, int P, cp_layout layout, int rank)
{
    return rank < 0 ? input_rows(S, P, layout) : padded_len(S, P, layout) / P;
}

}  // namespace

// =================================================================== C-ABI
extern "C" {

const char *cp_last_error(void) { return g_last_error.c_str(); }

int cp_attn_block_fwd(const void *q, const void *k, const void *v, float *out, float *lse,
                      int64_t Sq, int64_t Sk, int Hq, int Hkv, int D, int64_t q_offset,
                      int64_t k_offset, int causal, cp_dtype dtype, void *stream)
{
    int rc = check_attn_common(q, k, v, out, lse, Sq, Sk, Hq, Hkv, D, dtype);
    if (rc)
        return rc;
    if (Sq == 0)
        return ok();
    AttnLaunch a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.lse_ld = Sq;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.causal = causal ? 1 : 0;
    a.n_q = 1;
    QSeg &s = a.qs[0];
    s.row0 = 0;
    s.pos0 = q_offset;
    s.len = Sq;
    s.out_row0 = 0;
    s.merge = 0;
    s.n_kv = Sk > 0 ? 1 : 0;
    s.kv[0] = KvSeg{0, k_offset, Sk};
    rc = launch_attn(a, dtype, (hipStream_t)stream);
    return rc ? rc : ok();
}

int cp_lse_merge(const float *o1, const float *lse1, const float *o2, const float *lse2,
                 float *o, float *lse, int64_t Sq, int H, int D, void *stream)
{
    if (Sq != 0 && (!o1 || !lse1 || !o2 || !lse2 || !o || !lse))
        return fail(CP_ERR_NULL, "all merge pointers must be non-NULL");
    if (Sq < 0 || H < 1 || D < 1)
        return fail(CP_ERR_SHAPE, "need Sq >= 0, H >= 1, D >= 1");
    if (D % 4 != 0 || D > 256)
        return fail(CP_ERR_UNSUPPORTED, "merge needs D %% 4 == 0 and D <= 256 (D=%d)", D);
    if (!aligned(o1, 16) || !aligned(o2, 16) || !aligned(o, 16) || !aligned(lse1, 4) ||
        !aligned(lse2, 4) || !aligned(lse, 4))
        return fail(CP_ERR_ALIGN, "merge needs 16-byte aligned o buffers");
    const size_t ob = (size_t)Sq * H * D * 4, lb = (size_t)Sq * H * 4;
    auto bad_alias = [&](const void *x, size_t nx, const void *y, size_t ny) {
        return x != y && overlaps(x, nx, y, ny);
    };
    if (bad_alias(o, ob, o1, ob) || bad_alias(o, ob, o2, ob) || bad_alias(lse, lb, lse1, lb) ||
        bad_alias(lse, lb, lse2, lb) || overlaps(o, ob, lse, lb) || overlaps(o, ob, lse1, lb) ||
        overlaps(o, ob, lse2, lb) || overlaps(lse, lb, o1, ob) || overlaps(lse, lb, o2, ob))
        return fail(CP_ERR_ALIGN, "merge outputs may only alias an input exactly");
    if (Sq == 0)
        return ok();
    hipStream_t st = (hipStream_t)stream;
    int rc = timed_launch(CP_KERNEL_MERGE, st, [&] {
        return launch_lse_merge(o1, lse1, o2, lse2, o, lse, Sq, H, D, st);
    });
    return rc ? rc : ok();
}

int cp_layout_index(cp_layout layout, int64_t S, int P, int rank, int32_t *idx)
{
    if (!idx)
        return fail(CP_ERR_NULL, "idx must be non-NULL");
    int rc = check_ring_shape(S, P, layout, rank);
    if (rc)
        return rc;
    if (rank < 0)
        return fail(CP_ERR_SHAPE, "cp_layout_index needs a rank in [0, P)");
    const int64_t Sp = padded_len(S, P, layout);
    if (Sp >= (int64_t(1) << 31))
        return fail(CP_ERR_SHAPE, "cp_layout_index needs a padded length below 2^31");
    const int64_t rows = Sp / P;
    for (int64_t j = 0; j < rows; ++j) {
        int64_t pos;
        if (layout == CP_LAYOUT_CONTIGUOUS)
            pos = rank * rows + j;
        else if (layout == CP_LAYOUT_STRIPED)
            pos = rank + j * P;
        else {
            const int64_t C = rows / 2;
            pos = j < C ? rank * C + j : (2 * (int64_t)P - 1 - rank) * C + (j - C);
        }
        idx[j] = (int32_t)pos;
    }
    return ok();
}

int cp_ring_plan(int64_t S, int P, cp_layout layout, int rank, int causal,
                 cp_block_pair *pairs, int *n_pairs)
{
    if (!n_pairs)
        return fail(CP_ERR_NULL, "n_pairs must be non-NULL");
    int rc = check_ring_shape(S, P, layout, rank);
    if (rc)
        return rc;
    const int per_step = layout == CP_LAYOUT_ZIGZAG ? 4 : 1;
    const int64_t n_ranks = rank < 0 ? P : 1;
    const int64_t need = n_ranks * P * per_step;
    if (need > 0x7fffffff)
        return fail(CP_ERR_SHAPE, "plan too large");
    if (!pairs) {
        *n_pairs = (int)need;
        return ok();
    }
    if (*n_pairs < need) {
        const int cap = *n_pairs;
        *n_pairs = (int)need;
        return fail(CP_ERR_CAPACITY, "pairs holds %d entries, the plan needs %lld", cap,
                    (long long)need);
    }
    int n = 0;
    for (int r = (rank < 0 ? 0 : rank); r < (rank < 0 ? P : rank + 1); ++r)
        for (int t = 0; t < P; ++t) {
            const int src = ((r - t) % P + P) % P;
            RingPair rp[4];
            const int m = ring_step_pairs(layout, S, P, r, src, causal, rp);
            for (int i = 0; i < m; ++i) {
                cp_block_pair &p = pairs[n++];
                p.rank = r;
                p.step = t;
                p.q_chunk = rp[i].qc;
                p.k_chunk = rp[i].kc;
                p.q_offset = rp[i].q_pos;
                p.k_offset = rp[i].k_pos;
                p.len_q = rp[i].len_q;
                p.len_k = rp[i].len_k;
                p.kind = rp[i].kind;
                p.reserved = 0;
            }
        }
    *n_pairs = n;
    return ok();
}

int cp_ring_fwd(const void *q, const void *k, const void *v, float *out, float *lse, int64_t S,
                int Hq, int Hkv, int D, int P, cp_layout layout, int rank, int causal,
                cp_dtype dtype, void *stream)
{
    int rc = check_ring_shape(S, P, layout, rank);
    if (rc)
        return rc;
    const int64_t rows_in = input_rows(S, P, layout);
    const int64_t rows_out = ring_rows_out(S, P, layout, rank);
    // q, k, v span rows_in rows; out and lse span rows_out rows.
    if (S > 0 && (!q || !k || !v || !out || !lse))
        return fail(CP_ERR_NULL, "q, k, v, out and lse must be non-NULL");
    rc = check_attn_common(q, k, v, out, lse, rows_out, rows_in, Hq, Hkv, D, dtype);
    if (rc)
        return rc;
    {
        const size_t eb = dtype == CP_BF16 ? 2 : 4;
        const size_t qb = (size_t)rows_in * Hq * D * eb, kb = (size_t)rows_in * Hkv * D * eb;
        const size_t ob = (size_t)rows_out * Hq * D * 4, lb = (size_t)rows_out * Hq * 4;
        if (overlaps(q, qb, out, ob) || overlaps(q, qb, lse, lb) || overlaps(k, kb, out, ob) ||
            overlaps(k, kb, lse, lb) || overlaps(v, kb, out, ob) || overlaps(v, kb, lse, lb) ||
            overlaps(out, ob, lse, lb))
            return fail(CP_ERR_ALIGN, "q, k, v, out and lse must not overlap");
    }
    if (S == 0)
        return ok();

    hipStream_t st = (hipStream_t)stream;
    const int r_begin = rank < 0 ? 0 : rank;
    const int r_end = rank < 0 ? P : rank + 1;
    // started[r][slot]: has this query chunk received its first result yet?
    std::vector<std::vector<char>> started(P, std::vector<char>(2, 0));

    for (int t = 0; t < P; ++t) {
        AttnLaunch a{};
        a.q = q;
        a.k = k;
        a.v = v;
        a.out = out;
        a.lse = lse;
        a.lse_ld = rows_out;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.D = D;
        a.causal = causal ? 1 : 0;
        a.n_q = 0;
        auto flush = [&]() -> int {
            if (a.n_q == 0)
                return CP_OK;
            int r2 = launch_attn(a, dtype, st);
            a.n_q = 0;
            return r2;
        };
        for (int r = r_begin; r < r_end; ++r) {
            const int src = ((r - t) % P + P) % P;
            RingPair rp[4];
            const int m = ring_step_pairs(layout, S, P, r, src, causal, rp);
            for (int slot = 0; slot < n_slots(layout); ++slot) {
                QSeg seg{};
                seg.n_kv = 0;
                for (int i = 0; i < m; ++i) {
                    if (rp[i].slot != slot)
                        continue;
                    seg.row0 = rp[i].q_row;
                    seg.pos0 = rp[i].q_pos;
                    seg.len = rp[i].len_q;
                    seg.out_row0 = out_row_of(rank, rp[i]);
                    if (rp[i].kind == CP_PAIR_SKIP)
                        continue;
                    seg.kv[seg.n_kv++] = KvSeg{rp[i].k_row, rp[i].k_pos, rp[i].len_k};
                }
                if (seg.n_kv == 0)
                    continue;
                seg.merge = started[r][slot] ? 1 : 0;
                started[r][slot] = 1;
                if (a.n_q == kMaxQSegs && (rc = flush()))
                    return rc;
                a.qs[a.n_q++] = seg;
            }
        }
        if ((rc = flush()))
            return rc;
    }
    // Every query chunk with real rows sees its own (diagonal) chunk at step
    // 0, so every real output row has been written; the padding rows of the
    // output get (0, -inf).
    for (int r = r_begin; r < r_end; ++r) {
        RingPair rp[4];
        const int m = ring_step_pairs(layout, S, P, r, r, causal, rp);
        for (int slot = 0; slot < n_slots(layout); ++slot) {
            const RingPair *p = nullptr;
            for (int i = 0; i < m && !p; ++i)
                if (rp[i].slot == slot)
                    p = &rp[i];
            if (p->len_q > 0 && !started[r][slot])
                return fail(CP_ERR_HIP, "internal: ring left rank %d slot %d unwritten", r, slot);
            const int64_t o0 = out_row_of(rank, *p) + p->len_q;
            const int64_t pad = std::min(p->cap - p->len_q, rows_out - o0);
            if (pad > 0 && (rc = fill_pad_rows(out, lse, rows_out, Hq, D, o0, pad, st)))
                return rc;
        }
    }
    return ok();
}

int cp_attn_bwd_dvec(const float *out, const void *dout, float *dvec, int64_t Sq, int Hq, int D,
                     cp_dtype dtype, void *stream)
{
    if (Sq > 0 && (!out || !dout || !dvec))
        return fail(CP_ERR_NULL, "out, dout and dvec must be non-NULL");
    if (Sq < 0 || Hq < 1)
        return fail(CP_ERR_SHAPE, "need Sq >= 0 and Hq >= 1");
    if (dtype != CP_BF16 && dtype != CP_F32)
        return fail(CP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (D < 1 || D > 128)
        return fail(CP_ERR_UNSUPPORTED, "dvec supports 1 <= D <= 128 (D=%d)", D);
    if (!aligned(out, 4) || !aligned(dvec, 4) || !aligned(dout, dtype == CP_BF16 ? 2 : 4))
        return fail(CP_ERR_ALIGN, "misaligned out, dout or dvec");
    const size_t ob = (size_t)Sq * Hq * D * 4, db = (size_t)Sq * Hq * D * (dtype == CP_BF16 ? 2 : 4);
    if (overlaps(dvec, (size_t)Sq * Hq * 4, out, ob) || overlaps(dvec, (size_t)Sq * Hq * 4, dout, db))
        return fail(CP_ERR_ALIGN, "dvec must not overlap out or dout");
    if (Sq == 0)
        return ok();
    hipStream_t st = (hipStream_t)stream;
    int rc = timed_launch(CP_KERNEL_BWD_DVEC, st, [&] {
        return launch_bwd_dvec(out, dout, dtype == CP_BF16 ? 1 : 0, dvec, Sq, Sq, Hq, D, st);
    });
    return rc ? rc : ok();
}

int cp_attn_block_bwd(const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, const float *dvec, float *dq, float *dk, float *dv,
                      int64_t Sq, int64_t Sk, int Hq, int Hkv, int D, int64_t q_offset,
                      int64_t k_offset, int causal, int accumulate, cp_dtype dtype, void *stream)
{
    int rc = check_bwd(q, k, v, dout, lse, dvec, dq, dk, dv, Sq, Sk, Hq, Hkv, D, dtype);
    if (rc)
        return rc;
    if (Sq == 0 && Sk == 0)
        return ok();
    BwdLaunch b{};
    b.q = q;
    b.k = k;
    b.v = v;
    b.dout = dout;
    b.lse = lse;
    b.dvec = dvec;
    b.stat_ld = Sq;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.Sq = Sq;
    b.Sk = Sk;
    b.Hq = Hq;
    b.Hkv = Hkv;
    b.D = D;
    b.causal = causal ? 1 : 0;
    b.accumulate = accumulate ? 1 : 0;
    b.q_offset = q_offset;
    b.k_offset = k_offset;
    rc = launch_bwd(b, dtype, (hipStream_t)stream);
    return rc ? rc : ok();
}

}  // extern "C"

namespace {

// Argument checks of the ring backward (every one before any HIP call).
int ring_bwd_check(const void *q, const void *k, const void *v, const float *out,
                   const float *lse, const void *dout, float *dq, float *dk, float *dv,
                   const float *dvec, int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout,
                   int rank, cp_dtype dtype)
{
    int rc = check_ring_shape(S, P, layout, rank);
    if (rc)
        return rc;
    const int64_t rows_in = input_rows(S, P, layout);
    const int64_t rows_out = ring_rows_out(S, P, layout, rank);
    if (S > 0 && (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !dvec))
        return fail(CP_ERR_NULL, "every pointer of cp_ring_bwd must be non-NULL");
    // dq, dout, lse and dvec span rows_out rows; q, k, v, dk and dv span rows_in rows
    rc = check_bwd(q, k, v, dout, lse, dvec, dq, dk, dv, rows_out, rows_in, Hq, Hkv, D, dtype);
    if (rc)
        return rc;
    const size_t eb = dtype == CP_BF16 ? 2 : 4;
    const size_t qb = (size_t)rows_in * Hq * D * eb, ob = (size_t)rows_out * Hq * D * 4;
    const size_t gk = (size_t)rows_in * Hkv * D * 4;
    if (overlaps(q, qb, dq, ob) || overlaps(q, qb, dk, gk) || overlaps(q, qb, dv, gk) ||
        overlaps(out, ob, dq, ob) || overlaps(out, ob, dk, gk) || overlaps(out, ob, dv, gk) ||
        overlaps(dvec, (size_t)rows_out * Hq * 4, out, ob) ||
        overlaps(dvec, (size_t)rows_out * Hq * 4, dq, ob))
        return fail(CP_ERR_ALIGN, "gradient buffers must not overlap the inputs");
    if (!aligned(out, 4))
        return fail(CP_ERR_ALIGN, "out must be 4-byte aligned");
    return CP_OK;
}

// The bf16 launches of one ring step's computed pairs: per pair its dq
// launch, then its dk/dv launch, except that two pairs whose dk/dv launches
// would each hold fewer workgroups than the chip has CUs (the causal
// diagonal blocks of few KV heads) share one dk/dv launch when their dk/dv
// rows are disjoint; that launch follows the second pair's dq launch.  A
// pair goes into no dk/dv launch before one holding an earlier pair that
// writes the same rows, so every row still accumulates its pairs in pair
// order: the same sums, in the same order, as one launch per pair.
constexpr int64_t kChipCUs = 256;   // MI355X: 8 XCDs x 32 CUs
int launch_bwd_bf16_step(const BwdLaunch *bl, int nb, int Hkv, int D, hipStream_t st)
{
    int rc;
    int member[4][2], n_members[4], n_launch = 0, launch_of[4];
    for (int i = 0; i < nb; ++i) {
        int first = 0;      // launches before this one hold a pair writing its rows
        const size_t bi = (size_t)bl[i].Sk * Hkv * D * 4;
        for (int j = 0; j < i; ++j)
            if (overlaps(bl[i].dk, bi, bl[j].dk, (size_t)bl[j].Sk * Hkv * D * 4))
                first = std::max(first, launch_of[j] + 1);
        int L = n_launch;
        if (bwd_bf16_dkdv_units(bl[i]) < kChipCUs)
            for (int l = first; l < n_launch; ++l)
                if (n_members[l] == 1 && bwd_bf16_dkdv_units(bl[member[l][0]]) < kChipCUs) {
                    L = l;
                    break;
                }
        if (L == n_launch)
            n_members[n_launch++] = 0;
        member[L][n_members[L]++] = i;
        launch_of[i] = L;
    }
    // per pair: its dq launch, then the dk/dv launches (in order) whose
    // pairs have all had their dq launch
    int next = 0;
    for (int i = 0; i < nb; ++i) {
        rc = timed_launch(CP_KERNEL_BWD_BF16, st, [&] {
            hipError_t e = launch_bwd_bf16_dq(bl[i], st);
            for (; e == hipSuccess && next < n_launch; ++next) {
                if (member[next][n_members[next] - 1] > i)
                    break;
                BwdLaunch two[2];
                for (int m = 0; m < n_members[next]; ++m)
                    two[m] = bl[member[next][m]];
                e = launch_bwd_bf16_dkdv(two, n_members[next], st);
            }
            return e;
        });
        if (rc)
            return rc;
    }
    return CP_OK;
}

// The ring backward's launches, after ring_bwd_check: dvec of the output
// rows, zeroed gradients, then per ring step the dq and dk/dv launches of
// its computed pairs.
int ring_bwd_run(const void *q, const void *k, const void *v, const float *out,
                 const float *lse, const void *dout, float *dq, float *dk, float *dv,
                 float *dvec, int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout,
                 int rank, int causal, cp_dtype dtype, hipStream_t st)
{
    const int64_t rows_in = input_rows(S, P, layout);
    const int64_t rows_out = ring_rows_out(S, P, layout, rank);
    int rc = timed_launch(CP_KERNEL_BWD_DVEC, st, [&] {
        return launch_bwd_dvec(out, dout, dtype == CP_BF16 ? 1 : 0, dvec, rows_out, rows_out, Hq,
                               D, st);
    });
    if (rc)
        return rc;
    if ((rc = fill_zero(dq, rows_out * Hq * D, st)) ||
        (rc = fill_zero(dk, rows_in * Hkv * D, st)) || (rc = fill_zero(dv, rows_in * Hkv * D, st)))
        return rc;
    const size_t eb = dtype == CP_BF16 ? 2 : 4;
    const int r_begin = rank < 0 ? 0 : rank;
    const int r_end = rank < 0 ? P : rank + 1;
    for (int r = r_begin; r < r_end; ++r)
        for (int t = 0; t < P; ++t) {
            const int src = ((r - t) % P + P) % P;
            RingPair rp[4];
            const int m = ring_step_pairs(layout, S, P, r, src, causal, rp);
            BwdLaunch bl[4];
            int nb = 0;
            for (int i = 0; i < m; ++i) {
                const RingPair &p = rp[i];
                if (p.kind == CP_PAIR_SKIP)
                    continue;
                const int64_t orow = out_row_of(rank, p);
                BwdLaunch b{};
                b.q = (const char *)q + (size_t)p.q_row * Hq * D * eb;
                b.k = (const char *)k + (size_t)p.k_row * Hkv * D * eb;
                b.v = (const char *)v + (size_t)p.k_row * Hkv * D * eb;
                b.dout = (const char *)dout + (size_t)orow * Hq * D * eb;
                b.lse = lse + orow;
                b.dvec = dvec + orow;
                b.stat_ld = rows_out;
                b.dq = dq + (size_t)orow * Hq * D;
                b.dk = dk + (size_t)p.k_row * Hkv * D;
                b.dv = dv + (size_t)p.k_row * Hkv * D;
                b.Sq = p.len_q;
                b.Sk = p.len_k;
                b.Hq = Hq;
                b.Hkv = Hkv;
                b.D = D;
                b.causal = p.kind == CP_PAIR_DIAG ? 1 : 0;
                b.accumulate = 1;
                b.q_offset = p.q_pos;
                b.k_offset = p.k_pos;
                if (dtype != CP_BF16) {
                    if ((rc = launch_bwd(b, dtype, st)))
                        return rc;
                    continue;
                }
                bl[nb++] = b;
            }
            if ((rc = launch_bwd_bf16_step(bl, nb, Hkv, D, st)))
                return rc;
        }
    return CP_OK;
}

}  // namespace

extern "C" {

int cp_ring_bwd(const void *q, const void *k, const void *v, const float *out, const float *lse,
                const void *dout, float *dq, float *dk, float *dv, float *dvec, int64_t S, int Hq,
                int Hkv, int D, int P, cp_layout layout, int rank, int causal, cp_dtype dtype,
                void *stream)
{
    int rc = ring_bwd_check(q, k, v, out, lse, dout, dq, dk, dv, dvec, S, Hq, Hkv, D, P, layout,
                            rank, dtype);
    if (rc)
        return rc;
    if (S == 0)
        return ok();
    rc = ring_bwd_run(q, k, v, out, lse, dout, dq, dk, dv, dvec, S, Hq, Hkv, D, P, layout, rank,
                      causal, dtype, (hipStream_t)stream);
    return rc ? rc : ok();
}

int cp_ring_bwd_noalloc(const void *q, const void *k, const void *v, const float *out,
                        const float *lse, const void *dout, float *dq, float *dk, float *dv,
                        int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout, int rank,
                        int causal, cp_dtype dtype, void *stream)
{
    // dvec comes from the library's scratch array, which no caller buffer can
    // overlap: the checks run with lse (same shape, read only) in its place
    int rc = ring_bwd_check(q, k, v, out, lse, dout, dq, dk, dv, lse, S, Hq, Hkv, D, P, layout,
                            rank, dtype);
    if (rc)
        return rc;
    const int64_t need = (int64_t)Hq * ring_rows_out(S, P, layout, rank);
    if (need > kScratchFloats)
        return fail(CP_ERR_WORKSPACE,
                    "cp_ring_bwd_noalloc keeps Hq x output rows = %lld floats of dvec in its "
                    "scratch array, which holds %lld; use cp_ring_bwd with a caller buffer",
                    (long long)need, (long long)kScratchFloats);
    if (S == 0)
        return ok();
    float *dvec = nullptr;
    const hipError_t e = scratch_floats(&dvec);
    if (e != hipSuccess)
        return fail(CP_ERR_HIP, "scratch array lookup failed: %s", hipGetErrorString(e));
    rc = ring_bwd_run(q, k, v, out, lse, dout, dq, dk, dv, dvec, S, Hq, Hkv, D, P, layout, rank,
                      causal, dtype, (hipStream_t)stream);
    return rc ? rc : ok();
}

// One rank's head share, row by row: to_head copies y[t] <- x[t][p*Hp, (p+1)*Hp),
// otherwise y[t][p*Hp, (p+1)*Hp) <- x[t], for rows t in [0, rows).
static int head_share_copy(bool to_head, const void *x, void *y, int64_t rows, int H, int D,
                           int P, int p, size_t elem_bytes, hipStream_t st)
{
    if (rows == 0)
        return CP_OK;
    const int64_t unit = (int64_t)(H / P) * D * (int64_t)elem_bytes;
    const int64_t row = (int64_t)H * D * (int64_t)elem_bytes;
    UnitCopy c{};
    c.src = x;
    c.dst = y;
    c.unit_bytes = unit;
    c.n_units = rows;  // u = t
    c.per = rows;
    if (to_head) {
        c.src_base = p * unit, c.src_a = 0, c.src_b = row;
        c.dst_base = 0, c.dst_a = 0, c.dst_b = unit;
    } else {
        c.src_base = 0, c.src_a = 0, c.src_b = unit;
        c.dst_base = p * unit, c.dst_a = 0, c.dst_b = row;
    }
    return timed_launch(CP_KERNEL_PERMUTE, st, [&] { return launch_unit_copy(c, st); });
}

static int repack(bool to_head, const void *x, void *y, int64_t S, int H, int D, int P,
                  int rank, size_t elem_bytes, void *stream)
{
    if (S != 0 && (!x || !y))
        return fail(CP_ERR_NULL, "x and y must be non-NULL");
    if (S < 0 || H < 1 || D < 1 || P < 1)
        return fail(CP_ERR_SHAPE, "need S >= 0, H >= 1, D >= 1, P >= 1");
    if (H % P != 0)
        return fail(CP_ERR_SHAPE, "P must divide the head count (H=%d, P=%d)", H, P);
    if (S % P != 0)
        return fail(CP_ERR_SHAPE, "P must divide S (S=%lld, P=%d)", (long long)S, P);
    if (rank < -1 || rank >= P)
        return fail(CP_ERR_SHAPE, "rank must be -1 or in [0, P)");
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(CP_ERR_UNSUPPORTED, "elem_bytes must be 2 or 4");
    if (!aligned(x, elem_bytes) || !aligned(y, elem_bytes))
        return fail(CP_ERR_ALIGN, "x and y must be aligned to elem_bytes");
    const int64_t Hp = H / P;
    const int64_t unit = Hp * D * (int64_t)elem_bytes;  // bytes of one run
    const int64_t row = (int64_t)H * D * (int64_t)elem_bytes;
    // the natural tensor and the all-ranks tensor hold S*H*D elements, one
    // rank's head share S*Hp*D
    const size_t all_bytes = (size_t)S * H * D * elem_bytes;
    const size_t share_bytes = rank < 0 ? all_bytes : (size_t)S * Hp * D * elem_bytes;
    const size_t xb = to_head ? all_bytes : share_bytes;
    const size_t yb = to_head ? share_bytes : all_bytes;
    if (overlaps(x, xb, y, yb))
        return fail(CP_ERR_ALIGN, "x and y must not overlap");
    if (S == 0)
        return ok();
    hipStream_t st = (hipStream_t)stream;
    if (rank >= 0) {
        const int rc = head_share_copy(to_head, x, y, S, H, D, P, rank, elem_bytes, st);
        return rc ? rc : ok();
    }
    UnitCopy c{};
    c.src = x;
    c.dst = y;
    c.unit_bytes = unit;
    c.n_units = (int64_t)P * S;  // u = p*S + t
    c.per = S;
    if (to_head) {  // y[p][t] <- x[t][p*Hp]
        c.src_base = 0, c.src_a = unit, c.src_b = row;
        c.dst_base = 0, c.dst_a = S * unit, c.dst_b = unit;
    } else {        // y[t][p*Hp] <- x[p][t]
        c.src_base = 0, c.src_a = S * unit, c.src_b = unit;
        c.dst_base = 0, c.dst_a = unit, c.dst_b = row;
    }
    int rc = timed_launch(CP_KERNEL_PERMUTE, st, [&] { return launch_unit_copy(c, st); });
    return rc ? rc : ok();
}

int cp_seq_to_head(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                   size_t elem_bytes, void *stream)
{
    return repack(true, x, y, S, H, D, P, rank, elem_bytes, stream);
}

int cp_head_to_seq(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                   size_t elem_bytes, void *stream)
{
    return repack(false, x, y, S, H, D, P, rank, elem_bytes, stream);
}

// ------------------------------------------------------------------ USP
// Sizes of one USP call: the head shares and the workspace carve-up.
struct UspPlan {
    int Hp, Hkvp;
    size_t eb;
    int64_t rows_in, rows_out;
    size_t off_k, off_v, off_out, total;
};

static int usp_plan(int64_t S, int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout,
                    int rank, cp_dtype dtype, UspPlan *pl)
{
    if (P_u < 1 || P_r < 1)
        return fail(CP_ERR_SHAPE, "need P_u >= 1 and P_r >= 1 (P_u=%d, P_r=%d)", P_u, P_r);
    if ((int64_t)P_u * P_r > (1 << 20))
        return fail(CP_ERR_SHAPE, "P_u * P_r too large");
    const int P = P_u * P_r;
    if (rank < -1 || rank >= P)
        return fail(CP_ERR_SHAPE, "rank must be -1 or in [0, P_u*P_r) (rank=%d)", rank);
    int rc = check_ring_shape(S, P_r, layout, rank < 0 ? -1 : rank / P_u);
    if (rc)
        return rc;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
        return fail(CP_ERR_SHAPE, "need Hkv dividing Hq (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hkv % P_u != 0)
        return fail(CP_ERR_SHAPE,
                    "every Ulysses rank needs whole KV heads: P_u must divide Hkv (Hkv=%d, P_u=%d)",
                    Hkv, P_u);
    if (dtype != CP_BF16 && dtype != CP_F32)
        return fail(CP_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    pl->Hp = Hq / P_u;
    pl->Hkvp = Hkv / P_u;
    pl->eb = dtype == CP_BF16 ? 2 : 4;
    // a ring split that does not divide S is padded as by the ring itself:
    // rows_in rows of q, k, v (S, or S_pad in striped order), rows_out
    // output rows (padding rows (0, -inf))
    pl->rows_in = input_rows(S, P_r, layout);
    pl->rows_out = ring_rows_out(S, P_r, layout, rank < 0 ? -1 : rank / P_u);
    const size_t qb = up((size_t)pl->rows_in * pl->Hp * D * pl->eb);
    const size_t kb = up((size_t)pl->rows_in * pl->Hkvp * D * pl->eb);
    pl->off_k = qb;
    pl->off_v = qb + kb;
    pl->off_out = qb + 2 * kb;
    pl->total = pl->off_out + up((size_t)pl->rows_out * pl->Hp * D * 4);
    return CP_OK;
}

int cp_usp_fwd_workspace(int64_t S, int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout,
                         int rank, cp_dtype dtype, size_t *bytes)
{
    if (!bytes)
        return fail(CP_ERR_NULL, "bytes must be non-NULL");
    UspPlan pl{};
    const int rc = usp_plan(S, Hq, Hkv, D, P_u, P_r, layout, rank, dtype, &pl);
    if (rc)
        return rc;
    *bytes = S == 0 ? 0 : pl.total;
    return ok();
}

int cp_usp_fwd(const void *q, const void *k, const void *v, float *out, float *lse, int64_t S,
               int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout, int rank, int causal,
               cp_dtype dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    UspPlan pl{};
    int rc = usp_plan(S, Hq, Hkv, D, P_u, P_r, layout, rank, dtype, &pl);
    if (rc)
        return rc;
    rc = check_attn_common(q, k, v, out, lse, pl.rows_out, pl.rows_in, Hq, Hkv, D, dtype);
    if (rc)
        return rc;
    if (S == 0)
        return ok();
    if (!workspace)
        return fail(CP_ERR_NULL, "workspace must be non-NULL");
    if (workspace_bytes < pl.total)
        return fail(CP_ERR_WORKSPACE, "workspace holds %zu bytes, the call needs %zu",
                    workspace_bytes, pl.total);
    if (!aligned(workspace, 256))
        return fail(CP_ERR_ALIGN, "workspace must be 256-byte aligned");
    {
        const size_t qb = (size_t)pl.rows_in * Hq * D * pl.eb;
        const size_t kb = (size_t)pl.rows_in * Hkv * D * pl.eb;
        const size_t ob = (size_t)pl.rows_out * Hq * D * 4, lb = (size_t)pl.rows_out * Hq * 4;
        if (overlaps(workspace, pl.total, q, qb) || overlaps(workspace, pl.total, k, kb) ||
            overlaps(workspace, pl.total, v, kb) || overlaps(workspace, pl.total, out, ob) ||
            overlaps(workspace, pl.total, lse, lb) || overlaps(q, qb, out, ob) ||
            overlaps(k, kb, out, ob) || overlaps(v, kb, out, ob) || overlaps(out, ob, lse, lb))
            return fail(CP_ERR_ALIGN, "workspace, inputs and outputs must not overlap");
    }
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    void *ws_q = ws, *ws_k = ws + pl.off_k, *ws_v = ws + pl.off_v;
    float *ws_out = (float *)(ws + pl.off_out);
    const int r = rank < 0 ? -1 : rank / P_u;
    const size_t qrow = (size_t)Hq * D * pl.eb, qrow_p = (size_t)pl.Hp * D * pl.eb;
    for (int u = (rank < 0 ? 0 : rank % P_u); u < (rank < 0 ? P_u : rank % P_u + 1); ++u) {
        // 1. the all-to-all inside the ring group: query rows of the group(s)
        //    computed here, head share u
        if (r < 0) {
            rc = head_share_copy(true, q, ws_q, pl.rows_in, Hq, D, P_u, u, pl.eb, st);
        } else {
            RingPair rp[4];
            const int m = ring_step_pairs(layout, S, P_r, r, r, causal, rp);
            for (int i = 0; i < m && !rc; ++i) {
                if (rp[i].kc != rp[i].qc)   // one pair per query chunk of the group
                    continue;
                rc = head_share_copy(true, (const char *)q + rp[i].q_row * qrow,
                                     (char *)ws_q + rp[i].q_row * qrow_p, rp[i].len_q, Hq, D,
                                     P_u, u, pl.eb, st);
            }
        }
        // key and value rows of every group: the group's own by the
        // all-to-all, the others as the ring delivers them
        if (rc || (rc = head_share_copy(true, k, ws_k, pl.rows_in, Hkv, D, P_u, u, pl.eb, st)) ||
            (rc = head_share_copy(true, v, ws_v, pl.rows_in, Hkv, D, P_u, u, pl.eb, st)))
            return rc;
        // 2. the ring over the P_r groups on head share u
        rc = cp_ring_fwd(ws_q, ws_k, ws_v, ws_out, lse + (size_t)u * pl.Hp * pl.rows_out, S,
                         pl.Hp, pl.Hkvp, D, P_r, layout, r, causal, dtype, stream);
        if (rc)
            return rc;
        // 3. the all-to-all back: head share u of the output rows
        if ((rc = head_share_copy(false, ws_out, out, pl.rows_out, Hq, D, P_u, u, 4, st)))
            return rc;
    }
    return ok();
}

// Workspace of the USP backward: head shares of q, k, v (whole sequence),
// of dout and out (output rows), and the ring backward's dq, dk, dv and
// dvec for that share.
struct UspBwdPlan {
    size_t off_k, off_v, off_dout, off_out, off_dq, off_dk, off_dv, off_dvec, total;
};

static UspBwdPlan usp_bwd_plan(const UspPlan &pl, int64_t S, int D)
{
    auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
    UspBwdPlan b{};
    const size_t qb = up((size_t)pl.rows_in * pl.Hp * D * pl.eb);
    const size_t kb = up((size_t)pl.rows_in * pl.Hkvp * D * pl.eb);
    const size_t rows = (size_t)pl.rows_out;
    b.off_k = qb;
    b.off_v = b.off_k + kb;
    b.off_dout = b.off_v + kb;
    b.off_out = b.off_dout + up(rows * pl.Hp * D * pl.eb);
    b.off_dq = b.off_out + up(rows * pl.Hp * D * 4);
    b.off_dk = b.off_dq + up(rows * pl.Hp * D * 4);
    b.off_dv = b.off_dk + up((size_t)pl.rows_in * pl.Hkvp * D * 4);
    b.off_dvec = b.off_dv + up((size_t)pl.rows_in * pl.Hkvp * D * 4);
    b.total = b.off_dvec + up(rows * pl.Hp * 4);
    return b;
}

int cp_usp_bwd_workspace(int64_t S, int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout,
                         int rank, cp_dtype dtype, size_t *bytes)
{
    if (!bytes)
        return fail(CP_ERR_NULL, "bytes must be non-NULL");
    UspPlan pl{};
    const int rc = usp_plan(S, Hq, Hkv, D, P_u, P_r, layout, rank, dtype, &pl);
    if (rc)
        return rc;
    *bytes = S == 0 ? 0 : usp_bwd_plan(pl, S, D).total;
    return ok();
}

int cp_usp_bwd(const void *q, const void *k, const void *v, const float *out, const float *lse,
               const void *dout, float *dq, float *dk, float *dv, int64_t S, int Hq, int Hkv,
               int D, int P_u, int P_r, cp_layout layout, int rank, int causal, cp_dtype dtype,
               void *workspace, size_t workspace_bytes, void *stream)
{
    UspPlan pl{};
    int rc = usp_plan(S, Hq, Hkv, D, P_u, P_r, layout, rank, dtype, &pl);
    if (rc)
        return rc;
    if (S > 0 && (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv))
        return fail(CP_ERR_NULL, "every pointer of cp_usp_bwd must be non-NULL");
    rc = check_bwd(q, k, v, dout, lse, lse, dq, dk, dv, pl.rows_out, pl.rows_in, Hq, Hkv, D,
                   dtype);
    if (rc)
        return rc;
    if (S == 0)
        return ok();
    const UspBwdPlan bp = usp_bwd_plan(pl, S, D);
    if (!workspace)
        return fail(CP_ERR_NULL, "workspace must be non-NULL");
    if (workspace_bytes < bp.total)
        return fail(CP_ERR_WORKSPACE, "workspace holds %zu bytes, the call needs %zu",
                    workspace_bytes, bp.total);
    if (!aligned(workspace, 256) || !aligned(out, 4))
        return fail(CP_ERR_ALIGN, "workspace must be 256-byte aligned and out 4-byte aligned");
    {
        const size_t qb = (size_t)pl.rows_in * Hq * D * pl.eb;
        const size_t kb = (size_t)pl.rows_in * Hkv * D * pl.eb;
        const size_t rows = (size_t)pl.rows_out;
        const size_t ob = rows * Hq * D * 4, db = rows * Hq * D * pl.eb, lb = rows * Hq * 4;
        const size_t gk = (size_t)pl.rows_in * Hkv * D * 4;
        const void *ins[6] = {q, k, v, out, lse, dout};
        const size_t inb[6] = {qb, kb, kb, ob, lb, db};
        void *outs[3] = {dq, dk, dv};
        const size_t outb[3] = {ob, gk, gk};
        for (int i = 0; i < 6; ++i) {
            if (overlaps(workspace, bp.total, ins[i], inb[i]))
                return fail(CP_ERR_ALIGN, "workspace, inputs and gradients must not overlap");
            for (int j = 0; j < 3; ++j)
                if (overlaps(outs[j], outb[j], ins[i], inb[i]))
                    return fail(CP_ERR_ALIGN, "workspace, inputs and gradients must not overlap");
        }
        for (int j = 0; j < 3; ++j)
            if (overlaps(workspace, bp.total, outs[j], outb[j]) ||
                overlaps(outs[j], outb[j], outs[(j + 1) % 3], outb[(j + 1) % 3]))
                return fail(CP_ERR_ALIGN, "workspace, inputs and gradients must not overlap");
    }
    hipStream_t st = (hipStream_t)stream;
    char *ws = (char *)workspace;
    void *ws_q = ws, *ws_k = ws + bp.off_k, *ws_v = ws + bp.off_v, *ws_dout = ws + bp.off_dout;
    float *ws_out = (float *)(ws + bp.off_out), *ws_dq = (float *)(ws + bp.off_dq);
    float *ws_dk = (float *)(ws + bp.off_dk), *ws_dv = (float *)(ws + bp.off_dv);
    float *ws_dvec = (float *)(ws + bp.off_dvec);
    const int r = rank < 0 ? -1 : rank / P_u;
    const size_t qrow = (size_t)Hq * D * pl.eb, qrow_p = (size_t)pl.Hp * D * pl.eb;
    for (int u = (rank < 0 ? 0 : rank % P_u); u < (rank < 0 ? P_u : rank % P_u + 1); ++u) {
        // head share u of the query rows computed here, of every key and
        // value row, and of the output rows' out and dout
        if (r < 0) {
            rc = head_share_copy(true, q, ws_q, pl.rows_in, Hq, D, P_u, u, pl.eb, st);
        } else {
            RingPair rp[4];
            const int m = ring_step_pairs(layout, S, P_r, r, r, causal, rp);
            for (int i = 0; i < m && !rc; ++i)
                if (rp[i].kc == rp[i].qc)
                    rc = head_share_copy(true, (const char *)q + rp[i].q_row * qrow,
                                         (char *)ws_q + rp[i].q_row * qrow_p, rp[i].len_q, Hq,
                                         D, P_u, u, pl.eb, st);
        }
        if (rc || (rc = head_share_copy(true, k, ws_k, pl.rows_in, Hkv, D, P_u, u, pl.eb, st)) ||
            (rc = head_share_copy(true, v, ws_v, pl.rows_in, Hkv, D, P_u, u, pl.eb, st)) ||
            (rc = head_share_copy(true, dout, ws_dout, pl.rows_out, Hq, D, P_u, u, pl.eb, st)) ||
            (rc = head_share_copy(true, out, ws_out, pl.rows_out, Hq, D, P_u, u, 4, st)))
            return rc;
        // the ring backward over the P_r groups on head share u
        rc = cp_ring_bwd(ws_q, ws_k, ws_v, ws_out, lse + (size_t)u * pl.Hp * pl.rows_out,
                         ws_dout, ws_dq, ws_dk, ws_dv, ws_dvec, S, pl.Hp, pl.Hkvp, D, P_r, layout,
                         r, causal, dtype, stream);
        if (rc)
            return rc;
        // gradients back into head share u
        if ((rc = head_share_copy(false, ws_dq, dq, pl.rows_out, Hq, D, P_u, u, 4, st)) ||
            (rc = head_share_copy(false, ws_dk, dk, pl.rows_in, Hkv, D, P_u, u, 4, st)) ||
            (rc = head_share_copy(false, ws_dv, dv, pl.rows_in, Hkv, D, P_u, u, 4, st)))
            return rc;
    }
    return ok();
}

int cp_kv_seq_to_head(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                      size_t elem_bytes, void *stream)
{
    if (P >= 1 && H >= 1 && P <= H)
        return repack(true, x, y, S, H, D, P, rank, elem_bytes, stream);
    if (S != 0 && (!x || !y))
        return fail(CP_ERR_NULL, "x and y must be non-NULL");
    if (S < 0 || H < 1 || D < 1 || P < 1)
        return fail(CP_ERR_SHAPE, "need S >= 0, H >= 1, D >= 1, P >= 1");
    if (P % H != 0)
        return fail(CP_ERR_SHAPE, "KV replication needs H | P (H=%d, P=%d)", H, P);
    if (S % P != 0)
        return fail(CP_ERR_SHAPE, "P must divide S (S=%lld, P=%d)", (long long)S, P);
    if (rank < -1 || rank >= P)
        return fail(CP_ERR_SHAPE, "rank must be -1 or in [0, P)");
    if (elem_bytes != 2 && elem_bytes != 4)
        return fail(CP_ERR_UNSUPPORTED, "elem_bytes must be 2 or 4");
    if (!aligned(x, elem_bytes) || !aligned(y, elem_bytes))
        return fail(CP_ERR_ALIGN, "x and y must be aligned to elem_bytes");
    const size_t xb = (size_t)S * H * D * elem_bytes, share = (size_t)S * D * elem_bytes;
    if (overlaps(x, xb, y, rank < 0 ? share * P : share))
        return fail(CP_ERR_ALIGN, "x and y must not overlap");
    if (S == 0)
        return ok();
    // rank p receives KV head p / (P/H): the head share of rank p/(P/H) in
    // an H-way split (one head each)
    hipStream_t st = (hipStream_t)stream;
    const int rep = P / H;
    for (int p = (rank < 0 ? 0 : rank); p < (rank < 0 ? P : rank + 1); ++p) {
        void *dst = (char *)y + (rank < 0 ? (size_t)p * share : 0);
        const int rc = head_share_copy(true, x, dst, S, H, D, H, p / rep, elem_bytes, st);
        if (rc)
            return rc;
    }
    return ok();
}

int cp_timing_enable(int enable)
{
    Timing &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    t.enabled = enable != 0;
    return ok();
}

int cp_timing_reset(void)
{
    Timing &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    for (auto &rec : t.pending) {
        hipEventSynchronize(rec.stop);
        t.pool.push_back(rec.start);
        t.pool.push_back(rec.stop);
    }
    t.pending.clear();
    for (int i = 0; i < kKernelKinds; ++i) {
        t.total_ms[i] = 0;
        t.launches[i] = 0;
    }
    return ok();
}

int cp_timing_read(cp_kernel_kind kind, double *total_ms, int64_t *launches)
{
    if (!total_ms || !launches)
        return fail(CP_ERR_NULL, "total_ms and launches must be non-NULL");
    if ((int)kind < 0 || (int)kind >= kKernelKinds)
        return fail(CP_ERR_SHAPE, "unknown kernel kind %d", (int)kind);
    Timing &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    for (auto &rec : t.pending) {
        if (hipEventSynchronize(rec.stop) != hipSuccess)
            return fail(CP_ERR_HIP, "hipEventSynchronize failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, rec.start, rec.stop) != hipSuccess)
            return fail(CP_ERR_HIP, "hipEventElapsedTime failed");
        t.total_ms[rec.kind] += ms;
        t.launches[rec.kind] += 1;
        t.pool.push_back(rec.start);
        t.pool.push_back(rec.stop);
    }
    t.pending.clear();
    *total_ms = t.total_ms[kind];
    *launches = t.launches[kind];
    return ok();
}

}  // extern "C"
