/*
 * cp_attn.h -- C-ABI of libcpattn.so: blockwise causal attention with a
 * per-row log-sum-exp, the log-sum-exp merge, the ring schedule and the
 * Ulysses repacks, on one AMD Instinct MI355X (gfx950).
 *
 * Pages that define the operations (cited by title and section):
 *   [HB] "上下文并行：Ring Attention 与 Ulysses" (Context parallelism: Ring
 *        Attention and Ulysses), AI-infra handbook, train/model/context.
 *   [SP] "Sequence Parallel vs Context Parallel" blog (xxqk.cn), section 3.2,
 *        how the distributed softmax is merged; section 5.3, gradients with
 *        context parallelism checked against one card.
 *   [CP] practitioner blog comparing All-Gather, Ring, Ulysses and TE
 *        context parallelism (dpshk.com), section 4.2: the measured step is
 *        a forward plus a backward pass.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major and contiguous.  q is [Sq][Hq][D], k and v
 *     are [Sk][Hkv][D] (sequence-major, no batch dimension), out is
 *     [Sq][Hq][D] float32 and lse is [Hq][Sq] float32 holding natural-log
 *     log-sum-exp values.  A sub-chunk of the sequence is a pointer offset.
 *   - Device pointers are owned by the caller; the library never allocates
 *     or frees device memory.  Kernels are enqueued on `stream` (a
 *     hipStream_t; NULL means the default stream) and nothing synchronises
 *     the host: buffers must stay alive until the stream has drained.
 *   - Every argument is checked before any HIP call.  On failure nothing is
 *     enqueued, a non-zero cp_status is returned and cp_last_error() gives a
 *     message.  A HIP launch error returns CP_ERR_HIP.  No C++ exception
 *     crosses this interface.
 *   - bf16 tensors need 16-byte aligned base pointers; float32 tensors need
 *     4-byte alignment.  q, k, v must not overlap out or lse.  A pointer may
 *     be NULL only when its tensor is empty (zero rows).
 *   - The attention scale is fixed at 1/sqrt(D), D being the last dimension
 *     of q ([HB], section "哪些运算可以直接切", function attention()).
 *   - Query head h reads KV head h / (Hq / Hkv): contiguous head groups, as
 *     the Ulysses section of [HB] hands rank p the p-th contiguous share of
 *     heads.
 *   - A query row that sees no key yields out = 0 and lse = -inf; the merge
 *     treats lse = -inf as its identity.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CP_OK = 0,
    CP_ERR_NULL = 1,        /* a required pointer is NULL                       */
    CP_ERR_SHAPE = 2,       /* sizes inconsistent or not divisible              */
    CP_ERR_UNSUPPORTED = 3, /* valid request this build does not implement      */
    CP_ERR_CAPACITY = 4,    /* caller-provided host array too small             */
    CP_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed       */
    CP_ERR_ALIGN = 6,       /* pointer alignment or aliasing rule broken        */
    CP_ERR_WORKSPACE = 7    /* caller-provided device workspace too small       */
} cp_status;

typedef enum { CP_F32 = 0, CP_BF16 = 1 } cp_dtype;

/* How the sequence is split over P ranks ([HB], sections "Ring Attention：KV
 * 沿环传一圈" and "之字形切分"; [SP] section 3.3 for the striped split):
 *   CONTIGUOUS: rank r owns positions [r*S/P, (r+1)*S/P).
 *   ZIGZAG:     the sequence is cut into 2P chunks of C = S/(2P); rank r owns
 *               chunk r then chunk 2P-1-r, in that local order.
 *   STRIPED:    stripes of one token dealt round-robin: rank r owns positions
 *               r, r+P, r+2P, ... in that local order.  Sequence tensors for
 *               this layout are given in striped order: the ranks' S/P-row
 *               shards back to back (row r*S/P + j is position r + j*P). */
/* Lengths the split does not divide ([CP] section 7.1: pad up to a multiple
 * of the CP degree, compute, discard): the split is that of the padded
 * length S_pad = S rounded up to a multiple of P (2P for zigzag); positions
 * >= S are padding rows.  Padding is never read, never visible as a key and
 * costs no compute; a padding row of an output is written as out = 0,
 * lse = -inf (of a gradient: 0).  Natural-order tensors keep their S rows;
 * striped-order tensors hold S_pad rows (shard r, S_pad/P rows, ends in its
 * padding rows, whose contents are ignored). */
typedef enum {
    CP_LAYOUT_CONTIGUOUS = 0,
    CP_LAYOUT_ZIGZAG = 1,
    CP_LAYOUT_STRIPED = 2
} cp_layout;

/* Classification of one (query chunk, key chunk) pair of the ring. */
typedef enum { CP_PAIR_SKIP = 0, CP_PAIR_FULL = 1, CP_PAIR_DIAG = 2 } cp_pair_kind;

typedef struct {
    int32_t rank;      /* rank that owns the query chunk                        */
    int32_t step;      /* ring step t; the KV block is rank (rank - t) mod P's  */
    int32_t q_chunk;   /* chunk ids: P-way split (contiguous), 2P-way (zigzag); */
                       /* striped: the rank ids of the query and KV shards    */
    int32_t k_chunk;
    int64_t q_offset;  /* absolute first position of the query chunk            */
    int64_t k_offset;  /* absolute first position of the key chunk              */
    int64_t len_q;     /* chunk lengths                                         */
    int64_t len_k;
    int32_t kind;      /* cp_pair_kind                                          */
    int32_t reserved;  /* zero                                                  */
} cp_block_pair;

/*
 * cp_attn_block_fwd -- attention of one query chunk against one KV block at
 * given absolute sequence offsets ([HB], section "哪些运算可以直接切",
 * attention(q, k, v, causal, q_offset, k_offset)):
 *   s[i][j] = q[i].k[j] / sqrt(D); with causal != 0 key j is visible to row i
 *   iff k_offset + j <= q_offset + i (the diagonal is visible);
 *   lse[h][i] = log sum_j exp(s[i][j]) over visible j;
 *   out[i][h] = sum_j exp(s[i][j] - lse[h][i]) v[j].
 * dtype CP_BF16 (q, k, v bf16; D must be 128, Hkv * D < 2^24, Sq and Sk below
 * 2^30) runs on bf16 MFMA with float32
 * accumulation and the probabilities rounded to bf16 before the second
 * product; CP_F32 (1 <= D <= 128) runs in float32.
 * Sq == 0 is a no-op; Sk == 0 writes out = 0, lse = -inf.
 * Errors: CP_ERR_NULL, CP_ERR_SHAPE (negative sizes, Hq % Hkv != 0,
 * Hq or Hkv < 1), CP_ERR_UNSUPPORTED (D, or Hkv * D, Sq or Sk for bf16), CP_ERR_ALIGN,
 * CP_ERR_HIP.
 */
int cp_attn_block_fwd(const void *q, const void *k, const void *v, float *out, float *lse,
                      int64_t Sq, int64_t Sk, int Hq, int Hkv, int D,
                      int64_t q_offset, int64_t k_offset, int causal,
                      cp_dtype dtype, void *stream);

/*
 * cp_lse_merge -- fold two partial results over disjoint key sets into one
 * ([HB], section "Ring Attention：KV 沿环传一圈"; [SP] section 3.2):
 *   lse = log(exp(lse1) + exp(lse2)),
 *   o   = o1 * exp(lse1 - lse) + o2 * exp(lse2 - lse).
 * o* are [Sq][H][D] float32, lse* are [H][Sq] float32.  o/lse may alias
 * o1/lse1 or o2/lse2 exactly (in-place accumulation); partial overlap is not
 * allowed.  Two -inf inputs give (0, -inf).
 * Errors: CP_ERR_NULL, CP_ERR_SHAPE, CP_ERR_UNSUPPORTED (D % 4 != 0 or
 * D > 256), CP_ERR_ALIGN (16-byte alignment of o*), CP_ERR_HIP.
 */
int cp_lse_merge(const float *o1, const float *lse1, const float *o2, const float *lse2,
                 float *o, float *lse, int64_t Sq, int H, int D, void *stream);

/*
 * cp_ring_fwd -- the P-step ring schedule of [HB], section "Ring Attention：
 * KV 沿环传一圈", played by P virtual ranks on one GPU.  At step t rank r
 * holds the KV block of rank src = (r - t) mod P, attends its local queries
 * to it with the block's offsets and merges the result into its running
 * (out, lse) with the log-sum-exp rule.  With causal != 0, (query chunk,
 * key chunk) pairs whose keys all come after the queries are skipped
 * (cp_ring_plan lists them).  For the zigzag layout the KV block of a rank is
 * its two chunks; each of the rank's two query chunks attends to those of
 * them it can see.  For the striped layout ([SP] section 3.3) every step is
 * computed: rank r's local query i (position r + iP) sees local key j of
 * rank src (position src + jP) iff j <= i when src <= r and j <= i - 1 when
 * src > r, which is the causal mask at local offsets 0 and (src > r).
 * q, k, v are the whole sequence: q [S][Hq][D], k/v [S][Hkv][D], in natural
 * order (contiguous, zigzag) or striped order (striped; S_pad rows when
 * padded).  S is the real length and need not be divisible by the split.
 *   rank == -1: every rank; out [rows][Hq][D] and lse [Hq][rows] in the
 *   order of the inputs (rows = S, or S_pad for striped).
 *   0 <= rank < P: that rank's share only; out [S_pad/P][Hq][D] and lse
 *   [Hq][S_pad/P] in the rank's local row order (see cp_layout_index),
 *   padding rows (0, -inf).
 * The merge is fused into the attention epilogue; no workspace is needed.
 * Errors: as cp_attn_block_fwd, plus CP_ERR_SHAPE when P < 1, rank outside
 * [-1, P), S negative or above 2^40, or an unknown layout.
 */
int cp_ring_fwd(const void *q, const void *k, const void *v, float *out, float *lse,
                int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout, int rank,
                int causal, cp_dtype dtype, void *stream);

/*
 * Backward pass.  The pages give no algorithm for it: they measure forward
 * plus backward steps ([CP] section 4.2) and ask that gradients with context
 * parallelism match those of one card ([SP] section 5.3).  These entry
 * points compute the gradients of L = sum(dout * out) for the attention
 * defined above by the chain rule through its definition:
 *   P_ij = exp(s_ij - lse_i),        Dv_i = dout_i . out_i,
 *   dv_j = sum_i P_ij dout_i,        ds_ij = P_ij (dout_i . v_j - Dv_i),
 *   dq_i = sum_j ds_ij k_j / sqrt(D),  dk_j = sum_i ds_ij q_i / sqrt(D),
 * where lse and out are the query rows' final forward results (over every
 * key the rows see), so the block gradients of a ring add up to the
 * single-pass gradient.  KV head g receives the sum over its query heads.
 * Rows with lse = -inf contribute nothing.
 */

/*
 * cp_attn_bwd_dvec -- dvec[h][i] = sum_d dout[i][h][d] * out[i][h][d].
 * out [Sq][Hq][D] float32; dout [Sq][Hq][D] of dtype (CP_BF16 or CP_F32);
 * dvec [Hq][Sq] float32, the caller's buffer.  dvec must not overlap the
 * inputs.  Errors: CP_ERR_NULL, CP_ERR_SHAPE, CP_ERR_UNSUPPORTED (dtype, D
 * outside [1, 128]), CP_ERR_ALIGN, CP_ERR_HIP.
 */
int cp_attn_bwd_dvec(const float *out, const void *dout, float *dvec, int64_t Sq, int Hq, int D,
                     cp_dtype dtype, void *stream);

/*
 * cp_attn_block_bwd -- gradients of one query chunk against one KV block
 * with absolute offsets q_offset / k_offset (mask as cp_attn_block_fwd).
 * q, dout [Sq][Hq][D] and k, v [Sk][Hkv][D] of dtype; lse and dvec
 * [Hq][Sq] float32 (the rows' final log-sum-exp, and cp_attn_bwd_dvec of
 * their final out); dq [Sq][Hq][D], dk and dv [Sk][Hkv][D] float32.
 * accumulate == 0 overwrites dq, dk and dv; accumulate != 0 adds into them.
 * dtype CP_BF16 (D = 128, Hkv * D < 2^24, Sq and Sk below 2^30) runs on bf16
 * MFMA with float32 accumulation, P and ds rounded to bf16 before the products that take
 * them; CP_F32 (1 <= D <= 128) runs in float32.  dq, dk and dv must not
 * overlap each other or any input.
 * Errors: CP_ERR_NULL, CP_ERR_SHAPE, CP_ERR_UNSUPPORTED, CP_ERR_ALIGN,
 * CP_ERR_HIP.
 */
int cp_attn_block_bwd(const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, const float *dvec, float *dq, float *dk, float *dv,
                      int64_t Sq, int64_t Sk, int Hq, int Hkv, int D,
                      int64_t q_offset, int64_t k_offset, int causal, int accumulate,
                      cp_dtype dtype, void *stream);

/*
 * cp_ring_bwd -- the backward pass of cp_ring_fwd: every (query chunk, key
 * chunk) pair that the forward ring computes (cp_ring_plan, pairs not
 * SKIP) contributes its block gradients; dq accumulates on the query rows,
 * dk and dv on the KV block's rows (on a real ring these accumulators
 * travel with the KV block and return to its owner after P steps).
 * q, k, v: as in cp_ring_fwd (natural order, striped order for the striped
 * layout).  out, lse, dout and dq use the forward's output layout: rank ==
 * -1 the inputs' order ([S][Hq][D], [Hq][S]); 0 <= rank < P that rank's
 * local order ([S/P][Hq][D], [Hq][S/P]).  dout has dtype; out and lse are
 * float32 (cp_ring_fwd's results).  dq is overwritten.  dk and dv are
 * [rows of k][Hkv][D] float32 in the inputs' order and are overwritten with
 * the contributions of the rank(s) computed (padding rows 0).  dvec is a
 * caller-provided float32 scratch buffer of Hq * (rows of out) elements.
 * Errors: as cp_ring_fwd and cp_attn_block_bwd.
 */
int cp_ring_bwd(const void *q, const void *k, const void *v, const float *out,
                const float *lse, const void *dout, float *dq, float *dk, float *dv,
                float *dvec, int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout,
                int rank, int causal, cp_dtype dtype, void *stream);

/*
 * cp_ring_bwd_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): cp_ring_bwd with the same arguments except dvec, and the
 * same results, its dvec scratch kept in a device array of the library's
 * own.  It allocates nothing and calls no allocating routine.
 * Limit: Hq * (rows of out) <= 4194304 floats (16 MiB, e.g. 32 heads over
 * 131072 rows); a larger call returns CP_ERR_WORKSPACE before any HIP call.
 * Each GPU holds one such array (looked up on the current device at the
 * first call there, held until the process ends) and every call on that
 * GPU uses it: calls that overlap in time on one GPU (different streams or
 * host threads) race and must be ordered, e.g. on one stream.  Each call
 * rewrites every entry it reads, so nothing carries over between calls.
 * Errors: as cp_ring_bwd, plus CP_ERR_WORKSPACE.
 */
int cp_ring_bwd_noalloc(const void *q, const void *k, const void *v, const float *out,
                        const float *lse, const void *dout, float *dq, float *dk, float *dv,
                        int64_t S, int Hq, int Hkv, int D, int P, cp_layout layout, int rank,
                        int causal, cp_dtype dtype, void *stream);

/*
 * cp_seq_to_head / cp_head_to_seq -- the Ulysses layout changes of [HB],
 * section "Ulysses：在序列和头之间转置", done as local repacks: the all-to-all
 * between P ranks becomes a strided copy on one GPU.  Elements are opaque
 * (elem_bytes 2 or 4) and copied bit for bit.  Hp = H / P.
 *
 * cp_seq_to_head: x is the natural [S][H][D] tensor (all ranks' [S/P][H][D]
 * shards back to back).
 *   rank == -1: y = [P][S][Hp][D], y[p][t][j] = x[t][p*Hp + j].
 *   rank == p : y = [S][Hp][D], rank p's tensor after the all-to-all.
 * cp_head_to_seq: the inverse.
 *   rank == -1: x = [P][S][Hp][D] -> y natural [S][H][D].
 *   rank == p : x = [S][Hp][D] (rank p's head share) is written into head
 *               slice [p*Hp, (p+1)*Hp) of y [S][H][D]; the other heads of y
 *               are left untouched, so the P calls together fill y.
 * x and y must not overlap.  Errors: CP_ERR_NULL, CP_ERR_SHAPE (H % P != 0,
 * S % P != 0, rank outside [-1, P)), CP_ERR_UNSUPPORTED (elem_bytes),
 * CP_ERR_HIP.
 */
int cp_seq_to_head(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                   size_t elem_bytes, void *stream);
int cp_head_to_seq(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                   size_t elem_bytes, void *stream);

/*
 * cp_kv_seq_to_head -- seq_to_head for K and V past the KV-head limit
 * ([HB], section "练习", first exercise: with 8 KV heads Ulysses reaches
 * 8-way at most; for 16-way, copy every KV head to two ranks before the
 * all-to-all).  With P <= H it is cp_seq_to_head.  With P > H (H | P) every
 * KV head is replicated P/H times, consecutive copies, so rank p receives
 * KV head p / (P/H):
 *   rank == -1: y = [P][S][1][D], y[p][t][0] = x[t][p / (P/H)];
 *   rank == p : y = [S][1][D].
 * Elements are copied bit for bit.  Errors: as cp_seq_to_head, plus
 * CP_ERR_SHAPE when neither P | H nor H | P.
 */
int cp_kv_seq_to_head(const void *x, void *y, int64_t S, int H, int D, int P, int rank,
                      size_t elem_bytes, void *stream);

/*
 * cp_usp_fwd -- the hybrid the handbook names in its comparison of the two
 * schemes and in its GQA exercise (Ulysses inside a node, Ring Attention
 * across nodes: 32 query heads on 8 KV heads over 16 ranks as 8-way Ulysses
 * x 2-way ring), played by P = P_u * P_r virtual ranks on one GPU.
 * Rank numbering: rank = r * P_u + u, the P_u ranks of ring group r are
 * consecutive.  The sequence is split over the P_r ring groups with
 * `layout` (as cp_ring_fwd with P = P_r); inside group r its S/P_r rows, in
 * the group's local order, are cut into P_u consecutive shards.  Per head
 * share u (query heads [u*Hq/P_u, (u+1)*Hq/P_u), KV heads [u*Hkv/P_u, ...)):
 *   1. seq_to_head inside each group (the P_u-way all-to-all);
 *   2. the ring over the P_r groups on that head share (cp_ring_fwd);
 *   3. head_to_seq inside each group.
 * q [S][Hq][D], k/v [S][Hkv][D] of dtype, in natural order (striped order
 * for the striped layout), as cp_ring_fwd.
 *   rank == -1: every rank; out [S][Hq][D] and lse [Hq][S] in the inputs'
 *   order (equal to the single pass).
 *   rank == r*P_u + u: out [S/P_r][Hq][D] and lse [Hq][S/P_r] hold ring
 *   group r's rows in the group's local order (cp_layout_index with P_r);
 *   only query heads of share u are written, so the P_u ranks of a group
 *   together fill them (as cp_head_to_seq with a rank).  On one GPU the
 *   share's key/value head slices of every group are copied too: the
 *   group's own by the all-to-all, the others standing for the blocks the
 *   ring delivers.
 * workspace: caller-provided device memory, 256-byte aligned, of the size
 * cp_usp_fwd_workspace returns (head shares of q, k, v for the whole
 * sequence, and the ring's float32 output); reused across head shares, so
 * calls on one workspace must be ordered (same stream).
 * A ring split that does not divide S is padded as in cp_ring_fwd (with
 * P_r): q, k, v then hold rows_in rows (S, or the padded length in striped
 * order) and out/lse the padded output rows, padding rows (0, -inf); a
 * group's Ulysses shards are then of unequal length, which the copies on
 * one GPU never see.
 * Errors: as cp_ring_fwd (with P_r), plus CP_ERR_SHAPE when P_u < 1, rank
 * outside [-1, P_u*P_r), P_u not dividing Hkv (every Ulysses rank needs whole
 * KV heads); CP_ERR_NULL / CP_ERR_WORKSPACE /
 * CP_ERR_ALIGN for a missing, short or misaligned workspace or one that
 * overlaps the tensors.
 */
int cp_usp_fwd_workspace(int64_t S, int Hq, int Hkv, int D, int P_u, int P_r,
                         cp_layout layout, int rank, cp_dtype dtype, size_t *bytes);
int cp_usp_fwd(const void *q, const void *k, const void *v, float *out, float *lse,
               int64_t S, int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout,
               int rank, int causal, cp_dtype dtype, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * cp_usp_bwd -- the backward pass of cp_usp_fwd (no algorithm on the pages;
 * the plainest reading): per head share u, the head-share copies of q (the
 * rows computed here), k, v (every row), dout and out (output rows), the
 * ring backward over the P_r groups on that share (cp_ring_bwd), and the
 * copies of dq, dk, dv back into head share u.
 * q, k, v as cp_usp_fwd; out, lse, dout and dq in cp_usp_fwd's output
 * layout (rank == -1: [S] rows in the inputs' order; a rank: its ring
 * group's S/P_r rows in local order); out and lse are cp_usp_fwd's float32
 * results with every head written (rank == -1, or all P_u ranks of the
 * group); dout has dtype.  dq [rows][Hq][D], dk and dv [S][Hkv][D] float32:
 * rank == -1 writes the whole gradient; a rank writes only head share u of
 * dq and of dk, dv, where dk and dv hold that rank's contributions (its
 * group's queries), the other heads untouched.
 * workspace: 256-byte aligned, cp_usp_bwd_workspace bytes; calls sharing
 * one workspace must be ordered.
 * Errors: as cp_usp_fwd and cp_ring_bwd.
 */
int cp_usp_bwd_workspace(int64_t S, int Hq, int Hkv, int D, int P_u, int P_r,
                         cp_layout layout, int rank, cp_dtype dtype, size_t *bytes);
int cp_usp_bwd(const void *q, const void *k, const void *v, const float *out,
               const float *lse, const void *dout, float *dq, float *dk, float *dv,
               int64_t S, int Hq, int Hkv, int D, int P_u, int P_r, cp_layout layout,
               int rank, int causal, cp_dtype dtype, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * cp_layout_index -- host only, synchronous.  idx[j] (j < S/P) receives the
 * natural sequence position of rank `rank`'s local row j:
 *   contiguous: rank*S/P + j;
 *   zigzag (C = S/(2P)): j < C ? rank*C + j : (2P-1-rank)*C + (j - C);
 *   striped: rank + j*P.
 * idx is a host array of S_pad/P int32 (S_pad below 2^31); entries >= S
 * are padding rows.
 * Errors: CP_ERR_NULL, CP_ERR_SHAPE.
 */
int cp_layout_index(cp_layout layout, int64_t S, int P, int rank, int32_t *idx);

/*
 * cp_ring_plan -- host only, synchronous.  Lists every (rank, step, query
 * chunk, key chunk) pair the ring visits, in order rank, step, query chunk
 * in local order, key chunk in local order, each classified SKIP (causal and
 * the key chunk comes after the query chunk), DIAG (causal and the same
 * chunk) or FULL.  rank == -1 lists all ranks.  Contiguous: one pair per
 * step (P-way chunks); zigzag: four pairs per step (2P-way chunks);
 * striped: one pair per step, DIAG when causal (every shard holds early and
 * late positions), with the local offsets q_offset = 0 and k_offset =
 * (k_chunk > q_chunk) that its mask uses.  When S is padded, len_q and
 * len_k count the real rows of the chunks and a pair with none is SKIP.
 * *n_pairs is the capacity of `pairs` on entry and the number of pairs on
 * return; pairs == NULL only queries the count.
 * Errors: CP_ERR_NULL (n_pairs), CP_ERR_SHAPE, CP_ERR_CAPACITY (the needed
 * count is still written to *n_pairs).
 */
int cp_ring_plan(int64_t S, int P, cp_layout layout, int rank, int causal,
                 cp_block_pair *pairs, int *n_pairs);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char *cp_last_error(void);

/*
 * Kernel timing (measurement support).  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on the launch
 * stream.  cp_timing_read waits for the recorded events, adds their elapsed
 * times to the totals of the given kernel kind and returns the totals since
 * the last reset.  Calls are serialised by a mutex; timing adds two event
 * records per launch.
 */
typedef enum {
    CP_KERNEL_ATTN_BF16 = 0,
    CP_KERNEL_ATTN_F32 = 1,
    CP_KERNEL_MERGE = 2,
    CP_KERNEL_PERMUTE = 3,
    CP_KERNEL_BWD_BF16 = 4,   /* backward dq and dk/dv kernels, bf16 */
    CP_KERNEL_BWD_F32 = 5,    /* backward dq and dk/dv kernels, float32 */
    CP_KERNEL_BWD_DVEC = 6
} cp_kernel_kind;

int cp_timing_enable(int enable);
int cp_timing_reset(void);
int cp_timing_read(cp_kernel_kind kind, double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
