// cp_kernels.h -- internal interface between the host library (cp_api.cpp)
// and the HIP kernels.  Not part of the public C-ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

// One contiguous run of keys: rows [row0, row0 + len) of k and v, whose
// first row sits at absolute sequence position pos0.
struct KvSeg {
    int64_t row0;
    int64_t pos0;
    int64_t len;
};

// One contiguous run of query rows and the key runs it attends to in this
// launch.  Rows [row0, row0 + len) of q sit at absolute positions
// pos0, pos0 + 1, ...; their results go to rows out_row0.. of out/lse.
// merge == 0 writes the block result; merge == 1 folds it into the
// (out, lse) already stored there with the log-sum-exp rule.
struct QSeg {
    int64_t row0;
    int64_t pos0;
    int64_t len;
    int64_t out_row0;
    int32_t n_kv;
    int32_t merge;
    KvSeg kv[2];
};

constexpr int kMaxQSegs = 16;

struct AttnLaunch {
    const void *q;
    const void *k;
    const void *v;
    float *out;
    float *lse;
    int64_t lse_ld;   // row count of the [Hq][lse_ld] lse matrix
    int Hq;
    int Hkv;
    int D;
    int causal;
    int n_q;
    QSeg qs[kMaxQSegs];
};

// Each launcher computes its own tiling and returns hipGetLastError().
hipError_t launch_attn_bf16(const AttnLaunch &a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnLaunch &a, hipStream_t stream);
hipError_t launch_lse_merge(const float *o1, const float *lse1, const float *o2,
                            const float *lse2, float *o, float *lse, int64_t Sq, int H,
                            int D, hipStream_t stream);

// Strided unit copy used by both Ulysses repacks: for u in [0, n_units)
// copies unit_bytes bytes from src + src_off(u) to dst + dst_off(u), where
// off(u) = base + (u / per) * stride_a + (u % per) * stride_b (bytes).
struct UnitCopy {
    const void *src;
    void *dst;
    int64_t n_units;
    int64_t unit_bytes;
    int64_t per;
    int64_t src_base, src_a, src_b;
    int64_t dst_base, dst_a, dst_b;
};
hipError_t launch_unit_copy(const UnitCopy &c, hipStream_t stream);

// Backward of one (query chunk, KV block) pair.  q, dout: rows [0, Sq) of
// [Sq][Hq][D]; k, v: rows [0, Sk) of [Sk][Hkv][D]; lse and dvec: columns
// [0, Sq) of [Hq][ld] matrices (ld = stat_ld); dq [Sq][Hq][D], dk and dv
// [Sk][Hkv][D] float32, added into when accumulate != 0.
struct BwdLaunch {
    const void *q;
    const void *k;
    const void *v;
    const void *dout;
    const float *lse;
    const float *dvec;
    int64_t stat_ld;
    float *dq;
    float *dk;
    float *dv;
    int64_t Sq;
    int64_t Sk;
    int Hq;
    int Hkv;
    int D;
    int causal;
    int accumulate;
    int64_t q_offset;
    int64_t k_offset;
};
// dvec[h * ld + i] = sum_d dout[i][h][d] * out[i][h][d]; dout bf16 when
// dout_bf16 != 0, else float32.
hipError_t launch_bwd_dvec(const float *out, const void *dout, int dout_bf16, float *dvec,
                           int64_t ld, int64_t Sq, int Hq, int D, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdLaunch &b, hipStream_t stream);
// p[0, n) = 0 (a kernel, so that the library records no memset)
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);
// p[r * ld + c] = value for r < n_rows, c < n_cols.
hipError_t launch_fill_2d(float *p, int64_t ld, int64_t n_rows, int64_t n_cols, float value,
                          hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdLaunch &b, hipStream_t stream);
// The two halves of launch_bwd_bf16: dq of one block; dk/dv of n blocks
// (n = 1 or 2) in one launch, which requires their dk and dv rows to be
// disjoint (the blocks' units run concurrently).
hipError_t launch_bwd_bf16_dq(const BwdLaunch &b, hipStream_t stream);
hipError_t launch_bwd_bf16_dkdv(const BwdLaunch *bs, int n, hipStream_t stream);
// Workgroups (key-tile units) of one block's dk/dv launch.
int64_t bwd_bf16_dkdv_units(const BwdLaunch &b);

// The library's device scratch array (16 MiB of floats per GPU, held from
// the code object's load until the process ends): *ptr receives its address
// on the current device.  Calls on one device share the array.
constexpr int64_t kScratchFloats = (int64_t)1 << 22;
hipError_t scratch_floats(float **ptr);

}  // namespace cpattn
