// rr_internal.h -- host-side layout helpers and kernel launchers of librr.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rr {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shape of one call, with the derived sizes every stage uses.
struct Shape {
    int L, Hq, Hkv, d, B, S;
    int G;    // query heads per kv-head
    int nb;   // ceil(L / B) blocks
    int ns;   // L / S strides
    int c;    // B / S strides per block
    int c_last;        // strides in the last block
    long long P;       // packed (row, key-block) entries per head: c * nb(nb+1)/2
                       // (a short last block keeps the full stride c)
};

inline Shape make_shape(int L, int Hq, int Hkv, int d, int B, int S) {
    Shape s;
    s.L = L; s.Hq = Hq; s.Hkv = Hkv; s.d = d; s.B = B; s.S = S;
    s.G = Hq / Hkv;
    s.nb = (L + B - 1) / B;
    s.ns = L / S;
    s.c = B / S;
    s.c_last = s.ns - (s.nb - 1) * s.c;
    s.P = (long long)s.c * s.nb * (s.nb + 1) / 2;
    return s;
}

// Estimation workspace: pooled-key planes, per-(row, key-block) (max, sum)
// pairs and per-row (max, sum) pairs.
struct EstimateWs {
    uint16_t *kplanes;  // [3][Hkv][ns][d] bf16 (hi, mid, lo split of the fp32 mean)
    float2 *stats;      // [Hq][P] packed: block-row I owns c*(I+1) entries, J-major
    float2 *rowstat;    // [Hq][ns]
};

inline size_t estimate_ws_bytes(const Shape &s) {
    return align_up((size_t)3 * s.Hkv * s.ns * s.d * 2) + align_up((size_t)s.Hq * s.P * 8) +
           align_up((size_t)s.Hq * s.ns * 8);
}

inline EstimateWs carve_estimate(const Shape &s, void *ws) {
    EstimateWs w;
    char *p = (char *)ws;
    w.kplanes = (uint16_t *)p;
    p += align_up((size_t)3 * s.Hkv * s.ns * s.d * 2);
    w.stats = (float2 *)p;
    p += align_up((size_t)s.Hq * s.P * 8);
    w.rowstat = (float2 *)p;
    return w;
}

// Stored stride scores of the materialised estimate: per head, block-row I
// owns c rows of (I+1)c strides, i.e. c * P floats in all.
inline long long score_elems_per_head(const Shape &s) { return (long long)s.c * s.P; }

// Attention workspace: V transposed to [Hkv][d][nb*B] (zero-padded tail),
// then the work counter of the attention kernel (one 32-bit word in its own
// 256-byte slot).
inline size_t attn_vt_bytes(const Shape &s) { return align_up((size_t)s.Hkv * s.d * s.nb * s.B * 2); }
inline size_t attn_ws_bytes(const Shape &s) { return attn_vt_bytes(s) + kAlign; }

// rr_prefill's host-side argument checks (everything but the workspace) and
// its launch sequence on a workspace of at least rr_prefill_workspace_bytes;
// both return an rr_status code.
int check_prefill_args(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                       int Hkv, int d, int B, int S, float tau, const void *O, int o_dtype,
                       const int32_t *counts, const int32_t *block_idx);
int run_prefill(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
                int d, int B, int S, float tau, void *O, int o_dtype, int32_t *counts,
                int32_t *block_idx, void *ws, void *stream);

// Compute units of the current device (queried once per device).
int device_cu_count();

// Launchers (enqueue on `stream`, return the launch error).
hipError_t launch_pool_k(const uint16_t *K, const Shape &s, uint16_t *kplanes, hipStream_t st);
hipError_t launch_score(const uint16_t *Q, const Shape &s, const EstimateWs &w, hipStream_t st);
hipError_t launch_softmax_pool(const Shape &s, const EstimateWs &w, float *A, hipStream_t st);
hipError_t launch_score_store(const uint16_t *Q, const Shape &s, const EstimateWs &w, float *scores,
                              hipStream_t st);
hipError_t launch_pool_scores(const Shape &s, const float *scores, float *A, hipStream_t st);
hipError_t launch_topk_tau(const float *A, const Shape &s, float tau, int32_t *counts,
                           int32_t *block_idx, hipStream_t st);
hipError_t launch_transpose_v(const uint16_t *V, const Shape &s, uint16_t *Vt, unsigned *counter,
                              hipStream_t st);
hipError_t launch_block_sparse_fa(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt,
                                  unsigned *counter,
                                  const Shape &s, const int32_t *counts, const int32_t *block_idx,
                                  void *O, bool out_f32, hipStream_t st);
hipError_t launch_xscore(const uint16_t *Q, const uint16_t *K, const Shape &s, bool average,
                         const EstimateWs &w, hipStream_t st);
// Rescue workspace: block centroids of Q and K (fp32) and key-block radii.
inline size_t rescue_ws_bytes(const Shape &s) {
    return align_up(((size_t)(s.Hq + s.Hkv) * s.nb * s.d + (size_t)s.Hkv * s.nb) * 4);
}
hipError_t launch_rescue(const uint16_t *Q, const uint16_t *K, const Shape &s, float *ws,
                         float *A, hipStream_t st);
hipError_t launch_merge_lists(const int32_t *ca, const int32_t *ia, const int32_t *cb,
                              const int32_t *ib, int Hq, int nb, int32_t *co, int32_t *io,
                              hipStream_t st);
hipError_t launch_mask_quality(const int32_t *counts, const int32_t *block_idx,
                               const int32_t *ref_counts, const int32_t *ref_idx,
                               const float *mass, int Hq, int nb, float *rows, double *totals,
                               hipStream_t st);

}  // namespace rr
