// rr_api.hip -- the C ABI of librr (declared in include/rr.h).
//
// Host-side argument checks, workspace carving and the launch sequence of
// each stage.  No allocation, no synchronisation: every kernel is enqueued on
// the caller's stream.
#include <math.h>

#include <atomic>

#include "rr.h"
#include "rr_internal.h"

using namespace rr;

namespace {

constexpr int kMaxBlocks = 4096;  // longest Top-tau row the selection kernel holds (64 per lane)
constexpr int kMaxHeads = 1024;   // query heads per call

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int check_shape(int L, int Hq, int Hkv, int d, int B, int S, bool need_S) {
    if (L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || B <= 0) return RR_E_SHAPE;
    if (Hq % Hkv != 0) return RR_E_SHAPE;
    // Per-lane copy offsets inside one tile are 32-bit (a few hundred rows of
    // S * heads * d elements): bound the head count.
    if (Hq > kMaxHeads) return RR_E_UNSUPPORTED;
    if (need_S) {
        if (S <= 0 || S > B || B % S != 0 || L % S != 0) return RR_E_SHAPE;
        if (!is_pow2(S)) return RR_E_UNSUPPORTED;
    }
    if (d != 64 && d != 128) return RR_E_UNSUPPORTED;
    if (B != 64 && B != 128) return RR_E_UNSUPPORTED;
    if ((L + B - 1) / B > kMaxBlocks) return RR_E_UNSUPPORTED;
    // Element offsets are formed in 64-bit; the largest tensor must still fit
    // the 32-bit grid decode of the kernels.
    if ((long long)L * Hq > (1ll << 40)) return RR_E_UNSUPPORTED;
    return RR_OK;
}

int check_tau(float tau) {
    if (isnan(tau) || !(tau > 0.f) || tau > 1.f) return RR_E_TAU;
    return RR_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int run_estimate(const uint16_t *Q, const uint16_t *K, const Shape &s, float *A, void *ws,
                 hipStream_t st) {
    EstimateWs w = carve_estimate(s, ws);
    if (launch_pool_k(K, s, w.kplanes, st) != hipSuccess) return RR_E_HIP;
    if (launch_score(Q, s, w, st) != hipSuccess) return RR_E_HIP;
    if (launch_softmax_pool(s, w, A, st) != hipSuccess) return RR_E_HIP;
    return RR_OK;
}

int run_attn(const uint16_t *Q, const uint16_t *K, const uint16_t *V, const Shape &s,
             const int32_t *counts, const int32_t *block_idx, void *O, int o_dtype, void *ws,
             hipStream_t st) {
    uint16_t *Vt = (uint16_t *)ws;
    unsigned *counter = (unsigned *)((char *)ws + attn_vt_bytes(s));
    if (launch_transpose_v(V, s, Vt, counter, st) != hipSuccess) return RR_E_HIP;
    if (launch_block_sparse_fa(Q, K, Vt, counter, s, counts, block_idx, O, o_dtype == RR_OUT_F32, st) !=
        hipSuccess)
        return RR_E_HIP;
    return RR_OK;
}

}  // namespace

namespace rr {

// Compute units of the current device (queried once per device; threads
// that race on the first query store the same value).
int device_cu_count() {
    static std::atomic<int> cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int check_prefill_args(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                       int Hkv, int d, int B, int S, float tau, const void *O, int o_dtype,
                       const int32_t *counts, const int32_t *block_idx) {
    if (!Q || !K || !V || !O || !counts || !block_idx) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, S, true);
    if (rc != RR_OK) return rc;
    rc = check_tau(tau);
    if (rc != RR_OK) return rc;
    if (o_dtype != RR_OUT_BF16 && o_dtype != RR_OUT_F32) return RR_E_UNSUPPORTED;
    return RR_OK;
}

int run_prefill(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
                int d, int B, int S, float tau, void *O, int o_dtype, int32_t *counts,
                int32_t *block_idx, void *ws, void *stream) {
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    hipStream_t st = as_stream(stream);
    float *A = (float *)ws;
    void *rest = (char *)ws + align_up((size_t)s.Hq * s.nb * s.nb * 4);
    int rc = run_estimate(Q, K, s, A, rest, st);
    if (rc != RR_OK) return rc;
    if (launch_topk_tau(A, s, tau, counts, block_idx, st) != hipSuccess) return RR_E_HIP;
    return run_attn(Q, K, V, s, counts, block_idx, O, o_dtype, rest, st);
}

}  // namespace rr

extern "C" {

const char *rr_status_str(int status) {
    switch (status) {
        case RR_OK: return "RR_OK";
        case RR_E_NULL: return "RR_E_NULL: a required pointer is NULL";
        case RR_E_SHAPE: return "RR_E_SHAPE: invalid sizes (L, heads, d, B, S)";
        case RR_E_TAU: return "RR_E_TAU: tau must lie in (0, 1]";
        case RR_E_WORKSPACE: return "RR_E_WORKSPACE: workspace too small";
        case RR_E_UNSUPPORTED: return "RR_E_UNSUPPORTED: d, B or S not compiled, or too many blocks";
        case RR_E_HIP: return "RR_E_HIP: a HIP launch failed";
        default: return "RR_E_UNKNOWN";
    }
}

int rr_abi_version(void) { return 1; }

size_t rr_estimate_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S) {
    if (check_shape(L, Hq, Hkv, d, B, S, true) != RR_OK) return 0;
    return estimate_ws_bytes(make_shape(L, Hq, Hkv, d, B, S));
}

size_t rr_sparse_attn_workspace_bytes(int L, int Hq, int Hkv, int d, int B) {
    if (check_shape(L, Hq, Hkv, d, B, 1, false) != RR_OK) return 0;
    return attn_ws_bytes(make_shape(L, Hq, Hkv, d, B, 1));
}

size_t rr_prefill_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S) {
    if (check_shape(L, Hq, Hkv, d, B, S, true) != RR_OK) return 0;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    const size_t a = align_up((size_t)s.Hq * s.nb * s.nb * 4);
    const size_t e = estimate_ws_bytes(s), t = attn_ws_bytes(s);
    return a + (e > t ? e : t);
}

size_t rr_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S) {
    if (check_shape(L, Hq, Hkv, d, B, S, true) != RR_OK) return 0;
    // The prefill size covers rr_estimate, rr_xattn_estimate (same layout),
    // the materialised estimate (its pooled-key planes only) and
    // rr_sparse_attn; the rescue branch has its own layout.
    const size_t p = rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S);
    const size_t r = rescue_ws_bytes(make_shape(L, Hq, Hkv, d, B, S));
    return p > r ? p : r;
}

int rr_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B, int S,
                float *block_scores, void *ws, size_t ws_bytes, void *stream) {
    if (!Q || !K || !block_scores || !ws) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, S, true);
    if (rc != RR_OK) return rc;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    if (ws_bytes < estimate_ws_bytes(s)) return RR_E_WORKSPACE;
    return run_estimate(Q, K, s, block_scores, ws, as_stream(stream));
}

long long rr_stride_scores_count(int L, int Hq, int Hkv, int d, int B, int S) {
    if (check_shape(L, Hq, Hkv, d, B, S, true) != RR_OK || B / S < 4) return 0;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    return (long long)s.Hq * score_elems_per_head(s);
}

size_t rr_estimate_materialized_workspace_bytes(int L, int Hq, int Hkv, int d, int B, int S) {
    if (check_shape(L, Hq, Hkv, d, B, S, true) != RR_OK || B / S < 4) return 0;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    return align_up((size_t)3 * s.Hkv * s.ns * s.d * 2);  // the pooled-key planes
}

int rr_estimate_materialized(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d,
                             int B, int S, float *stride_scores, float *block_scores, void *ws,
                             size_t ws_bytes, void *stream) {
    if (!Q || !K || !stride_scores || !block_scores || !ws) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, S, true);
    if (rc != RR_OK) return rc;
    if (B / S < 4) return RR_E_UNSUPPORTED;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    if (ws_bytes < rr_estimate_materialized_workspace_bytes(L, Hq, Hkv, d, B, S)) return RR_E_WORKSPACE;
    EstimateWs w;
    w.kplanes = (uint16_t *)ws;
    w.stats = nullptr;
    w.rowstat = nullptr;
    hipStream_t st = as_stream(stream);
    if (launch_pool_k(K, s, w.kplanes, st) != hipSuccess) return RR_E_HIP;
    if (launch_score_store(Q, s, w, stride_scores, st) != hipSuccess) return RR_E_HIP;
    if (launch_pool_scores(s, stride_scores, block_scores, st) != hipSuccess) return RR_E_HIP;
    return RR_OK;
}

int rr_select(const float *block_scores, int Hq, int L, int B, float tau, int32_t *counts,
              int32_t *block_idx, void *stream) {
    if (!block_scores || !counts || !block_idx) return RR_E_NULL;
    if (L <= 0 || Hq <= 0 || B <= 0) return RR_E_SHAPE;
    if (Hq > kMaxHeads) return RR_E_UNSUPPORTED;
    if ((L + B - 1) / B > kMaxBlocks) return RR_E_UNSUPPORTED;
    int rc = check_tau(tau);
    if (rc != RR_OK) return rc;
    const Shape s = make_shape(L, Hq, Hq, 64, B, 1);
    if (launch_topk_tau(block_scores, s, tau, counts, block_idx, as_stream(stream)) != hipSuccess)
        return RR_E_HIP;
    return RR_OK;
}

int rr_sparse_attn(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
                   int d, int B, const int32_t *counts, const int32_t *block_idx, void *O,
                   int o_dtype, void *ws, size_t ws_bytes, void *stream) {
    if (!Q || !K || !V || !counts || !block_idx || !O || !ws) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, 1, false);
    if (rc != RR_OK) return rc;
    if (o_dtype != RR_OUT_BF16 && o_dtype != RR_OUT_F32) return RR_E_UNSUPPORTED;
    const Shape s = make_shape(L, Hq, Hkv, d, B, 1);
    if (ws_bytes < attn_ws_bytes(s)) return RR_E_WORKSPACE;
    return run_attn(Q, K, V, s, counts, block_idx, O, o_dtype, ws, as_stream(stream));
}

int rr_prefill(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq, int Hkv,
               int d, int B, int S, float tau, void *O, int o_dtype, int32_t *counts,
               int32_t *block_idx, void *ws, size_t ws_bytes, void *stream) {
    if (!ws) return RR_E_NULL;
    const int rc = rr::check_prefill_args(Q, K, V, L, Hq, Hkv, d, B, S, tau, O, o_dtype, counts,
                                          block_idx);
    if (rc != RR_OK) return rc;
    if (ws_bytes < rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S)) return RR_E_WORKSPACE;
    return rr::run_prefill(Q, K, V, L, Hq, Hkv, d, B, S, tau, O, o_dtype, counts, block_idx, ws,
                           stream);
}

int rr_mask_quality(const int32_t *counts, const int32_t *block_idx, const int32_t *ref_counts,
                    const int32_t *ref_block_idx, const float *mass, int Hq, int L, int B,
                    float *rows, double *totals, void *stream) {
    if (!counts || !block_idx || !ref_counts || !ref_block_idx || !mass || !rows || !totals)
        return RR_E_NULL;
    if (L <= 0 || Hq <= 0 || B <= 0) return RR_E_SHAPE;
    if (Hq > kMaxHeads) return RR_E_UNSUPPORTED;
    const int nb = (L + B - 1) / B;
    if (nb > kMaxBlocks) return RR_E_UNSUPPORTED;
    if (launch_mask_quality(counts, block_idx, ref_counts, ref_block_idx, mass, Hq, nb, rows,
                            totals, as_stream(stream)) != hipSuccess)
        return RR_E_HIP;
    return RR_OK;
}

int rr_xattn_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                      int S, int average, float *block_scores, void *ws, size_t ws_bytes,
                      void *stream) {
    if (!Q || !K || !block_scores || !ws) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, S, true);
    if (rc != RR_OK) return rc;
    const int c = B / S;
    if (c != 8 && c != 16 && c != 32) return RR_E_UNSUPPORTED;
    const Shape s = make_shape(L, Hq, Hkv, d, B, S);
    if (ws_bytes < estimate_ws_bytes(s)) return RR_E_WORKSPACE;
    const EstimateWs w = carve_estimate(s, ws);
    hipStream_t st = as_stream(stream);
    if (launch_xscore(Q, K, s, average != 0, w, st) != hipSuccess) return RR_E_HIP;
    if (launch_softmax_pool(s, w, block_scores, st) != hipSuccess) return RR_E_HIP;
    return RR_OK;
}

size_t rr_rescue_workspace_bytes(int L, int Hq, int Hkv, int d, int B) {
    if (check_shape(L, Hq, Hkv, d, B, 1, false) != RR_OK) return 0;
    return rescue_ws_bytes(make_shape(L, Hq, Hkv, d, B, 1));
}

int rr_rescue_estimate(const uint16_t *Q, const uint16_t *K, int L, int Hq, int Hkv, int d, int B,
                       float *block_scores, void *ws, size_t ws_bytes, void *stream) {
    if (!Q || !K || !block_scores || !ws) return RR_E_NULL;
    int rc = check_shape(L, Hq, Hkv, d, B, 1, false);
    if (rc != RR_OK) return rc;
    const Shape s = make_shape(L, Hq, Hkv, d, B, 1);
    if (ws_bytes < rescue_ws_bytes(s)) return RR_E_WORKSPACE;
    if (launch_rescue(Q, K, s, (float *)ws, block_scores, as_stream(stream)) != hipSuccess)
        return RR_E_HIP;
    return RR_OK;
}

int rr_merge_masks(const int32_t *counts_a, const int32_t *block_idx_a, const int32_t *counts_b,
                   const int32_t *block_idx_b, int Hq, int L, int B, int32_t *counts,
                   int32_t *block_idx, void *stream) {
    if (!counts_a || !block_idx_a || !counts_b || !block_idx_b || !counts || !block_idx)
        return RR_E_NULL;
    if (L <= 0 || Hq <= 0 || B <= 0) return RR_E_SHAPE;
    if (Hq > kMaxHeads) return RR_E_UNSUPPORTED;
    const int nb = (L + B - 1) / B;
    if (nb > kMaxBlocks) return RR_E_UNSUPPORTED;
    if (launch_merge_lists(counts_a, block_idx_a, counts_b, block_idx_b, Hq, nb, counts,
                           block_idx, as_stream(stream)) != hipSuccess)
        return RR_E_HIP;
    return RR_OK;
}

}  // extern "C"
