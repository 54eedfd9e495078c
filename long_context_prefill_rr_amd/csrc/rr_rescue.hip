// rr_rescue.hip -- RBS-style rescue branch and the union of two masks.
//
// RBS-Attention page (abstract and method summary): a block centroid can
// hide one highly relevant key among many irrelevant ones; a rescue branch
// built on the maximum key-block radius flags the blocks at risk, is
// thresholded on its own, and its mask is combined with the base branch's.
// Rescue logit of (query block I, key block J <= I) for query head h:
//   u = (1/sqrt(d)) * (qc_I . kc_J + ||qc_I|| * r_J)
// with qc_I the mean query of block I, kc_J the mean key of block J
// (kv-head g(h)) and r_J = max_{n in J} ||K[n] - kc_J||: the largest logit
// the mean query can reach against a key of block J.  Scores are the softmax
// of u over J <= I, so rr_select applies the same Top-tau rule to them.
//
// rr_block_centroids: one work-group per (head, block): column means over
//   the block's tokens, then (keys only) the largest distance to the mean.
// rr_rescue_softmax: one work-group per (block-row I, head h): u for
//   J <= I in LDS, then a max / sum-of-exp softmax, written as one row.
// rr_merge_lists: one work-group per (head, block-row): the two lists'
//   blocks as an LDS bitmap, compacted in ascending order.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

constexpr int kRescueMaxNb = 4096;

// X [L][H][D] bf16 -> cen [H][nb][D] fp32 (mean of block b's tokens) and, if
// rad is given, rad [H][nb] = max over the tokens of ||x - mean||_2.
template <int D>
__global__ __launch_bounds__(256) void rr_block_centroids(const uint16_t *__restrict__ X, int L,
                                                          int H, int B, int nb,
                                                          float *__restrict__ cen,
                                                          float *__restrict__ rad) {
    __shared__ float c[D];
    __shared__ float red[4];
    const int b = blockIdx.x, hh = blockIdx.y;
    const int t0 = b * B, t1 = min(L, t0 + B);
    const int tid = threadIdx.x;
    if (tid < D) {
        float s = 0.f;
        for (int t = t0; t < t1; ++t) s += bf16_to_f32(X[((size_t)t * H + hh) * D + tid]);
        c[tid] = s / (float)(t1 - t0);
        cen[((size_t)hh * nb + b) * D + tid] = c[tid];
    }
    if (rad == nullptr) return;
    __syncthreads();
    // Each wave takes tokens t0 + wid, t0 + wid + 4, ...; its lanes cover
    // the D elements (D / 64 each) and sum the squared differences.
    const int wid = tid >> 6, lane = tid & 63;
    float best = 0.f;
    for (int t = t0 + wid; t < t1; t += 4) {
        float s2 = 0.f;
#pragma unroll
        for (int k = lane; k < D; k += kWave) {
            const float e = bf16_to_f32(X[((size_t)t * H + hh) * D + k]) - c[k];
            s2 = fmaf(e, e, s2);
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) s2 += xor_lane(s2, o);
        best = fmaxf(best, s2);
    }
    if (lane == 0) red[wid] = best;
    __syncthreads();
    if (tid == 0) {
        const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        rad[(size_t)hh * nb + b] = sqrtf(m);
    }
}

// One row (h, I): A[h][I][J] = softmax_{J <= I}(u), zeros for J > I.  The
// logits are kept in log2 units (scale = log2(e)/sqrt(d)).
template <int D>
__global__ __launch_bounds__(256) void rr_rescue_softmax(const float *__restrict__ qcen,
                                                         const float *__restrict__ kcen,
                                                         const float *__restrict__ krad, int Hq,
                                                         int Hkv, int nb, float scale,
                                                         float *__restrict__ A) {
    __shared__ float q[D];
    __shared__ float u[kRescueMaxNb];
    __shared__ float red[8];
    const int I = blockIdx.x, h = blockIdx.y, g = h / (Hq / Hkv);
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    if (tid < D) q[tid] = qcen[((size_t)h * nb + I) * D + tid];
    __syncthreads();
    float qn2 = 0.f;
#pragma unroll 4
    for (int k = 0; k < D; ++k) qn2 = fmaf(q[k], q[k], qn2);
    const float qn = sqrtf(qn2);
    float mx = -INFINITY;
    for (int J = tid; J <= I; J += 256) {
        const float4 *kc = reinterpret_cast<const float4 *>(kcen + ((size_t)g * nb + J) * D);
        float dot = 0.f;
#pragma unroll 8
        for (int k4 = 0; k4 < D / 4; ++k4) {
            const float4 v = kc[k4];
            dot = fmaf(q[4 * k4], v.x, dot);
            dot = fmaf(q[4 * k4 + 1], v.y, dot);
            dot = fmaf(q[4 * k4 + 2], v.z, dot);
            dot = fmaf(q[4 * k4 + 3], v.w, dot);
        }
        const float x = scale * fmaf(qn, krad[(size_t)g * nb + J], dot);
        u[J] = x;
        mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) mx = fmaxf(mx, xor_lane(mx, o));
    if (lane == 0) red[wid] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float z = 0.f;
    for (int J = tid; J <= I; J += 256) {
        const float e = fast_exp2(u[J] - mx);
        u[J] = e;
        z += e;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) z += xor_lane(z, o);
    __syncthreads();
    if (lane == 0) red[4 + wid] = z;
    __syncthreads();
    const float inv = 1.f / (red[4] + red[5] + red[6] + red[7]);
    float *out = A + ((size_t)h * nb + I) * nb;
    for (int J = tid; J < nb; J += 256) out[J] = (J <= I) ? u[J] * inv : 0.f;
}

// Union of two block lists per (h, I): counts_out / idx_out in the layout of
// rr_select (ascending, -1 after the count).  Entries outside 0..I or past a
// list's count are ignored.
__global__ __launch_bounds__(256) void rr_merge_lists(const int32_t *__restrict__ ca,
                                                      const int32_t *__restrict__ ia,
                                                      const int32_t *__restrict__ cb,
                                                      const int32_t *__restrict__ ib, int nb,
                                                      int32_t *__restrict__ co,
                                                      int32_t *__restrict__ io) {
    __shared__ uint32_t bits[kRescueMaxNb / 32];
    __shared__ int part[4];
    const int I = blockIdx.x, h = blockIdx.y;
    const size_t row = (size_t)h * nb + I;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int nw = (nb + 31) >> 5;
    for (int i = tid; i < nw; i += 256) bits[i] = 0u;
    __syncthreads();
    const int na = min(max(ca[row], 0), nb), nbb = min(max(cb[row], 0), nb);
    for (int k = tid; k < na; k += 256) {
        const int J = ia[row * nb + k];
        if ((unsigned)J <= (unsigned)I) atomicOr(&bits[J >> 5], 1u << (J & 31));
    }
    for (int k = tid; k < nbb; k += 256) {
        const int J = ib[row * nb + k];
        if ((unsigned)J <= (unsigned)I) atomicOr(&bits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    // Thread tid owns blocks [tid*E, tid*E + E); prefix sums give positions.
    const int E = (nb + 255) / 256;
    const int j0 = tid * E;
    int cnt = 0;
    for (int e = 0; e < E; ++e) {
        const int J = j0 + e;
        if (J < nb && ((bits[J >> 5] >> (J & 31)) & 1u)) ++cnt;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) part[wid] = incl;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wid; ++w) pre += part[w];
    int pos = pre + incl - cnt;
    int32_t *out = io + row * nb;
    for (int e = 0; e < E; ++e) {
        const int J = j0 + e;
        if (J < nb && ((bits[J >> 5] >> (J & 31)) & 1u)) out[pos++] = J;
    }
    const int total = part[0] + part[1] + part[2] + part[3];
    for (int k = total + tid; k < nb; k += 256) out[k] = -1;
    if (tid == 0) co[row] = total;
}

hipError_t launch_rescue(const uint16_t *Q, const uint16_t *K, const Shape &s, float *ws,
                         float *A, hipStream_t st) {
    float *qcen = ws;
    float *kcen = qcen + (size_t)s.Hq * s.nb * s.d;
    float *krad = kcen + (size_t)s.Hkv * s.nb * s.d;
    const float scale = kLog2e / sqrtf((float)s.d);
    if (s.d == 128) {
        hipLaunchKernelGGL(rr_block_centroids<128>, dim3(s.nb, s.Hq), dim3(256), 0, st, Q, s.L,
                           s.Hq, s.B, s.nb, qcen, (float *)nullptr);
        hipLaunchKernelGGL(rr_block_centroids<128>, dim3(s.nb, s.Hkv), dim3(256), 0, st, K, s.L,
                           s.Hkv, s.B, s.nb, kcen, krad);
        hipLaunchKernelGGL(rr_rescue_softmax<128>, dim3(s.nb, s.Hq), dim3(256), 0, st, qcen, kcen,
                           krad, s.Hq, s.Hkv, s.nb, scale, A);
    } else {
        hipLaunchKernelGGL(rr_block_centroids<64>, dim3(s.nb, s.Hq), dim3(256), 0, st, Q, s.L,
                           s.Hq, s.B, s.nb, qcen, (float *)nullptr);
        hipLaunchKernelGGL(rr_block_centroids<64>, dim3(s.nb, s.Hkv), dim3(256), 0, st, K, s.L,
                           s.Hkv, s.B, s.nb, kcen, krad);
        hipLaunchKernelGGL(rr_rescue_softmax<64>, dim3(s.nb, s.Hq), dim3(256), 0, st, qcen, kcen,
                           krad, s.Hq, s.Hkv, s.nb, scale, A);
    }
    return hipGetLastError();
}

hipError_t launch_merge_lists(const int32_t *ca, const int32_t *ia, const int32_t *cb,
                              const int32_t *ib, int Hq, int nb, int32_t *co, int32_t *io,
                              hipStream_t st) {
    hipLaunchKernelGGL(rr_merge_lists, dim3(nb, Hq), dim3(256), 0, st, ca, ia, cb, ib, nb, co, io);
    return hipGetLastError();
}

}  // namespace rr
