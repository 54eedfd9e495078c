// rr_quality.hip -- selection quality of a kept-block mask against a
// reference mask (rr_mask_quality).
//
// The RRAttention summary page ("Key points") reports precision and F1 of
// the blocks a method selects.  Per (query head h, query block-row I) this
// counts the distinct valid blocks J <= I of the mask under test (kept), of
// the reference mask (ref) and of both (both), and the share of the row's
// block mass that the tested mask keeps: sum of mass[h][I][J] over its
// blocks / sum over all J <= I.  A second single-work-group pass sums the
// per-row values in a fixed order.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

constexpr int kQualMaxNb = 4096;

// One work-group (256 threads) per (block-row I, head h).
__global__ __launch_bounds__(256) void rr_mask_quality_rows(
    const int32_t *__restrict__ counts, const int32_t *__restrict__ block_idx,
    const int32_t *__restrict__ ref_counts, const int32_t *__restrict__ ref_idx,
    const float *__restrict__ mass, int nb, float *__restrict__ rows) {
    __shared__ uint32_t tbits[kQualMaxNb / 32], rbits[kQualMaxNb / 32];
    __shared__ float red_m[256], red_w[256];
    __shared__ int red_c[3][256];
    const int I = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t row = (size_t)h * nb + I;
    const int nw = (I >> 5) + 1;  // bitmap words covering J = 0..I
    for (int i = tid; i < nw; i += 256) {
        tbits[i] = 0u;
        rbits[i] = 0u;
    }
    __syncthreads();
    const int ct = min(max(counts[row], 0), nb), cr = min(max(ref_counts[row], 0), nb);
    const int32_t *lt = block_idx + row * nb, *lr = ref_idx + row * nb;
    for (int k = tid; k < ct; k += 256) {
        const int J = lt[k];
        if ((unsigned)J <= (unsigned)I) atomicOr(&tbits[J >> 5], 1u << (J & 31));
    }
    for (int k = tid; k < cr; k += 256) {
        const int J = lr[k];
        if ((unsigned)J <= (unsigned)I) atomicOr(&rbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    int kept = 0, ref = 0, both = 0;
    for (int i = tid; i < nw; i += 256) {
        kept += __popc(tbits[i]);
        ref += __popc(rbits[i]);
        both += __popc(tbits[i] & rbits[i]);
    }
    float mk = 0.f, w = 0.f;
    const float *mrow = mass + row * nb;
    for (int J = tid; J <= I; J += 256) {
        const float a = mrow[J];
        w += a;
        if ((tbits[J >> 5] >> (J & 31)) & 1u) mk += a;
    }
    red_m[tid] = mk;
    red_w[tid] = w;
    red_c[0][tid] = kept;
    red_c[1][tid] = ref;
    red_c[2][tid] = both;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            red_m[tid] += red_m[tid + o];
            red_w[tid] += red_w[tid + o];
            red_c[0][tid] += red_c[0][tid + o];
            red_c[1][tid] += red_c[1][tid + o];
            red_c[2][tid] += red_c[2][tid + o];
        }
        __syncthreads();
    }
    if (tid == 0) {
        float *out = rows + row * 4;
        out[0] = (float)red_c[0][0];
        out[1] = (float)red_c[1][0];
        out[2] = (float)red_c[2][0];
        out[3] = red_w[0] > 0.f ? red_m[0] / red_w[0] : 0.f;
    }
}

// Totals over n rows: sums of the four columns and the minimum kept share.
__global__ __launch_bounds__(256) void rr_mask_quality_totals(const float *__restrict__ rows,
                                                              long long n,
                                                              double *__restrict__ totals) {
    __shared__ double red[5][256];
    const int tid = threadIdx.x;
    double s0 = 0, s1 = 0, s2 = 0, s3 = 0, mn = 1e300;
    for (long long r = tid; r < n; r += 256) {
        const float *v = rows + r * 4;
        s0 += v[0];
        s1 += v[1];
        s2 += v[2];
        s3 += v[3];
        mn = fmin(mn, (double)v[3]);
    }
    red[0][tid] = s0;
    red[1][tid] = s1;
    red[2][tid] = s2;
    red[3][tid] = s3;
    red[4][tid] = mn;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
#pragma unroll
            for (int c = 0; c < 4; ++c) red[c][tid] += red[c][tid + o];
            red[4][tid] = fmin(red[4][tid], red[4][tid + o]);
        }
        __syncthreads();
    }
    if (tid < 5) totals[tid] = red[tid][0];
}

hipError_t launch_mask_quality(const int32_t *counts, const int32_t *block_idx,
                               const int32_t *ref_counts, const int32_t *ref_idx,
                               const float *mass, int Hq, int nb, float *rows, double *totals,
                               hipStream_t st) {
    hipLaunchKernelGGL(rr_mask_quality_rows, dim3(nb, Hq), dim3(256), 0, st, counts, block_idx,
                       ref_counts, ref_idx, mass, nb, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rr_mask_quality_totals, dim3(1), dim3(256), 0, st, rows,
                       (long long)Hq * nb, totals);
    return hipGetLastError();
}

}  // namespace rr
