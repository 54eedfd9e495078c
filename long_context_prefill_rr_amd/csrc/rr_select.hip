// rr_select.hip -- adaptive Top-tau block selection (rr_topk_tau).
//
// For block-row I of query head h: order the causal key blocks J <= I by
// (score descending, index ascending), keep the shortest prefix whose running
// sum reaches tau * W with W the row total, and emit the kept indices in
// ascending order (Top-tau rule of the RRAttention summary page; minimal set
// with mass >= tau as in find_blocks, XAttention review page, "threshold
// block selection").
//
// One work-group of 256 threads per row.  The row is sorted in LDS by a
// bitonic network on 64-bit keys (float bits of the non-negative score in the
// high word, ~J in the low word, so equal scores order by ascending J; the
// steps within one wave's quarter of the row run without work-group
// barriers), the
// sorted scores are prefix-summed with wave scans, the cut is found with an
// LDS atomicMin, and kept flags are compacted in index order by a second scan.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

constexpr int kSelThreads = 256;

// Inclusive scan of one value per thread across the work-group (float).
__device__ float block_inclusive_scan(float v, float *wsum) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    float pre = 0.f;
    for (int w = 0; w < wid; ++w) pre += wsum[w];
    __syncthreads();
    return v + pre;
}

__device__ int block_inclusive_scan_int(int v, int *wsum) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wid; ++w) pre += wsum[w];
    __syncthreads();
    return v + pre;
}

// Dynamic LDS: N 64-bit keys followed by N 32-bit flags (N = padded row length).
__global__ __launch_bounds__(kSelThreads) void rr_topk_tau(const float *__restrict__ A, int nb,
                                                           int Npad, float tau,
                                                           int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ block_idx) {
    extern __shared__ unsigned long long keys[];
    int *flags = reinterpret_cast<int *>(keys + Npad);
    __shared__ float fsum[4];
    __shared__ int isum[4];
    __shared__ int cut;

    const int I = blockIdx.x, h = blockIdx.y;
    const int n = I + 1;
    int N = 2;
    while (N < n) N <<= 1;
    const float *row = A + ((size_t)h * nb + I) * nb;
    const int tid = threadIdx.x;

    for (int i = tid; i < N; i += kSelThreads) {
        unsigned long long k = 0ull;
        if (i < n) k = ((unsigned long long)__float_as_uint(row[i]) << 32) | (unsigned)(~(unsigned)i);
        keys[i] = k;
        flags[i] = 0;
    }
    if (tid == 0) cut = n - 1;
    __syncthreads();

    // Bitonic sort, descending.  Pair p of a step with partner distance j is
    // (i, i + j) with i = (p / j) * 2j + p % j.  Each wave owns a segment of
    // M = N/4 keys (the whole row in wave 0 when N < 256); steps with j < M
    // stay inside one segment and run without work-group barriers (a wave's
    // LDS accesses complete in order; the wait and the wave barrier keep the
    // compiler from moving them across steps), so only the three steps with
    // j >= M synchronise the work-group (none when N < 256).
    {
        const int wid = tid >> 6, lane = tid & 63;
        const int M = N >= 256 ? N / 4 : N;
        const int nseg = N / M;
        auto cmpx = [&](int i, int j, int k) {
            const unsigned long long a = keys[i], b = keys[i + j];
            const bool desc = (i & k) == 0;
            if (desc ? (a < b) : (a > b)) {
                keys[i] = b;
                keys[i + j] = a;
            }
        };
        // j = 2^lj: the pair index splits with shifts and masks.
        auto lower = [&](int p, int j, int lj) { return ((p >> lj) << (lj + 1)) | (p & (j - 1)); };
        for (int k = 2; k <= N; k <<= 1) {
            int lj = 31 - __clz(k >> 1);
            for (int j = k >> 1; j > 0; j >>= 1, --lj) {
                if (j >= M) {
                    __syncthreads();
                    for (int p = tid; p < N / 2; p += kSelThreads) cmpx(lower(p, j, lj), j, k);
                    __syncthreads();
                } else if (wid < nseg) {
                    const int base = wid * M;
                    for (int p = lane; p < M / 2; p += 64) cmpx(base + lower(p, j, lj), j, k);
                    wait_lgkm0();
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }
        __syncthreads();
    }

    // Prefix sums of the sorted scores: thread t owns positions [t*E, t*E+E).
    const int E = (N + kSelThreads - 1) / kSelThreads;
    const int p0 = tid * E;
    float local = 0.f;
    for (int e = 0; e < E; ++e) {
        const int p = p0 + e;
        if (p < n) local += __uint_as_float((unsigned)(keys[p] >> 32));
    }
    const float incl = block_inclusive_scan(local, fsum);
    __shared__ float total;
    if (tid == kSelThreads - 1) total = incl;
    __syncthreads();
    if (tau < 1.f) {
        const float thr = tau * total;
        float run = incl - local;
        for (int e = 0; e < E; ++e) {
            const int p = p0 + e;
            if (p >= n) break;
            run += __uint_as_float((unsigned)(keys[p] >> 32));
            if (run >= thr) {
                atomicMin(&cut, p);
                break;
            }
        }
    }
    __syncthreads();
    const int kstar = cut;
    for (int p = tid; p <= kstar; p += kSelThreads) flags[~(unsigned)(keys[p] & 0xffffffffull)] = 1;
    __syncthreads();

    // Ascending compaction of the kept flags.
    int fl = 0;
    for (int e = 0; e < E; ++e) {
        const int J = p0 + e;
        if (J < n) fl += flags[J];
    }
    const int fincl = block_inclusive_scan_int(fl, isum);
    int pos = fincl - fl;
    int32_t *out = block_idx + ((size_t)h * nb + I) * nb;
    for (int e = 0; e < E; ++e) {
        const int J = p0 + e;
        if (J < n && flags[J]) out[pos++] = J;
    }
    for (int q = kstar + 1 + tid; q < nb; q += kSelThreads) out[q] = -1;
    if (tid == 0) counts[(size_t)h * nb + I] = kstar + 1;
}

hipError_t launch_topk_tau(const float *A, const Shape &s, float tau, int32_t *counts,
                           int32_t *block_idx, hipStream_t st) {
    int Npad = 2;
    while (Npad < s.nb) Npad <<= 1;
    const size_t lds = (size_t)Npad * (8 + 4);
    hipLaunchKernelGGL(rr_topk_tau, dim3(s.nb, s.Hq), dim3(kSelThreads), lds, st, A, s.nb, Npad,
                       tau, counts, block_idx);
    return hipGetLastError();
}

}  // namespace rr
