// rr_select.hip -- adaptive Top-tau block selection (rr_topk_tau).
//
// For block-row I of query head h: order the causal key blocks J <= I by
// (score descending, index ascending), keep the shortest prefix whose running
// sum reaches tau * W with W the row total, and emit the kept indices in
// ascending order (Top-tau rule of the RRAttention summary page; minimal set
// with mass >= tau as in find_blocks, XAttention review page, "threshold
// block selection").
//
// The prefix is found without sorting.  For a score threshold t let F(t) be
// the mass of the entries whose score is >= t.  F does not grow with t, so
// the cut score s* = max{t : F(t) >= tau W} is found bit by bit from the top
// of the float bit pattern (scores are non-negative, so their bits order as
// the values do).  Every entry above s* is kept; of the entries equal to s*
// (ties, ordered by ascending J) the shortest run that lifts the mass to
// tau W is kept, found by a second bit-by-bit search over J.  Up to rounding
// of the sums this is the sorted prefix.
//
// One wave per row, no LDS and no barriers: lane l holds entries J = 64e + l
// in registers.  Each F is a lane sum in fixed order followed by a butterfly
// across the wave, so every lane holds the same value and, the scores being
// non-negative, F computed this way is exactly monotone in t (dropping terms
// from a fixed summation tree never raises the rounded sum).  Kept flags are
// compacted in index order with ballots.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

constexpr int kSelWaves = 4;   // rows per work-group (one per wave)

// Sum over the wave; every lane gets the bitwise-same result (each butterfly
// step adds the same two values in both lanes of a pair).
__device__ __forceinline__ float wave_sum_all(float v) {
    v = xor32_sum(v);
    v = xor16_sum(v);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return __builtin_amdgcn_readfirstlane(v);
}

// One row on one wave with NE entry slots per lane (NE a power of two,
// 64 NE >= the row length n): every loop over the slots is unrolled and
// unguarded.  Scores are compared through their bits read as signed
// integers; slots past the row hold -0.0, whose bits read as INT_MIN, below
// every non-negative score, so no threshold selects them, no tie matches
// them, and a sum they do enter gains nothing.
//
// The rule is defined for finite scores >= 0.  An entry that is negative,
// NaN or infinite is read as +0.0 (zero mass), so the bit order and the
// monotone mass search hold for any input.
template <int NE>
__device__ __forceinline__ void topk_row(const float *__restrict__ row, int n, int nb, float tau,
                                         int32_t *__restrict__ out, int32_t *__restrict__ count) {
    const int lane = threadIdx.x & 63;
    float x[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int J = 64 * e + lane;
        if (J < n) {
            const float v = row[J];
            x[e] = (v > 0.f && v <= 3.402823466e38f) ? v : 0.f;
        } else {
            x[e] = -0.f;
        }
    }

    int kept = n;
    if (tau < 1.f) {
        // Mass of the entries that pass `sel`, in the fixed order.
        auto mass = [&](auto sel) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) s += sel(e) ? x[e] : 0.f;
            return wave_sum_all(s);
        };
        int mb = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e) mb = max(mb, __float_as_int(x[e]));
        mb = wave_max_i(mb);
        const float thr = tau * mass([&](int) { return true; });

        // s* = the largest bit pattern t <= max with F(t) >= thr (F(0) is
        // the total, which is >= thr).
        int t = 0;
        for (int b = 30; b >= 0; --b) {
            const int c = t | (1 << b);
            if (c > mb) continue;
            if (mass([&](int e) { return __float_as_int(x[e]) >= c; }) >= thr) t = c;
        }

        // Ties at s*: keep those with J <= Jc, where Jc is the first tie whose
        // running mass (all entries above s*, then the ties in ascending J)
        // reaches thr.  u = the largest count such that the ties with J < u
        // still leave the mass below thr (0 when the first tie already
        // reaches it); Jc = the first tie with J >= u.
        int ties = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e) ties += __popcll(__ballot(__float_as_int(x[e]) == t));
        int u = 0;
        if (ties > 1) {
            for (int b = 12; b >= 0; --b) {
                const int c = u | (1 << b);
                if (c > n) continue;
                const float f = mass([&](int e) {
                    const int bits = __float_as_int(x[e]);
                    return bits > t || (bits == t && 64 * e + lane < c);
                });
                if (f < thr) u = c;
            }
        }
        int jc = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int J = 64 * e + lane;
            if (J >= u && __float_as_int(x[e]) == t) jc = min(jc, J);
        }
        jc = wave_min_i(jc);

        // Compact the kept indices in ascending J.
        int base = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int J = 64 * e + lane;
            const int bits = __float_as_int(x[e]);
            const bool k = bits > t || (bits == t && J <= jc);
            const unsigned long long m = __ballot(k);
            const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((unsigned)m, 0));
            if (k) out[base + below] = J;
            base += __popcll(m);
        }
        kept = base;
    } else {
        for (int J = lane; J < n; J += 64) out[J] = J;
    }
    for (int q = kept + lane; q < nb; q += 64) out[q] = -1;
    if (lane == 0) *count = kept;
}

// E = the largest slot count a row of this call needs (a power of two >=
// ceil(nb / 64)); each row runs with the smallest power of two that holds
// it.  Rows are taken longest first: work-group b holds rows 4b .. 4b+3 of
// the (I descending, h) order.
template <int E>
__global__ __launch_bounds__(kSelWaves * 64) void rr_topk_tau(const float *__restrict__ A, int nb,
                                                              int Hq, float tau,
                                                              int32_t *__restrict__ counts,
                                                              int32_t *__restrict__ block_idx) {
    const int r = blockIdx.x * kSelWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= Hq * nb) return;
    const int I = nb - 1 - r / Hq, h = r % Hq;
    const int n = I + 1;
    const float *row = A + ((size_t)h * nb + I) * nb;
    int32_t *out = block_idx + ((size_t)h * nb + I) * nb;
    int32_t *cnt = counts + (size_t)h * nb + I;
    if (n <= 64) topk_row<1>(row, n, nb, tau, out, cnt);
    else if (E >= 2 && n <= 128) topk_row<(E >= 2 ? 2 : 1)>(row, n, nb, tau, out, cnt);
    else if (E >= 4 && n <= 256) topk_row<(E >= 4 ? 4 : 1)>(row, n, nb, tau, out, cnt);
    else if (E >= 8 && n <= 512) topk_row<(E >= 8 ? 8 : 1)>(row, n, nb, tau, out, cnt);
    else if (E >= 16 && n <= 1024) topk_row<(E >= 16 ? 16 : 1)>(row, n, nb, tau, out, cnt);
    else if (E >= 32 && n <= 2048) topk_row<(E >= 32 ? 32 : 1)>(row, n, nb, tau, out, cnt);
    else if (E >= 64) topk_row<(E >= 64 ? 64 : 1)>(row, n, nb, tau, out, cnt);
}

hipError_t launch_topk_tau(const float *A, const Shape &s, float tau, int32_t *counts,
                           int32_t *block_idx, hipStream_t st) {
    const int rows = s.Hq * s.nb;
    const dim3 grid((rows + kSelWaves - 1) / kSelWaves), block(kSelWaves * 64);
    const int need = (s.nb + 63) / 64;
#define RR_TOPK_CASE(EE)                                                                       \
    if (need <= EE) {                                                                          \
        hipLaunchKernelGGL(rr_topk_tau<EE>, grid, block, 0, st, A, s.nb, s.Hq, tau, counts,     \
                           block_idx);                                                         \
        return hipGetLastError();                                                              \
    }
    RR_TOPK_CASE(1)
    RR_TOPK_CASE(2)
    RR_TOPK_CASE(4)
    RR_TOPK_CASE(8)
    RR_TOPK_CASE(16)
    RR_TOPK_CASE(32)
    RR_TOPK_CASE(64)
#undef RR_TOPK_CASE
    return hipErrorInvalidValue;
}

}  // namespace rr
