// rr_estimate.hip -- the estimation kernels of the round-robin block scores.
//
//   rr_pool_k               K -> stride-mean keys, split into three bf16 planes
//   rr_score32              sampled queries x pooled keys on bf16 MFMA (32 x 32
//                           tiles, blocks of 4 to 16 strides); per (row,
//                           key-block) max / sum-of-exponentials
//   rr_score                the same with 16 x 16 tiles, for the other block
//                           sizes (1, 2, 32, 64, 128 strides)
//   rr_stride_softmax_pool  causal row softmax folded into B x B block sums
//
// and the materialised variant of the same estimate, which writes every
// stride score to memory and pools it in a second pass:
//
//   rr_score<..., STORE>           the same products; the scaled scores of
//                                  every (row, stride j <= block end) stored
//   rr_stride_softmax_pool_scores  reads each row of scores once: per-block
//                                  max / sum in LDS, the row softmax, then
//                                  the block sums
//
// Method: one query per stride of S tokens, offset h mod S rotating with the
// query head, scored against the mean key of every earlier-or-equal stride,
// softmax over strides, probabilities summed per block (RRAttention summary
// page, "Summary" and "Key points"; RRAttention abstract).
//
// Precision: the pooled key is an fp32 mean of bf16 keys.  Rounding it to one
// bf16 moves scores enough to flip Top-tau decisions, so it is carried as
// hi + mid + lo bf16 planes (24 significand bits) and each plane is a
// separate MFMA pass with fp32 accumulation.  Scores live in the log2 domain
// (scaled by log2(e)/sqrt(d)) so exponentials are single v_exp_f32.
#include <algorithm>
#include <type_traits>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

// ---------------------------------------------------------------------------
// rr_pool_k: Kbar[g][j][:] = (1/S) sum_t K[jS+t][g][:], written as three bf16
// planes.  One thread per (stride, kv-head, 8 consecutive channels); the
// token-major K makes each group of d/8 threads read one contiguous key row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void rr_pool_k(const uint16_t *__restrict__ K, int Hkv, int ns,
                                                 int S, float invS,
                                                 uint16_t *__restrict__ planes) {
    constexpr int C8 = D / 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)ns * Hkv * C8;
    if (idx >= total) return;
    const int c8 = (int)(idx % C8);
    const long long r = idx / C8;
    const int g = (int)(r % Hkv);
    const int j = (int)(r / Hkv);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const uint16_t *src = K + ((size_t)j * S * Hkv + g) * D + c8 * 8;
    for (int t = 0; t < S; ++t) {
        uint4 v = ld16(src + (size_t)t * Hkv * D);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(w[e] << 16);
            acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
        }
    }
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x0 = acc[2 * e] * invS, x1 = acc[2 * e + 1] * invS;
        uint16_t h0 = bf16_bits(x0), h1 = bf16_bits(x1);
        float r0 = x0 - bf16_to_f32(h0), r1 = x1 - bf16_to_f32(h1);
        uint16_t m0 = bf16_bits(r0), m1 = bf16_bits(r1);
        float q0 = r0 - bf16_to_f32(m0), q1 = r1 - bf16_to_f32(m1);
        hi[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        mid[e] = (uint32_t)m0 | ((uint32_t)m1 << 16);
        lo[e] = pack_bf16x2(q0, q1);
    }
    const size_t plane = (size_t)Hkv * ns * D;
    uint16_t *dst = planes + ((size_t)g * ns + j) * D + c8 * 8;
    st16(dst, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    st16(dst + plane, make_uint4(mid[0], mid[1], mid[2], mid[3]));
    st16(dst + 2 * plane, make_uint4(lo[0], lo[1], lo[2], lo[3]));
}

// Offset of the (stride row i = I*C + a, key block J <= I) entry inside one
// head's packed area: block-row I owns C*(I+1) entries starting at
// C*I*(I+1)/2, ordered by J then a, so the C strides of one key block are
// contiguous (one 16-row MFMA tile stores 16 adjacent entries).
__device__ __forceinline__ long long packed_offset(int C, int I, int a, int J) {
    return (long long)C * I * (I + 1) / 2 + (long long)J * C + a;
}

// Offset of stride score (row (I, a), stride j) in a head's stored scores:
// block-row I owns c rows of (I+1)c strides, row-major, after the c^2 I(I+1)/2
// entries of block-rows 0 .. I-1.
__device__ __forceinline__ long long score_offset(int C, int I, int a, int j) {
    return (long long)C * C * I * (I + 1) / 2 + (long long)a * (I + 1) * C + j;
}

// ---------------------------------------------------------------------------
// rr_score: one work-group per (group of R consecutive query block-rows
// I0 .. I0+R-1, kv-head g, chunk of up to 256 sampled rows).  The rows are
// the (block-row, query head, stride) triples of the G heads that share
// kv-head g: row (I, hh, a) samples token (I*C + a)*S + ((g*G + hh) mod S).
// R is chosen so that a work-group holds about 256 rows: every pooled-key
// fragment streamed from memory then feeds 16 row tiles, which keeps the
// vector-memory path (the bound of a 64-row design) well below the matrix
// unit's rate.  The rows' Q tile sits in LDS (XOR-swizzled 16-byte slots).
// Each wave computes S^T = Kbar . Q^T tiles of 16 strides x 16 rows on
// v_mfma_f32_16x16x32_bf16 (3 planes x d/32 steps) for all rows; the waves
// split the key strides 0 .. (I0+R)*C-1 into units of 16 strides
// (C >= 16: whole blocks J = wave, wave+4, ...; C < 16: 16-stride units).
// Fragments of the unit after next are loaded while a unit is processed.
// For every (row, key-block) it writes max and sum of 2^(s - max) over the
// block's strides j <= i; per-row totals are merged across waves into
// rowstat.  Nothing of the [rows x strides] score matrix reaches memory.
// ---------------------------------------------------------------------------
constexpr int kScoreRows = 256;

// With STORE set, the statistics are replaced by the scores themselves:
// scores[h][c^2 I(I+1)/2 + a (I+1)c + j] = s(row (I, a), stride j) in log2
// units, -inf for j > i, for every j < (I+1)c (layout of score_offset).
template <int D, int C, bool STORE = false>
__global__ __launch_bounds__(256) void rr_score(const uint16_t *__restrict__ Q,
                                                const uint16_t *__restrict__ Kp, int Hq, int Hkv,
                                                int S, int nb, int ns, int G, int R, int nchunks,
                                                long long P, float scale2,
                                                float2 *__restrict__ stats,
                                                float2 *__restrict__ rowstat,
                                                float *__restrict__ scores = nullptr) {
    static_assert(!STORE || C >= 4, "stored scores are written four strides at a time");
    constexpr int KS = D / 32;
    constexpr int CPR = D / 8;                 // 16-byte chunks per Q row
    constexpr int NSUB = C >= 16 ? C / 16 : 1;
    constexpr int MT = kScoreRows / 16;        // row tiles per work-group
    __shared__ __attribute__((aligned(16))) uint16_t qs[kScoreRows * D];
    __shared__ float2 red[4][kScoreRows];

    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 15, lg = lane >> 4;

    // Decode: block-row groups in descending order (long rows first).
    int b = blockIdx.x;
    const int chunk = b % nchunks;
    b /= nchunks;
    const int g = b % Hkv;
    const int ngrp = (nb + R - 1) / R;
    const int I0 = (ngrp - 1 - b / Hkv) * R;
    const int GC = G * C;
    const int rows_total = min(R, nb - I0) * GC;           // rows of this block-row group
    const int row0 = chunk * kScoreRows;
    const int rows_here = min(kScoreRows, rows_total - row0);
    const int NT = (rows_here + 15) >> 4;
    const int Itop = min(I0 + R, nb) - 1;                   // last block-row of the group
    const size_t plane = (size_t)Hkv * ns * D;
    const uint16_t *kb = Kp + (size_t)g * ns * D;

    // Row f (0..rows_here) -> (block-row, head, stride); -1 stride if invalid.
    auto row_of = [&](int f, int &I, int &h, int &i) {
        const int ff = row0 + f;
        I = I0 + ff / GC;
        const int rem = ff % GC, hh = rem / C, a = rem % C;
        h = g * G + hh;
        const int cI = min(C, ns - I * C);
        i = (f < rows_here && a < cI) ? I * C + a : -1;
    };

    // Stage the Q rows in LDS: chunk c of row f at slot c ^ (f & 15).
    for (int idx = threadIdx.x; idx < kScoreRows * CPR; idx += 256) {
        const int f = idx / CPR, c = idx % CPR;
        int I, h, i;
        row_of(f, I, h, i);
        uint4 v = zero_u4();
        if (i >= 0) {
            const int t = i * S + (h % S);
            v = ld16(Q + ((size_t)t * Hq + h) * D + c * 8);
        }
        st16(&qs[f * D + ((c ^ (f & 15)) & (CPR - 1)) * 8], v);
    }

    // This lane's row in each tile (column of the S^T tiles).
    int row_i[MT], row_h[MT];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
        int I, h, i;
        row_of(rt * 16 + lr, I, h, i);
        row_i[rt] = (rt < NT) ? i : -1;
        row_h[rt] = h;
    }
    __syncthreads();

    float rM[MT], rZ[MT];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
        rM[rt] = -INFINITY;
        rZ[rt] = 0.f;
    }

    // Units of this wave (16 strides each) over the strides of blocks 0..Itop.
    const int nkeys = (Itop + 1) * C;
    int nunits;
    if constexpr (C >= 16) {
        const int nblk = (Itop >= wid) ? (Itop - wid) / 4 + 1 : 0;
        nunits = nblk * NSUB;
    } else {
        const int ng = (nkeys + 15) / 16;
        nunits = (ng > wid) ? (ng - 1 - wid) / 4 + 1 : 0;
    }
    auto unit_j0 = [&](int t) -> int {
        if constexpr (C >= 16)
            return (wid + 4 * (t / NSUB)) * C + (t % NSUB) * 16;
        else
            return (wid + 4 * t) * 16;
    };
    auto load = [&](int t, bf16x8 (&ka)[3][KS]) {
        const int jr = min(unit_j0(t) + lr, ns - 1);
        const uint16_t *src = kb + (size_t)jr * D + lg * 8;
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[p][ks] = as_bf16x8(ld16(src + p * plane + ks * 32));
    };

    float bm[MT], bz[MT];  // running block statistics when a block spans units
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
        bm[rt] = -INFINITY;
        bz[rt] = 0.f;
    }

    auto write_stat = [&](int rt, int J, float m, float z) {
        if (lg == 0 && row_i[rt] >= 0 && J * C <= row_i[rt] && m != -INFINITY) {
            const int I = row_i[rt] / C, a = row_i[rt] - I * C;
            stats[(size_t)row_h[rt] * P + packed_offset(C, I, a, J)] = make_float2(m, z);
            merge_max_sum(rM[rt], rZ[rt], m, z);
        }
    };

    auto process = [&](int t, bf16x8 (&ka)[3][KS]) {
        const int j0 = unit_j0(t);
        // Causal masking only where a unit reaches the first stride of block I0.
        const bool diag = j0 + 15 >= I0 * C;
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) {
            if (rt >= NT) break;
            const int f = rt * 16 + lr;
            const uint16_t *qrow = &qs[f * D];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = ks * 4 + lg;
                const bf16x8 qb = as_bf16x8(ld16(qrow + ((c ^ (f & 15)) & (CPR - 1)) * 8));
#pragma unroll
                for (int p = 0; p < 3; ++p) acc = mfma16x16x32(ka[p][ks], qb, acc);
            }
            if (diag) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j0 + lg * 4 + e > row_i[rt]) acc[e] = -INFINITY;
            }
            if constexpr (STORE) {
                // Strides j0 + 4 lg .. + 3 of this lane's row, if they lie in
                // the row's packed range j < (I+1)c (C >= 4: all four or none).
                const int jj = j0 + lg * 4;
                if (row_i[rt] >= 0) {
                    const int I = row_i[rt] / C, a = row_i[rt] - I * C;
                    if (jj < (I + 1) * C) {
                        const float4 v = make_float4(acc[0] * scale2, acc[1] * scale2, acc[2] * scale2,
                                                     acc[3] * scale2);
                        *reinterpret_cast<float4 *>(scores + (size_t)row_h[rt] * (size_t)(C * P) +
                                                    score_offset(C, I, a, jj)) = v;
                    }
                }
            } else if constexpr (C >= 16) {
                const int J = j0 / C;
                const int sub = (j0 % C) / 16;
                float mr = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
                mr = xor16_max(mr);
                mr = xor32_max(mr);
                const float m = mr * scale2;
                float z = 0.f;
                if (mr != -INFINITY) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) z += fast_exp2(fmaf(acc[e], scale2, -m));
                }
                z = xor16_sum(z);
                z = xor32_sum(z);
                if constexpr (NSUB == 1) {
                    write_stat(rt, J, m, z);
                } else {
                    merge_max_sum(bm[rt], bz[rt], m, z);
                    if (sub == NSUB - 1) {
                        write_stat(rt, J, bm[rt], bz[rt]);
                        bm[rt] = -INFINITY;
                        bz[rt] = 0.f;
                    }
                }
            } else {
                constexpr int KPB = C < 4 ? C : 4;  // keys of one block held by a lane
                constexpr int BPL = 4 / KPB;        // blocks per lane
#pragma unroll
                for (int bi = 0; bi < BPL; ++bi) {
                    float mr = -INFINITY;
#pragma unroll
                    for (int e = bi * KPB; e < (bi + 1) * KPB; ++e) mr = fmaxf(mr, acc[e]);
                    if constexpr (C == 8) mr = xor16_max(mr);
                    const float m = mr * scale2;
                    float z = 0.f;
                    if (mr != -INFINITY) {
#pragma unroll
                        for (int e = bi * KPB; e < (bi + 1) * KPB; ++e) z += fast_exp2(fmaf(acc[e], scale2, -m));
                    }
                    if constexpr (C == 8) z = xor16_sum(z);
                    const int J = (j0 + lg * 4 + bi * KPB) / C;
                    const bool writer = (C == 8) ? ((lg & 1) == 0) : true;
                    if (writer && row_i[rt] >= 0 && mr != -INFINITY) {
                        const int I = row_i[rt] / C, a = row_i[rt] - I * C;
                        stats[(size_t)row_h[rt] * P + packed_offset(C, I, a, J)] = make_float2(m, z);
                        merge_max_sum(rM[rt], rZ[rt], m, z);
                    }
                }
            }
        }
        // The fragments are consumed: refill them with the unit after next.
        if (t + 2 < nunits) load(t + 2, ka);
    };

    bf16x8 kA[3][KS], kB[3][KS];
    if (nunits > 0) load(0, kA);
    if (nunits > 1) load(1, kB);
    for (int t = 0; t < nunits; t += 2) {
        process(t, kA);
        if (t + 1 >= nunits) break;
        process(t + 1, kB);
    }

    if constexpr (STORE) return;
    // Per-row totals: butterfly over the four lane groups, then across waves.
#pragma unroll
    for (int rt = 0; rt < MT; ++rt) {
        float m2 = xor_lane(rM[rt], 16), z2 = xor_lane(rZ[rt], 16);
        merge_max_sum(rM[rt], rZ[rt], m2, z2);
        m2 = xor_lane(rM[rt], 32);
        z2 = xor_lane(rZ[rt], 32);
        merge_max_sum(rM[rt], rZ[rt], m2, z2);
    }
    if (lg == 0) {
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) red[wid][rt * 16 + lr] = make_float2(rM[rt], rZ[rt]);
    }
    __syncthreads();
    {
        const int r = threadIdx.x;  // kScoreRows == 256 threads
        float M = -INFINITY, Z = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) merge_max_sum(M, Z, red[w][r].x, red[w][r].y);
        int I, h, i;
        row_of(r, I, h, i);
        if (i >= 0) rowstat[(size_t)h * ns + i] = make_float2(M, Z);
    }
}

// ---------------------------------------------------------------------------
// rr_score32: rr_score's rows and outputs for blocks of 4, 8 or 16 strides,
// with 32 x 32 tiles on v_mfma_f32_32x32x16_bf16.  The pooled-key rows fed
// to the matrix unit are permuted so that accumulator register e of lane
// (row q, half) holds stride 16*half + e of the 32-stride unit: a lane owns
// whole key blocks of its row, and each block's max and sum of exponentials
// are taken in registers with no cross-lane step (the 16-stride tiles of
// rr_score spread a block over four lanes).
//
// The four waves walk the 32-stride units 0, 1, ... together, and wave w
// owns row tiles w and w+4 for the whole pass: their Q fragments stay in
// registers, and every pooled-key fragment read from LDS feeds the products
// of both tiles (two independent accumulation chains).  Each unit's three
// planes (32 strides x d) are copied global -> LDS by the work-group
// (buffer_load ... lds, no registers) one unit ahead, into one of two
// buffers; rows past the last stride read as zeros and are masked causally.
// A wave whose rows all end before a unit only copies and waits for it.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int score_swz(int r) {
    // 16-byte slot XOR per pooled-key row: the 16 rows one 16-lane group
    // reads for one fragment fall in 16 distinct bank groups.
    if constexpr (D == 128) return (r & 7) | (((r >> 4) & 1) << 3);
    else return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}

template <int D, int C>
__global__ __launch_bounds__(256, 3) void rr_score32(const uint16_t *__restrict__ Q,
                                                     const uint16_t *__restrict__ Kp, int Hq, int Hkv,
                                                     int S, int nb, int ns, int G, int R, int nchunks,
                                                     long long P, float scale2,
                                                     float2 *__restrict__ stats,
                                                     float2 *__restrict__ rowstat) {
    static_assert(C == 4 || C == 8 || C == 16, "blocks of 4, 8 or 16 strides");
    constexpr int NKS = D / 16;                // 16-wide contraction steps
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int BPL = 16 / C;                // key blocks per lane per unit
    constexpr int PLANE_B = 32 * D * 2;        // one plane of a unit in LDS
    constexpr int UNIT_B = 3 * PLANE_B;
    constexpr int CPW = UNIT_B / (4 * 1024);   // 1 KiB copies per wave per unit
    constexpr int CPP = PLANE_B / 1024;        // copies per plane
    static_assert(CPW * 4 * 1024 == UNIT_B && CPP * 1024 == PLANE_B, "whole copies");
    constexpr int LA = 1;                      // fragment look-ahead (steps): 160 VGPRs, 3 waves per SIMD
    __shared__ __attribute__((aligned(1024))) char kb0[UNIT_B];
    __shared__ __attribute__((aligned(1024))) char kb1[UNIT_B];

    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int q = lane & 31, hk = lane >> 5;

    // Decode: block-row groups in descending order (long rows first).
    int b = blockIdx.x;
    const int chunk = b % nchunks;
    b /= nchunks;
    const int g = b % Hkv;
    const int ngrp = (nb + R - 1) / R;
    const int I0 = (ngrp - 1 - b / Hkv) * R;
    const int GC = G * C;
    const int rows_total = min(R, nb - I0) * GC;
    const int row0 = chunk * kScoreRows;
    const int rows_here = min(kScoreRows, rows_total - row0);
    const int NT = (rows_here + 31) >> 5;
    const int Itop = min(I0 + R, nb) - 1;
    const size_t plane = (size_t)Hkv * ns * D;

    // Row f (0..rows_here) -> (block-row, head, stride); -1 stride if invalid.
    auto row_of = [&](int f, int &I, int &h, int &i) {
        const int ff = row0 + f;
        I = I0 + ff / GC;
        const int rem = ff % GC, hh = rem / C, a = rem % C;
        h = g * G + hh;
        const int cI = min(C, ns - I * C);
        i = (f < rows_here && a < cI) ? I * C + a : -1;
    };

    // This wave's row tiles w and w+4 (so a 4-tile work-group keeps every
    // wave busy): lane row, head and Q fragments (B operand: lane (q, half)
    // holds d = 16 ks + 8 half .. + 7 of row q).
    const int nt_w = (wid < NT ? 1 : 0) + (wid + 4 < NT ? 1 : 0);   // valid tiles (wave-uniform)
    int row_i[2], row_h[2];
    bf16x8 qf[2][NKS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        int I, h, i;
        row_of((wid + 4 * u) * 32 + q, I, h, i);
        row_i[u] = (u < nt_w) ? i : -1;
        row_h[u] = h;
        const uint16_t *qp = Q + ((size_t)(max(i, 0) * S + (h % S)) * Hq + h) * D + hk * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[u][ks] = as_bf16x8(row_i[u] >= 0 ? ld16(qp + ks * 16) : zero_u4());
    }
    // Last stride any row of this wave scores (units past it are skipped).
    int imax = max(row_i[0], row_i[1]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) imax = max(imax, __shfl_xor(imax, o, 64));
    imax = __builtin_amdgcn_readfirstlane(imax);

    float rM[2] = {-INFINITY, -INFINITY}, rZ[2] = {0.f, 0.f};

    // Copies: copy c of this wave moves 64 16-byte chunks of plane c / CPP;
    // LDS slot (row r, s) holds source chunk s ^ swz(r).
    uint32_t coff[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int p = ((wid * CPW + c) % CPP) * 64 + lane;
        const int r = p / CPR, s = p % CPR;
        coff[c] = (uint32_t)((r * D + (s ^ score_swz<D>(r)) * 8) * 2);
    }
    const uint16_t *kbase = Kp + (size_t)g * ns * D;
    auto issue = [&](int t, char *kb) {
        const int j0 = t * 32;
        const int bytes = max(ns - j0, 0) * D * 2;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int cc = wid * CPW + c;
            const __amdgpu_buffer_rsrc_t r =
                buf_rsrc_n(kbase + (cc / CPP) * plane + (size_t)j0 * D, bytes);
            buf2lds16(r, coff[c], (lds_char *)kb + cc * 1024);
        }
    };

    // Pooled-key row of this lane's A operand (see the permutation above).
    const int krow = 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
    const int ksw = score_swz<D>(krow);

    // Block statistics of one tile's 32 x 32 scores for unit j0.
    auto tile_stats = [&](int u, f32x16 &acc, int j0, bool diag) {
        const int ri = row_i[u];
        if (diag) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (j0 + 16 * hk + e > ri) acc[e] = -INFINITY;
        }
#pragma unroll
        for (int bi = 0; bi < BPL; ++bi) {
            float mr = -INFINITY;
#pragma unroll
            for (int e = bi * C; e < (bi + 1) * C; ++e) mr = fmaxf(mr, acc[e]);
            const float m = mr * scale2;
            const float mu = (mr == -INFINITY) ? 0.f : m;
            // The block's C exponentials summed as two interleaved chains.
            float z0 = fast_exp2(fmaf(acc[bi * C], scale2, -mu));
            float z1 = fast_exp2(fmaf(acc[bi * C + 1], scale2, -mu));
#pragma unroll
            for (int e = 2; e < C; e += 2) {
                z0 += fast_exp2(fmaf(acc[bi * C + e], scale2, -mu));
                z1 += fast_exp2(fmaf(acc[bi * C + e + 1], scale2, -mu));
            }
            const float z = z0 + z1;
            // A block with an unmasked stride j <= i lies at or before the
            // row's own block.
            const bool ok = ri >= 0 && mr != -INFINITY;
            if (ok) {
                const int J = (j0 + 16 * hk) / C + bi;
                const int I = ri / C, a = ri - I * C;
                stats[(size_t)row_h[u] * P + packed_offset(C, I, a, J)] = make_float2(m, z);
            }
            // Exact online merge into the row total with one exponential:
            // e = 2^-|m - rM| scales whichever side is smaller.
            const float dd = m - rM[u];
            const float e = fast_exp2(-fabsf(dd));
            const float nz = dd > 0.f ? fmaf(rZ[u], e, z) : fmaf(z, e, rZ[u]);
            rZ[u] = ok ? nz : rZ[u];
            rM[u] = ok ? fmaxf(rM[u], m) : rM[u];
        }
    };

    // Products and statistics of unit t (pooled keys in kb) for NTW tiles.
    auto compute = [&](auto ntw, int t, const char *kb) {
        constexpr int NTW = decltype(ntw)::value;
        const int j0 = t * 32;
        const char *kr = kb + krow * (D * 2);
        uint4 fr[NKS][3];
        auto rd = [&](int ks) {
            const int off = ((2 * ks + hk) ^ ksw) << 4;
#pragma unroll
            for (int p = 0; p < 3; ++p) fr[ks][p] = *reinterpret_cast<const uint4 *>(kr + p * PLANE_B + off);
        };
        f32x16 acc[NTW];
#pragma unroll
        for (int u = 0; u < NTW; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < LA; ++ks) rd(ks);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ks + LA < NKS) rd(ks + LA);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int u = 0; u < NTW; ++u) acc[u] = mfma32x32x16(as_bf16x8(fr[ks][p]), qf[u][ks], acc[u]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Causal masking only where the unit reaches the first stride of block I0.
        const bool diag = j0 + 31 >= I0 * C;
#pragma unroll
        for (int u = 0; u < NTW; ++u) tile_stats(u, acc[u], j0, diag);
    };
    auto unit = [&](int t, const char *kb) {
        if (t * 32 > imax) return;     // every row of this wave ends before the unit
        if (nt_w == 2)
            compute(std::integral_constant<int, 2>(), t, kb);
        else if (nt_w == 1)
            compute(std::integral_constant<int, 1>(), t, kb);
    };

    // Units over the strides of blocks 0..Itop, one barrier each: every
    // wave's copies of unit t have landed (vmcnt 0) and every wave has read
    // unit t-1's buffer (lgkmcnt 0) before the copies of unit t+1 start.
    const int nu = ((Itop + 1) * C + 31) / 32;
    issue(0, kb0);
    for (int t = 0; t < nu; t += 2) {
        wait_vmcnt<0>();
        wait_lgkm0();
        bar();
        if (t + 1 < nu) issue(t + 1, kb1);
        unit(t, kb0);
        if (t + 1 >= nu) break;
        wait_vmcnt<0>();
        wait_lgkm0();
        bar();
        if (t + 2 < nu) issue(t + 2, kb0);
        unit(t + 1, kb1);
    }
    wait_vmcnt<0>();

    // Per-row totals: the two lane halves hold other blocks of the same row.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float m2 = xor_lane(rM[u], 32), z2 = xor_lane(rZ[u], 32);
        merge_max_sum(rM[u], rZ[u], m2, z2);
        if (hk == 0 && row_i[u] >= 0) rowstat[(size_t)row_h[u] * ns + row_i[u]] = make_float2(rM[u], rZ[u]);
    }
}

// ---------------------------------------------------------------------------
// rr_stride_softmax_pool: one work-group per (block-row I, query head h).
// A[h][I][J] = sum_a z(a,J) 2^(m(a,J) - M_a) / Z_a over the strides a of
// block I, i.e. the causal softmax of each sampled row summed over the
// block's strides.  For C >= 2, lane t of a pass reads the entry pair
// 2t, 2t+1 (one 16-byte load; a pair never straddles two key blocks), adds
// its two terms and the C/2 lanes of one J are summed by a fixed butterfly;
// each thread keeps four loads in flight.  For C = 1 thread p reads entry
// p.  The block-row's entries are read once, coalesced, and every sum runs
// in a fixed order, so the result does not depend on timing.  Entries J > I
// are written as zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rr_stride_softmax_pool(const float2 *__restrict__ stats,
                                                              const float2 *__restrict__ rowstat,
                                                              int C, int nb, int ns, long long P,
                                                              float *__restrict__ A) {
    const int I = blockIdx.x, h = blockIdx.y;
    const int cI = min(C, ns - I * C);
    __shared__ float sM[128], sInvZ[128];
    for (int a = threadIdx.x; a < cI; a += blockDim.x) {
        float2 rs = rowstat[(size_t)h * ns + I * C + a];
        sM[a] = rs.x;
        sInvZ[a] = 1.f / rs.y;
    }
    __syncthreads();
    const float2 *base = stats + (size_t)h * P + (long long)C * I * (I + 1) / 2;
    float *out = A + ((size_t)h * nb + I) * nb;
    const int span = (I + 1) * C;
    const int lg2C = __builtin_ctz(C);
    if (C >= 2) {
        // Entry pairs: the packed offsets C*I(I+1)/2 and h*P are even, so
        // every pair is 16-byte aligned.
        const float4 *b4 = reinterpret_cast<const float4 *>(base);
        const int half = C >> 1;    // lanes holding one J
        const int span2 = span >> 1;
        for (int q0 = 0; q0 < span2; q0 += 4 * 256) {
            float4 st[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int qq = q0 + u * 256 + (int)threadIdx.x;
                st[u] = qq < span2 ? b4[qq] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int qq = q0 + u * 256 + (int)threadIdx.x;
                const int p = 2 * qq, J = p >> lg2C, a = p & (C - 1);
                float v = 0.f;
                if (qq < span2) {
                    if (a < cI) v = st[u].y * fast_exp2(st[u].x - sM[a]) * sInvZ[a];
                    if (a + 1 < cI) v += st[u].w * fast_exp2(st[u].z - sM[a + 1]) * sInvZ[a + 1];
                }
                for (int o = 1; o < half; o <<= 1) v += xor_lane(v, o);
                if (qq < span2 && a == 0) out[J] = v;
            }
        }
    } else {
        for (int p0 = 0; p0 < span; p0 += 256) {
            const int p = p0 + (int)threadIdx.x;
            if (p < span) {
                const float2 st = base[p];
                out[p] = st.y * fast_exp2(st.x - sM[0]) * sInvZ[0];
            }
        }
    }
    for (int J = I + 1 + (int)threadIdx.x; J < nb; J += blockDim.x) out[J] = 0.f;
}

// ---------------------------------------------------------------------------
// rr_stride_softmax_pool_scores: the pooling of the materialised variant.
// One work-group per (block-row I, query head h); the block-row's rows are
// taken one after the other.  For row a, lane t reads strides 4t .. 4t+3 of
// each 1024-stride pass (float4, coalesced): the C/4 lanes of one block give
// its (max, sum of 2^(s - max)) by a butterfly and park it in LDS, and the
// lanes' running (max, sum) give the row's (M_a, Z_a) through a work-group
// reduction (the loads of four passes are issued before any is used, for
// more bytes in flight).  Then A[J] += z_J 2^(m_J - M_a) / Z_a for every
// J <= I, in LDS.
// Each score is read once; all sums run in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kPoolMaxNb = 4096;

template <int C>
__global__ __launch_bounds__(256) void rr_stride_softmax_pool_scores(const float *__restrict__ scores,
                                                                     int nb, int ns, long long SP,
                                                                     float *__restrict__ A) {
    static_assert(C >= 4 && C <= 128, "blocks of 4 .. 128 strides");
    constexpr int LPB = C / 4;  // lanes per block
    __shared__ float2 bst[kPoolMaxNb];
    __shared__ float acc[kPoolMaxNb];
    __shared__ float2 red[4];
    const int I = blockIdx.x, h = blockIdx.y;
    const int cI = min(C, ns - I * C);
    const int span = (I + 1) * C;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    for (int J = tid; J <= I; J += 256) acc[J] = 0.f;
    const float *rowbase = scores + (size_t)h * SP + (size_t)C * C * I * (I + 1) / 2;
    for (int a = 0; a < cI; ++a) {
        const float4 *row = reinterpret_cast<const float4 *>(rowbase + (size_t)a * span);
        float rm = -INFINITY, rz = 0.f;
        const int nq = span / 4;
        // Four 1024-stride passes per round: their loads are issued together.
        for (int q0 = 0; q0 < nq; q0 += 4 * 256) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = q0 + u * 256 + tid;
                v[u] = q < nq ? row[q] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = q0 + u * 256 + tid;
                float m = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)), z = 0.f;
                if (m != -INFINITY)
                    z = fast_exp2(v[u].x - m) + fast_exp2(v[u].y - m) + fast_exp2(v[u].z - m) +
                        fast_exp2(v[u].w - m);
#pragma unroll
                for (int o = 1; o < LPB; o <<= 1) {
                    const float m2 = xor_lane(m, o), z2 = xor_lane(z, o);
                    merge_max_sum(m, z, m2, z2);
                }
                if (q < nq && (lane & (LPB - 1)) == 0) bst[q / LPB] = make_float2(m, z);
                merge_max_sum(rm, rz, m, z);
            }
        }
        // Row totals: butterfly within each wave (lanes of one block already
        // agree), then the four waves in order.
#pragma unroll
        for (int o = LPB; o < kWave; o <<= 1) {
            const float m2 = xor_lane(rm, o), z2 = xor_lane(rz, o);
            merge_max_sum(rm, rz, m2, z2);
        }
        if (lane == 0) red[wid] = make_float2(rm, rz);
        __syncthreads();
        float M = -INFINITY, Z = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) merge_max_sum(M, Z, red[w].x, red[w].y);
        const float invZ = 1.f / Z;
        for (int J = tid; J <= I; J += 256) {
            const float2 b = bst[J];
            if (b.x != -INFINITY) acc[J] += b.y * fast_exp2(b.x - M) * invZ;
        }
        __syncthreads();
    }
    float *out = A + ((size_t)h * nb + I) * nb;
    for (int J = tid; J < nb; J += 256) out[J] = (J <= I) ? acc[J] : 0.f;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_pool_k(const uint16_t *K, const Shape &s, uint16_t *kplanes, hipStream_t st) {
    const long long total = (long long)s.ns * s.Hkv * (s.d / 8);
    const unsigned grid = (unsigned)((total + 255) / 256);
    const float invS = 1.f / (float)s.S;
    if (s.d == 128)
        hipLaunchKernelGGL(rr_pool_k<128>, dim3(grid), dim3(256), 0, st, K, s.Hkv, s.ns, s.S, invS, kplanes);
    else
        hipLaunchKernelGGL(rr_pool_k<64>, dim3(grid), dim3(256), 0, st, K, s.Hkv, s.ns, s.S, invS, kplanes);
    return hipGetLastError();
}

template <int D>
static void launch_score_d(const uint16_t *Q, const Shape &s, const EstimateWs &w, hipStream_t st) {
    const int GC = s.G * s.c;
    int R = std::max(1, std::min(s.nb, kScoreRows / GC));  // block-rows per work-group
    if (s.c == 4 || s.c == 8 || s.c == 16) {
        // Short inputs: fewer block-rows per work-group (down to four 32-row
        // tiles, one per wave) until there are about two work-groups per CU.
        const int want = 2 * device_cu_count();
        while (R > 1 && (R / 2) * GC >= 128 && ((s.nb + R - 1) / R) * s.Hkv < want) R /= 2;
    }
    const int nchunks = (R * GC + kScoreRows - 1) / kScoreRows;
    const int ngrp = (s.nb + R - 1) / R;
    const dim3 grid((unsigned)(ngrp * s.Hkv * nchunks));
    const float scale2 = kLog2e / sqrtf((float)D);
#define RR_SCORE_CASE(KERNEL, CC)                                                              \
    case CC:                                                                                   \
        hipLaunchKernelGGL((KERNEL<D, CC>), grid, dim3(256), 0, st, Q, w.kplanes, s.Hq, s.Hkv,    \
                           s.S, s.nb, s.ns, s.G, R, nchunks, s.P, scale2, w.stats, w.rowstat); \
        break;
    // Blocks of 4 to 16 strides: 32 x 32 tiles, one lane per (row, block).
    switch (s.c) {
        RR_SCORE_CASE(rr_score, 1)
        RR_SCORE_CASE(rr_score, 2)
        RR_SCORE_CASE(rr_score32, 4)
        RR_SCORE_CASE(rr_score32, 8)
        RR_SCORE_CASE(rr_score32, 16)
        RR_SCORE_CASE(rr_score, 32)
        RR_SCORE_CASE(rr_score, 64)
        RR_SCORE_CASE(rr_score, 128)
        default: break;
    }
#undef RR_SCORE_CASE
}

hipError_t launch_score(const uint16_t *Q, const Shape &s, const EstimateWs &w, hipStream_t st) {
    if (s.d == 128)
        launch_score_d<128>(Q, s, w, st);
    else
        launch_score_d<64>(Q, s, w, st);
    return hipGetLastError();
}

template <int D>
static void launch_score_store_d(const uint16_t *Q, const Shape &s, const EstimateWs &w, float *scores,
                                 hipStream_t st) {
    const int GC = s.G * s.c;
    const int R = std::max(1, std::min(s.nb, kScoreRows / GC));
    const int nchunks = (R * GC + kScoreRows - 1) / kScoreRows;
    const int ngrp = (s.nb + R - 1) / R;
    const dim3 grid((unsigned)(ngrp * s.Hkv * nchunks));
    const float scale2 = kLog2e / sqrtf((float)D);
#define RR_SCORE_STORE_CASE(CC)                                                                \
    case CC:                                                                                   \
        hipLaunchKernelGGL((rr_score<D, CC, true>), grid, dim3(256), 0, st, Q, w.kplanes, s.Hq,  \
                           s.Hkv, s.S, s.nb, s.ns, s.G, R, nchunks, s.P, scale2, (float2 *)nullptr, \
                           (float2 *)nullptr, scores);                                         \
        break;
    switch (s.c) {
        RR_SCORE_STORE_CASE(4)
        RR_SCORE_STORE_CASE(8)
        RR_SCORE_STORE_CASE(16)
        RR_SCORE_STORE_CASE(32)
        RR_SCORE_STORE_CASE(64)
        RR_SCORE_STORE_CASE(128)
        default: break;
    }
#undef RR_SCORE_STORE_CASE
}

hipError_t launch_score_store(const uint16_t *Q, const Shape &s, const EstimateWs &w, float *scores,
                              hipStream_t st) {
    if (s.d == 128)
        launch_score_store_d<128>(Q, s, w, scores, st);
    else
        launch_score_store_d<64>(Q, s, w, scores, st);
    return hipGetLastError();
}

hipError_t launch_pool_scores(const Shape &s, const float *scores, float *A, hipStream_t st) {
    const long long SP = score_elems_per_head(s);
#define RR_POOL_SCORES_CASE(CC)                                                                \
    case CC:                                                                                   \
        hipLaunchKernelGGL(rr_stride_softmax_pool_scores<CC>, dim3(s.nb, s.Hq), dim3(256), 0, st, \
                           scores, s.nb, s.ns, SP, A);                                         \
        break;
    switch (s.c) {
        RR_POOL_SCORES_CASE(4)
        RR_POOL_SCORES_CASE(8)
        RR_POOL_SCORES_CASE(16)
        RR_POOL_SCORES_CASE(32)
        RR_POOL_SCORES_CASE(64)
        RR_POOL_SCORES_CASE(128)
        default: break;
    }
#undef RR_POOL_SCORES_CASE
    return hipGetLastError();
}

hipError_t launch_softmax_pool(const Shape &s, const EstimateWs &w, float *A, hipStream_t st) {
    hipLaunchKernelGGL(rr_stride_softmax_pool, dim3(s.nb, s.Hq), dim3(256), 0, st, w.stats,
                       w.rowstat, s.c, s.nb, s.ns, s.P, A);
    return hipGetLastError();
}

}  // namespace rr
