// rr_xattn.hip -- XAttention's antidiagonal block estimate on the same
// statistics, softmax pooling and Top-tau as the round-robin path.
//
// XAttention review page, "importance prediction" and "threshold block
// selection" steps 1-2: inside every S x S sub-block of the attention map
// the elements on the antidiagonal (lower-left to upper-right) are summed,
// and a softmax over those sums gives the probabilities find_blocks
// thresholds.  Sub-block (i, j) pairs query token iS+t with key token
// jS+S-1-t, so its score is one dot product of length S*d:
//   x[h][i][j] = (1/sqrt(d)) * sum_t Q[iS+t][h] . K[jS+S-1-t][g(h)].
// As in the round-robin estimate, stride row i sees key strides j <= i and
// its softmax is summed over the B/S x B/S sub-blocks of each B x B block.
// The page sums the antidiagonal logits; the mean (sum / S, the softmax at
// single-token temperature) is offered as an alternative reading.
//
// rr_xscore computes all x[h][i][j] as a GEMM with a fused statistics
// epilogue: one work-group per (query head, tile of 256 query strides)
// walks the key-stride tiles of 256 at or below its diagonal.  The
// contraction runs in chunks of 64 elements (chunk kc covers t = kc/(d/64),
// elements (kc mod d/64)*64 ..+63): the K~ tile [256 key strides][64] and
// the Q~ tile [256 query strides][64] are copied global -> LDS with
// buffer_load_dwordx4 ... lds into two buffers, one chunk ahead of the one
// being used.  Eight waves each own 64 key strides x 128 query strides
// (2 x 4 tiles of v_mfma_f32_32x32x16_bf16, S^T orientation): per 8
// products a wave reads 6 fragments from LDS (1 per product with 2 x 2
// tiles, which left the kernel bound by LDS bandwidth).  The key rows fed to the
// matrix unit are permuted so that accumulator e of lane (query q, half hk)
// holds key stride 16*hk + e of its 32-stride tile; after a key tile the
// lane therefore has whole 16-stride runs of one query row and writes the
// per-(row, block) max and sum of 2^(x - max) directly, in the packed layout
// rr_stride_softmax_pool reads.  Row totals are merged across the lane
// halves and the four key-quarter waves at the end.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

namespace {

constexpr int kXM = 256;        // query strides per work-group
constexpr int kXT = 256;        // key strides per tile
constexpr int kXK = 64;         // contraction elements per chunk
constexpr int kXRowB = kXK * 2; // bytes per LDS row (8 slots of 16 bytes)
constexpr int kXKB = kXT * kXRowB;   // bytes of one key tile chunk (32 KiB)
constexpr int kXQB = kXM * kXRowB;   // bytes of one query tile chunk (32 KiB)

// Slot swizzles (16-byte slot XOR per row) for the two operands: the key
// operand is read in the permuted row order, the query operand in natural
// order; each keeps the 16 rows one 16-lane group reads in 16 distinct bank
// groups.
__device__ __forceinline__ int swz_key(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
__device__ __forceinline__ int swz_query(int r) { return (r >> 1) & 7; }

// Packed (row i = I*C + a, key block J) entry, as in the round-robin estimate.
__device__ __forceinline__ long long xpacked_offset(int C, int I, int a, int J) {
    return (long long)C * I * (I + 1) / 2 + (long long)J * C + a;
}

}  // namespace

template <int D, int C>
__global__ __launch_bounds__(512, 1) void rr_xscore(const uint16_t *__restrict__ Q,
                                                    const uint16_t *__restrict__ K, int Hq,
                                                    int Hkv, int S, int ns, int ntm, long long P,
                                                    float scale2, float2 *__restrict__ stats,
                                                    float2 *__restrict__ rowstat) {
    static_assert(C == 8 || C == 16 || C == 32, "strides per block");
    constexpr int CPT = D / kXK;  // chunks per sub-block offset t
    __shared__ __attribute__((aligned(1024))) char Ka0[kXKB];
    __shared__ __attribute__((aligned(1024))) char Qa0[kXQB];
    __shared__ __attribute__((aligned(1024))) char Ka1[kXKB];
    __shared__ __attribute__((aligned(1024))) char Qa1[kXQB];
    __shared__ float2 red[4][kXM];

    const int G = Hq / Hkv;
    const int bx = blockIdx.x;
    const int h = bx % Hq;
    const int m = ntm - 1 - bx / Hq;  // long rows first
    const int g = h / G;
    const int i0 = m * kXM;
    const int ntn = (i0 + kXM - 1) / kXT + 1;  // key tiles j0 = 0 .. up to the last query
    const int nkc = S * CPT;                    // chunks per key tile
    const int total = ntn * nkc;

    const int tid = threadIdx.x;
    // Uniform wave index: the copy destinations stay in scalar registers.
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, hk = lane >> 5;
    const int wq = wid & 1, wk = wid >> 1;     // 128-query half, 64-key quarter

    // Copies: lane l of an instruction writes slot l & 7 of row base + (l >> 3)
    // (8 rows x 128 bytes per instruction), holding element chunk
    // (l & 7) ^ swz(row).  Wave w fills key rows 32w .. 32w+31 and query rows
    // 32w .. 32w+31 (4 instructions each).
    const int lrow = lane >> 3;
    const int cslot = lane & 7;
    // The copies are buffer loads: a resource based at the chunk's first key
    // (query) row, clamped to the last stride, plus a per-lane byte offset
    // that stays below 2^32 (at most 255 rows of S * heads * d elements).
    const int ib = min(i0, ns - 1);
    auto issue = [&](int idx, char *ka, char *qa) {
        const int tile = idx / nkc, kc = idx - tile * nkc;
        const int t = kc / CPT, e0 = (kc - t * CPT) * kXK;
        const int j0 = tile * kXT;
        const int jb = min(j0, ns - 1);
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(K + ((size_t)(jb * S + S - 1 - t) * Hkv + g) * D + e0);
        const __amdgpu_buffer_rsrc_t rq = buf_rsrc(Q + ((size_t)(ib * S + t) * Hq + h) * D + e0);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int r = 32 * wid + 8 * n + lrow;
            const int j = min(j0 + r, ns - 1);  // >= jb
            const int ck = cslot ^ swz_key(r);
            const uint32_t off = (uint32_t)(((j - jb) * S * Hkv * D + ck * 8) * 2);
            buf2lds16(rk, off, (lds_char *)ka + (32 * wid + 8 * n) * kXRowB);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int r = 32 * wid + 8 * n + lrow;
            const int i = min(i0 + r, ns - 1);  // >= ib
            const int cq = cslot ^ swz_query(r);
            const uint32_t off = (uint32_t)(((i - ib) * S * Hq * D + cq * 8) * 2);
            buf2lds16(rq, off, (lds_char *)qa + (32 * wid + 8 * n) * kXRowB);
        }
    };

    // Key row fed to MFMA row `col`: accumulator e of lane (col, hk) is key
    // 16*hk + e of the 32-row tile.
    const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    constexpr int NA = 2, NB = 4;  // key and query 32-row tiles of a wave
    int arow[NA], brow[NB];
#pragma unroll
    for (int u = 0; u < NA; ++u) arow[u] = 64 * wk + 32 * u + krow;
#pragma unroll
    for (int u = 0; u < NB; ++u) brow[u] = 128 * wq + 32 * u + col;

    f32x16 acc[NA][NB];
    auto zero_acc = [&]() {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
    };
    zero_acc();

    auto compute = [&](const char *ka, const char *qa) {
#pragma unroll
        for (int ks = 0; ks < kXK / 16; ++ks) {
            const int slot = ks * 2 + hk;
            bf16x8 fa[NA], fb[NB];
#pragma unroll
            for (int u = 0; u < NA; ++u)
                fa[u] = *reinterpret_cast<const bf16x8 *>(ka + arow[u] * kXRowB + ((slot ^ swz_key(arow[u])) << 4));
#pragma unroll
            for (int u = 0; u < NB; ++u)
                fb[u] = *reinterpret_cast<const bf16x8 *>(qa + brow[u] * kXRowB + ((slot ^ swz_query(brow[u])) << 4));
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[a][b] = mfma32x32x16(fa[a], fb[b], acc[a][b]);
        }
    };

    float rM[NB], rZ[NB];
    int qi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        rM[b] = -INFINITY;
        rZ[b] = 0.f;
        qi[b] = i0 + brow[b];
    }

    // Statistics of one finished key tile.
    auto epilogue = [&](int tile) {
        const int j0 = tile * kXT;
        const bool masked = (j0 + kXT - 1 > i0);  // the tile reaches past the first query
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int jb = j0 + 64 * wk + 32 * a + 16 * hk;  // key stride of e = 0
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int i = qi[b];
                float v[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    v[e] = acc[a][b][e];
                    if (masked && jb + e > i) v[e] = -INFINITY;
                }
                constexpr int RUN = C < 16 ? C : 16;  // strides of one block in this lane
#pragma unroll
                for (int s0 = 0; s0 < 16; s0 += RUN) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int e = s0; e < s0 + RUN; ++e) mx = fmaxf(mx, v[e]);
                    const float mm = mx * scale2;
                    float z = 0.f;
                    if (mx != -INFINITY) {
#pragma unroll
                        for (int e = s0; e < s0 + RUN; ++e) z += fast_exp2(fmaf(v[e], scale2, -mm));
                    }
                    float m2 = mm, z2 = z;
                    if constexpr (C == 32) {
                        // The block's other 16 strides sit in the other lane
                        // half: rescale both sums to the common maximum.
                        const float mo = xor32_max(mm);
                        const float sc = (mm == -INFINITY) ? 0.f : z * fast_exp2(mm - mo);
                        m2 = mo;
                        z2 = xor32_sum(sc);
                    }
                    const int J = (jb + s0) / C;
                    const bool writer = (C == 32) ? (hk == 0) : true;
                    if (writer && i < ns && m2 != -INFINITY) {
                        const int I = i / C, aa = i - I * C;
                        stats[(size_t)h * P + xpacked_offset(C, I, aa, J)] = make_float2(m2, z2);
                        merge_max_sum(rM[b], rZ[b], m2, z2);
                    }
                }
            }
        }
        zero_acc();
    };

    // Two buffers, copies one chunk ahead.  Each wave waits for its own
    // copies of the chunk (vmcnt, together with any statistics stores of the
    // last epilogue), then the barrier for everyone's; the buffer refilled
    // after the barrier was last read before it.
    auto step = [&](int idx, char *ka, char *qa, char *kn, char *qn) {
        wait_vmcnt<0>();
        bar();
        // Past the end the last chunk is copied again, into a buffer no one
        // reads any more: every step issues the same copies.
        issue(min(idx + 1, total - 1), kn, qn);
        compute(ka, qa);
        if ((idx + 1) % nkc == 0) epilogue(idx / nkc);
    };
    issue(0, Ka0, Qa0);
    for (int idx = 0; idx < total; idx += 2) {
        step(idx, Ka0, Qa0, Ka1, Qa1);
        if (idx + 1 >= total) break;
        step(idx + 1, Ka1, Qa1, Ka0, Qa0);
    }
    wait_vmcnt<0>();

    // Row totals: the two lane halves, then the four key-quarter waves.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float m2 = xor_lane(rM[b], 32), z2 = xor_lane(rZ[b], 32);
        if (C == 32) {  // both halves hold the same blocks: hk = 1 wrote nothing
            m2 = -INFINITY;
            z2 = 0.f;
        }
        merge_max_sum(rM[b], rZ[b], m2, z2);
    }
    __syncthreads();
    if (hk == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) red[wk][brow[b]] = make_float2(rM[b], rZ[b]);
    }
    __syncthreads();
    if (tid < kXM) {
        float M = -INFINITY, Z = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) merge_max_sum(M, Z, red[w][tid].x, red[w][tid].y);
        const int i = i0 + tid;
        if (i < ns) rowstat[(size_t)h * ns + i] = make_float2(M, Z);
    }
}

hipError_t launch_xscore(const uint16_t *Q, const uint16_t *K, const Shape &s, bool average,
                         const EstimateWs &w, hipStream_t st) {
    const int ntm = (s.ns + kXM - 1) / kXM;
    const dim3 grid((unsigned)(ntm * s.Hq));
    // log2(e)/sqrt(d), and 1/S more for the mean of the antidiagonal.
    const float scale2 = kLog2e / sqrtf((float)s.d) / (average ? (float)s.S : 1.f);
#define RR_XSCORE(DD, CC)                                                                      \
    hipLaunchKernelGGL((rr_xscore<DD, CC>), grid, dim3(512), 0, st, Q, K, s.Hq, s.Hkv, s.S, s.ns, \
                       ntm, s.P, scale2, w.stats, w.rowstat)
    if (s.d == 128) {
        if (s.c == 8) RR_XSCORE(128, 8);
        else if (s.c == 16) RR_XSCORE(128, 16);
        else RR_XSCORE(128, 32);
    } else {
        if (s.c == 8) RR_XSCORE(64, 8);
        else if (s.c == 16) RR_XSCORE(64, 16);
        else RR_XSCORE(64, 32);
    }
#undef RR_XSCORE
    return hipGetLastError();
}

}  // namespace rr
