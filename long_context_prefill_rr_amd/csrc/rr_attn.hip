// rr_attn.hip -- causal block-sparse attention with GQA over a compacted
// block list (rr_block_sparse_fa), plus the V transpose it reads.
//
// Attention runs only on the key blocks kept for each (query head, query
// block-row) (RRAttention abstract: about half of the blocks are computed);
// within a kept block it is exact causal softmax attention with scale
// 1/sqrt(d), and query head h reads kv-head h / (Hq/Hkv) (GQA).
//
// Work-group = one (kv-head g, query block I, pair of query heads of g): two
// groups of BLK/32 waves, one per head, each wave owning 32 query rows.  The
// two heads' kept lists are merged in LDS into their union (ascending key
// blocks, each tagged with the heads that keep it); the work-group walks the
// union in stages of 64 keys and every K/V stage brought on chip serves both
// heads, while a wave skips the stages its own head did not keep.
//   * the K tiles [64 keys][d] and V^T tiles [d][64 keys] of the next two
//     stages are copied global -> LDS by buffer_load_dwordx4 ... lds (no
//     registers) into one pair of buffers while the two stages held by the
//     other pair are computed, with one barrier per pair of stages; rows are
//     XOR-swizzled in 16-byte slots against LDS bank conflicts;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16.  The K rows fed to the
//     matrix unit are permuted so that accumulator register e of lane
//     (column q, half hk) holds key 16*hk + e of each 32-key sub-tile:
//     every lane owns one query column, and a row maximum, when one is
//     taken, needs a single cross-half exchange;
//   * online softmax in the log2 domain (scores pre-scaled by
//     log2(e)/sqrt(d)), diagonal block masked causally; the running maximum
//     is checked through each 16-key group's weight sum rather than taken
//     per score;
//   * P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T . P^T: its registers already hold 8 consecutive keys per
//     lane half, and the matching V^T rows are 16-byte LDS reads.
// O^T stays in registers (one query column per lane) and is divided by the
// softmax sum at the end.
//
// Grid order: kv-head major, block-row descending, the head pairs of one
// (g, I) adjacent and on the same XCD (work-groups are dealt to the 8 XCDs
// round-robin), so the K/V tiles they share are served from that XCD's L2
// and one kv-head's K/V (64 MiB at 128K) stays in the last-level cache while
// its rows run; long rows start first.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

// K fragments are read this many d-steps ahead of the products that use them.
constexpr int KLA = 2;

// V [L][Hkv][d] -> Vt [Hkv][d][Lp], tokens >= L zero-filled.  64x64 tiles.
__global__ __launch_bounds__(256) void rr_transpose_v(const uint16_t *__restrict__ V, int L, int Lp,
                                                      int Hkv, int D, uint16_t *__restrict__ Vt) {
    __shared__ uint16_t tile[64][66];
    const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, g = blockIdx.z;
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
        const int r = i >> 5, c2 = (i & 31) * 2;
        const int t = t0 + r;
        uint32_t v = 0;
        if (t < L) v = *reinterpret_cast<const uint32_t *>(V + ((size_t)t * Hkv + g) * D + d0 + c2);
        tile[r][c2] = (uint16_t)(v & 0xffff);
        tile[r][c2 + 1] = (uint16_t)(v >> 16);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
        const int r = i >> 5, c2 = (i & 31) * 2;
        const uint32_t v = (uint32_t)tile[c2][r] | ((uint32_t)tile[c2 + 1][r] << 16);
        *reinterpret_cast<uint32_t *>(Vt + ((size_t)g * D + d0 + r) * Lp + t0 + c2) = v;
    }
}

// Tile constants of the attention kernel.  A work-group holds two head
// groups of BLK/32 waves (two query heads that share one kv-head); each wave
// owns one 32-row query tile.  Keys are walked in 64-key stages.
template <int D, int BLK>
struct FaCfg {
    static constexpr int NWG = BLK / 32;                // waves per head group
    static constexpr int NW = 2 * NWG;                  // waves per work-group
    static constexpr int NT = NW * 64;                  // threads
    static constexpr int KT = 64;                       // keys per pipeline stage
    static constexpr int SPB = BLK / KT;                // stages per key block
    static constexpr int CPRK = D / 8;                  // 16-byte chunks per K row
    static constexpr int IK = KT * CPRK / 64 / NW;      // K copies per wave per stage
    static constexpr int IV = D * (KT / 8) / 64 / NW;   // V^T copies per wave per stage
    static constexpr int LPW = IK + IV;                 // copies per wave per stage
    static constexpr int KBYTES = KT * D * 2;
    static constexpr int VBYTES = D * KT * 2;
    static constexpr int NDT = D / 32;
    static constexpr int NKS = D / 16;
    static constexpr int MAXNB = 4096;                  // longest block list
};

// LDS swizzles (16-byte slot XOR per row) chosen so that the 16 rows read by
// one 16-lane group of a ds_read_b128 land in 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (D == 128) return (r & 7) | (((r >> 4) & 1) << 3);
    else return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }

// Online softmax with a checked reference maximum (log2 units).  A 16-key
// group's weights are first formed against the running reference maximum m;
// only if a lane's eight weights sum to more than kGroupMax (a score above m
// by a few units, or m not yet set: an inf / NaN sum) is the group's maximum
// taken, O and the normaliser rescaled, and the group's weights formed
// again.  The common path computes no per-score maximum.  Weights stay <= 64,
// and m follows the row maximum closely: the key that sets m gets weight
// exactly 1, so the largest weights carry little bf16 rounding (a limit of
// 4096 measured about 20% larger output errors).
constexpr float kGroupMax = 64.f;

// max / sum of x over both 32-lane halves, for every lane (v_permlane32_swap).
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A 64-row block makes a 4-wave work-group that fits once per CU (LDS): one
// wave per SIMD.
template <int D, int BLK, bool OUT_F32>
__global__ __launch_bounds__(BLK * 4, BLK == 128 ? 2 : 1) void rr_block_sparse_fa(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ Vt,
    int L, int Lp, int Hq, int Hkv, int nb, int nq, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ block_idx, void *__restrict__ O, float scale2) {
    using C = FaCfg<D, BLK>;
    __shared__ __attribute__((aligned(1024))) char Kb0[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb1[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb2[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb3[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb0[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb1[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb2[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb3[C::VBYTES];
    __shared__ uint32_t ulist[C::MAXNB];          // union of the two kept lists
    __shared__ uint32_t bits[2][C::MAXNB / 32];   // per-head membership bitmaps
    __shared__ int scan_part[C::NW];
    __shared__ int nunion;

    const int G = Hq / Hkv;
    const int npair = (G + 1) >> 1;
    // Work decode: (kv-head g, block-row I) pairs qi in kv-head-major order
    // with I descending, times head pairs.  Work-groups are dealt to the 8
    // XCDs round-robin, so XCD x runs bx = x, x+8, ...: its slot-th work-group
    // gets pair qi = (slot / npair)*8 + x and head pair slot % npair.  The 8
    // XCDs work on neighbouring block-rows of one kv-head at a time (their
    // K/V tiles meet in the shared last-level cache) and the head pairs of
    // one row stay on one XCD (sharing its L2).
    const int bx = blockIdx.x;
    const int x = bx & 7, slot = bx >> 3;
    const int pp = slot % npair;
    const int qi = (slot / npair) * 8 + x;
    if (qi >= nq) return;
    const int g = qi / nb;
    const int I = nb - 1 - qi % nb;

    const int tid = threadIdx.x;
    // The wave index is uniform: readfirstlane lets the compiler keep it and
    // everything derived from it (LDS copy bases, head group) in SGPRs.
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int gr = wid / C::NWG;              // head group of this wave
    const int rw = wid % C::NWG;              // 32-row tile of this wave
    const int col = lane & 31, hk = lane >> 5;
    const bool head_ok = 2 * pp + gr < G;     // odd G: the last pair has one head
    const int h = g * G + min(2 * pp + gr, G - 1);
    const int tq = I * BLK + rw * 32 + col;
    const int wave_last_row = I * BLK + rw * 32 + 31;

    // Union of the two heads' kept lists (ascending key blocks, each tagged
    // with the heads that keep it), built in LDS: membership bitmaps, then a
    // work-group scan compacts the set blocks in index order.
    const int nbw = (nb + 31) >> 5;
    for (int i = tid; i < 2 * (C::MAXNB / 32); i += C::NT) (&bits[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (2 * pp + q >= G) continue;
        const int hq = g * G + 2 * pp + q;
        const int cq = min(max(counts[(size_t)hq * nb + I], 0), nb);
        const int32_t *lq = block_idx + ((size_t)hq * nb + I) * nb;
        for (int k = tid; k < cq; k += C::NT) {
            const int J = lq[k];
            if ((unsigned)J <= (unsigned)I) atomicOr(&bits[q][J >> 5], 1u << (J & 31));
        }
    }
    __syncthreads();
    {
        const int E = (nb + C::NT - 1) / C::NT;
        const int j0 = tid * E;
        int cnt_local = 0;
        for (int e = 0; e < E; ++e) {
            const int J = j0 + e;
            if (J < nb && ((bits[0][J >> 5] | bits[1][J >> 5]) >> (J & 31)) & 1u) ++cnt_local;
        }
        int incl = cnt_local;
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) {
            const int t = __shfl_up(incl, o2, 64);
            if (lane >= o2) incl += t;
        }
        if (lane == 63) scan_part[wid] = incl;
        __syncthreads();
        int pre = 0;
        for (int w = 0; w < wid; ++w) pre += scan_part[w];
        int pos = pre + incl - cnt_local;
        for (int e = 0; e < E; ++e) {
            const int J = j0 + e;
            if (J >= nb) break;
            const uint32_t b0 = (bits[0][J >> 5] >> (J & 31)) & 1u, b1 = (bits[1][J >> 5] >> (J & 31)) & 1u;
            if (b0 | b1) ulist[pos++] = (uint32_t)J | (b0 << 16) | (b1 << 17);
        }
        if (tid == C::NT - 1) nunion = pre + incl;
        __syncthreads();
    }
    (void)nbw;

    bf16x8 qf[C::NKS];
    {
        const uint16_t *qp = Q + ((size_t)min(tq, L - 1) * Hq + h) * D + hk * 8;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = as_bf16x8(ld16(qp + ks * 16));
    }

    f32x16 o[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    // MFMA row r = col of the S^T tile reads K row 16*((r>>2)&1) + 4*(r>>3) + (r&3)
    // of its 32-key sub-tile, so accumulator e of lane (col, hk) is key 16*hk + e.
    const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    const int ksw = swz_k<D>(krow);
    const int vsw = swz_v(col);

    const int nst = nunion * C::SPB;

    // Union entry of stage st: key block in the low 16 bits, bit 16+q set
    // when head q of the pair keeps it.  Read from LDS, made wave-uniform.
    auto stage_entry = [&](int st) -> int {
        if (st >= nst) return -1;
        return __builtin_amdgcn_readfirstlane((int)ulist[st / C::SPB]);
    };
    // Copy target of stage st: a stage past the end re-copies the last one
    // (into a buffer no one reads), so every step issues the same copies.
    auto copy_stage = [&](int st) -> int { return min(st, nst - 1); };

    // Per-lane byte offsets of this wave's copies inside one stage (the same
    // for every stage): K chunk (row r, slot c^swz) and V^T chunk.  Each copy
    // is then a uniform per-stage base plus a fixed 32-bit lane offset.
    uint32_t koff[C::IK], voff[C::IV];
#pragma unroll
    for (int i = 0; i < C::IK; ++i) {
        const int p = (wid * C::IK + i) * 64 + lane;
        const int r = p / C::CPRK, c = (p % C::CPRK) ^ swz_k<D>(r);
        koff[i] = (uint32_t)((r * Hkv * D + c * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < C::IV; ++i) {
        const int p = (wid * C::IV + i) * 64 + lane;
        const int r = p >> 3, c = (p & 7) ^ swz_v(r);
        voff[i] = (uint32_t)((r * Lp + c * 8) * 2);
    }
    const char *kbase = reinterpret_cast<const char *>(K + (size_t)g * D);
    const char *vbase = reinterpret_cast<const char *>(Vt + (size_t)g * D * Lp);

    // Start the copies of stage st (key block J) into (kb, vb).
    auto issue = [&](int st, char *kb, char *vb) {
        st = copy_stage(st);
        const int ent = __builtin_amdgcn_readfirstlane((int)ulist[st / C::SPB]);
        const int J = ent & 0xffff;
        const int key0 = J * BLK + (st % C::SPB) * C::KT;
        const bool full = key0 + C::KT <= L;
        // Buffer resources based at this stage's first K row (clamped to row
        // L-1 for a stage that starts at or past L) and first V^T column;
        // each lane adds its byte offset.
        const int krow0 = full ? key0 : min(key0, L - 1);
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kbase + (size_t)krow0 * Hkv * D * 2);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vbase + (size_t)key0 * 2);
#pragma unroll
        for (int i = 0; i < C::IK; ++i) {
            uint32_t off = koff[i];
            if (!full) {
                // Short last stage: rows past L re-read row L-1 (masked later).
                // krow0 <= min(key0 + r, L - 1), so the offset is not negative.
                const int p = (wid * C::IK + i) * 64 + lane;
                const int r = p / C::CPRK, c = (p % C::CPRK) ^ swz_k<D>(r);
                const int rr = min(key0 + r, L - 1) - krow0;
                off = (uint32_t)((rr * Hkv * D + c * 8) * 2);
            }
            buf2lds16(rk, off, (lds_char *)kb + (wid * C::IK + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < C::IV; ++i) buf2lds16(rv, voff[i], (lds_char *)vb + (wid * C::IV + i) * 1024);
    };

    // The entry is passed in (read at the top of the iteration, before the
    // copies), so no LDS read of the list is pending during the products.
    auto compute = [&](int st, int ent, const char *kb, const char *vb) {
        if (ent < 0 || !((ent >> (16 + gr)) & 1)) return;  // not kept by this wave's head
        const int J = ent & 0xffff;
        const int key0 = J * BLK + (st % C::SPB) * C::KT;
        const bool diag = (J == I);
        if (diag && wave_last_row < key0) return;  // whole stage above this wave's rows

        // S^T for both 32-key sub-tiles, d-step by d-step.  K fragments are
        // read two d-steps ahead of their products; scheduling barriers keep
        // the compiler from sinking each read next to its consumer, which
        // would expose one LDS round trip per pair of products.
        f32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
        const char *kr0 = kb + krow * (D * 2);
        const char *kr1 = kr0 + 32 * (D * 2);
        uint4 fa[C::NKS], fb[C::NKS];
        auto rd = [&](int ks) {
            const int off = ((2 * ks + hk) ^ ksw) << 4;
            fa[ks] = *reinterpret_cast<const uint4 *>(kr0 + off);
            fb[ks] = *reinterpret_cast<const uint4 *>(kr1 + off);
        };
#pragma unroll
        for (int ks = 0; ks < KLA; ++ks) rd(ks);
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            if (ks + KLA < C::NKS) rd(ks + KLA);
            __builtin_amdgcn_sched_barrier(0);
            sacc[0] = mfma32x32x16(as_bf16x8(fa[ks]), qf[ks], sacc[0]);
            sacc[1] = mfma32x32x16(as_bf16x8(fb[ks]), qf[ks], sacc[1]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // V^T fragments of 16-key group gi (kt = gi / 2, mm = gi % 2), one per
        // 32-row d-tile; groups 0 and 1 are read before the softmax starts and
        // each later group's two groups ahead of its products.
        auto rdv = [&](int gi, uint4 (&a)[C::NDT]) {
            const int voff = ((4 * (gi >> 1) + 2 * hk + (gi & 1)) ^ vsw) << 4;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
                a[dt] = *reinterpret_cast<const uint4 *>(vb + (dt * 32 + col) * (C::KT * 2) + voff);
        };
        uint4 vf[4][C::NDT];
        rdv(0, vf[0]);
        rdv(1, vf[1]);
        __builtin_amdgcn_sched_barrier(0);

        if (diag) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = key0 + kt * 32 + 16 * hk + e;
                    if (key > tq) sacc[kt][e] = -INFINITY;
                }
        }

#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const int kt = gi >> 1, mm = gi & 1;
            uint32_t pk[4];
            float gsum;
            // The normaliser sums the same bf16 weights the P.V product uses.
            auto weights = [&](float nm) {
                gsum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = fast_exp2(fmaf(sacc[kt][8 * mm + 2 * e], scale2, nm));
                    const float p1 = fast_exp2(fmaf(sacc[kt][8 * mm + 2 * e + 1], scale2, nm));
                    pk[e] = pack_bf16x2(p0, p1);
                    gsum = add_bf16x2(pk[e], gsum);
                }
            };
            weights(-m);
            if (__ballot(!(gsum <= kGroupMax)) != 0ull) {
                // Maximum over the group (both lane halves hold the same
                // query row).
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sacc[kt][8 * mm + e]);
                const float mn = fmaxf(m, max_halves(mx) * scale2);
                const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
                m = mn;
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
                weights(-m);
            }
            lsum += gsum;
            const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
            if (gi + 2 < 4) rdv(gi + 2, vf[gi + 2]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) o[dt] = mfma32x32x16(as_bf16x8(vf[gi][dt]), pb, o[dt]);
        }
    };

    // Stages are taken two at a time between barriers, from two pairs of
    // buffers: while one pair is computed the copies of the next two stages
    // fill the other.  One barrier per pair: every wave's copies of the pair
    // have landed (vmcnt 0) and every wave has finished reading the other
    // pair (lgkmcnt 0) before it.
    if (nst > 0) {
        issue(0, Kb0, Vb0);
        issue(1, Kb1, Vb1);
        for (int st = 0; st < nst; st += 4) {
            {
                const int E0 = stage_entry(st), E1 = stage_entry(st + 1);
                wait_vmcnt<0>();
                wait_lgkm0();
                bar();
                issue(st + 2, Kb2, Vb2);
                issue(st + 3, Kb3, Vb3);
                compute(st, E0, Kb0, Vb0);
                compute(st + 1, E1, Kb1, Vb1);
            }
            if (st + 2 >= nst) break;
            {
                const int E2 = stage_entry(st + 2), E3 = stage_entry(st + 3);
                wait_vmcnt<0>();
                wait_lgkm0();
                bar();
                issue(st + 4, Kb0, Vb0);
                issue(st + 5, Kb1, Vb1);
                compute(st + 2, E2, Kb2, Vb2);
                compute(st + 3, E3, Kb3, Vb3);
            }
        }
        wait_vmcnt<0>();
    }

    const float tot = sum_halves(lsum);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (tq >= L || !head_ok) return;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const int d0 = dt * 32 + 8 * e4 + 4 * hk;
            const float v0 = o[dt][4 * e4] * inv, v1 = o[dt][4 * e4 + 1] * inv;
            const float v2 = o[dt][4 * e4 + 2] * inv, v3 = o[dt][4 * e4 + 3] * inv;
            if constexpr (OUT_F32) {
                float *op = reinterpret_cast<float *>(O) + ((size_t)tq * Hq + h) * D + d0;
                *reinterpret_cast<float4 *>(op) = make_float4(v0, v1, v2, v3);
            } else {
                uint16_t *op = reinterpret_cast<uint16_t *>(O) + ((size_t)tq * Hq + h) * D + d0;
                *reinterpret_cast<uint2 *>(op) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
        }
    }
}

hipError_t launch_transpose_v(const uint16_t *V, const Shape &s, uint16_t *Vt, hipStream_t st) {
    const int Lp = s.nb * s.B;
    hipLaunchKernelGGL(rr_transpose_v, dim3(Lp / 64, s.d / 64, s.Hkv), dim3(256), 0, st, V, s.L, Lp,
                       s.Hkv, s.d, Vt);
    return hipGetLastError();
}

template <int D, int BLK>
static void launch_fa_t(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, const Shape &s,
                        const int32_t *counts, const int32_t *block_idx, void *O, bool out_f32,
                        hipStream_t st) {
    const int nq = s.nb * s.Hkv;
    const int nq8 = (nq + 7) / 8 * 8;
    const dim3 grid((unsigned)(nq8 * ((s.G + 1) / 2)));
    const float scale2 = kLog2e / sqrtf((float)D);
    const int Lp = s.nb * BLK;
    if (out_f32)
        hipLaunchKernelGGL((rr_block_sparse_fa<D, BLK, true>), grid, dim3(BLK * 4), 0, st, Q, K, Vt,
                           s.L, Lp, s.Hq, s.Hkv, s.nb, nq, counts, block_idx, O, scale2);
    else
        hipLaunchKernelGGL((rr_block_sparse_fa<D, BLK, false>), grid, dim3(BLK * 4), 0, st, Q, K,
                           Vt, s.L, Lp, s.Hq, s.Hkv, s.nb, nq, counts, block_idx, O, scale2);
}

hipError_t launch_block_sparse_fa(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt,
                                  const Shape &s, const int32_t *counts, const int32_t *block_idx,
                                  void *O, bool out_f32, hipStream_t st) {
    if (s.d == 128 && s.B == 128)
        launch_fa_t<128, 128>(Q, K, Vt, s, counts, block_idx, O, out_f32, st);
    else if (s.d == 128 && s.B == 64)
        launch_fa_t<128, 64>(Q, K, Vt, s, counts, block_idx, O, out_f32, st);
    else if (s.d == 64 && s.B == 128)
        launch_fa_t<64, 128>(Q, K, Vt, s, counts, block_idx, O, out_f32, st);
    else
        launch_fa_t<64, 64>(Q, K, Vt, s, counts, block_idx, O, out_f32, st);
    return hipGetLastError();
}

}  // namespace rr
