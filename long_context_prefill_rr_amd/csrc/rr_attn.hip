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
//     other pair are computed, with one barrier per pair of stages and the
//     copies issued between the pair's two stages; rows are XOR-swizzled in
//     16-byte slots against LDS bank conflicts;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16.  The K rows fed to the
//     matrix unit are permuted so that accumulator register e of lane
//     (column q, half hk) holds key 16*hk + e of each 32-key sub-tile:
//     every lane owns one query column, and a row maximum, when one is
//     taken, needs a single cross-half exchange;
//   * online softmax in the log2 domain (scores pre-scaled by
//     log2(e)/sqrt(d)), diagonal block masked causally; the running maximum
//     is checked through the weight sums of each 32-key sub-tile's two
//     16-key groups rather than taken per score;
//   * P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T . P^T: its registers already hold 8 consecutive keys per
//     lane half, and the matching V^T rows are 16-byte LDS reads.
// O^T stays in registers (one query column per lane) and is divided by the
// softmax sum at the end.
//
// Work order: work-groups take items from a device counter (reset by
// rr_transpose_v, which runs just before on the same stream), ordered
// block-row descending within one kv-head at a time (all kv-heads together
// when each CU takes at most 8 items), then kv-head and head pair: long rows
// start first, the K/V in use stays in the last-level cache, and a CU that
// finishes an item early simply takes the next.  (Work-groups are dealt to
// the 8 XCDs by block index; a fixed mapping from block index to rows left
// the XCDs with up to 41% different work on the 64K video shape.)
//
// For rows of up to 128 blocks, and of up to 512 blocks when G is odd (the
// last head pair would hold a single head), a work-group serves one query
// head (SINGLE): BLK/32 waves, two stage buffers with one barrier per stage,
// and LDS for two work-groups per CU.  The work-groups are persistent (two per CU, looping over items),
// and the two waves a SIMD holds then belong to different work-groups whose
// barriers are independent, so one wave's softmax meets the other's
// products more often than in the head-pair work-group, whose barrier keeps
// its two waves per SIMD in step; no wave waits on a stage its head did not
// keep.  Otherwise head pairs serve: on longer rows sharing each staged K/V
// tile between two heads matters more.
#include <algorithm>

#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

// K fragment reads kept in flight ahead of the products that use them.
constexpr int KLA = 4;

// V [L][Hkv][d] -> Vt [Hkv][d][Lp], tokens >= L zero-filled.  64x64 tiles.
// Also resets the attention kernel's work counter.
__global__ __launch_bounds__(256) void rr_transpose_v(const uint16_t *__restrict__ V, int L, int Lp,
                                                      int Hkv, int D, uint16_t *__restrict__ Vt,
                                                      unsigned *__restrict__ counter) {
    __shared__ uint16_t tile[64][66];
    const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, g = blockIdx.z;
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *counter = 0u;
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
// groups of BLK/32 waves (two query heads that share one kv-head), or one
// with SINGLE; each wave owns one 32-row query tile.  Keys are walked in
// 64-key stages.
template <int D, int BLK, bool SINGLE = false>
struct FaCfg {
    static constexpr int NWG = BLK / 32;                // waves per head group
    static constexpr int NW = SINGLE ? NWG : 2 * NWG;   // waves per work-group
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
    static constexpr int MAXNB = SINGLE ? 2048 : 4096;  // longest block list
};

// LDS swizzles (16-byte slot XOR per row) chosen so that the 16 rows read by
// one 16-lane group of a ds_read_b128 land in 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (D == 128) return (r & 7) | (((r >> 4) & 1) << 3);
    else return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }

// Online softmax with a checked reference maximum (log2 units).  The weights
// of a 32-key sub-tile (two 16-key groups) are first formed against the
// running reference maximum m; only if a lane's eight weights of either group
// sum to more than kGroupMax (a score above m by a few units, or m not yet
// set: an inf / NaN sum) is the sub-tile's maximum taken, O and the
// normaliser rescaled, and both groups' weights formed again.  The common
// path computes no per-score maximum.  Weights stay <= 64, and m follows the
// row maximum closely: the key that sets m gets weight exactly 1, so the
// largest weights carry little bf16 rounding (a limit of 4096 measured about
// 20% larger output errors).  The first sub-tile a row meets always holds an
// unmasked key of that row (key 0 of its first kept block), so m is finite
// before any fully masked group is weighed.
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
//
// PERSIST: the grid holds about one work-group per CU (two with SINGLE) and
// each loops over work items; otherwise the grid holds one work-group per
// item (the loop body runs once).  The loop costs registers, and at long rows
// (nb > 512) the launch of a new work-group per item is a smaller cost than
// that.  SINGLE: one query head per work-group (see the file header).
template <int D, int BLK, bool OUT_F32, bool PERSIST, bool SINGLE>
__global__ __launch_bounds__(SINGLE ? BLK * 2 : BLK * 4, BLK == 128 ? 2 : 1) void rr_block_sparse_fa(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ Vt,
    unsigned *__restrict__ counter, int nitems, int hchunk, int L, int Lp, int Hq, int Hkv, int nb,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ block_idx, void *__restrict__ O,
    float scale2) {
    using C = FaCfg<D, BLK, SINGLE>;
    __shared__ __attribute__((aligned(1024))) char Kb0[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb1[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb2[SINGLE ? 16 : C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Kb3[SINGLE ? 16 : C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb0[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb1[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb2[SINGLE ? 16 : C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char Vb3[SINGLE ? 16 : C::VBYTES];
    __shared__ uint32_t ulist[C::MAXNB];          // union of the two kept lists
    __shared__ uint32_t bits[2][C::MAXNB / 32];   // per-head membership bitmaps
    __shared__ int scan_part[C::NW];
    __shared__ int nunion;

    const int G = Hq / Hkv;
    const int npair = (G + 1) >> 1;
    const int tid = threadIdx.x;
    // The wave index is uniform: readfirstlane lets the compiler keep it and
    // everything derived from it (LDS copy bases, head group) in SGPRs.
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int gr = wid / C::NWG;              // head group of this wave
    const int rw = wid % C::NWG;              // 32-row tile of this wave
    const int col = lane & 31, hk = lane >> 5;

    // Work items come from the counter until they run out (PERSIST), or one
    // per work-group.  Items are ordered by chunks of hchunk kv-heads (one,
    // or all of them when there are few items per CU), then block-row
    // descending, then kv-head, then head pair, so the longest rows of every
    // kv-head of a chunk start first.  Every wave of the work-group
    // reads the same item, so all leave together.
    __shared__ int item_sh, bad_sh;
    for (;;) {
    __syncthreads();   // every wave is done with the previous item's LDS
    if (tid == 0) {
        item_sh = (int)atomicAdd(counter, 1u);
        bad_sh = 0;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(item_sh);
    if (item >= nitems) break;
    const int nsub = SINGLE ? G : npair;      // items per (kv-head, block-row)
    const int per_chunk = hchunk * nb * nsub;
    const int c_ = item / per_chunk, r_ = item - c_ * per_chunk;
    const int I = nb - 1 - r_ / (hchunk * nsub);
    const int r2 = r_ % (hchunk * nsub);
    const int g = c_ * hchunk + r2 / nsub;
    const int pp = r2 % nsub;                 // head pair, or the head itself with one head
    const bool head_ok = SINGLE || 2 * pp + gr < G;     // odd G: the last pair has one head
    const int h = SINGLE ? g * G + pp : g * G + min(2 * pp + gr, G - 1);
    const int tq = I * BLK + rw * 32 + col;
    const int wave_last_row = I * BLK + rw * 32 + 31;

    // With SINGLE, a strictly ascending list of blocks J <= I (what the
    // selection writes) is copied into LDS as it is; any other list, and the
    // two lists of a head pair, take the general path below.
    bool listed = false;
    if constexpr (SINGLE) {
        const int cq = min(max(counts[(size_t)h * nb + I], 0), nb);
        const int32_t *lq = block_idx + ((size_t)h * nb + I) * nb;
        for (int k = tid; k < cq; k += C::NT) {
            const int J = lq[k];
            const int Jn = k + 1 < cq ? lq[k + 1] : I + 1;
            if (!(J >= 0 && J < Jn)) bad_sh = 1;
            ulist[k] = (uint32_t)J | (1u << 16);
        }
        if (tid == 0) nunion = cq;
        __syncthreads();
        listed = bad_sh == 0;
    }
    // Union of the two heads' kept lists (ascending key blocks, each tagged
    // with the heads that keep it; with SINGLE the one head's list), built in
    // LDS: membership bitmaps, then a work-group scan compacts the set blocks
    // in index order.  The bitmaps also drop repeated and out-of-range
    // entries of a malformed list.
    if (!listed) {
    for (int i = tid; i < 2 * (C::MAXNB / 32); i += C::NT) (&bits[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (SINGLE ? q > 0 : 2 * pp + q >= G) continue;
        const int hq = SINGLE ? g * G + pp : g * G + 2 * pp + q;
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
    }  // general path

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
    // Running reference maximum, kept negated (nm = -m) so the weights' FMA
    // takes it as is; +inf until the first key is seen.
    float nm = INFINITY, lsum = 0.f;

    // MFMA row r = col of the S^T tile reads K row 16*((r>>2)&1) + 4*(r>>3) + (r&3)
    // of its 32-key sub-tile, so accumulator e of lane (col, hk) is key 16*hk + e.
    const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
    const int ksw = swz_k<D>(krow);
    // Byte offset of this lane's K fragment of d-step ks inside a stage buffer
    // (row krow, swizzled slot): the buffer's own address is then a constant
    // that the LDS read takes in its offset field.
    uint32_t kfo[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) kfo[ks] = (uint32_t)(krow * (D * 2) + (((2 * ks + hk) ^ ksw) << 4));
    const int vsw = swz_v(col);

    const int nst = nunion * C::SPB;

    // Copy target of stage st: a stage past the end re-copies the last one
    // (into a buffer no one reads), so every step issues the same copies.
    auto copy_stage = [&](int st) -> int { return min(st, nst - 1); };
    // Union entry of the stage that step st copies: key block in the low 16
    // bits, bit 16+q set when head q of the pair keeps it.  Read from LDS
    // before the wait that precedes a barrier and made wave-uniform after
    // it, so no LDS round trip follows the barrier.
    auto raw_entry = [&](int st) -> uint32_t { return ulist[copy_stage(st) / C::SPB]; };
    auto uni = [&](uint32_t r) -> int { return __builtin_amdgcn_readfirstlane((int)r); };

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

    // Start the copies of stage st (key block J) into (kb, vb).  The K
    // resource is based at the stage's first key row and ends after key row
    // L-1: the rows of a short last stage past L are read as zeros (their
    // scores are masked causally).  V^T is zero-padded to Lp.
    auto issue = [&](int st, int ent, char *kb, char *vb) {
        st = copy_stage(st);
        const int J = ent & 0xffff;
        const int key0 = J * BLK + (st % C::SPB) * C::KT;
        const __amdgpu_buffer_rsrc_t rk =
            buf_rsrc_n(kbase + (size_t)key0 * Hkv * D * 2, max(L - key0, 0) * Hkv * D * 2);
        const __amdgpu_buffer_rsrc_t rv = buf_rsrc(vbase + (size_t)key0 * 2);
#pragma unroll
        for (int i = 0; i < C::IK; ++i) buf2lds16(rk, koff[i], (lds_char *)kb + (wid * C::IK + i) * 1024);
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

        // S^T sub-tile 0 (keys key0 .. key0+31) first, then sub-tile 1, so
        // that sub-tile 0's weights are formed while sub-tile 1's products
        // run.  K fragments are read four steps ahead of their products.
        f32x16 sacc[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
        constexpr int NS = 2 * C::NKS, LA = KLA;
        uint4 kf[NS];
        auto rd = [&](int s) {
            kf[s] = *reinterpret_cast<const uint4 *>(kb + kfo[s % C::NKS] + (s / C::NKS) * 32 * (D * 2));
        };
        // V^T fragments of 16-key group gi (kt = gi / 2, mm = gi % 2), one per
        // 32-row d-tile.
        auto rdv = [&](int gi, uint4 (&a)[C::NDT]) {
            const int voff = ((4 * (gi >> 1) + 2 * hk + (gi & 1)) ^ vsw) << 4;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
                a[dt] = *reinterpret_cast<const uint4 *>(vb + (dt * 32 + col) * (C::KT * 2) + voff);
        };
        auto mask_diag = [&](int kt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = key0 + kt * 32 + 16 * hk + e;
                if (key > tq) sacc[kt][e] = -INFINITY;
            }
        };
        // Weights of group gi against the reference maximum nm: packed bf16
        // pairs and their sum (the normaliser sums the same bf16 weights the
        // P.V product uses).
        auto weights = [&](int gi, float nmv, uint32_t (&pk)[4]) -> float {
            const int kt = gi >> 1, mm = gi & 1;
            float gs = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sacc[kt][8 * mm + 2 * e], scale2, nmv));
                const float p1 = fast_exp2(fmaf(sacc[kt][8 * mm + 2 * e + 1], scale2, nmv));
                pk[e] = pack_bf16x2(p0, p1);
                gs = add_bf16x2(pk[e], gs);
            }
            return gs;
        };
        // Weights of the two groups of sub-tile kt; if a lane's sum for
        // either exceeds kGroupMax, the reference maximum moves to the
        // maximum over both groups, O and the normaliser are rescaled and
        // both groups' weights are formed again.
        auto check = [&](int kt, uint32_t (&pa)[4], uint32_t (&pb)[4], float &ga, float &gb) {
            if (__ballot(!(ga <= kGroupMax) || !(gb <= kGroupMax)) != 0ull) {
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][e]);
                const float mn = fmaxf(-nm, max_halves(mx) * scale2);
                const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(-nm - mn);
                nm = -mn;
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
                ga = weights(2 * kt, nm, pa);
                gb = weights(2 * kt + 1, nm, pb);
            }
            lsum += ga + gb;
        };
        auto pv = [&](const uint32_t (&pk)[4], const uint4 (&v)[C::NDT]) {
            const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) o[dt] = mfma32x32x16(as_bf16x8(v[dt]), pb, o[dt]);
        };

#pragma unroll
        for (int s = 0; s < LA; ++s) rd(s);
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) {
            rd(s + LA);
            __builtin_amdgcn_sched_barrier(0);
            sacc[0] = mfma32x32x16(as_bf16x8(kf[s]), qf[s], sacc[0]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (diag) mask_diag(0);

        uint4 vf[4][C::NDT];
        uint32_t pk[4][4];
        float gs[4];
        // Sub-tile 1's products, beside sub-tile 0's weights and the V^T
        // fragments of groups 0 and 1.
#pragma unroll
        for (int s = C::NKS; s < NS; ++s) {
            if (s + LA < NS) rd(s + LA);
            sacc[1] = mfma32x32x16(as_bf16x8(kf[s]), qf[s - C::NKS], sacc[1]);
        }
        rdv(0, vf[0]);
        rdv(1, vf[1]);
        gs[0] = weights(0, nm, pk[0]);
        gs[1] = weights(1, nm, pk[1]);
        __builtin_amdgcn_sched_barrier(0);
        check(0, pk[0], pk[1], gs[0], gs[1]);
        if (diag) mask_diag(1);

        // Groups 0 and 1's products, beside sub-tile 1's weights and the V^T
        // fragments of groups 2 and 3.
        pv(pk[0], vf[0]);
        pv(pk[1], vf[1]);
        rdv(2, vf[2]);
        rdv(3, vf[3]);
        gs[2] = weights(2, nm, pk[2]);
        gs[3] = weights(3, nm, pk[3]);
        __builtin_amdgcn_sched_barrier(0);
        check(1, pk[2], pk[3], gs[2], gs[3]);
        pv(pk[2], vf[2]);
        pv(pk[3], vf[3]);
    };

    // Stages are taken two at a time between barriers, from two pairs of
    // buffers: while one pair is computed the copies of the next two stages
    // fill the other.  One barrier per pair: every wave's copies of the pair
    // have landed (vmcnt 0) and every wave has finished reading the other
    // pair (lgkmcnt 0) before it.  The copies are issued between the pair's
    // two stages rather than right after the barrier (measured faster: their
    // landing then overlaps the second stage's products instead of the
    // first's).
    if constexpr (SINGLE) {
        // One head: two buffers, one stage per barrier.
        if (nst > 0) {
            issue(0, uni(raw_entry(0)), Kb0, Vb0);
            for (int st = 0; st < nst; st += 2) {
                {
                    const uint32_t r0 = raw_entry(st), r1 = raw_entry(st + 1);
                    wait_vmcnt<0>();
                    wait_lgkm0();
                    bar();
                    issue(st + 1, uni(r1), Kb1, Vb1);
                    compute(st, uni(r0), Kb0, Vb0);
                }
                if (st + 1 >= nst) break;
                {
                    const uint32_t r1 = raw_entry(st + 1), r2 = raw_entry(st + 2);
                    wait_vmcnt<0>();
                    wait_lgkm0();
                    bar();
                    issue(st + 2, uni(r2), Kb0, Vb0);
                    compute(st + 1, uni(r1), Kb1, Vb1);
                }
            }
            wait_vmcnt<0>();
        }
    } else if (nst > 0) {
        issue(0, uni(raw_entry(0)), Kb0, Vb0);
        issue(1, uni(raw_entry(1)), Kb1, Vb1);
        for (int st = 0; st < nst; st += 4) {
            {
                const uint32_t r0 = raw_entry(st), r1 = raw_entry(st + 1);
                const uint32_t r2 = raw_entry(st + 2), r3 = raw_entry(st + 3);
                wait_vmcnt<0>();
                wait_lgkm0();
                bar();
                compute(st, uni(r0), Kb0, Vb0);
                issue(st + 2, uni(r2), Kb2, Vb2);
                issue(st + 3, uni(r3), Kb3, Vb3);
                compute(st + 1, st + 1 < nst ? uni(r1) : -1, Kb1, Vb1);
            }
            if (st + 2 >= nst) break;
            {
                const uint32_t r2 = raw_entry(st + 2), r3 = raw_entry(st + 3);
                const uint32_t r4 = raw_entry(st + 4), r5 = raw_entry(st + 5);
                wait_vmcnt<0>();
                wait_lgkm0();
                bar();
                compute(st + 2, uni(r2), Kb2, Vb2);
                issue(st + 4, uni(r4), Kb0, Vb0);
                issue(st + 5, uni(r5), Kb1, Vb1);
                compute(st + 3, st + 3 < nst ? uni(r3) : -1, Kb3, Vb3);
            }
        }
        wait_vmcnt<0>();
    }

    const float tot = sum_halves(lsum);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (tq < L && head_ok) {
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
    if constexpr (!PERSIST) break;
    }  // work items
}

hipError_t launch_transpose_v(const uint16_t *V, const Shape &s, uint16_t *Vt, unsigned *counter,
                              hipStream_t st) {
    const int Lp = s.nb * s.B;
    hipLaunchKernelGGL(rr_transpose_v, dim3(Lp / 64, s.d / 64, s.Hkv), dim3(256), 0, st, V, s.L, Lp,
                       s.Hkv, s.d, Vt, counter);
    return hipGetLastError();
}

// Longest block count for which the persistent form is launched.
constexpr int kPersistMaxNb = 512;
// Longest block count for which one head per work-group serves every G.
constexpr int kSingleMaxNb = 128;
// Items per resident work-group (one per CU with head pairs, two with one
// head) up to which the items of all kv-heads are interleaved (block-rows
// descending over every kv-head: the longest rows start first, which matters
// when each work-group takes only a few items).  With more items per
// work-group one kv-head at a time keeps the K/V in use small: with head
// pairs, interleaving two kv-heads measured 8% slower at 128K and 2.5%
// slower at 32K, all eight 10% faster at 8K (4 items per CU).
constexpr int kInterleaveMaxItemsPerCu = 8;


template <int D, int BLK, bool OUT_F32, bool PERSIST, bool SINGLE>
static void launch_fa_k(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, unsigned *counter,
                        const Shape &s, int nitems, int hchunk, const int32_t *counts,
                        const int32_t *block_idx, void *O, unsigned grid, hipStream_t st) {
    const float scale2 = kLog2e / sqrtf((float)D);
    hipLaunchKernelGGL((rr_block_sparse_fa<D, BLK, OUT_F32, PERSIST, SINGLE>), dim3(grid),
                       dim3(FaCfg<D, BLK, SINGLE>::NT), 0, st, Q, K, Vt, counter, nitems, hchunk, s.L,
                       s.nb * BLK, s.Hq, s.Hkv, s.nb, counts, block_idx, O, scale2);
}

// SINGLE (one head per work-group) is launched in the persistent form only,
// as are head pairs of 64-row blocks up to kPersistMaxNb blocks; head pairs of
// 128-row blocks serve rows longer than that, one work-group per item.
template <int D, int BLK, bool SINGLE>
static void launch_fa_t(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt, unsigned *counter,
                        const Shape &s, const int32_t *counts, const int32_t *block_idx, void *O,
                        bool out_f32, hipStream_t st) {
    const int nitems = s.nb * s.Hkv * (SINGLE ? s.G : (s.G + 1) / 2);
    const int ncu = device_cu_count();
    const int slots = (SINGLE ? 2 : 1) * ncu;   // resident work-groups of the persistent form
    const int hchunk = nitems <= kInterleaveMaxItemsPerCu * slots ? s.Hkv : 1;
    constexpr bool kPersistOnly = SINGLE;
    constexpr bool kPersistNever = !SINGLE && BLK == 128;
    const bool persist = kPersistOnly || (!kPersistNever && s.nb <= kPersistMaxNb);
    if (persist) {
        if constexpr (!kPersistNever) {
            const unsigned grid = (unsigned)std::min(nitems, slots);
            if (out_f32)
                launch_fa_k<D, BLK, true, true, SINGLE>(Q, K, Vt, counter, s, nitems, hchunk, counts, block_idx, O,
                                                        grid, st);
            else
                launch_fa_k<D, BLK, false, true, SINGLE>(Q, K, Vt, counter, s, nitems, hchunk, counts, block_idx,
                                                         O, grid, st);
        }
    } else {
        if constexpr (!kPersistOnly) {
            if (out_f32)
                launch_fa_k<D, BLK, true, false, SINGLE>(Q, K, Vt, counter, s, nitems, hchunk, counts, block_idx,
                                                         O, (unsigned)nitems, st);
            else
                launch_fa_k<D, BLK, false, false, SINGLE>(Q, K, Vt, counter, s, nitems, hchunk, counts,
                                                          block_idx, O, (unsigned)nitems, st);
        }
    }
}

hipError_t launch_block_sparse_fa(const uint16_t *Q, const uint16_t *K, const uint16_t *Vt,
                                  unsigned *counter, const Shape &s, const int32_t *counts,
                                  const int32_t *block_idx, void *O, bool out_f32, hipStream_t st) {
    // One query head per work-group, two work-groups per CU (the persistent
    // form), for short rows, and up to kPersistMaxNb blocks for an odd G,
    // whose last head pair would hold a single head; head pairs otherwise.
    // Measured against the other form: 8K Llama-shaped rows (64 blocks)
    // 2.5% faster with one head, 32K (256 blocks, G = 4) 3.5% faster in
    // pairs, the 64K video shape (512 blocks, G = 7) 11% faster with one
    // head.
    const bool single = s.nb <= kSingleMaxNb || ((s.Hq / s.Hkv) % 2 == 1 && s.nb <= kPersistMaxNb);
    if (s.d == 128 && s.B == 128) {
        if (single) launch_fa_t<128, 128, true>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
        else launch_fa_t<128, 128, false>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
    } else if (s.d == 128 && s.B == 64)
        launch_fa_t<128, 64, false>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
    else if (s.d == 64 && s.B == 128) {
        if (single) launch_fa_t<64, 128, true>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
        else launch_fa_t<64, 128, false>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
    } else
        launch_fa_t<64, 64, false>(Q, K, Vt, counter, s, counts, block_idx, O, out_f32, st);
    return hipGetLastError();
}

}  // namespace rr
