// rr_attn.hip -- causal block-sparse attention with GQA over a compacted
// block list (rr_block_sparse_fa), plus the V transpose it reads.
//
// Attention runs only on the key blocks kept for each (query head, query
// block-row) (RRAttention abstract: about half of the blocks are computed);
// within a kept block it is exact causal softmax attention with scale
// 1/sqrt(d), and query head h reads kv-head h / (Hq/Hkv) (GQA).
//
// Work-group = one (query head h, query block I): BLK/32 waves, each owning 32
// query rows.  Per kept key block J (ascending):
//   * the K tile [BLK keys][d] and the V^T tile [d][BLK keys] are staged in
//     LDS (row pitch padded by 16 bytes against bank conflicts);
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16.  The K rows fed to the
//     matrix unit are permuted so that accumulator register e of lane
//     (column q, half hk) holds key 16*hk + e of each 32-key sub-tile:
//     every lane owns one query column, and the row softmax needs a single
//     cross-half exchange;
//   * online softmax in the log2 domain (scores pre-scaled by
//     log2(e)/sqrt(d)), diagonal block masked causally;
//   * P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T . P^T: its registers already hold 8 consecutive keys per
//     lane half, and the matching V^T rows are 16-byte LDS reads.
// O^T stays in registers (one query column per lane) and is divided by the
// softmax sum at the end.
//
// Grid order: (block-row descending, kv-head), the G query heads of one
// (I, g) pair adjacent and on the same XCD (work-groups are dealt to the 8
// XCDs round-robin), so the K/V tiles they share are served from that XCD's
// L2; long rows start first.
#include "rr_device.h"
#include "rr_internal.h"

namespace rr {

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

template <int D, int BLK, bool OUT_F32>
__global__ __launch_bounds__(BLK * 2) void rr_block_sparse_fa(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ Vt,
    int L, int Lp, int Hq, int Hkv, int nb, int nq, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ block_idx, void *__restrict__ O, float scale2) {
    constexpr int NT = BLK * 2;   // threads
    constexpr int KP = D + 8;     // K tile pitch (elements)
    constexpr int VP = BLK + 8;   // V^T tile pitch (elements)
    constexpr int NSUB = BLK / 32;
    constexpr int NDT = D / 32;
    constexpr int NKS = D / 16;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[D * VP];

    const int G = Hq / Hkv;
    // XCD-aware decode: x = XCD slot, then heads of one (I, g) pair.
    const int bx = blockIdx.x;
    const int x = bx & 7, slot = bx >> 3;
    const int hh = slot % G;
    const int qi = (slot / G) * 8 + x;
    if (qi >= nq) return;
    const int I = nb - 1 - qi / Hkv;
    const int g = qi % Hkv;
    const int h = g * G + hh;

    const int tid = threadIdx.x;
    const int wid = tid >> 6, lane = tid & 63;
    const int col = lane & 31, hk = lane >> 5;
    const int tq = I * BLK + wid * 32 + col;

    bf16x8 qf[NKS];
    {
        const bool ok = tq < L;
        const uint16_t *qp = Q + ((size_t)(ok ? tq : 0) * Hq + h) * D + hk * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = ok ? as_bf16x8(ld16(qp + ks * 16)) : as_bf16x8(zero_u4());
    }

    f32x16 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    // Key row of the K tile fed as MFMA row r = col: 16*((r>>2)&1) + 4*(r>>3) + (r&3).
    const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

    // A malformed list (count outside [0, nb], index outside [0, I]) must not
    // read outside K / V^T: such entries are skipped.
    const int cnt = min(max(counts[(size_t)h * nb + I], 0), nb);
    const int32_t *lst = block_idx + ((size_t)h * nb + I) * nb;
    for (int it = 0; it < cnt; ++it) {
        const int J = lst[it];
        if ((unsigned)J > (unsigned)I) continue;  // uniform across the work-group
        // Stage K tile and V^T tile.
#pragma unroll
        for (int cidx = tid; cidx < BLK * D / 8; cidx += NT) {
            const int r = cidx / (D / 8), c8 = cidx % (D / 8);
            const int key = J * BLK + r;
            uint4 v = zero_u4();
            if (key < L) v = ld16(K + ((size_t)key * Hkv + g) * D + c8 * 8);
            st16(&Ks[r * KP + c8 * 8], v);
        }
#pragma unroll
        for (int cidx = tid; cidx < D * BLK / 8; cidx += NT) {
            const int r = cidx / (BLK / 8), c8 = cidx % (BLK / 8);
            st16(&Vs[r * VP + c8 * 8], ld16(Vt + ((size_t)g * D + r) * Lp + (size_t)J * BLK + c8 * 8));
        }
        __syncthreads();

        f32x16 sacc[NSUB];
#pragma unroll
        for (int kt = 0; kt < NSUB; ++kt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
            const uint16_t *kr = &Ks[(kt * 32 + krow) * KP + hk * 8];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                sacc[kt] = mfma32x32x16(as_bf16x8(ld16(kr + ks * 16)), qf[ks], sacc[kt]);
        }

        float mx = -INFINITY;
        const bool diag = (J == I);
#pragma unroll
        for (int kt = 0; kt < NSUB; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float s = sacc[kt][e] * scale2;
                if (diag) {
                    const int key = J * BLK + kt * 32 + 16 * hk + e;
                    if (key > tq) s = -INFINITY;
                }
                sacc[kt][e] = s;
                mx = fmaxf(mx, s);
            }
        mx = fmaxf(mx, xor_lane(mx, 32));
        const float mnew = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;

#pragma unroll
        for (int kt = 0; kt < NSUB; ++kt) {
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = fast_exp2(sacc[kt][8 * mm + 2 * e] - mnew);
                    const float p1 = fast_exp2(sacc[kt][8 * mm + 2 * e + 1] - mnew);
                    lsum += p0 + p1;
                    pk[e] = pack_bf16x2(p0, p1);
                }
                const bf16x8 pb = as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3]));
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const uint16_t *vr = &Vs[(dt * 32 + col) * VP + kt * 32 + 16 * hk + 8 * mm];
                    o[dt] = mfma32x32x16(as_bf16x8(ld16(vr)), pb, o[dt]);
                }
            }
        }
        __syncthreads();
    }

    const float tot = lsum + xor_lane(lsum, 32);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (tq >= L) return;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
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
    const dim3 grid((unsigned)(nq8 * s.G));
    const float scale2 = kLog2e / sqrtf((float)D);
    const int Lp = s.nb * BLK;
    if (out_f32)
        hipLaunchKernelGGL((rr_block_sparse_fa<D, BLK, true>), grid, dim3(BLK * 2), 0, st, Q, K, Vt,
                           s.L, Lp, s.Hq, s.Hkv, s.nb, nq, counts, block_idx, O, scale2);
    else
        hipLaunchKernelGGL((rr_block_sparse_fa<D, BLK, false>), grid, dim3(BLK * 2), 0, st, Q, K,
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
