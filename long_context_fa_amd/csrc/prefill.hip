// prefill.hip -- blockwise online-softmax attention forward with BLASST block
// skipping, for gfx950.
//
// Method: "BLASST: Dynamic BLocked Attention Sparsity via Softmax
// Thresholding" (gist.science/pt/paper/2512.12087, section 2): for each key
// block, form the block-local row max m~ from the scores the FlashAttention
// loop already computes; when m~ - m < ln(lambda) against the running row max
// m the block is skipped: no exponential, no V-block load, no P.V product.
// Prefill is compute bound (page 1 section 3; Hindi explainer, section 2
// "kernel optimisation"), so the savings are the exp work and the P.V MFMAs;
// here the V load is also predicated on the decision.
//
// Work decomposition (one workgroup per (query tile, query head, batch)):
//  * BR query rows, BR/32 waves, each wave owns 32 consecutive query rows.
//  * Scores are computed transposed, S^T = K_j Q^T, with the 32x32x16 bf16
//    MFMA: lane (n, h) holds query n's scores for 32 of the 64 keys, so the
//    row max, running max, running sum and rescale are per-lane scalars and
//    the only cross-lane step is one exchange with lane n+32.
//  * The P^T registers feed the P.V product O^T += V^T P^T directly as the
//    B operand (no shuffles); V^T is staged in LDS by a transposing store.
//  * Skip vote: a lane meets the test when its row does; the tile skips when
//    every valid row of every wave does (one LDS word per wave, exchanged at
//    the barrier the K double-use needs anyway), so the branch is uniform.
//  * Base-2 arithmetic: scores are scaled by scale*log2(e) in fp32, the test
//    compares against log2(lambda), exponentials are v_exp_f32.
#include "device.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int BC = 64; // key block

template <int D, int BR, bool CAUSAL, bool SKIP, bool OUT_BF16>
__global__ __launch_bounds__(2 * BR) __attribute__((amdgpu_waves_per_eu((D * 64 / BR) <= 64 ? 2 : 1, 2))) void prefill_kernel(const PrefillArgs a)
{
    constexpr int NW = BR / 32;         // waves
    constexpr int NT = 64 * NW;         // threads
    constexpr int KP = D + 8;           // K row pitch in LDS (elements)
    constexpr int VP = BC + 4;          // V^T row pitch in LDS (elements)
    constexpr int DG = D / 8;           // 16-byte groups per row
    constexpr int KCH = BC * DG / NT;   // K chunks of 16 B per thread
    constexpr int VK = BC * DG / NT;    // keys per thread in the V^T store
    static_assert(KCH >= 1 && VK >= 2 && VK % 2 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
    __shared__ int vote[NW];
    __shared__ float gapw[NW];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, hh = lane >> 5;

    // Longest (latest) query tiles first; heads and batches inner.
    const int per_t = a.Hq * a.B;
    const int t = a.nqt - 1 - (int)blockIdx.x / per_t;
    const int rem = (int)blockIdx.x % per_t;
    const int h = rem % a.Hq, b = rem / a.Hq;
    const int hk = h / (a.Hq / a.Hkv);
    const int r0 = t * BR;
    const int L = a.L;
    const int qrow = r0 + 32 * w + n;
    const bool row_valid = qrow < L;
    const bool want_maps = a.skip_map != nullptr || a.gap_map != nullptr;

    const uint16_t *qp = a.q + b * a.q_sb + h * a.q_sh;
    const uint16_t *kp = a.k + b * a.k_sb + hk * a.k_sh;
    const uint16_t *vp = a.v + b * a.v_sb + hk * a.v_sh;

    // Q^T as the B operand: lane (n, hh) holds q[qrow][16kk + 8hh .. +7].
    bf16x8 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 u = {0, 0, 0, 0};
        if (row_valid)
            u = *(const u32x4 *)(qp + (int64_t)qrow * a.q_st + 16 * kk + 8 * hh);
        qf[kk] = as_bf16x8(u);
    }

    const int last_row = (r0 + BR < L ? r0 + BR : L) - 1;
    const int nvis = CAUSAL ? (last_row / BC + 1 < a.nkb ? last_row / BC + 1 : a.nkb) : a.nkb;

    // K tile: row-major [64][D] in LDS, 16-byte chunks, coalesced rows.
    u32x4 kr[KCH];
    auto load_k = [&](int j) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT, row = c / DG, col = c % DG;
            const int key = j * BC + row;
            u32x4 u = {0, 0, 0, 0};
            if (key < L)
                u = *(const u32x4 *)(kp + (int64_t)key * a.k_st + col * 8);
            kr[i] = u;
        }
    };
    auto store_k = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT, row = c / DG, col = c % DG;
            *(u32x4 *)(Ks + row * KP + col * 8) = kr[i];
        }
    };
    // V tile: thread owns VK consecutive keys x 8 features; stored transposed
    // ([D][64] with pitch VP) so that a lane's MFMA operand is 4 consecutive keys.
    const int vkg = (tid & 3) + 4 * (tid / (4 * DG));
    const int vdg = (tid >> 2) % DG;
    u32x4 vr[VK];

    load_k(0);
    store_k();
    __syncthreads();

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = f32x16{};
    float m2 = neg_inf(); // running max of this lane's row (base-2 units)
    float lsum = 0.f;     // running sum over this lane's half of each block
    int n_skipped = 0;

    for (int j = 0; j < nvis; ++j) {
        if (j + 1 < nvis)
            load_k(j + 1);

        // S^T = K_j Q^T: two 32-key tiles.
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                bf16x8 ka = as_bf16x8(*(const u32x4 *)(Ks + (32 * kt + n) * KP + 16 * kk + 8 * hh));
                s[kt] = mfma32(ka, qf[kk], s[kt]);
            }
        }
        // Mask the causal diagonal and the ragged tail (-inf entries).
        const int k0 = j * BC;
        if ((CAUSAL && k0 + BC - 1 > r0) || k0 + BC > L) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= L || (CAUSAL && key > qrow))
                        s[kt][r] = neg_inf();
                }
        }
        float mt = neg_inf();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mt = fmaxf(mt, s[kt][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mt2 = mt * a.scale_log2; // block-local row max, base 2

        bool skip = false;
        if (SKIP || want_maps) {
            // d = m~ - m with the infinity rules: -inf if the row sees no key in
            // the block, +inf if the row has no running max yet.
            const float dgap = (!row_valid || mt2 == neg_inf()) ? neg_inf() : mt2 - m2;
            if (SKIP) {
                const bool ok = !(dgap >= a.lnlam2); // also true for -inf rows
                const int wall = __all(ok);
                if (lane == 0)
                    vote[w] = wall;
            }
            if (want_maps) {
                const float wg = wave_max(dgap);
                if (lane == 0)
                    gapw[w] = wg;
            }
        }
        __syncthreads(); // (A) votes visible; every wave is done reading Ks

        if (SKIP) {
            int all = 1;
#pragma unroll
            for (int i = 0; i < NW; ++i)
                all &= vote[i];
            skip = all != 0;
        }
        if (want_maps && tid == 0) {
            float g = neg_inf();
#pragma unroll
            for (int i = 0; i < NW; ++i)
                g = fmaxf(g, gapw[i]);
            const int64_t idx = ((int64_t)(b * a.Hq + h) * a.nqt + t) * a.nkb + j;
            if (a.skip_map)
                a.skip_map[idx] = skip ? 1 : 0;
            if (a.gap_map)
                a.gap_map[idx] = g * 0.69314718055994531f; // back to natural log
        }

        if (!skip) {
            // V_j loads, issued only for executed blocks.
#pragma unroll
            for (int i = 0; i < VK; ++i) {
                const int key = k0 + vkg * VK + i;
                u32x4 u = {0, 0, 0, 0};
                if (key < L)
                    u = *(const u32x4 *)(vp + (int64_t)key * a.v_st + vdg * 8);
                vr[i] = u;
            }
            // Online-softmax update of this lane's row.
            const float mnew = fmaxf(m2, mt2);
            const float msafe = mnew == neg_inf() ? 0.f : mnew;
            const float alpha = exp2_hw(m2 - msafe);
            float rs = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x8 lo, hi;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float p0 = exp2_hw(__builtin_fmaf(s[kt][r], a.scale_log2, -msafe));
                    const float p1 = exp2_hw(__builtin_fmaf(s[kt][r + 8], a.scale_log2, -msafe));
                    lo[r] = p0;
                    hi[r] = p1;
                    rs += p0 + p1;
                }
                pf[2 * kt] = cvt_bf16x8(lo);
                pf[2 * kt + 1] = cvt_bf16x8(hi);
            }
            lsum = alpha * lsum + rs;
            m2 = mnew;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                o[dt] *= alpha;
            // Transposing store of V_j into Vt[d][key].
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = vdg * 8 + e;
#pragma unroll
                for (int i = 0; i < VK; i += 2) {
                    const uint32_t x = vr[i][e >> 1], y = vr[i + 1][e >> 1];
                    const uint32_t packed = (e & 1) ? ((x >> 16) | (y & 0xffff0000u))
                                                    : ((x & 0xffffu) | (y << 16));
                    *(uint32_t *)(Vt + d * VP + vkg * VK + i) = packed;
                }
            }
            __syncthreads(); // (B) V^T visible
            // O^T += V^T P^T, k-steps of 16 keys.
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const uint16_t *vrow = Vt + (32 * dt + n) * VP + 16 * u + 4 * hh;
                    const u32x2 lo = *(const u32x2 *)vrow;
                    const u32x2 hi = *(const u32x2 *)(vrow + 8);
                    const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
                    o[dt] = mfma32(as_bf16x8(va), pf[u], o[dt]);
                }
            }
        } else {
            ++n_skipped;
        }
        if (j + 1 < nvis)
            store_k();
        __syncthreads(); // (C) next K visible; V^T reads done
    }

    // Finalize: O = acc / l, l summed over the two lane halves.
    const float l = lsum + __shfl_xor(lsum, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_valid) {
        char *ob = (char *)a.o;
        const int64_t base = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)qrow * a.o_st;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                f32x4 v4 = {o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                            o[dt][4 * g + 3] * inv};
                if (OUT_BF16) {
                    bf16x4 bv = __builtin_convertvector(v4, bf16x4);
                    *(bf16x4 *)(ob + 2 * (base + d)) = bv;
                } else {
                    *(f32x4 *)(ob + 4 * (base + d)) = v4;
                }
            }
    }
    if (tid == 0) {
        if (want_maps)
            for (int j = nvis; j < a.nkb; ++j) {
                const int64_t idx = ((int64_t)(b * a.Hq + h) * a.nqt + t) * a.nkb + j;
                if (a.skip_map)
                    a.skip_map[idx] = 255;
                if (a.gap_map)
                    a.gap_map[idx] = neg_inf();
            }
        if (a.counters) {
            atomicAdd(a.counters, (unsigned long long)nvis);
            atomicAdd(a.counters + 1, (unsigned long long)n_skipped);
        }
    }
}

template <int D, int BR, bool CAUSAL, bool SKIP, bool OUT_BF16>
hipError_t launch_one(const PrefillArgs &a, hipStream_t stream)
{
    const unsigned grid = (unsigned)a.nqt * (unsigned)a.Hq * (unsigned)a.B;
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL((prefill_kernel<D, BR, CAUSAL, SKIP, OUT_BF16>), dim3(grid), dim3(2 * BR), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int BR>
hipError_t launch_tile(const PrefillArgs &a, bool causal, bool skip, bool out_bf16, hipStream_t s)
{
    if (causal) {
        if (skip)
            return out_bf16 ? launch_one<D, BR, true, true, true>(a, s) : launch_one<D, BR, true, true, false>(a, s);
        return out_bf16 ? launch_one<D, BR, true, false, true>(a, s) : launch_one<D, BR, true, false, false>(a, s);
    }
    if (skip)
        return out_bf16 ? launch_one<D, BR, false, true, true>(a, s) : launch_one<D, BR, false, true, false>(a, s);
    return out_bf16 ? launch_one<D, BR, false, false, true>(a, s) : launch_one<D, BR, false, false, false>(a, s);
}

} // namespace

hipError_t launch_prefill(const PrefillArgs &a, int d, int tile_q, bool causal, bool skip, bool out_bf16,
                          hipStream_t stream)
{
    if (d == 128 && tile_q == 128)
        return launch_tile<128, 128>(a, causal, skip, out_bf16, stream);
    if (d == 128 && tile_q == 64)
        return launch_tile<128, 64>(a, causal, skip, out_bf16, stream);
    if (d == 64 && tile_q == 128)
        return launch_tile<64, 128>(a, causal, skip, out_bf16, stream);
    if (d == 64 && tile_q == 64)
        return launch_tile<64, 64>(a, causal, skip, out_bf16, stream);
    return hipErrorInvalidValue;
}

} // namespace blasst
