// prefill.hip -- blockwise online-softmax attention forward with BLASST block
// skipping, for gfx950.
//
// Method: "BLASST: Dynamic BLocked Attention Sparsity via Softmax
// Thresholding" (gist.science/pt/paper/2512.12087, section 2): for each key
// block, form the block-local row max m~ from the scores the FlashAttention
// loop already computes; when m~ - m < ln(lambda) against the running row max
// m the block is skipped: no exponential, no V-block load, no P.V product.
// Prefill is compute bound (BLASST summary, section 3; Hindi explainer, section 2
// "kernel optimisation"), so the savings are the exp work and the P.V MFMAs;
// here the V load is also predicated on the decision.
//
// Work decomposition (one workgroup per (query tile, query head, batch)):
//  * BR query rows, BR/32 waves, each wave owns 32 consecutive query rows.
//  * Scores are computed transposed, S^T = K_j Q^T, with the 32x32x16 bf16
//    MFMA: lane (n, h) holds query n's scores for 32 of the 64 keys, so the
//    row max, running max, running sum and rescale are per-lane scalars and
//    the only cross-lane step is one exchange with lane n+32.
//  * The P^T registers feed O^T += V^T P^T directly as the B operand.  V stays
//    row-major in LDS; its A operand (4 consecutive keys of one feature per
//    lane) comes from the gfx950 transpose read ds_read_b64_tr_b16.
//  * K and V tiles are copied global -> LDS with global_load_lds_dwordx4 (no
//    registers), into a row-major layout whose 16-byte chunks are XOR-swizzled
//    by row (pswz) so that MFMA operand reads are bank-conflict free.  K and V
//    each run in a ring of 2 buffers; V is requested only once the block's
//    vote says it executes, one iteration before its P.V product.
//  * Software pipeline with one barrier per key block: iteration j finishes
//    the P.V product of block j-1, forms the scores of block j+1 and the
//    softmax of block j, so a skipped block costs its Q.K product, its row
//    max and its vote, and a V copy has most of an iteration to land.
//  * Skip vote: a lane meets the test when its row does; the tile skips when
//    every valid row of every wave does (one LDS byte per wave, the bytes
//    read back as one word after the barrier that also publishes the next
//    K tile), so the branch is uniform across the workgroup.
//  * Base-2 arithmetic: scores are scaled by scale*log2(e) in fp32, the test
//    compares against log2(lambda), exponentials are v_exp_f32.  The
//    accumulator rescale is skipped when no row of the wave raised its max
//    (after the first blocks the running max rarely moves).
//  * Gap pass (GAPS): the same loop with the executed work removed -- no V
//    copy, no exponential, no P.V, no O -- and the running max advanced over
//    every block.  A skip never changes the running max (a skipped block has
//    m~ < m + ln(lambda) <= m), so these are the gaps and decisions of the
//    full pass; calibration needs only them (BLASST summary, section 2
//    "Calibracao Automatica": lambda is found by a search over the achieved
//    sparsity).
#include "device.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int BC = 64;       // key block

// Chunk swizzle of the K and V tiles: physical 16-byte chunk = logical chunk ^
// pswz(row).  The K operand read (ds_read_b128) serves 16 lanes per LDS cycle:
// 16 consecutive rows at one logical chunk.  The V^T operand read
// (ds_read_b64_tr_b16) serves 32 lanes: a 4-aligned quad of rows x an aligned
// group of 4 chunks.  256-byte rows (d = 128) each span all banks, so the
// swizzle must permute the rows mod 16 and give the 4 rows of a quad distinct
// bits 2-3.  128-byte rows (d = 64) share a bank line in pairs, so with e =
// row / 2 it must permute e mod 8 and give e and e+1 (e even) distinct bit 2.
template <int DG>
__device__ __forceinline__ int pswz(int row)
{
    if (DG > 8)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    const int e = row >> 1;
    return ((e & 1) << 2) | ((e >> 1) & 3);
}

// Phase 0..3 of query tile t in the unit order: four stretches of equal work.
// A causal head's tiles >= t carry work ~nqt^2 - t^2, so the quarters end at
// nqt * sqrt(3/4), sqrt(1/2), sqrt(1/4); without causal masking, at 3/4, 1/2,
// 1/4 of nqt.
template <bool CAUSAL>
__device__ __forceinline__ int tile_phase(int t, int nqt)
{
    const int t1 = CAUSAL ? (int)(((int64_t)nqt * 222) >> 8) : (int)(((int64_t)nqt * 3) >> 2);
    const int t2 = CAUSAL ? (int)(((int64_t)nqt * 181) >> 8) : nqt >> 1;
    const int t3 = CAUSAL ? nqt >> 1 : nqt >> 2;
    return t >= t1 ? 0 : t >= t2 ? 1 : t >= t3 ? 2 : 3;
}

template <int D, int BR, bool CAUSAL, bool SKIP, bool OUT_BF16, bool GAPS>
__global__ __launch_bounds__(2 * BR)
__attribute__((amdgpu_waves_per_eu((D * 64 / BR) <= 64 ? 2 : 1, GAPS ? 4 : 2))) // no O or P: the gap pass fits more
void prefill_kernel(const PrefillArgs a)
{
    constexpr int NW = BR / 32;          // waves
    constexpr int RB = D * 2;            // bytes per K/V row
    constexpr int DG = D / 8;            // 16-byte chunks per row
    constexpr int TB = BC * RB;          // bytes per tile
    constexpr int KI = TB / 1024 / NW;   // 1 KB copy instructions per tile per wave
    constexpr int RPI = 64 / DG;         // rows per copy instruction
    static_assert(KI >= 1 && KI * NW * 1024 == TB, "tile shape");

    // K ring (2 tiles) and V ring (2 tiles).
    __shared__ __attribute__((aligned(1024))) char smem[(GAPS ? 2 : 4) * TB]; // the gap pass has no V ring
    // Tile votes, one byte per wave (1: every row of the wave meets the
    // test); bytes past NW stay 1, so the tile skips when the word reads
    // 0x01010101 -- one LDS read and one scalar compare per block.
    __shared__ __attribute__((aligned(4))) uint8_t vote[2][4];
    __shared__ float gapw[2][NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;

    // Unit mapping.  Longest (latest) query tiles first.  Consecutive
    // workgroups go to the 8 XCDs in turn; when the KV groups divide evenly,
    // an XCD serves one KV group in each of four phases of the tile order
    // (of equal work, tile_phase), so
    // that group's K/V stays in its L2.  The group changes with the phase --
    // XCD x serves groups x, x^4, x^2, x^6 (+8k) in turn -- so that groups
    // that skip less do not all land on one XCD: each XCD carries a quarter
    // of four groups' work.  With fewer than 8 groups, each group is spread
    // over 8 / (B * Hkv) XCDs by head slices, with the same rotation.
    const int G = a.Hq / a.Hkv;
    const int nkvg = a.B * a.Hkv;
    int t, h, b;
    {
        const int k = blockIdx.x;
        if (nkvg % 8 == 0) {
            // Group-major within an XCD: with several KV groups per XCD
            // (B * Hkv > 8), column j -- one group per phase -- is walked
            // longest tile first before column j + 1, so the XCD's L2 holds
            // one group's K/V at a time and the grid still ends on short tiles.
            const int xcd = k & 7, s = k >> 3;
            const int per_col = a.nqt * G;
            const int jcol = s / per_col, rem = s % per_col;
            t = a.nqt - 1 - rem / G;
            const int p = tile_phase<CAUSAL>(t, a.nqt);
            const int c = ((p & 1) << 2) | (p & 2); // 0, 4, 2, 6
            const int kvg = jcol * 8 + (xcd ^ c);
            b = kvg / a.Hkv;
            h = (kvg % a.Hkv) * G + rem % G;
        } else if (8 % nkvg == 0 && G % (8 / nkvg) == 0) {
            // Fewer than 8 KV groups (B * Hkv in {1, 2, 4}): each group is
            // spread over 8 / (B * Hkv) XCDs, each taking an equal slice of
            // its query heads, so an XCD's L2 holds one group's K/V.  The
            // group of a slice rotates with the same four phases as above.
            const int xcd = k & 7, s = k >> 3;
            const int gh = G * nkvg / 8; // heads per XCD
            t = a.nqt - 1 - s / gh;
            const int p = tile_phase<CAUSAL>(t, a.nqt);
            const int kvg = (xcd + p) % nkvg, slice = xcd / nkvg;
            b = kvg / a.Hkv;
            h = (kvg % a.Hkv) * G + slice * gh + s % gh;
        } else {
            const int per_t = a.Hq * a.B;
            t = a.nqt - 1 - k / per_t;
            const int r = k % per_t;
            h = r % a.Hq;
            b = r / a.Hq;
        }
    }
    const int hk = h / G;
    const int r0 = t * BR;
    const int L = a.L;
    const int qrow = r0 + 32 * w + n;
    const bool row_valid = qrow < L;
    // the gap pass always forms the tile gap (its skip count needs it)
    const bool want_maps = GAPS || a.skip_map != nullptr || a.gap_map != nullptr;

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
    // Sliding window (causal): row i sees keys > i - win, so the tile visits
    // blocks jlo .. nvis-1, every one of which some row sees.
    const int jlo = CAUSAL && r0 - a.win + 1 > 0 ? (r0 - a.win + 1) / BC : 0;

    // Tile copy: wave w fills rows [w*KI*RPI, (w+1)*KI*RPI); lane -> (row, chunk)
    // with the chunk XOR-swizzled by the row (pswz).  Per-lane byte offsets of
    // a whole tile are computed once: a block that lies entirely inside the
    // tile's key range costs one scalar add per tile copy.  Keys no row of the
    // tile sees -- past L, or below the window of its first row -- re-read the
    // nearest key some row sees (kmin or L-1): they are masked to -inf, and
    // their 0 * V then repeats a value the tile already multiplies, so a
    // non-finite V outside the tile's keys never reaches it.
    uint32_t koff[KI], voff[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int row = (w * KI + i) * RPI + lane / DG;
        const int c = (lane % DG) ^ pswz<DG>(row);
        koff[i] = (uint32_t)((row * a.k_st + c * 8) * 2);
        voff[i] = (uint32_t)((row * a.v_st + c * 8) * 2);
    }
    const int kmin = CAUSAL && r0 - a.win + 1 > 0 ? r0 - a.win + 1 : 0; // lowest key a row of the tile sees
    auto copy_tile = [&](const uint16_t *base, int64_t st, const uint32_t *off, int j, uint32_t dst) {
        if ((j + 1) * BC <= L && j * BC >= kmin) {
            const uint16_t *sb = base + (int64_t)j * BC * st;
#pragma unroll
            for (int i = 0; i < KI; ++i)
                copy16_to_lds_s(sb, off[i], dst + (w * KI + i) * 1024u);
        } else {
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int ins = w * KI + i;
                const int row = ins * RPI + lane / DG;
                const int c = (lane % DG) ^ pswz<DG>(row);
                int key = j * BC + row;
                key = key < L ? (key > kmin ? key : kmin) : L - 1;
                copy16_to_lds(base + (int64_t)key * st + c * 8, dst + ins * 1024u);
            }
        }
    };
    auto kbuf = [&](int j) { return smem + (j & 1) * TB; };
    auto vbuf = [&](int j) { return smem + (2 + (j & 1)) * TB; };
    // the same slots as LDS byte addresses, for the copies
    const uint32_t smem_lds = lds_addr(smem);
    auto kbuf_l = [&](int j) { return smem_lds + (uint32_t)((j & 1) * TB); };
    auto vbuf_l = [&](int j) { return smem_lds + (uint32_t)((2 + (j & 1)) * TB); };

    // S^T = K_j Q^T (two 32-key tiles) with the causal / ragged mask, and the
    // block-local row max (base 2).
    auto scores = [&](int j, f32x16 (&s)[2], float &mt2) {
        const char *kb = kbuf(j);
        s[0] = f32x16{};
        s[1] = f32x16{};
        // K operands are read three k-steps ahead of their MFMAs so that the
        // LDS latency hides behind the matrix work.
        constexpr int NK = D / 16;
        // Row 32 kt + n, logical chunk 2 kk + hh: since pswz depends on the
        // row mod 16 only and 2 kk, hh occupy disjoint bits, the byte offset is
        // n RB + 32 kt RB + (32 kk ^ kx) with one lane constant kx (laundered
        // per call so that the compiler does not hoist 8 offsets per lane).
        int kx = 16 * (hh ^ pswz<DG>(n)), nrb = n * RB;
        asm volatile("" : "+v"(kx), "+v"(nrb));
        auto kread = [&](int kk, int kt) {
            return *(const u32x4 *)(kb + nrb + 32 * kt * RB + ((32 * kk) ^ kx));
        };
        u32x4 ka[3][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                ka[kk][kt] = kread(kk, kt);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            if (kk + 2 < NK) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    ka[(kk + 2) % 3][kt] = kread(kk + 2, kt);
            }
            __builtin_amdgcn_sched_barrier(0); // keep the reads ahead of the MFMAs
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                s[kt] = mfma32(as_bf16x8(ka[kk % 3][kt]), qf[kk], s[kt]);
        }
        const int k0 = j * BC;
        if ((CAUSAL && (k0 + BC - 1 > r0 || k0 <= r0 + BR - 1 - a.win)) || k0 + BC > L) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= L || (CAUSAL && (key > qrow || key <= qrow - a.win)))
                        s[kt][r] = neg_inf();
                }
        }
        float mt = neg_inf();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mt = fmaxf(mt, s[kt][r]);
        mt2 = max_xor32(mt) * a.scale_log2;
        // The scaled block max is a rounded fp32 value in every instantiation:
        // the gap mt2 - m2 must not fuse the scale into its subtraction in
        // some kernels and not in others, so that the gap pass, the dense
        // pass and the skip pass write bit-identical gap maps.
        asm volatile("" : "+v"(mt2));
    };

    float m2 = neg_inf(); // running max of this lane's row (base 2)
    float lsum = 0.f;     // running sum over this lane's half of each block
    int n_skipped = 0;
    bool rescale = false; // O waits for a rescale by alpha_p before the next P.V
    float alpha_p = 1.f;

    // Wave vote on block j against the running max; d = m~ - m with the
    // infinity rules (-inf if the row sees no key in the block, +inf while the
    // row has no running max).
    auto vote_block = [&](int j, float mt2) {
        if (SKIP || want_maps) {
            const float dgap = (!row_valid || mt2 == neg_inf()) ? neg_inf() : mt2 - m2;
            if (SKIP) {
                const int wall = __all(!(dgap >= a.lnlam2)); // -inf rows always meet it
                if (lane == 0)
                    vote[j & 1][w] = (uint8_t)wall;
            }
            if (want_maps) {
                const float wg = wave_max(dgap);
                if (lane == 0)
                    gapw[j & 1][w] = wg;
            }
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = f32x16{};

    // V operand addressing for the transpose read (fixed per lane).
    const int vg = lane >> 4, vs = lane & 15;
    const int vmb = vg & 1, vh = vg >> 1, vj = vs >> 2, vq = vs & 3;

    // O^T += V_j^T P_j^T, k-steps of 16 keys.
    // The V^T operands are read three MFMAs ahead (flattened over (u, dt)) so
    // that the LDS latency hides behind the matrix work.
    auto pv = [&](int j, const bf16x8 (&pf)[4]) {
        // The rescale of the accumulator by the previous softmax's alpha,
        // deferred to here: the MFMAs that last wrote O finished an iteration
        // ago, so the multiply does not wait for the matrix pipe.
        if (rescale) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                o[dt] *= alpha_p;
        }
        const char *Vb = vbuf(j);
        constexpr int NDT = D / 32, NM = 4 * NDT;
        // Rows ra = 16 u + 4 vh + vj and rb = ra + 8, logical chunk
        // 4 dt + 2 vmb + vq/2: pswz of both rows does not depend on u and the
        // chunk's dt bits are disjoint from the rest, so the byte offsets are
        // vb0 + 16 u RB (+ 8 RB) + (64 dt ^ vxa or vxb) with lane constants.
        int vb0 = (4 * vh + vj) * RB + (vq & 1) * 8;
        int vxa = 16 * ((2 * vmb + (vq >> 1)) ^ pswz<DG>(4 * vh + vj));
        int vxb = 16 * ((2 * vmb + (vq >> 1)) ^ pswz<DG>(4 * vh + vj + 8));
        asm volatile("" : "+v"(vb0), "+v"(vxa), "+v"(vxb));
        auto vread = [&](int m) {
            const int u = m / NDT, dt = m % NDT;
            const i16x4 x0 = lds_read_tr16(Vb + vb0 + 16 * u * RB + ((64 * dt) ^ vxa));
            const i16x4 x1 = lds_read_tr16(Vb + vb0 + (16 * u + 8) * RB + ((64 * dt) ^ vxb));
            const u32x2 y0 = __builtin_bit_cast(u32x2, x0), y1 = __builtin_bit_cast(u32x2, x1);
            return u32x4{y0[0], y0[1], y1[0], y1[1]};
        };
        u32x4 va[4];
#pragma unroll
        for (int m = 0; m < 3; ++m)
            va[m] = vread(m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + 3 < NM)
                va[(m + 3) % 4] = vread(m + 3);
            __builtin_amdgcn_sched_barrier(0); // keep the reads ahead of the MFMAs
            o[m % NDT] = mfma32(as_bf16x8(va[m % 4]), pf[m / NDT], o[m % NDT]);
        }
    };

    // Online-softmax update of an executed block: new running max, P (bf16,
    // the B operand of the next P.V) and row sum.  The accumulator's rescale
    // by alpha (needed when a row of the wave raised its max) is left to the
    // block's P.V: until then O only receives nothing, and the P.V of the
    // previous block, issued just before, would otherwise have to drain first.
    auto softmax = [&](const f32x16 (&s)[2], float mt2, bf16x8 (&pf)[4]) {
        const float mnew = fmaxf(m2, mt2);
        const float msafe = mnew == neg_inf() ? 0.f : mnew;
        float rs = 0.f;
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
        const float alpha = mnew > m2 ? exp2_hw(m2 - msafe) : 1.f; // 0 on the first block
        lsum = alpha * lsum + rs;
        rescale = __any(mnew > m2) != 0;
        alpha_p = alpha;
        m2 = mnew;
    };

    // Software pipeline, one barrier per block.  Entering iteration j:
    //   S_j and its row max are in registers and its vote is in LDS;
    //   K_{j+1} and (if block j-1 executed) V_{j-1} are in flight;
    //   P_{j-1} is in registers if block j-1 executed.
    // Iteration j: barrier; read the votes on block j and request K_{j+2}
    // (no decision needed); O += V_{j-1} P_{j-1} (MFMA) while the votes
    // arrive; request V_j if block j executes, then its softmax (VALU) and
    // the scores of block j+1 (MFMA); finally vote on block j+1.  The other
    // workgroup on the compute unit fills the matrix / vector gaps.  By the
    // barrier of iteration j+1 the V_j and K_{j+2} copies have had most of an
    // iteration to land.  S_j and S_{j+1} live in two register sets that alternate between
    // consecutive blocks (the loop is unrolled by two), so the loop carries no
    // register copies.
    bf16x8 pprev[4];
    int eprev = 0; // block j-1 executed (a scalar 0/1, like the flags below)
    auto iter = [&](int j, f32x16(&sc)[2], float mtc, f32x16(&sn)[2], float &mtn) {
        wait_vmcnt<0>();
        lds_barrier(); // votes_j, K_{j+1}, V_{j-1} visible; iteration j-1 done everywhere
        const int par = j & 1;
        // The votes are read before the K refill is issued, so that their LDS
        // latency passes while the copies are accepted.
        uint32_t votes = 0;
        if (SKIP)
            votes = *(const uint32_t *)&vote[par][0];
        if (j + 2 < nvis)
            copy_tile(kp, a.k_st, koff, j + 2, kbuf_l(j)); // K ring refill
        // P.V of block j-1 first: its MFMAs cover the LDS latency of the
        // votes.  The decision is then taken from lane 0 as a 0/1 int pinned
        // to an SGPR, so that the skip count and the branches on it stay
        // scalar (as a bool, the compiler kept it as a lane mask and
        // converted it with vector instructions on every block).
        if (!GAPS && eprev)
            pv(j - 1, pprev); // P_{j-1} is dead afterwards
        int skip = 0;
        if (SKIP) {
            skip = __builtin_amdgcn_readfirstlane(votes == 0x01010101u ? 1 : 0); // uniform across the workgroup
            asm volatile("" : "+s"(skip));
        }
        if (want_maps && tid == 0) {
            float g = neg_inf();
#pragma unroll
            for (int i = 0; i < NW; ++i)
                g = fmaxf(g, gapw[par][i]);
            const int64_t idx = ((int64_t)(b * a.Hq + h) * a.nqt + t) * a.nkb + j;
            if (a.skip_map)
                a.skip_map[idx] = (uint8_t)skip;
            if (a.gap_map)
                a.gap_map[idx] = g * 0.69314718055994531f; // back to natural log
        }
        n_skipped += skip;
        const int ecur = skip ^ 1;
        if (!GAPS && ecur)
            copy_tile(vp, a.v_st, voff, j, vbuf_l(j)); // V_j only for an executed block

        if (GAPS) {
            m2 = fmaxf(m2, mtc); // the running max, over every block
        } else {
            if (ecur)
                softmax(sc, mtc, pprev); // P_j reuses its registers
        }
        if (j + 1 < nvis) {
            scores(j + 1, sn, mtn); // into the other register set
            vote_block(j + 1, mtn);
        }
        eprev = GAPS ? 0 : ecur;
    };

    if (NW < 4 && tid < 8 && (tid & 3) >= NW)
        vote[tid >> 2][tid & 3] = 1; // bytes no wave writes (published by the barrier below)
    copy_tile(kp, a.k_st, koff, jlo, kbuf_l(jlo));
    if (jlo + 1 < nvis) {
        copy_tile(kp, a.k_st, koff, jlo + 1, kbuf_l(jlo + 1));
        wait_vmcnt<KI>();
    } else {
        wait_vmcnt<0>();
    }
    lds_barrier();
    f32x16 sa[2], sb[2];
    float mta, mtb;
    scores(jlo, sa, mta);
    vote_block(jlo, mta);
    for (int j = jlo; j < nvis; j += 2) {
        iter(j, sa, mta, sb, mtb);
        if (j + 1 < nvis)
            iter(j + 1, sb, mtb, sa, mta);
    }
    if (eprev) {
        wait_vmcnt<0>();
        lds_barrier(); // V of the last executed block visible
        pv(nvis - 1, pprev);
    }

    // Finalize: O = acc / l, l summed over the two lane halves; exactly 0 for
    // a row that saw no key (l = 0), NaN when l is NaN.
    const float l = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.f / l;
    const bool none = l == 0.f;
    if (!GAPS && row_valid) {
        char *ob = (char *)a.o;
        const int64_t base = (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)qrow * a.o_st;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                f32x4 v4 = {o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                            o[dt][4 * g + 3] * inv};
                if (none)
                    v4 = f32x4{};
                if (OUT_BF16) {
                    bf16x4 bv = __builtin_convertvector(v4, bf16x4);
                    *(bf16x4 *)(ob + 2 * (base + d)) = bv;
                } else {
                    *(f32x4 *)(ob + 4 * (base + d)) = v4;
                }
            }
    }
    if (tid == 0) {
        if (want_maps) {
            auto unvisited = [&](int j) {
                const int64_t idx = ((int64_t)(b * a.Hq + h) * a.nqt + t) * a.nkb + j;
                if (a.skip_map)
                    a.skip_map[idx] = 255;
                if (a.gap_map)
                    a.gap_map[idx] = neg_inf();
            };
            for (int j = 0; j < jlo; ++j)
                unvisited(j);
            for (int j = nvis; j < a.nkb; ++j)
                unvisited(j);
        }
        if (a.counters) {
            if (blockIdx.x == 0)
                atomicAdd(a.counters, a.visited_total);
            if (n_skipped > 0)
                atomicAdd(a.counters + 1, (unsigned long long)n_skipped);
        }
    }
}

template <int D, int BR, bool CAUSAL, bool SKIP, bool OUT_BF16, bool GAPS = false>
hipError_t launch_one(const PrefillArgs &a, hipStream_t stream)
{
    const unsigned grid = (unsigned)a.nqt * (unsigned)a.Hq * (unsigned)a.B;
    if (grid == 0)
        return hipSuccess;
    hipLaunchKernelGGL((prefill_kernel<D, BR, CAUSAL, SKIP, OUT_BF16, GAPS>), dim3(grid), dim3(2 * BR), 0,
                       stream, a);
    return hipGetLastError();
}

template <int D, int BR>
hipError_t launch_tile(const PrefillArgs &a, bool causal, bool skip, bool out_bf16, hipStream_t s, bool gaps)
{
    if (gaps) // decisions through the skip kernel's vote; O is not written
        return causal ? launch_one<D, BR, true, true, false, true>(a, s) : launch_one<D, BR, false, true, false, true>(a, s);
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
                          hipStream_t stream, bool gaps)
{
    if (d == 128 && tile_q == 128)
        return launch_tile<128, 128>(a, causal, skip, out_bf16, stream, gaps);
    if (d == 128 && tile_q == 64)
        return launch_tile<128, 64>(a, causal, skip, out_bf16, stream, gaps);
    if (d == 64 && tile_q == 128)
        return launch_tile<64, 128>(a, causal, skip, out_bf16, stream, gaps);
    if (d == 64 && tile_q == 64)
        return launch_tile<64, 64>(a, causal, skip, out_bf16, stream, gaps);
    return hipErrorInvalidValue;
}

} // namespace blasst
