// decode.hip -- split-K decode attention with BLASST block skipping, gfx950.
//
// Method: "BLASST: Dynamic BLocked Attention Sparsity via Softmax
// Thresholding" (gist.science/pt/paper/2512.12087, section 2 and section 3
// "Decode (limitado por memória)"): decode is memory bound, so the saving
// that matters is the V-block load from HBM that a skipped block never
// issues.  The Hindi explainer (gist.science/hi/paper/2512.12087, section 2,
// "kernel optimisation") adds "batched load scheduling": several Q.K products
// are computed before deciding which V blocks to fetch, to avoid pipeline
// bubbles from conditional loads.
//
// Here a workgroup (4 waves) owns one (split, KV head, sequence) unit and walks
// its key blocks in batches of 4, one block per wave:
//  1. every wave loads its block's K straight into MFMA operand registers and
//     computes S^T = K q^T (16x16x32 bf16 MFMA; the G <= 16 query heads that
//     share the KV head are the 16 columns, padded with zeros);
//  2. the 4 block maxima are exchanged through LDS and every wave evaluates
//     the 4 decisions in order.  The running max never depends on earlier
//     decisions (a skipped block has m~ < m + ln(lambda) <= m), so the
//     decision of block i uses the exclusive prefix max of the block maxima;
//  3. a wave whose block is executed copies V global -> LDS into its own slice
//     (global_load_lds, no registers; K and V loads carry the non-temporal
//     hint, since a step reads each cache row once), then issues the next
//     batch's K loads,
//     computes the exponentials while both are in flight, and accumulates
//     O^T += V^T P^T with the V^T operand taken by the gfx950 transpose read.
//     A skipped block issues no V load at all.
// Each wave keeps its own online-softmax state; the 4 states are merged with
// the log-sum-exp rule at the end, and across splits by the combine kernel.
#include "device.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int BC = 64;
constexpr int NWD = 4; // waves per decode workgroup = blocks per batch

// V tile chunk swizzle (physical chunk = logical chunk ^ dswz(row)).  The
// transpose read of the 16x16x32 A operand serves 32 lanes per LDS cycle: 8
// consecutive rows (8-aligned) x an aligned pair of chunks.  256-byte rows
// each span all banks, so bits 1-3 of the swizzle must differ across the 8
// rows; 128-byte rows share a bank line in pairs, so they must differ across
// the 4 rows of each parity.
template <int DG>
__device__ __forceinline__ int dswz(int row)
{
    return DG > 8 ? (row & 7) << 1 : ((row >> 1) & 3) << 1;
}

template <int D, bool SKIP, bool OUT_BF16, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_gqa_kernel(const DecodeArgs a)
{
    constexpr int RB = D * 2;          // bytes per V row
    constexpr int DG = D / 8;          // 16-byte chunks per row
    constexpr int TB = BC * RB;        // bytes per V tile
    constexpr int VI = TB / 1024;      // 1 KB copies per V tile (one wave copies a tile)
    constexpr int RPI = 64 / DG;       // rows per copy
    static_assert(16 % RPI == 0, "a V copy must stay inside one 16-row group");
    constexpr int NS = D / 32;         // 32-wide k-steps of the QK product
    constexpr int NDT = D / 16;        // 16-row d tiles of O^T
    constexpr int KLOADS = 4 * NS;     // K register loads per wave per block
    __shared__ __attribute__((aligned(1024))) char vsm[NWD * TB];
    __shared__ float mblk[2][NWD][16];
    __shared__ float mw_s[NWD][16], lw_s[NWD][16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int S = a.num_splits, G = a.G;
    // Split index rotated by the sequence: workgroups reach the 8 XCDs in
    // linear-id order, and with an unrotated split index XCD x would only see
    // splits x mod S (the first split of a sequence, seeded by the sink
    // block, skips far more than the others).
    const int g = blockIdx.y, b = blockIdx.z;
    const int s = (int)((blockIdx.x + blockIdx.z) % (unsigned)S);
    const bool want_maps = a.skip_map != nullptr || a.gap_map != nullptr;

    int len = a.seq_lens[b];
    len = len < 0 ? 0 : (len > a.Lmax ? a.Lmax : len);
    const int nkb_b = (len + BC - 1) / BC;
    // Sliding window: the query (position len-1) sees keys klo .. len-1, and
    // the splits cut the blocks j0 .. nkb_b-1 that hold them.
    const int klo = len - a.win > 0 ? len - a.win : 0;
    const int j0 = klo / BC;
    const int per = (nkb_b - j0 + S - 1) / S;
    const int jb = j0 + s * per;
    const int je = (jb + per < nkb_b) ? jb + per : nkb_b;

    // Cache rows.  Contiguous cache: row r of the sequence at kp + r * k_st.
    // Paged cache: pool page page_table[b][r >> page_shift], row r & pmask of
    // that page.  A page holds a power of two >= 16 rows, so the 16 rows of an
    // aligned group share one page.  Rows outside klo .. len-1 are read as the
    // nearest row inside (finite data under a zero probability, never a row
    // of a page that may not exist), which lies in the page of the group's
    // first row clamped into klo .. len-1.
    // The 4 group ids of a block come from one vector load (lane kt < 4 reads
    // group kt's entry) issued a batch ahead, right behind the K loads of the
    // batch before; they are moved to SGPRs before the next V copy is issued,
    // so a table read never stalls a cache load.
    const uint16_t *kp = a.k + (PAGED ? 0 : b * a.k_sb) + g * a.k_sh;
    const uint16_t *vp = a.v + (PAGED ? 0 : b * a.v_sb) + g * a.v_sh;
    const int pmask = PAGED ? (1 << a.page_shift) - 1 : -1;
    auto ids_load = [&](int j) -> int {
        if (!PAGED)
            return 0;
        int g0 = j * BC + 16 * (lane & 3);
        g0 = (j < je && g0 < len) ? (g0 > klo ? g0 : klo) : len - 1;
        return a.page_table[b * a.pt_stride + (g0 >> a.page_shift)];
    };
    auto ids_take = [&](int v, int (&ids)[4]) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            int id = __builtin_amdgcn_readlane(v, kt);
            id = id < 0 ? 0 : (id < a.num_pages ? id : a.num_pages - 1);
            asm volatile("" : "+s"(id)); // in SGPRs here, before any later copy
            ids[kt] = id;
        }
    };
    auto page_off = [&](const int (&ids)[4], int grp16, int64_t sb) -> int64_t {
        return PAGED ? (int64_t)ids[grp16] * sb : 0;
    };
    char *const vt = vsm + w * TB; // this wave's V slice

    // q^T as the B operand: lane (n, grp) holds q[head n][32 st + 8 grp .. +7].
    bf16x8 qf[NS];
    {
        const uint16_t *qp = a.q + b * a.q_sb + (int64_t)(g * G + n) * a.q_sh;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            u32x4 u = {0, 0, 0, 0};
            if (n < G)
                u = *(const u32x4 *)(qp + 32 * st + 8 * grp);
            qf[st] = as_bf16x8(u);
        }
    }

    // K operand of S^T = K q^T for one 64-key block, straight from HBM into
    // registers: tile kt = 16 keys, lane (m = key, grp) holds
    // K[key][32 st + 8 grp .. +7].  Every lane always issues all KLOADS loads:
    // keys outside the split read row len-1 (finite; their scores are masked
    // to -inf below), because the V wait counts on exactly KLOADS younger
    // vector-memory operations (plus the id load of a paged cache).
    u32x4 kr[4][NS];
    auto load_k = [&](int j, const int (&ids)[4]) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int key = j * BC + 16 * kt + n;
            const int kc = (j < je && key < len) ? (key > klo ? key : klo) : len - 1;
            const uint16_t *rp = kp + page_off(ids, kt, a.k_sb) + (int64_t)(kc & pmask) * a.k_st;
#pragma unroll
            for (int st = 0; st < NS; ++st)
                kr[kt][st] = __builtin_nontemporal_load((const u32x4 *)(rp + 32 * st + 8 * grp));
        }
    };
    // V tile of block j -> this wave's slice, row-major with the 16-byte
    // chunks XOR-swizzled by row (rows past len re-read row len-1: finite
    // values whose probabilities are exactly 0).
    auto copy_v = [&](int j, const int (&ids)[4]) {
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int row = i * RPI + lane / DG;
            const int c = (lane % DG) ^ dswz<DG>(row);
            int key = j * BC + row;
            key = key < len ? (key > klo ? key : klo) : len - 1;
            copy16_to_lds<true>(vp + page_off(ids, (i * RPI) >> 4, a.v_sb) + (int64_t)(key & pmask) * a.v_st + c * 8,
                          vt + i * 1024);
        }
    };

    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        o[dt] = f32x4{};
    float m2 = neg_inf();   // this wave's running max for head n (base 2)
    float lsum = 0.f;       // this lane's partial running sum for head n
    float pmax = neg_inf(); // exclusive prefix max of block maxima (decisions)
    int n_skipped = 0;

    // Transpose-read addressing of the V^T operand (16x16x32 A layout).
    const int vj = (lane & 15) >> 2, vq = lane & 3, vgrp = lane >> 4;

    // Page ids (paged cache): pc for this batch's block (its V copy), pn for
    // the next batch's (its K loads); idv is the vector load in flight.
    int pc[4] = {0, 0, 0, 0}, pn[4] = {0, 0, 0, 0}, idv = 0;

    // Sink seed (splits after the first): the decisions' prefix max starts
    // from the row maxima of block j0 instead of -inf.  Every wave scores
    // the block itself (the rows of its K land in L2 once).
    if (a.sink_seed && s > 0 && jb < je) {
        ids_take(ids_load(j0), pc);
        load_k(j0, pc);
        f32x4 sc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sc[kt] = f32x4{};
#pragma unroll
            for (int st = 0; st < NS; ++st)
                sc[kt] = mfma16(as_bf16x8(kr[kt][st]), qf[st], sc[kt]);
        }
        float mt = neg_inf();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = j0 * BC + 16 * kt + 4 * grp + r;
                if (key < len && key >= klo)
                    mt = fmaxf(mt, sc[kt][r]);
            }
        mt = max_xor32(max_xor16(mt));
        pmax = mt * a.scale_log2;
    }
    if (jb < je) {
        ids_take(ids_load(jb + w), pc);
        load_k(jb + w, pc);
        idv = ids_load(jb + NWD + w);
    }
    int it = 0;
    for (int j0 = jb; j0 < je; j0 += NWD, ++it) {
        const int j = j0 + w; // this wave's block
        const int par = it & 1;
        f32x4 sc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sc[kt] = f32x4{};
#pragma unroll
            for (int st = 0; st < NS; ++st)
                sc[kt] = mfma16(as_bf16x8(kr[kt][st]), qf[st], sc[kt]);
        }
        if (PAGED)
            ids_take(idv, pn); // issued behind the K loads just consumed
        // Mask keys outside klo .. len-1 (and the whole block if j >= je).
        const int k0 = j * BC;
        if (j >= je || k0 + BC > len || k0 < klo) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * kt + 4 * grp + r;
                    if (j >= je || key >= len || key < klo)
                        sc[kt][r] = neg_inf();
                }
        }
        float mt = neg_inf();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                mt = fmaxf(mt, sc[kt][r]);
        mt = max_xor32(max_xor16(mt));
        const float mt2 = mt * a.scale_log2;
        if (grp == 0)
            mblk[par][w][n] = mt2;
        lds_barrier();

        // Decisions of the batch, in block order, identical in every wave.
        bool my_skip = false;
        int batch_skipped = 0;
#pragma unroll
        for (int i = 0; i < NWD; ++i) {
            if (j0 + i >= je)
                break;
            const float mb = mblk[par][i][n];
            const bool valid_head = n < G;
            const float dgap = (!valid_head || mb == neg_inf()) ? neg_inf() : mb - pmax;
            bool skip_i = false;
            if (SKIP)
                skip_i = __all(!(dgap >= a.lnlam2)) != 0;
            if (want_maps) {
                const float gg = wave_max(dgap);
                if (w == 0 && lane == 0) {
                    const int64_t idx = (int64_t)(b * a.Hkv + g) * a.nkb + j0 + i;
                    if (a.skip_map)
                        a.skip_map[idx] = skip_i ? 1 : 0;
                    if (a.gap_map)
                        a.gap_map[idx] = gg * 0.69314718055994531f;
                }
            }
            pmax = fmaxf(pmax, mb);
            if (i == w)
                my_skip = skip_i;
            batch_skipped += skip_i ? 1 : 0;
        }
        n_skipped += batch_skipped;

        const bool exec = j < je && !my_skip;
        if (exec)
            copy_v(j, pc); // V only for an executed block
        const bool more = j0 + NWD < je;
        if (more) {
            load_k(j0 + NWD + w, pn); // next batch's K in flight
            if (PAGED) {
                idv = ids_load(j0 + 2 * NWD + w);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
                    pc[kt] = pn[kt];
            }
        }

        if (exec) {
            // Online-softmax update with this wave's running max.
            const float mnew = fmaxf(m2, mt2);
            const float msafe = mnew == neg_inf() ? 0.f : mnew;
            const float alpha = exp2_hw(m2 - msafe);
            float rs = 0.f;
            bf16x8 pf[2];
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2) {
                f32x8 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p0 = exp2_hw(__builtin_fmaf(sc[2 * u2][r], a.scale_log2, -msafe));
                    const float p1 = exp2_hw(__builtin_fmaf(sc[2 * u2 + 1][r], a.scale_log2, -msafe));
                    pv[r] = p0;
                    pv[r + 4] = p1;
                    rs += p0 + p1;
                }
                pf[u2] = cvt_bf16x8(pv);
            }
            lsum = alpha * lsum + rs;
            m2 = mnew;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                o[dt] *= alpha;
            // The V copy is older than the next K loads (and, paged, the id
            // load behind them): wait for it only.
            if (more)
                wait_vmcnt<KLOADS + (PAGED ? 1 : 0)>();
            else
                wait_vmcnt<0>();
            compiler_fence();
            // O^T += V^T P^T: two k-steps of 32 keys.  A operand lane (m = d,
            // grp) slot i <-> key 32 u2 + 16 (i / 4) + 4 grp + i % 4.
#pragma unroll
            for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int c = 2 * dt + (vq >> 1);
                    const int ra = 32 * u2 + 4 * vgrp + vj, rb = ra + 16;
                    const i16x4 x0 = lds_read_tr16(vt + ra * RB + ((c ^ dswz<DG>(ra)) * 16) + (vq & 1) * 8);
                    const i16x4 x1 = lds_read_tr16(vt + rb * RB + ((c ^ dswz<DG>(rb)) * 16) + (vq & 1) * 8);
                    const u32x2 y0 = __builtin_bit_cast(u32x2, x0), y1 = __builtin_bit_cast(u32x2, x1);
                    const u32x4 va = {y0[0], y0[1], y1[0], y1[1]};
                    o[dt] = mfma16(as_bf16x8(va), pf[u2], o[dt]);
                }
        }
    }

    // Merge the 4 wave states (log-sum-exp), then write O or the split partial.
    float l = lsum;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (grp == 0) {
        mw_s[w][n] = m2;
        lw_s[w][n] = l;
    }
    lds_barrier();
    float M = neg_inf();
#pragma unroll
    for (int i = 0; i < NWD; ++i)
        M = fmaxf(M, mw_s[i][n]);
    const float Msafe = M == neg_inf() ? 0.f : M;
    const float cw = exp2_hw(m2 - Msafe);
    // Stage the scaled wave accumulators as fp32 [wave][head][D] (reuses the V slices).
    float *stage = (float *)vsm;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        *(f32x4 *)(stage + (w * 16 + n) * D + 16 * dt + 4 * grp) = o[dt] * cw;
    lds_barrier();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int hd = idx / D, d = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < NWD; ++i)
            acc += stage[(i * 16 + hd) * D + d];
        float Mh = neg_inf(), lh = 0.f;
#pragma unroll
        for (int i = 0; i < NWD; ++i)
            Mh = fmaxf(Mh, mw_s[i][hd]);
        const float Mhs = Mh == neg_inf() ? 0.f : Mh;
#pragma unroll
        for (int i = 0; i < NWD; ++i)
            lh += lw_s[i][hd] * exp2_hw(mw_s[i][hd] - Mhs);
        if (S == 1) {
            const float val = lh > 0.f ? acc / lh : 0.f;
            const int64_t off = (int64_t)b * a.o_sb + (int64_t)(g * G + hd) * a.o_sh + d;
            if (OUT_BF16)
                ((__bf16 *)a.o)[off] = (__bf16)val;
            else
                ((float *)a.o)[off] = val;
        } else {
            const int64_t pu = ((int64_t)(b * a.Hkv + g) * S + s) * G + hd;
            a.part_o[pu * D + d] = acc;
            if (d == 0) {
                a.part_ml[2 * pu] = Mh;
                a.part_ml[2 * pu + 1] = lh;
            }
        }
    }

    if (tid == 0) {
        // Blocks that no split visits: before the window (first split writes
        // them) and past the sequence (last split).
        if (want_maps) {
            auto unvisited = [&](int j) {
                const int64_t idx = (int64_t)(b * a.Hkv + g) * a.nkb + j;
                if (a.skip_map)
                    a.skip_map[idx] = 255;
                if (a.gap_map)
                    a.gap_map[idx] = neg_inf();
            };
            if (s == 0)
                for (int j = 0; j < j0; ++j)
                    unvisited(j);
            if (s == S - 1)
                for (int j = nkb_b; j < a.nkb; ++j)
                    unvisited(j);
        }
        if (a.counters && je > jb) {
            atomicAdd(a.counters, (unsigned long long)(je - jb));
            atomicAdd(a.counters + 1, (unsigned long long)n_skipped);
        }
    }
}

// Log-sum-exp merge of split partials.  A thread owns 4 consecutive output
// columns of one (sequence, query head); a workgroup covers 256 / (dv/4)
// heads.  Weights are exp2(m_s - M) with M the largest split max among
// splits that saw keys (kept as a running max, one chunk of splits at a
// time); splits with l = 0 contribute nothing.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeArgs a, int dv)
{
    const int tph = dv / 4, hpw = 256 / tph;
    const int hq = blockIdx.x * hpw + (int)threadIdx.x / tph;
    const int b = blockIdx.y;
    if (hq >= a.Hq)
        return;
    const int d = 4 * ((int)threadIdx.x % tph);
    const int G = a.G, g = hq / G, hd = hq % G, S = a.num_splits;
    const int64_t pu0 = ((int64_t)(b * a.Hkv + g) * S) * G + hd;
    // One pass over the splits, CH at a time: the loads of a chunk are all
    // issued before any is used, and the running (M, num, den) is rescaled
    // when a chunk raises the max.  Indices past S re-read split S-1 and are
    // masked.
    constexpr int CH = 8;
    float M = neg_inf(), den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += CH) {
        float2 ml[CH];
        f32x4 po[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t pu = pu0 + (int64_t)(s0 + i < S ? s0 + i : S - 1) * G;
            ml[i] = *(const float2 *)(a.part_ml + 2 * pu);
            po[i] = *(const f32x4 *)(a.part_o + pu * dv + d);
        }
        float Mc = M;
#pragma unroll
        for (int i = 0; i < CH; ++i)
            if (s0 + i < S && ml[i].y > 0.f)
                Mc = fmaxf(Mc, ml[i].x);
        const float Ms = Mc == neg_inf() ? 0.f : Mc;
        const float r = M == neg_inf() ? 0.f : exp2_hw(M - Ms);
        num *= r;
        den *= r;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float wgt = (s0 + i < S && ml[i].y > 0.f) ? exp2_hw(ml[i].x - Ms) : 0.f;
            num += wgt * po[i];
            den += wgt * ml[i].y;
        }
        M = Mc;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const f32x4 val = num * inv;
    const int64_t off = (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + d;
    if (OUT_BF16)
        *(bf16x4 *)((__bf16 *)a.o + off) = __builtin_convertvector(val, bf16x4);
    else
        *(f32x4 *)((float *)a.o + off) = val;
}

} // namespace

hipError_t launch_combine(const DecodeArgs &a, int dv, bool out_bf16, hipStream_t stream)
{
    const int hpw = 256 / (dv / 4);
    const dim3 grid((a.Hq + hpw - 1) / hpw, a.B), block(256);
    if (out_bf16)
        hipLaunchKernelGGL((decode_combine_kernel<true>), grid, block, 0, stream, a, dv);
    else
        hipLaunchKernelGGL((decode_combine_kernel<false>), grid, block, 0, stream, a, dv);
    return hipGetLastError();
}

namespace {

template <int D, bool SKIP, bool OUT_BF16>
hipError_t launch_gqa(const DecodeArgs &a, hipStream_t stream)
{
    const dim3 grid(a.num_splits, a.Hkv, a.B);
    if (a.page_table)
        hipLaunchKernelGGL((decode_gqa_kernel<D, SKIP, OUT_BF16, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_gqa_kernel<D, SKIP, OUT_BF16, false>), grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1)
        return e;
    return launch_combine(a, D, OUT_BF16, stream);
}

} // namespace

hipError_t launch_mla(const DecodeArgs &a, bool skip, bool out_bf16, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs &a, int dqk, int dv, bool skip, bool out_bf16, hipStream_t stream)
{
    if (a.B == 0)
        return hipSuccess;
    if (dqk == dv && a.G <= 16) {
        if (dqk == 128) {
            if (skip)
                return out_bf16 ? launch_gqa<128, true, true>(a, stream) : launch_gqa<128, true, false>(a, stream);
            return out_bf16 ? launch_gqa<128, false, true>(a, stream) : launch_gqa<128, false, false>(a, stream);
        }
        if (dqk == 64) {
            if (skip)
                return out_bf16 ? launch_gqa<64, true, true>(a, stream) : launch_gqa<64, true, false>(a, stream);
            return out_bf16 ? launch_gqa<64, false, true>(a, stream) : launch_gqa<64, false, false>(a, stream);
        }
    }
    if (dqk == 576 && dv == 512 && a.G == 128)
        return launch_mla(a, skip, out_bf16, stream);
    return hipErrorInvalidValue;
}

} // namespace blasst
