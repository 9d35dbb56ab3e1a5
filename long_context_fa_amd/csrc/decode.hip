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
//  1. every wave copies its block's K global -> LDS into its own K slot
//     (global_load_lds, whole 256-byte rows per instruction: the loads go to
//     memory as full 128-byte lines, where MFMA-layout register loads would
//     take 64 bytes of 16 rows each and run the compute unit out of
//     outstanding-miss entries at ~5.7 TB/s), reads it back into MFMA operand
//     registers and computes S^T = K q^T (16x16x32 bf16 MFMA; the G <= 64
//     query heads that share the KV head are the columns, in groups of 16
//     padded with zeros, all groups on the same K operands); the next
//     batch's K copy goes out as soon as the slot is read;
//  2. the 4 block maxima are exchanged through LDS and every wave evaluates
//     the 4 decisions in order.  The running max never depends on earlier
//     decisions (a skipped block has m~ < m + ln(lambda) <= m), so the
//     decision of block i uses the exclusive prefix max of the block maxima;
//  3. a wave whose block is executed copies V global -> LDS into its own V
//     slot (K and V copies carry the non-temporal hint, since a step reads
//     each cache row once), computes the exponentials while it is in flight,
//     and accumulates O^T += V^T P^T with the V^T operand taken by the gfx950
//     transpose read.
//     A skipped block issues no V load at all.
// Each wave keeps its own online-softmax state; the 4 states are merged with
// the log-sum-exp rule at the end, and across splits by the combine kernel.
// The gap pass (GAPS) keeps steps 1-2 and the maps: no V copy, no
// exponential, no P.V, no partials (the decisions use the prefix max, which
// does not depend on them).
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

// K slot chunk swizzle.  The operand read (ds_read_b128) serves 8 lanes per
// LDS cycle: rows 16 kt + 0..7 (or + 8..15) at one logical chunk.  A row is
// one (d = 64) or two (d = 128) full bank lines, so the 8 rows' physical
// chunks must differ in bits 0-2.  The XOR stays inside a 128-byte line, so
// each aligned group of 8 lanes of a copy still reads one whole line.
__device__ __forceinline__ int kswz(int row) { return row & 7; }

// PG: 0 contiguous cache; 1 paged, pages of 16 or 32 rows (a block spans
// several pages: one id per 16-row group); 2 paged, pages of 64 rows or more
// (a block lies in one page: one id).
// NG: 16-head column groups per wave (G <= 16 NG): every group's scores and
// P.V reuse the same K and V operand registers.
template <int D, bool SKIP, bool OUT_BF16, int PG, bool GAPS, int NG>
// With d = 128 the K and V slots hold one workgroup per compute unit (one
// wave per SIMD), so the wave may use the whole register file; otherwise two,
// unless several head groups need the registers.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((D > 64 || NG > 1) && !GAPS ? 1 : 2,
                                                                     (D > 64 || NG > 1) && !GAPS ? 1 : 2)))
void decode_gqa_kernel(const DecodeArgs a)
{
    constexpr bool PAGED = PG != 0;
    constexpr int NID = PG == 2 ? 1 : 4; // page ids per block
    constexpr int RB = D * 2;          // bytes per V row
    constexpr int DG = D / 8;          // 16-byte chunks per row
    constexpr int TB = BC * RB;        // bytes per V tile
    constexpr int VI = TB / 1024;      // 1 KB copies per V tile (one wave copies a tile)
    constexpr int RPI = 64 / DG;       // rows per copy
    static_assert(16 % RPI == 0, "a V copy must stay inside one 16-row group");
    constexpr int NS = D / 32;         // 32-wide k-steps of the QK product
    constexpr int NDT = D / 16;        // 16-row d tiles of O^T
    // K slots (one 64-row tile per wave) and V slots; the V slots are reused
    // as fp32 staging by the final merge.  With d = 128 the 128 KB hold one
    // workgroup (4 waves) per compute unit, which keeps enough whole-line
    // copies in flight.
    // The gap pass has no V slices: each wave keeps two K slots instead and
    // copies its block two batches ahead.
    constexpr int KS = GAPS ? 2 : 1; // K slots per wave
    __shared__ __attribute__((aligned(1024))) char ksm[NWD * TB * KS];
    __shared__ __attribute__((aligned(1024))) char vsm[GAPS ? 1024 : NWD * TB];
    constexpr int NH = 16 * NG; // head slots per wave
    __shared__ float mblk[2][NWD][NH];
    __shared__ float mw_s[NWD][NH], lw_s[NWD][NH];

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
    auto ids_take = [&](int v, int (&ids)[NID]) {
#pragma unroll
        for (int kt = 0; kt < NID; ++kt) {
            int id = __builtin_amdgcn_readlane(v, kt);
            id = id < 0 ? 0 : (id < a.num_pages ? id : a.num_pages - 1);
            asm volatile("" : "+s"(id)); // in SGPRs here, before any later copy
            ids[kt] = id;
        }
    };
    auto page_off = [&](const int (&ids)[NID], int grp16, int64_t sb) -> int64_t {
        return PAGED ? (int64_t)ids[grp16 & (NID - 1)] * sb : 0;
    };
    char *const vt = vsm + w * TB; // this wave's V slice

    // q^T as the B operand: lane (n, grp) holds q[head 16 h + n][32 st + 8 grp .. +7]
    // for head group h (zeros for slots past G).
    bf16x8 qf[NG][NS];
#pragma unroll
    for (int h = 0; h < NG; ++h) {
        const uint16_t *qp = a.q + b * a.q_sb + (int64_t)(g * G + 16 * h + n) * a.q_sh;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            u32x4 u = {0, 0, 0, 0};
            if (16 * h + n < G)
                u = *(const u32x4 *)(qp + 32 * st + 8 * grp);
            qf[h][st] = as_bf16x8(u);
        }
    }

    // K of block j -> this wave's K slot, row-major with the 16-byte chunks
    // XOR-swizzled by row (kswz).  Keys outside the split or past len re-read
    // row len-1 (finite; their scores are masked to -inf below).
    char *const kt_slot = ksm + w * KS * TB; // slot 0 (slot 1 follows it in the gap pass)
    // Tile copy (K or V): copy i moves RPI rows (1 KB).  When every row of
    // block j is a visible key (the common case), the 16 rows of a group lie
    // in one page (or one sequence) from a wave-uniform base, walked with one
    // scalar add per copy, and a lane's byte offset from the copy's first
    // row depends only on the parity of i (the swizzles depend on the row
    // mod 8).  Otherwise each lane clamps its own row.
    const int rin = lane / DG, pch = lane % DG;
    const bool offs32 = (int64_t)RPI * (a.k_st > a.v_st ? a.k_st : a.v_st) * 2 < ((int64_t)1 << 30);
    auto lane_off = [&](int i, int64_t st, bool isk) -> uint32_t {
        const int row = i * RPI + rin;
        const int c = pch ^ (isk ? kswz(row) : dswz<DG>(row));
        return (uint32_t)((int64_t)rin * st * 2 + c * 16);
    };
    const uint32_t koff[2] = {lane_off(0, a.k_st, true), lane_off(1, a.k_st, true)};
    const uint32_t voff[2] = {lane_off(0, a.v_st, false), lane_off(1, a.v_st, false)};
    auto copy_rows = [&](const uint16_t *base, int64_t st, int64_t sb, const int (&ids)[NID], int j, uint32_t dst,
                         const uint32_t (&off)[2], bool isk) __attribute__((always_inline)) {
        if (PG == 2 && offs32 && j < je && j * BC >= klo && (j + 1) * BC <= len) {
            // the block's 64 rows are consecutive rows of one page
            uint64_t addr = (uint64_t)(uintptr_t)(base + (int64_t)ids[0] * sb + (int64_t)((j * BC) & pmask) * st);
#pragma unroll
            for (int i = 0; i < VI; ++i) {
                copy16_to_lds_s<true>((const void *)(uintptr_t)addr, off[i & 1], dst + i * 1024u);
                addr += (uint64_t)(RPI * 2) * (uint64_t)st;
                asm volatile("" : "+s"(addr));
            }
        } else if (offs32 && j < je && j * BC >= klo && (j + 1) * BC <= len) {
            constexpr int CPG = 16 / RPI; // copies per 16-row group
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint16_t *gb = base + page_off(ids, g, sb) + (int64_t)((j * BC + 16 * g) & pmask) * st;
                uint64_t addr = (uint64_t)(uintptr_t)gb;
#pragma unroll
                for (int q = 0; q < CPG; ++q) {
                    const int i = g * CPG + q;
                    copy16_to_lds_s<true>((const void *)(uintptr_t)addr, off[i & 1], dst + i * 1024u);
                    addr += (uint64_t)(RPI * 2) * (uint64_t)st;
                    asm volatile("" : "+s"(addr)); // one running base, not one register pair per copy
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < VI; ++i) {
                const int row = i * RPI + rin;
                const int c = pch ^ (isk ? kswz(row) : dswz<DG>(row));
                const int key = j * BC + row;
                const int kc = (j < je && key < len) ? (key > klo ? key : klo) : len - 1;
                copy16_to_lds<true>(base + page_off(ids, (i * RPI) >> 4, sb) + (int64_t)(kc & pmask) * st + c * 8,
                                    dst + i * 1024u);
            }
        }
    };
    const uint32_t kt_lds = lds_addr(kt_slot), vt_lds = lds_addr(vt);
    // K of block j into K slot p (p = batch parity in the gap pass, else 0)
    auto copy_k = [&](int j, const int (&ids)[NID], int p = 0) {
        copy_rows(kp, a.k_st, a.k_sb, ids, j, kt_lds + (uint32_t)((KS == 2 ? (p & 1) : 0) * TB), koff, true);
    };
    // K operand of S^T = K q^T from the slot: tile kt = 16 keys, lane
    // (m = key, grp) holds K[key][32 st + 8 grp .. +7] (logical chunk
    // 4 st + grp).  The caller waits for the copy first.
    u32x4 kr[4][NS];
    auto read_k = [&](int p = 0) {
        const char *slot = kt_slot + (KS == 2 ? (p & 1) : 0) * TB;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int row = 16 * kt + n;
#pragma unroll
            for (int st = 0; st < NS; ++st)
                kr[kt][st] = *(const u32x4 *)(slot + row * RB + (((4 * st + grp) ^ kswz(row)) * 16));
        }
    };
    // The slot is refilled only once every read of it has returned.
    auto reads_done = [&]() { __builtin_amdgcn_s_waitcnt(0xC07F); }; // lgkmcnt(0)
    // V tile of block j -> this wave's slice, row-major with the 16-byte
    // chunks XOR-swizzled by row (rows past len re-read row len-1: finite
    // values whose probabilities are exactly 0).
    auto copy_v = [&](int j, const int (&ids)[NID]) { copy_rows(vp, a.v_st, a.v_sb, ids, j, vt_lds, voff, false); };

    f32x4 o[NG][NDT];
    float m2[NG], lsum[NG], pmax[NG];
#pragma unroll
    for (int h = 0; h < NG; ++h) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            o[h][dt] = f32x4{};
        m2[h] = neg_inf();   // this wave's running max for head 16 h + n (base 2)
        lsum[h] = 0.f;       // this lane's partial running sum for that head
        pmax[h] = neg_inf(); // exclusive prefix max of block maxima (decisions)
    }
    int n_skipped = 0;

    // Transpose-read addressing of the V^T operand (16x16x32 A layout).
    const int vj = (lane & 15) >> 2, vq = lane & 3, vgrp = lane >> 4;

    // Page ids (paged cache): pc for this batch's block (its V copy), pn for
    // the next batch's (its K copy, issued first thing in a batch); idv is
    // the vector load of the next batch's ids, issued a batch ahead beside
    // the K copy so that the wait for one covers the other.
    int pc[NID] = {}, pn[NID] = {}, idv = 0;

    // Sink seed (splits after the first): the decisions' prefix max starts
    // from the row maxima of block j0 instead of -inf.  Every wave scores
    // the block itself (the rows of its K land in L2 once).
    if (a.sink_seed && s > 0 && jb < je) {
        ids_take(ids_load(j0), pc);
        copy_k(j0, pc);
        wait_vmcnt<0>();
        compiler_fence();
        read_k();
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            f32x4 sc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                sc[kt] = f32x4{};
#pragma unroll
                for (int st = 0; st < NS; ++st)
                    sc[kt] = mfma16(as_bf16x8(kr[kt][st]), qf[h][st], sc[kt]);
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
            pmax[h] = mt * a.scale_log2;
        }
    }
    if (jb < je) {
        ids_take(ids_load(jb + w), pc);
        reads_done(); // (the sink block's reads, if any)
        compiler_fence();
        copy_k(jb + w, pc);
        if (GAPS && jb + NWD < je)
            copy_k(jb + NWD + w, pc, 1); // the gap pass reads no page table
        idv = ids_load(jb + NWD + w);
    }
    int it = 0;
    for (int j0 = jb; j0 < je; j0 += NWD, ++it) {
        const int j = j0 + w; // this wave's block
        const int par = it & 1;
        const bool more = j0 + NWD < je;
        // K of this block landed (and every older copy: V of the last
        // batch was waited for before its P.V); read it, then refill the
        // slot with the next batch's block right away.  The gap pass lets the
        // next batch's copy (the youngest VI copies, from the last batch)
        // stay in flight and refills the slot with the block after it.
        if (GAPS && more)
            wait_vmcnt<VI>();
        else
            wait_vmcnt<0>();
        compiler_fence();
        read_k(it);
        if (PAGED)
            ids_take(idv, pn); // the next batch's page ids (landed with this block's K)
        reads_done();
        compiler_fence();
        if (GAPS) {
            if (j0 + 2 * NWD < je)
                copy_k(j0 + 2 * NWD + w, pn, it);
        } else if (more) {
            copy_k(j0 + NWD + w, pn);
            if (PAGED)
                idv = ids_load(j0 + 2 * NWD + w);
        }
        f32x4 sc[NG][4];
#pragma unroll
        for (int h = 0; h < NG; ++h)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                sc[h][kt] = f32x4{};
#pragma unroll
                for (int st = 0; st < NS; ++st)
                    sc[h][kt] = mfma16(as_bf16x8(kr[kt][st]), qf[h][st], sc[h][kt]);
            }
        // Mask keys outside klo .. len-1 (and the whole block if j >= je).
        const int k0 = j * BC;
        if (j >= je || k0 + BC > len || k0 < klo) {
#pragma unroll
            for (int h = 0; h < NG; ++h)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = k0 + 16 * kt + 4 * grp + r;
                        if (j >= je || key >= len || key < klo)
                            sc[h][kt][r] = neg_inf();
                    }
        }
        float mt2[NG];
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            float mt = neg_inf();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mt = fmaxf(mt, sc[h][kt][r]);
            mt = max_xor32(max_xor16(mt));
            mt2[h] = mt * a.scale_log2;
            if (grp == 0)
                mblk[par][w][16 * h + n] = mt2[h];
        }
        lds_barrier();

        // Decisions of the batch, in block order, identical in every wave.
        bool my_skip = false;
        int batch_skipped = 0;
#pragma unroll
        for (int i = 0; i < NWD; ++i) {
            if (j0 + i >= je)
                break;
            bool meets = true;     // every head slot of this lane meets the test
            float dmax = neg_inf(); // largest gap over this lane's head slots
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                const float mb = mblk[par][i][16 * h + n];
                const bool valid_head = 16 * h + n < G;
                const float dgap = (!valid_head || mb == neg_inf()) ? neg_inf() : mb - pmax[h];
                meets = meets && !(dgap >= a.lnlam2);
                dmax = fmaxf(dmax, dgap);
                pmax[h] = fmaxf(pmax[h], mb);
            }
            bool skip_i = false;
            if (SKIP)
                skip_i = __all(meets) != 0;
            if (want_maps) {
                const float gg = wave_max(dmax);
                if (w == 0 && lane == 0) {
                    const int64_t idx = (int64_t)(b * a.Hkv + g) * a.nkb + j0 + i;
                    if (a.skip_map)
                        a.skip_map[idx] = skip_i ? 1 : 0;
                    if (a.gap_map)
                        a.gap_map[idx] = gg * 0.69314718055994531f;
                }
            }
            if (i == w)
                my_skip = skip_i;
            batch_skipped += skip_i ? 1 : 0;
        }
        n_skipped += batch_skipped;

        const bool exec = !GAPS && j < je && !my_skip;
        if (exec)
            copy_v(j, pc); // V only for an executed block

        if (exec) {
            // Online-softmax update with this wave's running max, per head group.
            bf16x8 pf[NG][2];
#pragma unroll
            for (int h = 0; h < NG; ++h) {
                const float mnew = fmaxf(m2[h], mt2[h]);
                const float msafe = mnew == neg_inf() ? 0.f : mnew;
                const float alpha = exp2_hw(m2[h] - msafe);
                float rs = 0.f;
#pragma unroll
                for (int u2 = 0; u2 < 2; ++u2) {
                    f32x8 pv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float p0 = exp2_hw(__builtin_fmaf(sc[h][2 * u2][r], a.scale_log2, -msafe));
                        const float p1 = exp2_hw(__builtin_fmaf(sc[h][2 * u2 + 1][r], a.scale_log2, -msafe));
                        pv[r] = p0;
                        pv[r + 4] = p1;
                        rs += p0 + p1;
                    }
                    pf[h][u2] = cvt_bf16x8(pv);
                }
                lsum[h] = alpha * lsum[h] + rs;
                m2[h] = mnew;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    o[h][dt] *= alpha;
            }
            // The V copy is the youngest vector-memory operation (the next
            // K copy and, paged, the id load went out before it).
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
#pragma unroll
                    for (int h = 0; h < NG; ++h)
                        o[h][dt] = mfma16(as_bf16x8(va), pf[h][u2], o[h][dt]);
                }
        }
        if (PAGED && more) {
#pragma unroll
            for (int kt = 0; kt < NID; ++kt)
                pc[kt] = pn[kt]; // the next batch's block (its V copy)
        }
    }

    // Merge the 4 wave states (log-sum-exp), then write O or the split partial.
    if (!GAPS) {
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            float l = lsum[h];
            l += __shfl_xor(l, 16);
            l += __shfl_xor(l, 32);
            if (grp == 0) {
                mw_s[w][16 * h + n] = m2[h];
                lw_s[w][16 * h + n] = l;
            }
        }
        // One head group at a time: stage its scaled wave accumulators as fp32
        // [wave][head][D] (reusing the V slices), then merge them.
        float *stage = (float *)vsm;
#pragma unroll
        for (int h = 0; h < NG; ++h) {
            lds_barrier(); // the group's statistics are in; the last group's staging is consumed
            float M = neg_inf();
#pragma unroll
            for (int i = 0; i < NWD; ++i)
                M = fmaxf(M, mw_s[i][16 * h + n]);
            const float Msafe = M == neg_inf() ? 0.f : M;
            const float cw = exp2_hw(m2[h] - Msafe);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(f32x4 *)(stage + (w * 16 + n) * D + 16 * dt + 4 * grp) = o[h][dt] * cw;
            lds_barrier();
            const int gh = G - 16 * h < 16 ? G - 16 * h : 16; // heads of this group
            for (int idx = tid; idx < gh * D; idx += 256) {
                const int hl = idx / D, d = idx % D, hd = 16 * h + hl;
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < NWD; ++i)
                    acc += stage[(i * 16 + hl) * D + d];
                float Mh = neg_inf(), lh = 0.f;
#pragma unroll
                for (int i = 0; i < NWD; ++i)
                    Mh = fmaxf(Mh, mw_s[i][hd]);
                const float Mhs = Mh == neg_inf() ? 0.f : Mh;
#pragma unroll
                for (int i = 0; i < NWD; ++i)
                    lh += lw_s[i][hd] * exp2_hw(mw_s[i][hd] - Mhs);
                if (S == 1) {
                    const float val = lh != 0.f ? acc / lh : 0.f; // 0 when no key was seen; NaN l gives NaN
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
        if (a.part_cnt) {
            const int64_t w = ((int64_t)(b * a.Hkv + g) * S + s) * 2;
            a.part_cnt[w] = je > jb ? je - jb : 0;
            a.part_cnt[w + 1] = je > jb ? n_skipped : 0;
        } else if (a.counters && je > jb) {
            atomicAdd(a.counters, (unsigned long long)(je - jb));
            atomicAdd(a.counters + 1, (unsigned long long)n_skipped);
        }
    }
}

// Log-sum-exp merge of split partials.  A thread owns 4 consecutive output
// columns of one (sequence, query head); a workgroup covers 256 / (dv/4)
// heads.  Weights are exp2(m_s - M) with M the largest split max among
// splits that saw keys (kept as a running max, one chunk of splits at a
// time); splits with l = 0 contribute nothing, and a NaN l (a NaN score)
// takes part, so the NaN reaches O.  The first workgroup of each sequence
// also sums the split workgroups' block counts into the counters.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeArgs a, int dv)
{
    if (a.part_cnt && blockIdx.x == 0 && threadIdx.x < 64) {
        const int n = a.Hkv * a.num_splits;
        const int32_t *pc = a.part_cnt + (int64_t)blockIdx.y * n * 2;
        unsigned long long vis = 0, skp = 0;
        for (int i = (int)threadIdx.x; i < n; i += 64) {
            vis += (unsigned)pc[2 * i];
            skp += (unsigned)pc[2 * i + 1];
        }
        for (int off = 32; off > 0; off >>= 1) {
            vis += __shfl_down(vis, off);
            skp += __shfl_down(skp, off);
        }
        if (threadIdx.x == 0 && vis != 0) {
            atomicAdd(a.counters, vis);
            atomicAdd(a.counters + 1, skp);
        }
    }
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
            if (s0 + i < S && ml[i].y != 0.f)
                Mc = fmaxf(Mc, ml[i].x);
        const float Ms = Mc == neg_inf() ? 0.f : Mc;
        const float r = M == neg_inf() ? 0.f : exp2_hw(M - Ms);
        num *= r;
        den *= r;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (s0 + i < S && ml[i].y != 0.f) {
                const float wgt = exp2_hw(ml[i].x - Ms);
                num += wgt * po[i];
                den += wgt * ml[i].y;
            }
        }
        M = Mc;
    }
    const f32x4 val = den != 0.f ? num * (1.f / den) : f32x4{};
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

template <int D, int NG, bool SKIP, bool OUT_BF16>
hipError_t launch_gqa(const DecodeArgs &a, hipStream_t stream, bool gaps)
{
    const dim3 grid(a.num_splits, a.Hkv, a.B);
    if (gaps) { // decisions through the skip kernel's rule, nothing executed, no partials
        hipLaunchKernelGGL((decode_gqa_kernel<D, true, false, 0, true, NG>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    if (a.page_table && a.page_shift >= 6)
        hipLaunchKernelGGL((decode_gqa_kernel<D, SKIP, OUT_BF16, 2, false, NG>), grid, dim3(256), 0, stream, a);
    else if (a.page_table)
        hipLaunchKernelGGL((decode_gqa_kernel<D, SKIP, OUT_BF16, 1, false, NG>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_gqa_kernel<D, SKIP, OUT_BF16, 0, false, NG>), grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1)
        return e;
    return launch_combine(a, D, OUT_BF16, stream);
}

template <int D, int NG>
hipError_t launch_gqa_g(const DecodeArgs &a, bool skip, bool out_bf16, hipStream_t stream, bool gaps)
{
    if (skip)
        return out_bf16 ? launch_gqa<D, NG, true, true>(a, stream, gaps) : launch_gqa<D, NG, true, false>(a, stream, gaps);
    return out_bf16 ? launch_gqa<D, NG, false, true>(a, stream, gaps) : launch_gqa<D, NG, false, false>(a, stream, gaps);
}

template <int D>
hipError_t launch_gqa_d(const DecodeArgs &a, bool skip, bool out_bf16, hipStream_t stream, bool gaps)
{
    if (a.G <= 16)
        return launch_gqa_g<D, 1>(a, skip, out_bf16, stream, gaps);
    if (a.G <= 32)
        return launch_gqa_g<D, 2>(a, skip, out_bf16, stream, gaps);
    return launch_gqa_g<D, 4>(a, skip, out_bf16, stream, gaps);
}

} // namespace

hipError_t launch_mla(const DecodeArgs &a, bool skip, bool out_bf16, hipStream_t stream, bool gaps);

hipError_t launch_decode(const DecodeArgs &a, int dqk, int dv, bool skip, bool out_bf16, hipStream_t stream,
                         bool gaps)
{
    if (a.B == 0)
        return hipSuccess;
    if (dqk == dv && a.G >= 1 && a.G <= 64) {
        if (dqk == 128)
            return launch_gqa_d<128>(a, skip, out_bf16, stream, gaps);
        if (dqk == 64)
            return launch_gqa_d<64>(a, skip, out_bf16, stream, gaps);
    }
    if (dqk == 576 && dv == 512 && a.G >= 1 && a.G <= 128)
        return launch_mla(a, skip, out_bf16, stream, gaps);
    return hipErrorInvalidValue;
}

} // namespace blasst
