// mla.hip -- latent (MLA, absorbed form) decode with BLASST block skipping,
// gfx950: up to 128 query heads share one latent KV head of width 576 (512
// latent + 64 rotary); the value of a token is the first 512 columns of its
// latent row, so V costs no bytes of its own.
//
// Method: "BLASST: Dynamic BLocked Attention Sparsity via Softmax
// Thresholding" (gist.science/pt/paper/2512.12087, section 2; section 3 lists
// MHA/GQA/MQA/MLA support).  A query tile is the group of heads sharing the KV
// head -- here all G <= 128 -- and a key block is skipped when every head
// meets m~ - m < ln(lambda).  With V aliasing the latent K, a skipped block saves the
// exponentials and the P.V product (about half the matrix work), not bytes.
//
// One workgroup (4 waves x 32 heads, one wave per SIMD so that each wave can
// hold the 576-wide Q^T operand in VGPRs and its 512x32 O^T accumulator in
// AGPRs) walks the key blocks of one (sequence, split).  With G < 128 heads
// (e.g. 16 or 32 per GPU when the heads are sharded across GPUs) lane slot
// 32 w + n >= G computes head (32 w + n) mod G again: a repeated head leaves
// every vote (an AND over heads), block maximum and gap (maxima over heads)
// unchanged, so the loop needs no per-lane head test; only the writes of O or
// of the partials are limited to slots < G.  A wave on its own SIMD costs the
// others nothing:
//  * the 64 x 576 bf16 K tile (72 KB) is copied global -> LDS with
//    global_load_lds_dwordx4 into a double buffer, issued between the score
//    MFMAs of the previous block, with the non-temporal hint (a step reads
//    each cache row once).  In LDS a tile is a latent region (64 rows
//    of 512 columns, one 1 KB copy per row) and a rope region (64 rows of 64
//    columns); 16-byte chunks are XOR-swizzled by row so that the operand
//    reads hit distinct banks;
//  * S^T = K Q^T with the 32x32x16 bf16 MFMA (per-lane head statistics, as in
//    prefill); the 4 wave votes are exchanged through LDS;
//  * executed blocks: online softmax (rescale skipped when no head raised
//    its max) and O^T += V^T P^T with the V^T operand transpose-read
//    (ds_read_b64_tr_b16) from the same K tile;
//  * split partials (O, max, sum) go to the workspace for the log-sum-exp
//    combine kernel, or O is written directly for a single split.
// The gap pass (GAPS) keeps the tile copies, the scores, the votes and the
// maps, advances the running max over every block (a skip never changes it)
// and executes nothing.
#include "acc.h"
#include "kernels.h"

namespace blasst {

namespace {

constexpr int BC = 64;
constexpr int DQK = 576, DV = 512;
constexpr int LRB = DV * 2;              // 1024 bytes per latent row in LDS
constexpr int RRB = (DQK - DV) * 2;      // 128 bytes per rope row in LDS
constexpr int ROPE = BC * LRB;           // rope region offset in a tile (64 KB)
constexpr int TB = BC * (LRB + RRB);     // 73728 bytes per tile
constexpr int NWM = 4;                   // waves (32 heads each)
constexpr int CPW = TB / 1024 / NWM;     // 1 KB copies per tile per wave (18)
constexpr int NKK = DQK / 16;        // QK k-steps (36)
constexpr int NDT = DV / 32;         // O^T d tiles (16)

// Register placement.  Each wave owns 32 heads.  The O^T accumulator
// (512 x 32 fp32) is pinned in the 256 AGPRs, d-tile dt in a[16dt, 16dt+16)
// (acc.h); Q^T, the scores and the MFMA operands live in the 256 VGPRs.

// Chunk swizzles.  Latent rows (64 chunks, bank-aligned): physical chunk p of
// row r holds logical chunk p ^ swzl(r), a 4-bit XOR that is a permutation
// over r mod 16, so the 16 rows of a ds_read_b128 phase hit 16 distinct bank
// groups, and whose bits 2-3 differ across each aligned quad of rows, so the
// 4 rows x 4 chunks of a 32-lane ds_read_b64_tr_b16 phase do too.  Rope rows
// (8 chunks, 128 bytes): p ^ swzr(r), distinct over the 8 even and the 8 odd
// rows of a phase.
__host__ __device__ constexpr int swzl(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__host__ __device__ constexpr int swzr(int r) { return (r >> 1) & 7; }

// Sum of the 8 bf16 values of a P operand, in fp32.  The row sum adds the
// probabilities as the P.V product sees them (rounded to bf16), so that O is
// a weighted mean of V rows with one set of weights: with the latent rows'
// large values, an fp32 sum beside bf16 products leaves an error of up to
// 2^-9 of |V| when one key dominates.
__device__ __forceinline__ float sum_bf16x8(bf16x8 x)
{
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s += __builtin_bit_cast(float, u[i] << 16) + __builtin_bit_cast(float, u[i] & 0xffff0000u);
    return s;
}

template <bool SKIP, bool OUT_BF16, bool PAGED, bool GAPS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mla_kernel(const DecodeArgs a)
{
    __shared__ __attribute__((aligned(1024))) char smem[2 * TB];
    __shared__ int vote[2][NWM];
    __shared__ float gapw[2][NWM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, hh = lane >> 5;
    const int s = blockIdx.x, b = blockIdx.z;
    const int S = a.num_splits;
    const int head = 32 * w + n;
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

    // Rows of wave w's copies: the aligned 16-row group 16w.. of a block.  A
    // contiguous cache holds row r at kp + r * k_st; a paged cache holds it in
    // pool page page_table[b][r >> page_shift] at row r & pmask, and a page
    // of >= 16 rows holds the whole group (rows outside klo .. len-1 read the
    // nearest row inside, in the page of the group's first row clamped into
    // klo .. len-1): one wave-uniform page lookup per block.
    const uint16_t *kp = a.k + (PAGED ? 0 : b * a.k_sb);
    const int pmask = PAGED ? (1 << a.page_shift) - 1 : -1;
    auto group_base = [&](int j) -> const uint16_t * {
        if (!PAGED)
            return kp;
        int g0 = j * BC + 16 * w;
        g0 = g0 < len ? (g0 > klo ? g0 : klo) : len - 1;
        int id = a.page_table[b * a.pt_stride + (g0 >> a.page_shift)];
        id = id < 0 ? 0 : (id < a.num_pages ? id : a.num_pages - 1);
        return kp + (int64_t)id * a.k_sb;
    };

    // Q^T as the B operand: lane (n, hh) holds q[head][16kk + 8hh .. +7].
    bf16x8 qf[NKK];
    {
        // heads past G repeat head (32 w + n) mod G
        const uint16_t *qp = a.q + b * a.q_sb + (int64_t)(head % a.G) * a.q_sh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            qf[kk] = as_bf16x8(*(const u32x4 *)(qp + 16 * kk + 8 * hh));
    }

    // Tile copy: wave w fills rows [16w, 16w+16) with 18 DMA copies of 1 KB:
    // copy i < 16 is the latent part of row 16w+i (lane l loads logical
    // chunk l ^ swzl(i) into physical chunk l), copies 16 and 17 are the rope
    // parts of 8 rows each (lane l: row +l/8, physical chunk l%8, logical
    // chunk (l%8) ^ swzr(row)).  Rows outside klo .. len-1 re-read the nearest
    // row inside (finite data, masked later).  Offsets are 32-bit from the sequence (or page)
    // base gb = group_base(j) (the host checks rows * row stride).
    auto tile = [&](int it) { return smem + (it & 1) * TB; };
    const uint32_t smem_lds = lds_addr(smem); // the tiles as LDS byte addresses, for the copies
    auto tile_l = [&](int it) { return smem_lds + (uint32_t)((it & 1) * TB); };
    const uint32_t rowb = (uint32_t)a.k_st * 2;
    auto copy_one = [&](const uint16_t *gb, int j, uint32_t t, int i) {
        if (i < 16) {
            int key = j * BC + 16 * w + i;
            key = key < len ? (key > klo ? key : klo) : len - 1;
            copy16_to_lds_s<true>(gb + (int64_t)(key & pmask) * a.k_st, (uint32_t)(16 * (lane ^ swzl(i))),
                            t + (uint32_t)((16 * w + i) * LRB));
        } else {
            const int e = i - 16;
            int lr = lane >> 3;
            asm volatile("" : "+v"(lr)); // no loop-carried per-lane key registers
            int key = j * BC + 16 * w + 8 * e + lr;
            key = key < len ? (key > klo ? key : klo) : len - 1;
            const uint32_t off = LRB + 16 * ((lane & 7) ^ ((4 * e + (lane >> 4)) & 7)); // swzr of the row
            copy16_to_lds_s<true>(gb, (uint32_t)(key & pmask) * rowb + off, t + (uint32_t)(ROPE + (16 * w + 8 * e) * RRB));
        }
    };

    // LDS read offsets.  K operand, lane (n, hh), logical chunk c = 2kk + hh:
    // latent (kk < 32) at row n, chunk (c & 48) | ((c & 15) ^ swzl(n)): 8
    // per-lane offsets (kk % 8) plus immediates, the same for row n + 32; rope
    // (kk >= 32) at row n, chunk (c - 64) ^ swzr(n), computed per block.  V^T
    // operand: rows 16u + 4vh + vj and that + 8, logical chunk
    // 4dt + 2vmb + vq/2: 4 per-lane offsets (dt % 4) for each row quad.
    const int vg = lane >> 4, vs = lane & 15;
    const int vmb = vg & 1, vh = vg >> 1, vj = vs >> 2, vq = vs & 3;
    int koffl[8], voffv[2][4];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        koffl[q] = n * LRB + ((2 * q + hh) ^ swzl(n)) * 16;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ra = 4 * vh + vj + 8 * t;
#pragma unroll
        for (int x = 0; x < 4; ++x)
            voffv[t][x] = ra * LRB + ((4 * x + 2 * vmb + (vq >> 1)) ^ swzl(ra)) * 16 + (vq & 1) * 8;
    }

    if (!GAPS) // the gap pass holds no accumulator
        acc_zero();
    float m2 = neg_inf(), lsum = 0.f;
    int n_skipped = 0;

    // Iteration it handles block jb + it; with a sink seed (splits after the
    // first), a leading score-only iteration it = -1 handles block j0 and
    // sets the running max to its row maxima.  Tiles alternate by iteration.
    const int it0 = (a.sink_seed && s > 0 && jb < je) ? -1 : 0;
    if (jb < je) {
        const int jf = it0 < 0 ? j0 : jb;
        const uint16_t *gb = group_base(jf);
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            copy_one(gb, jf, tile_l(it0), i);
        wait_vmcnt<0>();
        lds_barrier();
    }
    for (int it = it0; jb + it < je; ++it) {
        const int j = it < 0 ? j0 : jb + it;
        const int jn = jb + it + 1; // block of the next iteration
        const char *kb = tile(it);
        // S^T = K_j Q^T, K operands read one k-step ahead.  The copy of
        // K_jn into the other buffer (free since the last barrier) is
        // issued between the score MFMAs, one 1 KB copy every two k-steps
        // (a DMA instruction holds the wave until the address unit accepts
        // it, so a burst would stall the MFMA stream).
        const bool dma = jn < je;
        const uint16_t *gbn = group_base(jn);
        const uint32_t tn = tile_l(it + 1);
        f32x16 sc[2];
        // rope offsets are recomputed here (4 per block) to spare registers
        int nl = n;
        asm volatile("" : "+v"(nl));
        auto kread = [&](int kk, int kt) {
            if (kk < 32)
                return *(const u32x4 *)(kb + koffl[kk & 7] + 256 * (kk >> 3) + kt * 32 * LRB);
            const int koffr = ROPE + nl * RRB + ((2 * (kk - 32) + hh) ^ swzr(nl)) * 16;
            return *(const u32x4 *)(kb + koffr + kt * 32 * RRB);
        };
        u32x4 ka[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
            ka[0][kt] = kread(0, kt);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (kk + 1 < NKK) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    ka[(kk + 1) & 1][kt] = kread(kk + 1, kt);
            }
            __builtin_amdgcn_sched_barrier(0);
            if ((kk & 1) == 0 && dma)
                copy_one(gbn, jn, tn, kk >> 1);
            if (kk == 0) {
                mfma_v_first2(sc[0], sc[1], ka[0][0], ka[0][1], qf[0]);
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    mfma_v(sc[kt], ka[kk & 1][kt], qf[kk]);
            }
        }
        mfma_v_drain2(sc[0], sc[1]);
        const int k0 = j * BC;
        if (k0 + BC > len || k0 < klo) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= len || key < klo)
                        sc[kt][r] = neg_inf();
                }
        }
        float mt = neg_inf();
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mt = fmaxf(mt, sc[kt][r]);
        mt = max_xor32(mt);
        float mt2 = mt * a.scale_log2;
        asm volatile("" : "+v"(mt2)); // a rounded value: the gap mt2 - m2 is the same in every kernel variant
        if (it < 0) {
            m2 = mt2; // the seed: no vote, no P.V for this block
            wait_vmcnt<0>();
            lds_barrier();
            continue;
        }
        const int par = it & 1;
        if (SKIP || want_maps) {
            const float dgap = mt2 == neg_inf() ? neg_inf() : mt2 - m2;
            if (SKIP) {
                const int wall = __all(!(dgap >= a.lnlam2));
                if (lane == 0)
                    vote[par][w] = wall;
            }
            if (want_maps) {
                const float wgap = wave_max(dgap);
                if (lane == 0)
                    gapw[par][w] = wgap;
            }
        }
        // Votes visible after this (the copy of K_{j+1} stays in flight).
        lds_barrier();
        bool skip = false;
        if (SKIP) {
            int all = 1;
#pragma unroll
            for (int i = 0; i < NWM; ++i)
                all &= vote[par][i];
            skip = __builtin_amdgcn_readfirstlane(all) != 0;
        }
        if (want_maps && tid == 0) {
            float g = neg_inf();
#pragma unroll
            for (int i = 0; i < NWM; ++i)
                g = fmaxf(g, gapw[par][i]);
            const int64_t idx = (int64_t)b * a.nkb + j;
            if (a.skip_map)
                a.skip_map[idx] = skip ? 1 : 0;
            if (a.gap_map)
                a.gap_map[idx] = g * 0.69314718055994531f;
        }
        if (GAPS) {
            m2 = fmaxf(m2, mt2); // the running max, over every block
            n_skipped += skip ? 1 : 0;
        } else if (!skip) {
            const float mnew = fmaxf(m2, mt2);
            const float msafe = mnew == neg_inf() ? 0.f : mnew;
            const float alpha = mnew > m2 ? exp2_hw(m2 - msafe) : 1.f;
            if (__any(mnew > m2))
                acc_scale(alpha);
            m2 = mnew;
            // P^T for k-step u (keys 16u..16u+15 in the sigma order) is
            // sc[u/2][8(u%2) + r]; the exponentials of step u+1 are spread
            // between the P.V MFMAs of step u.
            float rs = 0.f;
            f32x8 pv8;
            auto pexp = [&](int u, int r) {
                const float p = exp2_hw(__builtin_fmaf(sc[u >> 1][8 * (u & 1) + r], a.scale_log2, -msafe));
                pv8[r] = p;
            };
#pragma unroll
            for (int r = 0; r < 8; ++r)
                pexp(0, r);
            bf16x8 pf = cvt_bf16x8(pv8);
            rs += sum_bf16x8(pf);
            // O^T += V^T P^T, V = first 512 columns of the K tile.
            auto vread = [&](int m) {
                const int u = m / NDT, dt = m % NDT;
                const char *vb = kb + 16 * u * LRB + 256 * (dt >> 2);
                const i16x4 x0 = lds_read_tr16(vb + voffv[0][dt & 3]);
                const i16x4 x1 = lds_read_tr16(vb + voffv[1][dt & 3]);
                const u32x2 y0 = __builtin_bit_cast(u32x2, x0), y1 = __builtin_bit_cast(u32x2, x1);
                return u32x4{y0[0], y0[1], y1[0], y1[1]};
            };
            constexpr int NM = 4 * NDT;
            u32x4 va[3];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                va[m] = vread(m);
            bf16x8 pnext = pf;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int u = m / NDT, dt = m % NDT;
                if (m + 2 < NM)
                    va[(m + 2) % 3] = vread(m + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (dt == 0)
                    pf = pnext;
                acc_mfma(16 * dt, va[m % 3], pf);
                if (u + 1 < 4) {
                    if (dt < 8)
                        pexp(u + 1, dt);
                    else if (dt == 8) {
                        pnext = cvt_bf16x8(pv8);
                        rs += sum_bf16x8(pnext);
                    }
                }
            }
            mfma_drain();
            lsum = alpha * lsum + rs;
        } else {
            ++n_skipped;
        }
        // Own part of K_jn landed; after the barrier every wave is done
        // with this tile and all of K_jn is visible.
        wait_vmcnt<0>();
        lds_barrier();
    }

    // Output: O^T lane (n, hh) holds head `head`, d = 32dt + 8g + 4hh + i.
    const float l = lsum + __shfl_xor(lsum, 32);
    if (GAPS) {
        // no output
    } else if (32 * w >= a.G) {
        // no heads, no output
    } else if (S == 1) {
        const bool head_ok = head < a.G;
        const float inv = 1.f / l; // exactly 0 below when l = 0 (no key seen); NaN l gives NaN
        const bool none = l == 0.f;
        char *ob = (char *)a.o;
        const int64_t base = (int64_t)b * a.o_sb + (int64_t)head * a.o_sh;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const f32x16 od = acc_read(16 * dt);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                f32x4 v4 = {od[4 * g] * inv, od[4 * g + 1] * inv, od[4 * g + 2] * inv, od[4 * g + 3] * inv};
                if (none)
                    v4 = f32x4{};
                if (!head_ok)
                    continue;
                if (OUT_BF16)
                    *(bf16x4 *)(ob + 2 * (base + d)) = __builtin_convertvector(v4, bf16x4);
                else
                    *(f32x4 *)(ob + 4 * (base + d)) = v4;
            }
        }
    } else {
        const bool head_ok = head < a.G;
        const int64_t pu = ((int64_t)b * S + s) * a.G + head; // Hkv = 1
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const f32x16 od = acc_read(16 * dt);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * hh;
                if (head_ok)
                    *(f32x4 *)(a.part_o + pu * DV + d) =
                        f32x4{od[4 * g], od[4 * g + 1], od[4 * g + 2], od[4 * g + 3]};
            }
        }
        if (hh == 0 && head_ok) {
            a.part_ml[2 * pu] = m2;
            a.part_ml[2 * pu + 1] = l;
        }
    }
    if (tid == 0) {
        // Blocks that no split visits: before the window (first split writes
        // them) and past the sequence (last split).
        if (want_maps) {
            auto unvisited = [&](int j) {
                const int64_t idx = (int64_t)b * a.nkb + j;
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
            const int64_t w = ((int64_t)b * S + s) * 2; // Hkv = 1
            a.part_cnt[w] = je > jb ? je - jb : 0;
            a.part_cnt[w + 1] = je > jb ? n_skipped : 0;
        } else if (a.counters && je > jb) {
            atomicAdd(a.counters, (unsigned long long)(je - jb));
            atomicAdd(a.counters + 1, (unsigned long long)n_skipped);
        }
    }
}

} // namespace

hipError_t launch_combine(const DecodeArgs &a, int dv, bool out_bf16, hipStream_t stream);

namespace {

template <bool SKIP, bool OUT_BF16>
void launch_mla_variant(const DecodeArgs &a, dim3 grid, hipStream_t stream)
{
    if (a.page_table)
        hipLaunchKernelGGL((decode_mla_kernel<SKIP, OUT_BF16, true, false>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mla_kernel<SKIP, OUT_BF16, false, false>), grid, dim3(256), 0, stream, a);
}

} // namespace

hipError_t launch_mla(const DecodeArgs &a, bool skip, bool out_bf16, hipStream_t stream, bool gaps)
{
    if (a.G < 1 || a.G > 128 || a.Hkv != 1)
        return hipErrorInvalidValue;
    const dim3 grid(a.num_splits, 1, a.B);
    if (gaps) {
        hipLaunchKernelGGL((decode_mla_kernel<true, false, false, true>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    if (skip) {
        if (out_bf16)
            launch_mla_variant<true, true>(a, grid, stream);
        else
            launch_mla_variant<true, false>(a, grid, stream);
    } else {
        if (out_bf16)
            launch_mla_variant<false, true>(a, grid, stream);
        else
            launch_mla_variant<false, false>(a, grid, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1)
        return e;
    return launch_combine(a, DV, out_bf16, stream);
}

} // namespace blasst
