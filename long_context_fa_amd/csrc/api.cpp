// api.cpp -- the C ABI of libblasst.so: argument validation, planning and
// dispatch to the HIP kernels.  Declarations and the full contract are in
// include/blasst.h.
#include "blasst.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

blasst_status fail(blasst_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

constexpr double kLog2e = 1.4426950408889634;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A bf16/fp32 tensor whose feature rows are loaded 16 bytes at a time.
blasst_status check_tensor(const blasst_tensor &t, const char *name, bool three_d, bool allow_fp32)
{
    if (t.ptr == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "%s: null pointer", name);
    if (t.dtype != BLASST_BF16 && !(allow_fp32 && t.dtype == BLASST_FP32))
        return fail(BLASST_ERR_UNSUPPORTED, "%s: unsupported dtype %d", name, (int)t.dtype);
    if (t.sb < 0 || t.sh < 0 || (!three_d && t.st <= 0))
        return fail(BLASST_ERR_INVALID_ARG, "%s: negative or zero stride", name);
    if (!aligned16(t.ptr))
        return fail(BLASST_ERR_INVALID_ARG, "%s: pointer not 16-byte aligned", name);
    const int64_t unit = t.dtype == BLASST_BF16 ? 8 : 4; // elements per 16 bytes
    if (t.sb % unit || t.sh % unit || (!three_d && t.st % unit))
        return fail(BLASST_ERR_INVALID_ARG, "%s: strides must be multiples of 16 bytes", name);
    return BLASST_OK;
}

blasst_status check_lambda(double lambda)
{
    if (!(lambda >= 0.0 && lambda < 1.0))
        return fail(BLASST_ERR_INVALID_ARG, "lambda must be in [0, 1) (got %g)", lambda);
    return BLASST_OK;
}

float log2_lambda(double lambda)
{
    return lambda == 0.0 ? -INFINITY : (float)std::log2(lambda);
}

// Kernel form of a sliding window: no window, or one at least as long as the
// sequence, becomes 2^30 (> any length the library accepts), so the kernels'
// lower-edge tests are never true.
int window_arg(int64_t window, int64_t len)
{
    return (window <= 0 || window >= len) ? (1 << 30) : (int)window;
}

} // namespace

extern "C" {

const char *blasst_status_str(blasst_status s)
{
    // A C caller may pass any int; reading it as an enum of this C++ file
    // would be undefined outside the enumerators, so its bytes are read.
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case BLASST_OK: return "ok";
    case BLASST_ERR_INVALID_ARG: return "invalid argument";
    case BLASST_ERR_UNSUPPORTED: return "unsupported configuration";
    case BLASST_ERR_WORKSPACE: return "workspace missing or too small";
    case BLASST_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char *blasst_last_error(void) { return g_last_error; }

int blasst_abi_version(void) { return BLASST_ABI_VERSION; }

} // extern "C"

namespace {

// gaps: the gap pass (blasst_prefill_gaps): o is neither read nor written.
blasst_status run_prefill(const blasst_prefill_params *p, void *hip_stream, bool gaps)
{
    if (p == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "params: null pointer");
    if (gaps && p->gap_map == nullptr && p->skip_map == nullptr && p->counters == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "the gap pass needs gap_map, skip_map or counters");
    if (p->B < 0 || p->L < 0)
        return fail(BLASST_ERR_INVALID_ARG, "B and L must be >= 0");
    if (p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv != 0)
        return fail(BLASST_ERR_INVALID_ARG, "need Hq, Hkv > 0 and Hq %% Hkv == 0 (Hq=%lld Hkv=%lld)",
                    (long long)p->Hq, (long long)p->Hkv);
    if (blasst_status s = check_lambda(p->lambda))
        return s;
    if (std::isnan(p->scale) || std::isinf(p->scale))
        return fail(BLASST_ERR_INVALID_ARG, "scale must be finite");
    if (p->window < 0 || (p->window > 0 && !p->causal))
        return fail(BLASST_ERR_INVALID_ARG, "window must be >= 0, and a window needs causal masking");
    if (p->B == 0 || p->L == 0)
        return BLASST_OK; // empty problem: nothing to read or write, buffers may be null
    if (blasst_status s = check_tensor(p->q, "q", false, false))
        return s;
    if (blasst_status s = check_tensor(p->k, "k", false, false))
        return s;
    if (blasst_status s = check_tensor(p->v, "v", false, false))
        return s;
    if (!gaps)
        if (blasst_status s = check_tensor(p->o, "o", false, true))
            return s;
    if (p->d != p->dv || (p->d != 64 && p->d != 128))
        return fail(BLASST_ERR_UNSUPPORTED, "prefill supports d = dv in {64, 128} (got d=%lld dv=%lld)",
                    (long long)p->d, (long long)p->dv);
    if (p->tile_q != 64 && p->tile_q != 128)
        return fail(BLASST_ERR_UNSUPPORTED, "tile_q must be 64 or 128 (got %d)", p->tile_q);
    if (p->block_k != 64)
        return fail(BLASST_ERR_UNSUPPORTED, "block_k must be 64 (got %d)", p->block_k);
    const int64_t nqt = (p->L + p->tile_q - 1) / p->tile_q;
    const int64_t nkb = (p->L + p->block_k - 1) / p->block_k;
    // One workgroup of 2 * tile_q threads per (query tile, head, batch).  A
    // launch counts work-items in 32 bits, so at most (2^32 - 1) / (2 tile_q)
    // workgroups fit (below 2^31 - 1, so B, Hq and the count also fit an int).
    // The bound is divided out so that no product of caller sizes overflows.
    const int64_t max_units = (int64_t)UINT32_MAX / (2 * p->tile_q);
    if (p->L > (int64_t)1 << 30 || p->Hq > max_units || p->B > max_units / (nqt * p->Hq))
        return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
    // The tile copies address the 64 rows of a K/V block with 32-bit byte
    // offsets from the block's first row.
    if (p->k.st > ((int64_t)1 << 24) || p->v.st > ((int64_t)1 << 24))
        return fail(BLASST_ERR_UNSUPPORTED, "k/v token strides above 2^24 elements are not supported");

    blasst::PrefillArgs a{};
    a.q = (const uint16_t *)p->q.ptr;
    a.k = (const uint16_t *)p->k.ptr;
    a.v = (const uint16_t *)p->v.ptr;
    a.o = p->o.ptr;
    a.q_sb = p->q.sb; a.q_sh = p->q.sh; a.q_st = p->q.st;
    a.k_sb = p->k.sb; a.k_sh = p->k.sh; a.k_st = p->k.st;
    a.v_sb = p->v.sb; a.v_sh = p->v.sh; a.v_st = p->v.st;
    a.o_sb = p->o.sb; a.o_sh = p->o.sh; a.o_st = p->o.st;
    a.B = (int)p->B; a.Hq = (int)p->Hq; a.Hkv = (int)p->Hkv; a.L = (int)p->L;
    a.nqt = (int)nqt; a.nkb = (int)nkb;
    const double scale = p->scale > 0 ? p->scale : 1.0 / std::sqrt((double)p->d);
    a.scale_log2 = (float)(scale * kLog2e);
    a.lnlam2 = log2_lambda(p->lambda);
    a.skip_map = p->skip_map;
    a.gap_map = p->gap_map;
    a.counters = p->counters;
    a.win = window_arg(p->window, p->L);
    if (p->counters) {
        // visited blocks of each query tile, as the kernel walks them: the
        // causal range ends at the block of the tile's last row and a window
        // starts it at the block of its first row's lowest key
        int64_t per_head = 0;
        for (int64_t t = 0; t < nqt; ++t) {
            const int64_t r0 = t * p->tile_q;
            const int64_t last_row = std::min<int64_t>(r0 + p->tile_q, p->L) - 1;
            const int64_t nvis = p->causal ? std::min<int64_t>(last_row / 64 + 1, nkb) : nkb;
            const int64_t jlo = (p->causal && r0 - a.win + 1 > 0) ? (r0 - a.win + 1) / 64 : 0;
            per_head += nvis - jlo;
        }
        a.visited_total = (unsigned long long)(per_head * p->B * p->Hq);
    }
    const bool skip = p->lambda > 0.0;
    hipError_t e = blasst::launch_prefill(a, (int)p->d, p->tile_q, p->causal != 0, skip,
                                          p->o.dtype == BLASST_BF16, (hipStream_t)hip_stream, gaps);
    if (e == hipErrorInvalidValue)
        return fail(BLASST_ERR_UNSUPPORTED, "no prefill kernel for this configuration");
    if (e != hipSuccess)
        return fail(BLASST_ERR_LAUNCH, "prefill launch failed: %s", hipGetErrorString(e));
    return BLASST_OK;
}

} // namespace

extern "C" {

blasst_status blasst_prefill(const blasst_prefill_params *p, void *hip_stream)
{
    return run_prefill(p, hip_stream, false);
}

blasst_status blasst_prefill_gaps(const blasst_prefill_params *p, void *hip_stream)
{
    return run_prefill(p, hip_stream, true);
}

namespace {

enum DecodeKind { KIND_NONE, KIND_GQA, KIND_MLA };

DecodeKind decode_kind(const blasst_decode_params *p)
{
    const int64_t G = p->Hq / p->Hkv;
    if (p->dqk == p->dv && (p->dqk == 64 || p->dqk == 128) && G >= 1 && G <= 64)
        return KIND_GQA;
    if (p->dqk == 576 && p->dv == 512 && p->Hkv == 1 && G >= 1 && G <= 128)
        return KIND_MLA;
    return KIND_NONE;
}

// pg: the paging fields of blasst_decode_paged, nullptr for a contiguous cache.
// gaps: the gap pass (blasst_decode_gaps), which does not touch o.
blasst_status validate_decode(const blasst_decode_params *p, const blasst_decode_paged_params *pg = nullptr,
                              bool gaps = false)
{
    if (p == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "params: null pointer");
    if (p->B < 0 || p->Lmax <= 0)
        return fail(BLASST_ERR_INVALID_ARG, "need B >= 0 and Lmax > 0");
    if (p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv != 0)
        return fail(BLASST_ERR_INVALID_ARG, "need Hq, Hkv > 0 and Hq %% Hkv == 0");
    if (blasst_status s = check_lambda(p->lambda))
        return s;
    if (std::isnan(p->scale) || std::isinf(p->scale))
        return fail(BLASST_ERR_INVALID_ARG, "scale must be finite");
    if (p->window < 0)
        return fail(BLASST_ERR_INVALID_ARG, "window must be >= 0");
    if (p->num_splits < 0 || p->num_splits > (p->Lmax + 63) / 64)
        return fail(BLASST_ERR_INVALID_ARG, "num_splits must be in 0..ceil(Lmax/64)");
    if (p->B == 0)
        return BLASST_OK; // empty batch: nothing to read or write, buffers may be null
    if (p->seq_lens == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "seq_lens: null pointer");
    if (blasst_status s = check_tensor(p->q, "q", true, false))
        return s;
    if (blasst_status s = check_tensor(p->k_cache, "k_cache", false, false))
        return s;
    if (blasst_status s = check_tensor(p->v_cache, "v_cache", false, false))
        return s;
    if (!gaps)
        if (blasst_status s = check_tensor(p->o, "o", true, true))
            return s;
    if (p->block_k != 64)
        return fail(BLASST_ERR_UNSUPPORTED, "block_k must be 64 (got %d)", p->block_k);
    const DecodeKind kind = decode_kind(p);
    if (kind == KIND_NONE)
        return fail(BLASST_ERR_UNSUPPORTED,
                    "decode supports dqk = dv in {64,128} with Hq/Hkv <= 64, or dqk=576, dv=512, Hkv=1, Hq <= 128");
    if (kind == KIND_MLA && p->v_cache.ptr != p->k_cache.ptr)
        return fail(BLASST_ERR_UNSUPPORTED, "latent decode needs v_cache to alias k_cache");
    if (p->Lmax > (int64_t)1 << 30 || p->B > 65535 || p->Hkv > 65535)
        return fail(BLASST_ERR_UNSUPPORTED, "problem too large for one launch");
    if (pg) {
        if (pg->page_table == nullptr)
            return fail(BLASST_ERR_INVALID_ARG, "page_table: null pointer");
        if (pg->num_pages < 1 || pg->num_pages > INT32_MAX)
            return fail(BLASST_ERR_INVALID_ARG, "num_pages must be in 1..2^31-1");
        if (pg->page_size < 16 || pg->page_size > ((int64_t)1 << 30) || (pg->page_size & (pg->page_size - 1)))
            return fail(BLASST_ERR_INVALID_ARG, "page_size must be a power of two >= 16 (got %lld)",
                        (long long)pg->page_size);
        if (pg->page_table_stride < (p->Lmax + pg->page_size - 1) / pg->page_size)
            return fail(BLASST_ERR_INVALID_ARG, "page_table_stride must be >= ceil(Lmax / page_size)");
    }
    // the latent kernel addresses a sequence's (or a page's) cache rows with
    // 32-bit byte offsets: rows * token stride * 2 < 2^31, tested by division
    const int64_t span = std::max<int64_t>(pg ? std::min(pg->page_size, p->Lmax) : p->Lmax, 1);
    if (kind == KIND_MLA && p->k_cache.st > (((int64_t)1 << 31) - 1) / (2 * span))
        return fail(BLASST_ERR_UNSUPPORTED, "latent decode needs rows * token stride * 2 < 2^31 bytes "
                                            "(rows = Lmax, or the page size of a paged cache)");
    return BLASST_OK;
}

int choose_splits(const blasst_decode_params *p)
{
    int64_t nkb = (p->Lmax + 63) / 64;
    if (p->window > 0 && (p->window + 63) / 64 + 1 < nkb)
        nkb = (p->window + 63) / 64 + 1; // blocks a window of this length can touch
    if (p->num_splits > 0)
        return p->num_splits;
    const int64_t units = p->B * p->Hkv;
    // GQA with up to 16 heads per KV head: aim for >= 4096 workgroups, about
    // sixteen rounds of the 256 resident at d = 128, so that the last, partly
    // filled round is a small share of the step.  Wider groups (17..64 heads)
    // and latent decode: one round of 256.  Their workgroups carry more fixed
    // work (the query load, one merge per 16 heads, larger partials), so more
    // splits cost more than the balance they buy (64 x 32K MQA at 70%: 4
    // splits 184 us, 32 splits 264 us).  Splits keep >= 64 blocks each, except
    // that >= 16 will do while the workgroups do not yet fill one round: a
    // workgroup's fixed work outweighs the balance that shorter splits buy
    // (148 x 32/8 x 4096 at 70%: 1 split 250 us, 4 splits 273 us).
    const int64_t want = (decode_kind(p) == KIND_MLA || p->Hq / p->Hkv > 16) ? 256 : 4096;
    int s = 1;
    while (units * s < want && (nkb / (2 * s) >= 64 || (units * s < 256 && nkb / (2 * s) >= 16)))
        s *= 2;
    return s;
}

size_t workspace_for(const blasst_decode_params *p, int S)
{
    if (S <= 1 || p->B == 0)
        return 0;
    const int64_t G = p->Hq / p->Hkv;
    const int64_t units = p->B * p->Hkv * S * G;
    const int64_t wgs = p->B * p->Hkv * S; // (visited, skipped) per split workgroup
    return (size_t)units * (size_t)(p->dv + 2) * sizeof(float) + (size_t)wgs * 2 * sizeof(int32_t) + 256;
}

} // namespace

blasst_status blasst_decode_plan(const blasst_decode_params *p, int *num_splits_used, size_t *workspace_bytes)
{
    if (blasst_status s = validate_decode(p))
        return s;
    const int S = choose_splits(p);
    if (num_splits_used)
        *num_splits_used = S;
    if (workspace_bytes)
        *workspace_bytes = workspace_for(p, S);
    return BLASST_OK;
}

} // extern "C"

namespace {

blasst_status run_decode(const blasst_decode_params *p, const blasst_decode_paged_params *pg, void *workspace,
                         size_t workspace_bytes, void *hip_stream, bool gaps = false)
{
    if (blasst_status s = validate_decode(p, pg, gaps))
        return s;
    if (gaps && p->gap_map == nullptr && p->skip_map == nullptr && p->counters == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "the gap pass needs gap_map, skip_map or counters");
    const int S = choose_splits(p);
    const size_t need = gaps ? 0 : workspace_for(p, S);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(BLASST_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned16(workspace))
        return fail(BLASST_ERR_INVALID_ARG, "workspace not 16-byte aligned");
    if (p->B == 0)
        return BLASST_OK;

    blasst::DecodeArgs a{};
    a.q = (const uint16_t *)p->q.ptr;
    a.k = (const uint16_t *)p->k_cache.ptr;
    a.v = (const uint16_t *)p->v_cache.ptr;
    a.o = p->o.ptr;
    a.q_sb = p->q.sb; a.q_sh = p->q.sh;
    a.k_sb = p->k_cache.sb; a.k_sh = p->k_cache.sh; a.k_st = p->k_cache.st;
    a.v_sb = p->v_cache.sb; a.v_sh = p->v_cache.sh; a.v_st = p->v_cache.st;
    a.o_sb = p->o.sb; a.o_sh = p->o.sh;
    a.seq_lens = p->seq_lens;
    a.B = (int)p->B; a.Hq = (int)p->Hq; a.Hkv = (int)p->Hkv; a.G = (int)(p->Hq / p->Hkv);
    a.Lmax = (int)p->Lmax; a.nkb = (int)((p->Lmax + 63) / 64); a.num_splits = S;
    const double scale = p->scale > 0 ? p->scale : 1.0 / std::sqrt((double)p->dqk);
    a.scale_log2 = (float)(scale * kLog2e);
    a.lnlam2 = log2_lambda(p->lambda);
    if (S > 1 && !gaps) {
        const int64_t units = p->B * p->Hkv * S * a.G;
        a.part_o = (float *)workspace;
        a.part_ml = a.part_o + units * p->dv;
        if (p->counters)
            a.part_cnt = (int32_t *)(a.part_ml + 2 * units);
    }
    a.skip_map = p->skip_map;
    a.gap_map = p->gap_map;
    a.counters = p->counters;
    a.win = window_arg(p->window, p->Lmax);
    a.sink_seed = p->sink_seed != 0;
    if (pg) {
        a.page_table = pg->page_table;
        a.pt_stride = pg->page_table_stride;
        a.num_pages = (int)pg->num_pages;
        int shift = 0;
        while (((int64_t)1 << shift) < pg->page_size)
            ++shift;
        a.page_shift = shift;
    }
    hipError_t e = blasst::launch_decode(a, (int)p->dqk, (int)p->dv, p->lambda > 0.0, p->o.dtype == BLASST_BF16,
                                         (hipStream_t)hip_stream, gaps);
    if (e == hipErrorInvalidValue)
        return fail(BLASST_ERR_UNSUPPORTED, "no decode kernel for this configuration");
    if (e != hipSuccess)
        return fail(BLASST_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
    return BLASST_OK;
}

} // namespace

extern "C" {

blasst_status blasst_decode(const blasst_decode_params *p, void *workspace, size_t workspace_bytes, void *hip_stream)
{
    return run_decode(p, nullptr, workspace, workspace_bytes, hip_stream);
}

blasst_status blasst_decode_gaps(const blasst_decode_params *p, void *hip_stream)
{
    return run_decode(p, nullptr, nullptr, 0, hip_stream, true);
}

blasst_status blasst_decode_paged_plan(const blasst_decode_paged_params *p, int *num_splits_used,
                                       size_t *workspace_bytes)
{
    if (p == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "params: null pointer");
    if (blasst_status s = validate_decode(&p->d, p))
        return s;
    const int S = choose_splits(&p->d);
    if (num_splits_used)
        *num_splits_used = S;
    if (workspace_bytes)
        *workspace_bytes = workspace_for(&p->d, S);
    return BLASST_OK;
}

blasst_status blasst_decode_paged(const blasst_decode_paged_params *p, void *workspace, size_t workspace_bytes,
                                  void *hip_stream)
{
    if (p == nullptr)
        return fail(BLASST_ERR_INVALID_ARG, "params: null pointer");
    return run_decode(&p->d, p, workspace, workspace_bytes, hip_stream);
}

} // extern "C"

// ------------------------------------------------------ no-allocation decode
// Split partials of blasst_decode_noalloc live in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy from module load until the process ends.  In host code the name is
// only a stand-in: its device address is taken once per device with
// hipGetSymbolAddress and that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[BLASST_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on that device).
blasst_status scratch_for_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(BLASST_ERR_LAUNCH, "no current HIP device (or device id >= %d)", kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(BLASST_ERR_LAUNCH, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BLASST_OK;
}

} // namespace

extern "C" blasst_status blasst_decode_noalloc(const blasst_decode_params *p, void *hip_stream)
{
    if (blasst_status s = validate_decode(p))
        return s;
    const size_t need = workspace_for(p, choose_splits(p));
    if (need > (size_t)BLASST_NOALLOC_SCRATCH_BYTES)
        return fail(BLASST_ERR_WORKSPACE,
                    "the split partials need %zu bytes but the no-allocation scratch holds %zu: pass a smaller "
                    "num_splits, or call blasst_decode with a workspace",
                    need, (size_t)BLASST_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0)
        if (blasst_status s = scratch_for_current_device(&ws))
            return s;
    return run_decode(p, nullptr, ws, need, hip_stream);
}

extern "C" {

// ------------------------------------------------------------- calibration
blasst_status blasst_calibrate(const blasst_calib_table *t, double target, int64_t L, int tile_q, int block_k,
                               int num_splits, double *lambda_out)
{
    if (t == nullptr || lambda_out == nullptr || t->target == nullptr || t->a == nullptr || t->n < 1)
        return fail(BLASST_ERR_INVALID_ARG, "calibration table or output missing");
    if (tile_q != t->tile_q || block_k != t->block_k || num_splits != t->num_splits)
        return fail(BLASST_ERR_INVALID_ARG,
                    "table fitted with tile_q=%d block_k=%d num_splits=%d; the call uses tile_q=%d block_k=%d "
                    "num_splits=%d (decisions depend on the tiling)",
                    t->tile_q, t->block_k, t->num_splits, tile_q, block_k, num_splits);
    for (int i = 0; i < t->n; ++i) {
        if (!(t->a[i] > 0.0) || std::isinf(t->a[i]))
            return fail(BLASST_ERR_INVALID_ARG, "table a[%d] must be positive and finite", i);
        if (i > 0 && !(t->target[i] > t->target[i - 1]))
            return fail(BLASST_ERR_INVALID_ARG, "table targets must be strictly increasing");
    }
    if (L <= 0)
        return fail(BLASST_ERR_INVALID_ARG, "L must be positive");
    if (!(target >= t->target[0] && target <= t->target[t->n - 1]))
        return fail(BLASST_ERR_INVALID_ARG, "target %g outside the calibrated range [%g, %g]", target,
                    t->target[0], t->target[t->n - 1]);
    int i = 0;
    while (i + 1 < t->n && target > t->target[i + 1])
        ++i;
    double lna;
    if (i + 1 >= t->n || target == t->target[i]) {
        lna = std::log(t->a[i]);
    } else {
        const double w = (target - t->target[i]) / (t->target[i + 1] - t->target[i]);
        lna = (1.0 - w) * std::log(t->a[i]) + w * std::log(t->a[i + 1]);
    }
    const double lam = std::exp(lna) / (double)L;
    if (!(lam < 1.0))
        return fail(BLASST_ERR_INVALID_ARG, "lambda = a/L = %g is not below 1", lam);
    *lambda_out = lam;
    return BLASST_OK;
}

blasst_status blasst_calibrate_search(const float *gaps, int64_t n, double target, double *lambda_out,
                                      double *reached_out)
{
    if (gaps == nullptr || lambda_out == nullptr || n < 1)
        return fail(BLASST_ERR_INVALID_ARG, "gaps/lambda_out missing or n < 1");
    if (!(target >= 0.0 && target <= 1.0))
        return fail(BLASST_ERR_INVALID_ARG, "target must be in [0, 1]");
    std::vector<double> g;
    g.reserve((size_t)n);
    for (int64_t i = 0; i < n; ++i)
        if (gaps[i] != -INFINITY && !std::isnan(gaps[i]))
            g.push_back((double)gaps[i]);
    const int64_t N = (int64_t)g.size();
    if (N == 0)
        return fail(BLASST_ERR_INVALID_ARG, "no visited pair in the gap map");
    std::sort(g.begin(), g.end());
    const int64_t k = std::min<int64_t>(N, std::max<int64_t>(0, (int64_t)std::ceil(target * (double)N)));
    double thr; // ln(lambda)
    if (k == 0)
        thr = -INFINITY;
    else if (k == N || std::isinf(g[(size_t)k]))
        thr = g[(size_t)k - 1] + 1.0;
    else
        thr = 0.5 * (g[(size_t)k - 1] + g[(size_t)k]);
    if (!(thr < 0.0))
        thr = -0x1p-40; // lambda must stay below 1
    const double lam = std::exp(thr);
    if (reached_out) {
        int64_t below = 0;
        for (double x : g)
            below += x < thr;
        *reached_out = (double)below / (double)N;
    }
    *lambda_out = lam;
    return BLASST_OK;
}

blasst_status blasst_calibrate_fit(const double *lambda_at_L, const int64_t *L, int n, double *a_out)
{
    if (lambda_at_L == nullptr || L == nullptr || a_out == nullptr || n < 1)
        return fail(BLASST_ERR_INVALID_ARG, "inputs missing or n < 1");
    double sum = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!(lambda_at_L[i] > 0.0 && lambda_at_L[i] < 1.0) || L[i] <= 0)
            return fail(BLASST_ERR_INVALID_ARG, "need 0 < lambda < 1 and L > 0 (entry %d)", i);
        sum += std::log(lambda_at_L[i] * (double)L[i]);
    }
    *a_out = std::exp(sum / n);
    return BLASST_OK;
}

} // extern "C"
