// kernels.h -- internal launch interface between the C-ABI layer and the
// HIP kernels of libblasst.so (not installed, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

struct PrefillArgs {
    const uint16_t *q, *k, *v; // bf16 bit patterns
    void *o;
    int64_t q_sb, q_sh, q_st, k_sb, k_sh, k_st, v_sb, v_sh, v_st, o_sb, o_sh, o_st;
    int B, Hq, Hkv, L, nqt, nkb;
    float scale_log2; // scale * log2(e): scores are kept in base-2 units
    float lnlam2;     // log2(lambda), -inf for lambda = 0
    uint8_t *skip_map;
    float *gap_map;
    unsigned long long *counters;
    int win; // sliding window: query i sees keys > i - win (2^30 when there is none)
    // (tile, block) pairs the launch visits, computed on the host: workgroup 0
    // adds it to counters[0] once, and a workgroup adds its skipped count to
    // counters[1] only when it skipped a block, so that a launch does not end
    // with thousands of workgroups adding into the same two words.
    unsigned long long visited_total;
};

// Launches the prefill kernel for (d, tile_q, causal, skip, out dtype); gaps
// selects the gap pass (maps and counters only, O untouched).
// Returns hipErrorInvalidValue if no kernel is compiled for the combination.
hipError_t launch_prefill(const PrefillArgs &a, int d, int tile_q, bool causal, bool skip,
                          bool out_bf16, hipStream_t stream, bool gaps);

struct DecodeArgs {
    const uint16_t *q, *k, *v;
    void *o;
    int64_t q_sb, q_sh, k_sb, k_sh, k_st, v_sb, v_sh, v_st, o_sb, o_sh;
    const int32_t *seq_lens;
    int B, Hq, Hkv, G, Lmax, nkb, num_splits;
    int win; // sliding window: the query sees the last win keys (2^30 when there is none)
    int sink_seed; // splits s >= 1 start the running max from the row maxima of block j0
    float scale_log2;
    float lnlam2;
    float *part_o;  // [B][Hkv][S][G][dv] fp32 (num_splits > 1)
    float *part_ml; // [B][Hkv][S][G][2]  fp32 (max in log2 units, sum)
    uint8_t *skip_map;
    float *gap_map;
    unsigned long long *counters;
    // Split workgroups' (visited, skipped) block counts, [B][Hkv][S][2]
    // int32, summed into counters by the combine kernel: set when counters
    // are asked for with num_splits > 1, so that thousands of workgroups do
    // not each add into the same two words.  Null: workgroups add directly.
    int32_t *part_cnt;
    // Paged cache (page_table != nullptr): k/v point at page pools whose
    // batch stride is the page stride; row r of sequence b lives in pool page
    // page_table[b * pt_stride + (r >> page_shift)] (ids clamped into
    // [0, num_pages)), at row r & (2^page_shift - 1) of that page.
    const int32_t *page_table;
    int64_t pt_stride;
    int num_pages, page_shift;
};

// GQA/MQA/MHA decode (dqk = dv in {64, 128}, G <= 64) and latent (MLA) decode
// (dqk 576, dv 512, G 128).  The combine kernel runs when num_splits > 1.
// gaps selects the gap pass (maps and counters only: no O, no partials).
hipError_t launch_decode(const DecodeArgs &a, int dqk, int dv, bool skip, bool out_bf16,
                         hipStream_t stream, bool gaps);

// Log-sum-exp merge of the split partials into O (num_splits > 1).
hipError_t launch_combine(const DecodeArgs &a, int dv, bool out_bf16, hipStream_t stream);

} // namespace blasst
