/*
 * c_abi_demo.c -- the C ABI of libblasst.so used from plain C, with no Python
 * and no torch (a check that the boundary stands on its own).
 *
 *   c_abi_demo host   host-only calls: ABI version, status strings, the
 *                     calibration calls, the decode planner, and the
 *                     rejection of an invalid argument.  Needs no GPU.
 *   c_abi_demo gpu    a small causal prefill on the GPU (buffers from
 *                     hipMalloc, bf16 inputs built here): at lambda = 0 nothing
 *                     is skipped, so O must equal dense causal softmax
 *                     attention, computed here in double on the same bf16
 *                     values; then the same call at lambda = 0.3 with a skip
 *                     map, whose entries must be 0, 1 or 255.
 *
 * Exit status 0 when every check holds.  Test code, not part of the library.
 */
#include <blasst.h>
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define CHECK(cond, ...)                                                                   \
    do {                                                                                   \
        if (!(cond)) {                                                                     \
            fprintf(stderr, "c_abi_demo: check failed (%s:%d): ", __FILE__, __LINE__);     \
            fprintf(stderr, __VA_ARGS__);                                                  \
            fprintf(stderr, "\n");                                                         \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

static uint16_t f2bf(float f) /* round to nearest even */
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static double bf2d(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t rng = 12345u;
static float urand(void) /* uniform in [-2, 2) */
{
    rng = rng * 1664525u + 1013904223u;
    return (float)(rng >> 8) / (float)(1u << 24) * 4.f - 2.f;
}

static int host_checks(void)
{
    CHECK(blasst_abi_version() == BLASST_ABI_VERSION, "abi version %d", blasst_abi_version());
    CHECK(strcmp(blasst_status_str(BLASST_OK), "ok") == 0, "status string");

    /* lambda = a / L: the fit of exact a / L values returns a */
    const double a = 1e-3;
    const int64_t Ls[3] = {4096, 8192, 32768};
    const double lam[3] = {a / 4096, a / 8192, a / 32768};
    double a_fit = 0;
    CHECK(blasst_calibrate_fit(lam, Ls, 3, &a_fit) == BLASST_OK, "fit: %s", blasst_last_error());
    CHECK(fabs(a_fit / a - 1) < 1e-12, "fit a = %g", a_fit);

    /* ln a interpolated linearly in the target */
    const double tg[2] = {0.5, 0.7}, av[2] = {1e-3, 1e-2};
    const blasst_calib_table table = {2, tg, av, 128, 64, 0}; /* fitted for tile 128, block 64, prefill */
    double l6 = 0;
    CHECK(blasst_calibrate(&table, 0.6, 8192, 128, 64, 0, &l6) == BLASST_OK, "calibrate: %s", blasst_last_error());
    CHECK(blasst_calibrate(&table, 0.6, 8192, 64, 64, 0, &l6) == BLASST_ERR_INVALID_ARG, "other tiling accepted");
    CHECK(fabs(l6 / (sqrt(1e-3 * 1e-2) / 8192) - 1) < 1e-9, "calibrate lambda = %g", l6);

    /* exact quantile of a gap map: half of the 4 visited gaps below ln(lambda) */
    const float gaps[6] = {-3.f, -2.f, -1.f, INFINITY, -INFINITY, -INFINITY};
    double ls = 0, reached = 0;
    CHECK(blasst_calibrate_search(gaps, 6, 0.5, &ls, &reached) == BLASST_OK, "search: %s", blasst_last_error());
    CHECK(log(ls) > -2 && log(ls) < -1 && fabs(reached - 0.5) < 1e-12, "search lambda %g reached %g", ls, reached);

    /* the planner validates without touching device memory (16-byte aligned
     * placeholders stand in for the buffers) */
    void *fake = (void *)(uintptr_t)0x100000;
    blasst_decode_params dp;
    memset(&dp, 0, sizeof dp);
    dp.B = 148; dp.Hq = 32; dp.Hkv = 8; dp.Lmax = 32768; dp.dqk = 128; dp.dv = 128;
    dp.q = (blasst_tensor){fake, BLASST_BF16, 32 * 128, 128, 0};
    dp.o = (blasst_tensor){fake, BLASST_BF16, 32 * 128, 128, 0};
    dp.k_cache = (blasst_tensor){fake, BLASST_BF16, 8 * 32768 * 128, 32768 * 128, 128};
    dp.v_cache = dp.k_cache;
    dp.seq_lens = (const int32_t *)fake;
    dp.lambda = 1e-3;
    dp.block_k = 64;
    int splits = 0;
    size_t ws = 0;
    CHECK(blasst_decode_plan(&dp, &splits, &ws) == BLASST_OK, "plan: %s", blasst_last_error());
    CHECK(splits >= 1 && ws > 0, "plan splits %d workspace %zu", splits, ws);

    /* invalid lambda: rejected before any launch, with a message */
    blasst_prefill_params pp;
    memset(&pp, 0, sizeof pp);
    pp.B = 1; pp.Hq = 1; pp.Hkv = 1; pp.L = 64; pp.d = 64; pp.dv = 64;
    pp.lambda = 2.0; pp.tile_q = 64; pp.block_k = 64; pp.causal = 1;
    CHECK(blasst_prefill(&pp, NULL) == BLASST_ERR_INVALID_ARG, "lambda = 2 accepted");
    CHECK(strstr(blasst_last_error(), "lambda") != NULL, "message: %s", blasst_last_error());
    printf("c_abi_demo host: ok (abi %d, %d splits, %zu workspace bytes)\n", blasst_abi_version(), splits, ws);
    return 0;
}

static int gpu_checks(void)
{
    enum { B = 1, HQ = 2, HKV = 1, L = 300, D = 64 };
    const size_t nq = (size_t)B * HQ * L * D, nk = (size_t)B * HKV * L * D;
    uint16_t *hq = malloc(nq * 2), *hk = malloc(nk * 2), *hv = malloc(nk * 2);
    float *ho = malloc(nq * 4);
    CHECK(hq && hk && hv && ho, "host allocation");
    for (size_t i = 0; i < nq; ++i)
        hq[i] = f2bf(urand());
    for (size_t i = 0; i < nk; ++i) {
        hk[i] = f2bf(urand());
        hv[i] = f2bf(urand());
    }
    void *dq, *dk, *dv, *dout;
    uint8_t *dskip;
    const int nqt = (L + 63) / 64, nkb = (L + 63) / 64;
    CHECK(hipMalloc(&dq, nq * 2) == hipSuccess && hipMalloc(&dk, nk * 2) == hipSuccess &&
              hipMalloc(&dv, nk * 2) == hipSuccess && hipMalloc(&dout, nq * 4) == hipSuccess &&
              hipMalloc((void **)&dskip, (size_t)B * HQ * nqt * nkb) == hipSuccess,
          "hipMalloc");
    CHECK(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(dk, hk, nk * 2, hipMemcpyHostToDevice) == hipSuccess &&
              hipMemcpy(dv, hv, nk * 2, hipMemcpyHostToDevice) == hipSuccess,
          "hipMemcpy to device");

    blasst_prefill_params p;
    memset(&p, 0, sizeof p);
    p.q = (blasst_tensor){dq, BLASST_BF16, (int64_t)HQ * L * D, (int64_t)L * D, D};
    p.k = (blasst_tensor){dk, BLASST_BF16, (int64_t)HKV * L * D, (int64_t)L * D, D};
    p.v = (blasst_tensor){dv, BLASST_BF16, (int64_t)HKV * L * D, (int64_t)L * D, D};
    p.o = (blasst_tensor){dout, BLASST_FP32, (int64_t)HQ * L * D, (int64_t)L * D, D};
    p.B = B; p.Hq = HQ; p.Hkv = HKV; p.L = L; p.d = D; p.dv = D;
    p.causal = 1; p.scale = 0.0; p.lambda = 0.0; p.tile_q = 64; p.block_k = 64;
    CHECK(blasst_prefill(&p, NULL) == BLASST_OK, "prefill: %s", blasst_last_error());
    CHECK(hipDeviceSynchronize() == hipSuccess, "sync");
    CHECK(hipMemcpy(ho, dout, nq * 4, hipMemcpyDeviceToHost) == hipSuccess, "hipMemcpy to host");

    /* dense causal softmax attention on the same bf16 values, in double */
    const double scale = 1.0 / sqrt((double)D);
    double maxerr = 0, sumerr = 0;
    double *s = malloc(sizeof(double) * L), *acc = malloc(sizeof(double) * D);
    CHECK(s && acc, "host allocation");
    for (int h = 0; h < HQ; ++h)
        for (int i = 0; i < L; ++i) {
            const uint16_t *qi = hq + ((size_t)h * L + i) * D;
            double m = -INFINITY, l = 0;
            for (int c = 0; c <= i; ++c) {
                double dot = 0;
                for (int e = 0; e < D; ++e)
                    dot += bf2d(qi[e]) * bf2d(hk[(size_t)c * D + e]);
                s[c] = dot * scale;
                m = s[c] > m ? s[c] : m;
            }
            memset(acc, 0, sizeof(double) * D);
            for (int c = 0; c <= i; ++c) {
                const double pc = exp(s[c] - m);
                l += pc;
                for (int e = 0; e < D; ++e)
                    acc[e] += pc * bf2d(hv[(size_t)c * D + e]);
            }
            for (int e = 0; e < D; ++e) {
                const double err = fabs(acc[e] / l - ho[((size_t)h * L + i) * D + e]);
                maxerr = err > maxerr ? err : maxerr;
                sumerr += err;
            }
        }
    const double meanerr = sumerr / (double)nq;
    CHECK(maxerr <= 1e-2 && meanerr <= 1e-3, "lambda = 0 against dense attention: max %g mean %g", maxerr,
          meanerr);

    /* lambda = 0.3 with a skip map: every entry 0 (executed), 1 (skipped) or 255 */
    p.lambda = 0.3;
    p.skip_map = dskip;
    CHECK(blasst_prefill(&p, NULL) == BLASST_OK, "prefill lambda 0.3: %s", blasst_last_error());
    uint8_t *hs = malloc((size_t)B * HQ * nqt * nkb);
    CHECK(hs != NULL, "host allocation");
    CHECK(hipDeviceSynchronize() == hipSuccess &&
              hipMemcpy(hs, dskip, (size_t)B * HQ * nqt * nkb, hipMemcpyDeviceToHost) == hipSuccess,
          "skip map copy");
    int skipped = 0;
    for (int i = 0; i < B * HQ * nqt * nkb; ++i) {
        CHECK(hs[i] == 0 || hs[i] == 1 || hs[i] == 255, "skip map entry %d = %d", i, hs[i]);
        skipped += hs[i] == 1;
    }
    printf("c_abi_demo gpu: ok (lambda 0: max-abs %.2e mean-abs %.2e against dense; lambda 0.3: %d blocks "
           "skipped)\n", maxerr, meanerr, skipped);
    (void)hipFree(dq); (void)hipFree(dk); (void)hipFree(dv); (void)hipFree(dout); (void)hipFree(dskip);
    free(hq); free(hk); free(hv); free(ho); free(s); free(acc); free(hs);
    return 0;
}

int main(int argc, char **argv)
{
    if (argc == 2 && strcmp(argv[1], "host") == 0)
        return host_checks();
    if (argc == 2 && strcmp(argv[1], "gpu") == 0)
        return gpu_checks();
    fprintf(stderr, "usage: c_abi_demo host|gpu\n");
    return 2;
}
