/*
 * abi_check.c -- libep.so's C ABI used from plain C: no Python, no torch, only
 * include/ep.h and the HIP runtime.  Test infrastructure.
 *
 *   abi_check cpu   static calls and argument validation (no device work)
 *   abi_check gpu   a fresh dispatch, its handle's layout and a combine on
 *                   the device, each checked here from its definition
 *                   ("Dispatch Operation" and "Combine Operation" of the
 *                   DeepEP Buffer Class API page): packed row i is the row
 *                   of token recv_src_idx[i]; segments follow rank order and
 *                   token order inside a segment; the combine of the packed
 *                   rows gives n_t * x_t (small integers, so every fp32 sum
 *                   and the bf16 rounding are exact).
 * Prints one line and exits 0 on success; on a failed check prints it and
 * exits 1.
 */
/* Built by gcc, not hipcc: the HIP runtime header needs its platform named
 * (hipcc would define this itself).  There is no other platform here. */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"

#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "abi_check: %s:%d: check failed: %s\n", __FILE__, \
                    __LINE__, #c);                                            \
            return 1;                                                         \
        }                                                                     \
    } while (0)
#define HIPOK(c) CHECK((c) == hipSuccess)

static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t bf16_exact(float f) /* f exactly representable in bf16 */
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int cpu_checks(void)
{
    CHECK(ep_version() == ((2 << 16) | 4));
    CHECK(strcmp(ep_status_str(EP_OK), "ok") == 0);
    CHECK(strcmp(ep_status_str(42), "unknown status") == 0);
    ep_dims d = {16, 64, 2, 8, 4, 1};
    CHECK(ep_max_recv_rows(&d) == 16 * 2);
    ep_dims bad = {16, 12, 2, 8, 4, 1}; /* rows not whole 16-byte vectors */
    ep_handle *h = NULL;
    CHECK(ep_dispatch(&bad, NULL, NULL, NULL, NULL, &h, NULL, NULL, NULL, 0, NULL, NULL) ==
          EP_ERR_ALIGN);
    bad.hidden = 64;
    bad.num_experts = 10; /* not a multiple of the ranks */
    CHECK(ep_get_dispatch_layout(&bad, NULL, NULL, NULL, &h, NULL) == EP_ERR_INVALID);
    CHECK(h == NULL);
    CHECK(ep_combine(NULL, 64, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
          EP_ERR_HANDLE);
    CHECK(ep_handle_nbytes(NULL) == 0);
    ep_handle_free(NULL);
    int a, b, c;
    CHECK(ep_tuning_list("ll", -1, &a, &b, &c) == 3);
    CHECK(ep_tuning_list("dispatch", -1, &a, &b, &c) > 0);
    return 0;
}

static int gpu_checks(void)
{
    enum { T = 300, H = 136, K = 3, E = 24, R = 6, C = 5 };
    const int epr = E / R;
    ep_dims d = {T, H, K, E, R, C};
    const int64_t cap = ep_max_recv_rows(&d);
    CHECK(cap == (int64_t)T * K);

    int64_t *topk = malloc(sizeof(int64_t) * T * K);
    float *w = malloc(sizeof(float) * T * K);
    uint16_t *x = malloc(sizeof(uint16_t) * T * H);
    uint32_t s = 12345u;
    for (int t = 0; t < T; ++t) {
        int used[E];
        memset(used, 0, sizeof used);
        for (int k = 0; k < K; ++k) {
            s = s * 1664525u + 1013904223u;
            int e = (int)((s >> 8) % E);
            while (used[e])
                e = (e + 1) % E;
            used[e] = 1;
            topk[t * K + k] = ((s >> 4) % 11 == 0) ? -1 : e; /* some masked slots */
            w[t * K + k] = 0.25f * (float)(k + 1);
        }
        for (int hh = 0; hh < H; ++hh)
            x[t * H + hh] = bf16_exact((float)((t * 7 + hh) % 17 - 8));
    }

    void *dx, *drecv, *dout;
    int64_t *dtopk, *drti;
    float *dw, *drtw, *dcw;
    int32_t *dsrc, *drpm;
    HIPOK(hipMalloc(&dx, sizeof(uint16_t) * T * H));
    HIPOK(hipMalloc((void **)&dtopk, sizeof(int64_t) * T * K));
    HIPOK(hipMalloc((void **)&dw, sizeof(float) * T * K));
    HIPOK(hipMalloc(&drecv, sizeof(uint16_t) * cap * H));
    HIPOK(hipMalloc((void **)&drti, sizeof(int64_t) * cap * K));
    HIPOK(hipMalloc((void **)&drtw, sizeof(float) * cap * K));
    HIPOK(hipMalloc(&dout, sizeof(uint16_t) * T * H));
    HIPOK(hipMalloc((void **)&dcw, sizeof(float) * T * K));
    HIPOK(hipMalloc((void **)&dsrc, sizeof(int32_t) * cap));
    HIPOK(hipMalloc((void **)&drpm, sizeof(int32_t) * R));
    HIPOK(hipMemcpy(dx, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dtopk, topk, sizeof(int64_t) * T * K, hipMemcpyHostToDevice));
    HIPOK(hipMemcpy(dw, w, sizeof(float) * T * K, hipMemcpyHostToDevice));

    ep_handle *h = NULL;
    int64_t n = -1;
    CHECK(ep_dispatch(&d, dx, dtopk, dw, NULL, &h, drecv, drti, drtw, cap, &n, NULL) == EP_OK);
    CHECK(h != NULL && n > 0 && n <= cap);
    ep_layout_out lo;
    memset(&lo, 0, sizeof lo);
    lo.rank_prefix_matrix = drpm;
    lo.recv_src_idx = dsrc;
    lo.recv_src_cap = cap;
    CHECK(ep_handle_copy_layout(h, &lo, NULL) == EP_OK);
    CHECK(ep_combine(h, H, drecv, cap, drtw, NULL, NULL, NULL, dout, dcw, NULL) == EP_OK);
    HIPOK(hipDeviceSynchronize());

    uint16_t *recv = malloc(sizeof(uint16_t) * n * H);
    int64_t *rti = malloc(sizeof(int64_t) * n * K);
    float *rtw = malloc(sizeof(float) * n * K);
    uint16_t *out = malloc(sizeof(uint16_t) * T * H);
    float *cw = malloc(sizeof(float) * T * K);
    int32_t *src = malloc(sizeof(int32_t) * n);
    int32_t rpm[R];
    HIPOK(hipMemcpy(recv, drecv, sizeof(uint16_t) * n * H, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(rti, drti, sizeof(int64_t) * n * K, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(rtw, drtw, sizeof(float) * n * K, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(out, dout, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(cw, dcw, sizeof(float) * T * K, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(src, dsrc, sizeof(int32_t) * n, hipMemcpyDeviceToHost));
    HIPOK(hipMemcpy(rpm, drpm, sizeof(rpm), hipMemcpyDeviceToHost));

    /* segment r holds, in token order, the tokens with a valid slot on r */
    int64_t row = 0;
    for (int r = 0; r < R; ++r) {
        for (int t = 0; t < T; ++t) {
            int hit = 0;
            for (int k = 0; k < K; ++k)
                hit |= topk[t * K + k] >= 0 && topk[t * K + k] / epr == r;
            if (!hit)
                continue;
            CHECK(row < n);
            CHECK(src[row] == t);
            CHECK(memcmp(recv + row * H, x + t * H, sizeof(uint16_t) * H) == 0);
            for (int k = 0; k < K; ++k) {
                const int64_t e = topk[t * K + k];
                const int mine = e >= 0 && e / epr == r;
                CHECK(rti[row * K + k] == (mine ? e - (int64_t)r * epr : -1));
                CHECK(rtw[row * K + k] == (mine ? w[t * K + k] : 0.0f));
            }
            ++row;
        }
        CHECK(rpm[r] == row);
    }
    CHECK(row == n);
    /* combine of the packed rows: n_t copies of x_t */
    for (int t = 0; t < T; ++t) {
        int nt = 0;
        for (int r = 0; r < R; ++r) {
            int hit = 0;
            for (int k = 0; k < K; ++k)
                hit |= topk[t * K + k] >= 0 && topk[t * K + k] / epr == r;
            nt += hit;
        }
        for (int hh = 0; hh < H; ++hh)
            CHECK(bf16_value(out[t * H + hh]) == (float)nt * bf16_value(x[t * H + hh]));
        for (int k = 0; k < K; ++k)
            CHECK(cw[t * K + k] == (topk[t * K + k] >= 0 ? w[t * K + k] : 0.0f));
    }
    ep_handle_free(h);
    CHECK(ep_pool_trim() == EP_OK);
    printf("abi_check gpu: ok (N=%lld packed rows checked)\n", (long long)n);
    return 0;
}

int main(int argc, char **argv)
{
    if (cpu_checks() != 0)
        return 1;
    if (argc > 1 && strcmp(argv[1], "gpu") == 0)
        return gpu_checks();
    printf("abi_check cpu: ok\n");
    return 0;
}
