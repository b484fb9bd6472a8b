/* Test support: calls every entry point of the CPU oracle (oracle/oracle.c)
 * on small, ragged and edge-case shapes, so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py) checks the
 * oracle's indexing and arithmetic for out-of-bounds accesses and undefined
 * behaviour.  Prints one line per case; the exit status is 0 when every call
 * returned its expected status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint32_t rng_state = 12345u;
static uint32_t rnd(void)                    /* xorshift32 */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
/* finite 16-bit patterns of moderate magnitude: sign, exponent near the
 * bias, random mantissa */
static void fill16(uint16_t* p, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r = rnd();
        if (dtype == OR_BF16)
            p[i] = (uint16_t)(((r & 1u) << 15) | ((120u + (r >> 1) % 10u) << 7) | ((r >> 8) & 0x7Fu));
        else
            p[i] = (uint16_t)(((r & 1u) << 15) | ((10u + (r >> 1) % 8u) << 10) | ((r >> 8) & 0x3FFu));
    }
}
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) exit(3); return p; }

static int fails = 0;
static void expect(const char* what, int got, int want)
{
    printf("%-44s %s\n", what, got == want ? "ok" : "FAILED");
    if (got != want) fails++;
}

static void norm_ops(int64_t T, int64_t H, int dtype)
{
    uint16_t *x = xmalloc(2 * T * H), *r = xmalloc(2 * T * H), *ro = xmalloc(2 * T * H);
    uint16_t *g = xmalloc(2 * T * H), *sc = xmalloc(2 * T * H), *sh = xmalloc(2 * T * H);
    uint16_t *w = xmalloc(2 * H), *b = xmalloc(2 * H);
    uint8_t* q = xmalloc(T * H);
    uint8_t* s8 = xmalloc(T * H / 16 + 1);
    float* fs = xmalloc(4 * T + 4);
    fill16(x, T * H, dtype); fill16(r, T * H, dtype); fill16(g, T * H, dtype);
    fill16(sc, T * H, dtype); fill16(sh, T * H, dtype); fill16(w, H, dtype); fill16(b, H, dtype);
    char name[96];
    for (int wm = 0; wm < 3; ++wm)
        for (int qm = 0; qm < 2; ++qm) {
            snprintf(name, sizeof name, "resid_rmsnorm_fp8 T%lld H%lld w%d q%d", (long long)T, (long long)H, wm, qm);
            expect(name, oracle_resid_rmsnorm_fp8(x, r, ro, w, wm, 1e-6f, q, qm, 56.0f, fs, T, H, dtype), 0);
        }
    snprintf(name, sizeof name, "adarms_gate_res_fp8 T%lld H%lld", (long long)T, (long long)H);
    expect(name, oracle_adarms_gate_res_fp8(x, g, r, ro, sc, sh, 1e-6f, q, 1, 0.0f, fs, T, H, dtype), 0);
    if (H % 32 == 0) {
        snprintf(name, sizeof name, "resid_rmsnorm_mxfp4 T%lld H%lld", (long long)T, (long long)H);
        expect(name, oracle_resid_rmsnorm_mxfp4(x, r, ro, w, 1, 1e-6f, q, s8, T, H, dtype), 0);
        snprintf(name, sizeof name, "resid_layernorm mxfp4 T%lld H%lld", (long long)T, (long long)H);
        expect(name, oracle_resid_layernorm(x, r, ro, w, b, 1e-6f, 1, q, 0, 0.0f, fs, s8, T, H, dtype), 0);
    }
    snprintf(name, sizeof name, "resid_rmsnorm_nvfp4 T%lld H%lld", (long long)T, (long long)H);
    expect(name, oracle_resid_rmsnorm_nvfp4(x, r, ro, w, 2, 1e-6f, 0.02f, q, s8, T, H, dtype), 0);
    snprintf(name, sizeof name, "resid_layernorm_nvfp4 T%lld H%lld", (long long)T, (long long)H);
    expect(name, oracle_resid_layernorm_nvfp4(x, r, ro, w, b, 1e-6f, 0.02f, q, s8, T, H, dtype), 0);
    expect(name, oracle_resid_layernorm_nvfp4(x, r, ro, w, NULL, 1e-6f, 3.0f, q, s8, T, H, dtype), 0);
    snprintf(name, sizeof name, "resid_layernorm fp8 T%lld H%lld", (long long)T, (long long)H);
    expect(name, oracle_resid_layernorm(x, r, ro, w, NULL, 1e-6f, 0, q, 1, 0.0f, fs, s8, T, H, dtype), 0);
    free(x); free(r); free(ro); free(g); free(sc); free(sh); free(w); free(b); free(q); free(s8); free(fs);
}

static void qkv_ops(int64_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t pages, int dtype)
{
    int64_t NH = Hq + 2 * Hkv;
    uint16_t *qkv = xmalloc(2 * T * NH * D), *qo = xmalloc(2 * T * Hq * D);
    uint16_t *ko = xmalloc(2 * T * Hkv * D), *vo = xmalloc(2 * T * Hkv * D);
    uint16_t *kc = xmalloc(2 * (size_t)pages * P * Hkv * D), *vc = xmalloc(2 * (size_t)pages * P * Hkv * D);
    uint16_t *qw = xmalloc(2 * (size_t)Hq * D), *kw = xmalloc(2 * (size_t)Hq * D);
    int32_t* pos = xmalloc(4 * 3 * T);
    int32_t* table = xmalloc(4 * pages);
    fill16(qkv, T * NH * D, dtype); fill16(qw, (int64_t)Hq * D, dtype); fill16(kw, (int64_t)Hq * D, dtype);
    memset(kc, 0, 2 * (size_t)pages * P * Hkv * D); memset(vc, 0, 2 * (size_t)pages * P * Hkv * D);
    for (int i = 0; i < pages; ++i) table[i] = pages - 1 - i;
    /* in range, then -1 and one past the table: the error flag path */
    for (int64_t t = 0; t < T; ++t) pos[t] = (int32_t)(t % ((int64_t)P * pages));
    if (T > 2) { pos[1] = -1; pos[2] = P * pages; }
    int32_t err = 0;
    char name[96];
    for (int style = 0; style < 2; ++style) {
        snprintf(name, sizeof name, "qkv_normrope_kvwrite T%lld D%d style%d", (long long)T, D, style);
        oracle_qkv_normrope_kvwrite(qkv, qw, kw, 1e-6f, pos, 1e4f, style, 0.125f, qo, kc, vc, table,
                                    pages, P, pages, &err, T, Hq, Hkv, D, dtype);
        expect(name, err, T > 2 ? 1 : 0);
    }
    for (int t = 0; t < 3 * T; ++t) pos[t] = (int32_t)(rnd() % 64);
    int32_t sec[3] = {D / 2 - 2 * (D / 6), D / 6, D / 6};
    for (int kind = 0; kind < 3; ++kind)
        for (int full = 0; full < 2; ++full) {
            snprintf(name, sizeof name, "qk_norm_rope T%lld D%d kind%d full%d", (long long)T, D, kind, full);
            expect(name, oracle_qk_norm_rope(qkv, kind, full, qw, full ? NULL : kw, kw, NULL, 1e-6f, pos,
                                             full ? 3 : 1, sec, 1e4f, full, 1.0f, qo, ko, vo, T, Hq, Hkv,
                                             D, dtype), 0);
        }
    free(qkv); free(qo); free(ko); free(vo); free(kc); free(vc); free(qw); free(kw); free(pos); free(table);
}

static void act_ops(int64_t T, int64_t I, int dtype)
{
    uint16_t* gu = xmalloc(2 * T * 2 * I);
    double* gd = xmalloc(8 * T * 2 * I);
    uint8_t* q = xmalloc(T * I);
    uint8_t* s8 = xmalloc(T * I / 32 + 1);
    float* fs = xmalloc(4 * T * (I / 128) + 4);
    fill16(gu, T * 2 * I, dtype);
    for (int64_t i = 0; i < T * 2 * I; ++i) gd[i] = (double)(int32_t)(rnd() % 2001u - 1000) / 250.0;
    char name[96];
    for (int a = 0; a < 3; ++a) {
        snprintf(name, sizeof name, "gated_act_fp8 T%lld I%lld act%d", (long long)T, (long long)I, a);
        expect(name, oracle_gated_act_fp8(gu, a, q, fs, T, I, dtype), 0);
        snprintf(name, sizeof name, "gated_act_mxfp4 T%lld I%lld act%d", (long long)T, (long long)I, a);
        expect(name, oracle_gated_act_mxfp4(gu, a, q, s8, T, I, dtype), 0);
        snprintf(name, sizeof name, "gated_act_fp8_f64 T%lld I%lld act%d", (long long)T, (long long)I, a);
        expect(name, oracle_gated_act_fp8_f64(gd, a, q, fs, T, I), 0);
    }
    free(gu); free(gd); free(q); free(s8); free(fs);
}

int main(void)
{
    norm_ops(1, 16, OR_F16);
    norm_ops(3, 1040, OR_BF16);          /* ragged: not a multiple of 32 */
    norm_ops(2, 4096, OR_BF16);
    norm_ops(0, 64, OR_F16);             /* no rows */
    qkv_ops(5, 4, 2, 64, 4, 3, OR_BF16);
    qkv_ops(3, 2, 1, 96, 2, 2, OR_F16);
    qkv_ops(2, 1, 1, 256, 1, 2, OR_BF16);
    act_ops(2, 384, OR_BF16);
    act_ops(1, 128, OR_F16);
    /* codecs over every code / a sweep */
    for (int c = 0; c < 65536; ++c) {
        or_f16_encode(or_f16_decode((uint16_t)c));
        or_bf16_encode(or_bf16_decode((uint16_t)c));
    }
    for (int c = 0; c < 256; ++c) or_e4m3_encode(or_e4m3_decode((uint8_t)c));
    for (int c = 0; c < 16; ++c) or_e2m1_encode(or_e2m1_decode((uint8_t)c));
    for (int k = -140; k < 140; ++k) or_mx_scale_code(1.5 * (k < 0 ? 1.0 / (double)(1ull << ((-k) % 60)) : (double)(1ull << (k % 60))));
    printf("%d failures\n", fails);
    return fails ? 1 : 0;
}
