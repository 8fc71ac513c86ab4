/* Driver of the sanitizer build of the C ABI's host code: calls every entry
 * point of include/ssd.h with host buffers of exactly the documented sizes
 * (the launchers are stubs that touch every byte a kernel would), and every
 * error path, checking the returned status.  Exit status 0 = all checks
 * passed; AddressSanitizer / UndefinedBehaviorSanitizer abort on a finding. */
#define _POSIX_C_SOURCE 200112L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssd.h"

uint64_t stub_launches(void);

static int g_fail = 0;
#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        if (!(cond)) {                                                          \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);                \
            fprintf(stderr, __VA_ARGS__);                                       \
            fprintf(stderr, " (%s)\n", ssd_last_error());                       \
            g_fail = 1;                                                         \
        }                                                                       \
    } while (0)

static void *buf(size_t n) {
    /* 16-byte aligned, never NULL, exactly n bytes as far as ASan knows */
    void *p = NULL;
    if (posix_memalign(&p, 64, n ? n : 1) != 0) abort();
    memset(p, 0, n ? n : 1);
    return p;
}

typedef struct {
    int64_t b, L, H, P, N, G, Q;
    int io;           /* SSD_F32 or SSD_BF16 */
    int with_D, with_seq, with_init, with_final, split_len, headdim_block, fused;
} fwd_case;

static void run_fwd(const fwd_case *c) {
    ssd_shape_t s = {c->b, c->L, c->H, c->P, c->N, c->G};
    const size_t esz = c->io == SSD_BF16 ? 2 : 4;
    const size_t nx = (size_t)(c->b * c->L * c->H * c->P), nbc = (size_t)(c->b * c->L * c->G * c->N);
    const size_t nst = (size_t)(c->b * c->H * c->P * c->N);
    void *x = buf(nx * esz), *y = buf(nx * esz), *B = buf(nbc * esz), *C = buf(nbc * esz);
    float *dt = buf((size_t)(c->b * c->L * c->H) * 4), *A = buf((size_t)c->H * 4);
    float *D = c->with_D ? buf((size_t)c->H * 4) : NULL;
    int32_t *seq = c->with_seq ? buf((size_t)(c->b * c->L) * 4) : NULL;
    float *h0 = c->with_init ? buf(nst * 4) : NULL, *fs = c->with_final ? buf(nst * 4) : NULL;
    ssd_options_t o;
    memset(&o, 0, sizeof(o));
    o.split_len = c->split_len;
    o.headdim_block = c->headdim_block;
    const size_t ws_bytes = ssd_fwd_ex_workspace_bytes(&s, c->Q, c->io, &o);
    void *ws = ws_bytes ? buf(ws_bytes) : NULL;
    ssd_status_t st;
    if (c->fused) {
        ssd_fused_t f;
        memset(&f, 0, sizeof(f));
        f.dt_bias = buf((size_t)c->H * 4);
        f.z = buf(nx * esz);
        f.dt_softplus = 1;
        f.dt_clamp = 1;
        f.dt_min = 1e-4f;
        f.dt_max = 1.f;
        st = ssd_fwd_fused(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, &f, ws, ws_bytes, &o, NULL);
        free((void *)f.dt_bias);
        free((void *)f.z);
    } else {
        st = ssd_fwd_ex(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, ws, ws_bytes, &o, NULL);
    }
    CHECK(st == SSD_OK, "fwd b%lld L%lld H%lld P%lld N%lld G%lld Q%lld io%d split%d pb%d: status %d",
          (long long)c->b, (long long)c->L, (long long)c->H, (long long)c->P, (long long)c->N,
          (long long)c->G, (long long)c->Q, c->io, c->split_len, c->headdim_block, (int)st);
    if (c->io == SSD_BF16 && ws_bytes) {
        /* the per-group operands survive: the reuse option over the same workspace */
        o.flags = SSD_OPT_REUSE_GROUP_OPERANDS;
        st = ssd_fwd_ex(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, ws, ws_bytes, &o, NULL);
        CHECK(st == SSD_OK, "reuse: status %d", (int)st);
        /* the segsum ablation's mask variants in the head kernel: chunk 256,
           dstate 64 or 128, headdim blocks of 32 or 64 */
        const int64_t pb = c->headdim_block ? c->headdim_block : ssd_plan_headdim_block(&s, c->Q, c->io);
        const int var_ok = c->Q == 256 && (c->N == 64 || c->N == 128) && (pb == 32 || pb == 64);
        for (int v = 0; v < 2; ++v) {
            o.flags = SSD_OPT_REUSE_GROUP_OPERANDS | (v ? SSD_OPT_SEGSUM_DIFF : SSD_OPT_SEGSUM_DIRECT);
            st = ssd_fwd_ex(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, ws, ws_bytes, &o, NULL);
            CHECK(st == (var_ok ? SSD_OK : SSD_ERR_UNSUPPORTED), "segsum variant %d (pb %lld): status %d", v,
                  (long long)pb, (int)st);
        }
        o.flags = 0;
        /* the head kernel's segsum factors */
        const int64_t words = ssd_segsum_record_words(c->Q);
        const int64_t nch = (c->L + c->Q - 1) / c->Q;
        float *rec = buf((size_t)(c->b * c->H * nch * words) * 4);
        st = ssd_debug_fwd_segsum_factors(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, ws,
                                          ws_bytes, &o, rec, NULL);
        CHECK(st == SSD_OK, "segsum factors (head kernel): status %d", (int)st);
        st = ssd_debug_segsum_factors(&s, dt, A, seq, c->Q, rec, NULL);
        CHECK(st == SSD_OK, "segsum factors (export): status %d", (int)st);
        free(rec);
    }
    {
        /* the mask exports: whole mask of the last chunk, and per-chunk sums */
        const int64_t nch = (c->L + c->Q - 1) / c->Q;
        float *mask = buf((size_t)(c->b * c->H * c->Q * c->Q) * 4);
        float *sums = buf((size_t)(c->b * c->H * nch) * 4);
        st = ssd_debug_chunk_mask(&s, dt, A, seq, c->Q, nch - 1, 1, mask, NULL);
        CHECK(st == SSD_OK, "mask export: status %d", (int)st);
        for (int v = 0; v < 3; ++v) {
            st = ssd_debug_chunk_mask_ex(&s, dt, A, seq, c->Q, 0, nch, v, NULL, sums, NULL);
            CHECK(st == SSD_OK, "mask sums, variant %d: status %d", v, (int)st);
        }
        st = ssd_debug_chunk_mask_ex(&s, dt, A, seq, c->Q, nch - 1, 2, 0, mask, NULL, NULL);
        CHECK(st == SSD_ERR_SHAPE, "mask range past the end: status %d", (int)st);
        free(mask);
        free(sums);
    }
    /* the allocation-free entry point: its fixed workspace, or a clear refusal */
    if (!c->fused && c->split_len == 0 && c->headdim_block == 0) {
        st = ssd_fwd_noalloc(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, NULL);
        if (ws_bytes <= SSD_NOALLOC_WORKSPACE_BYTES)
            CHECK(st == SSD_OK, "noalloc: status %d", (int)st);
        else
            CHECK(st == SSD_ERR_WORKSPACE, "noalloc beyond its array: status %d", (int)st);
    }
    /* one byte too little workspace */
    if (ws_bytes) {
        st = ssd_fwd_ex(&s, c->io, x, dt, A, B, C, D, seq, c->Q, h0, y, fs, ws, ws_bytes - 1, &o, NULL);
        CHECK(st == SSD_ERR_WORKSPACE, "short workspace: status %d", (int)st);
    }
    free(x); free(y); free(B); free(C); free(dt); free(A); free(D); free(seq); free(h0); free(fs);
    free(ws);
}

static void run_bwd(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int io, int full) {
    ssd_shape_t s = {b, L, H, P, N, G};
    const size_t esz = io == SSD_BF16 ? 2 : 4;
    const size_t nx = (size_t)(b * L * H * P), nbc = (size_t)(b * L * G * N), nst = (size_t)(b * H * P * N);
    void *x = buf(nx * esz), *dy = buf(nx * esz), *B = buf(nbc * esz), *C = buf(nbc * esz);
    float *dt = buf((size_t)(b * L * H) * 4), *A = buf((size_t)H * 4), *D = full ? buf((size_t)H * 4) : NULL;
    int32_t *seq = full ? buf((size_t)(b * L) * 4) : NULL;
    float *h0 = full ? buf(nst * 4) : NULL, *dfinal = full ? buf(nst * 4) : NULL;
    float *dx = buf(nx * 4), *ddt = buf((size_t)(b * L * H) * 4), *dA = buf((size_t)H * 4);
    float *dB = buf(nbc * 4), *dC = buf(nbc * 4), *dD = full ? buf((size_t)H * 4) : NULL;
    float *dinit = full ? buf(nst * 4) : NULL;
    const size_t ws_bytes = ssd_bwd_workspace_bytes(&s, io);
    void *ws = buf(ws_bytes);
    ssd_status_t st = ssd_bwd(&s, io, x, dt, A, B, C, D, seq, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD,
                              dinit, ws, ws_bytes, NULL);
    CHECK(st == SSD_OK, "bwd b%lld L%lld H%lld P%lld N%lld: status %d", (long long)b, (long long)L,
          (long long)H, (long long)P, (long long)N, (int)st);
    st = ssd_bwd(&s, io, x, dt, A, B, C, D, seq, h0, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit, ws,
                 ws_bytes - 1, NULL);
    CHECK(st == SSD_ERR_WORKSPACE, "bwd short workspace: status %d", (int)st);
    free(x); free(dy); free(B); free(C); free(dt); free(A); free(D); free(seq); free(h0); free(dfinal);
    free(dx); free(ddt); free(dA); free(dB); free(dC); free(dD); free(dinit); free(ws);
}

static void run_decode(int64_t b, int64_t H, int64_t P, int64_t N, int64_t G, int io, int fused) {
    ssd_shape_t s = {b, 1, H, P, N, G};
    const size_t esz = io == SSD_BF16 ? 2 : 4;
    void *x = buf((size_t)(b * H * P) * esz), *y = buf((size_t)(b * H * P) * esz);
    void *B = buf((size_t)(b * G * N) * esz), *C = buf((size_t)(b * G * N) * esz);
    float *dt = buf((size_t)(b * H) * 4), *A = buf((size_t)H * 4), *D = buf((size_t)H * 4);
    float *state = buf((size_t)(b * H * P * N) * 4);
    ssd_fused_t f;
    memset(&f, 0, sizeof(f));
    if (fused) {
        f.dt_bias = buf((size_t)H * 4);
        f.z = buf((size_t)(b * H * P) * esz);
        f.dt_softplus = 1;
    }
    ssd_status_t st = ssd_decode_step_fused(&s, io, x, dt, A, B, C, D, state, y, fused ? &f : NULL, NULL);
    CHECK(st == SSD_OK, "decode: status %d", (int)st);
    s.seqlen = 2;
    st = ssd_decode_step(&s, io, x, dt, A, B, C, D, state, y, NULL);
    CHECK(st == SSD_ERR_SHAPE, "decode seqlen 2: status %d", (int)st);
    if (fused) {
        free((void *)f.dt_bias);
        free((void *)f.z);
    }
    free(x); free(y); free(B); free(C); free(dt); free(A); free(D); free(state);
}

static void run_errors(void) {
    ssd_shape_t s = {2, 1000, 8, 64, 128, 2};
    const uintptr_t F = 0x100000; /* never dereferenced: every call fails validation */
    void *P = (void *)F;
    CHECK(ssd_fwd(NULL, SSD_BF16, P, P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_NULL, "null shape");
    CHECK(ssd_fwd(&s, (ssd_dtype_t)7, P, P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_UNSUPPORTED, "io");
    CHECK(ssd_fwd(&s, SSD_BF16, P, P, P, P, P, NULL, NULL, 100, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_UNSUPPORTED, "chunk");
    CHECK(ssd_fwd(&s, SSD_BF16, NULL, P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_NULL, "x");
    CHECK(ssd_fwd(&s, SSD_BF16, (void *)(F + 2), P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_ALIGN, "align");
    CHECK(ssd_fwd(&s, SSD_BF16, P, P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL, 0, NULL) == SSD_ERR_WORKSPACE, "workspace");
    ssd_shape_t huge = {1 << 20, 1, 65536, 16, 16, 1};   /* 2^36 units: above the launch limit */
    CHECK(ssd_fwd_workspace_bytes(&huge, 64, SSD_BF16) == 0, "huge workspace query");
    CHECK(ssd_fwd(&huge, SSD_BF16, P, P, P, P, P, NULL, NULL, 64, NULL, P, NULL, P, 1 << 20, NULL) == SSD_ERR_UNSUPPORTED, "huge");
    ssd_shape_t bad = {2, 1000, 8, 48, 128, 2};
    CHECK(ssd_fwd_workspace_bytes(&bad, 256, SSD_BF16) == 0, "bad headdim query");
    uint32_t *cnt = buf(3 * 64 * 4);
    CHECK(ssd_debug_exp2_probe(0, 16, cnt, 64, NULL) == SSD_ERR_UNSUPPORTED, "probe positive range");
    CHECK(ssd_debug_exp2_probe(0xFF800000u, 2, cnt, 64, NULL) == SSD_ERR_UNSUPPORTED, "probe beyond -inf");
    CHECK(ssd_debug_exp2_probe(0x80000000u, 1000, NULL, 64, NULL) == SSD_ERR_NULL, "probe null");
    CHECK(ssd_debug_exp2_probe(0x80000000u, 1000, cnt, 0, NULL) == SSD_ERR_UNSUPPORTED, "probe threads");
    CHECK(ssd_debug_exp2_probe(0x80000000u, 0x43200001u, cnt, 64, NULL) == SSD_OK, "probe");
    CHECK(ssd_segsum_record_words(256) == 4 * 256 + 32 + 8 && ssd_segsum_record_words(100) == 0, "record words");
    CHECK(ssd_debug_segsum_factors(&s, P, P, NULL, 256, NULL, NULL) == SSD_ERR_NULL, "factors null");
    CHECK(ssd_debug_fwd_segsum_factors(&s, SSD_F32, P, P, P, P, P, NULL, NULL, 256, NULL, P, NULL, NULL,
                                       0, NULL, P, NULL) == SSD_ERR_UNSUPPORTED, "factors f32");
    free(cnt);
}

int main(void) {
    const fwd_case cases[] = {
        /* b  L     H    P   N    G  Q    io        D  seq h0 fs split pb fused */
        {8, 2048, 80, 64, 128, 1, 256, SSD_BF16, 1, 0, 0, 1, 0, 0, 0},     /* the 2.7B layer */
        {2, 600, 144, 64, 128, 2, 256, SSD_BF16, 1, 0, 0, 1, 0, 0, 0},     /* half-headdim tail units */
        {2, 600, 144, 64, 128, 2, 256, SSD_BF16, 1, 0, 1, 1, 256, 0, 0},  /* and three splits */
        {1, 20000, 16, 64, 64, 1, 256, SSD_BF16, 1, 0, 0, 1, 0, 0, 0},    /* planner splits */
        {1, 5000, 32, 128, 64, 8, 128, SSD_BF16, 1, 1, 1, 1, 0, 0, 0},    /* packed, groups */
        {2, 333, 4, 32, 16, 2, 64, SSD_BF16, 0, 1, 0, 0, 128, 16, 1},     /* fused, forced blocks */
        {2, 515, 3, 128, 32, 1, 128, SSD_BF16, 1, 0, 1, 1, 0, 64, 0},
        {1, 256, 2, 16, 16, 1, 64, SSD_F32, 1, 0, 0, 1, 0, 0, 0},          /* fp32 */
        {2, 700, 4, 64, 64, 2, 128, SSD_F32, 1, 1, 1, 1, 256, 0, 1},
        {1, 1, 1, 16, 16, 1, 64, SSD_BF16, 0, 0, 0, 0, 0, 0, 0},           /* one token */
        {1, 32768, 32, 128, 64, 8, 128, SSD_BF16, 1, 1, 0, 1, 0, 0, 0},   /* beyond the noalloc array */
    };
    for (size_t k = 0; k < sizeof(cases) / sizeof(cases[0]); ++k) run_fwd(&cases[k]);
    run_bwd(1, 300, 4, 64, 64, 2, SSD_BF16, 1);
    run_bwd(2, 130, 2, 128, 32, 1, SSD_F32, 0);
    run_bwd(1, 300, 272, 16, 16, 1, SSD_BF16, 1);   /* 272 walks: the last 16 split in two */
    run_decode(4, 8, 64, 128, 2, SSD_BF16, 0);
    run_decode(2, 4, 32, 16, 1, SSD_F32, 1);
    run_errors();
    CHECK(stub_launches() > 80, "only %llu launches reached the stubs", (unsigned long long)stub_launches());
    if (g_fail) return 1;
    printf("abi driver: all checks passed (%llu launches)\n", (unsigned long long)stub_launches());
    return 0;
}
