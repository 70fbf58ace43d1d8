/*
 * Host-side driver of libcnhwc's C ABI for the sanitizer build (AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host code; no kernel is launched).
 *
 * It runs the descriptor validation, the dispatcher, the chunk planner, the
 * workspace sizing, the override and the pointer / workspace / overlap checks
 * of the entry points over fixed and pseudo-random descriptors -- valid ones,
 * every refusal the validator has, extreme sizes near the 2^31 and int64
 * limits -- and checks the status codes and reason strings.  Every call of
 * cnhwc_fwd / cnhwc_dgrad / cnhwc_wgrad is built to be refused before any
 * launch (NULL, misaligned or overlapping pointers, a short workspace), so the
 * program needs no GPU.  Prints "ok <calls>" and exits 0, or the first failed
 * expectation and exits 1; the sanitizers abort on any finding.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/cnhwc.h"

static long g_calls;
static int g_fail;

#define EXPECT(cond, ...)                                                   \
    do {                                                                    \
        if (!(cond)) {                                                      \
            if (!g_fail) {                                                  \
                printf("FAIL line %d: ", __LINE__);                         \
                printf(__VA_ARGS__);                                        \
                printf(" (last error: %s)\n", cnhwc_last_error());          \
            }                                                               \
            g_fail = 1;                                                     \
        }                                                                   \
    } while (0)

static cnhwc_problem P(int64_t n, int64_t h, int64_t w, int64_t c, int64_t k, int64_t r, int64_t s,
                       int stride, int ph, int pw, int groups, int dtype) {
    cnhwc_problem p;
    memset(&p, 0, sizeof p);
    p.n = n; p.h = h; p.w = w; p.c = c; p.k = k; p.r = r; p.s = s;
    p.stride = stride; p.pad_h = ph; p.pad_w = pw; p.groups = groups; p.dtype = dtype;
    return p;
}

static uint64_t g_rng = 0x243f6a8885a308d3ull;
static uint32_t rnd(uint32_t m) {
    g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_rng >> 33) % m;
}

/* Every query call on one descriptor; returns 1 if the descriptor is valid. */
static int query(const cnhwc_problem* p) {
    int64_t ho = -1, wo = -1;
    int st = cnhwc_out_dims(p, &ho, &wo);
    g_calls++;
    if (st != CNHWC_OK) {
        EXPECT(st == CNHWC_INVALID_ARG, "out_dims status %d", st);
        EXPECT(cnhwc_last_error()[0] != '\0', "refusal without a reason");
        return 0;
    }
    EXPECT(ho >= 1 && wo >= 1, "out dims %lld x %lld", (long long)ho, (long long)wo);
    EXPECT(ho == (p->h + 2 * (int64_t)p->pad_h - p->r) / p->stride + 1, "ho");
    EXPECT(wo == (p->w + 2 * (int64_t)p->pad_w - p->s) / p->stride + 1, "wo");
    const int ops[3] = {CNHWC_OP_FWD, CNHWC_OP_DGRAD, CNHWC_OP_WGRAD};
    for (int i = 0; i < 3; ++i) {
        char name[256], tiny[5];
        int32_t var = -1;
        st = cnhwc_plan(p, ops[i], name, sizeof name, &var);
        g_calls++;
        if (st != CNHWC_OK) {
            EXPECT(st == CNHWC_UNSUPPORTED, "plan status %d", st);
            EXPECT(cnhwc_last_error()[0] != '\0', "plan refusal without a reason");
            continue;
        }
        EXPECT(strlen(name) > 0 && var > 0, "plan name/variant");
        st = cnhwc_plan(p, ops[i], tiny, sizeof tiny, NULL);
        g_calls++;
        EXPECT(st == CNHWC_OK && strlen(tiny) == sizeof tiny - 1 && strncmp(tiny, name, 4) == 0,
               "truncated name");
        st = cnhwc_plan(p, ops[i], tiny, 1, NULL);
        g_calls++;
        EXPECT(st == CNHWC_OK && tiny[0] == '\0', "cap 1 name");
        st = cnhwc_plan(p, ops[i], NULL, 0, NULL);
        g_calls++;
        EXPECT(st == CNHWC_OK, "plan with no outputs");
        size_t ws = 0;
        st = cnhwc_workspace_size(p, ops[i], &ws);
        g_calls++;
        if (st != CNHWC_OK) {
            EXPECT(st == CNHWC_UNSUPPORTED, "workspace status %d", st);
            continue;
        }
        int64_t counts[8], nch = -1;
        st = cnhwc_chunk_plan(p, ops[i], counts, 8, &nch);
        g_calls++;
        EXPECT(st == CNHWC_OK && nch >= 1, "chunk plan status %d", st);
        if (st == CNHWC_OK) {
            int64_t sum = 0, mx = 0, mn = INT64_MAX;
            for (int64_t j = 0; j < nch && j < 8; ++j) {
                sum += counts[j];
                if (counts[j] > mx) mx = counts[j];
                if (counts[j] < mn) mn = counts[j];
            }
            if (nch <= 8) EXPECT(sum == p->n && mx - mn <= 1, "chunk balance");
        }
        st = cnhwc_chunk_plan(p, ops[i], NULL, 0, &nch);
        g_calls++;
        EXPECT(st == CNHWC_OK, "chunk plan without counts");
        /* refused launches: NULL input, misaligned output, short workspace */
        int8_t dummy[64];
        void* al = (void*)(((uintptr_t)dummy + 15) & ~(uintptr_t)15);
        void* mis = (void*)((char*)al + 2);
        int (*entry)(const cnhwc_problem*, const void*, const void*, void*, void*, size_t, void*) =
            ops[i] == CNHWC_OP_FWD ? cnhwc_fwd : ops[i] == CNHWC_OP_DGRAD ? cnhwc_dgrad : cnhwc_wgrad;
        st = entry(p, NULL, al, al, NULL, 0, NULL);
        g_calls++;
        EXPECT(st == CNHWC_INVALID_ARG, "NULL input accepted (%d)", st);
        st = entry(p, (void*)0x100000, (void*)0x200000, mis, NULL, 0, NULL);
        g_calls++;
        EXPECT(st == CNHWC_MISALIGNED, "misaligned output accepted (%d)", st);
        if (ws > 0) {
            /* far-apart fake device addresses: only the workspace check can refuse */
            st = entry(p, (void*)0x100000000000ull, (void*)0x200000000000ull, (void*)0x300000000000ull,
                       (void*)0x400000000000ull, ws - 1, NULL);
            g_calls++;
            EXPECT(st == CNHWC_WORKSPACE_TOO_SMALL, "short workspace accepted (%d)", st);
        }
    }
    return 1;
}

int main(void) {
    /* the refusals, one field at a time */
    cnhwc_problem base = P(1, 6, 6, 8, 8, 3, 3, 1, 1, 1, 1, CNHWC_F16);
    cnhwc_problem bad[12];
    for (int i = 0; i < 12; ++i) bad[i] = base;
    bad[0].groups = 0; bad[1].groups = -4; bad[2].groups = 3; bad[3].stride = 0;
    bad[4].pad_h = -1; bad[5].pad_w = -2; bad[6].n = 0; bad[7].r = 9; bad[7].s = 9;
    bad[8].dtype = 7; bad[9].reserved = 1; bad[10].c = (int64_t)1 << 31; bad[11].k = -5;
    for (int i = 0; i < 12; ++i) EXPECT(query(&bad[i]) == 0, "refusal %d accepted", i);
    EXPECT(cnhwc_out_dims(NULL, NULL, NULL) == CNHWC_INVALID_ARG, "NULL descriptor");
    EXPECT(cnhwc_plan(&base, 3, NULL, 0, NULL) == CNHWC_INVALID_ARG, "bad op");

    /* the workload shapes */
    const cnhwc_problem wl[] = {
        P(1, 8, 8, 16, 16, 1, 1, 1, 0, 0, 1, CNHWC_F16),
        P(32, 56, 56, 64, 256, 1, 1, 1, 0, 0, 1, CNHWC_F16),
        P(32, 28, 28, 256, 256, 3, 3, 1, 1, 1, 1, CNHWC_F16),
        P(32, 56, 56, 256, 256, 3, 3, 2, 1, 1, 1, CNHWC_F16),
        P(8, 7, 7, 2048, 512, 3, 3, 1, 1, 1, 1, CNHWC_BF16),
        P(32, 28, 28, 256, 256, 3, 3, 1, 1, 1, 32, CNHWC_BF16),
        P(16, 56, 56, 384, 384, 3, 3, 1, 1, 1, 384, CNHWC_F16),
        P(16, 56, 56, 384, 384, 7, 7, 1, 3, 3, 384, CNHWC_F16),
        P(16, 56, 56, 384, 384, 7, 7, 2, 3, 3, 384, CNHWC_F16),
        P(8, 32, 32, 256, 256, 31, 31, 1, 15, 15, 256, CNHWC_F16),
        P(8, 32, 32, 256, 256, 51, 5, 1, 25, 2, 256, CNHWC_F16),
        P(8, 32, 32, 256, 256, 5, 51, 1, 2, 25, 256, CNHWC_F16),
        P(1024, 56, 56, 384, 384, 3, 3, 1, 1, 1, 384, CNHWC_F16),   /* chunked */
        P(3, 4096, 4096, 64, 64, 3, 3, 1, 1, 1, 1, CNHWC_F16),      /* one image near the limit */
        P(1, 65536, 65536, 8, 8, 1, 1, 1, 0, 0, 1, CNHWC_F16),      /* one image over it */
    };
    for (size_t i = 0; i < sizeof wl / sizeof wl[0]; ++i) EXPECT(query(&wl[i]) == 1, "workload %zu", i);

    /* overrides: every variant forced on a few shapes, bad values refused */
    cnhwc_override ov;
    memset(&ov, 0, sizeof ov);
    ov.cpl = 3;
    EXPECT(cnhwc_set_override(&ov) == CNHWC_INVALID_ARG, "cpl 3");
    ov.cpl = 0; ov.split_c = -1;
    EXPECT(cnhwc_set_override(&ov) == CNHWC_INVALID_ARG, "split -1");
    for (int v = 0; v <= 20; ++v) {
        for (int sc = 0; sc <= 4; sc += 2) {
            memset(&ov, 0, sizeof ov);
            ov.variant = v; ov.split_c = sc; ov.tune = v % 3; ov.chunk_limit_bytes = v % 2 ? 4096 : 0;
            EXPECT(cnhwc_set_override(&ov) == CNHWC_OK, "override %d", v);
            for (size_t i = 0; i < 6; ++i) query(&wl[i]);
            query(&base);
        }
    }
    EXPECT(cnhwc_set_override(NULL) == CNHWC_OK, "clear override");

    /* pseudo-random descriptors, valid and invalid */
    for (int i = 0; i < 20000; ++i) {
        const int g = 1 + (int)rnd(4) * (rnd(3) == 0 ? 8 : 1);
        const int64_t c = (int64_t)g * (1 + rnd(24)), k = (int64_t)g * (1 + rnd(24));
        cnhwc_problem p = P(1 + rnd(5), 1 + rnd(40), 1 + rnd(40), c, k, 1 + rnd(9), 1 + rnd(9),
                            1 + (int)rnd(6), (int)rnd(6) - (rnd(50) == 0), (int)rnd(6), g,
                            rnd(40) == 0 ? 2 : (int)rnd(2));
        if (rnd(10) == 0) { p.groups = (int)p.c; p.k = p.c; }   /* depthwise */
        query(&p);
    }
    if (g_fail) return 1;
    printf("ok %ld\n", g_calls);
    return 0;
}
