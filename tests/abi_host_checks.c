/*
 * abi_host_checks.c -- the host side of the C ABI (include/kve.h) driven
 * from C, for a build of the library whose host code carries AddressSanitizer
 * and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  No GPU is used:
 * every call either fails a host-side check (KVE_EINVAL, counters untouched),
 * is pure host arithmetic (pyramid_budgets, kve_kept_indices, the byte
 * helpers, kve_workspace_size, kve_strerror), or passes every check and then
 * finds no device (KVE_ENODEV, or KVE_ELAUNCH without code for one).
 * Prints "ok: <n> checks" and exits 0, or names the first failed check.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kve.h"

static int checks = 0;

#define CHECK(cond)                                                        \
    do {                                                                   \
        ++checks;                                                          \
        if (!(cond)) {                                                     \
            printf("FAIL line %d: %s\n", __LINE__, #cond);                 \
            exit(1);                                                       \
        }                                                                  \
    } while (0)

#define FAKE ((void *)(uintptr_t)0x10000)  /* aligned, never dereferenced */

static kve_layer layer(void)
{
    kve_layer L;
    memset(&L, 0, sizeof L);
    L.k = FAKE; L.v = FAKE; L.scores = (float *)FAKE; L.gumbel = (float *)FAKE;
    L.positions = (int32_t *)FAKE;
    L.bh = 8; L.cap = 33; L.d = 64; L.hh_base = 0;
    return L;
}

static int same(const kve_counters *c, int32_t n, int32_t np, int32_t p)
{
    return c->n_kept == n && c->next_pos == np && c->pos == p;
}

static int not_ran(int rc) { return rc == KVE_ENODEV || rc == KVE_ELAUNCH; }

static void keyformer_rejects(void)
{
    struct { const char *name; int field; intptr_t value; } cases[] = {
        {"null k", 0, 0}, {"null scores", 1, 0}, {"null positions", 2, 0},
        {"null gumbel", 3, 0}, {"misaligned k", 4, 2}, {"d 96", 5, 96},
        {"bh 0", 6, 0}, {"cap 32", 7, 32}, {"negative hh_base", 8, -1},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
        kve_layer L = layer();
        switch (cases[i].field) {
            case 0: L.k = NULL; break;
            case 1: L.scores = NULL; break;
            case 2: L.positions = NULL; break;
            case 3: L.gumbel = NULL; break;
            case 4: L.k = (char *)FAKE + cases[i].value; break;
            case 5: L.d = (int32_t)cases[i].value; break;
            case 6: L.bh = 0; break;
            case 7: L.cap = 32; break;
            case 8: L.hh_base = -1; break;
        }
        kve_counters c = {32, 100, 100};
        CHECK(keyformer_step(&L, FAKE, FAKE, &c, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) ==
              KVE_EINVAL);
        CHECK(same(&c, 32, 100, 100));
    }
    kve_layer L = layer();
    kve_counters c = {32, 100, 100};
    /* argument guards of init_keyformer_state and the layout */
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 4, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 32, -1, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 32, 4, -0.1, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 32, 4, 1.0, 2.0, -1, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 32, 4, 1.0, 2.0, 64, 0.0, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, NULL, FAKE, &c, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, (char *)FAKE + 8, &c, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                         NULL) == KVE_EINVAL);
    CHECK(keyformer_step(NULL, FAKE, FAKE, &c, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step(&L, FAKE, FAKE, NULL, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(same(&c, 32, 100, 100));
    kve_counters bad[] = {{33, 40, 40}, {-1, 0, 0}, {10, 50, 50}, {32, 10, 10}};
    for (size_t i = 0; i < 4; ++i) {
        kve_counters b = bad[i];
        CHECK(keyformer_step(&L, FAKE, FAKE, &b, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) ==
              KVE_EINVAL);
        CHECK(memcmp(&b, &bad[i], sizeof b) == 0);
    }
    L.cap = 12290;
    CHECK(keyformer_step(&L, FAKE, FAKE, &c, 12289, 4, 1.0, 2.0, 64, 1e4, 0, NULL, NULL) ==
          KVE_EINVAL);
    /* every host check passed: the call reaches the launch and finds no device */
    L = layer();
    L.gumbel = NULL;
    CHECK(not_ran(pyramid_step(&L, FAKE, FAKE, &c, 32, 4, 1e4, NULL, NULL)));
    CHECK(same(&c, 32, 100, 100));
    c.n_kept = 0; c.next_pos = 0; c.pos = 0;      /* under budget: no rotation tables */
    CHECK(not_ran(pyramid_step(&L, FAKE, FAKE, &c, 32, 4, 1e4, NULL, NULL)));
}

static void batched_rejects(void)
{
    const size_t layer_bytes = 8 * 33 * 64 * 2;
    kve_layer Ls[129];
    kve_counters cs[129];
    int32_t budgets[129];
    const void *ptrs[129];
    for (int i = 0; i < 129; ++i) {
        Ls[i] = layer();
        Ls[i].k = (char *)FAKE + (size_t)i * layer_bytes;
        cs[i].n_kept = 32; cs[i].next_pos = 100; cs[i].pos = 100;
        budgets[i] = 32;
        ptrs[i] = FAKE;
    }
    CHECK(keyformer_step_layers(0, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);
    CHECK(keyformer_step_layers(129, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);
    /* overlapping layers (the overlap check sorts the key buffers) */
    kve_layer saved = Ls[1];
    Ls[1].k = (char *)FAKE + layer_bytes - 256;
    CHECK(keyformer_step_layers(3, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);
    Ls[1] = Ls[0];
    CHECK(keyformer_step_layers(3, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);
    Ls[1] = saved;
    Ls[2].d = 128;
    CHECK(pyramid_step_layers(3, Ls, ptrs, ptrs, cs, budgets, 4, 1e4, NULL, NULL) == KVE_EINVAL);
    Ls[2].d = 64;
    cs[1].n_kept = 10; cs[1].next_pos = 50; cs[1].pos = 50;
    CHECK(keyformer_step_layers_tokens(3, 4, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4,
                                       0, NULL, NULL) == KVE_EINVAL);
    CHECK(cs[0].n_kept == 32 && cs[2].n_kept == 32 && cs[1].n_kept == 10);
    cs[1].n_kept = 32; cs[1].next_pos = 100; cs[1].pos = 100;
    CHECK(keyformer_step_layers_tokens(3, 129, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4,
                                       0, NULL, NULL) == KVE_EINVAL);
    CHECK(keyformer_step_tokens(NULL, 4, FAKE, FAKE, cs, 32, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);
    /* 40 layers: two launch groups, every layer checked first */
    for (int i = 0; i < 40; ++i) Ls[i].gumbel = NULL;
    CHECK(not_ran(pyramid_step_layers(40, Ls, ptrs, ptrs, cs, budgets, 4, 1e4, NULL, NULL)));
    for (int i = 0; i < 40; ++i) CHECK(cs[i].n_kept == 32 && cs[i].pos == 100);
    CHECK(keyformer_step_layers(40, Ls, ptrs, ptrs, cs, budgets, 4, 1.0, 2.0, 64, 1e4, 0, NULL,
                                NULL) == KVE_EINVAL);        /* no gumbel tensors */
}

static void policy_and_workspace(void)
{
    kve_layer Ls[2] = {layer(), layer()};
    Ls[1].k = (char *)FAKE + (1 << 20);
    kve_counters cs[2] = {{32, 100, 100}, {32, 100, 100}};
    int32_t budgets[2] = {32, 32};
    const void *ptrs[2] = {FAKE, FAKE};
    kve_policy p;
    memset(&p, 0, sizeof p);
    p.n_sink = 4; p.recent = 3; p.score = KVE_SCORE_CUMULATIVE; p.gumbel = 1;
    p.tau_init = 1.0; p.tau_end = 2.0; p.anneal_steps = 64; p.rope_base = 1e4; p.seed = 7;
    CHECK(kve_step(1, 1, Ls, ptrs, ptrs, cs, budgets, NULL, NULL, NULL) == KVE_EINVAL);
    p.score = 2;
    CHECK(kve_step(1, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_EINVAL);
    p.score = KVE_SCORE_CURRENT;
    p.gumbel = 2;
    CHECK(kve_step(1, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_EINVAL);
    p.gumbel = 0;
    p.recent = 28;                                      /* 4 + 28 == 32: no room */
    CHECK(kve_step(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_EINVAL);
    p.recent = 27;
    Ls[0].gumbel = NULL; Ls[1].gumbel = NULL;
    CHECK(not_ran(kve_step(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL)));
    CHECK(cs[0].n_kept == 32 && cs[1].pos == 100);

    /* the workspace form: alignment and size are checked before anything else */
    CHECK(kve_step_ws(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, (char *)FAKE + 16, 1 << 20,
                      NULL) == KVE_EINVAL);
    CHECK(kve_step_ws(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, FAKE, 767, NULL) ==
          KVE_EINVAL);                                  /* one item at d = 64 needs 768 */
    CHECK(kve_step_ws(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL, 4096, NULL) ==
          KVE_EINVAL);
    CHECK(kve_step_ws(2, 1, NULL, ptrs, ptrs, cs, budgets, &p, NULL, FAKE, 4096, NULL) ==
          KVE_EINVAL);
    CHECK(not_ran(kve_step_ws(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, FAKE, 768, NULL)));
    CHECK(not_ran(kve_step_ws(2, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL, 0, NULL)));
    CHECK(cs[0].n_kept == 32 && cs[1].pos == 100);
    CHECK(kve_workspace_size(256, 1024, 128) == 256 + 4096 * 32 + 4096 * 512);
    CHECK(kve_workspace_size(1, 2, 64) == 768);
    CHECK(kve_workspace_size(0, 1024, 128) == -1);
    CHECK(kve_workspace_size(256, 12289, 128) == -1);
    CHECK(kve_workspace_size(256, 1024, 96) == -1);
    CHECK(kve_workspace_size((int64_t)1 << 31, 1024, 128) == -1);
}

static void noalloc(void)
{
    /* 32 layers x 256 caches at budget 1024 would need 68 MiB of scratch */
    static kve_layer Ls[32];
    kve_counters cs[32];
    int32_t budgets[32];
    const void *ptrs[32];
    for (int i = 0; i < 32; ++i) {
        Ls[i] = layer();
        Ls[i].bh = 256; Ls[i].cap = 1025; Ls[i].d = 128;
        Ls[i].k = (char *)FAKE + (size_t)i * ((size_t)1 << 30);
        cs[i].n_kept = 1024; cs[i].next_pos = 5000; cs[i].pos = 5000;
        budgets[i] = 1024;
        ptrs[i] = FAKE;
    }
    kve_policy p;
    memset(&p, 0, sizeof p);
    p.n_sink = 4; p.score = KVE_SCORE_CUMULATIVE; p.gumbel = 1;
    p.tau_init = 1.0; p.tau_end = 2.0; p.anneal_steps = 512; p.rope_base = 1e4;
    CHECK(kve_workspace_size(32 * 256, 1024, 128) > KVE_NOALLOC_SCRATCH_BYTES);
    CHECK(kve_step_noalloc(32, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_ENOSPACE);
    CHECK(cs[0].n_kept == 1024 && cs[31].pos == 5000);
    /* one layer fits; arguments are checked before any device call */
    CHECK(not_ran(kve_step_noalloc(1, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL)));
    Ls[0].cap = 1000;
    CHECK(kve_step_noalloc(1, 1, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_EINVAL);
    Ls[0].cap = 1025;
    CHECK(kve_step_noalloc(1, 1, NULL, ptrs, ptrs, cs, budgets, &p, NULL, NULL) == KVE_EINVAL);
    CHECK(kve_step_noalloc(1, 1, Ls, ptrs, ptrs, cs, budgets, NULL, NULL, NULL) == KVE_EINVAL);
    /* several tokens hand nothing over: no scratch needed */
    CHECK(not_ran(kve_step_noalloc(32, 4, Ls, ptrs, ptrs, cs, budgets, &p, NULL, NULL)));
    CHECK(cs[0].n_kept == 1024 && cs[31].pos == 5000);
    CHECK(strstr(kve_strerror(KVE_ENOSPACE), "fixed") != NULL);
}

static void host_helpers(void)
{
    static const int32_t page[12] = {1019, 927, 835, 742, 650, 558, 466, 374, 282, 189, 97, 5};
    int32_t out[64];
    CHECK(pyramid_budgets(12, 512, 4, 2.0, out) == KVE_OK);
    CHECK(memcmp(out, page, sizeof page) == 0);
    CHECK(pyramid_budgets(32, 4096, 4, 1.5, out) == KVE_OK && out[0] == 6144 && out[31] == 2048);
    CHECK(pyramid_budgets(12, 512, 4, 0.5, out) == KVE_EINVAL);
    CHECK(pyramid_budgets(-1, 512, 4, 2.0, out) == KVE_EINVAL);
    CHECK(pyramid_budgets(12, 4, 4, 2.0, out) == KVE_EINVAL);
    CHECK(pyramid_budgets(3, 512, 4, 2.0, NULL) == KVE_EINVAL);
    CHECK(pyramid_budgets(0, 512, 4, 2.0, NULL) == KVE_OK);
    CHECK(pyramid_budgets(1, 77, 4, 3.0, out) == KVE_OK && out[0] == 77);

    int32_t ev[3] = {-1, 4, 0}, kept[8];
    CHECK(kve_kept_indices(3, 3, ev, kept) == 4);
    CHECK(kept[0] == 1 && kept[1] == 2 && kept[2] == 3 && kept[3] == 5);
    int32_t bad_hi[1] = {3}, bad_lo[1] = {-2};
    CHECK(kve_kept_indices(2, 1, bad_hi, kept) == KVE_EINVAL);
    CHECK(kve_kept_indices(2, 1, bad_lo, kept) == KVE_EINVAL);
    CHECK(kve_kept_indices(0, 1, NULL, NULL) == KVE_EINVAL);
    CHECK(kve_kept_indices(-1, 0, NULL, NULL) == KVE_EINVAL);
    CHECK(kve_kept_indices(0, 0, NULL, NULL) == 0);

    CHECK(kve_fp16_bytes(9, 64) == 4 * 9 * 64);
    CHECK(kve_full_fp16_bytes(3072, 128) == 4 * 3072 * 128);
    CHECK(kve_fp16_bytes(-1, 64) == -1 && kve_fp16_bytes(1, 0) == -1);
    CHECK(kve_fp16_bytes(INT64_MAX / 2, 128) == -1);
    CHECK(strcmp(kve_strerror(KVE_OK), "ok") == 0);
    CHECK(strcmp(kve_strerror(12345), "unknown error") == 0);
}

int main(void)
{
    keyformer_rejects();
    batched_rejects();
    policy_and_workspace();
    noalloc();
    host_helpers();
    printf("ok: %d checks\n", checks);
    return 0;
}
