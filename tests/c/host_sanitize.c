/* Host-side work of liblora_mi355x under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitize_cpu.py): every call
 * here runs on the CPU only -- segment building, workspace and size queries,
 * the page-frame allocator, the residency cache in its placement-only mode and
 * the argument checks of the GPU calls, which return before any GPU work.
 * Exits 0 when every check holds; a sanitizer report aborts the process. */
#define _POSIX_C_SOURCE 200112L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lora_mi355x.h"

static int failures;
#define CHECK(c)                                                                   \
    do {                                                                           \
        if (!(c)) {                                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);        \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static uint32_t rng_state = 12345u;
static uint32_t rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return rng_state >> 8;
}

static void segments_cases(void)
{
    enum { N = 40, CAP = 600 };
    uint64_t A[N], B[N];
    int32_t rank[N];
    float alpha[N];
    for (int i = 0; i < N; ++i) {
        A[i] = 0x100000000ull + 4096ull * (uint64_t)i;
        B[i] = 0x200000000ull + 4096ull * (uint64_t)i;
        rank[i] = 1 + (int32_t)(rnd() % 256);
        alpha[i] = (float)(1 + rnd() % 64);
    }
    const size_t bytes = lora_segments_bytes(CAP);
    CHECK(bytes > 0);
    void *buf = NULL;
    CHECK(posix_memalign(&buf, 64, bytes) == 0);
    lora_segments seg;
    CHECK(lora_segments_bind(buf, CAP, &seg) == LORA_OK);
    int32_t ids[CAP];
    const int32_t sizes[] = {0, 1, 2, 17, 255, 256, 257, 599, 600};
    for (size_t c = 0; c < sizeof sizes / sizeof sizes[0]; ++c) {
        const int32_t T = sizes[c];
        for (int32_t t = 0; t < T; ++t) ids[t] = (int32_t)(rnd() % (N + 1)) - 1;
        CHECK(lora_build_segments(T, ids, N, A, B, rank, alpha, &seg) == LORA_OK);
        int32_t adapted = 0;
        for (int32_t t = 0; t < T; ++t) adapted += ids[t] >= 0;
        CHECK(seg.num_tokens == adapted);
        CHECK(seg.batch_tokens == T);
        /* segments: contiguous, ascending adapter, tokens in order within one */
        for (int32_t s = 0; s < seg.num_segments; ++s) {
            CHECK(seg.seg_indptr[s] < seg.seg_indptr[s + 1]);
            if (s) CHECK(seg.seg_adapter[s - 1] < seg.seg_adapter[s]);
            const int32_t a = seg.seg_adapter[s];
            CHECK(seg.seg_rank[s] == rank[a]);
            CHECK(seg.seg_A[s] == A[a] && seg.seg_B[s] == B[a]);
            for (int32_t p = seg.seg_indptr[s]; p < seg.seg_indptr[s + 1]; ++p) {
                CHECK(ids[seg.perm[p]] == a);
                if (p > seg.seg_indptr[s]) CHECK(seg.perm[p - 1] < seg.perm[p]);
            }
        }
        if (seg.num_segments) CHECK(seg.seg_indptr[seg.num_segments] == adapted);
    }
    /* errors: id out of range, rank out of range, batch over capacity */
    ids[0] = N;
    CHECK(lora_build_segments(1, ids, N, A, B, rank, alpha, &seg) == LORA_ERR_ADAPTER_ID);
    ids[0] = 3;
    const int32_t keep = rank[3];
    rank[3] = 0;
    CHECK(lora_build_segments(1, ids, N, A, B, rank, alpha, &seg) == LORA_ERR_RANK);
    rank[3] = keep;
    CHECK(lora_build_segments(CAP + 1, ids, N, A, B, rank, alpha, &seg) != LORA_OK);
    CHECK(lora_build_segments(1, NULL, N, A, B, rank, alpha, &seg) == LORA_ERR_ARG);
    CHECK(lora_segments_bind((char *)buf + 4, CAP, &seg) == LORA_ERR_ALIGN);
    CHECK(strlen(lora_last_error()) > 0);
    free(buf);
}

static void pages_cases(void)
{
    CHECK(lora_pages_needed(0, 4096) == 0);
    CHECK(lora_pages_needed(4097, 4096) == 2);
    CHECK(lora_pages_needed(10, 100) == -1);
    lora_page_alloc *al = NULL;
    CHECK(lora_page_alloc_create(64, &al) == LORA_OK);
    int32_t got[64], back[64];
    int32_t held = 0;
    for (int round = 0; round < 200; ++round) {
        const int32_t want = (int32_t)(rnd() % 20);
        if (rnd() & 1) {
            const int st = lora_page_alloc_take(al, want, got);
            if (held + want <= 64) {
                CHECK(st == LORA_OK);
                for (int32_t i = 0; i < want; ++i) back[held + i] = got[i];
                held += want;
            } else {
                CHECK(st == LORA_ERR_WORKSPACE);
            }
        } else {
            const int32_t n = want < held ? want : held;
            CHECK(lora_page_alloc_give(al, back + held - n, n) == LORA_OK);
            held -= n;
        }
        CHECK(lora_page_alloc_free_count(al) == 64 - held);
    }
    if (held) CHECK(lora_page_alloc_give(al, back, 1) == LORA_OK);
    if (held) CHECK(lora_page_alloc_give(al, back, 1) == LORA_ERR_ARG); /* given twice */
    lora_page_alloc_destroy(al);
    CHECK(lora_page_alloc_free_count(NULL) == -1);
}

static void cache_cases(void)
{
    enum { N = 24, D_IN = 512, D_OUT = 256 };
    const size_t tab = lora_cache_table_bytes(N);
    const size_t bytes = tab + 6 * 2 * (size_t)16 * (D_IN + D_OUT) * 2;
    /* placement-only mode: the address is never dereferenced */
    void *fake_dev = (void *)(uintptr_t)0x7f0000000000ull;
    lora_cache *c = NULL;
    CHECK(lora_cache_create(fake_dev, bytes, N, LORA_BF16, D_IN, D_OUT, LORA_CACHE_DRY, &c) == LORA_OK);
    static uint16_t host[8];
    for (int a = 0; a < N; ++a)
        CHECK(lora_cache_register(c, a, host, host, 1 + (int32_t)(rnd() % 32), 16.0f) == LORA_OK);
    CHECK(lora_cache_pin(c, 5, 1) == LORA_OK);
    int32_t ids[32];
    int ok = 0;
    for (int b = 0; b < 300; ++b) {
        const int32_t T = 1 + (int32_t)(rnd() % 32);
        for (int32_t t = 0; t < T; ++t) ids[t] = (int32_t)(rnd() % 4) == 0 ? -1 : (int32_t)(rnd() % N);
        const int st = lora_cache_prepare(c, ids, T, NULL, NULL);
        CHECK(st == LORA_OK || st == LORA_ERR_WORKSPACE);
        ok += st == LORA_OK;
        lora_cache_view v;
        CHECK(lora_cache_view_get(c, &v) == LORA_OK);
        if (st == LORA_OK)
            for (int32_t t = 0; t < T; ++t)
                if (ids[t] >= 0) CHECK(v.pool_A_host[ids[t]] != 0);
    }
    CHECK(ok > 0);
    lora_cache_stats s;
    CHECK(lora_cache_stats_get(c, &s) == LORA_OK);
    CHECK(s.batches == ok);
    ids[0] = N;
    CHECK(lora_cache_prepare(c, ids, 1, NULL, NULL) == LORA_ERR_ADAPTER_ID);
    lora_cache_destroy(c);
}

static void argument_cases(void)
{
    /* every one of these returns before any GPU work */
    CHECK(lora_sgmv(NULL, LORA_BF16, NULL, 0, 0, NULL, NULL, 0, 0, NULL, 0) == LORA_ERR_ARG);
    CHECK(lora_bgmv(NULL, 7, 4, NULL, 0, 0, NULL, NULL, NULL, NULL, NULL, 0, 16, NULL, 0, 0, NULL, 0) ==
          LORA_ERR_DTYPE);
    CHECK(lora_fused_linear_e4m3(NULL, NULL, 0, 16, NULL, 0.0f, 16, NULL, NULL, 0, NULL, 0) != LORA_OK);
    CHECK(lora_probe_empty(NULL, 0) == LORA_ERR_ARG);
    CHECK(lora_profile_launches(NULL, NULL, 0) == LORA_OK);
    CHECK(lora_workspace_bytes(99, 1, 1, 1, 1) == (size_t)-1);
    CHECK(lora_workspace_bytes(LORA_OP_FUSED, 1024, 4096, 12288, 16) > 0);
    CHECK(lora_adapter_numel(16, 4096, 4096) == 16 * 8192);
    CHECK(lora_adapter_numel(-1, 1, 1) == -1);
    for (int st = -12; st <= 1; ++st) CHECK(lora_status_string(st) != NULL);
    CHECK(strstr(lora_version(), "gfx950") != NULL);
}

int main(void)
{
    segments_cases();
    pages_cases();
    cache_cases();
    argument_cases();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("host_sanitize: ok\n");
    return 0;
}
