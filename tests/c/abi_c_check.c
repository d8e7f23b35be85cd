/* Compiled as C99 against the public header and linked with the library:
 * checks that the boundary is a plain C ABI and exercises the host-only
 * entry points (no GPU call).  Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lora_mi355x.h"

#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,  \
                    lora_last_error());                                          \
            return 1;                                                             \
        }                                                                         \
    } while (0)

int main(void)
{
    /* r (d_in + d_out): the pages' Q projection example, rank 16, 8192 -> 8192 */
    CHECK(lora_adapter_numel(16, 8192, 8192) == 262144);
    CHECK(lora_adapter_numel(-1, 1, 1) == -1);
    CHECK(strcmp(lora_status_string(LORA_OK), "LORA_OK") == 0);
    CHECK(lora_workspace_bytes(LORA_OP_SGMV_SHRINK, 8, 64, 64, 8) == 0);
    CHECK(lora_workspace_bytes(99, 8, 64, 64, 8) == (size_t)-1);

    /* segments of 6 tokens over 3 adapters: ids 2, 0, -1, 2, 0, 2 */
    const int32_t T = 6, N = 3;
    const int32_t ids[6] = {2, 0, -1, 2, 0, 2};
    uint64_t pool_A[3], pool_B[3];
    const int32_t rank[3] = {4, 8, 16};
    const float alpha[3] = {8.f, 8.f, 32.f};
    for (int i = 0; i < 3; ++i) {
        pool_A[i] = 0x7f0000000000ull + 0x10000ull * (uint64_t)i;
        pool_B[i] = 0x7f0000008000ull + 0x10000ull * (uint64_t)i;
    }
    const size_t bytes = lora_segments_bytes(T);
    uint64_t *buf = (uint64_t *)calloc((bytes + 15) / 8 + 2, 8);
    CHECK(buf != NULL);
    void *aligned = (void *)(((uintptr_t)buf + 15) & ~(uintptr_t)15);
    lora_segments sg;
    CHECK(lora_segments_bind(aligned, T, &sg) == LORA_OK);
    CHECK(lora_build_segments(T, ids, N, pool_A, pool_B, rank, alpha, &sg) == LORA_OK);
    /* ascending adapter id, original order inside a segment, then the unadapted token */
    CHECK(sg.num_segments == 2 && sg.num_tokens == 5 && sg.batch_tokens == 6 && sg.max_rank == 16);
    CHECK(sg.seg_indptr[0] == 0 && sg.seg_indptr[1] == 2 && sg.seg_indptr[2] == 5);
    CHECK(sg.seg_adapter[0] == 0 && sg.seg_adapter[1] == 2);
    CHECK(sg.seg_rank[0] == 4 && sg.seg_rank[1] == 16);
    CHECK(sg.seg_A[0] == pool_A[0] && sg.seg_A[1] == pool_A[2] && sg.seg_B[1] == pool_B[2]);
    CHECK(sg.seg_scale[0] == 8.f / 4.f && sg.seg_scale[1] == 32.f / 16.f);
    const int32_t want[6] = {1, 4, 0, 3, 5, 2};
    for (int i = 0; i < 6; ++i) CHECK(sg.perm[i] == want[i]);
    /* the same segments through the buffer's own layout */
    const lora_plan_header *h = (const lora_plan_header *)aligned;
    CHECK(h->magic == LORA_PLAN_MAGIC && h->num_sorted == 5 && h->num_segments == 2);
    const lora_seg_desc *seg = (const lora_seg_desc *)((const char *)aligned + h->seg_offset);
    CHECK(seg[1].adapter == 2 && seg[1].start == 2 && seg[1].len == 3);

    /* host-side rejections */
    const int32_t bad[2] = {0, 3};
    CHECK(lora_build_segments(2, bad, N, pool_A, pool_B, rank, alpha, &sg) == LORA_ERR_ADAPTER_ID);
    lora_segments small;
    CHECK(lora_segments_bind(aligned, 2, &small) == LORA_OK);
    CHECK(lora_build_segments(T, ids, N, pool_A, pool_B, rank, alpha, &small) == LORA_ERR_WORKSPACE);
    CHECK(lora_segments_bind((char *)aligned + 4, T, &small) == LORA_ERR_ALIGN);
    CHECK(lora_profile_launches(NULL, NULL, -1) == LORA_ERR_ARG);

    /* grouped BGMV: workspace is a 256-byte status block, then per projection
     * three times its 256-byte-rounded region of fp32 slice partial sums (4
     * slices of d_in, T rows of round4(rank), plus 256 B of slack): those sums,
     * then the one-launch form's 8-byte tagged words; malformed calls are
     * rejected on the host */
    lora_proj pr[2];
    memset(pr, 0, sizeof(pr));
    for (int p = 0; p < 2; ++p) {
        pr[p].x = (const void *)0x7f1000000000ull;
        pr[p].y = (void *)(0x7f2000000000ull + 0x100000ull * (uint64_t)p);
        pr[p].pool_A_dev = (const uint64_t *)0x7f3000000000ull;
        pr[p].pool_B_dev = (const uint64_t *)0x7f3000001000ull;
        pr[p].pool_rank_dev = (const int32_t *)0x7f3000002000ull;
        pr[p].pool_alpha_dev = (const float *)0x7f3000003000ull;
        pr[p].ldx = 4096;
        pr[p].ldy = 1024;
        pr[p].d_in = 4096;
        pr[p].d_out = 1024;
        pr[p].max_rank = p == 0 ? 16 : 64;
    }
    const size_t r0 = 4u * 64u * 16u * 4u + 256u;
    const size_t r1 = 4u * 64u * 64u * 4u + 256u;
    CHECK(lora_workspace_bytes(LORA_OP_BGMV, 64, 4096, 1024, 16) > r0);
    CHECK(lora_workspace_bytes(LORA_OP_SGMV, 64, 4096, 1024, 16) > r0);
    CHECK(lora_bgmv_grouped_workspace_bytes(64, pr, 2) == 256 + 3 * ((r0 + 255) / 256 * 256) + 3 * ((r1 + 255) / 256 * 256));
    CHECK(lora_bgmv_grouped_workspace_bytes(64, pr, 0) == 0);
    CHECK(lora_bgmv_grouped_workspace_bytes(64, pr, LORA_MAX_PROJ + 1) == 0);
    CHECK(lora_bgmv_grouped(NULL, LORA_BF16, 64, NULL, 4, pr, LORA_MAX_PROJ + 1, NULL, 0) == LORA_ERR_ARG);
    CHECK(lora_bgmv_grouped(NULL, 7, 64, NULL, 4, pr, 2, NULL, 0) == LORA_ERR_DTYPE);
    pr[1].max_rank = 300;
    CHECK(lora_bgmv_grouped(NULL, LORA_BF16, 64, NULL, 4, pr, 2, NULL, 0) == LORA_ERR_RANK);
    CHECK(lora_bgmv_grouped_workspace_bytes(64, pr, 2) == 0);
    pr[1].max_rank = 64;
    pr[1].y = pr[0].y;
    CHECK(lora_bgmv_grouped(NULL, LORA_BF16, 64, NULL, 4, pr, 2, NULL, 0) == LORA_ERR_ARG);
    pr[1].y = (void *)0x7f2000100000ull;
    CHECK(lora_bgmv_grouped(NULL, LORA_BF16, 64, (const int32_t *)0x7f4000000000ull, 4, pr, 2, NULL, 0) ==
          LORA_ERR_WORKSPACE);
    CHECK(lora_profile_launches(NULL, NULL, 0) == LORA_OK && lora_profile_launches_used() == 0);

    /* paged storage, host side: page counts and the frame allocator */
    CHECK(lora_pages_needed(16 * 4096 * 2, 16384) == 8);
    CHECK(lora_pages_needed(1, 48) == -1);
    lora_page_alloc *pa = NULL;
    CHECK(lora_page_alloc_create(6, &pa) == LORA_OK && lora_page_alloc_free_count(pa) == 6);
    int32_t fr[6];
    CHECK(lora_page_alloc_take(pa, 4, fr) == LORA_OK && fr[0] == 0 && fr[3] == 3);
    CHECK(lora_page_alloc_take(pa, 3, fr + 4) == LORA_ERR_WORKSPACE);
    CHECK(lora_page_alloc_give(pa, fr + 1, 2) == LORA_OK && lora_page_alloc_free_count(pa) == 4);
    CHECK(lora_page_alloc_give(pa, fr + 1, 1) == LORA_ERR_ARG);
    lora_page_alloc_destroy(pa);
    free(buf);
    printf("ok\n");
    return 0;
}
