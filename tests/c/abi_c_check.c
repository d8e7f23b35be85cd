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

    /* plan of 6 tokens over 3 adapters: ids 2, 0, -1, 2, 0, 2 */
    const int32_t T = 6, N = 3;
    const int32_t ids[6] = {2, 0, -1, 2, 0, 2};
    uint64_t pool_A[3], pool_B[3];
    const int32_t rank[3] = {4, 8, 16};
    const float alpha[3] = {8.f, 8.f, 32.f};
    for (int i = 0; i < 3; ++i) {
        pool_A[i] = 0x7f0000000000ull + 0x10000ull * (uint64_t)i;
        pool_B[i] = 0x7f0000008000ull + 0x10000ull * (uint64_t)i;
    }
    const size_t bytes = lora_plan_bytes(T);
    uint64_t *plan = (uint64_t *)calloc((bytes + 7) / 8, 8);
    CHECK(plan != NULL);
    CHECK(lora_build_plan(T, ids, N, pool_A, pool_B, rank, alpha, plan, bytes) == LORA_OK);
    const lora_plan_header *h = (const lora_plan_header *)plan;
    CHECK(h->magic == LORA_PLAN_MAGIC);
    CHECK(h->num_tokens == 6 && h->num_sorted == 5 && h->num_segments == 2 && h->max_rank == 16);
    const lora_seg_desc *seg = (const lora_seg_desc *)((const char *)plan + h->seg_offset);
    const int32_t *perm = (const int32_t *)((const char *)plan + h->perm_offset);
    /* ascending adapter id, original order inside a segment, then the unadapted token */
    CHECK(seg[0].adapter == 0 && seg[0].start == 0 && seg[0].len == 2 && seg[0].scale == 8.f / 4.f);
    CHECK(seg[1].adapter == 2 && seg[1].start == 2 && seg[1].len == 3 && seg[1].scale == 32.f / 16.f);
    const int32_t want[6] = {1, 4, 0, 3, 5, 2};
    for (int i = 0; i < 6; ++i) CHECK(perm[i] == want[i]);

    /* host-side rejections */
    const int32_t bad[2] = {0, 3};
    CHECK(lora_build_plan(2, bad, N, pool_A, pool_B, rank, alpha, plan, bytes) == LORA_ERR_ADAPTER_ID);
    CHECK(lora_build_plan(T, ids, N, pool_A, pool_B, rank, alpha, plan, 16) == LORA_ERR_WORKSPACE);
    CHECK(lora_profile_launches(NULL, NULL, -1) == LORA_ERR_ARG);
    CHECK(lora_profile_launches(NULL, NULL, 0) == LORA_OK && lora_profile_launches_used() == 0);
    free(plan);
    printf("ok\n");
    return 0;
}
