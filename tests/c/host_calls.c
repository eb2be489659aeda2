/*
 * The host-side calls of abs.h used from plain C (no Python, no GPU): block
 * geometry, centroid offsets, selection capacity, workspace sizes, row
 * bytes, the launch plan, the debug-check switch, the block-size rule, and
 * the documented error statuses.  Device
 * pointers are placeholders; none of these calls dereferences them.
 * Prints one "name value..." line per result for the test to compare.
 */
#include <stdint.h>
#include <stdio.h>

#include "abs.h"

#define CHECK(call)                                                                       \
    do {                                                                                  \
        abs_status st_ = (call);                                                          \
        if (st_ != ABS_OK) {                                                              \
            printf("error %s %d %s\n", #call, (int)st_, abs_last_error());                \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

int main(void) {
    const int32_t seq_lens[3] = {300, 77, 1};
    const int32_t block_size[2] = {16, 64};
    void *fake = (void *)(uintptr_t)(1ull << 40);
    abs_paged_kv kv = {0};
    kv.num_seqs = 3;
    kv.num_q_heads = 8;
    kv.num_kv_heads = 2;
    kv.head_dim = 128;
    kv.page_size = 16;
    kv.max_pages_per_seq = 32;
    kv.num_pages = 64;
    kv.kv_dtype = ABS_BF16;
    kv.k_cache = kv.v_cache = fake;
    kv.page_table = (const int32_t *)fake;
    kv.seq_lens = (const int32_t *)fake;
    kv.seq_lens_host = seq_lens;
    abs_block_map map = {block_size, (const int32_t *)fake, (const int64_t *)fake};

    int64_t total = 0;
    CHECK(abs_total_blocks(&kv, &map, &total));
    printf("total_blocks %lld\n", (long long)total);

    int64_t off[7];
    CHECK(abs_centroid_offsets(&kv, &map, off));
    printf("offsets");
    for (int i = 0; i < 7; ++i) printf(" %lld", (long long)off[i]);
    printf("\n");
    CHECK(abs_centroid_offsets_capacity(&kv, &map, 512, off));
    printf("offsets_capacity");
    for (int i = 0; i < 7; ++i) printf(" %lld", (long long)off[i]);
    printf("\n");

    int32_t cap = 0;
    CHECK(abs_select_capacity(&kv, &map, 100, &cap));
    printf("select_capacity %d\n", cap);

    size_t ws[3];
    for (int op = 0; op < 3; ++op) CHECK(abs_workspace_bytes(&kv, &map, 100, (abs_op)op, &ws[op]));
    printf("workspace %zu %zu %zu\n", ws[0], ws[1], ws[2]);

    int64_t rb[5];
    for (int f = 0; f < 5; ++f) CHECK(abs_centroid_row_bytes(128, f, &rb[f]));
    printf("row_bytes %lld %lld %lld %lld %lld\n", (long long)rb[0], (long long)rb[1], (long long)rb[2],
           (long long)rb[3], (long long)rb[4]);

    abs_launch_plan plan;
    CHECK(abs_describe_launch(&kv, &map, 100, &plan));
    printf("plan %d %d %d %d %d %d %d %d\n", plan.splits, plan.pages_per_wg, plan.chunk, plan.pipelined, plan.fused,
           plan.score_workgroups, plan.max_blocks, plan.sel_cap);
    const int32_t was_on = abs_set_debug_checks(1);
    const int32_t now_on = abs_set_debug_checks(0);
    printf("debug_checks %d %d\n", was_on, now_on);

    const float recall[3 * 3] = {0.8f, 0.8f, 0.5f, 0.79f, 0.5f, 0.5f, 0.5f, 0.4f, 0.5f};
    int32_t map_out[3];
    CHECK(abs_assign_block_sizes(3, recall, 0.9375f, map_out));
    printf("assign %d %d %d\n", map_out[0], map_out[1], map_out[2]);

    /* documented errors: nothing written, a status and a message */
    kv.page_size = 8;
    printf("status_page_size %d\n", (int)abs_total_blocks(&kv, &map, &total));
    kv.page_size = 16;
    const int32_t bad_bs[2] = {16, 48};
    abs_block_map bad = {bad_bs, (const int32_t *)fake, (const int64_t *)fake};
    printf("status_block_size %d\n", (int)abs_total_blocks(&kv, &bad, &total));
    printf("status_capacity %d\n", (int)abs_centroid_offsets_capacity(&kv, &map, 100, off));
    printf("status_budget %d\n", (int)abs_select_capacity(&kv, &map, 0, &cap));
    printf("last_error_nonempty %d\n", abs_last_error()[0] != '\0');
    printf("status_str %s\n", abs_status_str(ABS_ERR_UNSUPPORTED));
    return 0;
}
