/*
 * c_consumer.c -- a plain C99 program that uses libzero_partition.so through
 * include/zero_partition.h alone (no C++, no HIP headers, no device work).
 *
 * It checks that the header is valid C and that the structs a C compiler lays
 * out have the sizes the library was built with, then builds the partition
 * layout of the tensor sizes given on the command line and prints it, one
 * record per line, for the test that compares it with the oracle:
 *
 *   usage: c_consumer N STAGE ALIGN BUCKET numel...
 *   output:
 *     sizes OK
 *     info psi S padded padding n_fills n_segments b16 g16 master mom var total
 *     offset i flat_off                       (one per tensor)
 *     rank r begin real_end end n_segments    (one per rank)
 *     seg tensor owner tensor_off flat_off len shard_off fill bucket_off
 *     arena total k offset bytes ...          (ping-pong, 2 contributions)
 *     error <status> <message>                (bad-argument calls)
 * Exit status 0 when every call behaved as the header states.
 */
#include <stdio.h>
#include <stdlib.h>

#include "zero_partition.h"

static int check_sizes(void)
{
    const struct { int which; long long size; const char* name; } s[] = {
        {0, (long long)sizeof(zero_layout_info), "zero_layout_info"},
        {1, (long long)sizeof(zero_segment), "zero_segment"},
        {2, (long long)sizeof(zero_shard_state), "zero_shard_state"},
        {3, (long long)sizeof(zero_adam_hparams), "zero_adam_hparams"},
        {4, (long long)sizeof(zero_loss_scaler), "zero_loss_scaler"},
        {5, (long long)sizeof(zero_arena_plan), "zero_arena_plan"},
    };
    size_t i;
    for (i = 0; i < sizeof(s) / sizeof(s[0]); ++i) {
        const long long lib = (long long)zero_abi_struct_size(s[i].which);
        if (lib != s[i].size) {
            printf("size mismatch %s: C %lld, library %lld\n", s[i].name, s[i].size, lib);
            return 1;
        }
    }
    printf("sizes OK\n");
    return 0;
}

static int expect_error(int rc, int want, const char* what)
{
    printf("error %d %s\n", rc, zero_last_error());
    if (rc != want) {
        printf("%s: got %d, expected %d\n", what, rc, want);
        return 1;
    }
    return 0;
}

int main(int argc, char** argv)
{
    int32_t n_ranks, stage;
    int64_t align, bucket, n_tensors, i, n_seg = 0, need = 0;
    int64_t* numel;
    int64_t* offs;
    zero_layout* lay = NULL;
    zero_layout_info info;
    zero_segment* segs;
    zero_arena_plan plan;
    int rc, r, bad = 0;

    if (argc < 5) {
        fprintf(stderr, "usage: %s N STAGE ALIGN BUCKET numel...\n", argv[0]);
        return 2;
    }
    if (zero_version() != ZERO_PARTITION_VERSION) {
        printf("version mismatch: header %d, library %d\n", ZERO_PARTITION_VERSION, zero_version());
        return 1;
    }
    if (check_sizes()) return 1;

    n_ranks = (int32_t)atoi(argv[1]);
    stage = (int32_t)atoi(argv[2]);
    align = (int64_t)atoll(argv[3]);
    bucket = (int64_t)atoll(argv[4]);
    n_tensors = argc - 5;
    numel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_tensors + 1));
    offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_tensors + 1));
    if (!numel || !offs) return 2;
    for (i = 0; i < n_tensors; ++i) numel[i] = (int64_t)atoll(argv[5 + i]);

    rc = zero_partition_layout(numel, n_tensors, n_ranks, stage, align, bucket, &lay);
    if (rc != ZERO_OK) {
        printf("layout failed: %d %s\n", rc, zero_last_error());
        return 1;
    }
    if (zero_layout_get_info(lay, &info) != ZERO_OK) return 1;
    printf("info %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld\n",
           (long long)info.psi, (long long)info.shard_elems, (long long)info.padded_elems,
           (long long)info.padding, (long long)info.n_fills, (long long)info.n_segments,
           (long long)info.bytes_param16, (long long)info.bytes_grad16,
           (long long)info.bytes_master, (long long)info.bytes_momentum,
           (long long)info.bytes_variance, (long long)info.bytes_total);

    if (zero_layout_tensor_offsets(lay, offs, n_tensors) != ZERO_OK) return 1;
    for (i = 0; i < n_tensors; ++i) printf("offset %lld %lld\n", (long long)i, (long long)offs[i]);

    for (r = 0; r < n_ranks; ++r) {
        int64_t b, re, e, nr = 0;
        if (zero_layout_rank_range(lay, r, &b, &re, &e) != ZERO_OK) return 1;
        /* sizing call: cap 0 reports the count */
        rc = zero_layout_rank_segments(lay, r, NULL, 0, &nr);
        if (rc != ZERO_OK && rc != ZERO_ERR_CAPACITY) return 1;
        printf("rank %d %lld %lld %lld %lld\n", r, (long long)b, (long long)re, (long long)e,
               (long long)nr);
    }

    /* all segments: size, then fetch */
    rc = zero_layout_segments(lay, NULL, 0, &need);
    if (rc != ZERO_OK && rc != ZERO_ERR_CAPACITY) return 1;
    segs = (zero_segment*)malloc(sizeof(zero_segment) * (size_t)(need + 1));
    if (!segs) return 2;
    if (need > 0) bad |= expect_error(zero_layout_segments(lay, segs, need - 1, &n_seg),
                                      ZERO_ERR_CAPACITY, "segments with a short array");
    if (zero_layout_segments(lay, segs, need, &n_seg) != ZERO_OK || n_seg != need) return 1;
    for (i = 0; i < n_seg; ++i)
        printf("seg %d %d %lld %lld %lld %lld %lld %lld\n", segs[i].tensor, segs[i].owner,
               (long long)segs[i].tensor_off, (long long)segs[i].flat_off, (long long)segs[i].len,
               (long long)segs[i].shard_off, (long long)segs[i].fill, (long long)segs[i].bucket_off);

    if (zero_arena_plan_for(lay, 1, 2, bucket > 0, 0, &plan) != ZERO_OK) return 1;
    printf("arena %lld", (long long)plan.total_bytes);
    for (r = 0; r < ZERO_ARENA_KINDS; ++r)
        if (plan.offset[r] >= 0) printf(" %d %lld %lld", r, (long long)plan.offset[r], (long long)plan.bytes[r]);
    printf("\n");

    /* argument errors leave the output untouched and set the message */
    {
        zero_layout* none = NULL;
        int64_t bad_numel[2] = {5, -1};
        bad |= expect_error(zero_partition_layout(bad_numel, 2, 2, 0, 1, 0, &none),
                            ZERO_ERR_INVALID_ARG, "negative size");
        bad |= expect_error(zero_partition_layout(numel, n_tensors, 0, 0, 1, 0, &none),
                            ZERO_ERR_INVALID_ARG, "zero ranks");
        bad |= expect_error(zero_layout_rank_range(lay, n_ranks, &need, &need, &need),
                            ZERO_ERR_INVALID_ARG, "rank out of range");
        if (none != NULL) {
            printf("a failed call wrote a handle\n");
            bad = 1;
        }
    }

    zero_layout_destroy(lay);
    zero_layout_destroy(NULL);
    free(segs);
    free(offs);
    free(numel);
    return bad;
}
