/*
 * Host-side validation of every entry point, run under AddressSanitizer (tests/test_asan.py builds the
 * library with the host code instrumented and this driver against it).  No GPU is needed: every call
 * here returns before a launch (argument errors, zero-size work, or the operand check failing without
 * a device), so the sanitizer watches the host code paths alone: descriptor parsing, stride and
 * overflow arithmetic, workspace layouts, the residency check.  Prints one line per group of checks
 * and exits non-zero on an unexpected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "msa_index.h"
#include "msa_produce.h"
#include "msa_project.h"
#include "msa_unfused.h"

static int failures = 0;

static void expect(const char* what, msa_status got, msa_status want)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d\n", what, (int)got, msa_status_str(got), (int)want);
        ++failures;
    }
}

static void expect_one_of(const char* what, msa_status got, msa_status a, msa_status b)
{
    if (got != a && got != b) {
        fprintf(stderr, "%s: status %d, expected %d or %d\n", what, (int)got, (int)a, (int)b);
        ++failures;
    }
}

/* Aligned addresses that are never dereferenced. */
#define ADDR(i) ((void*)(uintptr_t)(0x100000u * (i)))

static msa_cache_view view(int heads, int64_t sp, int64_t sh, int64_t st, int dtype)
{
    msa_cache_view v;
    v.data = ADDR(9);
    v.stride_page = sp;
    v.stride_head = sh;
    v.stride_token = st;
    v.num_heads = heads;
    v.dtype = dtype;
    v.scale = (const float*)ADDR(10);
    return v;
}

static msa_status produce(int32_t T, int64_t xs, int32_t D, int64_t pages, const msa_cache_view* k,
                          const msa_cache_view* v, const msa_cache_view* ik, int32_t page_size)
{
    return msa_produce((const uint16_t*)ADDR(1), xs, T, D, 16, 2, 2, 1, (const int32_t*)ADDR(2),
                       (const int32_t*)ADDR(3), (const int32_t*)ADDR(4), 160, 64, 160, page_size, pages,
                       (const uint16_t*)ADDR(5), (const uint16_t*)ADDR(5), (const uint16_t*)ADDR(5),
                       (const uint16_t*)ADDR(5), 1e-6f, 1e4, (uint16_t*)ADDR(6), (uint16_t*)ADDR(7), k, v, ik,
                       (int64_t*)ADDR(8), NULL);
}

int main(void)
{
    const msa_cache_view kv = view(2, 2 * 64 * 128, 64 * 128, 128, MSA_CACHE_FP8_E4M3);
    const msa_cache_view ik = view(1, 64 * 128, 64 * 128, 128, MSA_CACHE_FP8_E4M3);
    const msa_cache_view bad_st = view(2, 2 * 64 * 128, 64 * 128, 64, MSA_CACHE_FP8_E4M3);
    const msa_cache_view nhd = view(2, 64 * 2 * 128, 128, 2 * 128, MSA_CACHE_BF16);

    /* producer */
    expect("produce T=0", produce(0, 2944, 128, 10240, &kv, &kv, &ik, 64), MSA_OK);
    expect("produce head_dim", produce(64, 2944, 64, 10240, &kv, &kv, &ik, 64), MSA_ERR_UNSUPPORTED);
    expect("produce stride", produce(64, 2943, 128, 10240, &kv, &kv, &ik, 64), MSA_ERR_STRIDE);
    expect("produce overlap", produce(64, 2944, 128, 10240, &bad_st, &kv, &ik, 64), MSA_ERR_STRIDE);
    expect("produce overflow", produce(64, 2944, 128, (int64_t)1 << 50, &kv, &kv, &ik, 64), MSA_ERR_OVERFLOW);
    expect("produce null cache", produce(64, 2944, 128, 10240, NULL, &kv, &ik, 64), MSA_ERR_NULL_POINTER);
    expect("produce page size", produce(64, 2944, 128, 10240, &kv, &kv, &ik, 0), MSA_ERR_SHAPE);
    expect("produce nhd T=0", produce(0, 2944, 128, 10240, &nhd, &nhd, &ik, 64), MSA_OK);
    expect_one_of("produce valid, no device", produce(64, 2944, 128, 10240, &kv, &kv, &ik, 64), MSA_ERR_LAUNCH,
                  MSA_ERR_NOT_DEVICE);
    printf("producer checks done\n");

    /* step entry points */
    expect("rope_table n<0", msa_rope_table((const int32_t*)ADDR(1), -1, 1e4, 128, (float*)ADDR(2), (float*)ADDR(3), NULL),
           MSA_ERR_SHAPE);
    expect("quantize dtype", msa_quantize((const float*)ADDR(1), 16, 7, NULL, ADDR(2), NULL), MSA_ERR_DTYPE);
    expect("rms_scale eps", msa_rms_scale((const double*)ADDR(1), 16, 128, -1.0f, (float*)ADDR(2), NULL), MSA_ERR_SHAPE);
    {
        const void* ptrs[3] = {NULL, ADDR(1), ADDR(2)};
        const uint64_t bytes[3] = {0, 64, 64};
        int32_t bad = -7;
        expect("check pointers, no device", msa_check_device_pointers(ptrs, bytes, 3, &bad), MSA_ERR_NOT_DEVICE);
        if (bad != 1) {
            fprintf(stderr, "check pointers: first bad %d, expected 1\n", bad);
            ++failures;
        }
        expect("check pointers, empty", msa_check_device_pointers(NULL, NULL, 0, &bad), MSA_OK);
    }
    printf("step entry point checks done\n");

    /* indexer */
    expect("index_scores T=0",
           msa_index_scores((const uint16_t*)ADDR(1), 0, 128, 2, (const int32_t*)ADDR(2), (const int32_t*)ADDR(3),
                            (const int32_t*)ADDR(4), 160, 64, 160, 64, 10240, &ik, 128, 72, (double*)ADDR(5), NULL),
           MSA_OK);
    expect("index_scores groups",
           msa_index_scores((const uint16_t*)ADDR(1), 64, 128, 3, (const int32_t*)ADDR(2), (const int32_t*)ADDR(3),
                            (const int32_t*)ADDR(4), 160, 64, 160, 64, 10240, &kv, 128, 72, (double*)ADDR(5), NULL),
           MSA_ERR_SHAPE);
    expect("index_topk k", msa_index_topk((const double*)ADDR(1), 128, 72, 0, (int32_t*)ADDR(2), NULL, NULL),
           MSA_ERR_SHAPE);
    printf("indexer checks done\n");

    /* unfused path */
    {
        uint64_t need = 0;
        expect("unfused workspace size", msa_produce_unfused_workspace_size(65536, 2, 1, &need), MSA_OK);
        expect("unfused small workspace",
               msa_produce_unfused((const uint16_t*)ADDR(1), 2944, 64, 128, 16, 2, 2, 1, (const int32_t*)ADDR(2),
                                   (const int64_t*)ADDR(3), 64, 10240, (const uint16_t*)ADDR(5),
                                   (const uint16_t*)ADDR(5), (const uint16_t*)ADDR(5), (const uint16_t*)ADDR(5),
                                   1e-6f, 1e4, (uint16_t*)ADDR(6), (uint16_t*)ADDR(7), &kv, &kv, &ik, ADDR(8), 16,
                                   NULL),
               MSA_ERR_WORKSPACE);
        expect("slots null", msa_slots(NULL, NULL, 4, NULL, 160, 64, 160, 64, 10240, NULL, NULL),
               MSA_ERR_NULL_POINTER);
    }
    printf("unfused checks done\n");

    /* projection */
    {
        uint64_t need = 0;
        expect("project workspace size", msa_project_workspace_size(64, 3072, 23, &need), MSA_OK);
        expect("project hidden", msa_project((const uint16_t*)ADDR(1), 3000, 64, 3000, (const uint16_t*)ADDR(2),
                                             3000, 2944, (uint16_t*)ADDR(3), 2944, NULL, 0, NULL),
               MSA_ERR_SHAPE);
        expect("project workspace", msa_project((const uint16_t*)ADDR(1), 3072, 64, 3072, (const uint16_t*)ADDR(2),
                                                3072, 2944, (uint16_t*)ADDR(3), 2944, NULL, 0, NULL),
               MSA_ERR_WORKSPACE);
        expect("noalloc too large",
               msa_project_produce_noalloc((const uint16_t*)ADDR(1), 3072, 1024, 3072, (const uint16_t*)ADDR(2), 3072,
                                           128, 16, 2, 2, 1, (const float*)ADDR(3), (const float*)ADDR(3),
                                           (const int64_t*)ADDR(4), 64, 10240, (const uint16_t*)ADDR(5),
                                           (const uint16_t*)ADDR(5), (const uint16_t*)ADDR(5),
                                           (const uint16_t*)ADDR(5), 1e-6f, (uint16_t*)ADDR(6), (uint16_t*)ADDR(7),
                                           &kv, &kv, &ik, NULL),
               MSA_ERR_WORKSPACE);
    }
    printf("projection checks done\n");
    printf("%s\n", failures ? "FAILED" : "all host checks passed under the sanitizer");
    return failures ? 1 : 0;
}
