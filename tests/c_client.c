/* A plain C caller of libzero_mi355x: the header compiles as C99 and the
 * host entry points work without Python.  Prints one "name value..." line per
 * result for tests/test_c_abi.py to compare with the oracle and the pages'
 * memory table.  No call here touches a GPU: the planner calls are host
 * code, and the device calls are given arguments that their host-side
 * checks reject before any launch. */
#include <stdio.h>
#include <string.h>

#include "zero.h"

int main(void)
{
    uint64_t b = 0, e = 0, bytes = 0, n_segs = 0, offs[5];
    zero_segment segs[16];
    const uint64_t numel[5] = {1000, 37, 4096, 3, 2500};
    uint32_t stage;
    zero_status st;

    st = zero_partition(100291305472ull, 400, 399, &b, &e);
    printf("partition %d %llu %llu\n", (int)st, (unsigned long long)b, (unsigned long long)e);
    for (stage = 0; stage < 4; ++stage) {
        st = zero_mem_bytes(stage, 7500000000ull, 64, 12, &bytes);
        printf("mem_bytes %u %d %llu\n", stage, (int)st, (unsigned long long)bytes);
    }
    st = zero_bucket_plan(numel, 5, 1024, 500, 7000, segs, 16, &n_segs);
    printf("plan %d %llu", (int)st, (unsigned long long)n_segs);
    for (uint64_t i = 0; i < n_segs && i < 16; ++i)
        printf(" %llu:%llu:%llu:%llu:%llu", (unsigned long long)segs[i].bucket,
               (unsigned long long)segs[i].tensor, (unsigned long long)segs[i].src_off,
               (unsigned long long)segs[i].dst_off, (unsigned long long)segs[i].len);
    printf("\n");
    st = zero_state_layout(1000000, 1ull << 30, offs);
    printf("layout %d %llu %llu %llu %llu %llu\n", (int)st, (unsigned long long)offs[0],
           (unsigned long long)offs[1], (unsigned long long)offs[2], (unsigned long long)offs[3],
           (unsigned long long)offs[4]);

    /* errors: status, its name, and a non-empty detail */
    st = zero_partition(10, 0, 0, &b, &e);
    printf("error_partition %d %s %d\n", (int)st, zero_status_str(st),
           zero_last_error() && strlen(zero_last_error()) > 0);
    st = zero_adam_step(NULL, NULL, ZERO_F16, NULL, NULL, NULL, NULL, ZERO_F16, 0, NULL, NULL,
                        NULL, NULL);
    printf("error_adam %d %s\n", (int)st, zero_status_str(st));
    st = zero_bucket_flatten(NULL, numel, 5, (zero_dtype)7, 0, 10, NULL, NULL);
    printf("error_flatten %d %s\n", (int)st, zero_status_str(st));
    return 0;
}
