/* A C99 consumer of include/arrms.h linked against libarrms.so: the header
 * compiles as C and the host-side entry points (plans, predicate, errors) work
 * through the C ABI without a GPU. */
#include <stdio.h>
#include <string.h>

#include "arrms.h"

static int failures = 0;

static void expect(int ok, const char *what) {
    if (!ok) {
        ++failures;
        fprintf(stderr, "FAIL %s: %s\n", what, ar_rms_last_error());
    }
}

int main(void) {
    ar_rms_plan_t plan = NULL;
    expect(ar_rms_one_stage(4, 21, 6144, ARRMS_BF16, 1) == 1, "window holds at T=21");
    expect(ar_rms_one_stage(4, 22, 6144, ARRMS_BF16, 1) == 0, "window ends at T=22");
    expect(ar_rms_plan(4, 8, 4096, ARRMS_BF16, 0, &plan) == ARRMS_OK, "plan");
    expect(plan != NULL, "plan handle");
    expect(ar_rms_plan_kernel(plan) == ARRMS_KERNEL_ROW, "row kernel in the window");
    ar_rms_plan_destroy(plan);
    plan = NULL;
    expect(ar_rms_plan(8, 8192, 8192, ARRMS_FP16, ARRMS_ROUND_REDUCED, &plan) == ARRMS_OK,
           "prefill plan");
    expect(ar_rms_plan_kernel(plan) == ARRMS_KERNEL_SPLIT, "split kernel beyond the window");
    /* T == 0: nothing to do, no pointer needed, no launch */
    ar_rms_plan_destroy(plan);
    expect(ar_rms_plan(4, 0, 4096, ARRMS_BF16, 0, &plan) == ARRMS_OK, "empty plan");
    expect(ar_rms_run(plan, NULL, NULL, NULL, 1e-6f, 0, NULL, NULL, NULL) == ARRMS_EINVAL,
           "NULL partial array refused");
    {
        const void *none[4] = {NULL, NULL, NULL, NULL};
        /* an aligned address that is never dereferenced: T == 0 launches nothing */
        const void *weight = (const void *)(uintptr_t)0x10000;
        expect(ar_rms_run(plan, none, NULL, weight, 1e-6f, 0, NULL, NULL, NULL) == ARRMS_OK,
               "T == 0 is a no-op");
    }
    ar_rms_plan_destroy(plan);
    plan = (ar_rms_plan_t)0;
    expect(ar_rms_plan(0, 8, 4096, ARRMS_BF16, 0, &plan) == ARRMS_EINVAL, "W = 0 refused");
    expect(plan == NULL && strlen(ar_rms_last_error()) > 0, "no plan, a message");
    expect(ar_rms_plan(17, 8, 4096, ARRMS_BF16, 0, &plan) == ARRMS_ENOTSUP, "W = 17 refused");
    ar_rms_plan_destroy(NULL);
    printf("%s: %d failures\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
