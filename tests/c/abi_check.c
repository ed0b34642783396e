/* Host-only use of the C ABI from C99: the header must compile on its own with
 * -Wall -Werror -pedantic, and every entry point that needs no device must
 * answer as documented (sizes, plan description, argument rejection). */
#include "fusedproj.h"

#include <stdio.h>
#include <string.h>

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

int main(void) {
    char buf[256];
    /* workspace sizes: zero for M = 0 and for invalid shapes, positive otherwise */
    CHECK(fp_workspace_bytes(0, 4096, 6144, FP_BF16, FP_BF16) == 0);
    CHECK(fp_workspace_bytes(32, 4096, 6144, FP_BF16, FP_BF16) > 0);
    CHECK(fp_workspace_bytes(32, 100, 6144, FP_BF16, FP_BF16) == 0);
    /* plan description of the decode gate/up shape */
    CHECK(fp_describe_plan(32, 4096, 28672, FP_BF16, FP_BF16, FP_ACT_SWIGLU, buf, sizeof buf) == FP_OK);
    CHECK(strstr(buf, "family=stream") != NULL);
    CHECK(strstr(buf, "swiglu") != NULL);
    /* truncation keeps a terminated string */
    CHECK(fp_describe_plan(32, 4096, 28672, FP_BF16, FP_BF16, FP_ACT_SWIGLU, buf, 8) == FP_OK);
    CHECK(strlen(buf) == 7);
    /* rejected before any device work */
    CHECK(fp_describe_plan(32, 4096, 6144, FP_F16, FP_I8, FP_ACT_NONE, buf, sizeof buf) == FP_E_DTYPE);
    CHECK(fp_describe_plan(32, 4096, 6144, FP_BF16, FP_BF16, (fp_act)7, buf, sizeof buf) == FP_E_ARG);
    CHECK(fused_add_norm_qkv(NULL, NULL, NULL, NULL, NULL, FP_NORM_RMS, 1e-5f, NULL, NULL, NULL, NULL, NULL,
                             NULL, 32, 4096, 32, 8, 128, FP_BF16, FP_BF16, FP_BF16, NULL, 0, NULL) == FP_E_NULL);
    CHECK(strlen(fp_last_error()) > 0);
    CHECK(fused_gateup_act(NULL, NULL, NULL, NULL, NULL, FP_NORM_RMS, 1e-5f, NULL, NULL, NULL, NULL,
                           32, 4095, 14336, FP_ACT_SWIGLU, FP_BF16, FP_BF16, FP_BF16, NULL, 0, NULL) != FP_OK);
    CHECK(strcmp(fp_status_str(FP_OK), "ok") == 0);
    /* the boundary's status numbering: 0-6 as first specified, 7 and 8 appended */
    CHECK(FP_E_ALIAS == 5 && FP_E_HIP == 6 && FP_E_WORKSPACE == 7 && FP_E_ARG == 8);
    /* plan overrides: set, read back, reject out-of-range values, restore */
    {
        fp_plan_override o, back;
        memset(&o, 0, sizeof o);
        o.no_stream = 1;
        CHECK(fp_plan_override_set(&o) == FP_OK);
        CHECK(fp_plan_override_get(&back) == FP_OK && back.no_stream == 1);
        CHECK(fp_describe_plan(32, 4096, 6144, FP_BF16, FP_BF16, FP_ACT_NONE, buf, sizeof buf) == FP_OK);
        CHECK(strstr(buf, "family=tiled") != NULL);
        o.stream_nr = 3;
        CHECK(fp_plan_override_set(&o) == FP_E_ARG);
        CHECK(fp_plan_override_set(NULL) == FP_OK);
        CHECK(fp_plan_override_get(NULL) == FP_E_NULL);
    }
    if (fails == 0) printf("abi_check ok\n");
    return fails != 0;
}
