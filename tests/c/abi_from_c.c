/* A plain C99 caller of libsfi.so: include/sfi.h must compile as C, and every entry point must
 * reject a missing descriptor with SFI_E_INVALID before touching a GPU (so this program runs
 * on a machine without one).  Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "sfi.h"

static int fails = 0;

static void expect(const char* what, int got, int want) {
    printf("%-32s %s\n", what, got == want ? "ok" : "FAILED");
    if (got != want) ++fails;
}

int main(void) {
    sfi_kv_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 1;
    d.num_q_heads = 4;
    d.num_kv_heads = 1;
    d.head_dim = 96;                                  /* not built: 64 and 128 only */
    d.dtype = SFI_BF16;
    expect("workspace of a bad descriptor", (int)sfi_workspace_bytes(&d, SFI_OP_DENSE, 0, 0), 0);
    expect("dense, no descriptor",
           sfi_dense_decode(NULL, NULL, NULL, NULL, NULL, 0, NULL, 0, NULL), SFI_E_INVALID);
    expect("select, no descriptor",
           sfi_select(NULL, NULL, 0, 0, 0, 0, NULL, 0, NULL, NULL, 0, NULL), SFI_E_INVALID);
    expect("mask, no descriptor",
           sfi_sink_bypass_mask(NULL, NULL, 0, NULL, 0.25f, NULL, NULL), SFI_E_INVALID);
    expect("sparse, no descriptor",
           sfi_sparse_decode(NULL, NULL, NULL, 0, NULL, 0, NULL, NULL, NULL, NULL, 0, NULL),
           SFI_E_INVALID);
    expect("reorg, no descriptor", sfi_reorg(NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL),
           SFI_E_INVALID);
    expect("status strings differ",
           strcmp(sfi_status_string(SFI_OK), sfi_status_string(SFI_E_HIP)) != 0, 1);
    return fails ? 1 : 0;
}
