/* Host driver for the sanitizer build of the library's argument checks
 * (test_sanitizers.py): calls every C entry point with arguments that must be
 * rejected, or that are no-ops (M == 0), so no call reaches a GPU. Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host side; any
 * out-of-bounds access, overflow or undefined shift in the validation code
 * aborts the run. Prints "ok" and exits 0 when every status is as expected. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "w4a16.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, w4a16_last_error());
        ++failures;
    } else if (want != 0 && strlen(w4a16_last_error()) == 0) {
        printf("FAIL %s: no error message\n", what);
        ++failures;
    }
}

int main(void) {
    void *p = (void *)(uintptr_t)4096; /* never dereferenced: every call below fails validation or is a no-op */
    size_t sz = 0;
    expect("abi version", w4a16_abi_version() > 0 ? 0 : -1, 0);
    expect("packed_size ok", w4a16_packed_size(4096, 4096, 128, W4A16_UINT4, &sz), 0);
    expect("packed_size null", w4a16_packed_size(4096, 4096, 128, 0, NULL), W4A16_ERR_INVALID_ARG);
    expect("packed_size G", w4a16_packed_size(4096, 4096, 100, 0, &sz), W4A16_ERR_UNSUPPORTED);
    expect("packed_size K%G", w4a16_packed_size(4096, 4104, 128, 0, &sz), W4A16_ERR_UNSUPPORTED);
    expect("packed_size N<=0", w4a16_packed_size(0, 4096, 128, 0, &sz), W4A16_ERR_INVALID_ARG);
    expect("packed_size qtype", w4a16_packed_size(16, 128, 128, 7, &sz), W4A16_ERR_INVALID_ARG);
    expect("packed_size huge", w4a16_packed_size((int64_t)1 << 40, (int64_t)1 << 40, -1, 0, &sz),
           W4A16_ERR_UNSUPPORTED);
    expect("packed_size extreme", w4a16_packed_size(INT64_MAX - 7, 8, -1, 0, &sz), W4A16_ERR_UNSUPPORTED);
    expect("repack null", w4a16_repack(NULL, p, NULL, 16, 128, 128, 0, p, 1 << 20, NULL), W4A16_ERR_INVALID_ARG);
    expect("repack size", w4a16_repack(p, p, NULL, 4096, 4096, 128, 0, p, 16, NULL), W4A16_ERR_SIZE);
    expect("repack_layout dims", w4a16_repack_layout(p, 2, 0, p, 0, NULL, 0, 16, 128, 128, 0, p, 1 << 20, NULL),
           W4A16_ERR_INVALID_ARG);
    expect("unpack align", w4a16_unpack((void *)(uintptr_t)4100, 16, 128, 128, 0, NULL, NULL, NULL, NULL),
           W4A16_ERR_INVALID_ARG);
    expect("select_path", w4a16_select_path(8, 9, 0), W4A16_ERR_INVALID_ARG);
    expect("select_path ok", w4a16_select_path(8, 0, 0) == W4A16_PATH_SKINNY ? 0 : -1, 0);
    expect("workspace_size", w4a16_workspace_size(16, 4096, 14336, 128, 0, 0, &sz), 0);
    expect("workspace_size M", w4a16_workspace_size(-1, 4096, 14336, 128, 0, 0, &sz), W4A16_ERR_INVALID_ARG);
    expect("gemm M=0", w4a16_gemm(p, 0, 4096, p, 4096, 4096, 128, 0, 0, NULL, p, 4096, 0, 0, NULL, 0, NULL), 0);
    expect("gemm dtype", w4a16_gemm(p, 4, 4096, p, 4096, 4096, 128, 0, 5, NULL, p, 4096, 0, 0, NULL, 0, NULL),
           W4A16_ERR_INVALID_ARG);
    expect("gemm lda", w4a16_gemm(p, 4, 100, p, 4096, 4096, 128, 0, 0, NULL, p, 4096, 0, 0, NULL, 0, NULL),
           W4A16_ERR_INVALID_ARG);
    expect("gemm tiled lda", w4a16_gemm(p, 256, (int64_t)1 << 23, p, 4096, 4096, 128, 0, 0, NULL, p, 4096, 0, 0,
                                        NULL, 0, NULL), W4A16_ERR_UNSUPPORTED);
    expect("gemm huge lda", w4a16_gemm(p, 4, INT64_MAX / 4, p, 4096, 4096, 128, 0, 0, NULL, p, 4096, 1, 0, NULL, 0,
                                       NULL), W4A16_ERR_UNSUPPORTED);
    expect("gemm workspace", w4a16_gemm(p, 1, 4096, p, 1024, 4096, 128, 0, 0, NULL, p, 1024, 0, 0, NULL, 0, NULL),
           W4A16_ERR_SIZE);
    expect("gemm_noalloc M=0", w4a16_gemm_noalloc(p, 0, 4096, p, 4096, 4096, 128, 0, 0, NULL, p, 4096, 0, 0, NULL),
           0);
    expect("gemm_noalloc too big", w4a16_gemm_noalloc(p, 1, 131072, p, 2048, 131072, 128, 0, 0, NULL, p, 2048, 0, 0,
                                                      NULL), W4A16_ERR_SIZE);
    expect("dequant ldw", w4a16_dequant(p, 4096, 4096, 128, 0, 0, p, 100, NULL), W4A16_ERR_INVALID_ARG);
    expect("gemm_dense M=0", w4a16_gemm_dense(p, 0, 64, p, 64, 64, 64, 0, NULL, p, 64, NULL, 0, NULL), 0);
    expect("gemm_dense dtype", w4a16_gemm_dense(p, 4, 64, p, 64, 64, 64, 3, NULL, p, 64, NULL, 0, NULL),
           W4A16_ERR_INVALID_ARG);
    expect("a8 quantize K", w4a8_quantize(p, 4, 4100, 4104, 0, p, 4104, p, NULL), W4A16_ERR_UNSUPPORTED);
    expect("a8 quantize M=0", w4a8_quantize(p, 0, 4096, 4096, 0, p, 4096, p, NULL), 0);
    expect("a8 workspace", w4a8_workspace_size(300, 14336, 2048, 128, &sz), 0);
    expect("a8 gemm ldq", w4a8_gemm(p, p, 4, 100, p, 4096, 4096, 128, 0, NULL, p, 4096, NULL, 0, NULL),
           W4A16_ERR_INVALID_ARG);
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
