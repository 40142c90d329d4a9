/* Host-side driver for the AddressSanitizer build of libsrnl (host code
 * only, no device code object): every entry point on the paths that return
 * before any device work -- argument validation, empty grids, workspace
 * sizing with overflowing sizes, NULL pointers -- plus the host helpers over
 * whole grids. Nothing here touches a GPU. Prints "ok" and exits 0 when
 * every status matches; AddressSanitizer aborts on a memory error. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "srnl.h"

static int failures = 0;

#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            fprintf(stderr, "line %d: %s (last error: %s)\n", __LINE__, #cond, \
                    srnl_last_error());                                       \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static srnl_params params(unsigned flags)
{
    srnl_params p;
    memset(&p, 0, sizeof p);
    p.in_dtype = SRNL_F32;
    p.alpha_max = 0.9f;
    p.eps = 1e-6f;
    p.flags = flags;
    return p;
}

static void scan_args(void)
{
    srnl_params p = params(0);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, NULL, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 10, 2, 5, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 12, 2, 4, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 0, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 16, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, -1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1 << 30, 1 << 15, 1 << 15, 64, 1, 64, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1, 1 << 16, 1 << 16, 64, 1, 64, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 0, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_OK);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_PTR);
    p.alpha_max = 1.0f;
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_ARG);
    p = params(0x100u);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_ARG);
    p = params(SRNL_FLAG_RECORD);
    EXPECT(srnl_scan_workspace_bytes(2, 3, 4, 64, 2, 32, 15, &p) > 0);
    EXPECT(srnl_scan_workspace_bytes(2, 3, 4, 32, 2, 16, 15, &p) == 0);
    EXPECT(srnl_scan_workspace_bytes(1 << 22, 1 << 15, 1 << 15, 64, 2, 32, 15, &p) == 0);
    EXPECT(srnl_scan_fwd(NULL, 1 << 22, 1 << 15, 1 << 15, 64, 2, 32, 15, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 64, 2, 32, 15, &p, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_scan_bwd(NULL, 1, 2, 2, 64, 2, 32, 15, &p, NULL, NULL, 0, NULL, NULL, NULL) !=
           SRNL_OK);
    p = params(SRNL_FLAG_CHECK_FINITE);
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_PTR);
    p.in_dtype = (srnl_dtype)7;
    EXPECT(srnl_scan_fwd(NULL, 1, 2, 2, 8, 2, 4, 15, &p, NULL) == SRNL_ERR_DTYPE);

    p = params(0);
    EXPECT(srnl_scan_workspace_bytes(2, 3, 4, 8, 2, 4, 15, &p) == 0);
    p.flags = SRNL_FLAG_CHECK_FINITE;
    EXPECT(srnl_scan_workspace_bytes(2, 3, 4, 8, 2, 4, 15, &p) >= 8);
    EXPECT(srnl_scan_workspace_bytes(0, 3, 4, 8, 2, 4, 15, &p) == 0);
    EXPECT(srnl_scan_workspace_bytes(1 << 30, 1 << 15, 1 << 15, 64, 1, 64, 15, &p) == 0);
    EXPECT(srnl_scan_workspace_bytes(2, 3, 4, 8, 2, 4, 15, NULL) == 0);

    p = params(0);
    EXPECT(srnl_scan_1d(NULL, 1, 4, 8, 2, 4, NULL, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_scan_1d(NULL, 1, 4, 24, 2, 12, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_1d(NULL, 1, -1, 8, 2, 4, &p, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_1d(NULL, 1, 0, 8, 2, 4, &p, NULL) == SRNL_OK);
}

static void other_args(void)
{
    srnl_params p = params(0);
    EXPECT(srnl_fuse(NULL, 1, 2, 2, 6, 15, NULL, SRNL_F32, NULL, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_fuse(NULL, 1, 2, 2, 8, 15, NULL, (srnl_dtype)3, NULL, NULL) == SRNL_ERR_DTYPE);
    EXPECT(srnl_fuse(NULL, 0, 2, 2, 8, 15, NULL, SRNL_F32, NULL, NULL) == SRNL_OK);
    EXPECT(srnl_fuse(NULL, 1, 2, 2, 8, 15, NULL, SRNL_F32, NULL, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_route_gather(NULL, 1, 2, 2, 8, 31, SRNL_F32, NULL, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_route_gather(NULL, 1, 2, 2, 8, 15, (srnl_dtype)9, NULL, NULL) == SRNL_ERR_DTYPE);
    EXPECT(srnl_route_gather(NULL, 1, 2, 2, 8, 15, SRNL_BF16, NULL, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_init_states(NULL, 0, 4, 0, 0.02f, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_init_states(NULL, 1, 6, 0, 0.02f, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_init_states(NULL, 1, 4, 0, -1.0f, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_init_states(NULL, 1, 4, 0, 0.02f, NULL) == SRNL_ERR_PTR);

    EXPECT(srnl_scan_bwd_workspace_bytes(1, 4, 4, 64, 2, 32, 15, &p) > 0);
    EXPECT(srnl_scan_bwd_workspace_bytes(1, 4, 4, 60, 2, 32, 15, &p) == 0);
    EXPECT(srnl_scan_bwd_workspace_bytes(1 << 30, 1 << 15, 1 << 15, 64, 1, 64, 15, &p) == 0);
    EXPECT(srnl_scan_bwd_workspace_bytes(1, 4, 4, 64, 2, 32, 15, NULL) == 0);
    EXPECT(srnl_scan_bwd_workspace_bytes(1 << 22, 1 << 15, 1 << 15, 64, 2, 32, 15, &p) == 0);
    EXPECT(srnl_scan_bwd(NULL, 1 << 22, 1 << 15, 1 << 15, 64, 2, 32, 15, &p, NULL, NULL, 0, NULL,
                         NULL, NULL) == SRNL_ERR_ARG);
    EXPECT(srnl_scan_bwd(NULL, 1, 4, 4, 64, 2, 32, 15, NULL, NULL, NULL, 0, NULL, NULL, NULL) ==
           SRNL_ERR_PTR);
    EXPECT(srnl_scan_bwd(NULL, 1, 4, 4, 60, 2, 32, 15, &p, NULL, NULL, 0, NULL, NULL, NULL) ==
           SRNL_ERR_ARG);
    EXPECT(srnl_scan_bwd(NULL, 1, 4, 4, 64, 2, 32, 15, &p, NULL, NULL, 0, NULL, NULL, NULL) !=
           SRNL_OK);
    EXPECT(srnl_fuse_bwd_workspace_bytes(2, 4, 4, 64, 15) > 0);
    EXPECT(srnl_fuse_bwd_workspace_bytes(2, 4, 4, 64, 0) == 0);
    EXPECT(srnl_fuse_bwd(NULL, NULL, 1, 2, 2, 6, 15, NULL, NULL, NULL, NULL, 0, NULL) ==
           SRNL_ERR_ARG);
    EXPECT(srnl_fuse_bwd(NULL, NULL, 1, 2, 2, 8, 15, NULL, NULL, NULL, NULL, 0, NULL) != SRNL_OK);

    srnl_block_weights w;
    memset(&w, 0, sizeof w);
    w.ffn_hidden = 256;
    w.ln_eps = 1e-5f;
    EXPECT(srnl_block_workspace_bytes(2, 4, 4, 64, 15) > 0);
    EXPECT(srnl_block_workspace_bytes(1 << 30, 1 << 15, 1 << 15, 64, 15) == 0);
    EXPECT(srnl_block_fwd(NULL, 1, 4, 4, 64, 2, 32, 15, &p, NULL, NULL, 0, NULL) == SRNL_ERR_PTR);
    EXPECT(srnl_block_fwd(NULL, 1, 4, 4, 48, 2, 24, 15, &p, &w, NULL, 0, NULL) == SRNL_ERR_ARG);
    w.ffn_hidden = 40;
    EXPECT(srnl_block_fwd(NULL, 1, 4, 4, 64, 2, 32, 15, &p, &w, NULL, 0, NULL) == SRNL_ERR_ARG);
    w.ffn_hidden = 256;
    EXPECT(srnl_block_fwd(NULL, 1, 4, 4, 64, 2, 32, 15, &p, &w, NULL, 0, NULL) != SRNL_OK);
}

static void helpers(void)
{
    static const int dims[][2] = {{1, 1}, {1, 37}, {37, 1}, {2, 3}, {7, 7}, {14, 20}, {56, 56}};
    for (size_t g = 0; g < sizeof dims / sizeof dims[0]; ++g) {
        const int H = dims[g][0], W = dims[g][1];
        char *seen = (char *)malloc((size_t)H * W);
        for (int r = 0; r < 4; ++r) {
            memset(seen, 0, (size_t)H * W);
            for (long t = 0; t < (long)H * W; ++t) {
                int i = -1, j = -1;
                srnl_route_index(r, H, W, t, &i, &j);
                EXPECT(i >= 0 && i < H && j >= 0 && j < W);
                if (i >= 0 && i < H && j >= 0 && j < W)
                    seen[(size_t)i * W + j]++;
            }
            for (long c = 0; c < (long)H * W; ++c)
                EXPECT(seen[c] == 1);
            EXPECT(srnl_chunk_len(r, H, W, 0, 0) == (r < 2 ? W : H));
            EXPECT(srnl_chunk_len(r, H, W, 5, 3) == (r < 2 ? 5 : 3));
        }
        free(seen);
    }
    for (int s = -10; s <= 5; ++s)
        EXPECT(srnl_status_string((srnl_status)s) != NULL);
    EXPECT(srnl_last_error() != NULL);
}

int main(void)
{
    for (int rep = 0; rep < 3; ++rep) {
        scan_args();
        other_args();
    }
    helpers();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
