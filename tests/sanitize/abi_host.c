/*
 * Drives the host side of the C ABI (include/rbq.h) so that it can run
 * under AddressSanitizer and UndefinedBehaviorSanitizer: size and shape
 * arithmetic, kernel-family choice, argument checks of the compute calls,
 * and the program builder (which plans a whole op list on the host).  No
 * call here reaches a device; the pointers are aligned stand-in addresses
 * that the checks compare but never dereference.
 * Test infrastructure: built and run by tests/test_sanitizers_cpu.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rbq.h"

static int failures = 0;
#define CHECK(cond, ...)                                         \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                        \
            fputc('\n', stderr);                                 \
            ++failures;                                          \
        }                                                        \
    } while (0)

#define MiB ((uintptr_t)1 << 20)
static void *wbuf(int k) { return (void *)(((uintptr_t)1 << 30) + (uintptr_t)k * MiB); }
static void *abuf(int k) { return (void *)(((uintptr_t)2 << 30) + (uintptr_t)k * MiB); }

static rbq_shape shp(int out, int in, int K, int g)
{
    rbq_shape s = {out, in, K, g};
    return s;
}

static rbq_program_op op(int w, int x, int y, int out, int in, int wait_for, uint32_t layout, int group)
{
    rbq_program_op o;
    memset(&o, 0, sizeof(o));
    o.planes = (const uint32_t *)wbuf(2 * w);
    o.scales = (const uint16_t *)wbuf(2 * w + 1);
    o.x = (const uint16_t *)abuf(x);
    o.y = (uint16_t *)abuf(y);
    o.out_features = out;
    o.in_features = in;
    o.epilogue = RBQ_EPILOGUE_NONE;
    o.wait_for = wait_for;
    o.planes_layout = layout;
    o.group_size = group;
    return o;
}

static rbq_status build(const rbq_program_op *ops, int n, int K, size_t shrink)
{
    size_t bytes = rbq_program_bytes(n);
    CHECK(bytes > 0, "program bytes");
    unsigned char *img = malloc(bytes);
    rbq_status st = rbq_program_build(ops, n, K, img, bytes - shrink);
    free(img);
    return st;
}

int main(void)
{
    /* sizes and shape checks, including values near the int32 limits */
    const int outs[] = {-1, 0, 1, 5, 16, 4096, 11008, 22016, 65536, 1 << 30};
    const int ins[] = {-32, 0, 32, 96, 128, 4096, 11008, 13824, 16384, 1 << 30};
    const int Ks[] = {0, 1, 2, 3, 4, 8, 9};
    const int gs[] = {0, 64, 128, -128};
    for (size_t a = 0; a < sizeof outs / sizeof *outs; ++a)
        for (size_t b = 0; b < sizeof ins / sizeof *ins; ++b)
            for (size_t c = 0; c < sizeof Ks / sizeof *Ks; ++c)
                for (size_t d = 0; d < sizeof gs / sizeof *gs; ++d) {
                    rbq_shape s = shp(outs[a], ins[b], Ks[c], gs[d]);
                    rbq_status st = rbq_check_shape(s);
                    size_t pb = rbq_planes_bytes(s), sb = rbq_scales_bytes(s);
                    if (st != RBQ_OK)
                        CHECK(pb == 0 && sb == 0, "sizes of a refused shape");
                    for (int M = -1; M <= 2049; M += (M < 20 ? 1 : 1024)) {
                        (void)rbq_gemm_workspace_bytes(s, M);
                        (void)rbq_qat_backward_workspace_bytes(s, M);
                        (void)rbq_select_path(s, M);
                    }
                    (void)rbq_tiles_bytes(s);
                    (void)rbq_scale_tiles_bytes(s);
                    (void)rbq_dual_g_bytes(s);
                    (void)rbq_dual_h_bytes(s);
                    (void)rbq_encode_dual_workspace_bytes(s);
                }
    CHECK(rbq_planes_bytes(shp(4096, 11008, 2, 0)) == (size_t)2 * 4096 * 344 * 4, "planes bytes");

    /* argument errors of the compute calls, found before any launch */
    rbq_shape s = shp(64, 128, 2, 0);
    void *ok = (void *)(uintptr_t)0x10000;
    CHECK(rbq_encode(NULL, s, ok, ok, NULL, NULL) == RBQ_ERR_INVALID_ARG, "encode null W");
    CHECK(rbq_encode(ok, shp(64, 100, 2, 0), ok, ok, NULL, NULL) == RBQ_ERR_INVALID_ARG, "encode shape");
    CHECK(rbq_encode((const float *)((char *)ok + 2), s, ok, ok, NULL, NULL) == RBQ_ERR_ALIGNMENT,
          "encode alignment");
    CHECK(rbq_gemm(ok, ok, s, NULL, 1, ok, NULL, 0, NULL) == RBQ_ERR_INVALID_ARG, "gemm null x");
    CHECK(rbq_gemm(ok, ok, s, ok, -1, ok, NULL, 0, NULL) == RBQ_ERR_INVALID_ARG, "gemm M");
    CHECK(rbq_gemm_ex(ok, ok, s, ok, 1, ok, NULL, 0, 7, NULL) == RBQ_ERR_INVALID_ARG, "gemm_ex epilogue");
    CHECK(rbq_refit(NULL, s, ok, ok, NULL, NULL) == RBQ_ERR_INVALID_ARG, "refit null");
    CHECK(rbq_rebinarize(NULL, s, ok, ok, NULL, NULL) == RBQ_ERR_INVALID_ARG, "rebinarize null");
    CHECK(rbq_pack_tiles(NULL, s, ok, NULL) == RBQ_ERR_INVALID_ARG, "pack null");
    CHECK(rbq_qat_encode(NULL, s, ok, ok, NULL, NULL) == RBQ_ERR_INVALID_ARG, "qat encode null");
    CHECK(rbq_probe_read(NULL, 16, ok, NULL) == RBQ_ERR_INVALID_ARG, "probe null");
    CHECK(rbq_gemm_dual(ok, ok, ok, s, ok, -1, ok, NULL) == RBQ_ERR_INVALID_ARG, "gemm_dual M");
    CHECK(rbq_gemm_dual(ok, ok, (const uint16_t *)((char *)ok + 8), s, ok, 4, ok, NULL) == RBQ_ERR_ALIGNMENT,
          "gemm_dual h alignment");

    /* the program builder: valid lists of many ops, chains, tiles, g128 */
    enum { N = 224 };
    rbq_program_op ops[N];
    for (int i = 0; i < N; ++i)
        ops[i] = op(i, 0, 1 + i, 4096 + 16 * (i % 7), 4096, -1, RBQ_LAYOUT_ROWS, 0);
    CHECK(build(ops, N, 2, 0) == RBQ_OK, "224 independent ops");
    for (int i = 0; i < N; ++i)
        ops[i] = op(i, i, i + 1, 4096, 4096, i - 1, RBQ_LAYOUT_TILES, 0);
    CHECK(build(ops, N, 2, 0) == RBQ_OK, "a chain of 224 ops");
    CHECK(build(ops, N, 2, 16) == RBQ_ERR_INVALID_ARG, "image too small");
    CHECK(build(ops, N, 3, 0) == RBQ_ERR_UNSUPPORTED, "K = 3");
    for (int i = 0; i < 40; ++i)
        ops[i] = op(i, 0, 1 + i, i % 3 ? 13824 : 5120, i % 3 == 2 ? 13824 : 5120, -1, RBQ_LAYOUT_TILES,
                    128);
    CHECK(build(ops, 40, 4, 0) == RBQ_OK, "g128 ops");
    ops[1] = op(1, 0, 0, 4096, 4096, -1, RBQ_LAYOUT_ROWS, 0);      /* writes x of op 0, unordered */
    ops[0] = op(0, 0, 2, 4096, 4096, -1, RBQ_LAYOUT_ROWS, 0);
    ops[2] = op(2, 3, 4, 4096, 4096, -1, RBQ_LAYOUT_ROWS, 0);
    CHECK(build(ops, 3, 2, 0) == RBQ_ERR_INVALID_ARG, "unordered overlap");
    ops[0] = op(0, 0, 1, 250, 640, -1, RBQ_LAYOUT_ROWS, 0);
    CHECK(build(ops, 1, 2, 0) == RBQ_OK, "ragged rows");
    ops[0] = op(0, 0, 1, 250, 16512, -1, RBQ_LAYOUT_ROWS, 0);
    CHECK(build(ops, 1, 2, 0) == RBQ_ERR_UNSUPPORTED, "in beyond 16384");
    CHECK(rbq_program_build(NULL, 1, 2, NULL, 0) == RBQ_ERR_INVALID_ARG, "null ops");
    /* ops of two and four tokens */
    for (int i = 0; i < 128; ++i) {
        ops[i] = op(i, 0, 1 + i, i % 2 ? 22016 : 4096, 4096, -1, RBQ_LAYOUT_TILES, 0);
        ops[i].tokens = 4;
    }
    CHECK(build(ops, 128, 2, 0) == RBQ_OK, "four-token ops");
    ops[3].tokens = 2;
    CHECK(build(ops, 128, 2, 0) == RBQ_ERR_INVALID_ARG, "mixed token counts");
    for (int i = 0; i < 64; ++i) {
        ops[i] = op(i, 0, 1 + i, 4096, 11008, -1, RBQ_LAYOUT_TILES, 0);
        ops[i].tokens = 2;
    }
    CHECK(build(ops, 64, 2, 0) == RBQ_OK, "two-token ops");
    ops[0].in_features = 16384;
    CHECK(build(ops, 64, 2, 0) == RBQ_ERR_UNSUPPORTED, "two-token ops beyond 12288 columns");

    for (int st = 0; st < 8; ++st)
        CHECK(rbq_status_string((rbq_status)st) != NULL, "status string");
    CHECK(strstr(rbq_version(), "gfx950") != NULL, "version");

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("library host checks passed\n");
    return 0;
}
