/* Runs every tensor-level routine of the oracle (oracle/mx_oracle.c) under
 * AddressSanitizer, LeakSanitizer and UBSan on small tensors -- partial
 * blocks, one-row-block tensors, empty groups, every output set, element
 * format, scale rule, scale layout, pre-op and activation -- with every
 * input and output in a heap buffer of exactly the size its layout needs, so
 * that a read or write one byte outside it, an integer overflow or a leak
 * stops the run.  Values are not checked here (the oracle's pins do that);
 * each call must return 0. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_bf16_value(uint16_t b);
int64_t orc_tiled_scale_bytes(int64_t R, int64_t C);
int orc_mx_quantize(const uint16_t *x, const uint16_t *grad, int64_t M, int64_t K, unsigned axis,
                    int fusion, uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                    float *dbias, uint16_t *y_out);
int orc_mx_quantize_gated(const uint16_t *x, int64_t M, int64_t N, unsigned axis, int act,
                          uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                          uint16_t *y_out);
int orc_mx_quantize_dgated(const uint16_t *grad, const uint16_t *x, int64_t M, int64_t N,
                           unsigned axis, int act, uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                           uint8_t *s_col, uint16_t *y_out);
int orc_mx_quantize_grouped(const uint16_t *x, const uint16_t *grad, int64_t K, const int64_t *rows,
                            int G, unsigned axis, int fusion, uint8_t *q_row, uint8_t *s_row,
                            uint8_t *q_col, uint8_t *s_col, float *dbias);
int orc_mx_quantize_gated_grouped(const uint16_t *grad, const uint16_t *x, int64_t N,
                                  const int64_t *rows, int G, unsigned axis, int act,
                                  uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col);
float orc_absmax(const uint16_t *x, int64_t n);
int orc_nvfp4_quantize_transpose(const uint16_t *x, int64_t M, int64_t K, unsigned axis,
                                 float tensor_amax, uint8_t *q_row, uint8_t *s_row,
                                 uint8_t *q_col, uint8_t *s_col, float *sg_out);
int orc_nvfp4_quantize_transpose_2d(const uint16_t *x, int64_t M, int64_t K, unsigned axis,
                                    float tensor_amax, uint8_t *q_row, uint8_t *s_row,
                                    uint8_t *q_col, uint8_t *s_col, float *sg_out);
int orc_nvfp4_quantize_transpose_grouped(const uint16_t *x, int64_t K, const int64_t *rows, int G,
                                         const float *amax, int two_d, unsigned axis,
                                         uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                         uint8_t *s_col, float *sg_out);
void orc_set_threads(int n);

#define ROWS 1u
#define COLS 2u
#define E5M2 4u
#define ROUND_UP 8u
#define TILED 16u

static int failures = 0, calls = 0;

static void expect_ok(int rc, const char *what, long a, long b, unsigned axis, int extra)
{
    calls++;
    if (rc != 0) {
        fprintf(stderr, "%s(%ld, %ld, axis %u, %d) returned %d\n", what, a, b, axis, extra, rc);
        failures++;
    }
}

/* Exactly n bytes (NULL for n = 0 or an unused output). */
static void *buf(int64_t n) { return n > 0 ? malloc((size_t)n) : NULL; }

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint16_t next_bf16(void)
{
    rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
    uint16_t b = (uint16_t)(rng >> 32);
    if ((b & 0x7F80) == 0x7F80)   /* finite values only */
        b &= 0xBFFF;
    return b;
}

static uint16_t *input(int64_t n)
{
    uint16_t *x = (uint16_t *)malloc((size_t)n * 2);
    for (int64_t i = 0; i < n; i++)
        x[i] = next_bf16();
    if (n > 2)
        x[0] = 0x0000, x[1] = 0x8000;   /* +0, -0 */
    return x;
}

static int64_t nblocks(int64_t n) { return (n + 31) / 32; }

static int64_t scale_bytes(int64_t rows, int64_t cols, unsigned axis)
{
    if (rows == 0)
        return 0;
    return (axis & TILED) ? orc_tiled_scale_bytes(rows, nblocks(cols)) : rows * nblocks(cols);
}

/* One MXFP8 cast of a quantised [M][W] tensor through `which`:
 * 0 plain / pre-op (fusion), 1 gated (W = N), 2 gated backward (W = 2N). */
static void mx_case(int which, int64_t M, int64_t N, unsigned axis, int fusion_or_act)
{
    const int64_t W = which == 2 ? 2 * N : N;
    const int64_t nx = which == 0 ? M * N : M * 2 * N;
    uint16_t *x = input(nx), *g = input(M * N);
    uint8_t *qr = buf((axis & ROWS) ? M * W : 0), *sr = buf((axis & ROWS) ? scale_bytes(M, W, axis) : 0);
    uint8_t *qc = buf((axis & COLS) ? M * W : 0), *sc = buf((axis & COLS) ? scale_bytes(W, M, axis) : 0);
    uint16_t *y = (uint16_t *)buf(M * W * 2);
    float *db = (float *)buf(W * 4);
    int rc;
    if (which == 0)
        rc = orc_mx_quantize(x, g, M, N, axis, fusion_or_act, qr, sr, qc, sc, db, y);
    else if (which == 1)
        rc = orc_mx_quantize_gated(x, M, N, axis, fusion_or_act, qr, sr, qc, sc, y);
    else
        rc = orc_mx_quantize_dgated(g, x, M, N, axis, fusion_or_act, qr, sr, qc, sc, y);
    expect_ok(rc, which == 0 ? "mx_quantize" : which == 1 ? "gated" : "dgated", (long)M, (long)N,
              axis, fusion_or_act);
    if (which == 0) {   /* and without y_out, so the oracle allocates its own */
        rc = orc_mx_quantize(x, g, M, N, axis, fusion_or_act, qr, sr, qc, sc, db, NULL);
        expect_ok(rc, "mx_quantize (no y)", (long)M, (long)N, axis, fusion_or_act);
    }
    free(x), free(g), free(qr), free(sr), free(qc), free(sc), free(y), free(db);
}

/* Grouped casts of a stack of G groups: which 0 plain / pre-op (W = K),
 * 1 gated (W = K), 2 gated backward (W = 2K). */
static void grouped_call(int which, const int64_t *rows, int G, int64_t K, unsigned axis, int f)
{
    const int64_t W = which == 2 ? 2 * K : K;
    int64_t M = 0, srb = 0, scb = 0;
    for (int g = 0; g < G; g++) {
        M += rows[g];
        srb += scale_bytes(rows[g], W, axis), scb += scale_bytes(W, rows[g], axis);
    }
    uint16_t *x = input(which == 0 ? M * K : M * 2 * K), *g = input(M * K);
    uint8_t *qr = buf((axis & ROWS) ? M * W : 0), *qc = buf((axis & COLS) ? M * W : 0);
    uint8_t *sr = buf((axis & ROWS) ? srb : 0), *sc = buf((axis & COLS) ? scb : 0);
    float *db = (float *)buf(G * K * 4);
    int rc;
    if (which == 0)
        rc = orc_mx_quantize_grouped(x, g, K, rows, G, axis, f, qr, sr, qc, sc, db);
    else
        rc = orc_mx_quantize_gated_grouped(which == 2 ? g : NULL, x, K, rows, G, axis, f, qr, sr,
                                           qc, sc);
    expect_ok(rc, which == 0 ? "grouped" : which == 1 ? "gated_grouped" : "dgated_grouped",
              (long)M, (long)K, axis, f);
    free(x), free(g), free(qr), free(sr), free(qc), free(sc), free(db);
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void nvfp4_case(int64_t M, int64_t K, unsigned axis, int two_d, float amax)
{
    uint16_t *x = input(M * K);
    uint8_t *qr = buf((axis & ROWS) ? M * cdiv(K, 2) : 0), *sr = buf((axis & ROWS) ? M * cdiv(K, 16) : 0);
    uint8_t *qc = buf((axis & COLS) ? K * cdiv(M, 2) : 0), *sc = buf((axis & COLS) ? K * cdiv(M, 16) : 0);
    float *sg = (float *)buf(4);
    const float a = amax < 0 ? orc_absmax(x, M * K) : amax;
    expect_ok((two_d ? orc_nvfp4_quantize_transpose_2d : orc_nvfp4_quantize_transpose)(
                  x, M, K, axis, a, qr, sr, qc, sc, sg),
              two_d ? "nvfp4_2d" : "nvfp4", (long)M, (long)K, axis, two_d);
    free(x), free(qr), free(sr), free(qc), free(sc), free(sg);
}

static void nvfp4_grouped_case(const int64_t *rows, int G, int64_t K, unsigned axis, int two_d)
{
    int64_t M = 0, qcb = 0, scb = 0;
    for (int g = 0; g < G; g++) {
        M += rows[g];
        qcb += K * cdiv(rows[g], 2), scb += K * cdiv(rows[g], 16);
    }
    uint16_t *x = input(M * K);
    uint8_t *qr = buf((axis & ROWS) ? M * cdiv(K, 2) : 0), *sr = buf((axis & ROWS) ? M * cdiv(K, 16) : 0);
    uint8_t *qc = buf((axis & COLS) ? qcb : 0), *sc = buf((axis & COLS) ? scb : 0);
    float *amax = (float *)buf(G * 4), *sg = (float *)buf(G * 4);
    for (int g = 0, r = 0; g < G; r += (int)rows[g], g++)
        amax[g] = rows[g] ? orc_absmax(x + r * K, rows[g] * K) : 0.0f;
    expect_ok(orc_nvfp4_quantize_transpose_grouped(x, K, rows, G, amax, two_d, axis, qr, sr, qc, sc,
                                                   sg),
              "nvfp4_grouped", (long)M, (long)K, axis, two_d);
    expect_ok(orc_nvfp4_quantize_transpose_grouped(x, K, rows, G, NULL, two_d, axis, qr, sr, qc, sc,
                                                   NULL),
              "nvfp4_grouped (own amax)", (long)M, (long)K, axis, two_d);
    free(x), free(qr), free(sr), free(qc), free(sc), free(amax), free(sg);
}

int main(void)
{
    orc_set_threads(2);
    const int64_t shapes[][2] = {{16, 8}, {32, 32}, {48, 40}, {16, 264}, {272, 56}, {64, 520},
                                 {1, 1}, {17, 9}, {3, 70}, {70, 3}};
    const unsigned axes[] = {ROWS, COLS, ROWS | COLS};
    const unsigned variants[] = {0, E5M2, ROUND_UP, E5M2 | ROUND_UP, TILED, TILED | E5M2};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; s++)
        for (size_t a = 0; a < 3; a++)
            for (size_t v = 0; v < sizeof variants / sizeof variants[0]; v++) {
                const unsigned axis = axes[a] | variants[v];
                const int64_t M = shapes[s][0], K = shapes[s][1];
                for (int fusion = 0; fusion <= 3; fusion++) {
                    mx_case(0, M, K, axis, fusion);
                    mx_case(0, M, K, axis, fusion | 0x10);
                }
                for (int act = 1; act <= 2; act++) {
                    mx_case(1, M, K, axis, act);
                    mx_case(2, M, K, axis, act);
                }
            }
    const int64_t g1[] = {16, 0, 48, 32}, g2[] = {0, 0, 16}, g3[] = {144}, g4[] = {5, 0, 33, 1};
    struct { const int64_t *rows; int G; } groups[] = {{g1, 4}, {g2, 3}, {g3, 1}, {g4, 4}};
    const unsigned gvariants[] = {0, TILED | ROUND_UP};
    for (size_t i = 0; i < 4; i++)
        for (size_t a = 0; a < 3; a++)
            for (size_t v = 0; v < 2; v++)
                for (int64_t K = 8; K <= 296; K += 288) {
                    const unsigned axis = axes[a] | gvariants[v];
                    grouped_call(0, groups[i].rows, groups[i].G, K, axis, 0x10 | 1);
                    grouped_call(0, groups[i].rows, groups[i].G, K, axis, 3);
                    grouped_call(1, groups[i].rows, groups[i].G, K, axis, 1);
                    grouped_call(2, groups[i].rows, groups[i].G, K, axis, 2);
                }
    const int64_t nshapes[][2] = {{16, 16}, {32, 48}, {48, 272}, {144, 32},
                                  {1, 1}, {17, 9}, {5, 31}, {33, 50}};
    for (size_t s = 0; s < 8; s++)
        for (size_t a = 0; a < 3; a++)
            for (int two_d = 0; two_d <= 1; two_d++) {
                nvfp4_case(nshapes[s][0], nshapes[s][1], axes[a], two_d, -1.0f);
                nvfp4_case(nshapes[s][0], nshapes[s][1], axes[a], two_d, 0.0f);
                nvfp4_case(nshapes[s][0], nshapes[s][1], axes[a], two_d, 1e-38f);
            }
    for (size_t i = 0; i < 4; i++)
        for (size_t a = 0; a < 3; a++)
            for (int two_d = 0; two_d <= 1; two_d++) {
                nvfp4_grouped_case(groups[i].rows, groups[i].G, 48, axes[a], two_d);
                nvfp4_grouped_case(groups[i].rows, groups[i].G, 13, axes[a], two_d);
            }
    printf("%d oracle calls, %d failed\n", calls, failures);
    return failures ? 1 : 0;
}
