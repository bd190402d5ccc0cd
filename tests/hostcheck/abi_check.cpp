// Host-only run of libmxcast's entry points (csrc/api.cpp) under
// AddressSanitizer and UBSan, with the kernel launchers replaced by
// recorders (launch_record.cpp).  Device pointers are distinct fake
// addresses 4 TiB apart that are never dereferenced: validation only
// compares and offsets them.
//
//   * malformed calls (NULL, enum, shape, alignment, workspace, overlap) at
//     and beyond the size limits, including sizes whose products overflow
//     int64: the expected status, and no launch;
//   * valid calls at the size limits of every entry point: MX_OK, one launch,
//     and a launch plan the kernels can run (tile counts, walk lengths within
//     the LDS stage, grids below 2^31 workgroups, group tables that tile the
//     stacked rows).
//
// Exit status 0 when every check holds; the sanitizers abort on the first
// finding.
#include <stdint.h>
#include <stdio.h>

#include "launch_record.h"
#include "mxcast.h"

using mxk::g_rec;

static int failures = 0, checks = 0;

#define CHECK(cond)                                                               \
    do {                                                                          \
        checks++;                                                                 \
        if (!(cond)) {                                                            \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            failures++;                                                           \
        }                                                                         \
    } while (0)

static const int64_t kDim = int64_t(1) << 23;
static const int64_t kBig = INT64_MAX;

// Fake device buffer i (4 TiB apart, 256-byte aligned) plus a byte offset.
template <class T = uint8_t>
static T *P(int i, uint64_t off = 0)
{
    return reinterpret_cast<T *>((uint64_t(i + 1) << 42) + off);
}

static int launches() { return g_rec.calls + g_rec.reduces; }

// The call returns `want`; it launches something exactly when want is MX_OK.
#define EXPECT(want, call)                                                          \
    do {                                                                            \
        const int before = launches();                                              \
        const mx_status got = (call);                                               \
        checks++;                                                                   \
        if (got != (want)) {                                                        \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, \
                    #call, (int)got, (int)(want));                                  \
            failures++;                                                             \
        }                                                                           \
        CHECK(((want) == MX_OK) == (launches() > before));                          \
    } while (0)

static int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// A single-tensor launch plan of an M x K quantised tensor.
static void check_plan(int64_t M, int64_t K, int tiles_m, int tiles_k, int group, int groups_m,
                       bool tiled)
{
    CHECK(tiles_m == ceil_div(M, mxk::kTileM));
    CHECK(tiles_k == ceil_div(K, mxk::kTileK));
    CHECK(group >= 1 && group <= mxk::kMaxGroup);
    CHECK(!tiled || group % 2 == 0 || group >= tiles_m);
    CHECK(groups_m == ceil_div(tiles_m, group));
    CHECK((int64_t)groups_m * tiles_k <= INT32_MAX);
}

// The launch plan of the any-shape kernel for one M x K tensor: 64 x 128
// steps, walks of at most kAnyMaxWalk steps, one group.
static void check_any_plan(int64_t M, int64_t K)
{
    const mxk::MxArgs &a = g_rec.mx;
    const mxk::GroupTable &gt = g_rec.gt;
    CHECK(a.tiles_m == ceil_div(M, mxk::kAnyTileM) && a.tiles_k == ceil_div(K, mxk::kAnyTileK));
    CHECK(a.group >= 1 && a.group <= mxk::kAnyMaxWalk);
    CHECK(a.groups_m == ceil_div(a.tiles_m, a.group));
    CHECK((int64_t)a.groups_m * a.tiles_k <= INT32_MAX);
    CHECK(gt.count == 1 && gt.len[0] == a.group && gt.walk0[0] == 0 && gt.walk0[1] == a.groups_m);
    CHECK(gt.row0[0] == 0 && gt.row0[1] == M && gt.srow_off[0] == 0 && gt.scol_off[0] == 0);
}

// The kernel an M x K cast goes to: the tiled kernel for row lengths that
// are multiples of 8, its variant for transposed rows at any byte when the
// transposed output is asked for and M is not a multiple of 16, the
// any-shape kernel for other row lengths.
static int mx_route(int64_t M, int64_t K, bool col = true)
{
    if (K % 8 != 0)
        return mxk::kLaunchMxAny;
    return col && M % 16 != 0 ? mxk::kLaunchMxRagged : mxk::kLaunchMx;
}

static void check_mx(int64_t M, int64_t K, bool tiled, int kind = mxk::kLaunchMx)
{
    const mxk::MxArgs &a = g_rec.mx;
    CHECK(a.M == M && a.K == K);
    CHECK((a.tiled != 0) == tiled);
    CHECK(g_rec.kind == kind);
    if (kind == mxk::kLaunchMxAny) {
        check_any_plan(M, K);
        return;
    }
    check_plan(M, K, a.tiles_m, a.tiles_k, a.group, a.groups_m, tiled);
    if (kind == mxk::kLaunchMxRagged) {
        // the tensor as a stack of one group, with the tiled kernel's walks,
        // at most kMaxRagGroup sub-tiles long (the double stage's budget)
        CHECK(a.group <= mxk::kMaxRagGroup);
        const mxk::GroupTable &gt = g_rec.gt;
        CHECK(gt.count == 1 && gt.len[0] == a.group && gt.walk0[0] == 0 && gt.walk0[1] == a.groups_m);
        CHECK(gt.row0[0] == 0 && gt.row0[1] == M && gt.srow_off[0] == 0 && gt.scol_off[0] == 0);
        CHECK(a.qcol_nt == 0);
    }
}

// A group table over G groups of the given row counts, stacked (walks of the
// tiled kernel, or with any of the any-shape kernel).
static void check_groups(const int64_t *rows, int G, int walks_total, bool any = false)
{
    const mxk::GroupTable &gt = g_rec.gt;
    const int tile = any ? mxk::kAnyTileM : mxk::kTileM;
    const int maxlen = any ? mxk::kAnyMaxWalk : mxk::kMaxGroup;
    CHECK(gt.count == G);
    int64_t r = 0;
    for (int g = 0; g < G; g++) {
        CHECK(gt.row0[g] == r);
        CHECK(gt.len[g] >= 1 && gt.len[g] <= maxlen);
        CHECK(gt.walk0[g + 1] - gt.walk0[g] == ceil_div(ceil_div(rows[g], tile), gt.len[g]));
        r += rows[g];
    }
    CHECK(gt.row0[G] == r);
    CHECK(gt.walk0[0] == 0 && gt.walk0[G] == walks_total);
}

static void mx_quantize_cases()
{
    const unsigned both = MX_ROWWISE | MX_COLWISE;
    uint8_t *qr = P(2), *sr = P(3), *qc = P(4), *sc = P(5);
    float *db = P<float>(6);
    void *ws = P(7);
    // valid: the metric shape, the size limits, every format / layout flag
    EXPECT(MX_OK, mx_quantize(P(0), nullptr, 16384, 16384, both, 0, qr, sr, qc, sc, nullptr,
                              nullptr, 0, 0));
    check_mx(16384, 16384, false);
    // ... and shapes for the any-shape kernel: rows or row lengths that are
    // not multiples of 16 and 8, down to 1, up to the limits
    const int64_t shapes[][2] = {{kDim, 1 << 17}, {1 << 17, kDim}, {16, kDim}, {kDim, 8},
                                 {16, 8}, {kDim, kDim >> 6}, {16400, 7176},
                                 {1, 1}, {1, kDim}, {kDim, 1}, {17, 9}, {16383, 16383},
                                 {kDim - 1, (1 << 17) - 1}, {(1 << 17) - 3, kDim}, {40, 64},
                                 {kDim, 12}, {kDim >> 6, kDim - 4}, {16383, 16384}, {1, 8},
                                 {kDim - 1, 8}, {(1 << 17) - 1, kDim}, {100, 7168}};
    for (auto &s : shapes) {
        for (unsigned flags : {0u, (unsigned)MX_SCALE_TILED, MX_ELEM_E5M2 | MX_SCALE_ROUND_UP}) {
            for (int fusion : {0, MX_FUSE_GELU, MX_FUSE_DGELU | MX_FUSE_DBIAS, MX_FUSE_DSILU}) {
                const size_t need = mx_quantize_workspace_size(s[0], s[1], both | flags, fusion);
                CHECK(((fusion & MX_FUSE_DBIAS) != 0) == (need > 0));
                EXPECT(MX_OK, mx_quantize(P(0), P(1), s[0], s[1], both | flags, fusion, qr, sr, qc,
                                          sc, db, ws, need, 0));
                check_mx(s[0], s[1], flags & MX_SCALE_TILED, mx_route(s[0], s[1]));
                if (need) {
                    CHECK(g_rec.segments == g_rec.mx.groups_m);
                    CHECK(need == (size_t)g_rec.mx.groups_m * (size_t)s[1] * 4);
                    EXPECT(MX_ERR_WORKSPACE, mx_quantize(P(0), P(1), s[0], s[1], both | flags, fusion,
                                                         qr, sr, qc, sc, db, ws, need - 4, 0));
                }
            }
        }
        EXPECT(MX_OK, mx_quantize(P(0), nullptr, s[0], s[1], MX_ROWWISE, 0, qr, sr, nullptr,
                                  nullptr, nullptr, nullptr, 0, 0));
        check_mx(s[0], s[1], false, mx_route(s[0], s[1], false));
        EXPECT(MX_OK, mx_quantize(P(0), nullptr, s[0], s[1], MX_COLWISE, 0, nullptr, nullptr, qc,
                                  sc, nullptr, nullptr, 0, 0));
        check_mx(s[0], s[1], false, mx_route(s[0], s[1]));
    }
    // shapes
    const int64_t bad[][2] = {{kDim + 16, 8},  {16, kDim + 8}, {kDim, (1 << 17) + 8},
                              {0, 8},          {16, 0},        {-16, 8},
                              {16, -8},        {kDim + 1, 1},  {1, kDim + 1},
                              {kBig, kBig},    {kBig - 15, 8}, {16, kBig - 7},
                              {INT64_MIN, 8},  {int64_t(1) << 62, int64_t(1) << 62},
                              {kDim, (1 << 17) + 1}, {-1, -1}};
    for (auto &s : bad) {
        EXPECT(MX_ERR_SHAPE, mx_quantize(P(0), nullptr, s[0], s[1], both, 0, qr, sr, qc, sc,
                                         nullptr, nullptr, 0, 0));
        CHECK(mx_quantize_workspace_size(s[0], s[1], both, MX_FUSE_DBIAS) == 0);
        CHECK(mx_scale_size(s[0], s[1], both) == 0 || (s[0] > 0 && s[1] > 0));
    }
    CHECK(mx_scale_size(kBig, 1, MX_ROWWISE) == 0 && mx_scale_size(1, kBig, MX_ROWWISE) == 0);
    CHECK(mx_scale_size(kDim, kDim, MX_ROWWISE | MX_SCALE_TILED) ==
          (size_t)(kDim / 32) * (size_t)(kDim / 256) * 256);
    // enums, NULLs, alignment, overlap
    EXPECT(MX_ERR_ENUM, mx_quantize(P(0), nullptr, 16, 8, 0, 0, qr, sr, qc, sc, nullptr, nullptr, 0, 0));
    EXPECT(MX_ERR_ENUM, mx_quantize(P(0), nullptr, 16, 8, both | 32u, 0, qr, sr, qc, sc, nullptr,
                                    nullptr, 0, 0));
    EXPECT(MX_ERR_ENUM, mx_quantize(P(0), nullptr, 16, 8, both, 4, qr, sr, qc, sc, nullptr, nullptr, 0, 0));
    EXPECT(MX_ERR_ENUM, mx_quantize(P(0), nullptr, 16, 8, both, 0x20, qr, sr, qc, sc, nullptr,
                                    nullptr, 0, 0));
    EXPECT(MX_ERR_ENUM, mx_quantize(P(0), nullptr, 16, 8, both, -1, qr, sr, qc, sc, nullptr, nullptr, 0, 0));
    EXPECT(MX_ERR_NULL, mx_quantize(nullptr, nullptr, 16, 8, both, 0, qr, sr, qc, sc, nullptr,
                                    nullptr, 0, 0));
    EXPECT(MX_ERR_NULL, mx_quantize(P(0), nullptr, 16, 8, both, MX_FUSE_DSILU, qr, sr, qc, sc,
                                    nullptr, nullptr, 0, 0));
    EXPECT(MX_ERR_NULL, mx_quantize(P(0), nullptr, 16, 8, both, MX_FUSE_DBIAS, qr, sr, qc, sc,
                                    nullptr, ws, 1 << 20, 0));
    EXPECT(MX_ERR_NULL, mx_quantize(P(0), nullptr, 16, 8, both, 0, qr, nullptr, qc, sc, nullptr,
                                    nullptr, 0, 0));
    EXPECT(MX_ERR_ALIGN, mx_quantize(P(0, 2), nullptr, 16, 8, both, 0, qr, sr, qc, sc, nullptr,
                                     nullptr, 0, 0));
    EXPECT(MX_ERR_ALIGN, mx_quantize(P(0), nullptr, 16, 8, both, 0, qr, sr, qc, P(5, 8), nullptr,
                                     nullptr, 0, 0));
    EXPECT(MX_ERR_WORKSPACE, mx_quantize(P(0), nullptr, 16, 8, both, MX_FUSE_DBIAS, qr, sr, qc, sc,
                                         db, nullptr, 0, 0));
    // overlap: an output ending one byte into the input, outputs sharing a byte
    const uint64_t n = uint64_t(kDim) << 17;
    EXPECT(MX_ERR_ALIAS, mx_quantize(P(0), nullptr, kDim, 1 << 17, both, 0, P(0, 2 * n - 16), sr, qc,
                                     sc, nullptr, nullptr, 0, 0));
    EXPECT(MX_OK, mx_quantize(P(0), nullptr, kDim, 1 << 17, both, 0, P(0, 2 * n), sr, qc, sc,
                              nullptr, nullptr, 0, 0));
    EXPECT(MX_ERR_ALIAS, mx_quantize(P(0), nullptr, kDim, 1 << 17, both, 0, qr, P(2, n - 16), qc, sc,
                                     nullptr, nullptr, 0, 0));
    // the allocation-free variant: small dbias casts run, large ones are refused
    EXPECT(MX_OK, mx_quantize_noalloc(P(0), nullptr, 16384, 16384, both, MX_FUSE_DBIAS, qr, sr, qc,
                                      sc, db, 0));
    CHECK(g_rec.segments * 16384 * 4 <= (int64_t)MX_NOALLOC_SCRATCH_BYTES);
    EXPECT(MX_ERR_WORKSPACE, mx_quantize_noalloc(P(0), nullptr, 128, kDim, both, MX_FUSE_DBIAS, qr,
                                                 sr, qc, sc, db, 0));
    EXPECT(MX_OK, mx_quantize_noalloc(P(0), nullptr, kDim, 1 << 17, both, 0, qr, sr, qc, sc,
                                      nullptr, 0));
    EXPECT(MX_ERR_SHAPE, mx_quantize_noalloc(P(0), nullptr, kBig, kBig, both, MX_FUSE_DBIAS, qr, sr,
                                             qc, sc, db, 0));
}

static void gated_cases()
{
    const unsigned both = MX_ROWWISE | MX_COLWISE;
    uint8_t *qr = P(2), *sr = P(3), *qc = P(4), *sc = P(5);
    const int64_t ok[][2] = {{128, kDim / 2}, {kDim, 8}, {16, 8}, {kDim, 1 << 16}, {8192, 4096},
                             {1, 1}, {17, 4}, {kDim - 1, 1 << 16}, {128, kDim / 2 - 1}, {40, 12},
                             {kDim, (1 << 16) - 1}};
    for (auto &s : ok) {
        // the tiled kernel needs N a multiple of 8 (both halves aligned)
        const int kind = mx_route(s[0], s[1]);
        for (int act : {MX_GATED_SWIGLU, MX_GATED_GEGLU}) {
            EXPECT(MX_OK, mx_quantize_gated(P(0), s[0], s[1], both, act, qr, sr, qc, sc, 0));
            check_mx(s[0], s[1], false, kind);
            CHECK(g_rec.mx.ldx == 2 * s[1] && g_rec.mx.lin_off == s[1]);
            EXPECT(MX_OK, mx_quantize_gated(P(0), s[0], s[1], MX_ROWWISE, act, qr, sr, nullptr,
                                            nullptr, 0));
            check_mx(s[0], s[1], false, mx_route(s[0], s[1], false));
            EXPECT(MX_OK, mx_quantize_dgated(P(1), P(0), s[0], s[1], both | MX_SCALE_TILED, act, qr,
                                             sr, qc, sc, 0));
            check_mx(s[0], 2 * s[1], true, kind);
            CHECK(g_rec.mx.ldx == 2 * s[1] && g_rec.mx.ldg == s[1] && g_rec.mx.lin_off == s[1]);
        }
    }
    const int64_t bad[][2] = {{128, kDim / 2 + 8}, {kDim + 16, 8}, {16, 0}, {16, kBig},
                              {kBig, 8},           {16, kBig / 2 + 1}, {16, INT64_MIN},
                              {16, -8},            {int64_t(1) << 62, int64_t(1) << 62},
                              {0, 8},              {128, kDim / 2 + 1}};
    for (auto &s : bad) {
        EXPECT(MX_ERR_SHAPE, mx_quantize_gated(P(0), s[0], s[1], both, MX_GATED_SWIGLU, qr, sr, qc, sc, 0));
        EXPECT(MX_ERR_SHAPE, mx_quantize_dgated(P(1), P(0), s[0], s[1], both, MX_GATED_GEGLU, qr, sr,
                                                qc, sc, 0));
        if (s[1] > 0 && s[1] <= kDim / 2)
            continue;   // N itself is valid for the grouped casts below
        const int64_t rows[2] = {16, 16};
        EXPECT(MX_ERR_SHAPE, mx_quantize_gated_grouped(P(0), s[1], rows, 2, both, MX_GATED_SWIGLU, qr,
                                                       sr, qc, sc, 0));
        EXPECT(MX_ERR_SHAPE, mx_quantize_dgated_grouped(P(1), P(0), s[1], rows, 2, both,
                                                        MX_GATED_SWIGLU, qr, sr, qc, sc, 0));
    }
    EXPECT(MX_ERR_ENUM, mx_quantize_gated(P(0), 16, 8, both, 0, qr, sr, qc, sc, 0));
    EXPECT(MX_ERR_ENUM, mx_quantize_dgated(P(1), P(0), 16, 8, both, 3, qr, sr, qc, sc, 0));
    EXPECT(MX_ERR_NULL, mx_quantize_dgated(nullptr, P(0), 16, 8, both, 1, qr, sr, qc, sc, 0));
    EXPECT(MX_ERR_ALIAS, mx_quantize_dgated(P(1), P(0), 16, 8, both, 1, P(1, 16 * 8 * 2 - 16), sr, qc,
                                            sc, 0));
    // fused values alone
    for (int op : {MX_FUSE_GELU, MX_FUSE_DGELU, MX_FUSE_DSILU, MX_OP_GATED | MX_GATED_SWIGLU,
                   MX_OP_DGATED | MX_GATED_GEGLU}) {
        EXPECT(MX_OK, mx_fused_values(P(0), P(1), 16, 8, op, P(2), 0));
        CHECK(g_rec.kind == mxk::kLaunchValues);
        EXPECT(MX_OK, mx_fused_values(P(0), P(1), 3, 7, op, P(2), 0));
        CHECK(g_rec.kind == mxk::kLaunchValuesAny && g_rec.M == 3 && g_rec.K == 7);
        EXPECT(MX_ERR_SHAPE, mx_fused_values(P(0), P(1), 0, 8, op, P(2), 0));
        EXPECT(MX_ERR_SHAPE, mx_fused_values(P(0), P(1), kBig, kBig, op, P(2), 0));
        EXPECT(MX_ERR_SHAPE, mx_fused_values(P(0), P(1), 16, kBig / 2 + 1, op, P(2), 0));
    }
    EXPECT(MX_ERR_ENUM, mx_fused_values(P(0), P(1), 16, 8, 0, P(2), 0));
    EXPECT(MX_ERR_ENUM, mx_fused_values(P(0), P(1), 16, 8, MX_OP_GATED | 3, P(2), 0));
}

static void grouped_cases()
{
    const unsigned both = MX_ROWWISE | MX_COLWISE;
    uint8_t *qr = P(2), *sr = P(3), *qc = P(4), *sc = P(5);
    float *db = P<float>(6);
    void *ws = P(7);
    // 64 groups filling 2^23 rows, some empty; the 8-expert MoE shape; one group
    int64_t full[64];
    for (int g = 0; g < 64; g++)
        full[g] = g % 4 == 3 ? 0 : (kDim / 48) & ~int64_t(15);
    const int64_t moe[8] = {1104, 3008, 1072, 6560, 1632, 608, 2256, 144};
    const int64_t one[1] = {kDim};
    // row counts that are not multiples of 16 (the any-shape kernel)
    const int64_t ragged[8] = {1101, 3008, 0, 6563, 1, 608, 2255, 17};
    int64_t full_odd[64];
    for (int g = 0; g < 64; g++)
        full_odd[g] = g % 4 == 3 ? 0 : (kDim / 48) - 1;
    struct Case { const int64_t *rows; int G; int64_t K; } cases[] = {
        {full, 64, 1 << 17}, {moe, 8, 7168}, {one, 1, 1 << 17}, {moe, 8, 8}, {one, 1, 1 << 16},
        {full, 64, 1 << 16}, {ragged, 8, 7168}, {moe, 8, 7000}, {ragged, 8, 1}, {full_odd, 64, 1 << 17},
        {one, 1, (1 << 17) - 1}};
    for (auto &c : cases) {
        int64_t M = 0;
        bool rows16 = true;
        for (int g = 0; g < c.G; g++) {
            M += c.rows[g];
            rows16 = rows16 && c.rows[g] % 16 == 0;
        }
        const bool any = c.K % 8 != 0;
        const int kind = any ? mxk::kLaunchMxAny : rows16 ? mxk::kLaunchMxGrouped : mxk::kLaunchMxRagged;
        for (unsigned flags : {0u, (unsigned)MX_SCALE_TILED}) {
            for (int fusion : {0, MX_FUSE_DBIAS, MX_FUSE_DGELU | MX_FUSE_DBIAS}) {
                const size_t need = mx_quantize_grouped_workspace_size(c.K, c.rows, c.G, both | flags,
                                                                      fusion);
                EXPECT(MX_OK, mx_quantize_grouped(P(0), P(1), c.K, c.rows, c.G, both | flags, fusion,
                                                  qr, sr, qc, sc, db, ws, need, 0));
                CHECK(g_rec.kind == kind && g_rec.mx.M == M);
                if (kind == mxk::kLaunchMxRagged)
                    for (int g = 0; g < c.G; g++)
                        CHECK(g_rec.gt.len[g] <= mxk::kMaxRagGroup);
                CHECK(g_rec.mx.tiles_k == ceil_div(c.K, any ? mxk::kAnyTileK : mxk::kTileK));
                check_groups(c.rows, c.G, g_rec.mx.groups_m, any);
                if (fusion & MX_FUSE_DBIAS)
                    CHECK(need == (size_t)g_rec.mx.groups_m * (size_t)c.K * 4);
                CHECK((int64_t)g_rec.mx.groups_m * g_rec.mx.tiles_k <= INT32_MAX);
                const size_t srow = mx_grouped_scale_size(c.K, c.rows, c.G, both | flags, 0);
                const size_t scol = mx_grouped_scale_size(c.K, c.rows, c.G, both | flags, 1);
                int64_t s0 = 0, s1 = 0;
                for (int g = 0; g < c.G; g++) {
                    CHECK(g_rec.gt.srow_off[g] == s0 && g_rec.gt.scol_off[g] == s1);
                    s0 += (int64_t)mx_scale_size(c.rows[g], c.K, both | flags);
                    s1 += (int64_t)mx_scale_size(c.K, c.rows[g], both | flags);
                }
                CHECK((size_t)s0 == srow && (size_t)s1 == scol);
            }
        }
        // gated: x is [M][2N] with N = K (at most 2^40 elements, 2N <= 2^23)
        const bool gated_ok = 2 * c.K <= kDim && M * 2 * c.K <= (int64_t(1) << 40);
        EXPECT(gated_ok ? MX_OK : MX_ERR_SHAPE,
               mx_quantize_gated_grouped(P(0), c.K, c.rows, c.G, both, MX_GATED_SWIGLU, qr, sr, qc,
                                         sc, 0));
        if (gated_ok) {
            CHECK(g_rec.kind == kind);
            check_groups(c.rows, c.G, g_rec.mx.groups_m, any);
        }
        EXPECT(gated_ok ? MX_OK : MX_ERR_SHAPE,
               mx_quantize_dgated_grouped(P(1), P(0), c.K, c.rows, c.G, both | MX_SCALE_TILED,
                                          MX_GATED_GEGLU, qr, sr, qc, sc, 0));
        if (gated_ok) {
            CHECK(g_rec.mx.K == 2 * c.K && g_rec.mx.tiled == 1);
            check_groups(c.rows, c.G, g_rec.mx.groups_m, any);
        }
        {
            const bool nv_any = c.K % 16 != 0;
            const bool nv_rag = !nv_any && !rows16;
            for (int two_d : {0, 1}) {
                EXPECT(MX_OK, nvfp4_quantize_transpose_grouped(P(0), c.K, c.rows, c.G, P<float>(1), two_d,
                                                               both, qr, sr, qc, sc, P<float>(6), 0));
                CHECK(g_rec.kind == (nv_any ? mxk::kLaunchNvAny
                                            : nv_rag ? mxk::kLaunchNvRagged : mxk::kLaunchNvGrouped));
                if (nv_rag)
                    for (int g = 0; g < c.G; g++)
                        CHECK(g_rec.gt.len[g] % 2 == 0 && g_rec.gt.len[g] <= mxk::kMaxNvRagGroup);
                check_groups(c.rows, c.G, g_rec.nv.groups_m, nv_any);
                CHECK((int64_t)g_rec.nv.groups_m * g_rec.nv.tiles_k <= INT32_MAX);
                int64_t qo = 0, so = 0;
                for (int g = 0; g < c.G; g++) {
                    CHECK(g_rec.gt.qcol_off[g] == qo && g_rec.gt.scol_off[g] == so);
                    qo += c.K * ((c.rows[g] + 1) / 2), so += c.K * ((c.rows[g] + 15) / 16);
                }
            }
            EXPECT(MX_OK, mx_absmax_bf16_grouped(P(0), c.K, c.rows, c.G, P<float>(1), 0));
        }
    }
    // malformed group lists
    const int64_t neg[2] = {16, -16}, huge[2] = {16, kBig}, over[2] = {kDim, 16},
                  over1[2] = {kDim, 1}, empty[3] = {0, 0, 0}, wrap[3] = {kBig - 15, kBig - 15, 48},
                  neg1[2] = {17, -1};
    struct Bad { const int64_t *rows; int G; } bads[] = {
        {neg, 2}, {huge, 2}, {over, 2}, {over1, 2}, {empty, 3}, {wrap, 3}, {full, 65}, {full, 0},
        {full, -1}, {nullptr, 2}, {neg1, 2}};
    for (auto &b : bads) {
        const mx_status want = b.rows ? MX_ERR_SHAPE : MX_ERR_NULL;
        EXPECT(want, mx_quantize_grouped(P(0), nullptr, 256, b.rows, b.G, both, 0, qr, sr, qc, sc,
                                         nullptr, nullptr, 0, 0));
        EXPECT(want, mx_quantize_gated_grouped(P(0), 256, b.rows, b.G, both, 1, qr, sr, qc, sc, 0));
        EXPECT(want, nvfp4_quantize_transpose_grouped(P(0), 256, b.rows, b.G, P<float>(1), 0, both,
                                                      qr, sr, qc, sc, nullptr, 0));
        EXPECT(want, mx_absmax_bf16_grouped(P(0), 256, b.rows, b.G, P<float>(1), 0));
        CHECK(mx_quantize_grouped_workspace_size(256, b.rows, b.G, both, MX_FUSE_DBIAS) == 0);
        CHECK(mx_grouped_scale_size(256, b.rows, b.G, both, 0) == 0);
    }
    // row counts that are not multiples of 16: the tiled kernels' variants
    // whose transposed rows start at any byte (the plain grouped kernel for
    // the row-wise output alone)
    const int64_t odd[2] = {16, 8};
    EXPECT(MX_OK, nvfp4_quantize_transpose_grouped(P(0), 256, odd, 2, P<float>(1), 0, both, qr, sr,
                                                   qc, sc, nullptr, 0));
    CHECK(g_rec.kind == mxk::kLaunchNvRagged && g_rec.gt.qcol_off[1] == 256 * 8 &&
          g_rec.gt.scol_off[1] == 256);
    EXPECT(MX_OK, mx_absmax_bf16_grouped(P(0), 256, odd, 2, P<float>(1), 0));
    EXPECT(MX_OK, mx_quantize_grouped(P(0), nullptr, 256, odd, 2, both, 0, qr, sr, qc, sc, nullptr,
                                      nullptr, 0, 0));
    CHECK(g_rec.kind == mxk::kLaunchMxRagged);
    EXPECT(MX_OK, mx_quantize_grouped(P(0), nullptr, 256, odd, 2, MX_ROWWISE, 0, qr, sr, nullptr,
                                      nullptr, nullptr, nullptr, 0, 0));
    CHECK(g_rec.kind == mxk::kLaunchMxGrouped);
    EXPECT(MX_OK, mx_quantize_grouped(P(0), nullptr, 252, odd, 2, both, 0, qr, sr, qc, sc, nullptr,
                                      nullptr, 0, 0));
    CHECK(g_rec.kind == mxk::kLaunchMxAny);
    for (int64_t K : {kBig, int64_t(0), int64_t(-16), kDim + 16, INT64_MIN}) {
        EXPECT(MX_ERR_SHAPE, mx_quantize_grouped(P(0), nullptr, K, moe, 8, both, 0, qr, sr, qc, sc,
                                                 nullptr, nullptr, 0, 0));
        EXPECT(MX_ERR_SHAPE, nvfp4_quantize_transpose_grouped(P(0), K, moe, 8, P<float>(1), 0, both,
                                                              qr, sr, qc, sc, nullptr, 0));
        EXPECT(MX_ERR_SHAPE, mx_absmax_bf16_grouped(P(0), K, moe, 8, P<float>(1), 0));
        CHECK(mx_grouped_scale_size(K, moe, 8, both, 1) == 0);
    }
    EXPECT(MX_ERR_ENUM, nvfp4_quantize_transpose_grouped(P(0), 256, moe, 8, P<float>(1), 2, both, qr,
                                                         sr, qc, sc, nullptr, 0));
}

static void nvfp4_cases()
{
    const unsigned both = MX_ROWWISE | MX_COLWISE;
    uint8_t *qr = P(2), *sr = P(3), *qc = P(4), *sc = P(5);
    // multiples of 16 take the tiled kernel, any other shape the any-shape kernel
    const int64_t ok[][2] = {{16384, 16384}, {kDim, 1 << 17}, {16, kDim}, {kDim, 16}, {16400, 7168},
                             {8, 16}, {16, 8}, {1, 1}, {kDim, 1}, {1, kDim}, {16383, 16383},
                             {kDim - 1, (1 << 17) - 1}};
    for (auto &s : ok) {
        // K not a multiple of 16: the any-shape kernel; M not a multiple of
        // 16 (with the transposed output): the tiled kernel's ragged variant
        const bool any = s[1] % 16 != 0;
        const bool rag = !any && s[0] % 16 != 0;
        for (int two_d : {0, 1}) {
            EXPECT(MX_OK, (two_d ? nvfp4_quantize_transpose_2d : nvfp4_quantize_transpose)(
                              P(0), s[0], s[1], P<float>(1), both, qr, sr, qc, sc, P<float>(6), 0));
            const mxk::Nv4Args &a = g_rec.nv;
            CHECK(a.M == s[0] && a.K == s[1] && g_rec.two_d == (two_d != 0));
            CHECK(g_rec.kind == (any ? mxk::kLaunchNvAny : rag ? mxk::kLaunchNvRagged : mxk::kLaunchNv));
            if (rag) {
                const mxk::GroupTable &gt = g_rec.gt;
                CHECK(a.tiles_m == ceil_div(s[0], mxk::kTileM) && a.tiles_k == ceil_div(s[1], mxk::kTileK));
                CHECK(a.group % 2 == 0 && a.group <= mxk::kMaxNvRagGroup || a.group >= a.tiles_m);
                CHECK(gt.count == 1 && gt.row0[1] == s[0] && gt.walk0[1] == a.groups_m &&
                      gt.len[0] == a.group && a.groups_m == ceil_div(a.tiles_m, a.group));
                CHECK(gt.qcol_off[0] == 0 && gt.scol_off[0] == 0);
                CHECK((int64_t)a.groups_m * a.tiles_k <= INT32_MAX);
                EXPECT(MX_OK, nvfp4_quantize_transpose(P(0), s[0], s[1], P<float>(1), MX_ROWWISE, qr, sr,
                                                       nullptr, nullptr, nullptr, 0));
                CHECK(g_rec.kind == mxk::kLaunchNv);
            }
            if (any) {
                const mxk::GroupTable &gt = g_rec.gt;
                CHECK(a.tiles_m == ceil_div(s[0], mxk::kAnyTileM) &&
                      a.tiles_k == ceil_div(s[1], mxk::kAnyTileK));
                CHECK(gt.count == 1 && gt.row0[1] == s[0] && gt.walk0[1] == a.groups_m &&
                      gt.len[0] == a.group && a.group >= 1 && a.group <= mxk::kAnyMaxWalk);
                CHECK(gt.qcol_off[0] == 0 && gt.scol_off[0] == 0);
                CHECK((int64_t)a.groups_m * a.tiles_k <= INT32_MAX);
            } else {
                check_plan(s[0], s[1], a.tiles_m, a.tiles_k, a.group, a.groups_m, false);
            }
        }
        EXPECT(MX_OK, mx_absmax_bf16(P(0), s[0] * s[1], P<float>(1), 0));
    }
    // outputs sized [rows][ceil(cols/2)] and [rows][ceil(cols/16)]: q_col of a
    // 31 x 9 tensor is 9 * 16 bytes, so an s_col 144 bytes after it is
    // disjoint and one 128 bytes after it overlaps
    EXPECT(MX_OK, nvfp4_quantize_transpose(P(0), 31, 9, P<float>(1), both, qr, sr, P(4), P(4, 144),
                                           nullptr, 0));
    EXPECT(MX_ERR_ALIAS, nvfp4_quantize_transpose(P(0), 31, 9, P<float>(1), both, qr, sr, P(4),
                                                  P(4, 128), nullptr, 0));
    const int64_t bad[][2] = {{0, 16}, {16, 0}, {kDim + 16, 16}, {kDim, (1 << 17) + 16}, {kBig, kBig},
                              {-16, 16}, {16, INT64_MIN}, {int64_t(1) << 62, int64_t(1) << 62},
                              {kDim + 1, 1}, {kDim, (1 << 17) + 1}};
    for (auto &s : bad)
        for (int two_d : {0, 1})
            EXPECT(MX_ERR_SHAPE, (two_d ? nvfp4_quantize_transpose_2d : nvfp4_quantize_transpose)(
                                     P(0), s[0], s[1], P<float>(1), both, qr, sr, qc, sc, nullptr, 0));
    EXPECT(MX_ERR_ENUM, nvfp4_quantize_transpose(P(0), 16, 16, P<float>(1), 4, qr, sr, qc, sc, nullptr, 0));
    EXPECT(MX_ERR_NULL, nvfp4_quantize_transpose(P(0), 16, 16, nullptr, both, qr, sr, qc, sc, nullptr, 0));
    EXPECT(MX_ERR_ALIGN, nvfp4_quantize_transpose(P(0), 16, 16, P<float>(1, 2), both, qr, sr, qc, sc,
                                                  nullptr, 0));
    EXPECT(MX_ERR_ALIAS, nvfp4_quantize_transpose(P(0), 16, 16, P<float>(1), both, qr, sr, qc, sc,
                                                  P<float>(1), 0));
    for (int64_t n : {int64_t(0), int64_t(-1), kBig, INT64_MIN, (int64_t(1) << 40) + 1})
        EXPECT(MX_ERR_SHAPE, mx_absmax_bf16(P(0), n, P<float>(1), 0));
    EXPECT(MX_OK, mx_absmax_bf16(P(0), 7, P<float>(1), 0));   // any count of elements
    EXPECT(MX_OK, mx_absmax_bf16(P(0), int64_t(1) << 40, P<float>(1), 0));
    EXPECT(MX_ERR_ALIAS, mx_absmax_bf16(P(0), 1024, P<float>(0, 2044), 0));
}

int main()
{
    CHECK(mx_abi_version() == MXCAST_ABI_VERSION);
    for (int s : {-1, 0, 1, 8, 9, INT32_MAX, INT32_MIN})
        CHECK(mx_status_str(s) != nullptr);
    mx_quantize_cases();
    gated_cases();
    grouped_cases();
    nvfp4_cases();
    printf("%d checks, %d failed\n", checks, failures);
    return failures ? 1 : 0;
}
