// api.cpp -- the extern "C" entry points of libmxcast (declared and
// documented in include/mxcast.h): argument validation on the host, then one
// or two kernel launches on the caller's stream.  Validation is pure host
// code that runs before any HIP call, so a rejected call touches neither the
// device nor the runtime.

#include "mxcast.h"

#include <stdint.h>

#include "launch.h"

namespace {

// Largest row count and row length (in elements, for a gated input the full
// [gate | linear] row): the kernels address a 128-row sub-tile, and a strip
// of 256 transposed rows, with 32-bit byte offsets from its first element.
constexpr int64_t kMaxDim = int64_t(1) << 23;
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Span {
    const void *p;
    uint64_t n;   // bytes
};

bool overlap(const Span &a, const Span &b)
{
    if (!a.p || !b.p || a.n == 0 || b.n == 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Every output must be disjoint from every input and from every other output.
bool any_alias(const Span *in, int nin, const Span *out, int nout)
{
    for (int i = 0; i < nout; i++) {
        for (int j = 0; j < nin; j++)
            if (overlap(out[i], in[j]))
                return true;
        for (int j = i + 1; j < nout; j++)
            if (overlap(out[i], out[j]))
                return true;
    }
    return false;
}

int tiles(int64_t n, int64_t t) { return (int)((n + t - 1) / t); }

// Kernel op of an mx_quantize pre-op.
int cast_op(int pre)
{
    return pre == MX_FUSE_GELU ? mxk::OP_GELU : pre == MX_FUSE_DGELU ? mxk::OP_DGELU
         : pre == MX_FUSE_DSILU ? mxk::OP_DSILU : mxk::OP_PLAIN;
}

// Sub-tiles per walk of the cast kernel `op`: with the GEMM-ready scale
// layout a walk covers at least two sub-tiles, so that it starts on a
// column-scale tile boundary (8 blocks = 256 rows) and no two workgroups
// write one scale tile.
// rag: the transposed rows start at any byte (the transposed output of a
// tensor whose M is not a multiple of 16), which caps walks at kMaxRagGroup.
int walk_group(int tm, int tk, int op, bool dbias, bool tiled, bool rag)
{
    const int max_len = rag ? mxk::kMaxRagGroup : mxk::kMaxGroup;
    if (op == mxk::OP_PLAIN && !dbias) {
        // the plain cast: balanced walks on two resident workgroups per CU
        int len;
        mxk::plan_walks(&tm, 1, tk, mxk::kTargetWorkgroups, tiled, &len, max_len);
        return len;
    }
    const int g = mxk::pick_group(tm, tk, mxk::target_workgroups(op, dbias), max_len);
    return tiled && g < 2 ? 2 : g;
}

// Whether the tiled kernel's cast of an M x K tensor with these outputs
// writes transposed rows that start at any byte.
bool rag_rows(int64_t M, unsigned axis_mask) { return (axis_mask & MX_COLWISE) && M % 16 != 0; }

// Walks along M of the cast kernel `op` (with or without dbias) for an
// M x K tensor.
int walks_m(int64_t M, int64_t K, int op, bool dbias, bool tiled, bool rag)
{
    const int tm = tiles(M, mxk::kTileM), tk = tiles(K, mxk::kTileK);
    const int g = walk_group(tm, tk, op, dbias, tiled, rag);
    return (tm + g - 1) / g;
}

size_t dbias_workspace(int64_t M, int64_t K, int op, bool tiled, bool rag)
{
    return (size_t)walks_m(M, K, op, true, tiled, rag) * (size_t)K * sizeof(float);
}

void set_walk(mxk::MxArgs &a, int op, bool dbias, bool rag)
{
    a.tiles_k = tiles(a.K, mxk::kTileK);
    a.tiles_m = tiles(a.M, mxk::kTileM);
    a.group = walk_group(a.tiles_m, a.tiles_k, op, dbias, a.tiled != 0, rag);
    a.groups_m = (a.tiles_m + a.group - 1) / a.group;
}

// Bytes of the scales of a quantised [rows][cols] tensor blocked along cols:
// compact [rows][ceil(cols / 32)], or whole 32-row x 8-block tiles of 256
// bytes.
uint64_t scale_bytes(int64_t rows, int64_t cols, bool tiled)
{
    const int64_t blocks = (cols + 31) / 32;
    if (!tiled)
        return (uint64_t)(rows * blocks);
    return (uint64_t)(((rows + 31) / 32) * ((blocks + 7) / 8) * 256);
}

// Sizes of an MXFP8 cast: any positive M and K up to the limits; blocks at
// the right and bottom edges may be partial.
bool mx_size_ok(int64_t M, int64_t K)
{
    return M > 0 && K > 0 && M <= kMaxDim && K <= kMaxDim && M * K <= kMaxElems;
}

// Row lengths the tiled cast kernel takes: every row of the bf16 input starts
// on a 16-byte boundary and every row of q_row on an 8-byte one (K a multiple
// of 8), for any M.  With the transposed output and M not a multiple of 16,
// the rows of q_col start at any byte: the grouped kernel's variant for that
// writes them.  Other row lengths go to the any-shape kernel.
bool tiled_width(int64_t K) { return K % 8 == 0; }

// Group table of the any-shape kernel for one M x K tensor.
mxk::GroupTable any_table(int64_t M, int64_t K)
{
    mxk::GroupTable gt{};
    gt.count = 1;
    gt.len[0] = mxk::any_walk_len(&M, 1, K);
    gt.walk0[0] = 0;
    gt.walk0[1] = tiles(tiles(M, mxk::kAnyTileM), gt.len[0]);
    gt.row0[0] = 0;
    gt.row0[1] = M;
    gt.srow_off[0] = gt.scol_off[0] = 0;
    return gt;
}

// Bytes of dbias partials for one M x K tensor (either kernel).
size_t quantize_workspace(int64_t M, int64_t K, int op, bool tiled, unsigned axis_mask)
{
    if (!tiled_width(K))
        return (size_t)any_table(M, K).walk0[1] * (size_t)K * sizeof(float);
    return dbias_workspace(M, K, op, tiled, rag_rows(M, axis_mask));
}

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// Group table of a grouped cast: walks per group (the walk length chosen for
// the whole stack, at least two sub-tiles with tiled scales), rows, and each
// group's scale offsets.  False if a group size is invalid.  any is set when
// the stack goes to the any-shape kernel: the row length is not aligned for
// the tiled kernel (width_aligned false); the walks are then that kernel's.
// rag is set when the transposed output (col) is written and some group's
// rows are not a multiple of 16, so that the groups' transposed rows may
// start at any byte; walks are then at most kMaxRagGroup sub-tiles.
bool build_groups(const int64_t *rows, int G, int64_t K, int op, bool dbias, bool tiled,
                  bool width_aligned, bool col, mxk::GroupTable &gt, int64_t &M, int &group,
                  bool &any, bool &rag)
{
    if (!rows || G < 1 || G > mxk::kMaxGroups)
        return false;
    M = 0;
    bool rows16 = true;
    for (int g = 0; g < G; g++) {
        if (rows[g] < 0 || rows[g] > kMaxDim)
            return false;
        rows16 = rows16 && rows[g] % 16 == 0;
        M += rows[g];
    }
    if (M <= 0 || M > kMaxDim || !mx_size_ok(M, K))
        return false;
    any = !width_aligned;
    rag = !rows16 && col;
    const int max_len = rag ? mxk::kMaxRagGroup : mxk::kMaxGroup;
    int tm[mxk::kMaxGroups];
    for (int g = 0; g < G; g++)
        tm[g] = tiles(rows[g], any ? mxk::kAnyTileM : mxk::kTileM);
    gt = mxk::GroupTable{};
    if (any) {
        group = mxk::any_walk_len(rows, G, K);
    } else if (mxk::target_workgroups(op, dbias) == mxk::kTargetWorkgroupsFused) {
        // the casts bound by their arithmetic (fused pre-ops and gated casts
        // without dbias): walks of one sub-tile (two with the tile layout),
        // many short workgroups that the hardware hands out as others finish,
        // so that every CU stays busy to the end (measured on the 8-expert
        // gated backward: dSwiGLU 200 -> 148 us, dGeGLU 191 -> 138 us)
        group = tiled ? 2 : 1;
    } else {
        group = mxk::pick_group_rounds(tm, G, tiles(K, mxk::kTileK), 2, tiled ? 2 : 1, max_len);
    }
    for (int g = 0; g < G; g++)
        gt.len[g] = group;
    gt.count = G;
    int64_t walks = 0, r = 0, sr = 0, sc = 0;
    for (int g = 0; g < G; g++) {
        gt.walk0[g] = (int)walks;
        gt.row0[g] = r;
        r += rows[g];
        gt.srow_off[g] = sr;
        gt.scol_off[g] = sc;
        walks += (tm[g] + group - 1) / group;
        if (rows[g] > 0) {
            sr += (int64_t)scale_bytes(rows[g], K, tiled);
            sc += (int64_t)scale_bytes(K, rows[g], tiled);
        }
    }
    gt.walk0[G] = (int)walks;
    gt.row0[G] = M;
    return walks > 0;
}

// Group table of a grouped NVFP4 cast or absmax: any group sizes (empty
// groups allowed); walks per group with the walk length of the whole stack.
// any is set when the stack goes to the any-shape kernel: K is not a
// multiple of 16.  rag is set when the transposed output (col) is written and
// some group's rows are not multiples of 16, so that the groups' transposed
// rows may start at any byte; walks are then even, at most kMaxNvRagGroup
// sub-tiles.  Each group's q_col and s_col start after the previous groups'
// [K][ceil(rows/2)] and [K][ceil(rows/16)] bytes.
bool build_nv_groups(const int64_t *rows, int G, int64_t K, bool col, mxk::GroupTable &gt,
                     int64_t &M, int &group, bool &any, bool &rag)
{
    if (!rows || G < 1 || G > mxk::kMaxGroups)
        return false;
    M = 0;
    bool rows16 = true;
    for (int g = 0; g < G; g++) {
        if (rows[g] < 0 || rows[g] > kMaxDim)
            return false;
        rows16 = rows16 && rows[g] % 16 == 0;
        M += rows[g];
    }
    if (M <= 0 || M > kMaxDim || !mx_size_ok(M, K))
        return false;
    any = K % 16 != 0;
    rag = !any && !rows16 && col;
    int tm[mxk::kMaxGroups];
    for (int g = 0; g < G; g++)
        tm[g] = tiles(rows[g], any ? mxk::kAnyTileM : mxk::kTileM);
    gt = mxk::GroupTable{};
    const int tk = tiles(K, mxk::kTileK);
    group = any ? mxk::any_walk_len(rows, G, K)
                : rag ? mxk::pick_group_rounds(tm, G, tk, 2, 2, mxk::kMaxNvRagGroup)
                      : mxk::pick_group_rounds(tm, G, tk, 2, 1);
    for (int g = 0; g < G; g++)
        gt.len[g] = group;
    gt.count = G;
    int64_t walks = 0, r = 0, qc = 0, sc = 0;
    for (int g = 0; g < G; g++) {
        gt.walk0[g] = (int)walks;
        gt.row0[g] = r;
        gt.srow_off[g] = r * ((K + 15) / 16);
        gt.scol_off[g] = sc;
        gt.qcol_off[g] = qc;
        walks += (tm[g] + group - 1) / group;
        r += rows[g];
        qc += K * ((rows[g] + 1) / 2);
        sc += K * ((rows[g] + 15) / 16);
    }
    gt.walk0[G] = (int)walks;
    gt.row0[G] = M;
    return true;
}

// Bytes of NVFP4 outputs: codes [rows][ceil(cols/2)], scales
// [rows][ceil(cols/16)].
uint64_t nv_code_bytes(int64_t rows, int64_t cols) { return (uint64_t)(rows * ((cols + 1) / 2)); }
uint64_t nv_scale_bytes(int64_t rows, int64_t cols) { return (uint64_t)(rows * ((cols + 15) / 16)); }

// Total scale bytes of a grouped cast (the groups' scale tensors one after
// the other).
uint64_t grouped_scale_bytes(const int64_t *rows, int G, int64_t K, bool colwise, bool tiled)
{
    uint64_t n = 0;
    for (int g = 0; g < G; g++)
        if (rows[g] > 0)
            n += colwise ? scale_bytes(K, rows[g], tiled) : scale_bytes(rows[g], K, tiled);
    return n;
}

}  // namespace

// NVFP4 quantize-transpose with 1D (two_d = false) or 16 x 16 block scaling.
// The MXFP8 entry points' axis_mask: at least one of the two axis bits, plus
// optionally the format flags (E5M2 elements, round-up scale rule) and the
// GEMM-ready scale layout flag.
static const unsigned kFmtBits = MX_ELEM_E5M2 | MX_SCALE_ROUND_UP;
static const unsigned kModeBits = 3u | kFmtBits | MX_SCALE_TILED;
static_assert(MX_ELEM_E5M2 == (unsigned)mxk::kFmtE5M2 && MX_SCALE_ROUND_UP == (unsigned)mxk::kFmtRoundUp,
              "format flags are passed to the kernels unchanged");

static bool mx_mode_ok(unsigned axis_mask)
{
    return (axis_mask & 3u) != 0 && (axis_mask & ~kModeBits) == 0;
}

// One tensor (a.M x a.K, everything but the walk set) through the any-shape
// kernel; sets a.tiles_k, a.tiles_m, a.group and a.groups_m to its plan.
static mx_status launch_any(int op, unsigned axis_mask, bool dbias, mxk::MxArgs &a,
                            hipStream_t stream)
{
    const mxk::GroupTable gt = any_table(a.M, a.K);
    a.tiles_k = tiles(a.K, mxk::kAnyTileK);
    a.tiles_m = tiles(a.M, mxk::kAnyTileM);
    a.group = gt.len[0];
    a.groups_m = gt.walk0[1];
    return from_hip(mxk::launch_mx_cast_any(op, axis_mask & 3u, axis_mask & kFmtBits, dbias, a, gt,
                                            stream));
}

// One tensor (a.M x a.K, a.K a multiple of 8, everything but the walk set)
// through the tiled kernel; sets the walk.  With the transposed output and M
// not a multiple of 16 it goes to the variant whose transposed rows start at
// any byte, as a stack of one group.
static mx_status launch_tiled(int op, unsigned axis_mask, bool dbias, mxk::MxArgs &a,
                              hipStream_t stream)
{
    const bool rag = rag_rows(a.M, axis_mask);
    set_walk(a, op, dbias, rag);
    if (!rag)
        return from_hip(mxk::launch_mx_cast(op, axis_mask & 3u, axis_mask & kFmtBits, dbias, a,
                                            stream));
    mxk::GroupTable gt{};
    gt.count = 1;
    gt.len[0] = a.group;
    gt.walk0[0] = 0;
    gt.walk0[1] = a.groups_m;
    gt.row0[0] = 0;
    gt.row0[1] = a.M;
    gt.srow_off[0] = gt.scol_off[0] = 0;
    a.qcol_nt = 0;
    return from_hip(mxk::launch_mx_cast_ragged(op, axis_mask & 3u, axis_mask & kFmtBits, dbias, a,
                                               gt, stream));
}

static mx_status nvfp4_impl(bool two_d, const void *x, int64_t M, int64_t K, const float *amax,
                            unsigned axis_mask, uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                            uint8_t *s_col, float *global_scale_out, hipStream_t stream)
{
    if (axis_mask == 0 || (axis_mask & ~3u))
        return MX_ERR_ENUM;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || !amax || (row && (!q_row || !s_row)) || (col && (!q_col || !s_col)))
        return MX_ERR_NULL;
    if (!mx_size_ok(M, K))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(amax, 4) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))) ||
        (global_scale_out && !aligned(global_scale_out, 4)))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * K);
    const Span in[2] = {{x, 2 * n}, {amax, 4}};
    const Span out[5] = {{row ? q_row : nullptr, nv_code_bytes(M, K)},
                         {row ? s_row : nullptr, nv_scale_bytes(M, K)},
                         {col ? q_col : nullptr, nv_code_bytes(K, M)},
                         {col ? s_col : nullptr, nv_scale_bytes(K, M)},
                         {global_scale_out, 4}};
    if (any_alias(in, 2, out, 5))
        return MX_ERR_ALIAS;

    mxk::Nv4Args a;
    a.x = static_cast<const uint16_t *>(x);
    a.M = M;
    a.K = K;
    a.amax = amax;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.sg_out = global_scale_out;
    if (K % 16 == 0 && M % 16 != 0 && col) {
        // transposed rows at any byte: the tiled kernel's variant for them,
        // the tensor as a stack of one group (even walks of at most
        // kMaxNvRagGroup sub-tiles)
        a.tiles_k = tiles(K, mxk::kTileK);
        a.tiles_m = tiles(M, mxk::kTileM);
        mxk::plan_walks(&a.tiles_m, 1, a.tiles_k, mxk::kTargetWorkgroups, true, &a.group,
                        mxk::kMaxNvRagGroup);
        a.groups_m = (a.tiles_m + a.group - 1) / a.group;
        mxk::GroupTable gt{};
        gt.count = 1;
        gt.len[0] = a.group;
        gt.walk0[1] = a.groups_m;
        gt.row0[1] = M;
        return from_hip(mxk::launch_nvfp4_ragged(axis_mask, two_d, a, gt, stream));
    }
    if (K % 16 != 0) {
        const mxk::GroupTable gt = any_table(M, K);   // offsets 0: one tensor
        a.tiles_k = tiles(K, mxk::kAnyTileK);
        a.tiles_m = tiles(M, mxk::kAnyTileM);
        a.group = gt.len[0];
        a.groups_m = gt.walk0[1];
        return from_hip(mxk::launch_nvfp4_any(axis_mask, two_d, a, gt, stream));
    }
    a.tiles_k = tiles(K, mxk::kTileK);
    a.tiles_m = tiles(M, mxk::kTileM);
    mxk::plan_walks(&a.tiles_m, 1, a.tiles_k, mxk::kTargetWorkgroups, false, &a.group);
    a.groups_m = (a.tiles_m + a.group - 1) / a.group;
    return from_hip(mxk::launch_nvfp4(axis_mask, two_d, a, stream));
}

// The grouped gated casts: group g owns rows r_g .. r_g + rows[g] - 1 of
// x[M][2N] (and of grad[M][N] for the backward); the quantised tensor of a
// group has width W = N (forward) or 2N (backward).
static mx_status gated_grouped_impl(const void *grad, const void *x, int64_t N,
                                    const int64_t *group_rows, int G, unsigned axis_mask, int act,
                                    uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                    hipStream_t stream)
{
    const bool bwd = grad != nullptr;
    if (!mx_mode_ok(axis_mask) || (act != MX_GATED_SWIGLU && act != MX_GATED_GEGLU))
        return MX_ERR_ENUM;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || !group_rows || (row && (!q_row || !s_row)) || (col && (!q_col || !s_col)))
        return MX_ERR_NULL;
    const int op = bwd ? (act == MX_GATED_SWIGLU ? mxk::OP_DSWIGLU : mxk::OP_DGEGLU)
                       : (act == MX_GATED_SWIGLU ? mxk::OP_SWIGLU : mxk::OP_GEGLU);
    if (!mx_size_ok(16, N))   // N <= 2^23 before 2N is formed
        return MX_ERR_SHAPE;
    const int64_t W = bwd ? 2 * N : N;
    const bool tiled = (axis_mask & MX_SCALE_TILED) != 0;
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!build_groups(group_rows, G, W, op, false, tiled, N % 8 == 0, col, gt, M, group, any, rag) ||
        !mx_size_ok(M, 2 * N))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || (bwd && !aligned(grad, 16)) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * N);
    const Span in[2] = {{x, 4 * n}, {bwd ? grad : nullptr, 2 * n}};
    const Span out[4] = {{row ? q_row : nullptr, (uint64_t)(M * W)},
                         {row ? s_row : nullptr, grouped_scale_bytes(group_rows, G, W, false, tiled)},
                         {col ? q_col : nullptr, (uint64_t)(M * W)},
                         {col ? s_col : nullptr, grouped_scale_bytes(group_rows, G, W, true, tiled)}};
    if (any_alias(in, 2, out, 4))
        return MX_ERR_ALIAS;

    mxk::MxArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.aux = bwd ? static_cast<const uint16_t *>(grad) : nullptr;
    a.M = M;
    a.K = W;
    a.ldx = 2 * N;
    a.ldg = bwd ? N : 0;
    a.lin_off = N;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.partials = nullptr;
    a.tiled = tiled;
    a.qcol_nt = 0;
    a.tiles_k = tiles(W, any ? mxk::kAnyTileK : mxk::kTileK);
    a.tiles_m = tiles(M, mxk::kTileM);
    a.group = group;
    a.groups_m = gt.walk0[G];
    if (any)
        return from_hip(mxk::launch_mx_cast_any(op, axis_mask & 3u, axis_mask & kFmtBits, false, a,
                                                gt, stream));
    return from_hip((rag ? mxk::launch_mx_cast_ragged : mxk::launch_mx_cast_grouped)(
        op, axis_mask & 3u, axis_mask & kFmtBits, false, a, gt, stream));
}

extern "C" {

int mx_abi_version(void) { return MXCAST_ABI_VERSION; }

const char *mx_status_str(int s)
{
    switch (s) {
    case MX_OK: return "MX_OK";
    case MX_ERR_NULL: return "MX_ERR_NULL: a required pointer is NULL";
    case MX_ERR_ENUM: return "MX_ERR_ENUM: unknown axis mask, fusion or activation";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE: size not positive or too large";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN: pointer not 16-byte aligned";
    case MX_ERR_WORKSPACE: return "MX_ERR_WORKSPACE: workspace missing or too small";
    case MX_ERR_ALIAS: return "MX_ERR_ALIAS: an output overlaps an input or another output";
    case MX_ERR_HIP: return "MX_ERR_HIP: kernel launch failed";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    default: return "unknown mx_status";
    }
}

size_t mx_quantize_workspace_size(int64_t M, int64_t K, unsigned axis_mask, int fusion)
{
    if (!(fusion & MX_FUSE_DBIAS) || !mx_size_ok(M, K) || !mx_mode_ok(axis_mask) ||
        (fusion & ~0x1F) || (fusion & 0xF) > MX_FUSE_DSILU)
        return 0;
    return quantize_workspace(M, K, cast_op(fusion & 0xF), (axis_mask & MX_SCALE_TILED) != 0,
                              axis_mask);
}

size_t mx_scale_size(int64_t rows, int64_t cols, unsigned axis_mask)
{
    if (rows <= 0 || cols <= 0 || rows > kMaxDim || cols > kMaxDim || !mx_mode_ok(axis_mask))
        return 0;
    return (size_t)scale_bytes(rows, cols, (axis_mask & MX_SCALE_TILED) != 0);
}

static_assert(MX_NOALLOC_SCRATCH_BYTES == mxk::kNoAllocScratchBytes,
              "the header states the scratch size of the allocation-free cast");

// mx_quantize, and with noalloc its allocation-free variant, whose dbias
// partials live in the library's static device scratch instead of a
// caller's workspace.
static mx_status quantize_impl(const void *x, const void *grad, int64_t M, int64_t K,
                               unsigned axis_mask, int fusion, uint8_t *q_row, uint8_t *s_row,
                               uint8_t *q_col, uint8_t *s_col, float *dbias, void *workspace,
                               size_t workspace_bytes, bool noalloc, hipStream_t stream)
{
    const int pre = fusion & 0xF;
    const bool want_dbias = (fusion & MX_FUSE_DBIAS) != 0;
    if (!mx_mode_ok(axis_mask) || (fusion & ~0x1F) || pre > MX_FUSE_DSILU)
        return MX_ERR_ENUM;
    const bool has_grad = pre == MX_FUSE_DGELU || pre == MX_FUSE_DSILU;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || (has_grad && !grad) || (row && (!q_row || !s_row)) ||
        (col && (!q_col || !s_col)) || (want_dbias && !dbias))
        return MX_ERR_NULL;
    if (!mx_size_ok(M, K))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || (has_grad && !aligned(grad, 16)) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))) ||
        (want_dbias && (!aligned(dbias, 4) || (workspace && !aligned(workspace, 16)))))
        return MX_ERR_ALIGN;
    const int op = cast_op(pre);
    const bool tiled = (axis_mask & MX_SCALE_TILED) != 0;
    const size_t need = want_dbias ? quantize_workspace(M, K, op, tiled, axis_mask) : 0;
    if (noalloc ? need > mxk::kNoAllocScratchBytes
                : want_dbias && (!workspace || workspace_bytes < need))
        return MX_ERR_WORKSPACE;
    const uint64_t n = (uint64_t)(M * K);
    const Span in[2] = {{x, 2 * n}, {has_grad ? grad : nullptr, 2 * n}};
    const Span out[6] = {{row ? q_row : nullptr, n}, {row ? s_row : nullptr, scale_bytes(M, K, tiled)},
                         {col ? q_col : nullptr, n}, {col ? s_col : nullptr, scale_bytes(K, M, tiled)},
                         {want_dbias ? dbias : nullptr, 4 * (uint64_t)K},
                         {want_dbias && !noalloc ? workspace : nullptr, need}};
    if (any_alias(in, 2, out, 6))
        return MX_ERR_ALIAS;
    if (want_dbias && noalloc) {
        float *p = nullptr;
        if (mxk::noalloc_scratch(stream, &p) != hipSuccess)
            return MX_ERR_HIP;
        workspace = p;
    }

    mxk::MxArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.aux = has_grad ? static_cast<const uint16_t *>(grad) : nullptr;
    a.M = M;
    a.K = K;
    a.ldx = K;
    a.ldg = K;
    a.lin_off = 0;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.partials = want_dbias ? static_cast<float *>(workspace) : nullptr;
    a.tiled = tiled;
    a.qcol_nt = M * K >= mxk::kQcolNtBytes && M % 128 == 0;
    const mx_status st = tiled_width(K) ? launch_tiled(op, axis_mask, want_dbias, a, stream)
                                        : launch_any(op, axis_mask, want_dbias, a, stream);
    if (st != MX_OK || !want_dbias)
        return st;
    return from_hip(mxk::launch_dbias_reduce(a.partials, a.groups_m, K, dbias, stream));
}

mx_status mx_quantize(const void *x, const void *grad, int64_t M, int64_t K, unsigned axis_mask,
                      int fusion, uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                      float *dbias, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return quantize_impl(x, grad, M, K, axis_mask, fusion, q_row, s_row, q_col, s_col, dbias,
                         workspace, workspace_bytes, false, stream);
}

mx_status mx_quantize_noalloc(const void *x, const void *grad, int64_t M, int64_t K,
                              unsigned axis_mask, int fusion, uint8_t *q_row, uint8_t *s_row,
                              uint8_t *q_col, uint8_t *s_col, float *dbias, hipStream_t stream)
{
    return quantize_impl(x, grad, M, K, axis_mask, fusion, q_row, s_row, q_col, s_col, dbias,
                         nullptr, 0, true, stream);
}

size_t mx_quantize_grouped_workspace_size(int64_t K, const int64_t *group_rows, int G,
                                          unsigned axis_mask, int fusion)
{
    if (!(fusion & MX_FUSE_DBIAS) || !mx_mode_ok(axis_mask) || (fusion & ~0x1F) ||
        (fusion & 0xF) > MX_FUSE_DSILU)
        return 0;
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!build_groups(group_rows, G, K, cast_op(fusion & 0xF), true,
                      (axis_mask & MX_SCALE_TILED) != 0, K % 8 == 0,
                      (axis_mask & MX_COLWISE) != 0, gt, M, group, any, rag))
        return 0;
    return (size_t)gt.walk0[G] * (size_t)K * sizeof(float);
}

size_t mx_grouped_scale_size(int64_t K, const int64_t *group_rows, int G, unsigned axis_mask,
                             int colwise)
{
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!mx_mode_ok(axis_mask) ||
        !build_groups(group_rows, G, K, mxk::OP_PLAIN, false, (axis_mask & MX_SCALE_TILED) != 0,
                      K % 8 == 0, (axis_mask & MX_COLWISE) != 0, gt, M, group, any, rag))
        return 0;
    return (size_t)grouped_scale_bytes(group_rows, G, K, colwise != 0,
                                       (axis_mask & MX_SCALE_TILED) != 0);
}

mx_status mx_quantize_grouped(const void *x, const void *grad, int64_t K, const int64_t *group_rows,
                              int G, unsigned axis_mask, int fusion, uint8_t *q_row,
                              uint8_t *s_row, uint8_t *q_col, uint8_t *s_col, float *dbias,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int pre = fusion & 0xF;
    const bool want_dbias = (fusion & MX_FUSE_DBIAS) != 0;
    if (!mx_mode_ok(axis_mask) || (fusion & ~0x1F) || pre > MX_FUSE_DSILU)
        return MX_ERR_ENUM;
    const bool has_grad = pre == MX_FUSE_DGELU || pre == MX_FUSE_DSILU;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || !group_rows || (has_grad && !grad) || (row && (!q_row || !s_row)) ||
        (col && (!q_col || !s_col)) || (want_dbias && !dbias))
        return MX_ERR_NULL;
    const int op = cast_op(pre);
    const bool tiled = (axis_mask & MX_SCALE_TILED) != 0;
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!build_groups(group_rows, G, K, op, want_dbias, tiled, K % 8 == 0, col, gt, M, group, any,
                      rag))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || (has_grad && !aligned(grad, 16)) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))) ||
        (want_dbias && (!aligned(dbias, 4) || (workspace && !aligned(workspace, 16)))))
        return MX_ERR_ALIGN;
    const size_t need = want_dbias ? (size_t)gt.walk0[G] * (size_t)K * sizeof(float) : 0;
    if (want_dbias && (!workspace || workspace_bytes < need))
        return MX_ERR_WORKSPACE;
    const uint64_t n = (uint64_t)(M * K);
    const Span in[2] = {{x, 2 * n}, {has_grad ? grad : nullptr, 2 * n}};
    const Span out[6] = {{row ? q_row : nullptr, n},
                         {row ? s_row : nullptr, grouped_scale_bytes(group_rows, G, K, false, tiled)},
                         {col ? q_col : nullptr, n},
                         {col ? s_col : nullptr, grouped_scale_bytes(group_rows, G, K, true, tiled)},
                         {want_dbias ? dbias : nullptr, 4 * (uint64_t)K * (uint64_t)G},
                         {want_dbias ? workspace : nullptr, need}};
    if (any_alias(in, 2, out, 6))
        return MX_ERR_ALIAS;

    mxk::MxArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.aux = has_grad ? static_cast<const uint16_t *>(grad) : nullptr;
    a.M = M;
    a.K = K;
    a.ldx = K;
    a.ldg = K;
    a.lin_off = 0;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.partials = want_dbias ? static_cast<float *>(workspace) : nullptr;
    a.tiled = tiled;
    a.qcol_nt = 0;   // groups' transposed rows rarely fill whole lines
    a.tiles_k = tiles(K, any ? mxk::kAnyTileK : mxk::kTileK);
    a.tiles_m = tiles(M, mxk::kTileM);
    a.group = group;
    a.groups_m = gt.walk0[G];
    const auto launch = any ? mxk::launch_mx_cast_any
                            : rag ? mxk::launch_mx_cast_ragged : mxk::launch_mx_cast_grouped;
    mx_status st = from_hip(
        launch(op, axis_mask & 3u, axis_mask & kFmtBits, want_dbias, a, gt, stream));
    if (st != MX_OK || !want_dbias)
        return st;
    return from_hip(mxk::launch_dbias_reduce_grouped(a.partials, gt, K, dbias, stream));
}

mx_status mx_quantize_gated_grouped(const void *x, int64_t N, const int64_t *group_rows, int G,
                                    unsigned axis_mask, int act, uint8_t *q_row, uint8_t *s_row,
                                    uint8_t *q_col, uint8_t *s_col, hipStream_t stream)
{
    return gated_grouped_impl(nullptr, x, N, group_rows, G, axis_mask, act, q_row, s_row, q_col,
                              s_col, stream);
}

mx_status mx_quantize_dgated_grouped(const void *grad, const void *x, int64_t N,
                                     const int64_t *group_rows, int G, unsigned axis_mask, int act,
                                     uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                     uint8_t *s_col, hipStream_t stream)
{
    if (!grad)
        return MX_ERR_NULL;
    return gated_grouped_impl(grad, x, N, group_rows, G, axis_mask, act, q_row, s_row, q_col,
                              s_col, stream);
}

mx_status mx_quantize_gated(const void *x, int64_t M, int64_t N, unsigned axis_mask, int act,
                            uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                            hipStream_t stream)
{
    if (!mx_mode_ok(axis_mask) || (act != MX_GATED_SWIGLU && act != MX_GATED_GEGLU))
        return MX_ERR_ENUM;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || (row && (!q_row || !s_row)) || (col && (!q_col || !s_col)))
        return MX_ERR_NULL;
    if (!mx_size_ok(M, N) || !mx_size_ok(M, 2 * N))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * N);
    const bool tiled = (axis_mask & MX_SCALE_TILED) != 0;
    const Span in[1] = {{x, 4 * n}};
    const Span out[4] = {{row ? q_row : nullptr, n}, {row ? s_row : nullptr, scale_bytes(M, N, tiled)},
                         {col ? q_col : nullptr, n}, {col ? s_col : nullptr, scale_bytes(N, M, tiled)}};
    if (any_alias(in, 1, out, 4))
        return MX_ERR_ALIAS;

    mxk::MxArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.aux = nullptr;
    a.M = M;
    a.K = N;
    a.ldx = 2 * N;
    a.ldg = 0;
    a.lin_off = N;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.partials = nullptr;
    a.tiled = tiled;
    a.qcol_nt = 0;
    const int op = act == MX_GATED_SWIGLU ? mxk::OP_SWIGLU : mxk::OP_GEGLU;
    return tiled_width(N) ? launch_tiled(op, axis_mask, false, a, stream)
                          : launch_any(op, axis_mask, false, a, stream);
}

mx_status mx_quantize_dgated(const void *grad, const void *x, int64_t M, int64_t N,
                             unsigned axis_mask, int act, uint8_t *q_row, uint8_t *s_row,
                             uint8_t *q_col, uint8_t *s_col, hipStream_t stream)
{
    if (!mx_mode_ok(axis_mask) || (act != MX_GATED_SWIGLU && act != MX_GATED_GEGLU))
        return MX_ERR_ENUM;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!grad || !x || (row && (!q_row || !s_row)) || (col && (!q_col || !s_col)))
        return MX_ERR_NULL;
    if (!mx_size_ok(M, N) || !mx_size_ok(M, 2 * N))
        return MX_ERR_SHAPE;
    if (!aligned(grad, 16) || !aligned(x, 16) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * N);
    const bool tiled = (axis_mask & MX_SCALE_TILED) != 0;
    const Span in[2] = {{grad, 2 * n}, {x, 4 * n}};
    const Span out[4] = {{row ? q_row : nullptr, 2 * n},
                         {row ? s_row : nullptr, scale_bytes(M, 2 * N, tiled)},
                         {col ? q_col : nullptr, 2 * n},
                         {col ? s_col : nullptr, scale_bytes(2 * N, M, tiled)}};
    if (any_alias(in, 2, out, 4))
        return MX_ERR_ALIAS;

    mxk::MxArgs a;
    a.x = static_cast<const uint16_t *>(x);
    a.aux = static_cast<const uint16_t *>(grad);
    a.M = M;
    a.K = 2 * N;
    a.ldx = 2 * N;
    a.ldg = N;
    a.lin_off = N;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.partials = nullptr;
    a.tiled = tiled;
    a.qcol_nt = 0;
    const int op = act == MX_GATED_SWIGLU ? mxk::OP_DSWIGLU : mxk::OP_DGEGLU;
    // the tiled kernel needs both halves 8-column aligned
    return tiled_width(N) ? launch_tiled(op, axis_mask, false, a, stream)
                          : launch_any(op, axis_mask, false, a, stream);
}

mx_status mx_fused_values(const void *x, const void *grad, int64_t M, int64_t K, int op, void *y,
                          hipStream_t stream)
{
    int kop;
    switch (op) {
    case MX_FUSE_GELU: kop = mxk::OP_GELU; break;
    case MX_FUSE_DGELU: kop = mxk::OP_DGELU; break;
    case MX_OP_GATED | MX_GATED_SWIGLU: kop = mxk::OP_SWIGLU; break;
    case MX_OP_GATED | MX_GATED_GEGLU: kop = mxk::OP_GEGLU; break;
    case MX_FUSE_DSILU: kop = mxk::OP_DSILU; break;
    case MX_OP_DGATED | MX_GATED_SWIGLU: kop = mxk::OP_DSWIGLU; break;
    case MX_OP_DGATED | MX_GATED_GEGLU: kop = mxk::OP_DGEGLU; break;
    default: return MX_ERR_ENUM;
    }
    const bool gated = (op & (MX_OP_GATED | MX_OP_DGATED)) != 0;
    const bool dgated = (op & MX_OP_DGATED) != 0;
    const bool has_grad = kop == mxk::OP_DGELU || kop == mxk::OP_DSILU || dgated;
    if (!x || !y || (has_grad && !grad))
        return MX_ERR_NULL;
    if (!mx_size_ok(M, K) || (gated && !mx_size_ok(M, 2 * K)))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(y, 16) || (has_grad && !aligned(grad, 16)))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * K);
    const Span in[2] = {{x, gated ? 4 * n : 2 * n}, {has_grad ? grad : nullptr, 2 * n}};
    const Span out[1] = {{y, dgated ? 4 * n : 2 * n}};
    if (any_alias(in, 2, out, 1))
        return MX_ERR_ALIAS;
    // the 8-element kernel needs rows of a multiple of 8 elements
    return from_hip((K % 8 == 0 ? mxk::launch_fused_values : mxk::launch_fused_values_any)(
        kop, static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(grad), M, K,
        static_cast<uint16_t *>(y), stream));
}

mx_status mx_absmax_bf16(const void *x, int64_t n, float *amax, hipStream_t stream)
{
    if (!x || !amax)
        return MX_ERR_NULL;
    if (n <= 0 || n > kMaxElems)
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(amax, 4))
        return MX_ERR_ALIGN;
    const Span in[1] = {{x, 2 * (uint64_t)n}};
    const Span out[1] = {{amax, 4}};
    if (any_alias(in, 1, out, 1))
        return MX_ERR_ALIAS;
    return from_hip(mxk::launch_absmax(static_cast<const uint16_t *>(x), n, amax, stream));
}

mx_status nvfp4_quantize_transpose(const void *x, int64_t M, int64_t K, const float *amax,
                                   unsigned axis_mask, uint8_t *q_row, uint8_t *s_row,
                                   uint8_t *q_col, uint8_t *s_col, float *global_scale_out,
                                   hipStream_t stream)
{
    return nvfp4_impl(false, x, M, K, amax, axis_mask, q_row, s_row, q_col, s_col,
                      global_scale_out, stream);
}

mx_status mx_absmax_bf16_grouped(const void *x, int64_t K, const int64_t *group_rows, int G,
                                 float *amax, hipStream_t stream)
{
    if (!x || !amax || !group_rows)
        return MX_ERR_NULL;
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!build_nv_groups(group_rows, G, K, false, gt, M, group, any, rag))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(amax, 4))
        return MX_ERR_ALIGN;
    const Span in[1] = {{x, 2 * (uint64_t)(M * K)}};
    const Span out[1] = {{amax, 4 * (uint64_t)G}};
    if (any_alias(in, 1, out, 1))
        return MX_ERR_ALIAS;
    return from_hip(mxk::launch_absmax_grouped(static_cast<const uint16_t *>(x), K, gt, amax,
                                               stream));
}

mx_status nvfp4_quantize_transpose_grouped(const void *x, int64_t K, const int64_t *group_rows,
                                           int G, const float *amax, int scaling_2d,
                                           unsigned axis_mask, uint8_t *q_row, uint8_t *s_row,
                                           uint8_t *q_col, uint8_t *s_col,
                                           float *global_scale_out, hipStream_t stream)
{
    if (axis_mask == 0 || (axis_mask & ~3u) || (scaling_2d != 0 && scaling_2d != 1))
        return MX_ERR_ENUM;
    const bool row = axis_mask & MX_ROWWISE, col = axis_mask & MX_COLWISE;
    if (!x || !amax || !group_rows || (row && (!q_row || !s_row)) || (col && (!q_col || !s_col)))
        return MX_ERR_NULL;
    mxk::GroupTable gt;
    int64_t M;
    int group;
    bool any, rag;
    if (!build_nv_groups(group_rows, G, K, col, gt, M, group, any, rag))
        return MX_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(amax, 4) ||
        (row && (!aligned(q_row, 16) || !aligned(s_row, 16))) ||
        (col && (!aligned(q_col, 16) || !aligned(s_col, 16))) ||
        (global_scale_out && !aligned(global_scale_out, 4)))
        return MX_ERR_ALIGN;
    const uint64_t n = (uint64_t)(M * K);
    const Span in[2] = {{x, 2 * n}, {amax, 4 * (uint64_t)G}};
    const Span out[5] = {{row ? q_row : nullptr, nv_code_bytes(M, K)},
                         {row ? s_row : nullptr, nv_scale_bytes(M, K)},
                         {col ? q_col : nullptr, (uint64_t)gt.qcol_off[G - 1] + nv_code_bytes(K, group_rows[G - 1])},
                         {col ? s_col : nullptr, (uint64_t)gt.scol_off[G - 1] + nv_scale_bytes(K, group_rows[G - 1])},
                         {global_scale_out, 4 * (uint64_t)G}};
    if (any_alias(in, 2, out, 5))
        return MX_ERR_ALIAS;

    mxk::Nv4Args a;
    a.x = static_cast<const uint16_t *>(x);
    a.M = M;
    a.K = K;
    a.amax = amax;
    a.q_row = q_row;
    a.s_row = s_row;
    a.q_col = q_col;
    a.s_col = s_col;
    a.sg_out = global_scale_out;
    a.tiles_k = tiles(K, any ? mxk::kAnyTileK : mxk::kTileK);
    a.tiles_m = tiles(M, any ? mxk::kAnyTileM : mxk::kTileM);
    a.group = group;
    a.groups_m = gt.walk0[G];
    if (any)
        return from_hip(mxk::launch_nvfp4_any(axis_mask, scaling_2d != 0, a, gt, stream));
    return from_hip((rag ? mxk::launch_nvfp4_ragged : mxk::launch_nvfp4_grouped)(
        axis_mask, scaling_2d != 0, a, gt, stream));
}

mx_status nvfp4_quantize_transpose_2d(const void *x, int64_t M, int64_t K, const float *amax,
                                      unsigned axis_mask, uint8_t *q_row, uint8_t *s_row,
                                      uint8_t *q_col, uint8_t *s_col, float *global_scale_out,
                                      hipStream_t stream)
{
    return nvfp4_impl(true, x, M, K, amax, axis_mask, q_row, s_row, q_col, s_col,
                      global_scale_out, stream);
}

}  // extern "C"
