// launch.h -- internal interface between the host API (api.cpp) and the
// kernel translation units.  Not installed; the public ABI is mxcast.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mxk {

// Elementwise pre-op of a cast kernel.
enum Op : int {
    OP_PLAIN = 0, OP_GELU = 1, OP_DGELU = 2, OP_SWIGLU = 3, OP_GEGLU = 4,
    OP_DSILU = 5,                    // dsilu(x) * grad
    OP_DSWIGLU = 6, OP_DGEGLU = 7    // gated backward: [d_gate | d_linear]
};

// MX format variants, as flags (the same bits as the ABI's flags beside the
// axis bits): kFmtE5M2 selects E5M2 elements (bias 15, max 57344 =
// 1.75 * 2^15) instead of E4M3 (max 448 = 1.75 * 2^8); kFmtRoundUp selects
// the round-up E8M0 rule instead of the floor rule.
constexpr int kFmtE5M2 = 4, kFmtRoundUp = 8;

// Workgroup tile of the cast kernels.  A lane owns 16 rows x 8 columns; the
// two halves of a wave (lanes 0-31, 32-63) own rows 0-15 and 16-31 of the
// same 256 columns, so a wave covers 32 rows (one MXFP8 column block) and a
// workgroup of 4 waves covers 128 rows x 256 columns.
constexpr int kRowsPerLane = 16;
constexpr int kColsPerLane = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileM = 2 * kRowsPerLane * kWaves;  // 128
constexpr int kTileK = kColsPerLane * 32;          // 256
// A cast workgroup walks down up to kMaxGroup sub-tiles of a 256-column strip;
// up to kMaxRagGroup when its transposed rows start at any byte (its stage
// then holds two sub-tiles, and the walk's column scales must still fit two
// workgroups' LDS into a CU's 160 KB).
constexpr int kMaxGroup = 16;
constexpr int kMaxRagGroup = 14;
// The same for the NVFP4 cast (its stage holds two pairs of sub-tiles, and
// walks are even there so that each pair lies in one walk).
constexpr int kMaxNvRagGroup = 4;
// Workgroups the host aims to launch at least: two per MI355X compute unit
// for the plain cast (bound by memory, two resident per CU) and for the casts
// with dbias; four for the other fused casts (bound by their arithmetic,
// three resident per CU; more workgroups than slots keep every CU busy to
// the end).  Chosen by measurement on the 8192^2 and 16384^2 workloads.
constexpr int kTargetWorkgroups = 512;
constexpr int kTargetWorkgroupsFused = 1024;

inline int target_workgroups(int op, bool dbias)
{
    return op == OP_PLAIN || dbias ? kTargetWorkgroups : kTargetWorkgroupsFused;
}

// Sub-tiles per workgroup for a tiles_m x tiles_k grid of sub-tiles: the
// deepest power of two <= max_len that still yields `target` workgroups.
inline int pick_group(int tiles_m, int tiles_k, int target, int max_len = kMaxGroup)
{
    int g = 1;
    while (2 * g <= max_len)
        g *= 2;
    while (g > 1 && (int64_t)((tiles_m + g - 1) / g) * tiles_k < target)
        g >>= 1;
    return g;
}

// Sub-tiles per walk for groups of the given sub-tile row counts (the
// grouped casts): every group's walks end at its last sub-tile, so short
// groups leave partial walks, and the launch may need a last, nearly empty
// round of workgroups.  Among the walk lengths that fill at least 3/4 of the
// resident slots (slots_per_cu x 256 CUs) in the first round, take the one
// with the fewest estimated sub-tile steps, rounds x (walk + 1) (the 1 is a
// walk's fixed cost: its first load and its scale flush); ties go to the
// longer walk.  Reproduces pick_group's choice on the one-group workloads it
// was tuned on.
inline int pick_group_rounds(const int *tiles_m, int groups, int tiles_k, int slots_per_cu,
                             int min_group, int max_len = kMaxGroup)
{
    const int64_t slots = 256 * (int64_t)slots_per_cu;
    int best = 0;
    int64_t best_cost = 0;
    int top = 1;
    while (2 * top <= max_len)
        top *= 2;
    for (int g = top; g >= min_group; g >>= 1) {
        int64_t walks = 0;
        for (int i = 0; i < groups; i++)
            walks += (tiles_m[i] + g - 1) / g;
        const int64_t jobs = walks * tiles_k;
        if (4 * jobs < 3 * slots && g > min_group)
            continue;
        const int64_t cost = (jobs + slots - 1) / slots * (g + 1);
        if (best == 0 || cost < best_cost) {
            best = g;
            best_cost = cost;
        }
    }
    return best;
}

// Walk lengths for tensors (groups) of tiles_m[g] sub-tile rows, each cast
// in walks over all tiles_k strips, on `slots` resident workgroups (used for
// the plain MXFP8 and NVFP4 casts of one tensor; measured on the grouped
// workloads, whose short groups gain more from many short walks that the
// hardware hands out as workgroups finish, pick_group_rounds is better).  A
// target length L (1 .. kMaxGroup; even with `even`, which the GEMM-ready
// scale layout needs) gives group g the walks of balanced length
// len[g] = ceil(t / ceil(t / L)) (t = tiles_m[g]; rounded up to even), so a
// group's last walk is never much shorter than the rest.  Among the targets,
// take the one with the fewest estimated steps, rounds x (longest walk + 1)
// -- rounds of `slots` workgroups, the 1 a walk's fixed cost (its first load
// and its scale flush) -- ties to the longer walks.  For the metric tensor
// (one group of 128 sub-tile rows, 64 strips, 512 slots) this is 16, the
// deepest walk that fills every slot once.
inline void plan_walks(const int *tiles_m, int groups, int tiles_k, int slots, bool even,
                       int *len, int max_len = kMaxGroup)
{
    int best_L = 0, best_long = 0;
    int64_t best_cost = 0;
    for (int L = even ? 2 : 1; L <= max_len; L += even ? 2 : 1) {
        int64_t walks = 0;
        int longest = 0;
        for (int g = 0; g < groups; g++) {
            const int t = tiles_m[g];
            if (t == 0)
                continue;
            int lg = (t + (t + L - 1) / L - 1) / ((t + L - 1) / L);
            if (even)
                lg += lg & 1;
            walks += (t + lg - 1) / lg;
            longest = lg > longest ? lg : longest;
        }
        const int64_t rounds = (walks * tiles_k + slots - 1) / slots;
        const int64_t cost = rounds * (longest + 1);
        if (best_L == 0 || cost < best_cost || (cost == best_cost && longest > best_long)) {
            best_L = L;
            best_cost = cost;
            best_long = longest;
        }
    }
    for (int g = 0; g < groups; g++) {
        const int t = tiles_m[g];
        int lg = t == 0 ? 1 : (t + (t + best_L - 1) / best_L - 1) / ((t + best_L - 1) / best_L);
        if (even)
            lg += lg & 1;
        len[g] = lg;
    }
}

// The cast of any shape (mx_cast_any.hip): a workgroup walks down a
// 128-column strip in steps of 64 rows, up to kAnyMaxWalk steps.
constexpr int kAnyTileM = 64;
constexpr int kAnyTileK = 128;
constexpr int kAnyMaxWalk = 8;
// Workgroups the any-shape cast aims for: four per compute unit (its LDS
// allows four resident).
constexpr int kAnyTargetWorkgroups = 1024;

// Steps per walk of the any-shape cast for groups of the given row counts
// and row length K: the longest of 8, 4, 2, 1 steps that still gives
// kAnyTargetWorkgroups workgroups (1 if none does).
inline int any_walk_len(const int64_t *rows, int groups, int64_t K)
{
    const int64_t tk = (K + kAnyTileK - 1) / kAnyTileK;
    int len = kAnyMaxWalk;
    for (; len > 1; len >>= 1) {
        int64_t walks = 0;
        for (int g = 0; g < groups; g++)
            walks += ((rows[g] + kAnyTileM - 1) / kAnyTileM + len - 1) / len;
        if (walks * tk >= kAnyTargetWorkgroups)
            break;
    }
    return len;
}

struct MxArgs {
    const uint16_t *x;     // input (gated: [M][2N] with the linear half at lin_off)
    const uint16_t *aux;   // grad for dGELU, else unused
    int64_t M, K;          // rows and columns of the quantised tensor
    int64_t ldx;           // row stride of x in elements
    int64_t lin_off;       // gated: column offset of the linear half
    int64_t ldg;           // row stride of aux (grad) in elements
    uint8_t *q_row, *s_row, *q_col, *s_col;
    float *partials;       // dbias: [groups_m][K] fp32 column partial sums
    int tiles_k, tiles_m;  // 128 x 256 sub-tiles along K and M
    int group, groups_m;   // sub-tiles per workgroup walk, walks along M
    int tiled;             // scales in the GEMM-ready tile layout (walks of >= 2 sub-tiles)
    int qcol_nt;           // plain cast with both outputs: transposed stores non-temporal
};

// The plain cast's transposed stores are non-temporal only for a transposed
// output of at least this many bytes with whole 128-byte rows (measured on
// MI355X: below it, and for rows that share cache lines, the default policy
// is faster; above it much slower).
constexpr int64_t kQcolNtBytes = int64_t(1) << 27;

// Grouped cast: groups stacked along M, each cast as a tensor of its own in
// one launch.  Walks never cross a group boundary; walk0 numbers them across
// all groups.
constexpr int kMaxGroups = 64;
struct GroupTable {
    int count;                        // groups
    int walk0[kMaxGroups + 1];        // first walk of each group; walk0[count] = all walks
    int len[kMaxGroups];              // sub-tiles per walk of each group
    int64_t row0[kMaxGroups + 1];     // first row of each group; row0[count] = M
    int64_t srow_off[kMaxGroups];     // byte offset of each group's row scales
    int64_t scol_off[kMaxGroups];     // byte offset of each group's column scales
    int64_t qcol_off[kMaxGroups];     // NVFP4 of any shape: byte offset of each group's q_col
};

struct Nv4Args {
    const uint16_t *x;
    int64_t M, K;
    const float *amax;
    uint8_t *q_row, *s_row, *q_col, *s_col;
    float *sg_out;
    int tiles_k, tiles_m;  // 128 x 256 sub-tiles along K and M
    int group, groups_m;   // sub-tiles per workgroup walk, walks along M
};

// op: 0 plain, 1 GELU, 2 dGELU, 3 SwiGLU, 4 GeGLU.
hipError_t launch_mx_cast(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                          hipStream_t s);
// The same over the groups of gt (one launch); a.M, a.groups_m and the output
// pointers describe the whole stack.
hipError_t launch_mx_cast_grouped(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                                  const GroupTable &gt, hipStream_t s);
// launch_mx_cast_grouped for stacks whose transposed rows may start at any
// byte (a group's rows, or the rows before it, not multiples of 16; K, the
// row length, a multiple of 8); axis must include the column-wise output.
// A single tensor is a stack of one group.
hipError_t launch_mx_cast_ragged(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                                 const GroupTable &gt, hipStream_t s);
// The same operations for any shape (mx_cast_any.hip): a.tiles_k =
// ceil(K / kAnyTileK); gt gives each group's rows, walks (gt.len steps each)
// and scale offsets (one group for a single tensor); a.partials holds
// [gt.walk0[gt.count]][K] dbias partial sums.
hipError_t launch_mx_cast_any(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                              const GroupTable &gt, hipStream_t s);
hipError_t launch_dbias_reduce_grouped(const float *partials, const GroupTable &gt, int64_t K,
                                       float *dbias, hipStream_t s);
hipError_t launch_dbias_reduce(const float *partials, int segments, int64_t K, float *dbias,
                               hipStream_t s);

// Device scratch of the allocation-free cast (mx_quantize_noalloc): a static
// device array of this many bytes per GPU, holding the dbias partial sums.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
// Its address on the device of stream s, looked up once per device.
hipError_t noalloc_scratch(hipStream_t s, float **ptr);
// op as above (1..7); gated ops read x[M][2K]; the gated backward ops read
// grad aux[M][K] and write y[M][2K].
hipError_t launch_fused_values(int op, const uint16_t *x, const uint16_t *aux, int64_t M,
                               int64_t K, uint16_t *y, hipStream_t s);
// launch_fused_values for any M, K (one element per thread).
hipError_t launch_fused_values_any(int op, const uint16_t *x, const uint16_t *aux, int64_t M,
                                   int64_t K, uint16_t *y, hipStream_t s);
hipError_t launch_absmax(const uint16_t *x, int64_t n, float *amax, hipStream_t s);
// two_d: one scale per 16 x 16 block instead of per 16 elements of a row.
hipError_t launch_nvfp4(unsigned axis, bool two_d, const Nv4Args &a, hipStream_t s);
hipError_t launch_nvfp4_grouped(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                                hipStream_t s);
// launch_nvfp4_grouped for stacks whose transposed rows may start at any
// byte (a group's rows, or the rows before it, not multiples of 16; K a
// multiple of 16); axis must include the transposed output; gt holds each
// group's q_col and s_col offsets.  A single tensor is a stack of one group.
hipError_t launch_nvfp4_ragged(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                               hipStream_t s);
hipError_t launch_absmax_grouped(const uint16_t *x, int64_t K, const GroupTable &gt, float *amax,
                                 hipStream_t s);
// NVFP4 of any shape (nvfp4_any.hip): a.tiles_k = ceil(K / kAnyTileK); gt as
// for launch_mx_cast_any, with each group's q_col and s_col offsets.
hipError_t launch_nvfp4_any(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                            hipStream_t s);

}  // namespace mxk
