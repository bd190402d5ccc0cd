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
// A cast workgroup walks down up to kMaxGroup sub-tiles of a 256-column strip.
constexpr int kMaxGroup = 16;
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
// deepest power of two <= kMaxGroup that still yields `target` workgroups.
inline int pick_group(int tiles_m, int tiles_k, int target)
{
    int g = kMaxGroup;
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
                             int min_group)
{
    const int64_t slots = 256 * (int64_t)slots_per_cu;
    int best = 0;
    int64_t best_cost = 0;
    for (int g = kMaxGroup; g >= min_group; g >>= 1) {
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
    int64_t row0[kMaxGroups + 1];     // first row of each group; row0[count] = M
    int64_t srow_off[kMaxGroups];     // byte offset of each group's row scales
    int64_t scol_off[kMaxGroups];     // byte offset of each group's column scales
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
hipError_t launch_absmax(const uint16_t *x, int64_t n, float *amax, hipStream_t s);
// two_d: one scale per 16 x 16 block instead of per 16 elements of a row.
hipError_t launch_nvfp4(unsigned axis, bool two_d, const Nv4Args &a, hipStream_t s);
hipError_t launch_nvfp4_grouped(unsigned axis, bool two_d, const Nv4Args &a, const GroupTable &gt,
                                hipStream_t s);
hipError_t launch_absmax_grouped(const uint16_t *x, int64_t K, const GroupTable &gt, float *amax,
                                 hipStream_t s);

}  // namespace mxk
