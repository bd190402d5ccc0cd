// mx_cast_any.hip -- the MXFP8 casts for shapes the tiled kernel (mx_cast.h)
// does not take: any row count and any row length, so that rows of the
// input and of both outputs may start at any byte.  Same operations, same
// arithmetic, bit for bit: the plain cast, the GELU / dGELU / dSiLU pre-ops
// with or without dbias, the gated forward and backward casts, one tensor or
// groups stacked along M (TransformerEngine PR 3291 page, "MXFP8 generic
// quantize kernel" and "MXFP8 gated (swiglu / geglu) kernel"; torchao PR 12
// page for the dim1 cast).  A block at the end of a line that holds fewer
// than 32 elements is quantised from the elements it has.
//
// Layout of the work: a workgroup (4 waves) walks down a 128-column strip in
// steps of 64 rows.  Thread t loads column t % 128 of rows 32 (t / 128) ..
// 32 (t / 128) + 31 with 2-byte loads (a wave instruction reads 128
// contiguous bytes of one row), applies the pre-op, and holds exactly one
// column block: its amax, scale byte and 32 codes need no exchange.  The
// bf16 values also go to LDS, where thread t takes the 32-column row block
// (t % 4) of row t / 4 for the row-wise output.  Codes of both directions
// leave through LDS staging (any_common.h: the aligned dwords of each row,
// the aligned 64-byte chunks of each transposed row); row scales leave per
// step, column scales at the end of the walk.  Each scale byte of the
// GEMM-ready tile layout, padding included, is written by exactly one
// workgroup.  Loads and stores go through buffer resources (bufio.h); lanes
// outside the tensor get the out-of-range offset.

#include "any_common.h"

namespace mxk {

// LDS of one workgroup (37.5 KB: four workgroups per CU).  Row strides are
// multiples of 16 bytes, padded so that the 16-byte accesses of 8
// consecutive lanes fall into different banks.
struct alignas(16) AnyStage {
    // bf16 values of the step (272-byte rows).  Once the row pass has read
    // row r, the first 128 bytes of that row hold row r's codes: the four
    // threads of a row are lanes of one wave, whose reads precede its writes.
    uint16_t y[kAnyTileM][kAnyTileK + 8];
    // transposed codes, two steps per transposed row: step s at bytes
    // 64 (s % 2) .. 64 (s % 2) + 63 (144-byte rows), so that the bytes a
    // step leaves for the next 64-byte-aligned chunk stay next to it
    uint8_t qt[kAnyTileK][2 * kAnyTileM + 16];
    uint8_t sc[kAnyTileK][2 * kAnyMaxWalk];     // column scales of the walk
    float dsum[kAnyTileK];                      // dbias: column sums of rows 32..63
};

__device__ __forceinline__ uint8_t *qrow_stage(AnyStage &st, int r)
{
    return reinterpret_cast<uint8_t *>(st.y[r]);
}
__device__ __forceinline__ const uint8_t *qrow_stage(const AnyStage &st, int r)
{
    return reinterpret_cast<const uint8_t *>(st.y[r]);
}

// One tensor of the launch (the whole input, or one group of a stack).
struct AnyView {
    const uint16_t *x, *aux;
    int64_t M;
    uint8_t *q_row, *s_row, *q_col, *s_col;
};

// Column k of the quantised tensor, rows m .. m + 31 (those at or past the
// tensor's M read as 0), after the pre-op: word i holds rows 2i (low half)
// and 2i + 1 (high half).  A column outside the tensor reads as 0.  Every
// pre-op maps zero operands to +0, so such elements change no amax and no
// column sum.
template <int OP>
__device__ __forceinline__ void any_load(const MxArgs &a, const AnyView &v, int64_t m, int64_t k,
                                         bool col_ok, uint32_t (&w)[16])
{
    if constexpr (OP == OP_DSWIGLU || OP == OP_DGEGLU) {
        // output column k of [d_gate | d_linear] (each half N wide) reads
        // gate and grad at n = k mod N and, in the gate half, linear at N + n
        const int64_t N = a.lin_off;
        const bool gate_half = k < N;
        const uint32_t n2 = (uint32_t)(2 * (gate_half ? k : k - N));
        const uint32_t ox = step_offset(col_ok ? n2 : kDead);
        const uint32_t ol = step_offset(col_ok && gate_half ? n2 : kDead);
        const Rows32 vg = rows32(v.x, m, a.ldx, v.M), vd = rows32(v.aux, m, a.ldg, v.M);
        const Rows32 vl = rows32(v.x, m, a.ldx, v.M, N);
        // two batches of 16 rows: three operands of 32 rows in flight at
        // once would not fit the register budget of four waves per SIMD
#pragma unroll
        for (int r0 = 0; r0 < 32; r0 += 16) {
            uint32_t g[16], dy[16], li[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                g[i] = load_row(vg, r0 + i, ox);
                dy[i] = load_row(vd, r0 + i, ox);
                li[i] = load_row(vl, r0 + i, ol);
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
                w[r0 / 2 + i] = dgated_pair<OP>(pack2(g[2 * i], g[2 * i + 1]),
                                                pack2(dy[2 * i], dy[2 * i + 1]),
                                                pack2(li[2 * i], li[2 * i + 1]), gate_half);
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    const uint32_t ox = step_offset(col_ok ? (uint32_t)(2 * k) : kDead);
    const Rows32 vx = rows32(v.x, m, a.ldx, v.M);
    uint32_t e[32];
#pragma unroll
    for (int i = 0; i < 32; i++)
        e[i] = load_row(vx, i, ox);
    if constexpr (OP == OP_PLAIN) {
#pragma unroll
        for (int i = 0; i < 16; i++)
            w[i] = pack2(e[2 * i], e[2 * i + 1]);
    } else if constexpr (OP == OP_GELU) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t p = pack2(e[2 * i], e[2 * i + 1]);
            w[i] = fused_pair<OP>(p, p);
        }
    } else {
        // second operand: the linear half (gated) or grad (dGELU, dSiLU)
        constexpr bool gated = OP == OP_SWIGLU || OP == OP_GEGLU;
        const Rows32 vb = gated ? rows32(v.x, m, a.ldx, v.M, a.lin_off) : rows32(v.aux, m, a.ldg, v.M);
        uint32_t b[32];
#pragma unroll
        for (int i = 0; i < 32; i++)
            b[i] = load_row(vb, i, ox);
#pragma unroll
        for (int i = 0; i < 16; i++)
            w[i] = fused_pair<OP>(pack2(e[2 * i], e[2 * i + 1]), pack2(b[2 * i], b[2 * i + 1]));
    }
}

// The 32 elements of a block (16 packed words) -> scale byte and 32 codes,
// element 4j + i in byte i of o[j].  A block with an Inf or NaN gets scale
// 0xFF and codes 0x7F.
template <int FMT>
__device__ __forceinline__ uint32_t any_block(const uint32_t (&w)[16], uint32_t (&o)[8])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; i++)
        m = pk_max_u16(m, w[i] & 0x7FFF7FFFu);
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    const uint32_t sb = scale_byte<FMT>(lo > hi ? lo : hi);
    const uint32_t lim = sat_limit2<FMT>(sb);
    const float sc = e8m0_operand(sb);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t t = mx_pair<FMT, false>(w[2 * j], w[2 * j] & 0x7FFF7FFFu, lim, sc, 0u);
        o[j] = mx_pair<FMT, true>(w[2 * j + 1], w[2 * j + 1] & 0x7FFF7FFFu, lim, sc, t);
    }
    if (sb == 0xFFu) {
#pragma unroll
        for (int j = 0; j < 8; j++)
            o[j] = 0x7F7F7F7Fu;
    }
    return sb;
}

// Byte offset of scale (row r, block b) in the GEMM-ready tile layout of a
// matrix with RT row tiles: 256-byte tiles of 32 rows x 8 blocks, block-tile
// major; lane 32 (b % 2) + r % 32 of the tile holds, in byte (b % 8) / 2,
// block b of row r.
__device__ __forceinline__ int64_t tile_offset(int64_t r, int64_t b, int64_t RT)
{
    return ((b >> 3) * RT + (r >> 5)) * 256 + 4 * (32 * (b & 1) + (r & 31)) + ((b & 7) >> 1);
}

// Row scale of row m0 + r, block b (value sb) of a step: compact
// [M][ceil(K / 32)] or the tile layout (rows up to the last row tile, every
// block of the tile; padding holds 0).
__device__ __forceinline__ void any_store_srow(const MxArgs &a, const AnyView &v, int64_t m0,
                                               int tk, int r, int64_t b, uint32_t sb)
{
    const int64_t nb = (a.K + 31) >> 5;
    if (!a.tiled) {
        const rsrc_t rs = make_rsrc(v.s_row, m0 * nb, v.M * nb);
        const bool ok = m0 + r < v.M && b < nb;
        buf_store1(rs, ok ? (uint32_t)(r * nb + b) : kDead, (uint8_t)sb);
        return;
    }
    const int64_t RT = (v.M + 31) >> 5, CT = (nb + 7) >> 3;
    // row tile m0 / 32 of block tile b / 8 (= 4 tk / 8 for every block a
    // step writes, padding included), uniform across the workgroup
    const int64_t base = tile_offset(m0, (int64_t)(4 * tk) & ~7, RT);
    const rsrc_t rs = make_rsrc(v.s_row, base, RT * CT * 256);
    const bool ok = m0 + r < 32 * RT && b < 8 * CT;
    buf_store1(rs, ok ? (uint32_t)(tile_offset(m0 + r, b, RT) - base) : kDead, (uint8_t)sb);
}

// One 64 x 128 step (the s-th of the walk) at rows m0, columns k0; w: this
// thread's column values (column k0 + t % 128, rows m0 + 32 (t / 128) + i).
template <int FMT>
__device__ __forceinline__ void any_step(const MxArgs &a, const AnyView &v, AnyStage &st,
                                         const uint32_t (&w)[16], int64_t m0, int tk, int s,
                                         bool last_step, unsigned axis, bool dbias, bool last_tk,
                                         float &dacc)
{
    const int t = (int)threadIdx.x;
    const int c = t & (kAnyTileK - 1);
    const int h = __builtin_amdgcn_readfirstlane(t >> 7);   // uniform per wave
    const int64_t k0 = (int64_t)tk * kAnyTileK;
    const bool row = axis & 1u, col = (axis & 2u) != 0;

    if (row) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            st.y[32 * h + 2 * i][c] = (uint16_t)(w[i] & 0xFFFFu);
            st.y[32 * h + 2 * i + 1][c] = (uint16_t)(w[i] >> 16);
        }
    }
    float sum = 0.0f;
    if (dbias) {
        // this thread's 32 rows in order
#pragma unroll
        for (int i = 0; i < 16; i++) {
            sum += bf16_lo(w[i]);
            sum += bf16_hi(w[i]);
        }
        if (h == 1)
            st.dsum[c] = sum;
    }
    if (col) {
        uint32_t o[8];
        const uint32_t sb = any_block<FMT>(w, o);
        uint8_t *q = &st.qt[c][64 * (s & 1) + 32 * h];
        *reinterpret_cast<uint4 *>(q) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(q + 16) = make_uint4(o[4], o[5], o[6], o[7]);
        st.sc[c][2 * s + h] = (uint8_t)sb;
    }
    __syncthreads();
    if (dbias && h == 0)
        dacc += sum + st.dsum[c];   // rows 0..31 + rows 32..63, then step after step
    if (row) {
        const int r = t >> 2, q = t & 3;
        uint32_t wr[16];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint4 u = *reinterpret_cast<const uint4 *>(&st.y[r][32 * q + 8 * j]);
            wr[4 * j] = u.x; wr[4 * j + 1] = u.y; wr[4 * j + 2] = u.z; wr[4 * j + 3] = u.w;
        }
        uint32_t o[8];
        const uint32_t sb = any_block<FMT>(wr, o);
        uint8_t *qd = qrow_stage(st, r) + 32 * q;   // over row r's bf16 values, already read
        *reinterpret_cast<uint4 *>(qd) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4 *>(qd + 16) = make_uint4(o[4], o[5], o[6], o[7]);
        const int64_t b = (int64_t)4 * tk + q;
        any_store_srow(a, v, m0, tk, r, b, sb);
        // tile layout: the last strip also writes the padding blocks of its
        // block tile that no strip covers (zeros)
        if (a.tiled && last_tk && (tk & 1) == 0)
            any_store_srow(a, v, m0, tk, r, b + 4, 0u);
    }
    __syncthreads();
    const int mrem = (int)(v.M - m0 < kAnyTileM ? v.M - m0 : kAnyTileM);
    if (row)
        flush_rows<kAnyTileK>(v.q_row, a.K, m0, k0, v.M * a.K, mrem,
                              (int)(a.K - k0 < kAnyTileK ? a.K - k0 : kAnyTileK), qrow_stage(st, 0),
                              (int)sizeof(st.y[0]));
    if (col)
        flush_cols<kAnyTileM>(v.q_col, v.M, k0, a.K, m0, mrem, s, last_step, st.qt[0],
                              (int)sizeof(st.qt[0]));
    __syncthreads();
}

// Column scales of a walk over steps t0 .. t0 + n - 1 (blocks jb = 2 t0 ..
// jb + 2n - 1) of strip tk: compact [K][ceil(M / 32)], or the tile layout,
// where the group's last walk also writes the padding blocks up to the end
// of the last block tile, and the last strip the padding rows (both 0).
__device__ __forceinline__ void any_flush_scol(const MxArgs &a, const AnyView &v,
                                               const AnyStage &st, int t0, int n, int tk,
                                               bool last_walk)
{
    const int t = (int)threadIdx.x;
    const int64_t k0 = (int64_t)tk * kAnyTileK;
    const int64_t nb = (v.M + 31) >> 5;
    const int64_t jb = 2 * (int64_t)t0;
    const int cnt = 2 * n;
    if (!a.tiled) {
        const rsrc_t rs = make_rsrc(v.s_col, k0 * nb + jb, a.K * nb);
        for (int idx = t; idx < kAnyTileK * 2 * kAnyMaxWalk; idx += kThreads) {
            const int c = idx / (2 * kAnyMaxWalk), jj = idx % (2 * kAnyMaxWalk);
            const bool ok = jj < cnt && k0 + c < a.K && jb + jj < nb;
            buf_store1(rs, ok ? (uint32_t)(c * nb + jj) : kDead, st.sc[c][jj < cnt ? jj : 0]);
        }
        return;
    }
    const int64_t RT = (a.K + 31) >> 5, CT = (nb + 7) >> 3;
    const int64_t jend = last_walk ? 8 * CT : jb + cnt;
    const int span = (int)(jend - jb);                 // <= 2 n + 7
    const int64_t base = tile_offset(k0, jb & ~7, RT);
    const rsrc_t rs = make_rsrc(v.s_col, base, RT * CT * 256);
    for (int idx = t; idx < kAnyTileK * span; idx += kThreads) {
        const int c = idx / span, jj = idx % span;
        const int64_t kk = k0 + c, j = jb + jj;
        const bool ok = kk < 32 * RT && j < 8 * CT;
        const uint8_t val = jj < cnt ? st.sc[c][jj] : (uint8_t)0;
        buf_store1(rs, ok ? (uint32_t)(tile_offset(kk, j, RT) - base) : kDead, val);
    }
}

// Walk w (numbered across groups) of strip tk; group g holds walks
// walk0[g] .. walk0[g + 1] - 1, each of len[g] steps.
template <int OP, int FMT>
__global__ __launch_bounds__(kThreads, 4) void mx_cast_any_kernel(MxArgs a, GroupTable gt,
                                                               unsigned axis, int dbias)
{
    __shared__ AnyStage st;
    const int job = xcd_tile((int)blockIdx.x, (int)gridDim.x);
    const int walk = job / a.tiles_k;
    const int tk = job - walk * a.tiles_k;
    int g = 0;
    while (g + 1 < gt.count && gt.walk0[g + 1] <= walk)
        g++;
    const int64_t r0 = gt.row0[g];
    AnyView v;
    v.M = gt.row0[g + 1] - r0;
    v.x = a.x + r0 * a.ldx;
    v.aux = a.aux ? a.aux + r0 * a.ldg : nullptr;
    v.q_row = a.q_row ? a.q_row + r0 * a.K : nullptr;
    v.s_row = a.s_row ? a.s_row + gt.srow_off[g] : nullptr;
    v.q_col = a.q_col ? a.q_col + a.K * r0 : nullptr;
    v.s_col = a.s_col ? a.s_col + gt.scol_off[g] : nullptr;
    const int len = gt.len[g];
    const int t0 = (walk - gt.walk0[g]) * len;
    const int tiles_m = (int)((v.M + kAnyTileM - 1) / kAnyTileM);
    const int n = tiles_m - t0 < len ? tiles_m - t0 : len;
    const bool last_tk = tk + 1 == a.tiles_k;
    const int h = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 7);
    const int64_t k = (int64_t)tk * kAnyTileK + (threadIdx.x & (kAnyTileK - 1));
    const bool col_ok = k < a.K;
    float dacc = 0.0f;
    for (int s = 0; s < n; s++) {
        uint32_t w[16];
        any_load<OP>(a, v, (int64_t)(t0 + s) * kAnyTileM + 32 * h, k, col_ok, w);
        any_step<FMT>(a, v, st, w, (int64_t)(t0 + s) * kAnyTileM, tk, s, s + 1 == n, axis,
                      dbias != 0, last_tk, dacc);
    }
    if (axis & 2u)
        any_flush_scol(a, v, st, t0, n, tk, walk + 1 == gt.walk0[g + 1]);
    if (dbias) {
        const int64_t k = (int64_t)tk * kAnyTileK + (threadIdx.x & (kAnyTileK - 1));
        const rsrc_t rp = make_rsrc(a.partials, 4 * ((int64_t)walk * a.K + (int64_t)tk * kAnyTileK),
                                    4 * (int64_t)gt.walk0[gt.count] * a.K);
        const bool ok = threadIdx.x < kAnyTileK && k < a.K;
        buf_store4(rp, ok ? 4u * (threadIdx.x & (kAnyTileK - 1)) : kDead, __float_as_uint(dacc));
    }
}

template <int OP>
static hipError_t launch_any_op(unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                                const GroupTable &gt, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)gt.walk0[gt.count] * a.tiles_k));
    const int db = dbias ? 1 : 0;
    switch (fmt) {
    case 0u:
        hipLaunchKernelGGL((mx_cast_any_kernel<OP, 0>), grid, dim3(kThreads), 0, s, a, gt, axis, db);
        break;
    case kFmtE5M2:
        hipLaunchKernelGGL((mx_cast_any_kernel<OP, kFmtE5M2>), grid, dim3(kThreads), 0, s, a, gt,
                           axis, db);
        break;
    case kFmtRoundUp:
        hipLaunchKernelGGL((mx_cast_any_kernel<OP, kFmtRoundUp>), grid, dim3(kThreads), 0, s, a, gt,
                           axis, db);
        break;
    case kFmtE5M2 | kFmtRoundUp:
        hipLaunchKernelGGL((mx_cast_any_kernel<OP, kFmtE5M2 | kFmtRoundUp>), grid, dim3(kThreads),
                           0, s, a, gt, axis, db);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mx_cast_any(int op, unsigned axis, unsigned fmt, bool dbias, const MxArgs &a,
                              const GroupTable &gt, hipStream_t s)
{
    switch (op) {
    case OP_PLAIN: return launch_any_op<OP_PLAIN>(axis, fmt, dbias, a, gt, s);
    case OP_GELU: return launch_any_op<OP_GELU>(axis, fmt, dbias, a, gt, s);
    case OP_DGELU: return launch_any_op<OP_DGELU>(axis, fmt, dbias, a, gt, s);
    case OP_SWIGLU: return launch_any_op<OP_SWIGLU>(axis, fmt, false, a, gt, s);
    case OP_GEGLU: return launch_any_op<OP_GEGLU>(axis, fmt, false, a, gt, s);
    case OP_DSILU: return launch_any_op<OP_DSILU>(axis, fmt, dbias, a, gt, s);
    case OP_DSWIGLU: return launch_any_op<OP_DSWIGLU>(axis, fmt, false, a, gt, s);
    case OP_DGEGLU: return launch_any_op<OP_DGEGLU>(axis, fmt, false, a, gt, s);
    default: return hipErrorInvalidValue;
    }
}

// Fused values of any shape, one element per thread (the 16-byte kernel of
// mx_cast.hip needs rows of a multiple of 8 elements).
template <int OP>
__global__ __launch_bounds__(256) void fused_values_any_kernel(const uint16_t *x, const uint16_t *aux,
                                                               int64_t M, int64_t K, uint16_t *y)
{
    constexpr bool dgated = OP == OP_DSWIGLU || OP == OP_DGEGLU;
    constexpr bool gated = OP == OP_SWIGLU || OP == OP_GEGLU;
    const int64_t W = dgated ? 2 * K : K;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * W)
        return;
    const int64_t row = i / W, col = i - row * W;
    uint32_t o;
    if constexpr (dgated) {
        const bool gate_half = col < K;
        const int64_t n = gate_half ? col : col - K;
        o = dgated_pair<OP>(x[row * 2 * K + n], aux[row * K + n], x[row * 2 * K + K + n], gate_half);
    } else if constexpr (gated) {
        o = fused_pair<OP>(x[row * 2 * K + col], x[row * 2 * K + K + col]);
    } else {
        o = fused_pair<OP>(x[i], OP == OP_GELU ? x[i] : aux[i]);
    }
    y[i] = (uint16_t)(o & 0xFFFFu);
}

hipError_t launch_fused_values_any(int op, const uint16_t *x, const uint16_t *aux, int64_t M,
                                   int64_t K, uint16_t *y, hipStream_t s)
{
    const int64_t n = M * K * (op == OP_DSWIGLU || op == OP_DGEGLU ? 2 : 1);
    const dim3 grid((unsigned)((n + 255) / 256));
    switch (op) {
    case OP_GELU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_GELU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    case OP_DGELU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_DGELU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    case OP_SWIGLU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_SWIGLU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    case OP_GEGLU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_GEGLU>, grid, dim3(256), 0, s, x, x, M, K, y);
        break;
    case OP_DSILU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_DSILU>, grid, dim3(256), 0, s, x, aux, M, K, y);
        break;
    case OP_DSWIGLU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_DSWIGLU>, grid, dim3(256), 0, s, x, aux, M, K,
                           y);
        break;
    case OP_DGEGLU:
        hipLaunchKernelGGL(fused_values_any_kernel<OP_DGEGLU>, grid, dim3(256), 0, s, x, aux, M, K,
                           y);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mxk
