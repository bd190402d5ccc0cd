"""Host model of the cast kernels' buffer addressing at the sizes the ABI
accepts (pure CPU; no GPU, no library call).

Every global access of the cast kernels goes through a buffer descriptor
(`make_rsrc` in csrc/bufio.h): a base shifted by a 64-bit byte offset and a
size capped at 2^31 - 1, plus a 32-bit per-lane byte offset.  A lane that must
not touch memory gets the offset 2^31 ("dead"), or its access lies past the
descriptor's size, and the hardware then drops the access.  That scheme is
only sound if

  (a) every live access lies wholly inside its descriptor:
      offset + bytes <= size, and
  (b) every masked access (a dead lane, a row past M, a column past K) lies
      wholly outside it: offset >= size, without the 32-bit offset wrapping.

This file restates, site by site, the offset arithmetic of mx_cast.h and
nvfp4.hip (load_tile, row_pass, col_flush_q, srow_flush, col_flush_s[_tiled],
flush_scale_rows, nv_load, the NVFP4 row store, nv_flush_q, nv_flush_s,
nv_flush_srow) and checks (a) and (b) for every lane of the first and last
sub-tile of the first and last walk, at the largest shapes each entry point
accepts: rows and row lengths of 2^23, M * K = 2^40, a gated input's full row
2N = 2^23.  The model follows the kernels' own variable names so that each
line can be compared with the code by eye.
"""
import itertools

import numpy as np
import pytest

ROWS_PER_LANE, COLS_PER_LANE, WAVES = 16, 8, 4
THREADS = 64 * WAVES
TILE_M, TILE_K = 128, 256
MAX_GROUP = 16
MAX_RAG_GROUP = 14
MAX_NV_RAG_GROUP = 4
MAX_RECORDS = 0x7FFFFFFF
DEAD = 0x80000000
U32 = 1 << 32


def pick_group(tiles_m, tiles_k, target=512, max_len=16):
    g = 1
    while 2 * g <= max_len:
        g *= 2
    while g > 1 and ((tiles_m + g - 1) // g) * tiles_k < target:
        g >>= 1
    return g


def plan_walk(t, tiles_k, slots=512, even=False, max_len=16):
    """plan_walks (launch.h) for one tensor of t sub-tile rows."""
    best = None
    for L in range(2 if even else 1, max_len + 1, 2 if even else 1):
        lg = -(-t // -(-t // L))
        lg += lg & 1 if even else 0
        cost = -(-(-(-t // lg) * tiles_k) // slots) * (lg + 1)
        if best is None or cost < best[0] or (cost == best[0] and lg > best[1]):
            best = (cost, lg)
    return best[1]


class Desc:
    """make_rsrc(base, offset, total): bytes [offset, total) of an allocation,
    size 0 when offset >= total, at most MAX_RECORDS bytes."""

    def __init__(self, offset, total):
        left = total - offset
        self.base = offset if left > 0 else 0
        self.size = 0 if left <= 0 else min(left, MAX_RECORDS)
        self.total = total


class Checker:
    def __init__(self):
        self.bad = []

    def access(self, site, d, off, nbytes, live, addr=None):
        """off: uint32 per-lane offsets (numpy int64 holding the 32-bit value
        the kernel computes); live: bool mask of accesses that must happen.
        addr, when given, is the logical byte address of each access inside
        its allocation; live accesses must land exactly there."""
        off = np.asarray(off, dtype=np.int64)
        live = np.broadcast_to(np.asarray(live, dtype=bool), off.shape)
        if (off < 0).any() or (off >= U32).any():
            self.bad.append((site, "32-bit offset out of [0, 2^32)"))
            return
        inside = off + nbytes <= d.size
        outside = off >= d.size
        if (live & ~inside).any():
            i = np.argwhere(live & ~inside)[0]
            self.bad.append((site, f"live access past the descriptor: off {int(off[tuple(i)])} "
                                   f"+ {nbytes} > size {d.size}"))
        if (~live & ~outside).any():
            i = np.argwhere(~live & ~outside)[0]
            self.bad.append((site, f"masked access inside the descriptor: off {int(off[tuple(i)])}, "
                                   f"size {d.size}"))
        if addr is not None:
            addr = np.broadcast_to(np.asarray(addr, dtype=np.int64), off.shape)
            wrong = live & (d.base + off != addr)
            if wrong.any():
                i = np.argwhere(wrong)[0]
                self.bad.append((site, f"live access at {int(d.base + off[tuple(i)])}, "
                                       f"element at {int(addr[tuple(i)])}"))
            if (live & (addr + nbytes > d.total)).any():
                self.bad.append((site, "live element past the allocation"))

    def ok(self):
        assert not self.bad, self.bad[:6]


def lanes():
    """Per thread of a workgroup: wave, half, cl (lane & 31), first row."""
    t = np.arange(THREADS)
    wave, lane = t >> 6, t & 63
    half, cl = lane >> 5, lane & 31
    row = wave * 2 * ROWS_PER_LANE + half * ROWS_PER_LANE
    return t, wave, half, cl, row


def edge(n):
    return sorted({0, n - 1})


# ---------------------------------------------------------------------------
# MXFP8 cast kernel (mx_cast.h).  op: "plain", "grad" (dGELU / dSiLU: a second
# [M][K] input), "gated" (x [M][2N], K = N), "dgated" (grad [M][N], x [M][2N],
# K = 2N).
# ---------------------------------------------------------------------------
def mx_model(M, K, op="plain", tiled=False, ck=None):
    ck = ck or Checker()
    if op == "gated":
        ldx, lin_off, ldg = 2 * K, K, 0
    elif op == "dgated":
        ldx, lin_off, ldg = K, K // 2, K // 2
    else:
        ldx, lin_off, ldg = K, 0, K
    tiles_m, tiles_k = -(-M // TILE_M), -(-K // TILE_K)
    # walks of the variant for transposed rows at any byte: at most 14
    max_len = MAX_RAG_GROUP if M % 16 else MAX_GROUP
    if op == "plain":
        group = plan_walk(tiles_m, tiles_k, even=tiled, max_len=max_len)
    else:
        group = pick_group(tiles_m, tiles_k, max_len=max_len)
        if tiled and group < 2:
            group = 2
    groups_m = -(-tiles_m // group)
    t, wave, half, cl, row = lanes()
    r = np.arange(ROWS_PER_LANE)[:, None]
    strips = edge(tiles_k)
    if op == "dgated":
        # also the strips on either side of the gate / linear boundary
        strips = sorted(set(strips) | {(lin_off - 1) // TILE_K, lin_off // TILE_K} - {tiles_k})
    for tm, tk in itertools.product(edge(tiles_m) + [tiles_m], strips):
        # lane_live; tm == tiles_m is the prefetch past a walk's end
        live = (tm * TILE_M + wave * 32 < M) & (tk * TILE_K + cl * COLS_PER_LANE < K)
        in_rows = tm * TILE_M + row + r < M            # [16][256]
        # ---- load_tile
        if op == "dgated":
            N = lin_off
            k = tk * TILE_K + COLS_PER_LANE * cl
            gate_half = k < N
            n = np.where(gate_half, k, k - N)
            m0 = tm * TILE_M
            rx = Desc(2 * m0 * ldx, 2 * M * ldx)
            rg = Desc(2 * m0 * ldg, 2 * M * ldg)
            rl = Desc(2 * (m0 * ldx + N), 2 * M * ldx)
            sx, sg = 2 * ldx, 2 * ldg
            ox = np.where(live, row * sx + 2 * n, DEAD)
            og = np.where(live, row * sg + 2 * n, DEAD)
            ol = np.where(live & gate_half, ox, DEAD)
            rowabs = m0 + row + r
            ck.access("dgated gate", rx, ox + r * sx, 16, live & in_rows,
                      2 * (rowabs * ldx + n))
            ck.access("dgated grad", rg, og + r * sg, 16, live & in_rows,
                      2 * (rowabs * ldg + n))
            ck.access("dgated linear", rl, ol + r * sx, 16, live & gate_half & in_rows,
                      2 * (rowabs * ldx + N + n))
        else:
            tile = tm * TILE_M * ldx + tk * TILE_K
            total = M * ldx
            rx = Desc(2 * tile, 2 * total)
            rs = 2 * ldx
            off = np.where(live, row * rs + 2 * COLS_PER_LANE * cl, DEAD)
            col = tk * TILE_K + COLS_PER_LANE * cl
            addr = 2 * ((tm * TILE_M + row + r) * ldx + col)
            ck.access(f"{op} x", rx, off + r * rs, 16, live & in_rows, addr)
            if op == "grad":
                gtile = tm * TILE_M * ldg + tk * TILE_K
                rb = Desc(2 * gtile, 2 * M * ldg)
                boff = np.where(live, row * 2 * ldg + 2 * COLS_PER_LANE * cl, DEAD)
                ck.access("grad", rb, boff + r * 2 * ldg, 16, live & in_rows,
                          2 * ((tm * TILE_M + row + r) * ldg + col))
            elif op == "gated":
                rb = Desc(2 * (tile + lin_off), 2 * total)
                ck.access("gated linear", rb, off + r * rs, 16, live & in_rows,
                          2 * ((tm * TILE_M + row + r) * ldx + lin_off + col))
        if tm == tiles_m:
            continue                                    # the prefetch only loads
        # ---- row_pass: 8-byte row stores
        rq = Desc(tm * TILE_M * K + tk * TILE_K, M * K)
        off = np.where(live, row * K + COLS_PER_LANE * cl, DEAD)
        ck.access("q_row", rq, off + r * K, 8, live & in_rows,
                  (tm * TILE_M + row + r) * K + tk * TILE_K + COLS_PER_LANE * cl)
        # ---- col_flush_q: thread t writes chunk t % 8 of transposed rows t / 8 + 32 i
        jr = t & 7
        mt, k0 = tm * TILE_M, tk * TILE_K
        if M % 16:
            # col_flush_q_rag, at the sub-tile's place in its walk
            g = tm % group
            n = min(tiles_m - (tm - g), group)
            for site, d, off, nb_, lv, addr in model_col_flush_q_rag(0, M, K, tm, tk, g == 0,
                                                                     g == n - 1):
                ck.access(site, d, off, nb_, lv, addr)
        else:
            rc = Desc(k0 * M + mt, K * M)
            chunk_live = mt + 16 * jr < M
            kr = (t >> 3)[None, :] + 32 * np.arange(TILE_K // 32)[:, None]
            ok = chunk_live & (k0 + kr < K)
            ck.access("q_col", rc, np.where(ok, kr * M + 16 * jr, DEAD), 16, ok,
                      (k0 + kr) * M + mt + 16 * jr)
        # ---- srow_flush
        nb = -(-K // 32)
        if tiled:
            RT = -(-M // 32)
            size = RT * (-(-nb // 8)) * 256
            rs_ = Desc((tk * RT + 4 * tm) * 256, size)
            w = t >> 6
            lv = tm * TILE_M + 32 * w < M
            ck.access("s_row tiled", rs_, np.where(lv, 4 * t, DEAD), 4, lv)
        else:
            rrow = tm * TILE_M + t
            rs_ = Desc(tm * TILE_M * nb + (k0 >> 5), M * nb)
            o = np.where((t < TILE_M) & (rrow < M), t * nb, DEAD)
            if K % 256 == 0:
                ck.access("s_row", rs_, o, 8, (t < TILE_M) & (rrow < M),
                          rrow * nb + (k0 >> 5))
            else:
                blocks = nb - (k0 >> 5)
                b = np.arange(TILE_K // 32)[:, None]
                lv = (b < blocks) & (t < TILE_M) & (rrow < M)
                ck.access("s_row bytes", rs_, np.where(b < blocks, o + b, DEAD), 1, lv,
                          rrow * nb + (k0 >> 5) + b)
    # ---- col_flush_s at the end of the first and last walk of each edge strip
    nblk = -(-M // 32)
    for rg, tk in itertools.product(edge(groups_m), edge(tiles_k)):
        n = min(tiles_m - rg * group, group)
        k0 = tk * TILE_K
        if tiled:
            RT = -(-K // 32)
            CT = -(-nblk // 8)
            bt0, rt0 = rg * (group >> 1), tk * (TILE_K // 32)
            nbt = (4 * n + 7) >> 3
            rs_ = Desc((bt0 * RT + rt0) * 256, RT * CT * 256)
            idx = t[None, :] + THREADS * np.arange(2 * nbt)[:, None]
            btl, rtl, lane = idx >> 9, (idx >> 6) & 7, idx & 63
            lv = rt0 + rtl < RT
            ck.access("s_col tiled", rs_, np.where(lv, (btl * RT + rtl) * 256 + 4 * lane, DEAD),
                      4, lv, ((bt0 + btl) * RT + rt0 + rtl) * 256 + 4 * lane)
        else:
            first = rg * group * 4
            count = min(nblk - first, 4 * n)
            rs_ = Desc(k0 * nblk + first, K * nblk)
            scale_rows(ck, "s_col", rs_, k0, K, nblk, first, count)
    return ck


def model_rag_lines(d, base, pitch, rows, addr0, rem, first, last):
    """rag_flush_lines (rag_flush.h): one step of a walk over transposed rows
    pitch bytes apart, `rows` of them from the strip's first, as (site,
    descriptor, offsets, bytes, live, address) -- d the descriptor from the
    line boundary at or below the step's first byte of the strip's first row
    (base bytes before it), addr0(kr) the address of row kr's first byte of
    the step."""
    t = np.arange(THREADS)
    j = t & 7
    lo = 0 if first else -128
    out = []
    for i in range(256 // 32):
        kr = (t >> 3) + 32 * i
        at = base + kr * pitch
        sft = at % 128
        for p in (0, 128) if last else (0,):
            p0 = p + 16 * j - sft
            whole = (kr < rows) & (p0 >= lo) & (p0 + 16 <= rem)
            out.append(("rag W=16", d, np.where(whole, at - sft + p + 16 * j, DEAD), 16, whole,
                        addr0(kr) + p0))
    if not (first or last):
        return out
    # the end pieces, one row per thread, in naturally aligned stores:
    # upwards from the head range's first byte while its low bits are set,
    # then downwards by size
    kr = t
    at = base + kr * pitch
    sft = at % 128
    o, et = sft % 16, (rem + sft) % 16
    qh, qt = sft >> 4, (rem - 1 + sft) >> 4
    head = (kr < rows) & first & (o != 0)
    tail = (kr < rows) & last & (et != 0) & ~(head & (qt == qh))
    for on, q, b, b1, up in ((head, qh, o, np.minimum(16, o + rem), True),
                             (tail, qt, np.zeros_like(t), et, False)):
        if not on.any():
            continue
        for size, go, bs in range_stores(on, b, b1, up):
            out.append((f"rag end W={size}", d, np.where(go, at - sft + 16 * q + bs, DEAD), size, go,
                        addr0(kr) + 16 * q - sft + bs))
    return out


def range_stores(on, b0, b1, up):
    """rag_store_range (rag_flush.h): the stores (size, lanes that store,
    first byte) of bytes b0 .. b1 - 1 of a 16-byte piece."""
    steps = ([(1, True), (2, True), (4, True), (8, True)] if up else []) + \
            [(8, False), (4, False), (2, False), (1, False)]
    b = b0
    out = []
    for size, by_bit in steps:
        go = on & (b + size <= b1) & (((b & size) != 0) if by_bit else True)
        out.append((size, go, b))
        b = np.where(go, b + size, b)
    return out


def test_range_stores_cover_any_range_once_aligned():
    """Every partial byte range of a 16-byte piece (from byte 0 without the
    upward pass): each byte stored exactly once, every store naturally
    aligned and inside the range."""
    b0, b1 = np.meshgrid(np.arange(16), np.arange(17), indexing="ij")
    b0, b1 = b0.ravel(), b1.ravel()
    keep = (b0 < b1) & (b1 - b0 < 16)
    b0, b1 = b0[keep], b1[keep]
    for up in (True, False):
        sel = np.ones_like(b0, bool) if up else b0 == 0
        lo, hi = b0[sel], b1[sel]
        cover = np.zeros((lo.size, 16), np.int64)
        for size, go, b in range_stores(np.ones(lo.size, bool), lo, hi, up):
            assert (b[go] % size == 0).all()
            assert ((b[go] >= lo[go]) & (b[go] + size <= hi[go])).all()
            for k in range(size):
                np.add.at(cover, (np.nonzero(go)[0], b[go] + k), 1)
        want = (np.arange(16) >= lo[:, None]) & (np.arange(16) < hi[:, None])
        assert (cover == want).all()


def model_col_flush_q_rag(base, M, K, tm, tk, first, last):
    """col_flush_q_rag (mx_cast.h): sub-tile tm of strip tk, addresses from
    the start of the tensor's (or group's) q_col, which lies at `base` modulo
    128."""
    mt, k0 = tm * TILE_M, tk * TILE_K
    rem = min(M - mt, TILE_M)
    d0 = (base + k0 * M) % 128
    # make_rsrc(row0 - d0, mt, (K - k0) * M + d0), row0 = q_col + k0 M
    d = Desc(k0 * M - d0 + mt, K * M)
    return model_rag_lines(d, d0, M, K - k0, lambda kr: (k0 + kr) * M + mt, rem, first, last)


def model_nv_flush_q_rag(base, M, K, tm, tk, parts, first, last):
    """nv_flush_q_rag (nvfp4.hip): the pair of sub-tiles starting at tm
    (parts 1: that sub-tile only), rows of ceil(M/2) bytes."""
    k0 = tk * TILE_K
    ld = (M + 1) >> 1
    b0 = tm * (TILE_M // 2)
    rem = min(ld - b0, 64 * parts)
    d0 = (base + k0 * ld) % 128
    d = Desc(k0 * ld - d0 + b0, K * ld)
    return model_rag_lines(d, d0, ld, K - k0, lambda kr: (k0 + kr) * ld + b0, rem, first, last)


RAG_STACKS = [([1], 8), ([17], 24), ([129], 256), ([300], 264), ([255, 1], 8), ([16, 8], 256),
              ([1, 17, 0, 300, 129, 5], 40), ([1104, 3008, 1072, 6563, 1], 8),
              ([250, 131, 9], 520)]


@pytest.mark.parametrize("base", [0, 5, 16, 127])
@pytest.mark.parametrize("L", [1, 2, 3, 14])
@pytest.mark.parametrize("rows,K", RAG_STACKS)
def test_ragged_transposed_writes_every_byte_once(rows, K, L, base):
    """col_flush_q_rag over every walk of walk length L of every group of a
    stack (the groups' [K][rows] transposes one after the other, the stack's
    q_col at `base` modulo 128): every byte written exactly once, 16-byte
    stores aligned, away from walk ends only in whole lines, every access
    inside its descriptor."""
    total = K * sum(rows)
    count = np.zeros(total, np.int64)
    ck = Checker()
    r0 = 0
    for M in rows:
        if M == 0:
            continue
        gbase = (base + K * r0) % 128
        tiles_m, tiles_k = -(-M // TILE_M), -(-K // TILE_K)
        for w in range(-(-tiles_m // L)):
            n = min(L, tiles_m - w * L)
            for tk in range(tiles_k):
                for g in range(n):
                    for site, d, off, nb_, live, addr in model_col_flush_q_rag(
                            gbase, M, K, w * L + g, tk, g == 0, g == n - 1):
                        ck.access(site, d, off, nb_, live, addr)
                        a = np.broadcast_to(addr, live.shape)[live]
                        assert (a >= 0).all()
                        assert ((gbase + a) % nb_ == 0).all(), f"{nb_}-byte store not aligned"
                        if nb_ == 16:
                            if 0 < g < n - 1 and a.size:
                                # a sub-tile inside the walk writes each row's line whole
                                lines = (gbase + a) // 128
                                assert (np.bincount(lines - lines.min()) % 8 == 0).all()
                        for b in range(nb_):
                            np.add.at(count, K * r0 + a + b, 1)
        r0 += M
    ck.ok()
    assert (count == 1).all(), (int((count == 0).sum()), int((count > 1).sum()))


@pytest.mark.parametrize("base", [0, 5, 64, 127])
@pytest.mark.parametrize("L", [2, 4])
@pytest.mark.parametrize("rows,K", [([1], 16), ([17], 32), ([257], 256), ([300], 272),
                                    ([255, 1], 16), ([16, 8], 256), ([1, 17, 0, 300, 129, 5], 48),
                                    ([1104, 3008, 1072, 6563, 1], 16), ([250, 131, 9], 528)])
def test_nvfp4_ragged_transposed_writes_every_byte_once(rows, K, L, base):
    """nv_flush_q_rag over every pair of every walk (even length L) of every
    group of a stack (the groups' [K][ceil(rows/2)] transposes one after the
    other, at `base` modulo 128): every byte written exactly once, every
    access inside its descriptor."""
    total = K * sum(-(-m // 2) for m in rows)
    count = np.zeros(total, np.int64)
    ck = Checker()
    off = 0
    for M in rows:
        if M == 0:
            continue
        gbase = (base + off) % 128
        tiles_m, tiles_k = -(-M // TILE_M), -(-K // TILE_K)
        for w in range(-(-tiles_m // L)):
            n = min(L, tiles_m - w * L)
            for tk in range(tiles_k):
                for g in range(1, n + 1, 2):       # the flushes: g odd, or a walk's lone last
                    parts = 2 if g < n else 1
                    tm = w * L + (g - 1)
                    for site, d, o, nb_, live, addr in model_nv_flush_q_rag(
                            gbase, M, K, tm, tk, parts, g < 2, g + 1 >= n):
                        ck.access(site, d, o, nb_, live, addr)
                        a = np.broadcast_to(addr, live.shape)[live]
                        assert (a >= 0).all()
                        assert ((gbase + a) % nb_ == 0).all(), f"{nb_}-byte store not aligned"
                        for b in range(nb_):
                            np.add.at(count, off + a + b, 1)
        off += K * -(-M // 2)
    ck.ok()
    assert (count == 1).all(), (int((count == 0).sum()), int((count > 1).sum()))


def scale_rows(ck, site, rs, k0, K, pitch, first, count, base_align=0):
    """flush_scale_rows (stage_flush.h): row c's `count` bytes in pieces of
    the widest size CH that pitch, first, count and the base allow."""
    align = pitch | first | count | base_align
    CH = next(c for c in (16, 8, 4, 2, 1) if align % c == 0)
    t = np.arange(THREADS)
    pieces = count // CH
    if pieces == 0:
        return
    idx = t[None, :] + THREADS * np.arange(pieces)[:, None]
    c, q = idx // pieces, idx % pieces
    lv = k0 + c < K
    ck.access(site, rs, np.where(lv, c * pitch + CH * q, DEAD), CH, lv,
              (k0 + c) * pitch + first + CH * q)


# ---------------------------------------------------------------------------
# NVFP4 kernel (nvfp4.hip)
# ---------------------------------------------------------------------------
def nv_model(M, K, ck=None):
    ck = ck or Checker()
    tiles_m, tiles_k = -(-M // TILE_M), -(-K // TILE_K)
    rag = M % 16 != 0
    group = plan_walk(tiles_m, tiles_k, even=rag, max_len=MAX_NV_RAG_GROUP if rag else 16)
    groups_m = -(-tiles_m // group)
    t, wave, half, cl, row = lanes()
    r = np.arange(ROWS_PER_LANE)[:, None]
    for tm, tk in itertools.product(edge(tiles_m) + [tiles_m], edge(tiles_k)):
        live = (tm * TILE_M + row < M) & (tk * TILE_K + cl * COLS_PER_LANE < K)
        # a live lane's rows past M (M not a multiple of 16) fall outside
        in_rows = tm * TILE_M + row + r < M
        tile = tm * TILE_M * K + tk * TILE_K
        rx = Desc(2 * tile, 2 * M * K)
        rs = 2 * K
        off = np.where(live, row * rs + 2 * COLS_PER_LANE * cl, DEAD)
        ck.access("nv x", rx, off + r * rs, 16, live & in_rows,
                  2 * ((tm * TILE_M + row + r) * K + tk * TILE_K + COLS_PER_LANE * cl))
        if tm == tiles_m:
            continue
        ld = K >> 1
        rq = Desc(tm * TILE_M * ld + tk * (TILE_K // 2), M * ld)
        qoff = np.where(live, row * ld + 4 * cl, DEAD)
        ck.access("nv q_row", rq, qoff + r * ld, 4, live & in_rows,
                  (tm * TILE_M + row + r) * ld + tk * (TILE_K // 2) + 4 * cl)
        nb = K >> 4
        rrow = tm * TILE_M + t
        k0 = tk * TILE_K
        rs_ = Desc(tm * TILE_M * nb + (k0 >> 4), M * nb)
        o = np.where((t < TILE_M) & (rrow < M), t * nb, DEAD)
        if K % 256 == 0:
            ck.access("nv s_row", rs_, o, 16, (t < TILE_M) & (rrow < M), rrow * nb + (k0 >> 4))
        else:
            blocks = nb - (k0 >> 4)
            b = np.arange(TILE_K // 16)[:, None]
            lv = (b < blocks) & (t < TILE_M) & (rrow < M)
            ck.access("nv s_row bytes", rs_, np.where(b < blocks, o + b, DEAD), 1, lv,
                      rrow * nb + (k0 >> 4) + b)
    # nv_flush_q for the pair starting at each edge sub-tile (parts 1 and 2)
    for tm, tk, parts in itertools.product(edge(tiles_m), edge(tiles_k), (1, 2)):
        if rag:
            for first, last in ((True, False), (False, True), (True, True)):
                for site, d, off, nb_, lv, addr in model_nv_flush_q_rag(0, M, K, tm, tk, parts,
                                                                        first, last):
                    ck.access("nv q_col " + site, d, off, nb_, lv, addr)
            continue
        jr = t & 7
        m0, k0 = tm * TILE_M, tk * TILE_K
        ld = M >> 1
        rc = Desc(k0 * ld + (m0 >> 1), K * ld)
        row0 = m0 + 32 * jr
        in_pair = jr < 4 * parts
        kr = (t >> 3)[None, :] + 32 * np.arange(TILE_K // 32)[:, None]
        col_ok = in_pair & (k0 + kr < K)
        off = kr * ld + 16 * jr
        addr = (k0 + kr) * ld + (m0 >> 1) + 16 * jr
        if M % 32 == 0:
            lv = col_ok & (row0 < M)
            ck.access("nv q_col", rc, np.where(lv, off, DEAD), 16, lv, addr)
        else:
            lv = col_ok & (row0 < M)
            ck.access("nv q_col lo", rc, np.where(lv, off, DEAD), 8, lv, addr)
            lv = col_ok & (row0 + 16 < M)
            ck.access("nv q_col hi", rc, np.where(lv, off + 8, DEAD), 8, lv, addr + 8)
    nblk = (M + 15) >> 4
    for rg, tk in itertools.product(edge(groups_m), edge(tiles_k)):
        n = min(tiles_m - rg * group, group)
        tm0 = rg * group
        k0 = tk * TILE_K
        first = tm0 * (TILE_M // 16)
        count = min(nblk - first, 8 * n)
        rs_ = Desc(k0 * nblk + first, K * nblk)
        scale_rows(ck, "nv s_col", rs_, k0, K, nblk, first, count)
    return ck


MAXD = 1 << 23

MX_SHAPES = [(MAXD, 32), (MAXD, 8), (MAXD - 16, 40), (32, MAXD), (16, MAXD), (128, MAXD),
             (144, MAXD - 8), (1 << 17, MAXD), (MAXD, 1 << 17), (16400, 7176), (16384, 16384),
             # rows that are not multiples of 16: transposed rows at any byte
             (MAXD - 1, 8), (MAXD - 1, 1 << 17), ((1 << 17) - 1, MAXD), (1, MAXD), (17, MAXD - 8),
             (16383, 16384), (129, 7168)]


@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,K", MX_SHAPES)
@pytest.mark.parametrize("op", ["plain", "grad"])
def test_mx_quantize_offsets(M, K, op, tiled):
    mx_model(M, K, op, tiled).ok()


# gated: the quantised tensor is [M][N] with N <= 2^22 (full row 2N <= 2^23);
# gated backward: [M][2N].
GATED_N = [(MAXD, 8), (128, 1 << 22), (144, (1 << 22) - 8), (1 << 17, 1 << 22),
           (16, 1 << 22), (8192, 4096), (16400, 3592), (MAXD - 1, 8), (129, 1 << 22),
           (8191, 4096)]


@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,N", GATED_N)
def test_gated_offsets(M, N, tiled):
    mx_model(M, N, "gated", tiled).ok()


@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,N", GATED_N)
def test_dgated_offsets(M, N, tiled):
    mx_model(M, 2 * N, "dgated", tiled).ok()


NV_SHAPES = [(MAXD, 16), (16, MAXD), (128, MAXD), (144, MAXD - 16), (1 << 17, MAXD),
             (MAXD, 1 << 17), (16400, 7168), (16384, 16384),
             # rows that are not multiples of 16: transposed rows at any byte
             (MAXD - 1, 16), (MAXD - 1, 1 << 17), (1, MAXD), (17, MAXD - 16), ((1 << 17) - 1, MAXD),
             (16383, 16384), (129, 7168)]


@pytest.mark.parametrize("M,K", NV_SHAPES)
def test_nvfp4_offsets(M, K):
    nv_model(M, K).ok()


def test_model_sees_the_linear_half_overrun():
    """The model is sharp enough to see the fault it was written for: with the
    linear half's 2N bytes added to the lane offset (instead of to the
    descriptor's base), the last row's load at 2N = 2^23 ends at 2^31,
    past the largest descriptor."""
    M, N = 128, 1 << 22
    ck = Checker()
    ldx, K = 2 * N, 2 * N
    t, wave, half, cl, row = lanes()
    r = np.arange(ROWS_PER_LANE)[:, None]
    tk = -(-K // TILE_K) // 2 - 1                     # last strip of the gate half
    k = tk * TILE_K + COLS_PER_LANE * cl
    rx = Desc(0, 2 * M * ldx)
    ox = row * 2 * ldx + 2 * k
    ck.access("old linear", rx, ox + 2 * N + r * 2 * ldx, 16, np.ones_like(ox + r, dtype=bool))
    assert ck.bad and "past the descriptor" in ck.bad[0][1]


# ---------------------------------------------------------------------------
# The any-shape MXFP8 cast (mx_cast_any.hip): 64 x 128 steps, walks of up to
# 8 steps, one descriptor per row for the loads (scalar: the row is the same
# for every lane of a wave), staged stores in pieces of W = 16, 4 or 1 bytes.
# ---------------------------------------------------------------------------
ANY_M, ANY_K, ANY_WALK, ANY_TARGET = 64, 128, 8, 1024


def any_walk_len(rows, K):
    """any_walk_len (launch.h)."""
    tk = -(-K // ANY_K)
    L = ANY_WALK
    while L > 1:
        walks = sum(-(-(-(-r // ANY_M)) // L) for r in rows)
        if walks * tk >= ANY_TARGET:
            break
        L >>= 1
    return L


def tile_offset(r, b, RT):
    return ((b >> 3) * RT + (r >> 5)) * 256 + 4 * (32 * (b & 1) + (r & 31)) + ((b & 7) >> 1)


def piece_width(n):
    return 16 if n % 16 == 0 else 4 if n % 4 == 0 else 1


def model_flush_rows(site, base, stride, row0, col0, total, rows_left, seg, SEG):
    """flush_rows<SEG> (any_common.h): rows row0 .. row0 + rows_left - 1, each
    a segment of seg bytes at (row0 + r) * stride + col0; base: the output's
    start address modulo 64."""
    t = np.arange(THREADS)
    lane, wv = t & 63, t >> 6
    d = Desc(row0 * stride + col0, total)
    out = []
    if stride % 16 == 0 and base % 16 == 0:
        per = SEG // 16
        rows_per = 64 // per
        sub, p = lane // per, lane % per
        for i in range(ANY_M // (4 * rows_per)):
            for w in range(WAVES):
                sel = wv == w
                r = rows_per * (w + 4 * i) + sub
                ok = (r < rows_left) & (16 * p < seg)
                out.append((f"{site} W=16", d, np.where(ok, r * stride + 16 * p, DEAD)[sel], 16,
                            ok[sel], ((row0 + r) * stride + col0 + 16 * p)[sel]))
        return out
    per = SEG // 4
    rows_per = 64 // per
    for i in range(ANY_M // (4 * rows_per)):
        for w in range(WAVES):
            sel = wv == w
            r, u = rows_per * (w + 4 * i) + lane // per, lane % per
            al = (base + (row0 + r) * stride + col0) & 3
            head = np.minimum(seg, (4 - al) & 3)
            nd = (seg - head) >> 2
            i0 = head + 4 * u
            ok = (r < rows_left) & (u < nd)
            out.append((f"{site} W=4", d, np.where(ok, r * stride + i0, DEAD)[sel], 4, ok[sel],
                        ((row0 + r) * stride + col0 + i0)[sel]))
    for i in range(2):
        for w in range(WAVES):
            sel = wv == w
            r, slot = 8 * (w + 4 * i) + (lane >> 3), lane & 7
            al = (base + (row0 + r) * stride + col0) & 3
            head = np.minimum(seg, (4 - al) & 3)
            tail0 = head + 4 * ((seg - head) >> 2)
            b = np.where(slot < 3, slot, tail0 + slot - 3)
            ok = (r < rows_left) & np.where(slot < 3, slot < head, (slot < 6) & (b < seg))
            out.append((f"{site} W=1", d, np.where(ok, r * stride + b, DEAD)[sel], 1, ok[sel],
                        ((row0 + r) * stride + col0 + b)[sel]))
    return out


def model_flush_cols(site, base, tstride, k0, K, pos, rem, s, last, CH):
    """flush_cols<CH> (any_common.h): transposed rows k0 .. k0 + 127 of K,
    tstride bytes apart, this step's rem bytes at byte pos of each; base: the
    output's start address modulo 64."""
    t = np.arange(THREADS)
    npc = (CH // 16) * (2 if last else 1)
    d = Desc(k0 * tstride, K * tstride)
    out = []
    for i in range(ANY_K * npc // THREADS):
        idx = t + THREADS * i
        cc, j = idx // npc, idx % npc
        sft = (base + (k0 + cc) * tstride + pos) % CH
        lo = np.where(s > 0, 0, sft)
        hi = sft + rem
        co = cc * tstride + pos - sft
        row_ok = k0 + cc < K
        whole = row_ok & (lo <= 16 * j) & (16 * j + 16 <= hi)
        out.append((f"{site} W=16", d, np.where(whole, co + 16 * j, DEAD), 16, whole,
                    (k0 + cc) * tstride + pos - sft + 16 * j))
        part = row_ok & ~whole & (16 * j < hi) & (16 * j + 16 > lo)
        if part.any():
            b0 = np.where(lo > 16 * j, lo - 16 * j, 0)
            b1 = np.where(hi < 16 * j + 16, hi - 16 * j, 16)
            for size, go, b in range_stores(part, b0, b1, True):
                out.append((f"{site} W={size}", d, np.where(go, co + 16 * j + b, DEAD), size, go,
                            (k0 + cc) * tstride + pos - sft + 16 * j + b))
    return out


def any_sites(M, K, op, tiled, walk, tk, steps, qrow_base=0, qcol_base=0, L=None):
    """Every access of workgroup (walk, tk) for the given steps of its walk,
    as (site, descriptor, offsets, bytes, live, logical address) tuples."""
    if op == "gated":
        ldx, lin_off, ldg = 2 * K, K, 0
    elif op == "dgated":
        ldx, lin_off, ldg = K, K // 2, K // 2
    elif op == "grad":
        ldx, lin_off, ldg = K, 0, K
    else:
        ldx, lin_off, ldg = K, 0, 0
    L = L or any_walk_len([M], K)
    tiles_m, tiles_k = -(-M // ANY_M), -(-K // ANY_K)
    walks = -(-tiles_m // L)
    t = np.arange(THREADS)
    c, lane = t & 127, t & 63
    wv = t >> 6
    nbK, nbM = (K + 31) >> 5, (M + 31) >> 5
    t0 = walk * L
    n = min(L, tiles_m - t0)
    k0 = tk * ANY_K
    k = k0 + c
    col_ok = k < K
    out = []
    for s in steps:
        if s >= n:
            continue
        m0 = (t0 + s) * ANY_M
        # loads: thread (c, h) reads rows m0 + 32 h + i of column k through
        # one descriptor per operand from row m0 + 32 h (at the operand's
        # first column) to the tensor's end, row i at byte i * 2 ld of it
        for h in (0, 1):
            # the threads of half h (128 of them: columns c = 0..127)
            kh, okh = k[t >> 7 == h], col_ok[t >> 7 == h]
            mh = m0 + 32 * h
            for i in (0, 1, 15, 16, 30, 31):
                row = mh + i
                if op == "dgated":
                    N = lin_off
                    gate = kh < N
                    nn = np.where(gate, kh, kh - N)
                    ox = np.where(okh, 2 * nn, DEAD)
                    ol = np.where(okh & gate, 2 * nn, DEAD)
                    live = okh & (row < M)
                    out.append(("any gate", Desc(2 * mh * ldx, 2 * M * ldx), ox + i * 2 * ldx, 2,
                                live, 2 * (row * ldx + nn)))
                    out.append(("any grad", Desc(2 * mh * ldg, 2 * M * ldg), ox + i * 2 * ldg, 2,
                                live, 2 * (row * ldg + nn)))
                    out.append(("any linear", Desc(2 * (mh * ldx + N), 2 * M * ldx),
                                ol + i * 2 * ldx, 2, live & gate, 2 * (row * ldx + N + nn)))
                    continue
                ox = np.where(okh, 2 * kh, DEAD)
                live = okh & (row < M)
                out.append(("any x", Desc(2 * mh * ldx, 2 * M * ldx), ox + i * 2 * ldx, 2, live,
                            2 * (row * ldx + kh)))
                if op == "gated":
                    out.append(("any linear", Desc(2 * (mh * ldx + lin_off), 2 * M * ldx),
                                ox + i * 2 * ldx, 2, live, 2 * (row * ldx + lin_off + kh)))
                elif op == "grad":
                    out.append(("any grad", Desc(2 * mh * ldg, 2 * M * ldg), ox + i * 2 * ldg, 2,
                                live, 2 * (row * ldg + kh)))
        # row scales: thread (r = t / 4, q = t % 4), block b = 4 tk + q
        r, q = t >> 2, t & 3
        blocks = [4 * tk + q]
        if tiled and tk + 1 == tiles_k and tk % 2 == 0:
            blocks.append(4 * tk + q + 4)
        for b in blocks:
            if not tiled:
                ok = (m0 + r < M) & (b < nbK)
                out.append(("any s_row", Desc(m0 * nbK, M * nbK), np.where(ok, r * nbK + b, DEAD),
                            1, ok, (m0 + r) * nbK + b))
            else:
                RT, CT = (M + 31) >> 5, (nbK + 7) >> 3
                base = tile_offset(m0, (4 * tk) & ~7, RT)
                ok = (m0 + r < 32 * RT) & (b < 8 * CT)
                to = tile_offset(m0 + r, b, RT)
                out.append(("any s_row tiled", Desc(base, RT * CT * 256),
                            np.where(ok, to - base, DEAD), 1, ok, to))
        krem = min(K - k0, ANY_K)
        mrem = min(M - m0, ANY_M)
        out += model_flush_rows("any q_row", qrow_base, K, m0, k0, M * K, mrem, krem, 128)
        out += model_flush_cols("any q_col", qcol_base, M, k0, K, m0, mrem, s, s == n - 1, 64)
    # column scales at the walk's end
    jb, cnt = 2 * t0, 2 * n
    last_walk = walk + 1 == walks
    if not tiled:
        idx = np.arange(ANY_K * 2 * ANY_WALK)
        cc, jj = idx // (2 * ANY_WALK), idx % (2 * ANY_WALK)
        ok = (jj < cnt) & (k0 + cc < K) & (jb + jj < nbM)
        out.append(("any s_col", Desc(k0 * nbM + jb, K * nbM), np.where(ok, cc * nbM + jj, DEAD), 1,
                    ok, (k0 + cc) * nbM + jb + jj))
    else:
        RT, CT = (K + 31) >> 5, (nbM + 7) >> 3
        jend = 8 * CT if last_walk else jb + cnt
        span = jend - jb
        base = tile_offset(k0, jb & ~7, RT)
        idx = np.arange(ANY_K * span)
        cc, jj = idx // span, idx % span
        kk, j = k0 + cc, jb + jj
        ok = (kk < 32 * RT) & (j < 8 * CT)
        to = tile_offset(kk, j, RT)
        out.append(("any s_col tiled", Desc(base, RT * CT * 256), np.where(ok, to - base, DEAD), 1,
                    ok, to))
    # dbias partials
    ok = (t < ANY_K) & (k < K)
    out.append(("any partials", Desc(4 * (walk * K + k0), 4 * walks * K),
                np.where(ok, 4 * (t & 127), DEAD), 4, ok, 4 * (walk * K + k)))
    return out


def any_model(M, K, op="plain", tiled=False, ck=None, qrow_base=0, qcol_base=0):
    """qrow_base, qcol_base: the outputs' start addresses modulo 64 (a group
    of a stack starts anywhere)."""
    ck = ck or Checker()
    L = any_walk_len([M], K)
    tiles_m, tiles_k = -(-M // ANY_M), -(-K // ANY_K)
    walks = -(-tiles_m // L)
    for walk in edge(walks):
        n = min(L, tiles_m - walk * L)
        for tk in edge(tiles_k):
            for site, d, off, nbytes, live, addr in any_sites(M, K, op, tiled, walk, tk,
                                                              sorted({0, min(1, n - 1), n - 1}),
                                                              qrow_base, qcol_base):
                ck.access(site, d, off, nbytes, live, addr)
                base = qrow_base if "q_row" in site else qcol_base if "q_col" in site else 0
                a = np.broadcast_to(np.asarray(addr, dtype=np.int64), np.shape(live))[live]
                if nbytes > 1 and ((base + a) % nbytes != 0).any():
                    ck.bad.append((site, f"{nbytes}-byte store not {nbytes}-byte aligned"))
    return ck


ANY_SHAPES = [(MAXD, 1), (1, MAXD), (MAXD - 1, 9), (MAXD, 12), (MAXD, (1 << 17) - 1),
              ((1 << 17) - 3, MAXD), (17, MAXD - 1), (16383, 16383), (1, 1), (40, 64), (100, 36)]


@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,K", ANY_SHAPES)
@pytest.mark.parametrize("op", ["plain", "grad"])
def test_any_shape_offsets(M, K, op, tiled):
    any_model(M, K, op, tiled).ok()
    any_model(M, K, op, tiled, qrow_base=13, qcol_base=37).ok()


ANY_GATED_N = [(MAXD, 1), (128, (1 << 22) - 1), (17, 1 << 22), (MAXD - 1, 4), (16383, 4093)]


@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,N", ANY_GATED_N)
def test_any_shape_gated_offsets(M, N, tiled):
    any_model(M, N, "gated", tiled).ok()
    any_model(M, 2 * N, "dgated", tiled).ok()


@pytest.mark.parametrize("bases", [(0, 0), (5, 22), (16, 48)], ids=["b0", "b5-22", "b16-48"])
@pytest.mark.parametrize("tiled", [False, True], ids=["compact", "tiled"])
@pytest.mark.parametrize("M,K", [(1, 1), (17, 9), (33, 40), (95, 130), (200, 300), (64, 520),
                                 (129, 257), (300, 12), (12, 300), (600, 64), (1100, 20)])
@pytest.mark.parametrize("walk", [None, 2, 3, 8], ids=["planned", "L2", "L3", "L8"])
def test_any_shape_writes_every_byte_once(M, K, tiled, bases, walk):
    """Over all workgroups and steps, every byte of q_row, q_col and of both
    scale tensors (compact, or the tile layout with its padding) is written
    exactly once, and nothing else is -- for the planned walk length and for
    forced longer walks (whose transposed bytes carry across steps)."""
    L = walk or any_walk_len([M], K)
    tiles_m, tiles_k = -(-M // ANY_M), -(-K // ANY_K)
    walks = -(-tiles_m // L)
    nbK, nbM = (K + 31) >> 5, (M + 31) >> 5
    size = {"q_row": M * K, "q_col": K * M,
            "s_row": ((M + 31) >> 5) * ((nbK + 7) >> 3) * 256 if tiled else M * nbK,
            "s_col": ((K + 31) >> 5) * ((nbM + 7) >> 3) * 256 if tiled else K * nbM}
    count = {name: np.zeros(n, np.int64) for name, n in size.items()}
    for w in range(walks):
        for tk in range(tiles_k):
            for site, d, off, nbytes, live, addr in any_sites(M, K, "plain", tiled, w, tk,
                                                              range(L), *bases, L=L):
                name = next((nm for nm in count if site.startswith("any " + nm)), None)
                if name is None:
                    continue
                a = np.broadcast_to(addr, live.shape)[live]
                for b in range(nbytes):
                    np.add.at(count[name], a + b, 1)
    for name, cnt in count.items():
        assert (cnt == 1).all(), (name, int((cnt == 0).sum()), int((cnt > 1).sum()))


# ---------------------------------------------------------------------------
# NVFP4 of any shape (nvfp4_any.hip): the same walk, 16-element blocks, codes
# [rows][ceil(cols/2)] (64 bytes per row and 32 per transposed row per step),
# scales [rows][ceil(cols/16)].
# ---------------------------------------------------------------------------
def nv_any_sites(M, K, walk, tk, steps, qrow_base=0, qcol_base=0, L=None):
    L = L or any_walk_len([M], K)
    tiles_m = -(-M // ANY_M)
    t = np.arange(THREADS)
    c = t & 127
    t0 = walk * L
    n = min(L, tiles_m - t0)
    k0 = tk * ANY_K
    k = k0 + c
    lk, lm = -(-K // 2), -(-M // 2)
    nbk, nbm = -(-K // 16), -(-M // 16)
    out = []
    for s in steps:
        if s >= n:
            continue
        m0 = (t0 + s) * ANY_M
        mrem = min(M - m0, ANY_M)
        for h in (0, 1):
            kh = k[t >> 7 == h]
            mh = m0 + 32 * h
            for i in (0, 1, 30, 31):
                row = mh + i
                ok = (kh < K) & (row < M)
                out.append(("nv x", Desc(2 * mh * K, 2 * M * K),
                            np.where(kh < K, 2 * kh, DEAD) + i * 2 * K, 2, ok, 2 * (row * K + kh)))
        r, qq = t >> 2, t & 3
        for bq in (0, 1):
            b = 8 * tk + 2 * qq + bq
            ok = (m0 + r < M) & (b < nbk)
            out.append(("nv s_row", Desc(m0 * nbk, M * nbk), np.where(ok, r * nbk + b, DEAD), 1, ok,
                        (m0 + r) * nbk + b))
        out += model_flush_rows("nv q_row", qrow_base, lk, m0, 64 * tk, M * lk, mrem,
                                min(64, lk - 64 * tk), 64)
        out += model_flush_cols("nv q_col", qcol_base, lm, k0, K, m0 // 2, -(-mrem // 2), s,
                                s == n - 1, 32)
    idx = np.arange(ANY_K * 4 * ANY_WALK)
    cc, jj = idx // (4 * ANY_WALK), idx % (4 * ANY_WALK)
    jb = 4 * t0
    ok = (jj < 4 * n) & (k0 + cc < K) & (jb + jj < nbm)
    out.append(("nv s_col", Desc(k0 * nbm + jb, K * nbm), np.where(ok, cc * nbm + jj, DEAD), 1, ok,
                (k0 + cc) * nbm + jb + jj))
    return out


NV_ANY_SHAPES = [(MAXD, 1), (1, MAXD), (MAXD - 1, 9), (MAXD, 12), (MAXD, (1 << 17) - 1),
                 ((1 << 17) - 3, MAXD), (17, MAXD - 1), (16383, 16383), (1, 1), (40, 64)]


@pytest.mark.parametrize("M,K", NV_ANY_SHAPES)
def test_nvfp4_any_shape_offsets(M, K):
    for bases in ((0, 0), (13, 37)):
        ck = Checker()
        L = any_walk_len([M], K)
        tiles_m, tiles_k = -(-M // ANY_M), -(-K // ANY_K)
        walks = -(-tiles_m // L)
        for walk in edge(walks):
            n = min(L, tiles_m - walk * L)
            for tk in edge(tiles_k):
                for site, d, off, nbytes, live, addr in nv_any_sites(M, K, walk, tk,
                                                                     sorted({0, min(1, n - 1), n - 1}),
                                                                     *bases):
                    ck.access(site, d, off, nbytes, live, addr)
                    base = bases[0] if "q_row" in site else bases[1] if "q_col" in site else 0
                    a = np.broadcast_to(np.asarray(addr, dtype=np.int64), np.shape(live))[live]
                    if nbytes > 1 and "nv x" not in site and ((base + a) % nbytes != 0).any():
                        ck.bad.append((site, f"{nbytes}-byte store not {nbytes}-byte aligned"))
        ck.ok()


@pytest.mark.parametrize("bases", [(0, 0), (5, 22), (16, 48)], ids=["b0", "b5-22", "b16-48"])
@pytest.mark.parametrize("M,K", [(1, 1), (17, 9), (33, 40), (95, 130), (200, 300), (64, 520),
                                 (129, 257), (300, 12), (12, 300), (600, 64), (1100, 20)])
@pytest.mark.parametrize("walk", [None, 2, 3, 8], ids=["planned", "L2", "L3", "L8"])
def test_nvfp4_any_shape_writes_every_byte_once(M, K, bases, walk):
    L = walk or any_walk_len([M], K)
    tiles_m, tiles_k = -(-M // ANY_M), -(-K // ANY_K)
    walks = -(-tiles_m // L)
    size = {"q_row": M * -(-K // 2), "s_row": M * -(-K // 16),
            "q_col": K * -(-M // 2), "s_col": K * -(-M // 16)}
    count = {name: np.zeros(n, np.int64) for name, n in size.items()}
    for w in range(walks):
        for tk in range(tiles_k):
            for site, d, off, nbytes, live, addr in nv_any_sites(M, K, w, tk, range(L), *bases, L=L):
                name = next((nm for nm in count if site.startswith("nv " + nm)), None)
                if name is None:
                    continue
                a = np.broadcast_to(addr, live.shape)[live]
                for b in range(nbytes):
                    np.add.at(count[name], a + b, 1)
    for name, cnt in count.items():
        assert (cnt == 1).all(), (name, int((cnt == 0).sum()), int((cnt > 1).sum()))
