"""The kernels' integer-only divisions, emulated exactly on the CPU.

div_exact (tile raster and the int8 k rotation): floor(n / d) as the high 64
bits of 2n * ceil(2^63 / d), claimed exact for 0 <= n < 2^31, 1 <= d <= 2^31.
udiv_small_quotient (the integer ln): restoring division for quotients below
2^31.  Both replace runtime divisions that the compiler would lower through a
float32 reciprocal estimate."""
import numpy as np


def div_magic(d):
    return (1 << 63) // d + ((1 << 63) % d != 0)


def div_exact(n, m):
    return ((2 * n) * m) >> 64


def udiv_small_quotient(n, d):
    q = 0
    for b in range(30, -1, -1):
        t = d << b
        if n >= t:
            n -= t
            q |= 1 << b
    return q


def test_div_exact_matches_floor_division():
    rng = np.random.default_rng(0)
    ds = [1, 2, 3, 5, 7, 8, 127, 255, 1000, 65535, 2 ** 20 + 1, 2 ** 30 - 1, 2 ** 30,
          2 ** 31 - 1, 2 ** 31] + [int(v) for v in rng.integers(1, 2 ** 31, 200)]
    for d in ds:
        m = div_magic(d)
        ns = {0, 1, d - 1, d, d + 1, 2 ** 31 - 1, (2 ** 31 - 1) // d * d,
              (2 ** 31 - 1) // d * d - 1} | {int(v) for v in rng.integers(0, 2 ** 31, 300)}
        for k in range(1, 6):
            ns |= {k * d - 1, k * d}
        for n in ns:
            if 0 <= n < 2 ** 31:
                assert div_exact(n, m) == n // d, (n, d)


def test_div_exact_small_divisors_exhaustive():
    """The raster divides by 1..8 and by 8 * grid_n: every n below 2^20."""
    n = np.arange(1 << 20, dtype=object)
    for d in range(1, 9):
        m = div_magic(d)
        assert all(div_exact(int(v), m) == int(v) // d for v in n[::97])


def test_udiv_small_quotient():
    rng = np.random.default_rng(1)
    for _ in range(2000):
        f = int(rng.integers(0, 2 ** 30))
        den = (2 << 30) + f
        n, d = 2 * (f << 30) + den, 2 * den
        assert udiv_small_quotient(n, d) == n // d


# ---------------------------------------------- packed W addresses of the tile
def swz(bkb, row):
    if bkb == 64:
        return (row >> 2) & 3
    if bkb == 128:
        return (row >> 1) & 7
    return row & 15


def packed_offset(v, k, R):
    """The header's formula for byte k of row v in the packed layout."""
    return (v // 128) * (128 * R + 16384) + (k // 128) * 16384 + (v % 128) * 128 + k % 128


def packed_bytes(V, R):
    """The header's size of the packed layout."""
    return (V + 127) // 128 * (128 * R + 16384)


def test_tile_packed_w_addresses():
    """The float head's tile kernel splits each packed W address into a
    per-lane part (fixed for the launch) and a per-stage part; emulated here
    for every tile width, stage width and row length the float plans use, with
    rows past V re-reading row V - 1: every lane of every stage must read the
    byte the row-major tile reads, at its packed position."""
    for R in (128, 384, 512, 1536, 4096):
        for BN in (128, 256):
            for BKB in (64, 128, 256, 512):
                if R % BKB:
                    continue
                nst, spans = R // BKB, BN * BKB // 1024
                for n0, V in ((0, 10 ** 6), (BN, BN + 77), (3 * BN, 3 * BN + 129)):
                    for span in range(spans):
                        for lane in range(64):
                            off = span * 1024 + lane * 16
                            row = min(n0 + off // BKB, V - 1) - n0
                            kb = 16 * (((off % BKB) >> 4) ^ swz(BKB, off // BKB))
                            woff = (row // 128) * (128 * R + 16384) + (
                                (kb // 128) * 16384 + (row % 128) * 128 + kb % 128)
                            assert woff < 2 ** 32
                            for s in range(nst):
                                o = s * BKB
                                wk = (o // 128) * 16384 + o % 128
                                got = (n0 // 128) * (128 * R + 16384) + wk + woff
                                assert got == packed_offset(n0 + row, o + kb, R), \
                                    (R, BN, BKB, n0, span, lane, s)
                                assert got + 16 <= packed_bytes(V, R)


# ------------------------------------------------- workgroup -> tile mapping
K_TILE_GROUP = 8  # row tiles walked per vocabulary tile


def tile_of(bid, G, grid_m, grid_n, w_packed, bm=128):
    """The tile kernel's map from workgroup id to (row tile, vocabulary tile),
    with its multiply-high divisions (bm: rows per tile)."""
    per = G >> 3
    if bm <= 128 and grid_m == 1 and w_packed:
        nb = bid
    elif bid < (per << 3):
        nb = (bid & 7) * per + (bid >> 3)
    else:
        nb = bid
    in_group = K_TILE_GROUP * grid_n
    group = div_exact(nb, div_magic(in_group))
    first_m = group * K_TILE_GROUP
    gsz = min(grid_m - first_m, K_TILE_GROUP)
    rem = nb - group * in_group
    tn = div_exact(rem, div_magic(gsz))
    return first_m + (rem - tn * gsz), tn


def test_tile_map_is_a_bijection():
    """Every grid the plans launch (any row tile count, vocabulary tile counts
    around the multiples of 8, both W layouts): each tile is computed by
    exactly one workgroup."""
    grid_ns = sorted({1, 2, 7, 8, 9, 63, 125, 126, 250, 251, 256, 257, 501, 1002} |
                     {8 * k + r for k in (15, 31) for r in range(8)})
    for grid_m in (1, 2, 3, 7, 8, 9, 16, 17):
        for grid_n in grid_ns:
            G = grid_m * grid_n
            for w_packed, bm in ((False, 128), (True, 128), (True, 256)):
                tiles = {tile_of(b, G, grid_m, grid_n, w_packed, bm) for b in range(G)}
                assert len(tiles) == G, (grid_m, grid_n, w_packed, bm)
                assert all(0 <= tm < grid_m and 0 <= tn < grid_n for tm, tn in tiles)


# ------------------------------------- top-2 of a tile with few live rows
# Lane pairings of the 32 column lanes of a wave half (ds_swizzle and DPP row
# permutations) and the lane bit each halving step keeps.
PAIR = {"x16": 16, "mirror": 15, "half_mirror": 7, "quad2": 2, "quad1": 1}
KEEP = {"x16": 16, "mirror": 8, "half_mirror": 4}


def _merge(a, b):
    s = sorted(set(a) | set(b), reverse=True)
    return (s[0], s[1])


def _halve(a, p, r):
    out = [list(x) for x in a]
    for j in range(32):
        q = j ^ PAIR[p]
        lo, qlo = (j & KEEP[p]) == 0, (q & KEEP[p]) == 0
        for i in range(r // 2):
            mine = a[j][i] if lo else a[j][i + r // 2]
            theirs = a[q][i + r // 2] if qlo else a[q][i]
            out[j][i] = _merge(mine, theirs)
    return out


def _full(a, p):
    return [[_merge(a[j][0], a[j ^ PAIR[p]][0])] + a[j][1:] for j in range(32)]


def acc_row(v, h):
    return 8 * (v >> 2) + 4 * h + (v & 3)


def test_few_live_rows_top2_lane_steps():
    """The top-2 epilogue of a tile with at most 16 live rows ranks NV = 1, 4
    or 8 accumulator values per lane: halving steps on j^16, j^15, j^7 (as
    many as NV needs), full merges on the rest of j^16, j^15, j^7, j^2, j^1.
    Emulated on random distinct keys: each writer lane (one per live row)
    must hold the brute-force top-2 of its row over all 32 column lanes, and
    the writers must cover exactly the rows of those values."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        for nv in (1, 4, 8):
            for h in (0, 1):
                keys = rng.choice(10 ** 9, size=(32, 16, 2), replace=False)
                a = [[tuple(sorted(map(int, keys[j, v]), reverse=True)) for v in range(16)]
                     for j in range(32)]
                steps = ["x16", "mirror", "half_mirror"]
                halvings = {1: 0, 4: 2, 8: 3}[nv]
                for s, p in enumerate(steps):
                    a = _halve(a, p, nv >> s) if s < halvings else _full(a, p)
                a = _full(_full(a, "quad2"), "quad1")
                rows = {}
                for j in range(32):
                    u = ((4 * ((j >> 4) & 1) + 2 * ((j >> 3) & 1) + ((j >> 2) & 1)) if nv == 8
                         else (2 * ((j >> 4) & 1) + ((j >> 3) & 1)) if nv == 4 else 0)
                    if (j & (32 // nv - 1)) == 0 and (nv > 1 or h == 0):
                        want = sorted({int(k) for k in keys[:, u].ravel()}, reverse=True)[:2]
                        assert a[j][0] == tuple(want), (trial, nv, h, j)
                        rows[acc_row(u, h)] = j
                expect = {acc_row(v, h) for v in range(nv)} if (nv > 1 or h == 0) else set()
                assert set(rows) == expect, (nv, h)
