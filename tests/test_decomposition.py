"""The balanced work split of the decode and prefill kernels, replayed on the CPU.

Host logic only: these functions restate, in Python, the index formulas the
kernels use (unit ranges per workgroup, the slot of each piece, the pieces the
merge reads back), and check over many random shapes that every unit is
processed exactly once, that every slot is unique and inside the workspace the
host sizes, and that each merge reads exactly the pieces written for its
segment.  A mistake in the scheme (an off-by-one in the owner formula, a slot
collision, a merge that skips or double-counts a piece) fails here without a GPU.
"""
from __future__ import annotations

import math
import random

import pytest


def steps_of(c):
    return (c + 15) >> 4 if c > 0 else 0


def begin(w, U, W):
    return w * U // W


def owner(x, U, W):
    return ((x + 1) * W - 1) // U


DEC_OV = {"f32": 2, "bf16": 2, "fp8": 6, "int8": 6, "int4": 6}   # decode_seg_ov (internal.h)
DEC_WT_EVEN, DEC_WT_ODD = 17, 16   # decode split weights by XCD parity (decode.hip)


def dec_weighted(W):
    return W % 8 == 0 and W <= 1 << 17


def dec_wsum(w):
    return DEC_WT_EVEN * ((w + 1) // 2) + DEC_WT_ODD * (w // 2)


def dec_begin(w, U, W):
    """wave_begin: floor(U S(w) / S(W)) in double precision, as the kernel takes it."""
    if dec_weighted(W):
        return int(math.floor(float(U) * float(dec_wsum(w)) / float(dec_wsum(W))))
    return int(math.floor(float(w) * float(U) / float(W)))


def dec_owner(x, U, W):
    """wave_of: the unweighted owner, corrected by single steps."""
    w = int(math.floor((float(x + 1) * float(W) - 1.0) / float(U)))
    if not dec_weighted(W):
        return w
    w = min(max(w, 0), W - 1)
    while w > 0 and dec_begin(w, U, W) > x:
        w -= 1
    while w + 1 < W and dec_begin(w + 1, U, W) <= x:
        w += 1
    return w


def replay_decode(ctx, n_kv, hw, W, ov=DEC_OV["int8"]):
    """Decode: units (sequence, head group, 16-token step), hw waves per
    workgroup; a segment with steps holds its steps after ov start-up units."""
    B, nhg = len(ctx), n_kv // hw
    cu = [0]
    for c in ctx:
        cu.append(cu[-1] + nhg * (steps_of(c) + ov if c > 0 else 0))
    U = cu[-1]
    entries = (W + B * nhg) * hw
    written, covered, seg_w = {}, [0] * (sum(nhg * steps_of(c) for c in ctx) * hw), {}
    scu = [0]
    for c in ctx:
        scu.append(scu[-1] + nhg * steps_of(c))
    for w in range(W):
        u0, u1 = dec_begin(w, U, W), dec_begin(w + 1, U, W)
        if u0 >= u1:
            continue
        s = next(i for i in range(B) if cu[i + 1] > u0)
        ln = steps_of(ctx[s]) + ov
        hg, off = (u0 - cu[s]) // ln, (u0 - cu[s]) % ln
        u = u0
        while True:
            steps = steps_of(ctx[s])
            end = min(steps + ov, off + (u1 - u))
            sb, se = max(off - ov, 0), max(end - ov, 0)
            slot = w + s * nhg + hg
            if se > sb:
                if sb == 0:                            # the kernel records the segment's
                    seg_w.setdefault((s, hg), [None, None])[0] = w   # first and last
                if se == steps:                        # steps' workgroups for the merge
                    seg_w.setdefault((s, hg), [None, None])[1] = w
                for wv in range(hw):
                    e = slot * hw + wv
                    assert 0 <= e < entries and e not in written
                    written[e] = (s, hg * hw + wv, sb, se)
                    for t in range(sb, se):
                        covered[(scu[s] + hg * steps + t) * hw + wv] += 1
            u += end - off
            if u >= u1:
                break
            off, hg = 0, hg + 1
            if hg == nhg:
                hg, s = 0, s + 1
                while steps_of(ctx[s]) == 0:
                    s += 1
    assert all(c == 1 for c in covered)
    b = [dec_begin(w, U, W) for w in range(W + 1)]
    assert b[0] == 0 and b[W] == U and all(x <= y for x, y in zip(b, b[1:]))
    if U >= 2 * W:
        assert all(x < y for x, y in zip(b, b[1:]))   # the merge's shortcut: no empty share
    read = set()
    for s in range(B):
        st = steps_of(ctx[s])
        if st == 0:
            continue
        for kvh in range(n_kv):
            hg, wv = kvh // hw, kvh % hw
            g0, g = cu[s] + hg * (st + ov) + ov, s * nhg + hg   # first step's unit
            w0, w1 = seg_w[(s, hg)]
            assert (w0, w1) == (dec_owner(g0, U, W), dec_owner(g0 + st - 1, U, W))
            assert (w0 + g) * hw + wv in written             # the merge's dummy piece exists
            got = 0
            for w in range(w0, w1 + 1):
                if dec_begin(w, U, W) >= dec_begin(w + 1, U, W):
                    continue                       # an empty workgroup holds no piece
                e = (w + g) * hw + wv
                assert e in written and written[e][:2] == (s, kvh)
                got += written[e][3] - written[e][2]
                read.add(e)
            assert got == st
    assert read == set(written)


PF_OV = 8                        # start-up units per segment with tiles (prefill.hip)
PF_WT = (64, 51, 39, 36)         # split weights of the dispatch rounds (prefill.hip)
PF_XW = (33, 32)                 # split weights of workgroups on even / odd XCDs
XCDS = 8


def pf_wsum(w, W, C, wt=PF_WT, xw=PF_XW):
    """Sum of the split weights of workgroups [0, w) in the XCD-local work order."""
    if not (C > 0 and C % XCDS == 0 and W % C == 0 and W // C <= 4 and W % XCDS == 0):
        return 64 * w
    M, P, R = W // XCDS, C // XCDS, W // C
    perx = sum(P * wt[r] for r in range(R))
    q, k = divmod(w, M)
    rk = k // P
    inside = sum(P * wt[r] for r in range(rk)) + (k - rk * P) * wt[rk] if q < XCDS else 0
    return ((q + 1) // 2 * xw[0] + q // 2 * xw[1]) * perx + xw[q % 2] * inside


def pf_split(U, W, C, wt=PF_WT, xw=PF_XW):
    """wg_begin: workgroup w takes units [b[w], b[w + 1])."""
    S = pf_wsum(W, W, C, wt, xw)
    return [U * pf_wsum(w, W, C, wt, xw) // S for w in range(W + 1)]


def prefill_planner_starts(cu, wgb):
    """The planner's step 4: each workgroup's first (segment, unit offset) and
    each segment's first workgroup, by binary search as the kernel does."""
    nseg, W, U = len(cu) - 1, len(wgb) - 1, cu[-1]
    start = {}
    for w in range(W):
        x = wgb[w]
        if x >= wgb[w + 1]:
            continue
        lo, hi = 0, nseg
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if cu[mid] <= x:
                lo = mid
            else:
                hi = mid
        start[w] = (lo, x - cu[lo])
    w0 = {}
    for g in range(nseg):
        if cu[g + 1] <= cu[g]:
            continue
        lo, hi = 0, W
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if wgb[mid] <= cu[g]:
                lo = mid
            else:
                hi = mid
        w0[g] = lo
    return start, w0


def pf_tile_order(split, tfull):
    """The kernel's key-tile order in a segment: step i < tfull computes tile
    (i + rot) mod tfull, rot chosen so that step `split` (where the segment's
    first split point falls) computes tile 0; the masked tiles follow in order."""
    rot = (tfull - split % tfull) % tfull if tfull > 0 else 0
    return lambda i: (i + rot) % tfull if i < tfull else i


def replay_prefill(tiles, W, C=0, wt=PF_WT, ov=PF_OV, tfull=None):
    """Prefill: a segment with n key tiles holds n + ov units (start-up units
    first); workgroup w takes units [wg_begin[w], wg_begin[w + 1]); a piece of
    workgroup w in segment g -> slot w + g, computing the steps of its range in
    the rotated tile order (tiles below tfull[g] rotated); the merge walks the
    workgroups from seg_w0[g] and reads the pieces with tiles.  Returns, per
    segment, the first tile of each piece in order."""
    if tfull is None:
        tfull = list(tiles)
    units = [n + ov if n > 0 else 0 for n in tiles]
    cu = [0]
    for n in units:
        cu.append(cu[-1] + n)
    U, nseg = cu[-1], len(tiles)
    wgb = pf_split(U, W, C, wt)
    assert wgb[0] == 0 and wgb[W] == U and all(a <= b for a, b in zip(wgb, wgb[1:]))
    start, w0 = prefill_planner_starts(cu, wgb)
    written, covered = {}, [[0] * n for n in tiles]
    firsts = [[] for _ in tiles]
    for w in range(W):
        u0, u1 = wgb[w], wgb[w + 1]
        if u0 >= u1:
            continue
        g, off = start[w]
        assert cu[g] <= u0 < cu[g + 1]
        u = u0
        while True:
            nu = cu[g + 1] - cu[g]
            end = min(nu, off + (u1 - u))
            tb, te = max(off - ov, 0), max(end - ov, 0)
            if te > tb:
                if not (tb == 0 and te == nu - ov):
                    slot = w + g
                    assert slot < W + nseg and slot not in written
                    written[slot] = (g, tb, te)
                split = max(wgb[w0[g] + 1] - cu[g] - ov, 0)
                order = pf_tile_order(split, tfull[g])
                if tb == split and split < tfull[g]:
                    assert order(tb) == 0
                firsts[g].append(order(tb))
                for t in range(tb, te):
                    covered[g][order(t)] += 1
            u += end - off
            if u >= u1:
                break
            g, off = g + 1, 0
            while cu[g + 1] == cu[g]:
                g += 1
    assert all(c == 1 for row in covered for c in row)
    read = set()
    for g in range(nseg):
        c0, c1 = cu[g], cu[g + 1]
        if c1 <= c0:
            continue
        w = w0[g]
        assert wgb[w] <= c0 < wgb[w + 1]
        if wgb[w + 1] >= c1:
            assert (w + g) not in written          # written whole by one workgroup
            continue
        got, whole = 0, False
        while w < W and wgb[w] < c1:
            b, e = max(wgb[w], c0) - c0, min(wgb[w + 1], c1) - c0
            tb, te = max(b - ov, 0), max(e - ov, 0)
            if te > tb:
                if tb == 0 and te == tiles[g]:
                    whole = True
                    break
                assert written[w + g] == (g, tb, te)
                got += te - tb
                read.add(w + g)
            w += 1
        assert whole or got == tiles[g]
    assert read == set(written)
    return firsts


def test_decode_weighted_split_owner_and_exactness():
    """With the XCD-parity weights, wave_of's corrected owner holds each unit,
    odd workgroups take 16/17 of an even one's share, and the double-precision
    quotient equals the integer one up to U < 2^31, W = 2^17."""
    rng = random.Random(11)
    for _ in range(200):
        W = 8 * rng.randint(1, 200)
        U = rng.randint(1, 60 * W)
        for x in sorted(rng.sample(range(U), min(U, 300))) + [0, U - 1]:
            w = dec_owner(x, U, W)
            assert dec_begin(w, U, W) <= x < dec_begin(w + 1, U, W)
    W, U = 256, 10 ** 6
    sh = [dec_begin(w + 1, U, W) - dec_begin(w, U, W) for w in range(W)]
    even, odd = sum(sh[0::2]), sum(sh[1::2])
    assert abs(odd / even - DEC_WT_ODD / DEC_WT_EVEN) < 1e-3
    for U in (2 ** 31 - 1, 2 ** 31 - 12345, 987654321):
        W = 1 << 17
        for w in [0, 1, 2, 3, W // 3, W // 2 + 1, W - 2, W - 1, W] + rng.sample(range(W), 200):
            assert dec_begin(w, U, W) == U * dec_wsum(w) // dec_wsum(W)


@pytest.mark.parametrize("seed", range(4))
def test_decode_split_covers_every_unit_once(seed):
    rng = random.Random(seed)
    for _ in range(300):
        B = rng.randint(1, 12)
        n_kv = rng.choice([1, 2, 4, 8, 16, 32])
        hw = rng.choice([h for h in (1, 2, 4, 8) if n_kv % h == 0])
        ctx = [rng.choice([0, 0, 1, 15, 16, 17, rng.randint(1, 300)]) for _ in range(B)]
        if sum(ctx) == 0:
            continue
        for W in (1, 2, 3, 7, 8, 64, 256, 1000, 1024):
            replay_decode(ctx, n_kv, hw, W)
            replay_decode(ctx, n_kv, hw, W, ov=DEC_OV["bf16"])
            replay_decode(ctx, n_kv, hw, W, ov=rng.choice([0, 1, 7]))


@pytest.mark.parametrize("seed", range(4))
def test_prefill_split_covers_every_tile_once(seed):
    rng = random.Random(100 + seed)
    for _ in range(300):
        tiles = [rng.choice([0, 1, 2, 5, rng.randint(1, 40)]) for _ in range(rng.randint(1, 10))]
        if sum(tiles) == 0:
            continue
        tfull = [max(0, n - rng.choice([0, 0, 1, 2, n])) for n in tiles]
        for W, C in ((1, 0), (2, 0), (3, 0), (5, 0), (17, 0), (256, 0), (768, 256), (24, 8),
                     (512, 256), (1024, 256), (17, 256), (912, 304)):
            replay_prefill(tiles, W, C, tfull=tfull)
            replay_prefill(tiles, W, C, wt=(7, 5, 3, 1), ov=rng.choice([0, 1, 5]), tfull=tfull)


def test_prefill_tile_order_aligns_the_split_points():
    """Equal segments split at equal unit counts: the pieces that start at the
    k-th split point of each segment start at the same key tile (the first split
    point at tile 0), so the query tiles of one (sequence, KV head) read the same
    K/V tiles at the same time."""
    for n, nseg, W in ((92, 16, 64), (92, 16, 48), (1040, 16, 80)):
        units = (n + PF_OV) * nseg
        if units % W:
            continue
        firsts = replay_prefill([n] * nseg, W, 0, ov=PF_OV)
        A = units // W
        heads = [f for f in firsts if len(f) > 1]
        assert heads
        for f in heads:
            assert f[1] == 0
            assert f[1:] == [(k * A) % n for k in range(len(f) - 1)]


PF_ROWS, PF_BN = 128, 32


def prefill_plan(lens, ctx, n_kv, G, causal, route=False):
    """The prefill planner's segment list: for each sequence, each KV head, each
    query tile of QB = 128 / G queries; per segment the key tiles its last query needs.
    With route (blocks of 16 tokens or more) a sequence of one query has no segment:
    it goes to the decode path instead (prefill_decode_rows)."""
    QB = PF_ROWS // G
    segs = []
    for s, (L, T) in enumerate(zip(lens, ctx)):
        nq = 0 if route and L == 1 else -(-L // QB)
        for kvh in range(n_kv):
            for qt in range(nq):
                last = min(L, (qt + 1) * QB) - 1
                vis = min(T, T - L + last + 1) if causal else T
                segs.append((s, kvh, qt, -(-vis // PF_BN) if vis > 0 else 0))
    return segs


def nseg_bound(num_seqs, total_q, max_q, n_kv, G):
    """The workspace's segment bound, as the host computes it."""
    QB = PF_ROWS // G
    return n_kv * min((total_q + num_seqs * (QB - 1)) // QB, num_seqs * -(-max_q // QB))


@pytest.mark.parametrize("seed", range(4))
def test_prefill_plan_covers_every_row_once(seed):
    """Ragged batches of chunks and decode rows (L = 1): each (sequence, query, head)
    row lies in exactly one segment, under the workspace bound, and its segment
    holds every key tile the row sees; the split of those tiles is then replayed."""
    rng = random.Random(200 + seed)
    for _ in range(200):
        B = rng.randint(1, 12)
        n_kv = rng.choice([1, 2, 8])
        G = rng.choice([1, 2, 4, 8])
        QB = PF_ROWS // G
        causal = rng.random() < 0.7
        lens = [rng.choice([0, 1, 1, 1, QB - 1, QB, QB + 1, rng.randint(1, 400)]) for _ in range(B)]
        ctx = [L + rng.choice([0, 0, 1, 31, 32, rng.randint(0, 500)]) for L in lens]
        segs = prefill_plan(lens, ctx, n_kv, G, causal)
        assert len(segs) <= nseg_bound(B, sum(lens), max(lens), n_kv, G)
        seen = {}
        for g, (s, kvh, qt, tiles) in enumerate(segs):
            T, L = ctx[s], lens[s]
            for rr in range(PF_ROWS):                  # query-major rows of the segment
                qi, h = qt * QB + rr // G, rr % G
                wave_ok = qt * QB + (rr // 32) * 32 // G < L
                if qi < L:
                    assert wave_ok
                    key = (s, qi, kvh * G + h)
                    assert key not in seen
                    seen[key] = g
                    last_key = (T - L + qi) if causal else T - 1
                    assert last_key < tiles * PF_BN  # the segment loads every key it sees
        assert len(seen) == sum(lens) * n_kv * G
        tiles = [t for (_, _, _, t) in segs]
        tfull = []
        for (s, _, qt, _) in segs:                       # tiles every row of the segment sees
            T, L = ctx[s], lens[s]
            tfull.append(min(T, T - L + qt * QB + 1 if causal else T) // PF_BN)
        if sum(tiles):
            for W, C in ((1, 0), (3, 0), (64, 0), (1000, 0), (768, 256)):
                replay_prefill(tiles, W, C, tfull=tfull)


def decode_row_lists(lens, ctx):
    """The planner's lists for the decode path: per sequence, the context when its
    chunk is one query long (else 0) and that query's row of q and out (else -1)."""
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    row_ctx = [T if L == 1 else 0 for L, T in zip(lens, ctx)]
    row_map = [cu[s] if L == 1 else -1 for s, L in enumerate(lens)]
    return row_ctx, row_map


@pytest.mark.parametrize("seed", range(4))
def test_prefill_plan_with_decode_rows_covers_every_row_once(seed):
    """With the rows of length 1 on the decode path, every (sequence, query, head)
    row is computed exactly once: by a segment of the tile kernel or, for a
    one-query chunk, by the decode split over row_ctx / row_map (whose units are
    the sequence's whole context, the key range a one-query chunk sees, causal or
    not).  The decode merge writes exactly the mapped rows."""
    rng = random.Random(400 + seed)
    for _ in range(200):
        B = rng.randint(1, 12)
        n_kv = rng.choice([1, 2, 8])
        G = rng.choice([1, 2, 4, 8])
        QB = PF_ROWS // G
        causal = rng.random() < 0.7
        lens = [rng.choice([0, 1, 1, 1, 2, QB, QB + 1, rng.randint(1, 400)]) for _ in range(B)]
        ctx = [L + rng.choice([0, 0, 1, 31, 32, rng.randint(0, 500)]) for L in lens]
        segs = prefill_plan(lens, ctx, n_kv, G, causal, route=True)
        assert len(segs) <= nseg_bound(B, sum(lens), max(lens), n_kv, G)
        row_ctx, row_map = decode_row_lists(lens, ctx)
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        seen = {}
        for g, (s, kvh, qt, tiles) in enumerate(segs):
            assert lens[s] != 1
            for rr in range(PF_ROWS):
                qi, h = qt * QB + rr // G, rr % G
                if qi < lens[s]:
                    key = (cu[s] + qi, kvh * G + h)
                    assert key not in seen
                    seen[key] = ("tile", g)
        for s in range(B):
            if row_map[s] < 0:
                assert row_ctx[s] == 0
                continue
            assert lens[s] == 1 and row_map[s] == cu[s] and row_ctx[s] == ctx[s]
            # one query at position T - 1 sees keys [0, T): causal or not, the decode range
            last_key = ctx[s] - 1
            assert (ctx[s] - lens[s] + 0 if causal else ctx[s] - 1) == last_key
            for h in range(n_kv * G):
                key = (row_map[s], h)
                assert key not in seen
                seen[key] = ("decode", s)
        assert len(seen) == sum(lens) * n_kv * G
        # the mapped output rows are distinct rows of out
        mapped = [r for r in row_map if r >= 0]
        assert len(set(mapped)) == len(mapped) and all(0 <= r < sum(lens) for r in mapped)


def test_prefill_planner_workgroup_starts():
    """The planner's binary searches give workgroup w the segment whose units
    hold its first unit (never a segment of no units) and give each segment the
    workgroup holding its first unit; with equal weights the split is
    floor(w U / W), as in the decode kernel."""
    rng = random.Random(300)
    for _ in range(500):
        tiles = [rng.choice([0, 0, 1, 2, 7, rng.randint(1, 60)]) for _ in range(rng.randint(1, 30))]
        units = [n + PF_OV if n > 0 else 0 for n in tiles]
        U = sum(units)
        if U == 0:
            continue
        cu = [0]
        for n in units:
            cu.append(cu[-1] + n)
        for W, C in ((1, 0), (2, 0), (7, 0), (64, 0), (768, 256), (1024, 256), (768, 0)):
            wgb = pf_split(U, W, C)
            if C == 0:
                assert wgb == [begin(w, U, W) for w in range(W + 1)]
            start, w0 = prefill_planner_starts(cu, wgb)
            for w, (g, off) in start.items():
                assert units[g] > 0 and 0 <= off < units[g] and cu[g] + off == wgb[w]
            for g, w in w0.items():
                assert wgb[w] <= cu[g] < wgb[w + 1]


def test_prefill_split_weights_follow_the_rounds():
    """With three rounds of 256 CUs (768 workgroups in the XCD-local order), the
    workgroups of round r on XCD x take units in proportion PF_WT[r] PF_XW[x % 2]."""
    U, W, C = 10 ** 6, 768, 256
    wgb = pf_split(U, W, C)
    share = [wgb[w + 1] - wgb[w] for w in range(W)]
    total = (C // XCDS) * sum(PF_WT[:3]) * (XCDS // 2) * (PF_XW[0] + PF_XW[1])
    for w in range(W):
        x, k = divmod(w, W // XCDS)            # XCD, index inside the XCD's range
        r = k // (C // XCDS)                   # its dispatch round
        assert abs(share[w] - U * PF_WT[r] * PF_XW[x % 2] / total) <= 1


def row_g(t):
    """Chunk swizzle of token row t in the decode kernel's LDS rows."""
    return ((t & 7) << 1) | ((t >> 2) & 1)


# LDS bank groups as gfx950's SQ_LDS_BANK_CONFLICT counter shows them (one access
# pattern per probe kernel): 16-byte accesses are served 8 lanes at a time and
# conflict unless the 8 chunks differ in address bits 4..6; ds_read_b64_tr_b16 is
# served 32 lanes at a time and conflicts unless the 32 pieces differ in bits 3..7.
def b128_conflict_free(offsets):
    return all(len({(o >> 4) & 7 for o in offsets[g:g + 8]}) == 8 for g in range(0, 64, 8))


def tr64_conflict_free(offsets):
    return all(len({(o >> 3) & 31 for o in offsets[g:g + 32]}) == 32 for g in (0, 32))


def test_bank_model_separates_the_measured_patterns():
    """The model above reproduces what the counter showed: a conflict for the
    slice writes with row swizzle ((t & 7) << 1) | (t >> 3), for rows padded to
    288 bytes, and for transposed reads of a stage swizzled by c ^ t; none for
    row_g, linear runs or the padded rows' transposed reads."""
    lanes = [(l >> 4, l & 15) for l in range(64)]
    old_g = lambda t: ((t & 7) << 1) | ((t >> 3) & 1)
    assert not b128_conflict_free([r * 256 + 16 * ((2 * j) ^ old_g(r)) for j, r in lanes])
    assert not b128_conflict_free([r * 288 + 32 * j for j, r in lanes])
    assert b128_conflict_free([r * 256 + 16 * ((2 * j) ^ row_g(r)) for j, r in lanes])
    assert b128_conflict_free([16 * l for l in range(64)])
    tr = lambda j, r: (4 * j + (r >> 2), (r >> 1) & 1, 8 * (r & 1))
    assert not tr64_conflict_free([t * 1024 + 16 * (cb ^ t) + h for t, cb, h in (tr(j, r) for j, r in lanes)])
    assert tr64_conflict_free([t * 1024 + 16 * (cb ^ row_g(t)) + h for t, cb, h in (tr(j, r) for j, r in lanes)])
    assert tr64_conflict_free([t * 288 + 16 * cb + h for t, cb, h in (tr(j, r) for j, r in lanes)])
    assert tr64_conflict_free([8 * l for l in range(64)])


def stage_maps(hw, row):
    """The staged decode load maps for one head group: per (wave, lane, k) the
    (token, 16-byte chunk) a lane loads and the stage slot it writes, and per
    (wave, lane, piece) the slot it reads back."""
    rc = hw * row // 16                      # chunks per token row of the group
    loads = {}
    for wv in range(hw):
        for lane in range(64):
            for k in range(row // 64):
                q = (k * hw + wv) * 64 + lane
                t, c = q // rc, q % rc
                loads[(wv, lane, k)] = ((t, c), t * rc + (c ^ row_g(t)))
    reads = {}
    for wv in range(hw):
        for lane in range(64):
            j, r = lane >> 4, lane & 15
            for k in range(row // 64):
                c = wv * (row // 16) + j + 4 * k
                reads[(wv, lane, k)] = ((r, c), r * rc + (c ^ row_g(r)))
    return rc, loads, reads


@pytest.mark.parametrize("hw,row", [(8, 64), (4, 64), (8, 128), (4, 128), (2, 128), (8, 256),
                                    (1, 256), (4, 256)])
def test_decode_stage_maps(hw, row):
    """Every chunk of a step is loaded once, lands in a distinct stage slot, and
    each lane reads back the piece of its own head that the per-head layout
    gives it (token r, chunk j + 4k of head wv's row); the stage writes, the
    per-head reads and (bf16 rows) the transposed V reads meet no bank conflict
    in the model above."""
    rc, loads, reads = stage_maps(hw, row)
    assert (hw * row) % 256 == 0 and row >= 64          # where the kernel stages
    chunks = [tc for tc, _ in loads.values()]
    assert sorted(chunks) == [(t, c) for t in range(16) for c in range(rc)]
    slots = {pos: tc for tc, pos in loads.values()}
    assert len(slots) == 16 * rc and max(slots) < 16 * rc
    for key, (tc, pos) in reads.items():
        assert slots[pos] == tc, key
    for table in (loads, reads):
        for wv in range(hw):
            for k in range(row // 64):
                assert b128_conflict_free([16 * table[(wv, lane, k)][1] for lane in range(64)])
    if row % 128 == 0:
        # bf16 rows: the transposed V reads go to the stage directly.  Lane
        # (j, r) of head wv, block b wants the 8 bytes at 32 b + 8 (r % 4) of
        # token 4 j + r / 4's row: chunk 2 b + (r / 2) % 2, half r % 2.
        cpr = row // 16
        for wv in range(hw):
            for b in range(row // 32):
                offs = []
                for lane in range(64):
                    j, r = lane >> 4, lane & 15
                    t = 4 * j + (r >> 2)
                    c = wv * cpr + 2 * b + ((r >> 1) & 1)
                    pos = t * rc + (c ^ row_g(t))
                    assert slots[pos] == (t, c), (wv, lane, b)
                    offs.append(16 * pos + 8 * (r & 1))
                assert tr64_conflict_free(offs), (wv, b)


def test_decode_split_quotients_in_double_are_exact():
    """The decode kernels take floor(w U / W) and floor(((x + 1) W - 1) / U) in
    IEEE double precision (a correctly rounded division, then floor).  Check
    that this equals the integer quotient over the whole supported range: up to
    2^31 - 1 units and 2^20 workgroups, at the extremes and at random."""
    import numpy as np

    rng = np.random.default_rng(0)
    W_MAX, U_MAX = 1 << 20, (1 << 31) - 1
    Us = np.concatenate([[1, 2, 3, W_MAX - 1, W_MAX, W_MAX + 1, U_MAX - 1, U_MAX],
                         rng.integers(1, U_MAX, 4000, endpoint=True)]).astype(np.int64)
    Ws = np.concatenate([[1, 2, 255, 256, 768, W_MAX - 1, W_MAX, 7, W_MAX, 3],
                         rng.integers(1, W_MAX, 3998, endpoint=True)]).astype(np.int64)
    for U, W in zip(Us, Ws):
        ws = np.unique(np.concatenate([[0, 1, W - 1, W], rng.integers(0, W, 64, endpoint=True)]))
        got = np.floor(ws.astype(np.float64) * float(U) / float(W)).astype(np.int64)
        want = np.array([int(w) * int(U) // int(W) for w in ws], dtype=np.int64)
        assert np.array_equal(got, want), (U, W)
        xs = np.unique(np.concatenate([[0, U - 1], rng.integers(0, U - 1, 64, endpoint=True)]))
        got = np.floor(((xs + 1).astype(np.float64) * float(W) - 1.0) / float(U)).astype(np.int64)
        want = np.array([((int(x) + 1) * int(W) - 1) // int(U) for x in xs], dtype=np.int64)
        assert np.array_equal(got, want), (U, W)


def int4_append_lane_reads(lane, total_lanes, lanes_per_row, n_kv, clamp_piece=True):
    """(token, head, piece) whose source rows and key scales lane `lane` of
    kv_append_int4_kernel reads.  Idle lanes past the last row take the last
    lane's row and piece (clamp_piece=False restates the unclamped piece index,
    which idle lanes pushed past the row)."""
    lc = min(lane, total_lanes - 1)
    row = lc // lanes_per_row
    j = (lc if clamp_piece else lane) - row * lanes_per_row
    return row // n_kv, row % n_kv, j


@pytest.mark.parametrize("head_dim", [64, 128])
def test_int4_append_reads_stay_in_bounds(head_dim):
    """Every lane of the grid (256-lane workgroups, the last one partly idle) reads
    inside k_new / v_new ([tokens][n_kv][head_dim]) and k_channel_scales
    ([n_kv][head_dim]), for lane counts that are not multiples of 256."""
    lpr = head_dim // 8
    for tokens in (1, 3, 7, 33):
        for n_kv in (1, 2, 3, 8):
            total = tokens * n_kv * lpr
            grid = (total + 255) // 256 * 256
            src_elems = tokens * n_kv * head_dim
            bad = 0
            for lane in range(grid):
                tok, head, j = int4_append_lane_reads(lane, total, lpr, n_kv)
                assert 0 <= tok < tokens and 0 <= head < n_kv and 0 <= j < lpr
                row_elem = (tok * n_kv + head) * head_dim + j * 8
                assert row_elem + 8 <= src_elems                       # 8 source elements
                assert head * head_dim + j * 8 + 8 <= n_kv * head_dim   # 8 key scales
                t2, h2, j2 = int4_append_lane_reads(lane, total, lpr, n_kv, clamp_piece=False)
                bad += (t2 * n_kv + h2) * head_dim + j2 * 8 + 8 > src_elems
            # the unclamped piece index reads past the rows whenever lanes are idle
            assert (bad > 0) == (grid > total)


def vslice_off(hd, t, byte):
    """Byte of (token row t, byte) in a wave's swizzled V slice of the matrix-core
    decode: 16-byte chunk c of row t at chunk c ^ g(t)."""
    g = row_g(t) if hd == 128 else (t & 7)
    return t * 2 * hd + 16 * ((byte >> 4) ^ g) + (byte & 15)


def mf_dim0(t, j, hd, ebits):
    dpj = hd // 4
    ps = min(dpj * ebits // 8, 16)
    dpp = ps * 8 // ebits
    cpp = dpp // 8
    return (j + 4 * (t // cpp)) * dpp + 8 * (t % cpp)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("ebits", [8, 4])
def test_decode_vslice_swizzle(hd, ebits):
    """The V slice map is a bijection of each row's bytes; the slice writes (16
    bytes a lane) and the transposed reads (8 bytes a lane) meet no bank conflict
    in the model above; and every lane's transposed read finds the bytes the
    writing lane put there."""
    rb = 2 * hd
    for t in range(16):
        assert sorted(vslice_off(hd, t, b) for b in range(rb)) == list(range(t * rb, (t + 1) * rb))
    written = {}
    for tt in range(hd // 32):
        offs = []
        for lane in range(64):
            j, r = lane >> 4, lane & 15
            byte = 2 * mf_dim0(tt, j, hd, ebits)
            offs.append(vslice_off(hd, r, byte))
            for k in range(16):
                written[vslice_off(hd, r, byte + k)] = (r, byte + k)
        assert b128_conflict_free(offs), tt
    for b in range(hd // 16):
        offs = []
        for lane in range(64):
            j, r = lane >> 4, lane & 15
            row, byte = 4 * j + (r >> 2), 32 * b + 8 * (r & 3)
            offs.append(vslice_off(hd, row, byte))
            for k in range(8):
                assert written[vslice_off(hd, row, byte + k)] == (row, byte + k)
        assert tr64_conflict_free(offs), b
