"""CPU replay of the decode split kernel's work partition and load addressing.

The split kernel (csrc/decode.hip, decode_split_kernel) cuts the list of
32-key tiles of all (sequence, head group) segments into equal ranges, one
per workgroup, walks each range segment by segment ("pieces"), and has every
wave issue its K/V loads through clamped 16-key block indices.  This module
restates that integer arithmetic in Python, line for line with the kernel's
own, and checks on the CPU, for ragged lengths with empty sequences at the
edges and in the middle and grids of 1 to 300 workgroups, that:
  * every piece holds at least one tile (no empty piece is formed);
  * every block-table index a load or a scale lookup uses lies in
    [0, pages of the sequence), and every key row it reads in [0, ctx);
  * a 16-key block's key rows lie in the page of its block index (the page id
    is wave-uniform);
  * every tile is computed exactly once, partial slots are unique and inside
    the workspace, and the merge kernel's workgroup range for each segment is
    exactly the set of workgroups that wrote it.
It also shows that the walk as it was before empty sequences were skipped
reads a block-table index of -1 (one entry before the row).
"""
import numpy as np
import pytest

TILE = 32
WAVES = 8


def seg_tiles(ctx, window_left):
    ctx = max(ctx, 0)
    lo = max(0, ctx - 1 - window_left) if window_left >= 0 else 0
    return (ctx + TILE - 1) // TILE - lo // TILE


def heads_per_wg(hkv):
    h = 8
    while hkv % h:
        h >>= 1
    return h


def cdiv_trunc(a, b):
    """C integer division (truncates toward zero)."""
    q = abs(a) // abs(b)
    return q if (a >= 0) == (b >= 0) else -q


def replay(ctx_lens, window_left, hkv, nwg, page_size, nb_inflight, i8, skip_empty=True):
    """Returns (pieces, accesses): pieces (j, b, hg, t_first, len); accesses
    (b, block_index, (first key, last key)) for the 16 rows of every 16-key
    block a wave loads, and (b, block_index, None) for every scale lookup."""
    lp = page_size.bit_length() - 1
    hpw = heads_per_wg(hkv)
    ngr = hkv // hpw
    wph = WAVES // hpw
    W = window_left
    tiles = [seg_tiles(c, W) for c in ctx_lens]
    prefix = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    total = ngr * int(prefix[-1])
    pieces, accesses = [], []
    if total == 0:
        return pieces, accesses
    active = max(1, min(nwg, total))
    for j in range(active):
        start = j * total // active
        end = (j + 1) * total // active
        b = next(bb for bb in range(len(ctx_lens)) if start < ngr * (prefix[bb] + tiles[bb]))
        nb = tiles[b]
        r0 = start - ngr * int(prefix[b])
        hg = r0 // nb
        tloc = r0 - hg * nb
        remaining = end - start
        while remaining > 0:
            ln = min(nb - tloc, remaining)
            ctx = ctx_lens[b]
            lo = max(0, ctx - 1 - W) if W >= 0 else 0
            t_first = lo // TILE + tloc
            k_begin = max(lo, t_first * TILE)
            k_end = min(ctx, (t_first + ln) * TILE)
            pieces.append((j, b, hg, t_first, ln))
            lo16 = k_begin & ~15
            hi16 = (k_end - 1) & ~15
            for w in range(WAVES):
                sub = w // hpw
                n_w = cdiv_trunc(ln - sub + wph - 1, wph)
                n_iter = cdiv_trunc(n_w + nb_inflight - 1, nb_inflight) * nb_inflight if n_w > 0 else 0
                # loads: the prefetch of indices 0..NB-1, then index i + NB in step i
                for i in list(range(nb_inflight)) + [i + nb_inflight for i in range(n_iter)]:
                    t = t_first + sub + wph * min(i, n_w - 1)
                    for kb in range(2):
                        bs = min(max(t * TILE + 16 * kb, lo16), hi16)
                        # lanes r16 = 0..15 read clamped keys; the clamp is
                        # monotonic, so the first and last lane bound them
                        k_first = min(max(t * TILE + 16 * kb, k_begin), k_end - 1)
                        k_last = min(max(t * TILE + 16 * kb + 15, k_begin), k_end - 1)
                        accesses.append((b, bs >> lp, (k_first, k_last)))
                # int8 scale lookups in step i (unclamped tile index)
                if i8:
                    for i in range(n_iter):
                        key0 = (t_first + sub + wph * i) * TILE
                        for kb in range(2):
                            bs = min(max(key0 + 16 * kb, lo16), hi16)
                            accesses.append((b, bs >> lp, None))
            remaining -= ln
            tloc = 0
            hg += 1
            if hg == ngr and remaining > 0:
                hg = 0
                b += 1
                nb = tiles[b]
                if skip_empty:
                    while nb == 0:
                        b += 1
                        nb = tiles[b]
    return pieces, accesses


def check(ctx_lens, window_left, hkv, nwg, page_size, nb_inflight, i8):
    pieces, accesses = replay(ctx_lens, window_left, hkv, nwg, page_size, nb_inflight, i8)
    lp = page_size.bit_length() - 1
    hpw = heads_per_wg(hkv)
    ngr = hkv // hpw
    B = len(ctx_lens)
    for b, blk, keys in accesses:
        pages_b = -(-ctx_lens[b] // page_size)
        assert 0 <= blk < pages_b, (ctx_lens, nwg, b, blk)
        if keys is not None:
            for key in keys:
                assert 0 <= key < ctx_lens[b], (ctx_lens, nwg, b, key)
                assert key >> lp == blk, (ctx_lens, nwg, b, key, blk)
    # every tile of every segment once; slots unique and in the workspace
    seen = {}
    slots = set()
    for j, b, hg, t_first, ln in pieces:
        assert ln >= 1
        for t in range(t_first, t_first + ln):
            assert (b, hg, t) not in seen
            seen[(b, hg, t)] = j
        slot = b * ngr + hg + j
        assert slot not in slots and slot < B * ngr + nwg
        slots.add(slot)
    tiles = [seg_tiles(c, window_left) for c in ctx_lens]
    want = {(b, hg, window_start + t)
            for b in range(B) for hg in range(ngr)
            for window_start in [(max(0, ctx_lens[b] - 1 - window_left) if window_left >= 0 else 0) // TILE]
            for t in range(tiles[b])}
    assert set(seen) == want
    # the merge kernel's range of workgroups per segment
    prefix = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)
    total = ngr * int(prefix[-1])
    if total:
        active = max(1, min(nwg, total))
        for b in range(B):
            if tiles[b] == 0:
                continue
            for hg in range(ngr):
                f0 = ngr * int(prefix[b]) + hg * tiles[b]
                f1 = f0 + tiles[b] - 1
                j_lo = ((f0 + 1) * active - 1) // total
                j_hi = ((f1 + 1) * active - 1) // total
                wrote = {j for j, bb, g, _, _ in pieces if (bb, g) == (b, hg)}
                assert wrote == set(range(j_lo, j_hi + 1)), (b, hg, wrote, j_lo, j_hi)


def test_old_walk_reads_before_the_row_on_an_empty_sequence():
    """The reproduction on the CPU: lengths [300, 0, 300], 2 KV heads, 16-key
    pages, grid 7.  Without the skip, a workgroup steps onto the empty
    sequence, forms an empty piece and loads through block index -1."""
    _, acc = replay([300, 0, 300], -1, 2, 7, 16, 1, False, skip_empty=False)
    assert min(blk for _, blk, _ in acc) == -1
    _, acc = replay([300, 0, 300], -1, 2, 7, 16, 1, False, skip_empty=True)
    assert min(blk for _, blk, _ in acc) >= 0


@pytest.mark.parametrize("i8", [False, True])
def test_partition_stays_in_range_with_empty_sequences(i8):
    r = np.random.default_rng(17 + i8)
    nb_inflight = 2 if i8 else 1
    cases = [
        [300, 0, 300],
        [0, 0, 5000, 0],
        [0, 1, 0, 33, 0],
        [300, 0, 0, 4000, 0, 2500],
    ]
    for _ in range(6):
        n = int(r.integers(3, 10))
        c = r.integers(1, 3000, size=n)
        c[r.random(n) < 0.4] = 0
        c[0] = 0 if r.random() < 0.5 else c[0]
        c[-1] = 0
        cases.append([int(x) for x in c])
    grids = [1, 2, 3, 7, 16, 64, 255, 256, 300]
    for ctx in cases:
        for hkv in (8, 2, 1, 6):
            for page_size in (16, 256):
                for window in (-1, 100):
                    for nwg in grids:
                        check(ctx, window, hkv, nwg, page_size, nb_inflight, i8)


def test_layered_int8_part_with_empty_sequences_default_grid():
    """The int8 part of a layered decode: sequences of at most F tokens have
    no int8 keys, among 64k-128k-token ones, with more tiles than the 256
    workgroups of the default grid (so each workgroup walks several)."""
    lens = [70000 - 128, 0, 90000 - 128, 0, 0, 66000 - 128, 100000 - 128, 0]
    for hkv in (8, 2):
        check(lens, -1, hkv, 256, 256, 2, True)
