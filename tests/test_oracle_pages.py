"""Pins of the page-pool model (oracle/pages.py): a scenario worked out by
hand from the rules (allocate per logical page, lowest free id first; shared
prompt pages counted; release clears the row; a shared partly filled page is
copied before it is written), structural invariants after every step of
random scripts, and a simulation of page contents showing that every
sequence still reads exactly its own tokens after forks, appends, copies and
releases."""
import numpy as np
import pytest

from oracle import pages


def test_hand_worked_scenario():
    m = pages.PagePoolModel(num_pages=10, page_size=16, max_seqs=4, max_pages_per_seq=4)
    assert m.extend(0, 20) == [] and m.rows[0] == [0, 1]
    m.fork(0, 1, 20)
    assert m.rows[1] == [0, 1] and m.refcount[:2] == [2, 2]
    # seq 1 writes position 20, slot 4 of the shared page 1: private copy into page 2
    assert m.extend(1, 25) == [(1, 2)] and m.rows[1] == [0, 2] and m.refcount[:3] == [2, 1, 1]
    # page 1 is seq 0's alone now: no copy; position 32 needs a new page (3)
    assert m.extend(0, 40) == [] and m.rows[0] == [0, 1, 3]
    m.fork(0, 2, 16)
    assert m.rows[2] == [0] and m.refcount[0] == 3
    # seq 2 ends on a page boundary: its next token opens a fresh page, no copy
    assert m.extend(2, 17) == [] and m.rows[2] == [0, 4]
    m.release(0)
    assert m.rows[0] == [] and m.lens[0] == 0 and m.refcount[:5] == [2, 0, 1, 0, 1]
    assert m.extend(3, 48) == [] and m.rows[3] == [1, 3, 5]
    want = np.array([[-1, -1, -1, -1], [0, 2, -1, -1], [0, 4, -1, -1], [1, 3, 5, -1]], dtype=np.int32)
    assert np.array_equal(m.block_table(), want)
    assert m.free_pages() == [6, 7, 8, 9]


def test_out_of_pages_changes_nothing():
    m = pages.PagePoolModel(num_pages=3, page_size=16, max_seqs=2, max_pages_per_seq=4)
    m.extend(0, 40)
    before = (list(m.refcount), [list(r) for r in m.rows], list(m.lens))
    with pytest.raises(MemoryError):
        m.extend(1, 17)
    assert (list(m.refcount), [list(r) for r in m.rows], list(m.lens)) == before


def random_script(seed, n_ops=120, max_seqs=6, page_size=16, max_pages=8):
    """Seeded random operations (op, args) over a small pool."""
    rng = np.random.default_rng(seed)
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        s = int(rng.integers(max_seqs))
        if r < 0.55:
            ops.append(("extend", s, int(rng.integers(1, 40))))        # grow by 1..39 tokens
        elif r < 0.8:
            ops.append(("fork", s, int(rng.integers(max_seqs)), float(rng.random())))
        else:
            ops.append(("release", s))
    return ops


def run_model_step(m, op, content, expect, label):
    """Apply one op to the model and to a content simulation: page slots hold
    token labels; `expect[s]` is the label list sequence s must read."""
    if op[0] == "extend":
        s, grow = op[1], op[2]
        old = m.lens[s]
        new = min(old + grow, m.max_pages * m.page_size)
        try:
            copies = m.extend(s, new)
        except MemoryError:
            return "out_of_pages"
        for src, dst in copies:
            content[dst] = list(content[src])
        for pos in range(old, new):
            page = m.rows[s][pos // m.page_size]
            content[page][pos % m.page_size] = label
            expect[s].append(label)
            label += 1
        return label
    if op[0] == "fork":
        parent, child, frac = op[1], op[2], op[3]
        if parent == child or m.lens[child] != 0 or m.lens[parent] == 0:
            return label
        n = max(1, int(frac * m.lens[parent]))
        m.fork(parent, child, n)
        expect[child] = list(expect[parent][:n])
        return label
    m.release(op[1])
    expect[op[1]] = []
    return label


def check_invariants(m):
    held = [0] * len(m.refcount)
    for s, row in enumerate(m.rows):
        assert len(row) == -(-m.lens[s] // m.page_size)
        for p in row:
            held[p] += 1
    assert held == m.refcount
    assert m.free_pages() == [p for p, r in enumerate(m.refcount) if r == 0]


@pytest.mark.parametrize("seed", range(6))
def test_random_scripts_keep_invariants_and_contents(seed):
    m = pages.PagePoolModel(num_pages=24, page_size=16, max_seqs=6, max_pages_per_seq=8)
    content = [[None] * 16 for _ in range(24)]
    expect = [[] for _ in range(6)]
    label = 0
    for op in random_script(seed):
        free_before = m.free_pages()
        rows_before = [list(r) for r in m.rows]
        res = run_model_step(m, op, content, expect, label)
        if res != "out_of_pages":
            label = res
        check_invariants(m)
        # pages taken by this step are the lowest ones free before it
        taken = sorted({p for r in m.rows for p in r} - {p for r in rows_before for p in r})
        assert taken == free_before[: len(taken)]
        for s in range(6):
            got = [content[m.rows[s][pos // 16]][pos % 16] for pos in range(m.lens[s])]
            assert got == expect[s], (op, s)


def test_copy_pages_is_a_page_copy():
    rng = np.random.default_rng(3)
    k, v = rng.standard_normal((5, 4, 2, 8)), rng.standard_normal((5, 4, 2, 8))
    ks, vs = rng.random((5, 2)), rng.random((5, 2))
    k2, v2, ks2, vs2 = pages.copy_pages(k, v, [1, 3], [4, 0], ks, vs)
    assert np.array_equal(k2[4], k[1]) and np.array_equal(v2[0], v[3]) and np.array_equal(ks2[4], ks[1])
    assert np.array_equal(vs2[0], vs[3]) and np.array_equal(k2[2], k[2]) and np.array_equal(v2[1], v[1])
