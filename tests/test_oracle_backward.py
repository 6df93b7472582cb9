"""Pins of oracle.attention_backward_paged (gradients of paged attention):
central finite differences of a scalar loss through the forward oracle,
torch autograd in float64 over a dense formulation written independently,
GQA as the sum over a repeated-head MHA, and zero gradient for keys no
query sees."""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward

CASES = [
    # (seq q_lens, ctx_lens, hq, hkv, d, page_size, causal, window)
    ((3, 5), (3, 7), 4, 2, 8, 4, True, -1),     # second sequence: chunked (q_len < ctx)
    ((6,), (6,), 2, 1, 8, 4, True, 2),          # window
    ((4,), (4,), 2, 2, 8, 4, False, -1),        # no mask
]


def _problem(case, seed):
    q_lens, ctx, hq, hkv, d, P, causal, window = case
    rng = np.random.default_rng(seed)
    pages = [-(-c // P) for c in ctx]
    n_pages = sum(pages) + 1
    perm = rng.permutation(n_pages)
    bt = np.zeros((len(ctx), max(pages)), dtype=np.int64)
    at = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[at:at + n]
        at += n
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q = rng.standard_normal((cu[-1], hq, d))
    k = rng.standard_normal((n_pages, P, hkv, d))
    v = rng.standard_normal((n_pages, P, hkv, d))
    w = rng.standard_normal((cu[-1], hq, d))        # loss = sum(O * w), so dO = w
    return dict(q=q, cu=cu, k=k, v=v, bt=bt, ctx=np.array(ctx), P=P, causal=causal, window=window, w=w)


def _loss(pr, q=None, k=None, v=None):
    o, _ = oracle.attention_paged(pr["q"] if q is None else q, pr["cu"], pr["k"] if k is None else k,
                                  pr["v"] if v is None else v, pr["bt"], pr["ctx"], pr["P"],
                                  causal=pr["causal"], window_left=pr["window"])
    return float((o * pr["w"]).sum())


def _grads(pr):
    return backward.attention_backward_paged(pr["q"], pr["cu"], pr["k"], pr["v"], pr["bt"], pr["ctx"], pr["P"],
                                             pr["w"], causal=pr["causal"], window_left=pr["window"])


def _used_slots(pr):
    out = []
    for b, c in enumerate(pr["ctx"]):
        for t in range(int(c)):
            out.append((int(pr["bt"][b, t // pr["P"]]), t % pr["P"]))
    return out


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    pr = _problem(case, 5)
    dq, dk, dv = _grads(pr)
    eps = 1e-6
    rng = np.random.default_rng(6)
    for name, arr, grad in (("q", pr["q"], dq), ("k", pr["k"], dk), ("v", pr["v"], dv)):
        if name == "q":
            idx = [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(12)]
        else:
            slots = _used_slots(pr)
            idx = [slots[i] + (int(rng.integers(arr.shape[2])), int(rng.integers(arr.shape[3])))
                   for i in rng.integers(0, len(slots), 12)]
        for ix in idx:
            plus, minus = arr.copy(), arr.copy()
            plus[ix] += eps
            minus[ix] -= eps
            num = (_loss(pr, **{name: plus}) - _loss(pr, **{name: minus})) / (2 * eps)
            assert abs(num - grad[ix]) <= 1e-6 * max(1.0, abs(num)), (name, ix, num, grad[ix])


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_torch_autograd(case):
    pr = _problem(case, 7)
    dq, dk, dv = _grads(pr)
    hq, hkv = pr["q"].shape[1], pr["k"].shape[2]
    for b in range(len(pr["ctx"])):
        q0, q1, ctx = int(pr["cu"][b]), int(pr["cu"][b + 1]), int(pr["ctx"][b])
        rows = [(int(pr["bt"][b, t // pr["P"]]), t % pr["P"]) for t in range(ctx)]
        kd = torch.tensor(np.stack([pr["k"][p, s] for p, s in rows]), requires_grad=True)
        vd = torch.tensor(np.stack([pr["v"][p, s] for p, s in rows]), requires_grad=True)
        qd = torch.tensor(pr["q"][q0:q1], requires_grad=True)
        i = torch.arange(q1 - q0)[:, None] + (ctx - (q1 - q0))
        j = torch.arange(ctx)[None, :]
        allowed = torch.ones(q1 - q0, ctx, dtype=torch.bool)
        if pr["causal"]:
            allowed &= j <= i
        if pr["window"] >= 0:
            allowed &= (i - j) <= pr["window"]
        loss = 0
        for h in range(hq):
            g = h * hkv // hq
            sc = (qd[:, h] @ kd[:, g].T) / np.sqrt(qd.shape[-1])
            pmat = torch.softmax(sc.masked_fill(~allowed, float("-inf")), dim=-1)
            loss = loss + ((pmat @ vd[:, g]) * torch.tensor(pr["w"][q0:q1, h])).sum()
        loss.backward()
        assert np.allclose(dq[q0:q1], qd.grad.numpy(), atol=1e-10, rtol=0)
        assert np.allclose(np.stack([dk[p, s] for p, s in rows]), kd.grad.numpy(), atol=1e-10, rtol=0)
        assert np.allclose(np.stack([dv[p, s] for p, s in rows]), vd.grad.numpy(), atol=1e-10, rtol=0)


def test_gqa_gradient_is_the_sum_over_repeated_heads():
    pr = _problem(((5,), (5,), 4, 1, 8, 4, True, -1), 8)
    dq, dk, dv = _grads(pr)
    rep = dict(pr, k=np.repeat(pr["k"], 4, axis=2), v=np.repeat(pr["v"], 4, axis=2))
    dq4, dk4, dv4 = _grads(rep)
    assert np.allclose(dq, dq4, atol=1e-12, rtol=0)
    assert np.allclose(dk[:, :, 0], dk4.sum(axis=2), atol=1e-12, rtol=0)
    assert np.allclose(dv[:, :, 0], dv4.sum(axis=2), atol=1e-12, rtol=0)


def test_keys_no_query_sees_get_zero_gradient():
    # chunked rows 4..5 of a 6-key context with a window of 1: keys 0..2 are out of reach
    pr = _problem(((2,), (6,), 2, 1, 8, 4, True, 1), 9)
    _, dk, dv = _grads(pr)
    for t in range(6):
        p, s = int(pr["bt"][0, t // 4]), t % 4
        seen = t >= 3
        assert (np.abs(dk[p, s]).max() > 0) == seen and (np.abs(dv[p, s]).max() > 0) == seen
