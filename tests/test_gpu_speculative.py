"""The acceptance rule of speculative decoding on the GPU (pkv_spec_accept)
against the oracle (oracle/speculative.py).

Probabilities are seeded random distributions (float32), drafts are drawn
from the draft distribution, uniforms are seeded in [0, 1). The keep tests
are the same float32 decision on both sides, so the number of kept drafts
must match exactly. The drawn token must match exactly too, unless u * total
lies within rounding of a boundary of the running sums (float64 sums in a
different order); there the GPU's token must still be a valid draw: positive
weight, running sum above the target, the one before not above it.
"""
import numpy as np
import pytest

import oracle.speculative as spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _dists(g, shape):
    x = g.exponential(size=shape) ** 2
    return (x / x.sum(axis=-1, keepdims=True)).astype(np.float32)


def _case(seed, B, gamma, V, same=False):
    g = np.random.default_rng(seed)
    p = _dists(g, (B, gamma + 1, V))
    q = p[:, :gamma].copy() if same else _dists(g, (B, gamma, V))
    draft = np.zeros((B, gamma), np.int32)
    for b in range(B):
        for i in range(gamma):
            w = q[b, i].astype(np.float64)
            draft[b, i] = g.choice(V, p=w / w.sum())
    u = g.random((B, gamma + 1)).astype(np.float32)
    return p, q, draft, u


def _gpu(pkv, p, q, draft, u):
    import torch
    B = p.shape[0]
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_spec_accept(torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda(),
                        torch.from_numpy(draft).cuda(), torch.from_numpy(u).cuda(), n, tok,
                        err_flag=err)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy(), int(err.item())


def _valid_draw(weights, u, y):
    """y is a correct inverse-CDF draw of weights with uniform u, allowing
    for rounding of the running sums."""
    w = np.asarray(weights, np.float64)
    c = np.cumsum(w)
    target = float(u) * c[-1]
    eps = 1e-12 * c[-1]
    return w[y] > 0 and c[y] > target - eps and (y == 0 or c[y - 1] <= target + eps)


def _compare(p, q, draft, u, n, tok):
    exact = 0
    for b in range(p.shape[0]):
        n_ref, tok_ref = spec.verify_tokens(p[b], q[b], draft[b], u[b, :-1], u[b, -1])
        assert n[b] == n_ref, (b, n[b], n_ref)
        if tok[b] == tok_ref:
            exact += 1
            continue
        gamma = draft.shape[1]
        w = spec.leftover_weights(p[b, n_ref], q[b, n_ref]) if n_ref < gamma else p[b, gamma]
        if not w.astype(np.float64).sum() > 0:
            w = p[b, n_ref]
        assert _valid_draw(w, u[b, -1], tok[b]), (b, tok[b], tok_ref)
    return exact


CASES = [  # seed, B, gamma, V
    (1, 64, 4, 1000),
    (2, 64, 1, 257),
    (3, 32, 7, 5),
    (4, 16, 4, 32000),
    (5, 4, 4, 128256),
    (6, 64, 0, 300),
    (7, 8, 64, 50),
    (8, 16, 3, 8193),     # 5 tiles: the second 4-tile workgroup holds one tile
    (9, 64, 4, 128256),   # the benchmark's batch and vocabulary (16 workgroups per sequence)
    (10, 3, 2, 140000),   # 69 tiles: the draw's prefix sums over two rounds of 64
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[1]}-g{c[2]}-V{c[3]}" for c in CASES])
def test_accept_matches_oracle(pkv, case):
    seed, B, gamma, V = case
    p, q, draft, u = _case(seed, B, gamma, V)
    n, tok, err = _gpu(pkv, p, q, draft, u)
    assert err == 0
    exact = _compare(p, q, draft, u, n, tok)
    print(f"B {B} gamma {gamma} V {V}: kept {n.tolist()[:8]}..., tokens equal {exact}/{B}")
    assert exact >= B - 1


def test_draft_equals_target_keeps_everything(pkv):
    """p = q: every draft is kept and the extra token comes from p_gamma."""
    p, q, draft, u = _case(11, 32, 4, 700, same=True)
    n, tok, err = _gpu(pkv, p, q, draft, u)
    assert err == 0 and (n == 4).all()
    _compare(p, q, draft, u, n, tok)


def test_rejected_draft_with_empty_leftover(pkv):
    """q >= p everywhere at draft 1 (q = p, raised by half at the drafted
    token) and a uniform above 2/3: the draft is rejected, the leftover
    max(0, p - q) has no weight, and the token is drawn from p_1 itself, on
    both sides."""
    p, q, draft, u = _case(12, 8, 3, 64, same=True)
    for b in range(8):
        q[b, 1, draft[b, 1]] *= np.float32(1.5)
    u[:, 0] = 0.5
    u[:, 1] = 0.9
    n, tok, err = _gpu(pkv, p, q, draft, u)
    assert err == 0 and (n == 1).all()
    _compare(p, q, draft, u, n, tok)


def test_bad_draft_flagged(pkv):
    import paged_kv_cache_468_amd as lib
    p, q, draft, u = _case(13, 4, 2, 100)
    draft[2, 1] = 100
    n, tok, err = _gpu(pkv, p, q, draft, u)
    assert err & lib.PKV_DEVERR_TOKEN
    assert n[2] == -1 and tok[2] == -1
    keep = [0, 1, 3]
    _compare(p[keep], q[keep], draft[keep], u[keep], n[keep], tok[keep])


def test_workspace_reused_across_calls(pkv):
    """One workspace for two calls in a row (a larger vocabulary, then a
    smaller one): each call writes every tile sum it reads."""
    import torch
    p1, q1, d1, u1 = _case(21, 8, 3, 9000)
    p2, q2, d2, u2 = _case(22, 5, 2, 700)
    ws = torch.empty(pkv.pkv_spec_accept_workspace_bytes(8, 9000), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for p, q, d, u in ((p1, q1, d1, u1), (p2, q2, d2, u2)):
        B = p.shape[0]
        n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        tok = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        pkv.pkv_spec_accept(torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda(),
                            torch.from_numpy(d).cuda(), torch.from_numpy(u).cuda(), n, tok,
                            workspace=ws)
        outs.append((n, tok))
    torch.cuda.synchronize()
    for (p, q, d, u), (n, tok) in zip(((p1, q1, d1, u1), (p2, q2, d2, u2)), outs):
        _compare(p, q, d, u, n.cpu().numpy(), tok.cpu().numpy())


def test_workspace_too_small_refused(pkv):
    import torch
    p, q, draft, u = _case(23, 4, 2, 5000)
    need = pkv.pkv_spec_accept_workspace_bytes(4, 5000)
    assert need == 16 * 4 * 3
    n = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as info:
        pkv.pkv_spec_accept(torch.from_numpy(p).cuda(), torch.from_numpy(q).cuda(),
                            torch.from_numpy(draft).cuda(), torch.from_numpy(u).cuda(), n, n.clone(),
                            workspace=torch.empty(need - 8, dtype=torch.uint8, device="cuda"))
    assert info.value.status == pkv.PKV_EWORKSPACE
    torch.cuda.synchronize()
    assert (n.cpu().numpy() == -7).all()
