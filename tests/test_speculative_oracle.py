"""Pins of the acceptance-rule oracle (oracle/speculative.py) to the pages
and the mathematics, and a check that each plausible mistake in it fails
at least one pin. CPU only.

Pins:
  * the Exercises' worked values (tests/golden/speculative.json): a token with
    p = 0.3, q = 0.5 is kept with probability 0.6; with independent
    acceptance 0.8 and four drafts a pass yields 3.3616 tokens on average,
    obtained here by running the rule over every accept/reject pattern
    weighted by its probability;
  * exactness ("Module 23: Serving", 23.5: the output follows the target's
    distribution whatever the draft does): the first token of a pass,
    integrated over the draft's choice and both uniforms by quadrature, has
    the target's distribution p_0;
  * all drafts kept: the extra token has the distribution p_gamma;
  * drafts after the first rejection never matter.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

import oracle.speculative as spec_default

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "speculative.json")
SRC = spec_default.__file__


def _quadrature(n):
    return (np.arange(n) + 0.5) / n


def check_exercise_accept(spec):
    g = json.load(open(GOLDEN))["accept"]
    assert abs(spec.accept_probability(g["p"], g["q"]) - g["answer"]) <= g["tol"], g["cite"]
    # the decision with uniforms on either side of 0.6
    assert spec.accepts(0.5999, g["p"], g["q"]) and not spec.accepts(0.6001, g["p"], g["q"])
    # a token the target wants more than the draft is always kept
    assert spec.accepts(0.99999, 0.5, 0.3)


def _rule_with_alpha(spec, alpha, gamma, pattern):
    """One pass where every drafted token has p/q = alpha; pattern[i] says
    whether draft i's uniform falls below alpha."""
    V = 4
    p = np.full((gamma + 1, V), 0.25, np.float32)
    q = np.full((gamma, V), 0.25, np.float32)
    p[:gamma, 1] = np.float32(0.5 * alpha)
    p[:gamma, 0] = np.float32(0.5 - 0.5 * alpha + 0.25)
    q[:, 1] = np.float32(0.5)
    q[:, 0] = np.float32(0.0)
    draft = np.ones(gamma, np.int32)
    u = np.array([alpha / 2 if keep else (1 + alpha) / 2 for keep in pattern], np.float32)
    return spec.verify_tokens(p, q, draft, u, 0.5)


def check_exercise_tokens_per_pass(spec):
    g = json.load(open(GOLDEN))["tokens_per_pass"]
    alpha, gamma = g["alpha"], g["gamma"]
    mean = 0.0
    for bits in range(2 ** gamma):
        pattern = [(bits >> i) & 1 == 1 for i in range(gamma)]
        prob = np.prod([alpha if k else 1 - alpha for k in pattern])
        n_acc, _ = _rule_with_alpha(spec, alpha, gamma, pattern)
        mean += prob * (n_acc + 1)
    assert abs(mean - g["answer"]) <= g["tol"], (mean, g["cite"])
    assert abs(spec.expected_tokens_per_pass(alpha, gamma) - g["answer"]) <= g["tol"]


def _random_dist(g, V):
    x = g.random(V) ** 3 + 1e-3
    return (x / x.sum()).astype(np.float32)


def check_output_is_target_distribution(spec):
    """P(first token = y), over draft x ~ q_0, u ~ U[0,1), u_final ~ U[0,1),
    equals p_0(y). Quadrature over the uniforms (n points each): for each
    draft, the fraction of u that keeps it, and the token the rule draws
    for each u_final after a rejection."""
    g = np.random.default_rng(5)
    V, n = 6, 1000
    for _ in range(3):
        p = np.stack([_random_dist(g, V), _random_dist(g, V)])
        q = _random_dist(g, V)[None]
        dist = np.zeros(V)
        for x in range(V):
            kept = [spec.verify_tokens(p, q, np.array([x]), np.array([u], np.float32), 0.5)[0]
                    for u in _quadrature(n)]
            kept_frac = float(np.mean(kept))
            dist[x] += q[0, x] * kept_frac
            if kept_frac < 1:
                u_rej = _quadrature(n)[kept.index(0)]
                for uf in _quadrature(n):
                    n_acc, tok = spec.verify_tokens(p, q, np.array([x]),
                                                    np.array([u_rej], np.float32), uf)
                    assert n_acc == 0
                    dist[tok] += q[0, x] * (1 - kept_frac) / n
        assert np.allclose(dist, p[0], atol=3e-3), (dist, p[0])


def check_bonus_token(spec):
    """Every draft kept: the extra token is drawn from p_gamma."""
    g = np.random.default_rng(6)
    V, gamma, n = 7, 3, 2000
    p = np.stack([_random_dist(g, V) for _ in range(gamma + 1)])
    q = p[:gamma].copy()                   # p = q: every draft is kept
    draft = np.array([1, 4, 2])
    dist = np.zeros(V)
    for uf in _quadrature(n):
        n_acc, tok = spec.verify_tokens(p, q, draft, np.full(gamma, 0.5, np.float32), uf)
        assert n_acc == gamma
        dist[tok] += 1 / n
    assert np.allclose(dist, p[gamma], atol=2e-3)


def check_stops_at_first_rejection(spec):
    """Drafts after the first rejection are discarded: changing them (or
    their uniforms) changes nothing, and the count is the rejection's index."""
    g = np.random.default_rng(7)
    V, gamma = 8, 4
    p = np.stack([_random_dist(g, V) for _ in range(gamma + 1)])
    q = np.stack([_random_dist(g, V) for _ in range(gamma)])
    draft = np.array([int(np.argmax(q[i] - p[i])) for i in range(gamma)])   # p < q there
    u = np.array([0.0, 0.9999, 0.0, 0.0], np.float32)      # keep 0, reject 1
    base = spec.verify_tokens(p, q, draft, u, 0.3)
    assert base[0] == 1
    draft2 = draft.copy()
    draft2[2:] = (draft2[2:] + 3) % V
    u2 = u.copy()
    u2[2:] = 0.99
    assert spec.verify_tokens(p, q, draft2, u2, 0.3) == base
    # the replacement comes from the leftover: never a token with p <= q
    for uf in _quadrature(50):
        _, tok = spec.verify_tokens(p, q, draft, u, uf)
        assert p[1, tok] > q[1, tok]


CHECKS = [check_exercise_accept, check_exercise_tokens_per_pass,
          check_output_is_target_distribution, check_bonus_token, check_stops_at_first_rejection]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check(spec_default)


MUTANTS = {
    "accept_flipped": ("np.float32(u) * np.float32(q_x) < np.float32(p_x)",
                       "np.float32(u) * np.float32(q_x) > np.float32(p_x)"),
    "accept_ratio_inverted": ("return min(1.0, p_x / q_x)", "return min(1.0, q_x / p_x)"),
    "leftover_not_clipped": ("return np.maximum(np.asarray(p, np.float32) - np.asarray(q, np.float32), np.float32(0))",
                             "return np.abs(np.asarray(p, np.float32) - np.asarray(q, np.float32))"),
    "leftover_reversed": ("return np.maximum(np.asarray(p, np.float32) - np.asarray(q, np.float32), np.float32(0))",
                          "return np.maximum(np.asarray(q, np.float32) - np.asarray(p, np.float32), np.float32(0))"),
    "draw_unscaled": ("target = float(u) * total", "target = float(u)"),
    "bonus_from_last_draft_position": ("return gamma, draw(np.asarray(p[gamma], np.float32), u_final)",
                                       "return gamma, draw(np.asarray(p[gamma - 1], np.float32), u_final)"),
    "no_stop_at_rejection": ("        return i, draw(w, u_final)\n", "        pass\n"),
    "rejection_counts_as_accepted": ("        return i, draw(w, u_final)", "        return i + 1, draw(w, u_final)"),
    "replacement_from_target": ("        w = leftover_weights(p[i], q[i])\n",
                                "        w = np.asarray(p[i], np.float32)\n"),
    "closed_form_gamma": ("alpha ** (gamma + 1)", "alpha ** gamma"),
}


def _mutant_module(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"spec_{name}.py"
    path.write_text(text.replace(old, new))
    sp = importlib.util.spec_from_file_location(f"spec_{name}", path)
    mod = importlib.util.module_from_spec(sp)
    sp.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    mod = _mutant_module(name, tmp_path)
    failed = []
    for check in CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
