"""Acceptance rule of speculative decoding -- TEST INFRASTRUCTURE ONLY.

Plain Python and numpy, written from "Module 23: Serving", 23.5 and its
Exercises, "Scaling LLM serving", "Speculative decoding", and "Designing an
LLM serving system", "Speculative decoding":

  * A draft model proposes gamma tokens x_0 .. x_{gamma-1}; the target
    model's single verification pass gives its distributions p_0 .. p_gamma
    (p_i for the token after the first i drafts; p_gamma for the token after
    all of them). q_i is the draft's distribution x_i was drawn from.
  * Drafts are checked in order. x_i is accepted with probability
    min(1, p_i(x_i) / q_i(x_i)).
  * At the first rejection the remaining drafts are discarded and one token
    is drawn from the leftover distribution max(0, p_i - q_i), normalised.
  * If every draft is accepted, one more token is drawn from p_gamma. So a
    pass yields n_accepted + 1 tokens.

The random numbers are inputs: u[i] for the test of draft i (accept iff
u[i] < p_i(x_i) / q_i(x_i)), u_final for the one draw at the end. A draw from
weights w with uniform u returns the smallest index x whose running sum
w_0 + .. + w_x exceeds u * (w_0 + .. + w_{V-1}) (inverse of the cumulative
distribution).

Precision. Probabilities are float32, as a model's softmax gives them. The
accept test is a decision on floats, so it is written as the float32
product and comparison u * q(x) < p(x) (the same decision as u < p/q, without
the division's extra rounding), which the library's kernel takes in the
same precision. The leftover weights max(0, p - q) are float32 differences;
their running sums are taken in float64 (to within rounding the exact
cumulative distribution of those weights). Where the leftover has no
positive weight (p = q up to rounding, so a rejection could not happen in
exact arithmetic) the token is drawn from p_i instead.
"""
import numpy as np


def accept_probability(p_x, q_x):
    """min(1, p(x) / q(x)): the chance a drafted token is kept."""
    return min(1.0, p_x / q_x)


def accepts(u, p_x, q_x):
    """The accept test with uniform u, in float32: u * q(x) < p(x)."""
    return bool(np.float32(u) * np.float32(q_x) < np.float32(p_x))


def leftover_weights(p, q):
    """max(0, p - q) elementwise in float32 (not yet normalised)."""
    return np.maximum(np.asarray(p, np.float32) - np.asarray(q, np.float32), np.float32(0))


def draw(weights, u):
    """Smallest x with cumsum(weights)[x] > u * sum(weights), sums in
    float64. weights must have a positive sum."""
    c = np.cumsum(np.asarray(weights, np.float64))
    total = c[-1]
    if not total > 0:
        raise ValueError("draw: weights with no positive mass")
    target = float(u) * total
    for x in range(len(c)):
        if c[x] > target:
            return x
    return len(c) - 1   # u * total == total only for u = 1, outside [0, 1)


def verify_tokens(p, q, draft, u, u_final):
    """One verification of gamma drafts.

    p: [gamma + 1][V] float32 target probabilities; q: [gamma][V] float32
    draft probabilities; draft: [gamma] token ids; u: [gamma] uniforms;
    u_final: one uniform. Returns (n_accepted, next_token)."""
    gamma = len(draft)
    for i in range(gamma):
        x = int(draft[i])
        if accepts(u[i], p[i][x], q[i][x]):
            continue
        w = leftover_weights(p[i], q[i])
        if not np.float64(w.astype(np.float64).sum()) > 0:
            w = np.asarray(p[i], np.float32)
        return i, draw(w, u_final)
    return gamma, draw(np.asarray(p[gamma], np.float32), u_final)


def expected_tokens_per_pass(alpha, gamma):
    """Tokens per verification pass when every draft is accepted
    independently with probability alpha ([M23] Exercises): the closed form
    (1 - alpha^(gamma+1)) / (1 - alpha)."""
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)
