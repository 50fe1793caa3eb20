"""Speculative-sampling verification of one drafted block (oracle side).

Definitions followed:

* [D3D, 前置知识: 投机解码] and [DScout, 前置知识: 推测解码]: the target verifies all drafts in
  one forward; the prefix before the first rejection is kept; at the first rejection one token is
  resampled from the residual distribution, and on a full accept a bonus token is appended; this
  keeps the output distribution equal to the target's.
* [DScout, 前置知识: 接受加权损失 AWL 与推测采样接受规则]: draft token y_j is accepted with
  probability alpha_j = min(1, P_j(y_j) / Q_j(y_j)), P_j the target and Q_j the draft distribution.
* [DScout, 前置知识: 平均接受长度 MAT] and [D3D, 前置知识: 接受长度 τ]:
  tau = 1 + sum_{k=1}^{B-1} S(k), S(k) = prod_{j<=k} a_j, counting the target's own token.

Readings where the pages leave a step open:

* Rows are 0-based: target row j (j = 0..B-1) and draft row j (j = 0..B-2); row j judges draft
  token y_j (rejection position k = j + 1); target row B-1 is the bonus row.
* P_j = softmax(z^P_j / T), Q_j = softmax(z^Q_j / T) with T the sampling temperature (a float32
  value, as the library receives it). The acceptance test is strict: accept while u_j < alpha_j,
  so alpha = 1 always accepts and alpha = 0 always rejects. If Q_j(y_j) = 0, alpha_j = 1.
* The residual is r = max(0, P_j* - Q_j*) normalised by Z = sum r; the bonus law is P_{B-1}.
  The token is the smallest v whose inclusive cumulative mass C(v) = sum_{i<=v} r_i exceeds u'Z
  (ascending token id). If rounding leaves no such v, the last v with r_v > 0 is taken. If Z = 0
  after a rejection (impossible in exact arithmetic) the draw falls back to P_j* and flag bit 2 is
  set.
* S(k) = prod_{j<k} alpha_j over 0-based rows, so S(k) is the paper's a_1...a_k; tau uses the
  alpha of every row whatever the sampled outcome.
* T = 0 is greedy: alpha_j = 1 exactly when y_j is the first argmax of z^P_j, else 0; the
  replacement (or bonus) is the first argmax of the target row. Draft logits are not read. A
  target row whose logits are all -inf has no argmax: its draft is rejected and the emitted token
  is -1 (no token), the value the drafting selection gives such a row.
* Uniforms: u_j = Philox(seed; j, request, round, purpose 0); u' = Philox(seed; 0, request, round,
  purpose 1). Flags: bit 0 = some decision j <= j* had |u_j - alpha_j| < 1e-6; bit 1 =
  |u'Z - C(v*)| < 1e-6 Z or |u'Z - C(v*-1)| < 1e-6 Z; bit 2 = Z fallback.

TEST INFRASTRUCTURE: see the package docstring.
"""

from dataclasses import dataclass

import numpy as np

from . import philox

FLAG_NEAR_ACCEPT = 1
FLAG_NEAR_SAMPLE = 2
FLAG_Z_FALLBACK = 4
NEAR = 1e-6


def as_temperature(temperature):
    """The temperature as the library sees it: a float32 value, widened to float64."""
    return float(np.float32(temperature))


def row_softmax(z, temperature):
    """softmax(z / T) along the last axis, in float64."""
    x = np.asarray(z, dtype=np.float64) / as_temperature(temperature)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def acceptance_ratios(z_target, z_draft, tokens, temperature):
    """alpha_j for the B-1 drafts of one block (float64 [B-1])."""
    z_target = np.asarray(z_target)
    tokens = np.asarray(tokens, dtype=np.int64)
    n_draft = tokens.size
    rows = np.arange(n_draft)
    if as_temperature(temperature) == 0.0:
        return np.array([float(greedy_argmax(z_target[j]) == tokens[j]) for j in range(n_draft)])
    p = row_softmax(z_target[:n_draft], temperature)[rows, tokens]
    q = row_softmax(z_draft, temperature)[rows, tokens]
    alpha = np.ones(n_draft, dtype=np.float64)
    nz = q > 0
    alpha[nz] = np.minimum(1.0, p[nz] / q[nz])
    return alpha


def greedy_argmax(row):
    """First index of the largest logit, or -1 when every logit is -inf (no most likely token)."""
    row = np.asarray(row)
    if not np.any(row > -np.inf):
        return -1
    return int(np.argmax(row))


def first_rejection(alpha, u):
    """Index of the first draft with u_j >= alpha_j, or len(alpha) when every draft is accepted."""
    for j, (a, uj) in enumerate(zip(alpha, u)):
        if not (uj < a):
            return j
    return len(alpha)


def survival(alpha):
    """S(k) = prod_{j<k} alpha_j for k = 1..B-1, and tau = 1 + sum_k S(k)."""
    s = np.cumprod(np.asarray(alpha, dtype=np.float64))
    return s, 1.0 + float(s.sum())


def residual_mass(z_target_row, z_draft_row, temperature):
    """Unnormalised residual r = max(0, P - Q) of one rejected row (float64 [V])."""
    return np.maximum(0.0, row_softmax(z_target_row, temperature) - row_softmax(z_draft_row, temperature))


def inverse_cdf(r, u):
    """Smallest v with inclusive C(v) = sum_{i<=v} r_i > u * Z; returns (v, Z, C(v), C(v-1))."""
    r = np.asarray(r, dtype=np.float64)
    c = np.cumsum(r)
    z = float(c[-1])
    target = u * z
    hits = np.nonzero(c > target)[0]
    if hits.size:
        v = int(hits[0])
    else:
        v = int(np.nonzero(r > 0)[0][-1])
    c_prev = float(c[v - 1]) if v > 0 else 0.0
    return v, z, float(c[v]), c_prev


@dataclass
class Outcome:
    n_accepted: int
    next_token: int
    alpha: np.ndarray
    survival: np.ndarray
    tau: float
    flags: int
    u_accept: np.ndarray
    u_sample: float
    sample_mass: np.ndarray  # the unnormalised law the next token was drawn from


def verify_request(z_target, z_draft, tokens, temperature, seed=0, round_=0, request=0,
                   u_accept=None, u_sample=None):
    """Verify one drafted block.

    z_target: [B, V] target logits; z_draft: [B-1, V] draft logits; tokens: [B-1] draft tokens.
    u_accept ([B-1]) and u_sample override the Philox uniforms when given.
    """
    z_target = np.asarray(z_target)
    tokens = np.asarray(tokens, dtype=np.int64)
    n_draft = tokens.size
    if z_target.shape[0] != n_draft + 1:
        raise ValueError("need B target rows for B-1 drafts")
    T = as_temperature(temperature)
    if u_accept is None:
        u_accept = philox.uniforms(seed, np.arange(n_draft), request, round_, philox.PURPOSE_ACCEPT)
    u_accept = np.asarray(u_accept, dtype=np.float64)
    if u_sample is None:
        u_sample = float(philox.uniforms(seed, 0, request, round_, philox.PURPOSE_SAMPLE))

    alpha = acceptance_ratios(z_target, z_draft, tokens, T)
    s, tau = survival(alpha)
    j_star = first_rejection(alpha, u_accept)
    flags = 0

    if T == 0.0:
        row = z_target[j_star]
        token = greedy_argmax(row)
        mass = np.zeros(row.shape[-1])
        if token >= 0:
            mass[token] = 1.0
        return Outcome(j_star, token, alpha, s, tau, 0, u_accept, u_sample, mass)

    decided = min(j_star, n_draft - 1)
    if n_draft and np.any(np.abs(u_accept[:decided + 1] - alpha[:decided + 1]) < NEAR):
        flags |= FLAG_NEAR_ACCEPT

    if j_star < n_draft:
        mass = residual_mass(z_target[j_star], z_draft[j_star], T)
        if not mass.sum() > 0.0:
            mass = row_softmax(z_target[j_star], T)
            flags |= FLAG_Z_FALLBACK
    else:
        mass = row_softmax(z_target[n_draft], T)
    token, z, c_v, c_prev = inverse_cdf(mass, u_sample)
    target = u_sample * z
    if abs(target - c_v) < NEAR * z or abs(target - c_prev) < NEAR * z:
        flags |= FLAG_NEAR_SAMPLE
    return Outcome(j_star, token, alpha, s, tau, flags, u_accept, u_sample, mass)


def verify_batch(z_target, z_draft, tokens, temperature, seed, round_):
    """Verify n_req blocks: z_target [n_req, B, V], z_draft [n_req, B-1, V], tokens [n_req, B-1]."""
    return [verify_request(z_target[i], z_draft[i], tokens[i], temperature, seed, round_, i)
            for i in range(len(tokens))]
