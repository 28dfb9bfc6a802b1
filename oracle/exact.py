"""Exact rational model of tree sampling verification (TEST INFRASTRUCTURE ONLY).

The modified rejection sampling rule of the hierarchical speculative decoding blog
(section on modified rejection sampling): a draft token x drawn with probability q(x)
is kept with probability min(1, p(x)/q(x)); on refusal the remaining guesses are dropped
and a correction is drawn from max(0, p-q) renormalised; min(q,p) + max(0,p-q) = p makes
the emitted token follow p.  On a tree (our reading), a node's children are tried in
ascending id, each against the residual left by the previous refusals.

Everything here is exact (fractions.Fraction), with no sampling: it yields the exact
probability of every outcome.  It pins the oracle's sampler statistically (outcome
frequencies over many Philox streams) and pins the reading itself (losslessness).
"""
from __future__ import annotations

from collections import defaultdict
from fractions import Fraction


def _frac_row(row):
    return [Fraction(float(x)) for x in row]


def _accept_prob(pcur_x, q_x):
    if q_x == 0:
        return Fraction(1) if pcur_x > 0 else Fraction(0)
    return min(Fraction(1), pcur_x / q_x)


def _residual(pcur, q):
    res = [max(Fraction(0), a - b) for a, b in zip(pcur, q)]
    s = sum(res)
    if s == 0:
        return pcur          # empty residual: keep the current distribution
    return [r / s for r in res]


def outcome_distribution(p_rows, q_rows, kids, tokens):
    """Exact distribution of (accepted path, next token) for fixed draft tokens.

    p_rows[u], q_rows[u]: distributions (sequences of numbers, normalised here) for
    node u (0 = virtual root); kids[u]: children of u in the order they are tried;
    tokens[c]: draft token of node c.  Returns {(path tuple, token): Fraction}."""
    P = {u: _normalise(_frac_row(r)) for u, r in p_rows.items()}
    Q = {u: _normalise(_frac_row(r)) for u, r in q_rows.items()}
    out = defaultdict(Fraction)

    def walk(u, pcur, path, prob):
        ch = kids.get(u, [])
        if not ch:
            for x, px in enumerate(pcur):
                if px:
                    out[(path, x)] += prob * px
            return
        q = Q[u]
        for c in ch:
            a = _accept_prob(pcur[tokens[c]], q[tokens[c]])
            if a > 0:
                walk(c, P[c], path + (c,), prob * a)
            prob = prob * (1 - a)
            if prob == 0:
                return
            pcur = _residual(pcur, q)
        for x, px in enumerate(pcur):
            if px:
                out[(path, x)] += prob * px

    walk(0, P[0], (), Fraction(1))
    return dict(out)


def _normalise(row):
    s = sum(row)
    return [x / s for x in row]


def emitted_first_tokens(p_of_path, q_of_path, shape, V):
    """Losslessness on a tree whose draft tokens are drawn i.i.d. from q.

    shape: nested list of children counts, e.g. [2, [1, 0]] means the root has two
    children; shape[1][i] is the shape under child i (an int = that many leaf children).
    p_of_path(tokens_tuple), q_of_path(tokens_tuple) give the teacher / draft
    distributions after the committed prefix followed by those tokens.
    Returns (dist of first emitted token, {x: dist of second emitted token given that
    the first token x was an accepted draft})."""
    first = defaultdict(Fraction)
    second = defaultdict(lambda: defaultdict(Fraction))
    accepted_first = defaultdict(Fraction)

    def children_shapes(sh):
        if isinstance(sh, int):
            return [0] * sh
        n, subs = sh[0], sh[1] if len(sh) > 1 else [0] * sh[0]
        return [subs[i] if i < len(subs) else 0 for i in range(n)]

    def run(sh, ctx, pcur, prob, emit_cb):
        """Enumerate draws of the children tokens at this node and the accept/reject
        outcomes; emit_cb(token, accepted, sub_shape, prob) on the token emitted here."""
        subs = children_shapes(sh)
        q = _normalise(_frac_row(q_of_path(ctx)))

        def try_child(i, pcur, prob):
            if i == len(subs):
                for x, px in enumerate(pcur):
                    if px:
                        emit_cb(x, False, None, prob * px)
                return
            for x in range(V):
                if q[x] == 0:
                    continue
                a = _accept_prob(pcur[x], q[x])
                if a > 0:
                    emit_cb(x, True, subs[i], prob * q[x] * a)
                if a < 1:
                    try_child(i + 1, _residual(pcur, q), prob * q[x] * (1 - a))

        if not subs:
            for x, px in enumerate(pcur):
                if px:
                    emit_cb(x, False, None, prob * px)
            return
        try_child(0, pcur, prob)

    def on_first(x, accepted, sub, prob):
        first[x] += prob
        if accepted:
            accepted_first[x] += prob
            ctx = (x,)

            def on_second(y, acc2, sub2, prob2):
                second[x][y] += prob2

            run(sub, ctx, _normalise(_frac_row(p_of_path(ctx))), prob, on_second)

    run(shape, (), _normalise(_frac_row(p_of_path(()))), Fraction(1), on_first)
    cond = {x: {y: pr / accepted_first[x] for y, pr in d.items()} for x, d in second.items()}
    return dict(first), cond
