"""Shared comparison rules of the GPU parity tests (imported by test modules;
not collected itself).

Sampled acceptance: the GPU and the oracle must give the same accept length,
path and tokens, except where the first decision on which they part lies within
EXEMPT of its threshold -- a child test with |u - ratio| < EXEMPT, or the bonus
draw with u * total within EXEMPT * total of a cumulative boundary.  The
oracle's trace gives each decision's (row, slot, u, ratio or margin).
"""
EXEMPT = 1e-6


def first_divergence_exempt(tr, par, g_len, g_path, o_len, o_path):
    """True when the first decision on which the GPU's result (g_len, g_path) and
    the oracle's (o_len, o_path, trace tr) part lies within EXEMPT of its
    threshold.  par: flattened parent rows of the sequence's tree."""
    k = 0
    while k < min(g_len, o_len) and g_path[k] == o_path[k]:
        k += 1
    cur = 0 if k == 0 else int(o_path[k - 1])
    kids = [j for j in range(len(par)) if par[j] == cur]
    g_next = int(g_path[k]) if k < g_len else None
    o_next = int(o_path[k]) if k < o_len else None
    if g_next == o_next:  # the same path: the bonus draw differs
        rows = [r for r in tr if int(r[0]) == cur and r[1] < 0]
        return bool(rows) and rows[-1][3] < EXEMPT
    # the earlier of the two accepted slots (a side that accepted nothing here
    # rejected every child): the decision at that slot went differently
    slot = min(kids.index(x) if x is not None else len(kids) for x in (g_next, o_next))
    rows = [r for r in tr if int(r[0]) == cur and int(r[1]) == slot]
    return bool(rows) and abs(rows[-1][2] - rows[-1][3]) < EXEMPT
