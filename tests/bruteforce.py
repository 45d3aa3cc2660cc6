"""Exhaustive path enumeration for tiny alignment problems (test helper).

This is deliberately a different mechanism from the oracle's dynamic
programming: it lists every alignment path explicitly and scores each one
from its op string, so a wrong recurrence term, sign or index in the oracle
shows up as a disagreement.

A path starts at (0, 0).  'M' moves (i, j) -> (i+1, j+1) and scores
sub(a[i], b[j]); 'I' moves (i, j) -> (i, j+1) (query only); 'D' moves
(i, j) -> (i+1, j) (target only).  Every maximal run of g equal gap letters
costs open + g * extend (an I-run directly followed by a D-run is two runs).
"""
import itertools

NEG = None


def sub(x, y, sc):
    """x from the target, y from the query."""
    x, y = x.upper(), y.upper()
    if "matrix" in sc:
        if x == "N" or y == "N":
            return sc["n_score"]
        return sc["matrix"]["ACGT".index(x)]["ACGT".index(y)]
    if x == y:
        return sc["match"]
    purine = set("AG")
    if (x in purine) == (y in purine):
        return sc["transition"]
    return sc["transversion"]


def path_score(ops, a, b, sc, start=(0, 0)):
    """Score of an op string applied from `start` (no validity checks)."""
    i, j = start
    total = 0
    prev = None
    for op in ops:
        if op == "M":
            total += sub(a[i], b[j], sc)
            i += 1
            j += 1
        else:
            total -= sc["gap_extend"]
            if prev != op:
                total -= sc["gap_open"]
            if op == "I":
                j += 1
            else:
                i += 1
        prev = op
    return total


def _extend(cell, op):
    i, j = cell
    if op == "M":
        return (i + 1, j + 1)
    if op == "I":
        return (i, j + 1)
    return (i + 1, j)


def ydrop_enumerate(a, b, sc, ydrop):
    """Anchored extension from (0,0) with anti-diagonal y-drop, by enumeration.

    Cells are settled one anti-diagonal d = i + j at a time.  V(c) is the best
    score over all paths to c whose earlier cells are all live; c is live when
    V(c) >= T_d, T_d = (best V over live cells of diagonals < d) - ydrop
    (ydrop None = no pruning).  Returns (V, live, paths) where paths[c] lists
    (score, ops) of every admissible path to c.
    """
    m, n = len(a), len(b)
    paths = {(0, 0): [(0, "")]}
    V = {(0, 0): 0}
    live = {(0, 0)}
    best = 0
    for d in range(1, m + n + 1):
        thr = None if ydrop is None else best - ydrop
        newly = []
        for i in range(max(0, d - n), min(m, d) + 1):
            c = (i, d - i)
            plist = []
            for op in "MID":
                # predecessor p with _extend(p, op) == c
                if op == "M":
                    p = (c[0] - 1, c[1] - 1)
                elif op == "I":
                    p = (c[0], c[1] - 1)
                else:
                    p = (c[0] - 1, c[1])
                if p not in live:
                    continue
                for _, ops in paths[p]:
                    nops = ops + op
                    plist.append((path_score(nops, a, b, sc), nops))
            if not plist:
                continue
            v = max(s for s, _ in plist)
            V[c] = v
            paths[c] = plist
            if thr is None or v >= thr:
                newly.append(c)
        for c in newly:
            live.add(c)
        if newly:
            best = max(best, max(V[c] for c in newly))
    return V, live, paths


def _rank(prev, op):
    # Reversed-path tie order: after an 'I' (inside an insertion) the gap is
    # preferably opened here, so M < D < I; otherwise M < I < D.
    if prev == "I":
        return {"M": 0, "D": 1, "I": 2}[op]
    return {"M": 0, "I": 1, "D": 2}[op]


def tie_key(ops):
    """Key that orders op strings by the traceback tie rules, read end-first."""
    rev = ops[::-1]
    key = []
    prev = None
    for op in rev:
        key.append(_rank(prev, op))
        prev = op
    return tuple(key)


def extension_brute(a, b, sc, ydrop):
    """Best live cell (max V, then smallest d, then smallest i) and the tie-ruled
    optimal path to it."""
    V, live, paths = ydrop_enumerate(a, b, sc, ydrop)
    best = max(V[c] for c in live)
    cands = sorted((c[0] + c[1], c[0]) for c in live if V[c] == best)
    d, i = cands[0]
    end = (i, d - i)
    opt = [ops for s, ops in paths[end] if s == best]
    ops = min(opt, key=tie_key)
    return dict(score=best, ie=end[0], je=end[1], ops=ops, live=live, V=V)


def local_brute(a, b, sc):
    """Local alignment by enumeration: best score over every start cell and
    every path, floored at 0; end = smallest d then smallest i."""
    m, n = len(a), len(b)
    best = {(i, j): 0 for i in range(m + 1) for j in range(n + 1)}
    for i0 in range(m + 1):
        for j0 in range(n + 1):
            frontier = [((i0, j0), "")]
            while frontier:
                nxt = []
                for cell, ops in frontier:
                    for op in "MID":
                        c = _extend(cell, op)
                        if c[0] > m or c[1] > n:
                            continue
                        nops = ops + op
                        s = path_score(nops, a, b, sc, start=(i0, j0))
                        if s > best[c]:
                            best[c] = s
                        nxt.append((c, nops))
                frontier = nxt
    top = max(best.values())
    d, i = min((c[0] + c[1], c[0]) for c, v in best.items() if v == top)
    return dict(score=top, ie=i, je=d - i)


def all_strings(alphabet, length):
    return ["".join(p) for p in itertools.product(alphabet, repeat=length)]
