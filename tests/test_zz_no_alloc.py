"""fz_extend_batch_noalloc (the entry point that allocates nothing, for
callers that cannot allocate device memory) against fz_extend_batch without
traceback, on the same seeded inputs: every field of every hit, bit for bit,
on calls in a row with shrinking inputs (the static scratch keeps the last
call's contents), plus its size limits and flag checks."""
import random

import numpy as np
import pytest

from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402


def log(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    c = fz.Context(0)
    yield c
    c.close()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def both(ctx, w, ydrop=None, query_rc=False):
    T, Q, S = dev(w["target"]), dev(w["query"]), dev(w["seeds"])
    yd = w["ydrop"] if ydrop is None else ydrop
    log("noalloc: %d seeds, target %d, query %d" % (S.shape[0], T.numel(), Q.numel()))
    h0, _, st0 = ctx.extend(T, Q, S, w["scoring"], yd, traceback=False, want_stats=True, query_rc=query_rc)
    h1, st1 = ctx.extend_noalloc(T, Q, S, w["scoring"], yd, want_stats=True, query_rc=query_rc)
    torch.cuda.synchronize()
    log("noalloc: done")
    a, b = h0.cpu().numpy(), h1.cpu().numpy()
    bad = np.argwhere(a != b)
    assert bad.size == 0, "first mismatches (row, field): %s; %s vs %s" % (
        bad[:4].tolist(), a[bad[0][0]].tolist(), b[bad[0][0]].tolist())
    assert st0["cells"] == st1["cells"] and st0["n_overflow"] == st1["n_overflow"]
    return a, st1


def one_seed(t, q, tp, qp, L):
    T = np.frombuffer(t.encode(), dtype=np.uint8).copy()
    Q = np.frombuffer(q.encode(), dtype=np.uint8).copy()
    S = np.array([[tp, qp, L, 0, len(t), 0, len(q)]], dtype=np.int64)
    return dict(target=T, query=Q, seeds=S, scoring=dict(W.DEFAULT_SCORING), ydrop=9400)


def test_noalloc_matches_extend_batch(ctx):
    # a skewed batch near the size limits, then smaller batches on the same scratch
    w = W.skewed(target_len=3_000_000, n_seeds=60_000, seed=1)
    assert len(w["target"]) <= fz.FZ_NOALLOC_MAX_BASES and len(w["query"]) <= fz.FZ_NOALLOC_MAX_BASES
    h, st = both(ctx, w)
    assert st["cells"] > 0 and (h[:, 1] == 0).mean() > 0.99
    both(ctx, W.tiny(n_seeds=300, seed=4))
    both(ctx, W.tiny(n_seeds=40, seed=6), query_rc=True)
    # a band that outgrows the standard window: the wide retry runs from the scratch too
    rng = random.Random(8)
    s = "".join(rng.choice("ACGT") for _ in range(719))
    h, st = both(ctx, one_seed(s, s, 0, 0, 19), ydrop=fz.FZ_YDROP_INF)
    assert st["n_overflow"] == 1
    # matrix scoring with N
    both(ctx, W.with_matrix_and_n(W.tiny(n_seeds=120, seed=7), 20, 1, 12, seed=3))


def test_noalloc_limits_and_flags(ctx):
    w = W.tiny(n_seeds=4, seed=2)
    T, Q, S = dev(w["target"]), dev(w["query"]), dev(w["seeds"])
    big = torch.zeros(fz.FZ_NOALLOC_MAX_BASES + 1, dtype=torch.uint8, device="cuda:0") + ord("A")
    with pytest.raises(fz.FzError) as e:
        ctx.extend_noalloc(big, Q, S, w["scoring"], 9400)
    assert e.value.code == fz.FZ_EINVAL and "at most" in str(e.value)
    many = S[:1].repeat(fz.FZ_NOALLOC_MAX_SEEDS + 1, 1).contiguous()
    with pytest.raises(fz.FzError) as e:
        ctx.extend_noalloc(T, Q, many, w["scoring"], 9400)
    assert e.value.code == fz.FZ_EINVAL and "at most" in str(e.value)
    with pytest.raises(fz.FzError) as e:
        fz.fz_extend_batch_noalloc(ctx.h, T, Q, S, w["scoring"], 9400, flags=fz.FZ_TRACEBACK)
    assert e.value.code == fz.FZ_EINVAL
    # a valid call after the rejected ones
    both(ctx, w)
