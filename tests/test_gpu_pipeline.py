"""The whole chain on the GPU -- seed stage, then covered-seed rounds -- on
both strands of a chromosome pair, against the oracle's seed stage and
rounds on the same inputs: every seed, every covered flag, every field and
CIGAR of every extended seed."""
import numpy as np
import pytest

import oracle
from smith_waterman_dp_amd import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from smith_waterman_dp_amd import fz  # noqa: E402

from test_gpu_parity import compare  # noqa: E402


def log(msg):
    print("[gpu] " + msg, flush=True)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.zeros(1, device="cuda:0").add_(1)
    torch.cuda.synchronize()
    c = fz.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("rc", [False, True])
def test_seed_stage_then_rounds(ctx, rc):
    w = W.chromosome(length=250_000, inv_min=20_000, inv_max=60_000, seed=12)
    T = torch.from_numpy(w["target"]).to("cuda:0")
    Q = torch.from_numpy(w["query"]).to("cuda:0")
    seeds, nh = ctx.find_seeds(T, Q, k=19, flank=32768, query_rc=rc)
    qo = oracle.revcomp(w["query"]) if rc else w["query"]
    ref_seeds, ref_nh = oracle.find_seeds(w["target"], w["query"], 19, 32768, query_rc=rc)
    assert nh == ref_nh and np.array_equal(seeds.cpu().numpy(), ref_seeds)
    # a seeded order, the same on both sides
    perm = np.random.default_rng(5).permutation(len(ref_seeds))
    S = ref_seeds[perm]
    log("%s strand: %d seeds" % ("reverse" if rc else "forward", len(S)))
    h, c, _ = ctx.extend_rounds(T, Q, seeds[torch.from_numpy(perm).to("cuda:0")], w["scoring"], w["ydrop"], 3000,
                                128, query_rc=rc)
    gh, gc = h.cpu().numpy(), c.cpu().numpy().view(np.uint32)
    oh, ow, oo = oracle.extend_rounds(w["target"], qo, S, w["scoring"], w["ydrop"], 3000, 128)
    gcov = (gh[:, 1] & fz.FZ_HIT_COVERED) != 0
    assert np.array_equal(gcov, (oh["status"] & oracle.STATUS_COVERED) != 0)
    idx = np.nonzero(~gcov)[0]
    compare(gh, gc, oh[idx], ow, oo[idx], idx=idx, label="pipeline %s" % ("rc" if rc else "fwd"))
    log("covered %d, extended %d" % (gcov.sum(), idx.size))


def test_chain_with_n_and_matrix(ctx):
    """Sequences with runs of N scored with the 4x4 matrix: the seed stage
    skips k-mers with N, the rounds extend through N with the N score."""
    w = W.chromosome(length=150_000, inv_min=10_000, inv_max=30_000, seed=13)
    rng = np.random.default_rng(14)
    Tn = W.plant_n_runs(rng, w["target"], 15, 5, 400)
    Qn = W.plant_n_runs(rng, w["query"], 15, 5, 400)
    sc = W.matrix_scoring()
    T = torch.from_numpy(Tn).to("cuda:0")
    Q = torch.from_numpy(Qn).to("cuda:0")
    seeds, nh = ctx.find_seeds(T, Q, k=19, flank=32768)
    ref_seeds, ref_nh = oracle.find_seeds(Tn, Qn, 19, 32768)
    assert nh == ref_nh and np.array_equal(seeds.cpu().numpy(), ref_seeds)
    perm = np.random.default_rng(15).permutation(len(ref_seeds))
    h, c, _ = ctx.extend_rounds(T, Q, seeds[torch.from_numpy(perm).to("cuda:0")], sc, w["ydrop"], 3000, 64)
    gh, gc = h.cpu().numpy(), c.cpu().numpy().view(np.uint32)
    oh, ow, oo = oracle.extend_rounds(Tn, Qn, ref_seeds[perm], sc, w["ydrop"], 3000, 64)
    gcov = (gh[:, 1] & fz.FZ_HIT_COVERED) != 0
    assert np.array_equal(gcov, (oh["status"] & oracle.STATUS_COVERED) != 0)
    idx = np.nonzero(~gcov)[0]
    compare(gh, gc, oh[idx], ow, oo[idx], idx=idx, label="chain with N and matrix")
    log("%d seeds, covered %d" % (len(perm), gcov.sum()))


def test_two_contexts_two_threads(ctx):
    """Both strands at once, each on its own context and stream from its own
    host thread, give exactly the results of running them one after the
    other (the library keeps no state outside a context)."""
    import concurrent.futures

    w = W.chromosome(length=200_000, inv_min=20_000, inv_max=50_000, seed=16)
    T = torch.from_numpy(w["target"]).to("cuda:0")
    Q = torch.from_numpy(w["query"]).to("cuda:0")
    torch.cuda.synchronize()

    def chain(c, rc, strm):
        with torch.cuda.stream(strm):
            s, _ = c.find_seeds(T, Q, k=19, flank=32768, query_rc=rc, stream=strm)
            h, cg, _ = c.extend_rounds(T, Q, s, w["scoring"], w["ydrop"], 3000, 64, query_rc=rc, doubling=True,
                                       stream=strm)
            strm.synchronize()
        return s.cpu().numpy(), h.cpu().numpy(), cg.cpu().numpy()

    serial = [chain(ctx, rc, torch.cuda.Stream()) for rc in (False, True)]
    ctxs = [fz.Context(0), fz.Context(0)]
    try:
        with concurrent.futures.ThreadPoolExecutor(2) as pool:
            par = list(pool.map(lambda a: chain(ctxs[a], bool(a), torch.cuda.Stream()), (0, 1)))
    finally:
        for c in ctxs:
            c.close()
    for x, y in zip(serial, par):
        for u, v in zip(x, y):
            assert np.array_equal(u, v)
    log("strands: %d and %d seeds" % (len(serial[0][0]), len(serial[1][0])))
