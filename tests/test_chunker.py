"""The library's adaptive chunker (host code, no GPU) against the oracle's
(the article's §6.2 adaptive chunking, with the reading stated in
include/gq.h): identical predictions after every observation of random
sequences, and identical plans."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def gq():
    from gradient_compression_allreduce_amd import gq as mod
    return mod


@pytest.mark.parametrize("capacity,alpha", [(100, 0.25), (7, 0.5), (1, 0.25), (30, 1.0),
                                            (100, 0.1)])
def test_predictions_match_oracle(gq, oracle, capacity, alpha):
    rng = np.random.default_rng(capacity * 100 + int(alpha * 100))
    menu = [int(v) * 8192 for v in rng.choice(np.arange(1, 129), 6, replace=False)]
    ch = gq.gq_chunker_create(capacity, alpha, 131072)
    sizes, lats = [], []
    assert gq.gq_chunker_predict(ch) == oracle.chunker_predict([], [], capacity, alpha)
    for k in range(400):
        c = menu[int(rng.integers(0, len(menu)))]
        # latencies with a per-size trend and noise, some exactly tied
        lat = float(c) * (1e-9 * (1 + menu.index(c) % 3)) * (1 + 0.3 * rng.standard_normal()
                                                              if k % 5 else 1.0)
        lat = abs(lat)
        gq.gq_chunker_update(ch, c, lat)
        sizes.append(c)
        lats.append(lat)
        assert gq.gq_chunker_predict(ch) == oracle.chunker_predict(sizes, lats, capacity,
                                                                   alpha), k


def test_plan_uses_prediction(gq, oracle):
    ch = gq.gq_chunker_create()
    for c, lat in [(65536, 1.0), (262144, 3.0), (131072, 2.5)]:
        gq.gq_chunker_update(ch, c, lat)
    pred = gq.gq_chunker_predict(ch)
    assert pred == oracle.chunker_predict([65536, 262144, 131072], [1.0, 3.0, 2.5]) == 262144
    for n, e in [(1 << 20, 4), (335_000, 2), (1, 4), (30522 * 1024, 2)]:
        assert np.array_equal(gq.gq_chunker_plan(ch, n, e), oracle.plan_chunks(n, e, pred, 64))


def test_chunker_errors(gq):
    L = gq.lib
    import ctypes
    h = ctypes.c_void_p()
    for cap, a, d in [(0, 0.25, 1), (100, 0.0, 1), (100, 1.5, 1), (100, float("nan"), 1),
                      (100, 0.25, 0), ((1 << 20) + 1, 0.25, 1)]:
        assert L.gq_chunker_create(cap, a, d, ctypes.byref(h)) == gq.GQ_ERR_INVALID
        assert not h.value
    ch = gq.gq_chunker_create()
    for c, lat in [(0, 1.0), (100, -1.0), (100, float("inf")), (100, float("nan"))]:
        with pytest.raises(gq.GQError) as e:
            gq.gq_chunker_update(ch, c, lat)
        assert e.value.status == gq.GQ_ERR_INVALID
    assert gq.gq_chunker_predict(ch) == 131072
    assert L.gq_chunker_destroy(None) == gq.GQ_OK
