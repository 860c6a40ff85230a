"""The cost model against the gustavoai lesson's printed figures (CPU)."""
from conftest import golden_kv
from oracle import opcount


def _model():
    g = golden_kv("opcount_minigpt.txt")
    m = dict(L=int(g["layers"][0]), d_model=int(g["d_model"][0]), d_ff=int(g["d_ff"][0]),
             vocab=int(g["vocab"][0]))
    return g, m


def test_c_row():
    g, m = _model()
    assert opcount.c_row(**m) == int(g["c_row"][0])


def test_totals_over_window():
    g, m = _model()
    T = int(g["T"][0])
    c = opcount.total_cached(T, **m)
    u = opcount.total_uncached(T, **m)
    assert c == int(g["total_cached"][0])
    assert u == int(g["total_uncached"][0])
    assert u // c == int(g["ratio_int"][0])


def test_uncached_is_t_times_cached():
    _, m = _model()
    for t in (1, 8, 64, 1000):
        assert opcount.cost_uncached(t, **m) == t * opcount.cost_cached(t, **m)


def test_crossover_and_flatness():
    g, m = _model()
    assert opcount.attention_equals_matrices_at(**m) == int(g["crossover_t"][0])
    pct = (opcount.cost_cached(64, **m) / opcount.cost_cached(1, **m) - 1) * 100
    assert int(pct) == int(g["c64_over_c1_pct_int"][0])


def test_score_memory_one_head():
    g = golden_kv("score_memory.txt")
    n, b = int(g["n"][0]), int(g["elem_bytes"][0])
    assert opcount.score_bytes_per_step(n, b, cached=False) == int(g["recompute_bytes"][0])
    assert opcount.score_bytes_per_step(n, b, cached=True) == int(g["cached_bytes"][0])
