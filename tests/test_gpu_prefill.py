"""GPU parity of the causal prefill chunk (compressed entries at ratio 2)
against the oracle: indexer scores exact, per-query Top-512 indices
bit-exact, attention of every layer within tolerance.  Small chunks span
several 32-query x 512-entry score tiles with ragged tails, short contexts
(fewer visible entries than k) and caches longer than the visible range;
the full 4,096-query chunk over 64K entries is checked on sampled queries."""
import numpy as np
import pytest
import torch

import oracle
from oracle import workloads as ow
from synth import configs as C
from gpu_helpers import assert_attention_close, dev, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_quant_amd import workloads
    return workloads


def _small(**kw):
    return C.ENCODER_PREFILL_128K.with_(**kw)


@pytest.mark.parametrize("weights", [False, True])
def test_prefill_scores_are_exact(wl, weights):
    import fp4_kv_cache_quant_amd as csa2
    cfg = _small(n_entries=1537, n_q=45, t0=2 * 1537 - 60)
    print_case(f"prefill scores n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0} weights={weights}")
    inp = wl.build_prefill_inputs(cfg)
    q = inp.idx_q[0]
    w = None
    w_host = None
    if weights:  # small integer and fractional weights, exactly representable
        rng = np.random.default_rng(7)
        w_host = (rng.integers(-2, 5, size=(cfg.n_q, 8)) * 0.25).astype(np.float32)
        w = torch.from_numpy(w_host).cuda()
    scores = torch.empty(cfg.n_q, cfg.n_entries, dtype=torch.float32, device="cuda")
    n_vis = torch.empty(cfg.n_q, dtype=torch.int32, device="cuda")
    csa2.prefill_index_score(q, inp.entry_k, cfg.t0, cfg.ratio, scores, n_vis, w=w)
    got = scores.cpu().numpy()
    nv = n_vis.cpu().numpy()
    keys = ow.prefill_entry_keys(cfg)
    qh = q.cpu().numpy().view(np.uint16)
    for i in range(cfg.n_q):
        v = oracle.prefill_visible_entries(cfg.t0 + i, cfg.ratio, cfg.n_entries)
        assert nv[i] == v
        ref = oracle.index_score(qh[i], keys, np.arange(v), None if w_host is None else w_host[i])
        assert np.array_equal(got[i, :v], ref.astype(np.float32)), f"query {i}"
        assert np.all(np.isneginf(got[i, v:])), f"query {i} invisible entries"


CHUNKS = {
    # the chunk ends at the end of the cache: visible counts grow to n_entries
    "tail": _small(n_entries=3000, n_q=37, t0=2 * 3000 - 37),
    # fewer visible entries than k: every visible entry is selected, -1 padded
    "short": _small(n_entries=300, n_q=20, t0=2 * 300 - 20),
    # the cache holds more entries than any query of the chunk can see
    "mid_cache": _small(n_entries=2500, n_q=45, t0=3000),
    # a Reindex layer rescores with its own Q; Reuse layers follow both
    "reindex": _small(n_entries=1500, n_q=24, t0=2 * 1500 - 24,
                      layers=((C.FULL, 0, 0), (C.REUSE, 0, 0), (C.REINDEX, 0, 0), (C.REUSE, 0, 0))),
    # ratio 1 (every token an entry), window shorter than 128
    "ratio1_swa16": _small(n_entries=900, n_q=33, t0=900 - 33, ratio=1, swa=16),
    # the earliest chunk start a 128-token window allows (t0 = 127), ratio 3:
    # 42 .. 65 visible entries, fewer than k
    "start_ratio3": _small(n_entries=400, n_q=70, t0=127, ratio=3),
    # a one-token window from token 0: the first queries see no entry at all
    # (the window alone is attended)
    "no_entries_swa1": _small(n_entries=50, n_q=40, t0=0, ratio=3, swa=1),
    # no sliding window: the selected entries alone are attended
    "no_window": _small(n_entries=600, n_q=25, t0=2 * 600 - 25, swa=0),
    # a long Reuse run
    "long_reuse": _small(n_entries=700, n_q=30, t0=2 * 700 - 30,
                         layers=((C.FULL, 0, 0),) + ((C.REUSE, 0, 0),) * 9),
}


@pytest.mark.parametrize("name", list(CHUNKS))
def test_prefill_chunk_matches_oracle(wl, name):
    cfg = CHUNKS[name]
    print_case(f"prefill chunk {name}: n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0} "
               f"ratio={cfg.ratio} layers={len(cfg.layers)}")
    inp = wl.build_prefill_inputs(cfg)
    pf, io = wl.make_prefill(inp)
    for rep in range(2):  # the workspace is left ready for the next call
        pf.run(io)
        torch.cuda.synchronize()
    keys = ow.prefill_entry_keys(cfg)
    idx = [t.cpu().numpy() if t is not None else None for t in inp.idx]
    outs = [o.cpu().numpy() for o in inp.out]
    for i in range(cfg.n_q):
        ref = ow.prefill_reference(cfg, i, entry_keys=keys)
        src = None
        for l, r in enumerate(ref):
            if cfg.layers[l][0] != C.REUSE:
                src = l
                assert np.array_equal(idx[l][i], r.idx), f"query {i} layer {l} indices"
            else:
                assert np.array_equal(idx[src][i], r.idx)
            assert_attention_close(outs[l][i], r.out, f"query {i} layer {l}")


def test_prefill_full_chunk_sampled_queries(wl):
    """The 4,096-query chunk over 65,536 entries (131,072 tokens), as the
    benchmark runs it; sampled queries against the oracle."""
    cfg = C.ENCODER_PREFILL_128K
    print_case(f"prefill full chunk n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0}")
    inp = wl.build_prefill_inputs(cfg)
    pf, io = wl.make_prefill(inp)
    pf.run(io)
    torch.cuda.synchronize()
    keys = ow.prefill_entry_keys(cfg)
    rng = np.random.default_rng(3)
    sample = sorted({0, 1, 31, 32, 2047, 4094, 4095, *rng.integers(0, cfg.n_q, 5).tolist()})
    idx0 = inp.idx[0].cpu().numpy()
    assert np.all(np.diff(idx0, axis=1) > 0)          # ascending, all 512 selected
    for i in sample:
        ref = ow.prefill_reference(cfg, i, entry_keys=keys)
        assert np.array_equal(idx0[i], ref[0].idx), f"query {i} indices"
        for l in range(len(cfg.layers)):
            assert_attention_close(inp.out[l][i].cpu().numpy(), ref[l].out, f"query {i} layer {l}")


MANY_ROWS = {
    # 300 queries over a 40,000-entry cache (rows long enough for the
    # many-row selection) of which each query sees about half: half of the
    # sampled slots lie past the visible range
    "half_visible": _small(n_entries=40000, n_q=300, t0=40000),
    # ratio 1, 4,101 .. 4,400 visible entries: a row needs 4,229 of them for
    # a threshold estimate (the r-th largest of 1,024 samples with r <= 256),
    # so queries 0..127 take the fallback and 128..299 the estimate
    "estimate_edge": _small(n_entries=40000, n_q=300, t0=4100, ratio=1),
}


@pytest.mark.parametrize("name", list(MANY_ROWS))
def test_prefill_many_rows_partial_visibility(wl, name):
    cfg = MANY_ROWS[name]
    print_case(f"prefill many rows {name}: n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0} ratio={cfg.ratio}")
    inp = wl.build_prefill_inputs(cfg)
    pf, io = wl.make_prefill(inp)
    pf.run(io)
    torch.cuda.synchronize()
    keys = ow.prefill_entry_keys(cfg)
    rng = np.random.default_rng(11)
    sample = sorted({0, 1, 126, 127, 128, 129, 255, 256, 298, 299, *rng.integers(0, cfg.n_q, 4).tolist()})
    idx0 = inp.idx[0].cpu().numpy()
    for i in sample:
        ref = ow.prefill_reference(cfg, i, entry_keys=keys)
        assert np.array_equal(idx0[i], ref[0].idx), f"query {i} indices"
        for l in range(len(cfg.layers)):
            assert_attention_close(inp.out[l][i].cpu().numpy(), ref[l].out, f"query {i} layer {l}")


def _sampled_entries(n_entries: int) -> np.ndarray:
    """The entries whose scores give a query's threshold estimate: 64 runs of
    16 entries, one at the start of each 64th of the cache."""
    i = np.arange(1024)
    return (i >> 4) * (n_entries >> 6) + (i & 15)


@pytest.mark.parametrize("planted", ["high", "zero"])
def test_prefill_selection_when_the_estimate_fails(wl, planted):
    """Many queries are selected from each query's candidates at or above a
    threshold estimated on sampled entries.  Planted keys make the estimate
    fail: 64.0 in every dim of 40 sampled entries (more than the estimate's
    rank, about 34 here) puts the threshold above every other entry's
    score, so fewer than k candidates pass; zero keys on all sampled entries
    put it at 0, so every score passes and the candidate regions overflow.
    Such queries take the full selection over their score rows; the indices
    must still be the oracle's."""
    cfg = _small(n_entries=40000, n_q=300, t0=2 * 40000 - 300)
    print_case(f"prefill estimate failure ({planted}): n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0}")
    inp = wl.build_prefill_inputs(cfg)
    keys = ow.prefill_entry_keys(cfg).copy()
    rows = _sampled_entries(cfg.n_entries)
    if planted == "high":
        keys[rows[:40]] = 0x4280                                # bf16 64.0
    else:
        keys[rows] = 0x0000                                     # bf16 +0.0
    inp.entry_k.copy_(torch.from_numpy(keys.view(np.int16)).to(inp.entry_k.device).view(inp.entry_k.dtype))
    pf, io = wl.make_prefill(inp)
    pf.run(io)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    sample = sorted({0, 1, 150, 298, 299, *rng.integers(0, cfg.n_q, 3).tolist()})
    idx0 = inp.idx[0].cpu().numpy()
    for i in sample:
        ref = ow.prefill_reference(cfg, i, entry_keys=keys)
        assert np.array_equal(idx0[i], ref[0].idx), f"query {i} indices"
        assert_attention_close(inp.out[0][i].cpu().numpy(), ref[0].out, f"query {i} layer 0")


SELECT_CASES = {
    # the chunk's shape class that is filtered while scoring (n_q >= 256, k <= 512, 32,769..65,536 entries)
    "filtered": dict(n_entries=40000, n_q=300, t0=2 * 40000 - 300, weights=False, plant=None),
    # the same with dyadic head weights (every product and sum exact in binary32)
    "filtered_weights": dict(n_entries=40000, n_q=300, t0=2 * 40000 - 300, weights=True, plant=None),
    # sampled entries planted high: the estimate admits fewer than k, the rows are scored again in full
    "filtered_fallback": dict(n_entries=40000, n_q=300, t0=2 * 40000 - 300, weights=False, plant="high"),
    # ratio 1 with 4,101..4,400 visible entries: rows without an estimate next to rows with one
    "filtered_edge": dict(n_entries=40000, n_q=300, t0=4100, ratio=1, weights=False, plant=None),
    # fewer queries than the filtered path takes: every score is written and selected
    "unfiltered": dict(n_entries=40000, n_q=100, t0=2 * 40000 - 100, weights=False, plant=None),
    # a small k on the filtered path (thresholds a little over twice 64 entries)
    "filtered_k64": dict(n_entries=40000, n_q=300, t0=2 * 40000 - 300, weights=False, plant=None, k=64),
    # k above the filtered path's 512 at the filtered shape: scores written and selected
    "unfiltered_k1024": dict(n_entries=40000, n_q=300, t0=2 * 40000 - 300, weights=False, plant=None, k=1024),
    # the filtered path's edges: the fewest queries (256) over the most entries (65,536, 128 lists of 512)
    "filtered_edge_max": dict(n_entries=65536, n_q=256, t0=2 * 65536 - 256, weights=False, plant=None),
    # the fewest entries it takes (32,769: a last list of one entry) and a last query block of one query
    "filtered_edge_min": dict(n_entries=32769, n_q=257, t0=2 * 32769 - 257, weights=False, plant=None),
}


@pytest.mark.parametrize("name", list(SELECT_CASES))
def test_prefill_select_matches_oracle(wl, name):
    """csa2_prefill_select: each query's Top-512 over its visible entries
    and the visible counts, on sampled queries against the oracle's scores
    and selection; the call runs twice on one workspace."""
    import fp4_kv_cache_quant_amd as csa2
    c = dict(SELECT_CASES[name])
    weights, plant, ratio, k = c.pop("weights"), c.pop("plant"), c.pop("ratio", 2), c.pop("k", None)
    cfg = _small(ratio=ratio, **c)
    print_case(f"prefill select {name}: n_entries={cfg.n_entries} n_q={cfg.n_q} t0={cfg.t0} ratio={cfg.ratio}")
    inp = wl.build_prefill_inputs(cfg)
    keys = ow.prefill_entry_keys(cfg).copy()
    if plant == "high":
        keys[_sampled_entries(cfg.n_entries)[:40]] = 0x4280    # bf16 64.0
    keys_d = torch.from_numpy(keys.view(np.int16)).cuda().view(torch.bfloat16)
    q = inp.idx_q[0]
    w_host = w = None
    if weights:
        rng = np.random.default_rng(3)
        w_host = (rng.integers(-2, 5, size=(cfg.n_q, 8)) * 0.25).astype(np.float32)
        w = torch.from_numpy(w_host).cuda()
    k = k or cfg.topk
    ws = torch.zeros(csa2.prefill_select_workspace_size(cfg.n_entries, cfg.n_q, k), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty(cfg.n_q, k, dtype=torch.int32, device="cuda")
    n_vis = torch.empty(cfg.n_q, dtype=torch.int32, device="cuda")
    qh = q.cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(17)
    sample = sorted({i for i in (0, 1, 127, 128, cfg.n_q - 1) if i < cfg.n_q} | set(rng.integers(0, cfg.n_q, 5).tolist()))
    for rep in range(2):
        idx.fill_(-7)
        csa2.prefill_select(q, keys_d, cfg.t0, cfg.ratio, idx, n_vis, ws, w=w)
        torch.cuda.synchronize()
        got, nv = idx.cpu().numpy(), n_vis.cpu().numpy()
        for i in sample:
            v = oracle.prefill_visible_entries(cfg.t0 + i, cfg.ratio, cfg.n_entries)
            assert nv[i] == v, f"query {i} visible count"
            ids = np.arange(v)
            sc = oracle.index_score(qh[i], keys, ids, None if w_host is None else w_host[i])
            ref = oracle.select(sc, ids, k)
            assert np.array_equal(got[i], ref), f"call {rep} query {i} indices"
