"""The C ABI on a host without a GPU: the library loads, exports every entry
point declared in include/csa2.h, and rejects bad arguments on the host
before anything is enqueued (no call here reaches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def csa2():
    import fp4_kv_cache_quant_amd as m
    return m


def test_every_declared_symbol_is_exported(csa2):
    names = _declared_symbols()
    assert len(names) >= 14, names
    lib = ctypes.CDLL(csa2.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_abi_version(csa2):
    assert csa2.abi_version() == 7


def _err(csa2):
    return csa2._last_error().decode()


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def test_topk_rejects_bad_k_and_n(csa2):
    W = 1 << 30

    def call(scores=FAKE, n=100, len_div=1, k=512, pool=None, n_pool=0, ws=FAKE, ws_bytes=W, n_seq=1):
        return csa2._topk(scores, n, None, len_div, k, pool, n_pool, 8, FAKE, ws, ws_bytes, n_seq, None)

    assert call(k=0) == -2 and "k must be" in _err(csa2)
    assert call(k=4096) == -2
    assert call(n=2_000_000) == -2
    assert call(pool=FAKE, n_pool=10) == -2          # n != n_pool * blk
    assert call(scores=None) == -1
    assert call(ws=None) == -1
    assert call(ws=FAKE + 8) == -1                   # alignment
    assert call(len_div=0) == -1
    assert call(ws_bytes=csa2.topk_workspace_size(100, 1) - 1) == -3
    assert call(scores=None, n_seq=0) == 0           # n_seq = 0: no-op
    assert csa2.topk_workspace_size(100, 2) > csa2.topk_workspace_size(100, 1) > 0


def test_index_score_rejects_bad_shapes(csa2):
    assert csa2._index_score(FAKE, None, FAKE, 100, FAKE, 1, None, 0, 8, FAKE, 200, 1, None) == -2
    assert "exceeds key_cap" in _err(csa2)
    assert csa2._index_score(FAKE, None, FAKE, 100, FAKE, 1, FAKE, 10, 8, FAKE, 81, 1, None) == -2
    assert csa2._index_score(FAKE + 2, None, FAKE, 100, FAKE, 1, None, 0, 8, FAKE, 50, 1, None) == -1
    assert "aligned" in _err(csa2)
    assert csa2._index_score(FAKE, None, None, 100, FAKE, 1, None, 0, 8, FAKE, 50, 1, None) == -1


def test_attention_rejects_small_workspace_and_bad_sizes(csa2):
    kv = csa2._FP4KV(FAKE, FAKE, 1000, 1)
    need = csa2.sparse_attn_workspace_size(1, 512, 128)
    assert need > 0
    args = dict(q=FAKE, n_q=1, q_per_seq=1, idx=FAKE, k_idx=512, swa=FAKE, st=128, swa_len=FAKE, swa_max=128)

    def call(ws_bytes, **kw):
        a = {**args, **kw}
        return csa2._attn(a["q"], a["n_q"], ctypes.byref(kv), a["q_per_seq"], a["idx"], a["k_idx"], a["swa"],
                          a["st"], a["swa_len"], a["swa_max"], 0.04, FAKE, FAKE, ws_bytes, None)

    assert call(need - 1) == -3 and "workspace" in _err(csa2)
    assert call(need, swa_max=5000) == -2
    assert call(need, k_idx=0, swa_max=0) == -2
    assert call(need, n_q=2) == -2  # two queries, one cache sequence
    assert call(need, q=FAKE + 8) == -1
    assert call(need, st=-1) == -1 and "stride" in _err(csa2)


def test_context_parallel_share_and_merge_reject_bad_arguments(csa2):
    kv = csa2._FP4KV(FAKE, FAKE, 1000, 1)
    need = csa2.sparse_attn_workspace_size(1, 512, 128)

    def share(out_ml, **kw):
        a = dict(q=FAKE, n_q=1, k_idx=512, swa_max=128, out_o=FAKE)
        a.update(kw)
        return csa2._attn_partial(a["q"], a["n_q"], ctypes.byref(kv), 1, FAKE, a["k_idx"], FAKE, 128, FAKE,
                                  a["swa_max"], 0.04, a["out_o"], out_ml, FAKE, need, None)

    assert share(None) == -1 and "out_ml" in _err(csa2)
    assert share(FAKE + 4) == -1 and "align" in _err(csa2)
    assert share(FAKE, out_o=FAKE + 8) == -1
    assert share(FAKE, swa_max=5000) == -2
    assert share(None, n_q=0) == 0  # nothing to do, nothing checked past n_q
    merge = csa2._attn_merge
    assert merge(FAKE, FAKE, 0, 4, FAKE, None) == -2 and "n_parts" in _err(csa2)
    assert merge(FAKE, FAKE, 2, 70000, FAKE, None) == -2
    assert merge(None, FAKE, 2, 4, FAKE, None) == -1
    assert merge(FAKE, FAKE + 4, 2, 4, FAKE, None) == -1 and "align" in _err(csa2)
    assert merge(FAKE + 8, FAKE, 2, 4, FAKE, None) == -1
    assert merge(None, None, 3, 0, None, None) == 0


def test_quant_calls_reject_bad_arguments(csa2):
    assert csa2._quant_rows(FAKE, -1, FAKE, FAKE, None) == -2
    assert csa2._quant_rows(FAKE + 4, 3, FAKE, FAKE, None) == -1
    assert csa2._quant_rows(None, 0, None, None, None) == 0
    bad = csa2._FP4KV(FAKE, FAKE, 0, 1)
    assert csa2._quant_append(FAKE, bad, FAKE, None, None) == -2


def test_scheduler_rejects_invalid_tables(csa2):
    L = csa2.Layer
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.Sched([L(csa2.REUSE)], n_seq=1, key_cap=100)
    assert e.value.code == -4
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.Sched([L(csa2.REINDEX)], n_seq=1, key_cap=100)
    assert e.value.code == -4
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.Sched([L(csa2.FULL), L(7)], n_seq=1, key_cap=100)
    assert e.value.code == -4
    with pytest.raises(csa2.Csa2Error) as e:  # flat selection over too many positions
        csa2.Sched([L(csa2.FULL)], n_seq=1, key_cap=(1 << 20) + 1)
    assert e.value.code == -2
    with pytest.raises(csa2.Csa2Error) as e:  # hierarchical: blocks must cover key_cap
        csa2.Sched([L(csa2.FULL, 0, True)], n_seq=1, key_cap=1 << 20, blk_cap=1000)
    assert e.value.code == -2


def _prefill_desc(csa2, layers=None, **kw):
    layers = layers or [csa2.Layer(csa2.FULL)] + [csa2.Layer(csa2.REUSE)] * 5
    arr = (csa2._Layer * len(layers))(*[csa2._Layer(l.mode, l.kv_id, int(l.hierarchical)) for l in layers])
    a = dict(n_entries=65536, ratio=2, n_q=4096, t0=131072 - 4096, topk=512, swa=128)
    a.update(kw)
    d = csa2._PrefillDesc(len(layers), ctypes.cast(arr, ctypes.c_void_p), a["n_entries"], a["ratio"], a["n_q"],
                          a["t0"], a["topk"], a["swa"], 512 ** -0.5)
    d._keep = arr
    return d


def test_prefill_workspace_and_table_validation(csa2):
    ws = lambda d: csa2._prefill_ws(ctypes.byref(d))
    full = ws(_prefill_desc(csa2))
    assert full >= 4096 * 65536 * 4          # the score matrix dominates
    assert ws(_prefill_desc(csa2, t0=126)) == 0 and "t0" in _err(csa2)
    assert ws(_prefill_desc(csa2, t0=127)) > 0
    assert ws(_prefill_desc(csa2, n_q=0)) == 0
    assert ws(_prefill_desc(csa2, n_entries=2_000_000)) == 0
    assert ws(_prefill_desc(csa2, layers=[csa2.Layer(csa2.REUSE)])) == 0 and "Reuse" in _err(csa2)
    assert ws(_prefill_desc(csa2, layers=[csa2.Layer(csa2.FULL, 0, True)])) == 0 and "hierarchical" in _err(csa2)
    assert ws(_prefill_desc(csa2, layers=[csa2.Layer(csa2.FULL), csa2.Layer(csa2.REINDEX)])) == full


def test_prefill_calls_reject_bad_arguments(csa2):
    assert csa2._prefill_score(FAKE, None, FAKE, 100, 0, 2, 10, FAKE, None, None) == -1      # n_vis null
    assert csa2._prefill_score(FAKE + 2, None, FAKE, 100, 0, 2, 10, FAKE, FAKE, None) == -1  # alignment
    assert csa2._prefill_score(FAKE, None, FAKE, 100, 0, 0, 10, FAKE, FAKE, None) == -1      # ratio 0
    assert csa2._prefill_score(None, None, None, 100, 0, 2, 0, None, None, None) == 0        # n_q = 0: no-op
    assert csa2._prefill_score(FAKE, None, FAKE, (1 << 30) + 1, 0, 2, 10, FAKE, FAKE, None) == -2  # entries
    d = _prefill_desc(csa2, n_entries=1000, n_q=16, t0=1984)
    need = csa2._prefill_ws(ctypes.byref(d))
    io = csa2._PrefillIO()
    assert csa2._prefill_chunk(ctypes.byref(d), ctypes.byref(io), FAKE, need - 1, None) == -3
    assert csa2._prefill_chunk(ctypes.byref(d), ctypes.byref(io), FAKE + 16, need, None) == -1
    assert csa2._prefill_chunk(ctypes.byref(d), ctypes.byref(io), FAKE, need, None) == -1    # io pointers null


def test_prefill_select_rejects_bad_arguments(csa2):
    need = csa2.prefill_select_workspace_size(65536, 4096, 512)
    # filtered shape: candidate lists (2 KiB per query and 512 entries) on top of the scores
    assert need >= 4096 * 65536 * 4 + 4096 * 128 * 256 * 8
    # outside the filtered shapes (too few queries, k > 512) no lists are carved
    assert csa2.prefill_select_workspace_size(65536, 255, 512) < 255 * 65536 * 4 + 255 * 128 * 256 * 8
    assert csa2.prefill_select_workspace_size(65536, 4096, 1024) < need
    with pytest.raises(csa2.Csa2Error):
        csa2.prefill_select_workspace_size(65536, 0, 512)
    with pytest.raises(csa2.Csa2Error):
        csa2.prefill_select_workspace_size(65536, 16, 4096)

    def call(q=FAKE, keys=FAKE, n_entries=1000, t0=0, ratio=2, n_q=16, k=512, idx=FAKE, n_vis=FAKE, ws=FAKE * 16,
             ws_bytes=1 << 30):
        return csa2._prefill_select(q, None, keys, n_entries, t0, ratio, n_q, k, idx, n_vis, ws, ws_bytes, None)

    assert call(n_q=0) == -2 and call(n_q=65536) == -2
    assert call(k=0) == -2 and call(k=4096) == -2 and call(n_entries=(1 << 20) + 1) == -2
    assert call(ratio=0) == -1 and call(t0=-1) == -1
    assert call(idx=None) == -1 and call(n_vis=None) == -1 and call(ws=None) == -1
    assert call(q=FAKE + 2) == -1 and "aligned" in _err(csa2)
    assert call(ws=FAKE * 16 + 16) == -1
    assert call(ws_bytes=csa2.prefill_select_workspace_size(1000, 16, 512) - 1) == -3


def test_key_maintenance_rejects_bad_arguments(csa2):
    assert csa2._block_keys(FAKE, 100, FAKE, 8, FAKE, 12, 1, None) == -2        # 12 * 8 < 100
    assert csa2._block_keys(None, 100, FAKE, 8, FAKE, 13, 1, None) == -1
    assert csa2._block_keys(None, 100, None, 8, None, 13, 0, None) == 0        # n_seq = 0: no-op
    assert csa2._append_keys(FAKE, FAKE, 0, None, 0, 8, FAKE, None, 1, None) == -2
    assert csa2._append_keys(FAKE, FAKE, 100, FAKE, 0, 8, FAKE, None, 1, None) == -2
    assert csa2._append_keys(None, FAKE, 100, None, 0, 8, FAKE, None, 1, None) == -1


def test_flat_select_rejects_bad_arguments(csa2):
    def call(q=FAKE, keys=FAKE, key_cap=1000, lens=FAKE, k=512, out=FAKE, ws=FAKE * 16, ws_bytes=1 << 30, n_seq=1):
        return csa2._flat_select(q, None, keys, key_cap, lens, k, out, ws, ws_bytes, n_seq, None)

    assert call(n_seq=0, q=None) == 0
    assert call(q=None) == -1 and "null" in _err(csa2)
    assert call(key_cap=0) == -2 and call(key_cap=(1 << 20) + 1) == -2
    assert call(k=0) == -2 and call(k=4096) == -2
    assert call(ws=FAKE * 16 + 16) == -1 and "alignment" in _err(csa2)
    assert call(ws_bytes=csa2.flat_select_workspace_size(1000, 512, 1) - 1) == -3
    assert csa2.flat_select_workspace_size(0, 512, 1) == 0
    assert csa2.flat_select_workspace_size(1000, 0, 1) == 0
    # long inputs keep per-workgroup candidates instead of every score
    assert csa2.flat_select_workspace_size(1 << 19, 512, 1) < csa2.flat_select_workspace_size(1 << 19, 2048, 1)
