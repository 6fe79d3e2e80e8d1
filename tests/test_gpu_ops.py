"""GPU parity of each C-ABI operation against the CPU oracle.

Quantised bytes, scores (integer-valued inputs), selected indices and pool
blocks must match bit-exactly; attention must be within rel. L2 1e-3 and max
abs 5e-3 per (query, head) in fp32.  Both sides read the same seeded inputs
from ``synth``; neither side's output feeds the other.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (SEED, SM_SCALE, assert_attention_close, dev, host_u16, kv_source, print_case)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_kv_cache_quant_amd as m
    return m


def _bf16_of(x):
    return synth._f32_to_bf16_rne(np.asarray(x, np.float32))


# ---------------------------------------------------------------- step (a)
def test_quant_rows_exhaustive_bit_exact(csa2):
    """Every (bf16 magnitude, scale) pair the quantiser can meet, both signs,
    and every bf16 magnitude as a group's amax: bytes equal the oracle's."""
    from quant_sweep import sweep

    src, _, _ = sweep()
    print_case(f"quant_rows exhaustive rows={len(src)}")
    n = len(src)
    codes = torch.zeros(n, 256, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(n, 32, dtype=torch.uint8, device="cuda")
    csa2.quant_rows(dev(src), codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_rows(src)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_rows_normal_and_edge_rows(csa2):
    src = kv_source(0, 1, 3000)[0]
    edge = np.zeros((6, 512), np.uint16)
    edge[1] = 0x8000                                  # -0 everywhere
    edge[2] = 0x7F7F                                  # largest finite bf16
    edge[3, ::2], edge[3, 1::2] = 0x0001, 0x8001      # smallest subnormals
    edge[4] = _bf16_of(np.tile([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25], 64))  # exact midpoints
    edge[5] = _bf16_of(np.linspace(-448 * 6, 448 * 6, 512))
    src = np.concatenate([src, edge])
    print_case(f"quant_rows normal+edge rows={len(src)}")
    codes = torch.zeros(len(src), 256, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(len(src), 32, dtype=torch.uint8, device="cuda")
    csa2.quant_rows(dev(src), codes, scales)
    rc, rs = oracle.quant_rows(src)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_append_writes_row_lens_and_capacity_flag(csa2):
    n_seq, cap = 3, 5
    print_case("quant_append cap=5")
    kv = csa2.FP4KV.empty(n_seq, cap)
    lens = torch.tensor([0, 4, 5], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    src = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_NEW_ROW), synth.NORMAL, range(n_seq), [0], 512)[:, 0]
    csa2.quant_append(dev(src), kv, lens, err)
    assert lens.cpu().tolist() == [1, 5, 5] and err.item() == 1
    rc, rs = oracle.quant_rows(src)
    codes, scales = kv.codes.cpu().numpy(), kv.scales.cpu().numpy()
    assert np.array_equal(codes[0, 0], rc[0]) and np.array_equal(scales[0, 0], rs[0])
    assert np.array_equal(codes[1, 4], rc[1]) and np.array_equal(scales[1, 4], rs[1])
    assert not codes[2].any() and not codes[0, 1:].any() and not codes[1, :4].any()


# ---------------------------------------------------------------- step (b)
def _int_keys(tid, n_seq, n_rows, seed=SEED):
    return synth.gen_rows(seed, tid, synth.INT9, range(n_seq), np.arange(n_rows), 64)


@pytest.mark.parametrize("weights", [None, "int", "dyadic"])
def test_index_score_flat_exact(csa2, weights):
    n_seq, key_cap = 3, 5000
    lens = np.array([4096, 1, 4999], np.int32)
    keys = _int_keys(synth.tensor_id(synth.KIND_IDX_K), n_seq, key_cap)
    q = _int_keys(synth.tensor_id(synth.KIND_IDX_Q), n_seq, 8)
    w = None
    if weights == "int":
        w = np.array([[1, 2, 0, 3, 1, 1, 4, 2]] * n_seq, np.float32)
    elif weights == "dyadic":
        # fractional and negative weights whose products and partial sums are
        # exact in binary32, so that any summation order gives the same score
        w = (np.random.default_rng(7).integers(-16, 17, size=(n_seq, 8)) / 8).astype(np.float32)
    print_case(f"index_score flat weights={weights}")
    scores = torch.empty(n_seq, key_cap, dtype=torch.float32, device="cuda")
    csa2.index_score(dev(q), dev(keys), dev(lens), scores, w=None if w is None else dev(w))
    got = scores.cpu().numpy()
    for b in range(n_seq):
        ref = oracle.index_score(q[b], keys[b], np.arange(lens[b]), w=None if w is None else w[b])
        assert np.array_equal(got[b, :lens[b]], ref)
        assert np.all(got[b, lens[b]:] == -np.inf)


def test_index_score_blocks_len_div_and_pool_mode(csa2):
    n_seq, key_cap, blk = 2, 4000, 8
    lens = np.array([3999, 1234], np.int32)
    keys = _int_keys(synth.tensor_id(synth.KIND_IDX_K), n_seq, key_cap)
    bkeys = _int_keys(synth.tensor_id(synth.KIND_BLK_K), n_seq, 500)
    q = _int_keys(synth.tensor_id(synth.KIND_IDX_Q), n_seq, 8)
    print_case("index_score blocks + pool")
    bs = torch.empty(n_seq, 500, dtype=torch.float32, device="cuda")
    csa2.index_score(dev(q), dev(bkeys), dev(lens), bs, len_div=blk)
    got = bs.cpu().numpy()
    for b in range(n_seq):
        nb = (lens[b] + 7) // 8
        assert np.array_equal(got[b, :nb], oracle.index_score(q[b], bkeys[b], np.arange(nb)))
        assert np.all(got[b, nb:] == -np.inf)
    rng = np.random.default_rng(3)
    pool = np.full((n_seq, 64), -1, np.int32)
    pool[0, :60] = np.sort(rng.choice(500, 60, replace=False))
    pool[1, :64] = np.sort(rng.choice(160, 64, replace=False))  # some blocks beyond lens[1]
    ps = torch.empty(n_seq, 64 * blk, dtype=torch.float32, device="cuda")
    csa2.index_score(dev(q), dev(keys), dev(lens), ps, pool=dev(pool), blk=blk)
    got = ps.cpu().numpy()
    for b in range(n_seq):
        for p in range(64 * blk):
            blkid = pool[b, p // blk]
            pos = blkid * blk + p % blk
            if blkid < 0 or pos >= lens[b]:
                assert got[b, p] == -np.inf
            else:
                assert got[b, p] == oracle.index_score(q[b], keys[b], [pos])[0]


# ---------------------------------------------------------------- step (c)
@pytest.mark.parametrize("n,k,levels,L", [
    (4096, 512, 9000, 4096), (4096, 512, 3, 4096), (65537, 512, 50, 65537), (131073, 2048, 400, 131073),
    (131085, 2048, 10 ** 6, 131073), (300, 512, 4, 300), (5000, 512, 1, 5000), (5000, 512, 2, 1),
    (20000, 512, 1, 19999), (262144, 2048, 7, 262144),
    # past 262,144 slots the selection and tie bitmaps live in global memory
    (262145, 512, 3, 262145), (524288, 2048, 13, 524288), (700001, 2048, 2, 650000),
    (1048576, 512, 10 ** 6, 1048576 - 5)])
def test_topk_matches_oracle(csa2, n, k, levels, L):
    n_seq = 2
    rng = np.random.default_rng(n + k + levels)
    sc = rng.integers(0, levels, size=(n_seq, n)).astype(np.float32)
    sc[1, ::97] = -np.inf                      # some non-candidates
    lens = np.array([L, max(1, L // 2)], np.int32)
    print_case(f"topk n={n} k={k} levels={levels} L={L}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out, lens=dev(lens))
    got = out.cpu().numpy()
    for b in range(n_seq):
        nv = min(n, lens[b])
        ref = oracle.select(sc[b, :nv], np.arange(nv), k)
        assert np.array_equal(got[b], ref), b


def test_topk_workspace_reused_across_calls(csa2):
    """One workspace, several calls of different lengths and paths: the
    histogram and counters the calls leave behind must be zero."""
    rng = np.random.default_rng(21)
    n_seq = 3
    n_max = 70000
    ws = torch.zeros(csa2.topk_workspace_size(n_max, n_seq), dtype=torch.uint8, device="cuda")
    print_case("topk shared workspace")
    for n, k, levels in [(70000, 2048, 300), (5000, 512, 40), (70000, 512, 2), (1000, 512, 3)]:
        sc = rng.integers(0, levels, size=(n_seq, n)).astype(np.float32)
        out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
        csa2.topk(dev(sc), k, out, ws=ws[:csa2.topk_workspace_size(n, n_seq)])
        got = out.cpu().numpy()
        for b in range(n_seq):
            assert np.array_equal(got[b], oracle.select(sc[b], np.arange(n), k)), (n, k, b)


def test_topk_global_bitmaps_reused_across_calls(csa2):
    """Inputs longer than the LDS bitmaps: one workspace for calls of
    different lengths, the tie bitmap left clear for the next call."""
    rng = np.random.default_rng(23)
    n_seq, n_max = 2, 600000
    ws = torch.zeros(csa2.topk_workspace_size(n_max, n_seq), dtype=torch.uint8, device="cuda")
    print_case("topk global bitmaps, shared workspace")
    for n, k, levels in [(600000, 2048, 3), (600000, 512, 5000), (400000, 2048, 1), (100000, 512, 4)]:
        sc = rng.integers(0, levels, size=(n_seq, n)).astype(np.float32)
        out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
        csa2.topk(dev(sc), k, out, ws=ws[:csa2.topk_workspace_size(n, n_seq)])
        got = out.cpu().numpy()
        for b in range(n_seq):
            assert np.array_equal(got[b], oracle.select(sc[b], np.arange(n), k)), (n, k, b)


@pytest.mark.parametrize("n,k,cluster", [(131072, 512, 600), (524288, 512, 1000), (524288, 2048, 3000),
                                         (100000, 2048, 8000)])
def test_topk_threshold_bin_clustered_in_one_region(csa2, n, k, cluster):
    """The threshold bin's keys all sit in one filter workgroup's slots:
    more than that workgroup's share of the candidate buffer, so the final
    pass rescans the scores."""
    n_seq = 2
    rng = np.random.default_rng(n + cluster)
    sc = rng.integers(0, 100, size=(n_seq, n)).astype(np.float32)
    base = 9000 if n > 100000 else 50
    sc[0, base:base + cluster] = 1e6 + rng.integers(0, 1000, size=cluster)   # one top-digit bin
    sc[1, n - cluster:] = 1e6 + np.arange(cluster) % 7                        # heavy ties, last region
    print_case(f"topk clustered threshold bin n={n} k={k} cluster={cluster}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out)
    got = out.cpu().numpy()
    for b in range(n_seq):
        assert np.array_equal(got[b], oracle.select(sc[b], np.arange(n), k)), b


@pytest.mark.parametrize("n,k", [(65536, 512), (40000, 512), (65536, 2048)])
def test_topk_many_long_rows(csa2, n, k):
    """Many rows of more than 32,768 slots (a prefill chunk's queries): the
    threshold estimate taken by every filter workgroup of a row, candidates
    per workgroup region, then the selection per row -- with rows whose
    estimate holds (integer-valued and continuous scores), a row whose
    threshold bin overflows a region, rows too short to estimate, an empty
    row, NaN scores, an all-negative row, signed zeros and ragged lengths,
    all of which must equal the oracle."""
    n_seq = 300
    rng = np.random.default_rng(n + k)
    q = rng.integers(-4, 5, size=(8, 64))
    sc = np.empty((n_seq, n), np.float32)
    for b in range(n_seq):
        if b % 3 == 0:
            sc[b] = rng.standard_normal(n).astype(np.float32)
        else:
            keys = rng.integers(-4, 5, size=(n, 64))
            sc[b] = np.maximum(keys @ q.T, 0).sum(1).astype(np.float32)
    sc[7, :9000] = 1e5 + (np.arange(9000) % 3)        # 9,000 keys in one bin, in one region
    sc[8, :] = -np.inf                                  # no candidate
    sc[40, ::7] = np.nan                                # NaN is never a candidate
    sc[41] = -np.abs(sc[41]) - 1.0                      # all scores (and the threshold) negative
    sc[42] = -np.abs(sc[42]) - 1.0                      # the top scores: -0 and +0, which tie
    sc[42, ::5] = -0.0
    sc[42, 1::5] = 0.0
    lens = np.full(n_seq, n, np.int32)
    lens[9], lens[10], lens[11] = 3 * k, 1000, 4 * k + 5   # too short to estimate / just enough
    lens[12:40] = rng.integers(4 * k, n, size=28)
    print_case(f"topk many long rows n={n} k={k}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out, lens=dev(lens))
    got = out.cpu().numpy()
    for b in sorted({0, 1, 2, 7, 8, 9, 10, 11, 12, 13, 39, 40, 41, 42, 150, n_seq - 1}):
        nv = lens[b]
        ref = oracle.select(sc[b, :nv], np.arange(nv), k)
        assert np.array_equal(got[b], ref), b


@pytest.mark.parametrize("case", ["continuous", "wide_bin", "top_unsampled"])
def test_topk_sampled_first_pass_and_fallback(csa2, case):
    """Single-workgroup selection with its sampled first pass: continuous
    scores (the pass holds), 9,000 keys in the threshold's top-digit bin
    (too many to keep: the full passes run), and the top keys placed off
    the sampled slots."""
    n, k, n_seq = 60000, 512, 2
    rng = np.random.default_rng({"continuous": 1, "wide_bin": 2, "top_unsampled": 3}[case])
    if case == "continuous":
        sc = rng.standard_normal((n_seq, n)).astype(np.float32)
    elif case == "wide_bin":
        sc = rng.integers(0, 3, size=(n_seq, n)).astype(np.float32)
        sc[:, rng.choice(n, 9000, replace=False)] = 5.0 + rng.integers(0, 2, size=9000) * 0.25
    else:
        sc = rng.integers(0, 1000, size=(n_seq, n)).astype(np.float32)
        slots = np.arange(n)
        sampled = (slots % 1024) % 64 == slots // 1024     # slot = (t % 64) * 1024 + t
        top = rng.choice(slots[~sampled], 600, replace=False)
        sc[:, top] = 5000 + rng.integers(0, 50, size=600)
    print_case(f"topk sampled first pass {case}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out)
    got = out.cpu().numpy()
    for b in range(n_seq):
        assert np.array_equal(got[b], oracle.select(sc[b], np.arange(n), k)), b


@pytest.mark.parametrize("key_cap,k,lens,weights", [
    (5000, 512, (5000, 1234), False),           # scores in registers
    (300001, 512, (300001, 150000), False),     # per-workgroup candidates
    (300001, 512, (299999, 8192), True),
    (300001, 2048, (300001, 100), False),       # too many candidates: multi-workgroup passes
    (1 << 20, 512, (1 << 20, 700001), False),   # the largest input, 65,536 candidates
])
def test_flat_select_matches_oracle(csa2, key_cap, k, lens, weights):
    """Scoring + Top-k of a flat Full layer in one call against the oracle's
    flat selection (every position scored, ties to the lower position)."""
    n_seq = 2
    rng = np.random.default_rng(key_cap + k + int(weights))
    keys = _bf16_of(rng.integers(-4, 5, size=(n_seq, key_cap, 64)))
    q = _bf16_of(rng.integers(-4, 5, size=(n_seq, 8, 64)))
    w = (rng.integers(-2, 5, size=(n_seq, 8)) * 0.25).astype(np.float32) if weights else None
    L = np.array(lens, np.int32)
    print_case(f"flat_select key_cap={key_cap} k={k} lens={lens} weights={weights}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    ws = torch.zeros(csa2.flat_select_workspace_size(key_cap, k, n_seq), dtype=torch.uint8, device="cuda")
    for rep in range(2):  # the workspace is left ready for the next call
        out.fill_(-7)
        csa2.flat_select(dev(q), dev(keys), dev(L), k, out, w=dev(w) if weights else None, ws=ws)
        got = out.cpu().numpy()
        for b in range(n_seq):
            ref = oracle.flat_select(q[b], keys[b], int(L[b]), k, None if w is None else w[b])
            assert np.array_equal(got[b], ref), (rep, b)


def test_flat_select_many_sequences_per_workgroup_candidates(csa2):
    """64 sequences over 24,577 positions: four scoring workgroups each
    (the last holds one position), 256 in all, so the per-workgroup
    candidates path is taken below 65,536 positions.  Ragged lengths
    around the 8,192-position workgroup edges, fewer positions than k, and
    one position; every sequence against the oracle."""
    n_seq, key_cap, k = 64, 24577, 512
    rng = np.random.default_rng(23)
    keys = _bf16_of(rng.integers(-4, 5, size=(n_seq, key_cap, 64)))
    q = _bf16_of(rng.integers(-4, 5, size=(n_seq, 8, 64)))
    L = rng.integers(1, key_cap + 1, size=n_seq).astype(np.int32)
    L[:9] = [key_cap, 1, 511, 512, 513, 8192, 8193, 16384, 24576]
    print_case(f"flat_select n_seq={n_seq} key_cap={key_cap} k={k}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    ws = torch.zeros(csa2.flat_select_workspace_size(key_cap, k, n_seq), dtype=torch.uint8, device="cuda")
    csa2.flat_select(dev(q), dev(keys), dev(L), k, out, ws=ws)
    got = out.cpu().numpy()
    for b in range(n_seq):
        ref = oracle.flat_select(q[b], keys[b], int(L[b]), k)
        assert np.array_equal(got[b], ref), b


def test_topk_signed_scores_and_zero_signs(csa2):
    rng = np.random.default_rng(11)
    sc = rng.standard_normal((1, 10000)).astype(np.float32)
    sc[0, :3000:3] = 0.0
    sc[0, 1:3000:3] = -0.0
    sc[0, 5000:5100] = np.nan
    print_case("topk signed + zero signs")
    for k in (512, 2048, 7000 // 4):
        out = torch.empty(1, k, dtype=torch.int32, device="cuda")
        csa2.topk(dev(sc), k, out)
        ref = oracle.select(sc[0], np.arange(10000), k)
        assert np.array_equal(out.cpu().numpy()[0], ref)


def test_topk_pool_mapping(csa2):
    n_seq, n_pool, blk, k = 2, 2048, 8, 512
    rng = np.random.default_rng(5)
    pool = np.stack([np.sort(rng.choice(131073, n_pool, replace=False)) for _ in range(n_seq)]).astype(np.int32)
    pool[1, 2000:] = -1
    sc = rng.integers(0, 30, size=(n_seq, n_pool * blk)).astype(np.float32)
    sc[1, 2000 * blk:] = -np.inf
    print_case("topk pool mapping")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out, pool=dev(pool), blk=blk)
    got = out.cpu().numpy()
    for b in range(n_seq):
        ids = (pool[b][:, None].astype(np.int64) * blk + np.arange(blk)).ravel()
        assert np.all(sc[b][np.repeat(pool[b], blk) < 0] == -np.inf)  # empty blocks hold no candidate
        assert np.array_equal(got[b], oracle.select(sc[b], ids, k))


# ------------------------------------------------------------ steps (d)+(e)
def _device_cache(csa2, src):
    """Quantise bf16 sources [n_seq][cap][512] on the device."""
    n_seq, cap, _ = src.shape
    kv = csa2.FP4KV.empty(n_seq, cap)
    csa2.quant_rows(dev(src.reshape(-1, 512)), kv.codes, kv.scales)
    return kv


@pytest.mark.parametrize("k_idx,swa_lens", [(512, [128, 5, 0]), (512, [0, 0, 1]), (100, [128, 128, 7]),
                                            (0, [128, 3, 64]), (2000, [128, 0, 20])])
def test_sparse_attn_matches_oracle(csa2, k_idx, swa_lens):
    n_q, cap = 3, 2500
    src = kv_source(0, n_q, cap)
    kv = _device_cache(csa2, src)
    rng = np.random.default_rng(k_idx + sum(swa_lens))
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32) \
        if k_idx else np.zeros((n_q, 0), np.int32)
    if k_idx:
        idx[1, k_idx // 2:] = -1              # padded selection
        idx[2, :3] = idx[2, 3]                # duplicates attend twice
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA), synth.NORMAL, range(n_q), np.arange(128), 512)
    swa_len = np.array(swa_lens, np.int32)
    swa_dev = swa.copy()
    for b in range(n_q):
        swa_dev[b, swa_len[b]:] = 0x7FC0       # rows past the window hold NaN: never used
    print_case(f"sparse_attn k_idx={k_idx} swa={swa_lens}")
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx) if k_idx else None, dev(swa_dev), dev(swa_len), SM_SCALE, out)
    got = out.cpu().numpy()
    for b in range(n_q):
        codes, scales = oracle.quant_rows(src[b])
        ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa[b], swa_len[b], SM_SCALE)
        if k_idx == 0 and swa_len[b] == 0:
            assert np.all(got[b] == 0)
        else:
            assert_attention_close(got[b], ref, f"query {b}")


def test_sparse_attn_all_positions_is_dense(csa2):
    cap = 400
    src = kv_source(1, 1, cap)
    kv = _device_cache(csa2, src)
    idx = np.arange(512, dtype=np.int32)[None]
    idx[0, cap:] = -1
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 1), synth.NORMAL, [0], np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 1), synth.NORMAL, [0], np.arange(128), 512)
    print_case("sparse_attn dense")
    out = torch.empty(1, 16, 512, dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa), dev(np.array([128], np.int32)), SM_SCALE, out)
    codes, scales = oracle.quant_rows(src[0])
    x = np.stack([oracle.dequant_row(codes[i], scales[i]) for i in range(cap)]
                 + [synth.bf16_to_f32(r).astype(np.float64) for r in swa[0]])
    qf = synth.bf16_to_f32(q[0]).astype(np.float64)
    z = SM_SCALE * qf @ x.T
    p = np.exp(z - z.max(axis=1, keepdims=True))
    ref = (p / p.sum(axis=1, keepdims=True)) @ x
    assert_attention_close(out.cpu().numpy()[0], ref, "dense")


def test_device_generator_matches_host_generator(csa2):
    print_case("synth device fill")
    for kind in (synth.INT9, synth.NORMAL):
        t = torch.empty(3, 100, 64, dtype=torch.int16, device="cuda")
        synth.fill_rows_device(t, 5, 77, kind, b0=2, row0=1000)
        assert np.array_equal(host_u16(t), synth.gen_rows(5, 77, kind, [2, 3, 4], np.arange(1000, 1100), 64))


def test_sparse_attn_workspace_reused_across_calls(csa2):
    n_q, cap = 2, 600
    src = kv_source(2, n_q, cap)
    kv = _device_cache(csa2, src)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 2), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 2), synth.NORMAL, range(n_q), np.arange(128), 512)
    ws = torch.zeros(csa2.sparse_attn_workspace_size(n_q, 512, 128), dtype=torch.uint8, device="cuda")
    print_case("sparse_attn shared workspace")
    outs = []
    for rep in range(3):
        idx = np.stack([np.sort(np.random.default_rng(rep * 10 + b).choice(cap, 512, replace=False))
                        for b in range(n_q)]).astype(np.int32)
        out = torch.empty(n_q, 16, 512, dtype=torch.float32, device="cuda")
        csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa), dev(np.array([128, 77], np.int32)), SM_SCALE, out, ws=ws)
        outs.append((idx, out.cpu().numpy()))
    for idx, got in outs:
        for b in range(n_q):
            codes, scales = oracle.quant_rows(src[b])
            ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa[b], [128, 77][b], SM_SCALE)
            assert_attention_close(got[b], ref)


def test_sparse_attn_split_shapes_share_a_workspace(csa2):
    """Few queries split over several workgroups whose partials are merged
    with log-sum-exp weights: 1, 2, 13, 16 and 64 queries at 5, 17 and 33
    splits (k_idx 512, 2,000 and 4,000).  All calls share one workspace, in
    an order that moves between shapes, so that a call whose partials sit
    where another shape's did still reads only its own; padded selections
    and ragged window lengths; every output against the oracle."""
    cap = 4200
    n_max = 64
    src = kv_source(4, n_max, cap)
    kv = _device_cache(csa2, src)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 4), synth.NORMAL, range(n_max), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 4), synth.NORMAL, range(n_max), np.arange(128), 512)
    cases = [(16, 512), (13, 512), (64, 512), (16, 512), (2, 2000), (1, 4000), (1, 512), (16, 512)]
    need = max(csa2.sparse_attn_workspace_size(n, k, 128) for n, k in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    oracle_rows = {}
    for i, (n_q, k_idx) in enumerate(cases):
        rng = np.random.default_rng(100 + i)
        idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
        if n_q > 3:
            idx[3, k_idx // 3:] = -1
        swa_len = rng.integers(0, 129, n_q).astype(np.int32)
        swa_len[0] = 128
        print_case(f"sparse_attn split merge case {i}: n_q={n_q} k_idx={k_idx}")
        out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
        csa2.sparse_attn(dev(q[:n_q]), kv, dev(idx), dev(swa[:n_q]), dev(swa_len), SM_SCALE, out, ws=ws)
        got = out.cpu().numpy()
        assert not np.isnan(got).any(), f"case {i}: NaN output"
        for b in range(n_q):
            if b not in oracle_rows:
                oracle_rows[b] = oracle.quant_rows(src[b])
            codes, scales = oracle_rows[b]
            ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa[b], swa_len[b], SM_SCALE)
            assert_attention_close(got[b], ref, f"case {i} query {b}")


@pytest.mark.parametrize("n_q", [300, 1100])
def test_sparse_attn_many_queries_one_cache(csa2, n_q):
    """Many queries over one cache sequence with per-query window offsets
    (the prefill layout): 300 queries run multi-chunk splits plus the
    combine; 1,100 run one 4-wavefront workgroup per query over all its
    chunks.  Ragged k_idx and window lengths; sampled queries vs the oracle."""
    cap, k_idx, swa_max = 3000, 500, 100
    src = kv_source(3, 1, cap)
    kv = _device_cache(csa2, src)
    rng = np.random.default_rng(n_q)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[5, 300:] = -1
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 3), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa_rows = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 3), synth.NORMAL, [0],
                              np.arange(n_q + swa_max - 1), 512)[0]
    swa_len = rng.integers(0, swa_max + 1, size=n_q).astype(np.int32)
    swa_len[0], swa_len[1] = swa_max, 0
    print_case(f"sparse_attn many queries n_q={n_q}")
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa_rows), dev(swa_len), SM_SCALE, out, q_per_seq=n_q,
                     swa_q_stride_rows=1, swa_max=swa_max)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    codes, scales = oracle.quant_rows(src[0])
    for b in sorted({0, 1, 5, n_q // 2, n_q - 1, *rng.integers(0, n_q, 6).tolist()}):
        ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa_rows[b:b + swa_max], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"query {b}")


def test_sparse_attn_many_queries_scales_around_single_f16_bound(csa2):
    """Many queries (two wavefronts each): a 32-row chunk of FP4 rows whose
    E4M3 scales are all <= 1.25 (|x| <= 7.5) takes P rounded once to f16,
    any other chunk P as f16 hi + lo.  The cache's rows are N(0,1) latents
    times 1 (scales below the bound), 2.5 (group maxima near 6 * 1.25:
    scales on both sides of it) or 4 (scales above it); queries select
    from one kind or from all, so that chunks of either form, and queries
    that mix them, occur.  Sampled queries vs the oracle at
    the attention bar (the single-f16 error bound, 2^-11 * 7.5 < 3.7e-3,
    is inside its 5e-3 absolute limit)."""
    n_q, cap, k_idx, swa_max = 1024, 4096, 512, 128
    base = kv_source(5, 1, cap)[0]
    kinds = np.arange(cap) * 3 // cap
    factor = np.array([1.0, 2.5, 4.0])[kinds][:, None]
    src = synth._f32_to_bf16_rne(synth.bf16_to_f32(base) * factor)[None]
    codes, scales = oracle.quant_rows(src[0])
    small = np.all(scales <= 0x3A, axis=1)  # E4M3 code 0x3A = 1.25
    assert small[kinds == 0].all() and not small[kinds == 2].any()
    assert 0 < small[kinds == 1].sum() < (kinds == 1).sum()
    kv = _device_cache(csa2, src)
    rng = np.random.default_rng(55)
    pools = [np.flatnonzero(kinds == i) for i in range(3)] + [np.arange(cap)]
    idx = np.empty((n_q, k_idx), np.int32)
    for b in range(n_q):
        idx[b] = np.sort(rng.choice(pools[b % 4], k_idx, replace=False))
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 5), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa_rows = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 5), synth.NORMAL, [0],
                              np.arange(n_q + swa_max - 1), 512)[0]
    swa_len = rng.integers(0, swa_max + 1, size=n_q).astype(np.int32)
    swa_len[:3] = swa_max
    print_case("sparse_attn many queries, scales around the single-f16 bound")
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa_rows), dev(swa_len), SM_SCALE, out, q_per_seq=n_q,
                     swa_q_stride_rows=1, swa_max=swa_max)
    got = out.cpu().numpy()
    for b in sorted({0, 1, 2, 3, 4, 5, 6, 7, n_q - 1, *rng.integers(0, n_q, 9).tolist()}):
        ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa_rows[b:b + swa_max], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"query {b}")


@pytest.mark.parametrize("where", ["window", "selected"])
def test_sparse_attn_many_queries_late_maximum(csa2, where):
    """Many queries (one wavefront each) where a row late in a query's order
    scores far above every earlier row (more than 2^15 in softmax weight):
    the last window row, or the last selected row, is a large multiple of
    the sign pattern of the query's head 0.  Sampled queries vs the oracle;
    the queries without the row check the ordinary path beside them."""
    cap, k_idx, swa_max, n_q = 3000, 512, 128, 1024
    src = kv_source(6, 1, cap)
    rng = np.random.default_rng(29)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 6), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa_rows = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 6), synth.NORMAL, [0],
                              np.arange(n_q + swa_max - 1), 512)[0]
    swa_len = np.full(n_q, swa_max, np.int32)
    hot = [0, 3, 700, n_q - 1]
    sign0 = np.where(synth.bf16_to_f32(q[hot[0], 0]) >= 0, 1.0, -1.0)
    if where == "window":
        for b in hot:                       # window row 127 of query b is swa_rows[b + 127]
            sgn = np.where(synth.bf16_to_f32(q[b, 0]) >= 0, 1.0, -1.0)
            swa_rows[b + swa_max - 1] = _bf16_of(4.0 * sgn)
    else:
        hot = [0]                           # one cache row, last in query 0's selection
        idx[0, -1] = cap - 1
        src[0, cap - 1] = _bf16_of(4.0 * sign0)
    kv = _device_cache(csa2, src)
    print_case(f"sparse_attn many queries, late maximum in the {where}")
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa_rows), dev(swa_len), SM_SCALE, out, q_per_seq=n_q,
                     swa_q_stride_rows=1, swa_max=swa_max)
    got = out.cpu().numpy()
    codes, scales = oracle.quant_rows(src[0])
    for b in sorted(set(hot) | {1, 2, 500}):
        ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa_rows[b:b + swa_max], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"query {b}")


# ------------------------------------------------------------- FP8 window
def test_quant_fp8_rows_all_bf16_patterns(csa2):
    """Every bf16 bit pattern (128 rows of 512) -> E4M3 codes, bit-exact with
    the oracle (ties to even, saturation, signed zeros, NaN)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(128, 512)
    print_case("quant_fp8_rows all bf16")
    dst = torch.empty(128, 512, dtype=torch.uint8, device="cuda")
    csa2.quant_fp8_rows(dev(bits), dst)
    assert np.array_equal(dst.cpu().numpy(), oracle.fp8_rows(bits))


@pytest.mark.parametrize("k_idx,swa_lens", [(512, [128, 77, 0]), (0, [128, 5, 1]), (300, [64, 128, 128])])
def test_sparse_attn_fp8_window_matches_oracle(csa2, k_idx, swa_lens):
    n_q, cap = 3, 2500
    src = kv_source(4, n_q, cap)
    kv = _device_cache(csa2, src)
    rng = np.random.default_rng(k_idx + 7 * sum(swa_lens))
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32) \
        if k_idx else np.zeros((n_q, 0), np.int32)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 4), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 4), synth.NORMAL, range(n_q), np.arange(128), 512)
    swa8 = np.stack([oracle.fp8_rows(swa[b]) for b in range(n_q)])
    swa_len = np.array(swa_lens, np.int32)
    swa8_dev = swa8.copy()
    for b in range(n_q):
        swa8_dev[b, swa_len[b]:] = 0x7F        # E4M3 NaN past the window: never used
    print_case(f"sparse_attn fp8 window k_idx={k_idx} swa={swa_lens}")
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx) if k_idx else None, torch.from_numpy(swa8_dev).cuda(), dev(swa_len),
                     SM_SCALE, out)
    got = out.cpu().numpy()
    for b in range(n_q):
        codes, scales = oracle.quant_rows(src[b])
        ref = oracle.sparse_attn_fp8w(q[b], codes, scales, idx[b], swa8[b], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"query {b}")


# ------------------------------------------------------------ edge cases
@pytest.mark.parametrize("n,k", [(1, 1), (2, 2048), (70000, 1), (3000, 2048), (40000, 2048)])
def test_topk_extreme_k_and_special_scores(csa2, n, k):
    """k = 1 and k = 2048, lengths below, inside and above the register
    path; NaN and -inf are not candidates, +inf is the largest score."""
    n_seq = 2
    rng = np.random.default_rng(n * 7 + k)
    sc = rng.integers(-3, 4, size=(n_seq, n)).astype(np.float32)
    sc[0, ::5] = np.nan
    sc[1, 1::7] = -np.inf
    sc[1, ::11] = np.inf
    print_case(f"topk extremes n={n} k={k}")
    out = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(dev(sc), k, out)
    got = out.cpu().numpy()
    for b in range(n_seq):
        ref = oracle.select(sc[b], np.arange(n), k)
        assert np.array_equal(got[b], ref), b


def test_zero_sized_calls_are_no_ops(csa2):
    """n_seq = 0 / n_q = 0 / n_rows = 0 enqueue nothing and succeed."""
    empty16 = torch.empty(0, dtype=torch.int16, device="cuda")
    csa2.quant_rows(empty16.view(0, 512), torch.empty(0, 256, dtype=torch.uint8, device="cuda"),
                    torch.empty(0, 32, dtype=torch.uint8, device="cuda"))
    csa2.quant_fp8_rows(empty16.view(0, 512), torch.empty(0, 512, dtype=torch.uint8, device="cuda"))
    assert csa2._topk(None, 100, None, 1, 512, None, 0, 8, None, None, 0, 0, None) == 0
    assert csa2._index_score(None, None, None, 100, None, 1, None, 0, 8, None, 50, 0, None) == 0
    torch.cuda.synchronize()


def test_sparse_attn_maximum_rows(csa2):
    """The largest attended set one call accepts: 8,064 selected rows + a
    128-row window = 8,192 rows (64 chunks, 64 split workgroups)."""
    n_q, cap, k_idx = 2, 9000, 8064
    src = kv_source(5, n_q, cap)
    kv = _device_cache(csa2, src)
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 5), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 5), synth.NORMAL, range(n_q), np.arange(128), 512)
    swa_len = np.array([128, 31], np.int32)
    print_case("sparse_attn 8,192 rows")
    out = torch.empty(n_q, 16, 512, dtype=torch.float32, device="cuda")
    csa2.sparse_attn(dev(q), kv, dev(idx), dev(swa), dev(swa_len), SM_SCALE, out)
    got = out.cpu().numpy()
    for b in range(n_q):
        codes, scales = oracle.quant_rows(src[b])
        ref = oracle.sparse_attn(q[b], codes, scales, idx[b], swa[b], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"query {b}")


def _f16_toward_zero(x):
    """bf16/f32 values as the attention kernel reads main Q and window rows:
    converted to f16 rounding toward zero, saturating at +-65504 (the
    documented contract of csa2_sparse_attn)."""
    x = np.clip(np.asarray(x, np.float64), -65504.0, 65504.0)
    y = x.astype(np.float16)                       # nearest even ...
    away = np.abs(y.astype(np.float64)) > np.abs(x)
    y[away] = np.nextafter(y[away], np.float16(0))  # ... stepped back toward zero
    return y.astype(np.float64)


def test_sparse_attn_f16_conversion_of_large_and_tiny_values(csa2):
    """Main Q and window values outside f16's normal range are neither
    rejected nor flagged: they are converted to f16 toward zero (saturating
    at 65504, subnormal below 2^-14), as csa2.h documents.  The output must
    match dense softmax attention over the converted values, and differ
    clearly from attention over the unconverted ones."""
    rng = np.random.default_rng(17)
    n_rows = 64
    x = rng.standard_normal((n_rows, 512)).astype(np.float32)
    x[:, 5] *= 1e-4
    x[10, 11], x[20, 12], x[30, 13], x[40, 14] = 1.0e5, -3.0e5, 1.0e-7, 3.0e-6
    q = rng.standard_normal((16, 512)).astype(np.float32)
    q[0, 5], q[1, 5] = 1.0e5, -7.0e4          # saturate
    q[2] = rng.standard_normal(512) * 1e-6     # f16 subnormals
    q[3, 11] = 3.0e-3                          # picks up window row 10's large value
    qb, xb = _bf16_of(q), _bf16_of(x)
    qv, xv = synth.bf16_to_f32(qb).astype(np.float64), synth.bf16_to_f32(xb).astype(np.float64)
    kv = csa2.FP4KV.empty(1, 16)
    print_case("sparse_attn f16 conversion of out-of-range values")
    out = torch.empty(1, 16, 512, dtype=torch.float32, device="cuda")
    idx = np.full((1, 16), -1, np.int32)       # window rows only
    swa = xb[None]
    csa2.sparse_attn(dev(qb[None]), kv, dev(idx), dev(swa), dev(np.array([n_rows], np.int32)), SM_SCALE, out)
    got = out.cpu().numpy()[0]

    def dense(qf, xf):
        z = SM_SCALE * qf @ xf.T
        p = np.exp(z - z.max(axis=1, keepdims=True))
        return (p / p.sum(axis=1, keepdims=True)) @ xf

    ref = dense(_f16_toward_zero(qv), _f16_toward_zero(xv))
    assert_attention_close(got, ref, "converted")
    raw = dense(qv, xv)
    rel = np.linalg.norm(raw - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel[[0, 1, 3]].min() > 1e-2, rel[:4]  # the conversion is visible in the heads that meet it


@pytest.mark.parametrize("case", ["full_pool", "ragged_pool", "short", "weights", "blk16", "ties"])
def test_pool_select_matches_oracle(csa2, case):
    """Scores + Top-k of a pool's positions in one call (csa2_pool_select)
    against the oracle's pool selection: a full 2,048-block pool, a pool
    with empty blocks and blocks past the sequence, fewer candidates than k,
    dyadic head weights, 16-position blocks (32,768 slots: the path without
    the bound), and integer keys of three values (ties everywhere)."""
    n_seq, k = 3, 512
    rng = np.random.default_rng(hash(case) % 1000)
    blk = 16 if case == "blk16" else 8
    key_cap = 8 * 20000 + 3
    lens = np.array([key_cap, key_cap - 7, 8 * 1500 + 5], np.int32)
    if case == "short":
        lens = np.array([300, 9, 4000], np.int32)
    lo, hi = (-1, 1) if case == "ties" else (-4, 4)
    keys = _bf16_of(rng.integers(lo, hi + 1, size=(n_seq, key_cap, 64)))
    q = _bf16_of(rng.integers(-4, 5, size=(n_seq, 8, 64)))
    w = (rng.integers(-16, 17, size=(n_seq, 8)) / 8).astype(np.float32) if case == "weights" else None
    n_pool = 2048
    pool = np.full((n_seq, n_pool), -1, np.int32)
    for b in range(n_seq):
        nb = -(-int(lens[b]) // blk)
        m = min(n_pool, nb + 40)                  # some blocks past the sequence's end
        cand = np.sort(rng.choice(max(nb + 40, m), m, replace=False))
        pool[b, :m] = cand
        if case == "ragged_pool":
            pool[b, m // 2:] = -1                 # empty blocks (the tail of the list)
            pool[b, :m // 2] = np.sort(rng.choice(nb, m // 2, replace=False))
    print_case(f"pool_select {case}")
    out = torch.full((n_seq, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(csa2.pool_select_workspace_size(n_pool, blk, n_seq), dtype=torch.uint8, device="cuda")
    for rep in range(2):  # the workspace is left ready for the next call
        csa2.pool_select(dev(q), dev(keys), dev(lens), dev(pool), k, out, blk=blk,
                         w=dev(w) if w is not None else None, ws=ws)
        got = out.cpu().numpy()
        for b in range(n_seq):
            ref = oracle.pool_select(q[b], keys[b], int(lens[b]), pool[b].astype(np.int64), k, blk,
                                     None if w is None else w[b])
            assert np.array_equal(got[b], ref), (case, rep, b)
