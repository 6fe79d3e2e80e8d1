"""The context-parallel split on one GPU: a rank's share of the attention
(csa2_sparse_attn_partial) and the merge of the shares (csa2_attn_merge)
against the oracle, and one selecting decode layer of a sequence sharded
over four ranks, the ranks emulated on one device (the exchange between
them, an all-gather over xGMI in a deployment, is a concatenation here)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import SEED, SM_SCALE, assert_attention_close, dev, kv_source, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_kv_cache_quant_amd as m
    return m


def _cache(csa2, src):
    n_seq, cap, _ = src.shape
    kv = csa2.FP4KV.empty(n_seq, cap)
    csa2.quant_rows(dev(src.reshape(-1, 512)), kv.codes, kv.scales)
    return kv


def _check_share(o, ml, ref_o, ref_ml, what):
    """A share against the oracle's: m to 1e-4 (base-2 units), l to 1e-4
    relative, o / l at the attention bar, and o itself per head to 1e-3
    relative L2."""
    m, l = ml[..., 0].astype(np.float64), ml[..., 1].astype(np.float64)
    rm, rl = ref_ml[..., 0], ref_ml[..., 1]
    empty = rm == -np.inf
    assert np.all(m[empty] == -np.inf) and np.all(l[empty] == 0) and np.all(o[empty] == 0), what
    assert np.all(np.abs(m[~empty] - rm[~empty]) <= 1e-4 * np.maximum(1, np.abs(rm[~empty]))), what
    assert np.all(np.abs(l[~empty] - rl[~empty]) <= 1e-4 * rl[~empty]), what
    if (~empty).any():
        assert_attention_close(o[~empty] / l[~empty][:, None], ref_o[~empty] / rl[~empty][:, None], what)
        err = np.linalg.norm(o[~empty] - ref_o[~empty], axis=1) / np.linalg.norm(ref_o[~empty], axis=1)
        assert err.max() <= 1e-3, what


@pytest.mark.parametrize("n_q,k_idx", [(3, 512), (16, 512), (16, 2000), (1100, 300)])
def test_share_matches_oracle(csa2, n_q, k_idx):
    """Shares at the split-K shapes (3 and 16 queries, merged by the combine
    kernel left unnormalised) and the one-workgroup-per-query shape (1,100
    queries over one cache, written in place); padded selections, ragged and
    empty windows, and one query with no row at all."""
    many = n_q >= 1024
    n_seq = 1 if many else n_q
    cap = 3000 if many else 2500
    src = kv_source(6, n_seq, cap)
    kv = _cache(csa2, src)
    rng = np.random.default_rng(n_q + k_idx)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[1, k_idx // 2:] = -1
    idx[2, :] = -1                          # query 2: no selected row ...
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 6), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa_max = 128
    if many:
        swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 6), synth.NORMAL, [0],
                             np.arange(n_q + swa_max - 1), 512)[0]
        stride, q_per_seq = 1, n_q
    else:
        swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 6), synth.NORMAL, range(n_q),
                             np.arange(swa_max), 512)
        stride, q_per_seq = swa_max, 1
    swa_len = rng.integers(0, swa_max + 1, size=n_q).astype(np.int32)
    swa_len[0], swa_len[2] = swa_max, 0     # ... and no window row
    print_case(f"sparse_attn_partial n_q={n_q} k_idx={k_idx}")
    out_o = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    out_ml = torch.full((n_q, 16, 2), float("nan"), dtype=torch.float32, device="cuda")
    csa2.sparse_attn_partial(dev(q), kv, dev(idx), dev(swa), dev(swa_len), SM_SCALE, out_o, out_ml,
                             q_per_seq=q_per_seq, swa_q_stride_rows=stride, swa_max=swa_max)
    o, ml = out_o.cpu().numpy(), out_ml.cpu().numpy()
    rows = {}
    sample = sorted({0, 1, 2, n_q - 1, *rng.integers(0, n_q, 4).tolist()})
    for b in sample:
        s = b // q_per_seq
        if s not in rows:
            rows[s] = oracle.quant_rows(src[s])
        codes, scales = rows[s]
        win = swa[b:b + swa_max] if many else swa[b]
        ref_o, ref_ml = oracle.sparse_attn_partial(q[b], codes, scales, idx[b], win, swa_len[b], SM_SCALE)
        _check_share(o[b], ml[b], ref_o, ref_ml, f"query {b}")


def test_merge_matches_oracle_merge(csa2):
    """csa2_attn_merge of three shares per query (from csa2_sparse_attn_partial
    over a random split of each query's rows, the window on one share, some
    shares empty) against the oracle's merge of the oracle's shares."""
    n_q, cap, k_idx = 8, 2000, 512
    src = kv_source(7, n_q, cap)
    kv = _cache(csa2, src)
    rng = np.random.default_rng(77)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    owner = rng.integers(0, 3, size=idx.shape)
    owner[0] = rng.integers(0, 2, size=k_idx)   # query 0: share 2 holds no selected row
    tail = rng.integers(0, 3, size=n_q)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 7), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 7), synth.NORMAL, range(n_q), np.arange(128), 512)
    parts_o = torch.empty(3, n_q, 16, 512, dtype=torch.float32, device="cuda")
    parts_ml = torch.empty(3, n_q, 16, 2, dtype=torch.float32, device="cuda")
    print_case("attn_merge of three shares")
    for s in range(3):
        idx_s = np.where(owner == s, idx, -1).astype(np.int32)
        swa_len = np.where(tail == s, 128, 0).astype(np.int32)
        csa2.sparse_attn_partial(dev(q), kv, dev(idx_s), dev(swa), dev(swa_len), SM_SCALE, parts_o[s], parts_ml[s])
    out = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.attn_merge(parts_o, parts_ml, out)
    got = out.cpu().numpy()
    for b in range(n_q):
        codes, scales = oracle.quant_rows(src[b])
        shares = [oracle.sparse_attn_partial(q[b], codes, scales, np.where(owner[b] == s, idx[b], -1), swa[b],
                                             128 if tail[b] == s else 0, SM_SCALE) for s in range(3)]
        ref = oracle.attn_merge(np.stack([o for o, _ in shares]), np.stack([m for _, m in shares]))
        assert_attention_close(got[b], ref, f"query {b}")
        assert_attention_close(got[b], oracle.sparse_attn(q[b], codes, scales, idx[b], swa[b], 128, SM_SCALE),
                               f"query {b} vs attention over all rows")


def test_decode_layer_sharded_over_four_ranks(csa2):
    """One Full layer of 4 sequences of 65,536 positions, sharded over 4
    ranks of 16,384 positions each.  Each rank: its flat Top-512 with global
    ids (csa2_flat_select on its shard) and their scores (csa2_index_score
    over those positions); the gathered 4 x 512 (score, id) pairs give the
    global Top-512 (csa2_topk with the ids as a pool of blocks of 1), which
    must equal the unsharded selection bit for bit; each rank's share over
    the selected rows it holds (the last rank also the window), merged,
    must match the unsharded attention and the oracle."""
    n_seq, G, Ls, k = 4, 4, 16384, 512
    L = G * Ls
    rng = np.random.default_rng(404)
    keys = synth._f32_to_bf16_rne(rng.integers(-4, 5, size=(n_seq, L, 64)).astype(np.float32))
    iq = synth._f32_to_bf16_rne(rng.integers(-4, 5, size=(n_seq, 8, 64)).astype(np.float32))
    src = kv_source(8, n_seq, L)
    kv = _cache(csa2, src)
    q = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_MAIN_Q, 8), synth.NORMAL, range(n_seq), np.arange(16), 512)
    swa = synth.gen_rows(SEED, synth.tensor_id(synth.KIND_SWA, 8), synth.NORMAL, range(n_seq), np.arange(128), 512)
    swa_len = np.array([128, 128, 77, 128], np.int32)
    keys_d, iq_d, q_d, swa_d, swa_len_d = dev(keys), dev(iq), dev(q), dev(swa), dev(swa_len)

    print_case("context-parallel layer: unsharded reference")
    idx_full = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.flat_select(iq_d, keys_d, dev(np.full(n_seq, L, np.int32)), k, idx_full)
    out_full = torch.empty(n_seq, 16, 512, dtype=torch.float32, device="cuda")
    csa2.sparse_attn(q_d, kv, idx_full, swa_d, swa_len_d, SM_SCALE, out_full)

    print_case("context-parallel layer: per-rank selection")
    lens_s = dev(np.full(n_seq, Ls, np.int32))
    cand_score = torch.empty(n_seq, G * k, dtype=torch.float32, device="cuda")
    cand_id = torch.empty(n_seq, G * k, dtype=torch.int32, device="cuda")
    for s in range(G):
        keys_s = keys_d[:, s * Ls:(s + 1) * Ls].contiguous()
        local = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
        csa2.flat_select(iq_d, keys_s, lens_s, k, local)
        sc = torch.empty(n_seq, k, dtype=torch.float32, device="cuda")
        csa2.index_score(iq_d, keys_s, lens_s, sc, pool=local, blk=1)
        cand_score[:, s * k:(s + 1) * k] = sc                     # the all-gather
        cand_id[:, s * k:(s + 1) * k] = torch.where(local >= 0, local + s * Ls, local)
    idx_cp = torch.empty(n_seq, k, dtype=torch.int32, device="cuda")
    csa2.topk(cand_score, k, idx_cp, pool=cand_id, blk=1)
    assert torch.equal(idx_cp, idx_full), "the sharded selection differs from the unsharded one"

    print_case("context-parallel layer: per-rank shares and the merge")
    parts_o = torch.empty(G, n_seq, 16, 512, dtype=torch.float32, device="cuda")
    parts_ml = torch.empty(G, n_seq, 16, 2, dtype=torch.float32, device="cuda")
    for s in range(G):
        kv_s = csa2.FP4KV(kv.codes[:, s * Ls:(s + 1) * Ls].contiguous(), kv.scales[:, s * Ls:(s + 1) * Ls].contiguous())
        mine = (idx_cp >= s * Ls) & (idx_cp < (s + 1) * Ls)
        idx_s = torch.where(mine, idx_cp - s * Ls, torch.full_like(idx_cp, -1))
        if s == G - 1:  # the rank with the tail holds the window
            csa2.sparse_attn_partial(q_d, kv_s, idx_s, swa_d, swa_len_d, SM_SCALE, parts_o[s], parts_ml[s])
        else:
            csa2.sparse_attn_partial(q_d, kv_s, idx_s, None, swa_len_d, SM_SCALE, parts_o[s], parts_ml[s],
                                     swa_max=0)
    out_cp = torch.full((n_seq, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
    csa2.attn_merge(parts_o, parts_ml, out_cp)
    got, full = out_cp.cpu().numpy(), out_full.cpu().numpy()
    idx_h = idx_cp.cpu().numpy()
    for b in range(n_seq):
        assert_attention_close(got[b], full[b], f"sequence {b} vs unsharded")
    for b in (0, n_seq - 1):
        assert np.array_equal(idx_h[b], oracle.flat_select(iq[b], keys[b], L, k))
        codes, scales = oracle.quant_rows(src[b])
        ref = oracle.sparse_attn(q[b], codes, scales, idx_h[b], swa[b], swa_len[b], SM_SCALE)
        assert_attention_close(got[b], ref, f"sequence {b} vs oracle")
