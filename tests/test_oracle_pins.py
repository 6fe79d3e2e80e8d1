"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test checks one oracle function against a worked example stored under
tests/golden/, a library routine (torch's E4M3FN cast, numpy sorting and
matmul, torch float64 attention), a closed form, or an invariant of the
method -- chosen so that a dropped term, a wrong sign or index, a swapped
operand or a wrong tie rule in the oracle fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def f32_to_bf16(x):
    return synth._f32_to_bf16_rne(np.asarray(x, np.float32))


# ------------------------------------------------------------------ formats
def test_e2m1_grid_matches_golden():
    for code, val in _golden_lines("e2m1_grid.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code


def test_e4m3_landmarks_match_golden():
    for code, val in _golden_lines("e4m3fn_points.txt"):
        got = oracle.e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert Fraction(got) == Fraction(val), code
            if val.startswith("-"):
                assert math.copysign(1, got) < 0


def test_e4m3_all_codes_match_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_positive_values_strictly_increase():
    v = [oracle.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(v, v[1:]))
    assert v[-1] == 448.0 and v[0] == 0.0


def test_e2m1_rne_at_unit_scale_golden():
    for x, code in _golden_lines("e2m1_rne_unit_scale.txt"):
        assert oracle.e2m1_code(float(x), 0, 1.0) == int(code), x
        assert oracle.e2m1_code(float(x), 1, 1.0) == int(code) | 8, x


def _all_positive_finite_bf16():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    return bits, synth.bf16_to_f32(bits).astype(np.float64)


def test_scale_code_all_bf16_amax_vs_torch_cast():
    """Every non-negative finite bf16 amax: E4M3 RNE of amax/6 equals torch's
    float -> float8_e4m3fn cast (round-to-nearest-even) wherever that cast does
    not overflow; above 464 (half-way past 448) the oracle saturates at 448."""
    bits, a = _all_positive_finite_bf16()
    got = np.array([oracle.scale_code(x) for x in a], dtype=np.uint8)
    q = a / 6.0
    fits = q < 464.0
    ref = torch.from_numpy(q[fits]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[fits], ref)
    assert np.all(got[~fits] == 0x7E)


def test_scale_code_exact_rational_sample():
    """Exact-rational nearest-even by bisection over the E4M3 values built as
    Fractions from the landmarks' rule, on a stratified sample incl. all ties."""
    vals = sorted({Fraction(oracle.e4m3_value(c)) for c in range(127)})
    assert len(vals) == 127
    samples = []
    for i in range(126):  # exact midpoints (ties) and neighbours, times 6
        mid = (vals[i] + vals[i + 1]) / 2
        samples += [6 * mid, 6 * vals[i], 6 * mid * Fraction(1023, 1024), 6 * mid * Fraction(1025, 1024)]
    import bisect
    for a in samples:
        af = float(a)
        if Fraction(af) != a:  # only values exact in double
            continue
        t = a / 6
        j = bisect.bisect_left(vals, t)
        if j == len(vals):
            want = 126
        elif vals[j] == t or j == 0:
            want = j
        else:
            lo, hi = vals[j - 1], vals[j]
            want = (j - 1) if (t - lo < hi - t or (t - lo == hi - t and (j - 1) % 2 == 0)) else j
        assert oracle.scale_code(af) == want, a


def test_element_codes_all_bf16_times_all_scales():
    """All finite bf16 magnitudes x all 126 nonzero E4M3 scales: the oracle's
    E2M1 code equals an independent float64 computation (the quotient x/s is
    correctly rounded, and it is exactly a grid midpoint iff x is) followed
    by numpy's half-to-even rounding on each uniform stretch of the grid."""
    _, x = _all_positive_finite_bf16()
    # all 32,640 magnitudes x 126 scales (unreachable pairs included: x > 6.375 s saturates)
    lib = oracle.lib()
    for sc in range(1, 127):
        s = oracle.e4m3_value(sc)
        r = x / s
        ref = np.where(r < 2.0, np.round(2 * r),                   # 0, .5, 1, 1.5 -> codes 0..3 (+2.0 -> 4)
              np.where(r < 4.0, np.round(r) + 2,                  # 2, 3, 4 -> codes 4..6
              np.where(r <= 6.0, np.round(r / 2) + 4, 7)))        # 4, 6 -> codes 6, 7; saturate
        ref = np.minimum(ref, 7).astype(np.int64)
        got = np.array([lib.orc_e2m1_code(v, 0, s) for v in x], dtype=np.int64)
        assert np.array_equal(got, ref), sc


def test_quant_rows_exhaustive_sweep():
    """Every (bf16 magnitude, scale) pair the quantiser can meet, in both
    signs, and every bf16 magnitude as a group's amax (tests/quant_sweep.py:
    expected codes from numpy float64 and torch's E4M3 cast): the oracle's
    quantised bytes equal them all."""
    from quant_sweep import sweep

    rows, codes, scales = sweep()
    rc, rs = oracle.quant_rows(rows)
    assert np.array_equal(rs, scales)
    assert np.array_equal(rc, codes)


def test_quant_row_worked_example():
    lines = open(os.path.join(GOLDEN, "quant_row_worked.txt")).read().splitlines()
    row = np.zeros(512, np.float32)
    want_scale = np.zeros(32, np.uint8)
    want_codes = np.zeros(256, np.uint8)
    for l in lines:
        if l.startswith("#") or not l.strip():
            continue
        head, rest = l.split(":")
        g = int(head.split()[1])
        kind = head.split()[2]
        vals = rest.split()
        if kind == "values":
            row[16 * g:16 * g + 16] = [float(v) for v in vals]
        elif kind == "scale":
            want_scale[g] = int(vals[0], 16)
        else:
            want_codes[8 * g:8 * g + 8] = [int(v, 16) for v in vals]
    bits = f32_to_bf16(row)
    bits[15] = 0x8000  # -0 in group 0
    codes, scales = oracle.quant_rows(bits)
    assert np.array_equal(scales[0], want_scale)
    assert np.array_equal(codes[0], want_codes)


def test_dequant_of_quant_is_identity_on_grid_rows():
    """A group whose values are grid points times s, with 6s present, has
    amax/6 = s exactly, so the scale is s and every value is reproduced."""
    rng = np.random.default_rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    for sc in list(range(1, 127, 5)) + [126]:
        s = oracle.e4m3_value(sc)
        g = rng.choice(grid, size=512) * rng.choice([-1, 1], size=512)
        g[::16] = 6.0
        x = (g * s).astype(np.float32)
        bits = f32_to_bf16(x)
        assert np.array_equal(synth.bf16_to_f32(bits), x)
        codes, scales = oracle.quant_rows(bits)
        assert np.all(scales == sc)
        assert np.array_equal(oracle.dequant_row(codes[0], scales[0]), x.astype(np.float64))


def test_row_bytes_closed_form():
    """256 code bytes + 32 scale bytes = 288 B per 512-d row, 0.5625 of an
    8-bit row: the pages' 'nearly halves storage against FP8'."""
    codes, scales = oracle.quant_rows(np.zeros((1, 512), np.uint16))
    assert codes.nbytes + scales.nbytes == 288
    assert Fraction(288, 512) == Fraction(9, 16)


# ------------------------------------------------------------------ scoring
def _int_bf16(rng, shape, lo=-4, hi=4):
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16(v), v.astype(np.int64)


def test_score_one_hot_closed_forms():
    rng = np.random.default_rng(1)
    kb, kv = _int_bf16(rng, (100, 64))
    q = np.zeros((8, 64), np.float32)
    dims = [3, 17, 0, 63, 40, 5, 5, 22]
    for h, d in enumerate(dims):
        q[h, d] = -1.0 if h % 3 == 0 else 2.0
    s = oracle.index_score(f32_to_bf16(q), kb, np.arange(100))
    want = sum(np.maximum(q[h, d] * kv[:, d], 0) for h, d in enumerate(dims))
    assert np.array_equal(s, want.astype(np.float32))


def test_score_matches_int64_matmul_relu_sum():
    rng = np.random.default_rng(2)
    qb, qv = _int_bf16(rng, (8, 64))
    kb, kv = _int_bf16(rng, (3000, 64))
    ids = rng.permutation(3000)[:1000]
    s = oracle.index_score(qb, kb, ids)
    want = np.maximum(kv[ids] @ qv.T, 0).sum(axis=1)
    assert np.array_equal(s, want.astype(np.float32))
    # per-head ReLU, not ReLU of the head sum
    assert np.any(want != np.maximum((kv[ids] @ qv.T).sum(axis=1), 0))


def _exact_weighted_score(qv, kv_row, w):
    """sum_h w_h * max(0, q_h . k) in exact rational arithmetic, rounded once
    to binary32 (Fraction -> float is correctly rounded to double; the value
    is a short dyadic or the double is then rounded to binary32 by numpy)."""
    total = Fraction(0)
    for h in range(8):
        dot = sum(int(a) * int(b) for a, b in zip(qv[h], kv_row))
        total += Fraction(float(w[h])) * max(dot, 0)
    return np.float32(float(total))


def test_score_weights_exact_rational():
    """Weighted scores against exact rational arithmetic (fractions.Fraction):
    dyadic weights, whose products and partial sums are exact in binary32 (the
    inputs the library scores bit-exactly), negative ones included; and
    N(0,1) binary32 weights, where the oracle's sum must still be the real sum
    rounded once."""
    rng = np.random.default_rng(3)
    qb, qv = _int_bf16(rng, (8, 64))
    kb, kv = _int_bf16(rng, (300, 64))
    for w in (np.array([1, 2, 0, 3, 1, 1, 4, 2], np.float32),
              (rng.integers(-16, 17, size=8) / 8).astype(np.float32),
              (rng.integers(-3, 40, size=8) * 0.25).astype(np.float32),
              rng.standard_normal(8).astype(np.float32)):
        s = oracle.index_score(qb, kb, np.arange(300), w=w)
        want = np.array([_exact_weighted_score(qv, kv[i], w) for i in range(300)], np.float32)
        assert np.array_equal(s, want), w
    # unit weights are the unweighted score
    ones = np.ones(8, np.float32)
    assert np.array_equal(oracle.index_score(qb, kb, np.arange(300), w=ones), oracle.index_score(qb, kb, np.arange(300)))


# ---------------------------------------------------------------- selection
def _brute_select(scores, ids, k):
    """Top-k by a full sort: NaN and -inf are not candidates; among the rest
    score descending (float64 keys, so -0 and +0 compare equal), then id
    ascending; ids written ascending, -1 padded."""
    scores = np.asarray(scores, np.float32)
    ids = np.asarray(ids, np.int64)
    cand = ~np.isnan(scores) & (scores != -np.inf)
    s, i = scores[cand].astype(np.float64), ids[cand]
    order = np.lexsort((i, -s))  # score desc, id asc
    keep = np.sort(i[order[:k]])
    return np.concatenate([keep, -np.ones(k - len(keep), np.int64)])


@pytest.mark.parametrize("n,k,levels", [(5000, 512, 10000), (5000, 512, 3), (300, 512, 5),
                                        (4096, 512, 1), (20000, 2048, 50), (1, 512, 1), (0, 16, 1)])
def test_select_matches_lexsort(n, k, levels):
    rng = np.random.default_rng(n + levels)
    scores = rng.integers(0, levels, size=n).astype(np.float32)
    ids = rng.permutation(10 * n + 1)[:n].astype(np.int64)
    assert np.array_equal(oracle.select(scores, ids, k), _brute_select(scores, ids, k))


@pytest.mark.parametrize("k", [1, 50, 512, 3000])
def test_select_non_candidates_and_signed_zeros(k):
    """NaN and -inf scores are never selected (also when fewer than k finite
    scores remain: the rest is -1), +inf is the largest score, and -0 ties
    with +0 (the lower id wins)."""
    rng = np.random.default_rng(k)
    n = 4000
    scores = rng.integers(-3, 4, size=n).astype(np.float32)
    scores[::5] = np.nan
    scores[1::7] = -np.inf
    scores[2::11] = np.inf
    scores[3:600:9] = -0.0
    scores[4:600:9] = 0.0
    ids = rng.permutation(3 * n)[:n].astype(np.int64)
    got = oracle.select(scores, ids, k)
    assert np.array_equal(got, _brute_select(scores, ids, k))
    assert not np.any(np.isin(got, ids[np.isnan(scores) | (scores == -np.inf)]))
    # only NaN / -inf: nothing is selected
    bad = np.where(np.arange(100) % 2 == 0, np.nan, -np.inf).astype(np.float32)
    assert np.all(oracle.select(bad, np.arange(100), 8) == -1)
    # -0 and +0 tie: the lower id is kept whatever the sign
    z = np.array([0.0, -0.0, 0.0, -0.0], np.float32)
    assert list(oracle.select(z, [7, 3, 5, 1], 2)) == [1, 3]


def test_select_ties_take_lower_ids():
    scores = np.zeros(1000, np.float32)
    got = oracle.select(scores, np.arange(1000), 512)
    assert np.array_equal(got, np.arange(512))
    scores[700] = 1.0
    got = oracle.select(scores, np.arange(1000), 4)
    assert list(got) == [0, 1, 2, 700]


def _synthetic_seq(seed, L, n_blk=None):
    tk = synth.gen_rows(seed, synth.tensor_id(synth.KIND_IDX_K), synth.INT9, [0], np.arange(L), 64)[0]
    nb = n_blk if n_blk is not None else (L + 7) // 8
    bk = synth.gen_rows(seed, synth.tensor_id(synth.KIND_BLK_K), synth.INT9, [0], np.arange(nb), 64)[0]
    q = synth.gen_rows(seed, synth.tensor_id(synth.KIND_IDX_Q), synth.INT9, [0], np.arange(8), 64)[0]
    return tk, bk, q


def test_flat_select_is_select_over_all_positions():
    tk, _, q = _synthetic_seq(0, 3000)
    s = oracle.index_score(q, tk, np.arange(3000))
    assert np.array_equal(oracle.flat_select(q, tk, 3000), _brute_select(s, np.arange(3000), 512))


@pytest.mark.parametrize("L", [1, 7, 8, 9, 1000, 16383, 16384])
def test_hierarchical_equals_flat_when_all_blocks_fit(L):
    tk, bk, q = _synthetic_seq(1, L)
    pool = oracle.pool_blocks(q, bk, L)
    nb = (L + 7) // 8
    assert np.array_equal(pool[:nb], np.arange(nb)) and np.all(pool[nb:] == -1)
    assert np.array_equal(oracle.pool_select(q, tk, L, pool), oracle.flat_select(q, tk, L))


def test_hierarchical_pool_invariants():
    L = 8 * 3000 + 5
    tk, bk, q = _synthetic_seq(2, L)
    pool = oracle.pool_blocks(q, bk, L, n_pool=256)
    nb = (L + 7) // 8
    bs = oracle.index_score(q, bk, np.arange(nb))
    assert np.array_equal(pool, _brute_select(bs, np.arange(nb), 256))
    idx = oracle.pool_select(q, tk, L, pool)
    assert np.all(np.isin(idx // 8, pool)) and np.all(idx < L)
    cand = (pool[:, None] * 8 + np.arange(8)).ravel()
    cand = cand[cand < L]
    ts = oracle.index_score(q, tk, cand)
    assert np.array_equal(idx, _brute_select(ts, cand, 512))


# ---------------------------------------------------------------- attention
def _dense_attention_torch(q, x, sm_scale):
    qt = torch.from_numpy(q.astype(np.float64))
    xt = torch.from_numpy(x.astype(np.float64))
    p = torch.softmax(sm_scale * (qt @ xt.T), dim=-1)
    return (p @ xt).numpy()


def _random_cache(seed, n_rows):
    src = synth.gen_rows(seed, synth.tensor_id(synth.KIND_KV_SRC), synth.NORMAL, [0], np.arange(n_rows), 512)[0]
    return oracle.quant_rows(src)


def test_attention_with_all_positions_is_dense_softmax_attention():
    codes, scales = _random_cache(3, 300)
    q = synth.gen_rows(3, synth.tensor_id(synth.KIND_MAIN_Q), synth.NORMAL, [0], np.arange(16), 512)[0]
    swa = synth.gen_rows(3, synth.tensor_id(synth.KIND_SWA), synth.NORMAL, [0], np.arange(128), 512)[0]
    idx = np.concatenate([np.arange(300), -np.ones(212, np.int64)])  # k = 512 >= L = 300
    out = oracle.sparse_attn(q, codes, scales, idx, swa, 100, 1 / math.sqrt(512))
    x = np.stack([oracle.dequant_row(codes[i], scales[i]) for i in range(300)]
                 + [synth.bf16_to_f32(swa[j]).astype(np.float64) for j in range(100)])
    ref = _dense_attention_torch(synth.bf16_to_f32(q), x, 1 / math.sqrt(512))
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_attention_special_cases():
    codes, scales = _random_cache(4, 10)
    q = synth.gen_rows(4, synth.tensor_id(synth.KIND_MAIN_Q), synth.NORMAL, [0], np.arange(16), 512)[0]
    empty_swa = np.zeros((1, 512), np.uint16)
    x3 = oracle.dequant_row(codes[3], scales[3])
    # a single key returns that key for every head
    out = oracle.sparse_attn(q, codes, scales, [3, -1, -1], empty_swa, 0, 0.1)
    assert np.array_equal(out, np.tile(x3.astype(np.float32), (16, 1)))
    # equal keys return that key
    out = oracle.sparse_attn(q, codes, scales, [3, 3, 3, 3], empty_swa, 0, 0.1)
    assert np.allclose(out, np.tile(x3, (16, 1)), rtol=0, atol=1e-6)
    # q = 0 gives the mean of the attended rows
    out = oracle.sparse_attn(np.zeros((16, 512), np.uint16), codes, scales, np.arange(10), empty_swa, 0, 0.1)
    mean = np.mean([oracle.dequant_row(codes[i], scales[i]) for i in range(10)], axis=0)
    assert np.allclose(out, np.tile(mean, (16, 1)), rtol=1e-6, atol=1e-7)
    # nothing to attend gives zeros
    out = oracle.sparse_attn(q, codes, scales, [-1, -1], empty_swa, 0, 0.1)
    assert np.all(out == 0)
    # the SWA rows count: only SWA rows -> softmax over them alone
    swa = synth.gen_rows(4, synth.tensor_id(synth.KIND_SWA), synth.NORMAL, [0], np.arange(5), 512)[0]
    out = oracle.sparse_attn(q, codes, scales, [-1], swa, 5, 0.2)
    ref = _dense_attention_torch(synth.bf16_to_f32(q), synth.bf16_to_f32(swa).astype(np.float64), 0.2)
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)


def test_attention_share_normalises_to_attention_over_its_rows():
    codes, scales = _random_cache(8, 400)
    q = synth.gen_rows(8, synth.tensor_id(synth.KIND_MAIN_Q), synth.NORMAL, [0], np.arange(16), 512)[0]
    swa = synth.gen_rows(8, synth.tensor_id(synth.KIND_SWA), synth.NORMAL, [0], np.arange(128), 512)[0]
    rng = np.random.default_rng(8)
    idx = np.sort(rng.choice(400, 150, replace=False)).astype(np.int64)
    idx[::7] = -1
    sm = 1 / math.sqrt(512)
    o, ml = oracle.sparse_attn_partial(q, codes, scales, idx, swa, 60, sm)
    ref = oracle.sparse_attn(q, codes, scales, idx, swa, 60, sm)
    assert np.allclose(o / ml[:, 1:2], ref, rtol=1e-6, atol=1e-7)
    # m is the largest base-2 logit over the rows (numpy float64 matmul), and l >= 1
    x = np.stack([oracle.dequant_row(codes[i], scales[i]) for i in idx if i >= 0]
                 + [synth.bf16_to_f32(swa[j]).astype(np.float64) for j in range(60)])
    logits = sm / math.log(2) * (synth.bf16_to_f32(q).astype(np.float64) @ x.T)
    assert np.allclose(ml[:, 0], logits.max(axis=1), rtol=1e-12, atol=1e-12)
    assert np.all(ml[:, 1] >= 1.0) and np.all(ml[:, 1] <= x.shape[0])
    # an empty share
    o, ml = oracle.sparse_attn_partial(q, codes, scales, [-1, -1], swa, 0, sm)
    assert np.all(o == 0) and np.all(ml[:, 0] == -np.inf) and np.all(ml[:, 1] == 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_shares_equals_attention_over_all_rows(seed):
    """The rows of one query split at random over 3 shares (the window on
    one of them, one share possibly empty): the merge of the shares is the
    attention over all the rows."""
    codes, scales = _random_cache(9 + seed, 600)
    q = synth.gen_rows(9 + seed, synth.tensor_id(synth.KIND_MAIN_Q), synth.NORMAL, [0], np.arange(16), 512)[0]
    swa = synth.gen_rows(9 + seed, synth.tensor_id(synth.KIND_SWA), synth.NORMAL, [0], np.arange(128), 512)[0]
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(600, 512, replace=False)).astype(np.int64)
    owner = rng.integers(0, 3 if seed else 2, size=idx.size)  # seed 0: share 2 holds no row
    tail = int(rng.integers(0, 3))
    sm = 1 / math.sqrt(512)
    o_parts, ml_parts = [], []
    for s in range(3):
        o, ml = oracle.sparse_attn_partial(q, codes, scales, np.where(owner == s, idx, -1), swa,
                                           128 if s == tail else 0, sm)
        o_parts.append(o)
        ml_parts.append(ml)
    got = oracle.attn_merge(np.stack(o_parts), np.stack(ml_parts))
    ref = oracle.sparse_attn(q, codes, scales, idx, swa, 128, sm)
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-7)
    # one share merges to its own attention
    one = oracle.attn_merge(o_parts[tail][None], ml_parts[tail][None])
    assert np.allclose(one, oracle.sparse_attn(q, codes, scales, np.where(owner == tail, idx, -1), swa, 128, sm),
                       rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- layer walk
def _layer_inputs(seed, n_layers, modes):
    ins = []
    for l in range(n_layers):
        iq = None
        if modes[l] != oracle.REUSE:
            iq = synth.gen_rows(seed, synth.tensor_id(synth.KIND_IDX_Q, l), synth.INT9, [0], np.arange(8), 64)[0]
        mq = synth.gen_rows(seed, synth.tensor_id(synth.KIND_MAIN_Q, l), synth.NORMAL, [0], np.arange(16), 512)[0]
        sw = synth.gen_rows(seed, synth.tensor_id(synth.KIND_SWA, l), synth.NORMAL, [0], np.arange(128), 512)[0]
        ins.append(oracle.LayerInputs(idx_q=iq, main_q=mq, swa=sw, swa_len=128))
    return ins


def test_reuse_layers_reproduce_latest_indices_and_reindex_with_full_q_equals_full():
    L = 8 * 2500 + 3
    tk, bk, _ = _synthetic_seq(6, L)
    codes, scales = _random_cache(6, L)
    modes = [oracle.FULL, oracle.REUSE, oracle.REUSE, oracle.REINDEX, oracle.REUSE, oracle.REINDEX]
    layers = [oracle.Layer(m, 0, True) for m in modes]
    ins = _layer_inputs(6, len(layers), modes)
    ins[5].idx_q = ins[0].idx_q  # Reindex with the Full layer's own indexer Q
    seq = oracle.SeqState(L=L, tok_keys=tk, blk_keys=bk,
                          kv_rows=lambda kv, ids: (codes, scales))
    res = oracle.decode_layers(layers, seq, ins, 1 / math.sqrt(512), n_pool=256)
    assert np.array_equal(res[1].idx, res[0].idx) and np.array_equal(res[2].idx, res[0].idx)
    assert np.array_equal(res[4].idx, res[3].idx)
    assert not np.array_equal(res[3].idx, res[0].idx)
    assert np.array_equal(res[5].idx, res[0].idx)
    # Reuse layers attend with their own Q: outputs differ though indices agree
    assert not np.allclose(res[1].out, res[0].out)


def test_full_layer_with_own_keys_and_its_reindex():
    """A Full layer with its own indexer K selects over those keys, the
    Reindex layer after it rescores the same keys, and earlier layers keep the
    shared keys; own keys equal to the shared ones change nothing."""
    L = 3000
    tk, _, _ = _synthetic_seq(9, L)
    k2 = synth.gen_rows(9, synth.tensor_id(synth.KIND_IDX_K, 2), synth.INT9, [0], np.arange(L), 64)[0]
    codes, scales = _random_cache(9, L)
    modes = [oracle.FULL, oracle.REUSE, oracle.FULL, oracle.REINDEX]
    layers = [oracle.Layer(m, 0, False) for m in modes]
    ins = _layer_inputs(9, len(layers), modes)

    def walk(layer_keys):
        seq = oracle.SeqState(L=L, tok_keys=tk, kv_rows=lambda kv, ids: (codes, scales), layer_keys=layer_keys)
        return oracle.decode_layers(layers, seq, ins, 1 / math.sqrt(512), attend=False)

    def brute(q, keys):  # every position scored, the top 512 by (score desc, id asc)
        sc = oracle.index_score(q, keys, np.arange(L))
        order = np.lexsort((np.arange(L), -sc.astype(np.float64)))
        return np.sort(order[:512])

    res = walk({2: k2})
    assert np.array_equal(res[0].idx, brute(ins[0].idx_q, tk))
    assert np.array_equal(res[2].idx, brute(ins[2].idx_q, k2))
    assert np.array_equal(res[3].idx, brute(ins[3].idx_q, k2))
    assert not np.array_equal(res[3].idx, brute(ins[3].idx_q, tk))
    same = walk({2: tk})
    plain = walk(None)
    for a, b in zip(same, plain):
        assert np.array_equal(a.idx, b.idx)


def test_table_validation():
    with pytest.raises(ValueError):
        oracle.check_table([oracle.Layer(oracle.REUSE)])
    with pytest.raises(ValueError):
        oracle.check_table([oracle.Layer(oracle.REINDEX)])
    oracle.check_table([oracle.Layer(oracle.FULL), oracle.Layer(oracle.REINDEX), oracle.Layer(oracle.REUSE)])


def test_prefill_visibility_ratio_two():
    # entry e = tokens {2e, 2e+1}: visible once token 2e+1 has been seen
    assert [oracle.prefill_visible_entries(t, 2) for t in range(6)] == [0, 1, 1, 2, 2, 3]


@pytest.mark.parametrize("ratio", [1, 2, 3])
def test_prefill_visibility_by_enumeration(ratio):
    # brute force: count the entries whose every token is at or before t
    for t in range(40):
        for n_entries in (5, 1000):
            want = sum(1 for e in range(n_entries) if all(ratio * e + j <= t for j in range(ratio)))
            assert oracle.prefill_visible_entries(t, ratio, n_entries) == want, (t, ratio, n_entries)


def test_prefill_window_by_enumeration():
    for swa in (1, 4, 128):
        for t in range(300):
            toks = [u for u in range(t + 1) if t - u < swa]
            assert oracle.prefill_window(t, swa) == (toks[0], len(toks))


# ------------------------------------------------------------- FP8 window
def test_fp8_code_golden_worked_values():
    for h, _value, code, *_ in _golden_lines("fp8_e4m3_rne.txt"):
        assert oracle.fp8_code(int(h, 16)) == int(code, 16), h


def test_fp8_codes_of_all_bf16_vs_torch_cast():
    """Every bf16 pattern: where torch's float -> float8_e4m3fn cast does not
    overflow (|x| < 464, half-way past 448) the codes agree bit for bit,
    signed zeros included; beyond, the oracle saturates to +-448; NaN maps
    to NaN with the sign kept."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = synth.bf16_to_f32(bits).astype(np.float32)
    got = oracle.fp8_rows(bits.reshape(-1, 512)).reshape(-1)   # 128 rows of 512
    nan = np.isnan(x)
    fits = ~nan & (np.abs(x) < 464.0)
    ref = torch.from_numpy(x[fits]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[fits], ref)
    big = ~nan & ~fits
    assert np.all(got[big] == np.where(x[big] > 0, 0x7E, 0xFE))
    assert np.all((got[nan] & 0x7F) == 0x7F) and np.all((got[nan] >> 7) == (bits[nan] >> 15))


def test_fp8_window_attention_equals_bf16_window_on_exact_rows():
    """With window rows whose values FP8 holds exactly, attention over the
    FP8 window equals attention over the same rows in bf16."""
    rng = np.random.default_rng(11)
    codes8 = rng.integers(0, 256, size=(40, 512)).astype(np.uint8)
    codes8[(codes8 & 0x7F) == 0x7F] = 0x3C                     # no NaN
    vals = np.array([oracle.lib().orc_e4m3_value(int(c)) for c in range(256)])
    rows_bf16 = f32_to_bf16(vals[codes8].astype(np.float32))   # exact: E4M3 values are bf16 values
    assert np.array_equal(oracle.fp8_rows(rows_bf16), codes8)
    src = synth.gen_rows(0, 99, synth.NORMAL, [0], np.arange(50), 512)[0]
    codes, scales = oracle.quant_rows(src)
    q = synth.gen_rows(0, 98, synth.NORMAL, [0], np.arange(16), 512)[0]
    idx = np.array([3, 7, -1, 20, 49], np.int64)
    a = oracle.sparse_attn(q, codes, scales, idx, rows_bf16, 37, 512 ** -0.5)
    b = oracle.sparse_attn_fp8w(q, codes, scales, idx, codes8, 37, 512 ** -0.5)
    assert np.array_equal(a, b)


# ------------------------------------------------- block-key maintenance
@pytest.mark.parametrize("L", [1, 8, 9, 63, 64, 200])
def test_block_keys_are_sums_of_integer_keys(L):
    """Integer-valued keys: each block key is the exact int64 sum of its
    positions' keys (numpy), the partial last block summing only positions
    < L; a block never includes a position of its neighbours."""
    keys = synth.gen_rows(0, 4242, synth.INT9, [0], np.arange(208), 64)[0]
    ints = synth.bf16_to_f32(keys).astype(np.int64)
    got = synth.bf16_to_f32(oracle.block_keys(keys, L, 8)).astype(np.int64)
    nb = -(-L // 8)
    want = np.stack([ints[8 * b:min(8 * b + 8, L)].sum(axis=0) for b in range(nb)])
    assert np.array_equal(got, want)


def test_block_key_one_hot():
    keys = np.zeros((16, 64), np.float32)
    keys[9, 5] = 3.0       # block 1, dimension 5
    keys[15, 5] = -1.0     # block 1, dimension 5
    keys[7, 0] = 2.0       # block 0, dimension 0
    bk = synth.bf16_to_f32(oracle.block_keys(f32_to_bf16(keys), 16, 8))
    expect = np.zeros((2, 64), np.float32)
    expect[1, 5] = 2.0
    expect[0, 0] = 2.0
    assert np.array_equal(bk, expect)
