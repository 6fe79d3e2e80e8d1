"""GPU parity of whole decode steps through the native scheduler against the
oracle's layer walk, on the pages' layer tables at reduced sizes that still
span many tiles and ragged tails: selected indices and pool blocks
bit-exact, appended FP4 rows bit-exact, attention within tolerance."""
import numpy as np
import pytest
import torch

import oracle
from oracle import workloads as ow
from synth import configs as C
from gpu_helpers import assert_attention_close, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wl():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_quant_amd import workloads
    return workloads


CASES = {
    "single_4k": (C.SINGLE_LAYER_4K, 1),
    "group_small": (C.GROUP_64K.with_(n_seq=4, L0=3000), 3),
    "hier_small": (C.HIER_1M.with_(n_seq=2, L0=8 * 3000 + 5), 1),
    "decoder20_small": (C.DECODER_20L_1M.with_(n_seq=2, L0=8 * 2500 + 3, q_sets=2), 3),
    "decoder20_short_ctx": (C.DECODER_20L_1M.with_(n_seq=2, L0=300, q_sets=2, pool_blocks=16), 2),
    # more than 32K blocks: the multi-workgroup filter pass of the block Top-k
    "hier_long": (C.HIER_1M.with_(n_seq=2, L0=8 * 40000 + 3), 1),
    # window rows stored as E4M3 (FP8)
    "decoder20_fp8_window": (C.DECODER_20L_1M.with_(n_seq=2, L0=8 * 2500 + 3, q_sets=2, swa_fp8=True), 2),
    # encoder groups at ratio 2, each Full layer with its own indexer K
    "encoder_small": (C.ENCODER_DECODE_1M.with_(n_seq=2, L0=3001, q_sets=2), 2),
    # more entries than the selection bitmaps held in LDS (262,144)
    "encoder_long": (C.ENCODER_DECODE_1M.with_(n_seq=2, L0=300001, q_sets=1), 1),
    # Top-2048 over 300K entries: too many per-workgroup candidates, so the
    # scores go through the multi-workgroup selection instead
    "encoder_long_k2048": (C.ENCODER_DECODE_1M.with_(n_seq=2, L0=300001, q_sets=1, topk=2048), 1),
    # a long Reuse run, and Reuse layers on another main-KV tensor
    "long_reuse_runs": (C.GROUP_64K.with_(n_seq=3, L0=2000, n_kv=2, q_sets=1,
                                          layers=((C.FULL, 0, 0),) + ((C.REUSE, 0, 0),) * 9
                                          + ((C.REUSE, 1, 0),) * 2), 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_steps_match_oracle(wl, name):
    cfg, steps = CASES[name]
    print_case(f"sched {name}: n_seq={cfg.n_seq} L0={cfg.L0} layers={len(cfg.layers)} steps={steps}")
    inp = wl.build_decode_inputs(cfg, steps)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    for step in range(steps):
        sched.decode_step(ios[step % cfg.q_sets])
        idx = [sched.indices(l).cpu().numpy() for l in range(len(cfg.layers))]
        pool = sched.pool()
        pool = pool.cpu().numpy() if pool is not None else None
        outs = [o.cpu().numpy() for o in inp.out]
        assert inp.lens.cpu().tolist() == [cfg.lens_at(step)] * cfg.n_seq
        for b in range(cfg.n_seq):
            ref = ow.reference_step(cfg, step, b)
            for l, r in enumerate(ref):
                assert np.array_equal(idx[l][b], r.idx), f"step {step} seq {b} layer {l} indices"
                if r.pool is not None and cfg.layers[l][0] == C.FULL:
                    assert np.array_equal(pool[b], r.pool), f"step {step} seq {b} pool"
                assert_attention_close(outs[l][b], r.out, f"step {step} seq {b} layer {l}")
    assert sched.check() == 0
    if cfg.append:  # every appended row, bit-exact
        kv = inp.kv[cfg.append_kv]
        pos = np.arange(cfg.L0, cfg.L0 + steps)
        for b in range(cfg.n_seq):
            codes, scales = oracle.quant_rows(ow.kv_source_rows(cfg, cfg.append_kv, b, pos))
            assert np.array_equal(kv.codes[b, cfg.L0:cfg.L0 + steps].cpu().numpy(), codes)
            assert np.array_equal(kv.scales[b, cfg.L0:cfg.L0 + steps].cpu().numpy(), scales)
    sched.close()


def test_reuse_layers_share_indices_and_append_overflow_flag(wl):
    cfg = C.GROUP_64K.with_(n_seq=2, L0=500, q_sets=1)
    print_case("sched overflow flag")
    inp = wl.build_decode_inputs(cfg, 1)
    sched = wl.make_sched(inp)
    io = wl.step_ios(sched, inp)[0]
    sched.decode_step(io)
    a = [sched.indices(l).cpu().numpy() for l in range(4)]
    assert all(np.array_equal(a[0], x) for x in a[1:])
    sched.decode_step(io)  # cache is full now: the append reports and leaves lens alone
    assert sched.check() == 1 and inp.lens.cpu().tolist() == [501, 501]
    assert sched.check() == 0
    # Steps on a side stream, checked on that stream without a device-wide
    # synchronisation: the read waits for the steps enqueued before it.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            sched.decode_step(io)
        assert sched.check(side) == 1
        assert sched.check(side) == 0
    torch.cuda.synchronize()
    sched.close()


FULL_SIZE = {
    # the workloads at their full sizes, in the launch configuration the
    # benchmark times (native scheduler, one call per step); sampled
    # sequences against the oracle, every appended row checked bit-exact
    "group_64k_b32": (C.GROUP_64K, 2, [0, 31]),
    "hier_1m_b8": (C.HIER_1M, 1, [0, 7]),
    "decoder20_1m_b16": (C.DECODER_20L_1M, 3, [0, 9, 15]),
    "decoder20_1m_b16_fp8_window": (C.DECODER_20L_1M_FP8_WINDOW, 2, [0, 15]),
    "decoder20_1m_b16_maintained_keys": (C.DECODER_20L_1M_KEYS, 3, [0, 15]),
    "encoder_1m_b16": (C.ENCODER_DECODE_1M, 2, [0, 15]),
}


@pytest.mark.parametrize("name", list(FULL_SIZE))
def test_full_size_steps_sampled_sequences(wl, name):
    cfg, steps, seqs = FULL_SIZE[name]
    print_case(f"sched full size {name}: n_seq={cfg.n_seq} L0={cfg.L0} steps={steps} seqs={seqs}")
    inp = wl.build_decode_inputs(cfg, steps)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    for step in range(steps):
        sched.decode_step(ios[step % cfg.q_sets])
        idx = [sched.indices(l).cpu().numpy() for l in range(len(cfg.layers))]
        pool = sched.pool()
        pool = pool.cpu().numpy() if pool is not None else None
        outs = [o.cpu().numpy() for o in inp.out]
        for b in seqs:
            ref = ow.reference_step(cfg, step, b)
            for l, r in enumerate(ref):
                assert np.array_equal(idx[l][b], r.idx), f"step {step} seq {b} layer {l} indices"
                if r.pool is not None and cfg.layers[l][0] == C.FULL:
                    assert np.array_equal(pool[b], r.pool), f"step {step} seq {b} pool"
                assert_attention_close(outs[l][b], r.out, f"step {step} seq {b} layer {l}")
    assert sched.check() == 0
    if cfg.append:
        kv = inp.kv[cfg.append_kv]
        pos = np.arange(cfg.L0, cfg.L0 + steps)
        for b in range(cfg.n_seq):
            codes, scales = oracle.quant_rows(ow.kv_source_rows(cfg, cfg.append_kv, b, pos))
            assert np.array_equal(kv.codes[b, cfg.L0:cfg.L0 + steps].cpu().numpy(), codes)
            assert np.array_equal(kv.scales[b, cfg.L0:cfg.L0 + steps].cpu().numpy(), scales)
    sched.close()
    del inp
    torch.cuda.empty_cache()


KEY_CASES = {
    # hierarchical selection over maintained block keys: more than 2,048
    # blocks, the appends start and extend partial blocks
    "hier_keys": (C.HIER_1M.with_(n_seq=2, L0=8 * 3000 + 5, append=True, maintain_keys=True, q_sets=3), 5),
    "decoder20_keys": (C.DECODER_20L_1M.with_(n_seq=2, L0=8 * 2500 + 6, q_sets=3, maintain_keys=True), 4),
}


@pytest.mark.parametrize("name", list(KEY_CASES))
def test_decode_steps_with_maintained_keys(wl, name):
    """Every step appends the new position's indexer key and updates its
    block's key on the GPU; indexer K rows, block keys, pools, indices and
    outputs match the oracle, which forms block keys as sums."""
    cfg, steps = KEY_CASES[name]
    print_case(f"sched maintained keys {name}: n_seq={cfg.n_seq} L0={cfg.L0} steps={steps}")
    inp = wl.build_decode_inputs(cfg, steps)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    for step in range(steps):
        sched.decode_step(ios[step % cfg.q_sets])
        L = cfg.lens_at(step)
        idx = [sched.indices(l).cpu().numpy() for l in range(len(cfg.layers))]
        pool = sched.pool().cpu().numpy()
        outs = [o.cpu().numpy() for o in inp.out]
        for b in range(cfg.n_seq):
            tok = ow.index_key_rows(cfg, b, L)
            assert np.array_equal(inp.idx_k[b, :L].cpu().numpy().view(np.uint16), tok), f"step {step} idx_k"
            nb = -(-L // cfg.blk)
            assert np.array_equal(inp.blk_k[b, :nb].cpu().numpy().view(np.uint16),
                                  oracle.block_keys(tok, L, cfg.blk)), f"step {step} seq {b} block keys"
            ref = ow.reference_step(cfg, step, b)
            for l, r in enumerate(ref):
                assert np.array_equal(idx[l][b], r.idx), f"step {step} seq {b} layer {l} indices"
                if cfg.layers[l][0] == C.FULL:
                    assert np.array_equal(pool[b], r.pool), f"step {step} seq {b} pool"
                assert_attention_close(outs[l][b], r.out, f"step {step} seq {b} layer {l}")
    assert sched.check() == 0
    sched.close()


def test_layer_keys_only_on_flat_full_layers(wl):
    """An own indexer K given for a Reuse layer is rejected before any launch."""
    import fp4_kv_cache_quant_amd as csa2
    cfg = C.ENCODER_DECODE_1M.with_(n_seq=1, L0=600, q_sets=1)
    print_case("sched layer keys validation")
    inp = wl.build_decode_inputs(cfg, 1)
    sched = wl.make_sched(inp)
    bad = list(inp.layer_idx_k)
    bad[1] = inp.idx_k
    io = sched.prepare(kv=inp.kv, lens=inp.lens, idx_k=inp.idx_k, main_q=inp.main_q[0], swa=inp.swa,
                       swa_len=inp.swa_len, out=inp.out, idx_q=inp.idx_q[0], layer_idx_k=bad)
    with pytest.raises(csa2.Csa2Error, match="layer_idx_k"):
        sched.decode_step(io)
    sched.close()


def test_step_rejects_misaligned_tensors(wl):
    """A main Q that is not 16-byte aligned is rejected before any launch."""
    import torch

    import fp4_kv_cache_quant_amd as csa2
    cfg = C.ENCODER_DECODE_1M.with_(n_seq=1, L0=600, q_sets=1)
    print_case("sched alignment validation")
    inp = wl.build_decode_inputs(cfg, 1)
    sched = wl.make_sched(inp)
    mq = list(inp.main_q[0])
    base = torch.empty(mq[2].numel() + 8, dtype=mq[2].dtype, device=mq[2].device)
    mq[2] = base[1:1 + mq[2].numel()].view(mq[2].shape)          # 2 bytes off
    io = sched.prepare(kv=inp.kv, lens=inp.lens, idx_k=inp.idx_k, main_q=mq, swa=inp.swa,
                       swa_len=inp.swa_len, out=inp.out, idx_q=inp.idx_q[0], layer_idx_k=inp.layer_idx_k)
    with pytest.raises(csa2.Csa2Error, match="16-byte aligned"):
        sched.decode_step(io)
    sched.close()


def test_checkpoint_and_resume_reproduces_the_steps(wl):
    """Everything a decode step carries across steps -- the FP4 caches,
    lengths, indexer K, (maintained) block keys and the window rings --
    copied to host memory after 3 steps, restored into new device buffers
    under a new scheduler, and stepped on: steps 3..5 give bit-identical
    indices, pool and outputs to an uninterrupted run."""
    cfg = C.DECODER_20L_1M_KEYS.with_(n_seq=2, L0=8 * 900 + 3, q_sets=6)
    steps, cut = 6, 3
    nl = len(cfg.layers)

    def snapshot(sched, inp):
        return ([sched.indices(l).cpu().numpy() for l in range(nl)], sched.pool().cpu().numpy(),
                [o.cpu().numpy() for o in inp.out])

    print_case("checkpoint / resume, 20-layer table with maintained keys")
    inp = wl.build_decode_inputs(cfg, steps)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    ref = []
    for s in range(steps):
        sched.decode_step(ios[s])
        if s >= cut:
            ref.append(snapshot(sched, inp))
    assert sched.check() == 0
    sched.close()
    del inp, ios, sched

    inp = wl.build_decode_inputs(cfg, steps)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    for s in range(cut):
        sched.decode_step(ios[s])
    torch.cuda.synchronize()
    saved = {"kv": [(t.codes.cpu(), t.scales.cpu()) for t in inp.kv], "lens": inp.lens.cpu(),
             "idx_k": inp.idx_k.cpu(), "blk_k": inp.blk_k.cpu(), "swa": [t.cpu() for t in inp.swa]}
    sched.close()
    del ios, sched
    # restore into new buffers (the old ones are dropped) and a new scheduler
    inp.kv = [csa2_fp4(c.cuda(), s_.cuda()) for c, s_ in saved["kv"]]
    inp.lens, inp.idx_k, inp.blk_k = saved["lens"].cuda(), saved["idx_k"].cuda(), saved["blk_k"].cuda()
    inp.swa = [t.cuda() for t in saved["swa"]]
    torch.cuda.synchronize()
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    for i, s in enumerate(range(cut, steps)):
        sched.decode_step(ios[s])
        idx, pool, out = snapshot(sched, inp)
        r_idx, r_pool, r_out = ref[i]
        assert np.array_equal(pool, r_pool), s
        for l in range(nl):
            assert np.array_equal(idx[l], r_idx[l]), (s, l)
            assert np.array_equal(out[l], r_out[l]), (s, l)
    assert sched.check() == 0 and inp.lens.cpu().tolist() == [cfg.L0 + steps] * cfg.n_seq
    sched.close()


def csa2_fp4(codes, scales):
    import fp4_kv_cache_quant_amd as csa2
    return csa2.FP4KV(codes, scales)


def test_pool_selection_all_ties_and_partly_tied_rows(wl):
    """The hierarchical path with its pool Top-k after bounded scoring, when
    the bound admits more keys than the selection's LDS list: a zero indexer
    Q makes every block and pool score 0 (ties everywhere: the first 2,048
    blocks, then the first 512 positions), and a Reindex Q of zeros in one
    sequence only; indices, pool and outputs against the oracle."""
    import oracle as orc
    cfg = C.HIER_1M.with_(n_seq=2, L0=8 * 3000 + 5, q_sets=1)
    print_case("pool selection, all scores tied")
    inp = wl.build_decode_inputs(cfg, 1)
    inp.idx_q[0][0].zero_()        # Full layer, both sequences
    inp.idx_q[0][1][1].zero_()     # Reindex layer, sequence 1
    sched = wl.make_sched(inp)
    sched.decode_step(wl.step_ios(sched, inp)[0])
    torch.cuda.synchronize()
    pool = sched.pool().cpu().numpy()
    idx = [sched.indices(l).cpu().numpy() for l in range(2)]
    for b in range(cfg.n_seq):
        assert np.array_equal(pool[b], np.arange(2048)), b
        assert np.array_equal(idx[0][b], np.arange(512)), b
        st = ow.seq_state(cfg, b, 0)
        q = inp.idx_q[0][1][b].cpu().numpy().view(np.uint16)
        ref = orc.pool_select(q, st.tok_keys, st.L, pool[b].astype(np.int64))
        assert np.array_equal(idx[1][b], ref), b
        if b == 1:
            assert np.array_equal(idx[1][b], np.arange(512))
    assert sched.check() == 0
    sched.close()
