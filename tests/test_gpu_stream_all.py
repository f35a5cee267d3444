"""The batched all-cluster stream (flashhead_plan_step path 4) on the GPU,
through the C ABI, against the oracle.

Path 4 computes the stage-1 keys and, for every cluster and batch row, the
best decode key and log-sum-exp of the cluster's candidates in one launch,
before any selection exists; a second kernel selects each row's clusters and
folds only their records.  The stream keeps no per-candidate logits (the
debug candidates come from a second gather, covered by the parity tests of
the B=64 and INT4 B=32 workloads), so these tests run without them: per row
they check the stage-1 scores, R1 on the
GPU's selection, R3 (greedy) or R4 (sampling) with the oracle decoding the
candidates of the GPU's own selection, and the sampling lse against the
oracle's lse over those candidates.  The paths' tokens are also compared
with the select-first path (3) on the same inputs: where both paths select
the same clusters, tokens must agree exactly."""
import numpy as np
import pytest

from oracle import flashhead_ref as ref
from two_stage_retrieval_amd import synth

from .parity import Stats, check_selection, check_token
from .test_gpu_adaptive import count_bounds
from .test_gpu_parity import case, dev_tensor, fh, report  # noqa: F401

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PATH_SELECT_FIRST, PATH_STREAM_ALL = 3, 4
UNUSED = 0x7FFFFFFF


def prepare(fhmod, cs, max_batch, max_p, flags):
    quant = fhmod.FH_QUANT_INT4_G128 if cs.wl.quant == "int4_g128" else fhmod.FH_QUANT_NONE
    return fhmod.FlashHead(cs.E_dev, cs.head.c2t, cs.C_dev, quant=quant, max_batch=max_batch,
                           max_p=max_p, flags=flags)


def seeds_dev(seeds):
    return torch.from_numpy(seeds.view(np.int64)).cuda()


def run(fhmod, head, H_dev, B, p, mode, tau=1.0, seeds=None, adaptive=None):
    """One step with the scores and the selection read back (no candidate
    logits: only what the step itself computes)."""
    dbg = {
        "scores": torch.empty(B, head.c, dtype=torch.float32, device="cuda"),
        "clusters": torch.empty(B, p, dtype=torch.int32, device="cuda"),
    }
    lse = torch.empty(B, dtype=torch.float32, device="cuda") if mode == "sample" else None
    out_p = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    if adaptive is None:
        if mode == "greedy":
            out = head.greedy(H_dev, p, debug=dbg)
        else:
            out = head.sample(H_dev, p, tau, seeds, out_lse=lse, debug=dbg)
    else:
        p_min, eps = adaptive
        if mode == "greedy":
            out = head.greedy_adaptive(H_dev, p_min, p, eps, out_p=out_p, debug=dbg)
        else:
            out = head.sample_adaptive(H_dev, p_min, p, eps, tau, seeds, out_lse=lse,
                                       out_p=out_p, debug=dbg)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in dbg.items()}
    res["tokens"] = out.cpu().numpy()
    res["path"] = fhmod.flashhead_query(head.handle, 10)
    res["p"] = out_p.cpu().numpy()
    if lse is not None:
        res["lse"] = lse.cpu().numpy()
    return res


def check_row(cs, res, r, h64, scores, p, mode, tau, seed, stats, score_tol=2e-2):
    assert np.max(np.abs(res["scores"][r] - scores)) <= score_tol
    sel = res["clusters"][r][:p]
    check_selection(sel, ref.select_keys(scores, mode, tau, seed), p, stats)
    ids = ref.candidate_tokens(np.sort(sel), cs.head.c2t)
    z = ref.exact_logits(cs.rows, ids, h64)
    check_token(res["tokens"][r], ids, z, mode, tau, seed, stats)
    if mode == "sample":
        assert res["lse"][r] == pytest.approx(ref.logsumexp(z / tau), abs=1e-3, rel=1e-5)
    stats.rows += 1


def check_steps(cs, steps, p, mode="greedy", tau=1.0, stats=None, score_tol=2e-2):
    from concurrent.futures import ThreadPoolExecutor
    sc = cs.oracle_scores_many(np.concatenate([H64 for _, H64, _ in steps]))
    jobs = []
    i = 0
    for res, H64, seeds in steps:
        for r in range(H64.shape[0]):
            jobs.append((res, r, H64[r], sc[i], int(seeds[r]) if seeds is not None else 0))
            i += 1

    def one(job):
        res, r, h64, scores, seed = job
        st = Stats()
        check_row(cs, res, r, h64, scores, p, mode, tau, seed, st, score_tol)
        return st

    with ThreadPoolExecutor(max_workers=8) as ex:
        for st in ex.map(one, jobs):
            stats.merge(st)


def test_llama_greedy_b64_stream_all(fh):
    """16 batches of 64 rows (1024 rows) on the all-cluster stream."""
    cs = case(2)
    head = prepare(fh, cs, 64, 512, fh.FH_FLAG_STREAM_ALL)
    st = Stats()
    steps = []
    for i in range(16):
        H, H64 = cs.hidden(64, offset=64 * i)
        res = run(fh, head, dev_tensor(H), 64, 512, "greedy")
        assert res["path"] == PATH_STREAM_ALL
        steps.append((res, H64, None))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 512, stats=st)
    report("llama3.2-1b-head-b64 greedy B=64 stream-all", st)
    assert st.rows == 1024


def test_gemma_int4_b32_stream_all(fh):
    """8 batches of 32 rows: INT4 stage-1 tiles inside the stream."""
    cs = case(4)
    head = prepare(fh, cs, 32, 1024, fh.FH_FLAG_STREAM_ALL)
    st = Stats()
    steps = []
    H, H64 = cs.hidden(256)
    for lo in range(0, 256, 32):
        res = run(fh, head, dev_tensor(H[lo:lo + 32]), 32, 1024, "greedy")
        assert res["path"] == PATH_STREAM_ALL
        steps.append((res, H64[lo:lo + 32], None))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 1024, stats=st)
    report("gemma3-1b-head-int4 greedy B=32 stream-all", st)
    assert st.rows == 256


@pytest.mark.parametrize("tau", [0.7, 1.0])
def test_llama_sample_b16_stream_all(fh, tau):
    """16 steps of 16 rows per temperature, sampled on the all-cluster
    stream (Gumbel keys in stage 1 and on every candidate; lse folded from
    the selected clusters' records)."""
    cs = case(3)
    head = prepare(fh, cs, 16, 512, fh.FH_FLAG_STREAM_ALL)
    st = Stats()
    steps = []
    for step in range(16):
        H, H64 = cs.hidden(16, offset=16 * step)
        seeds = synth.make_seeds(step, 16)
        res = run(fh, head, dev_tensor(H), 16, 512, "sample", tau, seeds_dev(seeds))
        assert res["path"] == PATH_STREAM_ALL
        steps.append((res, H64, seeds))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 512, "sample", tau, stats=st)
    report(f"llama3.2-1b-head-sample-b16 tau={tau} B=16 stream-all", st)
    assert st.rows == 256


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_stream_all_matches_select_first(fh, mode):
    """Same rows through paths 3 and 4: equal selections give equal tokens
    (and lse within float rounding of the fold order)."""
    cs = case(2)
    a = prepare(fh, cs, 64, 512, fh.FH_FLAG_SELECT_FIRST)
    b = prepare(fh, cs, 64, 512, fh.FH_FLAG_STREAM_ALL)
    same = rows = 0
    for i in range(4):
        H, _ = cs.hidden(64, offset=2000 + 64 * i)
        x = dev_tensor(H)
        sd = seeds_dev(synth.make_seeds(300 + i, 64))
        ra = run(fh, a, x, 64, 512, mode, 0.8, sd)
        rb = run(fh, b, x, 64, 512, mode, 0.8, sd)
        assert ra["path"] == PATH_SELECT_FIRST and rb["path"] == PATH_STREAM_ALL
        for r in range(64):
            rows += 1
            if not np.array_equal(ra["clusters"][r], rb["clusters"][r]):
                continue
            same += 1
            assert ra["tokens"][r] == rb["tokens"][r]
            if mode == "sample":
                assert rb["lse"][r] == pytest.approx(ra["lse"][r], abs=1e-4, rel=1e-6)
    assert fh.flashhead_query(a.handle, 9) == 0 and fh.flashhead_query(b.handle, 9) == 0
    assert same >= 0.9 * rows
    print(f"stream-all vs select-first {mode}: {same}/{rows} rows with the same selection")


@pytest.mark.parametrize("wid,over,B,ps", [
    # c = 50: stage-1 items end inside a 16-row item and inside a unit
    (1, (("c", 50), ("b", 16), ("d", 256), ("seed", 77)), 5, (1, 7, 50)),
    # b = 32: two 16-row items per cluster; 17 rows: a partial second tile of H
    (1, (("c", 37), ("b", 32), ("d", 384), ("seed", 78)), 17, (3, 37)),
    # INT4 stage-1 tiles with a ragged last tile
    (4, (("c", 40), ("b", 16), ("d", 384), ("seed", 79)), 3, (1, 9, 40)),
])
def test_stream_all_ragged(fh, wid, over, B, ps):
    cs = case(wid, **dict(over))
    head = prepare(fh, cs, B, max(ps), fh.FH_FLAG_STREAM_ALL)
    H, H64 = cs.hidden(2 * B, offset=5)
    for p in ps:
        for mode in ("greedy", "sample"):
            st = Stats()
            for lo in range(0, 2 * B, B):
                seeds = synth.make_seeds(400 + lo, B)
                res = run(fh, head, dev_tensor(H[lo:lo + B]), B, p, mode, 0.9, seeds_dev(seeds))
                assert res["path"] == PATH_STREAM_ALL
                sc = cs.oracle_scores_many(H64[lo:lo + B])
                for r in range(B):
                    check_row(cs, res, r, H64[lo + r], sc[r], p, mode, 0.9, int(seeds[r]), st)
    assert fh.flashhead_query(head.handle, 9) == 0


@pytest.mark.parametrize("B", [50, 64])
def test_wide_engine_ragged(fh, B):
    """d = 2048 with four 16-column tiles of H (B = 49-64), greedy: the
    engine's two-items-per-wave unrolled K walk, in the all-cluster stream
    and in the dense head.  c = 47 clusters: a partial last stage-1 item and
    a partial last unit of items; B = 50: the last tile's rows past the batch
    (read as zeros) must not reach any output."""
    cs = case(1, c=47, b=16, d=2048, seed=81)
    head = prepare(fh, cs, B, 47, fh.FH_FLAG_STREAM_ALL)
    dense = fh.DenseHead(cs.E_dev, max_batch=B)
    H, H64 = cs.hidden(B, offset=9)
    x = dev_tensor(H)
    sc = cs.oracle_scores_many(H64)
    for p in (1, 12, 47):
        st = Stats()
        res = run(fh, head, x, B, p, "greedy")
        assert res["path"] == PATH_STREAM_ALL
        for r in range(B):
            check_row(cs, res, r, H64[r], sc[r], p, "greedy", 1.0, 0, st)
        assert st.rows == B
    lse = torch.empty(B, dtype=torch.float32, device="cuda")
    toks = dense(x, out_lse=lse).cpu().numpy()
    lses = lse.cpu().numpy()
    for r in range(B):
        z = ref.dense_logits(cs.rows, cs.wl.v, H64[r])
        tok, m2, want_lse, keys = ref.decode_tokens(np.arange(cs.wl.v), z, "greedy", 1.0, 0)
        if m2 > 1e-3:
            assert toks[r] == tok
        else:
            assert keys[toks[r]] >= keys.max() - 1e-3
        assert lses[r] == pytest.approx(want_lse, abs=1e-3, rel=1e-5)
    assert fh.flashhead_query(head.handle, 9) == 0


def test_stream_all_equal_scores_pick_lowest_ids(fh):
    """h = 0: every score and logit is 0; ties go to the lowest ids."""
    cs = case(1, c=50, b=16, d=256)
    head = prepare(fh, cs, 4, 20, fh.FH_FLAG_STREAM_ALL)
    H = np.zeros((4, cs.wl.d), dtype=cs.head.E.dtype)
    res = run(fh, head, dev_tensor(H), 4, 20, "greedy")
    assert res["path"] == PATH_STREAM_ALL
    T = ref.candidate_tokens(np.arange(20), cs.head.c2t)
    for r in range(4):
        assert np.array_equal(np.sort(res["clusters"][r]), np.arange(20))
        assert res["tokens"][r] == T.min()
    assert fh.flashhead_query(head.handle, 9) == 0


@pytest.mark.parametrize("mode,tau,eps", [("greedy", 1.0, 0.1), ("sample", 0.7, 0.02)])
def test_stream_all_adaptive(fh, mode, tau, eps):
    """The adaptive probe count on path 4: p' per row from the plain
    stage-1 scores, the selection and fold at p', entries past p' unused."""
    cs = case(3)
    head = prepare(fh, cs, 16, 512, fh.FH_FLAG_STREAM_ALL)
    st = Stats()
    exact = 0
    for step in range(2):
        H, H64 = cs.hidden(16, offset=3100 + 16 * step)
        seeds = synth.make_seeds(60 + step, 16)
        res = run(fh, head, dev_tensor(H), 16, 512, mode, tau, seeds_dev(seeds),
                  adaptive=(4, eps))
        assert res["path"] == PATH_STREAM_ALL
        sc = cs.oracle_scores_many(H64)
        for r in range(16):
            rt = 1.0 / tau if mode == "sample" else 1.0
            pg = int(res["p"][r])
            lo, hi = count_bounds(sc[r], rt, eps, 4, 512)
            assert lo <= pg <= hi
            want, _ = ref.adaptive_p(sc[r], tau if mode == "sample" else 1.0, eps, 4, 512)
            exact += pg == want
            assert np.all(res["clusters"][r][pg:] == UNUSED)
            check_row(cs, res, r, H64[r], sc[r], pg, mode, tau, int(seeds[r]), st)
    assert fh.flashhead_query(head.handle, 9) == 0
    assert exact >= 30
    report(f"{cs.wl.name} adaptive {mode} B=16 stream-all", st)
