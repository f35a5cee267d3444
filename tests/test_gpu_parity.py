"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Inputs come from the seeded generator; the oracle computes everything it
compares from those inputs alone.  Where the GPU needs prepare-time data
that the oracle defines (centroid means, INT4 codes), the parity tests feed
the oracle's values to both sides, and separate tests compare the library's
own prepare-time results with the oracle's.
"""
import math

import numpy as np
import pytest

from oracle import flashhead_ref as ref
from two_stage_retrieval_amd import synth

from .parity import Stats, check_row

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="session")
def fh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from two_stage_retrieval_amd import binding
    return binding


def dev_tensor(arr):
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


class Case:
    """A workload with its oracle-side data, built once per session."""

    def __init__(self, wid, **over):
        self.head = synth.make_head(wid, **over)
        self.wl = self.head.wl
        self.dtype = self.wl.dtype
        self.rows = ref.rows_accessor(self.head.E, self.dtype)
        if self.head.C_given is not None:
            self.C64 = ref.as_f64(self.head.C_given, self.dtype)
            self.C_store = self.head.C_given
        else:
            self.C64 = ref.centroid_means(self.rows, self.head.c2t)
            self.C_store = (ref.bf16_bits_of(self.C64) if self.dtype == "bf16"
                            else self.C64.astype(np.float32))
        self.E_dev = dev_tensor(self.head.E)
        self.C_dev = dev_tensor(self.C_store)
        self.int4 = None
        if self.wl.quant == "int4_g128":
            self.int4 = ref.int4_quantize(self.C64)

    def hidden(self, n, offset=0):
        H = synth.make_hidden(self.head, n, offset=offset)
        return H, ref.as_f64(H, self.dtype)

    def prepare(self, fh, max_batch, max_p, with_C=True, quant=None, flags=0):
        # quant: a FH_QUANT_* code, or None for the workload's own
        if quant is None:
            quant = (fh.FH_QUANT_INT4_G128 if self.wl.quant == "int4_g128"
                     else fh.FH_QUANT_NONE)
        q = quant
        return fh.FlashHead(self.E_dev, self.head.c2t,
                            self.C_dev if with_C else None, quant=q,
                            max_batch=max_batch, max_p=max_p, flags=flags)

    def oracle_scores(self, h64):
        if self.int4 is not None:
            return ref.stage1_scores_int4(self.int4[0], self.int4[1], h64)
        return ref.stage1_scores(self.C64, h64)

    def oracle_scores_many(self, H64):
        """The oracle's stage-1 scores of several rows at once: the same sums
        (INT4: per group, integer codes times h, then times the group's
        scale), as matrix products; the first row is also scored by the
        oracle's own function and must agree."""
        if self.int4 is None:
            out = (self.C64 @ H64.T).T
        else:
            if not hasattr(self, "_q64"):
                q, _ = self.int4
                self._q64 = np.ascontiguousarray(q, dtype=np.float64)
            q, sc = self._q64, np.asarray(self.int4[1], np.float64)
            c, d = q.shape
            G = d // 128
            out = np.zeros((H64.shape[0], c))
            for g in range(G):
                cols = slice(128 * g, 128 * g + 128)
                out += (q[:, cols] @ H64[:, cols].T).T * sc[:, g]
        assert np.allclose(out[0], self.oracle_scores(H64[0]), rtol=0, atol=1e-9)
        return out


_CASES = {}


def case(wid, **over):
    key = (wid, tuple(sorted(over.items())))
    if key not in _CASES:
        _CASES[key] = Case(wid, **over)
    return _CASES[key]


def run_debug(fhmod, head, H_dev, B, p, mode, tau=1.0, seeds=None):
    c, b = head.c, head.b
    dbg = {
        "scores": torch.empty(B, c, dtype=torch.float32, device="cuda"),
        "clusters": torch.empty(B, p, dtype=torch.int32, device="cuda"),
        "cand_ids": torch.empty(B, p * b, dtype=torch.int32, device="cuda"),
        "cand_logits": torch.empty(B, p * b, dtype=torch.float32,
                                   device="cuda"),
    }
    lse = None
    if mode == "greedy":
        out = head.greedy(H_dev, p, debug=dbg)
    else:
        lse = torch.empty(B, dtype=torch.float32, device="cuda")
        out = head.sample(H_dev, p, tau, seeds, out_lse=lse, debug=dbg)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in dbg.items()}
    res["tokens"] = out.cpu().numpy()
    # the single launch lists its clusters in two ascending runs
    res["runs"] = 2 if fhmod.flashhead_query(head.handle, 10) == 1 else 1
    if lse is not None:
        res["lse"] = lse.cpu().numpy()
    return res


def check_one(cs, res, r, h64, p, mode="greedy", tau=1.0, seed=0, stats=None,
              score_tol=None, scores=None):
    """Rules R1-R4 for batch row r of one GPU step (res from run_debug)."""
    if scores is None:
        scores = cs.oracle_scores(h64)
    tol = score_tol if score_tol is not None else (
        1e-4 if cs.dtype == "f32" else 2e-2)
    assert np.max(np.abs(res["scores"][r] - scores)) <= tol
    keys1 = ref.select_keys(scores, mode, tau, seed)
    check_row(gpu_token=res["tokens"][r], gpu_sel=res["clusters"][r],
              gpu_ids=res["cand_ids"][r], gpu_logits=res["cand_logits"][r],
              keys1=keys1, p=p, c2t=cs.head.c2t, rows=cs.rows, h64=h64,
              dtype=cs.dtype, mode=mode, tau=tau, seed=seed, stats=stats,
              runs=res.get("runs", 1))
    if mode == "sample":
        z = ref.exact_logits(cs.rows, res["cand_ids"][r], h64)
        assert res["lse"][r] == pytest.approx(ref.logsumexp(z / tau),
                                              abs=1e-3, rel=1e-5)


def check_batch(cs, res, H64, p, mode="greedy", tau=1.0, seeds=None,
                stats=None, score_tol=None):
    for r in range(H64.shape[0]):
        seed = int(seeds[r]) if seeds is not None else 0
        check_one(cs, res, r, H64[r], p, mode, tau, seed, stats, score_tol)


def check_steps(cs, steps, p, mode="greedy", tau=1.0, stats=None,
                score_tol=None, workers=8):
    """Rules R1-R4 over many GPU steps at once: steps is a list of
    (res, H64 rows, seeds or None).  The oracle's stage-1 scores come from
    one product per step; the per-row checks run on a pool of host threads
    (numpy releases the interpreter lock in its kernels).  Each row gets its
    own counters, merged in row order afterwards."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    sc = cs.oracle_scores_many(np.concatenate([H64 for _, H64, _ in steps]))
    i = 0
    for res, H64, seeds in steps:
        for r in range(H64.shape[0]):
            seed = int(seeds[r]) if seeds is not None else 0
            jobs.append((res, r, H64[r], seed, sc[i]))
            i += 1

    def one(job):
        res, r, h64, seed, scores = job
        st = Stats()
        check_one(cs, res, r, h64, p, mode, tau, seed, st, score_tol, scores)
        return st

    with ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(one, jobs))
    if stats is not None:
        for st in parts:
            stats.merge(st)


def report(name, st):
    """One line per parity run, collected into the per-workload table."""
    print(f"PARITY {name}: {st}", flush=True)


# --------------------------------------------------------------------------
# tiny fp32 workload
# --------------------------------------------------------------------------

@pytest.mark.parametrize("p", [8, 1, 64])
def test_tiny_greedy_parity(fh, p):
    cs = case(0)
    head = cs.prepare(fh, max_batch=4, max_p=64)
    H, H64 = cs.hidden(256)
    st = Stats()
    for lo in range(0, 256, 4):
        res = run_debug(fh, head, dev_tensor(H[lo:lo + 4]), 4, p, "greedy")
        check_batch(cs, res, H64[lo:lo + 4], p, stats=st)
    print(st)
    assert st.rows == 256


@pytest.mark.parametrize("tau", [0.7, 1.0])
def test_tiny_sample_parity(fh, tau):
    cs = case(0)
    head = cs.prepare(fh, max_batch=4, max_p=64)
    H, H64 = cs.hidden(64)
    st = Stats()
    for lo in range(0, 64, 4):
        seeds = synth.make_seeds(lo, 4)
        res = run_debug(fh, head, dev_tensor(H[lo:lo + 4]), 4, 8, "sample",
                        tau, torch.from_numpy(seeds.view(np.int64)).cuda())
        check_batch(cs, res, H64[lo:lo + 4], 8, "sample", tau, seeds,
                    stats=st)
    print(st)


def test_tiny_p_equals_c_matches_dense(fh):
    cs = case(0)
    head = cs.prepare(fh, max_batch=8, max_p=64)
    dense = fh.DenseHead(cs.E_dev, max_batch=8)
    H, H64 = cs.hidden(64)
    for lo in range(0, 64, 8):
        Hd = dev_tensor(H[lo:lo + 8])
        seeds = synth.make_seeds(7, 8) + np.uint64(lo)
        sd = torch.from_numpy(seeds.view(np.int64)).cuda()
        g1 = head.greedy(Hd, 64).cpu().numpy()
        g2 = dense(Hd).cpu().numpy()
        lse1 = torch.empty(8, device="cuda")
        lse2 = torch.empty(8, device="cuda")
        s1 = head.sample(Hd, 64, 0.7, sd, out_lse=lse1).cpu().numpy()
        s2 = dense(Hd, fh.FH_MODE_SAMPLE, 0.7, sd,
                   out_lse=lse2).cpu().numpy()
        assert np.array_equal(g1, g2) and np.array_equal(s1, s2)
        for r in range(8):
            tok, m2, lse, _ = ref.dense_head(cs.rows, cs.wl.v, H64[r + lo])
            if m2 > 1e-3:
                assert g2[r] == tok
            tok, m2, lse, _ = ref.dense_head(cs.rows, cs.wl.v, H64[r + lo],
                                             "sample", 0.7, int(seeds[r]))
            if m2 > 1e-3:
                assert s2[r] == tok
            assert lse2[r].item() == pytest.approx(lse, abs=1e-3, rel=1e-5)
            assert lse1[r].item() == pytest.approx(lse, abs=1e-3, rel=1e-5)


# --------------------------------------------------------------------------
# Llama-3.2-1B-shaped head (bf16)
# --------------------------------------------------------------------------

def test_llama_centroids_computed_on_device(fh):
    cs = case(1)
    head = cs.prepare(fh, max_batch=1, max_p=512, with_C=False)
    got = ref.decode_bf16(head.centroids())
    want = cs.C64
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    diff = np.abs(got - want)
    assert np.all(diff <= ulp + 1e-30), "centroid off by more than one ulp"
    frac = np.mean(diff > 0)
    print(f"centroid elements differing by one bf16 ulp: {frac:.2e}")
    assert frac < 1e-3


def test_llama_greedy_parity(fh):
    """All 1024 hidden vectors of the Llama-shaped workload, batch 1 (the
    single-launch decode), each call checked, self-check word included."""
    cs = case(1)
    head = cs.prepare(fh, max_batch=1, max_p=512)
    H, H64 = cs.hidden(1024)
    st = Stats()
    steps = []
    for i in range(1024):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, 512, "greedy")
        steps.append((res, H64[i:i + 1], None))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 512, stats=st)
    report("llama3.2-1b-head greedy B=1", st)
    assert st.rows == 1024


@pytest.mark.parametrize("B", [64, 1])
def test_llama_dense_head(fh, B):
    """The in-library dense head on 64 hidden vectors: greedy, and sampled
    at both temperatures with its lse, one batch of 64 (matrix cores) or 64
    calls of one row (row-dot)."""
    cs = case(1)
    n = 64
    dense = fh.DenseHead(cs.E_dev, max_batch=B)
    H, H64 = cs.hidden(n, offset=100)
    seeds = synth.make_seeds(11, n)
    out = {}
    for mode, tau in (("greedy", 1.0), ("sample", 0.7), ("sample", 1.0)):
        toks = np.empty(n, dtype=np.int64)
        lses = np.empty(n)
        for lo in range(0, n, B):
            Hd = dev_tensor(H[lo:lo + B])
            lse = torch.empty(B, dtype=torch.float32, device="cuda")
            if mode == "greedy":
                t = dense(Hd, out_lse=lse)
            else:
                sd = torch.from_numpy(seeds[lo:lo + B].view(np.int64)).cuda()
                t = dense(Hd, fh.FH_MODE_SAMPLE, tau, sd, out_lse=lse)
            toks[lo:lo + B] = t.cpu().numpy()
            lses[lo:lo + B] = lse.cpu().numpy()
        out[(mode, tau)] = (toks, lses)
    st = Stats()
    for r in range(n):
        z = ref.dense_logits(cs.rows, cs.wl.v, H64[r])
        for (mode, tau), (toks, lses) in out.items():
            st.rows += 1
            tok, m2, lse, keys = ref.decode_tokens(np.arange(cs.wl.v), z, mode,
                                                   tau, int(seeds[r]))
            if m2 > 1e-3:
                assert toks[r] == tok
            else:
                st.tok_band += 1
                st.tok_diff += int(toks[r] != tok)
                assert keys[toks[r]] >= keys.max() - 1e-3
            assert lses[r] == pytest.approx(lse, abs=1e-3, rel=1e-5)
    report(f"llama3.2-1b dense head greedy+sample(0.7,1.0) B={B}", st)


@pytest.mark.parametrize("tau", [0.7, 1.0])
def test_llama_sample_b16_parity(fh, tau):
    """16 steps of 16 rows per temperature, a Philox key per (step, row)."""
    cs = case(3)
    head = cs.prepare(fh, max_batch=16, max_p=512)
    st = Stats()
    steps = []
    for step in range(16):
        H, H64 = cs.hidden(16, offset=16 * step)
        seeds = synth.make_seeds(step, 16)
        res = run_debug(fh, head, dev_tensor(H), 16, 512, "sample", tau,
                        torch.from_numpy(seeds.view(np.int64)).cuda())
        steps.append((res, H64, seeds))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 512, "sample", tau, stats=st)
    report(f"llama3.2-1b-head-sample-b16 tau={tau} B=16", st)
    assert st.rows == 256


@pytest.mark.parametrize("path", [3, 4])
def test_llama_greedy_b64_parity(fh, path):
    """16 batches of 64 rows on each batched matrix-core path (3: select
    first; 4: the all-cluster stream, whose debug candidates come from a
    second gather of the selected rows)."""
    cs = case(2)
    flags = fh.FH_FLAG_SELECT_FIRST if path == 3 else fh.FH_FLAG_STREAM_ALL
    head = cs.prepare(fh, max_batch=64, max_p=512, flags=flags)
    st = Stats()
    steps = []
    for i in range(16):
        H, H64 = cs.hidden(64, offset=64 * i)
        res = run_debug(fh, head, dev_tensor(H), 64, 512, "greedy")
        assert fh.flashhead_query(head.handle, 10) == path
        steps.append((res, H64, None))
    assert fh.flashhead_query(head.handle, 9) == 0
    check_steps(cs, steps, 512, stats=st)
    report(f"llama3.2-1b-head-b64 greedy B=64 path {path}", st)
    assert st.rows == 1024


# --------------------------------------------------------------------------
# Gemma-3-1B-shaped head with INT4 stage 1
# --------------------------------------------------------------------------

def unpack_int4(codes, scales, c, d):
    G, ntiles = d // 128, (c + 15) // 16
    by = codes.reshape(ntiles, G, 64, 16)
    lo = (by & 0xF).astype(np.int8)
    hi = (by >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    q = np.zeros((ntiles * 16, d), dtype=np.int8)
    for t in range(ntiles):
        for g in range(G):
            for lane in range(64):
                row = 16 * t + (lane % 16)
                col0 = 128 * g + 32 * (lane // 16)
                q[row, col0:col0 + 32:2] = lo[t, g, lane]
                q[row, col0 + 1:col0 + 32:2] = hi[t, g, lane]
    s = ref.decode_bf16(scales.reshape(ntiles, G, 16).transpose(0, 2, 1)
                        .reshape(ntiles * 16, G))
    return q[:c], s[:c]


def test_gemma_int4_codes_match_oracle(fh):
    cs = case(4)
    head = cs.prepare(fh, max_batch=1, max_p=1024)
    codes, scales = head.int4()
    q, s = unpack_int4(codes, scales, cs.wl.c, cs.wl.d)
    assert np.array_equal(q, cs.int4[0])
    assert np.array_equal(s, cs.int4[1])


@pytest.mark.parametrize("B,flags", [(1, 0), (32, "SELECT_FIRST"), (32, "STREAM_ALL")])
def test_gemma_int4_greedy_parity(fh, B, flags):
    """All 1024 hidden vectors at batch 1; 8 batches of 32 on each batched
    path."""
    cs = case(4)
    fl = getattr(fh, "FH_FLAG_" + flags) if flags else 0
    head = cs.prepare(fh, max_batch=B, max_p=1024, flags=fl)
    st = Stats()
    n = 1024 if B == 1 else 8 * 32
    H, H64 = cs.hidden(n)
    steps = []
    for lo in range(0, n, B):
        res = run_debug(fh, head, dev_tensor(H[lo:lo + B]), B, 1024, "greedy")
        steps.append((res, H64[lo:lo + B], None))
    assert fh.flashhead_query(head.handle, 9) == 0
    assert fh.flashhead_query(head.handle, 10) == {0: 1, "SELECT_FIRST": 3, "STREAM_ALL": 4}[flags]
    check_steps(cs, steps, 1024, stats=st, score_tol=2e-2)
    report(f"gemma3-1b-head-int4 greedy B={B}" + (f" path {fh.flashhead_query(head.handle, 10)}"
                                                   if B > 1 else ""), st)
    assert st.rows == n


# --------------------------------------------------------------------------
# batch 1 across p (the selection inside stage 1)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("p", [1, 2, 64])
def test_batch1_tiny_all_p(fh, p):
    cs = case(0)
    head = cs.prepare(fh, max_batch=1, max_p=64)
    H, H64 = cs.hidden(32, offset=50)
    for i in range(32):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, p, "greedy")
        check_batch(cs, res, H64[i:i + 1], p)
    assert fh.flashhead_query(head.handle, 9) == 0


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("p", [1, 7, 50])
def test_ragged_small_head(fh, p):
    """c = 50 (not a multiple of any tile), b = 8, d = 128, B = 3."""
    cs = case(1, c=50, b=8, d=128, seed=77)
    head = cs.prepare(fh, max_batch=3, max_p=50)
    H, H64 = cs.hidden(9)
    for lo in range(0, 9, 3):
        res = run_debug(fh, head, dev_tensor(H[lo:lo + 3]), 3, p, "greedy")
        check_batch(cs, res, H64[lo:lo + 3], p)


@pytest.mark.parametrize("p", [1, 300])
def test_many_clusters_separate_select_kernel(fh, p):
    """c = 20000 > 16384: selection runs in its own kernel (b = 2, d = 128)."""
    cs = case(1, c=20000, b=2, d=128, seed=91)
    head = cs.prepare(fh, max_batch=2, max_p=300)
    H, H64 = cs.hidden(4)
    for lo in range(0, 4, 2):
        res = run_debug(fh, head, dev_tensor(H[lo:lo + 2]), 2, p, "greedy")
        check_batch(cs, res, H64[lo:lo + 2], p)
    assert fh.flashhead_query(head.handle, 9) == 0


@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("wid, over, p", [(0, (), None), (1, (), None),
                                          (1, (("c", 50), ("b", 16), ("d", 256)), 20)])
def test_all_equal_scores_pick_lowest_ids(fh, wid, over, p, B):
    """h = 0: every score and logit is 0; ties go to the lowest ids (also
    with c not a multiple of the keys each selecting thread holds)."""
    cs = case(wid, **dict(over))
    p = p or cs.wl.p
    head = cs.prepare(fh, max_batch=B, max_p=p)
    H = np.zeros((B, cs.wl.d), dtype=cs.head.E.dtype)
    res = run_debug(fh, head, dev_tensor(H), B, p, "greedy")
    for r in range(B):
        assert np.array_equal(np.sort(res["clusters"][r]), np.arange(p))
        T = ref.candidate_tokens(np.arange(p), cs.head.c2t)
        assert res["tokens"][r] == T.min()
    assert fh.flashhead_query(head.handle, 9) == 0


def test_repeated_calls_are_deterministic(fh):
    cs = case(1)
    head = cs.prepare(fh, max_batch=4, max_p=512)
    H, _ = cs.hidden(4)
    Hd = dev_tensor(H)
    a = run_debug(fh, head, Hd, 4, 512, "greedy")
    b = run_debug(fh, head, Hd, 4, 512, "greedy")
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_call_errors_return_status(fh):
    cs = case(0)
    head = cs.prepare(fh, max_batch=2, max_p=8)
    H, _ = cs.hidden(3)
    Hd = dev_tensor(H)
    out = torch.empty(3, dtype=torch.int32, device="cuda")
    with pytest.raises(fh.FlashHeadError) as e:
        fh.flashhead_greedy(head.handle, Hd, 3, 8, out)
    assert e.value.status == fh.FH_ERR_INVALID_ARG
    for p in (0, 9):
        with pytest.raises(fh.FlashHeadError):
            fh.flashhead_greedy(head.handle, Hd, 2, p, out)
    sd = torch.zeros(2, dtype=torch.int64, device="cuda")
    for tau in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(fh.FlashHeadError):
            fh.flashhead_sample(head.handle, Hd, 2, 8, tau, sd, out)
    with pytest.raises(fh.FlashHeadError):
        fh.flashhead_sample(head.handle, Hd, 2, 8, 1.0, None, out)


# --------------------------------------------------------------------------
# sampling distribution on the tiny workload (1e5 draws)
# --------------------------------------------------------------------------

def _pooled_chisq(obs, prob):
    """Chi-square p-value of counts against probabilities; cells with an
    expected count below 5 are pooled into one."""
    from scipy import stats
    exp = np.asarray(prob, dtype=np.float64) * obs.sum()
    keep = exp >= 5
    o = np.append(obs[keep], obs[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return stats.chisquare(o, e * o.sum() / e.sum()).pvalue



def test_tiny_sampling_chisquare_p_equals_c(fh):
    cs = case(0)
    head = cs.prepare(fh, max_batch=64, max_p=64)
    H, H64 = cs.hidden(1, offset=5)
    tau = 0.7
    Hd = dev_tensor(np.repeat(H, 64, axis=0))
    n_calls = 100_000 // 64 + 1
    counts = np.zeros(cs.wl.v)
    out = torch.empty(64, dtype=torch.int32, device="cuda")
    outs = []
    for j in range(n_calls):
        seeds = synth.make_seeds(j, 64)
        head.sample(Hd, 64, tau, torch.from_numpy(seeds.view(np.int64)).cuda(),
                    out=out)
        outs.append(out.clone())
    toks = torch.cat(outs).cpu().numpy()[:100_000]
    np.add.at(counts, toks, 1)
    z = ref.dense_logits(cs.rows, cs.wl.v, H64[0]) / tau
    prob = np.exp(z - z.max())
    prob /= prob.sum()
    assert _pooled_chisq(counts, prob) > 1e-3


@pytest.mark.parametrize("B,n", [(64, 100_000), (1, 20_000)])
def test_tiny_head_sampling_matches_exact_marginal(fh, B, n):
    """v = 24, c = 6, b = 4, p = 2 (fp32, d = 8): the distribution of the
    GPU's sampled tokens against the exact marginal sum_S P(S) softmax_S(z/tau)
    ([notes] Module 2 sampling mode and Formula 3), P(S) from enumerating the
    ordered successive draws without replacement.  B = 64 rows per call take
    the two-launch path, B = 1 the single launch."""
    from scipy import special

    from .test_oracle_pins import _plackett_luce_set_probs
    head = synth.make_head(0, v=24, c=6, b=4, d=8, seed=31)
    H = synth.make_hidden(head, 1, offset=3)
    h64 = H[0].astype(np.float64)
    C64 = head.C_given.astype(np.float64)
    tau, p = 1.0, 2
    s = ref.stage1_scores(C64, h64)
    z = ref.exact_logits(ref.rows_accessor(head.E, "f32"), np.arange(24), h64)
    marg = np.zeros(24)
    for S, pS in _plackett_luce_set_probs(np.exp(s / tau), p).items():
        T = ref.candidate_tokens(np.array(S), head.c2t)
        marg[T] += pS * special.softmax(z[T] / tau)
    assert marg.sum() == pytest.approx(1.0)
    fhh = fh.FlashHead(dev_tensor(head.E), head.c2t, dev_tensor(head.C_given),
                       max_batch=B, max_p=p)
    Hd = dev_tensor(np.repeat(H, B, axis=0))
    seeds = torch.from_numpy((np.arange(n, dtype=np.uint64) + (np.uint64(77) << np.uint64(32)))
                             .view(np.int64)).cuda()
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    for lo in range(0, n, B):
        fhh.sample(Hd, p, tau, seeds[lo:lo + B], out=out[lo:lo + B])
    toks = out.cpu().numpy()
    assert fh.flashhead_query(fhh.handle, 9) == 0
    assert fh.flashhead_query(fhh.handle, 10) == (2 if B > 1 else 1)
    counts = np.bincount(toks, minlength=24)
    assert counts.sum() == n and np.all(counts[marg == 0] == 0)
    assert _pooled_chisq(counts, marg) > 1e-3
    fhh.close()


def test_tiny_sampling_homogeneity_p8(fh):
    """p = 8: GPU draws vs oracle draws (disjoint seeds), chi-square test of
    homogeneity on the token counts."""
    from scipy import stats
    cs = case(0)
    head = cs.prepare(fh, max_batch=64, max_p=8)
    H, H64 = cs.hidden(1, offset=9)
    tau = 1.0
    Hd = dev_tensor(np.repeat(H, 64, axis=0))
    out = torch.empty(64, dtype=torch.int32, device="cuda")
    outs = []
    for j in range(100_000 // 64 + 1):
        seeds = synth.make_seeds(j, 64)
        head.sample(Hd, 8, tau, torch.from_numpy(seeds.view(np.int64)).cuda(),
                    out=out)
        outs.append(out.clone())
    g = torch.cat(outs).cpu().numpy()[:100_000]
    n_or = 20_000
    o = np.empty(n_or, dtype=np.int64)
    for i in range(n_or):
        seed = int(synth.make_seeds(10**6 + i, 1)[0])
        o[i] = ref.flashhead_step(cs.rows, cs.head.c2t, H64[0], 8,
                                  C_f64=cs.C64, mode="sample", tau=tau,
                                  seed=seed).token
    toks = np.union1d(np.unique(g), np.unique(o))
    gc = np.array([np.sum(g == t) for t in toks], dtype=np.float64)
    oc = np.array([np.sum(o == t) for t in toks], dtype=np.float64)
    exp_small = (gc + oc) * (n_or / (len(g) + n_or)) < 5
    table = np.array([np.append(gc[~exp_small], gc[exp_small].sum()),
                      np.append(oc[~exp_small], oc[exp_small].sum())])
    table = table[:, table.sum(axis=0) > 0]
    assert stats.chi2_contingency(table)[1] > 1e-3


# --------------------------------------------------------------------------
# mean-shifted INT4 centroids
# --------------------------------------------------------------------------

def _mean_shifted(cs):
    """The case with the oracle's mean-shifted codes in place of the plain."""
    import copy
    cm = copy.copy(cs)
    cm.int4 = ref.int4_quantize(cs.C64, shift=ref.int4_mean_shift(cs.C64))
    return cm


def test_gemma_int4_mean_shift_codes_and_parity(fh):
    cs = case(4)
    cm = _mean_shifted(cs)
    head = cs.prepare(fh, max_batch=32, max_p=1024, quant=fh.FH_QUANT_INT4_G128_MEAN)
    codes, scales = head.int4()
    q, s = unpack_int4(codes, scales, cs.wl.c, cs.wl.d)
    assert np.array_equal(q, cm.int4[0])
    assert np.array_equal(s, cm.int4[1])
    st = Stats()
    H, H64 = cs.hidden(8, offset=1700)
    for i in range(8):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, 1024, "greedy")
        check_batch(cm, res, H64[i:i + 1], 1024, stats=st, score_tol=2e-2)
    H32, H32_64 = cs.hidden(32, offset=1800)
    res = run_debug(fh, head, dev_tensor(H32), 32, 1024, "greedy")
    check_batch(cm, res, H32_64, 1024, stats=st, score_tol=2e-2)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


def test_int4_mean_shift_flips_fewer_boundary_clusters(fh):
    # rows that share a direction (as a trained output embedding's do): the
    # plain codes spend their range on the shared part, the shifted ones do
    # not; count the clusters each INT4 selection swaps against the selection
    # from the unquantized bf16 centroids
    cs = case(4, common=8.0)
    H, H64 = cs.hidden(32, offset=1900)
    p = 1024
    flips = {}
    for name, quant in (("plain", fh.FH_QUANT_INT4_G128), ("mean", fh.FH_QUANT_INT4_G128_MEAN)):
        head = cs.prepare(fh, max_batch=32, max_p=p, quant=quant)
        res = run_debug(fh, head, dev_tensor(H), 32, p, "greedy")
        n = 0
        for r in range(32):
            ref_set = set(ref.order_desc(cs.C64 @ H64[r])[:p].tolist())
            n += len(set(res["clusters"][r].tolist()) - ref_set)
        flips[name] = n / (32 * p)
        head.close()
    print("boundary swaps per selected cluster vs bf16:", flips)
    assert flips["mean"] < flips["plain"]
