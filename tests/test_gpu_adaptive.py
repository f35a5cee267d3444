"""The adaptive probe count on the GPU (through the C ABI) against the oracle:
per row, p' from the stage-1 scores (reading of the notes' "Potential
improvements"; see oracle.flashhead_ref.adaptive_p), then rules R1-R4 of the
step at p = p'.  Covered on every kernel path: the single launch (Llama
shape bf16, Gemma shape INT4), the batched matrix-core path, the two-launch
row-dot path and the separate selection kernel, greedy and sampling.

p' is an integer decided by floating point: where no score lies within 1e-3
(in units of s / tau) of the threshold it must equal the oracle's; otherwise
it may be any count the scores within that band allow."""
import math

import numpy as np
import pytest

from oracle import flashhead_ref as ref
from two_stage_retrieval_amd import synth

from .parity import Stats, check_row
from .test_gpu_parity import case, dev_tensor, fh  # noqa: F401

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

UNUSED = 0x7FFFFFFF


def run_adaptive(fhmod, head, H_dev, B, p_min, p_max, eps, mode, tau=1.0, seeds=None):
    c, b = head.c, head.b
    dbg = {
        "scores": torch.empty(B, c, dtype=torch.float32, device="cuda"),
        "clusters": torch.empty(B, p_max, dtype=torch.int32, device="cuda"),
        "cand_ids": torch.empty(B, p_max * b, dtype=torch.int32, device="cuda"),
        "cand_logits": torch.empty(B, p_max * b, dtype=torch.float32, device="cuda"),
    }
    out_p = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lse = None
    if mode == "greedy":
        out = head.greedy_adaptive(H_dev, p_min, p_max, eps, out_p=out_p, debug=dbg)
    else:
        lse = torch.empty(B, dtype=torch.float32, device="cuda")
        out = head.sample_adaptive(H_dev, p_min, p_max, eps, tau, seeds, out_lse=lse,
                                   out_p=out_p, debug=dbg)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in dbg.items()}
    res["tokens"] = out.cpu().numpy()
    res["p"] = out_p.cpu().numpy()
    res["path"] = fhmod.flashhead_query(head.handle, 10)
    if lse is not None:
        res["lse"] = lse.cpu().numpy()
    return res


def count_bounds(scores, rt, eps, p_min, p_max, band=1e-3):
    """The counts the rule allows when scores within `band` of the threshold
    may fall either way (clamped)."""
    x = np.asarray(scores, np.float64) * rt
    thr = x.max() - math.log(1.0 / eps)
    lo = int(np.count_nonzero(x >= thr + band))
    hi = int(np.count_nonzero(x >= thr - band))
    clamp = lambda n: min(max(n, p_min), p_max)  # noqa: E731
    return clamp(max(lo, 1)), clamp(hi)


def check_adaptive(cs, res, H64, p_min, p_max, eps, mode="greedy", tau=1.0, seeds=None,
                   stats=None, score_tol=None):
    b = cs.wl.b
    for r in range(H64.shape[0]):
        h64 = H64[r]
        scores = cs.oracle_scores(h64)
        tol = score_tol or (1e-4 if cs.dtype == "f32" else 2e-2)
        assert np.max(np.abs(res["scores"][r] - scores)) <= tol
        rt = 1.0 / tau if mode == "sample" else 1.0
        pg = int(res["p"][r])
        lo, hi = count_bounds(scores, rt, eps, p_min, p_max)
        assert lo <= pg <= hi, (r, pg, lo, hi)
        want, margin = ref.adaptive_p(scores, tau if mode == "sample" else 1.0, eps, p_min,
                                      p_max)
        if lo == hi:
            assert pg == want
        if stats is not None:
            stats.p_exact = getattr(stats, "p_exact", 0) + int(pg == want)
            stats.p_sum = getattr(stats, "p_sum", 0) + pg
        assert np.all(res["clusters"][r][pg:] == UNUSED)
        seed = int(seeds[r]) if seeds is not None else 0
        check_row(gpu_token=res["tokens"][r], gpu_sel=res["clusters"][r][:pg],
                  gpu_ids=res["cand_ids"][r][:pg * b], gpu_logits=res["cand_logits"][r][:pg * b],
                  keys1=ref.select_keys(scores, mode, tau, seed), p=pg, c2t=cs.head.c2t,
                  rows=cs.rows, h64=h64, dtype=cs.dtype, mode=mode, tau=tau, seed=seed,
                  stats=stats, runs=2 if res["path"] == 1 else 1)
        if mode == "sample":
            z = ref.exact_logits(cs.rows, res["cand_ids"][r][:pg * b], h64)
            assert res["lse"][r] == pytest.approx(ref.logsumexp(z / tau), abs=1e-3, rel=1e-5)


def _report(name, st, n):
    print(f"ADAPTIVE {name}: rows={st.rows} p_equal_oracle={st.p_exact} mean_p={st.p_sum / n:.1f} "
          f"set_in_band={st.set_band} set_differs={st.set_diff} tok_differs={st.tok_diff} "
          f"max_logit_err={st.max_logit_err:.3g}", flush=True)


@pytest.mark.parametrize("wid,mode,tau,eps,p_min,path", [
    (1, "greedy", 1.0, 0.1, 4, 1), (1, "sample", 0.7, 0.02, 4, 1),
    (4, "greedy", 1.0, 0.1, 8, 1), (4, "sample", 0.7, 0.02, 8, 1)])
def test_adaptive_single_launch(fh, wid, mode, tau, eps, p_min, path):
    cs = case(wid)
    p_max = cs.wl.p
    head = cs.prepare(fh, max_batch=1, max_p=p_max)
    n = 32
    H, H64 = cs.hidden(n, offset=3000)
    st = Stats()
    ps = []
    for i in range(n):
        seeds = synth.make_seeds(50 + i, 1)
        sd = torch.from_numpy(seeds.view(np.int64)).cuda()
        res = run_adaptive(fh, head, dev_tensor(H[i:i + 1]), 1, p_min, p_max, eps, mode, tau, sd)
        assert res["path"] == path
        assert fh.flashhead_query(head.handle, 11) == 0
        check_adaptive(cs, res, H64[i:i + 1], p_min, p_max, eps, mode, tau,
                       seeds if mode == "sample" else None, stats=st, score_tol=2e-2)
        ps.append(int(res["p"][0]))
    assert fh.flashhead_query(head.handle, 9) == 0
    assert len(set(ps)) > 4  # the count does adapt across these rows
    _report(f"{cs.wl.name} {mode} B=1", st, n)


@pytest.mark.parametrize("mode,tau,eps", [("greedy", 1.0, 0.1), ("sample", 0.7, 0.02)])
def test_adaptive_batched(fh, mode, tau, eps):
    cs = case(3)
    head = cs.prepare(fh, max_batch=16, max_p=512)
    st = Stats()
    for step in range(2):
        H, H64 = cs.hidden(16, offset=3100 + 16 * step)
        seeds = synth.make_seeds(60 + step, 16)
        sd = torch.from_numpy(seeds.view(np.int64)).cuda()
        res = run_adaptive(fh, head, dev_tensor(H), 16, 4, 512, eps, mode, tau, sd)
        assert res["path"] == 3
        check_adaptive(cs, res, H64, 4, 512, eps, mode, tau,
                       seeds if mode == "sample" else None, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    _report(f"{cs.wl.name} {mode} B=16", st, 32)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("shape", ["tiny-b4", "large-p", "many-clusters"])
def test_adaptive_two_launch_paths(fh, mode, shape):
    if shape == "tiny-b4":        # fp32 at batch 4: stage 1 selects, then row-dot
        cs, B, p_max, eps = case(0), 4, 64, 0.5
    elif shape == "large-p":      # batch 1 beyond the single launch's probes
        cs, B, p_max, eps = case(1, c=4096, b=16, d=128, seed=57), 1, 3000, 0.05
    else:                         # more clusters than stage 1 selects: own kernel
        cs, B, p_max, eps = case(1, c=20000, b=2, d=128, seed=91), 2, 300, 0.2
    head = cs.prepare(fh, max_batch=B, max_p=p_max)
    tau = 0.8
    st = Stats()
    H, H64 = cs.hidden(2 * B, offset=33)
    for lo in range(0, 2 * B, B):
        seeds = synth.make_seeds(70 + lo, B)
        sd = torch.from_numpy(seeds.view(np.int64)).cuda()
        res = run_adaptive(fh, head, dev_tensor(H[lo:lo + B]), B, 1, p_max, eps, mode, tau, sd)
        assert res["path"] == 2
        check_adaptive(cs, res, H64[lo:lo + B], 1, p_max, eps, mode, tau,
                       seeds if mode == "sample" else None, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


def test_adaptive_limits_match_fixed_p(fh):
    # eps toward 0 probes p_max clusters: the fixed-p step, id for id; eps = 1
    # probes the top score's cluster, clamped up to p_min
    cs = case(1)
    head = cs.prepare(fh, max_batch=16, max_p=512)
    for B in (1, 16):
        H, _ = cs.hidden(B, offset=3300)
        x = dev_tensor(H)
        seeds = torch.from_numpy(synth.make_seeds(80, B).view(np.int64)).cuda()
        out_p = torch.empty(B, dtype=torch.int32, device="cuda")
        a = head.greedy_adaptive(x, 1, 512, 1e-30, out_p=out_p).cpu().numpy()
        assert np.all(out_p.cpu().numpy() == 512)
        assert np.array_equal(a, head.greedy(x, 512).cpu().numpy())
        la, lb = torch.empty(B, device="cuda"), torch.empty(B, device="cuda")
        a = head.sample_adaptive(x, 1, 512, 1e-30, 0.9, seeds, out_lse=la).cpu().numpy()
        b = head.sample(x, 512, 0.9, seeds, out_lse=lb).cpu().numpy()
        assert np.array_equal(a, b) and torch.equal(la, lb)
        head.greedy_adaptive(x, 37, 512, 1.0, out_p=out_p)
        assert np.all(out_p.cpu().numpy() == 37)
    assert fh.flashhead_query(head.handle, 9) == 0
    # argument errors
    x = dev_tensor(cs.hidden(1)[0])
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    for p_min, p_max, eps in ((0, 512, 0.1), (600, 512, 0.1), (1, 513, 0.1), (1, 512, 0.0),
                              (1, 512, 1.5), (1, 512, float("nan"))):
        with pytest.raises(fh.FlashHeadError):
            fh.flashhead_greedy_adaptive(head.handle, x, 1, p_min, p_max, eps, out)
