"""Stage 2 over the caller's E (FH_FLAG_BORROW_E) against stage 2 over the
cluster-major copy: the same candidate rows in the same order, so tokens,
candidates, logits and lse agree bit for bit on every kernel path, and the
borrowed head also passes the oracle's rules."""
import numpy as np
import pytest

from two_stage_retrieval_amd import synth

from .parity import Stats
from .test_gpu_parity import case, check_batch, dev_tensor, fh, run_debug  # noqa: F401

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _pair(fhmod, cs, max_batch, max_p):
    copy = cs.prepare(fhmod, max_batch=max_batch, max_p=max_p)
    quant = (fhmod.FH_QUANT_INT4_G128 if cs.wl.quant == "int4_g128" else fhmod.FH_QUANT_NONE)
    borrowed = fhmod.FlashHead(cs.E_dev, cs.head.c2t, cs.C_dev, quant=quant,
                               max_batch=max_batch, max_p=max_p, flags=fhmod.FH_FLAG_BORROW_E)
    return copy, borrowed


def _same(a, b):
    for k in ("tokens", "clusters", "cand_ids", "cand_logits", "scores"):
        assert np.array_equal(a[k], b[k]), k
    if "lse" in a:
        assert np.array_equal(a["lse"], b["lse"])


@pytest.mark.parametrize("wid,B,p,mode", [(1, 1, 512, "greedy"), (1, 1, 512, "sample"),
                                          (4, 1, 1024, "greedy"), (2, 64, 512, "greedy"),
                                          (3, 16, 512, "sample"), (4, 32, 1024, "greedy")])
def test_borrowed_rows_match_the_copy(fh, wid, B, p, mode):
    cs = case(wid)
    copy, borrowed = _pair(fh, cs, B, p)
    E_bytes = cs.wl.v * cs.wl.d * 2
    assert (fh.flashhead_query(copy.handle, 8) - fh.flashhead_query(borrowed.handle, 8)
            == E_bytes)
    st = Stats()
    for step in range(4 if B == 1 else 1):
        H, H64 = cs.hidden(B, offset=2100 + step * B)
        seeds = synth.make_seeds(30 + step, B)
        sd = torch.from_numpy(seeds.view(np.int64)).cuda()
        args = (B, p, mode, 0.8, sd) if mode == "sample" else (B, p, mode)
        a = run_debug(fh, copy, dev_tensor(H), *args)
        b = run_debug(fh, borrowed, dev_tensor(H), *args)
        assert fh.flashhead_query(copy.handle, 10) == fh.flashhead_query(borrowed.handle, 10)
        _same(a, b)
        check_batch(cs, b, H64, p, mode, 0.8, seeds if mode == "sample" else None, stats=st,
                    score_tol=2e-2)
    assert fh.flashhead_query(borrowed.handle, 9) == 0
    print(st)
    borrowed.close()


def test_borrowed_two_launch_path_and_monte_carlo(fh):
    cs = case(1, c=4096, b=16, d=128, seed=57)
    copy, borrowed = _pair(fh, cs, 1, 3000)
    H, H64 = cs.hidden(2, offset=5)
    for i in range(2):
        a = run_debug(fh, copy, dev_tensor(H[i:i + 1]), 1, 3000, "greedy")
        b = run_debug(fh, borrowed, dev_tensor(H[i:i + 1]), 1, 3000, "greedy")
        assert fh.flashhead_query(borrowed.handle, 10) == 2
        _same(a, b)
        check_batch(cs, b, H64[i:i + 1], 3000)
    # the Monte Carlo marginal reads the same rows
    x = dev_tensor(H[:1])
    seeds = torch.from_numpy((np.arange(256, dtype=np.uint64) + (np.uint64(9) << np.uint64(32)))
                             .view(np.int64)).cuda()
    toks = torch.from_numpy(np.arange(0, cs.wl.v, 997, dtype=np.int32)).cuda()
    la = torch.empty(256, device="cuda")
    lb = torch.empty(256, device="cuda")
    pa = copy.mc_marginal(x, 64, 0.9, seeds, toks, out_lse=la).cpu().numpy()
    pb = borrowed.mc_marginal(x, 64, 0.9, seeds, toks, out_lse=lb).cpu().numpy()
    assert np.array_equal(pa, pb) and torch.equal(la, lb)
    assert fh.flashhead_query(borrowed.handle, 9) == 0
    borrowed.close()
