"""dense_head_static: the dense head with the library's own fixed workspace
(for callers that cannot allocate), through the C ABI, against dense_head
with a caller's workspace: two calls in a row, the second on a smaller
input, each compared id for id and lse for lse (the same kernels run)."""
import numpy as np
import pytest

from two_stage_retrieval_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _both(fh, E, H, mode, tau, seeds):
    B = H.shape[0]
    dense = fh.DenseHead(E, max_batch=B)
    t_ref = torch.empty(B, dtype=torch.int32, device="cuda")
    l_ref = torch.empty(B, dtype=torch.float32, device="cuda")
    dense(H, mode, tau, seeds, out=t_ref, out_lse=l_ref)
    t = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lse = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    fh.dense_head_static(E, H, B, mode, tau, seeds, t, lse)
    torch.cuda.synchronize()
    return t_ref.cpu().numpy(), l_ref.cpu().numpy(), t.cpu().numpy(), lse.cpu().numpy()


def test_static_dense_head_matches_dense_head_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from two_stage_retrieval_amd import binding as fh
    # first call: the Llama-shaped head, 16 rows (the matrix-core kernels),
    # sampled; second call: the tiny fp32 head, one row (the row-dot kernel
    # with the arrival counters), greedy then sampled
    big = synth.make_head(1)
    Hb = _dev(synth.make_hidden(big, 16, offset=500))
    Eb = _dev(big.E)
    sb = torch.from_numpy(synth.make_seeds(3, 16).view(np.int64)).cuda()
    a = _both(fh, Eb, Hb, fh.FH_MODE_SAMPLE, 0.8, sb)
    assert np.array_equal(a[0], a[2]) and np.array_equal(a[1], a[3])
    small = synth.make_head(0)
    Hs = _dev(synth.make_hidden(small, 1, offset=9))
    Es = _dev(small.E)
    ss = torch.from_numpy(synth.make_seeds(4, 1).view(np.int64)).cuda()
    for mode in (fh.FH_MODE_GREEDY, fh.FH_MODE_SAMPLE):
        b = _both(fh, Es, Hs, mode, 0.7, ss)
        assert np.array_equal(b[0], b[2]) and np.array_equal(b[1], b[3])
    # more rows than the fixed workspace holds: refused on the host
    H17 = _dev(synth.make_hidden(small, 17))
    out = torch.empty(17, dtype=torch.int32, device="cuda")
    with pytest.raises(fh.FlashHeadError) as e:
        fh.dense_head_static(Es, H17, 17, fh.FH_MODE_GREEDY, 1.0, None, out)
    assert e.value.status == fh.FH_ERR_INVALID_ARG
