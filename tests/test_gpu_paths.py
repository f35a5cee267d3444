"""Parity of each kernel path the library picks, at the shapes that select
it, and of its edge cases (through the C ABI, against the CPU oracle):

* path 1: the single-launch batch-1 decode (B = 1, c <= 16384, p <= 2048);
* path 2: stage 1 and stage 2 as separate row-dot launches (B = 1 with a
  larger p, or shapes the matrix-core path does not take);
* path 3: the batched matrix-core path (bf16, B >= 2, b a multiple of 16,
  d a multiple of 128), at ragged batch sizes.
"""
import numpy as np
import pytest

from oracle import flashhead_ref as ref
from two_stage_retrieval_amd import synth

from .parity import Stats
from .test_gpu_parity import case, check_batch, dev_tensor, fh, run_debug  # noqa: F401

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

PATH_SINGLE_LAUNCH, PATH_ROWDOT, PATH_BATCHED = 1, 2, 3


def path_of(fhmod, head):
    return fhmod.flashhead_query(head.handle, 10)


def seeds_dev(seeds):
    return torch.from_numpy(seeds.view(np.int64)).cuda()


@pytest.mark.parametrize("flags", ["SELECT_FIRST", None])
def test_batched_list_and_all_cluster_walks_alternate(fh, flags):
    # below 16 rows stage 2 walks the union list, from 16 rows on every
    # cluster; one handle alternating between the two must find the row
    # masks cleared by whichever ran before (greedy and sampling).  Without
    # a path flag the same handle also alternates between the select-first
    # path and the all-cluster stream (1 - (1 - 40/400)^B: B = 24 streams,
    # B = 16, 2, 3, 5 select first)
    cs = case(1, c=400, b=16, d=256, seed=56)
    fl = getattr(fh, "FH_FLAG_" + flags) if flags else 0
    head = cs.prepare(fh, max_batch=24, max_p=40, flags=fl)
    H, H64 = cs.hidden(24, offset=7)
    st = Stats()
    seen = set()
    for step, B in enumerate((24, 3, 24, 5, 16, 2)):
        res = run_debug(fh, head, dev_tensor(H[:B]), B, 40, "greedy")
        want = fh.flashhead_plan_step(400, 16, 256, fh.FH_DTYPE_BF16, 0, B, 40, 256, 1, fl)[0]
        assert path_of(fh, head) == want
        assert want == PATH_BATCHED or (not flags and want == 4)
        seen.add(want)
        check_batch(cs, res, H64[:B], 40, stats=st)
        seeds = synth.make_seeds(step, B)
        res = run_debug(fh, head, dev_tensor(H[:B]), B, 40, "sample", 0.8, seeds_dev(seeds))
        check_batch(cs, res, H64[:B], 40, "sample", 0.8, seeds, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    assert seen == ({3} if flags else {3, 4})
    print(st)


@pytest.mark.parametrize("path", [3, 4])
@pytest.mark.parametrize("B", [3, 17, 33, 50])
def test_batched_path_ragged_batches(fh, B, path):
    # 16-row MFMA tiles over B columns: 1, 2, 3 and 4 column tiles, each
    # with a partial last tile; c = 50 leaves a partial 16-row stage-1 tile;
    # on both batched paths
    cs = case(1, c=50, b=16, d=256, seed=55)
    flags = fh.FH_FLAG_SELECT_FIRST if path == 3 else fh.FH_FLAG_STREAM_ALL
    head = cs.prepare(fh, max_batch=B, max_p=20, flags=flags)
    H, H64 = cs.hidden(B, offset=B)
    st = Stats()
    res = run_debug(fh, head, dev_tensor(H), B, 20, "greedy")
    assert path_of(fh, head) == path
    check_batch(cs, res, H64, 20, stats=st)
    seeds = synth.make_seeds(5, B)
    res = run_debug(fh, head, dev_tensor(H), B, 20, "sample", 0.8, seeds_dev(seeds))
    check_batch(cs, res, H64, 20, "sample", 0.8, seeds, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


@pytest.mark.parametrize("B", [9, 40, 64])
def test_int4_select_first_tiles_per_workgroup(fh, B):
    # the batched INT4 stage 1 on path 3 with several tiles per workgroup:
    # 1025 tiles, the last with 6 rows, so four tiles per workgroup with one
    # column tile of H and two from three column tiles on, with a last
    # workgroup that holds one live tile; d = 384 gives 3 groups of 128
    # columns over 4 waves, so one wave has none
    cs = case(4, c=16390, b=16, d=384, seed=81)
    head = cs.prepare(fh, max_batch=B, max_p=48, flags=fh.FH_FLAG_SELECT_FIRST)
    H, H64 = cs.hidden(B, offset=3 * B)
    st = Stats()
    res = run_debug(fh, head, dev_tensor(H), B, 48, "greedy")
    assert path_of(fh, head) == 3
    check_batch(cs, res, H64, 48, stats=st)
    seeds = synth.make_seeds(9, B)
    res = run_debug(fh, head, dev_tensor(H), B, 48, "sample", 0.8, seeds_dev(seeds))
    check_batch(cs, res, H64, 48, "sample", 0.8, seeds, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


def test_single_launch_p_equals_c_matches_dense(fh):
    # every cluster probed: the head is the dense argmax, id for id
    cs = case(1, c=50, b=16, d=256, seed=56)
    head = cs.prepare(fh, max_batch=1, max_p=50)
    dense = fh.DenseHead(cs.E_dev, max_batch=1)
    H, H64 = cs.hidden(8)
    for i in range(8):
        x = dev_tensor(H[i:i + 1])
        t_head = int(head.greedy(x, 50).cpu().numpy()[0])
        assert path_of(fh, head) == PATH_SINGLE_LAUNCH
        t_dense = int(dense(x).cpu().numpy()[0])
        assert t_head == t_dense
        z = ref.dense_logits(cs.rows, cs.wl.v, H64[i])
        tok, m2, _, keys = ref.decode_tokens(np.arange(cs.wl.v), z, "greedy", 1.0, 0)
        if m2 > 1e-3:
            assert t_head == tok
        else:
            assert keys[t_head] >= keys.max() - 1e-3


def test_single_launch_alternating_p(fh):
    # consecutive launches alternate buffer sets; p changes between them
    cs = case(1)
    head = cs.prepare(fh, max_batch=1, max_p=512)
    H, H64 = cs.hidden(6, offset=300)
    st = Stats()
    for i, p in enumerate([512, 37, 512, 1, 200, 512]):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, p, "greedy")
        assert path_of(fh, head) == PATH_SINGLE_LAUNCH
        check_batch(cs, res, H64[i:i + 1], p, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


def test_single_launch_buffers_stay_consistent_across_grids(fh):
    # the single launch's grid follows p (256 workgroups at p = 512, 251 at
    # p = 37 on this head); after every call the buffer set the next launch
    # uses must be back in its pending state, also the merge slots of
    # workgroups beyond the last grid; sampling with the lse checks that no
    # stale partial reaches the merge
    cs = case(1)
    head = cs.prepare(fh, max_batch=1, max_p=512)
    H, H64 = cs.hidden(8, offset=310)
    st = Stats()
    assert fh.flashhead_query(head.handle, 11) == 0
    for i, p in enumerate([512, 37, 512, 1, 200, 512, 37, 512]):
        seeds = synth.make_seeds(40 + i, 1)
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, p, "sample", 0.9,
                        seeds_dev(seeds))
        assert path_of(fh, head) == PATH_SINGLE_LAUNCH
        assert fh.flashhead_query(head.handle, 11) == 0
        check_batch(cs, res, H64[i:i + 1], p, "sample", 0.9, seeds, stats=st)
        x = dev_tensor(H[i:i + 1])
        head.greedy(x, p)
        assert fh.flashhead_query(head.handle, 11) == 0
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


def test_single_launch_plan_matches_the_device(fh):
    # the handle's own plan inputs give the path each step takes
    cs = case(1)
    head = cs.prepare(fh, max_batch=4, max_p=512)
    ncu = fh.flashhead_query(head.handle, 13)
    bpc = fh.flashhead_query(head.handle, 12)
    assert ncu >= 1 and bpc >= 1
    H, _ = cs.hidden(4, offset=20)
    for B, p in ((1, 512), (1, 37), (4, 512)):
        head.greedy(dev_tensor(H[:B]), p)
        path, grid = fh.flashhead_plan_step(cs.wl.c, cs.wl.b, cs.wl.d, fh.FH_DTYPE_BF16, 0,
                                            B, p, ncu, bpc)
        assert path_of(fh, head) == path
        if path == PATH_SINGLE_LAUNCH:
            assert 1 <= grid <= min(ncu, 512)
    assert fh.flashhead_query(head.handle, 9) == 0


def test_cooperative_launch_gives_the_same_results(fh):
    cs = case(1)
    plain = cs.prepare(fh, max_batch=1, max_p=512)
    coop = fh.FlashHead(cs.E_dev, cs.head.c2t, cs.C_dev, max_batch=1, max_p=512,
                        flags=fh.FH_FLAG_COOPERATIVE)
    assert fh.flashhead_query(coop.handle, 14) == fh.FH_FLAG_COOPERATIVE
    H, _ = cs.hidden(16, offset=40)
    for i in range(16):
        x = dev_tensor(H[i:i + 1])
        sd = seeds_dev(synth.make_seeds(i, 1))
        a = plain.greedy(x, 512).cpu().numpy()
        b = coop.greedy(x, 512).cpu().numpy()
        assert path_of(fh, coop) == PATH_SINGLE_LAUNCH
        assert np.array_equal(a, b)
        la = torch.empty(1, device="cuda")
        lb = torch.empty(1, device="cuda")
        a = plain.sample(x, 512, 0.8, sd, out_lse=la).cpu().numpy()
        b = coop.sample(x, 512, 0.8, sd, out_lse=lb).cpu().numpy()
        assert np.array_equal(a, b) and torch.equal(la, lb)
    assert fh.flashhead_query(coop.handle, 9) == 0
    assert fh.flashhead_query(coop.handle, 11) == 0
    coop.close()


def test_large_p_takes_the_two_launch_path(fh):
    # p above what the single launch keeps in LDS
    cs = case(1, c=4096, b=16, d=128, seed=57)
    head = cs.prepare(fh, max_batch=1, max_p=3000)
    H, H64 = cs.hidden(2)
    st = Stats()
    for i in range(2):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, 3000, "greedy")
        assert path_of(fh, head) == PATH_ROWDOT
        check_batch(cs, res, H64[i:i + 1], 3000, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


@pytest.mark.parametrize("B", [1, 16, 64])
def test_debug_outputs_do_not_change_results(fh, B):
    cs = case(3)
    head = cs.prepare(fh, max_batch=B, max_p=512)
    H, _ = cs.hidden(B, offset=900)
    x = dev_tensor(H)
    seeds = seeds_dev(synth.make_seeds(3, B))
    plain = head.greedy(x, 512).cpu().numpy()
    dbg = run_debug(fh, head, x, B, 512, "greedy")["tokens"]
    assert np.array_equal(plain, dbg)
    lse = torch.empty(B, dtype=torch.float32, device="cuda")
    s_plain = head.sample(x, 512, 0.7, seeds).cpu().numpy()
    s_lse = head.sample(x, 512, 0.7, seeds, out_lse=lse).cpu().numpy()
    s_dbg = run_debug(fh, head, x, B, 512, "sample", 0.7, seeds)
    assert np.array_equal(s_plain, s_lse)
    assert np.array_equal(s_plain, s_dbg["tokens"])
    assert np.array_equal(lse.cpu().numpy(), s_dbg["lse"])


def test_stream_read_reference(fh):
    buf = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    fh.flashhead_stream_read(buf, sink)
    torch.cuda.synchronize()
    # the data-dependent write does not happen for this content
    assert sink.cpu().numpy().tolist() == [0, 0, 0, 0]
    with pytest.raises(fh.FlashHeadError):
        fh.flashhead_stream_read(buf[1:], sink)  # misaligned, not a multiple of 16 bytes


def with_outlier_centroids(cs, frac=0.01, factor=32.0, seed=91):
    """A copy of the case whose centroid rows include a few scaled by a
    power of two (exact in bf16): their scores spread far beyond the
    others', which inflates the spread of all keys while leaving only a
    handful far above the mean."""
    import copy
    rng = np.random.default_rng(seed)
    out = copy.copy(cs)
    C64 = cs.C64.copy()
    rows = rng.choice(C64.shape[0], size=max(1, int(frac * C64.shape[0])), replace=False)
    C64[rows] *= factor
    out.C64 = C64
    out.C_store = ref.bf16_bits_of(C64) if cs.dtype == "bf16" else C64.astype(np.float32)
    out.C_dev = dev_tensor(out.C_store)
    return out


@pytest.mark.parametrize("B", [1, 4])
def test_selection_with_outlier_keys(fh, B):
    # few keys far above the rest: the histogram range the key moments
    # suggest holds fewer than p keys, and the selection redoes it over the
    # full range (both the single-launch and the batched selection)
    cs = with_outlier_centroids(case(1))
    head = cs.prepare(fh, max_batch=B, max_p=64)
    H, H64 = cs.hidden(B, offset=700)
    # the case does take the second pass: fewer than p scores lie above
    # mean + z sd, z the normal quantile with upper tail 4 p / c
    from scipy.stats import norm
    z = norm.isf(4 * 64 / cs.wl.c)
    for r in range(B):
        sc = cs.oracle_scores(H64[r])
        assert np.count_nonzero(sc >= sc.mean() + z * sc.std()) < 64
    st = Stats()
    res = run_debug(fh, head, dev_tensor(H), B, 64, "greedy")
    check_batch(cs, res, H64, 64, stats=st)
    seeds = synth.make_seeds(9, B)
    res = run_debug(fh, head, dev_tensor(H), B, 64, "sample", 0.7, seeds_dev(seeds))
    check_batch(cs, res, H64, 64, "sample", 0.7, seeds, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)


# --------------------------------------------------------------------------
# c / p variants of the Llama head shape ([paper] Table 7): same kernels,
# other cluster sizes and probe counts
# --------------------------------------------------------------------------

@pytest.mark.parametrize("c,b,p", [(4008, 32, 128), (4008, 32, 256), (4008, 32, 512),
                                   (8016, 16, 128)])
def test_cp_variants_parity(fh, c, b, p):
    cs = case(1, c=c, b=b)
    head = cs.prepare(fh, max_batch=16, max_p=p)
    st = Stats()
    H, H64 = cs.hidden(8, offset=1500)
    for i in range(8):
        res = run_debug(fh, head, dev_tensor(H[i:i + 1]), 1, p, "greedy")
        assert path_of(fh, head) == PATH_SINGLE_LAUNCH
        check_batch(cs, res, H64[i:i + 1], p, stats=st)
    seeds = synth.make_seeds(6, 16)
    H16, H16_64 = cs.hidden(16, offset=1600)
    res = run_debug(fh, head, dev_tensor(H16), 16, p, "sample", 0.8, seeds_dev(seeds))
    # 16 rows at p / c = 512 / 4008 are expected to select 89% of the
    # clusters between them: the all-cluster stream; the others select first
    assert path_of(fh, head) == fh.flashhead_plan_step(c, b, cs.wl.d, fh.FH_DTYPE_BF16, 0, 16,
                                                       p, 256, 1)[0]
    assert path_of(fh, head) in (PATH_BATCHED, 4)
    check_batch(cs, res, H16_64, p, "sample", 0.8, seeds, stats=st)
    assert fh.flashhead_query(head.handle, 9) == 0
    print(st)
