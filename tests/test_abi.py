"""The C ABI without a GPU: the library loads, exports every function that
include/flashhead.h declares, and rejects bad arguments on the host before
any device work (these paths never reach the HIP runtime)."""
from __future__ import annotations

import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashhead.h")
LIB = os.path.join(ROOT, "two_stage_retrieval_amd", "libflashhead.so")

# an aligned address that is never dereferenced: every call below fails its
# host-side checks before touching device memory
FAKE_DEV = 0x10000


def declared_functions() -> set[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return {n for n in names if not n.startswith("FH_")}


@pytest.fixture(scope="module")
def fh():
    if not os.path.exists(LIB):
        pytest.fail("libflashhead.so is not built (run __graft_entry__.build())")
    from two_stage_retrieval_amd import binding
    return binding


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("flashhead_prepare", "flashhead_destroy", "flashhead_greedy",
              "flashhead_sample", "dense_head", "flashhead_status_string"):
        assert n in names


def test_library_exports_every_declared_function(fh):
    names = declared_functions()
    lib = C.CDLL(LIB)
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"
    # the same set with the dynamic symbol table, independent of ctypes
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert names <= exported
    # the Python binding wraps exactly the declared set
    assert set(fh.EXPORTED) == names


def test_status_strings(fh):
    for code in (fh.FH_OK, fh.FH_ERR_INVALID_ARG, fh.FH_ERR_NOT_PERMUTATION,
                 fh.FH_ERR_UNSUPPORTED, fh.FH_ERR_HIP, fh.FH_ERR_OOM):
        s = fh.status_string(code)
        assert s and s != "unknown status"
    assert fh.status_string(12345) == "unknown status"
    assert fh.flashhead_last_hip_error() == "hipSuccess"


def _desc(fh, c2t, *, v=None, d=256, dtype=None, lde=None, E=FAKE_DEV, C_init=None,
          quant=0, max_batch=1, max_p=1, flags=0):
    c, b = c2t.shape
    dtype = fh.FH_DTYPE_F32 if dtype is None else dtype
    return fh.fh_desc(c * b if v is None else v, d, c, b, dtype, d if lde is None else lde,
                      E, c2t.ctypes.data, C_init, quant, max_batch, max_p, None, flags)


def _prepare(fh, desc) -> int:
    h = C.c_void_p()
    st = fh.lib.flashhead_prepare(C.byref(desc), C.byref(h))
    assert h.value is None
    return st


def test_prepare_rejects_bad_descriptors(fh):
    c2t = np.arange(64, dtype=np.int32).reshape(8, 8)
    inv, uns = fh.FH_ERR_INVALID_ARG, fh.FH_ERR_UNSUPPORTED
    assert fh.lib.flashhead_prepare(None, None) == inv
    h = C.c_void_p()
    assert fh.lib.flashhead_prepare(None, C.byref(h)) == inv
    assert _prepare(fh, _desc(fh, c2t, E=None)) == inv
    assert _prepare(fh, _desc(fh, c2t, v=65)) == inv             # v != c * b
    assert _prepare(fh, _desc(fh, c2t, max_batch=0)) == inv
    assert _prepare(fh, _desc(fh, c2t, max_batch=65)) == inv
    assert _prepare(fh, _desc(fh, c2t, max_p=9)) == inv          # p > c
    assert _prepare(fh, _desc(fh, c2t, lde=255)) == inv          # lde < d
    assert _prepare(fh, _desc(fh, c2t, dtype=7)) == uns
    assert _prepare(fh, _desc(fh, c2t, d=250)) == uns            # rows not 16-byte multiples
    assert _prepare(fh, _desc(fh, c2t, E=FAKE_DEV + 4)) == uns   # misaligned E
    assert _prepare(fh, _desc(fh, c2t, quant=5)) == uns
    assert _prepare(fh, _desc(fh, c2t, quant=fh.FH_QUANT_INT4_G128)) == uns  # INT4 needs bf16
    assert _prepare(fh, _desc(fh, c2t, dtype=fh.FH_DTYPE_BF16, d=200,
                              quant=fh.FH_QUANT_INT4_G128)) == uns            # d % 128
    assert _prepare(fh, _desc(fh, c2t, quant=fh.FH_QUANT_INT4_G128_MEAN)) == uns
    assert _prepare(fh, _desc(fh, c2t, dtype=fh.FH_DTYPE_BF16, d=200,
                              quant=fh.FH_QUANT_INT4_G128_MEAN)) == uns
    assert _prepare(fh, _desc(fh, c2t, flags=16)) == inv         # unknown flag bit
    assert _prepare(fh, _desc(fh, c2t, flags=fh.FH_FLAG_STREAM_ALL |
                              fh.FH_FLAG_SELECT_FIRST)) == inv      # both path flags


@pytest.mark.parametrize("kind", ["repeat", "out_of_range", "negative"])
def test_prepare_rejects_c2t_that_is_not_a_permutation(fh, kind):
    c2t = np.random.default_rng(3).permutation(64).astype(np.int32).reshape(8, 8)
    if kind == "repeat":
        c2t[5, 2] = c2t[1, 1]
    elif kind == "out_of_range":
        c2t[0, 0] = 64
    else:
        c2t[7, 7] = -1
    assert _prepare(fh, _desc(fh, c2t)) == fh.FH_ERR_NOT_PERMUTATION


def test_step_calls_reject_null_handle_and_arguments(fh):
    lib = fh.lib
    inv = fh.FH_ERR_INVALID_ARG
    out = C.c_void_p(FAKE_DEV)
    assert lib.flashhead_greedy(None, FAKE_DEV, 1, 1, out, None, None) == inv
    assert lib.flashhead_sample(None, FAKE_DEV, 1, 1, C.c_float(1.0), FAKE_DEV, out, None,
                                None, None) == inv
    lib.flashhead_destroy(None)  # a no-op
    v = C.c_int64()
    assert lib.flashhead_query(None, 0, C.byref(v)) == inv
    calls = C.c_int32()
    stage = (C.c_double * 3)()
    assert lib.flashhead_profile_end(None, stage, C.byref(calls)) == inv
    assert lib.flashhead_profile_begin(None, 4) == inv


def test_dense_head_host_checks(fh):
    lib = fh.lib
    inv, uns = fh.FH_ERR_INVALID_ARG, fh.FH_ERR_UNSUPPORTED
    ws = FAKE_DEV
    args = dict(E=FAKE_DEV, v=4096, d=256, dtype=fh.FH_DTYPE_F32, lde=256, H=FAKE_DEV, B=1,
                mode=fh.FH_MODE_GREEDY, tau=1.0, seeds=None, out=FAKE_DEV, lse=None, ws=ws)

    def call(**kw):
        a = dict(args, **kw)
        return lib.dense_head(a["E"], a["v"], a["d"], a["dtype"], a["lde"], a["H"], a["B"],
                              a["mode"], C.c_float(a["tau"]), a["seeds"], a["out"], a["lse"],
                              a["ws"], None)

    assert call(E=None) == inv
    assert call(ws=None) == inv
    assert call(B=0) == inv
    assert call(B=65) == inv
    assert call(lde=100) == inv
    assert call(mode=3) == inv
    assert call(mode=fh.FH_MODE_SAMPLE) == inv                  # no seeds
    assert call(mode=fh.FH_MODE_SAMPLE, seeds=FAKE_DEV, tau=0.0) == inv
    assert call(mode=fh.FH_MODE_SAMPLE, seeds=FAKE_DEV, tau=float("inf")) == inv
    assert call(dtype=9) == uns
    assert call(H=FAKE_DEV + 8) == uns


def test_dense_workspace_size(fh):
    assert fh.dense_head_workspace_bytes(0) == 0
    for B in (1, 4, 64):
        n = fh.dense_head_workspace_bytes(B)
        # best keys, counters (16-byte padded) and per-block partials
        assert n >= B * 8 + B * 4 + B * 8 and n % 8 == 0
        assert fh.dense_head_workspace_bytes(B + 1) > n


def test_kmeans_host_checks(fh):
    # every rejection is decided on the host before any device work
    lib = fh.lib
    inv, uns = fh.FH_ERR_INVALID_ARG, fh.FH_ERR_UNSUPPORTED
    good = np.arange(0, 4096, 64, dtype=np.int32)  # 64 distinct ids

    def call(E=FAKE_DEV, v=4096, d=256, dtype=fh.FH_DTYPE_F32, lde=256, c=64, init=good,
             iters=3, c2t=FAKE_DEV):
        n = C.c_int32(-1)
        st = lib.flashhead_kmeans(E, v, d, dtype, lde, c,
                                  None if init is None else init.ctypes.data, iters, c2t, None,
                                  C.byref(n), None)
        assert n.value == 0
        return st

    assert call(E=None) == inv
    assert call(c2t=None) == inv
    assert call(init=None) == inv
    assert call(v=4000) == inv            # v % c != 0
    assert call(iters=0) == inv
    assert call(lde=200) == inv
    assert call(d=0) == inv
    dup = good.copy()
    dup[5] = dup[4]
    assert call(init=dup) == inv
    out = good.copy()
    out[0] = 4096
    assert call(init=out) == inv
    neg = good.copy()
    neg[1] = -1
    assert call(init=neg) == inv
    assert call(dtype=9) == uns
    assert call(E=FAKE_DEV + 2) == uns    # not aligned to its fp32 elements
    assert call(c=2, init=good[:2]) == uns  # 2048 tokens per cluster


# --------------------------------------------------------------------------
# the host-side plan: which kernels a step takes, and the residency rule of
# the single launch (its workgroups wait on one another)
# --------------------------------------------------------------------------

def test_plan_step_paths(fh):
    BF, F32 = fh.FH_DTYPE_BF16, fh.FH_DTYPE_F32
    plan = fh.flashhead_plan_step
    # the Llama-3.2-1B head shape at batch 1: one launch, one workgroup per
    # compute unit
    assert plan(8016, 16, 2048, BF, 0, 1, 512, 256, 1) == (1, 256)
    # fewer compute units: the grid shrinks with them
    assert plan(8016, 16, 2048, BF, 0, 1, 512, 80, 1) == (1, 80)
    # a kernel no compute unit can hold: never the single launch
    assert plan(8016, 16, 2048, BF, 0, 1, 512, 256, 0) == (2, 0)
    # the Gemma-3-1B head with INT4 centroids
    assert plan(16384, 16, 1152, BF, fh.FH_QUANT_INT4_G128, 1, 1024, 256, 2) == (1, 256)
    # a small head: the grid covers its rows, not every compute unit
    path, grid = plan(64, 64, 256, F32, 0, 1, 8, 256, 1)
    assert path == 1 and 1 <= grid < 256
    # batches: matrix cores for bf16 with b a multiple of 16, else row-dot;
    # select first while the rows' selections are expected to leave many
    # clusters unread (1 - (1 - p/c)^B below 0.85), else stream every
    # cluster, on heads whose width the stream walks in 256-wide chunks
    assert plan(8016, 16, 2048, BF, 0, 2, 512, 256, 1) == (3, 0)
    assert plan(8016, 16, 2048, BF, 0, 16, 512, 256, 1) == (3, 0)     # 0.65
    assert plan(8016, 16, 2048, BF, 0, 28, 512, 256, 1) == (3, 0)     # 0.842
    assert plan(8016, 16, 2048, BF, 0, 29, 512, 256, 1) == (4, 0)     # 0.853
    assert plan(8016, 16, 2048, BF, 0, 64, 512, 256, 1) == (4, 0)     # 0.985
    # d = 1152: select first at any coverage
    assert plan(16384, 16, 1152, BF, fh.FH_QUANT_INT4_G128, 32, 1024, 256, 1) == (3, 0)
    assert plan(16384, 16, 1152, BF, fh.FH_QUANT_INT4_G128, 64, 1024, 256, 1) == (3, 0)
    assert plan(16384, 16, 1152, BF, 0, 64, 1024, 256, 1) == (3, 0)
    # the path flags override the rule, for batches only
    SF, SA = fh.FH_FLAG_SELECT_FIRST, fh.FH_FLAG_STREAM_ALL
    assert plan(8016, 16, 2048, BF, 0, 64, 512, 256, 1, SF) == (3, 0)
    assert plan(8016, 16, 2048, BF, 0, 2, 512, 256, 1, SA) == (4, 0)
    assert plan(8016, 16, 2048, BF, 0, 1, 512, 256, 1, SA) == (1, 256)
    assert plan(50, 8, 128, BF, 0, 3, 7, 256, 1, SA) == (2, 0)
    assert plan(50, 8, 128, BF, 0, 3, 7, 256, 1) == (2, 0)
    assert plan(4096, 1, 256, F32, 0, 4, 8, 256, 1) == (2, 0)
    # more probes than the single launch holds, or more clusters than it selects
    assert plan(4096, 16, 128, BF, 0, 1, 3000, 256, 1) == (2, 0)
    assert plan(20000, 2, 128, BF, 0, 1, 300, 256, 1) == (2, 0)


def test_plan_step_rejects_bad_sizes(fh):
    BF = fh.FH_DTYPE_BF16
    g = C.c_int32(7)
    inv = fh.FH_ERR_INVALID_ARG
    lib = fh.lib
    assert lib.flashhead_plan_step(8016, 16, 2048, BF, 0, 1, 512, 256, 1, 0, None) == inv
    both = fh.FH_FLAG_STREAM_ALL | fh.FH_FLAG_SELECT_FIRST
    for args in ((8016, 16, 2048, BF, 0, 1, 8017, 256, 1, 0),   # p > c
                 (8016, 16, 2048, BF, 0, 0, 512, 256, 1, 0),    # B = 0
                 (8016, 16, 2048, BF, 0, 65, 512, 256, 1, 0),   # B > FH_MAX_BATCH
                 (8016, 16, 2048, 5, 0, 1, 512, 256, 1, 0),     # dtype
                 (8016, 16, 2048, BF, 3, 1, 512, 256, 1, 0),    # quant
                 (8016, 16, 2048, BF, 0, 1, 512, 0, 1, 0),      # no compute unit
                 (8016, 16, 2048, BF, 0, 64, 512, 256, 1, both)):  # both path flags
        assert lib.flashhead_plan_step(*args, C.byref(g)) == inv
        assert g.value == 0


def test_dense_head_static_host_checks(fh):
    # rejected on the host, before the library's fixed workspace is looked up
    lib = fh.lib
    inv = fh.FH_ERR_INVALID_ARG
    assert fh.FH_DENSE_STATIC_MAX_BATCH == 16
    assert fh.dense_head_workspace_bytes(16) <= 4 << 20
    for B in (17, 64):
        assert lib.dense_head_static(FAKE_DEV, 4096, 256, fh.FH_DTYPE_F32, 256, FAKE_DEV, B,
                                     fh.FH_MODE_GREEDY, C.c_float(1.0), None, FAKE_DEV, None,
                                     None) == inv
