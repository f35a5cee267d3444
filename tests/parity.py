"""Comparison rules between the HIP path and the CPU oracle.

R1  cluster set: equal when the oracle's gap between the p-th and (p+1)-th
    selection keys exceeds 1e-3; otherwise the sets may differ only inside
    that tie band.
R2  candidate logits: compared by token id, max-abs 2e-2 (bf16 inputs) or
    1e-4 (fp32 inputs).
R3  token: the oracle re-decodes the GPU's candidate set; ids must match when
    the top-2 key margin exceeds 1e-3, else the GPU's token must lie within
    1e-3 of the top key.
R4  sampling: R1-R3 on the Gumbel-perturbed keys.
"""
from __future__ import annotations

import numpy as np

from oracle import flashhead_ref as ref

BAND = 1e-3
TOL = {"f32": 1e-4, "bf16": 2e-2}


class Stats:
    def __init__(self):
        self.rows = 0
        self.set_band = 0
        self.set_diff = 0
        self.tok_band = 0
        self.tok_diff = 0
        self.max_logit_err = 0.0

    def merge(self, o: "Stats"):
        self.rows += o.rows
        self.set_band += o.set_band
        self.set_diff += o.set_diff
        self.tok_band += o.tok_band
        self.tok_diff += o.tok_diff
        self.max_logit_err = max(self.max_logit_err, o.max_logit_err)

    def __repr__(self):
        return (f"rows={self.rows} set_in_band={self.set_band} "
                f"set_differs={self.set_diff} tok_in_band={self.tok_band} "
                f"tok_differs={self.tok_diff} "
                f"max_logit_err={self.max_logit_err:.3g}")


def check_selection(gpu_sel, keys1, p, stats: Stats | None = None, runs: int = 1):
    """R1 for one row; keys1 = oracle selection keys (float64, length c).
    The GPU's list is `runs` ascending runs at most (the method leaves the
    order open; the library lists ascending, or, in the single-launch batch-1
    decode, the clusters published before the boundary bin, then the rest);
    the set is what is compared."""
    c = len(keys1)
    glist = np.asarray(gpu_sel, dtype=np.int64)
    assert len(glist) == p, "wrong number of clusters"
    assert len(np.unique(glist)) == p, "duplicate cluster"
    assert np.count_nonzero(np.diff(glist) < 0) <= runs - 1, "clusters out of order"
    gsel = np.sort(glist)
    assert gsel.min() >= 0 and gsel.max() < c
    order = ref.order_desc(keys1)
    osel = np.sort(order[:p])
    m1 = keys1[order[p - 1]] - keys1[order[p]] if p < c else np.inf
    if m1 > BAND:
        assert np.array_equal(gsel, osel), "cluster set differs outside band"
        return
    if stats is not None:
        stats.set_band += 1
    kp = keys1[order[p - 1]]
    assert np.all(keys1[gsel] >= kp - BAND), "selected cluster below band"
    if p < c:
        kp1 = keys1[order[p]]
        mask = np.ones(c, dtype=bool)
        mask[gsel] = False
        assert np.all(keys1[mask] <= kp1 + BAND), "dropped cluster above band"
    if stats is not None and not np.array_equal(gsel, osel):
        stats.set_diff += 1


def check_candidates(gpu_sel, gpu_ids, c2t):
    """Candidate ids are the selected clusters' C2T rows, in order."""
    want = ref.candidate_tokens(np.asarray(gpu_sel), c2t)
    assert np.array_equal(np.asarray(gpu_ids, dtype=np.int64), want)


def check_logits(gpu_ids, gpu_logits, rows, h64, dtype, stats=None):
    z = ref.exact_logits(rows, np.asarray(gpu_ids, dtype=np.int64), h64)
    err = float(np.max(np.abs(np.asarray(gpu_logits, np.float64) - z)))
    if stats is not None:
        stats.max_logit_err = max(stats.max_logit_err, err)
    assert err <= TOL[dtype], f"candidate logit error {err}"
    return z


def check_token(gpu_token, gpu_ids, z, mode, tau, seed, stats=None):
    """R3: decode the GPU's candidate set with the oracle."""
    tok, m2, _, keys2 = ref.decode_tokens(gpu_ids, z, mode, tau, seed)
    if m2 > BAND:
        assert int(gpu_token) == tok, f"token {gpu_token} != oracle {tok}"
        return
    if stats is not None:
        stats.tok_band += 1
        stats.tok_diff += int(gpu_token) != tok
    ids = np.asarray(gpu_ids)
    where = np.nonzero(ids == int(gpu_token))[0]
    assert len(where) == 1, "token not among the candidates"
    assert keys2[where[0]] >= keys2.max() - BAND, "token outside the tie band"


def check_row(*, gpu_token, gpu_sel, gpu_ids, gpu_logits, keys1, p, c2t,
              rows, h64, dtype, mode="greedy", tau=1.0, seed=0, stats=None, runs=1):
    if stats is not None:
        stats.rows += 1
    check_selection(gpu_sel, keys1, p, stats, runs)
    check_candidates(gpu_sel, gpu_ids, c2t)
    z = check_logits(gpu_ids, gpu_logits, rows, h64, dtype, stats)
    check_token(gpu_token, gpu_ids, z, mode, tau, seed, stats)
