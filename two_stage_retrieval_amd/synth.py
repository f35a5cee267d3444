"""Seeded synthetic workloads shaped like the FlashHead pages' head shapes.

This module only draws data.  It holds none of the head's arithmetic (no
scoring, no selection, no centroid update, no quantization): it produces the
token-embedding matrix E, the equal-size cluster-to-token table C2T, the hidden
vectors H, and for the tiny workload the given centroid matrix.  Both the HIP
path and the CPU oracle take their inputs from here and from nowhere else.

Shapes follow the FlashHead paper's models (Llama-3.2-1B: v=128256, d=2048,
c=8016 clusters of b=16 tokens, p=512 probes; Gemma-3-1B-sized head:
v=262144, d=1152, c=16384, p=1024).  No dataset, checkpoint or trained weight
is used anywhere: real embeddings and benchmark prompts are replaced by the
recipe below.

Recipe (per workload, numpy PCG64 streams):
  * data stream (seed ``data_seed``):
      mu   = rows of a c x d standard normal matrix, each scaled to unit norm
      perm = a uniform permutation of [0, v); C2T[k, j] = perm[k*b + j]
      norms= LogNormal(0, sigma_ln), one per token slot (drawn for all v first)
      row for slot (k, j) = norms[k*b+j] * unit(mu_k + sigma_n * N(0, I_d)),
      stored at E[perm[k*b + j]]; noise is drawn cluster-block by
      cluster-block in order (block size fixed below) so the stream is fixed.
  * hidden stream (seed ``hidden_seed``): t ~ U[0, v) then
      h = h_dir * unit(E[t]) + h_noise * N(0, I_d)
    (for bf16 workloads E[t] is decoded from its stored bf16 bits first).
  * storage: fp32, or bf16 by round-to-nearest-even of the fp32 value.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_head", "make_hidden",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "Head",
]

_NOISE_BLOCK_ROWS = 4096   # rows of noise drawn per block (fixes the stream)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    v: int
    d: int
    c: int
    b: int
    p: int
    dtype: str                 # "f32" or "bf16": storage of E, H (and C)
    batch: int
    sigma_n: float
    sigma_ln: float
    h_dir: float
    h_noise: float
    data_seed: int
    hidden_seed: int
    n_hidden: int              # hidden vectors (B=1) or rows in all batches
    centroids: str             # "given" (unit random) or "means" (computed)
    quant: str = "none"        # "none" or "int4_g128" for stage 1
    mode: str = "greedy"       # "greedy" or "sample"
    taus: tuple = ()
    batches: tuple = ()        # batch sizes run on this workload


WORKLOADS = {
    0: Workload("tiny-f32", v=4096, d=256, c=64, b=64, p=8, dtype="f32",
                batch=1, sigma_n=0.3, sigma_ln=0.2, h_dir=4.0,
                h_noise=math.sqrt(0.5), data_seed=1000, hidden_seed=2000,
                n_hidden=256, centroids="given", batches=(1,)),
    1: Workload("llama3.2-1b-head", v=128256, d=2048, c=8016, b=16, p=512,
                dtype="bf16", batch=1, sigma_n=0.5, sigma_ln=0.25, h_dir=1.0,
                h_noise=1.5, data_seed=1001, hidden_seed=2001, n_hidden=1024,
                centroids="means", batches=(1,)),
    2: Workload("llama3.2-1b-head-b64", v=128256, d=2048, c=8016, b=16,
                p=512, dtype="bf16", batch=64, sigma_n=0.5, sigma_ln=0.25,
                h_dir=1.0, h_noise=1.5, data_seed=1001, hidden_seed=2002,
                n_hidden=200 * 64, centroids="means", batches=(64,)),
    3: Workload("llama3.2-1b-head-sample-b16", v=128256, d=2048, c=8016,
                b=16, p=512, dtype="bf16", batch=16, sigma_n=0.5,
                sigma_ln=0.25, h_dir=1.0, h_noise=1.5, data_seed=1001,
                hidden_seed=2003, n_hidden=200 * 16, centroids="means",
                mode="sample", taus=(0.7, 1.0), batches=(16,)),
    4: Workload("gemma3-1b-head-int4", v=262144, d=1152, c=16384, b=16,
                p=1024, dtype="bf16", batch=1, sigma_n=0.5, sigma_ln=0.25,
                h_dir=1.0, h_noise=1.5, data_seed=1004, hidden_seed=2004,
                n_hidden=1024, centroids="means", quant="int4_g128",
                batches=(1, 32)),
}


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# --------------------------------------------------------------------------
# storage conversion (data plumbing only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float64))
    n[n == 0] = 1.0
    return (x / n[:, None].astype(x.dtype)).astype(np.float32)


@dataclasses.dataclass
class Head:
    wl: Workload
    E: np.ndarray                  # (v, d) float32, or uint16 bf16 bits
    c2t: np.ndarray                # (c, b) int32
    C_given: Optional[np.ndarray]  # (c, d) in E's storage type, or None

    def rows_f32(self, idx) -> np.ndarray:
        r = self.E[idx]
        return bf16_bits_to_f32(r) if self.wl.dtype == "bf16" else r


_HEAD_CACHE: dict = {}


def make_head(wl: Workload | int, *, v=None, d=None, c=None, b=None,
              seed=None, common=0.0, cache=True) -> Head:
    """Draw E and C2T for a workload (shape overrides give small variants).

    common > 0 adds common * m, for one unit vector m shared by all rows, to
    every row before it is normalised: rows that share a direction, as the
    rows of a trained output embedding do.  m comes from a stream of its
    own, so common = 0 gives the workload's usual head."""
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    over = {k: x for k, x in dict(v=v, d=d, c=c, b=b).items() if x is not None}
    if seed is not None:
        over["data_seed"] = seed
    if over:
        if "v" not in over and ("c" in over or "b" in over):
            over["v"] = over.get("c", wl.c) * over.get("b", wl.b)
        wl = dataclasses.replace(wl, **over)
    key = (wl.v, wl.d, wl.c, wl.b, wl.dtype, wl.sigma_n, wl.sigma_ln,
           wl.data_seed, wl.centroids, float(common))
    if cache and key in _HEAD_CACHE:
        h = _HEAD_CACHE[key]
        return Head(wl, h.E, h.c2t, h.C_given)
    if wl.c * wl.b != wl.v:
        raise ValueError("workload needs v == c*b")
    rng = np.random.Generator(np.random.PCG64(wl.data_seed))
    shared = None
    if common:
        shared = _unit_rows(np.random.Generator(np.random.PCG64(wl.data_seed + 7777))
                            .standard_normal((1, wl.d), dtype=np.float32))[0]
        shared *= np.float32(common)
    mu = _unit_rows(rng.standard_normal((wl.c, wl.d), dtype=np.float32))
    perm = rng.permutation(wl.v).astype(np.int32)
    c2t = perm.reshape(wl.c, wl.b).copy()
    norms = rng.lognormal(0.0, wl.sigma_ln, size=wl.v).astype(np.float32)
    E = np.empty((wl.v, wl.d), dtype=np.uint16 if wl.dtype == "bf16"
                 else np.float32)
    slot = 0
    while slot < wl.v:
        n = min(_NOISE_BLOCK_ROWS, wl.v - slot)
        ks = np.arange(slot, slot + n) // wl.b
        x = rng.standard_normal((n, wl.d), dtype=np.float32)
        x *= np.float32(wl.sigma_n)
        x += mu[ks]
        if shared is not None:
            x += shared
        x = _unit_rows(x) * norms[slot:slot + n, None]
        dst = perm[slot:slot + n]
        E[dst] = f32_to_bf16_bits(x) if wl.dtype == "bf16" else x
        slot += n
    C_given = None
    if wl.centroids == "given":
        C_given = f32_to_bf16_bits(mu) if wl.dtype == "bf16" else mu
    head = Head(wl, E, c2t, C_given)
    if cache:
        _HEAD_CACHE[key] = head
    return head


def make_hidden(head: Head, n: int, *, seed=None, offset=0) -> np.ndarray:
    """n hidden vectors (rows offset..offset+n of the workload's stream)."""
    wl = head.wl
    rng = np.random.Generator(np.random.PCG64(
        wl.hidden_seed if seed is None else seed))
    total = offset + n
    t = rng.integers(0, wl.v, size=total)[offset:]
    out = np.empty((n, wl.d), dtype=np.float32)
    # draw the noise rows for all preceding rows so that row i is fixed
    done = 0
    while done < total:
        m = min(1024, total - done)
        z = rng.standard_normal((m, wl.d), dtype=np.float32)
        lo, hi = max(done, offset), done + m
        if hi > lo:
            out[lo - offset:hi - offset] = z[lo - done:hi - done]
        done += m
    dirs = _unit_rows(head.rows_f32(t).astype(np.float32))
    h = np.float32(wl.h_dir) * dirs + np.float32(wl.h_noise) * out
    return f32_to_bf16_bits(h) if wl.dtype == "bf16" else h.astype(np.float32)


def make_seeds(step: int, rows: int) -> np.ndarray:
    """Philox keys per (decode step, batch row): (step << 32) | row."""
    r = np.arange(rows, dtype=np.uint64)
    return (np.uint64(step) << np.uint64(32)) | r
