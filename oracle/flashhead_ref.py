"""Plain CPU oracle for FlashHead's two-stage retrieval head.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the package entry's smoke check and the benchmark's CPU-baseline
leg may call it.  It shares no code with the HIP path.

Every floating-point step runs in float64 on exactly decoded inputs (bf16
storage is decoded by placing its 16 bits in the top half of an fp32 word).
Sources, cited by page and section:

  [notes]  "FlashHead: Efficient Drop-In Replacement for the Classification
           Head in Language Model Inference" -- reading notes (dihengye.cn):
           sections "Overall architecture", "Module 1: equal-size spherical
           k-means", "Module 2: multi-probe retrieval", "Module 3: selective
           quantization", "Module 4: Monte Carlo probability estimation",
           "Key formulas" 1-7, "Figure 1".
  [paper]  the FlashHead paper page (thelatestinai.com, arXiv 2603.14591):
           abstract, Figure 1 caption, Tables 3-8.

Readings taken where the pages are silent (each listed in the design notes):
  * ties: higher key first, then the lower index (cluster id or token id);
  * stage-1 score is the raw inner product C_k . h ([notes] Figure 1);
  * sampling mode scales stage-1 logits by the same temperature tau as the
    token sampler and samples p clusters without replacement by successive
    (Plackett-Luce) draws, realised as Gumbel-top-p;
  * the token sampler draws from the softmax over the candidate set only
    (Formula 3 restricted to the candidates), realised as Gumbel-max;
  * random numbers: Philox4x32-10 (Salmon et al., SC'11), key = seed,
    counter = (idx >> 2, stream, 0, 0), word idx & 3; stream 0 draws per
    cluster id, stream 1 per token id; u = (2*(x >> 9) + 1) * 2**-24,
    g = -log(-log u);
  * INT4 stage-1 centroids: symmetric signed 4-bit codes per group of 128
    columns, scale = bf16(amax / 7), codes = round-half-even(C / scale);
  * centroids when computed: bf16 of the unit-normalised mean of the raw
    cluster rows ([notes] Formula 5);
  * equal-size spherical k-means ([notes] Module 1): tokens are placed by
    cosine in descending order of the (token, cluster) pairs, each into a
    cluster with room (the unique stable capacity-b assignment); centroids
    start from the unit rows of caller-drawn distinct token ids and stay in
    float64 between iterations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)

# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------


def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits), ties to even.

    Returns float64 values that are exactly representable in bf16.  The
    spacing of bf16 numbers near x is 2**(e-8) where x = m * 2**e with
    0.5 <= |m| < 1; below the normal range the spacing stays at 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing_exp = np.maximum(e - 8, -133)
    y = np.rint(np.ldexp(x, -spacing_exp))          # rint: half to even
    return np.ldexp(y, spacing_exp)


def bf16_bits_of(x) -> np.ndarray:
    """Bit patterns of float64 values that are already bf16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def as_f64(arr, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# validation ([notes] Module 1: every cluster holds exactly b = v / c tokens
# and the cluster-to-token map is a dense c x b table)
# --------------------------------------------------------------------------


def validate(v: int, c: int, b: int, c2t, p: Optional[int] = None,
             tau: Optional[float] = None) -> None:
    if c <= 0 or b <= 0 or c * b != v:
        raise ValueError("need v == c * b with c, b > 0")
    t = np.asarray(c2t)
    if t.shape != (c, b):
        raise ValueError("C2T must be c x b")
    flat = t.reshape(-1).astype(np.int64)
    if flat.min() < 0 or flat.max() >= v:
        raise ValueError("C2T entry out of [0, v)")
    if not np.all(np.bincount(flat, minlength=v) == 1):
        raise ValueError("C2T is not a permutation of [0, v)")
    if p is not None and not (1 <= p <= c):
        raise ValueError("p must lie in [1, c]")
    if tau is not None and not (math.isfinite(tau) and tau > 0):
        raise ValueError("tau must be finite and > 0")


# --------------------------------------------------------------------------
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As
# Easy as 1, 2, 3", SC'11).  Written from the paper's definition: each round
# multiplies words 0 and 2 by two fixed odd constants, swaps the high/low
# halves across the lanes and mixes in the round key; the key is bumped by
# two Weyl constants between rounds.
# --------------------------------------------------------------------------

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key):
    """Vectorised block function.  ctr: 4 uint arrays, key: 2 uint arrays."""
    x0, x1, x2, x3 = (np.asarray(w, dtype=np.uint64) & MASK32 for w in ctr)
    k0, k1 = (np.asarray(w, dtype=np.uint64) & MASK32 for w in key)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & MASK32
        p0 = m0 * x0          # < 2**64: exact in uint64
        p1 = m1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def philox_words(seed: int, stream: int, idx) -> np.ndarray:
    """The 32-bit word drawn for index idx of a stream under key `seed`."""
    idx = np.asarray(idx, dtype=np.uint64)
    seed = np.uint64(seed)
    key = (seed & MASK32, seed >> np.uint64(32))
    zeros = np.zeros_like(idx)
    ctr = (idx >> np.uint64(2), zeros + np.uint64(stream), zeros, zeros)
    outs = philox4x32_10(ctr, key)
    sel = (idx & np.uint64(3)).astype(np.int64)
    return np.choose(sel, outs).astype(np.uint64)


def uniform_open01(words) -> np.ndarray:
    """(2 * (x >> 9) + 1) * 2**-24: 2**23 odd multiples of 2**-24 in (0,1)."""
    w = np.asarray(words, dtype=np.uint64)
    return ((w >> np.uint64(9)) * np.uint64(2) + np.uint64(1)).astype(
        np.float64) * 2.0 ** -24


def gumbel(seed: int, stream: int, idx) -> np.ndarray:
    """Standard Gumbel noise -log(-log u) per (seed, stream, index)."""
    u = uniform_open01(philox_words(seed, stream, idx))
    return -np.log(-np.log(u))


STREAM_CLUSTER = 0
STREAM_TOKEN = 1

# --------------------------------------------------------------------------
# prepare-time data
# --------------------------------------------------------------------------


def centroid_means(rows_f64: Callable[[np.ndarray], np.ndarray], c2t
                   ) -> np.ndarray:
    """[notes] Formula 5: c_k = mean of the cluster's rows, L2-normalised.

    Returns the bf16-rounded centroids as float64 values (c x d).  A cluster
    whose mean is the zero vector gets the zero centroid.
    """
    c2t = np.asarray(c2t)
    out = []
    for k in range(c2t.shape[0]):
        m = rows_f64(c2t[k]).sum(axis=0) / c2t.shape[1]
        n = math.sqrt(float(np.dot(m, m)))
        out.append(m / n if n > 0 else m * 0.0)
    return round_to_bf16(np.stack(out))


def int4_mean_shift(C_f64) -> np.ndarray:
    """The shift of the mean-shifted INT4 variant: the column means of C over
    its c rows, rounded to bf16 (t = 1, the data-free choice)."""
    return round_to_bf16(np.asarray(C_f64, dtype=np.float64).mean(axis=0))


def int4_quantize(C_f64, group: int = 128, shift=None):
    """[notes] Module 3 (INT4 stage-1 centroids), symmetric per-group codes.

    For each row k and group g of `group` consecutive columns:
      amax = max |C[k, g]|, s = bf16(amax / 7),
      q = round_half_even(C / s) clipped to [-8, 7]   (q = 0 where s = 0).
    With `shift` (a d-vector), C - shift is quantized instead: every score
    then moves by the same shift . h, which changes neither the top p nor a
    Gumbel-top-p draw, while the codes cover a narrower range when the rows
    share a common direction.
    Returns (q int8 c x d, s float64 c x G with bf16 values).
    """
    C = np.asarray(C_f64, dtype=np.float64)
    if shift is not None:
        C = C - np.asarray(shift, dtype=np.float64)[None, :]
    c, d = C.shape
    if d % group:
        raise ValueError("d must be a multiple of the group size")
    G = d // group
    Cg = C.reshape(c, G, group)
    amax = np.abs(Cg).max(axis=2)
    s = round_to_bf16(amax / 7.0)
    safe = np.where(s > 0, s, 1.0)
    q = np.rint(Cg / safe[:, :, None])
    q = np.where(s[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(c, d), s


# --------------------------------------------------------------------------
# stage 1 ([notes] Overall architecture, Figure 1: inner products of h with
# the c centroids; Module 3 for the INT4 variant)
# --------------------------------------------------------------------------


def stage1_scores(C_f64, h_f64) -> np.ndarray:
    return np.asarray(C_f64, np.float64) @ np.asarray(h_f64, np.float64)


def stage1_scores_int4(q, s, h_f64, group: int = 128) -> np.ndarray:
    """s_k = sum_g scale[k, g] * sum_{j in g} q[k, j] * h[j]."""
    q = np.asarray(q, dtype=np.float64)
    c, d = q.shape
    G = d // group
    inner = (q.reshape(c, G, group) *
             np.asarray(h_f64, np.float64).reshape(1, G, group)).sum(axis=2)
    return (np.asarray(s, np.float64) * inner).sum(axis=1)


# --------------------------------------------------------------------------
# selection ([notes] Module 2: greedy mode keeps the p clusters with the
# highest centroid logits; sampling mode draws p clusters without
# replacement from the softmax of the (temperature-scaled) centroid logits)
# --------------------------------------------------------------------------


def order_desc(keys) -> np.ndarray:
    """Indices sorted by key descending, ties by index ascending."""
    keys = np.asarray(keys, dtype=np.float64)
    return np.lexsort((np.arange(len(keys)), -keys))


def select_keys(scores, mode: str, tau: float = 1.0, seed: int = 0):
    s = np.asarray(scores, dtype=np.float64)
    if mode == "greedy":
        return s.copy()
    if mode == "sample":
        return s / tau + gumbel(seed, STREAM_CLUSTER, np.arange(len(s)))
    raise ValueError(mode)


def select_clusters(scores, p: int, mode: str = "greedy", tau: float = 1.0,
                    seed: int = 0):
    """Returns (S sorted by key desc, keys, margin m1 between p-th/p+1-th)."""
    keys = select_keys(scores, mode, tau, seed)
    order = order_desc(keys)
    S = order[:p]
    m1 = (keys[order[p - 1]] - keys[order[p]]) if p < len(keys) else math.inf
    return S, keys, m1


# --------------------------------------------------------------------------
# adaptive probe count.  [notes] "Potential improvements" names an adaptive
# number of probes (fewer for easy tokens, more for hard ones) and gives no
# rule.  Reading taken: probe every cluster whose stage-1 softmax weight at
# temperature tau is at least eps times the largest weight, that is every k
# with s_k / tau >= max_j s_j / tau - ln(1 / eps), and clamp the count to
# [p_min, p_max].  Greedy decoding uses tau = 1 for the rule.
# --------------------------------------------------------------------------


def adaptive_p(scores, tau: float, eps: float, p_min: int, p_max: int):
    """Returns (p', margin): p' the clamped count, margin the distance (in
    units of s / tau) from the threshold to the nearest score."""
    if not (0.0 < eps <= 1.0) or not (1 <= p_min <= p_max):
        raise ValueError("need 0 < eps <= 1 and 1 <= p_min <= p_max")
    x = np.asarray(scores, dtype=np.float64) / tau
    thr = x.max() - math.log(1.0 / eps)
    n = int(np.count_nonzero(x >= thr))
    margin = float(np.min(np.abs(x - thr)))
    return min(max(n, p_min), p_max), margin


# --------------------------------------------------------------------------
# stage 2 ([notes] Module 1: the dense c x b table lets candidate i be found
# by modulo arithmetic; Overall architecture: exact logits of the p*b rows)
# --------------------------------------------------------------------------


def candidate_tokens(S, c2t) -> np.ndarray:
    c2t = np.asarray(c2t)
    b = c2t.shape[1]
    i = np.arange(len(S) * b)
    return c2t[np.asarray(S)[i // b], i % b].astype(np.int64)


def exact_logits(rows_f64: Callable, T, h_f64) -> np.ndarray:
    return rows_f64(np.asarray(T)) @ np.asarray(h_f64, np.float64)


def logsumexp(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return float(m + math.log(np.exp(x - m).sum()))


def decode_tokens(T, z, mode: str = "greedy", tau: float = 1.0,
                  seed: int = 0):
    """[notes] Formulas 2 and 3 over the candidate set.

    Greedy: the candidate with the largest logit (ties: smaller token id).
    Sample: Gumbel-max over z/tau with noise keyed by token id, an exact
    draw from softmax(z/tau) restricted to the candidates.
    Returns (token, margin m2 between the top two keys, lse of z/tau).
    """
    T = np.asarray(T, dtype=np.int64)
    z = np.asarray(z, dtype=np.float64)
    if mode == "greedy":
        keys = z.copy()
    elif mode == "sample":
        keys = z / tau + gumbel(seed, STREAM_TOKEN, T)
    else:
        raise ValueError(mode)
    order = np.lexsort((T, -keys))
    tok = int(T[order[0]])
    m2 = (keys[order[0]] - keys[order[1]]) if len(T) > 1 else math.inf
    return tok, m2, logsumexp(z / tau), keys


# --------------------------------------------------------------------------
# one decode step of the head, and the dense head it replaces
# --------------------------------------------------------------------------


@dataclass
class StepResult:
    token: int
    S: np.ndarray            # selected cluster ids, by key descending
    scores: np.ndarray       # stage-1 scores (c)
    keys1: np.ndarray        # stage-1 selection keys (c)
    m1: float
    T: np.ndarray            # candidate token ids (p*b)
    z: np.ndarray            # their exact logits
    keys2: np.ndarray        # decode keys over T
    m2: float
    lse: float
    p: int = 0               # probes used (the adaptive count, or p)
    ma: float = math.inf     # margin of the adaptive count (inf if fixed)


def flashhead_step(rows_f64: Callable, c2t, h_f64, p: int, *,
                   C_f64=None, int4=None, mode: str = "greedy",
                   tau: float = 1.0, seed: int = 0,
                   adaptive=None) -> StepResult:
    """[notes] Overall architecture + Figure 1, in the pages' order.
    adaptive = (p_min, eps): the probe count is adaptive_p(scores, tau (1 for
    greedy), eps, p_min, p) instead of p."""
    if int4 is not None:
        scores = stage1_scores_int4(int4[0], int4[1], h_f64)
    else:
        scores = stage1_scores(C_f64, h_f64)
    ma = math.inf
    if adaptive is not None:
        p_min, eps = adaptive
        p, ma = adaptive_p(scores, tau if mode == "sample" else 1.0, eps, p_min, p)
    S, keys1, m1 = select_clusters(scores, p, mode, tau, seed)
    T = candidate_tokens(S, c2t)
    z = exact_logits(rows_f64, T, h_f64)
    tok, m2, lse, keys2 = decode_tokens(T, z, mode, tau, seed)
    return StepResult(tok, S, scores, keys1, m1, T, z, keys2, m2, lse, p, ma)


def dense_logits(rows_f64: Callable, v: int, h_f64,
                 chunk: int = 16384) -> np.ndarray:
    """[notes] Formula 1: z = E h over the whole vocabulary."""
    out = np.empty(v, dtype=np.float64)
    for lo in range(0, v, chunk):
        idx = np.arange(lo, min(v, lo + chunk))
        out[lo:lo + len(idx)] = rows_f64(idx) @ np.asarray(h_f64, np.float64)
    return out


def dense_head(rows_f64: Callable, v: int, h_f64, mode: str = "greedy",
               tau: float = 1.0, seed: int = 0):
    """Formula 1 followed by Formula 2 (argmax) or 3 (sample, Gumbel-max)."""
    z = dense_logits(rows_f64, v, h_f64)
    tok, m2, lse, _ = decode_tokens(np.arange(v), z, mode, tau, seed)
    return tok, m2, lse, z


def rows_accessor(E, dtype: str) -> Callable[[np.ndarray], np.ndarray]:
    def rows(idx):
        return as_f64(np.asarray(E)[np.asarray(idx)], dtype)
    return rows


# --------------------------------------------------------------------------
# Monte Carlo marginal ([notes] Module 4 and Formula 7): N independent draws
# S_1..S_N of the probed clusters share one stage-1 scoring; draw i gives the
# conditional p(v | h, S_i), the softmax of z / tau over S_i's candidates
# (zero for a token outside them); the estimate of p(v | h) is their mean.
# --------------------------------------------------------------------------


@dataclass
class MCResult:
    prob: np.ndarray         # the estimate for each query token
    per_draw: np.ndarray     # N x Q conditionals p(v | h, S_i)
    lse: np.ndarray          # N: lse of z / tau over each draw's candidates
    m1: np.ndarray           # N: gap between the p-th and (p+1)-th key
    S: list                  # N arrays of selected cluster ids


def mc_marginal(rows_f64: Callable, c2t, h_f64, p: int, tau: float, seeds,
                tokens, *, C_f64=None, int4=None) -> MCResult:
    """[notes] Formula 7 with the draws of Module 2's sampling mode."""
    if int4 is not None:
        scores = stage1_scores_int4(int4[0], int4[1], h_f64)
    else:
        scores = stage1_scores(C_f64, h_f64)
    c2t = np.asarray(c2t)
    c, b = c2t.shape
    cluster_of = np.empty(c * b, dtype=np.int64)
    cluster_of[c2t.reshape(-1)] = np.repeat(np.arange(c), b)
    tokens = np.asarray(tokens, dtype=np.int64)
    zq = exact_logits(rows_f64, tokens, h_f64)
    z_of_cluster = {}        # exact logits of a cluster's rows, computed once
    seeds = [int(x) for x in seeds]
    per_draw = np.zeros((len(seeds), len(tokens)))
    lses = np.zeros(len(seeds))
    m1s = np.zeros(len(seeds))
    Ss = []
    for i, seed in enumerate(seeds):
        S, _, m1 = select_clusters(scores, p, "sample", tau, seed)
        for k in S:
            if k not in z_of_cluster:
                z_of_cluster[k] = exact_logits(rows_f64, c2t[k], h_f64)
        z = np.concatenate([z_of_cluster[k] for k in S])
        lse = logsumexp(z / tau)
        member = np.isin(cluster_of[tokens], S)
        per_draw[i] = np.where(member, np.exp(zq / tau - lse), 0.0)
        lses[i], m1s[i] = lse, m1
        Ss.append(S)
    return MCResult(per_draw.mean(axis=0), per_draw, lses, m1s, Ss)


# --------------------------------------------------------------------------
# equal-size spherical k-means ([notes] Module 1, Formulas 4 and 5)
# --------------------------------------------------------------------------


def unit_rows(X) -> np.ndarray:
    """Rows scaled to unit L2 norm (a zero row stays zero)."""
    X = np.asarray(X, dtype=np.float64)
    n = np.sqrt((X * X).sum(axis=1, keepdims=True))
    return np.divide(X, n, out=np.zeros_like(X), where=n > 0)


def equal_size_assign(S, b: int) -> np.ndarray:
    """Capacity-b assignment of v tokens to c clusters from the cosine table
    S (v x c), v = c * b ([notes] Module 1: every cluster holds exactly b
    tokens; how the pages enforce it is not stated).

    Reading: the (token, cluster) pairs are taken in descending cosine
    (ties: lower token id, then lower cluster id); a pair is kept when the
    token is still unplaced and the cluster has room.  With tokens and
    clusters ranking each other by the same cosine this is the unique
    stable assignment (no token and cluster that both prefer each other to
    what they hold).  Returns C2T, c x b, each row ascending."""
    S = np.asarray(S, dtype=np.float64)
    v, c = S.shape
    assert v == c * b
    ii, kk = np.meshgrid(np.arange(v), np.arange(c), indexing="ij")
    order = np.lexsort((kk.ravel(), ii.ravel(), -S.ravel()))
    owner = np.full(v, -1, dtype=np.int64)
    room = np.full(c, b, dtype=np.int64)
    left = v
    for f in order:
        i, k = divmod(int(f), c)
        if owner[i] < 0 and room[k] > 0:
            owner[i] = k
            room[k] -= 1
            left -= 1
            if left == 0:
                break
    c2t = np.empty((c, b), dtype=np.int64)
    for k in range(c):
        c2t[k] = np.sort(np.nonzero(owner == k)[0])
    return c2t


def unit_cluster_means(rows_f64, c2t) -> np.ndarray:
    """Formula 5 in float64: the mean of each cluster's raw rows, scaled to
    unit norm (a zero mean stays zero)."""
    rows_f64 = np.asarray(rows_f64, dtype=np.float64)
    return unit_rows(np.stack([rows_f64[t].mean(axis=0) for t in np.asarray(c2t)]))


@dataclass
class KMeansResult:
    c2t: np.ndarray        # c x b, rows ascending
    C: np.ndarray          # c x d float64: Formula 5 centroids of c2t
    iters: int             # assignment steps run
    objective: float       # sum of the tokens' cosines in the last assignment


def kmeans_equal_size(rows_f64, c: int, init, max_iter: int) -> KMeansResult:
    """Equal-size spherical k-means ([notes] Module 1; Formula 4 objective:
    the summed cosine of each token to its cluster's unit centroid; Formula 5
    update), in the pages' order: cosines of the unit rows to the current
    centroids, the equal-size assignment, then the centroid update.  The
    initial centroids are the unit rows of the c distinct token ids `init`
    (drawn by the caller).  Stops after max_iter assignments, or earlier
    when an assignment repeats the previous one (the centroids are then
    already its means)."""
    rows_f64 = np.asarray(rows_f64, dtype=np.float64)
    v = rows_f64.shape[0]
    assert v % c == 0 and max_iter >= 1
    init = np.asarray(init, dtype=np.int64)
    assert init.shape == (c,) and len(set(init.tolist())) == c
    assert init.min() >= 0 and init.max() < v
    b = v // c
    X = unit_rows(rows_f64)
    C = X[init]
    prev = None
    for it in range(max_iter):
        S = X @ C.T
        c2t = equal_size_assign(S, b)
        obj = float(sum(S[c2t[k], k].sum() for k in range(c)))
        if prev is not None and np.array_equal(c2t, prev):
            return KMeansResult(c2t, C, it + 1, obj)
        C = unit_cluster_means(rows_f64, c2t)
        prev = c2t
    return KMeansResult(prev, C, max_iter, obj)


# --------------------------------------------------------------------------
# algorithmic work ([notes] Formula 6, [paper] Table 8 parameter counts)
# --------------------------------------------------------------------------


def active_head_params(c: int, d: int, p: int, b: int) -> int:
    """Rows touched per token: c centroids plus p*b candidate rows, d each."""
    return c * d + p * b * d
