"""CPU oracle for CRISP sparse-prefill attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

Everything here is plain NumPy in float64 on the exact values of the inputs
(bf16 inputs are upcast exactly), written to be checked by eye against the
pages it follows:

* [CRISP §2]   CRISP paper, "problem" paragraph: sparse attention restricted to
               an index set S through a mask M_S (0 on S, -inf elsewhere), and
               FlexPrefill's background (proxy attention on a representative
               query subset, vertical = column, slash = diagonal scores, PE
               "flattened, sorted, accumulated" until mass >= gamma).
* [CRISP §3.2] C_struct: proxy mass on the sink window (first w_sink keys) and
               the recency window (last w_local keys); route to Vertical-Slash
               iff C_struct >= tau.
* [CRISP §4]   noise floor: the first and last blocks are always kept, mu is
               the mean residual mass over the other N_b - 2 blocks, a block is
               kept iff its mass exceeds alpha * mu; both directions (vertical
               = column means, slash = diagonal means) are thresholded
               separately and unioned.
* [rcap.io CRISP summary, per-head pseudo-code] where the paper's display
               equations were lost, this summary supplies them: the proxy map is
               the scaled, softmaxed product of the last query block with every
               key; the structural mass is that map's total on the sink and
               recency columns, averaged over the proxy rows; the vertical and
               slash scores are its column and diagonal averages summed per
               block; the floor is the mass left outside the two end blocks
               (never negative) spread over the remaining N_b - 2 blocks; a
               block survives when its score is above alpha times that floor;
               Pooled-Estimation heads use the cumulative-mass cut on block
               means of Q and K at gamma = 0.95.

Readings where the pages are silent (each is repeated in the design notes):
causal mask inside the proxy; C_struct over the union of the two windows;
column/diagonal means divide by b (all b proxy rows, masked entries count 0);
diagonal offset o = q_r - j at token level, bin k = offsets [kb, (k+1)b);
slash bin k selects key block qb - k for query block qb; every list holds the
anchor blocks 0 and qb; PE pools every query block, softmaxes each pooled row
over its causal key blocks and cuts the flattened causal matrix globally
against gamma * sum(P), ties broken by lower flat (row-major) index, plus the
two anchors per row; the min-budget top-up takes the largest remaining score,
ties to the lower index.

Variants the pages compare CRISP against (same proxy, same lists, same
attention; only a decision rule changes):

* [CRISP §2, FlexPrefill background] JSD router: the pooled estimate
               a_bar = softmax over key blocks of the pooled last-block query
               against the block means of K (softmax after pooling), the
               per-query mean a_hat = the block-pooled column mean of A_hat
               (softmax before averaging, i.e. p^v); Vertical-Slash iff
               JSD(a_bar, a_hat) >= tau.
* [CRISP §2, FlexPrefill background] coverage budget for Vertical-Slash:
               each direction sorted by descending score and accumulated until
               the mass reaches gamma, union plus the first and last blocks.
* [CRISP appendix on the noise floor, median alternative] the floor is the
               median of the non-anchor block scores instead of their mean.

Decision arithmetic (route, mu, threshold) is spelled out in float32 in a
fixed order so that, given the GPU's float32 scores, the oracle's decisions are
the exact ones the GPU must reproduce.
"""
from __future__ import annotations

import math
import numpy as np

FLT_MIN = np.float32(np.finfo(np.float32).tiny)
TIE_REL = 1e-6


# =============================================================== stage 1: proxy attention

def proxy_attention(q_last: np.ndarray, k: np.ndarray) -> np.ndarray:
    """A_hat = causal softmax(Q_last K^T / sqrt(d)) for the last query block.

    [rcap.io pseudo-code, first line; CRISP §2 "representative query subset"].
    q_last: [b, d] (rows are the queries at positions n-b .. n-1), k: [n, d].
    Returns A_hat [b, n] in float64; row r is a softmax over keys j <= n-b+r.
    """
    b, d = q_last.shape
    n = k.shape[0]
    s = (q_last.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
    pos = n - b + np.arange(b)
    s[np.arange(n)[None, :] > pos[:, None]] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def vertical_scores(A: np.ndarray, blk: int) -> np.ndarray:
    """p^v: column means of A_hat, pooled into key blocks by summation [CRISP §4]."""
    b, n = A.shape
    a_v = A.sum(axis=0) / b
    return a_v.reshape(n // blk, blk).sum(axis=1)


def slash_scores(A: np.ndarray, blk: int) -> np.ndarray:
    """p^s: diagonal means of A_hat, pooled into offset bins by summation [CRISP §4].

    Diagonal o holds the entries (r, q_r - o), q_r = n - b + r; a_s[o] is their
    sum divided by b; bin k gathers offsets [k*blk, (k+1)*blk).
    """
    b, n = A.shape
    a_s = np.zeros(n)
    for r in range(b):
        q = n - b + r
        a_s[:q + 1] += A[r, q::-1]          # A[r, q - o] for o = 0..q
    a_s /= b
    return a_s.reshape(n // blk, blk).sum(axis=1)


def c_struct(A: np.ndarray, w_sink: int, w_local: int) -> float:
    """Structural mass on the sink and recency windows [CRISP §3.2; rcap.io pseudo-code].

    Sum of A_hat over the union of columns [0, w_sink) and [n - w_local, n),
    divided by the number of proxy rows b.
    """
    b, n = A.shape
    cols = np.zeros(n, bool)
    cols[:min(w_sink, n)] = True
    cols[max(n - w_local, 0):] = True
    return float(A[:, cols].sum() / b)


def proxy_literal(q_last, k, blk, w_sink, w_local):
    """The same three quantities by explicit loops over every (r, j); tiny n only.

    A second, independent transcription used to pin the vectorised version.
    """
    b, d = q_last.shape
    n = k.shape[0]
    A = np.zeros((b, n))
    for r in range(b):
        q = n - b + r
        logits = [sum(float(q_last[r, t]) * float(k[j, t]) for t in range(d)) / math.sqrt(d) for j in range(q + 1)]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        z = sum(w)
        for j in range(q + 1):
            A[r, j] = w[j] / z
    pv = [0.0] * (n // blk)
    ps = [0.0] * (n // blk)
    cs = 0.0
    for r in range(b):
        q = n - b + r
        for j in range(q + 1):
            pv[j // blk] += A[r, j] / b
            ps[(q - j) // blk] += A[r, j] / b
            if j < w_sink or j >= n - w_local:
                cs += A[r, j] / b
    return A, np.array(pv), np.array(ps), cs


# =============================================================== stage 2: routing

def route_decision(c: np.float32, tau: float) -> bool:
    """Vertical-Slash iff C_struct >= tau, compared in float32 [CRISP §3.2]."""
    return bool(np.float32(c) >= np.float32(tau))


def route_tie(c: float, tau: float) -> bool:
    return abs(float(c) - float(tau)) <= TIE_REL * abs(float(tau))


def pooled_estimate(q_last: np.ndarray, k: np.ndarray, blk: int) -> np.ndarray:
    """a_bar: softmax over the key blocks of (mean of the last block's query
    rows) . (block mean of K) / sqrt(d) -- softmax applied after pooling
    queries and keys [CRISP §2, FlexPrefill's pooled estimate].  Every key
    block takes part (all of them precede or contain the last query block)."""
    d = q_last.shape[1]
    qm = q_last.astype(np.float64).mean(axis=0)
    L = block_means(k, blk) @ qm / math.sqrt(d)
    e = np.exp(L - L.max())
    return e / e.sum()


def jsd(a: np.ndarray, b: np.ndarray) -> float:
    """Jensen-Shannon divergence with natural logarithms:
    JSD = KL(a || m)/2 + KL(b || m)/2, m = (a + b)/2, terms with a zero weight
    contribute 0.  Bounded by ln 2."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    m = 0.5 * (a + b)

    def kl(x):
        nz = x > 0
        return float(np.sum(x[nz] * np.log(x[nz] / m[nz])))

    return 0.5 * kl(a) + 0.5 * kl(b)


def route_jsd(j: float, tau: float) -> bool:
    """FlexPrefill's router as the pages state it: Vertical-Slash iff
    JSD(a_bar, a_hat) >= tau [CRISP §2]; the divergence is a float64 value,
    tau the float32 parameter."""
    return bool(float(j) >= float(np.float32(tau)))


# =============================================================== stage 3a: Vertical-Slash selection

def noise_floor_f32(p: np.ndarray) -> np.float32:
    """mu = max(1 - p_0 - p_last, 0) / (N_b - 2) in float32, left to right [CRISP §4]."""
    p = np.asarray(p, np.float32)
    nb = p.shape[0]
    t = np.float32(1.0) - p[0]
    t = np.float32(t - p[nb - 1])
    t = np.float32(max(t, np.float32(0.0)))
    return np.float32(t / np.float32(nb - 2))


def threshold_f32(p: np.ndarray, alpha: float) -> np.float32:
    return np.float32(np.float32(alpha) * noise_floor_f32(p))


def vs_select_direction(p: np.ndarray, alpha: float, min_blocks: int = 0) -> np.ndarray:
    """S_d = {k : p_k > alpha mu_d} plus the anchors 0 and N_b - 1 [CRISP §4].

    With min_blocks > |S_d|, the set is topped up with the largest remaining
    p_k (ties to the lower k) until it holds min_blocks indices.
    Returns the sorted int array of selected indices.
    """
    p = np.asarray(p, np.float32)
    nb = p.shape[0]
    thr = threshold_f32(p, alpha)
    sel = p > thr
    sel[0] = True
    sel[nb - 1] = True
    return _top_up(sel, p, min_blocks)


def median_floor_f32(p: np.ndarray) -> np.float32:
    """Median of the non-anchor scores p_1 .. p_{N_b-2} in float32 [CRISP
    appendix on the noise floor: the median as the robust alternative to the
    mean over non-retained blocks].  For an even count it is the float32 mean
    of the two middle values, (a + b) * 0.5, rounded once per operation."""
    p = np.asarray(p, np.float32)
    r = np.sort(p[1:-1])[::-1]
    m = r.size
    if m % 2:
        return np.float32(r[(m - 1) // 2])
    return np.float32(np.float32(r[m // 2 - 1] + r[m // 2]) * np.float32(0.5))


def vs_select_median(p: np.ndarray, alpha: float, min_blocks: int = 0) -> np.ndarray:
    """S_d = {k : p_k > alpha * median} plus the anchors 0 and N_b - 1, topped up
    like vs_select_direction."""
    p = np.asarray(p, np.float32)
    nb = p.shape[0]
    thr = np.float32(np.float32(alpha) * median_floor_f32(p))
    sel = p > thr
    sel[0] = True
    sel[nb - 1] = True
    return _top_up(sel, p, min_blocks)


def _top_up(sel: np.ndarray, p: np.ndarray, min_blocks: int) -> np.ndarray:
    need = min(min_blocks, sel.size) - int(sel.sum())
    if need > 0:
        rest = np.flatnonzero(~sel)
        order = sorted(rest, key=lambda i: (-float(p[i]), int(i)))
        sel[np.array(order[:need], dtype=int)] = True
    return np.flatnonzero(sel)


def median_ties(p: np.ndarray, alpha: float) -> np.ndarray:
    """Indices whose score lies within 1e-6 relative of alpha * median."""
    p = np.asarray(p, np.float32)
    thr = float(np.float32(np.float32(alpha) * median_floor_f32(p)))
    band = TIE_REL * max(thr, float(FLT_MIN))
    return np.flatnonzero(np.abs(p.astype(np.float64) - thr) <= band)


def coverage_cut(vals: np.ndarray, gamma: float):
    """Shortest prefix of the entries in descending order (ties to the lower
    index) whose sum reaches gamma * sum(vals); gamma >= 1 keeps everything.
    Sums in extended precision.  Returns (kept indices, info) with the same
    info fields as pe_cut."""
    vals = np.asarray(vals, np.float64)
    idx = np.arange(vals.size)
    order = np.lexsort((idx, -vals))
    csum = np.cumsum(vals[order].astype(np.longdouble))
    total = csum[-1] if vals.size else np.longdouble(0)
    if gamma >= 1.0:
        kstar, target = vals.size, total
    else:
        target = np.longdouble(gamma) * total
        kstar = min(int(np.searchsorted(csum, target, side="left")) + 1, vals.size)
    info = dict(kstar=kstar, target=float(target), total=float(total), entries=int(vals.size),
                prefix=float(csum[kstar - 1]) if kstar > 0 else 0.0,
                prefix_before=float(csum[kstar - 2]) if kstar > 1 else 0.0)
    return order[:kstar], info


def vs_select_coverage(p: np.ndarray, gamma: float, min_blocks: int = 0):
    """FlexPrefill's Vertical-Slash budget for one direction [CRISP §2]: the
    blocks sorted by descending score and accumulated until the mass reaches
    gamma of the direction's total, plus the anchors 0 and N_b - 1, topped up
    like vs_select_direction.  Returns (sorted indices, cut info)."""
    p = np.asarray(p, np.float32)
    nb = p.shape[0]
    keep, info = coverage_cut(p.astype(np.float64), gamma)
    sel = np.zeros(nb, bool)
    sel[keep] = True
    sel[0] = True
    sel[nb - 1] = True
    return _top_up(sel, p, min_blocks), info


def vs_ties(p: np.ndarray, alpha: float) -> np.ndarray:
    """Indices whose score lies within 1e-6 relative of the threshold."""
    p = np.asarray(p, np.float32)
    thr = float(threshold_f32(p, alpha))
    band = TIE_REL * max(thr, float(FLT_MIN))
    return np.flatnonzero(np.abs(p.astype(np.float64) - thr) <= band)


def vs_block_lists(sv: np.ndarray, ss: np.ndarray, nb: int) -> list:
    """Key-block list of every query block for a Vertical-Slash head.

    list(qb) = sorted unique ({kb in S_v : kb <= qb} U {qb - k : k in S_s, k <= qb} U {0, qb})
    [CRISP §2: "S_v U S_s plus the first and last blocks"; §4: union of the two
    directions].
    """
    out = []
    sv = np.asarray(sv)
    ss = np.asarray(ss)
    for qb in range(nb):
        s = set(int(x) for x in sv[sv <= qb])
        s |= set(int(qb - x) for x in ss[ss <= qb])
        s |= {0, qb}
        out.append(np.array(sorted(s), dtype=np.int64))
    return out


# =============================================================== stage 3b: Pooled-Estimation selection

def block_means(x: np.ndarray, blk: int) -> np.ndarray:
    """Mean of every block of blk consecutive rows."""
    n, d = x.shape
    return x.astype(np.float64).reshape(n // blk, blk, d).mean(axis=1)


def pe_probabilities(q: np.ndarray, k: np.ndarray, blk: int) -> np.ndarray:
    """Pooled estimate: causal row softmax of pool(Q) pool(K)^T / sqrt(d).

    [rcap.io pseudo-code gamma_cumsum(pool(Q), pool(K)); CRISP §2 "applying
    softmax after pooling both queries and keys"].  Returns P [N_b, N_b] with
    zeros above the diagonal.
    """
    d = q.shape[1]
    qm = block_means(q, blk)
    km = block_means(k, blk)
    L = (qm @ km.T) / math.sqrt(d)
    nb = L.shape[0]
    L[np.triu(np.ones((nb, nb), bool), 1)] = -np.inf
    L -= L.max(axis=1, keepdims=True)
    e = np.exp(L)
    return e / e.sum(axis=1, keepdims=True)


def pe_cut(P: np.ndarray, gamma: float):
    """Global gamma-cumsum over the flattened causal pooled matrix [CRISP §2, PE path].

    Entries (qb, kb <= qb) are ordered by descending P, ties by ascending
    row-major flat index; the shortest prefix whose sum reaches gamma * sum(P)
    is kept; gamma >= 1 keeps everything.  The anchors (qb, 0) and (qb, qb) of
    every row are then added.  Sums are accumulated in extended precision
    (np.longdouble) so that their rounding stays far below any tie band.
    Returns (mask [N_b, N_b] bool, info dict with the cut position and mass).
    """
    P = np.asarray(P, np.float64)
    nb = P.shape[0]
    qi, ki = np.tril_indices(nb)
    vals = P[qi, ki]
    flat = qi * nb + ki
    order = np.lexsort((flat, -vals))
    csum = np.cumsum(vals[order].astype(np.longdouble))
    total = csum[-1] if vals.size else np.longdouble(0)
    mask = np.zeros((nb, nb), bool)
    if gamma >= 1.0:
        kstar = vals.size
        target = total
    else:
        target = np.longdouble(gamma) * total
        kstar = int(np.searchsorted(csum, target, side="left")) + 1
        kstar = min(kstar, vals.size)
    take = order[:kstar]
    mask[qi[take], ki[take]] = True
    mask[np.arange(nb), 0] = True
    mask[np.arange(nb), np.arange(nb)] = True
    info = dict(kstar=kstar, target=float(target), total=float(total), entries=int(vals.size),
                prefix=float(csum[kstar - 1]) if kstar > 0 else 0.0,
                prefix_before=float(csum[kstar - 2]) if kstar > 1 else 0.0,
                cut_value=float(vals[order[kstar - 1]]) if kstar > 0 else 0.0,
                next_value=float(vals[order[kstar]]) if kstar < vals.size else -1.0)
    return mask, info


def pe_tie(info: dict, rel: float = TIE_REL, band: float = 0.0) -> bool:
    """True when gamma*T lies within max(rel * gamma*T, band) of the prefix sum
    just before or at the cut, i.e. where the summation arithmetic of an
    implementation can move the cut by one entry.  Equal values straddling the
    cut are not a tie: the lower flat index wins on every implementation."""
    t = info["target"]
    if t <= 0:
        return False
    eps = max(rel * t, band)
    return bool(abs(info["prefix"] - t) <= eps or abs(info["prefix_before"] - t) <= eps)


def mask_to_lists(mask: np.ndarray) -> list:
    return [np.flatnonzero(mask[qb, :qb + 1]).astype(np.int64) for qb in range(mask.shape[0])]


def lists_to_csr(per_head_lists: list):
    """[[list per qb] per head] -> (row_ptr [H*N_b + 1], col_idx) in head-major order."""
    counts = [len(l) for lists in per_head_lists for l in lists]
    row_ptr = np.zeros(len(counts) + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col = np.concatenate([l for lists in per_head_lists for l in lists]) if counts else np.zeros(0, np.int64)
    return row_ptr, col


def dense_lists(nb: int) -> list:
    return [np.arange(qb + 1, dtype=np.int64) for qb in range(nb)]


# =============================================================== stage 4: attention

def attention_block_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, qb: int, kblocks, blk: int) -> np.ndarray:
    """Rows of query block qb attending causally to the listed key blocks.

    O_i = sum_{j in J_i} softmax_j(q_i . k_j / sqrt(d)) v_j with
    J_i = {j <= i : block(j) in list}  [CRISP §2, mask M_S; exact softmax on
    the selected blocks].  An empty J_i gives a zero row.
    """
    d = q.shape[1]
    rows = np.arange(qb * blk, (qb + 1) * blk)
    kb = np.asarray(sorted(int(x) for x in kblocks), dtype=np.int64)
    if kb.size == 0:
        return np.zeros((blk, v.shape[1]))
    cols = (kb[:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
    s = (q[rows].astype(np.float64) @ k[cols].astype(np.float64).T) / math.sqrt(d)
    s[cols[None, :] > rows[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    out = np.zeros((blk, v.shape[1]))
    ok = np.isfinite(m[:, 0])
    e = np.exp(s[ok] - m[ok])
    out[ok] = (e @ v[cols].astype(np.float64)) / e.sum(axis=1, keepdims=True)
    return out


def block_sparse_attention(q, k, v, lists, blk):
    """Whole-head block-sparse causal attention, one query block at a time."""
    return np.concatenate([attention_block_rows(q, k, v, qb, lists[qb], blk) for qb in range(len(lists))])


def dense_causal_attention(q, k, v):
    """softmax(q k^T / sqrt(d) + causal mask) v, the all-blocks special case."""
    n, d = q.shape
    s = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
    s[np.triu(np.ones((n, n), bool), 1)] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e @ v.astype(np.float64)) / e.sum(axis=1, keepdims=True)


def masked_attention_literal(q, k, v, M):
    """softmax(q k^T / sqrt(d) + M) v with an explicit n x n mask matrix M
    (0 where allowed, -inf elsewhere) [CRISP §2 problem statement]; tiny n."""
    d = q.shape[1]
    s = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d) + M
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        if np.isfinite(s[i]).any():
            e = np.exp(s[i] - s[i].max())
            out[i] = e @ v.astype(np.float64) / e.sum()
    return out


def mask_matrix(lists, n, blk):
    """M_S: 0 on allowed (i, j) (j <= i and block(j) listed for block(i)), -inf elsewhere."""
    M = np.full((n, n), -np.inf)
    for qb, kbs in enumerate(lists):
        for kb in kbs:
            for i in range(qb * blk, (qb + 1) * blk):
                for j in range(kb * blk, (kb + 1) * blk):
                    if j <= i:
                        M[i, j] = 0.0
    return M


# =============================================================== per-head pipeline

def _vs_sets(pv, ps, alpha, gamma, min_blocks, budget):
    """Both Vertical-Slash directions under one budget rule: "mean" (the CRISP
    noise floor), "median" (median floor) or "coverage" (FlexPrefill's
    gamma-cumsum).  Returns (sv, ss, infos)."""
    pv = np.asarray(pv, np.float32)
    ps = np.asarray(ps, np.float32)
    if budget == "mean":
        return vs_select_direction(pv, alpha, min_blocks), vs_select_direction(ps, alpha, min_blocks), None
    if budget == "median":
        return vs_select_median(pv, alpha, min_blocks), vs_select_median(ps, alpha, min_blocks), None
    if budget == "coverage":
        sv, iv = vs_select_coverage(pv, gamma, min_blocks)
        ss, is_ = vs_select_coverage(ps, gamma, min_blocks)
        return sv, ss, (iv, is_)
    raise ValueError(budget)


def select_head(q, k, blk, w_sink, w_local, tau, alpha, gamma, min_blocks=0, dense_below_n=0,
                router="cstruct", budget="mean"):
    """Stages 1-3 for one query head from its own Q [n, d] and its KV head's K.

    Returns a dict with the float64 scores, the decisions and the per-block
    lists.  route is 1 (VS), 0 (PE) or -1 (dense fallback: N_b <= 2, or n below
    the length gate, where mu is undefined or sparsity does not pay).
    router "cstruct" (CRISP) or "jsd" (FlexPrefill); budget "mean" (CRISP),
    "median" or "coverage" (FlexPrefill) for Vertical-Slash heads.
    """
    n = k.shape[0]
    nb = n // blk
    out = dict(nb=nb)
    if nb <= 2 or n < dense_below_n:
        out.update(route=-1, lists=dense_lists(nb))
        return out
    A = proxy_attention(q[n - blk:], k)
    pv, ps = vertical_scores(A, blk), slash_scores(A, blk)
    cs = c_struct(A, w_sink, w_local)
    out.update(pv=pv, ps=ps, c_struct=cs)
    if router == "jsd":
        abar = pooled_estimate(q[n - blk:], k, blk)
        out.update(abar=abar, jsd=jsd(abar, pv))
        vs = route_jsd(out["jsd"], tau)
    else:
        vs = route_decision(np.float32(cs), tau)
    out["route"] = 1 if vs else 0
    if vs:
        sv, ss, infos = _vs_sets(pv, ps, alpha, float(np.float32(gamma)), min_blocks, budget)
        out.update(sv=sv, ss=ss, vs_info=infos, lists=vs_block_lists(sv, ss, nb))
    else:
        P = pe_probabilities(q, k, blk)
        mask, info = pe_cut(P, float(np.float32(gamma)))
        out.update(P=P, pe_info=info, lists=mask_to_lists(mask))
    return out


def decide_from_scores(route_in, c, pv, ps, P, nb, tau, alpha, gamma, min_blocks=0, router="cstruct",
                       budget="mean", abar=None):
    """Stages 2-3 given float32 scores computed elsewhere (the GPU's).

    route_in == -1 marks the dense fallback.  Returns (route, sv, ss, lists,
    info); P is only read for Pooled-Estimation heads.  With router "jsd" the
    route is JSD(abar, pv) >= tau on the given float32 abar and pv; with budget
    "coverage" info holds the two directions' cut infos for VS heads.
    """
    if route_in == -1:
        return -1, None, None, dense_lists(nb), None
    gamma = float(np.float32(gamma))        # the parameter as the float32 it is passed as
    if router == "jsd":
        vs = route_jsd(jsd(np.asarray(abar, np.float32), np.asarray(pv, np.float32)), tau)
    else:
        vs = route_decision(np.float32(c), tau)
    if vs:
        sv, ss, infos = _vs_sets(pv, ps, alpha, gamma, min_blocks, budget)
        return 1, sv, ss, vs_block_lists(sv, ss, nb), infos
    mask, info = pe_cut(np.asarray(P, np.float32).astype(np.float64), gamma)
    return 0, None, None, mask_to_lists(mask), info


def prefill_head(q, k, v, blk=128, w_sink=128, w_local=128, tau=0.3, alpha=1.0, gamma=0.95,
                 min_blocks=0, dense_below_n=0, router="cstruct", budget="mean"):
    """All four stages for one head: selection then block-sparse attention."""
    sel = select_head(q, k, blk, w_sink, w_local, tau, alpha, gamma, min_blocks, dense_below_n, router, budget)
    sel["O"] = block_sparse_attention(q, k, v, sel["lists"], blk)
    return sel
