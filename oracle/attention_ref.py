"""Plain fp64 CPU oracle for exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY. This module is the checker that the HIP library is
compared against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library itself never
does, and this module imports nothing from the library.

Everything here is written for a reader who has the pages open and wants to
check the arithmetic by eye: no blocking, fusion or reordering beyond what the
cited definition or algorithm states.  Arrays are numpy float64; a problem is
one attention head with Q, K, V of shape [N, d].  Batched helpers loop over
leading (batch, head) axes one head at a time.

Sources (page title -> part used):

* "Overview of Flash Attention series", section *Standard Attention
  Implementation / Forward Pass*: S = Q K^T, P = softmax(S) row-wise, O = P V.
* "Transformer 入门" (Transformer primer), *flash attention* definitions:
  S = Q K^T / sqrt(d), m = rowmax(S), l = rowsum(exp(S - m)), and the
  safe-softmax one-liner.
* "FlashAttention in NeurIPS 2022" (coreui blog), section 2.1 *拆分*
  (splitting): the max-shifted softmax, the block-wise update of m and l, and
  the normalised update of the output vector o.
* "Overview of Flash Attention series", section *Tiling* (the two-block
  decomposition of m, f, l) and *Analysis / Correctness*, Theorem 1 (the
  invariants after each K/V block).
* "Как работает FlashAttention математически" (How FlashAttention works
  mathematically), sections 3-4 (online softmax; the running output kept
  un-normalised and divided once at the end).
* "Overview of Flash Attention series", section *Backward Pass of
  flashattention*: dV = P^T dO, dP = dO V^T, D_i = P_i:^T dP_i: = do_i^T o_i,
  dS = P o (dP - D), dq_i = sum_j dS_ij k_j, dk_j = sum_i dS_ij q_i.
* "Overview of Flash Attention series", section *Block-sparse
  Flashattention*: attention under a mask M in {0,1}^{N x N} whose nonzero
  entries come in blocks of a coarser block mask, computed by skipping the
  zero blocks.
* "Как работает FlashAttention математически", section 5 (the backward
  recomputes P from the saved statistics, and dropout masks are not kept as
  N x N arrays) and "Overview of Flash Attention series", Backward Pass
  (masks are regenerated in the backward from what the forward kept).
  Dropout here draws its mask from the counter-based generator Philox4x32-10
  (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
  3", SC 2011), written from that paper's definition.
* "Как работает FlashAttention математически", section 9 (FlashDecoding:
  generation with cached K, V and a single new query token) with the merge
  of partial results over key blocks from "Overview of Flash Attention
  series", section *Tiling* (m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2).

Readings taken where the pages are silent or disagree (each one is listed in
the design notes of the repository):

* The scale factor is an explicit argument applied to S before the softmax;
  the default is 1/sqrt(d) as in the primer's definitions.  Because
  S = scale * Q K^T, the chain rule puts a factor ``scale`` on dQ and dK.
* The causal mask keeps key index <= query index; masked scores are -inf
  (zero weight after the softmax), not 0.
* The stored row statistic is lse_i = m_i + ln l_i = ln sum_j exp(S_ij) over
  the unmasked j, natural log, of the *scaled* scores.
* In the coreui worked example the split is along keys (what the primer calls
  T_c / B_c); a block holds keys [j*Bc, (j+1)*Bc), end exclusive.
* Decoding: the Nq query rows are the last Nq positions of the sequence, so
  with the causal mask query i sees keys 0 .. Nk - Nq + i (the rows line up
  with the end of the key sequence); without it, every key.
* Dropout: the pages name no generator and no layout.  Reading: dropout
  acts on the probabilities after the softmax, O = (P o Z) V / (1 - p), with
  lse that of the undropped scores; the mask Z is a pure function of (seed,
  offset, head, query, key), so the backward regenerates it.  The drop
  probability is quantised to t / 256 (t = round(256 p), 0 <= t <= 255): one
  random byte per element, dropped when the byte is < t.  Element (i, j) of
  head bh takes byte 4 (i mod 4) + (j mod 4) (little-endian within the four
  32-bit words) of Philox4x32-10 at counter (j div 4, i div 4, bh, offset)
  with the 64-bit seed as key.
* FP8 inputs: the pages only name FP8 (for Hopper) without a format or a
  scaling rule.  Reading: Q, K and V are stored in the OCP 8-bit float E4M3
  (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
  infinities, S.1111.111 is NaN; largest finite 448), each tensor with one
  positive descale factor: the value of a stored code c is decode(c) times
  that factor.  What is computed is exact attention of those values; the
  output is bfloat16.
* Block-sparse attention: the page writes softmax(S o 1_M) with masked
  entries set to 0, but its algorithm skips the zero blocks, so they carry no
  weight at all.  Reading: masked entries are excluded (-inf), as for the
  causal mask.  A row with no remaining entry has O = 0 and lse = -inf (the
  empty sum).

Parity status: every public function here is pinned by tests/test_oracle.py
(page worked example, closed forms, library cross-checks, brute force,
finite differences); none is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "default_scale",
    "scores",
    "softmax_stats",
    "forward_head",
    "forward",
    "forward_rows",
    "backward_head",
    "backward",
    "online_softmax_blocks",
    "blockwise_forward_head",
    "brute_force_forward_head",
    "finite_difference_grads",
    "expand_block_mask",
    "forward_block_sparse_head",
    "forward_block_sparse",
    "backward_block_sparse_head",
    "backward_block_sparse",
    "decode_head",
    "decode",
    "merge_partials",
    "split_kv_decode_head",
    "philox4x32",
    "dropout_threshold",
    "dropout_keep_mask",
    "dropout_keep_rows",
    "forward_dropout_head",
    "forward_dropout_rows",
    "backward_dropout_head",
    "finite_difference_grads_dropout",
    "e4m3_decode",
    "forward_fp8_head",
    "fp8_p_rounding_bound",
]


def default_scale(d: int) -> float:
    """1/sqrt(d): the primer's definition S = Q K^T / sqrt(d)."""
    return 1.0 / math.sqrt(d)


def _as_f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T for one head, with S[r, c] = -inf where c > r if causal.

    Standard attention, forward pass ("Overview of Flash Attention series");
    the scale as in the primer's definitions.  q: [Nq, d], k: [Nk, d].
    """
    s = scale * (_as_f64(q) @ _as_f64(k).T)
    if causal:
        nq, nk = s.shape
        rows = np.arange(nq)[:, None]
        cols = np.arange(nk)[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def softmax_stats(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row-wise safe softmax of a score matrix: returns (P, m, l).

    m = rowmax(S), f = exp(S - m), l = rowsum(f), P = f / l
    (coreui blog section 2.1; primer definitions of m and l).
    """
    m = np.max(s, axis=-1)
    f = np.exp(s - m[..., None])
    l = np.sum(f, axis=-1)
    p = f / l[..., None]
    return p, m, l


def forward_head(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """Standard attention for one head: returns (O, lse).

    S = scale Q K^T (masked if causal), P = softmax(S), O = P V,
    lse = m + ln l.  Materialises the N x N matrices S and P, which is
    exactly what the tiled method avoids; this is the definition it must
    reproduce (Theorem 1, "Overview of Flash Attention series").
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, m, l = softmax_stats(s)
    o = p @ v
    lse = m + np.log(l)
    return o, lse


def _loop_heads(fn, arrays, *args):
    """Apply a one-head function over the leading axes of [..., N, d] arrays."""
    lead = arrays[0].shape[:-2]
    outs = None
    for idx in np.ndindex(*lead):
        res = fn(*[a[idx] for a in arrays], *args)
        if outs is None:
            outs = [np.empty(lead + r.shape, dtype=np.float64) for r in res]
        for o, r in zip(outs, res):
            o[idx] = r
    return tuple(outs)


def forward(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """Standard attention over [..., N, d] inputs, one head at a time."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    return _loop_heads(forward_head, (q, k, v), causal, scale)


def forward_rows(q, k, v, rows, causal: bool = False, scale: Optional[float] = None,
                 q_selected: bool = False):
    """Standard attention restricted to the query rows ``rows`` of one head.

    The same definition as :func:`forward_head`, evaluated only for the listed
    query indices (each output row depends on its own query row and on all of
    K and V, with the causal mask taken at the row's own index).  Used to
    check sampled outputs of full-size problems.  With ``q_selected`` q holds
    just the listed rows, in the order of ``rows``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scale * ((q if q_selected else q[rows]) @ k.T)
    if causal:
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows[:, None], -np.inf, s)
    p, m, l = softmax_stats(s)
    return p @ v, m + np.log(l)


def backward_head(q, k, v, do, causal: bool = False, scale: Optional[float] = None):
    """Naive chain-rule backward of standard attention for one head.

    With S = scale Q K^T, P = softmax(S), O = P V and upstream gradient dO
    ("Overview of Flash Attention series", Backward Pass):
      dV = P^T dO
      dP = dO V^T
      D_i = P_i:^T dP_i:            (the row term of the softmax Jacobian)
      dS = P o (dP - D)            (elementwise, D broadcast along rows)
      dQ = scale * dS K            (dq_i = sum_j dS_ij k_j, times scale)
      dK = scale * dS^T Q          (dk_j = sum_i dS_ij q_i, times scale)
    Returns (dQ, dK, dV).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, _, _ = softmax_stats(s)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1)
    ds = p * (dp - dsum[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward(q, k, v, do, causal: bool = False, scale: Optional[float] = None):
    """Chain-rule backward over [..., N, d] inputs, one head at a time."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if scale is None:
        scale = default_scale(q.shape[-1])
    return _loop_heads(backward_head, (q, k, v, do), causal, scale)


def online_softmax_blocks(s_row, v, block: int):
    """The coreui blog's block-by-block softmax of one score row, with output.

    Section 2.1 of "FlashAttention in NeurIPS 2022": start from m = -inf,
    l = 0, o = 0; for each key block i with local max m_i, numerator vector
    p_i = exp(s_block - m_i) and local sum l_i:
      m_new = max(m, m_i)
      l_new = exp(m - m_new) * l + exp(m_i - m_new) * l_i
      o_new = (l * exp(m - m_new) * o + exp(m_i - m_new) * p_i V_i) / l_new
    Returns the list of (m, l, o) after each block.
    """
    s_row = _as_f64(s_row)
    v = _as_f64(v)
    m = -np.inf
    l = 0.0
    o = np.zeros(v.shape[1], dtype=np.float64)
    history = []
    for start in range(0, s_row.shape[0], block):
        blk = s_row[start:start + block]
        m_i = np.max(blk)
        p_i = np.exp(blk - m_i)
        l_i = np.sum(p_i)
        m_new = max(m, m_i)
        a_old = math.exp(m - m_new) if m > -np.inf else 0.0
        a_new = math.exp(m_i - m_new)
        l_new = a_old * l + a_new * l_i
        o = (l * a_old * o + a_new * (p_i @ v[start:start + block])) / l_new
        m, l = m_new, l_new
        history.append((m, l, o.copy()))
    return history


def _block_stats(s_blk, v_blk):
    """One key block's own softmax statistics for each score row:
    m_b = rowmax(S_b), f_b = exp(S_b - m_b), l_b = rowsum(f_b), and the
    block's un-normalised output f_b V_b.  A row whose scores in the block
    are all -inf (masked) has m_b = -inf, l_b = 0 and output 0."""
    m_b = np.max(s_blk, axis=1)
    safe = np.where(np.isfinite(m_b), m_b, 0.0)
    f_b = np.exp(s_blk - safe[:, None])          # exp(-inf) = 0 for masked entries
    return m_b, np.sum(f_b, axis=1), f_b @ v_blk


def _fold(m1, l1, o1, m2, l2, o2, normalised: bool):
    """Combine the statistics of two disjoint key blocks, row by row, by the
    decomposition of the softmax over a concatenated vector x = [x1, x2]
    ("Overview of Flash Attention series", Tiling; the same update of m and l
    in section 2.1 of "FlashAttention in NeurIPS 2022"):
      m = max(m1, m2),  l = e^(m1 - m) l1 + e^(m2 - m) l2,
    and for the output either the un-normalised sum
      O~ = e^(m1 - m) O~1 + e^(m2 - m) O~2
    or, with each O_k normalised by its own l_k,
      O = (e^(m1 - m) l1 O1 + e^(m2 - m) l2 O2) / l.
    A side whose m is -inf (no unmasked score yet) carries weight 0."""
    m = np.maximum(m1, m2)
    safe = np.where(np.isfinite(m), m, 0.0)
    w1 = np.where(np.isfinite(m1), np.exp(m1 - safe), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(m2 - safe), 0.0)
    l = w1 * l1 + w2 * l2
    if not normalised:
        return m, l, w1[:, None] * o1 + w2[:, None] * o2
    with np.errstate(invalid="ignore", divide="ignore"):
        inv = np.where(l > 0, 1.0 / l, 0.0)
    return m, l, (inv * w1 * l1)[:, None] * o1 + (inv * w2 * l2)[:, None] * o2


def blockwise_forward_head(q, k, v, block_q: int, block_k: int, causal: bool = False,
                           scale: Optional[float] = None, form: str = "deferred",
                           check_invariants: bool = False):
    """Tiled forward for one head: returns (O, lse).

    Q is cut into blocks of ``block_q`` rows and K, V into blocks of
    ``block_k`` rows (primer: T_r = ceil(N/B_r), T_c = ceil(N/B_c)); the
    query blocks are independent (the primer's "V2" order, Q outer; the
    result does not depend on the order).  For a query block the statistics
    (m, l, O) start as those of no keys at all (-inf, 0, 0), and each key
    block in turn is folded in: its own statistics (:func:`_block_stats`)
    are combined with the running ones by the two-block decomposition of
    the softmax (:func:`_fold`).  The output is kept either

    * ``form="normalised"``: O normalised after every block (the running
      output of section 2.1 of "FlashAttention in NeurIPS 2022"), or
    * ``form="deferred"``: un-normalised, divided by l once after the last
      block ("Как работает FlashAttention математически", section 4).

    lse = m + ln l at the end.  With ``check_invariants`` the invariants of
    Theorem 1 ("Overview of Flash Attention series", Correctness) are
    asserted after each key block: m = rowmax of the scores seen so far,
    l = rowsum(exp(S_seen - m)), and the normalised O = softmax(S_seen) V_seen.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if form not in ("deferred", "normalised"):
        raise ValueError(form)
    normalised = form == "normalised"
    n_q, d = q.shape
    n_k = k.shape[0]
    if scale is None:
        scale = default_scale(d)
    o_all = np.zeros((n_q, v.shape[1]))
    lse_all = np.zeros(n_q)
    s_full = scores(q, k, scale, causal) if check_invariants else None
    for qs in range(0, n_q, block_q):
        rows = np.arange(qs, min(qs + block_q, n_q))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        o = np.zeros((rows.size, v.shape[1]))
        for ks in range(0, n_k, block_k):
            cols = np.arange(ks, min(ks + block_k, n_k))
            s_blk = scale * (q[rows] @ k[cols].T)
            if causal:
                s_blk = np.where(cols[None, :] > rows[:, None], -np.inf, s_blk)
            m_b, l_b, o_b = _block_stats(s_blk, v[cols])
            if normalised:
                with np.errstate(invalid="ignore", divide="ignore"):
                    o_b = np.where(l_b[:, None] > 0, o_b / l_b[:, None], 0.0)
            m, l, o = _fold(m, l, o, m_b, l_b, o_b, normalised)
            if check_invariants:
                seen = s_full[rows][:, :cols[-1] + 1]
                ref_m = np.max(seen, axis=1)
                assert np.array_equal(np.isfinite(ref_m), np.isfinite(m))
                fin = np.isfinite(ref_m)
                np.testing.assert_allclose(m[fin], ref_m[fin], rtol=0, atol=1e-12)
                ref_l = np.sum(np.exp(seen[fin] - ref_m[fin][:, None]), axis=1)
                np.testing.assert_allclose(l[fin], ref_l, rtol=1e-12, atol=0)
                ref_o = (np.exp(seen[fin] - ref_m[fin][:, None]) / ref_l[:, None]) @ v[:cols[-1] + 1]
                got_o = o[fin] if normalised else o[fin] / l[fin][:, None]
                np.testing.assert_allclose(got_o, ref_o, rtol=1e-12, atol=1e-12)
        if not normalised:
            o = o / l[:, None]
        o_all[rows] = o
        lse_all[rows] = m + np.log(l)
    return o_all, lse_all


def brute_force_forward_head(q, k, v, causal: bool = False, scale: Optional[float] = None, allowed=None):
    """Attention by scalar loops with math.exp, for tiny problems only.

    Each output row o_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij) with
    s_ij = scale * sum_c q_ic k_jc ("Overview of Flash Attention series",
    Forward Pass of flashattention: the normaliser L_i and o_i written per
    row), evaluated with a max shift for range.  No numpy arithmetic, so it
    shares no code path with :func:`forward_head`.  ``allowed(i, j)``, if
    given, further restricts the keys of row i (block-sparse masks); a row
    with no key left gets o_i = 0 and lse_i = -inf.
    """
    q = [[float(x) for x in row] for row in np.asarray(q)]
    k = [[float(x) for x in row] for row in np.asarray(k)]
    v = [[float(x) for x in row] for row in np.asarray(v)]
    n_q, d = len(q), len(q[0])
    dv = len(v[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_rows: List[List[float]] = []
    lse_rows: List[float] = []
    for i in range(n_q):
        keys = [j for j in range(len(k)) if not (causal and j > i) and (allowed is None or allowed(i, j))]
        if not keys:
            o_rows.append([0.0] * dv)
            lse_rows.append(-math.inf)
            continue
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        o_rows.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot for c in range(dv)])
        lse_rows.append(mx + math.log(tot))
    return np.array(o_rows), np.array(lse_rows)


def finite_difference_grads(q, k, v, g, causal: bool = False, scale: Optional[float] = None,
                            h: float = 1e-6):
    """Central differences of phi(Q, K, V) = sum(O * G) for one head.

    The gradient of phi with respect to O is G, so these are the dQ, dK, dV
    that the backward must return for dO = G.  Every element is perturbed by
    +-h in turn; tiny problems only.
    """
    q, k, v, g = _as_f64(q).copy(), _as_f64(k).copy(), _as_f64(v).copy(), _as_f64(g)
    if scale is None:
        scale = default_scale(q.shape[-1])

    def phi():
        o, _ = forward_head(q, k, v, causal, scale)
        return float(np.sum(o * g))

    grads = []
    for x in (q, k, v):
        gx = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = phi()
            x[idx] = keep - h
            dn = phi()
            x[idx] = keep
            gx[idx] = (up - dn) / (2.0 * h)
        grads.append(gx)
    return tuple(grads)


def expand_block_mask(block_mask, n_q: int, n_k: int, block_q: int, block_k: int) -> np.ndarray:
    """Element mask of a block mask: M[r, c] = B[r // block_q, c // block_k].

    "Overview of Flash Attention series", Block-sparse Flashattention: the
    mask M in {0,1}^{N x N} is constant on blocks of block_q query rows by
    block_k keys, and B says which blocks are kept.  Returns a bool [n_q, n_k].
    """
    b = np.asarray(block_mask) != 0
    rows = np.arange(n_q) // block_q
    cols = np.arange(n_k) // block_k
    return b[rows[:, None], cols[None, :]]


def forward_block_sparse_head(q, k, v, block_mask, block_q: int, block_k: int, causal: bool = False,
                              scale: Optional[float] = None):
    """Block-sparse attention for one head: returns (O, lse).

    S = scale Q K^T; entries outside the expanded block mask (and, if causal,
    keys after the query) are excluded, P = softmax of what remains in each
    row, O = P V, lse = m + ln l ("Overview of Flash Attention series",
    Block-sparse Flashattention, with masked entries excluded as the
    block-skipping algorithm does).  A row with no remaining entry has
    O = 0 and lse = -inf.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    keep = expand_block_mask(block_mask, q.shape[0], k.shape[0], block_q, block_k)
    s = np.where(keep, s, -np.inf)
    empty = np.all(np.isneginf(s), axis=-1)
    o = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    if np.any(~empty):
        p, m, l = softmax_stats(s[~empty])
        o[~empty] = p @ v
        lse[~empty] = m + np.log(l)
    return o, lse


def forward_block_sparse(q, k, v, block_mask, block_q: int, block_k: int, causal: bool = False,
                         scale: Optional[float] = None):
    """Block-sparse attention over [B, H, N, d] inputs, one head at a time.

    ``block_mask`` is [Hm, ceil(N / block_q), ceil(N / block_k)] with Hm = 1
    (one mask for every head) or Hm = H (one per head, shared by the batch).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    bm = np.asarray(block_mask)
    B, H = q.shape[0], q.shape[1]
    o = np.empty(q.shape[:-1] + (v.shape[-1],))
    lse = np.empty(q.shape[:-1])
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_block_sparse_head(q[b, h], k[b, h], v[b, h], bm[h if bm.shape[0] > 1 else 0],
                                                           block_q, block_k, causal, scale)
    return o, lse


def backward_block_sparse_head(q, k, v, do, block_mask, block_q: int, block_k: int, causal: bool = False,
                               scale: Optional[float] = None):
    """Chain-rule backward of block-sparse attention for one head: (dQ, dK, dV).

    The same steps as :func:`backward_head` ("Overview of Flash Attention
    series", Backward Pass), on the P of :func:`forward_block_sparse_head`:
    excluded entries have P = 0, so they pass no gradient, and a row that
    keeps no entry has P = 0 throughout (its O is 0 and nothing depends on
    its scores).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    keep = expand_block_mask(block_mask, q.shape[0], k.shape[0], block_q, block_k)
    s = np.where(keep, s, -np.inf)
    empty = np.all(np.isneginf(s), axis=-1)
    p = np.zeros_like(s)
    if np.any(~empty):
        p[~empty], _, _ = softmax_stats(s[~empty])
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1)
    ds = p * (dp - dsum[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def backward_block_sparse(q, k, v, do, block_mask, block_q: int, block_k: int, causal: bool = False,
                          scale: Optional[float] = None):
    """Block-sparse backward over [B, H, N, d] inputs, one head at a time (mask as
    in :func:`forward_block_sparse`)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if scale is None:
        scale = default_scale(q.shape[-1])
    bm = np.asarray(block_mask)
    out = [np.empty(q.shape) for _ in range(3)]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            g = backward_block_sparse_head(q[b, h], k[b, h], v[b, h], do[b, h], bm[h if bm.shape[0] > 1 else 0],
                                           block_q, block_k, causal, scale)
            for x, y in zip(out, g):
                x[b, h] = y
    return tuple(out)


def decode_head(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """Attention of Nq new query rows over Nk cached keys, one head: (O, lse).

    The queries are the last Nq positions of the sequence: with ``causal``,
    query i sees keys 0 .. Nk - Nq + i; without it, all Nk keys
    ("Как работает FlashAttention математически", section 9, FlashDecoding:
    K, V cached, Q the new token(s)).  q: [Nq, d]; k, v: [Nk, d].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        rows = np.arange(nq)[:, None] + (nk - nq)
        cols = np.arange(nk)[None, :]
        s = np.where(cols > rows, -np.inf, s)
    p, m, l = softmax_stats(s)
    return p @ v, m + np.log(l)


def decode(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """:func:`decode_head` over [B, H, Nq, d] queries and [B, H, Nk, d] keys/values."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    o = np.empty(q.shape[:-1] + (v.shape[-1],))
    lse = np.empty(q.shape[:-1])
    for idx in np.ndindex(*q.shape[:-2]):
        o[idx], lse[idx] = decode_head(q[idx], k[idx], v[idx], causal, scale)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Merge attention results over disjoint key blocks into one.

    Each part s holds O_s = softmax over its keys times V and lse_s = ln of
    its normaliser.  With lse = ln sum_s e^(lse_s), the whole-row result is
    O = sum_s e^(lse_s - lse) O_s ("Overview of Flash Attention series",
    Tiling: the two-block decomposition of m and l, written with lse = m +
    ln l).  A part whose keys were all masked has lse_s = -inf and weight 0.
    o_parts: [S, Nq, d]; lse_parts: [S, Nq].
    """
    o_parts, lse_parts = _as_f64(o_parts), _as_f64(lse_parts)
    m = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - m[None, :])
    tot = np.sum(w, axis=0)
    lse = m + np.log(tot)
    o = np.sum(w[:, :, None] * o_parts, axis=0) / tot[:, None]
    return o, lse


def split_kv_decode_head(q, k, v, splits: int, causal: bool = False, scale: Optional[float] = None):
    """Split-KV decoding by the algorithm's steps: cut the Nk keys into
    ``splits`` consecutive chunks, attend to each chunk alone (partial O and
    lse per chunk; queries with no visible key in a chunk get lse = -inf),
    then merge the partials with :func:`merge_partials`."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    nq, nk = q.shape[0], k.shape[0]
    bounds = np.linspace(0, nk, splits + 1).round().astype(int)
    o_parts, lse_parts = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        s = scale * (q @ k[a:b].T)
        if causal:
            rows = np.arange(nq)[:, None] + (nk - nq)
            cols = np.arange(a, b)[None, :]
            s = np.where(cols > rows, -np.inf, s)
        o_s = np.zeros((nq, v.shape[1]))
        lse_s = np.full(nq, -np.inf)
        live = ~np.all(np.isneginf(s), axis=1) if s.shape[1] else np.zeros(nq, dtype=bool)
        if np.any(live):
            p, m, l = softmax_stats(s[live])
            o_s[live] = p @ v[a:b]
            lse_s[live] = m + np.log(l)
        o_parts.append(o_s)
        lse_parts.append(lse_s)
    return merge_partials(np.stack(o_parts), np.stack(lse_parts))


# --- Dropout with a regenerated mask ---------------------------------------

_M32 = 0xFFFFFFFF
# Philox4x32 multipliers and Weyl key increments, as published by Salmon et al.
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)


def philox4x32(counter, key, rounds: int = 10) -> np.ndarray:
    """Philox4x32-R of Salmon, Moraes, Dror and Shaw (SC 2011).

    counter: integers [..., 4] (32-bit words), key: [..., 2] (broadcastable).
    One round maps (c0, c1, c2, c3) with key (k0, k1) to
      (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0)),
    hi/lo being the upper/lower 32 bits of the 64-bit product; the key is
    bumped by the Weyl constants (W0, W1) before every round after the first.
    Returns the four 32-bit output words as uint64 values [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & np.uint64(_M32)
    k = np.asarray(key, dtype=np.uint64) & np.uint64(_M32)
    c0, c1, c2, c3 = (c[..., n] for n in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    m0, m1 = np.uint64(_PHILOX_M[0]), np.uint64(_PHILOX_M[1])
    mask, sh = np.uint64(_M32), np.uint64(32)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & mask
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & mask
        p0 = m0 * c0
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> sh) ^ c1 ^ k0, p1 & mask, (p0 >> sh) ^ c3 ^ k1, p0 & mask)
    return np.stack([c0, c1, c2, c3], axis=-1)


def dropout_threshold(p_drop: float) -> int:
    """t = round(256 p) in float32 arithmetic (half away from zero): an element is
    dropped when its random byte is < t, so the drop probability is t / 256."""
    t = int(math.floor(float(np.float32(np.float32(p_drop) * np.float32(256.0))) + 0.5))
    if not 0 <= t <= 255:
        raise ValueError("dropout probability must round to t / 256 with 0 <= t <= 255")
    return t


def dropout_keep_mask(bh: int, n_q: int, n_k: int, seed: int, offset: int, t: int) -> np.ndarray:
    """Keep mask Z [n_q, n_k] (bool) of head index ``bh`` (= b * H + h).

    Element (i, j) uses byte 4 (i % 4) + (j % 4) of
    philox4x32(counter=(j // 4, i // 4, bh, offset), key=(seed low, seed high)),
    bytes numbered little-endian within the four output words; kept when
    that byte is >= t.
    """
    return dropout_keep_rows(bh, np.arange(n_q), n_k, seed, offset, t)


def dropout_keep_rows(bh: int, rows, n_k: int, seed: int, offset: int, t: int) -> np.ndarray:
    """The rows ``rows`` (query indices) of :func:`dropout_keep_mask`: [len(rows), n_k]
    bool, the same definition evaluated only there (for sampled checks of long
    sequences)."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_k)
    qg = (rows // 4)[:, None]
    kg = (cols // 4)[None, :]
    ctr = np.stack(np.broadcast_arrays(kg, qg, np.full_like(qg, bh), np.full_like(qg, offset)), axis=-1)
    key = np.array([seed & _M32, (seed >> 32) & _M32], dtype=np.uint64)
    words = philox4x32(ctr, key)                                    # [n_q, n_k, 4]
    word = np.take_along_axis(words, (rows % 4)[:, None, None].repeat(n_k, axis=1), axis=-1)[..., 0]
    byte = (word >> (8 * (cols % 4)).astype(np.uint64)[None, :]) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def forward_dropout_head(q, k, v, keep, t: int, causal: bool = False, scale: Optional[float] = None):
    """Attention with dropout on the probabilities, one head: returns (O, lse).

    P = softmax(S) as in :func:`forward_head`; O = (P o Z) V / (1 - t/256)
    with the keep mask Z = ``keep``; lse is that of the undropped S.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, m, l = softmax_stats(s)
    rs = 256.0 / (256.0 - t)
    o = (p * keep * rs) @ v
    return o, m + np.log(l)


def forward_dropout_rows(q, k, v, rows, keep_rows, t: int, causal: bool = False, scale: Optional[float] = None,
                         q_selected: bool = False):
    """:func:`forward_dropout_head` restricted to the query rows ``rows`` (the
    row-wise definition, as :func:`forward_rows`); ``keep_rows`` are those rows
    of the keep mask (:func:`dropout_keep_rows`).  Returns (O rows, lse rows)."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scale * ((q if q_selected else q[rows]) @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    p, m, l = softmax_stats(s)
    rs = 256.0 / (256.0 - t)
    return (p * keep_rows * rs) @ v, m + np.log(l)


def backward_dropout_head(q, k, v, do, keep, t: int, causal: bool = False, scale: Optional[float] = None):
    """Chain-rule backward of :func:`forward_dropout_head` for one head.

    With Pd = P o Z / (1 - t/256) and O = Pd V:
      dV = Pd^T dO
      dP = (dO V^T) o Z / (1 - t/256)      (gradient reaching P through the mask)
      D_i = P_i:^T dP_i:                   (= do_i . o_i, as without dropout)
      dS = P o (dP - D)
      dQ = scale * dS K,   dK = scale * dS^T Q
    Returns (dQ, dK, dV).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, _, _ = softmax_stats(s)
    rs = 256.0 / (256.0 - t)
    zr = keep * rs
    dv = (p * zr).T @ do
    dp = (do @ v.T) * zr
    dsum = np.sum(p * dp, axis=-1)
    ds = p * (dp - dsum[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), dv


def finite_difference_grads_dropout(q, k, v, g, keep, t: int, causal: bool = False,
                                    scale: Optional[float] = None, h: float = 1e-6):
    """Central differences of sum(O * G) for the dropout forward with a fixed
    keep mask (tiny problems only); see :func:`finite_difference_grads`."""
    q, k, v, g = _as_f64(q).copy(), _as_f64(k).copy(), _as_f64(v).copy(), _as_f64(g)
    if scale is None:
        scale = default_scale(q.shape[-1])

    def phi():
        o, _ = forward_dropout_head(q, k, v, keep, t, causal, scale)
        return float(np.sum(o * g))

    grads = []
    for x in (q, k, v):
        gx = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep_val = x[idx]
            x[idx] = keep_val + h
            up = phi()
            x[idx] = keep_val - h
            dn = phi()
            x[idx] = keep_val
            gx[idx] = (up - dn) / (2.0 * h)
        grads.append(gx)
    return tuple(grads)


# --- FP8 (OCP E4M3) inputs -------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP E4M3 codes (uint8 array) as float64.

    Bit 7 is the sign, bits 6..3 the exponent e (bias 7), bits 2..0 the
    mantissa m: e > 0 gives (1 + m/8) 2^(e - 7), e = 0 the subnormal
    (m/8) 2^(-6); exponent and mantissa all ones (0x7F, 0xFF) is NaN.  There
    are no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e - 7.0), (m / 8.0) * 2.0 ** -6)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def forward_fp8_head(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                     causal: bool = False, scale: Optional[float] = None):
    """Attention of E4M3-stored inputs, one head: (O, lse) of the decoded,
    descaled Q, K, V by the definition of :func:`forward_head`."""
    q = e4m3_decode(q8) * q_descale
    k = e4m3_decode(k8) * k_descale
    v = e4m3_decode(v8) * v_descale
    if scale is None:
        scale = default_scale(q.shape[-1])
    return forward_head(q, k, v, causal, scale)


def fp8_p_rounding_bound(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                         causal: bool = False, scale: Optional[float] = None, lazy: float = 2.0 ** 8):
    """Elementwise bound [N, d] on |O_computed - O| when the probabilities are
    rounded to E4M3 before they multiply V (the scores, l and the products
    themselves exact up to fp32).

    A probability is rounded as p' = e^(s - c) for some shift c with
    m - ln(lazy) <= c <= m (m the row max; lazy >= 1 the largest factor by
    which p' may exceed 1) and then divided by the normaliser, which is at
    least sum_j e^(s_j - m).  Rounding to nearest E4M3 errs by at most 2^-4 of
    p' where p' >= 2^-6 (normal numbers, 3 mantissa bits) and by at most
    min(p', 2^-10) below (subnormal spacing 2^-9).  Hence
      |dO_ic| <= sum_j [2^-4 P_ij + min(2^-10, lazy e^(s_ij - m_i)) / L_i] |v_jc|,
    with P the exact probabilities and L_i = sum_j e^(s_ij - m_i).
    """
    q = e4m3_decode(q8) * q_descale
    k = e4m3_decode(k8) * k_descale
    v = np.abs(e4m3_decode(v8) * v_descale)
    if scale is None:
        scale = default_scale(q.shape[-1])
    s = scores(q, k, scale, causal)
    p, m, l = softmax_stats(s)
    f = np.exp(s - m[:, None])                     # e^(s - m); 0 where masked
    sub = np.minimum(2.0 ** -10, lazy * f) / l[:, None]
    return (2.0 ** -4 * p + sub) @ v
