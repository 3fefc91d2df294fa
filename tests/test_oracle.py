"""Pins for the fp64 oracle: it is checked against things other than itself.

* the coreui blog's worked example (section 2.1), stored under tests/golden/
  in the page's own notation and evaluated here with math.exp;
* closed forms (N = 1, K = 0, scale = 0, constant V, causal row 0);
* independent library routines (torch's float64 scaled_dot_product_attention
  and autograd, scipy's logsumexp);
* brute force by scalar loops on tiny inputs;
* central finite differences for the backward;
* invariants the pages state (rows of P sum to 1, block-wise recurrence equals
  the one-shot softmax, Theorem 1's per-block invariants, D_i = do_i . o_i).

All CPU-only.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_softmax.json")


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _page_sum(terms):
    return math.fsum(math.exp(a - b) for a, b in terms)


@pytest.fixture(scope="module")
def worked():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example

def test_worked_example_block_history(worked):
    s = np.array(worked["scores"], dtype=np.float64)
    v = np.array(worked["V"], dtype=np.float64)
    hist = ref.online_softmax_blocks(s, v, worked["block"])
    assert len(hist) == len(worked["after_block"])
    for (m, l, o), page in zip(hist, worked["after_block"]):
        assert m == page["m"]
        assert l == pytest.approx(_page_sum(page["l"]), rel=1e-15)
        num = np.zeros(2)
        for a, b, r in page["o_numerator"]:
            num += math.exp(a - b) * v[r]
        o_page = num / _page_sum(page["o_denominator"])
        np.testing.assert_allclose(o, o_page, rtol=1e-14, atol=0)


def test_worked_example_final_equals_softmax_times_v(worked):
    s = np.array(worked["scores"], dtype=np.float64)
    v = np.array(worked["V"], dtype=np.float64)
    den = _page_sum(worked["softmax_shifted_denominator"])
    p_page = np.array([math.exp(a - b) for a, b in worked["softmax_shifted_numerators"]]) / den
    # unshifted form as first printed on the page: e^{s_j} / sum_k e^{s_k}
    p_plain = np.array([math.exp(x) for x in s]) / math.fsum(math.exp(x) for x in s)
    np.testing.assert_allclose(p_page, p_plain, rtol=1e-14)
    m, l, o = ref.online_softmax_blocks(s, v, worked["block"])[-1]
    np.testing.assert_allclose(o, p_page @ v, rtol=1e-14)
    # the final l equals the one-shot shifted denominator
    assert l == pytest.approx(den, rel=1e-15)
    assert m == max(worked["scores"])


@pytest.mark.parametrize("form", ["deferred", "normalised"])
def test_worked_example_as_attention_problem(worked, form):
    """q = [1], k_j = [s_j], scale 1 reproduces the page's score row."""
    s = np.array(worked["scores"], dtype=np.float64)
    v = np.array(worked["V"], dtype=np.float64)
    q = np.ones((1, 1))
    k = s[:, None]
    den = _page_sum(worked["softmax_shifted_denominator"])
    num = sum(math.exp(a - b) * v[r] for (a, b), r in zip(worked["softmax_shifted_numerators"], range(4)))
    o_page = num / den
    lse_page = 10.0 + math.log(den)
    o, lse = ref.blockwise_forward_head(q, k, v, 1, worked["block"], scale=1.0, form=form,
                                        check_invariants=True)
    np.testing.assert_allclose(o[0], o_page, rtol=1e-14)
    assert lse[0] == pytest.approx(lse_page, rel=1e-15)
    o1, lse1 = ref.forward_head(q, k, v, scale=1.0)
    np.testing.assert_allclose(o1[0], o_page, rtol=1e-14)
    assert lse1[0] == pytest.approx(lse_page, rel=1e-15)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 2), (3, 4), (5, 3), (8, 8)])
def test_forward_matches_brute_force(n, d, causal):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d + 1), 3)
    o, lse = ref.forward_head(q, k, v, causal=causal, scale=0.7)
    o_b, lse_b = ref.brute_force_forward_head(q, k, v, causal=causal, scale=0.7)
    np.testing.assert_allclose(o, o_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-12)


def test_forward_rectangular_brute_force():
    q, k, v = _rand((3, 4), 4), _rand((7, 4), 5), _rand((7, 2), 6)
    o, lse = ref.forward_head(q, k, v, scale=0.3)
    o_b, lse_b = ref.brute_force_forward_head(q, k, v, scale=0.3)
    np.testing.assert_allclose(o, o_b, atol=1e-12)
    np.testing.assert_allclose(lse, lse_b, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [None, 0.05, 1.3])
def test_forward_matches_torch_sdpa_float64(causal, scale):
    b, h, n, d = 2, 3, 67, 16
    q, k, v = _rand((b, h, n, d), 7), _rand((b, h, n, d), 8), _rand((b, h, n, d), 9)
    o, lse = ref.forward(q, k, v, causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=0, atol=1e-12)
    sc = ref.default_scale(d) if scale is None else scale
    s = sc * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_forward_rows_equals_full_rows():
    q, k, v = _rand((50, 8), 10), _rand((50, 8), 11), _rand((50, 8), 12)
    rows = [0, 3, 17, 49]
    for causal in (False, True):
        o, lse = ref.forward_head(q, k, v, causal=causal)
        o_r, lse_r = ref.forward_rows(q, k, v, rows, causal=causal)
        np.testing.assert_allclose(o_r, o[rows], atol=1e-13)
        np.testing.assert_allclose(lse_r, lse[rows], atol=1e-13)


def test_closed_form_single_key():
    q, k, v = _rand((1, 6), 13), _rand((1, 6), 14), _rand((1, 6), 15)
    o, lse = ref.forward_head(q, k, v, scale=0.4)
    np.testing.assert_allclose(o, v, rtol=0, atol=0)
    assert lse[0] == pytest.approx(0.4 * float(q[0] @ k[0]), rel=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_zero_keys_and_zero_scale(causal):
    n, d = 9, 5
    q, v = _rand((n, d), 16), _rand((n, d), 17)
    allowed = np.arange(1, n + 1) if causal else np.full(n, n)
    means = np.array([v[: allowed[r]].mean(axis=0) for r in range(n)])
    o, lse = ref.forward_head(q, np.zeros((n, d)), v, causal=causal)
    np.testing.assert_allclose(o, means, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(allowed), atol=1e-14)
    o0, lse0 = ref.forward_head(q, _rand((n, d), 18), v, causal=causal, scale=0.0)
    np.testing.assert_allclose(o0, means, atol=1e-14)
    np.testing.assert_allclose(lse0, np.log(allowed), atol=1e-14)


def test_closed_form_constant_values_and_causal_first_row():
    n, d = 12, 4
    q, k = _rand((n, d), 19), _rand((n, d), 20)
    o, _ = ref.forward_head(q, k, np.full((n, d), 2.5))
    np.testing.assert_allclose(o, 2.5, atol=1e-14)
    v = _rand((n, d), 21)
    o, lse = ref.forward_head(q, k, v, causal=True, scale=0.9)
    np.testing.assert_allclose(o[0], v[0], atol=0)
    assert lse[0] == pytest.approx(0.9 * float(q[0] @ k[0]), rel=1e-15)


def test_rows_of_p_sum_to_one_and_mask_is_exact_zero():
    q, k = _rand((40, 8), 22), _rand((40, 8), 23)
    s = ref.scores(q, k, 0.5, causal=True)
    p, m, l = ref.softmax_stats(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)
    assert np.all(p[np.triu(np.ones((40, 40), bool), 1)] == 0.0)
    assert np.all(p >= 0)


def test_softmax_shift_invariance():
    s = _rand((5, 11), 24, 3.0)
    p, _, _ = ref.softmax_stats(s)
    p2, _, _ = ref.softmax_stats(s + _rand((5, 1), 25, 50.0))
    np.testing.assert_allclose(p, p2, atol=1e-14)
    np.testing.assert_allclose(p, scipy.special.softmax(s, axis=1), atol=1e-15)


def test_causal_prefix_property():
    n, d = 30, 6
    q, k, v = _rand((n, d), 26), _rand((n, d), 27), _rand((n, d), 28)
    o, lse = ref.forward_head(q, k, v, causal=True)
    r = 11
    k2, v2 = k.copy(), v.copy()
    k2[r + 1:] += 5.0
    v2[r + 1:] -= 3.0
    o2, lse2 = ref.forward_head(q, k2, v2, causal=True)
    np.testing.assert_array_equal(o2[: r + 1], o[: r + 1])
    np.testing.assert_array_equal(lse2[: r + 1], lse[: r + 1])
    assert not np.allclose(o2[r + 1:], o[r + 1:])


@pytest.mark.parametrize("form", ["deferred", "normalised"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (5, 2), (16, 3), (7, 7), (64, 64), (33, 65)])
def test_blockwise_equals_one_shot(form, causal, bq, bk):
    n, d = 65, 8
    q, k, v = _rand((n, d), 29, 2.0), _rand((n, d), 30, 2.0), _rand((n, d), 31)
    o, lse = ref.forward_head(q, k, v, causal=causal)
    ob, lseb = ref.blockwise_forward_head(q, k, v, bq, bk, causal=causal, form=form,
                                          check_invariants=(bq * bk <= 256))
    np.testing.assert_allclose(ob, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lseb, lse, rtol=1e-12, atol=1e-12)


def test_blockwise_with_large_key_outliers():
    """Later key blocks raise the running max many times (rescaling path)."""
    n, d = 96, 16
    q, k, v = _rand((n, d), 32, 0.5), _rand((n, d), 33, 0.5), _rand((n, d), 34, 0.5)
    k[np.arange(5, n, 17)] *= 40.0
    o, lse = ref.forward_head(q, k, v, causal=True)
    for form in ("deferred", "normalised"):
        ob, lseb = ref.blockwise_forward_head(q, k, v, 32, 8, causal=True, form=form,
                                              check_invariants=True)
        np.testing.assert_allclose(ob, o, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(lseb, lse, rtol=1e-12, atol=1e-11)


def test_batched_forward_equals_per_head():
    q, k, v = _rand((2, 2, 9, 4), 35), _rand((2, 2, 9, 4), 36), _rand((2, 2, 9, 4), 37)
    o, lse = ref.forward(q, k, v, causal=True)
    for b in range(2):
        for h in range(2):
            o1, l1 = ref.forward_head(q[b, h], k[b, h], v[b, h], causal=True)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)


# ---------------------------------------------------------------- backward pins

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 2), (3, 4), (5, 2), (8, 4)])
def test_backward_matches_finite_differences(n, d, causal):
    q, k, v, g = (_rand((n, d), s) for s in (40, 41, 42, 43))
    dq, dk, dv = ref.backward_head(q, k, v, g, causal=causal, scale=0.8)
    fq, fk, fv = ref.finite_difference_grads(q, k, v, g, causal=causal, scale=0.8)
    np.testing.assert_allclose(dq, fq, rtol=0, atol=1e-7)
    np.testing.assert_allclose(dk, fk, rtol=0, atol=1e-7)
    np.testing.assert_allclose(dv, fv, rtol=0, atol=1e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_float64(causal):
    b, h, n, d = 2, 2, 45, 8
    q, k, v, do = (_rand((b, h, n, d), s) for s in (44, 45, 46, 47))
    dq, dk, dv = ref.backward(q, k, v, do, causal=causal, scale=0.6)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.6)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_d_identity_and_gradient_invariants():
    """D_i = P_i:^T dP_i: = do_i . o_i, and two sums fixed by the softmax."""
    n, d = 33, 8
    q, k, v, do = (_rand((n, d), s) for s in (48, 49, 50, 51))
    for causal in (False, True):
        s = ref.scores(q, k, 0.35, causal)
        p, _, _ = ref.softmax_stats(s)
        o, _ = ref.forward_head(q, k, v, causal=causal, scale=0.35)
        dp = do @ v.T
        np.testing.assert_allclose((p * dp).sum(axis=1), (do * o).sum(axis=1), atol=1e-12)
        dq, dk, dv = ref.backward_head(q, k, v, do, causal=causal, scale=0.35)
        # shifting every key by the same vector adds a per-row constant to S:
        # O is unchanged, so the key gradients sum to zero
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        # shifting every value row by c shifts every output row by c
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_backward_single_key_closed_form():
    q, k, v, do = (_rand((1, 5), s) for s in (52, 53, 54, 55))
    dq, dk, dv = ref.backward_head(q, k, v, do)
    np.testing.assert_allclose(dv, do, atol=0)
    np.testing.assert_allclose(dq, 0.0, atol=0)
    np.testing.assert_allclose(dk, 0.0, atol=0)


# ---------------------------------------------------------------- planted mistakes

def _fd_pin(backward_fn):
    n, d = 4, 3
    q, k, v, g = (_rand((n, d), s) for s in (60, 61, 62, 63))
    got = backward_fn(q, k, v, g, True, 0.8)
    want = ref.finite_difference_grads(q, k, v, g, causal=True, scale=0.8)
    return all(np.allclose(a, b, atol=1e-7) for a, b in zip(got, want))


def test_pins_catch_planted_backward_mistakes():
    """Each plausible slip in the chain rule fails the finite-difference pin."""
    assert _fd_pin(ref.backward_head)

    def no_scale_on_dq(q, k, v, do, causal, scale):
        dq, dk, dv = ref.backward_head(q, k, v, do, causal, scale)
        return dq / scale, dk, dv

    def wrong_d_sign(q, k, v, do, causal, scale):
        s = ref.scores(q, k, scale, causal)
        p, _, _ = ref.softmax_stats(s)
        dp = do @ v.T
        ds = p * (dp + np.sum(p * dp, axis=1)[:, None])
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    def transposed_dv(q, k, v, do, causal, scale):
        dq, dk, _ = ref.backward_head(q, k, v, do, causal, scale)
        s = ref.scores(q, k, scale, causal)
        p, _, _ = ref.softmax_stats(s)
        return dq, dk, p @ do

    def dropped_d(q, k, v, do, causal, scale):
        s = ref.scores(q, k, scale, causal)
        p, _, _ = ref.softmax_stats(s)
        ds = p * (do @ v.T)
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    for bad in (no_scale_on_dq, wrong_d_sign, transposed_dv, dropped_d):
        assert not _fd_pin(bad), bad.__name__


def test_pins_catch_planted_forward_mistakes(worked):
    """A wrong rescale factor in the recurrence fails the worked-example pin."""
    s = np.array(worked["scores"], dtype=np.float64)
    v = np.array(worked["V"], dtype=np.float64)
    page = worked["after_block"][-1]
    num = sum(math.exp(a - b) * v[r] for a, b, r in page["o_numerator"])
    o_page = num / _page_sum(page["o_denominator"])

    def recurrence(alpha_sign):
        m, l, o = -np.inf, 0.0, np.zeros(2)
        for st in range(0, 4, 2):
            blk = s[st:st + 2]
            m_i = blk.max()
            p_i = np.exp(blk - m_i)
            m_new = max(m, m_i)
            a_old = math.exp(alpha_sign * (m - m_new)) if m > -np.inf else 0.0
            a_new = math.exp(m_i - m_new)
            l_new = a_old * l + a_new * p_i.sum()
            o = (l * a_old * o + a_new * (p_i @ v[st:st + 2])) / l_new
            m, l = m_new, l_new
        return o

    np.testing.assert_allclose(recurrence(+1), o_page, rtol=1e-14)
    assert not np.allclose(recurrence(-1), o_page, rtol=1e-6)


def test_the_pages_numpy_exercise_tiled_equals_standard():
    """"Как работает FlashAttention математически", the NumPy exercise: random
    Q, K, V with n = 1024, d = 64, S = Q K^T (no scale), blocks of 128; the
    tiled forward with the online-softmax correction must match standard
    attention within 1e-5 (here, in fp64, far closer), in both forms of the
    recurrence, and so must the backward by recomputation from m and l."""
    n, d, blk = 1024, 64, 128
    q, k, v, g = (_rand((n, d), 790 + i) for i in range(4))
    o_std, lse_std = ref.forward_head(q, k, v, False, 1.0)
    for form in ("deferred", "normalised"):
        o_t, lse_t = ref.blockwise_forward_head(q, k, v, blk, blk, scale=1.0, form=form)
        assert np.max(np.abs(o_t - o_std)) < 1e-5
        np.testing.assert_allclose(o_t, o_std, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse_t, lse_std, rtol=1e-12)
    # backward with recomputation: P rebuilt from the stored lse equals the one-shot P
    dq, dk, dv = ref.backward_head(q, k, v, g, False, 1.0)
    p_re = np.exp(ref.scores(q, k, 1.0, False) - lse_t[:, None])
    p_std, _, _ = ref.softmax_stats(ref.scores(q, k, 1.0, False))
    np.testing.assert_allclose(p_re, p_std, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(p_re.T @ g, dv, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- block-sparse attention
# "Overview of Flash Attention series", Block-sparse Flashattention: a mask
# that is constant on blocks; zero blocks are skipped (no weight at all).

def _block_mask(tq, tk, density, seed):
    return (np.random.default_rng(seed).random((tq, tk)) < density).astype(np.uint8)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_all_ones_is_dense(causal):
    n, d = 40, 8
    q, k, v = (_rand((n, d), 700 + i) for i in range(3))
    ones = np.ones((3, 5), dtype=np.uint8)          # block_q = 16, block_k = 8 (ragged last blocks)
    o, lse = ref.forward_block_sparse_head(q, k, v, ones, 16, 8, causal, 0.4)
    o_d, lse_d = ref.forward_head(q, k, v, causal, 0.4)
    np.testing.assert_allclose(o, o_d, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-13)


@pytest.mark.parametrize("n,bq,bk,causal", [(12, 4, 3, False), (13, 4, 2, True), (9, 2, 4, False), (16, 8, 8, True)])
def test_block_sparse_matches_brute_force(n, bq, bk, causal):
    d = 3
    q, k, v = (_rand((n, d), 710 + i) for i in range(3))
    bm = _block_mask(-(-n // bq), -(-n // bk), 0.5, 77 + n)
    bm[0, 0] = 1
    o, lse = ref.forward_block_sparse_head(q, k, v, bm, bq, bk, causal, 0.7)
    o_b, lse_b = ref.brute_force_forward_head(q, k, v, causal, 0.7, allowed=lambda i, j: bm[i // bq][j // bk] != 0)
    np.testing.assert_allclose(o, o_b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_b, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_matches_torch_sdpa_with_boolean_mask(causal):
    n, d, bq, bk = 48, 16, 16, 8
    q, k, v = (_rand((2, 3, n, d), 720 + i) for i in range(3))
    bm = np.stack([_block_mask(3, 6, 0.45, 90 + h) for h in range(3)])
    bm[:, :, 0] = 1                                  # every row keeps key block 0 (row 0 keeps key 0 when causal)
    o, lse = ref.forward_block_sparse(q, k, v, bm, bq, bk, causal, 0.3)
    keep = np.stack([ref.expand_block_mask(bm[h], n, n, bq, bk) for h in range(3)])   # torch's mask: True = attend
    if causal:
        keep = keep & np.tril(np.ones((n, n), dtype=bool))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(keep)[None], scale=0.3)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=1e-12, atol=1e-13)
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k)
    lse_s = scipy.special.logsumexp(np.where(keep[None], s, -np.inf), axis=-1)
    np.testing.assert_allclose(lse, lse_s, rtol=1e-12)


def test_block_sparse_single_key_block_is_attention_on_that_slice():
    """Keeping only key block c of a row block gives dense attention over the
    keys of that block alone -- fails on a wrong block-to-index mapping."""
    n, d, bq, bk = 32, 8, 8, 4
    q, k, v = (_rand((n, d), 730 + i) for i in range(3))
    bm = np.zeros((4, 8), dtype=np.uint8)
    for r in range(4):
        bm[r, (3 * r + 1) % 8] = 1
    o, lse = ref.forward_block_sparse_head(q, k, v, bm, bq, bk, False, 0.5)
    for r in range(4):
        c = (3 * r + 1) % 8
        rows, cols = slice(r * bq, (r + 1) * bq), slice(c * bk, (c + 1) * bk)
        o_s, lse_s = ref.forward_head(q[rows], k[cols], v[cols], False, 0.5)
        np.testing.assert_allclose(o[rows], o_s, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[rows], lse_s, rtol=1e-13)


def test_block_sparse_empty_row_is_zero_with_minus_inf_lse():
    n, d = 16, 4
    q, k, v = (_rand((n, d), 740 + i) for i in range(3))
    bm = np.array([[1, 0], [0, 0], [0, 1], [1, 1]], dtype=np.uint8)   # block_q = 4, block_k = 8
    o, lse = ref.forward_block_sparse_head(q, k, v, bm, 4, 8, False, 0.5)
    assert np.all(o[4:8] == 0.0) and np.all(np.isneginf(lse[4:8]))
    assert np.all(np.isfinite(lse[:4])) and np.all(np.isfinite(lse[8:]))
    # causal: row block 2 keeps only key block 1 (keys 8..15), so rows 8..15 see keys 8..row
    o_c, lse_c = ref.forward_block_sparse_head(q, k, v, bm, 4, 8, True, 0.5)
    o_r, lse_r = ref.forward_head(q[8:12], k[8:16], v[8:16], True, 0.5)
    np.testing.assert_allclose(o_c[8:12], o_r, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse_c[8:12], lse_r, rtol=1e-13)


def _fd_block_sparse(q, k, v, g, bm, bq, bk, causal, scale, h=1e-6):
    """Central differences of phi = sum(O * G) of the block-sparse forward oracle."""
    out = []
    for x in (q, k, v):
        grad = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            op, _ = ref.forward_block_sparse_head(q, k, v, bm, bq, bk, causal, scale)
            x[idx] = keep - h
            om, _ = ref.forward_block_sparse_head(q, k, v, bm, bq, bk, causal, scale)
            x[idx] = keep
            grad[idx] = np.sum((op - om) * g) / (2 * h)
        out.append(grad)
    return out


@pytest.mark.parametrize("n,bq,bk,causal", [(8, 2, 4, False), (9, 2, 2, True), (10, 4, 3, True), (7, 2, 3, False)])
def test_block_sparse_backward_matches_finite_differences(n, bq, bk, causal):
    """The chain rule on the block-sparse P against central differences of the
    block-sparse forward, with masks that leave some rows empty."""
    d = 3
    q, k, v, g = (_rand((n, d), 750 + i + n) for i in range(4))
    bm = _block_mask(-(-n // bq), -(-n // bk), 0.55, 60 + n + bq)
    bm[-1, :] = 0                          # the last row block keeps nothing: O = 0, no gradient through it
    bm[0, 0] = 1
    dq, dk, dv = ref.backward_block_sparse_head(q, k, v, g, bm, bq, bk, causal, 0.6)
    fq, fk, fv = _fd_block_sparse(q, k, v, g, bm, bq, bk, causal, 0.6)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-7)
    assert np.all(dq[(-(-n // bq) - 1) * bq:] == 0.0)   # rows that keep no key get no dQ


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_matches_torch_autograd_with_boolean_mask(causal):
    """Independent implementation: torch SDPA in float64 with the expanded
    boolean mask, differentiated by autograd (every row keeps a key)."""
    n, d, bq, bk = 48, 16, 16, 8
    q, k, v, g = (_rand((2, 3, n, d), 760 + i) for i in range(4))
    bm = np.stack([_block_mask(3, 6, 0.45, 95 + h) for h in range(3)])
    bm[:, :, 0] = 1
    dq, dk, dv = ref.backward_block_sparse(q, k, v, g, bm, bq, bk, causal, 0.3)
    keep = np.stack([ref.expand_block_mask(bm[h], n, n, bq, bk) for h in range(3)])
    if causal:
        keep = keep & np.tril(np.ones((n, n), dtype=bool))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(keep)[None], scale=0.3)
    o.backward(torch.from_numpy(g))
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_all_ones_is_dense(causal):
    n, d = 40, 8
    q, k, v, g = (_rand((n, d), 770 + i) for i in range(4))
    ones = np.ones((3, 5), dtype=np.uint8)
    got = ref.backward_block_sparse_head(q, k, v, g, ones, 16, 8, causal, 0.4)
    want = ref.backward_head(q, k, v, g, causal, 0.4)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_block_sparse_pins_catch_planted_mistakes():
    """A transposed block mask or masked scores set to 0 instead of excluded
    (the page's literal S o 1_M) both fail the brute-force pin."""
    n, d, blk = 12, 3, 4
    q, k, v = (_rand((n, d), 750 + i) for i in range(3))
    bm = np.array([[1, 0, 1], [0, 1, 1], [1, 0, 0]], dtype=np.uint8)   # not symmetric
    o_b, _ = ref.brute_force_forward_head(q, k, v, False, 0.7, allowed=lambda i, j: bm[i // blk][j // blk] != 0)

    def zero_filled(q, k, v):
        s = ref.scores(q, k, 0.7, False)
        s = np.where(ref.expand_block_mask(bm, n, n, blk, blk), s, 0.0)
        p, _, _ = ref.softmax_stats(s)
        return p @ v

    o_tr, _ = ref.forward_block_sparse_head(q, k, v, bm.T, blk, blk, False, 0.7)
    assert not np.allclose(zero_filled(q, k, v), o_b, atol=1e-6)
    assert not np.allclose(o_tr, o_b, atol=1e-6)
    o_ok, _ = ref.forward_block_sparse_head(q, k, v, bm, blk, blk, False, 0.7)
    np.testing.assert_allclose(o_ok, o_b, rtol=1e-12, atol=1e-13)


def test_block_sparse_backward_pins_catch_planted_mistakes():
    """Backward slips fail the finite-difference pin: the softmax row term D
    dropped, dK's scale dropped, a transposed mask, or dV taken from dS."""
    n, d, bq, bk = 8, 3, 4, 4
    q, k, v, g = (_rand((n, d), 780 + i) for i in range(4))
    bm = np.array([[1, 0], [1, 1]], dtype=np.uint8)     # not symmetric; its transpose leaves no row empty
    fq, fk, fv = _fd_block_sparse(q, k, v, g, bm, bq, bk, False, 0.6)

    def planted(which):
        s = ref.scores(q, k, 0.6, False)
        s = np.where(ref.expand_block_mask(bm.T if which == "mask_t" else bm, n, n, bq, bk), s, -np.inf)
        p, _, _ = ref.softmax_stats(s)
        dp = g @ v.T
        dsum = 0.0 if which == "no_D" else np.sum(p * dp, axis=-1)[:, None]
        ds = p * (dp - dsum)
        dv = ds.T @ g if which == "dv_from_ds" else p.T @ g
        dk = (1.0 if which == "no_scale" else 0.6) * (ds.T @ q)
        return 0.6 * (ds @ k), dk, dv

    for which in ("no_D", "no_scale", "dv_from_ds", "mask_t"):
        got = planted(which)
        assert not all(np.allclose(a, b, atol=1e-5) for a, b in zip(got, (fq, fk, fv))), which
    ok = ref.backward_block_sparse_head(q, k, v, g, bm, bq, bk, False, 0.6)
    for a, b in zip(ok, (fq, fk, fv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-7)


def test_dropout_rows_are_rows_of_the_whole_head():
    """The row-restricted mask and forward used for long-sequence samples agree
    with the whole-head definitions on the rows they cover."""
    n, d, t = 37, 5, 51
    q, k, v = (_rand((n, d), 795 + i) for i in range(3))
    rows = np.array([0, 3, 4, 17, 36])
    full = ref.dropout_keep_mask(9, n, n, 0xABCDEF1234, 3, t)
    part = ref.dropout_keep_rows(9, rows, n, 0xABCDEF1234, 3, t)
    assert np.array_equal(part, full[rows])
    for causal in (False, True):
        o, lse = ref.forward_dropout_head(q, k, v, full, t, causal, 0.5)
        o_r, lse_r = ref.forward_dropout_rows(q, k, v, rows, part, t, causal, 0.5)
        np.testing.assert_allclose(o_r, o[rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse_r, lse[rows], rtol=1e-13)


# ---------------------------------------------------------------- decoding (split-KV)
# "Как работает FlashAttention математически" section 9 (FlashDecoding) and the
# merge of key-block partials from "Overview of Flash Attention series", Tiling.

@pytest.mark.parametrize("nq,nk", [(1, 17), (3, 40), (8, 8), (5, 64)])
def test_decode_is_the_last_rows_of_causal_attention(nq, nk):
    """The Nq new queries are the last rows of a length-Nk causal problem."""
    d = 6
    q_full, k, v = (_rand((nk, d), 800 + i + nq) for i in range(3))
    o_full, lse_full = ref.forward_head(q_full, k, v, True, 0.45)
    o, lse = ref.decode_head(q_full[nk - nq:], k, v, True, 0.45)
    np.testing.assert_allclose(o, o_full[nk - nq:], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full[nk - nq:], rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_sdpa_float64(causal):
    nq, nk, d = 4, 37, 16
    q, k, v = _rand((2, 3, nq, d), 810), _rand((2, 3, nk, d), 811), _rand((2, 3, nk, d), 812)
    o, lse = ref.decode(q, k, v, causal, 0.3)
    mask = None
    if causal:
        mask = torch.from_numpy(np.arange(nk)[None, :] <= np.arange(nq)[:, None] + nk - nq)
    o_t = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                                           attn_mask=mask, scale=0.3)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=1e-12, atol=1e-13)
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(mask.numpy(), s, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-12)


def test_decode_single_query_brute_force():
    nk, d = 11, 3
    q, k, v = _rand((1, d), 820), _rand((nk, d), 821), _rand((nk, d), 822)
    o, lse = ref.decode_head(q, k, v, False, 0.9)
    s = [0.9 * math.fsum(q[0, c] * k[j, c] for c in range(d)) for j in range(nk)]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    tot = math.fsum(w)
    np.testing.assert_allclose(o[0], [math.fsum(w[j] * v[j, c] for j in range(nk)) / tot for c in range(d)],
                               rtol=1e-13, atol=1e-15)
    assert abs(lse[0] - (mx + math.log(tot))) < 1e-13


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_split_kv_equals_definition(splits, causal):
    nq, nk, d = 5, 50, 8
    q, k, v = _rand((nq, d), 830), _rand((nk, d), 831, 2.0), _rand((nk, d), 832)
    o, lse = ref.split_kv_decode_head(q, k, v, splits, causal, 0.6)
    o_d, lse_d = ref.decode_head(q, k, v, causal, 0.6)
    np.testing.assert_allclose(o, o_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_d, rtol=1e-12)


def test_merge_of_two_blocks_is_the_tiling_identity():
    """Two key blocks of the coreui worked example merge to the one-shot result."""
    s = np.array([1.0, 2.0, 3.0, 10.0])
    v = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    parts_o, parts_l = [], []
    for a in (0, 2):
        e = np.exp(s[a:a + 2] - s[a:a + 2].max())
        parts_o.append((e / e.sum()) @ v[a:a + 2])
        parts_l.append(s[a:a + 2].max() + math.log(e.sum()))
    o, lse = ref.merge_partials(np.array(parts_o)[:, None, :], np.array(parts_l)[:, None])
    e = np.exp(s - s.max())
    np.testing.assert_allclose(o[0], (e / e.sum()) @ v, rtol=1e-14)
    assert abs(lse[0] - (s.max() + math.log(e.sum()))) < 1e-14
    # a fully masked part (lse = -inf) carries no weight
    o2, lse2 = ref.merge_partials(np.array(parts_o + [np.full(2, 9.0)])[:, None, :],
                                  np.array(parts_l + [-np.inf])[:, None])
    np.testing.assert_allclose(o2, o, rtol=1e-15)
    # a wrong sign in the weights is caught
    m = max(parts_l)
    bad = sum(math.exp(m - l) * po for l, po in zip(parts_l, parts_o))
    assert not np.allclose(bad / sum(math.exp(m - l) for l in parts_l), o[0], atol=1e-6)


# --- dropout: Philox4x32-10 and the regenerated mask ----------------------

KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answer_vectors():
    with open(KAT) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        out = ref.philox4x32(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in vec["output"]]
    # vectorised over a batch of counters gives the same as one at a time
    ctrs = np.array([[int(x, 16) for x in v["counter"]] for v in kat["vectors"]], dtype=np.uint64)
    keys = np.array([[int(x, 16) for x in v["key"]] for v in kat["vectors"]], dtype=np.uint64)
    batch = ref.philox4x32(ctrs, keys)
    assert [[int(x) for x in row] for row in batch] == [[int(x, 16) for x in v["output"]] for v in kat["vectors"]]


@pytest.mark.parametrize("p,t", [(0.0, 0), (0.1, 26), (0.25, 64), (0.5, 128), (0.99, 253), (255 / 256, 255)])
def test_dropout_threshold_rounding(p, t):
    assert ref.dropout_threshold(p) == t


@pytest.mark.parametrize("p", [-0.01, 1.0, 0.999])
def test_dropout_threshold_rejects_out_of_range(p):
    with pytest.raises(ValueError):
        ref.dropout_threshold(p)


@pytest.mark.parametrize("t", [0, 1, 26, 128, 255])
def test_dropout_keep_rate_matches_threshold(t):
    keep = ref.dropout_keep_mask(3, 384, 512, seed=0x1234_5678_9ABC, offset=7, t=t)
    n = keep.size
    want = 1.0 - t / 256.0
    sigma = math.sqrt(want * (1.0 - want) / n)
    assert abs(keep.mean() - want) <= 5 * sigma + 1e-12
    if t == 0:
        assert keep.all()


def test_dropout_mask_bytes_are_uniform():
    # the byte each element draws: 256 equally likely values (chi-square, 255 dof, p ~ 1e-6 bound)
    keep_prev = ref.dropout_keep_mask(0, 256, 256, seed=99, offset=0, t=0)
    assert keep_prev.all()
    # recover each element's byte as the largest t that still keeps it (binary search over t)
    lo = np.zeros((256, 256), dtype=np.int64)
    hi = np.full((256, 256), 256, dtype=np.int64)
    for _ in range(8):
        mid = (lo + hi) // 2
        keep = np.zeros((256, 256), dtype=bool)
        for t in np.unique(mid):
            sel = mid == t
            keep[sel] = ref.dropout_keep_mask(0, 256, 256, seed=99, offset=0, t=int(min(t, 255)))[sel]
        lo = np.where(keep, mid, lo)
        hi = np.where(keep, hi, mid)
    counts = np.bincount(lo.ravel(), minlength=256)
    expected = lo.size / 256.0
    chi2 = float(np.sum((counts - expected) ** 2 / expected))
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)


def test_dropout_mask_is_a_function_of_seed_offset_and_head():
    a = ref.dropout_keep_mask(5, 64, 96, seed=42, offset=3, t=128)
    assert np.array_equal(a, ref.dropout_keep_mask(5, 64, 96, seed=42, offset=3, t=128))
    for other in (ref.dropout_keep_mask(6, 64, 96, seed=42, offset=3, t=128),
                  ref.dropout_keep_mask(5, 64, 96, seed=43, offset=3, t=128),
                  ref.dropout_keep_mask(5, 64, 96, seed=42 + (1 << 32), offset=3, t=128),
                  ref.dropout_keep_mask(5, 64, 96, seed=42, offset=4, t=128)):
        agree = float(np.mean(a == other))
        assert 0.4 < agree < 0.6           # independent halves agree half the time
    # a sub-rectangle of a larger mask is the mask of the smaller problem (position-keyed)
    big = ref.dropout_keep_mask(5, 100, 130, seed=42, offset=3, t=128)
    assert np.array_equal(big[:64, :96], a)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_with_t0_is_plain_attention(causal):
    n, d = 13, 8
    q, k, v, do = (_rand((n, d), s) for s in (1, 2, 3, 4))
    keep = np.ones((n, n), dtype=bool)
    o, lse = ref.forward_dropout_head(q, k, v, keep, 0, causal, 0.4)
    o2, lse2 = ref.forward_head(q, k, v, causal, 0.4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    for a, b in zip(ref.backward_dropout_head(q, k, v, do, keep, 0, causal, 0.4),
                    ref.backward_head(q, k, v, do, causal, 0.4)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)


def _torch_dropout_attention(q, k, v, keep, t, causal, scale):
    """Dropout attention composed from torch float64 ops (autograd differentiates it)."""
    s = scale * (q @ k.T)
    if causal:
        n = s.shape[0]
        s = s.masked_fill(torch.ones(n, s.shape[1], dtype=torch.bool).triu(1), float("-inf"))
    p = torch.softmax(s, dim=-1)
    return (p * torch.from_numpy(keep.astype(np.float64)) / (1.0 - t / 256.0)) @ v, torch.logsumexp(s, dim=-1)


@pytest.mark.parametrize("causal,t", [(False, 26), (True, 26), (True, 128)])
def test_dropout_forward_backward_match_torch_autograd_float64(causal, t):
    n, d = 24, 16
    q, k, v, do = (_rand((n, d), s) for s in (11, 12, 13, 14))
    keep = ref.dropout_keep_mask(2, n, n, seed=7, offset=1, t=t)
    assert 0 < keep.sum() < keep.size
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o_t, lse_t = _torch_dropout_attention(tq, tk, tv, keep, t, causal, 0.3)
    o_t.backward(torch.from_numpy(do))
    o, lse = ref.forward_dropout_head(q, k, v, keep, t, causal, 0.3)
    np.testing.assert_allclose(o, o_t.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_t.detach().numpy(), rtol=0, atol=1e-13)
    dq, dk, dv = ref.backward_dropout_head(q, k, v, do, keep, t, causal, 0.3)
    for mine, theirs in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, theirs.numpy(), rtol=0, atol=1e-12)


def test_dropout_backward_matches_finite_differences():
    n, d = 6, 3
    q, k, v, g = (_rand((n, d), s) for s in (21, 22, 23, 24))
    keep = ref.dropout_keep_mask(0, n, n, seed=5, offset=0, t=100)
    want = ref.finite_difference_grads_dropout(q, k, v, g, keep, 100, True, 0.7)
    got = ref.backward_dropout_head(q, k, v, g, keep, 100, True, 0.7)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-7)


def test_dropout_is_unbiased_in_expectation():
    # averaging O over many independent masks approaches the undropped O (E[Z] / (1 - t/256) = 1)
    n, d, t = 8, 4, 64
    q, k, v = (_rand((n, d), s) for s in (31, 32, 33))
    o_ref, _ = ref.forward_head(q, k, v, True, 0.5)
    samples = np.stack([ref.forward_dropout_head(q, k, v, ref.dropout_keep_mask(0, n, n, 77, off, t), t, True, 0.5)[0]
                        for off in range(3000)])
    mean, std = samples.mean(axis=0), samples.std(axis=0)
    assert np.all(np.abs(mean - o_ref) <= 5 * std / math.sqrt(len(samples)) + 1e-12)


def test_dropout_pins_catch_an_unmasked_dp():
    # a planted mistake in the oracle's own arithmetic (the mask left off dP) fails the autograd pin
    n, d, t = 16, 8, 64
    q, k, v, do = (_rand((n, d), s) for s in (41, 42, 43, 44))
    keep = ref.dropout_keep_mask(1, n, n, seed=3, offset=0, t=t)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    o_t, _ = _torch_dropout_attention(tq, tk, tv, keep, t, False, 0.5)
    o_t.backward(torch.from_numpy(do))
    p, _, _ = ref.softmax_stats(ref.scores(q, k, 0.5, False))
    dp_wrong = do @ v.T                                  # mistake: no keep mask, no 1/(1 - p)
    ds = p * (dp_wrong - np.sum(p * dp_wrong, axis=-1)[:, None])
    assert np.max(np.abs(0.5 * ds @ k - tq.grad.numpy())) > 1e-3


# --- FP8 (OCP E4M3) inputs --------------------------------------------------

def test_e4m3_decode_matches_torch_float8_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = ref.e4m3_decode(codes)
    theirs = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))
    ok = ~np.isnan(mine)
    assert np.array_equal(mine[ok], theirs[ok])


def test_e4m3_decode_special_values():
    # values fixed by the format: largest finite, smallest normal and subnormal, one, sign
    assert ref.e4m3_decode(0x7E) == 448.0
    assert ref.e4m3_decode(0x08) == 2.0 ** -6
    assert ref.e4m3_decode(0x01) == 2.0 ** -9
    assert ref.e4m3_decode(0x38) == 1.0
    assert ref.e4m3_decode(0xB8) == -1.0
    assert ref.e4m3_decode(0x00) == 0.0 and np.signbit(ref.e4m3_decode(0x80))
    assert np.isnan(ref.e4m3_decode(0x7F)) and np.isnan(ref.e4m3_decode(0xFF))
    # 127 distinct finite non-negative values, strictly increasing with the code
    pos = ref.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def _fp8_codes(shape, seed, mult=1.0):
    x = torch.from_numpy(_rand(shape, seed, mult)).float()
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8_is_attention_of_the_decoded_inputs(causal):
    n, d = 20, 16
    q8, k8, v8 = (_fp8_codes((n, d), s) for s in (51, 52, 53))
    o, lse = ref.forward_fp8_head(q8, k8, v8, 0.5, 2.0, 0.25, causal, 0.3)
    tq = torch.from_numpy(q8).view(torch.float8_e4m3fn).double() * 0.5
    tk = torch.from_numpy(k8).view(torch.float8_e4m3fn).double() * 2.0
    tv = torch.from_numpy(v8).view(torch.float8_e4m3fn).double() * 0.25
    o_t = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3)
    np.testing.assert_allclose(o, o_t.numpy(), rtol=0, atol=1e-13)


def test_fp8_rounding_bound_holds_for_probabilities_rounded_to_e4m3():
    # emulate the rounding the bound describes (p' = e^(s - c) rounded to E4M3, c = m or m - ln 256)
    n, d = 48, 32
    q8, k8, v8 = (_fp8_codes((n, d), s, 1.5) for s in (61, 62, 63))
    q, k, v = (ref.e4m3_decode(x) for x in (q8, k8, v8))
    s = ref.scores(q, k, 0.4, True)
    m = np.max(s, axis=-1)
    o_exact, _ = ref.forward_head(q, k, v, True, 0.4)
    bound = ref.fp8_p_rounding_bound(q8, k8, v8, 1.0, 1.0, 1.0, True, 0.4)
    for shift in (0.0, math.log(256.0)):
        pp = np.exp(s - (m - shift)[:, None])
        pq = torch.from_numpy(pp).float().to(torch.float8_e4m3fn).double().numpy()
        l = np.sum(pp, axis=-1)
        o_rounded = (pq @ v) / l[:, None]
        err = np.abs(o_rounded - o_exact)
        assert np.all(err <= bound + 1e-12)
        assert err.max() > 0.01 * bound.max()        # the bound is not vacuous
