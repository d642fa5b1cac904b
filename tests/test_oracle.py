"""Pins for the CPU fp64 oracle: checks that tie it to something other than itself.

The pages print no worked attention values, so the pins are the mathematics
the method fixes: closed forms, invariants, an independent scalar brute force
(exact fsum and 50-digit decimal), the library routine torch's CPU fp64
scaled_dot_product_attention with autograd, and central finite differences.
The planted-mistake test at the end compiles mutated copies of oracle.c and
checks that each mutation fails at least one pin.
"""
import math
import os
import re
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(12345)


def rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


# ----------------------------------------------------------------------------
# independent scalar brute force (pure Python, exact summation with math.fsum)
# ----------------------------------------------------------------------------

def vis(j, pos, causal, window, bm=None, block=(1, 1)):
    """Key j visible to a row at key position pos (independent restatement of the mask).

    bm: optional block mask (nested lists or a 2-D array) indexed [pos // bq][j // bk]."""
    wl, wr = window
    ok = (not causal or j <= pos) and (wl < 0 or j >= pos - wl) and (wr < 0 or j <= pos + wr)
    if ok and bm is not None:
        ok = bool(bm[pos // block[0]][j // block[1]])
    return ok


def brute_fwd(q, k, v, causal, scale, window=(-1, -1), bm=None, block=(1, 1)):
    """O and lse of one head by the definition, scalar Python, math.fsum sums.

    Rows are aligned to the end of the keys (row i at key position i + nk - nq).
    A row with no visible key gives O = 0, lse = -inf.
    """
    n, d = len(q), len(q[0])
    nk = len(k)
    O, L = [], []
    for i in range(n):
        pos = i + nk - n
        vis_j = [j for j in range(nk) if vis(j, pos, causal, window, bm, block)]
        if not vis_j:
            O.append([0.0] * d)
            L.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis_j}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in vis_j}
        l = math.fsum(e.values())
        O.append([math.fsum(e[j] / l * v[j][c] for j in vis_j) for c in range(d)])
        L.append(m + math.log(l))
    return np.array(O), np.array(L)


def brute_bwd_jacobian(q, k, v, do, causal, scale, window=(-1, -1), bm=None, block=(1, 1)):
    """Gradients through the explicit softmax Jacobian dP_ij/dS_ij' = P_ij (delta_jj' - P_ij').

    A different route from the oracle's D-trick: it builds the full per-row
    Jacobian (the O(n^2) formulation) and contracts it, scalar Python.
    """
    n, d = len(q), len(q[0])
    nk = len(k)
    dq = [[0.0] * d for _ in range(n)]
    dk = [[0.0] * d for _ in range(nk)]
    dv = [[0.0] * d for _ in range(nk)]
    for i in range(n):
        pos = i + nk - n
        vis_j = [j for j in range(nk) if vis(j, pos, causal, window, bm, block)]
        if not vis_j:
            continue
        s = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in vis_j}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in vis_j}
        l = math.fsum(e.values())
        P = {j: e[j] / l for j in vis_j}
        # dL/dP_ij = <dO_i, v_j>; dL/dv_j += P_ij dO_i
        gP = {j: math.fsum(do[i][c] * v[j][c] for c in range(d)) for j in vis_j}
        for j in vis_j:
            for c in range(d):
                dv[j][c] += P[j] * do[i][c]
        # dL/dS_ij = sum_j' gP_ij' * P_ij' (delta_j'j - P_ij)
        gS = {}
        for j in vis_j:
            gS[j] = math.fsum(gP[jp] * P[jp] * ((1.0 if jp == j else 0.0) - P[j]) for jp in vis_j)
        for j in vis_j:
            for c in range(d):
                dq[i][c] += scale * gS[j] * k[j][c]
                dk[j][c] += scale * gS[j] * q[i][c]
    return np.array(dq), np.array(dk), np.array(dv)


def decimal_fwd(q, k, v, causal, scale, digits=50):
    """O and lse of one head in 50-digit decimal arithmetic."""
    getcontext().prec = digits
    D = lambda x: Decimal(float(x))  # exact conversion of the double
    n, d = len(q), len(q[0])
    O, L = [], []
    for i in range(n):
        vis = [j for j in range(len(k)) if (not causal) or j <= i]
        s = {j: D(scale) * sum((D(q[i][c]) * D(k[j][c]) for c in range(d)), Decimal(0)) for j in vis}
        m = max(s.values())
        e = {j: (s[j] - m).exp() for j in vis}
        l = sum(e.values(), Decimal(0))
        O.append([float(sum((e[j] * D(v[j][c]) for j in vis), Decimal(0)) / l) for c in range(d)])
        L.append(float(m + l.ln()))
    return np.array(O), np.array(L)


def relerr(a, b):
    """max|a - b| / max|b| over finite entries; infinite when the shapes differ, a
    NaN appears, or the two sides are not infinite in exactly the same places."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape or np.isnan(a).any() or np.isnan(b).any():
        return math.inf
    fa, fb = np.isfinite(a), np.isfinite(b)
    if not np.array_equal(fa, fb) or not np.array_equal(a[~fa], b[~fb]):
        return math.inf
    a, b = a[fa], b[fb]
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# ----------------------------------------------------------------------------
# a battery of pins; the real oracle must pass it, every planted mistake must fail it
# ----------------------------------------------------------------------------

def pin_battery(lib):
    """Run the fast pins against an OracleLib; return the list of failures."""
    fails = []
    rng = np.random.default_rng(7)
    for causal in (False, True):
        for (n, d) in ((1, 3), (5, 3), (8, 4)):
            q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
            scale = 0.7
            o, lse = lib.fwd(q, k, v, causal, scale)
            bo, bl = brute_fwd(q.tolist(), k.tolist(), v.tolist(), causal, scale)
            if relerr(o[0], bo) > 1e-13 or relerr(lse[0], bl) > 1e-13:
                fails.append("brute fwd n=%d causal=%d" % (n, causal))
            dq, dk, dv = lib.bwd(q, k, v, do, causal, scale)
            bq, bk, bv = brute_bwd_jacobian(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, scale)
            for name, a, b in (("dq", dq[0], bq), ("dk", dk[0], bk), ("dv", dv[0], bv)):
                if relerr(a, b) > 1e-12:
                    fails.append("brute %s n=%d causal=%d" % (name, n, causal))
            for blk in (1, 3, n):
                oo, ll = lib.fwd_online(q, k, v, causal, scale, blk)
                if relerr(oo, o) > 1e-12 or relerr(ll, lse) > 1e-12:
                    fails.append("online blk=%d n=%d causal=%d" % (blk, n, causal))
        # rectangular shapes (rows aligned to the end of the keys) and sliding windows
        for (nq, nk, window) in ((3, 7, (-1, -1)), (7, 3, (-1, -1)), (6, 6, (2, -1)), (6, 6, (1, 1)),
                                 (4, 9, (3, 0)), (8, 5, (-1, 2))):
            d = 3
            q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
            k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
            o, lse = lib.fwd(q, k, v, causal, 0.8, window=window)
            bo, bl = brute_fwd(q.tolist(), k.tolist(), v.tolist(), causal, 0.8, window)
            if relerr(o[0], bo) > 1e-13 or relerr(lse[0], bl) > 1e-13:
                fails.append("brute fwd %dx%d window=%s causal=%d" % (nq, nk, window, causal))
            dq, dk, dv = lib.bwd(q, k, v, do, causal, 0.8, window=window)
            bq, bk, bv = brute_bwd_jacobian(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, 0.8, window)
            for name, a, b in (("dq", dq[0], bq), ("dk", dk[0], bk), ("dv", dv[0], bv)):
                if relerr(a, b) > 1e-12:
                    fails.append("brute %s %dx%d window=%s causal=%d" % (name, nq, nk, window, causal))
            oo, ll = lib.fwd_online(q, k, v, causal, 0.8, 2, window=window)
            if relerr(oo, o) > 1e-12 or relerr(ll, lse) > 1e-12:
                fails.append("online %dx%d window=%s causal=%d" % (nq, nk, window, causal))
        # block masks with unequal block sides (one block row fully masked)
        for (n, block) in ((9, (2, 3)), (8, (3, 2))):
            d = 3
            nqb, nkb = -(-n // block[0]), -(-n // block[1])
            bm = (rng.random((nqb, nkb)) < 0.6).astype(np.uint8)
            bm[1, :] = 0
            q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
            o, lse = lib.fwd(q, k, v, causal, 0.9, block_mask=bm, block=block)
            bo, bl = brute_fwd(q.tolist(), k.tolist(), v.tolist(), causal, 0.9, bm=bm, block=block)
            if relerr(o[0], bo) > 1e-13 or relerr(lse[0], bl) > 1e-13:
                fails.append("brute fwd block mask %s causal=%d" % (block, causal))
            dq, dk, dv = lib.bwd(q, k, v, do, causal, 0.9, block_mask=bm, block=block)
            bq, bk, bv = brute_bwd_jacobian(q.tolist(), k.tolist(), v.tolist(), do.tolist(), causal, 0.9,
                                            bm=bm, block=block)
            for name, a, b in (("dq", dq[0], bq), ("dk", dk[0], bk), ("dv", dv[0], bv)):
                if relerr(a, b) > 1e-12:
                    fails.append("brute %s block mask %s causal=%d" % (name, block, causal))
            oo, ll = lib.fwd_online(q, k, v, causal, 0.9, 2, block_mask=bm, mask_block=block)
            if relerr(oo, o) > 1e-12 or relerr(ll, lse) > 1e-12:
                fails.append("online block mask %s causal=%d" % (block, causal))
    return fails


def test_battery_passes_on_the_oracle():
    assert pin_battery(oracle._load()) == []


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    # V = identity (d = n) turns O into the probability matrix P itself.
    n = 8
    q, k = rand(3, n, n), rand(3, n, n, scale=2.0)
    v = np.broadcast_to(np.eye(n), (3, n, n))
    P, _ = oracle.fwd(q, k, v, causal, 0.9)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-13
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)  # keys after the query get exactly zero weight


@pytest.mark.parametrize("causal", [False, True])
def test_v_ones_gives_ones_and_zero_qk_gradients(causal):
    G, n, d = 2, 33, 8
    q, k, do = rand(G, n, d), rand(G, n, d, scale=3.0), rand(G, n, d)
    v = np.ones((G, n, d))
    o, _ = oracle.fwd(q, k, v, causal, 0.5)
    assert np.max(np.abs(o - 1.0)) <= 1e-14
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, 0.5)
    assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_v(causal):
    G, n, d = 2, 40, 5
    q = np.zeros((G, n, d))
    k, v = rand(G, n, d), rand(G, n, d)
    o, lse = oracle.fwd(q, k, v, causal, 0.3)
    if causal:
        ref = np.cumsum(v, axis=1) / np.arange(1, n + 1)[None, :, None]
        ref_lse = np.log(np.arange(1, n + 1))[None, :].repeat(G, 0)
    else:
        ref = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
        ref_lse = np.full((G, n), math.log(n))
    assert np.max(np.abs(o - ref)) <= 1e-13
    assert np.max(np.abs(lse - ref_lse)) <= 1e-13


def test_single_key_and_causal_first_row():
    d, scale = 6, 0.4
    q, k, v = rand(1, 1, d), rand(1, 1, d), rand(1, 1, d)
    o, lse = oracle.fwd(q, k, v, False, scale)
    assert np.array_equal(o, v)  # weight exactly 1
    assert abs(lse[0, 0] - scale * float(q[0, 0] @ k[0, 0])) <= 1e-15
    qn, kn, vn = rand(2, 17, d), rand(2, 17, d), rand(2, 17, d)
    o, lse = oracle.fwd(qn, kn, vn, True, scale)
    assert np.array_equal(o[:, 0], vn[:, 0])
    assert np.max(np.abs(lse[:, 0] - scale * np.einsum("gd,gd->g", qn[:, 0], kn[:, 0]))) <= 1e-15


def test_no_visible_key_gives_zero_and_minus_inf():
    # query position -1 under causal masking sees no key at all
    q, k, v = rand(1, 2, 3), rand(1, 4, 3), rand(1, 4, 3)
    o, lse = oracle.fwd(q, k, v, True, 1.0, qpos=np.array([-1, 0]))
    assert np.all(o[0, 0] == 0.0) and lse[0, 0] == -math.inf
    assert np.array_equal(o[0, 1], v[0, 0])


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_translation_of_keys(causal):
    G, n, d, scale = 2, 50, 7, 0.6
    q, k, v = rand(G, n, d), rand(G, n, d), rand(G, n, d)
    u = rand(G, 1, d)
    o1, l1 = oracle.fwd(q, k, v, causal, scale)
    o2, l2 = oracle.fwd(q, k + u, v, causal, scale)
    assert relerr(o2, o1) <= 1e-12
    shift = scale * np.einsum("gnd,gd->gn", q, u[:, 0])
    assert np.max(np.abs(l2 - l1 - shift)) <= 1e-12 * max(1.0, np.max(np.abs(l1)))


def test_permutation_equivariance():
    G, n, d = 2, 45, 6
    q, k, v = rand(G, n, d), rand(G, n, d), rand(G, n, d)
    o, l = oracle.fwd(q, k, v, False, 0.5)
    perm = RNG.permutation(n)
    o2, l2 = oracle.fwd(q, k[:, perm], v[:, perm], False, 0.5)  # joint key/value permutation
    assert relerr(o2, o) <= 1e-13 and relerr(l2, l) <= 1e-13
    o3, l3 = oracle.fwd(q[:, perm], k, v, False, 0.5)  # query permutation permutes rows
    assert relerr(o3, o[:, perm]) <= 1e-13 and relerr(l3, l[:, perm]) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    G, n, d, scale = 2, 37, 5, 0.8
    q, k, v, do = rand(G, n, d), rand(G, n, d), rand(G, n, d), rand(G, n, d)
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, scale)
    # rows of dS sum to zero  =>  sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0
    assert np.max(np.abs(dk.sum(1))) <= 1e-12 * np.max(np.abs(dk))
    # rows of P sum to one  =>  sum_j dV_j = sum_i dO_i
    assert np.max(np.abs(dv.sum(1) - do.sum(1))) <= 1e-12 * np.max(np.abs(do.sum(1)))
    z = oracle.bwd(q, k, v, np.zeros_like(do), causal, scale)
    assert all(np.all(t == 0.0) for t in z)


def test_online_matches_three_pass_large_logits():
    # a few key rows scaled x20 push the logits to about +-100: exp would overflow unshifted
    G, n, d = 3, 130, 16
    q, k, v = rand(G, n, d), rand(G, n, d), rand(G, n, d)
    k[:, RNG.choice(n, 3, replace=False)] *= 20.0
    for causal in (False, True):
        o, l = oracle.fwd(q, k, v, causal, 1.0)
        assert np.isfinite(o).all() and np.isfinite(l).all()
        for blk in (1, 7, 64, n):
            oo, ll = oracle.fwd_online(q, k, v, causal, 1.0, blk)
            assert relerr(oo, o) <= 1e-12 and relerr(ll, l) <= 1e-12


# ----------------------------------------------------------------------------
# brute force in high precision, library routine, finite differences
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_fifty_digit_decimal(causal):
    n, d = 6, 3
    q, k, v = rand(n, d), rand(n, d, scale=4.0), rand(n, d)
    o, l = oracle.fwd(q, k, v, causal, 0.75)
    ro, rl = decimal_fwd(q.tolist(), k.tolist(), v.tolist(), causal, 0.75)
    assert relerr(o[0], ro) <= 1e-14 and relerr(l[0], rl) <= 1e-14


def _torch_ref(q, k, v, do, causal, scale):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq.detach() @ tk.detach().transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(s, -1)
    return o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("G,n,d,causal", [(4, 256, 64, False), (3, 300, 128, True), (2, 1024, 128, True)])
def test_against_torch_sdpa_fp64(G, n, d, causal):
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = rand(G, n, d), rand(G, n, d), rand(G, n, d), rand(G, n, d)
    to, tl, tdq, tdk, tdv = _torch_ref(q, k, v, do, causal, scale)
    o, l = oracle.fwd(q, k, v, causal, scale)
    assert relerr(o, to) <= 1e-12 and relerr(l, tl) <= 1e-12
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, scale)
    assert relerr(dq, tdq) <= 1e-11 and relerr(dk, tdk) <= 1e-11 and relerr(dv, tdv) <= 1e-11


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    n, d, scale, h = 5, 3, 0.9, 1e-6
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    dq, dk, dv = (g[0] for g in oracle.bwd(q, k, v, do, causal, scale))
    loss = lambda q_, k_, v_: float(np.sum(do * oracle.fwd(q_, k_, v_, causal, scale)[0][0]))
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(n, d):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert relerr(num, grad) <= 1e-7, which


# ----------------------------------------------------------------------------
# the selection API (sampled rows) agrees with the full computation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_row_and_key_selection(causal):
    G, n, d = 2, 70, 8
    q, k, v, do = rand(G, n, d), rand(G, n, d), rand(G, n, d), rand(G, n, d)
    o, l = oracle.fwd(q, k, v, causal, 0.5)
    rows = np.array([0, 5, 69, 33])
    os_, ls_ = oracle.fwd(q[:, rows], k, v, causal, 0.5, qpos=rows)
    assert np.array_equal(os_, o[:, rows]) and np.array_equal(ls_, l[:, rows])
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, 0.5)
    keys = np.array([69, 0, 12])
    sq, sk, sv = oracle.bwd(q, k, v, do, causal, 0.5, rows=rows, keys=keys)
    assert np.array_equal(sq, dq[:, rows])
    assert np.array_equal(sk, dk[:, keys]) and np.array_equal(sv, dv[:, keys])
    sq, sk, sv = oracle.bwd(q, k, v, do, causal, 0.5, rows=rows, keys=[])
    assert np.array_equal(sq, dq[:, rows]) and sk.shape == (G, 0, d)


# ----------------------------------------------------------------------------
# planted mistakes: each mutated copy of oracle.c must fail the battery
# ----------------------------------------------------------------------------

MUTANTS = {
    "causal_excludes_diagonal": ("if (mk.causal && j > pos) return 0;", "if (mk.causal && j >= pos) return 0;"),
    "causal_flipped": ("if (mk.causal && j > pos) return 0;", "if (mk.causal && j < pos) return 0;"),
    "lse_drops_max": ("lse[g * nq + i] = m + log(l);\n        }\n        free(s);",
                      "lse[g * nq + i] = log(l);\n        }\n        free(s);"),
    "unnormalised_weights": ("for (int64_t j = 0; j < nk; ++j) s[j] /= l;", ""),
    "scale_dropped_in_scores": ("s[j] = visible(mk, g, j, qpos[i]) ? scale * dot(qi, kg + j * d, d) : -INFINITY;\n            /* pass 2",
                                "s[j] = visible(mk, g, j, qpos[i]) ? dot(qi, kg + j * d, d) : -INFINITY;\n            /* pass 2"),
    "online_no_output_rescale": ("for (int64_t c = 0; c < d; ++c) acc[c] *= alpha;", ""),
    "online_no_sum_rescale": ("l *= alpha;", ""),
    "window_left_off_by_one": ("if (mk.wl >= 0 && j < pos - mk.wl) return 0;", "if (mk.wl >= 0 && j <= pos - mk.wl) return 0;"),
    "window_right_ignored": ("if (mk.wr >= 0 && j > pos + mk.wr) return 0;", ""),
    "bwd_ignores_qpos": ("if (!visible(mk, g, j, qpos[i])) continue;\n            const double* qi", "if (!visible(mk, g, j, i)) continue;\n            const double* qi"),
    "ds_sign": ("double ds = p * (dot(doi, vg + j * d, d) - D[g * nq + i]);",
                "double ds = p * (D[g * nq + i] - dot(doi, vg + j * d, d));"),
    "D_missing_P": ("Di += s[j] * dp[j];", "Di += dp[j];"),
    "dk_transposed_operand": ("dkj[c] += scale * ds * qi[c];", "dkj[c] += scale * ds * kj[c];"),
    "dq_missing_scale": ("dqi[c] += scale * ds * kg[j * d + c];", "dqi[c] += ds * kg[j * d + c];"),
    "dv_uses_ds": ("dvj[c] += p * doi[c];", "dvj[c] += ds * doi[c];"),
    "dq_wrong_operand": ("dqi[c] += scale * ds * kg[j * d + c];", "dqi[c] += scale * ds * vg[j * d + c];"),
    "block_key_index_uses_row_side": ("j / mk.bk]", "j / mk.bq]"),
    "block_row_index_uses_key": ("pos / mk.bq)", "j / mk.bq)"),
    "block_mask_inverted": ("if (mk.bm && !mk.bm[", "if (mk.bm && mk.bm["),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation anchor not found: %r" % old
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = oracle.OracleLib(oracle.compile_source(str(path), str(tmp_path / ("lib%s.so" % name))))
    assert pin_battery(lib) != [], "planted mistake %s passed every pin" % name


# ----------------------------------------------------------------------------
# rectangular shapes, sliding windows, variable-length batches
# ----------------------------------------------------------------------------

def _mask_matrix(nq, nk, causal, window):
    pos = np.arange(nq)[:, None] + (nk - nq)
    j = np.arange(nk)[None, :]
    m = np.ones((nq, nk), bool)
    if causal:
        m &= j <= pos
    if window[0] >= 0:
        m &= j >= pos - window[0]
    if window[1] >= 0:
        m &= j <= pos + window[1]
    return m


def _torch_masked(q, k, v, do, mask, scale):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    tm = torch.tensor(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq.detach() @ tk.detach().transpose(-1, -2))
    lse = torch.logsumexp(s.masked_fill(~tm, float("-inf")), -1)
    return o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("nq,nk,causal,window", [
    (96, 160, True, (-1, -1)), (160, 160, False, (31, 17)), (128, 128, True, (40, -1)),
    (70, 200, False, (-1, 0)), (200, 200, True, (63, 0)),
])
def test_rectangular_and_window_against_torch_masked(nq, nk, causal, window):
    G, d, scale = 2, 16, 0.3
    q, do = rand(G, nq, d), rand(G, nq, d)
    k, v = rand(G, nk, d), rand(G, nk, d)
    mask = _mask_matrix(nq, nk, causal, window)
    assert mask.any(axis=1).all()  # every row sees a key (torch gives NaN otherwise)
    to, tl, tdq, tdk, tdv = _torch_masked(q, k, v, do, mask, scale)
    o, l = oracle.fwd(q, k, v, causal, scale, window=window)
    assert relerr(o, to) <= 1e-12 and relerr(l, tl) <= 1e-12
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, scale, window=window)
    assert relerr(dq, tdq) <= 1e-11 and relerr(dk, tdk) <= 1e-11 and relerr(dv, tdv) <= 1e-11


def test_rows_without_keys_in_rectangular_causal():
    # more queries than keys: the first nq - nk rows see no key at all
    q, k, v, do = rand(1, 9, 4), rand(1, 5, 4), rand(1, 5, 4), rand(1, 9, 4)
    o, l = oracle.fwd(q, k, v, True, 0.5)
    assert np.all(o[0, :4] == 0.0) and np.all(l[0, :4] == -np.inf) and np.isfinite(l[0, 4:]).all()
    dq, dk, dv = oracle.bwd(q, k, v, do, True, 0.5)
    assert np.all(dq[0, :4] == 0.0)
    bq, bk, bv = brute_bwd_jacobian(q[0].tolist(), k[0].tolist(), v[0].tolist(), do[0].tolist(), True, 0.5)
    assert relerr(dq[0], bq) <= 1e-12 and relerr(dk[0], bk) <= 1e-12 and relerr(dv[0], bv) <= 1e-12


def test_window_q_zero_gives_window_mean():
    n, d, wl = 50, 3, 7
    q = np.zeros((1, n, d))
    k, v = rand(1, n, d), rand(1, n, d)
    o, l = oracle.fwd(q, k, v, True, 0.4, window=(wl, -1))
    for i in range(n):
        lo = max(0, i - wl)
        assert np.max(np.abs(o[0, i] - v[0, lo:i + 1].mean(0))) <= 1e-13
        assert abs(l[0, i] - math.log(i + 1 - lo)) <= 1e-13


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (True, (5, 0))])
def test_varlen_against_block_diagonal_torch(causal, window):
    H, d, scale = 3, 8, 0.35
    lq = [5, 0, 17, 1, 9]
    lk = [5, 3, 20, 1, 12]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q, do = rand(H, tq, d), rand(H, tq, d)
    k, v = rand(H, tk, d), rand(H, tk, d)
    o, l = oracle.fwd_varlen(q, k, v, cu_q, cu_k, causal, scale, window)
    dq, dk, dv = oracle.bwd_varlen(q, k, v, do, cu_q, cu_k, causal, scale, window)
    # one big masked attention over the packed rows: block diagonal x per-sequence mask
    mask = np.zeros((tq, tk), bool)
    for b in range(len(lq)):
        mask[cu_q[b]:cu_q[b + 1], cu_k[b]:cu_k[b + 1]] = _mask_matrix(lq[b], lk[b], causal, window)
    seen = mask.any(axis=1)
    to, tl, tdq, tdk, tdv = _torch_masked(q, k, v, do, mask, scale)
    assert relerr(o[:, seen], to[:, seen]) <= 1e-12 and relerr(l[:, seen], tl[:, seen]) <= 1e-12
    assert relerr(dq[:, seen], tdq[:, seen]) <= 1e-11
    assert relerr(dk, np.where(np.isnan(tdk), 0.0, tdk)) <= 1e-11
    assert relerr(dv, np.where(np.isnan(tdv), 0.0, tdv)) <= 1e-11
    assert np.all(o[:, ~seen] == 0.0) and np.all(l[:, ~seen] == -np.inf)


# ----------------------------------------------------------------------------
# block masks
# ----------------------------------------------------------------------------

def _block_mask_matrix(n, bm, block, causal):
    pos = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    m = bm[pos // block[0], j // block[1]] != 0
    if causal:
        m &= j <= pos
    return m


@pytest.mark.parametrize("n,block,causal", [(300, (128, 128), False), (300, (128, 128), True),
                                            (257, (64, 32), True), (200, (32, 96), False)])
def test_block_mask_against_torch_masked(n, block, causal):
    G, d, scale = 2, 16, 0.3
    rng = np.random.default_rng(n + block[0])
    nqb, nkb = -(-n // block[0]), -(-n // block[1])
    bm = (rng.random((G, nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, :, 0] = 1       # most rows see something ...
    bm[0, 1, :] = 0       # ... but one block row of head 0 sees nothing
    q, k, v, do = rand(G, n, d), rand(G, n, d), rand(G, n, d), rand(G, n, d)
    o, l = oracle.fwd(q, k, v, causal, scale, block_mask=bm, block=block)
    dq, dk, dv = oracle.bwd(q, k, v, do, causal, scale, block_mask=bm, block=block)
    for g in range(G):
        mask = _block_mask_matrix(n, bm[g], block, causal)
        seen = mask.any(axis=1)
        to, tl, tdq, tdk, tdv = _torch_masked(q[g:g + 1], k[g:g + 1], v[g:g + 1], do[g:g + 1], mask, scale)
        assert relerr(o[g, seen], to[0, seen]) <= 1e-12 and relerr(l[g, seen], tl[0, seen]) <= 1e-12
        assert relerr(dq[g, seen], tdq[0, seen]) <= 1e-11
        assert relerr(dk[g], np.where(np.isnan(tdk[0]), 0.0, tdk[0])) <= 1e-11
        assert relerr(dv[g], np.where(np.isnan(tdv[0]), 0.0, tdv[0])) <= 1e-11
        assert np.all(o[g, ~seen] == 0.0) and np.all(l[g, ~seen] == -np.inf) and np.all(dq[g, ~seen] == 0.0)
    assert (~_block_mask_matrix(n, bm[0], block, causal).any(axis=1)).any()  # the empty rows were exercised


def test_block_mask_all_ones_and_block_causal():
    n, d = 200, 8
    q, k, v = rand(1, n, d), rand(1, n, d), rand(1, n, d)
    ones = np.ones((2, 4), np.uint8)
    for causal in (False, True):
        o1, l1 = oracle.fwd(q, k, v, causal, 0.5)
        o2, l2 = oracle.fwd(q, k, v, causal, 0.5, block_mask=ones, block=(128, 64))
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # causal inside a lower-triangular block mask of square blocks is just causal
    tri = np.tril(np.ones((4, 4), np.uint8))
    o1, l1 = oracle.fwd(q, k, v, True, 0.5)
    o2, l2 = oracle.fwd(q, k, v, True, 0.5, block_mask=tri, block=(64, 64))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # an all-zero mask: no row sees a key
    o3, l3 = oracle.fwd(q, k, v, False, 0.5, block_mask=np.zeros((2, 2), np.uint8), block=(128, 128))
    assert np.all(o3 == 0.0) and np.all(l3 == -np.inf)
