"""Checks that pin the CPU oracle to what the pages and the mathematics fix.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` when the oracle disagrees.  ``tests/test_oracle_pins.py``
runs them on the real oracle; ``tests/test_oracle_mutants.py`` runs them on
copies of the oracle with planted mistakes and expects a failure.

Printed values come from ``tests/golden/`` (each file names its source).
Closed forms and invariants come from the proof section (証明) of the formula
page "トランスフォーマーの注意機構" and from footnote 4 of
"Aufmerksamkeit ist alles, was Sie brauchen".
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _printed_close(got, printed, decimals):
    """True if ``got`` rounds to the printed value: within half a unit of the
    last printed decimal (plus a hair for binary representation)."""
    return abs(got - printed) <= 0.5 * 10.0 ** (-decimals) + 1e-12


def _weights_via_identity(orc, q, keys, tau):
    """Attention weights of one query read off the output with V = identity.

    Pads q and keys with zeros to width n = number of keys (dot products are
    unchanged) so that V can be the n x n identity; then output row = weights.
    """
    n, d = keys.shape
    width = max(n, d)
    qp = np.zeros((1, 1, 1, width))
    qp[0, 0, 0, :d] = q
    kp = np.zeros((1, 1, n, width))
    kp[0, 0, :, :d] = keys
    vp = np.zeros((1, 1, n, width))
    vp[0, 0, :, :n] = np.eye(n)
    out, lse = orc.sdpa(qp, kp, vp, tau=tau)
    return out[0, 0, 0, :n], lse[0, 0, 0]


def _score_via_single_key(orc, q, k, tau=None):
    """With one key the log-sum-exp equals that key's score."""
    d = q.shape[-1]
    _, lse = orc.sdpa(q.reshape(1, 1, 1, d), k.reshape(1, 1, 1, d),
                      np.zeros((1, 1, 1, d)), tau=tau)
    return lse[0, 0, 0]


# --------------------------------------------------------------------------
# Values printed on the formula page
# --------------------------------------------------------------------------

def pin_worked_example_output(orc):
    """d_k = 4 example: output (0.70, 1.44, 0.28, 0.26) with V = K, and the
    exp-sum 31.68 as e^{lse}."""
    g = _golden("worked_example.json")
    keys = np.array(g["keys"], dtype=np.float64)
    q = np.array(g["query"], dtype=np.float64)
    out, lse = orc.sdpa(q.reshape(1, 1, 1, 4), keys.reshape(1, 1, 8, 4),
                        keys.reshape(1, 1, 8, 4))
    pr = g["printed"]
    for got, want in zip(out[0, 0, 0], pr["output"]["value"]):
        assert _printed_close(got, want, pr["output"]["decimals"]), (out, pr["output"])
    assert _printed_close(math.exp(lse[0, 0, 0]), pr["exp_sum"]["value"],
                          pr["exp_sum"]["decimals"]), lse


def pin_worked_example_weights(orc):
    """Weights 0.634 (魚), 0.141 (おいしかった), 0.067 (それ), 0.032 (others)."""
    g = _golden("worked_example.json")
    keys = np.array(g["keys"], dtype=np.float64)
    q = np.array(g["query"], dtype=np.float64)
    w, _ = _weights_via_identity(orc, q, keys, tau=g["printed"]["divisor"])
    pw = g["printed"]["weights"]
    for tok, a in zip(g["tokens"], w):
        want = pw.get(tok, pw["others"])
        assert _printed_close(a, want, pw["decimals"]), (tok, a, want)


def pin_worked_example_scores(orc):
    """Dot products 6 / 3 / 1.5 / 0 and, divided by sqrt(4) = 2, 3 / 1.5 / 0.75 / 0."""
    g = _golden("worked_example.json")
    keys = np.array(g["keys"], dtype=np.float64)
    q = np.array(g["query"], dtype=np.float64)
    pr = g["printed"]
    for tok, k in zip(g["tokens"], keys):
        dot = pr["dot_products"].get(tok, pr["dot_products"]["others"])
        scaled = pr["scaled_scores"].get(tok, pr["scaled_scores"]["others"])
        assert abs(_score_via_single_key(orc, q, k, tau=1.0) - dot) < 1e-12, tok
        assert abs(_score_via_single_key(orc, q, k) - scaled) < 1e-12, tok


def pin_temperature(orc):
    """Same scores divided by 1 and by 8: fish weight 0.932 and 0.217."""
    g = _golden("worked_example.json")
    keys = np.array(g["keys"], dtype=np.float64)
    q = np.array(g["query"], dtype=np.float64)
    fish = g["tokens"].index("魚")
    pr = g["printed"]
    w1, _ = _weights_via_identity(orc, q, keys, tau=1.0)
    w8, _ = _weights_via_identity(orc, q, keys, tau=8.0)
    assert _printed_close(w1[fish], pr["fish_weight_divided_by_1"]["value"], 3), w1
    assert _printed_close(w8[fish], pr["fish_weight_divided_by_8"]["value"], 3), w8


def pin_two_keys_d64(orc):
    """d_k = 64, dot products 8 apart: 0.9997/0.0003 unscaled, 0.731/0.269
    scaled; a(1-a) 0.0003 vs 0.197, a gain of about 590."""
    g = _golden("two_keys_d64.json")
    d, gap = g["d_k"], g["dot_product_gap"]
    q = np.zeros(d); q[0] = gap
    keys = np.zeros((2, d)); keys[0, 0] = 1.0
    pr = g["printed"]
    ws, _ = _weights_via_identity(orc, q, keys, tau=math.sqrt(d))
    wu, _ = _weights_via_identity(orc, q, keys, tau=1.0)
    # default tau must be sqrt(d): check through the default path too
    out, _ = orc.sdpa(q.reshape(1, 1, 1, d), keys.reshape(1, 1, 2, d),
                      np.eye(2, d).reshape(1, 1, 2, d))
    wd = out[0, 0, 0, :2]
    for w in (ws, wd):
        for got, want in zip(w, pr["scaled_weights"]["value"]):
            assert _printed_close(got, want, pr["scaled_weights"]["decimals"]), w
    for got, want in zip(wu, pr["unscaled_weights"]["value"]):
        assert _printed_close(got, want, pr["unscaled_weights"]["decimals"]), wu
    assert abs(wu[0] / wu[1] - pr["unscaled_ratio"]["value"]) < 1.0
    gu = wu[0] * (1 - wu[0])
    gs = ws[0] * (1 - ws[0])
    assert _printed_close(gu, pr["unscaled_a_one_minus_a"]["value"], 4), gu
    assert _printed_close(gs, pr["scaled_a_one_minus_a"]["value"], 3), gs
    gain = gs / gu
    assert abs(gain / pr["gradient_gain"]["value"] - 1) < pr["gradient_gain"]["relative_tolerance"], gain


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

def pin_softmax_row_properties(orc, seed=11):
    """Weights are positive, sum to 1, and a_j / a_i = e^{s_j - s_i}."""
    rng = np.random.default_rng(seed)
    d, n = 16, 12
    q = rng.standard_normal(d)
    keys = rng.standard_normal((n, d))
    w, _ = _weights_via_identity(orc, q, keys, tau=math.sqrt(d))
    assert np.all(w > 0)
    assert abs(w.sum() - 1.0) < 1e-12
    s = np.array([_score_via_single_key(orc, q, k) for k in keys])
    lr = np.log(w[:, None] / w[None, :])
    assert np.max(np.abs(lr - (s[:, None] - s[None, :]))) < 1e-10


def pin_temperature_limits(orc, seed=12):
    """tau -> 0 selects the value of the unique best key; tau -> inf gives the
    mean of the values, and at q = 0 exactly the mean with lse = ln n."""
    rng = np.random.default_rng(seed)
    d, n = 8, 10
    keys = rng.standard_normal((n, d))
    vals = rng.standard_normal((n, d))
    q = keys[3] * 2.0
    dots = keys @ q
    best = int(np.argmax(dots))
    assert np.sort(dots)[-1] - np.sort(dots)[-2] > 0.1
    out, _ = orc.sdpa(q.reshape(1, 1, 1, d), keys.reshape(1, 1, n, d),
                      vals.reshape(1, 1, n, d), tau=1e-4)
    assert np.max(np.abs(out[0, 0, 0] - vals[best])) < 1e-12
    out, _ = orc.sdpa(q.reshape(1, 1, 1, d), keys.reshape(1, 1, n, d),
                      vals.reshape(1, 1, n, d), tau=1e9)
    assert np.max(np.abs(out[0, 0, 0] - vals.mean(axis=0))) < 1e-6
    out, lse = orc.sdpa(np.zeros((1, 1, 1, d)), keys.reshape(1, 1, n, d),
                        vals.reshape(1, 1, n, d))
    assert np.max(np.abs(out[0, 0, 0] - vals.mean(axis=0))) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(n)) < 1e-14


def pin_causal(orc, seed=13):
    """Causal: row 0 equals V[0] exactly with lse = s_00; row i equals the
    unmasked attention over keys 0..i."""
    rng = np.random.default_rng(seed)
    B, H, L, d = 2, 3, 9, 5
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    out, lse = orc.sdpa(q, k, v, causal=True)
    assert np.array_equal(out[:, :, 0], v[:, :, 0])
    for b in range(B):
        for h in range(H):
            s00 = _score_via_single_key(orc, q[b, h, 0], k[b, h, 0])
            assert abs(lse[b, h, 0] - s00) < 1e-14
    for i in (1, 4, L - 1):
        o2, l2 = orc.sdpa(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1])
        assert np.max(np.abs(out[:, :, i] - o2[:, :, 0])) < 1e-14
        assert np.max(np.abs(lse[:, :, i] - l2[:, :, 0])) < 1e-14
    # non-causal rows differ (the mask really is applied above the diagonal)
    full, _ = orc.sdpa(q, k, v)
    assert np.max(np.abs(full[:, :, 0] - out[:, :, 0])) > 1e-3
    # causal with Lq != Lk is top-left aligned: row i sees keys 0..i
    o3, l3 = orc.sdpa(q[:, :, :4], k, v, causal=True)
    assert np.array_equal(o3, out[:, :, :4]) and np.array_equal(l3, lse[:, :, :4])


def pin_padding(orc, seed=14):
    """key_lens: equal to the problem cut to its first len keys; padded K/V
    contents (even NaN / 1e30) change nothing; len = 0 gives O = 0, lse = -inf."""
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 3, 2, 5, 11, 4
    q = rng.standard_normal((B, H, Lq, d))
    k = rng.standard_normal((B, H, Lk, d))
    v = rng.standard_normal((B, H, Lk, d))
    lens = np.array([7, 11, 0], dtype=np.int32)
    out, lse = orc.sdpa(q, k, v, key_lens=lens)
    for b in range(2):
        n = lens[b]
        o2, l2 = orc.sdpa(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n])
        assert np.max(np.abs(out[b] - o2[0])) < 1e-14
        assert np.max(np.abs(lse[b] - l2[0])) < 1e-14
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))
    kp, vp = k.copy(), v.copy()
    kp[0, :, 7:] = np.nan
    vp[0, :, 7:] = 1e30
    o3, l3 = orc.sdpa(q, kp, vp, key_lens=lens)
    assert np.array_equal(o3, out) and np.array_equal(l3, lse)
    # lengths beyond Lk clamp to Lk; negative lengths clamp to 0
    o4, l4 = orc.sdpa(q, k, v, key_lens=np.array([7, 99, -5], dtype=np.int32))
    assert np.array_equal(o4, out) and np.array_equal(l4, lse)


def pin_lse_bounds(orc, seed=15):
    """max_j s_j <= lse <= max_j s_j + ln n."""
    rng = np.random.default_rng(seed)
    d, n = 6, 9
    for _ in range(5):
        q = rng.standard_normal(d) * 3
        keys = rng.standard_normal((n, d))
        s = np.array([_score_via_single_key(orc, q, k) for k in keys])
        _, lse = orc.sdpa(q.reshape(1, 1, 1, d), keys.reshape(1, 1, n, d),
                          np.zeros((1, 1, n, d)))
        assert s.max() - 1e-12 <= lse[0, 0, 0] <= s.max() + math.log(n) + 1e-12
    # equality cases: one key gives lse = s; n equal scores give s + ln n
    q = rng.standard_normal(d)
    keys = np.tile(rng.standard_normal(d), (n, 1))
    s = _score_via_single_key(orc, q, keys[0])
    _, lse = orc.sdpa(q.reshape(1, 1, 1, d), keys.reshape(1, 1, n, d), np.zeros((1, 1, n, d)))
    assert abs(lse[0, 0, 0] - (s + math.log(n))) < 1e-12


def pin_shift_invariance(orc, seed=16):
    """K + 1 u^T shifts row i's scores by q_i . u / sqrt(d): weights (hence O)
    unchanged, lse shifted by that amount."""
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 1, 2, 4, 6, 8
    # dyadic grid: every sum below is exact in fp64
    q = rng.integers(-16, 16, size=(B, H, Lq, d)) / 8.0
    k = rng.integers(-16, 16, size=(B, H, Lk, d)) / 8.0
    v = rng.standard_normal((B, H, Lk, d))
    u = rng.integers(-16, 16, size=d) / 8.0
    out, lse = orc.sdpa(q, k, v)
    out2, lse2 = orc.sdpa(q, k + u, v)
    assert np.max(np.abs(out2 - out)) < 1e-12
    shift = (q @ u) / math.sqrt(d)
    assert np.max(np.abs(lse2 - lse - shift)) < 1e-12


def pin_score_variance(orc, seed=17, n=20000):
    """Footnote 4 / proof section: for iid N(0, 1) components q . k has
    variance d_k, and q . k / sqrt(d_k) variance 1, for d = 4, 16, 64."""
    rng = np.random.default_rng(seed)
    for d in (4, 16, 64):
        # one key per problem: the n pairs are laid out as n batch entries
        qq = rng.standard_normal((n, 1, 1, d))
        kk = rng.standard_normal((n, 1, 1, d))
        _, s = orc.sdpa(qq, kk, np.zeros_like(kk))
        _, z_unscaled = orc.sdpa(qq, kk, np.zeros_like(kk), tau=1.0)
        var_s = float(np.var(s))
        var_z = float(np.var(z_unscaled))
        assert abs(var_s - 1.0) < 0.06, (d, var_s)
        assert abs(var_z / d - 1.0) < 0.06, (d, var_z)


def pin_head_batch_permutation(orc, seed=18):
    """Each (b, h) slice is an independent instance: permuting slices permutes
    the outputs bitwise."""
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 3, 4, 5, 7, 6
    q = rng.standard_normal((B, H, Lq, d))
    k = rng.standard_normal((B, H, Lk, d))
    v = rng.standard_normal((B, H, Lk, d))
    out, lse = orc.sdpa(q, k, v)
    perm = rng.permutation(B * H)
    qp = q.reshape(B * H, Lq, d)[perm].reshape(B, H, Lq, d)
    kp = k.reshape(B * H, Lk, d)[perm].reshape(B, H, Lk, d)
    vp = v.reshape(B * H, Lk, d)[perm].reshape(B, H, Lk, d)
    o2, l2 = orc.sdpa(qp, kp, vp)
    assert np.array_equal(o2.reshape(B * H, Lq, d), out.reshape(B * H, Lq, d)[perm])
    assert np.array_equal(l2.reshape(B * H, Lq), lse.reshape(B * H, Lq)[perm])


def pin_brute_force(orc, seed=19):
    """Agreement with the pure-Python per-query loops (no max shift) to 1e-12
    on the toy shapes and random tiny shapes, with and without masks."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    cases = [
        # (B, H, Lq, Lk, d, causal, key_lens)
        (1, 2, 8, 8, 3, False, None),     # toy encoder self-attention
        (1, 2, 4, 4, 3, True, None),      # toy decoder masked self-attention
        (1, 2, 4, 8, 3, False, None),     # toy cross-attention
        (2, 3, 5, 9, 7, False, [4, 9]),
        (2, 1, 6, 6, 2, True, [3, 0]),
        (1, 1, 7, 3, 5, True, None),      # causal with Lq > Lk
    ]
    for B, H, Lq, Lk, d, causal, kl in cases:
        q = rng.standard_normal((B, H, Lq, d))
        k = rng.standard_normal((B, H, Lk, d))
        v = rng.standard_normal((B, H, Lk, d))
        out, lse = orc.sdpa(q, k, v, causal=causal, key_lens=kl)
        bo, bl = brute.attention(q, k, v, causal=causal, key_lens=kl)
        bo = np.array(bo)
        bl = np.array(bl)
        assert np.max(np.abs(out - bo)) < 1e-12, (B, H, Lq, Lk, d, causal, kl)
        fin = np.isfinite(bl)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.max(np.abs(lse[fin] - bl[fin]), initial=0.0) < 1e-12


def pin_rows_match_full(orc, seed=20):
    """The row-subset entry point returns exactly the rows of the full one."""
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 2, 3, 6, 9, 4
    q = rng.standard_normal((B, H, Lq, d))
    k = rng.standard_normal((B, H, Lk, d))
    v = rng.standard_normal((B, H, Lk, d))
    kl = np.array([5, 9], dtype=np.int32)
    for causal in (False, True):
        out, lse = orc.sdpa(q, k, v, causal=causal, key_lens=kl)
        rows = rng.choice(B * H * Lq, size=10, replace=False)
        ro, rl = orc.sdpa_rows(q, k, v, rows, causal=causal, key_lens=kl)
        assert np.array_equal(ro, out.reshape(-1, d)[rows])
        assert np.array_equal(rl, lse.reshape(-1)[rows])


def pin_input_widening(orc):
    """fp32 and bf16 inputs are widened exactly: the same values given as
    fp64, fp32 and bf16 bits give identical results."""
    rng = np.random.default_rng(21)
    vals = rng.integers(-64, 64, size=(1, 2, 5, 4)) / 16.0   # exact in bf16
    kv = rng.integers(-64, 64, size=(1, 2, 6, 4)) / 16.0
    ref = orc.sdpa(vals, kv, kv)
    f32 = orc.sdpa(vals.astype(np.float32), kv.astype(np.float32), kv.astype(np.float32))
    to_bf16 = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bf = orc.sdpa(to_bf16(vals), to_bf16(kv), to_bf16(kv), bf16=True)
    for a, b in ((ref, f32), (ref, bf)):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# Backward: gradients of a loss L given dL/d(out)
# --------------------------------------------------------------------------

def pin_bwd_two_keys_gradient(orc):
    """The two-key example of section 応用 seen through the gradient.  With
    v_1 = e_0, v_2 = 0 and dL/d(out) = e_0 the loss is a_1, so the Jacobian
    display gives dL/ds_1 = a_1 (1 - a_1) and dL/ds_2 = -a_1 a_2: the page's
    gradient factor, 0.197 scaled and 0.0003 unscaled.  It is read off dq
    (= sum_l dL/ds_l k_l / tau with k_1 = e_0, k_2 = 0); dk_1, dk_2 and dv_1
    follow from the same numbers."""
    g = _golden("two_keys_d64.json")
    d, gap = g["d_k"], g["dot_product_gap"]
    pr = g["printed"]
    q = np.zeros((1, 1, 1, d)); q[..., 0] = gap
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = 1.0
    v = np.zeros((1, 1, 2, d)); v[0, 0, 0, 0] = 1.0
    gout = np.zeros((1, 1, 1, d)); gout[..., 0] = 1.0
    for tau, key, dec in ((math.sqrt(d), "scaled_a_one_minus_a", 3),
                          (1.0, "unscaled_a_one_minus_a", 4)):
        dq, dk, dv = orc.sdpa_bwd(q, k, v, gout, tau=tau)
        ds1 = dq[0, 0, 0, 0] * tau
        assert _printed_close(ds1, pr[key]["value"], dec), (tau, ds1)
        assert np.allclose(dq[0, 0, 0, 1:], 0.0)
        assert abs(dk[0, 0, 0, 0] - ds1 * gap / tau) < 1e-12
        assert abs(dk[0, 0, 1, 0] + ds1 * gap / tau) < 1e-12
        a1 = 0.5 + math.sqrt(0.25 - ds1)          # root of a(1-a) = ds1 above 1/2
        assert abs(dv[0, 0, 0, 0] - a1) < 1e-9 and abs(dv[0, 0, 1, 0] - (1 - a1)) < 1e-9


def pin_bwd_finite_differences(orc, seed=21):
    """Central differences of the (pinned) forward: each gradient entry equals
    (L(x + h) - L(x - h)) / 2h with L = sum(dout * out), on tiny fp64 problems
    with and without masks."""
    rng = np.random.default_rng(seed)
    h = 1e-6
    for causal, kl in ((False, None), (True, None), (False, [3, 0]), (True, [5, 2])):
        B, H, Lq, Lk, d = 2, 1, 4, 5, 3
        q = rng.standard_normal((B, H, Lq, d))
        k = rng.standard_normal((B, H, Lk, d))
        v = rng.standard_normal((B, H, Lk, d))
        gout = rng.standard_normal((B, H, Lq, d))
        grads = orc.sdpa_bwd(q, k, v, gout, causal=causal, key_lens=kl)

        def loss():
            out, _ = orc.sdpa(q, k, v, causal=causal, key_lens=kl)
            return float(np.sum(out * gout))
        for arr, grad in zip((q, k, v), grads):
            for idx in np.ndindex(arr.shape):
                x0 = arr[idx]
                arr[idx] = x0 + h
                lp = loss()
                arr[idx] = x0 - h
                lm = loss()
                arr[idx] = x0
                assert abs((lp - lm) / (2 * h) - grad[idx]) < 1e-6, (causal, kl, idx)


def pin_bwd_brute_force(orc, seed=22):
    """The C gradients equal the full-Jacobian pure-Python route
    (oracle/brute.py) to 1e-12 on the toy shapes."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    for (B, H, Lq, Lk, d, causal, kl) in ((1, 2, 8, 8, 3, False, None),    # toy encoder
                                          (1, 2, 4, 4, 3, True, None),     # toy decoder
                                          (1, 2, 4, 8, 3, False, None),    # toy cross
                                          (2, 1, 5, 6, 4, True, [4, 0])):
        q = rng.standard_normal((B, H, Lq, d))
        k = rng.standard_normal((B, H, Lk, d))
        v = rng.standard_normal((B, H, Lk, d))
        gout = rng.standard_normal((B, H, Lq, d))
        got = orc.sdpa_bwd(q, k, v, gout, causal=causal, key_lens=kl)
        ref = brute.attention_grad(q.tolist(), k.tolist(), v.tolist(), gout.tolist(), causal, kl)
        for a, b in zip(got, ref):
            assert np.max(np.abs(a - np.array(b))) < 1e-12


def pin_bwd_invariants(orc, seed=23):
    """Weights sum to 1 and depend only on score differences, so per row the
    score gradients sum to 0: the key gradients of a slice sum to 0, and the
    value gradients sum to the dL/d(out) rows that see any key.  Keys nobody
    sees and rows that see no key get exactly zero."""
    rng = np.random.default_rng(seed)
    B, H, Lq, Lk, d = 2, 2, 6, 7, 4
    kl = [5, 0]
    for causal in (False, True):
        q = rng.standard_normal((B, H, Lq, d))
        k = rng.standard_normal((B, H, Lk, d))
        v = rng.standard_normal((B, H, Lk, d))
        gout = rng.standard_normal((B, H, Lq, d))
        dq, dk, dv = orc.sdpa_bwd(q, k, v, gout, causal=causal, key_lens=kl)
        for b in range(B):
            n = min(Lk, kl[b])
            seen = [i for i in range(Lq) if (min(n, i + 1) if causal else n) > 0]
            for hh in range(H):
                assert np.max(np.abs(dk[b, hh].sum(axis=0))) < 1e-12
                want = gout[b, hh, seen].sum(axis=0) if seen else np.zeros(d)
                assert np.max(np.abs(dv[b, hh].sum(axis=0) - want)) < 1e-12
                assert np.all(dk[b, hh, n:] == 0) and np.all(dv[b, hh, n:] == 0)
                unseen = [i for i in range(Lq) if i not in seen]
                assert np.all(dq[b, hh, unseen] == 0)


# --------------------------------------------------------------------------
# General form: values of width d_v, any divisor, additive mask
# --------------------------------------------------------------------------

def pin_ex_worked_example(orc):
    """The d_k = 4 example through the general form with values of other
    widths: V = the 8 x 8 identity (d_v = 8) returns the weights themselves
    (0.634 / 0.141 / 0.067 / 0.032 at divisor 2; fish 0.932 at 1 and 0.217 at
    8); V = the first two columns of K (d_v = 2) returns the first two printed
    outputs 0.70, 1.44."""
    g = _golden("worked_example.json")
    keys = np.array(g["keys"], dtype=np.float64).reshape(1, 1, 8, 4)
    q = np.array(g["query"], dtype=np.float64).reshape(1, 1, 1, 4)
    pr = g["printed"]
    eye = np.eye(8).reshape(1, 1, 8, 8)
    w, _ = orc.sdpa_ex(q, keys, eye, tau=pr["divisor"])
    pw = pr["weights"]
    for tok, a in zip(g["tokens"], w[0, 0, 0]):
        assert _printed_close(a, pw.get(tok, pw["others"]), pw["decimals"]), (tok, a)
    fish = g["tokens"].index("魚")
    w1, _ = orc.sdpa_ex(q, keys, eye, tau=1.0)
    w8, _ = orc.sdpa_ex(q, keys, eye, tau=8.0)
    assert _printed_close(w1[0, 0, 0, fish], pr["fish_weight_divided_by_1"]["value"], 3)
    assert _printed_close(w8[0, 0, 0, fish], pr["fish_weight_divided_by_8"]["value"], 3)
    out2, lse = orc.sdpa_ex(q, keys, np.ascontiguousarray(keys[..., :2]))
    for got, want in zip(out2[0, 0, 0], pr["output"]["value"][:2]):
        assert _printed_close(got, want, pr["output"]["decimals"]), out2
    assert _printed_close(math.exp(lse[0, 0, 0]), pr["exp_sum"]["value"], pr["exp_sum"]["decimals"])


def pin_ex_additive_causal(orc, seed=24):
    """A -inf mask on the strict upper triangle (the toy model's additive
    decoder mask) is the causal mask: same outputs and lse."""
    rng = np.random.default_rng(seed)
    for Lq, Lk in ((6, 6), (7, 4), (3, 9)):
        q = rng.standard_normal((2, 2, Lq, 5))
        k = rng.standard_normal((2, 2, Lk, 5))
        v = rng.standard_normal((2, 2, Lk, 3))
        mask = np.where(np.arange(Lk)[None, :] > np.arange(Lq)[:, None], -np.inf, 0.0)
        o1, l1 = orc.sdpa_ex(q, k, v, mask=mask)
        o2, l2 = orc.sdpa_ex(q, k, v, causal=True)
        assert np.max(np.abs(o1 - o2)) < 1e-14 and np.array_equal(np.isneginf(l1), np.isneginf(l2))
        fin = np.isfinite(l2)
        assert np.max(np.abs(l1[fin] - l2[fin])) < 1e-14


def pin_ex_mask_shift_and_weights(orc, seed=25):
    """A mask constant along a row leaves the output and shifts lse by that
    constant (the ratio identity); with q = 0 every score is 0 and a mask
    ln w_j makes the weights w_j / sum w, so o = sum w_j v_j / sum w and
    lse = ln sum w (closed form, no attention code)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 3, 4, 6))
    k = rng.standard_normal((1, 3, 5, 6))
    v = rng.standard_normal((1, 3, 5, 2))
    c = rng.standard_normal((1, 3, 4, 1)) * 5
    o0, l0 = orc.sdpa_ex(q, k, v)
    o1, l1 = orc.sdpa_ex(q, k, v, mask=np.broadcast_to(c, (1, 3, 4, 5)))
    assert np.max(np.abs(o1 - o0)) < 1e-12
    assert np.max(np.abs(l1 - (l0 + c[..., 0]))) < 1e-12
    w = rng.uniform(0.1, 3.0, size=5)
    o, l = orc.sdpa_ex(np.zeros((1, 1, 1, 6)), k[:, :1], v[:, :1], mask=np.log(w))
    want = (w[:, None] * v[0, 0]).sum(0) / w.sum()
    assert np.max(np.abs(o[0, 0, 0] - want)) < 1e-12
    assert abs(l[0, 0, 0] - math.log(w.sum())) < 1e-12


def pin_ex_masked_rows_and_padding(orc, seed=26):
    """-inf on keys >= len is the key-length mask; a row whose keys all carry
    -inf is empty: o = 0 and lse = -inf."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((2, 1, 4, 3))
    k = rng.standard_normal((2, 1, 7, 3))
    v = rng.standard_normal((2, 1, 7, 5))
    lens = [5, 2]
    mask = np.zeros((2, 1, 4, 7))
    for b, n in enumerate(lens):
        mask[b, :, :, n:] = -np.inf
    o1, l1 = orc.sdpa_ex(q, k, v, mask=mask)
    o2, l2 = orc.sdpa_ex(q, k, v, key_lens=lens)
    assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14
    mask[1, 0, 2, :] = -np.inf
    o3, l3 = orc.sdpa_ex(q, k, v, mask=mask)
    assert np.all(o3[1, 0, 2] == 0) and np.isneginf(l3[1, 0, 2])
    assert np.all(np.isfinite(o3)) and np.sum(np.isneginf(l3)) == 1


def pin_ex_brute_force(orc, seed=27):
    """General form against the pure-Python route with a bias term, to 1e-12:
    d_v != d_k, divisors other than sqrt(d_k), finite random masks, causal and
    key lengths."""
    from oracle import brute
    rng = np.random.default_rng(seed)
    for (B, H, Lq, Lk, d, dv, tau, causal, kl) in ((1, 2, 4, 6, 3, 5, 0.7, False, None),
                                                   (2, 1, 5, 5, 4, 2, 3.0, True, [3, 5]),
                                                   (1, 1, 3, 8, 2, 7, None, False, [6])):
        q = rng.standard_normal((B, H, Lq, d))
        k = rng.standard_normal((B, H, Lk, d))
        v = rng.standard_normal((B, H, Lk, dv))
        mask = rng.standard_normal((B, H, Lq, Lk))
        o, l = orc.sdpa_ex(q, k, v, causal=causal, key_lens=kl, tau=tau, mask=mask)
        t = tau if tau is not None else math.sqrt(d)
        for b in range(B):
            for h in range(H):
                for i in range(Lq):
                    n = Lk if kl is None else min(Lk, kl[b])
                    if causal:
                        n = min(n, i + 1)
                    ro, rl = brute.attention_row_biased(q[b, h, i].tolist(), k[b, h, :n].tolist(),
                                                        v[b, h, :n].tolist(), t,
                                                        mask[b, h, i, :n].tolist())
                    assert np.max(np.abs(o[b, h, i] - np.array(ro))) < 1e-12
                    assert abs(l[b, h, i] - rl) < 1e-12


ALL_PINS = [
    pin_worked_example_output, pin_worked_example_weights, pin_worked_example_scores,
    pin_temperature, pin_two_keys_d64, pin_softmax_row_properties,
    pin_temperature_limits, pin_causal, pin_padding, pin_lse_bounds,
    pin_shift_invariance, pin_score_variance, pin_head_batch_permutation,
    pin_brute_force, pin_rows_match_full, pin_input_widening,
    pin_bwd_two_keys_gradient, pin_bwd_finite_differences, pin_bwd_brute_force,
    pin_bwd_invariants,
    pin_ex_worked_example, pin_ex_additive_causal, pin_ex_mask_shift_and_weights,
    pin_ex_masked_rows_and_padding, pin_ex_brute_force,
]
