"""Pins for the CPU oracle, against things other than the oracle itself.

The MosaicQuant summary prints no worked example, so the pins are closed forms,
special cases that reduce to a library routine (numpy's fp16 conversion, int64
einsum, float64 matmul, argsort), invariants the readings imply, brute force on
tiny inputs, and one hand-worked fixture (tests/golden/handworked_small.json).
Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong tie rule) fails it.
"""
import itertools
import json
import os

import numpy as np
import pytest

from tests.nibbles import f16_bits_to_f32, f32_to_f16_bits, residual_dense, unpack_int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_small.json")
F32_EPS = np.float32(2.0 ** -23)


# --------------------------------------------------------------------------- fp16
def test_f16_conversion_matches_numpy(orc):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 3000),
        # ties between fp16 neighbours, subnormals, overflow boundary
        (np.arange(1, 400, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24),
        np.float32([65504, 65505, 65519, 65520, 65536, 1e9, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -26,
                    0.0, -0.0, 1.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 6.1035156e-05, 6.0975552e-05]),
    ]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    expect = f32_to_f16_bits(vals)
    got = np.array([orc.f16_bits(float(v)) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, expect)
    back = np.array([orc.f16_value(int(b)) for b in expect], np.float32)
    np.testing.assert_array_equal(back, expect.view(np.float16).astype(np.float32))


# --------------------------------------------------------------------------- hand-worked fixture
def test_handworked_fixture(orc):
    g = json.load(open(GOLDEN))
    x = np.array(g["x"], np.float32)
    xq, sx = orc.quantize_act(x)
    np.testing.assert_array_equal(xq, np.array(g["xq"], np.uint8))
    np.testing.assert_array_equal(sx, np.array(g["sx"], np.float32))
    np.testing.assert_array_equal(unpack_int4(xq), np.array(g["xq_codes"], np.int8))

    w = np.array(g["w"], np.float32)
    d = orc.quantize_weights(w, group=g["group"])
    np.testing.assert_array_equal(d["q"], np.array(g["q"], np.int8))
    np.testing.assert_array_equal(d["r"], np.array(g["r"], np.int8))
    np.testing.assert_array_equal(d["e"], np.array(g["e"], np.float32))
    np.testing.assert_array_equal(d["sw"], np.array(g["sw_bits"], np.uint16))

    rp = np.array(g["all_blocks_row_ptr"], np.int32)
    ci = np.array(g["all_blocks_col_idx"], np.int32)
    wq, sw, rq = orc.pack_weights(w, rp, ci, group=g["group"], bn=g["bn"], bk=g["bk"])
    np.testing.assert_array_equal(wq, np.array(g["wq"], np.uint8))
    np.testing.assert_array_equal(rq.reshape(-1), np.array(g["all_blocks_rq"], np.uint8))

    P, Pr = orc.accumulators(xq, wq, rp, ci, rq, w.shape[1], group=g["group"], bn=g["bn"],
                             bk=g["bk"])
    np.testing.assert_array_equal(P[0], np.array(g["P"], np.int32))
    np.testing.assert_array_equal(Pr[0], np.array(g["Pr_all_blocks"], np.int32))
    y = orc.output(sx, sw, P, Pr)
    np.testing.assert_allclose(y[0], g["y_all_blocks"], rtol=1e-14, atol=0)

    # selecting every block via the score path gives the same CSR
    h = orc.hessian_diag(x)
    rp2, ci2, delta, _ = orc.select_blocks(w, h, 8, group=g["group"], bn=g["bn"], bk=g["bk"])
    np.testing.assert_array_equal(rp2, rp)
    np.testing.assert_array_equal(ci2, ci)


# --------------------------------------------------------------------------- O1 activations
def _rand_act(rng, M, K, outliers=3):
    x = rng.standard_normal((M, K)).astype(np.float32)
    ch = rng.choice(K, outliers, replace=False)
    x[:, ch] *= 40
    return x


def test_act_quant_bounds_and_special_rows(orc):
    rng = np.random.default_rng(2)
    M, K = 9, 256
    x = _rand_act(rng, M, K)
    x[3] = 0.0                     # all-zero token
    x[4] = 0.0
    x[4, 17] = -3.25               # one-hot token
    x[5] = np.float32(1.0)         # constant token
    xq, sx = orc.quantize_act(x)
    q = unpack_int4(xq).astype(np.float64)
    s = sx.astype(np.float64)[:, None]
    # scale is the fp32 quotient absmax/7
    np.testing.assert_array_equal(sx, (np.abs(x).max(axis=1) / np.float32(7)).astype(np.float32))
    assert np.all(np.abs(q) <= 7)
    err = np.abs(x.astype(np.float64) - s * q)
    assert np.all(err <= s * 0.5 * (1 + 4 * F32_EPS))
    # the absmax element maps to +-7
    for m in range(M):
        if sx[m] > 0:
            k = np.argmax(np.abs(x[m]))
            assert abs(q[m, k]) == 7 and np.sign(q[m, k]) == np.sign(x[m, k])
    assert sx[3] == 0 and np.all(q[3] == 0)
    assert q[4, 17] == -7 and np.count_nonzero(q[4]) == 1
    assert np.all(q[5] == 7)


def test_act_quant_ties_to_even(orc):
    # absmax 7 -> s = 1 exactly; values j + 1/2 are exact ties
    j = np.arange(-7, 7, dtype=np.float32)
    row = np.concatenate([j + np.float32(0.5), np.float32([7.0, -7.0])])
    x = np.zeros((1, 32), np.float32)
    x[0, :row.size] = row
    xq, sx = orc.quantize_act(x)
    assert sx[0] == 1.0
    q = unpack_int4(xq)[0, :row.size].astype(np.int64)
    np.testing.assert_array_equal(q, np.rint(row.astype(np.float64)).astype(np.int64))
    assert q[list(row).index(np.float32(0.5))] == 0 and q[list(row).index(np.float32(1.5))] == 2


def test_act_quant_bf16_equals_f32_of_same_values(orc):
    import synth
    rng = np.random.default_rng(3)
    x = _rand_act(rng, 5, 384)
    bits = synth.f32_to_bf16_bits(x)
    xa, sa = orc.quantize_act(bits)
    xb, sb = orc.quantize_act(synth.bf16_bits_to_f32(bits))
    np.testing.assert_array_equal(xa, xb)
    np.testing.assert_array_equal(sa, sb)


# --------------------------------------------------------------------------- O4 Hessian
def test_hessian_diag_exact_on_integers_and_mean(orc):
    rng = np.random.default_rng(4)
    xi = rng.integers(-50, 50, size=(37, 96)).astype(np.float32)
    h = orc.hessian_diag(xi)
    # integer squares sum exactly in any order
    expect = (np.sum(xi.astype(np.int64) ** 2, axis=0) / 37.0).astype(np.float32)
    np.testing.assert_array_equal(h, expect)
    x = _rand_act(rng, 64, 128)
    np.testing.assert_allclose(h := orc.hessian_diag(x), np.mean(x.astype(np.float64) ** 2, axis=0),
                               rtol=2 ** -23)
    assert np.all(h >= 0)


# --------------------------------------------------------------------------- O2/O3 weights
def _rand_w(rng, N, K, frac=0.01):
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    idx = rng.choice(N * K, int(frac * N * K), replace=False)
    w.reshape(-1)[idx] *= 10
    return w


def test_weight_base_and_residual_closed_forms(orc):
    rng = np.random.default_rng(5)
    N, K, G = 24, 512, 128
    w = _rand_w(rng, N, K)
    w[2, 0:128] = 0.0                     # an all-zero group
    w[3, 128:256] = 0.0
    w[3, 200] = 1.5                       # one-hot group
    d = orc.quantize_weights(w, group=G)
    a = np.abs(w).reshape(N, K // G, G).max(axis=2)
    # fp16 scale = round-to-nearest-even of the fp32 quotient absmax/7
    np.testing.assert_array_equal(d["sw"], f32_to_f16_bits((a / np.float32(7)).astype(np.float32)))
    s = np.repeat(f16_bits_to_f32(d["sw"]).astype(np.float64), G, axis=1)
    q = d["q"].astype(np.float64)
    r = d["r"].astype(np.float64)
    assert np.all(np.abs(q) <= 7) and np.all(np.abs(r) <= 7)
    # base error is exact (w and s*q are within a factor of two of each other) ...
    np.testing.assert_array_equal(d["e"].astype(np.float64), w.astype(np.float64) - s * q)
    # ... and bounded by half a step
    assert np.all(np.abs(d["e"]) <= s * 0.5 * (1 + 8 * F32_EPS) + 0.0)
    # residual grid is fl32(s/14); e' is the single-rounded e - s_r*r
    sr = (s.astype(np.float32) / np.float32(14)).astype(np.float64)
    np.testing.assert_array_equal(d["ep"], (d["e"].astype(np.float64) - sr * r).astype(np.float32))
    assert np.all(np.abs(d["ep"]) <= sr * 0.5 * (1 + 8 * F32_EPS))
    assert np.all(np.abs(d["ep"]) <= np.abs(d["e"]))
    # special groups
    assert np.all(d["sw"][2, 0] == 0) and np.all(q[2, 0:128] == 0) and np.all(r[2, 0:128] == 0)
    assert q[3, 200] == 7 and np.count_nonzero(q[3, 128:256]) == 1
    # the absmax element of every non-zero group maps to +-7
    for n in range(N):
        for g in range(K // G):
            if a[n, g] > 0:
                k = g * G + np.argmax(np.abs(w[n, g * G:(g + 1) * G]))
                assert abs(q[n, k]) == 7


def test_full_budget_reconstructs_to_residual_precision(orc):
    """With every block chosen, W^ = s*q + s_r*r to within half a residual step."""
    rng = np.random.default_rng(6)
    N, K, G, bn, bk = 128, 256, 128, 64, 64
    w = _rand_w(rng, N, K)
    x = _rand_act(rng, 8, K)
    h = orc.hessian_diag(x)
    nb = (N // bn) * (K // bk)
    rp, ci, delta, sel = orc.select_blocks(w, h, nb, G, bn, bk)
    assert np.all(sel == 1)
    wq, sw, rq = orc.pack_weights(w, rp, ci, G, bn, bk)
    s = np.repeat(f16_bits_to_f32(sw).astype(np.float32), G, axis=1)
    sr = (s / np.float32(14)).astype(np.float64)
    q = unpack_int4(wq).astype(np.float64)
    R = residual_dense(rq, rp, ci, N, K, bn, bk).astype(np.float64)
    err = np.abs(w.astype(np.float64) - s.astype(np.float64) * q - sr * R)
    assert np.all(err <= sr * 0.5 * (1 + 8 * F32_EPS))
    # and without residual the error is only bounded by half a base step
    assert np.max(np.abs(w - s * q) / np.maximum(s, 1e-30)) > 0.4


# --------------------------------------------------------------------------- O5 Delta
def _diag_x(K, seed):
    """X = diag(d) with M = K: X^T X is diagonal and h_k = d_k^2 / K is exact in fp32."""
    rng = np.random.default_rng(seed)
    d = rng.integers(1, 64, size=K).astype(np.float32)
    d[rng.choice(K, 3, replace=False)] = 64.0   # outlier channels
    return np.diag(d).astype(np.float32), d


def test_delta_equals_exact_distortion_reduction_when_hessian_diagonal(orc):
    N, K, G, bn, bk = 32, 64, 32, 16, 16
    x, d = _diag_x(K, 7)
    w = _rand_w(np.random.default_rng(8), N, K, frac=0.05)
    h = orc.hessian_diag(x)
    np.testing.assert_array_equal(h, (d.astype(np.float64) ** 2 / K).astype(np.float32))
    delta = orc.delta_scores(w, h, G, bn, bk)
    nb = delta.size
    none = np.zeros(nb, np.uint8)
    d0, dd0 = orc.distortion(x, w, h, none, G, bn, bk)
    assert d0 == pytest.approx(dd0, rel=1e-12)
    for b in range(nb):
        m = none.copy()
        m[b] = 1
        d1, dd1 = orc.distortion(x, w, h, m, G, bn, bk)
        assert d0 - d1 == pytest.approx(K * delta[b], rel=1e-9, abs=1e-18)
        assert dd0 - dd1 == pytest.approx(K * delta[b], rel=1e-9, abs=1e-18)
    assert np.all(delta >= 0)


def test_topk_by_delta_is_exact_optimum_by_brute_force(orc):
    N, K, G, bn, bk = 64, 64, 32, 16, 16          # 16 blocks
    x, _ = _diag_x(K, 9)
    w = _rand_w(np.random.default_rng(10), N, K, frac=0.03)
    h = orc.hessian_diag(x)
    nb = (N // bn) * (K // bk)
    for kb in (1, 3):
        rp, ci, delta, sel = orc.select_blocks(w, h, kb, G, bn, bk)
        best, best_set = None, None
        for sub in itertools.combinations(range(nb), kb):
            m = np.zeros(nb, np.uint8)
            m[list(sub)] = 1
            de, _ = orc.distortion(x, w, h, m, G, bn, bk)
            if best is None or de < best:
                best, best_set = de, set(sub)
        got = orc.distortion(x, w, h, sel, G, bn, bk)[0]
        assert got == pytest.approx(best, rel=1e-12)
        assert set(np.flatnonzero(sel)) == best_set


def test_delta_tracks_exact_reduction_on_random_activations(orc):
    """General X (M >> K): Delta is an approximation; its ranking must still track
    the exact single-block distortion reduction (threshold fixed at this seed)."""
    rng = np.random.default_rng(11)
    N, K, G, bn, bk = 64, 128, 64, 16, 16          # 32 blocks
    x = _rand_act(rng, 1024, K, outliers=4)
    w = _rand_w(rng, N, K, frac=0.03)
    h = orc.hessian_diag(x)
    delta = orc.delta_scores(w, h, G, bn, bk)
    nb = delta.size
    none = np.zeros(nb, np.uint8)
    d0 = orc.distortion(x, w, h, none, G, bn, bk)[0]
    exact = []
    for b in range(nb):
        m = none.copy()
        m[b] = 1
        exact.append(d0 - orc.distortion(x, w, h, m, G, bn, bk)[0])
    exact = np.array(exact)
    ra = np.argsort(np.argsort(-delta))
    rb = np.argsort(np.argsort(-exact))
    rho = 1 - 6 * np.sum((ra - rb) ** 2) / (nb * (nb * nb - 1))
    assert rho > 0.9, rho
    top = max(1, nb // 10)
    assert len(set(np.argsort(-delta)[:top]) & set(np.argsort(-exact)[:top])) >= top - 1


def test_variant_scores_would_fail_the_diagonal_pin(orc):
    """Scores that drop the residual term (h * e^2) or the Hessian weight
    (e^2 - e'^2) do not equal the exact reduction: the diagonal pin can tell."""
    N, K, G, bn, bk = 32, 64, 32, 16, 16
    x, _ = _diag_x(K, 12)
    w = _rand_w(np.random.default_rng(13), N, K, frac=0.05)
    h = orc.hessian_diag(x)
    d = orc.quantize_weights(w, group=G)
    e = d["e"].astype(np.float64)
    ep = d["ep"].astype(np.float64)
    nbr, nbc = N // bn, K // bk
    blk = lambda a: a.reshape(nbr, bn, nbc, bk).sum(axis=(1, 3)).reshape(-1)
    true = blk(h[None, :] * (e * e - ep * ep))
    np.testing.assert_allclose(orc.delta_scores(w, h, G, bn, bk), true, rtol=1e-12)
    assert not np.allclose(blk(h[None, :] * e * e), true, rtol=1e-3)
    assert not np.allclose(blk(e * e - ep * ep), true, rtol=1e-3)


# --------------------------------------------------------------------------- O6 selection
def test_selection_matches_argsort_and_ties_break_by_id(orc):
    rng = np.random.default_rng(14)
    nbr, nbc = 6, 10
    delta = rng.random(nbr * nbc)
    delta[[3, 5, 17, 40]] = 2.0                 # a four-way tie at the top
    delta[[21, 33]] = delta[9]                  # and one further down
    delta[[7, 8]] = 0.0
    order = np.lexsort((np.arange(delta.size), -delta))
    prev = set()
    for k in sorted({0, 1, 2, 3, 4, 5, 6, 13, 30, nbr * nbc, int(np.flatnonzero(order == 9)[0]) + 1}):
        rp, ci, sel = orc.select_topk(delta, nbr, nbc, k)
        chosen = set(order[:k].tolist())
        assert set(np.flatnonzero(sel).tolist()) == chosen
        assert prev <= chosen                   # nested across budgets
        prev = chosen
        assert rp[0] == 0 and rp[-1] == k and np.all(np.diff(rp) >= 0)
        for i in range(nbr):
            cols = ci[rp[i]:rp[i + 1]]
            assert np.all(np.diff(cols) > 0)
            assert set((i * nbc + cols).tolist()) == {b for b in chosen if b // nbc == i}
    # the tied top blocks enter in id order: 3, then 5, then 17, then 40
    for k, expect in [(1, {3}), (2, {3, 5}), (3, {3, 5, 17})]:
        _, _, sel = orc.select_topk(delta, nbr, nbc, k)
        assert set(np.flatnonzero(sel).tolist()) == expect


# --------------------------------------------------------------------------- O8/O9 GEMM
def _pipeline(orc, x, w, kb, G=128, bn=64, bk=64):
    h = orc.hessian_diag(x)
    rp, ci, delta, sel = orc.select_blocks(w, h, kb, G, bn, bk)
    wq, sw, rq = orc.pack_weights(w, rp, ci, G, bn, bk)
    xq, sx = orc.quantize_act(x)
    P, Pr = orc.accumulators(xq, wq, rp, ci, rq, w.shape[1], G, bn, bk)
    return h, rp, ci, wq, sw, rq, xq, sx, P, Pr


def test_accumulators_equal_int64_einsum(orc):
    rng = np.random.default_rng(15)
    M, N, K, G, bn, bk = 7, 192, 512, 128, 64, 64
    x = _rand_act(rng, M, K)
    w = _rand_w(rng, N, K)
    nb = (N // bn) * (K // bk)
    h, rp, ci, wq, sw, rq, xq, sx, P, Pr = _pipeline(orc, x, w, nb // 4, G, bn, bk)
    X = unpack_int4(xq).astype(np.int64).reshape(M, K // G, G)
    Q = unpack_int4(wq).astype(np.int64).reshape(N, K // G, G)
    R = residual_dense(rq, rp, ci, N, K, bn, bk).astype(np.int64).reshape(N, K // G, G)
    np.testing.assert_array_equal(P, np.einsum("mgk,ngk->mng", X, Q))
    np.testing.assert_array_equal(Pr, np.einsum("mgk,ngk->mng", X, R))
    assert np.abs(P).max() <= 128 * 49 and np.abs(Pr).max() <= 128 * 49
    assert np.count_nonzero(Pr) > 0


def test_output_equals_dequantized_float64_matmul(orc):
    """Y = (s_x * Xq) @ (s*Q + s_r*R)^T: a plain float64 matmul over K of the
    dequantized operands, a different factorisation from the per-group sum."""
    rng = np.random.default_rng(16)
    M, N, K, G, bn, bk = 6, 256, 384, 128, 128, 64
    x = _rand_act(rng, M, K)
    w = _rand_w(rng, N, K)
    nb = (N // bn) * (K // bk)
    h, rp, ci, wq, sw, rq, xq, sx, P, Pr = _pipeline(orc, x, w, nb // 3, G, bn, bk)
    y = orc.output(sx, sw, P, Pr)
    s = np.repeat(f16_bits_to_f32(sw), G, axis=1)
    sr = (s / np.float32(14)).astype(np.float64)
    Wd = s.astype(np.float64) * unpack_int4(wq) + sr * residual_dense(rq, rp, ci, N, K, bn, bk)
    Xd = sx.astype(np.float64)[:, None] * unpack_int4(xq)
    np.testing.assert_allclose(y, Xd @ Wd.T, rtol=1e-10, atol=1e-12)
    # all scales 1, no residual: Y is the exact integer sum
    P1 = P.copy()
    y1 = orc.output(np.ones(M, np.float32), f32_to_f16_bits(np.ones_like(sw, np.float32)), P1,
                    np.zeros_like(Pr))
    np.testing.assert_array_equal(y1, P1.sum(axis=2).astype(np.float64))


def test_zero_budget_output_is_dense_base(orc):
    rng = np.random.default_rng(17)
    M, N, K = 3, 128, 256
    x = _rand_act(rng, M, K)
    w = _rand_w(rng, N, K)
    *_, xq, sx, P, Pr = _pipeline(orc, x, w, 0)
    assert np.all(Pr == 0)


# --------------------------------------------------------------------------- O10 monotone error
def test_distortion_non_increasing_in_budget(orc):
    rng = np.random.default_rng(18)
    N, K, G, bn, bk = 64, 128, 64, 16, 16        # 32 blocks
    x = _rand_act(rng, 512, K, outliers=4)
    w = _rand_w(rng, N, K, frac=0.03)
    h = orc.hessian_diag(x)
    nb = (N // bn) * (K // bk)
    prev_e, prev_d = np.inf, np.inf
    for kb in range(nb + 1):
        _, _, _, sel = orc.select_blocks(w, h, kb, G, bn, bk)
        de, dd = orc.distortion(x, w, h, sel, G, bn, bk)
        assert dd <= prev_d * (1 + 1e-12)       # a theorem: every Delta >= 0
        assert de <= prev_e * (1 + 1e-12)       # checked along this nested sweep
        prev_e, prev_d = de, dd


# --------------------------------------------------------------------------- O0 migration
def _migration_layer():
    import synth
    cfg = synth.custom_config("mig", M=48, K=256, N=96, bn=32, x_bf16=True, x_channel_frac=0.02,
                              x_channel_scale=60.0)
    inp = synth.make_inputs(cfg, seed=7)
    inp.X_bits[:, 11] = 0          # a dead input channel
    inp.X[:, 11] = 0.0
    return inp


def test_migration_is_an_equivalent_transform(orc):
    """X^ W^T equals X W^T (float64 products of the fp32 values) up to the two
    per-element roundings."""
    inp = _migration_layer()
    xh, wh, s, r = orc.migrate(inp.x_raw(), inp.W)
    ref = inp.X.astype(np.float64) @ inp.W.astype(np.float64).T
    got = xh.astype(np.float64) @ wh.astype(np.float64).T
    scale = np.abs(inp.X.astype(np.float64)) @ np.abs(inp.W.astype(np.float64)).T
    assert np.max(np.abs(got - ref) / np.maximum(scale, 1e-30)) < 3e-7


def test_migration_balances_channel_ranges(orc):
    """alpha = 1/2 makes every live channel's activation range equal its weight
    range, both sqrt(max|x_k| * max|w_k|); a dead channel keeps s = r = 1."""
    inp = _migration_layer()
    xh, wh, s, r = orc.migrate(inp.x_raw(), inp.W)
    a = np.abs(inp.X).max(axis=0).astype(np.float64)
    b = np.abs(inp.W).max(axis=0).astype(np.float64)
    live = (a > 0) & (b > 0)
    target = np.sqrt(a * b)
    np.testing.assert_allclose(np.abs(xh).max(axis=0)[live], target[live], rtol=4e-7)
    np.testing.assert_allclose(np.abs(wh).max(axis=0)[live], target[live], rtol=4e-7)
    assert s[11] == 1.0 and r[11] == 1.0 and not live[11]
    # the outlier channels' range shrinks by sqrt(a/b): they migrate into the weights
    assert np.abs(xh).max() < 0.2 * np.abs(inp.X).max()
