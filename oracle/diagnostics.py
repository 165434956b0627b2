"""Selection diagnostics: distortion-recovery curves of residual allocations.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the HIP library never
uses it. It builds on the oracle's own quantizers, Hessian estimate and
Delta-scores, and evaluates on small synthetic layers how much of the output
distortion ||X (W^ - W_S)^T||_F^2 a residual budget recovers, for

* the Delta-score top-K block selection the method uses (MosaicQuant summary,
  Methodology 2 "Block-wise Residual Allocation": blocks ranked by the residual
  error weighted by the diagonal-Hessian sensitivity of their input channels);
* exact greedy block selection: at each step the block whose residual lowers the
  exact output distortion most (brute force over the remaining blocks), the
  costly evaluation the Delta-score stands in for;
* channel-wise allocation at the same number of residual weights: whole input
  channels ranked by the same h-weighted error reduction, the granularity the
  method's block-level allocation is contrasted with;
* random block selection (a floor).

Recovery at a selection S is (D(empty) - D(S)) / (D(empty) - D(all)), with D the
exact output distortion in float64. W_S = s*q + s_r*r on the selected weights and
s*q elsewhere (the oracle's quantizers), so D(all) is the distortion left by the
full 4-bit residual.
"""
from __future__ import annotations

import numpy as np

from . import Oracle


def _errors(orc: Oracle, w, group):
    d = orc.quantize_weights(w, group)
    return d["e"].astype(np.float64), d["ep"].astype(np.float64)


def _distortion(x64, err):
    out = x64 @ err.T
    return float(np.sum(out * out))


def curves(x, w, group=128, bn=64, bk=64, budgets=None, seed=0, orc: Oracle | None = None,
           greedy=True):
    """Distortion-recovery curves for the four allocations at the given budgets
    (percent of blocks; channel-wise uses the same number of residual weights).
    Returns dict(budgets, k_blocks, delta_topk, greedy_exact, channel, random,
    d_empty, d_all) with recoveries in [0, 1] (greedy_exact is None if greedy=False)."""
    orc = orc or Oracle()
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    M, K = x.shape
    N = w.shape[0]
    nbr, nbc = N // bn, K // bk
    nb = nbr * nbc
    if budgets is None:
        budgets = list(range(0, 101, 10))
    ks = [(p * nb) // 100 for p in budgets]
    x64 = x.astype(np.float64)
    e, ep = _errors(orc, w, group)
    d_empty = _distortion(x64, e)
    d_all = _distortion(x64, ep)
    span = d_empty - d_all

    def rec(d):
        return (d_empty - d) / span if span > 0 else 1.0

    def block_mask(sel):
        m = np.zeros((N, K), bool)
        for b in sel:
            i, j = divmod(int(b), nbc)
            m[i * bn:(i + 1) * bn, j * bk:(j + 1) * bk] = True
        return m

    # Delta-score top-K (the oracle's scores and its tie rule)
    h = orc.hessian_diag(x)
    delta = orc.delta_scores(w, h, group, bn, bk)
    order = np.lexsort((np.arange(nb), -delta))
    delta_curve = [rec(_distortion(x64, np.where(block_mask(order[:k]), ep, e))) for k in ks]

    # random blocks
    rng = np.random.default_rng(seed)
    rorder = rng.permutation(nb)
    random_curve = [rec(_distortion(x64, np.where(block_mask(rorder[:k]), ep, e))) for k in ks]

    # channel-wise: input channels by sum_n h_k (e^2 - e'^2), as many residual weights
    ch_score = (h.astype(np.float64) * np.sum(e * e - ep * ep, axis=0))
    ch_order = np.lexsort((np.arange(K), -ch_score))
    chan_curve = []
    for k in ks:
        c = (k * bn * bk) // N
        m = np.zeros((N, K), bool)
        m[:, ch_order[:c]] = True
        chan_curve.append(rec(_distortion(x64, np.where(m, ep, e))))

    # exact greedy: output error E = X D^T updated block by block
    greedy_curve = None
    if greedy:
        E = x64 @ e.T                                   # M x N
        chosen = np.zeros(nb, bool)
        dcur = d_empty
        kmax = max(ks)
        gains_at = {0: d_empty}
        for step in range(1, kmax + 1):
            best, best_gain, best_new = -1, -np.inf, None
            for b in np.nonzero(~chosen)[0]:
                i, j = divmod(int(b), nbc)
                rows, cols = slice(i * bn, (i + 1) * bn), slice(j * bk, (j + 1) * bk)
                corr = x64[:, cols] @ (e[rows, cols] - ep[rows, cols]).T    # M x bn
                old = E[:, rows]
                new = old - corr
                gain = float(np.sum(old * old) - np.sum(new * new))
                if gain > best_gain:
                    best, best_gain, best_new = b, gain, new
            i, j = divmod(int(best), nbc)
            E[:, i * bn:(i + 1) * bn] = best_new
            chosen[best] = True
            dcur -= best_gain
            gains_at[step] = dcur
        greedy_curve = [rec(gains_at[k]) for k in ks]

    return dict(budgets=list(budgets), k_blocks=ks, delta_topk=delta_curve, greedy_exact=greedy_curve,
                channel=chan_curve, random=random_curve, d_empty=d_empty, d_all=d_all)


def _main():
    import json
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import synth
    out = {}
    for name, cfg in [
        ("llama_like", synth.custom_config("diag_llama", M=512, K=512, N=256, bn=32, bk=32, x_bf16=False)),
        ("qwen_like", synth.custom_config("diag_qwen", M=512, K=512, N=256, bn=32, bk=32, x_bf16=False,
                                          x_dist="t3", x_channel_frac=0.02, x_channel_scale=40.0)),
    ]:
        inp = synth.make_inputs(cfg)
        out[name] = curves(inp.X, inp.W, group=128, bn=cfg.bn, bk=cfg.bk,
                           budgets=[0, 5, 10, 20, 30, 50, 75, 100])
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    _main()
