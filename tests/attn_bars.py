"""Bars for comparing a GPU attention output with the oracle's tiled path.

The spec bar is one relative L2 over the whole output (<= 5e-3 against
the oracle's quantised tiled path).  On its own it can hide a local fault: one
wrong head among 48, or a bad tail block, barely moves a global norm, and on
the long workload the output is dominated by the V mean that the epilogue adds
exactly.  So every attention comparison also checks:

  * the same relative L2 per (b, h);
  * the attention term: after allowing each element its bf16 output rounding
    (half an ulp of the oracle value, plus 1/128 of that for a neighbouring
    binade), the remaining deviation, as an L2 norm, is at most 5e-3 of the
    L2 norm of (oracle - v_mean) -- globally and per (b, h);
  * a max-abs guard: no element deviates (beyond its rounding allowance) by
    more than 1/16 of the largest |oracle - v_mean| of its head.  One FP8
    rounding of one probability that lands on the other side of a midpoint
    moves an output by at most 1/8 of that probability's share times the
    spread of V, so a valid kernel stays far inside this; a wrong row, a
    wrong head or garbage does not.
"""
import numpy as np

TOL_ORACLE = 5e-3
MAXABS_FRAC = 1.0 / 16


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half an ulp of bf16 at |x| (8 significant bits); subnormal floor 2^-134."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64)) * (1.0 + 2.0 ** -7)


def _rel(x, ref):
    n = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((x - ref).ravel()) / n) if n > 0 else float(np.linalg.norm(x.ravel()))


def attention_report(got: np.ndarray, tiled: np.ndarray, v_mean: np.ndarray) -> dict:
    """got, tiled: fp64 [B, H, R, D]; v_mean: [B, H, D].  Returns the measured
    figures (global, worst head) for every bar above."""
    got = np.asarray(got, np.float64)
    tiled = np.asarray(tiled, np.float64)
    vm = np.asarray(v_mean, np.float64)[:, :, None, :]
    term = tiled - vm
    excess = np.maximum(np.abs(got - tiled) - bf16_half_ulp(tiled), 0.0)
    B, H = got.shape[:2]
    rel_head, term_head, maxabs_head = [], [], []
    for b in range(B):
        for h in range(H):
            rel_head.append(_rel(got[b, h], tiled[b, h]))
            tn = np.linalg.norm(term[b, h].ravel())
            term_head.append(float(np.linalg.norm(excess[b, h].ravel()) / tn) if tn > 0
                             else float(np.linalg.norm(excess[b, h].ravel())))
            tmax = float(np.abs(term[b, h]).max())
            maxabs_head.append(float(excess[b, h].max()) / tmax if tmax > 0 else float(excess[b, h].max()))
    tn = np.linalg.norm(term.ravel())
    return {
        "rel": _rel(got, tiled),
        "rel_head_max": max(rel_head),
        "term": float(np.linalg.norm(excess.ravel()) / tn) if tn > 0 else float(np.linalg.norm(excess.ravel())),
        "term_head_max": max(term_head),
        "maxabs_head_max": max(maxabs_head),
        "finite": bool(np.isfinite(got).all()),
    }


def check_attention(got, tiled, v_mean, log=print, label=""):
    r = attention_report(got, tiled, v_mean)
    log(f"  {label}vs oracle: rel L2 {r['rel']:.3e} (worst head {r['rel_head_max']:.3e}); "
        f"attention term {r['term']:.3e} (worst head {r['term_head_max']:.3e}); "
        f"max excess / head max|O-v_mean| {r['maxabs_head_max']:.3e}")
    assert r["finite"]
    assert r["rel"] <= TOL_ORACLE
    assert r["rel_head_max"] <= TOL_ORACLE
    assert r["term"] <= TOL_ORACLE
    assert r["term_head_max"] <= TOL_ORACLE
    assert r["maxabs_head_max"] <= MAXABS_FRAC
    return r
