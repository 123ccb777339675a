"""Comparison of the HIP path's outputs with the oracle's, at the bars the benchmark spec sets:

* lse, entropy: |delta| <= 2e-3 |ref|, or <= 1e-6 nats absolute (entropy near 0);
* self-conditioning rows: ||delta||_2 <= 2e-3 ||ref||_2;
* argmax / Gumbel tokens, accept masks, renoised tokens, convergence flags: bit-exact,
  except where the oracle's decision margin is below 1e-4 (counted and reported).
"""
from __future__ import annotations

import numpy as np

REL_TOL = 2e-3
ABS_FLOOR = 1e-6
MARGIN = 1e-4


def _close(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    ok = (err <= REL_TOL * np.abs(ref)) | (err <= ABS_FLOOR)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    return ok, rel


def compare_vocab(out: dict, ref, commit_row: np.ndarray) -> dict:
    """out: host copies of the HIP outputs restricted to ref.rows (keys lse, entropy, argmax,
    gumbel, sc (optional)).  commit_row: bool per global row.  Returns a report; raises
    AssertionError on any failure."""
    rows = ref.rows
    cm = np.asarray(commit_row, bool)[rows]
    nc = ~cm
    rep = {"rows": int(rows.size), "commit_rows": int(cm.sum())}

    ex_a = ref.mu_argmax < MARGIN
    bad_a = (np.asarray(out["argmax"]) != ref.argmax) & ~ex_a
    rep["argmax_exempt"] = int(ex_a.sum())
    rep["argmax_exempt_differ"] = int(((np.asarray(out["argmax"]) != ref.argmax) & ex_a).sum())
    assert not bad_a.any(), f"argmax mismatch at rows {rows[bad_a][:8]}"

    if nc.any():
        ex_g = ref.mu_gumbel[nc] < MARGIN
        dg = np.asarray(out["gumbel"])[nc] != ref.gumbel[nc]
        rep["gumbel_exempt"] = int(ex_g.sum())
        rep["gumbel_exempt_differ"] = int((dg & ex_g).sum())
        assert not (dg & ~ex_g).any(), f"gumbel mismatch at rows {rows[nc][dg & ~ex_g][:8]}"
        if out.get("lse") is not None:
            ok, rel = _close(np.asarray(out["lse"])[nc], ref.lse[nc])
            rep["lse_max_rel"] = float(rel.max())
            assert ok.all(), f"lse off at rows {rows[nc][~ok][:8]}"
        ok, rel = _close(np.asarray(out["entropy"])[nc], ref.entropy[nc])
        rep["entropy_max_rel"] = float(rel.max())
        rep["entropy_floor_passes"] = int((ok & (rel > REL_TOL)).sum())
        assert ok.all(), f"entropy off at rows {rows[nc][~ok][:8]}"
        if out.get("sc") is not None:
            got = np.asarray(out["sc"], np.float64)[nc]
            want = ref.sc[nc]
            num = np.linalg.norm(got - want, axis=1)
            den = np.linalg.norm(want, axis=1)
            rel = num / np.maximum(den, 1e-30)
            rep["sc_max_rel"] = float(rel.max())
            assert (rel <= REL_TOL).all(), f"selfcond off at rows {rows[nc][rel > REL_TOL][:8]}"
    if cm.any():
        # commit rows: only argmax is written
        if out.get("lse") is not None:
            assert np.all(np.isnan(np.asarray(out["lse"])[cm]))
        assert np.all(np.isnan(np.asarray(out["entropy"])[cm]))
        assert np.all(np.asarray(out["gumbel"])[cm] == -7)
        if out.get("sc") is not None:
            assert np.all(np.isnan(np.asarray(out["sc"])[cm]))
    return rep


def compare_sampler(got: dict, ref, commit: np.ndarray, C: int) -> dict:
    """got: host arrays next_tokens, accept, converged, mean_entropy, prev_argmax,
    stable_count.  ref: oracle SamplerResult."""
    n = ref.converged.shape[0]
    cm = np.repeat(np.asarray(commit, bool), C) if commit is not None else np.zeros(n * C, bool)
    ex = ref.mu_accept < MARGIN
    d_acc = np.asarray(got["accept"]) != ref.accept
    rep = {"accept_exempt": int(ex.sum()), "accept_exempt_differ": int((d_acc & ex).sum())}
    assert not (d_acc & ~ex).any(), f"accept mismatch at {np.nonzero(d_acc & ~ex)[0][:8]}"
    same_dec = ~d_acc
    d_tok = np.asarray(got["next_tokens"]) != ref.next_tokens
    assert not (d_tok & same_dec).any(), f"token mismatch at {np.nonzero(d_tok & same_dec)[0][:8]}"
    assert np.array_equal(np.asarray(got["prev_argmax"]), ref.prev_argmax)
    assert np.array_equal(np.asarray(got["stable_count"]), ref.stable_count)
    exc = ref.mu_conv < MARGIN
    d_conv = np.asarray(got["converged"]) != ref.converged
    assert not (d_conv & ~exc).any()
    ncv = ~np.asarray(commit, bool) if commit is not None else np.ones(n, bool)
    if ncv.any() and got.get("mean_entropy") is not None:
        me = np.asarray(got["mean_entropy"], np.float64)[ncv]
        assert np.allclose(me, ref.mean_entropy[ncv], rtol=1e-6, atol=1e-7)
    return rep
