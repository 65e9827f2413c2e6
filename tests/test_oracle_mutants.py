"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The oracle's source is read, one edit is applied, and the edited copy is run in
a fresh module namespace (the real oracle is untouched).  A mutant passes the
test only if at least one of the pins in oracle_pins.py rejects it.
"""
import os
import types

import pytest

import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(fname, edit):
    src = open(os.path.join(ROOT, "oracle", fname)).read()
    old, new, nth = edit
    pos = -1
    for _ in range(nth + 1):
        pos = src.index(old, pos + 1)
    src = src[:pos] + new + src[pos + len(old):]
    mod = types.ModuleType("oracle_mutant_" + fname[:-3])
    exec(compile(src, fname, "exec"), mod.__dict__)
    return mod


# (file, (old text, new text, which occurrence), checks that should catch it)
MUTANTS = {
    "diagonal dropped": ("attention.py", ("p = j <= i", "p = j < i", 0), "fwd"),
    "one token of lookahead": ("attention.py", ("p = j <= i", "p = j <= i + 1", 0), "fwd"),
    "scores transposed": ("attention.py", ("(q[r0:r1] @ k[:nc].T)", "(k[r0:r1] @ q[:nc].T)", 0), "fwd"),
    "scale 1/4": ("attention.py", ("@ k[:nc].T) * scale", "@ k[:nc].T) * 0.25", 0), "fwd"),
    "lse in log2": ("attention.py", ("lse[r0:r1] = m + np.log(z)", "lse[r0:r1] = m + np.log2(z)", 0), "fwd"),
    "not normalised": ("attention.py", ("_sum_present(w / z[:, None],", "_sum_present(w,", 0), "fwd"),
    "max added": ("attention.py", ("np.exp(s - m[:, None])", "np.exp(s + m[:, None])", 0), "fwd"),
    "absent pairs multiplied": ("attention.py",
                                ("out[:, d] += np.where(present[:, j], term, 0.0)",
                                 "out[:, d] += np.nan_to_num(term, nan=0.0)", 0), "fwd"),
    "group-by joined on j": ("attention.py", ("m = best[rows]", "m = best[cols]", 0), "fwd"),
    "dS sign": ("attention.py", ("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])", 0), "bwd"),
    "delta without P": ("attention.py", ("delta = np.sum(p * dp, axis=1)", "delta = np.sum(dp, axis=1)", 0), "bwd"),
    "dQ unscaled": ("attention.py", ("dq[r0:r1] = (ds @ k[:nc]) * scale", "dq[r0:r1] = (ds @ k[:nc])", 0), "bwd"),
    "dK from k": ("attention.py", ("(ds.T @ q[r0:r1])", "(ds.T @ k[r0:r1])", 0), "bwd"),
    "dV from v": ("attention.py", ("dv[:nc] += p.T @ dout[r0:r1]", "dv[:nc] += p.T @ v[r0:r1]", 0), "bwd"),
    "dP from k": ("attention.py", ("dout[r0:r1] @ v[:nc].T", "dout[r0:r1] @ k[:nc].T", 0), "bwd"),
    "dS transposed in dQ": ("attention.py", ("(ds @ k[:nc])", "(ds.T[:r1 - r0, :] @ k[:nc])", 0), "bwd"),
    "backward unmasked": ("attention.py", ("present = _present(r0, r1, nc, mask, window, seg)",
                                           "present = np.ones((r1 - r0, nc), dtype=bool)", 1), "bwd"),
    "window one key wider": ("attention.py", ("(i - j < window)", "(i - j <= window)", 0), "mask"),
    "window not causal": ("attention.py", ("p = (j <= i) & (i - j < window)",
                                           "p = np.abs(i - j) < window", 0), "mask"),
    "full keeps the causal predicate": ("attention.py",
                                        ("p = np.ones((r1 - r0, ncols), dtype=bool)",
                                         "p = np.broadcast_to(j <= i, (r1 - r0, ncols))", 0),
                                        "mask"),
    "full sees only earlier blocks' keys": ("attention.py",
                                            ('return n if mask == "full" else r1', "return r1", 0),
                                            "mask"),
    "loss without the half": ("attention.py", ("np.sum(o * o) / 2", "np.sum(o * o)", 0), "loss"),
    "loss not squared": ("attention.py", ("np.sum(o * o) / 2", "np.sum(o) / 2", 0), "loss"),
    "loss of |o|": ("attention.py", ("np.sum(o * o) / 2", "np.sum(np.abs(o)) / 2", 0), "loss"),
    "forward heads shifted": ("attention.py", ("o[bi, hi] = oh", "o[bi, (hi + 1) % o.shape[1]] = oh", 0),
                              "batch"),
    "forward lse of another batch": ("attention.py", ("lse[bi, hi] = lh",
                                                      "lse[(bi + 1) % lse.shape[0], hi] = lh", 0),
                                     "batch"),
    "backward heads shifted": ("attention.py", ("dst[bi, hi] = g", "dst[bi, (hi + 1) % dst.shape[1]] = g", 0),
                               "batch"),
    "backward ignores dout": ("attention.py", ("arrays = (q, k, v, np.asarray(dout, dtype=np.float64))",
                                               "arrays = (q, k, v, np.asarray(dout, dtype=np.float64) * 0 + q)", 0),
                              "batch_dout"),
    "segments ignored": ("attention.py", ("p = p & (seg[r0:r1, None] == seg[None, :ncols])",
                                          "p = p", 0), "seg"),
    "segments ordered instead of equal": ("attention.py",
                                          ("(seg[r0:r1, None] == seg[None, :ncols])",
                                           "(seg[r0:r1, None] >= seg[None, :ncols])", 0), "seg"),
    "key segments shifted by one": ("attention.py", ("seg[None, :ncols])",
                                                     "np.roll(seg, 1)[None, :ncols])", 0), "seg"),
    "batch 0's segments for every batch": ("attention.py", ("np.asarray(seg)[b]",
                                                            "np.asarray(seg)[0]", 0), "seg"),
    "backward ignores segments": ("attention.py", ("present = _present(r0, r1, nc, mask, window, seg)",
                                                   "present = _present(r0, r1, nc, mask, window)", 1),
                                  "seg"),
    "bandwidth 2h^2": ("nw.py", ("/ denom", "/ (2 * denom)", 0), "nw"),
    "y against x": ("nw.py", ("(ty[r0:r1, None] - sy[None, :])", "(ty[r0:r1, None] - sx[None, :])", 0), "nw"),
    "mean of weights": ("nw.py", ("(w @ sv) / w.sum(axis=1)", "(w @ sv) / w.shape[1]", 0), "nw"),
    "min subtracted": ("nw.py", ("e.max(axis=1, keepdims=True)", "e.min(axis=1, keepdims=True)", 0), "nw"),
}

GROUPS = {"seg": oracle_pins.SEG_CHECKS,
          "loss": oracle_pins.LOSS_CHECKS,
          "batch": oracle_pins.BATCH_CHECKS,
          "batch_dout": oracle_pins.BATCH_CHECKS,
          "fwd": oracle_pins.ATTENTION_FORWARD_CHECKS,
          "bwd": oracle_pins.ATTENTION_BACKWARD_CHECKS,
          "nw": oracle_pins.NW_CHECKS,
          "mask": oracle_pins.MASK_CHECKS}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name):
    fname, edit, group = MUTANTS[name]
    mod = _load(fname, edit)
    import oracle
    names = ("forward_head", "forward_head_relational", "backward_head", "loss", "forward",
             "backward", "nw_average")
    orc = types.SimpleNamespace(**{a: getattr(oracle, a) for a in names})
    for attr in names:
        if hasattr(mod, attr):
            setattr(orc, attr, getattr(mod, attr))
    caught = []
    for check in GROUPS[group]:
        try:
            check(orc)
        except Exception as e:  # noqa: BLE001 - any rejection counts
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name!r} passed every {group} pin"
