"""Parity checks shared by the GPU tests: each compares what the GPU stored or
computed with the fp64 oracle's result on the same seeded inputs.

  T  window entries: bit-exact bfloat16; where the oracle flags the rounding
     of T k as undecided by fp64, either bfloat16 neighbour is accepted.
  Q  codes: >= 99.99 % equal and every mismatch one level off with the
     oracle's code coordinate within 1e-5 of a rounding boundary; binary16
     scale and zero within 1e-6 relative (strict=True: every code, scale and
     zero identical).  A key group holding an undecided element is compared
     with the oracle's quantization of each of its bfloat16 variants and must
     equal one of them.
  A  attention output per (sequence, query head):
     max_i |o_i - r_i| <= 2e-3 * max_i |r_i|.

Every check returns its statistics and records them under the running test's
name; tests/conftest.py prints one line per test and the worst margins at the
end of the session.
"""
import os
import threading

import numpy as np

import oracle

ATOL_REL = 2e-3
MAX_ENUM = 6          # undecided elements per group enumerated (2^6 variants)

STATS = {}            # test id -> {"T": [...], "Q": [...], "A": [...]}
_lock = threading.Lock()


def _test_id():
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]


def record(stage, d):
    with _lock:
        STATS.setdefault(_test_id(), {}).setdefault(stage, []).append(d)


def check_windows(gpu, orc):
    """T stage: bf16 window entries equal the oracle's rounding of T k (and of v)."""
    L, S, sq = orc["L"], orc["S"], orc["squant"]
    win = np.r_[np.arange(0, min(S, L)), np.arange(max(sq, S), L)].astype(int)
    if win.size == 0:
        return dict(entries=0, ambiguous=0)
    amb = orc["k_ambiguous"][win]
    gk, ok_ = gpu["kwin"][win], orc["k_bf16"][win]
    assert np.array_equal(gk[~amb], ok_[~amb]), "window keys differ from bf16(T k)"
    if amb.any():
        alt = orc["k_alt"][win]
        assert np.all((gk[amb] == ok_[amb]) | (gk[amb] == alt[amb])), \
            "undecided window keys are neither bfloat16 neighbour"
    assert np.array_equal(gpu["vwin"][win], orc["v_bf16"][win]), "window values differ"
    st = dict(entries=int(2 * win.size * 128), ambiguous=int(amb.sum()))
    record("T", st)
    return st


def _requantize(orc, x):
    if orc.get("alpha") is None:
        return oracle.quantize(x[None], orc["bits"], orc["p_lo"], orc["p_hi"])
    return oracle.quantize_rms(x[None], orc["bits"], orc["alpha"])


def _resolve_group(orc, p, gc, gs, gz):
    """True when the GPU's codes / scale / zero of key group p equal the
    oracle's quantization of one bfloat16 variant of the group (undecided
    elements take either neighbour)."""
    idx = np.flatnonzero(orc["k_ambiguous"][p])
    if idx.size > MAX_ENUM:
        return False
    base = orc["k_bf16"][p].copy()
    alt = orc["k_alt"][p]
    for mask in range(1 << idx.size):
        x = base.copy()
        for b, e in enumerate(idx):
            if mask >> b & 1:
                x[e] = alt[e]
        r = _requantize(orc, x)
        if r["s16"][0] == gs and r["z16"][0] == gz and np.array_equal(r["codes"][0], gc):
            return True
    return False


def check_codes(gpu, orc, bits, strict=False):
    """Q stage on every quantized position of the unit."""
    q = np.asarray(orc["qpos"], dtype=int)
    st = dict(positions=int(q.size), codes=0, mismatch=0, off_by_one_at_tie=0,
              max_scale_rel=0.0, max_zero_rel=0.0, enumerated_groups=0)
    if q.size == 0:
        record("Q", st)
        return st
    rel = lambda a, b: np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
    for kind in ("k", "v"):
        gc = gpu[f"{kind}codes"][q].astype(int)
        oc = orc[f"{kind}codes"][q].astype(int)
        u = orc[f"{kind}u"][q]
        gs, gz = gpu[f"{kind}s16"][q], gpu[f"{kind}z16"][q]
        os_, oz = orc[f"{kind}s16"][q], orc[f"{kind}z16"][q]
        skip = orc["k_ambiguous"][q].any(axis=1) if kind == "k" else np.zeros(q.size, dtype=bool)
        for j in np.flatnonzero(skip):
            assert _resolve_group(orc, q[j], gc[j], gs[j], gz[j]), \
                f"key group at position {q[j]} matches no bfloat16 variant"
        st["enumerated_groups"] += int(skip.sum())
        keep = ~skip
        srel = rel(gs[keep], os_[keep])
        zrel = np.abs(gz[keep] - oz[keep]) / np.maximum(np.abs(oz[keep]), 1e-30)
        zrel[(gz[keep] == oz[keep])] = 0.0
        st["max_scale_rel"] = max(st["max_scale_rel"], float(srel.max(initial=0.0)))
        st["max_zero_rel"] = max(st["max_zero_rel"], float(zrel.max(initial=0.0)))
        if strict:
            assert np.array_equal(gs[keep], os_[keep]), f"{kind} scale differs"
            assert np.array_equal(gz[keep], oz[keep]), f"{kind} zero differs"
        else:
            assert np.all(srel <= 1e-6), f"{kind} scale mismatch"
            assert np.all(np.abs(gz[keep] - oz[keep]) <= 1e-6 * np.abs(oz[keep])), \
                f"{kind} zero mismatch"
        mism = (gc != oc) & keep[:, None]
        n = int(keep.sum()) * 128
        st["codes"] += n
        st["mismatch"] += int(mism.sum())
        if strict:
            assert not mism.any(), f"{kind} codes differ at {int(mism.sum())} elements"
        frac = mism.sum() / max(1, n)
        assert frac <= 1e-4, f"{kind} code mismatch fraction {frac}"
        if mism.any():
            assert np.all(np.abs(gc[mism] - oc[mism]) == 1)
            uu = u[mism]
            assert np.all(np.abs(uu - np.floor(uu) - 0.5) <= 1e-5), "mismatch off a boundary"
            st["off_by_one_at_tie"] += int(mism.sum())
    record("Q", st)
    return st


def check_attention(got, ref):
    """A stage; returns the largest err / (2e-3 max|ref|) over the rows."""
    worst = 0.0
    for j in range(ref.shape[0]):
        err = float(np.max(np.abs(got[j] - ref[j])))
        scale = float(np.max(np.abs(ref[j])))
        ratio = err / (ATOL_REL * scale) if scale > 0 else (0.0 if err == 0 else np.inf)
        worst = max(worst, ratio)
        assert err <= ATOL_REL * scale, (j, err, scale)
    st = dict(rows=int(ref.shape[0]), max_err_over_tol=worst)
    record("A", st)
    return st


def reference_attention(w, T, q_seq, units_of_head):
    """Oracle attention of one sequence's G*n_kv query heads over oracle units."""
    K = np.stack([oracle.readback(units_of_head[h])[0] for h in range(w.n_kv)])
    V = np.stack([oracle.readback(units_of_head[h])[1] for h in range(w.n_kv)])
    qc = np.concatenate([oracle.compensate(T[h].astype(np.float64),
                                           q_seq[h * w.group:(h + 1) * w.group].double().numpy())
                         for h in range(w.n_kv)])
    return oracle.attention(qc, K, V)


def summarize(stats):
    """One line of a test's parity statistics."""
    parts = []
    t = stats.get("T")
    if t:
        parts.append(f"T {sum(x['entries'] for x in t)} window entries"
                     f" ({sum(x['ambiguous'] for x in t)} undecided)")
    q = stats.get("Q")
    if q:
        n = sum(x["codes"] for x in q)
        m = sum(x["mismatch"] for x in q)
        match = 100.0 * (1 - m / n) if n else 100.0
        parts.append(f"Q {n} codes {match:.4f}% equal ({m} one level off at a tie)"
                     f", scale rel {max(x['max_scale_rel'] for x in q):.1e}"
                     f", zero rel {max(x['max_zero_rel'] for x in q):.1e}"
                     f", {sum(x['enumerated_groups'] for x in q)} groups by rounding variants")
    a = stats.get("A")
    if a:
        parts.append(f"A {sum(x['rows'] for x in a)} rows, max err/tol "
                     f"{max(x['max_err_over_tol'] for x in a):.3f}")
    return "; ".join(parts)
