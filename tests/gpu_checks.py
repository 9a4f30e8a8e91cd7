"""Parity checks shared by the GPU tests: each compares what the GPU stored or
computed with the fp64 oracle's result on the same seeded inputs.

  T  window entries: bit-exact bfloat16 except where the oracle flags the
     rounding of T k as undecided by fp64.
  Q  codes: >= 99.99 % equal and every mismatch one level off with the
     oracle's code coordinate within 1e-5 of a rounding boundary; binary16
     scale and zero within 1e-6 relative.
  A  attention output per (sequence, query head):
     max_i |o_i - r_i| <= 2e-3 * max_i |r_i|.
"""
import numpy as np

import oracle

ATOL_REL = 2e-3


def check_windows(gpu, orc):
    """T stage: bf16 window entries equal the oracle's rounding of T k (and of v)."""
    L, S, sq = orc["L"], orc["S"], orc["squant"]
    win = np.r_[np.arange(0, min(S, L)), np.arange(max(sq, S), L)].astype(int)
    if win.size == 0:
        return 0
    amb = orc["k_ambiguous"][win]
    gk, ok_ = gpu["kwin"][win], orc["k_bf16"][win]
    assert np.array_equal(gk[~amb], ok_[~amb]), "window keys differ from bf16(T k)"
    assert np.array_equal(gpu["vwin"][win], orc["v_bf16"][win]), "window values differ"
    return int(amb.sum())


def check_codes(gpu, orc, bits):
    """Q stage on every quantized position (groups whose transformed keys hold an
    undecided bf16 rounding are compared on values only)."""
    q = np.asarray(orc["qpos"], dtype=int)
    if q.size == 0:
        return dict(n=0)
    stats = {}
    for kind in ("k", "v"):
        gc = gpu[f"{kind}codes"][q].astype(int)
        oc = orc[f"{kind}codes"][q].astype(int)
        u = orc[f"{kind}u"][q]
        gs, gz = gpu[f"{kind}s16"][q], gpu[f"{kind}z16"][q]
        os_, oz = orc[f"{kind}s16"][q], orc[f"{kind}z16"][q]
        if kind == "k":
            skip = orc["k_ambiguous"][q].any(axis=1)
        else:
            skip = np.zeros(q.size, dtype=bool)
        keep = ~skip
        rel = lambda a, b: np.abs(a - b) / np.maximum(np.abs(b), 1e-30)
        assert np.all(rel(gs[keep], os_[keep]) <= 1e-6), f"{kind} scale mismatch"
        assert np.all(np.abs(gz[keep] - oz[keep]) <= 1e-6 * np.abs(oz[keep])), f"{kind} zero mismatch"
        mism = (gc != oc) & keep[:, None]
        frac = mism.sum() / max(1, keep.sum() * 128)
        assert frac <= 1e-4, f"{kind} code mismatch fraction {frac}"
        if mism.any():
            assert np.all(np.abs(gc[mism] - oc[mism]) == 1)
            uu = u[mism]
            assert np.all(np.abs(uu - np.floor(uu) - 0.5) <= 1e-5), "mismatch off a boundary"
        stats[kind] = dict(mismatch=int(mism.sum()), skipped_groups=int(skip.sum()))
    return stats


def check_attention(got, ref):
    for j in range(ref.shape[0]):
        err = np.max(np.abs(got[j] - ref[j]))
        assert err <= ATOL_REL * np.max(np.abs(ref[j])), (j, err, np.max(np.abs(ref[j])))


def reference_attention(w, T, q_seq, units_of_head):
    """Oracle attention of one sequence's G*n_kv query heads over oracle units."""
    K = np.stack([oracle.readback(units_of_head[h])[0] for h in range(w.n_kv)])
    V = np.stack([oracle.readback(units_of_head[h])[1] for h in range(w.n_kv)])
    qc = np.concatenate([oracle.compensate(T[h].astype(np.float64),
                                           q_seq[h * w.group:(h + 1) * w.group].double().numpy())
                         for h in range(w.n_kv)])
    return oracle.attention(qc, K, V)


