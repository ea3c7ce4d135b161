"""Comparison rules shared by the parity tests.

rel = max_i |got_i - ref_i| / max_i |ref_i| per output tensor (the journal's staged parity
table, §3.19, prints exactly this ratio), accepted at <= 2e-3.  Greedy ids are compared teacher
forced: both sides get the oracle's token each step and must pick the same id, except at steps
where the oracle's two largest logits are closer than 1e-3 (several ids are then correct).
"""
import numpy as np

REL_TOL = 2e-3
TIE_GAP = 1e-3


def rel_err(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def top2_gap(logits) -> float:
    v = np.sort(np.asarray(logits, np.float64).ravel())
    return float(v[-1] - v[-2])


def ids_agree(got_id, ref_logits) -> bool:
    """True when got_id is the oracle's argmax, or the oracle's top-2 gap is below TIE_GAP and
    got_id is one of the near-tied maxima."""
    ref_logits = np.asarray(ref_logits, np.float64)
    best = int(np.argmax(ref_logits))
    if int(got_id) == best:
        return True
    return top2_gap(ref_logits) < TIE_GAP and ref_logits[int(got_id)] >= ref_logits[best] - TIE_GAP
