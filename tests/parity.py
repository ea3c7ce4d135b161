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


DRAW_MARGIN = 1e-4


def topk_draw_margins(logits, k, temperature, u):
    """For the top-k draw (temperature, k largest with ties to the lower index, softmax, first
    index in descending order whose cumulative mass exceeds u * total), in fp64:
    (distance of u * total from the nearest cumulative boundary, relative to the total;
     gap between the k-th and (k+1)-th largest logit, inf when k covers the vocabulary).
    A fp32 draw may legitimately differ from the fp64 one when the first is below DRAW_MARGIN
    or the second below TIE_GAP."""
    v = np.asarray(logits, np.float64).ravel()
    n = v.size
    k = n if k <= 0 or k > n else k
    order = sorted(range(n), key=lambda i: (-v[i], i))
    top = order[:k]
    z = np.exp(v[top] / temperature - v[top[0]] / temperature)
    c = np.cumsum(z)
    total = c[-1]
    margin = float(np.min(np.abs(c - u * total)) / total)
    gap = float(v[order[k - 1]] - v[order[k]]) if k < n else float("inf")
    return margin, gap


# ---- the sampler chain ------------------------------------------------------------------------

def sampling_of(cfg):
    """The GPU model's sampling dict for a config (None: plain greedy)."""
    mode = cfg.get("sample_mode", 0)
    pen = cfg.get("rep_penalty", 1.0)
    if mode == 0 and pen in (0.0, 1.0) and not cfg.get("cfg", 0):
        return None
    return dict(mode=mode, top_k=cfg.get("top_k", 0), temperature=cfg.get("temperature", 1.0), seed=cfg.get("seed", 0),
                top_p=cfg.get("top_p", 0.0), min_p=cfg.get("min_p", 0.0), rep_penalty=pen,
                order=cfg.get("sample_order", "t3"), cfg=cfg.get("cfg", 0), cfg_weight=cfg.get("cfg_weight", 0.0))


def uses_chain(cfg) -> bool:
    return sampling_of(cfg) is not None


def chain_margins(logits, cfg, u, hist=(), penalty=True):
    """The oracle's id and decision margins for one head (penalty False: a head the repetition
    penalty does not cover)."""
    import oracle
    return oracle.sample_chain(logits, u, mode=cfg.get("sample_mode", 0), top_k=cfg.get("top_k", 0),
                               temperature=cfg.get("temperature", 1.0), top_p=cfg.get("top_p", 0.0),
                               min_p=cfg.get("min_p", 0.0),
                               rep_penalty=cfg.get("rep_penalty", 1.0) if penalty else 1.0,
                               order=cfg.get("sample_order", "t3"), hist=hist)


def chain_near_boundary(margins, mass_tol=DRAW_MARGIN, gap_tol=TIE_GAP) -> bool:
    """True when a fp32 run may take another decision than the fp64 oracle: the draw, the top-p
    or the min-p cut lies within mass_tol of its boundary, or the top-k cut, the greedy argmax or
    the walk order around the drawn id is decided by a logit gap below gap_tol (an exact tie,
    gap 0, is decided by index on both sides and does not count)."""
    return (margins["draw"] < mass_tol or margins["top_p"] < mass_tol or margins["min_p"] < mass_tol
            or 0.0 < margins["top_k"] < gap_tol or margins["greedy"] < gap_tol
            or 0.0 < margins["order"] < gap_tol)
