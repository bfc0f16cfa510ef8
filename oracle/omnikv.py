"""OmniKV-style cross-layer reuse of top-k token indices (oracle side).

[tokendh] section "把边界划在'生命周期'上": OmniKV judges which history matters
at some layers and hands that judgement to the following layers, which reuse
it instead of recomputing it.

Readings taken where the pages are silent:
  * a filter layer runs full attention and scores each valid token by the sum,
    over the query heads of a KV head, of their softmax weights on it;
  * its view is the top_k tokens by that score (ties to the lower position),
    ascending, one view per (batch, KV head), the newest token included;
  * layers before the first filter layer run full attention; every other
    non-filter layer attends only over the view of the nearest filter layer
    below it; selection is redone at every decode step.
"""
import numpy as np

from .attention import unit_attention
from .selection import boundary_gap, top_k_ascending


def omnikv_scores(logits, lse, n):
    """logits [G][>=n], lse [G] over slots [0, n) -> score [n] = sum_h exp(logit_h - lse_h)."""
    p = np.exp(np.asarray(logits, np.float64)[:, :n] - np.asarray(lse, np.float64)[:, None])
    return p.sum(axis=0)


def omnikv_select(logits, lse, n, top_k):
    """Ascending top_k token ids of one unit (float32 decisions)."""
    return top_k_ascending(omnikv_scores(logits, lse, n), top_k)


def omnikv_layer_views(n_layers, filters):
    """Per layer: ("dense", None), ("filter", None) or ("sparse", f) with f the filter layer it reuses."""
    plan = []
    for layer in range(n_layers):
        below = [f for f in filters if f < layer]
        if layer in filters:
            plan.append(("filter", None))
        elif not below:
            plan.append(("dense", None))
        else:
            plan.append(("sparse", max(below)))
    return plan


def unit_sweep(q_layers, K_layers, V_layers, n, filters, top_k, scale, layers=None, gaps=None):
    """One unit, one decode step through a layer stack.
    q_layers[l] [G][D]; K_layers[l] [>=n][D]; V_layers[l] [>=n][Dv].
    Returns (outs {layer: [G][Dv]}, views {filter layer: ascending ids}).  If `gaps` is
    a dict, the relative top-k boundary gap of each filter layer is stored in it."""
    plan = omnikv_layer_views(len(q_layers), filters)
    views, outs = {}, {}
    want = set(range(len(q_layers))) if layers is None else set(layers)
    last = max(want)
    for layer, (mode, src) in enumerate(plan):
        if layer > last:
            break
        if mode == "sparse":
            if layer not in want:
                continue
            toks = views[src]
        else:
            toks = np.arange(n)
        Kt = np.asarray(K_layers[layer], np.float64)[toks]
        Vt = np.asarray(V_layers[layer], np.float64)[toks]
        out, lse, logits = unit_attention(q_layers[layer], Kt, Vt, scale)
        if mode == "filter":
            views[layer] = omnikv_select(logits, lse, n, top_k)
            if gaps is not None:
                gaps[layer] = boundary_gap(omnikv_scores(logits, lse, n), top_k)
        outs[layer] = out
    return outs, views
