"""Chain Cache bookkeeping (oracle side).

[tokendh] section "聊天记录也能'续命':Chain Cache": a method may have physically
deleted part of a conversation's KV, yet the system remembers the logical
prefix (the tokens that were said), keeps it apart from the physical storage
(the rows still held), recognises a new turn that continues that prefix, and
computes only the new part.  [netics] "SparseEngine 统一接入十五种稀疏注意力":
the ChainCacheIndex ties a session to its retained per-layer KV, the method's
metadata and the logical token prefix.

Readings taken:
  * a stored session is reusable for a request when its logical prefix is a
    prefix of the request's tokens (the new turn continues it); among reusable
    sessions the longest prefix wins, the lower session index on equal lengths;
  * each unit keeps a position map: physical row -> logical position;
  * a compaction that keeps physical rows kept[0..n) gives the map
    map_out[i] = map_in[kept[i]] (identity map_in before the first one);
  * appending n new tokens after the n_phys retained rows gives them logical
    positions logical_len .. logical_len + n - 1.
"""
import numpy as np


def match_prefix(prefixes, tokens):
    """(session index, matched length) of the longest stored prefix that `tokens`
    continues; (-1, 0) if none."""
    best, blen = -1, 0
    for s, p in enumerate(prefixes):
        n = len(p)
        if n <= len(tokens) and list(tokens[:n]) == list(p) and (best < 0 or n > blen):
            best, blen = s, n
    return best, blen


def compose_positions(map_in, kept, n_keep):
    """map_out[i] = map_in[kept[i]] for i < n_keep (map_in None: kept itself), -1 after."""
    kept = np.asarray(kept)
    out = np.full(kept.shape, -1, np.int64)
    src = kept[:n_keep] if map_in is None else np.asarray(map_in)[kept[:n_keep]]
    out[:n_keep] = src
    return out


def append_positions(pos_map, n_phys, logical_len, n_new):
    """Positions of n_new rows appended after n_phys retained rows (copy of pos_map)."""
    out = np.array(pos_map, np.int64, copy=True)
    out[n_phys:n_phys + n_new] = logical_len + np.arange(n_new)
    return out
