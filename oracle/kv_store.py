"""KV-pool scatter (oracle).

The new tokens' K and V rows are written at the pool slots listed for them
(the "out_cache_loc" of the v0.2 runtime walkthrough in the SGLang handbook
chapter on v0.2, "CUDA Graph" section, where padded entries point at slot 0).
The pool after the store equals the pool before with those rows replaced.
"""

import numpy as np


def kv_store(pool, new_rows, loc):
    """pool: [N+1, Hkv, D]; new_rows: [T, Hkv, D]; loc: [T] slot indices.
    Returns the updated copy.  Later entries win on repeated slots."""
    out = np.array(pool, copy=True)
    for t, s in enumerate(np.asarray(loc, dtype=np.int64)):
        out[s] = new_rows[t]
    return out
