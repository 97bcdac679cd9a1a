"""The library's dispatch layout, derived from the oracle's dispatch for the parity tests.

The library runs the always-on shared expert as a group of its own in front of the routed
experts. That placement is a layout choice of the library, not part of the method, so it lives
here with the tests rather than in the oracle: rows [0, S) are group 0 and hold tokens 0..S-1 in
order; routed expert e is group e + 1, its rows in the order of ``oracle.dispatch`` shifted by S.
offsets has N_r + 2 entries; counts stay per routed expert.
"""
import numpy as np

import oracle


def dispatch_with_shared(idx, N_r: int, shared_rows: int) -> dict:
    d = oracle.dispatch(idx, N_r)
    S = int(shared_rows)
    offsets = np.concatenate([[0], S + d["offsets"]]).astype(np.int32)
    row_token = np.concatenate([np.arange(S, dtype=np.int32), d["row_token"]]).astype(np.int32)
    return {"counts": d["counts"], "offsets": offsets, "row_token": row_token,
            "slot_row": (d["slot_row"] + S).astype(np.int32)}
