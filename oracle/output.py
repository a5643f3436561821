"""The attention output projection (oracle; test only).

DeepSeek-V2 paper (Chinese translation), section 2.1.1: the attention output
of a token is W_O applied to the concatenation of the heads' outputs
[o_1; ...; o_H]; section 2.1.2 notes that W_UV can be absorbed into W_O.
Float64.
"""

import numpy as np


def output_projection(o, w_o):
    """u [B, hidden] = W_O [o[b, 0]; ...; o[b, H-1]] for o [B, H, d_v] and
    w_o [hidden, H * d_v] (columns grouped by head)."""
    o = np.asarray(o, dtype=np.float64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, dtype=np.float64).T
