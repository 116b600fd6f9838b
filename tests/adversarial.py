"""Hand-built adversarial routings (no randomness): extreme placements the plan rule must
handle.  Used by the oracle pins (CPU) and the GPU parity tests."""

import numpy as np


def _ids(rows):
    return np.asarray(rows, dtype=np.int32)


def routings():
    """(name, R, E, K, S, slots, ids [R*S, K]) for each case."""
    out = []
    R, E, K, S = 8, 64, 4, 128
    T = R * S
    out.append(("one expert takes every token", R, E, K, S, 8,
                _ids([[0, 1 + t % 63, 1 + (t + 21) % 63, 1 + (t + 42) % 63] for t in range(T)])))
    R, E, K, S = 4, 16, 2, 64
    T = R * S
    out.append(("rank 0 has no load", R, E, K, S, 4,
                _ids([[4 + t % 12, 4 + (t + 6) % 12] for t in range(T)])))
    R, E, K, S = 4, 16, 4, 32
    T = R * S
    out.append(("every token on one rank's experts", R, E, K, S, 4,
                _ids([[12, 13, 14, 15] for _ in range(T)])))
    R, E, K, S = 4, 16, 3, 50
    T = R * S
    out.append(("identical routing for every token", R, E, K, S, 2,
                _ids([[0, 5, 10] for _ in range(T)])))
    R, E, K, S = 8, 32, 2, 64
    T = R * S
    out.append(("no slots under heavy skew", R, E, K, S, 0,
                _ids([[0, 1 + t % 31] for t in range(T)])))
    R, E, K, S = 64, 1024, 2, 8
    T = R * S
    out.append(("the last expert of 1024 takes every token", R, E, K, S, 4,
                _ids([[1023, t % 1023] for t in range(T)])))
    R, E, K, S = 2, 1024, 4, 256
    T = R * S
    even = _ids([[(4 * t + k) % 512 for k in range(K)] for t in range(T)])
    out.append(("one rank's 512 experts share every token, 4 slots", R, E, K, S, 4, even))
    out.append(("one rank's 512 experts share every token, 256 slots", R, E, K, S, 256, even))
    return out
