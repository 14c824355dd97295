"""SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", 2014) and the uniform [-1, 1) draws built from it, for inputs
that a C program generates on its own side (tests/c_abi/mfa_c_demo.cpp
implements the same generator from the same definition)."""

import numpy as np

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1


def splitmix64(state, count):
    """`count` outputs starting from `state`; returns (uint64 array, new state)."""
    with np.errstate(over="ignore"):
        s = (np.uint64(state) + np.arange(1, count + 1, dtype=np.uint64) * np.uint64(_GAMMA))
        z = s
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z, (int(state) + count * _GAMMA) & _MASK


def uniform_pm1(state, count):
    """float32 values 2 * ((x >> 40) / 2^24) - 1 in [-1, 1); returns (values, new state)."""
    z, state = splitmix64(state, count)
    u = (z >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    return u * np.float32(2.0) - np.float32(1.0), state
