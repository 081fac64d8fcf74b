"""Seeded ragged problem shapes for the GPU parity sweeps: lengths on, just
below or just past the kernels' tile edges, or anywhere below a cap, with
Nq and Nk drawn independently, so partial tiles, single-tile rows, causal
Nq != Nk and per-wave ranges that end before, at or after their
workgroup's last tile all occur."""
import numpy as np


def ragged_cases(n, seed, edges, cap, causal_frac=0.6):
    """n tuples (B, H, Nq, Nk, d, dtype, causal); reproducible from seed."""
    rng = np.random.default_rng(seed)

    def length():
        if rng.random() < 0.6:
            return max(1, int(rng.choice(edges)) + int(rng.integers(-1, 2)))
        return int(rng.integers(1, cap))

    cases = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), length(), length(), d,
                      str(rng.choice(["fp16", "bf16"])), bool(rng.random() < causal_frac)))
    return cases


def case_id(c):
    return "B{}H{}q{}k{}d{}{}{}".format(c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else "")
