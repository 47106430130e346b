"""Prints the oracle's largest |dq|, |dk|, |dv| for the seeded inputs of the backward
parity tests (tests/test_gpu_two_stream_bwd.py). Those tests bound each tensor's error
at 4 bf16 half-ulps of this magnitude and check that the magnitude has not moved.

CPU only; it calls nothing but the seeded input generators and the oracle.
    python -m tests.make_bwd_ref_max [--full]
(--full adds the full-size cases, about a minute and a half.)
"""

import sys

import numpy as np

import oracle
import synth

# (b, L, B, Hq, Hkv, d, mask_mode); inputs seeded with 6000 + L
CASES = [(1, 256, 4, 4, 2, 64, 0), (1, 200, 7, 2, 2, 64, 0), (1, 130, 1, 2, 1, 128, 0),
         (1, 96, 96, 2, 2, 64, 0), (1, 5, 2, 1, 1, 64, 0), (1, 200, 4, 4, 2, 128, 1),
         (2, 320, 8, 6, 3, 64, 1), (1, 256, 16, 8, 2, 128, 0), (1, 160, 16, 7, 1, 128, 0)]
# name: (seed, b, L, B, Hq, Hkv, d, mask_mode, compared (batch, KV head) groups)
FULL = {
    "FULL_05B": (1002, 8, 2048, 4, 14, 2, 64, 0, [(0, 0), (7, 1)]),
    "FULL_7B": (1003, 4, 4096, 16, 28, 4, 128, 0, [(0, 0), (3, 3)]),
    "FULL_7B_CAUSAL": (1004, 4, 4096, 16, 28, 4, 128, 1, [(2, 1)]),
}


def ref_max(seed, b, L, B, Hq, Hkv, d, mode, groups=None):
    q, k, v = synth.two_stream_qkv(seed, b, L, Hq, Hkv, d, "bf16")
    do, _, _ = synth.two_stream_qkv(seed + 77, b, L, Hq, Hkv, d, "bf16")
    rq, rk, rv = oracle.attn_two_stream_backward(q.f32, k.f32, v.f32, do.f32, L, B,
                                                 mask_mode=mode, groups=groups)
    if groups is None:
        return tuple(float(np.max(np.abs(x))) for x in (rq, rk, rv))
    g = Hq // Hkv
    mq = max(float(np.max(np.abs(rq[bi, :, kv * g:(kv + 1) * g]))) for bi, kv in groups)
    mk = max(float(np.max(np.abs(rk[bi, :, kv]))) for bi, kv in groups)
    mv = max(float(np.max(np.abs(rv[bi, :, kv]))) for bi, kv in groups)
    return mq, mk, mv


def main():
    for case in CASES:
        b, L, B, Hq, Hkv, d, mode = case
        m = ref_max(6000 + L, b, L, B, Hq, Hkv, d, mode)
        print(f"    {case}: ({m[0]:.3f}, {m[1]:.3f}, {m[2]:.3f}),", flush=True)
    if "--full" in sys.argv:
        for name, (seed, b, L, B, Hq, Hkv, d, mode, groups) in FULL.items():
            m = ref_max(seed, b, L, B, Hq, Hkv, d, mode, groups)
            print(f"{name} = ({m[0]:.4f}, {m[1]:.4f}, {m[2]:.4f})", flush=True)


if __name__ == "__main__":
    main()
