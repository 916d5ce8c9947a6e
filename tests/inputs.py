"""Seeded workload inputs for the parity tests, with the near-tie rule:
a token whose 6th/7th routing keys are closer than 1e-4 (oracle, fp64) is
drawn again from the next attempt of its x stream."""
import numpy as np

import oracle
import synth

GAP = 1e-4
SEED = 20261202


def x_with_clear_routing(seed, fam, layer, wg, b, T, k, max_attempts=64, transform=None):
    """x rows (bf16 bits) whose routing has no near tie; `transform` (bits ->
    bits) is applied to each draw before the routing is checked."""
    H = wg.shape[1]
    attempts = [0] * T
    for _ in range(max_attempts):
        x = synth.x_rows(seed, fam, layer, H, attempts)
        if transform is not None:
            x = transform(x)
        r = oracle.router(wg, b, x, k)
        bad = [t for t in range(T) if r["gap"][t] < GAP]
        if not bad:
            return x, r, attempts
        for t in bad:
            attempts[t] += 1
    raise RuntimeError("no clear routing found")


def layer(seed, fam, li, E, H, I, T, k=6, fmt="nvfp4", sigma_g=0.02, bank_out=None):
    bank = synth.expert_bank(seed, fam, li, E, H, I, fmt, out=bank_out)
    wg, b = synth.router(seed, fam, li, E, H, sigma_g)
    x, r, att = x_with_clear_routing(seed, fam, li, wg, b, T, k)
    return dict(bank=bank, wg=wg, b=b, x=x, route=r, attempts=att, fmt=fmt)
