"""Finds the router-bias scale of the congested layer (T=16384, d=768, E=64,
c=2.0): the bias of expert e is -1.1 * ln(e + 1) * beta (a Zipf(1.1) profile),
and beta is bisected so that expert 0 gets 15 % of the raw top-1 choices under
the fp64 oracle router.  Prints the value stored as workloads.ZIPF_BETA.

Uses only the seeded generators and the oracle.  Run:  python -m oracle.calibrate_bias
"""
import numpy as np

import workloads
from oracle.switch_oracle import router_logits


def top_share(beta: float) -> float:
    cfg = workloads.CONFIGS[3]
    inp = workloads.make_router_inputs(cfg, beta=beta)
    z = router_logits(inp.x, inp.w_r, inp.b_r)
    return float(np.mean(np.argmax(z, axis=1) == 0))


def main():
    lo, hi = 0.0, 1.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if top_share(mid) < 0.15:
            lo = mid
        else:
            hi = mid
    beta = float(np.float32(0.5 * (lo + hi)))
    print(f"beta = {beta!r}  top share = {top_share(beta):.5f}")


if __name__ == "__main__":
    main()
