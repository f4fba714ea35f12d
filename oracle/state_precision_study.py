"""CPU study: decode with the SATA state kept in fp16 or bf16.

Test infrastructure, like the oracle it uses (no GPU, no library code).  A
head's state after a prefill is rounded to the storage format, then every
decode token adds its rank-1 update S += phi(k) v^T and the sum is rounded
back to the format (the order-0 row, a running sum of v, and z are kept
exact), as a decode kernel with a half-size state would do.  Each step's
output is compared with the fp64 recurrence (row-normwise error, the measure
of the parity tests).  The state of the SATA summary page's "Engineering of
constant compute cost" section accumulates phi(k) v over the processed
tokens; this asks whether 16-bit storage keeps the outputs within the 3e-3
gate of bf16 inputs.

Usage:  python -m oracle.state_precision_study [d] [n_prefill] [n_decode] [heads]
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import sata_oracle as O


def _bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


ROUND = {
    "fp32": lambda x: x.astype(np.float32).astype(np.float64),
    "fp16": lambda x: x.astype(np.float16).astype(np.float64),
    "bf16": _bf16,
}


def study(d: int, n0: int, nd: int, heads: int, seed: int = 4242, every: int = 64):
    """Max row-normwise decode error per storage format over `heads` heads."""
    import workloads as W
    P = 4
    basis = O.enumerate_basis(d, P)
    q, k, v = W.make_qkv(1, heads, n0 + nd, d, d, W.BF16, seed)
    worst = {}
    for name, rnd in ROUND.items():
        err = 0.0
        for h in range(heads):
            qh, kh, vh = (x[0, h].astype(np.float64) for x in (q, k, v))
            S64, z64 = O.direct_state(kh[:n0], vh[:n0], basis)
            S, z = rnd(S64), z64.copy()
            fk = O.features_k(kh[n0:], basis)
            for t in range(nd):
                S64 += np.outer(fk[t], vh[n0 + t])
                z64 += fk[t]
                S = rnd(S + np.outer(fk[t], vh[n0 + t]))
                S[0] = S64[0]          # order-0 row: running sum of v, kept exact
                z = z + fk[t]          # z kept exact
                if t % every == every - 1 or t == nd - 1:
                    got = O.state_readout(qh[n0 + t:n0 + t + 1], S, z, basis)
                    ref = O.state_readout(qh[n0 + t:n0 + t + 1], S64, z64, basis)
                    err = max(err, O.row_normwise_error(got, ref))
        worst[name] = err
    return worst


if __name__ == "__main__":
    args = [int(a) for a in sys.argv[1:]] + [16, 4096, 1024, 8][len(sys.argv) - 1:]
    d, n0, nd, heads = args[:4]
    for name, e in study(d, n0, nd, heads).items():
        print(f"d={d} prefill {n0} + decode {nd}, {heads} heads: state {name}: max row-normwise error {e:.2e}")
