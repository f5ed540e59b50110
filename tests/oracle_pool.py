"""Runs the oracle's encoder over large fp32 bit-pattern ranges in worker
processes (spawned, numpy only), for the exhaustive encoder comparison."""
import numpy as np


def encode_range(args):
    lo, hi = args
    import oracle
    bits = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32)
    return oracle.e4m3_encode(bits.view(np.float32))
