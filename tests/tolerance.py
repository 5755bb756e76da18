"""Floating-point agreement bar for attention outputs.

Both must hold for every query on its own (its [heads, d_v] output block): max |gpu - ref| <=
2e-2 and the normwise relative error ||gpu - ref||_F / ||ref||_F <= 1e-2. The normwise bound is
the discriminating one: decode outputs have an element spread near 2e-3, so an all-zero output
would meet the max-abs bound alone, while one wrong index out of 2048 moves one query's
normwise error by about 3%. Pooled over 32 queries the same mistake would move it by about
0.55% and pass, so the bar is never applied to a stack of queries.
"""
import numpy as np

MAX_ABS = 2e-2
REL_FRO = 1e-2


def attn_errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def attn_close(got, ref, max_abs=MAX_ABS, rel_fro=REL_FRO):
    a, r = attn_errors(got, ref)
    return a <= max_abs and r <= rel_fro, a, r
