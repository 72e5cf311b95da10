"""Parity gates between a device result and the fp64 oracle.

bf16 path: max |o - o*| <= 2e-2 and mean |o - o*| <= 2e-3 over every element
(the stated tolerance for bf16 inputs with fp32 accumulation), plus a relative
Frobenius gate ||o - o*|| / ||o*|| <= 1e-2 so that an all-zero or mean-pooled
output cannot pass on small-magnitude outputs.  fp32 path: max-abs <= 1e-4.
LSE (natural log) is checked to 2e-2 absolute on bf16 and 1e-4 on fp32.
"""
import numpy as np

BF16_GATES = {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_fro": 1e-2}
F32_GATES = {"max_abs": 1e-4, "mean_abs": 1e-5, "rel_fro": 1e-4}


def gates_for(dtype):
    return BF16_GATES if dtype == "bf16" else F32_GATES


def error_stats(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = out - ref
    return {
        "max_abs": float(np.abs(d).max()) if d.size else 0.0,
        "mean_abs": float(np.abs(d).mean()) if d.size else 0.0,
        "rel_fro": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0,
        "finite": bool(np.isfinite(out).all()),
    }


def passes(stats, gates):
    return stats["finite"] and all(stats[k] <= gates[k] for k in gates)


def assert_gates(out, ref, dtype, what=""):
    st = error_stats(out, ref)
    g = gates_for(dtype)
    assert passes(st, g), f"{what}: {st} vs gates {g}"
    return st
