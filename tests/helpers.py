"""Shared helpers of the test suite (no method arithmetic lives here)."""
import numpy as np

REL_L2_TOL = 2e-3      # relative L2 error bound on the fp32 outputs
ELEM_TOL = 1e-2        # per-element bound, in units of rms(out)


def moe_close(got, ref, rel_l2=REL_L2_TOL, elem=ELEM_TOL):
    """The parity bar for fp32 outputs: ||got-ref|| <= rel_l2 ||ref|| and
    max |got-ref| <= elem * rms(ref).  Returns (rel_l2_err, max_err/rms)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = got - ref
    nref = np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    r = np.linalg.norm(err) / max(nref, 1e-300)
    e = np.max(np.abs(err)) / max(rms, 1e-300) if err.size else 0.0
    assert r <= rel_l2, f"relative L2 error {r:.3e} > {rel_l2}"
    assert e <= elem, f"max element error {e:.3e} rms > {elem}"
    return r, e


def public_header_symbols(path, prefix="moe_ffn_"):
    import re
    txt = open(path).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(" + prefix + r"\w+)\s*\(", txt, re.M)))
