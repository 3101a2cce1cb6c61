"""Helpers shared by the GPU parity tests: device upload of seeded inputs,
the tolerance checks and the top-K comparison rule.  Nothing here computes
attention; expected values come from the fp64 oracle."""
import functools
import math
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import vsa_oracle as vo

# Parity bars.  fp32 path: max abs 1e-4.  bf16 inputs with fp32
# accumulation: max abs 2e-2 and relative RMS 4e-3 over the whole tensor.
F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 4e-3
# Near-tie exemption for top-K rows, read on probabilities: the K-th and
# (K+1)-th coarse probabilities within a factor (1 - 1e-3), i.e. logits
# within -ln(1 - 1e-3).
TIE_LOGIT_GAP = -math.log1p(-1e-3)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    """fp32 numpy (bf16-exact when dtype is bf16) -> contiguous GPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).cuda().contiguous()


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(actual, expected, dtype, what=""):
    actual = np.asarray(actual, dtype=np.float64)
    expected = np.asarray(expected, dtype=np.float64)
    assert actual.shape == expected.shape, (what, actual.shape, expected.shape)
    assert np.all(np.isfinite(actual)), f"{what}: non-finite values"
    err = np.abs(actual - expected)
    max_abs = float(err.max()) if err.size else 0.0
    if dtype == torch.float32:
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {F32_MAX_ABS}"
        return max_abs, None
    denom = float(np.linalg.norm(expected))
    rel = float(np.linalg.norm(actual - expected)) / denom if denom > 0 else float(np.linalg.norm(actual))
    assert max_abs <= BF16_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_RMS, f"{what}: rel RMS {rel:.3e} > {BF16_REL_RMS}"
    return max_abs, rel


def check_selection_row(sel_row, logits_row, K):
    """GPU top-K ids of one query cube against the fp64 logits.

    Returns True when the row equals the exact top-K (logit desc, index asc),
    False when it differs only at a near-tie (every differing cube within
    TIE_LOGIT_GAP of the K-th logit); raises otherwise.  The ids must be K
    distinct, ascending values in range.
    """
    sel_row = np.asarray(sel_row, dtype=np.int64)
    nc = logits_row.shape[0]
    assert sel_row.shape == (K,)
    assert np.all(np.diff(sel_row) > 0), f"ids not strictly ascending: {sel_row}"
    assert sel_row.min() >= 0 and sel_row.max() < nc
    order = np.lexsort((np.arange(nc), -logits_row))
    ref = np.sort(order[:K])
    if np.array_equal(ref, sel_row):
        return True
    kth = logits_row[order[K - 1]]
    diff = np.setxor1d(ref, sel_row)
    bad = diff[np.abs(logits_row[diff] - kth) > TIE_LOGIT_GAP]
    assert bad.size == 0, f"selection differs beyond near-ties: ids {bad}, gaps {logits_row[bad] - kth}"
    return False


def check_selection(sel, S, K):
    """All rows; returns the number of exempted near-tie rows."""
    sel = np.asarray(sel)
    exempt = 0
    for idx in np.ndindex(sel.shape[:-1]):
        if not check_selection_row(sel[idx], S[idx], K):
            exempt += 1
    return exempt


# Band for the stand-in mass rule: a GPU list may be one longer or shorter
# than the exact rule's only where the ranked prefix's probability mass
# crosses `mass` within this distance of it.  The GPU sums fp32
# probabilities whose logits carry up to about 1e-5 absolute error (bf16 x 3
# products), so its prefix masses are within a few 1e-5 of exact ones.
MASS_BAND = 1e-4


def check_mass_row(ids_row, logits_row, mass, k_min, k_max):
    """GPU list of the mass rule for one query cube against fp64 logits.

    The length must equal the oracle's, or differ by one where the mass of
    the shorter prefix lies within MASS_BAND of `mass`; the ids must then be
    the top-length cubes of the ranking (near-tie rule of
    check_selection_row).  Returns True when the length is exact."""
    ids_row = np.asarray(ids_row, dtype=np.int64)
    lists, lengths = vo.select_mass(logits_row[None], mass, k_min, k_max)
    n_ref, n = int(lengths[0]), len(ids_row)
    exact = n == n_ref
    if not exact:
        assert abs(n - n_ref) == 1, f"length {n}, oracle {n_ref}"
        p = np.exp(logits_row - logits_row.max())
        p /= p.sum()
        order = np.lexsort((np.arange(len(logits_row)), -logits_row))
        crossing = np.cumsum(p[order])[min(n, n_ref) - 1]
        assert abs(crossing - mass) <= MASS_BAND, (
            f"length {n} vs oracle {n_ref} with prefix mass {crossing:.6f}, mass {mass}")
    check_selection_row(ids_row, logits_row, n)
    return exact


# ------------------------------------------------ whole-tensor comparisons
def oracle_workers():
    """Threads for per-head oracle runs: the host cores this process may use
    (at most 16, the share of one GPU's host on the test boxes)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def per_head(fn, pairs):
    """fn(b, h) for every (b, h) in pairs, in a thread pool with BLAS held to
    one thread per worker (numpy releases the GIL in its kernels).  Results
    in the order of pairs."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(oracle_workers()) as ex:
        return list(ex.map(lambda bh: fn(*bh), pairs))


class Stats:
    """Whole-tensor error statistics accumulated slice by slice: max abs
    error, and the squared norms that give the relative RMS error
    ||actual - expected|| / ||expected|| over the whole tensor."""

    def __init__(self):
        self.max_abs = 0.0
        self.err2 = 0.0
        self.ref2 = 0.0
        self.count = 0

    @staticmethod
    def of(actual, expected):
        st = Stats()
        actual = np.asarray(actual, dtype=np.float64)
        expected = np.asarray(expected, dtype=np.float64)
        assert actual.shape == expected.shape, (actual.shape, expected.shape)
        if not np.all(np.isfinite(actual)):
            st.max_abs = math.inf
        else:
            d = actual - expected
            st.max_abs = float(np.abs(d).max()) if d.size else 0.0
            st.err2 = float(np.sum(d * d))
        st.ref2 = float(np.sum(expected * expected))
        st.count = actual.size
        return st

    def add(self, other):
        self.max_abs = max(self.max_abs, other.max_abs)
        self.err2 += other.err2
        self.ref2 += other.ref2
        self.count += other.count
        return self

    @property
    def rel_rms(self):
        return math.sqrt(self.err2 / self.ref2) if self.ref2 > 0 else math.sqrt(self.err2)

    def check(self, dtype, what):
        """The parity bar over the whole tensor (fp32: max abs; bf16 inputs:
        max abs and relative RMS)."""
        assert math.isfinite(self.max_abs), f"{what}: non-finite values"
        if dtype == torch.float32:
            assert self.max_abs <= F32_MAX_ABS, f"{what}: max abs {self.max_abs:.3e} > {F32_MAX_ABS}"
        else:
            assert self.max_abs <= BF16_MAX_ABS, f"{what}: max abs {self.max_abs:.3e} > {BF16_MAX_ABS}"
            assert self.rel_rms <= BF16_REL_RMS, f"{what}: rel RMS {self.rel_rms:.3e} > {BF16_REL_RMS}"
        return f"{what}: {self.count} values, max abs {self.max_abs:.3e}, rel RMS {self.rel_rms:.3e}"


def sum_stats(items):
    total = Stats()
    for st in items:
        total.add(st)
    return total


@functools.lru_cache(maxsize=2)
def cached_inputs(name, with_varlen):
    """Seeded inputs of a named workload, kept for the next test on the same
    workload (drawing the largest ones takes most of a test's time)."""
    from workloads import WORKLOADS, workload_inputs
    return workload_inputs(WORKLOADS[name], with_varlen=with_varlen)
