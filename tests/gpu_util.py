"""Helpers for the GPU tests: move seeded problems to the device and run the
library through its C ABI."""
import sys

import numpy as np

from few_row_quantized_amd import qgemv as q


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceProblem:
    def __init__(self, p, device="cuda:0"):
        import torch
        self.p = p
        self.codes = torch.from_numpy(p.codes).to(device)
        self.scales = torch.from_numpy(p.scales.view(np.int16)).to(device)
        self.biases = torch.from_numpy(p.biases.view(np.int16)).to(device)
        self.x = torch.from_numpy(p.x.view(np.int16)).to(device)
        self.device = device

    def run(self, M: int, path="auto", y=None):
        import torch
        p = self.p
        if y is None:
            y = torch.full((M, p.N), float("nan"), dtype=torch.float32, device=self.device)
        q.qgemv_run_path(path, self.codes, self.scales, self.biases, self.x, y, M, p.N, p.K,
                         p.bits, p.group_size)
        torch.cuda.synchronize()
        return y

    def run_host(self, M: int, path="auto") -> np.ndarray:
        return self.run(M, path).cpu().numpy()


class OracleRows:
    """The fp64 oracle's y and sum|x*w| for the first rows of a problem,
    computed once; rows of the oracle do not depend on how many are asked
    for (a pinned invariant), so an M-row call is checked against the first M
    rows (for the gathered product: the first pairs)."""

    def __init__(self, ref: np.ndarray, absum: np.ndarray, cols=None):
        self.ref, self.absum, self.cols = ref, absum, cols

    @classmethod
    def affine(cls, p, m_max: int, cols=None):
        import oracle
        ref = oracle.qgemv_reference(p.codes, p.scales, p.biases, p.x, m_max, p.N, p.K, p.bits,
                                     p.group_size, rows=cols)
        absum = oracle.abs_product_sum(p.codes, p.scales, p.biases, p.x, m_max, p.N, p.K, p.bits,
                                       p.group_size, rows=cols)
        return cls(ref, absum, cols)

    @classmethod
    def fp(cls, p, m_max: int, cols=None):
        import oracle
        fmt = p.shape.fmt
        ref = oracle.qgemv_fp_reference(p.codes, p.scales, p.x, m_max, p.N, p.K, fmt, rows=cols)
        absum = oracle.fp_abs_product_sum(p.codes, p.scales, p.x, m_max, p.N, p.K, fmt, rows=cols)
        return cls(ref, absum, cols)

    @classmethod
    def gather(cls, p, x_idx, e_idx, cols=None):
        import oracle
        s = p.shape
        ref = oracle.qgemv_gather_reference(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N, s.K,
                                            s.bits, s.group_size, rows=cols)
        absum = oracle.gather_abs_product_sum(p.codes, p.scales, p.biases, p.x, x_idx, e_idx, s.N,
                                              s.K, s.bits, s.group_size, rows=cols)
        return cls(ref, absum, cols)

    def check(self, y: np.ndarray, M: int, label: str = "", residual=None) -> float:
        """Every element (of the selected columns) of the first M rows within
        the tolerance; with a residual r, within the fused sum's bar
        1e-3*S + 1e-6 + 2^-23*(|r| + S).  Returns the worst |dy|/tol."""
        import oracle
        yy = y if self.cols is None else y[:, self.cols]
        ref, absum = self.ref[:M], self.absum[:M]
        if residual is None:
            ok, worst, idx = oracle.check_close(yy, ref, absum)
        else:
            r = residual[:M] if self.cols is None else residual[:M][:, self.cols]
            ok, worst, idx = oracle.check_close(yy, ref + r.astype(np.float64), absum, residual_abs=r)
        assert ok, f"{label}: worst |dy|/tol = {worst:.3g} at {idx}"
        return worst
