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


def sample_columns(N: int, count: int, seed: int = 0) -> np.ndarray:
    """Spread of output columns for sampled checks: both ends, every tile
    edge near them, and random columns."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 15, 16, 17, 31, N // 2, N - 17, N - 16, N - 2, N - 1}
    fixed = {c for c in fixed if 0 <= c < N}
    rest = rng.choice(N, size=min(count, N), replace=False)
    return np.array(sorted(fixed | set(int(c) for c in rest)))
