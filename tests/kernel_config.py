"""Host-side mirror of the long-K MFMA kernel's launch search (the LDS budget
loop of qgemv_persist_x.hip's launcher), used by the tests to predict which
M values of a shape share one kernel configuration.  Row invariance across M
is promised bit for bit only within a configuration; the GPU test
`test_long_k_row_invariance_by_configuration` checks this mirror against the
library (rows agree bitwise exactly where the mirror says the configuration
is the same), and `test_kernel_config.py` pins the thresholds stated in the
library header."""

LDS_MAX = 160 * 1024
MAX_WAVES = 12
MAX_PHASES = 2
PERSIST_WAVES = {(4, 32): (16, 2), (4, 64): (16, 1), (4, 128): (12, 1), (2, 64): (12, 2), (2, 128): (12, 1)}


def register_persistent_fits(K: int, bits: int, gs: int) -> bool:
    """The register-resident persistent kernel's reach: waves * blocks per
    wave bias blocks of 4 groups."""
    maxw, bpw = PERSIST_WAVES[(bits, gs)]
    return K // (4 * gs) <= maxw * bpw


def long_k_config(M: int, N: int, K: int, bits: int, gs: int, cus: int):
    """(phases, blocks per wave, waves) of the long-K kernel, or None when it
    does not run (fewer tiles than CUs, or no configuration fits the LDS)."""
    bsc = 4 * gs // (512 // bits)
    small = 1 if bsc >= 2 else 2
    narrow = 1 if bsc >= 4 else 4 // bsc
    wide = 2 if bsc == 4 else narrow
    nblk = K // (4 * gs)
    if nblk < 2:
        return None
    nbp_min, nbp_max = nblk // 2, nblk - nblk // 2
    tiles = (N + 15) // 16
    if tiles < cus:
        return None
    grid = 2 * (cus // 2)
    ntile_max = (tiles + grid // 2 - 1) // (grid // 2)
    for phases in range(1, min(MAX_PHASES, nbp_min) + 1):
        nbq_max = (nbp_max + phases - 1) // phases
        for variant, bpw in enumerate((small, narrow, wide)):
            if phases > 1 and variant == 2 and wide != narrow:
                continue
            waves = (nbq_max + bpw - 1) // bpw
            if waves > MAX_WAVES:
                continue
            pitch = nbq_max * 4 * gs * 2 + 16
            lds = M * pitch + M * nbq_max * 4 * 4 + ntile_max * waves * 256 * 4
            if lds > LDS_MAX:
                continue
            return (phases, bpw, waves)
    return None


def mfma_configuration(M: int, N: int, K: int, bits: int, gs: int, cus: int):
    """Which MFMA kernel configuration an affine call runs, for shapes whose
    kernel choice can depend on M (more tiles than CUs, K beyond the
    register-resident persistent kernel): ("long_k", phases, bpw, waves) or
    ("single_pass",)."""
    tiles = (N + 15) // 16
    if K % (4 * gs) != 0:  # a partial last bias block: the single-pass kernel only
        return ("single_pass",)
    if tiles > cus and not register_persistent_fits(K, bits, gs):
        c = long_k_config(M, N, K, bits, gs, cus)
        if c is not None:
            return ("long_k",) + c
    return ("single_pass",)
