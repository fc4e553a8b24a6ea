"""Write the stored HiPPO-LegS DPLR initialization tables under synth/data.

Calls only the fp64 oracle (``oracle.dplr_legs``).  Run from the repository
root:  python -m synth.write_init_tables
"""
from __future__ import annotations

import os

import numpy as np

from oracle import dplr_legs

_DATA = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")


def write(N: int) -> str:
    lam, P, B, _ = dplr_legs(N)
    rows = np.stack([lam.real, lam.imag, P.real, P.imag, B.real, B.imag], axis=1)
    path = os.path.join(_DATA, f"hippo_legs_dplr_N{N}.txt")
    header = (f"HiPPO-LegS DPLR initialization, N={N} poles, written by "
              f"synth/write_init_tables.py from oracle.dplr_legs (fp64).\n"
              "columns: Re(Lambda) Im(Lambda) Re(P) Im(P) Re(B) Im(B)")
    np.savetxt(path, rows, fmt="%.17e", header=header)
    return path


if __name__ == "__main__":
    os.makedirs(_DATA, exist_ok=True)
    for n in (16, 64):
        print(write(n))
