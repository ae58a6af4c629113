"""Helpers for the GPU parity tests: device transfer and oracle comparison."""

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_ids_equal(got: np.ndarray, exp: np.ndarray, what: str):
    if not np.array_equal(got, exp):
        bad = np.argwhere(got != exp)
        r, c = bad[0]
        raise AssertionError(
            f"{what}: {len(bad)} mismatches, first at row {r} col {c}: got {got[r, c]} "
            f"expected {exp[r, c]}; row got {got[r, max(0, c - 3):c + 4].tolist()} "
            f"expected {exp[r, max(0, c - 3):c + 4].tolist()}")
