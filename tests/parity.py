"""Comparison helpers shared by the GPU parity tests.

bf16 outputs: per row, max |Yg - Yo| <= 1e-2 * max |Yo| (a zero oracle row
must come back exactly zero), and ||Yg - Yo||_F / ||Yo||_F <= 2e-3, in fp64.
Integer tensors (codes, partials) and fp32 scales are compared bit-exactly.
"""
import numpy as np
import torch

from block_quantized_int8_amd.workloads import bf16_bits_to_f32

ROW_TOL = 1e-2
FRO_TOL = 2e-3


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_close(y_gpu_bits: np.ndarray, y_oracle_bits: np.ndarray, what=""):
    g = bf16_bits_to_f32(y_gpu_bits).astype(np.float64)
    o = bf16_bits_to_f32(y_oracle_bits).astype(np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    rowmax = np.abs(o).max(axis=1)
    err = np.abs(g - o).max(axis=1)
    zero = rowmax == 0
    assert np.all(err[zero] == 0), f"{what}: nonzero output in an all-zero oracle row"
    bad = np.nonzero(err > ROW_TOL * rowmax)[0]
    assert bad.size == 0, f"{what}: row tolerance violated in rows {bad[:8]} " \
                          f"(err {err[bad[:4]]}, rowmax {rowmax[bad[:4]]})"
    den = np.linalg.norm(o)
    rel = np.linalg.norm(g - o) / den if den > 0 else np.linalg.norm(g)
    assert rel <= FRO_TOL, f"{what}: relative Frobenius error {rel:.3e} > {FRO_TOL}"
    return rel
