"""Helpers shared by the GPU parity tests: moving stored input codes to the
oracle, the error metric, and the split rule of the decode ABI."""
import numpy as np
import torch

import oracle

# Tolerances of the parity bar: max |gpu - ref| / max |ref| per tensor.
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def bits16(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bits8(t):
    return t.contiguous().cpu().view(torch.uint8).numpy()


def f64(t):
    """bf16 tensor -> float64 numpy through the oracle's own decoder."""
    return oracle.bf16_to_f64(bits16(t))


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def cache_args(x):
    """Oracle keyword arguments describing the stored cache of DecodeInputs x."""
    fp8 = x.workload.dtype == "fp8_e4m3"
    conv = bits8 if fp8 else bits16
    return dict(
        kv_codes=conv(x.kv_rows), pe_codes=conv(x.pe_rows),
        dtype="fp8_e4m3" if fp8 else "bf16",
        seq_stride=x.seq_stride if x.block_table is None else None,
        block_table=None if x.block_table is None else x.block_table.cpu().numpy(),
        block_size=x.block_size if x.block_table is not None else None,
        token_scale=None if x.token_scale is None else x.token_scale.cpu().numpy())


def split_bounds(T, max_seq_len, num_splits):
    """Token ranges of the splits as the decode ABI defines them:
    chunk = 32 * ceil(ceil(max_seq_len / P) / 32); split i covers
    [i * chunk, min((i + 1) * chunk, T))."""
    per = -(-max_seq_len // num_splits)
    chunk = 32 * (-(-per // 32))
    edges = [min(i * chunk, T) for i in range(num_splits)] + [T]
    return edges


def sample_batch(B, k=4):
    """A spread of sequence indices for checking large batches."""
    if B <= k:
        return list(range(B))
    return sorted(set([0, B - 1] + list(np.linspace(0, B - 1, k).round().astype(int))))
