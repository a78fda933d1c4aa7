"""Helpers shared by the GPU parity tests: moving stored input codes to the
oracle, the error metric, and the split rule of the decode ABI."""
import numpy as np
import torch

import oracle

# Tolerances of the parity bar: max |gpu - ref| / max |ref| per tensor, for a
# bf16 cache and for an E4M3 cache.
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def tol_for(x):
    """The parity bar of DecodeInputs x's cache format."""
    return TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16


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


# ---------------------------------------------------------------------------
# Guarded outputs: every output buffer handed to the library sits between two
# guard regions, and the buffer and the guards start filled with a 16-bit
# pattern that is a NaN both as bf16 (0xFFC1) and as fp32 (0xFFC1FFC1).  After
# the call, the guards must still hold the pattern (nothing was written outside
# the output), and an output element the kernels failed to write stays NaN,
# which fails every comparison.
# ---------------------------------------------------------------------------
GUARD_BYTES = 64 * 1024
_PATTERN16 = -63  # int16 view of 0xFFC1


def mismatch_report(a, c, names=None):
    """Where two equally shaped tensors differ bit for bit: the count, the
    first differing indices (named by `names`), NaN counts and the largest
    difference -- printed by bitwise tests before they fail."""
    a_bits = a.contiguous().view(-1).view(torch.int16 if a.element_size() == 2 else torch.int32)
    c_bits = c.contiguous().view(-1).view(torch.int16 if c.element_size() == 2 else torch.int32)
    diff = (a_bits != c_bits).nonzero().view(-1).cpu()
    if diff.numel() == 0:
        return "bit-identical"
    idx = [np.unravel_index(int(i), tuple(a.shape)) for i in diff[:8]]
    fa, fc = a.float(), c.float()
    both = torch.isfinite(fa) & torch.isfinite(fc)
    md = float((fa - fc)[both].abs().max()) if bool(both.any()) else float("nan")
    head = ", ".join(names) if names else "index"
    return (f"{diff.numel()} of {a.numel()} differ; first ({head}): {[tuple(int(v) for v in i) for i in idx]}; "
            f"NaN {int(torch.isnan(fa).sum())} / {int(torch.isnan(fc).sum())}; max |diff| {md:.3g}")


class Guarded:
    def __init__(self, shape, dtype, device):
        elem = torch.empty((), dtype=dtype).element_size()
        self.nbytes = int(np.prod(shape)) * elem
        total = GUARD_BYTES + self.nbytes + GUARD_BYTES
        self.buf = torch.full((total // 2,), _PATTERN16, dtype=torch.int16, device=device)
        raw = self.buf.view(torch.uint8)
        self.tensor = raw[GUARD_BYTES:GUARD_BYTES + self.nbytes].view(dtype).view(shape)
        self.shape = tuple(shape)

    def guards_intact(self):
        raw = self.buf.view(torch.uint8)
        head = raw[:GUARD_BYTES].view(torch.int16)
        tail = raw[GUARD_BYTES + self.nbytes:].view(torch.int16)
        return bool((head == _PATTERN16).all().item()) and bool((tail == _PATTERN16).all().item())


def guarded(device, *specs):
    """Guarded buffers for (shape, dtype) specs; returns the list of Guarded."""
    return [Guarded(shape, dtype, device) for shape, dtype in specs]


def assert_guards(*gs):
    for i, g in enumerate(gs):
        assert g.guards_intact(), f"write outside output {i} of shape {g.shape}"


def oracle_prefill_rows(x, q_lat, q_pe, q_start, max_len, rows):
    """Oracle o_lat / lse of prefill query rows (b, i): latent attention of
    query i of sequence b over its causal prefix, tokens 0 .. q_start[b] + i
    (clamped to max_len)."""
    args = cache_args(x)
    ql, qp = f64(q_lat), f64(q_pe)
    os_, ls_ = [], []
    for b, i in rows:
        T = min(int(q_start[b]) + i + 1, max_len)
        slots = oracle.token_slots(b, T, args["seq_stride"], args["block_table"], args["block_size"])
        c, k_r = oracle.load_rows(args["kv_codes"], args["pe_codes"], slots, args["dtype"], args["token_scale"])
        o, l = oracle.latent_attention(ql[b, i], qp[b, i], c, k_r, x.scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)
