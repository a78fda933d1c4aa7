"""Parity of mla_cache_append (through the C ABI) with the oracle's
cache_append_rows on the same seeded rows.

What must agree exactly: the latent half of a bf16 cache (a copy), every
untouched slot, rows at position 0 (rotation by angle 0 is the identity on
both sides, so their E4M3 codes and scales are bit-exact, ties included).
The rotated key goes through fp64 sin/cos, whose last bit may differ between
the device's math library and the host's; that moves the fp32 / bf16
rounding only when the exact value lies within about one fp64 ulp of a
rounding boundary, so rotated keys must agree to one bf16 step (one E4M3
code step) and bit for bit in at least 99.9% of the elements.
"""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, TOL_FP8, bits8, bits16, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SENTINEL16 = 0x5A5A   # bf16 pattern of untouched slots
SENTINEL8 = 0x5A


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _slots(b, positions, seq_stride=None, table=None, block_size=None):
    """Slots of positions (array) of sequence b through the oracle's addressing,
    -1 where the position has no slot."""
    out = np.full(len(positions), -1, dtype=np.int64)
    for k, p in enumerate(positions):
        if p < 0:
            continue
        if table is None:
            if p < seq_stride:
                out[k] = oracle.token_slots(b, p + 1, seq_stride=seq_stride)[p]
        else:
            if p // block_size < table.shape[1] and table[b, p // block_size] >= 0:
                out[k] = oracle.token_slots(b, p + 1, block_table=table, block_size=block_size)[p]
    return out


class Cache:
    """A fused [num_slots, 576] cache (bf16 or E4M3 + scales) filled with a
    sentinel, plus its ABI description."""

    def __init__(self, num_slots, fp8, seq_stride=0, table=None, block_size=0):
        self.fp8 = fp8
        dt = torch.uint8 if fp8 else torch.int16
        fill = SENTINEL8 if fp8 else SENTINEL16
        self.store = torch.full((num_slots, 576), fill, dtype=dt, device=DEV)
        if not fp8:
            self.store = self.store.view(torch.bfloat16)
        self.scale = torch.full((num_slots,), -7.0, dtype=torch.float32, device=DEV) if fp8 else None
        self.table_np = table
        self.table = None if table is None else torch.from_numpy(table.astype(np.int32)).to(DEV)
        self.desc = binding.make_cache(self.store[:, :512], self.store[:, 512:], seq_stride=seq_stride,
                                       block_table=self.table, block_size=block_size, token_scale=self.scale)

    def codes(self):
        return bits8(self.store) if self.fp8 else bits16(self.store)


def _run_append(B, n, positions, fp8, seed, seq_stride=0, table=None, block_size=0, num_slots=None, base=10000.0):
    rows = datagen.random_projection_rows(B, n, seed, device=DEV)
    if num_slots is None:
        num_slots = B * seq_stride if table is None else (int(table.max()) + 1) * block_size
    c = Cache(num_slots, fp8, seq_stride=seq_stride, table=table, block_size=block_size)
    pos_t = torch.tensor(positions, dtype=torch.int32, device=DEV)
    d = binding.dims(B, 128, 0.07)
    binding.mla_cache_append(d, c.desc, rows, pos_t, rope_base=base)
    torch.cuda.synchronize()
    want = oracle.cache_append_rows(bits16(rows), np.asarray(positions), "fp8_e4m3" if fp8 else "bf16",
                                    rope_base=base)
    return rows, c, want


def _check(c, want, positions, seq_stride=0, table=None, block_size=None):
    """Compare every written slot with the oracle and every other slot with the
    sentinel; returns the number of rows written."""
    pos, kv, pe, scale = want
    got = c.codes()
    got_scale = None if scale is None else c.scale.cpu().numpy()
    written = np.zeros(got.shape[0], dtype=bool)
    key_total = key_exact = 0
    for b in range(pos.shape[0]):
        slots = _slots(b, pos[b], seq_stride=seq_stride, table=table, block_size=block_size)
        for j, s in enumerate(slots):
            if s < 0:
                continue
            written[s] = True
            zero_angle = pos[b, j] == 0
            if scale is None:
                assert np.array_equal(got[s, :512], kv[b, j]), (b, j)
                gk = got[s, 512:].astype(np.int32)
                wk = pe[b, j].astype(np.int32)
            else:
                same = got_scale[s] == scale[b, j]
                if zero_angle:
                    assert same, (b, j, got_scale[s], scale[b, j])
                else:
                    assert abs(float(got_scale[s]) / float(scale[b, j]) - 1.0) <= 2.0 ** -20, (b, j)
                if same:  # the same scale: latent quotients and their codes are identical
                    assert np.array_equal(got[s, :512], kv[b, j]), (b, j)
                gk = got[s, 512:].astype(np.int32)
                wk = pe[b, j].astype(np.int32)
            if zero_angle:
                assert np.array_equal(gk, wk), (b, j)
            # one step of the pattern, same sign (E4M3 / bf16 patterns are monotone in |x|)
            assert np.all((np.abs(gk - wk) <= 1) & ((gk ^ wk) & (0x80 if c.fp8 else 0x8000) == 0)), (b, j)
            key_total += gk.size
            key_exact += int(np.sum(gk == wk))
    if key_total:
        assert key_exact / key_total >= 0.999, (key_exact, key_total)
    fill = SENTINEL8 if c.fp8 else SENTINEL16
    assert np.all(got[~written] == fill)
    if got_scale is not None:
        assert np.all(got_scale[~written] == -7.0)
    return int(written.sum())


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_append_contiguous(fp8):
    """Ragged positions (0, mid-sequence, near the end) and 37 new tokens per
    sequence; rows past seq_stride and negative positions are skipped."""
    announce(f"append contiguous fp8={fp8} B=5 n=37")
    B, n, S = 5, 37, 160
    positions = [0, 5, 100, 140, -3]   # 140 + 37 > 160: 17 rows skipped; -3: first 3 rows skipped
    _, c, want = _run_append(B, n, positions, fp8, seed=31, seq_stride=S)
    wrote = _check(c, want, positions, seq_stride=S)
    assert wrote == 37 + 37 + 37 + 20 + 34


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("block_size", [64, 16, 5])
def test_append_paged(fp8, block_size):
    """Permuted block table with unallocated (-1) entries; positions spanning
    several blocks and running past the table."""
    announce(f"append paged fp8={fp8} block_size={block_size}")
    B, n, max_blocks = 3, 70, 6
    rng = np.random.default_rng(block_size)
    table = rng.permutation(B * max_blocks).reshape(B, max_blocks).astype(np.int64)
    table[1, 2] = -1
    positions = [0, block_size - 3, (max_blocks - 1) * block_size - 7]
    _, c, want = _run_append(B, n, positions, fp8, seed=32, table=table, block_size=block_size,
                             num_slots=B * max_blocks * block_size)
    _check(c, want, positions, table=table, block_size=block_size)


def test_append_fp8_ties_and_special_rows():
    """Rows at position 0 (no rotation) built to hit E4M3 rounding ties, signed
    zeros, subnormal codes and an all-zero row: codes and scales must equal the
    oracle's bit for bit."""
    announce("append fp8 ties / zeros / subnormals at position 0")
    grid = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2                     # 126 midpoints, each a tie
    rows = np.zeros((4, 576), dtype=np.float64)
    # row 0: scale exactly 1 (max 448), every midpoint with alternating signs
    rows[0, 0] = 448.0
    rows[0, 1:127] = mids * np.where(np.arange(126) % 2 == 0, 1.0, -1.0)
    rows[0, 127:] = np.resize(-grid[::-1], 576 - 127)
    # row 1: scale 2^-4 (max 28), midpoints scaled by the same power of two
    rows[1, 0] = -28.0
    rows[1, 1:127] = mids / 16.0
    rows[1, 200] = -0.0
    # row 2: all zero (scale = smallest normal fp32), with negative zeros
    rows[2, ::3] = -0.0
    # row 3: tiny values in E4M3's subnormal range after scaling
    rows[3, 0] = 448.0 * 2.0 ** -10
    rows[3, 1:40] = grid[1:40] * 2.0 ** -10
    bits = torch.from_numpy(rows.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.bf16_to_f64(bits.view(torch.int16).numpy().view(np.uint16)),
                          rows.astype(np.float32).astype(np.float64))  # all exact in bf16
    kv_in = bits.view(4, 1, 576).to(DEV)
    c = Cache(4 * 8, True, seq_stride=8)
    pos = torch.zeros(4, dtype=torch.int32, device=DEV)
    binding.mla_cache_append(binding.dims(4, 128, 0.07), c.desc, kv_in, pos)
    torch.cuda.synchronize()
    _, kv, pe, scale = oracle.cache_append_rows(bits16(kv_in), np.zeros(4, dtype=np.int64), "fp8_e4m3")
    got = c.codes()
    sc = c.scale.cpu().numpy()
    for b in range(4):
        assert np.array_equal(got[8 * b, :512], kv[b, 0]), b
        assert np.array_equal(got[8 * b, 512:], pe[b, 0]), b
        assert sc[8 * b] == scale[b, 0], b
    assert sc[16] == np.finfo(np.float32).tiny


def test_append_fp8_every_bf16_pattern():
    """Every finite bfloat16 value in [-448, 448], appended at position 0 in
    rows whose largest magnitude is 448 (scale exactly 1) and 448 * 2^-7
    (scale 2^-7, values scaled down by the same power, the tiniest ones set
    to zero so that every value stays exact): all codes equal the oracle's
    encoder."""
    announce("append fp8 every bf16 pattern")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(pats)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    vals = vals[keep]
    per = 575
    n_rows = -(-len(vals) // per)
    base = np.zeros((n_rows, 576))
    flat = np.zeros(n_rows * per)
    flat[:len(vals)] = vals
    base[:, 1:] = flat.reshape(n_rows, per)
    base[:, 0] = 448.0
    small = np.where(np.abs(base) < 2.0 ** -100, 0.0, base) * 2.0 ** -7  # stays exact in bf16
    rows = np.concatenate([base, small])
    rows_t = torch.from_numpy(rows.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(oracle.bf16_to_f64(bits16(rows_t)), rows)
    B = rows.shape[0]
    kv_in = rows_t.view(B, 1, 576).to(DEV)
    c = Cache(B, True, seq_stride=1)
    binding.mla_cache_append(binding.dims(B, 128, 0.07), c.desc, kv_in, torch.zeros(B, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    _, kv, pe, scale = oracle.cache_append_rows(bits16(kv_in), np.zeros(B, dtype=np.int64), "fp8_e4m3")
    got = c.codes()
    assert np.array_equal(c.scale.cpu().numpy(), scale[:, 0])
    assert np.array_equal(got[:, :512], kv[:, 0])
    assert np.array_equal(got[:, 512:], pe[:, 0])


def test_append_then_decode_against_oracle():
    """Prefill-style append of T tokens, a decode, then a decode-style append
    of one token per sequence at position T and a decode at T + 1: the
    decode outputs match the oracle run on the oracle's own appended cache."""
    announce("append T then decode, append 1 then decode (bf16 and fp8)")
    B, H, T, S = 3, 128, 300, 320
    for fp8 in (False, True):
        rows = datagen.random_projection_rows(B, T + 1, 41, device=DEV)
        c = Cache(B * S, fp8, seq_stride=S)
        d = binding.dims(B, H, 192 ** -0.5)
        zero = torch.zeros(B, dtype=torch.int32, device=DEV)
        binding.mla_cache_append(d, c.desc, rows[:, :T].contiguous(), zero)
        dt = "fp8_e4m3" if fp8 else "bf16"
        _, kv, pe, scale = oracle.cache_append_rows(bits16(rows), np.zeros(B, dtype=np.int64), dt)
        q_lat = datagen.random_latent_queries(B, H, seed=42, device=DEV)
        q_pe = datagen.random_latent_queries(B, H, seed=43, device=DEV)[..., :64].contiguous()
        kv_codes = kv.reshape(B * (T + 1), 512)
        pe_codes = pe.reshape(B * (T + 1), 64)
        sc = None if scale is None else scale.reshape(-1)
        for L in (T, T + 1):
            if L == T + 1:
                binding.mla_cache_append(d, c.desc, rows[:, T:T + 1].contiguous(), torch.full((B,), T, dtype=torch.int32,
                                                                                 device=DEV))
            lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
            o_lat, lse = binding.mla_decode_latent(d, c.desc, q_lat, q_pe, lens, L, 1)
            torch.cuda.synchronize()
            ro, rl = oracle.latent_decode(f64(q_lat), f64(q_pe), kv_codes, pe_codes, [L] * B, 192 ** -0.5,
                                          dtype=dt, seq_stride=T + 1, token_scale=sc)
            tol = TOL_FP8 if fp8 else TOL_BF16
            assert rel_err(f64(o_lat), ro) <= tol, (fp8, L)
            assert np.max(np.abs(lse.cpu().numpy() - rl)) <= tol, (fp8, L)


@pytest.mark.parametrize("fp8,B,T", [(False, 32, 4096), (True, 64, 32768)], ids=["bf16_b32_s4096", "fp8_b64_s32768"])
def test_append_full_size_sampled(fp8, B, T):
    """Whole-history appends at the decode workloads' sizes (one call writes
    every token), checked on sampled tokens against the oracle."""
    announce(f"append full size fp8={fp8} B={B} T={T}")
    rows = datagen.random_projection_rows(B, T, 51, device=DEV)
    c = Cache(B * T, fp8, seq_stride=T)
    binding.mla_cache_append(binding.dims(B, 128, 0.07), c.desc, rows, torch.zeros(B, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    bs = sorted(set([0, B - 1] + list(rng.integers(0, B, 4))))
    ts = sorted(set([0, 1, 31, 32, T - 1] + list(rng.integers(0, T, 60))))
    tsel = torch.tensor(ts, device=DEV)
    for b in bs:
        sub = rows[b:b + 1, tsel].contiguous()
        # oracle rows at their true positions: one call per sampled token
        got_rows = c.store[b * T + tsel]
        got = bits8(got_rows) if fp8 else bits16(got_rows)
        for k, t in enumerate(ts):
            _, kv, pe, scale = oracle.cache_append_rows(bits16(sub[:, k:k + 1]), np.array([t]),
                                                        "fp8_e4m3" if fp8 else "bf16")
            gk, wk = got[k, 512:].astype(np.int32), pe[0, 0].astype(np.int32)
            assert np.all(np.abs(gk - wk) <= 1), (b, t)
            if fp8:
                s = float(c.scale[b * T + t])
                assert abs(s / float(scale[0, 0]) - 1.0) <= 2.0 ** -20, (b, t)
                if s == scale[0, 0]:
                    assert np.array_equal(got[k, :512], kv[0, 0]), (b, t)
            else:
                assert np.array_equal(got[k, :512], kv[0, 0]), (b, t)
