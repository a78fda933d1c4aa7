"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/mla_absorb.h declares, and its host-side checks reject bad
arguments (naming the field) before anything is launched.  No call here
reaches a kernel launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mla_absorbed_latent_absorb_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_absorb.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libmla_absorb.so is not built: run __graft_entry__.build()")
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def _prototypes():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return re.findall(r"^(?:mla_status|int32_t|const char \*)\s*(mla_[a-z_0-9]+)\s*\(", text, flags=re.M)


def test_header_compiles_cleanly_as_c_and_cpp(tmp_path):
    """The public header is valid C and C++ under -Wall -Wextra -Werror
    (no stray comment openers, no duplicate or conflicting prototypes)."""
    import shutil
    import subprocess
    for compiler, lang in (("gcc", "c"), ("g++", "c++")):
        if shutil.which(compiler) is None:
            pytest.skip(f"{compiler} not available")
        src = tmp_path / f"use_header.{'c' if lang == 'c' else 'cpp'}"
        src.write_text('#include "mla_absorb.h"\nint main(void) { return (int)MLA_OK; }\n')
        res = subprocess.run([compiler, "-Wall", "-Wextra", "-Werror", "-Wcomment", "-I", os.path.dirname(HEADER),
                              "-x", lang, "-fsyntax-only", str(src)], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr


def test_each_prototype_declared_once():
    protos = _prototypes()
    assert len(protos) == len(set(protos)), sorted(p for p in protos if protos.count(p) > 1)
    assert set(protos) == set(declared_functions())


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTED)


def test_cache_byte_helpers_match_oracle(lib):
    d = binding.dims(32, 128, 0.07)
    assert binding.mla_kv_cache_bytes(d) == oracle.latent_cache_bytes_per_token(512, 64, 2) == 1152
    assert binding.mla_kv_cache_bytes(d, binding.MLA_DTYPE_FP8_E4M3) == oracle.latent_cache_bytes_per_token(512, 64, 1) + 4
    assert binding.mla_decode_kv_read_bytes(d, [4096] * 32) == oracle.decode_kv_read_bytes(32, 4096, 512, 64, 2)
    d1 = binding.dims(1, 16, 0.07)
    assert binding.mla_decode_kv_read_bytes(d1, [26]) == 29952  # 26-token V2-Lite active cache
    lens = np.random.default_rng(0).integers(1024, 16385, 128)
    d4 = binding.dims(128, 128, 0.07)
    assert binding.mla_decode_kv_read_bytes(d4, lens) == int(lens.sum()) * 1152


@pytest.mark.parametrize("field", ["kv_lora_rank", "qk_rope_head_dim"])
def test_missing_required_dim_names_the_field(lib, field):
    kw = {field: 0}
    d = binding.dims(4, 16, 0.07, **kw)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_kv_cache_bytes(d)
    assert e.value.status == 2 and field in e.value.message


def _call_absorb(lib, d, a=16, b=16, c=16):
    return lib.mla_absorb_q(ctypes.byref(d), ctypes.c_void_p(a), ctypes.c_void_p(b), ctypes.c_void_p(c), None)


def test_validation_rejects_before_launch(lib):
    good = binding.dims(4, 16, 0.07)
    cases = [
        (binding.dims(0, 16, 0.07), 2, "batch"),
        (binding.dims(4, 0, 0.07), 2, "num_heads"),
        (binding.dims(4, 16, 0.0), 2, "softmax_scale"),
        (binding.dims(4, 16, -1.0), 3, "softmax_scale"),
        (binding.dims(4, 16, 0.07, kv_lora_rank=256), 3, "kv_lora_rank"),
        (binding.dims(4, 16, 0.07, qk_rope_head_dim=32), 3, "qk_rope_head_dim"),
        (binding.dims(4, 24, 0.07), 3, "num_heads"),
        (binding.dims(4, 16, 0.07, v_head_dim=0), 2, "v_head_dim"),
    ]
    for d, status, word in cases:
        st = _call_absorb(lib, d)
        assert st == status, (word, st)
        assert word in lib.mla_last_error().decode()
    assert _call_absorb(lib, good, a=0) == 1 and "q_nope" in lib.mla_last_error().decode()
    assert _call_absorb(lib, good, b=8) == 6 and "w_uk" in lib.mla_last_error().decode()


def _decode(lib, d, cache, max_len=64, splits=1, o_part=0, lse_part=0, o_lat=64, lse=64, q=16, qpe=16, lens=16):
    P = ctypes.c_void_p
    return lib.mla_decode_latent(ctypes.byref(d), ctypes.byref(cache) if cache is not None else None, P(q), P(qpe),
                                 P(lens), max_len, splits, P(o_part) if o_part else None,
                                 P(lse_part) if lse_part else None, P(o_lat) if o_lat else None,
                                 P(lse) if lse else None, None)


def test_decode_latent_validation(lib):
    d = binding.dims(2, 16, 0.07)
    base = dict(dtype=0, kv=1024, pe=2048, kv_stride=576, pe_stride=576, token_scale=None, seq_stride=64,
                block_table=None, block_size=0, max_blocks_per_seq=0)

    def cache(**kw):
        c = dict(base)
        c.update(kw)
        return binding.MlaCache(**c)

    assert _decode(lib, d, None) == 1
    # E4M3 cache: needs the per-slot scales and 16-byte row strides; bf16 takes no scales
    assert _decode(lib, d, cache(dtype=1)) == 1 and "token_scale" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(dtype=1, token_scale=4098)) == 6 and "token_scale" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(dtype=1, token_scale=4096, kv_stride=520)) == 5
    assert _decode(lib, d, cache(token_scale=4096)) == 5 and "token_scale" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(dtype=2)) == 3 and "dtype" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(kv=None)) == 1
    assert _decode(lib, d, cache(kv=1032)) == 6
    assert _decode(lib, d, cache(kv_stride=500)) == 5 and "kv_stride" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(pe_stride=60)) == 5
    assert _decode(lib, d, cache(seq_stride=32), max_len=64) == 5 and "seq_stride" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(), max_len=0) == 4
    assert _decode(lib, d, cache(), splits=0) == 4
    assert _decode(lib, d, cache(block_table=4096, block_size=48, max_blocks_per_seq=4)) == 4
    assert _decode(lib, d, cache(block_table=4096, block_size=64, max_blocks_per_seq=0)) == 5
    # split outputs must match num_splits
    assert _decode(lib, d, cache(), splits=2) == 1 and "o_part" in lib.mla_last_error().decode()
    assert _decode(lib, d, cache(), splits=2, o_part=4096, lse_part=4096) == 5  # o_lat given with P > 1
    assert _decode(lib, d, cache(), splits=1, o_part=4096) == 5
    assert _decode(lib, d, cache(), lens=0) == 1 and "seq_lens" in lib.mla_last_error().decode()


def test_combine_and_expand_validation(lib):
    d = binding.dims(2, 16, 0.07)
    P = ctypes.c_void_p
    assert lib.mla_combine_splits(ctypes.byref(d), P(16), P(16), 0, P(16), P(16), None) == 4
    assert lib.mla_combine_splits(ctypes.byref(d), None, P(16), 2, P(16), P(16), None) == 1
    assert lib.mla_expand_v(ctypes.byref(d), P(16), None, P(16), None) == 1
    assert "w_uv" in lib.mla_last_error().decode()
    ce = lib.mla_combine_expand_v
    assert ce(ctypes.byref(d), P(16), P(16), 0, P(16), P(16), None, None, None) == 4
    assert ce(ctypes.byref(d), None, P(16), 2, P(16), P(16), None, None, None) == 1
    assert ce(ctypes.byref(d), P(16), None, 2, P(16), P(16), None, None, None) == 1
    assert "lse_part" in lib.mla_last_error().decode()
    assert ce(ctypes.byref(d), P(16), P(16), 2, None, P(16), None, None, None) == 1
    assert "w_uv" in lib.mla_last_error().decode()
    assert ce(ctypes.byref(d), P(16), P(16), 2, P(16), None, None, None, None) == 1
    assert ce(ctypes.byref(d), P(16), P(16), 2, P(16), P(16), P(24), None, None) == 6  # o_lat misaligned
    assert ce(ctypes.byref(d), P(16), P(16), 2, P(16), P(16), None, P(18), None) == 6  # lse misaligned
    assert "mla_combine_expand_v" in lib.mla_last_error().decode()


def test_recommended_splits(lib):
    assert binding.mla_recommended_splits(binding.dims(32, 128, 0.07), 4096, 256) == 8
    assert binding.mla_recommended_splits(binding.dims(64, 16, 0.07), 4096, 256) == 4
    assert binding.mla_recommended_splits(binding.dims(1, 16, 0.07), 26, 256) == 1


def _append(lib, d, cache, kv_in=4096, in_stride=576, positions=4096, num_new=1, rope_base=10000.0):
    P = ctypes.c_void_p
    return lib.mla_cache_append(ctypes.byref(d), ctypes.byref(cache) if cache is not None else None,
                                P(kv_in) if kv_in else None, in_stride, P(positions) if positions else None,
                                num_new, rope_base, None)


def test_cache_append_validation(lib):
    d = binding.dims(2, 16, 0.07)
    base = dict(dtype=0, kv=1024, pe=2048, kv_stride=576, pe_stride=576, token_scale=None, seq_stride=64,
                block_table=None, block_size=0, max_blocks_per_seq=0)

    def cache(**kw):
        c = dict(base)
        c.update(kw)
        return binding.MlaCache(**c)

    def err():
        return lib.mla_last_error().decode()

    assert _append(lib, binding.dims(0, 16, 0.07), cache()) == 2 and "batch" in err()
    assert _append(lib, binding.dims(2, 16, 0.07, kv_lora_rank=0), cache()) == 2 and "kv_lora_rank" in err()
    assert _append(lib, binding.dims(2, 16, 0.07, qk_rope_head_dim=32), cache()) == 3
    assert _append(lib, d, cache(), rope_base=0.0) == 2 and "rope_base" in err()
    assert _append(lib, d, cache(), rope_base=-1.0) == 3 and "rope_base" in err()
    assert _append(lib, d, None) == 1
    assert _append(lib, d, cache(dtype=5)) == 3 and "dtype" in err()
    assert _append(lib, d, cache(dtype=1)) == 1 and "token_scale" in err()
    assert _append(lib, d, cache(token_scale=4096)) == 5 and "token_scale" in err()
    assert _append(lib, d, cache(kv=None)) == 1 and "mla_cache.kv" in err()
    assert _append(lib, d, cache(pe=2050)) == 6
    assert _append(lib, d, cache(kv_stride=516)) == 5 and "kv_stride" in err()
    assert _append(lib, d, cache(dtype=1, token_scale=4096, pe_stride=72)) == 5 and "pe_stride" in err()
    assert _append(lib, d, cache(seq_stride=0)) == 5 and "seq_stride" in err()
    assert _append(lib, d, cache(block_table=4096, block_size=0, max_blocks_per_seq=4)) == 4
    assert _append(lib, d, cache(block_table=4096, block_size=64, max_blocks_per_seq=0)) == 5
    assert _append(lib, d, cache(block_table=4098, block_size=64, max_blocks_per_seq=4)) == 6
    assert _append(lib, d, cache(), kv_in=0) == 1 and "kv_in" in err()
    assert _append(lib, d, cache(), kv_in=4100) == 6 and "kv_in" in err()
    assert _append(lib, d, cache(), in_stride=572) == 5 and "in_stride" in err()
    assert _append(lib, d, cache(), in_stride=580) == 5 and "in_stride" in err()
    assert _append(lib, d, cache(), positions=0) == 1 and "positions" in err()
    assert _append(lib, d, cache(), num_new=-1) == 4 and "num_new" in err()
    # nothing to append: accepted, and nothing is launched (this machine has no GPU)
    assert _append(lib, d, cache(), num_new=0) == 0 and err() == ""
    assert _append(lib, d, cache(block_table=4096, block_size=48, max_blocks_per_seq=4), num_new=0) == 0


def test_decode_step_fused_validation(lib):
    d = binding.dims(2, 16, 0.07)
    P = ctypes.c_void_p
    base = dict(dtype=0, kv=1024, pe=2048, kv_stride=576, pe_stride=576, token_scale=None, seq_stride=64,
                block_table=None, block_size=0, max_blocks_per_seq=0)

    def call(cache=True, max_len=64, qn=16, qpe=16, wuk=16, wuv=16, lens=16, out=16, o_lat=0, lse=0, dd=d, **kw):
        c = dict(base)
        c.update(kw)
        cc = binding.MlaCache(**c)
        return lib.mla_decode_step_fused(ctypes.byref(dd), ctypes.byref(cc) if cache else None, P(qn), P(qpe),
                                         P(wuk) if wuk else None, P(wuv) if wuv else None, P(lens) if lens else None,
                                         max_len, P(out) if out else None, P(o_lat) if o_lat else None,
                                         P(lse) if lse else None, None)

    def err():
        return lib.mla_last_error().decode()

    assert call(dd=binding.dims(2, 0, 0.07)) == 2 and "num_heads" in err()
    assert call(cache=False) == 1 and "cache" in err()
    assert call(dtype=1) == 1 and "token_scale" in err()
    assert call(kv_stride=500) == 5 and "kv_stride" in err()
    assert call(max_len=0) == 4
    assert call(seq_stride=32) == 5 and "seq_stride" in err()
    assert call(wuk=0) == 1 and "w_uk" in err()
    assert call(wuv=8) == 6 and "w_uv" in err()
    assert call(lens=0) == 1 and "seq_lens" in err()
    assert call(out=0) == 1 and "out" in err()
    assert call(o_lat=8) == 6 and "o_lat" in err()
    assert call(lse=2) == 6 and "lse" in err()
    assert call(block_table=4096, block_size=48, max_blocks_per_seq=4) == 4


def test_naive_decode_validation(lib):
    d = binding.dims(2, 16, 0.07)
    P = ctypes.c_void_p
    need = binding.mla_naive_workspace_bytes(d, 64)
    assert need == 2 * 64 * 16 * 256 * 2
    cache = binding.MlaCache(dtype=0, kv=1024, pe=2048, kv_stride=576, pe_stride=576, token_scale=None,
                             seq_stride=64, block_table=None, block_size=0, max_blocks_per_seq=0)

    def call(ws=4096, ws_bytes=need, out=16, wuk=16, max_len=64):
        return lib.mla_naive_decode(ctypes.byref(d), ctypes.byref(cache), P(16), P(16), P(wuk) if wuk else None,
                                    P(16), P(16), max_len, P(ws) if ws else None, ws_bytes, P(out) if out else None,
                                    None)

    def err():
        return lib.mla_last_error().decode()

    assert call(ws=0) == 1 and "workspace" in err()
    assert call(ws_bytes=need - 1) == 5 and "workspace_bytes" in err()
    assert call(out=0) == 1 and "out" in err()
    assert call(wuk=0) == 1 and "w_uk" in err()
    assert call(max_len=0) == 4
    with pytest.raises(binding.MlaError):
        binding.mla_naive_workspace_bytes(d, 0)


def test_prefill_latent_validation(lib):
    d = binding.dims(2, 16, 0.07)
    P = ctypes.c_void_p
    cache = binding.MlaCache(dtype=0, kv=1024, pe=2048, kv_stride=576, pe_stride=576, token_scale=None,
                             seq_stride=64, block_table=None, block_size=0, max_blocks_per_seq=0)

    def call(starts=16, num_q=4, max_len=64, splits=1, o_lat=64, lse=64):
        return lib.mla_prefill_latent(ctypes.byref(d), ctypes.byref(cache), P(16), P(16), P(starts) if starts else None,
                                      num_q, max_len, splits, None, None, P(o_lat) if o_lat else None,
                                      P(lse) if lse else None, None)

    def err():
        return lib.mla_last_error().decode()

    assert call(starts=0) == 1 and "q_start" in err()
    assert call(starts=18) == 6 and "q_start" in err()
    assert call(num_q=0) == 4 and "num_q" in err()
    assert call(max_len=0) == 4
    assert call(max_len=128) == 5 and "seq_stride" in err()
    assert call(splits=2) == 1 and "o_part" in err()
    assert call(o_lat=0) == 1 and "o_lat" in err()
