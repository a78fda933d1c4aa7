"""Pins of the float64 oracle against facts that do not come from the oracle.

Each ``check_*`` function takes the oracle module as an argument and raises
AssertionError (or any exception) when the oracle disagrees with:

* numbers printed on the source pages (tests/golden/cache_sizes.json),
* closed forms (a two-token worked example, lse of a uniform softmax, the
  E4M3 and bfloat16 encodings),
* brute force in pure-Python loops on tiny inputs,
* special cases that reduce to a library routine (PyTorch's
  scaled_dot_product_attention in float64, torch's bfloat16 / float8 casts),
* identities the pages state: naive == absorbed (matrix associativity),
  prefill + incremental decode == one-shot forward, and RoPE on the content
  key breaking absorption (the reason RoPE is decoupled).

``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutations.py`` plants plausible mistakes in copies of the
oracle and checks that some pin catches each one.
"""

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MiB = 1024.0 ** 2
GiB = 1024.0 ** 3


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(rng, H, T, d_c, d_r, d_n, d_v):
    return dict(
        q_nope=rng.standard_normal((H, d_n)),
        q_pe=rng.standard_normal((H, d_r)),
        c=rng.standard_normal((T, d_c)),
        k_r=rng.standard_normal((T, d_r)),
        w_uk=rng.standard_normal((H, d_n, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
    )


def _absorbed_one(orc, p, scale):
    q_lat = orc.absorb_q(p["q_nope"][None], p["w_uk"])[0]
    o_lat, lse = orc.latent_attention(q_lat, p["q_pe"], p["c"], p["k_r"], scale)
    out = orc.expand_v(o_lat[None], p["w_uv"])[0]
    return q_lat, o_lat, lse, out


# ---------------------------------------------------------------------------
# closed forms printed on the pages
# ---------------------------------------------------------------------------

def check_cache_sizes(orc):
    g = json.load(open(os.path.join(GOLDEN, "cache_sizes.json")))

    a = g["v2lite_active_26_tokens_bf16"]
    d = a["dims"]
    T, H, e = d["tokens"], d["heads"], d["elem_bytes"]
    per_tok = orc.latent_cache_bytes_per_token(d["kv_lora_rank"], d["qk_rope_head_dim"], e)
    assert T * per_tok == a["absorb_total"]
    assert orc.latent_cache_bytes_per_token(d["kv_lora_rank"], 0, e) * T == a["absorb_latent"]
    assert orc.latent_cache_bytes_per_token(0, d["qk_rope_head_dim"], e) * T == a["absorb_rope"]
    naive = orc.naive_cache_bytes_per_token(H, d["qk_nope_head_dim"], d["qk_rope_head_dim"], d["v_head_dim"], e)
    assert T * naive == a["naive_total"]
    assert T * orc.naive_cache_bytes_per_token(H, d["qk_nope_head_dim"], d["qk_rope_head_dim"], 0, e) == a["naive_key"]
    assert T * orc.naive_cache_bytes_per_token(H, 0, 0, d["v_head_dim"], e) == a["naive_value"]
    assert abs(naive / per_tok - a["ratio_naive_over_absorb"]) < 1e-12
    assert abs(100.0 * (1 - per_tok / naive) - a["reduction_percent"]) < 1e-12
    # decode read of the whole 26-token history = active latent bytes
    assert orc.decode_kv_read_bytes(1, T, d["kv_lora_rank"], d["qk_rope_head_dim"], e) == a["absorb_total"]

    s = g["v2lite_allocated_32_slots_bf16"]
    n = s["slots"]
    assert n * orc.latent_cache_bytes_per_token(d["kv_lora_rank"], d["qk_rope_head_dim"], e) == s["absorb_total"]
    assert n * orc.latent_cache_bytes_per_token(d["kv_lora_rank"], 0, e) == s["absorb_latent"]
    assert n * orc.latent_cache_bytes_per_token(0, d["qk_rope_head_dim"], e) == s["absorb_rope"]
    assert n * naive == s["naive_total"]
    assert n * orc.naive_cache_bytes_per_token(H, d["qk_nope_head_dim"], d["qk_rope_head_dim"], 0, e) == s["naive_key"]
    assert n * orc.naive_cache_bytes_per_token(H, 0, 0, d["v_head_dim"], e) == s["naive_value"]

    t = g["v2lite_per_token_per_layer_bf16"]
    assert naive == t["expanded_bytes"] and naive // e == t["expanded_elements"]
    assert per_tok == t["latent_bytes"] and per_tok // e == t["latent_elements"]
    assert round(naive / per_tok, 4) == t["ratio"]

    f = g["per_token_fp16_table"]["deepseek_v2_style"]
    mha = orc.mha_cache_bytes_per_token(f["n_h"], f["d_h"], 2)
    gqa = orc.gqa_cache_bytes_per_token(f["n_kv"], f["d_h"], 2)
    mla = orc.latent_cache_bytes_per_token(f["kv_lora_rank"], f["qk_rope_head_dim"], 2)
    assert (mha, gqa, mla) == (f["mha"], f["gqa8"], f["mla"])
    assert round(mha / mla, 1) == f["mha_over_mla"]
    tot = f["layers"] * f["tokens"]
    assert round(tot * mha / GiB, 2) == f["mha_total_GiB"]
    assert round(tot * gqa / GiB, 2) == f["gqa_total_GiB"]
    assert round(tot * mla / GiB, 2) == f["mla_total_GiB"]
    l3 = g["per_token_fp16_table"]["llama3_70b_like"]
    assert orc.mha_cache_bytes_per_token(l3["n_h"], l3["d_h"], 2) == l3["mha"]
    assert orc.gqa_cache_bytes_per_token(l3["n_kv"], l3["d_h"], 2) == l3["gqa8"]
    assert round(tot * orc.mha_cache_bytes_per_token(l3["n_h"], l3["d_h"], 2) / GiB, 2) == l3["mha_total_GiB"]

    for row in g["live_allocation_fp16"]["rows"]:
        L = row["L"]
        assert L * mha / MiB == row["mha_MiB"]
        assert L * mla / MiB == row["mla_MiB"]
        assert round(mha / mla, 1) == row["ratio"]

    r = g["latency_runs_cache_fp16"]
    mha_r = orc.mha_cache_bytes_per_token(r["n_h"], r["d_h"], 2)
    mla_r = orc.latent_cache_bytes_per_token(r["kv_lora_rank"], r["qk_rope_head_dim"], 2)
    for row in r["rows"]:
        L = row["prefill"] + r["decode_tokens"]
        assert round(L * mha_r / MiB, 2) == row["mha_MiB"]
        assert round(L * mla_r / MiB, 2) == row["mla_MiB"]

    v3 = g["deepseek_v3_ratio"]
    ratio = orc.mha_equivalent_ratio(v3["kv_lora_rank"], v3["qk_rope_head_dim"], v3["n_h"], v3["d_h"])
    assert round(1.0 / ratio) == v3["one_over_ratio_rounded"]
    assert abs(ratio - 576.0 / 32768.0) < 1e-15
    assert orc.equivalent_gqa_groups(v3["kv_lora_rank"], v3["qk_rope_head_dim"], v3["d_h"]) == v3["gqa_groups"]

    f8 = g["deepseek_v3_fp8_decode_read"]
    for B in (1, 7, 32):
        assert orc.decode_kv_read_bytes(B, f8["s_ctx"], f8["kv_lora_rank"], f8["qk_rope_head_dim"],
                                        f8["elem_bytes"]) == B * f8["per_sequence_bytes"]
    # grows with the context length, and has no head-count argument at all
    reads = [orc.decode_kv_read_bytes(4, s, 512, 64, 2) for s in (1, 2, 100, 4096, 32768)]
    assert all(x < y for x, y in zip(reads, reads[1:]))


def check_required_fields(orc):
    for kwargs, field in (({"kv_lora_rank": None, "qk_rope_head_dim": 64}, "kv_lora_rank"),
                          ({"kv_lora_rank": 512, "qk_rope_head_dim": None}, "qk_rope_head_dim")):
        try:
            orc.latent_cache_bytes_per_token(elem_bytes=2, source="test config dict", **kwargs)
        except ValueError as exc:
            assert field in str(exc) and "test config dict" in str(exc)
        else:
            raise AssertionError(f"missing {field} did not raise")
        try:
            orc.decode_kv_read_bytes(1, 10, elem_bytes=1, **kwargs)
        except ValueError as exc:
            assert field in str(exc)
        else:
            raise AssertionError(f"missing {field} did not raise (decode read)")


# ---------------------------------------------------------------------------
# element decoders against the library's own casts and spec values
# ---------------------------------------------------------------------------

def check_bf16_decode(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert orc.bf16_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert orc.bf16_to_f64(np.array([0xC000], dtype=np.uint16))[0] == -2.0


def check_e4m3_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    spec = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in spec.items():
        assert orc.e4m3fn_to_f64(np.array([c], dtype=np.uint8))[0] == v
    assert np.isnan(orc.e4m3fn_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


# ---------------------------------------------------------------------------
# attention: worked example, brute force, library special case, identities
# ---------------------------------------------------------------------------

def check_worked_example(orc):
    """Two tokens, one head, scores ln 3 and 0 by construction:
    p = (3/4, 1/4), o_lat = (3/4, 1/4), lse = ln 4, out = W_UV o_lat."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    q_lat = np.array(g["q_lat"], dtype=np.float64)
    q_pe = np.array(g["q_pe"], dtype=np.float64)
    c = np.array(g["c"], dtype=np.float64)
    k_r = np.array(g["k_r"], dtype=np.float64)
    o, lse = orc.latent_attention(q_lat, q_pe, c, k_r, g["scale"])
    assert np.allclose(o, np.array(g["o_lat"]), rtol=0, atol=1e-15)
    assert abs(lse[0] - math.log(g["lse_exp"])) < 1e-15
    out = orc.expand_v(o[None], np.array(g["w_uv"], dtype=np.float64))[0]
    assert np.allclose(out, np.array(g["out"]), rtol=0, atol=1e-15)


def _brute(p, scale):
    """Pure-Python loops over the plain definition (expanded keys/values)."""
    H, d_n = p["q_nope"].shape
    T, d_c = p["c"].shape
    d_r = p["k_r"].shape[1]
    d_v = p["w_uv"].shape[1]
    outs, olats, lses = [], [], []
    for h in range(H):
        scores = []
        for t in range(T):
            s = 0.0
            for i in range(d_n):
                k_i = 0.0
                for j in range(d_c):
                    k_i += p["w_uk"][h][i][j] * p["c"][t][j]
                s += p["q_nope"][h][i] * k_i
            for i in range(d_r):
                s += p["q_pe"][h][i] * p["k_r"][t][i]
            scores.append(scale * s)
        z = sum(math.exp(s) for s in scores)
        probs = [math.exp(s) / z for s in scores]
        lses.append(math.log(z))
        olats.append([sum(probs[t] * p["c"][t][j] for t in range(T)) for j in range(d_c)])
        o = []
        for i in range(d_v):
            acc = 0.0
            for t in range(T):
                v = 0.0
                for j in range(d_c):
                    v += p["w_uv"][h][i][j] * p["c"][t][j]
                acc += probs[t] * v
            o.append(acc)
        outs.append(o)
    return np.array(outs), np.array(olats), np.array(lses)


def check_brute_force(orc):
    for seed, (H, T, d_c, d_r, d_n, d_v) in enumerate([(2, 3, 4, 2, 3, 5), (3, 5, 6, 4, 2, 3), (1, 1, 3, 2, 2, 2)]):
        p = _rand_problem(_rng(100 + seed), H, T, d_c, d_r, d_n, d_v)
        scale = 0.37 + 0.1 * seed
        ref_out, ref_olat, ref_lse = _brute(p, scale)
        _, o_lat, lse, out = _absorbed_one(orc, p, scale)
        assert _rel(out, ref_out) < 1e-12, (seed, _rel(out, ref_out))
        assert _rel(o_lat, ref_olat) < 1e-12
        assert np.max(np.abs(lse - ref_lse)) < 1e-12
        nv = orc.naive_attention(p["q_nope"], p["q_pe"], p["c"], p["k_r"], p["w_uk"], p["w_uv"], scale)
        assert _rel(nv, ref_out) < 1e-12


def check_textbook_sdpa(orc):
    """H=1, W_UK = W_UV = I (d_n = d_v = d_c): MLA decode is single-head
    attention with keys [c_t ; k_R,t] and values c_t."""
    rng = _rng(7)
    d_c, d_r, T = 8, 4, 13
    q = rng.standard_normal((1, 1, 1, d_c + d_r))
    c = rng.standard_normal((T, d_c))
    k_r = rng.standard_normal((T, d_r))
    scale = 1.0 / math.sqrt(d_c + d_r)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.concatenate([c, k_r], 1))[None, None],
        torch.from_numpy(c)[None, None], scale=scale).numpy()[0, 0, 0]
    eye = np.eye(d_c)[None]
    p = dict(q_nope=q[0, 0, :, :d_c], q_pe=q[0, 0, :, d_c:], c=c, k_r=k_r, w_uk=eye, w_uv=eye)
    _, o_lat, _, out = _absorbed_one(orc, p, scale)
    assert _rel(out[0], ref) < 1e-12
    assert _rel(o_lat[0], ref) < 1e-12
    nv = orc.naive_attention(p["q_nope"], p["q_pe"], c, k_r, eye, eye, scale)
    assert _rel(nv[0], ref) < 1e-12


def check_naive_equals_absorbed(orc):
    """Matrix associativity: expanded keys/values and absorbed weights give
    the same output ([AUDIT] §2.2-§2.3)."""
    for seed, dims in enumerate([(4, 37, 16, 8, 12, 10), (16, 26, 512, 64, 128, 128)]):
        p = _rand_problem(_rng(200 + seed), *dims)
        scale = 1.0 / math.sqrt(dims[4] + dims[3])
        _, _, _, out = _absorbed_one(orc, p, scale)
        nv = orc.naive_attention(p["q_nope"], p["q_pe"], p["c"], p["k_r"], p["w_uk"], p["w_uv"], scale)
        assert _rel(out, nv) < 1e-12, _rel(out, nv)


def check_special_cases(orc):
    rng = _rng(300)
    H, d_c, d_r = 3, 10, 4
    c = rng.standard_normal((1, d_c))
    k_r = rng.standard_normal((1, d_r))
    q_lat = rng.standard_normal((H, d_c))
    q_pe = rng.standard_normal((H, d_r))
    # one cached token: the softmax is 1, o_lat is that token's latent row
    o, lse = orc.latent_attention(q_lat, q_pe, c, k_r, 0.3)
    assert np.array_equal(o, np.repeat(c, H, axis=0))
    assert np.allclose(lse, 0.3 * (q_lat @ c[0] + q_pe @ k_r[0]), rtol=0, atol=1e-14)
    # zero query: uniform softmax, o_lat = mean row, lse = ln T
    T = 9
    c = rng.standard_normal((T, d_c))
    k_r = rng.standard_normal((T, d_r))
    o, lse = orc.latent_attention(np.zeros((H, d_c)), np.zeros((H, d_r)), c, k_r, 0.3)
    assert np.allclose(o, np.repeat(c.mean(0, keepdims=True), H, axis=0), rtol=0, atol=1e-15)
    assert np.allclose(lse, math.log(T), rtol=0, atol=1e-15)
    # every latent row equal: o_lat is that row whatever the scores
    same = np.repeat(c[:1], T, axis=0)
    o, _ = orc.latent_attention(q_lat, q_pe, same, k_r, 0.3)
    assert np.allclose(o, np.repeat(c[:1], H, axis=0), rtol=0, atol=1e-14)
    # permuting the cached tokens changes nothing
    perm = rng.permutation(T)
    o1, l1 = orc.latent_attention(q_lat, q_pe, c, k_r, 0.3)
    o2, l2 = orc.latent_attention(q_lat, q_pe, c[perm], k_r[perm], 0.3)
    assert _rel(o1, o2) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13
    # the rope half enters the score: only token 4 has a non-zero rope key
    # and q_pe points along it, so (with a zero content query) token 4 takes
    # all but e^-50 of the weight
    k_r1 = np.zeros((T, d_r))
    k_r1[4, 0] = 1.0
    q_pe1 = np.zeros((1, d_r))
    q_pe1[0, 0] = 50.0
    o3, lse3 = orc.latent_attention(np.zeros((1, d_c)), q_pe1, c, k_r1, 1.0)
    assert _rel(o3[0], c[4]) < 10 * (T - 1) * math.exp(-50.0)
    assert abs(lse3[0] - (50.0 + math.log1p((T - 1) * math.exp(-50.0)))) < 1e-13
    # empty range: no weight
    o, lse = orc.latent_attention(q_lat, q_pe, c[:0], k_r[:0], 0.3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def check_split_combine(orc):
    """A softmax over a union of disjoint ranges equals the log-sum-exp merge
    of the per-range results, for any partition (empty ranges included)."""
    rng = _rng(400)
    H, T, d_c, d_r = 4, 50, 12, 6
    c = rng.standard_normal((T, d_c))
    k_r = rng.standard_normal((T, d_r))
    q_lat = 2.0 * rng.standard_normal((H, d_c))
    q_pe = rng.standard_normal((H, d_r))
    o_ref, lse_ref = orc.latent_attention(q_lat, q_pe, c, k_r, 0.4)
    partitions = [[0, T], [0, 0, T], [0, 10, 10, 33, T, T], [0, 1, 2, 3, 4, T],
                  sorted([0, T] + list(rng.integers(0, T, 6)))]
    for bounds in partitions:
        o_p, l_p = orc.latent_attention_ranges(q_lat, q_pe, c, k_r, 0.4, bounds)
        o, lse = orc.combine_splits(o_p, l_p)
        assert _rel(o, o_ref) < 1e-13, bounds
        assert np.max(np.abs(lse - lse_ref)) < 1e-13
    # merge closed form for two parts with known lse: weights e^a/(e^a+e^b)
    o_p = np.stack([np.ones((1, 2)), 3 * np.ones((1, 2))])
    o, lse = orc.combine_splits(o_p, np.array([[math.log(1.0)], [math.log(3.0)]]))
    assert np.allclose(o, 2.5, rtol=0, atol=1e-15) and abs(lse[0] - math.log(4.0)) < 1e-15


def check_rope(orc):
    # position 0 is the identity; (1, 0) at position 1 rotates by 1 rad in the
    # first pair; the k-th pair's angle per position is base**(-2k/d)
    x = np.array([[1.0, 0.0, 1.0, 0.0]])
    assert np.array_equal(orc.rope_interleaved(x, [0]), x)
    y = orc.rope_interleaved(x, [1], base=10000.0)
    assert np.allclose(y[0], [math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)], rtol=0, atol=1e-15)
    x2 = np.array([[0.0, 1.0]])
    assert np.allclose(orc.rope_interleaved(x2, [2])[0], [-math.sin(2), math.cos(2)], rtol=0, atol=1e-15)
    # norm preserved; the dot product of two rotated vectors depends on the
    # position difference only
    rng = _rng(500)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((1, 16))
    qr = orc.rope_interleaved(np.repeat(q, 3, 0), [5, 9, 40])
    kr = orc.rope_interleaved(np.repeat(k, 3, 0), [2, 6, 37])
    assert np.allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q), rtol=1e-14)
    d = qr @ kr.T
    assert abs(d[0, 0] - d[1, 1]) < 1e-12 and abs(d[0, 0] - d[2, 2]) < 1e-12


def check_prefill_decode_vs_oneshot(orc):
    """Prefill of L-1 tokens then one decode step against the cache equals
    the one-shot causal forward over L tokens ([MLA80] §2 cache test): the
    prefill rows agree and the decoded row agrees.  The decode step runs in
    absorbed form against the rotated rope cache."""
    rng = _rng(600)
    L, H, d_c, d_r, d_n, d_v = 26, 16, 512, 64, 128, 128
    q_nope = rng.standard_normal((L, H, d_n))
    q_pe_raw = rng.standard_normal((L, H, d_r))
    c = rng.standard_normal((L, d_c))
    k_r_raw = rng.standard_normal((L, d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c)
    scale = orc.softmax_scale_default(d_n, d_r)
    full = orc.causal_naive_forward(q_nope, q_pe_raw, c, k_r_raw, w_uk, w_uv, scale)
    pre = orc.causal_naive_forward(q_nope[:-1], q_pe_raw[:-1], c[:-1], k_r_raw[:-1], w_uk, w_uv, scale)
    assert _rel(pre, full[:-1]) < 1e-12
    pe_cache = orc.rope_interleaved(k_r_raw, np.arange(L))
    q_pe_dec = orc.rope_interleaved(q_pe_raw[-1:], [L - 1])[0]
    q_lat = orc.absorb_q(q_nope[-1:], w_uk)[0]
    o_lat, _ = orc.latent_attention(q_lat, q_pe_dec, c, pe_cache, scale)
    dec = orc.expand_v(o_lat[None], w_uv)[0]
    assert _rel(dec, full[-1]) < 1e-12, _rel(dec, full[-1])
    assert abs(scale - 1.0 / math.sqrt(192.0)) < 1e-16


def check_rope_on_content_breaks_absorption(orc):
    """Absorbed content scores equal the expanded ones; rotating the expanded
    content key by position makes them disagree at O(1) ([MLA80] §4)."""
    rng = _rng(700)
    Lq, Lk, d_n, d_c = 4, 64, 32, 48
    q = rng.standard_normal((Lq, d_n))
    c = rng.standard_normal((Lk, d_c))
    w = rng.standard_normal((d_n, d_c)) / math.sqrt(d_c)
    a = orc.content_scores(q, c, w, absorbed=False)
    b = orc.content_scores(q, c, w, absorbed=True)
    assert _rel(b, a) < 1e-12
    a_rot = orc.content_scores(q, c, w, absorbed=False, rope_on_content=True,
                               positions_q=np.arange(Lk - Lq, Lk), positions_k=np.arange(Lk))
    assert _rel(b, a_rot) > 0.1


def check_cache_addressing(orc):
    """Paged rows behind a permuted block table decode to the same attention
    as the contiguous rows; E4M3 rows are code value times token scale."""
    rng = _rng(800)
    B, bs, d_c, d_r, H = 3, 4, 8, 4, 2
    lens = np.array([5, 12, 1])
    S = 12
    vals = rng.standard_normal((B, S, d_c + d_r)).astype(np.float32)
    bits = (torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    flat = bits.reshape(B * S, -1)
    q_lat = rng.standard_normal((B, H, d_c))
    q_pe = rng.standard_normal((B, H, d_r))
    o_ref, l_ref = orc.latent_decode(q_lat, q_pe, flat[:, :d_c], flat[:, d_c:], lens, 0.5, seq_stride=S)
    # hand-checked slots
    assert list(orc.token_slots(1, 3, seq_stride=S)) == [12, 13, 14]
    nblk = [(int(t) + bs - 1) // bs for t in lens]
    perm = rng.permutation(sum(nblk))
    pool = np.zeros((sum(nblk) * bs, d_c + d_r), dtype=np.uint16)
    table = np.zeros((B, max(nblk)), dtype=np.int32)
    k = 0
    for b in range(B):
        for j in range(nblk[b]):
            blk = perm[k]
            k += 1
            table[b, j] = blk
            n = min(bs, lens[b] - j * bs)
            pool[blk * bs: blk * bs + n] = bits[b, j * bs: j * bs + n]
    assert list(orc.token_slots(1, 6, block_table=table, block_size=bs)) == \
        [table[1, 0] * bs + i for i in range(4)] + [table[1, 1] * bs + i for i in range(2)]
    o_pg, l_pg = orc.latent_decode(q_lat, q_pe, pool[:, :d_c], pool[:, d_c:], lens, 0.5,
                                   block_table=table, block_size=bs)
    assert np.array_equal(o_pg, o_ref) and np.array_equal(l_pg, l_ref)
    codes = np.array([[0x38, 0xB8, 0x7E], [0x01, 0x00, 0x40]], dtype=np.uint8)
    sc = np.array([0.5, 4.0], dtype=np.float32)
    kv, pe = orc.load_rows(codes[:, :2], codes[:, 2:], np.array([1, 0]), "fp8_e4m3", sc)
    assert np.array_equal(kv, [[4.0 * 2 ** -9, 0.0], [0.5, -0.5]])
    assert np.array_equal(pe, [[4.0 * 2.0], [224.0]])


# ---------------------------------------------------------------------------
# encoders used by the cache append
# ---------------------------------------------------------------------------

def check_bf16_encode(orc):
    """float32 -> bfloat16 nearest-even against torch's cast, exact bfloat16
    values unchanged, and hand-made ties (to the even pattern)."""
    rng = _rng(900)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits(x), ref)
    codes = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    fin = codes[((codes >> 7) & 0xFF) != 0xFF]
    vals = orc.bf16_to_f64(fin).astype(np.float32)
    assert np.array_equal(orc.f32_to_bf16_bits(vals), fin)
    # 1 + 2^-8 lies halfway between 1 (0x3F80, even) and 1 + 2^-7 (0x3F81)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    assert list(orc.f32_to_bf16_bits(ties)) == [0x3F80, 0x3F82, 0xBF80]


def check_e4m3_encode(orc):
    """E4M3 nearest-even: every finite code is its own value's encoding,
    midpoints go to the even code, and torch's float8 cast agrees."""
    codes = np.arange(256, dtype=np.uint8)
    fin = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(orc.e4m3fn_encode(orc.e4m3fn_to_f64(fin)), fin)
    grid = orc.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    want = np.where(np.arange(len(mids)) % 2 == 0, np.arange(len(mids)), np.arange(1, len(mids) + 1))
    assert np.array_equal(orc.e4m3fn_encode(mids), want.astype(np.uint8))
    eps = 1e-9 * np.maximum(grid[1:] - grid[:-1], 0)
    assert np.array_equal(orc.e4m3fn_encode(mids - eps), np.arange(len(mids)).astype(np.uint8))
    assert np.array_equal(orc.e4m3fn_encode(mids + eps), np.arange(1, len(mids) + 1).astype(np.uint8))
    rng = _rng(901)
    x = np.clip(rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000), -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3fn_encode(x), ref)
    assert orc.e4m3fn_encode(np.array([-0.0]))[0] == 0x80 and orc.e4m3fn_encode(np.array([448.0]))[0] == 0x7E
    # per-token quantisation: the largest magnitude maps to +-448, every value
    # is within half an E4M3 step (relative 2^-4) of value / scale
    v = (rng.standard_normal((5, 576)) * 3).astype(np.float32)
    c, sc = orc.e4m3_quantize_token(v)
    assert np.allclose(sc, np.abs(v).max(axis=1) / 448.0, rtol=1e-7, atol=0)
    back = orc.e4m3fn_to_f64(c) * sc[:, None].astype(np.float64)
    big = np.abs(v) > 2.0 ** -6 * sc[:, None]
    assert np.all(np.abs(back - v)[big] <= np.abs(v)[big] * 2.0 ** -4 + 1e-12)
    assert np.all(np.abs(orc.e4m3fn_to_f64(c[np.arange(5), np.abs(v).argmax(axis=1)])) == 448.0)


def check_cache_append(orc):
    """Appended rows read back through the decoders: the latent half is the
    input exactly (bf16) or within E4M3 rounding; the key half is the input
    rotated at the row's position (RoPE by hand for one pair); positions run
    on from positions[b]."""
    rng = _rng(902)
    B, n = 2, 3
    vals = rng.standard_normal((B, n, 576)).astype(np.float32)
    bits = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = orc.bf16_to_f64(bits)
    positions = np.array([0, 41])
    pos, kv, pe, sc = orc.cache_append_rows(bits, positions, "bf16")
    assert pos.tolist() == [[0, 1, 2], [41, 42, 43]] and sc is None
    assert np.array_equal(kv, bits[..., :512])
    # pair i of the key rotated by pos * 10000^(-2i/64), written out by hand
    for b in range(B):
        for j in range(n):
            p = float(pos[b, j])
            for i in (0, 5, 31):
                a0, a1 = x[b, j, 512 + 2 * i], x[b, j, 513 + 2 * i]
                th = p * 10000.0 ** (-2.0 * i / 64.0)
                want = np.array([a0 * math.cos(th) - a1 * math.sin(th), a1 * math.cos(th) + a0 * math.sin(th)])
                got = orc.bf16_to_f64(pe[b, j, 2 * i:2 * i + 2])
                assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + 1e-30), (b, j, i)
    assert np.array_equal(pe[0, 0], bits[0, 0, 512:576])  # position 0: identity
    pos8, kv8, pe8, sc8 = orc.cache_append_rows(bits, positions, "fp8_e4m3")
    assert np.array_equal(pos8, pos)
    back = orc.e4m3fn_to_f64(kv8) * sc8[..., None]
    assert np.all(np.abs(back - x[..., :512]) <= np.abs(x[..., :512]) * 2.0 ** -4 + 2.0 ** -9 * sc8[..., None])
    back_pe = orc.e4m3fn_to_f64(pe8) * sc8[..., None]
    rot = orc.bf16_to_f64(pe)
    assert np.all(np.abs(back_pe - rot) <= np.abs(rot) * (2.0 ** -4 + 2.0 ** -7) + 2.0 ** -9 * sc8[..., None])


ALL_CHECKS = [
    check_cache_sizes, check_required_fields, check_bf16_decode, check_e4m3_decode,
    check_worked_example, check_brute_force, check_textbook_sdpa, check_naive_equals_absorbed,
    check_special_cases, check_split_combine, check_rope, check_prefill_decode_vs_oneshot,
    check_rope_on_content_breaks_absorption, check_cache_addressing,
    check_bf16_encode, check_e4m3_encode, check_cache_append,
]
