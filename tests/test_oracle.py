"""Pins for the CPU fp64 oracle: closed forms, invariants, brute force, and an
online-softmax emulation. None of these re-types the oracle's formula: each checks it
against something the mathematics fixes independently.

The mutation tests at the bottom plant a plausible mistake in the oracle (on the CPU) and
check that at least one pin rejects it.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oracle_mod
from workloads import (C4_LENGTHS, CONFIGS, cu_seqlens_from_lengths, dense_inputs,
                       round_to_dtype, sampled_rows, varlen_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
VARIANTS = ["full", "rows", "varlen", "varlen_rows"]


def run_variant(variant, q, k, v, *, causal, scale):
    """Route one dense problem through one of the oracle's entry points and return the
    full [B,Hq,Nq,d] result."""
    B, Hq, Nq, d = q.shape
    if variant == "full":
        return oracle.attention_ref(q, k, v, causal=causal, scale=scale)
    if variant == "rows":
        rows = np.random.default_rng(7).permutation(Nq)
        part = oracle.attention_ref_rows(q, k, v, rows, causal=causal, scale=scale)
        out = np.empty_like(part)
        out[:, :, rows] = part
        return out
    # varlen variants: one packed sequence per batch entry; needs Hq == Hkv, Nq == Nk
    assert k.shape[1] == Hq and k.shape[2] == Nq
    qkv = np.stack([q, k, v], axis=2)              # [B, H, 3, N, d]
    qkv = qkv.transpose(0, 3, 2, 1, 4).reshape(B * Nq, 3, Hq, d)
    cu = cu_seqlens_from_lengths([Nq] * B)
    if variant == "varlen":
        o = oracle.attention_ref_varlen(qkv, cu, causal=causal, scale=scale)
    else:
        toks = np.random.default_rng(8).permutation(B * Nq)
        part = oracle.attention_ref_varlen_rows(qkv, cu, toks, causal=causal, scale=scale)
        o = np.empty_like(part)
        o[toks] = part
    return o.reshape(B, Nq, Hq, d).transpose(0, 2, 1, 3)


def _variants_for(q, k):
    same = (k.shape[1] == q.shape[1] and k.shape[2] == q.shape[2])
    return VARIANTS if same else ["full", "rows"]


def rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("variant", ["full", "rows"])
@pytest.mark.parametrize("scale", [0.125, 37.0, -2.5, 1e-3])
def test_single_key_returns_v(variant, scale):
    # one key: softmax over a single entry is 1, so every query returns V[0]
    q = rand((2, 4, 5, 8), 1)
    k = rand((2, 2, 1, 8), 2)
    v = rand((2, 2, 1, 8), 3)
    o = run_variant(variant, q, k, v, causal=False, scale=scale)
    expect = np.repeat(v, 2, axis=1)[:, :, :1, :].repeat(5, axis=2)
    assert np.array_equal(o, expect)


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_token_causal(variant):
    q, k, v = rand((1, 2, 1, 16), 4), rand((1, 2, 1, 16), 5), rand((1, 2, 1, 16), 6)
    assert np.array_equal(run_variant(variant, q, k, v, causal=True, scale=0.3), v)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(variant, causal):
    # all keys equal -> all scores in a row equal -> uniform weights over allowed keys
    B, H, N, d = 2, 3, 9, 4
    q = rand((B, H, N, d), 10)
    krow = rand((B, H, 1, d), 11)
    k = np.repeat(krow, N, axis=2)
    v = rand((B, H, N, d), 12)
    o = run_variant(variant, q, k, v, causal=causal, scale=0.7)
    if causal:
        expect = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    else:
        expect = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.max(np.abs(o - expect)) < 1e-12


@pytest.mark.parametrize("variant", VARIANTS)
def test_causal_row0_is_v0(variant):
    q, k, v = rand((2, 4, 7, 8), 20, 3.0), rand((2, 4, 7, 8), 21, 3.0), rand((2, 4, 7, 8), 22)
    o = run_variant(variant, q, k, v, causal=True, scale=1.0)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :])


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_mean_of_allowed_v(variant, causal):
    B, H, N, d = 1, 2, 6, 5
    q, k, v = rand((B, H, N, d), 30), rand((B, H, N, d), 31), rand((B, H, N, d), 32)
    o = run_variant(variant, q, k, v, causal=causal, scale=0.0)
    if causal:
        expect = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    else:
        expect = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.max(np.abs(o - expect)) < 1e-12


@pytest.mark.parametrize("variant", ["full", "rows"])
def test_two_keys_closed_form(variant):
    # scores (a, b) -> weights (sigmoid(a-b), sigmoid(b-a)); values written out by hand
    q = np.array([[[[1.0, 0.0]], [[0.0, 2.0]]]])            # [1, 2, 1, 2]
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])              # [1, 1, 2, 2]
    v = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    scale = 0.5
    o = run_variant(variant, q, k, v, causal=False, scale=scale)
    for h, (a, b) in enumerate([(0.5, 0.0), (0.0, 1.0)]):
        w0 = 1.0 / (1.0 + math.exp(b - a))
        w1 = 1.0 - w0
        expect = [w0 * 1.0 + w1 * 3.0, w0 * 2.0 + w1 * 4.0]
        assert np.max(np.abs(o[0, h, 0] - expect)) < 1e-15


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_dominant_key(variant, causal):
    # key j* scores >= 60 above every other allowed key: O = V[j*] to about e^-60
    N, d = 8, 16
    rng = np.random.default_rng(40)
    q = rng.standard_normal((1, 1, N, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, 1, N, d)) * 0.01
    jstar = 2
    v = rng.standard_normal((1, 1, N, d))
    k[0, 0, jstar] = 0.0
    # make key j* align with every query: sum of all queries, scaled
    k[0, 0, jstar] = 200.0 * q[0, 0].sum(axis=0) / np.linalg.norm(q[0, 0].sum(axis=0))
    # keep only queries that really prefer j* (dot >= 60 above the rest)
    s = q[0, 0] @ k[0, 0].T
    good = [i for i in range(N) if all(s[i, jstar] - s[i, j] >= 60 for j in range(N)
                                      if j != jstar)]
    assert len(good) >= 3
    o = run_variant(variant, q, k, v, causal=causal, scale=1.0)
    for i in good:
        if causal and i < jstar:
            continue
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, jstar])) < 1e-15


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_shift_keys_by_constant_vector(variant, causal):
    # S[i,j] -> S[i,j] + scale*q_i.c: a per-row constant, which softmax ignores
    B, H, N, d = 2, 2, 10, 8
    q, k, v = rand((B, H, N, d), 50), rand((B, H, N, d), 51), rand((B, H, N, d), 52)
    c = rand((B, H, 1, d), 53, 2.0)
    o1 = run_variant(variant, q, k, v, causal=causal, scale=0.4)
    o2 = run_variant(variant, q, k + c, v, causal=causal, scale=0.4)
    assert np.max(np.abs(o1 - o2)) < 1e-12


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_and_linearity(variant, causal):
    B, H, N, d = 1, 2, 11, 6
    q, k = rand((B, H, N, d), 60), rand((B, H, N, d), 61)
    c = rand((B, H, 1, d), 62)
    o = run_variant(variant, q, k, np.repeat(c, N, axis=2), causal=causal, scale=0.9)
    assert np.max(np.abs(o - np.repeat(c, N, axis=2))) < 1e-12
    v1, v2 = rand((B, H, N, d), 63), rand((B, H, N, d), 64)
    a, b = 1.7, -0.3
    lhs = run_variant(variant, q, k, a * v1 + b * v2, causal=causal, scale=0.9)
    rhs = (a * run_variant(variant, q, k, v1, causal=causal, scale=0.9)
           + b * run_variant(variant, q, k, v2, causal=causal, scale=0.9))
    assert np.max(np.abs(lhs - rhs)) < 1e-12


@pytest.mark.parametrize("variant", ["full", "rows"])
def test_joint_kv_permutation_noncausal(variant):
    q, k, v = rand((1, 4, 7, 8), 70), rand((1, 2, 13, 8), 71), rand((1, 2, 13, 8), 72)
    perm = np.random.default_rng(73).permutation(13)
    o1 = run_variant(variant, q, k, v, causal=False, scale=0.5)
    o2 = run_variant(variant, q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.5)
    assert np.max(np.abs(o1 - o2)) < 1e-12


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
def test_output_is_convex_combination(variant, causal):
    B, H, N, d = 1, 2, 12, 5
    q, k, v = rand((B, H, N, d), 80, 2.0), rand((B, H, N, d), 81, 2.0), rand((B, H, N, d), 82)
    o = run_variant(variant, q, k, v, causal=causal, scale=1.3)
    for i in range(N):
        allowed = v[:, :, : i + 1] if causal else v
        lo, hi = allowed.min(axis=2), allowed.max(axis=2)
        assert np.all(o[:, :, i] >= lo - 1e-12) and np.all(o[:, :, i] <= hi + 1e-12)


def test_gqa_equals_repeat_interleaved_kv():
    # query head hq reads kv head hq // G: same as dense attention on K/V with every kv
    # head repeated G times in place (torch.repeat_interleave along the head axis)
    G = 3
    q = rand((2, 6, 9, 8), 90)
    k, v = rand((2, 2, 9, 8), 91), rand((2, 2, 9, 8), 92)
    for causal in (False, True):
        o_gqa = oracle.attention_ref(q, k, v, causal=causal, scale=0.35)
        o_rep = oracle.attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                                     causal=causal, scale=0.35)
        assert np.array_equal(o_gqa, o_rep)
        rows = [8, 0, 4]
        o_rows = oracle.attention_ref_rows(q, k, v, rows, causal=causal, scale=0.35)
        o_rep_rows = oracle.attention_ref_rows(q, np.repeat(k, G, axis=1),
                                               np.repeat(v, G, axis=1), rows,
                                               causal=causal, scale=0.35)
        assert np.array_equal(o_rows, o_rep_rows)


def test_mqa_single_kv_head():
    q = rand((1, 4, 6, 8), 93)
    k, v = rand((1, 1, 6, 8), 94), rand((1, 1, 6, 8), 95)
    o = oracle.attention_ref(q, k, v, causal=True, scale=0.5)
    for h in range(4):
        oh = oracle.attention_ref(q[:, h:h + 1], k, v, causal=True, scale=0.5)
        assert np.array_equal(o[:, h:h + 1], oh)


# ---------------------------------------------------------------- varlen

def test_varlen_golden_cu_seqlens_example():
    with open(os.path.join(GOLDEN, "cu_seqlens_example.json")) as f:
        g = json.load(f)
    cu = np.array(g["cu_seqlens"], dtype=np.int32)
    assert len(cu) - 1 == g["batch_size"]
    assert cu[-1] == g["total_tokens"]
    H, d = 2, 8
    qkv = rand((g["total_tokens"], 3, H, d), 100)
    for causal in (False, True):
        o = oracle.attention_ref_varlen(qkv, cu, causal=causal, scale=0.5)
        assert o.shape == (g["total_tokens"], H, d)
        for a, e in g["segments"]:
            seg = qkv[a:e]
            q, k, v = (seg[:, c].transpose(1, 0, 2)[None] for c in range(3))
            dense = oracle.attention_ref(q, k, v, causal=causal, scale=0.5)[0]
            assert np.array_equal(o[a:e], dense.transpose(1, 0, 2))
        # tokens of the second sequence never influence the first
        qkv2 = qkv.copy()
        qkv2[5:12] += 10.0
        o2 = oracle.attention_ref_varlen(qkv2, cu, causal=causal, scale=0.5)
        assert np.array_equal(o[0:5], o2[0:5])


def test_varlen_empty_and_unit_sequences():
    lengths = [0, 1, 5, 0, 3, 1]
    cu = cu_seqlens_from_lengths(lengths)
    qkv = rand((int(cu[-1]), 3, 2, 4), 101)
    o = oracle.attention_ref_varlen(qkv, cu, causal=True, scale=0.9)
    # a length-1 sequence returns its own V; a causal first token returns its own V
    for s, L in enumerate(lengths):
        if L >= 1:
            a = cu[s]
            assert np.array_equal(o[a], qkv[a, 2])
    toks = [0, 6, 1, 8]
    o_rows = oracle.attention_ref_varlen_rows(qkv, cu, toks, causal=True, scale=0.9)
    assert np.array_equal(o_rows, o[toks])


def test_varlen_validation():
    qkv = rand((5, 3, 1, 4), 102)
    with pytest.raises(ValueError):
        oracle.attention_ref_varlen(qkv, [0, 3, 4], causal=False, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_ref_varlen(qkv, [1, 5], causal=False, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_ref_varlen(qkv[:, :2], [0, 5], causal=False, scale=1.0)


def test_dense_validation():
    q = rand((1, 3, 4, 8), 103)
    k = rand((1, 2, 4, 8), 104)
    with pytest.raises(ValueError):
        oracle.attention_ref(q, k, k, causal=False, scale=1.0)
    q = rand((1, 2, 4, 8), 105)
    k = rand((1, 2, 5, 8), 106)
    with pytest.raises(ValueError):
        oracle.attention_ref(q, k, k, causal=True, scale=1.0)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, causal, scale, shift=0):
    """Pure-Python loops with math.exp: no numpy arithmetic at all. With ``shift``, query i
    sees keys j <= i + shift under causal masking."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = [[[[0.0] * d for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(Nq):
                scores = []
                for j in range(Nk):
                    if causal and j > i + shift:
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += float(q[b, h, i, c]) * float(k[b, hk, j, c])
                    scores.append((j, sc * dot))
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                tot = sum(x for _, x in w)
                for c in range(d):
                    acc = 0.0
                    for j, x in w:
                        acc += x * float(v[b, hk, j, c])
                    out[b][h][i][c] = acc / tot
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(200 + seed)
    G = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    N = int(rng.integers(1, 9))
    d = int(rng.integers(1, 9))
    causal = bool(seed % 2)
    scale = float(rng.uniform(-2, 2))
    q = rng.standard_normal((2, Hkv * G, N, d))
    Nk = N if causal else int(rng.integers(1, 9))
    k = rng.standard_normal((2, Hkv, Nk, d))
    v = rng.standard_normal((2, Hkv, Nk, d))
    ref = brute_force(q, k, v, causal, scale)
    for variant in _variants_for(q, k):
        o = run_variant(variant, q, k, v, causal=causal, scale=scale)
        assert np.max(np.abs(o - ref)) < 1e-12, variant


# ---------------------------------------------------------------- online softmax

def online_softmax_emulation(q, k, v, causal, scale, BM, BN):
    """Tile-by-tile fp64 emulation of the streaming algorithm: running row max m, running
    row sum l and a rescaled accumulator, one K/V tile at a time (the online softmax of
    the FlashAttention-T best-practice notes and the FlashAttention-2 block loop of the
    xxqk.cn article, section 2.2). Test helper, not the oracle."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, Nq, d))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i0 in range(0, Nq, BM):
                rows = np.arange(i0, min(i0 + BM, Nq))
                m = np.full(rows.size, -np.inf)
                l = np.zeros(rows.size)
                acc = np.zeros((rows.size, d))
                last = Nk if not causal else min(Nk, rows[-1] + 1)
                for j0 in range(0, last, BN):
                    cols = np.arange(j0, min(j0 + BN, Nk))
                    s = sc * (q[b, h, rows] @ k[b, hk, cols].T)
                    if causal:
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m, s.max(axis=1))
                    alpha = np.exp(m - m_new)
                    p = np.exp(s - m_new[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, hk, cols]
                    m = m_new
                out[b, h, rows] = acc / l[:, None]
    return out


@pytest.mark.parametrize("BM,BN", [(4, 4), (3, 5), (8, 2), (16, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_equals_two_pass(BM, BN, causal):
    q = rand((1, 4, 13, 8), 300, 2.0)
    k = rand((1, 2, 13, 8), 301, 2.0)
    v = rand((1, 2, 13, 8), 302)
    ref = oracle.attention_ref(q, k, v, causal=causal, scale=0.6)
    emu = online_softmax_emulation(q, k, v, causal, 0.6, BM, BN)
    assert np.max(np.abs(ref - emu)) < 1e-12


# ---------------------------------------------------------------- inputs

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(400).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]   # ties
    ours = round_to_dtype(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)
    ours16 = round_to_dtype(x, "f16")
    ref16 = torch.from_numpy(x).to(torch.float16).float().numpy()
    assert np.array_equal(ours16, ref16)


def test_workload_recipes():
    c4 = CONFIGS["c4_bf16_varlen"]
    assert [int(x) for x in c4.lengths()] == C4_LENGTHS
    assert sum(C4_LENGTHS) == 25903
    rows = sampled_rows(32768)
    assert rows.size == 64 and len(set(rows.tolist())) == 64
    assert {0, 1, 2, 63, 64, 4095, 4096, 32766, 32767} <= set(rows.tolist())
    assert np.array_equal(rows, sampled_rows(32768))
    c1 = CONFIGS["c1_f32_dense"]
    q, k, v = c1.inputs()
    assert q.shape == (1, 2, 128, 64) and k.shape == (1, 2, 128, 64)
    q2, _, _ = dense_inputs(1, 2, 2, 128, 128, 64, seed=0, dtype="f32")
    assert np.array_equal(q, q2)
    assert abs(CONFIGS["c3_bf16_causal_gqa"].flops() - 549.89e9) / 549.89e9 < 1e-4
    assert abs(CONFIGS["c5_bf16_long_gqa"].flops() - 8.796e12) / 8.796e12 < 1e-3
    assert abs(c4.flops() - 249.34e9) / 249.34e9 < 1e-4


def test_short_workload_recipe():
    """The short cross-attention workload: 64 queries against 77 keys, 12 heads of 64
    channels, batch 256, non-causal; FLOPs and compulsory bytes as the bench reports them."""
    from workloads import SHORT_CONFIGS
    s1 = SHORT_CONFIGS["s1_bf16_short_cross"]
    assert (s1.batch, s1.heads_q, s1.heads_kv, s1.seqlen_q, s1.seqlen_k, s1.head_dim) == (256, 12, 12, 64, 77, 64)
    assert not s1.causal and s1.softmax_scale == 0.125
    assert s1.flops() == 4 * 64 * 12 * 256 * 64 * 77 == 3875536896
    assert s1.bytes_compulsory() == 2 * 64 * 256 * (2 * 12 * 64 + 2 * 12 * 77) == 110886912
    small = type(s1)("t", "bf16", 2, 4, 2, 5, 7, 8, False, seed=7)
    q, k, v = small.inputs()
    assert q.shape == (2, 4, 5, 8) and k.shape == (2, 2, 7, 8) and v.shape == (2, 2, 7, 8)
    q2, k2, v2 = dense_inputs(2, 4, 2, 5, 7, 8, seed=7, dtype="bf16")
    assert np.array_equal(q, q2) and np.array_equal(k, k2) and np.array_equal(v, v2)
    causal = type(s1)("t", "bf16", 1, 1, 1, 6, 6, 8, True, seed=7)
    assert causal.pairs() == 21


def test_config1_full_oracle_runs():
    c1 = CONFIGS["c1_f32_dense"]
    q, k, v = c1.inputs()
    o = oracle.attention_ref(q, k, v, causal=c1.causal, scale=c1.softmax_scale)
    assert o.shape == q.shape and np.all(np.isfinite(o))


# ---------------------------------------------------------------- decoding against a KV cache

@pytest.mark.parametrize("Nq", [1, 2, 5, 16])
def test_decode_tail_of_full_causal(Nq):
    """Decoding the last Nq positions against the whole cache reproduces the last Nq rows
    of causal attention over the full sequence."""
    rng = np.random.default_rng(300 + Nq)
    Nk, d, Hkv, G = 16, 8, 2, 2
    q_full = rng.standard_normal((2, Hkv * G, Nk, d))
    k = rng.standard_normal((2, Hkv, Nk, d))
    v = rng.standard_normal((2, Hkv, Nk, d))
    full = oracle.attention_ref(q_full, k, v, causal=True, scale=0.4)
    dec = oracle.attention_ref_decode(q_full[:, :, Nk - Nq:], k, v, causal=True, scale=0.4)
    np.testing.assert_allclose(dec, full[:, :, Nk - Nq:], rtol=0, atol=1e-12)


def test_decode_single_query_sees_whole_cache():
    rng = np.random.default_rng(311)
    q = rng.standard_normal((1, 4, 1, 16))
    k = rng.standard_normal((1, 2, 37, 16))
    v = rng.standard_normal((1, 2, 37, 16))
    a = oracle.attention_ref_decode(q, k, v, causal=True, scale=0.25)
    b = oracle.attention_ref(q, k, v, causal=False, scale=0.25)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_decode_noncausal_is_plain_attention():
    rng = np.random.default_rng(312)
    q = rng.standard_normal((2, 2, 3, 8))
    k = rng.standard_normal((2, 1, 9, 8))
    v = rng.standard_normal((2, 1, 9, 8))
    np.testing.assert_allclose(oracle.attention_ref_decode(q, k, v, causal=False, scale=1.3),
                               oracle.attention_ref(q, k, v, causal=False, scale=1.3),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_decode_brute_force_tiny(seed):
    rng = np.random.default_rng(320 + seed)
    Hkv, G = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Nk = int(rng.integers(1, 9))
    Nq = int(rng.integers(1, Nk + 1))
    d = int(rng.integers(1, 7))
    scale = float(rng.uniform(-2, 2))
    q = rng.standard_normal((1, Hkv * G, Nq, d))
    k = rng.standard_normal((1, Hkv, Nk, d))
    v = rng.standard_normal((1, Hkv, Nk, d))
    ref = brute_force(q, k, v, True, scale, shift=Nk - Nq)
    got = oracle.attention_ref_decode(q, k, v, causal=True, scale=scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_decode_validation():
    q = np.zeros((1, 1, 5, 4))
    k = np.zeros((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle.attention_ref_decode(q, k, k, causal=True, scale=1.0)
    oracle.attention_ref_decode(q, k, k, causal=False, scale=1.0)   # non-causal: any Nq


# ---------------------------------------------------------------- log-sum-exp and gradients

def test_lse_single_key_and_uniform_scores():
    rng = np.random.default_rng(401)
    q = rng.standard_normal((1, 2, 3, 5))
    k = rng.standard_normal((1, 1, 1, 5))
    lse = oracle.attention_ref_lse(q, k, k, causal=False, scale=0.7)
    sc = float(np.float32(0.7))
    np.testing.assert_allclose(lse[0, :, :], sc * (q[0] @ k[0, 0, 0]), rtol=0, atol=1e-13)
    q = rng.standard_normal((1, 1, 6, 4))
    k = rng.standard_normal((1, 1, 6, 4))
    lse = oracle.attention_ref_lse(q, k, k, causal=True, scale=0.0)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 7)), rtol=0, atol=1e-13)


def test_lse_brute_force():
    rng = np.random.default_rng(402)
    q = rng.standard_normal((1, 2, 4, 3))
    k = rng.standard_normal((1, 2, 5, 3))
    got = oracle.attention_ref_lse(q, k, k, causal=False, scale=1.1)
    sc = float(np.float32(1.1))
    for h in range(2):
        for i in range(4):
            tot = 0.0
            for j in range(5):
                dot = sum(float(q[0, h, i, c]) * float(k[0, h, j, c]) for c in range(3))
                tot += math.exp(sc * dot)
            assert abs(got[0, h, i] - math.log(tot)) < 1e-12


def _finite_difference_grads(q, k, v, do, causal, scale, h=1e-6):
    """Central differences of L = sum(O * do) through the forward oracle."""
    def loss(q_, k_, v_):
        return float(np.sum(oracle.attention_ref(q_, k_, v_, causal=causal, scale=scale) * do))
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    rng = np.random.default_rng(410 + causal)
    B, Hkv, G, N, d = 1, 1, 2, 4, 3
    q = rng.standard_normal((B, Hkv * G, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hkv * G, N, d))
    dq, dk, dv = oracle.attention_ref_bwd(q, k, v, do, causal=causal, scale=0.8)
    fq, fk, fv = _finite_difference_grads(q, k, v, do, causal, 0.8)
    np.testing.assert_allclose(dq, fq, rtol=0, atol=1e-7)
    np.testing.assert_allclose(dk, fk, rtol=0, atol=1e-7)
    np.testing.assert_allclose(dv, fv, rtol=0, atol=1e-7)


def test_backward_single_key():
    """One key: P = 1 everywhere, so dV = sum of dO over the rows and heads that read it,
    and Q, K get no gradient."""
    rng = np.random.default_rng(420)
    q = rng.standard_normal((1, 4, 3, 5))
    k = rng.standard_normal((1, 2, 1, 5))
    v = rng.standard_normal((1, 2, 1, 5))
    do = rng.standard_normal((1, 4, 3, 5))
    dq, dk, dv = oracle.attention_ref_bwd(q, k, v, do, causal=False, scale=0.5)
    np.testing.assert_allclose(dq, 0, atol=1e-13)
    np.testing.assert_allclose(dk, 0, atol=1e-13)
    np.testing.assert_allclose(dv[0, 0, 0], do[0, 0:2].sum(axis=(0, 1)), atol=1e-13)
    np.testing.assert_allclose(dv[0, 1, 0], do[0, 2:4].sum(axis=(0, 1)), atol=1e-13)


# ---------------------------------------------------------------- score modifiers

def _mods_inputs(lengths, H, d, seed):
    rng = np.random.default_rng(seed)
    cu = cu_seqlens_from_lengths(lengths)
    return rng.standard_normal((int(cu[-1]), 3, H, d)), cu


@pytest.mark.parametrize("causal", [False, True])
def test_mods_defaults_are_plain_varlen(causal):
    qkv, cu = _mods_inputs([5, 9, 1, 0, 4], 2, 4, 501)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=causal, scale=0.5)
    ref = oracle.attention_ref_varlen(qkv, cu, causal=causal, scale=0.5)
    np.testing.assert_allclose(got, ref, atol=1e-13)


def test_window_unbounded_left_zero_right_is_causal():
    qkv, cu = _mods_inputs([7, 3, 12], 3, 5, 502)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=False, scale=0.3, window=(-1, 0))
    ref = oracle.attention_ref_varlen(qkv, cu, causal=True, scale=0.3)
    np.testing.assert_allclose(got, ref, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_returns_own_value(causal):
    """A (0, 0) window leaves each query only its own key: O = V row for row, exactly."""
    qkv, cu = _mods_inputs([6, 1, 9], 2, 3, 503)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=causal, scale=0.7, window=(0, 0),
                                           softcap=2.0, alibi_slopes=[0.5, 0.25])
    np.testing.assert_array_equal(got, qkv[:, 2])


@pytest.mark.parametrize("window", [(3, 1), (0, 4), (2, -1), (-1, 2)])
def test_window_identical_keys_mean(window):
    """Equal keys give equal scores, so each query averages V over its window: keys
    max(0, i - left) .. min(L - 1, i + right); with V = identity that is a box row."""
    L = 10
    qkv = np.zeros((L, 3, 1, L))
    qkv[:, 0, 0] = np.random.default_rng(511).standard_normal((L, L))
    qkv[:, 1, 0] = np.random.default_rng(512).standard_normal(L)[None, :]
    qkv[:, 2, 0] = np.eye(L)
    cu = np.array([0, L], dtype=np.int32)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=False, scale=0.9, window=window)
    left, right = window
    ref = np.zeros((L, L))
    for i in range(L):
        lo = 0 if left < 0 else max(0, i - left)
        hi = L - 1 if right < 0 else min(L - 1, i + right)
        ref[i, lo:hi + 1] = 1.0 / (hi - lo + 1)
    np.testing.assert_allclose(got[:, 0], ref, atol=1e-13)


def _brute_mods(qkv, cu, causal, scale, window, softcap, slopes):
    """Element by element in plain Python (math.exp / math.tanh), straight from the reading
    of the modifiers."""
    T, _, H, d = qkv.shape
    left, right = window
    sl = None if slopes is None else np.asarray(slopes, dtype=np.float32).reshape(-1, H)
    out = np.zeros((T, H, d))
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            slope = 0.0 if sl is None else float(sl[s if sl.shape[0] > 1 else 0, h])
            for i in range(e - a):
                xs, vs = [], []
                for j in range(e - a):
                    if causal and j > i:
                        continue
                    if left >= 0 and j < i - left:
                        continue
                    if right >= 0 and j > i + right:
                        continue
                    x = scale * sum(qkv[a + i, 0, h, c] * qkv[a + j, 1, h, c] for c in range(d))
                    if softcap > 0:
                        x = softcap * math.tanh(x / softcap)
                    x -= slope * abs(i - j)
                    xs.append(x)
                    vs.append(qkv[a + j, 2, h])
                mx = max(xs)
                ws = [math.exp(x - mx) for x in xs]
                out[a + i, h] = sum(w * v for w, v in zip(ws, vs)) / sum(ws)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_mods_brute_force_tiny(seed):
    rng = np.random.default_rng(600 + seed)
    lengths = list(rng.integers(0, 8, size=3))
    H, d = 2, 3
    qkv, cu = _mods_inputs(lengths, H, d, 610 + seed)
    qkv *= 2.0
    causal = bool(seed % 2)
    window = (int(rng.integers(-1, 4)), int(rng.integers(-1, 4)))
    if causal and window[1] > 0:
        window = (window[0], 0)
    softcap = [0.0, 1.5, 4.0][seed % 3]
    slopes = None if seed % 3 == 1 else (rng.uniform(0, 1, size=(3, H)).astype(np.float32)
                                         if seed % 2 else rng.uniform(0, 1, size=H).astype(np.float32))
    scale = 0.6
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=causal, scale=scale, window=window,
                                           softcap=softcap, alibi_slopes=slopes)
    ref = _brute_mods(qkv, cu, causal, float(np.float32(scale)), window, softcap, slopes)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_causal_alibi_is_a_key_bias():
    """Under causal masking -slope * (i - j) = slope * j - slope * i, and a per-row constant
    leaves the softmax unchanged: ALiBi equals plain causal attention with one extra
    dimension carrying q = 1, k = slope * j / scale."""
    L, H, d, scale = 11, 2, 4, 0.5
    qkv, cu = _mods_inputs([L], H, d, 504)
    slopes = np.array([0.375, 1.25], dtype=np.float32)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=True, scale=scale, alibi_slopes=slopes)
    q = np.concatenate([qkv[:, 0], np.ones((L, H, 1))], axis=2).transpose(1, 0, 2)[None]
    j = np.arange(L, dtype=np.float64)[:, None, None]
    kx = (j * slopes.astype(np.float64)[None, :, None]) / scale
    k = np.concatenate([qkv[:, 1], np.broadcast_to(kx, (L, H, 1))], axis=2).transpose(1, 0, 2)[None]
    v = np.concatenate([qkv[:, 2], np.zeros((L, H, 1))], axis=2).transpose(1, 0, 2)[None]
    ref = oracle.attention_ref(q, k, v, causal=True, scale=scale)[0].transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref[..., :d], atol=1e-12)


def test_alibi_identical_keys_closed_form():
    """Equal keys give equal scores, so non-causal ALiBi weights are exp(-slope |i - j|)
    normalised; with V = identity, O[i] is that weight row."""
    L, slope = 9, 0.8
    qkv = np.zeros((L, 3, 1, L))
    qkv[:, 0, 0] = np.random.default_rng(505).standard_normal((L, L))
    qkv[:, 1, 0] = np.random.default_rng(506).standard_normal(L)[None, :]
    qkv[:, 2, 0] = np.eye(L)
    cu = np.array([0, L], dtype=np.int32)
    got = oracle.attention_ref_varlen_mods(qkv, cu, causal=False, scale=0.4,
                                           alibi_slopes=np.array([slope], dtype=np.float32))
    s32 = float(np.float32(slope))
    w = np.exp(-s32 * np.abs(np.arange(L)[:, None] - np.arange(L)[None, :]))
    np.testing.assert_allclose(got[:, 0], w / w.sum(axis=1, keepdims=True), atol=1e-13)


def test_softcap_limits():
    """A cap far above the scores changes nothing; scores far above the cap saturate at
    +-cap, so the weights depend only on the sign of q.k."""
    qkv, cu = _mods_inputs([10], 2, 4, 507)
    plain = oracle.attention_ref_varlen(qkv, cu, causal=True, scale=0.5)
    big = oracle.attention_ref_varlen_mods(qkv, cu, causal=True, scale=0.5, softcap=1e20)
    np.testing.assert_allclose(big, plain, atol=1e-13)
    cap = 3.0
    sat = oracle.attention_ref_varlen_mods(qkv, cu, causal=False, scale=1e12, softcap=cap)
    for h in range(2):
        sign = np.sign(qkv[:, 0, h] @ qkv[:, 1, h].T)
        w = np.exp(cap * sign)
        ref = (w @ qkv[:, 2, h]) / w.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(sat[:, h], ref, atol=1e-12)


def test_mods_tokens_subset_matches_full():
    qkv, cu = _mods_inputs([13, 4, 20], 2, 5, 508)
    kw = dict(causal=True, scale=0.45, window=(5, 0), softcap=2.5, alibi_slopes=[0.1, 0.7])
    full = oracle.attention_ref_varlen_mods(qkv, cu, **kw)
    toks = np.random.default_rng(509).permutation(37)[:15]
    part = oracle.attention_ref_varlen_mods(qkv, cu, tokens=toks, **kw)
    np.testing.assert_array_equal(part, full[toks])


def test_mods_validation():
    qkv, cu = _mods_inputs([4], 2, 3, 510)
    for kw in (dict(window=(-2, 0)), dict(window=(0, -3)), dict(softcap=-1.0),
               dict(softcap=float("inf")), dict(alibi_slopes=np.ones(3)),
               dict(alibi_slopes=np.ones((2, 2)))):
        with pytest.raises(ValueError):
            oracle.attention_ref_varlen_mods(qkv, cu, causal=False, scale=1.0, **kw)


# ---------------------------------------------------------------- mutation checks

def _pins_pass():
    """Run a compact set of the pins above; return False if any of them fails."""
    checks = [
        lambda: test_causal_row0_is_v0("full"),
        lambda: test_identical_keys_give_mean_of_v("full", True),
        lambda: test_scale_zero_gives_mean_of_allowed_v("full", True),
        lambda: test_two_keys_closed_form("full"),
        lambda: test_gqa_equals_repeat_interleaved_kv(),
        lambda: test_brute_force_tiny(1),
        lambda: test_brute_force_tiny(2),
        lambda: test_dominant_key("full", False),
        lambda: test_varlen_golden_cu_seqlens_example(),
        lambda: test_single_key_returns_v("full", 0.125),
        lambda: test_decode_tail_of_full_causal(5),
        lambda: test_decode_brute_force_tiny(0),
        lambda: test_backward_matches_finite_differences(True),
        lambda: test_lse_single_key_and_uniform_scores(),
        lambda: test_window_zero_returns_own_value(False),
        lambda: test_window_identical_keys_mean((3, 1)),
        lambda: test_mods_brute_force_tiny(0),
        lambda: test_mods_brute_force_tiny(3),
        lambda: test_alibi_identical_keys_closed_form(),
        lambda: test_softcap_limits(),
    ]
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, ValueError, FloatingPointError):
            return False
    return True


def test_pins_accept_the_oracle():
    assert _pins_pass()


def _mut_softmax_no_normalise(S, V):
    m = S.max(axis=1, keepdims=True)
    return np.exp(S - m) @ V


def _mut_softmax_wrong_axis(S, V):
    S2 = np.where(np.isinf(S), -1e300, S)
    m = S2.max(axis=0, keepdims=True)
    P = np.exp(S2 - m)
    return (P @ V) / P.sum(axis=0, keepdims=True).T[: S.shape[0]].reshape(-1, 1)


def _mut_softmax_sign(S, V):
    m = (-S).max(axis=1, keepdims=True)
    P = np.exp(-S - m)
    return (P @ V) / P.sum(axis=1, keepdims=True)


def _window_swapped(rows, n, left, right):
    rows = np.asarray(rows)[:, None]
    j = np.arange(n)[None, :]
    out = np.zeros((rows.shape[0], n), dtype=bool)
    if right >= 0:
        out |= j < rows - right
    if left >= 0:
        out |= j > rows + left
    return out


MUTANTS = {
    "kv_head_modulo": ("_kv_head", lambda hq, G: hq % max(1, G)),
    "causal_mask_includes_diagonal": ("_causal_masked",
                                      lambda rows, n: np.arange(n)[None, :] >= np.asarray(rows)[:, None]),
    "causal_mask_transposed": ("_causal_masked",
                               lambda rows, n: np.arange(n)[None, :] < np.asarray(rows)[:, None]),
    "no_normalisation": ("_softmax_rows_times_v", _mut_softmax_no_normalise),
    "softmax_wrong_axis": ("_softmax_rows_times_v", _mut_softmax_wrong_axis),
    "softmax_sign_flipped": ("_softmax_rows_times_v", _mut_softmax_sign),
    "scale_inverted": ("_scale64", lambda s: 1.0 / float(np.float32(s)) if s else 0.0),
    "scale_dropped": ("_scale64", lambda s: 1.0),
    "softmax_backward_no_rowsum": ("_softmax_backward", lambda P, dP: P * dP),
    "lse_without_max_shift": ("_lse_rows", lambda S: np.log(np.exp(S).sum(axis=1)) + 1e-3),
    "window_edge_key_masked": ("_window_masked",
                               lambda rows, n, left, right: (
                                   (np.arange(n)[None, :] <= np.asarray(rows)[:, None] - left) if left >= 0
                                   else np.zeros((len(rows), n), bool)) | (
                                   (np.arange(n)[None, :] > np.asarray(rows)[:, None] + right) if right >= 0
                                   else np.zeros((len(rows), n), bool))),
    "window_sides_swapped": ("_window_masked", _window_swapped),
    "softcap_factor_dropped": ("_softcap", lambda S, cap: np.tanh(S / cap)),
    "softcap_inner_scale_dropped": ("_softcap", lambda S, cap: cap * np.tanh(S)),
    "alibi_sign_flipped": ("_alibi_bias",
                           lambda rows, n, slope: slope * np.abs(np.asarray(rows)[:, None] - np.arange(n)[None, :])),
    "alibi_without_abs": ("_alibi_bias",
                          lambda rows, n, slope: -slope * (np.asarray(rows)[:, None] - np.arange(n)[None, :]).astype(float)),
    "decode_mask_top_left": ("_decode_masked",
                             lambda nq, nk: np.arange(nk)[None, :] > np.arange(nq)[:, None]),
    "decode_mask_includes_next_key": ("_decode_masked",
                                      lambda nq, nk: np.arange(nk)[None, :] > (np.arange(nq) + nk - nq + 1)[:, None]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oracle_mod, attr, fn)
    assert not _pins_pass(), f"no pin caught mutant {name}"
