"""GPU parity of the attention backward (aule_attn_fwd_lse + aule_attn_bwd, through the C-ABI
library) against the CPU fp64 oracle's attention_ref_lse and attention_ref_bwd on the same
seeded, dtype-rounded inputs.

Bars. The per-row log-sum-exp is fp32, but the 16-bit forward sums the probabilities after
rounding them to the dtype (the same P that multiplies V, so that O is a convex combination of
V rows), which moves the sum by at most the unit roundoff u of the dtype relative and the log
by at most about u: |err| <= (u + 2e-5) * max(1, |lse|), with u = 2^-8 (bf16), 2^-11 (fp16)
and 0 (fp32), 2e-5 covering the fp32 sums and the exp2/log2 instructions.
The gradients are compared on the max abs error over every element, divided by
max(1, max |reference|) of that tensor, against the forward's bars: 1e-5 for fp32, 2e-3 for
fp16 and 1e-2 for bf16. Each gradient is a sum of products of rounded inputs with O (itself
rounded to the dtype by the forward, which enters through D_i = do_i . o_i) and with P (from
the lse above), then rounded once to the dtype: the output rounding alone is 2^-11 (fp16) /
2^-8 (bf16) relative to the largest element, and the O and lse terms add a few more unit
roundoffs, which the 16-bit bars (about 4 u) cover."""
import math

import numpy as np
import pytest

import oracle
import tiled_attention_02_amd as aule
from workloads import BWD_CONFIGS, dense_inputs, output_grad

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GTOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
TOL_F32_OUT = 1e-5   # the forward's fp32 bar on O
LSE_TOL = {"f32": 2e-5, "f16": 2.0 ** -11 + 2e-5, "bf16": 2.0 ** -8 + 2e-5}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aule.load_library()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=TDT[dtype])


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref))) / max(1.0, float(np.max(np.abs(ref))))


def run(B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale=None, seed=0):
    print(f"bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"scale={scale} seed={seed}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, dtype=dtype)
    do = output_grad(q.shape, seed=seed, dtype=dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    tq, tk, tv, tdo = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    o, lse = aule.flash_attention(tq, tk, tv, causal=causal, scale=sc, return_lse=True)
    dq, dk, dv = aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=causal, scale=sc)
    torch.cuda.synchronize()
    return (q, k, v, do, sc), (host(o), host(lse), host(dq), host(dk), host(dv))


def check(B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale=None, seed=0):
    (q, k, v, do, sc), (o, lse, dq, dk, dv) = run(B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale, seed)
    ref_lse = oracle.attention_ref_lse(q, k, v, causal=causal, scale=sc)
    assert np.all(np.isfinite(lse))
    lse_err = float(np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))))
    assert lse_err <= LSE_TOL[dtype], f"lse err {lse_err}"
    rdq, rdk, rdv = oracle.attention_ref_bwd(q, k, v, do, causal=causal, scale=sc)
    errs = {}
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        assert np.all(np.isfinite(got)), name
        errs[name] = rel_err(got, ref)
    print("  errors", errs, flush=True)
    for name, e in errs.items():
        assert e <= GTOL[dtype], f"{name} relative err {e} > {GTOL[dtype]}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 31, 100, 257])
def test_bwd_shapes(dtype, causal, N):
    check(2, 4, 2, N, N, 64, dtype, causal, seed=N)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [8, 40, 64, 72, 96, 128])
def test_bwd_head_dims(dtype, d):
    check(1, 4, 1, 77, 77, d, dtype, True, seed=d)


@pytest.mark.parametrize("Nq,Nk", [(40, 70), (70, 40), (1, 300), (300, 1)])
def test_bwd_cross_lengths(Nq, Nk):
    check(1, 6, 2, Nq, Nk, 128, "bf16", False, seed=Nq * 7 + Nk)


@pytest.mark.parametrize("G", [1, 2, 8, 32])
def test_bwd_gqa_groups(G):
    check(1, G * 2, 2, 96, 96, 128, "bf16", True, seed=G)


@pytest.mark.parametrize("which", ["zero", "neg", "big"])
def test_bwd_scales(which):
    sc = {"zero": 0.0, "neg": -0.3, "big": 0.5}[which]
    check(1, 2, 2, 65, 65, 64, "f32", True, scale=sc, seed=3)
    check(1, 2, 1, 65, 65, 64, "f16", False, scale=sc, seed=4)


def test_bwd_training_shape_sampled():
    """bf16 causal GQA at a training length (B1 Hq32 Hkv8 N2048 d128): every gradient row
    of two query heads and their shared key/value head against the oracle, which needs only
    those heads (a key/value head's gradient is the sum over its own query group)."""
    B, Hq, Hkv, N, d = 1, 32, 8, 2048, 128
    (q, k, v, do, sc), (o, lse, dq, dk, dv) = run(B, Hq, Hkv, N, N, d, "bf16", True, seed=77)
    hk = 5
    sl = slice(hk * 4, hk * 4 + 4)                     # the 4 query heads sharing kv head 5
    rdq, rdk, rdv = oracle.attention_ref_bwd(q[:, sl], k[:, hk:hk + 1], v[:, hk:hk + 1],
                                             do[:, sl], causal=True, scale=sc)
    errs = {"dq": rel_err(dq[:, sl], rdq), "dk": rel_err(dk[:, hk:hk + 1], rdk),
            "dv": rel_err(dv[:, hk:hk + 1], rdv)}
    print("  errors", errs, flush=True)
    for name, e in errs.items():
        assert e <= GTOL["bf16"], f"{name} relative err {e}"
    ref_lse = oracle.attention_ref_lse(q[:, sl], k[:, hk:hk + 1], v[:, hk:hk + 1], causal=True,
                                       scale=sc)
    assert float(np.max(np.abs(lse[:, sl] - ref_lse) / np.maximum(1, np.abs(ref_lse)))) <= \
        LSE_TOL["bf16"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_no_queries_gives_zero_kv_gradients(dtype):
    """seqlen_q = 0 against 50 keys (non-causal): dK and dV are written as zeros."""
    k = torch.randn(1, 2, 50, 64, device="cuda", dtype=dtype)
    q = torch.empty(1, 4, 0, 64, device="cuda", dtype=dtype)
    lse = torch.empty(1, 4, 0, device="cuda", dtype=torch.float32)
    dq, dk, dv = aule.flash_attention_backward(q, k, k.clone(), q, q.clone(), lse, causal=False)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and bool((dk == 0).all()) and bool((dv == 0).all())


def test_f32_slice_past_32bit_offsets():
    """An fp32 (batch, head) slice of 1 GiB or more (2^21 + 32 keys at head_dim 128) is past the
    fp32 matrix-core kernels' 32-bit buffer offsets, so the forward and the backward take the
    vector-ALU kernels: output, LSE and gradients against the oracle."""
    Nk = (1 << 21) + 32
    (q, k, v, do, sc), (o, lse, dq, dk, dv) = run(1, 2, 1, 8, Nk, 128, "f32", False, seed=91)
    assert np.max(np.abs(o - oracle.attention_ref(q, k, v, causal=False, scale=sc))) <= TOL_F32_OUT
    ref_lse = oracle.attention_ref_lse(q, k, v, causal=False, scale=sc)
    assert float(np.max(np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse)))) <= LSE_TOL["f32"]
    rdq, rdk, rdv = oracle.attention_ref_bwd(q, k, v, do, causal=False, scale=sc)
    errs = {"dq": rel_err(dq, rdq), "dk": rel_err(dk, rdk), "dv": rel_err(dv, rdv)}
    print("  errors", errs, flush=True)
    for name, e in errs.items():
        assert e <= GTOL["f32"], f"{name} relative err {e}"


def test_bwd_f32_matrix_core_shapes():
    """fp32 gradients on the fp32 matrix-core kernels: head_dim 128 over several 128-key
    blocks and 32-row tiles with ragged ends (causal and not), GQA groups of 4 and 8, cross
    lengths both ways, a padded head_dim."""
    check(1, 8, 2, 300, 300, 128, "f32", True, seed=81)
    check(2, 4, 1, 200, 200, 128, "f32", False, seed=82)
    check(1, 4, 2, 130, 270, 96, "f32", False, seed=83)
    check(1, 4, 2, 270, 130, 128, "f32", False, seed=84)
    check(1, 16, 2, 150, 150, 64, "f32", True, seed=85)


def test_bwd_non_default_stream():
    q, k, v = dense_inputs(1, 2, 1, 70, 70, 64, seed=9, dtype="f16")
    do = output_grad(q.shape, seed=9, dtype="f16")
    tq, tk, tv, tdo = dev(q, "f16"), dev(k, "f16"), dev(v, "f16"), dev(do, "f16")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = aule.flash_attention(tq, tk, tv, causal=True, return_lse=True)
        dq, dk, dv = aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=True)
    s.synchronize()
    rdq, rdk, rdv = oracle.attention_ref_bwd(q, k, v, do, causal=True, scale=1 / 8)
    for got, ref in ((dq, rdq), (dk, rdk), (dv, rdv)):
        assert rel_err(host(got), ref) <= GTOL["f16"]


def test_bwd_b1_shape_groups():
    """The benchmarked backward shape (B4 Hq32 Hkv8 N4096 d128, bf16 causal GQA): every
    gradient element of eight (batch, kv head) groups, one per kv head and spread over the
    batch, against the oracle (a kv head's gradient sums over its own query group only)."""
    c = BWD_CONFIGS["b1_bf16_causal_gqa_bwd"]
    q, k, v = c.inputs()
    do = c.grad()
    sc = c.softmax_scale
    tq, tk, tv, tdo = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(do, "bf16")
    o, lse = aule.flash_attention(tq, tk, tv, causal=True, scale=sc, return_lse=True)
    dq, dk, dv = aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=True, scale=sc)
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    G = c.heads_q // c.heads_kv
    for hk in range(c.heads_kv):
        b = hk % c.batch
        sl = slice(hk * G, hk * G + G)
        rdq, rdk, rdv = oracle.attention_ref_bwd(q[b:b + 1, sl], k[b:b + 1, hk:hk + 1],
                                                 v[b:b + 1, hk:hk + 1], do[b:b + 1, sl],
                                                 causal=True, scale=sc)
        errs = {"dq": rel_err(dq[b:b + 1, sl], rdq), "dk": rel_err(dk[b:b + 1, hk:hk + 1], rdk),
                "dv": rel_err(dv[b:b + 1, hk:hk + 1], rdv)}
        print(f"  b={b} hk={hk} errors {errs}", flush=True)
        for name, e in errs.items():
            assert e <= GTOL["bf16"], f"{name} relative err {e} (b={b}, hk={hk})"


def test_bwd_grouped_walk_noncausal():
    """Non-causal bf16 at head_dim 128 with 32 (batch, kv head) groups of 16 key blocks
    (B4 Hq8 Hkv8 N4096): the dK / dV passes give each XCD two groups at a time, the second
    pair walking the query tiles upwards. Every gradient element of one group from the first
    pair (b=0, kv head 3) and one from the second (b=3, kv head 5) against the oracle."""
    B, Hq, Hkv, N, d = 4, 8, 8, 4096, 128
    (q, k, v, do, sc), (o, lse, dq, dk, dv) = run(B, Hq, Hkv, N, N, d, "bf16", False, seed=21)
    for b, hk in ((0, 3), (3, 5)):
        rdq, rdk, rdv = oracle.attention_ref_bwd(q[b:b + 1, hk:hk + 1], k[b:b + 1, hk:hk + 1],
                                                 v[b:b + 1, hk:hk + 1], do[b:b + 1, hk:hk + 1],
                                                 causal=False, scale=sc)
        errs = {"dq": rel_err(dq[b:b + 1, hk:hk + 1], rdq), "dk": rel_err(dk[b:b + 1, hk:hk + 1], rdk),
                "dv": rel_err(dv[b:b + 1, hk:hk + 1], rdv)}
        print(f"  b={b} hk={hk} errors {errs}", flush=True)
        for name, e in errs.items():
            assert e <= GTOL["bf16"], f"{name} relative err {e} (b={b}, hk={hk})"


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal", [
    (2, 8, 2, 517, 128, "bf16", True),      # key blocks slowest, ragged tiles
    (4, 8, 8, 4096, 128, "bf16", False),    # the grouped walk (both directions)
    (1, 8, 2, 300, 64, "f16", True),
    (1, 4, 2, 270, 128, "f32", True),
])
def test_bwd_deterministic_and_fully_written(B, Hq, Hkv, N, d, dtype, causal):
    """Two backward calls on the same inputs give bitwise equal gradients (no atomics, a
    fixed summation order), and every element of gradient buffers prefilled with NaN is
    written."""
    print(f"bwd determinism B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} causal={causal}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, N, N, d, seed=57, dtype=dtype)
    do = output_grad(q.shape, seed=57, dtype=dtype)
    tq, tk, tv, tdo = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    o, lse = aule.flash_attention(tq, tk, tv, causal=causal, return_lse=True)
    runs = []
    for _ in range(2):
        grads = tuple(torch.full_like(t, float("nan")) for t in (tq, tk, tv))
        aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=causal, grads=grads)
        runs.append(grads)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), runs[0], runs[1]):
        assert torch.isfinite(a).all(), f"{name} not fully written"
        assert torch.equal(a, b), f"{name} differs between calls"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_guard_regions_untouched(dtype):
    """Each gradient buffer sits inside a larger allocation with 256 guard elements on each
    side: the backward (the D pre-pass writes into dq's rows) touches none of them, and the
    gradients equal those written into plain buffers."""
    B, Hq, Hkv, N, d = 1, 4, 2, 333, 128
    print(f"bwd guards {dtype}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, N, N, d, seed=61, dtype=dtype)
    do = output_grad(q.shape, seed=61, dtype=dtype)
    tq, tk, tv, tdo = dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(do, dtype)
    o, lse = aule.flash_attention(tq, tk, tv, causal=True, return_lse=True)
    ref = aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=True)
    G = 256
    bufs, views = [], []
    for t in (tq, tk, tv):
        big = torch.full((t.numel() + 2 * G,), 7.0, dtype=t.dtype, device=t.device)
        bufs.append(big)
        views.append(big[G:G + t.numel()].view(t.shape))
    aule.flash_attention_backward(tq, tk, tv, o, tdo, lse, causal=True, grads=tuple(views))
    torch.cuda.synchronize()
    for name, big, view, r in zip(("dq", "dk", "dv"), bufs, views, ref):
        assert bool((big[:G] == 7.0).all()) and bool((big[-G:] == 7.0).all()), f"{name} guard touched"
        assert torch.equal(view, r), f"{name} differs from the plain-buffer call"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_autograd_sum_backward(dtype):
    """flash_attention recorded for autograd: out.sum().backward() (dO = 1) fills q.grad,
    k.grad and v.grad with the oracle's gradients (GQA: a kv head sums its query group)."""
    B, Hq, Hkv, N, d = 2, 8, 2, 256, 64
    q, k, v = dense_inputs(B, Hq, Hkv, N, N, d, seed=91, dtype=dtype)
    tq, tk, tv = (dev(x, dtype).requires_grad_(True) for x in (q, k, v))
    out = aule.flash_attention(tq, tk, tv, causal=True)
    assert out.grad_fn is not None
    out.sum().backward()
    torch.cuda.synchronize()
    sc = 1.0 / math.sqrt(d)
    ref_o = oracle.attention_ref(q, k, v, causal=True, scale=sc)
    assert rel_err(host(out.detach()), ref_o) <= GTOL[dtype]
    rdq, rdk, rdv = oracle.attention_ref_bwd(q, k, v, np.ones(q.shape), causal=True, scale=sc)
    for name, got, ref in (("dq", tq.grad, rdq), ("dk", tk.grad, rdk), ("dv", tv.grad, rdv)):
        assert got is not None and got.dtype == TDT[dtype], name
        e = rel_err(host(got), ref)
        print(f"  autograd {dtype} {name} err {e:.3e}", flush=True)
        assert e <= GTOL[dtype], f"{name} relative err {e}"


def test_autograd_no_grad_and_lse():
    """Without requires_grad (or under no_grad) the call records nothing; with return_lse the
    log-sum-exp comes back non-differentiable next to a differentiable output."""
    q, k, v = dense_inputs(1, 2, 2, 64, 64, 64, seed=92, dtype="bf16")
    tq, tk, tv = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    assert aule.flash_attention(tq, tk, tv).grad_fn is None
    tq.requires_grad_(True)
    with torch.no_grad():
        assert aule.flash_attention(tq, tk, tv).grad_fn is None
    o, lse = aule.flash_attention(tq, tk, tv, return_lse=True)
    assert o.grad_fn is not None and not lse.requires_grad
    with pytest.raises(ValueError):
        aule.flash_attention(tq, tk, tv, out=torch.empty_like(tq))
