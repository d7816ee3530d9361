"""GPU parity of the short-sequence path (dense fp16/bf16, at most 128 keys): the HIP kernel
through the C-ABI against the CPU fp64 oracle on the same seeded, dtype-rounded inputs.

Shapes with at most 128 keys and at most 16 (query head, 32-row block) items per kv head
take the short-sequence kernel; the rest (e.g. 8 query heads per kv head at 128 rows)
take the tiled kernel, and both are checked here at the forward's bars (2e-3 fp16, 1e-2
bf16, max abs error over every element).
"""
import math

import numpy as np
import pytest

import oracle
import tiled_attention_02_amd as aule
from workloads import SHORT_CONFIGS, dense_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 1e-2}
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aule.load_library()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=TDT[dtype])


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale=None, seed=0, stream=None, rel=False):
    """rel: compare |got - ref| / max(1, |ref|) per element. The bars are stated for O(1)
    outputs; above the standard scale the softmax sharpens towards single keys, |O| reaches
    |V| (about 3.5 here) and rounding O to the dtype alone moves it by u|O|."""
    print(f"short B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"scale={scale} seed={seed}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, dtype=dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.full((B, Hq, Nq, d), float("nan"), dtype=TDT[dtype], device="cuda")
    if stream is None:
        aule.flash_attention(dev(q, dtype), dev(k, dtype), dev(v, dtype), causal=causal, scale=sc,
                             out=out)
    else:
        qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            aule.flash_attention(qd, kd, vd, causal=causal, scale=sc, out=out)
        stream.synchronize()
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(np.isfinite(got)), "output not fully written"
    ref = oracle.attention_ref(q, k, v, causal=causal, scale=sc)
    diff = np.abs(got - ref)
    if rel:
        diff = diff / np.maximum(1.0, np.abs(ref))
    err = float(np.max(diff))
    assert err <= TOL[dtype], f"max {'rel' if rel else 'abs'} err {err} > {TOL[dtype]}"
    return err


def test_s1_short_cross_full():
    """The diffusion cross-attention workload in full: 256 x 12 heads, 64 queries, 77 keys."""
    c = SHORT_CONFIGS["s1_bf16_short_cross"]
    print(f"workload {c.name}", flush=True)
    q, k, v = c.inputs()
    out = aule.flash_attention(dev(q, c.dtype), dev(k, c.dtype), dev(v, c.dtype), causal=c.causal,
                               scale=c.softmax_scale)
    torch.cuda.synchronize()
    got = host(out)
    ref = oracle.attention_ref(q, k, v, causal=c.causal, scale=c.softmax_scale)
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL[c.dtype], f"max abs err {err}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 77), (31, 13), (64, 77), (100, 128), (128, 128),
                                   (77, 64), (128, 33), (33, 96), (200, 20)])
def test_short_cross_lengths(dtype, Nq, Nk):
    check(3, 4, 4, Nq, Nk, 64, dtype, False, seed=Nq * 1000 + Nk)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N", [1, 5, 31, 32, 33, 64, 96, 127, 128])
def test_short_causal(dtype, N):
    check(2, 4, 2, N, N, 128, dtype, True, seed=N)


@pytest.mark.parametrize("G,Nq", [(2, 64), (4, 128), (8, 64), (16, 32), (8, 128), (32, 16)])
@pytest.mark.parametrize("causal", [False, True])
def test_short_gqa(G, Nq, causal):
    check(2, 2 * G, 2, Nq, Nq, 64, "bf16", causal, seed=G)


@pytest.mark.parametrize("d", [8, 16, 40, 64, 72, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_short_head_dims(d, causal):
    check(2, 3, 3, 50, 50, d, "bf16", causal, seed=d)


@pytest.mark.parametrize("scale", [0.0, -0.125, 1.0, 2.0])
def test_short_scales(scale):
    # |scale| above 1/sqrt(64) sharpens the softmax: |O| is no longer O(1)
    rel = abs(scale) > 1 / math.sqrt(64)
    check(2, 2, 2, 64, 77, 64, "f16", False, scale=scale, seed=11, rel=rel)
    check(2, 2, 2, 64, 64, 64, "bf16", True, scale=scale, seed=12, rel=rel)


def test_short_lse():
    """The per-row log-sum-exp the backward reads, from the short kernel."""
    for dtype, causal in (("bf16", True), ("f16", False)):
        q, k, v = dense_inputs(2, 8, 2, 96, 96, 128, seed=21, dtype=dtype)
        sc = 1 / math.sqrt(128)
        out, lse = aule.flash_attention(dev(q, dtype), dev(k, dtype), dev(v, dtype),
                                        causal=causal, scale=sc, return_lse=True)
        torch.cuda.synchronize()
        ref = oracle.attention_ref_lse(q, k, v, causal=causal, scale=sc)
        u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
        got = lse.cpu().numpy().astype(np.float64)
        bar = (u + 2e-5) * np.maximum(1.0, np.abs(ref))
        assert np.all(np.abs(got - ref) <= bar), float(np.max(np.abs(got - ref)))
        ro = oracle.attention_ref(q, k, v, causal=causal, scale=sc)
        assert float(np.max(np.abs(host(out) - ro))) <= TOL[dtype]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d", [(512, 4, 4, 32, 40, 64), (1024, 4, 2, 32, 33, 64),
                                            (600, 2, 2, 64, 96, 64), (300, 3, 3, 64, 77, 128)])
def test_short_many_units(B, Hq, Hkv, Nq, Nk, d):
    """Many (batch, kv head) units, several rounds of workgroups on the chip, GQA and plain,
    head_dim 64 and 128, bf16 and fp16 with a negative scale."""
    check(B, Hq, Hkv, Nq, Nk, d, "bf16", False, seed=B + Nk)
    check(B, Hq, Hkv, Nq, Nk, d, "f16", False, scale=-0.2, seed=B + Nk + 1)


def test_short_non_default_stream():
    check(4, 4, 4, 64, 77, 64, "bf16", False, seed=5, stream=torch.cuda.Stream())


def test_short_deterministic():
    q, k, v = dense_inputs(8, 12, 12, 64, 77, 64, seed=9, dtype="bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    a = aule.flash_attention(qd, kd, vd, causal=False)
    b = aule.flash_attention(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
