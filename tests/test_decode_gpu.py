"""GPU parity of the split-KV decoding path (aule_attn_fwd_splitkv, through the C-ABI
library) against the CPU fp64 oracle's attention_ref_decode on the same seeded,
dtype-rounded inputs. Bars as for the forward: 1e-5 fp32,
2e-3 fp16, 1e-2 bf16, max abs error over every element."""
import math

import numpy as np
import pytest

import oracle
import tiled_attention_02_amd as aule
from workloads import DECODE_CONFIGS, dense_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
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


def tolerance(dtype, scale, d):
    """The stated bar of the dtype (max abs error for O(1) outputs), at every scale."""
    return TOL[dtype]


def check(B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale=None, num_splits=0, seed=0):
    print(f"decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"splits={num_splits} seed={seed}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, dtype=dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o = aule.flash_attention_decode(dev(q, dtype), dev(k, dtype), dev(v, dtype), causal=causal,
                                    scale=sc, num_splits=num_splits)
    torch.cuda.synchronize()
    got = host(o)
    ref = oracle.attention_ref_decode(q, k, v, causal=causal, scale=sc)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    tol = tolerance(dtype, sc, d)
    assert err <= tol, f"max abs err {err} > {tol}"
    return err


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("G,Nq,Nk", [(1, 1, 1), (4, 1, 1000), (4, 4, 1000), (8, 8, 64),
                                     (1, 64, 64), (32, 2, 300), (2, 16, 5000), (4, 3, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_decode_shapes(dtype, G, Nq, Nk, causal):
    check(2, 2 * G, 2, Nq, Nk, 128, dtype, causal, seed=Nk + Nq)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [8, 40, 64, 72, 128])
def test_decode_head_dims(dtype, d):
    check(1, 8, 2, 2, 777, d, dtype, True, seed=d)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 1000])
def test_decode_split_counts(num_splits):
    check(1, 4, 1, 4, 2000, 128, "bf16", True, num_splits=num_splits, seed=11)


@pytest.mark.parametrize("which", ["zero", "neg", "big"])
def test_decode_scales(which):
    sc = {"zero": 0.0, "neg": -0.3, "big": 2.0}[which]
    check(1, 8, 8, 1, 513, 64, "f16", False, scale=sc, seed=12)
    check(1, 8, 8, 1, 513, 64, "f32", True, scale=sc, seed=13)


def test_decode_equals_forward_when_lengths_match():
    """With seqlen_q == seqlen_k the bottom-right mask is the forward's causal mask
    (4 heads per kv head x 16 queries = the 64-row limit)."""
    q, k, v = dense_inputs(1, 8, 2, 16, 16, 64, seed=21, dtype="bf16")
    a = aule.flash_attention_decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=True)
    b = aule.flash_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=True)
    torch.cuda.synchronize()
    assert float(np.max(np.abs(host(a) - host(b)))) <= 2e-2   # two kernels, each within 1e-2


def test_decode_workload_full():
    c = DECODE_CONFIGS["d1_bf16_decode_gqa"]
    print(f"workload {c.name}", flush=True)
    q, k, v = c.inputs()
    o = aule.flash_attention_decode(dev(q, c.dtype), dev(k, c.dtype), dev(v, c.dtype),
                                    causal=c.causal, scale=c.softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.attention_ref_decode(q, k, v, causal=c.causal, scale=c.softmax_scale)
    err = float(np.max(np.abs(host(o) - ref)))
    assert err <= TOL[c.dtype], err


def test_decode_workspace_reuse_and_guard_regions():
    """Two calls in a row through one workspace (the second smaller) are both correct, and
    the bytes around O stay untouched."""
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    for (Nq, Nk, seed) in ((4, 3000, 31), (1, 100, 32)):
        q, k, v = dense_inputs(2, 8, 2, Nq, Nk, 128, seed=seed, dtype="bf16")
        n = q.size
        buf = torch.full((n + 2 * 64,), float("nan"), dtype=torch.bfloat16, device="cuda")
        out = buf[64:64 + n].view(q.shape)
        aule.flash_attention_decode(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=True,
                                    out=out, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.attention_ref_decode(q, k, v, causal=True, scale=1 / math.sqrt(128))
        assert float(np.max(np.abs(host(out) - ref))) <= TOL["bf16"]
        assert torch.isnan(buf[:64]).all() and torch.isnan(buf[64 + n:]).all()


def test_decode_non_default_stream():
    q, k, v = dense_inputs(1, 4, 1, 2, 900, 64, seed=41, dtype="f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o = aule.flash_attention_decode(dev(q, "f16"), dev(k, "f16"), dev(v, "f16"), causal=True)
    s.synchronize()
    ref = oracle.attention_ref_decode(q, k, v, causal=True, scale=1 / 8)
    assert float(np.max(np.abs(host(o) - ref))) <= TOL["f16"]


def test_decode_small_workspace_is_rejected_before_launch():
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 500, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(aule.AuleError):
        aule.flash_attention_decode(q, k, k, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
