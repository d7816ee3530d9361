"""GPU parity of the varlen score modifiers (aule_attn_fwd_varlen_mods through the C-ABI
library: sliding window, soft cap, ALiBi) against the CPU fp64 oracle's
attention_ref_varlen_mods on the same seeded, dtype-rounded inputs. Bars as for the
forward: 1e-5 fp32 (scaled with |scale|*sqrt(d)), 2e-3 fp16, 1e-2 bf16, on
|got - ref| / max(1, |ref|) element by element. A narrow window leaves a query only a few
keys, so O is not averaged down and |O| reaches |V| (about 4): rounding O to the dtype alone
moves it by up to the unit roundoff times |O|, hence the per-element relative form (which is
the plain absolute error wherever |O| <= 1)."""
import math

import numpy as np
import pytest

import oracle
import tiled_attention_02_amd as aule
from workloads import MODS_CONFIGS, alibi_slopes, varlen_inputs

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


def tolerance(dtype, scale, d):
    """The stated bar of the dtype (max abs error for O(1) outputs), at every scale."""
    return TOL[dtype]


def run(qkv, cu, dtype, causal, scale, window, softcap, slopes):
    a = None if slopes is None else torch.from_numpy(np.asarray(slopes, dtype=np.float32)).cuda()
    cu_d = torch.from_numpy(cu).cuda()
    L = int(np.max(np.diff(cu))) if cu.size > 1 else 0
    o = aule.flash_attn_varlen_qkvpacked_func(dev(qkv, dtype), cu_d, L, softmax_scale=scale,
                                              causal=causal, window_size=window,
                                              softcap=softcap, alibi_slopes=a)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def check(lengths, H, d, dtype, causal, window=(-1, -1), softcap=0.0, slopes=None, scale=None,
          seed=0, tokens=None):
    print(f"mods lengths={lengths} H={H} d={d} {dtype} causal={causal} window={window} "
          f"softcap={softcap} alibi={'none' if slopes is None else np.shape(slopes)} "
          f"scale={scale} seed={seed}", flush=True)
    qkv, cu = varlen_inputs(lengths, H, d, seed=seed, dtype=dtype)
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    got = run(qkv, cu, dtype, causal, sc, window, softcap, slopes)
    ref = oracle.attention_ref_varlen_mods(qkv, cu, causal=causal, scale=sc, window=window,
                                           softcap=softcap, alibi_slopes=slopes, tokens=tokens)
    if tokens is not None:
        got = got[tokens]
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref)))) if got.size else 0.0
    tol = tolerance(dtype, sc, d)
    assert err <= tol, f"max abs err {err} > {tol}"
    return err


LENGTHS = [1, 33, 200, 513, 64, 0, 129]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("window", [(0, 0), (1, 0), (31, 0), (32, 0), (33, 0), (100, 0),
                                    (-1, 0), (1000, 0)])
def test_window_causal(dtype, window):
    check(LENGTHS, 3, 128, dtype, True, window=window, seed=window[0] + 7)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("window", [(0, 0), (1, 1), (64, 5), (5, 64), (-1, 3), (40, -1),
                                    (300, 300)])
def test_window_noncausal(dtype, window):
    check(LENGTHS, 2, 64, dtype, False, window=window, seed=window[1] + 11)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_window_int32_max(dtype, causal):
    """Windows of 2^31 - 1 keys mask nothing (and must not overflow a row + window sum)."""
    big = 2 ** 31 - 1
    check(LENGTHS, 3, 128, dtype, causal, window=(big, 0 if causal else big), seed=8)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("softcap", [0.5, 5.0, 50.0])
def test_softcap(dtype, causal, softcap):
    check(LENGTHS, 2, 128, dtype, causal, softcap=softcap, scale=0.3, seed=int(softcap * 10))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("per_seq", [False, True])
def test_alibi(dtype, causal, per_seq):
    H = 4
    rng = np.random.default_rng(5)
    slopes = (rng.uniform(0.0, 0.5, size=(len(LENGTHS), H)).astype(np.float32) if per_seq
              else alibi_slopes(H))
    check(LENGTHS, H, 64, dtype, causal, slopes=slopes, seed=17 + per_seq)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [8, 40, 64, 72, 128])
def test_all_modifiers_head_dims(dtype, d):
    check([77, 300, 5], 2, d, dtype, True, window=(50, 0), softcap=8.0, slopes=alibi_slopes(2),
          seed=d)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.7])
def test_all_modifiers_scales(scale):
    check([150, 40], 2, 128, "bf16", False, window=(20, 30), softcap=3.0,
          slopes=alibi_slopes(2), scale=scale, seed=23)
    check([150, 40], 2, 128, "f32", True, window=(20, 0), softcap=3.0,
          slopes=alibi_slopes(2), scale=scale, seed=24)


def test_modifiers_off_is_the_plain_path_bit_for_bit():
    """Every modifier off through the modifier entry point launches the plain kernels."""
    qkv, cu = varlen_inputs([100, 257], 2, 128, seed=31, dtype="bf16")
    t, cu_d = dev(qkv, "bf16"), torch.from_numpy(cu).cuda()
    a = aule.flash_attn_varlen_qkvpacked_func(t, cu_d, 257, causal=True)
    b = torch.empty_like(a)
    st = aule.aule_attn_fwd_varlen_mods(t.data_ptr(), cu_d.data_ptr(), b.data_ptr(), 2, 357, 257,
                                        2, 128, 1, 1 / math.sqrt(128), -1, -1, 0.0, None, 0,
                                        aule.dtype_code(t.dtype), None)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(a, b)


def test_mods_workload_sampled():
    """The full modifier workload (16 sequences of 64-4096 tokens, 16 heads, d=128, causal,
    window 1024, soft cap 50, ALiBi) on seeded sampled tokens of every sequence."""
    c = MODS_CONFIGS["m1_bf16_varlen_mods"]
    qkv, cu = c.inputs()
    got = run(qkv, cu, c.dtype, c.causal, c.softmax_scale, (c.window_left, c.window_right),
              c.softcap, c.slopes())
    rng = np.random.default_rng(77)
    toks = []
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        pick = {a, e - 1, min(e - 1, a + 1024), min(e - 1, a + 1025)}
        pick |= set(int(x) for x in rng.integers(a, e, size=4))
        toks += sorted(pick)
    toks = np.array(toks)
    ref = oracle.attention_ref_varlen_mods(qkv, cu, causal=c.causal, scale=c.softmax_scale,
                                           window=(c.window_left, c.window_right),
                                           softcap=c.softcap, alibi_slopes=c.slopes(),
                                           tokens=toks)
    err = float(np.max(np.abs(got[toks] - ref) / np.maximum(1.0, np.abs(ref))))
    assert err <= TOL[c.dtype], err
