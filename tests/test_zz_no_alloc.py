"""GPU test of aule_attn_fwd_splitkv_noalloc, the split-KV decoding entry point that allocates
nothing (its split partials live in the library's own device array): called through the
C-ABI, it must return what aule_attn_fwd_splitkv returns with a caller workspace (same split
plan, same kernels), within the dtype's bar, and both must match the CPU oracle. Two calls in
a row on the shared array, the second with a smaller input, so that the second call starts
from the first one's leftover partials."""
import math

import numpy as np
import pytest

import oracle
import tiled_attention_02_amd as aule
from workloads import dense_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CODE = {"f32": aule.AULE_DTYPE_F32, "f16": aule.AULE_DTYPE_F16, "bf16": aule.AULE_DTYPE_BF16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aule.load_library()


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=TDT[dtype])


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def both(B, Hq, Hkv, Nq, Nk, d, dtype, causal, seed, num_splits=0):
    print(f"noalloc B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
          f"splits={num_splits}", flush=True)
    q, k, v = dense_inputs(B, Hq, Hkv, Nq, Nk, d, seed=seed, dtype=dtype)
    tq, tk, tv = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    sc = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    # the existing entry point, with a caller-owned workspace
    need = aule.aule_attn_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, CODE[dtype], num_splits)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws = torch.full_like(tq, float("nan"))
    st = aule.aule_attn_fwd_splitkv(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o_ws.data_ptr(),
                                    B, Hq, Hkv, Nq, Nk, d, causal, sc, CODE[dtype], num_splits,
                                    ws.data_ptr(), need, stream)
    assert st == aule.AULE_OK, aule.aule_last_error()
    # the entry point that allocates nothing
    o_na = torch.full_like(tq, float("nan"))
    st = aule.aule_attn_fwd_splitkv_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(),
                                            o_na.data_ptr(), B, Hq, Hkv, Nq, Nk, d, causal, sc,
                                            CODE[dtype], num_splits, stream)
    assert st == aule.AULE_OK, aule.aule_last_error()
    torch.cuda.synchronize()
    got_ws, got_na = host(o_ws), host(o_na)
    assert np.all(np.isfinite(got_na))
    diff = float(np.max(np.abs(got_na - got_ws)))
    print(f"  noalloc vs workspace max abs diff {diff:.3e}", flush=True)
    assert diff <= TOL[dtype]
    ref = oracle.attention_ref_decode(q, k, v, causal=causal, scale=sc)
    assert float(np.max(np.abs(got_na - ref))) <= TOL[dtype]


def test_noalloc_two_calls_second_smaller():
    both(4, 32, 8, 1, 4096, 128, "bf16", True, seed=61)
    both(2, 8, 2, 3, 1000, 64, "f16", False, seed=62)


def test_noalloc_fp32_and_explicit_splits():
    both(1, 4, 1, 4, 2000, 128, "f32", True, seed=63, num_splits=7)
    both(1, 2, 2, 1, 77, 40, "bf16", True, seed=64, num_splits=3)


def test_noalloc_rejects_oversized_partials():
    """Partials beyond the fixed array are refused before any launch: the output is
    untouched and the status says why."""
    B, Hq, Hkv, Nq, Nk, d = 64, 64, 64, 1, 8192, 128
    need = aule.aule_attn_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, aule.AULE_DTYPE_BF16, 64)
    assert need > 32 << 20
    # small real buffers: the size check comes before anything reads them
    q = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    st = aule.aule_attn_fwd_splitkv_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(),
                                            B, Hq, Hkv, Nq, Nk, d, True, 0.1, aule.AULE_DTYPE_BF16,
                                            64, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == aule.AULE_ERR_UNSUPPORTED
    assert "holds" in aule.aule_last_error()
    assert bool((o == 3.0).all())
