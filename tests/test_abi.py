"""C-ABI contract tests that need no GPU: the library loads, exports every function the
header declares, and rejects every invalid argument with the documented status before
any HIP call (so no device is touched). Fake, never-dereferenced pointer values are used
where a pointer must be non-null."""
import math
import os
import re
import subprocess

import pytest

import tiled_attention_02_amd as aule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aule_attn.h")

F32, F16, BF16 = aule.AULE_DTYPE_F32, aule.AULE_DTYPE_F16, aule.AULE_DTYPE_BF16
OK, INV, UNS = aule.AULE_OK, aule.AULE_ERR_INVALID_ARGUMENT, aule.AULE_ERR_UNSUPPORTED

# distinct, 16-byte aligned, never dereferenced: each call below fails validation first
P = {"q": 0x10000000, "k": 0x20000000, "v": 0x30000000, "o": 0x40000000,
     "qkv": 0x50000000, "cu": 0x60000000, "ws": 0x70000000}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(aule.LIB_PATH):
        from tiled_attention_02_amd.build import build
        build()
    return aule.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aule_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(aule.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", aule.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (aule_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    assert aule.aule_status_string(OK) == "AULE_OK"
    assert aule.aule_status_string(INV) == "AULE_ERR_INVALID_ARGUMENT"
    assert aule.aule_status_string(UNS) == "AULE_ERR_UNSUPPORTED"
    assert aule.aule_status_string(aule.AULE_ERR_HIP) == "AULE_ERR_HIP"
    assert aule.aule_status_string(99) == "AULE_STATUS_UNKNOWN"


def fwd(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], o=P["o"], batch=1, heads_q=4, heads_kv=2,
             seqlen_q=16, seqlen_k=16, head_dim=64, causal=1, scale=0.125, dtype=BF16,
             stream=None)
    a.update(kw)
    return aule.aule_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads_q"],
                              a["heads_kv"], a["seqlen_q"], a["seqlen_k"], a["head_dim"],
                              a["causal"], a["scale"], a["dtype"], a["stream"])


def varlen(**kw):
    a = dict(qkv=P["qkv"], cu=P["cu"], o=P["o"], num_seqs=2, total_tokens=12, max_seqlen=7,
             heads=2, head_dim=64, causal=1, scale=0.125, dtype=F16, stream=None)
    a.update(kw)
    return aule.aule_attn_fwd_varlen(a["qkv"], a["cu"], a["o"], a["num_seqs"],
                                     a["total_tokens"], a["max_seqlen"], a["heads"],
                                     a["head_dim"], a["causal"], a["scale"], a["dtype"],
                                     a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(o=None), INV),
    (dict(batch=-1), INV), (dict(seqlen_q=-3), INV),
    (dict(heads_q=0), INV), (dict(heads_kv=0), INV), (dict(heads_q=6, heads_kv=4), INV),
    (dict(seqlen_k=0, causal=0), INV),
    (dict(head_dim=0), INV), (dict(head_dim=-8), INV),
    (dict(head_dim=136), UNS), (dict(head_dim=256), UNS), (dict(head_dim=60), UNS),
    (dict(head_dim=4), UNS),
    (dict(seqlen_q=16, seqlen_k=32, causal=1), UNS),
    (dict(scale=math.inf), INV), (dict(scale=math.nan), INV), (dict(scale=-math.inf), INV),
    (dict(dtype=7), UNS), (dict(dtype=-1), UNS),
    (dict(q=P["q"] + 8), INV), (dict(o=P["o"] + 2), INV),
    (dict(o=P["q"]), INV), (dict(o=P["k"] + 64), INV),
])
def test_fwd_rejects_invalid_arguments(lib, kw, status):
    assert fwd(**kw) == status
    assert aule.aule_last_error() != ""


def test_fwd_empty_problems_are_noops(lib):
    # nothing is launched: null pointers are fine for an empty problem
    assert fwd(batch=0, q=None, k=None, v=None, o=None) == OK
    assert fwd(seqlen_q=0, seqlen_k=0, q=None, k=None, v=None, o=None) == OK
    assert aule.aule_last_error() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), INV), (dict(cu=None), INV), (dict(o=None), INV),
    (dict(num_seqs=0), INV), (dict(num_seqs=-2), INV), (dict(total_tokens=-1), INV),
    (dict(max_seqlen=-1), INV), (dict(max_seqlen=0), INV), (dict(heads=0), INV),
    (dict(head_dim=200), UNS), (dict(head_dim=12), UNS), (dict(dtype=3), UNS),
    (dict(scale=math.nan), INV),
    (dict(qkv=P["qkv"] + 4), INV), (dict(cu=P["cu"] + 2), INV),
    (dict(o=P["qkv"] + 1024), INV),
])
def test_varlen_rejects_invalid_arguments(lib, kw, status):
    assert varlen(**kw) == status
    assert aule.aule_last_error() != ""


# far-apart fake pointers for problems whose tensors span gigabytes (never dereferenced)
BIG = {"q": 0x100000000000, "k": 0x200000000000, "v": 0x300000000000, "o": 0x400000000000,
       "qkv": 0x500000000000, "cu": 0x600000000000}


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_oversized_16bit_slices_are_refused(lib, dtype):
    """A 16-bit problem whose (sequence, head) slice spans 1 GiB or more (past the
    matrix-core kernels' 32-bit offsets) is refused before any launch, not sent to another
    kernel; fp32 takes the vector-ALU kernel, which has no such bound."""
    st = varlen(qkv=BIG["qkv"], cu=BIG["cu"], o=BIG["o"], num_seqs=1, total_tokens=100000,
                max_seqlen=100000, heads=64, head_dim=128, dtype=dtype)
    assert st == UNS and "1 GiB" in aule.aule_last_error()
    st = fwd(q=BIG["q"], k=BIG["k"], v=BIG["v"], o=BIG["o"], batch=1, heads_q=1, heads_kv=1,
             seqlen_q=5_000_000, seqlen_k=5_000_000, head_dim=128, causal=0, dtype=dtype)
    assert st == UNS


def test_varlen_empty_problem_is_noop(lib):
    assert varlen(total_tokens=0, qkv=None, cu=None, o=None) == OK


def varlen_mods(**kw):
    a = dict(qkv=P["qkv"], cu=P["cu"], o=P["o"], num_seqs=2, total_tokens=12, max_seqlen=7,
             heads=2, head_dim=64, causal=1, scale=0.125, wl=4, wr=0, softcap=0.0,
             alibi=0xD0000000, astride=0, dtype=F16, stream=None)
    a.update(kw)
    return aule.aule_attn_fwd_varlen_mods(a["qkv"], a["cu"], a["o"], a["num_seqs"],
                                          a["total_tokens"], a["max_seqlen"], a["heads"],
                                          a["head_dim"], a["causal"], a["scale"], a["wl"],
                                          a["wr"], a["softcap"], a["alibi"], a["astride"],
                                          a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(wl=-2), INV), (dict(wr=-5, causal=0), INV), (dict(wr=3, causal=1), INV),
    (dict(softcap=-1.0), INV), (dict(softcap=math.inf), INV), (dict(softcap=math.nan), INV),
    (dict(alibi=0xD0000002), INV), (dict(astride=1), INV), (dict(astride=-2), INV),
    (dict(alibi=P["o"] + 16), INV),                       # slopes overlap the output
    (dict(qkv=None), INV), (dict(head_dim=12), UNS), (dict(num_seqs=0), INV),
])
def test_varlen_mods_rejects_invalid_arguments(lib, kw, status):
    assert varlen_mods(**kw) == status
    assert aule.aule_last_error() != ""


def test_varlen_mods_empty_problem_is_noop(lib):
    assert varlen_mods(total_tokens=0, qkv=None, cu=None, o=None, alibi=None) == OK


def splitkv(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], o=P["o"], batch=2, heads_q=8, heads_kv=2,
             seqlen_q=1, seqlen_k=1000, head_dim=128, causal=1, scale=0.088, dtype=BF16,
             num_splits=0, ws=P["ws"], ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return aule.aule_attn_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads_q"],
                                      a["heads_kv"], a["seqlen_q"], a["seqlen_k"], a["head_dim"],
                                      a["causal"], a["scale"], a["dtype"], a["num_splits"],
                                      a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(o=None), INV), (dict(ws=None), INV),
    (dict(batch=-1), INV), (dict(seqlen_q=-1), INV), (dict(heads_kv=3), INV),
    (dict(seqlen_k=0), INV), (dict(num_splits=-1), INV),
    (dict(head_dim=136), UNS), (dict(head_dim=20), UNS), (dict(dtype=5), UNS),
    (dict(seqlen_q=3, seqlen_k=2, causal=1), UNS),
    (dict(seqlen_q=17, heads_q=8, heads_kv=2, causal=0), UNS),     # 4 * 17 > 64 rows
    (dict(scale=math.nan), INV), (dict(ws=P["ws"] + 8), INV), (dict(ws_bytes=16), INV),
    (dict(ws=P["q"]), INV), (dict(o=P["k"] + 16), INV),
])
def test_splitkv_rejects_invalid_arguments(lib, kw, status):
    assert splitkv(**kw) == status
    assert aule.aule_last_error() != ""


def test_splitkv_empty_problems_are_noops(lib):
    assert splitkv(batch=0, q=None, k=None, v=None, o=None, ws=None) == OK
    assert splitkv(seqlen_q=0, q=None, k=None, v=None, o=None, ws=None) == OK


def test_splitkv_workspace_size(lib):
    ws = aule.aule_attn_splitkv_workspace_size
    # 2 x 8 output rows; 1000 keys = 16 tiles of 64; explicit 4 splits of 4 tiles each:
    # m, l rounded up to 256 bytes, then 4 x 16 x 128 floats
    rows, s = 2 * 8 * 1, 4
    assert ws(2, 8, 2, 1, 1000, 128, BF16, 4) == ((s * rows * 8 + 255) // 256 * 256) + s * rows * 128 * 4
    # more splits than tiles are clamped; fp32 tiles are 32 keys
    assert ws(1, 1, 1, 1, 64, 64, F16, 100) == 256 + 1 * 1 * 64 * 4
    assert ws(1, 1, 1, 1, 64, 64, F32, 100) == 256 + 2 * 1 * 64 * 4
    # automatic choice: about C / (batch * heads_kv) splits, clamped to the tiles; C = 1024
    # for the vector-ALU kernel, the CU count (256 on MI355X, and without a device) for the
    # matrix-core one (16-bit, at most 32 query rows per kv head)
    assert ws(2, 8, 2, 1, 1 << 16, 64, F32, 0) == ws(2, 8, 2, 1, 1 << 16, 64, F32, 256)
    assert ws(2, 8, 2, 1, 1 << 16, 64, BF16, 0) == ws(2, 8, 2, 1, 1 << 16, 64, BF16, 64)
    assert ws(2, 8, 2, 16, 1 << 16, 64, BF16, 0) == ws(2, 8, 2, 16, 1 << 16, 64, BF16, 256)
    # empty or rejected arguments -> 0
    assert ws(0, 8, 2, 1, 100, 64, BF16, 0) == 0
    assert ws(1, 8, 3, 1, 100, 64, BF16, 0) == 0 and aule.aule_last_error() != ""


def bwd(**kw):
    a = dict(q=P["q"], k=P["k"], v=P["v"], o=P["o"], do=0x80000000, lse=0x90000000,
             dq=0xA0000000, dk=0xB0000000, dv=0xC0000000, batch=1, heads_q=4, heads_kv=2,
             seqlen_q=16, seqlen_k=16, head_dim=64, causal=1, scale=0.125, dtype=BF16, stream=None)
    a.update(kw)
    return aule.aule_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                              a["dv"], a["batch"], a["heads_q"], a["heads_kv"], a["seqlen_q"],
                              a["seqlen_k"], a["head_dim"], a["causal"], a["scale"], a["dtype"],
                              a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(do=None), INV), (dict(lse=None), INV), (dict(dq=None), INV),
    (dict(dk=None), INV), (dict(dv=None), INV), (dict(heads_q=6, heads_kv=4), INV),
    (dict(seqlen_k=32), UNS), (dict(head_dim=136), UNS), (dict(scale=math.nan), INV),
    (dict(dq=P["q"]), INV), (dict(dk=P["v"] + 16), INV), (dict(dv=0xB0000000), INV),
    (dict(lse=0x90000002), INV), (dict(dq=0xA0000008), INV), (dict(dtype=9), UNS),
])
def test_bwd_rejects_invalid_arguments(lib, kw, status):
    assert bwd(**kw) == status
    assert aule.aule_last_error() != ""


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_bwd_oversized_16bit_slices_are_refused(lib, dtype):
    """The backward's matrix-core kernels address one (batch, head) slice with 32-bit buffer
    offsets: a 16-bit slice of 1 GiB or more is refused before any launch."""
    big = dict(q=BIG["q"], k=BIG["k"], v=BIG["v"], o=BIG["o"], do=0x700000000000,
               lse=0x800000000000, dq=0x900000000000, dk=0xA00000000000, dv=0xB00000000000)
    st = bwd(**big, heads_q=1, heads_kv=1, seqlen_q=4_200_000, seqlen_k=4_200_000, head_dim=128,
             causal=0, dtype=dtype)
    assert st == UNS and "1 GiB" in aule.aule_last_error()


def test_fwd_lse_rejects_null_lse(lib):
    st = aule.aule_attn_fwd_lse(P["q"], P["k"], P["v"], P["o"], None, 1, 4, 2, 16, 16, 64, 1,
                                0.125, BF16, None)
    assert st == INV
    assert aule.aule_attn_fwd_lse(P["q"], P["k"], P["v"], P["o"], P["q"] + 64, 1, 4, 2, 16, 16,
                                  64, 1, 0.125, BF16, None) == INV     # lse overlaps q


def test_bwd_empty_problem_is_noop(lib):
    assert bwd(batch=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None,
               dv=None) == OK


def test_python_wrappers_refuse_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        aule.flash_attention(q, q, q)
    qkv = torch.zeros(8, 3, 2, 64, dtype=torch.float16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError):
        aule.flash_attn_varlen_qkvpacked_func(qkv, cu, 8)
    with pytest.raises(ValueError):
        aule.flash_attention_decode(q, q, q)
    for kw in (dict(dropout_p=0.1), dict(return_attn_probs=True)):
        with pytest.raises(NotImplementedError):
            aule.flash_attn_varlen_qkvpacked_func(qkv, cu, 8, **kw)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(aule, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        aule.load_library(str(tmp_path / "absent.so"))
