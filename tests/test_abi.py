"""The C-ABI library on the CPU: it loads, exports what include/vfa.h declares,
and rejects bad arguments with the documented status before any launch.

Every call below fails validation on host values, so nothing is launched
(the pointers passed are dummies that are never dereferenced).
"""
import ctypes
import os
import re

import pytest

import varlen_flash_attention_amd as vfa
from varlen_flash_attention_amd import build as vbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vfa.h")

OK, NULL, SHAPE, UNSUP, WS, LAUNCH = 0, 1, 2, 3, 4, 5
P = 0x10000          # dummy, 16-byte aligned, never dereferenced
F32, BF16 = 0, 1


def declared_functions():
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    # test_host_sanitizer.py runs this file against a build of the C-ABI layer
    # with sanitizers and stub launchers, named by VFA_TEST_LIBRARY.
    alt = os.environ.get("VFA_TEST_LIBRARY")
    if alt:
        vfa._LIB = None
        vfa.library_path = lambda: alt
    elif not os.path.exists(vfa.library_path()):
        vbuild.build()
    return vfa.load_library()


@pytest.fixture(autouse=True)
def no_launch(request):
    """With the stub build, no call in this file may reach a launcher or a device check."""
    if "lib" not in request.fixturenames:
        yield
        return
    lib = request.getfixturevalue("lib")
    count = getattr(lib, "vfa_stub_launch_count", None)
    before = count() if count else 0
    yield
    if count:
        assert count() == before, "a call reached the GPU side"


def test_exports_match_header(lib):
    exported = set(vbuild.exported_symbols())
    declared = set(declared_functions())
    assert declared, "no functions parsed from the header"
    assert declared <= exported, f"declared but not exported: {declared - exported}"
    assert exported <= declared, f"exported but not declared: {exported - declared}"


def test_abi_version(lib):
    assert lib.vfa_abi_version() == vfa._header_abi_version() == 8


def test_status_strings(lib):
    for code in range(6):
        s = lib.vfa_status_string(code).decode()
        assert s.startswith("VFA_")
    assert lib.vfa_status_string(99).decode() == "unknown vfa status"


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=BF16, cu_q=P, cu_k=P, batch=2, total_q=8, total_k=8, max_q=4, max_k=4,
             hq=4, hkv=2, d=128, scale=0.125, causal=1, out=P, out_dtype=BF16, lse=P, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.varlen_attn_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["cu_q"], a["cu_k"], a["batch"],
                               a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["hq"], a["hkv"], a["d"],
                               a["scale"], a["causal"], a["out"], a["out_dtype"], a["lse"], a["ws"],
                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), OK),                     # empty batch: nothing to do, nothing launched
    (dict(total_q=0), OK),
    (dict(batch=0, q=None), OK),
    (dict(batch=-1), SHAPE),
    (dict(total_q=-3), SHAPE),
    (dict(max_q=-1), SHAPE),
    (dict(q=None), NULL),
    (dict(k=None), NULL),
    (dict(v=None), NULL),
    (dict(cu_q=None), NULL),
    (dict(cu_k=None), NULL),
    (dict(out=None), NULL),
    (dict(lse=None), NULL),
    (dict(hq=6, hkv=4), SHAPE),              # Hq % Hkv != 0
    (dict(hq=0), SHAPE),
    (dict(hkv=0), SHAPE),
    (dict(causal=2), SHAPE),
    (dict(max_q=9), SHAPE),                  # bound above the token count
    (dict(max_q=3), SHAPE),                  # 2 sequences of <= 3 tokens cannot hold 8
    (dict(d=96), UNSUP),
    (dict(d=256), UNSUP),
    (dict(hq=128, hkv=2), UNSUP),            # G = 64 > 32
    (dict(in_dtype=7), UNSUP),
    (dict(in_dtype=F32, out_dtype=BF16), UNSUP),
    (dict(out_dtype=5), UNSUP),
    (dict(scale=0.0), UNSUP),
    (dict(scale=-1.0), UNSUP),
    (dict(scale=float("nan")), UNSUP),
    (dict(scale=float("inf")), UNSUP),
    (dict(q=P + 2), UNSUP),                  # not 16-byte aligned
    (dict(out=P + 8), UNSUP),
    # decode-shaped call (Lq = 1, long keys) needs a workspace
    (dict(batch=4, total_q=4, total_k=8192, max_q=1, max_k=4096, hq=32, hkv=4), WS),
    (dict(batch=4, total_q=4, total_k=8192, max_q=1, max_k=4096, hq=32, hkv=4, ws=P, ws_bytes=16), WS),
    (dict(batch=4, total_q=4, total_k=8192, max_q=1, max_k=4096, hq=32, hkv=4, ws=P + 4, ws_bytes=1 << 30), WS),
])
def test_fwd_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_fwd_offset_validation(lib):
    a = (P, P, P, BF16, P, P)
    rest = (2, 8, 8, 4, 4, 4, 2, 128, 0.125)
    tail = (P, BF16, P, None, 0, None)
    off = lib.varlen_attn_fwd_offset
    assert off(*a, None, *rest, 1, *tail) == NULL                     # causal needs the offsets
    assert off(*a, None, 0, 8, 8, 4, 4, 4, 2, 128, 0.125, 1, *tail) == OK   # empty batch
    assert off(*a, P, 2, 8, 8, 4, 4, 4, 2, 96, 0.125, 1, *tail) == UNSUP     # same checks as varlen_attn_fwd
    assert off(*a, P, -1, 8, 8, 4, 4, 4, 2, 128, 0.125, 1, *tail) == SHAPE


def _noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=BF16, cu_q=P, cu_k=P, batch=2, total_q=8, total_k=8, max_q=4, max_k=4,
             hq=4, hkv=2, d=128, scale=0.125, causal=1, out=P, out_dtype=BF16, lse=P, stream=None)
    a.update(kw)
    return lib.varlen_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["in_dtype"], a["cu_q"], a["cu_k"], a["batch"],
                                       a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["hq"], a["hkv"],
                                       a["d"], a["scale"], a["causal"], a["out"], a["out_dtype"], a["lse"],
                                       a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), OK),
    (dict(batch=-1), SHAPE),
    (dict(q=None), NULL),
    (dict(lse=None), NULL),
    (dict(hq=6, hkv=4), SHAPE),
    (dict(d=96), UNSUP),
    (dict(in_dtype=F32, out_dtype=BF16), UNSUP),
    (dict(out=P + 8), UNSUP),
    # 256 decode sequences with keys up to 32768 in 4096-key splits: 8 * 256 * 32 * 129 * 4 B = 33.8 MB of
    # partials, more than the 16 MiB static array holds
    (dict(batch=256, total_q=256, total_k=256 * 32768, max_q=1, max_k=32768, hq=32, hkv=4), WS),
])
def test_noalloc_validation(lib, kw, code):
    # The same checks as varlen_attn_fwd, and a call whose split-KV partials exceed the static array is
    # rejected before anything is launched (or looked up).
    assert _noalloc(lib, **kw) == code


def test_noalloc_limit_matches_the_workspace_plan(lib):
    limit = vfa.STATIC_SCRATCH_BYTES
    with open(HEADER) as fh:
        assert re.search(r"#define\s+VFA_STATIC_SCRATCH_BYTES\s+\(16u << 20\)", fh.read())
    assert limit == 16 << 20
    ws = lib.varlen_attn_fwd_workspace_size
    assert ws(64, 64, 1, 32768, 32, 4, 128) <= limit            # the decode workload fits
    assert ws(256, 256, 1, 32768, 32, 4, 128) > limit           # the case rejected above does not


def _upd(lib, **kw):
    a = dict(lse=P, go=P, go_dtype=F32, sp=8, bsh=2048, hd=128, update_type=1, out=P, lse_out=P, stream=None)
    a.update(kw)
    return lib.attn_update(a["lse"], a["go"], a["go_dtype"], a["sp"], a["bsh"], a["hd"], a["update_type"],
                           a["out"], a["lse_out"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(bsh=0), OK),
    (dict(sp=0), SHAPE),
    (dict(sp=-2), SHAPE),
    (dict(bsh=-1), SHAPE),
    (dict(update_type=2), SHAPE),
    (dict(lse=None), NULL),
    (dict(go=None), NULL),
    (dict(out=None), NULL),
    (dict(lse_out=None), NULL),              # update_type 1 needs lse_out
    (dict(hd=96), UNSUP),
    (dict(go_dtype=3), UNSUP),
    (dict(go=P + 4), UNSUP),
    (dict(out=P + 8), UNSUP),
])
def test_update_validation(lib, kw, code):
    assert _upd(lib, **kw) == code


@pytest.mark.parametrize("args,code", [
    ((P, F32, P, 0, 10, P, None), OK),
    ((P, F32, P, 4, 0, P, None), OK),
    ((P, F32, P, -1, 10, P, None), SHAPE),
    ((P, F32, P, 4, -1, P, None), SHAPE),
    ((None, F32, P, 4, 10, P, None), NULL),
    ((P, F32, None, 4, 10, P, None), NULL),
    ((P, F32, P, 4, 10, None, None), NULL),
    ((P, 9, P, 4, 10, P, None), UNSUP),
])
def test_gather_validation(lib, args, code):
    assert lib.varlen_last_token_gather(*args) == code


def test_workspace_size_plan(lib):
    # Decode-shaped calls (G heads x query tokens <= 16, long keys) get a split-KV workspace of
    # n_splits * total_q * Hq * (D + 1) fp32 values; prefill-shaped calls need none.
    ws = lib.varlen_attn_fwd_workspace_size
    assert ws(64, 64, 1, 32768, 32, 4, 128) == 8 * 64 * 32 * 129 * 4       # 4096-key splits
    assert ws(2, 2, 1, 4096, 32, 4, 128) == 16 * 2 * 32 * 129 * 4          # 256-key splits for a small batch
    assert ws(16, 46000, 8192, 8192, 32, 8, 128) == 1024                    # long prefill: work counters
    # The persistent kernel needs (max_seqlen_k + 256) * Hkv * D * 2 bytes of keys below 2^32; past that the
    # sequence runs on the kernel without counters.
    assert ws(1, 8192, 8192, 2**32 // 2048 - 257, 64, 8, 128) == 1024
    assert ws(1, 8192, 8192, 2**32 // 2048 - 256, 64, 8, 128) == 0
    assert ws(2, 812, 512, 2_100_001, 64, 8, 128) == 0
    assert ws(64, 18000, 512, 512, 16, 8, 128) == 0                         # short prefill: none
    assert ws(64, 64, 1, 300, 32, 4, 128) == 0                              # short keys: no split
    assert ws(8, 24, 3, 8192, 32, 4, 128) == 0                              # 3 tokens x 8 heads > 16 columns
    assert ws(8, 16, 2, 8192, 16, 2, 64) > 0                                # 2 tokens x 8 heads = 16 columns


def _paged(lib, **kw):
    a = dict(q=P, in_dtype=BF16, kc=P, vc=P, table=P, max_pages=4, num_pages=16, page=16, cu_q=P, used=P,
             batch=2, total_q=2, max_q=1, max_k=64, hq=32, hkv=4, d=128, scale=0.125, causal=1, out=P,
             out_dtype=BF16, lse=P, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.paged_attn_decode(a["q"], a["in_dtype"], a["kc"], a["vc"], a["table"], a["max_pages"],
                                 a["num_pages"], a["page"], a["cu_q"], a["used"], a["batch"], a["total_q"],
                                 a["max_q"], a["max_k"], a["hq"], a["hkv"], a["d"], a["scale"], a["causal"],
                                 a["out"], a["out_dtype"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), OK),
    (dict(total_q=0), OK),
    (dict(batch=0, q=None), OK),
    (dict(batch=-1), SHAPE),
    (dict(max_k=-1), SHAPE),
    (dict(max_pages=-1), SHAPE),
    (dict(num_pages=-1), SHAPE),
    (dict(page=0), SHAPE),
    (dict(q=None), NULL),
    (dict(kc=None), NULL),
    (dict(vc=None), NULL),
    (dict(table=None), NULL),
    (dict(cu_q=None), NULL),
    (dict(used=None), NULL),
    (dict(out=None), NULL),
    (dict(lse=None), NULL),
    (dict(hq=6, hkv=4), SHAPE),
    (dict(causal=2), SHAPE),
    (dict(max_q=3), SHAPE),                  # bound above the token count
    (dict(total_q=3), SHAPE),                # 2 sequences of <= 1 token cannot hold 3
    (dict(max_k=65), SHAPE),                 # more keys than 4 pages of 16 can hold
    (dict(num_pages=0), SHAPE),              # keys but no pages
    (dict(d=96), UNSUP),
    (dict(in_dtype=F32, out_dtype=F32), UNSUP),
    (dict(out_dtype=5), UNSUP),
    (dict(page=8, max_pages=8), UNSUP),      # pages below 16 keys
    (dict(page=24), UNSUP),                  # not a power of two
    (dict(page=8192, max_pages=1), UNSUP),
    (dict(page=4096, max_pages=1, hkv=4096, hq=4096), UNSUP),        # page * hkv * D = 2^31
    (dict(scale=0.0), UNSUP),
    (dict(kc=P + 2), UNSUP),
    (dict(out=P + 8), UNSUP),
    # long keys need a split workspace
    (dict(max_k=8192, max_pages=512), WS),
    (dict(max_k=8192, max_pages=512, ws=P, ws_bytes=16), WS),
    (dict(max_k=8192, max_pages=512, ws=P + 4, ws_bytes=1 << 30), WS),
])
def test_paged_validation(lib, kw, code):
    assert _paged(lib, **kw) == code


def test_paged_workspace_plan(lib):
    # (sequence, kv head, 16-column group) units set the split length: 4096 keys, halved while fewer than
    # 2048 (unit, split) pairs; the workspace holds fp32 partial O and lse per split and query row, as on
    # the contiguous decode path; none when a single split covers max_seqlen_k.
    ws = lib.paged_attn_decode_workspace_size
    assert ws(64, 64, 1, 32768, 32, 4, 128) == 8 * 64 * 32 * 129 * 4
    assert ws(2, 2, 1, 4096, 32, 4, 128) == 16 * 2 * 32 * 129 * 4              # 256-key splits
    assert ws(2, 6, 3, 4096, 32, 1, 64) == 16 * 6 * 32 * 65 * 4                # 3 tokens x 32 heads = 6 groups
    assert ws(2, 2, 1, 40000, 32, 1, 64) == 157 * 2 * 32 * 65 * 4              # 2 units: 256-key splits
    assert ws(64, 64, 1, 256, 32, 4, 128) == 0                                  # one split
    assert ws(0, 0, 1, 4096, 32, 4, 128) == 0


def _qknr(lib, **kw):
    a = dict(q=P, k=P, dtype=BF16, wq=P, wk=P, cos=P, sin=P, t=16, hq=32, hkv=8, d=128, eps=1e-6, qo=P, ko=P,
             stream=None)
    a.update(kw)
    return lib.qk_norm_rope(a["q"], a["k"], a["dtype"], a["wq"], a["wk"], a["cos"], a["sin"], a["t"], a["hq"],
                            a["hkv"], a["d"], a["eps"], a["qo"], a["ko"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=0), OK),
    (dict(hq=0, hkv=0), OK),
    (dict(t=0, q=None), OK),
    (dict(t=-1), SHAPE),
    (dict(hq=-1), SHAPE),
    (dict(cos=None), NULL),
    (dict(sin=None), NULL),
    (dict(q=None), NULL),
    (dict(wk=None), NULL),
    (dict(ko=None), NULL),
    (dict(d=96), UNSUP),
    (dict(dtype=F32), UNSUP),
    (dict(eps=-1.0), UNSUP),
    (dict(eps=float("nan")), UNSUP),
    (dict(q=P + 2), UNSUP),
    (dict(cos=P + 4), UNSUP),
    (dict(hkv=0, k=None, wk=None, ko=None, d=96), UNSUP),   # k side unused: only the head_dim check fails
])
def test_qk_norm_rope_validation(lib, kw, code):
    assert _qknr(lib, **kw) == code


def _gdn(lib, **kw):
    # max_seqlen 8 takes the token-by-token path, which needs no workspace.
    a = dict(q=P, k=P, v=P, dtype=BF16, g=P, beta=P, cu=P, batch=2, t=16, ms=8, hqk=16, hv=32, dk=128, dv=128,
             scale=0.088, s0=None, out=P, s1=None, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.gated_delta_rule_fwd(a["q"], a["k"], a["v"], a["dtype"], a["g"], a["beta"], a["cu"], a["batch"],
                                    a["t"], a["ms"], a["hqk"], a["hv"], a["dk"], a["dv"], a["scale"], a["s0"],
                                    a["out"], a["s1"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), OK),
    (dict(batch=-1), SHAPE),
    (dict(hqk=0), SHAPE),
    (dict(hqk=3, hv=32), SHAPE),             # Hv not a multiple of Hqk
    (dict(q=None), NULL),
    (dict(g=None), NULL),
    (dict(cu=None), NULL),
    (dict(out=None), NULL),
    (dict(dtype=F32), UNSUP),
    (dict(dk=96), UNSUP),
    (dict(dv=32), UNSUP),
    (dict(scale=float("inf")), UNSUP),
    (dict(ms=-1), SHAPE),
    (dict(ms=100), WS),                              # chunked path without a workspace
    (dict(ms=100, ws=P, wsb=16 * 32 * 520 + 16384 - 1), WS),
    (dict(ms=100, ws=P, wsb=16 * 32 * 520 + 16384, dv=32), UNSUP),
    (dict(s0=P + 4), UNSUP),                         # states move in 16-byte pieces
    (dict(s1=P + 8), UNSUP),
    (dict(q=P + 2), UNSUP),                          # so do token rows
    (dict(v=P + 8), UNSUP),
    (dict(out=P + 4), UNSUP),
    (dict(ms=100, ws=P + 8, wsb=16 * 32 * 520 + 16384 + 8), WS),   # and the workspace
    (dict(ms=100, ws=P, wsb=1 << 60, hqk=1 << 18, hv=1 << 18), UNSUP),   # chunk spans past 32-bit offsets
])
def test_gated_delta_validation(lib, kw, code):
    assert _gdn(lib, **kw) == code


def test_gated_delta_workspace_size(lib):
    """Lengths up to 16 take the recurrence (no workspace); above, the chunked form keeps two 64-wide
    bf16 hi / lo rows (T and M) and two fp32 decay factors per (token, value head): 520 bytes; plus a
    fixed 16 KiB slot for the order in which the chunk kernel takes the sequences (up to 4096 ranked)."""
    ws = lib.gated_delta_rule_fwd_workspace_size
    assert ws(35324, 32, 16) == 0
    assert ws(35324, 32, 17) == 35324 * 32 * 520 + 16384
    assert ws(0, 32, 8192) == 0
    assert ws(1, 1, 8192) == 520 + 16384
