"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects malformed calls before touching the device."""
import os
import re

import pytest

from memory_efficient_attention_amd import _native
from memory_efficient_attention_amd._native import (MEA_BF16, MEA_ERR_INVALID, MEA_ERR_UNSUPPORTED,
                                                    MEA_F16, MEA_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mea.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_native.library_path()),
                                reason="libmea.so not built (run __graft_entry__.build())")


def header_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"MEA_EXPORT\s+[\w\s\*]+?\b(mea_\w+)\s*\(", txt)))


def test_header_declares_the_binding_symbols():
    assert header_symbols() == sorted(_native.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = _native.load()
    for name in header_symbols():
        assert hasattr(lib, name), name


def test_only_declared_c_symbols_are_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _native.library_path()],
                         capture_output=True, text=True, check=True).stdout
    mea = sorted({ln.split()[-1] for ln in out.splitlines() if ln.split() and ln.split()[-1].startswith("mea_")})
    assert mea == header_symbols()


def test_every_kernel_stub_is_defined():
    """A kernel whose host-side launch stub is missing would only fail at load time."""
    import subprocess
    out = subprocess.run(["nm", "-C", "--undefined-only", _native.library_path()],
                         capture_output=True, text=True, check=True).stdout
    assert "__device_stub__" not in out


def test_version_and_strings():
    assert _native.mea_abi_version() == 10
    for st in range(4):
        assert _native.mea_status_string(st).startswith("MEA_")
    assert "unknown" in _native.mea_status_string(99)


# Plausible, aligned fake device addresses: validation never dereferences them.
P = 1 << 20


def call(**kw):
    a = dict(q=P, k=P, v=P, out=P, lse=None, seqstart_q=P, seqstart_k=P, num_seqs=4, total_q=365,
             total_k=365, max_seqlen_q=200, max_seqlen_k=200, Hq=8, Hkv=8, D=64, dtype=MEA_F16, causal=0,
             alibi_slopes=None, scale=0.125, workspace=None, workspace_bytes=0, stream=None)
    chunk = kw.pop("chunk_keys", None)
    a.update(kw)
    if chunk is None:
        return _native.mea_fwd(**a)
    return _native.mea_fwd_splitkv(**a, chunk_keys=chunk)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(out=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(seqstart_k=None), MEA_ERR_INVALID, "seqstart"),
    (dict(num_seqs=-1), MEA_ERR_INVALID, "negative"),
    (dict(Hq=8, Hkv=3), MEA_ERR_INVALID, "Hq % Hkv"),
    (dict(Hkv=0), MEA_ERR_INVALID, "Hkv > 0"),
    (dict(causal=2), MEA_ERR_INVALID, "causal"),
    (dict(max_seqlen_q=0), MEA_ERR_INVALID, "max_seqlen_q == 0"),
    (dict(D=96), MEA_ERR_UNSUPPORTED, "D=96"),
    (dict(D=256), MEA_ERR_UNSUPPORTED, "D=256"),
    (dict(dtype=7), MEA_ERR_UNSUPPORTED, "dtype"),
    (dict(scale=float("nan")), MEA_ERR_UNSUPPORTED, "scale"),
    (dict(scale=float("inf")), MEA_ERR_UNSUPPORTED, "scale"),
    (dict(scale=-0.5), MEA_ERR_UNSUPPORTED, "scale"),
    (dict(q=P + 8), MEA_ERR_UNSUPPORTED, "16-byte"),
    (dict(lse=P + 2), MEA_ERR_UNSUPPORTED, "4-byte"),
    (dict(num_seqs=70000), MEA_ERR_UNSUPPORTED, "65535"),
    (dict(max_seqlen_k=1 << 20, Hq=8, Hkv=8, D=128), MEA_ERR_UNSUPPORTED, "2^31"),
    # decode path (max_seqlen_q == 1) without the workspace it needs
    (dict(num_seqs=4, total_q=4, max_seqlen_q=1, max_seqlen_k=5000), MEA_ERR_INVALID, "workspace"),
    (dict(num_seqs=4, total_q=4, max_seqlen_q=1, max_seqlen_k=5000, workspace=P, workspace_bytes=100),
     MEA_ERR_INVALID, "workspace"),
    # prefill needs the V^T images in the workspace
    (dict(), MEA_ERR_INVALID, "workspace"),
    (dict(workspace=P, workspace_bytes=1000), MEA_ERR_INVALID, "workspace"),
    (dict(total_k=-1), MEA_ERR_INVALID, "negative"),
    # forced split entry point
    (dict(chunk_keys=100, total_q=4, max_seqlen_q=1), MEA_ERR_INVALID, "chunk_keys"),
    (dict(chunk_keys=0, total_q=4, max_seqlen_q=1), MEA_ERR_INVALID, "chunk_keys"),
    (dict(chunk_keys=256), MEA_ERR_INVALID, "max_seqlen_q == 1"),
])
def test_rejected_before_launch(kw, status, needle):
    assert call(**kw) == status
    assert needle in _native.mea_last_error()


def test_empty_key_side_may_be_null():
    """No keys at all: k and v are never read, so NULL passes the pointer
    check (the call below then stops at a later rule, before any launch);
    with keys, a NULL k is rejected."""
    assert call(k=None, v=None, total_k=0, max_seqlen_k=0, D=96) == MEA_ERR_UNSUPPORTED
    assert "D=96" in _native.mea_last_error()
    assert call(q=None, out=None, num_seqs=4, total_q=0, max_seqlen_q=0, D=96) == MEA_ERR_UNSUPPORTED
    assert call(k=None, total_k=365) == MEA_ERR_INVALID
    assert "non-NULL" in _native.mea_last_error()
    assert call(out=None) == MEA_ERR_INVALID


def call_paged(**kw):
    a = dict(q=P, k_cache=P, v_cache=P, out=P, lse=None, seqstart_q=P, seqstart_k=P, block_table=P,
             num_seqs=4, total_q=4, total_k=365, max_seqlen_q=1, max_seqlen_k=200, page_size=64,
             num_pages=10, max_blocks=4, Hq=8, Hkv=8, D=64, dtype=MEA_F16, causal=0, alibi_slopes=None,
             scale=0.125, workspace=P, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return _native.mea_fwd_paged(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(block_table=None), MEA_ERR_INVALID, "block_table"),
    (dict(block_table=P + 2), MEA_ERR_UNSUPPORTED, "block_table"),
    (dict(page_size=0), MEA_ERR_INVALID, "page_size > 0"),
    (dict(num_pages=0), MEA_ERR_INVALID, "num_pages > 0"),
    (dict(max_blocks=0), MEA_ERR_INVALID, "max_blocks > 0"),
    (dict(page_size=16), MEA_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(page_size=96), MEA_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(max_blocks=3), MEA_ERR_INVALID, "max_seqlen_k"),
    (dict(page_size=1 << 20, D=128, max_blocks=1), MEA_ERR_UNSUPPORTED, "2^31"),
    (dict(k_cache=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(D=96), MEA_ERR_UNSUPPORTED, "D=96"),
    (dict(workspace=None, workspace_bytes=0), MEA_ERR_INVALID, "workspace"),
])
def test_paged_rejected_before_launch(kw, status, needle):
    assert call_paged(**kw) == status
    assert needle in _native.mea_last_error()


def test_paged_empty_problem_is_a_noop():
    assert call_paged(num_seqs=0, total_q=0) == MEA_OK


@pytest.mark.parametrize("kw", [dict(num_seqs=0, total_q=0), dict(total_q=0, max_seqlen_q=0)])
def test_empty_problem_is_a_noop(kw):
    assert call(**kw) == MEA_OK


def test_workspace_size():
    ws = _native.mea_fwd_workspace_size
    # prefill: one D x 64 16-bit V^T image per key/value head and tile slot,
    # then one int32 flag per image, each part rounded up to 256 bytes, then
    # 256 bytes of work counters
    r256 = lambda x: -(-x // 256) * 256
    slots = (365 // 64 + 4) * 8
    assert ws(4, 365, 200, 200, 8, 8, 64, 0) == r256(slots * 64 * 128) + r256(slots * 4) + 256
    slots = (137663 // 64 + 64) * 8
    assert ws(64, 137663, 4085, 4085, 32, 8, 128, 0) == r256(slots * 128 * 128) + r256(slots * 4) + 256
    assert ws(4, 0, 200, 0, 8, 8, 64, 0) == 0
    # decode: float32 partials per (sequence, partial slot, query head); the
    # key axis is cut into pieces of W keys, ~256 (piece, head group)
    # workgroups in all; here 2 head groups (8 key/value heads, 4 per group)
    W = _native.mea_default_chunk_keys(1101299, 64, 8)
    assert W == 8608                                   # ceil(1101299 * 2 / 256) -> multiple of 32
    slots = -(-32680 // W) + 1                         # a sequence touches at most ceil(L / W) + 1 pieces
    assert ws(64, 1101299, 1, 32680, 64, 8, 128, 0) == 64 * slots * 64 * 129 * 4
    assert ws(64, 1101299, 1, 32680, 64, 8, 128, 256) == 64 * (128 + 1) * 64 * 129 * 4
    assert ws(64, 1101299, 1, 32680, 64, 8, 128, 100) == 0                  # not a multiple of 32
    assert ws(64, 1101299, 1, 32680, 64, 8, 128, 96) == 64 * (341 + 1) * 64 * 129 * 4
    assert ws(2, 200, 1, 100, 6, 4, 128, 0) == 0                            # Hq % Hkv != 0
    assert ws(4, 0, 1, 0, 8, 8, 128, 0) == 0                                # no keys at all
    assert _native.mea_default_chunk_keys(32768, 64, 8) == 256              # 2 x 32768 / 256
    assert _native.mea_default_chunk_keys(16384, 64, 8) == 128              # 2 x 16384 / 256
    assert _native.mea_default_chunk_keys(8192, 64, 8) == 128               # floor of 128 keys
    assert _native.mea_default_chunk_keys(0, 64, 8) == 128
    assert _native.mea_default_chunk_keys(0, 0, 0) == 128
    assert _native.mea_default_chunk_keys(1 << 24, 32, 1) == (1 << 24) * 2 // 256  # 1 head x 2 slices
    for T, Hq, h in [(1000, 1, 1), (8 * 4096, 64, 8), (200 * 32768, 64, 8), (3 * 77, 4, 2)]:
        c = _native.mea_default_chunk_keys(T, Hq, h)
        assert c % 32 == 0 and c >= 128


def call_bwd(**kw):
    a = dict(q=P, k=P, v=P, out=P, lse=P, dout=P, dq=P, dk=P, dv=P, seqstart_q=P, seqstart_k=P,
             num_seqs=4, total_q=365, total_k=365, max_seqlen_q=200, max_seqlen_k=200, Hq=8, Hkv=2, D=64,
             dtype=MEA_BF16, causal=1, alibi_slopes=None, scale=0.125, workspace=P,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return _native.mea_bwd(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lse=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(dout=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(out=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(dk=None), MEA_ERR_INVALID, "dq, dk and dv"),
    (dict(seqstart_q=None), MEA_ERR_INVALID, "seqstart"),
    (dict(total_q=-1), MEA_ERR_INVALID, "negative"),
    (dict(Hq=8, Hkv=3), MEA_ERR_INVALID, "Hq % Hkv"),
    (dict(causal=3), MEA_ERR_INVALID, "causal"),
    (dict(max_seqlen_q=0), MEA_ERR_INVALID, "max_seqlen_q == 0"),
    (dict(max_seqlen_k=0), MEA_ERR_INVALID, "max_seqlen_k == 0"),
    (dict(D=32), MEA_ERR_UNSUPPORTED, "D=32"),
    (dict(dtype=5), MEA_ERR_UNSUPPORTED, "dtype"),
    (dict(scale=0.0), MEA_ERR_UNSUPPORTED, "scale"),
    (dict(dv=P + 4), MEA_ERR_UNSUPPORTED, "16-byte"),
    (dict(dout=P + 2), MEA_ERR_UNSUPPORTED, "16-byte"),
    (dict(lse=P + 1), MEA_ERR_UNSUPPORTED, "4-byte"),
    (dict(num_seqs=70000), MEA_ERR_UNSUPPORTED, "65535"),
    (dict(max_seqlen_q=1 << 20, Hq=8, D=128), MEA_ERR_UNSUPPORTED, "2^31"),
    (dict(max_seqlen_k=1 << 22, Hkv=2, D=128), MEA_ERR_UNSUPPORTED, "2^31"),
    (dict(workspace=None, workspace_bytes=0), MEA_ERR_INVALID, "workspace"),
    (dict(workspace_bytes=1000), MEA_ERR_INVALID, "workspace"),
    (dict(workspace=P + 16), MEA_ERR_UNSUPPORTED, "256-byte"),
])
def test_bwd_rejected_before_launch(kw, status, needle):
    assert call_bwd(**kw) == status
    assert needle in _native.mea_last_error()


@pytest.mark.parametrize("kw", [dict(num_seqs=0), dict(total_q=0, total_k=0, max_seqlen_q=0, max_seqlen_k=0)])
def test_bwd_empty_problem_is_a_noop(kw):
    assert call_bwd(**kw) == MEA_OK


def test_bwd_workspace_size():
    ws = _native.mea_bwd_workspace_size

    def al(x):
        return -(-x // 256) * 256

    # two float32 [Hq, total_q] row terms (lse in log2 units, rowsum(dO * O))
    assert ws(4, 365, 365, 8, 2, 64) == 2 * al(8 * 365 * 4)
    assert ws(64, 137663, 137663, 32, 8, 128) == 2 * al(32 * 137663 * 4)
    assert ws(4, 0, 365, 8, 2, 64) == 0                 # keys only: nothing per row
    assert ws(4, 365, 0, 8, 2, 64) == 2 * al(8 * 365 * 4)
    assert ws(0, 10, 10, 8, 2, 64) == 0
    assert ws(4, 365, 365, 8, 3, 64) == 0
    assert ws(4, 365, 365, 8, 2, 96) == 0


def call_fp8(**kw):
    a = dict(q=P, k=P, v=P, q_scale=0.01, k_scale=0.02, v_scale=0.03, out=P, lse=None, seqstart_q=P,
             seqstart_k=P, num_seqs=4, total_q=365, total_k=365, max_seqlen_q=200, max_seqlen_k=200, Hq=8, Hkv=2,
             D=128, out_dtype=MEA_BF16, causal=1, alibi_slopes=None, scale=0.088, workspace=P,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return _native.mea_fwd_fp8(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(D=64), MEA_ERR_UNSUPPORTED, "D=128"),
    (dict(q_scale=0.0), MEA_ERR_UNSUPPORTED, "fp8 scales"),
    (dict(v_scale=float("inf")), MEA_ERR_UNSUPPORTED, "fp8 scales"),
    (dict(k_scale=-1.0), MEA_ERR_UNSUPPORTED, "fp8 scales"),
    (dict(q=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(out_dtype=9), MEA_ERR_UNSUPPORTED, "dtype"),
    (dict(workspace=None, workspace_bytes=0), MEA_ERR_INVALID, "workspace"),
    # decode-shaped calls take the split-KV kernels and their float32 partials
    (dict(total_q=4, max_seqlen_q=1, workspace=None, workspace_bytes=0), MEA_ERR_INVALID, "workspace"),
])
def test_fp8_rejected_before_launch(kw, status, needle):
    assert call_fp8(**kw) == status
    assert needle in _native.mea_last_error()


def call_paged_fp8(**kw):
    a = dict(q=P, k_cache=P, v_cache=P, q_scale=0.01, k_scale=0.02, v_scale=0.03, out=P, lse=None, seqstart_q=P,
             seqstart_k=P, block_table=P, num_seqs=4, total_q=4, total_k=365, max_seqlen_q=1, max_seqlen_k=200,
             page_size=64, num_pages=10, max_blocks=4, Hq=8, Hkv=2, D=128, out_dtype=MEA_BF16, causal=0,
             alibi_slopes=None, scale=0.088, workspace=P, workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return _native.mea_fwd_paged_fp8(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(D=64), MEA_ERR_UNSUPPORTED, "D=128"),
    (dict(k_scale=-1.0), MEA_ERR_UNSUPPORTED, "fp8 scales"),
    (dict(block_table=None), MEA_ERR_INVALID, "block_table"),
    (dict(page_size=96), MEA_ERR_UNSUPPORTED, "multiple of 64"),
    (dict(max_blocks=3), MEA_ERR_INVALID, "max_seqlen_k"),
    (dict(workspace=None, workspace_bytes=0), MEA_ERR_INVALID, "workspace"),
    (dict(max_seqlen_q=200, total_q=365, workspace_bytes=100), MEA_ERR_INVALID, "workspace"),
])
def test_paged_fp8_rejected_before_launch(kw, status, needle):
    """Validation of the paged fp8 entry point: the fp8 rules and the page
    rules both apply, before anything is launched."""
    assert call_paged_fp8(**kw) == status
    assert needle in _native.mea_last_error()


def test_paged_fp8_empty_call_is_ok():
    assert call_paged_fp8(num_seqs=0, total_q=0) == MEA_OK


def test_fp8_workspace_size():
    ws = _native.mea_fwd_fp8_workspace_size
    # prefill-shaped: the V^T tile images (and flags) of the 16-bit prefill path
    slots = (137663 // 64 + 64) * 8
    assert ws(64, 137663, 4094, 4094, 32, 8, 128) == -(-slots * 128 * 128 // 256) * 256 + -(-slots * 4 // 256) * 256 + 256
    # decode-shaped: float32 partials, num_seqs x slots x Hq x (D + 1) floats,
    # slots = ceil(max_seqlen_k / W) + 1 for pieces of W keys.  16-bit: two
    # groups of 4 key/value heads, W = 1101299 * 2 / 256 -> 8608 (a multiple
    # of 32); fp8 with 8 key/value heads: one group of 8 heads since
    # W = 1101299 / 256 -> 4320 is at least 2048 keys
    part = lambda slots: 64 * slots * 64 * 129 * 4
    assert _native.mea_fwd_workspace_size(64, 1101299, 1, 32680, 64, 8, 128, 0) == part(-(-32680 // 8608) + 1)
    assert ws(64, 1101299, 1, 32680, 64, 8, 128) == part(-(-32680 // 4320) + 1)
    # one 131072-key sequence: the 8-head pieces would be 512 keys, so fp8
    # keeps the 16-bit grouping and size; likewise with 4 key/value heads
    for args in [(1, 131072, 1, 131072, 64, 8, 128), (64, 1101299, 1, 32680, 32, 4, 128)]:
        w16 = _native.mea_fwd_workspace_size(*args, 0)
        assert w16 > 0 and ws(*args) == w16
    assert ws(4, 365, 2, 200, 8, 2, 64) == 0
    assert ws(0, 365, 2, 200, 8, 2, 128) == 0
    assert ws(4, 0, 2, 0, 8, 2, 128) == 0


def call_ffn(**kw):
    a = dict(x=P, w_gate=P, w_up=P, w_down=P, hidden=P, out=P, tokens=100, d_model=4096, d_ff=11008,
             dtype=MEA_BF16, stream=None)
    a.update(kw)
    return _native.mea_swiglu_ffn(**a)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(hidden=None), MEA_ERR_INVALID, "non-NULL"),
    (dict(tokens=-1), MEA_ERR_INVALID, "negative"),
    (dict(d_ff=0), MEA_ERR_INVALID, "d_ff > 0"),
    (dict(d_model=4000), MEA_ERR_UNSUPPORTED, "multiple of 256"),
    (dict(d_ff=11000), MEA_ERR_UNSUPPORTED, "multiple of 128"),
    (dict(d_model=1 << 17), MEA_ERR_UNSUPPORTED, "65536"),
    (dict(dtype=3), MEA_ERR_UNSUPPORTED, "dtype"),
    (dict(w_down=P + 8), MEA_ERR_UNSUPPORTED, "16-byte"),
])
def test_ffn_rejected_before_launch(kw, status, needle):
    assert call_ffn(**kw) == status
    assert needle in _native.mea_last_error()


def test_ffn_empty_is_a_noop():
    assert call_ffn(tokens=0) == MEA_OK


def test_noalloc_rejects_calls_beyond_its_scratch():
    """mea_fwd_noalloc checks the scratch a call needs against its fixed array
    before touching any device."""
    big = dict(num_seqs=64, total_q=137663, total_k=137663, max_seqlen_q=4085, max_seqlen_k=4085, Hq=32, Hkv=8,
               D=128)
    need = _native.mea_fwd_workspace_size(64, 137663, 4085, 4085, 32, 8, 128, 0)
    assert need > (32 << 20)
    st = _native.mea_fwd_noalloc(P, P, P, P, P, P, P, big["num_seqs"], big["total_q"], big["total_k"],
                                 big["max_seqlen_q"], big["max_seqlen_k"], big["Hq"], big["Hkv"], big["D"],
                                 MEA_BF16, 1, None, 0.088, None)
    assert st == MEA_ERR_UNSUPPORTED
    assert "scratch" in _native.mea_last_error() and str(need) in _native.mea_last_error()
    # malformed arguments are rejected by the usual validation, still before any device call
    st = _native.mea_fwd_noalloc(P, P, P, P, P, P, P, 2, 10, 10, 5, 5, 6, 4, 64, MEA_F16, 0, None, 0.125, None)
    assert st == MEA_ERR_INVALID


def test_mixed_workspace_size():
    """mea_fwd_mixed: the prefill part's V^T images and flags, then (256-byte
    aligned) the decode part's partials sized for the decode keys alone."""
    mws = _native.mea_fwd_mixed_workspace_size
    r256 = lambda x: -(-x // 256) * 256
    # 3 prefills (201 tokens, 437 keys) + 3 decode steps (1933 keys, longest 1000), Hq 8, Hkv 2, D 128
    pre = _native.mea_fwd_workspace_size(3, 437, 130, 1000, 8, 2, 128, 0)
    slots = (437 // 64 + 3) * 2
    assert pre == r256(slots * 128 * 128) + r256(slots * 4) + 256
    W = _native.mea_default_chunk_keys(1933, 8, 2)
    dec = 3 * (-(-1000 // W) + 1) * 8 * 129 * 4
    assert mws(6, 437 + 1933, 130, 1000, 3, 437, 1000, 8, 2, 128) == r256(pre) + dec
    assert mws(6, 2370, 130, 1000, 0, 0, 1000, 8, 2, 128) == _native.mea_fwd_workspace_size(6, 2370, 1, 1000, 8, 2,
                                                                                           128, 0)
    assert mws(6, 2370, 130, 1000, 7, 0, 1000, 8, 2, 128) == 0          # more prefills than sequences
    assert mws(6, 2370, 130, 1000, 3, 437, 1000, 6, 4, 128) == 0        # Hq % Hkv != 0


@pytest.mark.parametrize("mixed, needle", [
    ((7, 0, 0, 0), "num_prefill_seqs"),
    ((2, 2, 5, 0), "one query each"),
    ((2, 3, 5, 99), "decode_max_seqlen_k"),
    ((2, -1, 5, 0), "prefill_total_q"),
])
def test_mixed_rejected_before_launch(mixed, needle):
    n_pre, pre_q, pre_k, dmk = mixed
    st = _native.mea_fwd_mixed(P, P, P, P, P, P, P, 4, 5, 40, 4, 20, n_pre, pre_q, pre_k, dmk, 8, 2, 64,
                               MEA_F16, 1, None, 0.125, P, 1 << 20, None)
    assert st == MEA_ERR_INVALID
    assert needle in _native.mea_last_error()
