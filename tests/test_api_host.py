"""Host-side logic of the Python binding (no GPU): masks, splitting, layouts."""
import pytest
import torch

from memory_efficient_attention_amd import BlockDiagonalCausalMask, BlockDiagonalMask
from memory_efficient_attention_amd.api import _kv_heads_bmghk


def test_from_seqlens_offsets():
    m = BlockDiagonalMask.from_seqlens([37, 120, 8, 200])
    assert m.q_seqstart == [0, 37, 157, 165, 365] and m.kv_seqstart == m.q_seqstart
    assert (m.num_seqs, m.total_q, m.max_seqlen_q, m.causal) == (4, 365, 200, False)
    c = BlockDiagonalCausalMask.from_seqlens([1, 1], [10, 20])
    assert c.causal and c.kv_seqstart == [0, 10, 30] and c.max_seqlen_kv == 20


def test_split_shapes_match_the_tutorial():
    """Packed [1, 365, 8, 64] output splits into [1, L_b, 8, 64] pieces
    (tutorial page, section 4)."""
    m = BlockDiagonalMask.from_seqlens([37, 120, 8, 200])
    out = torch.arange(365 * 8 * 64, dtype=torch.float32).view(1, 365, 8, 64)
    pieces = m.split(out)
    assert [tuple(p.shape) for p in pieces] == [(1, 37, 8, 64), (1, 120, 8, 64), (1, 8, 8, 64), (1, 200, 8, 64)]
    assert torch.equal(torch.cat(pieces, dim=1), out)
    assert pieces[1].data_ptr() == out[0, 37].data_ptr()            # views, not copies
    assert [tuple(p.shape) for p in m.split(out[0])] == [(1, 37, 8, 64), (1, 120, 8, 64), (1, 8, 8, 64), (1, 200, 8, 64)]


def test_bad_masks():
    with pytest.raises(ValueError):
        BlockDiagonalMask.from_seqlens([1, 2], [3])
    with pytest.raises(ValueError):
        BlockDiagonalMask.from_seqlens([-1])
    with pytest.raises(ValueError):
        BlockDiagonalMask.from_seqlens([3, 4]).split(torch.zeros(1, 8, 2))


def test_bmghk_kv_head_axis():
    B, M, G, Hg, K = 2, 5, 2, 4, 8
    k = torch.randn(B, M, G, 1, K)
    kk = _kv_heads_bmghk(k, Hg)
    assert kk.shape == (B, M, G, K) and torch.equal(kk, k[:, :, :, 0])
    ke = _kv_heads_bmghk(k.expand(B, M, G, Hg, K), Hg)                # broadcast view
    assert torch.equal(ke, kk)
    full = torch.randn(B, M, G, Hg, K)
    kf = _kv_heads_bmghk(full, Hg)
    assert kf.shape == (B, M, G * Hg, K) and torch.equal(kf[:, :, 5], full[:, :, 1, 1])
    with pytest.raises(ValueError):
        _kv_heads_bmghk(torch.randn(B, M, G, 3, K), Hg)


def test_to_paged_round_trip():
    """The paging helper used by the paged parity tests: gathering every
    sequence's pages back in block-table order reproduces its keys and values,
    and every other slot holds the filler."""
    import math as _m
    from mea_workloads import random_case, to_paged
    inp = random_case(5, [1, 1, 1, 1], [0, 64, 65, 300], Hq=4, Hkv=2, D=64, dtype="fp16")
    pk = to_paged(inp, 64, seed=3, spare_pages=2)
    sk = inp.seqstart_k.tolist()
    used = set()
    for b, L in enumerate(inp.seqlens_k):
        nb = -(-L // 64)
        pages = pk.block_table[b, :nb].tolist()
        used.update(pages)
        k = torch.cat([pk.k_cache[p] for p in pages])[:L] if nb else pk.k_cache[:0, 0]
        v = torch.cat([pk.v_cache[p] for p in pages])[:L] if nb else pk.v_cache[:0, 0]
        assert torch.equal(k, inp.k[sk[b]:sk[b + 1]]) and torch.equal(v, inp.v[sk[b]:sk[b + 1]])
        if nb and L % 64:
            assert torch.isnan(pk.k_cache[pages[-1], L % 64:].float()).all()
    assert len(used) == sum(-(-L // 64) for L in inp.seqlens_k)
    spare = [p for p in range(pk.k_cache.shape[0]) if p not in used]
    assert len(spare) == 2 and all(torch.isnan(pk.v_cache[p].float()).all() for p in spare)
    assert not _m.isnan(float(pk.block_table.sum()))


def test_output_buffer_checks():
    """Caller-supplied outputs are validated before any pointer reaches the
    kernels (they store full-size rows through it)."""
    from memory_efficient_attention_amd.api import _check_out
    dev = torch.device("cpu")
    good = torch.empty(5, 4, 64, dtype=torch.bfloat16)
    _check_out(good, "out", (5, 4, 64), torch.bfloat16, dev)
    _check_out(None, "out", (5, 4, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError, match="shape"):
        _check_out(torch.empty(4, 4, 64, dtype=torch.bfloat16), "out", (5, 4, 64), torch.bfloat16, dev)
    with pytest.raises(TypeError, match="must be torch.bfloat16"):
        _check_out(torch.empty(5, 4, 64, dtype=torch.float32), "out", (5, 4, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError, match="contiguous"):
        _check_out(torch.empty(4, 5, 64, dtype=torch.bfloat16).transpose(0, 1), "out", (5, 4, 64),
                   torch.bfloat16, dev)
    with pytest.raises(ValueError, match="must be on"):
        _check_out(torch.empty(5, 4, 64, dtype=torch.bfloat16, device="meta"), "out", (5, 4, 64),
                   torch.bfloat16, dev)
    with pytest.raises(ValueError, match="lse must have shape"):
        _check_out(torch.empty(5, 4, dtype=torch.float32), "lse", (4, 5), torch.float32, dev)


def test_workspace_checks():
    from memory_efficient_attention_amd.api import _workspace
    dev = torch.device("cpu")
    assert _workspace(None, 0, dev) is None
    ws = torch.empty(4096, dtype=torch.uint8)
    assert _workspace(ws, 4096, dev) is ws
    assert _workspace(ws, 1000, dev) is ws
    bigger = _workspace(ws, 4097, dev)                   # too small: a new one
    assert bigger is not ws and bigger.numel() == 4097
    assert _workspace(torch.empty(1024, dtype=torch.float32), 4096, dev).numel() == 1024  # bytes, not elements
    with pytest.raises(ValueError, match="contiguous"):
        _workspace(torch.empty(64, 128, dtype=torch.uint8).t(), 16, dev)
    with pytest.raises(ValueError, match="must be on"):
        _workspace(torch.empty(64, dtype=torch.uint8, device="meta"), 16, dev)


def test_mixed_split():
    """A batch of prefills followed by one-query decode steps is recognised
    (the layout the mixed entry point serves); anything else is not."""
    m = BlockDiagonalCausalMask.from_seqlens([130, 7, 64, 1, 1, 1], [130, 7, 300, 900, 33, 1000])
    assert m.mixed_split() == (3, 201, 437, 1000)
    assert BlockDiagonalMask.from_seqlens([1, 1, 1], [10, 20, 30]).mixed_split() is None     # decode only
    assert BlockDiagonalMask.from_seqlens([10, 20], [10, 20]).mixed_split() is None          # prefill only
    assert BlockDiagonalMask.from_seqlens([1, 50, 1], [9, 50, 9]).mixed_split() == (2, 51, 59, 9)
    assert BlockDiagonalMask.from_seqlens([1, 1, 1, 1], [9, 8, 7, 6]).mixed_split() is None
    assert BlockDiagonalMask.from_seqlens([0, 2, 1], [5, 2, 7]).mixed_split() == (2, 2, 7, 7)
