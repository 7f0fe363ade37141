"""The seeded input generator: determinism, page tables, positions, poison."""
import math

import pytest
import torch

import mla_inputs as M
from mla_inputs.configs import EXTRA_WORKLOADS, WORKLOAD_ORDER


@pytest.mark.parametrize("name", WORKLOAD_ORDER + EXTRA_WORKLOADS)
def test_mini_deterministic_and_consistent(name):
    a = M.make(name, 3, mini=True)
    b = M.make(name, 3, mini=True)
    assert torch.equal(a.q_nope, b.q_nope) and torch.equal(a.w_uv, b.w_uv)
    for sa, sb in zip(a.segments, b.segments):
        assert torch.equal(sa.cache.view(-1).float(), sb.cache.view(-1).float())
    spec = a.spec
    assert a.q_nope.shape == (spec.n_tok, spec.heads, spec.d_nope)
    assert a.q_pe.shape == (spec.n_tok, spec.heads, spec.d_rope)
    assert a.w_uk.shape == (spec.heads, spec.d_nope, spec.d_c)
    assert a.w_uv.shape == (spec.heads, spec.d_v, spec.d_c)
    for seg in a.segments:
        for bi in range(spec.batch):
            assert seg.rows(bi).shape == (int(seg.seq_lens[bi]), spec.row_width)
    c = M.make(name, 4, mini=True)
    assert not torch.equal(a.q_nope, c.q_nope)


def test_paged_block_table_is_injective():
    x = M.make("dsv3", 5, mini=True, poison=True)
    seg = x.segments[0]
    ids = seg.block_table[seg.block_table >= 0]
    assert ids.unique().numel() == ids.numel()
    assert int(ids.max()) < seg.cache.shape[0]
    # padding is -1 exactly past each request's pages
    for b in range(x.spec.batch):
        n = (int(seg.seq_lens[b]) + 63) // 64
        assert (seg.block_table[b, :n] >= 0).all() and (seg.block_table[b, n:] == -1).all()
        assert not seg.rows(b).float().isnan().any()
    # unused pages and page tails are poisoned
    assert seg.cache.float().isnan().any()


def test_poison_only_unreadable_rows():
    x = M.make("small", 1, mini=True, poison=True)
    seg = x.segments[0]
    for b in range(x.spec.batch):
        t = int(seg.seq_lens[b])
        assert not seg.cache[b, :t].float().isnan().any()
        assert seg.cache[b, t:].float().isnan().all()


def test_merge_positions():
    x = M.make("merge", 2, mini=True)
    off, on, onl = x.segments
    s_q = x.spec.s_q
    for b in range(x.spec.batch):
        o_b = int(x.offsets[b])
        assert int(off.shift[b]) == o_b and int(off.stored_base[b]) == 0
        assert int(on.shift[b]) == 0 and int(on.stored_base[b]) == o_b
        assert int(onl.stored_base[b]) == o_b + int(on.seq_lens[b])
        for s in range(s_q):
            # the query tokens are the last s_q rows of the online segment
            assert int(x.q_pos[b * s_q + s]) == o_b + int(on.seq_lens[b]) + int(onl.seq_lens[b]) - s_q + s
    assert (off.head_begin, off.head_count) == (0, 56)
    assert (on.head_begin, on.head_count) == (56, 8)
    assert (onl.head_begin, onl.head_count, onl.causal) == (0, 64, True)


def test_full_spec_structure():
    """Shapes of the five full-size configurations (no draws)."""
    s = M.WORKLOADS
    assert s["toy"].softmax_scale == pytest.approx(1 / math.sqrt(6))
    assert s["small"].softmax_scale == pytest.approx(1 / math.sqrt(192))
    assert s["dsv3"].segments[0].length_range == (1024, 32768)
    assert s["long"].segments[0].length == 262144
    assert s["merge"].offset_range == (0, 200000)
    assert [g.length for g in s["merge"].segments] == [16384, 16384, 2048]
