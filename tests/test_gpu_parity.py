"""GPU parity: the HIP library against the fp64 oracle, through the C ABI.

Every test here needs an MI355X and the built ``libmla_latent.so``.
"""
from __future__ import annotations

import math
from dataclasses import replace

import numpy as np
import pytest
import torch

import mla_inputs as M
import oracle.mla_direct as O
from mla_inputs.configs import EXTRA_WORKLOADS, SegSpec, Spec, WORKLOADS, WORKLOAD_ORDER
from parity_util import check_step, f64, sample_pairs, tol_check

pytestmark = pytest.mark.gpu

SEEDS = {name: i for i, name in enumerate(WORKLOAD_ORDER + EXTRA_WORKLOADS)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from mla_latent_cache_amd import load
    load()  # loud failure if the library is not built
    yield


def _run(x, **kw):
    from mla_latent_cache_amd.step import step_from_inputs
    st = step_from_inputs(x, **kw)
    out, o_lat, lse = st.run()
    torch.cuda.synchronize()
    return st, out, o_lat, lse


# ------------------------------------------------------------ whole chain, small
@pytest.mark.parametrize("name", WORKLOAD_ORDER + EXTRA_WORKLOADS)
def test_chain_mini(name):
    x = M.make(name, SEEDS[name], mini=True, poison=True)
    print(f"[parity] mini {name} seed {SEEDS[name]}", flush=True)
    _, out, o_lat, lse = _run(x)
    errs = check_step(x, out, o_lat, lse, label=name)
    print(f"[parity] {name}: {errs}", flush=True)


@pytest.mark.parametrize("name", ["dsv3", "long", "merge", "prefill", "int4", "int8", "qknorm_dsv3"])
@pytest.mark.parametrize("split_query", [True, False])
def test_chain_mini_query_format(name, split_query):
    """The row-owning kernel's two query formats: bf16 hi and lo planes
    written by the fused query kernel (what the step picks for these
    workloads), and the fp32 query split inside the decode."""
    x = M.make(name, SEEDS[name] + 40, mini=True, poison=True)
    print(f"[parity] mini {name} split_query={split_query}", flush=True)
    st, out, o_lat, lse = _run(x, split_query=split_query)
    assert st.q_split == split_query
    check_step(x, out, o_lat, lse, label=f"{name} split_query={split_query}")


@pytest.mark.parametrize("n_wg", [1, 3, 8, 64, 256])
def test_split_invariance_dsv3_mini(n_wg):
    x = M.make("dsv3", 7, mini=True, poison=True)
    _, out, o_lat, lse = _run(x, n_wg=n_wg)
    check_step(x, out, o_lat, lse, label=f"dsv3-mini n_wg={n_wg}")


@pytest.mark.parametrize("n_split", [1, 2, 3, 9, 40, 130])
def test_forced_n_split(n_split):
    x = M.make("long", 8, mini=True, poison=True)
    _, out, o_lat, lse = _run(x, n_wg=64, n_split=[n_split])
    check_step(x, out, o_lat, lse, label=f"long-mini n_split={n_split}")


@pytest.mark.parametrize("n_wg", [1, 3, 2048])
def test_grid_extremes(n_wg):
    """One workgroup for all the work, an odd count, and many more
    workgroups than shares of work (the idle ones plan, find no piece and
    exit); the merge layout's three segments and several row groups."""
    x = M.make("merge", 12, mini=True, poison=True)
    print(f"[parity] merge-mini n_wg={n_wg}", flush=True)
    _, out, o_lat, lse = _run(x, n_wg=n_wg)
    check_step(x, out, o_lat, lse, label=f"merge-mini n_wg={n_wg}")


@pytest.mark.parametrize("name", ["merge", "qknorm_dsv3"])
def test_repeatable_bitwise(name):
    x = M.make(name, 9, mini=True)
    st, out, o_lat, lse = _run(x)
    a = (out.clone(), o_lat.clone(), lse.clone())
    st.run()
    torch.cuda.synchronize()
    for u, v in zip(a, (st.out, st.o_lat, st.lse)):
        assert torch.equal(u.view(torch.uint8) if u.dtype != torch.float32 else u.view(torch.int32),
                           v.view(torch.uint8) if v.dtype != torch.float32 else v.view(torch.int32))


def test_outputs_fully_overwritten():
    x = M.make("dsv3", 10, mini=True, poison=True)
    from mla_latent_cache_amd.step import step_from_inputs
    st = step_from_inputs(x)
    for t in (st.o_lat, st.lse, st.out, st.q_lat):
        t.fill_(float("nan"))
    st.run()
    torch.cuda.synchronize()
    for t in (st.o_lat, st.lse, st.out, st.q_lat):
        assert torch.isfinite(t.float()).all()
    check_step(x, st.out, st.o_lat, st.lse, label="sentinel")


# ------------------------------------------------------------ edge cases
def _custom(name, dtype="bf16", heads=16, s_q=1, batch=None, segs=None, **kw):
    dims = dict(d_c=512, d_nope=128, d_rope=64, d_v=128) if dtype == "bf16" else \
        dict(d_c=4, d_nope=4, d_rope=2, d_v=4)
    return Spec(name=name, batch=batch, heads=heads, s_q=s_q, dtype=dtype, segments=segs, **dims, **kw)


EDGE = {
    "empty_and_one_row": _custom("edge-empty", batch=5, segs=(
        SegSpec("kv", lengths=(0, 1, 0, 65, 33), online=True),)),
    "all_empty": _custom("edge-all-empty", batch=2, segs=(SegSpec("kv", lengths=(0, 0), online=True),)),
    "many_requests": _custom("edge-many", batch=150, heads=8, segs=(
        SegSpec("kv", length_range=(0, 40), layout="paged", page_size=64, online=True),)),
    "rows_17": _custom("edge-rows17", batch=3, heads=17, segs=(
        SegSpec("kv", lengths=(100, 31, 257), online=True),)),
    "rows_48_sq3": _custom("edge-rows48", batch=2, heads=16, s_q=3, segs=(
        SegSpec("kv", lengths=(90, 3), causal=True, online=True),)),
    "rows_100": _custom("edge-rows100", batch=2, heads=100, segs=(
        SegSpec("kv", lengths=(300, 64), layout="paged", page_size=64, spare_pages=2, online=True),)),
    "causal_short_online": _custom("edge-causal", batch=2, heads=64, s_q=4, offset_range=(0, 200000), segs=(
        SegSpec("doc_off", lengths=(40, 0), head_begin=0, head_count=56, shift_offset=True),
        SegSpec("doc_on", lengths=(40, 0), head_begin=56, head_count=8, base_offset=True),
        SegSpec("online", lengths=(2, 5), causal=True, base_offset=True, base_after="doc_on", online=True),
    )),
    # 64-row groups score with the bf16-rounded latent query and correct the
    # lse to first order; scores twice as spread as the default scale and a
    # one-row request (lse = its score) make an uncorrected rounding of the
    # query miss the lse bound several times over
    "peaked_rows64": _custom("edge-peaked", batch=4, heads=64, scale=2 / math.sqrt(192), segs=(
        SegSpec("kv", lengths=(1, 37, 300, 1000), online=True),)),
    # four times the default spread: the first-order correction's remaining
    # lse error, evaluated on the CPU for these inputs, is 5e-5 (uncorrected
    # 1.5e-2; tests/test_lse_correction.py)
    "peaked4_rows64": _custom("edge-peaked4", batch=4, heads=64, scale=4 / math.sqrt(192), segs=(
        SegSpec("kv", lengths=(1, 37, 300, 1000), online=True),)),
    "toy_f32_ragged": _custom("edge-f32", dtype="f32", batch=3, heads=2, scale=1 / math.sqrt(6), segs=(
        SegSpec("kv", lengths=(16, 0, 130), layout="paged", page_size=8, spare_pages=1, online=True),)),
    # the fp32-cache decode at its largest dims and at odd ones
    "f32_max_dims": Spec(name="edge-f32-max", batch=3, heads=3, s_q=1, dtype="f32", d_c=512, d_nope=96,
                         d_rope=128, d_v=40, segments=(
                             SegSpec("kv", lengths=(1, 70, 257), layout="paged", page_size=64, spare_pages=1,
                                     online=True),)),
    "f32_odd_dims": Spec(name="edge-f32-odd", batch=3, heads=5, s_q=2, dtype="f32", d_c=300, d_nope=20,
                         d_rope=6, d_v=7, segments=(
                             SegSpec("kv", lengths=(0, 33, 100), causal=True, layout="paged", page_size=16,
                                     spare_pages=2, online=True),)),
    # QK-Norm: per-row key factors through each row-group size (16, 32, 64
    # query rows), contiguous and paged, and the fp32 path
    "qknorm_paged_rows64": _custom("edge-qkn64", batch=4, heads=64, qk_norm=True, segs=(
        SegSpec("kv", lengths=(1, 37, 300, 1000), layout="paged", page_size=64, spare_pages=2, online=True),)),
    "qknorm_rows32_sq2": _custom("edge-qkn32", batch=3, heads=16, s_q=2, qk_norm=True, qk_eps=0.5, segs=(
        SegSpec("kv", lengths=(2, 95, 513), causal=True, online=True),)),
    # 9 x 64 = 576 query rows: beyond the fused QK-Norm prepare, so the
    # query normalisation runs as its own launch before mla_prepare_q
    "qknorm_two_launch_rows576": _custom("edge-qkn576", batch=9, heads=64, qk_norm=True, segs=(
        SegSpec("kv", lengths=(0, 1, 5, 37, 64, 65, 100, 130, 300), online=True),)),
    # QK-Norm on the row-owning kernel: 128-row groups (two groups at 192
    # rows), twice-spread scores against the lse's first-order lo share with
    # the mean row factor, and the merge layout's segments in one launch
    "qknorm_rows128_peaked": _custom("edge-qkn128", batch=4, heads=128, qk_norm=True, scale=2 / math.sqrt(192),
                                     segs=(SegSpec("kv", lengths=(1, 37, 300, 1000), layout="paged", page_size=64,
                                                   spare_pages=2, online=True),)),
    "qknorm_rows192": _custom("edge-qkn192", batch=3, heads=64, s_q=3, qk_norm=True, segs=(
        SegSpec("kv", lengths=(3, 95, 513), causal=True, online=True),)),
    "qknorm_merge": _custom("edge-qknm", batch=2, heads=64, s_q=4, qk_norm=True, offset_range=(0, 200000), segs=(
        SegSpec("doc_off", lengths=(300, 33), head_begin=0, head_count=56, shift_offset=True),
        SegSpec("doc_on", lengths=(300, 33), head_begin=56, head_count=8, base_offset=True),
        SegSpec("online", lengths=(70, 4), causal=True, base_offset=True, base_after="doc_on", online=True),
    )),
    "qknorm_toy_f32": _custom("edge-qknf32", dtype="f32", batch=3, heads=2, qk_norm=True, segs=(
        SegSpec("kv", lengths=(16, 0, 130), layout="paged", page_size=8, spare_pages=1, online=True),)),
    # int8 latent cache (64-row groups of the row-owning kernel): one wave
    # with rows (16 rows), contiguous and paged, empty and one-row requests,
    # causal rows, the first-order lse correction with twice-spread scores,
    # two 64-row groups of one request (128 heads) and the merge layout's
    # segments in one launch
    "int8_rows16": _custom("edge-i8-16", batch=4, heads=16, quant="int8", segs=(
        SegSpec("kv", lengths=(0, 1, 37, 300), online=True),)),
    "int8_rows32_causal": _custom("edge-i8-32", batch=3, heads=16, s_q=2, quant="int8", segs=(
        SegSpec("kv", lengths=(2, 95, 513), causal=True, layout="paged", page_size=64, spare_pages=1,
                online=True),)),
    "int8_peaked_rows64": _custom("edge-i8-64", batch=4, heads=64, quant="int8", scale=2 / math.sqrt(192), segs=(
        SegSpec("kv", lengths=(1, 37, 300, 1000), online=True),)),
    "int8_rows128_paged": _custom("edge-i8-128", batch=3, heads=128, quant="int8", segs=(
        SegSpec("kv", lengths=(64, 130, 1500), layout="paged", page_size=64, spare_pages=3, online=True),)),
    "int8_merge_layout": replace(M.mini_spec("merge"), name="edge-i8-merge", quant="int8"),
    # int4 cache (latent and rotary codes, two scales per row): one wave with
    # rows (16 rows), causal rows over pages, 64-row groups with
    # twice-spread scores, two 64-row groups of one request (128 heads) and
    # the merge layout's segments in one launch
    "int4_rows16": _custom("edge-i4-16", batch=4, heads=16, quant="int4", segs=(
        SegSpec("kv", lengths=(0, 1, 37, 300), online=True),)),
    "int4_rows32_causal": _custom("edge-i4-32", batch=3, heads=16, s_q=2, quant="int4", segs=(
        SegSpec("kv", lengths=(2, 95, 513), causal=True, layout="paged", page_size=64, spare_pages=1,
                online=True),)),
    "int4_peaked_rows64": _custom("edge-i4-64", batch=4, heads=64, quant="int4", scale=2 / math.sqrt(192), segs=(
        SegSpec("kv", lengths=(1, 37, 300, 1000), online=True),)),
    "int4_rows128_paged": _custom("edge-i4-128", batch=3, heads=128, quant="int4", segs=(
        SegSpec("kv", lengths=(64, 130, 1500), layout="paged", page_size=64, spare_pages=3, online=True),)),
    "int4_merge_layout": replace(M.mini_spec("merge"), name="edge-i4-merge", quant="int4"),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_case(case):
    x = M.make_inputs(EDGE[case], seed=11, poison=True)
    print(f"[parity] edge {case}", flush=True)
    _, out, o_lat, lse = _run(x)
    check_step(x, out, o_lat, lse, label=case)


@pytest.mark.parametrize("case", ["qknorm_rows128_peaked", "qknorm_rows192", "qknorm_merge"])
def test_qknorm_rows_fp32_query(case):
    """QK-Norm on the row-owning kernel with the fp32 latent query (the kernel
    splits it itself) instead of the split planes the step writes by default."""
    x = M.make_inputs(EDGE[case], seed=12, poison=True)
    print(f"[parity] edge {case} fp32 query", flush=True)
    st, out, o_lat, lse = _run(x, split_query=False)
    assert not st.q_split
    check_step(x, out, o_lat, lse, label=case + " fp32 query")


# ------------------------------------------------------------ single calls
def _rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_relocate_call(dtype):
    from mla_latent_cache_amd import ops
    n_tok, H, d_r = 9, 5, (64 if dtype == torch.bfloat16 else 2)
    q_pe = _rand((n_tok, H, d_r), dtype, 1)
    g = torch.Generator().manual_seed(2)
    pos = torch.randint(0, 262144, (n_tok,), generator=g, dtype=torch.int64)
    shift = torch.randint(0, 200001, (n_tok,), generator=g, dtype=torch.int64)
    for sh, odt in ((None, dtype), (shift, dtype), (shift, torch.float32)):
        got = ops.rope_relocate_q(q_pe.cuda(), pos.cuda(), None if sh is None else sh.cuda(), 10000.0,
                                  out_dtype=odt)
        ref = O.rope_relocate(f64(q_pe), pos.numpy(), np.zeros(n_tok, np.int64) if sh is None else sh.numpy(),
                              10000.0)
        err = np.abs(f64(got) - ref)
        if odt == torch.float32:
            assert err.max() <= 1e-5, err.max()
        else:
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5), err.max()


@pytest.mark.parametrize("dtype,dims", [(torch.float32, (4, 4, 7)), (torch.bfloat16, (128, 512, 33)),
                                        (torch.bfloat16, (128, 512, 1)), (torch.bfloat16, (128, 512, 100))])
def test_absorb_and_out_uv_calls(dtype, dims):
    from mla_latent_cache_amd import ops
    d_nope, d_c, n_tok = dims
    H = 6
    q = _rand((n_tok, H, d_nope), dtype, 3)
    w = (_rand((H, d_nope, d_c), torch.float32, 4) / math.sqrt(d_c)).to(dtype)
    ref = O.absorb_query(f64(w), f64(q))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    for odt in {dtype, torch.float32}:
        got = ops.absorb_q(q.cuda(), w.cuda(), out_dtype=odt)
        rel = 1e-6 if odt == torch.float32 else 2.0 ** -8
        assert np.all(np.abs(f64(got) - ref) <= rel * np.abs(ref) + 1e-5 * rms), odt
    o = _rand((n_tok, H, d_c), dtype, 5)
    wv = (_rand((H, d_nope, d_c), torch.float32, 6) / math.sqrt(d_c)).to(dtype)
    ref = O.output_expand(f64(wv), f64(o))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    for odt in {dtype, torch.float32}:
        got = ops.out_uv(o.cuda(), wv.cuda(), out_dtype=odt)
        rel = 1e-6 if odt == torch.float32 else 2.0 ** -8
        assert np.all(np.abs(f64(got) - ref) <= rel * np.abs(ref) + 1e-5 * rms), odt


def _out_proj_bound(x, w, ref, rel):
    """|got - ref| <= rel |ref| (output rounding) + 1e-6 sum_k |x_k w_k| (fp32
    accumulation over k_in <= 16384 terms)."""
    s = np.abs(f64(x).reshape(x.shape[0], -1)) @ np.abs(f64(w)).T
    return rel * np.abs(ref) + 1e-6 * s


@pytest.mark.parametrize("dtype,n_tok,k_in,d_model", [
    (torch.float32, 1, 8, 8),            # fp32 toy: 2 heads x d_v 4
    (torch.bfloat16, 1, 2048, 2048),     # one token, 16 heads x 128
    (torch.bfloat16, 5, 2048, 2088),     # ragged feature tail (2088 = 32 x 64 + 40)
    (torch.bfloat16, 70, 4096, 1000),    # two token blocks, ragged tokens and features
    (torch.bfloat16, 64, 16384, 7168),   # 128 heads x 128, a wide model
    (torch.bfloat16, 3, 264, 100),       # k_in not a multiple of 256: the plain kernel
])
def test_out_proj_call(dtype, n_tok, k_in, d_model):
    """mla_out_proj against the oracle's shared output projection (fp64)."""
    from mla_latent_cache_amd import ops
    H = 2 if k_in == 8 else (k_in // 128 if k_in % 128 == 0 else 1)
    d_v = k_in // H
    v = _rand((n_tok, H, d_v), dtype, 31)
    w_o = (_rand((d_model, k_in), torch.float32, 32) / math.sqrt(k_in)).to(dtype)
    ref = O.output_projection(f64(w_o), f64(v))
    for odt in {dtype, torch.float32}:
        got = ops.out_proj(v.cuda(), w_o.cuda(), out_dtype=odt)
        assert got.shape == (n_tok, d_model)
        rel = 0.0 if odt == torch.float32 else 2.0 ** -8
        bound = _out_proj_bound(v, w_o, ref, rel)
        if dtype == torch.float32:  # the toy's bar: 1e-5 relative
            bound = np.maximum(bound, 1e-5 * np.abs(ref).max())
        err = np.abs(f64(got) - ref)
        assert np.all(err <= bound), (odt, float(err.max()), float((err - bound).max()))


def test_out_proj_after_out_uv_and_folded():
    """U_V then W_O (two calls, bf16 in between) and the folded form (o_lat
    against W_O[:, head h] U_V[h] side by side) both match the oracle's
    output_projection(W_O, output_expand(U_V, o_lat))."""
    from mla_latent_cache_amd import ops
    n_tok, H, d_c, d_v, d_model = 9, 16, 512, 128, 1536
    o = _rand((n_tok, H, d_c), torch.bfloat16, 33)
    wv = (_rand((H, d_v, d_c), torch.float32, 34) / math.sqrt(d_c)).to(torch.bfloat16)
    w_o = (_rand((d_model, H * d_v), torch.float32, 35) / math.sqrt(H * d_v)).to(torch.bfloat16)
    ref = O.output_projection(f64(w_o), O.output_expand(f64(wv), f64(o)))
    # two calls: the heads' outputs rounded to bf16 (relative 2^-9 each) before W_O
    v = ops.out_uv(o.cuda(), wv.cuda(), out_dtype=torch.bfloat16)
    got = ops.out_proj(v, w_o.cuda(), out_dtype=torch.float32)
    v_ref = O.output_expand(f64(wv), f64(o))
    s_v = np.abs(v_ref).reshape(n_tok, -1) @ np.abs(f64(w_o)).T
    err = np.abs(f64(got) - ref)
    assert np.all(err <= 2.0 ** -8 * s_v + 1e-5 * s_v), float(err.max())
    # folded: the fold rounded to bf16 (relative 2^-9 per entry)
    fold = O.fold_value_into_output(f64(w_o), f64(wv))          # [H, d_model, d_c]
    w_f = torch.from_numpy(np.ascontiguousarray(fold.transpose(1, 0, 2).reshape(d_model, H * d_c)))
    w_f = w_f.to(torch.bfloat16)
    got_f = ops.out_proj(o.cuda().reshape(n_tok, H * d_c), w_f.cuda(), out_dtype=torch.float32)
    s_f = np.abs(f64(o)).reshape(n_tok, -1) @ np.abs(f64(w_f)).T
    err_f = np.abs(f64(got_f) - ref)
    assert np.all(err_f <= 2.0 ** -8 * s_f + 1e-5 * s_f), float(err_f.max())


@pytest.mark.parametrize("dtype,dims", [(torch.float32, (4, 4, 2, 7)), (torch.bfloat16, (128, 512, 64, 33))])
def test_prepare_call(dtype, dims):
    """mla_prepare_q (rope for several shifts + absorb in one launch, or the
    two kernels in turn off the MFMA path) gives exactly what the separate
    calls give, and matches the oracle."""
    from mla_latent_cache_amd import ops
    d_nope, d_c, d_r, n_tok = dims
    H = 6
    q = _rand((n_tok, H, d_nope), dtype, 21)
    q_pe = _rand((n_tok, H, d_r), dtype, 22)
    w = (_rand((H, d_nope, d_c), torch.float32, 23) / math.sqrt(d_c)).to(dtype)
    g = torch.Generator().manual_seed(24)
    pos = torch.randint(0, 262144, (n_tok,), generator=g, dtype=torch.int64)
    shifts = [None] + [torch.randint(0, 200001, (n_tok,), generator=g, dtype=torch.int64) for _ in range(2)]
    dq, dpe, dw, dpos = q.cuda(), q_pe.cuda(), w.cuda(), pos.cuda()
    dsh = [None if s is None else s.cuda() for s in shifts]
    q_lat, q_rots = ops.prepare_q(dq, dpe, dw, dpos, dsh, 10000.0, lat_dtype=torch.float32,
                                  rot_dtype=torch.float32)
    lat_sep = ops.absorb_q(dq, dw, out_dtype=torch.float32)
    assert torch.equal(q_lat, lat_sep)
    for s, r in zip(dsh, q_rots):
        assert torch.equal(r, ops.rope_relocate_q(dpe, dpos, s, 10000.0, out_dtype=torch.float32))
    ref = O.absorb_query(f64(w), f64(q))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(f64(q_lat) - ref) <= 1e-6 * np.abs(ref) + 1e-5 * rms)
    for s, r in zip(shifts, q_rots):
        ref_r = O.rope_relocate(f64(q_pe), pos.numpy(), np.zeros(n_tok, np.int64) if s is None else s.numpy(),
                                10000.0)
        assert np.abs(f64(r) - ref_r).max() <= 1e-5


def test_prepare_fp32_query_bf16_weights():
    """mla_prepare_q with an fp32 query and bf16 U_K (the QK-Norm query): the
    MFMA path multiplies bf16 hi + lo parts of the query, so q_lat matches
    the fp64 absorption of the fp32 query to fp32 accumulation."""
    from mla_latent_cache_amd import ops
    H, d_nope, d_c, d_r, n_tok = 16, 128, 512, 64, 37
    q = _rand((n_tok, H, d_nope), torch.float32, 31) * 3
    q_pe = _rand((n_tok, H, d_r), torch.bfloat16, 32)
    w = (_rand((H, d_nope, d_c), torch.float32, 33) / math.sqrt(d_c)).to(torch.bfloat16)
    pos = torch.arange(n_tok, dtype=torch.int64) * 97
    q_lat, q_rots = ops.prepare_q(q.cuda(), q_pe.cuda(), w.cuda(), pos.cuda(), [None], 10000.0,
                                  lat_dtype=torch.float32, rot_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.absorb_query(f64(w), f64(q))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(f64(q_lat) - ref)
    assert np.all(err <= 1e-5 * np.abs(ref) + 2e-5 * rms), float(np.max(err / rms))
    # a bf16-rounded query would be off by ~2^-9 relative: the lo part is used
    ref_hi = O.absorb_query(f64(w), f64(q.to(torch.bfloat16)))
    assert np.max(np.abs(ref_hi - ref)) > 50 * np.max(err)
    ref_r = O.rope_relocate(f64(q_pe), pos.numpy(), np.zeros(n_tok, np.int64), 10000.0)
    assert np.abs(f64(q_rots[0]) - ref_r).max() <= 1e-5


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float32])
def test_prepare_split_query(q_dtype):
    """mla_prepare_q with lat_dtype MLA_BF16X2: its two planes are exactly
    the bf16 rounding of the fp32 result and the bf16 rounding of what that
    leaves (the same MFMA sums, only stored differently)."""
    from mla_latent_cache_amd import ops
    H, d_nope, d_c, d_r, n_tok = 16, 128, 512, 64, 37
    q = (_rand((n_tok, H, d_nope), torch.float32, 41) * 3).to(q_dtype)
    q_pe = _rand((n_tok, H, d_r), torch.bfloat16, 42)
    w = (_rand((H, d_nope, d_c), torch.float32, 43) / math.sqrt(d_c)).to(torch.bfloat16)
    pos = torch.arange(n_tok, dtype=torch.int64) * 31
    dq, dpe, dw, dpos = q.cuda(), q_pe.cuda(), w.cuda(), pos.cuda()
    q32, r32 = ops.prepare_q(dq, dpe, dw, dpos, [None], 10000.0, lat_dtype=torch.float32, rot_dtype=torch.float32)
    qx2, rx2 = ops.prepare_q(dq, dpe, dw, dpos, [None], 10000.0, rot_dtype=torch.float32, split=True)
    torch.cuda.synchronize()
    assert qx2.shape == (n_tok, H, 2, d_c) and qx2.dtype == torch.bfloat16
    hi = q32.to(torch.bfloat16)
    lo = (q32 - hi.float()).to(torch.bfloat16)
    assert torch.equal(qx2[:, :, 0], hi)
    assert torch.equal(qx2[:, :, 1], lo)
    assert torch.equal(rx2[0], r32[0])


@pytest.mark.parametrize("q_dtype,n_tok,H", [(torch.bfloat16, 1, 16), (torch.float32, 17, 16),
                                             (torch.bfloat16, 32, 16), (torch.float32, 4, 128)])
def test_prepare_qknorm_call(q_dtype, n_tok, H):
    """mla_prepare_q_qknorm: q_lat = U_K^T (g_q g_k q / rms over all heads)
    against the oracle's definition (one token, a ragged second token block,
    the 512-row limit with 16 and with 128 heads), its rotary outputs, and
    agreement with the two-launch form (mla_qknorm_query, then mla_prepare_q
    with the fp32 query) to the same fp32 bound."""
    from mla_latent_cache_amd import ops
    d_nope, d_c, d_r, eps = 128, 512, 64, 0.25
    q = _rand((n_tok, H, d_nope), q_dtype, 51) * 3
    q[0, 0] = 0                                     # one zero head: the statistic still spans all heads
    g_q = 1 + 0.1 * _rand((H, d_nope), torch.float32, 52)
    g_k = 1 + 0.1 * _rand((H, d_nope), torch.float32, 53)
    q_pe = _rand((n_tok, H, d_r), torch.bfloat16, 54)
    w = (_rand((H, d_nope, d_c), torch.float32, 55) / math.sqrt(d_c)).to(torch.bfloat16)
    pos = torch.arange(n_tok, dtype=torch.int64) * 131
    shift = torch.arange(n_tok, dtype=torch.int64) * 7 + 3
    qc, gqc, gkc, pec, wc, posc = (t.cuda() for t in (q, g_q, g_k, q_pe, w, pos))
    q_lat, q_rots = ops.prepare_q_qknorm(qc, gqc, gkc, eps, pec, wc, posc, [None, shift.cuda()],
                                         lat_dtype=torch.float32, rot_dtype=torch.float32)
    q_two, _ = ops.prepare_q(ops.qknorm_query(qc, gqc, gkc, eps), pec, wc, posc, [], lat_dtype=torch.float32)
    torch.cuda.synchronize()
    qn = np.stack([f64(g_q) * f64(g_k) * f64(q[t]) * O.rms_inverse(f64(q[t]), eps) for t in range(n_tok)])
    ref = O.absorb_query(f64(w), qn)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    for got in (q_lat, q_two):
        err = np.abs(f64(got) - ref)
        assert np.all(err <= 1e-5 * np.abs(ref) + 2e-5 * rms), float(np.max(err / rms))
    for sh, got in ((np.zeros(n_tok, np.int64), q_rots[0]), (shift.numpy(), q_rots[1])):
        ref_r = O.rope_relocate(f64(q_pe), pos.numpy(), sh, 10000.0)
        assert np.abs(f64(got) - ref_r).max() <= 1e-5


@pytest.mark.parametrize("out_dtype,n_rows,n_part", [(torch.float32, 37, 5), (torch.bfloat16, 37, 5),
                                                     (torch.float32, 600, 5), (torch.float32, 1100, 5),
                                                     (torch.bfloat16, 1030, 9),     # a wave per row from 1024 rows
                                                     (torch.float32, 1024, 130),    # ... over three slot chunks
                                                     (torch.bfloat16, 9, 300),      # slots beyond 128
                                                     (torch.float32, 7, 1024)])     # the largest slot count
@pytest.mark.parametrize("part_dtype", [torch.float32, torch.bfloat16])
def test_combine_call(out_dtype, n_rows, n_part, part_dtype):
    """Partials stored fp32 or bf16 (the oracle merges the same stored values)."""
    from mla_latent_cache_amd import ops
    d_c = 512
    g = torch.Generator().manual_seed(12)
    o_part = torch.randn((n_rows, n_part, d_c), generator=g).to(part_dtype)
    lse_part = torch.randn((n_rows, n_part), generator=g) * 4
    lse_part[3, :] = -math.inf                # empty row
    lse_part[4, 1:] = -math.inf               # one live slot
    lse_part[5, ::2] = -math.inf
    o_part[lse_part == -math.inf] = float("nan")  # never read
    o_lat, lse = ops.combine_lse(o_part.cuda(), lse_part.cuda(), out_dtype)
    torch.cuda.synchronize()
    for r in range(n_rows):
        o_ref, l_ref = O.merge_lse(f64(o_part[r]), f64(lse_part[r]))
        got = f64(o_lat[r])
        if math.isinf(l_ref):
            assert float(lse[r]) == -math.inf and not np.any(got)
            continue
        assert abs(float(lse[r]) - l_ref) <= 1e-5 * max(1.0, abs(l_ref))
        rel = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
        assert np.all(np.abs(got - o_ref) <= rel * np.abs(o_ref) + 1e-6), r


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_qknorm_query_wide(dtype):
    """mla_qknorm_query on rows wider than 16384 entries (160 heads x 128):
    the kernel that reads each row in rounds of four loads per thread."""
    from mla_latent_cache_amd import ops
    n_tok, H, d_nope, eps = 3, 160, 128, 1e-6
    q = _rand((n_tok, H, d_nope), dtype, 51)
    g_q = 1 + 0.1 * _rand((H, d_nope), torch.float32, 52)
    g_k = 1 + 0.1 * _rand((H, d_nope), torch.float32, 53)
    q_out = ops.qknorm_query(q.cuda(), g_q.cuda(), g_k.cuda(), eps)
    torch.cuda.synchronize()
    for t in range(n_tok):
        ref = f64(g_q) * f64(g_k) * f64(q[t]) * O.rms_inverse(f64(q[t]), eps)
        assert np.all(np.abs(f64(q_out[t]) - ref) <= 1e-5 * np.abs(ref) + 1e-7), t


@pytest.mark.parametrize("dtype,dims", [(torch.float32, (7, 5, 24, 40, 48, 37)),
                                        (torch.bfloat16, (3, 16, 128, 512, 576, 70)),
                                        (torch.float32, (4, 3, 6, 8, 10, 20)),        # 18 per token: scalar loads
                                        (torch.bfloat16, (5, 128, 128, 512, 576, 40))])  # 16384 per token
def test_qknorm_calls(dtype, dims):
    """mla_qknorm_query / _key_gram / _key_rinv against the direct RMS of the
    query over all heads and of each row's expanded key U_K c over all heads."""
    from mla_latent_cache_amd import ops
    n_tok, H, d_nope, d_c, rw, n_rows = dims
    eps = 0.25
    q = _rand((n_tok, H, d_nope), dtype, 41)
    g_q = 1 + 0.1 * _rand((H, d_nope), torch.float32, 42)
    g_k = 1 + 0.1 * _rand((H, d_nope), torch.float32, 43)
    w = (_rand((H, d_nope, d_c), torch.float32, 44) / math.sqrt(d_c)).to(dtype)
    rows = _rand((n_rows, rw), dtype, 45)
    rows[3] = 0                                 # zero key: rinv = 1/sqrt(eps) = 2
    q_out = ops.qknorm_query(q.cuda(), g_q.cuda(), g_k.cuda(), eps)
    gram = ops.qknorm_key_gram(w.cuda())
    rinv = ops.qknorm_key_rinv(rows.cuda(), gram, H, d_nope, eps)
    torch.cuda.synchronize()
    for t in range(n_tok):
        ref = f64(g_q) * f64(g_k) * f64(q[t]) * O.rms_inverse(f64(q[t]), eps)
        assert np.all(np.abs(f64(q_out[t]) - ref) <= 1e-5 * np.abs(ref) + 1e-7), t
    wf = f64(w).reshape(H * d_nope, d_c)
    g_ref = wf.T @ wf
    assert np.max(np.abs(f64(gram) - g_ref)) <= 1e-5 * np.max(np.abs(g_ref))
    r_ref = O.key_rms_inverse(f64(w), f64(rows)[:, :d_c], eps)
    assert abs(float(rinv[3]) - 2.0) <= 1e-6
    assert np.all(np.abs(f64(rinv) - r_ref) <= 1e-4 * r_ref)


def test_quantize_call():
    """mla_quantize_latent_i8 against the oracle's quantizer, bit for bit:
    codes, scales and the rotary bytes.  Rows: random at many magnitudes, a
    zero row, a row at unit scale with exact ties, one with a single nonzero."""
    import oracle.mla_quant as Q
    from mla_latent_cache_amd import ops
    g = torch.Generator().manual_seed(17)
    n, d_c, d_r = 1000, 512, 64
    rows = torch.randn((n, d_c + d_r), generator=g) * torch.exp(torch.empty((n, 1)).uniform_(-10, 10, generator=g))
    rows[3] = 0
    rows[4, :d_c] = torch.tensor([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -126.5, 126.5] * 64)
    rows[5, :d_c] = 0
    rows[5, 17] = -3.0
    rows = rows.to(torch.bfloat16)
    packed, scales = ops.quantize_latent_i8(rows.cuda(), d_c)
    torch.cuda.synchronize()
    packed = packed.cpu()
    codes_ref, scales_ref = Q.quantize_latent_i8(rows[:, :d_c].float().numpy())
    got_codes = packed[:, :d_c].view(torch.int8).numpy()
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), scales_ref.view(np.uint32))
    assert np.array_equal(got_codes, codes_ref), int(np.sum(got_codes != codes_ref))
    assert np.array_equal(packed[:, d_c:].numpy(), rows[:, d_c:].contiguous().view(torch.uint8).numpy())
    assert got_codes[4, :8].tolist() == [127, 0, 2, 2, 0, -2, -126, 126]
    assert float(scales[3]) == 0.0 and not np.any(got_codes[3])
    assert got_codes[5, 17] == -127 and int(np.count_nonzero(got_codes[5])) == 1


def test_quantize_i4_call():
    """mla_quantize_latent_i4 against the oracle's int4 quantizer, bit for
    bit: packed bytes and both scales.  Rows: random at many magnitudes, a
    zero row, a row at unit scale with exact ties in both parts, one with a
    single nonzero latent entry."""
    import oracle.mla_quant as Q
    from mla_latent_cache_amd import ops
    g = torch.Generator().manual_seed(18)
    n, d_c, d_r = 1000, 512, 64
    rows = torch.randn((n, d_c + d_r), generator=g) * torch.exp(torch.empty((n, 1)).uniform_(-10, 10, generator=g))
    rows[3] = 0
    rows[4] = torch.tensor([7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -6.5, 6.5] * 72)
    rows[5, :d_c] = 0
    rows[5, 17] = -3.0
    rows = rows.to(torch.bfloat16)
    packed, scales = ops.quantize_latent_i4(rows.cuda(), d_c)
    torch.cuda.synchronize()
    packed, scales = packed.cpu().numpy(), scales.cpu().numpy()
    p_ref, s_ref = Q.quantize_cache_i4(rows.float().numpy(), d_c)
    assert packed.shape == p_ref.shape and scales.shape == s_ref.shape
    assert np.array_equal(scales.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(packed, p_ref), int(np.sum(packed != p_ref))
    codes = Q.unpack_i4(packed)
    assert codes[4, :8].tolist() == [7, 0, 2, 2, 0, -2, -6, 6]
    assert codes[4, d_c:d_c + 8].tolist() == [7, 0, 2, 2, 0, -2, -6, 6]
    assert float(scales[3, 0]) == 0.0 and float(scales[3, 1]) == 0.0 and not np.any(packed[3])
    assert codes[5, 17] == -7 and int(np.count_nonzero(codes[5, :d_c])) == 1


# ------------------------------------------------------------ full sizes, sampled
@pytest.mark.parametrize("out_dtype,w_dtype,dims", [
    (torch.bfloat16, torch.bfloat16, (4, 16, 65, 512, 128)),   # the 512-column register path
    (torch.float32, torch.bfloat16, (3, 5, 9, 512, 128)),
    (torch.float32, torch.bfloat16, (2, 3, 7, 64, 8)),          # bf16 weights, other widths
    (torch.float32, torch.float32, (3, 2, 5, 4, 4)),            # the toy widths
    (torch.bfloat16, torch.float32, (2, 3, 7, 36, 20)),
    (torch.bfloat16, torch.bfloat16, (8, 12, 9, 512, 128)),    # 96 rows: two blocks per row
    (torch.float32, torch.bfloat16, (3, 50, 5, 512, 128)),     # 150 rows: one block per row
    # slots loaded ahead of their weights (up to 128 at four blocks per row,
    # 64 below) and the compacted rounds beyond
    (torch.bfloat16, torch.bfloat16, (1, 16, 65, 512, 128)),   # the small step's 65 slots
    (torch.float32, torch.bfloat16, (2, 8, 128, 512, 128)),
    (torch.float32, torch.bfloat16, (1, 4, 200, 512, 128)),
    (torch.bfloat16, torch.bfloat16, (5, 20, 70, 512, 128)),   # 100 rows: two blocks per row, 70 > 64
])
@pytest.mark.parametrize("part_dtype", [torch.float32, torch.bfloat16])
def test_combine_out_uv_call(out_dtype, w_dtype, dims, part_dtype):
    """Partials stored fp32 or bf16 (the oracle merges the same stored values)."""
    from mla_latent_cache_amd import ops
    n_tok, H, n_part, d_c, d_v = dims
    g = torch.Generator().manual_seed(13)
    o_part = torch.randn((n_tok, H, n_part, d_c), generator=g).to(part_dtype)
    lse_part = torch.randn((n_tok, H, n_part), generator=g) * 4
    lse_part[0, 0, :] = -math.inf              # empty row
    lse_part[0, 1 % H, 1:] = -math.inf         # one live slot
    lse_part[-1, -1, ::2] = -math.inf
    o_part[lse_part == -math.inf] = float("nan")  # never read
    w = (torch.randn((H, d_v, d_c), generator=g) / math.sqrt(d_c)).to(w_dtype)
    out, o_lat, lse = ops.combine_out_uv(o_part.cuda(), lse_part.cuda(), w.cuda(), out_dtype)
    torch.cuda.synchronize()
    o_ref = np.zeros((n_tok, H, d_c))
    l_ref = np.zeros((n_tok, H))
    for t in range(n_tok):
        for h in range(H):
            o_ref[t, h], l_ref[t, h] = O.merge_lse(f64(o_part[t, h]), f64(lse_part[t, h]))
    out_ref = O.output_expand(f64(w), o_ref)
    assert float(lse[0, 0]) == -math.inf and not np.any(f64(o_lat[0, 0])) and not np.any(f64(out[0, 0]))
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(f64(lse)), fin)
    assert np.all(np.abs(f64(lse)[fin] - l_ref[fin]) <= 1e-5 * np.maximum(1.0, np.abs(l_ref[fin])))
    rel = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(f64(o_lat) - o_ref) <= rel * np.abs(o_ref) + 1e-6)
    rms = float(np.sqrt(np.mean(out_ref ** 2)))
    assert np.all(np.abs(f64(out) - out_ref) <= rel * np.abs(out_ref) + 1e-5 * rms)


@pytest.mark.parametrize("name", ["small", "dsv3", "long", "merge", "prefill", "qknorm", "int8", "int4",
                                  "qknorm_dsv3"])
def test_full_size_sampled(name):
    """The bench's launch configuration (default grid) at full size; the
    oracle checks sampled (request, head) pairs."""
    x = M.make(name, SEEDS[name])
    print(f"[parity] full {name} seed {SEEDS[name]}", flush=True)
    _, out, o_lat, lse = _run(x)
    n_req = {"small": 2, "dsv3": 3, "long": 1, "merge": 2, "prefill": 1, "qknorm": 2, "int8": 1, "int4": 1,
             "qknorm_dsv3": 3}[name]
    reqs, heads = sample_pairs(x, n_req, 3, seed=SEEDS[name])
    errs = check_step(x, out, o_lat, lse, requests=reqs, heads=heads, label=f"{name} full")
    print(f"[parity] {name} full reqs={reqs} heads={heads}: {errs}", flush=True)
    # every output finite, every lse finite (no request is empty at full size)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


# ------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name", ["dsv3", "merge", "qknorm", "int8", "small", "qknorm_dsv3"])
def test_graph_replay_matches_eager(name):
    """The five calls enqueue only kernels on the caller's stream, so a step
    can be captured into a HIP graph; every replay must equal the eager run."""
    from mla_latent_cache_amd.step import run_calls, step_from_inputs
    x = M.make(name, 21, mini=True, poison=True)
    st = step_from_inputs(x)
    st.run()
    torch.cuda.synchronize()
    ref = (st.out.clone(), st.o_lat.clone(), st.lse.clone())
    cap = torch.cuda.Stream()
    pre, dec, post = st.bind(cap)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run_calls(pre)
        run_calls(dec)
        run_calls(post)
    for rep in range(3):
        for t in (st.out, st.o_lat, st.lse):
            t.fill_(float("nan"))         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (st.out, st.o_lat, st.lse)):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
