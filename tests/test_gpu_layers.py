"""GPU parity of the layers and the backbone against the oracle.

Each case runs the HIP path through the C ABI and the float64 oracle on the
same seeded inputs (bf16-rounded where the device stores bf16) and compares
X', the residual branch dX = X' - X, the attention output A and the gated
Y = GLN2(A) (.) U element by element:  max|gpu - ref| <= tol * max|ref| per
tensor, tol = 1e-2 for bf16 storage / fp32 accumulation, 1e-4 for fp32.
dX is read through the stored X', so the half-ulp rounding of X' itself is
allowed for before its error is taken relative to max|dX_ref|.
"""
import numpy as np
import pytest

import synth
from oracle import model as om
from tests._parity import TOL_BF16, TOL_F32, Report, rounded_inputs, say, target_key_splits, to_np, ws_tensor

pytestmark = pytest.mark.gpu


def _run_layer(wl, kind, users_ref=None, inplace=False):
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    say(f"layer parity: {wl.name} {kind} rows={wl.batch.total_rows} users={wl.batch.n_users}")
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    op = B.OP_FULL if kind == "full" else B.OP_TARGET
    ws = B.workspace(dw.batch, dw.dims, op)
    x_in = dw.x
    x_out = x_in.clone() if inplace else torch.empty_like(x_in)
    if kind == "full":
        B.attn_full(dw.batch, dw.dims, meta, dw.full[0], x_out if inplace else x_in, x_out, ws)
    else:
        B.attn_target(dw.batch, dw.dims, meta, dw.target[0], x_out if inplace else x_in, x_out, ws)
    torch.cuda.synchronize()
    off_a, off_y = B.workspace_probe(dw.batch, dw.dims, op)
    hd = wl.dims.n_q_heads * wl.dims.head_dim
    rows = wl.batch.total_rows if kind == "full" else wl.batch.total_t_rows
    a = to_np(ws_tensor(ws, off_a, rows, hd, wl.dtype))
    y = to_np(ws_tensor(ws, off_y, rows, hd, wl.dtype))
    return to_np(x_in), to_np(x_out), a, y


def _ref_layer(wl, kind):
    x, full, tgt = rounded_inputs(wl)
    if kind == "full":
        out, parts = om.full_layer(wl.batch, x, full[0], wl.dims, return_parts=True)
    else:
        out, parts = om.target_layer(wl.batch, x, tgt[0], wl.dims, return_parts=True)
    return x, out, parts


def _compare(wl, kind, got, tol):
    x_dev, out_dev, a_dev, y_dev = got
    x_ref, out_ref, parts = _ref_layer(wl, kind)
    np.testing.assert_array_equal(x_dev, x_ref)        # the device saw the same inputs
    r = Report(tol)
    r.close("X'", out_dev, out_ref)
    r.branch("dX", out_dev, out_ref, x_ref, wl.dtype)
    r.close("A", a_dev, parts["a"])
    r.close("Y", y_dev, parts["y"])
    r.check()
    return out_ref


def test_config0_full_layer_fp32():
    wl = synth.config0()
    _compare(wl, "full", _run_layer(wl, "full"), TOL_F32)


def test_config1_full_layer_bf16():
    wl = synth.config1()
    _compare(wl, "full", _run_layer(wl, "full"), TOL_BF16)


@pytest.mark.parametrize("split", [1, 4])
def test_config2_target_layer_bf16(split):
    wl = synth.config2(split)
    got = _run_layer(wl, "target")
    _compare(wl, "target", got, TOL_BF16)
    x_dev, out_dev = got[0], got[1]
    for u in range(wl.batch.n_users):      # H and R rows are copied bit-exactly
        r0 = wl.batch.row_off[u]
        lc = int(wl.batch.lens[u, 0] + wl.batch.lens[u, 1])
        np.testing.assert_array_equal(out_dev[r0:r0 + lc], x_dev[r0:r0 + lc])


def test_config2_target_layer_in_place():
    wl = synth.config2(4)
    a = _run_layer(wl, "target", inplace=False)
    b = _run_layer(wl, "target", inplace=True)
    np.testing.assert_array_equal(a[1], b[1])


def _small_workload(lens, split, dtype, seed, dims=None, w_std=0.05):
    rng = np.random.default_rng(seed)
    batch = synth.make_batch(rng, np.asarray(lens, np.int32), split)
    dims = dims or synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    wf = synth.full_weights(rng, dims, w_std, w_std)
    wt = synth.target_weights(rng, dims, split, w_std, w_std)
    return synth.Workload(f"edge_{seed}", batch, dims, dtype, x, full=[wf], target=[wt])


EDGE_LENS = [[0, 0, 0], [64, 0, 0], [0, 64, 0], [0, 0, 3], [130, 64, 17], [1, 0, 1], [63, 1, 0], [0, 0, 0],
             [65, 63, 33], [5, 200, 2]]


@pytest.mark.parametrize("split", [1, 4])
@pytest.mark.parametrize("kind", ["full", "target"])
def test_edge_users_bf16(kind, split):
    wl = _small_workload(EDGE_LENS, split, "bf16", 40 + split)
    _compare(wl, kind, _run_layer(wl, kind), TOL_BF16)


@pytest.mark.parametrize("kind", ["full", "target"])
def test_edge_users_fp32(kind):
    dims = synth.Dims(128, 4, 2, 32)
    wl = _small_workload(EDGE_LENS, 4, "f32", 50, dims=dims, w_std=0.1)
    _compare(wl, kind, _run_layer(wl, kind), TOL_F32)


@pytest.mark.parametrize("n_users", [2048, 2049])
def test_many_users_with_and_without_work_order(n_users):
    """Up to 2048 users the attention grids take the XCD-balanced work order from the metadata;
    past that the plain XCD-contiguous order.  Both on many small users, every row against the oracle."""
    rng = np.random.default_rng(90)
    lens = np.stack([rng.integers(0, 41, n_users), rng.integers(0, 21, n_users), rng.integers(0, 7, n_users)], 1)
    wl = _small_workload(lens, 1, "bf16", 91)
    _compare(wl, "full", _run_layer(wl, "full"), TOL_BF16)
    _compare(wl, "target", _run_layer(wl, "target"), TOL_BF16)



def test_longest_user_within_the_key_offset_bound():
    """The longest user the bf16 attention takes at d 1024 with 16 query and 16 KV heads (8 KB
    of U|Q|K|V per packed row): 262,000 rows, whose keys span 2.15e9 bytes of the K buffer the
    kernel addresses through 32-bit offsets from the user's first row.  Behind a 60-row user (so
    the long user starts mid-tile), its sampled rows against the oracle; one row more than the
    bound allows (262,100) is refused with MTFM_E_UNSUPPORTED before the attention launch."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    rng = np.random.default_rng(93)
    dims = synth.Dims(1024, 16, 16, 64)
    l_h, l_r, l_t = 200_000, 61_992, 8
    batch = synth.make_batch(rng, np.array([[37, 20, 3], [l_h, l_r, l_t]], np.int32), 1)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    wl = synth.Workload("longest_user", batch, dims, "bf16", x, full=[synth.full_weights(rng, dims, 0.02, 0.02)])
    x_dev, out_dev, _, _ = _run_layer(wl, "full")
    xr, full, _ = rounded_inputs(wl)
    np.testing.assert_array_equal(x_dev, xr)
    off = batch.row_off
    r = Report(TOL_BF16)
    r.close("X' (60-row user)", out_dev[off[0]:off[1]], om.full_layer(batch.subset([0]), xr[off[0]:off[1]], full[0], dims))
    # first and last rows of each part and of 64-row tiles, and the T rows
    sel = np.array([0, 1, 63, 64, 131_071, l_h - 1, l_h, l_h + 1, l_h + 31_000, l_h + l_r - 1] +
                   list(range(l_h + l_r, l_h + l_r + l_t)))
    say(f"  oracle on {len(sel)} rows of the {l_h + l_r + l_t}-row user")
    ts_r = batch.ts_r[batch.r_off[1]:batch.r_off[2]]
    ts_t = batch.ts_t[batch.t_off[1]:batch.t_off[2]]
    ref = om.full_layer_rows(xr[off[1]:off[2]], l_h, l_r, l_t, 1, ts_r, ts_t, full[0], dims, sel)
    r.close("X' (262,000-row user, sampled rows)", out_dev[off[1] + sel], ref)
    r.branch("dX (262,000-row user, sampled rows)", out_dev[off[1] + sel], ref, xr[off[1] + sel], "bf16")
    r.check()
    del x_dev, out_dev, xr, x
    torch.cuda.empty_cache()

    over = synth.make_batch(rng, np.array([[262_100, 0, 0]], np.int32), 1)
    wl2 = synth.Workload("over_the_bound", over, dims, "bf16", np.zeros((over.total_rows, dims.d_model), np.float32),
                         full=[wl.full[0]])
    dw = DeviceWorkload(wl2)
    meta = B.mask_build(dw.batch)
    ws = B.workspace(dw.batch, dw.dims, B.OP_FULL)
    with pytest.raises(B.MtfmError) as e:
        B.attn_full(dw.batch, dw.dims, meta, dw.full[0], dw.x, torch.empty_like(dw.x), ws)
    assert e.value.status == B.E_UNSUPPORTED


def test_fp32_head_dim_64_and_gqa_ratio_1():
    dims = synth.Dims(128, 2, 2, 64)
    wl = _small_workload([[20, 9, 4], [70, 3, 1]], 1, "f32", 51, dims=dims, w_std=0.1)
    _compare(wl, "full", _run_layer(wl, "full"), TOL_F32)


@pytest.mark.parametrize("heads", [(8, 8), (8, 4), (8, 1)])
def test_bf16_other_gqa_ratios(heads):
    dims = synth.Dims(512, heads[0], heads[1], 64)
    wl = _small_workload([[150, 40, 20], [70, 90, 5]], 1, "bf16", 52, dims=dims)
    _compare(wl, "full", _run_layer(wl, "full"), TOL_BF16)
    _compare(wl, "target", _run_layer(wl, "target"), TOL_BF16)


def test_layers_are_deterministic():
    wl = synth.config1()
    a = _run_layer(wl, "full")
    b = _run_layer(wl, "full")
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])


def _backbone_gpu(wl, hoist=True):
    """Run the backbone; hoist=False gives it only the layer-by-layer workspace."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    dw = DeviceWorkload(wl)
    meta = B.mask_build(dw.batch)
    ws = B.workspace(dw.batch, dw.dims, B.OP_BACKBONE, k_target=wl.k_target if hoist else 0)
    x = dw.x.clone()
    B.backbone_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, x, ws)
    torch.cuda.synchronize()
    return to_np(dw.x), to_np(x)


def test_config3_backbone_sampled_users():
    """Full 160-user, 16-layer bf16 batch on the GPU (the benchmarked launch); oracle on sampled users."""
    wl = synth.config3()
    say(f"backbone parity: {wl.batch.n_users} users, {wl.batch.total_rows} rows, 16 layers")
    x0, got = _backbone_gpu(wl)
    xr, full, tgt = rounded_inputs(wl)
    np.testing.assert_array_equal(x0, xr)
    users = [0, 77, 159]
    ref = om.backbone(wl.batch, xr, full, tgt, wl.dims, wl.n_blocks, wl.k_target, boundary=om.bf16_round,
                      users=users)
    rows = wl.batch.rows_of(users)
    assert np.all(np.isfinite(got))
    r = Report(TOL_BF16)
    r.close("X' (3 users)", got[rows], ref)
    r.branch("dX (3 users, 16 roundings allowed)", got[rows], ref, xr[rows], "bf16", roundings=16)
    r.check()


def test_config3_backbone_composition_fp32():
    """The same 16-layer stack and weights for 3 of its users through the fp32 path (no bf16
    boundary rounding): the residual branch is resolved to fp32 precision."""
    wl = synth.config3()
    users = [0, 77, 159]
    xr, full, tgt = rounded_inputs(wl)
    sub = synth.Workload("cfg3_3users_f32", wl.batch.subset(users), wl.dims, "f32",
                         xr[wl.batch.rows_of(users)].astype(np.float32), full=full, target=tgt,
                         n_blocks=wl.n_blocks, k_target=wl.k_target)
    x0, got = _backbone_gpu(sub)
    ref = om.backbone(sub.batch, x0, full, tgt, wl.dims, wl.n_blocks, wl.k_target)
    r = Report(TOL_F32)
    r.close("X'", got, ref)
    r.branch("dX", got, ref, x0, "f32", roundings=16)
    r.check()


def _small_backbone(split, seed, n_blocks=2, k_target=3):
    rng = np.random.default_rng(seed)
    lens = np.stack([rng.integers(40, 200, 6), rng.integers(0, 90, 6), rng.integers(0, 20, 6)], 1).astype(np.int32)
    lens[2] = (70, 0, 5)      # no R rows
    lens[4] = (30, 50, 0)     # no T rows
    batch = synth.make_batch(rng, lens, split)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    full = [synth.full_weights(rng, dims, 0.02, 0.02) for _ in range(n_blocks)]
    tgt = [synth.target_weights(rng, dims, split, 0.02, 0.02) for _ in range(n_blocks * k_target)]
    return synth.Workload(f"small_backbone_s{split}", batch, dims, "bf16", x, full=full, target=tgt,
                          n_blocks=n_blocks, k_target=k_target)


@pytest.mark.parametrize("split,k_target", [(1, 3), (4, 3), (1, 1), (1, 2), (4, 4)])
def test_backbone_context_stage_matches_layer_by_layer(split, k_target):
    """The block-level context stage (one normalisation pass and the K/V of all target layers
    right after the full layer, one grouped projection launch) computes bit-identical outputs to
    running the layers one by one, for 1 to 4 target layers per block."""
    wl = _small_backbone(split, 60 + split + 10 * k_target, k_target=k_target)
    _, a = _backbone_gpu(wl, hoist=True)
    _, b = _backbone_gpu(wl, hoist=False)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)



def _long_context_backbone(split, seed, lens):
    rng = np.random.default_rng(seed)
    batch = synth.make_batch(rng, np.asarray(lens, np.int32), split)
    dims = synth.Dims(512, 8, 2, 64)
    x = rng.standard_normal((batch.total_rows, dims.d_model)).astype(np.float32)
    full = [synth.full_weights(rng, dims, 0.02, 0.02)]
    tgt = [synth.target_weights(rng, dims, split, 0.02, 0.02) for _ in range(2)]
    return synth.Workload(f"long_context_s{split}", batch, dims, "bf16", x, full=full, target=tgt, n_blocks=1,
                          k_target=2)


@pytest.mark.parametrize("split,lens", [
    (1, [[6000, 2000, 40], [3000, 500, 24]]),
    (4, [[6000, 2000, 10], [3000, 500, 6]]),
    # degenerate users beside a long one: no context at all, no R rows, one T row
    (1, [[6000, 2000, 30], [0, 0, 3], [5, 0, 2], [0, 12, 1], [700, 0, 9]]),
], ids=["s1", "s4", "degenerate_users"])
def test_backbone_with_key_split_target_attention(split, lens):
    """Few T rows against long contexts (two users, 64 candidates): the target attention splits
    each slice's key tiles over several workgroups and the gated LayerNorm adds their fp32
    partials.  The hoisted backbone (which splits) against the oracle, and against the
    layer-by-layer entry points (which keep one workgroup per slice) to rounding.

    Branch bar against the oracle: two half-ulps per layer.  Both sides round X' to bf16 at every
    layer boundary, so after a layer they can sit one ulp apart whichever path runs: on this
    workload the unsplit path's T rows, after three layers, reach exactly one half-ulp past a
    one-half-ulp-per-layer allowance, as the split path's do."""
    wl = _long_context_backbone(split, 96 + split + len(lens), lens)
    batch, dims = wl.batch, wl.dims
    ks = target_key_splits(batch, dims)
    say(f"key splits: {ks}")
    assert ks >= 8
    x0, got = _backbone_gpu(wl, hoist=True)
    _, lbl = _backbone_gpu(wl, hoist=False)
    xr, fw, tw = rounded_inputs(wl)
    np.testing.assert_array_equal(x0, xr)
    ref = om.backbone(batch, xr, fw, tw, dims, 1, 2, boundary=om.bf16_round)
    r = Report(TOL_BF16)
    r.close("X'", got, ref)
    r.branch("dX vs oracle (6 roundings allowed)", got, ref, xr, "bf16", roundings=6)
    r.branch("dX vs layer by layer (6 roundings allowed)", got, lbl, xr, "bf16", roundings=6)
    r.check()


def test_small_v2_backbone_against_oracle():
    """2 blocks x (1 full + 3 target), V2 sub-tokens, all users checked against the oracle."""
    wl = _small_backbone(4, 70)
    x0, got = _backbone_gpu(wl)
    xr, full, tgt = rounded_inputs(wl)
    np.testing.assert_array_equal(x0, xr)
    ref = om.backbone(wl.batch, xr, full, tgt, wl.dims, wl.n_blocks, wl.k_target, boundary=om.bf16_round)
    r = Report(TOL_BF16)
    r.close("X'", got, ref)
    r.branch("dX (8 roundings allowed)", got, ref, xr, "bf16", roundings=8)
    r.check()


@pytest.mark.parametrize("packed,kind", [(False, "small"), (True, "small"), (False, "key_split")])
def test_backbone_forward_replays_from_a_hip_graph(packed, kind):
    """The hoisted backbone forward captured into a HIP graph: every replay, with eager runs in
    between, equals the eager result bit for bit, with dense and with packed (2:4) weights (each
    block's context projections one grouped launch over per-layer weight matrices), and on long
    contexts with few T rows (the target attention's key splits and their summed partials)."""
    import torch
    from hybrid_masked_attention_amd import binding as B
    from hybrid_masked_attention_amd.tensors import DeviceWorkload
    if kind == "small":
        wl = _small_backbone(4, 80)
    else:
        wl = _long_context_backbone(1, 81, [[6000, 2000, 40], [0, 0, 3], [3000, 500, 24]])
        assert target_key_splits(wl.batch, wl.dims) >= 8
    dw = DeviceWorkload(wl)
    if packed:
        dw.pack_s24()
    meta = B.mask_build(dw.batch)
    ws = B.workspace(dw.batch, dw.dims, B.OP_BACKBONE, k_target=wl.k_target)

    def eager():
        x = dw.x.clone()
        B.backbone_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, x, ws)
        torch.cuda.synchronize()
        return x

    ref = eager()
    xg = dw.x.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.backbone_fwd(dw.batch, dw.dims, wl.n_blocks, wl.k_target, meta, dw.full, dw.target, xg, ws)
    for i in range(3):
        xg.copy_(dw.x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, ref), f"replay {i}"
        assert torch.equal(eager(), ref)
