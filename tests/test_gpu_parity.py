"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: grouping bit-exact; y within rel-L2 5e-3 and max-abs 3e-2 of the fp32
oracle on the same bf16-rounded inputs (fp32 layers: same bar); per-slot and
deduplicating results agree to fp32 summation order (rel-L2 <= 1e-4: the two
kernels may cut a gate/up tile's K range at different points), and every kernel
is deterministic (bitwise equal results on repeated passes).
"""
import itertools

import numpy as np
import pytest
import torch

import expert_ffn_amd as efa
import oracle
import synth
from synth import routing
from synth.device import to_torch

from .gpu_cases import LAYOUTS, SUMMATION_TOL, SYNC_BYTES, DeviceLayer, assert_close, errors, say, step_multiple

pytestmark = pytest.mark.gpu


def _ids_dev(ids):
    return torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()


def _check_group(ids, N):
    st, count, offset, sbe, distinct, U = oracle.route_group(ids, N)
    g = efa.route_group(_ids_dev(ids), N)
    torch.cuda.synchronize()
    assert np.array_equal(g.count.cpu().numpy(), count)
    assert np.array_equal(g.offset.cpu().numpy(), offset)
    assert np.array_equal(g.slot_by_expert.cpu().numpy(), sbe)
    assert np.array_equal(g.distinct.cpu().numpy(), distinct)
    ue = g.u_and_err.cpu().numpy()
    assert ue[0] == U and ue[1] == (0 if st == oracle.OR_OK else efa._abi.MOE_E_IDS)


def test_route_group_brute_force_small():
    say("route_group brute force N=4 m=2 n=3")
    pairs = list(itertools.permutations(range(4), 2))
    for rows in itertools.product(pairs, repeat=3):
        _check_group(np.array(rows, np.int32), 4)


def test_route_group_configs_and_invalid():
    rng = np.random.default_rng(0)
    for N, m, n in [(8, 2, 1), (64, 6, 8), (128, 8, 8), (128, 8, 32), (1024, 4, 64), (16, 16, 16), (8, 2, 64)]:
        say("route_group N=%d m=%d n=%d" % (N, m, n))
        for _ in range(10):
            ids = np.stack([rng.choice(N, m, replace=False) for _ in range(n)]).astype(np.int32)
            _check_group(ids, N)
    say("route_group invalid ids")
    _check_group(np.array([[0, 7], [3, -1], [2, 2], [9, 1]], np.int32), 5)
    _check_group(np.full((4, 2), 3, np.int32), 5)


def _agree(ys, yd, what):
    rel, _ = errors(ys, yd)
    assert rel <= SUMMATION_TOL, "%s: per-slot and dedup differ, rel_l2=%.3e" % (what, rel)


def _compare(dl, x, ids, w, what, shared=False, tokens=None):
    ys, yd, info = dl.run(x, ids, w, shared=shared)
    assert info[0] == oracle.union_count(ids, dl.spec.N) and info[1] == 0
    ref = dl.oracle_y(x, ids, w, shared=bool(shared), tokens=tokens)
    sel = slice(None) if tokens is None else tokens
    r1 = assert_close(ys[sel], ref, what + " perslot")
    r2 = assert_close(yd[sel], ref, what + " dedup")
    _agree(ys, yd, what)
    return r1, r2


@pytest.mark.parametrize("dtype,shape", [("bf16", (3, 64, 40)), ("bf16", (5, 2048, 1408)), ("f32", (4, 72, 136)),
                                          ("f32", (2, 32, 8))])
def test_pack_w_down_bit_exact(dtype, shape):
    """moe_pack_w_down against the layout definition: packed[e][c][i][k] = W[e][i][8c + k]."""
    say("pack", dtype, shape)
    N, d, d_ff = shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    wd = torch.randn(N, d, d_ff, generator=g, device="cuda").to(tdt)
    wg = torch.zeros(N, d_ff, d, dtype=tdt, device="cuda")
    layer = efa.Layer(wg, wg, wd, m=1)
    out = torch.full((N, d_ff // 8, d, 8), 7, dtype=tdt, device="cuda")
    efa.pack_w_down(layer, wd, out)
    torch.cuda.synchronize()
    ref = wd.cpu().reshape(N, d, d_ff // 8, 8).permute(0, 2, 1, 3).contiguous()
    assert torch.equal(out.cpu().view(torch.int16 if dtype == "bf16" else torch.int32),
                       ref.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("dtype,E,R,K", [("bf16", 3, 64, 96), ("bf16", 2, 1408, 2048), ("bf16", 2, 2048, 1408),
                                         ("f32", 4, 48, 80), ("f32", 1, 16, 16)])
@pytest.mark.parametrize("mat", [efa.MOE_MAT_GATE_UP, efa.MOE_MAT_DOWN])
def test_pack_tiled_bit_exact(dtype, E, R, K, mat):
    """moe_pack_tiled against the layout definition: block (e, r, s) of 16 rows x one
    64-byte step, lane l = 16 q + i holding row 16 r + i, elements s*step + q*per on,
    i.e. tiled[e][r][s][q][i][:] = W[e][16 r + i][s*step + q*per : +per]."""
    say("pack tiled", dtype, E, R, K, mat)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    per = 8 if dtype == "bf16" else 4
    step = 4 * per
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    w = torch.randn(E, R, K, generator=g, device="cuda").to(tdt)
    # a layer whose (d_ff, d) make the matrix [R][K]: gate/up rows d_ff, down rows d
    d_ff, d = (R, K) if mat == efa.MOE_MAT_GATE_UP else (K, R)
    z = torch.zeros(1, d_ff, d, dtype=tdt, device="cuda")
    layer = efa.Layer(z, z, torch.zeros(1, d, d_ff, dtype=tdt, device="cuda"), m=1)
    out = torch.full_like(w, 7)
    efa.pack_tiled(layer, w, out, mat)
    torch.cuda.synchronize()
    ref = w.cpu().reshape(E, R // 16, 16, K // step, 4, per).permute(0, 1, 3, 4, 2, 5).contiguous()
    iv = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(out.cpu().view(iv).reshape(-1), ref.view(iv).reshape(-1))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_tiny_fp32_many_seeds(layout):
    spec = synth.CONFIGS["tiny"]
    for seed in range(1000):
        if seed % 100 == 0:
            say("tiny seeds", seed, "..", seed + 99, "layout", layout)
        dl = DeviceLayer(spec, seed, layout=layout)
        tr = routing.uniform_trace(spec.N, spec.m, 4, routing.rng_for(seed, 0, "uniform"))
        x = synth.pass_x(spec, seed, 0, 0, 4)
        (rel, mx), _ = _compare(dl, x, tr.ids, tr.w, "tiny seed %d" % seed)
        assert rel < 1e-5  # fp32 weights, fp32 MFMA: far inside the bar


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,m,d,d_ff,n", [
    (5, 3, 72, 136, 1), (5, 3, 72, 136, 3), (5, 3, 72, 136, 17), (6, 2, 40, 24, 33),
    (4, 4, 8, 8, 64), (12, 4, 264, 200, 64), (9, 1, 1032, 40, 20),
    # d_ff too long for the down weights to sit in registers: the streaming down path,
    # with few down items each (unit, row tile) cut into 4 parts of the d_ff contraction
    (7, 2, 136, 1560, 5), (7, 2, 136, 1560, 40), (3, 2, 64, 2048, 2), (3, 1, 1024, 1040, 1),
    # 128..1024 gate/up tiles: K ranges shared between work groups (split tiles)
    (40, 4, 72, 1000, 3), (40, 4, 200, 520, 5),
    # multiples of 32, fewer tiles than half the compute units (each tile cut in two)
    (6, 3, 96, 160, 1), (6, 3, 96, 160, 8), (33, 8, 256, 64, 7), (4, 4, 64, 96, 8), (12, 6, 512, 352, 5)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_ragged_shapes(dtype, N, m, d, d_ff, n, layout):
    if layout == "tiled":  # the same case with d and d_ff in whole steps (tiles, tails and parts stay ragged)
        d, d_ff = step_multiple(d, dtype), step_multiple(d_ff, dtype)
    say("ragged", dtype, N, m, d, d_ff, n, "layout", layout)
    spec = synth.layer_spec("tiny", N=N, m=m, d=d, d_ff=d_ff, dtype=dtype, sigma=0.05)
    dl = DeviceLayer(spec, 17, layout=layout)
    tr = routing.correlated_trace(N, m, n, 0.7, routing.rng_for(17, 0, "correlated"))
    x = synth.pass_x(spec, 17, 0, 1, n)
    _compare(dl, x, tr.ids, tr.w, "ragged")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_max_reuse_and_no_reuse(layout):
    spec = synth.layer_spec("tiny", N=70, m=4, d=128, d_ff=96, dtype="bf16")
    dl = DeviceLayer(spec, 3, layout=layout)
    rng = np.random.default_rng(3)
    for n in (1, 8, 16, 17, 32, 33, 64):
        say("max reuse n", n)
        row = rng.choice(spec.N, spec.m, replace=False)
        ids = np.tile(row, (n, 1)).astype(np.int32)  # every token the same experts: groups of n
        w = rng.random((n, spec.m)).astype(np.float32)
        x = synth.pass_x(spec, 3, 0, n, n)
        _compare(dl, x, ids, w, "max reuse n=%d" % n)
    say("no reuse n=17")
    ids = np.arange(68, dtype=np.int32).reshape(17, 4)
    w = rng.random((17, 4)).astype(np.float32)
    _compare(dl, synth.pass_x(spec, 3, 0, 99, 17), ids, w, "no reuse")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_invalid_ids_skip_slot_and_flag(layout):
    spec = synth.layer_spec("tiny", N=8, m=2, d=64, d_ff=64, dtype="bf16")
    dl = DeviceLayer(spec, 5, layout=layout)
    ids = np.array([[0, 3], [5, 9], [2, 1]], np.int32)   # slot (1,1) out of range
    w = np.array([[0.5, 0.5], [0.7, 0.3], [0.6, 0.4]], np.float32)
    x = synth.pass_x(spec, 5, 0, 0, 3)
    say("invalid ids")
    ys, yd, info = dl.run(x, ids, w)
    assert info[1] == efa._abi.MOE_E_IDS and info[0] == 5
    ids_ok = ids.copy()
    ids_ok[1, 1] = 7
    w_ok = w.copy()
    w_ok[1, 1] = 0.0  # the skipped slot adds nothing
    ref = dl.oracle_y(x, ids_ok, w_ok)
    assert_close(ys, ref, "invalid perslot")
    assert_close(yd, ref, "invalid dedup")
    _agree(ys, yd, "invalid")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_accumulate_and_determinism(layout):
    spec = synth.layer_spec("tiny", N=16, m=4, d=256, d_ff=128, dtype="bf16")
    dl = DeviceLayer(spec, 8, layout=layout)
    tr = routing.uniform_trace(16, 4, 6, routing.rng_for(8, 0, "uniform"))
    x = synth.pass_x(spec, 8, 0, 0, 6)
    say("determinism")
    a = dl.run(x, tr.ids, tr.w)
    for _ in range(3):
        b = dl.run(x, tr.ids, tr.w)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    say("accumulate")
    xd = to_torch(x)
    ids = _ids_dev(tr.ids)
    w = torch.from_numpy(tr.w).cuda()
    y0 = torch.randn(6, 256, device="cuda")
    y = y0.clone()
    efa.expert_perslot(dl.dev, xd, ids, w, y=y, ws=dl.dev.workspace(6), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), (y0 + torch.from_numpy(a[0]).cuda()).cpu())
    say("workspace type")  # sizes are counted in bytes: a workspace is uint8 (nothing launches)
    wsf = torch.zeros(dl.dev.workspace(6).numel() // 4 + 1, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        efa.expert_dedup(dl.dev, xd, ids, w, ws=wsf)


# ------------------------------ full-size layers ------------------------------

@pytest.fixture(scope="module")
def dsv2():
    say("upload dsv2lite layer")
    return DeviceLayer(synth.CONFIGS["dsv2lite"], 2026, with_shared=True)


@pytest.fixture(scope="module")
def dsv2p(dsv2):
    """The same layer with W_down packed."""
    say("pack dsv2lite layer")
    dl = DeviceLayer(dsv2.spec, 2026, with_shared=True, host=dsv2.host, packed=True)
    return dl


@pytest.fixture(scope="module")
def dsv2t(dsv2):
    """The same layer with all three matrices tiled."""
    say("tile dsv2lite layer")
    return DeviceLayer(dsv2.spec, 2026, with_shared=True, host=dsv2.host, layout="tiled")


@pytest.fixture(scope="module")
def dsv2_by_layout(dsv2, dsv2p, dsv2t):
    return {"plain": dsv2, "packed": dsv2p, "tiled": dsv2t}


@pytest.mark.parametrize("kind", ["uniform", "correlated"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_dsv2lite_windows(dsv2_by_layout, kind, layout):
    dsv2 = dsv2_by_layout[layout]
    spec = dsv2.spec
    tr = routing.make_trace(spec, kind, 512, seed=2026, p=0.5)
    starts = routing.window_starts(512, 8, 8, seed=2026)
    for n in range(1, 9):
        st = int(starts[n - 1])
        ids, w = routing.window(tr, st, n)
        x = synth.pass_x(spec, 2026, 0, 1000 + n, n)
        sh = "separate" if n in (1, 5) else ("fused" if n in (2, 3, 8) else False)
        say("dsv2lite", kind, "n", n, "start", st, "shared", sh)
        _compare(dsv2, x, ids, w, "dsv2lite %s n=%d" % (kind, n), shared=sh)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_dedup_down_form_follows_distinct_experts(dsv2_by_layout, layout):
    """The deduplicating kernel picks register-mode or streaming down items on the
    device, from the U distinct experts it finds.  DeepSeek-V2-Lite shape, both shared
    experts in the call, n = 2, passes naming exactly U = 6 .. 12 experts: with
    U + 2 units of 44 gate/up tiles and 128 register-mode items each, the pass fits
    the 2112 work groups of register mode up to U = 10 (528 + 1536) and streams from
    U = 11 (572 + 1664); every pass matches the oracle and the per-slot kernel."""
    dsv2 = dsv2_by_layout[layout]
    spec = dsv2.spec
    rng = np.random.default_rng(77)
    x = synth.pass_x(spec, 2026, 0, 2000, 2)
    for U in range(6, 13):
        ids, w = routing.chosen_pass(spec.N, spec.m, 2, U, rng)
        say("dsv2lite chosen U", U, layout)
        _compare(dsv2, x, ids, w, "dsv2lite n=2 U=%d" % U, shared="fused")


@pytest.mark.parametrize("base,n_shared,d,d_ff", [("tiny", 1, 64, 128), ("tiny", 3, 72, 40),
                                                   ("dsv2lite", 2, 96, 160), ("dsv2lite", 1, 256, 352)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_shared_experts_in_the_same_call(base, n_shared, d, d_ff, layout):
    """Always-on experts computed in the same launch as the routed ones (each read once
    per pass against all n tokens, weight 1), for both kernels, against the oracle's
    shared-expert sum; n = 17 and 20 take two token columns per MFMA pass."""
    if layout == "tiled":
        d, d_ff = step_multiple(d, "bf16"), step_multiple(d_ff, "bf16")
    spec = synth.layer_spec(base, N=12, m=3, d=d, d_ff=d_ff, n_shared=n_shared)
    dl = DeviceLayer(spec, 31, with_shared=True, layout=layout)
    tr = routing.make_trace(spec, "correlated", 64, seed=31, p=0.5)
    for n in (1, 2, 5, 8, 17, 20):
        ids, w = routing.window(tr, 3, n)
        x = synth.pass_x(spec, 31, 0, n, n)
        say("shared", base, n_shared, d, d_ff, "layout", layout, "n", n)
        _compare(dl, x, ids, w, "shared %s S=%d n=%d" % (base, n_shared, n), shared="fused")


@pytest.mark.parametrize("layout", ["packed", "tiled"])
def test_shared_experts_accumulate_and_most_units(layout):
    """With MOE_FLAG_ACCUMULATE the fused call adds to y; a pass at the unit limit
    (n*m + n_shared = 256) still matches the oracle."""
    spec = synth.layer_spec("dsv2lite", N=64, m=4, d=128, d_ff=96, n_shared=4)
    dl = DeviceLayer(spec, 5, with_shared=True, layout=layout)
    tr = routing.make_trace(spec, "uniform", 128, seed=5)
    n = 63  # 63*4 + 4 = 256 units
    ids, w = routing.window(tr, 0, n)
    x_h = synth.pass_x(spec, 5, 0, 0, n)
    say("shared at the unit limit, n", n)
    _compare(dl, x_h, ids, w, "shared unit limit", shared="fused")
    x = to_torch(x_h)
    idd = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    wd = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    y0 = torch.randn(n, spec.d, dtype=torch.float32, device="cuda")
    ws = dl.fused.workspace(n)
    for fn in (efa.expert_perslot, efa.expert_dedup):
        y = y0.clone()
        fn(dl.fused, x, idd, wd, y=y, ws=ws, accumulate=True)
        ref = dl.oracle_y(x_h, ids, w, shared=True)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy() - y0.cpu().numpy(), ref, "accumulate " + fn.__name__)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_qwen3_layer_zipf_and_tree(layout):
    spec = synth.CONFIGS["qwen3"]
    say("upload qwen3 layer", "layout", layout)
    dl = DeviceLayer(spec, 77, layer=3, layout=layout)
    tr = routing.make_trace(spec, "zipf", 256, seed=77, layer=3, s=1.1)
    for n in (1, 2, 4, 8):
        ids, w = routing.window(tr, 5 * n, n)
        x = synth.pass_x(spec, 77, 3, n, n)
        say("qwen3 zipf n", n)
        _compare(dl, x, ids, w, "qwen3 n=%d" % n)
    parents, ttr = routing.tree_routing(spec.N, spec.m, 0.5, routing.rng_for(77, 3, "tree"))
    x = synth.pass_x(spec, 77, 3, 500, 32)
    say("tree pass n=32, every token")
    _compare(dl, x, ttr.ids, ttr.w, "tree")
    # 32 tokens sharing one expert (a group of 32: the deduplicating kernel stages its
    # h in several chunks) and every other token a second one (a group of 16)
    rng = np.random.default_rng(78)
    ids = np.empty((32, spec.m), np.int32)
    for t in range(32):
        rest = rng.choice(np.arange(2, spec.N), spec.m - 2, replace=False)
        ids[t] = np.concatenate(([0, 1 if t % 2 == 0 else int(rng.integers(2, spec.N))], rest))
        while len(set(ids[t].tolist())) < spec.m:
            ids[t, 1] = int(rng.integers(2, spec.N))
    w = rng.random((32, spec.m)).astype(np.float32)
    say("n=32 pass with groups of 32 and 16 tokens")
    _compare(dl, synth.pass_x(spec, 77, 3, 501, 32), ids, w, "large groups")


@pytest.mark.parametrize("kind", ["uniform", "correlated"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_repeated_passes_bitwise_stable(dsv2_by_layout, kind, layout):
    """Many back-to-back passes on one workspace, per-slot and dedup alternating:
    every result bitwise equal to the first of its kind, the two kinds equal to
    summation order.  Data handed between workgroups (h, O, partial sums) that
    were not yet visible, or counters not reset between calls, would break it."""
    dsv2 = dsv2_by_layout[layout]
    spec = dsv2.spec
    tr = routing.make_trace(spec, kind, 256, seed=31, p=0.5)
    ws = dsv2.dev.workspace(8)
    info = torch.zeros(3, dtype=torch.int32, device="cuda")
    for n in (1, 3, 8):
        ids_h, w_h = routing.window(tr, 7 * n, n)
        x = to_torch(synth.pass_x(spec, 31, 0, n, n))
        ids, w = _ids_dev(ids_h), torch.from_numpy(w_h).cuda()
        say("repeat", kind, "n", n)
        refs = [efa.expert_perslot(dsv2.dev, x, ids, w, ws=ws).clone(),
                efa.expert_dedup(dsv2.dev, x, ids, w, ws=ws).clone()]
        outs = []
        for it in range(40):
            fn = efa.expert_perslot if it % 2 == 0 else efa.expert_dedup
            outs.append(fn(dsv2.dev, x, ids, w, ws=ws, info=info).clone())
        torch.cuda.synchronize()
        for it, o in enumerate(outs):
            assert torch.equal(o, refs[it % 2]), (n, it)
        _agree(refs[0].cpu().numpy(), refs[1].cpu().numpy(), "repeat n=%d" % n)
        assert int(info[2].item()) == 0


@pytest.mark.parametrize("other", ["packed", "tiled"])
def test_layouts_agree_with_plain(dsv2_by_layout, other):
    """The same passes with plain weights and with W_down packed or all three tiled
    agree to fp32 summation order, routed experts alone and with the shared experts
    in the call."""
    dsv2 = dsv2_by_layout["plain"]
    spec = dsv2.spec
    tr = routing.make_trace(spec, "correlated", 256, seed=5, p=0.5)
    for n in (1, 2, 5, 8, 9):
        ids_h, w_h = routing.window(tr, 3 * n, n)
        x = synth.pass_x(spec, 5, 0, n, n)
        sh = "fused" if n in (2, 9) else False
        say("plain vs", other, "n", n, "shared", sh)
        a = dsv2.run(x, ids_h, w_h, shared=sh)
        b = dsv2_by_layout[other].run(x, ids_h, w_h, shared=sh)
        _agree(a[0], b[0], "perslot plain/%s n=%d" % (other, n))
        _agree(a[1], b[1], "dedup plain/%s n=%d" % (other, n))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_repeated_ids_count_as_often_as_they_appear(layout):
    """An id repeated within a token (flagged MOE_E_IDS) counts as often as it appears in
    both kernels; with 8 tokens listing one expert 4 times its group has 32 slots, more
    than one 16-column tile."""
    spec = synth.layer_spec("tiny", N=20, m=4, d=128, d_ff=96, dtype="bf16")
    dl = DeviceLayer(spec, 4, layout=layout)
    rng = np.random.default_rng(4)
    ids = np.stack([rng.choice(spec.N, spec.m, replace=False) for _ in range(8)]).astype(np.int32)
    ids[:, :] = 3
    ids[2, 1] = 7
    w = rng.random((8, spec.m)).astype(np.float32)
    x = synth.pass_x(spec, 4, 0, 0, 8)
    say("repeated ids layout", layout)
    ys, yd, info = dl.run(x, ids, w)
    assert info[1] == efa._abi.MOE_E_IDS and info[0] == 2
    _agree(ys, yd, "repeated ids")
    # the same sums with each repeat folded into one slot of summed weight
    ids1 = np.array([[3, 7] if t == 2 else [3, 5] for t in range(8)], np.int32)
    w1 = np.array([[w[t, 0] + w[t, 2] + w[t, 3], w[t, 1]] if t == 2 else [w[t].sum(), 0.0] for t in range(8)],
                  np.float32)
    ref = oracle.moe_ffn(*dl.host, x, ids1, w1, "bf16")
    assert_close(ys, ref, "repeated ids perslot")
    assert_close(yd, ref, "repeated ids dedup")


def test_expert_auto_runs_the_kernel_the_crossover_names():
    """moe_expert_auto: the deduplicating kernel from n >= crossover, the per-slot
    kernel below, crossover 0 always per-slot; same bits as the kernel called directly."""
    spec = synth.layer_spec("dsv2lite", N=16, m=4, d=256, d_ff=176, n_shared=0)
    dl = DeviceLayer(spec, 21, packed=True)
    tr = routing.make_trace(spec, "correlated", 32, seed=21, p=0.5)
    ws = dl.dev.workspace(8)
    for n in (1, 2, 5):
        ids_h, w_h = routing.window(tr, 4, n)
        x = to_torch(synth.pass_x(spec, 21, 0, n, n))
        ids, w = torch.from_numpy(ids_h).cuda(), torch.from_numpy(w_h).cuda()
        ys = efa.expert_perslot(dl.dev, x, ids, w, ws=ws)
        yd = efa.expert_dedup(dl.dev, x, ids, w, ws=ws)
        for c in (0, 1, 3):
            say("auto n", n, "crossover", c)
            y, kind = efa.expert_auto(dl.dev, x, ids, w, c, ws=ws)
            want = efa.MOE_KIND_DEDUP if (c > 0 and n >= c) else efa.MOE_KIND_SLOT
            assert kind == want
            assert torch.equal(y, yd if want == efa.MOE_KIND_DEDUP else ys)


def test_hip_graph_replays_equal_eager_calls():
    """Both kernels captured in a HIP graph over static id / weight buffers, replayed
    three times with eager kernel calls, torch work and new windows copied in between:
    every replay bitwise equal to the eager call on the same window (the kernels issue
    no memset; the workspace counters are reset by the kernels themselves)."""
    spec = synth.layer_spec("dsv2lite", N=16, m=4, d=256, d_ff=192, n_shared=2)
    dl = DeviceLayer(spec, 41, with_shared=True, layout="tiled")
    layer = dl.fused
    n = 6
    tr = routing.make_trace(spec, "correlated", 64, seed=41, p=0.5)
    x = to_torch(synth.pass_x(spec, 41, 0, 0, n))
    ids = torch.zeros(n, spec.m, dtype=torch.int32, device="cuda")
    w = torch.zeros(n, spec.m, dtype=torch.float32, device="cuda")
    ws_g, ws_e = layer.workspace(n), layer.workspace(n)
    yg = {k: torch.zeros(n, spec.d, dtype=torch.float32, device="cuda") for k in ("slot", "dedup")}
    fns = {"slot": efa.expert_perslot, "dedup": efa.expert_dedup}
    i0, w0 = routing.window(tr, 0, n)
    ids.copy_(torch.from_numpy(i0))
    w.copy_(torch.from_numpy(w0))
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()  # default priority
    graphs = {}
    for k, fn in fns.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            fn(layer, x, ids, w, y=yg[k], ws=ws_g, stream=cap)
        graphs[k] = g
    torch.cuda.synchronize()
    for rep in range(3):
        ih, wh = routing.window(tr, 5 + 7 * rep, n)
        ids.copy_(torch.from_numpy(ih))
        w.copy_(torch.from_numpy(wh))
        for k, fn in fns.items():
            say("graph replay", rep, k)
            graphs[k].replay()
            torch.cuda.synchronize()
            ye = fn(layer, x, ids, w, ws=ws_e)  # eager, own workspace
            _ = (ye * 2.0).sum()                # unrelated torch work between replays
            torch.cuda.synchronize()
            assert torch.equal(yg[k], ye), (rep, k)
        ref = dl.oracle_y(synth.pass_x(spec, 41, 0, 0, n), ih, wh, shared=True)
        assert_close(yg["slot"].cpu().numpy(), ref, "graph slot rep %d" % rep)
        assert_close(yg["dedup"].cpu().numpy(), ref, "graph dedup rep %d" % rep)
    assert np.all(ws_g[:SYNC_BYTES].cpu().numpy() == 0)


@pytest.mark.parametrize("layout", ["plain", "tiled"])
def test_limits_experts_slots_width(layout):
    """At the limits of the boundary: N = 1024 experts with ids up to 1023 and
    n*m = 256 slots (n = 64); d_model = 16384, the widest layer (1024 down row tiles,
    every arrival counter line in use); m = N (every token selects every expert)."""
    rng = np.random.default_rng(9)
    # N = 1024, n = 64, m = 4: slots at the unit limit, ids drawn from the top of the range
    spec = synth.layer_spec("tiny", N=1024, m=4, d=64, d_ff=64, dtype="bf16", sigma=0.05)
    dl = DeviceLayer(spec, 9, layout=layout)
    ids = np.stack([rng.choice(np.arange(960, 1024), 4, replace=False) for _ in range(64)]).astype(np.int32)
    ids[0] = [1023, 0, 512, 1022]
    w = rng.random((64, 4)).astype(np.float32)
    say("limits N=1024 n=64", layout)
    _compare(dl, synth.pass_x(spec, 9, 0, 0, 64), ids, w, "N=1024 n=64")
    # d_model = 16384
    spec = synth.layer_spec("tiny", N=3, m=2, d=16384, d_ff=64, dtype="bf16", sigma=0.02)
    dl = DeviceLayer(spec, 10, layout=layout)
    for n in (1, 3):
        ids = np.stack([rng.choice(3, 2, replace=False) for _ in range(n)]).astype(np.int32)
        w = rng.random((n, 2)).astype(np.float32)
        say("limits d=16384 n", n, layout)
        _compare(dl, synth.pass_x(spec, 10, 0, n, n), ids, w, "d=16384 n=%d" % n)
    # m = N
    spec = synth.layer_spec("tiny", N=4, m=4, d=96, d_ff=128, dtype="bf16", sigma=0.05)
    dl = DeviceLayer(spec, 11, layout=layout)
    ids = np.stack([rng.permutation(4) for _ in range(8)]).astype(np.int32)
    w = rng.random((8, 4)).astype(np.float32)
    say("limits m=N", layout)
    _compare(dl, synth.pass_x(spec, 11, 0, 0, 8), ids, w, "m=N")
