"""The C-ABI library on the host (no GPU needed): it loads, exports every symbol
the header declares, rejects bad arguments before any launch, and its host-only
functions (bytes_requested, step_time_model) agree with the oracle."""
import ctypes
import os
import random
import re
from fractions import Fraction as F

import numpy as np
import pytest

import oracle
from oracle import step_exact as se
import expert_ffn_amd as efa
from expert_ffn_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_expert.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t|size_t)\s+(\w+)\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    names = _declared()
    assert set(names) == set(_abi.EXPORTS)
    for nm in names:
        assert hasattr(L, nm), nm
    out = os.popen("nm -D --defined-only %s" % _abi.SO_PATH).read()
    for nm in names:
        assert re.search(r"\bT %s\b" % nm, out), nm


def _desc(**kw):
    d = dict(N=8, m=2, d_model=64, d_ff=128, dtype=_abi.MOE_F32, flags=0, n_shared=0)
    d.update(kw)
    return _abi.LayerDesc(d["N"], d["m"], d["d_model"], d["d_ff"], d["dtype"], d["flags"], d["n_shared"])


def test_host_validation_rejects_before_launch():
    L = _abi.lib()
    vp = ctypes.c_void_p
    fake = vp(0x1000)  # never dereferenced: validation fails first
    W = _abi.LayerWeights(0x1000, 0x1000, 0x1000)
    cases = [
        (_desc(m=0), _abi.MOE_E_INVAL),
        (_desc(m=9), _abi.MOE_E_INVAL),
        (_desc(d_model=60), _abi.MOE_E_DTYPE),
        (_desc(d_ff=100), _abi.MOE_E_DTYPE),
        (_desc(dtype=7), _abi.MOE_E_DTYPE),
        (_desc(flags=8), _abi.MOE_E_INVAL),  # unknown flag bit
        # tiled weights: not together with packed W_down, and only for whole 64-byte steps
        (_desc(flags=_abi.MOE_FLAG_TILED | _abi.MOE_FLAG_WDOWN_PACKED), _abi.MOE_E_INVAL),
        (_desc(flags=_abi.MOE_FLAG_TILED, d_model=40), _abi.MOE_E_INVAL),
        (_desc(flags=_abi.MOE_FLAG_TILED, d_ff=136), _abi.MOE_E_INVAL),
        (_desc(flags=_abi.MOE_FLAG_TILED, dtype=_abi.MOE_BF16, d_model=48), _abi.MOE_E_INVAL),
        (_desc(N=2000, m=2), _abi.MOE_E_INVAL),
    ]
    for desc, want in cases:
        st = L.moe_expert_perslot(ctypes.byref(desc), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake, 1 << 30,
                                  None)
        assert st == want
    d = _desc()
    # n out of range, n*m above the slot limit
    assert L.moe_expert_perslot(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 0, fake, None, fake, 1 << 30,
                                None) == _abi.MOE_E_INVAL
    assert L.moe_expert_perslot(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 65, fake, None, fake, 1 << 30,
                                None) == _abi.MOE_E_INVAL
    # null pointer, misaligned pointer, small workspace, misaligned workspace
    assert L.moe_expert_perslot(ctypes.byref(d), ctypes.byref(W), None, fake, fake, 4, fake, None, fake, 1 << 30,
                                None) == _abi.MOE_E_INVAL
    Wm = _abi.LayerWeights(0x1004, 0x1000, 0x1000)
    assert L.moe_expert_perslot(ctypes.byref(d), ctypes.byref(Wm), fake, fake, fake, 4, fake, None, fake, 1 << 30,
                                None) == _abi.MOE_E_INVAL
    need = L.moe_workspace_bytes(ctypes.byref(d), 4, 0)
    # sync area + h + O + partial sums of split tiles (256-aligned pieces): fewer gate/up
    # tiles than half the compute units are each cut in two, so the workspace holds
    # 3 contributors x n*m x d_ff x (gate, up) fp32
    assert need == 229376 + 4 * 2 * 128 * 4 + 4 * 2 * 64 * 4 + 3 * 4 * 2 * 128 * 8
    assert L.moe_workspace_bytes(ctypes.byref(d), 4, 1) == need
    # 128 .. 511 gate/up tiles: the workspace also holds partial sums of split
    # tiles, 3 contributors x n*m x d_ff x (gate, up) fp32 (per-slot: 44 tiles per
    # slot, split for one token); the size is the largest over 1..n tokens
    big = _desc(N=64, m=6, d_model=2048, d_ff=1408, dtype=_abi.MOE_BF16)

    def one(n, split):
        nm = n * 6
        return 229376 + nm * 1408 * 4 + nm * 2048 * 4 + (3 * nm * 1408 * 8 if split else 0)

    assert L.moe_workspace_bytes(ctypes.byref(big), 1, 0) == one(1, True)
    assert L.moe_workspace_bytes(ctypes.byref(big), 1, 1) == one(1, True)
    assert L.moe_workspace_bytes(ctypes.byref(big), 3, 0) == max(one(1, True), one(3, False))
    assert L.moe_workspace_bytes(ctypes.byref(big), 8, 0) == one(8, False)
    for k in (0, 1):  # n*m <= 256: n <= 42
        sizes = [L.moe_workspace_bytes(ctypes.byref(big), n, k) for n in range(1, 43)]
        assert all(sizes) and all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert L.moe_workspace_bytes(ctypes.byref(big), 43, 0) == 0
    assert L.moe_expert_perslot(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake, need - 1,
                                None) == _abi.MOE_E_WORKSPACE
    assert L.moe_expert_dedup(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 4, fake, None, vp(0x1010), need,
                              None) == _abi.MOE_E_INVAL
    assert L.moe_expert_dedup(ctypes.byref(d), ctypes.byref(W), fake, None, fake, 4, fake, None, fake, need,
                              None) == _abi.MOE_E_INVAL
    # events: wrong count, null events
    ev = (vp * 3)(0x1, 0x2, 0x3)
    assert L.moe_expert_perslot_ev(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake, need,
                                   None, ev, 3) == _abi.MOE_E_INVAL
    assert L.moe_expert_dedup_ev(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake, need,
                                 None, None, 2) == _abi.MOE_E_INVAL
    # shared experts: count limit, units limit (n*m + n_shared <= 256), null or
    # misaligned shared pointers; the workspace grows by n_shared*n slots
    Ws = _abi.LayerWeights(0x1000, 0x1000, 0x1000, 0x2000, 0x2000, 0x2000)
    for desc, Wx, n in ((_desc(n_shared=17), Ws, 4), (_desc(n_shared=-1), Ws, 4),
                        (_desc(N=64, m=4, n_shared=5), Ws, 63), (_desc(n_shared=2), W, 4),
                        (_desc(n_shared=2), _abi.LayerWeights(0x1000, 0x1000, 0x1000, 0x2000, 0x2008, 0x2000), 4)):
        for fn in (L.moe_expert_perslot, L.moe_expert_dedup):
            assert fn(ctypes.byref(desc), ctypes.byref(Wx), fake, fake, fake, n, fake, None, fake, 1 << 30,
                      None) == _abi.MOE_E_INVAL
    assert L.moe_workspace_bytes(ctypes.byref(_desc(N=64, m=4, n_shared=4)), 63, 0) > 0
    assert L.moe_workspace_bytes(ctypes.byref(_desc(N=64, m=4, n_shared=5)), 63, 0) == 0
    ds = _desc(n_shared=2)
    S = 4 * 2 + 2 * 4
    assert L.moe_workspace_bytes(ctypes.byref(ds), 4, 0) == 229376 + S * 128 * 4 + S * 64 * 4 + 3 * S * 128 * 8
    assert L.moe_kernels_per_call(0) == 1 and L.moe_kernels_per_call(1) == 1
    assert L.moe_kernels_per_call(5) == _abi.MOE_E_INVAL
    # grouping limits
    assert L.moe_route_group(fake, 129, 2, 8, fake, fake, fake, fake, fake, None) == _abi.MOE_E_INVAL
    assert L.moe_route_group(fake, 4, 9, 8, fake, fake, fake, fake, fake, None) == _abi.MOE_E_INVAL
    assert L.moe_route_group(None, 4, 2, 8, fake, fake, fake, fake, fake, None) == _abi.MOE_E_INVAL


def test_pack_tiled_host_validation():
    """moe_pack_tiled rejects a bad matrix code, sizes that are not whole steps, null,
    misaligned or overlapping pointers, before any launch; the tiled flag is accepted
    (a workspace size) exactly where the layout is defined."""
    L = _abi.lib()
    vp = ctypes.c_void_p
    a, b = vp(0x100000), vp(0x900000)
    d = _desc()  # fp32, d_model 64, d_ff 128, 8 experts: 256 KiB a tensor
    for mat in (-1, 2):
        assert L.moe_pack_tiled(ctypes.byref(d), a, b, mat, None) == _abi.MOE_E_INVAL
    for mat in (_abi.MOE_MAT_GATE_UP, _abi.MOE_MAT_DOWN):
        assert L.moe_pack_tiled(ctypes.byref(_desc(d_model=40)), a, b, mat, None) == _abi.MOE_E_INVAL
        assert L.moe_pack_tiled(ctypes.byref(_desc(dtype=_abi.MOE_BF16, d_ff=144)), a, b, mat, None) == _abi.MOE_E_INVAL
        assert L.moe_pack_tiled(ctypes.byref(_desc(dtype=9)), a, b, mat, None) == _abi.MOE_E_DTYPE
        assert L.moe_pack_tiled(ctypes.byref(d), None, b, mat, None) == _abi.MOE_E_INVAL
        assert L.moe_pack_tiled(ctypes.byref(d), a, None, mat, None) == _abi.MOE_E_INVAL
        assert L.moe_pack_tiled(ctypes.byref(d), vp(0x100008), b, mat, None) == _abi.MOE_E_INVAL
        assert L.moe_pack_tiled(ctypes.byref(d), a, vp(0x100000 + 4096), mat, None) == _abi.MOE_E_INVAL  # overlap
    assert L.moe_pack_tiled(None, a, b, 0, None) == _abi.MOE_E_INVAL
    T = _abi.MOE_FLAG_TILED
    assert L.moe_workspace_bytes(ctypes.byref(_desc(flags=T)), 4, 0) == L.moe_workspace_bytes(ctypes.byref(_desc()), 4, 0)
    assert L.moe_workspace_bytes(ctypes.byref(_desc(flags=T, dtype=_abi.MOE_BF16, d_model=2048, d_ff=1408)), 4, 0) > 0
    assert L.moe_workspace_bytes(ctypes.byref(_desc(flags=T, dtype=_abi.MOE_BF16, d_ff=144)), 4, 0) == 0


@pytest.mark.parametrize("cfg", ["tiny", "dsv2lite", "qwen3", "mixtral"])
def test_bytes_requested_matches_oracle(cfg):
    import synth
    from synth import routing
    spec = synth.CONFIGS[cfg]
    tr = routing.make_trace(spec, "correlated", 64, seed=4, p=0.5)
    for n in range(1, 9):
        for start in (0, 17, 40):
            ids = tr.ids[start:start + n]
            for kind in (0, 1):
                got = efa.bytes_requested(kind, spec.N, spec.m, spec.d, spec.d_ff, spec.dtype, ids)
                want = oracle.bytes_requested(kind, spec.N, spec.m, spec.d, spec.d_ff, spec.elem_bytes, ids)
                assert got == want
    bad = tr.ids[:2].copy()
    bad[0, 0] = spec.N
    with pytest.raises(efa.MoeError):
        efa.bytes_requested(0, spec.N, spec.m, spec.d, spec.d_ff, spec.dtype, bad)
    if spec.m > 1:
        dup = tr.ids[:2].copy()
        dup[1, 1] = dup[1, 0]
        with pytest.raises(efa.MoeError):
            efa.bytes_requested(1, spec.N, spec.m, spec.d, spec.d_ff, spec.dtype, dup)


def _rand_model(rng, n_max):
    E_slot = [rng.uniform(1, 2) * n for n in range(1, n_max + 1)]
    U = [1.0]
    for n in range(2, n_max + 1):
        U.append(U[-1] + rng.uniform(0.3, 1.0))
    E_dedup = [u for u in U]
    b_slot = [rng.uniform(0.8, 1.2) for _ in range(n_max)]
    b_dedup = [b_slot[0]] + [rng.uniform(0.4, 1.1) for _ in range(n_max - 1)]
    kv = [rng.uniform(0, 0.05) * k for k in range(n_max)]
    h = [rng.uniform(0, 0.1) for _ in range(n_max)]
    phi = [[rng.uniform(0, 0.05) for _ in range(n_max)] for _ in range(2)]
    return dict(E=[E_slot, E_dedup], beta=[b_slot, b_dedup], kv=kv, h=h, phi=phi,
                t0=rng.uniform(0, 0.2), D=rng.uniform(0, 1), beta_D=rng.uniform(0.5, 2), m_W=E_slot[0])


def test_step_time_model_matches_exact_oracle():
    rng = random.Random(11)
    a = [i / 21 for i in range(22)]
    for trial in range(25):
        n_max = rng.choice([3, 5, 8, 9])
        M = _rand_model(rng, n_max)
        out = efa.step_time_model(n_max, a, **M)
        Fx = lambda v: F(v)  # noqa: E731  exact value of each double input
        tau = [[se.tau(n, Fx(M["t0"]), Fx(M["D"]), [Fx(v) for v in M["kv"]], Fx(M["beta_D"]), Fx(M["E"][p][n - 1]),
                       Fx(M["beta"][p][n - 1]), Fx(M["phi"][p][n - 1])) for n in range(1, n_max + 1)] for p in (0, 1)]
        for p in (0, 1):
            for n in range(n_max):
                assert abs(out["tau"][p][n] - float(tau[p][n])) <= 1e-12 * float(tau[p][n])
        S = {n: tau[0][n - 1] - tau[1][n - 1] for n in range(1, n_max + 1)}
        assert out["crossover"] == se.crossover(S, n_max)
        for p in (0, 1):
            V = [tau[0][0] + Fx(M["h"][0])] + [tau[p][k] + Fx(M["h"][k]) for k in range(1, n_max)]
            for k in range(n_max):
                assert abs(out["V"][p][k] - float(V[k])) <= 1e-12 * float(V[k])
            assert abs(out["a0"][p] - float(se.a0(V))) <= 1e-12
            for ia, av in enumerate(a):
                af = F(av)
                ks = se.kstar(af, V)
                # skip exact near-ties, where double rounding may pick the other maximizer
                Ts = sorted((se.T(af, k, V) for k in range(n_max)), reverse=True)
                if n_max > 1 and (Ts[0] - Ts[1]) <= F(1, 10 ** 9) * Ts[0]:
                    continue
                assert out["kstar"][p][ia] == ks
                assert abs(out["speedup"][p][ia] - float(se.speedup(af, ks, V))) <= 1e-12
            for j in range(1, n_max):
                lo, hi = se.step_point_bracket(j, V)
                assert float(lo) - 1e-12 <= out["step_point"][p][j] <= float(hi) + 1e-12
            assert out["convex"][p] == int(se.is_convex_nondecreasing(V))
            assert abs(out["a1_convex"][p] - float(se.a1_convex(V))) <= 1e-12
        for ia, av in enumerate(a):
            af = F(av)
            for k in range(1, n_max):
                want = se.rho_star_time(k, af, 1, Fx(M["m_W"]), tau[0][0], Fx(M["beta"][0][0]),
                                        Fx(M["beta"][1][k]), Fx(M["kv"][k]) - Fx(M["kv"][0]), Fx(M["beta_D"]),
                                        Fx(M["phi"][1][k]) - Fx(M["phi"][0][0]))
                assert abs(out["rho_star"][ia][k] - float(want)) <= 1e-9 * max(1.0, abs(float(want)))
                wb = se.rho_star_bytes(k, af, 1, Fx(M["m_W"]), Fx(M["D"]), [Fx(v) for v in M["kv"]])
                assert abs(out["rho_star_bytes"][ia][k] - float(wb)) <= 1e-9 * max(1.0, abs(float(wb)))


def test_step_time_model_printed_examples():
    # Appendix B.3 'Jumps': V = (1, 2, 2) with one bandwidth: E_dedup = (1, 2, 2), beta = 1
    out = efa.step_time_model(3, [0.5, 0.9], 1.0, E=[[1, 2, 3], [1, 2, 2]], beta=[[1, 1, 1], [1, 1, 1]])
    assert list(out["V"][1]) == [1, 2, 2]
    assert out["kstar"][1][0] == 0 and out["kstar"][1][1] == 2
    # Appendix B.2: rho*_1 = 7/20, rho*_2 = 371/800 at a = 13/20 (byte form, m W = 1, D = kv = 0)
    out = efa.step_time_model(3, [13 / 20], 1.0, E=[[1, 2, 3], [1, 2, 2]], beta=[[1, 1, 1], [1, 1, 1]])
    assert abs(out["rho_star_bytes"][0][1] - 7 / 20) < 1e-15
    assert abs(out["rho_star_bytes"][0][2] - 371 / 800) < 1e-15
    # and the time form equals the byte form for one bandwidth and t0 = phi = 0
    assert abs(out["rho_star"][0][1] - 7 / 20) < 1e-15 and abs(out["rho_star"][0][2] - 371 / 800) < 1e-15


def test_step_time_model_rejects_bad_input():
    with pytest.raises(efa.MoeError):
        efa.step_time_model(1, [0.5], 1.0, E=[[1], [1]], beta=[[1], [1]])
    with pytest.raises(efa.MoeError):
        efa.step_time_model(2, [0.5], 1.0, E=[[1, 2], [1, 2]], beta=[[1, 0], [1, 1]])
    with pytest.raises(efa.MoeError):
        efa.step_time_model(2, [1.5], 1.0, E=[[1, 2], [1, 2]], beta=[[1, 1], [1, 1]])


def test_router_host_validation():
    L = _abi.lib()
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    assert L.moe_router_workspace_bytes(ctypes.byref(_desc(N=64, m=6, d_model=2048, dtype=_abi.MOE_BF16)), 8) == (
        4 * 8 * 64 * 4)
    d = _desc(N=512, m=8, d_model=2048, dtype=_abi.MOE_BF16)
    need = L.moe_router_workspace_bytes(ctypes.byref(d), 8)
    # 32 expert blocks x 1 token block: 4 parts of the contraction (the most)
    assert need == 4 * 8 * 512 * 4
    assert L.moe_router_workspace_bytes(ctypes.byref(_desc(N=64, m=65)), 8) == 0
    assert L.moe_router_topk(ctypes.byref(_desc(N=64, m=6)), fake, fake, 8, fake, fake, fake, fake, 255,
                             None) == _abi.MOE_E_WORKSPACE
    assert L.moe_router_topk(ctypes.byref(_desc(N=64, m=6)), fake, fake, 8, fake, fake, fake, None, 1 << 20,
                             None) == _abi.MOE_E_INVAL
    assert L.moe_router_workspace_bytes(ctypes.byref(d), 65) == 0
    args = lambda dd, n, ws_bytes: (ctypes.byref(dd), fake, fake, n, fake, fake, fake, fake, ws_bytes, None)
    assert L.moe_router_topk(*args(d, 8, need - 1)) == _abi.MOE_E_WORKSPACE
    assert L.moe_router_topk(*args(_desc(N=64, m=65), 8, need)) == _abi.MOE_E_INVAL
    assert L.moe_router_topk(*args(_desc(d_model=60), 8, need)) == _abi.MOE_E_DTYPE
    assert L.moe_router_topk(ctypes.byref(d), vp(0x1004), fake, 8, fake, fake, fake, fake, need,
                             None) == _abi.MOE_E_INVAL


def test_expert_auto_rejects_negative_crossover():
    L = _abi.lib()
    fake = ctypes.c_void_p(0x1000)
    W = _abi.LayerWeights(0x1000, 0x1000, 0x1000)
    d = _desc()
    assert L.moe_expert_auto(ctypes.byref(d), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake, 1 << 30, -1,
                             None, None) == _abi.MOE_E_INVAL
    # a bad descriptor is reported by the kernel it would run, before any launch
    assert L.moe_expert_auto(ctypes.byref(_desc(m=0)), ctypes.byref(W), fake, fake, fake, 4, fake, None, fake,
                             1 << 30, 2, None, None) == _abi.MOE_E_INVAL


def test_c_program_uses_the_abi(tmp_path):
    """The header compiles as C99 (-Wall -Werror) and a C program linked against the
    library gets host results equal to the Python binding's, and validation errors
    before any launch (no GPU needed)."""
    exe = str(tmp_path / "abi_host")
    lib_dir = os.path.dirname(_abi.SO_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, "-L", lib_dir, "-lmoe_expert",
           "-Wl,-rpath," + lib_dir]
    import subprocess
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    out = dict(l.split(" ", 1) for l in r.stdout.strip().splitlines())
    assert out["failures"] == "0"
    d = _desc(N=64, m=6, d_model=2048, d_ff=1408, dtype=_abi.MOE_BF16)
    assert int(out["workspace_slot_n8"]) == _abi.lib().moe_workspace_bytes(ctypes.byref(d), 8, 0)


def test_missing_library_fails_loudly():
    """Without the built library every op raises at once: there is no other path."""
    import subprocess
    import sys
    code = ("import expert_ffn_amd as efa\n"
            "from expert_ffn_amd import _abi\n"
            "_abi.SO_PATH = _abi.SO_PATH + '.absent'\n"
            "try:\n"
            "    efa.kernels_per_call(efa.MOE_KIND_SLOT)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=root)
    assert p.returncode == 0, p.stderr
    assert p.stdout.startswith("raised:") and "not built" in p.stdout


def test_gate_up_split_covers_every_step_once(tmp_path):
    """The gate/up work split the kernels use (gate_up_groups and the share
    arithmetic of k_expert, compiled from the kernel header into a host program):
    over tile counts 1 .. 808, K step counts 1 .. 512 and both kernels' bounds, every
    (tile, K step) is covered by exactly one work group, each cut tile's computed
    contributors are exactly the work groups meeting it (consecutive, at most
    kMaxContrib, the finaliser last), and the arithmetic stays below 2^31; the same
    for the remainder cut (RcPlan) over tile counts up to 131067 and K steps 2..512."""
    exe = str(tmp_path / "gate_up_plan_check")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    import subprocess
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "gate_up_plan_check.cpp"), "-o", exe],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout
