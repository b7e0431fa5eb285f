"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects invalid arguments on the host before touching a
GPU.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_15_amd as moe
from mixture_experts_layer_15_amd import configs
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    """Every function the headers under include/ declare."""
    import glob
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from mixture_experts_layer_15_amd import build
        build.build()
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    decl = _declared()
    assert set(decl) == set(moe.EXPORTS), decl
    for name in decl:
        assert hasattr(L, name), name
    # the exported names are plain C symbols (no C++ mangling)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = set(re.findall(r" T (moe_\w+)", out))
    assert set(decl) <= syms


def test_status_codes_and_strings(L):
    # the status values the header declares: 0 for success, negative errors
    text = open(HEADER).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"\b(MOE_(?:OK|ERR_\w+))\s*=\s*(-?\d+)", text))
    assert codes == {"MOE_OK": 0, "MOE_ERR_INVALID_ARG": -1, "MOE_ERR_UNSUPPORTED": -2,
                     "MOE_ERR_WORKSPACE": -3, "MOE_ERR_HIP": -4}
    for name, v in codes.items():
        assert getattr(moe, name) == v
        assert L.moe_status_string(v) == name.encode()
    assert L.moe_status_string(99) == b"MOE_ERR_UNKNOWN"
    assert L.moe_status_string(3) == b"MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("ci", range(len(configs.CONFIGS)))
def test_capacity_matches_oracle(L, ci):
    cfg = configs.CONFIGS[ci]
    want = orc.capacity(cfg.T, cfg.E, cfg.k, cfg.cap_num, cfg.cap_den)
    assert moe.capacity(cfg) == want
    assert moe.max_rows(cfg) == min(cfg.T * cfg.k, min(want, cfg.T) * cfg.E)


def test_capacity_edge_values(L):
    base = configs.get("tiny")
    for (T, E, k, n, dd, want) in [(10, 3, 1, 5, 4, 5), (12, 3, 1, 1, 1, 4), (7, 2, 2, 0, 1, 0),
                                   (0, 4, 1, 5, 4, 0), (1 << 20, 256, 8, 1 << 30, 1, None)]:
        c = base.scaled(T=T, E=E, k=k, cap_num=n, cap_den=dd)
        got = moe.capacity(c)
        if want is None:   # huge factor: exact ceil, no overflow
            assert got == -(-(n * k * T) // (dd * E))
        else:
            assert got == want == orc.capacity(T, E, k, n, dd)


BAD = [
    (dict(k=5), "k"), (dict(k=9, E=16), "k"), (dict(E=0, k=1), "E"), (dict(E=257), "E"),
    (dict(d=96), "d"), (dict(d=0), "d"), (dict(d_ff=100), "d_ff"), (dict(T=-1), "T"),
    (dict(T=1 << 30, k=2, E=4), "T * k"), (dict(temperature=0.0), "temperature"),
    (dict(temperature=-1.0), "temperature"), (dict(temperature=float("inf")), "temperature"),
    (dict(temperature=float("nan")), "temperature"), (dict(cap_num=-1, cap_den=4), "capacity"),
    (dict(cap_den=-1), "capacity"), (dict(drop_policy=2), "drop_policy"),
    (dict(drop_policy=-1), "drop_policy"),
]


@pytest.mark.parametrize("kw,word", BAD)
def test_invalid_config_rejected_on_host(L, kw, word):
    cfg = configs.get("tiny").scaled(**kw)
    c = moe.cconfig(cfg)
    assert L.moe_capacity(ctypes.byref(c)) == -1
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_workspace_size(ctypes.byref(c), ctypes.byref(n)) == \
        moe.MOE_ERR_INVALID_ARG
    fake = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    st = L.moe_route(ctypes.byref(c), fake, fake, None, fake, fake, fake, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    assert word in L.moe_last_error().decode()


def test_bad_flags_and_dtype(L):
    c = moe.cconfig(configs.get("tiny"))
    c.renormalize = 2
    assert L.moe_capacity(ctypes.byref(c)) == -1
    c = moe.cconfig(configs.get("tiny"))
    c.dtype = 7
    n = ctypes.c_size_t(0)
    assert L.moe_dispatch_workspace_size(ctypes.byref(c), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size(None, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch_workspace_size(None, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_rejected(L):
    c = moe.cconfig(configs.get("zaya1"))
    ok = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert L.moe_route(ctypes.byref(c), None, ok, None, ok, ok, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert b"x is NULL" in L.moe_last_error()
    assert L.moe_route(ctypes.byref(c), ok, odd, None, ok, ok, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert b"aligned" in L.moe_last_error()
    assert L.moe_combine(ctypes.byref(c), ok, ok, ok, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(ctypes.byref(c), ok, None, ok, ok, ok, ok, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_from_logits(ctypes.byref(c), ok, ok, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_load_stats(ctypes.byref(c), None, ok, None) == moe.MOE_ERR_INVALID_ARG
    assert b"expert_count is NULL" in L.moe_last_error()
    assert L.moe_load_stats(ctypes.byref(c), ok, None, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_load_stats(ctypes.byref(c), ok, odd, None) == moe.MOE_ERR_INVALID_ARG


def test_mlp_router_validation_on_host(L):
    cfg = configs.get("zaya1")
    c = moe.cconfig(cfg)
    ok = 1 << 20
    n = ctypes.c_size_t(0)
    good = dict(r=256, m=1024, gamma=0.5, eps=1e-6, w_down=ok, w1=ok, w2=ok, w3=ok)
    r = moe.CMLPRouter(**good)
    assert L.moe_mlp_router_workspace_size(ctypes.byref(c), ctypes.byref(r), ctypes.byref(n)) == 0
    T, rr, m, E = cfg.T, 256, 1024, cfg.E
    al = lambda v: (v + 255) // 256 * 256
    assert n.value == 2 * al(T * rr * 2) + 2 * al(T * m * 2) + al(E * 4)
    for bad, word in [(dict(r=96), "r ="), (dict(r=2048), "r ="), (dict(m=100), "m ="),
                      (dict(gamma=float("nan")), "gamma"), (dict(eps=-1.0), "eps")]:
        rb = moe.CMLPRouter(**dict(good, **bad))
        assert L.moe_mlp_router_workspace_size(ctypes.byref(c), ctypes.byref(rb),
                                               ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
        assert word in L.moe_last_error().decode()
    assert L.moe_mlp_router_workspace_size(ctypes.byref(c), None, ctypes.byref(n)) == \
        moe.MOE_ERR_INVALID_ARG
    f32 = moe.cconfig(configs.get("tiny"))
    assert L.moe_mlp_router_workspace_size(ctypes.byref(f32), ctypes.byref(r), ctypes.byref(n)) == \
        moe.MOE_ERR_UNSUPPORTED
    # missing weight, missing workspace: rejected before any launch
    rw = moe.CMLPRouter(**dict(good, w2=None))
    v = ctypes.c_void_p(ok)
    assert L.moe_route_mlp(ctypes.byref(c), ctypes.byref(rw), v, None, v, v, v, v, 1 << 40,
                           None) == moe.MOE_ERR_INVALID_ARG
    assert b"w2 is NULL" in L.moe_last_error()
    assert L.moe_route_mlp(ctypes.byref(c), ctypes.byref(r), v, None, v, v, v, None, 0,
                           None) == moe.MOE_ERR_WORKSPACE


def test_choice_order_workspace_is_sized_for_the_walked_choices(L):
    # the dispatch tables hold 2 * nblk * E int32, nblk <= 256 blocks of whole
    # 256-token chunks over the walked tokens: T in token order, T*k single
    # choices in choice order
    def want(walked, E):
        chunks = -(-walked // 256)
        blk = max(-(-chunks // 256), 1) * 256
        return 2 * max(-(-walked // blk), 1) * E * 4
    for name in ("wide", "skewed", "longseq"):
        cfg = configs.get(name)
        assert moe.workspace_bytes(cfg, dispatch_only=True) == want(cfg.T, cfg.E)
        assert moe.workspace_bytes(cfg.scaled(drop_policy=1), dispatch_only=True) == \
            want(cfg.T * cfg.k, cfg.E)


def _al(v):
    return (v + 255) // 256 * 256


def _fwd_ws_want(cfg, x_perm: bool, y_perm: bool, parts: bool):
    """moe_forward's workspace, region by region (each 256-byte aligned):
    logits, topk idx and gate, counts, offsets, row_of, token_of_row, the
    dispatch tables, then x_perm / h / y_perm / fp32 K-slice partials."""
    R, d, F, E, T, k = moe.max_rows(cfg), cfg.d, cfg.d_ff, cfg.E, cfg.T, cfg.k
    es = 2 if cfg.dtype == "bf16" else 4
    tor = max(T * k, R)
    fixed = _al(T * E * 4) + 2 * _al(T * k * 4) + _al(E * 4) + _al((E + 1) * 4) + \
        _al(T * k * 4) + _al(tor * 4) + _al(moe.workspace_bytes(cfg, dispatch_only=True))
    return fixed + _al(R * d * es if x_perm else 0) + _al(R * F * es) + \
        _al(R * d * es if y_perm else 0) + _al(2 * R * d * 4 if parts else 0)


def test_forward_workspace_holds_only_the_buffers_the_path_uses(L):
    # bf16 compact layers gather x rows inside the gate/up GEMM (no x_perm);
    # bf16 top-1 layers that keep every token have the down GEMM write y (no
    # y_perm), and with too few experts to fill the CUs with down tiles (the
    # ZAYA1-like layer: 16 experts, 128 tiles of 320 x 256) the down GEMM runs
    # in two K slices whose fp32 partials [2][R][d] live in the workspace.
    # Host-only: sizes, no GPU call.
    assert moe.workspace_bytes(configs.get("zaya1")) == \
        _fwd_ws_want(configs.get("zaya1"), x_perm=False, y_perm=False, parts=True)
    for name in ("wide", "skewed", "longseq"):
        cfg = configs.get(name)
        assert moe.workspace_bytes(cfg) == _fwd_ws_want(cfg, x_perm=False, y_perm=True,
                                                       parts=False), name
    # fp32: the staged buffers all present
    tiny = configs.get("tiny")
    assert moe.workspace_bytes(tiny) == _fwd_ws_want(tiny, x_perm=True, y_perm=True, parts=False)
    # the padded layout scatters x into x_perm
    pad = configs.get("wide").scaled(layout=1)
    assert moe.workspace_bytes(pad) == _fwd_ws_want(pad, x_perm=True, y_perm=True, parts=False)
    # top-1 with drops: y_perm and a combine
    capped = configs.get("zaya1").scaled(cap_num=1, cap_den=1)
    assert moe.workspace_bytes(capped) == _fwd_ws_want(capped, x_perm=False, y_perm=True,
                                                       parts=False)


def test_workspace_too_small_rejected(L):
    cfg = configs.get("wide")
    c = moe.cconfig(cfg)
    ok = ctypes.c_void_p(1 << 20)
    need = moe.workspace_bytes(cfg, dispatch_only=True)
    st = L.moe_dispatch(ctypes.byref(c), ok, ok, ok, ok, ok, ok, ok, ok, need - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE and b"need" in L.moe_last_error()
    st = L.moe_dispatch(ctypes.byref(c), ok, ok, ok, ok, ok, ok, ok, None, need, None)
    assert st == moe.MOE_ERR_WORKSPACE
    fneed = moe.workspace_bytes(cfg)
    st = L.moe_forward(ctypes.byref(c), ok, ok, None, ok, ok, ok, ok, ok, fneed - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE


def test_workspace_sizes_cover_intermediates(L):
    for cfg in configs.CONFIGS:
        R = moe.max_rows(cfg)
        es = 2 if cfg.dtype == "bf16" else 4
        inter = R * cfg.d_ff * es + cfg.T * (cfg.E + 4 * cfg.k) * 4
        assert moe.workspace_bytes(cfg) >= inter
        assert 0 < moe.workspace_bytes(cfg, dispatch_only=True) <= 2 * 256 * cfg.E * 4


def test_python_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", "/nonexistent/libmoe_mi355x.so")
    with pytest.raises(RuntimeError, match="not found"):
        moe.lib()


def test_backward_validation_on_host(L):
    cfg = configs.get("zaya1")
    c = moe.cconfig(cfg)
    n = ctypes.c_size_t(0)
    assert L.moe_backward_workspace_size(ctypes.byref(c), ctypes.byref(n)) == 0
    R, T, d, E, F, k = moe.max_rows(cfg), cfg.T, cfg.d, cfg.E, cfg.d_ff, cfg.k
    # the recomputed pre-activations, dg/du in place, gate * h, the per-row gate
    # and dgate partials (one per 64 columns; dh itself is never stored), x and
    # dy in expert order, the expert input gradients (fp32, up to four K
    # slices), the routing maps and the logit gradients
    base = R * F * 3 * 2 + R * 4 + R * (F // 64) * 4 + 2 * R * d * 2 + T * E * 4 * 2 + \
        T * k * 4 * 4
    assert n.value >= base + 2 * R * d * 4
    assert n.value < base + 8 * R * d * 4 + (64 << 20)
    # fp32 layers too: their rows and pre-activations take 4 bytes per element
    t32 = configs.get("tiny")
    f32 = moe.cconfig(t32)
    n32 = ctypes.c_size_t(0)
    assert L.moe_backward_workspace_size(ctypes.byref(f32), ctypes.byref(n32)) == 0
    R32 = moe.max_rows(t32)
    assert n32.value >= R32 * t32.d_ff * 3 * 4 + 2 * R32 * t32.d * 4 + R32 * t32.d * 4
    assert L.moe_backward_workspace_size(ctypes.byref(c), None) == moe.MOE_ERR_INVALID_ARG
    ok = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    big = 1 << 40

    def call(**over):
        a = dict(x=ok, wr=ok, bias=None, wg=ok, wu=ok, wd=ok, dy=ok, dx=ok, dwr=ok, db=None,
                 dwg=ok, dwu=ok, dwd=ok, dgate=None, ws=ok, nbytes=big)
        a.update(over)
        return L.moe_backward(ctypes.byref(c), a["x"], a["wr"], a["bias"], a["wg"], a["wu"],
                              a["wd"], a["dy"], a["dx"], a["dwr"], a["db"], a["dwg"], a["dwu"],
                              a["dwd"], a["dgate"], a["ws"], a["nbytes"], None)
    for name in ("x", "dy", "dx", "dwr", "dwg", "dwu", "dwd", "wd"):
        assert call(**{name: None}) == moe.MOE_ERR_INVALID_ARG
        assert b"is NULL" in L.moe_last_error()
    assert call(dwg=odd) == moe.MOE_ERR_INVALID_ARG
    assert b"aligned" in L.moe_last_error()
    assert call(nbytes=n.value - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    bad = moe.cconfig(cfg)
    bad.k = 0
    assert L.moe_backward(ctypes.byref(bad), *([ok] * 15), big, None) == moe.MOE_ERR_INVALID_ARG


def test_padded_layout_validation_and_sizes(L):
    n = ctypes.c_size_t(0)
    bad = moe.cconfig(configs.get("wide"))
    bad.layout = 2
    assert L.moe_max_rows(ctypes.byref(bad)) == -1
    assert b"moe_layout" in L.moe_last_error()
    nocap = moe.cconfig(configs.get("zaya1").scaled(layout=1))
    assert L.moe_workspace_size(ctypes.byref(nocap), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert b"capacity limit" in L.moe_last_error()
    huge = moe.cconfig(configs.get("wide").scaled(T=(1 << 28) - 1, E=256, k=8, layout=1))
    assert L.moe_max_rows(ctypes.byref(huge)) == -1 and b"2^31" in L.moe_last_error()
    for name in ("wide", "skewed", "longseq"):
        cfg = configs.get(name)
        C = min(moe.capacity(cfg), cfg.T)
        pad = cfg.scaled(layout=1)
        assert moe.max_rows(pad) == cfg.E * C >= moe.max_rows(cfg)
        assert moe.workspace_bytes(pad) > moe.workspace_bytes(cfg)
        # the backward runs on it too, its workspace sized for the E * C rows
        nc = ctypes.c_size_t(0)
        assert L.moe_backward_workspace_size(ctypes.byref(moe.cconfig(pad)), ctypes.byref(n)) == 0
        assert L.moe_backward_workspace_size(ctypes.byref(moe.cconfig(cfg)), ctypes.byref(nc)) == 0
        assert n.value >= nc.value
        # token_of_row holds one entry per row of the padded layout (E * C of
        # them, more than the T * k assignment slots here)
        assert cfg.E * C > cfg.T * cfg.k
        assert n.value - nc.value >= (cfg.E * C - cfg.T * cfg.k) * 4
    # token_of_row must cover max(T * k, rows): too small a buffer is not checked
    # on the host (it is a device pointer), but the binding sizes it that way
    cfg = configs.get("skewed").scaled(layout=1)
    assert max(cfg.T * cfg.k, moe.max_rows(cfg)) == moe.max_rows(cfg)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_dynamic_expert_count_validation_on_host(L):
    # each token takes k_min .. k experts by a softmax-mass threshold: host
    # checks of its fields, and the one place it is not supported, the padded
    # layout (no GPU call)
    cfg = configs.get("tiny").scaled(dtype="bf16", k=4, E=16, k_min=2, route_threshold=0.6,
                                     renormalize=True, cap_num=5, cap_den=4)
    ok = ctypes.c_void_p(1 << 20)
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(moe.cconfig(cfg)), ctypes.byref(n)) == moe.MOE_OK
    # capacity and rows: the bound for T * k assignments
    assert moe.capacity(cfg) == orc.capacity(cfg.T, cfg.E, cfg.k, 5, 4)
    # the backward runs it too, with the workspace of the fixed-k layer (rows
    # bounded by the same capacity)
    nb = ctypes.c_size_t(0)
    fixed = moe.cconfig(cfg.scaled(k_min=0, route_threshold=0.0))
    assert L.moe_backward_workspace_size(ctypes.byref(moe.cconfig(cfg)), ctypes.byref(n)) == \
        moe.MOE_OK
    assert L.moe_backward_workspace_size(ctypes.byref(fixed), ctypes.byref(nb)) == moe.MOE_OK
    assert n.value == nb.value > 0
    pad = moe.cconfig(cfg.scaled(layout=1))
    assert L.moe_workspace_size(ctypes.byref(pad), ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    for bad in (cfg.scaled(k_min=0), cfg.scaled(k_min=5), cfg.scaled(route_threshold=1.5),
                cfg.scaled(route_threshold=0.0), cfg.scaled(route_threshold=float("nan")),
                cfg.scaled(route_threshold=-0.5)):
        assert L.moe_route(ctypes.byref(moe.cconfig(bad)), ok, ok, None, ok, ok, ok, None) == \
            moe.MOE_ERR_INVALID_ARG


def test_pid_update_validation_on_host(L):
    # the load-balance PID controller: NULL and non-finite arguments are
    # rejected before any launch
    cfg = moe.cconfig(configs.get("tiny").scaled(E=16, k=2))
    ok = ctypes.c_void_p(1 << 20)
    good = moe.CPIDGains(kp=0.2, ki=0.02, kd=0.0, scale=1.0)
    inv = moe.MOE_ERR_INVALID_ARG
    assert L.moe_pid_update(ctypes.byref(cfg), None, ok, ok, ok, None) == inv
    for f in ("kp", "ki", "kd", "scale"):
        for v in (float("nan"), float("inf")):
            g = moe.CPIDGains(kp=0.2, ki=0.02, kd=0.0, scale=1.0)
            setattr(g, f, v)
            assert L.moe_pid_update(ctypes.byref(cfg), ctypes.byref(g), ok, ok, ok, None) == inv
            assert f in L.moe_last_error().decode() or "finite" in L.moe_last_error().decode()
    for args in ((None, ok, ok), (ok, None, ok), (ok, ok, None)):
        assert L.moe_pid_update(ctypes.byref(cfg), ctypes.byref(good), *args, None) == inv
    bad = moe.cconfig(configs.get("tiny").scaled(E=16, k=2))
    bad.E = 0
    assert L.moe_pid_update(ctypes.byref(bad), ctypes.byref(good), ok, ok, ok, None) == inv
