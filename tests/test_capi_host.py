"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host before any HIP call
(a rejected call never reaches the device, so fake pointers are safe here)."""

import ctypes
import os
import re

import pytest

import mamba_selective_scan_ssm_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.LIB_PATH):
        pytest.skip("libssmscan.so not built")
    return ssm.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_scan_fwd_workspace_size", "ssm_state_update", "ssm_ssd_fwd",
              "ssm_ssd_fwd_workspace_size", "ssm_conv1d_fwd", "ssm_conv1d_update",
              "ssm_scan_fwd_ex", "ssm_state_update_ex", "ssm_ssd_fwd_ex", "ssm_decode_steps",
              "ssm_scan_bwd", "ssm_scan_bwd_workspace_size", "ssm_scan_bwd_workspace_size_ex",
              "ssm_scan_fwd_train",
              "ssm_status_string", "ssm_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert ssm.version() >= 100
    for code in range(5):
        assert lib.ssm_status_string(code)


# fake, distinct, 256-byte-aligned "device" addresses: never dereferenced
P = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(16)]


def scan(lib, B=2, L=8, D=64, N=16, dt=F32, ptrs=None, ws=None, ws_len=0, tun=None, **over):
    p = dict(x=P[0], delta=P[1], A=P[2], Bm=P[3], Cm=P[4], D_skip=P[5], z=P[6], h0=P[7], y=P[8],
             h_final=P[9])
    p.update(over)
    return lib.ssm_scan_fwd(B, L, D, N, dt, p["x"], p["delta"], p["A"], p["Bm"], p["Cm"],
                            p["D_skip"], p["z"], p["h0"], p["y"], p["h_final"], ws, ws_len,
                            ctypes.byref(tun) if tun is not None else None, None)


def test_scan_rejects_negative_sizes(lib):
    for kw in (dict(B=-1), dict(L=-1), dict(D=-5), dict(N=-2)):
        assert scan(lib, **kw) == INVALID


def test_scan_rejects_large_n_and_bad_dtype(lib):
    assert scan(lib, N=65) == UNSUPPORTED
    assert scan(lib, dt=7) == INVALID
    assert scan(lib, B=1, L=1 << 20, D=1024, dt=BF16) == UNSUPPORTED   # 2 GiB plane


def test_scan_rejects_null_required(lib):
    for name in ("x", "delta", "A", "Bm", "Cm", "y"):
        assert scan(lib, **{name: None}) == INVALID, name


def test_scan_rejects_aliasing(lib):
    assert scan(lib, y=P[0]) == INVALID                        # y on x
    assert scan(lib, h_final=P[7]) == INVALID                  # h_final on h0
    assert scan(lib, y=ctypes.c_void_p(P[1].value + 64)) == INVALID  # y inside delta


def test_scan_empty_batch_is_noop(lib):
    assert scan(lib, B=0) == OK
    assert scan(lib, D=0) == OK


def test_scan_tuning_validation(lib):
    t = ssm.Tuning(5, 0)  # variants 0..4
    assert scan(lib, tun=t) == INVALID
    t = ssm.Tuning(2, 12)
    assert scan(lib, tun=t) == INVALID
    t = ssm.Tuning(0, 0)
    t.reserved[2] = 1
    assert scan(lib, tun=t) == INVALID


def test_scan_chunked_needs_workspace(lib):
    t = ssm.Tuning(2, 64)
    need = lib.ssm_scan_fwd_workspace_size(2, 1024, 64, 16, ctypes.byref(t))
    summaries = 2 * 2 * 16 * 64 * 16       # (a, h) x B x segments x D x N, fp32
    assert need == summaries * 4
    assert scan(lib, L=1024, tun=t) == WORKSPACE
    assert scan(lib, L=1024, tun=t, ws=P[12], ws_len=need - 4) == WORKSPACE
    # workspace overlapping an input is rejected too
    assert scan(lib, L=1024, tun=t, ws=P[0], ws_len=need) == INVALID


def test_sequential_needs_no_workspace(lib):
    for spl in (0, 2, 4, 8, 16):
        t = ssm.Tuning(1, 0, spl)
        assert lib.ssm_scan_fwd_workspace_size(8, 4096, 5120, 16, ctypes.byref(t)) == 0
    t = ssm.Tuning(1, 0, 3)
    assert scan(lib, tun=t) == INVALID


def step(lib, S=4, D=64, N=16, dt=BF16, **over):
    p = dict(state=P[0], x=P[1], delta=P[2], A=P[3], Bm=P[4], Cm=P[5], D_skip=P[6], z=P[7], y=P[8])
    p.update(over)
    return lib.ssm_state_update(S, D, N, dt, p["state"], p["x"], p["delta"], p["A"], p["Bm"], p["Cm"],
                                p["D_skip"], p["z"], p["y"], None)


def test_state_update_validation(lib):
    assert step(lib, S=-1) == INVALID
    assert step(lib, N=80) == UNSUPPORTED
    assert step(lib, state=None) == INVALID
    assert step(lib, y=P[0]) == INVALID   # y on the state
    assert step(lib, y=P[1]) == INVALID   # y on x
    assert step(lib, S=0) == OK


def ssd(lib, B=1, L=512, H=8, P_=64, G=2, N=128, chunk=256, dt=BF16, ws=None, ws_len=0, **over):
    p = dict(x=P[0], dtv=P[1], A=P[2], Bm=P[3], Cm=P[4], D_skip=P[5], z=P[6], h0=P[7], y=P[8],
             h_final=P[9])
    p.update(over)
    return lib.ssm_ssd_fwd(B, L, H, P_, G, N, chunk, dt, p["x"], p["dtv"], p["A"], p["Bm"], p["Cm"],
                           p["D_skip"], p["z"], p["h0"], p["y"], p["h_final"], ws, ws_len, None)


def test_ssd_validation(lib):
    # every call here is refused on the host, before any launch
    assert ssd(lib, B=-1) == INVALID
    assert ssd(lib, dt=7) == INVALID
    assert ssd(lib, N=300) == UNSUPPORTED                   # above SSM_SSD_MAX_N
    assert ssd(lib, chunk=0) == UNSUPPORTED
    assert ssd(lib, H=8, G=3) == UNSUPPORTED
    assert ssd(lib, y=P[0]) == INVALID
    assert ssd(lib, dt=F32, y=P[0]) == INVALID              # fp32 takes the token-by-token path,
    assert ssd(lib, P_=48, h_final=P[7]) == INVALID         # P != 64 too: same argument checks
    assert ssd(lib, A=None) == INVALID
    assert ssd(lib, B=0) == OK
    assert ssd(lib, P_=0) == OK
    # the matrix-core path needs its workspace; the other path needs none
    assert ssd(lib) == WORKSPACE
    assert lib.ssm_ssd_fwd_workspace_size(1, 512, 8, 64, 2, 128, 256) > 0
    for shape in ((1, 512, 8, 48, 2, 128, 256), (1, 512, 8, 64, 2, 100, 256), (1, 512, 8, 64, 2, 128, 100)):
        assert lib.ssm_ssd_fwd_workspace_size(*shape) == 0, shape


def test_scan_lanesplit_variant_limits(lib):
    """Variant 3 (states split over lanes) exists for N in {4, 8, 16, 32, 64}
    with 16-byte aligned B and C; elsewhere it is refused before any launch."""
    t = ssm.Tuning(3, 0)
    assert scan(lib, N=5, tun=t) == UNSUPPORTED
    assert scan(lib, N=12, tun=t) == UNSUPPORTED
    odd = ctypes.c_void_p(P[3].value + 2)
    assert scan(lib, Bm=odd, tun=t) == UNSUPPORTED


def conv(lib, B=2, L=8, D=64, K=4, dt=F32, act=1, **over):
    p = dict(x=P[0], w=P[1], bias=P[2], s_in=P[3], y=P[4], s_out=P[5])
    p.update(over)
    return lib.ssm_conv1d_fwd(B, L, D, K, dt, p["x"], p["w"], p["bias"], p["s_in"], act, p["y"],
                              p["s_out"], None)


def conv_upd(lib, S=2, D=64, K=4, dt=F32, act=1, **over):
    p = dict(state=P[0], x=P[1], w=P[2], bias=P[3], y=P[4])
    p.update(over)
    return lib.ssm_conv1d_update(S, D, K, dt, p["state"], p["x"], p["w"], p["bias"], act, p["y"], None)


def test_conv_validation(lib):
    assert conv(lib, B=-1) == INVALID
    assert conv(lib, act=2) == INVALID
    assert conv(lib, dt=7) == INVALID
    assert conv(lib, K=1) == UNSUPPORTED
    assert conv(lib, K=9) == UNSUPPORTED
    assert conv(lib, B=0) == OK
    assert conv(lib, D=0) == OK
    assert conv(lib, w=None) == INVALID
    assert conv(lib, x=None) == INVALID
    assert conv(lib, y=None) == INVALID
    assert conv(lib, y=P[0]) == INVALID                  # y on x
    assert conv(lib, s_out=P[3]) == INVALID              # state_out on state_in
    assert conv(lib, L=1 << 30) == UNSUPPORTED


def test_conv_update_validation(lib):
    assert conv_upd(lib, S=-1) == INVALID
    assert conv_upd(lib, act=-1) == INVALID
    assert conv_upd(lib, K=9) == UNSUPPORTED
    assert conv_upd(lib, S=0) == OK
    assert conv_upd(lib, state=None) == INVALID
    assert conv_upd(lib, y=P[0]) == INVALID              # y on the state
    assert conv_upd(lib, x=P[0]) == INVALID              # x on the state
    assert conv_upd(lib, S=65536) == UNSUPPORTED   # one grid row per sequence


def test_delta_opts_validation(lib):
    """The step-size options are checked on the host like every argument."""
    def scan_ex(opts, **over):
        p = dict(x=P[0], delta=P[1], A=P[2], Bm=P[3], Cm=P[4], D_skip=P[5], z=P[6], h0=P[7], y=P[8],
                 h_final=P[9])
        p.update(over)
        return lib.ssm_scan_fwd_ex(2, 8, 64, 16, F32, p["x"], p["delta"], p["A"], p["Bm"], p["Cm"],
                                   p["D_skip"], p["z"], p["h0"], p["y"], p["h_final"], None, 0,
                                   None, ctypes.byref(opts) if opts is not None else None, None)
    assert scan_ex(ssm.DeltaOpts(None, 2)) == INVALID                 # softplus must be 0/1
    o = ssm.DeltaOpts(None, 1)
    o.reserved[1] = 5
    assert scan_ex(o) == INVALID                                       # reserved must be zero
    assert scan_ex(ssm.DeltaOpts(P[8].value, 1)) == INVALID           # bias on y


def test_decode_steps_validation(lib):
    def ds(S=4, T=3, D=64, N=16, pool=8, slots=None, **over):
        p = dict(pool=P[0], x=P[1], delta=P[2], A=P[3], Bm=P[4], Cm=P[5], D_skip=P[6], z=P[7], y=P[8])
        p.update(over)
        return lib.ssm_decode_steps(S, T, D, N, F32, p["pool"], pool, slots, p["x"], p["delta"], p["A"],
                                    p["Bm"], p["Cm"], p["D_skip"], p["z"], p["y"], None, None)
    assert ds(S=-1) == INVALID
    assert ds(pool=-1) == INVALID
    assert ds(N=65) == UNSUPPORTED
    assert ds(T=0) == OK and ds(S=0) == OK
    assert ds(pool=2) == INVALID                  # identity slots need pool_rows >= S
    assert ds(y=P[1]) == INVALID                  # y on x
    assert ds(pool=8, y=P[0]) == INVALID          # y inside the pool
    assert ds(x=None) == INVALID
    # an empty pool with slot indices: every slot is outside it, every
    # sequence is skipped and nothing is launched (no state row may be read)
    assert ds(pool=0, slots=P[9]) == OK
    assert ds(pool=0, slots=P[9], T=1) == OK
    assert ds(pool=0, slots=P[9], T=40) == OK


Q = [ctypes.c_void_p(0x4000000 * (i + 1)) for i in range(24)]  # 64 MiB apart


_DEFAULT = object()


def bwd(lib, B=2, L=8, D=64, N=16, dt=F32, ws=_DEFAULT, ws_len=None, **over):
    """Every call below must be rejected on the host: none may reach a launch."""
    names = ["x", "delta", "A", "Bm", "Cm", "D_skip", "z", "h0", "dy", "dh_final", "h_ckpt", "dx", "ddelta",
             "dz", "dA", "dB", "dC", "dD", "dh0", "dbias"]
    p = {k: Q[i] for i, k in enumerate(names)}
    p["h_ckpt"] = None
    p.update(over)
    if ws is _DEFAULT:
        ws = Q[21]
    if ws_len is None:
        ws_len = lib.ssm_scan_bwd_workspace_size(B, L, D, N)
    return lib.ssm_scan_bwd(B, L, D, N, dt, *(p[k] for k in names), None, ws, ws_len, None)


def test_scan_bwd_workspace_size(lib):
    assert lib.ssm_scan_bwd_workspace_size(2, 8, 64, 12) == 0
    # entering states (1 segment) + dB|dC partials (1 tile) + dA partials + dD, dbias partials
    want = (2 * 1 * 64 * 16 + 2 * 8 * 1 * 32 + 2 * 64 * 16 + 2 * 2 * 64) * 4
    assert lib.ssm_scan_bwd_workspace_size(2, 8, 64, 16) == want
    # 8-token segments, 64-channel tiles at N = 16
    assert lib.ssm_scan_bwd_workspace_size(1, 17, 65, 16) == (3 * 2 * 65 * 16 // 2 + 17 * 2 * 32 + 65 * 16 + 2 * 65) * 4
    # the _ex form: the same without saved states, no state region with them
    assert lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 16, 0) == want
    assert lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 16, 1) == want - 2 * 1 * 64 * 16 * 4
    assert lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 16, 2) == 0
    assert lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 12, 1) == 0


def test_scan_bwd_saved_states_take_the_smaller_workspace(lib):
    # with the forward's states a workspace of the _ex(.., 1) size is enough,
    # so the call passes validation (it would launch: stop at the size check
    # by giving one byte less, which must be rejected)
    need1 = lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 16, 1)
    assert bwd(lib, h_ckpt=Q[10], ws_len=need1 - 1) == WORKSPACE
    need0 = lib.ssm_scan_bwd_workspace_size_ex(2, 8, 64, 16, 0)
    assert bwd(lib, ws_len=need1) == WORKSPACE                 # recomputing needs the larger one
    assert need0 > need1


def test_scan_bwd_validation(lib):
    assert bwd(lib, B=-1) == INVALID
    assert bwd(lib, dt=7) == INVALID
    assert bwd(lib, N=12) == UNSUPPORTED
    assert bwd(lib, N=128) == UNSUPPORTED
    assert bwd(lib, B=70000) == UNSUPPORTED
    assert bwd(lib, dy=None) == INVALID
    assert bwd(lib, dx=None) == INVALID
    assert bwd(lib, dz=None) == INVALID                       # gate given, its gradient not
    assert bwd(lib, z=None) == INVALID                        # dz given without a gate
    assert bwd(lib, dB=None) == INVALID
    assert bwd(lib, A=ctypes.c_void_p(Q[2].value + 4)) == UNSUPPORTED
    assert bwd(lib, dh0=ctypes.c_void_p(Q[18].value + 8)) == UNSUPPORTED
    assert bwd(lib, h_ckpt=ctypes.c_void_p(Q[10].value + 8)) == UNSUPPORTED
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws_len=64) == WORKSPACE
    assert bwd(lib, ws=ctypes.c_void_p(Q[21].value + 4)) == WORKSPACE
    assert bwd(lib, dx=Q[0]) == INVALID                       # output on an input
    assert bwd(lib, dC=Q[15]) == INVALID                      # two outputs on one buffer
    assert bwd(lib, dA=Q[21]) == INVALID                      # output on the workspace
    assert bwd(lib, dB=Q[10], h_ckpt=Q[10]) == INVALID        # output on the saved states


def test_scan_fwd_train_validation(lib):
    def tr(B=2, L=16, D=64, N=16, dt=F32, **over):
        names = ["x", "delta", "A", "Bm", "Cm", "D_skip", "z", "h0", "y", "h_final", "h_ckpt"]
        p = {k: Q[i] for i, k in enumerate(names)}
        p.update(over)
        return lib.ssm_scan_fwd_train(B, L, D, N, dt, *(p[k] for k in names), None, None)
    assert tr(B=-1) == INVALID
    assert tr(h_ckpt=None) == INVALID
    assert tr(h_ckpt=ctypes.c_void_p(Q[10].value + 4)) == UNSUPPORTED
    assert tr(N=12) == UNSUPPORTED                            # lane-split schedule only
    assert tr(D=63) == UNSUPPORTED                            # odd D
    assert tr(h_ckpt=Q[9]) == INVALID                         # on h_final
    assert tr(y=Q[0]) == INVALID
    assert tr(N=65) == UNSUPPORTED


def test_scan_noalloc_limit_and_validation(lib):
    """ssm_scan_fwd_noalloc: a schedule needing more than the 16 MiB device
    scratch is refused with SSM_ERR_WORKSPACE, and bad arguments as in
    ssm_scan_fwd_ex -- all on the host, before any device call."""
    def na(B=2, L=8, D=64, N=16, dt=F32, tun=None, **over):
        p = dict(x=Q[0], delta=Q[1], A=Q[2], Bm=Q[3], Cm=Q[4], D_skip=Q[5], z=Q[6], h0=Q[7], y=Q[8],
                 h_final=Q[9])
        p.update(over)
        return lib.ssm_scan_fwd_noalloc(B, L, D, N, dt, p["x"], p["delta"], p["A"], p["Bm"], p["Cm"],
                                        p["D_skip"], p["z"], p["h0"], p["y"], p["h_final"],
                                        None if tun is None else ctypes.byref(tun), None, None)
    t = ssm.Tuning(2, 64)
    big = dict(B=4, L=4096, D=256, N=64)         # 33.5 MB of segment summaries
    assert lib.ssm_scan_fwd_workspace_size(*big.values(), ctypes.byref(t)) > 16 << 20
    assert na(**big, tun=t) == WORKSPACE
    assert na(B=-1) == INVALID
    assert na(y=None) == INVALID
    assert na(y=Q[0]) == INVALID                     # y on x
    assert na(N=65) == UNSUPPORTED
    assert na(tun=ssm.Tuning(5, 0)) == INVALID
