"""The C ABI without a GPU: the library loads, exports every symbol the header declares, and
rejects bad arguments on the host before enqueueing anything (no device work is started)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k3x.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(k3x_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def k3x():
    import mxfp4_routed_expert_k3x_amd as k

    k.load_library()
    return k


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("k3x_expert_pool_create", "k3x_route_topk", "k3x_moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(k3x):
    lib = k3x.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(k3x.EXPORTS) == set(declared_functions())


def test_python_binding_has_the_c_names(k3x):
    for n in declared_functions():
        assert hasattr(k3x, n), n


def _gpu_present():
    import torch

    return torch.cuda.is_available()


def _desc(k3x, **kw):
    d = k3x.k3x_pool_desc()
    d.n_experts, d.hidden, d.inter, d.group = 8, 256, 384, 32
    base = 1 << 40  # fake, never dereferenced: validation is host-only
    for i, n in enumerate(k3x.TENSOR_ORDER):
        setattr(d, n, base + i * (1 << 32))
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _create(k3x, d):
    h = ctypes.c_void_p()
    st = k3x.lib().k3x_expert_pool_create(ctypes.byref(d), ctypes.byref(h))
    return st, h.value


def test_pool_create_accepts_valid_desc(k3x):
    st, h = _create(k3x, _desc(k3x))
    assert st == k3x.K3X_OK and h
    k3x.lib().k3x_expert_pool_destroy(h)
    k3x.lib().k3x_expert_pool_destroy(None)  # no-op
    # SiTU-GLU with the checkpoint's caps; SwiGLU ignores the caps
    for kw in ({"activation": 1, "situ_b1": 4.0, "situ_b2": 25.0},
               {"activation": 0, "situ_b1": -1.0, "situ_b2": float("nan")}):
        st, h = _create(k3x, _desc(k3x, **kw))
        assert st == k3x.K3X_OK and h, kw
        k3x.lib().k3x_expert_pool_destroy(h)


@pytest.mark.parametrize("kw,want", [
    ({"group": 16}, -2),
    ({"group": 64}, -2),
    ({"hidden": 3500}, -2),
    ({"inter": 100}, -2),
    ({"hidden": 0}, -1),
    ({"n_experts": 0}, -1),
    ({"n_experts": 20000}, -1),
    ({"w2_scale": None}, -1),
    ({"w1_packed": (1 << 40) + 8}, -2),
    ({"activation": 2}, -1),
    ({"activation": -1}, -1),
    ({"activation": 1, "situ_b1": 0.0, "situ_b2": 25.0}, -1),
    ({"activation": 1, "situ_b1": 4.0, "situ_b2": -25.0}, -1),
    ({"activation": 1, "situ_b1": float("inf"), "situ_b2": 25.0}, -1),
    ({"activation": 1, "situ_b1": 4.0, "situ_b2": float("nan")}, -1),
])
def test_pool_create_refuses(k3x, kw, want):
    st, h = _create(k3x, _desc(k3x, **kw))
    assert st == want and not h
    assert k3x.k3x_last_error() != ""


def test_pool_create_refuses_small_or_misaligned_stride(k3x):
    d = _desc(k3x)
    d.stride_bytes[0] = 100  # below the dense size of w1_packed
    assert _create(k3x, d)[0] == k3x.K3X_E_INVALID_ARG
    d = _desc(k3x)
    d.stride_bytes[4] = 384 * 256 // 2 + 8  # packed stride must keep 16-byte alignment
    assert _create(k3x, d)[0] == k3x.K3X_E_UNSUPPORTED
    assert _create(k3x, _desc(k3x))[0] == k3x.K3X_OK


def test_moe_forward_host_validation(k3x):
    lib = k3x.lib()
    st, h = _create(k3x, _desc(k3x))
    assert st == 0
    try:
        need = lib.k3x_moe_workspace_size(h, 4, 16)
        assert need > 0
        assert lib.k3x_moe_workspace_size(h, 4, 65) == 0
        assert lib.k3x_moe_workspace_size(h, -1, 16) == 0
        fake = 1 << 40
        # bad topk, negative T, missing or small or misaligned workspace: no launch happens
        assert lib.k3x_moe_forward(h, fake, 4, fake, fake, 0, fake, fake, need, None) == -1
        assert lib.k3x_moe_forward(h, fake, -1, fake, fake, 16, fake, fake, need, None) == -1
        assert lib.k3x_moe_forward(h, fake, 4, fake, fake, 16, fake, None, need, None) == -3
        assert lib.k3x_moe_forward(h, fake, 4, fake, fake, 16, fake, fake, need - 1, None) == -3
        assert lib.k3x_moe_forward(h, fake, 4, fake, fake, 16, fake, fake + 8, need, None) == -3
        assert lib.k3x_moe_forward(h, None, 4, fake, fake, 16, fake, fake, need, None) == -1
        assert lib.k3x_moe_forward(h, fake + 2, 4, fake, fake, 16, fake, fake, need, None) == -2
        assert lib.k3x_moe_forward(None, fake, 4, fake, fake, 16, fake, fake, need, None) == -1
    finally:
        lib.k3x_expert_pool_destroy(h)


def test_router_host_validation(k3x):
    lib = k3x.lib()
    fake = 1 << 40
    r = k3x.k3x_router_desc()
    r.weight, r.bias, r.n_experts, r.hidden, r.topk, r.renorm, r.routed_scale = fake, None, 896, 3584, 16, 1, 1.0
    need = lib.k3x_route_workspace_size(ctypes.byref(r), 4)
    assert need >= 4 * 896 * 4
    # T = 0 is a no-op that succeeds
    assert lib.k3x_route_topk(ctypes.byref(r), fake, 0, fake, fake, fake, need, None) == 0
    assert lib.k3x_route_topk(ctypes.byref(r), fake, 4, fake, fake, fake, need - 4, None) == -3
    for field, val, want in (("topk", 0, -1), ("topk", 897, -1), ("hidden", 3583, -2),
                             ("n_experts", 5000, -1), ("weight", None, -1)):
        r2 = k3x.k3x_router_desc()
        ctypes.pointer(r2)[0] = r
        setattr(r2, field, val)
        assert lib.k3x_route_topk(ctypes.byref(r2), fake, 4, fake, fake, fake, need, None) == want
        assert lib.k3x_route_workspace_size(ctypes.byref(r2), 4) == 0


def test_norm_helpers_host_validation(k3x):
    lib = k3x.lib()
    fake = 1 << 40
    assert lib.k3x_rmsnorm_bf16(fake, 1, 3583, 1e-6, fake, None) == -2
    assert lib.k3x_rmsnorm_bf16(fake, -1, 3584, 1e-6, fake, None) == -1
    assert lib.k3x_rmsnorm_bf16(fake, 0, 3584, 1e-6, fake, None) == 0
    assert lib.k3x_residual_add_bf16(fake, fake, 1, 3583, None) == -2
    assert lib.k3x_residual_add_bf16(None, fake, 1, 3584, None) == -1
    f = ctypes.c_float(1e-6)
    fused = lib.k3x_residual_add_rmsnorm_bf16
    assert fused(fake, fake + (1 << 20), 1, 3583, f, fake + (2 << 20), None) == -2
    assert fused(fake, fake + (1 << 20), 1, 16392, f, fake + (2 << 20), None) == -2
    assert fused(fake, fake + (1 << 20), -1, 3584, f, fake + (2 << 20), None) == -1
    assert fused(fake, fake + (1 << 20), 0, 3584, f, fake + (2 << 20), None) == 0
    assert fused(None, fake + (1 << 20), 1, 3584, f, fake + (2 << 20), None) == -1
    assert fused(fake, fake + (1 << 20), 1, 3584, f, fake + 8, None) == -2  # misaligned out
    # out overlapping x (same buffer, or partly) or y is refused before any launch
    assert fused(fake, fake + (1 << 20), 1, 3584, f, fake, None) == -1
    assert fused(fake, fake + (1 << 20), 2, 3584, f, fake + 7168, None) == -1
    assert fused(fake, fake + (1 << 20), 1, 3584, f, fake + (1 << 20) + 4096, None) == -1
    assert lib.k3x_fetch_drops(None, None, None) == -1


def test_latent_block_host_validation(k3x):
    lib = k3x.lib()
    fake = 1 << 40
    st, h = _create(k3x, _desc(k3x, hidden=512))  # routed experts on a 512-wide latent
    assert st == 0
    try:
        def desc(**kw):
            d = k3x.k3x_latent_desc()
            d.hidden, d.shared_inter = 1024, 512
            d.down, d.up, d.sh1, d.sh3, d.sh2 = (fake + i * (1 << 32) for i in range(5))
            d.latent_norm, d.norm_weight, d.eps = 1, fake + (6 << 32), 1e-5
            d.shared_activation, d.situ_b1, d.situ_b2 = k3x.K3X_ACT_SITU, 4.0, 25.0
            for k, v in kw.items():
                setattr(d, k, v)
            return d

        def router(**kw):
            r = k3x.k3x_router_desc()
            r.weight, r.bias, r.n_experts, r.hidden, r.topk, r.renorm, r.routed_scale = \
                fake + (7 << 32), None, 8, 1024, 2, 1, 1.0
            for k, v in kw.items():
                setattr(r, k, v)
            return r

        def fwd(d, r, T=3, x=fake + (8 << 32), out=fake + (9 << 32), ws=fake + (10 << 32),
                nbytes=None):
            need = lib.k3x_latent_workspace_size(ctypes.byref(desc()), h, ctypes.byref(router()), T)
            return lib.k3x_latent_forward(ctypes.byref(d), h, ctypes.byref(r), x, T, out, ws,
                                          need if nbytes is None else nbytes, None)

        need = lib.k3x_latent_workspace_size(ctypes.byref(desc()), h, ctypes.byref(router()), 3)
        offs = (ctypes.c_size_t * 6)()
        assert lib.k3x_latent_ws_layout(ctypes.byref(desc()), h, ctypes.byref(router()), 3,
                                        offs) == 0
        assert all(o % 256 == 0 for o in offs) and list(offs) == sorted(offs)
        off = offs[5]
        assert need > off > 0
        # every intermediate fits before the next: idx, gates [3][2]; z [3][512] bf16;
        # acc [3][512] fp32; s [3][512] bf16
        sizes = [3 * 2 * 4, 3 * 2 * 4, 3 * 512 * 2, 3 * 512 * 4, 3 * 512 * 2]
        assert all(offs[i] + sizes[i] <= offs[i + 1] for i in range(5))
        assert lib.k3x_latent_ws_layout(ctypes.byref(desc(hidden=1000)), h,
                                        ctypes.byref(router(hidden=1000)), 3, offs) == k3x.K3X_E_UNSUPPORTED
        assert lib.k3x_latent_ws_layout(ctypes.byref(desc()), h, ctypes.byref(router()), 3,
                                        None) == k3x.K3X_E_INVALID_ARG
        assert need - off >= lib.k3x_moe_workspace_size(h, 3, 2)
        if not _gpu_present():
            # an empty call still enqueues the reset of the routed experts' drop counter; with no
            # device that launch fails (on a GPU the fake workspace must not be touched)
            assert fwd(desc(), router(), T=0) == k3x.K3X_E_HIP
        E_ARG, E_UNS, E_WS = k3x.K3X_E_INVALID_ARG, k3x.K3X_E_UNSUPPORTED, k3x.K3X_E_WORKSPACE
        cases = [
            (desc(hidden=1536), router(), E_ARG),           # router width != block width
            (desc(), router(n_experts=9, weight=fake), E_ARG),  # router experts != pool experts
            (desc(), router(topk=9), E_ARG),
            (desc(hidden=1000), router(hidden=1000), E_UNS),  # not a multiple of 512
            (desc(hidden=8704), router(hidden=8704), E_UNS),  # above 8192
            (desc(shared_inter=768), router(), E_UNS),
            (desc(shared_inter=9728), router(), E_UNS),      # L + S above 9728
            (desc(down=None), router(), E_ARG),
            (desc(sh2=None), router(), E_ARG),
            (desc(up=fake + 8), router(), E_UNS),            # misaligned weight
            (desc(norm_weight=fake + 4), router(), E_UNS),
            (desc(eps=-1.0), router(), E_ARG),
            (desc(eps=float("nan")), router(), E_ARG),
            (desc(shared_activation=2), router(), E_ARG),
            (desc(situ_b1=0.0), router(), E_ARG),
            (desc(situ_b2=float("inf")), router(), E_ARG),
        ]
        for d, r, want in cases:
            assert fwd(d, r) == want, (d.hidden, d.shared_inter, want)
            assert lib.k3x_latent_workspace_size(ctypes.byref(d), h, ctypes.byref(r), 3) == 0
        assert fwd(desc(), router(), T=-1) == E_ARG
        assert fwd(desc(), router(), nbytes=need - 1) == E_WS
        assert fwd(desc(), router(), ws=None) == E_WS
        assert fwd(desc(), router(), ws=fake + 64) == E_WS
        assert fwd(desc(), router(), x=None) == E_ARG
        assert fwd(desc(), router(), out=fake + 4) == E_UNS
        assert lib.k3x_latent_forward(None, h, ctypes.byref(router()), fake, 3, fake, fake, need,
                                      None) == E_ARG
        assert lib.k3x_latent_forward(ctypes.byref(desc()), None, ctypes.byref(router()), fake, 3,
                                      fake, fake, need, None) == E_ARG
    finally:
        lib.k3x_expert_pool_destroy(h)


def test_route_moe_host_validation(k3x):
    lib = k3x.lib()
    fake = 1 << 40
    st, h = _create(k3x, _desc(k3x))  # E 8, hidden 256
    assert st == 0
    try:
        def router(**kw):
            r = k3x.k3x_router_desc()
            r.weight, r.bias, r.n_experts, r.hidden, r.topk, r.renorm, r.routed_scale = \
                fake, None, 8, 256, 2, 1, 1.0
            for k, v in kw.items():
                setattr(r, k, v)
            return r

        R = ctypes.byref
        need = lib.k3x_route_moe_workspace_size(R(router()), h, 3)
        assert need >= lib.k3x_moe_workspace_size(h, 3, 2) + 3 * 8 * 4
        fwd = lambda r, T=3, x=fake, ws=fake, n=need: lib.k3x_route_moe_forward(
            R(r), h, x, T, fake, fake, fake, ws, n, None)
        if not _gpu_present():
            # an empty call enqueues only the reset of the drop counter: no device, a HIP error
            assert fwd(router(), T=0) == k3x.K3X_E_HIP
        assert fwd(router(n_experts=9)) == k3x.K3X_E_INVALID_ARG
        assert fwd(router(hidden=512)) == k3x.K3X_E_INVALID_ARG
        assert fwd(router(topk=9)) == k3x.K3X_E_INVALID_ARG
        assert fwd(router(), T=-1) == k3x.K3X_E_INVALID_ARG
        assert fwd(router(), n=need - 1) == k3x.K3X_E_WORKSPACE
        assert fwd(router(), ws=fake + 64) == k3x.K3X_E_WORKSPACE
        assert fwd(router(), x=None) == k3x.K3X_E_INVALID_ARG
        assert fwd(router(), x=fake + 2) == k3x.K3X_E_UNSUPPORTED
        assert lib.k3x_route_moe_workspace_size(R(router(n_experts=9)), h, 3) == 0
        assert lib.k3x_route_moe_forward(R(router()), None, fake, 3, fake, fake, fake, fake,
                                         need, None) == k3x.K3X_E_INVALID_ARG
    finally:
        lib.k3x_expert_pool_destroy(h)
    st, h = _create(k3x, _desc(k3x, n_experts=100))
    try:
        r = k3x.k3x_router_desc()
        r.weight, r.bias, r.n_experts, r.hidden, r.topk, r.renorm, r.routed_scale = \
            fake, None, 100, 256, 65, 1, 1.0
        assert lib.k3x_route_moe_forward(ctypes.byref(r), h, fake, 1, fake, fake, fake, fake,
                                         1 << 30, None) == k3x.K3X_E_UNSUPPORTED
    finally:
        lib.k3x_expert_pool_destroy(h)


def test_residual_route_moe_host_validation(k3x):
    """k3x_residual_route_moe_forward refuses bad arguments before enqueuing anything: the
    route_moe checks, NULL outputs, a missing x_next when y_prev is given, misalignment, and
    x_next or xn overlapping another operand (y may be y_prev)."""
    lib = k3x.lib()
    fake = 1 << 40
    st, h = _create(k3x, _desc(k3x))  # E 8, hidden 256
    assert st == 0
    try:
        r = k3x.k3x_router_desc()
        r.weight, r.bias, r.n_experts, r.hidden, r.topk, r.renorm, r.routed_scale = \
            fake, None, 8, 256, 2, 1, 1.0
        R = ctypes.byref
        T = 3
        need = lib.k3x_route_moe_workspace_size(R(r), h, T)
        xb, yb = T * 256 * 2, T * 256 * 4
        X, YP, XN, XNX, Y = fake, fake + (1 << 24), fake + (2 << 24), fake + (3 << 24), fake + (4 << 24)

        def fwd(x=X, y_prev=YP, x_next=XNX, xn=XN, y=Y, T=T, ws=fake + (5 << 24), n=need, rr=r):
            return lib.k3x_residual_route_moe_forward(R(rr), h, x, y_prev, 1e-6, x_next, xn, T,
                                                      fake, fake, y, ws, n, None)

        E_ARG, E_UNS, E_WS = k3x.K3X_E_INVALID_ARG, k3x.K3X_E_UNSUPPORTED, k3x.K3X_E_WORKSPACE
        assert fwd(T=-1) == E_ARG
        assert fwd(n=need - 1) == E_WS
        assert fwd(xn=None) == E_ARG
        assert fwd(x=None) == E_ARG
        assert fwd(y=None) == E_ARG
        assert fwd(x_next=None) == E_ARG            # y_prev given, nowhere to put x + y_prev
        assert fwd(x=X + 2) == E_UNS
        assert fwd(y_prev=YP + 4) == E_UNS
        assert fwd(x_next=XNX + 8) == E_UNS
        assert fwd(x_next=X + xb - 16) == E_ARG     # x_next overlaps x
        assert fwd(x_next=YP + yb - 16) == E_ARG    # x_next overlaps y_prev
        assert fwd(x_next=XN) == E_ARG              # x_next is xn
        assert fwd(xn=X + 16) == E_ARG              # xn overlaps x
        assert fwd(xn=Y + yb - 16) == E_ARG         # xn overlaps y
        bad = k3x.k3x_router_desc()
        bad.weight, bad.bias, bad.n_experts, bad.hidden, bad.topk, bad.renorm, bad.routed_scale = \
            fake, None, 9, 256, 2, 1, 1.0
        assert fwd(rr=bad) == E_ARG                 # router experts != pool experts
        if not _gpu_present():
            # accepted arguments reach the device: without one, a HIP error (y may be y_prev,
            # and without y_prev neither x_next nor its overlaps matter)
            assert fwd(y=YP) == k3x.K3X_E_HIP
            assert fwd(y_prev=None, x_next=X) == k3x.K3X_E_HIP
    finally:
        lib.k3x_expert_pool_destroy(h)


def test_contract_pool_checks(k3x):
    lib = k3x.lib()
    assert _create(k3x, _desc(k3x, contract=2))[0] == k3x.K3X_E_INVALID_ARG
    assert _create(k3x, _desc(k3x, contract=1, hidden=8192))[0] == k3x.K3X_E_UNSUPPORTED
    st, h = _create(k3x, _desc(k3x, contract=1))
    assert st == 0
    try:
        fake = 1 << 40
        # one token per call in the contract arithmetic; more is refused before any launch
        assert lib.k3x_moe_forward(h, fake, 2, fake, fake, 4, fake, fake, 1 << 30, None) == \
            k3x.K3X_E_UNSUPPORTED
        n1 = lib.k3x_moe_workspace_size(h, 1, 4)
        st0, h0 = _create(k3x, _desc(k3x))
        assert n1 >= lib.k3x_moe_workspace_size(h0, 1, 4) and n1 >= 256 + 4 * 4 * (384 + 256)
        lib.k3x_expert_pool_destroy(h0)
    finally:
        lib.k3x_expert_pool_destroy(h)


def test_status_strings(k3x):
    for s in (0, -1, -2, -3, -4, -5):
        assert k3x.k3x_status_str(s)
    assert k3x.k3x_status_str(7) == "unknown status"


def test_noalloc_host_refusals(k3x):
    """k3x_moe_forward_noalloc refuses on the host, before touching any device: a NULL pool,
    topk out of range, and a call whose workspace exceeds the built-in scratch."""
    lib = k3x.lib()
    fake = 1 << 40
    d = _desc(k3x, hidden=3584, inter=3072)
    d.n_experts = 896
    st, h = _create(k3x, d)
    assert st == 0
    try:
        f = lambda pool, T, k, drops=None: lib.k3x_moe_forward_noalloc(
            pool, fake, T, fake, fake, k, fake, drops, None)
        assert f(None, 4, 16) == k3x.K3X_E_INVALID_ARG
        assert f(h, 4, 0) == k3x.K3X_E_INVALID_ARG
        assert f(h, -1, 16) == k3x.K3X_E_INVALID_ARG
        assert lib.k3x_moe_workspace_size(h, 102, 16) <= k3x.K3X_NOALLOC_SCRATCH_BYTES
        assert lib.k3x_moe_workspace_size(h, 103, 16) > k3x.K3X_NOALLOC_SCRATCH_BYTES
        assert f(h, 103, 16) == k3x.K3X_E_UNSUPPORTED
        assert b"scratch" in lib.k3x_last_error()
        assert f(h, 4, 16, drops=fake + 4) == k3x.K3X_E_INVALID_ARG
    finally:
        lib.k3x_expert_pool_destroy(h)
