"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, sizes workspaces, computes capacities exactly, and rejects bad
arguments before any HIP call (so none of these tests touches a GPU)."""
import os
import random
import re

import pytest

import sparse_mixture_experts_order_amd as sw
from oracle.switch_oracle import capacity as oracle_capacity

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "switch_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(switch_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = sw.lib()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert sorted(sw.EXPORTS) == names


def test_library_is_built_from_the_current_sources(tmp_path):
    """The library carries the hash of the sources it was built from; a file
    with another hash (or none) is not current, and lib() would refuse it."""
    from sparse_mixture_experts_order_amd.build import source_hash
    assert sw.library_hash() == source_hash()
    assert sw.library_current()
    other = tmp_path / "lib.so"
    other.write_bytes(b"\x7fELF...switch-source-hash:" + b"0" * 32 + b"\0rest")
    assert sw.library_hash(str(other)) == "0" * 32
    assert not sw.library_current(str(other))
    none = tmp_path / "none.so"
    none.write_bytes(b"\x7fELF no tag")
    assert sw.library_hash(str(none)) is None and not sw.library_current(str(none))


def test_noalloc_dispatch_validates_before_any_hip_call():
    """The allocation-free dispatch checks its arguments and its fixed scratch
    size on the host: these return an error with nothing enqueued."""
    L = sw.lib()
    none = [None] * 6
    # 1024 tiles x 4096 experts: 16 MiB of counts
    assert L.switch_dispatch_noalloc(None, None, 1 << 18, 64, 4096, 1, *none, None) == sw.SWITCH_E_UNSUPPORTED
    assert b"scratch" in L.switch_last_error()
    assert L.switch_dispatch_noalloc(None, None, 100, 64, 4, 10, *none, None) == sw.SWITCH_E_INVALID
    assert L.switch_dispatch_noalloc(None, None, 100, 64, 0, 10, *none, None) == sw.SWITCH_E_INVALID


def test_capacity_matches_oracle():
    cases = [(512, 4, 1.25), (16384, 128, 1.0), (16384, 64, 2.0), (32768, 128, 1.25), (65536, 2048, 1.0),
             (64, 4, 1.25), (100, 10, 1.0), (30, 3, 0.1), (0, 5, 3.0), (7, 7, 0.0), (1, 4096, 1e-300),
             (2**31 - 1, 1, 1.0), (1000, 3, 1 / 3), (999, 7, 0.7)]
    rng = random.Random(0)
    for _ in range(2000):
        cases.append((rng.randrange(0, 1 << 20), rng.randrange(1, 5000), rng.choice([rng.random() * 4, rng.randrange(0, 9) / 4])))
    for T, E, c in cases:
        assert sw.switch_capacity(T, E, c) == oracle_capacity(T, E, c), (T, E, c)


@pytest.mark.parametrize("args", [(-1, 4, 1.0), (10, 0, 1.0), (10, 4, -0.5), (10, 4, float("nan")),
                                  (10, 4, float("inf")), (2**31 - 1, 1, 2.0)])
def test_capacity_rejects(args):
    with pytest.raises(sw.SwitchError) as ei:
        sw.switch_capacity(*args)
    assert ei.value.status == sw.SWITCH_E_INVALID


def test_workspace_sizes():
    assert sw.switch_workspace_bytes(16384, 768, 3072, 128, 128) >= 128 * 128 * 3072 * 2 + 128 * 128 * 768 * 6
    assert sw.switch_expert_ffn_workspace_bytes(128, 128, 3072) >= 128 * 128 * 3072 * 2
    assert sw.switch_dispatch_workspace_bytes(16384, 128) >= (16384 // 256) * 128 * 4
    # E <= 256: the fused router needs only the split weights and partial sums
    assert sw.switch_route_workspace_bytes(16384, 768, 128) >= 3 * 768 * 128 * 2
    # wider routers keep the logits in the workspace when the caller gives no logits array
    assert sw.switch_route_workspace_bytes(65536, 1024, 2048) >= 3 * 1024 * 2048 * 2 + 65536 * 2048 * 4
    assert sw.switch_aux_loss_workspace_bytes(10, 4) == 0
    assert sw.switch_workspace_bytes(10, 64, 64, 0, 1) == 0      # E = 0 is invalid
    assert sw.switch_workspace_bytes(10, 64, 64, 5000, 1) == 0   # E above the limit


def test_first_gemm_token_tile():
    """The first expert GEMM's token-tile height (no device work; without a
    GPU the library counts 256 compute units, the MI355X's): 32/64/128 rows by
    the buffer rows, 320-row tall tiles where experts are expected to fill
    more than 128 rows and E * ceil(d_ff / 256) >= 4 * 256 tiles."""
    f = sw.switch_ffn_gemm1_token_tile
    assert f(128, 128, 16384, 3072) == 128                # Switch-Base shape: 128 rows fill
    assert f(128, 320, 32768, 4096) == 320                # Switch-Large shape: 256 rows fill, 2048 tiles
    assert f(64, 512, 16384, 3072) == 128                 # congested: 768 tiles, under four per CU
    assert f(2048, 32, 65536, 1024) == 32                 # many small experts
    assert f(100, 61, 0, 512) == 64
    assert f(128, 256, 16384 * 2, 3072) == 320            # top-2 at the Switch-Base shape
    assert f(128, 16384 // 64 * 1, 16384, 3072) == 128    # routing groups: 256 rows, 128 filled
    assert f(64, 200, 12800, 4096) == 320                 # the parity tests' tall edge shapes
    assert f(64, 500, 16000, 4096) == 320
    assert f(64, 325, 20800, 4032) == 320
    assert f(64, 200, 12800, 4032 - 256 * 16) == 0        # d_ff <= 0
    assert f(0, 128, 100, 256) == 0 and f(4, 0, 100, 256) == 0
    assert f(64, 200, 0, 4096) == 320                     # fill unknown: the buffer rows count


def _status(fn, *a):
    with pytest.raises(sw.SwitchError) as ei:
        fn(*a)
    return ei.value.status


FAKE = 1 << 20   # an aligned non-NULL address; never dereferenced because validation fails first


def test_route_validation():
    L = sw.lib()
    st = L.switch_route(None, FAKE, None, None, 16, 64, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_INVALID and b"x" in L.switch_last_error()
    st = L.switch_route(FAKE, FAKE, None, None, 16, 48, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_UNSUPPORTED
    st = L.switch_route(FAKE, FAKE, None, None, 16, 64, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_INVALID
    st = L.switch_route(FAKE, FAKE, None, None, 16, 64, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None)
    assert st == sw.SWITCH_E_WORKSPACE
    st = L.switch_route(FAKE + 2, FAKE, None, None, 16, 64, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_INVALID and b"aligned" in L.switch_last_error()
    st = L.switch_route(FAKE, FAKE, None, None, -1, 64, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_INVALID
    st = L.switch_route(FAKE, FAKE, None, None, 16, 64, 5000, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == sw.SWITCH_E_UNSUPPORTED


def test_dispatch_validation():
    L = sw.lib()
    ok = dict(x=FAKE, e=FAKE, T=16, d=64, E=4, C=4, pos=FAKE, keep=FAKE, cnt=FAKE, acc=FAKE, st=None, buf=FAKE,
              ws=FAKE, wsn=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.switch_dispatch(a["x"], a["e"], a["T"], a["d"], a["E"], a["C"], a["pos"], a["keep"], a["cnt"],
                                 a["acc"], a["st"], a["buf"], a["ws"], a["wsn"], None)
    assert call(C=-1) == sw.SWITCH_E_INVALID
    assert call(x=None) == sw.SWITCH_E_INVALID
    assert call(buf=None) == sw.SWITCH_E_INVALID
    assert call(d=12) == sw.SWITCH_E_UNSUPPORTED
    assert call(wsn=0) == sw.SWITCH_E_WORKSPACE
    assert call(E=1 << 16, C=1 << 16) == sw.SWITCH_E_UNSUPPORTED
    assert call(ws=FAKE + 64) == sw.SWITCH_E_INVALID


def test_ffn_combine_aux_validation():
    L = sw.lib()
    assert L.switch_expert_ffn(FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 128, FAKE, FAKE, 1 << 30, None) == sw.SWITCH_E_UNSUPPORTED
    assert L.switch_expert_ffn(FAKE, FAKE, None, FAKE, 4, 8, 64, 128, FAKE, FAKE, 1 << 30, None) == sw.SWITCH_E_INVALID
    assert L.switch_expert_ffn(FAKE, FAKE, FAKE, FAKE, 4, 8, 64, 128, FAKE, FAKE, 64, None) == sw.SWITCH_E_WORKSPACE
    assert L.switch_combine(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 4, 4, FAKE, None) == sw.SWITCH_E_INVALID  # alias
    assert L.switch_combine(FAKE, None, FAKE, FAKE, FAKE, None, 16, 64, 4, 4, FAKE, None) == sw.SWITCH_E_INVALID
    assert L.switch_aux_loss(FAKE, FAKE, None, None, 16, 4, float("nan"), FAKE, FAKE, FAKE, None, None, 0, None) == sw.SWITCH_E_INVALID
    assert L.switch_aux_loss(FAKE, FAKE, None, FAKE, 16, 4, 0.01, FAKE, FAKE, FAKE, FAKE, None, 0, None) == sw.SWITCH_E_INVALID
    assert L.switch_stream_copy(FAKE, FAKE, 15, None) == sw.SWITCH_E_INVALID


def test_layer_validation():
    L = sw.lib()
    a = sw.LayerArgs()
    a.T, a.d, a.d_ff, a.E, a.C, a.alpha, a.residual = 16, 64, 128, 4, 8, 0.01, 1
    assert L.switch_layer_fwd(None, FAKE, 1 << 30, None) == sw.SWITCH_E_INVALID
    import ctypes
    assert L.switch_layer_fwd(ctypes.byref(a), FAKE, 1 << 30, None) == sw.SWITCH_E_INVALID   # NULL pointers
    a.d = 96
    assert L.switch_layer_fwd(ctypes.byref(a), FAKE, 1 << 30, None) == sw.SWITCH_E_UNSUPPORTED
    a.d = 64
    assert L.switch_layer_fwd(ctypes.byref(a), FAKE, 16, None) == sw.SWITCH_E_WORKSPACE


def test_status_strings():
    L = sw.lib()
    for s in range(5):
        assert L.switch_status_string(s)
    assert L.switch_kernel_name(7) == b"expert_gemm1"


def test_group_topk_validation():
    """Routing groups and top-k: k in [1, min(E, 4)], T a multiple of the
    group size, group sizes that are multiples of 64, priority 0 or 1."""
    L = sw.lib()
    ok = dict(x=FAKE, e=FAKE, T=256, d=64, E=4, k=2, G=128, C=64, pr=0, pos=FAKE, keep=FAKE, slot=FAKE, cnt=FAKE,
              acc=FAKE, tot=FAKE, st=None, buf=FAKE, ws=FAKE, wsn=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.switch_dispatch_ex(a["x"], a["e"], a["T"], a["d"], a["E"], a["k"], a["G"], a["C"], a["pr"],
                                    a["pos"], a["keep"], a["slot"], a["cnt"], a["acc"], a["tot"], a["st"], a["buf"],
                                    a["ws"], a["wsn"], None)
    assert call(k=0) == sw.SWITCH_E_INVALID
    assert call(k=5, E=8) == sw.SWITCH_E_UNSUPPORTED
    assert call(k=5) == sw.SWITCH_E_INVALID                 # k > E
    assert call(G=96) == sw.SWITCH_E_INVALID                # 256 % 96 != 0
    assert call(T=96, G=32) == sw.SWITCH_E_UNSUPPORTED      # 32 is not a multiple of 64
    assert call(pr=2) == sw.SWITCH_E_INVALID
    assert call(G=-1) == sw.SWITCH_E_INVALID
    assert call(tot=None) == sw.SWITCH_E_INVALID            # several groups need accepted_total
    assert call(slot=None) == sw.SWITCH_E_INVALID
    assert call(wsn=0) == sw.SWITCH_E_WORKSPACE
    # one group (group = 0 or T) needs neither slot nor accepted_total; the
    # failure left is the workspace, reached only after every other check
    assert call(G=0, slot=None, tot=None, wsn=0) == sw.SWITCH_E_WORKSPACE
    assert call(G=256, slot=None, tot=None, wsn=0) == sw.SWITCH_E_WORKSPACE
    st = L.switch_route_ex(FAKE, FAKE, None, None, 256, 64, 4, 3, 96, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                           None)
    assert st == sw.SWITCH_E_INVALID
    st = L.switch_aux_loss_ex(FAKE, FAKE, None, None, 256, 4, 5, 64, 0.01, FAKE, FAKE, FAKE, None, None)
    assert st == sw.SWITCH_E_INVALID
    assert L.switch_combine_ex(FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 64, 4, 0, 4, FAKE, None) == sw.SWITCH_E_INVALID


def test_group_topk_workspace_sizes():
    # one group and k = 1 give the Switch layer's sizes exactly
    for T, d, F, E, C in [(16384, 768, 3072, 128, 128), (512, 64, 128, 4, 160), (65536, 1024, 1024, 2048, 32)]:
        assert sw.switch_workspace_bytes_ex(T, d, F, E, C, 1, 0) == sw.switch_workspace_bytes(T, d, F, E, C)
        assert sw.switch_workspace_bytes_ex(T, d, F, E, C, 1, T) == sw.switch_workspace_bytes(T, d, F, E, C)
        assert sw.switch_dispatch_workspace_bytes_ex(T, E, 1, 0) == sw.switch_dispatch_workspace_bytes(T, E)
    # groups of 64 with top-2: scan tiles of 128 choices, per-group bases, rows = groups * C
    T, E, G, k = 16384, 128, 64, 2
    ng = T // G
    assert sw.switch_dispatch_workspace_bytes_ex(T, E, k, G) >= (T * k // 128) * E * 4 + ng * E * 4 + E * 4
    C = sw.switch_capacity(k * G, E, 1.0)
    assert C == 1
    assert sw.switch_workspace_bytes_ex(T, 768, 3072, E, C, k, G) >= E * ng * C * 768 * 6 + T * k * 4
    assert sw.switch_workspace_bytes_ex(T, 768, 3072, E, C, k, 100) == 0     # T % 100 != 0
    assert sw.switch_workspace_bytes_ex(T, 768, 3072, E, C, 5, G) == 0       # k above the limit
