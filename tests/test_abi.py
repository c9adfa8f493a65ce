"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments before touching a device. No kernel runs here: every
forward call below carries an argument the host checks refuse."""

import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infini_attn.h")


@pytest.fixture(scope="module")
def lib():
    from compressive_memory_transformers_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from compressive_memory_transformers_amd import build
        build.build()
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(infini_attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "infini_attn_backward", "infini_attn_backward_workspace_size",
        "infini_attn_block_forward", "infini_attn_block_forward_timed",
        "infini_attn_block_workspace_size", "infini_attn_block_forward_kv",
        "infini_attn_block_workspace_size_kv", "infini_attn_decode_step", "infini_attn_error_string",
        "infini_attn_decode_workspace_size", "infini_attn_decode_step_kv",
        "infini_attn_decode_workspace_size_kv",
        "infini_attn_forward", "infini_attn_forward_kv", "infini_attn_forward_kv_timed",
        "infini_attn_forward_noalloc", "infini_attn_forward_timed",
        "infini_attn_forward_train", "infini_attn_forward_train_kv",
        "infini_attn_backward_kv", "infini_attn_backward_workspace_size_kv", "infini_attn_status_string", "infini_attn_version",
        "infini_attn_workspace_size", "infini_attn_workspace_size_kv"])


def test_library_exports_every_declared_symbol(lib):
    from compressive_memory_transformers_amd import binding
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.SIGNATURES
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                        capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", nm, flags=re.M))
    assert set(declared_functions()) <= exported


def test_library_is_built_for_gfx950(lib):
    from compressive_memory_transformers_amd import binding
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_version_and_status_strings(lib):
    assert lib.infini_attn_version() == 100
    names = {s: lib.infini_attn_status_string(s).decode() for s in range(7)}
    assert names[0] == "ok" and names[4] == "workspace too small"
    assert names[6] == "unknown status"
    assert lib.infini_attn_status_string(-3).decode() == "unknown status"
    for st in range(-1, 8):  # the second name is the same function
        assert lib.infini_attn_error_string(st) == lib.infini_attn_status_string(st)


def ws(lib, *args):
    full, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.infini_attn_workspace_size(*args, ctypes.byref(full), ctypes.byref(least))
    return st, full.value, least.value


def _al(n):
    return (n + 255) // 256 * 256


def overlap_extra(units, dk, dv, e):
    """Bytes the full size adds beyond the per-segment data when there are
    several segments: the head slot (one snapshot per unit, M^T in the element
    type and z in float, each aligned to 256 bytes) and the alignment slack
    of the second region's five sub-buffers."""
    return _al(units * dk * dv * e) + _al(units * dk * 4) + 5 * 256


def test_workspace_sizes(lib):
    # Llama-3-8B-shaped, bf16, delta rule: seg_len >= d, so the scan runs in
    # affine form. Per segment and unit: snapshots (d*d bf16 + d floats),
    # column sums (d floats), B_s (d*d floats) and A_s (d*d bf16).
    st, full, least = ws(lib, 4, 32, 8, 32768, 128, 2048, 1, 1)
    assert st == 0
    d = 128
    per_seg = 32 * (d * d * 2 + d * 4 + d * 4 + d * d * 4 + d * d * 2)
    assert full - least == 15 * per_seg + overlap_extra(32, d, d, 2)
    assert least >= per_seg + 2 * 32 * (d * d + d) * 4
    # the linear rule needs no A_s
    st, full_lin, least_lin = ws(lib, 4, 32, 8, 32768, 128, 2048, 0, 1)
    assert full - full_lin == 16 * 32 * d * d * 2
    # direct scan (seg_len < d): snapshots only
    st, full_dir, least_dir = ws(lib, 16, 32, 32, 32768, 128, 64, 1, 1)
    assert full_dir - least_dir == 511 * 512 * (d * d * 2 + d * 4) + overlap_extra(512, d, d, 2)
    # from seg_len = d on, the affine form's matrices too
    st, full_aff, least_aff = ws(lib, 16, 32, 32, 32768, 128, 128, 1, 1)
    assert full_aff - least_aff == (255 * 512 * (d * d * 2 + d * 4 + d * 4 + d * d * 4 + d * d * 2)
                                    + overlap_extra(512, d, d, 2))
    st, full32, _ = ws(lib, 4, 32, 8, 32768, 128, 2048, 1, 0)
    assert st == 0 and full32 > full
    # a ragged final segment counts as a segment
    st, a, _ = ws(lib, 1, 1, 1, 100, 32, 30, 0, 0)
    st, b, _ = ws(lib, 1, 1, 1, 120, 32, 30, 0, 0)
    assert a == b


def ws_kv(lib, *args):
    full, least = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.infini_attn_workspace_size_kv(*args, ctypes.byref(full), ctypes.byref(least))
    return st, full.value, least.value


def test_workspace_sizes_with_separate_key_and_value_widths(lib):
    # d_key = d_value: the square call's sizes, affine form included
    for args in [(4, 32, 8, 32768, 128, 2048, 1, 1), (2, 4, 2, 64, 32, 16, 0, 0)]:
        B, Hq, Hkv, L, d, N, rule, dt = args
        assert ws_kv(lib, B, Hq, Hkv, L, d, d, N, rule, dt) == ws(lib, *args)
    # d_key != d_value: the direct scan's snapshots only, M^T [dv][dk] in the
    # element type and z [dk] in float, per (unit, segment)
    for dk, dv, e, dt in [(64, 128, 2, 1), (128, 32, 4, 0), (32, 64, 2, 1)]:
        st, full, least = ws_kv(lib, 2, 8, 2, 1000, dk, dv, 300, 1, dt)
        assert st == 0
        per_seg = 2 * 2 * (dv * dk * e + dk * 4)
        # 4 segments, the last one ragged
        assert full - least == 3 * per_seg + overlap_extra(4, dk, dv, e)
        assert least >= per_seg + 2 * 4 * (dk * dv + dk) * 4


@pytest.mark.parametrize("dk,dv,status", [(64, 48, 2), (96, 64, 2), (64, 256, 2), (0, 64, 1),
                                          (64, 0, 1)])
def test_workspace_size_kv_rejects(lib, dk, dv, status):
    assert ws_kv(lib, 1, 2, 2, 64, dk, dv, 16, 0, 1)[0] == status


def test_forward_kv_rejects_before_any_launch(lib):
    # sizes of q, k (d_key 64) and v, out (d_value 128) in bf16
    B, Hq, Hkv, L, dk, dv = 1, 2, 1, 64, 64, 128
    sizes = dict(q=B * Hq * L * dk * 2, k=B * Hkv * L * dk * 2, v=B * Hkv * L * dv * 2,
                 beta=Hq * 4, M0=B * Hkv * dk * dv * 4, z0=B * Hkv * dk * 4,
                 out=B * Hq * L * dv * 2, M_final=B * Hkv * dk * dv * 4, z_final=B * Hkv * dk * 4,
                 workspace=1 << 40)
    addr, base = {}, 1 << 44
    for name, n in sizes.items():
        addr[name] = base
        base += (n + 4095) // 4096 * 4096 + 4096

    def call(dk_=dk, dv_=dv, wsb=1 << 40, **over):
        a = {**addr, **over}
        return lib.infini_attn_forward_kv(
            B, Hq, Hkv, L, dk_, dv_, 16, 1, 1,
            *[ctypes.c_void_p(a[n]) for n in ("q", "k", "v", "beta", "M0", "z0", "out",
                                               "M_final", "z_final", "workspace")], wsb, None)
    assert call(dv_=48) == 2
    assert call(dk_=96) == 2
    assert call(q=None) == 1
    assert call(v=addr["v"] + 8) == 3
    # out is [B,Hq,L,dv]: its last bytes reach past a q-sized buffer
    assert call(out=addr["v"] + sizes["v"] - 64) == 1
    assert call(M_final=addr["z0"]) == 1
    _, _, least = ws_kv(lib, B, Hq, Hkv, L, dk, dv, 16, 1, 1)
    assert call(wsb=least - 1) == 4


def test_decode_kv_sizes_and_rejections(lib):
    """The decode step with separate widths: the workspace holds the chunk
    partials (d_value + 2 floats per head and chunk) and a one-segment fold
    plan; bad widths and overlaps are refused before any launch."""
    def dws(*args):
        n = ctypes.c_size_t(0)
        return lib.infini_attn_decode_workspace_size_kv(*args, ctypes.byref(n)), n.value
    st, same = dws(1, 4, 2, 64, 64, 256, 1, 1)
    n2 = ctypes.c_size_t(0)
    assert st == 0 and lib.infini_attn_decode_workspace_size(1, 4, 2, 64, 256, 1, 1,
                                                             ctypes.byref(n2)) == 0
    assert same == n2.value  # d_key == d_value: the square call's size
    st, wide = dws(1, 4, 2, 64, 128, 256, 1, 1)
    assert st == 0 and wide > same
    assert dws(1, 4, 2, 64, 48, 256, 1, 1)[0] == 2
    assert dws(1, 4, 2, 64, 0, 256, 1, 1)[0] == 1
    # q, k: d_key 64; v, caches of v, out: d_value 128 (bf16)
    B, Hq, Hkv, dk, dv, N = 1, 4, 2, 64, 128, 256
    sizes = dict(q=B * Hq * dk * 2, k=B * Hkv * dk * 2, v=B * Hkv * dv * 2, beta=Hq * 4,
                 k_cache=B * Hkv * N * dk * 2, v_cache=B * Hkv * N * dv * 2,
                 M=B * Hkv * dk * dv * 4, z=B * Hkv * dk * 4, out=B * Hq * dv * 2,
                 workspace=1 << 30)
    addr, base = {}, 1 << 44
    for name, n in sizes.items():
        addr[name] = base
        base += (n + 4095) // 4096 * 4096 + 4096

    def call(pos=0, dv_=dv, **over):
        a = {**addr, **over}
        return lib.infini_attn_decode_step_kv(
            B, Hq, Hkv, dk, dv_, N, pos, 1, 1,
            *[ctypes.c_void_p(a[n]) for n in ("q", "k", "v", "beta", "k_cache", "v_cache", "M",
                                               "z", "out", "workspace")], 1 << 30, None)
    assert call(pos=N) == 1
    assert call(dv_=96) == 2
    assert call(out=None) == 1
    assert call(v_cache=addr["v_cache"] + 8) == 3
    # the value cache is d_value wide: a k_cache-sized buffer after it would overlap
    assert call(M=addr["v_cache"] + sizes["v_cache"] - 256) == 1


@pytest.mark.parametrize("args,status", [
    ((0, 1, 1, 8, 32, 4, 0, 0), 1),     # B < 1
    ((1, 3, 2, 8, 32, 4, 0, 0), 1),     # Hq % Hkv
    ((1, 1, 1, 0, 32, 4, 0, 0), 1),     # L < 1
    ((1, 1, 1, 8, 32, 0, 0, 0), 1),     # seg_len < 1
    ((1, 1, 1, 8, 32, 4, 2, 0), 1),     # bad rule
    ((1, 1, 1, 8, 32, 4, 0, 5), 1),     # bad dtype
    ((1, 1, 1, 8, 48, 4, 0, 0), 2),     # d unsupported
    ((1, 1, 1, 8, 256, 4, 0, 0), 2),
    ((1 << 20, 1 << 20, 1, 1 << 20, 128, 4, 0, 1), 1),  # element count overflow
])
def test_workspace_size_rejects(lib, args, status):
    assert ws(lib, *args)[0] == status


class FakeBuffers:
    """Distinct, aligned, never-dereferenced addresses sized like real buffers."""

    def __init__(self, B, Hq, Hkv, L, d, e):
        sizes = dict(q=B * Hq * L * d * e, k=B * Hkv * L * d * e, v=B * Hkv * L * d * e,
                     beta=Hq * 4, M0=B * Hkv * d * d * 4, z0=B * Hkv * d * 4,
                     out=B * Hq * L * d * e, M_final=B * Hkv * d * d * 4, z_final=B * Hkv * d * 4,
                     workspace=1 << 40)
        base = 1 << 44
        self.addr, self.size = {}, sizes
        for name, n in sizes.items():
            self.addr[name] = base
            base += (n + 4095) // 4096 * 4096 + 4096


def call(lib, shape, bufs, **over):
    B, Hq, Hkv, L, d, N, rule, dt = shape
    a = {**bufs.addr, **over}
    wsb = over.get("workspace_bytes", bufs.size["workspace"])
    return lib.infini_attn_forward(
        B, Hq, Hkv, L, d, N, rule, dt,
        *[ctypes.c_void_p(a[n]) for n in ("q", "k", "v", "beta", "M0", "z0", "out", "M_final",
                                           "z_final", "workspace")],
        wsb, None)


SHAPE = (2, 4, 2, 64, 32, 16, 1, 1)


def test_forward_rejects_bad_sizes(lib):
    bufs = FakeBuffers(2, 4, 2, 64, 32, 2)
    assert call(lib, (2, 3, 2, 64, 32, 16, 1, 1), bufs) == 1
    assert call(lib, (2, 4, 2, 64, 40, 16, 1, 1), bufs) == 2
    assert call(lib, (2, 4, 2, 64, 32, 16, 7, 1), bufs) == 1
    assert call(lib, (2, 4, 2, 64, 32, 16, 1, 9), bufs) == 1


@pytest.mark.parametrize("name", ["q", "k", "v", "beta", "M0", "z0", "out", "M_final", "z_final",
                                  "workspace"])
def test_forward_rejects_null_and_misaligned(lib, name):
    bufs = FakeBuffers(2, 4, 2, 64, 32, 2)
    assert call(lib, SHAPE, bufs, **{name: None}) == 1
    assert call(lib, SHAPE, bufs, **{name: bufs.addr[name] + 8}) == 3


def test_forward_rejects_overlaps(lib):
    bufs = FakeBuffers(2, 4, 2, 64, 32, 2)
    a = bufs.addr
    assert call(lib, SHAPE, bufs, out=a["q"]) == 1
    assert call(lib, SHAPE, bufs, out=a["k"] + 256) == 1
    assert call(lib, SHAPE, bufs, M_final=a["z0"]) == 1
    assert call(lib, SHAPE, bufs, z_final=a["M0"] + 16) == 1
    assert call(lib, SHAPE, bufs, M_final=a["M0"] + 16) == 1    # partial overlap
    assert call(lib, SHAPE, bufs, workspace=a["v"]) == 1
    assert call(lib, SHAPE, bufs, M_final=a["out"]) == 1


def test_forward_rejects_small_workspace(lib):
    bufs = FakeBuffers(2, 4, 2, 64, 32, 2)
    _, full, least = ws(lib, 2, 4, 2, 64, 32, 16, 1, 1)
    assert call(lib, SHAPE, bufs, workspace_bytes=least - 1) == 4
    assert call(lib, SHAPE, bufs, workspace_bytes=0) == 4


def test_forward_noalloc_rejects_on_the_host(lib):
    """The scratch-array forward checks sizes like infini_attn_forward and
    refuses a call whose minimum workspace exceeds the array (64 MiB) before
    it looks up the array or touches a device."""
    def noalloc(shape):
        B, Hq, Hkv, L, d, N, rule, dt = shape
        bufs = FakeBuffers(B, Hq, Hkv, L, d, 2)
        return lib.infini_attn_forward_noalloc(
            B, Hq, Hkv, L, d, N, rule, dt,
            *[ctypes.c_void_p(bufs.addr[n]) for n in ("q", "k", "v", "beta", "M0", "z0", "out",
                                                       "M_final", "z_final")], None)
    assert noalloc((2, 3, 2, 64, 32, 16, 1, 1)) == 1    # Hq % Hkv
    assert noalloc((2, 4, 2, 64, 40, 16, 1, 1)) == 2    # d unsupported
    assert noalloc((2, 4, 2, 64, 32, 16, 1, 9)) == 1    # bad dtype
    big = (64, 64, 64, 64, 128, 16, 1, 1)                # 4096 units: two states alone > 64 MiB
    _, _, least = ws(lib, *big)
    assert least > 64 << 20
    assert noalloc(big) == 4


def test_binding_validates_before_the_library():
    import compressive_memory_transformers_amd as m
    x = torch.zeros(1, 2, 8, 32)
    with pytest.raises(ValueError):
        m.forward(x, x[:, :1], x, torch.zeros(2), torch.zeros(1, 1, 32, 32),
                  torch.ones(1, 1, 32), 4, "linear")
    with pytest.raises(ValueError):
        m.forward(x, x, x, torch.zeros(2), torch.zeros(1, 2, 32, 32), torch.ones(1, 2, 32),
                  4, "hebbian")
    with pytest.raises(ValueError):  # host tensors are refused: no CPU path exists
        m.forward(x, x, x, torch.zeros(2), torch.zeros(1, 2, 32, 32), torch.ones(1, 2, 32),
                  4, "linear")


def test_missing_library_fails_loudly(tmp_path):
    env = dict(os.environ, INFINI_ATTN_LIB=str(tmp_path / "absent.so"))
    res = subprocess.run([sys.executable, "-c", "import compressive_memory_transformers_amd"],
                         cwd=ROOT, env=env, capture_output=True, text=True)
    assert res.returncode != 0
    assert "is not built" in res.stderr


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "compressive_memory_transformers_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f


# ---- streaming decode ----------------------------------------------------------

def dws(lib, *args):
    n = ctypes.c_size_t(0)
    st = lib.infini_attn_decode_workspace_size(*args, ctypes.byref(n))
    return st, n.value


def test_decode_workspace_size(lib):
    # Llama-3-8B-shaped: 32 units, 32 chunks of 64 rows, 4 query heads a unit,
    # the retrieval's numerators and denominators of the group's heads, plus
    # the one-segment recurrence workspace of the forward
    st, n = dws(lib, 4, 32, 8, 128, 2048, 1, 1)
    assert st == 0
    _, _, fold = ws(lib, 4, 32, 8, 2048, 128, 2048, 1, 1)
    up = lambda x: (x + 255) // 256 * 256
    part = 32 * 32 * 4 * (128 + 2) * 4
    retr, rden = 32 * 4 * 128 * 4, 32 * 4 * 4
    assert n == up(part) + up(retr) + up(rden) + fold


@pytest.mark.parametrize("args,status", [
    ((0, 1, 1, 32, 16, 0, 0), 1),        # B < 1
    ((1, 3, 2, 32, 16, 0, 0), 1),        # Hq % Hkv
    ((1, 1, 1, 32, 0, 0, 0), 1),         # seg_len < 1
    ((1, 1, 1, 48, 16, 0, 0), 2),        # d unsupported
    ((1, 17, 1, 32, 16, 0, 0), 2),       # more than 16 query heads per KV head
    ((1, 1, 1, 32, 16385, 0, 0), 2),     # segment longer than 256 chunks of 64
    ((1, 1, 1, 32, 16, 2, 0), 1),        # bad rule
])
def test_decode_workspace_size_rejects(lib, args, status):
    assert dws(lib, *args)[0] == status


class FakeDecodeBuffers:
    def __init__(self, B, Hq, Hkv, d, N, e):
        sizes = dict(q=B * Hq * d * e, k=B * Hkv * d * e, v=B * Hkv * d * e, beta=Hq * 4,
                     k_cache=B * Hkv * N * d * e, v_cache=B * Hkv * N * d * e,
                     M=B * Hkv * d * d * 4, z=B * Hkv * d * 4, out=B * Hq * d * e,
                     workspace=1 << 40)
        base = 1 << 44
        self.addr, self.size = {}, sizes
        for name, n in sizes.items():
            self.addr[name] = base
            base += (n + 4095) // 4096 * 4096 + 4096


def dcall(lib, shape, pos, bufs, **over):
    B, Hq, Hkv, d, N, rule, dt = shape
    a = {**bufs.addr, **over}
    wsb = over.get("workspace_bytes", bufs.size["workspace"])
    return lib.infini_attn_decode_step(
        B, Hq, Hkv, d, N, pos, rule, dt,
        *[ctypes.c_void_p(a[n]) for n in ("q", "k", "v", "beta", "k_cache", "v_cache", "M", "z",
                                           "out", "workspace")],
        wsb, None)


DSHAPE = (2, 4, 2, 64, 40, 1, 1)


@pytest.mark.parametrize("pos", [-1, 40, 1000])
def test_decode_rejects_positions_outside_the_segment(lib, pos):
    assert dcall(lib, DSHAPE, pos, FakeDecodeBuffers(2, 4, 2, 64, 40, 2)) == 1


@pytest.mark.parametrize("name", ["q", "k", "v", "beta", "k_cache", "v_cache", "M", "z", "out",
                                  "workspace"])
def test_decode_rejects_null_and_misaligned_pointers(lib, name):
    bufs = FakeDecodeBuffers(2, 4, 2, 64, 40, 2)
    assert dcall(lib, DSHAPE, 3, bufs, **{name: 0}) == 1
    assert dcall(lib, DSHAPE, 3, bufs, **{name: bufs.addr[name] + 8}) == 3


@pytest.mark.parametrize("a,b", [("out", "q"), ("k_cache", "v_cache"), ("k_cache", "k"),
                                 ("M", "z"), ("workspace", "M"), ("v_cache", "out")])
def test_decode_rejects_overlaps(lib, a, b):
    bufs = FakeDecodeBuffers(2, 4, 2, 64, 40, 2)
    assert dcall(lib, DSHAPE, 3, bufs, **{a: bufs.addr[b]}) == 1


def test_decode_rejects_small_workspace(lib):
    bufs = FakeDecodeBuffers(2, 4, 2, 64, 40, 2)
    _, need = dws(lib, 2, 4, 2, 64, 40, 1, 1)
    assert dcall(lib, DSHAPE, 3, bufs, workspace_bytes=need - 1) == 4


# ---- training forward and backward ---------------------------------------------

def test_forward_train_rejects_bad_lse(lib):
    bufs = FakeBuffers(2, 4, 2, 64, 32, 2)
    a = bufs.addr
    lse = (1 << 43)  # a distinct aligned address
    args = lambda lse_addr, **over: [2, 4, 2, 64, 32, 16, 1, 1] + [
        ctypes.c_void_p({**a, **over}[n]) for n in ("q", "k", "v", "beta", "M0", "z0", "out",
                                                    "M_final", "z_final")] + [
        ctypes.c_void_p(lse_addr), ctypes.c_void_p(a["workspace"]),
        over.get("workspace_bytes", bufs.size["workspace"]), None]
    assert lib.infini_attn_forward_train(*args(None)) == 1
    assert lib.infini_attn_forward_train(*args(lse + 4)) == 3
    assert lib.infini_attn_forward_train(*args(a["out"])) == 1     # overlaps out
    assert lib.infini_attn_forward_train(*args(a["k"] + 64)) == 1  # overlaps an input
    assert lib.infini_attn_forward_train(*args(lse, workspace_bytes=0)) == 4


def bws(lib, *args):
    n = ctypes.c_size_t(0)
    st = lib.infini_attn_backward_workspace_size(*args, ctypes.byref(n))
    return st, n.value


def test_backward_workspace_size(lib):
    st, n = bws(lib, 2, 4, 2, 64, 32, 16, 1, 1)
    assert st == 0
    units, S, d, e, L = 4, 4, 32, 2, 64
    # at least the float gradient accumulators and the per-segment matrices
    assert n > 2 * 4 * L * d * 4 + 3 * units * S * d * d * e
    assert bws(lib, 2, 3, 2, 64, 32, 16, 1, 1)[0] == 1
    assert bws(lib, 2, 4, 2, 64, 48, 16, 1, 1)[0] == 2
    # the linear rule needs no delta-rule buffers
    assert bws(lib, 2, 4, 2, 64, 32, 16, 0, 1)[1] < n


def test_backward_workspace_of_the_fused_path(lib):
    """bf16 with d = 64 and at most 64 query heads per KV head runs the fused
    kernels, which keep sigma(Q) M, sigma(K) dM_s and sigma(K) M_{s-1} in
    registers: the workspace drops the float row buffers the product path
    needs. With 65 query heads per KV head the same shape takes them again."""
    B, L, d, N = 1, 64, 64, 16
    for rule in (0, 1):
        fused = bws(lib, B, 64, 1, L, d, N, rule, 1)
        product = bws(lib, B, 65, 1, L, d, N, rule, 1)
        assert fused[0] == 0 and product[0] == 0
        qrows, krows = B * 64 * L, B * L
        # at least nm (float) and du_buf (float); for delta also p_buf (float)
        # and u_el, dp_el (bf16); one more query head only adds to the rest
        saved = qrows * d * 4 + krows * d * 4 + (krows * d * (4 + 2 + 2) if rule else 0)
        assert product[1] - fused[1] >= saved, (rule, fused, product)


BWD_NAMES = ("q", "k", "v", "beta", "M0", "z0", "out", "lse", "d_out", "dM_final", "dz_final",
             "dq", "dk", "dv", "dbeta", "dM0", "dz0", "workspace")


class FakeBwdBuffers:
    def __init__(self, B, Hq, Hkv, L, d, e):
        q, kv, M, z = B * Hq * L * d * e, B * Hkv * L * d * e, B * Hkv * d * d * 4, B * Hkv * d * 4
        sizes = dict(q=q, k=kv, v=kv, beta=Hq * 4, M0=M, z0=z, out=q, lse=B * Hq * L * 4, d_out=q,
                     dM_final=M, dz_final=z, dq=q, dk=kv, dv=kv, dbeta=Hq * 4, dM0=M, dz0=z,
                     workspace=1 << 40)
        base = 1 << 44
        self.addr, self.size = {}, sizes
        for name in BWD_NAMES:
            self.addr[name] = base
            base += (sizes[name] + 4095) // 4096 * 4096 + 4096


def bcall(lib, bufs, **over):
    a = {**bufs.addr, **over}
    wsb = over.get("workspace_bytes", bufs.size["workspace"])
    return lib.infini_attn_backward(2, 4, 2, 64, 32, 16, 1, 1,
                                    *[ctypes.c_void_p(a[n]) for n in BWD_NAMES], wsb, None)


def test_backward_accepts_null_final_gradients_then_checks_the_workspace(lib):
    bufs = FakeBwdBuffers(2, 4, 2, 64, 32, 2)
    # dM_final / dz_final may be NULL; the call still fails on the workspace
    # size, so nothing launches
    assert bcall(lib, bufs, dM_final=None, dz_final=None, workspace_bytes=16) == 4


@pytest.mark.parametrize("name", [n for n in BWD_NAMES if n not in ("dM_final", "dz_final")])
def test_backward_rejects_null_and_misaligned(lib, name):
    bufs = FakeBwdBuffers(2, 4, 2, 64, 32, 2)
    assert bcall(lib, bufs, **{name: None}) == 1
    assert bcall(lib, bufs, **{name: bufs.addr[name] + 8}) == 3


@pytest.mark.parametrize("a,b", [("dq", "q"), ("dk", "dv"), ("dbeta", "beta"), ("dM0", "M0"),
                                 ("dz0", "dz_final"), ("workspace", "lse"), ("dq", "d_out"),
                                 ("dk", "workspace")])
def test_backward_rejects_overlaps(lib, a, b):
    bufs = FakeBwdBuffers(2, 4, 2, 64, 32, 2)
    assert bcall(lib, bufs, **{a: bufs.addr[b]}) == 1


def test_backward_rejects_small_workspace_and_bad_sizes(lib):
    bufs = FakeBwdBuffers(2, 4, 2, 64, 32, 2)
    _, need = bws(lib, 2, 4, 2, 64, 32, 16, 1, 1)
    assert bcall(lib, bufs, workspace_bytes=need - 1) == 4
    a = bufs.addr
    assert lib.infini_attn_backward(2, 3, 2, 64, 32, 16, 1, 1,
                                    *[ctypes.c_void_p(a[n]) for n in BWD_NAMES], 1 << 40,
                                    None) == 1


# ---- the block with its projections -------------------------------------------

BLOCK_NAMES = ["x", "w_qkv", "w_o", "beta", "M0", "z0", "y", "M_final", "z_final", "workspace"]
BLOCK_SHAPE = (2, 64, 96, 4, 2, 32, 16, 1, 1)  # B, L, d_model, Hq, Hkv, d, seg_len, rule, dtype


def blk_ws(lib, *args):
    n = ctypes.c_size_t(0)
    st = lib.infini_attn_block_workspace_size(*args, ctypes.byref(n))
    return st, n.value


class FakeBlockBuffers:
    def __init__(self, B, L, dm, Hq, Hkv, d):
        sizes = dict(x=B * L * dm * 2, w_qkv=(Hq + 2 * Hkv) * d * dm * 2, w_o=dm * Hq * d * 2,
                     beta=Hq * 4, M0=B * Hkv * d * d * 4, z0=B * Hkv * d * 4, y=B * L * dm * 2,
                     M_final=B * Hkv * d * d * 4, z_final=B * Hkv * d * 4, workspace=1 << 40)
        base = 1 << 44
        self.addr, self.size = {}, sizes
        for name in BLOCK_NAMES:
            self.addr[name] = base
            base += (sizes[name] + 4095) // 4096 * 4096 + 4096


def blk_call(lib, bufs, shape=BLOCK_SHAPE, **over):
    a = {**bufs.addr, **over}
    wsb = over.get("workspace_bytes", 16)  # too small: a call that passes every
    return lib.infini_attn_block_forward(  # other check stops at the workspace
        *shape, *[ctypes.c_void_p(a[n]) for n in BLOCK_NAMES], wsb, None)


def test_block_workspace_size(lib):
    B, L, dm, Hq, Hkv, d, N = 4, 32768, 4096, 32, 8, 128, 2048
    st, n = blk_ws(lib, B, L, dm, Hq, Hkv, d, N, 1, 1)
    assert st == 0
    _, fwd_full, _ = ws(lib, B, Hq, Hkv, L, d, N, 1, 1)
    # q and a [B,Hq,L,d], k and v [B,Hkv,L,d] in bf16, then a full forward workspace
    assert n == 2 * B * Hq * L * d * 2 + 2 * B * Hkv * L * d * 2 + fwd_full


def test_block_workspace_size_with_separate_widths(lib):
    def blk_ws_kv(*args):
        n = ctypes.c_size_t(0)
        st = lib.infini_attn_block_workspace_size_kv(*args, ctypes.byref(n))
        return st, n.value
    B, L, dm, Hq, Hkv, N = 4, 32768, 4096, 32, 8, 2048
    # equal widths: the square call's size
    assert blk_ws_kv(B, L, dm, Hq, Hkv, 128, 128, N, 1, 1) == blk_ws(lib, B, L, dm, Hq, Hkv, 128,
                                                                      N, 1, 1)
    dk, dv = 64, 128
    st, n = blk_ws_kv(B, L, dm, Hq, Hkv, dk, dv, N, 1, 1)
    assert st == 0
    _, fwd_full, _ = ws_kv(lib, B, Hq, Hkv, L, dk, dv, N, 1, 1)
    # q [B,Hq,L,dk], k [B,Hkv,L,dk], v [B,Hkv,L,dv], a [B,Hq,L,dv] in bf16, then the forward's
    assert n == (B * Hq * L * dk + B * Hkv * L * dk + B * Hkv * L * dv + B * Hq * L * dv) * 2 \
        + fwd_full
    assert blk_ws_kv(B, L, dm, Hq, Hkv, 64, 96, N, 1, 1)[0] == 2     # d_value unsupported
    assert blk_ws_kv(B, L, dm, Hq, Hkv, 64, 0, N, 1, 1)[0] == 1      # d_value < 1
    assert blk_ws_kv(B, L, dm, Hq, Hkv, 64, 128, N, 1, 0)[0] == 2    # float
    assert lib.infini_attn_block_workspace_size_kv(B, L, dm, Hq, Hkv, 64, 128, N, 1, 1,
                                                   None) == 1


@pytest.mark.parametrize("args,status", [
    ((2, 64, 96, 4, 2, 32, 16, 1, 0), 2),     # float: the projections are bf16 only
    ((2, 64, 100, 4, 2, 32, 16, 1, 1), 2),    # d_model not a multiple of 32
    ((2, 64, 0, 4, 2, 32, 16, 1, 1), 1),      # d_model < 1
    ((2, 64, 96, 4, 3, 32, 16, 1, 1), 1),     # Hq % Hkv
    ((2, 64, 96, 4, 2, 48, 16, 1, 1), 2),     # d unsupported
    ((2, 64, 1 << 22, 4, 2, 32, 16, 1, 1), 1),  # d_model too large
    ((1 << 16, 1 << 16, 96, 4, 2, 32, 16, 1, 1), 1),  # B L >= 2^31
])
def test_block_workspace_size_rejects(lib, args, status):
    assert blk_ws(lib, *args)[0] == status


def test_block_forward_stops_at_the_workspace_check(lib):
    bufs = FakeBlockBuffers(2, 64, 96, 4, 2, 32)
    assert blk_call(lib, bufs) == 4
    _, need = blk_ws(lib, *BLOCK_SHAPE)
    assert blk_call(lib, bufs, workspace_bytes=need - 1) == 4


@pytest.mark.parametrize("name", BLOCK_NAMES)
def test_block_forward_rejects_null_and_misaligned(lib, name):
    bufs = FakeBlockBuffers(2, 64, 96, 4, 2, 32)
    assert blk_call(lib, bufs, **{name: None}) == 1
    assert blk_call(lib, bufs, **{name: bufs.addr[name] + 8}) == 3


@pytest.mark.parametrize("a,b", [("y", "x"), ("y", "w_o"), ("workspace", "w_qkv"),
                                 ("M_final", "z0"), ("y", "M_final"), ("workspace", "y"),
                                 ("z_final", "beta")])
def test_block_forward_rejects_overlaps(lib, a, b):
    bufs = FakeBlockBuffers(2, 64, 96, 4, 2, 32)
    _, need = blk_ws(lib, *BLOCK_SHAPE)
    assert blk_call(lib, bufs, workspace_bytes=need, **{a: bufs.addr[b]}) == 1


def test_block_forward_rejects_bad_sizes_and_events(lib):
    bufs = FakeBlockBuffers(2, 64, 96, 4, 2, 32)
    assert blk_call(lib, bufs, shape=(2, 64, 96, 4, 2, 32, 16, 1, 0)) == 2
    assert blk_call(lib, bufs, shape=(2, 64, 96, 4, 2, 32, 16, 5, 1)) == 1
    a = bufs.addr
    _, need = blk_ws(lib, *BLOCK_SHAPE)
    ev = (ctypes.c_void_p * 2)(None, None)
    assert lib.infini_attn_block_forward_timed(
        *BLOCK_SHAPE, *[ctypes.c_void_p(a[n]) for n in BLOCK_NAMES], need, None, ev, 2) == 1
    assert lib.infini_attn_block_forward_timed(
        *BLOCK_SHAPE, *[ctypes.c_void_p(a[n]) for n in BLOCK_NAMES], need, None, None, 1) == 1


def test_block_binding_validates_before_the_library():
    import compressive_memory_transformers_amd as m
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(4 * 32, 64, dtype=torch.bfloat16)
    wo = torch.zeros(64, 2 * 32, dtype=torch.bfloat16)
    beta, M0, z0 = torch.zeros(2), torch.zeros(1, 1, 32, 32), torch.ones(1, 1, 32)
    with pytest.raises(ValueError):  # host tensors are refused
        m.block_forward(x, w, wo, beta, M0, z0, 4, "delta", 2, 1)
    with pytest.raises(ValueError):  # w_o of the wrong shape
        m.block_forward(x, w, wo[:, :32], beta, M0, z0, 4, "delta", 2, 1)
    with pytest.raises(TypeError):  # float x
        m.block_forward(x.float(), w, wo, beta, M0, z0, 4, "delta", 2, 1)
