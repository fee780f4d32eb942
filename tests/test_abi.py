"""C ABI checks that need no GPU: the library loads, exports every entry point
declared under include/, and rejects bad arguments on the host before
any device call."""

import ctypes
import os
import re

import pytest

import int4_quantized_expert_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b((?:moe|gdn)_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "moe_layer_forward" in names and "gdn_recurrence_forward" in names and len(names) >= 8
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def good_desc(**kw):
    d = M.desc_for(2048, 512, 10, 512, 512, 4, "bf16", "bf16", "f32", pool_bytes=512 * 1769472)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_sizes_of_named_shapes():
    d = good_desc()
    assert M.blob_bytes(d, False) == 1769472
    assert d.blob_stride == 1769472
    d8 = M.desc_for(2048, 256, 8, 512, 512, 8, "bf16", "bf16", "f32", pool_bytes=1 << 34)
    assert M.blob_bytes(d8, False) == 3342336
    dt = M.desc_for(256, 16, 2, 128, 128, 4, "f32", "f32", "f32", pool_bytes=1 << 20)
    assert M.blob_bytes(dt, True) == 61440
    assert M.workspace_bytes(d, 8) > M.workspace_bytes(d, 1) > 0


@pytest.mark.parametrize("field,value", [
    ("hidden", 1000), ("hidden", 4096), ("inter", 96), ("n_experts", 0), ("n_experts", 2048),
    ("top_k", 0), ("top_k", 513), ("bits", 2), ("group_size", 32), ("act_dtype", 7),
    ("blob_stride", 1769472 - 256), ("blob_stride", 1769472 + 100), ("shared_stride", 4096),
    ("pool_bytes", 100),
])
def test_bad_descriptor_rejected(field, value):
    d = good_desc(**{field: value})
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    rc = M.lib().moe_layer_forward(ctypes.byref(d), 1, p, p, p, p, p, p, p, 1 << 10, None, None, None)
    assert rc == -1
    assert M.last_error()


def test_null_and_misaligned_pointers_rejected():
    d = good_desc()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    L = M.lib()
    assert L.moe_layer_forward(ctypes.byref(d), 1, None, p, p, p, p, p, p, 1 << 12, None, None, None) == -1
    assert L.moe_layer_forward(ctypes.byref(d), 1, p + 2, p, p, p, p, p, p, 1 << 12, None, None, None) == -1
    assert L.moe_layer_forward(ctypes.byref(d), 1, p, p, p, p + 16, p, p, p, 1 << 12, None, None, None) == -1
    assert L.moe_router_topk(ctypes.byref(d), 1, p, p, None, p, p, 1 << 12, None) == -1


def test_small_workspace_is_enomem_and_negative_T_einval():
    d = good_desc()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    L = M.lib()
    need = M.workspace_bytes(d, 8)
    assert L.moe_layer_forward(ctypes.byref(d), 8, p, p, p, p, p, p, p, need - 1, None, None, None) == -4
    assert L.moe_layer_forward(ctypes.byref(d), -1, p, p, p, p, p, p, p, need, None, None, None) == -1
    assert M.lib().moe_workspace_bytes(ctypes.byref(d), -3) == 0


def test_zero_tokens_enqueue_nothing():
    """T == 0 returns MOE_OK after validation without any device call."""
    d = good_desc()
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    need = M.workspace_bytes(d, 0)
    assert M.lib().moe_layer_forward(ctypes.byref(d), 0, p, p, p, p, p, p, p, need, None, None, None) == 0


def test_synth_device_fill_library_loads():
    from synth import gpu
    assert hasattr(gpu.lib(), "synth_fill_blobs")


def test_launch_event_hook_argument_checks():
    """moe_set_launch_events validates on the host and NULL events clear it."""
    L = M.lib()
    n = ctypes.c_int32(-5)
    ev = (ctypes.c_void_p * 2)(None, None)
    assert L.moe_set_launch_events(None, 0, None) == 0
    assert L.moe_set_launch_events(ev, 0, ctypes.byref(n)) == -1
    assert L.moe_set_launch_events(ev, 2, None) == -1
    # A call rejected before any launch records nothing and clears the setting.
    assert L.moe_set_launch_events(ev, 2, ctypes.byref(n)) == 0
    assert n.value == 0
    d = good_desc()
    assert L.moe_layer_forward(ctypes.byref(d), -1, None, None, None, None, None, None, None, 0, None, None,
                               None) == -1
    assert n.value == 0
    n.value = 7
    assert L.moe_layer_forward(ctypes.byref(d), -1, None, None, None, None, None, None, None, 0, None, None,
                               None) == -1
    assert n.value == 7, "a consumed setting must not be written again"


def test_chain_rejects_x_next_overlapping_x_or_out():
    """x_next must share no byte with x or out (the fused combine writes them
    element by element while other blocks still read x)."""
    d = good_desc()
    T, H = 2, 2048
    buf = ctypes.create_string_buffer(1 << 20)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    x, out, ws = p, p + 65536, p + 131072
    L = M.lib()
    need = M.workspace_bytes(d, T)

    def chain(x_next):
        return L.moe_layer_forward_chain(ctypes.byref(d), T, x, p, p, p, p, out, x_next, ws, need, None, None,
                                         None)
    assert chain(x) == -1                          # in place
    assert chain(x + 16) == -1                     # x at an offset
    assert chain(x - T * H * 2 + 16) == -1         # ends inside x
    assert chain(out) == -1                        # x_next == out
    assert chain(out + T * H * 4 - 16) == -1       # starts inside out
    assert "overlaps" in M.last_error()


def test_residual_add_rejects_partial_overlap():
    T, H = 2, 256
    buf = ctypes.create_string_buffer(1 << 16)
    p = ctypes.addressof(buf) // 256 * 256 + 256
    x, y = p, p + 8192
    L = M.lib()
    assert L.moe_residual_add(T, H, M.MOE_BF16, x, y, x + 2, None) == -1     # shifted in-place
    assert L.moe_residual_add(T, H, M.MOE_BF16, x, y, y + 4, None) == -1     # into y
    assert L.moe_residual_add(T, H, M.MOE_F32, x, y, y - 4, None) == -1      # ends inside y
    assert L.moe_residual_add(0, H, M.MOE_BF16, x, y, x, None) == 0          # exact in place is fine


def _gdn_args():
    """Host buffers standing in for device pointers: every call below is
    rejected (or is a no-op) before any device work, so they are never read."""
    buf = ctypes.create_string_buffer(1 << 20)
    base = ctypes.addressof(buf) // 256 * 256 + 256
    B, T, nk, nv, dk, dv = 2, 3, 2, 4, 128, 64
    q = base
    k = q + B * T * nk * dk * 2
    v = k + B * T * nk * dk * 2
    al = v + B * T * nv * dv * 2
    be = al + B * T * nv * 4 + 64
    st = (be + B * T * nv * 4 + 255) // 256 * 256
    out = st + B * nv * dv * dk * 4
    return buf, dict(B=B, T=T, q=q, k=k, v=v, al=al, be=be, st=st, out=out)


def _gdn_call(d, a, **over):
    a = {**a, **over}
    return M.lib().gdn_recurrence_forward(ctypes.byref(d), a["B"], a["T"], a["q"], a["k"], a["v"], a["al"], a["be"],
                                          a["st"], a["out"], None)


@pytest.mark.parametrize("field,value", [
    ("n_k_heads", 0), ("n_v_heads", 3), ("n_v_heads", 2048), ("d_k", 96), ("d_k", 256), ("d_v", 8), ("d_v", 72),
    ("d_v", 272), ("act_dtype", 5), ("out_dtype", -1), ("scale", float("inf")), ("eps", -1.0), ("eps", float("nan")),
])
def test_gdn_bad_descriptor_rejected(field, value):
    keep, a = _gdn_args()
    d = M.gdn_desc(2, 4, 128, 64)
    setattr(d, field, value)
    assert _gdn_call(d, a) == -1
    assert M.last_error()


def test_gdn_pointer_and_size_checks():
    keep, a = _gdn_args()
    d = M.gdn_desc(2, 4, 128, 64, act="bf16", out="f32")
    assert _gdn_call(d, a, q=None) == -1
    assert _gdn_call(d, a, st=a["st"] + 8) == -1            # state not 16-byte aligned
    assert _gdn_call(d, a, al=a["al"] + 2) == -1            # alpha not 4-byte aligned
    assert _gdn_call(d, a, B=-1) == -1
    assert _gdn_call(d, a, T=(1 << 20) + 1) == -1
    assert _gdn_call(d, a, out=a["st"] + 256) == -1         # out inside the state
    assert _gdn_call(d, a, st=a["v"]) == -1                 # state over v
    assert _gdn_call(d, a, out=a["q"]) == -1                # out over q
    assert _gdn_call(d, a, B=0) == 0                        # nothing to do: no device call
    assert _gdn_call(d, a, T=0) == 0
