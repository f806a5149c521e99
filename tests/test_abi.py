"""The C-ABI library loads, exports every entry point of include/smoe.h, and
rejects bad arguments before enqueuing anything (no GPU needed: these calls
return from argument checking and never reach the HIP runtime)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smoe.h")
LIB = os.path.join(ROOT, "quantized_speculative_expert_amd", "libsmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB),
                                reason="libsmoe.so not built (run __graft_entry__.build())")

EINVAL, EUNSUPPORTED = -1, -2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smoe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    l = ctypes.CDLL(LIB)
    l.smoe_status_string.restype = ctypes.c_char_p
    l.smoe_last_error.restype = ctypes.c_char_p
    l.smoe_ffn_workspace_bytes.restype = ctypes.c_size_t
    return l


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"smoe_route_topk", "smoe_align_by_expert", "smoe_elb_accumulate_topm",
            "smoe_w4a16_expert_ffn", "smoe_fp16_expert_ffn", "smoe_combine",
            "smoe_ffn_workspace_bytes", "smoe_status_string", "smoe_last_error",
            "smoe_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_signatures_cover_header():
    # the Python binding declares a signature for every C entry point
    src = open(os.path.join(ROOT, "quantized_speculative_expert_amd", "_lib.py")).read()
    for n in declared_functions():
        assert f'"{n}"' in src, n


def test_status_strings(lib):
    assert lib.smoe_abi_version() == 4
    assert lib.smoe_status_string(0) == b"SMOE_OK"
    assert b"EINVAL" in lib.smoe_status_string(EINVAL)
    assert b"EUNSUPPORTED" in lib.smoe_status_string(EUNSUPPORTED)
    assert b"EHIP" in lib.smoe_status_string(-3)


def test_workspace_bytes(lib):
    f = lib.smoe_ffn_workspace_bytes
    f.argtypes = [ctypes.c_int] * 6
    # holds at least the intermediate activations of every routed slot and
    # shared-expert token, grows with the window, and an empty window needs none
    need = f(17, 6, 64, 2048, 1408, 0)
    assert need >= 17 * 6 * 1408 * 2 and need % 256 == 0
    assert f(544, 6, 64, 2048, 1408, 0) >= need + (544 - 17) * 6 * 1408 * 2
    with_shared = f(17, 6, 64, 2048, 1408, 2816)
    assert with_shared >= need + 17 * 2816 * 2 and with_shared % 256 == 0
    assert f(-1, 6, 64, 2048, 1408, 0) == 0
    assert f(0, 6, 64, 2048, 1408, 0) == 0
    assert f(17, 6, 64, 2048, 1408, -128) == 0


N = None


def test_route_argument_checks(lib):
    f = lib.smoe_route_topk
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 6
    assert f(N, N, N, 17, 2048, 0, 6, 0, N, N, N, N, N, N) == EINVAL
    assert f(N, N, N, 17, 2048, 300, 6, 0, N, N, N, N, N, N) == EUNSUPPORTED
    assert f(N, N, N, 17, 2048, 64, 9, 0, N, N, N, N, N, N) == EUNSUPPORTED
    assert f(N, N, N, 17, 2000, 64, 6, 0, N, N, N, N, N, N) == EUNSUPPORTED
    assert f(N, N, N, 17, 2048, 64, 6, 4, N, N, N, N, N, N) == EINVAL       # bad flag
    assert f(N, N, N, 17, 2048, 64, 6, 0, N, N, N, N, N, N) == EINVAL       # null x
    assert b"null" in lib.smoe_last_error()
    assert f(16, 16, N, 17, 2048, 64, 6, 0, 16, 16, N, N, N, N) == EINVAL   # logits required
    assert f(8, 16, N, 17, 2048, 64, 6, 0, 16, 16, 16, N, N, N) == EINVAL   # x alignment
    assert f(N, N, N, 0, 2048, 64, 6, 0, N, N, N, N, N, N) == 0             # empty window


def test_route_align_elb_argument_checks(lib):
    f = lib.smoe_route_align_elb
    f.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 11 +
                  [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2 + [ctypes.c_int, ctypes.c_void_p])
    r = [16, 16, N]                      # x, w_router, bias
    o = [16, 16, 16, N, N]               # ids, weights, logits, gate_w, gate
    al = [16, 16, 16, 16, 16]            # counts, offsets, sorted, active, n_active
    assert f(*r, 17, 2048, 300, 6, 0, *o, *al, N, 0, 0, 0, N, N, 0, N) == EUNSUPPORTED
    assert f(*r, 17, 2048, 64, 6, 0, 16, 16, N, N, N, *al, N, 0, 0, 0, N, N, 0, N) == EINVAL
    assert f(*r, 17, 2048, 64, 6, 0, *o, 16, N, 16, 16, 16, N, 0, 0, 0, N, N, 0, N) == EINVAL
    assert b"align_by_expert" in lib.smoe_last_error()
    assert f(*r, 17, 2048, 64, 6, 0, *o, *al, 16, 1, 1, 0, N, N, 0, N) == EINVAL  # layer >= L
    assert b"elb_accumulate_topm" in lib.smoe_last_error()
    assert f(*r, 17, 2048, 64, 6, 0, *o, *al, 16, 1, 0, 32, N, N, 0, N) == EINVAL  # plan_ids


def test_align_argument_checks(lib):
    f = lib.smoe_align_by_expert
    f.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 6
    assert f(N, 17, 6, 0, N, N, N, N, N, N) == EINVAL
    assert f(N, 17, 6, 257, N, N, N, N, N, N) == EUNSUPPORTED
    assert f(N, 17, 6, 64, N, N, N, N, N, N) == EINVAL


def test_elb_argument_checks(lib):
    f = lib.smoe_elb_accumulate_topm
    f.argtypes = ([ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p] +
                  [ctypes.c_int] * 5 + [ctypes.c_void_p] * 2 + [ctypes.c_int, ctypes.c_void_p])
    assert f(N, 1, 64, N, 0, 0, 0, 1, 32, N, N, 0, N) == EINVAL            # null counter
    assert f(1, 1, 64, N, 0, 0, 0, 1, 65, 1, N, 0, N) == EINVAL            # M > E
    assert f(1, 1, 64, N, 0, 0, 0, 1, 32, N, N, 0, N) == EINVAL            # null plan
    assert f(1, 1, 64, 1, 0, 2, 17, 6, 32, 1, N, 0, N) == EINVAL           # layers out of range
    assert f(1, 1, 64, N, 0, 0, 0, 1, 32, 1, N, 2, N) == EINVAL            # bad flag


def test_ffn_argument_checks(lib):
    f = lib.smoe_w4a16_expert_ffn
    f.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 8 +
                  [ctypes.c_int] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p])
    w = [16] * 8                   # weights, scales, sorted slots, offsets
    ns = [0, N, N, N]              # no shared expert
    ws = 1 << 30
    assert f(16, 17, 6, 64, 2048, 1408, 96, *w, *ns, 256, ws, 16, N, N) == EUNSUPPORTED  # G
    assert f(16, 17, 6, 64, 2048, 1400, 128, *w, *ns, 256, ws, 16, N, N) == EUNSUPPORTED  # I
    assert f(16, 17, 9, 64, 2048, 1408, 128, *w, *ns, 256, ws, 16, N, N) == EUNSUPPORTED  # k
    # k > E passes the limits (a call over one expert's slots): the workspace
    # check after them is what fails here
    assert f(16, 17, 6, 1, 2048, 1408, 128, *w, *ns, 256, 10, 16, N, N) == EINVAL
    assert b"workspace" in lib.smoe_last_error()
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, *ns, 256, 10, 16, N, N) == EINVAL  # small ws
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, *ns, 8, ws, 16, N, N) == EINVAL  # ws align
    # shared expert: size checks, pointers and alignment
    sh = [16, 16, 16]
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, -128, *sh, 256, ws, 16, 16, N) == EINVAL
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, 100, *sh, 256, ws, 16, 16, N) == EUNSUPPORTED
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, 2816, *sh, 256, ws, 16, N, N) == EINVAL
    assert b"shared" in lib.smoe_last_error()
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, 2816, 16, 16, 8, 256, ws, 16, 16,
             N) == EINVAL
    small = lib.smoe_ffn_workspace_bytes(17, 6, 64, 2048, 1408, 0)
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, 2816, *sh, 256, small, 16, 16,
             N) == EINVAL  # workspace without room for the shared expert
    g = lib.smoe_fp16_expert_ffn
    g.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5 +
                  [ctypes.c_int] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p])
    w16 = [16] * 5
    assert g(N, 17, 6, 64, 2048, 1408, *w16, *ns, 256, ws, 16, N, N) == EINVAL
    assert g(16, 17, 0, 64, 2048, 1408, *w16, *ns, 256, ws, 16, N, N) == EINVAL
    assert g(16, 17, 6, 64, 2048, 1408, *w16, 2816, *sh, 256, ws, 16, N, N) == EINVAL


def test_combine_argument_checks(lib):
    f = lib.smoe_combine
    f.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 4
    assert f(N, N, 17, 6, 2048, N, 16, N, N) == EINVAL   # gate without shared output
    assert f(N, N, 17, 9, 2048, N, N, N, N) == EUNSUPPORTED
    assert f(N, N, 17, 6, 2048, N, N, N, N) == EINVAL
    assert f(8, 16, 17, 6, 2048, N, N, 16, N) == EINVAL  # misaligned slot_out
    assert f(N, N, 0, 6, 2048, N, N, N, N) == 0


def test_binding_refuses_short_tensors(lib):
    # the Python binding checks every buffer's size against the shapes the
    # call implies before any pointer reaches the library (CPU tensors: the
    # size check comes first, so nothing is launched)
    import torch
    from quantized_speculative_expert_amd import _lib as smoe
    i32 = dict(dtype=torch.int32)
    f16, f32 = dict(dtype=torch.float16), dict(dtype=torch.float32)
    T, k, E, H, I, G = 17, 2, 8, 256, 512, 64
    x = torch.zeros((T, H), **f16)
    codes = torch.zeros(E * I * H // 8, **i32)
    scales = torch.zeros(E * I * H // G, **f16)
    ok = dict(sorted_slots=torch.zeros(T * k, **i32), expert_offsets=torch.zeros(E + 1, **i32),
              workspace=torch.zeros(16, dtype=torch.uint8), slot_out=torch.zeros(T * k * H, **f32))

    def ffn(**over):
        a = dict(wg_q=codes, wg_s=scales, wu_q=codes, wu_s=scales, wd_q=codes, wd_s=scales, **ok)
        a.update(over)
        smoe.smoe_w4a16_expert_ffn(x, k, E, I, G, a["wg_q"], a["wg_s"], a["wu_q"], a["wu_s"],
                                   a["wd_q"], a["wd_s"], a["sorted_slots"], a["expert_offsets"],
                                   a["workspace"], a["slot_out"])

    for name, short in (("wg_q", codes[:-1]), ("wd_s", scales[:-1]),
                        ("sorted_slots", ok["sorted_slots"][:-1]),
                        ("expert_offsets", ok["expert_offsets"][:E]),
                        ("slot_out", ok["slot_out"][:-1])):
        with pytest.raises(ValueError, match=name):
            ffn(**{name: short})
    with pytest.raises(ValueError, match="logits"):
        smoe.smoe_route_topk(x, torch.zeros((E, H), **f32), None, k, 0, torch.zeros(T * k, **i32),
                             torch.zeros(T * k, **f32), torch.zeros(T * E - 1, **f32))
    with pytest.raises(ValueError, match="y holds"):
        smoe.smoe_combine(torch.zeros(T * k * H, **f32), torch.zeros((T, k), **f32), None, None,
                          torch.zeros((T - 1, H), **f16))


def test_layer_call_argument_checks(lib):
    # every step's checks run before anything is enqueued, with the errors
    # the separate calls give
    f = lib.smoe_moe_layer_w4a16
    f.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 11 +
                  [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 3 +
                  [ctypes.c_void_p] * 6 + [ctypes.c_int] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_size_t] + [ctypes.c_void_p] * 4)
    r = [16, 16, N]                      # x, w_router, bias
    o = [16, 16, 16, N, N]               # ids, weights, logits, gate_w, gate
    al = [16, 16, 16, 16, 16]            # counts, offsets, sorted, active, n_active
    elb = [N, 0, 0, 0, N, N, 0]          # no activation counter
    w = [16] * 6                         # routed codes and scales
    ns = [0, N, N, N]                    # no shared expert
    ws = 1 << 30

    def call(T=17, H=2048, E=64, k=6, I=1408, G=128, x=16, route=None, align=None, elb_=None,
             weights=None, shared=None, wsp=256, wsb=ws, slot_out=16, shared_out=N, y=16):
        return f(x, *r[1:], T, H, E, k, 0, *(route or o), *(align or al), *(elb_ or elb), I, G,
                 *(weights or w), *(shared or ns), wsp, wsb, slot_out, shared_out, y, N)

    assert call(E=300) == EUNSUPPORTED                                  # routing limits
    assert b"route_topk" in lib.smoe_last_error()
    assert call(align=[16, N, 16, 16, 16]) == EINVAL                    # align outputs
    assert b"align_by_expert" in lib.smoe_last_error()
    assert call(elb_=[16, 1, 1, 0, N, N, 0]) == EINVAL                  # layer >= L
    assert b"elb_accumulate_topm" in lib.smoe_last_error()
    assert call(G=96) == EUNSUPPORTED                                   # group size
    assert call(I=1400) == EUNSUPPORTED                                 # FFN limits
    assert call(wsb=10) == EINVAL                                       # workspace size
    assert b"workspace" in lib.smoe_last_error()
    assert call(shared=[2816, 16, 16, 16]) == EINVAL                    # no shared_out
    assert call(route=[16, 16, 16, 16, 16]) == EINVAL                   # gate without shared
    assert b"combine" in lib.smoe_last_error()
    assert call(y=N) == EINVAL                                          # combine output
    assert call(weights=[16, 16, N, 16, 16, 16]) == EINVAL              # null weight
    assert b"weight" in lib.smoe_last_error()
    assert call(T=0, x=N) == 0                                          # empty window


def test_tiled_calls_check_like_row_major(lib):
    # the tiled-layout calls take the row-major calls' arguments and checks
    f = lib.smoe_w4a16_expert_ffn_tiled
    f.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 8 +
                  [ctypes.c_int] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p])
    w = [16] * 8
    ns = [0, N, N, N]
    ws = 1 << 30
    assert f(16, 17, 6, 64, 2048, 1408, 96, *w, *ns, 256, ws, 16, N, N) == EUNSUPPORTED
    assert b"w4a16_expert_ffn_tiled" in lib.smoe_last_error()
    assert f(16, 17, 6, 64, 2048, 1408, 128, *w, *ns, 256, 10, 16, N, N) == EINVAL
    assert f(N, 0, 6, 64, 2048, 1408, 128, *w, *ns, 256, ws, 16, N, N) == 0  # empty window
    g = lib.smoe_fp16_expert_ffn_tiled
    g.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 5 + [ctypes.c_void_p] * 5 +
                  [ctypes.c_int] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p])
    assert g(N, 17, 6, 64, 2048, 1408, *[16] * 5, *ns, 256, ws, 16, N, N) == EINVAL
    assert b"fp16_expert_ffn_tiled" in lib.smoe_last_error()


def test_tile_weights_argument_checks(lib):
    f = lib.smoe_tile_weights
    f.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    a, b = 1 << 20, 1 << 30          # two well-separated (never dereferenced) addresses
    assert f(a, a, 2, 8, 256, 128, b, b, N) == EUNSUPPORTED       # N not a multiple of 16
    assert f(a, a, 2, 16, 200, 128, b, b, N) == EUNSUPPORTED      # K not a multiple of 128
    assert f(a, a, 2, 16, 256, 16, b, b, N) == EUNSUPPORTED       # group size
    assert b"group size" in lib.smoe_last_error()
    assert f(-1, a, 2, 16, 256, 128, b, b, N) == EINVAL            # negative E
    assert f(N, a, 2, 16, 256, 128, b, b, N) == EINVAL             # null weights
    assert f(a, N, 2, 16, 256, 128, b, b, N) == EINVAL             # INT4 without scales
    assert f(a, a, 2, 16, 256, 128, a + 16, b, N) == EINVAL        # overlapping copy
    assert b"overlap" in lib.smoe_last_error()
    assert f(a + 8, a, 2, 16, 256, 128, b, b, N) == EINVAL         # misaligned
    assert f(a, a, 0, 16, 256, 128, b, b, N) == 0                  # nothing to tile


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES", "") != "" or
                    os.path.exists("/dev/kfd"),
                    reason="passes host-side addresses; run only where no GPU can be reached")
def test_tile_weights_checks_scales_before_any_launch(lib):
    # codes that do not overlap but scales that do: the call must refuse
    # before it enqueues the code-tiling kernel (a launch here, without a
    # GPU, would report SMOE_EHIP instead)
    f = lib.smoe_tile_weights
    f.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    a, b, c = 1 << 20, 1 << 30, 1 << 34
    assert f(a, c, 2, 16, 256, 128, b, c + 16, N) == EINVAL
    assert b"scales_tiled must not overlap" in lib.smoe_last_error()



def test_noalloc_ffn_refuses_oversize_before_touching_a_device(lib):
    # 544 tokens x top-6 need about 98 MB of workspace, above the library's
    # static 16 MiB: refused from host values alone (no GPU here)
    f = lib.smoe_w4a16_expert_ffn_noalloc
    f.argtypes = ([ctypes.c_void_p] + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 8 +
                  [ctypes.c_int] + [ctypes.c_void_p] * 6)
    w = [16] * 8
    assert f(16, 544, 6, 64, 2048, 1408, 128, *w, 0, N, N, N, 16, N, N) == EUNSUPPORTED
    assert b"static workspace" in lib.smoe_last_error()
    assert f(16, 17, 6, 64, 2048, 1408, 96, *w, 0, N, N, N, 16, N, N) == EUNSUPPORTED  # G
    assert f(N, 0, 6, 64, 2048, 1408, 128, *w, 0, N, N, N, 16, N, N) == 0  # empty window
