"""The C ABI library loads, exports every function include/gdn.h declares, and its
host-side argument checks return the documented status before any launch.
No GPU is touched: every call here fails validation (or the workspace check),
which happens before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_69_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from gated_delta_rule_69_amd import build
        build.build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"gdn_chunk_fwd", "gdn_final_state", "gdn_recurrent_step",
                          "gdn_chunk_prepare", "gdn_chunk_scan", "gdn_asym_stabilize",
                          "gdn_recurrent_bwd", "gdn_bwd_workspace_bytes",
                          "gdn_workspace_bytes", "gdn_status_str", "gdn_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gdn_abi_version() == 3


def test_status_strings(lib):
    from gated_delta_rule_69_amd import _lib
    for code in (0, -1, -2, -3, -4):
        assert _lib.gdn_status_str(code) != "unknown status"
    assert _lib.gdn_status_str(7) == "unknown status"


FAKE = 1 << 20  # an aligned, never-dereferenced address


def good_args(**over):
    from gated_delta_rule_69_amd._lib import GdnArgs
    a = GdnArgs()
    a.variant, a.dtype = 0, 1
    a.B, a.T, a.H, a.dk, a.dv = 2, 100, 4, 64, 64
    a.chunk, a.n_h = 64, 1
    for f in ("q", "k", "v", "alpha", "beta", "o"):
        setattr(a, f, FAKE)
    for key, val in over.items():
        setattr(a, key, val)
    return a


def call_chunk(lib, a, ws=None, nbytes=0):
    return lib.gdn_chunk_fwd(ctypes.byref(a), ws, nbytes, None)


def test_valid_args_reach_the_workspace_check(lib):
    a = good_args()
    need = lib.gdn_workspace_bytes(ctypes.byref(a))
    assert need > 0
    # 2*4 heads * 2 chunks * record; the record holds at least W, U~, A^, Q+ in fp16
    assert need >= 2 * 4 * 2 * (4 * 64 * 64 * 2)
    assert call_chunk(lib, a) == -3
    assert call_chunk(lib, a, FAKE, need - 1) == -3
    assert call_chunk(lib, a, FAKE + 16, need) == -3      # not 256-byte aligned


@pytest.mark.parametrize("field,value,status", [
    ("variant", 9, -1), ("dtype", 5, -1), ("B", 0, -1), ("H", 0, -1), ("T", -1, -1),
    ("dk", 48, -2), ("dv", 256, -2), ("chunk", 128, -2), ("chunk", 8, -2), ("n_h", 2, -1),
    ("k", 0, -1), ("v", FAKE + 4, -1), ("alpha", 0, -1), ("beta", 0, -1), ("q", 0, -1),
    ("o", 0, -1), ("j", FAKE, -1), ("s0", FAKE + 8, -1), ("beta_v", FAKE + 2, -1),
])
def test_rejections(lib, field, value, status):
    a = good_args(**{field: value})
    assert call_chunk(lib, a, FAKE, 1 << 40) == status


def test_variant_specific_rules(lib):
    # FG2 with one beta vector needs dk == dv
    assert call_chunk(lib, good_args(dv=32), FAKE, 1 << 40) == -1
    # ... but FG2-GDN+ (beta_v) lifts it: reaches the launch, so only check sizing
    assert lib.gdn_workspace_bytes(ctypes.byref(good_args(dv=32, beta_v=FAKE))) > 0
    # KDA may not pass beta_v
    assert call_chunk(lib, good_args(variant=1, beta_v=FAKE), FAKE, 1 << 40) == -1
    # ASYM needs j and eta
    assert call_chunk(lib, good_args(variant=4), FAKE, 1 << 40) == -1
    # DeltaProduct: a chunk holds whole tokens of n_step steps (n_h; 4 for n_h = 3; 8
    # for n_h = 5..7) and at least 8 output rows (valid calls stop at the workspace)
    dp = dict(variant=3, n_h=3)
    ws_of = lambda **kw: lib.gdn_workspace_bytes(ctypes.byref(good_args(**kw)))  # noqa: E731
    assert call_chunk(lib, good_args(**dp)) == -3                        # 64 = 16 tokens x 4
    assert call_chunk(lib, good_args(chunk=32, **dp)) == -3              # 8 output rows
    assert call_chunk(lib, good_args(chunk=16, **dp), FAKE, 1 << 40) == -2  # 4 output rows
    assert ws_of(**dp) == ws_of(variant=3, n_h=4)
    for n_h in (5, 6, 7, 8):                                             # 8 tokens x 8 steps
        assert call_chunk(lib, good_args(variant=3, n_h=n_h)) == -3, n_h
        assert ws_of(variant=3, n_h=n_h) == ws_of(variant=3, n_h=8) > 0, n_h
    assert call_chunk(lib, good_args(variant=3, n_h=8, chunk=32), FAKE, 1 << 40) == -2
    assert call_chunk(lib, good_args(variant=3, n_h=9), FAKE, 1 << 40) == -2
    assert call_chunk(lib, good_args(variant=3, n_h=0), FAKE, 1 << 40) == -1
    assert call_chunk(lib, good_args(variant=3, n_h=2), FAKE, 0) == -3


def test_final_state_and_recurrent_checks(lib):
    a = good_args(q=0, o=0)
    assert lib.gdn_final_state(ctypes.byref(a), FAKE, 1 << 40, None) == -1  # s_final required
    a = good_args(q=0, o=0, s_final=FAKE)
    assert lib.gdn_final_state(ctypes.byref(a), None, 0, None) == -3
    a = good_args()
    assert lib.gdn_recurrent_step(ctypes.byref(a), None, None) == -1
    assert lib.gdn_recurrent_step(ctypes.byref(a), FAKE + 4, None) == -1
    assert lib.gdn_recurrent_step(ctypes.byref(good_args(variant=3, n_h=9)), FAKE, None) == -2
    assert lib.gdn_recurrent_step(None, FAKE, None) == -1


def test_fused_stabilizer_field(lib):
    # ASYM only, modes 0..2; checked before the workspace
    asym = dict(variant=4, j=FAKE, eta=FAKE)
    assert call_chunk(lib, good_args(**asym, stabilize=1)) == -3
    assert call_chunk(lib, good_args(**asym, stabilize=2)) == -3
    assert call_chunk(lib, good_args(**asym, stabilize=3), FAKE, 1 << 40) == -1
    assert call_chunk(lib, good_args(**asym, stabilize=-1), FAKE, 1 << 40) == -1
    assert call_chunk(lib, good_args(stabilize=1), FAKE, 1 << 40) == -1
    assert lib.gdn_recurrent_step(ctypes.byref(good_args(stabilize=2)), FAKE, None) == -1
    assert lib.gdn_workspace_bytes(ctypes.byref(good_args(**asym, stabilize=1))) == \
        lib.gdn_workspace_bytes(ctypes.byref(good_args(**asym)))


def test_backward_checks(lib):
    from gated_delta_rule_69_amd._lib import GdnGrads
    a = good_args()
    need = lib.gdn_bwd_workspace_bytes(ctypes.byref(a))
    assert need > 0
    full = GdnGrads(dq=FAKE, dk=FAKE, dv=FAKE, dalpha=FAKE, dbeta=FAKE)
    call = lambda args, g, ws=FAKE, n=need: lib.gdn_recurrent_bwd(  # noqa: E731
        ctypes.byref(args), FAKE, None, ctypes.byref(g) if g is not None else None, ws, n, None)
    assert call(a, full, None, 0) == -3
    assert call(a, full, FAKE, need - 1) == -3
    assert call(a, None) == -1
    assert call(a, GdnGrads(dq=FAKE, dk=FAKE, dv=FAKE, dalpha=FAKE)) == -1          # dbeta missing
    assert call(a, GdnGrads(dq=FAKE, dk=FAKE, dv=FAKE, dalpha=FAKE, dbeta=FAKE, dj=FAKE)) == -1
    assert call(good_args(variant=4, j=FAKE, eta=FAKE, stabilize=1), GdnGrads(dq=FAKE, dk=FAKE, dv=FAKE, dalpha=FAKE, dj=FAKE, deta=FAKE)) == -2
    assert lib.gdn_bwd_workspace_bytes(ctypes.byref(good_args(dk=48))) == 0
    # at most 2^33 steps over all heads (every launch grid stays in 32 bits)
    big = dict(B=1, H=1 << 10, T=1 << 23)
    assert lib.gdn_bwd_workspace_bytes(ctypes.byref(good_args(**big))) > 0          # 2^33 steps
    assert lib.gdn_bwd_workspace_bytes(ctypes.byref(good_args(B=2, H=1 << 10, T=1 << 23))) == 0
    assert call(good_args(B=2, H=1 << 10, T=1 << 23), full, FAKE, 1 << 62) == -2
    assert lib.gdn_bwd_workspace_bytes(ctypes.byref(good_args(variant=3, n_h=2, **big))) == 0


def test_stabilize_checks(lib):
    def stab(mode=1, out=FAKE, **over):
        a = good_args(**{"variant": 4, "j": FAKE, "eta": FAKE, **over})
        return lib.gdn_asym_stabilize(ctypes.byref(a), mode, out, None)

    assert stab(mode=0) == -1 and stab(mode=3) == -1
    assert stab(variant=0) == -1                      # ASYM inputs only
    for f in ("k", "j", "alpha", "eta"):
        assert stab(**{f: 0}) == -1, f
        assert stab(**{f: FAKE + 8}) == -1, f
    assert stab(out=None) == -1 and stab(out=FAKE + 4) == -1
    assert stab(dk=48) == -2
    # T = 0: nothing to do, nothing required, no launch
    assert stab(T=0, k=0, j=0, alpha=0, eta=0, out=None) == 0
    assert lib.gdn_asym_stabilize(None, 1, FAKE, None) == -1


def test_fp32_dk128_chunk64_runs_as_chunk32(lib):
    f32 = dict(dtype=0, dk=128, dv=128)
    w64 = lib.gdn_workspace_bytes(ctypes.byref(good_args(chunk=64, **f32)))
    w32 = lib.gdn_workspace_bytes(ctypes.byref(good_args(chunk=32, **f32)))
    assert w64 == w32 > 0
    assert call_chunk(lib, good_args(chunk=64, **f32)) == -3     # valid: reaches the workspace check
    # DeltaProduct in the 32-step chunks: 8 output rows with 4 steps a token, 4 with 8
    assert call_chunk(lib, good_args(chunk=64, variant=3, n_h=4, **f32)) == -3
    assert call_chunk(lib, good_args(chunk=64, variant=3, n_h=8, **f32), FAKE, 1 << 40) == -2


def test_workspace_bytes_grows_with_tokens(lib):
    # records of B * H * chunks items, then one flag byte per item rounded to 256
    def flags(items):
        return (items + 255) // 256 * 256
    small = lib.gdn_workspace_bytes(ctypes.byref(good_args(T=64)))       # 2 * 4 items
    big = lib.gdn_workspace_bytes(ctypes.byref(good_args(T=6400)))       # 2 * 4 * 100 items
    assert big - flags(800) == 100 * (small - flags(8))
    assert (small - flags(8)) % 256 == 0
    assert lib.gdn_workspace_bytes(ctypes.byref(good_args(dk=48))) == 0
    assert lib.gdn_workspace_bytes(None) == 0


def test_static_entry_rejects_what_its_buffer_cannot_hold(lib):
    """gdn_chunk_fwd_static checks its size limit before any HIP call: 1024 sequences
    of bf16 records (dk = dv = 128, chunk 64) exceed its buffer in a single chunk."""
    a = good_args(B=2, H=512, dk=128, dv=128)
    assert lib.gdn_chunk_fwd_static(ctypes.byref(a), None) == -2
    # without s_final the carried state counts too: 482 sequences no longer fit
    a = good_args(B=2, H=241, dk=128, dv=128)
    assert lib.gdn_chunk_fwd_static(ctypes.byref(a), None) == -2
    # and the ordinary argument checks come first
    assert lib.gdn_chunk_fwd_static(ctypes.byref(good_args(B=0)), None) == -1
