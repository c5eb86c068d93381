"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/megamoe.h declares, and rejects bad arguments
synchronously without touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from moe_expert_ffn_amd import megamoe as MM

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(megamoe_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = MM.load()
    declared = _declared()
    assert declared, "no declarations found"
    for n in sorted(declared):
        assert hasattr(lib, n), f"missing export {n}"
    assert declared == set(MM.EXPORTED)


def test_check_dims_limits():
    ok = MM.dims(2048, 7168, 32, 8, 2048)
    assert MM.megamoe_check_dims(ok) == 0
    bad = [
        (MM.dims(0, 128, 4, 2, 128), 1),
        (MM.dims(4, 100, 4, 2, 128), 2),      # K % 128
        (MM.dims(4, 128, 4, 5, 128), 2),      # top_k > E
        (MM.dims(4, 128, 300, 2, 128), 2),    # E > 256
        (MM.dims(4, 128, 4, 2, 130), 2),      # I % 128
        (MM.dims(1 << 20, 32768, 8, 8, 128), 2),  # R * K overflows int32
    ]
    for d, code in bad:
        assert MM.megamoe_check_dims(d) == code, d


def test_workspace_and_packed_sizes():
    d = MM.dims(2048, 7168, 32, 8, 2048)
    ws = MM.megamoe_workspace_bytes(d)
    R = 2048 * 8
    # intermediates: the token-major quantised x [M, K] plus gmC + q2 +
    # gmm2_out, all [R, .], dominate
    assert ws >= 2048 * 7168 + R * 4096 * 2 + R * 2048 + R * 7168 * 2
    assert ws < R * 7168 * 6
    assert MM.megamoe_packed_weight_bytes(d) == (32 * 7168 * 4096, 32 * 2048 * 7168)
    # the packed layout pads each expert's output columns to whole 256-row blocks
    d = MM.dims(64, 384, 16, 4, 128)
    assert MM.megamoe_packed_weight_bytes(d) == (16 * 384 * 256, 16 * 128 * 512)
    assert MM.megamoe_permute_workspace_bytes(d) >= 4
    with pytest.raises(MM.MegaMoEError):
        MM.megamoe_workspace_bytes(MM.dims(4, 100, 4, 2, 128))


def test_null_and_misaligned_pointers_rejected():
    lib = MM.load()
    d = MM.dims(16, 256, 4, 2, 128)
    P = ctypes.c_void_p
    null = [None] * 12
    assert lib.megamoe_forward(ctypes.byref(d), *null[:9], ctypes.c_size_t(1 << 30), None) == 1
    odd = P(0x1000 + 4)
    good = P(0x1000)
    rc = lib.megamoe_unpermute(ctypes.byref(d), odd, good, good, good, good, None)
    assert rc == 1
    rc = lib.megamoe_gmm1(ctypes.byref(d), good, good, good, good, good, odd, None)
    assert rc == 1
    # workspace too small is reported before anything is launched
    rc = lib.megamoe_forward(ctypes.byref(d), *([good] * 9), ctypes.c_size_t(16), None)
    assert rc == 3
    # the same for GMM1's K-split buffer: one byte short of its size
    need = MM.megamoe_gmm1_split_workspace_bytes(d)
    rc = lib.megamoe_gmm1_gather_split(ctypes.byref(d), *([good] * 7), ctypes.c_size_t(need - 1),
                                       None)
    assert rc == 3


def test_split_workspace_size():
    """GMM1's K-split buffer holds a counter block and 4 partial int32 tiles of
    256 x 256 for each of up to 64 leftover tiles, whatever the dims."""
    sizes = {MM.megamoe_gmm1_split_workspace_bytes(MM.dims(*a))
             for a in ((16, 256, 4, 2, 128), (2048, 7168, 32, 8, 2048), (4096, 4096, 64, 6, 1408))}
    assert len(sizes) == 1
    (n,) = sizes
    assert 64 * 4 * 256 * 256 * 4 < n <= 64 * 4 * 256 * 256 * 4 + 4096
    # the forward's workspace holds the same partial tiles
    d = MM.dims(2048, 7168, 32, 8, 2048)
    assert MM.megamoe_workspace_bytes(d) > 64 * 4 * 256 * 256 * 4 + 2048 * 8 * 7168 * 2


def test_set_overlap_modes():
    lib = MM.load()
    for bad in (-1, 3, 1 << 20):
        assert lib.megamoe_set_overlap(bad) == 1
    for mode in (1, 2, 0):  # ends on the default
        assert lib.megamoe_set_overlap(mode) == 0


def test_strerror():
    assert MM.strerror(0) == "ok"
    assert "workspace" in MM.strerror(3)
    assert "dropped" in MM.strerror(MM.MEGAMOE_EDEVICE)


# Every device-pointer argument of the compute entry points, by position after
# the dims pointer; None marks the workspace size (a size_t).  Nullable
# arguments (the debug accumulators) are listed separately.
_POINTER_ARGS = {
    "megamoe_prepack_w1": (2, ()),
    "megamoe_prepack_w2": (2, ()),
    "megamoe_forward": (9, ()),               # x .. out, workspace, then its size
    "megamoe_permute": (9, ()),
    "megamoe_permute_tokens": (9, ()),
    "megamoe_permute_noalloc": (9, ()),
    "megamoe_gmm1": (6, (5,)),
    "megamoe_gmm1_gather": (7, (6,)),
    "megamoe_gmm1_gather_split": (7, ()),     # qx .. gmC, split buffer, then its size
    "megamoe_permute_tokens_paired": (10, ()),
    "megamoe_swiglu_quant_paired": (6, ()),
    "megamoe_gmm2_paired": (6, (5,)),
    "megamoe_swiglu_quant": (5, ()),
    "megamoe_gmm2": (6, (5,)),
    "megamoe_unpermute": (5, ()),
}


def _no_gpu():
    try:
        import torch
    except ImportError:
        return True
    return torch.cuda.device_count() == 0  # counts devices without initialising one


@pytest.mark.skipif(not _no_gpu(), reason="passes placeholder device addresses; host-only")
@pytest.mark.parametrize("name", sorted(_POINTER_ARGS))
def test_every_pointer_argument_checked(name):
    """For every required device pointer of every compute entry point, a null
    or a misaligned value is rejected with MEGAMOE_EINVAL, and a misaligned
    nullable one too; nothing is launched."""
    lib = MM.load()
    fn = getattr(lib, name)
    n_ptr, nullable = _POINTER_ARGS[name]
    d = MM.dims(16, 256, 4, 2, 128)
    good, odd = 0x10000, 0x10004
    sized = name in ("megamoe_forward", "megamoe_permute", "megamoe_permute_tokens",
                     "megamoe_permute_tokens_paired", "megamoe_gmm1_gather_split")

    def call(ptrs):
        args = [ctypes.byref(d)] + [ctypes.c_void_p(v) if v else None for v in ptrs]
        if sized:
            args.append(ctypes.c_size_t(1 << 40))
        args.append(None)  # stream
        return fn(*args)

    for pos in range(n_ptr):
        for bad in ((0, odd) if pos not in nullable else (odd,)):
            ptrs = [good] * n_ptr
            ptrs[pos] = bad
            assert call(ptrs) == 1, (name, pos, hex(bad))
