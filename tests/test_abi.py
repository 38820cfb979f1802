"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_02_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_tiled_attention_02_amd import build
        build.build()
    return fa.load()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd", "fa_decode", "fa_strerror",
              "fa_release_workspace", "fa_decode_workgroups", "fa_read_probe", "fa_decode_fp8",
              "fa_decode_fp8_workgroups", "fa_decode_int8", "fa_decode_int8_workgroups"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr), name


P = None  # a NULL pointer
FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    # (q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale)
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 96, 1, 0.1), 3),      # d unsupported
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 3, 8, 8, 64, 1, 0.1), 2),      # Hq % Hkv
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 0, 8, 8, 64, 1, 0.1), 2),      # Hkv = 0
    ((FAKE, FAKE, FAKE, FAKE, P, -1, 4, 2, 8, 8, 64, 1, 0.1), 2),     # negative B
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, -8, 8, 64, 1, 0.1), 2),     # negative Tq
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, -1, 64, 1, 0.1), 2),     # negative Tk
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, 1, float("nan")), 2),
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, 1, float("inf")), 2),
    ((P, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, 1, 0.1), 1),         # q NULL
    ((FAKE, P, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, 1, 0.1), 1),         # k NULL with Tk > 0
    ((FAKE, FAKE, FAKE, P, P, 1, 4, 2, 8, 8, 64, 1, 0.1), 1),         # o NULL
    ((P, P, P, P, P, 0, 4, 2, 8, 8, 64, 1, 0.1), 0),                  # empty batch: no-op
    ((P, P, P, P, P, 2, 4, 2, 0, 8, 64, 0, 0.1), 0),                  # no query rows: no-op
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 1, 1, 65535 * 32 + 1, 8, 64, 1, 0.1), 2),  # too many rows
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, 3, 0.1), 2),      # causal mode 3
    ((FAKE, FAKE, FAKE, FAKE, P, 1, 4, 2, 8, 8, 64, -1, 0.1), 2),     # causal mode -1
])
@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_f32"])
def test_fwd_validation(lib, entry, args, status):
    fn = getattr(lib, entry)
    assert fn(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # (q, k, v, qs, ks, vs, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale)
    ((FAKE,) * 8 + (1, 4, 2, 8, 8, 96, 1, 0.1), 3),
    ((FAKE,) * 8 + (1, 4, 3, 8, 8, 64, 1, 0.1), 2),
    ((FAKE,) * 8 + (1, 4, 2, 8, 8, 64, 3, 0.1), 2),
    ((FAKE,) * 8 + (1, 4, 2, 8, 8, 64, 1, float("inf")), 2),
    ((FAKE, FAKE, FAKE, P, FAKE, FAKE, FAKE, P) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # qscale NULL
    ((FAKE, FAKE, FAKE, FAKE, P, FAKE, FAKE, P) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # kscale NULL
    ((FAKE, FAKE, FAKE, FAKE, FAKE, P, FAKE, P) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # vscale NULL
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, P, P) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # o NULL
    ((P,) * 8 + (0, 4, 2, 8, 8, 64, 1, 0.1), 0),
])
def test_fwd_fp8_validation(lib, args, status):
    assert lib.fa_fwd_fp8(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # (q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Tq, Tk, d, causal, scale)
    ((FAKE,) * 9 + (1, 4, 2, 8, 8, 96, 1, 0.1), 3),                 # d unsupported
    ((FAKE,) * 9 + (1, 4, 3, 8, 8, 64, 1, 0.1), 2),                 # Hq % Hkv
    ((FAKE,) * 9 + (1, 4, 0, 8, 8, 64, 1, 0.1), 2),                 # Hkv = 0
    ((FAKE,) * 9 + (-1, 4, 2, 8, 8, 64, 1, 0.1), 2),                # negative B
    ((FAKE,) * 9 + (1, 4, 2, -1, 8, 64, 1, 0.1), 2),                # negative Tq
    ((FAKE,) * 9 + (1, 4, 2, 8, -1, 64, 1, 0.1), 2),                # negative Tk
    ((FAKE,) * 9 + (1, 4, 2, 8, 8, 64, 1, float("nan")), 2),
    ((FAKE,) * 9 + (1, 4, 2, 8, 8, 64, 3, 0.1), 2),                 # causal mode 3
    ((FAKE,) * 4 + (P,) + (FAKE,) * 4 + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # lse NULL
    ((FAKE,) * 5 + (P,) + (FAKE,) * 3 + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # dout NULL
    ((FAKE,) * 6 + (P,) + (FAKE,) * 2 + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),   # dq NULL
    ((FAKE,) * 7 + (P, FAKE) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),            # dk NULL
    ((FAKE,) * 8 + (P,) + (1, 4, 2, 8, 8, 64, 1, 0.1), 1),                 # dv NULL
    ((P, FAKE, FAKE, P, P, P, P, P, FAKE) + (1, 4, 2, 0, 8, 64, 1, 0.1), 1),     # Tq = 0: dk still needed
    ((P,) * 9 + (0, 4, 2, 8, 8, 64, 1, 0.1), 0),                    # empty batch
    ((P,) * 9 + (2, 4, 2, 0, 0, 64, 0, 0.1), 0),                    # no rows, no keys
    ((FAKE,) * 9 + (1, 1, 1, (1 << 31) // 512 + 1, 8, 128, 1, 0.1), 2),   # plane over 2^31 bytes
    ((FAKE,) * 9 + (1 << 20, 1 << 10, 1, 256, 8, 64, 0, 0.1), 2),  # grid overflow
], ids=lambda a: "case" if isinstance(a, tuple) else str(a))
def test_bwd_validation(lib, args, status):
    assert lib.fa_bwd(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # (q, kc, vc, seqlens, o, B, Hq, Hkv, Tk_max, d, num_splits)
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, 32, 4), 3),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 3, 64, 128, 4), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, 128, -1), 2),
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, -5, 128, 4), 2),
    ((FAKE, FAKE, FAKE, P, FAKE, 2, 8, 2, 64, 128, 4), 1),          # seqlens NULL
    ((FAKE, P, FAKE, FAKE, FAKE, 2, 8, 2, 64, 128, 4), 1),          # kcache NULL
    ((P, FAKE, FAKE, FAKE, FAKE, 2, 8, 2, 64, 128, 4), 1),
    ((P, P, P, P, P, 0, 8, 2, 64, 128, 4), 0),                      # empty batch
    ((FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 28, 8, 2, 64, 128, 4), 2), # B*Hq merge grid overflow
])
def test_decode_validation(lib, args, status):
    assert lib.fa_decode(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # (q, kc, vc, ks, vs, seqlens, o, B, Hq, Hkv, Tk_max, d, num_splits)
    ((FAKE,) * 7 + (2, 8, 2, 64, 32, 4), 3),
    ((FAKE,) * 7 + (2, 8, 3, 64, 128, 4), 2),
    ((FAKE,) * 7 + (2, 8, 2, 64, 128, -1), 2),
    ((FAKE, FAKE, FAKE, P, FAKE, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # kscale NULL
    ((FAKE, FAKE, FAKE, FAKE, P, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # vscale NULL
    ((FAKE, FAKE, FAKE, FAKE, FAKE, P, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # seqlens NULL
    ((FAKE, P, FAKE, FAKE, FAKE, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # kcache NULL
    ((P,) * 7 + (0, 8, 2, 64, 128, 4), 0),                                  # empty batch
    ((FAKE,) * 7 + (1 << 28, 8, 2, 64, 128, 4), 2),
])
def test_decode_fp8_validation(lib, args, status):
    assert lib.fa_decode_fp8(*args, None) == status


@pytest.mark.parametrize("args,status", [
    # (q, kc, vc, ks, vs, seqlens, o, B, Hq, Hkv, Tk_max, d, num_splits)
    ((FAKE,) * 7 + (2, 8, 2, 64, 32, 4), 3),
    ((FAKE,) * 7 + (2, 8, 3, 64, 128, 4), 2),
    ((FAKE,) * 7 + (2, 8, 2, 64, 128, -1), 2),
    ((FAKE, FAKE, FAKE, P, FAKE, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # kscale NULL
    ((FAKE, FAKE, FAKE, FAKE, P, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # vscale NULL
    ((FAKE, FAKE, FAKE, FAKE, FAKE, P, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # seqlens NULL
    ((FAKE, FAKE, P, FAKE, FAKE, FAKE, FAKE) + (2, 8, 2, 64, 128, 4), 1),   # vcache NULL
    ((P,) * 7 + (0, 8, 2, 64, 128, 4), 0),                                  # empty batch
    ((FAKE,) * 7 + (1 << 28, 8, 2, 64, 128, 4), 2),
])
def test_decode_int8_validation(lib, args, status):
    assert lib.fa_decode_int8(*args, None) == status


def test_decode_int8_workgroup_planning(lib):
    assert lib.fa_decode_int8_workgroups(16, 32, 8, 32768, 128, 16) == 16
    assert lib.fa_decode_int8_workgroups(16, 30, 8, 32768, 128, 16) == -fa.STATUS_CODES["FA_ERR_SHAPE"]
    assert lib.fa_decode_int8_workgroups(16, 32, 8, 32768, 96, 16) == -fa.STATUS_CODES["FA_ERR_UNSUPPORTED"]


def test_decode_workgroup_planning(lib):
    # An explicit count is used as given, capped at 2^20; bad shapes give
    # minus the status code.  (The automatic choice needs a device and is
    # covered by the GPU tests.)
    assert lib.fa_decode_workgroups(16, 32, 8, 32768, 128, 16) == 16
    assert lib.fa_decode_workgroups(16, 32, 8, 32768, 128, 7) == 7
    assert lib.fa_decode_workgroups(16, 32, 8, 32768, 128, 1 << 30) == 1 << 20
    assert lib.fa_decode_workgroups(1, 1, 1, 0, 64, 3) == 3
    assert lib.fa_decode_workgroups(16, 30, 8, 32768, 128, 16) == -fa.STATUS_CODES["FA_ERR_SHAPE"]
    assert lib.fa_decode_workgroups(16, 32, 8, 32768, 96, 16) == -fa.STATUS_CODES["FA_ERR_UNSUPPORTED"]
    assert lib.fa_decode_workgroups(16, 32, 8, 32768, 128, -1) == -fa.STATUS_CODES["FA_ERR_SHAPE"]


def test_read_probe_validation(lib):
    # (src, bytes, sink): checked before any launch.
    assert lib.fa_read_probe(FAKE, 17, FAKE, None) == fa.STATUS_CODES["FA_ERR_SHAPE"]
    assert lib.fa_read_probe(None, 1024, FAKE, None) == fa.STATUS_CODES["FA_ERR_NULL"]
    assert lib.fa_read_probe(FAKE, 1024, None, None) == fa.STATUS_CODES["FA_ERR_NULL"]
    assert lib.fa_read_probe(None, 0, None, None) == fa.STATUS_CODES["FA_OK"]


def test_strerror(lib):
    for st in range(7):
        assert fa.fa_strerror(st)
    assert fa.fa_strerror(99) == "unknown status"
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 2, 8, 8, 96, True, 0.1)
    assert e.value.status == 3
