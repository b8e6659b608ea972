"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before any GPU work (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "routing_permute_grouped_moe_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_layer_calls():
    names = set(declared())
    for n in ["moe_route", "moe_route_bwd", "moe_permute", "moe_permute_bwd",
              "moe_grouped_gemm_fwd", "moe_grouped_gemm_bwd_dx", "moe_grouped_gemm_bwd_dw",
              "moe_unpermute_combine", "moe_unpermute_combine_bwd", "moe_router_logits",
              "moe_router_logits_bwd"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from routing_permute_grouped_moe_amd import abi
    assert sorted(abi.EXPORTED) == declared()


@pytest.fixture(scope="module")
def abi():
    from routing_permute_grouped_moe_amd import abi as a
    return a


FAKE = 0x10000        # an aligned address that is never dereferenced on these paths
FAKE_ODD = 0x10002


def status(abi, name, *args):
    return getattr(abi._lib, name)(*args)


def test_status_strings(abi):
    assert abi.moe_status_string(0) == "ok"
    assert abi.moe_status_string(3) == "workspace too small"
    assert abi.moe_abi_version() >= 1


def test_route_rejects_bad_k_and_e(abi):
    assert status(abi, "moe_route", FAKE, 4, 8, 9, FAKE, FAKE, None) == abi.MOE_ERR_UNSUPPORTED
    assert "k = 9" in abi.moe_last_error()
    assert status(abi, "moe_route", FAKE, 4, 8, 0, FAKE, FAKE, None) == abi.MOE_ERR_UNSUPPORTED
    assert status(abi, "moe_route", FAKE, 4, 2000, 2, FAKE, FAKE, None) == abi.MOE_ERR_UNSUPPORTED
    assert "E = 2000" in abi.moe_last_error()


def test_route_rejects_null_and_negative(abi):
    assert status(abi, "moe_route", None, 4, 8, 2, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert "logits is NULL" in abi.moe_last_error()
    assert status(abi, "moe_route", FAKE, -1, 8, 2, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_noop(abi):
    assert status(abi, "moe_route", None, 0, 8, 2, None, None, None) == abi.MOE_OK
    assert status(abi, "moe_route_bwd", None, None, None, 0, 8, 2, None, None) == abi.MOE_OK
    assert status(abi, "moe_unpermute_combine", None, None, None, None, 1, 0, 128, 2, 0, None,
                  None) == abi.MOE_OK
    assert status(abi, "moe_permute_bwd", None, None, 1, 0, 128, 2, 0, None, None, None,
                  None) == abi.MOE_OK


def test_permute_workspace(abi):
    need = abi.moe_permute_workspace_bytes(100, 8, 2)
    # one int per expert for every rank block of 4096 (token, slot) pairs
    assert need == 4 * 8 * ((100 * 2 + 4095) // 4096)
    assert abi.moe_permute_workspace_bytes(8192, 256, 8) == 4 * 256 * 16
    st = status(abi, "moe_permute", FAKE, 1, FAKE, 100, 128, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE,
                FAKE, need - 4, None)
    assert st == abi.MOE_ERR_WORKSPACE


def test_shape_limits(abi):
    # H not a multiple of 64
    st = status(abi, "moe_unpermute_combine", FAKE, FAKE, FAKE, None, 1, 4, 100, 2, 8, FAKE,
                None)
    assert st == abi.MOE_ERR_UNSUPPORTED
    # misaligned pointer
    st = status(abi, "moe_unpermute_combine", FAKE_ODD, FAKE, FAKE, None, 1, 4, 128, 2, 8, FAKE,
                None)
    assert st == abi.MOE_ERR_INVALID_ARG
    # unknown dtype
    st = status(abi, "moe_unpermute_combine", FAKE, FAKE, FAKE, None, 7, 4, 128, 2, 8, FAKE,
                None)
    assert st == abi.MOE_ERR_INVALID_ARG
    # grouped GEMM: I not a multiple of 64, window beyond 1024 experts
    st = status(abi, "moe_grouped_gemm_fwd", FAKE, FAKE, 0, 8, 64, 1, 128, 96, FAKE, FAKE, FAKE,
                FAKE, FAKE, None, None, 0, None)
    assert st == abi.MOE_ERR_UNSUPPORTED
    st = status(abi, "moe_grouped_gemm_fwd", FAKE, FAKE, 1000, 100, 64, 1, 128, 64, FAKE, FAKE,
                FAKE, FAKE, FAKE, None, None, 0, None)
    # a workspace that is too small
    st2 = status(abi, "moe_grouped_gemm_fwd", FAKE, FAKE, 0, 8, 64, 1, 128, 64, FAKE, FAKE, FAKE,
                 FAKE, FAKE, None, FAKE, 16, None)
    assert st2 == abi.MOE_ERR_WORKSPACE
    assert st == abi.MOE_ERR_UNSUPPORTED
    # a row longer than the row kernels keep in registers
    st = status(abi, "moe_unpermute_combine", FAKE, FAKE, FAKE, None, 0, 4, 16384, 2, 8, FAKE,
                None)
    assert st == abi.MOE_ERR_UNSUPPORTED


def test_load_stats_rejects_bad_arguments(abi):
    st = status(abi, "moe_load_stats", FAKE, 0, 1, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_UNSUPPORTED
    st = status(abi, "moe_load_stats", FAKE, 2048, 1, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_UNSUPPORTED
    st = status(abi, "moe_load_stats", FAKE, 64, 6, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_INVALID_ARG and "does not divide" in abi.moe_last_error()
    st = status(abi, "moe_load_stats", FAKE, 64, 0, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_INVALID_ARG
    st = status(abi, "moe_load_stats", None, 64, 8, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_INVALID_ARG and "counts is NULL" in abi.moe_last_error()
    st = status(abi, "moe_load_stats", FAKE, 64, 8, FAKE_ODD, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_INVALID_ARG


def test_recompute_variant_rejects_bad_arguments(abi):
    # fwd_gather(x, src_token, T, offsets, g0, G, R, dt, H, I, w13, w2, h13, act, yp, sh, ws, wsb, s)
    args = [FAKE, FAKE, 100, FAKE, 0, 4, 600, 1, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None,
            None, 0, None]
    bad = list(args); bad[7] = 0                                  # fp32 storage
    assert status(abi, "moe_grouped_gemm_fwd_gather", *bad) == abi.MOE_ERR_UNSUPPORTED
    bad = list(args); bad[1] = None                               # no src_token
    assert status(abi, "moe_grouped_gemm_fwd_gather", *bad) == abi.MOE_ERR_INVALID_ARG
    bad = list(args); bad[2] = 1 << 20                            # x of 2^20 x 1024 bf16 = 2 GiB
    bad[8] = 1024
    assert status(abi, "moe_grouped_gemm_fwd_gather", *bad) == abi.MOE_ERR_UNSUPPORTED
    # bwd_dw_recompute(x, src, T, h13, act, dyp, dh13, offsets, g0, G, R, dt, H, I, dw13, dw2, ...)
    args = [FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, 600, 1, 256, 128, FAKE, FAKE,
            None, None, 0, None]
    bad = list(args); bad[3] = None                               # no h13 to recompute from
    assert status(abi, "moe_grouped_gemm_bwd_dw_recompute", *bad) == abi.MOE_ERR_INVALID_ARG
    bad = list(args); bad[11] = 0
    assert status(abi, "moe_grouped_gemm_bwd_dw_recompute", *bad) == abi.MOE_ERR_UNSUPPORTED


def test_binding_raises_with_detail(abi):
    with pytest.raises(abi.MoeError) as ei:
        abi.moe_route(FAKE, 4, 8, 9, FAKE, FAKE, stream=0)
    assert ei.value.status == abi.MOE_ERR_UNSUPPORTED
    assert "k = 9" in str(ei.value)


def test_noalloc_permute_size_limit(abi):
    # 4 MiB of rank scratch: T*k = 2^24 pairs at E = 256 fit exactly, one
    # block more does not; the limit is checked on the host before any HIP call
    assert abi.moe_permute_noalloc_max_scratch_bytes() == 4 << 20
    assert abi.moe_permute_workspace_bytes(1 << 21, 256, 8) == 4 << 20
    st = status(abi, "moe_permute_noalloc", FAKE, 1, FAKE, (1 << 21) + 1, 128, 256, 8, FAKE,
                FAKE, FAKE, FAKE, FAKE, None)
    assert st == abi.MOE_ERR_UNSUPPORTED and "moe_permute with a workspace" in abi.moe_last_error()
    # the other host checks still apply
    st = status(abi, "moe_permute_noalloc", FAKE, 1, FAKE, 100, 100, 8, 2, FAKE, FAKE, FAKE,
                FAKE, FAKE, None)
    assert st == abi.MOE_ERR_UNSUPPORTED


def test_router_bwd_rejects_unknown_flags(abi):
    # dlogits, x, dt, wg, T, H, E, dx, dwg, dbias, flags, ws, ws_bytes, stream
    args = [FAKE, FAKE, abi.MOE_BF16, FAKE, 512, 256, 64, FAKE, FAKE, None, 2, FAKE, 1 << 30, None]
    assert status(abi, "moe_router_logits_bwd", *args) == abi.MOE_ERR_INVALID_ARG
    assert "flags" in abi.moe_last_error()
