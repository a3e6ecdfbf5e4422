"""C ABI checks that need no GPU: the library loads, exports every function
include/mla_decode.h declares, and rejects bad arguments with the documented
status codes before anything reaches the device."""
import ctypes
import os
import re

import pytest

import mla_decode_attention_split_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def header_constants():
    return dict((k, int(v)) for k, v in re.findall(r"#define\s+(MLA_[A-Z_]+)\s+\(?(-?\d+)\)?",
                                                   open(HEADER).read()))


def test_header_declares_the_two_calls_and_helpers():
    names = header_functions()
    for n in ("mla_get_metadata", "mla_decode", "mla_get_metadata_shape",
              "mla_decode_workspace_size", "mla_status_string", "mla_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mla.library_path())
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = mla._load()
    c = header_constants()
    assert lib.mla_status_string(c["MLA_OK"]) == b"ok"
    assert b"workspace" in lib.mla_status_string(c["MLA_ERR_WORKSPACE"])
    assert lib.mla_status_string(12345) == b"unknown status"


def test_workspace_size_formula():
    lib = mla._load()
    # (batch + num_parts) pieces x h_kv x rows x (512 fp32 + one fp32 lse, 256-B aligned)
    n = lib.mla_decode_workspace_size(32, 16, 1, 256)
    rows = (32 + 256) * 16
    assert n == rows * 512 * 4 + ((rows * 4 + 255) // 256) * 256
    assert lib.mla_decode_workspace_size(0, 16, 1, 256) == 0
    assert lib.mla_decode_workspace_size(4, 0, 1, 256) == 0
    assert lib.mla_decode_workspace_size(4, 16, 1, 0) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced: every call below
                # fails argument checks on the host before any HIP call


def decode_call(**over):
    lib = mla._load()
    args = dict(q=FAKE, k=FAKE, bt=FAKE, sl=FAKE, batch=2, s_q=1, h_q=16, h_kv=1, d=576, dv=512,
                dtype=0, num_pages=8, page=64, max_blocks=4, meta=FAKE, num_parts=8, splits=FAKE, causal=0,
                scale=0.0416, out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(over)
    rc = lib.mla_decode(args["q"], args["k"], args["bt"], args["sl"], args["batch"], args["s_q"],
                        args["h_q"], args["h_kv"], args["d"], args["dv"], args["dtype"], args["num_pages"],
                        args["page"], args["max_blocks"], args["meta"], args["num_parts"],
                        args["splits"], args["causal"], args["scale"], args["out"], args["lse"],
                        args["ws"], args["ws_bytes"], args["stream"])
    return rc, lib.mla_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(d=575), "MLA_ERR_UNSUPPORTED"),
    (dict(dv=256), "MLA_ERR_UNSUPPORTED"),
    (dict(page=32), "MLA_ERR_UNSUPPORTED"),
    (dict(dtype=2), "MLA_ERR_UNSUPPORTED"),
    (dict(dtype=-1), "MLA_ERR_UNSUPPORTED"),
    (dict(batch=0), "MLA_ERR_INVALID_ARG"),
    (dict(h_q=16, h_kv=3), "MLA_ERR_INVALID_ARG"),
    (dict(s_q=64, h_q=128), "MLA_ERR_UNSUPPORTED"),
    (dict(q=None), "MLA_ERR_INVALID_ARG"),
    (dict(ws=None), "MLA_ERR_INVALID_ARG"),
    (dict(out=FAKE + 8), "MLA_ERR_INVALID_ARG"),
    (dict(num_parts=0), "MLA_ERR_INVALID_ARG"),
    (dict(scale=float("nan")), "MLA_ERR_INVALID_ARG"),
    (dict(scale=0.0), "MLA_ERR_INVALID_ARG"),
    (dict(scale=-0.0416), "MLA_ERR_INVALID_ARG"),
    (dict(ws_bytes=100), "MLA_ERR_WORKSPACE"),
])
def test_decode_rejects_bad_arguments(over, status):
    rc, msg = decode_call(**over)
    assert rc == header_constants()[status], (rc, msg)
    assert msg


def test_metadata_rejects_bad_arguments():
    lib = mla._load()
    c = header_constants()
    assert lib.mla_get_metadata(FAKE, 0, 16, 1, 8, 2, FAKE, FAKE, None) == c["MLA_ERR_INVALID_ARG"]
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, 0, 2, FAKE, FAKE, None) == c["MLA_ERR_INVALID_ARG"]
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, 8, 0, FAKE, FAKE, None) == c["MLA_ERR_INVALID_ARG"]
    assert lib.mla_get_metadata(None, 4, 16, 1, 8, 2, FAKE, FAKE, None) == c["MLA_ERR_INVALID_ARG"]
    assert lib.mla_get_metadata(FAKE, 4, 0, 1, 8, 2, FAKE, FAKE, None) == c["MLA_ERR_UNSUPPORTED"]
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, 8, 2, FAKE + 4, FAKE, None) == \
        c["MLA_ERR_INVALID_ARG"]


def test_binding_rejects_wrong_value_dim():
    with pytest.raises(mla.MlaError):
        mla.flash_mla_with_kvcache(None, None, None, None, 256, None, None)


def test_ceiling_helpers_reject_bad_arguments():
    """The measurement helpers check their arguments on the host (no GPU call)."""
    lib = mla._load()
    c = header_constants()
    bad = c["MLA_ERR_INVALID_ARG"]
    page = 64 * 1152
    assert lib.mla_ceiling_stream(None, 8, page, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page // 2, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, (1 << 31) // page + 1, page, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page, FAKE, 0, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page, FAKE, 4, 0, FAKE, None) == bad
    assert lib.mla_ceiling_mfma(None, 4, 10, None) == bad
    assert lib.mla_ceiling_mfma(FAKE, 0, 10, None) == bad
    assert lib.mla_ceiling_mfma(FAKE, 4, 0, None) == bad
