"""C ABI checks that need no GPU: the library loads, exports every function
include/mla_decode.h declares, and rejects bad arguments with the documented
status codes before anything reaches the device."""
import ctypes
import os
import re
import subprocess

import pytest

import mla_decode_attention_split_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")
CEILING_HEADER = os.path.join(ROOT, "include", "mla_ceiling.h")
CEILING_LIB = os.path.join(os.path.dirname(mla.library_path()), "libmla_ceiling.so")

# The documented entry points of each library: the boundary's two calls, their
# sizing helpers and override hook, the split halves of the decode, the decode
# without a workspace argument, and the status helpers.
DECODE_API = {"mla_status_string", "mla_last_error", "mla_metadata_shape", "mla_tile_shape",
              "mla_get_metadata", "mla_get_metadata_ex", "mla_workspace_bytes", "mla_decode",
              "mla_decode_splitkv", "mla_decode_combine", "mla_decode_noalloc"}
CEILING_API = {"mla_ceiling_stream", "mla_ceiling_mfma", "mla_ceiling_last_error"}


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def header_constants():
    return dict((k, int(v)) for k, v in re.findall(r"#define\s+(MLA_[A-Z_]+)\s+\(?(-?\d+)\)?",
                                                   open(HEADER).read()))


def exported_symbols(lib_path):
    """Names of the global functions a shared library defines (nm -D)."""
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}


def test_headers_declare_the_documented_api():
    assert set(header_functions(HEADER)) == DECODE_API
    assert set(header_functions(CEILING_HEADER)) == CEILING_API


def test_library_exports_exactly_the_declared_symbols():
    exported = {n for n in exported_symbols(mla.library_path()) if n.startswith("mla_")}
    assert exported == DECODE_API, exported ^ DECODE_API
    lib = ctypes.CDLL(mla.library_path())
    for name in header_functions(HEADER):
        assert hasattr(lib, name), name


def test_ceiling_library_is_separate():
    exported = {n for n in exported_symbols(CEILING_LIB) if n.startswith("mla_")}
    assert exported == CEILING_API, exported ^ CEILING_API
    assert not (exported_symbols(mla.library_path()) & CEILING_API)


def test_status_strings():
    lib = mla._load()
    c = header_constants()
    assert lib.mla_status_string(c["MLA_OK"]) == b"ok"
    assert b"workspace" in lib.mla_status_string(c["MLA_ERR_WORKSPACE"])
    assert lib.mla_status_string(12345) == b"unknown status"


def test_workspace_size_formula():
    lib = mla._load()
    # (batch + num_parts) pieces x h_kv x rows x (512 16-bit values + one fp32 lse, 256-B aligned)
    n = lib.mla_workspace_bytes(32, 16, 1, 256, 512)
    rows = (32 + 256) * 16
    assert n == rows * 512 * 2 + ((rows * 4 + 255) // 256) * 256
    assert lib.mla_workspace_bytes(0, 16, 1, 256, 512) == 0
    assert lib.mla_workspace_bytes(4, 0, 1, 256, 512) == 0
    assert lib.mla_workspace_bytes(4, 16, 1, 0, 512) == 0
    assert lib.mla_workspace_bytes(4, 16, 1, 256, 256) == 0


def test_tile_shape_needs_no_device():
    """mla_tile_shape is pure host arithmetic: 16/32/64-row tiles up to 64 rows
    per KV head, 128-row tiles above with one KV head (64-row tiles with
    several); the default cost is one stage per 32 tile rows plus one, and at
    least 3."""
    for M, h_kv, tr in [(1, 1, 16), (16, 1, 16), (17, 1, 32), (32, 1, 32), (33, 1, 64), (64, 1, 64),
                        (65, 1, 128), (256, 1, 128), (4096, 1, 128), (16, 2, 16), (64, 2, 64),
                        (65, 2, 64), (256, 4, 64), (4096, 2, 64)]:
        tile, m_tiles, fixed = mla.mla_tile_shape(M, h_kv)
        assert (tile, m_tiles, fixed) == (tr, (M + tr - 1) // tr, max(3, (tr + 31) // 32 + 1))
    with pytest.raises(mla.MlaError):
        mla.mla_tile_shape(0, 1)
    with pytest.raises(mla.MlaError):
        mla.mla_tile_shape(4097, 1)


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
    bad, unsup = c["MLA_ERR_INVALID_ARG"], c["MLA_ERR_UNSUPPORTED"]
    assert lib.mla_get_metadata(FAKE, 0, 16, 1, FAKE, FAKE, None) == bad
    assert lib.mla_get_metadata(None, 4, 16, 1, FAKE, FAKE, None) == bad
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, None, FAKE, None) == bad
    assert lib.mla_get_metadata(FAKE, 4, 0, 1, FAKE, FAKE, None) == unsup
    assert lib.mla_get_metadata(FAKE, 4, 16, 1, FAKE + 4, FAKE, None) == bad
    assert lib.mla_get_metadata_ex(FAKE, 4, 16, 1, FAKE, FAKE, None, -1, 0) == bad
    assert lib.mla_get_metadata_ex(FAKE, 4, 16, 1, FAKE, FAKE, None, 65537, 0) == bad
    assert lib.mla_get_metadata_ex(FAKE, 4, 16, 1, FAKE, FAKE, None, 8, -1) == bad
    assert lib.mla_metadata_shape(0, 16, 1, None, None) == bad
    assert lib.mla_metadata_shape(4, 4097, 1, None, None) == unsup


def test_binding_rejects_wrong_value_dim():
    with pytest.raises(mla.MlaError):
        mla.flash_mla_with_kvcache(None, None, None, None, 256, None, None)


def test_ceiling_helpers_reject_bad_arguments():
    """The measurement probes check their arguments on the host (no GPU call)."""
    lib = ctypes.CDLL(CEILING_LIB)
    p, i = ctypes.c_void_p, ctypes.c_int
    lib.mla_ceiling_stream.argtypes = [p, i, i, p, i, i, p, p]
    lib.mla_ceiling_mfma.argtypes = [p, i, i, i, p]
    bad = header_constants()["MLA_ERR_INVALID_ARG"]
    page = 64 * 1152
    assert lib.mla_ceiling_stream(None, 8, page, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page // 2, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, (1 << 31) // page + 1, page, FAKE, 4, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page, FAKE, 0, 2, FAKE, None) == bad
    assert lib.mla_ceiling_stream(FAKE, 8, page, FAKE, 4, 0, FAKE, None) == bad
    assert lib.mla_ceiling_mfma(None, 4, 10, 0, None) == bad
    assert lib.mla_ceiling_mfma(FAKE, 0, 10, 0, None) == bad
    assert lib.mla_ceiling_mfma(FAKE, 4, 0, 0, None) == bad
    assert lib.mla_ceiling_mfma(FAKE, 4, 10, 2, None) == bad
