"""CPU checks of the C ABI: the library loads, exports every entry point that
include/kda.h declares, reports its ABI version, and rejects bad arguments
with KDA_EINVAL before any launch (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "spec_decode_amd", "libkda.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(kda_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("kda_decay", "kda_commit", "kda_verify", "kda_fused_replay_verify",
                 "kda_fused_conv_replay_verify", "kda_gate_projection",
                 "kda_defer_commit", "kda_flush_plan", "kda_last_error", "kda_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    lib.kda_abi_version.restype = ctypes.c_int
    text = open(HEADER).read()
    want = int(re.search(r"#define KDA_ABI_VERSION (\d+)", text).group(1))
    assert lib.kda_abi_version() == want


def _err(lib):
    lib.kda_last_error.restype = ctypes.c_char_p
    return lib.kda_last_error().decode()


def _verify_args(tokens, *, state=None, dtype=0, stride=4 * 128 * 128, rq=8, rows=None,
                 pending=None, gate=None, norm_weight=None, fused=False):
    """kda_verify / kda_fused_replay_verify arguments in declaration order."""
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    args = [ctypes.c_int(4), ctypes.c_int(tokens), ctypes.c_int(2)] + [fake] * 7 + [
        ctypes.c_float(-5.0), ctypes.c_int(dtype), fake if state is None else P(state),
        ctypes.c_int64(stride), fake, ctypes.c_int(0), fake, fake, ctypes.c_int(rq), P(rows)]
    if fused:
        args.append(P(pending))
    args.append(P(None))  # query_start_loc
    if fused:
        args += [P(None), P(None)]  # boundaries, boundary_lens
    return args + [P(gate), P(norm_weight), ctypes.c_float(1e-5), fake, P(None)]


def test_rejects_bad_arguments_without_launch(lib):
    lib.kda_verify.restype = ctypes.c_int
    lib.kda_fused_replay_verify.restype = ctypes.c_int
    assert lib.kda_verify(*_verify_args(9)) == 1
    assert "tokens must be in 1..8" in _err(lib)
    assert lib.kda_verify(*_verify_args(0)) == 1
    assert "tokens must be in 1..8" in _err(lib)

    assert lib.kda_fused_replay_verify(*_verify_args(4, rq=4, fused=True)) == 1
    assert "record_rows and pending are required" in _err(lib)

    # gate without norm_weight
    assert lib.kda_fused_replay_verify(*_verify_args(4, rq=4, rows=0x1000, pending=0x1000,
                                                     gate=0x1000, fused=True)) == 1
    assert "gate and norm_weight" in _err(lib)

    # record_tokens below tokens
    assert lib.kda_fused_replay_verify(*_verify_args(4, rq=3, fused=True)) == 1
    assert "record_tokens" in _err(lib)

    # a misaligned state base
    assert lib.kda_fused_replay_verify(*_verify_args(4, rq=4, rows=0x1000, pending=0x1000,
                                                     state=0x1004, fused=True)) == 1
    assert "16-byte aligned" in _err(lib)

    # an unknown state type; a BF16 slot stride that breaks 16-byte alignment
    assert lib.kda_verify(*_verify_args(4, dtype=2)) == 1
    assert "state_dtype" in _err(lib)
    assert lib.kda_verify(*_verify_args(4, dtype=1, stride=4 * 128 * 128 + 4)) == 1
    assert "state_slot_stride" in _err(lib)

    # a non-finite lower bound
    P = ctypes.c_void_p
    fake = P(0x1000)
    lib.kda_decay.restype = ctypes.c_int
    assert lib.kda_decay(fake, ctypes.c_int64(3), ctypes.c_int(2), fake, fake,
                         ctypes.c_float(float("nan")), fake, P(None)) == 1
    assert "finite" in _err(lib)
    # an element count beyond the 64-bit range (2^56 tokens x 64 heads x 128 channels)
    assert lib.kda_decay(fake, ctypes.c_int64(1 << 56), ctypes.c_int(64), fake, fake,
                         ctypes.c_float(-5.0), fake, P(None)) == 1
    assert "too large" in _err(lib)


def test_conv_entry_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)
    f = lib.kda_fused_conv_replay_verify
    f.restype = ctypes.c_int

    def call(x_stride=3 * 4 * 128, q_scale=128 ** -0.5, strides=(100, 10, 1), x=0x1000,
             tokens=4):
        I64 = ctypes.c_int64
        return f(ctypes.c_int(4), ctypes.c_int(tokens), ctypes.c_int(2), P(x), I64(x_stride),
                 fake, P(None), fake, I64(strides[0]), I64(strides[1]), I64(strides[2]),
                 ctypes.c_float(q_scale), fake, fake, fake, fake, ctypes.c_float(-5.0),
                 ctypes.c_int(0), fake, I64(4 * 128 * 128), fake, ctypes.c_int(0), fake, fake,
                 ctypes.c_int(4), fake, fake, P(None), P(None), P(None), P(None),
                 ctypes.c_float(1e-5), fake, P(None))

    assert call(x_stride=3 * 4 * 128 - 1) == 1 and "x_row_stride" in _err(lib)
    assert call(q_scale=float("inf")) == 1 and "q_scale" in _err(lib)
    assert call(strides=(100, 0, 1)) == 1 and "strides" in _err(lib)
    assert call(x=0) == 1 and "null pointer" in _err(lib)
    assert call(tokens=9) == 1 and "tokens" in _err(lib)


def test_gate_projection_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    f = lib.kda_gate_projection
    f.restype = ctypes.c_int
    I64 = ctypes.c_int64

    def call(tokens=10, heads=2, stride=136, fa=0x1000, fb=0x2000, out=0x3000):
        return f(I64(tokens), ctypes.c_int(heads), P(fa), I64(stride), P(fb), P(out), P(None))

    assert call(stride=100) == 1 and "f_a_row_stride" in _err(lib)
    assert call(stride=130) == 1 and "f_a_row_stride" in _err(lib)
    assert call(heads=0) == 1 and "heads" in _err(lib)
    assert call(tokens=-1) == 1 and "tokens" in _err(lib)
    assert call(fa=0x1008) == 1 and "aligned" in _err(lib)
    assert call(out=0) == 1 and "null" in _err(lib)
    assert call(tokens=0, fa=0, fb=0, out=0) == 0


def test_commit_rejects_bad_tables(lib):
    lib.kda_commit.restype = ctypes.c_int
    P = ctypes.c_void_p
    fake = P(0x1000)
    U64 = ctypes.c_uint64 * 1
    I64 = ctypes.c_int64 * 1

    def call(window=4, stride=2 * 128 * 128, bnd=None, blen=None, addr=0x2000, dtype=1):
        return lib.kda_commit(ctypes.c_int(1), ctypes.c_int(2), ctypes.c_int(window),
                              ctypes.c_int(3), ctypes.c_int(dtype), U64(addr), I64(stride),
                              U64(0x3000), I64(2 * window * 128), U64(0x4000),
                              I64(2 * window * 256), fake, fake, fake, fake, fake,
                              P(bnd), P(blen), P(None), ctypes.c_float(-5.0), ctypes.c_int(0),
                              P(None))

    assert call(window=9) == 1 and "window" in _err(lib)
    assert call(window=0) == 1 and "window" in _err(lib)
    assert call(stride=100) == 1 and "slot stride" in _err(lib)
    assert call(stride=2 * 128 * 128 + 3) == 1 and "slot stride" in _err(lib)
    assert call(bnd=0x5000) == 1 and "together" in _err(lib)
    assert call(addr=0x2008) == 1 and "16-byte aligned" in _err(lib)
    assert call(dtype=7) == 1 and "state_dtype" in _err(lib)


def test_zero_batch_is_a_no_op(lib):
    P = ctypes.c_void_p
    lib.kda_defer_commit.restype = ctypes.c_int
    assert lib.kda_defer_commit(ctypes.c_int(0), P(None), P(None), P(None), P(None), P(None),
                                ctypes.c_int(0), P(None)) == 0
    assert _err(lib) == ""
    lib.kda_flush_plan.restype = ctypes.c_int
    assert lib.kda_flush_plan(ctypes.c_int(0), ctypes.c_int(4), *([P(None)] * 7),
                              ctypes.c_int(0), P(None)) == 0
    # The window length is checked before the batch shortcut.
    for bad in (0, 9):
        assert lib.kda_flush_plan(ctypes.c_int(0), ctypes.c_int(bad), *([P(None)] * 7),
                                  ctypes.c_int(0), P(None)) == 1
        assert "spec_query_len" in _err(lib)
    assert lib.kda_flush_plan(ctypes.c_int(-1), ctypes.c_int(4), *([P(None)] * 7),
                              ctypes.c_int(0), P(None)) == 1
    assert "batch" in _err(lib)


def test_binding_rejects_short_per_request_arrays(lib):
    """The binding checks per-request array lengths on the host: a tensor
    shorter than the batch would be read past its end by the kernels."""
    import torch
    import spec_decode_amd as kda
    B = 4
    i32 = lambda n: torch.zeros(n, dtype=torch.int32)
    base = dict(heads=1, tokens=2, batch=B, q=None, k=None, v=None, raw_g=None, raw_beta=None,
                a_log=None, dt_bias=None, lower_bound=-5.0, state=None, state_slot_stride=0,
                corr=None, kg=None, record_tokens=2, out=None)
    with pytest.raises(ValueError, match="boundaries"):
        kda.kda_fused_replay_verify(state_indices=i32(B), record_rows=i32(B), pending=i32(B),
                                    boundaries=i32(B - 1), boundary_lens=i32(B), **base)
    with pytest.raises(ValueError, match="query_start_loc"):
        kda.kda_verify(state_indices=i32(B), query_start_loc=i32(B), **base)
    with pytest.raises(ValueError, match="state_indices"):
        kda.kda_defer_commit(batch=B, state_indices=i32(B - 2), commit_lens=i32(B),
                             record_rows=i32(B), pending=i32(B))


def test_product_path_is_independent_of_the_oracle():
    """The binding and the HIP sources never load or name the oracle, and the
    oracle never names the HIP library: the two share no code (only the seeded
    input generators in workloads/ serve both)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import spec_decode_amd; "
            "print('oracle' in sys.modules, any(m.startswith('oracle') for m in sys.modules))"
            % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.split() == ["False", "False"], out.stdout
    imports = re.compile(r"^\s*(import|from)\s+(\w+)", re.M)
    pkg = os.path.join(ROOT, "spec_decode_amd")
    for base, _, files in os.walk(pkg):
        if "_build" in base:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(base, f)).read()
                assert "oracle" not in {m[1] for m in imports.findall(text)}, f
                assert "kda_o_" not in text and "libkda_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "spec_decode_amd" not in {m[1] for m in imports.findall(text)}, f
            assert "libkda.so" not in text, f


def test_build_scripts_load_without_the_built_library():
    """build() must work on a fresh checkout, where libkda.so does not exist yet:
    it loads the two build scripts by path and never imports the package (whose
    __init__ refuses to load without the library) before compiling."""
    import subprocess
    import sys

    code = (
        "import os, sys\n"
        "sys.path.insert(0, %r)\n"
        "import __graft_entry__ as g\n"
        "m = g._load_script(os.path.join(%r, 'spec_decode_amd', 'build.py'), '_b1')\n"
        "o = g._load_script(os.path.join(%r, 'oracle', 'build.py'), '_b2')\n"
        "assert callable(m.build) and callable(o.build)\n"
        "assert 'spec_decode_amd' not in sys.modules, 'package imported before the build'\n"
        "assert m.LIB.endswith('libkda.so') and o.LIB.endswith('libkda_oracle.so')\n"
    ) % (ROOT, ROOT, ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
