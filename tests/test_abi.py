"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the header declares, the parameter struct has the same
layout in C and in the binding, and every argument error returns its status
before any HIP call (fake device pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import subquadratic_attention_amd as sqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sqa.LIB_PATH):
        from subquadratic_attention_amd import build

        build.build()
    return sqa.load_library()


def header_functions():
    src = open(sqa.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lizard_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for want in ("lizard_attn_fwd", "lizard_attn_bwd", "lizard_attn_bwd_workspace_size", "lizard_decode_step",
                 "lizard_attn_fwd_logit", "lizard_attn_bwd_logit", "lizard_decode_step_logit",
                 "lizard_decode_tokens", "lizard_decode_tokens_logit", "lizard_attn_fwd_continue",
                 "lizard_softmax_attn_fwd", "lizard_transfer_loss", "lizard_attn_fwd_split",
                 "lizard_attn_fwd_split_workspace_size", "lizard_attn_fwd_train", "lizard_attn_bwd_train",
                 "lizard_attn_chunk_states_size",
                 "lizard_status_string", "lizard_abi_version"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sqa.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\b[TW] (\w+)$", out.stdout, flags=re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else leaks out under the library's prefix
    assert {n for n in exported if n.startswith("lizard_")} == set(header_functions())


def test_param_struct_layout_matches_c(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "lizard_attn.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(lizard_params_t), offsetof(lizard_params_t, n_meta),"
        " offsetof(lizard_params_t, alpha), offsetof(lizard_params_t, softmax_scale), offsetof(lizard_params_t, dtype));"
        "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    c_vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    P = sqa.LizardParams
    py_vals = [ctypes.sizeof(P), P.n_meta.offset, P.alpha.offset, P.softmax_scale.offset, P.dtype.offset]
    assert c_vals == py_vals


def test_version_and_strings(lib):
    assert lib.lizard_abi_version() == 4
    for code, name in sqa.STATUS.items():
        s = lib.lizard_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.lizard_status_string(123) == b"unknown status"


FAKE = 0x10000  # aligned, never dereferenced
MIS = 0x10008   # 8-byte aligned only


def params(**kw):
    base = dict(B=2, H=3, L=128, d=128, window=64, n_meta=4, alpha=0.5, dtype=sqa.LIZARD_BF16)
    base.update(kw)
    d = base.pop("d")
    return sqa.make_params(base.pop("B"), base.pop("H"), base.pop("L"), d, **base)


def fwd(lib, p, q=FAKE, meta=FAKE, lse=None):
    return lib.lizard_attn_fwd(ctypes.byref(p), q, FAKE, FAKE, FAKE, meta, FAKE, lse, None, None, None)


def bwd(lib, p, ws=FAKE, ws_bytes=1 << 40, dy=FAKE):
    return lib.lizard_attn_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dy, FAKE, FAKE, FAKE, FAKE, FAKE,
                               ws, ws_bytes, None)


def dec(lib, p, pos=5, state=FAKE):
    return lib.lizard_decode_step(ctypes.byref(p), pos, FAKE, FAKE, FAKE, FAKE, FAKE, state, FAKE, FAKE, FAKE, None)


S = sqa.STATUS_CODE


def test_null_params(lib):
    assert lib.lizard_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None) == S["LIZARD_E_NULL"]
    assert lib.lizard_attn_bwd_workspace_size(None) == 0


@pytest.mark.parametrize("call", ["fwd", "bwd", "dec"])
def test_argument_errors(lib, call):
    f = {"fwd": fwd, "bwd": bwd, "dec": dec}[call]
    assert f(lib, params(dtype=7)) == S["LIZARD_E_DTYPE"]
    assert f(lib, params(B=-1)) == S["LIZARD_E_SHAPE"]
    assert f(lib, params(window=0)) == S["LIZARD_E_SHAPE"]
    assert f(lib, params(n_meta=-2)) == S["LIZARD_E_SHAPE"]
    assert f(lib, params(alpha=float("nan"))) == S["LIZARD_E_SHAPE"]
    assert f(lib, params(softmax_scale=-1.0)) == S["LIZARD_E_SHAPE"]
    assert f(lib, params(d=96)) == S["LIZARD_E_UNSUPPORTED"]
    assert f(lib, params(d=128, dtype=sqa.LIZARD_F32)) == S["LIZARD_E_UNSUPPORTED"]
    assert f(lib, params(window=65)) == S["LIZARD_E_UNSUPPORTED"]
    assert f(lib, params(n_meta=17)) == S["LIZARD_E_UNSUPPORTED"]
    assert f(lib, params(chunk=32)) == S["LIZARD_E_UNSUPPORTED"]
    p = params()
    p.dv = 64
    assert f(lib, p) == S["LIZARD_E_UNSUPPORTED"]


def test_fwd_pointer_errors(lib):
    assert fwd(lib, params(), q=None) == S["LIZARD_E_NULL"]
    assert fwd(lib, params(n_meta=4), meta=None) == S["LIZARD_E_NULL"]
    assert fwd(lib, params(), q=MIS) == S["LIZARD_E_ALIGN"]
    assert fwd(lib, params(), lse=MIS) == S["LIZARD_E_ALIGN"]
    assert fwd(lib, params(L=-5)) == S["LIZARD_E_SHAPE"]


def test_sequence_length_limit(lib):
    """L above 2^26 is refused before any launch; at the limit, row offsets
    of up to L * d elements are formed in 64-bit arithmetic in the kernels
    (here only the check is exercised: a misaligned q makes the call return
    before anything is launched, so the fake pointers are never read)."""
    assert fwd(lib, params(L=(1 << 26) + 1)) == S["LIZARD_E_SHAPE"]
    assert fwd(lib, params(L=1 << 26), q=MIS) == S["LIZARD_E_ALIGN"]
    assert bwd(lib, params(L=(1 << 26) + 1)) == S["LIZARD_E_SHAPE"]
    assert lib.lizard_attn_bwd_workspace_size(ctypes.byref(params(L=(1 << 26) + 1))) == 0


def test_bwd_workspace_checks(lib):
    p = params()
    need = lib.lizard_attn_bwd_workspace_size(ctypes.byref(p))
    if need > 0:
        assert bwd(lib, p, ws_bytes=need - 1) == S["LIZARD_E_WORKSPACE"]
        assert bwd(lib, p, ws=None) == S["LIZARD_E_WORKSPACE"]
    assert bwd(lib, p, dy=None) == S["LIZARD_E_NULL"]
    assert bwd(lib, p, ws=MIS) == S["LIZARD_E_ALIGN"]


def test_decode_errors(lib):
    assert dec(lib, params(), pos=-1) == S["LIZARD_E_SHAPE"]
    assert dec(lib, params(), state=None) == S["LIZARD_E_NULL"]
    assert dec(lib, params(), state=MIS) == S["LIZARD_E_ALIGN"]


def test_empty_calls_do_nothing(lib):
    # B*H == 0: valid, nothing to launch, the fake pointers are never touched
    assert fwd(lib, params(B=0)) == 0
    assert dec(lib, params(H=0)) == 0


def test_binding_refuses_without_library(tmp_path):
    mod = sqa
    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(ImportError):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def test_logit_entry_points_check_their_gate_argument(lib):
    """The *_logit calls run the same checks; their gate pointer is the
    logits (a NULL or misaligned one is caught before any launch)."""
    p = params()
    f = lambda x: lib.lizard_attn_fwd_logit(ctypes.byref(p), FAKE, FAKE, FAKE, x, FAKE, FAKE, None, None, None, None)
    assert f(None) == S["LIZARD_E_NULL"]
    assert f(MIS) == S["LIZARD_E_ALIGN"]
    b = lambda x, dx: lib.lizard_attn_bwd_logit(ctypes.byref(p), FAKE, FAKE, FAKE, x, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, dx, FAKE, FAKE, 1 << 40, None)
    assert b(None, FAKE) == S["LIZARD_E_NULL"]
    assert b(FAKE, None) == S["LIZARD_E_NULL"]
    assert b(FAKE, MIS) == S["LIZARD_E_ALIGN"]
    dec_ = lambda x: lib.lizard_decode_step_logit(ctypes.byref(p), 3, FAKE, FAKE, FAKE, x, FAKE, FAKE, FAKE, FAKE,
                                                   FAKE, None)
    assert dec_(None) == S["LIZARD_E_NULL"]
    assert dec_(MIS) == S["LIZARD_E_ALIGN"]
    assert lib.lizard_attn_fwd_logit(ctypes.byref(params(dtype=7)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                      None, None) == S["LIZARD_E_DTYPE"]


def test_decode_tokens_checks(lib):
    """Token count and position-array checks of the serving decode."""
    p = params()
    f = lambda pos, T, st=FAKE: lib.lizard_decode_tokens(ctypes.byref(p), pos, T, FAKE, FAKE, FAKE, FAKE, FAKE, st,
                                                          FAKE, FAKE, FAKE, None)
    assert f(None, 1) == S["LIZARD_E_NULL"]
    assert f(FAKE, 0) == S["LIZARD_E_SHAPE"]
    assert f(FAKE, -3) == S["LIZARD_E_SHAPE"]
    assert f(FAKE, (1 << 16) + 1) == S["LIZARD_E_SHAPE"]
    assert f(FAKE + 4, 2) == S["LIZARD_E_ALIGN"]
    assert f(FAKE, 2, st=MIS) == S["LIZARD_E_ALIGN"]
    pe = params(B=0)
    assert lib.lizard_decode_tokens(ctypes.byref(pe), None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    None) == 0


def test_continue_checks(lib):
    p = params(window=16)
    f = lambda lg, xg, hl, kh=FAKE, vh=FAKE, si=FAKE: lib.lizard_attn_fwd_continue(
        ctypes.byref(p), FAKE, FAKE, FAKE, lg, xg, FAKE, si, kh, vh, hl, FAKE, None, None, None, None)
    assert f(FAKE, FAKE, 0) == S["LIZARD_E_SHAPE"]          # both gate forms
    assert f(None, None, 0) == S["LIZARD_E_NULL"]           # neither
    assert f(FAKE, None, 16) == S["LIZARD_E_SHAPE"]         # halo longer than window - 1
    assert f(FAKE, None, -1) == S["LIZARD_E_SHAPE"]
    assert f(FAKE, None, 3, kh=None) == S["LIZARD_E_NULL"]
    assert f(FAKE, None, 3, vh=MIS) == S["LIZARD_E_ALIGN"]
    assert f(FAKE, None, 0, si=MIS) == S["LIZARD_E_ALIGN"]


def test_split_checks(lib):
    """The split forward: its workspace size (0 where one pass fills the chip
    or the sequence is short) and the workspace checks, before any launch."""
    long_ = params(B=1, H=32, L=32768, window=64)
    need = lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(long_))
    # 4 segments of 128 chunks: states, totals, per-chunk sums, transposed incoming states, live ends
    assert need == 32 * 4 * 128 * 128 * 4 + 32 * 4 * 128 * 4 + 32 * 512 * 128 * 4 + 32 * 4 * 128 * 128 * 2 + 512
    assert lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(params(B=4, H=32, L=4096))) == 0
    assert lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(params(B=1, H=1, L=960))) == 0   # 15 chunks
    assert lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(params(B=1, H=1, L=1024))) > 0
    assert lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(params(dtype=7))) == 0
    f = lambda p, ws, nb, lg=FAKE, xg=None: lib.lizard_attn_fwd_split(
        ctypes.byref(p), FAKE, FAKE, FAKE, lg, xg, FAKE, None, None, None, 0, FAKE, None, None, None, ws, nb, None)
    assert f(long_, FAKE, need - 1) == S["LIZARD_E_WORKSPACE"]
    assert f(long_, None, need) == S["LIZARD_E_WORKSPACE"]
    assert f(long_, MIS, need) == S["LIZARD_E_ALIGN"]
    assert f(long_, FAKE, need, lg=FAKE, xg=FAKE) == S["LIZARD_E_SHAPE"]
    assert f(params(B=0), None, 0) == 0


def test_train_entry_points_check_their_arguments(lib):
    """The training forward and backward: the chunk-states size and the
    checks of the saved states and gate arguments, before any launch."""
    p = params(B=2, H=3, L=130, d=128)
    assert lib.lizard_attn_chunk_states_size(ctypes.byref(p)) == 2 * 3 * 3 * 128 * 128 * 2
    assert lib.lizard_attn_chunk_states_size(ctypes.byref(params(dtype=7))) == 0
    fw = lambda cs, lg=FAKE, xg=None: lib.lizard_attn_fwd_train(ctypes.byref(p), FAKE, FAKE, FAKE, lg, xg, FAKE, FAKE,
                                                              FAKE, None, None, cs, None)
    assert fw(None) == S["LIZARD_E_NULL"]
    assert fw(MIS) == S["LIZARD_E_ALIGN"]
    assert fw(FAKE, lg=FAKE, xg=FAKE) == S["LIZARD_E_SHAPE"]
    assert fw(FAKE, lg=None, xg=None) == S["LIZARD_E_NULL"]
    bw = lambda cs, ws=FAKE, nb=1 << 40: lib.lizard_attn_bwd_train(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                                                   FAKE, cs, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nb,
                                                                   None)
    assert bw(None) == S["LIZARD_E_NULL"]
    assert bw(MIS) == S["LIZARD_E_ALIGN"]
    need = lib.lizard_attn_bwd_workspace_size(ctypes.byref(p))
    assert bw(FAKE, nb=need - 1) == S["LIZARD_E_WORKSPACE"]
    pe = params(B=0)
    assert lib.lizard_attn_fwd_train(ctypes.byref(pe), None, None, None, FAKE, None, FAKE, None, None, None, None,
                                     None, None) == 0
