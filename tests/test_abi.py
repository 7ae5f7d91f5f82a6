"""The C-ABI library loads and exports every function include/falqon.h
declares, and rejects bad arguments before launching anything (these calls
never reach the GPU, so they run on a host without one)."""
import ctypes
import os
import re

import pytest

import fp8_quantized_lora_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "falqon.h")

EINVAL = 1


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_][a-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ["fp8_quantize", "melded_linear_fwd", "melded_linear_bwd", "adapter_step",
              "rowwise_proxy_update"]:
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(fq.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_call():
    for n in declared_functions():
        if n.startswith("falq_"):
            continue
        assert hasattr(fq, n), n


def test_status_strings_and_version():
    lib = fq.load()
    assert lib.falq_status_string(0) == b"FALQ_OK"
    assert b"EINVAL" in lib.falq_status_string(1)
    assert fq.version().count(".") == 2


def test_workspace_queries():
    assert fq.fp8_quantize_workspace_bytes(1 << 24) >= 8 * 1024
    b = fq.melded_linear_bwd_workspace_bytes(4096, 4096, 4096, 64)
    assert b >= 4096 * 4096                    # at least W~^T for the dX product
    assert fq.melded_linear_bwd_workspace_bytes(0, 512, 512, 16) == 512 * 512
    assert fq.rowwise_proxy_update_workspace_bytes(4096, 4096, 64) >= 4096 * 4
    assert fq.melded_linear_bwd_workspace_bytes(-1, 16, 16, 1) == 0


# Argument errors: FALQ_EINVAL before any launch.  Pointers are fake host
# addresses with the stated alignment; they are never dereferenced.
P = 1 << 20        # a 16-byte aligned fake address
MIS = P + 1        # misaligned


def test_quantize_rejects_bad_arguments():
    lib = fq.load()
    ws = fq.fp8_quantize_workspace_bytes(16)
    assert lib.fp8_quantize(P, 0, -1, None, P, P, None, None, P, ws, None) == EINVAL
    assert lib.fp8_quantize(P, 7, 16, None, P, P, None, None, P, ws, None) == EINVAL      # dtype
    assert lib.fp8_quantize(None, 0, 16, None, P, P, None, None, P, ws, None) == EINVAL   # x null
    assert lib.fp8_quantize(MIS, 0, 16, None, P, P, None, None, P, ws, None) == EINVAL    # align
    assert lib.fp8_quantize(P, 0, 16, None, P, None, None, None, P, ws, None) == EINVAL   # scale
    assert lib.fp8_quantize(P, 0, 16, None, P, P, None, None, P, ws - 1, None) == EINVAL  # short ws
    assert lib.fp8_quantize(P, 0, 16, None, P, P, None, None, MIS, ws, None) == EINVAL    # ws align


def test_linear_rejects_bad_arguments():
    lib = fq.load()
    # d_in not a multiple of 16
    assert lib.melded_linear_fwd(P, P, P, P, 8, 24, 32, P, None) == EINVAL
    assert lib.melded_linear_fwd(P, P, P, P, -1, 32, 32, P, None) == EINVAL
    assert lib.melded_linear_fwd(P, None, P, P, 8, 32, 32, P, None) == EINVAL             # s_x
    assert lib.melded_linear_fwd(P, P, P, P, 8, 32, 32, None, None) == EINVAL             # y
    # more 256 x 256 output tiles than a 32-bit grid holds
    assert lib.melded_linear_fwd(P, P, P, P, 1 << 30, 32, 1 << 30, P, None) == EINVAL
    ws = fq.melded_linear_bwd_workspace_bytes(8, 32, 32, 4)
    args = [P, P, P, P, P, P, P, P, 8, 32, 32, 4, P, P, P, P, ws, None]
    bad_r = list(args); bad_r[11] = -1
    assert lib.melded_linear_bwd(*bad_r) == EINVAL
    short = list(args); short[16] = ws - 1
    assert lib.melded_linear_bwd(*short) == EINVAL
    no_db = list(args); no_db[14] = None
    assert lib.melded_linear_bwd(*no_db) == EINVAL
    assert lib.adapter_step(P, P, P, None, 4, 32, 32, 1e-3, None) == EINVAL               # dB null
    assert lib.adapter_step(P, P, P, P, -4, 32, 32, 1e-3, None) == EINVAL


def test_adamw_rejects_bad_arguments():
    lib = fq.load()
    ok = [P, P, P, P, P, P, P, P, 4, 32, 32, 1e-3, 0.9, 0.999, 1e-8, 0.0, P, None]
    for idx, val in [(3, None), (6, None), (7, MIS), (0, None), (4, None), (8, -1), (16, None),
                     (16, P + 4), (12, 1.0), (13, -0.1), (14, 0.0), (14, float("inf")),
                     (11, float("nan")), (15, float("inf"))]:
        a = list(ok)
        a[idx] = val
        assert lib.adapter_step_adamw(*a) == EINVAL, idx
    # frozen A: A, mA and vA may be null
    frozen = list(ok)
    frozen[0] = frozen[2] = frozen[4] = frozen[5] = None
    a = list(frozen); a[7] = None
    assert lib.adapter_step_adamw(*a) == EINVAL                  # vB is still required


def test_frozen_a_calls_reject_bad_arguments():
    lib = fq.load()
    assert lib.fp8_dequantize(P, None, 16, P, None) == EINVAL
    assert lib.fp8_dequantize(MIS, P, 16, P, None) == EINVAL
    assert lib.fp8_dequantize(P, P, -1, P, None) == EINVAL
    fw = fq.melded_linear_fwd_frozen_a_workspace_bytes(64, 32, 4)
    ok = [P, P, P, P, P, P, 64, 32, 48, 4, P, P, P, fw, None]
    for idx, val in [(4, None), (5, None), (11, None), (11, MIS), (7, 20), (9, -1), (13, fw - 1)]:
        a = list(ok)
        a[idx] = val
        assert lib.melded_linear_fwd_frozen_a(*a) == EINVAL, idx
    bw = fq.melded_linear_bwd_frozen_a_workspace_bytes(64, 32, 48, 4)
    assert bw >= 32 * 48
    ok = [P, P, P, P, P, 64, 32, 48, 4, P, P, P, bw, None]
    for idx, val in [(4, None), (10, None), (1, None), (9, MIS), (12, bw - 1), (6, 17)]:
        a = list(ok)
        a[idx] = val
        assert lib.melded_linear_bwd_frozen_a(*a) == EINVAL, idx


def test_topk_rank_proxy_rejects_bad_arguments():
    lib = fq.load()
    ws = fq.rowwise_proxy_update_topk_rank_workspace_bytes(32, 32, 8, 3)
    assert ws >= fq.rowwise_proxy_update_workspace_bytes(32, 32, 3)
    assert fq.rowwise_proxy_update_topk_rank_workspace_bytes(32, 32, 8, 9) == 0     # k > r
    ok = [P, P, P, P, 32, 32, 8, 3, 0.5, 0, P, P, None, P, P, ws, None]
    for idx, val in [(7, 9), (7, -1), (6, 70000), (13, None), (4, 20), (15, ws - 1), (1, None),
                     (10, None)]:
        a = list(ok)
        a[idx] = val
        assert lib.rowwise_proxy_update_topk_rank(*a) == EINVAL, idx


def test_proxy_rejects_bad_arguments():
    lib = fq.load()
    ws = fq.rowwise_proxy_update_workspace_bytes(32, 32, 4)
    ok = [P, P, P, P, 32, 32, 4, 0.5, 0, P, P, None, P, ws, None]
    for idx, val in [(4, 20), (6, -1), (8, -2), (9, None), (10, None), (13, ws - 1), (12, MIS),
                     (1, None)]:
        a = list(ok)
        a[idx] = val
        assert lib.rowwise_proxy_update(*a) == EINVAL, idx


def test_melded_linear_buffers_on_host():
    """MeldedLinear allocates every buffer up front (built here on the CPU
    device only to check shapes; its calls need the GPU)."""
    m = fq.MeldedLinear(64, 32, 4, 16, device="cpu", optimizer="adamw",
                        adamw={"beta1": 0.8, "weight_decay": 0.1})
    assert m.adamw == {"beta1": 0.8, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.1}
    assert m.mA.shape == m.vA.shape == (4, 32) and m.mB.shape == m.vB.shape == (64, 4)
    assert m.adam_state.numel() * m.adam_state.element_size() == fq.ADAMW_STATE_BYTES
    assert not m.adam_state.any()
    assert not m.mB.any() and not m.vB.any()
    frozen = fq.MeldedLinear(64, 32, 4, 16, device="cpu", optimizer="adamw", train_a=False)
    assert frozen.dA is None and frozen.mA is None and frozen.vA is None
    assert fq.MeldedLinear(64, 32, 4, 16, device="cpu").optimizer == "sgd"
    with pytest.raises(ValueError):
        fq.MeldedLinear(64, 32, 4, 16, device="cpu", optimizer="adam")


def test_fp4_calls_reject_bad_arguments():
    lib = fq.load()
    ws = fq.fp8_quantize_workspace_bytes(16)
    assert lib.fp4_quantize(P, 0, 15, None, P, P, None, None, P, ws, None) == EINVAL      # odd n
    assert lib.fp4_quantize(P, 0, -2, None, P, P, None, None, P, ws, None) == EINVAL
    assert lib.fp4_quantize(P, 3, 16, None, P, P, None, None, P, ws, None) == EINVAL      # dtype
    assert lib.fp4_quantize(P, 0, 16, None, None, P, None, None, P, ws, None) == EINVAL   # q null
    assert lib.fp4_quantize(P, 0, 16, None, P, P, None, None, P, ws - 1, None) == EINVAL  # short ws
    # d_in must be a multiple of 256, d_out of 16
    assert lib.melded_linear_fwd_fp4(P, P, P, P, 8, 128, 32, P, None) == EINVAL
    assert lib.melded_linear_fwd_fp4(P, P, P, P, 8, 256, 24, P, None) == EINVAL
    assert lib.melded_linear_fwd_fp4(P, None, P, P, 8, 256, 32, P, None) == EINVAL        # s_x
    assert lib.melded_linear_fwd_fp4(P, P, P, P, 8, 256, 32, None, None) == EINVAL        # y
    assert lib.melded_linear_fwd_fp4(P, P, P, P, 0, 256, 32, P, None) == 0                # T = 0


def test_quantize_noalloc_argument_errors():
    """fp8_quantize_noalloc validates like fp8_quantize before any HIP call."""
    lib = fq.load()
    fake = ctypes.c_void_p(1 << 20)                 # never dereferenced
    assert lib.fp8_quantize_noalloc(fake, 0, -1, 0, None, fake, fake, None, None, None) == EINVAL
    assert lib.fp8_quantize_noalloc(fake, 7, 16, 0, None, fake, fake, None, None, None) == EINVAL
    assert lib.fp8_quantize_noalloc(fake, 0, 16, 9, None, fake, fake, None, None, None) == EINVAL
    assert lib.fp8_quantize_noalloc(None, 0, 16, 0, None, fake, fake, None, None, None) == EINVAL
    assert lib.fp8_quantize_noalloc(fake, 0, 16, 0, None, fake, None, None, None, None) == EINVAL
    assert fq.QUANTIZE_SCRATCH_BYTES >= fq.fp8_quantize_workspace_bytes(1 << 30)


def test_quantize_wait_ticks_round_trip():
    """The one-launch quantize's wait setting is host state: set, read back
    through the previous value, restored (no GPU call)."""
    lib = fq.load()
    prev = lib.fp8_quantize_wait_ticks(1234)
    assert prev == 50000                            # the default: 500 us of the 100 MHz counter
    assert lib.fp8_quantize_wait_ticks(0) == 1234
    assert fq.fp8_quantize_wait_ticks(prev) == 0
    with pytest.raises(fq.FalqError):
        fq.fp8_quantize_wait_ticks(-1)


def test_transpose_calls_reject_bad_arguments():
    """fp8_transpose, rowwise_proxy_update_t and melded_linear_bwd_xa_t
    validate before any HIP call (no GPU here: only error paths and the
    zero-size no-ops run)."""
    lib = fq.load()
    P = ctypes.c_void_p(1 << 20)                    # never dereferenced
    Q = ctypes.c_void_p(1 << 21)
    assert lib.fp8_transpose(P, 24, 32, Q, None) == EINVAL          # rows not a multiple of 16
    assert lib.fp8_transpose(P, 32, 8, Q, None) == EINVAL
    assert lib.fp8_transpose(P, 32, 32, P, None) == EINVAL          # in place
    assert lib.fp8_transpose(None, 32, 32, Q, None) == EINVAL
    assert lib.fp8_transpose(P, 32, 32, ctypes.c_void_p((1 << 21) + 4), None) == EINVAL
    assert lib.fp8_transpose(None, 0, 32, None, None) == 0          # empty: nothing to do
    n = ctypes.c_void_p(1 << 22)
    ws = ctypes.c_void_p(1 << 23)
    big = 1 << 30
    # d_out must be a multiple of 16 for the transpose (the plain update allows any d_out)
    assert lib.rowwise_proxy_update_t(P, Q, n, P, P, 32, 24, 4, 0.5, 0, P, n, None, ws, big,
                                      None) == EINVAL
    assert lib.rowwise_proxy_update_t(P, P, n, P, P, 32, 32, 4, 0.5, 0, P, n, None, ws, big,
                                      None) == EINVAL               # wqT == wq
    assert lib.rowwise_proxy_update_t(P, None, n, P, P, 32, 32, 4, 0.5, 0, P, n, None, ws, big,
                                      None) == EINVAL
    assert lib.rowwise_proxy_update_t(P, Q, n, P, P, 32, 32, 4, 0.5, -1, P, n, None, ws, big,
                                      None) == EINVAL               # k_max
    # the dX product needs the transpose when dx is wanted
    f = lib.melded_linear_bwd_xa_t
    assert f(P, 0, n, P, n, None, n, P, P, P, 64, 64, 64, 4, P, P, P, ws, big, None) == EINVAL
    assert f(P, 7, n, P, n, Q, n, P, P, P, 64, 64, 64, 4, P, P, P, ws, big, None) == EINVAL
    assert f(P, 0, n, P, n, Q, n, P, P, P, 64, 60, 64, 4, P, P, P, ws, big, None) == EINVAL


def test_adapter_pieces_calls_reject_bad_arguments():
    """The calls around A's pieces validate before any HIP call."""
    lib = fq.load()
    assert fq.adapter_pieces_bytes(0, 128) == 0
    assert fq.adapter_pieces_bytes(8, 100) == 0                   # d_in not a multiple of 128
    nb = fq.adapter_pieces_bytes(13, 256)
    # three planes of 16 padded rows x 256 codes, and 2 x 16 x 4 scale bytes
    assert nb >= 3 * 16 * 256 + 2 * 16 * 4
    assert lib.adapter_pieces(None, 13, 256, P, nb, None) == EINVAL            # A null
    assert lib.adapter_pieces(P, 13, 256, P, nb - 1, None) == EINVAL           # short buffer
    assert lib.adapter_pieces(P, 13, 200, P, nb, None) == EINVAL               # d_in
    assert lib.adapter_pieces(P, 13, 256, MIS, nb, None) == EINVAL             # alignment
    assert lib.adapter_step_pieces(P, P, None, P, 13, 256, 64, 1e-3, P, nb, None) == EINVAL
    assert lib.adapter_step_pieces(P, None, P, P, 13, 256, 64, 1e-3, P, nb, None) == EINVAL
    assert lib.adapter_step_pieces(P, P, P, P, 13, 256, -1, 1e-3, P, nb, None) == EINVAL
    assert lib.adapter_step_pieces(P, P, P, P, 13, 256, 64, 1e-3, P, nb - 1, None) == EINVAL
    # the forward from the pieces needs the unit columns: r <= d_out / 64 (4096 / 64 = 64 >= 13)
    assert lib.melded_linear_fwd_xa_pieces(P, P, P, P, P, nb, 8, 256, 512, 13, P, P,
                                           None) == EINVAL    # 2 column tiles carry no units
    assert lib.melded_linear_fwd_xa_pieces(P, None, P, P, P, nb, 8, 256, 1024, 13, P, P,
                                           None) == EINVAL    # s_x
    assert lib.melded_linear_fwd_xa_pieces(P, P, P, P, P, nb - 1, 8, 256, 1024, 13, P, P,
                                           None) == EINVAL    # short buffer
    assert lib.melded_linear_fwd_xa_pieces(P, P, P, P, P, nb, 8, 256, 1024, 13, None, P,
                                           None) == EINVAL    # y
