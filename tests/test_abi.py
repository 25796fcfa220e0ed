"""The C ABI on the CPU: the library loads, exports every entry point
include/dr.h declares, and rejects bad arguments with the documented status
before any device call.  No call here reaches a kernel launch: every one
either fails validation or has M == 0."""
import ctypes
import os
import re

import pytest

import deterministic_gemm_amd as dr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dr.h")

OK, INVALID, UNSUPPORTED = dr.DR_OK, dr.DR_ERR_INVALID, dr.DR_ERR_UNSUPPORTED
A = 0x10000  # a 16-byte aligned stand-in address, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(dr_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dr.LIB_PATH):
        from deterministic_gemm_amd import build
        build.build()
    return dr.load_library()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(L, n), n
    assert set(dr.EXPORTED) == set(names)


def _route(L, x=A, xd=0, W=A, M=4, K=2048, E=256, k=8, ld=0, ids=A, w=A, lg=A, mg=A, flags=0, variant=None):
    args = [ctypes.c_void_p(x) if x else None, xd, ctypes.c_void_p(W) if W else None, M, K, E, k, ld,
            ctypes.c_void_p(ids) if ids else None, ctypes.c_void_p(w) if w else None,
            ctypes.c_void_p(lg) if lg else None, ctypes.c_void_p(mg) if mg else None, flags]
    if variant is None:
        return L.dr_route(*args, None)
    return L.dr_route_variant(*args, variant, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), INVALID),
    (dict(k=257), INVALID),
    (dict(M=-1), INVALID),
    (dict(K=0), INVALID),
    (dict(E=0), INVALID),
    (dict(x=0), INVALID),
    (dict(W=0), INVALID),
    (dict(ids=0), INVALID),
    (dict(x=A + 4), INVALID),
    (dict(mg=A + 8), INVALID),
    (dict(flags=2), INVALID),
    (dict(xd=7), INVALID),
    (dict(ld=3), INVALID),
    (dict(E=100, k=8), UNSUPPORTED),
    (dict(E=2048, k=8), UNSUPPORTED),
    (dict(K=16385), UNSUPPORTED),
    (dict(E=64, k=33), UNSUPPORTED),
])
def test_route_rejects(L, kw, status):
    assert _route(L, **kw) == status
    assert L.dr_last_error().decode() != ""


def test_route_variant_rejects(L):
    assert _route(L, variant=9) == INVALID
    assert _route(L, variant=7) == INVALID
    assert _route(L, E=1024, k=8, variant=2) == UNSUPPORTED  # the tiled family stops at E=512
    # the split family writes the logits and reads them back: it needs that
    # output, fp32 x in whole 16-byte pieces and E in {256, 512}
    assert _route(L, lg=0, variant=3) == UNSUPPORTED
    assert _route(L, xd=1, K=8192, variant=3) == UNSUPPORTED  # bf16 x: K <= 4096 and K % 8 == 0
    assert _route(L, xd=1, K=2044, variant=3) == UNSUPPORTED
    assert _route(L, K=2046, variant=3) == UNSUPPORTED
    assert _route(L, E=128, k=8, variant=3) == UNSUPPORTED
    assert _route(L, M=0, variant=3) == OK
    # the narrow family has the same needs, with any E up to 512
    assert _route(L, lg=0, variant=4) == UNSUPPORTED
    assert _route(L, xd=1, K=2044, variant=4) == UNSUPPORTED  # bf16 x: K % 8 == 0
    assert _route(L, E=1024, k=8, variant=4) == UNSUPPORTED
    # the one-launch family: E = 256 only; the logits output is optional
    assert _route(L, E=512, k=8, variant=6) == UNSUPPORTED
    assert _route(L, K=2046, variant=6) == UNSUPPORTED
    assert _route(L, xd=1, K=8192, variant=6) == UNSUPPORTED
    assert _route(L, M=0, lg=0, variant=6) == OK


def test_halves_reject(L):
    P = ctypes.c_void_p
    assert L.dr_route_logits(P(A), P(A), 4, 2048, 256, 0, None, None) == INVALID       # no output
    assert L.dr_route_logits(P(A), P(A), 4, 2048, 256, 5, P(A), None) == INVALID       # bad dtype
    assert L.dr_route_logits(P(A), P(A + 4), 4, 2048, 256, 0, P(A), None) == INVALID   # misaligned
    assert L.dr_route_logits(P(A), P(A), 4, 2046, 256, 0, P(A), None) == UNSUPPORTED   # K % 4
    assert L.dr_route_logits(P(A), P(A), 4, 2048, 1024, 0, P(A), None) == UNSUPPORTED  # E
    assert L.dr_route_logits(None, None, 0, 2048, 256, 0, None, None) == OK
    assert L.dr_route_select(P(A), 0, 4, 256, 8, None, None, None, 0, None) == INVALID  # no ids
    assert L.dr_route_select(P(A), 0, 4, 256, 0, P(A), None, None, 0, None) == INVALID  # k = 0
    assert L.dr_route_select(P(A), 0, 4, 256, 8, P(A), None, None, 2, None) == INVALID  # flags
    assert L.dr_route_select(P(A), 0, 4, 2048, 8, P(A), None, None, 0, None) == UNSUPPORTED
    assert L.dr_route_select(P(A), 0, 4, 256, 33, P(A), None, None, 0, None) == UNSUPPORTED
    assert L.dr_route_select(None, 0, 0, 256, 8, None, None, None, 0, None) == OK


def test_row_bounds(L):
    # 2^22 tokens per call at most; a forced vector-ALU call at most 4 * 65535
    assert _route(L, M=(1 << 22) + 1) == INVALID
    assert _route(L, M=4 * 65535 + 1, variant=dr.VARIANTS["tiny"]) == UNSUPPORTED
    P = ctypes.c_void_p
    assert L.dr_gate_dot(P(A), 0, P(A), 0, P(A), None, (1 << 22) + 1, 64, None) == INVALID
    assert L.dr_moe_permute(P(A), (1 << 22) + 1, 1, 8, P(A), P(A), P(A), None) == INVALID


def test_empty_batch_returns_ok_without_launch(L):
    assert _route(L, M=0) == OK
    assert _route(L, M=0, x=0, W=0, ids=0) == OK
    assert L.dr_last_error().decode() == ""


def test_gate_and_gemm_reject(L):
    P = ctypes.c_void_p
    assert L.dr_gate_dot(P(A), 0, P(A), 0, None, None, 4, 64, None) == INVALID   # no output
    assert L.dr_gate_dot(P(A), 0, P(A), 5, P(A), None, 4, 64, None) == INVALID   # bad dtype
    assert L.dr_gate_dot(P(A), 0, P(A), 0, P(A), None, 4, 0, None) == INVALID
    assert L.dr_gate_dot(P(A), 0, P(A), 0, P(A), None, 4, 20000, None) == UNSUPPORTED
    assert L.dr_gate_dot(P(A), 0, P(A), 0, P(A), None, 0, 64, None) == OK
    assert L.dr_gemm_bf16(P(A), P(A), P(A), 4, 48, 128, None) == UNSUPPORTED     # K % 32
    assert L.dr_gemm_bf16(P(A), P(A), P(A), 4, 64, 100, None) == UNSUPPORTED     # N % 128
    assert L.dr_gemm_bf16(None, P(A), P(A), 4, 64, 128, None) == INVALID
    assert L.dr_gemm_bf16(P(A), P(A), P(A), 0, 64, 128, None) == OK


def test_moe_calls_reject(L):
    P = ctypes.c_void_p
    # dr_moe_permute(ids, M, k, E, offsets, rows, pos, stream); M == 0 still launches (offsets)
    assert L.dr_moe_permute(P(A), 4, 0, 8, P(A), P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), 4, 2, 0, P(A), P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), -1, 2, 8, P(A), P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), 4, 2, 8, None, P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), 4, 2, 8, P(A), None, P(A), None) == INVALID
    assert L.dr_moe_permute(P(A + 4), 4, 2, 8, P(A), P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), 4, 33, 64, P(A), P(A), P(A), None) == UNSUPPORTED
    assert L.dr_moe_permute(P(A), 4, 2, 1025, P(A), P(A), P(A), None) == UNSUPPORTED
    assert L.dr_moe_permute(P(A), 1 << 31, 1, 8, P(A), P(A), P(A), None) == INVALID
    assert L.dr_moe_permute(P(A), 1 << 30, 2, 8, P(A), P(A), P(A), None) == INVALID
    # dr_moe_gather(x, dtype, M, D, rows, P, xp, stream)
    assert L.dr_moe_gather(P(A), 0, 4, 0, P(A), 8, P(A), None) == INVALID
    assert L.dr_moe_gather(P(A), 7, 4, 16, P(A), 8, P(A), None) == INVALID
    assert L.dr_moe_gather(None, 0, 4, 16, P(A), 8, P(A), None) == INVALID
    assert L.dr_moe_gather(P(A), 0, 4, 16, P(A), 1 << 31, P(A), None) == UNSUPPORTED
    assert L.dr_moe_gather(P(A), 0, 4, 16, P(A), 0, P(A), None) == OK
    # dr_moe_combine(y, ydt, P, w, ids, pos, shared, sdt, gate, M, k, D, out, stream)
    assert L.dr_moe_combine(P(A), 0, 8, P(A), P(A), P(A), None, 0, None, 4, 0, 16, P(A), None) == INVALID
    assert L.dr_moe_combine(P(A), 0, 0, P(A), P(A), P(A), None, 0, None, 4, 2, 16, P(A), None) == INVALID
    assert L.dr_moe_combine(P(A), 0, 8, P(A), P(A), P(A), P(A), 0, None, 4, 2, 16, P(A), None) == INVALID
    assert L.dr_moe_combine(P(A), 3, 8, P(A), P(A), P(A), None, 0, None, 4, 2, 16, P(A), None) == INVALID
    assert L.dr_moe_combine(P(A), 0, 8, P(A), None, P(A), None, 0, None, 4, 2, 16, P(A), None) == INVALID
    assert L.dr_moe_combine(P(A), 0, 8, P(A), P(A), P(A), None, 0, None, 4, 33, 16, P(A), None) == UNSUPPORTED
    assert L.dr_moe_combine(P(A), 0, 8, P(A), P(A), P(A), None, 0, None, 0, 2, 16, P(A), None) == OK
    assert L.dr_moe_combine(P(A), 0, 8, P(A), P(A), P(A), None, 0, None, (1 << 22) + 1, 2, 16, P(A), None) == UNSUPPORTED


def test_route_bf16_gemm_rejects(L):
    P = ctypes.c_void_p
    # dr_route_bf16_gemm(x, W, M, K, E, k, ids, weights, logits, margins, flags, stream)
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 256, 0, P(A), None, P(A), None, 0, None) == INVALID
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 256, 8, P(A), None, None, None, 0, None) == INVALID
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 256, 8, P(A), None, P(A), None, 4, None) == INVALID
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 48, 256, 8, P(A), None, P(A), None, 0, None) == UNSUPPORTED
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 64, 8, P(A), None, P(A), None, 0, None) == UNSUPPORTED
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 2048, 8, P(A), None, P(A), None, 0, None) == UNSUPPORTED
    assert L.dr_route_bf16_gemm(P(A), P(A), 4, 64, 256, 33, P(A), None, P(A), None, 0, None) == UNSUPPORTED
    assert L.dr_route_bf16_gemm(P(A), P(A), 0, 64, 256, 8, P(A), None, P(A), None, 0, None) == OK


def test_grouped_gemm_rejects(L):
    P = ctypes.c_void_p
    # dr_grouped_gemm_bf16(x, Mx, rows, W, offsets, E, P, K, N, out, stream)
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 0, 8, 64, 128, P(A), None) == INVALID
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), None, 4, 8, 64, 128, P(A), None) == INVALID
    assert L.dr_grouped_gemm_bf16(P(A), 4, None, P(A), P(A), 4, 8, 64, 128, P(A), None) == INVALID  # P > Mx
    assert L.dr_grouped_gemm_bf16(P(A + 8), 8, P(A), P(A), P(A), 4, 8, 64, 128, P(A), None) == INVALID
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 4, 8, 48, 128, P(A), None) == UNSUPPORTED
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 4, 8, 64, 96, P(A), None) == UNSUPPORTED
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 1025, 8, 64, 128, P(A), None) == UNSUPPORTED
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 4, 1 << 24, 64, 128, P(A), None) == UNSUPPORTED
    assert L.dr_grouped_gemm_bf16(P(A), 8, P(A), P(A), P(A), 4, 0, 64, 128, P(A), None) == OK


def test_auto_variant_is_a_function_of_shape(L):
    picks = [dr.auto_variant(M, 2048, 256, logits=False) for M in range(19, 81)]
    assert picks[0] == "rowwise" and picks[-1] == "tiled"
    # exactly one switch, inside the m-scan range
    switches = sum(1 for a, b in zip(picks, picks[1:]) if a != b)
    assert switches == 1
    assert dr.auto_variant(8192, 2048, 1024, logits=False) == "rowwise"
    # small batches that ask for the logits: the vector-ALU family while its
    # workgroups fit the CUs at once (256 here: 64 tokens at K = 2048, E = 256;
    # 16 at K = 4096; 128 at K = 1024), then narrow tiles (the switch lies
    # inside the m-scan range); up to 4096 tokens where the narrow family does
    # not take E
    assert [dr.auto_variant(M, 2048, 256) for M in (1, 19, 32, 33, 64, 65, 80)] == ["tiny"] * 5 + ["narrow"] * 2
    assert [dr.auto_variant(M, 4096, 256) for M in (16, 17)] == ["tiny", "narrow"]
    assert [dr.auto_variant(M, 2048, 512) for M in (32, 33)] == ["tiny", "narrow"]
    assert [dr.auto_variant(M, 1024, 256) for M in (128, 129)] == ["tiny", "narrow"]
    assert dr.auto_variant(19, 2048, 1024) == "tiny"
    # E = 1024: the two-kernel family right after the vector-ALU family
    assert [dr.auto_variant(M, 2048, 1024) for M in (64, 65, 8192)] == ["tiny", "split", "split"]
    assert [dr.auto_variant(M, 4096, 1024) for M in (32, 33)] == ["tiny", "split"]
    assert [dr.auto_variant(M, 8192, 1024) for M in (1, 8192)] == ["split", "split"]
    assert dr.auto_variant(19, 8192, 256) == "narrow"   # K above the vector family's 4096
    # large batches that ask for the logits take the two-kernel family: at
    # 1024 < K <= 4096 above 2048 tokens for E = 256 and 1024 for E = 512
    # (where the narrow family's largest tile stops fitting 256 CUs at once),
    # above 1280 at other K
    assert dr.auto_variant(8192, 2048, 256) == "split"
    assert [dr.auto_variant(M, 2048, 256) for M in (1280, 2048, 2049)] == ["narrow", "narrow", "split"]
    assert [dr.auto_variant(M, 2048, 512) for M in (1024, 1025)] == ["narrow", "split"]
    assert [dr.auto_variant(M, 4096, 512) for M in (240, 1024, 1025)] == ["narrow", "narrow", "split"]
    assert [dr.auto_variant(M, 8192, 256) for M in (1280, 1281)] == ["narrow", "split"]
    assert [dr.auto_variant(M, 1024, 256) for M in (2048, 2049)] == ["narrow", "split"]
    assert [dr.auto_variant(M, 1024, 512) for M in (1280, 1281)] == ["narrow", "split"]
    assert dr.auto_variant(8192, 2048, 256, logits=False) == "tiled"
    assert dr.auto_variant(8192, 2048, 256, x_dtype="bf16") == "split"  # bf16 x staged as it is
    assert dr.auto_variant(8192, 8192, 256, x_dtype="bf16") == "tiled"
    assert dr.auto_variant(8192, 2046, 256) == "tiled"


def test_contract(L):
    c = dr.contract()
    assert c == {"version": 1, "kblock": 256, "tree": 1, "acc_bits": 32, "fma": 1, "exp_id": 1,
                 "tie_break": 1, "max_k": 32}


def test_status_strings(L):
    for s in (0, 1, 2, 3):
        assert L.dr_status_string(s)


def test_widen_bf16_validation(L):
    assert L.dr_widen_bf16(None, -1, None, None) == INVALID
    assert L.dr_widen_bf16(None, 8, A, None) == INVALID
    assert L.dr_widen_bf16(A, 8, None, None) == INVALID
    assert L.dr_widen_bf16(A + 2, 8, A, None) == INVALID  # misaligned x
    assert L.dr_widen_bf16(A, 8, A + 4, None) == INVALID  # misaligned out
    assert L.dr_widen_bf16(None, 0, None, None) == OK      # empty: nothing launched
    assert not dr.widen_bf16_used(8192, 8192 * 4, 256)     # K above the fp32 families' limits
    # small batches: the vector-ALU family reads bf16 x itself (K % 8 == 0)
    assert [dr.auto_variant(M, 2048, 256, "bf16") for M in (1, 64, 65)] == ["tiny", "tiny", "narrow"]
    assert dr.auto_variant(1, 2044, 256, "bf16") != "tiny" and dr.auto_variant(1, 2044, 256) == "tiny"
    # the narrow tiles and the two-kernel family stage bf16 x themselves
    # (K % 8 == 0; the two-kernel family K <= 4096); the binding widens bf16
    # x only where they do not
    assert [dr.auto_variant(M, 2048, 256, "bf16") for M in (2048, 2049, 8192)] == ["narrow", "split", "split"]
    assert dr.auto_variant(8192, 8192, 256, "bf16") != "split" and dr.auto_variant(8192, 8192, 256) == "split"
    assert dr.auto_variant(8192, 2044, 256, "bf16") != "split"
    assert not any(dr.widen_bf16_used(M, 2048, 256) for M in (1, 64, 65, 2048, 2049, 8192))
    assert dr.widen_bf16_used(8192, 8192, 256) and not dr.widen_bf16_used(1024, 8192, 256)


def test_binding_validates_out_tensors():
    """The binding checks every caller-supplied output (and extra input)
    tensor against what the C call writes through its pointer -- dtype,
    shape, device, contiguity -- before any call; a mismatch raises instead of
    letting a kernel write past a smaller allocation.  The checks run on
    host tensors here (no GPU needed); the entry points themselves refuse
    host tensors first."""
    import torch

    cpu = torch.device("cpu")
    ok = torch.empty((4, 8), dtype=torch.int32)
    assert dr._out_tensor(ok, "ids", torch.int32, (4, 8), cpu) is ok
    bad = [
        (torch.empty((4, 7), dtype=torch.int32), ValueError),           # too few columns
        (torch.empty((3, 8), dtype=torch.int32), ValueError),           # too few rows
        (torch.empty((4, 8), dtype=torch.int64), TypeError),            # wrong dtype
        (torch.empty((8, 4), dtype=torch.int32).t(), ValueError),       # not contiguous
        (torch.empty((4, 8), dtype=torch.int32, device="meta"), ValueError),  # another device
        (ok.numpy(), TypeError),                                        # not a tensor
    ]
    for t, exc in bad:
        with pytest.raises(exc):
            dr._out_tensor(t, "ids", torch.int32, (4, 8), cpu)
    with pytest.raises(ValueError):
        dr._same_device(torch.empty(3, device="meta"), "W", cpu)
    # every entry point refuses host operands before touching its outputs
    x = torch.zeros((4, 64))
    with pytest.raises(TypeError):
        dr.route(x, torch.zeros((64, 256)), 8, out=(ok, None, None, None))
    with pytest.raises(TypeError):
        dr.gemm_bf16(x.to(torch.bfloat16), torch.zeros((64, 128), dtype=torch.bfloat16))


def test_noalloc_refuses_batches_past_its_buffer(L):
    """dr_route_noalloc checks the size of the logits it would keep in its
    static device buffer before touching the device: 16384 x 256 fp32
    logits fit, one token more does not (bf16 logits take half)."""
    P = ctypes.c_void_p

    def call(M, E=256, ld=0, lg=None, x=A):
        return L.dr_route_noalloc(P(x) if x else None, 0, P(A), M, 2048, E, 8, ld, P(A), None, lg, None, 0, None)

    assert call(16385) == UNSUPPORTED
    assert "exceed" in L.dr_last_error().decode()
    assert call(16385 * 2, ld=1) == UNSUPPORTED
    assert call(8193, E=512) == UNSUPPORTED
    assert call(0, x=0) == OK                      # empty batch: nothing launched, no device touched
    assert call(1, x=0) == INVALID                 # the usual argument checks come first
