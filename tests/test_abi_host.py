"""Host-side checks of the C ABI (CPU only, no kernel is launched).

The library must load, export every function include/nf4moe.h declares, and
reject bad arguments on the host before anything is enqueued -- so these run
without a GPU.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from grouped_nf4_gemm_quantize_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4moe.h")

FAKE = 0x10000  # a 64 KiB-aligned non-null pointer; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libnf4moe.so is not built (run __graft_entry__.build())")
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("nf4_quantize_experts", "moe_route_permute", "grouped_nf4_gemm",
              "moe_expert_forward"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_codebook_bits_match_the_oracle(lib):
    buf = (ctypes.c_float * 16)()
    assert lib.nf4moe_codebook(buf) == 0
    got = np.array(list(buf), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    assert lib.nf4moe_codebook(None) == -1


def test_fp4_codebook_bits_match_the_oracle(lib):
    buf = (ctypes.c_float * 16)()
    assert lib.nbit_codebook(1, buf) == 0
    got = np.array(list(buf), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.fp4_codebook().view(np.uint32))
    assert lib.nbit_codebook(0, buf) == 0
    got = np.array(list(buf), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.nf4_codebook().view(np.uint32))
    assert lib.nbit_codebook(2, buf) == -1
    assert lib.nbit_codebook(1, None) == -1


def test_nbit_entry_points_reject_unknown_modes(lib):
    assert lib.nbit_quantize_experts(7, FAKE, 0, 1, 1, 64, 64, FAKE, FAKE, None, None) == -1
    assert "storage mode" in _last(lib)
    assert lib.grouped_nbit_gemm(-1, FAKE, 2, 8, None, 1, FAKE, FAKE, FAKE, 1, 8, 64, 64,
                                 None, 0, None, None, FAKE, 2, None) == -1
    assert lib.moe_expert_forward_nbit(9, FAKE, 1, FAKE, 1, 64, 64, 8, 2, 1, FAKE, FAKE,
                                       FAKE, FAKE, None, None, FAKE, 1, FAKE, 1 << 20,
                                       None) == -1
    # a known mode reaches the usual validation (blocksize)
    assert lib.nbit_quantize_experts(1, FAKE, 0, 1, 1, 64, 32, FAKE, FAKE, None, None) == -3


def test_passthrough_modes_host_checks(lib):
    """bf16 (5) and fp16 (6) passthrough: no codebook, no absmax needed, no
    adapters, no dgrad; the 4- and 8-bit modes still need their absmax."""
    buf = (ctypes.c_float * 16)()
    assert lib.nbit_codebook(5, buf) == -1 and lib.nbit_codebook(6, buf) == -1
    gemm = lambda qt, absmax, lora: lib.grouped_nbit_gemm(
        qt, FAKE, 2, 8, None, 1, FAKE, absmax, FAKE, 1, 8, 64, 64, lora, 0, None, None,
        FAKE, 2, None)
    good = binding.LoraStruct(FAKE, FAKE, 8, 2.0, 1)
    assert gemm(5, None, ctypes.byref(good)) == -1   # absmax may be NULL; adapters refused
    assert "adapters" in _last(lib)
    assert gemm(6, None, ctypes.byref(good)) == -1
    assert gemm(3, None, None) == -1                 # int8 needs its absmax
    assert "absmax" in _last(lib)
    assert lib.grouped_nbit_gemm_dgrad(5, FAKE, 2, 8, None, 1, FAKE, None, FAKE, 1, 8, 64, 64,
                                       0, None, 2, None, None, FAKE, 2, None) == -1
    # the conversion needs 16-byte aligned buffers (bf16 input at 8 bytes)
    assert lib.nbit_quantize_experts(5, FAKE + 8, 1, 1, 1, 64, 64, FAKE, None, None,
                                     None) == -1
    assert "16-byte" in _last(lib)


@pytest.mark.parametrize("E,N,K", [(128, 1536, 2048), (128, 2048, 768), (8, 256, 256),
                                   (64, 2048, 2048), (1, 16, 64)])
def test_packed_bytes_matches_the_format(lib, E, N, K):
    assert lib.nf4moe_packed_bytes(E, N, K) == oracle.packed_bytes(E, N, K)


def test_packed_bytes_rejects_bad_sizes(lib):
    assert lib.nf4moe_packed_bytes(1, 1, 100) == -2
    assert lib.nf4moe_packed_bytes(0, 1, 64) == -1


def _last(lib):
    return lib.nf4moe_last_error().decode()


def test_quantize_validation(lib):
    q = lib.nf4_quantize_experts
    assert q(None, 0, 1, 1, 64, 64, FAKE, FAKE, None, None) == -1
    assert q(FAKE, 0, 1, 1, 64, 32, FAKE, FAKE, None, None) == -3  # blocksize
    assert "nf4/64" in _last(lib)
    assert q(FAKE, 0, 1, 1, 96, 64, FAKE, FAKE, None, None) == -2  # K % 64
    assert q(FAKE, 2, 1, 1, 64, 64, FAKE, FAKE, None, None) == -5  # F16 input
    assert q(FAKE, 0, 0, 1, 64, 64, FAKE, FAKE, None, None) == -1
    assert q(FAKE + 4, 0, 1, 1, 64, 64, FAKE, FAKE, None, None) == -1  # misaligned
    assert "misaligned" in _last(lib)
    # the 8-bit modes store whole words of codes; the flag is an int32
    qn = lib.nbit_quantize_experts
    assert qn(3, FAKE, 0, 1, 1, 64, 64, FAKE + 2, FAKE, None, None) == -1  # int8, packed % 4
    assert qn(4, FAKE, 0, 1, 1, 64, 64, FAKE + 2, FAKE, None, None) == -1  # fp8, packed % 4
    assert q(FAKE, 0, 1, 1, 64, 64, FAKE, FAKE, FAKE + 2, None) == -1  # nonfinite_flag % 4


def test_route_validation(lib):
    r = lib.moe_route_permute
    ws = lib.moe_route_permute_workspace(64, 8, 2)
    assert ws > 0
    args = dict(logits=FAKE, T=64, E=8, k=2, renorm=1, ids=FAKE, w=FAKE, sp=FAKE,
                pos=None, off=FAKE, ws=FAKE, wsb=ws, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return r(a["logits"], a["T"], a["E"], a["k"], a["renorm"], a["ids"], a["w"],
                 a["sp"], a["pos"], a["off"], a["ws"], a["wsb"], a["stream"])

    assert call(logits=None) == -1
    assert call(k=0) == -4
    assert call(k=9) == -4
    assert call(k=33, E=64) == -4
    assert call(E=2000) == -2
    assert call(T=0) == -1
    assert call(renorm=2) == -1
    assert call(wsb=ws - 1) == -6
    assert call(ws=None) == -6
    assert call(T=2 ** 30, k=8, E=64) == -7


def test_gemm_validation(lib):
    g = lib.grouped_nf4_gemm

    def call(**kw):
        a = dict(a=FAKE, adt=2, arows=10, gather=None, gdiv=1, packed=FAKE, absmax=FAKE,
                 off=FAKE, E=4, P=10, N=64, K=128, lora=None, epi=0, rs=None, sc=None,
                 out=FAKE, odt=0, stream=None)
        a.update(kw)
        return g(a["a"], a["adt"], a["arows"], a["gather"], a["gdiv"], a["packed"],
                 a["absmax"], a["off"], a["E"], a["P"], a["N"], a["K"], a["lora"], a["epi"],
                 a["rs"], a["sc"], a["out"], a["odt"], a["stream"])

    assert call(a=None) == -1
    assert call(K=96) == -2
    assert call(N=40) == -2
    assert call(N=48, epi=1) == -2  # SwiGLU needs N % 32 == 0
    assert call(epi=7) == -1
    assert call(adt=0) == -5  # fp32 activations are not an MFMA operand type
    assert call(odt=9) == -5
    assert call(E=0) == -1
    assert call(E=4096) == -2
    assert call(gather=FAKE, gdiv=0) == -1
    assert call(a=FAKE + 8) == -1
    bad = binding.LoraStruct(FAKE, FAKE, 0, 2.0, 1)
    assert call(lora=ctypes.byref(bad)) == -1
    bad = binding.LoraStruct(FAKE, FAKE, 8, 2.0, 0)
    assert call(lora=ctypes.byref(bad)) == -5
    bad = binding.LoraStruct(FAKE, FAKE, 17, 2.0, 1)
    assert call(lora=ctypes.byref(bad)) == -1
    # sizes past the kernels' 32-bit row indexing and 32-bit buffer offsets
    assert call(P=2**31 - 1) == -7
    assert call(N=2**30 + 16) == -7
    assert call(arows=2**21, K=1024) == -7  # 4 GiB of activations
    assert call(N=2**19, K=2**14) == -7     # one expert's stack past 4 GiB
    # P == 0 is a valid empty problem: nothing is enqueued
    assert call(P=0) == 0


def test_forward_validation(lib):
    f = lib.moe_expert_forward
    T, H, I, E, k = 64, 256, 128, 8, 2
    wsb = lib.moe_expert_forward_workspace(T, H, I, E, k, 0)
    assert wsb > T * k * (H + I) * 2
    # adapters of rank r take their fp16 copies on top: E * r * (2H + 3I) * 2 bytes
    r = 8
    extra = lib.moe_expert_forward_workspace(T, H, I, E, k, r) - wsb
    assert E * r * (2 * H + 3 * I) * 2 <= extra < E * r * (2 * H + 3 * I) * 2 + 4 * 256
    assert lib.moe_expert_forward_workspace(T, H, I, E, k, -1) == 0
    assert lib.moe_expert_forward_workspace(T, H, I, E, k, 17) == 0

    def call(**kw):
        a = dict(x=FAKE, xdt=1, lg=FAKE, T=T, H=H, I=I, E=E, k=k, renorm=1, gp=FAKE,
                 ga=FAKE, dp=FAKE, da=FAKE, gl=None, dl=None, y=FAKE, ydt=1, ws=FAKE,
                 wsb=wsb, stream=None)
        a.update(kw)
        return f(a["x"], a["xdt"], a["lg"], a["T"], a["H"], a["I"], a["E"], a["k"],
                 a["renorm"], a["gp"], a["ga"], a["dp"], a["da"], a["gl"], a["dl"],
                 a["y"], a["ydt"], a["ws"], a["wsb"], a["stream"])

    assert call(x=None) == -1
    assert call(H=200) == -2
    assert call(I=96) == -2
    assert call(k=9) == -4
    assert call(xdt=0) == -5
    assert call(ydt=5) == -5
    assert call(wsb=wsb - 1) == -6
    assert call(ws=FAKE + 64) == -1  # workspace must be 256-byte aligned
    bad = binding.LoraStruct(None, FAKE, 8, 2.0, 1)
    assert call(gl=ctypes.byref(bad)) == -1
    # an adapter needs the workspace sized for its rank
    good = binding.LoraStruct(FAKE, FAKE, 8, 2.0, 1)
    assert call(dl=ctypes.byref(good)) == -6
    assert "adapter rank 8" in _last(lib)
    # sizes past the 32-bit pair indexing and the kernels' 32-bit buffer offsets
    assert call(T=2**31 // k + 1) == -7     # T * k pairs overflow int32
    assert call(T=2**20, H=2**12) == -7     # 8 GiB of token rows
    assert call(T=2**22, I=512) == -7       # h, T * k * I fp16 values, 8 GiB (x 2 GiB)
    assert call(H=2**16, I=2**16) == -7     # one expert's gate_up stack past 4 GiB


def test_noalloc_forward_validation(lib):
    """The allocation-free forward reports argument errors as the forward does
    and refuses sizes whose workspace exceeds its scratch, before any launch."""
    f = lib.moe_expert_forward_noalloc
    T, H, I, E, k = 64, 256, 128, 8, 2

    def call(**kw):
        a = dict(x=FAKE, xdt=1, lg=FAKE, T=T, H=H, I=I, E=E, k=k, renorm=1, gp=FAKE,
                 ga=FAKE, dp=FAKE, da=FAKE, gl=None, dl=None, y=FAKE, ydt=1, stream=None)
        a.update(kw)
        return f(a["x"], a["xdt"], a["lg"], a["T"], a["H"], a["I"], a["E"], a["k"],
                 a["renorm"], a["gp"], a["ga"], a["dp"], a["da"], a["gl"], a["dl"],
                 a["y"], a["ydt"], a["stream"])

    assert call(x=None) == -1
    assert call(H=200) == -2
    assert call(k=9) == -4
    assert call(ydt=5) == -5
    T_big = 1024
    need = lib.moe_expert_forward_workspace(T_big, 2048, 768, 128, 8, 0)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert call(T=T_big, H=2048, I=768, E=128, k=8) == -6
    assert "scratch" in _last(lib)
    # the limit sits where the workspace size query says it does
    assert lib.moe_expert_forward_workspace(670, 2048, 768, 128, 8, 0) <= \
        binding.NOALLOC_SCRATCH_BYTES


def test_status_strings(lib):
    for s in range(0, -9, -1):
        assert lib.nf4moe_strerror(s).decode() != "unknown status"
    assert lib.nf4moe_version().decode().count(".") == 2


def test_dgrad_rejects_bad_arguments_on_the_host(lib):
    ok_args = dict(a=FAKE, a_dtype=2, a_rows=8, gather=None, gather_div=1, packed=FAKE,
                   absmax=FAKE, offsets=FAKE, E=1, P=8, N=128, K=64, epi=0, g=None,
                   g_dtype=2, rs=None, scatter=None, out=FAKE, out_dtype=2, stream=None)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.grouped_nf4_gemm_dgrad(*a.values())

    assert call(a=None) == -1
    assert call(N=96) == -2            # the contraction runs in 64-row steps
    assert call(K=96) == -2
    assert call(epi=1) == -1           # NF4MOE_EPI_SWIGLU is a forward epilogue
    assert call(epi=2) == -1           # the SwiGLU backward needs g_pre
    assert "g_pre" in _last(lib)
    assert call(epi=2, g=FAKE, g_dtype=0) == -5
    assert call(a_dtype=0) == -5
    assert call(out_dtype=7) == -5
    assert call(E=0) == -1
    assert call(P=0) == 0              # nothing to do: no launch
    assert lib.grouped_nbit_gemm_dgrad(5, *ok_args.values()) == -1


def test_swiglu_bwd_gemm_rejects_bad_arguments_on_the_host(lib):
    ok_args = dict(a=FAKE, a_rows=8, gather=None, gather_div=1, packed=FAKE, absmax=FAKE,
                   offsets=FAKE, E=1, P=8, N=128, K=64, lora=None, dh=FAKE, out=FAKE,
                   h=None, stream=None)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.grouped_nf4_gemm_swiglu_bwd(*a.values())

    assert call(dh=None) == -1
    assert "dh" in _last(lib)
    assert call(dh=FAKE + 8) == -1     # dh and h_out need 16 bytes
    assert call(h=FAKE + 2) == -1
    assert call(a=None) == -1
    assert call(out=None) == -1
    assert call(N=120) == -2           # N = 2I with I a multiple of 16
    assert call(K=96) == -2
    assert call(E=0) == -1
    assert call(P=-1) == -1
    assert call(P=0) == 0              # nothing to do: no launch


def test_backward_rejects_bad_arguments_on_the_host(lib):
    lora = binding.LoraStruct(FAKE, FAKE, 8, 2.0, 1)
    base = dict(x=FAKE, x_dtype=1, logits=FAKE, dy=FAKE, dy_dtype=1, T=4, H=64, I=64, E=4,
                k=2, renorm=1, gup=FAKE, gua=FAKE, dnp=FAKE, dna=FAKE, gul=None, dnl=None,
                dx=FAKE, dx_dtype=1, dAg=None, dBg=None, dAd=None, dBd=None, ws=FAKE,
                ws_bytes=1 << 30, stream=None)

    def call(**kw):
        a = dict(base, **kw)
        return lib.moe_expert_backward(*a.values())

    assert call(dy=None) == -1
    assert call(dy_dtype=0) == -5
    assert call(dx_dtype=9) == -5
    assert call(H=96) == -2
    assert call(k=5) == -4
    assert call(gul=ctypes.pointer(lora)) == -1        # dA_gu / dB_gu missing
    assert "d_gu_A" in _last(lib)
    small = lib.moe_expert_backward_workspace(4, 64, 64, 4, 2, 0)
    assert small > 0
    assert lib.moe_expert_backward_workspace(4, 64, 64, 4, 2, 8) > small
    assert lib.moe_expert_backward_workspace(4, 64, 64, 4, 2, 17) == 0
    assert call(ws_bytes=small - 1) == -6
    assert lib.moe_expert_backward_nbit(9, *base.values()) == -1


def test_mxfp4_entry_points_check_shapes_on_the_host(lib):
    # K must be a multiple of 128 (whole dwords of scale bytes per row)
    assert lib.grouped_mxfp4_gemm(FAKE, 2, 8, None, 1, FAKE, FAKE, FAKE, 1, 8, 64, 192, 0,
                                  None, None, FAKE, 2, None) == -2
    assert "128" in _last(lib)
    assert lib.grouped_mxfp4_gemm(None, 2, 8, None, 1, FAKE, FAKE, FAKE, 1, 8, 64, 256, 0,
                                  None, None, FAKE, 2, None) == -1
    assert lib.moe_expert_forward_mxfp4(FAKE, 1, FAKE, 4, 192, 128, 4, 2, 1, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, 1, FAKE, 1 << 30, None) == -2


def test_f16_range_check_validation(lib):
    f = lib.nf4moe_f16_range_check
    assert f(None, 1, 8, FAKE, None) == -1
    assert f(FAKE, 1, 8, None, None) == -1
    assert f(FAKE, 1, 0, FAKE, None) == -1
    assert f(FAKE, 2, 8, FAKE, None) == -5  # F16 values need no check
    assert f(FAKE + 4, 0, 8, FAKE, None) == -1  # F32 needs 16 bytes
    assert f(FAKE, 1, 8, FAKE + 2, None) == -1
