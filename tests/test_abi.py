"""The C-ABI library loads, exports every entry point that include/fr.h
declares, and rejects bad arguments on the host before any HIP call (CPU
only: no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import memory_bound_amd as fr
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fr.h")

# fake, 16-byte aligned, never dereferenced device addresses
A, B, C, D_, E, F, G = (0x10000 * (i + 1) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fr_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_ops_and_helpers():
    names = declared_functions()
    assert names == sorted([
        "fr_resid_rmsnorm_fp8", "fr_adarms_gate_res_fp8",
        "fr_qkv_normrope_kvwrite", "fr_gated_act_fp8", "fr_gemm_gated_act_fp8",
        "fr_gemm_pack_weights", "fr_resid_rmsnorm_mxfp4", "fr_gated_act_mxfp4",
        "fr_resid_rmsnorm_nvfp4",
        "fr_decode_chain_persistent", "fr_qk_norm_rope", "fr_resid_layernorm_fp8",
        "fr_resid_layernorm_mxfp4", "fr_resid_layernorm_nvfp4", "fr_status_string",
        "fr_abi_version"])


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fr.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\S+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(fr.lib, name)
    # nothing else with the public prefix leaks out
    assert {n for n in exported if n.startswith("fr_")} == set(declared_functions())


def test_abi_version_and_status_strings():
    assert fr.abi_version() == 3
    for s in range(8):
        assert fr.status_string(s).startswith("FR_")
    assert fr.status_string(99) == "unknown fr_status"


def rms(**kw):
    args = dict(x=A, residual=B, residual_out=C, weight=D_, wmode=fr.W_NONE,
                eps=1e-6, out_fp8=E, qmode=fr.Q_STATIC, static_scale=56.0,
                out_scales=F, T=10, H=1024, dtype=fr.F16)
    args.update(kw)
    L = fr.lib
    return L.fr_resid_rmsnorm_fp8(*(fr._ptr(args[k]) if k in (
        "x", "residual", "residual_out", "weight", "out_fp8", "out_scales")
        else args[k] for k in ("x", "residual", "residual_out", "weight",
                               "wmode", "eps", "out_fp8", "qmode",
                               "static_scale", "out_scales", "T", "H",
                               "dtype")), None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fr.FR_ERR_NULL),
    (dict(out_fp8=None), fr.FR_ERR_NULL),
    (dict(wmode=fr.W_MUL, weight=None), fr.FR_ERR_NULL),
    (dict(qmode=fr.Q_TOKEN, out_scales=None), fr.FR_ERR_NULL),
    (dict(x=A + 8), fr.FR_ERR_ALIGN),
    (dict(out_fp8=E + 4), fr.FR_ERR_ALIGN),
    (dict(H=1000), fr.FR_ERR_SHAPE),
    (dict(H=0), fr.FR_ERR_SHAPE),
    (dict(T=-1), fr.FR_ERR_SHAPE),
    (dict(H=32768 + 16), fr.FR_ERR_UNSUPPORTED),
    (dict(dtype=2), fr.FR_ERR_DTYPE),
    (dict(wmode=3), fr.FR_ERR_MODE),
    (dict(qmode=2), fr.FR_ERR_MODE),
    (dict(eps=-1.0), fr.FR_ERR_MODE),
    (dict(eps=float("nan")), fr.FR_ERR_MODE),
    (dict(static_scale=0.0), fr.FR_ERR_MODE),
    (dict(static_scale=float("inf")), fr.FR_ERR_MODE),
    (dict(T=0), fr.FR_OK),
])
def test_resid_rmsnorm_validation(kw, status):
    assert rms(**kw) == status


def test_adarms_validation():
    L = fr.lib
    ok = [A, B, C, D_, E, F, 1e-6, G, fr.Q_STATIC, 56.0, None, 10, 1024,
          fr.F16, None]
    assert L.fr_adarms_gate_res_fp8(*ok[:11], 0, *ok[12:]) == fr.FR_OK
    bad = list(ok)
    bad[1] = None
    assert L.fr_adarms_gate_res_fp8(*bad) == fr.FR_ERR_NULL
    bad = list(ok)
    bad[4] = E + 2
    assert L.fr_adarms_gate_res_fp8(*bad) == fr.FR_ERR_ALIGN
    bad = list(ok)
    bad[8] = fr.Q_TOKEN
    assert L.fr_adarms_gate_res_fp8(*bad) == fr.FR_ERR_NULL
    bad = list(ok)
    bad[12] = 24
    assert L.fr_adarms_gate_res_fp8(*bad) == fr.FR_ERR_SHAPE


def qkv(**kw):
    args = dict(qkv=A, q_norm_w=None, k_norm_w=None, eps=1e-6, positions=B,
                rope_theta=1e4, rope_style=fr.ROPE_HALF, q_scale=1.0, q_out=C, k_cache=D_,
                v_cache=E, page_table=F, page_table_len=1, page_size=1024,
                num_pages=1, err_flag=None, T=10, Hq=8, Hkv=1, D=256,
                dtype=fr.F16)
    args.update(kw)
    order = ["qkv", "q_norm_w", "k_norm_w", "eps", "positions", "rope_theta",
             "rope_style", "q_scale", "q_out", "k_cache", "v_cache", "page_table",
             "page_table_len", "page_size", "num_pages", "err_flag", "T", "Hq",
             "Hkv", "D", "dtype"]
    return fr.lib.fr_qkv_normrope_kvwrite(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), fr.FR_ERR_NULL),
    (dict(positions=None), fr.FR_ERR_NULL),
    (dict(page_table=None), fr.FR_ERR_NULL),
    (dict(D=100), fr.FR_ERR_SHAPE),
    (dict(D=512), fr.FR_ERR_UNSUPPORTED),
    (dict(Hkv=0), fr.FR_ERR_SHAPE),
    (dict(page_size=0), fr.FR_ERR_SHAPE),
    (dict(page_table_len=0), fr.FR_ERR_SHAPE),
    (dict(num_pages=0), fr.FR_ERR_SHAPE),
    (dict(rope_style=2), fr.FR_ERR_MODE),
    (dict(rope_theta=1.0), fr.FR_ERR_MODE),
    (dict(rope_theta=float("nan")), fr.FR_ERR_MODE),
    (dict(q_scale=0.0), fr.FR_ERR_MODE),
    (dict(q_scale=float("inf")), fr.FR_ERR_MODE),
    (dict(q_scale=-0.125), fr.FR_ERR_MODE),
    (dict(q_norm_w=G + 8), fr.FR_ERR_ALIGN),
    (dict(positions=B + 2), fr.FR_ERR_ALIGN),
    (dict(err_flag=G + 1), fr.FR_ERR_ALIGN),
    (dict(dtype=-1), fr.FR_ERR_DTYPE),
    (dict(T=0), fr.FR_OK),
])
def test_qkv_validation(kw, status):
    assert qkv(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fr.FR_ERR_NULL),
    (dict(out_scales=None), fr.FR_ERR_NULL),
    (dict(wmode=fr.W_MUL, weight=None), fr.FR_ERR_NULL),
    (dict(out_fp4=E + 4), fr.FR_ERR_ALIGN),
    (dict(out_scales=F + 1), fr.FR_OK),                         # byte stores: any alignment
    (dict(H=1032), fr.FR_ERR_SHAPE),
    (dict(H=32768 + 16), fr.FR_ERR_UNSUPPORTED),
    (dict(wmode=3), fr.FR_ERR_MODE),
    (dict(global_scale=0.0), fr.FR_ERR_MODE),
    (dict(global_scale=float("inf")), fr.FR_ERR_MODE),
    (dict(global_scale=-1.0), fr.FR_ERR_MODE),
    (dict(dtype=7), fr.FR_ERR_DTYPE),
    (dict(T=0), fr.FR_OK),
])
def test_resid_rmsnorm_nvfp4_validation(kw, status):
    args = dict(x=A, residual=B, residual_out=C, weight=D_, wmode=fr.W_NONE,
                eps=1e-6, global_scale=1.0 / 448, out_fp4=E, out_scales=F, T=0, H=1040,
                dtype=fr.F16)
    args.update(kw)
    order = ["x", "residual", "residual_out", "weight", "wmode", "eps", "global_scale",
             "out_fp4", "out_scales", "T", "H", "dtype"]
    assert fr.lib.fr_resid_rmsnorm_nvfp4(*[args[k] for k in order], None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 0, B, C, 10, 6144, fr.BF16), fr.FR_ERR_NULL),
    ((A, 0, B, None, 10, 6144, fr.BF16), fr.FR_ERR_NULL),
    ((A, 3, B, C, 10, 6144, fr.BF16), fr.FR_ERR_MODE),
    ((A, 0, B, C, 10, 6100, fr.BF16), fr.FR_ERR_SHAPE),
    ((A, 0, B, C, -2, 6144, fr.BF16), fr.FR_ERR_SHAPE),
    ((A, 0, B + 4, C, 10, 6144, fr.BF16), fr.FR_ERR_ALIGN),
    ((A, 0, B, C, 10, 6144, 5), fr.FR_ERR_DTYPE),
    ((A, 0, B, C, 0, 6144, fr.BF16), fr.FR_OK),
])
def test_gated_act_validation(args, status):
    assert fr.lib.fr_gated_act_fp8(*args, None) == status


def test_binding_raises_on_bad_arguments():
    with pytest.raises(fr.FrError) as e:
        fr.fr_gated_act_fp8(A, 0, B, C, 10, 100, fr.BF16, stream=0)
    assert e.value.status == fr.FR_ERR_SHAPE


@pytest.mark.parametrize("args,status", [
    ((None, B, C, D_, 0, E, F, 10, 2048, 6144), fr.FR_ERR_NULL),
    ((A, B, C, D_, 0, E, None, 10, 2048, 6144), fr.FR_ERR_NULL),
    ((A, B, C, D_, 3, E, F, 10, 2048, 6144), fr.FR_ERR_MODE),
    ((A, B, C, D_, 0, E, F, 10, 2000, 6144), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, 0, E, F, 10, 2048, 6100), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, 0, E, F, -1, 2048, 6144), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, 0, E, F, 10, 16384 + 128, 6144), fr.FR_ERR_UNSUPPORTED),
    ((A + 8, B, C, D_, 0, E, F, 10, 2048, 6144), fr.FR_ERR_ALIGN),
    ((A, B + 2, C, D_, 0, E, F, 10, 2048, 6144), fr.FR_ERR_ALIGN),
    ((A, B, C, D_, 0, E, F, 0, 2048, 6144), fr.FR_OK),
])
def test_gemm_gated_act_validation(args, status):
    assert fr.lib.fr_gemm_gated_act_fp8(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, B, 64, 256), fr.FR_ERR_NULL),
    ((A, None, 64, 256), fr.FR_ERR_NULL),
    ((A, B, 48, 256), fr.FR_ERR_SHAPE),
    ((A, B, 64, 200), fr.FR_ERR_SHAPE),
    ((A, B, -32, 256), fr.FR_ERR_SHAPE),
    ((A, B, 64, 16384 + 128), fr.FR_ERR_UNSUPPORTED),
    ((A + 4, B, 64, 256), fr.FR_ERR_ALIGN),
    ((A, B + 8, 64, 256), fr.FR_ERR_ALIGN),
    ((A, B, 0, 256), fr.FR_OK),
])
def test_gemm_pack_weights_validation(args, status):
    assert fr.lib.fr_gemm_pack_weights(*args, None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fr.FR_ERR_NULL),
    (dict(out_scales=None), fr.FR_ERR_NULL),
    (dict(wmode=fr.W_MUL, weight=None), fr.FR_ERR_NULL),
    (dict(out_fp4=E + 4), fr.FR_ERR_ALIGN),
    (dict(H=1040), fr.FR_ERR_SHAPE),
    (dict(H=32768 + 32), fr.FR_ERR_UNSUPPORTED),
    (dict(wmode=3), fr.FR_ERR_MODE),
    (dict(eps=-1.0), fr.FR_ERR_MODE),
    (dict(dtype=7), fr.FR_ERR_DTYPE),
    (dict(T=0), fr.FR_OK),
])
def test_resid_rmsnorm_mxfp4_validation(kw, status):
    args = dict(x=A, residual=B, residual_out=C, weight=D_, wmode=fr.W_NONE,
                eps=1e-6, out_fp4=E, out_scales=F, T=10, H=1024, dtype=fr.F16)
    args.update(kw)
    order = ["x", "residual", "residual_out", "weight", "wmode", "eps",
             "out_fp4", "out_scales", "T", "H", "dtype"]
    assert fr.lib.fr_resid_rmsnorm_mxfp4(*[args[k] for k in order], None) == status


@pytest.mark.parametrize("args,status", [
    ((None, 0, B, C, 10, 6144, fr.BF16), fr.FR_ERR_NULL),
    ((A, 0, B, None, 10, 6144, fr.BF16), fr.FR_ERR_NULL),
    ((A, 3, B, C, 10, 6144, fr.BF16), fr.FR_ERR_MODE),
    ((A, 0, B, C, 10, 6112, fr.BF16), fr.FR_ERR_SHAPE),
    ((A, 0, B + 2, C, 10, 6144, fr.BF16), fr.FR_ERR_ALIGN),
    ((A, 0, B, C + 2, 10, 6144, fr.BF16), fr.FR_ERR_ALIGN),     # E8M0 codes: 4-byte stores
    ((A, 0, B, C, 10, 6144, 9), fr.FR_ERR_DTYPE),
    ((A, 0, B, C, 0, 6144, fr.BF16), fr.FR_OK),
])
def test_gated_act_mxfp4_validation(args, status):
    assert fr.lib.fr_gated_act_mxfp4(*args, None) == status


def chain(**kw):
    args = dict(x=A, gate=B, ada_scale=C, ada_shift=D_, residual=E, out_fp8=F,
                eps=1e-6, static_scale=56.0, qkv=G, positions=A, rope_theta=1e4,
                rope_style=fr.ROPE_HALF, q_out=B, k_cache=C, v_cache=D_,
                page_table=E, page_table_len=1, page_size=1024, num_pages=1,
                err_flag=None, layers=18, steps=10, T=10, H=1024, Hq=8, Hkv=1,
                D=256, dtype=fr.F16)
    args.update(kw)
    order = ["x", "gate", "ada_scale", "ada_shift", "residual", "out_fp8", "eps",
             "static_scale", "qkv", "positions", "rope_theta", "rope_style",
             "q_out", "k_cache", "v_cache", "page_table", "page_table_len",
             "page_size", "num_pages", "err_flag", "layers", "steps", "T", "H",
             "Hq", "Hkv", "D", "dtype"]
    return fr.lib.fr_decode_chain_persistent(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), fr.FR_ERR_NULL),
    (dict(page_table=None), fr.FR_ERR_NULL),
    (dict(T=65), fr.FR_ERR_UNSUPPORTED),
    (dict(H=2048), fr.FR_ERR_UNSUPPORTED),
    (dict(D=512), fr.FR_ERR_UNSUPPORTED),
    (dict(H=1000), fr.FR_ERR_SHAPE),
    (dict(layers=0), fr.FR_ERR_SHAPE),
    (dict(static_scale=0.0), fr.FR_ERR_MODE),
    (dict(rope_style=5), fr.FR_ERR_MODE),
    (dict(q_out=B + 8), fr.FR_ERR_ALIGN),
    (dict(dtype=3), fr.FR_ERR_DTYPE),
    (dict(T=0), fr.FR_OK),
])
def test_decode_chain_persistent_validation(kw, status):
    assert chain(**kw) == status


def qknr(**kw):
    args = dict(qkv=A, norm_kind=1, norm_scope=0, q_norm_w=None, q_norm_b=None,
                k_norm_w=None, k_norm_b=None, eps=1e-6, positions=B, rope_dims=1,
                sec_t=0, sec_h=0, sec_w=0, rope_theta=1e4, rope_style=0, q_scale=1.0,
                q_out=C, k_out=D_, v_out=E, T=10, Hq=8, Hkv=2, D=128, dtype=fr.BF16)
    args.update(kw)
    order = ["qkv", "norm_kind", "norm_scope", "q_norm_w", "q_norm_b", "k_norm_w",
             "k_norm_b", "eps", "positions", "rope_dims", "sec_t", "sec_h", "sec_w",
             "rope_theta", "rope_style", "q_scale", "q_out", "k_out", "v_out", "T",
             "Hq", "Hkv", "D", "dtype"]
    return fr.lib.fr_qk_norm_rope(*[args[k] for k in order], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), fr.FR_ERR_NULL),
    (dict(v_out=None), fr.FR_ERR_NULL),
    (dict(norm_kind=3), fr.FR_ERR_MODE),
    (dict(norm_scope=2), fr.FR_ERR_MODE),
    (dict(rope_dims=2), fr.FR_ERR_MODE),
    (dict(rope_dims=3, sec_t=20, sec_h=20, sec_w=20), fr.FR_ERR_SHAPE),
    (dict(rope_dims=3, sec_t=64, sec_h=0, sec_w=0), fr.FR_ERR_SHAPE),
    (dict(rope_dims=3, sec_t=22, sec_h=21, sec_w=21), fr.FR_OK),
    (dict(D=100), fr.FR_ERR_SHAPE),
    (dict(D=512), fr.FR_ERR_UNSUPPORTED),
    (dict(Hq=300, Hkv=20), fr.FR_ERR_UNSUPPORTED),
    (dict(q_scale=0.0), fr.FR_ERR_MODE),
    (dict(q_norm_w=F + 4), fr.FR_ERR_ALIGN),
    (dict(positions=B + 2), fr.FR_ERR_ALIGN),
    (dict(dtype=4), fr.FR_ERR_DTYPE),
    (dict(T=0), fr.FR_OK),
])
def test_qk_norm_rope_validation(kw, status):
    kw = dict(kw)
    if kw.get("rope_dims") == 3 and kw.get("sec_t") == 22:
        kw["T"] = 0                       # valid sections; launch nothing
    assert qknr(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, None, None, 1e-6, E, 0, 56.0, None, 10, 1024, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, G + 2, 1e-6, E, 0, 56.0, None, 10, 1024, fr.F16), fr.FR_ERR_ALIGN),
    ((A, B, C, D_, None, 1e-6, E, 1, 0.0, None, 10, 1024, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, None, 1e-6, E, 0, 56.0, None, 10, 1000, fr.F16), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, G, 1e-6, E, 0, 56.0, None, 0, 1024, fr.F16), fr.FR_OK),
])
def test_resid_layernorm_fp8_validation(args, status):
    assert fr.lib.fr_resid_layernorm_fp8(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, None, None, 1e-6, E, F, 10, 1024, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, None, 1e-6, E, None, 10, 1024, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, None, 1e-6, E, F, 10, 1040, fr.F16), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, None, 1e-6, E + 8, F, 10, 1024, fr.F16), fr.FR_ERR_ALIGN),
    ((A, B, C, D_, G, 1e-6, E, F, 0, 1024, fr.F16), fr.FR_OK),
])
def test_resid_layernorm_mxfp4_validation(args, status):
    assert fr.lib.fr_resid_layernorm_mxfp4(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, None, None, 1e-6, 0.02, E, F, 10, 1040, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, None, 1e-6, 0.02, E, None, 10, 1040, fr.F16), fr.FR_ERR_NULL),
    ((A, B, C, D_, None, 1e-6, 0.02, E, F, 10, 1032, fr.F16), fr.FR_ERR_SHAPE),
    ((A, B, C, D_, None, 1e-6, 0.02, E, F, 10, 32784, fr.F16), fr.FR_ERR_UNSUPPORTED),
    ((A, B, C, D_, None, 1e-6, 0.0, E, F, 10, 1040, fr.F16), fr.FR_ERR_MODE),
    ((A, B, C, D_, None, 1e-6, float("nan"), E, F, 10, 1040, fr.F16), fr.FR_ERR_MODE),
    ((A, B, C, D_, None, -1.0, 0.02, E, F, 10, 1040, fr.F16), fr.FR_ERR_MODE),
    ((A, B, C, D_, None, 1e-6, 0.02, E + 8, F, 10, 1040, fr.F16), fr.FR_ERR_ALIGN),
    ((A, B, C, D_, G + 4, 1e-6, 0.02, E, F, 10, 1040, fr.F16), fr.FR_ERR_ALIGN),
    ((A, B, C, D_, None, 1e-6, 0.02, E, F + 1, 0, 1040, fr.F16), fr.FR_OK),
    ((A, B, C, D_, None, 1e-6, 0.02, E, F, 10, 1040, 9), fr.FR_ERR_DTYPE),
    ((A, B, C, D_, G, 1e-6, 0.02, E, F, 0, 1040, fr.BF16), fr.FR_OK),
])
def test_resid_layernorm_nvfp4_validation(args, status):
    """Add + LayerNorm -> NVFP4: H % 16, the tensor scale, alignment (the
    block-scale codes may sit at any byte), dtype; no launch happens (T = 0
    or an error)."""
    assert fr.lib.fr_resid_layernorm_nvfp4(*args, None) == status
