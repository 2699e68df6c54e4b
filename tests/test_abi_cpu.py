"""The C ABI library on the CPU (no GPU needed): it loads, exports every
function include/moe_mi355x.h declares, and refuses invalid arguments on the
host before any HIP call, with a message."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_top_amd as m

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_mi355x.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+[\s\*]+(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = m.lib()
    names = _declared_functions()
    assert set(names) >= {"moe_route", "moe_build_indices", "moe_grouped_ffn", "moe_combine"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert set(names) == set(m.ENTRY_POINTS)
    assert lib.moe_abi_version() == 8


def test_struct_layouts_match_header_sizes():
    # pointer-size fields and natural alignment: these sizes follow from the header
    assert ctypes.sizeof(m.RouteArgs) == 6 * 4 + 3 * 8 + 8 + 3 * 8 + 4 + 4 + 3 * 8 + 8   # + router_dtype, padded
    assert ctypes.sizeof(m.CombineArgs) == 3 * 4 + 4 + 8 + 4 + 4 + 8 * 4 + 4 + 4 + 2 * 8


STRUCTS = {"RouteArgs": "moe_route_args_t", "IndexArgs": "moe_index_args_t",
           "FfnArgs": "moe_ffn_args_t", "CombineArgs": "moe_combine_args_t",
           "CombineBwdArgs": "moe_combine_backward_args_t", "FfnBwdArgs": "moe_ffn_backward_args_t"}


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """Every binding struct has the size and field offsets that a C compiler
    gives the header's struct (gcc on this host, same ABI as the library)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for py, c in STRUCTS.items():
        lines.append(f'printf("{py} size %zu\\n", sizeof({c}));')
        for name, _ in getattr(m, py)._fields_:
            lines.append(f'printf("{py} {name} %zu\\n", offsetof({c}, {name}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {(a, b): int(v) for a, b, v in (ln.split() for ln in out if ln)}
    for py in STRUCTS:
        cls = getattr(m, py)
        assert got[(py, "size")] == ctypes.sizeof(cls), py
        for name, _ in cls._fields_:
            assert got[(py, name)] == getattr(cls, name).offset, f"{py}.{name}"


def _err(fn, args):
    st = fn(ctypes.byref(args), None)
    return st, m.lib().moe_last_error_message().decode()


def _route(**kw):
    base = dict(router_kind=0, num_tokens=4, n_routed_experts=8, n_experts_per_tok=2, n_shared_experts=0,
                hidden_dim=64, x=16, w_gate=32, logits=None, logits_ld=0, route_scale=1.0, renormalize=1,
                expert_indices=48, expert_weights=64)
    base.update(kw)
    return m.RouteArgs(**base)


@pytest.mark.parametrize("kw,frag", [
    (dict(n_experts_per_tok=9), "n_experts_per_tok"),
    (dict(n_experts_per_tok=0), "n_experts_per_tok"),
    (dict(n_routed_experts=0), "n_routed_experts"),
    (dict(num_tokens=-1), "num_tokens"),
    (dict(n_shared_experts=2), "sink"),
    (dict(expert_bias=80), "expert_bias"),
    (dict(hidden_dim=60), "hidden_dim"),
    (dict(hidden_dim=(1 << 22) + 8), "hidden_dim"),
    (dict(x=17), "aligned"),
    (dict(n_routed_experts=200, n_experts_per_tok=2), "<= 128"),
    (dict(x=None, w_gate=None, logits=96, logits_ld=4), "logits_ld"),
    (dict(router_kind=1, x=None, w_gate=None, logits=96, logits_ld=8, n_experts_per_tok=3), "power of two"),
    (dict(router_kind=1, x=None, w_gate=None, logits=96, logits_ld=8, n_experts_per_tok=2,
          n_shared_experts=2), "logits_ld"),
    (dict(router_kind=1, x=None, w_gate=None, logits=96, logits_ld=10, n_experts_per_tok=2,
          n_shared_experts=2), "sink_weights"),
    (dict(router_kind=1, x=None, w_gate=None, logits=96, logits_ld=200, n_routed_experts=128,
          n_experts_per_tok=64, n_shared_experts=64), "power of two"),
    (dict(router_kind=7), "router_kind"),
    (dict(expert_indices=None), "required"),
    (dict(route_scale=float("inf")), "route_scale"),
])
def test_route_validation(kw, frag):
    st, msg = _err(m.lib().moe_route, _route(**kw))
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


def _ffn(**kw):
    base = dict(max_rows=64, hidden_dim=256, moe_dim=512, n_local_experts=8, expert_offsets=16,
                operand_dtype=0, x_perm=32, w_gate_up=48, w_gate_up_layout=1, gate_up_format=0, w_down=64,
                w_down_layout=1, activation=0, alpha=0.0, limit=0.0, act_workspace=80,
                act_workspace_bytes=1 << 20, out_dtype=2, expert_out=96)
    base.update(kw)
    return m.FfnArgs(**base)


@pytest.mark.parametrize("kw,status,frag", [
    (dict(alpha=1.0), m.MOE_ERR_INVALID_ARGUMENT, "alpha"),
    (dict(activation=2, limit=7.0), m.MOE_ERR_INVALID_ARGUMENT, "gelu_tanh"),
    (dict(limit=-1.0), m.MOE_ERR_INVALID_ARGUMENT, "limit"),
    (dict(activation=5), m.MOE_ERR_INVALID_ARGUMENT, "activation"),
    (dict(hidden_dim=250), m.MOE_ERR_INVALID_ARGUMENT, "hidden_dim"),
    (dict(moe_dim=0), m.MOE_ERR_INVALID_ARGUMENT, "moe_dim"),
    (dict(n_local_experts=0), m.MOE_ERR_INVALID_ARGUMENT, "n_local_experts"),
    (dict(n_local_experts=2000), m.MOE_ERR_INVALID_ARGUMENT, "n_local_experts"),
    (dict(gate_up_format=3), m.MOE_ERR_INVALID_ARGUMENT, "gate_up_format"),
    (dict(out_dtype=1), m.MOE_ERR_INVALID_ARGUMENT, "out_dtype"),
    (dict(x_perm=None), m.MOE_ERR_INVALID_ARGUMENT, "gather"),
    (dict(x=128, sorted_token=144), m.MOE_ERR_INVALID_ARGUMENT, "not both"),
    (dict(w_down=None), m.MOE_ERR_INVALID_ARGUMENT, "w_down"),
    (dict(expert_out=100), m.MOE_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(act_workspace_bytes=100), m.MOE_ERR_WORKSPACE_TOO_SMALL, "act_workspace"),
    (dict(operand_dtype=1, hidden_dim=200), m.MOE_ERR_INVALID_ARGUMENT, "128"),
    (dict(operand_dtype=9), m.MOE_ERR_INVALID_ARGUMENT, "operand_dtype"),
    # MX (MXFP4 weights x MXFP8 activations)
    (dict(operand_dtype=4, hidden_dim=224, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144),
     m.MOE_ERR_INVALID_ARGUMENT, "128"),
    (dict(operand_dtype=4, w_gate_up_scale=128, w_down_scale=144), m.MOE_ERR_INVALID_ARGUMENT, "x_perm_scale"),
    (dict(operand_dtype=4, x_perm_scale=112), m.MOE_ERR_INVALID_ARGUMENT, "w_gate_up_scale"),
    (dict(operand_dtype=4, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144, b_down=170),
     m.MOE_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(operand_dtype=4, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144, w_down_layout=0),
     m.MOE_ERR_UNSUPPORTED, "OUT_IN"),
    # the gather form bounds x [num_tokens, hidden_dim] (or, without num_tokens, max_rows x hidden_dim)
    (dict(x_perm=None, x=128, sorted_token=144, num_tokens=1 << 19, hidden_dim=4096, act_workspace_bytes=1 << 22),
     m.MOE_ERR_INVALID_ARGUMENT,
     "num_tokens x hidden_dim"),
    (dict(x_perm=None, x=128, sorted_token=144, max_rows=1 << 19, hidden_dim=4096,
          act_workspace_bytes=1 << 40), m.MOE_ERR_INVALID_ARGUMENT, "pass num_tokens"),
    # bf16 reads the stacked (IN_OUT) gate_up weights in the concatenated format only
    (dict(w_gate_up_layout=0, gate_up_format=1, act_workspace_bytes=1 << 21), m.MOE_ERR_UNSUPPORTED, "concatenated"),
    (dict(operand_dtype=1, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144, w_gate_up_layout=0),
     m.MOE_ERR_UNSUPPORTED, "OUT_IN"),
])
def test_grouped_ffn_validation(kw, status, frag):
    st, msg = _err(m.lib().moe_grouped_ffn, _ffn(**kw))
    assert st == status and frag in msg, msg


@pytest.mark.parametrize("kw,status,frag", [
    (dict(hidden_dim=96), m.MOE_ERR_INVALID_ARGUMENT, "64"),
    (dict(moe_dim=200), m.MOE_ERR_INVALID_ARGUMENT, "128"),
    (dict(operand_dtype=1), m.MOE_ERR_INVALID_ARGUMENT, "BF16"),
    (dict(alpha=1.0), m.MOE_ERR_INVALID_ARGUMENT, "alpha"),
    (dict(x_perm=None), m.MOE_ERR_INVALID_ARGUMENT, "gather"),
    (dict(w_gate_up_layout=0), m.MOE_ERR_UNSUPPORTED, "OUT_IN"),
    (dict(act_workspace_bytes=64 * 512 * 2), m.MOE_ERR_WORKSPACE_TOO_SMALL, "act_workspace"),
    (dict(operand_dtype=m.DTYPE_FP8_E4M3_TOKENS), m.MOE_ERR_INVALID_ARGUMENT, "MXFP4_W4A16"),
    # W4A16: bf16 activations (no x_perm_scale), MXFP4 weight scales
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A16, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144),
     m.MOE_ERR_INVALID_ARGUMENT, "no x_perm_scale"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A16, w_gate_up_scale=128), m.MOE_ERR_INVALID_ARGUMENT, "w_down_scale"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A16, w_gate_up_scale=128, w_down_scale=144, hidden_dim=192),
     m.MOE_ERR_INVALID_ARGUMENT, "128"),
    # MXFP4 x MXFP8: hidden_dim in whole 128-element stages, the activation and weight scales
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, hidden_dim=192, x_perm_scale=112, w_gate_up_scale=128,
          w_down_scale=144), m.MOE_ERR_INVALID_ARGUMENT, "128"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, w_gate_up_scale=128, w_down_scale=144), m.MOE_ERR_INVALID_ARGUMENT,
     "x_perm_scale"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, x_perm_scale=112, w_down_scale=144), m.MOE_ERR_INVALID_ARGUMENT,
     "w_gate_up_scale"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, x_perm_scale=116, w_gate_up_scale=128, w_down_scale=144),
     m.MOE_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144,
          w_down_layout=0), m.MOE_ERR_UNSUPPORTED, "OUT_IN"),
    # gather form: x holds num_tokens rows of codes, which must stay under 2 GiB
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, x_perm=None, x=128, sorted_token=144, x_perm_scale=112,
          w_gate_up_scale=128, w_down_scale=144, num_tokens=1 << 22, hidden_dim=1024, act_workspace_bytes=1 << 40),
     m.MOE_ERR_INVALID_ARGUMENT, "2 GiB"),
    (dict(operand_dtype=m.DTYPE_MXFP4_W4A8, x_perm_scale=112, w_gate_up_scale=128, w_down_scale=144,
          act_workspace_bytes=64 * 512 * 2), m.MOE_ERR_WORKSPACE_TOO_SMALL, "act_workspace"),
])
def test_grouped_ffn_fused_validation(kw, status, frag):
    st, msg = _err(m.lib().moe_grouped_ffn_fused, _ffn(**kw))
    assert st == status and frag in msg, msg


def test_fused_workspace_bytes():
    lib = m.lib()
    hdr = 1280    # 4 control words + 256 split counters, rounded up to 256 bytes

    def rb(R, L):  # bound on the 32-row blocks: ceil(R/32) plus one partial block per expert with rows
        return -(-R // 32) + min(L, R)

    def up(b):
        return -(-b // 256) * 256

    # D < 3 H: no split, so no partial tiles
    assert lib.moe_ffn_fused_workspace_bytes(64, 512, 256, 8) == hdr + 64 * 256 * 2 + up(4 * rb(64, 8))
    assert lib.moe_ffn_fused_workspace_bytes(64, 512, 1408, 8) == hdr + 64 * 1408 * 2 + up(4 * rb(64, 8))
    # Mixtral decode, 128 rows: D/H = 3.5 -> 2 parts; 12 row blocks x 16 column tiles = 192 tiles
    assert lib.moe_ffn_fused_workspace_bytes(128, 4096, 14336, 8) == (
        hdr + 128 * 14336 * 2 + 192 * 2 * 32 * 256 * 4 + up(4 * 12))
    # many rows: the split tiles are capped at 256
    assert lib.moe_ffn_fused_workspace_bytes(8192, 4096, 14336, 8) == (
        hdr + 8192 * 14336 * 2 + 256 * 2 * 32 * 256 * 4 + up(4 * rb(8192, 8)))
    # parts are capped at 8
    assert lib.moe_ffn_fused_workspace_bytes(32, 256, 8192, 1) == hdr + 32 * 8192 * 2 + 2 * 8 * 32 * 256 * 4 + 256
    # a smaller max_rows needs no more
    assert lib.moe_ffn_fused_workspace_bytes(17, 4096, 14336, 8) <= lib.moe_ffn_fused_workspace_bytes(128, 4096, 14336, 8)
    # MX: A is e4m3 codes and one scale byte per 32, each region rounded to
    # 256 bytes, which the bf16 size covers except for the tiniest rows x moe_dim
    assert lib.moe_ffn_fused_workspace_bytes(1, 128, 128, 1) == hdr + 256 + 256 + up(4 * rb(1, 1))
    assert lib.moe_ffn_fused_workspace_bytes(0, 4096, 14336, 8) == hdr
    assert lib.moe_ffn_fused_workspace_bytes(-1, 4096, 14336, 8) == 0


def _idx(**kw):
    base = dict(num_tokens=16, n_experts_per_tok=2, experts_start_idx=0, n_local_experts=8, expert_indices=16,
                expert_offsets=32, sorted_token=48, row_of_slot=64, workspace=80, workspace_bytes=1 << 16)
    base.update(kw)
    return m.IndexArgs(**base)


@pytest.mark.parametrize("kw,status,frag", [
    (dict(n_local_experts=0), m.MOE_ERR_INVALID_ARGUMENT, "n_local_experts"),
    (dict(n_experts_per_tok=0), m.MOE_ERR_INVALID_ARGUMENT, "n_experts_per_tok"),
    (dict(num_tokens=-3), m.MOE_ERR_INVALID_ARGUMENT, "num_tokens"),
    (dict(num_tokens=1 << 30, n_experts_per_tok=4), m.MOE_ERR_INVALID_ARGUMENT, "2^31"),
    (dict(expert_offsets=None), m.MOE_ERR_INVALID_ARGUMENT, "expert_offsets"),
    (dict(workspace_bytes=4), m.MOE_ERR_WORKSPACE_TOO_SMALL, "workspace"),
    (dict(x=96, hidden_dim=256), m.MOE_ERR_INVALID_ARGUMENT, "x_perm"),
    (dict(x=96, hidden_dim=250, x_perm=112), m.MOE_ERR_INVALID_ARGUMENT, "hidden_dim"),
    (dict(x=96, hidden_dim=200, x_perm=112, xperm_dtype=1, x_perm_scale=128), m.MOE_ERR_INVALID_ARGUMENT, "128"),
    (dict(x=96, hidden_dim=256, x_perm=112, xperm_dtype=1), m.MOE_ERR_INVALID_ARGUMENT, "x_perm_scale"),
    (dict(x=96, hidden_dim=240, x_perm=112, xperm_dtype=6, x_perm_scale=128), m.MOE_ERR_INVALID_ARGUMENT, "32"),
    (dict(x=96, hidden_dim=256, x_perm=112, xperm_dtype=5), m.MOE_ERR_INVALID_ARGUMENT, "x_perm_scale"),
    (dict(x=96, hidden_dim=256, x_perm=112, xperm_dtype=7), m.MOE_ERR_INVALID_ARGUMENT, "xperm_dtype"),
])
def test_build_indices_validation(kw, status, frag):
    st, msg = _err(m.lib().moe_build_indices, _idx(**kw))
    assert st == status and frag in msg, msg


@pytest.mark.parametrize("kw,status,frag", [
    (dict(), m.MOE_ERR_INVALID_ARGUMENT, "workspace must be NULL"),          # a workspace is not taken
    (dict(workspace=None, workspace_bytes=0, n_local_experts=0), m.MOE_ERR_INVALID_ARGUMENT, "n_local_experts"),
    # 2^20 tokens x 4 slots = 8192 blocks x 1024 experts x 4 bytes = 32 MiB > the 16 MiB static scratch
    (dict(workspace=None, workspace_bytes=0, num_tokens=1 << 20, n_experts_per_tok=4, n_local_experts=1024),
     m.MOE_ERR_WORKSPACE_TOO_SMALL, "static scratch"),
])
def test_build_indices_noalloc_validation(kw, status, frag):
    """The allocation-free form refuses a workspace argument and any call
    whose per-block counts exceed its static scratch, before any HIP call."""
    st, msg = _err(m.lib().moe_build_indices_noalloc, _idx(**kw))
    assert st == status and frag in msg, msg
    assert m.lib().moe_build_indices_workspace_bytes(1 << 20, 4, 1024) == 32 * 1024 * 1024
    assert m.lib().moe_build_indices_workspace_bytes(1 << 19, 4, 1024) == 16 * 1024 * 1024


@pytest.mark.parametrize("kw,frag", [
    (dict(hidden_dim=100), "hidden_dim"),
    (dict(n_experts_per_tok=0), "n_experts_per_tok"),
    (dict(out_dtype=1), "out_dtype"),
    (dict(y=None), "required"),
    (dict(y=40), "aligned"),
])
def test_combine_validation(kw, frag):
    base = dict(num_tokens=8, n_experts_per_tok=2, hidden_dim=256, expert_out=16, out_dtype=2, row_of_slot=32,
                y=48)
    base.update(kw)
    st, msg = _err(m.lib().moe_combine, m.CombineArgs(**base))
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(n_shared=2), "shared_out"),
    (dict(n_shared=-1), "n_shared"),
    (dict(n_shared=1, shared_out=72), "aligned"),
])
def test_combine_shared_validation(kw, frag):
    base = dict(num_tokens=8, n_experts_per_tok=2, hidden_dim=256, expert_out=16, out_dtype=2, row_of_slot=32,
                y=48)
    base.update(kw)
    st, msg = _err(m.lib().moe_combine, m.CombineArgs(**base))
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


@pytest.mark.parametrize("T,n,off,st_,frag", [
    (-1, 2, 16, 32, "num_tokens"),
    (8, 0, 16, 32, "n_shared"),
    (8, 2, None, 32, "required"),
    (1 << 30, 4, 16, 32, "2^31"),
])
def test_shared_indices_validation(T, n, off, st_, frag):
    lib = m.lib()
    st = lib.moe_shared_indices(T, n, off, st_, None)
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in lib.moe_last_error_message().decode()


def test_workspace_queries_and_status_strings():
    lib = m.lib()
    assert lib.moe_build_indices_workspace_bytes(16384, 8, 256) >= 256 * 32 * 4
    # bf16: A, then 256 split-K arrival counters and min(256, R/16) fp32 256x256 partial tiles
    assert lib.moe_ffn_workspace_bytes(8192, 14336, 0) == 8192 * 14336 * 2 + 256 * 4 + 256 * 256 * 256 * 4
    assert lib.moe_ffn_workspace_bytes(64, 512, 0) == 64 * 512 * 2 + 256 * 4 + 4 * 256 * 256 * 4
    assert lib.moe_ffn_workspace_bytes(100, 256, 1) >= 100 * 256 + 100 * 2 * 4
    # MX: e4m3 A, then one E8M0 byte per 32 columns, each rounded up to 256 bytes
    assert lib.moe_ffn_workspace_bytes(100, 256, 4) == 25600 + 1024
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"


# ---------------------------------------------------------------- backward entry points

def _bwd(**kw):
    base = dict(max_rows=64, hidden_dim=256, moe_dim=512, n_local_experts=8, expert_offsets=16, x_perm=32,
                w_gate_up=48, w_gate_up_stacked=64, w_down_stacked=80, gate_up_format=0, activation=0, alpha=0.0,
                limit=0.0, d_expert_out=96, d_x_perm=112, d_w_gate_up=128, d_w_down=144, workspace=160,
                workspace_bytes=1 << 30)
    base.update(kw)
    return m.FfnBwdArgs(**base)


@pytest.mark.parametrize("kw,status,frag", [
    (dict(hidden_dim=96), m.MOE_ERR_INVALID_ARGUMENT, "64"),
    (dict(moe_dim=200), m.MOE_ERR_INVALID_ARGUMENT, "64"),
    (dict(n_local_experts=0), m.MOE_ERR_INVALID_ARGUMENT, "n_local_experts"),
    (dict(activation=7), m.MOE_ERR_INVALID_ARGUMENT, "activation"),
    (dict(alpha=1.0), m.MOE_ERR_INVALID_ARGUMENT, "alpha"),
    (dict(activation=2, limit=7.0), m.MOE_ERR_INVALID_ARGUMENT, "gelu_tanh"),
    (dict(gate_up_format=5), m.MOE_ERR_INVALID_ARGUMENT, "gate_up_format"),
    (dict(w_down_stacked=None), m.MOE_ERR_INVALID_ARGUMENT, "w_down_stacked"),
    (dict(d_w_down=None), m.MOE_ERR_INVALID_ARGUMENT, "d_w_down"),
    (dict(d_expert_out=None), m.MOE_ERR_INVALID_ARGUMENT, "d_expert_out"),
    (dict(x_perm=None), m.MOE_ERR_INVALID_ARGUMENT, "gather"),
    (dict(x=8, sorted_token=8), m.MOE_ERR_INVALID_ARGUMENT, "not both"),
    (dict(d_x_perm=120), m.MOE_ERR_INVALID_ARGUMENT, "aligned"),
    (dict(workspace_bytes=4096), m.MOE_ERR_WORKSPACE_TOO_SMALL, "workspace"),
])
def test_grouped_ffn_backward_validation(kw, status, frag):
    st, msg = _err(m.lib().moe_grouped_ffn_backward, _bwd(**kw))
    assert st == status and frag in msg, msg


def test_backward_workspace_bytes():
    lib = m.lib()

    def up(b):
        return -(-b // 256) * 256

    for R, H, D, L in ((64, 256, 512, 8), (8192, 4096, 14336, 8), (7, 64, 64, 3), (0, 64, 64, 1)):
        rp = -(-(R + 63 * min(L, R)) // 64) * 64  # every expert's rows padded to a multiple of 64
        want = (up(4 * (L + 1)) + 2 * up(R * D * 2) + up(R * 2 * D * 2) + up(H * rp * 2) + up(D * rp * 2)
                + up(2 * D * rp * 2) + up(H * rp * 2))
        assert lib.moe_ffn_backward_workspace_bytes(R, H, D, L) == want, (R, H, D, L)
    assert lib.moe_ffn_backward_workspace_bytes(-1, 64, 64, 1) == 0


@pytest.mark.parametrize("kw,frag", [
    (dict(hidden_dim=12), "hidden_dim"),
    (dict(out_dtype=1), "out_dtype"),
    (dict(d_expert_out=None), "required"),
    (dict(expert_out=None), "expert_out is required"),
    (dict(dy=24), "aligned"),
])
def test_combine_backward_validation(kw, frag):
    base = dict(num_tokens=4, n_experts_per_tok=2, hidden_dim=64, dy=16, expert_out=32, out_dtype=2,
                row_of_slot=48, d_expert_out=64, d_expert_weights=80)
    base.update(kw)
    st, msg = _err(m.lib().moe_combine_backward, m.CombineBwdArgs(**base))
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


@pytest.mark.parametrize("args,frag", [
    ((16, 32, 1, 65, 64), "multiples of 64"),
    ((16, 16, 1, 64, 64), "same buffer"),
    ((0, 32, 1, 64, 64), "required"),
    ((16, 40, 1, 64, 64), "aligned"),
])
def test_transpose_validation(args, frag):
    src, dst, b, r, c = args
    st = m.lib().moe_transpose_bf16(src or None, dst, b, r, c, None)
    msg = m.lib().moe_last_error_message().decode()
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


@pytest.mark.parametrize("args,frag", [
    ((2, 1, 1, 16), "kind"),
    ((0, 0, 1, 16), "workgroups"),
    ((0, 1, 0, 16), "iters"),
    ((1, 1, 1, 0), "out is required"),
])
def test_probe_mfma_validation(args, frag):
    kind, wg, it, out = args
    st = m.lib().moe_probe_mfma(kind, wg, it, out or None, None)
    msg = m.lib().moe_last_error_message().decode()
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


@pytest.mark.parametrize("args,frag", [
    ((16, 4096, 24), "multiple of 16"),
    ((0, 4096, 64), "required"),
    ((24, 4096, 64), "aligned"),
    ((16, 48, 64), "overlap"),
])
def test_probe_stream_copy_validation(args, frag):
    src, dst, n = args
    st = m.lib().moe_probe_stream_copy(src or None, dst, n, None)
    msg = m.lib().moe_last_error_message().decode()
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


def test_probe_stream_copy_zero_bytes_is_a_no_op():
    assert m.lib().moe_probe_stream_copy(None, None, 0, None) == m.MOE_OK


@pytest.mark.parametrize("args,frag", [
    ((4096, 24, 64, 4), "multiple of 16"),
    ((0, 32, 64, 4), "required"),
    ((4096, 32, 0, 4), "required"),
    ((24, 32, 64, 4), "aligned"),
    ((4096, 32, 64, 3), "out_len"),
])
def test_probe_stream_read_validation(args, frag):
    src, n, out, out_len = args
    st = m.lib().moe_probe_stream_read(src or None, n, out or None, out_len, None)
    msg = m.lib().moe_last_error_message().decode()
    assert st == m.MOE_ERR_INVALID_ARGUMENT and frag in msg, msg


def test_probe_stream_read_zero_bytes_is_a_no_op():
    assert m.lib().moe_probe_stream_read(None, 0, None, 0, None) == m.MOE_OK


@pytest.mark.parametrize("sl,frag", [((7, 2), "not a slice"), ((-1, 2), "not a slice"), ((0, 0), "not a slice")])
def test_layer_expert_slice_validation(sl, frag):
    """MoELayer refuses an expert slice outside the routed experts before it
    touches any tensor."""
    import torch
    import synth
    cfg = synth.get_config(1)
    with pytest.raises(ValueError, match=frag):
        m.MoELayer(cfg, {"x": torch.zeros(1)}, expert_slice=sl)


def test_layer_expert_slice_refuses_shared_experts():
    import torch
    import synth
    cfg = synth.get_config(3)
    with pytest.raises(ValueError, match="without shared experts"):
        m.MoELayer(cfg, {"x": torch.zeros(1)}, expert_slice=(0, 16))
