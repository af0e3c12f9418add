"""CPU-side tests of the C ABI (no GPU needed, no kernel is launched).

* librownorm.so loads and exports every function include/rownorm.h declares;
* rn_plan's validation and variant choice (a host-only function);
* the entry points reject bad arguments before touching HIP.
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

import row_wise_normalization_fp32_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rownorm.h")

OK, NULL, SHAPE, DTYPE, ALIAS, UNSUP, HIP, ALIGN, WORKSPACE = range(9)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)
    assert names, "no declarations parsed"
    return names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(rn.LIB_PATH)
    names = _declared_functions()
    for n in ("ln_forward", "rms_norm", "fused_add_rms_norm", "fused_add_layer_norm", "softmax_forward",
              "rn_forward_ex", "rn_forward_workspace_bytes", "ln_backward", "rms_norm_backward", "rn_backward_workspace_bytes",
              "rn_plan_backward", "rn_plan", "rn_status_string"):
        assert n in names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_library_exports_nothing_else():
    # the ELF dynamic symbol table holds only the declared C entry points among the
    # library's own defined functions (internal C++ helpers are hidden)
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", rn.LIB_PATH], capture_output=True, text=True, check=True).stdout
    funcs = {l.split()[-1] for l in out.splitlines() if len(l.split()) == 3 and l.split()[1] == "T"}
    assert funcs == set(_declared_functions()), sorted(funcs ^ set(_declared_functions()))


def test_status_strings_and_version():
    for code, name in rn.STATUS.items():
        assert rn._lib.rn_status_string(code).decode() == name
    assert rn._lib.rn_status_string(99).decode() == "unknown status"
    assert rn.version() == 10100


@pytest.mark.parametrize("op,dtype,rows,N,variant,W,V,persistent", [
    ("ln", torch.float32, 64, 1024, "wave", 1, 4, False),              # C1: 256 chunks
    ("ln", torch.float32, 128, 4096, "workgroup", 4, 4, False),        # C2: 1024 chunks
    ("rms", torch.float16, 2048, 4096, "workgroup", 2, 4, True),       # C3: 512 chunks, 1024 workgroups of 2 rows
    # C4: 2 rows per workgroup would make 128 workgroups; one row per 4-wave workgroup instead
    ("fused_add_rms", torch.float16, 256, 4096, "workgroup", 4, 2, True),
    ("fused_add_rms", torch.bfloat16, 256, 4096, "workgroup", 4, 2, True),
    ("fused_add_rms", torch.bfloat16, 64, 4096, "workgroup", 4, 2, False),
    ("ln", torch.bfloat16, 511, 4096, "workgroup", 2, 4, True),       # 256 workgroups of 2 rows
    ("rms", torch.float16, 255, 3072, "workgroup", 4, 2, False),      # 384 chunks, not exact
    ("ln", torch.bfloat16, 4096, 16384, "workgroup", 8, 4, True),      # C5: 2048 chunks, 4096 groups
    ("fused_add_rms", torch.float16, 8192, 4096, "workgroup", 2, 4, True),
    ("ln", torch.float32, 16, 16384, "workgroup", 16, 4, False),
    ("rms", torch.bfloat16, 16, 32768, "workgroup", 16, 4, False),
    ("rms", torch.float32, 16, 16388, "workgroup", 16, 8, False),      # 4097 chunks: 16 waves x 8 chunks
    ("ln", torch.float32, 16, 16388, "workgroup", 16, 8, False),      # no workspace for split rows: one workgroup
    ("fused_add_rms", torch.float16, 16, 65536, "workgroup", 16, 8, False),  # likewise, 8192 chunks
    ("softmax", torch.float32, 16, 32768, "workgroup", 16, 8, False),  # 128 KiB rows, one workgroup each
    ("fused_add_ln", torch.bfloat16, 8, 32776, "general", 0, 0, False),  # no room for 8 chunks: split (no workspace)
    ("ln", torch.float32, 16, 32772, "general", 0, 0, False),          # beyond a workgroup's registers
    ("ln", torch.float32, 16, 1000, "wave", 1, 4, False),              # ragged: 250 chunks
    ("ln", torch.float16, 16, 1001, "element", 1, 8, False),           # not whole 16-byte chunks: 501 pairs
    ("rms", torch.float32, 3, 1, "element", 1, 1, False),
    ("rms", torch.bfloat16, 8, 16383, "element", 16, 8, False),        # 8192 pairs
    ("rms", torch.float32, 8, 16383, "element", 16, 16, False),
    ("ln", torch.bfloat16, 8, 16385, "general", 0, 0, False),          # odd and beyond the element kernel
    ("ln", torch.float32, 8, 65536, "general", 0, 0, False),           # long rows without a workspace
    ("fused_add_ln", torch.bfloat16, 8192, 4096, "workgroup", 2, 4, True),
    ("fused_add_ln", torch.float32, 256, 4096, "workgroup", 4, 4, True),   # 256 workgroups: persistent from there
    ("fused_add_ln", torch.float32, 255, 4096, "workgroup", 4, 4, False),
    ("softmax", torch.float32, 128, 4096, "workgroup", 4, 4, False),
    ("softmax", torch.float32, 8192, 4096, "workgroup", 4, 4, True),   # persistent without parameters
    ("softmax", torch.float16, 64, 333, "element", 1, 4, False),
    ("softmax", torch.float32, 64, 333, "element", 1, 8, False),
    ("ln", torch.bfloat16, 16384, 4095, "workgroup", 2, 4, True),      # many ragged rows: byte-addressed,
    ("ln", torch.float32, 16384, 4095, "workgroup", 4, 4, True),       # persistent
    ("ln", torch.bfloat16, 200, 4095, "element", 4, 8, False),         # few ragged rows: element / pair
    ("ln", torch.bfloat16, 16384, 4088, "workgroup", 2, 4, True),      # whole chunks, 511 of 512: byte-addressed
])
def test_plan_variant_choice(op, dtype, rows, N, variant, W, V, persistent):
    ptrs = {"gamma": 1 << 44, "beta": (1 << 44) + (1 << 30)}
    st, info = rn.plan(op, rows, N, dtype, ptrs=ptrs)
    assert st == OK
    assert info["variant"] == variant
    assert info["chunks_per_lane"] == V
    assert info["persistent"] == persistent
    if variant == "general":
        assert info["grid_blocks"] == rows and info["block_threads"] == 256
        return
    if variant == "element":
        assert info["waves_per_row"] == W and not info["exact"] and info["lds_bytes"] == 0
        assert info["persistent"] == persistent
        # 16-bit rows of contiguous tensors move as element pairs: up to N + 1 positions
        # (a row may start in the upper half of a 4-byte word)
        pairs = dtype != torch.float32
        assert info["pairs"] == pairs
        n = (N + 2) // 2 if pairs else N
        assert 64 * W * V >= n and (V == 1 or 64 * W * V // 2 < n or W > 1)
        return
    assert info["waves_per_row"] == W
    rpb = 4 // W if W <= 4 else 1
    assert info["rows_per_block"] == rpb
    assert info["block_threads"] == 64 * W * rpb
    assert info["grid_blocks"] == (rows + rpb - 1) // rpb
    s = torch.tensor([], dtype=dtype).element_size()
    C = (N * s + 15) // 16  # chunks per row, the last one partial when N * s is not a multiple of 16
    assert info["exact"] == (C == 64 * W * V)
    # rows that are not whole chunks, or that do not fill the row group, run byte-addressed
    assert info["ragged"] == (persistent and (N * s % 16 != 0 or C != 64 * W * V))
    if persistent:
        # one parameter vector staged in LDS (softmax has none)
        assert info["lds_bytes"] == (0 if op == "softmax" else C * 16)


def test_plan_persistent_launches():
    # without gamma / beta nothing is staged: persistent, but no LDS
    st, info = rn.plan("ln", 4096, 16384, torch.bfloat16)
    assert st == OK and info["persistent"] and info["lds_bytes"] == 0
    st, info = rn.plan("softmax", 8192, 4096, torch.bfloat16)
    assert st == OK and info["persistent"] and info["lds_bytes"] == 0
    # with parameters: one parameter vector in LDS
    st, info = rn.plan("rms", 8192, 4096, torch.bfloat16, ptrs={"gamma": 1 << 44})
    assert st == OK and info["persistent"] and info["lds_bytes"] == 4096 * 2
    # vectorized launches are persistent from 256 workgroups, the element / pair kernels from 2048
    assert rn.plan("softmax", 2048, 4096, torch.bfloat16)[1]["persistent"]  # 1024 workgroups
    # 510 rows would be 255 workgroups of 2 rows: one row per workgroup instead, 510 workgroups
    st, info = rn.plan("softmax", 510, 4096, torch.bfloat16)
    assert info["persistent"] and info["rows_per_block"] == 1 and info["waves_per_row"] == 4
    st, info = rn.plan("softmax", 512, 4096, torch.bfloat16)
    assert info["persistent"] and info["rows_per_block"] == 2 and info["waves_per_row"] == 2
    assert not rn.plan("softmax", 255, 4096, torch.bfloat16)[1]["persistent"]  # 255 workgroups of 1 row
    # ragged rows: the byte-addressed vectorized kernel from 256 row blocks (fp32 4095: 4-wave
    # rows, one per workgroup), the element kernel (forced) from 2048 workgroups
    assert not rn.plan("ln", 255, 4095, torch.float32)[1]["persistent"]
    st, info = rn.plan("ln", 256, 4095, torch.float32)
    assert info["persistent"] and info["ragged"] and info["variant"] == "workgroup"
    assert not rn.plan("ln", 2047, 4095, torch.float32, variant="element")[1]["persistent"]
    assert rn.plan("ln", 2048, 4095, torch.float32, variant="element")[1]["persistent"]
    # whole-chunk rows that do not fill the row group (250 of 256 chunks): byte-addressed from
    # 256 row blocks, grid per row below
    st, info = rn.plan("rms", 1 << 15, 1000, torch.float32, ptrs={"gamma": 1 << 44})
    assert st == OK and not info["exact"] and info["persistent"] and info["ragged"]
    st, info = rn.plan("rms", 1020, 1000, torch.float32, ptrs={"gamma": 1 << 44})
    assert st == OK and not info["exact"] and not info["persistent"] and not info["ragged"]


def test_plan_grid_is_capped():
    st, info = rn.plan("rms", 1 << 23, 64, torch.float16)
    assert st == OK and info["grid_blocks"] == 1 << 20


def test_plan_misaligned_pointer_takes_element_path():
    st, info = rn.plan("ln", 8, 1024, torch.float32, ptrs={"x": (1 << 40) + 4})
    assert st == OK and info["variant"] == "element" and info["waves_per_row"] == 2
    st, _ = rn.plan("ln", 8, 1024, torch.float32, ptrs={"x": (1 << 40) + 4}, variant="wave")
    assert st == UNSUP
    st, info = rn.plan("ln", 8, 32768, torch.float16, ptrs={"x": (1 << 40) + 2})
    assert st == OK and info["variant"] == "general"


def test_plan_element_pairs():
    # 16-bit element rows move as 4-byte pairs when every row tensor has the same position
    # in its 4-byte word on every row: same address bit 1 and same stride parity.
    bf, base = torch.bfloat16, 1 << 40
    far = 1 << 42

    def pairs(op="ln", rows=8, N=4095, **kw):
        st, info = rn.plan(op, rows, N, bf, **kw)
        assert st == OK and info["variant"] == "element", info
        return info["pairs"]

    assert pairs()
    assert pairs(ptrs={"x": base + 2, "y": far + 2})       # both start in an upper half
    assert not pairs(ptrs={"x": base + 2, "y": far})       # x does, y does not
    assert not pairs(ptrs={"x": base, "y": far + 6})
    assert pairs(ptrs={"x": base + 4, "y": far})           # 4-byte offsets keep the halves
    assert pairs(strides={"x": 4097, "y": 4099})           # both odd
    assert not pairs(strides={"x": 4097, "y": 4096})       # parities differ ...
    assert pairs(rows=1, strides={"x": 4097, "y": 4096})   # ... which one row never sees
    # fused ops: residual and residual_out count too
    assert pairs("fused_add_rms", ptrs={"residual": far + (1 << 30)})
    assert not pairs("fused_add_rms", ptrs={"residual": far + (1 << 30) + 2})
    assert not pairs("fused_add_ln", strides={"residual_out": 4096})
    # 16 waves x 8 slots hold 8192 words: rows of up to 16384 elements when no row starts in
    # an upper half, else up to 16383; fp32 never pairs
    st, info = rn.plan("ln", 8, 16383, bf, variant="element")
    assert info["pairs"] and info["waves_per_row"] == 16 and info["chunks_per_lane"] == 8
    st, info = rn.plan("ln", 8, 16384, bf, variant="element")
    assert info["pairs"] and info["waves_per_row"] == 16 and info["chunks_per_lane"] == 8
    st, info = rn.plan("ln", 8, 16384, bf, variant="element", ptrs={"x": base + 2, "y": far + 2})
    assert st == OK and not info["pairs"] and info["chunks_per_lane"] == 16
    # even rows that all start on a word need N / 2 words: 2048 for 4096 elements (4 waves)
    st, info = rn.plan("ln", 8, 4096, bf, variant="element")
    assert info["pairs"] and info["waves_per_row"] == 4 and info["chunks_per_lane"] == 8
    st, info = rn.plan("ln", 8, 4096, bf, variant="element", ptrs={"x": base + 2, "y": far + 2})
    assert info["pairs"] and info["waves_per_row"] == 8 and info["chunks_per_lane"] == 8
    assert not rn.plan("ln", 8, 4095, torch.float32)[1]["pairs"]
    assert not rn.plan("ln", 8, 4096, bf)[1]["pairs"]  # vectorized


def test_plan_long_softmax_rows_stay_in_one_workgroup():
    f32, bf = torch.float32, torch.bfloat16
    ws = 1 << 24
    # byte-addressed rows on one 16-wave workgroup, grid per row (fp32: 16 chunks per lane, up
    # to 16384 chunks; 16-bit: 8, up to 8192)
    for dt, V in ((f32, 16), (bf, 8)):
        st, info = rn.plan("softmax", 8, 50257, dt, workspace_bytes=ws)
        assert st == OK and info["variant"] == "workgroup" and info["ragged"] and not info["persistent"], info
        assert (info["waves_per_row"], info["chunks_per_lane"]) == (16, V), info
    st, info = rn.plan("softmax", 8, 16385, f32)  # 4097 chunks: 8 per lane
    assert st == OK and info["ragged"] and (info["waves_per_row"], info["chunks_per_lane"]) == (16, 8), info
    # the element kernel when forced
    st, info = rn.plan("softmax", 8, 50257, f32, variant="element")
    assert st == OK and info["variant"] == "element" and info["waves_per_row"] == 16 and info["chunks_per_lane"] == 64
    st, info = rn.plan("softmax", 8, 50257, bf, variant="element")
    assert st == OK and info["variant"] == "element" and info["pairs"] and info["chunks_per_lane"] == 32
    # up to 65536 elements; the other ops split such rows
    st, info = rn.plan("softmax", 8, 65536, f32, ptrs={"x": (1 << 40) + 4}, workspace_bytes=ws)
    assert info["variant"] == "workgroup" and info["ragged"] and info["chunks_per_lane"] == 16, info
    assert rn.plan("softmax", 8, 65537, f32, workspace_bytes=ws)[1]["variant"] == "wide"  # byte-addressed one pass
    assert rn.plan("rms", 8, 50257, f32, workspace_bytes=ws)[1]["variant"] == "wide"
    assert rn.plan("softmax", 8, 65537, f32, variant="element")[0] == UNSUP
    assert rn.plan("ln", 8, 16385, f32, variant="element")[0] == UNSUP


def test_plan_row_strides():
    f16 = torch.float16
    # padded rows whose stride is a whole number of 16-byte chunks keep the vectorized path
    st, info = rn.plan("ln", 64, 4096, f16, strides={"x": 4096 + 64, "y": 4096})
    assert st == OK and info["variant"] == "workgroup"
    # a stride that is not a whole chunk takes the element kernel
    st, info = rn.plan("ln", 64, 4096, f16, strides={"x": 4097})
    assert st == OK and info["variant"] == "element"
    st, _ = rn.plan("ln", 64, 4096, f16, strides={"x": 4097}, variant="workgroup")
    assert st == UNSUP
    # stride below N, or absurdly large
    assert rn.plan("ln", 64, 4096, f16, strides={"y": 4095})[0] == SHAPE
    assert rn.plan("ln", 4, 64, f16, strides={"x": 1 << 41})[0] == SHAPE
    # unused entries are ignored (no residual in LayerNorm)
    assert rn.plan("ln", 4, 64, f16, strides={"residual": 1})[0] == OK
    # in place needs the same stride
    base = 1 << 40
    assert rn.plan("rms", 4, 64, f16, ptrs={"x": base, "y": base}, strides={"x": 128, "y": 128})[0] == OK
    assert rn.plan("rms", 4, 64, f16, ptrs={"x": base, "y": base}, strides={"x": 128})[0] == ALIAS
    # two column slices of one buffer interleave: refused (address ranges overlap)
    assert rn.plan("rms", 4, 64, f16, ptrs={"x": base, "y": base + 128}, strides={"x": 128, "y": 128})[0] == ALIAS


def test_plan_forced_variants():
    assert rn.plan("ln", 4, 4096, torch.float32, variant="workgroup")[1]["waves_per_row"] == 4
    assert rn.plan("ln", 4, 64, torch.float32, variant="workgroup")[1]["waves_per_row"] == 2
    assert rn.plan("ln", 4, 4096, torch.float32, variant="wave")[1]["chunks_per_lane"] == 16
    assert rn.plan("ln", 4, 8192, torch.float16, variant="wave")[1]["chunks_per_lane"] == 16
    assert rn.plan("ln", 4, 8192, torch.float32, variant="wave")[0] == UNSUP
    assert rn.plan("softmax", 4, 32768, torch.float32, variant="workgroup")[1]["chunks_per_lane"] == 8
    assert rn.plan("softmax", 4, 65536, torch.float32, variant="workgroup")[1]["chunks_per_lane"] == 16
    assert rn.plan("softmax", 4, 65540, torch.float32, variant="workgroup")[0] == UNSUP
    assert rn.plan("softmax", 4, 65544, torch.bfloat16, variant="workgroup")[0] == UNSUP
    # LayerNorm rows of 8192 chunks: one workgroup, with or without a workspace (split rows
    # only when forced); fused add + RMSNorm rows: one workgroup without a workspace, split
    # rows with one
    assert rn.plan("ln", 4, 32768, torch.float32, variant="workgroup")[1]["chunks_per_lane"] == 8
    need = rn.forward_workspace_bytes("ln", 4, 32768, torch.float32)
    assert rn.plan("ln", 4, 32768, torch.float32, workspace_bytes=need)[1]["variant"] == "workgroup"
    assert rn.plan("ln", 4, 32768, torch.float32, variant="wide", workspace_bytes=need)[1]["variant"] == "wide"
    assert rn.plan("ln", 4, 32768, torch.float32, variant="workgroup", workspace_bytes=need)[0] == OK
    assert rn.plan("fused_add_rms", 4, 65536, torch.float16, variant="workgroup")[1]["chunks_per_lane"] == 8
    need = rn.forward_workspace_bytes("fused_add_rms", 4, 65536, torch.float16)
    assert rn.plan("fused_add_rms", 4, 65536, torch.float16, workspace_bytes=need)[1]["variant"] == "wide"
    assert rn.plan("fused_add_rms", 4, 65536, torch.float16, variant="workgroup", workspace_bytes=need)[0] == UNSUP
    assert rn.plan("ln", 4, 32772, torch.float32, variant="workgroup")[0] == UNSUP  # 8193 chunks
    assert rn.plan("ln", 4, 64, torch.float32, variant="general")[1]["variant"] == "general"
    assert rn.plan("ln", 4, 4096, torch.float32, variant="element")[1]["variant"] == "element"
    assert rn.plan("ln", 4, 16385, torch.float32, variant="element")[0] == UNSUP
    assert rn.plan("ln", 4, 64, torch.float32, variant=7)[0] == UNSUP


def test_plan_argument_errors():
    f32 = torch.float32
    assert rn.plan("ln", -1, 64, f32)[0] == SHAPE
    assert rn.plan("ln", 4, 0, f32)[0] == SHAPE
    assert rn.plan("ln", 4, 64, f32, eps=-1.0)[0] == SHAPE
    assert rn.plan("ln", 4, 64, f32, eps=float("nan"))[0] == SHAPE
    assert rn.plan("ln", 4, 64, f32, eps=float("inf"))[0] == SHAPE
    assert rn.plan("ln", 1 << 40, 1 << 30, f32)[0] == SHAPE  # rows * N * 4 overflows
    assert rn.plan("ln", 4, 64, f32, ptrs={"x": None})[0] == NULL
    assert rn.plan("ln", 4, 64, f32, ptrs={"y": None})[0] == NULL
    assert rn.plan("fused_add_rms", 4, 64, f32, ptrs={"residual": None})[0] == NULL
    assert rn.plan("fused_add_rms", 4, 64, f32, ptrs={"residual_out": None})[0] == NULL
    assert rn.plan("ln", 4, 64, f32, ptrs={"x": (1 << 40) + 2})[0] == ALIGN
    assert rn.plan("ln", 4, 64, torch.float16, ptrs={"x": (1 << 40) + 1})[0] == ALIGN
    assert rn.plan("ln", 4, 64, f32, ptrs={"mean": (1 << 44) + 2})[0] == ALIGN


def test_plan_zero_rows_is_a_noop_even_without_buffers():
    st, info = rn.plan("ln", 0, 64, torch.float32, ptrs={"x": None, "y": None})
    assert st == OK and info["grid_blocks"] == 0


def test_plan_aliasing_rules():
    f32 = torch.float32
    base = 1 << 40
    rows, N = 4, 64
    nbytes = rows * N * 4
    far = base + (1 << 30)
    # exact in-place is allowed
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": base})[0] == OK
    assert rn.plan("rms", rows, N, f32, ptrs={"x": base, "y": base})[0] == OK
    assert rn.plan("fused_add_rms", rows, N, f32,
                   ptrs={"x": base, "residual": far, "residual_out": far, "y": base})[0] == OK
    assert rn.plan("fused_add_rms", rows, N, f32,
                   ptrs={"x": base, "residual": far, "residual_out": base, "y": far})[0] == OK
    # partial overlap of an output with an input
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": base + 256})[0] == ALIAS
    # an output on top of a parameter vector
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": far, "gamma": far + 128})[0] == ALIAS
    # two outputs on the same memory
    assert rn.plan("fused_add_rms", rows, N, f32,
                   ptrs={"x": base, "residual": base + nbytes, "residual_out": far, "y": far})[0] == ALIAS
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": far, "mean": far + nbytes,
                                            "rstd": far + nbytes})[0] == ALIAS
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": far, "mean": base + 16})[0] == ALIAS
    # inputs may overlap each other
    assert rn.plan("ln", rows, N, f32, ptrs={"x": base, "y": far, "gamma": base, "beta": base})[0] == OK
    # beta is not part of RMSNorm, so it is ignored there
    assert rn.plan("rms", rows, N, f32, ptrs={"x": base, "y": far, "beta": far})[0] == OK


def test_entry_points_reject_before_launch():
    # Every call below fails validation, so no HIP call is made: safe without a GPU.
    lib = rn._lib
    assert lib.ln_forward(None, None, None, 0x1000, None, None, 4, 64, 1e-5, 0, None) == NULL
    assert lib.ln_forward(0x1000, None, None, 0x100000, None, None, 4, 64, 1e-5, 9, None) == DTYPE
    assert lib.ln_forward(0x1000, None, None, 0x100000, None, None, -3, 64, 1e-5, 0, None) == SHAPE
    assert lib.rms_norm(0x1000, None, 0x1000 + 64, None, 4, 64, 1e-6, 0, None) == ALIAS
    assert lib.fused_add_rms_norm(0x1000, None, None, 0x100000, 0x200000, None, 4, 64, 1e-6, 1, None) == NULL
    assert lib.ln_forward_variant(0x1000, None, None, 0x100000, None, None, 4, 8192, 1e-5, 0, None, 1) == UNSUP
    assert lib.ln_forward(None, None, None, None, None, None, 0, 64, 1e-5, 0, None) == OK
    assert lib.softmax_forward(None, 0x100000, None, None, 4, 64, 0, None) == NULL
    assert lib.softmax_forward(0x1000, 0x1000 + 64, None, None, 4, 64, 0, None) == ALIAS
    assert lib.fused_add_layer_norm(0x1000, 0x200000, None, None, 0x300000, None, None, None, 4, 64, 1e-5, 2,
                                    None) == NULL
    assert lib.rn_forward_ex(9, 0x1000, None, None, None, 0x100000, None, None, None, 4, 64, 1e-5, 0, None, 0,
                             None, 0, None) == SHAPE


def test_python_binding_rejects_cpu_tensors():
    with pytest.raises(ValueError):
        rn.ln_forward(torch.zeros(2, 8))
    with pytest.raises(ValueError):
        rn.rms_norm(torch.zeros(2, 8))


def test_backward_plan_and_validation():
    bf16, f32 = torch.bfloat16, torch.float32
    ws = {"dgamma": 1 << 45, "dbeta": (1 << 45) + (1 << 20), "workspace": 1 << 46}
    st, info = rn.plan_backward("ln", 4096, 16384, bf16, ptrs=ws)
    assert st == OK and info["variant"] == "workgroup" and info["waves_per_row"] == 16
    assert info["chunks_per_lane"] == 2 and info["block_threads"] == 1024 and info["grid_blocks"] == 1024
    st, info = rn.plan_backward("rms", 2048, 4096, torch.float16, ptrs=ws)
    assert st == OK and info["waves_per_row"] == 4 and info["rows_per_block"] == 4 and info["lds_bytes"] == 4096 * 4
    # rows that are not whole chunks: element kernel; beyond 16384 elements: split rows
    assert rn.plan_backward("ln", 8, 1001, bf16, ptrs=ws)[1]["variant"] == "element"
    assert rn.plan_backward("ln", 8, 16384, f32, ptrs=ws)[1]["variant"] == "element"
    st, info = rn.plan_backward("ln", 8, 32768, bf16, ptrs=ws)
    assert st == OK and info["variant"] == "wide" and info["block_threads"] == 512 and info["exact"]
    assert info["chunks_per_lane"] == 16 and info["grid_blocks"] == 8  # min(rows, 2048 / 4 segments)
    st, info = rn.plan_backward("rms", 4096, 40001, f32, ptrs=ws)  # element-aligned rows: 5 segments
    assert st == OK and info["variant"] == "wide" and not info["exact"] and info["grid_blocks"] == 2048 // 5
    st, info = rn.plan_backward("ln", 8, 32768, bf16, ptrs={**ws, "x": (1 << 40) + 2})  # x not 16-byte aligned
    assert st == OK and info["variant"] == "wide" and not info["exact"]
    # split rows keep their segment records in the workspace: needed even for dx alone
    assert rn.plan_backward("ln", 8, 32768, bf16)[0] == 8
    assert rn.plan_backward("ln", 8, 32768, bf16, ptrs={"workspace": 1 << 46})[0] == OK
    assert rn.plan_backward("ln", 8, 16384, bf16)[0] == OK
    # split-row workspace: partial rows (sets x min(rows, 2048 / S) x N x 4), then from a
    # 256-byte boundary a 256-byte header (ticket counter, time-out flag) and the records
    # (rows x S x 16)
    assert rn.backward_workspace_bytes("ln", 100, 32768) == 2 * 100 * 32768 * 4 + 256 + 100 * 4 * 16
    assert rn.backward_workspace_bytes("rms", 4096, 40001) == \
        -(-(409 * 40001 * 4) // 256) * 256 + 256 + 4096 * 5 * 16
    # workspace: required for parameter gradients, at least rn_backward_workspace_bytes
    assert rn.backward_workspace_bytes("ln", 4096, 16384) == 2 * 1024 * 16384 * 4
    assert rn.backward_workspace_bytes("rms", 100, 64) == 100 * 64 * 4
    assert rn.plan_backward("ln", 64, 256, bf16, ptrs={"dgamma": 1 << 45})[0] == 8
    assert rn.plan_backward("ln", 64, 256, bf16, ptrs=ws, workspace_bytes=100)[0] == 8
    assert rn.plan_backward("ln", 64, 256, bf16)[0] == OK  # dx only: no workspace needed
    assert rn.plan_backward("ln", 0, 256, bf16, ptrs={"dgamma": 1 << 45, "dy": None, "x": None})[0] == OK
    # required inputs
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={"mean": None})[0] == NULL
    assert rn.plan_backward("rms", 4, 256, bf16, ptrs={"mean": None})[0] == OK
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={"rstd": None})[0] == NULL
    # aliasing: dx may be dy or x; the workspace and the parameter gradients overlap nothing
    base = 1 << 40
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={"dy": base, "dx": base})[0] == OK
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={"x": base, "dx": base, "dy": base + (1 << 30)})[0] == OK
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={"dy": base, "dx": base + 64})[0] == ALIAS
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={**ws, "dbeta": (1 << 45) + 16})[0] == ALIAS
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={**ws, "workspace": (1 << 45) + 64})[0] == ALIAS
    assert rn.plan_backward("ln", 4, 256, bf16, ptrs={**ws, "workspace": (1 << 46) + 2})[0] == ALIGN
    assert rn.plan_backward("softmax", 4, 256, bf16)[0] == SHAPE
    assert rn.plan_backward("ln", 4, 256, 9)[0] == DTYPE


def test_backward_entry_points_reject_before_launch():
    lib = rn._lib
    assert lib.ln_backward(None, None, None, None, None, None, None, None, 4, 64, 0, None, 0, None) == NULL
    assert lib.ln_backward(0x1000, 0x2000, None, 0x3000, 0x4000, None, 0x5000, None, 4, 64, 0, None, 0,
                           None) == 8
    assert lib.rms_norm_backward(0x1000, 0x2000, None, 0x4000, 0x1000 + 64, None, 4, 64, 0, None, 0, None) == ALIAS
    # 65536-element rows are split across workgroups: the workspace for their records is missing
    assert lib.rms_norm_backward(0x1000, 0x200000, None, 0x400000, None, None, 4, 65536, 0, None, 0, None) == 8


def test_plan_split_rows():
    f32, bf16 = torch.float32, torch.bfloat16
    # room for either split-row form: the two launches keep one 16-byte record per
    # 8192-element segment; the one pass a 256-byte header and four 64-bit words per 32 KiB
    # chunk segment (rows of whole chunks)
    need = rn.forward_workspace_bytes("ln", 64, 65536, f32)
    assert need == 256 + 64 * 8 * 32
    assert rn.forward_workspace_bytes("ln", 64, 16384, f32) == 0  # fits one workgroup
    assert rn.forward_workspace_bytes("ln", 64, 16385, bf16) == max(64 * 3 * 16, 256 + 64 * 2 * 32)
    assert rn.forward_workspace_bytes("ln", 64, 65537, bf16) == max(64 * 9 * 16, 256 + 64 * 5 * 32)
    assert rn.forward_workspace_bytes("ln", 64, 131072, bf16) == 256 + 64 * 8 * 32
    assert rn.forward_workspace_bytes("ln", 0, 65536, f32) == 0
    # the two-launch form needs only its records: a workspace of that size still splits rows
    st, info = rn.plan("ln", 64, 65536, f32, workspace_bytes=64 * 8 * 16)
    assert st == OK and info["variant"] == "wide"
    # whole 16-byte chunks: segments of 2048 chunks
    st, info = rn.plan("ln", 64, 65536, f32, workspace_bytes=need)
    assert st == OK and info["variant"] == "wide" and info["grid_blocks"] == 64 * 8 and info["exact"]
    st, info = rn.plan("softmax", 8, 65544, bf16, workspace_bytes=8 * 9 * 16)
    assert st == OK and info["variant"] == "wide" and not info["exact"] and info["grid_blocks"] == 8 * 5
    # softmax, RMSNorm and LayerNorm rows up to 128 KiB stay in one workgroup (16 waves x 8
    # chunks); the fused ops split them
    ws = rn.forward_workspace_bytes("ln", 8, 32776, bf16)
    for op in ("softmax", "rms", "ln"):
        assert rn.plan(op, 8, 32776, bf16, workspace_bytes=ws)[1]["variant"] == "workgroup"
    for op in ("fused_add_rms", "fused_add_ln"):
        assert rn.plan(op, 8, 32776, bf16, workspace_bytes=ws)[1]["variant"] == "wide"
    # bf16 rows of whole chunks up to 32768 elements stay in one workgroup, workspace or not
    assert rn.plan("ln", 8, 32768, bf16, workspace_bytes=8 * 8 * 16)[1]["variant"] == "workgroup"
    # other rows longer than 16384 elements: with room for the one-pass layout, byte-addressed
    # segments of up to 2048 chunks (the last chunk partial); 16-bit rows at odd 2-byte
    # positions, and with only the two-launch form's records or in place any rows, segments of
    # 8192 elements
    for N, dt, ptrs, strides, one in [(65537, f32, None, None, True), (50257, bf16, None, None, False),
                                      (50258, bf16, None, None, True), (65536, f32, {"x": (1 << 40) + 4}, None, True),
                                      (20000, bf16, None, {"x": 20001}, False),
                                      (20000, bf16, {"x": (1 << 40) + 4}, None, True)]:
        ws = rn.forward_workspace_bytes("ln", 8, N, dt)
        st, info = rn.plan("ln", 8, N, dt, workspace_bytes=ws, ptrs=ptrs, strides=strides)
        C = (N * (4 if dt == f32 else 2) + 15) // 16
        if one:
            assert st == OK and info["variant"] == "wide" and info["ragged"] and not info["exact"], (N, info)
            assert info["grid_blocks"] == 8 * ((C + 2047) // 2048) and info["chunks_per_lane"] == 4
        else:
            assert st == OK and info["variant"] == "wide_element" and not info["ragged"], (N, info)
        S = (N + 8191) // 8192
        for kw in ({"workspace_bytes": 8 * S * 16}, {"workspace_bytes": ws, "in_place": True}):
            pp, sd = dict(ptrs or {}), dict(strides or {})
            if kw.pop("in_place", False):  # y over x: same address, same row stride
                pp["y"] = pp["x"] = pp.get("x", 1 << 42)
                if "x" in sd:
                    sd["y"] = sd["x"]
            st, info = rn.plan("ln", 8, N, dt, ptrs=pp, strides=sd or None, **kw)
            assert st == OK and info["variant"] == "wide_element", (N, kw, info)
            assert info["grid_blocks"] == 8 * S and info["block_threads"] == 512 and info["chunks_per_lane"] == 16
            assert info["exact"] == (N % 8192 == 0) and not info["ragged"]
        # below the two-launch form's records (one per 8192 elements): no split rows
        assert rn.plan("ln", 8, N, dt, workspace_bytes=8 * S * 16 - 16, ptrs=ptrs,
                       strides=strides)[1]["variant"] == "general"
    # too small a workspace: the general kernel (auto) or an error (forced)
    assert rn.plan("ln", 64, 65536, f32, workspace_bytes=64 * 8 * 16 - 16)[1]["variant"] == "general"
    assert rn.plan("ln", 64, 65536, f32, variant="wide")[0] == WORKSPACE
    assert rn.plan("ln", 64, 65537, f32, variant="wide_element")[0] == WORKSPACE
    assert rn.plan("ln", 64, 4096, f32, variant="wide", workspace_bytes=1 << 20)[0] == UNSUP
    assert rn.plan("ln", 64, 65537, f32, variant="wide", workspace_bytes=1 << 20)[0] == UNSUP
    assert rn.plan("ln", 64, 16384, f32, variant="wide_element", workspace_bytes=1 << 20)[0] == UNSUP
    assert rn.plan("ln", 64, 65536, f32, variant="wide_element", workspace_bytes=need)[1]["variant"] == "wide_element"
    # workspace alignment and overlap
    assert rn.plan("ln", 64, 65536, f32, workspace_bytes=need, ptrs={"workspace": (1 << 47) + 4})[0] == ALIGN
    assert rn.plan("ln", 64, 65536, f32, workspace_bytes=need, ptrs={"workspace": 1 << 40})[0] == ALIAS


def test_python_wrapper_names():
    # the C ABI names, plus layer_norm for the LayerNorm forward
    assert rn.layer_norm is rn.ln_forward
    for n in ("ln_forward", "layer_norm", "rms_norm", "fused_add_rms_norm", "fused_add_layer_norm",
              "softmax_forward", "ln_backward", "rms_norm_backward"):
        assert callable(getattr(rn, n)) and n in rn.__all__


def test_plan_ragged_rows_rule():
    # many rows that are not whole 16-byte chunks, or that do not fill the row group: the
    # byte-addressed vectorized kernel, except 16-bit rows at odd 2-byte positions of the fused
    # ops from 4 waves per row and of RMSNorm from 8 (the element / pair kernels)
    f16, bf16, f32 = torch.float16, torch.bfloat16, torch.float32
    rag = lambda *a, **k: rn.plan(*a, **k)[1]["ragged"]  # noqa: E731
    assert rag("fused_add_rms", 16384, 4095, f16)                  # 2 waves
    assert not rag("fused_add_rms", 8192, 8191, f16)               # 4 waves, odd N
    assert not rag("fused_add_ln", 8192, 8191, bf16)
    assert rag("fused_add_rms", 8192, 8190, f16)                   # even N: rows at 4-byte positions
    assert not rag("fused_add_rms", 8192, 8192, f16, ptrs={"x": (1 << 44) + 2})  # x at an odd element
    assert rag("rms", 8192, 8191, bf16) and not rag("rms", 4096, 16383, f16)     # 4 and 8 waves
    assert rag("ln", 4096, 16383, bf16) and rag("softmax", 8192, 8191, bf16)
    assert rag("rms", 4096, 16383, f32) and rag("fused_add_rms", 8192, 8191, f32)  # fp32: always
    st, info = rn.plan("fused_add_rms", 8192, 8191, f16)
    assert info["variant"] == "element" and info["pairs"] and info["persistent"]
