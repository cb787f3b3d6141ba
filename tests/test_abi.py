"""C-ABI checks that need no GPU: the library loads, exports every entry point
its header declares, mirrors the options struct, sizes the workspace, and
rejects bad arguments before making any HIP call (so only invalid calls are
made here)."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_logits_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = moe.load_library()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_opts_struct_mirror_matches_library():
    o = moe.new_opts()
    assert o.struct_size == ctypes.sizeof(moe.MoeOpts)
    assert o.dtype == 0 and o.routed_scale == 1.0 and o.flags == 0 and o.workspace is None


def test_workspace_bytes_valid_and_monotone():
    a = moe.workspace_bytes(32, 4096, 6400, 16, 2)
    b = moe.workspace_bytes(4096, 4096, 6400, 16, 2)
    c = moe.workspace_bytes(4096, 4096, 6400, 16, 2, shared_I=1024)
    assert 0 < a < b < c
    assert a % 256 == 0 and b % 256 == 0
    # h (bf16) and the fp32 slots dominate: T*k*(2I + 4H) bytes
    assert b >= 4096 * 2 * (2 * 6400 + 4 * 4096)
    assert moe.workspace_bytes(0, 64, 64, 4, 2) >= 0


@pytest.mark.parametrize("T,H,I,E,k,msg", [
    (4, 4096, 6400, 16, 0, "k = 0"),
    (4, 4096, 6400, 16, 17, "k = 17"),
    (4, 4100, 6400, 16, 2, "H = 4100"),
    (4, 4096, 6404, 16, 2, "I = 6404"),
    (4, 4096, 6400, 257, 2, "E = 257"),
    (-1, 4096, 6400, 16, 2, "T = -1"),
])
def test_workspace_bytes_rejects_bad_sizes(T, H, I, E, k, msg):
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_bytes(T, H, I, E, k)
    assert ei.value.status == -1 and msg in str(ei.value)


def call(T=4, H=64, I=32, E=4, k=2, opts=None, ptrs=None, out=None):
    """moe_forward with fake device addresses: only argument checks may run."""
    lib = moe.load_library()
    base = 1 << 40
    p = ptrs or dict(hidden=base, router_w=base + (1 << 30), gate_up=base + (2 << 30), down=base + (3 << 30))
    if out is None:
        out = base + (4 << 30)
    o = opts if opts is not None else moe.new_opts()
    vp = ctypes.c_void_p
    rc = lib.moe_forward(vp(p["hidden"]), vp(p["router_w"]), vp(p["gate_up"]), vp(p["down"]), T, H, I, E, k,
                         ctypes.byref(o) if o is not False else None, vp(out))
    return rc, moe.last_error()


def good_opts(nbytes=1 << 30):
    o = moe.new_opts()
    o.workspace = (1 << 40) + (8 << 30)
    o.workspace_bytes = nbytes
    return o


def test_rejects_null_opts():
    assert call(opts=False)[0] == -1


def test_rejects_wrong_struct_size():
    o = good_opts()
    o.struct_size = 64
    rc, msg = call(opts=o)
    assert rc == -1 and "struct_size" in msg


def test_rejects_bad_k_and_dtype():
    assert call(k=5, opts=good_opts())[0] == -1
    o = good_opts()
    o.dtype = 7
    assert call(opts=o)[0] == -1


def test_zero_tokens_succeeds_without_pointers():
    rc, _ = call(T=0, opts=good_opts(), ptrs=dict(hidden=0, router_w=0, gate_up=0, down=0), out=0)
    assert rc == 0


def test_rejects_null_and_misaligned_pointers():
    base = 1 << 40
    p = dict(hidden=0, router_w=base + (1 << 30), gate_up=base + (2 << 30), down=base + (3 << 30))
    assert call(opts=good_opts(), ptrs=p)[0] == -1
    p["hidden"] = base + 8
    rc, msg = call(opts=good_opts(), ptrs=p)
    assert rc == -4 and "aligned" in msg


def test_rejects_small_or_missing_workspace():
    rc, msg = call(opts=good_opts(nbytes=100))
    assert rc == -3 and "needed" in msg
    o = good_opts()
    o.workspace = None
    assert call(opts=o)[0] == -3
    o = good_opts()
    o.workspace = (1 << 40) + (8 << 30) + 16
    assert call(opts=o)[0] == -4


def test_rejects_output_aliasing_an_input():
    base = 1 << 40
    rc, msg = call(opts=good_opts(), out=base + 64)
    assert rc == -1 and "overlaps" in msg


def test_rejects_shared_expert_without_weights_and_bad_flags():
    o = good_opts()
    o.shared_I = 16
    assert call(opts=o)[0] == -1
    o = good_opts()
    o.shared_I = 12
    assert call(opts=o)[0] == -1
    o = good_opts()
    o.flags = moe.FLAG_FORCE_TILED | moe.FLAG_FORCE_SKINNY
    assert call(opts=o)[0] == -1
    o = good_opts()
    o.flags = 0x80
    assert call(opts=o)[0] == -1
    o = good_opts()
    o.routed_scale = float("nan")
    assert call(opts=o)[0] == -1


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(FileNotFoundError):
        moe.load_library()


def fp8_opts():
    o = good_opts(nbytes=100)  # too small: a valid call stops at the workspace check, before any HIP call
    o.weight_format = moe.WEIGHTS_FP8_E4M3
    o.gate_up_scale = (1 << 40) + (5 << 30)
    o.down_scale = (1 << 40) + (6 << 30)
    return o


def test_fp8_weight_options_are_checked():
    rc, msg = call(opts=fp8_opts())  # valid apart from the fake addresses: reaches the workspace check
    assert rc == -3, msg
    o = fp8_opts()
    o.gate_up_scale = None
    rc, msg = call(opts=o)
    assert rc == -1 and "scale" in msg
    o = fp8_opts()
    o.dtype = 1
    rc, msg = call(opts=o)
    assert rc == -2 and "bf16" in msg
    o = fp8_opts()
    o.flags = moe.FLAG_FORCE_TILED
    assert call(opts=o)[0] == -2
    rc, msg = call(H=72, opts=fp8_opts())  # H a multiple of 8 but not of 16
    assert rc == -2 and "16" in msg
    o = fp8_opts()
    o.weight_format = 9
    assert call(opts=o)[0] == -1
    o = fp8_opts()
    o.down_scale = (1 << 40) + (6 << 30) + 2
    assert call(opts=o)[0] == -4
    rc, msg = call(opts=fp8_opts(), out=(1 << 40) + (6 << 30))  # out on top of down_scale
    assert rc == -1 and "overlaps" in msg


def test_quantize_entry_point_checks_arguments():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    base = 1 << 40
    w, q, s = vp(base), vp(base + (1 << 30)), vp(base + (2 << 30))
    assert lib.moe_quantize_fp8_rows(w, 0, 64, q, s, None) == 0  # no rows: nothing to do
    assert lib.moe_quantize_fp8_rows(w, 4, 40, q, s, None) == -1  # cols not a multiple of 16
    assert lib.moe_quantize_fp8_rows(w, -1, 64, q, s, None) == -1
    assert lib.moe_quantize_fp8_rows(None, 4, 64, q, s, None) == -1
    assert lib.moe_quantize_fp8_rows(vp(base + 8), 4, 64, q, s, None) == -4
    assert lib.moe_quantize_fp8_rows(w, 4, 64, vp(base + 64), s, None) == -1  # q overlaps w


def test_router_stats_outputs_must_be_aligned():
    o = good_opts(nbytes=100)
    o.aux_loss = (1 << 40) + (7 << 30) + 2
    assert call(opts=o)[0] == -4
    o = good_opts(nbytes=100)
    o.router_prob_mean = (1 << 40) + (7 << 30)
    o.stats_mask = (1 << 40) + (7 << 30) + 4096
    assert call(opts=o)[0] == -3  # valid: stops at the (too small) workspace, before any HIP call


def scoring_opts(score_func=moe.SCORE_SIGMOID, n_group=0, topk_group=0):
    o = good_opts(nbytes=100)  # valid calls stop at the workspace check, before any HIP call
    o.score_func = score_func
    o.selection_bias = (1 << 40) + (7 << 30)
    o.n_group = n_group
    o.topk_group = topk_group
    return o


def test_scoring_options_are_checked():
    E, k = 16, 4
    assert call(E=E, k=k, opts=scoring_opts())[0] == -3
    assert call(E=E, k=k, opts=scoring_opts(n_group=4, topk_group=2))[0] == -3
    assert call(E=E, k=k, opts=scoring_opts(n_group=1, topk_group=0))[0] == -3  # one group: no grouping
    rc, msg = call(E=E, k=k, opts=scoring_opts(score_func=3))
    assert rc == -1 and "score_func" in msg
    rc, msg = call(E=E, k=k, opts=scoring_opts(n_group=3, topk_group=1))
    assert rc == -1 and "multiple of n_group" in msg
    for tg in (0, 5):
        rc, msg = call(E=E, k=k, opts=scoring_opts(n_group=4, topk_group=tg))
        assert rc == -1 and "topk_group" in msg
    rc, msg = call(E=E, k=k, opts=scoring_opts(n_group=8, topk_group=1))  # 2 experts < k
    assert rc == -1 and "k = 4" in msg
    rc, msg = call(E=256, k=k, opts=scoring_opts(n_group=128, topk_group=4))
    assert rc == -2 and "n_group" in msg
    assert call(E=E, k=k, opts=scoring_opts(n_group=-2))[0] == -1
    o = scoring_opts()
    o.selection_bias = (1 << 40) + (7 << 30) + 2
    assert call(E=E, k=k, opts=o)[0] == -4
    rc, msg = call(E=E, k=k, opts=scoring_opts(), out=(1 << 40) + (7 << 30))  # out on top of the bias
    assert rc == -1 and "overlaps" in msg


def test_sparsemixer_options_are_checked():
    o = moe.new_opts()
    assert abs(o.jitter_eps - 0.01) < 1e-9  # PhiMoE's router_jitter_noise
    assert call(E=16, k=2, opts=scoring_opts(score_func=moe.SCORE_SPARSEMIXER))[0] == -1  # no selection bias
    o = scoring_opts(score_func=moe.SCORE_SPARSEMIXER)
    o.selection_bias = None
    assert call(E=16, k=2, opts=o)[0] == -3
    o.n_group, o.topk_group = 4, 2
    rc, msg = call(E=16, k=2, opts=o)
    assert rc == -1 and "sparsemixer" in msg
    for eps in (-0.5, float("nan"), float("inf")):
        o = scoring_opts(score_func=moe.SCORE_SPARSEMIXER)
        o.selection_bias = None
        o.jitter_eps = eps
        rc, msg = call(E=16, k=2, opts=o)
        assert rc == -1 and "jitter_eps" in msg


def mxfp4_opts():
    o = good_opts(nbytes=100)  # too small: a valid call stops at the workspace check
    o.weight_format = moe.WEIGHTS_MXFP4
    o.gate_up_block_scale = (1 << 40) + (5 << 30)
    o.down_block_scale = (1 << 40) + (6 << 30) + 1  # byte arrays: any alignment
    return o


def test_mxfp4_weight_options_are_checked():
    rc, msg = call(opts=mxfp4_opts())
    assert rc == -3, msg
    o = mxfp4_opts()
    o.down_block_scale = None
    rc, msg = call(opts=o)
    assert rc == -1 and "block_scale" in msg
    o = mxfp4_opts()
    o.dtype = 1
    assert call(opts=o)[0] == -2
    o = mxfp4_opts()
    o.flags = moe.FLAG_FORCE_TILED
    assert call(opts=o)[0] == -2
    rc, msg = call(H=80, opts=mxfp4_opts())  # a multiple of 16 but not of 32
    assert rc == -2 and "32" in msg
    rc, msg = call(opts=mxfp4_opts(), out=(1 << 40) + (5 << 30))  # out on top of a block scale
    assert rc == -1 and "overlaps" in msg


def test_mxfp4_quantize_entry_point_checks_arguments():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    base = 1 << 40
    w, q, s = vp(base), vp(base + (1 << 30)), vp(base + (2 << 30))
    assert lib.moe_quantize_mxfp4_rows(w, 0, 64, q, s, None) == 0
    assert lib.moe_quantize_mxfp4_rows(w, 4, 48, q, s, None) == -1  # not a multiple of 32
    assert lib.moe_quantize_mxfp4_rows(w, -1, 64, q, s, None) == -1
    assert lib.moe_quantize_mxfp4_rows(None, 4, 64, q, s, None) == -1
    assert lib.moe_quantize_mxfp4_rows(vp(base + 8), 4, 64, q, s, None) == -4
    assert lib.moe_quantize_mxfp4_rows(w, 4, 64, vp(base + 64), s, None) == -1  # q overlaps w


def test_rejects_shared_expert_past_32_bit_offsets():
    # 2 * shared_I * H = 2^31 elements: the shared expert's offsets would overflow
    with pytest.raises(moe.MoeError) as ei:
        moe.workspace_bytes(4, 4096, 64, 4, 2, shared_I=1 << 18)
    assert ei.value.status == -2 and "shared expert" in str(ei.value)
    assert moe.workspace_bytes(4, 4096, 64, 4, 2, shared_I=(1 << 18) - 8) > 0


def test_rejects_workspace_overlapping_an_input():
    base = 1 << 40
    o = good_opts()
    o.workspace = base + (3 << 30)  # on top of down
    rc, msg = call(opts=o)
    assert rc == -1 and "workspace overlaps" in msg


def test_rejects_optional_outputs_overlapping_inputs_workspace_out_or_each_other():
    base = 1 << 40
    o = good_opts(nbytes=100)
    o.topk_ids = base + (8 << 30) + 32  # inside the workspace
    rc, msg = call(opts=o)
    assert rc == -1 and "optional output" in msg
    o = good_opts(nbytes=100)
    o.perm = base + 256  # inside hidden
    rc, msg = call(opts=o)
    assert rc == -1 and "optional output" in msg
    o = good_opts(nbytes=100)
    o.router_logits = base + (4 << 30) + 64  # inside out
    rc, msg = call(opts=o)
    assert rc == -1 and "overlaps out" in msg
    o = good_opts(nbytes=100)
    o.expert_counts = base + (9 << 30)
    o.expert_offsets = base + (9 << 30) + 8  # E = 4: counts span 16 bytes
    rc, msg = call(opts=o)
    assert rc == -1 and "two optional outputs" in msg
    o = good_opts(nbytes=100)
    o.expert_counts = base + (9 << 30)
    o.expert_offsets = base + (9 << 30) + 16  # adjacent, not overlapping: reaches the workspace check
    assert call(opts=o)[0] == -3


CONCURRENT_FIRST_CALLS = r"""
import ctypes, sys, threading
sys.path.insert(0, sys.argv[1])
import sparse_mixture_experts_logits_amd as moe
lib = moe.load_library()
vp = ctypes.c_void_p
base = 1 << 40
cases = [(5, -1, "k = 5"), (0, -1, "k = 0"), (3, -3, "needed"), (2, -3, "needed")] * 8
start = threading.Barrier(len(cases))
bad = []
def run(i, k, want_rc, want_msg):
    o = moe.MoeOpts()
    lib.moe_opts_init(ctypes.byref(o))
    o.workspace = base + (8 << 30)
    o.workspace_bytes = 64
    start.wait()
    for _ in range(200):
        rc = lib.moe_forward(vp(base), vp(base + (1 << 30)), vp(base + (2 << 30)), vp(base + (3 << 30)),
                             16, 64, 32, 4, k, ctypes.byref(o), vp(base + (4 << 30)))
        msg = lib.moe_last_error().decode()
        if rc != want_rc or want_msg not in msg:
            bad.append((i, k, rc, msg))
            return
threads = [threading.Thread(target=run, args=(i, *c)) for i, c in enumerate(cases)]
for t in threads: t.start()
for t in threads: t.join()
print("BAD" if bad else "OK", bad[:3])
"""


def test_concurrent_first_calls_on_check_paths():
    """Many host threads make their first calls at once (a fresh process):
    each sees its own status and its own thread-local message."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", CONCURRENT_FIRST_CALLS, ROOT], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("OK"), r.stdout


def test_noalloc_entry_point_checks_arguments():
    # the allocation-free entry point takes no workspace and rejects sizes its
    # scratch cannot hold, before any HIP call
    o = moe.new_opts()
    o.workspace = (1 << 40) + (8 << 30)
    o.workspace_bytes = 1 << 20
    lib = moe.load_library()
    vp = ctypes.c_void_p
    base = 1 << 40
    args = (vp(base), vp(base + (1 << 30)), vp(base + (2 << 30)), vp(base + (3 << 30)))
    rc = lib.moe_forward_noalloc(*args, 4, 64, 32, 4, 2, ctypes.byref(o), vp(base + (4 << 30)))
    assert rc == -1 and "workspace must be NULL" in moe.last_error()
    o = moe.new_opts()
    rc = lib.moe_forward_noalloc(*args, 4096, 4096, 6400, 16, 2, ctypes.byref(o), vp(base + (4 << 30)))
    assert rc == -2 and "scratch" in moe.last_error()
    assert moe.workspace_bytes(4096, 4096, 6400, 16, 2) > moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(*args, 4, 64, 32, 4, 0, ctypes.byref(o), vp(base + (4 << 30))) == -1
    assert lib.moe_forward_noalloc(*args, 4, 64, 32, 4, 2, None, vp(base + (4 << 30))) == -1
    # T = 0 succeeds without touching the device
    assert lib.moe_forward_noalloc(None, None, None, None, 0, 64, 32, 4, 2, ctypes.byref(o), None) == 0
    # the decode step fits
    assert moe.workspace_bytes(32, 4096, 6400, 16, 2) <= moe.NOALLOC_SCRATCH_BYTES


def test_low_precision_weights_serve_the_streaming_schedule_only():
    # FP8 / MXFP4 weights have no tiled kernel: batches past T*k <= 32*E are
    # refused (before any HIP call) instead of re-streaming every expert's
    # weights once per 16 rows
    for make in (fp8_opts, mxfp4_opts):
        rc, msg = call(T=64, E=4, k=2, opts=make())  # 128 <= 128: reaches the workspace check
        assert rc == -3, msg
        rc, msg = call(T=65, E=4, k=2, opts=make())
        assert rc == -2 and "T*k <= 32*E" in msg


def test_workspace_of_each_schedule():
    # at most 32 tokens: the streaming kernels alone, no split-tile buffer;
    # more tokens but few rows per expert on average: the mixed schedule,
    # whose tiled launch may split its few tiles along K (the buffer), and
    # which still fits the allocation-free entry point's scratch
    split = 256 * 8 * 9 * 4096  # partial sums of 256 split pieces
    decode = moe.workspace_bytes(32, 4096, 6400, 16, 2)
    assert decode < split
    mixed = moe.workspace_bytes(256, 4096, 6400, 16, 2)
    forced = moe.workspace_bytes(256, 4096, 6400, 16, 2, flags=moe.FLAG_FORCE_SKINNY)
    assert mixed - forced >= split
    assert mixed <= moe.NOALLOC_SCRATCH_BYTES


def blocks_opts():
    o = good_opts(nbytes=100)  # too small: a valid call stops at the workspace check
    o.weight_layout = moe.LAYOUT_TILE_BLOCKS
    return o


def test_tile_blocks_bytes_follow_the_header():
    # E * ceil(I/128) * ceil(H/32) * 16 KB (gate_up), E * ceil(H/256) * ceil(I/32) * 16 KB (down)
    for E, I, H in ((16, 6400, 4096), (4, 200, 328), (1, 8, 8), (64, 1024, 2048), (3, 136, 264)):
        gu = moe.tile_blocks_bytes(moe.PACK_GATE_UP, E, I, H)
        dn = moe.tile_blocks_bytes(moe.PACK_DOWN, E, I, H)
        assert gu == E * (-(-I // 128)) * (-(-H // 32)) * 256 * 32 * 2
        assert dn == E * (-(-H // 256)) * (-(-I // 32)) * 256 * 32 * 2
        # never smaller than the nn.Linear layout; equal when the blocks tile it exactly
        assert gu >= E * 2 * I * H * 2 and dn >= E * H * I * 2
    assert moe.tile_blocks_bytes(moe.PACK_GATE_UP, 16, 6400, 4096) == 16 * 2 * 6400 * 4096 * 2
    lib = moe.load_library()
    assert lib.moe_tile_blocks_bytes(2, 4, 32, 64) == -1          # which
    assert lib.moe_tile_blocks_bytes(0, 0, 32, 64) == -1          # E
    assert lib.moe_tile_blocks_bytes(0, 4, 36, 64) == -1          # I not a multiple of 8
    assert lib.moe_tile_blocks_bytes(1, 4, 32, 0) == -1           # H
    assert lib.moe_tile_blocks_bytes(0, 4, 8, 1 << 24) == -2      # one expert's blocks past 2^31 bytes


def test_pack_tile_blocks_checks_arguments():
    lib = moe.load_library()
    vp = ctypes.c_void_p
    base = 1 << 40
    w, out = vp(base), vp(base + (1 << 30))
    assert lib.moe_pack_tile_blocks(3, w, 4, 32, 64, out, None) == -1
    assert lib.moe_pack_tile_blocks(0, None, 4, 32, 64, out, None) == -1
    assert lib.moe_pack_tile_blocks(0, w, 4, 32, 64, None, None) == -1
    assert lib.moe_pack_tile_blocks(0, vp(base + 8), 4, 32, 64, out, None) == -4
    assert lib.moe_pack_tile_blocks(1, w, 4, 32, 64, vp(base + 4096), None) == -1  # out overlaps w
    assert "overlaps" in moe.last_error()


def test_tile_block_layout_options_are_checked():
    rc, msg = call(opts=blocks_opts())  # valid apart from the fake addresses: reaches the workspace check
    assert rc == -3, msg
    o = blocks_opts()
    o.weight_layout = 5
    rc, msg = call(opts=o)
    assert rc == -1 and "weight_layout" in msg
    o = blocks_opts()
    o.dtype = 1
    assert call(opts=o)[0] == -2
    o = blocks_opts()
    o.weight_format = moe.WEIGHTS_FP8_E4M3
    o.gate_up_scale = (1 << 40) + (5 << 30)
    o.down_scale = (1 << 40) + (6 << 30)
    assert call(opts=o)[0] == -2
    o = blocks_opts()
    o.flags = moe.FLAG_FORCE_SKINNY
    rc, msg = call(opts=o)
    assert rc == -1 and "tiled" in msg
    # the blocks are larger than the rows when the tiles overhang (I = 200: two
    # 128-row halves per expert): out just past the rows' end but inside the blocks
    E, I, H = 4, 200, 328
    rows_end = (1 << 40) + (2 << 30) + E * 2 * I * H * 2
    rc, msg = call(T=4, H=H, I=I, E=E, opts=blocks_opts(), out=rows_end + 256)
    assert rc == -1 and "overlaps" in msg
    rc, _ = call(T=4, H=H, I=I, E=E, opts=good_opts(nbytes=100), out=rows_end + 256)
    assert rc == -3  # the row layout ends before out


def test_tile_blocks_take_the_tiled_schedule_at_any_size():
    # the blocks are read by the tiled kernels only: a decode-sized call sizes
    # the split-K buffer of the tiled schedule
    o = moe.new_opts()
    o.weight_layout = moe.LAYOUT_TILE_BLOCKS
    lib = moe.load_library()
    blocks = lib.moe_workspace_bytes(32, 4096, 6400, 16, 2, ctypes.byref(o))
    tiled = moe.workspace_bytes(32, 4096, 6400, 16, 2, flags=moe.FLAG_FORCE_TILED)
    assert blocks == tiled > moe.workspace_bytes(32, 4096, 6400, 16, 2)
