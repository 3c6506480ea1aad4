"""C-ABI checks that need no GPU: exports, plan validation, counts and layout."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import block_sparse_mixed_amd as da2
from oracle.draft import budget_counts
from oracle.geometry import Geometry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "da2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(da2_\w+)\s*\([^;{]*\)\s*;", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(da2.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", da2.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (da2_\w+)$", out, flags=re.M))
    missing = set(names) - exported
    assert not missing, missing
    lib = ctypes.CDLL(da2.LIB_PATH)
    for n in names:
        assert hasattr(lib, n)


def _cfg(**kw):
    base = dict(batch=1, heads=12, frames=21, grid_h=30, grid_w=52, head_dim=128, win_h=8, win_w=16,
                budget_hi=0.15, budget_lo=0.35)
    base.update(kw)
    return da2.make_config(**base)


def test_plan_wan_shape_matches_oracle_geometry_and_counts():
    p = da2.da2_plan(_cfg())
    i = p.info
    g = Geometry(21, 30, 52, 8, 16)
    assert (i.n_blocks, i.block_size, i.n_wy, i.n_wx) == (g.n_blocks, 128, g.n_wy, g.n_wx) == (336, 128, 4, 4)
    assert (i.n_hi, i.n_lo) == budget_counts(336, 0.15, 0.35) == (50, 118)
    assert i.tokens == 32760 and i.slots == 43008
    assert i.tau == pytest.approx(1 / np.sqrt(128), rel=0, abs=0)


def test_plan_packed_wan_shape():
    p = da2.da2_plan(_cfg(flags=da2.DA2_FLAG_PACK_EDGES))
    i = p.info
    g = Geometry(21, 30, 52, 8, 16, pack_edges=True)
    assert (i.n_blocks, i.n_full, i.flags) == (g.n_blocks, g.n_full, 1) == (256, 189, 1)
    assert (i.n_hi, i.n_lo) == budget_counts(256, 0.15, 0.35) == (38, 90)
    assert i.tokens == 32760 and i.slots == 32768


def test_budget_counts_agree_with_oracle_on_many_configs():
    rng = np.random.default_rng(0)
    for _ in range(300):
        frames, gh, gw = rng.integers(1, 9), rng.integers(1, 40), rng.integers(1, 70)
        wh, ww = [(4, 4), (8, 16), (8, 8), (2, 16)][rng.integers(0, 4)]
        hi = float(rng.choice([0.0, 0.05, 0.1, 0.15, 0.25, 1 / 3, 0.5, 1.0, rng.random()]))
        lo = float(rng.choice([0.0, 0.2, 0.35, 0.4, 1.0, rng.random()]))
        pack = bool(rng.integers(0, 2))
        nb = Geometry(int(frames), int(gh), int(gw), wh, ww, pack_edges=pack).n_blocks
        flags = da2.DA2_FLAG_PACK_EDGES if pack else 0
        try:
            want = budget_counts(nb, hi, lo)
        except ValueError:
            with pytest.raises(da2.Da2Error) as e:
                da2.da2_plan(_cfg(frames=int(frames), grid_h=int(gh), grid_w=int(gw), win_h=wh, win_w=ww,
                                  budget_hi=hi, budget_lo=lo, flags=flags))
            assert e.value.status == da2.DA2_ERR_INVALID_ARG
            continue
        p = da2.da2_plan(_cfg(frames=int(frames), grid_h=int(gh), grid_w=int(gw), win_h=wh, win_w=ww,
                              budget_hi=hi, budget_lo=lo, flags=flags))
        assert (p.info.n_blocks, p.info.n_hi, p.info.n_lo) == (nb, *want)
        assert p.info.flags == flags and p.info.n_full == Geometry(int(frames), int(gh), int(gw), wh, ww).n_full


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), da2.DA2_ERR_INVALID_ARG),
    (dict(head_dim=100), da2.DA2_ERR_UNSUPPORTED),
    (dict(head_dim=256), da2.DA2_ERR_UNSUPPORTED),
    (dict(win_h=16, win_w=16), da2.DA2_ERR_UNSUPPORTED),
    (dict(budget_hi=-0.1), da2.DA2_ERR_INVALID_ARG),
    (dict(budget_hi=1.5), da2.DA2_ERR_INVALID_ARG),
    (dict(budget_hi=0.0, budget_lo=0.0), da2.DA2_ERR_INVALID_ARG),
    (dict(out_dtype=7), da2.DA2_ERR_INVALID_ARG),
    (dict(flags=2), da2.DA2_ERR_INVALID_ARG),
    (dict(flags=3), da2.DA2_ERR_INVALID_ARG),
    (dict(frames=200, grid_h=64, grid_w=64), da2.DA2_ERR_UNSUPPORTED),
    (dict(grid_h=2 ** 31 - 1), da2.DA2_ERR_UNSUPPORTED),
    # launches past 32 bits of work-items: the attention grid (32000 x 336
    # workgroups of 512), the draft logits grid (600 x 2 x 128^2 of 256)
    (dict(batch=2000, heads=16), da2.DA2_ERR_UNSUPPORTED),
    (dict(batch=600, heads=1, frames=128, grid_h=64, grid_w=64), da2.DA2_ERR_UNSUPPORTED),
])
def test_plan_rejects(kw, status):
    with pytest.raises(da2.Da2Error) as e:
        da2.da2_plan(_cfg(**kw))
    assert e.value.status == status


def test_plan_accepts_the_largest_launches():
    # just inside both launch limits: 511 x 2 x 128^2 draft-logits workgroups
    # of 256 and 511 x 4096 attention workgroups of 512 work-items
    p = da2.da2_plan(_cfg(batch=511, heads=1, frames=128, grid_h=64, grid_w=64))
    assert p.info.n_blocks == 4096
    p = da2.da2_plan(_cfg(batch=1560, heads=16, frames=21))        # 24960 x 336 attention workgroups
    assert 24960 * 336 * 512 <= 2 ** 32 - 1


def test_plan_clamps_lo_budget():
    p = da2.da2_plan(_cfg(budget_hi=1.0, budget_lo=0.4))
    assert (p.info.n_hi, p.info.n_lo) == (336, 0)
    p = da2.da2_plan(_cfg(budget_hi=0.0, budget_lo=1.0))
    assert (p.info.n_hi, p.info.n_lo) == (0, 336)


def test_workspace_layout_is_aligned_and_disjoint():
    p = da2.da2_plan(_cfg())
    i = p.info
    bh, nb, T, P = 12, 336, 128, 128
    sizes = {"pool": 4 * bh * nb * P * 8, "k8": bh * nb * T * P,
             "q8": bh * nb * T * P, "v8t": bh * nb * P * T,
             "e8": 3 * bh * nb, "q4": bh * nb * T * P // 2, "k4": bh * nb * T * P // 2, "v4t": bh * nb * P * T // 2,
             "sq4": bh * nb * T * 4, "sk4": bh * nb * T * 4, "sv4t": bh * nb * P * 4, "scores": 2 * bh * nb * nb * 8,
             "labels": bh * nb * nb, "hi": bh * nb * 50 * 4, "lo": bh * nb * 118 * 4, "status": 16,
             "bias": (nb + 1) * T * 4}
    spans = sorted((getattr(i, "off_" + k), getattr(i, "off_" + k) + v) for k, v in sizes.items())
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert all(s % 256 == 0 for s, _ in spans)
    assert spans[-1][1] <= i.workspace_bytes


def test_enqueue_calls_validate_before_touching_the_gpu():
    p = da2.da2_plan(_cfg())
    lib = da2._lib
    fake = 1 << 20     # aligned, never dereferenced: every call below fails validation first
    assert lib.da2_prepare(None, fake, fake, fake, fake, 1 << 40, None) == da2.DA2_ERR_INVALID_ARG
    assert lib.da2_prepare(p.handle, None, fake, fake, fake, 1 << 40, None) == da2.DA2_ERR_INVALID_ARG
    assert lib.da2_prepare(p.handle, fake, fake, fake, fake + 16, 1 << 40, None) == da2.DA2_ERR_WORKSPACE
    assert lib.da2_prepare(p.handle, fake, fake, fake, fake, 100, None) == da2.DA2_ERR_WORKSPACE
    assert lib.da2_attention(p.handle, fake, 100, fake, None) == da2.DA2_ERR_WORKSPACE
    assert lib.da2_attention(p.handle, fake, 1 << 40, None, None) == da2.DA2_ERR_INVALID_ARG
    assert lib.da2_set_labels(p.handle, fake, 1 << 40, None, None) == da2.DA2_ERR_INVALID_ARG
    assert lib.da2_plan_info(None, None) == da2.DA2_ERR_INVALID_ARG
    lib.da2_plan_destroy(None)
    for s in range(5):
        assert da2.status_string(s)
    assert da2.status_string(99) == "unknown status"


def test_last_hip_error_is_clear_before_any_failure():
    name = ctypes.c_char_p()
    assert da2._lib.da2_last_hip_error(ctypes.byref(name)) == 0
    assert name.value.decode() == "hipSuccess"
    assert da2._lib.da2_last_hip_error(None) == 0


def test_wrapper_rejects_mismatched_tensors_before_any_call():
    import torch
    q = torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16)
    args = (1, 8, 8, 4, 4, 0.25, 0.25)
    kt = torch.zeros(1, 64, 2, 32, dtype=torch.bfloat16).transpose(1, 2)     # other strides
    with pytest.raises(ValueError, match="strides"):
        da2.attention(q, kt, q, *args)
    with pytest.raises(ValueError, match="bfloat16"):
        da2.attention(q.float(), q.float(), q.float(), *args)
    with pytest.raises(ValueError, match="shape"):
        da2.attention(q, q[:, :1], q, *args)
    dt = torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16).transpose(2, 3)     # d not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        da2.attention(dt, dt, dt, *args)
    # the token count must be the latent grid's: fewer rows would be read and
    # written past the tensors' ends, more would be left unwritten
    for grid in ((1, 8, 7), (2, 8, 8)):
        with pytest.raises(ValueError, match="latent grid"):
            da2.attention(q, q, q, *grid, *args[3:])
    # the tensors must be on a GPU (these are on the CPU), and the output
    # dtype one the library writes
    with pytest.raises(ValueError, match="GPU"):
        da2.attention(q, q, q, *args)
    with pytest.raises(ValueError, match="out_dtype"):
        da2.attention(q, q, q, *args, out_dtype=torch.float16)


def test_binding_checks_tensor_arguments_before_any_call():
    # tensors handed to the binding's enqueue calls: their dtype, an extent
    # that covers every element the plan's strides reach, and a GPU device,
    # all checked before the library sees a pointer (these are CPU tensors)
    import torch
    n, d = 64, 32
    p = da2.da2_plan(da2.make_config(1, 2, 1, 8, 8, d, 4, 4, 0.25, 0.25))       # fp32 output
    full = torch.zeros(1, 2, n, d, dtype=torch.bfloat16)
    ws = torch.zeros(int(p.info.workspace_bytes), dtype=torch.uint8)
    with pytest.raises(ValueError, match="storage holds"):
        da2.da2_prepare(p, torch.zeros(2 * n * d - 1, dtype=torch.bfloat16), full, full, ws)   # one short
    with pytest.raises(ValueError, match="dtype"):
        da2.da2_prepare(p, full, full.float(), full, ws)
    with pytest.raises(ValueError, match="workspace: dtype"):
        da2.da2_prepare(p, full, full, full, ws.view(torch.int32))
    with pytest.raises(ValueError, match="q must be on a GPU"):
        da2.da2_prepare(p, full, full, full, ws)                                # the right sizes, on the CPU
    with pytest.raises(ValueError, match="out: dtype"):
        da2.da2_attention(p, ws, full)                                          # the plan writes fp32
    with pytest.raises(ValueError, match="storage holds"):
        da2.da2_attention(p, ws, torch.zeros(1, 2, n - 1, d))
    with pytest.raises(ValueError, match="storage holds"):
        da2.da2_forward_scratch(p, full, full, full, torch.zeros(1, 2, n, d - 1))
    with pytest.raises(ValueError, match="labels: dtype"):
        da2.da2_set_labels(p, ws, torch.zeros(2, 16, 16, dtype=torch.uint8))
    # slices of a fused [B, N, 3, H, d] buffer: the strides reach past each
    # slice's own rows, and the last slice ends where the buffer does
    qkv = torch.zeros(1, n, 3, 2, d, dtype=torch.bfloat16)
    sp = da2.da2_plan(da2.make_config(1, 2, 1, 8, 8, d, 4, 4, 0.25, 0.25, strides=(n * 6 * d, d, 6 * d)))
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    with pytest.raises(ValueError, match="q must be on a GPU"):
        da2.da2_prepare(sp, q, k, v, ws)                                        # extents fine
    cut = torch.zeros(qkv.numel() - 1, dtype=torch.bfloat16)                  # a buffer one element short
    with pytest.raises(ValueError, match="v: the plan reaches"):
        da2.da2_prepare(sp, q, k, cut[4 * d:], ws)                              # v's slice of it


def test_enqueue_calls_reject_unaligned_pointers_and_strides():
    # q, k, v and out are read and written in 16-byte vectors: their pointers
    # must be 16-byte aligned and the strides multiples of 8 elements, else
    # DA2_ERR_UNSUPPORTED, reported before anything is enqueued
    lib = da2._lib
    fake = 1 << 20
    big = 1 << 40
    p = da2.da2_plan(_cfg())
    for off in (2, 8):
        assert lib.da2_prepare(p.handle, fake + off, fake, fake, fake, big, None) == da2.DA2_ERR_UNSUPPORTED
        assert lib.da2_prepare(p.handle, fake, fake, fake + off, fake, big, None) == da2.DA2_ERR_UNSUPPORTED
        assert lib.da2_attention(p.handle, fake, big, fake + off, None) == da2.DA2_ERR_UNSUPPORTED
    n = 32760
    for strides in ((12 * n * 132, n * 132, 132), (12 * n * 128 + 4, n * 128, 128), (12 * n * 128, n * 128 + 2, 128),
                    (12 * n * 129, n * 129, 129)):
        p = da2.da2_plan(_cfg(strides=strides))
        assert lib.da2_prepare(p.handle, fake, fake, fake, fake, big, None) == da2.DA2_ERR_UNSUPPORTED
        assert lib.da2_attention(p.handle, fake, big, fake, None) == da2.DA2_ERR_UNSUPPORTED


def test_forward_scratch_rejects_calls_beyond_the_static_workspace():
    # the no-allocation entry point checks its arguments before touching the
    # GPU: a plan whose workspace exceeds the library's static array (a whole
    # Wan-480p step, 12 heads: 393 MiB > 256 MiB) is DA2_ERR_WORKSPACE, and
    # the pointer and stride rules are those of prepare / attention
    lib = da2._lib
    fake = 1 << 20
    big = da2.da2_plan(_cfg())
    assert big.info.workspace_bytes > da2.SCRATCH_BYTES
    assert lib.da2_forward_scratch(big.handle, fake, fake, fake, fake, None) == da2.DA2_ERR_WORKSPACE
    small = da2.da2_plan(_cfg(heads=6))
    assert small.info.workspace_bytes <= da2.SCRATCH_BYTES
    assert lib.da2_forward_scratch(small.handle, fake, fake, fake, fake + 4, None) == da2.DA2_ERR_UNSUPPORTED
    assert lib.da2_forward_scratch(small.handle, fake, None, fake, fake, None) == da2.DA2_ERR_INVALID_ARG
    assert lib.da2_forward_scratch(None, fake, fake, fake, fake, None) == da2.DA2_ERR_INVALID_ARG
