"""Hardware probes behind the design of the kernels (gfx950), run through
libda2_probes.so. Test and measurement infrastructure, not the product path.

    python -m block_sparse_mixed_amd.probes     prints the issue-cost table and
                                                the exactness summaries (needs a GPU)
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(_HERE, "lib", "libda2_probes.so")
_lib = None

KINDS = {0: "v_fma_f32", 1: "v_exp_f32", 2: "v_cvt_pk_fp8_f32 (2 values)", 3: "v_cvt_scalef32_pk_fp4_f32 (2 values)",
         4: "v_cvt_scalef32_pk_bf16_fp8 (2 values)", 5: "v_mfma_f32_32x32x16_bf16",
         6: "v_mfma_scale_f32_32x32x64_f8f6f4 (fp8)", 7: "v_mfma_scale_f32_32x32x64_f8f6f4 (fp4)",
         8: "v_mfma_f32_32x32x16_fp8_fp8", 9: "v_cvt_scalef32_pk_fp8_bf16 (2 values)",
         10: "v_cvt_scalef32_pk_fp4_bf16 (2 values)", 14: "v_mfma_f64_16x16x4_f64", 15: "v_fma_f64"}
ITERS, PER_ITER = 2048, 16


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is missing: build it with `python -m block_sparse_mixed_amd.build`")
        _lib = ctypes.CDLL(PROBE_LIB)
        P = ctypes.c_void_p
        _lib.da2p_widen_fp8.argtypes = [P]
        _lib.da2p_to_fp8.argtypes = [P, P, ctypes.c_int]
        _lib.da2p_to_fp4.argtypes = [P, P, ctypes.c_int]
        _lib.da2p_mfma_fp8.argtypes = [P, P, P, ctypes.c_int]
        _lib.da2p_mfma_f64.argtypes = [P, P, P]
        _lib.da2p_bf16_to.argtypes = [P, ctypes.c_float, P, ctypes.c_int, ctypes.c_int]
        _lib.da2p_issue.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
        _lib.da2p_mem_issue.argtypes = [ctypes.c_int, P, P, P]
        _lib.da2p_lds_read.argtypes = [ctypes.c_int, P, P]
        _lib.da2p_stream.argtypes = [P, P, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, P]
    return _lib


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: HIP error {rc}")


def widen_fp8():
    """bf16 bit patterns [256 codes][4 byte positions] from v_cvt_scalef32_pk_bf16_fp8."""
    import torch
    out = torch.empty(1024, dtype=torch.int16, device="cuda")
    _ok(lib().da2p_widen_fp8(out.data_ptr()), "widen_fp8")
    return out.cpu().numpy().view(np.uint16).reshape(256, 4)


def to_fp8(x: np.ndarray) -> np.ndarray:
    """E4M3 codes of float32 values from v_cvt_pk_fp8_f32."""
    import torch
    xi = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.empty(xi.numel(), dtype=torch.uint8, device="cuda")
    _ok(lib().da2p_to_fp8(xi.data_ptr(), out.data_ptr(), xi.numel()), "to_fp8")
    return out.cpu().numpy()


def to_fp4(x: np.ndarray) -> np.ndarray:
    """E2M1 codes (one per byte) of float32 values from v_cvt_scalef32_pk_fp4_f32, scale 1."""
    import torch
    xi = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.empty(xi.numel(), dtype=torch.uint8, device="cuda")
    _ok(lib().da2p_to_fp4(xi.data_ptr(), out.data_ptr(), xi.numel()), "to_fp4")
    return out.cpu().numpy()


MFMA_PATHS = {"f8f6f4": 0, "bf16": 1, "fp8_k16": 2}


def bf16_to(x_bits: np.ndarray, scale: float, fmt: str) -> np.ndarray:
    """E4M3 (fmt "fp8") or E2M1 (fmt "fp4", one code per byte) codes of bf16
    values (uint16 bit patterns, even count) from v_cvt_scalef32_pk_fp8_bf16 /
    v_cvt_scalef32_pk_fp4_bf16 with the given scale operand."""
    import torch
    xb = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if xb.size % 2:
        raise ValueError("an even number of values")
    xi = torch.from_numpy(xb.view(np.int16)).cuda()
    out = torch.empty(xb.size, dtype=torch.uint8, device="cuda")
    _ok(lib().da2p_bf16_to(xi.data_ptr(), float(scale), out.data_ptr(), xb.size, {"fp8": 0, "fp4": 1}[fmt]), "bf16_to")
    return out.cpu().numpy()


def mfma_fp8(a_codes: np.ndarray, b_codes: np.ndarray, path: str) -> np.ndarray:
    """D = A B for E4M3 code matrices A [32][64], B^T [32][64] (k contiguous),
    on one scaled f8f6f4 MFMA ("f8f6f4"), on bf16 MFMAs over the exactly
    widened codes ("bf16"), or on four unscaled 32x32x16 fp8 MFMAs ("fp8_k16")."""
    import torch
    a = torch.from_numpy(np.ascontiguousarray(a_codes, dtype=np.uint8)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_codes, dtype=np.uint8)).cuda()
    d = torch.empty(32 * 32, dtype=torch.float32, device="cuda")
    _ok(lib().da2p_mfma_fp8(a.data_ptr(), b.data_ptr(), d.data_ptr(), MFMA_PATHS[path]), "mfma_fp8")
    return d.cpu().numpy().reshape(32, 32)


def mfma_f64(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """One 16x16x4 fp64 MFMA on A [16][4] and B [4][16], read back with the
    result layout the draft logits kernel assumes (lane l, element e -> row
    l / 16 + 4 e, column l % 16): equals A @ B when that layout holds."""
    import torch
    at = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).cuda()
    bt = torch.from_numpy(np.ascontiguousarray(b, dtype=np.float64)).cuda()
    d = torch.empty(16 * 16, dtype=torch.float64, device="cuda")
    _ok(lib().da2p_mfma_f64(at.data_ptr(), bt.data_ptr(), d.data_ptr()), "mfma_f64")
    return d.cpu().numpy().reshape(16, 16)


# flops per MFMA instruction of kinds 5, 6, 7, 8
MFMA_FLOP = {5: 2 * 32 * 32 * 16, 6: 2 * 32 * 32 * 64, 7: 2 * 32 * 32 * 64, 8: 2 * 32 * 32 * 16, 14: 2 * 16 * 16 * 4,
             15: 2 * 64}


def _issue_raw(kind: int, waves_per_simd: int):
    import time

    import torch
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(256 * 8, dtype=torch.int64, device="cuda")
    _ok(lib().da2p_issue(kind, waves_per_simd, sink.data_ptr(), cyc.data_ptr()), "issue")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _ok(lib().da2p_issue(kind, waves_per_simd, sink.data_ptr(), cyc.data_ptr()), "issue")   # synchronises
    wall = time.perf_counter() - t0
    return cyc.cpu().numpy()[: 256 * 4 * waves_per_simd].reshape(256, 4 * waves_per_simd), wall


def issue_cycles(kind: int, waves_per_simd: int):
    """(clock-counter ticks per instruction of one kind per wave, averaged over
    the launch; wall seconds of the launch) for one workgroup per CU and 1 or
    2 waves per SIMD (256 workgroups)."""
    c, wall = _issue_raw(kind, waves_per_simd)
    return float(c.mean()) / (ITERS * PER_ITER), wall


def overlap():
    """Whether an exponential or an E2M1 pack conversion shares issue time with
    independent FMAs: ticks per step of an exponential (pack conversion) paired
    with an FMA in one wave per SIMD, beside the ticks of each alone; and, with
    two waves per SIMD, one issuing exponentials and the other FMAs, each
    wave's ticks per instruction and the launch's wall time beside the
    two-wave launches of either kind alone."""
    step = ITERS * PER_ITER
    t_fma, w_fma2 = issue_cycles(0, 1)[0], issue_cycles(0, 2)[1]
    t_exp, w_exp2 = issue_cycles(1, 1)[0], issue_cycles(1, 2)[1]
    t_cvt = issue_cycles(3, 1)[0]
    t11 = issue_cycles(11, 1)[0]
    t12 = issue_cycles(12, 1)[0]
    c13, w13 = _issue_raw(13, 2)
    return {"fma": t_fma, "exp": t_exp, "cvt_pk_fp4": t_cvt, "exp+fma": t11, "cvt_pk_fp4+fma": t12,
            "mixed_exp_wave": float(c13[:, :4].mean()) / step, "mixed_fma_wave": float(c13[:, 4:].mean()) / step,
            "mixed_wall": w13, "exp2_wall": w_exp2, "fma2_wall": w_fma2}


MEM_MODES = {0: "16 FMAs only", 1: "global_load_dwordx4 + 16 FMAs", 2: "global_load_lds_dwordx4 + 16 FMAs",
             3: "ds_write_b128 + 16 FMAs", 4: "global_load_dwordx4, 8 back to back", 5: "global_load_lds_dwordx4, 8 back to back",
             6: "ds_write_b128, 8 back to back"}


def mem_issue_cycles(mode: int) -> float:
    """Clocks per (memory instruction + 16 FMAs), one wave per SIMD, per wave."""
    import torch
    src = torch.zeros(256 * 4 * 512 + 64, 4, dtype=torch.int32, device="cuda")
    out = torch.empty(256 * 256, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(256 * 4, dtype=torch.int64, device="cuda")
    for _ in range(2):
        _ok(lib().da2p_mem_issue(mode, src.data_ptr(), out.data_ptr(), cyc.data_ptr()), "mem_issue")
    return float(cyc.cpu().numpy().mean()) / (512 * 8)


def lds_read_rate(waves: int):
    """(clocks per ds_read_b128 per wave, bytes per clock per CU, wall TB/s
    over the chip) for one workgroup of `waves` waves per CU streaming reads
    from LDS."""
    import time

    import torch
    sink = torch.empty(256 * 1024, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(256 * 16, dtype=torch.int64, device="cuda")
    _ok(lib().da2p_lds_read(waves, sink.data_ptr(), cyc.data_ptr()), "lds_read")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _ok(lib().da2p_lds_read(waves, sink.data_ptr(), cyc.data_ptr()), "lds_read")   # synchronises
    wall = time.perf_counter() - t0
    c = float(cyc.view(256, 16)[:, :waves].float().mean())
    reads = 1024 * 16
    return c / reads, waves * reads * 1024 / c, 256 * waves * reads * 1024 / wall / 1e12


# The preparation's algorithmic traffic at the Wan-480p shape (12 heads,
# 32760 tokens, d 128): the bf16 Q, K and V read once (exact), and about
# 312 MB of codes, scales and pools for the padded tiles written.
PREP_READ_BYTES = 3 * 12 * 32760 * 128 * 2
PREP_WRITE_BYTES = 312_000_000


def stream_bandwidth(read_bytes: int, write_bytes: int, grids=(1024, 2048, 4096, 8192), reps: int = 5):
    """{grid: TB/s} of a plain streaming kernel that reads read_bytes and
    writes write_bytes: the shortest of `reps` launches after a warm-up, each
    timed alone with HIP events in the probe library."""
    import torch
    read_bytes, write_bytes = read_bytes // 16 * 16, write_bytes // 16 * 16
    src = torch.ones(max(read_bytes, 16), dtype=torch.uint8, device="cuda")
    dst = torch.empty(max(write_bytes, 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    out = {}
    for grid in grids:
        ms = ctypes.c_float()
        _ok(lib().da2p_stream(src.data_ptr(), dst.data_ptr(), read_bytes, write_bytes, grid, reps, ctypes.byref(ms)),
            "stream")
        out[grid] = (read_bytes + write_bytes) / (ms.value * 1e-3) / 1e12
    return out

def main():
    import torch
    print(f"device: {torch.cuda.get_device_name(0)}")
    print("\nticks: clock-counter ticks (shader cycles) per instruction with one wave per SIMD;")
    print("two waves: the same instruction stream in two waves per SIMD, as ticks per instruction")
    print("per SIMD from the wall-time ratio of the two launches (ticks_1 * wall_2 / (2 * wall_1)).")
    print("\n| instruction | ticks, 1 wave/SIMD | ticks per instruction per SIMD, 2 waves | TFLOP/s, 1 / 2 waves |")
    print("|---|---|---|---|")
    for k, name in KINDS.items():
        t1, w1 = issue_cycles(k, 1)
        _, w2 = issue_cycles(k, 2)
        n1 = 256 * 4 * ITERS * PER_ITER
        tf = f"{n1 * MFMA_FLOP[k] / w1 / 1e12:.0f} / {2 * n1 * MFMA_FLOP[k] / w2 / 1e12:.0f}" if k in MFMA_FLOP else ""
        print(f"| {name} | {t1:.1f} | {t1 * w2 / (2 * w1):.1f} | {tf} |")
    o = overlap()
    print("\noverlap of exponentials and pack conversions with independent FMAs (ticks per step):")
    print("\n| stream | ticks | the two alone, summed |")
    print("|---|---|---|")
    print(f"| v_exp_f32 + v_fma_f32, one wave per SIMD | {o['exp+fma']:.1f} | {o['exp'] + o['fma']:.1f} |")
    print(f"| v_cvt_scalef32_pk_fp4_f32 + v_fma_f32, one wave per SIMD | {o['cvt_pk_fp4+fma']:.1f} | "
          f"{o['cvt_pk_fp4'] + o['fma']:.1f} |")
    print(f"\ntwo waves per SIMD, one of exponentials and one of FMAs: exponential wave "
          f"{o['mixed_exp_wave']:.1f} ticks per instruction, FMA wave {o['mixed_fma_wave']:.1f}; wall "
          f"{o['mixed_wall'] * 1e3:.2f} ms against {o['exp2_wall'] * 1e3:.2f} ms (two exponential waves) and "
          f"{o['fma2_wall'] * 1e3:.2f} ms (two FMA waves)")
    print("\nmemory instructions among independent FMAs, one wave per SIMD (ticks per memory instruction")
    print("and its 16 FMAs; the difference to the FMA-only row is the memory instruction's issue cost):")
    print("\n| stream | ticks |")
    print("|---|---|")
    for mode, name in MEM_MODES.items():
        print(f"| {name} | {mem_issue_cycles(mode):.1f} |")
    print("\nLDS reads (ds_read_b128, 1 KiB per instruction), one workgroup per CU:")
    print("\n| waves per CU | clocks per read per wave | bytes per clock per CU | TB/s over 256 CUs (wall) |")
    print("|---|---|---|---|")
    for waves in (4, 8, 16):
        per, bpc, tbs = lds_read_rate(waves)
        print(f"| {waves} | {per:.1f} | {bpc:.0f} | {tbs:.0f} |")
    print("\nstreaming HBM bandwidth of a plain kernel (16-byte accesses, 256 threads a workgroup), best of 5:")
    print("\n| traffic | 1024 groups | 2048 | 4096 | 8192 |")
    print("|---|---|---|---|---|")
    for name, r, w in (("the preparation's volume at Wan-480p: 302 MB read + 312 MB written", PREP_READ_BYTES,
                        PREP_WRITE_BYTES), ("302 MB read", PREP_READ_BYTES, 0), ("312 MB written", 0, PREP_WRITE_BYTES)):
        bw = stream_bandwidth(r, w)
        print(f"| {name} | " + " | ".join(f"{bw[g]:.2f} TB/s" for g in (1024, 2048, 4096, 8192)) + " |")

if __name__ == "__main__":
    main()
