"""Host-side check that every buffer range the GEMM, block-product and Gram
kernels build stays inside its operand, for the launches of every shape the
GPU tests and bench.py run and for the largest shapes the library accepts.
The ranges come from the kernels' own header (csrc/ranges.h), compiled here
with the host compiler; tests/ranges_check.cpp enumerates the workgroups."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))

# (m, n, b, N) of the layers the GPU tests and the bench run
SHAPES = [
    (96, 80, 32, 37), (300, 200, 64, 50), (256, 512, 128, 33), (600, 520, 256, 70), (1100, 700, 512, 40),
    (70, 90, 32, 1), (20, 40, 32, 5), (512, 256, 256, 129), (4360, 4104, 256, 45), (2048, 2048, 256, 45),
    (2112, 2240, 64, 70), (256, 768, 256, 70), (130, 64, 64, 45), (64, 300, 64, 45), (200, 96, 32, 37),
    (512, 1024, 512, 24), (512, 1024, 32, 20), (384, 320, 64, 4), (256, 256, 64, 40), (512, 384, 128, 96),
    (256, 256, 32, 64), (2048, 2048, 256, 4096),
    (2048, 2048, 256, 8192), (5632, 2048, 256, 8192), (2048, 5632, 256, 8192),
    (11008, 4096, 64, 8192), (11008, 4096, 128, 8192), (11008, 4096, 256, 8192), (11008, 4096, 512, 8192),
    (5632, 2048, 256, 2432), (5632, 2048, 256, 896),   # token chunks of the allocation-free forward
    # the largest layer the library accepts, with token counts around the 32-bit cuts
    (32768, 32768, 256, 8192), (32768, 32768, 512, 4096), (32768, 32768, 128, 40000), (32768, 2048, 256, 70000),
]


def launches(m, n, b, N):
    kR, kP = m // b, n // b
    out = ["gemm nt %d %d %d %d %d" % (N, m, n, n, n),       # z2' = z1' W0p^T
           "gemm nn %d %d %d %d %d" % (N, n, m, m, n)]       # gz1' = gz2' W0p
    for W, k in ((n, kP), (m, kR)):
        if k == 0:
            continue
        if b <= 256 and W % 8 == 0:
            out.append("bdiag %d %d %d %d %d" % (N, W, W, b, k))
        else:   # block products as a batched GEMM: one batch item per block
            out.append("gemm nt %d %d %d %d %d" % (N, b, b, W, b))
        if b in (128, 256) and W % 8 == 0:
            out.append("gram %d %d %d %d" % (N, W, b, k))
    # merge: the P side on W0p's rows, the R side as a batched NN product per row block
    if kP and b <= 256 and n % 8 == 0:
        out.append("bdiag %d %d %d %d %d" % (m, n, n, b, kP))
    if kR and n % 8 == 0:
        out.append("gemm nn %d %d %d %d %d" % (b, n, b, b, n))
    return out


def test_buffer_ranges_stay_inside_operands(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "ranges_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", os.path.join(HERE, "ranges_check.cpp"), "-o", exe], check=True)
    lines = [l for s in SHAPES for l in launches(*s)]
    p = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True)
    assert p.returncode == 0 and p.stdout.startswith("ok"), p.stdout + p.stderr
    assert int(p.stdout.split()[1]) == len(lines)


def test_range_check_catches_a_whole_row_range(tmp_path):
    """The check fails a range that covers whole rows of a strided operand
    (the last row's range would run lda - K elements past the operand)."""
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = open(os.path.join(HERE, "ranges_check.cpp")).read()
    # plant the old whole-row formula in a copy of the header the check includes
    hdr = open(os.path.join(HERE, "..", "orthogonal_reparameterized_poetx_amd", "csrc", "ranges.h")).read()
    old = "  return tile_range(m0, (M - m0 < GEMM_TILE ? M - m0 : GEMM_TILE), 0, K, lda, 2);"
    assert old in hdr
    bad = hdr.replace(old, "  const int64_t rows = M - m0 < GEMM_TILE ? M - m0 : GEMM_TILE;\n"
                           "  return BufRange{m0 * lda, rows * lda * 2};")
    d = tmp_path / "orthogonal_reparameterized_poetx_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "ranges.h").write_text(bad)
    (tmp_path / "t").mkdir()
    (tmp_path / "t" / "ranges_check.cpp").write_text(src)
    exe = str(tmp_path / "bad_check")
    subprocess.run([cxx, "-std=c++17", "-O2", str(tmp_path / "t" / "ranges_check.cpp"), "-o", exe], check=True)
    # batched block products: A is a [N][W] activation read b columns at a time
    p = subprocess.run([exe], input="gemm nt 70 512 512 1104 512\n", capture_output=True, text=True)
    assert p.returncode == 1 and "FAIL gemm A" in p.stdout
