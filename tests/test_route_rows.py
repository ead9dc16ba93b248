"""The closed-form route rows that bsa_decode_routed generates inside its kernel
(route_row_count / route_row_entry in csrc/bsa_internal.hpp), checked on the CPU against the
oracle's route sets ("BF1 ...", section 3: the BF1 neighbourhood; the block-diagonal, dense and
sliding routes).  The header's functions are host+device; this test builds them for the host
with g++ and prints every row, so a wrong index, a dropped dyadic block or a misplaced block 0
shows here without a GPU.
"""

import os
import shutil
import subprocess

import pytest

from oracle import routes as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_block_amd", "csrc")

PROGRAM = r"""
#include "bsa_internal.hpp"
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
    const int kind = atoi(argv[1]), L = atoi(argv[2]), kf = atoi(argv[3]);
    const long i0 = atol(argv[4]), i1 = atol(argv[5]);
    for (long i = i0; i < i1; ++i) {
        const long c = (long)bsa::route_row_count(kind, i, L, kf, 0);
        printf("%ld:", i);
        for (long x = 0; x < c; ++x) printf(" %ld", (long)bsa::route_row_entry(kind, i, L, kf, x));
        printf("\n");
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def rows_exe(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are not available")
    d = tmp_path_factory.mktemp("rows")
    src, exe = d / "rows.cpp", d / "rows"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, str(src), "-o", str(exe)], check=True)

    def rows(kind, n_local, keep_first, i0, i1):
        out = subprocess.run([str(exe), str(kind), str(n_local), str(int(keep_first)), str(i0), str(i1)],
                             check=True, capture_output=True, text=True).stdout
        got = {}
        for line in out.splitlines():
            head, _, tail = line.partition(":")
            got[int(head)] = [int(x) for x in tail.split()]
        return got
    return rows


def oracle_set(kind, i, n_local, keep_first):
    if kind == R.BF1:
        return R.bf1_set(i, n_local=n_local, keep_first=keep_first)
    if kind == R.BLOCK_DIAGONAL:
        return R.block_diagonal_set(i)
    if kind == R.DENSE_CAUSAL:
        return R.dense_causal_set(i)
    return R.sliding_window_set(i, n_local)


@pytest.mark.parametrize("kind", [R.BF1, R.BLOCK_DIAGONAL, R.DENSE_CAUSAL, R.SLIDING_WINDOW])
@pytest.mark.parametrize("n_local", [0, 1, 2, 3, 5, 8])
@pytest.mark.parametrize("keep_first", [False, True])
def test_rows_equal_the_oracle_sets_in_ascending_order(rows_exe, kind, n_local, keep_first):
    got = rows_exe(kind, n_local, keep_first, 0, 300)
    for i in range(300):
        assert got[i] == sorted(oracle_set(kind, i, n_local, keep_first)), (kind, n_local, keep_first, i)


@pytest.mark.parametrize("i0", [2**20 - 3, 2**30 - 2, 2**31 - 4])
def test_bf1_rows_far_out(rows_exe, i0):
    # large block indices: dyadic offsets up to 2^30, powers of two and their neighbours
    got = rows_exe(R.BF1, 2, True, i0, i0 + 3)
    for i in range(i0, i0 + 3):
        assert got[i] == sorted(R.bf1_set(i, n_local=2, keep_first=True)), i
