"""The closed-form route rows that bsa_decode_routed generates inside its kernel
(route_row_count / route_row_entry in csrc/bsa_internal.hpp), and the closed-form row starts
(route_row_start) that the one-launch route builder writes, checked on the CPU against the
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
    if (argc > 6) {  // row starts: "i: start count" (argv[6] = n_random)
        const int nr = atoi(argv[6]);
        for (long i = i0; i < i1; ++i)
            printf("%ld: %lld %lld\n", i, (long long)bsa::route_row_start(kind, i, L, kf, nr),
                   (long long)bsa::route_row_count(kind, i, L, kf, nr));
        return 0;
    }
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

    def rows(kind, n_local, keep_first, i0, i1, n_random=None):
        extra = [] if n_random is None else [str(n_random)]
        out = subprocess.run([str(exe), str(kind), str(n_local), str(int(keep_first)), str(i0), str(i1), *extra],
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


@pytest.mark.parametrize("kind,params", [
    (R.BF1, dict(n_local=2, keep_first=1)), (R.BF1, dict(n_local=0, keep_first=0)),
    (R.BF1, dict(n_local=0, keep_first=1)), (R.BF1, dict(n_local=1, keep_first=1)),
    (R.BF1, dict(n_local=5, keep_first=1)), (R.BF1, dict(n_local=3, keep_first=0)),
    (R.BF1, dict(n_local=8, keep_first=1)),
    (R.BLOCK_DIAGONAL, {}), (R.DENSE_CAUSAL, {}),
    (R.STATIC_RANDOM, dict(n_random=14, keep_first=1)), (R.STATIC_RANDOM, dict(n_random=5, keep_first=0)),
    (R.STATIC_RANDOM, dict(n_random=0, keep_first=1)), (R.STATIC_RANDOM, dict(n_random=70, keep_first=1)),
    (R.SLIDING_WINDOW, dict(n_local=0)), (R.SLIDING_WINDOW, dict(n_local=8)), (R.SLIDING_WINDOW, dict(n_local=70)),
])
def test_row_starts_equal_the_oracle_row_pointers(rows_exe, kind, params):
    """route_row_start(i) is row_ptr[i] of the oracle's CSR route for every i <= nqb (300 blocks)."""
    nqb = 300
    orp, _ = R.route_csr(kind, nqb * 64, 64, n_local=params.get("n_local", 2),
                         keep_first=bool(params.get("keep_first", 1)), n_random=params.get("n_random", 14), seed=17)
    got = rows_exe(kind, params.get("n_local", 2), params.get("keep_first", 1), 0, nqb + 1,
                   n_random=params.get("n_random", 14))
    assert [got[i][0] for i in range(nqb + 1)] == [int(x) for x in orp], (kind, params)


@pytest.mark.parametrize("i0", [2**20 - 3, 2**30 - 2, 2**31 - 5])
def test_bf1_row_starts_far_out(rows_exe, i0):
    # consecutive starts differ by the oracle's row sizes, and the start itself matches a sum of
    # the oracle's row sizes written out by powers of two (rows 2^k .. 2^(k+1)-1 hold 2 + k entries
    # each, plus block 0 for all but the first)
    got = rows_exe(R.BF1, 2, True, i0, i0 + 4, n_random=0)
    for i in range(i0, i0 + 3):
        assert got[i + 1][0] - got[i][0] == len(R.bf1_set(i, n_local=2, keep_first=True)), i
    i = i0
    want = 1 + 2 + 3  # rows 0, 1, 2
    k = 1
    while 2 ** (k + 1) <= i - 1:  # full power-of-two ranges [2^k, 2^(k+1)) with 2^k >= 2
        lo, hi = 2 ** k, 2 ** (k + 1) - 1
        lo = max(lo, 3)
        want += sum_rows(lo, hi, k)
        k += 1
    want += sum_rows(max(2 ** k, 3), i - 1, k)
    assert got[i][0] == want


def sum_rows(lo, hi, k):
    """Entries of BF1 rows lo .. hi (n_local 2, block 0 kept) when floor(log2 r) = k throughout:
    2 + k entries (self, two local blocks, the dyadic blocks with offset above 2) plus block 0 for
    every r that is not a power of two."""
    if hi < lo:
        return 0
    cnt = hi - lo + 1
    pow2 = 1 if lo == 2 ** k else 0
    return cnt * (2 + k) + (cnt - pow2)
