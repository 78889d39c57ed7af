"""GPU parity on the edge inputs of tests/edge_inputs.py: every kernel that
q4k_gemv can choose, forced through q4k_gemv_ex, against the oracle under the
rule of tests/checks.py (the per-output bound 1e-5 * sum|w||x| for every
finite exact result, NaN and infinities where the exact result has them).

The inputs: x from 2^-149 to 2^127 (tiny, subnormal, huge, y beyond the f32
range), a sub-block whose largest x sits on a zero weight while the rest of
the output comes from values 2^23 times smaller, activation outliers on zero
weights, rows whose weights all cancel exactly (bound 0: y must be 0) or
all but one per sub-block, and inf/NaN in x and in d/dmin.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import checks  # noqa: E402
import edge_inputs  # noqa: E402
from block_quantized_decode_q4_amd import q4k  # noqa: E402

pytestmark = pytest.mark.gpu

# kernels and the vectors one call of each takes
KERNELS = [1, 2, 3, 4, 5, 6, 7]
MAX_M = {1: 8, 2: 1, 3: 1, 4: 2, 5: 16, 6: 16, 7: 16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4k.load_library()
    yield


_cases = edge_inputs.all_cases()


def _run(w_d, x, n, k, kernel):
    m = x.shape[0]
    x_d = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y_d = torch.full((m, n), 12345.0, dtype=torch.float32, device="cuda")
    q4k.q4k_gemv_ex(w_d, x_d, y_d, n, k, m, kernel=kernel)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", _cases, ids=lambda c: c.name)
def test_edge_inputs(oracle_mod, case, kernel):
    print("edge input '%s' n=%d k=%d m=%d kernel %d" % (case.name, case.n, case.k, case.m, kernel),
          flush=True)
    if kernel in (4, 7) and case.k % 2048 != 0:
        pytest.skip("kernels 4 and 7 take rows of whole 8-superblock slabs only (k % 2048 == 0)")
    y_ref, bound = oracle_mod.gemv(case.w, case.x, case.n)
    w_d = torch.from_numpy(case.w).cuda()
    step = MAX_M[kernel]
    y = np.concatenate([_run(w_d, case.x[b:b + step], case.n, case.k, kernel)
                        for b in range(0, case.m, step)])
    checks.assert_y(y, y_ref, bound, "%s, kernel %d" % (case.name, kernel),
                    strict_kind=case.strict_kind)
