"""q4_gemv_chain_static: the chained GEMV with the library's static sync
words, for callers that cannot allocate.  Its outputs must equal
q4_gemv_chain's bit for bit (same kernels), on two calls in a row, the
second with a smaller chain; the second call reuses the static words the
first left behind.  The chains include tasks that wait for earlier outputs,
so the static grid-barrier counters are exercised."""

import pytest
import torch

from bit_group_wise_amd import q4
from _helpers import DEV, TORCH_ACT

pytestmark = pytest.mark.gpu


def _weight(N, K, fmt, g, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    w = torch.empty((N, K), dtype=torch.float16, device=DEV).normal_(0.0, 0.02, generator=gen)
    return q4.quantize(w, fmt, g)


def _chain(shapes, fmt, g, act, seed):
    """Tasks of the given (N, K); a task whose K equals the previous task's
    N reads that task's output (a waiting task)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    tasks = []
    for i, (N, K) in enumerate(shapes):
        q = _weight(N, K, fmt, g, seed + i)
        if i > 0 and shapes[i - 1][0] == K:
            tasks.append((None, q, 0))          # x = the previous output
        else:
            x = torch.randn((1, K), generator=gen, device=DEV).to(TORCH_ACT[act])
            tasks.append((x, q, q4.TASK_NO_WAIT))
    return tasks


def _run(fn, tasks, act):
    """Run the chain with fresh outputs (x of a waiting task is the previous
    task's output buffer)."""
    spec, outs = [], []
    for x, q, flags in tasks:
        y = torch.full((1, q.N), 3.0, dtype=TORCH_ACT[act], device=DEV)
        spec.append((outs[-1] if x is None else x, q, y, flags))
        outs.append(y)
    fn(spec)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("fmt,g,act", [(q4.NF4, 64, q4.BF16), (q4.INT4_ASYM, 32, q4.F16),
                                       (q4.NF4_DQ, 64, q4.BF16)])
def test_static_chain_equals_chain(fmt, g, act):
    big = _chain([(4096, 4096), (2048, 4096), (1024, 2048), (512, 11008), (4096, 512),
                  (96, 4096)], fmt, g, act, seed=10)
    small = _chain([(256, 1024), (64, 256)], fmt, g, act, seed=20)
    for tasks in (big, small):
        want = _run(q4.gemv_chain, tasks, act)
        got = _run(q4.gemv_chain_static, tasks, act)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"task {i} differs"
