"""q4_gemv_chain: a list of M = 1 GEMVs in one persistent launch.

The chain must give, bit for bit, what consecutive q4_gemv calls give on the
same inputs (same kernels' arithmetic: x in registers for rows of one stage,
staged in LDS for longer rows).  Covered: every format, group size and
activation dtype; ragged K (a partial last stage), K of several stages up to
the largest supported, tasks with fewer rows than the grid has waves (most
waves skip them), a task whose x is an earlier task's y (the grid-wide wait),
the Q4_TASK_NO_WAIT flag, the longest chain, and reuse of the sync buffer
(the kernel leaves its counters at zero and sets no timeout flag), and
chains of dependent tasks rerun into the same buffers.  One chain
is also checked against the fp64 oracle within the product tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_group_wise_amd import q4, synth
from _helpers import DEV, TORCH_ACT, assert_product_ok, dev16

pytestmark = pytest.mark.gpu

GROUPS = {q4.NF4: [32, 64, 128], q4.INT4_SYM: [32, 64, 128], q4.INT4_ASYM: [32, 64, 128],
          q4.NF4_DQ: [32, 64, 128], q4.FP4: [32, 64, 128]}


def _weight(N, K, fmt, g, seed, sigma=0.02):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    w = torch.empty((N, K), dtype=torch.float16, device=DEV).normal_(0.001, sigma, generator=gen)
    return q4.quantize(w, fmt, g)


def _x(K, act, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    return torch.randn((1, K), generator=gen, device=DEV).to(TORCH_ACT[act])


# (N, K) of independent tasks: one stage, ragged one stage, two stages, few
# rows, the largest K, a single row
SHAPES = [(4096, 4096), (2051, 2176), (5000, 8192), (37, 1024), (3, 16384), (1, 11008)]


def _build_chain(fmt, g, act, seed):
    """Tasks and the sequential reference: independent shapes, then a task
    reading the y of the first task as its x (N0 = 4096 -> K = 4096)."""
    tasks, ref = [], []
    for i, (N, K) in enumerate(SHAPES):
        q = _weight(N, K, fmt, g, seed + i)
        x = _x(K, act, seed + 100 + i)
        y = torch.full((1, N), 7.0, dtype=TORCH_ACT[act], device=DEV)
        tasks.append([x, q, y])
        ref.append(q4.gemv(x, q))
    # dependent task: x is task 0's output buffer (pre-filled with 7.0, so a
    # read before task 0 wrote it gives a different result)
    qd = _weight(640, 4096, fmt, g, seed + 50)
    yd = torch.empty((1, 640), dtype=TORCH_ACT[act], device=DEV)
    tasks.append([tasks[0][2], qd, yd])
    ref.append(q4.gemv(ref[0], qd))
    # and one more after it that reads the dependent task's output (K = 640)
    qe = _weight(96, 640, fmt, g, seed + 51)
    ye = torch.empty((1, 96), dtype=TORCH_ACT[act], device=DEV)
    tasks.append([yd, qe, ye])
    ref.append(q4.gemv(ref[-1], qe))
    return tasks, ref


def _assert_same(outs, ref, tag):
    for i, (a, b) in enumerate(zip(outs, ref)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (
            f"{tag} task {i}: {int((a != b).sum())} outputs differ from q4_gemv")


@pytest.mark.parametrize("act", [q4.BF16, q4.F16])
@pytest.mark.parametrize("fmt", [q4.NF4, q4.INT4_SYM, q4.INT4_ASYM, q4.NF4_DQ, q4.FP4])
def test_chain_equals_consecutive_gemv(fmt, act):
    for g in GROUPS[fmt]:
        tag = f"fmt{fmt} g{g} act{act}"
        print(tag, flush=True)
        tasks, ref = _build_chain(fmt, g, act, seed=1000 * fmt + g + act)
        sync = q4.chain_sync(DEV)
        for rep in range(2):                      # the sync buffer is reused
            for t in tasks[:6]:
                t[2].fill_(7.0)
            outs = q4.gemv_chain([tuple(t) for t in tasks], sync=sync)
            torch.cuda.synchronize()
            _assert_same(outs, ref, f"{tag} rep{rep}")
            assert not sync.any().item(), f"{tag}: sync words not clear"


def test_chain_no_wait_flag():
    """Independent tasks flagged Q4_TASK_NO_WAIT give the same bits."""
    fmt, g, act = q4.NF4, 64, q4.BF16
    tasks, ref = _build_chain(fmt, g, act, seed=77)
    flagged = [(x, q, y, q4.TASK_NO_WAIT if i < len(SHAPES) else 0)
               for i, (x, q, y) in enumerate(tasks)]
    # the dependent tasks keep the wait
    outs = q4.gemv_chain(flagged)
    torch.cuda.synchronize()
    _assert_same(outs, ref, "no-wait")


# (N, K) of a long run of independent tasks: x slots reused many times over,
# runs of four-stage tasks (each slot set freed only by the task before),
# one-stage tasks (several in flight at once), three-stage tasks that wrap
# the slots, and tasks of a few rows that most waves only pass through
SLOT_SHAPES = ([(700, 16384)] * 3 + [(1500, 4096)] * 10 + [(257, 11008), (1, 1024), (3000, 11008),
               (900, 8192), (64, 16384), (2051, 2176), (5, 4096)] + [(333, 2176)] * 6)


@pytest.mark.parametrize("fmt,g,act", [(q4.NF4, 64, q4.BF16), (q4.INT4_SYM, 128, q4.F16),
                                       (q4.NF4_DQ, 32, q4.BF16)])
def test_chain_slot_reuse(fmt, g, act):
    """Independent tasks of mixed stage counts (their x prefetched into the
    LDS slots while earlier tasks run), with a task reading an earlier
    output in the middle, give the bits of consecutive GEMVs."""
    tasks, ref = [], []
    for i, (N, K) in enumerate(SLOT_SHAPES):
        q = _weight(N, K, fmt, g, 7000 + 17 * i)
        x = _x(K, act, 7100 + i)
        y = torch.full((1, N), 7.0, dtype=TORCH_ACT[act], device=DEV)
        tasks.append((x, q, y, q4.TASK_NO_WAIT))
        ref.append(q4.gemv(x, q))
    # after the tenth task: one reading the first one-stage task's output
    # (N = 1500 -> K = 1500 is not a whole number of groups; 1024 of it is)
    src = tasks[3][2][:, :1024]
    qd = _weight(400, 1024, fmt, g, 7999)
    yd = torch.empty((1, 400), dtype=TORCH_ACT[act], device=DEV)
    tasks.insert(10, (src, qd, yd, 0))
    ref.insert(10, q4.gemv(ref[3][:, :1024].contiguous(), qd))
    sync = q4.chain_sync(DEV)
    for rep in range(2):
        for t in tasks:
            t[2].fill_(7.0)
        outs = q4.gemv_chain(tasks, sync=sync)
        torch.cuda.synchronize()
        _assert_same(outs, ref, f"slots fmt{fmt} g{g} rep{rep}")
        assert not sync.any().item()


@pytest.mark.parametrize("fmt,g,act", [(q4.NF4, 64, q4.BF16), (q4.INT4_ASYM, 32, q4.F16),
                                       (q4.NF4_DQ, 64, q4.BF16)])
def test_chain_blocked_rows(fmt, g, act):
    """A chain with no waiting task deals each workgroup a contiguous block
    of the tasks' rows (balanced by stage count): the blocks cross task
    boundaries, rows of one to four stages mix, and in the small chains most
    workgroups get no rows at all.  Outputs equal consecutive GEMVs."""
    chains = [SLOT_SHAPES, [(1, 1024), (3, 16384), (5, 2176), (2, 11008), (1, 64 if g <= 64 else 128)],
              [(7, 4096)], [(40000, 4096)]]
    sync = q4.chain_sync(DEV)
    for ci, shapes in enumerate(chains):
        tasks, ref = [], []
        for i, (N, K) in enumerate(shapes):
            q = _weight(N, K, fmt, g, 8000 + 31 * ci + i)
            x = _x(K, act, 8100 + 31 * ci + i)
            y = torch.full((1, N), 7.0, dtype=TORCH_ACT[act], device=DEV)
            tasks.append((x, q, y, q4.TASK_NO_WAIT))
            ref.append(q4.gemv(x, q))
        for rep in range(2):
            for t in tasks:
                t[2].fill_(7.0)
            outs = q4.gemv_chain(tasks, sync=sync)
            torch.cuda.synchronize()
            _assert_same(outs, ref, f"blocked chain {ci} fmt{fmt} g{g} rep{rep}")
            assert not sync.any().item()


def test_chain_longest():
    """Q4_GEMV_CHAIN_MAX tasks, each reading the previous task's y."""
    fmt, g, act = q4.INT4_ASYM, 32, q4.F16
    K = 512
    # sigma = 1/sqrt(K) keeps |y| near |x| along the chain
    qs = [_weight(K, K, fmt, g, 9000 + i, sigma=K ** -0.5) for i in range(q4.CHAIN_MAX)]
    x0 = _x(K, act, 4242)
    ys = [torch.empty((1, K), dtype=torch.float16, device=DEV) for _ in qs]
    tasks = [(x0 if i == 0 else ys[i - 1], q, ys[i]) for i, q in enumerate(qs)]
    outs = q4.gemv_chain(tasks)
    ref, x = [], x0
    for q in qs:
        x = q4.gemv(x, q)
        ref.append(x)
    torch.cuda.synchronize()
    _assert_same(outs, ref, "longest")
    assert torch.isfinite(outs[-1].float()).all()


@pytest.mark.parametrize("fmt,g,act", [(q4.NF4, 64, q4.BF16), (q4.INT4_ASYM, 32, q4.F16)])
def test_chain_dependent_reuse(fmt, g, act):
    """Tasks that each read the previous task's output, run again and again
    into the same output buffers with a new first input each time: a read
    of an output before it was written (a copy left from the previous run,
    held in some XCD's L2 by a kernel that read the buffers in between)
    would give the previous run's bits."""
    dims = [4096, 4096, 11008, 4096, 2176, 4096]
    qs = [_weight(n, k, fmt, g, 9500 + i, sigma=k ** -0.5) for i, (k, n) in
          enumerate(zip(dims[:-1], dims[1:]))]
    ys = [torch.empty((1, q.N), dtype=TORCH_ACT[act], device=DEV) for q in qs]
    sync = q4.chain_sync(DEV)
    for rep in range(4):
        x0 = _x(dims[0], act, 9600 + rep)
        tasks = [(x0 if i == 0 else ys[i - 1], q, ys[i]) for i, q in enumerate(qs)]
        # pull the previous run's outputs into the L2s of the XCDs that run
        # a reduction over them
        _ = [float(y.float().sum()) for y in ys]
        outs = q4.gemv_chain(tasks, sync=sync)
        ref, x = [], x0
        for q in qs:
            x = q4.gemv(x, q)
            ref.append(x)
        torch.cuda.synchronize()
        _assert_same(outs, ref, f"dependent reuse fmt{fmt} rep{rep}")
        assert not sync.any().item()


def test_chain_against_oracle():
    """A chain's outputs within the product tolerance of the fp64 oracle."""
    for fmt, g, act in [(q4.NF4, 64, q4.BF16), (q4.INT4_ASYM, 32, q4.F16), (q4.NF4_DQ, 32, q4.BF16)]:
        shapes = [(300, 4096), (64, 8192), (5, 2176)]
        tasks, refs = [], []
        for i, (N, K) in enumerate(shapes):
            w = synth.weight_f16_bits(N, K, 31 + i)
            oc, os_, oz = oracle.quantize(fmt, g, w)
            q = q4.quantize(dev16(w), fmt, g)
            xb = synth.act_bits(1, K, 61 + i, act)
            tasks.append((dev16(xb, act), q, None))
            refs.append(oracle.matmul(fmt, g, act, xb, oc, os_, oz, N, K))
        outs = q4.gemv_chain(tasks)
        torch.cuda.synchronize()
        for i, (y, (yr, ad)) in enumerate(zip(outs, refs)):
            assert_product_ok(y, yr, ad, tag=f"chain fmt{fmt} task {i}")
