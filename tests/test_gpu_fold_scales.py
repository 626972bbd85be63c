"""Per-chunk scales folded inside the server pass and the update (shapes
whose rows hold at most 64 partials, and n times that at most 1024) against
the separate finalize dispatches that OB_DEBUG_SEPARATE_SCALES forces.

Twin handles take the same gradients; after every step every field is
bit-identical: x, m, v, the worker and server errors, sign words and scales.
The shapes put 1, a ragged count and exactly 64 partials in a row, and cover
every server form (run-time count, 1/2/4 workers, 8-worker tables, segment
partials at 32 and 64 workers), both gradient types and the 0/1 Adam steps.
The launch counts show which form ran: none of the finalize kernels when
folded, one each per step otherwise (also just past the shape limit).
Parity of the folded form with the CPU oracle is covered by the parity
tests, whose small shapes take it."""
import pytest

import synth
from gpu_common import log

pytestmark = pytest.mark.gpu

ob = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global ob
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from communication_compressed_distributed_02_amd import ob_adam
    ob = ob_adam


CASES = [
    # (name, L, n, bf16, folds)
    ("n1_64_quads", 256 * 1024, 1, False, True),
    ("n4_c1_shape", 256 * 1024, 4, False, True),
    ("n4_65_quads", 257 * 1024, 4, False, False),
    ("n3_ragged", 37 * 1024 + 448, 3, False, True),
    ("n2_bf16_one_quad", 3 * 1024 + 64, 2, True, True),
    ("n5_generic", 20 * 1024 + 192, 5, False, True),
    ("n8_bf16", 64 * 1024 + 320, 8, True, True),
    ("n16_at_limit", 256 * 1024, 16, False, True),
    ("n32_segment_partials", 32 * 1024, 32, False, True),
    ("n32_past_limit", 33 * 1024, 32, False, False),
    ("n64_segment_partials", 15 * 1024 + 576, 64, True, True),
]


def grads(d, n, t, bf16):
    import torch
    out = []
    for w in range(n):
        g = torch.empty(d, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
        synth.fill_gpu(g, 0, t, w, sigma=1e-3 if bf16 else 1e-2)
        out.append(g)
    return out


def same_state(a, b, n, where):
    import torch
    fields = [(ob.OB_X, 0), (ob.OB_M, 0), (ob.OB_V, 0), (ob.OB_E_SERVER, 0),
              (ob.OB_BITS_SERVER, 0), (ob.OB_SCALE_SERVER, 0)]
    fields += [(f, w) for w in range(n)
               for f in (ob.OB_E_WORKER, ob.OB_BITS_WORKER, ob.OB_SCALE_WORKER)]
    for f, w in fields:
        assert torch.equal(a.get(f, w), b.get(f, w)), "%s: field %d worker %d differs" % (
            where, f, w)


def twins(d, n, bf16, method):
    gt = ob.OB_GRAD_BF16 if bf16 else ob.OB_GRAD_F32
    a = ob.OneBitAdam(d, n, gt, method=method)
    b = ob.OneBitAdam(d, n, gt, method=method)
    ob.ob_adam_set_debug(b.h, ob.OB_DEBUG_SEPARATE_SCALES)
    return a, b


def finalize_launches(opt):
    kt, _ = ob.ob_adam_kernel_times(opt.h)
    return kt["worker_scale"][1], kt["server_scale"][1]


@pytest.mark.parametrize("name,L,n,bf16,folds", CASES, ids=[c[0] for c in CASES])
def test_folded_scales_equal_separate_finalize(name, L, n, bf16, folds):
    import torch
    d = L * n
    log("case %s: d=%d n=%d bf16=%s folds=%s" % (name, d, n, bf16, folds))
    a, b = twins(d, n, bf16, ob.OB_METHOD_ONE_BIT)
    warm, comp = 2, 4
    for opt in (a, b):
        ob.ob_adam_set_timing(opt.h, 8 * comp + 8)
    for t in range(warm + comp):
        g = grads(d, n, t, bf16)
        lr = 1e-3 * (1 + t % 3)
        for opt in (a, b):
            (opt.warmup_step if t < warm else opt.compressed_step)(g, lr)
        torch.cuda.synchronize()
        if t >= warm:
            same_state(a, b, n, "%s step %d" % (name, t))
    assert finalize_launches(a) == ((0, 0) if folds else (comp, comp))
    assert finalize_launches(b) == (comp, comp)
    for opt in (a, b):
        ob.ob_adam_set_timing(opt.h, 0)
        assert opt.check_guards() == -1


@pytest.mark.parametrize("L,n,bf16", [(256 * 1024, 4, False), (37 * 1024 + 448, 3, False),
                                      (64 * 1024, 8, True), (15 * 1024 + 576, 64, False)])
def test_folded_scales_zero_one(L, n, bf16):
    """0/1 Adam: local steps, synchronizations and refreshes; the
    synchronizing steps take the folded form."""
    import torch
    d = L * n
    log("0/1 d=%d n=%d bf16=%s" % (d, n, bf16))
    a, b = twins(d, n, bf16, ob.OB_METHOD_ZERO_ONE)
    plan = [(False, False), (True, True), (False, False), (False, False), (True, False),
            (True, True)]
    for t in range(1 + len(plan)):
        g = grads(d, n, t, bf16)
        lr = 1e-3 * (1 + t % 3)
        for opt in (a, b):
            if t == 0:
                opt.warmup_step(g, lr)
            else:
                sync, refresh = plan[t - 1]
                opt.zero_one_step(g, lr, sync=sync, refresh=refresh)
        torch.cuda.synchronize()
        if t > 0 and plan[t - 1][0]:
            same_state(a, b, n, "0/1 step %d" % t)


def test_graph_replays_folded_step():
    """A folded compressed step (c1's shape) captured in a HIP graph and
    replayed with new gradients each time equals the same steps run eagerly
    with separate finalizes."""
    import torch
    L, n = 256 * 1024, 4
    d = L * n
    side = torch.cuda.Stream()
    a = ob.OneBitAdam(d, n, stream=side)
    b = ob.OneBitAdam(d, n)
    ob.ob_adam_set_debug(b.h, ob.OB_DEBUG_SEPARATE_SCALES)
    for t in range(2):  # warm-up, and the first compressed step (fp32 momentum)
        g = grads(d, n, t, False)
        torch.cuda.synchronize()
        for opt in (a, b):
            (opt.warmup_step if t == 0 else opt.compressed_step)(g, 1e-3)
    static = [torch.empty_like(x) for x in g]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        a.compressed_step(static, 1e-3)
    torch.cuda.synchronize()
    for t in range(2, 6):
        g = grads(d, n, t, False)
        for s, x in zip(static, g):
            s.copy_(x)
        torch.cuda.synchronize()
        graph.replay()
        b.compressed_step(g, 1e-3)
        torch.cuda.synchronize()
        same_state(a, b, n, "graph replay %d" % t)
