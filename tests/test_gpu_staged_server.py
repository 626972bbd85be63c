"""The server pass for 8, 16, 32 and 64 workers with each segment's sign
words staged in LDS (chunks of an even number of rows) against the same pass
loading them straight into registers (OB_DEBUG_UNSTAGED_SERVER).

Twin handles take the same gradients; after every compressed step every
field is bit-identical: x, m, v, the worker and server errors, sign words
and scales.  The shapes give full segments and ragged chunk ends of 2, 4, 8
and 14 rows, both gradient types, the in-pass and the separate scale
finalize, and a 0/1 Adam schedule.  Parity of the staged form with the CPU
oracle is covered by the parity tests (the *_staged_* shapes) and by the
full-size stored oracle values, whose workloads all have an even number of
rows per chunk."""
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
    # (name, L, n, bf16, separate scales)
    ("n8_ragged_14_rows", 64 * 1024 + 896, 8, True, False),
    ("n16_full_segments", 48 * 1024, 16, False, False),
    ("n16_ragged_2_rows", 48 * 1024 + 128, 16, False, True),
    ("n32_ragged_8_rows", 40 * 1024 + 512, 32, True, False),
    ("n64_ragged_4_rows", 15 * 1024 + 256, 64, False, False),
    ("n64_ragged_separate_scales", 80 * 1024 + 256, 64, True, True),
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


@pytest.mark.parametrize("name,L,n,bf16,separate", CASES, ids=[c[0] for c in CASES])
def test_staged_server_equals_unstaged(name, L, n, bf16, separate):
    import torch
    assert (L // 64) % 2 == 0
    d = L * n
    log("case %s: d=%d n=%d bf16=%s separate scales=%s" % (name, d, n, bf16, separate))
    gt = ob.OB_GRAD_BF16 if bf16 else ob.OB_GRAD_F32
    a = ob.OneBitAdam(d, n, gt)
    b = ob.OneBitAdam(d, n, gt)
    extra = ob.OB_DEBUG_SEPARATE_SCALES if separate else 0
    ob.ob_adam_set_debug(a.h, extra)
    ob.ob_adam_set_debug(b.h, extra | ob.OB_DEBUG_UNSTAGED_SERVER)
    warm, comp = 1, 4
    for t in range(warm + comp):
        g = grads(d, n, t, bf16)
        lr = 1e-3 * (1 + t % 3)
        for opt in (a, b):
            (opt.warmup_step if t < warm else opt.compressed_step)(g, lr)
        torch.cuda.synchronize()
        if t >= warm:
            same_state(a, b, n, "%s step %d" % (name, t))
    for opt in (a, b):
        assert opt.check_guards() == -1


def test_staged_server_zero_one():
    import torch
    L, n, bf16 = 24 * 1024 + 384, 16, False
    d = L * n
    a = ob.OneBitAdam(d, n, ob.OB_GRAD_F32, method=ob.OB_METHOD_ZERO_ONE)
    b = ob.OneBitAdam(d, n, ob.OB_GRAD_F32, method=ob.OB_METHOD_ZERO_ONE)
    ob.ob_adam_set_debug(b.h, ob.OB_DEBUG_UNSTAGED_SERVER)
    # warm-up, then local steps with a synchronization every second step and
    # a variance refresh at the second synchronization
    sched = [None, (False, False), (True, False), (False, False), (True, True), (True, False)]
    for t, flags in enumerate(sched):
        g = grads(d, n, t, bf16)
        for opt in (a, b):
            if flags is None:
                opt.warmup_step(g, 1e-3)
            else:
                opt.zero_one_step(g, 1e-3, *flags)
        torch.cuda.synchronize()
        if flags is not None and flags[0]:
            same_state(a, b, n, "0/1 step %d" % t)
    for opt in (a, b):
        assert opt.check_guards() == -1
