"""Parity at the full sizes of the four large workloads (and of idx64, whose
element indices run past 2^31), in the launch configuration bench.py times,
against values the CPU oracle stored (tests/golden/<workload>/chunk_<j>.json
and .npz, written by make_golden.py from the oracle and the seeded input
generator only).

For every sampled chunk:
 - at every compressed step: the n worker scales and the server scale
   bit-exact, and xxh64 digests of all workers' sign words and of the
   server's sign words over the chunk equal;
 - after the warm-up: x, m, v at 4096 sampled elements (the chunk's first and
   last segments and 2048 more) within 1e-5 relative / 1e-6 absolute;
 - after the middle compressed step and after the last one: xxh64 digests of
   the whole chunk's x, m, v, server error and every worker's error equal
   (the kernels reproduce the oracle's fp32 arithmetic exactly), and the
   sampled values of those fields (the errors of the first and the last
   worker) within the same tolerance;
 - the step counter equal.
The BERT-Large and GPT-2-XL workloads run a second time through the
torch.optim front end (optim.OneBitAdamOptimizer over their 390 and 580
tensors, gradients written tensor by tensor), against the same values.
The 0/1 Adam workloads (z2, z3) run their schedule of local and
synchronizing steps: the per-step checks above at every synchronization,
digests of every worker's local and mean momenta over the chunk at every
local step, and the mid checkpoint (inside a local period) also compares
every worker's local model."""
import glob
import json
import os

import numpy as np
import pytest
import xxhash

from gpu_common import log, within_tol

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden(name):
    recs = []
    for f in sorted(glob.glob(os.path.join(HERE, "golden", name, "chunk_*.json"))):
        with open(f) as fh:
            rec = json.load(fh)
        npz = f[:-len(".json")] + ".npz"
        rec["arrays"] = None
        if os.path.exists(npz):
            with np.load(npz) as z:  # allow_pickle stays off
                rec["arrays"] = {k: z[k] for k in z.files}
        recs.append(rec)
    return recs


def f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def check_sampled(what, got, want_bits):
    want = f32(want_bits)
    ok = within_tol(got, want)
    if not ok.all():
        i = int(np.flatnonzero(~ok)[0])
        raise AssertionError("%s: %d of %d sampled values outside tolerance (first: %r vs %r)"
                             % (what, int((~ok).sum()), ok.size, got[i], want[i]))


def tensor_sizes(name):
    from synth import workloads as W
    return {"c3": W.bert_large_sizes, "c4": W.gpt2_xl_sizes}[name]()


class FrontEnd:
    """The workload stepped through the torch.optim front end: one zero fp32
    parameter per tensor of the architecture, each worker's gradients written
    tensor by tensor at the tensor's flat offset, optimizer.step() per step
    with the workload's learning rate."""

    def __init__(self, w, dev):
        import torch

        from communication_compressed_distributed_02_amd.optim import OneBitAdamOptimizer
        sizes = tensor_sizes(w.name)
        self.w = w
        self.params = [torch.nn.Parameter(torch.zeros(k, device=dev)) for k in sizes]
        self.opt = OneBitAdamOptimizer(self.params, w.n, lr=float(w.lr),
                                       betas=(w.beta1, w.beta2), eps=w.eps,
                                       warmup_steps=w.warmup,
                                       lr_schedule=lambda t: w.lr_at(t))
        self.core = self.opt.core

    def step(self, t):
        import synth
        for i in range(self.w.n):
            for g, off in zip(self.opt.worker_grads(i), self.opt.offsets):
                synth.fill_gpu(g.view(-1), off, t, i, self.w.dist, self.w.sigma)
        self.opt.step()


@pytest.mark.parametrize("name,front_end", [("c2", False), ("c3", False), ("c4", False),
                                            ("c5", False), ("idx64", False),
                                            ("c3", True), ("c4", True),
                                            ("z2", False), ("z3", False)],
                         ids=["c2", "c3", "c4", "c5", "idx64", "c3_optim", "c4_optim",
                              "z2_zero_one", "z3_zero_one"])
def test_full_size_against_stored_oracle(name, front_end):
    import torch

    import synth
    from communication_compressed_distributed_02_amd import ob_adam as ob
    from synth import workloads as W

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    recs = load_golden(name)
    if not recs:
        pytest.skip("no stored oracle values for %s" % name)
    if any(r.get("arrays") is None for r in recs):
        pytest.skip("stored oracle values for %s predate the 4096-sample format (no .npz): "
                    "rewrite them with tests/golden/make_golden.py" % name)
    w = W.make(name)
    L, n = w.L, w.n
    wpc = L // 64  # sign words per chunk
    for r in recs:
        assert (r["d"], r["n"], r["L"]) == (w.d, w.n, w.L)
        assert r["arrays"]["loc"].size == r["samples"] >= 4096
        assert r["mid_t"] == recs[0]["mid_t"]
    log("%s%s: d=%d n=%d, chunks %s, %d+%d steps"
        % (name, " (torch.optim front end)" if front_end else "", w.d, n,
           [r["chunk"] for r in recs], w.warmup, w.compressed))
    dev = torch.device("cuda:0")
    gdt = torch.bfloat16 if w.bf16 else torch.float32
    if front_end:
        from communication_compressed_distributed_02_amd.optim import flat_layout
        fe = FrontEnd(w, dev)
        offsets, d = flat_layout(tensor_sizes(name), n)
        assert d == w.d and fe.opt.d == w.d and fe.opt.offsets == offsets
        assert len(fe.params) == w.tensors
        # the gaps between the tensors and the tail are exactly the padding
        # (adjacent padding ranges merged)
        ends = [o + k for o, k in zip(offsets, tensor_sizes(name))]
        gaps = [(e, o) for e, o in zip(ends, offsets[1:] + [d]) if o > e]
        merged = []
        for lo, hi in w.pads:
            if merged and merged[-1][1] == lo:
                merged[-1] = (merged[-1][0], hi)
            else:
                merged.append((lo, hi))
        assert gaps == merged
        opt = fe.core
    else:
        zero_one = w.method == "zero_one"
        opt = ob.OneBitAdam(w.d, n, ob.OB_GRAD_BF16 if w.bf16 else ob.OB_GRAD_F32, w.beta1,
                            w.beta2, w.eps, device=dev,
                            method=ob.OB_METHOD_ZERO_ONE if zero_one else ob.OB_METHOD_ONE_BIT)

    def fill(buf, worker, t):
        synth.fill_gpu(buf, 0, t, worker, w.dist, w.sigma)
        for lo, hi in w.pads:
            buf[lo:hi].zero_()

    def chunk(field, rec, worker=0):
        return opt.get(field, worker, rec["chunk"] * L, L)

    # whole-chunk digests go through one pinned host buffer (a pageable copy
    # plus a bytes copy of every chunk made the 0/1 workloads' per-step
    # digests of every worker's local momenta take minutes)
    pinned = torch.empty(L * 4, dtype=torch.uint8, pin_memory=True)

    def host_view(t):
        nb = t.numel() * t.element_size()
        pinned[:nb].copy_(t.contiguous().view(torch.uint8))
        return memoryview(pinned[:nb].numpy())

    def digest_chunk(field, rec, worker=0, h=None):
        h = h if h is not None else xxhash.xxh64()
        h.update(host_view(chunk(field, rec, worker)))
        return h

    def sampled(field, rec, worker=0):
        loc = torch.as_tensor(rec["arrays"]["loc"].astype(np.int64), device=dev)
        return chunk(field, rec, worker).index_select(0, loc).cpu().numpy()

    def check_checkpoint(tag, t):
        """Whole-chunk digests bit-exact, samples within tolerance."""
        for rec in recs:
            j, arr, dig = rec["chunk"], rec["arrays"], rec[tag + "_digest"]
            for key, field in (("x", ob.OB_X), ("m", ob.OB_M), ("v", ob.OB_V),
                               ("es", ob.OB_E_SERVER)):
                check_sampled("%s chunk %d %s step %d: %s" % (name, j, tag, t, key),
                              sampled(field, rec), arr["%s_%s" % (tag, key)])
                got = digest_chunk(field, rec).hexdigest()
                assert got == dig[key], "%s chunk %d %s step %d: %s digest" % (name, j, tag, t, key)
            for k, i in enumerate(rec["error_workers"]):
                check_sampled("%s chunk %d %s step %d: e_w%d" % (name, j, tag, t, i),
                              sampled(ob.OB_E_WORKER, rec, i), arr["%s_e" % tag][k])
            for i in range(n):
                got = digest_chunk(ob.OB_E_WORKER, rec, i)
                assert got.hexdigest() == dig["e"][i], \
                    "%s chunk %d %s step %d: e_w%d digest" % (name, j, tag, t, i)
            for i, want in enumerate(dig.get("xl", [])):  # inside a 0/1 local period
                got = digest_chunk(ob.OB_X_LOCAL, rec, i)
                assert got.hexdigest() == want, \
                    "%s chunk %d %s step %d: local model of worker %d" % (name, j, tag, t, i)
        log("%s: %s checkpoint (step %d) matches: whole-chunk digests and samples"
            % (name, tag, t))

    # a staged workload regenerates each worker's gradient into one buffer, in
    # the warm-up as in the compression phase
    if w.staged:
        one = torch.empty(w.d, dtype=gdt, device=dev)
    elif not front_end:
        full = torch.empty((n, w.d), dtype=gdt, device=dev)
    for t in range(w.warmup):
        if front_end:
            fe.step(t)
        elif w.staged:
            for i in range(n):
                fill(one, i, t)
                opt.warmup_worker(i, one)
            opt.warmup_finish(w.lr_at(t))
        else:
            for i in range(n):
                fill(full[i], i, t)
            opt.warmup_step(list(full.unbind(0)), w.lr_at(t))
    torch.cuda.synchronize()
    for rec in recs:
        for key, field in (("x", ob.OB_X), ("m", ob.OB_M), ("v", ob.OB_V)):
            check_sampled("%s chunk %d after warm-up: %s" % (name, rec["chunk"], key),
                          sampled(field, rec), rec["arrays"]["aw_" + key])

    for si, t in enumerate(range(w.warmup, w.steps)):
        lr = w.lr_at(t)
        sync = True
        if front_end:
            assert fe.opt.compressing
            fe.step(t)
        elif w.method == "zero_one":
            for i in range(n):
                fill(full[i], i, t)
            sync, refresh = w.zo_flags(t)
            opt.zero_one_step(list(full.unbind(0)), lr, sync, refresh)
        elif w.staged:
            for i in range(n):
                fill(one, i, t)
                opt.compress_worker(i, one)
            opt.compressed_finish(lr)
        else:
            for i in range(n):
                fill(full[i], i, t)
            opt.compressed_step(list(full.unbind(0)), lr)
        if not sync:  # a 0/1 local step: every worker's momenta over the chunk
            for rec in recs:
                j, want = rec["chunk"], rec["steps"][si]
                assert want["t"] == t and want["sync"] is False
                for key, field in (("mh", ob.OB_M_LOCAL), ("ah", ob.OB_A_LOCAL)):
                    h = xxhash.xxh64()
                    for i in range(n):
                        digest_chunk(field, rec, i, h)
                    assert h.hexdigest() == want[key], "%s step %d chunk %d %s" % (name, t, j, key)
            log("%s step %d/%d (local) ok" % (name, t + 1, w.steps))
            if t == recs[0]["mid_t"]:
                check_checkpoint("mid", t)
            continue
        ws = np.stack([opt.get(ob.OB_SCALE_WORKER, i).cpu().numpy() for i in range(n)])
        ss = opt.get(ob.OB_SCALE_SERVER).cpu().numpy()
        for rec in recs:
            j = rec["chunk"]
            want = rec["steps"][si]
            assert want["t"] == t
            assert want["lr_bits"] == int(np.float32(lr).view(np.uint32))
            got_ws = ws[:, j].view(np.uint32).tolist()
            assert got_ws == want["ws"], "%s step %d chunk %d worker scales" % (name, t, j)
            assert int(ss[j:j + 1].view(np.uint32)[0]) == want["ss"], \
                "%s step %d chunk %d server scale" % (name, t, j)
            h = xxhash.xxh64()
            for i in range(n):
                h.update(opt.get(ob.OB_BITS_WORKER, i, j * wpc, wpc).cpu().numpy().tobytes())
            assert h.hexdigest() == want["wh"], "%s step %d chunk %d worker sign words" % (name, t, j)
            sh = xxhash.xxh64(opt.get(ob.OB_BITS_SERVER, 0, j * wpc, wpc).cpu().numpy().tobytes())
            assert sh.hexdigest() == want["sh"], "%s step %d chunk %d server sign words" % (name, t, j)
        log("%s step %d/%d ok" % (name, t + 1, w.steps))
        if t == recs[0]["mid_t"]:
            check_checkpoint("mid", t)

    check_checkpoint("fin", w.steps - 1)
    for rec in recs:
        assert opt.steps[0] == rec["t"]
    if front_end:  # the parameters are views of the library's x
        x = fe.opt.flat_params()
        for p, off in zip(fe.params[:: max(1, len(fe.params) // 16)], fe.opt.offsets[:: max(
                1, len(fe.params) // 16)]):
            assert torch.equal(p.detach(), x[off:off + p.numel()])
    assert opt.check_guards() == -1, "a kernel wrote past the end of a workspace buffer"
    log("%s: %d chunks match the oracle at every step" % (name, len(recs)))
