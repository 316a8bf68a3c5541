"""bole_forest_build_noalloc (the budget selection for callers that cannot
allocate: its scratch is the library's fixed per-GPU array) against
bole_forest_build (the same kernels on a caller-provided workspace), through
the C ABI: bit-exact rho, packed parent / candidate arrays, offsets and error
bits on two calls in a row, the second with a smaller input, so the second
call runs on the array the first one left behind; and the shape limit is
rejected on the host."""

import sys

import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU hosts
    pytest.skip("no GPU", allow_module_level=True)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(M_total, B, capacity, dev):
    return dict(rho=torch.full((M_total,), 7.0, dtype=torch.float32, device=dev),
                parent=torch.full((capacity,), 99, dtype=torch.int32, device=dev),
                cand_of=torch.full((capacity,), 99, dtype=torch.int32, device=dev),
                tree_off=torch.full((B + 1,), 99, dtype=torch.int32, device=dev),
                err=torch.zeros(1, dtype=torch.int32, device=dev))


def _run(fn, c, capacity, max_tree, dev, workspace=None):
    from linear_attention_tree_amd import bole
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    cp, pd, co = d(c.cand_parent), d(c.p_draft), d(c.cand_off)
    out = _outputs(len(c.cand_parent), c.B, capacity, dev)
    args = [cp, pd, co, capacity, max_tree, out["rho"], out["parent"], out["cand_of"],
            out["tree_off"]]
    if workspace is not None:
        args.append(workspace)
    getattr(bole, fn)(*args, err=out["err"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def test_noalloc_matches_workspace_entry_on_two_calls():
    from linear_attention_tree_amd import bole
    dev = torch.device("cuda:0")
    # the first call fills the whole array (B * max_tree = 16384), the second
    # is smaller and reads keys the first left in the slots past its own
    runs = [(W.make_candidates(256, seed=31), 4096, 64),
            (W.make_candidates(12, seed=32), 300, 48)]
    for c, capacity, max_tree in runs:
        say(f"noalloc forest: B={c.B} M_total={int(c.cand_off[-1])} capacity={capacity} "
            f"max_tree={max_tree}")
        ws = torch.empty(bole.bole_forest_workspace_bytes(c.B, max_tree), dtype=torch.uint8,
                         device=dev)
        ref = _run("bole_forest_build", c, capacity, max_tree, dev, workspace=ws)
        got = _run("bole_forest_build_noalloc", c, capacity, max_tree, dev)
        assert ref["err"][0] == 0
        for k in ("parent", "cand_of", "tree_off", "err"):
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["rho"].view(np.uint32), ref["rho"].view(np.uint32))
        say(f"  bit-exact, {int(got['tree_off'][-1])} nodes packed")


def test_noalloc_rejects_shapes_beyond_its_array():
    from linear_attention_tree_amd import bole
    dev = torch.device("cuda:0")
    c = W.make_candidates(257, seed=33)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    out = _outputs(len(c.cand_parent), c.B, 1000, dev)
    with pytest.raises(bole.BoleError):  # 257 x 64 listed slots exceed the array
        bole.bole_forest_build_noalloc(d(c.cand_parent), d(c.p_draft), d(c.cand_off), 1000, 64,
                                       out["rho"], out["parent"], out["cand_of"], out["tree_off"],
                                       err=out["err"])
    torch.cuda.synchronize()
    assert int(out["tree_off"][0].item()) == 99  # nothing was launched
