"""The whole verify step can be captured in a HIP graph (through torch's graph
capture): the library allocates nothing, records no memset and takes its
plans on the host at capture time.  Every replay, with eager steps and
synchronisations in between, must give the eager step's bits."""
import pytest
import torch

pytestmark = pytest.mark.gpu

from parity import bits_equal, log, make  # noqa: E402


def _outputs(vs):
    return [t.clone() for t in (vs.mask, vs.attn_out, vs.acc.accept_len, vs.acc.path,
                                vs.acc.tokens, vs.acc.child_p, vs.new_len)]


@pytest.mark.parametrize("name,kw,acceptance,T", [
    ("dynamic", dict(B=6, L=("uniform", 30, 700), V=5000), "sample", 1.0),
    ("specinfer", dict(B=3, L=700, Hq=16, Hkv=2, V=6000), "topk", 0.8),
    ("medusa", dict(L=200, V=3000, Hq=4, Hkv=4), "sample", 0.0),
])
def test_step_replays_in_a_graph(name, kw, acceptance, T):
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    w = make(name, **({"draft": "topk"} if acceptance == "topk" else {}), **kw)
    vs = VerifyStep(w, temperature=T, seed=3, step=1, acceptance=acceptance)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vs.run()                              # warm-up on a side stream, as capture wants
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    vs.run()
    torch.cuda.synchronize()
    ref = _outputs(vs)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vs.run()
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, _outputs(vs)):
            assert bits_equal(a, b), f"replay {i} differs from the eager step"
        vs.run()                              # eager work between replays
        torch.cuda.synchronize()
    log(f"[graph] {name}/{acceptance}: 3 replays identical to the eager step")


@pytest.mark.parametrize("T,store", [(1.0, True), (0.0, False)])
def test_head_step_replays_in_a_graph(T, store):
    """The step with the fused LM head in place of the given logits
    (spec_lm_head_accept) replays bit for bit too, logits included."""
    import workloads as W
    from tree_attention_verification_02_amd.pipeline import VerifyStep
    w = make("dynamic", B=6, L=("uniform", 30, 700), V=5000, Hq=4, Hkv=1)
    hidden, weight = W.heads.head_inputs(w, H=256)
    vs = VerifyStep(w, temperature=T, seed=3, step=1, head=(hidden, weight),
                    store_head_logits=store)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vs.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    vs.run()
    torch.cuda.synchronize()
    ref = _outputs(vs) + [vs.head_logits.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vs.run()
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, _outputs(vs) + [vs.head_logits]):
            assert bits_equal(a, b), f"replay {i} differs from the eager step"
        vs.run()
        torch.cuda.synchronize()
    log(f"[graph] head T={T}: 3 replays identical to the eager step")
