"""The pilot-shaped decoder stack (110M parameters, 12 layers, width 768,
Q2 x Q2 SwiGLU FFN of width 1536) generating with the library's FFN: the
method inside the model against the oracle, the whole model against a CPU
reference, and HIP-graph generation against eager generation.  Needs an
MI355X; goes through the C ABI for every FFN call."""
import numpy as np
import pytest
import torch

import associative_algebra_block_amd as aa
import oracle
from associative_algebra_block_amd.pilot_stack import PilotConfig, PilotGenerator, make_weights
from tests import _pilot_reference as R
from tests._gpu_util import assert_parity, host, metrics, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = PilotConfig()
B, P, STEPS = 2, 8, 4


@pytest.fixture(scope="module")
def model():
    assert torch.cuda.is_available()
    aa.load()
    w = make_weights(CFG, 0, DEV)
    g = torch.Generator(device="cpu")
    g.manual_seed(11)
    prompt = torch.randint(0, CFG.vocab, (B, P), generator=g).to(DEV)
    return w, prompt


def _generate(gen, prompt, steps):
    """Prefill, then `steps` decode steps; returns the token sequences
    (prompt + chosen tokens) and the final hidden states and logits of every
    decode step."""
    gen.prefill(prompt)
    toks = [prompt.cpu().numpy()]
    hid, logits = [], []
    for _ in range(steps):
        toks.append(gen.token.cpu().numpy()[:, None])
        gen.decode_step()
        hid.append(host(gen.hidden))
        logits.append(host(gen.logits))
    torch.cuda.synchronize()
    return np.concatenate(toks, axis=1), hid, logits


def test_ffn_calls_inside_the_model_match_the_oracle(model):
    """Every FFN call of a prefill (positions 0..7 of two sequences) and of
    four decode steps (positions 8..11, types from the device position)
    against the oracle's FFN of the GPU's own input (H rounded to bf16, as the
    library stores it), at the plain bounds."""
    w, prompt = model
    say("pilot model ffn calls", B, P, STEPS)
    gen = PilotGenerator(CFG, w, "algebra", B, DEV)
    gen.trace = []
    _generate(gen, prompt, STEPS)
    assert len(gen.trace) == CFG.layers * (1 + STEPS)
    for n, (l, f, y, plen, types) in enumerate(gen.trace):
        lw = w["layers"][l]
        fh = host(f)
        if plen:
            t = oracle.types_pos_mod(fh.shape[0], CFG.q, 0, plen)
        else:
            pos = P + (n // CFG.layers) - 1
            t = types.cpu().numpy()
            assert np.all(t == pos % CFG.q), (pos, t)
        G = oracle.project(fh, host(lw["Wg"]), "Q2xQ2", CFG.q, t)
        U = oracle.project(fh, host(lw["Wu"]), "Q2xQ2", CFG.q, t)
        Hh = torch.from_numpy(oracle.silu(G) * U).to(torch.bfloat16).double().numpy()
        ref = oracle.project(Hh, host(lw["Wd"]), "Q2xQ2", CFG.q, t)
        rel, mx = metrics(host(y), ref)
        assert rel <= 5e-3 and mx <= 2e-2, (n, l, plen, rel, mx)
    say(f"pilot model: {len(gen.trace)} FFN calls within the bounds")


@pytest.mark.parametrize("ffn", ["algebra", "dense"])
def test_generation_matches_cpu_reference(model, ffn):
    """Teacher-forced on the GPU's own token sequences, the CPU reference (the
    same architecture in float64, bf16 where the GPU stores bf16, the FFN from
    the oracle) gives the same final hidden states and logits within the
    drift that rounding to bf16 at every layer allows, and every token the
    GPU chose is a largest reference logit up to that drift."""
    w, prompt = model
    say("pilot model generation", ffn, B, P, STEPS)
    gen = PilotGenerator(CFG, w, ffn, B, DEV)
    toks, hid, logits = _generate(gen, prompt, STEPS)
    hf, lg = R.forward(CFG, R.host_weights(w), toks, ffn)
    # decode step s feeds position P + s: its hidden state and logits are the
    # reference's at that position; the token it picks is fed at step s + 1
    rms0 = float(np.sqrt(np.mean(lg[:, P - 1] ** 2)))
    for b in range(B):   # the prefill's pick
        assert lg[b, P - 1, toks[b, P]] >= lg[b, P - 1].max() - 0.1 * rms0, b
    for s in range(STEPS):
        ref_l = lg[:, P + s]
        rel_h, _ = metrics(hid[s], hf[:, P + s])
        rel_l, mx_l = metrics(logits[s], ref_l)
        say(f"{ffn} step {s}: hidden rel {rel_h:.2e}  logits rel {rel_l:.2e} max/rms {mx_l:.2e}")
        assert rel_h <= 2e-2 and rel_l <= 2e-2, (s, rel_h, rel_l)
        if s + 1 < STEPS:
            rms = float(np.sqrt(np.mean(ref_l ** 2)))
            for b in range(B):
                assert ref_l[b, toks[b, P + s + 1]] >= ref_l[b].max() - 0.1 * rms, (s, b)


def test_graph_generation_equals_eager(model):
    """One decode step captured in a HIP graph (device-side position, types
    and token) replayed for six consecutive positions, with eager work and a
    synchronisation between replays, gives the eager generation's logits and
    tokens bit for bit."""
    w, prompt = model
    say("pilot model graph", B, P)
    eager = PilotGenerator(CFG, w, "algebra", B, DEV)
    eager.prefill(prompt)
    ref = []
    for _ in range(6):
        eager.decode_step()
        ref.append((eager.logits.clone(), eager.token.clone()))
    gen = PilotGenerator(CFG, w, "algebra", B, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up before capture
        gen.prefill(prompt)
        for _ in range(2):
            gen.decode_step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gen.decode_step()
    gen.prefill(prompt)   # back to the state after the prompt
    other = torch.empty(64, CFG.d, dtype=torch.float32, device=DEV)
    for r in range(6):
        graph.replay()
        aa.aa_project_fwd(gen.down_dec, torch.ones(64, CFG.ffn, dtype=torch.bfloat16, device=DEV),
                          gen.packed[0][2], other, None, 0, torch.zeros(64, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        assert torch.equal(gen.logits, ref[r][0]) and torch.equal(gen.token, ref[r][1]), r
