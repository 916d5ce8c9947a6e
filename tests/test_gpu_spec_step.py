"""The speculative decode step (three W4A4 drafter passes with the FP8
lm_head, then the 4-token W4A16 verify with the NVFP4 lm_head) on the GPU:
every stage against the oracle on that stage's own GPU input (the chain's
routing and argmax decisions drawn clear of near ties), and the step
captured as one graph, replayed with eager work in between, bit for bit
equal to the eager step, also after the input changes."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import host, ws_view
from inputs import SEED
from q4moe_testutil import bf16_bits_to_f64, gate_f32, gate_out
from spec_step import DRAFT_LAYER, H, I, K, SpecStep
from test_gpu_w4a4_decode import check_w4a4_decode

pytestmark = pytest.mark.gpu

GAP = 1e-4


@pytest.fixture(scope="module")
def step():
    return SpecStep(torch, g, synth, SEED)


def _argmax_clear(lg):
    srt = np.sort(lg, axis=1)
    return bool(np.all(srt[:, -1] - srt[:, -2] >= 1e-3 * np.maximum(1.0, np.abs(lg).max(axis=1))))


def _run_clear(step):
    """Eager steps over x0 attempts until every routing and argmax decision
    of the chain is clear of near ties on the GPU's own stage inputs."""
    for attempt in range(24):
        step.set_x0(synth.x_rows(SEED, synth.FAM_W4A4, DRAFT_LAYER, H, [attempt])[0])
        step.step()
        torch.cuda.synchronize()
        out = step.outputs()
        xv, yv = out["xv"].view(np.uint16), out["yv"].view(np.uint16)
        rd = oracle.router(step.dwg, step.db, xv[:3], K)  # draft pass i reads row i - 1
        rv = oracle.router(step.wg, step.b, xv, K)
        if min(rd["gap"]) < GAP or min(rv["gap"]) < GAP:
            continue
        fq = [oracle.fp8_quant(bf16_bits_to_f64(xv[i]).astype(np.float32), step.fp8_is) for i in (1, 2, 3)]
        flg = np.stack([oracle.fp8_gemv(step.fp8_codes, q, step.fp8_ws, step.fp8_is) for q in fq])
        vlg, vam, vgap = oracle.gemv_nvfp4(step.lm_codes, step.lm_scales, step.lm_g, yv)
        if not _argmax_clear(flg) or np.any(vgap < 1e-3 * np.maximum(1.0, np.abs(vlg).max(axis=1))):
            continue
        return out, rd, rv, fq, flg, vlg, vam
    raise RuntimeError("no clear chain found")


def test_spec_step_stages(step):
    out, rd, rv, fq, flg, vlg, vam = _run_clear(step)
    xv = out["xv"].view(np.uint16)
    # draft passes: the W4A4 MoE stage by stage (its taps), the FP8 lm_head
    tp = g.q4moe_w4a4_decode_taps(step.drouter, step.dex, 1)
    for i in (1, 2, 3):
        b = host(step.d_ws[i - 1])
        o = dict(y=xv[i:i + 1], ids=out["d_ids"][i - 1:i], w=out["d_w"][i - 1:i],
                 y32=ws_view(b, tp.y32, H, np.float32)[None],
                 h32=ws_view(b, tp.h32, K * I, np.float32).reshape(K, I),
                 xq_codes=ws_view(b, tp.xq_codes, H // 2, np.uint8)[None],
                 xq_scales=ws_view(b, tp.xq_scales, H // 16, np.uint8)[None],
                 hq_codes=ws_view(b, tp.hq_codes, K * I // 2, np.uint8).reshape(K, I // 2),
                 hq_scales=ws_view(b, tp.hq_scales, K * I // 16, np.uint8).reshape(K, I // 16))
        L = dict(bank=step.draft_bank, x=xv[i - 1:i], route={k: v[i - 1:i] for k, v in rd.items()})
        worst = check_w4a4_decode(L, o)[0]
        off = g.q4moe_fp8_gemv_taps(step.fp8, 1)
        assert np.array_equal(ws_view(host(step.f_ws[i - 1]), off, H, np.uint8), fq[i - 1]), "fp8 codes differ"
        ok, wl = gate_f32(out["d_logits"][i - 1:i], flg[i - 1:i])
        assert ok, f"draft {i}: fp8 logit gate exceeded ({wl:.3f})"
        assert out["d_am"][i - 1] == int(np.argmax(flg[i - 1]))
        print(f"draft pass {i}: MoE worst bf16 ratio {worst:.3f}, lm_head logit ratio {wl:.4f}", flush=True)
    # verify: the W4A16 MoE on the 4 rows, then the NVFP4 lm_head on its output
    ob = oracle.Bank.from_dict(oracle.NVFP4, step.bank)
    assert np.array_equal(out["v_ids"], rv["ids"])
    np.testing.assert_allclose(out["v_w"], rv["w"], rtol=1e-5)
    yhat, _ = oracle.moe_w4a16(ob, xv, rv["ids"], rv["w"])
    ok, worst = gate_out(out["yv"].view(np.uint16), yhat)
    assert ok, f"verify MoE gate exceeded ({worst:.3f})"
    ok, wl = gate_f32(out["v_logits"], vlg)
    assert ok, f"verify lm_head gate exceeded ({wl:.3f})"
    assert np.array_equal(out["v_am"], vam)
    print(f"verify: MoE worst bf16 ratio {worst:.3f}, lm_head logit ratio {wl:.4f}; drafts "
          f"{out['d_am'].tolist()}, verify argmax {out['v_am'].tolist()}", flush=True)


def test_spec_step_graph_replays(step):
    step.set_x0(synth.x_rows(SEED, synth.FAM_W4A4, DRAFT_LAYER, H, [0])[0])
    step.step()
    torch.cuda.synchronize()
    ref = step.outputs()
    graph = step.capture()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for k in ref:
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), f"replay {rep}: {k} differs"
        step.step()  # eager work between replays
        torch.cuda.synchronize()
    # a new input: the replay follows it like the eager step
    step.set_x0(synth.x_rows(SEED, synth.FAM_W4A4, DRAFT_LAYER, H, [5])[0])
    step.step()
    torch.cuda.synchronize()
    ref2 = step.outputs()
    assert not np.array_equal(ref2["xv"], ref["xv"])
    graph.replay()
    torch.cuda.synchronize()
    got = step.outputs()
    for k in ref2:
        assert np.array_equal(got[k].view(np.uint8), ref2[k].view(np.uint8)), f"new input: {k} differs"
    for ws in step.d_ws + [step.v_ws]:
        assert g.q4moe_ws_check(ws) == 0
