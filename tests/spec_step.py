"""One speculative decode step through one MoE layer, as the worklog runs
it ("Let's optimize Nemotron 3.5 Lightning - a worklog", Step 5: k = 3 drafts
verified 4 tokens at a time; Step 6: the drafter's experts NVFP4; Step 7:
the drafter's passes recorded as one graph; "Quantization (PTQ + QAD)", MTP
Drafter Precision: drafter experts NVFP4 W4A4, the lm_head it uses FP8):

  draft pass i = 1..3: the drafter's W4A4 MoE on one token, then its FP8
  lm_head GEMV + argmax;
  verify: the backbone's W4A16 NVFP4 MoE on the real token and the three
  drafts (4 tokens), then the NVFP4 lm_head GEMV + argmax.

Only the hot path is here: the embedding, attention and Mamba blocks around
the MoE are not.  Their place in the chain is taken by the MoE outputs
themselves: draft pass i reads row i - 1 of the verify input xv [4][H] and
writes its MoE output into row i, so row 0 is the real token and rows 1-3
the drafts.  Every buffer is allocated here, so that the whole step can be
captured as one graph."""
import numpy as np

H, I, E, K, V = 2688, 1856, 128, 6, 131072
DRAFT_LAYER = 40  # the drafter's seeded layer index (distinct from the backbone's 0..22)


class SpecStep:
    def __init__(self, torch, g, synth, seed, x0=None):
        from gpu_util import dev
        self.torch, self.g = torch, g
        cuda = "cuda"
        # drafter: a W4A4 NVFP4 MoE layer and the FP8 lm_head
        db = synth.expert_bank(seed, synth.FAM_W4A4, DRAFT_LAYER, E, H, I, "nvfp4")
        self.draft_bank = db
        t = {k: dev(v) for k, v in db.items()}
        self.dex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                             t["up_gscale"], t["down_gscale"])
        self.dwg, self.db = synth.router(seed, synth.FAM_W4A4, DRAFT_LAYER, E, H)
        self.drouter = g.Router(dev(self.dwg), dev(self.db), K)
        self.fp8_codes, self.fp8_ws, self.fp8_is = synth.lm_head_fp8(seed, synth.FAM_W4A4, DRAFT_LAYER, V, H)
        self.fp8 = g.Fp8Mat(dev(self.fp8_codes), self.fp8_ws, self.fp8_is)
        # backbone: a W4A16 NVFP4 MoE layer and the NVFP4 lm_head
        bb = synth.expert_bank(seed, synth.FAM_NVFP4, 0, E, H, I, "nvfp4")
        self.bank = bb
        t = {k: dev(v) for k, v in bb.items()}
        self.ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                            t["up_gscale"], t["down_gscale"])
        self.wg, self.b = synth.router(seed, synth.FAM_NVFP4, 0, E, H)
        self.router = g.Router(dev(self.wg), dev(self.b), K)
        self.lm_codes, self.lm_scales, self.lm_g = synth.lm_head(seed, 0, 0, V, H)
        self.lm = g.QMat(g.NVFP4, dev(self.lm_codes), dev(self.lm_scales),
                         dev(np.array([self.lm_g], np.float32)))
        # buffers
        self.xv = torch.zeros((4, H), dtype=torch.int16, device=cuda)
        if x0 is not None:
            self.set_x0(x0)
        self.yv = torch.empty((4, H), dtype=torch.int16, device=cuda)
        self.d_ids = torch.empty((3, K), dtype=torch.int32, device=cuda)
        self.d_w = torch.empty((3, K), dtype=torch.float32, device=cuda)
        self.d_logits = torch.empty((3, V), dtype=torch.float32, device=cuda)
        self.d_am = torch.empty(3, dtype=torch.int32, device=cuda)
        self.v_ids = torch.empty((4, K), dtype=torch.int32, device=cuda)
        self.v_w = torch.empty((4, K), dtype=torch.float32, device=cuda)
        self.v_logits = torch.empty((4, V), dtype=torch.float32, device=cuda)
        self.v_am = torch.empty(4, dtype=torch.int32, device=cuda)
        # one workspace per pass, so that every pass's taps survive the step
        self.d_ws = [g.workspace(g.q4moe_w4a4_decode_ws_bytes(self.drouter, self.dex, 1)) for _ in range(3)]
        self.f_ws = [g.workspace(g.q4moe_fp8_gemv_ws_bytes(self.fp8, 1)) for _ in range(3)]
        self.v_ws = g.workspace(g.q4moe_w4a16_decode_ws_bytes(self.router, self.ex, 4))
        self.l_ws = g.workspace(g.q4moe_w4a16_gemv_ws_bytes(self.lm, 4))

    def set_x0(self, x0_bits):
        from gpu_util import dev
        self.xv[0].copy_(dev(np.asarray(x0_bits, np.uint16).reshape(H)))

    def draft(self, i):
        """Draft pass i (1..3): input row i - 1 of xv, output into row i."""
        g = self.g
        g.q4moe_w4a4_decode(self.drouter, self.dex, self.xv[i - 1:i], self.xv[i:i + 1], self.d_ids[i - 1:i],
                            self.d_w[i - 1:i], ws=self.d_ws[i - 1])
        g.q4moe_fp8_gemv(self.fp8, self.xv[i:i + 1], self.d_logits[i - 1:i], self.d_am[i - 1:i],
                         ws=self.f_ws[i - 1])

    def verify(self):
        g = self.g
        g.q4moe_w4a16_decode(self.router, self.ex, self.xv, self.yv, self.v_ids, self.v_w, ws=self.v_ws)
        g.q4moe_w4a16_gemv(self.lm, self.yv, self.v_logits, self.v_am, ws=self.l_ws)

    def step(self):
        for i in (1, 2, 3):
            self.draft(i)
        self.verify()

    def outputs(self):
        """Every output of the step, as host arrays."""
        return {k: getattr(self, k).detach().cpu().numpy().copy()
                for k in ("xv", "yv", "d_ids", "d_w", "d_logits", "d_am", "v_ids", "v_w", "v_logits", "v_am")}

    def capture(self):
        """The whole step as one graph (after one eager step)."""
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        torch.cuda.synchronize()
        return graph
