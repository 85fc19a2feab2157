"""The allocation-free LM-head entry point (static device scratch) against the
workspace entry point: two calls in a row, the second with fewer rows, must
give bit-identical entropies, argmaxes and top-2 gaps; a row count beyond the
static scratch is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_noalloc_lm_head_matches_the_workspace_entry():
    from diffusion_decoding_amd import _lib
    from diffusion_decoding_amd import runtime as rt
    from workloads import make_inputs, tiny_config

    _lib.load()
    vocab, d = 262144, 2048
    cfg = tiny_config(name="noalloc_lm", act_dtype="bf16", expert_dtype="bf16", vocab=vocab, d_model=d,
                      canvas_len=256, head_dim=128, n_heads=16, d_expert=32, d_shared=32, prompt_len=64)
    inp = make_inputs(cfg, device="cuda")
    model = rt.Model(inp)
    g = torch.Generator("cuda").manual_seed(5)
    for T in (256, 100):
        print(f"LM head at {T} x {d} x {vocab}: workspace entry vs static-scratch entry", flush=True)
        hf = torch.randn(T, d, device="cuda", generator=g).to(torch.bfloat16)
        e1, a1, g1 = rt.test_lm_head(model, hf)
        e2 = torch.full((T,), float("nan"), device="cuda")
        a2 = torch.full((T,), -1, dtype=torch.int32, device="cuda")
        g2 = torch.full((T,), float("nan"), device="cuda")
        rt.lm_head_confidence_noalloc(model, hf, e2, a2, g2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(e1.cpu().numpy().view(np.uint32), e2.cpu().numpy().view(np.uint32))
        np.testing.assert_array_equal(a1.cpu().numpy(), a2.cpu().numpy())
        np.testing.assert_array_equal(g1.cpu().numpy().view(np.uint32), g2.cpu().numpy().view(np.uint32))
    big = torch.zeros(410, d, dtype=torch.bfloat16, device="cuda")
    out_e = torch.empty(410, device="cuda")
    out_a = torch.empty(410, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.DGError) as e:
        rt.lm_head_confidence_noalloc(model, big, out_e, out_a)
    assert e.value.status == _lib.DG_ERR_SHAPE and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    model.close()
