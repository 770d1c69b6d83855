"""The modulation entry point that allocates nothing
(dit_modulation_forward_noalloc, scratch in the library's fixed device
array) against dit_modulation_forward with a caller workspace: the same
kernels, so the results must agree bit for bit, on consecutive calls of
decreasing batch (the fixed array keeps the previous call's contents) and
on a second configuration."""
import dataclasses

import numpy as np
import pytest

from diffusion_transformer_fwd_amd import dit, synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    dit.lib()


def _weights(cfg):
    return dit.ModelWeights(synth.ModelWeights(dataclasses.replace(cfg, n_dual=0, n_single=0), 0))


@pytest.mark.parametrize("cfg", [synth.FLUX2_KLEIN,
                                 synth.DitConfig(hidden=256, heads=2, head_dim=128,
                                                 mlp_hidden=768, n_dual=0, n_single=0,
                                                 in_channels=128, txt_channels=256)],
                         ids=["d3072", "d256"])
def test_noalloc_modulation_matches_workspace_entry(cfg):
    dw = _weights(cfg)
    for sig in ([0.75, 0.3, 0.9, 0.1, 0.55, 1.0, 0.0], [0.42, 0.8]):
        want = dit.modulation(cfg, dw, sig)
        got = dit.modulation_noalloc(cfg, dw, sig)
        torch.cuda.synchronize()
        log(f"noalloc modulation D={cfg.hidden} B={len(sig)}")
        assert torch.equal(got, want), f"B={len(sig)}"


def test_noalloc_modulation_largest_batch():
    cfg = synth.FLUX2_KLEIN
    dw = _weights(cfg)
    sig = list(np.linspace(0.0, 1.0, dit.MAX_BATCH))
    want = dit.modulation(cfg, dw, sig)
    got = dit.modulation_noalloc(cfg, dw, sig)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
