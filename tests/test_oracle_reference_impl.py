"""The oracle against the torch implementation that the Gated DeltaNet API page
links as the reference of torch_chunk_gated_delta_rule (page
"core.ssm.gated_delta_net.gdn", the "Reference:" link of that function: the
Hugging Face transformers Qwen3-Next module, installed in this image).

That implementation computes in float32, so agreement is checked to 1e-5 of
each tensor's scale (per element, floored at the tensor's RMS).  It pins the
readings the pages leave open to the implementation they cite:
  * the state layout: its initial and final states are [B, H, K, V], the same
    [K, V] layout (element [i][j] = S[j][i]) as the oracle's;
  * the default scale 1/sqrt(K) (that implementation has no scale argument);
  * the in-kernel L2 norm x / sqrt(sum x^2 + 1e-6), including rows whose squared
    norm is near the epsilon, where its placement changes the result at O(1);
  * decay before the delta, beta on both terms, chunking that restarts per call.
It runs on the CPU only and never touches the GPU library.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
ref = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")


def _inputs(seed, B, T, H, K, V, tiny_rows=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, K))
    k = r.standard_normal((B, T, H, K))
    if tiny_rows:
        # every third row scaled so that its squared norm is ~1e-6 (0.3e-6 .. 3e-6)
        sq = np.sqrt(r.uniform(0.3e-6, 3e-6, (B, T, H, 1)))
        sk = np.sqrt(r.uniform(0.3e-6, 3e-6, (B, T, H, 1)))
        m = (np.arange(T) % 3 == 0)[None, :, None, None]
        q = np.where(m, q / np.linalg.norm(q, axis=-1, keepdims=True) * sq, q)
        k = np.where(m, k / np.linalg.norm(k, axis=-1, keepdims=True) * sk, k)
    v = r.standard_normal((B, T, H, V))
    g = -r.uniform(0.0, 0.3, (B, T, H))
    beta = r.uniform(0.05, 0.95, (B, T, H))
    s0 = 0.5 * r.standard_normal((B, H, K, V))
    # inputs rounded to float32 so both sides start from the same values
    return [x.astype(np.float32).astype(np.float64) for x in (q, k, v, g, beta, s0)]


def _err(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


def _reference(which, q, k, v, g, beta, s0, l2):
    t = lambda a: torch.tensor(a, dtype=torch.float32)  # noqa: E731
    if which == "chunk":
        o, fs = ref.torch_chunk_gated_delta_rule(
            t(q), t(k), t(v), t(g), t(beta), chunk_size=64, initial_state=t(s0),
            output_final_state=True, use_qk_l2norm_in_kernel=l2)
    else:
        o, fs = ref.torch_recurrent_gated_delta_rule(
            t(q), t(k), t(v), t(g), t(beta), initial_state=t(s0), output_final_state=True,
            use_qk_l2norm_in_kernel=l2)
    return o.double().numpy(), fs.double().numpy()


@pytest.mark.parametrize("which", ["chunk", "recurrent"])
@pytest.mark.parametrize("l2", [False, True])
@pytest.mark.parametrize("K,V", [(16, 16), (32, 64)])
def test_oracle_matches_cited_implementation(which, l2, K, V):
    # T = 203 is not a multiple of the 64-token chunk; non-zero initial state
    q, k, v, g, beta, s0 = _inputs(3, 2, 203, 2, K, V)
    if not l2:
        q = q / np.linalg.norm(q, axis=-1, keepdims=True)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                           use_qk_l2norm=l2)
    ro, rf = _reference(which, q, k, v, g, beta, s0, l2)
    assert ro.shape == o.shape and rf.shape == fs.shape
    assert _err(o, ro) <= 1e-5, _err(o, ro)
    assert _err(fs, rf) <= 1e-5, _err(fs, rf)


@pytest.mark.parametrize("which", ["chunk", "recurrent"])
def test_l2norm_epsilon_matches_cited_implementation(which):
    """Rows with squared norm ~1e-6: only the epsilon's placement decides them."""
    q, k, v, g, beta, s0 = _inputs(4, 1, 150, 2, 16, 16, tiny_rows=True)
    o, fs = oracle.prefill(q, k, v, g, beta, initial_state=s0, output_final_state=True,
                           use_qk_l2norm=True)
    ro, rf = _reference(which, q, k, v, g, beta, s0, True)
    assert _err(o, ro) <= 1e-5, _err(o, ro)
    assert _err(fs, rf) <= 1e-5, _err(fs, rf)
    # the same rows with the epsilon outside the square root move the outputs by O(1)
    qn = q / (np.linalg.norm(q, axis=-1, keepdims=True) + 1e-6)
    kn = k / (np.linalg.norm(k, axis=-1, keepdims=True) + 1e-6)
    o2, _ = oracle.prefill(qn, kn, v, g, beta, initial_state=s0, output_final_state=True)
    assert _err(o2, ro) > 1e-2
