"""The split forward without allocation, lizard_attn_fwd_split_noalloc (its
workspace in the library's fixed per-GPU scratch), against
lizard_attn_fwd_split with a caller workspace: the same kernels on the same
inputs, so every output must match bit for bit.  Two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents,
which no call may depend on).  And the refusal, before anything is
launched, of sizes whose workspace exceeds the scratch."""
import ctypes

import pytest

import subquadratic_attention_amd as sqa
from tests.gpu_util import log

FAKE = 0x10000   # 16-byte aligned; never dereferenced (the call returns first)


def test_refuses_sizes_beyond_the_scratch():
    lib = sqa.load_library()
    p = sqa.make_params(1, 1, 1 << 26, 128, window=64, n_meta=4, alpha=0.5, dtype=sqa.LIZARD_BF16)
    need = lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(p))
    assert need > sqa.NOALLOC_SCRATCH_BYTES
    st = lib.lizard_attn_fwd_split_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, 0,
                                           FAKE, None, None, None, None)
    assert st == sqa.STATUS_CODE["LIZARD_E_WORKSPACE"]
    # the 32-head, 32K-token prefill fits
    p = sqa.make_params(1, 32, 32768, 128, window=64, n_meta=4, alpha=0.5, dtype=sqa.LIZARD_BF16)
    assert 0 < lib.lizard_attn_fwd_split_workspace_size(ctypes.byref(p)) <= sqa.NOALLOC_SCRATCH_BYTES
    assert f"#define LIZARD_NOALLOC_SCRATCH_BYTES ({sqa.NOALLOC_SCRATCH_BYTES >> 20}u << 20)" in \
        open(sqa.HEADER_PATH).read()


def _inputs(B, H, L, d, m, halo, seed):
    import torch

    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16

    def rn(*shape, sd=0.125):
        return (torch.randn(*shape, generator=g, device="cuda") * sd).to(dt)

    x = {"q": rn(B, H, L, d), "k": rn(B, H, L, d), "v": rn(B, H, L, d), "meta": rn(H, m, d)}
    logit = torch.randn(B, H, L, d, generator=g, device="cuda") * 2.0 + 2.0
    x["gate_logit"] = logit.to(dt)
    x["log_g"] = torch.nn.functional.logsigmoid(logit).contiguous()
    x["state_in"] = torch.randn(B, H, d, d, generator=g, device="cuda") * 0.1
    x["k_halo"] = rn(B, H, halo, d)
    x["v_halo"] = rn(B, H, halo, d)
    return x


def _nan_out(x):
    import torch

    q = x["q"]
    B, H, L, d = q.shape
    nan = float("nan")
    return {"y": torch.full_like(q, nan), "lse": torch.full((B, H, L), nan, device="cuda"),
            "y_anchor": torch.full_like(q, nan), "state": torch.full((B, H, d, d), nan, device="cuda")}


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_call(gpu_lib):
    import torch

    cases = [
        # (B, H, L, d, m, halo, gates, continued): the 32-head 32K-token prefill, then a smaller
        # continued segment fed with gate logits
        (1, 32, 32768, 128, 4, 0, "log_g", False),
        (1, 4, 5000, 128, 3, 40, "gate_logit", True),
    ]
    runs = []
    for i, (B, H, L, d, m, halo, gates, cont) in enumerate(cases):
        x = _inputs(B, H, L, d, m, halo, 700 + i)
        kw = dict(window=64, alpha=0.5, need_lse=True, need_y_anchor=True, need_state=True)
        kw[gates] = x[gates]
        if cont:
            kw.update(state_in=x["state_in"], k_halo=x["k_halo"], v_halo=x["v_halo"])
        ref = gpu_lib.lizard_attn_fwd_split(x["q"], x["k"], x["v"], x["meta"], **kw)
        runs.append((x, kw, ref))
    torch.cuda.synchronize()
    # the no-allocation calls in a row, the second on the smaller input
    got = []
    for x, kw, _ in runs:
        got.append(sqa.lizard_attn_fwd_split_noalloc(x["q"], x["k"], x["v"], x["meta"], out=_nan_out(x), **kw))
    torch.cuda.synchronize()
    for (x, kw, ref), o in zip(runs, got):
        log(f"noalloc shape {tuple(x['q'].shape)}")
        for key in ("y", "lse", "y_anchor", "state"):
            iv = torch.int16 if o[key].dtype == torch.bfloat16 else torch.int32
            assert torch.equal(o[key].view(iv), ref[key].view(iv)), key
