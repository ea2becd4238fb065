"""Host-side checks of the Python binding (no GPU needed): a tensor of the
wrong shape, dtype or device is refused with an error naming it before any
pointer reaches the library (a kernel handed a float32 buffer where it
expects bfloat16, or a shorter one, would read past the allocation).  The
tensors live on the CPU, so a call whose arguments all pass the checks
would stop at the device check instead; every case below must stop earlier,
at the named argument."""
import os

import pytest
import torch

import subquadratic_attention_amd as sqa

B, H, L, d, m, w = 2, 3, 40, 64, 4, 16


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(sqa.LIB_PATH):
        from subquadratic_attention_amd import build

        build.build()
    return sqa.load_library()


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def seq():
    return dict(q=t(B, H, L, d), k=t(B, H, L, d), v=t(B, H, L, d), log_g=t(B, H, L, d, dtype=torch.float32),
                meta=t(H, m, d), lse=t(B, H, L, dtype=torch.float32), dy=t(B, H, L, d))


def fwd(x):
    return sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta"], window=w, alpha=0.5)


def bwd(x):
    return sqa.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta"], x["lse"], x["dy"], window=w, alpha=0.5)


def test_valid_arguments_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        fwd(seq())
    with pytest.raises(ValueError, match="GPU"):
        bwd(seq())


@pytest.mark.parametrize("name,bad,err", [
    ("log_g", t(B, H, L, d), TypeError),                          # bfloat16 log-gates: half the bytes read twice over
    ("log_g", t(B, H, L - 1, d, dtype=torch.float32), ValueError),
    ("k", t(B, H, L + 1, d), ValueError),
    ("v", t(B, H, L, d, dtype=torch.float32), TypeError),
    ("meta", t(H, m, d + 1), ValueError),
    ("meta", t(H + 1, m, d), ValueError),
    ("meta", t(H, m, d, dtype=torch.float32), TypeError),
])
def test_forward_refuses(name, bad, err):
    x = seq()
    x[name] = bad
    with pytest.raises(err, match="log_g|k:|v:|meta_k"):
        fwd(x)


@pytest.mark.parametrize("key,bad,err", [
    ("y", t(B, H, L, d, dtype=torch.float32), TypeError),
    ("lse", t(B, H, L + 1, dtype=torch.float32), ValueError),
    ("state", t(B, H, d, d), TypeError),
    ("y_anchor", t(B, H, L, d - 1), ValueError),
])
def test_forward_refuses_outputs(key, bad, err):
    x = seq()
    with pytest.raises(err, match=key):
        sqa.lizard_attn_fwd(x["q"], x["k"], x["v"], x["log_g"], x["meta"], window=w, alpha=0.5,
                            out={key: bad}, need_lse=True, need_state=True, need_y_anchor=True)


@pytest.mark.parametrize("name,bad,err,match", [
    ("lse", t(B, H, L), TypeError, "lse"),
    ("lse", t(B, H, L, 1, dtype=torch.float32), ValueError, "lse"),
    ("dy", t(B, H, L, d, dtype=torch.float32), TypeError, "dy"),
    ("log_g", t(B, H, L, d), TypeError, "log_g"),
])
def test_backward_refuses(name, bad, err, match):
    x = seq()
    x[name] = bad
    with pytest.raises(err, match=match):
        bwd(x)


@pytest.mark.parametrize("key,bad,err", [
    ("dq", t(B, H, L, d, dtype=torch.float32), TypeError),
    ("dlog_g", t(B, H, L, d), TypeError),
    ("dmeta", t(H, m, d), TypeError),
    ("dv", t(B, H, L - 1, d), ValueError),
])
def test_backward_refuses_outputs(key, bad, err):
    x = seq()
    with pytest.raises(err, match=key):
        sqa.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta"], x["lse"], x["dy"], window=w, alpha=0.5,
                            out={key: bad})


def test_backward_refuses_a_short_workspace():
    x = seq()
    with pytest.raises(ValueError, match="workspace"):
        sqa.lizard_attn_bwd(x["q"], x["k"], x["v"], x["log_g"], x["meta"], x["lse"], x["dy"], window=w, alpha=0.5,
                            workspace=torch.zeros(16, dtype=torch.uint8))


def test_logit_calls_take_logits_in_q_dtype():
    x = seq()
    with pytest.raises(TypeError, match="gate_logit"):
        sqa.lizard_attn_fwd_logit(x["q"], x["k"], x["v"], x["log_g"], x["meta"], window=w, alpha=0.5)
    with pytest.raises(TypeError, match="gate_logit"):
        sqa.lizard_attn_bwd_logit(x["q"], x["k"], x["v"], x["log_g"], x["meta"], x["lse"], x["dy"], window=w,
                                  alpha=0.5)


def decode_args():
    return dict(q=t(B, H, d), k=t(B, H, d), v=t(B, H, d), g=t(B, H, d, dtype=torch.float32), meta=t(H, m, d),
                state=t(B, H, d, d, dtype=torch.float32), kr=t(B, H, w, d), vr=t(B, H, w, d))


@pytest.mark.parametrize("name,bad,err,match", [
    ("state", t(B, H, d, d), TypeError, "state"),
    ("state", t(B, H, d, d - 1, dtype=torch.float32), ValueError, "state"),
    ("g", t(B, H, d), TypeError, "gates"),
    ("vr", t(B, H, w + 1, d), ValueError, "v_ring"),
    ("kr", t(B, H, w, d, dtype=torch.float32), TypeError, "k_ring"),
    ("k", t(B, H, d + 1), ValueError, "k"),
])
def test_decode_refuses(name, bad, err, match):
    x = decode_args()
    x[name] = bad
    with pytest.raises(err, match=match):
        sqa.lizard_decode_step(5, x["q"], x["k"], x["v"], x["g"], x["meta"], x["state"], x["kr"], x["vr"], alpha=0.5)


def test_decode_tokens_refuses():
    T = 3
    x = dict(q=t(B, H, T, d), k=t(B, H, T, d), v=t(B, H, T, d), g=t(B, H, T, d, dtype=torch.float32))
    dd = decode_args()
    with pytest.raises(ValueError, match="pos"):
        sqa.lizard_decode_tokens(torch.zeros(B, dtype=torch.int32), x["q"], x["k"], x["v"], x["g"], dd["meta"],
                                 dd["state"], dd["kr"], dd["vr"], alpha=0.5)
    with pytest.raises(ValueError, match="y"):
        sqa.lizard_decode_tokens(torch.zeros(B, dtype=torch.int64), x["q"], x["k"], x["v"], x["g"], dd["meta"],
                                 dd["state"], dd["kr"], dd["vr"], alpha=0.5, y=t(B, H, T + 1, d))


def test_continue_and_split_refuse():
    x = seq()
    for fn in (sqa.lizard_attn_fwd_continue, sqa.lizard_attn_fwd_split):
        with pytest.raises(ValueError, match="exactly one"):
            fn(x["q"], x["k"], x["v"], x["meta"], log_g=x["log_g"], gate_logit=x["q"], window=w, alpha=0.5)
        with pytest.raises(TypeError, match="state_in"):
            fn(x["q"], x["k"], x["v"], x["meta"], log_g=x["log_g"], state_in=t(B, H, d, d), window=w, alpha=0.5)
        with pytest.raises(ValueError, match="halo"):
            fn(x["q"], x["k"], x["v"], x["meta"], log_g=x["log_g"], k_halo=t(B, H, 5, d), window=w, alpha=0.5)
        with pytest.raises(ValueError, match="v_halo"):
            fn(x["q"], x["k"], x["v"], x["meta"], log_g=x["log_g"], k_halo=t(B, H, 5, d), v_halo=t(B, H, 4, d),
               window=w, alpha=0.5)


def test_training_pair_refuses():
    x = seq()
    nc = (L + 63) // 64
    with pytest.raises(TypeError, match="chunk_states"):
        sqa.lizard_attn_fwd_train(x["q"], x["k"], x["v"], x["meta"], log_g=x["log_g"], window=w, alpha=0.5,
                                  out={"chunk_states": t(B, H, nc, d, d, dtype=torch.float32)})
    with pytest.raises(ValueError, match="chunk_states"):
        sqa.lizard_attn_bwd_train(x["q"], x["k"], x["v"], x["meta"], x["lse"], t(B, H, nc + 1, d, d), x["dy"],
                                  log_g=x["log_g"], window=w, alpha=0.5)


def test_stage1_calls_refuse():
    x = seq()
    with pytest.raises(TypeError, match="v"):
        sqa.lizard_softmax_attn_fwd(x["q"], x["k"], t(B, H, L, d, dtype=torch.float32))
    with pytest.raises(TypeError, match="y_teacher"):
        sqa.lizard_transfer_loss(x["q"], t(B, H, L, d, dtype=torch.float32))
    with pytest.raises(ValueError, match="loss_bh"):
        sqa.lizard_transfer_loss(x["q"], x["k"], loss_bh=t(B, H + 1, dtype=torch.float32))
