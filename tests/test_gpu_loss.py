"""The step's loss (Stack._lm_loss_backward): mean next-token cross-entropy of the frozen
lm_head and its gradient into the final hidden state, computed in one chunked pass over the
lm_head with a running softmax.

Checked against the plain definition in float64 (exact logits of the fp32 hidden state and
the bf16 lm_head), at a vocabulary that is not a whole number of chunks:
  * loss within 1e-4 relative, gradient within the parity bar (2e-2 RMS);
  * rows whose target holds almost all the probability (1 - softmax of the target between
    1e-30 and 1e-6), where the gradient is the small remainder sum_v p_v lm_v - lm_target:
    each such row within 2e-2 of its own RMS;
  * the gradient scales with the accumulation scale, the returned loss does not;
  * the streamed lm_head (pinned host memory, chunks through the device ring) gives the
    resident one's loss and gradient bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import assert_parity

pytestmark = pytest.mark.gpu
msq = pytest.importorskip("memory_streamed_qlora_amd")
from memory_streamed_qlora_amd import stack as S  # noqa: E402

VOCAB = 5000  # two chunks of 4224 rows, the second ragged
SHAPE = S.Shape(64, 2, 1, 32, 128, 1, vocab=VOCAB)
T = 96


def _stack(mode):
    return S.Stack.random(SHAPE, T, seed=5, r=4, alpha=8.0, mode=mode, n_slots=2, window_blocks=1)


def _lm(st):
    return (st.lm_host if st.lm_host is not None else st.lm.cpu()).float().numpy().astype(np.float64)


def _logits(hn, lm64):
    """float64 logits of the first T-1 rows (fp32 hidden state, bf16 lm_head: exact products)."""
    return hn[:-1].cpu().numpy().astype(np.float64) @ lm64.T


def _reference(hn, lm64, tokens):
    """float64 loss and d loss / d hn of the mean next-token cross-entropy over T-1 tokens."""
    h = hn.cpu().numpy().astype(np.float64)
    n = h.shape[0] - 1
    logits = _logits(hn, lm64)
    tgt = tokens[1:].cpu().numpy()
    rows = np.arange(n)
    mx = logits.max(1, keepdims=True)
    e = np.exp(logits - mx)
    Z = e.sum(1, keepdims=True)
    lse = (mx + np.log(Z))[:, 0]
    loss = float(np.mean(lse - logits[rows, tgt]))
    dl = e / Z
    # softmax of the target minus one, as minus the other rows' share summed on its own (a
    # difference Z - e_target would lose it below float64's 1e-16)
    other = e.copy()
    other[rows, tgt] = 0.0
    rest = other.sum(1) / Z[:, 0]
    dl[rows, tgt] = -rest
    dh = np.zeros_like(h)
    dh[:n] = dl @ lm64 / n
    return loss, dh, rest


def _run(st, hn0, tokens, scale=1.0):
    hn = hn0.clone().requires_grad_()
    loss = st._lm_loss_backward(hn, tokens, scale)
    torch.cuda.synchronize()
    assert hn.grad.dtype == torch.float32
    return loss.item(), hn.grad.cpu().numpy().astype(np.float64), hn.grad.clone()


def test_loss_and_gradient_against_the_definition():
    st = _stack("streamed")
    lm64 = _lm(st)
    g = torch.Generator(device="cpu").manual_seed(1)
    hn = (torch.randn(T, SHAPE.hidden, generator=g) * 2).cuda()
    tokens = torch.randint(0, VOCAB, (T,), generator=g)
    loss, dh, _ = _run(st, hn, tokens)
    rloss, rdh, _ = _reference(hn, lm64, tokens)
    print(f"[loss] {loss:.6f} vs {rloss:.6f}", flush=True)
    assert abs(loss - rloss) <= 1e-4 * abs(rloss)
    assert_parity(dh, rdh, name="d hn")
    # the accumulation scale reaches the gradient only
    loss2, dh2, _ = _run(st, hn, tokens, scale=0.25)
    assert loss2 == loss
    assert_parity(dh2, 0.25 * rdh, name="d hn, scale 0.25")
    st.close()


def test_confident_rows():
    """Large logits, half the targets at each row's argmax: their softmax is 1 - 1e-6 or
    closer, and their gradient is the small remainder sum_v p_v lm_v - lm_target."""
    st = _stack("streamed")
    lm64 = _lm(st)
    g = torch.Generator(device="cpu").manual_seed(2)
    h = torch.randn(T, SHAPE.hidden, generator=g)
    h = h / h.norm(dim=1, keepdim=True) * 5e3  # logits with a standard deviation ~100
    hn = h.cuda()
    n = T - 1
    logits = _logits(hn, lm64)
    tokens = torch.randint(0, VOCAB, (T,), generator=g)
    conf = np.arange(n) % 2 == 0
    tokens[1:][torch.from_numpy(conf)] = torch.from_numpy(logits.argmax(1)[conf])
    loss, dh, _ = _run(st, hn, tokens)
    rloss, rdh, rest = _reference(hn, lm64, tokens)
    assert abs(loss - rloss) <= 1e-4 * abs(rloss) + 1e-6
    sharp = conf & (rest < 1e-6) & (rest > 1e-30)
    print(f"[loss] confident rows with 1e-30 < 1 - p_target < 1e-6: {int(sharp.sum())}", flush=True)
    assert sharp.sum() >= 8
    for t in np.nonzero(sharp)[0]:
        r = np.sqrt(np.mean(rdh[t] ** 2))
        assert np.max(np.abs(dh[t] - rdh[t])) <= 2e-2 * r + 1e-30, f"row {t}"
    assert_parity(dh, rdh, name="d hn")
    st.close()


def test_streamed_lm_head_equals_resident_bitwise():
    g = torch.Generator(device="cpu").manual_seed(3)
    hn = (torch.randn(T, SHAPE.hidden, generator=g) * 2).cuda()
    tokens = torch.randint(0, VOCAB, (T,), generator=g)
    outs = []
    for mode in ("resident", "streamed"):
        st = _stack(mode)
        assert (st.lm_host is not None) == (mode == "streamed")
        loss, _, grad = _run(st, hn, tokens)
        outs.append((loss, grad))
        st.close()
    assert outs[0][0] == outs[1][0]
    assert torch.equal(outs[0][1], outs[1][1])
