"""Test-side utilities: BF16 bit conversions, decoding through torch's FP8 types, and an
exact (FP64, autograd) softmax attention on packed causal documents.  None of this is the
method: it is the independent side the oracle is pinned against."""
import numpy as np
import torch


def bf16_bits(x):
    """BF16 torch tensor -> numpy uint16 bit patterns."""
    return x.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f64(b):
    """numpy uint16 BF16 bits -> float64 numpy."""
    t = torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f16_bits_to_f64(b):
    return np.ascontiguousarray(b).view(np.float16).astype(np.float64)


def decode_e4m3(codes):
    """E4M3 codes -> float64 via torch's float8_e4m3fn type."""
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def dequant(codes, scales):
    """codes [T,H,d] u8, scales [H,T] u8 -> float64 [T,H,d]."""
    v = decode_e4m3(codes)
    e = scales.astype(np.int64).T[:, :, None] - 127
    return v * np.exp2(e.astype(np.float64))


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def dequant4(codes, scales):
    """4-bit copy -> float64 [T,H,d]: codes [T,H,d/2] u8 (even channel in the low nibble, E2M1
    per the OCP table), scales [H,T,d/32] u8 (one E8M0 byte per 32 channels)."""
    T, H, d2 = codes.shape
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(T, H, 2 * d2)
    e = np.repeat(scales.transpose(1, 0, 2).astype(np.int64) - 127, 32, axis=2)
    return _E2M1[nib] * np.exp2(e.astype(np.float64))


def exact_attention(q, k, v, cu, softmax_scale, do=None, causal=True):
    """Softmax attention per document (causal, or every key of the document), FP64, GQA by
    contiguous head groups.
    q [T,Hq,d], k, v [T,Hkv,d] (numpy float64).  Returns O, and (dQ, dK, dV, dS-per-doc)
    when the output gradient ``do`` is given."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=do is not None)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=do is not None)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=do is not None)
    outs = []
    s_list = []
    o = torch.zeros((T, Hq, d), dtype=torch.float64)
    pieces = []
    for a, b in zip(cu[:-1], cu[1:]):
        a, b = int(a), int(b)
        if b <= a:
            continue
        qq = qt[a:b].permute(1, 0, 2)                     # [Hq, L, d]
        kk = kt[a:b].permute(1, 0, 2).repeat_interleave(grp, 0)
        vv = vt[a:b].permute(1, 0, 2).repeat_interleave(grp, 0)
        s = softmax_scale * torch.matmul(qq, kk.transpose(1, 2).contiguous())
        if do is not None:
            s.retain_grad()
        L = b - a
        mask = torch.ones(L, L, dtype=torch.bool)
        if causal:
            mask = mask.tril()
        p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
        od = torch.matmul(p, vv).permute(1, 0, 2)
        pieces.append((a, b, od))
        s_list.append((a, b, s))
    rows = [torch.zeros((0, Hq, d), dtype=torch.float64)]
    cur = 0
    for a, b, od in pieces:
        if a > cur:
            rows.append(torch.zeros((a - cur, Hq, d), dtype=torch.float64))
        rows.append(od)
        cur = b
    if cur < T:
        rows.append(torch.zeros((T - cur, Hq, d), dtype=torch.float64))
    o = torch.cat(rows, 0)
    if do is None:
        return o.detach().numpy()
    o.backward(torch.tensor(do, dtype=torch.float64))
    ds = [(a, b, s.grad.numpy()) for a, b, s in s_list]
    return o.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), ds


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 or nb == 0:
        return 1.0 if na == nb else 0.0
    return float(a @ b / (na * nb))


def rms(a):
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0
