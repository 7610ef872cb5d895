"""Shared test helpers: moving seeded bf16 inputs to the GPU and the numeric
gate used for every GPU-vs-oracle comparison."""
from __future__ import annotations

import numpy as np

from masked_gqa_attention_action_amd import synth

# Gate for floating-point outputs (bf16 storage, fp32 accumulation):
# max |err| <= 2e-2 * RMS(oracle output) and cosine >= 0.9995.
ERR_REL_RMS = 2e-2
MIN_COS = 0.9995
# Branch check of a whole layer (out - x, beyond the output gate): the branch
# passes through five bf16 roundings of intermediates (xn1, q/k/v, ctx, xn2,
# h), each up to 2^-9 relative per element; their sum bounds the branch error
# at about 5 * 2^-9 ~ 1e-2 of a branch element, and branch elements reach
# ~4-5x the branch RMS, so the bound is 5e-2 of the branch RMS.
LAYER_BRANCH_REL = 5e-2


def to_dev(bits, dtype="bf16"):
    import torch
    a = np.ascontiguousarray(bits)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def f64(bits) -> np.ndarray:
    return synth.bf16_to_f64(bits)


def gate(name, got, ref, rel=ERR_REL_RMS, min_cos=MIN_COS):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref)))
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    msg = f"{name}: max|err|={err:.3e} rms={rms:.3e} ratio={err / max(rms, 1e-300):.3e} cos={cos:.7f}"
    print(msg, flush=True)
    assert err <= rel * rms, msg
    assert cos >= min_cos, msg
    return err / max(rms, 1e-300), cos


def stage_gate(name, got, ref, rel=ERR_REL_RMS, min_cos=MIN_COS, roundings=1):
    """Gate for a single stage whose output is stored as bf16: the layer gate
    plus one bf16 rounding of the output, element by element:
    |err_i| <= rel * RMS(ref) + roundings * 2^-8 * |ref_i|, and cosine >=
    min_cos.  roundings > 1 where the path stores the value in bf16 that many
    times on its way out (a split partial, then the merged output)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(got - ref)
    excess = float(np.max(err - roundings * 2.0 ** -8 * np.abs(ref)))
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
    msg = (f"{name}: max|err|={float(err.max()):.3e} rms={rms:.3e} "
           f"max(|err|-{roundings}*2^-8|ref|)/rms={excess / max(rms, 1e-300):.3e} cos={cos:.7f}")
    print(msg, flush=True)
    assert excess <= rel * rms, msg
    assert cos >= min_cos, msg


def delta_gate(name, got_out, ref_out, base, rel=ERR_REL_RMS, min_cos=0.999):
    """Gate on the branch a residual block adds (out - base), so the residual
    cannot hide an error in it.  The stored output carries one bf16 rounding:
    |err_i| <= rel * RMS(ref_out - base) + 2^-8 * |ref_out_i|; the branch
    itself must have cosine >= min_cos."""
    got_out = np.asarray(got_out, dtype=np.float64).ravel()
    ref_out = np.asarray(ref_out, dtype=np.float64).ravel()
    base = np.asarray(base, dtype=np.float64).ravel()
    d_ref, d_got = ref_out - base, got_out - base
    rms = float(np.sqrt(np.mean(d_ref * d_ref)))
    excess = float(np.max(np.abs(got_out - ref_out) - 2.0 ** -8 * np.abs(ref_out)))
    cos = float(d_got @ d_ref / (np.linalg.norm(d_got) * np.linalg.norm(d_ref) + 1e-300))
    msg = f"{name}: branch rms={rms:.3e} max(|err|-2^-8|out|)/rms={excess / max(rms, 1e-300):.3e} cos={cos:.7f}"
    print(msg, flush=True)
    assert excess <= rel * rms, msg
    assert cos >= min_cos, msg


def to_dev_w(bits):
    """A weight matrix on the device in the library's tiled layout."""
    import masked_gqa_attention_action_amd as dmx
    return dmx.pack_weight(to_dev(bits))


def device_weights(wbits: dict) -> dict:
    """Layer weights on the device: matrices tiled, vectors plain."""
    import masked_gqa_attention_action_amd as dmx
    return dmx.pack_layer_weights({k: to_dev(v) for k, v in wbits.items()})


def oracle_weights(wbits: dict) -> dict:
    return {k: f64(v) for k, v in wbits.items()}


def untile(flat_bits, rows, cols, dtype="bf16"):
    """Row-major [rows][cols] float64 copy of a tiled activation buffer.

    Tiled layout of the library (16 x 32 tiles of 512 elements): tile (rt, kt)
    starts at element (rt * cols/32 + kt) * 512; inside it, the 8-element
    chunk of row rt*16 + r, columns kt*32 + 8g .. +7 sits at (r + 16 g) * 8.
    flat_bits: numpy uint16 (bf16 bits) of at least rows * cols elements."""
    assert rows % 16 == 0 and cols % 32 == 0
    a = np.asarray(flat_bits)[: rows * cols].reshape(rows // 16, cols // 32, 4, 16, 8)  # rt, kt, g, r, e
    a = a.transpose(0, 3, 1, 2, 4).reshape(rows, cols)  # rt, r, kt, g, e
    if dtype == "bf16":
        return synth.bf16_to_f64(np.ascontiguousarray(a))
    return a.astype(np.float64)


def dev_bits(t) -> np.ndarray:
    """The raw bytes of a device tensor as numpy uint16 (bf16 bit patterns)."""
    import torch
    return t.detach().view(torch.uint8).cpu().numpy().view(np.uint16)
