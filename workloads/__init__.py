"""Seeded synthetic inputs shaped like video-VAE decoder workloads.

This module only draws random numbers and names shapes.  It holds none of the
convolution or normalisation arithmetic, so both the HIP path and the oracle
may use it without sharing any of the method.

Recipe (one numpy PCG64 stream per tensor):
  * workload k uses ``numpy.random.SeedSequence(1000 + k)``, spawned into one
    child per tensor in a fixed order (x, then per layer gamma, beta, w, b);
  * activations ~ N(0, 1), drawn as float32 and rounded once to fp16 (RNE);
  * weights ~ U(-a, a) drawn in float64, rounded once to fp16, with
    a = 1/sqrt(27*Cin) for the small zero-padded workload and the
    Kaiming-uniform bound a = sqrt(6 / fan_in), fan_in = kt*kh*kw*Cin, elsewhere;
  * biases ~ N(0, 0.1) for the small workload and N(0, 0.02) elsewhere;
  * GroupNorm gamma ~ N(1, 0.1), beta ~ N(0, 0.1);
  * the channel-changing workload scales round(1% of Cin) = 5 of 512 input
    channels, picked by a seeded permutation, by 50 before the fp16 cast.

Layouts: activations NDHWC [N, T, H, W, C]; weights [Cout, kt, kh, kw, Cin].
"""
from __future__ import annotations

import concurrent.futures
import os
from dataclasses import dataclass, replace

import numpy as np

TPAD_ZERO = 0
TPAD_REPLICATE = 1


@dataclass(frozen=True)
class ConvShape:
    """Input-side description of one stride-1 conv3d (padding is given, not derived)."""
    n: int
    t: int
    h: int
    w: int
    cin: int
    cout: int
    kt: int = 3
    kh: int = 3
    kw: int = 3
    pad_t_front: int = 2
    pad_t_back: int = 0
    pad_h: int = 1
    pad_w: int = 1
    tmode: int = TPAD_REPLICATE

    @property
    def pads(self):
        return (self.pad_t_front, self.pad_t_back, self.pad_h, self.pad_w)

    @property
    def x_shape(self):
        return (self.n, self.t, self.h, self.w, self.cin)

    @property
    def w_shape(self):
        return (self.cout, self.kt, self.kh, self.kw, self.cin)


# The five workloads.  Index k below is the workload number used for seeding.
SMALL_ZERO = ConvShape(1, 5, 16, 16, 32, 32, pad_t_front=1, pad_t_back=1, tmode=TPAD_ZERO)
CAUSAL_512 = ConvShape(1, 9, 64, 64, 512, 512)
CAUSAL_256 = ConvShape(1, 17, 128, 128, 256, 256)
CAUSAL_256_T1 = replace(CAUSAL_256, t=1)
STAGE_3X3 = ConvShape(1, 33, 256, 256, 512, 256)
STAGE_1X1 = ConvShape(1, 33, 256, 256, 256, 128, kt=1, kh=1, kw=1, pad_t_front=0, pad_t_back=0,
                      pad_h=0, pad_w=0, tmode=TPAD_ZERO)
BLOCK_CONV = ConvShape(1, 17, 128, 128, 256, 256)
BLOCK_GROUPS = 32
BLOCK_EPS = 1e-6

WORKLOADS = {
    0: "conv3d 3x3x3 zero-pad, N=1 T=5 H=W=16 Cin=Cout=32",
    1: "causal conv3d 3x3x3, N=1 T=9 H=W=64 Cin=Cout=512",
    2: "causal conv3d 3x3x3, N=1 T=17 H=W=128 Cin=Cout=256 (and T=1)",
    3: "causal conv3d 3x3x3 512->256 + conv3d 1x1x1 256->128, N=1 T=33 H=W=256",
    4: "3D ResNet decoder block GN(32)+SiLU -> causal conv -> GN+SiLU -> causal conv -> +x, "
       "N=1 C=256 T=17 H=W=128",
}


def kaiming_bound(shape: ConvShape) -> float:
    return float(np.sqrt(6.0 / (shape.kt * shape.kh * shape.kw * shape.cin)))


def _seeds(seed: int, count: int):
    return np.random.SeedSequence(seed).spawn(count)


def _gen(ss):
    return np.random.Generator(np.random.PCG64(ss))


CHUNK = 1 << 24  # elements per independently seeded chunk of an activation tensor


def _fill_chunks(flat, ss, draw):
    """Fill flat[k*CHUNK:(k+1)*CHUNK] from child seed k of ss, in a thread pool.

    The values depend only on ss and the chunk index, never on the thread
    count (numpy's Generator releases the GIL while it fills).
    """
    nchunks = (flat.size + CHUNK - 1) // CHUNK
    kids = ss.spawn(nchunks)

    def one(k):
        s, e = k * CHUNK, min(flat.size, (k + 1) * CHUNK)
        flat[s:e] = draw(_gen(kids[k]), s, e)

    if nchunks == 1:
        one(0)
    else:
        workers = min(nchunks, max(1, min(16, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(nchunks)))


def to_bf16(a):
    """float32 values -> bf16 storage (uint16 bits), rounded once to nearest even.

    Finite inputs only (the generators here draw finite values).  bf16 is the
    upper half of an IEEE binary32, so rounding adds half an ulp of the kept
    part (one less on an even tie) before truncating the lower 16 bits.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def _store(v, dtype):
    """float32 draws -> the storage of dtype ("f16": float16, "bf16": uint16 bits)."""
    return to_bf16(v) if dtype == "bf16" else v.astype(np.float16)


def _storage(dtype):
    return np.uint16 if dtype == "bf16" else np.float16


def normal_f16(ss, shape, mean=0.0, std=1.0, channel_scale=None, dtype="f16"):
    """N(mean, std) drawn as float32, optionally scaled per channel (last axis), rounded once to fp16.

    dtype="bf16" rounds the same draws to bf16 instead (uint16 bits).
    """
    out = np.empty(shape, _storage(dtype))
    flat = out.reshape(-1)
    c = shape[-1]

    def draw(g, s, e):
        v = g.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        if channel_scale is not None:
            # chunk starts are multiples of CHUNK, itself a multiple of c (c divides 2^24 here)
            v.reshape(-1, c)[:, channel_scale[0]] *= np.float32(channel_scale[1])
        return _store(v, dtype)

    if channel_scale is not None and CHUNK % c:
        raise ValueError("channel count must divide the chunk size")
    _fill_chunks(flat, ss, draw)
    return out


def ternary_f16(ss, shape, dtype="f16"):
    """Values drawn uniformly from {-1, 0, 1}, in chunks (multi-GB tensors need no wide temporary)."""
    out = np.empty(shape, _storage(dtype))
    _fill_chunks(out.reshape(-1), ss,
                 lambda g, s, e: _store(g.integers(-1, 2, e - s, dtype=np.int8).astype(np.float32), dtype))
    return out


def uniform_f16(ss, shape, bound, dtype="f16"):
    return _store(_gen(ss).uniform(-bound, bound, size=shape).astype(np.float32), dtype)


def conv_inputs(shape: ConvShape, seed: int, w_bound=None, b_std=0.02, with_bias=True,
                hot_channels=0, hot_scale=50.0, dtype="f16"):
    """x, w, b (fp16 numpy; bf16 bits as uint16 with dtype="bf16") for one conv.

    ``hot_channels`` input channels are scaled by hot_scale.
    """
    sx, sw, sb, sp = _seeds(seed, 4)
    if w_bound is None:
        w_bound = kaiming_bound(shape)
    scale = None
    if hot_channels:
        hot = np.sort(_gen(sp).permutation(shape.cin)[:hot_channels])
        scale = (hot, hot_scale)
    x = normal_f16(sx, shape.x_shape, channel_scale=scale, dtype=dtype)
    w = uniform_f16(sw, shape.w_shape, w_bound, dtype)
    b = normal_f16(sb, (shape.cout,), 0.0, b_std, dtype=dtype) if with_bias else None
    return {"x": x, "w": w, "b": b}


def workload_inputs(k: int):
    """Inputs of workload k (0..4) as fp16 numpy arrays, seeded SeedSequence(1000+k)."""
    seed = 1000 + k
    if k == 0:
        s = SMALL_ZERO
        return dict(shape=s, **conv_inputs(s, seed, w_bound=1.0 / np.sqrt(27 * s.cin), b_std=0.1))
    if k == 1:
        return dict(shape=CAUSAL_512, **conv_inputs(CAUSAL_512, seed))
    if k == 2:
        return dict(shape=CAUSAL_256, **conv_inputs(CAUSAL_256, seed))
    if k == 3:
        st1 = conv_inputs(STAGE_3X3, seed, hot_channels=5)
        st2 = conv_inputs(STAGE_1X1, seed + 100)
        return {"shape": STAGE_3X3, "x": st1["x"], "w": st1["w"], "b": st1["b"],
                "shape2": STAGE_1X1, "w2": st2["w"], "b2": st2["b"]}
    if k == 4:
        return block_inputs(BLOCK_CONV, seed)
    raise KeyError(k)


def block_inputs(shape: ConvShape, seed: int, dtype="f16"):
    """Decoder-block tensors in the order x, gamma1, beta1, w1, b1, gamma2, beta2, w2, b2."""
    r = _seeds(seed, 9)
    c = shape.cin
    bound = kaiming_bound(shape)
    return {
        "shape": shape,
        "x": normal_f16(r[0], shape.x_shape, dtype=dtype),
        "gamma1": normal_f16(r[1], (c,), 1.0, 0.1, dtype=dtype),
        "beta1": normal_f16(r[2], (c,), 0.0, 0.1, dtype=dtype),
        "w1": uniform_f16(r[3], shape.w_shape, bound, dtype),
        "b1": normal_f16(r[4], (shape.cout,), 0.0, 0.02, dtype=dtype),
        "gamma2": normal_f16(r[5], (c,), 1.0, 0.1, dtype=dtype),
        "beta2": normal_f16(r[6], (c,), 0.0, 0.1, dtype=dtype),
        "w2": uniform_f16(r[7], shape.w_shape, bound, dtype),
        "b2": normal_f16(r[8], (shape.cout,), 0.0, 0.02, dtype=dtype),
        "groups": BLOCK_GROUPS,
        "eps": BLOCK_EPS,
    }


def gn_inputs(n: int, thw_shape, c: int, seed: int, mean=0.0, std=1.0, dtype="f16"):
    """x [n, *thw_shape, c] ~ N(mean, std), gamma ~ N(1, 0.1), beta ~ N(0, 0.1), all fp16 (or bf16)."""
    sx, sg, sb = _seeds(seed, 3)
    x = normal_f16(sx, (n,) + tuple(thw_shape) + (c,), mean, std, dtype=dtype)
    return {"x": x, "gamma": normal_f16(sg, (c,), 1.0, 0.1, dtype=dtype),
            "beta": normal_f16(sb, (c,), 0.0, 0.1, dtype=dtype)}
