"""Counter-based synthetic value streams (host side, NumPy).

Every large synthetic array (KV history, per-step q / k / v candidates, recall
head weights, hidden states) is a pure function of (stream key, element index),
so any slice can be regenerated on the host without generating the rest, and
the device fill kernels in ``synth/csrc/synth.hip`` produce the same bits.

Definition (both sides implement exactly this):

* SplitMix64 output for counter i under key k (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
      z = k + (i + 1) * 0x9E3779B97F4A7C15            (mod 2^64)
      z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
      z = (z ^ (z >> 27)) * 0x94D049BB133111EB
      r = z ^ (z >> 31)
* Approximately standard normal value (Irwin-Hall sum of four uniforms):
      c = sum of the four 16-bit fields of r  - 131070      (exact integer)
      x = float32(c) * float32(scale)                       (one IEEE rounding)
  with scale = sigma / sqrt(4 * (65536^2 - 1) / 12). The sum has mean 0,
  variance sigma^2 and support |x| <= 3.46 sigma.
* bf16 values are x rounded to nearest-even on the upper 16 bits.

This module holds none of the decode method's arithmetic: it only makes inputs.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
IH4_SD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)


def splitmix64_scalar(key, i):
    """Reference SplitMix64 output for counter i (Python integers)."""
    z = (key + (i + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * M1) & MASK64
    z = ((z ^ (z >> 27)) * M2) & MASK64
    return z ^ (z >> 31)


def mix_key(*ids):
    """Stream key from a tuple of small integers (config, component, sub-id...)."""
    k = 0x243F6A8885A308D3
    for v in ids:
        k = splitmix64_scalar(k ^ (int(v) & MASK64), 0)
    return k


def unit_scale(sigma=1.0):
    """float32 factor that maps the centred Irwin-Hall sum to standard deviation sigma."""
    return np.float32(sigma / IH4_SD)


def _raw(key, start, count):
    i = np.arange(start + 1, start + 1 + count, dtype=np.uint64)
    z = i * np.uint64(GAMMA)
    z += np.uint64(key)
    t = z >> np.uint64(30)
    z ^= t
    z *= np.uint64(M1)
    t = z >> np.uint64(27)
    z ^= t
    z *= np.uint64(M2)
    t = z >> np.uint64(31)
    z ^= t
    return z


def _normal_chunk(key, start, count, scale):
    z = _raw(key, start, count)
    m = np.uint64(0xFFFF)
    s = (z & m).astype(np.int64)
    s += ((z >> np.uint64(16)) & m).astype(np.int64)
    s += ((z >> np.uint64(32)) & m).astype(np.int64)
    s += (z >> np.uint64(48)).astype(np.int64)
    s -= 131070
    x = s.astype(np.float32)
    x *= np.float32(scale)
    return x


def f32_to_bf16_bits(x):
    """Round-to-nearest-even of float32 values to bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 22


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def _fill(key, start, count, scale, out, conv):
    starts = list(range(0, count, _CHUNK))

    def work(c0):
        n = min(_CHUNK, count - c0)
        out[c0:c0 + n] = conv(_normal_chunk(key, start + c0, n, scale))

    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out


def normal_f32(key, start, count, scale):
    """float32 values for element indices start .. start+count-1 of stream `key`."""
    out = np.empty(count, dtype=np.float32)
    return _fill(key, start, count, scale, out, lambda x: x)


def normal_bf16(key, start, count, scale):
    """bf16 bit patterns (uint16) for element indices start .. start+count-1."""
    out = np.empty(count, dtype=np.uint16)
    return _fill(key, start, count, scale, out, f32_to_bf16_bits)
