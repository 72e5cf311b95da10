"""Counter-based random numbers and storage rounding for the synthetic inputs.

* splitmix64 is Sebastiano Vigna's 64-bit mixer (public domain, 2015): state
  advances by the golden-ratio increment 0x9E3779B97F4A7C15 and each output is
  the state passed through two xor-shift-multiply rounds and a final xor-shift.
  Here it is used counter-style: element i of a stream with seed s is
  mix(s + (i + 1) * increment), so any slice can be drawn independently.
* Uniforms take the top 53 bits and land in (0, 1] so that log(u) is finite.
* Gaussians use the Box-Muller transform (G. Box and M. Muller, 1958): a pair of
  uniforms (u1, u2) gives sqrt(-2 ln u1) * (cos 2 pi u2, sin 2 pi u2).
  numpy's normal generator is avoided on purpose so the recipe is fully stated.
* Drawn values are rounded to fp32, then (for bf16 storage) to bf16 with
  round-to-nearest-even; NaN maps to the quiet NaN 0x7FC0.
"""
import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1


def _mix(z):
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed, n):
    """n outputs of the splitmix64 stream whose initial state is `seed`."""
    with np.errstate(over="ignore"):
        ctr = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & _MASK64) + ctr * _GAMMA
        return _mix(z)


def _mix_scalar(x):
    x &= _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


# stream tags (top 16 bits of the sub-stream key)
TAGS = {"Q": 1, "K": 2, "V": 3, "K_STEP0": 4, "V_STEP0": 5, "PK": 6, "PV": 7, "X30": 8, "KSTAR": 9, "VSTAR": 10,
        "KH": 11, "VH": 12, "QM": 13, "QP": 14, "QKV": 15, "GQ": 16, "GK": 17,
        "DK": 18, "DV": 19, "DQ": 20, "DGK": 21, "DGV": 22, "DGQ": 23}


def substream_seed(base, tag, chunk=0, step=0, bank=0):
    """Seed of one named sub-stream: mix(base ^ tag<<48 ^ chunk<<16 ^ step<<8 ^ bank)."""
    key = (base ^ (TAGS[tag] << 48) ^ ((chunk & 0xFFFFFFFF) << 16) ^ ((step & 0xFF) << 8) ^ (bank & 0xFF)) & _MASK64
    return _mix_scalar((key + 0x9E3779B97F4A7C15) & _MASK64)


def uniform01(seed, n):
    """n doubles in (0, 1] from the top 53 bits of splitmix64 outputs."""
    z = splitmix64(seed, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)


def normal(seed, n):
    """n standard normal doubles by Box-Muller over consecutive uniform pairs."""
    m = (n + 1) // 2
    u = uniform01(seed, 2 * m)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = 2.0 * np.pi * u[1::2]
    out = np.empty(2 * m, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n]


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    nan = np.isnan(f)
    with np.errstate(over="ignore"):
        rounded = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), rounded)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
