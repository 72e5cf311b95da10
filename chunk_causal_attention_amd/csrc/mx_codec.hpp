// bf16 -> MXFP6 / FP8 encoders and their decoders, in integer arithmetic.
//
// Reduced-precision video attention ("The road to the fastest, cheapest H3", Accelerating the
// denoiser, item 2) takes MXFP6 queries and keys and FP8 values.  Formats (OCP Microscaling
// specification v1.0):
//   E2M3 (FP6): sign | 2 exponent bits, bias 1 | 3 mantissa bits; largest 7.5, no inf/NaN.
//   E4M3 (FP8): sign | 4 exponent bits, bias 7 | 3 mantissa bits; largest 448, S.1111.111 NaN.
//   MXFP6: 32 consecutive elements share the scale 2^X, stored as the E8M0 byte X + 127, with
//   X = floor(log2 max|x|) - 2 clamped to >= -127 (bf16 inputs keep X <= 125).
// Rounding: nearest, ties to the even mantissa, saturating at the largest value; the sign bit
// is the input's.  Inputs must be finite.
//
// A bf16 magnitude is M * 2^F with an integer significand M (128 + mantissa, or the mantissa
// alone for subnormals).  In a binade be of the target format (counted from its smallest
// normal binade, 0 for subnormals) the representable values are spaced 2^(qexp) with
// qexp = (smallest normal exponent + be) - 3, so the rounded value is n * 2^qexp with
// n = rne(M / 2^(qexp - F)) in [8, 16] (normal) or [0, 8] (subnormal), and its code is
// be * 8 + n: n = 16 carries into the next binade and n = 8 out of the subnormals, exactly
// as the codes are laid out.  Every step is exact, so the codes are bit-identical wherever
// these functions run (append, in-kernel query quantization, host tools).
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define SR_HD __host__ __device__ __forceinline__
#else
#define SR_HD inline
#endif

namespace sr {
namespace mx {

constexpr int kBlock = 32;       // elements per MXFP6 scale block
constexpr int kE2m3Max = 31;     // code of 7.5
constexpr int kE4m3Max = 0x7E;   // code of 448
constexpr int kScaleMin = -127;

struct Mag {
  int M;   // integer significand
  int F;   // value = M * 2^F
  int Ex;  // floor(log2 value); meaningless when M == 0
};

SR_HD int top_bit(unsigned v) { return 31 - __builtin_clz(v); }

// |x| of a bf16 bit pattern (sign ignored).
SR_HD Mag bf16_mag(unsigned x) {
  const int e = int((x >> 7) & 0xFFu), m = int(x & 0x7Fu);
  if (e) return Mag{128 | m, e - 134, e - 127};
  return Mag{m, -133, m ? top_bit(unsigned(m)) - 133 : 0};
}

// Round M / 2^sh to the nearest integer, ties to even (sh >= 1, M < 2^8).
SR_HD int rne_shift(int M, int sh) {
  if (sh > 9) return 0;
  return (M + (1 << (sh - 1)) - 1 + ((M >> sh) & 1)) >> sh;
}

// Block exponent X of 32 bf16 values.
SR_HD int block_exponent(const unsigned* x) {
  unsigned amax = 0;
  for (int e = 0; e < kBlock; ++e) {
    const unsigned a = x[e] & 0x7FFFu;
    amax = a > amax ? a : amax;
  }
  if (!amax) return kScaleMin;
  const int X = bf16_mag(amax).Ex - 2;
  return X < kScaleMin ? kScaleMin : X;
}

// E2M3 code (6 bits) of x / 2^X.
SR_HD unsigned e2m3_code(unsigned x, int X) {
  const Mag v = bf16_mag(x & 0x7FFFu);
  int code = 0;
  if (v.M) {
    const int be = v.Ex - X > 0 ? v.Ex - X : 0;  // E2M3 binade, 0 = subnormals / [1, 2)
    const int qexp = X + be - 3;
    code = be * 8 + rne_shift(v.M, qexp - v.F);
    code = code > kE2m3Max ? kE2m3Max : code;
  }
  return unsigned(code) | ((x >> 15) & 1u) << 5;
}

// E4M3 code (8 bits) of x.
SR_HD unsigned e4m3_code(unsigned x) {
  const Mag v = bf16_mag(x & 0x7FFFu);
  int code = 0;
  if (v.M) {
    const int be = v.Ex + 6 > 0 ? v.Ex + 6 : 0;  // E4M3 binade counted from 2^-6
    const int qexp = be - 9;
    code = be * 8 + rne_shift(v.M, qexp - v.F);
    code = code > kE4m3Max ? kE4m3Max : code;
  }
  return unsigned(code) | ((x >> 15) & 1u) << 7;
}

// Quantizes one block: packs the 32 E2M3 codes little-endian, 6 bits each (element e at bits
// 6e .. 6e+5 of w[0..5]), and returns X.
SR_HD int quantize_block(const unsigned* x, unsigned* w) {
  const int X = block_exponent(x);
  for (int i = 0; i < 6; ++i) w[i] = 0;
  for (int e = 0; e < kBlock; ++e) {
    const unsigned c = e2m3_code(x[e], X);
    const int bit = 6 * e, word = bit >> 5, sh = bit & 31;
    w[word] |= c << sh;
    if (sh > 26) w[word + 1] |= c >> (32 - sh);
  }
  return X;
}

// bf16 bit pattern of M * 2^E (M < 16, exactly representable: the decoders below only make
// such values).
SR_HD unsigned bf16_of(int M, int E) {
  if (!M) return 0;
  const int p = top_bit(unsigned(M));
  const int ef = p + E + 127;  // biased exponent of the value
  if (ef >= 1) return unsigned(ef) << 7 | ((unsigned(M) << (7 - p)) & 0x7Fu);
  return unsigned(M) << (E + 133);  // subnormal: M * 2^E = (M << (E + 133)) * 2^-133
}

// Value of an E2M3 code times 2^X, as bf16 bits.
SR_HD unsigned e2m3_to_bf16(unsigned code, int X) {
  const int c = int(code & 31u);
  const unsigned s = (code >> 5 & 1u) << 15;
  if (c < 8) return s | bf16_of(c, X - 3);
  return s | bf16_of(8 + (c & 7), X + (c >> 3) - 4);
}

// Value of an E4M3 code (never NaN here), as bf16 bits.
SR_HD unsigned e4m3_to_bf16(unsigned code) {
  const int c = int(code & 0x7Fu);
  const unsigned s = (code >> 7 & 1u) << 15;
  if (c < 8) return s | bf16_of(c, -9);
  return s | bf16_of(8 + (c & 7), (c >> 3) - 10);
}

}  // namespace mx
}  // namespace sr
