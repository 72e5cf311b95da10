"""The split schedule's key-tile cuts (kernels.hpp: piece_begin, split_pieces), checked on the
host for every item length up to the longest key list (1024 tiles) and a range of per-CU shares.

The library's own header is compiled with g++ into a small checker (no GPU): for each (T, share)
the pieces must cover the item's tiles [0, T) in order without gaps or overlaps, number at most
kMaxPieces with split_pieces counting the non-empty ones, start with a first piece of 85% of the
share (clamped to [1, T]), and continue by halving what is left while the half is at least
kMinPiece tiles, the last piece taking the rest; and the two c1 and c3 cuts the design notes
quote are reproduced exactly.
"""
import os
import subprocess

import pytest

import harness

CSRC = os.path.join(harness.ROOT, "chunk_causal_attention_amd", "csrc")

CHECKER = r'''
#include <cstdio>
#include "kernels.hpp"
using namespace sr;
static int fails = 0;
#define CHECK(c, T, S) do { if (!(c)) { if (fails++ < 10) std::printf("fail %s T=%d share=%d\n", #c, T, S); } } while (0)
int main() {
  for (int T = 1; T <= 1024; ++T) {
    for (int S = 1; S <= 1100; S += (S < 64 ? 1 : 7)) {
      CHECK(piece_begin(T, S, 0) == 0, T, S);
      CHECK(piece_begin(T, S, kMaxPieces) == T, T, S);
      CHECK(piece_begin(T, S, kMaxPieces + 3) == T, T, S);
      int p0 = S * 85 / 100;
      p0 = p0 < 1 ? 1 : (p0 > T ? T : p0);
      CHECK(piece_begin(T, S, 1) == p0, T, S);
      int nonempty = 0, last = -1;
      for (int k = 0; k < kMaxPieces; ++k) {
        const int b = piece_begin(T, S, k), e = piece_begin(T, S, k + 1);
        CHECK(b <= e && e <= T, T, S);
        if (e > b) { ++nonempty; last = k; }
      }
      CHECK(nonempty == split_pieces(T, S), T, S);
      CHECK(nonempty >= 1 && nonempty <= kMaxPieces, T, S);
      // pieces 1 .. last-1 are halves of what was left, each at least kMinPiece; nothing
      // empty before the last non-empty piece
      for (int k = 1; k < last; ++k) {
        const int b = piece_begin(T, S, k), e = piece_begin(T, S, k + 1);
        CHECK(e - b == (T - b) / 2 && e - b >= kMinPiece, T, S);
      }
      for (int k = 0; k < last; ++k) CHECK(piece_begin(T, S, k + 1) > piece_begin(T, S, k), T, S);
      // the last piece is the rest: either because halving it would go below kMinPiece, or
      // because the item already has kMaxPieces pieces
      if (last >= 1 && last < kMaxPieces - 1) {
        const int b = piece_begin(T, S, last);
        CHECK((T - b) / 2 < kMinPiece, T, S);
      }
    }
  }
  // the cuts of c1 (128 tiles, 100 split tiles per CU) and c3 (261 tiles, 139 per CU)
  const int c1[] = {0, 85, 106, 117, 128}, c3[] = {0, 118, 189, 225, 243, 252, 261};
  for (int k = 0; k < 5; ++k) CHECK(piece_begin(128, 100, k) == c1[k], 128, 100);
  for (int k = 0; k < 7; ++k) CHECK(piece_begin(261, 139, k) == c3[k], 261, 139);
  CHECK(split_pieces(128, 100) == 4 && split_pieces(261, 139) == 6, 0, 0);
  std::printf("fails %d\n", fails);
  return fails != 0;
}
'''


def test_piece_cuts(tmp_path):
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs the HIP headers")
    src = tmp_path / "cuts.cpp"
    src.write_text(CHECKER)
    exe = tmp_path / "cuts"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I", os.path.join(harness.ROOT, "include"), "-I", CSRC, str(src), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and "fails 0" in out.stdout, out.stdout + out.stderr
