// Definitions shared by the host side (C ABI, launch interface) and the kernels: plain
// C++ with no device code, so the host side also builds with an ordinary C++ compiler.
#pragma once

namespace zg {

constexpr int kMaxHalfRot = 64;  // rotary_dim / 2 <= 64 (d <= 128)
// Positions must be exact in fp32 (|p| < 2^24).
#define ZGATTN_POS_LIMIT (1 << 24)

// Per-pair RoPE phase step in revolutions per position, f_k = base^(-2k/r) / (2 pi),
// split into an fp32 head and tail (computed in double on the host) so that the phase
// p * f_k keeps ~44 significant bits for positions up to 2^24.
struct RopeFreq {
  float hi[kMaxHalfRot];
  float lo[kMaxHalfRot];
};

}  // namespace zg
