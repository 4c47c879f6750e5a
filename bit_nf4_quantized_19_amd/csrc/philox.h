// Counter-based random bits for LoRA dropout: Philox4x32 with 10 rounds
// (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC'11). Each round multiplies words 0 and 2 by two constants (full
// 64-bit products), mixes the high halves with words 1 and 3 and the key;
// the key is bumped by two Weyl constants between rounds.
//
// Dropout mask (LLM tutorial ch. 3, 3.3 and Day-25 notes 4.3: lora_dropout
// on the adapter input): element e = m * k + c of X (M x k) keeps when word
// e % 4 of philox(counter = (e / 4 low, e / 4 high, 0, 0), key = seed) is
// >= floor(p * 2^32).
#pragma once

#include "common.h"

struct DropParams {
  uint32_t k0, k1;     // seed (low, high word)
  uint32_t thr;        // floor(p * 2^32)
  float inv_keep;      // fl32(1 / (1 - p))
  int on;              // p > 0
  int mask_write;      // 1: the kernel that draws the bits also stores them in mask
  uint8_t *mask;       // keep bits stored between forward and backward (one nibble per
                       // four elements: byte (m*C + c)/4, bit c%4), or NULL
};

QL_DEV uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
    const uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Keep bits of elements e .. e+3 (e a multiple of 4): bit j for element e+j.
QL_DEV uint32_t keep4(const DropParams &dp, uint64_t e) {
  const uint64_t b = e >> 2;
  const uint4 r = philox4x32_10(make_uint4((uint32_t)b, (uint32_t)(b >> 32), 0u, 0u), dp.k0, dp.k1);
  return (r.x >= dp.thr ? 1u : 0u) | (r.y >= dp.thr ? 2u : 0u) | (r.z >= dp.thr ? 4u : 0u) |
         (r.w >= dp.thr ? 8u : 0u);
}

// Zero the dropped bf16 elements of 8 consecutive ones (bits 0-7 of keep).
QL_DEV uint4 mask_bf16x8(uint4 v, uint32_t keep) {
  const auto m2 = [](uint32_t w, uint32_t k2) {
    return (w & ((k2 & 1u) ? 0x0000FFFFu : 0u)) | (w & ((k2 & 2u) ? 0xFFFF0000u : 0u));
  };
  return make_uint4(m2(v.x, keep), m2(v.y, keep >> 2), m2(v.z, keep >> 4), m2(v.w, keep >> 6));
}
