// fp16 matrix-core operands from quantised cache codes, shared by the decode and prefill
// kernels.  Both expansions are exact: each code lands under the fp16 exponent of 1024, so the
// operand is a constant offset plus the code, and the caller removes offset x (sum of the other
// operand) from the product sums.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef _Float16 qf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t qu32x4 __attribute__((ext_vector_type(4)));

// Eight int8 codes c -> eight fp16 values 1152 + c (exact).  Flipping the sign bit gives the
// byte u = c + 128; a byte permute then sets each u under the fp16 exponent of 1024, giving
// 1024 + u.  Three ALU ops per four codes; the caller takes the 1152 offset out of the sums.
__device__ __forceinline__ qf16x8 codes_to_f16(uint32_t x0, uint32_t x1) {
  constexpr uint32_t kExp = 0x64646464u;  // high byte of fp16 1024
  const uint32_t u0 = x0 ^ 0x80808080u, u1 = x1 ^ 0x80808080u;
  qu32x4 r;
  // v_perm_b32 picks result bytes from {src0 = bytes 4..7, src1 = bytes 0..3}
  r[0] = __builtin_amdgcn_perm(u0, kExp, 0x00050004u);  // {u.b0, 0x64, u.b1, 0x64}
  r[1] = __builtin_amdgcn_perm(u0, kExp, 0x00070006u);
  r[2] = __builtin_amdgcn_perm(u1, kExp, 0x00050004u);
  r[3] = __builtin_amdgcn_perm(u1, kExp, 0x00070006u);
  return __builtin_bit_cast(qf16x8, r);
}
constexpr float kCodeOffset = 1152.f;  // codes_to_f16(c) = kCodeOffset + c

// int4 cache: eight packed codes (elements 0..3 in the low nibbles of the four bytes, 4..7 in
// the high nibbles, each nibble c + 8) -> eight fp16 operands in six ALU ops.  A byte permute
// puts each byte (both of its nibbles) under the fp16 exponent of 1024, and two masks keep
// either the low nibble (1024 + n) or the high one in place (1024 + 16 n).  Elements 0..3 come
// out as kNibbleOffset + c, elements 4..7 as kNibbleOffsetHi16 + 16 c (exact); the caller
// divides the other operand's elements 4..7 by 16 (exact) and removes each half's offset.
__device__ __forceinline__ qf16x8 nibbles_to_f16_hi16(uint32_t x) {
  constexpr uint32_t kExp = 0x64646464u;
  const uint32_t p01 = __builtin_amdgcn_perm(x, kExp, 0x00050004u);  // {b0, 0x64, b1, 0x64}
  const uint32_t p23 = __builtin_amdgcn_perm(x, kExp, 0x00070006u);  // {b2, 0x64, b3, 0x64}
  qu32x4 r;
  r[0] = p01 & 0x640f640fu;  // elements 0, 1
  r[1] = p23 & 0x640f640fu;  // 2, 3
  r[2] = p01 & 0x64f064f0u;  // 4, 5, times 16
  r[3] = p23 & 0x64f064f0u;  // 6, 7, times 16
  return __builtin_bit_cast(qf16x8, r);
}
constexpr float kNibbleOffset = 1032.f;      // 1024 + (c + 8)
constexpr float kNibbleOffsetHi16 = 1152.f;  // 1024 + 16 (c + 8)

}  // namespace pa
