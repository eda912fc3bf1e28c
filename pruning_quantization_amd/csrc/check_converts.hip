// Exhaustive check that gfx950's hardware conversions used by the kernels
// (v_cvt_pk_fp8_f32, v_cvt_scalef32_pk_fp4_f32 at scale 1, v_cvt_f32_fp8,
// v_cvt_scalef32_pk_f32_fp4 at scale 1) give exactly the codes of the exact
// integer encoders enc_e4m3 / enc_e2m1 (round to nearest even, saturating,
// sign copied) for every finite fp32 input, that decoding every e4m3 code
// matches dec_e4m3 (one code per instruction, and two per instruction from
// either half of a dword: v_cvt_pk_f32_fp8), and that decoding every byte of
// E2M1 pairs, from each byte position of a dword, matches dec_e2m1.
// Every store goes to cnt[0..6] or slots[0..63], guarded by the slot index;
// the grid-stride loop is bounded by 2^32.  Exit status 0 = no mismatch.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>
#include "device_common.hpp"
using namespace sparq24;

__global__ void probe(unsigned long long* cnt, unsigned* slots) {
  const unsigned long long n = 1ull << 32;
  unsigned long long loc[4] = {0, 0, 0, 0};
  for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (unsigned long long)gridDim.x * blockDim.x) {
    const unsigned u = (unsigned)i;
    const float x = __uint_as_float(u);
    if (!__builtin_isfinite(x)) continue;
    // fp8: clamp then hardware convert (operand a -> byte 0)
    const float y = __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
    const unsigned hw8 = __builtin_amdgcn_cvt_pk_fp8_f32(y, -y, 0u, false);
    const unsigned sw8 = enc_e4m3(x);
    const unsigned sw8n = enc_e4m3(-y);
    if ((hw8 & 0xFFu) != sw8 || ((hw8 >> 8) & 0xFFu) != sw8n) {
      if (loc[0]++ == 0) { unsigned long long k = atomicAdd(&cnt[0], 1ull); if (k < 16) slots[0 + k] = u; }
    }
    // fp4 scaled convert, scale 1: a -> low nibble?, b -> high nibble?
    const unsigned hw4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, -x, 1.0f, 0);
    const unsigned sw4 = enc_e2m1(x) | (enc_e2m1(-x) << 4);
    if ((hw4 & 0xFFu) != sw4) {
      if (loc[1]++ == 0) { unsigned long long k = atomicAdd(&cnt[1], 1ull); if (k < 16) slots[16 + k] = u; }
    }
    // fp4 with clamp to +-6 first
    const float z = __builtin_fminf(__builtin_fmaxf(x, -6.0f), 6.0f);
    const unsigned hw4c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, z, -z, 1.0f, 0);
    if ((hw4c & 0xFFu) != sw4) {
      if (loc[2]++ == 0) { unsigned long long k = atomicAdd(&cnt[2], 1ull); if (k < 16) slots[32 + k] = u; }
    }
    // fp8 without clamp for |x| < 464 (RNE must give 448 on (448, 464))
    if (__builtin_fabsf(x) < 464.0f) {
      const unsigned hw8u = __builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0u, false);
      if ((hw8u & 0xFFu) != sw8) {
        if (loc[3]++ == 0) { unsigned long long k = atomicAdd(&cnt[3], 1ull); if (k < 16) slots[48 + k] = u; }
      }
    }
  }
  for (int c = 0; c < 4; ++c)
    if (loc[c] > 1) atomicAdd(&cnt[c], loc[c] - 1);
  // e4m3 decode of all 256 codes (NaN codes 0x7F/0xFF skipped)
  const unsigned long long g = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g < 256 && (g & 0x7F) != 0x7F) {
    const float hw = __builtin_amdgcn_cvt_f32_fp8((int)g, 0);
    if (__float_as_uint(hw) != __float_as_uint(dec_e4m3((unsigned)g))) atomicAdd(&cnt[4], 1ull);
  }
  // packed e4m3 decode of every pair of codes, as either half of a dword
  if (g < 65536 && (g & 0x7F) != 0x7F && ((g >> 8) & 0x7F) != 0x7F) {
    const unsigned w = (unsigned)g * 0x10001u;
    const f32x2 p0 = dec_e4m3_hw_x2<0>(w), p1 = dec_e4m3_hw_x2<1>(w);
    const unsigned lo = __float_as_uint(dec_e4m3((unsigned)g & 0xFFu));
    const unsigned hi = __float_as_uint(dec_e4m3((unsigned)g >> 8));
    if (__float_as_uint(p0.x) != lo || __float_as_uint(p0.y) != hi ||
        __float_as_uint(p1.x) != lo || __float_as_uint(p1.y) != hi)
      atomicAdd(&cnt[6], 1ull);
  }
  if (g < 256) {
    const unsigned lo = dec_e2m1_bits((unsigned)g & 15u), hi = dec_e2m1_bits((unsigned)g >> 4);
    const unsigned w = (unsigned)g * 0x01010101u;  // the byte in all four positions
    const f32x2 d0 = dec_e2m1_hw_x2<0>(w), d1 = dec_e2m1_hw_x2<1>(w);
    const f32x2 d2 = dec_e2m1_hw_x2<2>(w), d3 = dec_e2m1_hw_x2<3>(w);
    const f32x2 d[4] = {d0, d1, d2, d3};
    for (int k = 0; k < 4; ++k)
      if (__float_as_uint(d[k].x) != lo || __float_as_uint(d[k].y) != hi) atomicAdd(&cnt[5], 1ull);
  }
}

int main() {
  unsigned long long* cnt;
  unsigned* slots;
  if (hipMalloc(&cnt, 7 * sizeof(unsigned long long)) != hipSuccess) return 1;
  if (hipMalloc(&slots, 64 * sizeof(unsigned)) != hipSuccess) return 1;
  (void)hipMemset(cnt, 0, 7 * sizeof(unsigned long long));
  (void)hipMemset(slots, 0, 64 * sizeof(unsigned));
  hipLaunchKernelGGL(probe, dim3(65536), dim3(256), 0, 0, cnt, slots);
  if (hipDeviceSynchronize() != hipSuccess) { printf("kernel failed\n"); return 2; }
  unsigned long long h[7];
  unsigned s[64];
  (void)hipMemcpy(h, cnt, sizeof(h), hipMemcpyDeviceToHost);
  (void)hipMemcpy(s, slots, sizeof(s), hipMemcpyDeviceToHost);
  const char* names[4] = {"e4m3 encode, clamped to 448", "e2m1 encode", "e2m1 encode, clamped to 6",
                          "e4m3 encode, unclamped, |x| < 464"};
  for (int c = 0; c < 4; ++c) {
    printf("%s: %llu mismatches\n", names[c], h[c]);
    for (int k = 0; k < 16 && k < (int)h[c]; ++k) {
      float f; unsigned u = s[16 * c + k]; memcpy(&f, &u, 4);
      printf("   x=%a (0x%08x)\n", f, u);
    }
  }
  printf("e4m3 decode: %llu mismatches\n", h[4]);
  printf("e2m1 pair decode, scale 1, byte positions 0..3: %llu mismatches\n", h[5]);
  printf("e4m3 pair decode, both halves: %llu mismatches\n", h[6]);
  return (h[0] | h[1] | h[2] | h[3] | h[4] | h[5] | h[6]) ? 3 : 0;
}
