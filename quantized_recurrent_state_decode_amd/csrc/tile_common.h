// Device helpers shared by the tile kernels: FP16 scale rounding, packed code
// extraction / insertion for the column-pair blocked layout, LDS geometry.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sq_internal.h"

namespace sqk {

constexpr float kFp16Min = 6.103515625e-05f;  // 2^-14
constexpr float kFp16Max = 65504.0f;

// Scales are stored as binary16 after clamping to [2^-14, 65504] and rounding
// to nearest even (STEPQuant App. B.5 gives this clamp for its INT6 scales).
__device__ __forceinline__ float fp16_scale(float x) {
  x = fminf(fmaxf(x, kFp16Min), kFp16Max);
  return __half2float(__float2half_rn(x));
}
__device__ __forceinline__ uint32_t half_bits(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float half_from_bits(uint32_t b) {
  return __half2float(__ushort_as_half((unsigned short)(b & 0xffffu)));
}

// Per-dword masks of the sign bits of b-bit fields laid end to end: xor-ing a
// two's-complement field with its sign bit gives the offset-binary value
// z + 2^(b-1), which converts to float without a sign extension.
template <int BITS>
__device__ __forceinline__ constexpr uint32_t sign_mask(int wi) {
  if constexpr (BITS == 2) return 0xAAAAAAAAu;
  else if constexpr (BITS == 4) return 0x88888888u;
  else if constexpr (BITS == 8) return 0x80808080u;
  else return (wi % 3 == 0) ? 0x20820820u : (wi % 3 == 1) ? 0x08208208u : 0x82082082u;
}

// 64 offset-binary codes (as floats) of one lane chunk; value n = 2m + c.
template <int BITS>
__device__ __forceinline__ void unpack_codes(const uint32_t (&w)[2 * BITS], float (&x)[64]) {
  uint32_t f[2 * BITS];
#pragma unroll
  for (int i = 0; i < 2 * BITS; ++i) f[i] = w[i] ^ sign_mask<BITS>(i);
#pragma unroll
  for (int n = 0; n < 64; ++n) {
    const int pos = n * BITS, wi = pos >> 5, off = pos & 31;
    uint32_t raw = f[wi] >> off;
    if (off + BITS > 32) raw |= f[wi + 1] << (32 - off);
    x[n] = (float)(raw & ((1u << BITS) - 1u));
  }
}

// Inverse of unpack_codes: u[n] holds integer-valued floats in [1, 2^BITS - 1].
template <int BITS>
__device__ __forceinline__ void pack_codes(const float (&u)[64], uint32_t (&w)[2 * BITS]) {
#pragma unroll
  for (int i = 0; i < 2 * BITS; ++i) w[i] = 0u;
#pragma unroll
  for (int n = 0; n < 64; ++n) {
    const uint32_t val = (uint32_t)u[n];
    const int pos = n * BITS, wi = pos >> 5, off = pos & 31;
    w[wi] |= val << off;
    if (off + BITS > 32) w[wi + 1] |= val >> (32 - off);
  }
#pragma unroll
  for (int i = 0; i < 2 * BITS; ++i) w[i] ^= sign_mask<BITS>(i);
}

// Byte offset of piece q of the chunk owned by (row block rb, column pair p).
template <int BITS, int NP>
__device__ __forceinline__ int piece_off(int rb, int p, int q) {
  return ((rb * (BITS / 2) + q) * NP + p) * 16;
}

template <int BITS, int NP>
__device__ __forceinline__ void load_chunk(const unsigned char* region, int rb, int p,
                                           uint32_t (&w)[2 * BITS]) {
#pragma unroll
  for (int q = 0; q < BITS / 2; ++q) {
    const uint4 v = *reinterpret_cast<const uint4*>(region + piece_off<BITS, NP>(rb, p, q));
    w[4 * q + 0] = v.x;
    w[4 * q + 1] = v.y;
    w[4 * q + 2] = v.z;
    w[4 * q + 3] = v.w;
  }
}

template <int BITS, int NP>
__device__ __forceinline__ void store_chunk(unsigned char* region, int rb, int p,
                                            const uint32_t (&w)[2 * BITS]) {
#pragma unroll
  for (int q = 0; q < BITS / 2; ++q)
    *reinterpret_cast<uint4*>(region + piece_off<BITS, NP>(rb, p, q)) =
        make_uint4(w[4 * q + 0], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// Lane geometry of a d_k x d_v tile: lane (rb, p) owns rows 32 rb .. 32 rb + 31
// of columns 2p, 2p+1 (64 values, held in registers).
template <int DK, int DV>
struct Geo {
  static constexpr int NP = DV / 2;    // column pairs = lanes per row block
  static constexpr int NRB = DK / 32;  // row blocks
  static constexpr int NT = NP * NRB;  // threads per tile
};

// Resolve the tile a workgroup owns.  Returns false if it must be skipped
// (slot id or head id out of range); the decode op then writes NaN outputs.
__device__ __forceinline__ bool resolve_tile(const TileArgs& a, int tile, int& h,
                                             unsigned char*& base) {
  if (a.head_ids) {
    h = a.head_ids[tile];
    if (h < 0 || h >= a.P.H) return false;
    base = a.out + (long long)tile * a.out_stride;
    return true;
  }
  const int bi = tile / a.P.H;
  h = tile - bi * a.P.H;
  const int slot = a.slots[bi];
  if (slot < 0 || (long long)slot >= a.n_slots) return false;
  base = a.pool + (long long)slot * a.P.slot_bytes + a.P.head_off[h];
  return true;
}

}  // namespace sqk
