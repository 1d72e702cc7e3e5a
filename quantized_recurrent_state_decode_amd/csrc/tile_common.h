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

// ---------------------------------------------------------------------------
// Fast code paths.  unpack_offset<BITS> gives the 64 values of a lane chunk as
// offset-binary floats u = z + 2^(BITS-1) (value n = 2m + c).  Codes are
// rounded with the magic constant 1.5 * 2^23: m = fma(P, tau, kMagic) rounds
// the exact product P * tau to the nearest integer (ties to even) and leaves
// it, in two's complement, in the low bits of m; pack_magic<BITS> packs those
// bits without converting back.
constexpr float kMagic = 12582912.0f;

// byte k of w as a float: one v_cvt_f32_ubyte{k} (written out so that the
// compiler does not narrow it to a bit-field extract plus a conversion)
__device__ __forceinline__ float ubyte(uint32_t w, int k) {
  float r;
  if (k == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(w));
  else if (k == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(w));
  else if (k == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(w));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <int BITS>
__device__ __forceinline__ void unpack_offset(const uint32_t (&w)[2 * BITS], float (&x)[64]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {              // dword d: rows 4d..4d+3, both columns
      const uint32_t f = w[d] ^ 0x88888888u;
      // (the high nibbles shifted first: one shift and one three-input op)
      const uint32_t lo = f & 0x0f0f0f0fu, hi = ((w[d] >> 4) ^ 0x08080808u) & 0x0f0f0f0fu;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[8 * d + 2 * k] = ubyte(lo, k);
        x[8 * d + 2 * k + 1] = ubyte(hi, k);
      }
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const uint32_t f = w[d] ^ 0x80808080u;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[4 * d + k] = ubyte(f, k);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {              // dword d: values 16d .. 16d+15
      const uint32_t f = w[d] ^ 0xaaaaaaaau;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t g = (f >> (2 * s)) & 0x03030303u;
#pragma unroll
        for (int k = 0; k < 4; ++k) x[16 * d + 4 * k + s] = ubyte(g, k);
      }
    }
  } else {
    unpack_codes<BITS>(w, x);
  }
}

// Codes as binary16 subnormals.  An offset-binary code u placed in the low
// bits of a half (exponent field 0) is the subnormal u * 2^-24, exactly; a
// mixed-precision FMA (v_fma_mix_f32, binary16 denormals kept) reads it
// straight from its half, so the code costs no conversion instruction and the
// factor 2^24 goes into the other operand (the exact product is unchanged).
// unpack_half<BITS> fills 32 registers with two codes each: register
// hreg(n), half hhi(n) holds value n = 2m + c (any width up to 8 bits:
// 2^(BITS-1) + z < 1024 fits the 10-bit significand).
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int BITS>
__device__ __forceinline__ constexpr int hreg(int n) {
  if constexpr (BITS == 2) return 8 * (n >> 4) + (n & 7);       // n, n + 8
  else if constexpr (BITS == 8) return 2 * (n >> 2) + (n & 1);  // n, n + 2
  else return 4 * (n >> 3) + (n & 3);                           // n, n + 4 (4 and 6 bits)
}
template <int BITS>
__device__ __forceinline__ constexpr int hhi(int n) {
  return BITS == 2 ? (n >> 3) & 1 : BITS == 8 ? (n >> 1) & 1 : (n >> 2) & 1;
}
// value n as a float (u * 2^-24): folds into the FMA that consumes it
template <int BITS>
__device__ __forceinline__ float hcode(const uint32_t (&h)[32], int n) {
  const half2v v = __builtin_bit_cast(half2v, h[hreg<BITS>(n)]);
  return (float)(hhi<BITS>(n) ? v.y : v.x);
}
template <int BITS>
__device__ __forceinline__ void unpack_half(const uint32_t (&w)[2 * BITS], uint32_t (&h)[32]) {
  // each register takes the fields 16 bits apart: shift the dword by the
  // field's offset, flip the sign bits, keep BITS bits of each half
  constexpr uint32_t keep = ((1u << BITS) - 1u) * 0x00010001u;
  constexpr uint32_t sgn = (1u << (BITS - 1)) * 0x00010001u;
  if constexpr (BITS == 6) {
    // 16 fields per 3 dwords, field t at bit 6t.  Fields t and t + 4 are three
    // bytes apart at the same offset within their byte, so one byte
    // permutation brings both 16 bits apart and one shift aligns them.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = (j & 3) + 8 * (j >> 2);    // fields t, t + 4 -> register 8g + j
        const int b0 = (6 * t) >> 3, sh = (6 * t) & 7, dlo = b0 >> 2;
        const int bytes[4] = {b0, b0 + 1, b0 + 3, b0 + 4};
        uint32_t sel = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k)            // byte 12 lies past the group: zero
          sel |= (uint32_t)(bytes[k] < 12 ? bytes[k] - 4 * dlo : 0x0c) << (8 * k);
        const uint32_t lo = w[3 * g + dlo], hi = dlo < 2 ? w[3 * g + dlo + 1] : lo;
        h[8 * g + j] = ((__builtin_amdgcn_perm(hi, lo, sel) >> sh) ^ sgn) & keep;
      }
    }
  } else {
    constexpr int per = 16 / BITS;               // registers per dword
#pragma unroll
    for (int d = 0; d < 2 * BITS; ++d) {
#pragma unroll
      for (int j = 0; j < per; ++j) h[per * d + j] = ((w[d] >> (BITS * j)) ^ sgn) & keep;
    }
  }
}

// dword of the low bytes of four floats' bit patterns
__device__ __forceinline__ uint32_t low_bytes4(float a, float b, float c, float d) {
  const uint32_t ab = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// 16 six-bit fields (the low bits of mg[0..15]) into 3 dwords, field t at
// bit 6t.  v_alignbit shifts a dword right and brings the next field's low
// bits in at the top, one instruction per field and no masks: a dword is
// built from the fields that end in it, the last shift sized to leave its
// first field at bit 0.
__device__ __forceinline__ void pack6(const float* mg, uint32_t* w) {
  auto in = [&](uint32_t acc, int t, int sh) {
    return __builtin_amdgcn_alignbit(__float_as_uint(mg[t]), acc, sh);
  };
  uint32_t a = __float_as_uint(mg[0]) << 26;   // fields 0..5 (field 5: its low 2 bits)
#pragma unroll
  for (int t = 1; t < 5; ++t) a = in(a, t, 6);
  w[0] = in(a, 5, 2);
  a = __float_as_uint(mg[5]) << 26;            // fields 5 (high 4 bits) .. 10 (low 4)
#pragma unroll
  for (int t = 6; t < 10; ++t) a = in(a, t, 6);
  w[1] = in(a, 10, 4);
  a = __float_as_uint(mg[10]) << 26;           // fields 10 (high 2 bits) .. 15
#pragma unroll
  for (int t = 11; t < 16; ++t) a = in(a, t, 6);
  w[2] = a;
}

template <int BITS>
__device__ __forceinline__ void pack_magic(const float (&mg)[64], uint32_t (&w)[2 * BITS]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t lo = low_bytes4(mg[8 * d], mg[8 * d + 2], mg[8 * d + 4], mg[8 * d + 6]);
      const uint32_t hi = low_bytes4(mg[8 * d + 1], mg[8 * d + 3], mg[8 * d + 5], mg[8 * d + 7]);
      w[d] = (lo & 0x0f0f0f0fu) | ((hi << 4) & 0xf0f0f0f0u);
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int d = 0; d < 16; ++d)
      w[d] = low_bytes4(mg[4 * d], mg[4 * d + 1], mg[4 * d + 2], mg[4 * d + 3]);
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t acc = 0u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t g = low_bytes4(mg[16 * d + s], mg[16 * d + 4 + s], mg[16 * d + 8 + s],
                                      mg[16 * d + 12 + s]);
        acc |= (g & 0x03030303u) << (2 * s);
      }
      w[d] = acc;
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) pack6(&mg[16 * g], &w[3 * g]);
  }
}

// Byte offset of piece q of the chunk owned by (row block rb, column pair p).
template <int BITS, int NP>
__device__ __forceinline__ int piece_off(int rb, int p, int q) {
  return ((rb * (BITS / 2) + q) * NP + p) * 16;
}

// The packed state is streamed: each chunk is read once and written once per
// step, so loads and stores are nontemporal (the caches keep the inputs and
// tables instead; measured faster on every packed workload).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BITS, int NP>
__device__ __forceinline__ void load_chunk(const unsigned char* region, int rb, int p,
                                           uint32_t (&w)[2 * BITS]) {
#pragma unroll
  for (int q = 0; q < BITS / 2; ++q) {
    const u32x4 v =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(region + piece_off<BITS, NP>(rb, p, q)));
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
  for (int q = 0; q < BITS / 2; ++q) {
    const u32x4 v = {w[4 * q + 0], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(region + piece_off<BITS, NP>(rb, p, q)));
  }
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
// A value equal on every active lane of the wave (a per-tile index, offset or
// coefficient loaded from memory), moved to a scalar register so that it and
// the pointers built from it take no vector registers.
__device__ __forceinline__ int wuni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ long long wuni(long long v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)v);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ float wuni(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Orders LDS accesses among the lanes of one wave: rows owned by a single wave
// only need the wave's own writes visible, not a workgroup barrier.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS accesses by byte address.  An address kept as a plain integer (passed
// through an empty asm) stays in one register, and the accesses built on it
// carry their constant parts as instruction offsets.
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
__device__ __forceinline__ int lds_addr(const void* ptr) { return (int)(uintptr_t)(const lds_u8*)ptr; }
__device__ __forceinline__ uint32_t lds_ld32(int a) { return *(const lds_u32*)(uintptr_t)a; }
typedef __attribute__((address_space(3))) signed char lds_s8;
// byte k (0 or 1) of w, sign-extended, as a float: one v_cvt_f32_i32 with an
// SDWA byte select (written out: the compiler otherwise emits a bit-field
// extract and a conversion)
template <int K>
__device__ __forceinline__ float sbyte_f(uint32_t w) {
  static_assert(K == 0 || K == 1, "byte 0 or 1");
  float r;
  if constexpr (K == 0)
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  else
    asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  return r;
}
// a byte, sign-extended (ds_read_i8), and a 16-bit word (ds_read_u16)
__device__ __forceinline__ int lds_ld8s(int a) { return *(const lds_s8*)(uintptr_t)a; }
__device__ __forceinline__ uint32_t lds_ld16(int a) { return *(const lds_u16*)(uintptr_t)a; }
__device__ __forceinline__ float4 lds_ld4(int a) {
  const f32x4 v = *(const lds_f32x4*)(uintptr_t)a;
  return make_float4(v.x, v.y, v.z, v.w);
}
// Row transposes of 16 rows: lane p writes its partial of row m at
// [m][p] and then reads 16 consecutive partials of one row with four 16-byte
// reads.  A row stride of NP + 4 floats keeps the rows 16-byte aligned and
// both the writes (consecutive lanes, consecutive words) and the reads (the
// 16 lanes of a read group start 4 banks apart) free of bank conflicts.
template <int NP>
struct RowT {
  static constexpr int S = NP + 4;
};
// combine of the 16 floats at f (16-byte aligned LDS): sum or max
template <bool MAX>
__device__ __forceinline__ float lds_fold16(const float* f) {
  const f32x4* v = reinterpret_cast<const f32x4*>(f);
  const f32x4 a = v[0], b = v[1], c = v[2], d = v[3];
  if constexpr (MAX) {
    const float m0 = fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w));
    const float m1 = fmaxf(fmaxf(b.x, b.y), fmaxf(b.z, b.w));
    const float m2 = fmaxf(fmaxf(c.x, c.y), fmaxf(c.z, c.w));
    const float m3 = fmaxf(fmaxf(d.x, d.y), fmaxf(d.z, d.w));
    return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
  } else {
    return (((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w))) +
           (((c.x + c.y) + (c.z + c.w)) + ((d.x + d.y) + (d.z + d.w)));
  }
}
__device__ __forceinline__ void lds_st8(int a, uint32_t v) { *(lds_u8*)(uintptr_t)a = (unsigned char)v; }
__device__ __forceinline__ void lds_st16(int a, uint32_t v) { *(lds_u16*)(uintptr_t)a = (unsigned short)v; }
__device__ __forceinline__ void lds_st32(int a, uint32_t v) { *(lds_u32*)(uintptr_t)a = v; }
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Lane i of a 16-lane row takes the value of the lane the DPP control names
// (quad_perm 0xB1: xor 1, 0x4E: xor 2; 0x141: half-row mirror; 0x140: row mirror).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}
// Sum over each 32-lane half of the wave (lanes 0-31, 32-63), valid in its
// upper 16 lanes (p = 16 .. 31 of the half): the 16-lane row sums, then
// row_bcast:15 adds the first row's total into the second (row mask 0b1010).
__device__ __forceinline__ float half32_sum_hi(float v) {
  v = row16_sum(v);
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
}
// Combination of each lane's value with the lane 16 (swap16) or 32 (swap32)
// away: v_permlane16/32_swap exchange the odd 16-lane rows (the upper 32
// lanes) of one copy with the even rows (lower 32 lanes) of the other.
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Sum of the parts of a transposed row statistic: lane p holds part p >> 4
// of row p & 15, so the parts sit 16 (and, with 64 lanes per row block, 32)
// lanes apart.
template <int NP>
__device__ __forceinline__ float parts_sum(float v) {
  float a, b;
  swap16(v, a, b);
  v = a + b;
  if constexpr (NP == 64) {
    swap32(v, a, b);
    v = a + b;
  }
  return v;
}
// Sum over the 64 lanes of the wave, in every lane.
__device__ __forceinline__ float wave_sum(float v) { return parts_sum<64>(row16_sum(v)); }

__device__ __forceinline__ bool resolve_tile(const TileArgs& a, int tile, int& h,
                                             unsigned char*& base) {
  if (a.out) {  // quantize-only: head head_ids[tile], or tile % H without ids
    h = a.head_ids ? wuni(a.head_ids[tile]) : tile % a.P.H;
    if (h < 0 || h >= a.P.H) return false;
    base = a.out + (long long)tile * a.out_stride;
    return true;
  }
  const int bi = tile / a.P.H;
  h = tile - bi * a.P.H;
  const int slot = wuni(a.slots[bi]);
  if (slot < 0 || (long long)slot >= a.n_slots) return false;
  base = a.pool + (long long)slot * a.P.slot_bytes + wuni(a.P.head_off[h]);
  return true;
}

}  // namespace sqk
