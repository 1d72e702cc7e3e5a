// Fused quantized decode step for STEP KDA heads: channel-wise retention
// D = diag(d), bit width chosen per key row (STEPQuant Sec. 4, unit = key
// row for KDA), FP16 pivot rows, one column-scale vector c shared by all
// integer rows of the head (App. D: the codebook normalisation is fixed by
// precision, so rows of different widths share c).
//
// Storage rows are ordered by (width, key row) and kept row-major, so a head
// is a run of variable-length rows.  The workgroup stages the packed head in
// LDS with coalesced 16-byte copies; lane (rb, p) extracts columns 2p, 2p+1
// of its 32 storage rows, writes the new codes back into the same LDS bytes
// and the head is copied out with 16-byte stores.  Because the rows are
// sorted, the rows of one block that share a width are consecutive: the block
// keeps one bit mask per width class and the byte offset of the class's first
// row, so a row's width and offset are scalar values.  On 64-lane blocks the
// reads take each row's address and width from a row table (arithmetic on
// the width, no branch), a block of a single 4- or 8-bit width has read and
// code passes of its own, and elsewhere the per-row branch of the code pass is
// a scalar branch to code specialised for that width.  Per-row inputs
// (d, k, q, w) are gathered through the storage permutation.  Per element,
// with rho_s the row's retained dequantisation factor (d_s r_s / q_b on
// integer rows, d_s on FP16 rows):
//   integer rows: x = c_j z;  kappa = k rho, gamma = beta k / rho,
//                 theta = q rho, Xt = X / rho
//   FP16 rows:    x = rho h;  kappa = k, gamma = beta k, theta = q, Xt = X
//   delta_j = sum_s kappa_s x_sj,  Xt = x + gamma_s e_j,
//   y_j = sum_s theta_s Xt_sj
// then the GDN kernel's row scales, column init, codes by magic rounding
// (per-width q_b) and fixed-code column refit over the integer rows.
#include <algorithm>

#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV>
struct SmemKdaCore {
  float rowc[8][DK];  // 0 kappa, 1 gamma, 2 theta, 3 rho, 4 pi or rho (FP16 rows),
                      // 5 lambda = w^2 r^2 / q_b, 6 mu = lambda / q_b, 7 q_b
                      // (5-7 are 0 on FP16 rows)
  float2 colA[DK / 32][DV / 2];
  float2 colB[DK / 32][DV / 2];
  float2 colM[DK / 32][DV / 2];
  float4 colC[DK / 32][DV / 2];
  float2 vin[DV / 2];  // the token's v, staged by row block 0
  int2 rowab[DK];      // storage row s: LDS byte address of its codes, its width
};
// Row m of a width class is addressed as (class base - lo * row bytes) + m *
// row bytes, the last term an instruction offset.  The first term may fall
// below the dynamic buffer by up to 31 rows of the widest class; the static
// block (placed before the dynamic one) is padded to at least that size, so
// the address register never goes negative.
template <int DK, int DV>
constexpr int kda_pad() {
  constexpr int need = 31 * 2 * DV, have = (int)sizeof(SmemKdaCore<DK, DV>);
  return need > have ? need - have : 16;
}
template <int DK, int DV>
struct SmemKda : SmemKdaCore<DK, DV> {
  unsigned char pad[kda_pad<DK, DV>()];
};

// The packed head (at most max_code_bytes) and, while no codes are live,
// the per-wave row transpose, share the dynamic LDS buffer; its last 16
// bytes are a spare slot for staging stores past the head's region (and
// hold the second dword read for the last lanes of the last row).
extern __shared__ uint4 kda_dyn[];

template <int DK, int DV>
__host__ __device__ constexpr int dyn_bytes(int max_code_bytes) {
  constexpr int transpose = (DK / 32) * 16 * RowT<DV / 2>::S * 4;
  return ((max_code_bytes > transpose ? max_code_bytes : transpose) + 15) / 16 * 16 + 16;
}


// Width classes 2, 4, 6, 8 bits and FP16 (16).
template <int B>
struct Wc {
  static constexpr int bits = B;
  static constexpr int idx = B == 2 ? 0 : B == 4 ? 1 : B == 6 ? 2 : B == 8 ? 3 : 4;
};

// The width classes of one row block: bit m of msk[c] marks row m of the
// block as class c (2, 4, 6, 8 bits, FP16), and b0[c] is the LDS byte address
// of a row 0 of class c numbered from the class's first row, so row m of the
// class starts at b0[c] + m * (DV * width / 8).  With 64 lanes per block these
// are wave-uniform (scalar registers); with 32 a wave holds two blocks and
// they are per lane.
struct RowCls {
  uint32_t msk[5];
  int b0[5];
};

// Lane addresses of each class for one pass: the row start b0[c] plus the
// lane's byte in the row, read (the dword holding the lane's first field
// bit) or written (the lane's bytes; 2- and 6-bit fields are written per
// group of four lanes).  Formed at the start of the pass that uses them.
template <bool WRITE>
__device__ __forceinline__ void lane_addrs(const RowCls& R, int p, int (&a)[5]) {
  const int rdb[5] = {4 * (p >> 3), 4 * (p >> 2), 4 * ((12 * p) >> 5), 4 * (p >> 1), 4 * p};
  const int wrb[5] = {2 * (p >> 2), p, 6 * (p >> 2) + 2 * (p & 3), 2 * p, 4 * p};
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    a[c] = R.b0[c] + (WRITE ? wrb[c] : rdb[c]);
    asm volatile("" : "+v"(a[c]));
  }
}

template <int DV, int C>
constexpr int row_bytes() {
  constexpr int W[5] = {2, 4, 6, 8, 16};
  return DV * W[C] / 8;
}

// Call f(Wc<width>) for the class of row m (classes tested in order of their
// share at a nominal 6 bits).
template <class F>
__device__ __forceinline__ void by_class(const RowCls& R, int m, F&& f) {
  const uint32_t bit = 1u << m;
  if (R.msk[2] & bit) f(Wc<6>{});
  else if (R.msk[1] & bit) f(Wc<4>{});
  else if (R.msk[3] & bit) f(Wc<8>{});
  else if (R.msk[4] & bit) f(Wc<16>{});
  else if (R.msk[0] & bit) f(Wc<2>{});
}

// Each pass over the rows tests the masks afresh: an empty asm that "changes"
// them stops the compiler from carrying one pass's per-row tests into the
// next as lane-mask values (whose use as a branch condition costs vector
// instructions per row).
template <bool WU>
__device__ __forceinline__ void fresh_masks(RowCls& R) {
  if constexpr (WU) {
#pragma unroll
    for (int c = 0; c < 5; ++c) asm volatile("" : "+s"(R.msk[c]));
  }
}

// lane i takes the value of lane i + n of its 16-lane row (n = 1, 2)
template <int N>
__device__ __forceinline__ uint32_t from_next(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xf, 0xf, false);
}

// The lane's two values (columns 2p, 2p+1) of a row of width B from the two
// dwords lo, hi read at the dword holding the first field bit: two's-
// complement integers starting at bit 2 B p of the row (the shift count of
// the funnel shift is taken mod 32), or FP16 values (B = 16, dword p).
template <int B>
__device__ __forceinline__ void decode_pair(uint32_t lo, uint32_t hi, int p, float& z0, float& z1) {
  if constexpr (B == 16) {
    z0 = half_from_bits(lo);
    z1 = half_from_bits(lo >> 16);
  } else {
    const uint32_t f = __builtin_amdgcn_alignbit(hi, lo, 2 * B * p);
    // the builtin returns an unsigned type: reinterpret as signed before converting
    z0 = (float)(int)__builtin_amdgcn_sbfe((int)f, 0, B);
    z1 = (float)(int)__builtin_amdgcn_sbfe((int)f, B, B);
  }
}

// Write the lane's two codes (magic-rounded floats m0, m1) of a row of width
// B < 16; a is the lane's write address in the row.  2- and 6-bit fields of a
// group of four lanes fill two or six bytes, which lanes of the group write as
// 16-bit words (lane q of a 6-bit group writes bytes 2q, 2q+1).
template <int B>
__device__ __forceinline__ void write_pair(int a, int p, float m0, float m1) {
  const uint32_t u0 = __float_as_uint(m0), u1 = __float_as_uint(m1);
  if constexpr (B == 4) {
    lds_st8(a, (u0 & 15u) | ((u1 & 15u) << 4));
  } else if constexpr (B == 8) {
    lds_st16(a, (u0 & 0xffu) | ((u1 & 0xffu) << 8));
  } else if constexpr (B == 2) {
    const uint32_t nib = (u0 & 3u) | ((u1 & 3u) << 2);
    const uint32_t n1 = nib | (from_next<1>(nib) << 4);
    const uint32_t n2 = n1 | (from_next<2>(n1) << 8);
    if ((p & 3) == 0) lds_st16(a, n2);
  } else {
    const uint32_t f = (u0 & 63u) | ((u1 & 63u) << 6);
    const uint32_t nx = from_next<1>(f);
    const int q = p & 3;
    if (q < 3) lds_st16(a, (f >> (4 * q)) | (nx << (12 - 4 * q)));
  }
}

// pass 4 over the lane's rows: codes by magic rounding with the scale
// q_b / c0_j (q_b of each row from the row table, the magic constant mgc
// held in a scalar register), the
// fixed-code refit sums N = sum_s lambda_s z P and D = sum_s mu_s z^2, the
// same arithmetic on every row (an FP16 row has q_b = 0, so z = 0, and zero
// weights), then the new codes (or FP16 values) written into the staged head
// by code specialised for the row's width
template <int DK, int DV, bool SAT>
__device__ __forceinline__ void codes_refit(float (&x)[64], const RowCls& R, const float* lam,
                                            const float* mu, const float* qbr, float ic0,
                                            float ic1, float mgc, int p, float& N0, float& N1,
                                            float& D0, float& D1) {
  int wra[5];
  lane_addrs<true>(R, p, wra);
#pragma unroll
  for (int m4 = 0; m4 < 32; m4 += 2) {
    const float2 l4 = *reinterpret_cast<const float2*>(lam + m4);
    const float2 u4 = *reinterpret_cast<const float2*>(mu + m4);
    const float2 q4 = *reinterpret_cast<const float2*>(qbr + m4);
    const float lv[2] = {l4.x, l4.y}, uv[2] = {u4.x, u4.y};
    const float qv[2] = {q4.x, q4.y};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = m4 + u;
      const float qb = qv[u];
      const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
      float mg0 = fmaf(pv0, qb * ic0, mgc), mg1 = fmaf(pv1, qb * ic1, mgc);
      if constexpr (SAT) {  // a column scale saturated at the FP16 maximum
        mg0 = __builtin_amdgcn_fmed3f(mg0, mgc - qb, mgc + qb);
        mg1 = __builtin_amdgcn_fmed3f(mg1, mgc - qb, mgc + qb);
      }
      const float z0 = mg0 - mgc, z1 = mg1 - mgc;
      N0 = fmaf(lv[u] * z0, pv0, N0);
      N1 = fmaf(lv[u] * z1, pv1, N1);
      D0 = fmaf(uv[u] * z0, z0, D0);
      D1 = fmaf(uv[u] * z1, z1, D1);
      // the sums are complete here: kept from sinking below the writes, which
      // would hold every row's rounded values live at once
      asm volatile("" : "+v"(N0), "+v"(N1), "+v"(D0), "+v"(D1));
      by_class(R, m, [&](auto w) {
        constexpr int B = decltype(w)::bits, C = decltype(w)::idx;
        const int a = wra[C] + m * row_bytes<DV, C>();
        if constexpr (B == 16) lds_st32(a, half_bits(pv0) | (half_bits(pv1) << 16));
        else write_pair<B>(a, p, mg0, mg1);
      });
    }
  }
}

// Pass 4 for blocks whose row masks are wave-uniform (64 lanes per block):
// the arithmetic runs inside the branch for the row's width, so the rounding
// scale q_b / c0_j of each width is a register formed once, and the
// denominator is summed per width, D = sum_B (sum_{rows of width B}
// lambda_s z^2) / q_b(B) (lambda_s carries one factor 1 / q_b, the other is
// applied per width at the end).  FP16 rows only store their values.
template <int DK, int DV, bool SAT>
__device__ __forceinline__ void codes_refit_wu(float (&x)[64], const RowCls& R, const float* lam,
                                               float ic0, float ic1, float mgc, int p, float& N0,
                                               float& N1, float& D0, float& D1) {
  constexpr float QB[4] = {1.f, 7.f, 31.f, 127.f};
  int wra[5];
  lane_addrs<true>(R, p, wra);
  float tau[4][2], dc[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    tau[c][0] = QB[c] * ic0;
    tau[c][1] = QB[c] * ic1;
    dc[c][0] = 0.f;
    dc[c][1] = 0.f;
  }
#pragma unroll
  for (int m4 = 0; m4 < 32; m4 += 2) {
    const float2 l4 = *reinterpret_cast<const float2*>(lam + m4);
    const float lv[2] = {l4.x, l4.y};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = m4 + u;
      const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
      by_class(R, m, [&](auto w) {
        constexpr int B = decltype(w)::bits, C = decltype(w)::idx;
        const int a = wra[C] + m * row_bytes<DV, C>();
        if constexpr (B == 16) {
          lds_st32(a, half_bits(pv0) | (half_bits(pv1) << 16));
        } else {
          float mg0 = fmaf(pv0, tau[C][0], mgc), mg1 = fmaf(pv1, tau[C][1], mgc);
          if constexpr (SAT) {  // a column scale saturated at the FP16 maximum
            mg0 = __builtin_amdgcn_fmed3f(mg0, mgc - QB[C], mgc + QB[C]);
            mg1 = __builtin_amdgcn_fmed3f(mg1, mgc - QB[C], mgc + QB[C]);
          }
          const float z0 = mg0 - mgc, z1 = mg1 - mgc;
          const float t0 = lv[u] * z0, t1 = lv[u] * z1;
          N0 = fmaf(t0, pv0, N0);
          N1 = fmaf(t1, pv1, N1);
          dc[C][0] = fmaf(t0, z0, dc[C][0]);
          dc[C][1] = fmaf(t1, z1, dc[C][1]);
          asm volatile("" : "+v"(N0), "+v"(N1), "+v"(dc[C][0]), "+v"(dc[C][1]));
          write_pair<B>(a, p, mg0, mg1);
        }
      });
    }
  }
  D0 = 0.f;
  D1 = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    D0 = fmaf(dc[c][0], 1.f / QB[c], D0);
    D1 = fmaf(dc[c][1], 1.f / QB[c], D1);
  }
}

// Pass 4 for a 64-lane row block whose rows all have width B (4 or 8 bits;
// no FP16 rows): no per-row dispatch, one rounding scale and one denominator.
template <int DK, int DV, int B>
__device__ __forceinline__ void codes_refit_one(float (&x)[64], const RowCls& R, const float* lam,
                                                float ic0, float ic1, float mgc, int p, float& N0,
                                                float& N1, float& D0, float& D1) {
  constexpr int C = Wc<B>::idx;
  constexpr float QB = (float)((1 << (B - 1)) - 1);
  int wra[5];
  lane_addrs<true>(R, p, wra);
  const float tau0 = QB * ic0, tau1 = QB * ic1;
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int m4 = 0; m4 < 32; m4 += 2) {
    const float2 l4 = *reinterpret_cast<const float2*>(lam + m4);
    const float lv[2] = {l4.x, l4.y};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = m4 + u;
      const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
      const float mg0 = fmaf(pv0, tau0, mgc), mg1 = fmaf(pv1, tau1, mgc);
      const float z0 = mg0 - mgc, z1 = mg1 - mgc;
      const float t0 = lv[u] * z0, t1 = lv[u] * z1;
      N0 = fmaf(t0, pv0, N0);
      N1 = fmaf(t1, pv1, N1);
      d0 = fmaf(t0, z0, d0);
      d1 = fmaf(t1, z1, d1);
      asm volatile("" : "+v"(N0), "+v"(N1), "+v"(d0), "+v"(d1));
      write_pair<B>(wra[C] + m * row_bytes<DV, C>(), p, mg0, mg1);
    }
  }
  D0 = d0 * (1.f / QB);
  D1 = d1 * (1.f / QB);
}

template <int DK, int DV, int OP>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void kda_tile_kernel(TileArgs a) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT;
  constexpr bool WU = NP % 64 == 0;  // a wave's lanes share their rows
  __shared__ SmemKda<DK, DV> sm;
  unsigned char* codes = reinterpret_cast<unsigned char*>(kda_dyn);
  float(*rowt)[16][RowT<NP>::S] = reinterpret_cast<float(*)[16][RowT<NP>::S]>(kda_dyn);
  const int tile = blockIdx.x;
  // Row blocks of one head differ in cost (widths, FP16 rows): on 64-lane
  // blocks wave w takes block (w + tile) mod NRB, so that the heavier block
  // positions do not always fall to the same wave slot of a workgroup
  // (measured +0.4 % on the KDA workload).
  const int t = threadIdx.x, wave = t / NP, p = t - wave * NP, j0 = 2 * p;
  const int rb = WU ? ((wave + tile) & (NRB - 1)) : wave, r0 = 32 * rb;
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  // The loads that do not depend on the slot go out before the slot is
  // resolved: the head's row metadata (the owner lanes p < 32 hold storage
  // row r0 + p) and, once the key rows arrive, the token's per-row inputs.
  // The slot id travels alongside, so a tile's start waits on two round
  // trips (slot -> codes, metadata -> inputs) rather than three.
  int h = 0, slot = 0;
  unsigned char* base = nullptr;
  bool ok = true;
  if (a.out) {
    ok = resolve_tile(a, tile, h, base);
  } else {
    const int bi = tile / a.P.H;
    h = tile - bi * a.P.H;
    slot = wuni(a.slots[bi]);
  }
  const int* rkey = a.P.row_key + h * DK;
  int rk = 0, rbits = 16, roff = 0;
  if (ok && p < 32) {
    const int s = r0 + p;
    rk = rkey[s];
    rbits = a.P.row_bits[h * DK + s];
    roff = a.P.row_off[h * DK + s];
  }
  // the row's impact factor (and its inverse) go out with the token's inputs;
  // they wait in LDS for the row-scale pass, so the key row need not stay live
  float d = 0.f, kk = 0.f, qq = 0.f, beta = 0.f, wv = 0.f, wiv = 0.f;
  if (ok && p < 32 && OP != OP_UNPACK) {
    wv = a.P.w[h * DK + rk];
    wiv = a.P.winv[h * DK + rk];
  }
  if constexpr (OP == OP_DECODE) {
    if (ok && p < 32) {
      d = a.gate[tk + rk];
      kk = a.k[tk + rk];
      qq = a.q[tk + rk];
    }
    beta = a.beta[tile];
  }
  // the token's v is needed after the first block barrier of pass 1; row
  // block 0 loads it with the other inputs and stages it in LDS (on the
  // other tile shapes the extra live range spills: v is read late there)
  constexpr bool EARLY_V = DK == 128 && DV == 128;
  float2 vin = make_float2(0.f, 0.f);
  if (EARLY_V && OP == OP_DECODE && ok && rb == 0) vin = *reinterpret_cast<const float2*>(a.v + tv + j0);
  if (!a.out) {
    ok = slot >= 0 && (long long)slot < a.n_slots;
    base = a.pool + (long long)(ok ? slot : 0) * a.P.slot_bytes + wuni(a.P.head_off[h]);
  }
  if (!ok) {
    if (OP == OP_DECODE && t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    return;
  }
  const int code_bytes = wuni(a.P.r_off[h]);
  __half* r_ptr = reinterpret_cast<__half*>(base + code_bytes);
  __half* c_ptr = reinterpret_cast<__half*>(base + wuni(a.P.c_off[h]));
  // width classes of the block's rows and the lane's field addresses
  static_assert((int)sizeof(SmemKda<DK, DV>) >= 31 * 2 * DV, "LDS address bases may go negative");
  RowCls R;
  {
    constexpr int W[5] = {2, 4, 6, 8, 16};
    const int lane = t & 63, half = WU ? 0 : (lane & 32);
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      const unsigned long long bal = __ballot(p < 32 && rbits == W[c]);
      const uint32_t mk = (uint32_t)(bal >> half);
      const int lo = mk ? __builtin_ctz(mk) : 0;
      const int first = WU ? __builtin_amdgcn_readlane(roff, lo) : __shfl(roff, half + lo);
      R.msk[c] = mk;
      R.b0[c] = lds_addr(codes) + first - lo * (DV * W[c] / 8);
    }
  }
  // a 64-lane block whose rows all have 4 (one = 1) or 8 bits (one = 3) takes
  // width-specialised read and code passes (about half the blocks of a
  // calibrated plan: rows sorted by width fill whole blocks of one width)
  const int one = !WU ? -1 : R.msk[1] == ~0u ? 1 : R.msk[3] == ~0u ? 3 : -1;
  float x[64];
  float y0 = 0.f, y1 = 0.f;
  if constexpr (OP == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int key = rkey[r0 + m];
      const float2 v2 = *reinterpret_cast<const float2*>(X + key * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    if (p < 32) {
      const int s = r0 + p;
      sm.rowc[3][s] = 1.0f;
      sm.rowc[5][s] = wv;
      sm.rowc[6][s] = wiv;
      sm.rowc[7][s] = rbits == 16 ? 0.f : (float)((1 << (rbits - 1)) - 1);
    }
    __syncthreads();
  } else {
    // The head's code rows are staged through registers, CH 16-byte chunks
    // per thread and round (one round covers 16 KB at 128 x 128): the loads
    // are unconditional (chunks past the region reread chunk 0) and so are
    // the stores (those chunks land in a spare slot past the largest region),
    // so nothing waits between them; the per-row inputs go out alongside.
    constexpr int CH = 4;
    const int nch = code_bytes >> 4;
    const int spare = dyn_bytes<DK, DV>(a.P.max_code_bytes) / 16 - 1;
    const u32x4* src = reinterpret_cast<const u32x4*>(base);
    u32x4* dst = reinterpret_cast<u32x4*>(codes);
    u32x4 v[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {  // first round, issued before the scale loads
      const int e = t + i * NT;
      v[i] = __builtin_nontemporal_load(src + (e < nch ? e : 0));
    }
    const float c0 = __half2float(c_ptr[j0]), c1 = __half2float(c_ptr[j0 + 1]);
    float rs = 0.f;
    if (p < 32) rs = __half2float(r_ptr[r0 + p]);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = t + i * NT;
      dst[e < nch ? e : spare] = v[i];
    }
    for (int c = CH * NT; c < nch; c += CH * NT) {  // heads larger than one round
      u32x4 w[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int e = c + t + i * NT;
        w[i] = __builtin_nontemporal_load(src + (e < nch ? e : 0));
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int e = c + t + i * NT;
        dst[e < nch ? e : spare] = w[i];
      }
    }
    if (p < 32) {
      const int s = r0 + p;
      const bool piv = rbits == 16;
      const float qb = piv ? 1.f : (float)((1 << (rbits - 1)) - 1);
      const float sc = piv ? 1.f : rs * frcp(qb);
      sm.rowc[5][s] = wv;
      sm.rowc[6][s] = wiv;
      sm.rowc[7][s] = piv ? 0.f : qb;
      if constexpr (OP == OP_UNPACK) {
        sm.rowc[3][s] = sc;
        sm.rowc[4][s] = 1.0f;
      } else {
        const float bk = beta * kk;
        const float rho = d * sc;
        if (piv) {
          // FP16 rows keep X itself: the unpacked value is scaled by rho, so
          // X = rho h + beta k e_j takes two roundings, as the stored FP16
          // value needs
          sm.rowc[0][s] = kk;
          sm.rowc[1][s] = bk;
          sm.rowc[2][s] = qq;
          sm.rowc[3][s] = 1.0f;
          sm.rowc[4][s] = rho;
        } else {
          // a vanishing retention keeps the division finite; the dropped part
          // (rp - rho) c_j z_sj is below 2^-60 of the write term
          const float rp = fmaxf(rho, fmaxf(fabsf(bk) * 0x1p-60f, 0x1p-100f));
          sm.rowc[0][s] = kk * rho;
          sm.rowc[1][s] = bk * frcp(rp);
          sm.rowc[2][s] = qq * rp;
          sm.rowc[3][s] = rp;
        }
      }
    }
    if (EARLY_V && OP == OP_DECODE && rb == 0) sm.vin[p] = vin;
    if (WU && p < 32) sm.rowab[r0 + p] = make_int2(lds_addr(codes) + roff, rbits);
    __syncthreads();  // codes staged, per-row constants ready
    if constexpr (WU) {
      // The rows' widths come from the row table, not from branches: lane p's
      // two fields of a row of width B start at bit 2 B p, so the read address
      // and the decode are arithmetic on B.  All rows' fields are read before
      // any is decoded (the LDS reads overlap; x holds the raw dwords in
      // between).  FP16 rows decode as 16-bit integers here and are redone
      // below.
      if (one == 1) {
        // every row 4 bits: lane p's two fields are byte p of the row, read
        // sign-extended (the high field is then an arithmetic shift)
        const int a0 = R.b0[1] + p;
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          const int v = lds_ld8s(a0 + m * row_bytes<DV, 1>());
          x[2 * m] = c0 * (float)(int)__builtin_amdgcn_sbfe(v, 0, 4);
          x[2 * m + 1] = c1 * (float)(v >> 4);
        }
      } else if (one == 3) {
        // every row 8 bits: lane p's two fields are the 16-bit word p
        const int a0 = R.b0[3] + 2 * p;
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          const uint32_t v = lds_ld16(a0 + m * row_bytes<DV, 3>());
          x[2 * m] = c0 * sbyte_f<0>(v);
          x[2 * m + 1] = c1 * sbyte_f<1>(v);
        }
      } else {
      const uint32_t p2 = 2u * p;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const int2 ab = sm.rowab[r0 + m];
        const uint32_t bp = __umul24((uint32_t)ab.y, p2);
        const int ad = ab.x + (int)((bp >> 5) << 2);
        x[2 * m] = __uint_as_float(lds_ld32(ad));
        x[2 * m + 1] = __uint_as_float(lds_ld32(ad + 4));
      }
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const int2 ab = sm.rowab[r0 + m];
        const uint32_t bp = __umul24((uint32_t)ab.y, p2);
        const uint32_t f = __builtin_amdgcn_alignbit(__float_as_uint(x[2 * m + 1]),
                                                     __float_as_uint(x[2 * m]), bp);
        // (the builtin returns an unsigned type: reinterpret as signed first)
        x[2 * m] = c0 * (float)(int)__builtin_amdgcn_sbfe((int)f, 0, ab.y);
        x[2 * m + 1] = c1 * (float)(int)__builtin_amdgcn_sbfe((int)f, ab.y, ab.y);
      }
      }
      if (R.msk[4]) {  // FP16 rows of the block: their values, times rho
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          if (R.msk[4] & (1u << m)) {
            const uint32_t h2 = lds_ld32(sm.rowab[r0 + m].x + 4 * p);
            const float f = sm.rowc[4][r0 + m];
            x[2 * m] = f * half_from_bits(h2);
            x[2 * m + 1] = f * half_from_bits(h2 >> 16);
          }
        }
      }
    } else {
      fresh_masks<WU>(R);
      int rda[5];
      lane_addrs<false>(R, p, rda);
      // all rows' fields are read before any is decoded, so the LDS reads of
      // the 32 rows overlap: the width only selects the address, and one
      // two-dword read (outside the branches) serves every width; x holds the
      // raw dwords in between
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        int ad = 0;
        by_class(R, m, [&](auto w) {
          constexpr int C = decltype(w)::idx;
          ad = rda[C] + m * row_bytes<DV, C>();
        });
        x[2 * m] = __uint_as_float(lds_ld32(ad));
        x[2 * m + 1] = __uint_as_float(lds_ld32(ad + 4));
      }
      fresh_masks<WU>(R);
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        by_class(R, m, [&](auto w) {
          constexpr int B = decltype(w)::bits;
          float z0, z1;
          decode_pair<B>(__float_as_uint(x[2 * m]), __float_as_uint(x[2 * m + 1]), p, z0, z1);
          if constexpr (B == 16) {
            const float f = sm.rowc[4][r0 + m];
            x[2 * m] = f * z0;
            x[2 * m + 1] = f * z1;
          } else {
            x[2 * m] = c0 * z0;
            x[2 * m + 1] = c1 * z1;
          }
        });
      }
    }
    if constexpr (OP == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float f = sm.rowc[3][r0 + m];
        *reinterpret_cast<float2*>(S + rkey[r0 + m] * DV + j0) = make_float2(f * x[2 * m], f * x[2 * m + 1]);
      }
      return;
    }
    // pass 1: delta_j = sum_s kappa_s x_sj
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sm.rowc[0][r0 + m]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a0 = fmaf(kv[u], x[2 * (m + u)], a0);
        a1 = fmaf(kv[u], x[2 * (m + u) + 1], a1);
      }
    }
    sm.colA[rb][p] = make_float2(a0, a1);
    __syncthreads();  // all rows unpacked: the code buffer may hold the transpose
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      d0 += sm.colA[r][p].x;
      d1 += sm.colA[r][p].y;
    }
    const float2 vv = EARLY_V ? sm.vin[p] : *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float e0 = vv.x - d0, e1 = vv.y - d1;
    // pass 2: Xt = x + gamma_s e_j, readout partials
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.rowc[1][r0 + m]);
      const float4 t4 = *reinterpret_cast<const float4*>(&sm.rowc[2][r0 + m]);
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, tv4[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v0 = fmaf(gv[u], e0, x[2 * (m + u)]);
        const float v1 = fmaf(gv[u], e1, x[2 * (m + u) + 1]);
        x[2 * (m + u)] = v0;
        x[2 * (m + u) + 1] = v1;
        y0 = fmaf(tv4[u], v0, y0);
        y1 = fmaf(tv4[u], v1, y1);
      }
    }
    sm.colB[rb][p] = make_float2(y0, y1);
  }
  // row statistics of Xt (integer rows), 16 rows at a time through a
  // per-wave transpose in the dynamic buffer; every lane ends up holding the
  // sum of row (p & 15) of the half, and the 32 owner lanes then derive the
  // stored scales of the block's rows in one pass
  float sh[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      rowt[rb][m][p] = fabsf(x[2 * (16 * hf + m)]) + fabsf(x[2 * (16 * hf + m) + 1]);
    wave_sync();
    const int mm = p & 15, part = p >> 4;
    float s = lds_fold16<false>(&rowt[rb][mm][part * 16]);
    s = parts_sum<NP>(s);
    sh[hf] = s;
    wave_sync();
  }
  if (p < 32) {
    // (the row index is laundered so that the address of r_ptr[si] is formed
    // here rather than kept live from the row-scale load)
    const int si = opaque(r0 + p);
    const float s = p < 16 ? sh[0] : sh[1];
    const float rp = sm.rowc[3][si], qb = sm.rowc[7][si];
    if (qb == 0.f) {  // FP16 row
      r_ptr[si] = __float2half_rn(0.0f);
      sm.rowc[4][si] = rp;  // FP16 rows: X = Xt (row factor 1)
      sm.rowc[5][si] = 0.f;
      sm.rowc[6][si] = 0.f;
    } else {
      const float wi = sm.rowc[5][si], iq = frcp(qb);
      // the hardware square root (1 ulp) only feeds an FP16 rounding
      const float ri =
          fp16_scale(__builtin_amdgcn_sqrtf(rp * s * (1.0f / (float)DV) * sm.rowc[6][si]));
      r_ptr[si] = __float2half_rn(ri);
      sm.rowc[4][si] = rp * frcp(ri);
      const float lam = wi * wi * ri * ri * iq;
      sm.rowc[5][si] = lam;
      sm.rowc[6][si] = lam * iq;
    }
  }
  wave_sync();
  fresh_masks<WU>(R);
  // pass 3: P = X / r on integer rows (column absmax), X on FP16 rows
  float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; m += 4) {
    const float4 f4 = *reinterpret_cast<const float4*>(&sm.rowc[4][r0 + m]);
    const float fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[2 * (m + u)] *= fv[u];
      x[2 * (m + u) + 1] *= fv[u];
    }
  }
  if (R.msk[4] == 0u) {  // no FP16 rows in the block (the common case)
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      mx0 = fmaxf(mx0, fabsf(x[2 * m]));
      mx1 = fmaxf(mx1, fabsf(x[2 * m + 1]));
    }
  } else {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if (!(R.msk[4] & (1u << m))) {
        mx0 = fmaxf(mx0, fabsf(x[2 * m]));
        mx1 = fmaxf(mx1, fabsf(x[2 * m + 1]));
      }
    }
  }
  sm.colM[rb][p] = make_float2(mx0, mx1);
  __syncthreads();
  if (OP == OP_DECODE && rb == 0) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      s0 += sm.colB[r][p].x;
      s1 += sm.colB[r][p].y;
    }
    *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(s0, s1);
  }
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    m0 = fmaxf(m0, sm.colM[r][p].x);
    m1 = fmaxf(m1, sm.colM[r][p].y);
  }
  const float cz0 = fp16_scale(m0), cz1 = fp16_scale(m1);
  const float ic0 = frcp(cz0), ic1 = frcp(cz1);
  // below the FP16 maximum every code lies within +-q_b unclamped; a wave
  // holding a saturated column clamps all its codes (a no-op on the others)
  const bool sat = __ballot(fmaxf(m0, m1) > kFp16Max) != 0ull;
  // pass 4: codes and the refit sums; the new codes go into the staged head
  float N0 = 0.f, N1 = 0.f, D0 = 0.f, D1 = 0.f;
  float mgc = kMagic;
  asm volatile("" : "+s"(mgc));
  fresh_masks<WU>(R);
  if constexpr (WU) {
    if (sat)
      codes_refit_wu<DK, DV, true>(x, R, &sm.rowc[5][r0], ic0, ic1, mgc, p, N0, N1, D0, D1);
    else if (one == 1)
      codes_refit_one<DK, DV, 4>(x, R, &sm.rowc[5][r0], ic0, ic1, mgc, p, N0, N1, D0, D1);
    else if (one == 3)
      codes_refit_one<DK, DV, 8>(x, R, &sm.rowc[5][r0], ic0, ic1, mgc, p, N0, N1, D0, D1);
    else
      codes_refit_wu<DK, DV, false>(x, R, &sm.rowc[5][r0], ic0, ic1, mgc, p, N0, N1, D0, D1);
  } else {
    if (sat)
      codes_refit<DK, DV, true>(x, R, &sm.rowc[5][r0], &sm.rowc[6][r0], &sm.rowc[7][r0], ic0, ic1,
                                mgc, p, N0, N1, D0, D1);
    else
      codes_refit<DK, DV, false>(x, R, &sm.rowc[5][r0], &sm.rowc[6][r0], &sm.rowc[7][r0], ic0,
                                 ic1, mgc, p, N0, N1, D0, D1);
  }
  sm.colC[rb][p] = make_float4(N0, N1, D0, D1);
  __syncthreads();
  for (int i = t * 16; i < code_bytes; i += NT * 16)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(codes + i),
                                reinterpret_cast<u32x4*>(base + i));
  if (rb == 0) {
    float n0 = 0.f, n1 = 0.f, dd0 = 0.f, dd1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float4 c = sm.colC[r][p];
      n0 += c.x;
      n1 += c.y;
      dd0 += c.z;
      dd1 += c.w;
    }
    c_ptr[j0] = __float2half_rn(dd0 > 0.f ? fp16_scale(n0 * frcp(dd0)) : cz0);
    c_ptr[j0 + 1] = __float2half_rn(dd1 > 0.f ? fp16_scale(n1 * frcp(dd1)) : cz1);
  }
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  constexpr int NP = DV / 2, NRB = DK / 32;
  const size_t dyn = (size_t)dyn_bytes<DK, DV>(a.P.max_code_bytes);
  const dim3 grid(a.n_tiles), block(NRB * NP);
  switch (a.op) {
    case OP_DECODE: hipLaunchKernelGGL((kda_tile_kernel<DK, DV, OP_DECODE>), grid, block, dyn, s, a); break;
    case OP_PACK: hipLaunchKernelGGL((kda_tile_kernel<DK, DV, OP_PACK>), grid, block, dyn, s, a); break;
    case OP_UNPACK: hipLaunchKernelGGL((kda_tile_kernel<DK, DV, OP_UNPACK>), grid, block, dyn, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_kda(const TileArgs& a, hipStream_t s) {
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(a, s);
  return hipErrorInvalidValue;
}
