// Fused quantized decode step for STEP KDA heads: channel-wise retention
// D = diag(d), bit width chosen per key row (STEPQuant Sec. 4, unit = key
// row for KDA), FP16 pivot rows, one column-scale vector c shared by all
// integer rows of the head (App. D: "codebook normalization fixed by
// precision", so rows of different widths share c).
//
// Storage rows are ordered by (width, key row) and kept row-major, so a
// head is a run of variable-length rows.  The workgroup stages the packed
// head in LDS with coalesced 16-byte copies, every lane extracts its two
// columns of its 32 storage rows (the row width is uniform across the wave
// at each row), and the new codes are assembled in LDS (bit-field OR) and
// copied back with 16-byte stores.  The arithmetic is the GDN kernel's with
// per-row q_b and per-row retention, in storage-row order; per-row inputs
// (d, k, q, w) are gathered through the storage permutation.
#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV>
struct SmemKda {
  float rowc[5][DK];
  float rho[DK];
  int bits[DK];
  int off[DK];
  float2 colA[DK / 32][DV / 2];
  float2 colB[DK / 32][DV / 2];
  float4 colC[DK / 32][DV / 2];
  union {
    uint32_t codes[DK * DV / 2];             // packed head (at most all-FP16 rows)
    float rowt[DK / 32][32][DV / 2 + 1];     // row partials, transposed
  } u;
};

// Two b-bit fields (columns 2p, 2p+1) of a row stored at byte `off`.
__device__ __forceinline__ void read_pair(const uint32_t* codes, int off, int b, int p,
                                          float& z0, float& z1) {
  if (b == 16) {
    const uint32_t w = codes[(off >> 2) + p];
    z0 = half_from_bits(w);
    z1 = half_from_bits(w >> 16);
    return;
  }
  const int bit = 2 * p * b;                  // first bit of the pair in the row
  const int wi = (off >> 2) + (bit >> 5), sh = bit & 31;
  uint64_t v = codes[wi];
  if (sh + 2 * b > 32) v |= (uint64_t)codes[wi + 1] << 32;
  const uint32_t f = (uint32_t)(v >> sh);
  const int s = 32 - b;
  z0 = (float)((int32_t)(f << s) >> s);
  z1 = (float)((int32_t)((f >> b) << s) >> s);
}

__device__ __forceinline__ void write_pair(uint32_t* codes, int off, int b, int p, float u0,
                                           float u1) {
  if (b == 16) {
    codes[(off >> 2) + p] = half_bits(u0) | (half_bits(u1) << 16);
    return;
  }
  const uint32_t m = (1u << b) - 1u;
  const uint64_t f = (uint64_t)(((uint32_t)(int32_t)u0 & m) | (((uint32_t)(int32_t)u1 & m) << b));
  const int bit = 2 * p * b;
  const int wi = (off >> 2) + (bit >> 5), sh = bit & 31;
  const uint64_t v = f << sh;
  atomicOr(&codes[wi], (uint32_t)v);
  if (sh + 2 * b > 32) atomicOr(&codes[wi + 1], (uint32_t)(v >> 32));
}

template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void kda_tile_kernel(TileArgs a) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT;
  __shared__ SmemKda<DK, DV> sm;
  const int tile = blockIdx.x;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (a.op == OP_DECODE && t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    return;
  }
  const int op = a.op;
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  const int* rkey = a.P.row_key + h * DK;
  const int code_bytes = a.P.r_off[h];
  __half* r_ptr = reinterpret_cast<__half*>(base + a.P.r_off[h]);
  __half* c_ptr = reinterpret_cast<__half*>(base + a.P.c_off[h]);
  if (t < DK) {
    sm.bits[t] = a.P.row_bits[h * DK + t];
    sm.off[t] = a.P.row_off[h * DK + t];
  }
  float x[64];
  float c0 = 1.f, c1 = 1.f;
  if (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int key = rkey[32 * rb + m];
      const float2 v2 = *reinterpret_cast<const float2*>(X + key * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    if (t < DK) sm.rho[t] = 1.0f;
  } else {
    for (int i = t * 16; i < code_bytes; i += NT * 16)
      *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(sm.u.codes) + i) =
          *reinterpret_cast<const uint4*>(base + i);
    c0 = __half2float(c_ptr[j0]);
    c1 = __half2float(c_ptr[j0 + 1]);
    if (t < DK) {
      const int b = a.P.row_bits[h * DK + t], key = rkey[t];
      const bool piv = b == 16;
      const float qb = piv ? 1.f : (float)((1 << (b - 1)) - 1);
      const float sc = piv ? 1.f : __half2float(r_ptr[t]) / qb;
      if (op == OP_UNPACK) {
        sm.rho[t] = sc;
      } else {
        const float d = a.gate[tk + key];
        const float kk = a.k[tk + key], qq = a.q[tk + key], bk = a.beta[tile] * kk;
        const float rho = d * sc;
        const float rp = fmaxf(rho, fmaxf(fabsf(bk) * 0x1p-60f, 0x1p-100f));
        sm.rowc[0][t] = kk * rho;
        sm.rowc[1][t] = bk / rp;
        sm.rowc[2][t] = qq * rp;
        sm.rho[t] = rp;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int s = 32 * rb + m;
      read_pair(sm.u.codes, sm.off[s], sm.bits[s], p, x[2 * m], x[2 * m + 1]);
    }
    if (op == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const int s = 32 * rb + m;
        const bool piv = sm.bits[s] == 16;
        const float f0 = piv ? 1.f : sm.rho[s] * c0, f1 = piv ? 1.f : sm.rho[s] * c1;
        *reinterpret_cast<float2*>(S + rkey[s] * DV + j0) = make_float2(f0 * x[2 * m], f1 * x[2 * m + 1]);
      }
      return;
    }
    // pass 1: delta_j = sum_s kappa_s c'_sj z_sj  (c' = c_j, or 1 on pivot rows)
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int s = 32 * rb + m;
      const bool piv = sm.bits[s] == 16;
      const float kap = sm.rowc[0][s];
      a0 = fmaf(kap * (piv ? 1.f : c0), x[2 * m], a0);
      a1 = fmaf(kap * (piv ? 1.f : c1), x[2 * m + 1], a1);
    }
    sm.colA[rb][p] = make_float2(a0, a1);
    __syncthreads();
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      d0 += sm.colA[r][p].x;
      d1 += sm.colA[r][p].y;
    }
    const float2 vv = *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float e0 = vv.x - d0, e1 = vv.y - d1;
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int s = 32 * rb + m;
      const bool piv = sm.bits[s] == 16;
      const float gam = sm.rowc[1][s], th = sm.rowc[2][s];
      const float v0 = fmaf(piv ? 1.f : c0, x[2 * m], gam * e0);
      const float v1 = fmaf(piv ? 1.f : c1, x[2 * m + 1], gam * e1);
      x[2 * m] = v0;
      x[2 * m + 1] = v1;
      y0 = fmaf(th, v0, y0);
      y1 = fmaf(th, v1, y1);
    }
    sm.colB[rb][p] = make_float2(y0, y1);
  }
  __syncthreads();  // codes buffer no longer needed: rowt may overwrite it
#pragma unroll
  for (int m = 0; m < 32; ++m)
    sm.u.rowt[rb][m][p] = fabsf(x[2 * m]) + fabsf(x[2 * m + 1]);
  __syncthreads();
  if (op == OP_DECODE && rb == 0) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      s0 += sm.colB[r][p].x;
      s1 += sm.colB[r][p].y;
    }
    *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(s0, s1);
  }
  {
    constexpr int LPR = NP / 32;
    const int m = p & 31, part = p >> 5;
    float s = 0.f;
#pragma unroll 8
    for (int pp = 0; pp < 32; ++pp) s += sm.u.rowt[rb][m][part * 32 + pp];
    if constexpr (LPR == 2) s += __shfl_xor(s, 32);
    if (part == 0) {
      const int si = 32 * rb + m;
      const int b = sm.bits[si];
      const float rp = sm.rho[si];
      if (b == 16) {
        r_ptr[si] = __float2half_rn(0.0f);
        sm.rowc[3][si] = 0.f;
        sm.rowc[4][si] = 0.f;
      } else {
        const float qb = (float)((1 << (b - 1)) - 1);
        const float wi = a.P.w[h * DK + rkey[si]];
        const float ri = fp16_scale(sqrtf(rp * s / (float)DV / wi));
        r_ptr[si] = __float2half_rn(ri);
        sm.rowc[3][si] = rp / ri;
        sm.rowc[4][si] = wi * wi * ri * ri / qb;
      }
    }
  }
  __syncthreads();
  // pass 3: P = X / r on integer rows, column absmax; pivot rows -> X
  float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int s = 32 * rb + m;
    if (sm.bits[s] == 16) {
      x[2 * m] *= sm.rho[s];
      x[2 * m + 1] *= sm.rho[s];
    } else {
      const float pi = sm.rowc[3][s];
      x[2 * m] *= pi;
      x[2 * m + 1] *= pi;
      mx0 = fmaxf(mx0, fabsf(x[2 * m]));
      mx1 = fmaxf(mx1, fabsf(x[2 * m + 1]));
    }
  }
  sm.colA[rb][p] = make_float2(mx0, mx1);
  __syncthreads();
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    m0 = fmaxf(m0, sm.colA[r][p].x);
    m1 = fmaxf(m1, sm.colA[r][p].y);
  }
  const float cz0 = fp16_scale(m0), cz1 = fp16_scale(m1);
  const float ic0 = 1.0f / cz0, ic1 = 1.0f / cz1;
  // the codes buffer is rebuilt from zero (bit fields are OR-ed in)
  for (int i = t; i < DK * DV / 2; i += NT) sm.u.codes[i] = 0u;
  __syncthreads();
  float N0 = 0.f, N1 = 0.f, D0 = 0.f, D1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int s = 32 * rb + m;
    const int b = sm.bits[s];
    if (b == 16) {
      write_pair(sm.u.codes, sm.off[s], 16, p, x[2 * m], x[2 * m + 1]);
      continue;
    }
    const float qb = (float)((1 << (b - 1)) - 1);
    const float lam = sm.rowc[4][s];
    const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
    const float z0 = fminf(fmaxf(rintf(pv0 * (qb * ic0)), -qb), qb);
    const float z1 = fminf(fmaxf(rintf(pv1 * (qb * ic1)), -qb), qb);
    const float t0 = lam * z0, t1 = lam * z1;
    N0 = fmaf(t0, pv0, N0);
    N1 = fmaf(t1, pv1, N1);
    D0 = fmaf(t0 / qb, z0, D0);
    D1 = fmaf(t1 / qb, z1, D1);
    write_pair(sm.u.codes, sm.off[s], b, p, z0, z1);
  }
  sm.colC[rb][p] = make_float4(N0, N1, D0, D1);
  __syncthreads();
  for (int i = t * 16; i < code_bytes; i += NT * 16)
    *reinterpret_cast<uint4*>(base + i) =
        *reinterpret_cast<const uint4*>(reinterpret_cast<unsigned char*>(sm.u.codes) + i);
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
    c_ptr[j0] = __float2half_rn(dd0 > 0.f ? fp16_scale(n0 / dd0) : cz0);
    c_ptr[j0 + 1] = __float2half_rn(dd1 > 0.f ? fp16_scale(n1 / dd1) : cz1);
  }
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kda_tile_kernel<DK, DV>), dim3(a.n_tiles), dim3((DK / 32) * (DV / 2)), 0, s, a);
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
