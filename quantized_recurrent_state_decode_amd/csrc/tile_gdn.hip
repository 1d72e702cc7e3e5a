// Fused quantized decode step for tile-uniform heads: uniform rowwise INT-b
// heads and STEP GDN heads (mixed width per head, FP16 pivot heads).
//
// One workgroup owns one (slot, head) tile.  Lane (rb, p) holds rows
// 32 rb .. 32 rb + 31 of columns 2p, 2p+1 in registers, so the column
// reductions of the step (k^T S, X^T q, max_i, the refit sums) are mostly
// lane-local and only combine the row blocks through LDS; the row
// reduction m_i goes through an LDS transpose.
//
// Arithmetic (STEPQuant Sec. 3 Eq. 1/4, Sec. 4.3, App. A and C):
//   S_hat_ij = rho_i c_j z_ij                (rho_i = alpha r_i / q_b, retained)
//   delta_j  = sum_i k_i S_hat_ij, e_j = v_j - delta_j
//   X_ij     = S_hat_ij + beta k_i e_j,  y_j = sum_i q_i X_ij
//   r_i = FP16(sqrt(mean_j |X_ij| / w_i)), c0_j = FP16(max_i |X_ij| / r_i)
//   z_ij = clamp(rne(q_b X_ij / (r_i c0_j)), +-q_b)
//   c_j  = FP16(sum_i w_i^2 r_i zt X / sum_i w_i^2 r_i^2 zt^2), zt = z / q_b
// The kernel keeps each row divided by rho_i (Xt = X / rho_i) so that the
// reconstruction + update costs two fused multiply-adds per element:
//   Xt_ij = c_j (z_ij + off) + (gamma_i e_j - off c_j),  gamma_i = beta k_i / rho_i
// where z + off is the offset-binary code produced by the unpacker.
#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV>
struct SmemGdn {
  float rowc[5][DK];                          // per-row constants of the current pass
  float rho[DK];                              // row factor of Xt
  float2 colA[DK / 32][DV / 2];               // column partials per row block
  float2 colB[DK / 32][DV / 2];
  float4 colC[DK / 32][DV / 2];
  float rowt[DK / 32][32][DV / 2 + 1];        // row partials, transposed
};

// Quantized (b in {2,4,6,8}) head: uniform (UNI) or STEP dual-axis.
template <int DK, int DV, int BITS, bool UNI>
__device__ __forceinline__ void quant_tile(const TileArgs& a, const int tile, const int h,
                                           unsigned char* base, SmemGdn<DK, DV>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  constexpr float QB = (float)((1 << (BITS - 1)) - 1);
  constexpr float OFF = (float)(1 << (BITS - 1));
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  const int op = a.op;
  __half* rs_ptr = reinterpret_cast<__half*>(base + a.P.r_off[h]);
  __half* c_ptr = UNI ? nullptr : reinterpret_cast<__half*>(base + a.P.c_off[h]);
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;

  float x[64];
  if (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float2 v2 = *reinterpret_cast<const float2*>(X + (32 * rb + m) * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    if (t < DK) sm.rho[t] = 1.0f;
  } else {
    uint32_t wd[2 * BITS];
    load_chunk<BITS, NP>(base, rb, p, wd);
    float c0 = 1.0f, c1 = 1.0f;
    if (!UNI) {
      c0 = __half2float(c_ptr[j0]);
      c1 = __half2float(c_ptr[j0 + 1]);
    }
    if (t < DK) {
      const float rsi = __half2float(rs_ptr[t]);
      const float sc = UNI ? rsi : rsi / QB;  // dequantisation row factor
      if (op == OP_UNPACK) {
        sm.rho[t] = sc;
      } else {
        const float alpha = a.gate[tile];
        const float kk = a.k[tk + t], qq = a.q[tk + t], bk = a.beta[tile] * kk;
        const float rho = alpha * sc;
        // a vanishing retention keeps the division finite; the dropped part
        // (rp - rho) c_j z_ij is below 2^-60 of the write term
        const float rp = fmaxf(rho, fmaxf(fabsf(bk) * 0x1p-60f, 0x1p-100f));
        sm.rowc[0][t] = kk * rho;  // kappa: key retrieval weight
        sm.rowc[1][t] = bk / rp;   // gamma
        sm.rowc[2][t] = qq * rp;   // theta: readout weight on Xt
        sm.rho[t] = rp;
      }
    }
    unpack_codes<BITS>(wd, x);
    __syncthreads();
    if (op == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const int i = 32 * rb + m;
        const float sc = sm.rho[i];
        *reinterpret_cast<float2*>(S + i * DV + j0) =
            make_float2(sc * c0 * (x[2 * m] - OFF), sc * c1 * (x[2 * m + 1] - OFF));
      }
      return;
    }
    // pass 1: key retrieval delta_j = c_j sum_i kappa_i (u_ij - off)
    float a0 = 0.f, a1 = 0.f, ks = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float kap = sm.rowc[0][32 * rb + m];
      a0 = fmaf(kap, x[2 * m], a0);
      a1 = fmaf(kap, x[2 * m + 1], a1);
      ks += kap;
    }
    sm.colA[rb][p] = make_float2(fmaf(-OFF, ks, a0), fmaf(-OFF, ks, a1));
    __syncthreads();
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float2 c = sm.colA[r][p];
      d0 += c.x;
      d1 += c.y;
    }
    const float2 vv = *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float e0 = vv.x - c0 * d0, e1 = vv.y - c1 * d1;
    // pass 2: Xt, readout partials
    const float o0 = -OFF * c0, o1 = -OFF * c1;
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int i = 32 * rb + m;
      const float gam = sm.rowc[1][i], th = sm.rowc[2][i];
      const float v0 = fmaf(c0, x[2 * m], fmaf(gam, e0, o0));
      const float v1 = fmaf(c1, x[2 * m + 1], fmaf(gam, e1, o1));
      x[2 * m] = v0;
      x[2 * m + 1] = v1;
      y0 = fmaf(th, v0, y0);
      y1 = fmaf(th, v1, y1);
    }
    sm.colB[rb][p] = make_float2(y0, y1);
  }
  // row statistics of Xt: sum |.| (STEP) or max |.| (uniform)
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float u0 = fabsf(x[2 * m]), u1 = fabsf(x[2 * m + 1]);
    sm.rowt[rb][m][p] = UNI ? fmaxf(u0, u1) : u0 + u1;
  }
  __syncthreads();
  if (op == OP_DECODE && rb == 0) {
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float2 c = sm.colB[r][p];
      y0 += c.x;
      y1 += c.y;
    }
    *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(y0, y1);
  }
  {
    constexpr int LPR = NP / 32;  // lanes per row in the transpose step
    const int m = p & 31, part = p >> 5;
    float s = 0.f;
#pragma unroll 8
    for (int pp = 0; pp < 32; ++pp) {
      const float vv = sm.rowt[rb][m][part * 32 + pp];
      s = UNI ? fmaxf(s, vv) : s + vv;
    }
    if constexpr (LPR == 2) {
      const float o = __shfl_xor(s, 32);
      s = UNI ? fmaxf(s, o) : s + o;
    }
    if (part == 0) {
      const int i = 32 * rb + m;
      const float rp = sm.rho[i];
      if (UNI) {
        const float si = fp16_scale(rp * s / QB);
        rs_ptr[i] = __float2half_rn(si);
        sm.rowc[3][i] = rp / si;  // code pre-value = Xt * sigma_i
      } else {
        const float wi = a.P.w[h * DK + i];
        const float ri = fp16_scale(sqrtf(rp * s / (float)DV / wi));
        rs_ptr[i] = __float2half_rn(ri);
        sm.rowc[3][i] = rp / ri;                  // pi: X / r_i = Xt * pi_i
        sm.rowc[4][i] = wi * wi * ri * ri / QB;   // lambda: refit weight
      }
    }
  }
  __syncthreads();
  if constexpr (UNI) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float sg = sm.rowc[3][32 * rb + m];
      x[2 * m] = fminf(fmaxf(rintf(fmaf(x[2 * m], sg, OFF)), OFF - QB), OFF + QB);
      x[2 * m + 1] = fminf(fmaxf(rintf(fmaf(x[2 * m + 1], sg, OFF)), OFF - QB), OFF + QB);
    }
  } else {
    // pass 3: P = X / r_i and the column absmax
    float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float pi = sm.rowc[3][32 * rb + m];
      x[2 * m] *= pi;
      x[2 * m + 1] *= pi;
      mx0 = fmaxf(mx0, fabsf(x[2 * m]));
      mx1 = fmaxf(mx1, fabsf(x[2 * m + 1]));
    }
    sm.colA[rb][p] = make_float2(mx0, mx1);
    __syncthreads();
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float2 c = sm.colA[r][p];
      m0 = fmaxf(m0, c.x);
      m1 = fmaxf(m1, c.y);
    }
    const float cz0 = fp16_scale(m0), cz1 = fp16_scale(m1);
    const float tau0 = QB / cz0, tau1 = QB / cz1;
    // pass 4: codes and the fixed-code weighted least-squares column sums
    float N0 = 0.f, N1 = 0.f, D0 = 0.f, D1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float lam = sm.rowc[4][32 * rb + m];
      const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
      const float u0 = fminf(fmaxf(rintf(fmaf(pv0, tau0, OFF)), OFF - QB), OFF + QB);
      const float u1 = fminf(fmaxf(rintf(fmaf(pv1, tau1, OFF)), OFF - QB), OFF + QB);
      const float z0 = u0 - OFF, z1 = u1 - OFF;
      const float t0 = lam * z0, t1 = lam * z1;
      N0 = fmaf(t0, pv0, N0);
      N1 = fmaf(t1, pv1, N1);
      D0 = fmaf(t0, z0, D0);
      D1 = fmaf(t1, z1, D1);
      x[2 * m] = u0;
      x[2 * m + 1] = u1;
    }
    sm.colC[rb][p] = make_float4(N0, N1, D0, D1);
    __syncthreads();
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
      const float cf0 = dd0 > 0.f ? fp16_scale(QB * n0 / dd0) : cz0;
      const float cf1 = dd1 > 0.f ? fp16_scale(QB * n1 / dd1) : cz1;
      c_ptr[j0] = __float2half_rn(cf0);
      c_ptr[j0 + 1] = __float2half_rn(cf1);
    }
  }
  uint32_t wd[2 * BITS];
  pack_codes<BITS>(x, wd);
  store_chunk<BITS, NP>(base, rb, p, wd);
}

// FP16 pivot head of a STEP GDN plan: the state is kept as FP16 values.
template <int DK, int DV>
__device__ __forceinline__ void pivot_tile(const TileArgs& a, const int tile, const int h,
                                           unsigned char* base, SmemGdn<DK, DV>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  const int op = a.op;
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  float x[64];
  if (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float2 v2 = *reinterpret_cast<const float2*>(X + (32 * rb + m) * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
  } else {
    uint32_t wd[32];
    load_chunk<16, NP>(base, rb, p, wd);
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      x[2 * m] = half_from_bits(wd[m]);
      x[2 * m + 1] = half_from_bits(wd[m] >> 16);
    }
    if (op == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m)
        *reinterpret_cast<float2*>(S + (32 * rb + m) * DV + j0) = make_float2(x[2 * m], x[2 * m + 1]);
      return;
    }
    const float alpha = a.gate[tile];
    if (t < DK) {
      const float kk = a.k[tk + t];
      sm.rowc[0][t] = alpha * kk;
      sm.rowc[1][t] = a.beta[tile] * kk;
      sm.rowc[2][t] = a.q[tk + t];
    }
    __syncthreads();
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float kap = sm.rowc[0][32 * rb + m];
      a0 = fmaf(kap, x[2 * m], a0);
      a1 = fmaf(kap, x[2 * m + 1], a1);
    }
    sm.colA[rb][p] = make_float2(a0, a1);
    __syncthreads();
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float2 c = sm.colA[r][p];
      d0 += c.x;
      d1 += c.y;
    }
    const float2 vv = *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float e0 = vv.x - d0, e1 = vv.y - d1;
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int i = 32 * rb + m;
      const float bk = sm.rowc[1][i], qq = sm.rowc[2][i];
      const float v0 = fmaf(alpha, x[2 * m], bk * e0);
      const float v1 = fmaf(alpha, x[2 * m + 1], bk * e1);
      x[2 * m] = v0;
      x[2 * m + 1] = v1;
      y0 = fmaf(qq, v0, y0);
      y1 = fmaf(qq, v1, y1);
    }
    sm.colB[rb][p] = make_float2(y0, y1);
    __syncthreads();
    if (rb == 0) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        const float2 c = sm.colB[r][p];
        s0 += c.x;
        s1 += c.y;
      }
      *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(s0, s1);
    }
  }
  uint32_t wd[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) wd[m] = half_bits(x[2 * m]) | (half_bits(x[2 * m + 1]) << 16);
  store_chunk<16, NP>(base, rb, p, wd);
}

template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void gdn_tile_kernel(TileArgs a) {
  __shared__ SmemGdn<DK, DV> sm;
  const int tile = blockIdx.x;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (a.op == OP_DECODE) {
      const int t = threadIdx.x;
      if (t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    }
    return;
  }
  const int bits = a.P.head_bits[h];
  const bool uni = a.P.mode == SQ_MODE_UNIFORM;
  switch (bits) {
    case 2:
      if (uni) quant_tile<DK, DV, 2, true>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 2, false>(a, tile, h, base, sm);
      break;
    case 4:
      if (uni) quant_tile<DK, DV, 4, true>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 4, false>(a, tile, h, base, sm);
      break;
    case 6:
      if (uni) quant_tile<DK, DV, 6, true>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 6, false>(a, tile, h, base, sm);
      break;
    case 8:
      if (uni) quant_tile<DK, DV, 8, true>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 8, false>(a, tile, h, base, sm);
      break;
    case 16:
      if (!uni) pivot_tile<DK, DV>(a, tile, h, base, sm);
      break;
    default:
      break;
  }
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((gdn_tile_kernel<DK, DV>), dim3(a.n_tiles), dim3((DK / 32) * (DV / 2)), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gdn(const TileArgs& a, hipStream_t s) {
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(a, s);
  return hipErrorInvalidValue;
}
