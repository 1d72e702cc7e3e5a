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
  // per-row constants: 0 kappa, 1 gamma, 2 theta, 3 rho (row factor of Xt),
  // 4 1 / w (STEP, until the row-scale pass), then pi (X / r = Xt pi) or
  // sigma (uniform), 5 the impact factor w (STEP), then lambda (refit weight)
  float rowc[6][DK];
  float ksum[DK / 32];                        // sum of kappa per row block
  float2 colA[DK / 32][DV / 2];               // column partials per row block
  float2 colB[DK / 32][DV / 2];
  float2 colM[DK / 32][DV / 2];
  float4 colC[DK / 32][DV / 2];               // (row block 0's part holds the token's v until pass 4)
  alignas(16) float rowt[DK / 32][16][RowT<DV / 2>::S];  // row partials of 16 rows, transposed
};



// Rows m .. m + R - 1 of both columns go into one output dword: R = 4 at 4 bits
// (rows 4d .. 4d+3), 2 at 8 bits, 8 at 2 bits.  6-bit fields straddle dwords
// and are packed after the loop.
template <int BITS>
__device__ __forceinline__ uint32_t pack_rows(const float* mg) {
  if constexpr (BITS == 4) {
    const uint32_t lo = low_bytes4(mg[0], mg[2], mg[4], mg[6]);
    const uint32_t hi = low_bytes4(mg[1], mg[3], mg[5], mg[7]);
    return (lo & 0x0f0f0f0fu) | ((hi << 4) & 0xf0f0f0f0u);
  } else if constexpr (BITS == 8) {
    return low_bytes4(mg[0], mg[1], mg[2], mg[3]);
  } else {
    uint32_t acc = 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc |= (low_bytes4(mg[s], mg[4 + s], mg[8 + s], mg[12 + s]) & 0x03030303u) << (2 * s);
    return acc;
  }
}

// Codes by magic rounding and the fixed-code weighted least-squares column
// sums (N_j, D_j), packed into w as they are produced.
template <int BITS, bool CLAMP>
__device__ __forceinline__ void codes_refit(float (&x)[64], int lam, float tau0, float tau1,
                                            float4& nd, uint32_t (&w)[2 * BITS]) {
  constexpr float QB = (float)((1 << (BITS - 1)) - 1);
  constexpr int R = BITS == 6 ? 8 : 16 / BITS;   // rows per output dword (3 dwords at 6 bits)
  constexpr int RG = R < 4 ? 4 : R;              // rows per ordered group
  float N0 = 0.f, N1 = 0.f, D0 = 0.f, D1 = 0.f;
#pragma unroll
  for (int g = 0; g < 32; g += RG) {
    // at 2 and 6 bits (8-row groups) order the work group by group so that rounded
    // values are packed while their rows are still the only ones in flight;
    // 4- and 8-bit codes schedule within the register budget unaided
    if constexpr (BITS == 2 || BITS == 6) {
#pragma unroll
      for (int k = 0; k < 2 * RG; ++k) asm volatile("" : "+v"(x[2 * g + k]));
    }
#pragma unroll
    for (int m = g; m < g + RG; m += 4) {
      const float4 l4 = lds_ld4(lam + 4 * m);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float pv0 = x[2 * (m + u)], pv1 = x[2 * (m + u) + 1];
        float mg0 = fmaf(pv0, tau0, kMagic), mg1 = fmaf(pv1, tau1, kMagic);
        if constexpr (CLAMP) {  // a column scale saturated at the FP16 maximum
          mg0 = __builtin_amdgcn_fmed3f(mg0, kMagic - QB, kMagic + QB);
          mg1 = __builtin_amdgcn_fmed3f(mg1, kMagic - QB, kMagic + QB);
        }
        const float z0 = mg0 - kMagic, z1 = mg1 - kMagic;
        const float t0 = lv[u] * z0, t1 = lv[u] * z1;
        N0 = fmaf(t0, pv0, N0);
        N1 = fmaf(t1, pv1, N1);
        D0 = fmaf(t0, z0, D0);
        D1 = fmaf(t1, z1, D1);
        x[2 * (m + u)] = mg0;
        x[2 * (m + u) + 1] = mg1;
      }
    }
    if constexpr (BITS == 6) {
      pack6(&x[2 * g], &w[3 * (g / 8)]);
#pragma unroll
      for (int k = 0; k < 3; ++k) asm volatile("" : "+v"(w[3 * (g / 8) + k]));
    } else {
#pragma unroll
      for (int d = g / R; d < (g + RG) / R; ++d) {
        w[d] = pack_rows<BITS>(&x[2 * R * d]);
        asm volatile("" : "+v"(w[d]));
      }
    }
    asm volatile("" : "+v"(N0), "+v"(N1), "+v"(D0), "+v"(D1));
  }
  nd = make_float4(N0, N1, D0, D1);
}

// Uniform rowwise codes: magic rounding of Xt * sigma_i, packed into w.
template <int BITS>
__device__ __forceinline__ void codes_rowwise(float (&x)[64], int sig, uint32_t (&w)[2 * BITS]) {
  constexpr float QB = (float)((1 << (BITS - 1)) - 1);
  constexpr int R = BITS == 6 ? 4 : 16 / BITS;
#pragma unroll
  for (int m = 0; m < 32; m += 4) {
    const float4 s4 = lds_ld4(sig + 4 * m);
    const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        x[2 * (m + u) + c] =
            __builtin_amdgcn_fmed3f(fmaf(x[2 * (m + u) + c], sv[u], kMagic), kMagic - QB, kMagic + QB);
      }
      if constexpr (BITS != 6) {
        const int row = m + u;
        if ((row + 1) % R == 0) w[row / R] = pack_rows<BITS>(&x[2 * (row + 1 - R)]);
      }
    }
  }
  if constexpr (BITS == 6) pack_magic<6>(x, w);
}

// Quantized (b in {2,4,6,8}) head: uniform (UNI) or STEP dual-axis.  LATE:
// the launch is one round of resident workgroups (see EARLY below).
template <int DK, int DV, int BITS, bool UNI, int OP, bool LATE = false>
__device__ __forceinline__ void quant_tile(const TileArgs& a, const int tile, const int h,
                                           unsigned char* base, SmemGdn<DK, DV>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  constexpr float QB = (float)((1 << (BITS - 1)) - 1);
  constexpr float OFF = (float)(1 << (BITS - 1));
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  const int r0 = 32 * rb;                     // first row of this lane's block
  constexpr int op = OP;
  // LDS address of row r0 of the per-row constants (array k at + 4 k DK)
  const int rcb = lds_addr(&sm.rowc[0][r0]);
  __half* rs_ptr = reinterpret_cast<__half*>(base + wuni(a.P.r_off[h]));
  __half* c_ptr = UNI ? nullptr : reinterpret_cast<__half*>(base + wuni(a.P.c_off[h]));
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  // The token's v (needed after the first block barrier) and the impact
  // factors (needed by the row-scale pass) go out with the codes and wait in
  // LDS, so no memory round trip is left on the path after a barrier.  On
  // the other tile shapes the extra live ranges spill, and in a launch that
  // the chip holds in one round of workgroups staging measured slower (all
  // tiles start together, and the start-up burst is the path): both are read
  // where they are used there.
  constexpr bool EARLY = DK == 128 && DV == 128 && !LATE;

  float x[64];
  float y0 = 0.f, y1 = 0.f;
  if (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float2 v2 = *reinterpret_cast<const float2*>(X + (r0 + m) * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    if (p < 32) {
      const int i = r0 + p;
      sm.rowc[3][i] = 1.0f;
      if (!UNI && EARLY) {
        sm.rowc[5][i] = a.P.w[h * DK + i];
        sm.rowc[4][i] = a.P.winv[h * DK + i];
      }
    }
    wave_sync();
  } else {
    // uniform decode reads the codes as binary16 subnormals (u 2^-24): the
    // retrieval weights and column scales that multiply them carry 2^24.  On
    // STEP heads the mixed-precision FMAs made the wave slower despite fewer
    // instructions (more cycles per wave, more waits on LDS issue), and at
    // d_v = 64 (a wave spans two row blocks) the longer live range spills;
    // those tiles convert the codes to floats.
    constexpr bool HC = OP == OP_DECODE && DV == 128 && UNI;
    constexpr float HS = HC ? 0x1p24f : 1.0f;
    uint32_t wd[2 * BITS];
    load_chunk<BITS, NP>(base, rb, p, wd);
    // row block 0 loads the token's v behind the codes
    float2 vin = make_float2(0.f, 0.f);
    if (EARLY && op == OP_DECODE && rb == 0) vin = *reinterpret_cast<const float2*>(a.v + tv + j0);
    float c0 = 1.0f, c1 = 1.0f;
    if (!UNI) {
      c0 = __half2float(c_ptr[j0]);
      c1 = __half2float(c_ptr[j0 + 1]);
    }
    if (p < 32) {
      const int i = r0 + p;
      const float rsi = __half2float(rs_ptr[i]);
      const float sc = UNI ? rsi : rsi * (1.0f / QB);  // dequantisation row factor
      if (op == OP_UNPACK) {
        sm.rowc[3][i] = sc;
      } else {
        const float alpha = wuni(a.gate[tile]);
        const float kk = a.k[tk + i], qq = a.q[tk + i], bk = wuni(a.beta[tile]) * kk;
        const float rho = alpha * sc;
        // a vanishing retention keeps the division finite; the dropped part
        // (rp - rho) c_j z_ij is below 2^-60 of the write term
        const float rp = fmaxf(rho, fmaxf(fabsf(bk) * 0x1p-60f, 0x1p-100f));
        const float kap = kk * rho;
        sm.rowc[0][i] = kap * HS;          // kappa: key retrieval weight
        sm.rowc[1][i] = bk * frcp(rp);     // gamma
        sm.rowc[2][i] = qq * rp;           // theta: readout weight on Xt
        sm.rowc[3][i] = rp;
        if (!UNI && EARLY) {  // the impact factors wait in LDS for the row-scale pass
          sm.rowc[5][i] = a.P.w[h * DK + i];
          sm.rowc[4][i] = a.P.winv[h * DK + i];
        }
        // sum of kappa over the block's 32 rows (offset of the unpacked codes)
        const float ksum = half32_sum_hi(kap);
        if (p == 16) sm.ksum[rb] = ksum;
      }
    }
    // (staged before the unpack: it arrives right behind the codes, and no
    // register stays live across pass 1)
    if (EARLY && op == OP_DECODE && rb == 0) sm.colC[0][p] = make_float4(vin.x, vin.y, 0.f, 0.f);
    uint32_t hc[32];
    if constexpr (HC) unpack_half<BITS>(wd, hc);
    else unpack_offset<BITS>(wd, x);
    // unpacked code n (an offset-binary integer, times 2^-24 when HC)
    auto code = [&](int n) -> float {
      if constexpr (HC) return hcode<BITS>(hc, n);
      else return x[n];
    };
    wave_sync();
    if (op == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float sc = sm.rowc[3][r0 + m];
        *reinterpret_cast<float2*>(S + (r0 + m) * DV + j0) =
            make_float2(sc * c0 * (x[2 * m] - OFF), sc * c1 * (x[2 * m + 1] - OFF));
      }
      return;
    }
    // pass 1: key retrieval delta_j = c_j sum_i kappa_i (u_ij - off)
    const float ks = sm.ksum[rb];
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 k4 = lds_ld4(rcb + 4 * (0 * DK + m));
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a0 = fmaf(kv[u], code(2 * (m + u)), a0);
        a1 = fmaf(kv[u], code(2 * (m + u) + 1), a1);
      }
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
    const float2 vv = EARLY ? make_float2(sm.colC[0][p].x, sm.colC[0][p].y)
                              : *reinterpret_cast<const float2*>(a.v + tv + j0);
    const float e0 = vv.x - c0 * d0, e1 = vv.y - c1 * d1;
    // pass 2: Xt = c_j (u - off) + gamma_i e_j, readout partials
    const float o0 = -OFF * c0, o1 = -OFF * c1;
    // the column scales enter the update as fp32 registers: the empty asm
    // keeps the compiler from folding their binary16-to-fp32 conversion into
    // mixed-precision FMAs, which issue more slowly than plain ones
    float cs0v = c0 * HS, cs1v = c1 * HS;
    asm volatile("" : "+v"(cs0v), "+v"(cs1v));
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 g4 = lds_ld4(rcb + 4 * (1 * DK + m)), t4 = lds_ld4(rcb + 4 * (2 * DK + m));
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, tv4[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float v0 = fmaf(cs0v, code(2 * (m + u)), fmaf(gv[u], e0, o0));
        const float v1 = fmaf(cs1v, code(2 * (m + u) + 1), fmaf(gv[u], e1, o1));
        x[2 * (m + u)] = v0;
        x[2 * (m + u) + 1] = v1;
        y0 = fmaf(tv4[u], v0, y0);
        y1 = fmaf(tv4[u], v1, y1);
      }
    }
    sm.colB[rb][p] = make_float2(y0, y1);
  }
  // row statistics of Xt (sum |.| for STEP, max |.| for uniform), 16 rows at a
  // time through a per-wave transpose; after the shuffle stage every lane
  // holds the statistic of row (p & 15) of the half, so one pass of the 32
  // owner lanes then derives the stored scale of every row of the block
  uint32_t wd[2 * BITS];
  float sh[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float u0 = fabsf(x[2 * (16 * hf + m)]), u1 = fabsf(x[2 * (16 * hf + m) + 1]);
      sm.rowt[rb][m][p] = UNI ? fmaxf(u0, u1) : u0 + u1;
    }
    wave_sync();
    const int mm = p & 15, part = p >> 4;
    float s = lds_fold16<UNI>(&sm.rowt[rb][mm][part * 16]);
    {  // combine the parts 16 (and 32) lanes apart
      float a0, b0;
      swap16(s, a0, b0);
      s = UNI ? fmaxf(a0, b0) : a0 + b0;
      if constexpr (NP == 64) {
        swap32(s, a0, b0);
        s = UNI ? fmaxf(a0, b0) : a0 + b0;
      }
    }
    sh[hf] = s;
    wave_sync();
  }
  if (p < 32) {
    const int i = r0 + p;
    const float s = p < 16 ? sh[0] : sh[1];
    const float rp = sm.rowc[3][i];
    if (UNI) {
      const float si = fp16_scale(rp * s * (1.0f / QB));
      rs_ptr[i] = __float2half_rn(si);
      sm.rowc[4][i] = rp * frcp(si);  // code pre-value = Xt * sigma_i
    } else {
      const float wi = EARLY ? sm.rowc[5][i] : a.P.w[h * DK + i];
      const float wiv = EARLY ? sm.rowc[4][i] : a.P.winv[h * DK + i];
      // the hardware square root (1 ulp) only feeds an FP16 rounding
      const float ri = fp16_scale(__builtin_amdgcn_sqrtf(rp * s * (1.0f / (float)DV) * wiv));
      rs_ptr[i] = __float2half_rn(ri);
      sm.rowc[4][i] = rp * frcp(ri);                  // pi: X / r_i = Xt * pi_i
      sm.rowc[5][i] = wi * wi * ri * ri * (1.0f / QB);  // lambda: refit weight
    }
  }
  wave_sync();
  if constexpr (UNI) {
    if (op == OP_DECODE) {
      __syncthreads();
      if (rb == 0) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
          s0 += sm.colB[r][p].x;
          s1 += sm.colB[r][p].y;
        }
        *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(s0, s1);
      }
    }
    codes_rowwise<BITS>(x, rcb + 4 * (4 * DK), wd);
  } else {
    // pass 3: P = X / r_i and the column absmax
    float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 p4 = lds_ld4(rcb + 4 * (4 * DK + m));
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[2 * (m + u)] *= pv[u];
        x[2 * (m + u) + 1] *= pv[u];
      }
      // a chain of three-input maxima: two new values per instruction
      mx0 = fmaxf(fmaxf(mx0, fabsf(x[2 * m])), fabsf(x[2 * m + 2]));
      mx0 = fmaxf(fmaxf(mx0, fabsf(x[2 * m + 4])), fabsf(x[2 * m + 6]));
      mx1 = fmaxf(fmaxf(mx1, fabsf(x[2 * m + 1])), fabsf(x[2 * m + 3]));
      mx1 = fmaxf(fmaxf(mx1, fabsf(x[2 * m + 5])), fabsf(x[2 * m + 7]));
    }
    sm.colM[rb][p] = make_float2(mx0, mx1);
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
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float2 c = sm.colM[r][p];
      m0 = fmaxf(m0, c.x);
      m1 = fmaxf(m1, c.y);
    }
    const float cz0 = fp16_scale(m0), cz1 = fp16_scale(m1);
    const float tau0 = QB * frcp(cz0), tau1 = QB * frcp(cz1);
    // below the FP16 maximum, c0 >= max |P| (1 - 2^-11) keeps every code within
    // +-q_b without a clamp; a wave holding a saturated column clamps all of
    // its codes (a no-op on the others), the decision staying wave-uniform
    const bool sat = __ballot(fmaxf(m0, m1) > kFp16Max) != 0ull;
    // pass 4: codes by magic rounding, fixed-code weighted least-squares sums
    float4 nd;
    if (sat) codes_refit<BITS, true>(x, rcb + 4 * (5 * DK), tau0, tau1, nd, wd);
    else codes_refit<BITS, false>(x, rcb + 4 * (5 * DK), tau0, tau1, nd, wd);
    sm.colC[rb][p] = nd;
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
      const float cf0 = dd0 > 0.f ? fp16_scale(QB * n0 * frcp(dd0)) : cz0;
      const float cf1 = dd1 > 0.f ? fp16_scale(QB * n1 * frcp(dd1)) : cz1;
      c_ptr[j0] = __float2half_rn(cf0);
      c_ptr[j0 + 1] = __float2half_rn(cf1);
    }
  }
  store_chunk<BITS, NP>(base, rb, p, wd);
}

// FP16 pivot head of a STEP GDN plan: the state is kept as FP16 values.
template <int DK, int DV, int OP>
__device__ __forceinline__ void pivot_tile(const TileArgs& a, const int tile, const int h,
                                           unsigned char* base, SmemGdn<DK, DV>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p;
  constexpr int op = OP;
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
    const float alpha = wuni(a.gate[tile]);
    if (t < DK) {
      const float kk = a.k[tk + t];
      sm.rowc[0][t] = alpha * kk;
      sm.rowc[1][t] = wuni(a.beta[tile]) * kk;
      sm.rowc[2][t] = a.q[tk + t];
    }
    if (rb == 0) {
      const float2 v2 = *reinterpret_cast<const float2*>(a.v + tv + j0);
      sm.colC[0][p] = make_float4(v2.x, v2.y, 0.f, 0.f);
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
    const float2 vv = make_float2(sm.colC[0][p].x, sm.colC[0][p].y);
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

template <int DK, int DV, int OP>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void gdn_tile_kernel(TileArgs a) {
  __shared__ SmemGdn<DK, DV> sm;
  const int tile = blockIdx.x;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (OP == OP_DECODE) {
      const int t = threadIdx.x;
      if (t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    }
    return;
  }
  const int bits = a.P.head_bits[h];
  const bool uni = a.P.mode == SQ_MODE_UNIFORM;
  switch (bits) {
    case 2:
      if (uni) quant_tile<DK, DV, 2, true, OP>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 2, false, OP>(a, tile, h, base, sm);
      break;
    case 4:
      if (uni) quant_tile<DK, DV, 4, true, OP>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 4, false, OP>(a, tile, h, base, sm);
      break;
    case 6:
      if (uni) quant_tile<DK, DV, 6, true, OP>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 6, false, OP>(a, tile, h, base, sm);
      break;
    case 8:
      if (uni) quant_tile<DK, DV, 8, true, OP>(a, tile, h, base, sm);
      else quant_tile<DK, DV, 8, false, OP>(a, tile, h, base, sm);
      break;
    case 16:
      if (!uni) pivot_tile<DK, DV, OP>(a, tile, h, base, sm);
      break;
    default:
      break;
  }
}


// Pick entry i of a five-entry kernel-argument array with selects, so the
// argument block is never indexed with a run-time subscript.
__device__ __forceinline__ int pick5(const int (&v)[5], int i) {
  int r = v[0];
#pragma unroll
  for (int j = 1; j < 5; ++j) r = i == j ? v[j] : r;
  return r;
}

// Decode of every code-width class in one grid.  Class i covers blockIdx in
// [cls_end[i-1], cls_end[i]); inside a class, tile t = (batch row t / cls_n,
// class head t % cls_n).  The width is uniform over a workgroup, so each
// workgroup runs exactly one of the width-specialised bodies; the kernel's
// register budget is the largest of them.
// Tile t of the class list: class c holds t in [cls_end[c-1], cls_end[c]).
template <int DK, int DV, bool UNI, bool LATE = false>
__device__ __forceinline__ void merged_tile(const TileArgs& a, int t, SmemGdn<DK, DV>& sm) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) c += t >= a.cls_end[j] ? 1 : 0;
  if (c > 0) t -= pick5(a.cls_end, c - 1);
  const int n = pick5(a.cls_n, c);
  const int bits = pick5(a.cls_bits, c);
  const int bi = t / n;
  const int h = wuni(a.P.cls_heads[pick5(a.cls_first, c) + (t - bi * n)]);
  const int tile = bi * a.P.H + h;
  const int slot = wuni(a.slots[bi]);
  if (slot < 0 || (long long)slot >= a.n_slots) {
    if (threadIdx.x < DV) a.y[(long long)tile * DV + threadIdx.x] = __builtin_nanf("");
    return;
  }
  unsigned char* base = a.pool + (long long)slot * a.P.slot_bytes + wuni(a.P.head_off[h]);
  switch (bits) {
    case 2: quant_tile<DK, DV, 2, UNI, OP_DECODE, LATE>(a, tile, h, base, sm); break;
    case 4: quant_tile<DK, DV, 4, UNI, OP_DECODE, LATE>(a, tile, h, base, sm); break;
    case 6: quant_tile<DK, DV, 6, UNI, OP_DECODE, LATE>(a, tile, h, base, sm); break;
    case 8: quant_tile<DK, DV, 8, UNI, OP_DECODE, LATE>(a, tile, h, base, sm); break;
    case 16:
      if constexpr (!UNI) pivot_tile<DK, DV, OP_DECODE>(a, tile, h, base, sm);
      break;
    default: break;
  }
}

// Tile of class 0 at batch row bi, class head j, its width fixed at compile time.
template <int DK, int DV, int BITS, bool UNI>
__device__ __forceinline__ void class0_tile(const TileArgs& a, int bi, int j, SmemGdn<DK, DV>& sm) {
  const int h = wuni(a.P.cls_heads[a.cls_first[0] + j]);
  const int tile = bi * a.P.H + h;
  const int slot = wuni(a.slots[bi]);
  if (slot < 0 || (long long)slot >= a.n_slots) {
    if (threadIdx.x < DV) a.y[(long long)tile * DV + threadIdx.x] = __builtin_nanf("");
    return;
  }
  unsigned char* base = a.pool + (long long)slot * a.P.slot_bytes + wuni(a.P.head_off[h]);
  if constexpr (BITS == 16) pivot_tile<DK, DV, OP_DECODE>(a, tile, h, base, sm);
  else quant_tile<DK, DV, BITS, UNI, OP_DECODE>(a, tile, h, base, sm);
}

// Decode of every code-width class in one grid.  Class i covers blockIdx in
// [cls_end[i-1], cls_end[i]); inside a class, tile t = (batch row t / cls_n,
// class head t % cls_n).  The width is uniform over a workgroup, so each
// workgroup runs exactly one of the width-specialised bodies; the kernel's
// register budget is the largest of them.
template <int DK, int DV, bool UNI, bool LATE>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void gdn_decode_kernel(TileArgs a) {
  __shared__ SmemGdn<DK, DV> sm;
  merged_tile<DK, DV, UNI, LATE>(a, blockIdx.x, sm);
}

// STEP decode of class 0 in its width-specialised body plus the other classes
// in one grid: rows y < pre_rows (cls_n[0] workgroups each) take the other
// classes' tiles first, so the heavier FP16 and small-class tiles start with
// the first wave of workgroups instead of in a second launch after the last.
template <int DK, int DV, int BITS>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void gdn_split_kernel(TileArgs a) {
  __shared__ SmemGdn<DK, DV> sm;
  const int y = blockIdx.y;
  if (y < a.pre_rows) {
    const int t = a.cls_end[0] + y * (int)gridDim.x + (int)blockIdx.x;
    if (t < a.n_tiles) merged_tile<DK, DV, false>(a, t, sm);
    return;
  }
  class0_tile<DK, DV, BITS, false>(a, y - a.pre_rows, blockIdx.x, sm);
}

// Decode of class 0 alone with its width fixed at compile time: the register
// allocation and schedule are those of that width only.
template <int DK, int DV, int BITS, bool UNI>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void gdn_class_kernel(TileArgs a) {
  __shared__ SmemGdn<DK, DV> sm;
  // grid (heads of the class, batch rows): the same order as tile
  // bi * n + j, without a division
  class0_tile<DK, DV, BITS, UNI>(a, blockIdx.y, blockIdx.x, sm);
}

// 256 CUs x 4 resident 256-lane workgroups: the tiles of one round
constexpr int kRoundTiles = 1024;

template <int DK, int DV, int BITS>
hipError_t launch_solo(const TileArgs& a, const dim3 grid, const dim3 block, hipStream_t s) {
  if (a.P.mode == SQ_MODE_UNIFORM) {
    if constexpr (BITS == 16) return hipErrorInvalidValue;
    else hipLaunchKernelGGL((gdn_class_kernel<DK, DV, BITS, true>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((gdn_class_kernel<DK, DV, BITS, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// solo: class 0 alone through its width-specialised kernel; otherwise every
// class of a through the merged kernel
template <int DK, int DV>
hipError_t launch_decode(const TileArgs& a, bool solo, hipStream_t s) {
  if (a.n_tiles <= 0) return hipSuccess;
  const dim3 grid(a.n_tiles), block((DK / 32) * (DV / 2));
  if (solo && a.B <= 65535) {
    const dim3 grid2(a.cls_n[0], a.B);
    switch (a.cls_bits[0]) {
      case 2: return launch_solo<DK, DV, 2>(a, grid2, block, s);
      case 4: return launch_solo<DK, DV, 4>(a, grid2, block, s);
      case 6: return launch_solo<DK, DV, 6>(a, grid2, block, s);
      case 8: return launch_solo<DK, DV, 8>(a, grid2, block, s);
      case 16: return launch_solo<DK, DV, 16>(a, grid2, block, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.P.mode == SQ_MODE_UNIFORM) {
    hipLaunchKernelGGL((gdn_decode_kernel<DK, DV, true, false>), grid, block, 0, s, a);
  } else {
    bool late = false;
    if constexpr (DK == 128 && DV == 128) late = a.n_tiles <= kRoundTiles;
    if (late) hipLaunchKernelGGL((gdn_decode_kernel<DK, DV, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gdn_decode_kernel<DK, DV, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  const dim3 grid(a.n_tiles), block((DK / 32) * (DV / 2));
  if (a.op == OP_DECODE) return hipErrorInvalidValue;  // decode goes through the width classes
  if (a.op == OP_PACK) hipLaunchKernelGGL((gdn_tile_kernel<DK, DV, OP_PACK>), grid, block, 0, s, a);
  else if (a.op == OP_UNPACK) hipLaunchKernelGGL((gdn_tile_kernel<DK, DV, OP_UNPACK>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gdn(const TileArgs& a, bool solo, hipStream_t s) {
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch_decode<128, 128>(a, solo, s);
  if (dk == 64 && dv == 64) return launch_decode<64, 64>(a, solo, s);
  if (dk == 128 && dv == 64) return launch_decode<128, 64>(a, solo, s);
  if (dk == 64 && dv == 128) return launch_decode<64, 128>(a, solo, s);
  return hipErrorInvalidValue;
}

template <int DK, int DV>
hipError_t launch_split(const TileArgs& a, hipStream_t s) {
  const dim3 grid(a.cls_n[0], a.B + a.pre_rows), block((DK / 32) * (DV / 2));
  switch (a.cls_bits[0]) {
    case 2: hipLaunchKernelGGL((gdn_split_kernel<DK, DV, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gdn_split_kernel<DK, DV, 4>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((gdn_split_kernel<DK, DV, 6>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((gdn_split_kernel<DK, DV, 8>), grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL((gdn_split_kernel<DK, DV, 16>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_split_gdn(const TileArgs& a, hipStream_t s) {
  if (a.P.mode != SQ_MODE_STEP || a.B + a.pre_rows > 65535) return hipErrorInvalidValue;
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch_split<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch_split<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch_split<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_split<64, 128>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_tile_gdn(const TileArgs& a, hipStream_t s) {
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(a, s);
  return hipErrorInvalidValue;
}
