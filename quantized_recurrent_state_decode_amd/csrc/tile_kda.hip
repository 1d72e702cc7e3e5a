// Fused quantized decode step for STEP KDA heads: channel-wise retention
// D = diag(d), bit width chosen per key row (STEPQuant Sec. 4, unit = key
// row for KDA), FP16 pivot rows, one column-scale vector c shared by all
// integer rows of the head (App. D: the codebook normalisation is fixed by
// precision, so rows of different widths share c).
//
// Storage rows are ordered by (width, key row) and kept row-major, so a head
// is a run of variable-length rows.  The workgroup stages the packed head in
// LDS with coalesced 16-byte copies; lane (rb, p) extracts columns 2p, 2p+1
// of its 32 storage rows (the width of a row is uniform across the wave),
// writes the new codes back into the same LDS bytes and the head is copied
// out with 16-byte stores.  Per-row inputs (d, k, q, w) are gathered through
// the storage permutation.  Per element, with c' = c_j (integer rows) or 1
// (FP16 rows) and rho_s the row's retained dequantisation factor:
//   x = c' * value;   delta_j = sum_s kappa_s x_sj          (kappa = k rho)
//   Xt = x + gamma_s e_j  (X = rho_s Xt, gamma = beta k / rho)
//   y_j = sum_s theta_s Xt_sj                              (theta = q rho)
// then the GDN kernel's row scales, column init, codes by magic rounding
// (per-row q_b) and fixed-code column refit over the integer rows.
#include <algorithm>

#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV>
struct SmemKda {
  float rowc[7][DK];  // 0 kappa, 1 gamma, 2 theta, 3 rho, 4 pi or rho (FP16 rows),
                      // 5 lambda_N = w^2 r^2 / q_b, 6 lambda_D = w^2 r^2 / q_b^2
  float qb[DK];       // q_b of storage row s (0 for FP16 rows)
  int bits[DK];
  int off[DK];
  float2 colA[DK / 32][DV / 2];
  float2 colB[DK / 32][DV / 2];
  float2 colM[DK / 32][DV / 2];
  float4 colC[DK / 32][DV / 2];
};

// The packed head (at most max_code_bytes) and, while no codes are live,
// the per-wave row transpose, share the dynamic LDS buffer; its last 16
// bytes are a spare slot for staging stores past the head's region.
extern __shared__ uint4 kda_dyn[];

template <int DK, int DV>
__host__ __device__ constexpr int dyn_bytes(int max_code_bytes) {
  constexpr int transpose = (DK / 32) * 16 * (DV / 2 + 1) * 4;
  return ((max_code_bytes > transpose ? max_code_bytes : transpose) + 15) / 16 * 16 + 16;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A per-row value: with 64 lanes per row block every lane of a wave works on
// the same storage row, so the value is wave-uniform and goes to a scalar
// register (row-wise branches become scalar); with 32 lanes a wave spans two
// row blocks and the value stays per lane.
template <bool WU>
__device__ __forceinline__ int rowu(int v) {
  if constexpr (WU) return wuni(v);
  else return v;
}
template <bool WU>
__device__ __forceinline__ float rowu(float v) {
  if constexpr (WU) return wuni(v);
  else return v;
}

// Two b-bit fields (columns 2p, 2p+1) of a row stored at byte `off` (rows
// start on 16-byte boundaries; fields are two's complement, least significant
// bit first).
__device__ __forceinline__ void read_pair(const unsigned char* codes, int off, int b, int p,
                                          float& z0, float& z1) {
  const unsigned char* row = codes + off;
  if (b == 16) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(row)[p];
    z0 = half_from_bits(v);
    z1 = half_from_bits(v >> 16);
    return;
  }
  uint32_t f;
  if (b == 8) {
    f = reinterpret_cast<const unsigned short*>(row)[p];
  } else if (b == 4) {
    f = row[p];
  } else if (b == 2) {
    f = (uint32_t)row[p >> 1] >> (4 * (p & 1));
  } else {  // 6 bits: the pair's 12 bits start at bit 12 p
    const int i = (3 * p) >> 1;
    f = ((uint32_t)row[i] | ((uint32_t)row[i + 1] << 8)) >> (4 * (p & 1));
  }
  // the builtin returns an unsigned type: reinterpret as signed before converting
  z0 = (float)(int)__builtin_amdgcn_sbfe((int)f, 0, b);
  z1 = (float)(int)__builtin_amdgcn_sbfe((int)f, b, b);
}

// Write the lane's two codes (magic-rounded floats m0, m1) of a b-bit row.
// Rows are byte-aligned; 2- and 6-bit pairs share bytes with the next lane's,
// so even lanes write both lanes' bits.
__device__ __forceinline__ void write_pair(unsigned char* codes, int off, int b, int p, float m0,
                                           float m1) {
  const uint32_t u0 = __float_as_uint(m0), u1 = __float_as_uint(m1);
  if (b == 4) {
    codes[off + p] = (unsigned char)((u0 & 15u) | ((u1 & 15u) << 4));
  } else if (b == 8) {
    *reinterpret_cast<unsigned short*>(codes + off + 2 * p) =
        (unsigned short)((u0 & 0xffu) | ((u1 & 0xffu) << 8));
  } else if (b == 2) {
    const uint32_t nib = (u0 & 3u) | ((u1 & 3u) << 2);
    const uint32_t nxt = __shfl_down(nib, 1);
    if (!(p & 1)) codes[off + (p >> 1)] = (unsigned char)(nib | (nxt << 4));
  } else {  // 6 bits: 12 bits per lane, 3 bytes per lane pair
    const uint32_t f = (u0 & 63u) | ((u1 & 63u) << 6);
    const uint32_t nxt = __shfl_down(f, 1);
    if (!(p & 1)) {
      const uint32_t v = f | (nxt << 12);
      unsigned char* d = codes + off + 3 * (p >> 1);
      d[0] = (unsigned char)v;
      d[1] = (unsigned char)(v >> 8);
      d[2] = (unsigned char)(v >> 16);
    }
  }
}

template <int DK, int DV, int OP>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void kda_tile_kernel(TileArgs a) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT;
  constexpr bool WU = NP % 64 == 0;  // a wave's lanes share their rows
  __shared__ SmemKda<DK, DV> sm;
  unsigned char* codes = reinterpret_cast<unsigned char*>(kda_dyn);
  float(*rowt)[16][NP + 1] = reinterpret_cast<float(*)[16][NP + 1]>(kda_dyn);
  const int tile = blockIdx.x;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (OP == OP_DECODE && t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    return;
  }
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  const int* rkey = a.P.row_key + h * DK;
  const int code_bytes = wuni(a.P.r_off[h]);
  __half* r_ptr = reinterpret_cast<__half*>(base + code_bytes);
  __half* c_ptr = reinterpret_cast<__half*>(base + wuni(a.P.c_off[h]));
  // per-storage-row metadata of this wave's rows (loaded first: the key row
  // indexes the token's inputs)
  int rk = 0, rbits = 16, roff = 0;
  if (p < 32) {
    const int s = r0 + p;
    rk = rkey[s];
    rbits = a.P.row_bits[h * DK + s];
    roff = a.P.row_off[h * DK + s];
  }
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
      sm.bits[s] = rbits;
      sm.off[s] = roff;
      sm.qb[s] = rbits == 16 ? 0.f : (float)((1 << (rbits - 1)) - 1);
      sm.rowc[3][s] = 1.0f;
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
    const uint4* src = reinterpret_cast<const uint4*>(base);
    uint4* dst = reinterpret_cast<uint4*>(codes);
    uint4 v[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {  // first round, issued before the per-row inputs
      const int e = t + i * NT;
      v[i] = src[e < nch ? e : 0];
    }
    // keep the key-indexed loads (which wait for the key rows) behind these
    const float c0 = __half2float(c_ptr[j0]), c1 = __half2float(c_ptr[j0 + 1]);
    float rs = 0.f, d = 0.f, kk = 0.f, qq = 0.f;
    if (p < 32) {
      rs = __half2float(r_ptr[r0 + p]);
      if constexpr (OP == OP_DECODE) {
        d = a.gate[tk + rk];
        kk = a.k[tk + rk];
        qq = a.q[tk + rk];
      }
    }
    const float beta = OP == OP_DECODE ? a.beta[tile] : 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int e = t + i * NT;
      dst[e < nch ? e : spare] = v[i];
    }
    for (int c = CH * NT; c < nch; c += CH * NT) {  // heads larger than one round
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int e = c + t + i * NT;
        v[i] = src[e < nch ? e : 0];
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int e = c + t + i * NT;
        dst[e < nch ? e : spare] = v[i];
      }
    }
    if (p < 32) {
      const int s = r0 + p, b = rbits;
      const float qb = b == 16 ? 0.f : (float)((1 << (b - 1)) - 1);
      sm.bits[s] = b;
      sm.off[s] = roff;
      sm.qb[s] = qb;
      const bool piv = b == 16;
      const float sc = piv ? 1.f : rs * frcp(qb);
      if constexpr (OP == OP_UNPACK) {
        sm.rowc[3][s] = sc;
      } else {
        const float bk = beta * kk;
        const float rho = d * sc;
        // a vanishing retention keeps the division finite; the dropped part
        // (rp - rho) c_j z_sj is below 2^-60 of the write term
        const float rp = fmaxf(rho, fmaxf(fabsf(bk) * 0x1p-60f, 0x1p-100f));
        sm.rowc[0][s] = kk * rho;
        sm.rowc[1][s] = bk * frcp(rp);
        sm.rowc[2][s] = qq * rp;
        sm.rowc[3][s] = rp;
      }
    }
    __syncthreads();  // codes staged, per-row constants ready
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int s = r0 + m;
      const int b = rowu<WU>(sm.bits[s]);
      float z0, z1;
      read_pair(codes, rowu<WU>(sm.off[s]), b, p, z0, z1);
      x[2 * m] = b == 16 ? z0 : c0 * z0;
      x[2 * m + 1] = b == 16 ? z1 : c1 * z1;
    }
    if constexpr (OP == OP_UNPACK) {
      float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float f = sm.bits[r0 + m] == 16 ? 1.f : sm.rowc[3][r0 + m];
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
    const float2 vv = *reinterpret_cast<const float2*>(a.v + tv + j0);
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
    float s = rowt[rb][mm][part * 16];
#pragma unroll
    for (int pp = 1; pp < 16; ++pp) s += rowt[rb][mm][part * 16 + pp];
#pragma unroll
    for (int o = 16; o < NP; o <<= 1) s += __shfl_xor(s, o);
    sh[hf] = s;
    wave_sync();
  }
  if (p < 32) {
    const int si = r0 + p;
    const float s = p < 16 ? sh[0] : sh[1];
    const float rp = sm.rowc[3][si];
    if (sm.bits[si] == 16) {
      r_ptr[si] = __float2half_rn(0.0f);
      sm.rowc[4][si] = rp;  // FP16 rows: X = rho Xt
      sm.rowc[5][si] = 0.f;
      sm.rowc[6][si] = 0.f;
    } else {
      const int key = rkey[si];
      const float wi = a.P.w[h * DK + key], iq = frcp(sm.qb[si]);
      // the hardware square root (1 ulp) only feeds an FP16 rounding
      const float ri =
          fp16_scale(__builtin_amdgcn_sqrtf(rp * s * (1.0f / (float)DV) * a.P.winv[h * DK + key]));
      r_ptr[si] = __float2half_rn(ri);
      const float ww = wi * wi * ri * ri * iq;
      sm.rowc[4][si] = rp * frcp(ri);
      sm.rowc[5][si] = ww;
      sm.rowc[6][si] = ww * iq;
    }
  }
  wave_sync();
  // pass 3: P = X / r on integer rows (column absmax), X on FP16 rows
  float mx0 = 0.f, mx1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int s = r0 + m;
    const float f = sm.rowc[4][s];
    x[2 * m] *= f;
    x[2 * m + 1] *= f;
    if (rowu<WU>(sm.bits[s]) != 16) {
      mx0 = fmaxf(mx0, fabsf(x[2 * m]));
      mx1 = fmaxf(mx1, fabsf(x[2 * m + 1]));
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
  // pass 4: codes (magic rounding, per-row q_b) and the refit sums; the new
  // codes go into the staged head in place
  float N0 = 0.f, N1 = 0.f, D0 = 0.f, D1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int s = r0 + m;
    const int b = rowu<WU>(sm.bits[s]), off = rowu<WU>(sm.off[s]);
    if (b == 16) {
      *reinterpret_cast<uint32_t*>(codes + off + 4 * p) =
          half_bits(x[2 * m]) | (half_bits(x[2 * m + 1]) << 16);
      continue;
    }
    const float qb = rowu<WU>(sm.qb[s]), ln = sm.rowc[5][s], ld = sm.rowc[6][s];
    const float pv0 = x[2 * m], pv1 = x[2 * m + 1];
    float mg0 = fmaf(pv0, qb * ic0, kMagic), mg1 = fmaf(pv1, qb * ic1, kMagic);
    if (sat) {  // a column scale saturated at the FP16 maximum
      mg0 = __builtin_amdgcn_fmed3f(mg0, kMagic - qb, kMagic + qb);
      mg1 = __builtin_amdgcn_fmed3f(mg1, kMagic - qb, kMagic + qb);
    }
    const float z0 = mg0 - kMagic, z1 = mg1 - kMagic;
    N0 = fmaf(ln * z0, pv0, N0);
    N1 = fmaf(ln * z1, pv1, N1);
    D0 = fmaf(ld * z0, z0, D0);
    D1 = fmaf(ld * z1, z1, D1);
    write_pair(codes, off, b, p, mg0, mg1);
  }
  sm.colC[rb][p] = make_float4(N0, N1, D0, D1);
  __syncthreads();
  for (int i = t * 16; i < code_bytes; i += NT * 16)
    *reinterpret_cast<uint4*>(base + i) = *reinterpret_cast<const uint4*>(codes + i);
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
