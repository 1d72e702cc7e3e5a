// Per-window decode (LeapQuant notes Sec. 2.3-2.6, GDN scalar gate).
//
// A head keeps a fixed INT8 boundary S0 = diag(C) (Z/127) diag(B) and the
// records (alpha_j, kt_j = beta_j k_j, u_j) of the tokens since the last
// rebuild.  With Gamma_{a:b} = alpha_b ... alpha_a (1 when a > b):
//   S_l^T x = Gamma_{1:l} S0^T x + sum_{j<=l} u_j (kt_j . Gamma_{j+1:l} x)
// Token i = l + 1:
//   u_i = v_i - S_{i-1}^T (alpha_i k_i)          (stored as float32)
//   o_i = S_i^T q_i                               (the head output)
// and when the window holds p records the dense state
//   S_p = Gamma_{1:p} S0 + sum_j Gamma_{j+1:p} kt_j u_j^T
// is rebuilt and re-encoded with key-row smoothing and per-column INT8
// (Sec. 2.5, App. B.3): C_a = max(sqrt(mean_j |S_aj|), c_floor),
// T = diag(C)^-1 S, B_j = max_a |T_aj|, Z = clamp(rne(127 T / B), +-127).
//
// Compensator tokens (Sec. 2.4-2.5, Eqs. 5-7, 10), rank r > 0: the boundary
// also holds r FP16 pairs (kc_h, uc_h), S0 = C (Z/127) B + sum_h kc_h uc_h^T.
// They decay with the boundary, so their readout term uc_h (kc_h . x) is
// scaled like the boundary's and rides in spare lanes of the record dot
// products.  A rebuild (and a pack) refits them by power iteration on the
// register-resident dense state, pair after pair on the residual, from the
// pair's previous uc_h (the all-ones vector at a pack or for a zero pair):
// iters times a = M b / |M b|, b = M^T a; then kc = FP16(sqrt|b| a),
// uc = FP16(b / sqrt|b|), M -= kc uc^T; the residual is what is quantized.
//
// Lanes own 2 columns x 32 rows of the INT8 boundary (blocked layout), so
// S0^T x costs one fused multiply-add per element for each of the two read
// vectors and the reduction over rows is lane-local plus one LDS combine.
// The window position is read first; the boundary, the token's inputs and
// then the records and pairs held (16-byte loads into registers, a fixed
// count per thread) all go out before any of them is waited on, and the
// records are committed to LDS together.  Record and compensator dot
// products over the wave's own rows take 16 or 32 lanes per set of units,
// with the rows split into segments over the remaining lanes; the decay
// suffix products come from a log-step scan over one wave's lanes, and the
// rebuild at a flush reads the records from LDS.
#include "tile_common.h"

using namespace sqk;

namespace {

constexpr int RM = SQ_MAX_COMP_RANK;  // compensator pairs per head, at most

// RMX: compensator pairs the kernel variant can hold (0 or RM)
template <int DK, int DV, int PM, int RMX>
struct SmemWin {
  float x1[DK], qv[DK], ktn[DK];  // alpha_i k_i, q_i, beta_i k_i (float32)
  float cx1[DK], cq[DK];          // C_a x1_a, C_a q_a
  float rowf[DK];                 // rebuild row factor, then 1 / C_a
  float al[PM + 1];               // record decays (+ a spare word)
  float g1[PM + 1], g2[PM + 1];   // suffix products of the decays
  float2 dots[DK / 32][PM + RMX];  // per row block: kt_j . x1, kt_j . q; then kc_h . x1, kc_h . q
  float2 esum[PM + RMX];           // the same summed over row blocks, decay-scaled
  float kc[RMX > 0 ? RMX : 1][DK];  // compensator pairs of the head (float)
  float uc[RMX > 0 ? RMX : 1][DV];
  float va[RMX > 0 ? DK : 1];       // compensator fit: a = M b, then the rounded kc
  float red[2][DK / 32 + 1];        // compensator fit: block sums (two buffers)
  float unew[DV];
  float crow[DK];                   // the boundary's row scales C, staged
  float2 bcol[DV / 2];              // its column scales B, staged
  float2 vin[DV / 2];               // the token's v, staged
  float2 colA[DK / 32][DV / 2];
  float2 colB[DK / 32][DV / 2];
  union {
    struct {
      float K[PM][DK];
      float U[PM][DV];
    } rec;                                   // records held, staged from the head
    alignas(16) float rowt[DK / 32][16][RowT<DV / 2>::S];  // row transposes (after the staging)
  } u;
};

struct WinPtrs {
  int* ell;
  float* alpha;
  unsigned char* Z;
  float *C, *B, *K, *U;
  __half *Kc, *Uc;  // compensator pairs [r][d_k], [r][d_v]
};

__device__ __forceinline__ WinPtrs win_ptrs(unsigned char* base, int zoff, int DK, int DV, int P,
                                            int R) {
  WinPtrs w;
  w.ell = reinterpret_cast<int*>(base);
  w.alpha = reinterpret_cast<float*>(base + 16);
  w.Z = base + zoff;
  w.C = reinterpret_cast<float*>(base + zoff + DK * DV);
  w.B = w.C + DK;
  w.K = w.B + DV;
  w.U = w.K + P * DK;
  w.Kc = reinterpret_cast<__half*>(w.U + P * DV);
  w.Uc = w.Kc + R * DK;
  return w;
}

// FP16 of a signed value, saturating at the largest finite magnitude.
__device__ __forceinline__ __half half_sat(float v) {
  return __float2half_rn(fminf(fmaxf(v, -kFp16Max), kFp16Max));
}


// The 64 INT8 boundary codes of a lane chunk (two's-complement bytes, value
// n = 2m + c) as floats: one sign-extending byte conversion each.
__device__ __forceinline__ void unpack_signed8(const uint32_t (&w)[16], float (&x)[64]) {
#pragma unroll
  for (int d = 0; d < 16; ++d) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[4 * d + k] = (float)(int)(signed char)(w[d] >> (8 * k));
  }
}

// Suffix products of the decays of records 0 .. n-1 (n <= PM), computed by
// the 64 lanes of the first wave together (a log-step product scan):
// g[j] = prod_{m=j+1}^{n-1} al[m] for j < PM, and g[PM] = the product of all.
template <int PM>
__device__ __forceinline__ void decay_suffix(const float* al, int n, float* g) {
  const int j = threadIdx.x;
  float a = j < n ? al[j] : 1.f;  // lanes past the records hold 1
#pragma unroll
  for (int off = 1; off < PM; off <<= 1) a *= __shfl_down(a, off, 64);
  const float e = __shfl_down(a, 1, 64);  // lane j + 1's inclusive product
  if (j < PM) g[j] = e;
  if (j == 0) g[PM] = a;
}

// The records and compensator pairs held by a head, staged through
// registers: `issue` starts every load (a fixed number per thread,
// predicated on what the head holds), `commit` stores them to LDS, so the
// loads share one memory round trip.
template <int DK, int DV, int PM, int RMX>
struct Staged {
  static constexpr int NT = (DK / 32) * (DV / 2);
  static constexpr int NK = (PM * DK / 4 + NT - 1) / NT;  // float4 of K rows per thread
  static constexpr int NU = (PM * DV / 4 + NT - 1) / NT;  // float4 of U rows per thread
  static constexpr int NC = RMX > 0 ? (RMX * (DK + DV) / 2 + NT - 1) / NT : 1;  // half2 of pairs
  f32x4 k[NK], u[NU];
  uint32_t c[NC];
  float al;

  // Loads are unconditional so that none waits for another: a slot the head
  // does not hold reads element 0 instead (a line other threads read anyway)
  // and is never committed.
  __device__ __forceinline__ void issue(const WinPtrs& wp, int n, int R) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = t + i * NT;
      k[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wp.K) + (e < n * DK / 4 ? e : 0));
    }
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int e = t + i * NT;
      u[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wp.U) + (e < n * DV / 4 ? e : 0));
    }
    if (RMX > 0) {
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int e = t + i * NT;
        c[i] = reinterpret_cast<const uint32_t*>(wp.Kc)[e < R * (DK + DV) / 2 ? e : 0];
      }
    }
    al = wp.alpha[t < n ? t : 0];
  }

  // Stores are unconditional too (a conditional store would pull its load
  // next to it): slots past the records held land in record rows that are
  // never read, those past the pairs held and the decays of threads past the
  // records held in spare LDS words.
  __device__ __forceinline__ void commit(int n, int R, SmemWin<DK, DV, PM, RMX>& sm) const {
    static_assert(NK * NT == PM * DK / 4 && NU * NT == PM * DV / 4, "staging slots");
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NK; ++i) reinterpret_cast<f32x4*>(&sm.u.rec.K[0][0])[t + i * NT] = k[i];
#pragma unroll
    for (int i = 0; i < NU; ++i) reinterpret_cast<f32x4*>(&sm.u.rec.U[0][0])[t + i * NT] = u[i];
    if (RMX > 0) {
      // pair values 2e, 2e+1 of the head's [Kc (R d_k) | Uc (R d_v)] run
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int e = t + i * NT, f = 2 * e;
        float* dst = e >= R * (DK + DV) / 2 ? &sm.va[f & (DK - 2)]
                     : f < R * DK           ? &sm.kc[0][0] + f
                                            : &sm.uc[0][0] + (f - R * DK);
        dst[0] = half_from_bits(c[i]);
        dst[1] = half_from_bits(c[i] >> 16);
      }
    }
    sm.al[t < n ? t : PM] = al;
  }
};

// Rank-R compensator fit of the dense state in x by power iteration, pair
// after pair on the residual (warm: start from the staged uc_h unless it is
// zero; else from the all-ones vector).  Stores the FP16 pairs in the head
// and leaves the residual in x.  All threads call this; it begins with a
// barrier, after which the record buffer may be reused.
template <int DK, int DV, int PM, int RMX>
__device__ __forceinline__ void fit_compensators(float (&x)[64], const WinPtrs& wp, int R,
                                                 int iters, bool warm, SmemWin<DK, DV, PM, RMX>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  __syncthreads();
  for (int h = 0; h < R; ++h) {
    float b0 = 1.f, b1 = 1.f;
    if (warm) {
      const float u0 = sm.uc[h][j0], u1 = sm.uc[h][j0 + 1];
      if (__syncthreads_or(u0 != 0.f || u1 != 0.f)) {
        b0 = u0;
        b1 = u1;
      }
    }
    float inv = 0.f;  // 1 / |M b| of the last iteration; 0 marks a zero pair
    for (int it = 0; it < iters; ++it) {
      // a = M b: row sums of the lane's two columns through the per-wave transpose
      float sh[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const int mr = 16 * hf + m;
          sm.u.rowt[rb][m][p] = fmaf(x[2 * mr], b0, x[2 * mr + 1] * b1);
        }
        wave_sync();
        const int mm = p & 15, part = p >> 4;
        float sv = lds_fold16<false>(&sm.u.rowt[rb][mm][part * 16]);
        sh[hf] = parts_sum<NP>(sv);
        wave_sync();
      }
      // |a|^2 partial and M^T a partial of the row block go out together;
      // buffers alternate by iteration so one barrier per iteration suffices
      float2(*part)[NP] = (it & 1) ? sm.colB : sm.colA;
      if (p < 32) sm.va[r0 + p] = p < 16 ? sh[0] : sh[1];
      // |a|^2 over the block: each 16-lane row holds the block's 16 row pairs
      // (sh[0], sh[1])
      const float q2 = row16_sum(fmaf(sh[0], sh[0], sh[1] * sh[1]));
      if (p == 0) sm.red[it & 1][rb] = q2;
      wave_sync();
      float c0 = 0.f, c1 = 0.f;
#pragma unroll
      for (int m = 0; m < 32; m += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(&sm.va[r0 + m]);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c0 = fmaf(av[q], x[2 * (m + q)], c0);
          c1 = fmaf(av[q], x[2 * (m + q) + 1], c1);
        }
      }
      part[rb][p] = make_float2(c0, c1);
      __syncthreads();
      float na2 = 0.f;
#pragma unroll
      for (int r = 0; r < NRB; ++r) na2 += sm.red[it & 1][r];
      if (!(na2 > 0.f)) {  // M b = 0: a zero pair (block-uniform)
        inv = 0.f;
        break;
      }
      inv = __builtin_amdgcn_rsqf(na2);  // a scale error only rescales the pair
      // b = M^T a / |a|
      b0 = 0.f;
      b1 = 0.f;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        b0 += part[r][p].x;
        b1 += part[r][p].y;
      }
      b0 *= inv;
      b1 *= inv;
    }
    // sigma = |b| over the columns (row block 0 holds each column once)
    const float s2 = wave_sum(rb == 0 ? fmaf(b0, b0, b1 * b1) : 0.f);
    if (t == 0) sm.red[0][NRB] = s2;
    __syncthreads();
    // hardware square roots (1 ulp): they only scale the pair before its FP16
    // rounding
    const float sigma = __builtin_amdgcn_sqrtf(sm.red[0][NRB]);
    const bool zero = !(inv > 0.f) || !(sigma > 0.f);
    const float sq = zero ? 0.f : __builtin_amdgcn_sqrtf(sigma);
    const float isq = zero ? 0.f : frcp(sq);
    float u0 = __half2float(half_sat(b0 * isq));
    float u1 = __half2float(half_sat(b1 * isq));
    if (p < 32) {
      const int i = r0 + p;
      const __half kh = half_sat(zero ? 0.f : sq * (sm.va[i] * inv));
      wp.Kc[h * DK + i] = kh;
      sm.va[i] = __half2float(kh);
    }
    if (rb == 0) {
      wp.Uc[h * DV + j0] = __float2half_rn(u0);
      wp.Uc[h * DV + j0 + 1] = __float2half_rn(u1);
    }
    wave_sync();
    // take the stored pair out of the state (the pair as fp32 registers: the
    // compiler would otherwise fold the FP16 value into mixed-precision FMAs,
    // which issue more slowly)
    asm volatile("" : "+v"(u0), "+v"(u1));
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sm.va[r0 + m]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * (m + q)] = fmaf(-kv[q], u0, x[2 * (m + q)]);
        x[2 * (m + q) + 1] = fmaf(-kv[q], u1, x[2 * (m + q) + 1]);
      }
    }
    __syncthreads();  // red, colA, colB and va are reused by the next pair
  }
}

// x holds S (fp32, lane layout); re-encode it into the head and reset the
// window.  All threads call this; it begins with a barrier, after which the
// record buffer may be reused.
template <int DK, int DV, int PM, int RMX>
__device__ __forceinline__ void encode_boundary(float (&x)[64], const WinPtrs& wp, float c_floor,
                                                SmemWin<DK, DV, PM, RMX>& sm, int P, bool clear_records) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB, NT = G::NT;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  __syncthreads();
  // C_a = max(sqrt(mean_j |S_aj|), floor): row sums through a per-wave transpose
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int m = 0; m < 16; ++m)
      sm.u.rowt[rb][m][p] = fabsf(x[2 * (16 * hf + m)]) + fabsf(x[2 * (16 * hf + m) + 1]);
    wave_sync();
    const int mm = p & 15, part = p >> 4;
    float s = lds_fold16<false>(&sm.u.rowt[rb][mm][part * 16]);
    s = parts_sum<NP>(s);
    if (part == 0) {
      const int a = r0 + 16 * hf + mm;
      const float ca = fmaxf(sqrtf(s / (float)DV), c_floor);
      wp.C[a] = ca;
      sm.rowf[a] = 1.0f / ca;
    }
    wave_sync();
  }
  float m0 = 0.f, m1 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; m += 2) {
    const float ic = sm.rowf[r0 + m], ic1 = sm.rowf[r0 + m + 1];
    x[2 * m] *= ic;
    x[2 * m + 1] *= ic;
    x[2 * m + 2] *= ic1;
    x[2 * m + 3] *= ic1;
    m0 = fmaxf(m0, fmaxf(fabsf(x[2 * m]), fabsf(x[2 * m + 2])));
    m1 = fmaxf(m1, fmaxf(fabsf(x[2 * m + 1]), fabsf(x[2 * m + 3])));
  }
  sm.colA[rb][p] = make_float2(m0, m1);
  __syncthreads();
  float b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    b0 = fmaxf(b0, sm.colA[r][p].x);
    b1 = fmaxf(b1, sm.colA[r][p].y);
  }
  // codes by magic rounding: |x| <= B_j and s = fl(127 / B_j) keep the exact
  // product within 127 (1 + 2^-24), so the rounded code never leaves +-127 and
  // its two's-complement byte is the low byte of m
  const float s0 = b0 > 0.f ? 127.0f / b0 : 0.f, s1 = b1 > 0.f ? 127.0f / b1 : 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    x[2 * m] = fmaf(x[2 * m], s0, kMagic);
    x[2 * m + 1] = fmaf(x[2 * m + 1], s1, kMagic);
  }
  uint32_t wd[16];
  pack_magic<8>(x, wd);
  store_chunk<8, NP>(wp.Z, rb, p, wd);
  if (rb == 0) *reinterpret_cast<float2*>(wp.B + j0) = make_float2(b0, b1);
  if (t == 0) wp.ell[0] = 0;
  if (clear_records) {
    if (t < 3) wp.ell[1 + t] = 0;
    for (int i = t; i < P; i += NT) wp.alpha[i] = 0.f;
    for (int i = t; i < P * (DK + DV); i += NT) wp.K[i] = 0.f;  // K and U are contiguous
  }
}

// Rebuild the dense state of L records (staged in LDS; record L-1 replaced by
// the current token's when `last_new`) and R compensator pairs (staged) into
// x, which holds the boundary codes Z on entry.
template <int DK, int DV, int PM, int RMX>
__device__ __forceinline__ void rebuild(float (&x)[64], const WinPtrs& wp, int L, int R,
                                        bool last_new, SmemWin<DK, DV, PM, RMX>& sm) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NT = G::NT;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  // factor of record j: prod_{m=j+1}^{L-1} al[m]; Gamma over all L records
  if (t < 64) decay_suffix<PM>(sm.al, L, sm.g1);
  __syncthreads();
  for (int i = t; i < L * DK; i += NT) {
    const int j = i / DK, a = i - j * DK;
    const float kt = (last_new && j == L - 1) ? sm.ktn[a] : sm.u.rec.K[j][a];
    sm.u.rec.K[j][a] = sm.g1[j] * kt;
  }
  if (last_new)
    for (int i = t; i < DV; i += NT) sm.u.rec.U[L - 1][i] = sm.unew[i];
  if (t < DK) sm.rowf[t] = sm.g1[PM] * sm.crow[t] * (1.0f / 127.0f);
  __syncthreads();
  const float2 bb = sm.bcol[p];
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float f = sm.rowf[r0 + m];
    x[2 * m] = (x[2 * m] * f) * bb.x;
    x[2 * m + 1] = (x[2 * m + 1] * f) * bb.y;
  }
  // compensator pairs decay with the boundary: Gamma_{1:L} kc_h uc_h^T
  const float gb = sm.g1[PM];
  for (int h = 0; h < R; ++h) {
    const float u0 = gb * sm.uc[h][j0], u1 = gb * sm.uc[h][j0 + 1];
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sm.kc[h][r0 + m]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * (m + q)] = fmaf(kv[q], u0, x[2 * (m + q)]);
        x[2 * (m + q) + 1] = fmaf(kv[q], u1, x[2 * (m + q) + 1]);
      }
    }
  }
  for (int j = 0; j < L; ++j) {
    const float2 u = *reinterpret_cast<const float2*>(&sm.u.rec.U[j][j0]);
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
      const float4 k4 = *reinterpret_cast<const float4*>(&sm.u.rec.K[j][r0 + m]);
      const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[2 * (m + q)] = fmaf(kv[q], u.x, x[2 * (m + q)]);
        x[2 * (m + q) + 1] = fmaf(kv[q], u.y, x[2 * (m + q) + 1]);
      }
    }
  }
}

template <int DK, int DV, int PM, int OP, int RMX>
__global__ __launch_bounds__((DK / 32) * (DV / 2))
__attribute__((amdgpu_waves_per_eu(4, 8))) void window_tile_kernel(TileArgs a) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  __shared__ SmemWin<DK, DV, PM, RMX> sm;
  const int tile = blockIdx.x;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  int h = 0;
  unsigned char* base = nullptr;
  if (!resolve_tile(a, tile, h, base)) {
    if (OP == OP_DECODE && t < DV) a.y[(long long)tile * DV + t] = __builtin_nanf("");
    return;
  }
  const int P = a.P.p, R = RMX > 0 ? a.P.rank : 0;
  const WinPtrs wp = win_ptrs(base, wuni(a.P.r_off[h]), DK, DV, P, R);
  constexpr int op = OP;
  float x[64];
  if constexpr (op == OP_PACK) {
    const float* X = a.X + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float2 v2 = *reinterpret_cast<const float2*>(X + (r0 + m) * DV + j0);
      x[2 * m] = v2.x;
      x[2 * m + 1] = v2.y;
    }
    if (R > 0) fit_compensators<DK, DV, PM, RMX>(x, wp, R, a.P.iters, false, sm);
    encode_boundary<DK, DV, PM, RMX>(x, wp, a.P.c_floor, sm, P, true);
    return;
  }
  // The window position is read first; the loads that do not depend on it
  // (boundary codes, the token's inputs) go out behind it, so that they share
  // one memory round trip with the staging of the records and pairs held.
  // A position outside [0, p) is not a state this library writes; it is
  // clamped so that every access stays inside the head.
  const int ell0 = wp.ell[0];
  uint32_t wd[16];
  load_chunk<8, NP>(wp.Z, rb, p, wd);
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  float kk = 0.f, qq = 0.f, alpha = 0.f, beta = 0.f;
  // the boundary's scales and the token's v are used after block barriers
  // (readout tail, rebuild): they go out with the codes and wait in LDS
  const float ca = p < 32 ? wp.C[r0 + p] : 0.f;
  float2 bcol = make_float2(0.f, 0.f), vin = make_float2(0.f, 0.f);
  if (rb == 0) bcol = *reinterpret_cast<const float2*>(wp.B + j0);
  if constexpr (op == OP_DECODE) {
    alpha = a.gate[tile];
    beta = a.beta[tile];
    if (p < 32) {
      const int r = r0 + p;
      kk = a.k[tk + r];
      qq = a.q[tk + r];
    }
    if (rb == 0) vin = *reinterpret_cast<const float2*>(a.v + tv + j0);
  }
  const int ell = min(max(ell0, 0), P - 1);
  {
    Staged<DK, DV, PM, RMX> stg;
    stg.issue(wp, ell, R);
    stg.commit(ell, R, sm);
    if (p < 32) sm.crow[r0 + p] = ca;
    if (rb == 0) {
      sm.bcol[p] = bcol;
      sm.vin[p] = vin;
    }
  }
  unpack_signed8(wd, x);  // Z
  if constexpr (op == OP_UNPACK || op == OP_FLUSH) {
    if (op == OP_FLUSH && ell == 0) return;
    __syncthreads();
    rebuild<DK, DV, PM, RMX>(x, wp, ell, R, false, sm);
    if constexpr (op == OP_FLUSH) {
      if (R > 0) fit_compensators<DK, DV, PM, RMX>(x, wp, R, a.P.iters, true, sm);
      encode_boundary<DK, DV, PM, RMX>(x, wp, a.P.c_floor, sm, P, false);
      return;
    }
    float* S = a.S_out + (long long)tile * DK * DV;
#pragma unroll
    for (int m = 0; m < 32; ++m)
      *reinterpret_cast<float2*>(S + (r0 + m) * DV + j0) = make_float2(x[2 * m], x[2 * m + 1]);
    return;
  }
  // ---- decode token i = ell + 1 (record index ell, 0-based)
  if (t == 0) sm.al[ell] = alpha;
  if (p < 32) {  // per-row constants of this wave's rows
    const int r = r0 + p;
    const float x1 = alpha * kk, kn = beta * kk;
    sm.x1[r] = x1;
    sm.qv[r] = qq;
    sm.ktn[r] = kn;
    sm.cx1[r] = ca * x1;
    sm.cq[r] = ca * qq;
    wp.K[ell * DK + r] = kn;  // the new record's key (record slot ell is free)
  }
  __syncthreads();
  // g1[j] = prod_{m=j+1}^{ell-1} al[m] (for u_i), g2[j] = prod_{m=j+1}^{ell} al[m]
  // (for o_i); index PM holds the products over all records
  if (t < 64) {
    decay_suffix<PM>(sm.al, ell, sm.g1);
    decay_suffix<PM>(sm.al, ell + 1, sm.g2);
  }
  // dot products over this wave's rows.  Unit u < PM is record u (the
  // token's own key at u = ell), unit PM + h compensator pair h; the units
  // take NU lanes (a power of two), and the wave's 32 rows are split into
  // SEG segments over the remaining lanes (lane p: unit p % NU, segment
  // p / NU), whose partial sums combine across lanes NU apart.  Each unit
  // walks its segment's rows in a rotated order, so the lanes of one
  // instruction read different rows of their key vectors rather than one
  // LDS bank.
  {
    constexpr int NU = PM + RMX <= 16 ? 16 : PM + RMX <= 32 ? 32 : 64;
    constexpr int SEG = NP / NU >= 4 ? 4 : NP / NU >= 2 ? 2 : 1;
    constexpr int L = 32 / SEG;
    const int u = p % NU, sg = p / NU;
    const bool rec = u < PM && u <= ell, cmp = u >= PM && u < PM + R;
    float d1 = 0.f, d2 = 0.f;
    if (sg < SEG && (rec || cmp)) {
      const float* src = cmp ? sm.kc[u - PM] : (u == ell ? sm.ktn : sm.u.rec.K[u]);
      const int rs = r0 + sg * L;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int rr = rs + ((i + u) & (L - 1));
        const float kt = src[rr];
        d1 = fmaf(kt, sm.x1[rr], d1);
        d2 = fmaf(kt, sm.qv[rr], d2);
      }
    }
    if constexpr (SEG >= 2) {  // partner lanes NU apart (16 or 32)
      float a0, b0, a1, b1;
      if constexpr (NU == 16) {
        swap16(d1, a0, b0);
        swap16(d2, a1, b1);
      } else {
        swap32(d1, a0, b0);
        swap32(d2, a1, b1);
      }
      d1 = a0 + b0;
      d2 = a1 + b1;
    }
    if constexpr (SEG == 4) {  // and 32 apart
      float a0, b0, a1, b1;
      swap32(d1, a0, b0);
      swap32(d2, a1, b1);
      d1 = a0 + b0;
      d2 = a1 + b1;
    }
    if (sg == 0 && (rec || cmp)) sm.dots[rb][u] = make_float2(d1, d2);
  }
  // boundary readouts: sum_a Z_aj (C_a x_a)
  float s10 = 0.f, s11 = 0.f, s20 = 0.f, s21 = 0.f;
#pragma unroll
  for (int m = 0; m < 32; m += 4) {
    const float4 f1 = *reinterpret_cast<const float4*>(&sm.cx1[r0 + m]);
    const float4 f2 = *reinterpret_cast<const float4*>(&sm.cq[r0 + m]);
    const float v1[4] = {f1.x, f1.y, f1.z, f1.w}, v2[4] = {f2.x, f2.y, f2.z, f2.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s10 = fmaf(v1[q], x[2 * (m + q)], s10);
      s11 = fmaf(v1[q], x[2 * (m + q) + 1], s11);
      s20 = fmaf(v2[q], x[2 * (m + q)], s20);
      s21 = fmaf(v2[q], x[2 * (m + q) + 1], s21);
    }
  }
  sm.colA[rb][p] = make_float2(s10, s11);
  sm.colB[rb][p] = make_float2(s20, s21);
  __syncthreads();
  if (rb == 0) {
    float r10 = 0.f, r11 = 0.f, r20 = 0.f, r21 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      r10 += sm.colA[r][p].x;
      r11 += sm.colA[r][p].y;
      r20 += sm.colB[r][p].x;
      r21 += sm.colB[r][p].y;
    }
    const float2 bb = sm.bcol[p];
    const float f0 = bb.x * (1.0f / 127.0f), f1 = bb.y * (1.0f / 127.0f);
    float pv0 = sm.g1[PM] * f0 * r10, pv1 = sm.g1[PM] * f1 * r11;
    float w0 = sm.g2[PM] * f0 * r20, w1 = sm.g2[PM] * f1 * r21;
    // each unit's dot products summed over the row blocks and scaled by its
    // decay, one lane per unit (records 0 .. ell, then the pairs), so the
    // serial loops below read one value per unit
    {
      const int u = p;
      if (u < PM + R && (u <= ell || u >= PM)) {
        float d1 = 0.f, d2 = 0.f;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
          d1 += sm.dots[r][u].x;
          d2 += sm.dots[r][u].y;
        }
        const int gi = u >= PM ? PM : u;  // compensators decay with the boundary
        sm.esum[u] = u == ell ? make_float2(0.f, d2) : make_float2(sm.g1[gi] * d1, sm.g2[gi] * d2);
      }
      wave_sync();
    }
    for (int hh = 0; hh < R; ++hh) {
      const float2 e = sm.esum[PM + hh];
      const float uc0 = sm.uc[hh][j0], uc1 = sm.uc[hh][j0 + 1];
      pv0 = fmaf(uc0, e.x, pv0);
      pv1 = fmaf(uc1, e.x, pv1);
      w0 = fmaf(uc0, e.y, w0);
      w1 = fmaf(uc1, e.y, w1);
    }
    for (int j = 0; j < ell; ++j) {
      const float2 e = sm.esum[j];
      const float2 u = *reinterpret_cast<const float2*>(&sm.u.rec.U[j][j0]);
      pv0 = fmaf(u.x, e.x, pv0);
      pv1 = fmaf(u.y, e.x, pv1);
      w0 = fmaf(u.x, e.y, w0);
      w1 = fmaf(u.y, e.y, w1);
    }
    const float dn = sm.esum[ell].y;  // kt_i . q
    const float2 vv = sm.vin[p];
    const float u0 = vv.x - pv0, u1 = vv.y - pv1;
    w0 = fmaf(u0, dn, w0);
    w1 = fmaf(u1, dn, w1);
    *reinterpret_cast<float2*>(wp.U + ell * DV + j0) = make_float2(u0, u1);
    *reinterpret_cast<float2*>(a.y + tv + j0) = make_float2(w0, w1);
    sm.unew[j0] = u0;
    sm.unew[j0 + 1] = u1;
  }
  if (ell + 1 < P) {
    if (t == 0) {
      wp.alpha[ell] = alpha;
      wp.ell[0] = ell + 1;
    }
    return;
  }
  // the window is full: rebuild S_p from the staged records, refit the
  // compensators and re-encode the residual
  __syncthreads();
  rebuild<DK, DV, PM, RMX>(x, wp, P, R, true, sm);
  if (R > 0) fit_compensators<DK, DV, PM, RMX>(x, wp, R, a.P.iters, true, sm);
  encode_boundary<DK, DV, PM, RMX>(x, wp, a.P.c_floor, sm, P, false);
}

template <int DK, int DV, int PM, int RMX>
hipError_t launch_op(const TileArgs& a, hipStream_t s) {
  const dim3 grid(a.n_tiles), block((DK / 32) * (DV / 2));
  switch (a.op) {
    case OP_DECODE: hipLaunchKernelGGL((window_tile_kernel<DK, DV, PM, OP_DECODE, RMX>), grid, block, 0, s, a); break;
    case OP_PACK: hipLaunchKernelGGL((window_tile_kernel<DK, DV, PM, OP_PACK, RMX>), grid, block, 0, s, a); break;
    case OP_UNPACK: hipLaunchKernelGGL((window_tile_kernel<DK, DV, PM, OP_UNPACK, RMX>), grid, block, 0, s, a); break;
    case OP_FLUSH: hipLaunchKernelGGL((window_tile_kernel<DK, DV, PM, OP_FLUSH, RMX>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DK, int DV, int PM>
hipError_t launch_pm(const TileArgs& a, hipStream_t s) {
  return a.P.rank > 0 ? launch_op<DK, DV, PM, RM>(a, s) : launch_op<DK, DV, PM, 0>(a, s);
}

template <int DK, int DV>
hipError_t launch(const TileArgs& a, hipStream_t s) {
  return a.P.p <= 16 ? launch_pm<DK, DV, 16>(a, s) : launch_pm<DK, DV, 32>(a, s);
}

}  // namespace

hipError_t launch_tile_window(const TileArgs& a, hipStream_t s) {
  if (a.P.p > 32 || a.P.p < 1 || a.P.rank < 0 || a.P.rank > RM) return hipErrorInvalidValue;
  // compensator lanes follow the record lanes inside one row block
  if (a.P.rank > 0 && (a.P.p <= 16 ? 16 : 32) + RM > a.P.dv / 2) return hipErrorInvalidValue;
  const int dk = a.P.dk, dv = a.P.dv;
  if (dk == 128 && dv == 128) return launch<128, 128>(a, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(a, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(a, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(a, s);
  return hipErrorInvalidValue;
}
