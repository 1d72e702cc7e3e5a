// Chunkwise (matrix-form) prefill of the gated delta rule on the matrix cores.
//
// The serving flow runs a prompt through a chunk kernel between unpacking the
// active states and packing the boundary states (STEPQuant App. F.1).  Over a
// block of C tokens starting from state S0, the recurrence
//   S_t = D_t S_{t-1} + k_t u_t^T,   u_t = beta_t (v_t - (D_t S_{t-1})^T k_t),
//   y_t = S_t^T q_t                    (STEPQuant Sec. 3, Eq. 1),
// unrolls with the decay products g_t = prod_{r<=t} d_r (per key row) and
// G_ts = prod_{s<r<=t} d_r into
//   (I + A) U = diag(beta) V - diag(beta) (K o g) S0,
//   A_ts = beta_t sum_c k_tc G_tsc k_sc            (s < t),
//   Y    = (Q o g) S0 + L U,  L_ts = sum_c q_tc G_tsc k_sc   (s <= t),
//   S_C  = diag(g_C) S0 + (K o G_C.)^T U.
// With T = (I + A)^-1 (unit lower triangular, one column per lane) and
// R = diag(beta) (K o g): U = T (diag(beta) V - R S0).  The products R S0,
// (Q o g) S0, T Z, L U and (K o G_C.)^T U are fp32 matrix-core products
// (v_mfma_f32_16x16x4); G enters as exact running products, never as a
// ratio of prefix products, so gates of 0 stay exact.  For GDN the decays are
// one factor per token: k_t.k_s and q_t.k_s are matrix-core products too, and
// g, beta and G_C. scale rows of the products in registers instead of copies
// of K and Q.  For KDA the decays differ per key channel: A and L are summed
// on the vector units with a running product per channel, and a walk per
// channel writes beta g o k, g o q and the keys decayed to the block end.
// The result equals the token-serial recurrence up to rounding order.
//
// One workgroup of 4 waves runs one (sequence, head) tile through all its
// blocks.  The state stays in registers in the matrix-core accumulator
// layout: wave w owns state columns [w d_v/4, (w+1) d_v/4), and a lane holds
// rows 16 ib + 4 (lane / 16) + r (r = 0..3) of column 16 jb + lane % 16 of
// each 16 x 16 block.  Because a product's reduction index may be permuted
// freely, that same register serves as the B operand of R S0, whose k-step r
// of row block ib takes rows 16 ib + 4 (lane / 16) + r, and the Z and U
// blocks the products leave in that layout serve as B operands of T Z, L U
// and (K o G_C.)^T U the same way.  Every B operand is a register; every A
// operand is an LDS read.  The columns of the state evolve independently
// (D_t acts on rows), so the four waves need no exchange in the products.
#include "tile_common.h"

using namespace sqk;

namespace {

template <int DK, int DV, bool KDA, int CH>
struct ChunkSmem {
  static constexpr int KP = DK + 4, CP = CH + 4;   // padded rows
  alignas(16) float K[CH][KP];    // keys; KDA: beta_t g_t o k_t after the walk (in place)
  alignas(16) float Q[CH][KP];    // queries; KDA: g_t o q_t after the walk (in place)
  alignas(16) float V[CH][DV];    // values
  alignas(16) float A[CH][CP];    // strictly lower A
  alignas(16) float L[CH][CP];    // lower L, zero above the diagonal
  alignas(16) float T[CH][CP];    // (I + A)^-1, unit lower triangular
  alignas(16) float be[CH];       // beta_t
  alignas(16) float glast[DK];    // g over the whole block (GDN: entry 0)
  // GDN: the scalar gates and their prefix and suffix products
  alignas(16) float al[KDA ? 1 : CH];
  alignas(16) float gp[KDA ? 1 : CH];
  alignas(16) float ge[KDA ? 1 : CH];
  // KDA: the channel gates and (K o G_end)^T, keys decayed to the block end
  alignas(16) float D[KDA ? CH : 1][KDA ? KP : 1];
  alignas(16) float KT[KDA ? DK : 1][KDA ? CP : 1];
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// x <- (I + A)^-1 x for one column held in registers (A strictly lower in
// LDS, every lane reading the same row).
template <int N, int CP>
__device__ __forceinline__ void unit_lower_solve(const float (*A)[CP], float (&x)[N]) {
#pragma unroll
  for (int t = 1; t < N; ++t) {
    float acc0 = x[t], acc1 = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < t; s4 += 4) {
      const f32x4 a = ld4(&A[t][s4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (s4 + e >= t) continue;
        if (e & 1) acc1 = fmaf(-a[e], x[s4 + e], acc1);
        else acc0 = fmaf(-a[e], x[s4 + e], acc0);
      }
    }
    x[t] = acc0 + acc1;
  }
}

// Column j of (I + A)^-1 into T.
template <int CH, int CP>
__device__ __forceinline__ void inverse_column(const float (*A)[CP], float (*T)[CP], int j) {
  float x[CH];
#pragma unroll
  for (int t = 0; t < CH; ++t) x[t] = t == j ? 1.f : 0.f;
  unit_lower_solve<CH, CP>(A, x);
#pragma unroll
  for (int t = 0; t < CH; ++t) T[t][j] = x[t];
}

// Two sums over the LPP lanes that share a key (16: a DPP row; 32: two rows)
// in one reduction: the even lane of each pair keeps a, the odd lane b, then
// the rotations by 2, 4 and 8 within a row keep each lane's parity, and the
// row exchange adds the other row.  Even lanes return the sum of a, odd
// lanes the sum of b.
template <int LPP>
__device__ __forceinline__ float pair_sum2(float a, float b, bool odd) {
  float v = (odd ? b : a) + dpp_f<0xB1>(odd ? a : b);   // quad_perm xor 1
  v += dpp_f<0x122>(v);                                  // row_ror:2
  v += dpp_f<0x124>(v);                                  // row_ror:4
  v += dpp_f<0x128>(v);                                  // row_ror:8
  if constexpr (LPP == 32) {
    float x, y;
    swap16(v, x, y);
    v = x + y;
  }
  return v;
}

template <int DK, int DV, bool KDA, int CH>
__global__ __launch_bounds__(256, 3) void chunk_prefill_kernel(
    int H, int T, float* S, const float* q, const float* k, const float* v, const float* beta,
    const float* gate, float* y) {
  using SM = ChunkSmem<DK, DV, KDA, CH>;
  constexpr int IB = DK / 16, JB = DV / 64, TB = CH / 16;
  __shared__ SM sm;
  const int tile = blockIdx.x, bi = tile / H, h = tile - bi * H;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const int jw = w * (DV / 4);   // first state column of this wave
  float* St = S + (long long)tile * DK * DV;
  const long long tok0 = (long long)bi * T;   // token s of this tile: (tok0 + s) H + h

  f32x4 st[IB][JB];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[ib][jb][r] = St[(16 * ib + 4 * g + r) * DV + jw + 16 * jb + l16];

  for (int c0 = 0; c0 < T; c0 += CH) {
    // ---- stage the block (tokens past T read as k = q = v = 0, beta = 0, gate 1)
#pragma unroll
    for (int m = 0; m < CH * DK / 1024; ++m) {
      const int e = tid + 256 * m, t = e / (DK / 4), c4 = 4 * (e % (DK / 4));
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, qv = kv, dv = {1.f, 1.f, 1.f, 1.f};
      if (c0 + t < T) {
        const long long o = ((tok0 + c0 + t) * H + h) * DK + c4;
        kv = ld4(k + o);
        qv = ld4(q + o);
        if constexpr (KDA) dv = ld4(gate + o);
      }
      *reinterpret_cast<f32x4*>(&sm.K[t][c4]) = kv;
      *reinterpret_cast<f32x4*>(&sm.Q[t][c4]) = qv;
      if constexpr (KDA) *reinterpret_cast<f32x4*>(&sm.D[t][c4]) = dv;
    }
#pragma unroll
    for (int m = 0; m < CH * DV / 1024; ++m) {
      const int e = tid + 256 * m, t = e / (DV / 4), c4 = 4 * (e % (DV / 4));
      f32x4 vv = {0.f, 0.f, 0.f, 0.f};
      if (c0 + t < T) vv = ld4(v + ((tok0 + c0 + t) * H + h) * DV + c4);
      *reinterpret_cast<f32x4*>(&sm.V[t][c4]) = vv;
    }
    if (tid < CH) {
      const bool in = c0 + tid < T;
      const long long th = (tok0 + c0 + tid) * H + h;
      sm.be[tid] = in ? beta[th] : 0.f;
      if constexpr (!KDA) sm.al[tid] = in ? gate[th] : 1.f;
    }
    __syncthreads();

    if constexpr (!KDA) {
      // ---- GDN: k_t . k_s and q_t . k_s on the matrix cores (one 16 x 16
      // block of the lower triangle per wave), G_ts and the gate products on
      // the last wave
      constexpr int NB = TB * (TB + 1) / 2;
      if (w < NB) {
        const int tb = w == 0 ? 0 : 1, sb = w == 2 ? 1 : 0;
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          const f32x4 kt = ld4(&sm.K[16 * tb + l16][16 * ib + 4 * g]);
          const f32x4 ks = ld4(&sm.K[16 * sb + l16][16 * ib + 4 * g]);
          const f32x4 qt = ld4(&sm.Q[16 * tb + l16][16 * ib + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kk = mfma4(kt[r], ks[r], kk);
            qk = mfma4(qt[r], ks[r], qk);
          }
        }
        // this lane's entries: t = t0 + r (r = 0..3), s; G_ts = prod_{s<r'<=t} alpha_r'
        const int t0 = 16 * tb + 4 * g, s = 16 * sb + l16;
        float P = 1.f;
#pragma unroll
        for (int t4 = 0; t4 < CH; t4 += 4) {
          const f32x4 a4 = ld4(&sm.al[t4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) P *= (t4 + e > s && t4 + e <= t0) ? a4[e] : 1.f;
        }
        const f32x4 at = ld4(&sm.al[t0]), bt = ld4(&sm.be[t0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = t0 + r;
          if (r > 0 && t > s) P *= at[r];
          sm.A[t][s] = s < t ? bt[r] * P * kk[r] : 0.f;
          sm.L[t][s] = s <= t ? P * qk[r] : 0.f;
        }
      } else if (w == 3 && l < CH) {   // the gate products of the block
        const int s = l;
        float gpv = 1.f, gev = 1.f;
#pragma unroll
        for (int t4 = 0; t4 < CH; t4 += 4) {
          const f32x4 a4 = ld4(&sm.al[t4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (t4 + e <= s) gpv *= a4[e];
            else gev *= a4[e];
          }
        }
        sm.gp[s] = gpv;   // prod_{r <= s} alpha_r
        sm.ge[s] = gev;   // prod_{r > s} alpha_r
        if (s == CH - 1) sm.glast[0] = gpv;
      }
      __syncthreads();
      // ---- T = (I + A)^-1 on wave 0
      if (w == 0 && l < CH) inverse_column<CH, SM::CP>(sm.A, sm.T, l);
      __syncthreads();
    } else {
      // ---- KDA: A and L on the vector units; the LPP lanes of a key s
      // split the channels and carry k_s decayed to token t (k_sc G_tsc, a
      // running product), pairs (s, CH-1-s) balance the triangle, and the
      // rows of token t + 1 are read while token t is reduced
      constexpr int LPP = 512 / CH, CPG = DK / LPP;
      {
        const int pr = tid / LPP, cg = tid % LPP, cb = cg * CPG;
        const bool odd = cg & 1;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int s = half ? CH - 1 - pr : pr;
          if (cg < 16) {   // L is zero above the diagonal of its 16 x 16 blocks
            const int t = (s & ~15) + cg;
            if (t < s) sm.L[t][s] = 0.f;
          }
          float kp[CPG], kn[CPG], qn[CPG], dn[CPG];
#pragma unroll
          for (int c = 0; c < CPG; ++c) {
            kp[c] = kn[c] = sm.K[s][cb + c];
            qn[c] = sm.Q[s][cb + c];
            dn[c] = 1.f;
          }
          for (int t = s; t < CH; ++t) {
            float kt[CPG], qt[CPG];
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
              kt[c] = kn[c];
              qt[c] = qn[c];
              kp[c] *= dn[c];   // 1 at t = s
            }
            if (t + 1 < CH) {
#pragma unroll
              for (int c = 0; c < CPG; ++c) {
                kn[c] = sm.K[t + 1][cb + c];
                qn[c] = sm.Q[t + 1][cb + c];
                dn[c] = sm.D[t + 1][cb + c];
              }
            }
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
              a = fmaf(kt[c], kp[c], a);
              b = fmaf(qt[c], kp[c], b);
            }
            const float sum = pair_sum2<LPP>(a, b, odd);
            if (cg < 2) {   // lane 0 writes A (the diagonal entry is never read), lane 1 L
              if (odd) sm.L[t][s] = sum;
              else sm.A[t][s] = sm.be[t] * sum;
            }
          }
        }
      }
      __syncthreads();
      // ---- decay walks, two lanes per key channel (the keys decayed to the
      // block end, then beta g o k in place; g o q), and T = (I + A)^-1 on
      // the last wave
      if (tid < DK) {
        const int c = tid;
        float gev = 1.f;
#pragma unroll
        for (int t = CH - 1; t >= 0; --t) {
          sm.KT[c][t] = sm.K[t][c] * gev;
          gev *= sm.D[t][c];
        }
        sm.glast[c] = gev;
        float gpv = 1.f;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          gpv *= sm.D[t][c];
          sm.K[t][c] = sm.be[t] * gpv * sm.K[t][c];
        }
      } else if (tid < 2 * DK) {
        const int c = tid - DK;
        float gpv = 1.f;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          gpv *= sm.D[t][c];
          sm.Q[t][c] *= gpv;
        }
      }
      if (w == 3 && l < CH) inverse_column<CH, SM::CP>(sm.A, sm.T, l);
      __syncthreads();
    }

    // ---- the state products on the matrix cores.  Z = diag(beta) V - R S
    // with R = diag(beta) (K o g), Y = (Q o g) S + L U, U = T Z.
    f32x4 z[TB][JB], yv[TB][JB], u[TB][JB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) z[tb][jb] = yv[tb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {   // z <- R S, yv <- (Q o g) S
      f32x4 wa[TB], qa[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        wa[tb] = ld4(&sm.K[16 * tb + l16][16 * ib + 4 * g]);
        qa[tb] = ld4(&sm.Q[16 * tb + l16][16 * ib + 4 * g]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            z[tb][jb] = mfma4(wa[tb][r], st[ib][jb][r], z[tb][jb]);
            yv[tb][jb] = mfma4(qa[tb][r], st[ib][jb][r], yv[tb][jb]);
          }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * g + r;
        const float bt = sm.be[t];
        const float gt = KDA ? 1.f : sm.gp[t];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float vt = sm.V[t][jw + 16 * jb + l16];
          if constexpr (KDA) {
            z[tb][jb][r] = fmaf(bt, vt, -z[tb][jb][r]);
          } else {  // GDN: the row factors beta_t g_t and g_t applied here
            z[tb][jb][r] = bt * fmaf(-gt, z[tb][jb][r], vt);
            yv[tb][jb][r] *= gt;
          }
        }
      }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb <= tb; ++sb) {
          const f32x4 ta = ld4(&sm.T[16 * tb + l16][16 * sb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = mfma4(ta[r], z[sb][jb][r], acc);
        }
        u[tb][jb] = acc;
      }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
        for (int sb = 0; sb <= tb; ++sb) {
          const f32x4 la = ld4(&sm.L[16 * tb + l16][16 * sb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) yv[tb][jb] = mfma4(la[r], u[sb][jb][r], yv[tb][jb]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tb + 4 * g + r;
          if (c0 + t < T) y[((tok0 + c0 + t) * H + h) * DV + jw + 16 * jb + l16] = yv[tb][jb][r];
        }
      }
    // ---- S <- diag(g_end) S + (K o G_end)^T U
    if constexpr (!KDA) {  // GDN: G_end is a factor per token, applied to U
#pragma unroll
      for (int sb = 0; sb < TB; ++sb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = sm.ge[16 * sb + 4 * g + r];
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) u[sb][jb][r] *= e;
        }
    }
    const float gl0 = KDA ? 0.f : sm.glast[0];
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      f32x4 gl, ka[TB];
      if constexpr (KDA) gl = ld4(&sm.glast[16 * ib + 4 * g]);
      else gl = f32x4{gl0, gl0, gl0, gl0};
#pragma unroll
      for (int sb = 0; sb < TB; ++sb) {
        if constexpr (KDA) {
          ka[sb] = ld4(&sm.KT[16 * ib + l16][16 * sb + 4 * g]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) ka[sb][r] = sm.K[16 * sb + 4 * g + r][16 * ib + l16];
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        st[ib][jb] *= gl;
#pragma unroll
        for (int sb = 0; sb < TB; ++sb)
#pragma unroll
          for (int r = 0; r < 4; ++r) st[ib][jb] = mfma4(ka[sb][r], u[sb][jb][r], st[ib][jb]);
      }
    }
    __syncthreads();   // the next block overwrites every array
  }

  // (the lane offset passes through an empty asm so that the compiler does
  // not keep the initial load's 64 addresses alive across the loop)
  float* So = St + opaque(4 * g * DV + jw + l16);
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) So[(16 * ib + r) * DV + 16 * jb] = st[ib][jb][r];
}

// Blocks of 16 tokens: 30 KB (GDN) and 48 KB (KDA) of LDS and at most 168
// registers per lane hold three workgroups per CU, whose phases overlap.
// (Blocks of 32 measured 13-22 % slower on the large batches: they fit two
// workgroups, and the longer triangular solve runs on one wave.)
template <int DK, int DV>
hipError_t launch(int kind, int H, int B, int T, float* S, const float* q, const float* k,
                  const float* v, const float* beta, const float* gate, float* y, hipStream_t s) {
  if (kind == SQ_KIND_KDA)
    hipLaunchKernelGGL((chunk_prefill_kernel<DK, DV, true, 16>), dim3(B * H), dim3(256), 0, s, H,
                       T, S, q, k, v, beta, gate, y);
  else
    hipLaunchKernelGGL((chunk_prefill_kernel<DK, DV, false, 16>), dim3(B * H), dim3(256), 0, s, H,
                       T, S, q, k, v, beta, gate, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_chunkwise(int kind, int H, int dk, int dv, int B, int T, float* S,
                                    const float* q, const float* k, const float* v,
                                    const float* beta, const float* gate, float* y, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch<128, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  return hipErrorInvalidValue;
}
