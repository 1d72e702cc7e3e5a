// Chunkwise (matrix-form) prefill of the gated delta rule on the matrix cores.
//
// The serving flow runs a prompt through a chunk kernel between unpacking the
// active states and packing the boundary states (STEPQuant App. F.1).  Over a
// chunk of C tokens starting from state S0, the recurrence
//   S_t = D_t S_{t-1} + k_t u_t^T,   u_t = beta_t (v_t - (D_t S_{t-1})^T k_t),
//   y_t = S_t^T q_t                    (STEPQuant Sec. 3, Eq. 1),
// unrolls with the decay products g_t = prod_{r<=t} d_r (per key row) and
// G_ts = prod_{s<r<=t} d_r into
//   (I + A) U = diag(beta) V - diag(beta) (K o g) S0,
//   A_ts = beta_t sum_c k_tc G_tsc k_sc            (s < t),
//   Y    = (Q o g) S0 + L U,  L_ts = sum_c q_tc G_tsc k_sc   (s <= t),
//   S_C  = diag(g_C) S0 + (K o G_C.)^T U,
// so with W = (I + A)^-1 diag(beta) (K o g) and U0 = (I + A)^-1 diag(beta) V,
// U = U0 - W S0.  The three state products W S0, (Q o g) S0 and (K o G)^T U
// and the intra-chunk L U are fp32 matrix-core products (v_mfma_f32_16x16x4);
// the decay products, A, L and the unit-triangular solves are vector work.
// The result equals the token-serial recurrence up to rounding order.
//
// One workgroup of 4 waves runs one (sequence, head) tile through all its
// chunks.  The state stays in registers in the matrix-core accumulator
// layout: wave w owns state columns [w d_v/4, (w+1) d_v/4), and a lane holds
// rows 16 ib + 4 (lane / 16) + r (r = 0..3) of column 16 jb + lane % 16 of
// each 16 x 16 block.  Because a product's reduction index may be permuted
// freely, that same register serves as the B operand of (W S0), whose k-step r
// of row block ib takes rows 16 ib + 4 (lane / 16) + r, and the U block that
// (W S0) produces serves as the B operand of L U and (K o G)^T U the same way.
// Every B operand is a register; every A operand is a 16-byte LDS read.  The
// columns of the state evolve independently (D_t acts on rows), so the four
// waves need no exchange in the product phase.
#include "tile_common.h"

using namespace sqk;

namespace {

constexpr int CH = 32;        // tokens per chunk
constexpr int CP = CH + 4;    // padded row of a [.][CH] array

template <int DK, int DV, bool KDA>
struct alignas(16) ChunkSmem {
  static constexpr int KP = DK + 4, VP = DV + 4;
  float K[CH][KP];    // keys; after the walk W (in place)
  float Q[CH][KP];    // queries; after the walk Q o g (in place)
  float V[CH][VP];    // values; after the solve U0 (in place)
  float KT[DK][CP];   // (K o G_C.)^T: keys decayed to the chunk end, transposed
  float A[CH][CP];    // strictly lower A (row t, column s)
  float L[CH][CP];    // lower L, zero above the diagonal of its 16 x 16 blocks
  float glast[DK];    // g over the whole chunk
  float be[CH];
  float al[CH];       // GDN: the chunk's gates alpha_t
  float D[KDA ? CH : 1][KDA ? KP : 1];  // KDA: the chunk's gates d_t

  __device__ __forceinline__ float gate(int t, int c) const {
    if constexpr (KDA) return D[t][c];
    else return al[t];
  }
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// x <- (I + A)^-1 x for one column held in registers (A unit lower
// triangular, its strictly lower part in LDS; every lane reads the same row).
template <int N>
__device__ __forceinline__ void unit_lower_solve(const float (&A)[CH][CP], float (&x)[N]) {
#pragma unroll
  for (int t = 1; t < N; ++t) {
    float acc = x[t];
#pragma unroll
    for (int s4 = 0; s4 < t; s4 += 4) {
      const f32x4 a = ld4(&A[t][s4]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (s4 + e < t) acc = fmaf(-a[e], x[s4 + e], acc);
    }
    x[t] = acc;
  }
}

template <int DK, int DV, bool KDA>
__global__ __launch_bounds__(256) void chunk_prefill_kernel(int H, int T, float* S, const float* q,
                                                            const float* k, const float* v,
                                                            const float* beta, const float* gate,
                                                            float* y) {
  constexpr int IB = DK / 16, JB = DV / 64, TB = CH / 16, CPG = DK / 16;
  __shared__ ChunkSmem<DK, DV, KDA> sm;
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
    // ---- stage the chunk (tokens past T read as k = q = v = 0, beta = 0, gate 1)
#pragma unroll
    for (int m = 0; m < CH * DK / 4 / 256; ++m) {
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
    for (int m = 0; m < CH * DV / 4 / 256; ++m) {
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

    // ---- A and L: lanes of a 16-lane row share a key s and split the channels
    {
      const int pr = tid >> 4, cg = tid & 15, cb = cg * CPG;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s = half ? CH - 1 - pr : pr;
        if (cg == 0)
          for (int t = s & ~15; t < s; ++t) sm.L[t][s] = 0.f;
        float ks[CPG], P[CPG];
#pragma unroll
        for (int c = 0; c < CPG; ++c) {
          ks[c] = sm.K[s][cb + c];
          P[c] = 1.f;
        }
        float ps = 1.f;
        for (int t = s; t < CH; ++t) {
          float a = 0.f, b = 0.f;
          if constexpr (KDA) {
            if (t > s) {
#pragma unroll
              for (int c = 0; c < CPG; ++c) P[c] *= sm.D[t][cb + c];
            }
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
              const float kp = ks[c] * P[c];
              a = fmaf(sm.K[t][cb + c], kp, a);
              b = fmaf(sm.Q[t][cb + c], kp, b);
            }
          } else {
            if (t > s) ps *= sm.al[t];
#pragma unroll
            for (int c = 0; c < CPG; ++c) {
              a = fmaf(sm.K[t][cb + c], ks[c], a);
              b = fmaf(sm.Q[t][cb + c], ks[c], b);
            }
            a *= ps;
            b *= ps;
          }
          a = row16_sum(a);
          b = row16_sum(b);
          if (cg == 0) {
            sm.A[t][s] = sm.be[t] * a;   // the diagonal entry is never read
            sm.L[t][s] = b;
          }
        }
      }
    }
    __syncthreads();

    // ---- decay walks and the unit-triangular solves, one column per lane
    if (tid < DK) {
      const int c = tid;
      float ge = 1.f;
#pragma unroll
      for (int t = CH - 1; t >= 0; --t) {
        sm.KT[c][t] = sm.K[t][c] * ge;
        ge *= sm.gate(t, c);
      }
      sm.glast[c] = ge;
      float x[CH], gp = 1.f;
#pragma unroll
      for (int t = 0; t < CH; ++t) {
        gp *= sm.gate(t, c);
        x[t] = sm.be[t] * sm.K[t][c] * gp;
        sm.Q[t][c] *= gp;
      }
      unit_lower_solve<CH>(sm.A, x);
#pragma unroll
      for (int t = 0; t < CH; ++t) sm.K[t][c] = x[t];
    } else if (tid < DK + DV) {
      const int j = tid - DK;
      float x[CH];
#pragma unroll
      for (int t = 0; t < CH; ++t) x[t] = sm.be[t] * sm.V[t][j];
      unit_lower_solve<CH>(sm.A, x);
#pragma unroll
      for (int t = 0; t < CH; ++t) sm.V[t][j] = x[t];
    }
    __syncthreads();

    // ---- the state products on the matrix cores
    f32x4 u[TB][JB], yv[TB][JB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        f32x4 ws = {0.f, 0.f, 0.f, 0.f}, yi = ws;
#pragma unroll
        for (int ib = 0; ib < IB; ++ib) {
          const f32x4 wa = ld4(&sm.K[16 * tb + l16][16 * ib + 4 * g]);
          const f32x4 qa = ld4(&sm.Q[16 * tb + l16][16 * ib + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ws = mfma4(wa[r], st[ib][jb][r], ws);
            yi = mfma4(qa[r], st[ib][jb][r], yi);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) u[tb][jb][r] = sm.V[16 * tb + 4 * g + r][jw + 16 * jb + l16] - ws[r];
        yv[tb][jb] = yi;
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
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      const f32x4 gl = ld4(&sm.glast[16 * ib + 4 * g]);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ib][jb][r] *= gl[r];
#pragma unroll
        for (int sb = 0; sb < TB; ++sb) {
          const f32x4 ka = ld4(&sm.KT[16 * ib + l16][16 * sb + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r) st[ib][jb] = mfma4(ka[r], u[sb][jb][r], st[ib][jb]);
        }
      }
    }
    __syncthreads();   // the next chunk overwrites every array
  }

#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) St[(16 * ib + 4 * g + r) * DV + jw + 16 * jb + l16] = st[ib][jb][r];
}

template <int DK, int DV>
hipError_t launch(int kind, int H, int B, int T, float* S, const float* q, const float* k,
                  const float* v, const float* beta, const float* gate, float* y, hipStream_t s) {
  if (kind == SQ_KIND_KDA)
    hipLaunchKernelGGL((chunk_prefill_kernel<DK, DV, true>), dim3(B * H), dim3(256), 0, s, H, T, S,
                       q, k, v, beta, gate, y);
  else
    hipLaunchKernelGGL((chunk_prefill_kernel<DK, DV, false>), dim3(B * H), dim3(256), 0, s, H, T, S,
                       q, k, v, beta, gate, y);
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
