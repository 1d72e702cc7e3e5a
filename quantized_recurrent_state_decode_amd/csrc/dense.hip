// Full-precision (fp32 state) gated delta-rule decode step: the FP32-state
// baseline the pages compare against (STEPQuant Sec. 5.1; LeapQuant notes
// Sec. 3.3), and the way large workloads build their warm-up states.
//   X = D S + beta k (v - (D S)^T k)^T,  y = X^T q,  S <- X (in place).
#include "tile_common.h"

using namespace sqk;

namespace {

// Lane (rb, p) owns rows 16 rb .. 16 rb + 15 of columns 4p .. 4p + 3, so
// every state access is one 16-byte load or store and a wave moves two
// contiguous 512-byte row segments per instruction (at d_v = 128).  The
// state is streamed with non-temporal loads and stores: each tile is read
// and written once per step, and keeping it out of the caches leaves them
// to the inputs (a 64 KB-tile read-modify-write sweep measured 5.7 TB/s
// this way against 5.2 TB/s with ordinary accesses).
template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void dense_kernel(
    int kind, int H, float* S, long long n_slots, const int* slots, const float* q,
    const float* k, const float* v, const float* beta, const float* gate, float* y) {
  constexpr int NP = DV / 4;                   // lanes per row (4 columns each)
  constexpr int NRB = DK / 16;                 // row blocks of 16 rows
  __shared__ float kd[DK], bk[DK], qq[DK], gg[DK];
  __shared__ float4 col[NRB][NP];
  const int tile = blockIdx.x, bi = tile / H, h = tile - bi * H;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 4 * p, r0 = 16 * rb;
  const long long tk = (long long)tile * DK, tv = (long long)tile * DV;
  const int slot = slots[bi];
  if (slot < 0 || (long long)slot >= n_slots) {
    if (t < DV) y[tv + t] = __builtin_nanf("");
    return;
  }
  float* St = S + ((long long)slot * H + h) * DK * DV;
  f32x4 x[16];
#pragma unroll
  for (int m = 0; m < 16; ++m)
    x[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(St + (r0 + m) * DV + j0));
  if (t < DK) {
    const float g = kind == SQ_KIND_GDN ? gate[tile] : gate[tk + t];
    const float kk = k[tk + t];
    kd[t] = kk * g;
    bk[t] = beta[tile] * kk;
    qq[t] = q[tk + t];
    gg[t] = g;
  }
  __syncthreads();
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const float kk = kd[r0 + m];
    a.x = fmaf(kk, x[m].x, a.x);
    a.y = fmaf(kk, x[m].y, a.y);
    a.z = fmaf(kk, x[m].z, a.z);
    a.w = fmaf(kk, x[m].w, a.w);
  }
  col[rb][p] = a;
  __syncthreads();
  float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < NRB; ++r) {
    const float4 c = col[r][p];
    d.x += c.x;
    d.y += c.y;
    d.z += c.z;
    d.w += c.w;
  }
  const float4 vv = *reinterpret_cast<const float4*>(v + tv + j0);
  const float4 e = make_float4(vv.x - d.x, vv.y - d.y, vv.z - d.z, vv.w - d.w);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int i = r0 + m;
    const float g = gg[i], b = bk[i], qv = qq[i];
    f32x4 n;
    n.x = fmaf(g, x[m].x, b * e.x);
    n.y = fmaf(g, x[m].y, b * e.y);
    n.z = fmaf(g, x[m].z, b * e.z);
    n.w = fmaf(g, x[m].w, b * e.w);
    o.x = fmaf(qv, n.x, o.x);
    o.y = fmaf(qv, n.y, o.y);
    o.z = fmaf(qv, n.z, o.z);
    o.w = fmaf(qv, n.w, o.w);
    __builtin_nontemporal_store(n, reinterpret_cast<f32x4*>(St + i * DV + j0));
  }
  __syncthreads();
  col[rb][p] = o;
  __syncthreads();
  if (rb == 0) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const float4 c = col[r][p];
      s.x += c.x;
      s.y += c.y;
      s.z += c.z;
      s.w += c.w;
    }
    *reinterpret_cast<float4*>(y + tv + j0) = s;
  }
}

// Prefill of one chunk: T tokens of the recurrence per (sequence, head) tile
// with the state held in registers for the whole chunk (the prefill step of
// the serving flow, "unpack active states, run the chunk kernel, pack
// boundary states", STEPQuant App. F.1).  Inputs are [B][T][H][...]; the
// output y_t of every token is written; the final state replaces S.  Row
// constants of token s (g_i, beta k_i, q_i, g_i k_i) are staged three tokens
// ahead in LDS, and the update of token s also forms the key-retrieval
// partials of token s + 1, so one workgroup barrier per token suffices.
template <int DK, int DV>
__global__ __launch_bounds__((DK / 32) * (DV / 2)) void prefill_kernel(
    int kind, int H, int T, float* S, const float* q, const float* k, const float* v,
    const float* beta, const float* gate, float* y) {
  using G = Geo<DK, DV>;
  constexpr int NP = G::NP, NRB = G::NRB;
  __shared__ float4 rc[3][DK];                 // g, beta k, q, g k of a token's rows
  __shared__ float2 colD[2][NRB][NP], colY[2][NRB][NP];
  const int tile = blockIdx.x, bi = tile / H, h = tile - bi * H;
  const int t = threadIdx.x, rb = t / NP, p = t - rb * NP, j0 = 2 * p, r0 = 32 * rb;
  float* St = S + (long long)tile * DK * DV;
  const long long base = (long long)bi * T * H + h;   // token s of this tile: base + s H
  auto stage = [&](int s) {
    if (t < DK) {
      const long long th = base + (long long)s * H, tk = th * DK;
      const float g = kind == SQ_KIND_GDN ? gate[th] : gate[tk + t];
      const float kk = k[tk + t];
      rc[s % 3][t] = make_float4(g, beta[th] * kk, q[tk + t], g * kk);
    }
  };
  float x[64];
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const float2 v2 = *reinterpret_cast<const float2*>(St + (r0 + m) * DV + j0);
    x[2 * m] = v2.x;
    x[2 * m + 1] = v2.y;
  }
  stage(0);
  if (T > 1) stage(1);
  __syncthreads();
  {  // key retrieval partials of token 0
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const float w = rc[0][r0 + m].w;
      a0 = fmaf(w, x[2 * m], a0);
      a1 = fmaf(w, x[2 * m + 1], a1);
    }
    colD[0][rb][p] = make_float2(a0, a1);
  }
  __syncthreads();
  for (int s = 0; s < T; ++s) {
    // the buffer of token s + 2 last held token s - 1, read before the barrier
    if (s + 2 < T) stage(s + 2);
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      d0 += colD[s & 1][r][p].x;
      d1 += colD[s & 1][r][p].y;
    }
    if (s > 0 && rb == 0) {  // the previous token's output
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        o0 += colY[(s - 1) & 1][r][p].x;
        o1 += colY[(s - 1) & 1][r][p].y;
      }
      *reinterpret_cast<float2*>(y + (base + (long long)(s - 1) * H) * DV + j0) =
          make_float2(o0, o1);
    }
    const float2 vv = *reinterpret_cast<const float2*>(v + (base + (long long)s * H) * DV + j0);
    const float e0 = vv.x - d0, e1 = vv.y - d1;
    float y0 = 0.f, y1 = 0.f, n0 = 0.f, n1 = 0.f;
    const int cur = s % 3, nxt = (s + 1) % 3;
    if (s + 1 < T) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float4 c = rc[cur][r0 + m];
        const float wn = rc[nxt][r0 + m].w;
        const float v0 = fmaf(c.x, x[2 * m], c.y * e0);
        const float v1 = fmaf(c.x, x[2 * m + 1], c.y * e1);
        x[2 * m] = v0;
        x[2 * m + 1] = v1;
        y0 = fmaf(c.z, v0, y0);
        y1 = fmaf(c.z, v1, y1);
        n0 = fmaf(wn, v0, n0);
        n1 = fmaf(wn, v1, n1);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float4 c = rc[cur][r0 + m];
        const float v0 = fmaf(c.x, x[2 * m], c.y * e0);
        const float v1 = fmaf(c.x, x[2 * m + 1], c.y * e1);
        x[2 * m] = v0;
        x[2 * m + 1] = v1;
        y0 = fmaf(c.z, v0, y0);
        y1 = fmaf(c.z, v1, y1);
      }
    }
    colY[s & 1][rb][p] = make_float2(y0, y1);
    colD[(s + 1) & 1][rb][p] = make_float2(n0, n1);
    __syncthreads();
  }
  if (rb == 0) {
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      o0 += colY[(T - 1) & 1][r][p].x;
      o1 += colY[(T - 1) & 1][r][p].y;
    }
    *reinterpret_cast<float2*>(y + (base + (long long)(T - 1) * H) * DV + j0) = make_float2(o0, o1);
  }
#pragma unroll
  for (int m = 0; m < 32; ++m)
    *reinterpret_cast<float2*>(St + (r0 + m) * DV + j0) = make_float2(x[2 * m], x[2 * m + 1]);
}

template <int DK, int DV>
hipError_t launch_prefill(int kind, int H, int B, int T, float* S, const float* q, const float* k,
                          const float* v, const float* beta, const float* gate, float* y,
                          hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(B * H), dim3((DK / 32) * (DV / 2)), 0, s, kind,
                     H, T, S, q, k, v, beta, gate, y);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch(int kind, int H, float* S, long long n_slots, const int* slots, int B,
                  const float* q, const float* k, const float* v, const float* beta,
                  const float* gate, float* y, hipStream_t s) {
  hipLaunchKernelGGL((dense_kernel<DK, DV>), dim3(B * H), dim3((DK / 32) * (DV / 2)), 0, s, kind, H, S,
                     n_slots, slots, q, k, v, beta, gate, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_step(int kind, int H, int dk, int dv, float* S, long long n_slots,
                             const int* slots, int B, const float* q, const float* k,
                             const float* v, const float* beta, const float* gate, float* y,
                             hipStream_t s) {
  if (dk == 128 && dv == 128) return launch<128, 128>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 64) return launch<64, 64>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 128 && dv == 64) return launch<128, 64>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 128) return launch<64, 128>(kind, H, S, n_slots, slots, B, q, k, v, beta, gate, y, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_chunk(int kind, int H, int dk, int dv, int B, int T, float* S,
                                const float* q, const float* k, const float* v, const float* beta,
                                const float* gate, float* y, hipStream_t s) {
  if (dk == 128 && dv == 128) return launch_prefill<128, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 64) return launch_prefill<64, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 128 && dv == 64) return launch_prefill<128, 64>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  if (dk == 64 && dv == 128) return launch_prefill<64, 128>(kind, H, B, T, S, q, k, v, beta, gate, y, s);
  return hipErrorInvalidValue;
}
