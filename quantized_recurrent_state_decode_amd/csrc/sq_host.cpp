// Host side of the C ABI: plans, lifetime-aware calibration, argument checks
// and kernel dispatch.  No device memory is allocated here; the caller owns
// pools, plan tables, inputs and outputs.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "sq_internal.h"

// Device scratch of sq_calib_distortion_noalloc: the packed heads of one
// call.  Each GPU the library runs on holds its own copy until the process
// ends; every call on that GPU reuses it.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

#ifdef SQ_HOSTCHECK
void sq_check_failed(const char* cond, const char* file, int line) {
  std::fprintf(stderr, "SQ_CHECK failed: %s (%s:%d)\n", cond, file, line);
  std::fflush(stderr);
  std::abort();
}
#endif

namespace {

thread_local std::string g_err;

sq_status fail(sq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sq_status ok() {
  g_err.clear();
  return SQ_OK;
}

sq_status hip_fail(hipError_t e, const char* what) {
  return fail(SQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

long long round_up(long long n, long long a) { return (n + a - 1) / a * a; }

bool supported_dim(int d) { return d == 64 || d == 128; }
bool code_bits(int b) { return b == 2 || b == 4 || b == 6 || b == 8; }

// Bytes of one stored row of d_v values at width b (FP16 for pivots).
int row_bytes(int dv, int b) { return b == SQ_PIVOT_BITS ? 2 * dv : dv * b / 8; }

template <class T>
size_t put(std::vector<unsigned char>& img, const std::vector<T>& v) {
  size_t off = round_up((long long)img.size(), 16);
  img.resize(off + std::max<size_t>(v.size() * sizeof(T), 16), 0);
  if (!v.empty()) std::memcpy(img.data() + off, v.data(), v.size() * sizeof(T));
  return off;
}

// Per-head byte offsets, the device-table image and derived sizes.
void finish_plan(sq_plan* P) {
  const int H = P->H, dk = P->dk, dv = P->dv;
  P->head_off.assign(H, 0);
  P->r_off.assign(H, 0);
  P->c_off.assign(H, 0);
  long long off = 0, payload = 0, analytic = 0;
  int maxh = 0;
  for (int h = 0; h < H; ++h) {
    long long used = 0;
    if (P->mode == SQ_MODE_UNIFORM) {
      P->r_off[h] = dk * dv * P->ubits / 8;
      used = P->r_off[h] + 2LL * dk;
      analytic += used;
    } else if (P->mode == SQ_MODE_WINDOW) {
      const long long z = round_up(16 + 4LL * P->p, 128);
      used = z + (long long)dk * dv + 4LL * dk + 4LL * dv + 4LL * P->p * (dk + dv) +
             2LL * P->rank * (dk + dv);
      P->r_off[h] = (int)z;  // start of Z
      analytic += used;
    } else if (P->kind == SQ_KIND_GDN) {
      const int b = P->head_bits[h];
      if (b == SQ_PIVOT_BITS) {
        used = 2LL * dk * dv;
        analytic += used + 2LL * dk + 2LL * dv;  // scale slots kept in the analytic count
      } else {
        P->r_off[h] = dk * dv * b / 8;
        P->c_off[h] = P->r_off[h] + 2 * dk;
        used = P->c_off[h] + 2LL * dv;
        analytic += used;
      }
    } else {
      long long codes = 0;
      for (int s = 0; s < dk; ++s) {
        P->row_off[h * dk + s] = (int)codes;
        codes += row_bytes(dv, P->row_bits[h * dk + s]);
      }
      P->r_off[h] = (int)codes;
      P->c_off[h] = (int)codes + 2 * dk;
      P->max_code_bytes = std::max<int>(P->max_code_bytes, (int)codes);
      used = codes + 2LL * dk + 2LL * dv;
      analytic += used;
    }
    const long long padded = round_up(used, 256);
    // the head's arrays lie inside its bytes, its bytes inside the slot
    SQ_CHECK(used > 0 && used <= padded && padded % 256 == 0);
    SQ_CHECK(P->r_off[h] >= 0 && P->r_off[h] <= used && P->c_off[h] >= 0 && P->c_off[h] <= used);
    if (P->mode == SQ_MODE_STEP && P->kind == SQ_KIND_KDA) {
      for (int s = 0; s < dk; ++s)
        SQ_CHECK(P->row_off[h * dk + s] + row_bytes(dv, P->row_bits[h * dk + s]) <= P->r_off[h]);
      SQ_CHECK(P->c_off[h] + 2LL * dv == used);
    }
    P->head_off[h] = off;
    off += padded;
    payload += used;
    maxh = std::max<int>(maxh, (int)padded);
  }
  SQ_CHECK(off % 256 == 0 && maxh % 256 == 0);  // 16-byte accesses stay aligned in every slot
  P->slot_bytes = off;
  P->payload_bytes = payload;
  P->analytic_bytes = analytic;
  P->max_head_bytes = maxh;

  // heads grouped by code width for the per-width decode launches
  const int widths[5] = {2, 4, 6, 8, 16};
  P->cls_heads.clear();
  for (int c = 0; c < 5; ++c) {
    P->cls_start[c] = (int)P->cls_heads.size();
    for (int h = 0; h < H; ++h)
      if (P->head_bits[h] == widths[c]) P->cls_heads.push_back(h);
    P->cls_count[c] = (int)P->cls_heads.size() - P->cls_start[c];
  }
  std::vector<unsigned char>& img = P->image;
  img.clear();
  P->o_head_off = put(img, P->head_off);
  P->o_head_bits = put(img, P->head_bits);
  P->winv.resize(P->w.size());
  for (size_t i = 0; i < P->w.size(); ++i) P->winv[i] = 1.0f / P->w[i];
  P->o_w = put(img, P->w);
  P->o_winv = put(img, P->winv);
  P->o_row_key = put(img, P->row_key);
  P->o_row_bits = put(img, P->row_bits);
  P->o_row_off = put(img, P->row_off);
  P->o_r_off = put(img, P->r_off);
  P->o_c_off = put(img, P->c_off);
  P->o_cls = put(img, P->cls_heads);
  img.resize(round_up((long long)img.size(), 256), 0);
  // every table the kernels index lies inside the image, at its full length
  SQ_CHECK(P->o_head_off + H * sizeof(long long) <= img.size());
  SQ_CHECK(P->o_head_bits + H * sizeof(int) <= img.size());
  SQ_CHECK(P->o_w + P->w.size() * sizeof(float) <= img.size());
  SQ_CHECK(P->o_winv + P->winv.size() * sizeof(float) <= img.size());
  SQ_CHECK(P->o_row_key + P->row_key.size() * sizeof(int) <= img.size());
  SQ_CHECK(P->o_row_bits + P->row_bits.size() * sizeof(int) <= img.size());
  SQ_CHECK(P->o_row_off + P->row_off.size() * sizeof(int) <= img.size());
  SQ_CHECK(P->o_r_off + H * sizeof(int) <= img.size() && P->o_c_off + H * sizeof(int) <= img.size());
  SQ_CHECK(P->o_cls + P->cls_heads.size() * sizeof(int) <= img.size());
  SQ_CHECK(P->mode != SQ_MODE_STEP || P->kind != SQ_KIND_GDN || (int)P->cls_heads.size() == H);
}

DevPlan dev_view(const sq_plan* P, const void* dev) {
  const unsigned char* b = static_cast<const unsigned char*>(dev);
  DevPlan d;
  d.mode = P->mode;
  d.kind = P->kind;
  d.H = P->H;
  d.dk = P->dk;
  d.dv = P->dv;
  d.ubits = P->ubits;
  d.p = P->p;
  d.rank = P->rank;
  d.iters = P->iters;
  d.c_floor = P->c_floor;
  d.slot_bytes = P->slot_bytes;
  d.max_head_bytes = P->max_head_bytes;
  d.max_code_bytes = P->max_code_bytes;
  d.head_off = reinterpret_cast<const long long*>(b + P->o_head_off);
  d.head_bits = reinterpret_cast<const int*>(b + P->o_head_bits);
  d.w = reinterpret_cast<const float*>(b + P->o_w);
  d.winv = reinterpret_cast<const float*>(b + P->o_winv);
  d.row_key = reinterpret_cast<const int*>(b + P->o_row_key);
  d.row_bits = reinterpret_cast<const int*>(b + P->o_row_bits);
  d.row_off = reinterpret_cast<const int*>(b + P->o_row_off);
  d.r_off = reinterpret_cast<const int*>(b + P->o_r_off);
  d.c_off = reinterpret_cast<const int*>(b + P->o_c_off);
  d.cls_heads = reinterpret_cast<const int*>(b + P->o_cls);
  return d;
}

sq_status check_dims(int H, int dk, int dv) {
  if (H <= 0) return fail(SQ_EINVAL, "heads must be positive (got %d)", H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(SQ_EUNSUPPORTED, "d_k, d_v must be 64 or 128 (got %d, %d)", dk, dv);
  return SQ_OK;
}

// Optional host-side check of slot ids (needs a device-to-host copy).
sq_status validate_slots(const int32_t* slots, int B, long long n_slots, hipStream_t st) {
  const char* env = std::getenv("SQ_VALIDATE");
  if (!env || std::strcmp(env, "1") != 0) return SQ_OK;
  std::vector<int32_t> h(B);
  hipError_t e = hipMemcpyAsync(h.data(), slots, sizeof(int32_t) * B, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "copying slot ids");
  std::vector<int32_t> s(h);
  for (int i = 0; i < B; ++i)
    if (h[i] < 0 || h[i] >= n_slots)
      return fail(SQ_ESLOT_RANGE, "slot id %d at position %d outside [0, %lld)", h[i], i, n_slots);
  std::sort(s.begin(), s.end());
  for (int i = 1; i < B; ++i)
    if (s[i] == s[i - 1]) return fail(SQ_EDUP_SLOT, "slot id %d repeated in one call", s[i]);
  return SQ_OK;
}

// Tiles of a class above which it gets a launch of its own (16 rounds of
// 1024 resident 256-lane workgroups).
constexpr long long kSoloTiles = 16384;

// Decode arguments covering classes order[lo .. hi) of P.
TileArgs class_args(const sq_plan* P, const TileArgs& a, const int* order, int lo, int hi) {
  TileArgs b = a;
  b.n_cls = hi - lo;
  int end = 0;
  for (int i = 0; i < 5; ++i) {
    if (i < b.n_cls) {
      const int c = order[lo + i];
      b.cls_first[i] = P->cls_start[c];
      b.cls_n[i] = P->cls_count[c];
      b.cls_bits[i] = (const int[]){2, 4, 6, 8, 16}[c];
      end += a.B * P->cls_count[c];
    } else {
      b.cls_first[i] = 0;
      b.cls_n[i] = 1;
      b.cls_bits[i] = 0;
    }
    b.cls_end[i] = end;
  }
  b.n_tiles = end;
  // each class's heads are a range of the class table, and its tiles the
  // grid range [cls_end[i-1], cls_end[i]) of B rows per head
  SQ_CHECK(b.n_cls >= 1 && b.n_cls <= 5);
  for (int i = 0; i < b.n_cls; ++i) {
    SQ_CHECK(b.cls_n[i] > 0 && b.cls_first[i] >= 0);
    SQ_CHECK(b.cls_first[i] + b.cls_n[i] <= (int)P->cls_heads.size());
    SQ_CHECK(b.cls_end[i] - (i ? b.cls_end[i - 1] : 0) == a.B * b.cls_n[i]);
  }
  return b;
}

// row impact factors w = (omega / geomean_head(omega))^(gamma/2) with a relative
// floor ([SQ] App. B, C); a head whose omega are all zero gets w = 1
void impact_factors(int H, int dk, const double* omega, double gamma, double floor_rel, float* w) {
  for (int h = 0; h < H; ++h) {
    const double* om = omega + (size_t)h * dk;
    double mx = 0.0;
    for (int i = 0; i < dk; ++i) mx = std::max(mx, om[i]);
    if (mx <= 0.0) {
      for (int i = 0; i < dk; ++i) w[h * dk + i] = 1.0f;
      continue;
    }
    std::vector<double> f(dk);
    double lsum = 0.0;
    for (int i = 0; i < dk; ++i) {
      f[i] = std::max(om[i], floor_rel * mx);
      lsum += std::log(f[i]);
    }
    const double gm = std::exp(lsum / dk);
    for (int i = 0; i < dk; ++i) w[h * dk + i] = (float)std::pow(f[i] / gm, gamma / 2.0);
  }
}

hipError_t dispatch(const sq_plan* P, const TileArgs& a, hipStream_t st) {
  if (P->mode == SQ_MODE_WINDOW) return launch_tile_window(a, st);
  if (P->mode == SQ_MODE_STEP && P->kind == SQ_KIND_KDA) return launch_tile_kda(a, st);
  if (a.op != OP_DECODE || a.head_ids) return launch_tile_gdn(a, st);
  // decode by width class, largest first.  A class that fills the chip many
  // times over runs alone in its width-specialised kernel; the other classes
  // share one merged launch (one grid, so small classes do not each pay a
  // launch's latency).
  int order[5] = {0, 1, 2, 3, 4};
  std::stable_sort(order, order + 5, [&](int x, int y) { return P->cls_count[x] > P->cls_count[y]; });
  int n = 0;
  while (n < 5 && P->cls_count[order[n]]) ++n;
  SQ_CHECK(a.n_tiles == a.B * P->H);
  if (n == 1) return launch_decode_gdn(class_args(P, a, order, 0, 1), true, st);
  if ((long long)a.B * P->cls_count[order[0]] < kSoloTiles)
    return launch_decode_gdn(class_args(P, a, order, 0, n), false, st);
  if (P->mode == SQ_MODE_STEP) {
    // one split launch: the other classes' tiles in rows ahead of the largest
    // class's batch rows
    TileArgs b = class_args(P, a, order, 0, n);
    const int n0 = b.cls_n[0];
    b.pre_rows = (b.n_tiles - b.cls_end[0] + n0 - 1) / n0;
    // the leading rows hold every tile of the smaller classes, and every
    // class together is the whole batch
    SQ_CHECK((long long)b.pre_rows * n0 >= b.n_tiles - b.cls_end[0]);
    SQ_CHECK(b.n_tiles == a.n_tiles);
    if ((long long)b.B + b.pre_rows <= 65535) return launch_split_gdn(b, st);
  }
  hipError_t e = launch_decode_gdn(class_args(P, a, order, 0, 1), true, st);
  if (e != hipSuccess) return e;
  return launch_decode_gdn(class_args(P, a, order, 1, n), false, st);
}

TileArgs base_args(const sq_plan* P, const void* dev_plan, int op) {
  TileArgs a;
  std::memset(&a, 0, sizeof(a));
  a.P = dev_view(P, dev_plan);
  a.op = op;
  return a;
}

}  // namespace

// ------------------------------------------------------------------ plans
extern "C" sq_status sq_plan_create_uniform(int32_t heads, int32_t d_k, int32_t d_v,
                                            int32_t bits, sq_plan** out) {
  if (!out) return fail(SQ_EINVAL, "out is null");
  *out = nullptr;
  sq_status s = check_dims(heads, d_k, d_v);
  if (s) return s;
  if (!code_bits(bits)) return fail(SQ_EUNSUPPORTED, "uniform bits must be 2, 4, 6 or 8 (got %d)", bits);
  sq_plan* P = new (std::nothrow) sq_plan;
  if (!P) return fail(SQ_ENOMEM, "plan allocation");
  P->mode = SQ_MODE_UNIFORM;
  P->kind = SQ_KIND_GDN;
  P->H = heads;
  P->dk = d_k;
  P->dv = d_v;
  P->ubits = bits;
  P->head_bits.assign(heads, bits);
  finish_plan(P);
  *out = P;
  return ok();
}

extern "C" sq_status sq_plan_create_window_lowrank(int32_t heads, int32_t d_k, int32_t d_v,
                                                   int32_t p, float c_floor, int32_t rank,
                                                   int32_t power_iters, sq_plan** out) {
  if (!out) return fail(SQ_EINVAL, "out is null");
  *out = nullptr;
  sq_status s = check_dims(heads, d_k, d_v);
  if (s) return s;
  if (p < 1 || p > 32) return fail(SQ_EUNSUPPORTED, "window length must be in [1, 32] (got %d)", p);
  if (!(c_floor > 0.0f) || !std::isfinite(c_floor))
    return fail(SQ_EINVAL, "smoothing floor must be positive and finite");
  if (rank < 0 || rank > SQ_MAX_COMP_RANK)
    return fail(SQ_EUNSUPPORTED, "compensator rank must be in [0, %d] (got %d)", SQ_MAX_COMP_RANK,
                rank);
  if (rank > 0 && (power_iters < 1 || power_iters > SQ_MAX_POWER_ITERS))
    return fail(SQ_EUNSUPPORTED, "power iterations must be in [1, %d] (got %d)",
                SQ_MAX_POWER_ITERS, power_iters);
  // the kernel gives each compensator pair a lane after the record lanes of a
  // row block (16 or 32 of them) among its d_v / 2 lanes
  if (rank > 0 && (p <= 16 ? 16 : 32) + SQ_MAX_COMP_RANK > d_v / 2)
    return fail(SQ_EUNSUPPORTED, "compensators with a window longer than 16 need d_v = 128");
  sq_plan* P = new (std::nothrow) sq_plan;
  if (!P) return fail(SQ_ENOMEM, "plan allocation");
  P->mode = SQ_MODE_WINDOW;
  P->kind = SQ_KIND_GDN;
  P->H = heads;
  P->dk = d_k;
  P->dv = d_v;
  P->p = p;
  P->rank = rank;
  P->iters = rank > 0 ? power_iters : 0;
  P->c_floor = c_floor;
  P->head_bits.assign(heads, 8);
  finish_plan(P);
  *out = P;
  return ok();
}

extern "C" sq_status sq_plan_create_window(int32_t heads, int32_t d_k, int32_t d_v, int32_t p,
                                           float c_floor, sq_plan** out) {
  return sq_plan_create_window_lowrank(heads, d_k, d_v, p, c_floor, 0, 0, out);
}

extern "C" sq_status sq_plan_create_step(int32_t kind, int32_t heads, int32_t d_k, int32_t d_v,
                                         const int32_t* unit_bits, const float* w,
                                         sq_plan** out) {
  if (!out) return fail(SQ_EINVAL, "out is null");
  *out = nullptr;
  if (!unit_bits || !w) return fail(SQ_EINVAL, "unit_bits and w must be given");
  if (kind != SQ_KIND_GDN && kind != SQ_KIND_KDA) return fail(SQ_EINVAL, "bad kind %d", kind);
  sq_status s = check_dims(heads, d_k, d_v);
  if (s) return s;
  const int U = kind == SQ_KIND_GDN ? heads : heads * d_k;
  for (int u = 0; u < U; ++u)
    if (!code_bits(unit_bits[u]) && unit_bits[u] != SQ_PIVOT_BITS)
      return fail(SQ_EUNSUPPORTED, "unit %d: width %d not in {2,4,6,8,16}", u, unit_bits[u]);
  for (int i = 0; i < heads * d_k; ++i)
    if (!(w[i] > 0.0f) || !std::isfinite(w[i]))
      return fail(SQ_EINVAL, "impact factor %d must be positive and finite", i);
  sq_plan* P = new (std::nothrow) sq_plan;
  if (!P) return fail(SQ_ENOMEM, "plan allocation");
  P->mode = SQ_MODE_STEP;
  P->kind = kind;
  P->H = heads;
  P->dk = d_k;
  P->dv = d_v;
  P->n_units = U;
  P->unit_bits.assign(unit_bits, unit_bits + U);
  P->w.assign(w, w + heads * d_k);
  if (kind == SQ_KIND_GDN) {
    P->head_bits = P->unit_bits;
  } else {
    P->head_bits.assign(heads, 0);
    P->row_key.resize(heads * d_k);
    P->row_bits.resize(heads * d_k);
    P->row_off.resize(heads * d_k);
    for (int h = 0; h < heads; ++h) {
      std::vector<int> ord(d_k);
      std::iota(ord.begin(), ord.end(), 0);
      const int32_t* rb = unit_bits + h * d_k;
      std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return rb[a] < rb[b]; });
      for (int s2 = 0; s2 < d_k; ++s2) {
        P->row_key[h * d_k + s2] = ord[s2];
        P->row_bits[h * d_k + s2] = rb[ord[s2]];
      }
    }
  }
  finish_plan(P);
  *out = P;
  return ok();
}

extern "C" sq_status sq_calibrate_bits(const sq_calib_stats* st, const sq_calib_opts* op,
                                       sq_plan** out) {
  if (!out) return fail(SQ_EINVAL, "out is null");
  *out = nullptr;
  if (!st || !op) return fail(SQ_EINVAL, "stats and opts must be given");
  if (st->kind != SQ_KIND_GDN && st->kind != SQ_KIND_KDA) return fail(SQ_EINVAL, "bad kind");
  sq_status s = check_dims(st->heads, st->d_k, st->d_v);
  if (s) return s;
  if (st->n_cand < 1 || !st->cand_bits || !st->ell || !st->dist || !st->omega)
    return fail(SQ_EINVAL, "incomplete statistics");
  for (int c = 0; c < st->n_cand; ++c) {
    if (!code_bits(st->cand_bits[c])) return fail(SQ_EUNSUPPORTED, "candidate width %d", st->cand_bits[c]);
    if (c && st->cand_bits[c] <= st->cand_bits[c - 1]) return fail(SQ_EINVAL, "candidates must ascend");
  }
  if (op->horizon < 1 || !(op->pivot_frac >= 0.0 && op->pivot_frac <= 1.0) ||
      !std::isfinite(op->nominal_bits) || !std::isfinite(op->gamma) || !(op->omega_floor_rel >= 0))
    return fail(SQ_EINVAL, "bad calibration options");
  const int H = st->heads, dk = st->d_k, dv = st->d_v, nc = st->n_cand;
  const bool gdn = st->kind == SQ_KIND_GDN;
  const int U = gdn ? H : H * dk;
  const double n_unit = gdn ? (double)dk * dv : (double)dv;
  for (int u = 0; u < U; ++u) {
    if (!std::isfinite(st->ell[u])) return fail(SQ_ENONFINITE, "ell[%d] is not finite", u);
    for (int c = 0; c < nc; ++c)
      if (!std::isfinite(st->dist[u * nc + c])) return fail(SQ_ENONFINITE, "dist[%d][%d] is not finite", u, c);
  }
  for (int i = 0; i < H * dk; ++i)
    if (!std::isfinite(st->omega[i]) || st->omega[i] < 0)
      return fail(SQ_ENONFINITE, "omega[%d] must be finite and non-negative", i);

  // lifetime weights L_u = sum_{j<horizon} exp(2 j ell_u)   ([SQ] Sec. 4, Eq. 7)
  std::vector<double> L(U);
  for (int u = 0; u < U; ++u) {
    double acc = 0.0;
    for (int j = 0; j < op->horizon; ++j) acc += std::exp(2.0 * j * st->ell[u]);
    if (!std::isfinite(acc)) return fail(SQ_ENONFINITE, "lifetime weight of unit %d overflows", u);
    L[u] = acc;
  }
  // pivots: largest L_u d_u(b_max), ties to the lower index   ([SQ] Sec. 4, App. D)
  const int n_piv = (int)std::ceil(op->pivot_frac * U - 1e-12);
  std::vector<int> ord(U);
  std::iota(ord.begin(), ord.end(), 0);
  std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
    return L[a] * st->dist[a * nc + nc - 1] > L[b] * st->dist[b * nc + nc - 1];
  });
  std::vector<char> piv(U, 0);
  for (int i = 0; i < n_piv; ++i) piv[ord[i]] = 1;
  // greedy under the residual budget b_bar N - 8 N_piv   ([SQ] Eq. 8, App. D)
  double budget = op->nominal_bits * n_unit * U;
  double used = 0.0;
  std::vector<int> level(U, 0);
  for (int u = 0; u < U; ++u) {
    if (piv[u]) budget -= 8.0 * n_unit;
    else used += n_unit * st->cand_bits[0];
  }
  if (used > budget + 1e-9)
    return fail(SQ_EBUDGET, "budget %.1f bits below the smallest width (%.1f bits needed)", budget, used);
  for (;;) {
    int best = -1;
    double best_gain = 0.0;
    for (int u = 0; u < U; ++u) {
      if (piv[u] || level[u] + 1 >= nc) continue;
      const double cost = n_unit * (st->cand_bits[level[u] + 1] - st->cand_bits[level[u]]);
      if (used + cost > budget + 1e-9) continue;
      const double gain = L[u] * (st->dist[u * nc + level[u]] - st->dist[u * nc + level[u] + 1]) / cost;
      if (best < 0 || gain > best_gain) {
        best = u;
        best_gain = gain;
      }
    }
    if (best < 0) break;
    used += n_unit * (st->cand_bits[level[best] + 1] - st->cand_bits[level[best]]);
    ++level[best];
  }
  std::vector<int32_t> bits(U);
  for (int u = 0; u < U; ++u) bits[u] = piv[u] ? SQ_PIVOT_BITS : st->cand_bits[level[u]];

  std::vector<float> w(H * dk);
  impact_factors(H, dk, st->omega, op->gamma, op->omega_floor_rel, w.data());
  return sq_plan_create_step(st->kind, H, dk, dv, bits.data(), w.data(), out);
}

extern "C" sq_status sq_plan_query(const sq_plan* P, sq_plan_desc* d) {
  if (!P || !d) return fail(SQ_EINVAL, "plan and desc must be given");
  std::memset(d, 0, sizeof(*d));
  d->mode = P->mode;
  d->kind = P->kind;
  d->heads = P->H;
  d->d_k = P->dk;
  d->d_v = P->dv;
  d->uniform_bits = P->ubits;
  d->window = P->p;
  d->n_units = P->n_units;
  d->slot_bytes = P->slot_bytes;
  d->payload_bytes = P->payload_bytes;
  d->analytic_bytes = P->analytic_bytes;
  d->head_off = reinterpret_cast<const int64_t*>(P->head_off.data());
  d->unit_bits = P->unit_bits.empty() ? nullptr : P->unit_bits.data();
  d->w = P->w.empty() ? nullptr : P->w.data();
  d->window_c_floor = P->c_floor;
  d->window_rank = P->rank;
  d->window_iters = P->iters;
  return ok();
}

extern "C" sq_status sq_plan_destroy(sq_plan* P) {
  delete P;
  return ok();
}

extern "C" sq_status sq_plan_device_bytes(const sq_plan* P, size_t* bytes) {
  if (!P || !bytes) return fail(SQ_EINVAL, "plan and bytes must be given");
  *bytes = P->image.size();
  return ok();
}

extern "C" sq_status sq_plan_upload(const sq_plan* P, void* dev, hipStream_t st) {
  if (!P || !dev) return fail(SQ_EINVAL, "plan and device buffer must be given");
  if (reinterpret_cast<uintptr_t>(dev) % 256) return fail(SQ_EINVAL, "device plan buffer must be 256-byte aligned");
  hipError_t e = hipMemcpyAsync(dev, P->image.data(), P->image.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "uploading plan tables");
  return ok();
}

extern "C" sq_status sq_max_head_bytes(const sq_plan* P, size_t* bytes) {
  if (!P || !bytes) return fail(SQ_EINVAL, "plan and bytes must be given");
  *bytes = (size_t)P->max_head_bytes;
  return ok();
}

// ------------------------------------------------------------------ pools
extern "C" sq_status sq_pool_bytes(const sq_plan* P, int64_t n_slots, size_t* bytes) {
  if (!P || !bytes || n_slots < 0) return fail(SQ_EINVAL, "bad arguments");
  *bytes = (size_t)(P->slot_bytes * n_slots);
  return ok();
}

extern "C" sq_status sq_pool_init(const sq_plan* P, const void* dev_plan, void* pool,
                                  int64_t n_slots, hipStream_t st) {
  if (!P || !dev_plan || !pool || n_slots <= 0) return fail(SQ_EINVAL, "bad arguments");
  hipError_t e = hipMemsetAsync(pool, 0, (size_t)(P->slot_bytes * n_slots), st);
  if (e != hipSuccess) return hip_fail(e, "clearing pool");
  return ok();
}

extern "C" sq_status sq_pool_pack(const sq_plan* P, const void* dev_plan, void* pool,
                                  int64_t n_slots, const int32_t* slots, int32_t B,
                                  const float* S, hipStream_t st) {
  if (!P || !dev_plan || !pool || n_slots <= 0 || B < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_pool_pack");
  if (B == 0) return ok();  // the batch arrays may be null
  if (!slots || !S) return fail(SQ_EINVAL, "bad arguments to sq_pool_pack");
  sq_status s = validate_slots(slots, B, n_slots, st);
  if (s) return s;
  TileArgs a = base_args(P, dev_plan, OP_PACK);
  a.pool = static_cast<unsigned char*>(pool);
  a.n_slots = n_slots;
  a.slots = slots;
  a.B = B;
  a.X = S;
  a.n_tiles = B * P->H;
  hipError_t e = dispatch(P, a, st);
  if (e != hipSuccess) return hip_fail(e, "launching pack");
  return ok();
}

extern "C" sq_status sq_pool_unpack(const sq_plan* P, const void* dev_plan, const void* pool,
                                    int64_t n_slots, const int32_t* slots, int32_t B,
                                    float* S_out, hipStream_t st) {
  if (!P || !dev_plan || !pool || n_slots <= 0 || B < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_pool_unpack");
  if (B == 0) return ok();  // the batch arrays may be null
  if (!slots || !S_out) return fail(SQ_EINVAL, "bad arguments to sq_pool_unpack");
  sq_status s = validate_slots(slots, B, n_slots, st);
  if (s) return s;
  TileArgs a = base_args(P, dev_plan, OP_UNPACK);
  a.pool = static_cast<unsigned char*>(const_cast<void*>(pool));
  a.n_slots = n_slots;
  a.slots = slots;
  a.B = B;
  a.S_out = S_out;
  a.n_tiles = B * P->H;
  hipError_t e = dispatch(P, a, st);
  if (e != hipSuccess) return hip_fail(e, "launching unpack");
  return ok();
}

extern "C" sq_status sq_decode_step(const sq_plan* P, const void* dev_plan, void* pool,
                                    int64_t n_slots, const int32_t* slots, int32_t B,
                                    const float* q, const float* k, const float* v,
                                    const float* beta, const float* gate, float* y,
                                    hipStream_t st) {
  if (!P || !dev_plan || !pool || n_slots <= 0 || B < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_decode_step");
  if (B == 0) return ok();  // the batch arrays may be null
  if (!slots || !q || !k || !v || !beta || !gate || !y)
    return fail(SQ_EINVAL, "bad arguments to sq_decode_step");
  sq_status s = validate_slots(slots, B, n_slots, st);
  if (s) return s;
  TileArgs a = base_args(P, dev_plan, OP_DECODE);
  a.pool = static_cast<unsigned char*>(pool);
  a.n_slots = n_slots;
  a.slots = slots;
  a.B = B;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.gate = gate;
  a.y = y;
  a.n_tiles = B * P->H;
  hipError_t e = dispatch(P, a, st);
  if (e != hipSuccess) return hip_fail(e, "launching decode step");
  return ok();
}

extern "C" sq_status sq_window_flush(const sq_plan* P, const void* dev_plan, void* pool,
                                     int64_t n_slots, const int32_t* slots, int32_t B,
                                     hipStream_t st) {
  if (!P || !dev_plan || !pool || n_slots <= 0 || B < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_window_flush");
  if (P->mode != SQ_MODE_WINDOW) return fail(SQ_EPLAN_MISMATCH, "sq_window_flush needs a window plan");
  if (B == 0) return ok();  // the slot array may be null
  if (!slots) return fail(SQ_EINVAL, "bad arguments to sq_window_flush");
  sq_status s = validate_slots(slots, B, n_slots, st);
  if (s) return s;
  TileArgs a = base_args(P, dev_plan, OP_FLUSH);
  a.pool = static_cast<unsigned char*>(pool);
  a.n_slots = n_slots;
  a.slots = slots;
  a.B = B;
  a.n_tiles = B * P->H;
  hipError_t e = launch_tile_window(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching window flush");
  return ok();
}

extern "C" sq_status sq_quantize_tiles(const sq_plan* P, const void* dev_plan, const float* X,
                                       int32_t n_tiles, const int32_t* head_ids, void* out,
                                       hipStream_t st) {
  if (!P || !dev_plan || n_tiles < 0) return fail(SQ_EINVAL, "bad arguments to sq_quantize_tiles");
  if (n_tiles == 0) return ok();  // the tile arrays may be null
  if (!X || !head_ids || !out) return fail(SQ_EINVAL, "bad arguments to sq_quantize_tiles");
  TileArgs a = base_args(P, dev_plan, OP_PACK);
  a.X = X;
  a.head_ids = head_ids;
  a.out = static_cast<unsigned char*>(out);
  a.out_stride = P->max_head_bytes;
  a.n_tiles = n_tiles;
  hipError_t e = dispatch(P, a, st);
  if (e != hipSuccess) return hip_fail(e, "launching quantize-only");
  return ok();
}

extern "C" sq_status sq_impact_factors(int32_t heads, int32_t d_k, const double* omega,
                                       double gamma, double floor_rel, float* w) {
  if (!omega || !w || heads <= 0 || d_k <= 0 || !std::isfinite(gamma) || !(floor_rel >= 0))
    return fail(SQ_EINVAL, "bad arguments to sq_impact_factors");
  for (long long i = 0; i < (long long)heads * d_k; ++i)
    if (!std::isfinite(omega[i]) || omega[i] < 0)
      return fail(SQ_ENONFINITE, "omega[%lld] must be finite and non-negative", i);
  impact_factors(heads, d_k, omega, gamma, floor_rel, w);
  return ok();
}

extern "C" sq_status sq_calib_gate_stats(int32_t kind, int32_t heads, int32_t d_k, int32_t n,
                                         const float* q, const float* k, const float* beta,
                                         const float* gate, double* log_sum, double* omega_sum,
                                         hipStream_t st) {
  if (kind != SQ_KIND_GDN && kind != SQ_KIND_KDA) return fail(SQ_EINVAL, "bad kind %d", kind);
  if (heads <= 0 || n < 0 || !q || !k || !beta || !gate || !log_sum || !omega_sum)
    return fail(SQ_EINVAL, "bad arguments to sq_calib_gate_stats");
  if (!supported_dim(d_k)) return fail(SQ_EUNSUPPORTED, "d_k must be 64 or 128 (got %d)", d_k);
  if (n == 0) return ok();
  hipError_t e = launch_calib_gate(kind, heads, d_k, n, q, k, beta, gate, log_sum, omega_sum, st);
  if (e != hipSuccess) return hip_fail(e, "launching calibration gate statistics");
  return ok();
}

extern "C" sq_status sq_calib_distortion(const sq_plan* P, const void* dev_plan, int32_t n,
                                         const float* S, void* packed, int32_t per_row,
                                         double* dist_sum, hipStream_t st) {
  if (!P || !dev_plan || !S || !packed || !dist_sum || n < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_calib_distortion");
  if (P->mode != SQ_MODE_STEP || P->kind != SQ_KIND_GDN)
    return fail(SQ_EPLAN_MISMATCH, "sq_calib_distortion needs a STEP plan of GDN heads");
  for (int h = 0; h < P->H; ++h)
    if (P->head_bits[h] == SQ_PIVOT_BITS)
      return fail(SQ_EPLAN_MISMATCH, "sq_calib_distortion needs integer heads (head %d is FP16)", h);
  if (n == 0) return ok();
  // the plan's own quantizer, quantize-only, tile t = (sequence t / H, head t % H)
  TileArgs a = base_args(P, dev_plan, OP_PACK);
  a.X = S;
  a.out = static_cast<unsigned char*>(packed);
  a.out_stride = P->max_head_bytes;
  a.n_tiles = n * P->H;
  hipError_t e = dispatch(P, a, st);
  if (e == hipSuccess)
    e = launch_calib_dist(a.P, a.n_tiles, a.out, a.out_stride, S, per_row ? 1 : 0, dist_sum, st);
  if (e != hipSuccess) return hip_fail(e, "launching calibration distortion");
  return ok();
}

namespace {

// Device address of `scratch` on the current GPU, looked up once per device
// with that device current (the array's host-side name is not a device
// address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sq_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "querying the current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(SQ_EINVAL, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "looking up the device scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace

extern "C" sq_status sq_calib_distortion_noalloc(const sq_plan* P, const void* dev_plan,
                                                 int32_t n, const float* S, int32_t per_row,
                                                 double* dist_sum, hipStream_t st) {
  if (!P || !dev_plan || !S || !dist_sum || n < 0)
    return fail(SQ_EINVAL, "bad arguments to sq_calib_distortion_noalloc");
  const size_t need = (size_t)n * (size_t)P->H * (size_t)P->max_head_bytes;
  if (need > kNoAllocScratchBytes)
    return fail(SQ_EINVAL,
                "sq_calib_distortion_noalloc needs n H max_head_bytes = %zu bytes of scratch; "
                "the limit is %zu (call it with fewer sequences)", need, kNoAllocScratchBytes);
  if (n == 0) return ok();
  void* ptr = nullptr;
  sq_status s = scratch_ptr(&ptr);
  if (s) return s;
  return sq_calib_distortion(P, dev_plan, n, S, ptr, per_row, dist_sum, st);
}

namespace {
// Shared argument checks of the two prefill forms; 1 = nothing to do.
sq_status prefill_args(const char* name, int32_t kind, int32_t H, int32_t dk, int32_t dv,
                       int32_t B, int32_t T, const float* S, const float* q, const float* k,
                       const float* v, const float* beta, const float* gate, const float* y,
                       bool* empty) {
  *empty = false;
  if (kind != SQ_KIND_GDN && kind != SQ_KIND_KDA) return fail(SQ_EINVAL, "bad kind %d", kind);
  sq_status s = check_dims(H, dk, dv);
  if (s) return s;
  if (B < 0 || T < 0) return fail(SQ_EINVAL, "bad arguments to %s", name);
  if (B == 0 || T == 0) {  // the arrays may be null
    *empty = true;
    return ok();
  }
  if (!S || !q || !k || !v || !beta || !gate || !y) return fail(SQ_EINVAL, "bad arguments to %s", name);
  if ((long long)B * H > 0x7fffffffLL)  // one workgroup per (sequence, head)
    return fail(SQ_EINVAL, "%s: batch x heads must stay below 2^31", name);
  return ok();
}
}  // namespace

extern "C" sq_status sq_prefill_chunk(int32_t kind, int32_t H, int32_t dk, int32_t dv,
                                      int32_t B, int32_t T, float* S, const float* q,
                                      const float* k, const float* v, const float* beta,
                                      const float* gate, float* y, hipStream_t st) {
  bool empty;
  sq_status s = prefill_args("sq_prefill_chunk", kind, H, dk, dv, B, T, S, q, k, v, beta, gate, y,
                             &empty);
  if (s || empty) return s;
  hipError_t e = launch_prefill_chunk(kind, H, dk, dv, B, T, S, q, k, v, beta, gate, y, st);
  if (e != hipSuccess) return hip_fail(e, "launching prefill chunk");
  return ok();
}

extern "C" sq_status sq_prefill_chunkwise(int32_t kind, int32_t H, int32_t dk, int32_t dv,
                                          int32_t B, int32_t T, float* S, const float* q,
                                          const float* k, const float* v, const float* beta,
                                          const float* gate, float* y, hipStream_t st) {
  bool empty;
  sq_status s = prefill_args("sq_prefill_chunkwise", kind, H, dk, dv, B, T, S, q, k, v, beta,
                             gate, y, &empty);
  if (s || empty) return s;
  hipError_t e = launch_prefill_chunkwise(kind, H, dk, dv, B, T, S, q, k, v, beta, gate, y, st);
  if (e != hipSuccess) return hip_fail(e, "launching chunkwise prefill");
  return ok();
}

extern "C" sq_status sq_dense_step(int32_t kind, int32_t H, int32_t dk, int32_t dv, float* S,
                                   int64_t n_slots, const int32_t* slots, int32_t B,
                                   const float* q, const float* k, const float* v,
                                   const float* beta, const float* gate, float* y,
                                   hipStream_t st) {
  if (kind != SQ_KIND_GDN && kind != SQ_KIND_KDA) return fail(SQ_EINVAL, "bad kind %d", kind);
  sq_status s = check_dims(H, dk, dv);
  if (s) return s;
  if (!S || n_slots <= 0 || B < 0) return fail(SQ_EINVAL, "bad arguments to sq_dense_step");
  if (B == 0) return ok();  // the batch arrays may be null
  if (!slots || !q || !k || !v || !beta || !gate || !y)
    return fail(SQ_EINVAL, "bad arguments to sq_dense_step");
  s = validate_slots(slots, B, n_slots, st);
  if (s) return s;
  hipError_t e = launch_dense_step(kind, H, dk, dv, S, n_slots, slots, B, q, k, v, beta, gate, y, st);
  if (e != hipSuccess) return hip_fail(e, "launching dense step");
  return ok();
}

extern "C" const char* sq_last_error(void) { return g_err.c_str(); }
