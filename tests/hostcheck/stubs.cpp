// Kernel launchers of the checked host build.  Each one checks the launch
// arguments its kernel grid relies on (tile counts against the batch and the
// plan, class ranges, grid limits) and then reports that there is no device,
// so the host logic of every entry point runs up to its launch and no kernel
// is ever started.
#include "sq_internal.h"

namespace {

void check_tiles(const TileArgs& a) {
  SQ_CHECK(a.n_tiles > 0);
  SQ_CHECK(a.P.H > 0 && (a.P.dk == 64 || a.P.dk == 128) && (a.P.dv == 64 || a.P.dv == 128));
  SQ_CHECK(a.P.head_off && a.P.r_off && a.P.c_off && a.P.head_bits);
  if (a.out) {  // quantize-only: one packed head per tile at a fixed stride
    SQ_CHECK(a.head_ids != nullptr && a.X != nullptr);
    SQ_CHECK(a.out_stride >= a.P.max_head_bytes && a.out_stride % 16 == 0);
  } else {
    SQ_CHECK(a.pool && a.slots && a.n_slots > 0 && a.B > 0);
    SQ_CHECK(a.n_tiles == a.B * a.P.H);
    SQ_CHECK(a.P.slot_bytes > 0 && a.P.slot_bytes % 256 == 0);
    SQ_CHECK(a.op != OP_DECODE || (a.q && a.k && a.v && a.beta && a.gate && a.y));
    SQ_CHECK(a.op != OP_PACK || a.X);
    SQ_CHECK(a.op != OP_UNPACK || a.S_out);
  }
}

}  // namespace

hipError_t launch_tile_gdn(const TileArgs& a, hipStream_t) {
  check_tiles(a);
  SQ_CHECK(a.P.mode == SQ_MODE_UNIFORM || (a.P.mode == SQ_MODE_STEP && a.P.kind == SQ_KIND_GDN));
  return hipErrorNoDevice;
}

hipError_t launch_decode_gdn(const TileArgs& a, bool solo, hipStream_t) {
  SQ_CHECK(a.op == OP_DECODE && a.slots && a.B > 0);
  SQ_CHECK(a.n_cls >= 1 && a.n_cls <= 5 && a.cls_end[a.n_cls - 1] == a.n_tiles);
  SQ_CHECK(!solo || a.n_cls == 1);
  SQ_CHECK(a.n_tiles % a.B == 0 && a.n_tiles <= a.B * a.P.H);
  return hipErrorNoDevice;
}

hipError_t launch_split_gdn(const TileArgs& a, hipStream_t) {
  SQ_CHECK(a.op == OP_DECODE && a.n_cls >= 2 && a.pre_rows >= 1);
  SQ_CHECK(a.n_tiles == a.B * a.P.H && a.cls_end[a.n_cls - 1] == a.n_tiles);
  SQ_CHECK((long long)a.B + a.pre_rows <= 65535 && a.cls_n[0] <= 65535);
  SQ_CHECK((long long)a.pre_rows * a.cls_n[0] >= a.n_tiles - a.cls_end[0]);
  return hipErrorNoDevice;
}

hipError_t launch_tile_kda(const TileArgs& a, hipStream_t) {
  check_tiles(a);
  SQ_CHECK(a.P.mode == SQ_MODE_STEP && a.P.kind == SQ_KIND_KDA);
  SQ_CHECK(a.P.max_code_bytes > 0 && a.P.row_key && a.P.row_bits && a.P.row_off);
  return hipErrorNoDevice;
}

hipError_t launch_tile_window(const TileArgs& a, hipStream_t) {
  check_tiles(a);
  SQ_CHECK(a.P.mode == SQ_MODE_WINDOW && a.P.p >= 1 && a.P.rank >= 0 && a.P.iters >= 0);
  return hipErrorNoDevice;
}

hipError_t launch_calib_gate(int kind, int H, int dk, int n, const float* q, const float* k,
                             const float* beta, const float* gate, double* log_sum,
                             double* om_sum, hipStream_t) {
  SQ_CHECK((kind == SQ_KIND_GDN || kind == SQ_KIND_KDA) && H > 0 && dk > 0 && n > 0);
  SQ_CHECK(q && k && beta && gate && log_sum && om_sum);
  return hipErrorNoDevice;
}

hipError_t launch_calib_dist(const DevPlan& P, int n_tiles, const unsigned char* packed,
                             long long stride, const float* S, int per_row, double* dist,
                             hipStream_t) {
  SQ_CHECK(n_tiles > 0 && packed && S && dist && stride >= P.max_head_bytes);
  (void)per_row;
  return hipErrorNoDevice;
}

hipError_t launch_prefill_chunk(int kind, int H, int dk, int dv, int B, int T, float* S,
                                const float* q, const float* k, const float* v, const float* beta,
                                const float* gate, float* y, hipStream_t) {
  SQ_CHECK((kind == SQ_KIND_GDN || kind == SQ_KIND_KDA) && H > 0 && B > 0 && T > 0);
  SQ_CHECK((dk == 64 || dk == 128) && (dv == 64 || dv == 128));
  SQ_CHECK(S && q && k && v && beta && gate && y);
  return hipErrorNoDevice;
}

hipError_t launch_prefill_chunkwise(int kind, int H, int dk, int dv, int B, int T, float* S,
                                    const float* q, const float* k, const float* v,
                                    const float* beta, const float* gate, float* y, hipStream_t) {
  SQ_CHECK((kind == SQ_KIND_GDN || kind == SQ_KIND_KDA) && H > 0 && B > 0 && T > 0);
  SQ_CHECK((dk == 64 || dk == 128) && (dv == 64 || dv == 128));
  SQ_CHECK(S && q && k && v && beta && gate && y);
  return hipErrorNoDevice;
}

hipError_t launch_dense_step(int kind, int H, int dk, int dv, float* S, long long n_slots,
                             const int* slots, int B, const float* q, const float* k,
                             const float* v, const float* beta, const float* gate, float* y,
                             hipStream_t) {
  SQ_CHECK((kind == SQ_KIND_GDN || kind == SQ_KIND_KDA) && H > 0 && B > 0 && n_slots > 0);
  SQ_CHECK((dk == 64 || dk == 128) && (dv == 64 || dv == 128));
  SQ_CHECK(S && slots && q && k && v && beta && gate && y);
  return hipErrorNoDevice;
}

// marks the checked build (the entry-point driver refuses any other library)
extern "C" int sq_hostcheck_build(void) { return 1; }
