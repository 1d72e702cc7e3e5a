// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "stepq.h"

// Host-side bounds asserts of the checked build (-DSQ_HOSTCHECK): the plan's
// byte layout, the device-table image and the launch arguments each kernel
// grid relies on.  A failed check prints the condition and aborts; in the
// normal build the checks compile to nothing.
#ifdef SQ_HOSTCHECK
[[noreturn]] void sq_check_failed(const char* cond, const char* file, int line);
#define SQ_CHECK(c) ((c) ? (void)0 : sq_check_failed(#c, __FILE__, __LINE__))
#else
#define SQ_CHECK(c) ((void)0)
#endif

// Device view of a plan: pointers into the caller-owned device table buffer.
struct DevPlan {
  int mode, kind, H, dk, dv, ubits, p;
  int rank, iters;            // window: compensator pairs, power iterations
  float c_floor;
  long long slot_bytes;
  int max_head_bytes;
  int max_code_bytes;         // KDA: largest code region of a head
  const long long* head_off;  // [H]
  const int* head_bits;       // [H] GDN/uniform width (16 = FP16 pivot head)
  const float* w;             // [H*dk] impact factors (STEP)
  const float* winv;          // [H*dk] 1 / w
  const int* row_key;         // [H*dk] KDA: key row held by storage row s
  const int* row_bits;        // [H*dk] KDA: width of storage row s
  const int* row_off;         // [H*dk] KDA: byte offset of storage row s in its head
  const int* r_off;           // [H] byte offset of the r (or s) array in the head
  const int* c_off;           // [H] byte offset of the c array in the head
  const int* cls_heads;       // [H] heads grouped by code width (2, 4, 6, 8, 16)
};

struct sq_plan {
  int mode = 0, kind = 0, H = 0, dk = 0, dv = 0, ubits = 0, p = 0;
  int rank = 0, iters = 0;
  float c_floor = 1e-6f;
  int n_units = 0;
  long long slot_bytes = 0, payload_bytes = 0, analytic_bytes = 0;
  int max_head_bytes = 0, max_code_bytes = 0;
  std::vector<long long> head_off;
  std::vector<int> head_bits, unit_bits, row_key, row_bits, row_off, r_off, c_off;
  std::vector<float> w, winv;
  // image of the device tables and the offsets of each array in it
  std::vector<unsigned char> image;
  std::vector<int> cls_heads;           // heads grouped by width
  int cls_start[5] = {0, 0, 0, 0, 0};   // per width class: first index in cls_heads
  int cls_count[5] = {0, 0, 0, 0, 0};   // per width class: number of heads
  size_t o_cls = 0;
  size_t o_head_off = 0, o_head_bits = 0, o_w = 0, o_winv = 0, o_row_key = 0, o_row_bits = 0,
         o_row_off = 0, o_r_off = 0, o_c_off = 0;
};

// Arguments of every tile kernel (one workgroup per (slot, head) tile).
enum { OP_DECODE = 0, OP_PACK = 1, OP_UNPACK = 2, OP_FLUSH = 3 };

struct TileArgs {
  DevPlan P;
  int op;
  unsigned char* pool;
  long long n_slots;
  const int* slots;          // [B] (null for quantize-only)
  int B;
  const float *q, *k, *v, *beta, *gate;
  float* y;                  // [B][H][dv]
  const float* X;            // pack: dense tiles [B*H][dk][dv]
  float* S_out;              // unpack: dense tiles [B*H][dk][dv]
  const int* head_ids;       // quantize-only: head of tile t (null otherwise)
  unsigned char* out;        // quantize-only: packed head t at out + t*out_stride
  long long out_stride;
  int n_tiles;
  // decode of STEP/uniform GDN: one launch over every width class.  Class i
  // (i < n_cls) holds heads cls_heads[cls_first[i] ..+ cls_n[i]) of width
  // cls_bits[i]; its tiles are blockIdx in [cls_end[i-1], cls_end[i]).
  int n_cls;
  int cls_first[5], cls_n[5], cls_bits[5], cls_end[5];
  // split launch (STEP GDN): grid rows of cls_n[0] workgroups ahead of class
  // 0's batch rows, which run the tiles of classes 1 .. n_cls-1
  int pre_rows;
};

// Kernel launchers (defined in the .hip files).
hipError_t launch_tile_gdn(const TileArgs& a, hipStream_t s);     // uniform + STEP GDN
// decode by width class: solo = class 0 alone in its width-specialised kernel,
// else every class of a in one merged launch
hipError_t launch_decode_gdn(const TileArgs& a, bool solo, hipStream_t s);
hipError_t launch_split_gdn(const TileArgs& a, hipStream_t s);
hipError_t launch_tile_kda(const TileArgs& a, hipStream_t s);     // STEP KDA
hipError_t launch_tile_window(const TileArgs& a, hipStream_t s);  // per-window variant
hipError_t launch_calib_gate(int kind, int H, int dk, int n, const float* q, const float* k,
                             const float* beta, const float* gate, double* log_sum,
                             double* om_sum, hipStream_t s);
hipError_t launch_calib_dist(const DevPlan& P, int n_tiles, const unsigned char* packed,
                             long long stride, const float* S, int per_row, double* dist,
                             hipStream_t s);
hipError_t launch_prefill_chunk(int kind, int H, int dk, int dv, int B, int T, float* S,
                                const float* q, const float* k, const float* v, const float* beta,
                                const float* gate, float* y, hipStream_t s);
hipError_t launch_prefill_chunkwise(int kind, int H, int dk, int dv, int B, int T, float* S,
                                    const float* q, const float* k, const float* v,
                                    const float* beta, const float* gate, float* y, hipStream_t s);
hipError_t launch_dense_step(int kind, int H, int dk, int dv, float* S, long long n_slots,
                             const int* slots, int B, const float* q, const float* k,
                             const float* v, const float* beta, const float* gate, float* y,
                             hipStream_t s);
