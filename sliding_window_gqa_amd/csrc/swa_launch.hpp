// swa_launch.hpp — host-side launchers implemented next to their kernels and
// called by the C ABI in swa_api.cpp after it has validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa_device.hpp"

namespace swa {

// Destination of a rotate-and-store launch.
enum WriteMode {
  kToCache = 0,  // rolling-buffer slots of k_cache / v_cache (survivors only)
  kToDense = 1,  // rotated K into a dense [B][n_tok][Hkv][D] buffer (V untouched)
  kToBoth = 2,   // both at once: every rotated key dense, survivors (k, v) into the caches
  kToDenseAligned = 3,   // kToDense for a chunk whose starts must be multiples of W: a
                         // sequence whose start is not gets NaN keys (see swa_prefill_chunk_aligned)
};

// Sequences of different chunk lengths, packed one after the other (rows of
// sequence j: row_off[j] .. row_off[j+1]-1), at most kVarMax per launch.
// With a VarTab the launchers below take n_tok / C as the longest length,
// sh.B as the number of sequences, and every pointer at the launch's first
// sequence; LSE rows are then [head][total] with total the row count of the
// whole packed batch.
constexpr int kVarMax = 64;
struct VarTab {
  int n;
  int total;
  int skip_len1;               // prefill: sequences of one token get no work items
  int row_off[kVarMax + 1];
  int item_off[kVarMax + 1];   // prefill work items, filled by the launcher
};

// kToBoth: kdst is the dense rotated-key buffer, vdst the value cache and
// kcache the key cache.
hipError_t launch_cache_write(const Shape& sh, const RopeTab& rt, bool f32, const void* k,
                              const void* v, const int32_t* start, int n_tok, void* kdst,
                              void* vdst, WriteMode mode, const VarTab* vt, hipStream_t st,
                              void* kcache = nullptr);

// kToCache of a previous chunk and kToDenseAligned of the next one in one
// launch (bf16, fixed length, both chunks of the same B sequences): the
// previous chunk's k_prev / v_prev [B][n_prev] from start_prev into the
// caches, the next chunk's rotated k [B][n_tok] from start into k_rot.  The
// launcher fills tpb, t_lo and nb_prev.
struct WriteRotate {
  const void* k_prev;
  const void* v_prev;
  const int32_t* start_prev;
  int n_prev;
  void* k_cache;
  void* v_cache;
  const void* k;
  const int32_t* start;
  int n_tok;
  void* k_rot;
  int tpb, t_lo, nb_prev;
};
hipError_t launch_write_rotate(const Shape& sh, const RopeTab& rt, WriteRotate j, hipStream_t st);

// LSE of a fixed-length batch [B][Hq][C] into its columns of a packed
// [Hq][total] array (dst = the batch's first column).
hipError_t launch_lse_pack(const float* src, float* dst, int B, int Hq, int C, long long total,
                           hipStream_t st);

// Fast bf16 prefill: head_dim 128, group size 4.
hipError_t launch_prefill_bf16_d128_g4(const Shape& sh, const RopeTab& rt, const void* q,
                                       const void* k_rot, const void* v, const void* kc,
                                       const void* vc, const int32_t* start, int C, void* out,
                                       float* lse, const VarTab* vt, hipStream_t st,
                                       bool aligned = false);
// aligned: every start is a multiple of W (fixed length, no sinks), so the
// rolling buffer holds positions start - W .. start - 1 in slot order.

// Generic prefill (float32 or bf16, head_dim 64 or 128, any group size).
hipError_t launch_prefill_generic(const Shape& sh, const RopeTab& rt, bool f32, const void* q,
                                  const void* k_rot, const void* v, const void* kc,
                                  const void* vc, const int32_t* start, int C, void* out,
                                  float* lse, const VarTab* vt, hipStream_t st);

// Split-K decode.  Partials: [B][Hq][n_splits][D + 2] float.  The fast
// kernel writes out and lse itself when n_splits == 1 (no combine pass).
// With a FusedWrite it first stores the new token's entry (raw k, v:
// [B][Hkv][D]) into k_cache / v_cache (the caches it reads) at slot(pos).
// A decode launch over some sequences of a varlen batch: work-group column
// z decodes sequence seq[z] (its position, its caches) whose token is row
// row[z] of the packed q / out; LSE is then [head][lse_hs].  n = 0: column
// z is sequence z and row z, LSE [B][Hq].
struct DecodeMap {
  int n;
  int lse_hs;
  int seq[kVarMax];
  int row[kVarMax];
};
struct FusedWrite {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
};

// The tail of a mixed step in one launch: the decode combine of the
// one-token sequences (map columns; csh.B = map.n), the run's LSE repack
// (pn elements of psrc [B][pHq][pC] into pdst [pHq][ptotal]) and the run's
// rolling-buffer write (wsh.B sequences of n_tok tokens at rows b * n_tok of
// k / v); a part with nothing to do has 0 sequences / elements.  The
// launcher fills the block counts.
struct StepTail {
  Shape csh;
  const float* part;
  int n_splits;
  void* out;
  float* lse;
  DecodeMap map;
  const float* psrc;
  float* pdst;
  int pHq, pC, pn;
  long long ptotal;
  Shape wsh;
  RopeTab rt;
  const void* k;
  const void* v;
  const int32_t* start;
  int n_tok;
  void* kc;
  void* vc;
  int nb_comb, nb_pack, nb_write, tpb, t_lo, bps;
};
hipError_t launch_step_tail(StepTail t, hipStream_t st);

int decode_splits(const Shape& sh);
// Splits of the fast decode kernel (a dilated window cuts its keys, fewer
// than the slots); never more than decode_splits(sh).
int decode_splits_fast(const Shape& sh);
hipError_t launch_decode_bf16_d128_g4(const Shape& sh, const RopeTab& rt, const void* q,
                                      const void* kc, const void* vc, const int32_t* pos,
                                      float* partial, int n_splits, void* out, float* lse,
                                      const FusedWrite* fw, const DecodeMap* map, hipStream_t st);
hipError_t launch_decode_generic(const Shape& sh, const RopeTab& rt, bool f32, const void* q,
                                 const void* kc, const void* vc, const int32_t* pos,
                                 float* partial, int n_splits, hipStream_t st);
hipError_t launch_decode_combine(const Shape& sh, bool f32, const float* partial, int n_splits,
                                 void* out, float* lse, const DecodeMap* map, hipStream_t st);

hipError_t launch_debug_slots(const Shape& sh, const int32_t* pos, int n, int32_t* slots,
                              hipStream_t st);
hipError_t launch_debug_mask(const Shape& sh, int q_pos, const int32_t* k_pos, int n,
                             uint8_t* mask, hipStream_t st);

}  // namespace swa
