// swa_api.cpp — the C ABI of libswa (declared in include/swa.h): argument
// validation on the host, then kernel launches on the caller's stream.  No
// HIP call is made before every argument has been checked.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/swa.h"
#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace {

using swa::RopeTab;
using swa::Shape;

size_t elem_size(int dtype) { return dtype == SWA_F32 ? 4 : 2; }

// Checks shared by every entry point; fills the kernel-side shape.
int check_params(const swa_params* p, Shape* sh) {
  if (!p) return SWA_ERR_NULL;
  if (p->dtype != SWA_BF16 && p->dtype != SWA_F32) return SWA_ERR_DTYPE;
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1) return SWA_ERR_SHAPE;
  if (p->n_q_heads % p->n_kv_heads != 0) return SWA_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return SWA_ERR_SHAPE;
  if (p->window < 1 || p->n_sink < 0 || p->n_sink > 4096) return SWA_ERR_SHAPE;
  if ((long long)p->n_sink + p->window > (1LL << 30)) return SWA_ERR_SHAPE;
  if (!(p->scale >= 0.f) || !isfinite(p->scale)) return SWA_ERR_SHAPE;
  if (!(p->rope_theta >= 0.f) || !isfinite(p->rope_theta)) return SWA_ERR_SHAPE;
  if (p->dilation < 0 || p->dilation > (1 << 20)) return SWA_ERR_SHAPE;
  if (sh) {
    sh->B = p->batch;
    sh->Hq = p->n_q_heads;
    sh->Hkv = p->n_kv_heads;
    sh->D = p->head_dim;
    sh->W = p->window;
    sh->n_sink = p->n_sink;
    sh->S = p->n_sink + p->window;
    sh->scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->head_dim));
    sh->scale_log2 = (float)((double)sh->scale * 1.4426950408889634);
    sh->rope = p->rope_theta > 0.f ? 1 : 0;
    sh->dil = p->dilation > 1 ? p->dilation : 1;
  }
  return SWA_OK;
}

RopeTab rope_table(const swa_params* p) {
  RopeTab rt;
  for (int k = 0; k < swa::kMaxPairs; ++k) rt.rev[k] = 0.0;
  if (p->rope_theta > 0.f)
    for (int k = 0; k < p->head_dim / 2; ++k)
      rt.rev[k] = pow((double)p->rope_theta, -2.0 * k / p->head_dim) / (2.0 * 3.14159265358979323846);
  return rt;
}

// The fast kernels (bf16, head_dim 128) take a group of 1, 2, 4 or 8 query
// heads per KV head, a dilated window only with 4, and address one
// sequence's cache with 32-bit byte offsets.
bool fast_path(const swa_params* p) {
  const long long seq_cache_bytes =
      (long long)(p->n_sink + p->window) * p->n_kv_heads * p->head_dim * 2;
  const int g = p->n_kv_heads > 0 ? p->n_q_heads / p->n_kv_heads : 0;
  const bool group = p->n_q_heads == g * p->n_kv_heads && (g == 1 || g == 2 || g == 4 || g == 8) &&
                     (g == 4 || p->dilation <= 1);
  return p->dtype == SWA_BF16 && p->head_dim == 128 && group && seq_cache_bytes < (1LL << 31);
}
bool fast_decode(const swa_params* p) { return fast_path(p); }

// The fast prefill kernel also addresses one sequence's chunk (Q, K, V, and
// a few tiles past its end) with 32-bit byte offsets.  A dilated window takes
// it without sinks and in fixed-length batches (varlen: dilated = false).
bool fast_prefill(const swa_params* p, int32_t chunk_len, bool varlen = false) {
  const long long seq_q_bytes = (long long)(chunk_len + 256) * p->n_q_heads * p->head_dim * 2;
  return fast_path(p) && seq_q_bytes < (1LL << 31) &&
         (p->dilation <= 1 || (!varlen && p->n_sink == 0));
}

int launched(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_LAUNCH; }

// Varlen batches: chunk_lens is a host array of batch lengths (each 0 ..
// 2^24, at least one token in all); the sequences are packed one after the
// other.  The total and the longest length are returned.
int check_lens(const swa_params* p, const int32_t* lens, long long* total, int* longest) {
  if (!lens) return SWA_ERR_NULL;
  long long t = 0;
  int mx = 0;
  for (int b = 0; b < p->batch; ++b) {
    if (lens[b] < 0 || lens[b] > (1 << 24)) return SWA_ERR_SHAPE;
    t += lens[b];
    if (lens[b] > mx) mx = lens[b];
  }
  if (t < 1 || t > (1LL << 30)) return SWA_ERR_SHAPE;
  *total = t;
  *longest = mx;
  return SWA_OK;
}

// Runs f(first sequence, VarTab, first row, longest length, group shape) for
// each run of at most kVarMax sequences that holds any token.
template <class F>
int for_var_groups(const Shape& sh, const int32_t* lens, long long total, F&& f) {
  long long row = 0;
  for (int g0 = 0; g0 < sh.B; g0 += swa::kVarMax) {
    swa::VarTab vt{};
    vt.n = sh.B - g0 < swa::kVarMax ? sh.B - g0 : swa::kVarMax;
    vt.total = (int)total;
    int mx = 0;
    for (int j = 0; j < vt.n; ++j) {
      vt.row_off[j + 1] = vt.row_off[j] + lens[g0 + j];
      if (lens[g0 + j] > mx) mx = lens[g0 + j];
    }
    if (vt.row_off[vt.n] > 0) {
      Shape gs = sh;
      gs.B = vt.n;
      if (f(g0, vt, row, mx, gs) != hipSuccess) return SWA_ERR_LAUNCH;
    }
    row += vt.row_off[vt.n];
  }
  return SWA_OK;
}

template <class T>
T* rows_at(T* p, long long rows, long long row_elems, size_t es) {
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return p ? (T*)((B*)p + rows * row_elems * (long long)es) : nullptr;
}

// Split-K decode (+ combine when there are several ranges); with fw the fast
// kernel also stores the new entry first.  Arguments are already checked.
int decode_launch(const swa_params* params, const Shape& sh, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* pos, void* out, float* lse,
                  void* workspace, const swa::FusedWrite* fw, hipStream_t stream) {
  const bool fast = fast_decode(params);
  const int n = fast ? swa::decode_splits_fast(sh) : swa::decode_splits(sh);
  const RopeTab rt = rope_table(params);
  const bool f32 = params->dtype == SWA_F32;
  float* part = static_cast<float*>(workspace);
  hipError_t e;
  if (fast) {
    e = swa::launch_decode_bf16_d128_g4(sh, rt, q, k_cache, v_cache, pos, part, n, out, lse, fw,
                                        nullptr, stream);
    if (n == 1) return launched(e);   // the kernel wrote out and lse
  } else {
    e = swa::launch_decode_generic(sh, rt, f32, q, k_cache, v_cache, pos, part, n, stream);
  }
  if (e != hipSuccess) return SWA_ERR_LAUNCH;
  return launched(swa::launch_decode_combine(sh, f32, part, n, out, lse, nullptr, stream));
}

// The decode launches of a mixed varlen step: the sequences of one token, at
// most kVarMax per launch.  f(map, sub-shape) for each.
template <class F>
int for_decode_groups(const Shape& sh, const int32_t* lens, long long total, F&& f) {
  swa::DecodeMap m{};
  m.lse_hs = (int)total;
  long long row = 0;
  for (int b = 0; b < sh.B; ++b) {
    if (lens[b] == 1) {
      m.seq[m.n] = b;
      m.row[m.n] = (int)row;
      ++m.n;
    }
    row += lens[b];
    if (m.n == swa::kVarMax || (b == sh.B - 1 && m.n > 0)) {
      Shape gs = sh;
      gs.B = m.n;
      const int st = f(m, gs);
      if (st != SWA_OK) return st;
      m.n = 0;
    }
  }
  return SWA_OK;
}

// Whether the sequences of more than one token among g0 .. g0+n-1 are one
// contiguous run [*j0, *j1) of a single length *len (*j0 == *j1: none).
bool equal_run(const int32_t* lens, int g0, int n, int* j0, int* j1, int* len) {
  *j0 = *j1 = -1;
  *len = 0;
  for (int j = 0; j < n; ++j) {
    const int l = lens[g0 + j];
    if (l <= 1) continue;
    if (*j0 < 0) {
      *j0 = j;
      *len = l;
    } else if (*j1 != j || l != *len) {
      return false;
    }
    *j1 = j + 1;
  }
  if (*j0 < 0) *j0 = *j1 = 0;
  return true;
}

// Whether every group of kVarMax sequences has its multi-token sequences in
// one equal-length run (the step's fixed-length path), and the largest run's
// LSE bytes ([run][Hq][len] floats) then.
bool equal_runs(const Shape& sh, const int32_t* lens, size_t* lse_bytes) {
  size_t mx = 0;
  for (int g0 = 0; g0 < sh.B; g0 += swa::kVarMax) {
    int j0, j1, len;
    if (!equal_run(lens, g0, std::min(swa::kVarMax, sh.B - g0), &j0, &j1, &len)) return false;
    const size_t b = (size_t)(j1 - j0) * sh.Hq * (size_t)len * sizeof(float);
    if (b > mx) mx = b;
  }
  *lse_bytes = mx;
  return true;
}

// Bytes of the decode partials of a varlen step's one-token sequences (the
// largest launch), rounded up to 256.
size_t step_part_bytes(const Shape& sh, const int32_t* lens, long long total) {
  size_t part = 0;
  for_decode_groups(sh, lens, total, [&](const swa::DecodeMap&, const Shape& gs) {
    const size_t need = (size_t)gs.B * gs.Hq * swa::decode_splits(gs) * (gs.D + 2) * sizeof(float);
    if (need > part) part = need;
    return SWA_OK;
  });
  return (part + 255) / 256 * 256;
}

// Bytes of the rotated keys of a varlen step, rounded up to 256.
size_t step_keys_bytes(const swa_params* p, long long total) {
  const size_t kb = (size_t)total * p->n_kv_heads * p->head_dim * elem_size(p->dtype);
  return (kb + 255) / 256 * 256;
}

}  // namespace

extern "C" {

int swa_cache_write(const swa_params* params, const void* k, const void* v,
                    const int32_t* start_pos, int32_t n_tok, void* k_cache, void* v_cache,
                    hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k || !v || !start_pos || !k_cache || !v_cache) return SWA_ERR_NULL;
  if (n_tok < 1) return SWA_ERR_SHAPE;
  if ((long long)sh.B * n_tok * sh.Hkv * (sh.D / 8) >= (1LL << 40)) return SWA_ERR_SHAPE;
  return launched(swa::launch_cache_write(sh, rope_table(params), params->dtype == SWA_F32, k, v,
                                          start_pos, n_tok, k_cache, v_cache, swa::kToCache,
                                          nullptr, stream));
}

size_t swa_prefill_workspace_bytes(const swa_params* params, int32_t chunk_len) {
  if (check_params(params, nullptr) != SWA_OK || chunk_len < 1) return 0;
  return (size_t)params->batch * chunk_len * params->n_kv_heads * params->head_dim *
         elem_size(params->dtype);
}

int swa_rope_keys(const swa_params* params, const void* k, const int32_t* start_pos,
                  int32_t n_tok, void* k_rot, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k || !start_pos || !k_rot) return SWA_ERR_NULL;
  if (n_tok < 1 || n_tok > (1 << 24)) return SWA_ERR_SHAPE;
  return launched(swa::launch_cache_write(sh, rope_table(params), params->dtype == SWA_F32, k,
                                          nullptr, start_pos, n_tok, k_rot, nullptr,
                                          swa::kToDense, nullptr, stream));
}

int swa_rope_keys_cache_write(const swa_params* params, const void* k, const void* v,
                              const int32_t* start_pos, int32_t n_tok, void* k_rot, void* k_cache,
                              void* v_cache, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k || !v || !start_pos || !k_rot || !k_cache || !v_cache) return SWA_ERR_NULL;
  if (n_tok < 1 || n_tok > (1 << 24)) return SWA_ERR_SHAPE;
  if ((long long)sh.B * n_tok * sh.Hkv * (sh.D / 8) >= (1LL << 40)) return SWA_ERR_SHAPE;
  return launched(swa::launch_cache_write(sh, rope_table(params), params->dtype == SWA_F32, k, v,
                                          start_pos, n_tok, k_rot, v_cache, swa::kToBoth, nullptr,
                                          stream, k_cache));
}

int swa_prefill_attention(const swa_params* params, const void* q, const void* k_rot,
                          const void* v, const void* k_cache, const void* v_cache,
                          const int32_t* start_pos, int32_t chunk_len, void* out, float* lse,
                          hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k_rot || !v || !start_pos || !out) return SWA_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return SWA_ERR_NULL;
  if (chunk_len < 1 || chunk_len > (1 << 24)) return SWA_ERR_SHAPE;
  const RopeTab rt = rope_table(params);
  hipError_t e;
  if (fast_prefill(params, chunk_len))
    e = swa::launch_prefill_bf16_d128_g4(sh, rt, q, k_rot, v, k_cache, v_cache, start_pos,
                                         chunk_len, out, lse, nullptr, stream);
  else
    e = swa::launch_prefill_generic(sh, rt, params->dtype == SWA_F32, q, k_rot, v, k_cache,
                                    v_cache, start_pos, chunk_len, out, lse, nullptr, stream);
  return launched(e);
}

int swa_prefill_chunk(const swa_params* params, const void* q, const void* k, const void* v,
                      const void* k_cache, const void* v_cache, const int32_t* start_pos,
                      int32_t chunk_len, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k || !v || !start_pos || !out) return SWA_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return SWA_ERR_NULL;
  if (chunk_len < 1 || chunk_len > (1 << 24)) return SWA_ERR_SHAPE;
  const size_t need = swa_prefill_workspace_bytes(params, chunk_len);
  if (!workspace || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  // rotated chunk keys -> workspace, then attention over them
  st = swa_rope_keys(params, k, start_pos, chunk_len, workspace, stream);
  if (st != SWA_OK) return st;
  return swa_prefill_attention(params, q, workspace, v, k_cache, v_cache, start_pos, chunk_len,
                               out, lse, stream);
}

int swa_prefill_chunk_aligned(const swa_params* params, const void* q, const void* k, const void* v,
                              const void* k_cache, const void* v_cache, const int32_t* start_pos,
                              int32_t chunk_len, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  // sinks, dilation or a shape off the fast kernel: the general path serves any start
  if (!fast_prefill(params, chunk_len) || sh.n_sink != 0 || sh.dil > 1)
    return swa_prefill_chunk(params, q, k, v, k_cache, v_cache, start_pos, chunk_len, out, lse,
                             workspace, workspace_bytes, stream);
  if (!q || !k || !v || !start_pos || !out) return SWA_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return SWA_ERR_NULL;
  if (chunk_len < 1 || chunk_len > (1 << 24)) return SWA_ERR_SHAPE;
  if (!workspace || workspace_bytes < swa_prefill_workspace_bytes(params, chunk_len))
    return SWA_ERR_WORKSPACE;
  const RopeTab rt = rope_table(params);
  hipError_t e = swa::launch_cache_write(sh, rt, false, k, nullptr, start_pos, chunk_len, workspace,
                                         nullptr, swa::kToDenseAligned, nullptr, stream);
  if (e == hipSuccess)
    e = swa::launch_prefill_bf16_d128_g4(sh, rt, q, workspace, v, k_cache, v_cache, start_pos, chunk_len,
                                         out, lse, nullptr, stream, true);
  return launched(e);
}

int swa_prefill_chunk_aligned_write_prev(const swa_params* params, const void* k_prev,
                                         const void* v_prev, const int32_t* start_prev, int32_t prev_len,
                                         const void* q, const void* k, const void* v, void* k_cache,
                                         void* v_cache, const int32_t* start_pos, int32_t chunk_len,
                                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k_prev || !v_prev || !start_prev || !q || !k || !v || !k_cache || !v_cache || !start_pos || !out)
    return SWA_ERR_NULL;
  if (prev_len < 1 || chunk_len < 1 || chunk_len > (1 << 24)) return SWA_ERR_SHAPE;
  if ((long long)sh.B * prev_len * sh.Hkv * (sh.D / 8) >= (1LL << 40)) return SWA_ERR_SHAPE;
  if (!workspace || workspace_bytes < swa_prefill_workspace_bytes(params, chunk_len))
    return SWA_ERR_WORKSPACE;
  // the general path: the two calls one after the other (every argument is
  // checked above, so the write is never left without its chunk)
  if (!fast_prefill(params, chunk_len) || sh.n_sink != 0 || sh.dil > 1) {
    st = swa_cache_write(params, k_prev, v_prev, start_prev, prev_len, k_cache, v_cache, stream);
    if (st != SWA_OK) return st;
    return swa_prefill_chunk_aligned(params, q, k, v, k_cache, v_cache, start_pos, chunk_len, out, lse,
                                     workspace, workspace_bytes, stream);
  }
  const RopeTab rt = rope_table(params);
  swa::WriteRotate j{};
  j.k_prev = k_prev;
  j.v_prev = v_prev;
  j.start_prev = start_prev;
  j.n_prev = prev_len;
  j.k_cache = k_cache;
  j.v_cache = v_cache;
  j.k = k;
  j.start = start_pos;
  j.n_tok = chunk_len;
  j.k_rot = workspace;
  hipError_t e = swa::launch_write_rotate(sh, rt, j, stream);
  if (e == hipSuccess)
    e = swa::launch_prefill_bf16_d128_g4(sh, rt, q, workspace, v, k_cache, v_cache, start_pos, chunk_len,
                                         out, lse, nullptr, stream, true);
  return launched(e);
}

size_t swa_decode_workspace_bytes(const swa_params* params) {
  Shape sh;
  if (check_params(params, &sh) != SWA_OK) return 0;
  const int n = swa::decode_splits(sh);
  return (size_t)sh.B * sh.Hq * n * (sh.D + 2) * sizeof(float);
}

int swa_decode(const swa_params* params, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* pos, void* out, float* lse, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k_cache || !v_cache || !pos || !out) return SWA_ERR_NULL;
  const size_t need = swa_decode_workspace_bytes(params);
  if (!workspace || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  return decode_launch(params, sh, q, k_cache, v_cache, pos, out, lse, workspace, nullptr, stream);
}

int swa_decode_step(const swa_params* params, const void* q, const void* k, const void* v,
                    void* k_cache, void* v_cache, const int32_t* pos, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k || !v || !k_cache || !v_cache || !pos || !out) return SWA_ERR_NULL;
  const size_t need = swa_decode_workspace_bytes(params);
  if (!workspace || workspace_bytes < need) return SWA_ERR_WORKSPACE;
  if (fast_decode(params)) {
    const swa::FusedWrite fw{k, v, k_cache, v_cache};
    return decode_launch(params, sh, q, k_cache, v_cache, pos, out, lse, workspace, &fw, stream);
  }
  // other shapes: the cache write, then the decode, on the same stream
  hipError_t e = swa::launch_cache_write(sh, rope_table(params), params->dtype == SWA_F32, k, v, pos,
                                         1, k_cache, v_cache, swa::kToCache, nullptr, stream);
  if (e != hipSuccess) return SWA_ERR_LAUNCH;
  return decode_launch(params, sh, q, k_cache, v_cache, pos, out, lse, workspace, nullptr, stream);
}

size_t swa_prefill_varlen_workspace_bytes(const swa_params* params, const int32_t* chunk_lens) {
  long long total;
  int longest;
  if (check_params(params, nullptr) != SWA_OK) return 0;
  if (check_lens(params, chunk_lens, &total, &longest) != SWA_OK) return 0;
  return (size_t)total * params->n_kv_heads * params->head_dim * elem_size(params->dtype);
}

int swa_rope_keys_varlen(const swa_params* params, const void* k, const int32_t* start_pos,
                         const int32_t* chunk_lens, void* k_rot, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k || !start_pos || !k_rot) return SWA_ERR_NULL;
  long long total;
  int longest;
  st = check_lens(params, chunk_lens, &total, &longest);
  if (st != SWA_OK) return st;
  const RopeTab rt = rope_table(params);
  const bool f32 = params->dtype == SWA_F32;
  const size_t es = elem_size(params->dtype);
  const long long kv_row = (long long)sh.Hkv * sh.D;
  return for_var_groups(sh, chunk_lens, total, [&](int g0, const swa::VarTab& vt, long long row, int mx,
                                                   const Shape& gs) {
    return swa::launch_cache_write(gs, rt, f32, rows_at(k, row, kv_row, es), nullptr, start_pos + g0,
                                   mx, rows_at(k_rot, row, kv_row, es), nullptr, swa::kToDense, &vt,
                                   stream);
  });
}

int swa_cache_write_varlen(const swa_params* params, const void* k, const void* v,
                           const int32_t* start_pos, const int32_t* chunk_lens, void* k_cache,
                           void* v_cache, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k || !v || !start_pos || !k_cache || !v_cache) return SWA_ERR_NULL;
  long long total;
  int longest;
  st = check_lens(params, chunk_lens, &total, &longest);
  if (st != SWA_OK) return st;
  const RopeTab rt = rope_table(params);
  const bool f32 = params->dtype == SWA_F32;
  const size_t es = elem_size(params->dtype);
  const long long kv_row = (long long)sh.Hkv * sh.D;
  return for_var_groups(sh, chunk_lens, total, [&](int g0, const swa::VarTab& vt, long long row, int mx,
                                                   const Shape& gs) {
    return swa::launch_cache_write(gs, rt, f32, rows_at(k, row, kv_row, es), rows_at(v, row, kv_row, es),
                                   start_pos + g0, mx, rows_at(k_cache, (long long)g0 * sh.S, kv_row, es),
                                   rows_at(v_cache, (long long)g0 * sh.S, kv_row, es), swa::kToCache,
                                   &vt, stream);
  });
}

int swa_prefill_attention_varlen(const swa_params* params, const void* q, const void* k_rot,
                                 const void* v, const void* k_cache, const void* v_cache,
                                 const int32_t* start_pos, const int32_t* chunk_lens, void* out,
                                 float* lse, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k_rot || !v || !start_pos || !out) return SWA_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return SWA_ERR_NULL;
  long long total;
  int longest;
  st = check_lens(params, chunk_lens, &total, &longest);
  if (st != SWA_OK) return st;
  const RopeTab rt = rope_table(params);
  const bool f32 = params->dtype == SWA_F32;
  const bool fast = fast_prefill(params, longest, true);
  const size_t es = elem_size(params->dtype);
  const long long kv_row = (long long)sh.Hkv * sh.D, q_row = (long long)sh.Hq * sh.D;
  return for_var_groups(sh, chunk_lens, total, [&](int g0, const swa::VarTab& vt, long long row, int mx,
                                                   const Shape& gs) {
    const void* qg = rows_at(q, row, q_row, es);
    const void* kg = rows_at(k_rot, row, kv_row, es);
    const void* vg = rows_at(v, row, kv_row, es);
    const void* kcg = rows_at(k_cache, (long long)g0 * sh.S, kv_row, es);
    const void* vcg = rows_at(v_cache, (long long)g0 * sh.S, kv_row, es);
    void* og = rows_at(out, row, q_row, es);
    float* lg = lse ? lse + row : nullptr;   // [Hq][total]: this run's columns
    if (fast)
      return swa::launch_prefill_bf16_d128_g4(gs, rt, qg, kg, vg, kcg, vcg, start_pos + g0, mx, og, lg,
                                              &vt, stream);
    return swa::launch_prefill_generic(gs, rt, f32, qg, kg, vg, kcg, vcg, start_pos + g0, mx, og, lg,
                                       &vt, stream);
  });
}

int swa_prefill_chunk_varlen(const swa_params* params, const void* q, const void* k, const void* v,
                             const void* k_cache, const void* v_cache, const int32_t* start_pos,
                             const int32_t* chunk_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k || !v || !start_pos || !out) return SWA_ERR_NULL;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return SWA_ERR_NULL;
  long long total;
  int longest;
  st = check_lens(params, chunk_lens, &total, &longest);
  if (st != SWA_OK) return st;
  if (!workspace || workspace_bytes < swa_prefill_varlen_workspace_bytes(params, chunk_lens))
    return SWA_ERR_WORKSPACE;
  st = swa_rope_keys_varlen(params, k, start_pos, chunk_lens, workspace, stream);
  if (st != SWA_OK) return st;
  return swa_prefill_attention_varlen(params, q, workspace, v, k_cache, v_cache, start_pos,
                                      chunk_lens, out, lse, stream);
}

size_t swa_step_varlen_workspace_bytes(const swa_params* params, const int32_t* chunk_lens) {
  Shape sh;
  long long total;
  int longest;
  if (check_params(params, &sh) != SWA_OK) return 0;
  if (check_lens(params, chunk_lens, &total, &longest) != SWA_OK) return 0;
  // the fixed-length path keeps each run's LSE [run][Hq][len] in a region of
  // its own after the decode partials, until the step's tail repacks it
  size_t run_lse = 0;
  if (!equal_runs(sh, chunk_lens, &run_lse)) run_lse = 0;
  return step_keys_bytes(params, total) + step_part_bytes(sh, chunk_lens, total) + run_lse;
}

int swa_step_varlen(const swa_params* params, const void* q, const void* k, const void* v,
                    void* k_cache, void* v_cache, const int32_t* start_pos,
                    const int32_t* chunk_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!q || !k || !v || !k_cache || !v_cache || !start_pos || !out) return SWA_ERR_NULL;
  long long total;
  int longest;
  st = check_lens(params, chunk_lens, &total, &longest);
  if (st != SWA_OK) return st;
  if (!workspace || workspace_bytes < swa_step_varlen_workspace_bytes(params, chunk_lens))
    return SWA_ERR_WORKSPACE;
  if (!fast_prefill(params, longest, true)) {
    // one path for every sequence: the prefill chunk, then the cache write
    st = swa_prefill_chunk_varlen(params, q, k, v, k_cache, v_cache, start_pos, chunk_lens, out, lse,
                                  workspace, workspace_bytes, stream);
    if (st != SWA_OK) return st;
    return swa_cache_write_varlen(params, k, v, start_pos, chunk_lens, k_cache, v_cache, stream);
  }
  const RopeTab rt = rope_table(params);
  const size_t es = elem_size(params->dtype);
  const long long kv_row = (long long)sh.Hkv * sh.D, q_row = (long long)sh.Hq * sh.D;
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + step_keys_bytes(params, total));
  float* run_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + step_part_bytes(sh, chunk_lens, total));
  // Chunks of one size (chunked prefill with a fixed chunk length): when in
  // every group of kVarMax sequences those of more than one token form one
  // contiguous run of a single length, each run takes the fixed-length
  // kernels (key rotation, attention, cache write) and the one-token
  // sequences the decode kernel that stores their new entries itself: the
  // launches of the separate fixed-length calls, in one call.
  size_t run_lse_bytes = 0;
  if (equal_runs(sh, chunk_lens, &run_lse_bytes) && sh.B <= swa::kVarMax) {
    // One group: the run's key rotation and attention, the one-token
    // sequences' decode (with its fused cache write), then one tail launch:
    // their combine, the run's LSE repack and the run's cache write (after
    // its attention; the decode touches other sequences' caches).
    int j0, j1, len;
    equal_run(chunk_lens, 0, sh.B, &j0, &j1, &len);
    long long r0 = 0;
    for (int j = 0; j < j0; ++j) r0 += chunk_lens[j];
    swa::StepTail tail{};
    if (j1 > j0) {
      Shape rs = sh;
      rs.B = j1 - j0;
      const int32_t* sp = start_pos + j0;
      const long long c0 = (long long)j0 * sh.S;
      void* kr = rows_at(workspace, r0, kv_row, es);
      hipError_t e = swa::launch_cache_write(rs, rt, false, rows_at(k, r0, kv_row, es), nullptr, sp, len,
                                             kr, nullptr, swa::kToDense, nullptr, stream);
      if (e == hipSuccess)
        e = swa::launch_prefill_bf16_d128_g4(rs, rt, rows_at(q, r0, q_row, es), kr, rows_at(v, r0, kv_row, es),
                                             rows_at((const void*)k_cache, c0, kv_row, es),
                                             rows_at((const void*)v_cache, c0, kv_row, es), sp, len,
                                             rows_at(out, r0, q_row, es), lse ? run_lse : nullptr, nullptr, stream);
      if (e != hipSuccess) return SWA_ERR_LAUNCH;
      if (lse) {
        tail.psrc = run_lse;
        tail.pdst = lse + r0;
        tail.pHq = sh.Hq;
        tail.pC = len;
        tail.pn = rs.B * sh.Hq * len;
        tail.ptotal = total;
      }
      tail.wsh = rs;
      tail.rt = rt;
      tail.k = rows_at(k, r0, kv_row, es);
      tail.v = rows_at(v, r0, kv_row, es);
      tail.start = sp;
      tail.n_tok = len;
      tail.kc = rows_at(k_cache, c0, kv_row, es);
      tail.vc = rows_at(v_cache, c0, kv_row, es);
    } else {
      tail.wsh.B = 0;
    }
    const swa::FusedWrite fw{k, v, k_cache, v_cache};
    st = for_decode_groups(sh, chunk_lens, total, [&](const swa::DecodeMap& m, const Shape& gs) {
      const int n = swa::decode_splits_fast(gs);
      hipError_t e = swa::launch_decode_bf16_d128_g4(gs, rt, q, k_cache, v_cache, start_pos, part, n, out,
                                                     lse, &fw, &m, stream);
      if (n > 1) {   // (one split writes out and lse itself)
        tail.csh = gs;
        tail.part = part;
        tail.n_splits = n;
        tail.out = out;
        tail.lse = lse;
        tail.map = m;
      }
      return launched(e);
    });
    if (st != SWA_OK) return st;
    return launched(swa::launch_step_tail(tail, stream));
  }
  if (equal_runs(sh, chunk_lens, &run_lse_bytes)) {
    long long row = 0;   // packed row of sequence g0
    for (int g0 = 0; g0 < sh.B; g0 += swa::kVarMax) {
      const int n = std::min(swa::kVarMax, sh.B - g0);
      int j0, j1, len;
      equal_run(chunk_lens, g0, n, &j0, &j1, &len);
      long long r0 = row;
      for (int j = 0; j < j0; ++j) r0 += chunk_lens[g0 + j];
      if (j1 > j0) {
        Shape rs = sh;
        rs.B = j1 - j0;
        const int32_t* sp = start_pos + g0 + j0;
        const long long c0 = (long long)(g0 + j0) * sh.S;
        void* kr = rows_at(workspace, r0, kv_row, es);
        hipError_t e = swa::launch_cache_write(rs, rt, false, rows_at(k, r0, kv_row, es), nullptr, sp, len,
                                               kr, nullptr, swa::kToDense, nullptr, stream);
        // the run's LSE [B][Hq][C] goes through the workspace into its packed columns
        float* lrun = lse ? run_lse : nullptr;
        if (e == hipSuccess)
          e = swa::launch_prefill_bf16_d128_g4(rs, rt, rows_at(q, r0, q_row, es), kr, rows_at(v, r0, kv_row, es),
                                               rows_at((const void*)k_cache, c0, kv_row, es),
                                               rows_at((const void*)v_cache, c0, kv_row, es), sp, len,
                                               rows_at(out, r0, q_row, es), lrun, nullptr, stream);
        if (e == hipSuccess && lse) e = swa::launch_lse_pack(run_lse, lse + r0, rs.B, sh.Hq, len, total, stream);
        if (e == hipSuccess)
          e = swa::launch_cache_write(rs, rt, false, rows_at(k, r0, kv_row, es), rows_at(v, r0, kv_row, es), sp,
                                      len, rows_at(k_cache, c0, kv_row, es), rows_at(v_cache, c0, kv_row, es),
                                      swa::kToCache, nullptr, stream);
        if (e != hipSuccess) return SWA_ERR_LAUNCH;
      }
      for (int j = 0; j < n; ++j) row += chunk_lens[g0 + j];
    }
    const swa::FusedWrite fw{k, v, k_cache, v_cache};
    return for_decode_groups(sh, chunk_lens, total, [&](const swa::DecodeMap& m, const Shape& gs) {
      const int n = swa::decode_splits_fast(gs);
      hipError_t e = swa::launch_decode_bf16_d128_g4(gs, rt, q, k_cache, v_cache, start_pos, part, n, out,
                                                     lse, &fw, &m, stream);
      if (e == hipSuccess && n > 1) e = swa::launch_decode_combine(gs, false, part, n, out, lse, &m, stream);
      return launched(e);
    });
  }
  // 1. every chunk's keys rotated into the workspace
  st = swa_rope_keys_varlen(params, k, start_pos, chunk_lens, workspace, stream);
  if (st != SWA_OK) return st;
  // 2. attention of the sequences of more than one token (they read the caches as they stand)
  st = for_var_groups(sh, chunk_lens, total, [&](int g0, swa::VarTab& vt, long long row, int mx,
                                                 const Shape& gs) {
    vt.skip_len1 = 1;
    return swa::launch_prefill_bf16_d128_g4(
        gs, rt, rows_at(q, row, q_row, es), rows_at((const void*)workspace, row, kv_row, es),
        rows_at(v, row, kv_row, es), rows_at((const void*)k_cache, (long long)g0 * sh.S, kv_row, es),
        rows_at((const void*)v_cache, (long long)g0 * sh.S, kv_row, es), start_pos + g0, mx,
        rows_at(out, row, q_row, es), lse ? lse + row : nullptr, &vt, stream);
  });
  if (st != SWA_OK) return st;
  // 3. every chunk into the rolling buffers
  st = swa_cache_write_varlen(params, k, v, start_pos, chunk_lens, k_cache, v_cache, stream);
  if (st != SWA_OK) return st;
  // 4. the one-token sequences through the decode kernel, which now finds
  //    their entries in the caches
  return for_decode_groups(sh, chunk_lens, total, [&](const swa::DecodeMap& m, const Shape& gs) {
    const int n = swa::decode_splits_fast(gs);
    hipError_t e = swa::launch_decode_bf16_d128_g4(gs, rt, q, k_cache, v_cache, start_pos, part, n, out,
                                                   lse, nullptr, &m, stream);
    if (e == hipSuccess && n > 1) e = swa::launch_decode_combine(gs, false, part, n, out, lse, &m, stream);
    return launched(e);
  });
}

const char* swa_status_string(int status) {
  switch (status) {
    case SWA_OK: return "SWA_OK";
    case SWA_ERR_NULL: return "SWA_ERR_NULL: a required pointer is NULL";
    case SWA_ERR_SHAPE: return "SWA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case SWA_ERR_DTYPE: return "SWA_ERR_DTYPE: unknown dtype";
    case SWA_ERR_UNSUPPORTED: return "SWA_ERR_UNSUPPORTED: not implemented for these arguments";
    case SWA_ERR_WORKSPACE: return "SWA_ERR_WORKSPACE: workspace missing or too small";
    case SWA_ERR_LAUNCH: return "SWA_ERR_LAUNCH: kernel launch failed";
    case SWA_ERR_SCRATCH: return "SWA_ERR_SCRATCH: needs more than the fixed scratch array";
    default: return "unknown swa_status";
  }
}

int swa_debug_slots(const swa_params* params, const int32_t* positions, int32_t n, int32_t* slots,
                    hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!positions || !slots) return SWA_ERR_NULL;
  if (n < 1) return SWA_ERR_SHAPE;
  return launched(swa::launch_debug_slots(sh, positions, n, slots, stream));
}

int swa_debug_mask(const swa_params* params, int32_t q_pos, const int32_t* k_pos, int32_t n,
                   uint8_t* mask, hipStream_t stream) {
  Shape sh;
  int st = check_params(params, &sh);
  if (st != SWA_OK) return st;
  if (!k_pos || !mask) return SWA_ERR_NULL;
  if (n < 1 || q_pos < 0) return SWA_ERR_SHAPE;
  return launched(swa::launch_debug_mask(sh, q_pos, k_pos, n, mask, stream));
}

}  // extern "C"
