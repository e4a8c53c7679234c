// swa_write.hip — RoPE + rolling-buffer scatter.
//
// Digest page "Rolling Buffer KV Cache 동작 설명", 쓰기(write) 단계: position p
// is stored at slot p mod W, overwriting the oldest entry once p >= W;
// explainer How It Works 3.  RoPE (theta from the digest's "Methods" table)
// is applied to keys here, at their absolute position, so the cache holds
// rotated keys and values verbatim.
//
// The same pass serves the dense key rotation (every rotated key into a
// [B][n_tok] buffer) and, for a chunk whose attention reads no cache, both
// at once: the key is rotated once and stored densely and, if it survives,
// into its slot.
//
// Varlen batches (a VarTab) take each sequence's rows from its packed run and
// its own length, in one grid row of exactly the blocks the sequences need;
// the rule for survivors is the same per sequence.
//
// One thread moves 8 consecutive elements (one 16-byte bf16 chunk, or two
// 16-byte float chunks) of one (token, kv-head) row.  A block covers whole
// tokens of one sequence (blockIdx.y): thread x handles chunk x mod cpt of
// token x / cpt of the block's run of 256 / cpt tokens (cpt = chunks per
// token), or loops over the chunks of one token when cpt > 256, so the index
// arithmetic stays in 32 bits with one division per thread.  Only positions
// that survive the call are written: a rolling position p is overwritten
// inside the same call iff p + W <= last position, so each slot has exactly
// one writer.
#include <climits>

#include "swa_device.hpp"
#include "swa_launch.hpp"
#include "swa_passes.hpp"

namespace swa {
namespace {

// Rotated keys of a token whose sequence started off a multiple of W in an
// aligned chunk: NaN, so that every output of the sequence is NaN rather
// than silently wrong.  Chunks ct0, ct0 + stride, .. of token row `row`.
template <bool F32>
__device__ inline void store_nan_keys(int cpt, long long row, int ct0, int stride, void* kdst) {
  const long long e0 = row * cpt * 8;
  for (int ct = ct0; ct < cpt; ct += stride) {
    if (F32) {
      float4* d = reinterpret_cast<float4*>(static_cast<float*>(kdst) + e0 + 8 * ct);
      const float qn = __builtin_nanf("");
      d[0] = d[1] = make_float4(qn, qn, qn, qn);
    } else {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(kdst) + e0 + 8 * ct) =
          u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    }
  }
}

template <bool F32, bool VAR>
__global__ void __launch_bounds__(256) cache_write_kernel(Shape sh, RopeTab rt, const void* __restrict__ k,
                                                         const void* __restrict__ v,
                                                         const int32_t* __restrict__ start, int n_tok,
                                                         void* __restrict__ kdst, void* __restrict__ vdst,
                                                         int mode, int tok_per_block, int t_lo, VarTab vt,
                                                         void* __restrict__ kcache) {
  const int cpt = sh.Hkv * (sh.D / 8);   // 16-byte chunks per token
  int b, blk;
  if (VAR) {
    // one grid row: block L is block L - item_off[b] of sequence b, the
    // number of sequences whose blocks end at or before L (counted over
    // the lanes; every lane of the block is still active here)
    const int L = blockIdx.x;
    const int ln = (int)threadIdx.x & 63;
    const int io = ln < vt.n ? vt.item_off[ln + 1] : INT_MAX;
    b = __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(io <= L)));
    blk = L - vt.item_off[b];
  } else {
    b = blockIdx.y;
    blk = blockIdx.x;
  }
  // the sequence's rows: b * n_tok .. + n_tok, or its packed run
  const int len = VAR ? vt.row_off[b + 1] - vt.row_off[b] : n_tok;
  const long long srow = VAR ? (long long)vt.row_off[b] : (long long)b * n_tok;
  const int tb = (int)threadIdx.x / cpt;  // token of this thread within the block's run
  const int t = t_lo + blk * tok_per_block + tb;
  if (tb >= tok_per_block || t >= len) return;
  const int s0 = start[b];
  if (mode == kToDenseAligned) {
    if (s0 % sh.W != 0) {   // the start breaks the caller's promise
      store_nan_keys<F32>(cpt, srow + t, (int)threadIdx.x - tb * cpt, (int)blockDim.x, kdst);
      return;
    }
    mode = kToDense;
  }
  rotate_store_token<F32>(sh, rt, k, v, b, srow, t, s0, s0 + len - 1, (int)threadIdx.x - tb * cpt,
                          (int)blockDim.x, kdst, vdst, mode, kcache);
}

// A chunk boundary of an aligned chunked prefill in one launch (bf16, fixed
// length): blocks [0, nb_prev) of grid row b store the previous chunk's
// surviving tokens into sequence b's rolling buffer (kToCache), the others
// rotate the next chunk's keys into the dense buffer (kToDenseAligned).  The
// two jobs write disjoint memory and read only their own inputs, so the
// result is that of the two passes one after the other.
__global__ void __launch_bounds__(256) write_rotate_kernel(Shape sh, RopeTab rt, WriteRotate j) {
  const int cpt = sh.Hkv * (sh.D / 8);
  const int b = blockIdx.y;
  const int tb = (int)threadIdx.x / cpt;
  const int ct0 = (int)threadIdx.x - tb * cpt;
  if (tb >= j.tpb) return;
  int blk = blockIdx.x;
  if (blk < j.nb_prev) {
    const int t = j.t_lo + blk * j.tpb + tb;
    if (t >= j.n_prev) return;
    const int s0 = j.start_prev[b];
    rotate_store_token<false>(sh, rt, j.k_prev, j.v_prev, b, (long long)b * j.n_prev, t, s0,
                              s0 + j.n_prev - 1, ct0, (int)blockDim.x, j.k_cache, j.v_cache, kToCache,
                              nullptr);
    return;
  }
  blk -= j.nb_prev;
  const int t = blk * j.tpb + tb;
  if (t >= j.n_tok) return;
  const int s0 = j.start[b];
  if (s0 % sh.W != 0) {
    store_nan_keys<false>(cpt, (long long)b * j.n_tok + t, ct0, (int)blockDim.x, j.k_rot);
    return;
  }
  rotate_store_token<false>(sh, rt, j.k, nullptr, b, (long long)b * j.n_tok, t, s0, s0 + j.n_tok - 1, ct0,
                            (int)blockDim.x, j.k_rot, nullptr, kToDense, nullptr);
}

// LSE rows of a fixed-length batch [B][Hq][C] into the columns of a packed
// [Hq][total] array: dst[h][b*C + t] = src[b][h][t] (dst points at the
// batch's first column).  One thread per element, in source order.
__global__ void __launch_bounds__(256) lse_pack_kernel(const float* src, float* dst, int Hq, int C,
                                                       long long total, int n) {
  const int e = blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= n) return;
  const int row = e / C, t = e - row * C;   // row = b * Hq + h
  const int b = row / Hq, h = row - b * Hq;
  dst[(long long)h * total + (long long)b * C + t] = src[e];
}

// The tail of a mixed step (swa_step_varlen with a run of equal chunks), in
// one launch of 128-thread blocks: the decode combine of the one-token
// sequences (blocks [0, nb_comb)), the run's LSE repack ([.., + nb_pack)) and
// the run's rolling-buffer write ([.., + nb_write)).  The three touch
// disjoint memory; each block does one job.
__global__ void __launch_bounds__(128) step_tail_kernel(StepTail t) {
  __shared__ float sm_m[kMaxSplits], sm_l[kMaxSplits], sm_f[kMaxSplits];
  int blk = blockIdx.x;
  if (blk < t.nb_comb) {
    combine_column<false>(t.csh, t.part, t.n_splits, t.out, t.lse, t.map, blk % t.csh.Hq, blk / t.csh.Hq,
                          (int)threadIdx.x, sm_m, sm_l, sm_f);
    return;
  }
  blk -= t.nb_comb;
  if (blk < t.nb_pack) {
    const int e = blk * 128 + (int)threadIdx.x;
    if (e < t.pn) {
      const int row = e / t.pC, c = e - row * t.pC;   // row = b * Hq + h
      const int b = row / t.pHq, h = row - b * t.pHq;
      t.pdst[(long long)h * t.ptotal + (long long)b * t.pC + c] = t.psrc[e];
    }
    return;
  }
  blk -= t.nb_pack;
  // the run's write: block blk covers tokens t_lo + tpb * (blk % bps) .. of sequence blk / bps
  const int cpt = t.wsh.Hkv * (t.wsh.D / 8);
  const int b = blk / t.bps, tb = (int)threadIdx.x / cpt;
  const int tok = t.t_lo + (blk - b * t.bps) * t.tpb + tb;
  if (b >= t.wsh.B || tb >= t.tpb || tok >= t.n_tok) return;
  const int s0 = t.start[b];
  rotate_store_token<false>(t.wsh, t.rt, t.k, t.v, b, (long long)b * t.n_tok, tok, s0, s0 + t.n_tok - 1,
                            (int)threadIdx.x - tb * cpt, 128, t.kc, t.vc, kToCache, nullptr);
}

}  // namespace

hipError_t launch_step_tail(StepTail t, hipStream_t st) {
  // combine: one block of D = 128 threads per (one-token sequence, query head)
  t.nb_comb = t.map.n > 0 ? t.map.n * t.csh.Hq : 0;
  if (t.nb_comb > 0 && (t.csh.D != 128 || t.n_splits < 2 || t.n_splits > kMaxSplits)) return hipErrorInvalidValue;
  t.nb_pack = t.pn > 0 ? (t.pn + 127) / 128 : 0;
  t.nb_write = 0;
  if (t.wsh.B > 0) {
    const int cpt = t.wsh.Hkv * (t.wsh.D / 8);
    if (cpt > 128) return hipErrorInvalidValue;
    t.tpb = 128 / cpt;
    // without sinks only the last W tokens of the run can survive it
    t.t_lo = (t.wsh.n_sink == 0 && t.n_tok > t.wsh.W) ? t.n_tok - t.wsh.W : 0;
    t.bps = (t.n_tok - t.t_lo + t.tpb - 1) / t.tpb;
    const long long nb = (long long)t.bps * t.wsh.B;
    if (nb > INT32_MAX / 2) return hipErrorInvalidValue;
    t.nb_write = (int)nb;
  }
  const long long total = (long long)t.nb_comb + t.nb_pack + t.nb_write;
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  step_tail_kernel<<<dim3((unsigned)total), dim3(128), 0, st>>>(t);
  return hipGetLastError();
}

hipError_t launch_write_rotate(const Shape& sh, const RopeTab& rt, WriteRotate j, hipStream_t st) {
  const int threads = 256;
  const int cpt = sh.Hkv * (sh.D / 8);
  j.tpb = cpt <= threads ? threads / cpt : 1;
  // as launch_cache_write: only the previous chunk's last W tokens can survive it
  j.t_lo = (sh.n_sink == 0 && j.n_prev > sh.W) ? j.n_prev - sh.W : 0;
  const long long bp = ((long long)(j.n_prev - j.t_lo) + j.tpb - 1) / j.tpb;
  const long long bn = ((long long)j.n_tok + j.tpb - 1) / j.tpb;
  if (j.n_prev < 1 || j.n_tok < 1 || bp + bn > INT32_MAX || sh.B > 65535) return hipErrorInvalidValue;
  j.nb_prev = (int)bp;
  write_rotate_kernel<<<dim3((unsigned)(bp + bn), (unsigned)sh.B), dim3(threads), 0, st>>>(sh, rt, j);
  return hipGetLastError();
}

hipError_t launch_lse_pack(const float* src, float* dst, int B, int Hq, int C, long long total,
                           hipStream_t st) {
  const long long n = (long long)B * Hq * C;
  if (n > INT32_MAX - 256 || B < 1 || Hq < 1 || C < 1) return hipErrorInvalidValue;
  lse_pack_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(src, dst, Hq, C, total, (int)n);
  return hipGetLastError();
}

hipError_t launch_cache_write(const Shape& sh, const RopeTab& rt, bool f32, const void* k,
                              const void* v, const int32_t* start, int n_tok, void* kdst,
                              void* vdst, WriteMode mode, const VarTab* vt, hipStream_t st,
                              void* kcache) {
  const int threads = 256;
  const int cpt = sh.Hkv * (sh.D / 8);
  const int tok_per_block = cpt <= threads ? threads / cpt : 1;
  // Without sinks only the last W tokens of a run can survive it, whatever
  // its start: the grid begins there (the per-token test stays exact).
  const int t_lo = (!vt && mode == kToCache && sh.n_sink == 0 && n_tok > sh.W) ? n_tok - sh.W : 0;
  long long bx = ((long long)(n_tok - t_lo) + tok_per_block - 1) / tok_per_block;
  if (bx > INT32_MAX || sh.B > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)bx, (unsigned)sh.B);
  VarTab t{};
  if (vt) {
    // varlen: exactly the blocks each sequence needs, numbered in sequence order
    t = *vt;
    t.item_off[0] = 0;
    for (int j = 0; j < t.n; ++j) {
      const long long len = t.row_off[j + 1] - t.row_off[j];
      const long long next = t.item_off[j] + (len + tok_per_block - 1) / tok_per_block;
      if (next > INT32_MAX) return hipErrorInvalidValue;
      t.item_off[j + 1] = (int)next;
    }
    if (t.item_off[t.n] == 0) return hipSuccess;
    grid = dim3((unsigned)t.item_off[t.n], 1u);
  }
  if (f32) {
    if (vt)
      cache_write_kernel<true, true><<<grid, dim3(threads), 0, st>>>(sh, rt, k, v, start, n_tok, kdst, vdst,
                                                                     (int)mode, tok_per_block, t_lo, t, kcache);
    else
      cache_write_kernel<true, false><<<grid, dim3(threads), 0, st>>>(sh, rt, k, v, start, n_tok, kdst, vdst,
                                                                      (int)mode, tok_per_block, t_lo, t, kcache);
  } else {
    if (vt)
      cache_write_kernel<false, true><<<grid, dim3(threads), 0, st>>>(sh, rt, k, v, start, n_tok, kdst, vdst,
                                                                      (int)mode, tok_per_block, t_lo, t, kcache);
    else
      cache_write_kernel<false, false><<<grid, dim3(threads), 0, st>>>(sh, rt, k, v, start, n_tok, kdst, vdst,
                                                                       (int)mode, tok_per_block, t_lo, t, kcache);
  }
  return hipGetLastError();
}

}  // namespace swa
