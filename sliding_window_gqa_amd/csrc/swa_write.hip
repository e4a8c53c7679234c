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

namespace swa {
namespace {

template <bool F32, bool VAR>
__global__ void __launch_bounds__(256) cache_write_kernel(Shape sh, RopeTab rt, const void* __restrict__ k,
                                                         const void* __restrict__ v,
                                                         const int32_t* __restrict__ start, int n_tok,
                                                         void* __restrict__ kdst, void* __restrict__ vdst,
                                                         int mode, int tok_per_block, int t_lo, VarTab vt,
                                                         void* __restrict__ kcache) {
  const int cpr = sh.D / 8;           // chunks per (token, head) row: 8 or 16
  const int cpt = sh.Hkv * cpr;       // chunks per token
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
  const int last = s0 + len - 1;
  const int p = s0 + t;
  const bool survives = p < sh.n_sink || p + sh.W > last;   // not overwritten later in this call
  if (mode == kToCache && !survives) return;
  const long long row0 = srow + t;                                                  // source token row
  const long long crow0 = (long long)b * sh.S + slot_of(p, sh.W, sh.n_sink);        // its cache slot
  const long long drow0 = mode == kToCache ? crow0 : row0;
  const bool to_cache = mode == kToCache || (mode == kToBoth && survives);
  for (int ct = (int)threadIdx.x - tb * cpt; ct < cpt; ct += (int)blockDim.x) {
    const int h = ct / cpr, c = ct - h * cpr;
    const long long src_off = (row0 * sh.Hkv + h) * sh.D + 8 * c;
    const long long dst_off = (drow0 * sh.Hkv + h) * sh.D + 8 * c;
    const long long cst_off = (crow0 * sh.Hkv + h) * sh.D + 8 * c;   // the cache entry (v, and k in kToBoth)

    float x[8];
    if (F32) {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(k) + src_off);
      const float4 a = src[0], bb = src[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = bb.x; x[5] = bb.y; x[6] = bb.z; x[7] = bb.w;
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(k) + src_off);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(w[j]);
        x[2 * j + 1] = bf16_hi(w[j]);
      }
    }
    if (sh.rope) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float cs, sn;
        rope_cs(p, rt.rev[4 * c + j], cs, sn);
        rotate(x[2 * j], x[2 * j + 1], cs, sn);
      }
    }
    if (F32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(kdst) + dst_off);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
      if (mode == kToBoth && survives) {
        float4* kd = reinterpret_cast<float4*>(static_cast<float*>(kcache) + cst_off);
        kd[0] = make_float4(x[0], x[1], x[2], x[3]);
        kd[1] = make_float4(x[4], x[5], x[6], x[7]);
      }
      if (to_cache) {
        const float4* vs = reinterpret_cast<const float4*>(static_cast<const float*>(v) + src_off);
        float4* vd = reinterpret_cast<float4*>(static_cast<float*>(vdst) + cst_off);
        vd[0] = vs[0];
        vd[1] = vs[1];
      }
    } else {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = pack_bf16(x[2 * j], x[2 * j + 1]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(kdst) + dst_off) = w;
      if (mode == kToBoth && survives) *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(kcache) + cst_off) = w;
      if (to_cache) {
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(vdst) + cst_off) =
            *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(v) + src_off);
      }
    }
  }
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

}  // namespace

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
