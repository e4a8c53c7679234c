// swa_passes.hpp — device bodies of the small passes, shared by their own
// kernels and by the step's tail kernel (swa_write.hip), which runs several
// of them in one launch.
#pragma once

#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace swa {

// Key rotation / rolling-buffer store of one token (digest "Rolling Buffer KV
// Cache 동작 설명", 쓰기(write) 단계; RoPE from the digest's "Methods"):
// the thread handles the 16-byte chunks ct0, ct0 + stride, ... of token t of
// sequence b (row srow + t of k / v, position s0 + t, the call's last
// position `last`).  kToCache stores only a survivor (no later token of the
// call takes its slot) into its slot; kToDense stores the rotated key at the
// token's own row of kdst; kToBoth does that and, for a survivor, also stores
// k and v into the caches (kcache, vdst).
template <bool F32>
__device__ inline void rotate_store_token(const Shape& sh, const RopeTab& rt, const void* __restrict__ k,
                                          const void* __restrict__ v, int b, long long srow, int t, int s0,
                                          int last, int ct0, int stride, void* __restrict__ kdst,
                                          void* __restrict__ vdst, int mode, void* __restrict__ kcache) {
  const int cpr = sh.D / 8;       // chunks per (token, head) row: 8 or 16
  const int cpt = sh.Hkv * cpr;   // chunks per token
  const int p = s0 + t;
  const bool survives = p < sh.n_sink || p + sh.W > last;   // not overwritten later in this call
  if (mode == kToCache && !survives) return;
  const long long row0 = srow + t;                                              // source token row
  const long long crow0 = (long long)b * sh.S + slot_of(p, sh.W, sh.n_sink);    // its cache slot
  const long long drow0 = mode == kToCache ? crow0 : row0;
  const bool to_cache = mode == kToCache || (mode == kToBoth && survives);
  for (int ct = ct0; ct < cpt; ct += stride) {
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

// Decode combine of one (sequence z, query head h), thread d owning element
// d of D: the splits' maxima and sums come in with one load per split,
// spread over the block, and each split's weight 2^(m_s - m*) is formed
// once; the partial outputs are then loaded eight splits at a time, so that
// the block waits for memory a few times rather than once per split.  The
// sums run over the splits in ascending order.  sm_*: kMaxSplits floats of
// LDS each; every thread of the block calls it (it synchronises the block).
constexpr int kMaxSplits = 512;   // decode_splits() never exceeds it
template <bool F32>
__device__ inline void combine_column(const Shape& sh, const float* part, int n_splits, void* out, float* lse,
                                      const DecodeMap& map, int h, int z, int d, float* sm_m, float* sm_l,
                                      float* sm_f) {
  const int r = map.n ? map.row[z] : z;   // the token's row in out
  const int D = sh.D;
  const float* src = part + ((long long)z * sh.Hq + h) * n_splits * (D + 2);
  // up to 8 splits: the partial outputs go out with the maxima and sums,
  // one wait for memory instead of two
  float xp[8];
  const bool few = n_splits <= 8;
#pragma unroll
  for (int u = 0; u < 8; ++u) xp[u] = (few && u < n_splits) ? src[u * (D + 2) + d] : 0.f;
  for (int s = d; s < n_splits; s += D) {
    sm_m[s] = src[s * (D + 2) + D];
    sm_l[s] = src[s * (D + 2) + D + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, sm_m[s]);
  for (int s = d; s < n_splits; s += D) sm_f[s] = (sm_m[s] == -INFINITY) ? 0.f : exp2f(sm_m[s] - M);
  __syncthreads();
  float L = 0.f, O = 0.f;
  for (int s = 0; s < n_splits; ++s) L += sm_l[s] * sm_f[s];
  int s = 0;
  if (few) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < n_splits) O += xp[u] * sm_f[u];
    s = n_splits;
  }
  for (; s + 8 <= n_splits; s += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = src[(s + u) * (D + 2) + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) O += x[u] * sm_f[s + u];
  }
  for (; s < n_splits; ++s) O += src[s * (D + 2) + d] * sm_f[s];
  const float val = O / L;
  const long long off = ((long long)r * sh.Hq + h) * D + d;
  if (F32)
    static_cast<float*>(out)[off] = val;
  else
    static_cast<uint16_t*>(out)[off] = to_bf16_bits(val);
  if (lse && d == 0) {
    const long long lo = map.n ? (long long)h * map.lse_hs + r : (long long)r * sh.Hq + h;
    lse[lo] = (M + log2f(L)) * 0.69314718055994531f;
  }
}

}  // namespace swa
