// swa_prefill.hip — attention of one prefill chunk.
//
// What is computed (essay §4.1 and Figure 3; explainer How It Works 4): the
// chunk's queries at positions s..s+C-1 attend causally to the chunk's own
// keys and, inside the sliding window, to the cache entries written before
// the chunk.  Keys j of query i: 0 <= j <= i and (i - W < j or j < n_sink).
// Attention is exact softmax attention evaluated block by block with a running
// max and sum (the FlashAttention-2 style block processing the digest page
// names as the basis of the SWA kernel, "Insights"/"핵심 주장").
//
// Fast kernel (bf16, head_dim 128, GQA group 4), MI355X / gfx950:
//  * One work-group = 64 query positions x the 4 query heads of one KV head
//    (256 query rows), 4 waves; wave w owns positions t0+16w .. t0+16w+15 for
//    all 4 heads, so the four 16-row query blocks of a wave share one mask.
//  * Key tiles of 64 keys.  K and V tiles are staged in LDS once per
//    work-group and used by all 4 heads (the GQA sharing of explainer How It
//    Works 1).  Tiles outside the band i-W < j <= i of the work-group are never
//    visited, so the work is O(N*W); a wave skips the matrix work of tiles
//    outside its own band and masks only the tiles that cut the diagonal or the
//    window edge.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16: in the
//    transposed form every lane owns one query column, so the softmax row
//    statistics stay in one lane plus a 4-lane exchange, and the score
//    accumulator is already the B operand of the PV product.
//  * V is transposed into LDS when it is stored, so every A operand of the PV
//    product is one 16-byte LDS read.
//  * Online softmax in the log2 domain; the output accumulator is rescaled
//    only when a running max grows by more than 2^8 (the result is the same:
//    numerator and denominator carry the same stale max).
//  * Work-groups are renumbered so that the 8 XCDs each take a contiguous
//    range of (sequence, KV head, query tile): the K/V of one KV head then
//    stays in one XCD's L2.  Query tiles run longest-first.
//
// Generic kernel: float32 or bf16, head_dim 64 or 128, any group size; one
// thread per query row, scalar loops.  Used for shapes the fast kernel does
// not cover (e.g. the float32 path).
#include <math.h>

#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace swa {
namespace {

constexpr int BM = 64;     // query positions per work-group
constexpr int BN = 64;     // keys per tile
constexpr int HD = 128;    // head_dim of the fast kernel
constexpr int KPITCH = 272;  // bytes per K row in LDS (256 + 16 pad)
constexpr int VPITCH = 144;  // bytes per V^T row in LDS (128 + 16 pad)
constexpr float kTau = 8.0f; // lazy-rescale threshold (log2 units)

__device__ inline float wave_max_g(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ inline float wave_sum_g(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

struct PrefillArgs {
  Shape sh;
  RopeTab rt;
  const uint16_t* q;
  const uint16_t* kr;   // rotated chunk keys [B][C][Hkv][128]
  const uint16_t* v;    // chunk values
  const uint16_t* kc;   // caches (may be null)
  const uint16_t* vc;
  const int32_t* start;
  int C;
  int n_qtiles;
  uint16_t* out;
  float* lse;
};

// Pointer to row `which` (0 = K, 1 = V) of the key at absolute position P for
// sequence b / kv head kvh, or null if that key does not exist.
__device__ inline const uint16_t* key_row(const PrefillArgs& a, int which, int b, int kvh, int s0,
                                          int P) {
  if (P < 0) return nullptr;
  const int u = P - s0;
  if (u >= 0) {
    if (u >= a.C) return nullptr;
    const uint16_t* base = which ? a.v : a.kr;
    return base + (((long long)b * a.C + u) * a.sh.Hkv + kvh) * HD;
  }
  const uint16_t* base = which ? a.vc : a.kc;
  if (!base) return nullptr;
  const int slot = slot_of(P, a.sh.W, a.sh.n_sink);
  return base + (((long long)b * a.sh.S + slot) * a.sh.Hkv + kvh) * HD;
}

__global__ void __launch_bounds__(256, 1) prefill_bf16_d128_g4_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BN * KPITCH + HD * VPITCH];
  uint8_t* Ks = smem;
  uint8_t* Vt = smem + BN * KPITCH;

  const Shape& sh = a.sh;
  // ---- work mapping: XCD-contiguous, longest tiles first ----
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, idx = wg >> 3, q8 = nwg >> 3, r8 = nwg & 7;
  const int L = xcd * q8 + min(xcd, r8) + idx;
  const int per_b = sh.Hkv * a.n_qtiles;
  const int b = L / per_b;
  const int rem = L - b * per_b;
  const int kvh = rem / a.n_qtiles;
  const int qt = a.n_qtiles - 1 - (rem - kvh * a.n_qtiles);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int s0 = a.start[b];
  const int C = a.C;
  const int t0 = qt * BM;
  const int q0w = t0 + 16 * w;   // first query of this wave (chunk-relative)
  const int tq = q0w + i;        // this lane's query
  const int h0 = kvh * 4;
  const int W = sh.W;

  // ---- Q prologue: rotated, rounded to bf16, in the B-operand layout ----
  // lane (i, g), step kk holds d = 8*(4kk+g) .. +7 of query tq, head h0+qb.
  bf16x8 qf[4][4];
  {
    float cs[4][4], sn[4][4];
    const int I = s0 + tq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (sh.rope) {
          rope_cs(I, a.rt.freq[4 * (4 * kk + g) + jj], cs[kk][jj], sn[kk][jj]);
        } else {
          cs[kk][jj] = 1.f;
          sn[kk][jj] = 0.f;
        }
      }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (tq < C)
          wv = *reinterpret_cast<const u32x4*>(
              a.q + (((long long)b * C + tq) * sh.Hq + h0 + qb) * HD + 8 * (4 * kk + g));
        u32x4 r;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float x0 = bf16_lo(wv[jj]), x1 = bf16_hi(wv[jj]);
          rotate(x0, x1, cs[kk][jj], sn[kk][jj]);
          r[jj] = pack_bf16(x0, x1);
        }
        qf[qb][kk] = __builtin_bit_cast(bf16x8, r);
      }
  }

  // ---- tile list ----
  const int tq_last = min(t0 + BM, C) - 1;
  const bool has_sink_tile = sh.n_sink > 0 && (s0 + tq_last - W) >= 0;
  const int k_lo = -((W - 1 + BN - 1) / BN);
  const int k_clip = -((s0 + t0 + BN - 1) / BN);
  const int kmin = max(k_lo, k_clip);
  const int n_band = 1 - kmin;
  const int n_tiles = n_band + (has_sink_tile ? 1 : 0);

  // tile it -> (is_sink, first key position relative to s0 for band tiles)
  auto tile_u0 = [&](int it) { return t0 + BN * (kmin + it - (has_sink_tile ? 1 : 0)); };

  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int it) {
    const bool is_sink = has_sink_tile && it == 0;
    const int base = is_sink ? 0 : s0 + tile_u0(it);   // absolute position of row 0
    const int c = tid & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 4) + 16 * j;
      const int P = base + r;
      const uint16_t* src = (is_sink && P >= sh.n_sink) ? nullptr : key_row(a, 0, b, kvh, s0, P);
      kreg[j] = src ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * (tid >> 4) + e;
      const int P = base + r;
      const uint16_t* src = (is_sink && P >= sh.n_sink) ? nullptr : key_row(a, 1, b, kvh, s0, P);
      vreg[e] = src ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&]() {
    const int c = tid & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(Ks + ((tid >> 4) + 16 * j) * KPITCH + c * 16) = kreg[j];
    // V^T: key k of the tile is stored at column pos(k) = 32(k/32) + 8((k%16)/4)
    // + 4((k%32)/16) + k%4, so that the 8 keys one lane needs for a PV step
    // (4 from each of two 16-key score blocks) are 16 contiguous bytes.
    const int quad = tid >> 4;
    const int pos = 32 * (quad >> 3) + 8 * (quad & 3) + 4 * ((quad >> 2) & 1);
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) {
      const int wd = jd >> 1;
      const bool hi = jd & 1;
      uint32_t e0 = hi ? (vreg[0][wd] >> 16) : (vreg[0][wd] & 0xffffu);
      uint32_t e1 = hi ? (vreg[1][wd] >> 16) : (vreg[1][wd] & 0xffffu);
      uint32_t e2 = hi ? (vreg[2][wd] >> 16) : (vreg[2][wd] & 0xffffu);
      uint32_t e3 = hi ? (vreg[3][wd] >> 16) : (vreg[3][wd] & 0xffffu);
      u32x2 val = {e0 | (e1 << 16), e2 | (e3 << 16)};
      *reinterpret_cast<u32x2*>(Vt + (8 * c + jd) * VPITCH + pos * 2) = val;
    }
  };

  float m_run[4], l_run[4];
  floatx4 o[8][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = sh.scale_log2;

  if (n_tiles > 0) load_tile(0);
  for (int it = 0; it < n_tiles; ++it) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(it + 1);

    const bool is_sink = has_sink_tile && it == 0;
    const int u0 = is_sink ? 0 : tile_u0(it);
    // classify this tile for this wave (wave-uniform)
    bool any, full;
    if (is_sink) {
      any = (s0 + q0w + 15 - W) >= 0;
      full = false;
    } else {
      any = !(u0 > q0w + 15 || u0 + BN - 1 <= q0w - W || s0 + u0 + BN - 1 < 0);
      full = (u0 + BN - 1 <= q0w) && (u0 > q0w + 15 - W) && (s0 + u0 >= 0);
    }
    if (!any) continue;

    // ---- S^T = K Q^T: s[kb][qb] rows = keys 16kb+4g+r, column = query i ----
    floatx4 s[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) s[kb][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 ka[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        ka[kb] = *reinterpret_cast<const bf16x8*>(Ks + (16 * kb + i) * KPITCH + (4 * kk + g) * 16);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qf[qb][kk], s[kb][qb], 0, 0, 0);
    }

    // ---- mask the tiles that cut the diagonal, the window edge or position 0 ----
    if (!full) {
      const int I = s0 + tq;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr_ = 16 * kb + 4 * g + r;
          bool ok;
          if (is_sink) {
            const int P = kr_;
            ok = P < sh.n_sink && P <= I - W;
          } else {
            const int u = u0 + kr_;
            ok = (u <= tq) && (u > tq - W) && (s0 + u >= 0);
          }
          if (!ok) {
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) s[kb][qb][r] = -INFINITY;
          }
        }
    }

    // ---- online softmax (log2 domain) ----
    bf16x8 pb[2][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = wave_max_g(mx) * c2;
      const bool need = mx > m_run[qb] + kTau;
      const float alpha = need ? exp2f(m_run[qb] - mx) : 1.f;
      if (need) m_run[qb] = mx;
      if (__any(need)) {
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
      }
      const float msub = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
      float p[4][4];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb][r] = exp2f(fmaf(s[kb][qb][r], c2, -msub));
          ls += p[kb][r];
        }
      l_run[qb] += ls;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 pk;
        pk[0] = pack_bf16(p[2 * s2][0], p[2 * s2][1]);
        pk[1] = pack_bf16(p[2 * s2][2], p[2 * s2][3]);
        pk[2] = pack_bf16(p[2 * s2 + 1][0], p[2 * s2 + 1][1]);
        pk[3] = pack_bf16(p[2 * s2 + 1][2], p[2 * s2 + 1][3]);
        pb[s2][qb] = __builtin_bit_cast(bf16x8, pk);
      }
    }

    // ---- O^T += V^T P^T: o[db][qb] rows = d 16db+4g+r, column = query i ----
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(Vt + (16 * db + i) * VPITCH + (32 * s2 + 8 * g) * 2);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[s2][qb], o[db][qb], 0, 0, 0);
      }
  }

  // ---- epilogue: O / l, LSE ----
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const float lt = wave_sum_g(l_run[qb]);
    const float inv = 1.f / lt;
    if (tq < C) {
      uint16_t* dst = a.out + (((long long)b * C + tq) * sh.Hq + h0 + qb) * HD;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x2 val = {pack_bf16(o[db][qb][0] * inv, o[db][qb][1] * inv),
                     pack_bf16(o[db][qb][2] * inv, o[db][qb][3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 16 * db + 4 * g) = val;
      }
      if (a.lse && g == 0)
        a.lse[((long long)b * sh.Hq + h0 + qb) * C + tq] = (m_run[qb] + log2f(lt)) * 0.69314718055994531f;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic kernel: one thread per (query position, query head).
// ---------------------------------------------------------------------------
template <bool F32>
__device__ inline float ld(const void* base, long long off) {
  if (F32) return static_cast<const float*>(base)[off];
  return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(base)[off]) << 16);
}
template <bool F32>
__device__ inline void st(void* base, long long off, float x) {
  if (F32)
    static_cast<float*>(base)[off] = x;
  else
    static_cast<uint16_t*>(base)[off] = to_bf16_bits(x);
}

template <bool F32, int D>
__global__ void __launch_bounds__(64) prefill_generic_kernel(Shape sh, RopeTab rt, const void* q,
                                                             const void* kr, const void* v,
                                                             const void* kc, const void* vc,
                                                             const int32_t* start, int C, void* out,
                                                             float* lse) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (t >= C) return;
  const int kvh = h / (sh.Hq / sh.Hkv);
  const int s0 = start[b];
  const int I = s0 + t;
  float qv[D];
  const long long qoff = (((long long)b * C + t) * sh.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = ld<F32>(q, qoff + d);
  if (sh.rope) {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      float cs, sn;
      rope_cs(I, rt.freq[kk], cs, sn);
      rotate(qv[2 * kk], qv[2 * kk + 1], cs, sn);
    }
  }
  if (!F32) {
    // the matrix path multiplies bf16 operands: round the rotated query alike
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = __uint_as_float(((uint32_t)to_bf16_bits(qv[d])) << 16);
  }
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  auto visit = [&](int j) {
    const void *kb, *vb;
    long long off;
    if (j >= s0) {
      kb = kr;
      vb = v;
      off = (((long long)b * C + (j - s0)) * sh.Hkv + kvh) * D;
    } else {
      if (!kc) return;
      kb = kc;
      vb = vc;
      off = (((long long)b * sh.S + slot_of(j, sh.W, sh.n_sink)) * sh.Hkv + kvh) * D;
    }
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], ld<F32>(kb, off + d), s);
    s *= sh.scale_log2;
    const float mn = fmaxf(m, s);
    const float al = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float pp = exp2f(s - mn);
    l = l * al + pp;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], al, pp * ld<F32>(vb, off + d));
    m = mn;
  };
  const int lo = max(0, I - sh.W + 1);
  for (int j = 0; j < min(sh.n_sink, lo); ++j) visit(j);
  for (int j = lo; j <= I; ++j) visit(j);
  const float inv = 1.f / l;
  const long long ooff = (((long long)b * C + t) * sh.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) st<F32>(out, ooff + d, o[d] * inv);
  if (lse) lse[((long long)b * sh.Hq + h) * C + t] = (m + log2f(l)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_prefill_bf16_d128_g4(const Shape& sh, const RopeTab& rt, const void* q,
                                       const void* k_rot, const void* v, const void* kc,
                                       const void* vc, const int32_t* start, int C, void* out,
                                       float* lse, hipStream_t st) {
  PrefillArgs a;
  a.sh = sh;
  a.rt = rt;
  a.q = static_cast<const uint16_t*>(q);
  a.kr = static_cast<const uint16_t*>(k_rot);
  a.v = static_cast<const uint16_t*>(v);
  a.kc = static_cast<const uint16_t*>(kc);
  a.vc = static_cast<const uint16_t*>(vc);
  a.start = start;
  a.C = C;
  a.n_qtiles = (C + BM - 1) / BM;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const long long nwg = (long long)a.n_qtiles * sh.Hkv * sh.B;
  prefill_bf16_d128_g4_kernel<<<dim3((unsigned)nwg), dim3(256), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_generic(const Shape& sh, const RopeTab& rt, bool f32, const void* q,
                                  const void* k_rot, const void* v, const void* kc,
                                  const void* vc, const int32_t* start, int C, void* out,
                                  float* lse, hipStream_t st) {
  dim3 grid((C + 63) / 64, sh.Hq, sh.B);
  if (f32) {
    if (sh.D == 64)
      prefill_generic_kernel<true, 64><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse);
    else
      prefill_generic_kernel<true, 128><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse);
  } else {
    if (sh.D == 64)
      prefill_generic_kernel<false, 64><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse);
    else
      prefill_generic_kernel<false, 128><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse);
  }
  return hipGetLastError();
}

}  // namespace swa
