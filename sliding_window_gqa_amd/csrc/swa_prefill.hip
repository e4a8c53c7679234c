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
//    (256 query rows), 8 waves, 2 per SIMD so that one wave's softmax runs
//    while the other's matrix instructions do.  Wave w owns positions
//    t0+16(w&3) .. +15 for 2 of the 4 heads: 32 query rows, about 190 VGPRs.
//  * Key tiles of 64 keys.  K and V tiles are staged in LDS once per
//    work-group and used by all 4 heads (the GQA sharing of explainer How It
//    Works 1), double-buffered so one barrier per tile suffices.  Tiles outside
//    the band i-W < j <= i of the work-group are never visited, so the work is
//    O(N*W); a wave skips the matrix work of tiles outside its own band and
//    masks only the tiles that cut the diagonal or the window edge.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16: in the
//    transposed form every lane owns one query column, so the softmax row
//    statistics stay in one lane plus a 4-lane exchange (permlane swaps), and
//    the score accumulator is already the B operand of the PV product.
//  * V stays row-major in LDS; the A operand of the PV product is read with
//    the transposing LDS load ds_read_b64_tr_b16.  Both tiles use XOR-swizzled
//    16-byte chunks so the operand reads are free of bank conflicts.
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

#include <type_traits>

#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace swa {
namespace {

constexpr int BM = 64;       // query positions per work-group
constexpr int BN = 64;       // keys per tile
constexpr int HD = 128;      // head_dim of the fast kernel
constexpr int ROWB = HD * 2; // bytes of one K or V row
constexpr int TILEB = BN * ROWB;  // bytes of one K (or V) tile in LDS
constexpr float kTau = 8.0f; // lazy-rescale threshold (log2 units)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// XOR swizzles of the 16-byte chunks of a 256-byte LDS row, chosen so that the
// QK^T operand reads (16 lanes: 16 rows, one chunk) and the transposing PV
// operand reads (4 consecutive rows, 2 chunks per 16 lanes) hit distinct banks.
__device__ inline int k_off(int r, int c) { return r * ROWB + ((c ^ (r & 15)) << 4); }
__device__ inline int v_off(int r, int c) { return r * ROWB + ((c ^ (((r & 7) << 1) | ((r >> 3) & 1))) << 4); }

// max / sum over the 4 lanes l, l^16, l^32, l^48 (one query column)
__device__ inline float xg_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float xg_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max of the 4 lanes of a float4 (NaN-propagating IEEE maximum: no
// canonicalising moves, v_maximum3_f32 on gfx950)
__device__ inline float vmax4(floatx4 v) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]),
                                       __builtin_elementwise_maximum(v[2], v[3]));
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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0, expcnt 6:4,
// lgkmcnt 11:8): wait until at most n vector-memory operations of this wave
// are outstanding.
#define SWA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

constexpr int NBUF = 3;              // LDS ring of K/V tiles (prefetch distance 2)
constexpr int LOADS_PER_TILE = 4;    // direct-to-LDS loads per wave per tile (2 K, 2 V)

// One work-group: 64 query positions x 4 query heads of one KV head, 8 waves.
// Wave w owns positions t0 + 16*(w&3) .. +15 and query heads hw, hw+1 with
// hw = 4*kvh + 2*(w>>2); lane (i, g) owns query column i of both 16-row
// query blocks.  K/V tiles of 64 keys go global -> LDS directly
// (global_load_lds_dwordx4, 1 KB per wave instruction) into a 3-deep ring.
__global__ void __launch_bounds__(512) prefill_bf16_d128_g4_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * 2 * TILEB];
  __shared__ double rope_freq[kMaxPairs];

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
  const int q0w = t0 + 16 * (w & 3);      // first query of this wave (chunk-relative)
  const int tq = q0w + i;                 // this lane's query
  const int hw = kvh * 4 + 2 * (w >> 2);  // first query head of this wave
  const int W = sh.W;
  const int S = sh.S;
  const int nsink = sh.n_sink;

  // ---- tile list: [sink tile] + band tiles k = kmin..0 (u0 = t0 + 64k) ----
  const int tq_last = min(t0 + BM, C) - 1;
  const bool has_sink_tile = nsink > 0 && (s0 + tq_last - W) >= 0;
  const int k_lo = -((W - 1 + BN - 1) / BN);
  const int k_clip = -((s0 + t0 + BN - 1) / BN);
  const int kmin = max(k_lo, k_clip);
  const int n_tiles = (1 - kmin) + (has_sink_tile ? 1 : 0);
  const int sink_off = has_sink_tile ? 1 : 0;

  // ---- direct-to-LDS tile loads ----
  // Wave w fills rows 8w .. 8w+7 of the K and of the V tile, 4 rows per
  // instruction; lane l lands at row 8w+4j+l/16, stored chunk l%16, and so
  // fetches the global chunk that the row's XOR swizzle puts there.
  const long long rowstride_c = (long long)sh.Hkv * HD;                // elements between tokens
  const uint16_t* kchunk = a.kr + ((long long)b * C * sh.Hkv + kvh) * HD;
  const uint16_t* vchunk = a.v + ((long long)b * C * sh.Hkv + kvh) * HD;
  const uint16_t* kcache = a.kc ? a.kc + ((long long)b * S * sh.Hkv + kvh) * HD : nullptr;
  const uint16_t* vcache = a.vc ? a.vc + ((long long)b * S * sh.Hkv + kvh) * HD : nullptr;
  // lane-constant byte offsets of this lane's two rows (8w+4j+lane/16) in a
  // run of consecutive source rows, including the chunk swizzle
  const int rowstride_b = sh.Hkv * ROWB;
  int voff_k[2], voff_v[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * w + 4 * j + (lane >> 4);
    const int pos = lane & 15;
    voff_k[j] = row * rowstride_b + 16 * (pos ^ (row & 15));
    voff_v[j] = row * rowstride_b + 16 * (pos ^ (((row & 7) << 1) | ((row >> 3) & 1)));
  }
  auto issue_tile = [&](int it) {
    const int buf = it % NBUF;
    const bool is_sink = has_sink_tile && it == 0;
    const int u0 = is_sink ? 0 : t0 + BN * (kmin + it - sink_off);
    // fast path: the 64 rows are 64 consecutive rows of one tensor
    const uint16_t* kbase = nullptr;
    const uint16_t* vbase = nullptr;
    if (!is_sink) {
      if (u0 >= 0) {
        if (u0 + BN <= C) {
          kbase = kchunk + (long long)u0 * rowstride_c;
          vbase = vchunk + (long long)u0 * rowstride_c;
        }
      } else {
        const int P0 = s0 + u0;
        if (P0 >= nsink) {
          const int slot0 = nsink + (P0 - nsink) % W;
          if (slot0 + BN <= S) {
            kbase = kcache + (long long)slot0 * rowstride_c;
            vbase = vcache + (long long)slot0 * rowstride_c;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint8_t* kl = smem + (buf * 2) * TILEB + (8 * w + 4 * j) * ROWB;
      uint8_t* vl = kl + TILEB;
      const uint8_t* kp;
      const uint8_t* vp;
      if (kbase) {
        kp = reinterpret_cast<const uint8_t*>(kbase) + voff_k[j];
        vp = reinterpret_cast<const uint8_t*>(vbase) + voff_v[j];
      } else {
        // edge tiles: each row located separately, clamped to a row that
        // exists (rows that are not keys of any query are masked later)
        const int row = 8 * w + 4 * j + (lane >> 4);
        const uint16_t* kb;
        const uint16_t* vb;
        int roff;
        if (is_sink) {
          const int P = min(row, nsink - 1);
          if (P < s0 && kcache) {
            kb = kcache; vb = vcache; roff = P;
          } else {
            kb = kchunk; vb = vchunk; roff = min(max(P - s0, 0), C - 1);
          }
        } else if (u0 >= 0) {
          kb = kchunk; vb = vchunk; roff = min(u0 + row, C - 1);
        } else {
          const int P = max(s0 + u0 + row, 0);
          kb = kcache; vb = vcache;
          roff = P < nsink ? P : nsink + (P - nsink) % W;
        }
        const long long rb = (long long)(roff - row) * rowstride_c;   // voff already holds row*stride
        kp = reinterpret_cast<const uint8_t*>(kb + rb) + voff_k[j];
        vp = reinterpret_cast<const uint8_t*>(vb + rb) + voff_v[j];
      }
      __builtin_amdgcn_global_load_lds(kp, (__attribute__((address_space(3))) void*)kl, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp, (__attribute__((address_space(3))) void*)vl, 16, 0, 0);
    }
  };
  // kick off the first two tiles before the Q prologue
  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  // ---- Q prologue: rotated, rounded to bf16, in the B-operand layout ----
  if (tid < kMaxPairs) rope_freq[tid] = a.rt.freq[tid];
  __syncthreads();
  bf16x8 qf[2][4];
  {
    const int I = s0 + tq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float cs[4], sn[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (sh.rope) {
          rope_cs(I, rope_freq[4 * (4 * kk + g) + jj], cs[jj], sn[jj]);
        } else {
          cs[jj] = 1.f;
          sn[jj] = 0.f;
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (tq < C)
          wv = *reinterpret_cast<const u32x4*>(
              a.q + (((long long)b * C + tq) * sh.Hq + hw + qb) * HD + 8 * (4 * kk + g));
        u32x4 r;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float x0 = bf16_lo(wv[jj]), x1 = bf16_hi(wv[jj]);
          rotate(x0, x1, cs[jj], sn[jj]);
          r[jj] = pack_bf16(x0, x1);
        }
        qf[qb][kk] = __builtin_bit_cast(bf16x8, r);
      }
    }
  }

  float m_run[2];
  floatx4 o[8][2];
  // row sums of P accumulate on the matrix core: an all-ones A operand makes
  // every row of lsum[qb] the sum over keys of P for this lane's query
  floatx4 lsum[2];
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m_run[qb] = -INFINITY;
    lsum[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = sh.scale_log2;
  const int I = s0 + tq;

  // One tile, as two 32-key halves: S^T = K Q^T, mask (MK 1: band edge or
  // diagonal, 2: sink tile), online softmax, O^T += V^T P^T.
  auto tile_body = [&](const uint8_t* Kb, lds_u8* Vb, int u0, auto mask_kind) {
    constexpr int MK = decltype(mask_kind)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // s[kb][qb]: rows = keys 32h + 16kb + 4g + r, column = query i
      floatx4 s[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[kb][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kb + k_off(32 * h + 16 * kb + i, 4 * kk + g));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qb][kk], s[kb][qb], 0, 0, 0);
        }
      }
      if constexpr (MK != 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kr_ = 32 * h + 16 * kb + 4 * g + r;
            bool ok;
            if constexpr (MK == 2) {
              ok = kr_ < nsink && kr_ <= I - W;
            } else {
              const int u = u0 + kr_;
              ok = (u <= tq) && (u > tq - W) && (s0 + u >= 0);
            }
            if (!ok) {
              s[kb][0][r] = -INFINITY;
              s[kb][1][r] = -INFINITY;
            }
          }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = __builtin_elementwise_maximum(vmax4(s[0][qb]), vmax4(s[1][qb]));
        mx = xg_max(mx) * c2;
        const bool need = mx > m_run[qb] + kTau;
        if (__builtin_expect(__any(need), 0)) {
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run[qb] - mx) : 1.f;
          if (need) m_run[qb] = mx;
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
        }
        const float msub = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
        float pv[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) pv[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c2, -msub));
        u32x4 pk;
        pk[0] = pack_bf16(pv[0][0], pv[0][1]);
        pk[1] = pack_bf16(pv[0][2], pv[0][3]);
        pk[2] = pack_bf16(pv[1][0], pv[1][1]);
        pk[3] = pack_bf16(pv[1][2], pv[1][3]);
        pb[qb] = __builtin_bit_cast(bf16x8, pk);
      }
      // A operand of the PV product from two transposing LDS reads: lane i of
      // a 16-lane group addresses key base+i/4, d 16db+4(i%4), and receives
      // V[base+e][16db+i] for e = 0..3.
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int cidx = 2 * db + ((i & 3) >> 1);
        const int boff = 8 * (i & 1);
        const int r0 = 32 * h + 4 * g + (i >> 2);
        const int r1 = r0 + 16;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(Vb + v_off(r0, cidx) + boff));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(Vb + v_off(r1, cidx) + boff));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb[qb], o[db][qb], 0, 0, 0);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb], lsum[qb], 0, 0, 0);
    }
  };

  for (int it = 0; it < n_tiles; ++it) {
    // my direct loads of tile it are done (tile it+1 may still be in flight)
    if (it + 1 < n_tiles) SWA_WAIT_VMCNT(LOADS_PER_TILE);
    else SWA_WAIT_VMCNT(0);
    __syncthreads();   // everyone's loads of tile it landed; everyone is done with tile it-1
    if (it + 2 < n_tiles) issue_tile(it + 2);   // into the buffer tile it-1 used

    const int buf = it % NBUF;
    const uint8_t* Kb = smem + (buf * 2) * TILEB;
    lds_u8* Vb = (lds_u8*)smem + (buf * 2) * TILEB + TILEB;
    if (has_sink_tile && it == 0) {
      if ((s0 + q0w + 15 - W) >= 0) tile_body(Kb, Vb, 0, std::integral_constant<int, 2>());
      continue;
    }
    const int u0 = t0 + BN * (kmin + it - sink_off);
    const bool any = !(u0 > q0w + 15 || u0 + BN - 1 <= q0w - W || s0 + u0 + BN - 1 < 0);
    const bool full = (u0 + BN - 1 <= q0w) && (u0 > q0w + 15 - W) && (s0 + u0 >= 0);
    if (full) tile_body(Kb, Vb, u0, std::integral_constant<int, 0>());
    else if (any) tile_body(Kb, Vb, u0, std::integral_constant<int, 1>());
  }

  // ---- epilogue: O / l, LSE ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = lsum[qb][0];
    const float inv = 1.f / lt;
    if (tq < C) {
      uint16_t* dst = a.out + (((long long)b * C + tq) * sh.Hq + hw + qb) * HD;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        u32x2 val = {pack_bf16(o[db][qb][0] * inv, o[db][qb][1] * inv),
                     pack_bf16(o[db][qb][2] * inv, o[db][qb][3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 16 * db + 4 * g) = val;
      }
      if (a.lse && g == 0)
        a.lse[((long long)b * sh.Hq + hw + qb) * C + tq] = (m_run[qb] + log2f(lt)) * 0.69314718055994531f;
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
  prefill_bf16_d128_g4_kernel<<<dim3((unsigned)nwg), dim3(512), 0, st>>>(a);
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
