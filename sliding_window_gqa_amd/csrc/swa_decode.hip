// swa_decode.hip — single-token decode against the rolling buffer.
//
// Digest page "Rolling Buffer KV Cache 동작 설명", 읽기(read) 단계: the query at
// position p reads the buffer entries of positions p-W+1 .. p, which sit in
// at most two contiguous runs of physical slots; the buffer is read in slot
// order and the position each slot holds is recovered from the slot index and
// p (slot_position), so slots not yet written (p < W-1) are never used.
// Reads per token are bounded by the window (essay §3.2, §3.4: decode is
// bound by cache reads; GQA cuts them 4x).
//
// Split-K: the S = n_sink + W slots of a sequence are cut into n_splits
// ranges; each (sequence, KV head, range) is one work-group that streams its
// K/V rows from HBM and leaves an unnormalised partial (m, l, o[D]); a
// combine pass merges the partials of each (sequence, query head):
//   m* = max m_s,  l* = sum l_s 2^(m_s - m*),  o = sum o_s 2^(m_s - m*) / l*.
//
// Fast kernel (bf16, head_dim 128, GQA group 4):
//  * A wave takes 32 slots at a time.  K goes global -> LDS directly (buffer
//    loads with the lds modifier), 16 lanes per whole 256-byte row, into a
//    per-wave double buffer, and is read back in the A-operand layout of
//    v_mfma_f32_16x16x32_bf16 (lane = slot, 8 consecutive head-dim
//    elements): S^T = K Q^T with the 4 query heads of the group as the B
//    columns (the other 12 columns are zero).  Loading K in the operand
//    layout straight from memory (16 rows x 64 bytes per instruction) reads
//    the cache ~8% slower than whole rows.
//  * Each lane loads 8 V rows (16 bytes at one head-dim offset; whole rows
//    per instruction) and transposes them in registers into the A operand of
//    O^T += V^T P^T.  The score accumulator is the B operand.
//  * The NW (4 or 8) waves of a work-group interleave over the range and merge through
//    LDS, so one partial per (sequence, query head, range) reaches memory.
#include <math.h>

#include <atomic>

#include "swa_device.hpp"
#include "swa_launch.hpp"
#include "swa_passes.hpp"

namespace swa {
namespace {

constexpr int HD = 128;
constexpr int kChunk = 32;     // slots per wave step
constexpr float kTau = 8.0f;

__device__ inline float xg_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float xg_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// p, as a value the compiler knows to be the same in every lane
__device__ inline void* uniform_ptr(const void* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
}

struct DecodeArgs {
  Shape sh;
  RopeTab rt;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* pos;
  float* part;
  int n_splits;
  int split_len;
  uint16_t* out;   // written directly (normalised) when n_splits == 1
  float* lse;
  // fused step: the new token's raw key and value [B][Hkv][D] (knew null
  // when there is none) and the caches to store them in (the ones read)
  const uint16_t* knew;
  const uint16_t* vnew;
  uint16_t* kdst;
  uint16_t* vdst;
  DecodeMap map;   // varlen batches: sequence and packed row of each column
};

// K chunks in LDS: 32 rows of 256 bytes, the 16-byte chunk c of row r at
// c ^ (r & 15), so that the 16 rows one operand read touches sit in 16
// different bank groups.
constexpr int DROWB = HD * 2;          // bytes per K row
constexpr int DTILE = kChunk * DROWB;  // one 32-slot K chunk
__device__ inline int dkswz(int r) { return r & 15; }
typedef __attribute__((address_space(3))) uint8_t lds_du8;

// Two direct global-to-LDS loads (each lane's 16 bytes at byte offset o of
// the buffer r, zeros when out of range, land at LDS address l + 16 * lane:
// 1 KB per instruction) with one save and restore of M0, which carries the
// LDS address; one wait state separates each M0 write from its load.  The
// loads are non-temporal, like the V loads: each cache byte is read once
// per call (and, with the caches full of dirty lines, allocating would cost
// their write-back).  The compiler does not count these loads: the loop
// waits for them explicitly.
__device__ inline void ddma2(__amdgpu_buffer_rsrc_t r0, int o0, unsigned l0,
                             __amdgpu_buffer_rsrc_t r1, int o1, unsigned l1) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %5, %6, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(l0), "v"(o0), "s"(r0), "s"(l1), "v"(o1), "s"(r1)
      : "memory");
}

// DIL: dilated window.  The work-groups then cut the sequence's keys, not
// its slots, into ranges: key v < n_sink is sink slot v, key n_sink + k the
// position p - k*dil (slot n_sink + (p - k*dil - n_sink) mod W).
//
// NW: waves per work-group (4 or 8), two waves per SIMD either way.
// G: query heads per KV head (1, 2, 4 or 8; the kernel's name keeps the
// group of 4 of the pages' model): the B operand's columns 0 .. G-1 are the
// group's heads, so every K/V byte read serves all G of them.
template <bool DIL, int NW, int G>
__global__ void __launch_bounds__(64 * NW, 2) decode_bf16_d128_g4_kernel(DecodeArgs a) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  __shared__ __attribute__((aligned(16))) uint8_t kvs[NW * 2 * DTILE];   // [wave][buffer] K
  __shared__ float sm_m[NW][G], sm_l[NW][G];
  __shared__ float sm_o[NW][G][HD];
  __shared__ double rope_rev[kMaxPairs];

  const Shape& sh = a.sh;
  const int split = blockIdx.x, kvh = blockIdx.y, z = blockIdx.z;
  // b: the sequence (position, caches); r: the row of its token in q / out
  const int b = a.map.n ? a.map.seq[z] : z;
  const int r = a.map.n ? a.map.row[z] : z;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int p = __builtin_amdgcn_readfirstlane(a.pos[b]);   // uniform: one sequence per work-group
  const int S = sh.S;
  // slots [0, min(S, p+1)) hold live positions; the others are never read.
  // DIL: the keys are the live sinks, then the window's positions p, p-dil,
  // ... (those past the sinks)
  const int dil = sh.dil, W = sh.W, nsink = sh.n_sink;
  const int n_live = DIL ? min(nsink, p + 1) +
                               (p >= nsink ? min((W + dil - 1) / dil, (p - nsink) / dil + 1) : 0)
                         : min(S, p + 1);
  const int sp0 = split * a.split_len;
  const int vend = min(min(S, sp0 + a.split_len), n_live);
  const int sp_w = p >= nsink ? (p - nsink) % W : 0;   // DIL: slot of p, less n_sink
  // DIL: the slot of key v (keys past vend read key vend-1's row, whose
  // values are finite; their scores are masked)
  auto key_slot = [&](int v) __attribute__((always_inline)) {
    v = min(v, vend - 1);
    if (v < nsink) return v;
    int t = (v - nsink) * dil;
    t = t >= W ? t - W : t;
    const int x = sp_w - t;
    return nsink + (x < 0 ? x + W : x);
  };
  const int h0 = kvh * G;

  const long long row_stride = (long long)sh.Hkv * HD;       // elements between slots
  const uint16_t* kbase = a.kc + ((long long)b * S * sh.Hkv + kvh) * HD;
  const uint16_t* vbase = a.vc + ((long long)b * S * sh.Hkv + kvh) * HD;
  const float c2 = sh.scale_log2;

  // ---- Q: B operand, column i = query head h0+i (i < G), rotated at p ----
  if (tid < kMaxPairs) rope_rev[tid] = a.rt.rev[tid];
  __syncthreads();

  // ---- fused step: the range that holds slot(p) stores the new entry of
  // this head (key rotated at p, as the cache write does it; value as is).
  // No other work-group reads that slot.  Without dilation the store is not
  // waited for: the wave whose chunk holds the slot reads the row from
  // memory like any other (old or new contents, whichever arrives) and then
  // overwrites it with the new entry, in LDS (K) and in its V registers,
  // before the products use it.  Lane (i, g) holds chunk i (head-dim
  // 8i .. 8i+7) of the new key (rotated) and value.
  const int vp = DIL ? (p < nsink ? p : nsink) : slot_of(p, sh.W, sh.n_sink);   // the key that is p
  const bool holder = a.knew != nullptr && vp >= sp0 && vp < sp0 + a.split_len;
  u32x4 knw = {0u, 0u, 0u, 0u}, vnw = {0u, 0u, 0u, 0u};
  if (holder) {
    const long long src = ((long long)r * sh.Hkv + kvh) * HD + 8 * i;
    knw = *reinterpret_cast<const u32x4*>(a.knew + src);
    vnw = *reinterpret_cast<const u32x4*>(a.vnew + src);
  }
  // Rotate the new key and store the entry: wave 0, lanes g = 0 the key,
  // g = 1 the value.  Without dilation this runs once the stream's first
  // loads are out and nothing waits for it.  With dilation the keys past the
  // live range read the row of the last live key (masked, but their values
  // must be finite), which can be the new entry: there the store completes
  // before the first load, as in the separate cache write.
  auto store_new = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float x0 = bf16_lo(knw[jj]), x1 = bf16_hi(knw[jj]);
      if (sh.rope) {
        float cs, sn;
        rope_cs(p, rope_rev[4 * i + jj], cs, sn);
        rotate(x0, x1, cs, sn);
      }
      knw[jj] = pack_bf16(x0, x1);
    }
    if (tid < 32) {
      const long long dst = ((long long)b * S + slot_of(p, sh.W, sh.n_sink)) * row_stride + kvh * HD + 8 * i;
      if (tid < 16)
        *reinterpret_cast<u32x4*>(a.kdst + dst) = knw;
      else
        *reinterpret_cast<u32x4*>(a.vdst + dst) = vnw;
    }
  };
  if (DIL && holder) {
    store_new();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  bf16x8 qf[4];
  auto load_q = [&]() __attribute__((always_inline)) {
    // (all four loads go out before the first is used; lanes i >= 4 load a
    // row that exists and drop it)
    u32x4 wq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      wq[kk] = *reinterpret_cast<const u32x4*>(a.q + ((long long)r * sh.Hq + h0 + (i & (G - 1))) * HD + 8 * (4 * kk + g));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 wv = i < G ? wq[kk] : u32x4{0u, 0u, 0u, 0u};
      u32x4 r;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float x0 = bf16_lo(wv[jj]), x1 = bf16_hi(wv[jj]);
        if (sh.rope) {
          float cs, sn;
          rope_cs(p, rope_rev[4 * (4 * kk + g) + jj], cs, sn);
          rotate(x0, x1, cs, sn);
        }
        r[jj] = pack_bf16(x0, x1);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, r);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  floatx4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Buffer loads: the descriptors cover exactly this head's rows of the live
  // slots [0, vend), so rows past vend read as zeros (and are masked out of
  // the softmax).  Each K/V byte is read once per call.
  const unsigned rowb = (unsigned)row_stride * 2u;
  const int nrec = __builtin_amdgcn_readfirstlane(((DIL ? S : vend) - 1) * (int)rowb + HD * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kbase), (short)0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vbase), (short)0, nrec, 0x00020000);
  // Load instruction e (0..7) of a chunk fills rows 4e .. 4e+3 (row 4e + g'
  // for lane (i', g')): the lane fetches the 16-byte chunk that belongs at
  // position i' under the swizzle.  The swizzles repeat every 4 instructions.
  int ko[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ko[e] = g * (int)rowb + 16 * (i ^ dkswz(4 * e + g));
  const unsigned lds_w = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((lds_du8*)kvs) + (unsigned)w * (2u * DTILE));
  auto dma_chunk = [&](int c0, int buf) __attribute__((always_inline)) {
    const int cb = c0 * (int)rowb;
    const unsigned lb = lds_w + (unsigned)buf * DTILE;
    if (DIL) {
      // lane (i, g) of load e fetches key c0 + 4e + g
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        ddma2(rk, key_slot(c0 + 4 * e + g) * (int)rowb + 16 * (i ^ dkswz(4 * e + g)), lb + 1024u * e,
              rk, key_slot(c0 + 4 * (e + 1) + g) * (int)rowb + 16 * (i ^ dkswz(4 * (e + 1) + g)),
              lb + 1024u * (e + 1));
    } else {
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        ddma2(rk, cb + 4 * e * (int)rowb + ko[e & 3], lb + 1024u * e,
              rk, cb + 4 * (e + 1) * (int)rowb + ko[(e + 1) & 3], lb + 1024u * (e + 1));
    }
  };
  // V: lane (i, g) loads slots kappa(g, e) = {4g+e, 16+4g+e-4}, d = 8i .. 8i+7
  unsigned voff[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) voff[e] = (unsigned)(e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4)) * rowb + 16u * i;
  constexpr int kNT = 2;
  auto load_v = [&](int c0, u32x4 (&vr)[8]) __attribute__((always_inline)) {
    const unsigned cb = (unsigned)c0 * rowb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = DIL ? key_slot(c0 + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4))) * (int)rowb + 16 * i
                          : (int)(cb + voff[e]);
      vr[e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kNT));
    }
  };
  // operand reads (as the chunk layout above): K rows 16kb + i, d-chunk 4kk+g
  int kofs[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kofs[kk] = i * DROWB + 16 * ((4 * kk + g) ^ dkswz(i));
  auto do_chunk = [&](int c0, int buf, const u32x4 (&vr)[8]) __attribute__((always_inline)) {
    const uint8_t* Kb = kvs + (w * 2 + buf) * DTILE;
    floatx4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(Kb + kofs[kk] + 16 * kb * DROWB);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qf[kk], s[kb], 0, 0, 0);
      }
    }
    // mask slots past the live range
    if (c0 + kChunk > vend) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (c0 + 16 * kb + 4 * g + r >= vend) s[kb][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xg_max(mx) * c2;
    const bool need = mx > m_run + kTau;
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
    if (need) m_run = mx;
    if (__any(need)) {
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    const float msub = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -msub));
        l_run += pv[kb][r];
      }
    u32x4 pk;
    pk[0] = pack_bf16(pv[0][0], pv[0][1]);
    pk[1] = pack_bf16(pv[0][2], pv[0][3]);
    pk[2] = pack_bf16(pv[1][0], pv[1][1]);
    pk[3] = pack_bf16(pv[1][2], pv[1][3]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
    // transpose: A operand of d-block db holds, for d = 8i+db, the 8 slots kappa(g, e)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int wd = db >> 1;
      u32x4 va;
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2)
        va[m2] = __builtin_amdgcn_perm(vr[2 * m2 + 1][wd], vr[2 * m2][wd], (db & 1) ? 0x07060302u : 0x05040100u);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb, o[db], 0, 0, 0);
    }
  };
  // The chunk row rr (0..31) that is the new entry: its K row in this
  // wave's LDS buffer (chunk i at i ^ dkswz(rr), written by lanes g = 0 once
  // the chunk's loads have landed) and its V row, which sits in register
  // e of the lanes g (rows 4g+e, then 16+4g+e-4, as load_v places them).
  auto put_new = [&](int rr, int buf, u32x4 (&vr)[8]) __attribute__((always_inline)) {
    if (g == 0)
      *reinterpret_cast<u32x4*>(kvs + (w * 2 + buf) * DTILE + rr * DROWB + 16 * (i ^ dkswz(rr))) = knw;
    const int gt = (rr & 15) >> 2, et = (rr & 3) + (rr >= 16 ? 4 : 0);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e == et && g == gt) vr[e] = vnw;
  };
  // Each wave takes chunks c0, c0 + 4*kChunk, ... of the range; the next
  // chunk's 16 loads go out before the current chunk is computed (past the
  // range they read zeros).  The buffer a load fills was last read by the
  // previous chunk's products, which have consumed their operands.
  // Step m: K(m+1) to LDS (8 loads), the products of chunk m, then V(m+2)
  // into the registers V(m) held.  K(m) is complete once at most the 16
  // younger loads (V(m+1), K(m+1)) are outstanding; the compiler's own wait
  // for V(m) (8 younger register loads in its count) leaves K(m+1) in flight.
  {
    const int cstep = NW * kChunk;
    int c0 = sp0 + kChunk * w;
    u32x4 vA[8], vB[8];
    if (c0 < vend) {
      dma_chunk(c0, 0);
      load_v(c0, vA);
      load_v(c0 + cstep, vB);
    }
    load_q();
    if (!DIL && holder) store_new();
    int buf = 0;
    while (c0 < vend) {
      dma_chunk(c0 + cstep, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      if (!DIL && holder && (unsigned)(vp - c0) < (unsigned)kChunk) put_new(vp - c0, buf, vA);
      do_chunk(c0, buf, vA);
      load_v(c0 + 2 * cstep, vA);
      c0 += cstep;
      buf ^= 1;
      if (c0 >= vend) break;
      dma_chunk(c0 + cstep, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      if (!DIL && holder && (unsigned)(vp - c0) < (unsigned)kChunk) put_new(vp - c0, buf, vB);
      do_chunk(c0, buf, vB);
      load_v(c0 + 2 * cstep, vB);
      c0 += cstep;
      buf ^= 1;
    }
    // the last loads must land before the work-group's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // ---- merge the NW waves through LDS ----
  const float lt = xg_sum(l_run);
  if (i < G) {
    if (g == 0) {
      sm_m[w][i] = m_run;
      sm_l[w][i] = lt;
    }
    // o[db][r]: head i, d = 8*(4g+r) + db
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[w][i][8 * (4 * g + r) + db] = o[db][r];
  }
  __syncthreads();
  for (int idx = tid; idx < G * HD; idx += 64 * NW) {
    const int hh = idx / HD, d = idx - hh * HD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float Lsum = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sm_m[ww][hh];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      Lsum += sm_l[ww][hh] * f;
      O += sm_o[ww][hh][d] * f;
    }
    if (a.n_splits == 1) {
      // one range covers the sequence: this is the final result
      const long long off = ((long long)r * sh.Hq + h0 + hh) * HD + d;
      a.out[off] = to_bf16_bits(O / Lsum);
      if (a.lse && d == 0) {
        const long long lo = a.map.n ? (long long)(h0 + hh) * a.map.lse_hs + r : (long long)b * sh.Hq + h0 + hh;
        a.lse[lo] = (M + log2f(Lsum)) * 0.69314718055994531f;
      }
    } else {
      float* dst = a.part + (((long long)z * sh.Hq + h0 + hh) * a.n_splits + split) * (HD + 2);
      dst[d] = O;
      if (d == 0) {
        dst[HD] = M;
        dst[HD + 1] = Lsum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Generic decode: one wave per (split, query head, sequence).  Lanes score 64
// slots at a time, then accumulate O over those slots with lane = head dim.
// ---------------------------------------------------------------------------
template <bool F32>
__device__ inline float ldv(const void* base, long long off) {
  if (F32) return static_cast<const float*>(base)[off];
  return __uint_as_float(((uint32_t) static_cast<const uint16_t*>(base)[off]) << 16);
}

template <bool F32, int D>
__global__ void __launch_bounds__(64) decode_generic_kernel(Shape sh, RopeTab rt, const void* q,
                                                            const void* kc, const void* vc,
                                                            const int32_t* pos, float* part,
                                                            int n_splits, int split_len) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int kvh = h / (sh.Hq / sh.Hkv);
  const int p = pos[b];
  float qv[D];
  const long long qoff = ((long long)b * sh.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = ldv<F32>(q, qoff + d);
  if (sh.rope) {
#pragma unroll
    for (int kk = 0; kk < D / 2; ++kk) {
      float cs, sn;
      rope_cs(p, rt.rev[kk], cs, sn);
      rotate(qv[2 * kk], qv[2 * kk + 1], cs, sn);
    }
  }
  if (!F32) {
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = __uint_as_float(((uint32_t)to_bf16_bits(qv[d])) << 16);
  }
  constexpr int E = D / 64;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int sp0 = split * split_len;
  const int sp1 = min(sh.S, sp0 + split_len);
  for (int c0 = sp0; c0 < sp1; c0 += 64) {
    const int slot = c0 + lane;
    int P = -1;
    if (slot < sp1) P = slot_position(slot, p, sh.W, sh.n_sink);
    // a rolling slot's position is inside the window; with dilation it is a
    // key only at a distance that is a multiple of dil
    if (P >= sh.n_sink && (p - P) % sh.dil != 0) P = -1;
    float sc = -INFINITY;
    const long long roff = (((long long)b * sh.S + slot) * sh.Hkv + kvh) * D;
    if (P >= 0) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(qv[d], ldv<F32>(kc, roff + d), acc);
      sc = acc * sh.scale_log2;
    }
    float cm = sc;
    for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float mn = fmaxf(m, cm);
    if (mn == -INFINITY) continue;
    const float al = (m == -INFINITY) ? 0.f : exp2f(m - mn);
    const float pj = (P >= 0) ? exp2f(sc - mn) : 0.f;
    float ps = pj;
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * al + ps;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= al;
    for (int jj = 0; jj < 64; ++jj) {
      const float pjj = __shfl(pj, jj);
      if (pjj != 0.f) {
        const long long voff = (((long long)b * sh.S + (c0 + jj)) * sh.Hkv + kvh) * D;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(pjj, ldv<F32>(vc, voff + lane + 64 * e), o[e]);
      }
    }
    m = mn;
  }
  float* dst = part + (((long long)b * sh.Hq + h) * n_splits + split) * (D + 2);
#pragma unroll
  for (int e = 0; e < E; ++e) dst[lane + 64 * e] = o[e];
  if (lane == 0) {
    dst[D] = m;
    dst[D + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// Combine: one work-group per (query head, sequence), one thread per head
// dim (the body, combine_column, is shared with the mixed step's tail).
// ---------------------------------------------------------------------------
template <bool F32>
__global__ void __launch_bounds__(128) decode_combine_kernel(Shape sh, const float* part, int n_splits,
                                                             void* out, float* lse, DecodeMap map) {
  __shared__ float sm_m[kMaxSplits], sm_l[kMaxSplits], sm_f[kMaxSplits];
  combine_column<F32>(sh, part, n_splits, out, lse, map, blockIdx.x, blockIdx.y, threadIdx.x, sm_m, sm_l, sm_f);
}

}  // namespace

// Splits: about one work-group per CU (256 CUs), each range at least 256
// slots.  Longer ranges per work-group beat more, shorter ones: the
// per-work-group prologue, the merge and the combine pass cost more than the
// load imbalance (16 sequences with 4096 slots stream at 5.17 TB/s with 2
// splits against 5.05 with 4, 8 sequences take 31.9 us with 4 splits against
// 32.3 with 8, one sequence 11.25 us per step with 16 against 11.5 with 32).
// Each range is a multiple of the 128 slots one work-group step covers.
// Keys a fast decode streams per (sequence, KV head): the slots, or with a
// dilated window the sinks and ceil(W/dil) window keys.
static Shape key_shape(const Shape& sh) {
  Shape k = sh;
  if (sh.dil > 1) k.S = sh.n_sink + (sh.W + sh.dil - 1) / sh.dil;
  return k;
}

int decode_splits_fast(const Shape& sh) { return decode_splits(key_shape(sh)); }

int decode_splits(const Shape& sh) {
  const int units = sh.B * sh.Hkv;
  int n = (256 + units - 1) / units;
  const int max_n = (sh.S + 8 * kChunk - 1) / (8 * kChunk);
  if (n > max_n) n = max_n;
  if (n > kMaxSplits) n = kMaxSplits;   // (the combine's LDS; 256 / units never exceeds it)
  if (n < 1) n = 1;
  return n;
}

static int split_len_of(const Shape& sh, int n_splits) {
  int len = (sh.S + n_splits - 1) / n_splits;
  len = (len + 4 * kChunk - 1) / (4 * kChunk) * (4 * kChunk);
  return len;
}

static int cu_count() {   // of the current device, 0 if unknown; cached per device
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Waves per work-group of the fast kernel (no dilation): 8 when the grid
// holds between a half and one work-group per CU and each range gives all 8
// waves slots, else 4.  With one work-group per CU the 8-wave form keeps
// twice the loads in flight per CU: 16 sequences x 8 KV heads x 2 ranges
// stream at 5.19 against 5.14 TB/s, 8 sequences x 4 ranges take 31.2 against
// 31.8 us; with two or more work-groups per CU (64 sequences) 4 waves are
// faster, and so with half the CUs or fewer (one sequence x 16 ranges: 11.25
// against 11.9 us per step).
static int decode_waves(const Shape& sh, int n_splits) {
  if (sh.dil > 1 || sh.Hq != 4 * sh.Hkv) return 4;
  const long long wgs = (long long)sh.B * sh.Hkv * n_splits;
  const int cus = cu_count();
  return (cus > 0 && 2 * wgs > cus && wgs <= cus && split_len_of(key_shape(sh), n_splits) >= 8 * kChunk) ? 8 : 4;
}

hipError_t launch_decode_bf16_d128_g4(const Shape& sh, const RopeTab& rt, const void* q,
                                      const void* kc, const void* vc, const int32_t* pos,
                                      float* partial, int n_splits, void* out, float* lse,
                                      const FusedWrite* fw, const DecodeMap* map, hipStream_t st) {
  DecodeArgs a;
  a.sh = sh;
  a.rt = rt;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kc);
  a.vc = static_cast<const uint16_t*>(vc);
  a.pos = pos;
  a.part = partial;
  a.n_splits = n_splits;
  a.split_len = split_len_of(key_shape(sh), n_splits);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.knew = fw ? static_cast<const uint16_t*>(fw->k) : nullptr;
  a.vnew = fw ? static_cast<const uint16_t*>(fw->v) : nullptr;
  a.kdst = fw ? static_cast<uint16_t*>(fw->k_cache) : nullptr;
  a.vdst = fw ? static_cast<uint16_t*>(fw->v_cache) : nullptr;
  if (map)
    a.map = *map;
  else
    a.map = DecodeMap{};
  const int nw = decode_waves(sh, n_splits);
  const int G = sh.Hq / sh.Hkv;
  const dim3 grid(n_splits, sh.Hkv, sh.B);
  if (G == 4) {
    if (sh.dil > 1)
      decode_bf16_d128_g4_kernel<true, 4, 4><<<grid, dim3(256), 0, st>>>(a);
    else if (nw == 8)
      decode_bf16_d128_g4_kernel<false, 8, 4><<<grid, dim3(512), 0, st>>>(a);
    else
      decode_bf16_d128_g4_kernel<false, 4, 4><<<grid, dim3(256), 0, st>>>(a);
  } else if (sh.dil > 1 || sh.Hq != G * sh.Hkv) {
    return hipErrorInvalidValue;   // (the host sends these shapes to the generic kernel)
  } else if (G == 1) {
    decode_bf16_d128_g4_kernel<false, 4, 1><<<grid, dim3(256), 0, st>>>(a);
  } else if (G == 2) {
    decode_bf16_d128_g4_kernel<false, 4, 2><<<grid, dim3(256), 0, st>>>(a);
  } else if (G == 8) {
    decode_bf16_d128_g4_kernel<false, 4, 8><<<grid, dim3(256), 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_generic(const Shape& sh, const RopeTab& rt, bool f32, const void* q,
                                 const void* kc, const void* vc, const int32_t* pos,
                                 float* partial, int n_splits, hipStream_t st) {
  const int split_len = split_len_of(sh, n_splits);
  dim3 grid(n_splits, sh.Hq, sh.B);
  if (f32) {
    if (sh.D == 64)
      decode_generic_kernel<true, 64><<<grid, 64, 0, st>>>(sh, rt, q, kc, vc, pos, partial, n_splits, split_len);
    else
      decode_generic_kernel<true, 128><<<grid, 64, 0, st>>>(sh, rt, q, kc, vc, pos, partial, n_splits, split_len);
  } else {
    if (sh.D == 64)
      decode_generic_kernel<false, 64><<<grid, 64, 0, st>>>(sh, rt, q, kc, vc, pos, partial, n_splits, split_len);
    else
      decode_generic_kernel<false, 128><<<grid, 64, 0, st>>>(sh, rt, q, kc, vc, pos, partial, n_splits, split_len);
  }
  return hipGetLastError();
}

hipError_t launch_decode_combine(const Shape& sh, bool f32, const float* partial, int n_splits,
                                 void* out, float* lse, const DecodeMap* map, hipStream_t st) {
  dim3 grid(sh.Hq, sh.B);
  const DecodeMap none{};
  const DecodeMap& m = map ? *map : none;
  if (f32)
    decode_combine_kernel<true><<<grid, sh.D, 0, st>>>(sh, partial, n_splits, out, lse, m);
  else
    decode_combine_kernel<false><<<grid, sh.D, 0, st>>>(sh, partial, n_splits, out, lse, m);
  return hipGetLastError();
}

}  // namespace swa
