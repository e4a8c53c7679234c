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
//    (256 query rows), 8 waves, two per SIMD.  Wave w owns positions
//    t0+16(w&3) .. +15 for 2 of the 4 heads (32 query columns), so every K or
//    V operand read from LDS feeds two matrix instructions (one per head):
//    the GQA sharing of explainer How It Works 1 applied inside the wave.
//  * Each tile takes two phases, a barrier after each: a matrix phase (the
//    QK^T and PV products, plus the LDS operand reads) and a vector phase
//    (masks, threshold checks, exponentials, tile loads).  The two waves of
//    a SIMD run one phase apart, so one feeds the matrix core while the
//    other works on the vector ALU.
//  * Key tiles of 32 keys in an 8-slot LDS ring.  Tiles outside the band
//    i-W < j <= i of the work-group are never visited, so the work is
//    O(N*W); only tiles that cut the diagonal or the window edge are
//    masked.  Tiles move global -> LDS directly (buffer loads with the lds
//    modifier, out-of-range rows read as zeros) four tiles ahead.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16: in the
//    transposed form every lane owns one query column, so the softmax column
//    statistics stay in one lane plus a 4-lane exchange (permlane swaps), and
//    the score accumulator is already the B operand of the PV product.
//  * V stays row-major in LDS; the A operand of the PV product is read with
//    the transposing LDS load ds_read_b64_tr_b16.  XOR-swizzled 16-byte
//    chunks keep the operand reads free of bank conflicts.
//  * Softmax in the log2 domain with a lazy reference: Q is scaled by
//    scale*log2(e) before its bf16 rounding, and the QK^T accumulator starts
//    at minus the column's reference, so the matrix core returns score - ref
//    and P = exp2 of it: one exponential and half a conversion per score on
//    the vector ALU.  The reference moves (and O and l are rescaled) only
//    when a score exceeds it by more than 2^8; numerator and denominator
//    carry the same reference, so the result is the same.
//  * Work-groups are renumbered so that the 8 XCDs each take a contiguous
//    range of (sequence, KV head, query tile): the K/V of one KV head then
//    stays in one XCD's L2.  Query tiles run longest-first.
//
// Generic kernel: float32 or bf16, head_dim 64 or 128, any group size; one
// thread per query row, scalar loops.  Used for shapes the fast kernel does
// not cover (e.g. the float32 path).
#include <math.h>

#include <atomic>
#include <climits>
#include <type_traits>

#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace swa {
namespace {

constexpr int BM = 64;       // query positions per work-group
constexpr int BN = 32;       // keys per tile (one pipeline step)
constexpr int HD = 128;      // head_dim of the fast kernel
constexpr int NTHR = 512;    // 8 waves, two per SIMD
constexpr int QB = 2;        // query heads per wave
constexpr float kTau = 8.0f; // lazy-rescale threshold (log2 units)
constexpr int NBUF = 8;      // LDS ring of K/V tiles
static_assert(BN == 32, "the tile arithmetic below divides by 32 with >> 5");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS tiles: 32 rows of 256 bytes, the 16-byte chunk c of row r stored at
// position c ^ kswz(r) (K) or c ^ vswz(r) (V).  The 16 rows one QK^T operand
// read touches then sit in 16 different bank groups, and so do the 8 rows x
// 32 bytes of a transposing PV read.  Rows are unpadded so that the direct
// global-to-LDS loads (1 KB per wave instruction) fill 4 whole rows.
constexpr int ROWB = HD * 2;
constexpr int KTILEB = BN * ROWB;
constexpr int VTILEB = BN * ROWB;
constexpr int RINGB = KTILEB + VTILEB;   // one K+V tile in the ring
__device__ inline int kswz(int r) { return r & 15; }
__device__ inline int vswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Work-group barrier for the tile ring.  __syncthreads() carries a release
// fence that makes the compiler wait for every outstanding vector-memory
// operation (including prefetched tiles) before s_barrier; here only the
// wave's own LDS operations are awaited, and the asm clobbers keep the
// compiler from moving LDS accesses across the barrier.
__device__ inline void ring_barrier() {
  // vmcnt(2): of the direct-to-LDS tile loads only the two of the newest
  // tile may still be in flight.  lgkmcnt(0) goes through the builtin so
  // that the compiler knows the LDS reads are complete and adds no waits of
  // its own after the barrier.
  asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct global-to-LDS load: every lane's 16 bytes at byte offset `off`
// of the buffer `rsrc` (zeros when out of range) land at LDS address
// lds + 16 * lane.  M0 carries the LDS address; it is saved and restored
// around the load, and one wait state separates its write from the load.
// The compiler does not count these loads: ring_barrier() waits for them.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, int off, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(rsrc)
      : "memory");
}

// max over the 4 lanes l, l^16, l^32, l^48 (one query column)
__device__ inline float xg_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// max of the 4 lanes of a float4 (NaN-propagating IEEE maximum: no
// canonicalising moves, v_maximum3_f32 on gfx950)
__device__ inline float vmax4(floatx4 v) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(v[0], v[1]),
                                       __builtin_elementwise_maximum(v[2], v[3]));
}

// p, as a value the compiler knows to be the same in every lane
__device__ inline void* uniform_ptr(const void* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
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
  int n_items;          // n_qtiles * Hkv * B
  uint16_t* out;
  float* lse;
};

// One work-group: 64 query positions x the 4 query heads of one KV head,
// 8 waves, two per SIMD.  Wave w owns positions t0 + 16(w&3) .. +15 for heads
// h0, h0+1 (h0 = 4 kvh + 2(w>>2)); lane (i, g) owns query column i of each
// of its heads.  Every K/V operand read from LDS feeds two matrix
// instructions (one per head).
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_d128_g4_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * RINGB];
  __shared__ double rope_rev[kMaxPairs];

  const Shape& sh = a.sh;
  const int tid = threadIdx.x;
  if (tid < kMaxPairs) rope_rev[tid] = a.rt.rev[tid];
  __syncthreads();

  // ---- work mapping ----
  // Items (sequence, KV head, query tile) are numbered sequence-major, KV
  // head next, query tiles longest first, and split into 8 contiguous
  // ranges, one per XCD (work-group w runs on XCD w mod 8), so that the K/V
  // of a KV head stays in one XCD's L2.  With one item per work-group the
  // hardware hands them out in that order; with fewer work-groups (one per
  // CU, a multiple of 8) each takes the items of its XCD's range in a
  // serpentine order over the rounds, which evens out the longest-first
  // lengths.
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  for (int round = 0;; ++round) {
    int L;
    if (G >= a.n_items) {
      if (round > 0) break;
      const int q8 = G >> 3, r8 = G & 7;
      L = xcd * q8 + min(xcd, r8) + (wg >> 3);
    } else {
      const int q8 = a.n_items >> 3, r8 = a.n_items & 7;
      const int lo = xcd * q8 + min(xcd, r8), cnt = q8 + (xcd < r8 ? 1 : 0);
      const int nl = G >> 3, li = wg >> 3;
      const int pos = round * nl + ((round & 1) ? nl - 1 - li : li);
      if (pos >= cnt) break;
      L = lo + pos;
    }
    const int per_b = sh.Hkv * a.n_qtiles;
    const int b = L / per_b;
    const int rem = L - b * per_b;
    const int kvh = rem / a.n_qtiles;
    const int qt = a.n_qtiles - 1 - (rem - kvh * a.n_qtiles);

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, i = lane & 15, g = lane >> 4;
    const int s0 = a.start[b];
    const int C = a.C;
    const int t0 = qt * BM;
    const int q0w = t0 + 16 * (w & 3);      // first query of this wave (chunk-relative)
    const int tq = q0w + i;                 // this lane's query
    const int I = s0 + tq;                  // its absolute position
    const int h0 = kvh * 4 + QB * (w >> 2); // first query head of this wave
    const int W = sh.W;
    const int S = sh.S;
    const int nsink = sh.n_sink;

    // ---- tile list: [sink tiles] + band tiles k = kmin..1 (u0 = t0 + 32k) ----
    // Band tiles cover chunk-relative key positions t0 - W + 1 .. t0 + 63;
    // sink tiles cover absolute positions 0 .. n_sink-1 for queries whose
    // window no longer contains them.
    const int tq_last = min(t0 + BM, C) - 1;
    const int n_stile = (nsink > 0 && (s0 + tq_last - W) >= 0) ? (nsink + BN - 1) / BN : 0;
    const int k_lo = -((W - 1 + BN - 1) / BN);
    const int k_clip = -((s0 + t0 + BN - 1) / BN);
    const int kmin = max(k_lo, k_clip);
    const int n_tiles = n_stile + (2 - kmin);
    auto band_u0 = [&](int t) __attribute__((always_inline)) { return t0 + BN * (kmin + t - n_stile); };

    // ---- tile loads: global -> staging VGPRs -> padded LDS ----
    // Thread (lr = tid/16, lc = tid%16) moves 16-byte chunk lc of row lr of
    // the K and of the V tile.  A tile's loads are issued one pipeline step
    // before it is stored.
    const long long rowstride_c = (long long)sh.Hkv * HD;                // elements between tokens
    const uint16_t* kchunk = a.kr + ((long long)b * C * sh.Hkv + kvh) * HD;
    const uint16_t* vchunk = a.v + ((long long)b * C * sh.Hkv + kvh) * HD;
    const uint16_t* kcache = a.kc ? a.kc + ((long long)b * S * sh.Hkv + kvh) * HD : nullptr;
    const uint16_t* vcache = a.vc ? a.vc + ((long long)b * S * sh.Hkv + kvh) * HD : nullptr;
    const int lr = tid >> 4, lc = tid & 15;
    const unsigned rowbytes = (unsigned)sh.Hkv * 2u * HD;
    const unsigned voff0 = (unsigned)lr * rowbytes + 16u * lc;
    u32x4 stage[2];   // K row lr, V row lr
    // The loader captures by value and selects pointer values only: with
    // captures by reference, or a struct returned from several places, the
    // compiler selects between addresses of the pointer variables and keeps
    // them in scratch memory.
    auto load_tile = [=](int t, u32x4 (&st)[2]) __attribute__((always_inline)) {
      const bool is_sink = t < n_stile;
      const int u0 = is_sink ? 0 : band_u0(t);
      const bool in_chunk = u0 >= 0;
      const int P0 = s0 + u0;
      // fast path: the 32 rows are 32 consecutive rows of the chunk or cache
      // (the slot arithmetic is done for cache tiles only)
      int slot0 = 0;
      bool fast = !is_sink && in_chunk && u0 + BN <= C;
      if (!is_sink && !in_chunk && P0 >= nsink) {
        slot0 = nsink + (P0 - nsink) % W;
        fast = slot0 + BN <= S;
      }
      if (fast) {
        const long long row0 = in_chunk ? u0 : slot0;
        const uint8_t* kb8 = reinterpret_cast<const uint8_t*>((in_chunk ? kchunk : kcache) + row0 * rowstride_c);
        const uint8_t* vb8 = reinterpret_cast<const uint8_t*>((in_chunk ? vchunk : vcache) + row0 * rowstride_c);
        st[0] = *reinterpret_cast<const u32x4*>(kb8 + voff0);
        st[1] = *reinterpret_cast<const u32x4*>(vb8 + voff0);
      } else {
        // edge tiles: each row is located on its own, clamped to a row that
        // exists (rows that are not keys of any query are masked later)
        {
          const int r = lr;
          // absolute position of the row; rows of band tiles with u0 < 0 are
          // cache rows, those with u0 >= 0 chunk rows
          const int P = is_sink ? min(BN * t + r, nsink - 1) : max(P0 + r, 0);
          const bool from_cache = P < s0 && kcache != nullptr;
          const int roff = from_cache ? (P < nsink ? P : nsink + (P - nsink) % W)
                                      : min(max(P - s0, 0), C - 1);
          const long long eoff = (long long)roff * rowstride_c + 8 * lc;
          st[0] = *reinterpret_cast<const u32x4*>((from_cache ? kcache : kchunk) + eoff);
          st[1] = *reinterpret_cast<const u32x4*>((from_cache ? vcache : vchunk) + eoff);
        }
      }
    };
    // Byte offset of tile t's ring slot.  The empty asm hides the value's
    // origin from loop strength reduction, which would otherwise keep one
    // induction variable per LDS address instead of folding the constant parts
    // into the instructions' offset fields.
    auto slot_off = [&](int t) __attribute__((always_inline)) {
      unsigned off = (unsigned)(t % NBUF) * RINGB;
      asm volatile("" : "+s"(off));
      return off;
    };
    auto store_tile = [&](int t, const u32x4 (&st)[2]) __attribute__((always_inline)) {
      uint8_t* Kb = smem + slot_off(t);
      *reinterpret_cast<u32x4*>(Kb + lr * ROWB + 16 * (lc ^ kswz(lr))) = st[0];
      *reinterpret_cast<u32x4*>(Kb + KTILEB + lr * ROWB + 16 * (lc ^ vswz(lr))) = st[1];
    };
    // Band tiles (all tiles but sink tiles, which can only be tiles 0 and 1)
    // go global -> LDS directly.  Wave w fills rows 4w .. 4w+3 of the K and of
    // the V tile: lane L loads the chunk that belongs at position L%16 of row
    // 4w + L/16 under the swizzle.  The descriptor (chunk or cache, uniform per
    // tile) covers exactly this head's rows of that tensor, so rows past its
    // end read as zeros; cache rows take the slot map, and rows before
    // position 0 read slot 0 (they are masked).
    const int nrec_c = __builtin_amdgcn_readfirstlane((C - 1) * (int)rowbytes + HD * 2);
    const int nrec_s = __builtin_amdgcn_readfirstlane(kcache ? (S - 1) * (int)rowbytes + HD * 2 : 0);
    const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kchunk), (short)0, nrec_c, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vchunk), (short)0, nrec_c, 0x00020000);
    const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kcache ? kcache : kchunk), (short)0, nrec_s, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(vcache ? vcache : vchunk), (short)0, nrec_s, 0x00020000);
    const int rdma = 4 * w + (lane >> 4);               // row of the tile this lane loads
    const int dk = 16 * ((lane & 15) ^ kswz(rdma));     // byte of that row, K
    const int dv = 16 * ((lane & 15) ^ vswz(rdma));     // byte of that row, V
    const int vrk = rdma * (int)rowbytes + dk;          // lane offsets within a chunk tile
    const int vrv = rdma * (int)rowbytes + dv;
    const unsigned lds_base = __builtin_amdgcn_readfirstlane(
        (unsigned)reinterpret_cast<uintptr_t>((lds_u8*)smem) + (unsigned)w * 1024u);
    auto dma_tile = [&](int t) __attribute__((always_inline)) {
      const int u0 = band_u0(t);
      const unsigned lk = lds_base + (unsigned)(t % NBUF) * RINGB;
      if (u0 >= 0) {
        const int srow = u0 * (int)rowbytes;   // uniform part of the offsets
        dma16(rkc, srow + vrk, lk);
        dma16(rvc, srow + vrv, lk + KTILEB);
      } else {
        const int P = max(s0 + u0 + rdma, 0);
        const int row = (P < nsink ? P : nsink + (P - nsink) % W) * (int)rowbytes;
        dma16(rks, row + dk, lk);
        dma16(rvs, row + dv, lk + KTILEB);
      }
    };
    // tiles 0 .. 3 in flight while Q is prepared; tiles 0 and 1 go through
    // registers when the work-group has sink tiles
    if (n_stile == 0) {
      dma_tile(0);
      dma_tile(1);
    } else {
      if (n_tiles > 0) {
        load_tile(0, stage);
        store_tile(0, stage);
      }
      if (n_tiles > 1) {
        load_tile(1, stage);
        store_tile(1, stage);
      }
    }
    dma_tile(2);
    dma_tile(3);

    // ---- Q prologue: rotated, scaled, rounded to bf16, in the B-operand layout ----
    // lane (i, g), step kk holds d = 8*(4kk+g) .. +7 of query tq, head h0+qb.
    // The softmax scale and log2(e) are applied before the rounding, so that
    // QK^T yields scores in the log2 domain directly.
    const float c2 = sh.scale_log2;
    bf16x8 qf[QB][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float cs[4], sn[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (sh.rope) {
          rope_cs(I, rope_rev[4 * (4 * kk + g) + jj], cs[jj], sn[jj]);
        } else {
          cs[jj] = 1.f;
          sn[jj] = 0.f;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (tq < C)
          wv = *reinterpret_cast<const u32x4*>(
              a.q + (((long long)b * C + tq) * sh.Hq + h0 + qb) * HD + 8 * (4 * kk + g));
        u32x4 r;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float x0 = bf16_lo(wv[jj]), x1 = bf16_hi(wv[jj]);
          rotate(x0, x1, cs[jj], sn[jj]);
          r[jj] = pack_bf16(x0 * c2, x1 * c2);
        }
        qf[qb][kk] = __builtin_bit_cast(bf16x8, r);
      }
    }

    // ---- softmax state of each query column (one per head qb) ----
    // ref[qb]: reference of the exponentials, the running max of the scores
    //          up to the lazy threshold; -inf until the column has seen a key.
    // The QK^T accumulator starts at -off (off = ref, or 0 while ref = -inf),
    // so the matrix core returns s = score - off and P = exp2(s).  A tile is
    // taken as is unless some s exceeds thr (kTau, or -inf while ref = -inf);
    // then the rare path moves ref to the new max, rescales O and l by
    // exp2(ref_old - ref_new) and shifts s.
    float ref[QB], thr[QB];
    floatx4 negoff[QB];
    floatx4 o[8][QB];
    // row sums of P accumulate on the matrix core: an all-ones A operand makes
    // every row of lsum[qb] the sum over keys of P for this lane's query
    floatx4 lsum[QB];
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      ref[qb] = -INFINITY;
      thr[qb] = -INFINITY;
      negoff[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
      lsum[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- operands and stages of one 32-key tile ----
    bf16x8 kop[2][4];   // K operand of the next QK^T: [kb][kk]
    bf16x8 vop[8];      // V^T operand of the next PV: [db]
    // K rows 16kb + i, d = 8(4kk+g) .. +7
    // lane offsets of the operand reads in a tile (rows 16 apart share a swizzle)
    int kofs[4], vofs[8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kofs[kk] = i * ROWB + 16 * ((4 * kk + g) ^ kswz(i));
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int r0 = 4 * g + (i >> 2);
      vofs[db] = r0 * ROWB + 16 * ((2 * db + ((i & 3) >> 1)) ^ vswz(r0)) + 8 * (i & 1);
    }
    auto read_k = [&](int t) __attribute__((always_inline)) {
      const uint8_t* Kb = smem + slot_off(t);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[kb][kk] = *reinterpret_cast<const bf16x8*>(Kb + kofs[kk] + 16 * kb * ROWB);
    };
    // Transposing reads: lane i of a 16-lane group addresses key base+i/4,
    // d 16db+4(i%4), and receives V[base+e][16db+i] for e = 0..3 (base = 4g,
    // then 16+4g), which is the A operand of O^T += V^T P^T.
    auto read_v = [&](int t) __attribute__((always_inline)) {
      lds_u8* Vb = (lds_u8*)smem + slot_off(t) + KTILEB;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(Vb + vofs[db]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(Vb + vofs[db] + 16 * ROWB));
        const v8i16 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        vop[db] = __builtin_bit_cast(bf16x8, va);
      }
    };
    // s[kb][qb] = K Q^T - off for heads q0, q0+1: rows = keys 16kb + 4g + r,
    // column = query i.  Four independent accumulation chains.
    auto qk_mma = [&](floatx4 (&s)[2][QB], int q0, int nq) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = q0; qb < q0 + nq; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][0], qf[qb][0], negoff[qb], 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < 4; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = q0; qb < q0 + nq; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb][kk], qf[qb][kk], s[kb][qb], 0, 0, 0);
    };
    // O^T += V^T P^T and l += 1 P^T for head qb
    auto pv_mma = [&](const bf16x8 (&p)[QB], int qb) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
        o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[db], p[qb], o[db][qb], 0, 0, 0);
      lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, p[qb], lsum[qb], 0, 0, 0);
    };
    // mask of tile j for this wave: 0 none, 1 band edge / diagonal, 2 sink tile.
    // Band tile j (keys u0 .. u0+31, u0 = t0 + 32(m + j)) needs no mask when
    // all its keys precede the wave's first query (u0 + 31 <= q0w), lie inside
    // the window of its last query (u0 > q0w + 15 - W) and exist (s0 + u0 >=
    // 0); each condition bounds j on one side, so the unmasked tiles are the
    // range jlo <= j <= jhi (>> 5 is the floor division by 32).
    const int mfull = kmin - n_stile, dq = q0w - t0;
    const int jhi = ((dq - (BN - 1)) >> 5) - mfull;
    const int jlo = max(max(n_stile, ((dq + 15 - W) >> 5) + 1 - mfull), -((s0 + t0) >> 5) - mfull);
    auto mask_kind = [&](int j) __attribute__((always_inline)) {
      if (j < n_stile) return 2;
      return (j >= jlo && j <= jhi) ? 0 : 1;
    };
    auto apply_mask = [&](int j, int mk, floatx4 (&s)[2][QB]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr_ = 16 * kb + 4 * g + r;
          bool ok;
          if (mk == 2) {
            const int P = BN * j + kr_;
            ok = P < nsink && P <= I - W;
          } else {
            const int u = band_u0(j) + kr_;
            ok = (u <= tq) && (u > tq - W) && (s0 + u >= 0);
          }
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = ok ? s[kb][qb][r] : -INFINITY;
        }
    };
    // P = exp2(s) of head qb, rounded to bf16 in the B-operand layout
    auto sexp = [&](const floatx4 (&s)[2][QB], bf16x8 (&p)[QB], int qb) __attribute__((always_inline)) {
      u32x4 pk;
      pk[0] = pack_bf16(__builtin_amdgcn_exp2f(s[0][qb][0]), __builtin_amdgcn_exp2f(s[0][qb][1]));
      pk[1] = pack_bf16(__builtin_amdgcn_exp2f(s[0][qb][2]), __builtin_amdgcn_exp2f(s[0][qb][3]));
      pk[2] = pack_bf16(__builtin_amdgcn_exp2f(s[1][qb][0]), __builtin_amdgcn_exp2f(s[1][qb][1]));
      pk[3] = pack_bf16(__builtin_amdgcn_exp2f(s[1][qb][2]), __builtin_amdgcn_exp2f(s[1][qb][3]));
      p[qb] = __builtin_bit_cast(bf16x8, pk);
    };
    // whether some s of head qb in this lane exceeds its column's threshold
    auto over = [&](const floatx4 (&s)[2][QB], int qb) __attribute__((always_inline)) {
      const float mx = __builtin_elementwise_maximum(vmax4(s[0][qb]), vmax4(s[1][qb]));
      return mx > thr[qb];
    };
    // the rare path: new references, rescaled O and l, shifted s
    auto rebase = [&](floatx4 (&s)[2][QB]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float off = -negoff[qb][0];
        const float cm = xg_max(__builtin_elementwise_maximum(vmax4(s[0][qb]), vmax4(s[1][qb]))) + off;
        const float nref = __builtin_elementwise_maximum(ref[qb], cm);
        if (nref > ref[qb] + kTau || (ref[qb] == -INFINITY && nref > -INFINITY)) {
          const float alpha = __builtin_amdgcn_exp2f(ref[qb] - nref);
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
          ref[qb] = nref;
        }
        const float noff = ref[qb] == -INFINITY ? 0.f : ref[qb];
        const float shift = noff - off;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb][qb] -= shift;
        negoff[qb] = floatx4{-noff, -noff, -noff, -noff};
        thr[qb] = ref[qb] == -INFINITY ? -INFINITY : kTau;
      }
    };

    // ---- software pipeline over tiles: two phases per tile ----
    // Matrix phase j: QK(j) (S of tile j, seeded with -off), then PV(j-1)
    // head by head, with K(j+1) and V(j) read from LDS into the operand
    // registers as the products release them.
    // Vector phase j: the mask and threshold checks of S(j), the rare rescale,
    // P(j) = exp2(S(j)), and the direct loads of tile j+4.  A barrier ends
    // every phase.  Waves 4..7 run one phase behind waves 0..3, so the two
    // waves of each SIMD (w and w+4) are always in different phases: one feeds
    // the matrix core and the LDS while the other uses the vector ALU.
    // Ring timing (phases counted from the first matrix phase of waves 0..3:
    // matrix phase j is phase 2j for those, 2j+1 for waves 4..7).  Every
    // barrier waits for all but the newest tile load of the wave, so tile t,
    // loaded in phases 2t-7 and 2t-6, is complete at the barrier ending phase
    // 2t-4 and visible before its first read (K(t) in phase 2t-2).  Its last
    // read (V(t), phase 2t+1) completes before the barrier ending the vector
    // phase that follows (lgkmcnt(0)), and the loads of tile t+8 into its slot
    // start in phase 2t+9.  Loads past the band read whatever the buffers hold
    // there (or zeros) and are never used.
    floatx4 s[2][QB];
    bf16x8 p[QB];
    auto mphase = [&](int j, bool qk, bool pv) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (qk) qk_mma(s, 0, QB);
      __builtin_amdgcn_sched_barrier(0);
      if (pv) {
        pv_mma(p, 0);
        if (qk) read_k(j + 1);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pv_mma(p, 1);
        if (qk) read_v(j);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      } else {
        read_k(j + 1);
        read_v(j);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto vphase = [&](int j) __attribute__((always_inline)) {
      const int mk = mask_kind(j);
      if (mk) apply_mask(j, mk, s);
      bool rare = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) rare |= over(s, qb);
      if (__builtin_expect(__any(rare), 0)) rebase(s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sexp(s, p, qb);
      // the empty asm keeps the exponentials in this phase
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(p[qb]));
      __builtin_amdgcn_sched_barrier(0);
      dma_tile(j + 4);
      ring_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    const bool lead = (w >> 2) == 0;
    __syncthreads();
    if (n_tiles > 0) {
      read_k(0);
      if (!lead) __builtin_amdgcn_s_barrier();
      mphase(0, true, false);
      vphase(0);
      for (int j = 1; j < n_tiles; ++j) {
        mphase(j, true, true);
        vphase(j);
      }
      mphase(n_tiles, false, true);
      if (lead) __builtin_amdgcn_s_barrier();
    }
    // the last tile loads must land before the work-group's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: O / l, LSE ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = lsum[qb][0];
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
          a.lse[((long long)b * sh.Hq + h0 + qb) * C + tq] = (ref[qb] + log2f(lt)) * 0.69314718055994531f;
      }
    }
  }  // items
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
      rope_cs(I, rt.rev[kk], cs, sn);
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

// Number of compute units of the current device (0 if unknown), cached per device.
static int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

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
  const long long n_items = (long long)a.n_qtiles * sh.Hkv * sh.B;
  if (n_items > INT32_MAX) return hipErrorInvalidValue;
  a.n_items = (int)n_items;
  // one work-group per CU (a multiple of 8), each looping over its items
  const long long ncu = (long long)(device_cu_count() & ~7);
  const long long nwg = (ncu >= 8 && n_items > ncu) ? ncu : n_items;
  prefill_bf16_d128_g4_kernel<<<dim3((unsigned)nwg), dim3(NTHR), 0, st>>>(a);
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
