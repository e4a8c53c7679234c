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
// Fast kernel (bf16, head_dim 128; written for the GQA group of 4, and
// taking groups of 1, 2 and 8 as described at the kernel), MI355X / gfx950:
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
//  * Key tiles of 32 keys in a 5-slot LDS ring.  Tiles outside the band
//    i-W < j <= i of the work-group are never visited, so the work is
//    O(N*W); only tiles that cut the diagonal or the window edge are
//    masked.  Tiles move global -> LDS directly (buffer loads with the lds
//    modifier, out-of-range rows read as zeros) four tiles ahead, as one
//    stream over all the items a work-group runs; the next item's query rows
//    wait in an LDS stage, so an item starts without waiting for memory.
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
//    stays in one XCD's L2.  Query tiles run longest-first; with more items
//    than CUs, one work-group per CU loops over its items.
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
constexpr int NBUF = 5;      // LDS ring of K/V tiles (the least the ring timing allows)
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
constexpr int QROWB = 4 * ROWB;          // the 4 query heads of one position
__device__ inline int kswz(int r) { return r & 15; }
__device__ inline int vswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// One direct global-to-LDS load: every lane's 16 bytes at byte offset `off`
// of the buffer `rsrc` (zeros when out of range) land at LDS address
// lds + 16 * lane.  M0 carries the LDS address; it is saved and restored
// around the load, and one wait state separates its write from the load.
// The compiler does not count these loads: the barriers of the tile loop
// wait for them (s_waitcnt vmcnt) explicitly.
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

// The K and the V row of one tile: as dma16, twice, with one save and
// restore of M0.  (The whole offset stays in the per-lane operand: the range
// check of a raw buffer does not cover the scalar offset, and rows past the
// end must read as zeros.)
__device__ inline void dma16x2(__amdgpu_buffer_rsrc_t rk, int ok, unsigned lk,
                               __amdgpu_buffer_rsrc_t rv, int ov, unsigned lv) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %5, %6, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lk), "v"(ok), "s"(rk), "s"(lv), "v"(ov), "s"(rv)
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
  int n_items;          // n_qtiles * Hkv * B, or the VarTab's item count
  uint16_t* out;
  float* lse;
  VarTab vt;            // packed sequences of their own lengths (varlen kernel)
};

// One work-group: 64 query positions x the 4 query heads of one KV head,
// 8 waves, two per SIMD.  Wave w owns positions t0 + 16(w&3) .. +15 for heads
// h0, h0+1 (h0 = 4 kvh + 2(w>>2)); lane (i, g) owns query column i of each
// of its heads.  Every K/V operand read from LDS feeds two matrix
// instructions (one per head).
//
// A work-group runs several items (sequence, KV head, query tile) one after
// the other.  The tile loads run ahead of the computation as one stream over
// all of the work-group's items: the last steps of an item already load the
// first tiles of the next one into the ring, and the next item's query rows
// go to an LDS stage while the current item runs, so that an item starts
// without waiting for memory.
//
// DIL (dilated window, no sinks): a query at i attends only keys j = i - k*dil,
// all of i's residue mod dil, so each residue class of a sequence's positions
// is plain sliding-window attention over its own rows (every dil-th row) with
// a window of ceil(W/dil) of them.  An item is then (sequence, KV head,
// residue, query tile); the band logic runs on a residue's decimated indices,
// RoPE and the cache slots on absolute positions.
//
// NC (fixed length, no sinks, and either no cache -- a first chunk, a whole
// prompt -- or a cache in slot order: every start a multiple of W, as when a
// prompt is prefilled from position 0 in chunks of W tokens).  A tile before
// the chunk then covers positions s0 + u0 .. s0 + u0 + 31 with u0 >= -W,
// which sit in slots u0 + W .. u0 + W + 31, so the sink and slot logic drops
// out.  With the scalar registers over-subscribed, the code without that
// logic places fewer of its spills in the tile loop: 1-1.5% on the
// 8192-token layer, 3-3.5% on a chunk that reads the cache.
//
// GQ, the query heads per KV head (1, 2, 4 or 8; DIL takes 4 only): an item
// always holds 4 query columns of 64 positions (the 4 "heads" of the stage
// and of the waves).  With 8, a KV head has two items per query tile
// (virtual heads 2 kvh and 2 kvh + 1, query heads 8 kvh .. +3 and +4 .. +7),
// which read the same K/V rows.  With 2, an item covers 128 positions of the
// group's 2 heads: column c is head c & 1 at positions t0 + 64 (c >> 1) ..,
// so waves 4..7 take the second 64 positions (their masks and band edges
// follow from their own positions; the item's tiles cover both blocks).
// With 1, the item's 4 columns are the group's head repeated and only the
// first is stored: 4 times the matrix work of the head.
template <bool VAR, bool DIL, bool NC, int GQ>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bf16_d128_g4_kernel(PrefillArgs a) {
  static_assert(GQ == 1 || GQ == 2 || GQ == 4 || GQ == 8, "group of 1, 2, 4 or 8 query heads");
  static_assert(GQ == 4 || !DIL, "a dilated window takes groups of 4");
  constexpr int GH = GQ < 4 ? GQ : 4;    // distinct query heads of an item
  constexpr int VS = GQ == 8 ? 1 : 0;    // items per (KV head, query tile): 1 << VS
  constexpr int PS = GQ == 2 ? 2 : 1;    // blocks of 64 positions per item
  constexpr int BMI = BM * PS;           // query positions per item
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * RINGB];
  __shared__ __attribute__((aligned(16))) uint8_t qstage[BM * QROWB];
  __shared__ double rope_rev[kMaxPairs];

  const Shape& sh = a.sh;
  const int tid = threadIdx.x;
  if (tid < kMaxPairs) rope_rev[tid] = a.rt.rev[tid];

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int C = a.C;
  const int W = sh.W;
  const int S = sh.S;
  const int nsink = NC ? 0 : sh.n_sink;
  const unsigned rowbytes = (unsigned)sh.Hkv * 2u * HD;   // bytes between tokens of K/V
  const unsigned qrowbytes = (unsigned)sh.Hq * 2u * HD;   // bytes between tokens of Q
  // DIL: the dilation, the window in a residue's rows, and the bytes between
  // a residue's consecutive rows of K/V and of Q
  const int dil = DIL ? sh.dil : 1;
  const int Wb = DIL ? (W + dil - 1) / dil : W;
  const unsigned rbd = DIL ? rowbytes * (unsigned)dil : rowbytes;
  const unsigned qrbd = DIL ? qrowbytes * (unsigned)dil : qrowbytes;

  // ---- work mapping ----
  // Items (sequence, KV head, query tile) are numbered sequence-major, KV
  // head next, query tiles longest first, and split into 8 contiguous
  // ranges, one per XCD (work-group w runs on XCD w mod 8), so that the K/V
  // of a KV head stays in one XCD's L2.  With one item per work-group the
  // hardware hands them out in that order; with fewer work-groups (one per
  // CU, a multiple of 8) each takes the items of its XCD's range in a
  // serpentine order over the rounds, which evens out the longest-first
  // lengths.  item_at(r) is the item of round r, or -1 past the last.
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  auto item_at = [&](int round) __attribute__((always_inline)) {
    int L = -1;
    if (G >= a.n_items) {
      const int q8 = G >> 3, r8 = G & 7;
      if (round == 0) L = xcd * q8 + min(xcd, r8) + (wg >> 3);
    } else {
      const int q8 = a.n_items >> 3, r8 = a.n_items & 7;
      const int lo = xcd * q8 + min(xcd, r8), cnt = q8 + (xcd < r8 ? 1 : 0);
      const int nl = G >> 3, li = wg >> 3;
      const int pos = round * nl + ((round & 1) ? nl - 1 - li : li);
      if (pos < cnt) L = lo + pos;
    }
    return L;
  };
  // An item's tiles: [sink tiles] + band tiles k = kmin..1 (keys u0 .. u0+31,
  // u0 = t0 + 32k).  Band tiles cover chunk-relative key positions
  // t0 - W + 1 .. t0 + 63; sink tiles cover absolute positions 0 ..
  // n_sink-1 for queries whose window no longer contains them.
  // Without caches (k_cache NULL) no position before the chunk exists: sa,
  // the number of positions before the chunk that can be read, is s0 with a
  // cache and 0 without, and keys below s0 - sa are outside every key set.
  struct Item {
    int b, kvh, t0, s0, sa, n_stile, kmin, n_tiles;
    int row0, len;   // varlen: the sequence's first packed row, its length
    int abs0;        // absolute position of row 0 (DIL: of the residue's first row)
  };
  // The start positions are read through the constant address space, so
  // that they come in with scalar loads, which the wait for the tile loads
  // (vector memory) does not cover.
  typedef __attribute__((address_space(4))) const int32_t c_i32;
  c_i32* start_c = (c_i32*)a.start;
  auto item_params = [&](int L) __attribute__((always_inline)) {
    Item it;
    if (VAR) {
      // the sequence whose items hold L: the number of sequences that end
      // at or before L, counted over the lanes
      int io_;
      {
        int ln_ = lane;
        asm volatile("" : "+v"(ln_));
        io_ = ln_ < a.vt.n ? a.vt.item_off[ln_ + 1] : INT_MAX;
      }
      it.b = __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(io_ <= L)));
      it.row0 = a.vt.row_off[it.b];
      it.len = a.vt.row_off[it.b + 1] - it.row0;
      const int nqt = (it.len + BMI - 1) / BMI;
      const int rem = L - a.vt.item_off[it.b];
      it.kvh = rem / nqt;
      it.t0 = (nqt - 1 - (rem - it.kvh * nqt)) * BMI;
    } else if (DIL) {
      // residue rho of sequence b: chunk rows r0, r0 + dil, ... (positions
      // = rho mod dil), decimated indices from s0 = (s0_abs + r0 - rho) / dil
      const int per_b = sh.Hkv * dil * a.n_qtiles;
      it.b = L / per_b;
      int rem = L - it.b * per_b;
      it.kvh = rem / (dil * a.n_qtiles);
      rem -= it.kvh * dil * a.n_qtiles;
      const int rho = rem / a.n_qtiles;
      it.t0 = (a.n_qtiles - 1 - (rem - rho * a.n_qtiles)) * BM;
      const int sabs = start_c[it.b];
      const int r0 = ((rho - sabs) % dil + dil) % dil;
      it.row0 = it.b * C + r0;
      it.len = r0 < C ? (C - r0 + dil - 1) / dil : 0;
      it.abs0 = sabs + r0;
      it.s0 = (sabs + r0 - rho) / dil;
    } else {
      const int per_b = (sh.Hkv << VS) * a.n_qtiles;   // items of a query tile: (virtual) heads
      it.b = L / per_b;
      const int rem = L - it.b * per_b;
      it.kvh = rem / a.n_qtiles;
      it.t0 = (a.n_qtiles - 1 - (rem - it.kvh * a.n_qtiles)) * BMI;
      it.row0 = it.b * C;
      it.len = C;
    }
    if (!DIL) it.s0 = start_c[it.b];
    it.sa = a.kc ? it.s0 : 0;
    const int tq_last = min(it.t0 + BMI, it.len) - 1;
    // sink tiles: some readable sink lies outside the window of some query
    it.n_stile = (!DIL && nsink > it.s0 - it.sa && tq_last - W + it.sa >= 0) ? (nsink + BN - 1) / BN : 0;
    const int k_lo = -((Wb - 1 + BN - 1) / BN);
    const int k_clip = -((it.sa + it.t0 + BN - 1) / BN);
    it.kmin = max(k_lo, k_clip);
    it.n_tiles = it.n_stile + (BMI / BN - it.kmin);
    return it;
  };

  // ---- the load stream: tiles global -> LDS ring, directly ----
  // Wave w fills rows 4w .. 4w+3 of the K and of the V tile: lane L loads the
  // chunk that belongs at position L%16 of row 4w + L/16 under the swizzle.
  // The descriptors (chunk or cache of the item being loaded) cover exactly
  // one KV head's rows of that tensor, so rows past its end read as zeros;
  // cache rows take the slot map, and rows before position 0 read slot 0
  // (they are masked).
  const int rdma = 4 * w + (lane >> 4);               // row of the tile this lane loads
  const int vrk = rdma * (int)rbd + 16 * ((lane & 15) ^ kswz(rdma));   // lane offsets
  const int vrv = rdma * (int)rbd + 16 * ((lane & 15) ^ vswz(rdma));   // in a chunk tile
  const unsigned lds_ring = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((lds_u8*)smem) + (unsigned)w * 1024u);
  const unsigned lds_q = __builtin_amdgcn_readfirstlane(
      (unsigned)reinterpret_cast<uintptr_t>((lds_u8*)qstage));
  const int nrec_c = (C - 1) * (int)rowbytes + HD * 2;
  const int nrec_s = a.kc ? (S - 1) * (int)rowbytes + HD * 2 : 0;
  const int nrec_q = (C - 1) * (int)qrowbytes + GH * ROWB;   // (the item's heads of the last row)

  // Cursor of the load stream: the item of round lr_round, its tile lt
  // (tiles past an item's end, once no item follows, load unused rows), and
  // the number of tiles loaded so far (the ring position of the next one).
  // Of the item only what the loads need is kept; the descriptors are made
  // at each load from the element offsets of its (sequence, KV head) rows.
  int lr_round = 0, lt = 0;
  unsigned lslot = 0;           // LDS offset of the ring slot the next load fills
  int l_nt, l_ns, l_u0, l_s0;   // tiles, sink tiles, u0 of the first band tile, start
  int l_a0 = 0;                 // DIL: absolute position of the item's row 0
  int l_nrec;                   // bytes of the item's rows of the chunk
  long long l_ec, l_es;         // element offset of the rows in the chunk, the cache
  auto rsrc = [&](const uint16_t* base, long long e, int nrec) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base + e), (short)0, nrec, 0x00020000);
  };
  // Descriptors of the rows the next straight-path tile reads: the item's
  // rows of the chunk's K and V (region 0) or of the caches (region 1; a
  // chunk without a cache has none: nrec_s = 0 reads zeros).  They are made
  // again only when the region changes, about twice per item, so that a
  // cache tile issues like a chunk tile.
  __amdgpu_buffer_rsrc_t rk, rv;
  int l_reg = -1;               // region rk / rv cover, -1 none
  auto use_region = [&](int reg) __attribute__((always_inline)) {
    if (reg != l_reg) {
      if (reg == 0) {
        rk = rsrc(a.kr, l_ec, l_nrec);
        rv = rsrc(a.v, l_ec, l_nrec);
      } else {
        const long long e = a.kc ? l_es : 0;
        rk = rsrc(a.kc ? a.kc : a.kr, e, nrec_s);
        rv = rsrc(a.vc ? a.vc : a.v, e, nrec_s);
      }
      l_reg = reg;
    }
  };
  int l_cm = -1;         // cache band tiles: see prepare()
  int l_cmn = -1;        // l_cm of the item's next tile when it is a cache band tile, or -1
  auto set_cursor = [&](int L) __attribute__((always_inline)) {
    const Item it = item_params(L);
    l_nt = it.n_tiles;
    l_ns = it.n_stile;
    l_u0 = it.t0 + BN * (it.kmin - it.n_stile);
    l_s0 = it.s0;
    if (DIL) l_a0 = it.abs0;
    const int kvh_ = it.kvh >> VS;   // the item's KV head
    l_ec = (VAR || DIL) ? ((long long)it.row0 * sh.Hkv + kvh_) * HD : ((long long)it.b * C * sh.Hkv + kvh_) * HD;
    l_es = ((long long)it.b * S * sh.Hkv + kvh_) * HD;
    l_nrec = (VAR || DIL) ? (it.len - 1) * (int)rbd + HD * 2 : nrec_c;
    l_reg = -1;
    l_cmn = -1;
  };
  set_cursor(item_at(0));
  // The next load is prepared one step ahead (prepare(), run while the
  // previous loads are awaited) and issued by issue(): band tiles of the
  // chunk and cache band tiles whose rows are consecutive slots, the common
  // cases, take the straight path with the uniform part of their offsets
  // (l_srow) and their region's descriptors ready.
  int l_slow = -1;       // >= 0 iff the next tile takes the straight path
  int l_srow = 0;        // its uniform byte offset
  auto prepare = [&]() __attribute__((always_inline)) {
    if (lt >= l_nt) {
      const int L = item_at(lr_round + 1);
      if (L >= 0) {
        ++lr_round;
        set_cursor(L);
        lt = 0;
      }
    }
    const int u0 = l_u0 + BN * lt;
    int reg = -1, srow = 0;
    if (lt >= l_ns) {
      if (u0 >= 0) {
        reg = 0;                                   // band tile of the chunk
        srow = u0 * (int)rbd;
      } else {
        // cache band tile: the rolling-buffer slot of the wave's first row,
        // less n_sink, when all its rows lie past the sinks; consecutive
        // cache tiles of an item are 32 slots apart
        const int P0 = (DIL ? l_a0 : l_s0) + dil * (u0 + 4 * w);
        if (NC) {
          // slot order: row u0 + W of the cache (without a cache no tile
          // precedes the chunk)
          reg = 1;
          srow = (u0 + W) * (int)rowbytes;
        } else if (P0 >= nsink) {
          l_cm = l_cmn >= 0 ? l_cmn : (int)((unsigned)(P0 - nsink) % (unsigned)W);
          const int nx = l_cm + BN * dil >= W ? l_cm + BN * dil - W : l_cm + BN * dil;
          l_cmn = nx < W ? nx : -1;
          if (l_cm + 3 * dil < W) {
            // its 4 rows per wave are slots dil apart (consecutive without dilation)
            reg = 1;
            srow = DIL ? (nsink + l_cm) * (int)rowbytes - 4 * w * (int)rbd : (nsink + l_cm - 4 * w) * (int)rowbytes;
          }
        } else {
          l_cm = -1;
        }
      }
    }
    l_slow = __builtin_amdgcn_readfirstlane(reg);
    l_srow = __builtin_amdgcn_readfirstlane(srow);
    asm volatile("" : "+s"(l_slow), "+s"(l_srow));   // (computed here, in the wait's shadow)
    if (l_slow >= 0) use_region(l_slow);
  };
  // load the prepared tile into its ring slot
  auto issue = [&]() __attribute__((always_inline)) {
    const unsigned lk = lds_ring + lslot;
    if (__builtin_expect(l_slow >= 0, 1)) {
      dma16x2(rk, l_srow + vrk, lk, rv, l_srow + vrv, lk + KTILEB);
    } else {
      // (lane offsets recomputed here rather than held in registers)
      int ln_ = lane;
      asm volatile("" : "+v"(ln_));
      const int r = ln_ >> 4, rd = 4 * w + r;
      const int dk_ = 16 * ((ln_ & 15) ^ kswz(rd)), dv_ = 16 * ((ln_ & 15) ^ vswz(rd));
      if (lt < l_ns) {
        // sink tile: absolute positions 32 lt + r (clamped to the last sink);
        // those before the item's chunk come from the cache, the rest from
        // the chunk
        const int P = min(BN * lt + rd, nsink - 1);
        if (P < l_s0 && a.kc != nullptr) {
          dma16(rsrc(a.kc, l_es, nrec_s), P * (int)rowbytes + dk_, lk);
          dma16(rsrc(a.vc, l_es, nrec_s), P * (int)rowbytes + dv_, lk + KTILEB);
        } else {
          const int rr = min(max(P - l_s0, 0), C - 1) * (int)rowbytes;
          dma16(rsrc(a.kr, l_ec, l_nrec), rr + dk_, lk);
          dma16(rsrc(a.v, l_ec, l_nrec), rr + dv_, lk + KTILEB);
        }
      } else {
        // cache rows (a chunk without a cache has none: nrec_s = 0 reads zeros)
        int sl;
        if (l_cm >= 0) {
          sl = l_cm + dil * r;
          sl = nsink + (DIL ? sl % W : (sl >= W ? sl - W : sl));
        } else {
          const int P = max((DIL ? l_a0 : l_s0) + dil * (l_u0 + BN * lt + rd), 0);
          sl = P < nsink ? P : nsink + (P - nsink) % W;
        }
        const int row = sl * (int)rowbytes;
        const uint16_t* kcb = a.kc ? a.kc : a.kr;
        const uint16_t* vcb = a.vc ? a.vc : a.v;
        dma16x2(rsrc(kcb, a.kc ? l_es : 0, nrec_s), row + dk_, lk,
                rsrc(vcb, a.kc ? l_es : 0, nrec_s), row + dv_, lk + KTILEB);
      }
    }
    ++lt;
    lslot = lslot + RINGB == NBUF * RINGB ? 0u : lslot + RINGB;
  };
  // Query rows of an item -> the LDS stage (64 positions x 1 KB: the 4 query
  // heads of the KV head).  Wave w loads positions 8w .. 8w+7; the 16-byte
  // chunk c of position q sits at c ^ (q & 15), so the 16 positions one
  // operand read touches fall in 16 different bank groups.  Rows past the
  // chunk read as zeros.
  auto load_q = [&](const Item& it) __attribute__((always_inline)) {
    const long long qrow = (VAR || DIL) ? (long long)it.row0 : (long long)it.b * C;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a.q + (qrow * sh.Hq + GH * it.kvh) * HD), (short)0,
        (VAR || DIL) ? (it.len - 1) * (int)qrbd + GH * ROWB : nrec_q, 0x00020000);
    int ln_ = lane;   // (computed here, not held in registers across the loop)
    asm volatile("" : "+v"(ln_));
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int q = 8 * w + m;
      if constexpr (PS == 2) {
        // stage column ln_ / 16 = c: head c & 1 at position t0 + q + 64 (c >> 1)
        const int src = (((ln_ >> 4) & 1) << 4) | ((ln_ ^ q) & 15);
        dma16(rq, (it.t0 + q + 64 * (ln_ >> 5)) * (int)qrbd + 16 * src, lds_q + (unsigned)q * QROWB);
      } else if constexpr (GQ < 4) {
        // the chunk of stage position ln_: head ln_ / 16 mod GQ, swizzled
        const int src = (((ln_ >> 4) & (GQ - 1)) << 4) | ((ln_ ^ q) & 15);
        dma16(rq, (it.t0 + q) * (int)qrbd + 16 * src, lds_q + (unsigned)q * QROWB);
      } else {
        dma16(rq, (it.t0 + q) * (int)qrbd + 16 * (ln_ ^ (q & 15)), lds_q + (unsigned)q * QROWB);
      }
    }
  };

  // the first item's query rows and the first four tiles of the stream
  {
    const int L0 = item_at(0);
    load_q(item_params(L0));
  }
  prepare();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    issue();
    prepare();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- operand reads ----
  // K rows 16kb + i, d = 8(4kk+g) .. +7; lane offsets of the operand reads in
  // a tile (rows 16 apart share a swizzle)
  int kofs[4], vofs[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) kofs[kk] = i * ROWB + 16 * ((4 * kk + g) ^ kswz(i));
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int r0 = 4 * g + (i >> 2);
    vofs[db] = r0 * ROWB + 16 * ((2 * db + ((i & 3) >> 1)) ^ vswz(r0)) + 8 * (i & 1);
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const float c2 = sh.scale_log2;
  const bool lead = (w >> 2) == 0;

  // ---- Q from the stage: rotated, scaled, rounded to bf16, in the B-operand layout ----
  // lane (i, g), step kk holds d = 8*(4kk+g) .. +7 of query t0 + 16(w&3) + i,
  // head 4 kvh + 2(w>>2) + qb.  The softmax scale and log2(e) are applied
  // before the rounding, so that QK^T yields scores in the log2 domain
  // directly.
  bf16x8 qf[QB][4];
  auto load_qf = [&](const Item& it) __attribute__((always_inline)) {
    // the lane's query position (PS = 2: waves 4..7 take the item's second 64)
    const int I = (DIL ? it.abs0 : it.s0) + dil * (it.t0 + (PS == 2 ? 64 * (w >> 2) : 0) + 16 * (w & 3) + i);
    // (the asm keeps the table addresses from being computed once for all
    // items and held in registers)
    int gi = g;
    asm volatile("" : "+v"(gi));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // without RoPE every rev is 0: the rotation is the identity
      float cs[4], sn[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) rope_cs(I, rope_rev[4 * (4 * kk + gi) + jj], cs[jj], sn[jj]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int c = 16 * (QB * (w >> 2) + qb) + 4 * kk + g;
        const u32x4 wv = *reinterpret_cast<const u32x4*>(qstage + (16 * (w & 3) + i) * QROWB + 16 * (c ^ i));
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
  };

  unsigned base = 0;   // stream position of the current item's first tile
  int L = item_at(0);
  Item it = item_params(L);
  load_qf(it);
  for (int round = 0;; ++round) {
    const int b = it.b, kvh = it.kvh, t0 = it.t0, s0 = it.s0, sa = it.sa;
    const int n_stile = it.n_stile, kmin = it.kmin, n_tiles = it.n_tiles;
    const int q0w = t0 + (PS == 2 ? 64 * (w >> 2) : 0) + 16 * (w & 3);   // first query of this wave (chunk-relative)
    const int tq = q0w + i;                 // this lane's query
    const int I = (DIL ? it.abs0 : s0) + dil * tq;   // its absolute position
    const int h0 = kvh * GH + (PS == 2 ? 0 : QB * (w >> 2)); // first query head of this wave
    // the next item, whose query rows go to the stage during this item
    const int Ln = item_at(round + 1);
    auto band_u0 = [&](int t) __attribute__((always_inline)) { return t0 + BN * (kmin + t - n_stile); };

    // ---- softmax state of each query column (one per head qb) ----
    // ref[qb]: reference of the exponentials, the running max of the scores
    //          up to the lazy threshold; -inf until the column has seen a key.
    // The QK^T accumulator starts at -off (off = ref, or 0 while ref = -inf),
    // so the matrix core returns s = score - off and P = exp2(s).  A tile is
    // taken as is unless some s exceeds thr (kTau, or -inf while ref = -inf);
    // then the rare path moves ref to the new max, rescales O and l by
    // exp2(ref_old - ref_new) and shifts s.
    float ref[QB], thr[QB];
    float thrm = -INFINITY;   // min(thr[0], thr[1])
    floatx4 negoff[QB];
    floatx4 o[8][QB];
    // row sums of P accumulate on the matrix core: an all-ones A operand makes
    // every row of lsum[qb] the sum over keys of P for this lane's query
    floatx4 lsum[QB];
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
    // Byte offset of tile t's ring slot.  The empty asm hides the value's
    // origin from loop strength reduction, which would otherwise keep one
    // induction variable per LDS address instead of folding the constant
    // parts into the instructions' offset fields.
    // Ring offsets of tile j (cur) and tile j+1 (nxt) in matrix phase j;
    // matrix phase j > 0 advances them after its QK^T products, while those
    // still execute.
    unsigned cur = (base % NBUF) * RINGB;
    unsigned nxt = cur + RINGB == NBUF * RINGB ? 0u : cur + RINGB;
    auto advance = [&]() __attribute__((always_inline)) {
      cur = nxt;
      nxt = nxt + RINGB == NBUF * RINGB ? 0u : nxt + RINGB;
      asm volatile("" : "+s"(cur), "+s"(nxt));
    };
    auto slot_off = [&](unsigned o) __attribute__((always_inline)) {
      asm volatile("" : "+s"(o));
      return o;
    };
    auto read_k = [&](unsigned so) __attribute__((always_inline)) {
      const uint8_t* Kb = smem + slot_off(so);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[kb][kk] = *reinterpret_cast<const bf16x8*>(Kb + kofs[kk] + 16 * kb * ROWB);
    };
    // Transposing reads: lane i of a 16-lane group addresses key base+i/4,
    // d 16db+4(i%4), and receives V[base+e][16db+i] for e = 0..3 (base = 4g,
    // then 16+4g), which is the A operand of O^T += V^T P^T.
    auto read_v = [&](unsigned so) __attribute__((always_inline)) {
      lds_u8* Vb = (lds_u8*)smem + slot_off(so) + KTILEB;
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
    const int jlo = max(max(n_stile, ((dq + 15 - Wb) >> 5) + 1 - mfull), -((sa + t0) >> 5) - mfull);
    auto mask_kind = [&](int j) __attribute__((always_inline)) {
      if (j < n_stile) return 2;
      return (j >= jlo && j <= jhi) ? 0 : 1;
    };
    // Each kind is one interval test per key: sink key P (absolute) is kept
    // iff s0 - sa <= P <= min(n_sink - 1, I - W); band key u (chunk-relative)
    // iff max(tq - W + 1, -sa) <= u <= tq (a non-empty interval: tq >= 0 >= -sa).
    auto apply_mask = [&](int j, int mk, floatx4 (&s)[2][QB]) __attribute__((always_inline)) {
      int k0, lo, span;   // key index of row 0 of this lane, interval [lo, lo + span]
      if (mk == 2) {
        k0 = BN * j + 4 * g;
        lo = a.kc ? INT_MIN / 2 : s0;
        span = min(nsink - 1, I - W) - lo;
        if (span < 0) {   // (no readable sink for this query: a one-key interval no key is in)
          lo = INT_MIN / 2 + 1;
          span = 0;
        }
      } else {
        k0 = band_u0(j) + 4 * g;
        lo = max(tq - Wb + 1, -sa);
        span = tq - lo;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (unsigned)(k0 + 16 * kb + r - lo) <= (unsigned)span;
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
    // v_maximum3_f32 (IEEE maximum, NaN-propagating, of three)
    auto mx3 = [](float x, float y, float z) __attribute__((always_inline)) {
      float m;
      asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(m) : "v"(x), "v"(y), "v"(z));
      return m;
    };
    // Whether some s in this lane may exceed its column's threshold: the
    // largest s of both heads against the smaller threshold (a head whose
    // reference is still -inf sends every tile to the rare path, which checks
    // each head on its own); 8 three-input maxima for the 16 values.
    auto over2 = [&](const floatx4 (&s)[2][QB]) __attribute__((always_inline)) {
      const floatx4 &a0 = s[0][0], &a1 = s[1][0], &b0 = s[0][1], &b1 = s[1][1];
      const float u0 = mx3(a0[0], a0[1], a0[2]), u1 = mx3(a0[3], a1[0], a1[1]);
      const float u2 = mx3(a1[2], a1[3], b0[0]), u3 = mx3(b0[1], b0[2], b0[3]);
      const float u4 = mx3(b1[0], b1[1], b1[2]);
      const float v0 = mx3(u0, u1, u2), v1 = mx3(u3, u4, b1[3]);
      return __builtin_elementwise_maximum(v0, v1) > thrm;
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
      thrm = __builtin_elementwise_minimum(thr[0], thr[1]);
    };

    // ---- software pipeline over tiles: two phases per tile ----
    // Matrix phase j: QK(j) (S of tile j, seeded with -off), then PV(j-1)
    // head by head, with K(j+1) and V(j) read from LDS into the operand
    // registers as the products release them.
    // Vector phase j: the mask and threshold checks of S(j), the rare rescale,
    // P(j) = exp2(S(j)), and the load of the stream's next tile (tile j+4 of
    // this item, or an early tile of the next).  A barrier ends every phase.
    // Waves 4..7 run one phase behind waves 0..3, so the two waves of each
    // SIMD (w and w+4) are always in different phases: one feeds the matrix
    // core and the LDS while the other uses the vector ALU.
    // Ring timing, counted in stream tiles T and in phases from the first
    // matrix phase of waves 0..3 (matrix phase j is phase 2j for those, 2j+1
    // for waves 4..7; the barriers between items only add phases).  Tile T
    // is loaded in the vector phase of tile T-4 (phases 2T-7 / 2T-6).  The
    // barrier ending every vector phase waits for all but the wave's newest
    // tile load, so T is complete at the barrier ending phase 2T-4 and
    // visible before its first read (K(T) in phase 2T-2).  Its last read (V(T),
    // phases 2T / 2T+1) completes before the barrier ending phase 2T+2
    // (lgkmcnt(0)), and the load of tile T+5 into its slot starts in phase
    // 2T+3.  The barriers ending matrix phases need no memory wait: no load
    // is issued in a matrix phase.
    floatx4 s[2][QB];
    bf16x8 p[QB];
    auto mphase = [&](int j, bool qk, bool pv) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (qk) qk_mma(s, 0, QB);
      __builtin_amdgcn_sched_barrier(0);
      if (j > 0) advance();
      if (pv) {
        pv_mma(p, 0);
        if (qk) read_k(nxt);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pv_mma(p, 1);
        if (qk) read_v(cur);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      } else {
        read_k(nxt);
        read_v(cur);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // masked: 0 no mask, 1 the mask kind is looked up, 2 a band-edge or sink mask
    auto vphase = [&](int j, bool first, int masked) __attribute__((always_inline)) {
      if (masked == 1) {
        const int mk = mask_kind(j);
        if (mk) apply_mask(j, mk, s);
      } else if (masked == 2) {
        apply_mask(j, j < n_stile ? 2 : 1, s);
      }
      if (__builtin_expect(__any(over2(s)), 0)) rebase(s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sexp(s, p, qb);
      // the empty asm keeps the exponentials in this phase
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(p[qb]));
      __builtin_amdgcn_sched_barrier(0);
      issue();
      prepare();
      if (first && Ln >= 0) {
        // The stage was read before the barrier that opened this item.  The
        // 8 query-row loads are younger than the tile load, so this barrier
        // still completes everything but the newest tile; the next vector
        // phase's barrier completes them.
        load_q(item_params(Ln));
        asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // all waves are done with the stage (and the previous item's operands)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_k(cur);
    if (!lead) __builtin_amdgcn_s_barrier();
    mphase(0, true, false);
    vphase(0, true, 1);
    // tiles 1 .. n-1: masked below jlo, unmasked jlo .. jhi, masked above
    const int ju = min(max(jlo, 1), n_tiles), jv = min(max(jhi + 1, ju), n_tiles);
    int j = 1;
    for (; j < ju; ++j) {
      mphase(j, true, true);
      vphase(j, false, 2);
    }
    for (; j < jv; ++j) {
      mphase(j, true, true);
      vphase(j, false, 0);
    }
    for (; j < n_tiles; ++j) {
      mphase(j, true, true);
      vphase(j, false, 2);
    }
    mphase(n_tiles, false, true);
    if (lead) __builtin_amdgcn_s_barrier();

    // ---- switch: the next item's query rows leave the stage, O / l goes
    // through it.  O is written to the stage as bf16 rows (the layout of
    // the query rows), so that each wave then stores whole 1 KB rows (the 4
    // heads of one position) to memory.
    Item itn = it;
    if (Ln >= 0) {
      itn = item_params(Ln);
      load_qf(itn);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // (lane indices through an empty asm: the addresses below are computed
    // here, not held in registers across the tile loop)
    int li_ = lane;
    asm volatile("" : "+v"(li_));
    const int ii = li_ & 15, gg = li_ >> 4;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float inv = 1.f / lsum[qb][0];
      uint8_t* row = qstage + (16 * (w & 3) + ii) * QROWB + 8 * (gg & 1);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int c = 16 * (QB * (w >> 2) + qb) + 2 * db + (gg >> 1);
        const u32x2 val = {pack_bf16(o[db][qb][0] * inv, o[db][qb][1] * inv),
                           pack_bf16(o[db][qb][2] * inv, o[db][qb][3] * inv)};
        *reinterpret_cast<u32x2*>(row + 16 * (c ^ ii)) = val;
      }
      if (a.lse && g == 0 && tq < it.len && (GQ >= 4 || PS == 2 || QB * (w >> 2) + qb < GQ)) {
        const long long lo = VAR ? (long long)(h0 + qb) * a.vt.total + it.row0 + tq
                             : DIL ? ((long long)b * sh.Hq + h0 + qb) * C + (it.row0 - b * C) + dil * tq
                                   : ((long long)b * sh.Hq + h0 + qb) * C + tq;
        a.lse[lo] = (ref[qb] + log2f(lsum[qb][0])) * 0.69314718055994531f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    {
      uint16_t* orow = a.out + (((VAR || DIL) ? (long long)it.row0 : (long long)b * C) * sh.Hq + GH * kvh) * HD;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int q = 8 * w + m;
        if constexpr (PS == 2) {
          // stage column li_ / 16 = c: head c & 1 at position t0 + q + 64 (c >> 1)
          const int row = t0 + q + 64 * (li_ >> 5);
          if (row < it.len) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(qstage + q * QROWB + 16 * li_);
            *reinterpret_cast<u32x4*>(orow + (long long)row * sh.Hq * HD + 128 * ((li_ >> 4) & 1) +
                                      8 * ((li_ ^ q) & 15)) = v;
          }
        } else if (t0 + q < it.len && (GQ >= 4 || (li_ >> 4) < GQ)) {   // (the repeated heads are not stored)
          const u32x4 v = *reinterpret_cast<const u32x4*>(qstage + q * QROWB + 16 * li_);
          *reinterpret_cast<u32x4*>(orow + (long long)(t0 + q) * dil * sh.Hq * HD + 8 * (li_ ^ (q & 15))) = v;
        }
      }
    }
    base += (unsigned)n_tiles;
    if (Ln < 0) break;
    it = itn;
    L = Ln;
  }  // items
  // the stream's last loads must land before the work-group's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Generic kernel: 16 lanes per (query position, query head); a work-group of
// 4 queries shares its key tiles in LDS.
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

// Sum over the 16 lanes of a DPP row, in every lane of the row: quad
// butterflies (lane ^ 1, lane ^ 2), then the half-row and the row mirrors.
template <int CTRL>
__device__ inline float dpp_f(float y) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), CTRL, 0xF, 0xF, true));
}
__device__ inline float row16_sum(float x) {
  x += dpp_f<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);   // row_half_mirror
  x += dpp_f<0x140>(x);   // row_mirror
  return x;
}

template <bool F32, int D>
__global__ void __launch_bounds__(64) prefill_generic_kernel(Shape sh, RopeTab rt, const void* q,
                                                             const void* kr, const void* v,
                                                             const void* kc, const void* vc,
                                                             const int32_t* start, int C, void* out,
                                                             float* lse, VarTab vt) {
  // One work-group (one wave) per GQ = 4 consecutive queries of one head;
  // 16 lanes per query, each owning DP = D/16 elements of q and o, so that a
  // score is 16 short partial dots and a 4-step reduction.  The candidate
  // keys of the 4 queries (the sinks below the first query's window, then
  // the union of the windows) stream through LDS in tiles of TK keys loaded
  // by the whole wave.
  constexpr int GQ = 4, TK = 32, DP = D / 16;
  __shared__ float ks[TK][D], vs[TK][D];
  const int tid = threadIdx.x, qi = tid >> 4, part = tid & 15;
  const int t_first = blockIdx.x * GQ, t = t_first + qi;
  const int h = blockIdx.y, b = blockIdx.z;
  // the sequence's rows: b * C .. + C, or its packed run (vt.n > 0)
  const long long r0 = vt.n ? (long long)vt.row_off[b] : (long long)b * C;
  const int len = vt.n ? vt.row_off[b + 1] - vt.row_off[b] : C;
  if (t_first >= len) return;   // (uniform: the whole work-group)
  const bool active = t < len;
  const int kvh = h / (sh.Hq / sh.Hkv);
  const int s0 = start[b];
  const int tq = active ? t : t_first;
  const int I = s0 + tq;
  float qv[DP];
  const long long qoff = ((r0 + tq) * sh.Hq + h) * D + part * DP;
#pragma unroll
  for (int d = 0; d < DP; ++d) qv[d] = ld<F32>(q, qoff + d);
  if (sh.rope) {
#pragma unroll
    for (int kk = 0; kk < DP / 2; ++kk) {
      float cs, sn;
      rope_cs(I, rt.rev[part * DP / 2 + kk], cs, sn);
      rotate(qv[2 * kk], qv[2 * kk + 1], cs, sn);
    }
  }
  if (!F32) {
    // the matrix path multiplies bf16 operands: round the rotated query alike
#pragma unroll
    for (int d = 0; d < DP; ++d) qv[d] = __uint_as_float(((uint32_t)to_bf16_bits(qv[d])) << 16);
  }
  float o[DP];
#pragma unroll
  for (int d = 0; d < DP; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  // candidate keys: [0, min(n_sink, wlo)) and [wlo, I_last]
  const int I_last = s0 + min(t_first + GQ - 1, len - 1);
  const int wlo = max(0, s0 + t_first - sh.W + 1);
  auto run = [&](int lo, int hi) {   // keys lo .. hi (inclusive)
    for (int j0 = lo; j0 <= hi; j0 += TK) {
      __syncthreads();   // the previous tile is consumed
      for (int e = tid; e < TK * D; e += 64) {
        const int kk = e / D, d = e - kk * D, j = j0 + kk;
        float kx = 0.f, vx = 0.f;
        if (j <= hi && (j >= s0 || kc)) {
          // a key of the chunk, or of the cache as it stood before the chunk
          const bool ch = j >= s0;
          const long long off = ch ? ((r0 + (j - s0)) * sh.Hkv + kvh) * D
                                   : (((long long)b * sh.S + slot_of(j, sh.W, sh.n_sink)) * sh.Hkv + kvh) * D;
          kx = ld<F32>(ch ? kr : kc, off + d);
          vx = ld<F32>(ch ? v : vc, off + d);
        }
        ks[kk][d] = kx;
        vs[kk][d] = vx;
      }
      __syncthreads();
      const int nk = min(TK, hi - j0 + 1);
      for (int kk = 0; kk < nk; ++kk) {
        const int j = j0 + kk;
        float sc = 0.f;
#pragma unroll
        for (int d = 0; d < DP; ++d) sc = fmaf(qv[d], ks[kk][part * DP + d], sc);
        sc = row16_sum(sc);   // the 16 lanes of the query add their partial dots
        if (!active || !key_in_set(I, j, sh.W, sh.n_sink, sh.dil) || (j < s0 && !kc)) continue;
        sc *= sh.scale_log2;
        const float mn = fmaxf(m, sc);
        const float al = (m == -INFINITY) ? 0.f : exp2f(m - mn);
        const float pp = exp2f(sc - mn);
        l = l * al + pp;
#pragma unroll
        for (int d = 0; d < DP; ++d) o[d] = fmaf(o[d], al, pp * vs[kk][part * DP + d]);
        m = mn;
      }
    }
  };
  run(0, min(sh.n_sink, wlo) - 1);
  run(wlo, I_last);
  if (!active) return;
  const float inv = 1.f / l;
  const long long ooff = ((r0 + t) * sh.Hq + h) * D + part * DP;
#pragma unroll
  for (int d = 0; d < DP; ++d) st<F32>(out, ooff + d, o[d] * inv);
  if (lse && part == 0) {
    const long long lo = vt.n ? (long long)h * vt.total + r0 + t : ((long long)b * sh.Hq + h) * C + t;
    lse[lo] = (m + log2f(l)) * 0.69314718055994531f;
  }
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
                                       float* lse, const VarTab* vt, hipStream_t st, bool aligned) {
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
  const bool dil = sh.dil > 1 && !vt;   // (the API sends dilated varlen batches to the generic kernel)
  const int rows = dil ? (C + sh.dil - 1) / sh.dil : C;   // the longest residue's rows
  const int gq = sh.Hq / sh.Hkv;
  if (sh.Hq != gq * sh.Hkv || (gq != 1 && gq != 2 && gq != 4 && gq != 8) || (dil && gq != 4))
    return hipErrorInvalidValue;
  const int bmi = gq == 2 ? 2 * BM : BM;   // query positions per item (a group of 2: two blocks)
  a.n_qtiles = (rows + bmi - 1) / bmi;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  const int nvh = gq == 8 ? 2 * sh.Hkv : sh.Hkv;   // items per (sequence, query tile)
  long long n_items = (long long)a.n_qtiles * nvh * sh.B * (dil ? sh.dil : 1);
  if (vt) {
    // items of sequence j: nvh x its own query tiles, numbered after those of 0 .. j-1
    a.vt = *vt;
    a.vt.item_off[0] = 0;
    for (int j = 0; j < vt->n; ++j) {
      const int len = vt->row_off[j + 1] - vt->row_off[j];
      const int qt = (vt->skip_len1 && len == 1) ? 0 : (len + bmi - 1) / bmi;
      const long long next = a.vt.item_off[j] + (long long)nvh * qt;
      if (next > INT32_MAX) return hipErrorInvalidValue;
      a.vt.item_off[j + 1] = (int)next;
    }
    n_items = a.vt.item_off[vt->n];
    if (n_items == 0) return hipSuccess;
  } else {
    a.vt = VarTab{};
  }
  if (n_items > INT32_MAX) return hipErrorInvalidValue;
  a.n_items = (int)n_items;
  // one work-group per CU (a multiple of 8), each looping over its items
  const long long ncu = (long long)(device_cu_count() & ~7);
  const long long nwg = (ncu >= 8 && n_items > ncu) ? ncu : n_items;
  const dim3 grid((unsigned)nwg), block(NTHR);
  const bool nc = (a.kc == nullptr || aligned) && sh.n_sink == 0;
  switch (gq) {
    case 4:
      if (vt)
        prefill_bf16_d128_g4_kernel<true, false, false, 4><<<grid, block, 0, st>>>(a);
      else if (dil)
        prefill_bf16_d128_g4_kernel<false, true, false, 4><<<grid, block, 0, st>>>(a);
      else if (nc)
        prefill_bf16_d128_g4_kernel<false, false, true, 4><<<grid, block, 0, st>>>(a);
      else
        prefill_bf16_d128_g4_kernel<false, false, false, 4><<<grid, block, 0, st>>>(a);
      break;
    case 8:
      if (vt)
        prefill_bf16_d128_g4_kernel<true, false, false, 8><<<grid, block, 0, st>>>(a);
      else if (nc)
        prefill_bf16_d128_g4_kernel<false, false, true, 8><<<grid, block, 0, st>>>(a);
      else
        prefill_bf16_d128_g4_kernel<false, false, false, 8><<<grid, block, 0, st>>>(a);
      break;
    case 2:
      if (vt)
        prefill_bf16_d128_g4_kernel<true, false, false, 2><<<grid, block, 0, st>>>(a);
      else if (nc)
        prefill_bf16_d128_g4_kernel<false, false, true, 2><<<grid, block, 0, st>>>(a);
      else
        prefill_bf16_d128_g4_kernel<false, false, false, 2><<<grid, block, 0, st>>>(a);
      break;
    default:
      if (vt)
        prefill_bf16_d128_g4_kernel<true, false, false, 1><<<grid, block, 0, st>>>(a);
      else if (nc)
        prefill_bf16_d128_g4_kernel<false, false, true, 1><<<grid, block, 0, st>>>(a);
      else
        prefill_bf16_d128_g4_kernel<false, false, false, 1><<<grid, block, 0, st>>>(a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_generic(const Shape& sh, const RopeTab& rt, bool f32, const void* q,
                                  const void* k_rot, const void* v, const void* kc,
                                  const void* vc, const int32_t* start, int C, void* out,
                                  float* lse, const VarTab* vt, hipStream_t st) {
  dim3 grid((C + 3) / 4, sh.Hq, sh.B);   // 4 queries per work-group
  const VarTab none{};
  const VarTab& t = vt ? *vt : none;
  if (f32) {
    if (sh.D == 64)
      prefill_generic_kernel<true, 64><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse, t);
    else
      prefill_generic_kernel<true, 128><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse, t);
  } else {
    if (sh.D == 64)
      prefill_generic_kernel<false, 64><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse, t);
    else
      prefill_generic_kernel<false, 128><<<grid, 64, 0, st>>>(sh, rt, q, k_rot, v, kc, vc, start, C, out, lse, t);
  }
  return hipGetLastError();
}

}  // namespace swa
