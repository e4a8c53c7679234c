// swa_device.hpp — device-side index math, RoPE and bf16 helpers shared by
// every libswa kernel, so that the slot map, the key-set predicate and the
// rotation are one definition on the GPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxPairs = 64;  // head_dim <= 128

// Shape and constants of one call, passed by value to every kernel.
struct Shape {
  int B, Hq, Hkv, D, W, n_sink, S;
  int dil;          // dilation of the window part (1: plain SWA)
  float scale;      // softmax scale (already defaulted to 1/sqrt(D))
  float scale_log2; // scale * log2(e)
  int rope;         // 0: no RoPE
};

// RoPE frequencies theta^(-2k/D), k < D/2, in revolutions per position
// (divided by 2 pi), formed in double on the host.
struct RopeTab {
  double rev[kMaxPairs];
};

// ---------------------------------------------------------------------------
// Rolling-buffer index math.  slot(p) = p mod W, with the first n_sink
// positions pinned to slots 0..n_sink-1 and the rest rolling over the others.
// ---------------------------------------------------------------------------
__host__ __device__ inline int slot_of(int p, int W, int n_sink) {
  return p < n_sink ? p : n_sink + (p - n_sink) % W;
}

// Key set A(i): 0 <= j <= i and ((i - W < j and (i - j) mod dil == 0) or
// j < n_sink).
__host__ __device__ inline bool key_in_set(int i, int j, int W, int n_sink, int dil) {
  return j >= 0 && j <= i && ((j > i - W && (i - j) % dil == 0) || j < n_sink);
}

// Position held by slot `s` of a cache whose newest position is p (p has
// already been written), or -1 if that slot holds no live position.  Sink
// slot s holds position s once p >= s.  Rolling slot s holds the newest
// position q <= p with slot(q) == s and q >= n_sink.
__device__ inline int slot_position(int s, int p, int W, int n_sink) {
  if (s < n_sink) return s <= p ? s : -1;
  if (p < n_sink) return -1;
  const int sp = n_sink + (p - n_sink) % W;          // slot of p
  int d = sp - s;
  if (d < 0) d += W;
  const int q = p - d;
  return q >= n_sink ? q : -1;
}

// ---------------------------------------------------------------------------
// RoPE: cos/sin of the angle p * theta^(-2k/D).  The angle in revolutions,
// p * rev[k], is formed in double and reduced to its signed fraction in
// [-1/2, 1/2] there; the hardware sine and cosine of revolutions
// (v_sin_f32 / v_cos_f32) take it from float.  Their largest absolute error
// over [-1/2, 1/2] measured on gfx950 is 1.3e-7, that of float rounding.
// ---------------------------------------------------------------------------
__device__ inline void rope_cs(int p, double rev, float& c, float& s) {
  const double a = (double)p * rev;
  const float t = (float)(a - rint(a));
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}

// Rotate the pair (x0, x1) counter-clockwise by the angle with cos c, sin s.
__device__ inline void rotate(float& x0, float& x1, float c, float s) {
  const float y0 = x0 * c - x1 * s;
  const float y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}

// ---------------------------------------------------------------------------
// bf16 helpers (bit patterns kept in uint32 halves)
// ---------------------------------------------------------------------------
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, a in the low half.
__device__ inline uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline uint16_t to_bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, (__bf16)a);
}

}  // namespace swa
