// Shared device helpers for libaveris (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "averis.h"

namespace av {

constexpr int kKPad = 256;  // storage padding multiple along K (one GEMM K-step)
// split_quant needs cols to be a multiple of this: a row-layout thread quantizes one 32-element
// (64-byte bf16) unit, all or nothing, and the code tails are zeroed in 16-byte (32-code) pieces
constexpr int kColMult = 32;

__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Block scales are stored tiled for the GEMM: for each group of 32 rows and each 256-element
// K-step the group's 32 x (256 / g) scale bytes are contiguous (row-major inside the piece), so
// one K-step of a 128-row tile fetches 4 contiguous pieces instead of 128 scattered rows.
// Byte offset of the scale of K-block `blk` (elements blk*g ..) of row `r`:
__host__ __device__ inline int64_t scale_offset(int64_t r, int64_t blk, int64_t k_pad, int g) {
  const int64_t spb = 256 / g;  // scale bytes per row per K-step
  return ((r >> 5) * (k_pad >> 8) + blk / spb) * (32 * spb) + (r & 31) * spb + blk % spb;
}
// Bytes of a tiled scale array: rows padded to a multiple of 32.
static inline int64_t scale_bytes(int64_t outer, int64_t k_pad, int g) { return round_up(outer, 32) * (k_pad / g); }

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two fp32 values as bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
  const v2bf16 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- element loads ------------
// Inputs are bf16 (bit patterns in uint16) or fp32.  VEC = elements per 16-byte load.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ static inline void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
  __device__ static inline float load1(const float* p) { return *p; }
};
template <> struct Elem<uint16_t> {
  static constexpr int VEC = 8;
  __device__ static inline void unpack(const uint4& w, float* v) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  __device__ static inline float load1(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
};

// ---------------------------------------------------------------- number formats -----------
// E4M3 (fn): bias 7, max 448 = 0x7E.  Round to nearest even, saturate (finite t >= 0 only).
__device__ inline uint32_t e4m3_encode(float t) {
  if (t >= 448.0f) return 0x7Eu;  // [448, 464) rounds to 448; above saturates
  const uint32_t u = __float_as_uint(t);
  const int ef = (int)(u >> 23);  // biased exponent (t >= 0)
  if (ef < 127 - 6) {             // below 2^-6: subnormal E4M3, quantum 2^-9
    return (uint32_t)__builtin_rintf(t * 512.0f);  // exact scaling; 8 == code 0x08 (2^-6)
  }
  const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) & ~0xFFFFFu;  // RNE to 3 mantissa bits
  return ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));             // (e - 127 + 7) << 3 | m
}

__device__ inline float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * (1.0f / 512.0f);
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E8M0 exponent of an MXFP4 block: floor(log2 amax) - 2 clamped to [-127, 127].  Zero and
// fp32-subnormal amax (exponent field 0) land on the clamp.
__device__ inline int mx_exponent(float amax) {
  const int ef = (int)(__float_as_uint(amax) >> 23);
  const int e = ef - 129;
  return e < -127 ? -127 : e;
}

// Two E2M1 codes (RNE, ties to even code, saturating, sign kept) into byte SEL of `old`;
// `a` goes to the low nibble.  Hardware conversion with unit scale.
template <int SEL>
__device__ inline uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Eight E2M1 codes of v[0..7] (already scaled) packed into one dword, element 0 lowest.
__device__ inline uint32_t pack8_fp4(const float* v) {
  uint32_t w = 0;
  w = cvt_fp4x2<0>(w, v[0], v[1]);
  w = cvt_fp4x2<1>(w, v[2], v[3]);
  w = cvt_fp4x2<2>(w, v[4], v[5]);
  w = cvt_fp4x2<3>(w, v[6], v[7]);
  return w;
}
// Eight E2M1 codes of v[j] / scale.  With an MXFP4 block scale 2^e the conversion's division is
// exact, fl(v / 2^e) == fl(v * 2^-e), so it replaces the separate multiply.
__device__ inline uint32_t pack8_fp4_div(const float* v, float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
  return w;
}
// 2^e of an MXFP4 scale code e + 127 as fp32 (2^-127 is subnormal).
__device__ inline float mx_scale_value(uint32_t sbyte) {
  return sbyte ? __uint_as_float(sbyte << 23) : __uint_as_float(0x00400000u);
}
__device__ inline uint32_t pack4_fp4(const float* v) {
  uint32_t w = 0;
  w = cvt_fp4x2<0>(w, v[0], v[1]);
  w = cvt_fp4x2<1>(w, v[2], v[3]);
  return w;
}

// Per-block quantization parameters.  `mul` scales elements before the E2M1 conversion;
// `dead` zeroes the block's codes; `sbyte` is the stored scale code.
struct BlockQ {
  float mul;
  uint32_t sbyte;
  bool dead;
};

template <int FMT>
__device__ inline BlockQ block_params(float amax, float s_dec) {
  BlockQ q;
  if (FMT == AVERIS_MXFP4) {
    const int e = mx_exponent(amax);
    q.mul = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
    q.sbyte = (uint32_t)(e + 127);
    q.dead = !(amax > 0.0f);
  } else {
    // e_b = E4M3(fl(fl(a/6)/s_dec)); S = fl(val(e_b) * s_dec); mul = fl(1/S)
    if (!(s_dec > 0.0f)) {
      q.mul = 0.0f; q.sbyte = 0; q.dead = true;
      return q;
    }
    const float t = __fdiv_rn(__fdiv_rn(amax, 6.0f), s_dec);
    const uint32_t e = e4m3_encode(t);
    const float S = __fmul_rn(e4m3_value(e), s_dec);
    q.sbyte = e;
    q.dead = (e == 0u) || !(S >= 1.17549435e-38f);
    q.mul = q.dead ? 0.0f : __fdiv_rn(1.0f, S);
  }
  return q;
}

__device__ inline float nvfp4_tensor_scale(float amax) { return __fdiv_rn(amax, 2688.0f); }

// ---------------------------------------------------------------- wave helpers -------------
__device__ inline float wave_xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

// Workgroup barrier that orders LDS accesses only: the wave waits for its own LDS operations,
// not for its global stores to be acknowledged (__syncthreads() waits for those too).  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- direct-to-LDS loads -----
typedef __attribute__((address_space(3))) void lds_void_t;

// Raw buffer resource over `bytes` bytes at `base` (bytes < 2^32): loads at offsets >= bytes
// return zero, which pads partial tiles with zeros and keeps them inside the allocation.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// One wave-wide direct-to-LDS load: lane L's SIZE bytes from rsrc[voff + soff] land at lds + L * SIZE.
template <int AUX>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, soff, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, voff, soff, 0, AUX);
}
// Wait until at most N vector-memory ops of this wave are outstanding and all its LDS ops are
// done (gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
// Cache policy bits of buffer stores: non-temporal (streamed past the caches).
constexpr int kNonTemporal = 2;

// 16-byte non-temporal global load.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------- grouped operands ---------
// Group e (an expert) covers input rows [off[e], off[e+1]).  Per group: len = l_e, and the
// exclusive prefix sums p32 = sum round_up(l_e', 32) (its first row in a grouped row layout)
// and p256 = sum round_up(l_e', 256) (its first token in a grouped column layout).
struct GroupPos {
  int e;          // group, or -1 past the last item
  int64_t local;  // item index inside the group
  int64_t base;   // items of the groups before it
  int64_t off, len, p32, p256;
};

// Values equal in every lane, moved to scalar registers so that the compiler knows it (buffer
// descriptors built from them stay uniform).
__device__ inline int uniform32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-wide scan over the groups, 64 at a time.  Group e owns cnt(l_e) consecutive items; with
// `by_item` the group holding item t is returned, otherwise group t itself.  Every lane of the
// wave gets the same answer.
template <class F>
__device__ inline GroupPos group_scan(const int64_t* __restrict__ off, int E, int64_t t, bool by_item, F cnt) {
  const int lane = threadIdx.x & 63;
  int64_t b_cnt = 0, b32 = 0, b256 = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int64_t len = e < E ? off[e + 1] - off[e] : 0;
    const int64_t c = e < E ? cnt(len) : 0, r32 = round_up(len, 32), r256 = round_up(len, 256);
    int64_t sc = c, s32 = r32, s256 = r256;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t x = __shfl_up(sc, d, 64), y = __shfl_up(s32, d, 64), z = __shfl_up(s256, d, 64);
      if (lane >= d) { sc += x; s32 += y; s256 += z; }
    }
    const bool mine = by_item ? (e < E && b_cnt + sc > t) : (e == t);
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int L = __builtin_ctzll(hit);
      GroupPos g;
      g.e = uniform32(e0 + L);
      g.base = uniform64(b_cnt + __shfl(sc, L, 64) - __shfl(c, L, 64));
      g.local = uniform64(t) - g.base;
      g.len = uniform64(__shfl(len, L, 64));
      g.off = uniform64(off[g.e]);
      g.p32 = uniform64(b32 + __shfl(s32, L, 64) - __shfl(r32, L, 64));
      g.p256 = uniform64(b256 + __shfl(s256, L, 64) - __shfl(r256, L, 64));
      return g;
    }
    b_cnt += __shfl(sc, 63, 64); b32 += __shfl(s32, 63, 64); b256 += __shfl(s256, 63, 64);
  }
  GroupPos g{};
  g.e = -1;
  return g;
}

// Persistent launches: the logical tiles [0, n) are cut into 8 contiguous runs, one per XCD
// (workgroups are dispatched round-robin over the 8 XCDs, so workgroup b runs on XCD b % 8);
// workgroup k of XCD x takes tiles start_x + k, start_x + k + G_x, ... where G_x is the number of
// workgroups on XCD x.  Neighbouring tiles are then in flight at the same time on one XCD.
__device__ inline void xcd_tiles(int b, int grid, int n, int& first, int& stride, int& end) {
  const int x = b & 7, k = b >> 3;
  const int q = n >> 3, r = n & 7;
  const int start = x * q + (x < r ? x : r), cnt = q + (x < r ? 1 : 0);
  first = start + k;
  stride = (grid >> 3) + ((grid & 7) > x ? 1 : 0);
  end = start + cnt;
}

// Workgroup-id remap so that consecutive logical tiles run on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs); partial cache lines written by neighbouring tiles
// then meet in that XCD's L2.
__device__ inline int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

}  // namespace av
