// Device-side building blocks shared by the decode, readout and merge kernels.
//
// Work decomposition. A state tile (one (batch, head) pair, d_k x d_v) is cut
// into 8 x 8 chunks. One lane owns one chunk: 8 consecutive key rows by 8
// consecutive value columns. A wavefront holds CL chunks across (8*CL
// columns) and RL = 64/CL chunks down (8*RL rows), CL = max(4, group/8), so a
// scale group (g consecutive columns of one row) never straddles wavefronts
// and its absmax needs at most log2(g/8) lane exchanges. Lane l owns column
// block lc = l % CL and row block rho = bitreverse(l / CL): the lowest row-block
// bit sits on lane bit 5, so a pairwise (cascade) sum over rows in row order
// combines lane l with lane l^32 first, then l^16, and so on.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace rsq {

// One entry per head, stored in the state buffer after the header.
struct HeadEntry {
  int32_t bits;          // 4, 6, 8 or 32
  float gamma;           // RetNet decay of this head (0 for other models)
  uint64_t head_offset;  // tile offset inside a batch row
  uint32_t scales;       // section offsets inside the tile (codes at 0)
  uint32_t bypass_u;
  uint32_t bypass_w;
  uint32_t ref;
};
static_assert(sizeof(HeadEntry) == 32, "head table entry is 32 bytes");

constexpr uint32_t kStatusNonfinite = 1u, kStatusScaleOverflow = 2u, kStatusClipped = 4u;
constexpr int kMaxCap = 32;   // bypass columns a kernel can hold

// OCP E4M3 (exponent bias 7, 3 mantissa bits, largest finite 448, no
// infinities): round to nearest-even, saturate to +-448 (infinities too),
// every NaN -> 0x7F. gfx950's conversion instructions use this format:
// v_cvt_pk_fp8_f32 rounds to nearest-even, and with its input clamped to
// +-448 first it saturates as above; v_cvt_f32_fp8 is exact. Checked against a
// bitwise software encoder over all 2^32 float inputs and all 256 codes: the
// two differ only in the byte a NaN gets, which is set here.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const float xc = fminf(fmaxf(x, -448.f), 448.f);
  const uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(xc, xc, 0, false) & 0xFFu;
  return (x == x) ? c : 0x7Fu;
}

// two codes at once: a in bits 0-7, b in bits 8-15
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  const float ac = fminf(fmaxf(a, -448.f), 448.f), bc = fminf(fmaxf(b, -448.f), 448.f);
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ac, bc, 0, false) & 0xFFFFu;
  if (!(a == a)) c = (c & 0xFF00u) | 0x7Fu;
  if (!(b == b)) c = (c & 0x00FFu) | 0x7F00u;
  return c;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// code SEL (byte SEL) of a packed word
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// the four codes of a packed word, byte 0 first
__device__ __forceinline__ void e4m3_bytes4(uint32_t w, float out[4]) {
  out[0] = e4m3_byte_to_f32<0>(w);
  out[1] = e4m3_byte_to_f32<1>(w);
  out[2] = e4m3_byte_to_f32<2>(w);
  out[3] = e4m3_byte_to_f32<3>(w);
}

// Round-to-nearest-even of an exact product through the float32 adder:
// fma(x, inv, 1.5*2^23) rounds x*inv + 1.5*2^23 once, at unit spacing, so the
// result minus the magic constant is RNE(x*inv) whenever |x*inv| < 2^22.
constexpr float kMagic = 12582912.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ void load8(bool bf16, const void* base, size_t idx, float out[8]) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      out[2 * p] = __uint_as_float(w[p] << 16);
      out[2 * p + 1] = __uint_as_float(w[p] & 0xFFFF0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    const float4 a = f[0], b = f[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

__device__ __forceinline__ void loadf8(const float* p, float out[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ __forceinline__ void storef8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ void load_scales8(bool sf16, const uint8_t* p, float s[8]) {
  if (sf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[2 * q] = __half2float(__ushort_as_half((uint16_t)(w[q] & 0xFFFFu)));
      s[2 * q + 1] = __half2float(__ushort_as_half((uint16_t)(w[q] >> 16)));
    }
  } else {
    loadf8(reinterpret_cast<const float*>(p), s);
  }
}

__device__ __forceinline__ void store_scales8(bool sf16, uint8_t* p, const float s[8]) {
  if (sf16) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = __half_as_ushort(__float2half_rn(s[2 * q]));
      const uint32_t hi = __half_as_ushort(__float2half_rn(s[2 * q + 1]));
      w[q] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    storef8(reinterpret_cast<float*>(p), s);
  }
}

// RN16(a * u) with a single rounding: the mixed-precision FMA forms a*u + 0
// exactly (float32 x binary16) and rounds once to binary16, nearest-even.
__device__ __forceinline__ __half mul_rn_half(float a, __half u) {
  uint32_t r;
  const uint32_t ub = (uint32_t)__half_as_ushort(u);
  asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(a), "v"(ub));
  return __ushort_as_half((uint16_t)(r & 0xFFFFu));
}

// ---------------------------------------------------------------- code chunks
// Load one 8x8 chunk (8 * BITS bytes) into 32-bit words.
template <int BITS>
struct Chunk {
  static constexpr int kWords = 2 * BITS;   // 8*BITS bytes / 4
  uint32_t w[kWords];
};

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* p, Chunk<BITS>& c) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < Chunk<BITS>::kWords / 4; ++i) {
    const uint4 u = q[i];
    c.w[4 * i] = u.x; c.w[4 * i + 1] = u.y; c.w[4 * i + 2] = u.z; c.w[4 * i + 3] = u.w;
  }
}

template <int BITS>
__device__ __forceinline__ void store_chunk(uint8_t* p, const Chunk<BITS>& c) {
  uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
  for (int i = 0; i < Chunk<BITS>::kWords / 4; ++i)
    q[i] = make_uint4(c.w[4 * i], c.w[4 * i + 1], c.w[4 * i + 2], c.w[4 * i + 3]);
}

// Codes of a chunk as exact floats: c[r][j] for row r, column j.
__device__ __forceinline__ void unpack(const Chunk<4>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t lo = (ch.w[r] << 4) & 0xF0F0F0F0u;
    const uint32_t hi = ch.w[r] & 0xF0F0F0F0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[r][b] = (float)(int8_t)(lo >> (8 * b)) * 0.0625f;
      c[r][b + 4] = (float)(int8_t)(hi >> (8 * b)) * 0.0625f;
    }
  }
}

__device__ __forceinline__ void unpack(const Chunk<8>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[r][b] = (float)(int8_t)(ch.w[2 * r] >> (8 * b));
      c[r][b + 4] = (float)(int8_t)(ch.w[2 * r + 1] >> (8 * b));
    }
}

__device__ __forceinline__ void unpack(const Chunk<6>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t lo = (ch.w[r] << 4) & 0xF0F0F0F0u;
    const uint32_t hi = ch.w[r] & 0xF0F0F0F0u;
    const uint32_t crumbs = ch.w[8 + (r >> 1)] >> ((r & 1) * 4);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int h0 = (int)(int8_t)(lo >> (8 * b)) >> 4;
      const int h1 = (int)(int8_t)(hi >> (8 * b)) >> 4;
      const int l0 = (crumbs >> (8 * b)) & 3;
      const int l1 = (crumbs >> (8 * b + 2)) & 3;
      c[r][b] = (float)(4 * h0 + l0);
      c[r][b + 4] = (float)(4 * h1 + l1);
    }
  }
}

__device__ __forceinline__ void pack(const int q[8][8], Chunk<4>& ch) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      w |= (((uint32_t)q[r][b] & 0xFu) | (((uint32_t)q[r][b + 4] & 0xFu) << 4)) << (8 * b);
    ch.w[r] = w;
  }
}

__device__ __forceinline__ void pack(const int q[8][8], Chunk<8>& ch) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t a = 0, b2 = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      a |= ((uint32_t)q[r][b] & 0xFFu) << (8 * b);
      b2 |= ((uint32_t)q[r][b + 4] & 0xFFu) << (8 * b);
    }
    ch.w[2 * r] = a;
    ch.w[2 * r + 1] = b2;
  }
}

__device__ __forceinline__ void pack(const int q[8][8], Chunk<6>& ch) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t h0 = (uint32_t)(q[r][b] >> 2) & 0xFu;
      const uint32_t h1 = (uint32_t)(q[r][b + 4] >> 2) & 0xFu;
      w |= (h0 | (h1 << 4)) << (8 * b);
    }
    ch.w[r] = w;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t v = ((uint32_t)q[2 * p][b] & 3u) | (((uint32_t)q[2 * p][b + 4] & 3u) << 2) |
                         (((uint32_t)q[2 * p + 1][b] & 3u) << 4) |
                         (((uint32_t)q[2 * p + 1][b + 4] & 3u) << 6);
      w |= v << (8 * b);
    }
    ch.w[8 + p] = w;
  }
}

// fp32 chunk (unquantized state and the yoked reference): 8 rows x 8 floats.
__device__ __forceinline__ void load_f32_chunk(const uint8_t* p, float x[8][8]) {
  const float* f = reinterpret_cast<const float*>(p);
#pragma unroll
  for (int r = 0; r < 8; ++r) loadf8(f + 8 * r, x[r]);
}

__device__ __forceinline__ void store_f32_chunk(uint8_t* p, const float x[8][8]) {
  float* f = reinterpret_cast<float*>(p);
#pragma unroll
  for (int r = 0; r < 8; ++r) storef8(f + 8 * r, x[r]);
}

// ---------------------------------------------------------------- lane helpers
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// In-lane cascade sum over the 8 rows of a chunk: ((t0+t1)+(t2+t3))+((t4+t5)+(t6+t7)).
__device__ __forceinline__ float tree8(const float t[8]) {
  const float a = __fadd_rn(t[0], t[1]), b = __fadd_rn(t[2], t[3]);
  const float c = __fadd_rn(t[4], t[5]), d = __fadd_rn(t[6], t[7]);
  return __fadd_rn(__fadd_rn(a, b), __fadd_rn(c, d));
}

}  // namespace rsq
