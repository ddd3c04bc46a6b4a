// Fused decode step: dequantize, decay, (delta-rule retrieval), update,
// readout, scale rule, requantize (+BDR), pack and store in place.
//
// One workgroup per state tile (batch b, head h); its wavefronts cover the
// tile as WRW row-wavefronts x WCW column-wavefronts (see rsq_device.hpp for
// the lane decomposition). Everything a step needs for one column lives in the
// column's wavefronts, so the only cross-wavefront traffic is the sum over key
// rows when d_k exceeds one wavefront's rows, and the bypass (a handful of
// fp16 column pairs shared by the tile).
//
// The arithmetic follows one fixed float32 chain so that codes come out the
// same as a plain CPU evaluation of the same chain:
//   c1 = fl(a_i s_iG); r_ij = fl(c_ij c1)                       decay (Table 1)
//   GDN: u_j = cascade sum over rows i (row order) of fl(k_i fl(c_ij s_iG)),
//        w_j = fl(beta fl(v_j - fl(alpha u_j)))                   delta rule
//   x_ij = fma(k_i, w_j, r_ij)
//   o_j = sum_i q_i x_ij (float32, any order)                     readout
//   s' = storage(fl(m/qmax)) (dynamic / yoked), or kept unless
//        m > fl(fl(trigger qmax) s) (persistent)                  scale rule
//   c' = clamp(RNE(x RN(1/s')))                                   requantize
// Table 1 and the update/requantize/BDR/LRB definitions are from "Preserving
// Updates in Low-Bit Recurrent State Quantization"; the scale policies from
// the abstract of "When Dynamic Scaling Fails ...".
//
// Instruction diet (the step moves ~1.2 bytes per element, so at HBM speed a
// lane has only a handful of VALU slots per element):
//  * codes are unpacked straight to F*c with one SDWA sign-extending convert
//    per code (F = 16, 4, 1 for 4, 6, 8 bits); 1/F is folded into the per-row
//    multipliers, which is exact whenever the multiplier is not deep in the
//    float32 subnormal range (checked; the exact long form runs otherwise);
//  * with bf16 keys and binary16 step sizes, k_i s_i and c k_i s_i are exact in
//    float32 (19 and <= 24 bits), so the first cascade level of the retrieval
//    is one FMA per pair of rows;
//  * row sums use permlane swaps / DPP, halving the carried columns per level;
//  * 1/s for a binary16 step is rcp + one Newton step, which reproduces the
//    correctly rounded reciprocal for every binary16 value (checked on the
//    device for all 31743 positive finite values);
//  * requantization is one FMA against 1.5*2^23 + 2^(b-1): the float's low bits
//    are then the offset-binary code; the clamp runs only when a step size is
//    small enough (a subnormal, or a yoked scale) for a code to leave the range.
#pragma once
#include "rsq_kernels.hpp"
#include "lane_ops.hpp"

namespace rsq {

template <int BITS>
struct Fmt {
  // unpacked value = F * code: 4-bit codes convert straight to c/16
  // (v_cvt_off_f32_i4), 6-bit ones assemble to 4c, 8-bit ones are c
  static constexpr float F = BITS == 4 ? 0.0625f : BITS == 6 ? 4.f : 1.f;
  static constexpr float invF = 1.f / F;
  static constexpr int qmax = (1 << (BITS - 1)) - 1;
  // t = fma(x, inv, magic) rounds x*inv once, at unit spacing, to magic + RNE(x*inv).
  // Its low byte is then the code as packing wants it: offset binary c + 8 for
  // 4 bits (a clean nibble), two's complement c mod 256 for 6 and 8 bits.
  static constexpr float magic = BITS == 4 ? 12582912.0f + 8.0f : 12582912.0f;
  static constexpr float lo_t = magic - (float)(qmax + 1), hi_t = magic + (float)qmax;
  // products c * (k s) stay exact in float32 (|c| < 2^(b-1), k s has 19 bits)
  static constexpr bool kExactPairs = BITS <= 6;
};

// ---------------------------------------------------------------- unpack to F*c
// c/16 of the two's complement nibble in bits 0-3 of byte B of w
template <int B>
__device__ __forceinline__ float cvt_off_byte(uint32_t w) {
  float r;
  if constexpr (B == 0) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
  else if constexpr (B == 1) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  else if constexpr (B == 2) asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  else asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  return r;
}

__device__ __forceinline__ void unpack_scaled(const Chunk<4>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t w = ch.w[r], hi = w >> 4;   // columns 0-3 in the low nibbles, 4-7 in the high ones
    c[r][0] = cvt_off_byte<0>(w);
    c[r][1] = cvt_off_byte<1>(w);
    c[r][2] = cvt_off_byte<2>(w);
    c[r][3] = cvt_off_byte<3>(w);
    c[r][4] = cvt_off_byte<0>(hi);
    c[r][5] = cvt_off_byte<1>(hi);
    c[r][6] = cvt_off_byte<2>(hi);
    c[r][7] = cvt_off_byte<3>(hi);
  }
}

__device__ __forceinline__ void unpack_scaled(const Chunk<8>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[r][b] = (float)(int8_t)(ch.w[2 * r] >> (8 * b));
      c[r][b + 4] = (float)(int8_t)(ch.w[2 * r + 1] >> (8 * b));
    }
}

// bytes hi<<4 | lo<<2 sign-extend to 16 hi + 4 lo = 4 c
__device__ __forceinline__ void unpack_scaled(const Chunk<6>& ch, float c[8][8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t cw = ch.w[8 + (r >> 1)] >> ((r & 1) * 4);
    const uint32_t lo = ((ch.w[r] << 4) & 0xF0F0F0F0u) | ((cw << 2) & 0x0C0C0C0Cu);
    const uint32_t hi = (ch.w[r] & 0xF0F0F0F0u) | (cw & 0x0C0C0C0Cu);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      c[r][b] = (float)(int8_t)(lo >> (8 * b));
      c[r][b + 4] = (float)(int8_t)(hi >> (8 * b));
    }
  }
}

// ---------------------------------------------------------------- pack codes from t
// t holds magic + c (Fmt): its low byte is the code in the form packing uses.
// Bytes [a.b0, b.b0, 0, 0] and [0, 0, c.b0, d.b0].
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x0c0c0400u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t c, uint32_t d) { return __builtin_amdgcn_perm(d, c, 0x04000c0cu); }
__device__ __forceinline__ uint32_t low_bytes(float a, float b, float c, float d) {
  return lo_pair(__float_as_uint(a), __float_as_uint(b)) | hi_pair(__float_as_uint(c), __float_as_uint(d));
}
// (a & m) | (b & ~m)
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// 4 bits: byte k of word r = nibble(col k) | nibble(col k+4) << 4, two's
// complement. From offset-binary nibbles (bits 4-7 of each low byte clear):
// one shift-or per byte pair, two byte gathers and one XOR with 0x88.
__device__ __forceinline__ void pack_t(const float t[8][8], Chunk<4>& ch) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint32_t p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = (__float_as_uint(t[r][k + 4]) << 4) | __float_as_uint(t[r][k]);
    ch.w[r] = (lo_pair(p[0], p[1]) | hi_pair(p[2], p[3])) ^ 0x88888888u;
  }
}

// 8 bits: the low bytes are the codes
__device__ __forceinline__ void pack_t(const float t[8][8], Chunk<8>& ch) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    ch.w[2 * r] = low_bytes(t[r][0], t[r][1], t[r][2], t[r][3]);
    ch.w[2 * r + 1] = low_bytes(t[r][4], t[r][5], t[r][6], t[r][7]);
  }
}

// 6 bits: word r (r < 8) holds the high 4 bits of the codes like the 4-bit
// layout; word 8+p holds the low 2 bits of rows 2p and 2p+1 (byte k: col k,
// col k+4, then the same of the next row, 2 bits each from the bottom)
__device__ __forceinline__ void pack_t(const float t[8][8], Chunk<6>& ch) {
  uint32_t L[8], H[8];   // two's complement code bytes of columns 0-3 and 4-7
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    L[r] = low_bytes(t[r][0], t[r][1], t[r][2], t[r][3]);
    H[r] = low_bytes(t[r][4], t[r][5], t[r][6], t[r][7]);
    ch.w[r] = bfi(0x0F0F0F0Fu, L[r] >> 2, H[r] << 2);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t x = bfi(0x03030303u, L[2 * q], H[2 * q] << 2);
    const uint32_t y = bfi(0x03030303u, L[2 * q + 1], H[2 * q + 1] << 2);
    ch.w[8 + q] = bfi(0x0F0F0F0Fu, x, y << 4);
  }
}

// correctly rounded 1/s of a binary16 value (s > 0 finite), see the header note
__device__ __forceinline__ float recip_f16val(float s) {
  const float r = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r, 1.0f);
  return __builtin_fmaf(r, e, r);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }
__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

// q[i] = fl(m[i] / Q) for Q = 7, 31, 127 and m >= 0: y = fl(m RN(1/Q)), then
// one FMA correction y + fl(m - y Q) RN(1/Q). That is the correctly rounded
// quotient for every m in [2^-100, 2^100] and for m = 0 (checked for all
// float32 m in [1, 2) for each Q; power-of-two scaling carries it over the
// range). Outside it, and for NaN, the wavefront divides.
template <int Q>
__device__ __forceinline__ void div_qmax(const float m[8], float q[8]) {
  constexpr float qf = (float)Q, zi = 1.0f / (float)Q;
  const float lo = min8(m), hi = max8(m);
  if (wave_all(hi <= 0x1p100f && (lo >= 0x1p-100f || lo == 0.f))) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = __fmul_rn(m[i], zi);
      const float r = __builtin_fmaf(-y, qf, m[i]);
      q[i] = __builtin_fmaf(r, zi, y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = m[i] / qf;
  }
}

// div_qmax for two values (same arithmetic, same range check)
template <int Q>
__device__ __forceinline__ void div_qmax2(const float m[2], float q[2]) {
  constexpr float qf = (float)Q, zi = 1.0f / (float)Q;
  const float lo = min_nc(m[0], m[1]), hi = max_nc(m[0], m[1]);
  if (wave_all(hi <= 0x1p100f && (lo >= 0x1p-100f || lo == 0.f))) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float y = __fmul_rn(m[i], zi);
      const float r = __builtin_fmaf(-y, qf, m[i]);
      q[i] = __builtin_fmaf(r, zi, y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) q[i] = m[i] / qf;
  }
}

// m / F (F a small power of two) is exact unless the quotient is subnormal
__device__ __forceinline__ bool subnormal(float m) { return __builtin_amdgcn_class(m, 0x90) != 0; }

// Compile-time specialisations of the per-call flags (0 = read them at run time):
// scale mode, step-size dtype, input dtype and scale group size.
enum { kSpecGeneric = 0, kSpecPersF16Bf16G32 = 1, kSpecDynF32Bf16G64 = 2, kSpecDynF16Bf16G32 = 3,
       kSpecDynF32F32G64 = 4 };
enum { kSpecPersF16Bf16 = kSpecPersF16Bf16G32, kSpecDynF32Bf16 = kSpecDynF32Bf16G64,
       kSpecDynF16Bf16 = kSpecDynF16Bf16G32, kSpecDynF32F32 = kSpecDynF32F32G64 };

template <int SPEC>
struct Spec {
  // lanes per scale group (0: run time)
  static constexpr int GL = SPEC == kSpecGeneric ? 0 : (SPEC == 1 || SPEC == 3) ? 4 : 8;
  static __device__ __forceinline__ int smode(const StepArgs& a) {
    return SPEC == kSpecGeneric ? a.smode : SPEC == kSpecPersF16Bf16 ? (int)kScalePersistent : (int)kScaleDynamic;
  }
  static __device__ __forceinline__ bool sf16(const StepArgs& a) {
    return SPEC == kSpecGeneric ? a.scale_f16 != 0 : (SPEC == kSpecPersF16Bf16 || SPEC == kSpecDynF16Bf16);
  }
  static __device__ __forceinline__ bool bf16(const StepArgs& a) {
    return SPEC == kSpecGeneric ? a.in_bf16 != 0 : SPEC != kSpecDynF32F32;
  }
};

// Pure-write window, pairs that stay ("Low-Bit GDN Recurrent-State
// Quantization ...", abstract: recent writes kept as FP8 pairs and carried
// through the full GDN transition). One wavefront per pair c:
//   d = cascade sum over rows (row order) of fl(k_i u_ci), b = fl(beta d),
//   u_ci <- e4m3(fl(alpha fl(u_ci - fl(b k_i)))),
// and z_c = sum_i u_ci q_i for the readout (any order). Lane l holds rows
// l R .. l R + R - 1 (R = d_k / 64, or one row for d_k < 64, lanes past d_k
// adding zeros), so the in-lane tree and then the butterfly over lanes 1, 2,
// ..., 32 apart give the cascade order. The new pair's z_s = sum_i e4m3(k_i) q_i.
// The same for d_k <= 256 (R <= 4 rows per lane) and at most 4 pairs per
// wavefront: the lane's key bytes of a pair are one dword, loaded for every
// pair before the first wait, and written back with one store. Same sums in
// the same order as pw_pairs.
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint16_t g_u16;
typedef __attribute__((address_space(1))) uint8_t g_u8;
// The words the pairs' phase reads, loaded in one batch before the state's
// stores (the loads then do not wait behind them on the in-order memory
// counter): lane l's key bytes of the pairs c = wave + nw m, and k, q of its
// rows (raw: a bf16 input's 16 bits, shifted into a float where used, so that
// no wait for them comes before the stores). Also, for the new pair and the
// readout's window term:
// k of row tid and v of column tid mod d_v, and the window's E4M3 w bytes of
// the readout's columns c = tid / d_v + m (block / d_v) (clamped indices: every
// load is unconditional).
struct PwPre {
  uint32_t pre[4], kb[4], qb[4];
  uint32_t kn, vn;
  uint32_t wb[4];
  float al, be;   // the step's gates, as the state's step loaded them
  __device__ __forceinline__ static float f(uint32_t raw, bool bf16) { return __uint_as_float(bf16 ? raw << 16 : raw); }
};
static __device__ __forceinline__ void pw_prefetch(const uint8_t* U8, const uint8_t* W8, const void* kp, const void* qp,
                                                   const void* vp, bool bf16, int tile, int dk, int dv, int W,
                                                   PwPre& p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int R = dk >= 64 ? dk >> 6 : 1;
  const int i0 = lane * R;
  const g_u32* U = (const g_u32*)reinterpret_cast<const uint32_t*>(U8);
  const int wi = min(i0, dk - 1) >> 2;
#pragma unroll
  for (int m = 0; m < 4; ++m) p.pre[m] = U[(size_t)min(wave + nw * m, W - 1) * (dk >> 2) + wi];
  const int t = threadIdx.x, P = (int)blockDim.x / dv, j = t % dv, pp = t / dv;
  const size_t ik = (size_t)tile * dk + min(t, dk - 1), iv = (size_t)tile * dv + j;
  if (bf16) {
    const g_u16* K16 = (const g_u16*)reinterpret_cast<const uint16_t*>(kp);
    const g_u16* Q16 = (const g_u16*)reinterpret_cast<const uint16_t*>(qp);
    const g_u16* V16 = (const g_u16*)reinterpret_cast<const uint16_t*>(vp);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t idx = (size_t)tile * dk + min(i0 + e, dk - 1);
      p.kb[e] = K16[idx];
      p.qb[e] = Q16[idx];
    }
    p.kn = K16[ik];
    p.vn = V16[iv];
  } else {
    const g_u32* K32 = (const g_u32*)reinterpret_cast<const uint32_t*>(kp);
    const g_u32* Q32 = (const g_u32*)reinterpret_cast<const uint32_t*>(qp);
    const g_u32* V32 = (const g_u32*)reinterpret_cast<const uint32_t*>(vp);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const size_t idx = (size_t)tile * dk + min(i0 + e, dk - 1);
      p.kb[e] = K32[idx];
      p.qb[e] = Q32[idx];
    }
    p.kn = K32[ik];
    p.vn = V32[iv];
  }
  const g_u8* Wb = (const g_u8*)W8;
#pragma unroll
  for (int m = 0; m < 4; ++m) p.wb[m] = Wb[(size_t)min(pp + m * max(P, 1), W - 1) * dv + j];
}

// R = d_k / 64 rows per lane (d_k a power of two, 64 .. 256), or one row
// (d_k < 64, lanes past d_k adding zeros)
template <int R>
static __device__ __forceinline__ void pw_pairs_r4(uint8_t* U8, const PwPre& pf, bool bf16, int dk, int W,
                                              int n, int slot, float al, float be, float* z) {
  const bool leaving = n == W;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int i0 = lane * R;                 // the lane's first row
  const bool rows_ok = i0 < dk;
  const int sh = 8 * (i0 & 3);
  float k4[R], q4[R];
#pragma unroll
  for (int e = 0; e < R; ++e) {
    k4[e] = rows_ok ? PwPre::f(pf.kb[e], bf16) : 0.f;
    q4[e] = rows_ok ? PwPre::f(pf.qb[e], bf16) : 0.f;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int c = wave + nw * m;
    if (c >= W) break;
    const bool is_new = c == slot;
    const bool stays = c < n && !(leaving && c == slot);
    if (!is_new && !stays) continue;
    float zacc = 0.f;
    if (is_new) {
#pragma unroll
      for (int e = 0; e < R; ++e) zacc = __builtin_fmaf(e4m3_to_f32(f32_to_e4m3(k4[e])), q4[e], zacc);
    } else {
      const uint32_t ub = pf.pre[m] >> sh;
      float ue[R], pe[R];
#pragma unroll
      for (int e = 0; e < R; ++e) {
        const float u = e == 0 ? e4m3_byte_to_f32<0>(ub) : e == 1 ? e4m3_byte_to_f32<1>(ub)
                      : e == 2 ? e4m3_byte_to_f32<2>(ub) : e4m3_byte_to_f32<3>(ub);
        ue[e] = rows_ok ? u : 0.f;
        pe[e] = __fmul_rn(k4[e], ue[e]);
      }
      if constexpr (R == 2) pe[0] = __fadd_rn(pe[0], pe[1]);
      if constexpr (R == 4) pe[0] = __fadd_rn(__fadd_rn(pe[0], pe[1]), __fadd_rn(pe[2], pe[3]));
      float d = pe[0];
      d = __fadd_rn(d, dpp_xor1(d));
      d = __fadd_rn(d, dpp_xor2(d));
      d = __fadd_rn(d, swz_xor(d, 4));
      d = __fadd_rn(d, dpp_ror8(d));
      d = __fadd_rn(d, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(d), 0x401F)));
      d = __fadd_rn(d, __shfl_xor(d, 32, 64));
      const float b = __fmul_rn(be, d);
      float nv[R];
#pragma unroll
      for (int e = 0; e < R; ++e) nv[e] = __fmul_rn(al, __fsub_rn(ue[e], __fmul_rn(b, k4[e])));
      uint32_t codes;
      if constexpr (R == 1) codes = f32_to_e4m3(nv[0]);
      else if constexpr (R == 2) codes = f32x2_to_e4m3(nv[0], nv[1]);
      else codes = f32x2_to_e4m3(nv[0], nv[1]) | (f32x2_to_e4m3(nv[2], nv[3]) << 16);
#pragma unroll
      for (int e = 0; e < R; ++e) {
        const float u = e == 0 ? e4m3_byte_to_f32<0>(codes) : e == 1 ? e4m3_byte_to_f32<1>(codes)
                      : e == 2 ? e4m3_byte_to_f32<2>(codes) : e4m3_byte_to_f32<3>(codes);
        zacc = __builtin_fmaf(u, q4[e], zacc);
      }
      if (rows_ok) {
        g_u8* dst = (g_u8*)(U8 + (size_t)c * dk + i0);
        if constexpr (R == 4) *(g_u32*)dst = codes;
        else if constexpr (R == 2) *(g_u16*)dst = (uint16_t)codes;
        else *dst = (uint8_t)codes;
      }
    }
    zacc = wave_sum64(zacc);
    if (lane == 0) z[c] = zacc;
  }
}

template <bool BF16>
static __device__ __noinline__ void pw_pairs(uint8_t* U, const void* kp, const void* qp, int tile, int dk, int W,
                                           int n, int slot, float al, float be, float* z) {
  constexpr bool bf16 = BF16;
  const bool leaving = n == W;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int R = dk >= 64 ? dk >> 6 : 1;   // rows per lane: 1 .. 16, a power of two
  // k and q of the lane's first four rows stay in registers for every pair
  float k4[4], q4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // unconditional loads at a clamped index (no branch between the loads)
    const int i = lane * R + e;
    const bool ok = e < R && i < dk;
    const float kv = in_elem(bf16, kp, (size_t)tile * dk + min(i, dk - 1));
    const float qv = in_elem(bf16, qp, (size_t)tile * dk + min(i, dk - 1));
    k4[e] = ok ? kv : 0.f;
    q4[e] = ok ? qv : 0.f;
  }
  auto kq = [&](int e, float& ke, float& qe) {
    const int i = lane * R + e;
    ke = in_elem(bf16, kp, (size_t)tile * dk + i);
    qe = in_elem(bf16, qp, (size_t)tile * dk + i);
  };
  // the lane's R <= 4 key bytes of the wavefront's first four pairs, one
  // load each and all issued before the first wait (a later load would
  // otherwise also wait for the stores of the pair before it)
  constexpr int kPre = 4;
  uint32_t pre[kPre];
  const bool preload = R <= 4;
  if (preload) {
    const uint32_t* U32 = reinterpret_cast<const uint32_t*>(U);
    const int wi = min(lane * R, dk - 1) >> 2;
#pragma unroll
    for (int m = 0; m < kPre; ++m) pre[m] = U32[(size_t)min(wave + nw * m, W - 1) * (dk >> 2) + wi];
  }
  int m = 0;
  for (int c = wave; c < W; c += nw, ++m) {
    const bool is_new = c == slot;
    const bool stays = c < n && !(leaving && c == slot);
    if (!is_new && !stays) continue;
    float zacc = 0.f;
    if (is_new) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = blk * 4 + e;
          if (r >= R || lane * R + r >= dk) continue;
          float ke = 0.f, qe = 0.f;
          if (blk == 0) ke = k4[e], qe = q4[e];
          else kq(r, ke, qe);
          zacc = __builtin_fmaf(e4m3_to_f32(f32_to_e4m3(ke)), qe, zacc);
        }
    } else {
      uint8_t* uc = U + (size_t)c * dk;
      // in-lane cascade over the lane's R rows, in blocks of four: each block
      // pairwise, then the block sums pairwise
      float u4[4], bs[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        bs[blk] = 0.f;
        if (blk * 4 >= R) continue;
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = blk * 4 + e, i = lane * R + r;
          float ue = 0.f, ke = 0.f, qe = 0.f;
          if (r < R && i < dk) {
            uint32_t byte = 0;
            if (blk == 0 && preload && m < kPre) {
#pragma unroll
              for (int mm = 0; mm < kPre; ++mm)
                if (mm == m) byte = (pre[mm] >> (8 * ((i & 3)))) & 0xFFu;
            } else {
              byte = uc[i];
            }
            ue = e4m3_to_f32(byte);
            if (blk == 0) ke = k4[e];
            else kq(r, ke, qe);
          }
          if (blk == 0) u4[e] = ue;
          pe[e] = __fmul_rn(ke, ue);
        }
        if (1 < R) { pe[0] = __fadd_rn(pe[0], pe[1]); pe[2] = __fadd_rn(pe[2], pe[3]); }
        if (2 < R) pe[0] = __fadd_rn(pe[0], pe[2]);
        bs[blk] = pe[0];
      }
      if (4 < R) { bs[0] = __fadd_rn(bs[0], bs[1]); bs[2] = __fadd_rn(bs[2], bs[3]); }
      if (8 < R) bs[0] = __fadd_rn(bs[0], bs[2]);
      // then over lanes 1, 2, 4, ..., 32 apart (both lanes of a pair form the same sum)
      float d = bs[0];
      d = __fadd_rn(d, dpp_xor1(d));
      d = __fadd_rn(d, dpp_xor2(d));
      d = __fadd_rn(d, swz_xor(d, 4));
      d = __fadd_rn(d, dpp_ror8(d));
      d = __fadd_rn(d, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(d), 0x401F)));
      d = __fadd_rn(d, __shfl_xor(d, 32, 64));
      const float b = __fmul_rn(be, d);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = blk * 4 + e, i = lane * R + r;
          if (r >= R || i >= dk) continue;
          float ue, ke, qe;
          if (blk == 0) ue = u4[e], ke = k4[e], qe = q4[e];
          else { ue = e4m3_to_f32(uc[i]); kq(r, ke, qe); }
          const uint32_t code = f32_to_e4m3(__fmul_rn(al, __fsub_rn(ue, __fmul_rn(b, ke))));
          uc[i] = (uint8_t)code;
          zacc = __builtin_fmaf(e4m3_to_f32(code), qe, zacc);
        }
    }
    zacc = wave_sum64(zacc);
    if (lane == 0) z[c] = zacc;
  }
}

template <int MODEL, int CL, int FEAT, int SPEC>
struct Decode {
  using SP = Spec<SPEC>;
  static constexpr int RL = 64 / CL;
  static constexpr int NB = (RL == 16) ? 4 : (RL == 8) ? 3 : 2;   // log2(RL)
  static constexpr int WR = 8 * RL;
  static constexpr int WC = 8 * CL;
  static constexpr int NSLOT = 8 >> (NB < 3 ? NB : 3);            // columns a lane holds after xtree
  static constexpr bool kF32 = FEAT == kFeatF32;
  static constexpr bool kBypass = FEAT == kFeatBypass;
  static constexpr bool kYoked = FEAT == kFeatYoked;
  static constexpr bool kDiag = FEAT == kFeatDiag;
  // INT4+Had: groups stored rotated; after the load phase x holds state values
  static constexpr bool kHad = FEAT == kFeatHad;
  // pure-write window (Gated DeltaNet): the history takes the transition with v = 0
  static constexpr bool kPW = FEAT == kFeatPW;
  static constexpr bool kDense = kF32;
  // BDR needs the pre-rounding x next to the codes; so do the diagnostics
  static constexpr bool kKeepX = !kF32 && (FEAT == kFeatBdr || kYoked || kDiag);

  struct Lds {
    float* w;      // [nwaves][WC]   per-wavefront broadcast of w (and of the reference's w)
    float* up;     // [wrw][dv]      retrieval partials across row-wavefronts
    float* op;     // [wrw][dv]      readout partials across row-wavefronts
    float* z;      // [kMaxCap] + [nw][kMaxCap]  bypass readout projections
    float* zk;     // [kMaxCap]  delta rule with a bypass: z_c = U_c^T k
    float* bz;     // [dv]       delta rule with a bypass: b = W z
    __half* wst;   // gdn_wstage_bytes(dv)  delta rule with a bypass: W's columns, staged
    uint8_t* ust;  // gdn_ustage_bytes(dk)  ... and U's
    uint8_t* stg;  // [nwaves][512 BITS bytes] the waves' code chunks, staged (run_piece)
  };

  static __device__ __forceinline__ void decays(const StepArgs& a, const HeadEntry& he, int tile, int i0,
                                                float dec[8]) {
    if constexpr (MODEL == kRetNet) {
#pragma unroll
      for (int r = 0; r < 8; ++r) dec[r] = he.gamma;
    } else if constexpr (MODEL == kGLA) {
      loadf8(a.alpha + (size_t)tile * a.dk + i0, dec);
    } else {
      const float al = a.alpha[tile];
#pragma unroll
      for (int r = 0; r < 8; ++r) dec[r] = al;
    }
  }

  // Finish a per-column row sum (v: NSLOT wave sums of this lane's columns)
  // across row-wavefronts in cascade order; every wave of the column stripe
  // ends with the full sum. The caller passes the LDS partial buffer.
  static __device__ __forceinline__ void across_waves(float v[8], float* part, int wrw, int wr, int j0,
                                                      int lane, int dv) {
    if (wrw <= 1) return;
    const bool writer = NB < 4 || ((lane >> 2) & 1) == 0;
#pragma unroll
    for (int s = 0; s < NSLOT; ++s)
      if (writer) part[wr * dv + j0 + xtree_col<NB>(s, lane)] = v[s];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const int col = j0 + xtree_col<NB>(s, lane);
      float l0 = part[col], l1 = part[dv + col];
      if (wrw == 2) {
        v[s] = __fadd_rn(l0, l1);
      } else {
        const float l2 = part[2 * dv + col], l3 = part[3 * dv + col];
        float a01 = __fadd_rn(l0, l1), a23 = __fadd_rn(l2, l3);
        if (wrw == 4) {
          v[s] = __fadd_rn(a01, a23);
        } else {
          const float b01 = __fadd_rn(__fadd_rn(part[4 * dv + col], part[5 * dv + col]),
                                      __fadd_rn(part[6 * dv + col], part[7 * dv + col]));
          v[s] = __fadd_rn(__fadd_rn(a01, a23), b01);
        }
      }
    }
    __syncthreads();
  }

  // u_j = sum_i k_i S_ij in cascade order for the lane's 8 columns, turned into
  // w_j = beta (v_j - alpha u_j), broadcast to every lane of the column block.
  // xs: the lane's 8x8 values with S_ij = xs_ij * mul_i (mul = s/F, or 1 for an
  // fp32 tile); kap: k_i s_i / F when `fast` (exact products), unused otherwise.
  // The gates and the lane's v values after the tree (`pre`, from dw_prefetch)
  // are loaded at the start of the step with the state, not here.
  // INT4+Had with bf16 inputs known at compile time: q and the lane's 8 v
  // values stay as their raw bf16 words (4 registers each instead of 8) until
  // they are used, which keeps the rotated step within 128 registers
  static constexpr bool kRawIn = kHad && SPEC != kSpecGeneric && SPEC != kSpecDynF32F32;
  struct DwPre {
    float al, be, v[kHad ? (kRawIn ? 1 : 8) : NSLOT];   // the rotation needs v of the lane's own 8 columns
    uint32_t vr[kRawIn ? 4 : 1];
  };
  // bf16 pair p of four raw words as two floats, converted where they are
  // used: the empty asm keeps the conversion from being hoisted to the load
  static __device__ __forceinline__ void raw_bf16x8(const uint32_t r[4], float out[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t w = r[p];
      asm volatile("" : "+v"(w));
      out[2 * p] = __uint_as_float(w << 16);
      out[2 * p + 1] = __uint_as_float(w & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ DwPre dw_prefetch(const StepArgs& a, int tile, int j0, int lane) {
    DwPre p;
    p.al = a.alpha[tile];
    p.be = a.beta[tile];
    if constexpr (kRawIn) {
      const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v) + (size_t)tile * a.dv + j0);
      p.vr[0] = u.x, p.vr[1] = u.y, p.vr[2] = u.z, p.vr[3] = u.w;
    } else if constexpr (kHad) {
      load8(SP::bf16(a), a.v, (size_t)tile * a.dv + j0, p.v);
    } else {
#pragma unroll
      for (int s = 0; s < NSLOT; ++s) p.v[s] = kPW ? 0.f : load_in1(a, tile, j0 + xtree_col<NB>(s, lane));
    }
    return p;
  }

  // With a bypass (bz non-null) the retrieval adds the bypass's share b_j,
  // u_j = fl(u~_j + b_j), and the row-wavefront 0 lanes holding column sums
  // store the new bypass column W[:, n] = fp16(w) at wn.
  template <int BITS>
  static __device__ __forceinline__ void delta_w(const StepArgs& a, int tile, const float xs[8][8],
                                                 const float kf[8], const float mul[8], const float kap[8],
                                                 bool fast, const DwPre& pre, float wv[8], float* wl,
                                                 float* up, int wrw, int wr, int j0, int lane, int wave,
                                                 const float* bz = nullptr, __half* wn = nullptr) {
    float v8[8];
    if (fast) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float t0 = __fmul_rn(xs[2 * q][j], kap[2 * q]);
          if constexpr (Fmt<BITS>::kExactPairs) {
            p[q] = __builtin_fmaf(xs[2 * q + 1][j], kap[2 * q + 1], t0);   // = fl(t0 + t1), t1 exact
          } else {
            p[q] = __fadd_rn(t0, __fmul_rn(xs[2 * q + 1][j], kap[2 * q + 1]));
          }
        }
        v8[j] = __fadd_rn(__fadd_rn(p[0], p[1]), __fadd_rn(p[2], p[3]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = __fmul_rn(kf[i], __fmul_rn(xs[i][j], mul[i]));
        v8[j] = tree8(t);
      }
    }
    xtree<NB>(v8, lane);
    across_waves(v8, up, wrw, wr, j0, lane, a.dv);
    const float al = pre.al, be = pre.be;
    // lanes holding column sums compute w and publish it (INT4+Had: they
    // publish the rotated sums u~, and every lane forms w for its own
    // columns from u = u~ H / g, then rotates it: w~ = H w)
    float* wrow = wl + wave * WC;
    const int lc = lane % CL;
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const int c = xtree_col<NB>(s, lane);
      const float u = (kBypass && bz) ? __fadd_rn(v8[s], bz[j0 + c]) : v8[s];
      const float w = kHad ? u : __fmul_rn(be, __fsub_rn(pre.v[s], __fmul_rn(al, u)));
      const bool writer = NB < 4 || ((lane >> 2) & 1) == 0;
      if (writer) wrow[8 * lc + c] = w;
      if constexpr (kBypass) {
        if (writer && wr == 0) wn[j0 + c] = __float2half_rn(w);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    loadf8(wrow + 8 * lc, wv);
    if constexpr (kHad) {
      const int gl = SP::GL > 0 ? SP::GL : (a.group >> 3);
      const float ig = 1.0f / (float)(8 * gl);   // 1/g, a power of two
      fwht8(wv, gl, lane);
      float v8l[8];
      if constexpr (kRawIn) raw_bf16x8(pre.vr, v8l);
      else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v8l[j] = pre.v[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = __fmul_rn(wv[j], ig);
        wv[j] = __fmul_rn(be, __fsub_rn(v8l[j], __fmul_rn(al, u)));
      }
      fwht8(wv, gl, lane);
    }
  }

  // Unnormalised Walsh-Hadamard transform of the lane's share of a vector
  // whose scale groups run along the columns (INT4+Had of "Preserving
  // Updates ...", Table 2): butterflies at column distance 1, 2, 4 inside the
  // lane's 8 columns, then 8, 16, ... across the group's gl lanes (lane bit m
  // = column bit 8m), each pair (a, b) at (j, j + h) becoming
  // (fl(a + b), fl(a - b)). Across lanes the partner's value p arrives by
  // DPP / swizzle, and fma(sign, x, p) forms fl(x + p) on the lower lane,
  // fl(p - x) on the upper.
  static __device__ __forceinline__ void fwht8(float v[8], int gl, int lane) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j & h) == 0) {
          const float lo = v[j], hi = v[j + h];
          v[j] = __fadd_rn(lo, hi);
          v[j + h] = __fsub_rn(lo, hi);
        }
#pragma unroll
    for (int lvl = 0; lvl < 4; ++lvl) {
      const int m = 1 << lvl;
      if (m >= gl) break;
      const float sg = (lane & m) ? -1.f : 1.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = v[j];
        const float p = lvl == 0 ? dpp_xor1(x) : lvl == 1 ? dpp_xor2(x) : lvl == 2 ? swz_xor(x, 4) : dpp_ror8(x);
        v[j] = __builtin_fmaf(sg, x, p);
      }
    }
  }

  static __device__ __forceinline__ float load_in1(const StepArgs& a, int tile, int j) {
    return in_elem(SP::bf16(a), a.v, (size_t)tile * a.dv + j);
  }

  // A wavefront's code chunks lie in memory as CL runs, one per column block:
  // the RL chunks of its rows are consecutive. Staged through the wave's LDS
  // area (the runs one after another), every load and store instruction moves
  // contiguous 16-byte pieces of whole runs, where a lane's own chunk would
  // take one 16-byte piece out of every 8*BITS bytes per instruction.
  template <int BITS>
  static __device__ __forceinline__ uint8_t* run_piece(uint8_t* tb, const StepArgs& a, int wc, int wr, int P) {
    constexpr int PR = RL * BITS / 2;   // 16-byte pieces per run
    const int r = P / PR, w = P - r * PR;
    return tb + ((size_t)(wc * CL + r) * (a.dk >> 3) + wr * RL) * (8 * BITS) + 16 * w;
  }
  // the lane's chunk inside the staged runs
  template <int BITS>
  static __device__ __forceinline__ uint4* staged_chunk(uint8_t* stg, int lc, int rho) {
    return reinterpret_cast<uint4*>(stg + (lc * RL + rho) * (8 * BITS));
  }
  // the new chunk back through the staged runs: each lane writes its chunk to
  // its place in the wave's area, then stores contiguous pieces
  template <int BITS>
  static __device__ __forceinline__ void stage_store(const StepArgs& a, uint8_t* tb, uint8_t* stg, int wc, int wr,
                                                     int lc, int rho, int lane, const Chunk<BITS>& ch) {
    uint4* mine = staged_chunk<BITS>(stg, lc, rho);
#pragma unroll
    for (int p = 0; p < BITS / 2; ++p) mine[p] = make_uint4(ch.w[4 * p], ch.w[4 * p + 1], ch.w[4 * p + 2], ch.w[4 * p + 3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i)
      *reinterpret_cast<uint4*>(run_piece<BITS>(tb, a, wc, wr, 64 * i + lane)) =
          reinterpret_cast<const uint4*>(stg)[64 * i + lane];
  }

  template <int BITS, bool BOOST = false>
  static __device__ __forceinline__ void body(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                              const Lds& L, uint32_t& flags, const BypassRegs* br = nullptr,
                                              bool byp_regs = false, PwPre* pwp = nullptr) {
    const bool bf16 = SP::bf16(a), sf16 = SP::sf16(a);
    const int smode = SP::smode(a);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wrw = a.dk / WR;
    const int wr = wave % wrw, wc = wave / wrw;
    const int lc = lane % CL, lr = lane / CL;
    const int rho = (int)(__builtin_bitreverse32((uint32_t)lr) >> (32 - NB));
    const int i0 = wr * WR + 8 * rho;
    const int j0 = wc * WC + 8 * lc;
    // group sizes are powers of two: the group index is a shift
    const int glog = SP::GL > 0 ? 3 + __builtin_ctz(SP::GL > 0 ? SP::GL : 1) : 31 - __builtin_clz(a.group);
    const int G = j0 >> glog;
    const int gl = SP::GL > 0 ? SP::GL : (a.group >> 3);   // lanes per group (1..16)
    constexpr float F = kF32 ? 1.f : Fmt<BITS == 32 ? 8 : BITS>::F;
    constexpr float invF = 1.f / F;

    uint8_t* cp = tb + ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * (8 * BITS);
    uint8_t* sp = tb + he.scales + ((size_t)G * a.dk + i0) * (sf16 ? 2 : 4);
    float x[8][8];
    float s_old[8];
    // quantized codes: the wave's runs go to its LDS area (run_piece), and
    // the lane's chunk is read from there once every load of the step is out.
    // Not in the raised-priority twin, whose grid is resident at once, nor
    // with a bypass (those grids fit at once too): there the extra LDS round
    // trip on the way in costs more than the coalesced accesses save
    // (measured on the 64 x 16 head workloads with and without a bypass, and
    // on the GLA 32 x 8 head one)
    constexpr bool kStaged = !kF32 && !BOOST && !kBypass;
    uint8_t* stg = kStaged ? L.stg + wave * (512 * BITS) : nullptr;
    if constexpr (kF32) {
      load_f32_chunk(cp, x);
    } else if constexpr (kStaged) {
#pragma unroll
      for (int i = 0; i < BITS / 2; ++i)
        __builtin_amdgcn_global_load_lds((g_cvoid*)run_piece<BITS>(tb, a, wc, wr, 64 * i + lane),
                                         (l_void*)(stg + 1024 * i), 16, 0, 0);
      load_scales8(sf16, sp, s_old);
    } else {
      Chunk<BITS> ch;
      load_chunk<BITS>(cp, ch);
      load_scales8(sf16, sp, s_old);
      unpack_scaled(ch, x);
    }
    // the pure-write window's leaving pair (the one written W steps ago):
    // its bytes load with the state's, it joins after the transition
    uint2 pw_ub = make_uint2(0u, 0u), pw_wb = make_uint2(0u, 0u);
    const bool pw_leaving = kPW && a.n == a.pw;
    if constexpr (kPW) {
      // loaded whether or not the pair leaves (the slot is always inside the
      // window's sections), so no branch separates these loads from the rest
      const int slot = (int)((a.t_next - 1) % a.pw);
      pw_ub = *reinterpret_cast<const uint2*>(tb + he.bypass_u + (size_t)slot * a.dk + i0);
      pw_wb = *reinterpret_cast<const uint2*>(tb + he.bypass_w + (size_t)slot * a.dv + j0);
    }
    float qf[kRawIn ? 1 : 8], kf[8], dec[8];
    uint32_t qr[kRawIn ? 4 : 1];
    if constexpr (kRawIn) {
      const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + (size_t)tile * a.dk + i0);
      qr[0] = u.x, qr[1] = u.y, qr[2] = u.z, qr[3] = u.w;
    } else {
      load8(bf16, a.q, (size_t)tile * a.dk + i0, qf);
    }
    load8(bf16, a.k, (size_t)tile * a.dk + i0, kf);
    decays(a, he, tile, i0, dec);
    DwPre dwp{};
    float wv[8];
    if constexpr (MODEL == kGDN) dwp = dw_prefetch(a, tile, j0, lane);
    else load8(bf16, a.v, (size_t)tile * a.dv + j0, wv);
    // keep every load of the step above this point: issued together at the
    // start, their latency overlaps instead of stalling the step midway (not
    // in the BDR, yoked and accounting variants, which already run at the
    // register limit)
    if constexpr (!(FEAT == kFeatBdr || kYoked || kDiag)) __builtin_amdgcn_sched_barrier(0);
    // the loads are out: back to the normal issue priority
    if constexpr (BOOST) __builtin_amdgcn_s_setprio(0);
    if constexpr (kStaged) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      Chunk<BITS> ch;
      const uint4* mine = staged_chunk<BITS>(stg, lc, rho);
#pragma unroll
      for (int p = 0; p < BITS / 2; ++p) {
        const uint4 u = mine[p];
        ch.w[4 * p] = u.x, ch.w[4 * p + 1] = u.y, ch.w[4 * p + 2] = u.z, ch.w[4 * p + 3] = u.w;
      }
      unpack_scaled(ch, x);
    }

    // per-row multipliers: c1/F (decay) and k s / F (retrieval). Dividing by
    // F = 1/16 (4 bits) is exact unless it overflows (not for binary16 steps);
    // by F = 4 (6 bits) unless the quotient is subnormal; F = 1 is no-op.
    constexpr bool kUp = !kDense && BITS == 4, kDown = !kDense && BITS == 6;
    float c1p[8], kap[8], smul[8];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c1 = kDense ? dec[i] : __fmul_rn(dec[i], s_old[i]);
      c1p[i] = (kUp || kDown) ? __fmul_rn(c1, invF) : c1;
      if constexpr (kDown) bad = bad || subnormal(c1p[i]);
      if constexpr (kUp) {
        if (!sf16) bad = bad || !(fabsf(c1p[i]) <= 3.4e38f);
      }
      smul[i] = kDense ? 1.f : s_old[i];
      if constexpr (MODEL == kGDN && !kDense) {
        const float ks = __fmul_rn(kf[i], s_old[i]);
        kap[i] = (kUp || kDown) ? __fmul_rn(ks, invF) : ks;
        if constexpr (kDown) bad = bad || subnormal(kap[i]);
        if constexpr (kUp) {
          if (!sf16) bad = bad || !(fabsf(kap[i]) <= 3.4e38f);
        }
      }
    }
    const bool fast = !wave_any(bad) && (kDense || MODEL != kGDN || (bf16 && sf16));
    if (!fast) {
      // exact long form: bring x back to the codes themselves
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c1p[i] = kF32 ? dec[i] : __fmul_rn(dec[i], s_old[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = __fmul_rn(x[i][j], invF);
      }
    }

    // update B_t: w = v (loaded at the start), or the delta rule; INT4+Had
    // steps in the rotated basis, so its update vector is w~ = H w
    if constexpr (kHad && MODEL != kGDN) fwht8(wv, gl, lane);
    if constexpr (MODEL == kGDN && kBypass) {
      // the bypass's share of the retrieval, b = W (U^T k), from the values
      // loaded at kernel start (the loop form ran before this step)
      if (byp_regs && a.n > 0) gdn_bypass_retrieval_regs(a, SP::bf16(a), *br, L.zk, L.bz, L.wst, L.ust);
      __half* wn = reinterpret_cast<__half*>(tb + he.bypass_w) + (size_t)a.n * a.dv;
      delta_w<BITS>(a, tile, x, kf, smul, kap, fast, dwp, wv, L.w, L.up, wrw, wr, j0, lane, wave,
                    a.n > 0 ? L.bz : nullptr, wn);
    } else if constexpr (MODEL == kGDN) {
      delta_w<BITS == 32 ? 8 : BITS>(a, tile, x, kf, smul, kap, fast && !kDense, dwp, wv, L.w, L.up, wrw, wr, j0,
                                     lane, wave);
    }

    // decay and update; r = fl(c fl(a s)) kept for BDR
    constexpr bool kKeepR = !kBypass && !kF32 && !kHad && !kPW;
    float r[kKeepR ? 8 : 1][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ri = __fmul_rn(x[i][j], c1p[i]);
        if constexpr (kKeepR) r[i][j] = ri;
        if constexpr (kBypass) x[i][j] = ri;
        else x[i][j] = __builtin_fmaf(kf[i], wv[j], ri);
      }

    // the leaving window pair joins after the transition: its key takes the
    // transition, u' = fl(a fl(u - fl(b k))) with b = fl(beta k^T u), and
    // x += u' w^T. k^T u is summed in the retrieval's pairwise row order:
    // the lane's rows, then the row lanes, then the row wavefronts.
    if constexpr (kPW) {
      if (pw_leaving) {
        float ue[8], we[8], t8[8];
        e4m3_bytes4(pw_ub.x, ue);
        e4m3_bytes4(pw_ub.y, ue + 4);
        e4m3_bytes4(pw_wb.x, we);
        e4m3_bytes4(pw_wb.y, we + 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) t8[i] = __fmul_rn(kf[i], ue[i]);
        float d = row_lane_sum<NB>(tree8(t8));
        if (wrw > 1) {
          if (wc == 0 && lane == 0) L.z[wr] = d;
          __syncthreads();
          const float l0 = L.z[0], l1 = L.z[1];
          if (wrw == 2) {
            d = __fadd_rn(l0, l1);
          } else {
            const float a01 = __fadd_rn(l0, l1), a23 = __fadd_rn(L.z[2], L.z[3]);
            d = wrw == 4 ? __fadd_rn(a01, a23)
                         : __fadd_rn(__fadd_rn(a01, a23),
                                     __fadd_rn(__fadd_rn(L.z[4], L.z[5]), __fadd_rn(L.z[6], L.z[7])));
          }
          __syncthreads();
        }
        const float b = __fmul_rn(dwp.be, d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u2 = __fmul_rn(dwp.al, __fsub_rn(ue[i], __fmul_rn(b, kf[i])));
#pragma unroll
          for (int j = 0; j < 8; ++j) x[i][j] = __builtin_fmaf(u2, we[j], x[i][j]);
        }
      }
    }

    // readout partial o_j over this wavefront's rows
    {
      float o8[8], q8[8];
      if constexpr (kRawIn) raw_bf16x8(qr, q8);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q8[i] = qf[i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = __fmul_rn(q8[0], x[0][j]);
#pragma unroll
        for (int i = 1; i < 8; ++i) acc = __builtin_fmaf(q8[i], x[i][j], acc);
        o8[j] = acc;
      }
      if constexpr (kHad) {
        // the readout of the rotated state is o~ = S~^T q; o = o~ H / g. The
        // rotation is linear, so it is applied to the lane's partial sums,
        // before the sum over rows (the readout's order is free)
        const float ig = 1.0f / (float)(8 * gl);   // 1/g, a power of two
        fwht8(o8, gl, lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) o8[j] = __fmul_rn(o8[j], ig);
      }
      xtree<NB>(o8, lane);
      const bool writer = NB < 4 || ((lane >> 2) & 1) == 0;
      if (wrw == 1 && !kBypass && !kPW) {
        // one wavefront covers every row: its sums are the readout
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
          const float o = o8[s];
          if (!(fabsf(o) <= 3.4e38f)) flags |= kStatusNonfinite;
          if (writer) a.o[(size_t)tile * a.dv + j0 + xtree_col<NB>(s, lane)] = o;
        }
      } else {
#pragma unroll
        for (int s = 0; s < NSLOT; ++s)
          if (writer) L.op[wr * a.dv + j0 + xtree_col<NB>(s, lane)] = o8[s];
      }
    }

    if constexpr (kF32) {
      store_f32_chunk(cp, x);
      return;
    } else {
      constexpr int qmax = Fmt<BITS>::qmax;
      constexpr float qmaxf = (float)qmax;
      constexpr float magic = Fmt<BITS>::magic;
      // yoked reference: the same recurrence on an fp32 tile; absmax comes from it
      float xr[kYoked ? 8 : 1][8];
      if constexpr (kYoked) {
        uint8_t* rp = tb + he.ref + ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * 256;
        load_f32_chunk(rp, xr);
        float wr_[8];
        if constexpr (MODEL == kGDN) {
          float ones[8], dummy[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) ones[i] = 1.f, dummy[i] = 0.f;
          delta_w<8>(a, tile, xr, kf, ones, dummy, false, dwp, wr_, L.w, L.up + wrw * a.dv, wrw, wr, j0, lane, wave);
        } else {
          load8(bf16, a.v, (size_t)tile * a.dv + j0, wr_);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) xr[i][j] = __builtin_fmaf(kf[i], wr_[j], __fmul_rn(dec[i], xr[i][j]));
        store_f32_chunk(rp, xr);
      }

      // scale rule per row of this lane's group
      // A group of 32 columns is a lane quad (4 lanes x 8 columns). There each
      // lane settles two of the quad's eight rows (rows 2q, 2q+1 for quad lane
      // q): the group maxima arrive by a reduce-scatter over the quad, the
      // step-size arithmetic runs on two rows instead of eight, and only the
      // reciprocals come back to every lane. Same values as the per-row form.
      constexpr bool kSplit = SP::GL == 4;
      // A group of 64 columns is 8 lanes: there each lane settles one row
      // (row q for group lane q), the same way.
      constexpr bool kSplit8 = SP::GL == 8 && !kYoked;
      float s_new[8], inv[8];
      float s2[2];                   // kSplit: steps of rows 2q, 2q+1; kSplit8: s2[0], row q
      bool tiny = false, grew_any = true;
      // reciprocals of the eight rows' steps, with the zero / overflow / tiny handling
      auto row_recips = [&]() {
        // the common case, every step of the wavefront normal and finite, needs
        // neither the zero / overflow handling nor the clamp
        const float s_lo = min8(s_new), s_hi = max8(s_new);
        const bool regular = sf16 ? (s_lo >= 0x1p-14f && s_hi <= 65504.f) : (s_lo >= 0x1p-100f && s_hi <= 0x1p100f);
#pragma unroll
        for (int i = 0; i < 8; ++i) inv[i] = sf16 ? recip_f16val(s_new[i]) : 1.0f / s_new[i];
        if (!wave_all(regular)) {
          // a zero step, or an infinite one (binary16 overflow), stores code 0;
          // tiny steps need the clamp
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (s_new[i] == 0.f || !(s_new[i] <= 3.4e38f)) inv[i] = 0.f;
          const float imax = max8(inv);
          if (!(s_hi <= 3.4e38f)) flags |= kStatusScaleOverflow;
          tiny = !(s_hi <= 3.4e38f) || !(imax <= (sf16 ? 16384.f : 0x1p100f));
        }
      };
      if constexpr (kSplit) {
        const bool h2 = (lane & 2) != 0, h1 = (lane & 1) != 0;
        float lm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) lm[i] = absmax8(x[i]);
        {
          // reduce-scatter of the row maxima (integer max of non-negative floats,
          // as group_absmax): first over lane q^2 (rows split 0-3 / 4-7), then q^1
          uint32_t kp[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t mine = __float_as_uint(h2 ? lm[4 + k] : lm[k]);
            const uint32_t other = __float_as_uint(h2 ? lm[k] : lm[4 + k]);
            kp[k] = max(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0x4E, 0xF, 0xF, false));
          }
          float m2[2], so[2], ratio[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t mine = h1 ? kp[2 + k] : kp[k], other = h1 ? kp[k] : kp[2 + k];
            m2[k] = __uint_as_float(max(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0xB1, 0xF, 0xF, false)));
            so[k] = h2 ? (h1 ? s_old[6 + k] : s_old[4 + k]) : (h1 ? s_old[2 + k] : s_old[k]);
          }
          if (smode == kScalePersistent) {
            // a group grows when its maximum exceeds fl(fl(trigger qmax) s)
            const float trig_q = __fmul_rn(a.trigger, qmaxf);
            bool grew[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              grew[k] = m2[k] > __fmul_rn(trig_q, so[k]);
              s2[k] = so[k];
            }
            grew_any = wave_any(grew[0] || grew[1]);
            if (grew_any) {
              div_qmax2<qmax>(m2, ratio);
#pragma unroll
              for (int k = 0; k < 2; ++k)
                if (grew[k]) s2[k] = sf16 ? __half2float(__float2half_rn(ratio[k])) : ratio[k];
            }
          } else {
            div_qmax2<qmax>(m2, ratio);
#pragma unroll
            for (int k = 0; k < 2; ++k) s2[k] = sf16 ? __half2float(__float2half_rn(ratio[k])) : ratio[k];
          }
          const float s_lo = min_nc(s2[0], s2[1]), s_hi = max_nc(s2[0], s2[1]);
          const bool regular = sf16 ? (s_lo >= 0x1p-14f && s_hi <= 65504.f) : (s_lo >= 0x1p-100f && s_hi <= 0x1p100f);
          float iv[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) iv[k] = sf16 ? recip_f16val(s2[k]) : 1.0f / s2[k];
          if (!wave_all(regular)) {
#pragma unroll
            for (int k = 0; k < 2; ++k)
              if (s2[k] == 0.f || !(s2[k] <= 3.4e38f)) iv[k] = 0.f;
            const float imax = max_nc(iv[0], iv[1]);
            if (!(s_hi <= 3.4e38f)) flags |= kStatusScaleOverflow;
            tiny = !(s_hi <= 3.4e38f) || !(imax <= (sf16 ? 16384.f : 0x1p100f));
          }
          // all-gather of the reciprocals: row 2q + b comes from quad lane q
          inv[0] = dpp_quad_bcast<0>(iv[0]);
          inv[1] = dpp_quad_bcast<0>(iv[1]);
          inv[2] = dpp_quad_bcast<1>(iv[0]);
          inv[3] = dpp_quad_bcast<1>(iv[1]);
          inv[4] = dpp_quad_bcast<2>(iv[0]);
          inv[5] = dpp_quad_bcast<2>(iv[1]);
          inv[6] = dpp_quad_bcast<3>(iv[0]);
          inv[7] = dpp_quad_bcast<3>(iv[1]);
        }
      } else if constexpr (kSplit8) {
        const int q = lane & 7;
        const bool h4 = (q & 4) != 0, h2 = (q & 2) != 0, h1 = (q & 1) != 0;
        float lm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) lm[i] = absmax8(x[i]);
        // reduce-scatter of the row maxima over the 8 lanes (integer max of
        // non-negative floats): halves across the half-row mirror (lane q and
        // 7 - q), then quads (q^2), then pairs (q^1); lane q ends with row q
        uint32_t k4[4], k2[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t mine = __float_as_uint(h4 ? lm[4 + r] : lm[r]);
          const uint32_t other = __float_as_uint(h4 ? lm[r] : lm[4 + r]);
          k4[r] = max(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0x141, 0xF, 0xF, false));
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t mine = h2 ? k4[2 + r] : k4[r], other = h2 ? k4[r] : k4[2 + r];
          k2[r] = max(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0x4E, 0xF, 0xF, false));
        }
        float m1[2], so1, ratio[2];
        {
          const uint32_t mine = h1 ? k2[1] : k2[0], other = h1 ? k2[0] : k2[1];
          m1[0] = __uint_as_float(max(mine, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other, 0xB1, 0xF, 0xF, false)));
          m1[1] = m1[0];
          const float a4 = h4 ? s_old[4] : s_old[0], b4 = h4 ? s_old[5] : s_old[1];
          const float c4 = h4 ? s_old[6] : s_old[2], d4 = h4 ? s_old[7] : s_old[3];
          const float lo2 = h2 ? c4 : a4, hi2 = h2 ? d4 : b4;
          so1 = h1 ? hi2 : lo2;
        }
        if (smode == kScalePersistent) {
          const float trig_q = __fmul_rn(a.trigger, qmaxf);
          const bool grew = m1[0] > __fmul_rn(trig_q, so1);
          s2[0] = so1;
          grew_any = wave_any(grew);
          if (grew_any) {
            div_qmax2<qmax>(m1, ratio);
            if (grew) s2[0] = sf16 ? __half2float(__float2half_rn(ratio[0])) : ratio[0];
          }
        } else {
          div_qmax2<qmax>(m1, ratio);
          s2[0] = sf16 ? __half2float(__float2half_rn(ratio[0])) : ratio[0];
        }
        const float sv = s2[0];
        const bool regular = sf16 ? (sv >= 0x1p-14f && sv <= 65504.f) : (sv >= 0x1p-100f && sv <= 0x1p100f);
        float iv = sf16 ? recip_f16val(sv) : 1.0f / sv;
        if (!wave_all(regular)) {
          if (sv == 0.f || !(sv <= 3.4e38f)) iv = 0.f;
          if (!(sv <= 3.4e38f)) flags |= kStatusScaleOverflow;
          tiny = !(sv <= 3.4e38f) || !(iv <= (sf16 ? 16384.f : 0x1p100f));
        }
        // all-gather of the reciprocals: pairs, quads, then halves (by q^4 via swizzle)
        float g2[2], g4v[4];
        const float p1 = dpp_xor1(iv);
        g2[0] = h1 ? p1 : iv;
        g2[1] = h1 ? iv : p1;
        const float p2a = dpp_xor2(g2[0]), p2b = dpp_xor2(g2[1]);
        g4v[0] = h2 ? p2a : g2[0];
        g4v[1] = h2 ? p2b : g2[1];
        g4v[2] = h2 ? g2[0] : p2a;
        g4v[3] = h2 ? g2[1] : p2b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = swz_xor(g4v[r], 4);
          inv[r] = h4 ? pr : g4v[r];
          inv[4 + r] = h4 ? g4v[r] : pr;
        }
      } else {
        auto row_max = [&](int i) {
          float m = kYoked ? absmax8(xr[i]) : absmax8(x[i]);
          if constexpr (SP::GL > 0) return group_absmax<SP::GL>(m);
          else return group_max_rt(m, gl);
        };
        if (smode == kScalePersistent) {
          // A group grows when its absmax m exceeds thr = fl(fl(trigger qmax) s):
          // exactly when some lane's own maximum does (thr is the same on every
          // lane of the group), so the exchange for the group maximum is only
          // needed on a step where some group of the wavefront grows.
          const float trig_q = __fmul_rn(a.trigger, qmaxf);
          float lm[8], thr[8], over[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            lm[i] = kYoked ? absmax8(xr[i]) : absmax8(x[i]);
            s_new[i] = s_old[i];
            thr[i] = __fmul_rn(trig_q, s_old[i]);
            // the sign of fl(m - thr) is the sign of m - thr
            over[i] = __fsub_rn(lm[i], thr[i]);
          }
          grew_any = wave_any(max8(over) > 0.f);
          if (grew_any) {
            // the rows that outgrew their range take fl(m / qmax) in the storage dtype
            float m[8], ratio[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              if constexpr (SP::GL > 0) m[i] = group_absmax<SP::GL>(lm[i]);
              else m[i] = group_max_rt(lm[i], gl);
            }
            div_qmax<qmax>(m, ratio);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float fresh = sf16 ? __half2float(__float2half_rn(ratio[i])) : ratio[i];
              if (m[i] > thr[i]) s_new[i] = fresh;
            }
          }
        } else {
          // dynamic / yoked: fl(m / qmax) in the storage dtype, every row
          float m[8], ratio[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) m[i] = row_max(i);
          div_qmax<qmax>(m, ratio);
#pragma unroll
          for (int i = 0; i < 8; ++i) s_new[i] = sf16 ? __half2float(__float2half_rn(ratio[i])) : ratio[i];
        }
        row_recips();
      }
      // codes can leave the range only for tiny steps, yoked scales, or a
      // persistent trigger above 1
      const bool clamp = kYoked || wave_any(tiny) || (smode == kScalePersistent && a.trigger > 1.f);

      // requantize: t = 1.5*2^23 + 2^(b-1) + RNE(x inv)   (+ BDR toward the update's sign)
      const bool bdr = (FEAT == kFeatBdr) || ((kYoked || kDiag) && a.bdr);
      constexpr float lo_t = Fmt<BITS>::lo_t, hi_t = Fmt<BITS>::hi_t;
      // BDR needs x after rounding; otherwise t overwrites x in place
      float xk[kKeepX ? 8 : 1][8];
      if constexpr (kKeepX) {
        if (bdr || kDiag) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) xk[i][j] = x[i][j];
        }
      }
      float (&t)[8][8] = x;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) t[i][j] = __builtin_fmaf(x[i][j], inv[i], magic);
      if (clamp) {
        bool clipped = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          clipped = clipped || max8(t[i]) > hi_t || min8(t[i]) < lo_t;
#pragma unroll
          for (int j = 0; j < 8; ++j) t[i][j] = med3_nc(t[i][j], lo_t, hi_t);
        }
        if (clipped) flags |= kStatusClipped;
      }
      if constexpr (kKeepX) {
        if (bdr) {
          const float gate_k = __fadd_rn(0.5f, a.bdr_eps);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (!(s_new[i] > 0.f)) continue;
            const float gate = __fmul_rn(gate_k, s_new[i]);
            const float sk = (float)((kf[i] > 0.f) - (kf[i] < 0.f));
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float sg = sk * (float)((wv[j] > 0.f) - (wv[j] < 0.f));
              const float c = t[i][j] - magic;
              const float val = __fmul_rn(c, s_new[i]);
              const bool rev = (sg > 0.f && val < r[i][j]) || (sg < 0.f && val > r[i][j]);
              const float cand = fminf(fmaxf(c + sg, -(float)(qmax + 1)), qmaxf);
              const float err = fabsf(__fsub_rn(xk[i][j], __fmul_rn(cand, s_new[i])));
              if (rev && err <= gate) t[i][j] = cand + magic;
            }
          }
        }
      }
      if constexpr (kDiag)
        diagnostics<BITS>(a, tile, i0, j0, t, xk, r, s_new, inv, kf, wv, dec);
      Chunk<BITS> out;
      pack_t(t, out);
      // the window's reads go out before the state's stores
      if constexpr (kPW) {
        if (pw_fits_r4(a)) {
          pw_prefetch(tb + he.bypass_u, tb + he.bypass_w, a.k, a.q, a.v, bf16, tile, a.dk, a.dv, a.pw, *pwp);
          pwp->al = dwp.al;
          pwp->be = dwp.be;
        }
      }
      if constexpr (kStaged) stage_store<BITS>(a, tb, stg, wc, wr, lc, rho, lane, out);
      else store_chunk<BITS>(cp, out);
      const bool store_s = smode != kScalePersistent || grew_any;
      if constexpr (kSplit8) {
        // each group lane stores its own row
        if (store_s) {
          uint8_t* sp1 = sp + (size_t)(lane & 7) * (sf16 ? 2 : 4);
          if (sf16) *reinterpret_cast<uint16_t*>(sp1) = __half_as_ushort(__float2half_rn(s2[0]));
          else *reinterpret_cast<float*>(sp1) = s2[0];
        }
      } else if constexpr (kSplit) {
        // each quad lane stores its own two rows
        uint8_t* sp2 = sp + (size_t)(2 * (lane & 3)) * (sf16 ? 2 : 4);
        if (store_s) {
          if (sf16) {
            const uint32_t lo = __half_as_ushort(__float2half_rn(s2[0])), hi = __half_as_ushort(__float2half_rn(s2[1]));
            *reinterpret_cast<uint32_t*>(sp2) = lo | (hi << 16);
          } else {
            *reinterpret_cast<float2*>(sp2) = make_float2(s2[0], s2[1]);
          }
        }
      } else {
        if (store_s && (lc & (gl - 1)) == 0) store_scales8(sf16, sp, s_new);
      }
    }
  }

  // Error accounting of one step ("Preserving Updates ...", Figs. 1, 2, 4 and
  // Table 5), per element of the lane's chunk, from the final codes:
  //   b = fl(k_i w_j), s_hat = c s', R = fl(s_hat - x);
  //   lost: b != 0 and c equals the code of the no-update value r on the same
  //   grid; moved: b != 0 otherwise; reversed: b != 0 and s_hat strictly on
  //   the far side of r from b;
  //   E <- fl(fl(a E) + R_m), D <- fl(fl(fl(a a) D) + fl(R_m R_m)) for
  //   m = all, lost, moved (R_m = R on the mask, 0 elsewhere);
  //   ratio = fl(|b| RN(1/s')) for updated elements with a finite step > 0, else -1.
  template <int BITS>
  static __device__ __forceinline__ void diagnostics(const StepArgs& a, int tile, int i0, int j0,
                                                     const float (&t)[8][8], const float (&xk)[8][8],
                                                     const float (&r)[8][8], const float s_new[8],
                                                     const float inv[8], const float kf[8], const float wv[8],
                                                     const float dec[8]) {
    constexpr float magic = Fmt<BITS>::magic, lo_t = Fmt<BITS>::lo_t, hi_t = Fmt<BITS>::hi_t;
    const size_t plane = (size_t)a.dk * a.dv;
    const size_t off = ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * 64;
    float* acc = a.dg_acc + (size_t)tile * 6 * plane + off;
    float* rat = a.dg_ratio ? a.dg_ratio + (size_t)tile * plane + off : nullptr;
    uint32_t n_upd = 0, n_lost = 0, n_moved = 0, n_rev = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = s_new[i];
      const bool finite_step = s > 0.f && s <= 3.4e38f;
      const float ai = dec[i], a2 = __fmul_rn(dec[i], dec[i]);
      float rr[8], rl[8], rm[8], ra[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float c = t[i][j] - magic;
        const float c0 = med3_nc(__builtin_fmaf(r[i][j], inv[i], magic), lo_t, hi_t) - magic;
        const float b = __fmul_rn(kf[i], wv[j]);
        const float shat = __fmul_rn(c, s);
        const float R = __fsub_rn(shat, xk[i][j]);
        const bool upd = b != 0.f;
        const bool lost = upd && c == c0;
        const bool rev = upd && s > 0.f && ((b > 0.f && shat < r[i][j]) || (b < 0.f && shat > r[i][j]));
        n_upd += upd;
        n_lost += lost;
        n_moved += upd && !lost;
        n_rev += rev;
        rr[j] = R;
        rl[j] = lost ? R : 0.f;
        rm[j] = (upd && !lost) ? R : 0.f;
        ra[j] = (upd && finite_step) ? __fmul_rn(fabsf(b), inv[i]) : -1.f;
      }
      const float* src[3] = {rr, rl, rm};
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        float* pe = acc + (size_t)(2 * p) * plane + 8 * i;
        float* pd = acc + (size_t)(2 * p + 1) * plane + 8 * i;
        float e[8], d[8];
        loadf8(pe, e);
        loadf8(pd, d);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float Rm = src[p][j];
          e[j] = __fadd_rn(__fmul_rn(ai, e[j]), Rm);
          d[j] = __fadd_rn(__fmul_rn(a2, d[j]), __fmul_rn(Rm, Rm));
        }
        storef8(pe, e);
        storef8(pd, d);
      }
      if (rat) storef8(rat + 8 * i, ra);
    }
    uint32_t cnt[4] = {n_upd, n_lost, n_moved, n_rev};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t v = cnt[k];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += (uint32_t)__shfl_xor((int)v, m, 64);
      if ((threadIdx.x & 63) == 0) atomicAdd(a.dg_counts + (size_t)tile * 4 + k, v);
    }
  }

  // Pure-write window: the pairs' transitions and the readout projections
  // (pw_pairs below), kept out of line so that its registers do not add to
  // the body's.
  // The pairs' phase reads its words from the batch loaded before the
  // state's stores when d_k <= 256 and every wavefront has at most 4 pairs.
  static __device__ __forceinline__ bool pw_fits_r4(const StepArgs& a) {
    return a.dk <= 256 && a.pw <= 4 * (int)(blockDim.x >> 6);
  }
  // ... and the new pair and the readout's window term too when every thread
  // has at most one row of k, one column of v and four window columns
  static __device__ __forceinline__ bool pw_fits_all(const StepArgs& a) {
    const int nt = blockDim.x;
    return pw_fits_r4(a) && a.dk <= nt && a.dv <= nt && a.pw <= 4 * (nt / a.dv);
  }
  static __device__ __forceinline__ void pw_phase(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                                  float* z, const PwPre& pf) {
    const int slot = (int)((a.t_next - 1) % a.pw);
    if (pw_fits_r4(a)) {
      const int R = a.dk >= 64 ? a.dk >> 6 : 1;
      if (R == 1) pw_pairs_r4<1>(tb + he.bypass_u, pf, SP::bf16(a), a.dk, a.pw, a.n, slot, pf.al, pf.be, z);
      else if (R == 2) pw_pairs_r4<2>(tb + he.bypass_u, pf, SP::bf16(a), a.dk, a.pw, a.n, slot, pf.al, pf.be, z);
      else pw_pairs_r4<4>(tb + he.bypass_u, pf, SP::bf16(a), a.dk, a.pw, a.n, slot, pf.al, pf.be, z);
      return;
    }
    if (SP::bf16(a)) pw_pairs<true>(tb + he.bypass_u, a.k, a.q, tile, a.dk, a.pw, a.n, slot, a.alpha[tile], a.beta[tile], z);
    else pw_pairs<false>(tb + he.bypass_u, a.k, a.q, tile, a.dk, a.pw, a.n, slot, a.alpha[tile], a.beta[tile], z);
  }

  // The new pure write (e4m3(k_t), e4m3(fl(beta_t v_t))) into slot (t - 1) mod W.
  static __device__ __forceinline__ void pw_write_new_pair(const StepArgs& a, const HeadEntry& he, uint8_t* tb,
                                                           int tile, const PwPre& pf) {
    const int slot = (int)((a.t_next - 1) % a.pw);
    const bool bf16 = SP::bf16(a);
    uint8_t* U = tb + he.bypass_u + (size_t)slot * a.dk;
    uint8_t* W = tb + he.bypass_w + (size_t)slot * a.dv;
    if (pw_fits_all(a)) {
      const int t = threadIdx.x;
      if (t < a.dk) U[t] = (uint8_t)f32_to_e4m3(PwPre::f(pf.kn, bf16));
      if (t < a.dv) W[t] = (uint8_t)f32_to_e4m3(__fmul_rn(pf.be, PwPre::f(pf.vn, bf16)));
      return;
    }
    const float be = a.beta[tile];
    for (int i = threadIdx.x; i < a.dk; i += blockDim.x)
      U[i] = (uint8_t)f32_to_e4m3(in_elem(bf16, a.k, (size_t)tile * a.dk + i));
    for (int j = threadIdx.x; j < a.dv; j += blockDim.x)
      W[j] = (uint8_t)f32_to_e4m3(__fmul_rn(be, in_elem(bf16, a.v, (size_t)tile * a.dv + j)));
  }

  // BOOST: every wavefront of the grid is resident from the start (the host
  // checks), and the ones still issuing their loads go ahead of those already
  // computing. With several rounds of workgroups this measured slower.
  template <bool BOOST = false>
  static __device__ void run(const StepArgs& a) {
    if constexpr (BOOST) __builtin_amdgcn_s_setprio(3);
    extern __shared__ float lds[];
    const int tile = blockIdx.x;
    const int bb = tile / a.H, h = tile - bb * a.H;
    const HeadEntry he = head_entry(a, h);
    uint8_t* tb = a.tiles + (size_t)bb * a.batch_stride + he.head_offset;
    const int wrw = a.dk / WR;
    const int nw = blockDim.x >> 6;
    Lds L;
    L.w = lds;                                // [nw][WC]
    L.up = L.w + nw * WC;                     // [2][wrw][dv]
    L.op = L.up + 2 * wrw * a.dv;             // [wrw][dv]
    L.z = L.op + wrw * a.dv;                  // [kMaxCap] + [nw][kMaxCap]
    L.zk = L.z + kMaxCap * (1 + nw);          // [kMaxCap]
    L.bz = L.zk + kMaxCap;                    // [dv]
    L.wst = reinterpret_cast<__half*>(L.bz + a.dv);
    L.ust = reinterpret_cast<uint8_t*>(L.wst) + gdn_wstage_bytes(a.dv);
    L.stg = reinterpret_cast<uint8_t*>(lds) + a.lds_stage;
    uint32_t flags = 0;

    // bypass: its loads join the state's (values held in registers) when
    // they fit, else the column loop runs first
    BypassRegs br;
    bool byp_regs = false;
    if constexpr (kBypass) {
      byp_regs = bypass_regs_fit(a, MODEL);
      if (byp_regs) {
        bypass_load(a, he, tb, tile, MODEL, SP::bf16(a), br, L.wst, L.ust);
      } else {
        // the delta rule reads the bypass before the decay below rewrites U
        if constexpr (MODEL == kGDN) {
          if (a.n > 0) gdn_bypass_retrieval_loop(a, he, tb, tile, L.zk, L.bz);
        }
        bypass_decode_phase(a, he, tb, tile, L.z, MODEL);
      }
    }

    PwPre pwp{};
    if constexpr (kF32) {
      body<32, BOOST>(a, he, tb, tile, L, flags);
    } else {
      switch (he.bits) {
        case 4: body<4, BOOST>(a, he, tb, tile, L, flags, &br, byp_regs, &pwp); break;
        case 6: body<6, BOOST>(a, he, tb, tile, L, flags, &br, byp_regs, &pwp); break;
        default: body<8, BOOST>(a, he, tb, tile, L, flags, &br, byp_regs, &pwp); break;
      }
    }
    if constexpr (kBypass) {
      if (byp_regs) bypass_store(a, he, tb, tile, MODEL, SP::bf16(a), br, L.z, L.ust);
    }
    // the staying window pairs: after the state's step, whose loads then go
    // out first (the pairs never touch the leaving pair's slot, which the
    // state's step reads)
    if constexpr (kPW) pw_phase(a, he, tb, tile, L.z, pwp);
    if constexpr (kPW) {
      // every wavefront has read the leaving pair: the new one takes its slot
      __syncthreads();
      pw_write_new_pair(a, he, tb, tile, pwp);
    }
    if (wrw > 1 || kBypass || kPW) {
      __syncthreads();
      // combine readout partials over row-wavefronts, add the bypass term, store o
      combine_o(a, he, tb, tile, L, wrw, flags, byp_regs, br, pwp);
    }
    finish(a, tile, flags);
  }

  static __device__ __forceinline__ void combine_o(const StepArgs& a, const HeadEntry& he, const uint8_t* tb,
                                                   int tile, const Lds& L, int wrw, uint32_t& flags,
                                                   bool byp_regs, BypassRegs& br, const PwPre& pf) {
    // bypass columns (fp16) / window pairs (E4M3): cnt columns of W, each
    // weighted by its z. The sum W z is spread over every thread of the
    // block: thread (p, j) takes columns p, p + P, ... of row j of W (its
    // loads in flight together), the P partials meet in LDS (L.up, free here:
    // P d_v <= 2 wrw d_v floats). The bypass's register path holds its W
    // entries in registers already.
    constexpr bool kWz = kBypass || kPW;
    const int cnt = kBypass ? a.n + 1 : kPW ? (a.n < a.pw ? a.n + 1 : a.pw) : 0;
    const int P = kWz ? (int)(blockDim.x / a.dv) : 0;
    auto wval = [&](int c, int j) {
      if constexpr (kPW) return e4m3_to_f32(tb[he.bypass_w + (size_t)c * a.dv + j]);
      else return __half2float(reinterpret_cast<const __half*>(tb + he.bypass_w)[(size_t)c * a.dv + j]);
    };
    if (kWz && P >= 1) {
      const int j = threadIdx.x % a.dv, pp = threadIdx.x / a.dv;
      if (pp < P) {
        float part = 0.f;
        if (kBypass && byp_regs) {
          // the delta rule's new column is fp16(w_j), w as published by the
          // first row-wavefront of column j's stripe
          const float w_new = MODEL == kGDN ? L.w[(j / WC) * wrw * WC + j % WC] : 0.f;
          part = bypass_wz_part(a, MODEL, SP::bf16(a), br, L.z, w_new, L.wst);
        }
        else if (kPW && pw_fits_all(a)) {
          // the window's w bytes from the early batch; the new pair's slot
          // holds e4m3(beta v_j) now
          const int slot = (int)((a.t_next - 1) % a.pw);
          const float wnew = e4m3_to_f32(f32_to_e4m3(__fmul_rn(pf.be, PwPre::f(pf.vn, SP::bf16(a)))));
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int c = pp + m * P;
            if (c < cnt) part = __builtin_fmaf(c == slot ? wnew : e4m3_to_f32(pf.wb[m]), L.z[c], part);
          }
        } else
          for (int c = pp; c < cnt; c += P) part = __builtin_fmaf(wval(c, j), L.z[c], part);
        L.up[pp * a.dv + j] = part;
      }
      __syncthreads();
    }
    for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
      float acc = L.op[j];
      for (int q = 1; q < wrw; ++q) acc += L.op[q * a.dv + j];
      if (kWz) {
        if (P >= 1) {
          for (int pp = 0; pp < P; ++pp) acc += L.up[pp * a.dv + j];
        } else {
          for (int c = 0; c < cnt; ++c) acc = __builtin_fmaf(wval(c, j), L.z[c], acc);
        }
      }
      if (!(fabsf(acc) <= 3.4e38f)) flags |= kStatusNonfinite;
      a.o[(size_t)tile * a.dv + j] = acc;
    }
  }


  static __device__ __forceinline__ void finish(const StepArgs& a, int tile, uint32_t flags) {
    if (wave_any(flags != 0)) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) flags |= (uint32_t)__shfl_xor((int)flags, m, 64);
      if ((threadIdx.x & 63) == 0) atomicOr(a.status, flags);
    }
    if (tile == 0 && threadIdx.x == 0) {
      *a.hdr_t = a.t_next;
      *a.hdr_n = kBypass ? a.n + 1 : kPW ? (a.n < a.pw ? a.n + 1 : a.pw) : 0;
    }
  }
};

template <int MODEL, int CL, int FEAT, int SPEC>
__global__ __launch_bounds__(512) void decode_kernel(StepArgs a) {
  Decode<MODEL, CL, FEAT, SPEC>::run(a);
}

// specialised steps held to at most 128 VGPRs: four wavefronts per SIMD
template <int MODEL, int CL, int FEAT, int SPEC, bool BOOST = false>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel_occ(StepArgs a) {
  Decode<MODEL, CL, FEAT, SPEC>::template run<BOOST>(a);
}

// The raised-priority twin of a decode kernel, for launches whose grid is
// resident at once, or nullptr. Only the plain and rotated Gated DeltaNet
// steps with binary16 persistent steps have one (measured on the 64 x 16 head
// workload; the windowed step gained nothing).
template <int MODEL, int CL>
DecodeFn decode_pick_boost(DecodeFn fn) {
  if constexpr (MODEL == kGDN && CL == 4) {
    if (fn == decode_kernel_occ<MODEL, CL, kFeatPlain, kSpecPersF16Bf16G32>)
      return decode_kernel_occ<MODEL, CL, kFeatPlain, kSpecPersF16Bf16G32, true>;
    if (fn == decode_kernel_occ<MODEL, CL, kFeatHad, kSpecPersF16Bf16G32>)
      return decode_kernel_occ<MODEL, CL, kFeatHad, kSpecPersF16Bf16G32, true>;
  }
  return nullptr;
}

template <int MODEL, int CL, int SPEC>
DecodeFn decode_pick_feat(int feat) {
  switch (feat) {
    case kFeatPlain:
      // the delta-rule step with binary16 persistent steps fits 128 VGPRs without
      // spilling; the others keep their natural allocation (a spill reload waits for
      // every outstanding load, which costs more than the lost occupancy)
      if constexpr (MODEL == kGDN && SPEC == kSpecPersF16Bf16G32) return decode_kernel_occ<MODEL, CL, kFeatPlain, SPEC>;
      else return decode_kernel<MODEL, CL, kFeatPlain, SPEC>;
    case kFeatBdr: return decode_kernel<MODEL, CL, kFeatBdr, kSpecGeneric>;
    case kFeatBypass: return decode_kernel<MODEL, CL, kFeatBypass, SPEC>;
    case kFeatYoked: return decode_kernel<MODEL, CL, kFeatYoked, kSpecGeneric>;
    case kFeatDiag: return decode_kernel<MODEL, CL, kFeatDiag, kSpecGeneric>;
    case kFeatHad:
      if constexpr (MODEL == kGDN && SPEC == kSpecPersF16Bf16G32) return decode_kernel_occ<MODEL, CL, kFeatHad, SPEC>;
      else return decode_kernel<MODEL, CL, kFeatHad, SPEC>;
    case kFeatPW:
      if constexpr (MODEL == kGDN && SPEC == kSpecPersF16Bf16G32) return decode_kernel_occ<MODEL, CL, kFeatPW, SPEC>;
      else if constexpr (MODEL == kGDN) return decode_kernel<MODEL, CL, kFeatPW, kSpecGeneric>;
      else return nullptr;
    default: return decode_kernel<MODEL, CL, kFeatF32, kSpecGeneric>;
  }
}

template <int MODEL, int CL>
DecodeFn decode_pick_spec(int feat, int spec) {
  if (feat != kFeatPlain && feat != kFeatBypass && feat != kFeatPW && feat != kFeatHad) spec = kSpecGeneric;
  // group-32 specialisations use 4 column lanes, group-64 ones 8
  if constexpr (CL == 4) {
    switch (spec) {
      case kSpecPersF16Bf16G32: return decode_pick_feat<MODEL, CL, kSpecPersF16Bf16G32>(feat);
      case kSpecDynF16Bf16G32: return decode_pick_feat<MODEL, CL, kSpecDynF16Bf16G32>(feat);
      default: break;
    }
  } else if constexpr (CL == 8) {
    switch (spec) {
      case kSpecDynF32Bf16G64: return decode_pick_feat<MODEL, CL, kSpecDynF32Bf16G64>(feat);
      case kSpecDynF32F32G64: return decode_pick_feat<MODEL, CL, kSpecDynF32F32G64>(feat);
      default: break;
    }
  }
  return decode_pick_feat<MODEL, CL, kSpecGeneric>(feat);
}

template <int MODEL>
DecodeFn decode_pick_cl(int cl, int feat, int spec) {
  switch (cl) {
    case 4: return decode_pick_spec<MODEL, 4>(feat, spec);
    case 8: return decode_pick_spec<MODEL, 8>(feat, spec);
    default: return decode_pick_spec<MODEL, 16>(feat, kSpecGeneric);
  }
}

DecodeFn decode_retnet(int cl, int feat, int spec);
DecodeFn decode_mamba2(int cl, int feat, int spec);
DecodeFn decode_gla(int cl, int feat, int spec);
DecodeFn decode_gdn(int cl, int feat, int spec);

}  // namespace rsq
