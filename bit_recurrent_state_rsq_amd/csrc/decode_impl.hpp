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
#pragma once
#include "rsq_kernels.hpp"

namespace rsq {

template <int MODEL, int CL, int FEAT>
struct Decode {
  static constexpr int RL = 64 / CL;
  static constexpr int NB = (RL == 16) ? 4 : (RL == 8) ? 3 : 2;   // log2(RL)
  static constexpr int WR = 8 * RL;
  static constexpr int WC = 8 * CL;

  // Row decays of the lane's 8 rows.
  static __device__ __forceinline__ void decays(const StepArgs& a, const HeadEntry& he, int tile,
                                                int i0, float dec[8]) {
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

  // Cascade sum of one lane value per column over the wavefront's row blocks,
  // in row-block order (lane bit 5 holds the lowest row-block bit).
  static __device__ __forceinline__ float rows_tree(float p) {
#pragma unroll
    for (int s = 0; s < NB; ++s) p = __fadd_rn(p, shfl_xor(p, 32 >> s));
    return p;
  }

  // Finish u_j across row-wavefronts (the top levels of the cascade).
  static __device__ __forceinline__ void rows_tree_waves(float u[8], float* upart, int wrw, int wr, int lr,
                                                         int j0, int dv) {
    if (wrw > 1) {
      if (lr == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) upart[wr * dv + j0 + j] = u[j];
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float lvl[8];
        for (int q = 0; q < wrw; ++q) lvl[q] = upart[q * dv + j0 + j];
        for (int n = wrw; n > 1; n >>= 1)
          for (int q = 0; q < n / 2; ++q) lvl[q] = __fadd_rn(lvl[2 * q], lvl[2 * q + 1]);
        u[j] = lvl[0];
      }
      __syncthreads();
    }
  }

  template <int BITS>
  static __device__ __forceinline__ void body(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                              float* lds_o, float* lds_u, float* lds_ur, uint32_t& flags) {
    constexpr bool kF32 = FEAT == kFeatF32;
    constexpr bool kBypass = FEAT == kFeatBypass;
    constexpr bool kYoked = FEAT == kFeatYoked;
    const bool bdr = (FEAT == kFeatBdr) || (kYoked && a.bdr);
    const bool bf16 = a.in_bf16 != 0, sf16 = a.scale_f16 != 0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wrw = a.dk / WR;
    const int wr = wave % wrw, wc = wave / wrw;
    const int lc = lane % CL, lr = lane / CL;
    const int rho = (int)(__builtin_bitreverse32((uint32_t)lr) >> (32 - NB));
    const int i0 = wr * WR + 8 * rho;
    const int j0 = wc * WC + 8 * lc;
    const int G = j0 / a.group;
    const int gl = a.group >> 3;        // lanes per group (1..16)

    float qf[8], kf[8], vf[8], dec[8];
    load8(bf16, a.q, (size_t)tile * a.dk + i0, qf);
    load8(bf16, a.k, (size_t)tile * a.dk + i0, kf);
    load8(bf16, a.v, (size_t)tile * a.dv + j0, vf);
    decays(a, he, tile, i0, dec);

    uint8_t* cp = tb + ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * (8 * BITS);
    uint8_t* sp = tb + he.scales + ((size_t)G * a.dk + i0) * (sf16 ? 2 : 4);
    // x starts as the codes (or the fp32 state) and becomes the updated state
    float x[8][8];
    float s_old[8];
    if constexpr (kF32) {
      load_f32_chunk(cp, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) s_old[i] = 1.f;
    } else {
      Chunk<BITS> ch;
      load_chunk<BITS>(cp, ch);
      load_scales8(sf16, sp, s_old);
      unpack(ch, x);
    }

    // delta rule: w = beta (v - alpha S^T k), S^T k as a cascade sum over rows
    float wv[8];
    if constexpr (MODEL == kGDN) {
      const float al = a.alpha[tile], be = a.beta[tile];
      float u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = __fmul_rn(kf[i], kF32 ? x[i][j] : __fmul_rn(x[i][j], s_old[i]));
        u[j] = rows_tree(tree8(t));
      }
      rows_tree_waves(u, lds_u, wrw, wr, lr, j0, a.dv);
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = __fmul_rn(be, __fsub_rn(vf[j], __fmul_rn(al, u[j])));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = vf[j];
    }

    // decay, then the update: x = fma(k_i, w_j, r_ij), r_ij = fl(c_ij fl(a_i s_i))
    float r[kBypass ? 1 : 8][8];   // kept for BDR only
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c1 = kF32 ? dec[i] : __fmul_rn(dec[i], s_old[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ri = __fmul_rn(x[i][j], c1);
        if constexpr (!kBypass) {
          r[i][j] = ri;
          x[i][j] = __builtin_fmaf(kf[i], wv[j], ri);
        } else {
          x[i][j] = ri;
        }
      }
    }

    // readout partial o_j = sum_i q_i x_ij over this wavefront's rows
    {
      float o8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(qf[i], x[i][j], acc);
#pragma unroll
        for (int s = 0; s < NB; ++s) acc += shfl_xor(acc, 32 >> s);
        o8[j] = acc;
      }
      if (lr == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) lds_o[wr * a.dv + j0 + j] = o8[j];
      }
    }

    if constexpr (kF32) {
      store_f32_chunk(cp, x);
      return;
    } else {
      // yoked reference: the same recurrence on an fp32 tile; absmax comes from it
      float xr[kYoked ? 8 : 1][8];
      if constexpr (kYoked) {
        uint8_t* rp = tb + he.ref + ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * 256;
        load_f32_chunk(rp, xr);
        float wr_[8];
        if constexpr (MODEL == kGDN) {
          const float al = a.alpha[tile], be = a.beta[tile];
          float u[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = __fmul_rn(kf[i], xr[i][j]);
            u[j] = rows_tree(tree8(t));
          }
          rows_tree_waves(u, lds_ur, wrw, wr, lr, j0, a.dv);
#pragma unroll
          for (int j = 0; j < 8; ++j) wr_[j] = __fmul_rn(be, __fsub_rn(vf[j], __fmul_rn(al, u[j])));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) wr_[j] = vf[j];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xr[i][j] = __builtin_fmaf(kf[i], wr_[j], __fmul_rn(dec[i], xr[i][j]));
        store_f32_chunk(rp, xr);
      }

      // scale rule per row of this lane's group
      constexpr int qmax = (1 << (BITS - 1)) - 1;
      constexpr float qmaxf = (float)qmax;
      float s_new[8], inv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (kYoked) m = fmaxf(m, fabsf(xr[i][j]));
          else m = fmaxf(m, fabsf(x[i][j]));
        }
        if (gl >= 2) m = fmaxf(m, shfl_xor(m, 1));
        if (gl >= 4) m = fmaxf(m, shfl_xor(m, 2));
        if (gl >= 8) m = fmaxf(m, shfl_xor(m, 4));
        if (gl >= 16) m = fmaxf(m, shfl_xor(m, 8));
        const float ratio = m / qmaxf;
        const float fresh = sf16 ? __half2float(__float2half_rn(ratio)) : ratio;
        float sn = fresh;
        if (a.smode == kScalePersistent) {
          const float thr = __fmul_rn(__fmul_rn(a.trigger, qmaxf), s_old[i]);
          sn = (m > thr) ? fresh : s_old[i];
        }
        if (isinf(sn)) flags |= kStatusScaleOverflow;
        s_new[i] = sn;
        inv[i] = (sn == 0.f) ? 0.f : 1.0f / sn;
      }

      // requantize (+ BDR toward the update's sign)
      int q[8][8];
      const float lo = (float)(-(1 << (BITS - 1))), hi = qmaxf;
      const float gate_k = __fadd_rn(0.5f, a.bdr_eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float gate = __fmul_rn(gate_k, s_new[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float t = __builtin_fmaf(x[i][j], inv[i], kMagic) - kMagic;
          if (t < lo || t > hi) flags |= kStatusClipped;
          float c = fminf(fmaxf(t, lo), hi);
          if constexpr (!kBypass) {
            if (bdr && s_new[i] > 0.f) {
              const float sg = (float)((kf[i] > 0.f) - (kf[i] < 0.f)) * (float)((wv[j] > 0.f) - (wv[j] < 0.f));
              if (sg != 0.f) {
                const float val = __fmul_rn(c, s_new[i]);
                const bool rev = (sg > 0.f) ? (val < r[i][j]) : (val > r[i][j]);
                if (rev) {
                  const float cand = fminf(fmaxf(c + sg, lo), hi);
                  const float err = fabsf(__fsub_rn(x[i][j], __fmul_rn(cand, s_new[i])));
                  if (err <= gate) c = cand;
                }
              }
            }
          }
          q[i][j] = (int)c;
        }
      }
      Chunk<BITS> out;
      pack(q, out);
      store_chunk<BITS>(cp, out);
      if ((lc & (gl - 1)) == 0) store_scales8(sf16, sp, s_new);
    }
  }

  static __device__ void run(const StepArgs& a) {
    extern __shared__ float lds[];
    const int tile = blockIdx.x;
    const int bb = tile / a.H, h = tile - bb * a.H;
    const HeadEntry he = a.heads[h];
    uint8_t* tb = a.tiles + (size_t)bb * a.batch_stride + he.head_offset;
    const int wrw = a.dk / WR;
    float* lds_o = lds;                       // [wrw][dv]
    float* lds_u = lds_o + wrw * a.dv;        // [wrw][dv]
    float* lds_ur = lds_u + wrw * a.dv;       // [wrw][dv]
    float* lds_z = lds_ur + wrw * a.dv;       // [kMaxCap] + [nwaves][kMaxCap]
    uint32_t flags = 0;

    if constexpr (FEAT == kFeatBypass) bypass_decode_phase(a, he, tb, tile, lds_z, MODEL);

    if constexpr (FEAT == kFeatF32) {
      body<32>(a, he, tb, tile, lds_o, lds_u, lds_ur, flags);
    } else {
      switch (he.bits) {
        case 4: body<4>(a, he, tb, tile, lds_o, lds_u, lds_ur, flags); break;
        case 6: body<6>(a, he, tb, tile, lds_o, lds_u, lds_ur, flags); break;
        default: body<8>(a, he, tb, tile, lds_o, lds_u, lds_ur, flags); break;
      }
    }
    __syncthreads();
    // combine readout partials over row-wavefronts, add the bypass term, store o
    for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
      float acc = 0.f;
      for (int q = 0; q < wrw; ++q) acc += lds_o[q * a.dv + j];
      if constexpr (FEAT == kFeatBypass) {
        const __half* W = reinterpret_cast<const __half*>(tb + he.bypass_w);
        for (int c = 0; c <= a.n; ++c) acc = __builtin_fmaf(__half2float(W[(size_t)c * a.dv + j]), lds_z[c], acc);
      }
      if (!isfinite(acc)) flags |= kStatusNonfinite;
      a.o[(size_t)tile * a.dv + j] = acc;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) flags |= (uint32_t)__shfl_xor((int)flags, m, 64);
    if (flags && (threadIdx.x & 63) == 0) atomicOr(a.status, flags);
    if (tile == 0 && threadIdx.x == 0) {
      *a.hdr_t = a.t_next;
      *a.hdr_n = (FEAT == kFeatBypass) ? a.n + 1 : 0;
    }
  }
};

template <int MODEL, int CL, int FEAT>
__global__ __launch_bounds__(512) void decode_kernel(StepArgs a) {
  Decode<MODEL, CL, FEAT>::run(a);
}

template <int MODEL, int CL>
DecodeFn decode_pick_feat(int feat) {
  switch (feat) {
    case kFeatPlain: return decode_kernel<MODEL, CL, kFeatPlain>;
    case kFeatBdr: return decode_kernel<MODEL, CL, kFeatBdr>;
    case kFeatBypass: return decode_kernel<MODEL, CL, kFeatBypass>;
    case kFeatYoked: return decode_kernel<MODEL, CL, kFeatYoked>;
    default: return decode_kernel<MODEL, CL, kFeatF32>;
  }
}

template <int MODEL>
DecodeFn decode_pick_cl(int cl, int feat) {
  switch (cl) {
    case 4: return decode_pick_feat<MODEL, 4>(feat);
    case 8: return decode_pick_feat<MODEL, 8>(feat);
    default: return decode_pick_feat<MODEL, 16>(feat);
  }
}

DecodeFn decode_retnet(int cl, int feat);
DecodeFn decode_mamba2(int cl, int feat);
DecodeFn decode_gla(int cl, int feat);
DecodeFn decode_gdn(int cl, int feat);

}  // namespace rsq
