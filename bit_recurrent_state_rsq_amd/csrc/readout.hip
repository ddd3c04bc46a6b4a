// Readout without an update: o = deq(S)^T q (+ W (U^T q) when a bypass is in
// use). The state is only read. The readout o_t = S_t^T q_t is the output of a
// linear-attention / SSM layer whose recurrence is Table 1 of "Preserving
// Updates in Low-Bit Recurrent State Quantization".
#include "rsq_kernels.hpp"

namespace rsq {

template <int CL>
struct Readout {
  static constexpr int RL = 64 / CL;
  static constexpr int NB = (RL == 16) ? 4 : (RL == 8) ? 3 : 2;
  static constexpr int WR = 8 * RL;
  static constexpr int WC = 8 * CL;

  template <int BITS>
  static __device__ __forceinline__ void body(const StepArgs& a, const HeadEntry& he, const uint8_t* tb, int tile,
                              float* lds_o) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wrw = a.dk / WR;
    const int wr = wave % wrw, wc = wave / wrw;
    const int lc = lane % CL, lr = lane / CL;
    const int rho = (int)(__builtin_bitreverse32((uint32_t)lr) >> (32 - NB));
    const int i0 = wr * WR + 8 * rho;
    const int j0 = wc * WC + 8 * lc;
    float qf[8];
    load8(a.in_bf16 != 0, a.q, (size_t)tile * a.dk + i0, qf);
    const uint8_t* cp = tb + ((size_t)(j0 >> 3) * (a.dk >> 3) + (i0 >> 3)) * (8 * BITS);
    float x[8][8];
    if constexpr (BITS == 32) {
      load_f32_chunk(cp, x);
    } else {
      const int G = j0 / a.group;
      float s[8];
      Chunk<BITS> ch;
      load_chunk<BITS>(cp, ch);
      load_scales8(a.scale_f16 != 0, tb + he.scales + ((size_t)G * a.dk + i0) * (a.scale_f16 ? 2 : 4), s);
      unpack(ch, x);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = __fmul_rn(x[i][j], s[i]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(qf[i], x[i][j], acc);
#pragma unroll
      for (int s = 0; s < NB; ++s) acc += __shfl_xor(acc, 32 >> s, 64);
      if (lr == 0) lds_o[wr * a.dv + j0 + j] = acc;
    }
  }

  static __device__ void run(const StepArgs& a) {
    extern __shared__ float lds[];
    const int tile = blockIdx.x;
    const int bb = tile / a.H, h = tile - bb * a.H;
    const HeadEntry he = head_entry(a, h);
    const uint8_t* tb = a.tiles + (size_t)bb * a.batch_stride + he.head_offset;
    const int wrw = a.dk / WR;
    float* lds_o = lds;
    float* lds_z = lds_o + wrw * a.dv;
    // bypass columns (fp16) or pure-write window pairs (E4M3 bytes)
    const bool fp8 = a.pw > 0;
    const int n = (a.bypass || fp8) ? a.n : 0;
    auto pair_u = [&](int c, int i) {
      return fp8 ? e4m3_to_f32(tb[he.bypass_u + (size_t)c * a.dk + i])
                 : __half2float(reinterpret_cast<const __half*>(tb + he.bypass_u)[(size_t)c * a.dk + i]);
    };
    auto pair_w = [&](int c, int j) {
      return fp8 ? e4m3_to_f32(tb[he.bypass_w + (size_t)c * a.dv + j])
                 : __half2float(reinterpret_cast<const __half*>(tb + he.bypass_w)[(size_t)c * a.dv + j]);
    };
    if (n > 0) {
      // z_c = sum_i U_ic q_i
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
      float* zpart = lds_z + kMaxCap;
      for (int c = 0; c < n; ++c) {
        float acc = 0.f;
        for (int i = threadIdx.x; i < a.dk; i += blockDim.x)
          acc = __builtin_fmaf(pair_u(c, i), in_elem(a.in_bf16 != 0, a.q, (size_t)tile * a.dk + i), acc);
        for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
        if (lane == 0) zpart[wave * kMaxCap + c] = acc;
      }
      __syncthreads();
      if ((int)threadIdx.x < n) {
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += zpart[w * kMaxCap + threadIdx.x];
        lds_z[threadIdx.x] = s;
      }
    }
    switch (he.bits) {
      case 4: body<4>(a, he, tb, tile, lds_o); break;
      case 6: body<6>(a, he, tb, tile, lds_o); break;
      case 8: body<8>(a, he, tb, tile, lds_o); break;
      default: body<32>(a, he, tb, tile, lds_o); break;
    }
    __syncthreads();
    if (a.hadamard) {
      // rotated groups (INT4+Had): the row sums above are sum_i q_i (c s)_ij;
      // o = (those sums) H / g per group, H[a][b] = (-1)^popcount(a & b)
      float* rot = lds_z + kMaxCap * (1 + (blockDim.x >> 6));
      for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
        float acc = 0.f;
        for (int q = 0; q < wrw; ++q) acc += lds_o[q * a.dv + j];
        rot[j] = acc;
      }
      __syncthreads();
      const int g = a.group;
      const float ig = 1.0f / (float)g;
      for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
        const int base = j & ~(g - 1), jj = j & (g - 1);
        float acc = 0.f;
        for (int b = 0; b < g; ++b) {
          const float v = rot[base + b];
          acc += (__builtin_popcount(jj & b) & 1) ? -v : v;
        }
        a.o[(size_t)tile * a.dv + j] = acc * ig;
      }
      return;
    }
    for (int j = threadIdx.x; j < a.dv; j += blockDim.x) {
      float acc = 0.f;
      for (int q = 0; q < wrw; ++q) acc += lds_o[q * a.dv + j];
      for (int c = 0; c < n; ++c) acc = __builtin_fmaf(pair_w(c, j), lds_z[c], acc);
      a.o[(size_t)tile * a.dv + j] = acc;
    }
  }
};

template <int CL>
__global__ __launch_bounds__(512) void readout_kernel(StepArgs a) {
  Readout<CL>::run(a);
}

DecodeFn readout_kernel_for(int cl) {
  switch (cl) {
    case 4: return readout_kernel<4>;
    case 8: return readout_kernel<8>;
    default: return readout_kernel<16>;
  }
}

}  // namespace rsq
