// Kernel arguments and the pieces shared by the decode, readout and merge
// kernels; host-side entry points to pick a kernel instance.
#pragma once
#include "rsq_device.hpp"

namespace rsq {

enum { kRetNet = 0, kMamba2 = 1, kGLA = 2, kGDN = 3 };
enum { kScaleDynamic = 0, kScalePersistent = 1, kScaleYoked = 2 };
// Compile-time feature variants of the decode kernel.
enum { kFeatPlain = 0, kFeatBdr = 1, kFeatBypass = 2, kFeatYoked = 3, kFeatF32 = 4, kFeatDiag = 5, kFeatHad = 6,
       kFeatPW = 7 };

struct StepArgs {
  uint8_t* tiles;            // state buffer + tiles offset
  const HeadEntry* heads;    // head table (device)
  uint32_t* status;          // device status word
  int64_t* hdr_t;            // header step count
  int32_t* hdr_n;            // header bypass fill
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* o;
  uint64_t batch_stride;
  int32_t H, dk, dv, group;
  int32_t smode;
  float trigger;
  int32_t bdr;
  float bdr_eps;
  int32_t bypass;            // 1 when a low-rank bypass is configured
  int32_t n;                 // bypass columns in use before this call
  int32_t cap;               // k + m
  int32_t lrb_k;
  float lrb_eps;
  int32_t in_bf16;           // q, k, v are bf16 (else fp32)
  int32_t scale_f16;         // step sizes are stored as fp16 (else fp32)
  int32_t hadamard;          // groups are stored rotated by the Sylvester-Hadamard matrix
  int32_t pw;                // pure-write window size W (0 = none); a.n = pairs held before the step
  int64_t t_next;
  // error accounting (kFeatDiag only): per tile 6 planes of d_k*d_v floats in
  // the fp32 chunk layout, optional |b|/step per element, 4 counters
  float* dg_acc;
  float* dg_ratio;
  uint32_t* dg_counts;
  // every head alike (same width; RetNet: same gamma): the head table entry
  // is `uni` with head_offset = h * uni_stride, so the kernels skip its load
  int32_t uniform;
  uint64_t uni_stride;
  HeadEntry uni;
};

// Head table entry of head h.
__device__ __forceinline__ HeadEntry head_entry(const StepArgs& a, int h) {
  if (a.uniform) {
    HeadEntry e = a.uni;
    e.head_offset = (uint64_t)h * a.uni_stride;
    return e;
  }
  return a.heads[h];
}

typedef void (*DecodeFn)(StepArgs);
DecodeFn decode_kernel_for(int model, int cl, int feat, int spec);
DecodeFn readout_kernel_for(int cl);
DecodeFn merge_kernel_for(int cl);
// dynamic LDS (floats) of the merge kernel for a tile of d_k x d_v split into
// wrw x wcw wavefronts with `cap` bypass columns
size_t merge_lds_floats(int dk, int dv, int wrw, int wcw, int cap);

// Decay of key row i of a tile (Table 1, A_t column).
__device__ __forceinline__ float row_decay(const StepArgs& a, const HeadEntry& he, int model,
                                           int tile, int i) {
  if (model == kRetNet) return he.gamma;
  if (model == kGLA) return a.alpha[(size_t)tile * a.dk + i];
  return a.alpha[tile];
}

__device__ __forceinline__ float in_elem(bool bf16, const void* p, size_t idx) {
  if (bf16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
  return reinterpret_cast<const float*>(p)[idx];
}

// Sum over the 64 lanes of a wavefront in a fixed order (every lane gets it):
// lane pairs 1, 2, 4, 8, 16 apart by DPP / swizzle, then the two halves.
__device__ __forceinline__ float wave_sum64(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x201F));
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

// Bypass side of a decode step (Low-Rank Bypass of "Preserving Updates in
// Low-Bit Recurrent State Quantization"; all of B_t goes to the bypass):
//   U[:, c] <- RN16(a_i U_ic) for c < n, U[:, n] = fp16(k), W[:, n] = fp16(w),
// and z_c = sum_i U_ic q_i (c <= n) for the readout term W z, left in lds_z.
// Column c belongs to wavefront c mod nw, whose lanes stride over the rows:
// the loads of a column are coalesced, and each column's sum is one wave
// reduction (the readout that uses it is order-free).
__device__ __forceinline__ void bypass_decode_phase(const StepArgs& a, const HeadEntry& he, uint8_t* tb, int tile,
                                                    float* lds_z, int model) {
  __half* U = reinterpret_cast<__half*>(tb + he.bypass_u);
  __half* W = reinterpret_cast<__half*>(tb + he.bypass_w);
  const int n = a.n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int c = wave; c <= n; c += nw) {
    __half* uc = U + (size_t)c * a.dk;
    float acc = 0.f;
    // four rows per lane at a time, all loads issued before the stores (which
    // could alias later loads for all the compiler knows)
    for (int i0 = lane; i0 < a.dk; i0 += 256) {
      float qv[4], av[4];
      __half uv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 64 * r;
        const bool ok = i < a.dk;
        qv[r] = ok ? in_elem(a.in_bf16, a.q, (size_t)tile * a.dk + i) : 0.f;
        if (c < n) {
          av[r] = ok ? row_decay(a, he, model, tile, i) : 0.f;
          uv[r] = ok ? uc[i] : __float2half_rn(0.f);
        } else {
          av[r] = ok ? in_elem(a.in_bf16, a.k, (size_t)tile * a.dk + i) : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 64 * r;
        if (i < a.dk) {
          const __half un = c < n ? mul_rn_half(av[r], uv[r]) : __float2half_rn(av[r]);
          uc[i] = un;
          acc = __builtin_fmaf(__half2float(un), qv[r], acc);
        }
      }
    }
    acc = wave_sum64(acc);
    if (lane == 0) lds_z[c] = acc;
  }
  for (int j = threadIdx.x; j < a.dv; j += blockDim.x)
    W[(size_t)n * a.dv + j] = __float2half_rn(in_elem(a.in_bf16, a.v, (size_t)tile * a.dv + j));
  __syncthreads();
}

}  // namespace rsq
